// permute.h -- row -> expert permutation and the grouped-GEMM work list
// (device code, run at the end of the routing kernel, see route_block.hip).
//
// Every routed (row, slot) pair gets a position in an expert-major order:
// experts ascending, and inside an expert rows ascending (the key
// expert, row*k + slot; a row routes to an expert at most once).  Each expert
// touched by the call is then streamed once, with its rows gathered next to
// each other (the CMF model card's "Hardware" section describes the same
// idea on Metal, where a block's experts are attached only once its routing
// has chosen them).
//
// The order is built without sorting: a bit mask per expert marks the rows
// routed to it, so a pair's rank inside its expert is a popcount of the
// mask bits below its row.  Counts, positions and tiles are all exact
// integer results, independent of thread timing.
//
// Two variants:
//  * permute_single: the call is one block of at most 32 rows, whose routing
//    workgroup still holds the top-k result and one mask word per expert in
//    LDS; two barriers and no global round trips.
//  * many blocks (permute_blocks.hip): every routing workgroup publishes one
//    mask word per expert; a scan kernel turns them into per-block prefixes
//    and counts, and one workgroup per block places its own rows.
#pragma once
#include "cmoe_device.h"
#include "cmoe_launch.h"

namespace cmoe {

// inclusive prefix sum over the 64 lanes of a wave (all lanes active):
// shifted adds inside each 16-lane row, then the totals of the rows below
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

struct PermuteLds {
  int cnt[256];
  int off[257];
};

// Run by one whole wave (lanes 0..63): expert e = 4*lane + i has L.cnt[e]
// pairs.  Writes the exclusive offsets to LDS and, with publish, to the
// call's buffers together with the work list: ceil(count / T) tiles per
// expert, experts ascending, then the shared expert's tiles over the N rows
// in order.
__device__ __forceinline__ void offsets_and_tiles(const Plan& p, PermuteLds& L, bool publish) {
  const int lane = threadIdx.x & 63;
  const int E = p.E, T = p.tile_rows;
  int c[4], nt[4], csum = 0, tsum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    c[i] = e < E ? L.cnt[e] : 0;
    nt[i] = (c[i] + T - 1) / T;
    csum += c[i];
    tsum += nt[i];
  }
  const int cinc = wave_incl_scan(csum), tinc = wave_incl_scan(tsum);
  const int ctot = __builtin_amdgcn_readlane(cinc, 63), ttot = __builtin_amdgcn_readlane(tinc, 63);
  int coff = cinc - csum, toff = tinc - tsum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (e < E) {
      L.off[e] = coff;
    }
    if (e < E && publish) {
      p.counts[e] = c[i];
      p.offsets[e] = coff;
      if (p.out_counts) p.out_counts[e] = c[i];
      if (p.out_offsets) p.out_offsets[e] = coff;
      for (int t = 0; t < nt[i]; ++t) {
        Tile tile;
        tile.expert = e;
        tile.start = coff + t * T;
        tile.rows = min(T, c[i] - t * T);
        tile.pad = 0;
        p.tiles[toff + t] = tile;
      }
    }
    coff += c[i];
    toff += nt[i];
  }
  if (lane == 0) L.off[E] = ctot;
  if (!publish) return;
  if (lane == 0) {
    p.offsets[E] = ctot;
    if (p.out_offsets) p.out_offsets[E] = ctot;
  }
  const int ns = p.Is > 0 ? (p.N + T - 1) / T : 0;
  for (int t = lane; t < ns; t += 64) {
    Tile tile;
    tile.expert = E;
    tile.start = t * T;
    tile.rows = min(T, p.N - t * T);
    tile.pad = 0;
    p.tiles[ttot + t] = tile;
  }
  if (lane == 0) *p.tile_count = ttot + ns;
}

// One block of N <= 32 rows: tk_s[N*K] holds the block's top-k (-1 for an
// empty slot) and mask_s[e] bit r is set iff row r routes to expert e.
// Called by all 1024 threads after a barrier that follows those writes.
__device__ inline void permute_single(const Plan& p, PermuteLds& L, const uint32_t* mask_s,
                               const int* tk_s) {
  const int tid = threadIdx.x;
  const int NK = p.N * p.K;
  if (tid < 64) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * tid + i;
      if (e < p.E) L.cnt[e] = __popc(mask_s[e]);
    }
    offsets_and_tiles(p, L, true);
  }
  __syncthreads();
  if (tid < NK) {
    const int e = tk_s[tid];
    int pos = -1;
    if (e >= 0) {
      const int r = tid / p.K;
      pos = L.off[e] + __popc(mask_s[e] & ((1u << r) - 1u));
      p.pair_row[pos] = r;
      if (p.out_perm) p.out_perm[pos] = tid;
    }
    p.pair_pos[tid] = pos;
  }
  if (p.out_perm)
    for (int i = L.off[p.E] + tid; i < NK; i += 1024) p.out_perm[i] = -1;
}

}  // namespace cmoe
