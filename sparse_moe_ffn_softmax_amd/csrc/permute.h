// permute.h -- row -> expert permutation and the grouped-GEMM work list
// (device code; run by the last routing workgroup of a call, see
// route_block.hip).
//
// Every routed (row, slot) pair gets a position in an expert-major order:
// experts ascending, and inside an expert rows ascending (the key
// expert, row*k + slot; a row routes to an expert at most once).  The experts
// a block uses are then streamed once each, with their rows gathered next to
// each other (the CMF model card's "Hardware" section describes the same
// idea on Metal: the experts a block uses are bound as they are routed).
//
// The order is built without sorting: a bit mask per expert marks the rows
// routed to it, so a pair's rank inside its expert is a popcount of the
// mask bits below its row.  Counts, positions and tiles are all exact
// integer results, independent of thread timing.
//
// One workgroup of 1024 threads does the whole call; the masks live in LDS
// when they fit (N <= 2048 rows at E = 256), else in the workspace, where they
// are touched only with device-scope atomics.
#pragma once
#include "cmoe_device.h"
#include "cmoe_launch.h"

namespace cmoe {

// exclusive scan of v over the 1024 threads of the workgroup; returns the
// thread's exclusive prefix and writes the total to *total.
__device__ int block_exclusive_scan(int v, int* scratch /*[16]*/, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wave_base = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int t = scratch[w];
    if (w < wave) wave_base += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return wave_base + incl - v;
}

// Row masks of E x W words (W = ceil(N/32)): in LDS when they fit (N <= 2048
// rows at E = 256), else in the workspace.  A coarse per-expert popcount
// prefix over groups of G mask words always lives in LDS; a pair's rank adds
// the popcounts of at most G-1 words of its group.
constexpr int kLdsMaskWords = 16384;
constexpr int kPrefixWords = 8192;

struct PermuteLds {
  int cnt[256];
  int off[257];
  int scan[16];
};

// The whole permutation, run by one workgroup of 1024 threads.
// mask_lds: kLdsMaskWords words (used when kLdsMask); pref_lds: kPrefixWords.
template <bool kLdsMask>
__device__ void permute_block(const Plan& p, PermuteLds& L, uint32_t* mask_lds, int32_t* pref_lds) {
  int* cnt_s = L.cnt;
  int* off_s = L.off;
  int* scan_scratch = L.scan;
  const int tid = threadIdx.x;
  const int N = p.N, K = p.K, E = p.E, W = p.mask_words;
  const int NK = N * K;
  uint32_t* masks = kLdsMask ? mask_lds : p.rowmask;
  auto mask_load = [&](size_t i) -> uint32_t {
    if constexpr (kLdsMask) return mask_lds[i];
    else return __hip_atomic_load(p.rowmask + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  for (int i = tid; i < E * W; i += 1024) {
    if constexpr (kLdsMask) mask_lds[i] = 0u;
    else __hip_atomic_store(p.rowmask + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < 256) cnt_s[tid] = 0;
  __syncthreads();

  // masks and counts
  for (int i = tid; i < NK; i += 1024) {
    const int e = p.topk[i];
    if (e >= 0) {
      const int r = i / K;
      atomicOr(masks + (size_t)e * W + (r >> 5), 1u << (r & 31));
      atomicAdd(&cnt_s[e], 1);
    }
  }
  __syncthreads();

  // offsets: exclusive scan of counts
  int total;
  {
    const int v = tid < E ? cnt_s[tid] : 0;
    const int ex = block_exclusive_scan(v, scan_scratch, &total);
    if (tid < E) {
      off_s[tid] = ex;
      p.counts[tid] = v;
      p.offsets[tid] = ex;
      if (p.out_counts) p.out_counts[tid] = v;
      if (p.out_offsets) p.out_offsets[tid] = ex;
    }
    if (tid == 0) {
      off_s[E] = total;
      p.offsets[E] = total;
      if (p.out_offsets) p.out_offsets[E] = total;
    }
  }

  // coarse exclusive popcount prefix per expert over groups of G words
  int G = 1;
  while (E * ((W + G - 1) / G) > kPrefixWords) G <<= 1;
  const int J = (W + G - 1) / G;
  for (int i = tid; i < E * J; i += 1024) {
    const int e = i / J, j = i % J;
    int c = 0;
    for (int w = j * G; w < min(W, j * G + G); ++w) c += __popc(mask_load((size_t)e * W + w));
    pref_lds[i] = c;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int j = 0; j < J; ++j) {
      const int c = pref_lds[e * J + j];
      pref_lds[e * J + j] = run;
      run += c;
    }
  }
  __syncthreads();

  // positions
  for (int i = tid; i < NK; i += 1024) {
    const int e = p.topk[i];
    int pos = -1;
    if (e >= 0) {
      const int r = i / K, w = r >> 5, j = w / G;
      int rank = pref_lds[e * J + j];
      for (int w2 = j * G; w2 < w; ++w2) rank += __popc(mask_load((size_t)e * W + w2));
      rank += __popc(mask_load((size_t)e * W + w) & ((1u << (r & 31)) - 1u));
      pos = off_s[e] + rank;
      p.pair_row[pos] = r;
      if (p.out_perm) p.out_perm[pos] = i;
    }
    p.pair_pos[i] = pos;
  }
  if (p.out_perm)
    for (int i = total + tid; i < NK; i += 1024) p.out_perm[i] = -1;

  // work tiles: experts ascending, then the shared expert (index E)
  {
    const bool has_shared = p.Is > 0;
    int n = 0;
    if (tid < E) n = cnt_s[tid];
    else if (tid == E && has_shared) n = N;
    const int T = p.tile_rows;
    const int nt = (n + T - 1) / T;
    int ntiles;
    const int base = block_exclusive_scan(tid <= E ? nt : 0, scan_scratch, &ntiles);
    if (tid <= E) {
      const int start0 = tid < E ? off_s[tid] : 0;
      for (int t = 0; t < nt; ++t) {
        Tile tile;
        tile.expert = tid;
        tile.start = start0 + t * T;
        tile.rows = min(T, n - t * T);
        tile.pad = 0;
        p.tiles[base + t] = tile;
      }
    }
    if (tid == 0) *p.tile_count = ntiles;
  }
}

}  // namespace cmoe
