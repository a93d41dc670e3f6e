// permute.hip -- row -> expert permutation and the grouped-GEMM work list.
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
// One workgroup of 1024 threads does the whole call; the masks live in the
// workspace and are touched only with device-scope atomics.
#include "cmoe_device.h"
#include "cmoe_launch.h"

namespace cmoe {

__device__ __forceinline__ uint32_t mask_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

__global__ __launch_bounds__(1024) void permute_kernel(Plan p) {
  __shared__ int cnt_s[256];
  __shared__ int off_s[257];
  __shared__ int scan_scratch[16];
  const int tid = threadIdx.x;
  const int N = p.N, K = p.K, E = p.E, W = p.mask_words;
  const int NK = N * K;

  for (int i = tid; i < E * W; i += 1024)
    __hip_atomic_store(p.rowmask + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid < 256) cnt_s[tid] = 0;
  __syncthreads();

  // masks and counts
  for (int i = tid; i < NK; i += 1024) {
    const int e = p.topk[i];
    if (e >= 0) {
      const int r = i / K;
      atomicOr(p.rowmask + (size_t)e * W + (r >> 5), 1u << (r & 31));
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

  // per-expert exclusive popcount prefix over mask words
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      p.prefix[(size_t)e * W + w] = run;
      run += __popc(mask_load(p.rowmask + (size_t)e * W + w));
    }
  }
  __syncthreads();

  // positions
  for (int i = tid; i < NK; i += 1024) {
    const int e = p.topk[i];
    int pos = -1;
    if (e >= 0) {
      const int r = i / K;
      const uint32_t word = mask_load(p.rowmask + (size_t)e * W + (r >> 5));
      const uint32_t below = word & ((1u << (r & 31)) - 1u);
      pos = off_s[e] + p.prefix[(size_t)e * W + (r >> 5)] + __popc(below);
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
    const int nt = (n + kTileRows - 1) / kTileRows;
    int ntiles;
    const int base = block_exclusive_scan(tid <= E ? nt : 0, scan_scratch, &ntiles);
    if (tid <= E) {
      const int start0 = tid < E ? off_s[tid] : 0;
      for (int t = 0; t < nt; ++t) {
        Tile tile;
        tile.expert = tid;
        tile.start = start0 + t * kTileRows;
        tile.rows = min(kTileRows, n - t * kTileRows);
        tile.pad = 0;
        p.tiles[base + t] = tile;
      }
    }
    if (tid == 0) *p.tile_count = ntiles;
  }
}

hipError_t launch_permute(const Plan& p, hipStream_t s) {
  permute_kernel<<<1, 1024, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace cmoe
