// permute_blocks.hip -- the row -> expert permutation and the grouped-GEMM
// work list for calls of many blocks (see permute.h for the order: experts
// ascending, rows ascending inside an expert; InfiniLM PR #604, "Summary":
// per-block coreset routing of the preview pass).
//
// The routing kernel leaves, for every block b and expert e, the mask word
// blockmask[b][e] whose bit r is set iff row r of the block routes to e (a
// block has at most 32 rows).  Two kernels follow it on the stream:
//
//   permute_scan : one wave per expert scans the popcounts of its column of
//                  mask words over the blocks: blockpre[b][e] = pairs of e in
//                  the blocks before b, counts[e] = all pairs of e.
//   permute_rows : one workgroup per block scans the counts over the experts
//                  (offsets) and places the block's own pairs:
//                  pos = offset[e] + blockpre[b][e] + popcount of the bits of
//                  rows below r in blockmask[b][e].  Block 0 also writes the
//                  offsets and the work list.
//
// Every result is an exact integer function of the masks, independent of
// thread timing, and the kernel boundaries order the writes and reads
// without any device-scope fence.
#include "cmoe_device.h"
#include "cmoe_launch.h"
#include "permute.h"

namespace cmoe {

__global__ __launch_bounds__(256) void permute_scan_kernel(Plan p) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= p.E) return;  // whole waves only
  int carry = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < p.B ? __popc(p.blockmask[(size_t)b * p.E + e]) : 0;
    const int inc = wave_incl_scan(c);
    if (b < p.B) p.blockpre[(size_t)b * p.E + e] = carry + inc - c;
    carry += __builtin_amdgcn_readlane(inc, 63);
  }
  if (lane == 0) p.counts[e] = carry;
}

__global__ __launch_bounds__(256) void permute_rows_kernel(Plan p) {
  __shared__ PermuteLds L;
  const int tid = threadIdx.x, b = blockIdx.x;
  if (tid < 64) {
    // unconditional loads (experts past E read expert 0), so the four are in
    // flight together
    int c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * tid + i;
      c[i] = p.counts[e < p.E ? e : 0];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * tid + i < p.E) L.cnt[4 * tid + i] = c[i];
    offsets_and_tiles(p, L, b == 0);
  }
  __syncthreads();
  const int RK = p.R * p.K;
  for (int j = tid; j < RK; j += 256) {
    const int i = b * RK + j;  // pair index row * K + slot
    const int e = p.topk[i];
    int pos = -1;
    if (e >= 0) {
      const int rl = j / p.K;  // row inside the block (< 32)
      const size_t be = (size_t)b * p.E + e;
      pos = L.off[e] + p.blockpre[be] + __popc(p.blockmask[be] & ((1u << rl) - 1u));
      p.pair_row[pos] = b * p.R + rl;
      if (p.out_perm) p.out_perm[pos] = i;
    }
    p.pair_pos[i] = pos;
  }
  if (b == 0 && p.out_perm)
    for (int i = L.off[p.E] + tid; i < p.N * p.K; i += 256) p.out_perm[i] = -1;
}

hipError_t launch_permute_blocks(const Plan& p, hipStream_t s) {
  permute_scan_kernel<<<(p.E + 3) / 4, 256, 0, s>>>(p);
  permute_rows_kernel<<<p.B, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace cmoe
