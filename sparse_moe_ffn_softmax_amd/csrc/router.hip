// router.hip -- router logits l[r,e] = x[r,:] . Wr[e,:] (+ b[e]) on the fp32
// vector ALU.
//
// The routing decisions downstream (coreset, top-k) must be reproducible bit
// for bit, so the dot product follows a fixed order rather than whatever a
// matrix core does internally: h is split into 8 contiguous chunks
// [j*H/8, (j+1)*H/8); each chunk accumulates ascending h with fp32 fma
// starting from +0; the 8 partial sums combine pairwise (j += j+4, then
// j += j+2, then j += j+1); the bias is one final fp32 add.  (256 experts and
// top-8 routing: Clover-35B-A3B-Preview CMF model card, introduction.)
//
// Parallel layout: a workgroup of 256 threads owns a tile of RT rows x ET
// experts; thread group c (32 threads) runs chunk c for every output of the
// tile, each thread keeping TR x TE independent accumulators.  Operands are
// staged through LDS in slices of KB positions per chunk.  The register tile
// only changes which thread runs a chain, never the order inside a chain.
#include "cmoe_device.h"
#include "cmoe_launch.h"

#pragma clang fp contract(off)

namespace cmoe {

template <typename XT>
__device__ __forceinline__ float load_act(const XT* p);
template <>
__device__ __forceinline__ float load_act<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <int TR, int TE, typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int N,
                                                            int H, int E) {
  constexpr int RT = 8 * TR;  // rows per workgroup
  constexpr int ET = 4 * TE;  // experts per workgroup
  constexpr int KB = 16;      // positions per chunk staged at a time
  __shared__ float xs[8][KB][RT + 1];
  __shared__ float ws[8][KB][ET + 1];
  __shared__ float part[8][RT][ET + 1];

  const int tid = threadIdx.x;
  const int c = tid >> 5;  // chunk run by this thread
  const int q = tid & 31;
  const int rq = q & 7;    // row group
  const int eq = q >> 3;   // expert group
  const int row0 = blockIdx.x * RT;
  const int e0 = blockIdx.y * ET;
  const int L = H / 8;     // chunk length (H is a multiple of 128)

  float acc[TR][TE];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.0f;

  for (int kb = 0; kb < L; kb += KB) {
    for (int i = tid; i < 8 * KB * RT; i += 256) {
      const int k = i % KB, r = (i / KB) % RT, cc = i / (KB * RT);
      const int row = row0 + r;
      xs[cc][k][r] = row < N ? load_act<XT>(x + (size_t)row * H + cc * L + kb + k) : 0.0f;
    }
    for (int i = tid; i < 8 * KB * ET; i += 256) {
      const int k = i % KB, e = (i / KB) % ET, cc = i / (KB * ET);
      const int ex = e0 + e;
      ws[cc][k][e] = ex < E ? w[(size_t)ex * H + cc * L + kb + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < KB; ++k) {
      float xv[TR], wv[TE];
#pragma unroll
      for (int i = 0; i < TR; ++i) xv[i] = xs[c][k][rq * TR + i];
#pragma unroll
      for (int j = 0; j < TE; ++j) wv[j] = ws[c][k][eq * TE + j];
#pragma unroll
      for (int i = 0; i < TR; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) acc[i][j] = __builtin_fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) part[c][rq * TR + i][eq * TE + j] = acc[i][j];
  __syncthreads();

  for (int o = tid; o < RT * ET; o += 256) {
    const int r = o / ET, e = o % ET;
    const int row = row0 + r, ex = e0 + e;
    if (row >= N || ex >= E) continue;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = part[j][r][e];
    p[0] = p[0] + p[4];
    p[1] = p[1] + p[5];
    p[2] = p[2] + p[6];
    p[3] = p[3] + p[7];
    p[0] = p[0] + p[2];
    p[1] = p[1] + p[3];
    p[0] = p[0] + p[1];
    float l = p[0];
    if (bias) l = l + bias[ex];
    logits[(size_t)row * E + ex] = l;
  }
}

hipError_t launch_router(const Plan& p, const void* x, const float* router_w,
                         const float* router_b, hipStream_t s) {
  // Few rows (a single block per call): one accumulator per thread keeps
  // enough workgroups in flight.  Many rows: 4x4 register tiles.
  if (p.N <= 256) {
    dim3 grid((p.N + 7) / 8, (p.E + 3) / 4);
    if (p.act == CMOE_BF16)
      router_logits_kernel<1, 1, uint16_t><<<grid, 256, 0, s>>>(
          static_cast<const uint16_t*>(x), router_w, router_b, p.logits, p.N, p.H, p.E);
    else
      router_logits_kernel<1, 1, float><<<grid, 256, 0, s>>>(
          static_cast<const float*>(x), router_w, router_b, p.logits, p.N, p.H, p.E);
  } else {
    dim3 grid((p.N + 31) / 32, (p.E + 15) / 16);
    if (p.act == CMOE_BF16)
      router_logits_kernel<4, 4, uint16_t><<<grid, 256, 0, s>>>(
          static_cast<const uint16_t*>(x), router_w, router_b, p.logits, p.N, p.H, p.E);
    else
      router_logits_kernel<4, 4, float><<<grid, 256, 0, s>>>(
          static_cast<const float*>(x), router_w, router_b, p.logits, p.N, p.H, p.E);
  }
  return hipGetLastError();
}

}  // namespace cmoe
