// route_block.hip -- per-block routing: softmax, block mass, coreset and
// restricted top-k with renormalised gates.  One workgroup per block.
//
// What is computed (Clover-35B-A3B-Preview CMF model card: introduction for
// "256 experts top-8 plus a shared expert", "Usage" for "the block's experts
// restricted to the set that carries 90% of its routing"; InfiniLM PR #604
// "Summary" for block coreset routing in the preview pass, "Motivation" for
// top-4 preview routing, "Notes for Reviewers" for the full-route replay):
//
//   u[r,e]   = exp(l[r,e] - max_e l[r,:])                         fp64
//   Z[r]     = sum_e u[r,e]   (8 contiguous chunks of e, ascending inside a
//                              chunk, pairwise combine j+=j+4, j+=j+2, j+=j+1)
//   mass[e]  = sum over the block's rows, ascending, of u[r,e] / Z[r]
//   order    = experts by (mass desc, id asc)
//   cum[i]   = sequential fp64 prefix sum of mass in that order
//   coreset  = order[0 : m], m the smallest with cum[m-1] >= tau * cum[E-1];
//              tau >= 1 gives m = E
//   per row  : the min(k, m) coreset experts with the largest fp32 logits,
//              ties to the lower id; gate_j = (float)(u_j / sum of u over the
//              chosen slots in slot order)
//
// exp is evaluated by Cody & Waite's (1980) argument reduction and the
// degree-13 Taylor polynomial of exp(r), Horner with fma, then scaled by
// 2^n; every operation is an IEEE fp64 primitive, so results are bitwise
// reproducible on any IEEE machine that follows the same sequence.
#include "cmoe_device.h"
#include "cmoe_launch.h"

#pragma clang fp contract(off)

namespace cmoe {

constexpr int kMaxRows = 32;
constexpr int kMaxExperts = 256;

// 1/ln 2 (correctly rounded); ln 2 split into a 42-bit head (so that n*head is
// exact for |n| < 2^11) and its correctly rounded tail; 1/i! for i = 0..13.
__constant__ double kInvLn2 = 0x1.71547652b82fep+0;
__constant__ double kLn2Head = 0x1.62e42fefa3800p-1;
__constant__ double kLn2Tail = 0x1.ef35793c76730p-45;
__constant__ double kInvFact[14] = {
    0x1.0000000000000p+0,  0x1.0000000000000p+0,  0x1.0000000000000p-1,  0x1.5555555555555p-3,
    0x1.5555555555555p-5,  0x1.1111111111111p-7,  0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13,
    0x1.a01a01a01a01ap-16, 0x1.71de3a556c734p-19, 0x1.27e4fb7789f5cp-22, 0x1.ae64567f544e4p-26,
    0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33};

__device__ __forceinline__ double exp_reduced(double d) {
  if (d < -708.0) return 0.0;  // below the normal range
  const double n = __builtin_rint(d * kInvLn2);
  double r = __builtin_fma(-n, kLn2Head, d);
  r = __builtin_fma(-n, kLn2Tail, r);
  double poly = kInvFact[13];
#pragma unroll
  for (int i = 12; i >= 0; --i) poly = __builtin_fma(poly, r, kInvFact[i]);
  return __builtin_ldexp(poly, static_cast<int>(n));
}

// (logit desc, id asc) ordering of top-k candidates; id >= E marks "none".
__device__ __forceinline__ bool better(float la, int ea, float lb, int eb, int E) {
  const bool va = ea < E, vb = eb < E;
  if (va != vb) return va;
  if (!va) return false;
  if (la != lb) return la > lb;
  return ea < eb;
}

__global__ __launch_bounds__(256) void route_block_kernel(
    const float* __restrict__ logits, int R, int E, int K, float tau, int32_t* __restrict__ topk,
    float* __restrict__ gates, int32_t* __restrict__ coreset_ids,
    int32_t* __restrict__ coreset_size, double* __restrict__ block_mass) {
  __shared__ float l_s[kMaxRows][kMaxExperts];
  __shared__ double u_s[kMaxRows][kMaxExperts];
  __shared__ double zpart[kMaxRows][8];
  __shared__ double z_s[kMaxRows];
  __shared__ double mass_s[kMaxExperts];
  __shared__ double cum_s[kMaxExperts];
  __shared__ int order_s[kMaxExperts];
  __shared__ int rank_s[kMaxExperts];
  __shared__ int m_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;
  const float* lb = logits + (size_t)b * R * E;

  for (int i = tid; i < R * E; i += 256) l_s[i / E][i % E] = lb[i];
  __syncthreads();

  // u = exp(l - row max); the max is exact and order-free.
  for (int r = wave; r < R; r += 4) {
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, l_s[r][e]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, shfl_xor_f(m, off));
    const double md = static_cast<double>(m);
    for (int e = lane; e < E; e += 64) u_s[r][e] = exp_reduced(static_cast<double>(l_s[r][e]) - md);
  }
  __syncthreads();

  // Z: chunk partial sums, one thread per (row, chunk).
  {
    const int r = tid >> 3, j = tid & 7;
    if (r < R) {
      const int lo = (j * E) / 8, hi = ((j + 1) * E) / 8;
      double acc = 0.0;
      for (int e = lo; e < hi; ++e) acc = acc + u_s[r][e];
      zpart[r][j] = acc;
    }
  }
  __syncthreads();
  if (tid < R) {
    double p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = zpart[tid][j];
    p[0] = p[0] + p[4];
    p[1] = p[1] + p[5];
    p[2] = p[2] + p[6];
    p[3] = p[3] + p[7];
    p[0] = p[0] + p[2];
    p[1] = p[1] + p[3];
    z_s[tid] = p[0] + p[1];
  }
  __syncthreads();

  // block mass, one thread per expert, rows ascending
  if (tid < E) {
    double acc = 0.0;
    for (int r = 0; r < R; ++r) acc = acc + u_s[r][tid] / z_s[r];
    mass_s[tid] = acc;
  }
  __syncthreads();

  // rank of each expert under (mass desc, id asc)
  if (tid < E) {
    const double me = mass_s[tid];
    int rank = 0;
    for (int e = 0; e < E; ++e) {
      const double mo = mass_s[e];
      rank += (mo > me) || (mo == me && e < tid);
    }
    rank_s[tid] = rank;
    order_s[rank] = tid;
  }
  __syncthreads();

  // sequential prefix sum in mass order (one lane; this order is the contract)
  if (tid == 0) {
    double c = 0.0;
    for (int i = 0; i < E; ++i) {
      c = c + mass_s[order_s[i]];
      cum_s[i] = c;
    }
    m_s = E;
  }
  __syncthreads();
  if (tau < 1.0f && tid < E) {
    const double thr = static_cast<double>(tau) * cum_s[E - 1];
    // cum is non-decreasing, so exactly one index is the first to reach thr
    if (cum_s[tid] >= thr && (tid == 0 || cum_s[tid - 1] < thr)) m_s = tid + 1;
  }
  __syncthreads();
  const int m = m_s;

  if (coreset_ids && tid < E) coreset_ids[(size_t)b * E + tid] = tid < m ? order_s[tid] : -1;
  if (coreset_size && tid == 0) coreset_size[b] = m;
  if (block_mass && tid < E) block_mass[(size_t)b * E + tid] = mass_s[tid];

  // restricted top-k: one wave per row; lane holds experts lane + 64*s
  for (int r = wave; r < R; r += 4) {
    const int row = b * R + r;
    float cl[4];
    int ce[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane + 64 * s;
      const bool ok = e < E && rank_s[e] < m;
      ce[s] = ok ? e : E;
      cl[s] = ok ? l_s[r][e] : 0.0f;
    }
    int chosen[8];
    int k_eff = 0;
    for (int j = 0; j < K; ++j) {
      float bl = 0.0f;
      int be = E;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (better(cl[s], ce[s], bl, be, E)) {
          bl = cl[s];
          be = ce[s];
        }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ol = shfl_xor_f(bl, off);
        const int oe = shfl_xor_i(be, off);
        if (better(ol, oe, bl, be, E)) {
          bl = ol;
          be = oe;
        }
      }
      if (be >= E) break;  // coreset exhausted
      chosen[j] = be;
      k_eff = j + 1;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (ce[s] == be) ce[s] = E;  // taken
    }
    if (lane == 0) {
      double U = 0.0;
      for (int j = 0; j < k_eff; ++j) U = U + u_s[r][chosen[j]];
      for (int j = 0; j < K; ++j) {
        const bool ok = j < k_eff;
        topk[(size_t)row * K + j] = ok ? chosen[j] : -1;
        gates[(size_t)row * K + j] = ok ? static_cast<float>(u_s[r][chosen[j]] / U) : 0.0f;
      }
    }
  }
}

hipError_t launch_route_blocks(const Plan& p, float tau, hipStream_t s) {
  route_block_kernel<<<p.B, 256, 0, s>>>(p.logits, p.R, p.E, p.K, tau, p.topk, p.gates,
                                         p.coreset_ids, p.coreset_size, p.block_mass);
  return hipGetLastError();
}

}  // namespace cmoe
