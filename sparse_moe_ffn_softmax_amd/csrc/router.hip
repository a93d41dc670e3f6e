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
// tile, each thread keeping TR x TE independent accumulators (rows strided by
// 8: the 8 row groups of a 16-lane LDS read then hit 8 different bank
// groups, where contiguous row quartets put two row groups on each).  Operands are
// staged through LDS in slices of KB positions per chunk.  With NBUF = 2 the
// slices are double-buffered (the global loads of slice s+1 are in flight
// while slice s is consumed); with NBUF = 1 one slice covers the whole chunk,
// so every load of the workgroup is issued at once and the kernel waits on a
// single memory round trip (the few-row case is latency-bound).  The
// register tile only changes which thread runs a chain, never the order
// inside a chain.
#include "cmoe_device.h"
#include "cmoe_launch.h"

#pragma clang fp contract(off)

namespace cmoe {

template <typename XT>
struct XVec;
template <>
struct XVec<uint16_t> {  // 8 bf16 per 16-byte load
  static constexpr int kN = 8;
  static __device__ __forceinline__ void widen(const u32x4& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct XVec<float> {  // 4 fp32 per 16-byte load
  static constexpr int kN = 4;
  static __device__ __forceinline__ void widen(const u32x4& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
  }
};

template <int TR, int TE, int KB, int NBUF, typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int N,
                                                            int H, int E, int emajor) {
  constexpr int RT = 8 * TR;                 // rows per workgroup
  constexpr int ET = 4 * TE;                 // experts per workgroup
  constexpr int KP = KB + 4;                 // padded LDS row (breaks bank aliasing)
  constexpr int XN = XVec<XT>::kN;
  constexpr int XV = RT * 8 * KB / XN;       // x vectors per slice
  constexpr int WV = ET * 8 * KB / 4;        // w vectors per slice
  constexpr int XPT = (XV + 255) / 256;      // per thread
  constexpr int WPT = (WV + 255) / 256;
  // one LDS buffer: the x and w staging slices, and (once the k loop is
  // done) the chunk partial sums over them
  constexpr int kXs = NBUF * 8 * RT * KP, kWs = NBUF * 8 * ET * KP, kPart = 8 * RT * (ET + 1);
  __shared__ float smem[(kXs + kWs) > kPart ? (kXs + kWs) : kPart];
  auto xs = reinterpret_cast<float(*)[8][RT][KP]>(smem);
  auto ws = reinterpret_cast<float(*)[8][ET][KP]>(smem + kXs);
  auto part = reinterpret_cast<float(*)[RT][ET + 1]>(smem);

  const int tid = threadIdx.x;
  const int c = tid >> 5;  // chunk run by this thread
  const int q = tid & 31;
  const int rq = q & 7;    // row group: rows rq, rq + 8, ..., rq + 8(TR-1)
  const int eq = q >> 3;   // expert group: experts eq*TE .. eq*TE + TE-1
  // emajor: expert slices along x, row groups along y (see launch_shape)
  const int row0 = (emajor ? blockIdx.y : blockIdx.x) * RT;
  const int e0 = (emajor ? blockIdx.x : blockIdx.y) * ET;
  const int L = H / 8;     // chunk length, a multiple of KB
  const int S = L / KB;    // slices (1 when NBUF == 1)

  // Staging loads are unconditional (rows past N and experts past E read the
  // last valid row or expert, and are zeroed when parked in LDS): the
  // compiler counts outstanding loads to place its waits, and a conditional
  // load makes it wait for every load in flight.
  // kDepth register sets of staged loads: on the fixed 16-slice schedule the
  // loads of slices s+1 .. s+kDepth are in flight while slice s is consumed
  constexpr int kDepth = NBUF > 1 ? 3 : 1;
  u32x4 xr_[kDepth][XPT], wr_[kDepth][WPT];
  auto fetch = [&](int s, int set = 0) {
    auto& xr = xr_[set];
    auto& wr = wr_[set];
    const int kb = s * KB;
#pragma unroll
    for (int t = 0; t < XPT; ++t) {
      const int v = tid + t * 256;
      if (XV % 256 == 0 || v < XV) {
        const int kk = (v % (KB / XN)) * XN, rest = v / (KB / XN), r = rest % RT, cc = rest / RT;
        const int row = min(row0 + r, N - 1);
        xr[t] = *reinterpret_cast<const u32x4*>(x + (size_t)row * H + cc * L + kb + kk);
      }
    }
#pragma unroll
    for (int t = 0; t < WPT; ++t) {
      const int v = tid + t * 256;
      if (WV % 256 == 0 || v < WV) {
        const int kk = (v % (KB / 4)) * 4, rest = v / (KB / 4), e = rest % ET, cc = rest / ET;
        const int ex = min(e0 + e, E - 1);
        wr[t] = *reinterpret_cast<const u32x4*>(w + (size_t)ex * H + cc * L + kb + kk);
      }
    }
  };
  auto stash = [&](int buf, int set = 0) {
    auto& xr = xr_[set];
    auto& wr = wr_[set];
#pragma unroll
    for (int t = 0; t < XPT; ++t) {
      const int v = tid + t * 256;
      if (XV % 256 == 0 || v < XV) {
        const int kk = (v % (KB / XN)) * XN, rest = v / (KB / XN), r = rest % RT, cc = rest / RT;
        float f[XN];
        XVec<XT>::widen(row0 + r < N ? xr[t] : u32x4{0u, 0u, 0u, 0u}, f);
#pragma unroll
        for (int i = 0; i < XN; ++i) xs[buf][cc][r][kk + i] = f[i];
      }
    }
#pragma unroll
    for (int t = 0; t < WPT; ++t) {
      const int v = tid + t * 256;
      if (WV % 256 == 0 || v < WV) {
        const int kk = (v % (KB / 4)) * 4, rest = v / (KB / 4), e = rest % ET, cc = rest / ET;
        const bool ok = e0 + e < E;
#pragma unroll
        for (int i = 0; i < 4; ++i) ws[buf][cc][e][kk + i] = ok ? __uint_as_float(wr[t][i]) : 0.0f;
      }
    }
  };

  float acc[TR][TE];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.0f;

  auto compute = [&](int buf) {
#pragma unroll 4
    for (int k = 0; k < KB; k += 4) {
      f32x4 xv[TR], wv[TE];
#pragma unroll
      for (int i = 0; i < TR; ++i) xv[i] = *reinterpret_cast<const f32x4*>(&xs[buf][c][rq + 8 * i][k]);
#pragma unroll
      for (int j = 0; j < TE; ++j) wv[j] = *reinterpret_cast<const f32x4*>(&ws[buf][c][eq * TE + j][k]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
          for (int j = 0; j < TE; ++j) acc[i][j] = __builtin_fmaf(xv[i][kk], wv[j][kk], acc[i][j]);
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  if constexpr (NBUF > 1) {
    if (S == 16) {
      // fully unrolled, so that every register set has a fixed name and the
      // waits count exactly: slice s+kDepth is fetched into the set slice s
      // was parked from
      static_for<1, kDepth>([&](auto J) { fetch(J, J); });
      static_for<0, 16>([&](auto J) {
        constexpr int st = decltype(J)::value;
        if constexpr (st + kDepth < 16) fetch(st + kDepth, (st + kDepth) % kDepth);
        compute(st & 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (st + 1 < 16) {
          stash((st + 1) & 1, (st + 1) % kDepth);
          __syncthreads();
        }
      });
    } else {
      // slice s+1's loads are in flight while slice s feeds the FMAs; it is
      // parked in the other buffer only after them (hoisted above them, its
      // wait for the loads would leave nothing to overlap), and the last
      // slice is peeled so that the loop body has no conditional load
      for (int s = 0; s + 1 < S; ++s) {
        fetch(s + 1);
        compute(s & 1);
        __builtin_amdgcn_sched_barrier(0);
        stash((s + 1) & 1);
        __syncthreads();
      }
      compute((S - 1) & 1);
    }
  } else {
    compute(0);
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) part[c][rq + 8 * i][eq * TE + j] = acc[i][j];
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

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2.  emajor puts the expert slices along x: the row groups
// of one slice then have ids a multiple of the slice count apart, which is a
// multiple of 8 for E = 256, so they share an XCD and its L2 holds that
// slice of Wr for all of them; x is then fetched by every XCD.  That is the
// cheaper side when there are few rows (one 32-row block: 3 MB instead of
// 8 MB from HBM), the dearer one with many (2048 rows: 66 MB instead of 24).
template <int TR, int TE, int KB, int NBUF = 2>
static void launch_shape(const Plan& p, const void* x, const float* w, const float* b, bool emajor,
                         hipStream_t s) {
  const unsigned rg = (p.N + 8 * TR - 1) / (8 * TR), es = (p.E + 4 * TE - 1) / (4 * TE);
  const dim3 grid = emajor ? dim3(es, rg) : dim3(rg, es);
  if (p.act == CMOE_BF16)
    router_logits_kernel<TR, TE, KB, NBUF, uint16_t><<<grid, 256, 0, s>>>(
        static_cast<const uint16_t*>(x), w, b, p.logits, p.N, p.H, p.E, emajor);
  else
    router_logits_kernel<TR, TE, KB, NBUF, float><<<grid, 256, 0, s>>>(
        static_cast<const float*>(x), w, b, p.logits, p.N, p.H, p.E, emajor);
}

hipError_t launch_router(const Plan& p, const void* x, const float* router_w,
                         const float* router_b, hipStream_t s) {
  // chunk length H/8 is a multiple of 16 (H is a multiple of 128)
  const int L = p.H / 8;
  if (p.N <= 256) {
    // few rows (one block per call): one accumulator per thread keeps
    // enough workgroups in flight; whole chunks in one slice where they fit
    if (L == 256) launch_shape<1, 1, 256, 1>(p, x, router_w, router_b, true, s);
    else if (L == 128) launch_shape<1, 1, 128, 1>(p, x, router_w, router_b, true, s);
    else if (L % 64 == 0) launch_shape<1, 1, 64>(p, x, router_w, router_b, true, s);
    else if (L % 32 == 0) launch_shape<1, 1, 32>(p, x, router_w, router_b, true, s);
    else launch_shape<1, 1, 16>(p, x, router_w, router_b, true, s);
  } else {
    // many rows: 4x4 register tiles, 16-position slices (about 60 KiB of
    // LDS, so two workgroups share a CU)
    launch_shape<4, 4, 16>(p, x, router_w, router_b, false, s);
  }
  return hipGetLastError();
}

}  // namespace cmoe
