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

// ---------------------------------------------------------------------------
// Many rows: the same chains on the matrix cores.  v_mfma_f32_32x32x1_2b_f32
// has depth 1: each step adds one product to each of its 2 x 32 x 32 fp32
// accumulators, and on gfx950 that step rounds exactly as an fp32 fma does
// (checked bit for bit against v_fma_f32 chains, with operands of ordinary
// and of denormal-range magnitude).  A chain of these MFMAs over ascending h
// is therefore the chunk's fma chain itself, for 2048 (row, expert, chunk)
// chains at once.
//
// A workgroup of 8 waves owns 64 rows x 32 experts.  Wave w takes the row
// block w / 4 and the chunk pair (w % 4, w % 4 + 4), one chunk per MFMA
// block: lane l supplies x[row l % 32] and Wr[expert l % 32] of chunk
// w % 4 + 4 (l / 32).  Output register v of lane l is block v / 16, row
// 8 ((v % 16) / 4) + 4 (l / 32) + v % 4, expert l % 32 (checked on gfx950),
// so lane l adds its chunk pair (p_c + p_{c+4}, the tree's first level) in
// registers; the other two levels run after an exchange through LDS.
//
// Operands are staged through LDS P positions of every chunk at a time
// (coalesced 16-byte loads through registers, double-buffered: the loads of
// stage s+1 are in flight while stage s feeds the MFMAs).  Read from global
// memory lane by lane instead, every load touches 64 different cache lines,
// and the per-CU fetch rate, not the matrix cores, sets the pace.  x keeps
// its storage type in LDS; rows are padded to 16 bytes past a multiple of
// 256, so the 32 rows a half-wave reads fall in distinct bank groups.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(32))) float f32x32;

template <typename XT, int P>
struct RouterStage {
  static constexpr int kXRow = 8 * P * (int)sizeof(XT) + 16;   // bytes per staged x row (8 chunks)
  static constexpr int kWRow = 8 * P * 4 + 16;                 // bytes per staged Wr row
  static constexpr int kBytes = 64 * kXRow + 32 * kWRow;       // one buffer
  static constexpr int kXV = P * (int)sizeof(XT) / 16;          // 16-byte vectors per row and chunk
  static constexpr int kWV = P * 4 / 16;
  static constexpr int kNX = 64 * 8 * kXV, kNW = 32 * 8 * kWV;  // vectors per stage
  static constexpr int kVPT = (kNX + kNW) / 512;                // per thread
  static_assert(kNX % 512 == 0 && kNW % 512 == 0, "whole rounds of 512 vectors");
  static_assert(2 * kBytes <= 160 * 1024 && 2 * kBytes >= 4 * 64 * 33 * 4, "LDS budget");
};

template <typename XT, int P>
__global__ __launch_bounds__(512) void router_mfma_kernel(const XT* __restrict__ x, const float* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int N, int H, int E) {
  using RS = RouterStage<XT, P>;
  constexpr int XN = XVec<XT>::kN;   // x values per 16-byte vector
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * RS::kBytes];
  auto part = reinterpret_cast<float(*)[64][33]>(smem);  // after the chains: s_c = p_c + p_{c+4}
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = wave >> 2, cp = wave & 3;
  const int blk = lane >> 5, i = lane & 31;
  const int row0 = blockIdx.x * 64, e0 = blockIdx.y * 32;
  const int L = H / 8, NS = L / P;   // chunk length and its stages
  const int c = cp + 4 * blk;        // this lane's chunk

  // staging: vector v = tid + 512 t; the first kNX are x (row, chunk, piece),
  // the rest Wr.  Rows past N and experts past E read the last valid one
  // (their results are not stored).
  u32x4 reg[RS::kVPT];
  auto gload = [&](int st) {
#pragma unroll
    for (int t = 0; t < RS::kVPT; ++t) {
      const int v = tid + 512 * t;
      if (t < RS::kNX / 512) {
        const int k = v % RS::kXV, rc = v / RS::kXV, cc = rc & 7, r = rc >> 3;
        const int row = min(row0 + r, N - 1);
        reg[t] = *reinterpret_cast<const u32x4*>(x + (size_t)row * H + (size_t)cc * L + st * P + k * XN);
      } else {
        const int vw = v - RS::kNX;
        const int k = vw % RS::kWV, ec = vw / RS::kWV, cc = ec & 7, e = ec >> 3;
        const int ex = min(e0 + e, E - 1);
        reg[t] = *reinterpret_cast<const u32x4*>(w + (size_t)ex * H + (size_t)cc * L + st * P + k * 4);
      }
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* base = smem + buf * RS::kBytes;
#pragma unroll
    for (int t = 0; t < RS::kVPT; ++t) {
      const int v = tid + 512 * t;
      if (t < RS::kNX / 512) {
        const int k = v % RS::kXV, rc = v / RS::kXV, cc = rc & 7, r = rc >> 3;
        *reinterpret_cast<u32x4*>(base + r * RS::kXRow + (cc * RS::kXV + k) * 16) = reg[t];
      } else {
        const int vw = v - RS::kNX;
        const int k = vw % RS::kWV, ec = vw / RS::kWV, cc = ec & 7, e = ec >> 3;
        *reinterpret_cast<u32x4*>(base + 64 * RS::kXRow + e * RS::kWRow + (cc * RS::kWV + k) * 16) = reg[t];
      }
    }
  };

  f32x32 acc = f32x32{};
  // this lane's operands inside a staged buffer: its row's and its expert's chunk c
  const int xoff = (32 * rb + i) * RS::kXRow + c * P * (int)sizeof(XT);
  const int woff = 64 * RS::kXRow + i * RS::kWRow + c * P * 4;
  auto compute = [&](int buf) {
    const uint8_t* base = smem + buf * RS::kBytes;
#pragma unroll
    for (int p = 0; p < P; p += 8) {
      float xv[8];
#pragma unroll
      for (int j = 0; j < 8 / XN; ++j)
        XVec<XT>::widen(*reinterpret_cast<const u32x4*>(base + xoff + (p + j * XN) * (int)sizeof(XT)), xv + j * XN);
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(base + woff + p * 4);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(base + woff + p * 4 + 16);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(xv[k], __uint_as_float(k < 4 ? w0[k] : w1[k - 4]), acc, 0, 0,
                                                   0);
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < NS; ++st) {
    if (st + 1 < NS) gload(st + 1);
    // (keeps the next stage's loads above the MFMAs: sunk to their stores,
    // each stage would wait a full memory round trip)
    __builtin_amdgcn_sched_barrier(0);
    compute(st & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < NS) lstore((st + 1) & 1);
    __syncthreads();
  }
  // first tree level in registers, then the exchange (over the staging buffers)
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 32 * rb + 8 * (v >> 2) + 4 * blk + (v & 3);
    part[cp][r][i] = acc[v] + acc[v + 16];
  }
  __syncthreads();
  for (int o = tid; o < 64 * 32; o += 512) {
    const int r = o >> 5, e = o & 31;
    const int rr = row0 + r, ee = e0 + e;
    if (rr >= N || ee >= E) continue;
    float l = (part[0][r][e] + part[2][r][e]) + (part[1][r][e] + part[3][r][e]);
    if (bias) l = l + bias[ee];
    logits[(size_t)rr * E + ee] = l;
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

template <typename XT>
static void launch_mfma(const Plan& p, const void* x, const float* w, const float* b, hipStream_t s) {
  const dim3 grid((p.N + 63) / 64, (p.E + 31) / 32);
  const XT* xt = static_cast<const XT*>(x);
  // 32 positions per stage where the chunk length allows it and the buffers
  // fit (bf16 x); else 16 (H/8 is a multiple of 16)
  if constexpr (sizeof(XT) == 2) {
    if ((p.H / 8) % 32 == 0) {
      router_mfma_kernel<XT, 32><<<grid, 512, 0, s>>>(xt, w, b, p.logits, p.N, p.H, p.E);
      return;
    }
  }
  router_mfma_kernel<XT, 16><<<grid, 512, 0, s>>>(xt, w, b, p.logits, p.N, p.H, p.E);
}

hipError_t launch_router(const Plan& p, const void* x, const float* router_w,
                         const float* router_b, hipStream_t s) {
  // chunk length H/8 is a multiple of 16 (H is a multiple of 128)
  const int L = p.H / 8;
  if (p.N <= 128) {
    // few rows (up to four 32-row blocks): one accumulator per thread keeps
    // enough workgroups in flight; whole chunks in one slice where they fit
    // (at 256 rows the 4x4 tiles below measured 21 against 32 us)
    if (L == 256) launch_shape<1, 1, 256, 1>(p, x, router_w, router_b, true, s);
    else if (L == 128) launch_shape<1, 1, 128, 1>(p, x, router_w, router_b, true, s);
    else if (L % 64 == 0) launch_shape<1, 1, 64>(p, x, router_w, router_b, true, s);
    else if (L % 32 == 0) launch_shape<1, 1, 32>(p, x, router_w, router_b, true, s);
    else launch_shape<1, 1, 16>(p, x, router_w, router_b, true, s);
  } else if ((long long)((p.N + 63) / 64) * ((p.E + 31) / 32) < 128) {
    // a few hundred rows: the matrix-core grid would leave most CUs idle
    // (measured at 512 rows: 24 us there, 19 us here); 4x4 register tiles,
    // 16-position slices (about 60 KiB of LDS, so two workgroups share a CU)
    launch_shape<4, 4, 16>(p, x, router_w, router_b, false, s);
  } else {
    // many rows: the matrix-core chains.  Row tiles along x: the expert
    // tiles of one row tile have linear ids a multiple of the row-tile count
    // apart, so with a multiple of 8 row tiles they share an XCD and x is
    // fetched by one XCD only; Wr (2 MB at E = 256) is fetched by all
    if (p.act == CMOE_BF16) launch_mfma<uint16_t>(p, x, router_w, router_b, s);
    else launch_mfma<float>(p, x, router_w, router_b, s);
  }
  return hipGetLastError();
}

}  // namespace cmoe
