// expert_gemm.hip -- grouped expert GEMMs on MFMA (gfx950).
//
//   expert_up   : h = silu(X_e W_gate^T) * (X_e W_up^T)   for every work tile
//   expert_down : y = h W2_e^T                            for every work tile
//
// The routed experts and the shared expert are SwiGLU FFNs (Clover-35B-A3B-
// Preview CMF model card, introduction: 256 routed experts, top-8, plus a
// shared expert).  Expert weights are streamed from HBM exactly once per
// work tile; with one 32-row block per call a touched expert sees about two
// rows, so this is a weight-streaming (HBM-bound) kernel and the matrix cores
// only need to keep up.
//
// Work decomposition.  The permutation kernel leaves a list of tiles
// (expert, first pair, up to 64 pairs).  A workgroup of 4 waves takes one
// tile and one slice of output columns:
//   expert_up   : 32 h columns; wave w computes 8 gate and the matching 8 up
//                 columns as one 16-column MFMA tile, so SwiGLU pairs lanes
//                 l and l+8 of the accumulator;
//   expert_down : 64 y columns, 16 per wave.
// Each wave streams its 16 weight rows straight from HBM into MFMA operand
// registers (no LDS: every weight byte is used by exactly one wave), and the
// gathered activation rows come from L2.  Rows of a tile beyond its count are
// zero-filled on load and never stored.
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16, checked on gfx950): lane l
// supplies A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16], and receives
// D[4*(l/16) + v][l%16], v = 0..3.  The k order inside a step only has to be
// the same for A and B.
//
// Storage formats: bf16 weights with bf16 activations; fp32 with fp32 (16x16x4
// fp32 MFMA, four per 16-wide k step); OCP e4m3 weights with fp32 scales per
// 128x128 block and bf16 activations (InfiniLM PR #584, "Benchmark": E4M3
// 128x128 weight blocks with BF16 activations).  fp8 codes are converted to
// bf16 exactly in registers, each 128-deep k block is accumulated separately
// and added into the result times its block scale.
#include "cmoe_device.h"
#include "cmoe_launch.h"

namespace cmoe {

enum class WFmt { BF16, F32, FP8 };

// ---------------------------------------------------------------------------
// fragments: what one lane loads for one k step
// ---------------------------------------------------------------------------
template <WFmt F>
struct Frag;

template <>
struct Frag<WFmt::BF16> {
  static constexpr int kStep = 32;  // k per MFMA step
  static constexpr int kLane = 8;   // elements per lane per step
  using A = u32x4;                  // 8 bf16
  using B = u32x4;
  using AT = uint16_t;
  using WT = uint16_t;
  static __device__ __forceinline__ A load_a(const AT* p) { return *reinterpret_cast<const u32x4*>(p); }
  static __device__ __forceinline__ B load_b(const WT* p) { return *reinterpret_cast<const u32x4*>(p); }
  static __device__ __forceinline__ A zero_a() { return u32x4{0u, 0u, 0u, 0u}; }
  static __device__ __forceinline__ f32x4 mma(A a, B b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Frag<WFmt::F32> {
  static constexpr int kStep = 16;
  static constexpr int kLane = 4;
  using A = f32x4;
  using B = f32x4;
  using AT = float;
  using WT = float;
  static __device__ __forceinline__ A load_a(const AT* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ B load_b(const WT* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ A zero_a() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
  static __device__ __forceinline__ f32x4 mma(A a, B b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

template <>
struct Frag<WFmt::FP8> {
  static constexpr int kStep = 32;
  static constexpr int kLane = 8;
  using A = u32x4;  // 8 bf16
  using B = u32x2;  // 8 e4m3 codes
  using AT = uint16_t;
  using WT = uint8_t;
  static __device__ __forceinline__ A load_a(const AT* p) { return *reinterpret_cast<const u32x4*>(p); }
  static __device__ __forceinline__ B load_b(const WT* p) { return *reinterpret_cast<const u32x2*>(p); }
  static __device__ __forceinline__ A zero_a() { return u32x4{0u, 0u, 0u, 0u}; }
  static __device__ __forceinline__ u32x4 widen(B b) {
    // exact e4m3 -> bf16 (scale 1.0), two codes per instruction
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[0], 1.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[0], 1.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[1], 1.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[1], 1.0f, true);
    return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
  }
  static __device__ __forceinline__ f32x4 mma(A a, B b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, widen(b)), c, 0, 0,
                                                   0);
  }
};

// ---------------------------------------------------------------------------
// one wave: acc[mt] (16 rows x 16 cols) = sum_k A_mt[:, k] * W[col, k] over
// k in [0, K).  wrow: pointer to this lane's weight row at its k offset;
// arow[mt]: this lane's activation row at its k offset, or nullptr (zeros).
// For fp8, wscale points at this lane's row of 128x128 block scales.
// ---------------------------------------------------------------------------
template <WFmt F, int MT>
__device__ __forceinline__ void wave_gemm(const typename Frag<F>::WT* __restrict__ wrow,
                                          const typename Frag<F>::AT* const (&arow)[MT], int K,
                                          const float* __restrict__ wscale, f32x4 (&acc)[MT]) {
  using Fr = Frag<F>;
  constexpr int U = 128 / Fr::kStep;  // steps per 128-deep k block
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += 128) {
    typename Fr::B b[U];
    typename Fr::A a[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = Fr::load_b(wrow + k0 + u * Fr::kStep);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int u = 0; u < U; ++u)
        a[mt][u] = arow[mt] ? Fr::load_a(arow[mt] + k0 + u * Fr::kStep) : Fr::zero_a();
    if constexpr (F == WFmt::FP8) {
      const float s = wscale[k0 / 128];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < U; ++u) t = Fr::mma(a[mt][u], b[u], t);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mt][v] = __builtin_fmaf(s, t[v], acc[mt][v]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = Fr::mma(a[mt][u], b[u], acc[mt]);
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_act(T* p, float v);
template <>
__device__ __forceinline__ void store_act<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_act<float>(float* p, float v) { *p = v; }

struct UpArgs {
  const void* x;
  const void* w13;
  const float* w13_scale;
  const void* sw13;
  const float* sw13_scale;
  const Tile* tiles;
  const int32_t* tile_count;
  const int32_t* pair_row;
  void* h;
  int N, H, E, I, Is, K, n_slices;
};

template <WFmt F, int MT>
__device__ __forceinline__ void up_tile(const UpArgs& a, const Tile& t, int slice) {
  using Fr = Frag<F>;
  using AT = typename Fr::AT;
  using WT = typename Fr::WT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const bool shared = t.expert == a.E;
  const int inter = shared ? a.Is : a.I;
  const int i0 = slice * kUpCols + wave * 8;
  const int wr = col < 8 ? i0 + col : inter + i0 + col - 8;  // gate row / up row
  const WT* W = shared ? static_cast<const WT*>(a.sw13)
                       : static_cast<const WT*>(a.w13) + (size_t)t.expert * 2 * a.I * a.H;
  const WT* wrow = W + (size_t)wr * a.H + kg * Fr::kLane;
  const float* wscale = nullptr;
  if constexpr (F == WFmt::FP8) {
    const float* S = shared ? a.sw13_scale : a.w13_scale + (size_t)t.expert * (2 * a.I / 128) * (a.H / 128);
    wscale = S + (size_t)(wr / 128) * (a.H / 128);
  }
  const AT* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + col;
    const int src = m < t.rows ? (shared ? t.start + m : a.pair_row[t.start + m]) : -1;
    arow[mt] = src >= 0 ? static_cast<const AT*>(a.x) + (size_t)src * a.H + kg * Fr::kLane : nullptr;
  }
  f32x4 acc[MT];
  wave_gemm<F, MT>(wrow, arow, a.H, wscale, acc);

  AT* h = static_cast<AT*>(a.h) +
          (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float g = acc[mt][v];
      const float up = shfl_xor_f(g, 8);
      const int m = mt * 16 + kg * 4 + v;
      if (col < 8 && m < t.rows) store_act<AT>(h + (size_t)m * inter + i0 + col, silu(g) * up);
    }
}

template <WFmt F>
__global__ __launch_bounds__(256) void expert_up_kernel(UpArgs a) {
  const int slot = blockIdx.x / a.n_slices, slice = blockIdx.x % a.n_slices;
  if (slot >= *a.tile_count) return;
  const Tile t = a.tiles[slot];
  const int inter = t.expert == a.E ? a.Is : a.I;
  if (slice * kUpCols >= inter) return;
  switch ((t.rows + 15) >> 4) {
    case 1: up_tile<F, 1>(a, t, slice); break;
    case 2: up_tile<F, 2>(a, t, slice); break;
    case 3: up_tile<F, 3>(a, t, slice); break;
    default: up_tile<F, 4>(a, t, slice); break;
  }
}

struct DownArgs {
  const void* w2;
  const float* w2_scale;
  const void* sw2;
  const float* sw2_scale;
  const Tile* tiles;
  const int32_t* tile_count;
  const void* h;
  float* y;
  int N, H, E, I, Is, K, n_slices;
};

template <WFmt F, int MT>
__device__ __forceinline__ void down_tile(const DownArgs& a, const Tile& t, int slice) {
  using Fr = Frag<F>;
  using AT = typename Fr::AT;
  using WT = typename Fr::WT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const bool shared = t.expert == a.E;
  const int inter = shared ? a.Is : a.I;
  const int c0 = slice * kDownCols + wave * 16;
  const WT* W = shared ? static_cast<const WT*>(a.sw2)
                       : static_cast<const WT*>(a.w2) + (size_t)t.expert * a.H * a.I;
  const WT* wrow = W + (size_t)(c0 + col) * inter + kg * Fr::kLane;
  const float* wscale = nullptr;
  if constexpr (F == WFmt::FP8) {
    const float* S = shared ? a.sw2_scale : a.w2_scale + (size_t)t.expert * (a.H / 128) * (a.I / 128);
    wscale = S + (size_t)((c0 + col) / 128) * (inter / 128);
  }
  const AT* hbase = static_cast<const AT*>(a.h) +
                    (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
  const AT* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + col;
    arow[mt] = m < t.rows ? hbase + (size_t)m * inter + kg * Fr::kLane : nullptr;
  }
  f32x4 acc[MT];
  wave_gemm<F, MT>(wrow, arow, inter, wscale, acc);

  float* y = a.y + ((shared ? (size_t)a.N * a.K : 0) + (size_t)t.start) * a.H;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = mt * 16 + kg * 4 + v;
      if (m < t.rows) y[(size_t)m * a.H + c0 + col] = acc[mt][v];
    }
}

template <WFmt F>
__global__ __launch_bounds__(256) void expert_down_kernel(DownArgs a) {
  const int slot = blockIdx.x / a.n_slices, slice = blockIdx.x % a.n_slices;
  if (slot >= *a.tile_count) return;
  const Tile t = a.tiles[slot];
  switch ((t.rows + 15) >> 4) {
    case 1: down_tile<F, 1>(a, t, slice); break;
    case 2: down_tile<F, 2>(a, t, slice); break;
    case 3: down_tile<F, 3>(a, t, slice); break;
    default: down_tile<F, 4>(a, t, slice); break;
  }
}

static WFmt fmt_of(const Plan& p) {
  if (p.wt == CMOE_FP8_E4M3) return WFmt::FP8;
  if (p.wt == CMOE_F32) return WFmt::F32;
  return WFmt::BF16;
}

hipError_t launch_expert_up(const Plan& p, const cmoe_weights& w, const void* x, hipStream_t s) {
  UpArgs a;
  a.x = x;
  a.w13 = w.w13;
  a.w13_scale = w.w13_scale;
  a.sw13 = w.shared_w13;
  a.sw13_scale = w.shared_w13_scale;
  a.tiles = p.tiles;
  a.tile_count = p.tile_count;
  a.pair_row = p.pair_row;
  a.h = p.h;
  a.N = p.N;
  a.H = p.H;
  a.E = p.E;
  a.I = p.I;
  a.Is = p.Is;
  a.K = p.K;
  a.n_slices = (p.I > p.Is ? p.I : p.Is) / kUpCols;
  const unsigned grid = (unsigned)p.max_tiles * (unsigned)a.n_slices;
  switch (fmt_of(p)) {
    case WFmt::BF16: expert_up_kernel<WFmt::BF16><<<grid, 256, 0, s>>>(a); break;
    case WFmt::F32: expert_up_kernel<WFmt::F32><<<grid, 256, 0, s>>>(a); break;
    case WFmt::FP8: expert_up_kernel<WFmt::FP8><<<grid, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_expert_down(const Plan& p, const cmoe_weights& w, hipStream_t s) {
  DownArgs a;
  a.w2 = w.w2;
  a.w2_scale = w.w2_scale;
  a.sw2 = w.shared_w2;
  a.sw2_scale = w.shared_w2_scale;
  a.tiles = p.tiles;
  a.tile_count = p.tile_count;
  a.h = p.h;
  a.y = p.y;
  a.N = p.N;
  a.H = p.H;
  a.E = p.E;
  a.I = p.I;
  a.Is = p.Is;
  a.K = p.K;
  a.n_slices = p.H / kDownCols;
  const unsigned grid = (unsigned)p.max_tiles * (unsigned)a.n_slices;
  switch (fmt_of(p)) {
    case WFmt::BF16: expert_down_kernel<WFmt::BF16><<<grid, 256, 0, s>>>(a); break;
    case WFmt::F32: expert_down_kernel<WFmt::F32><<<grid, 256, 0, s>>>(a); break;
    case WFmt::FP8: expert_down_kernel<WFmt::FP8><<<grid, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace cmoe
