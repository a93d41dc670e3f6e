// expert_gemm.hip -- grouped expert GEMMs on MFMA (gfx950).
//
//   expert_up   : h = silu(X_e W_gate^T) * (X_e W_up^T)   for every work tile
//   expert_down : y = h W2_e^T                            for every work tile
//
// The routed experts and the shared expert are SwiGLU FFNs (Clover-35B-A3B-
// Preview CMF model card, introduction: 256 routed experts, eight per token,
// and one shared expert).  Expert weights are streamed from HBM exactly once per
// work tile; with one 32-row block per call a touched expert sees about two
// rows, so this is a weight-streaming (HBM-bound) kernel and the matrix cores
// only need to keep up.
//
// Work decomposition.  The permutation leaves a list of tiles (expert, first
// pair, row count).  These kernels run the calls whose tiles hold at most 16
// rows (one MFMA row tile) and whose experts see only a few rows on average:
// one block, decode, verification, and a few blocks per call for bf16 and
// 4-bit weights (fp8 weights move to 32-row tiles from two rows per expert on
// average).  Other calls run the LDS-tiled kernels of expert_tiled.hip.  A
// workgroup takes one tile and one slice of output columns:
//   expert_up   : 4 waves, 8 h columns = one 16-column MFMA tile of 8 gate
//                 and the matching 8 up columns (SwiGLU pairs lanes l and l+8
//                 of the accumulator), 64 KiB of bf16 weights; the waves split
//                 the hidden dimension and their partial sums meet in LDS,
//                 added in wave order;
//   expert_down : kDownWaves = 2 waves, 32 y columns, 16 per wave (32 KiB of
//                 bf16 weights at I = 512; with 4 waves and 64 columns the
//                 last, partly filled round of workgroups cost about 1 us of
//                 the one-block down kernel's 55).
// 4-bit weights are four times smaller, so there a wave takes four (up) or
// four or two (down, by H) such column tiles, and each activation fragment it
// loads feeds one MFMA per column tile.
// Each wave streams its 16 weight rows straight from HBM into MFMA operand
// registers (no LDS: every weight byte is used by exactly one wave), and the
// gathered activation rows come from L2.  Rows of a tile beyond its count
// repeat its first row and are never stored.
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
// and added into the result times its block scale.  4-bit weights (the CMF
// card's "Files" section ships 4-bit experts; the stand-in format here is OCP
// MXFP4, E2M1 codes with an E8M0 scale per 32 elements) are widened to bf16
// times their power-of-two scale, which is exact, and need no per-block
// accumulator.
#include "cmoe_device.h"
#include "cmoe_launch.h"
#include "expert_frag.h"

namespace cmoe {

// ---------------------------------------------------------------------------
// one wave: acc[c][mt] (16 rows x 16 cols) = sum_k A_mt[:, k] * W_c[col, k]
// over k in [0, K), for NCT column tiles c.  wrow[c]: this lane's weight row
// of column tile c at its k offset; arow[mt]: this lane's activation row at
// its k offset; wscale[c]: that row's scales (fp8 128x128 blocks, fp4 E8M0).
//
// K is consumed in stages of 128; the loads of stage s+1 are issued before
// the MFMAs of stage s, so each wave always has a stage of weights in flight
// (two register buffers, alternating), or, on the fixed four-stage path, all
// four stages at once.
// ---------------------------------------------------------------------------
// k order inside a 128-deep stage (MFMA only needs A and B to agree on it):
// the element offset of the fragment lane group kg uses at step u.  fp8 pairs
// steps: lane group kg takes k [16kg, 16kg+16) of each 64-deep pair of steps,
// so its weights come as one 16-byte chunk per two steps instead of two
// 8-byte loads.  Every format's lane group then reads 16 weight bytes at
// byte 16kg of each 64 bytes of its row.
template <WFmt F>
__device__ __forceinline__ constexpr int a_koff(int u, int kg) {
  if constexpr (F == WFmt::FP8) return 64 * (u / 2) + 16 * kg + 8 * (u % 2);
  else return u * Frag<F>::kStepK + kg * Frag<F>::kGroupK;
}

template <WFmt F, int MT, int NCT>
struct Stage {
  static constexpr int U = 128 / Frag<F>::kStep;  // MFMA steps per stage
  typename Frag<F>::B b[NCT][U];
  typename Frag<F>::A a[MT][U];
  uint32_t sc[NCT];  // fp4: the stage's four E8M0 scale bytes of each weight row
};

// A wave computes NCT column tiles (16 weight rows each) over the same MT row
// tiles, so each activation fragment feeds NCT MFMAs.  wrow[c]: this lane's
// weight chunk 0 (at the wave's first k) of column tile c; wscale[c]: fp8:
// the row's 128x128 block scales at that k (fp32); fp4: its E8M0 bytes there.
template <WFmt F, int MT, int NCT, bool PK>
__device__ __forceinline__ void load_stage(Stage<F, MT, NCT>& st, const uint8_t* const (&wrow)[NCT],
                                           const void* const (&wscale)[NCT],
                                           const typename Frag<F>::AT* const (&arow)[MT], int k0) {
  using Fr = Frag<F>;
  using WT = typename Fr::WT;
  constexpr int U = Stage<F, MT, NCT>::U;
  constexpr int QB = kChunk<PK>;
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    if constexpr (F == WFmt::FP4) {
      // 32 codes (k 32kg .. +32 of the stage) in one chunk, and the stage's scales
      const u32x4 v = load_chunk<PK>(wrow[c] + (k0 / 128) * QB);
#pragma unroll
      for (int u = 0; u < U; ++u) st.b[c][u] = v[u];
      st.sc[c] = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(wscale[c]) + k0 / 32);
    } else if constexpr (F == WFmt::FP8) {
      // one chunk (16 codes) per pair of steps, see a_koff
#pragma unroll
      for (int j = 0; j < U / 2; ++j) {
        const u32x4 v = load_chunk<PK>(wrow[c] + (k0 / 64 + j) * QB);
        st.b[c][2 * j] = typename Fr::B{v[0], v[1]};
        st.b[c][2 * j + 1] = typename Fr::B{v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        st.b[c][u] = __builtin_bit_cast(typename Fr::B,
                                        load_chunk<PK>(wrow[c] + ((k0 + u * Fr::kStep) * (int)sizeof(WT) / 64) * QB));
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int u = 0; u < U; ++u)
      st.a[mt][u] = Fr::load_a(arow[mt] + k0 + a_koff<F>(u, 0));
}

template <WFmt F, int MT, int NCT>
__device__ __forceinline__ void mma_stage(const Stage<F, MT, NCT>& st, const void* const (&wscale)[NCT],
                                          int k0, f32x4 (&acc)[NCT][MT]) {
  using Fr = Frag<F>;
  constexpr int U = Stage<F, MT, NCT>::U;
  if constexpr (F == WFmt::FP4) {
    const int kg = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const float sc = Fr::scale_of((st.sc[c] >> (8 * kg)) & 0xFFu);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[c][mt] = Fr::mma(st.a[mt][u], st.b[c][u], sc, acc[c][mt]);
    }
  } else if constexpr (F == WFmt::FP8) {
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const float s = static_cast<const float*>(wscale[c])[k0 / 128];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < U; ++u) t = Fr::mma(st.a[mt][u], st.b[c][u], t);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c][mt][v] = __builtin_fmaf(s, t[v], acc[c][mt][v]);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[c][mt] = Fr::mma(st.a[mt][u], st.b[c][u], acc[c][mt]);
  }
}

// stages in flight per wave on the fixed four-stage path
constexpr int kDeepStages = 4;

// register words one stage holds per lane
template <WFmt F, int MT, int NCT>
constexpr int stage_words() { return (int)(sizeof(Stage<F, MT, NCT>) / 4); }

template <WFmt F, int MT, int NCT, bool PK, bool DEEP = (F == WFmt::FP4)>
__device__ __forceinline__ void wave_gemm(const uint8_t* const (&wrow)[NCT],
                                          const typename Frag<F>::AT* const (&arow)[MT], int K,
                                          const void* const (&wscale)[NCT], f32x4 (&acc)[NCT][MT]) {
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // DEEP (4-bit weights, and the fused decode kernel), K = 512 (the hidden
  // size split four ways, or the expert width): issue all four stages' loads
  // at once, then consume them in order.  Straight-line code lets the
  // compiler wait for exactly the stage it needs.  (For a large bf16 grid
  // the extra registers cost more occupancy than the deeper queue gains: the
  // two-stage loop below measured about 5% faster there.)
  if constexpr (DEEP && kDeepStages * stage_words<F, MT, NCT>() <= 160) {
    if (K == 512) {
      Stage<F, MT, NCT> st[4];
      static_for<0, kDeepStages>([&](auto S) { load_stage<F, MT, NCT, PK>(st[S], wrow, wscale, arow, S * 128); });
      static_for<0, 4>([&](auto S) {
        constexpr int next = S + kDeepStages;
        if constexpr (next < 4) load_stage<F, MT, NCT, PK>(st[next], wrow, wscale, arow, next * 128);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this stage's MFMAs
        mma_stage<F, MT, NCT>(st[S], wscale, S * 128, acc);
      });
      return;
    }
  }
  Stage<F, MT, NCT> s0, s1;
  load_stage<F, MT, NCT, PK>(s0, wrow, wscale, arow, 0);
  for (int k0 = 0; k0 < K; k0 += 256) {
    const bool two = k0 + 128 < K;
    if (two) load_stage<F, MT, NCT, PK>(s1, wrow, wscale, arow, k0 + 128);
    mma_stage<F, MT, NCT>(s0, wscale, k0, acc);
    if (!two) break;
    if (k0 + 256 < K) load_stage<F, MT, NCT, PK>(s0, wrow, wscale, arow, k0 + 256);
    mma_stage<F, MT, NCT>(s1, wscale, k0 + 128, acc);
  }
}

// column tiles per wave: 4-bit weights stream four times fewer bytes per
// tile, so a wave takes four tiles (the same bytes per workgroup as bf16)
template <WFmt F>
constexpr int up_nct() { return F == WFmt::FP4 ? 4 : 1; }
inline int down_nct(WFmt f, int H) { return f == WFmt::FP4 ? (H % 256 == 0 ? 4 : 2) : 1; }

struct UpArgs {
  const void* x;
  const void* w13;
  const void* w13_scale;
  const void* sw13;
  const void* sw13_scale;
  const Tile* tiles;
  const int32_t* tile_count;
  const int32_t* pair_row;
  void* h;
  int N, H, E, I, Is, K, n_slices;
};

template <WFmt F, int MT, int NCT, bool PK>
__device__ __forceinline__ void up_tile(const UpArgs& a, const Tile& t, int slice) {
  using Fr = Frag<F>;
  using AT = typename Fr::AT;
  using WT = typename Fr::WT;
  __shared__ f32x4 red[4][NCT][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const bool shared = t.expert == a.E;
  const int inter = shared ? a.Is : a.I;
  const int i0 = slice * kUpCols * NCT;  // column tile c: h columns i0 + 8c .. +8
  // the waves split the hidden dimension into ks equal parts (multiples of 128)
  const int ks = (a.H % 512 == 0) ? 4 : (a.H % 256 == 0) ? 2 : 1;
  const int klen = a.H / ks, kbeg = wave * klen;
  const size_t rowb = (size_t)a.H * sizeof(WT) / Fr::kPack;  // bytes per weight row
  const uint8_t* W = shared ? static_cast<const uint8_t*>(a.sw13)
                            : static_cast<const uint8_t*>(a.w13) + (size_t)t.expert * 2 * a.I * rowb;
  const size_t kbegb = (size_t)kbeg * sizeof(WT) / Fr::kPack;
  const uint8_t* wrow[NCT];
  const void* wscale[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int ic = i0 + 8 * c;
    const int wr = col < 8 ? ic + col : inter + ic + col - 8;  // gate row / up row
    // panels: column tile c is panel ic/8 (its gate rows, then its up rows)
    wrow[c] = PK ? W + (size_t)(ic / 8) * 16 * rowb + (kbegb / 64) * kChunk<PK> + 16 * lane
                 : W + (size_t)wr * rowb + kbegb + 16 * kg;
    wscale[c] = nullptr;
    if constexpr (F == WFmt::FP8) {
      const float* S = static_cast<const float*>(shared ? a.sw13_scale : a.w13_scale);
      if (!shared) S += (size_t)t.expert * (2 * a.I / 128) * (a.H / 128);
      wscale[c] = S + (size_t)(wr / 128) * (a.H / 128) + kbeg / 128;
    } else if constexpr (F == WFmt::FP4) {
      const uint8_t* S = static_cast<const uint8_t*>(shared ? a.sw13_scale : a.w13_scale);
      if (!shared) S += (size_t)t.expert * 2 * a.I * (a.H / 32);
      wscale[c] = S + (size_t)wr * (a.H / 32) + kbeg / 32;
    }
  }
  // rows past the tile's count read the tile's first row (every load is
  // unconditional, so the compiler can keep the next stage in flight); an
  // MFMA output row depends only on its own A row and those rows are never
  // stored
  const AT* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + col < t.rows ? mt * 16 + col : 0;
    const int src = shared ? t.start + m : a.pair_row[t.start + m];
    arow[mt] = static_cast<const AT*>(a.x) + (size_t)src * a.H + kbeg + a_koff<F>(0, kg);
  }
  f32x4 acc[NCT][MT];
  if (wave < ks) {
    wave_gemm<F, MT, NCT, PK>(wrow, arow, klen, wscale, acc);
  } else {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][c][mt][lane] = acc[c][mt];
  __syncthreads();
  // wave w finishes output tiles w, w+4, ... (column tile c, row tile mt): sum
  // the k parts in wave order, then SwiGLU
  AT* h = static_cast<AT*>(a.h) +
          (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
  for (int idx = wave; idx < NCT * MT; idx += 4) {
    const int c = idx % NCT, mt = idx / NCT;
    f32x4 z = red[0][c][mt][lane];
    for (int w = 1; w < ks; ++w) {
      const f32x4 o = red[w][c][mt][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) z[v] = z[v] + o[v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float g = z[v];
      const float up = shfl_xor_f(g, 8);
      const int m = mt * 16 + kg * 4 + v;
      if (col < 8 && m < t.rows) store_act<AT>(h + (size_t)m * inter + i0 + 8 * c + col, silu(g) * up);
    }
  }
}

// At least three waves per SIMD (at most 168 VGPRs): the 4-bit four-stage
// schedule otherwise takes 188 and runs two workgroups per CU; held to 168 it
// runs three without spilling (one block, 4-bit: gate/up 42.1 -> 38.7 us,
// down 25.6 -> 23.8 us; bf16 unchanged).  Four waves (128 VGPRs) spill.
constexpr int kMinWavesPerSimd = 3;

template <WFmt F, int MTMAX, int NCT, bool PK>
__global__ __launch_bounds__(256, kMinWavesPerSimd) void expert_up_kernel(UpArgs a) {
  const int slot = blockIdx.x / a.n_slices, slice = blockIdx.x % a.n_slices;
  if (slot >= *a.tile_count) return;
  const Tile t = a.tiles[slot];
  const int inter = t.expert == a.E ? a.Is : a.I;
  if (slice * kUpCols * NCT >= inter) return;
  const int mt = (t.rows + 15) >> 4;  // 1..MTMAX
  if constexpr (MTMAX >= 4) if (mt == 4) { up_tile<F, 4, NCT, PK>(a, t, slice); return; }
  if constexpr (MTMAX >= 3) if (mt == 3) { up_tile<F, 3, NCT, PK>(a, t, slice); return; }
  if constexpr (MTMAX >= 2) if (mt == 2) { up_tile<F, 2, NCT, PK>(a, t, slice); return; }
  up_tile<F, 1, NCT, PK>(a, t, slice);
}

struct DownArgs {
  const void* w2;
  const void* w2_scale;
  const void* sw2;
  const void* sw2_scale;
  const Tile* tiles;
  const int32_t* tile_count;
  const void* h;
  float* y;
  int N, H, E, I, Is, K, n_slices;
};

// acc[c][mt]: the tile's y for its MT row tiles and the NCT 16-column tiles
// of output columns starting at c0
template <WFmt F, int MT, int NCT, bool PK, bool DEEP = (F == WFmt::FP4)>
__device__ __forceinline__ void down_acc(const DownArgs& a, const Tile& t, int c0, f32x4 (&acc)[NCT][MT]) {
  using Fr = Frag<F>;
  using AT = typename Fr::AT;
  using WT = typename Fr::WT;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const bool shared = t.expert == a.E;
  const int inter = shared ? a.Is : a.I;
  const size_t rowb = (size_t)inter * sizeof(WT) / Fr::kPack;  // bytes per weight row
  const uint8_t* W = shared ? static_cast<const uint8_t*>(a.sw2)
                            : static_cast<const uint8_t*>(a.w2) + (size_t)t.expert * a.H * rowb;
  const uint8_t* wrow[NCT];
  const void* wscale[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int orow = c0 + 16 * c + col;  // W2 row = output column
    // panels: column tile c is panel (c0 + 16c) / 16
    wrow[c] = PK ? W + (size_t)((c0 + 16 * c) / 16) * 16 * rowb + 16 * lane : W + (size_t)orow * rowb + 16 * kg;
    wscale[c] = nullptr;
    if constexpr (F == WFmt::FP8) {
      const float* S = static_cast<const float*>(shared ? a.sw2_scale : a.w2_scale);
      if (!shared) S += (size_t)t.expert * (a.H / 128) * (a.I / 128);
      wscale[c] = S + (size_t)(orow / 128) * (inter / 128);
    } else if constexpr (F == WFmt::FP4) {
      const uint8_t* S = static_cast<const uint8_t*>(shared ? a.sw2_scale : a.w2_scale);
      if (!shared) S += (size_t)t.expert * a.H * (a.I / 32);
      wscale[c] = S + (size_t)orow * (inter / 32);
    }
  }
  const AT* hbase = static_cast<const AT*>(a.h) +
                    (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
  const AT* arow[MT];  // rows past the count read row 0, as in up_tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + col < t.rows ? mt * 16 + col : 0;
    arow[mt] = hbase + (size_t)m * inter + a_koff<F>(0, kg);
  }
  wave_gemm<F, MT, NCT, PK, DEEP>(wrow, arow, inter, wscale, acc);
}

template <WFmt F, int MT, int NCT, bool PK>
__device__ __forceinline__ void down_tile(const DownArgs& a, const Tile& t, int slice) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  // this wave's output columns: c0 + 16c .. +16 for its NCT column tiles
  const int c0 = (slice * kDownWaves + wave) * 16 * NCT;
  f32x4 acc[NCT][MT];
  down_acc<F, MT, NCT, PK>(a, t, c0, acc);

  const bool shared = t.expert == a.E;
  float* y = a.y + ((shared ? (size_t)a.N * a.K : 0) + (size_t)t.start) * a.H;
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = mt * 16 + kg * 4 + v;
        if (m < t.rows) y[(size_t)m * a.H + c0 + 16 * c + col] = acc[c][mt][v];
      }
}

template <WFmt F, int MTMAX, int NCT, bool PK>
__global__ __launch_bounds__(64 * kDownWaves, kMinWavesPerSimd) void expert_down_kernel(DownArgs a) {
  const int slot = blockIdx.x / a.n_slices, slice = blockIdx.x % a.n_slices;
  if (slot >= *a.tile_count) return;
  const Tile t = a.tiles[slot];
  const int mt = (t.rows + 15) >> 4;  // 1..MTMAX
  if constexpr (MTMAX >= 4) if (mt == 4) { down_tile<F, 4, NCT, PK>(a, t, slice); return; }
  if constexpr (MTMAX >= 3) if (mt == 3) { down_tile<F, 3, NCT, PK>(a, t, slice); return; }
  if constexpr (MTMAX >= 2) if (mt == 2) { down_tile<F, 2, NCT, PK>(a, t, slice); return; }
  down_tile<F, 1, NCT, PK>(a, t, slice);
}

// Calls with at most kFusedMaxTiles work tiles (one-row decode: 8 experts
// and the shared one): the down GEMM and the combine in one kernel.  A
// workgroup owns 16 output columns and runs one wave per work tile, each
// with all four k stages of its weights in flight; the tiles' y for those
// columns go to LDS, and after a barrier the combine sums them per row: the
// shared expert's row first, then fmaf of each filled slot in slot order.
// The y of a (tile, column) comes from the same MFMA sequence as in
// expert_down_kernel and the sum is the combine kernel's, so out is bitwise
// what the two kernels give.
constexpr int kFusedMaxTiles = 10;
constexpr int kFusedMaxPairs = 64;  // N*K + N

template <WFmt F, bool PK>
__global__ __launch_bounds__(64 * kFusedMaxTiles) void expert_down_combine_kernel(DownArgs a, const int32_t* pair_pos,
                                                                   const float* gates, void* out,
                                                                   int out_bf16, const uint8_t* live) {
  __shared__ float y_s[kFusedMaxPairs][16];
  __shared__ int pos_s[kFusedMaxPairs];
  __shared__ float g_s[kFusedMaxPairs];
  __shared__ uint8_t live_s[kFusedMaxPairs];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int c0 = blockIdx.x * 16;
  const int N = a.N, K = a.K, NK = N * K;  // NK + N <= 64 <= blockDim.x
  // The combine's slot positions, gates and live flags are loaded here, before
  // the GEMM, and parked in LDS after it, so their latency hides under the
  // GEMM's (read after the barrier, each slot's loads waited for the one
  // before).  The loads are unconditional: thread t reads slot min(t, NK-1),
  // and row flags come from the first bytes of pair_pos when there is no mask
  // (read, then ignored).
  const int tid = threadIdx.x;
  const int pv = pair_pos[min(tid, NK - 1)];
  const float gv = gates[min(tid, NK - 1)];
  const uint8_t* lp = live ? live : reinterpret_cast<const uint8_t*>(pair_pos);
  const uint8_t lv = lp[min(tid, N - 1)];
  const int nt = *a.tile_count;
  for (int slot = wave; slot < nt; slot += nw) {
    const Tile t = a.tiles[slot];
    f32x4 acc[1][1];
    down_acc<F, 1, 1, PK, true>(a, t, c0, acc);
    const int base = (t.expert == a.E ? NK : 0) + t.start;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = kg * 4 + v;
      if (m < t.rows) y_s[base + m][col] = acc[0][0][v];
    }
  }
  if (tid < NK) {
    pos_s[tid] = pv;
    g_s[tid] = gv;
  }
  if (tid < N) live_s[tid] = live == nullptr || lv != 0;
  __syncthreads();
  for (int i = tid; i < N * 16; i += blockDim.x) {
    const int r = i >> 4, cc = i & 15;
    if (!live_s[r]) continue;  // a resolved row keeps the caller's cached output
    float o = a.Is > 0 ? y_s[NK + r][cc] : 0.0f;
    for (int j = 0; j < K; ++j) {
      // an empty slot (pos < 0) reads row 0 and keeps o unchanged
      const int pos = pos_s[r * K + j];
      const float t = __builtin_fmaf(g_s[r * K + j], y_s[max(pos, 0)][cc], o);
      o = pos >= 0 ? t : o;
    }
    const size_t at = (size_t)r * a.H + c0 + cc;
    if (out_bf16) static_cast<uint16_t*>(out)[at] = f32_to_bf16(o);
    else static_cast<float*>(out)[at] = o;
  }
}

// these kernels serve single-row-tile calls (MTMAX = 1); many-row tiles run in
// expert_tiled.hip
template <WFmt F, bool PK>
static void launch_up(unsigned grid, hipStream_t s, const UpArgs& a) {
  expert_up_kernel<F, 1, up_nct<F>(), PK><<<grid, 256, 0, s>>>(a);
}
template <WFmt F, bool PK>
static void launch_down(int nct, unsigned grid, hipStream_t s, const DownArgs& a) {
  if constexpr (F == WFmt::FP4) {
    if (nct == 4) expert_down_kernel<F, 1, 4, PK><<<grid, 64 * kDownWaves, 0, s>>>(a);
    else expert_down_kernel<F, 1, 2, PK><<<grid, 64 * kDownWaves, 0, s>>>(a);
  } else {
    expert_down_kernel<F, 1, 1, PK><<<grid, 64 * kDownWaves, 0, s>>>(a);
  }
}
template <WFmt F>
static void launch_up(bool panels, unsigned grid, hipStream_t s, const UpArgs& a) {
  if (panels) launch_up<F, true>(grid, s, a);
  else launch_up<F, false>(grid, s, a);
}
template <WFmt F>
static void launch_down(bool panels, int nct, unsigned grid, hipStream_t s, const DownArgs& a) {
  if (panels) launch_down<F, true>(nct, grid, s, a);
  else launch_down<F, false>(nct, grid, s, a);
}
template <WFmt F>
static void launch_down_combine(bool panels, unsigned grid, unsigned block, hipStream_t s, const DownArgs& a,
                                const Plan& p, void* out) {
  const int bf16 = p.act == CMOE_BF16;
  if (panels)
    expert_down_combine_kernel<F, true><<<grid, block, 0, s>>>(a, p.pair_pos, p.gates, out, bf16, p.live);
  else
    expert_down_combine_kernel<F, false><<<grid, block, 0, s>>>(a, p.pair_pos, p.gates, out, bf16, p.live);
}

static WFmt fmt_of(const Plan& p) {
  if (p.wt == CMOE_FP4_E2M1) return WFmt::FP4;
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
  const WFmt f = fmt_of(p);
  const int nct = f == WFmt::FP4 ? up_nct<WFmt::FP4>() : 1;
  a.n_slices = (p.I > p.Is ? p.I : p.Is) / (kUpCols * nct);
  const unsigned grid = (unsigned)p.max_tiles * (unsigned)a.n_slices;
  switch (f) {
    case WFmt::BF16: launch_up<WFmt::BF16>(p.panels, grid, s, a); break;
    case WFmt::F32: launch_up<WFmt::F32>(p.panels, grid, s, a); break;
    case WFmt::FP8: launch_up<WFmt::FP8>(p.panels, grid, s, a); break;
    case WFmt::FP4: launch_up<WFmt::FP4>(p.panels, grid, s, a); break;
  }
  return hipGetLastError();
}

bool down_combine_fits(const Plan& p) {
  // (fp32 weights keep the two kernels: their fragments need more registers
  // than 16 waves per workgroup leave)
  return p.mt_max == 1 && !p.y_act && p.wt != CMOE_F32 && p.max_tiles <= kFusedMaxTiles &&
         p.N * p.K + p.N <= kFusedMaxPairs;
}

hipError_t launch_expert_down_combine(const Plan& p, const cmoe_weights& w, void* out, hipStream_t s) {
  DownArgs a;
  a.w2 = w.w2;
  a.w2_scale = w.w2_scale;
  a.sw2 = w.shared_w2;
  a.sw2_scale = w.shared_w2_scale;
  a.tiles = p.tiles;
  a.tile_count = p.tile_count;
  a.h = p.h;
  a.y = nullptr;  // y stays in LDS
  a.N = p.N;
  a.H = p.H;
  a.E = p.E;
  a.I = p.I;
  a.Is = p.Is;
  a.K = p.K;
  a.n_slices = 0;
  const int waves = p.max_tiles;  // one per tile (at most kFusedMaxTiles)
  const unsigned grid = (unsigned)(p.H / 16), block = 64u * (unsigned)waves;
  switch (fmt_of(p)) {
    case WFmt::BF16: launch_down_combine<WFmt::BF16>(p.panels, grid, block, s, a, p, out); break;
    case WFmt::F32: return hipErrorInvalidValue;  // excluded by down_combine_fits
    case WFmt::FP8: launch_down_combine<WFmt::FP8>(p.panels, grid, block, s, a, p, out); break;
    case WFmt::FP4: launch_down_combine<WFmt::FP4>(p.panels, grid, block, s, a, p, out); break;
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
  a.y = static_cast<float*>(p.y);  // fp32 whenever these kernels run
  a.N = p.N;
  a.H = p.H;
  a.E = p.E;
  a.I = p.I;
  a.Is = p.Is;
  a.K = p.K;
  const WFmt f = fmt_of(p);
  const int nct = down_nct(f, p.H);  // H is a multiple of 128, so of kDownCols * nct
  a.n_slices = p.H / (kDownCols * nct);
  const unsigned grid = (unsigned)p.max_tiles * (unsigned)a.n_slices;
  switch (f) {
    case WFmt::BF16: launch_down<WFmt::BF16>(p.panels, nct, grid, s, a); break;
    case WFmt::F32: launch_down<WFmt::F32>(p.panels, nct, grid, s, a); break;
    case WFmt::FP8: launch_down<WFmt::FP8>(p.panels, nct, grid, s, a); break;
    case WFmt::FP4: launch_down<WFmt::FP4>(p.panels, nct, grid, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace cmoe
