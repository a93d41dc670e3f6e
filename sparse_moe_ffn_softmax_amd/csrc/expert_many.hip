// expert_many.hip -- grouped expert GEMMs for calls that route many rows to
// each expert (many blocks per call), on the 32x32 MFMAs.
//
//   expert_down_many : y = h W2_e^T, a tile's whole h resident in LDS
//                      (bf16 MFMA; with fp8 activations, h quantised to MXFP8
//                      as it is staged and the scaled fp8 MFMA)
//   expert_up_mx     : h = silu(X_e W_gate^T) * (X_e W_up^T) with fp8 weights
//                      and MXFP8 x (quant.hip), on the scaled fp8 MFMA
//
// The fp8-activation kernels run only when the caller asks for them
// (cmoe_options.activation_fp8); the pages serve fp8 weights with bf16
// activations, which remains the default.
//
// SwiGLU experts and one shared expert (Clover-35B-A3B-Preview CMF model card,
// introduction); fp8 weights are E4M3 with one fp32 scale per 128x128 block
// and bf16 activations (InfiniLM PR #584, "Benchmark"); 4-bit weights are
// MXFP4 (E2M1 codes, E8M0 scale per 32 elements of a row), widened to bf16
// exactly with their scale.  Fragment layouts: expert_frag32.h.
//
// The grids are persistent: one workgroup of kManyWaves waves per CU, each
// owning a contiguous run of units (a work tile and a group of output
// columns), tiles in the work list's order.  Every unit moves the same weight
// bytes, so equal runs of units balance the HBM traffic across the CUs.  The
// weights stream through a ring of register stages that runs on across unit
// boundaries: while a stage's MFMAs run, the following stages (of this unit
// or the next) are in flight.  Each tile's 32-row MFMA tile count is
// dispatched at run time (rows / 32 rounded up).
#include "cmoe_device.h"
#include "cmoe_launch.h"
#include "expert_frag32.h"

#include <type_traits>

namespace cmoe {

struct ManyArgs {
  const void* x;     // activations [N,H] (gate/up)
  const void* w;     // W13 [E,2I,H] (gate/up) or W2 [E,H,I] (down)
  const void* ws;    // scales of w (fp8: fp32 per 128x128 block; fp4: E8M0 per 32 of a row)
  const void* sw;    // the shared expert's matrix
  const void* sws;   // its scales
  const Tile* tiles;
  const int32_t* tile_count;
  const int32_t* pair_row;
  void* h;           // [N*K*I + N*Is] bf16
  void* y;           // [N*K + N, H], bf16 (y_act) or fp32
  int y_act;
  int N, H, E, I, Is, K;
};

constexpr int kManyWaves = 8;
constexpr int kManyThreads = 64 * kManyWaves;

// fp32 to bf16 bits, rounded to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ---------------------------------------------------------------------------
// Down GEMM.  A tile's h (at most 128 rows of I = 512 bf16, 136 KiB with the
// row padding) is staged into LDS once per tile by direct global-to-LDS loads
// (a quarter-wave load fills one 256-byte stage row) and stays there for all
// of the tile's units.  A unit is the tile times 256 output columns, 32 per
// wave, over the four 128-deep stages of I; the ring holds the four stages of
// one unit, each refilled with the next unit's same stage as soon as its
// MFMAs have issued.
// ---------------------------------------------------------------------------
// The work tiles a workgroup's run of units touches, copied to LDS once: a
// tile record read from global memory inside the unit loop is a vector load,
// and the wait for it (vector loads complete in order) would also wait for
// every weight load in flight.
constexpr int kManySlots = 64;
struct TileCache {
  Tile t[kManySlots];
  int lo, n;
};
__device__ __forceinline__ void cache_tiles(TileCache& c, const Tile* tiles, int slot_lo, int slot_hi) {
  const int n = slot_hi - slot_lo + 1;  // <= kManySlots (the grid's size)
  if ((int)threadIdx.x < n) c.t[threadIdx.x] = tiles[slot_lo + threadIdx.x];
  if (threadIdx.x == 0) {
    c.lo = slot_lo;
    c.n = n;
  }
  __syncthreads();
}
// the tile of a slot in the run (the host sizes the grid so that no run spans
// more than kManySlots tiles).  The fields are made wave-uniform (scalar
// registers), so that branches on them are scalar branches: seen as
// divergent, every arm's registers would stay live at once.
__device__ __forceinline__ Tile cached_tile(const TileCache& c, int slot) {
  const Tile v = c.t[slot - c.lo];
  Tile t;
  t.expert = __builtin_amdgcn_readfirstlane(v.expert);
  t.start = __builtin_amdgcn_readfirstlane(v.start);
  t.rows = __builtin_amdgcn_readfirstlane(v.rows);
  t.pad = 0;
  return t;
}

constexpr int kDownManyCols = 32 * kManyWaves;  // y columns per unit
constexpr int kDownManyStages = 4;              // I = 512

// A8 (fp8 weights only): h is quantised to MXFP8 as it is staged (its codes
// in 144-byte rows per stage, its 16 scale bytes per row beside them) and the
// MFMAs are the scaled fp8 ones (expert_frag32.h).
template <WFmt F, int MTM, bool PK, bool A8>
__global__ __launch_bounds__(kManyThreads, 1) void expert_down_many_kernel(ManyArgs a) {
  static_assert(!A8 || F == WFmt::FP8, "fp8 activations with fp8 weights");
  using WF = typename std::conditional<A8, W32Mx<PK>, W32<F, PK>>::type;
  using Stage = typename WF::Stage;
  using WT = typename Frag<F>::WT;
  constexpr int S = kDownManyStages, T = 32 * MTM;
  constexpr int ABYTES = A8 ? S * T * kA8Pitch + T * 16 : S * T * kA32Pitch * 2;
  __shared__ __attribute__((aligned(16))) uint8_t Araw[ABYTES];
  uint16_t* As = reinterpret_cast<uint16_t*>(Araw);   // 16-bit h: [stage][row][kA32Pitch]
  uint8_t* As8 = Araw;                                 // fp8 h: [stage][row][kA8Pitch]
  uint8_t* Hsc = Araw + (A8 ? S * T * kA8Pitch : 0);   // fp8 h: [row][16] E8M0 bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane & 31, hh = lane >> 5;
  const int ncg = a.H / kDownManyCols;
  const long long total = (long long)(*a.tile_count) * ncg;
  const int u0 = (int)(total * blockIdx.x / gridDim.x);
  const int u1 = (int)(total * (blockIdx.x + 1) / gridDim.x);
  if (u0 >= u1) return;  // uniform over the workgroup
  __shared__ TileCache tc;
  cache_tiles(tc, a.tiles, u0 / ncg, (u1 - 1) / ncg);

  // the weight source of unit u for this lane
  struct Src {
    const uint8_t* base;
    const float* s8;
    const uint8_t* s4;
  };
  auto src_of = [&](int u) {
    const Tile t = cached_tile(tc, u / ncg);
    const bool shared = t.expert == a.E;
    const int inter = shared ? a.Is : a.I;
    const size_t rowb = (size_t)inter * sizeof(WT) / Frag<F>::kPack;
    const uint8_t* W = shared ? static_cast<const uint8_t*>(a.sw)
                              : static_cast<const uint8_t*>(a.w) + (size_t)t.expert * a.H * rowb;
    const int c0 = (u % ncg) * kDownManyCols + wave * 32;
    Src s;
    s.base = WF::lane_base(W, rowb, c0 + rl, c0 / 16 + rl / 16, lane);
    s.s8 = nullptr;
    s.s4 = nullptr;
    if constexpr (F == WFmt::FP8) {
      // the wave's 32 output rows lie in one 128-row scale block row
      const float* Sc = static_cast<const float*>(shared ? a.sws : a.ws);
      if (!shared) Sc += (size_t)t.expert * (a.H / 128) * (a.I / 128);
      s.s8 = Sc + (size_t)(c0 / 128) * (inter / 128);
    } else if constexpr (F == WFmt::FP4) {
      const uint8_t* Sc = static_cast<const uint8_t*>(shared ? a.sws : a.ws);
      if (!shared) Sc += (size_t)t.expert * a.H * (a.I / 32);
      s.s4 = Sc + (size_t)(c0 + rl) * (inter / 32);
    }
    return s;
  };

  // h of tile t into LDS: load j of this wave fills row r of stage st, the
  // first 16 lanes 16 bytes each (lane i lands at 16 i bytes from the row's
  // start).  Rows past the tile re-read row 0.
  auto stage_h = [&](const Tile& t, int mt) {
    const bool shared = t.expert == a.E;
    const int inter = shared ? a.Is : a.I;
    const uint16_t* hb = static_cast<const uint16_t*>(a.h) +
                         (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
    const int rows = 32 * mt;
    if constexpr (A8) {
      // one 32-element group per thread and round (rows x 16 groups, two
      // rounds at a time): bf16 in, MXFP8 codes and scale into LDS
      for (int g0 = tid; g0 < rows * 16; g0 += 2 * kManyThreads) {
        u32x4 v[2][4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int g = g0 + k * kManyThreads < rows * 16 ? g0 + k * kManyThreads : g0;
          const int r = g >> 4, grp = g & 15;
          const int rr = r < t.rows ? r : 0;
          const u32x4* src = reinterpret_cast<const u32x4*>(hb + (size_t)rr * inter + grp * 32);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[k][i] = src[i];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int g = g0 + k * kManyThreads < rows * 16 ? g0 + k * kManyThreads : g0;
          const int r = g >> 4, grp = g & 15;
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              amax = fmaxf(amax, fabsf(__uint_as_float(v[k][i][j] << 16)));
              amax = fmaxf(amax, fabsf(__uint_as_float(v[k][i][j] & 0xFFFF0000u)));
            }
          const int sb = mx8_scale_byte(amax);
          const float inv = __uint_as_float((uint32_t)(254 - sb) << 23);
          u32x4 o[2];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            int lo = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[k][i][0] << 16) * inv,
                                                     __uint_as_float(v[k][i][0] & 0xFFFF0000u) * inv, 0, false);
            lo = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[k][i][1] << 16) * inv,
                                                 __uint_as_float(v[k][i][1] & 0xFFFF0000u) * inv, lo, true);
            int hi = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[k][i][2] << 16) * inv,
                                                     __uint_as_float(v[k][i][2] & 0xFFFF0000u) * inv, 0, false);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[k][i][3] << 16) * inv,
                                                 __uint_as_float(v[k][i][3] & 0xFFFF0000u) * inv, hi, true);
            o[i >> 1][2 * (i & 1)] = (uint32_t)lo;
            o[i >> 1][2 * (i & 1) + 1] = (uint32_t)hi;
          }
          // group grp holds k 32 grp .. +32: stage grp/4, bytes 32 (grp%4) of its row
          uint8_t* dst = As8 + ((size_t)(grp >> 2) * T + r) * kA8Pitch + 32 * (grp & 3);
          reinterpret_cast<u32x4*>(dst)[0] = o[0];
          reinterpret_cast<u32x4*>(dst)[1] = o[1];
          Hsc[r * 16 + grp] = (uint8_t)sb;
        }
      }
    } else {
      for (int j = wave; j < S * rows; j += kManyWaves) {
        const int st = j / rows, r = j % rows;
        const int rr = r < t.rows ? r : 0;
        const uint16_t* src = hb + (size_t)rr * inter + st * 128 + (lane & 15) * 8;
        uint16_t* dst = As + ((size_t)st * T + r) * kA32Pitch;
        if (lane < 16)
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      }
    }
  };

  auto load_stage = [&](Stage& st, const Src& src, int s) {
    if constexpr (A8) WF::load(st, src.base, src.s8, s);
    else WF::load(st, src.base, src.s8, src.s4, s, lane);
  };

  Stage w[S];
  {
    const Src s0 = src_of(u0);
#pragma unroll
    for (int s = 0; s < S; ++s) load_stage(w[s], s0, s);
  }
  int cur_slot = -1;
  auto unit = [&](int u) {
    const Tile t = cached_tile(tc, u / ncg);
    const int slot = u / ncg;
    const int mt = (t.rows + 31) / 32;
    if (slot != cur_slot) {
      __syncthreads();  // every wave is done with the previous tile's h
      stage_h(t, mt);
      __syncthreads();  // (the compiler waits for the direct loads here)
      cur_slot = slot;
    }
    // the next unit's source (the last unit re-reads its own: every load is
    // unconditional, so the compiler's waits stay exact)
    const Src sn = src_of(u + 1 < u1 ? u + 1 : u);
    const int c = (u % ncg) * kDownManyCols + wave * 32 + rl;
    const bool shared = t.expert == a.E;
    const size_t y0 = ((shared ? (size_t)a.N * a.K : 0) + (size_t)t.start) * a.H;
    f32x16 acc[MTM];
#pragma unroll
    for (int i = 0; i < MTM; ++i) acc[i] = f32x16{};
    static_for<0, S>([&](auto SI) {
      constexpr int s = decltype(SI)::value;
      const uint16_t* As_s = As + (size_t)s * T * kA32Pitch;
      (void)As_s;
      // the tile's row-tile count, dispatched inside the stage so that the
      // ring registers have one definition per stage
      static_for<1, MTM + 1>([&](auto M) {
        constexpr int MT = decltype(M)::value;
        if (mt != MT) return;
        if constexpr (A8) {
          // row tiles two at a time: two scaled fp8 MFMAs per stage each, then
          // times the weight block scale
          const float sc = __uint_as_float(w[s].sc);
          static_for<0, (MT + 1) / 2>([&](auto PI) {
            constexpr int i0 = 2 * decltype(PI)::value;
            constexpr int NP = i0 + 1 < MT ? 2 : 1;
            f32x16 tmp[NP];
            int sa[NP];
#pragma unroll
            for (int j = 0; j < NP; ++j) {
              tmp[j] = f32x16{};
              sa[j] = (int)*reinterpret_cast<const uint32_t*>(Hsc + ((i0 + j) * 32 + rl) * 16 + 4 * s);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const i32x8 b = WF::operand(w[s], q);
#pragma unroll
              for (int j = 0; j < NP; ++j) {
                const uint8_t* row = As8 + ((size_t)s * T + (i0 + j) * 32 + rl) * kA8Pitch;
                tmp[j] = mfma_mx(lds_frag8(row, q, hh), b, (sa[j] >> (8 * (2 * q + hh))) & 0xFF, tmp[j]);
              }
            }
#pragma unroll
            for (int j = 0; j < NP; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i0 + j][v] = __builtin_fmaf(sc, tmp[j][v], acc[i0 + j][v]);
          });
        } else if constexpr (F == WFmt::FP8) {
          // row tiles two at a time: their stage partials, then times the
          // block scale; each widened weight step feeds both MFMAs
          const float sc = __uint_as_float(w[s].sc);
          static_for<0, (MT + 1) / 2>([&](auto PI) {
            constexpr int i0 = 2 * decltype(PI)::value;
            constexpr int NP = i0 + 1 < MT ? 2 : 1;
            f32x16 tmp[NP];
            u32x4 av[NP];
#pragma unroll
            for (int j = 0; j < NP; ++j) {
              tmp[j] = f32x16{};
              av[j] = lds_frag(As_s, (i0 + j) * 32 + rl, WF::ack(0, hh));
            }
#pragma unroll
            for (int tt = 0; tt < WF::STEPS; ++tt) {
              u32x4 an[NP];
#pragma unroll
              for (int j = 0; j < NP; ++j)
                an[j] = tt + 1 < WF::STEPS ? lds_frag(As_s, (i0 + j) * 32 + rl, WF::ack(tt + 1, hh)) : av[j];
              u32x2 codes = WF::codes8(w[s], tt);
              asm volatile("" : "+v"(codes));  // widen here, once per pair of row tiles
              const u32x4 b = Frag<WFmt::FP8>::widen(codes);
#pragma unroll
              for (int j = 0; j < NP; ++j) tmp[j] = mfma32(av[j], b, tmp[j]);
#pragma unroll
              for (int j = 0; j < NP; ++j) av[j] = an[j];
            }
#pragma unroll
            for (int j = 0; j < NP; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[i0 + j][v] = __builtin_fmaf(sc, tmp[j][v], acc[i0 + j][v]);
          });
        } else {
          u32x4 av[MT];
#pragma unroll
          for (int i = 0; i < MT; ++i) av[i] = lds_frag(As_s, i * 32 + rl, WF::ack(0, hh));
#pragma unroll
          for (int tt = 0; tt < WF::STEPS; ++tt) {
            u32x4 an[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
              an[i] = tt + 1 < WF::STEPS ? lds_frag(As_s, i * 32 + rl, WF::ack(tt + 1, hh)) : av[i];
            const u32x4 b = WF::bop(w[s], tt);
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[i] = mfma32(av[i], b, acc[i]);
#pragma unroll
            for (int i = 0; i < MT; ++i) av[i] = an[i];
          }
        }
      });
      // this stage's registers now carry the next unit's same stage (the
      // barriers keep the scheduler from hoisting the loads above the
      // MFMAs that still read the old contents)
      __builtin_amdgcn_sched_barrier(0);
      load_stage(w[s], sn, s);
      __builtin_amdgcn_sched_barrier(0);
    });
    // y in bf16 (this kernel runs on 16-bit activations only); whole 32-row
    // tiles unmasked, the tile's last one row by row
    // (H passes through an empty asm so that the row addresses are computed
    // here: hoisted out of the unit loop, all 16 * MTM of them stay live)
    int Hs = a.H;
    asm volatile("" : "+s"(Hs));
    uint16_t* yb = static_cast<uint16_t*>(a.y) + y0 + c + (size_t)(4 * hh) * Hs;
#pragma unroll
    for (int i = 0; i < MTM; ++i) {
      if (i >= mt) break;
      uint16_t* yr = yb + (size_t)(32 * i) * Hs;
      if ((i + 1) * 32 <= t.rows) {  // a scalar branch: no per-store lane masks
#pragma unroll
        for (int v = 0; v < 16; ++v) yr[(size_t)(8 * (v >> 2) + (v & 3)) * Hs] = bf16_bits(acc[i][v]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * i + 8 * (v >> 2) + 4 * hh + (v & 3) < t.rows)
            yr[(size_t)(8 * (v >> 2) + (v & 3)) * Hs] = bf16_bits(acc[i][v]);
      }
    }
  };
  // The first unit is peeled: the loop is then entered after the same
  // sequence of loads as its back edge, and the compiler's waits for the
  // ring registers stay exact (with the prologue's loads merged in at the
  // loop header they degrade to waiting for everything in flight).
  unit(u0);
  for (int u = u0 + 1; u < u1; ++u) unit(u);
}

// ---------------------------------------------------------------------------
// Gate/up GEMM + SwiGLU with fp8 weights and MXFP8 activations (x quantised
// by quant.hip).  A unit is a tile times 128 h columns (256 weight rows: 16
// h columns per wave, its 32 weight rows the two 16-row panels that pair those
// columns' gate and up rows); K = H runs in S stages of 128.  The gathered
// code rows of a stage (128 bytes each) and their four scale bytes pass
// through registers into one of two LDS slots, two stages ahead; the weights
// stream through a four-stage register ring that runs on into the next unit.
// Every stage ends with one workgroup barrier.
// ---------------------------------------------------------------------------
constexpr int kUpManyCols = 16 * kManyWaves;  // h columns per unit

template <int MTM, bool PK, int S>
__global__ __launch_bounds__(kManyThreads, 1) void expert_up_mx_kernel(ManyArgs a) {
  using WF = W32Mx<PK>;
  using Stage = typename WF::Stage;
  constexpr int T = 32 * MTM;
  constexpr int NV = 8 * T;                                      // 16-byte code vectors per stage
  constexpr int AV = (NV + kManyThreads - 1) / kManyThreads;     // per thread
  static_assert(S % 4 == 0, "stage count a multiple of the ring");
  __shared__ __attribute__((aligned(16))) uint8_t As[2][T * kA8Pitch];
  __shared__ uint32_t Asc[2][T];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane & 31, hh = lane >> 5;
  const int ncg = a.I / kUpManyCols;
  const long long total = (long long)(*a.tile_count) * ncg;
  const int u0 = (int)(total * blockIdx.x / gridDim.x);
  const int u1 = (int)(total * (blockIdx.x + 1) / gridDim.x);
  if (u0 >= u1) return;  // uniform over the workgroup
  __shared__ TileCache tc;
  cache_tiles(tc, a.tiles, u0 / ncg, (u1 - 1) / ncg);
  const uint8_t* x8 = static_cast<const uint8_t*>(a.x);
  const uint8_t* xs = x8 + (size_t)a.N * a.H;  // E8M0 scales [N, H/32] after the codes

  // this thread's staged vectors: code vector v = tid + i * threads (clamped
  // into the stage: surplus threads repeat a vector), row v / 8, piece v % 8;
  // scale word of row tid % T
  struct Rows {
    int src[AV];
    int ssrc;
  };
  auto rows_of = [&](int u) {
    const Tile t = cached_tile(tc, u / ncg);
    const bool shared = t.expert == a.E;
    Rows R;
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = (tid + i * kManyThreads) % NV;
      const int r = v >> 3;
      const int rr = r < t.rows ? r : 0;
      R.src[i] = shared ? t.start + rr : a.pair_row[t.start + rr];
    }
    const int r = tid % T;
    const int rr = r < t.rows ? r : 0;
    R.ssrc = shared ? t.start + rr : a.pair_row[t.start + rr];
    return R;
  };
  struct AReg {
    u32x4 v[AV];
    uint32_t sc;
  };
  auto load_a = [&](AReg& ar, const Rows& R, int s) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = (tid + i * kManyThreads) % NV;
      ar.v[i] = *reinterpret_cast<const u32x4*>(x8 + (size_t)R.src[i] * a.H + s * 128 + (v & 7) * 16);
    }
    ar.sc = *reinterpret_cast<const uint32_t*>(xs + (size_t)R.ssrc * (a.H / 32) + 4 * s);
  };
  auto store_a = [&](const AReg& ar, int slot) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int v = (tid + i * kManyThreads) % NV;
      *reinterpret_cast<u32x4*>(&As[slot][(v >> 3) * kA8Pitch + (v & 7) * 16]) = ar.v[i];
    }
    if (tid < T) Asc[slot][tid] = ar.sc;
  };

  // this lane's weight source for unit u: the gate and up rows of its panel pair
  struct Src {
    const uint8_t* base;
    const float* s8;
  };
  auto src_of = [&](int u) {
    const Tile t = cached_tile(tc, u / ncg);
    const bool shared = t.expert == a.E;
    const int inter = shared ? a.Is : a.I;
    const size_t rowb = (size_t)a.H;  // fp8: one byte per element
    const uint8_t* W = shared ? static_cast<const uint8_t*>(a.sw)
                              : static_cast<const uint8_t*>(a.w) + (size_t)t.expert * 2 * a.I * rowb;
    const int hc0 = (u % ncg) * kUpManyCols + wave * 16;
    const int pp = rl >> 4, i = rl & 15;
    const int row = i < 8 ? hc0 + 8 * pp + i : inter + hc0 + 8 * pp + i - 8;
    Src sr;
    sr.base = WF::lane_base(W, rowb, row, hc0 / 8 + pp, lane);
    const float* Sc = static_cast<const float*>(shared ? a.sws : a.ws);
    if (!shared) Sc += (size_t)t.expert * (2 * a.I / 128) * (a.H / 128);
    sr.s8 = Sc + (size_t)(row / 128) * (a.H / 128);
    return sr;
  };

  Stage w[4];
  AReg ar[2];
  Rows rc = rows_of(u0);
  Src wc = src_of(u0);
  // prologue: A stages 0 and 1, weight stages 0..3, stage 0 into LDS slot 0
  load_a(ar[0], rc, 0);
  load_a(ar[1], rc, 1);
#pragma unroll
  for (int s = 0; s < 4; ++s) WF::load(w[s], wc.base, wc.s8, s);
  store_a(ar[0], 0);
  __syncthreads();

  // One unit.  Invariant on entry: LDS slot 0 holds A stage 0, ar[1] has A
  // stage 1 in flight, w[0..3] hold weight stages 0..3 in flight.
  auto unit = [&](int u) {
    const Tile t = cached_tile(tc, u / ncg);
    const int mt = (t.rows + 31) / 32;
    const int un = u + 1 < u1 ? u + 1 : u;  // the last unit re-reads itself (unconditional loads)
    const Rows rn = rows_of(un);
    const Src wn = src_of(un);
    f32x16 acc[MTM];
#pragma unroll
    for (int i = 0; i < MTM; ++i) acc[i] = f32x16{};
    static_for<0, S>([&](auto SI) {
      constexpr int s = decltype(SI)::value;
      // A two stages ahead (into the register set stage s used)
      if constexpr (s + 2 < S) load_a(ar[s % 2], rc, s + 2);
      else load_a(ar[s % 2], rn, s + 2 - S);
      const uint8_t* Aslot = As[s % 2];
      const uint32_t* Sslot = Asc[s % 2];
      const float sc = __uint_as_float(w[s % 4].sc);
      static_for<1, MTM + 1>([&](auto M) {
        constexpr int MT = decltype(M)::value;
        if (mt != MT) return;
        static_for<0, (MT + 1) / 2>([&](auto PI) {
          constexpr int i0 = 2 * decltype(PI)::value;
          constexpr int NP = i0 + 1 < MT ? 2 : 1;
          f32x16 tmp[NP];
          int sa[NP];
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            tmp[j] = f32x16{};
            sa[j] = (int)Sslot[(i0 + j) * 32 + rl];
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const i32x8 b = WF::operand(w[s % 4], q);
#pragma unroll
            for (int j = 0; j < NP; ++j)
              tmp[j] = mfma_mx(lds_frag8(Aslot + ((i0 + j) * 32 + rl) * kA8Pitch, q, hh), b,
                               (sa[j] >> (8 * (2 * q + hh))) & 0xFF, tmp[j]);
          }
#pragma unroll
          for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i0 + j][v] = __builtin_fmaf(sc, tmp[j][v], acc[i0 + j][v]);
        });
      });
      // the ring slot now carries stage s + 4 (of this unit or the next)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (s + 4 < S) WF::load(w[s % 4], wc.base, wc.s8, s + 4);
      else WF::load(w[s % 4], wn.base, wn.s8, s + 4 - S);
      __builtin_amdgcn_sched_barrier(0);
      store_a(ar[(s + 1) % 2], (s + 1) % 2);  // A stage s + 1 (the next unit's 0 after the last)
      __syncthreads();
    });
    // SwiGLU: lane rl holds weight row rl of the wave's pair of panels (gate
    // rows at rl % 16 < 8, their up rows 8 lanes on); h in bf16
    const bool shared = t.expert == a.E;
    const int inter = shared ? a.Is : a.I;
    uint16_t* hb = static_cast<uint16_t*>(a.h) +
                   (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
    const int hcol = (u % ncg) * kUpManyCols + wave * 16 + 8 * (rl >> 4) + (rl & 7);
    int In = inter;
    asm volatile("" : "+s"(In));  // row addresses computed here, not hoisted out of the loop
    uint16_t* hrow = hb + (size_t)(4 * hh) * In + hcol;
#pragma unroll
    for (int i = 0; i < MTM; ++i) {
      if (i >= mt) break;
      uint16_t* hr = hrow + (size_t)(32 * i) * In;
      if ((i + 1) * 32 <= t.rows) {  // a scalar branch: whole row tiles need no row test
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float g = acc[i][v];
          const float upv = shfl_xor_f(g, 8);
          if ((rl & 15) < 8) hr[(size_t)(8 * (v >> 2) + (v & 3)) * In] = bf16_bits(silu(g) * upv);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float g = acc[i][v];
          const float upv = shfl_xor_f(g, 8);
          if ((rl & 15) < 8 && 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3) < t.rows)
            hr[(size_t)(8 * (v >> 2) + (v & 3)) * In] = bf16_bits(silu(g) * upv);
        }
      }
    }
    rc = rn;
    wc = wn;
  };
  unit(u0);  // peeled (see the down kernel)
  for (int u = u0 + 1; u < u1; ++u) unit(u);
}

// CUs of the current device, for the persistent grids (queried once per device)
static int cu_count() {
  static int counts[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!counts[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

static bool mx_up_stages_ok(int H) { return H == 512 || H == 1024 || H == 2048; }

bool expert_many_fits(const Plan& p, bool up) {
  // y in the activation dtype (the workspace plan's rule for tiles taller than 16 rows)
  const bool base = p.mt_max > 1 && p.act == CMOE_BF16 && p.y_act && p.wt != CMOE_F32 &&
                    (p.Is == 0 || p.Is == p.I) && p.tile_rows % 32 == 0;
  if (up) return base && p.act8 && mx_up_stages_ok(p.H) && p.I % kUpManyCols == 0;
  if (!base || p.I != 128 * kDownManyStages || p.H % kDownManyCols != 0) return false;
  if (p.act8) return true;  // the fp8-activation down GEMM exists only here
  // Against the LDS-tiled down kernel (expert_tiled.hip), by weight format and
  // work-tile height (measured, one MI355X, I = 512, H = 2048): bf16 tiled
  // 11-15% faster at 32-96 rows, this kernel 12% faster at 128; fp8 tiled
  // 4-5% faster at 32 and 64 rows, even at 96, this kernel 27% faster at 128;
  // 4-bit this kernel faster at 64-128 rows
  const int min_rows = p.wt == CMOE_BF16 ? 128 : p.wt == CMOE_FP8_E4M3 ? 96 : 32;
  return p.tile_rows >= min_rows;
}

// Persistent grid: one workgroup per CU, or more when a run of units could
// otherwise span more tiles than a workgroup caches.
static unsigned many_grid(int max_tiles, int units_per_tile) {
  const long long units = (long long)max_tiles * units_per_tile;
  const long long per = (long long)(kManySlots - 2) * units_per_tile;  // units a run may hold
  const long long need = (units + per - 1) / per;
  const long long g = cu_count();
  return (unsigned)(need > g ? need : g);
}

template <WFmt F, bool PK, bool A8>
static void launch_down_many(const ManyArgs& a, int mtm, int max_tiles, hipStream_t s) {
  const unsigned grid = many_grid(max_tiles, a.H / kDownManyCols);
  switch (mtm) {
    case 1: expert_down_many_kernel<F, 1, PK, A8><<<grid, kManyThreads, 0, s>>>(a); break;
    case 2: expert_down_many_kernel<F, 2, PK, A8><<<grid, kManyThreads, 0, s>>>(a); break;
    case 3: expert_down_many_kernel<F, 3, PK, A8><<<grid, kManyThreads, 0, s>>>(a); break;
    default: expert_down_many_kernel<F, 4, PK, A8><<<grid, kManyThreads, 0, s>>>(a); break;
  }
}

template <int MTM, bool PK>
static void launch_up_mx_s(const ManyArgs& a, unsigned grid, hipStream_t s) {
  switch (a.H / 128) {
    case 4: expert_up_mx_kernel<MTM, PK, 4><<<grid, kManyThreads, 0, s>>>(a); break;
    case 8: expert_up_mx_kernel<MTM, PK, 8><<<grid, kManyThreads, 0, s>>>(a); break;
    default: expert_up_mx_kernel<MTM, PK, 16><<<grid, kManyThreads, 0, s>>>(a); break;
  }
}

template <bool PK>
static void launch_up_mx(const ManyArgs& a, int mtm, int max_tiles, hipStream_t s) {
  const unsigned grid = many_grid(max_tiles, a.I / kUpManyCols);
  switch (mtm) {
    case 1: launch_up_mx_s<1, PK>(a, grid, s); break;
    case 2: launch_up_mx_s<2, PK>(a, grid, s); break;
    case 3: launch_up_mx_s<3, PK>(a, grid, s); break;
    default: launch_up_mx_s<4, PK>(a, grid, s); break;
  }
}

hipError_t launch_expert_many(const Plan& p, const cmoe_weights& w, const void* x, bool up, hipStream_t s) {
  ManyArgs a;
  a.x = up && p.act8 ? p.x8 : x;
  a.w = up ? w.w13 : w.w2;
  a.ws = up ? w.w13_scale : w.w2_scale;
  a.sw = up ? w.shared_w13 : w.shared_w2;
  a.sws = up ? w.shared_w13_scale : w.shared_w2_scale;
  a.tiles = p.tiles;
  a.tile_count = p.tile_count;
  a.pair_row = p.pair_row;
  a.h = p.h;
  a.y = p.y;
  a.y_act = p.y_act;
  a.N = p.N;
  a.H = p.H;
  a.E = p.E;
  a.I = p.I;
  a.Is = p.Is;
  a.K = p.K;
  const int mtm = p.tile_rows / 32;
  if (up) {
    // fp8 activations: x quantised to MXFP8 first, then the fp8 gate/up GEMM
    hipError_t e = launch_quant_mx8(x, p.N, p.H, p.x8, static_cast<uint8_t*>(p.x8) + (size_t)p.N * p.H, s);
    if (e != hipSuccess) return e;
    if (p.panels) launch_up_mx<true>(a, mtm, p.max_tiles, s);
    else launch_up_mx<false>(a, mtm, p.max_tiles, s);
    return hipGetLastError();
  }
  if (p.wt == CMOE_FP8_E4M3) {
    if (p.act8) {
      if (p.panels) launch_down_many<WFmt::FP8, true, true>(a, mtm, p.max_tiles, s);
      else launch_down_many<WFmt::FP8, false, true>(a, mtm, p.max_tiles, s);
    } else {
      if (p.panels) launch_down_many<WFmt::FP8, true, false>(a, mtm, p.max_tiles, s);
      else launch_down_many<WFmt::FP8, false, false>(a, mtm, p.max_tiles, s);
    }
  } else if (p.wt == CMOE_FP4_E2M1) {
    if (p.panels) launch_down_many<WFmt::FP4, true, false>(a, mtm, p.max_tiles, s);
    else launch_down_many<WFmt::FP4, false, false>(a, mtm, p.max_tiles, s);
  } else {
    if (p.panels) launch_down_many<WFmt::BF16, true, false>(a, mtm, p.max_tiles, s);
    else launch_down_many<WFmt::BF16, false, false>(a, mtm, p.max_tiles, s);
  }
  return hipGetLastError();
}

}  // namespace cmoe
