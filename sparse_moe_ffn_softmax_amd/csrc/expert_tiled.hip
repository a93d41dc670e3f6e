// expert_tiled.hip -- grouped expert GEMMs for calls that route several rows
// to each expert (work tiles of 32 to 128 rows; a tile with fewer rows runs
// only the 16-row MFMA tiles it fills).
//
//   expert_up_tiled   : h = silu(X_e W_gate^T) * (X_e W_up^T)
//   expert_down_tiled : y = h W2_e^T
//
// SwiGLU experts and one shared expert (Clover-35B-A3B-Preview CMF model card,
// introduction); fp8 weights are E4M3 with one fp32 scale per 128x128 block
// and bf16 activations (InfiniLM PR #584, "Benchmark"); 4-bit weights are
// MXFP4 (E2M1 codes, E8M0 scale per 32 elements of a row), widened to bf16
// exactly with their scale.
//
// With tens of rows per expert every weight byte feeds tens of MFMA rows, so
// the activation tile must not be fetched once per wave.  A workgroup of
// NW waves (below) owns one tile of up to T = 16*MT rows and a slice of
// output columns (up: 8 h columns = 16 weight columns per wave; down: 16 y
// columns per wave).  The
// hidden (or intermediate) dimension is consumed in stages of 256 bytes per
// row: the gathered activation rows of the next stage are loaded into
// registers and parked in the other half of a double-buffered LDS tile while
// the current stage feeds the MFMAs; every wave reads the whole activation
// tile from LDS and streams its own 16 weight columns from HBM straight into
// MFMA operand registers (also double-buffered).  fp8 codes are widened to
// bf16 exactly in registers; each 128-deep stage is accumulated separately and
// added times its block scale.
#include "cmoe_device.h"
#include "cmoe_launch.h"
#include "expert_frag.h"

#include <type_traits>

namespace cmoe {

// Waves per workgroup, 16 MFMA columns each, by row-tile count: 4 for tiles
// of at most 32 rows, 8 above.  Short tiles make long, few workgroups (16
// blocks: 272 tiles x 8 column slices of 8 waves is under three rounds of
// the chip), and halving the workgroup halves the last round's idle share
// (16 blocks: gate/up 183 -> 177 us, down 105 -> 101 us); tall tiles need
// the 8 waves to share their activation tile's LDS (64 blocks with 4 waves:
// gate/up 134 -> 171 us).
__host__ __device__ constexpr int tiled_waves(int mt) { return mt <= 2 ? 4 : 8; }
// The gate/up kernel runs 16 waves on 128-row tiles: one activation tile then
// feeds twice the weight columns (256 and 512 blocks, fp8 weights: 523 -> 442
// and 968 -> 816 us; 128 blocks bf16 358 -> 329 us, 4-bit 238 -> 227 us),
// where on 96-row tiles 16 waves were slower (64 blocks fp8: 146 -> 159 us).
__host__ __device__ constexpr int tiled_up_waves(int mt) { return mt == 8 ? 16 : tiled_waves(mt); }
__host__ __device__ constexpr int tiled_up_cols(int mt) { return 8 * tiled_up_waves(mt); }  // h columns per workgroup
__host__ __device__ constexpr int tiled_down_cols(int mt) { return 16 * tiled_waves(mt); }  // y columns per workgroup

struct TiledArgs {
  const void* x;     // up: activations [N,H]
  const void* w;     // up: W13 [E,2I,H]; down: W2 [E,H,I]
  const void* ws;    // scales of w (fp8: fp32 per 128x128 block; fp4: E8M0 per 32 of a row)
  const void* sw;    // shared expert's matrix
  const void* sws;   // its scales
  const Tile* tiles;
  const int32_t* tile_count;
  const int32_t* pair_row;
  void* h;           // [N*K*I + N*Is] activation dtype
  void* y;           // [N*K + N, H], activation dtype (y_act) or fp32
  int y_act;
  int N, H, E, I, Is, K, n_slices;
};

constexpr int kTiledMaxStages = 128;  // fp8 block scales held per weight row (hidden <= 16384)

// The k order, the LDS placement of staged activation rows, and one stage
// (128 k for 16-bit activations) of weight loads and MFMAs, shared by the
// tiled kernels below.  A stage of a staged activation row is 256 bytes,
// stored with a 288-byte pitch; PK: the weights are stored in MFMA panels.
template <WFmt F, bool PK>
struct StageOps {
  using Fr = Frag<F>;
  using AT = typename Fr::AT;
  using WT = typename Fr::WT;
  static constexpr int KS = 256 / (int)sizeof(AT);  // k per stage (256 bytes of a row)
  static constexpr int U = KS / Fr::kStep;          // MFMA steps per stage
  static constexpr int VPR = 16;                    // 16-byte vectors per row per stage
  // 288-byte rows: the MFMA fragment reads (16 rows at one offset, the four
  // lane groups 64 contiguous bytes) are free of bank conflicts (a 272-byte
  // pitch measured 3.7 conflict cycles per read on gfx950)
  static constexpr int PAD = 32 / (int)sizeof(AT);
  static constexpr int PITCH = KS + PAD;            // elements per staged row
  // k order inside a stage.  MFMA only needs A and B to agree on it, so fp8
  // pairs steps: lane group kg takes k [16kg, 16kg+16) of each 64-deep step
  // pair, and its weights arrive as one 16-byte load per two steps (8 fp8
  // codes per step) instead of two 8-byte ones.
  static constexpr bool kPair = (F == WFmt::FP8);
  static_assert(!kPair || U % 2 == 0, "paired fp8 steps");
  // element offset, within a stage, of the fragment lane group kg uses at step u
  static __device__ __forceinline__ int koff(int u, int kg) {
    return kPair ? 64 * (u / 2) + 16 * kg + 8 * (u % 2) : u * Fr::kStepK + kg * Fr::kGroupK;
  }
  // LDS placement of a staged row.  16-byte chunk c of the row (in k order;
  // the fragment at (u, kg) is chunk koff(u, kg) * sizeof(AT) / 16)
  // is stored at chunk apos(c), chosen so that the fragment a lane reads at
  // step u is chunk 4u + kg for every format, the pattern above.  Read in
  // place, the paired fp8 order (lane groups 32 bytes apart) and the fp4
  // order (64 bytes apart) measured 4 conflict cycles per read on gfx950.
  static __device__ __forceinline__ int apos(int c) {
    if constexpr (kPair) return (c & 8) | ((c & 1) << 2) | ((c >> 1) & 3);  // c = 8(u/2) + 2kg + u%2
    else if constexpr (F == WFmt::FP4) return ((c & 3) << 2) | (c >> 2);    // c = u + 4kg
    else return c;                                                          // c = 4u + kg
  }
  static __device__ __forceinline__ int aread(int u, int kg) { return (4 * u + kg) * (16 / (int)sizeof(AT)); }
  static __device__ __forceinline__ int aread_sw(int u, int kg, int swz) {
    return ((4 * u + kg) ^ swz) * (16 / (int)sizeof(AT));
  }
  // inverse of apos: the k-order chunk stored at position q
  static __device__ __forceinline__ int ainv(int q) {
    if constexpr (kPair) return (q & 8) | ((q & 3) << 1) | ((q >> 2) & 1);
    else if constexpr (F == WFmt::FP4) return ((q & 3) << 2) | (q >> 2);
    else return q;
  }
  // Each lane group kg reads the 16 weight bytes at byte 16kg of every 64
  // bytes of its row (fp8 through the paired order above), i.e. one chunk
  // (expert_frag.h) per 64 row bytes.
  // This lane's chunk 0 of a weight matrix W (rows of rowb bytes): in
  // row-major storage its weight row is row `row` of W; in panel storage it
  // is panel row lane % 16 of panel `panel` (16 rows, see clover_moe.h).
  static __device__ __forceinline__ const uint8_t* bchunk0(const uint8_t* W, size_t rowb, int row, int panel,
                                                           int lane) {
    if constexpr (PK) return W + (size_t)panel * 16 * rowb + 16 * lane;
    else return W + (size_t)row * rowb + 16 * (lane >> 4);
  }
  // one stage of this lane's weights; fp4 adds the stage's four E8M0 bytes of its row
  struct BSet {
    typename Fr::B b[U];
    uint32_t sc;
  };

  // Weights of the stage at k0: this lane's chunks from brow (its chunk 0);
  // bsc: fp4: this lane's row of E8M0 bytes.
  static __device__ __forceinline__ void load_b(BSet& bs, const uint8_t* brow, const void* bsc, int k0) {
    constexpr int QB = kChunk<PK>;
    auto& b = bs.b;
    if constexpr (F == WFmt::FP4) {
      const u32x4 v = load_chunk<PK>(brow + (k0 / 128) * QB);
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = v[u];
      bs.sc = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(bsc) + k0 / 32);
      // keep the next stage's loads ahead of this stage's scale use, which
      // would otherwise be hoisted and wait for every load in flight
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (kPair) {
#pragma unroll
      for (int j = 0; j < U / 2; ++j) {
        const u32x4 v = load_chunk<PK>(brow + (k0 / 64 + j) * QB);
        b[2 * j] = typename Fr::B{v[0], v[1]};
        b[2 * j + 1] = typename Fr::B{v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[u] = __builtin_bit_cast(typename Fr::B,
                                  load_chunk<PK>(brow + ((k0 + u * Fr::kStep) * (int)sizeof(WT) / 64) * QB));
    }
  }

  // MFMAs of one stage for MTX row tiles: a0 is this lane's staged row
  // (row `col` of the stage buffer), rows `pitch` elements apart, its
  // 16-byte chunk q stored at position q ^ swz; sc8: fp8: the stage's fp32
  // block scale.  Per k step the MTX activation fragments are read first,
  // then the MTX MFMAs issue.
  template <int MTX, bool kRewiden = false>
  static __device__ __forceinline__ void mma(const AT* a0, int pitch, int swz, const BSet& bs, float sc8,
                                             int kg, f32x4 (&acc)[MTX]) {
    const auto& b = bs.b;
    if constexpr (F == WFmt::FP4) {
      const float sc = Fr::scale_of((bs.sc >> (8 * kg)) & 0xFFu);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        typename Fr::A av[MTX];
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) av[mt] = Fr::load_a(a0 + mt * 16 * pitch + aread_sw(u, kg, swz));
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) acc[mt] = Fr::mma(av[mt], b[u], sc, acc[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (F == WFmt::FP8) {
      f32x4 tmp[MTX];
#pragma unroll
      for (int mt = 0; mt < MTX; ++mt) tmp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        typename Fr::A av[MTX];
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) av[mt] = Fr::load_a(a0 + mt * 16 * pitch + aread_sw(u, kg, swz));
        // kRewiden: widen here, from the codes, whatever the caller did
        // before: a caller running several passes over the same weights
        // would otherwise keep every widened step alive
        typename Fr::B bu = b[u];
        if constexpr (kRewiden) asm volatile("" : "+v"(bu));
        const u32x4 wb = Fr::widen(bu);
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) tmp[mt] = Fr::mma_wide(av[mt], wb, tmp[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int mt = 0; mt < MTX; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mt][v] = __builtin_fmaf(sc8, tmp[mt][v], acc[mt][v]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        typename Fr::A av[MTX];
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) av[mt] = Fr::load_a(a0 + mt * 16 * pitch + aread_sw(u, kg, swz));
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) acc[mt] = Fr::mma(av[mt], b[u], acc[mt]);
        // keep the scheduler from hoisting every k step's operands at once
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

// One workgroup's GEMM: acc[mt] (16 x 16 each) for this wave's 16 columns,
// over k in [0, Kdim).  asrc[i]: source row pointer (stage 0) of the i-th
// activation vector this thread stages (rows past the tile repeat the tile's
// first row, so that every load is unconditional); brow: this lane's weight
// chunk 0 (bchunk0); bsc: its fp8 block scales, one per 128 k, in LDS.  PK:
// the weights are stored in MFMA panels.
template <WFmt F, int MT, bool PK, int NWAVES = tiled_waves(MT)>
struct TiledGemm : StageOps<F, PK> {
  using Ops = StageOps<F, PK>;
  using Fr = Frag<F>;
  using AT = typename Fr::AT;
  using WT = typename Fr::WT;
  using BSet = typename Ops::BSet;
  static constexpr int T = 16 * MT;
  static constexpr int KS = Ops::KS, VPR = Ops::VPR, PITCH = Ops::PITCH;
  static constexpr int NW = NWAVES;                 // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int RPP = THREADS / VPR;         // rows staged per pass of the workgroup
  static constexpr int AV = T / RPP;                // vectors per thread per stage
  static_assert(AV * RPP == T, "whole staging passes");
  using Lds = AT[2][T][PITCH];

  // MTX: the row tiles that hold rows of this tile (1..MT), a compile-time
  // count chosen per tile by the caller: the MFMAs and fragment reads of the
  // others are skipped (their accumulators stay zero and are never stored).
  // Staging still covers all T rows, so the load counts stay fixed.
  template <int MTX = MT>
  static __device__ __forceinline__ void run(Lds& As, const AT* const (&asrc)[AV],
                                             const uint8_t* brow, const void* bsc, int Kdim,
                                             f32x4 (&acc)[MT]) {
    static_assert(MTX >= 1 && MTX <= MT, "row tiles");
    f32x4(&accx)[MTX] = *reinterpret_cast<f32x4(*)[MTX]>(&acc[0]);
    const int tid = threadIdx.x, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int seg = tid % VPR, r0 = tid / VPR;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 areg[AV];
    BSet b0, b1;
    auto load_a = [&](int k0) {
#pragma unroll
      for (int i = 0; i < AV; ++i)
        areg[i] = *reinterpret_cast<const u32x4*>(asrc[i] + k0);
    };
    auto store_a = [&](int buf) {
#pragma unroll
      for (int i = 0; i < AV; ++i)
        *reinterpret_cast<u32x4*>(&As[buf][r0 + i * RPP][Ops::apos(seg) * (16 / (int)sizeof(AT))]) = areg[i];
    };
    auto load_b = [&](BSet& bs, int k0) { Ops::load_b(bs, brow, bsc, k0); };
    // The MTX row tiles all run (rows past the tile in the last one repeat
    // the tile's first row in LDS, and their outputs are never stored): a
    // guard per row tile would make each MFMA wait for its own LDS read.
    auto compute = [&](BSet& bs, int buf, int k0) {
      const float sc8 = F == WFmt::FP8 ? static_cast<const float*>(bsc)[k0 / 128] : 0.f;
      Ops::template mma<MTX>(&As[buf][col][0], PITCH, 0, bs, sc8, kg, accx);
    };

    // Schedule: while stage s feeds the MFMAs, stage s+1's activations and
    // weights are in flight.  The compiler counts outstanding loads to place
    // its waits, and that count is only exact where every load is
    // unconditional: a conditional prefetch (or a load issued after the
    // prefetches and consumed in the same stage, as a per-stage scale load
    // was) makes it wait for everything, prefetch included.  So the
    // activations of rows past the tile are real loads, the scales come from
    // LDS, the last stage is peeled, and the common stage counts are fully
    // unrolled (a loop header also merges the counts conservatively).
    const int S = Kdim / KS;
    load_a(0);
    load_b(b0, 0);
    store_a(0);
    __syncthreads();
    auto unrolled = [&](auto SC) {
      constexpr int NS = decltype(SC)::value;
      static_for<0, NS>([&](auto J) {
        constexpr int st = decltype(J)::value;
        constexpr bool more = st + 1 < NS;
        if constexpr (st % 2 == 0) {
          if constexpr (more) {
            load_a((st + 1) * KS);
            load_b(b1, (st + 1) * KS);
          }
          compute(b0, 0, st * KS);
        } else {
          if constexpr (more) {
            load_a((st + 1) * KS);
            load_b(b0, (st + 1) * KS);
          }
          compute(b1, 1, st * KS);
        }
        if constexpr (more) {
          store_a((st + 1) % 2);
          __syncthreads();
        }
      });
    };
    if (S == 16) {
      unrolled(std::integral_constant<int, 16>{});
      return;
    }
    if (S == 4) {
      unrolled(std::integral_constant<int, 4>{});
      return;
    }
    int s = 0;
    for (; s + 2 < S; s += 2) {
      load_a((s + 1) * KS);
      load_b(b1, (s + 1) * KS);
      compute(b0, 0, s * KS);
      store_a(1);
      __syncthreads();
      load_a((s + 2) * KS);
      load_b(b0, (s + 2) * KS);
      compute(b1, 1, (s + 1) * KS);
      store_a(0);
      __syncthreads();
    }
    if (s + 1 < S) {
      load_a((s + 1) * KS);
      load_b(b1, (s + 1) * KS);
      compute(b0, 0, s * KS);
      store_a(1);
      __syncthreads();
      compute(b1, 1, (s + 1) * KS);
    } else {
      compute(b0, 0, s * KS);
    }
  }
};

// The GEMM of one tile with its own row-tile count: ceil(rows / 16), made
// wave-uniform so that one instantiation runs per tile.
template <class G, int MT>
__device__ __forceinline__ void run_rows(int rows, typename G::Lds& As, const typename G::AT* const (&asrc)[G::AV],
                                         const uint8_t* brow, const void* bsc, int Kdim, f32x4 (&acc)[MT]) {
  const int mtx = __builtin_amdgcn_readfirstlane((rows + 15) >> 4);
  static_for<1, MT>([&](auto M) {
    constexpr int MX = decltype(M)::value;
    if (mtx == MX) G::template run<MX>(As, asrc, brow, bsc, Kdim, acc);
  });
  if (mtx >= MT) G::template run<MT>(As, asrc, brow, bsc, Kdim, acc);
}

template <WFmt F, int MT, bool PK>
__global__ __launch_bounds__(64 * tiled_up_waves(MT)) void expert_up_tiled_kernel(TiledArgs a) {
  using G = TiledGemm<F, MT, PK, tiled_up_waves(MT)>;
  using AT = typename G::AT;
  using WT = typename G::WT;
  __shared__ typename G::Lds As;
  __shared__ float sc_s[2][kTiledMaxStages];
  int slot, slice;
  tile_of_block(blockIdx.x, a.n_slices, slot, slice);
  if (slot >= *a.tile_count) return;
  const Tile t = a.tiles[slot];
  const bool shared = t.expert == a.E;
  const int inter = shared ? a.Is : a.I;
  constexpr int UPC = tiled_up_cols(MT);
  if (slice * UPC >= inter) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int H = a.H;

  const AT* asrc[G::AV];
#pragma unroll
  for (int i = 0; i < G::AV; ++i) {
    const int r = tid / G::VPR + i * G::RPP;
    const int rr = r < t.rows ? r : 0;
    const int src = shared ? t.start + rr : a.pair_row[t.start + rr];
    asrc[i] = static_cast<const AT*>(a.x) + (size_t)src * H + (tid % G::VPR) * (16 / (int)sizeof(AT));
  }
  const size_t rowb = (size_t)H * sizeof(WT) / Frag<F>::kPack;  // bytes per weight row
  const uint8_t* W = shared ? static_cast<const uint8_t*>(a.sw)
                            : static_cast<const uint8_t*>(a.w) + (size_t)t.expert * 2 * a.I * rowb;
  const int i0 = slice * UPC + wave * 8;
  const int wr = col < 8 ? i0 + col : inter + i0 + col - 8;  // gate row / up row
  const uint8_t* brow = G::bchunk0(W, rowb, wr, i0 / 8, lane);
  const void* bsc = sc_s[col < 8 ? 0 : 1];
  if constexpr (F == WFmt::FP4) {
    // this lane's row of E8M0 bytes, read stage by stage
    const uint8_t* S = static_cast<const uint8_t*>(shared ? a.sws : a.ws);
    if (!shared) S += (size_t)t.expert * 2 * a.I * (H / 32);
    bsc = S + (size_t)wr * (H / 32);
  }
  if constexpr (F == WFmt::FP8) {
    const float* S = static_cast<const float*>(shared ? a.sws : a.ws);
    if (!shared) S += (size_t)t.expert * (2 * a.I / 128) * (H / 128);
    // the workgroup's gate rows share one 128-row scale block, its up rows
    // another; the first stage's barrier orders these writes before any read
    const int ns = H / 128;
    const int srow[2] = {(slice * UPC) / 128, (inter + slice * UPC) / 128};
    for (int i = tid; i < 2 * ns; i += G::THREADS) sc_s[i / ns][i % ns] = S[(size_t)srow[i / ns] * ns + i % ns];
  }
  f32x4 acc[MT];
  run_rows<G, MT>(t.rows, As, asrc, brow, bsc, H, acc);

  AT* h = static_cast<AT*>(a.h) +
          (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float gate = acc[mt][v];
      const float up = shfl_xor_f(gate, 8);
      const int m = mt * 16 + kg * 4 + v;
      if (col < 8 && m < t.rows) store_act<AT>(h + (size_t)m * inter + i0 + col, silu(gate) * up);
    }
}

template <WFmt F, int MT, bool PK>
__global__ __launch_bounds__(64 * tiled_waves(MT)) void expert_down_tiled_kernel(TiledArgs a) {
  using G = TiledGemm<F, MT, PK>;
  using AT = typename G::AT;
  using WT = typename G::WT;
  __shared__ typename G::Lds As;
  __shared__ float sc_s[2][kTiledMaxStages];
  int slot, slice;
  tile_of_block(blockIdx.x, a.n_slices, slot, slice);
  if (slot >= *a.tile_count) return;
  const Tile t = a.tiles[slot];
  const bool shared = t.expert == a.E;
  const int inter = shared ? a.Is : a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const int H = a.H;

  const AT* hb = static_cast<const AT*>(a.h) +
                 (shared ? (size_t)a.N * a.K * a.I + (size_t)t.start * a.Is : (size_t)t.start * a.I);
  const AT* asrc[G::AV];
#pragma unroll
  for (int i = 0; i < G::AV; ++i) {
    const int r = tid / G::VPR + i * G::RPP;
    asrc[i] = hb + (size_t)(r < t.rows ? r : 0) * inter + (tid % G::VPR) * (16 / (int)sizeof(AT));
  }
  const size_t rowb = (size_t)inter * sizeof(WT) / Frag<F>::kPack;  // bytes per weight row
  const uint8_t* W = shared ? static_cast<const uint8_t*>(a.sw)
                            : static_cast<const uint8_t*>(a.w) + (size_t)t.expert * H * rowb;
  const int c0 = slice * tiled_down_cols(MT) + wave * 16;
  const int orow = c0 + col;  // W2 row = output column
  const uint8_t* brow = G::bchunk0(W, rowb, orow, c0 / 16, lane);
  const void* bsc = sc_s[0];
  if constexpr (F == WFmt::FP4) {
    const uint8_t* S = static_cast<const uint8_t*>(shared ? a.sws : a.ws);
    if (!shared) S += (size_t)t.expert * H * (a.I / 32);
    bsc = S + (size_t)orow * (inter / 32);
  }
  if constexpr (F == WFmt::FP8) {
    // the workgroup's 64 or 128 output rows lie in one 128-row scale block row
    const float* S = static_cast<const float*>(shared ? a.sws : a.ws);
    if (!shared) S += (size_t)t.expert * (H / 128) * (a.I / 128);
    const int ns = inter / 128;
    const int srow = (slice * tiled_down_cols(MT)) / 128;
    for (int i = tid; i < ns; i += G::THREADS) sc_s[0][i] = S[(size_t)srow * ns + i];
  }
  f32x4 acc[MT];
  run_rows<G, MT>(t.rows, As, asrc, brow, bsc, inter, acc);

  const size_t y0 = ((shared ? (size_t)a.N * a.K : 0) + (size_t)t.start) * H;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = mt * 16 + kg * 4 + v;
      if (m < t.rows) {
        const size_t at = y0 + (size_t)m * H + c0 + col;
        if (a.y_act) store_act<AT>(static_cast<AT*>(a.y) + at, acc[mt][v]);
        else static_cast<float*>(a.y)[at] = acc[mt][v];
      }
    }
}

template <bool kUp, WFmt F, int MT, bool PK>
static void launch_tiled(const TiledArgs& a, unsigned grid, hipStream_t s) {
  if constexpr (kUp)
    expert_up_tiled_kernel<F, MT, PK><<<grid, 64 * tiled_up_waves(MT), 0, s>>>(a);
  else
    expert_down_tiled_kernel<F, MT, PK><<<grid, 64 * tiled_waves(MT), 0, s>>>(a);
}

template <bool kUp, WFmt F, bool PK>
static void launch_tiled_mt(const TiledArgs& a, int mt_max, unsigned grid, hipStream_t s) {
  switch (mt_max) {
    case 2: launch_tiled<kUp, F, 2, PK>(a, grid, s); break;
    case 4: launch_tiled<kUp, F, 4, PK>(a, grid, s); break;
    case 6: launch_tiled<kUp, F, 6, PK>(a, grid, s); break;
    default: launch_tiled<kUp, F, 8, PK>(a, grid, s); break;
  }
}

template <bool kUp, WFmt F>
static void launch_tiled_mt(const TiledArgs& a, bool panels, int mt_max, unsigned grid, hipStream_t s) {
  if (panels) launch_tiled_mt<kUp, F, true>(a, mt_max, grid, s);
  else launch_tiled_mt<kUp, F, false>(a, mt_max, grid, s);
}

hipError_t launch_expert_tiled(const Plan& p, const cmoe_weights& w, const void* x, bool up,
                               hipStream_t s) {
  TiledArgs a;
  a.x = x;
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
  a.n_slices = up ? (p.I > p.Is ? p.I : p.Is) / tiled_up_cols(p.mt_max) : p.H / tiled_down_cols(p.mt_max);
  const unsigned grid = tile_grid(p.max_tiles, a.n_slices);
  const WFmt f = p.wt == CMOE_FP4_E2M1   ? WFmt::FP4
                 : p.wt == CMOE_FP8_E4M3 ? WFmt::FP8
                 : p.wt == CMOE_F32      ? WFmt::F32
                                         : WFmt::BF16;
  if (up) {
    if (f == WFmt::FP4) launch_tiled_mt<true, WFmt::FP4>(a, p.panels, p.mt_max, grid, s);
    else if (f == WFmt::FP8) launch_tiled_mt<true, WFmt::FP8>(a, p.panels, p.mt_max, grid, s);
    else if (f == WFmt::F32) launch_tiled_mt<true, WFmt::F32>(a, p.panels, p.mt_max, grid, s);
    else launch_tiled_mt<true, WFmt::BF16>(a, p.panels, p.mt_max, grid, s);
  } else {
    if (f == WFmt::FP4) launch_tiled_mt<false, WFmt::FP4>(a, p.panels, p.mt_max, grid, s);
    else if (f == WFmt::FP8) launch_tiled_mt<false, WFmt::FP8>(a, p.panels, p.mt_max, grid, s);
    else if (f == WFmt::F32) launch_tiled_mt<false, WFmt::F32>(a, p.panels, p.mt_max, grid, s);
    else launch_tiled_mt<false, WFmt::BF16>(a, p.panels, p.mt_max, grid, s);
  }
  return hipGetLastError();
}

}  // namespace cmoe
