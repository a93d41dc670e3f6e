// expert_frag32.h -- weight and activation fragments of the grouped GEMMs that
// run on v_mfma_f32_32x32x16_bf16 (gfx950, wave64).
//
// On gfx950 the 32x32x16 bf16 MFMA sustains about twice the flop rate of the
// 16x16x32 one (measured: 2.18 against 1.21 PFLOP/s over independent chains),
// so the kernels for calls with many rows per expert use it.
//
// Lane layout (checked on gfx950 with an in-bounds probe): lane l supplies
// A[l%32][8(l/32) .. +8] and B[8(l/32) .. +8][l%32], and receives
// D[8(v/4) + 4(l/32) + v%4][l%32], v = 0..15.  MFMA needs A and B to agree
// on the k order only, so the k order of a step is chosen to suit the loads.
//
// A wave owns 32 weight rows: lane l's row is l%32 and its half is h = l/32.
// The rows are read in 128-deep stages; a stage of a row is 1, 2 or 4
// segments of 64 bytes (4-bit, fp8, bf16), and the lane takes two 16-byte
// pieces of each segment, pieces 2h and 2h+1.  In the MFMA-panel layout
// (clover_moe.h) 32 rows are two consecutive panels and piece p of segment q
// of panel row i is bytes [16(i + 16p), +16) of the panel's unit q, so every
// load of a wave covers whole, consecutive 256-byte runs; row-major, it is
// bytes 64q + 16p of the row.
//
// Activations are staged in LDS as rows of 128 bf16 per stage (256 bytes)
// with a 272-byte pitch.  Measured on gfx950 with 16 waves reading (rows
// l%32, one chunk per half-wave), against a contiguous read: pitch 272
// 0.92-1.05x, 288 1.33-1.41x, 320 2.1x, 256 3.5x.  A fragment's address is
// then a per-lane base plus an immediate offset.  (An unpadded row with an
// XOR-swizzled chunk order is also about as fast, but each fragment address
// is then its own register, and the compiler keeps them all live across the
// unit loop.)
#pragma once
#include "cmoe_device.h"
#include "expert_frag.h"

namespace cmoe {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

template <WFmt F, bool PK>
struct W32 {
  static_assert(F == WFmt::BF16 || F == WFmt::FP8 || F == WFmt::FP4, "16-bit activation formats");
  static constexpr int SEGS = F == WFmt::BF16 ? 4 : F == WFmt::FP8 ? 2 : 1;  // 64-byte segments per stage
  static constexpr int NC = 2 * SEGS;                                       // 16-byte pieces per lane
  static constexpr int SEGSTRIDE = PK ? 1024 : 64;
  static constexpr int PSTRIDE = PK ? 256 : 16;
  static constexpr int STEPS = 8;  // 32x32x16 MFMA steps per stage

  // One stage of this lane's weights.  sc: fp8: the fp32 block scale of the
  // lane's row for this stage (bits); fp4: the E8M0 bytes of its two pieces.
  struct Stage {
    u32x4 c[NC];
    uint32_t sc;
  };

  // This lane's piece 0 of segment 0: `row` is its weight row (row-major),
  // `panel` the panel holding it (panels).
  static __device__ __forceinline__ const uint8_t* lane_base(const uint8_t* W, size_t rowb, int row, int panel,
                                                             int lane) {
    const int rl = lane & 31, h = lane >> 5;
    if constexpr (PK) return W + (size_t)panel * 16 * rowb + 16 * (rl & 15) + 512 * h;
    else return W + (size_t)row * rowb + 32 * h;
  }

  // Stage s of this lane's row.  sc_fp8: the row's fp32 block scales (one per
  // 128 k); sc_fp4: the row's E8M0 bytes (one per 32 k).
  static __device__ __forceinline__ void load(Stage& st, const uint8_t* base, const float* sc_fp8,
                                              const uint8_t* sc_fp4, int s, int lane) {
#pragma unroll
    for (int q = 0; q < SEGS; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        st.c[2 * q + j] = load_chunk<PK>(base + (size_t)(s * SEGS + q) * SEGSTRIDE + j * PSTRIDE);
    if constexpr (F == WFmt::FP8) st.sc = __float_as_uint(sc_fp8[s]);
    else if constexpr (F == WFmt::FP4)
      st.sc = *reinterpret_cast<const uint16_t*>(sc_fp4 + 4 * s + 2 * (lane >> 5));
    else st.sc = 0;
  }

  // The B operand (8 bf16) of MFMA step t.  Step t takes, per half h:
  //   bf16: piece t          -> k 32(t/2) + 16h + 8(t%2) .. +8
  //   fp8:  piece t/2, codes 8(t%2) .. +8 -> k 64(t/4) + 32h + 16((t/2)%2) + 8(t%2) .. +8
  //   fp4:  piece t/4, codes 8(t%4) .. +8 -> k 64h + 32(t/4) + 8(t%4) .. +8
  // fp8 codes widen to bf16 exactly; fp4 codes widen with their E8M0 scale
  // (exact).  The fp8 block scale is applied by the caller.
  static __device__ __forceinline__ u32x4 bop(const Stage& st, int t) {
    if constexpr (F == WFmt::BF16) {
      return st.c[t];
    } else if constexpr (F == WFmt::FP8) {
      const u32x4 p = st.c[t >> 1];
      u32x2 codes = (t & 1) ? u32x2{p[2], p[3]} : u32x2{p[0], p[1]};
      return Frag<WFmt::FP8>::widen(codes);
    } else {
      const uint32_t codes = st.c[t >> 2][t & 3];
      return Frag<WFmt::FP4>::widen(codes, Frag<WFmt::FP4>::scale_of((st.sc >> (8 * (t >> 2))) & 0xFFu));
    }
  }

  // fp8: the raw codes of step t, and their exact widening (a caller widening
  // once per row tile keeps only the codes live)
  static __device__ __forceinline__ u32x2 codes8(const Stage& st, int t) {
    const u32x4 p = st.c[t >> 1];
    return (t & 1) ? u32x2{p[2], p[3]} : u32x2{p[0], p[1]};
  }

  // The 16-byte activation chunk (8 k) of step t for half h, within a stage
  static __device__ __forceinline__ int ack(int t, int h) {
    if constexpr (F == WFmt::BF16) return 4 * (t >> 1) + 2 * h + (t & 1);
    else if constexpr (F == WFmt::FP8) return 8 * (t >> 2) + 4 * h + 2 * ((t >> 1) & 1) + (t & 1);
    else return 8 * h + 4 * (t >> 2) + (t & 3);
  }
};

// ---------------------------------------------------------------------------
// fp8 activations (MXFP8: OCP e4m3 codes with an E8M0 scale per 32
// consecutive elements of a row) times fp8 weights on
// v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Scale blocks of that MFMA (checked on gfx950 with single-lane scale
// changes): of the 32 codes lane l supplies, the first 16 of lanes r and r+32
// form one 32-element block, scaled by lane r's E8M0 byte, and their last 16
// the other block, scaled by lane r+32's.  A 64-deep step over k [64q, 64q+64)
// therefore gives lane (r, h), h = l/32, the codes k 64q + 16h .. +16 and
// 64q + 32 + 16h .. +16, and its scale byte is that of group 2q + h (k
// 64q + 32h .. +32), so each activation group of 32 consecutive k is one
// scale block.  The weights follow the same k order: pieces h and h+2 of each
// 64-byte segment; their block scale is applied by the caller (unit MFMA
// scale, byte 127).
// ---------------------------------------------------------------------------
template <bool PK>
struct W32Mx {
  static constexpr int SEGS = 2;           // 64-byte segments per 128-deep stage
  static constexpr int SEGSTRIDE = PK ? 1024 : 64;
  static constexpr int PSTRIDE = PK ? 512 : 32;  // piece h+2 after piece h
  struct Stage {
    u32x4 c[4];      // [2q]: piece h of segment q, [2q+1]: piece h+2
    uint32_t sc;     // the row's fp32 block scale for the stage (bits)
  };
  static __device__ __forceinline__ const uint8_t* lane_base(const uint8_t* W, size_t rowb, int row, int panel,
                                                             int lane) {
    const int rl = lane & 31, h = lane >> 5;
    if constexpr (PK) return W + (size_t)panel * 16 * rowb + 16 * (rl & 15) + 256 * h;
    else return W + (size_t)row * rowb + 16 * h;
  }
  static __device__ __forceinline__ void load(Stage& st, const uint8_t* base, const float* sc_fp8, int s) {
#pragma unroll
    for (int q = 0; q < SEGS; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        st.c[2 * q + j] = load_chunk<PK>(base + (size_t)(s * SEGS + q) * SEGSTRIDE + j * PSTRIDE);
    st.sc = __float_as_uint(sc_fp8[s]);
  }
  static __device__ __forceinline__ i32x8 operand(const Stage& st, int q) {
    const u32x4 a = st.c[2 * q], b = st.c[2 * q + 1];
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  }
};

// fp8 x fp8 MFMA with the activation's E8M0 byte (scale_a) and unit weight scale
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, int scale_a, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, 127);
}

// Staged fp8 activation rows: 128 codes per stage with a 144-byte pitch (the
// 16 rows one read touches fall in distinct bank groups).
constexpr int kA8Pitch = 144;

// The two 16-byte pieces of lane (r, h)'s step q from a staged fp8 row
__device__ __forceinline__ i32x8 lds_frag8(const uint8_t* row, int q, int h) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(row + 64 * q + 16 * h);
  const u32x4 b = *reinterpret_cast<const u32x4*>(row + 64 * q + 32 + 16 * h);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// E8M0 scale of a group of 32 values whose largest magnitude is amax: the
// smallest e with amax / 2^e <= 448 (the largest e4m3 magnitude), from the
// bits of amax (448 = 1.75 * 2^8); byte e + 127, clamped to [0, 254].
__device__ __forceinline__ int mx8_scale_byte(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ex = (int)((b >> 23) & 0xFFu);       // biased exponent (0: zero or subnormal)
  if (ex == 0) return 0;                          // 2^-127: codes of such values are 0 or tiny
  const int e = (ex - 127) - ((b & 0x7FFFFFu) <= 0x600000u ? 8 : 7);
  const int s = e + 127;
  return s < 0 ? 0 : (s > 254 ? 254 : s);
}

constexpr int kA32Pitch = 136;  // elements per staged activation row (272 bytes)

// Activation fragment: row r of a staged LDS stage, chunk c (8 bf16)
__device__ __forceinline__ u32x4 lds_frag(const uint16_t* stage, int r, int c) {
  return *reinterpret_cast<const u32x4*>(stage + (size_t)r * kA32Pitch + (c << 3));
}

}  // namespace cmoe
