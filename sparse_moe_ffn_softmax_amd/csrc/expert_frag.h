// expert_frag.h -- MFMA operand fragments shared by the expert GEMM kernels
// (gfx950, wave64).
//
// v_mfma_f32_16x16x32_bf16 (layout checked on gfx950): lane l supplies
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16] and receives
// D[4*(l/16) + v][l%16], v = 0..3.  v_mfma_f32_16x16x4_f32 uses the same
// layout with one k per lane.  The k order inside a step only has to be the
// same for A and B, so each lane loads 16 contiguous bytes of its row.
//
// Inside a 128-deep stage, lane group kg (= l/16) covers k kGroupK*kg + u*kStepK
// .. +kLane at MFMA step u.  For bf16 and fp32 that is the natural order
// (kGroupK = kLane, kStepK = kStep).  For fp4 each lane group takes a
// contiguous 32 k (one MX scale block), so its 32 codes are one 16-byte load
// and it needs one scale per stage.  fp8 departs from its kGroupK/kStepK in
// both kernel families: lane group kg takes k [16kg, 16kg+16) of each 64-deep
// pair of steps, so its 16 codes are one 16-byte load per two steps.  In
// every format a lane group thus reads 16 weight bytes at byte 16kg of each
// 64 bytes of its row (one weight chunk, below).
#pragma once
#include "cmoe_device.h"

namespace cmoe {

enum class WFmt { BF16, F32, FP8, FP4 };

// ---------------------------------------------------------------------------
// fragments: what one lane loads for one k step
// ---------------------------------------------------------------------------
template <WFmt F>
struct Frag;

template <>
struct Frag<WFmt::BF16> {
  static constexpr int kStep = 32;  // k per MFMA step
  static constexpr int kLane = 8;   // elements per lane per step
  static constexpr int kGroupK = kLane, kStepK = kStep;
  static constexpr int kPack = 1;   // weight elements per WT unit
  using A = u32x4;                  // 8 bf16
  using B = u32x4;
  using AT = uint16_t;
  using WT = uint16_t;
  static __device__ __forceinline__ A load_a(const AT* p) { return *reinterpret_cast<const u32x4*>(p); }
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
  static constexpr int kGroupK = kLane, kStepK = kStep;
  static constexpr int kPack = 1;
  using A = f32x4;
  using B = f32x4;
  using AT = float;
  using WT = float;
  static __device__ __forceinline__ A load_a(const AT* p) { return *reinterpret_cast<const f32x4*>(p); }
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
  static constexpr int kGroupK = kLane, kStepK = kStep;
  static constexpr int kPack = 1;
  using A = u32x4;  // 8 bf16
  using B = u32x2;  // 8 e4m3 codes
  using AT = uint16_t;
  using WT = uint8_t;
  static __device__ __forceinline__ A load_a(const AT* p) { return *reinterpret_cast<const u32x4*>(p); }
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
  static __device__ __forceinline__ f32x4 mma(A a, B b, f32x4 c) { return mma_wide(a, widen(b), c); }
  // the MFMA on weights already widened by widen()
  static __device__ __forceinline__ f32x4 mma_wide(A a, u32x4 wb, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, wb),
                                                   c, 0, 0, 0);
  }
};

// MXFP4 (OCP Microscaling): E2M1 codes, two per byte, low nibble first, and
// one E8M0 scale byte per 32 consecutive elements of a row.  Widened to bf16
// exactly: an E2M1 value times a power of two is a bf16 value
// (v_cvt_scalef32_pk_bf16_fp4; nibble order and exactness checked on gfx950
// over all 256 bytes).  Scale bytes 1..254 (2^-126 .. 2^127) are supported.
template <>
struct Frag<WFmt::FP4> {
  static constexpr int kStep = 32;
  static constexpr int kLane = 8;
  static constexpr int kGroupK = 32, kStepK = 8;
  static constexpr int kPack = 2;
  using A = u32x4;      // 8 bf16
  using B = uint32_t;   // 8 E2M1 codes
  using AT = uint16_t;
  using WT = uint8_t;
  static __device__ __forceinline__ A load_a(const AT* p) { return *reinterpret_cast<const u32x4*>(p); }
  static __device__ __forceinline__ A zero_a() { return u32x4{0u, 0u, 0u, 0u}; }
  // 2^(s-127) as an fp32 bit pattern (s = 1..254: a normal float)
  static __device__ __forceinline__ float scale_of(uint32_t s) { return __uint_as_float(s << 23); }
  static __device__ __forceinline__ u32x4 widen(B b, float sc) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, sc, 3);
    return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
  }
  static __device__ __forceinline__ f32x4 mma(A a, B b, float sc, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, widen(b, sc)), c, 0, 0,
                                                   0);
  }
};

// Weights arrive in 16-byte chunks: chunk q of a lane is the 16 bytes its
// lane group needs from bytes [64q, 64q+64) of its weight row, counted from
// the lane's first k.  Chunk q is kChunk<PK> bytes after chunk 0: the next 64
// bytes of the row in row-major storage, the next 1 KiB unit of the panel in
// MFMA-panel storage (CMOE_LAYOUT_PANELS in clover_moe.h).
template <bool PK>
constexpr int kChunk = PK ? 1024 : 64;

// One weight chunk.  Panel chunks are read non-temporally: a wave's load
// there covers 1 KiB of contiguous whole cache lines, which the hint streams
// past the caches (row-major chunks are half cache lines, and the hint would
// evict each line before its other half is read).
template <bool PK>
__device__ __forceinline__ u32x4 load_chunk(const uint8_t* p) {
  if constexpr (PK) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

template <typename T>
__device__ __forceinline__ void store_act(T* p, float v);
template <>
__device__ __forceinline__ void store_act<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_act<float>(float* p, float v) { *p = v; }

}  // namespace cmoe
