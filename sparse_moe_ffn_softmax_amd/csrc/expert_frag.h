// expert_frag.h -- MFMA operand fragments shared by the expert GEMM kernels
// (gfx950, wave64).
//
// v_mfma_f32_16x16x32_bf16 (layout checked on gfx950): lane l supplies
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16] and receives
// D[4*(l/16) + v][l%16], v = 0..3.  v_mfma_f32_16x16x4_f32 uses the same
// layout with one k per lane.  The k order inside a step only has to be the
// same for A and B, so each lane loads 16 contiguous bytes of its row.
#pragma once
#include "cmoe_device.h"

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

template <typename T>
__device__ __forceinline__ void store_act(T* p, float v);
template <>
__device__ __forceinline__ void store_act<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_act<float>(float* p, float v) { *p = v; }

}  // namespace cmoe
