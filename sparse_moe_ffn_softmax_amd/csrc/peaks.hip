// peaks.hip -- achievable-peak probes for the benchmark (libclover_moe_peaks.so).
//
// Not part of the C ABI of include/clover_moe.h and not used by any call of
// it: the benchmark loads this library on its own to measure, on the GPU it
// runs on, what a plain kernel reaches, so that the kernels of the MoE path
// can be reported against both the datasheet peaks and these measured ones.
//
//  cmoe_peak_read:  every 16-byte vector of a buffer read once, with the
//                   non-temporal hint, by a grid of 16-lane groups reading 256
//                   contiguous bytes per load instruction (the pattern of the
//                   MFMA-panel weight loads); the XOR of everything read is
//                   written per workgroup so the loads cannot be dropped.
//  cmoe_peak_mfma:  every wave issues `iters` rounds of 8 independent MFMAs
//                   on register operands: kind 0 = v_mfma_f32_16x16x32_bf16
//                   (16384 flop each), kind 1 = v_mfma_scale_f32_16x16x128_f8f6f4
//                   with e4m3 operands and unit scales (65536 flop each).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^
           d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
    for (int t = 0; t < 256; ++t) v ^= red[t];
    sink[blockIdx.x] = v;
  }
}

template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma_kernel(f32x4* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = (__bf16)(float)((lane + j) & 7);
      b[j] = (__bf16)(float)((lane * 3 + j) & 7);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
  } else {
    i32x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = 0x38383838 + ((lane + j) & 3);  // e4m3 codes near 1.0
      b[j] = 0x38383838 + ((lane * 3 + j) & 3);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
    }
  }
  f32x4 s = acc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) s += acc[j];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) of device memory at `buf` (16-byte
// aligned) with `blocks` workgroups of 256 threads; sink: `blocks` uint32.
// Returns the hipError_t of the launch.
int cmoe_peak_read(const void* buf, size_t bytes, void* sink, int blocks, void* stream) {
  if (!buf || !sink || blocks < 1 || bytes % 16 || (uintptr_t)buf % 16) return (int)hipErrorInvalidValue;
  peak_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// `blocks` workgroups of 256 threads, each wave `iters` rounds of 8 MFMAs;
// out: blocks * 256 * 4 floats.  kind 0: bf16 16x16x32, kind 1: fp8 16x16x128.
int cmoe_peak_mfma(int kind, void* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1 || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0) peak_mfma_kernel<0><<<blocks, 256, 0, s>>>(static_cast<f32x4*>(out), iters);
  else peak_mfma_kernel<1><<<blocks, 256, 0, s>>>(static_cast<f32x4*>(out), iters);
  return (int)hipGetLastError();
}

// flop of one MFMA of each kind
long long cmoe_peak_mfma_flop(int kind) { return kind == 0 ? 16384LL : 65536LL; }

}  // extern "C"
