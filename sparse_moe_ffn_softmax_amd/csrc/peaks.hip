// peaks.hip -- achievable-peak probes for the benchmark (libclover_moe_peaks.so).
//
// Not part of the C ABI of include/clover_moe.h and not used by any call of
// it: the benchmark loads this library on its own to measure, on the GPU it
// runs on, what a plain kernel reaches, so that the kernels of the MoE path
// can be reported against both the datasheet peaks and these measured ones.
//
//  cmoe_peak_read:  every 16-byte vector of a buffer read once, with the
//                   non-temporal hint, each wave load covering 1 KiB of
//                   consecutive cache lines (the pattern of the MFMA-panel
//                   weight loads); pattern 0 strides the grid over the buffer
//                   with 4 loads in flight per thread, pattern 1 gives each
//                   workgroup a contiguous slab with 8 loads in flight per
//                   thread.  The XOR of everything read is written per
//                   workgroup so the loads cannot be dropped.
//  cmoe_peak_mfma:  every wave issues `iters` rounds of MFMAs on independent
//                   register chains: bf16 16x16x32 and 32x32x16, and the
//                   f8f6f4 16x16x128 and 32x32x64 with e4m3 operands and unit
//                   scales.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

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

__global__ __launch_bounds__(256) void peak_read_slab_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = per * blockIdx.x, hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(buf + i + j * 256);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < hi; i += 256) {
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

// Each chain j has its own B operand and its own start value, so that no two
// chains compute the same thing (identical chains are merged by the compiler).
template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma_kernel(f32x4* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  constexpr bool k32 = KIND >= 2;           // 32x32 output tiles: 4 chains of 16 floats
  constexpr int NC = k32 ? 4 : 8;
  typedef __attribute__((ext_vector_type(16))) float f32x16;
  using Acc = typename std::conditional<k32, f32x16, f32x4>::type;
  Acc acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    acc[c] = Acc{};
    acc[c][0] = (float)c;
  }
  if constexpr (KIND == 0 || KIND == 2) {
    bf16x8 a, b[NC];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = (__bf16)(float)((lane + j) & 7);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) b[c][j] = (__bf16)(float)((lane * 3 + j + c) & 7);
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (KIND == 0) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[c], acc[c], 0, 0, 0);
        else acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[c], acc[c], 0, 0, 0);
      }
    }
  } else {
    i32x8 a, b[NC];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = 0x38383838 + ((lane + j) & 3);  // e4m3 codes near 1.0
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) b[c][j] = 0x38383838 + ((lane * 3 + j + c) & 3);
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (KIND == 1)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[c], acc[c], 0, 0, 0, 127, 0, 127);
        else
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[c], acc[c], 0, 0, 0, 127, 0, 127);
      }
    }
  }
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) s[v] += acc[c][v];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) of device memory at `buf` (16-byte
// aligned) with `blocks` workgroups of 256 threads in the given pattern (0 or
// 1, above); sink: `blocks` uint32.  Returns the hipError_t of the launch.
int cmoe_peak_read(int pattern, const void* buf, size_t bytes, void* sink, int blocks, void* stream) {
  if (!buf || !sink || blocks < 1 || bytes % 16 || (uintptr_t)buf % 16 || (pattern != 0 && pattern != 1))
    return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pattern == 0)
    peak_read_kernel<<<blocks, 256, 0, s>>>(static_cast<const u32x4*>(buf), bytes / 16,
                                            static_cast<uint32_t*>(sink));
  else
    peak_read_slab_kernel<<<blocks, 256, 0, s>>>(static_cast<const u32x4*>(buf), bytes / 16,
                                                 static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// `blocks` workgroups of 256 threads, each wave `iters` rounds of MFMAs on
// independent chains; out: blocks * 256 * 4 floats.  kind 0: bf16 16x16x32
// (8 chains), 1: fp8 16x16x128 (8 chains), 2: bf16 32x32x16 (4 chains),
// 3: fp8 32x32x64 (4 chains).
int cmoe_peak_mfma(int kind, void* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1 || kind < 0 || kind > 3) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  f32x4* o = static_cast<f32x4*>(out);
  switch (kind) {
    case 0: peak_mfma_kernel<0><<<blocks, 256, 0, s>>>(o, iters); break;
    case 1: peak_mfma_kernel<1><<<blocks, 256, 0, s>>>(o, iters); break;
    case 2: peak_mfma_kernel<2><<<blocks, 256, 0, s>>>(o, iters); break;
    default: peak_mfma_kernel<3><<<blocks, 256, 0, s>>>(o, iters); break;
  }
  return (int)hipGetLastError();
}

// flop issued per wave per round of cmoe_peak_mfma of each kind
long long cmoe_peak_mfma_flop(int kind) {
  switch (kind) {
    case 0: return 8LL * 16 * 16 * 32 * 2;
    case 1: return 8LL * 16 * 16 * 128 * 2;
    case 2: return 4LL * 32 * 32 * 16 * 2;
    default: return 4LL * 32 * 32 * 64 * 2;
  }
}

}  // extern "C"
