// quant.hip -- bf16 rows to MXFP8 (OCP e4m3 codes with one E8M0 scale per 32
// consecutive elements of a row), the activation format of the fp8-MFMA
// grouped GEMMs (expert_many.hip, clover_moe.h: cmoe_options.activation_fp8).
//
// For each group of 32 values with largest magnitude amax the scale is 2^e
// with the smallest e such that amax / 2^e <= 448 (the largest e4m3
// magnitude), and each code is v / 2^e rounded to the nearest e4m3 value, ties
// to even (v_cvt_pk_fp8_f32; equal to torch's float8_e4m3fn cast on all
// values up to 448, checked on gfx950).  Dividing by 2^e is exact, so a code
// differs from v / 2^e by at most half an e4m3 unit in the last place.
#include "cmoe_device.h"
#include "cmoe_launch.h"
#include "expert_frag32.h"

namespace cmoe {

// One thread per group: 64 bytes of bf16 in, 32 bytes of codes and one scale
// byte out.  src [rows, cols], dst [rows, cols], scales [rows, cols/32].
__global__ __launch_bounds__(256) void quant_mx8_kernel(const uint16_t* __restrict__ src,
                                                        uint8_t* __restrict__ dst,
                                                        uint8_t* __restrict__ scales, long long groups) {
  const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= groups) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + g * 32);
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = s[i];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] & 0xFFFF0000u)));
    }
  const int sb = mx8_scale_byte(amax);
  // 2^-e as a float: exponent field 254 - sb (sb = e + 127 in [0, 254])
  const float inv = __uint_as_float((uint32_t)(254 - sb) << 23);
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[i][0] << 16) * inv,
                                             __uint_as_float(v[i][0] & 0xFFFF0000u) * inv, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[i][1] << 16) * inv,
                                         __uint_as_float(v[i][1] & 0xFFFF0000u) * inv, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[i][2] << 16) * inv,
                                             __uint_as_float(v[i][2] & 0xFFFF0000u) * inv, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[i][3] << 16) * inv,
                                         __uint_as_float(v[i][3] & 0xFFFF0000u) * inv, hi, true);
    out[i / 2][2 * (i % 2)] = (uint32_t)lo;
    out[i / 2][2 * (i % 2) + 1] = (uint32_t)hi;
  }
  u32x4* d = reinterpret_cast<u32x4*>(dst + g * 32);
  d[0] = out[0];
  d[1] = out[1];
  scales[g] = (uint8_t)sb;
}

hipError_t launch_quant_mx8(const void* src, long long rows, int cols, void* dst, void* scales, hipStream_t s) {
  const long long groups = rows * (cols / 32);
  const unsigned grid = (unsigned)((groups + 255) / 256);
  quant_mx8_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), static_cast<uint8_t*>(dst),
                                        static_cast<uint8_t*>(scales), groups);
  return hipGetLastError();
}

}  // namespace cmoe
