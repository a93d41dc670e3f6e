// combine.hip -- gate-weighted combine of the routed expert outputs plus the
// shared expert (Clover-35B-A3B-Preview CMF model card, introduction: top-8
// routed experts and one shared expert besides them):
//
//   out[r] = y_shared[r] + sum_j gate[r,j] * y[pos(r,j)]     (slots ascending)
//
// accumulated in fp32 with one rounding to the activation dtype at the end.
// y is fp32, or bf16 for calls with many rows per expert (the down GEMM
// rounds each pair's output once there).
// The order is fixed, so results are bitwise identical from run to run (no
// floating-point atomics anywhere on the path).
#include "cmoe_device.h"
#include "cmoe_launch.h"

namespace cmoe {

template <typename OT>
__device__ __forceinline__ void store4(OT* p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4 v) {
  u32x2 o;
  o[0] = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  o[1] = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<u32x2*>(p) = o;
}

// four y values from fp32 or bf16 storage
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const uint16_t* p) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
               __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
}

template <typename OT, typename YT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ gates,
                                                      OT* __restrict__ out, int N, int H, int K,
                                                      int has_shared,
                                                      const uint8_t* __restrict__ live) {
  const int r = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  // Every load is unconditional, so that all of them are in flight at once
  // (a conditional load makes the compiler wait for everything issued before
  // it): slots past K read a clamped index and are masked, empty slots read
  // pair row 0 and add nothing, the shared row is row 0 when there is no
  // shared expert, and the row's live flag is a byte of pair_pos when there
  // is no mask.  Then the sum, in the order above.
  const uint8_t* lp = live ? live + r : reinterpret_cast<const uint8_t*>(pair_pos);
  const uint8_t lv = *lp;
  // The row's positions and gates come in one vector load (lane j of the
  // wave reads slot j) and are handed to every lane by readlane; as eight
  // uniform loads the compiler issued them one after another.
  const int NK = N * K;
  const int slot_i = min(r * K + (int)(threadIdx.x & 7), NK - 1);
  const int pv = pair_pos[slot_i];
  const float gv = gates[slot_i];
  int pos[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pj = __builtin_amdgcn_readlane(pv, j);
    pos[j] = j < K ? pj : -1;
    g[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gv), j));
  }
  // (the flag passes through a vector register so that the shared row is a
  // plain load and a select, not a branch that waits for the loads above)
  int hs = has_shared;
  asm volatile("" : "+v"(hs));
  const f32x4 ysh = load4(y + (hs ? (size_t)NK + r : (size_t)0) * H + c);
  f32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = load4(y + (size_t)max(pos[j], 0) * H + c);
  // keep every load here: sunk into the conditional sums below, a load
  // issues only after the ones before it have been waited for
#pragma unroll
  for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(v[j]));
  asm volatile("" ::"v"(ysh));
  if (live && !lv) return;  // a resolved row keeps the caller's cached output
  f32x4 acc = hs ? ysh : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (pos[j] < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(g[j], v[j][i], acc[i]);
  }
  store4<OT>(out + (size_t)r * H + c, acc);
}

hipError_t launch_combine(const Plan& p, void* out, hipStream_t s) {
  dim3 grid((p.H / 4 + 255) / 256, p.N);
  const int sh = p.Is > 0;
  if (p.act == CMOE_BF16) {
    uint16_t* o = static_cast<uint16_t*>(out);
    if (p.y_act)
      combine_kernel<uint16_t, uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(p.y), p.pair_pos,
                                                              p.gates, o, p.N, p.H, p.K, sh, p.live);
    else
      combine_kernel<uint16_t, float><<<grid, 256, 0, s>>>(static_cast<const float*>(p.y), p.pair_pos,
                                                           p.gates, o, p.N, p.H, p.K, sh, p.live);
  } else {
    combine_kernel<float, float><<<grid, 256, 0, s>>>(static_cast<const float*>(p.y), p.pair_pos, p.gates,
                                                      static_cast<float*>(out), p.N, p.H, p.K, sh, p.live);
  }
  return hipGetLastError();
}

}  // namespace cmoe
