// pack.hip -- rearranges row-major expert weight matrices into MFMA panels
// (CMOE_LAYOUT_PANELS, defined in clover_moe.h).
//
// The expert GEMMs read each weight row in 16-byte chunks, one per lane group
// (16 rows x 4 lane groups = 64 lanes), so one wave-wide load of row-major
// weights touches half of 16 cache lines.  In a panel, the 64 chunks one
// load needs are 1 KiB of consecutive bytes, in lane order, and the GEMMs
// stream them with non-temporal loads.  This is a pure byte permutation done
// once when the weights are loaded; nothing is converted or rounded.
#include "cmoe_device.h"
#include "cmoe_launch.h"

namespace cmoe {

// One thread per 16-byte chunk of dst, grid-stride.  dst chunk d of matrix m
// is unit q, lane l of panel p; it holds bytes [64q + 16(l/16), +16) of the
// panel's row l%16.
__global__ __launch_bounds__(256) void pack_panels_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int64_t total, int rows, int row_bytes, int gate_up) {
  const int64_t per_matrix = (int64_t)rows * row_bytes / 16;  // chunks
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total; d += stride) {
    const int64_t m = d / per_matrix, dd = d % per_matrix;
    const int64_t p = dd / row_bytes;  // a panel is 16 rows = row_bytes chunks
    const int r = (int)(dd % row_bytes);
    const int q = r / 64, l = r % 64, i = l & 15;
    const int64_t row = gate_up ? (i < 8 ? 8 * p + i : rows / 2 + 8 * p + i - 8) : 16 * p + i;
    const int64_t sb = row * row_bytes + 64 * q + 16 * (l >> 4);  // source byte within the matrix
    dst[d] = src[m * per_matrix + sb / 16];
  }
}

hipError_t launch_pack_panels(const void* src, void* dst, int64_t count, int rows, int row_bytes, int gate_up,
                              hipStream_t s) {
  const int64_t total = count * rows * (int64_t)row_bytes / 16;
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  pack_panels_kernel<<<grid, 256, 0, s>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), total, rows,
                                          row_bytes, gate_up);
  return hipGetLastError();
}

}  // namespace cmoe
