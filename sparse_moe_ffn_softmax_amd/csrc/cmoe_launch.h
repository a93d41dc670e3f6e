// cmoe_launch.h -- internal interface between the host entry points (api.cpp)
// and the HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/clover_moe.h"

namespace cmoe {

// Rows of one grouped-GEMM work tile: 16 * mt_max, mt_max in {1, 2, 4, 6, 8} MFMA
// row tiles, chosen per call from the expected rows per expert and the weight
// format (layout() in api.cpp).
constexpr int kMaxTileRows = 128;
// h columns produced by one expert_up workgroup (one 16-column MFMA tile of 8
// gate + 8 up columns; the 4 waves split the hidden dimension).
constexpr int kUpCols = 8;
// waves of one expert_down workgroup, and the output columns it produces
// (16 per wave; 4-bit weights: 16 per column tile, see expert_gemm.hip)
constexpr int kDownWaves = 2;
constexpr int kDownCols = 16 * kDownWaves;

// One unit of grouped-GEMM work: `rows` consecutive pairs of one expert,
// starting at pair position `start` (expert == E means the shared expert,
// whose pairs are the N rows in order).
struct Tile {
  int32_t expert;
  int32_t start;
  int32_t rows;
  int32_t pad;
};

// Everything a launch needs: sizes plus device pointers carved out of the
// caller's workspace (or the caller's optional routing buffers).
struct Plan {
  int N, H, E, I, Is, R, B, K;
  int act, wt;           // cmoe_dtype codes
  bool panels;           // expert weights in MFMA panels (CMOE_LAYOUT_PANELS), else row-major
  int max_tiles;         // grid bound for the grouped GEMMs
  int mt_max;            // MFMA row tiles per work tile: 1, 2, 4, 6 or 8
  int tile_rows;         // 16 * mt_max
  float* logits;         // [N,E]
  int32_t* topk;         // [N,K]
  float* gates;          // [N,K]
  int32_t* counts;       // [E]
  int32_t* offsets;      // [E+1]
  int32_t* pair_row;     // [N*K]  source row of each routed pair, expert-major
  int32_t* pair_pos;     // [N*K]  pair position of (row, slot), -1 if unused
  uint32_t* blockmask;   // [B, E] bit r set iff row r of block b routes to expert e
  int32_t* blockpre;     // [B, E] pairs of expert e in the blocks before b
  Tile* tiles;           // [max_tiles]
  int32_t* tile_count;   // [1]
  void* h;               // routed [N*K, I] then shared [N, Is]; act_dtype elements
  void* y;               // [N*K + N][H]: routed pairs, then shared rows
  int y_act;             // y stored in act_dtype (else fp32), see carve()
  const uint8_t* live;   // [N] live-row mask, or nullptr (every row live)
  int budget;            // coreset cap per block, 0 = none
  int act8;              // fp8 (MXFP8) activations into the many-row GEMMs (cmoe_options.activation_fp8)
  void* x8;              // [N, H] e4m3 codes then [N, H/32] E8M0 scales (act8)
  // optional caller outputs
  int32_t* coreset_ids;
  int32_t* coreset_size;
  double* block_mass;
  int32_t* out_counts;
  int32_t* out_offsets;
  int32_t* out_perm;
};

size_t workspace_bytes(const cmoe_problem& pr, int top_k);
// Carves the workspace; routing buffers given by the caller replace the
// workspace copies where the layout is the same.
void carve(Plan& p, const cmoe_problem& pr, int top_k, void* ws, const cmoe_routing* rt);
// sizes, dtypes and the work-tile plan only (no workspace, pointers untouched)
void plan_shape(Plan& p, const cmoe_problem& pr, int top_k);
// fp8 activations cover the call (buffers planned, both GEMMs have the kernel)
bool act8_fits(const Plan& p);
// the kernels of stages 2 and 3 (cmoe_gemm_kind); fused: the down GEMM writes
// out and stage 4 is empty
struct KernelChoice {
  int up, down;
  bool fused;
};
KernelChoice choose_kernels(const Plan& p);

// XCD-aware work mapping for the LDS-tiled grouped GEMMs.  Workgroups are
// dispatched to the 8 XCDs round-robin by id, and each XCD has its own L2;
// every column slice of a tile reads the tile's gathered activation rows (up
// to 128 rows).  Tile t is therefore given to XCD t % 8, with its slices on
// consecutive ids of that XCD, so the rows come from memory once per tile
// instead of once per slice (64 blocks: gate/up reads 624 MB instead of 917).
// The one-row-tile kernels keep the plain mapping: their activations are a
// few KiB, and whole experts per XCD only unbalance the XCDs.  The mapping
// only affects locality: any dispatch order computes the same.
constexpr int kXcds = 8;
__host__ __device__ inline unsigned tile_grid(int max_tiles, int n_slices) {
  return (unsigned)((max_tiles + kXcds - 1) / kXcds) * kXcds * (unsigned)n_slices;
}
__device__ inline void tile_of_block(unsigned g, int n_slices, int& slot, int& slice) {
  const unsigned xcd = g % kXcds, local = g / kXcds;
  slot = (int)(local / (unsigned)n_slices) * kXcds + (int)xcd;
  slice = (int)(local % (unsigned)n_slices);
}

hipError_t launch_router(const Plan& p, const void* x, const float* router_w,
                         const float* router_b, hipStream_t s);
// per-block routing; a one-block call also builds the permutation and the
// work list in the same kernel, a many-block call with launch_permute_blocks
hipError_t launch_route_blocks(const Plan& p, float tau, hipStream_t s);
hipError_t launch_permute_blocks(const Plan& p, hipStream_t s);
// mt_max == 1: register-operand kernels (expert_gemm.hip)
hipError_t launch_expert_up(const Plan& p, const cmoe_weights& w, const void* x, hipStream_t s);
hipError_t launch_expert_down(const Plan& p, const cmoe_weights& w, hipStream_t s);
// calls with few routed pairs: the down GEMM and the combine in one kernel
bool down_combine_fits(const Plan& p);
hipError_t launch_expert_down_combine(const Plan& p, const cmoe_weights& w, void* out, hipStream_t s);
// mt_max > 1: LDS-staged activation tiles (expert_tiled.hip); up = gate/up + SwiGLU, else down
hipError_t launch_expert_tiled(const Plan& p, const cmoe_weights& w, const void* x, bool up,
                               hipStream_t s);
// mt_max > 1 on 16-bit activations with I = 512 (and Is = 0 or I): persistent
// kernels on the 32x32 MFMA (expert_many.hip); up = gate/up + SwiGLU (fp8
// activations only), else down (fp8 activations, or work tiles tall enough for
// the weight format: bf16 128 rows, fp8 96, 4-bit 32)
bool expert_many_fits(const Plan& p, bool up);
hipError_t launch_expert_many(const Plan& p, const cmoe_weights& w, const void* x, bool up, hipStream_t s);
hipError_t launch_combine(const Plan& p, void* out, hipStream_t s);
// bf16 rows [rows, cols] -> MXFP8 codes [rows, cols] and E8M0 scales [rows, cols/32]
hipError_t launch_quant_mx8(const void* src, long long rows, int cols, void* dst, void* scales, hipStream_t s);
// count row-major matrices of rows x row_bytes bytes -> MFMA panels (clover_moe.h)
hipError_t launch_pack_panels(const void* src, void* dst, int64_t count, int rows, int row_bytes, int gate_up,
                              hipStream_t s);

}  // namespace cmoe
