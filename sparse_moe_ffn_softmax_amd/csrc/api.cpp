// api.cpp -- the C entry points of include/clover_moe.h: argument checks,
// workspace layout and the launch sequence.
//
// Every check runs on the host before any HIP call, so an invalid call
// returns without queueing work or writing a byte (InfiniLM PR #604,
// "Notes for Reviewers": unsupported options are rejected explicitly, and
// conversions are rejected before writing; its checklist asks for mask,
// state and workspace bounds and lifetime contracts).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/clover_moe.h"
#include "cmoe_launch.h"

namespace {

thread_local std::string g_last_error;

cmoe_status fail(cmoe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
cmoe_status fail(cmoe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

// The workspace of clover_moe_block_forward_noalloc: one static array per
// GPU the library runs on, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (in host code the name is a host-side
// stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, taken once with that device current.
static __device__ __align__(256) uint8_t scratch[CLOVER_MOE_NOALLOC_MAX_WORKSPACE];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array, looked up on the
// first use on that device.
hipError_t scratch_address(int dev, void** ptr) {
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  *ptr = s.ptr;
  return s.err;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t dtype_size(int d) { return d == CMOE_F32 ? 4 : d == CMOE_BF16 ? 2 : 1; }

struct Range {
  const char* name;
  uintptr_t lo;
  size_t bytes;
  bool writable;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.lo || !b.lo || !a.bytes || !b.bytes) return false;
  return a.lo < b.lo + b.bytes && b.lo < a.lo + a.bytes;
}

cmoe_status check_problem(const cmoe_problem* p, int32_t top_k) {
  if (!p) return fail(CMOE_ERR_NULL, "problem is NULL");
  if (p->hidden < 128 || p->hidden > 16384 || p->hidden % 128)
    return fail(p->hidden <= 0 ? CMOE_ERR_VALUE : CMOE_ERR_UNSUPPORTED,
                "hidden=%d: must be a multiple of 128 in [128, 16384]", p->hidden);
  if (p->num_experts < 1) return fail(CMOE_ERR_VALUE, "num_experts=%d must be >= 1", p->num_experts);
  if (p->num_experts > 256)
    return fail(CMOE_ERR_UNSUPPORTED, "num_experts=%d: at most 256 experts", p->num_experts);
  if (p->inter < 128 || p->inter > 8192 || p->inter % 128)
    return fail(p->inter <= 0 ? CMOE_ERR_VALUE : CMOE_ERR_UNSUPPORTED,
                "inter=%d: must be a multiple of 128 in [128, 8192]", p->inter);
  if (p->shared_inter < 0) return fail(CMOE_ERR_VALUE, "shared_inter=%d < 0", p->shared_inter);
  if (p->shared_inter > 8192 || p->shared_inter % 128)
    return fail(CMOE_ERR_UNSUPPORTED, "shared_inter=%d: must be 0 or a multiple of 128 up to 8192",
                p->shared_inter);
  // 8, 16, 32: diffusion blocks; 1, 2, 4: autoregressive decode and the
  // verification of 1-4 drafted candidates
  const int R = p->block_rows;
  if (R != 1 && R != 2 && R != 4 && R != 8 && R != 16 && R != 32)
    return fail(R <= 0 ? CMOE_ERR_VALUE : CMOE_ERR_UNSUPPORTED,
                "block_rows=%d: must be 1, 2, 4, 8, 16 or 32", R);
  if (p->num_blocks < 1) return fail(CMOE_ERR_VALUE, "num_blocks=%d must be >= 1", p->num_blocks);
  if (p->num_blocks > 1024)
    return fail(CMOE_ERR_UNSUPPORTED, "num_blocks=%d: at most 1024 blocks per call", p->num_blocks);
  const bool ok_pair = (p->act_dtype == CMOE_F32 && p->weight_dtype == CMOE_F32) ||
                       (p->act_dtype == CMOE_BF16 && p->weight_dtype == CMOE_BF16) ||
                       (p->act_dtype == CMOE_BF16 && p->weight_dtype == CMOE_FP8_E4M3) ||
                       (p->act_dtype == CMOE_BF16 && p->weight_dtype == CMOE_FP4_E2M1);
  if (!ok_pair)
    return fail(CMOE_ERR_UNSUPPORTED,
                "dtype pair (act=%d, weight=%d) unsupported: use (F32,F32), (BF16,BF16), (BF16,FP8_E4M3) "
                "or (BF16,FP4_E2M1)",
                p->act_dtype, p->weight_dtype);
  if (top_k < 1 || top_k > p->num_experts)
    return fail(CMOE_ERR_VALUE, "top_k=%d must be in [1, num_experts=%d]", top_k, p->num_experts);
  if (top_k > 8) return fail(CMOE_ERR_UNSUPPORTED, "top_k=%d: at most 8", top_k);
  return CMOE_OK;
}

struct Layout {
  size_t logits, topk, gates, counts, offsets, pair_row, pair_pos, blockmask, blockpre, tiles,
      tile_count, h, y, x8, total;
  int max_tiles, mt_max, y_act;
};

Layout layout(const cmoe_problem& p, int K) {
  const size_t N = (size_t)p.block_rows * p.num_blocks, E = p.num_experts, H = p.hidden;
  const size_t NK = N * K;
  Layout L;
  // work-tile height: about 1.5x the mean rows per expert, in 16-row MFMA
  // tiles (1, 2, 4, 6 or 8); experts with more rows get several tiles
  const size_t want = (NK * 3 / 2 + E - 1) / E;
  static const int kTileChoices[] = {1, 2, 4, 6, 8};
  L.mt_max = 8;
  for (int mt : kTileChoices)
    if ((size_t)16 * mt >= want) {
      L.mt_max = mt;
      break;
    }
  // 16-row tiles run the register-operand kernels; from a few rows per expert
  // on, the LDS-tiled kernels with 32-row tiles are faster for fp8 and bf16
  // weights (measured, H = 2048, 256 experts, top-8: fp8 from 2 blocks of 32
  // rows, 2-25% faster; bf16 from 6 blocks, 2-11%; 4-bit weights 17-27% slower
  // there at 2-10 blocks, and so keep the register kernels)
  const size_t reg_max = p.weight_dtype == CMOE_FP8_E4M3 ? 2 : p.weight_dtype == CMOE_BF16 ? 8 : 16;
  if (L.mt_max == 1 && want > reg_max) L.mt_max = 2;
  const size_t T = 16 * (size_t)L.mt_max;
  L.max_tiles = (int)(NK / T + (E < NK ? E : NK) + (N + T - 1) / T + 1);
  const size_t hsz = p.act_dtype == CMOE_F32 ? 4 : 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L.logits = take(N * E * 4);
  L.topk = take(NK * 4);
  L.gates = take(NK * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.pair_row = take(NK * 4);
  L.pair_pos = take(NK * 4);
  const size_t B = p.num_blocks;
  L.blockmask = take(B * E * 4);
  L.blockpre = take(B * E * 4);
  L.tiles = take((size_t)L.max_tiles * sizeof(cmoe::Tile));
  L.tile_count = take(4);
  L.h = take((NK * p.inter + N * p.shared_inter) * hsz);
  // Per-pair down outputs: fp32 for small calls; with many rows per expert
  // (mt_max > 1) the buffer is large (about 150 MB at 2048 rows) and is
  // stored in the activation dtype, halving its write and read traffic.
  L.y_act = L.mt_max > 1 && p.act_dtype == CMOE_BF16;
  L.y = take((NK + N) * H * (L.y_act ? 2 : 4));
  // fp8 activations (cmoe_options.activation_fp8): x as MXFP8 codes [N, H]
  // and E8M0 scales [N, H/32], for the many-row fp8-weight GEMMs
  L.x8 = p.weight_dtype == CMOE_FP8_E4M3 && L.y_act ? take(N * H + N * H / 32) : 0;
  L.total = off;
  return L;
}

}  // namespace

namespace cmoe {

size_t workspace_bytes(const cmoe_problem& pr, int top_k) { return layout(pr, top_k).total; }

// sizes, dtypes and the work-tile plan; device pointers are left as they are
static void plan_shape(Plan& p, const cmoe_problem& pr, int K, const Layout& L) {
  p.N = pr.block_rows * pr.num_blocks;
  p.H = pr.hidden;
  p.E = pr.num_experts;
  p.I = pr.inter;
  p.Is = pr.shared_inter;
  p.R = pr.block_rows;
  p.B = pr.num_blocks;
  p.K = K;
  p.act = pr.act_dtype;
  p.wt = pr.weight_dtype;
  p.live = nullptr;
  p.budget = 0;
  p.max_tiles = L.max_tiles;
  p.mt_max = L.mt_max;
  p.tile_rows = 16 * L.mt_max;
  p.y_act = L.y_act;
  p.act8 = 0;
}

void plan_shape(Plan& p, const cmoe_problem& pr, int K) { plan_shape(p, pr, K, layout(pr, K)); }

void carve(Plan& p, const cmoe_problem& pr, int K, void* ws, const cmoe_routing* rt) {
  const Layout L = layout(pr, K);
  plan_shape(p, pr, K, L);
  char* base = static_cast<char*>(ws);
  p.logits = (rt && rt->logits) ? rt->logits : reinterpret_cast<float*>(base + L.logits);
  p.topk = (rt && rt->topk_idx) ? rt->topk_idx : reinterpret_cast<int32_t*>(base + L.topk);
  p.gates = (rt && rt->gates) ? rt->gates : reinterpret_cast<float*>(base + L.gates);
  p.counts = reinterpret_cast<int32_t*>(base + L.counts);
  p.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  p.pair_row = reinterpret_cast<int32_t*>(base + L.pair_row);
  p.pair_pos = reinterpret_cast<int32_t*>(base + L.pair_pos);
  p.blockmask = reinterpret_cast<uint32_t*>(base + L.blockmask);
  p.blockpre = reinterpret_cast<int32_t*>(base + L.blockpre);
  p.tiles = reinterpret_cast<Tile*>(base + L.tiles);
  p.tile_count = reinterpret_cast<int32_t*>(base + L.tile_count);
  p.h = base + L.h;
  p.y = base + L.y;
  p.x8 = L.x8 ? base + L.x8 : nullptr;
  p.coreset_ids = rt ? rt->coreset_ids : nullptr;
  p.coreset_size = rt ? rt->coreset_size : nullptr;
  p.block_mass = rt ? rt->block_mass : nullptr;
  p.out_counts = rt ? rt->expert_counts : nullptr;
  p.out_offsets = rt ? rt->expert_offsets : nullptr;
  p.out_perm = rt ? rt->perm : nullptr;
}

bool act8_fits(const Plan& p) {
  // the MXFP8 buffers exist for fp8 weights with y in the activation dtype
  return p.wt == CMOE_FP8_E4M3 && p.y_act && expert_many_fits(p, true) && expert_many_fits(p, false);
}

KernelChoice choose_kernels(const Plan& p) {
  KernelChoice c;
  c.fused = down_combine_fits(p);
  c.up = p.mt_max == 1 ? CMOE_GEMM_REGISTER : expert_many_fits(p, true) ? CMOE_GEMM_PERSISTENT : CMOE_GEMM_LDS_TILED;
  c.down = c.fused                       ? CMOE_GEMM_DOWN_COMBINE
           : p.mt_max == 1                ? CMOE_GEMM_REGISTER
           : expert_many_fits(p, false)   ? CMOE_GEMM_PERSISTENT
                                          : CMOE_GEMM_LDS_TILED;
  return c;
}

}  // namespace cmoe

static cmoe_status act8_unsupported(const cmoe_problem& p, const cmoe::Plan& plan) {
  return fail(CMOE_ERR_UNSUPPORTED,
              "activation_fp8 needs fp8 weights with bf16 activations, inter=512, shared_inter 0 or "
              "512, hidden 512, 1024 or 2048 and work tiles of 32 rows or more (N*top_k above about "
              "4/3 per expert); here weight=%d act=%d inter=%d shared_inter=%d hidden=%d, tile rows %d",
              p.weight_dtype, p.act_dtype, p.inter, p.shared_inter, p.hidden, plan.tile_rows);
}

extern "C" {

cmoe_status clover_moe_plan_info(const cmoe_problem* problem, int32_t top_k, const cmoe_options* options,
                                 cmoe_plan_info* info) {
  if (!info) return fail(CMOE_ERR_NULL, "info is NULL");
  const cmoe_status s = check_problem(problem, top_k);
  if (s != CMOE_OK) return s;
  const int act8 = options ? options->activation_fp8 : 0;
  if (act8 != 0 && act8 != 1) return fail(CMOE_ERR_VALUE, "activation_fp8=%d must be 0 or 1", act8);
  cmoe::Plan plan{};
  cmoe::plan_shape(plan, *problem, top_k);
  plan.act8 = act8;
  if (act8 && !cmoe::act8_fits(plan)) return act8_unsupported(*problem, plan);
  const cmoe::KernelChoice kc = cmoe::choose_kernels(plan);
  info->tile_rows = plan.tile_rows;
  info->gate_up = kc.up;
  info->down = kc.down;
  info->y_bytes = plan.y_act ? 2 : 4;  // y in the (bf16) activation dtype, else fp32
  // router, routing, [two permutation kernels], [MXFP8 rounding of x], gate/up, down, [combine]
  info->kernels = 4 + (plan.B > 1 ? 2 : 0) + (act8 ? 1 : 0) + (kc.fused ? 0 : 1);
  return CMOE_OK;
}

cmoe_status clover_moe_workspace_size(const cmoe_problem* problem, int32_t top_k, size_t* bytes) {
  if (!bytes) return fail(CMOE_ERR_NULL, "bytes is NULL");
  const cmoe_status s = check_problem(problem, top_k);
  if (s != CMOE_OK) return s;
  *bytes = cmoe::workspace_bytes(*problem, top_k);
  return CMOE_OK;
}

static cmoe_status forward_impl(const cmoe_problem* problem, const cmoe_weights* w,
                                const void* x, float mass_threshold, int32_t top_k,
                                const cmoe_options* options, void* out,
                                const cmoe_routing* routing, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* events,
                                int32_t n_events) {
  cmoe_status s = check_problem(problem, top_k);
  if (s != CMOE_OK) return s;
  const cmoe_problem& p = *problem;
  if (!w) return fail(CMOE_ERR_NULL, "weights is NULL");
  if (!x) return fail(CMOE_ERR_NULL, "x is NULL");
  if (!out) return fail(CMOE_ERR_NULL, "out is NULL");
  if (!w->router_w) return fail(CMOE_ERR_NULL, "weights->router_w is NULL");
  if (!w->w13) return fail(CMOE_ERR_NULL, "weights->w13 is NULL");
  if (!w->w2) return fail(CMOE_ERR_NULL, "weights->w2 is NULL");
  if (p.shared_inter > 0 && (!w->shared_w13 || !w->shared_w2))
    return fail(CMOE_ERR_NULL, "shared_inter > 0 but the shared expert weights are NULL");
  const bool fp8 = p.weight_dtype == CMOE_FP8_E4M3, fp4 = p.weight_dtype == CMOE_FP4_E2M1;
  if ((fp8 || fp4) && (!w->w13_scale || !w->w2_scale ||
                       (p.shared_inter > 0 && (!w->shared_w13_scale || !w->shared_w2_scale))))
    return fail(CMOE_ERR_NULL, "%s weights need every scale array",
                fp8 ? "fp8" : "fp4");
  if (w->layout != CMOE_LAYOUT_ROWS && w->layout != CMOE_LAYOUT_PANELS)
    return fail(CMOE_ERR_VALUE, "weights->layout=%d is not a cmoe_layout", w->layout);
  if (!(mass_threshold > 0.0f && mass_threshold <= 1.0f))
    return fail(CMOE_ERR_VALUE, "mass_threshold=%g must be in (0, 1]", (double)mass_threshold);
  const int budget = options ? options->expert_budget : 0;
  const uint8_t* live = options ? options->live_rows : nullptr;
  const int act8 = options ? options->activation_fp8 : 0;
  if (budget < 0 || budget > p.num_experts)
    return fail(CMOE_ERR_VALUE, "expert_budget=%d must be in [0, num_experts=%d]", budget,
                p.num_experts);
  if (act8 != 0 && act8 != 1) return fail(CMOE_ERR_VALUE, "activation_fp8=%d must be 0 or 1", act8);

  const size_t need = cmoe::workspace_bytes(p, top_k);
  if (!workspace || workspace_bytes < need)
    return fail(CMOE_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                workspace_bytes, workspace, need);

  // every device range the call touches
  const size_t N = (size_t)p.block_rows * p.num_blocks, E = p.num_experts, H = p.hidden,
               I = p.inter, Is = p.shared_inter, B = p.num_blocks, K = top_k;
  const size_t asz = dtype_size(p.act_dtype);
  // bytes of a [rows, cols] weight matrix in the weight dtype
  auto wbytes = [&](size_t rows, size_t cols) {
    return fp4 ? rows * cols / 2 : rows * cols * dtype_size(p.weight_dtype);
  };
  std::vector<Range> rs = {
      {"x", (uintptr_t)x, N * H * asz, false},
      {"router_w", (uintptr_t)w->router_w, E * H * 4, false},
      {"router_b", (uintptr_t)w->router_b, E * 4, false},
      {"w13", (uintptr_t)w->w13, E * wbytes(2 * I, H), false},
      {"w2", (uintptr_t)w->w2, E * wbytes(H, I), false},
      {"shared_w13", Is ? (uintptr_t)w->shared_w13 : 0, wbytes(2 * Is, H), false},
      {"shared_w2", Is ? (uintptr_t)w->shared_w2 : 0, wbytes(H, Is), false},
      {"live_rows", (uintptr_t)live, N, false},
      {"out", (uintptr_t)out, N * H * asz, true},
      {"workspace", (uintptr_t)workspace, need, true},
  };
  if (fp4) {
    rs.push_back({"w13_scale", (uintptr_t)w->w13_scale, E * 2 * I * (H / 32), false});
    rs.push_back({"w2_scale", (uintptr_t)w->w2_scale, E * H * (I / 32), false});
    if (Is) {
      rs.push_back({"shared_w13_scale", (uintptr_t)w->shared_w13_scale, 2 * Is * (H / 32), false});
      rs.push_back({"shared_w2_scale", (uintptr_t)w->shared_w2_scale, H * (Is / 32), false});
    }
  }
  if (fp8) {
    rs.push_back({"w13_scale", (uintptr_t)w->w13_scale, E * (2 * I / 128) * (H / 128) * 4, false});
    rs.push_back({"w2_scale", (uintptr_t)w->w2_scale, E * (H / 128) * (I / 128) * 4, false});
    if (Is) {
      rs.push_back({"shared_w13_scale", (uintptr_t)w->shared_w13_scale, (2 * Is / 128) * (H / 128) * 4, false});
      rs.push_back({"shared_w2_scale", (uintptr_t)w->shared_w2_scale, (H / 128) * (Is / 128) * 4, false});
    }
  }
  if (routing) {
    rs.push_back({"routing.topk_idx", (uintptr_t)routing->topk_idx, N * K * 4, true});
    rs.push_back({"routing.gates", (uintptr_t)routing->gates, N * K * 4, true});
    rs.push_back({"routing.coreset_ids", (uintptr_t)routing->coreset_ids, B * E * 4, true});
    rs.push_back({"routing.coreset_size", (uintptr_t)routing->coreset_size, B * 4, true});
    rs.push_back({"routing.expert_counts", (uintptr_t)routing->expert_counts, E * 4, true});
    rs.push_back({"routing.expert_offsets", (uintptr_t)routing->expert_offsets, (E + 1) * 4, true});
    rs.push_back({"routing.perm", (uintptr_t)routing->perm, N * K * 4, true});
    rs.push_back({"routing.logits", (uintptr_t)routing->logits, N * E * 4, true});
    rs.push_back({"routing.block_mass", (uintptr_t)routing->block_mass, B * E * 8, true});
  }
  for (const Range& r : rs)
    if (r.lo % 16)
      return fail(CMOE_ERR_ALIGN, "%s at %p is not 16-byte aligned", r.name, (void*)r.lo);
  for (size_t i = 0; i < rs.size(); ++i)
    for (size_t j = i + 1; j < rs.size(); ++j)
      if ((rs[i].writable || rs[j].writable) && overlap(rs[i], rs[j]))
        return fail(CMOE_ERR_ALIAS, "%s overlaps %s", rs[i].name, rs[j].name);

  if (events) {
    if (n_events != CLOVER_MOE_NUM_STAGES + 1)
      return fail(CMOE_ERR_VALUE, "n_events=%d, expected %d", n_events, CLOVER_MOE_NUM_STAGES + 1);
    for (int i = 0; i < n_events; ++i)
      if (!events[i]) return fail(CMOE_ERR_NULL, "stage_events[%d] is NULL", i);
  }

  cmoe::Plan plan;
  cmoe::carve(plan, p, top_k, workspace, routing);
  plan.live = live;
  plan.budget = budget;
  plan.panels = w->layout == CMOE_LAYOUT_PANELS;
  plan.act8 = act8;
  if (act8 && !cmoe::act8_fits(plan)) return act8_unsupported(p, plan);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // few routed pairs: the down GEMM writes `out` itself (stage 4 is empty)
  const cmoe::KernelChoice kc = cmoe::choose_kernels(plan);
  const bool fused = kc.fused;
  for (int stage = 0; stage <= CLOVER_MOE_NUM_STAGES && e == hipSuccess; ++stage) {
    if (events) {
      e = hipEventRecord(static_cast<hipEvent_t>(events[stage]), st);
      if (e != hipSuccess) break;
    }
    switch (stage) {
      case 0: e = cmoe::launch_router(plan, x, w->router_w, w->router_b, st); break;
      case 1:
        e = cmoe::launch_route_blocks(plan, mass_threshold, st);
        if (e == hipSuccess && plan.B > 1) e = cmoe::launch_permute_blocks(plan, st);
        break;
      case 2:
        e = kc.up == CMOE_GEMM_REGISTER     ? cmoe::launch_expert_up(plan, *w, x, st)
            : kc.up == CMOE_GEMM_PERSISTENT ? cmoe::launch_expert_many(plan, *w, x, true, st)
                                            : cmoe::launch_expert_tiled(plan, *w, x, true, st);
        break;
      case 3:
        e = kc.down == CMOE_GEMM_DOWN_COMBINE ? cmoe::launch_expert_down_combine(plan, *w, out, st)
            : kc.down == CMOE_GEMM_REGISTER   ? cmoe::launch_expert_down(plan, *w, st)
            : kc.down == CMOE_GEMM_PERSISTENT ? cmoe::launch_expert_many(plan, *w, x, false, st)
                                              : cmoe::launch_expert_tiled(plan, *w, x, false, st);
        break;
      case 4:
        if (!fused) e = cmoe::launch_combine(plan, out, st);
        break;
      default: break;
    }
  }
  if (e != hipSuccess) return fail(CMOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return CMOE_OK;
}

cmoe_status clover_moe_block_forward(const cmoe_problem* problem, const cmoe_weights* w,
                                     const void* x, float mass_threshold, int32_t top_k, void* out,
                                     const cmoe_routing* routing, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return forward_impl(problem, w, x, mass_threshold, top_k, nullptr, out, routing, workspace,
                      workspace_bytes, stream, nullptr, 0);
}

cmoe_status clover_moe_block_forward_ex(const cmoe_problem* problem, const cmoe_weights* w,
                                        const void* x, float mass_threshold, int32_t top_k,
                                        const cmoe_options* options, void* out,
                                        const cmoe_routing* routing, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return forward_impl(problem, w, x, mass_threshold, top_k, options, out, routing, workspace,
                      workspace_bytes, stream, nullptr, 0);
}

cmoe_status clover_moe_block_forward_staged(const cmoe_problem* problem, const cmoe_weights* w,
                                            const void* x, float mass_threshold, int32_t top_k,
                                            const cmoe_options* options, void* out,
                                            const cmoe_routing* routing, void* workspace,
                                            size_t workspace_bytes, void* stream,
                                            void* const* stage_events, int32_t n_events) {
  if (!stage_events) return fail(CMOE_ERR_NULL, "stage_events is NULL");
  return forward_impl(problem, w, x, mass_threshold, top_k, options, out, routing, workspace,
                      workspace_bytes, stream, stage_events, n_events);
}

cmoe_status clover_moe_block_forward_noalloc(const cmoe_problem* problem, const cmoe_weights* w,
                                             const void* x, float mass_threshold, int32_t top_k,
                                             const cmoe_options* options, void* out,
                                             const cmoe_routing* routing, void* stream) {
  const cmoe_status s = check_problem(problem, top_k);
  if (s != CMOE_OK) return s;
  const size_t need = cmoe::workspace_bytes(*problem, top_k);
  if (need > CLOVER_MOE_NOALLOC_MAX_WORKSPACE)
    return fail(CMOE_ERR_WORKSPACE,
                "this problem needs %zu bytes of workspace; the no-allocation entry point has %zu "
                "(use clover_moe_block_forward_ex with a caller workspace)",
                need, (size_t)CLOVER_MOE_NOALLOC_MAX_WORKSPACE);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CMOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CMOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return fail(CMOE_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(CMOE_ERR_VALUE, "stream belongs to device %d, the current device is %d", sdev, dev);
  }
  void* ws = nullptr;
  e = scratch_address(dev, &ws);
  if (e != hipSuccess || !ws)
    return fail(CMOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(e));
  return forward_impl(problem, w, x, mass_threshold, top_k, options, out, routing, ws,
                      CLOVER_MOE_NOALLOC_MAX_WORKSPACE, stream, nullptr, 0);
}

cmoe_status clover_moe_pack_weights(const void* src, void* dst, int64_t count, int32_t rows,
                                    int32_t row_bytes, int32_t gate_up, void* stream) {
  if (!src) return fail(CMOE_ERR_NULL, "src is NULL");
  if (!dst) return fail(CMOE_ERR_NULL, "dst is NULL");
  if (count < 1) return fail(CMOE_ERR_VALUE, "count=%lld must be >= 1", (long long)count);
  if (rows < 16 || rows % 16) return fail(CMOE_ERR_VALUE, "rows=%d must be a positive multiple of 16", rows);
  if (row_bytes < 64 || row_bytes % 64)
    return fail(CMOE_ERR_VALUE, "row_bytes=%d must be a positive multiple of 64", row_bytes);
  if (gate_up != 0 && gate_up != 1) return fail(CMOE_ERR_VALUE, "gate_up=%d must be 0 or 1", gate_up);
  if ((uintptr_t)src % 16 || (uintptr_t)dst % 16)
    return fail(CMOE_ERR_ALIGN, "src %p / dst %p not 16-byte aligned", src, dst);
  const size_t bytes = (size_t)count * (size_t)rows * (size_t)row_bytes;
  if (overlap({"src", (uintptr_t)src, bytes, false}, {"dst", (uintptr_t)dst, bytes, true}))
    return fail(CMOE_ERR_ALIAS, "src and dst overlap");
  const hipError_t e = cmoe::launch_pack_panels(src, dst, count, rows, row_bytes, gate_up,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(CMOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return CMOE_OK;
}

const char* clover_moe_status_string(cmoe_status s) {
  switch (s) {
    case CMOE_OK: return "ok";
    case CMOE_ERR_NULL: return "a required pointer is NULL";
    case CMOE_ERR_VALUE: return "an argument is out of its domain";
    case CMOE_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case CMOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case CMOE_ERR_ALIAS: return "an output overlaps an input or another output";
    case CMOE_ERR_WORKSPACE: return "workspace missing or too small";
    case CMOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* clover_moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
