// route_block.hip -- per-block routing: softmax, block mass, coreset and
// restricted top-k with renormalised gates.  One workgroup (16 waves) per
// block.
//
// What is computed (Clover-35B-A3B-Preview CMF model card: introduction for
// the 256 routed experts, eight per token, and the shared expert; "Usage" for
// limiting a block to the experts that hold 90% of its routing weight; InfiniLM PR #604
// "Summary" for block coreset routing in the preview pass, "Motivation" for
// top-4 preview routing, "Notes for Reviewers" for the full-route replay):
//
//   u[r,e]   = exp(l[r,e] - max_e l[r,:])                         fp64
//   Z[r]     = sum_e u[r,e]   (8 contiguous chunks of e, ascending inside a
//                              chunk, pairwise combine j+=j+4, j+=j+2, j+=j+1)
//   p[r,e]   = u[r,e] / Z[r]
//   mass[e]  = sum over the block's rows, ascending, of p[r,e]
//   order    = experts by (mass desc, id asc)
//   cum[i]   = sequential fp64 prefix sum of mass in that order
//   coreset  = order[0 : m], m the smallest with cum[m-1] >= tau * cum[E-1];
//              tau >= 1 gives m = E
//   per row  : the min(k, m) coreset experts with the largest fp32 logits,
//              ties to the lower id; gate_j = (float)(u_j / sum of u over the
//              chosen slots in slot order)
//
// With call options (InfiniLM PR #604, "Summary": expert-budget / live-row
// reuse): m is further cut to the expert budget; resolved rows (live mask 0)
// add nothing to the mass and take no route, and a block without live rows
// has m = 0.
//
// exp is evaluated by Cody & Waite's (1980) argument reduction and the
// degree-13 Taylor polynomial of exp(r), Horner with fma, then scaled by
// 2^n; every operation is an IEEE fp64 primitive, so results are bitwise
// reproducible on any IEEE machine that follows the same sequence.
//
// Parallel layout.  Everything that is order-free (row maxima, the
// exponentials, the divisions, ranks, the top-k selection) is spread over
// the 1024 threads; only the summations whose order is fixed above run as
// short serial chains.  Top-k candidates are 64-bit keys (order-preserving
// logit bits, complemented id): each half-wave owns a row, keeps 8 sorted
// candidates per lane and takes the best head per slot with DPP exchanges
// inside 16-lane rows and one lane swap across them.  The block's experts
// are ordered by (mass desc, id asc) with four 64-wide bitonic sorts in
// registers and a binary-search merge of the four sorted runs.
//
// The coreset cut needs the serial prefix sum cum[] only where it decides
// something.  A parallel scan gives every prefix P[i] in another summation
// order; recursive summation of n non-negative terms is within
// (n-1) u / (1 - (n-1) u) of the exact sum in relative terms (Higham,
// "Accuracy and Stability of Numerical Algorithms", 2002, section 4.2), and
// so is the scan with its depth in place of n-1.  With both bounds far below
// a margin of 2^-40, an index i is provably below the threshold when
// P[i] (1 + 2^-40) < tau P[E-1] (1 - 2^-40), and provably at or above it when
// P[i] (1 - 2^-40) >= tau P[E-1] (1 + 2^-40).  When the first index that is
// not provably below is provably at or above, it is the cut; otherwise (the
// threshold lies within about 1e-12 of a prefix sum) the serial sum runs.
//
// A one-block call goes on to build the row -> expert permutation and the
// GEMM work list in the same kernel (permute.h); with many blocks every block
// publishes its rows per expert as one mask word each, and two small kernels
// queued next build the permutation (permute_blocks.hip).
#include "cmoe_device.h"
#include "cmoe_launch.h"
#include "permute.h"

#pragma clang fp contract(off)

namespace cmoe {

constexpr int kMaxRows = 32;
constexpr int kMaxExperts = 256;
constexpr int kThreads = 1024;
constexpr int kPStride = kMaxExperts + kMaxExperts / 32;
__device__ __forceinline__ int pidx(int r, int e) { return r * kPStride + e + (e >> 5); }

// 1/ln 2 (correctly rounded); ln 2 split into a 42-bit head (so that n*head is
// exact for |n| < 2^11) and its correctly rounded tail; 1/i! for i = 0..13.
__constant__ double kInvLn2 = 0x1.71547652b82fep+0;
__constant__ double kLn2Head = 0x1.62e42fefa3800p-1;
__constant__ double kLn2Tail = 0x1.ef35793c76730p-45;
__constant__ double kInvFact[14] = {
    0x1.0000000000000p+0,  0x1.0000000000000p+0,  0x1.0000000000000p-1,  0x1.5555555555555p-3,
    0x1.5555555555555p-5,  0x1.1111111111111p-7,  0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13,
    0x1.a01a01a01a01ap-16, 0x1.71de3a556c734p-19, 0x1.27e4fb7789f5cp-22, 0x1.ae64567f544e4p-26,
    0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33};

// Every step is an fp64 primitive, so the result is reproducible bit for bit;
// below -708 (outside the normal range of the result) the value is 0.  The
// operations run unconditionally and the cut-off is a select, so a wave can
// interleave several independent evaluations.
__device__ __forceinline__ double exp_reduced(double d) {
  const double n = __builtin_rint(d * kInvLn2);
  double r = __builtin_fma(-n, kLn2Head, d);
  r = __builtin_fma(-n, kLn2Tail, r);
  double poly = kInvFact[13];
#pragma unroll
  for (int i = 12; i >= 0; --i) poly = __builtin_fma(poly, r, kInvFact[i]);
  // the clamp only matters for the discarded lanes (d < -708 or NaN)
  const int ni = static_cast<int>(__builtin_fmin(__builtin_fmax(n, -1100.0), 1100.0));
  const double v = __builtin_ldexp(poly, ni);
  return d < -708.0 ? 0.0 : v;
}

// DPP lane-exchange controls (within each row of 16 lanes)
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i inside 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// maximum over each 32-lane half of the wave, in every lane of that half:
// DPP inside each row of 16 lanes, then v_permlane16_swap, which hands each
// lane the value of its partner in the other row of the half (checked on
// gfx950: with both operands v, result 0 holds rows (0,0,2,2) and result 1
// rows (1,1,3,3) of v)
__device__ __forceinline__ uint32_t half_max_u32(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1]));
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kDppMirror>(__float_as_uint(v))));
  float m = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
#pragma unroll
  for (int row = 1; row < 4; ++row)
    m = fmaxf(m, __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), row * 16)));
  return m;
}

// sort 8 keys descending in registers (Batcher odd-even merge network)
__device__ __forceinline__ void cswap(uint64_t (&k)[8], int i, int j) {
  const uint64_t a = k[i], b = k[j];
  k[i] = a > b ? a : b;
  k[j] = a > b ? b : a;
}

__device__ __forceinline__ void sort8_desc(uint64_t (&k)[8]) {
  cswap(k, 0, 1); cswap(k, 2, 3); cswap(k, 4, 5); cswap(k, 6, 7);
  cswap(k, 0, 2); cswap(k, 1, 3); cswap(k, 4, 6); cswap(k, 5, 7);
  cswap(k, 1, 2); cswap(k, 5, 6);
  cswap(k, 0, 4); cswap(k, 1, 5); cswap(k, 2, 6); cswap(k, 3, 7);
  cswap(k, 2, 4); cswap(k, 3, 5);
  cswap(k, 1, 2); cswap(k, 3, 4); cswap(k, 5, 6);
}

// Candidate keys: (order-preserving logit bits) << 32 | ~id, so the larger
// key is the larger logit and, on equal logits, the lower id; 0 = none.
__device__ __forceinline__ uint32_t logit_key(float l) {
  const uint32_t b = __float_as_uint(l + 0.0f);  // -0 becomes +0: equal logits tie
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------
// (mass desc, id asc): the order the coreset and the mass prefix sum use.
// Masses are sums of non-negative probabilities from +0, so their fp64 bit
// patterns order as unsigned integers; with the complemented id below them,
// "a comes first" is one unsigned compare of 96-bit keys.
// ---------------------------------------------------------------------------
struct MassKey {
  uint64_t m;    // bits of the block mass
  uint32_t nid;  // ~expert id
};

__device__ __forceinline__ bool beats(const MassKey& a, const MassKey& b) {
  // b - a over the three words; the final borrow is set iff b < a
  unsigned c0, c1, c2;
  (void)__builtin_subc(b.nid, a.nid, 0u, &c0);
  (void)__builtin_subc(static_cast<unsigned>(b.m), static_cast<unsigned>(a.m), c0, &c1);
  (void)__builtin_subc(static_cast<unsigned>(b.m >> 32), static_cast<unsigned>(a.m >> 32), c1, &c2);
  return c2 != 0u;
}

// value of lane ^ J (J a power of two below 64), all lanes active
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
  if constexpr (J == 1) {
    return dpp<kDppXor1>(v);
  } else if constexpr (J == 2) {
    return dpp<kDppXor2>(v);
  } else if constexpr (J == 4) {
    return dpp<kDppHalfMirror>(dpp<0x1B>(v));  // (i ^ 3) then (i ^ 7) inside 8
  } else if constexpr (J == 8) {
    return dpp<0x128>(v);  // rotate by 8 inside 16 = i ^ 8
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? static_cast<uint32_t>(r[0]) : static_cast<uint32_t>(r[1]);
  } else {
    return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), J, 64));
  }
}

// one compare-exchange step of a bitonic sort over the 64 lanes: blocks of
// K lanes, partners J apart; the final order (K = 64) is descending
template <int K, int J>
__device__ __forceinline__ void bitonic_step(MassKey& k, int lane) {
  MassKey p;
  const uint32_t plo = xor_lane<J>(static_cast<uint32_t>(k.m), lane);
  const uint32_t phi = xor_lane<J>(static_cast<uint32_t>(k.m >> 32), lane);
  p.m = (static_cast<uint64_t>(phi) << 32) | plo;
  p.nid = xor_lane<J>(k.nid, lane);
  const bool keep_greater = ((lane & J) == 0) == ((lane & K) == 0);
  if (keep_greater == beats(p, k)) k = p;
}

template <int K, int J>
__device__ __forceinline__ void bitonic_merge(MassKey& k, int lane) {
  if constexpr (J > 0) {
    bitonic_step<K, J>(k, lane);
    bitonic_merge<K, J / 2>(k, lane);
  }
}

// sorts the wave's 64 keys, one per lane, so that lane i holds the i-th
template <int K = 2>
__device__ __forceinline__ void wave_sort64(MassKey& k, int lane) {
  if constexpr (K <= 64) {
    bitonic_merge<K, K / 2>(k, lane);
    wave_sort64<K * 2>(k, lane);
  }
}

// kMasked: the call passes a live-row mask.  Without one every row of the
// block is live and the mask is a register value, so the unmasked instance
// carries no mask load, broadcast or LDS read.
template <bool kMasked>
__global__ __launch_bounds__(kThreads) void route_block_kernel(Plan plan, float tau) {
  const int R = plan.R, E = plan.E, K = plan.K;
  int32_t* __restrict__ topk = plan.topk;
  float* __restrict__ gates = plan.gates;
  int32_t* __restrict__ coreset_ids = plan.coreset_ids;
  int32_t* __restrict__ coreset_size = plan.coreset_size;
  double* __restrict__ block_mass = plan.block_mass;
  __shared__ float l_s[kMaxRows][kMaxExperts];
  // u.  One pad slot per 32 experts keeps the per-chunk serial sums of
  // different (row, chunk) threads on different banks.
  __shared__ double p_s[kMaxRows * kPStride];
  __shared__ double zpart[kMaxRows][8];  // Z partials; later the chosen u
  __shared__ double z_s[kMaxRows];
  __shared__ float m_s[kMaxRows];
  __shared__ double mass_s[kMaxExperts];
  __shared__ double smass_s[kMaxExperts];  // masses in (mass desc, id asc) order
  __shared__ double cum_s[kMaxExperts];
  __shared__ int order_s[kMaxExperts];
  __shared__ int rank_s[kMaxExperts];
  __shared__ int rcnt[4][kMaxExperts];
  __shared__ MassKey run_s[4][64];   // four sorted runs of 64 experts
  __shared__ int runpos_s[kMaxExperts];  // an expert's place in its own run
  __shared__ double wtot_s[4];  // per-wave totals of the prefix scan
  __shared__ int cut_s;         // first index not provably below the threshold
  __shared__ uint32_t mask1_s[kMaxExperts];  // one-block calls: rows per expert
  __shared__ int tk_s[kMaxRows * 8];          // this block's top-k
  __shared__ int pick_s[kMaxRows * 8];        // expert taken by each (row, slot)
  __shared__ int m_sh;
  __shared__ uint32_t live_s;  // bit r: row r of the block is live
  __shared__ PermuteLds perm_lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;
  const float* lb = plan.logits + (size_t)b * R * E;

  if (tid == 0) m_sh = E;
  if (tid < kMaxExperts) mask1_s[tid] = 0u;
  // live rows (bit r: row r): all rows of the block unless the call passes a
  // mask; a resolved row adds nothing to the mass and takes no route.  A mask
  // is read by wave 0 and broadcast through LDS (read after the first
  // barrier below).
  if constexpr (kMasked) {
    if (wave == 0) {
      const uint8_t* live = plan.live + (size_t)b * R;
      const uint64_t lb64 = __ballot(lane < R && live[lane] != 0);
      if (lane == 0) live_s = static_cast<uint32_t>(lb64);
    }
  }
  auto row_is_live = [&](int r) -> bool {
    if constexpr (kMasked) return (live_s >> r) & 1u;
    else return r < R;
  };

  // The softmax, block mass and coreset are needed below a threshold of 1, for
  // an expert budget (a cut in mass order) and for the block-mass and coreset
  // outputs.  A full-route call without them (decode, verification) needs
  // only the row maxima, the top-k of the logits and the gates, whose u
  // values are recomputed for the chosen experts.
  const bool need_mass = tau < 1.0f || (plan.budget > 0 && plan.budget < E) || block_mass != nullptr ||
                         coreset_ids != nullptr;

  // rows w and w+16 on wave w: logits to LDS, row maxima (exact, order-free),
  // and u = exp(l - max) as 8 independent chains per lane (4 when only the
  // first row exists).  Rows past R and experts past E hold -inf logits; the
  // u of rows past R is not computed and never read.
  {
    // the 8 logit loads are unconditional (absent rows and experts read row 0,
    // expert 0 and are replaced by -inf), so they are in flight together: a
    // conditional load made each wait for the one before
    float raw[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = wave + 16 * h, e = lane + 64 * s;
        raw[h][s] = lb[(r < R ? r : 0) * E + (e < E ? e : 0)];
      }
    float lv[2][4], mx[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = wave + 16 * h;
      float mm = -INFINITY;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        const float v = r < R && e < E ? raw[h][s] : -INFINITY;
        l_s[r][e] = v;
        lv[h][s] = v;
        mm = fmaxf(mm, v);
      }
      mx[h] = wave_max_f32(mm);
      if (lane == 0) m_s[r] = mx[h];
    }
    // both rows when the second exists (the first then exists too: its u is
    // computed even if it is resolved, and never read), else the first alone
    if (need_mass && wave + 16 < R) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int r = wave + 16 * h, e = lane + 64 * s;
          p_s[pidx(r, e)] = exp_reduced(static_cast<double>(lv[h][s]) - static_cast<double>(mx[h]));
        }
    } else if (need_mass && wave < R) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        p_s[pidx(wave, e)] = exp_reduced(static_cast<double>(lv[0][s]) - static_cast<double>(mx[0]));
      }
    }
  }
  __syncthreads();

  if (need_mass) {

    // Z: chunk partial sums, one thread per (row, chunk), then the fixed tree
    // (live rows; the others have no u)
    if (tid < kMaxRows * 8) {
      const int r = tid >> 3, j = tid & 7;
      if (row_is_live(r)) {
        const int lo = (j * E) / 8, hi = ((j + 1) * E) / 8;
        double acc = 0.0;
#pragma unroll 8
        for (int e = lo; e < hi; ++e) acc = acc + p_s[pidx(r, e)];
        zpart[r][j] = acc;
      }
    }
    __syncthreads();
    if (tid < R) {
      double p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = zpart[tid][j];
      p[0] = p[0] + p[4];
      p[1] = p[1] + p[5];
      p[2] = p[2] + p[6];
      p[3] = p[3] + p[7];
      p[0] = p[0] + p[2];
      p[1] = p[1] + p[3];
      z_s[tid] = p[0] + p[1];
    }
    __syncthreads();

    // block mass, one thread per expert: p = u / Z for each row, summed over
    // rows ascending (the 8 divisions of a group are independent, only the adds
    // are chained); only live rows add: rows past R (blocks of 1, 2 or 4 rows)
    // and resolved rows have no u
    if (tid < E) {
      double acc = 0.0;
      for (int r0 = 0; r0 < R; r0 += 8) {
        double q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = p_s[pidx(r0 + i, tid)] / z_s[r0 + i];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (row_is_live(r0 + i)) acc = acc + q[i];
      }
      mass_s[tid] = acc;
    }
    if (tid == 0) cut_s = kMaxExperts;
    __syncthreads();

    // rank under (mass desc, id asc).  Waves 0..3 each sort 64 experts in
    // registers (experts past E carry mass +0 and the largest ids, so they sort
    // after every real expert); then thread
    // (expert e, run q) counts the experts of run q that beat e: e's place in
    // its own run, or a binary search (the beating experts are a prefix of a
    // sorted run).  The rank is the sum over the four runs.
    if (wave < 4) {
      const int e = 64 * wave + lane;
      MassKey k;
      k.m = e < E ? static_cast<uint64_t>(__double_as_longlong(mass_s[e])) : 0ull;
      k.nid = ~static_cast<uint32_t>(e);
      wave_sort64(k, lane);
      run_s[wave][lane] = k;
      runpos_s[~k.nid & 255] = lane;
    }
    __syncthreads();
    {
      const int e = tid & 255, q = tid >> 8;
      if (e < E) {
        int cnt;
        if (q == (e >> 6)) {
          cnt = runpos_s[e];
        } else {
          MassKey me;
          me.m = static_cast<uint64_t>(__double_as_longlong(mass_s[e]));
          me.nid = ~static_cast<uint32_t>(e);
          cnt = 0;
#pragma unroll
          for (int step = 32; step > 0; step >>= 1)
            if (beats(run_s[q][cnt + step - 1], me)) cnt += step;
          // the steps reach index 62 at most: all 64 beating e ends at 63
          if (cnt == 63 && beats(run_s[q][63], me)) cnt = 64;
        }
        rcnt[q][e] = cnt;
      }
    }
    __syncthreads();
    if (tid < E) {
      const int rank = rcnt[0][tid] + rcnt[1][tid] + rcnt[2][tid] + rcnt[3][tid];
      rank_s[tid] = rank;
      order_s[min(rank, kMaxExperts - 1)] = tid;
      smass_s[min(rank, kMaxExperts - 1)] = mass_s[tid];
    }
    __syncthreads();

    if (tau < 1.0f) {
      // the cut, certified from a parallel scan where the bounds decide it
      // (see the header); tid < 256 holds prefix index tid
      constexpr double kLo = 1.0 - 0x1p-40, kHi = 1.0 + 0x1p-40;
      double v = 0.0;
      if (tid < kMaxExperts) {
        v = tid < E ? smass_s[tid] : 0.0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const double o = __shfl_up(v, d, 64);
          if (lane >= d) v = v + o;
        }
        if (lane == 63) wtot_s[wave] = v;
      }
      __syncthreads();
      if (tid < kMaxExperts) {
        double off = 0.0;
        for (int w = 0; w < wave; ++w) off = off + wtot_s[w];
        const double pfx = v + off;
        const double total = ((wtot_s[0] + wtot_s[1]) + wtot_s[2]) + wtot_s[3];
        cum_s[tid] = pfx;
        // the first index of this wave that is not provably below the threshold
        const bool open = tid < E && !(pfx * kHi < static_cast<double>(tau) * total * kLo);
        const uint64_t bal = __ballot(open);
        if (bal != 0ull && lane == 0) atomicMin(&cut_s, 64 * wave + __builtin_ctzll(bal));
      }
      __syncthreads();
      const int i0 = cut_s;
      const double total = ((wtot_s[0] + wtot_s[1]) + wtot_s[2]) + wtot_s[3];
      const bool certified = i0 < E && cum_s[i0] * kLo >= static_cast<double>(tau) * total * kHi;
      if (certified) {
        if (tid == 0) m_sh = i0 + 1;
      } else {
        // the serial sum of the contract, one lane; batches of 16, the next
        // batch's loads in flight while this one adds (loads and stores are
        // unconditional: the arrays hold 256 entries, values past E unread)
        __syncthreads();  // everyone has read cum_s (the scan) above
        if (tid == 0) {
          double c = 0.0;
          double x[16], nxt[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = smass_s[i];
          for (int i0s = 0; i0s < E; i0s += 16) {
            const int n0 = min(i0s + 16, kMaxExperts - 16);
#pragma unroll
            for (int i = 0; i < 16; ++i) nxt[i] = smass_s[n0 + i];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              c = c + x[i];
              x[i] = c;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) cum_s[i0s + i] = x[i];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = nxt[i];
          }
        }
        __syncthreads();
        if (tid < E) {
          const double thr = static_cast<double>(tau) * cum_s[E - 1];
          // cum is non-decreasing, so exactly one index is the first to reach thr
          if (cum_s[tid] >= thr && (tid == 0 || cum_s[tid - 1] < thr)) m_sh = tid + 1;
        }
      }
    }
    __syncthreads();
  }  // need_mass
  // no live row: an empty coreset; else the threshold cut, then the budget
  int m = plan.budget > 0 ? min(m_sh, plan.budget) : m_sh;
  if constexpr (kMasked) m = live_s == 0u ? 0 : m;

  if (coreset_ids && tid < E) coreset_ids[(size_t)b * E + tid] = tid < m ? order_s[tid] : -1;
  if (coreset_size && tid == 0) coreset_size[b] = m;
  if (block_mass && tid < E) block_mass[(size_t)b * E + tid] = mass_s[tid];

  // restricted top-k: half a wave per row (rows 2w and 2w+1 on wave w); each
  // lane sorts its 8 candidates (experts (lane&31) + 32*s) by key in
  // registers, and every slot takes the best head of the half-wave: the largest high
  // word (logit), then, only if several lanes hold it, the largest low word
  // (lowest id).  The lane whose head was taken records it and moves on.
  // Waves whose two rows are past R (blocks of fewer than 32 rows) skip it.
  if (2 * wave < R) {
    const int half = lane >> 5, hl = lane & 31;
    const int r = 2 * wave + half;
    const bool row_ok = row_is_live(r);
    // (the LDS reads are unconditional and the tests bitwise: written with
    // short-circuit conditions, each candidate became a branch around its
    // own LDS round trip.  rank_s is unset without mass work, where m = E.)
    uint64_t key[8];
    int rk[8];
    float lg[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      rk[s] = rank_s[hl + 32 * s];
      lg[s] = l_s[r][hl + 32 * s];
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int e = hl + 32 * s;
      const bool ok = row_ok & (e < E) & ((m >= E) | (rk[s] < m));
      key[s] = ok ? (static_cast<uint64_t>(logit_key(lg[s])) << 32) | static_cast<uint32_t>(~e) : 0ull;
    }
    sort8_desc(key);
    // the lane's candidates stay in registers: a lane whose head is taken
    // shifts its list up by one
    int k_eff = 0;  // slots filled in this lane's row
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= K) break;
      const uint64_t head = key[0];
      const uint32_t hh = static_cast<uint32_t>(head >> 32), hlo = static_cast<uint32_t>(head);
      const uint32_t bh = half_max_u32(hh);
      const bool top = head != 0ull && hh == bh;  // (a real key has ~id != 0 below)
      const uint64_t tb = __ballot(top);
      const uint32_t tlo = static_cast<uint32_t>(tb), thi = static_cast<uint32_t>(tb >> 32);
      bool popped = top;
      if (__builtin_popcount(tlo) > 1 || __builtin_popcount(thi) > 1) {
        // equal logits in some row of this wave: the lowest id wins
        const uint32_t bl = half_max_u32(top ? hlo : 0u);
        popped = top && hlo == bl;
      }
      if (popped) pick_s[r * 8 + j] = static_cast<int>(~hlo);
      k_eff += (half ? thi : tlo) != 0u ? 1 : 0;
#pragma unroll
      for (int i = 0; i < 7; ++i) key[i] = popped ? key[i + 1] : key[i];
      key[7] = popped ? 0ull : key[7];
      if (tb == 0ull) break;  // both rows exhausted
    }
    __builtin_amdgcn_wave_barrier();
    const int my_e = hl < k_eff ? pick_s[r * 8 + hl] : -1;  // lane hl keeps slot hl
    // gates: u of the chosen experts (recomputed: same operations, same
    // bits); each lane sums its row's slots in order (empty slots add +0)
    const double u = my_e >= 0
                         ? exp_reduced(static_cast<double>(l_s[r][max(my_e, 0)]) - static_cast<double>(m_s[r]))
                         : 0.0;
    double* u_s = &zpart[0][0];  // [row][slot]
    if (hl < 8) u_s[r * 8 + hl] = u;
    __builtin_amdgcn_wave_barrier();
    double U = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) U = U + u_s[r * 8 + j];
    if (r < R && hl < K) {  // resolved rows too: their slots are -1 / 0
      const int row = b * R + r;
      const bool ok = hl < k_eff;
      const int e_out = ok ? my_e : -1;
      topk[(size_t)row * K + hl] = e_out;
      gates[(size_t)row * K + hl] = ok ? static_cast<float>(u / U) : 0.0f;
      tk_s[r * K + hl] = e_out;
      if (ok) atomicOr(&mask1_s[my_e], 1u << r);
    }
  }

  __syncthreads();
  if (plan.B == 1) {
    // a one-block call: its own routing is the whole call
    permute_single(plan, perm_lds, mask1_s, tk_s);
    return;
  }
  // many blocks: publish this block's rows per expert; the permutation is
  // built by the kernels queued next (permute_blocks.hip)
  if (tid < E) plan.blockmask[(size_t)b * E + tid] = mask1_s[tid];
}

hipError_t launch_route_blocks(const Plan& p, float tau, hipStream_t s) {
  if (p.live) route_block_kernel<true><<<p.B, kThreads, 0, s>>>(p, tau);
  else route_block_kernel<false><<<p.B, kThreads, 0, s>>>(p, tau);
  return hipGetLastError();
}

}  // namespace cmoe
