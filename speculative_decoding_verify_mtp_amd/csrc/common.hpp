// Shared device helpers of the verify-step kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mtp_verify.h"

namespace mtpv {

constexpr int kPage = MTP_PAGE_SIZE;
constexpr int kWave = 64;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Per-device sticky status word (MTP_DEV_* bits).  Kernels OR bits into it
// with a global atomic; the host reads it with hipMemcpyFromSymbol.
__device__ unsigned int g_status;

__device__ __forceinline__ void raise_status(unsigned bits) { atomicOr(&g_status, bits); }

// Splits of an output row whose accumulators the combine requests in its
// first batch (four 16-lane groups of kCombineFast / 4).
constexpr int kCombineFast = 32;
// In a combine launch of its own, split-layout rows with at most
// kGroupedMaxSplits splits are combined four rows per wave (one per 16-lane
// group), like the stream layout's, when there are enough rows for the waves
// to take several rounds (with few rows, one row per wave has all of a row's
// splits in flight at once).  The step's finish launch keeps one row per wave
// for the split layout (a larger finish kernel cost the latency-bound steps
// more than it saved).
constexpr int kGroupedMaxSplits = 16;
constexpr long kGroupedMinRows = 4096;
__host__ __device__ inline bool grouped_split_combine(int max_splits, long rows) {
  return max_splits <= kGroupedMaxSplits && rows >= kGroupedMinRows;
}

// Stores of partial rows (split partials, stream pieces) that a kernel
// writes as whole rows (1 KB per store instruction) and the next launch
// reads on any XCD.  With the sc1 cache policy the L2 writes them through as
// they are stored; plain stores leave them dirty in the writer's L2, to be
// written back at the end of the launch before the next one may start (the
// per-split kernel on one sequence: bitnet2b_chain step 14.2 -> 13.7 us,
// llama3_8b_tree 24.6 -> 23.2 us, its nested KV8 form 27.9 -> 26.5 us; the
// stream kernel's ragged batch step 903 -> 899 us; the D = 64 direct
// kernel, staging its rows through LDS for this, lca_segments 61.05 ->
// 60.86 us).  Stores of 16-byte pieces of rows straight from registers stay
// plain, merged into whole lines in the L2 (written through, the direct
// kernel's lca_segments partial took 53.0 -> 55.6 us), and so do the nested
// stream kernel's (ragged batch KV8 900 -> 913 us written through).
// `base` is wave-uniform (it becomes a buffer resource in scalar
// registers); `i` counts floats from it, below 2^29.
constexpr int kCpolSc1 = 16;  // cache-policy operand of the buffer builtins: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(float* base) {
  // the base from the first active lane (the same in every lane), so that
  // the resource is built in scalar registers without a loop over lanes
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  float* u = reinterpret_cast<float*>((uintptr_t)(((uint64_t)hi << 32) | lo));
  // num_records: 2^31 - 1 bytes; word 3: 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, 0x7fffffff, 0x00020000);
}
// base[i] = m, base[i + 1] = l
__device__ __forceinline__ void store_partial_ml(float* base, int i, float m, float l) {
  const __amdgpu_buffer_rsrc_t r = partial_rsrc(base);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), r, i * 4, 0, kCpolSc1);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), r, i * 4 + 4, 0, kCpolSc1);
}
// base[i .. i + 3] = v (16-byte aligned)
__device__ __forceinline__ void store_partial4(float* base, int i, float4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(u, partial_rsrc(base), i * 4, 0, kCpolSc1);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float qnan() { return __builtin_nanf(""); }

// 2^x on the transcendental unit; exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x * y rounded to fp32 and kept out of fp contraction: where one product is
// both compared (a running maximum) and subtracted from it inside an
// exponential, an fma would subtract from the exact product, leaving up to
// half an ulp of it (above 2^31 enough to overflow the exponential).
__device__ __forceinline__ float mul_rn(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const unsigned lo = __shfl((unsigned)v, src);
  const unsigned hi = __shfl((unsigned)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Reductions over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48), the result in every lane.  gfx950's lane swaps exchange rows
// inside the vector ALU (v_permlane16_swap: rows 2i and 2i + 1;
// v_permlane32_swap: the two 32-lane halves), with no LDS round trip as for
// ds_bpermute.  After a swap of a register with itself, the two results hold
// a lane's value and its partner's in some order, so a symmetric operation on
// them is the pairwise reduction: (x0 op x1) op (x2 op x3) in every lane.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// The same with IEEE maximum (NaN-propagating; no quieting of the inputs,
// two instructions fewer per level).
__device__ __forceinline__ float rows4_maximum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short h) {
  return __uint_as_float((unsigned)h << 16);
}

// In-block visibility of block node `lane` as a W-bit row (bit j set when the
// node may attend to block row j); lanes >= W return 0.  Every lane of the
// wave must be active.  `ok` (wave-uniform) reports whether the mask
// description is well formed.
//  CHAIN   : rows 0..i (the AR-causal verifier mask).
//  TREE    : the node and its ancestors; the ancestor closure is built by
//            pointer jumping, 6 rounds cover any depth below 64.
//  SEGMENT : own-segment rows up to i, plus rows of the `lookback` previous
//            segments (all earlier segments when lookback < 0).
// `id` is this lane's mask id (ids[lane] for lane < W, anything otherwise).
__device__ __forceinline__ uint64_t node_visibility(int kind, int id, int W, int lookback, int lane,
                                           bool& ok) {
  const bool in = lane < W;
  if (!in) id = 0;
  if (kind == MTP_MASK_CHAIN) {
    ok = true;
    return in ? (~0ull >> (63 - lane)) : 0ull;
  }
  if (kind == MTP_MASK_TREE) {
    const bool bad = in && lane >= 1 && (id < 0 || id >= lane);
    ok = __ballot(bad) == 0ull;
    if (!ok) return 0ull;
    int up = (in && lane >= 1) ? id : lane;
    uint64_t anc = in ? ((1ull << lane) | (lane >= 1 ? (1ull << id) : 0ull)) : 0ull;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      anc |= shfl64(anc, up);
      up = __shfl(up, up);
    }
    return anc;
  }
  if (kind == MTP_MASK_SEGMENT) {
    const int prev = __shfl(id, lane > 0 ? lane - 1 : 0);
    const int step = id - prev;
    const bool bad = in && (lane == 0 ? id != 0 : (step != 0 && step != 1));
    ok = __ballot(bad) == 0ull;
    if (!ok) return 0ull;
    uint64_t vis = 0;
    for (int j = 0; j < W; ++j) {
      const int sj = __shfl(id, j);
      const bool v = (sj == id && j <= lane) || (sj < id && (lookback < 0 || id - sj <= lookback));
      vis |= (uint64_t)v << j;
    }
    return in ? vis : 0ull;
  }
  ok = false;
  return 0ull;
}

// Arguments of the attention kernels (split-K partials + combine).
struct AttnParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const void* k_new;
  const void* v_new;
  const uint8_t* mask_kind;
  const int32_t* mask_ids;
  float* part_acc;  // [B, max_splits, Hkv, R, D]
  float* part_ml;   // [B, max_splits, Hkv, R, 2]: running max (log2 domain), sum
  float* out;       // [B, W, Hq, D]
  float* lse;       // [B, W, Hq] or null
  int B, W, Hq, Hkv, g, R;
  int nRB;         // row blocks per (sequence, KV head)
  int S;           // committed tokens per split (multiple of 32) past the first n1 splits
  int n1, S1;      // splits 0 .. n1 - 1 hold S1 tokens each (n1 = 0: every split holds S)
  int max_splits;  // splits of max_ctx
  int max_pages, num_pages, max_ctx, lookback;
  float scale_log2;  // softmax scale * log2(e)
  // The step's target prologue (per-split LDS kernel; logits == nullptr:
  // off): workgroup j < B * W of the launch also writes tgt[j], the argmax
  // of logits row j ([B, W, V] fp32), so that the acceptance after the
  // launch reads W targets instead of W rows of V logits.
  const float* logits = nullptr;
  int32_t* tgt = nullptr;
  int V = 0;
};

// Work item of the split-K kernels: (row block, KV head, split) of sequence
// blockIdx.y, row block fastest so that the waves of one workgroup read
// neighbouring KV rows.
struct Item {
  int rb, kvh, split;
};

__device__ __forceinline__ Item decode_item(int item, const AttnParams& p) {
  Item it;
  it.rb = item % p.nRB;
  const int t = item / p.nRB;
  it.kvh = t % p.Hkv;
  it.split = t / p.Hkv;
  return it;
}

// Work item of workgroup `item` out of `n_items` = nRB * (splits x heads).
// Workgroups are dealt to the eight XCDs round robin, and the nRB row blocks
// of one (split, head) read the same K/V: each group of 8 * nRB consecutive
// workgroups holds eight (split, head) units, row block r of unit u at
// position 8 r + u, so a unit's row blocks land on one XCD and share its L2.
// The last units (fewer than eight) take consecutive positions.
__device__ __forceinline__ Item decode_item_xcd(int item, int n_items, const AttnParams& p) {
  const int nrb = p.nRB;
  const int units = n_items / nrb;
  const int full = (units / 8) * 8 * nrb;  // workgroups in whole groups
  int u, rb;
  if (item < full) {
    const int grp = item / (8 * nrb);
    const int r = item - grp * 8 * nrb;
    rb = r >> 3;
    u = grp * 8 + (r & 7);
  } else {
    const int t = item - full;
    rb = t % nrb;
    u = full / nrb + t / nrb;
  }
  Item it;
  it.rb = rb;
  it.kvh = u % p.Hkv;
  it.split = u / p.Hkv;
  return it;
}

// Split geometry of the per-split kernels: splits 0 .. n1 - 1 hold S1
// committed tokens, the later ones S; a context of L tokens has
// num_splits(...) splits (at least one: the block's own rows).
__host__ __device__ inline int split_start(int s, int S, int n1, int S1) {
  return s <= n1 ? s * S1 : n1 * S1 + (s - n1) * S;
}
__host__ __device__ inline int num_splits(int L, int S, int n1, int S1) {
  if (L <= 0) return 1;
  const int head = n1 * S1;
  return L <= head ? (L + S1 - 1) / S1 : n1 + (L - head + S - 1) / S;
}
__device__ __forceinline__ int split_start(const AttnParams& p, int s) { return split_start(s, p.S, p.n1, p.S1); }
__device__ __forceinline__ int num_splits(const AttnParams& p, int L) { return num_splits(L, p.S, p.n1, p.S1); }

// Lane's mask id of sequence b (0 for lanes past the block).
__device__ __forceinline__ int lane_mask_id(const AttnParams& p, int b, int lane) {
  return lane < p.W ? p.mask_ids[(size_t)b * p.W + lane] : 0;
}

}  // namespace mtpv
