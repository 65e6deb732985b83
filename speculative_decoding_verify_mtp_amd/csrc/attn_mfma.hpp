// Split-K verify attention on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16).
//
// One wave = one work item: (sequence b, KV head, row block, split of the
// committed context).  The rows of a KV head are the W block rows times the
// g query heads of its GQA group (row rho = w * g + j reads query head
// kvh * g + j); a row block is RB tiles of 16 rows.  Every K/V row a wave
// loads feeds all RB*16 rows, so each committed byte is read once per row
// block.
//
// Scores are computed transposed, S^T = K Q^T, so that the probabilities come
// out of the accumulator already in the operand layout the PV product needs,
// and PV is computed as acc^T = V^T P^T:
//   * K is MFMA operand A: lane (i = lane%16, q = lane/16) holds key i,
//     elements [32m + 8q, +8) for d-chunk m -- for each chunk the four lanes
//     of a key read 64 contiguous bytes.
//   * Q^T is operand B with the same d mapping, loaded once per item.
//   * S^T accumulator: lane (j, q) holds S[row j][keys 4q..4q+3] of a 16-key
//     tile, so a lane owns one row and the row reductions need only the two
//     cross-quarter shuffles.
//   * V^T is operand A of PV.  The output d-index of MFMA column tile t, row
//     i is d = (D/16) * i + t, so lane (i, q) needs V[key][(D/16) i .. +D/16)
//     for its 8 keys: sixteen lanes read one whole K/V row per load (fully
//     coalesced), and operand t takes element t of each of the 8 vectors.
//   * P^T is operand B of PV: lane (j, q) supplies row j, keys
//     {4q..4q+3} of tile 0 and of tile 1 -- exactly the S^T registers.
//   * acc^T accumulator: lane (j, q) ends up owning row j, d in
//     [q * D/4, (q+1) * D/4).
// In attn_partial_mfma (launched for D = 64; D = 128 runs the same tile
// step from the LDS ring kernels) K and V go straight from HBM to registers
// with 8-byte loads; no LDS is needed.  Online softmax runs in the log2 domain.
#pragma once

#include "common.hpp"

namespace mtpv {

template <int D>
struct VRow;  // one lane's slice of a V row: D/16 bf16 values
template <>
struct VRow<128> {
  uint4 v;
};
template <>
struct VRow<64> {
  uint2 v;
};

template <int D>
__device__ __forceinline__ VRow<D> load_vrow(const uint16_t* p) {
  VRow<D> r;
  if constexpr (D == 128)
    r.v = *reinterpret_cast<const uint4*>(p);
  else
    r.v = *reinterpret_cast<const uint2*>(p);
  return r;
}

template <int D>
__device__ __forceinline__ unsigned vrow_dword(const VRow<D>& r, int i) {
  if constexpr (D == 128) {
    return i == 0 ? r.v.x : i == 1 ? r.v.y : i == 2 ? r.v.z : r.v.w;
  } else {
    return i == 0 ? r.v.x : r.v.y;
  }
}

// Operand A of the PV product for output column tile t: element t of each of
// the lane's 8 V vectors, packed pairwise with one byte permute per dword
// (v_perm_b32: selector bytes 0-3 pick from the second source, 4-7 from the
// first).
template <int D, int T>
__device__ __forceinline__ bf16x8 pack_v_operand(const VRow<D> (&vv)[8]) {
  constexpr unsigned kSel = (T & 1) ? 0x07060302u : 0x05040100u;
  unsigned w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned x = vrow_dword<D>(vv[2 * j], T >> 1);
    const unsigned y = vrow_dword<D>(vv[2 * j + 1], T >> 1);
    w[j] = __builtin_amdgcn_perm(y, x, kSel);  // (x, y) halves T&1 -> low, high
  }
  bf16x8 r;
  __builtin_memcpy(&r, w, sizeof(r));
  return r;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <int D, int RB>
struct MfmaState {
  float m[RB];           // reference row max (log2 domain), replicated over the 4 quarters
  float l[RB];           // this lane's share of the running row sum
  f32x4 acc[RB][D / 16];  // acc^T tiles
};

// The reference max of a row only moves when the row max exceeds it by more
// than this many log2 units, so the accumulator rescale (a read-modify-write
// of every accumulator register) is skipped on almost every tile.  Weights
// relative to the reference stay below 2^8, far from fp32 overflow.
constexpr float kRescaleSlack = 8.f;

// Log2-domain weights pe[e] = 2^(x[e] s - m + bias) of eight scores against
// the reference m (the rounded product mx s of the largest raw score mx, or
// an earlier one).  While |m| < 2^20 one fma per weight: its exact product
// differs from the rounded one by less than 2^-3.  Beyond, the product is
// rounded first, so that the argument of the largest score is exactly its
// distance to the reference: with an fma, half an ulp of a product above
// 2^31 would overflow the exponential (NaN rows for very large scores).
// The choice is wave-uniform.
__device__ __forceinline__ void log2_weights(const float (&x)[8], float s, float m, float bias,
                                             float (&pe)[8]) {
  if (__ballot(fabsf(m) > 0x1p20f) == 0ull) {
    const float c = bias - m;
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(fmaf(x[e], s, c));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = fast_exp2((mul_rn(x[e], s) - m) + bias);
  }
}

// Largest of eight scores.  IEEE maximum (NaN-propagating) maps to gfx950's
// three-input v_maximum3_f32 and, unlike fmaxf, needs no quieting of the
// MFMA results first; the masked scores are -inf, never NaN.  (Used by the
// nested-cache kernels, 1110 -> 1089 us with this and split_bf16_hi_lo on the
// ragged batch, and by the lean tile_softmax; the bf16 stream kernel measured
// 915 -> 928 us and 879 -> 892 us with them and keeps fmaxf and per-value
// conversions.)
__device__ __forceinline__ float max8(const float (&x)[8]) {
  const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), x[2]);
  const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[3], x[4]), x[5]);
  const float c = __builtin_elementwise_maximum(x[6], x[7]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// p = hi + lo with hi = bf16(p) (round to nearest even) and lo = bf16(p - hi)
// (p - hi is exact in fp32), eight values packed as two bf16x8 MFMA operands.
// Two values per conversion; hi comes back to fp32 by a shift or a mask.
__device__ __forceinline__ void split_bf16_hi_lo(const float (&p)[8], bf16x8& hi, bf16x8& lo) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  unsigned hw[4], lw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2 h2 = {(__bf16)p[2 * j], (__bf16)p[2 * j + 1]};
    unsigned u;
    __builtin_memcpy(&u, &h2, 4);
    hw[j] = u;
    const float h0 = __uint_as_float(u << 16), h1 = __uint_as_float(u & 0xffff0000u);
    const bf16x2 l2 = {(__bf16)(p[2 * j] - h0), (__bf16)(p[2 * j + 1] - h1)};
    __builtin_memcpy(&lw[j], &l2, 4);
  }
  __builtin_memcpy(&hi, hw, 16);
  __builtin_memcpy(&lo, lw, 16);
}

// Raw scores of one 32-key tile for the RB row tiles: x[k][e] = q . k of
// this lane's row of tile k and its e-th key (keys {4q..4q+3} of the first
// 16-key half, then the same of the second), unscaled.
template <int D, int RB>
__device__ __forceinline__ void tile_scores(const bf16x8 (&qf)[RB][D / 32],
                                            const bf16x8 (&kf)[2][D / 32], float (&x)[RB][8]) {
  constexpr int NC = D / 32;
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][m], qf[k][m], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][m], qf[k][m], s1, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[k][e] = s0[e];
      x[k][4 + e] = s1[e];
    }
  }
}

// Online-softmax update of one 32-key tile from its raw scores: the running
// max and sum of each row tile, the rescale of its accumulators when the
// reference max moves, and the tile's probabilities as the PV product's
// operand (P^T, bf16 hi + lo parts).  vis(k, e) tells whether row tile k may
// see key e of this lane's 8 keys.
// kLean: the row max by three-input IEEE maxima and the hi + lo parts by
// packed conversions (fewer instructions: per-split and direct kernels,
// llama3_8b_tree 18.0 -> 17.6 us, bitnet2b_chain 9.23 -> 9.13 us,
// lca_segments 54.2 -> 53.6 us); the stream kernel keeps the other form
// (ragged batch 879 us against 892 us lean).
template <int D, int RB, bool kLean = true, typename VisFn>
__device__ __forceinline__ void tile_softmax(float (&x)[RB][8], float scale_log2,
                                             MfmaState<D, RB>& st, bf16x8 (&pf)[RB],
                                             bf16x8 (&pl)[RB], VisFn vis) {
  constexpr int NT = D / 16;
  // P is split into bf16 hi + lo parts (two PV products): one bf16 rounding
  // of P alone costs up to 2^-9 relative per weight, which exceeds the
  // 1e-3 + 1e-2|ref| bound on short or peaked rows; hi + lo keeps ~16 bits.
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    // raw scores; the scale (> 0) is applied after the max and inside the exp
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!vis(k, e)) x[k][e] = neg_inf();
    float mx;
    if constexpr (kLean) {
      mx = mul_rn(rows4_maximum(max8(x[k])), scale_log2);
    } else {
      mx = fmaxf(fmaxf(fmaxf(x[k][0], x[k][1]), fmaxf(x[k][2], x[k][3])),
                 fmaxf(fmaxf(x[k][4], x[k][5]), fmaxf(x[k][6], x[k][7])));
      mx = mul_rn(rows4_max(mx), scale_log2);
    }
    const float mold = st.m[k];
    const float mref = mx > mold + kRescaleSlack ? mx : mold;
    const float muse = mref == neg_inf() ? 0.f : mref;
    float pw[8];
    log2_weights(x[k], scale_log2, muse, 0.f, pw);
    float sum = 0.f;
    if constexpr (kLean) {
      sum = ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
      split_bf16_hi_lo(pw, pf[k], pl[k]);
    } else {
      __bf16 ph[8], plo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = pw[e];
        sum += pe;
        ph[e] = (__bf16)pe;
        plo[e] = (__bf16)(pe - (float)ph[e]);
      }
      __builtin_memcpy(&pf[k], ph, sizeof(bf16x8));
      __builtin_memcpy(&pl[k], plo, sizeof(bf16x8));
    }
    if (__ballot(mref != mold) != 0ull) {  // wave-uniform: rare after the first tile
      const float alpha = fast_exp2(mold - muse);
      st.l[k] *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) st.acc[k][t] *= alpha;
    }
    st.l[k] += sum;
    st.m[k] = mref;
  }
}

// PV accumulate of one 32-key tile: acc^T += V^T P^T for the hi and the lo
// part of P.  vv: V vectors of keys {4q..4q+3, 16+4q..16+4q+3}.
template <int D, int RB>
__device__ __forceinline__ void tile_pv(const bf16x8 (&pf)[RB], const bf16x8 (&pl)[RB],
                                        const VRow<D> (&vv)[8], MfmaState<D, RB>& st) {
  constexpr int NT = D / 16;
#define MTPV_PV_STEP(T)                                                                 \
  if constexpr ((T) < NT) {                                                            \
    const bf16x8 a = pack_v_operand<D, (T)>(vv);                                       \
    _Pragma("unroll") for (int k = 0; k < RB; ++k) {                                   \
      st.acc[k][(T)] =                                                                 \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[k], st.acc[k][(T)], 0, 0, 0);   \
      st.acc[k][(T)] =                                                                 \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[k], st.acc[k][(T)], 0, 0, 0);   \
    }                                                                                  \
  }
  MTPV_PV_STEP(0)
  MTPV_PV_STEP(1)
  MTPV_PV_STEP(2)
  MTPV_PV_STEP(3)
  MTPV_PV_STEP(4)
  MTPV_PV_STEP(5)
  MTPV_PV_STEP(6)
  MTPV_PV_STEP(7)
#undef MTPV_PV_STEP
}

// One 32-key tile: scores, online-softmax update, PV accumulate.
// kf: K operands of the two 16-key halves; vv: V vectors of keys
// {4q..4q+3, 16+4q..16+4q+3}; vis(k, e) tells whether row tile k may see key
// e of this lane's 8 keys.
template <int D, int RB, typename VisFn>
__device__ __forceinline__ void mfma_tile(const bf16x8 (&qf)[RB][D / 32],
                                          const bf16x8 (&kf)[2][D / 32],
                                          const VRow<D> (&vv)[8], float scale_log2,
                                          MfmaState<D, RB>& st, VisFn vis) {
  float x[RB][8];
  tile_scores<D, RB>(qf, kf, x);
  bf16x8 pf[RB], pl[RB];
  tile_softmax<D, RB>(x, scale_log2, st, pf, pl, vis);
  tile_pv<D, RB>(pf, pl, vv, st);
}

// Key index (0..31) inside a 32-key tile of this lane's e-th PV key.
__device__ __forceinline__ int pv_key(int q, int e) { return e < 4 ? 4 * q + e : 16 + 4 * q + (e - 4); }

template <int D, int RB>
__global__ __launch_bounds__(256) void attn_partial_mfma(AttnParams p) {
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  constexpr int VE = D / 16;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int qd = lane >> 4;
  const int b = blockIdx.y;
  const Item it = decode_item(blockIdx.x * 4 + (threadIdx.x >> 6), p);
  if (it.split >= p.max_splits) return;
  const int start = split_start(p, it.split);

  // Loads that do not depend on the context length go out together with it:
  // the split's page indices (held in two registers per lane: lane i has
  // entries i and 64 + i; a split spans at most 128 pages; bounded by the
  // block table, not by the context) and the Q operands.
  const int32_t* btrow = p.block_table + (size_t)b * p.max_pages;
  const int pbase = start >> 4;
  const int pavail = p.max_pages - pbase;
  const int pr0 = lane < pavail ? btrow[pbase + lane] : 0;
  const int pr1 = lane + 64 < pavail ? btrow[pbase + lane + 64] : 0;

  const uint16_t* qbase = static_cast<const uint16_t*>(p.q);
  const uint16_t* kc = static_cast<const uint16_t*>(p.k_cache) + (size_t)it.kvh * D;
  const uint16_t* vc = static_cast<const uint16_t*>(p.v_cache) + (size_t)it.kvh * D;
  const size_t slot_stride = (size_t)p.Hkv * D;

  // Q^T operands of the RB row tiles.
  bf16x8 qf[RB][NC];
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    const int rho = (it.rb * RB + k) * 16 + c;
    if (rho < p.R) {
      const int w = rho / p.g;
      const int j = rho - w * p.g;
      const uint16_t* src =
          qbase + ((size_t)(b * p.W + w) * p.Hq + (size_t)it.kvh * p.g + j) * D + qd * 8;
#pragma unroll
      for (int m = 0; m < NC; ++m) qf[k][m] = load_bf16x8(src + m * 32);
    } else {
#pragma unroll
      for (int m = 0; m < NC; ++m) qf[k][m] = bf16x8{};
    }
  }

  const int mkind = p.mask_kind[b];
  const int mid = lane_mask_id(p, b, lane);
  const int L = p.ctx_lens[b];
  if (L < 0 || L > p.max_ctx) return;  // reported by the combine
  const int ns = num_splits(p, L);
  if (it.split >= ns) return;
  const int end = min(L, split_start(p, it.split + 1));
  const bool last = it.split == ns - 1;

  MfmaState<D, RB> st;
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    st.m[k] = neg_inf();
    st.l[k] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Committed keys [start, end), 32 per step (two pages; start is a multiple
  // of 32).  The K/V rows of the next step are requested before the current
  // step is reduced: one memory round trip per step, overlapped with the
  // compute.
  bool bad = false;
  struct Step {
    bf16x8 kf[2][NC];
    VRow<D> vv[8];
  };
  auto load_step = [&](int t0, Step& d) __attribute__((always_inline)) {
    const int nk = end - t0;  // keys of this tile that are committed (may exceed 32)
    const int pi = (t0 >> 4) - pbase;  // wave-uniform
    int pg0 = __builtin_amdgcn_readlane(pi < 64 ? pr0 : pr1, pi & 63);
    int pg1 = nk > 16 ? __builtin_amdgcn_readlane(pi + 1 < 64 ? pr0 : pr1, (pi + 1) & 63) : pg0;
    if ((unsigned)pg0 >= (unsigned)p.num_pages) {
      bad = true;
      pg0 = 0;
    }
    if ((unsigned)pg1 >= (unsigned)p.num_pages) {
      bad = true;
      pg1 = 0;
    }
    // Keys past the committed range load the tile's first row (always valid)
    // and are masked out of the softmax.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = kt * 16 + c;
      const bool v = key < nk;
      const int pg = v ? (kt ? pg1 : pg0) : pg0;
      const int slot = v ? c : 0;
      const uint16_t* src = kc + ((size_t)pg * kPage + slot) * slot_stride + qd * 8;
#pragma unroll
      for (int m = 0; m < NC; ++m) d.kf[kt][m] = load_bf16x8(src + m * 32);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = pv_key(qd, e);
      const bool v = key < nk;
      const int pg = v ? (e < 4 ? pg0 : pg1) : pg0;
      const int slot = v ? (key & 15) : 0;
      d.vv[e] = load_vrow<D>(vc + ((size_t)pg * kPage + slot) * slot_stride + c * VE);
    }
  };
  auto step = [&](int t0, const Step& d) __attribute__((always_inline)) {
    const int nk = end - t0;
    if (nk >= 32) {
      mfma_tile<D, RB>(qf, d.kf, d.vv, p.scale_log2, st, [](int, int) { return true; });
    } else {
      mfma_tile<D, RB>(qf, d.kf, d.vv, p.scale_log2, st,
                       [&](int, int e) { return (e < 4 ? 4 * qd + e : 16 + 4 * qd + e - 4) < nk; });
    }
  };
  if (start < end) {
    Step s0, s1;  // ping-pong: s0 holds steps t0, s1 steps t0 + 32
    load_step(start, s0);
    for (int t0 = start; t0 < end; t0 += 64) {
      if (t0 + 32 < end) load_step(t0 + 32, s1);
      step(t0, s0);
      if (t0 + 32 >= end) break;
      if (t0 + 64 < end) load_step(t0 + 64, s0);
      step(t0 + 32, s1);
    }
  }

  // In-block keys (the block's own K/V), masked per row, in the last split.
  if (last) {
    bool ok;
    const uint64_t vnode =
        node_visibility(mkind, mid, p.W, p.lookback, lane, ok);
    if (ok) {
      uint64_t vrow[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int rho = min((it.rb * RB + k) * 16 + c, p.R - 1);
        vrow[k] = shfl64(vnode, rho / p.g);
      }
      const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + (size_t)it.kvh * D;
      const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + (size_t)it.kvh * D;
      for (int j0 = 0; j0 < p.W; j0 += 32) {
        bf16x8 kf[2][NC];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          int j = j0 + kt * 16 + c;
          j = j < p.W ? j : 0;
          const uint16_t* src = kn + (size_t)(b * p.W + j) * slot_stride + qd * 8;
#pragma unroll
          for (int m = 0; m < NC; ++m) kf[kt][m] = load_bf16x8(src + m * 32);
        }
        VRow<D> vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int j = j0 + pv_key(qd, e);
          j = j < p.W ? j : 0;
          vv[e] = load_vrow<D>(vn + (size_t)(b * p.W + j) * slot_stride + c * VE);
        }
        // Bits >= W of a visibility row are zero, so padded keys are masked.
        mfma_tile<D, RB>(qf, kf, vv, p.scale_log2, st, [&](int k, int e) {
          const int j = j0 + (e < 4 ? 4 * qd + e : 16 + 4 * qd + e - 4);
          return ((vrow[k] >> j) & 1ull) != 0ull;
        });
      }
    }
  }

  if (bad) {
    if (lane == 0) raise_status(MTP_DEV_BAD_PAGE);
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      st.m[k] = qnan();
#pragma unroll
      for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{qnan(), qnan(), qnan(), qnan()};
    }
  }

  // Store the partial (m, l, unnormalised acc) of every real row: each wave
  // lays a 16-row tile out row-major in its own LDS region, then stores
  // whole rows written through the L2.
  constexpr int kPitch = D + 4;
  __shared__ float stage_rows[4][16 * kPitch];
  float* sw = stage_rows[threadIdx.x >> 6];
  const size_t item_row = (((size_t)b * p.max_splits + it.split) * p.Hkv + it.kvh) * (size_t)p.R;
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    float l = st.l[k];
    l = rows4_sum(l);
    const int rho0 = (it.rb * RB + k) * 16;
    const int rho = rho0 + c;
    if (qd == 0 && rho < p.R) store_partial_ml(p.part_ml + 2 * item_row, 2 * rho, st.m[k], l);
    float* rowp = sw + c * kPitch + qd * (D / 4);
    // lane holds d = qd*D/4 + e*(D/16) + t in acc[k][t][e]
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int t = 0; t < NT; t += 4)
        *reinterpret_cast<float4*>(rowp + e * (D / 16) + t) =
            make_float4(st.acc[k][t][e], st.acc[k][t + 1][e], st.acc[k][t + 2][e], st.acc[k][t + 3][e]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int f = lane; f < 16 * (D / 4); f += kWave) {
      const int row = f / (D / 4);
      const int col = f - row * (D / 4);
      if (rho0 + row < p.R)
        store_partial4(p.part_acc + item_row * D, (rho0 + row) * D + col * 4,
                       *reinterpret_cast<const float4*>(sw + row * kPitch + col * 4));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

}  // namespace mtpv
