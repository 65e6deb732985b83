// Nested KV4 / KV8 cache ("BitNest: Bit-Nested Speculative Decoding for
// Memory-Efficient LLM Inference Acceleration", Sec. 3.4 and Sec. A.2):
// quantization on write, the quantizing commit, and verify attention over the
// two code planes.
//
// Format (per token and KV head, D elements):
//   s = max|x| / 7, t = x / s, q4 = rint(t), qr = clamp(rint(16 t) - 16 q4, -8, 7)
//   (fp32, round half to even); KV4 = s q4, KV8 = (s / 16)(16 q4 + qr).
//   Codes are stored + 8 as nibbles, two per byte, even element low:
//   base / ref planes [pages, Hkv, 16, D/2] bytes, scales [pages, Hkv, 16] fp32.
//
// Attention dequantizes in registers.  With both nibbles of an element, the
// byte 16 (q4 + 8) + (qr + 8) = c8 + 136, c8 = 16 q4 + qr, is built for four
// elements at a time with two masks and a shift, converted exactly to float
// (v_cvt_f32_ubyte) and packed to bf16 (exact: at most 8 significant bits).
// The MFMA products therefore see u = c8 + 136 instead of c8; the offset is
// removed in fp32:
//   scores: q.k = (s_k / 16) (sum_d q_d u_d - 136 sum_d q_d) per key,
//   values: sum_t p_t v_t = sum_t p'_t u_t - 136 sum_t p'_t, p'_t = p_t s_t / 16,
// with sum_d q_d computed once per row and sum_t p'_t kept beside the row sum.
// A KV4 read uses the refinement nibble 8 (qr = 0) and loads no refinement.
#pragma once

#include "accept_commit.hpp"
#include "attn_mfma.hpp"
#include "common.hpp"

namespace mtpv {

constexpr float kNestByteOffset = 136.f;   // u = c8 + 136
constexpr unsigned kNestZeroRef = 0x88888888u;  // eight refinement codes 0

typedef unsigned u32x4n __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// quantization
// ---------------------------------------------------------------------------

__device__ __forceinline__ float load_elem(const void* p, int dtype, size_t i) {
  if (dtype == MTP_F32) return static_cast<const float*>(p)[i];
  return bf16_bits_to_float(static_cast<const unsigned short*>(p)[i]);
}

// Quantizes one vector of D <= 128 elements by one wave: lane l takes
// elements 2l and 2l + 1 and writes byte l of both planes; lane 0 writes the
// scale.  All lanes of the wave must be active.
__device__ __forceinline__ void wave_quantize(const void* x, int dtype, int D, uint8_t* base,
                                              uint8_t* ref, float* scale) {
  const int lane = threadIdx.x & 63;
  const bool in = 2 * lane < D;
  const float x0 = in ? load_elem(x, dtype, 2 * lane) : 0.f;
  const float x1 = in ? load_elem(x, dtype, 2 * lane + 1) : 0.f;
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float s = amax / 7.f;  // IEEE division, as the definition states
  const bool live = s > 0.f;
  const float t0 = live ? x0 / s : 0.f;
  const float t1 = live ? x1 / s : 0.f;
  const float a0 = rintf(t0), a1 = rintf(t1);
  const float r0 = fminf(fmaxf(rintf(16.f * t0) - 16.f * a0, -8.f), 7.f);
  const float r1 = fminf(fmaxf(rintf(16.f * t1) - 16.f * a1, -8.f), 7.f);
  if (in) {
    base[lane] = (uint8_t)(((int)a0 + 8) | (((int)a1 + 8) << 4));
    ref[lane] = (uint8_t)(((int)r0 + 8) | (((int)r1 + 8) << 4));
  }
  if (lane == 0) *scale = s;
}

// Row index of slot (page, head, slot) in the planes (rows of D/2 bytes, or one scale).
__device__ __forceinline__ size_t nest_row(int page, int h, int slot, int Hkv) {
  return ((size_t)page * Hkv + h) * kPage + slot;
}

struct QuantizeParams {
  const void* k_rows;  // [n, Hkv, D]
  const void* v_rows;
  const int32_t* slots;  // [n]: page * 16 + slot
  mtp_nested_kv kv;
  int n, Hkv, D, dtype, num_pages;
};

// One wave per (row, KV head, K or V).
__global__ __launch_bounds__(256) void kv_quantize_kernel(QuantizeParams p) {
  const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long)p.n * p.Hkv * 2) return;
  const bool is_v = item & 1;
  const int h = (int)((item >> 1) % p.Hkv);
  const int r = (int)((item >> 1) / p.Hkv);
  const int slot = p.slots[r];
  if (slot < 0 || slot >= p.num_pages * kPage) {
    if ((threadIdx.x & 63) == 0) raise_status(MTP_DEV_BAD_PAGE);
    return;
  }
  const size_t row = nest_row(slot >> 4, h, slot & 15, p.Hkv);
  const size_t src = ((size_t)r * p.Hkv + h) * p.D;
  const int esz = p.dtype == MTP_F32 ? 4 : 2;
  const char* x = static_cast<const char*>(is_v ? p.v_rows : p.k_rows) + src * esz;
  if (is_v)
    wave_quantize(x, p.dtype, p.D, p.kv.v_base + row * (p.D / 2), p.kv.v_ref + row * (p.D / 2),
                  p.kv.v_scale + row);
  else
    wave_quantize(x, p.dtype, p.D, p.kv.k_base + row * (p.D / 2), p.kv.k_ref + row * (p.D / 2),
                  p.kv.k_scale + row);
}

struct NestedCommitParams {
  CommitParams c;  // k_cache / v_cache / row_bytes unused
  mtp_nested_kv kv;
  int Hkv, D, dtype;
};

// The commit of the accepted rows into a nested cache: the plan of the plain
// commit, then each accepted (position, KV head, K or V) vector is quantized
// by one wave into its slot.
__global__ __launch_bounds__(256) void commit_nested_kernel(NestedCommitParams p) {
  __shared__ int s_src[MTP_MAX_W];
  __shared__ int s_dst[MTP_MAX_W];
  __shared__ int s_meta[2];
  const int b = blockIdx.x;
  commit_plan<false>(p.c, b, commit_prefetch(p.c, b), 0, nullptr, s_src, s_dst, s_meta);
  const int a = s_meta[0];
  const int first = s_meta[1];
  if (a < first) return;
  const int per = p.Hkv * 2;
  const int total = (a - first + 1) * per;
  const int esz = p.dtype == MTP_F32 ? 4 : 2;
  for (int item = threadIdx.x >> 6; item < total; item += blockDim.x >> 6) {
    const int k = first + item / per;
    const int h = (item % per) >> 1;
    const bool is_v = item & 1;
    const int dst = s_dst[k];
    const size_t row = nest_row(dst >> 4, h, dst & 15, p.Hkv);
    const size_t src = (((size_t)b * p.c.W + s_src[k]) * p.Hkv + h) * p.D;
    const char* x = static_cast<const char*>(is_v ? p.c.v_new : p.c.k_new) + src * esz;
    if (is_v)
      wave_quantize(x, p.dtype, p.D, p.kv.v_base + row * (p.D / 2), p.kv.v_ref + row * (p.D / 2),
                    p.kv.v_scale + row);
    else
      wave_quantize(x, p.dtype, p.D, p.kv.k_base + row * (p.D / 2), p.kv.k_ref + row * (p.D / 2),
                    p.kv.k_scale + row);
  }
}

// ---------------------------------------------------------------------------
// dequantization into MFMA operands
// ---------------------------------------------------------------------------

// Bytes u = c8 + 136 of 8 elements from their base and refinement dwords:
// `ev` holds elements 0, 2, 4, 6 (byte k = element 2k), `od` elements 1, 3, 5, 7.
__device__ __forceinline__ void nest_bytes(unsigned b, unsigned r, unsigned& ev, unsigned& od) {
  ev = ((b & 0x0F0F0F0Fu) << 4) | (r & 0x0F0F0F0Fu);
  od = (b & 0xF0F0F0F0u) | ((r >> 4) & 0x0F0F0F0Fu);
}

template <int K>
__device__ __forceinline__ float ubyte(unsigned w) {
  return (float)((w >> (8 * K)) & 0xFFu);  // v_cvt_f32_ubyte<K>
}

// bf16 pair (lo, hi) of two floats whose low 16 bits are zero.
__device__ __forceinline__ unsigned pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// K operand of 8 consecutive elements.
__device__ __forceinline__ bf16x8 nest_k_operand(unsigned b, unsigned r) {
  unsigned ev, od;
  nest_bytes(b, r, ev, od);
  unsigned w[4];
  w[0] = pack_bf16_exact(ubyte<0>(ev), ubyte<0>(od));
  w[1] = pack_bf16_exact(ubyte<1>(ev), ubyte<1>(od));
  w[2] = pack_bf16_exact(ubyte<2>(ev), ubyte<2>(od));
  w[3] = pack_bf16_exact(ubyte<3>(ev), ubyte<3>(od));
  bf16x8 out;
  __builtin_memcpy(&out, w, sizeof(out));
  return out;
}

// V operand of output column tile T: element T of each of the lane's 8 keys
// (ev / od: the key's composite bytes).
template <int T>
__device__ __forceinline__ bf16x8 nest_v_operand(const unsigned (&ev)[8], const unsigned (&od)[8]) {
  const unsigned(&src)[8] = (T & 1) ? od : ev;
  unsigned w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = pack_bf16_exact(ubyte<T / 2>(src[2 * j]), ubyte<T / 2>(src[2 * j + 1]));
  bf16x8 out;
  __builtin_memcpy(&out, w, sizeof(out));
  return out;
}

// ---------------------------------------------------------------------------
// verify attention over a nested cache (D = 128, bf16 queries)
// ---------------------------------------------------------------------------

// Codes of one 32-key stage held by one lane (c = lane % 16, q = lane / 16).
// K: key 16 kt + c, bytes [16 q, 16 q + 16) of its base / refinement row, i.e.
//    elements [32 q, 32 q + 32): MFMA chunk m takes elements 32 q + 8 m + (0..7)
//    (the queries use the same element order).
// V: keys pv_key(q, e), bytes [4 c, 4 c + 4): elements [8 c, 8 c + 8).
// Scales of keys pv_key(q, 0..3) and pv_key(q, 4..7).
struct NestStage {
  u32x4n kb[2], kr[2];
  unsigned vb[8], vr[8];
  float4 sk[2], sv[2];
};

struct NestedAttn {
  mtp_nested_kv kv;
  int kv8_recent;  // -1: all KV8; 0: all KV4; N: the N newest committed tokens in KV8
};

template <int RB>
__global__ __launch_bounds__(256) void attn_partial_nested(AttnParams p, NestedAttn na) {
  constexpr int D = 128;
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  constexpr int RowBytes = D / 2;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int qd = lane >> 4;
  const int b = blockIdx.y;
  const Item it = decode_item(blockIdx.x * 4 + (threadIdx.x >> 6), p);
  if (it.split >= p.max_splits) return;
  const int start = it.split * p.S;

  // loads that need no context length: the split's pages and Q
  const int32_t* btrow = p.block_table + (size_t)b * p.max_pages + start / kPage;
  const int pavail = p.max_pages - start / kPage;
  int pr0 = lane < pavail ? btrow[lane] : 0;
  int pr1 = lane + 64 < pavail ? btrow[lane + 64] : 0;
  bf16x8 qf[RB][NC];
  float nqs[RB];  // -136 * sum_d q_d of this lane's row
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    const int rho = (it.rb * RB + k) * 16 + c;
    float part = 0.f;
    if (rho < p.R) {
      const int w = rho / p.g;
      const int j = rho - w * p.g;
      const uint16_t* src = static_cast<const uint16_t*>(p.q) +
                            ((size_t)(b * p.W + w) * p.Hq + (size_t)it.kvh * p.g + j) * D + 32 * qd;
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        qf[k][m] = load_bf16x8(src + 8 * m);
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)qf[k][m][e];
      }
    } else {
#pragma unroll
      for (int m = 0; m < NC; ++m) qf[k][m] = bf16x8{};
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    nqs[k] = -kNestByteOffset * part;
  }

  const int L = p.ctx_lens[b];
  if (L < 0 || L > p.max_ctx) return;  // reported by the combine
  const int ns = num_splits(L, p.S);
  if (it.split >= ns) return;
  const int end = min(L, start + p.S);
  const bool last = it.split == ns - 1;
  const int npg = (end - start + kPage - 1) / kPage;
  bool bad = (lane < npg && (unsigned)pr0 >= (unsigned)p.num_pages) ||
             (lane + 64 < npg && (unsigned)pr1 >= (unsigned)p.num_pages);
  bad = __ballot(bad) != 0ull;
  if ((unsigned)pr0 >= (unsigned)p.num_pages) pr0 = 0;
  if ((unsigned)pr1 >= (unsigned)p.num_pages) pr1 = 0;
  // committed tokens at or past kv8_from are read in KV8
  const int kv8_from = na.kv8_recent < 0 ? 0 : max(0, L - na.kv8_recent);

  const int Hkv = p.Hkv;
  const uint8_t* kb = na.kv.k_base;
  const uint8_t* kr = na.kv.k_ref;
  const uint8_t* vb = na.kv.v_base;
  const uint8_t* vr = na.kv.v_ref;
  const float* ks = na.kv.k_scale;
  const float* vs = na.kv.v_scale;

  // Loads of stage s.  Keys past the committed range read slot 0 of the
  // stage's first page (always mapped) and are masked.
  auto load_stage = [&](int s, NestStage& st) {
    const int t0 = start + 32 * s;
    const int nk = end - t0;
    const int rp = 2 * s;
    const int p0 = __builtin_amdgcn_readlane(rp < 64 ? pr0 : pr1, rp & 63);
    const int p1 = nk > 16 ? __builtin_amdgcn_readlane(rp + 1 < 64 ? pr0 : pr1, (rp + 1) & 63) : p0;
    const bool any8 = min(t0 + 31, end - 1) >= kv8_from;  // a committed KV8 key in the stage
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = 16 * kt + c;
      const bool v = key < nk;
      const size_t row = nest_row(v ? (kt ? p1 : p0) : p0, it.kvh, v ? c : 0, Hkv);
      st.kb[kt] = *reinterpret_cast<const u32x4n*>(kb + row * RowBytes + 16 * qd);
      st.kr[kt] = any8 ? *reinterpret_cast<const u32x4n*>(kr + row * RowBytes + 16 * qd)
                       : u32x4n{kNestZeroRef, kNestZeroRef, kNestZeroRef, kNestZeroRef};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = pv_key(qd, e);
      const bool v = key < nk;
      const size_t row = nest_row(v ? (e < 4 ? p0 : p1) : p0, it.kvh, v ? (key & 15) : 0, Hkv);
      st.vb[e] = *reinterpret_cast<const unsigned*>(vb + row * RowBytes + 4 * c);
      st.vr[e] = any8 ? *reinterpret_cast<const unsigned*>(vr + row * RowBytes + 4 * c) : kNestZeroRef;
    }
    const size_t s0 = nest_row(p0, it.kvh, 4 * qd, Hkv);
    const size_t s1 = nest_row(p1, it.kvh, 4 * qd, Hkv);
    st.sk[0] = *reinterpret_cast<const float4*>(ks + s0);
    st.sk[1] = *reinterpret_cast<const float4*>(ks + s1);
    st.sv[0] = *reinterpret_cast<const float4*>(vs + s0);
    st.sv[1] = *reinterpret_cast<const float4*>(vs + s1);
  };

  MfmaState<D, RB> st;
  float lp[RB];  // this lane's share of sum_t p'_t
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    st.m[k] = neg_inf();
    st.l[k] = 0.f;
    lp[k] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int ncs = (end - start + 31) / 32;
  NestStage cur, nxt;
  if (ncs > 0) load_stage(0, cur);
  for (int s = 0; s < ncs; ++s) {
    if (s + 1 < ncs) load_stage(s + 1, nxt);
    const int t0 = start + 32 * s;
    const int nk = end - t0;
    // refinement of keys older than the KV8 window: code 0
    if (t0 < kv8_from && t0 + 31 >= kv8_from) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        if (t0 + 16 * kt + c < kv8_from)
          cur.kr[kt] = u32x4n{kNestZeroRef, kNestZeroRef, kNestZeroRef, kNestZeroRef};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (t0 + pv_key(qd, e) < kv8_from) cur.vr[e] = kNestZeroRef;
    }
    bf16x8 kf[2][NC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      kf[kt][0] = nest_k_operand(cur.kb[kt].x, cur.kr[kt].x);
      kf[kt][1] = nest_k_operand(cur.kb[kt].y, cur.kr[kt].y);
      kf[kt][2] = nest_k_operand(cur.kb[kt].z, cur.kr[kt].z);
      kf[kt][3] = nest_k_operand(cur.kb[kt].w, cur.kr[kt].w);
    }
    // the scales / 16 (exact) of the lane's 8 keys
    const float skv[8] = {cur.sk[0].x * 0.0625f, cur.sk[0].y * 0.0625f, cur.sk[0].z * 0.0625f,
                          cur.sk[0].w * 0.0625f, cur.sk[1].x * 0.0625f, cur.sk[1].y * 0.0625f,
                          cur.sk[1].z * 0.0625f, cur.sk[1].w * 0.0625f};
    const float svv[8] = {cur.sv[0].x * 0.0625f, cur.sv[0].y * 0.0625f, cur.sv[0].z * 0.0625f,
                          cur.sv[0].w * 0.0625f, cur.sv[1].x * 0.0625f, cur.sv[1].y * 0.0625f,
                          cur.sv[1].z * 0.0625f, cur.sv[1].w * 0.0625f};
    bool vis[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vis[e] = pv_key(qd, e) < nk;

    bf16x8 pf[RB], pl[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][m], qf[k][m], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][m], qf[k][m], s1, 0, 0, 0);
      }
      // q.k in units of the softmax input (before its scale): (s_k/16)(raw - 136 sum q)
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = skv[e] * (s0[e] + nqs[k]);
        x[4 + e] = skv[4 + e] * (s1[e] + nqs[k]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!vis[e]) x[e] = neg_inf();
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                       fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx *= p.scale_log2;
      const float mold = st.m[k];
      const float mref = mx > mold + kRescaleSlack ? mx : mold;
      const float muse = mref == neg_inf() ? 0.f : mref;
      float sum = 0.f, sump = 0.f;
      __bf16 ph[8], plo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = fast_exp2(fmaf(x[e], p.scale_log2, -muse));
        sum += pe;
        // masked keys may carry any scale (unwritten slots): select, never multiply
        const float pv = vis[e] ? pe * svv[e] : 0.f;
        sump += pv;
        ph[e] = (__bf16)pv;
        plo[e] = (__bf16)(pv - (float)ph[e]);
      }
      if (__ballot(mref != mold) != 0ull) {
        const float alpha = fast_exp2(mold - muse);
        st.l[k] *= alpha;
        lp[k] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) st.acc[k][t] *= alpha;
      }
      st.l[k] += sum;
      lp[k] += sump;
      st.m[k] = mref;
      __builtin_memcpy(&pf[k], ph, sizeof(bf16x8));
      __builtin_memcpy(&pl[k], plo, sizeof(bf16x8));
    }
    unsigned ev[8], od[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) nest_bytes(cur.vb[e], cur.vr[e], ev[e], od[e]);
#define MTPV_NEST_PV(T)                                                                  \
  {                                                                                      \
    const bf16x8 a = nest_v_operand<(T)>(ev, od);                                        \
    _Pragma("unroll") for (int k = 0; k < RB; ++k) {                                     \
      st.acc[k][(T)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[k], st.acc[k][(T)], 0, 0, 0); \
      st.acc[k][(T)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[k], st.acc[k][(T)], 0, 0, 0); \
    }                                                                                    \
  }
    MTPV_NEST_PV(0)
    MTPV_NEST_PV(1)
    MTPV_NEST_PV(2)
    MTPV_NEST_PV(3)
    MTPV_NEST_PV(4)
    MTPV_NEST_PV(5)
    MTPV_NEST_PV(6)
    MTPV_NEST_PV(7)
#undef MTPV_NEST_PV
    if (s + 1 < ncs) cur = nxt;
  }

  // remove the value offset: acc[row] -= 136 * sum_t p'_t (the row's full sum)
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    float lrow = lp[k];
    lrow += __shfl_xor(lrow, 16);
    lrow += __shfl_xor(lrow, 32);
    const float off = -kNestByteOffset * lrow;
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[k][t] += f32x4{off, off, off, off};
  }

  // in-block keys (the block's own bf16 K/V), masked per row, in the last split
  if (last) {
    bool ok;
    const uint64_t vnode =
        node_visibility(p.mask_kind[b], lane_mask_id(p, b, lane), p.W, p.lookback, lane, ok);
    if (ok) {
      uint64_t vrow[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int rho = min((it.rb * RB + k) * 16 + c, p.R - 1);
        vrow[k] = shfl64(vnode, rho / p.g);
      }
      const size_t slot_stride = (size_t)Hkv * D;
      const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + (size_t)it.kvh * D;
      const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + (size_t)it.kvh * D;
      for (int j0 = 0; j0 < p.W; j0 += 32) {
        bf16x8 kf[2][NC];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          int j = j0 + kt * 16 + c;
          j = j < p.W ? j : 0;
          const uint16_t* src = kn + (size_t)(b * p.W + j) * slot_stride + 32 * qd;
#pragma unroll
          for (int m = 0; m < NC; ++m) kf[kt][m] = load_bf16x8(src + 8 * m);
        }
        VRow<D> vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int j = j0 + pv_key(qd, e);
          j = j < p.W ? j : 0;
          vv[e] = load_vrow<D>(vn + (size_t)(b * p.W + j) * slot_stride + c * (D / 16));
        }
        mfma_tile<D, RB>(qf, kf, vv, p.scale_log2, st, [&](int k, int e) {
          return ((vrow[k] >> (j0 + pv_key(qd, e))) & 1ull) != 0ull;
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

#pragma unroll
  for (int k = 0; k < RB; ++k) {
    float l = st.l[k];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int rho = (it.rb * RB + k) * 16 + c;
    if (rho < p.R) {
      const size_t pidx =
          (((size_t)b * p.max_splits + it.split) * p.Hkv + it.kvh) * (size_t)p.R + rho;
      if (qd == 0) {
        p.part_ml[2 * pidx] = st.m[k];
        p.part_ml[2 * pidx + 1] = l;
      }
      float* dst = p.part_acc + pidx * D + qd * (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int t = 0; t < NT; t += 4) {
          float4 v;
          v.x = st.acc[k][t][e];
          v.y = st.acc[k][t + 1][e];
          v.z = st.acc[k][t + 2][e];
          v.w = st.acc[k][t + 3][e];
          *reinterpret_cast<float4*>(dst + e * (D / 16) + t) = v;
        }
      }
    }
  }
}

}  // namespace mtpv
