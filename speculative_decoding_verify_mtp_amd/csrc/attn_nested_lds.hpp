// Verify attention over the nested KV4 / KV8 cache (D = 128), LDS ring.
//
// One workgroup = one work item (sequence, KV head, row block, split), NR
// waves of RB row tiles each, as in the bf16 LDS kernel.  The committed codes
// stream through a ring of stages (32 keys each) by direct-to-LDS loads:
//   8 code images of 1 KB: K base, K ref, V base, V ref, each for keys 0-15
//   and 16-31 of the stage.  Image lane l holds the 16 bytes of key
//   (l % 16) ^ (l / 16), part l / 16 (bytes [16 part, +16) of its 64-byte row):
//   the XOR spreads the reads of the transcode over the LDS banks.
//   1 scale image of 256 bytes: K scales of the 32 keys, then V scales.
// Every stage is transcoded once per workgroup into operand images: the
// byte u = c8 + 136 of an element (nested.hpp) taken as the bf16 bit pattern
// 0x00uu, which is u 2^-133 exactly for every u in [0, 255] (below 128 a
// subnormal, from 128 the first normal binade, with the same spacing; gfx950's
// bf16 MFMA takes both exactly).  K images (0-7, the operand layout of the bf16
// LDS kernel) are four byte permutes per 8 elements; V images (8-15) keep the
// bytes themselves, 8 per lane, and the PV step spreads them into bf16 pairs
// with the permutes that pair its keys anyway.  The products stay in the
// normal fp32 range because Q enters scaled by 2^e per row (nest_scale_q) and
// P by 2^kNestPBias; the waves run the MFMA step of the bf16 kernel with the
// per-key scales applied to the scores and to P, and the offset and both
// powers of two removed at the end.  Operand images are double buffered: at
// iteration s one barrier proves that stage s + 1's codes have landed, that
// the operands of stage s are complete and that nobody reads the other
// operand buffer any more; then stage s + 1 is transcoded while stage s is
// computed.
//
// KV4 keys (older than the Recent-N window, or all with kv8_recent = 0) take
// the refinement code 0; their refinement images are loaded from the base
// plane instead (the same lines, so no extra HBM traffic) to keep the number
// of loads per stage fixed.
#pragma once

#include "attn_lds.hpp"
#include "attn_mfma.hpp"
#include "common.hpp"
#include "nested.hpp"

namespace mtpv {

constexpr int kNestRingStages = 5;
// Code stages in flight ahead of the one being transcoded (as in the bf16
// kernels, short memory queues pay: ragged batch KV8 955 -> 922 us with 2
// instead of 4, llama3_8b_tree 23.5 -> 23.2 us; 3 changed nothing).
constexpr int kNestAhead = 2;
static_assert(kNestAhead >= 1 && kNestAhead <= kNestRingStages - 1, "ring slots refilled after their last read");
constexpr int kNestCodeBytes = 8 * 1024 + 256;  // 8 code images + scales

// 4 bytes from global `g` into LDS at m0 + 4 * lane, m0 = lds (wave-uniform).
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(base)
      : "memory");
}

// Waits until at most N vector-memory operations of this wave are
// outstanding and its LDS writes are done, then joins the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vmem_lds_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int PER>
__device__ __forceinline__ void wait_code_stage_barrier(int n) {
  if (n <= 0)
    wait_vmem_lds_barrier<0>();
  else if (n == 1)
    wait_vmem_lds_barrier<PER>();
  else if (n == 2)
    wait_vmem_lds_barrier<2 * PER>();
  else
    wait_vmem_lds_barrier<3 * PER>();
}

// One stage's operand images: 8 K images of 1 KB (bf16 bit patterns 0x00uu),
// then 8 V byte images of 512 bytes.
constexpr int kNestImgBytesU = 8 * 1024 + 8 * 512;
constexpr float kNestPBias = 60.f;  // log2 of the scale of P in the committed stages

// K operand image dword k (elements 2k, 2k + 1) from the bytes u of the even
// (ev) and odd (od) elements: bf16 bit patterns 0x00uu.
__device__ __forceinline__ uint4 nest_k_operand(unsigned ev, unsigned od) {
  return make_uint4(__builtin_amdgcn_perm(od, ev, 0x0c040c00u), __builtin_amdgcn_perm(od, ev, 0x0c050c01u),
                    __builtin_amdgcn_perm(od, ev, 0x0c060c02u), __builtin_amdgcn_perm(od, ev, 0x0c070c03u));
}

// Scores and softmax of one committed stage for the RB row tiles of a wave.
// qs: the row tiles' scaled Q operands (nest_scale_q); kf: the K operand
// images (bit patterns 0x00uu); skv / svv: the raw scales of the lane's keys
// pv_key(q, 0..7); sl2r: the row's log2-domain scale (softmax scale * log2(e)
// / 16, times the 2^(133 - e) of its Q scaling).  P' = 2^kNestPBias p s_v
// goes to the PV product as bf16 hi + lo; the row sum carries the same
// 2^kNestPBias, lp = sum_t p_t s_t is kept in real units.  Keys past nk (the
// last stage of a split or range) are masked by selection and their V scales
// zeroed (a slot never written holds arbitrary scales; p = 0 must not meet a
// NaN).  One code path for full and partial stages.
template <int RB>
__device__ __forceinline__ void nest_scores_u(const bf16x8 (&qs)[RB][4], const bf16x8 (&kf)[2][4],
                                              const float (&skv)[8], float (&svv)[8],
                                              const float (&nqs)[RB], const float (&sl2r)[RB], int nk,
                                              MfmaState<128, RB>& st, float (&lp)[RB],
                                              bf16x8 (&pf)[RB], bf16x8 (&pl)[RB]) {
  const int qd = (threadIdx.x & 63) >> 4;
  float x[RB][8];
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][m], qs[k][m], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][m], qs[k][m], s1, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[k][e] = skv[e] * (s0[e] + nqs[k]);
      x[k][4 + e] = skv[4 + e] * (s1[e] + nqs[k]);
    }
  }
  if (nk < 32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (pv_key(qd, e) >= nk) {
        svv[e] = 0.f;
#pragma unroll
        for (int k = 0; k < RB; ++k) x[k][e] = neg_inf();
      }
    }
  }
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    const float mx = mul_rn(rows4_maximum(max8(x[k])), sl2r[k]);
    const float mold = st.m[k];
    const float mref = mx > mold + kRescaleSlack ? mx : mold;
    const float muse = mref == neg_inf() ? 0.f : mref;
    float pe[8], pv[8];
    log2_weights(x[k], sl2r[k], muse, kNestPBias, pe);
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = pe[e] * svv[e];
    const float sum = ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
    const float sump = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    if (__ballot(mref != mold) != 0ull) {
      const float alpha = fast_exp2(mold - muse);
      st.l[k] *= alpha;
      lp[k] *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) st.acc[k][t] *= alpha;
    }
    st.l[k] += sum;
    lp[k] = fmaf(sump, 0x1p-60f, lp[k]);  // in real units: lp stays far from overflow
    st.m[k] = mref;
    split_bf16_hi_lo(pv, pf[k], pl[k]);
  }
}

// PV accumulate of one committed stage from the V byte vectors (vb[e]: bytes
// u of d = 8c + 0, 2, 4, 6 in .x and 8c + 1, 3, 5, 7 in .y, key pv_key(q, e)):
// operand t pairs element t of keys 2j and 2j + 1 as bf16 bit patterns 0x00uu.
template <int RB>
__device__ __forceinline__ void tile_pv_u(const bf16x8 (&pf)[RB], const bf16x8 (&pl)[RB],
                                          const uint2 (&vb)[8], MfmaState<128, RB>& st) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const unsigned sel = 0x0c040c00u + (unsigned)(t >> 1) * 0x00010001u;
    unsigned w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned x = (t & 1) ? vb[2 * j].y : vb[2 * j].x;
      const unsigned y = (t & 1) ? vb[2 * j + 1].y : vb[2 * j + 1].x;
      w[j] = __builtin_amdgcn_perm(y, x, sel);
    }
    bf16x8 a;
    __builtin_memcpy(&a, w, sizeof(a));
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      st.acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[k], st.acc[k][t], 0, 0, 0);
      st.acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[k], st.acc[k][t], 0, 0, 0);
    }
  }
}

// Committed-stage Q operands of one row tile: Q 2^e (exact), e putting the
// row's largest |q| in [2^120, 2^121), so that the products with the operand
// bit patterns 0x00uu = u 2^-133 stay in the normal fp32 range; the factor
// 2^(133 - e) moves into the row's softmax scale (sl2r) and into the offset
// term nqs = -136 sum_d q_d 2^(e - 133).  qsum: this lane's share of
// sum_d q_d.
__device__ __forceinline__ void nest_scale_q(const bf16x8 (&qf)[4], float qsum, float sl2,
                                             bf16x8 (&qs)[4], float& nqs, float& sl2r) {
  float amax = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qf[m][e]));
  amax = rows4_max(amax);
  const int ex = amax > 0.f ? 121 - __builtin_amdgcn_frexp_expf(amax) : 120;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[m][e] = (__bf16)ldexpf((float)qf[m][e], ex);
  nqs = ldexpf(-kNestByteOffset * rows4_sum(qsum), ex - 133);
  sl2r = ldexpf(sl2, 133 - ex);
}

template <int RB, int NR>
__global__ __launch_bounds__(64 * NR) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 2 : 1)))
void attn_partial_nested_lds(AttnParams p, NestedAttn na) {
  constexpr int D = 128;
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  constexpr int CPW = 8 / NR;        // code images per wave per stage
  constexpr int PER = CPW + 1;       // loads per wave per stage (codes + scales)
  constexpr int IPW = 16 / NR;       // operand images transcoded per wave
  constexpr int SL = kWave / NR;     // scale lanes per wave
  __shared__ __attribute__((aligned(16))) char ring[kNestRingStages * kNestCodeBytes];
  __shared__ __attribute__((aligned(16))) char img[2 * kNestImgBytesU];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int qd = lane >> 4;
  const int b = blockIdx.y;
  const Item it = decode_item_xcd(blockIdx.x, gridDim.x, p);
  if (it.split >= p.max_splits) return;  // uniform over the workgroup
  const int start = split_start(p, it.split);

  const int32_t* btrow = p.block_table + (size_t)b * p.max_pages + start / kPage;
  const int pavail = p.max_pages - start / kPage;
  int pr0 = lane < pavail ? btrow[lane] : 0;
  int pr1 = lane + 64 < pavail ? btrow[lane + 64] : 0;
  const int row_tile0 = (it.rb * NR + wv) * RB;
  bf16x8 qf[RB][NC];  // Q operands (in-block keys)
  bf16x8 qs[RB][NC];  // Q 2^e (committed keys)
  float nqs[RB];      // -136 sum_d q_d of this lane's row, times 2^(e - 133)
  float sl2r[RB];     // the row's log2-domain scale for the committed keys
  const float sl2 = p.scale_log2 * 0.0625f;  // the key scales enter as s, not s / 16
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    const int rho = (row_tile0 + k) * 16 + c;
    float part = 0.f;
    if (rho < p.R) {
      const int w = rho / p.g;
      const int j = rho - w * p.g;
      const uint16_t* src = static_cast<const uint16_t*>(p.q) +
                            ((size_t)(b * p.W + w) * p.Hq + (size_t)it.kvh * p.g + j) * D + qd * 8;
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        qf[k][m] = load_bf16x8(src + m * 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)qf[k][m][e];
      }
    } else {
#pragma unroll
      for (int m = 0; m < NC; ++m) qf[k][m] = bf16x8{};
    }
    nest_scale_q(qf[k], part, sl2, qs[k], nqs[k], sl2r[k]);
  }

  // the mask description goes out with the set-up loads: the last split
  // needs it, and waiting for it after the context length would add a round
  // trip before the first stage is issued
  const int mkind = p.mask_kind[b];
  const int mid = lane_mask_id(p, b, lane);
  const int L = p.ctx_lens[b];
  if (L < 0 || L > p.max_ctx) return;
  const int ns = num_splits(p, L);
  if (it.split >= ns) return;
  const int end = min(L, split_start(p, it.split + 1));
  const bool last = it.split == ns - 1;
  const int npg = (end - start + kPage - 1) / kPage;
  bool bad = (lane < npg && (unsigned)pr0 >= (unsigned)p.num_pages) ||
             (lane + 64 < npg && (unsigned)pr1 >= (unsigned)p.num_pages);
  bad = __ballot(bad) != 0ull;
  if ((unsigned)pr0 >= (unsigned)p.num_pages) pr0 = 0;
  if ((unsigned)pr1 >= (unsigned)p.num_pages) pr1 = 0;
  const int kv8_from = na.kv8_recent < 0 ? 0 : max(0, L - na.kv8_recent);
  const int ncs = (end - start + 31) / 32;
  __builtin_amdgcn_s_waitcnt(0);

  // ---- code stage issue: this wave's code images and its share of the scales
  const uint32_t ring_base = lds_offset(ring);
  const int Hkv = p.Hkv;
  // image lane l <- key (l % 16) ^ (l / 16), part l / 16
  const int dkey = c ^ qd;
  const uint32_t doff = 64u * dkey + 16u * qd;
  // plane bases of the four code kinds: K base, K ref, V base, V ref
  const uint8_t* kbase = na.kv.k_base;
  const uint8_t* vbase = na.kv.v_base;
  const uint8_t* kref = na.kv.k_ref != nullptr ? na.kv.k_ref : na.kv.k_base;
  const uint8_t* vref = na.kv.v_ref != nullptr ? na.kv.v_ref : na.kv.v_base;
  auto issue = [&](int s) __attribute__((always_inline)) {
    const uint32_t slot = ring_base + (uint32_t)(s % kNestRingStages) * kNestCodeBytes;
    const int t0 = start + 32 * s;
    const int nk = end - t0;
    const int rp = 2 * s;
    const int p0 = __builtin_amdgcn_readlane(rp < 64 ? pr0 : pr1, rp & 63);
    const int p1 = nk > 16 ? __builtin_amdgcn_readlane(rp + 1 < 64 ? pr0 : pr1, (rp + 1) & 63) : p0;
    // refinement planes only when a committed key of the stage is read in KV8
    const bool any8 = min(t0 + 31, end - 1) >= kv8_from;
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
      const int im = wv + NR * k;  // 0..7: kind = im / 2, half = im % 2
      const int kind = im >> 1, half = im & 1;
      // two selects (a four-way choice would become a table in scratch memory)
      const uint8_t* b2 = (kind & 2) ? vbase : kbase;
      const uint8_t* r2 = (kind & 2) ? vref : kref;
      const uint8_t* plane = ((kind & 1) && any8) ? r2 : b2;
      const int pg = half ? p1 : p0;
      if (nk >= 32) {
        const uint64_t base = (uint64_t)(uintptr_t)plane + (((uint64_t)pg * Hkv + it.kvh) << 10);
        dma16_sbase(doff, base, slot + (uint32_t)im * 1024u);
      } else {
        const int key = 16 * half + dkey;
        const bool v = key < nk;
        const size_t row = nest_row(v ? pg : p0, it.kvh, v ? dkey : 0, Hkv);
        dma16(plane + row * 64 + 16 * qd, slot + (uint32_t)im * 1024u);
      }
    }
    // scales: wave w loads entries [w * SL, (w + 1) * SL) of the 64 (K keys 0-31, V keys 0-31)
    if (lane < SL) {
      const int g = wv * SL + lane;
      const int key = g & 31;
      const bool v = key < nk;
      const size_t row = nest_row(v ? (key < 16 ? p0 : p1) : p0, it.kvh, v ? (key & 15) : 0, Hkv);
      dma4((g < 32 ? na.kv.k_scale : na.kv.v_scale) + row, slot + 8192u + 4u * (uint32_t)(wv * SL));
    }
  };

  // ---- transcode stage s: this wave's operand images into buffer s % 2
  auto transcode = [&](int s) __attribute__((always_inline)) {
    const char* code = ring + (s % kNestRingStages) * kNestCodeBytes;
    char* out = img + (s & 1) * kNestImgBytesU;
    const int t0 = start + 32 * s;
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int im = wv + NR * k;
      if (im < 8) {
        // K operand (kt, m): key 16 kt + c, elements [32 m + 8 qd, +8) = part m, dword qd
        const int kt = im >> 2, m = im & 3;
        const int off = 16 * (16 * m + (c ^ m)) + 4 * qd;
        const unsigned bw = *reinterpret_cast<const unsigned*>(code + kt * 1024 + off);
        unsigned rw = *reinterpret_cast<const unsigned*>(code + 2048 + kt * 1024 + off);
        if (t0 + 16 * kt + c < kv8_from) rw = kNestZeroRef;
        unsigned ev, od;
        nest_bytes(bw, rw, ev, od);
        *reinterpret_cast<uint4*>(out + im * 1024 + 16 * lane) = nest_k_operand(ev, od);
      } else {
        // V vector e: key pv_key(qd, e), elements [8 c, +8) = part c / 4, dword c % 4
        const int e = im - 8;
        const int half = e >> 2;
        const int k16 = 4 * qd + (e & 3);
        const int part = c >> 2;
        const int off = 16 * (16 * part + (k16 ^ part)) + 4 * (c & 3);
        const unsigned bw = *reinterpret_cast<const unsigned*>(code + 4096 + half * 1024 + off);
        unsigned rw = *reinterpret_cast<const unsigned*>(code + 6144 + half * 1024 + off);
        if (t0 + 16 * half + k16 < kv8_from) rw = kNestZeroRef;
        unsigned ev, od;
        nest_bytes(bw, rw, ev, od);
        *reinterpret_cast<uint2*>(out + 8192 + (im - 8) * 512 + 8 * lane) = make_uint2(ev, od);
      }
    }
  };

  MfmaState<D, RB> st;
  float lp[RB];
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    st.m[k] = neg_inf();
    st.l[k] = 0.f;
    lp[k] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The ring keeps kNestAhead <= kNestRingStages - 1 stages ahead: the slot
  // refilled in iteration s (stage s + kNestAhead) last held stage
  // s + kNestAhead - kNestRingStages <= s - 1 (codes transcoded in iteration
  // s - 2, scales read in iteration s - 1), whose reads the barrier of
  // iteration s has ended.
  if (ncs > 0) {
    constexpr int kAhead = kNestAhead;
    for (int s = 0; s < kAhead && s < ncs; ++s) issue(s);
    // stage 0 landed (every later issued stage may still be in flight)
    wait_code_stage_barrier<PER>(min(kAhead, ncs) - 1);
    transcode(0);
    for (int s = 0; s < ncs; ++s) {
      // stage s + 1 landed, operands of s complete, the other buffer free
      const int issued = min(s + kAhead, ncs);  // stages 0 .. issued-1 issued
      wait_code_stage_barrier<PER>(max(0, issued - (s + 2)));
      if (s + kAhead < ncs) issue(s + kAhead);
      if (s + 1 < ncs) transcode(s + 1);

      const char* buf = img + (s & 1) * kNestImgBytesU + lane * 16;
      const char* vbuf = img + (s & 1) * kNestImgBytesU + 8192 + lane * 8;
      const char* code = ring + (s % kNestRingStages) * kNestCodeBytes;
      bf16x8 kf[2][NC];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int m = 0; m < NC; ++m)
          kf[kt][m] = *reinterpret_cast<const bf16x8*>(buf + (kt * 4 + m) * 1024);
      uint2 vb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vb[e] = *reinterpret_cast<const uint2*>(vbuf + e * 512);
      // scales / 16 of the lane's keys pv_key(qd, 0..7)
      const float4 sk0 = *reinterpret_cast<const float4*>(code + 8192 + 16 * qd);
      const float4 sk1 = *reinterpret_cast<const float4*>(code + 8192 + 64 + 16 * qd);
      const float4 sv0 = *reinterpret_cast<const float4*>(code + 8192 + 128 + 16 * qd);
      const float4 sv1 = *reinterpret_cast<const float4*>(code + 8192 + 192 + 16 * qd);
      float skv[8] = {sk0.x, sk0.y, sk0.z, sk0.w, sk1.x, sk1.y, sk1.z, sk1.w};
      float svv[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};
      const int nk = end - (start + 32 * s);
      bf16x8 pf[RB], pl[RB];
      nest_scores_u<RB>(qs, kf, skv, svv, nqs, sl2r, nk, st, lp, pf, pl);
      tile_pv_u<RB>(pf, pl, vb, st);
    }
  }

  // acc holds 2^-73 sum_t p_t s_t u_t and the row sum 2^60 sum_t p_t: the
  // committed part of the output row is (2^73 acc - 136 sum_t p_t s_t) / 16
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    const float off = -kNestByteOffset * 0.0625f * rows4_sum(lp[k]);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st.acc[k][t][e] = fmaf(st.acc[k][t][e], 0x1p69f, off);
    st.l[k] *= 0x1p-60f;
  }

  // in-block keys (bf16), masked per row, in the last split: direct loads
  if (last) {
    bool ok;
    const uint64_t vnode =
        node_visibility(mkind, mid, p.W, p.lookback, lane, ok);
    if (ok) {
      uint64_t vrow[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int rho = min((row_tile0 + k) * 16 + c, p.R - 1);
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
          const uint16_t* src = kn + (size_t)(b * p.W + j) * slot_stride + qd * 8;
#pragma unroll
          for (int m = 0; m < NC; ++m) kf[kt][m] = load_bf16x8(src + m * 32);
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
    if (threadIdx.x == 0) raise_status(MTP_DEV_BAD_PAGE);
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      st.m[k] = qnan();
#pragma unroll
      for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{qnan(), qnan(), qnan(), qnan()};
    }
  }

  const size_t item_row = (((size_t)b * p.max_splits + it.split) * p.Hkv + it.kvh) * (size_t)p.R;
  constexpr int kPitch = D + 4;  // padded rows: the 16 rows a write spans fall in different banks
  if constexpr (NR * RB * 16 * kPitch * 4 <= kNestRingStages * kNestCodeBytes) {
    // Rows staged row-major in the code ring, then stored as whole rows (1 KB
    // per store instruction) by every wave.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // nobody reads the ring any more
    float* sbuf = reinterpret_cast<float*>(ring);
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const float l = rows4_sum(st.l[k]);
      const int rho = (row_tile0 + k) * 16 + c;
      if (qd == 0 && rho < p.R) store_partial_ml(p.part_ml + 2 * item_row, 2 * rho, st.m[k], l);
      float* rowp = sbuf + (size_t)((wv * RB + k) * 16 + c) * kPitch + qd * (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < NT; t += 4)
          *reinterpret_cast<float4*>(rowp + e * (D / 16) + t) =
              make_float4(st.acc[k][t][e], st.acc[k][t + 1][e], st.acc[k][t + 2][e], st.acc[k][t + 3][e]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int row0 = it.rb * NR * RB * 16;  // first row of this workgroup's row block
    constexpr int kVecs = NR * RB * 16 * (D / 4);
#pragma unroll 4
    for (int f = threadIdx.x; f < kVecs; f += 64 * NR) {
      const int row = f / (D / 4);
      const int col = f - row * (D / 4);
      if (row0 + row < p.R)
        store_partial4(p.part_acc + item_row * D, (row0 + row) * D + col * 4,
                       *reinterpret_cast<const float4*>(sbuf + (size_t)row * kPitch + col * 4));
    }
  } else {
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      float l = st.l[k];
      l = rows4_sum(l);
      const int rho = (row_tile0 + k) * 16 + c;
      if (rho < p.R) {
        const size_t pidx = item_row + rho;
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
}

}  // namespace mtpv
