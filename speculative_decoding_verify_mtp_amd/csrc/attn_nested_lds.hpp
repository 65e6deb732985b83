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
// Every stage is transcoded once per workgroup into the sixteen bf16 operand
// images of the bf16 LDS kernel (images 0-7: K operands, 8-15: V vectors),
// holding u = c8 + 136 exactly (see nested.hpp); the waves then run the same
// MFMA step with the per-key scales applied to the scores and to P, and the
// offset removed at the end.  Operand images are double buffered: at
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
constexpr int kNestImgBytes = 16 * 1024;        // bf16 operand images of one stage

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

// Scores and softmax of one committed stage for the RB row tiles of a wave.
// skv / svv: the raw scales of the lane's keys pv_key(q, 0..7); sl2 = the
// softmax scale * log2(e) / 16 (so x * sl2 is the log2-domain score);
// P' = p * s_v (sixteen times p * s_v / 16: the 1/16 is applied with the
// offset at the end).  Keys past nk (the last stage of a split) are masked
// by selection and their V scales zeroed (a slot never written holds
// arbitrary scales; p = 0 must not meet a NaN).  One code path for full and partial stages: with a specialised
// copy for each, the compiler copied every accumulator register per stage.
template <int RB>
__device__ __forceinline__ void nest_scores(const bf16x8 (&qf)[RB][4], const bf16x8 (&kf)[2][4],
                                            const float (&skv)[8], float (&svv)[8],
                                            const float (&nqs)[RB], float sl2, int nk,
                                            MfmaState<128, RB>& st, float (&lp)[RB],
                                            bf16x8 (&pf)[RB], bf16x8 (&pl)[RB]) {
  const int qd = (threadIdx.x & 63) >> 4;
  float x[RB][8];
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][m], qf[k][m], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][m], qf[k][m], s1, 0, 0, 0);
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
    const float mx = mul_rn(rows4_max(max8(x[k])), sl2);
    const float mold = st.m[k];
    const float mref = mx > mold + kRescaleSlack ? mx : mold;
    const float muse = mref == neg_inf() ? 0.f : mref;
    float pe[8], pv[8];
    log2_weights(x[k], sl2, muse, 0.f, pe);
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
    lp[k] += sump;
    st.m[k] = mref;
    split_bf16_hi_lo(pv, pf[k], pl[k]);
  }
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
  __shared__ __attribute__((aligned(16))) char img[2 * kNestImgBytes];

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
  bf16x8 qf[RB][NC];
  float nqs[RB];  // -136 * sum_d q_d of this lane's row
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
    part = rows4_sum(part);
    nqs[k] = -kNestByteOffset * part;
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
  const float sl2 = p.scale_log2 * 0.0625f;  // the key scales enter as s, not s / 16
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
    char* out = img + (s & 1) * kNestImgBytes + 16 * lane;
    const int t0 = start + 32 * s;
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int im = wv + NR * k;
      unsigned w[4];
      if (im < 8) {
        // K operand (kt, m): key 16 kt + c, elements [32 m + 8 qd, +8) = part m, dword qd
        const int kt = im >> 2, m = im & 3;
        const int off = 16 * (16 * m + (c ^ m)) + 4 * qd;
        const unsigned bw = *reinterpret_cast<const unsigned*>(code + kt * 1024 + off);
        unsigned rw = *reinterpret_cast<const unsigned*>(code + 2048 + kt * 1024 + off);
        if (t0 + 16 * kt + c < kv8_from) rw = kNestZeroRef;
        unsigned ev, od;
        nest_bytes(bw, rw, ev, od);
        w[0] = pack_bf16_exact(ubyte<0>(ev), ubyte<0>(od));
        w[1] = pack_bf16_exact(ubyte<1>(ev), ubyte<1>(od));
        w[2] = pack_bf16_exact(ubyte<2>(ev), ubyte<2>(od));
        w[3] = pack_bf16_exact(ubyte<3>(ev), ubyte<3>(od));
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
        w[0] = pack_bf16_exact(ubyte<0>(ev), ubyte<0>(od));
        w[1] = pack_bf16_exact(ubyte<1>(ev), ubyte<1>(od));
        w[2] = pack_bf16_exact(ubyte<2>(ev), ubyte<2>(od));
        w[3] = pack_bf16_exact(ubyte<3>(ev), ubyte<3>(od));
      }
      *reinterpret_cast<uint4*>(out + im * 1024) = make_uint4(w[0], w[1], w[2], w[3]);
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

      const char* buf = img + (s & 1) * kNestImgBytes + lane * 16;
      const char* code = ring + (s % kNestRingStages) * kNestCodeBytes;
      bf16x8 kf[2][NC];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int m = 0; m < NC; ++m)
          kf[kt][m] = *reinterpret_cast<const bf16x8*>(buf + (kt * 4 + m) * 1024);
      uint4 vraw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vraw[e] = *reinterpret_cast<const uint4*>(buf + (8 + e) * 1024);
      // scales / 16 of the lane's keys pv_key(qd, 0..7)
      const float4 sk0 = *reinterpret_cast<const float4*>(code + 8192 + 16 * qd);
      const float4 sk1 = *reinterpret_cast<const float4*>(code + 8192 + 64 + 16 * qd);
      const float4 sv0 = *reinterpret_cast<const float4*>(code + 8192 + 128 + 16 * qd);
      const float4 sv1 = *reinterpret_cast<const float4*>(code + 8192 + 192 + 16 * qd);
      float skv[8] = {sk0.x, sk0.y, sk0.z, sk0.w, sk1.x, sk1.y, sk1.z, sk1.w};
      float svv[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};
      const int nk = end - (start + 32 * s);
      bf16x8 pf[RB], pl[RB];
      nest_scores<RB>(qf, kf, skv, svv, nqs, sl2, nk, st, lp, pf, pl);
      VRow<D> vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e].v = vraw[e];
      tile_pv<D, RB>(pf, pl, vv, st);
    }
  }

  // acc holds sum_t p_t s_t u_t: the committed part of the output row is
  // (acc - 136 sum_t p_t s_t) / 16
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    float lrow = lp[k];
    lrow = rows4_sum(lrow);
    const float off = -kNestByteOffset * 0.0625f * lrow;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st.acc[k][t][e] = fmaf(st.acc[k][t][e], 0.0625f, off);
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
      if (qd == 0 && rho < p.R) {
        p.part_ml[2 * (item_row + rho)] = st.m[k];
        p.part_ml[2 * (item_row + rho) + 1] = l;
      }
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
        *reinterpret_cast<float4*>(p.part_acc + (item_row + row0 + row) * D + col * 4) =
            *reinterpret_cast<const float4*>(sbuf + (size_t)row * kPitch + col * 4);
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
