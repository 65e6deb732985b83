// Split-K verify attention, D = 128, bf16 MFMA, K/V streamed through an LDS
// ring by direct-to-LDS loads (global_load_lds_dwordx4).
//
// One workgroup = one work item (sequence, KV head, row block, split).  Its
// NR waves (1, 2 or 4) split the rows: wave w owns RB row tiles of 16 rows.
// All waves consume the same K/V, so the committed context is read from HBM
// once per row block and shared through LDS.
//
// A stage is 32 keys (two pages) = 16 KB, stored as sixteen 1 KB "register
// images": image i holds, at byte 16 * lane, exactly the 16 bytes that lane
// needs as an MFMA operand (the layouts of attn_mfma.hpp):
//   images 0..7  : K operand of 16-key half kt = i / 4, d-chunk m = i % 4:
//                  lane (c, q) <- K[key 16 kt + c][32 m + 8 q .. +8)
//   images 8..15 : V vectors e = i - 8: lane (c, q) <- V[pv_key(q, e)][8 c .. +8)
// The direct-to-LDS load writes lane l's 16 bytes to M0 + 16 l, so a stage is
// sixteen such loads (16 / NR per wave) and every later LDS read is one
// conflict-free 16-byte read per lane.
//
// The ring holds kStages stages; kStages - 1 are in flight while one is being
// computed.  Each wave waits for its own loads of stage s (s_waitcnt vmcnt
// with an explicit count), then a workgroup barrier makes everybody's loads
// visible and also proves that stage s - 1 is no longer read, so its slot
// takes stage s + kStages - 1.  The loads are issued through inline assembly:
// the compiler would otherwise guard every LDS read with a full vmcnt(0) wait
// and serialise the pipeline.
#pragma once

#include "accept_commit.hpp"
#include "attn_mfma.hpp"
#include "common.hpp"

namespace mtpv {

constexpr int kLdsStages = 5;  // 80 KB per workgroup: two workgroups fill gfx950's 160 KB
// Stages in flight ahead of the one being reduced when a split streams
// through the ring.  Fewer outstanding stages per workgroup keep the memory
// queues short, so every workgroup's next stage arrives sooner: llama3_8b_tree
// 18.5-19.0 -> 17.1-17.8 us with 2 instead of 4 (3: 17.8-18.2 us, 1:
// 17.4 us); 4 sequences of 16000 tokens 67.0 -> 64.6 us; 2 of 30000 with
// W = 32 95.4 -> 90.8 us.
constexpr int kLdsAhead = 2;
static_assert(kLdsAhead >= 1 && kLdsAhead <= kLdsStages - 1, "ring slots refilled after their last read");
constexpr int kStageBytes = 16 * 1024;
constexpr int kMaxSplitPages = 128;  // page indices of a split held in two registers per lane

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16 bytes from global `g` into LDS at m0 + 16 * lane, m0 = lds (wave-uniform).
// m0 is saved and restored around the load.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(base)
      : "memory");
}

// Same, addressed as a wave-uniform 64-bit base (SGPRs) plus a per-lane 32-bit
// byte offset: the form used for whole stages, whose per-lane offsets are
// fixed for the whole item.
__device__ __forceinline__ void dma16_sbase(uint32_t voff, uint64_t sbase, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sbase);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(m0v)
      : "memory");
}

// Waits until at most N vector-memory operations of this wave are
// outstanding, then joins the workgroup barrier.  One asm statement with a
// memory clobber, so no LDS read can be scheduled above the barrier.
template <int N>
__device__ __forceinline__ void wait_vmem_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait for this wave's loads of a stage when n later stages (PER loads each)
// may stay in flight, then barrier.
template <int PER>
__device__ __forceinline__ void wait_stage_barrier(int n) {
  // covers up to three later stages (rings of at most five stages)
  if (n <= 0)
    wait_vmem_barrier<0>();
  else if (n == 1)
    wait_vmem_barrier<PER>();
  else if (n == 2)
    wait_vmem_barrier<2 * PER>();
  else
    wait_vmem_barrier<3 * PER>();
}

// Merge of a key slice's softmax state into slice 0's, lane by lane (the
// slices hold the same rows in the same lanes).  Stored per lane as 32
// accumulators, the reference max and the lane's share of the row sum.
constexpr int kSliceStateFloats = 34;

// RB = 1 kernels are held to 256 registers so that two waves share a SIMD.
// KS > 1 (key slices): the workgroup has NR * KS waves; wave (g, k) owns the
// row tiles of group g and the stages k, k + KS, ... of the item, and the KS
// softmax states of a row tile are merged through LDS at the end.  A split
// whose stages all fit the ring is then one wait and one barrier, and each
// wave reduces 1 / KS of its stages: for short splits (a single sequence,
// latency-bound) the per-stage compute chain is the critical path.
template <int RB, int NR, int KS = 1>
__global__ __launch_bounds__(64 * NR * KS) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 2 : 1)))
void attn_partial_lds(AttnParams p) {
  constexpr int D = 128;
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  constexpr int NW = NR * KS;   // waves
  constexpr int IPW = 16 / NW;  // images per wave per stage
  static_assert(KS == 1 || RB == 1, "key slices are used with one row tile per wave");
  static_assert(KS == 1 || NW * RB * kSliceStateFloats * 4 * kWave <= kLdsStages * kStageBytes,
                "slice states must fit the ring");
  __shared__ __attribute__((aligned(16))) char ring[kLdsStages * kStageBytes];

  const int lane = threadIdx.x & 63;
  // wave-uniform, so the issue path computes page addresses in scalar registers
  // (bitnet2b_chain partial 9.18 -> 9.01 us, llama3_8b_tree 19.9 -> 19.7 us;
  // the stream kernel measured 925 -> 934 us with the same change and keeps
  // the vector form)
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0 .. NW - 1
  const int tg = wv % NR;           // row-tile group
  const int ks = wv / NR;           // key slice
  const int c = lane & 15;
  const int qd = lane >> 4;
  const int b = blockIdx.y;
  const Item it = decode_item_xcd(blockIdx.x, gridDim.x, p);
  if (it.split >= p.max_splits) return;  // uniform over the workgroup
  const int start = split_start(p, it.split);

  // Loads that do not depend on the context length go out together with it:
  // the split's page indices (bounded by the block table) and Q.
  const int32_t* btrow = p.block_table + (size_t)b * p.max_pages + start / kPage;
  const int pavail = p.max_pages - start / kPage;
  int pr0 = lane < pavail ? btrow[lane] : 0;
  int pr1 = lane + 64 < pavail ? btrow[lane + 64] : 0;
  const int row_tile0 = (it.rb * NR + tg) * RB;
  bf16x8 qf[RB][NC];
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    const int rho = (row_tile0 + k) * 16 + c;
    if (rho < p.R) {
      const int w = rho / p.g;
      const int j = rho - w * p.g;
      const uint16_t* src = static_cast<const uint16_t*>(p.q) +
                            ((size_t)(b * p.W + w) * p.Hq + (size_t)it.kvh * p.g + j) * D + qd * 8;
#pragma unroll
      for (int m = 0; m < NC; ++m) qf[k][m] = load_bf16x8(src + m * 32);
    } else {
#pragma unroll
      for (int m = 0; m < NC; ++m) qf[k][m] = bf16x8{};
    }
  }

  // the mask description goes out with the set-up loads: the last split
  // needs it, and waiting for it after the context length would add a round
  // trip before the first stage is issued
  const int mkind = p.mask_kind[b];
  const int mid = lane_mask_id(p, b, lane);
  // the step's target prologue: wave 0 of workgroup j < B * W finds the
  // argmax of logits row j, its loads in the same round trip as the set-up
  // (the host enables it for V <= kRegV, V % 4 == 0, 16-byte aligned rows;
  // the reduction is the acceptance's own, so the targets are the same)
  const int L = p.ctx_lens[b];  // requested before the prologue waits for its row
  const int flat = (int)(blockIdx.y * gridDim.x + blockIdx.x);
  if (p.logits != nullptr && flat < p.B * p.W && wv == 0) {
    RegRow rr;
    load_reg_row(p.logits + (size_t)flat * p.V, p.V, rr);
    const int t = reg_row_argmax(rr, p.V);
    if (lane == 0) p.tgt[flat] = t;
  }
  if (L < 0 || L > p.max_ctx) return;
  const int ns = num_splits(p, L);
  if (it.split >= ns) return;
  const int end = min(L, split_start(p, it.split + 1));
  const bool last = it.split == ns - 1;

  const uint16_t* kc = static_cast<const uint16_t*>(p.k_cache) + (size_t)it.kvh * D;
  const uint16_t* vc = static_cast<const uint16_t*>(p.v_cache) + (size_t)it.kvh * D;
  const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + (size_t)it.kvh * D;
  const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + (size_t)it.kvh * D;
  const size_t slot_stride = (size_t)p.Hkv * D;

  // ---- page indices of the committed range: validate, clamp
  const int npg = (end - start + kPage - 1) / kPage;
  bool bad = (lane < npg && (unsigned)pr0 >= (unsigned)p.num_pages) ||
             (lane + 64 < npg && (unsigned)pr1 >= (unsigned)p.num_pages);
  bad = __ballot(bad) != 0ull;
  if ((unsigned)pr0 >= (unsigned)p.num_pages) pr0 = 0;
  if ((unsigned)pr1 >= (unsigned)p.num_pages) pr1 = 0;

  int ntail = 0;
  uint64_t vrow[RB];
#pragma unroll
  for (int k = 0; k < RB; ++k) vrow[k] = 0;
  if (last) {
    bool ok;
    const uint64_t vnode =
        node_visibility(mkind, mid, p.W, p.lookback, lane, ok);
    if (ok) {
      ntail = (p.W + 31) / 32;
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const int rho = min((row_tile0 + k) * 16 + c, p.R - 1);
        vrow[k] = shfl64(vnode, rho / p.g);
      }
    }
  }
  const int ncs = (end - start + 31) / 32;  // committed stages
  const int nst = ncs + ntail;
  // The set-up loads are complete before the first stage is issued (a wait the
  // compiler sees, so it adds none of its own inside the pipeline).
  __builtin_amdgcn_s_waitcnt(0);

  // ---- stage issue: this wave's images of stage s into ring slot s % kStages
  // Per-lane byte offsets inside a page for whole stages: a K image (kt, m)
  // is koff + 64 m, a V image e is voff + (e & 3) * slot_bytes; the page (p0 or
  // p1) goes into the wave-uniform base.
  const uint32_t ring_base = lds_offset(ring);
  const uint32_t slot_bytes = (uint32_t)(slot_stride * 2);
  const uint64_t page_bytes = (uint64_t)kPage * slot_bytes;
  const uint32_t koff = (uint32_t)c * slot_bytes + 16u * qd;
  const uint32_t voff = 4u * qd * slot_bytes + 16u * c;
  const uint64_t kc_addr = (uint64_t)(uintptr_t)kc, vc_addr = (uint64_t)(uintptr_t)vc;
  auto issue = [&](int s) {
    const uint32_t slot_base = ring_base + (uint32_t)(s % kLdsStages) * kStageBytes;
    if (s < ncs) {
      const int t0 = start + 32 * s;
      const int nk = end - t0;
      const int rp = 2 * s;  // page of the split holding key 0 of the stage
      const int p0 = __builtin_amdgcn_readlane(rp < 64 ? pr0 : pr1, rp & 63);
      const int p1 = nk > 16 ? __builtin_amdgcn_readlane(rp + 1 < 64 ? pr0 : pr1, (rp + 1) & 63) : p0;
      if (nk >= 32) {
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
          const int im = wv + NW * k;
          const bool second = im < 8 ? (im >> 2) != 0 : (im - 8) >= 4;
          const uint64_t base = (im < 8 ? kc_addr : vc_addr) + (uint64_t)(second ? p1 : p0) * page_bytes;
          const uint32_t off = im < 8 ? koff + 64u * (im & 3) : voff + ((im - 8) & 3) * slot_bytes;
          dma16_sbase(off, base, slot_base + (uint32_t)im * 1024u);
        }
        return;
      }
#pragma nounroll
      for (int im = wv; im < 16; im += NW) {
        const uint16_t* src;
        if (im < 8) {
          const int kt = im >> 2, m = im & 3;
          const int key = 16 * kt + c;
          const bool v = key < nk;
          const int pg = v ? (kt ? p1 : p0) : p0;
          src = kc + ((size_t)pg * kPage + (v ? c : 0)) * slot_stride + 32 * m + 8 * qd;
        } else {
          const int e = im - 8;
          const int key = pv_key(qd, e);
          const bool v = key < nk;
          const int pg = v ? (e < 4 ? p0 : p1) : p0;
          src = vc + ((size_t)pg * kPage + (v ? (key & 15) : 0)) * slot_stride + 8 * c;
        }
        dma16(src, slot_base + (uint32_t)im * 1024u);
      }
    } else {
      const int j0 = 32 * (s - ncs);
#pragma nounroll
      for (int im = wv; im < 16; im += NW) {
        const uint16_t* src;
        if (im < 8) {
          const int kt = im >> 2, m = im & 3;
          int j = j0 + 16 * kt + c;
          j = j < p.W ? j : 0;
          src = kn + (size_t)(b * p.W + j) * slot_stride + 32 * m + 8 * qd;
        } else {
          int j = j0 + pv_key(qd, im - 8);
          j = j < p.W ? j : 0;
          src = vn + (size_t)(b * p.W + j) * slot_stride + 8 * c;
        }
        dma16(src, slot_base + (uint32_t)im * 1024u);
      }
    }
  };

  MfmaState<D, RB> st;
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    st.m[k] = neg_inf();
    st.l[k] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int s) __attribute__((always_inline)) {
    const char* buf = ring + (s % kLdsStages) * kStageBytes + lane * 16;
    bf16x8 kf[2][NC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int m = 0; m < NC; ++m)
        kf[kt][m] = *reinterpret_cast<const bf16x8*>(buf + (kt * 4 + m) * 1024);
    VRow<D> vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vv[e].v = *reinterpret_cast<const uint4*>(buf + (8 + e) * 1024);

    // One softmax + PV code path for every stage (masks applied to the raw
    // scores first) reached from one loop: specialised copies of the tile
    // step made the compiler copy every accumulator register at each stage.
    float x[RB][8];
    tile_scores<D, RB>(qf, kf, x);
    if (s < ncs) {
      const int nk = end - (start + 32 * s);
      if (nk < 32) {
#pragma unroll
        for (int k = 0; k < RB; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (pv_key(qd, e) >= nk) x[k][e] = neg_inf();
      }
    } else {
      const int j0 = 32 * (s - ncs);
#pragma unroll
      for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (((vrow[k] >> (j0 + pv_key(qd, e))) & 1ull) == 0ull) x[k][e] = neg_inf();
    }
    bf16x8 pf[RB], pl[RB];
    tile_softmax<D, RB>(x, p.scale_log2, st, pf, pl, [](int, int) { return true; });
    tile_pv<D, RB>(pf, pl, vv, st);
  };

  // Every stage in the ring at once (key slices, short splits): one wait, one
  // barrier, then each slice reduces its own stages.  Otherwise a pipeline of
  // kLdsAhead stages in flight, slice ks reducing stages ks, ks + KS, ...
  const bool at_once = KS > 1 && nst <= kLdsStages;
  if (at_once) {
    for (int s = 0; s < nst; ++s) issue(s);
    wait_vmem_barrier<0>();
  } else {
    for (int s = 0; s < kLdsAhead && s < nst; ++s) issue(s);
  }
  for (int s = at_once ? ks : 0; s < nst; s += at_once ? KS : 1) {
    if (!at_once) {
      const int after = min(kLdsAhead - 1, nst - 1 - s);
      wait_stage_barrier<IPW>(after);
      if (s + kLdsAhead < nst) issue(s + kLdsAhead);
      if (s % KS != ks) continue;
    }
    compute(s);
  }

  if constexpr (KS > 1) {
    // Slices 1 .. KS - 1 hand their states to slice 0 through the ring.
    // Slice 0 merges them and lays its rows out row-major in the ring (row
    // pitch D + 4 floats, so the 16 rows a store instruction spans fall in
    // different banks); then every wave of the workgroup stores whole rows,
    // 1 KB per store instruction, instead of slice 0 storing 16-byte pieces
    // of 16 rows per instruction.  The row image (NR * 16 rows) ends below
    // the slice states (which start at NR * kSliceStateFloats floats per
    // lane), so slice 0 may write rows while another of its waves still
    // reads states.
    constexpr int kPitch = D + 4;
    static_assert(16 * kPitch <= kSliceStateFloats * kWave, "row image below the slice states");
    wait_vmem_barrier<0>();  // every wave is done with the ring
    float* sbuf = reinterpret_cast<float*>(ring);
    auto slot = [&](int slice) { return sbuf + ((size_t)(slice * NR + tg) * kSliceStateFloats * kWave) + lane; };
    if (ks > 0) {
      float* d = slot(ks);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) d[(4 * t + e) * kWave] = st.acc[0][t][e];
      d[32 * kWave] = st.m[0];
      d[33 * kWave] = st.l[0];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const size_t item_row = (((size_t)b * p.max_splits + it.split) * p.Hkv + it.kvh) * (size_t)p.R;
    if (ks == 0) {
#pragma unroll
      for (int o = 1; o < KS; ++o) {
        const float* d = slot(o);
        const float mo = d[32 * kWave];
        const float lo = d[33 * kWave];
        const float mm = fmaxf(st.m[0], mo);
        const float mu = mm == neg_inf() ? 0.f : mm;
        const float a = fast_exp2(st.m[0] - mu);
        const float bo = fast_exp2(mo - mu);
        st.l[0] = st.l[0] * a + lo * bo;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) st.acc[0][t][e] = st.acc[0][t][e] * a + d[(4 * t + e) * kWave] * bo;
        st.m[0] = mm;
      }
      if (bad) {
        if (threadIdx.x == 0) raise_status(MTP_DEV_BAD_PAGE);
        st.m[0] = qnan();
#pragma unroll
        for (int t = 0; t < NT; ++t) st.acc[0][t] = f32x4{qnan(), qnan(), qnan(), qnan()};
      }
      const float l = rows4_sum(st.l[0]);
      const int rho = row_tile0 * 16 + c;
      if (qd == 0 && rho < p.R) {
        store_partial_ml(p.part_ml + 2 * item_row, 2 * rho, st.m[0], l);
      }
      // float4 j of lane (c, qd) holds row c, d = qd * D / 4 + 4 j .. + 4
      float* rowp = sbuf + (size_t)(tg * 16 + c) * kPitch + qd * (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < NT; t += 4)
          *reinterpret_cast<float4*>(rowp + e * (D / 16) + t) =
              make_float4(st.acc[0][t][e], st.acc[0][t + 1][e], st.acc[0][t + 2][e], st.acc[0][t + 3][e]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int row0 = it.rb * NR * 16;  // first row of this workgroup's row block
    constexpr int kVecs = NR * 16 * (D / 4);
#pragma unroll
    for (int f = threadIdx.x; f < kVecs; f += 64 * NW) {
      const int row = f / (D / 4);
      const int col = f - row * (D / 4);
      if (row0 + row < p.R)
        store_partial4(p.part_acc + item_row * D, (row0 + row) * D + col * 4,
                       *reinterpret_cast<const float4*>(sbuf + (size_t)row * kPitch + col * 4));
    }
    return;
  }

  // One key slice: the waves lay their rows out row-major in the ring (as
  // the key-slice path does) and then store whole rows, 1 KB per store
  // instruction.
  constexpr int kPitch = D + 4;
  static_assert(NR * RB * 16 * kPitch * 4 <= kLdsStages * kStageBytes, "row image fits the ring");
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
  wait_vmem_barrier<0>();  // every wave is done with the ring
  float* sbuf = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int k = 0; k < RB; ++k) {
    const float l = rows4_sum(st.l[k]);
    const int rho = (row_tile0 + k) * 16 + c;
    if (qd == 0 && rho < p.R) {
      store_partial_ml(p.part_ml + 2 * item_row, 2 * rho, st.m[k], l);
    }
    float* rowp = sbuf + (size_t)((tg * RB + k) * 16 + c) * kPitch + qd * (D / 4);
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
  for (int f = threadIdx.x; f < kVecs; f += 64 * NW) {
    const int row = f / (D / 4);
    const int col = f - row * (D / 4);
    if (row0 + row < p.R)
      store_partial4(p.part_acc + item_row * D, (row0 + row) * D + col * 4,
                     *reinterpret_cast<const float4*>(sbuf + (size_t)row * kPitch + col * 4));
  }
}

}  // namespace mtpv
