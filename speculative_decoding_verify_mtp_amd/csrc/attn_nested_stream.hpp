// Stream-K verify attention over the nested KV4 / KV8 cache (D = 128).
//
// The schedule of attn_partial_stream (per KV head, the flat list of 32-key
// stages of every segment; a persistent grid cuts each head's list into
// contiguous ranges, the ranges of the first dispatch round longer; one
// partial piece per (range, segment); the workgroup holding a segment's first
// stage records its pieces for the combine), with the stage work of
// attn_partial_nested_lds: committed stages stream through the code ring and
// are transcoded once per workgroup into double-buffered operand images.  The
// byte u = c8 + 136 of an element goes into the MFMA as the bf16 bit pattern
// 0x00uu, which is u * 2^-133 exactly for every u in [0, 255] (below 128 a
// subnormal, from 128 the first normal binade, whose spacing is the same), so
// a code becomes an operand by a byte permute, with no conversion:
//   K images: four v_perm per 8 elements;
//   V images: the bytes themselves (8 per lane), spread into bf16 pairs by the
//   same permutes that pair the keys of the PV operand.
// Q enters the committed stages scaled by 2^e (a power of two per row, so that
// |Q 2^e| lies in [2^120, 2^121): the products with u * 2^-133 stay in the
// normal fp32 range), the factor 2^(133 - e) moving into the row's softmax
// scale; P enters scaled by 2^60 (an offset in the exp), for the same reason
// on the PV side: products of V scales down to about 2^-50 (|v| ~ 1e-14)
// stay normal, and P 2^60 s stays below the bf16 limit for s < 2^60.  The
// accumulators hold 2^-73 sum_t p_t s_t u_t and the row sum 2^60 sum_t p_t
// until the offset is removed; lp = sum_t p_t s_t is kept in real units.  That correction is linear
// in the state and commutes with later rescales, so it is applied once per
// segment part, when the part's committed stages are followed by in-block
// stages or when the piece is written.  A segment's in-block stages (bf16
// rows of the block) are read with direct loads.
//
// KV4 (every committed key read at 4 bits): only the base-plane images are
// loaded and transcoded (4 code images per stage instead of 8; the
// refinement code is the constant 0).
#pragma once

#include "attn_mfma.hpp"
#include "attn_nested_lds.hpp"
#include "attn_stream.hpp"
#include "common.hpp"
#include "nested.hpp"

namespace mtpv {

template <int NR, bool KV4>
__global__ __launch_bounds__(64 * NR) __attribute__((amdgpu_waves_per_eu(2)))
void attn_partial_nested_stream(AttnParams p, StreamParams sp, NestedAttn na) {
  constexpr int D = 128;
  constexpr int RB = 1;
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  constexpr int CPW = (KV4 ? 4 : 8) / NR;  // code images per wave per stage
  constexpr int PER = CPW + 1;  // loads per wave per stage (codes + scales)
  constexpr int IPW = 16 / NR;  // operand images transcoded per wave
  constexpr int SL = kWave / NR;
  constexpr int kAhead = kNestAhead;
  __shared__ __attribute__((aligned(16))) char ring[kNestRingStages * kNestCodeBytes];
  __shared__ __attribute__((aligned(16))) char img[2 * kNestImgBytesU];
  __shared__ int s_pref[kStreamMaxB + 1];

  const int wg = (int)blockIdx.x;
  const int G = (int)gridDim.x;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int qd = lane >> 4;

  stream_prefix(p, sp.nts, s_pref);
  const int total = s_pref[p.B];
  const int Gh = G / p.Hkv;
  const int gi = wg / p.Hkv;
  const int kvh = wg - gi * p.Hkv;
  const int piece0 = kvh * (Gh + p.B * p.nRB) + gi;
  const RangeCut cut(sp, total, Gh);
  int g = min(cut.start(gi), total);
  const int g_end = min(cut.start(gi + 1), total);
  if (g >= g_end) return;  // uniform over the workgroup

  const int Hkv = p.Hkv;
  const uint32_t ring_base = lds_offset(ring);
  const size_t slot_stride = (size_t)Hkv * D;
  const float sl2 = p.scale_log2 * 0.0625f;  // the key scales enter as s, not s / 16 (before the Q scaling)
  // code image lane l <- key (l % 16) ^ (l / 16), part l / 16
  const int dkey = c ^ qd;
  const uint32_t doff = 64u * dkey + 16u * qd;
  const uint8_t* kbase = na.kv.k_base;
  const uint8_t* vbase = na.kv.v_base;
  const uint8_t* kref = na.kv.k_ref != nullptr ? na.kv.k_ref : na.kv.k_base;
  const uint8_t* vref = na.kv.v_ref != nullptr ? na.kv.v_ref : na.kv.v_base;
  const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + (size_t)kvh * D;
  const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + (size_t)kvh * D;

  MfmaState<D, RB> st;
  float lp[RB];
  bool coded = false;  // acc and lp in code units (offset not yet removed)
  bf16x8 qf[RB][NC];  // Q operands (in-block stages)
  bf16x8 qs[RB][NC];  // Q 2^e (committed stages)
  float nqs[RB];      // -136 sum_d q_d, times 2^(e - 133)
  float sl2r[RB];     // sl2 2^(133 - e)
  uint64_t vrow[RB];
  int cur_sigma = -1;
  bool bad = false;

  // acc <- (2^73 acc - 136 lp) / 16 and the row sum <- 2^-60 l: the
  // committed keys' values and weights in real units
  auto settle = [&]() {
    if (!coded) return;
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const float off = -kNestByteOffset * 0.0625f * rows4_sum(lp[k]);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) st.acc[k][t][e] = fmaf(st.acc[k][t][e], 0x1p69f, off);
      st.l[k] *= 0x1p-60f;
      lp[k] = 0.f;
    }
    coded = false;
  };

  while (g < g_end) {
    // ---- locate the run: sequence b, segment, stages [i0, i1) of the segment
    int lo = 0, hi = p.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= g) lo = mid;
      else hi = mid;
    }
    const int b = lo;
    const int nb = (s_pref[b + 1] - s_pref[b]) / p.nRB;
    const int ncs = nb - sp.nts;
    const int off = g - s_pref[b];
    const int rb = off / nb;
    const int i0 = off - rb * nb;
    const int lsig = b * p.nRB + rb;
    const int sigma = b * sp.nseg + kvh * p.nRB + rb;
    const int seg_end_g = s_pref[b] + (rb + 1) * nb;
    const int i1 = min(nb, i0 + min(g_end - g, kRunStages));
    const int L = p.ctx_lens[b];
    const int row_tile0 = (rb * NR + wv) * RB;

    if (sigma != cur_sigma) {  // a new segment: fresh state, its Q operands and row sums
      cur_sigma = sigma;
      bad = false;
      coded = false;
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        st.m[k] = neg_inf();
        st.l[k] = 0.f;
        lp[k] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int rho = (row_tile0 + k) * 16 + c;
        float part = 0.f;
        if (rho < p.R) {
          const int w = rho / p.g;
          const int j = rho - w * p.g;
          const uint16_t* src = static_cast<const uint16_t*>(p.q) +
                                ((size_t)(b * p.W + w) * p.Hq + (size_t)kvh * p.g + j) * D + qd * 8;
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
        vrow[k] = 0;
      }
      if (i0 == 0 && threadIdx.x == 0) {
        sp.seg_info[2 * sigma] = piece0 + lsig;
        sp.seg_info[2 * sigma + 1] = cut.range_of(seg_end_g - 1) - gi + 1;
      }
    }

    // page window: pages [2 i0, ...) of sequence b for the committed stages of the run
    const int cend = min(i1, ncs);
    int pw[4] = {0, 0, 0, 0};
    if (cend > i0) {
      const int pfirst = 2 * i0;
      const int plast = (min(32 * cend, L) + kPage - 1) / kPage;
      const int32_t* btrow = p.block_table + (size_t)b * p.max_pages;
      bool badp = false;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pi = pfirst + 64 * k + lane;
        if (pi < plast) {
          int v = btrow[pi];
          if ((unsigned)v >= (unsigned)p.num_pages) {
            badp = true;
            v = 0;
          }
          pw[k] = v;
        }
      }
      bad = bad || (__ballot(badp) != 0ull);
    }
    // in-block visibility when the run reaches the in-block stages
    int iend = i1;
    if (i1 > ncs) {
      bool ok;
      const uint64_t vnode = node_visibility(p.mask_kind[b], lane_mask_id(p, b, lane), p.W,
                                             p.lookback, lane, ok);
      if (ok) {
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          const int rho = min((row_tile0 + k) * 16 + c, p.R - 1);
          vrow[k] = shfl64(vnode, rho / p.g);
        }
      } else {
        iend = ncs > i0 ? ncs : i0;  // malformed mask: the combine writes NaN rows
      }
    }
    const int kv8_from = na.kv8_recent < 0 ? 0 : max(0, L - na.kv8_recent);
    __builtin_amdgcn_s_waitcnt(0);  // run set-up loads done; the pipeline starts empty

    // ---- committed stages [i0, cend): code ring, transcode, MFMA
    const int ncr = cend - i0;
    auto issue = [&](int s) __attribute__((always_inline)) {
      const uint32_t slot = ring_base + (uint32_t)(s % kNestRingStages) * kNestCodeBytes;
      const int t0 = 32 * (i0 + s);
      const int nk = L - t0;
      const int rp = 2 * s;
      const int p0 = __builtin_amdgcn_readlane(pick4(pw, rp >> 6), rp & 63);
      const int p1 = nk > 16 ? __builtin_amdgcn_readlane(pick4(pw, (rp + 1) >> 6), (rp + 1) & 63) : p0;
      const bool any8 = min(t0 + 31, L - 1) >= kv8_from;
#pragma unroll
      for (int k = 0; k < CPW; ++k) {
        // image 0..7: kind = im / 2 (K base, K ref, V base, V ref), half = im % 2;
        // KV4 loads images 0, 1, 4, 5
        const int j = wv + NR * k;
        const int im = KV4 ? ((j >> 1) << 2) | (j & 1) : j;
        const int kind = im >> 1, half = im & 1;
        const uint8_t* b2 = (kind & 2) ? vbase : kbase;
        const uint8_t* r2 = (kind & 2) ? vref : kref;
        const uint8_t* plane = ((kind & 1) && any8) ? r2 : b2;
        const int pg = half ? p1 : p0;
        if (nk >= 32) {
          const uint64_t base = (uint64_t)(uintptr_t)plane + (((uint64_t)pg * Hkv + kvh) << 10);
          dma16_sbase(doff, base, slot + (uint32_t)im * 1024u);
        } else {
          const int key = 16 * half + dkey;
          const bool v = key < nk;
          const size_t row = nest_row(v ? pg : p0, kvh, v ? dkey : 0, Hkv);
          dma16(plane + row * 64 + 16 * qd, slot + (uint32_t)im * 1024u);
        }
      }
      if (lane < SL) {
        const int gk = wv * SL + lane;
        const int key = gk & 31;
        const bool v = key < nk;
        const size_t row = nest_row(v ? (key < 16 ? p0 : p1) : p0, kvh, v ? (key & 15) : 0, Hkv);
        dma4((gk < 32 ? na.kv.k_scale : na.kv.v_scale) + row, slot + 8192u + 4u * (uint32_t)(wv * SL));
      }
    };
    auto transcode = [&](int s) __attribute__((always_inline)) {
      const char* code = ring + (s % kNestRingStages) * kNestCodeBytes;
      char* out = img + (s & 1) * kNestImgBytesU;
      const int t0 = 32 * (i0 + s);
#pragma unroll
      for (int k = 0; k < IPW; ++k) {
        const int im = wv + NR * k;
        int off, key;
        const char* cb;
        if (im < 8) {  // K operand (kt, m): key 16 kt + c, part m, dword qd
          const int kt = im >> 2, m = im & 3;
          off = 16 * (16 * m + (c ^ m)) + 4 * qd;
          cb = code + kt * 1024;
          key = 16 * kt + c;
        } else {  // V vector e: key pv_key(qd, e), part c / 4, dword c % 4
          const int e = im - 8;
          const int half = e >> 2;
          const int k16 = 4 * qd + (e & 3);
          const int part = c >> 2;
          off = 16 * (16 * part + (k16 ^ part)) + 4 * (c & 3);
          cb = code + 4096 + half * 1024;
          key = 16 * half + k16;
        }
        const unsigned bw = *reinterpret_cast<const unsigned*>(cb + off);
        unsigned rw = kNestZeroRef;
        if constexpr (!KV4) {
          rw = *reinterpret_cast<const unsigned*>(cb + 2048 + off);
          if (t0 + key < kv8_from) rw = kNestZeroRef;
        }
        unsigned ev, od;
        nest_bytes(bw, rw, ev, od);
        if (im < 8)
          *reinterpret_cast<uint4*>(out + im * 1024 + 16 * lane) = nest_k_operand(ev, od);
        else
          *reinterpret_cast<uint2*>(out + 8192 + (im - 8) * 512 + 8 * lane) = make_uint2(ev, od);
      }
    };
    if (ncr > 0) {
      coded = true;
      for (int s = 0; s < kAhead && s < ncr; ++s) issue(s);
      wait_code_stage_barrier<PER>(min(kAhead, ncr) - 1);  // stage 0 landed
      transcode(0);
      for (int s = 0; s < ncr; ++s) {
        // stage s + 1 landed, operands of s complete, the other image buffer free
        const int issued = min(s + kAhead, ncr);
        wait_code_stage_barrier<PER>(max(0, issued - (s + 2)));
        if (s + kAhead < ncr) issue(s + kAhead);
        if (s + 1 < ncr) transcode(s + 1);

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
        const float4 sk0 = *reinterpret_cast<const float4*>(code + 8192 + 16 * qd);
        const float4 sk1 = *reinterpret_cast<const float4*>(code + 8192 + 64 + 16 * qd);
        const float4 sv0 = *reinterpret_cast<const float4*>(code + 8192 + 128 + 16 * qd);
        const float4 sv1 = *reinterpret_cast<const float4*>(code + 8192 + 192 + 16 * qd);
        float skv[8] = {sk0.x, sk0.y, sk0.z, sk0.w, sk1.x, sk1.y, sk1.z, sk1.w};
        float svv[8] = {sv0.x, sv0.y, sv0.z, sv0.w, sv1.x, sv1.y, sv1.z, sv1.w};
        const int nk = L - 32 * (i0 + s);
        bf16x8 pf[RB], pl[RB];
        nest_scores_u<RB>(qs, kf, skv, svv, nqs, sl2r, nk, st, lp, pf, pl);
        tile_pv_u<RB>(pf, pl, vb, st);
      }
      // every wave is done with the ring and the images before they are reused
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // ---- in-block stages [max(i0, ncs), iend): bf16 rows of the block, direct loads
    const int ib0 = max(i0, ncs);
    if (iend > ib0) {
      settle();
      for (int i = ib0; i < iend; ++i) {
        const int j0 = 32 * (i - ncs);
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

    g += i1 - i0;
    if (g == seg_end_g || g == g_end) {  // the segment (or this range) ends: write the piece
      settle();
      if (bad) {
        if (threadIdx.x == 0) raise_status(MTP_DEV_BAD_PAGE);
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          st.m[k] = qnan();
#pragma unroll
          for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{qnan(), qnan(), qnan(), qnan()};
        }
      }
      const size_t piece = (size_t)piece0 + lsig;
      constexpr int kPitch = D + 4;  // padded rows: the 16 rows a write spans fall in different banks
      static_assert(NR * RB * 16 * kPitch * 4 <= kNestRingStages * kNestCodeBytes, "rows fit the ring");
      // The ring is idle (no run is in flight): the waves lay the piece's rows
      // out row-major there, then store whole rows, 1 KB per store instruction.
      float* sbuf = reinterpret_cast<float*>(ring);
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        const float l = rows4_sum(st.l[k]);
        const int rl = (wv * RB + k) * 16 + c;
        if (qd == 0 && rb * sp.rows_block + rl < p.R) {
          const size_t pidx = piece * sp.rows_block + rl;
          p.part_ml[2 * pidx] = st.m[k];
          p.part_ml[2 * pidx + 1] = l;
        }
        float* rowp = sbuf + (size_t)rl * kPitch + qd * (D / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int t = 0; t < NT; t += 4)
            *reinterpret_cast<float4*>(rowp + e * (D / 16) + t) =
                make_float4(st.acc[k][t][e], st.acc[k][t + 1][e], st.acc[k][t + 2][e], st.acc[k][t + 3][e]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int nvec = sp.rows_block * (D / 4);
      for (int f = threadIdx.x; f < nvec; f += 64 * NR) {
        const int row = f / (D / 4);
        const int col = f - row * (D / 4);
        if (rb * sp.rows_block + row < p.R)
          *reinterpret_cast<float4*>(p.part_acc + (piece * sp.rows_block + row) * D + col * 4) =
              *reinterpret_cast<const float4*>(sbuf + (size_t)row * kPitch + col * 4);
      }
      // the next run refills the ring: every wave is done reading the rows
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      cur_sigma = -1;
    }
  }
}

}  // namespace mtpv
