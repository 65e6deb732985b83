// Stream-K verify attention, D = 128, bf16 MFMA, K/V through an LDS ring.
//
// The work of one launch is, per KV head, the flat list of 32-key stages of
// every segment (sequence b, row block) of that head, in that order: the
// segment of sequence b has ceil(L_b / 32) committed stages followed by
// ceil(W / 32) in-block stages.  The lists of all KV heads have the same
// length.  A persistent grid of G = Hkv * G' workgroups gives each head G'
// workgroups, which cut its list into G' contiguous ranges of fixed lengths:
// every workgroup streams a set number of stages whatever the mix of context
// lengths, and no workgroup is empty.  The ranges are equal, except that
// with two workgroups per compute unit the ranges of the first dispatch round
// (workgroups 0 .. 255, one per CU) are longer than those of the second: a
// SIMD issues the older of two ready waves first, so the first-round
// workgroup of a CU streams faster than its partner, and with equal ranges
// half of the grid idles while the other half finishes (the per-workgroup
// end times of the ragged batch were two groups about 20% apart, split
// exactly at the dispatch rounds).  Workgroup w serves head w % Hkv and
// range w / Hkv, so the Hkv workgroups of one range are dispatched together
// and walk the same pages at the same time, each reading its head's slice of
// every token slot: the DRAM rows they open are shared (measured: scattering
// the heads of a page over the dispatch order costs about 5% of the stream).
//
// A workgroup walks its range in runs: a run is at most kRunStages stages of
// one segment, covered by one window of page indices held in four registers
// per lane.  Each run loads its page window (and, when it opens a segment,
// the segment's Q operands and in-block visibility), then streams its stages
// through the same LDS ring and MFMA tile as attn_partial_lds.  The softmax
// state carries over runs of the same segment; when the segment (or the
// range) ends, the workgroup writes one partial "piece".
//
// Piece ids: within one head, a piece is a pair (range r, segment s) with
// range r overlapping segment s.  Walking the head's list, each step to the
// next piece raises r, s or both by one, so r + s is unique and below
// G' + B * row_blocks; head k's pieces take ids k * (G' + B * row_blocks) +
// r + s.  The pieces of one segment therefore have consecutive ids.  The
// workgroup that holds a segment's first stage records (first piece id,
// piece count) for the combine.
#pragma once

#include "attn_lds.hpp"
#include "attn_mfma.hpp"
#include "common.hpp"

namespace mtpv {

// 48 KB ring plus the 4 KB prefix table.  The four-wave kernel is compiled
// for three workgroups per CU (at most 168 VGPRs: three waves per SIMD; 156
// of gfx950's 160 KB of LDS), though the launch plan runs two per CU (see
// kStreamWgsPerCU): ragged batch 909 us with a 4-stage ring and a budget of
// two, 903-908 us with this ring and budget.
constexpr int kStreamStages = 3;
constexpr int kStreamMaxB = 1024;  // sequences whose stage prefix fits the LDS table
constexpr int kRunStages = 128;    // stages covered by one page window (256 pages)

struct StreamParams {
  int* seg_info;   // [B * nseg][2]: first piece id, number of pieces
  int nts;         // in-block stages per segment, ceil(W / 32)
  int nseg;        // segments per sequence, Hkv * nRB
  int rows_block;  // rows of a row block (NR * RB * 16)
  int h1 = 0;     // ranges per head in the first dispatch round (0: all ranges equal)
  int w_num = 1, w_den = 1;  // a first-round range is w_num / w_den times as long as the others
  int piece_rows = 0;  // combine: one row per wave (segments of many pieces)
};

// Stage ranges of one head's list: ranges r < h1 hold t1 stages, the others
// t2, with t1 ~ (w_num / w_den) t2 and h1 t1 + (G' - h1) t2 >= total.  Short
// ranges stay equal (contexts <= 4096 in 12 sequences, about 12 stages per
// range: 37.7 us equal, 38.8 us weighted; 64 stages per range and more gain
// 2-3.5%).
constexpr int kMinWeightedStages = 32;
struct RangeCut {
  int h1, t1, t2;
  __device__ RangeCut(const StreamParams& sp, int total, int Gh) {
    if (sp.h1 > 0 && sp.h1 < Gh && total >= kMinWeightedStages * Gh) {
      h1 = sp.h1;
      const long long den = (long long)h1 * sp.w_num + (long long)(Gh - h1) * sp.w_den;
      t2 = (int)max(1LL, ((long long)total * sp.w_den + den - 1) / den);
      t1 = (int)max(1LL, ((long long)t2 * sp.w_num + sp.w_den - 1) / sp.w_den);
    } else {
      h1 = 0;
      t1 = t2 = max(1, (total + Gh - 1) / Gh);
    }
  }
  __device__ int start(int r) const { return r <= h1 ? r * t1 : h1 * t1 + (r - h1) * t2; }
  __device__ int range_of(int x) const { return x < h1 * t1 ? x / t1 : h1 + (x - h1 * t1) / t2; }
};

__device__ __forceinline__ int pick4(const int (&v)[4], int k) {
  return k == 0 ? v[0] : k == 1 ? v[1] : k == 2 ? v[2] : v[3];
}

// Stage prefix over the sequences of one head's list: s_pref[b] = stages of
// sequences < b (s_pref[B] = the list's length), each sequence ceil(L / 32)
// committed and nts in-block stages per row block; a sequence whose context
// lies outside [0, max_ctx] has none.  Wave 0 computes it; all threads wait.
__device__ __forceinline__ void stream_prefix(const AttnParams& p, int nts, int* s_pref) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    int run = 0;
    for (int b0 = 0; b0 < p.B; b0 += kWave) {
      const int bb = b0 + lane;
      int n = 0;
      if (bb < p.B) {
        const int L = p.ctx_lens[bb];
        if (L >= 0 && L <= p.max_ctx) n = ((L + 31) / 32 + nts) * p.nRB;
      }
      int x = n;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (bb < p.B) s_pref[bb + 1] = run + x;
      run += __shfl(x, 63);
    }
    if (lane == 0) s_pref[0] = 0;
  }
  __syncthreads();
}

// Workgroups per compute unit each variant's register budget is compiled for.
__host__ __device__ constexpr int stream_wgs_per_cu(int RB, int NR) {
  return RB == 1 && NR == 4 ? 3 : RB == 1 ? 2 : 1;
}

template <int RB, int NR>
__global__ __launch_bounds__(64 * NR) __attribute__((amdgpu_waves_per_eu(stream_wgs_per_cu(RB, NR))))
void attn_partial_stream(AttnParams p, StreamParams sp) {
  constexpr int D = 128;
  constexpr int NC = D / 32;
  constexpr int NT = D / 16;
  constexpr int IPW = 16 / NR;
  constexpr int NS = kStreamStages;
  __shared__ __attribute__((aligned(16))) char ring[NS * kStageBytes];
  __shared__ int s_pref[kStreamMaxB + 1];

  const int wg = (int)blockIdx.x;
  const int G = (int)gridDim.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int c = lane & 15;
  const int qd = lane >> 4;

  stream_prefix(p, sp.nts, s_pref);
  const int total = s_pref[p.B];
  const int Gh = G / p.Hkv;          // ranges per head (the host makes G a multiple of Hkv)
  const int gi = wg / p.Hkv;         // this workgroup's range
  const int kvh = wg - gi * p.Hkv;   // and head
  const int piece0 = kvh * (Gh + p.B * p.nRB) + gi;
  const RangeCut cut(sp, total, Gh);
  int g = min(cut.start(gi), total);
  const int g_end = min(cut.start(gi + 1), total);
  if (g >= g_end) return;  // uniform over the workgroup

  const uint32_t ring_base = lds_offset(ring);
  const size_t slot_stride = (size_t)p.Hkv * D;
  const uint32_t slot_bytes = (uint32_t)(slot_stride * 2);
  const uint64_t page_bytes = (uint64_t)kPage * slot_bytes;
  const uint32_t koff = (uint32_t)c * slot_bytes + 16u * qd;
  const uint32_t voff = 4u * qd * slot_bytes + 16u * c;

  MfmaState<D, RB> st;
  bf16x8 qf[RB][NC];
  uint64_t vrow[RB];
  int cur_sigma = -1;
  bool bad = false;

  while (g < g_end) {
    // ---- locate the run: sequence b (last b with s_pref[b] <= g), segment, stage
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
    const int lsig = b * p.nRB + rb;  // segment index in this head's list
    const int sigma = b * sp.nseg + kvh * p.nRB + rb;
    const int seg_end_g = s_pref[b] + (rb + 1) * nb;
    const int i1 = min(nb, i0 + min(g_end - g, kRunStages));
    const int L = p.ctx_lens[b];

    const uint16_t* kc = static_cast<const uint16_t*>(p.k_cache) + (size_t)kvh * D;
    const uint16_t* vc = static_cast<const uint16_t*>(p.v_cache) + (size_t)kvh * D;
    const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + (size_t)kvh * D;
    const uint16_t* vn = static_cast<const uint16_t*>(p.v_new) + (size_t)kvh * D;
    const uint64_t kc_addr = (uint64_t)(uintptr_t)kc, vc_addr = (uint64_t)(uintptr_t)vc;
    const int row_tile0 = (rb * NR + wv) * RB;

    if (sigma != cur_sigma) {  // a new segment: fresh state and its Q operands
      cur_sigma = sigma;
      bad = false;
#pragma unroll
      for (int k = 0; k < RB; ++k) {
        st.m[k] = neg_inf();
        st.l[k] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) st.acc[k][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int rho = (row_tile0 + k) * 16 + c;
        if (rho < p.R) {
          const int w = rho / p.g;
          const int j = rho - w * p.g;
          const uint16_t* src = static_cast<const uint16_t*>(p.q) +
                                ((size_t)(b * p.W + w) * p.Hq + (size_t)kvh * p.g + j) * D + qd * 8;
#pragma unroll
          for (int m = 0; m < NC; ++m) qf[k][m] = load_bf16x8(src + m * 32);
        } else {
#pragma unroll
          for (int m = 0; m < NC; ++m) qf[k][m] = bf16x8{};
        }
        vrow[k] = 0;
      }
      if (i0 == 0 && threadIdx.x == 0) {
        sp.seg_info[2 * sigma] = piece0 + lsig;
        sp.seg_info[2 * sigma + 1] = cut.range_of(seg_end_g - 1) - gi + 1;
      }
    }

    // page window: pages [2 i0, ...) of sequence b for the committed stages of the run
    const int cend = min(i1, ncs);  // committed stages of the run are [i0, cend)
    int pw[4] = {0, 0, 0, 0};
    if (cend > i0) {
      const int pfirst = 2 * i0;
      const int plast = (min(32 * cend, L) + kPage - 1) / kPage;  // one past the last page needed
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
    __builtin_amdgcn_s_waitcnt(0);  // run set-up loads done; the pipeline starts empty

    auto issue = [&](int i, int slot) {
      const uint32_t slot_base = ring_base + (uint32_t)slot * kStageBytes;
      if (i < ncs) {
        const int t0 = 32 * i;
        const int nk = L - t0;
        const int rp = 2 * (i - i0);
        const int p0 = __builtin_amdgcn_readlane(pick4(pw, rp >> 6), rp & 63);
        const int p1 = nk > 16 ? __builtin_amdgcn_readlane(pick4(pw, (rp + 1) >> 6), (rp + 1) & 63) : p0;
        if (nk >= 32) {
#pragma unroll
          for (int k = 0; k < IPW; ++k) {
            const int im = wv + NR * k;
            const bool second = im < 8 ? (im >> 2) != 0 : (im - 8) >= 4;
            const uint64_t base = (im < 8 ? kc_addr : vc_addr) + (uint64_t)(second ? p1 : p0) * page_bytes;
            const uint32_t o = im < 8 ? koff + 64u * (im & 3) : voff + ((im - 8) & 3) * slot_bytes;
            dma16_sbase(o, base, slot_base + (uint32_t)im * 1024u);
          }
          return;
        }
#pragma nounroll
        for (int im = wv; im < 16; im += NR) {
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
        const int j0 = 32 * (i - ncs);
#pragma nounroll
        for (int im = wv; im < 16; im += NR) {
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

    const int nst = iend - i0;
    for (int s = 0; s < NS - 1 && s < nst; ++s) issue(i0 + s, s);
    for (int s = 0; s < nst; ++s) {
      wait_stage_barrier<IPW>(min(NS - 2, nst - 1 - s));
      if (s + NS - 1 < nst) issue(i0 + s + NS - 1, (s + NS - 1) % NS);
      const int i = i0 + s;
      const char* buf = ring + (s % NS) * kStageBytes + lane * 16;
      bf16x8 kf[2][NC];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int m = 0; m < NC; ++m)
          kf[kt][m] = *reinterpret_cast<const bf16x8*>(buf + (kt * 4 + m) * 1024);
      VRow<D> vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e].v = *reinterpret_cast<const uint4*>(buf + (8 + e) * 1024);
      // One softmax + PV code path for every stage, the masks (keys past the
      // committed range, the in-block visibility) applied to the raw scores
      // first.  With a single call site the accumulators stay in their
      // registers from stage to stage; three specialised copies of the tile
      // step made the compiler copy all 32 accumulator registers at every
      // stage (234 -> 169 VGPRs, about 210 -> 130 VALU instructions per
      // full stage; ragged batch 932 -> 909 us).
      float x[RB][8];
      tile_scores<D, RB>(qf, kf, x);
      if (i < ncs) {
        const int nk = L - 32 * i;
        if (nk < 32) {
#pragma unroll
          for (int k = 0; k < RB; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (pv_key(qd, e) >= nk) x[k][e] = neg_inf();
        }
      } else {
        const int j0 = 32 * (i - ncs);
#pragma unroll
        for (int k = 0; k < RB; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (((vrow[k] >> (j0 + pv_key(qd, e))) & 1ull) == 0ull) x[k][e] = neg_inf();
      }
      bf16x8 pf[RB], pl[RB];
      tile_softmax<D, RB, false>(x, p.scale_log2, st, pf, pl, [](int, int) { return true; });
      tile_pv<D, RB>(pf, pl, vv, st);
    }
    wait_vmem_barrier<0>();  // every wave is done with the ring before the next run fills it

    g += i1 - i0;
    if (g == seg_end_g || g == g_end) {  // the segment (or this range) ends: write the piece
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
      if constexpr (NR * RB * 16 * kPitch * 4 <= NS * kStageBytes) {
        // The ring is idle (the run has drained it): the waves lay the
        // piece's rows out row-major there, then store whole rows, 1 KB per
        // store instruction.
        float* sbuf = reinterpret_cast<float*>(ring);
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          const float l = rows4_sum(st.l[k]);
          const int rl = (wv * RB + k) * 16 + c;  // row within the block
          if (qd == 0 && rb * sp.rows_block + rl < p.R)
            store_partial_ml(p.part_ml + 2 * piece * sp.rows_block, 2 * rl, st.m[k], l);
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
            store_partial4(p.part_acc + piece * sp.rows_block * D, row * D + col * 4,
                           *reinterpret_cast<const float4*>(sbuf + (size_t)row * kPitch + col * 4));
        }
        // the next run refills the ring: every wave is done reading the rows
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      } else {
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          float l = st.l[k];
          l = rows4_sum(l);
          const int rl = (wv * RB + k) * 16 + c;  // row within the block
          const int rho = rb * sp.rows_block + rl;
          if (rho < p.R) {
            const size_t pidx = piece * sp.rows_block + rl;
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
      cur_sigma = -1;
    }
  }
}

}  // namespace mtpv
