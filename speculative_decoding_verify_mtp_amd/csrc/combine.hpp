// Split-K combine: merges the per-split partial softmax states of one output
// row (b, w, h) into out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s and
// lse = ln 2 * (M + log2 sum_s 2^(m_s - M) l_s).  Sequences with a malformed
// mask or context length get NaN rows.
//
// Split layout (combine_rows): one wave per row, `rows` rows per workgroup
// (waves past them idle).  Pass 1 spreads the splits over the lanes (one
// split per lane) for M and the denominator.  Pass 2 splits the wave into
// four groups of sixteen lanes: group q takes splits q, q+4, ..., each lane
// D/16 consecutive accumulators, so every load is 16-byte wide and many are
// in flight; the four group sums are folded with two shuffles.
// Few partials per row (combine_rows_grouped): four rows per wave, see there.
#pragma once

#include "accept_commit.hpp"
#include "attn_stream.hpp"
#include "common.hpp"

namespace mtpv {

// Partials of the split kernels, [B, splits, Hkv, R] rows.
template <int D>
__device__ __forceinline__ void combine_rows(const AttnParams& p, unsigned block, int rows) {
  constexpr int VPL = D / 16;  // accumulators per lane per split
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4, gl = lane & 15;
  const int wv = threadIdx.x >> 6;
  const size_t row = (size_t)block * rows + wv;
  if (wv >= rows || row >= (size_t)p.B * p.W * p.Hq) return;
  const int h = (int)(row % p.Hq);
  const size_t bw = row / p.Hq;
  const int w = (int)(bw % p.W);
  const int b = (int)(bw / p.W);
  const int kvh = h / p.g;
  const int rho = w * p.g + (h - kvh * p.g);

  // Loads that need neither the context length nor the split states go out
  // first: the accumulators of the first kCombineFast splits of the
  // launch-wide split count (splits past this row's count are dropped
  // by selection, never by a zero weight: stale workspace may hold NaN).
  constexpr int kBatch = kCombineFast / 4;  // splits per 16-lane group in flight
  const size_t base = (((size_t)b * p.max_splits) * p.Hkv + kvh) * (size_t)p.R + rho;
  const size_t sstride = (size_t)p.Hkv * p.R;
  float4 v[kBatch][VPL / 4];
  float m_spec = neg_inf(), l_spec = 0.f;  // split state of split `lane`
  if (lane < p.max_splits) {
    m_spec = p.part_ml[2 * (base + lane * sstride)];
    l_spec = p.part_ml[2 * (base + lane * sstride) + 1];
  }
  const int nspec = p.max_splits < 4 * kBatch ? p.max_splits : 4 * kBatch;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int sl = 4 * u + gq < nspec ? 4 * u + gq : 0;
    const float4* src = reinterpret_cast<const float4*>(p.part_acc + (base + sl * sstride) * D + gl * VPL);
#pragma unroll
    for (int j = 0; j < VPL / 4; ++j) v[u][j] = src[j];
  }

  const int L = p.ctx_lens[b];
  bool ok;
  node_visibility(p.mask_kind[b], lane_mask_id(p, b, lane), p.W, p.lookback, lane, ok);
  const bool ctx_ok = L >= 0 && L <= p.max_ctx;
  float* o = p.out + row * D;
  if (!ok || !ctx_ok) {
    if (lane == 0 && w == 0 && h == 0)
      raise_status((ok ? 0u : MTP_DEV_BAD_MASK) | (ctx_ok ? 0u : MTP_DEV_BAD_CTX));
    for (int i = lane; i < D; i += kWave) o[i] = qnan();
    if (p.lse != nullptr && lane == 0) p.lse[row] = qnan();
    return;
  }
  const int ns = num_splits(p, L);
  const int nfast = ns < 4 * kBatch ? ns : 4 * kBatch;

  const bool have = lane < ns;
  float M = have ? m_spec : neg_inf();
  for (int s = lane + kWave; s < ns; s += kWave) M = fmaxf(M, p.part_ml[2 * (base + s * sstride)]);
  M = wave_max(M);
  const float wlane = have ? fast_exp2(m_spec - M) : 0.f;  // weight of split `lane`
  float wl = have ? wlane * l_spec : 0.f;
  for (int s = lane + kWave; s < ns; s += kWave) {
    const size_t i = base + s * sstride;
    wl += fast_exp2(p.part_ml[2 * i] - M) * p.part_ml[2 * i + 1];
  }
  const float den = wave_sum(wl);

  // pass 2: weighted accumulator sums, four groups of sixteen lanes
  float a[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) a[j] = 0.f;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int s = 4 * u + gq;
    const float wt = __shfl(wlane, s & 63);
    if (s < nfast) {
#pragma unroll
      for (int j = 0; j < VPL / 4; ++j) {
        a[4 * j] = fmaf(wt, v[u][j].x, a[4 * j]);
        a[4 * j + 1] = fmaf(wt, v[u][j].y, a[4 * j + 1]);
        a[4 * j + 2] = fmaf(wt, v[u][j].z, a[4 * j + 2]);
        a[4 * j + 3] = fmaf(wt, v[u][j].w, a[4 * j + 3]);
      }
    }
  }
  // splits 32..63 (weights in lanes), in batches of eight per group
  const int nlane = ns < kWave ? ns : kWave;
  for (int s0 = 4 * kBatch; s0 < nlane; s0 += 4 * kBatch) {
    float wt[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + 4 * u + gq;
      wt[u] = __shfl(wlane, s & 63);
      const int sl = s < nlane ? s : 0;
      if (s >= nlane) wt[u] = 0.f;
      const float4* src = reinterpret_cast<const float4*>(p.part_acc + (base + sl * sstride) * D + gl * VPL);
#pragma unroll
      for (int j = 0; j < VPL / 4; ++j) v[u][j] = src[j];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
#pragma unroll
      for (int j = 0; j < VPL / 4; ++j) {
        a[4 * j] = fmaf(wt[u], v[u][j].x, a[4 * j]);
        a[4 * j + 1] = fmaf(wt[u], v[u][j].y, a[4 * j + 1]);
        a[4 * j + 2] = fmaf(wt[u], v[u][j].z, a[4 * j + 2]);
        a[4 * j + 3] = fmaf(wt[u], v[u][j].w, a[4 * j + 3]);
      }
    }
  }
  for (int s = kWave + gq; s < ns; s += 4) {  // rare: more than 64 splits
    const size_t i = base + s * sstride;
    const float wt = fast_exp2(p.part_ml[2 * i] - M);
    const float4* src = reinterpret_cast<const float4*>(p.part_acc + i * D + gl * VPL);
#pragma unroll
    for (int j = 0; j < VPL / 4; ++j) {
      const float4 v = src[j];
      a[4 * j] = fmaf(wt, v.x, a[4 * j]);
      a[4 * j + 1] = fmaf(wt, v.y, a[4 * j + 1]);
      a[4 * j + 2] = fmaf(wt, v.z, a[4 * j + 2]);
      a[4 * j + 3] = fmaf(wt, v.w, a[4 * j + 3]);
    }
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    a[j] = rows4_sum(a[j]);
  }
  const float inv = 1.f / den;
  if (gq == 0) {
    float4* dst = reinterpret_cast<float4*>(o + gl * VPL);
#pragma unroll
    for (int j = 0; j < VPL / 4; ++j)
      dst[j] = make_float4(a[4 * j] * inv, a[4 * j + 1] * inv, a[4 * j + 2] * inv, a[4 * j + 3] * inv);
  }
  if (p.lse != nullptr && lane == 0) p.lse[row] = (M + log2f(den)) * kLn2;
}

// Rows with few partials (the stream layout, where a segment spans one to a
// few ranges; the split layout with at most kGroupedMaxSplits splits): one
// row per wave would leave most lanes idle and the rows would take many
// rounds of waves, each paying its dependent round trips.  Here each 16-lane
// group of a wave takes its own row (rows 4 r .. 4 r + 3 of the flat
// [B, W, Hq] order), each lane D/16 consecutive columns, and folds the row's
// partials online, four partials' loads in flight at a time.  Partials past
// the row's count are dropped by selection.
template <int D, bool kStream>
__device__ __forceinline__ void combine_rows_grouped(const AttnParams& p, const StreamParams& sp,
                                                     unsigned block, unsigned nblocks, int waves) {
  constexpr int VPL = D / 16;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4, gl = lane & 15;
  const int wv = threadIdx.x >> 6;
  if (wv >= waves) return;  // uniform over the wave
  const size_t nrows = (size_t)p.B * p.W * p.Hq;
  // A wave takes rows 4 (i + k n) .. + 3 for k = 0, 1, ... (n = combine waves
  // of the launch): few workgroups, each kept busy, rather than one
  // workgroup per handful of rows (dispatching and retiring workgroups of the
  // step's finish launch costs more than their work).
  const size_t n = (size_t)nblocks * waves;
  for (size_t row0 = ((size_t)block * waves + wv) * 4; row0 < nrows; row0 += 4 * n) {
    const bool live = row0 + gq < nrows;
    const size_t row = live ? row0 + gq : row0;  // a group past the end repeats row 0, stores nothing
    const int h = (int)(row % p.Hq);
    const size_t bw = row / p.Hq;
    const int w = (int)(bw % p.W);
    const int b = (int)(bw / p.W);
    const int kvh = h / p.g;
    const int rho = w * p.g + (h - kvh * p.g);
    int ns;                // partials of the row (split layout: known once L is)
    size_t base, stride;   // row of partial s: base + s * stride
    if constexpr (kStream) {
      const int rb = rho / sp.rows_block;
      const int sigma = b * sp.nseg + kvh * p.nRB + rb;
      ns = sp.seg_info[2 * sigma + 1];
      base = (size_t)sp.seg_info[2 * sigma] * sp.rows_block + (rho - rb * sp.rows_block);
      stride = (size_t)sp.rows_block;
    } else {
      ns = 0;
      base = (((size_t)b * p.max_splits) * p.Hkv + kvh) * (size_t)p.R + rho;
      stride = (size_t)p.Hkv * p.R;
    }
    const int L = p.ctx_lens[b];

    // mask check once per distinct sequence of the wave's rows (the
    // visibility build needs the whole wave; its verdict is wave-uniform)
    bool ok = true;
    int prev_b = -1;
    bool prev_ok = true;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int bk = __shfl(b, 16 * k);
      bool okk = prev_ok;
      if (bk != prev_b) {
        node_visibility(p.mask_kind[bk], lane_mask_id(p, bk, lane), p.W, p.lookback, lane, okk);
        prev_b = bk;
        prev_ok = okk;
      }
      if (gq == k) ok = okk;
    }
    const bool ctx_ok = L >= 0 && L <= p.max_ctx;
    float* o = p.out + row * D + gl * VPL;
    if (!ok || !ctx_ok) {
      if (live) {
        if (gl == 0 && w == 0 && h == 0)
          raise_status((ok ? 0u : MTP_DEV_BAD_MASK) | (ctx_ok ? 0u : MTP_DEV_BAD_CTX));
#pragma unroll
        for (int j = 0; j < VPL; ++j) o[j] = qnan();
        if (p.lse != nullptr && gl == 0) p.lse[row] = qnan();
      }
      continue;
    }

    if constexpr (!kStream) ns = num_splits(p, L);
    float M = neg_inf(), den = 0.f;
    float a[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) a[j] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 4) {
      float ms[4], ls[4];
      float4 v[4][VPL / 4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sl = s0 + u < ns ? s0 + u : s0;  // in range; dropped below
        const size_t i = base + (size_t)sl * stride;
        ms[u] = p.part_ml[2 * i];
        ls[u] = p.part_ml[2 * i + 1];
        const float4* src = reinterpret_cast<const float4*>(p.part_acc + i * D + gl * VPL);
#pragma unroll
        for (int j = 0; j < VPL / 4; ++j) v[u][j] = src[j];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (s0 + u < ns) {
          const float mn = fmaxf(M, ms[u]);
          const float mu = mn == neg_inf() ? 0.f : mn;
          const float cold = fast_exp2(M - mu);
          const float cnew = fast_exp2(ms[u] - mu);
          den = den * cold + ls[u] * cnew;
#pragma unroll
          for (int j = 0; j < VPL / 4; ++j) {
            a[4 * j] = a[4 * j] * cold + v[u][j].x * cnew;
            a[4 * j + 1] = a[4 * j + 1] * cold + v[u][j].y * cnew;
            a[4 * j + 2] = a[4 * j + 2] * cold + v[u][j].z * cnew;
            a[4 * j + 3] = a[4 * j + 3] * cold + v[u][j].w * cnew;
          }
          M = mn;
        }
      }
    }
    if (live) {
      // Streaming stores: the output is not read again in this step, and
      // kept out of L2 it does not have to be written back at the launch
      // boundary (the ragged batch's step is ~8 us shorter).
      const float inv = 1.f / den;
      f32x4* dst = reinterpret_cast<f32x4*>(o);
#pragma unroll
      for (int j = 0; j < VPL / 4; ++j)
        __builtin_nontemporal_store(
            f32x4{a[4 * j] * inv, a[4 * j + 1] * inv, a[4 * j + 2] * inv, a[4 * j + 3] * inv}, dst + j);
      if (p.lse != nullptr && gl == 0) p.lse[row] = (M + log2f(den)) * kLn2;
    }
  }
}

// Stream layout with many pieces per segment (a few long sequences spread
// over the whole grid: a segment then has one piece per range it crosses,
// up to tens): one row per wave as in combine_rows, so that the row's pieces
// are loaded in parallel rather than folded four at a time.  Pass 1 takes
// the piece states over the lanes; pass 2 gives group q pieces q, q + 4, ...,
// eight of them in flight at a time.  Waves loop over rows.
template <int D>
__device__ __forceinline__ void combine_stream_rows(const AttnParams& p, const StreamParams& sp,
                                                    unsigned block, unsigned nblocks, int waves) {
  constexpr int VPL = D / 16;  // columns per lane
  constexpr int kBatch = 8;    // pieces per 16-lane group in flight
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4, gl = lane & 15;
  const int wv = threadIdx.x >> 6;
  if (wv >= waves) return;  // uniform over the wave
  const size_t nrows = (size_t)p.B * p.W * p.Hq;
  for (size_t row = (size_t)block * waves + wv; row < nrows; row += (size_t)nblocks * waves) {
    const int h = (int)(row % p.Hq);
    const size_t bw = row / p.Hq;
    const int w = (int)(bw % p.W);
    const int b = (int)(bw / p.W);
    const int kvh = h / p.g;
    const int rho = w * p.g + (h - kvh * p.g);
    const int rb = rho / sp.rows_block;
    const int sigma = b * sp.nseg + kvh * p.nRB + rb;
    const int ns = sp.seg_info[2 * sigma + 1];
    const size_t base = (size_t)sp.seg_info[2 * sigma] * sp.rows_block + (rho - rb * sp.rows_block);
    const size_t stride = (size_t)sp.rows_block;
    const int L = p.ctx_lens[b];
    bool ok;
    node_visibility(p.mask_kind[b], lane_mask_id(p, b, lane), p.W, p.lookback, lane, ok);
    const bool ctx_ok = L >= 0 && L <= p.max_ctx;
    float* o = p.out + row * D;
    if (!ok || !ctx_ok) {
      if (lane == 0 && w == 0 && h == 0)
        raise_status((ok ? 0u : MTP_DEV_BAD_MASK) | (ctx_ok ? 0u : MTP_DEV_BAD_CTX));
      for (int i = lane; i < D; i += kWave) o[i] = qnan();
      if (p.lse != nullptr && lane == 0) p.lse[row] = qnan();
      continue;
    }
    float M = neg_inf();
    for (int s = lane; s < ns; s += kWave) M = fmaxf(M, p.part_ml[2 * (base + s * stride)]);
    M = wave_max(M);
    float wl = 0.f;
    for (int s = lane; s < ns; s += kWave) {
      const size_t i = base + s * stride;
      wl += fast_exp2(p.part_ml[2 * i] - M) * p.part_ml[2 * i + 1];
    }
    const float den = wave_sum(wl);
    float a[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) a[j] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 4 * kBatch) {
      float wt[kBatch];
      float4 v[kBatch][VPL / 4];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int s = s0 + 4 * u + gq;
        const int sl = s < ns ? s : 0;  // in range; dropped by its zero weight below
        const size_t i = base + sl * stride;
        wt[u] = p.part_ml[2 * i];
        const float4* src = reinterpret_cast<const float4*>(p.part_acc + i * D + gl * VPL);
#pragma unroll
        for (int j = 0; j < VPL / 4; ++j) v[u][j] = src[j];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float wu = s0 + 4 * u + gq < ns ? fast_exp2(wt[u] - M) : 0.f;
#pragma unroll
        for (int j = 0; j < VPL / 4; ++j) {
          a[4 * j] = fmaf(wu, v[u][j].x, a[4 * j]);
          a[4 * j + 1] = fmaf(wu, v[u][j].y, a[4 * j + 1]);
          a[4 * j + 2] = fmaf(wu, v[u][j].z, a[4 * j + 2]);
          a[4 * j + 3] = fmaf(wu, v[u][j].w, a[4 * j + 3]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) a[j] = rows4_sum(a[j]);
    const float inv = 1.f / den;
    if (gq == 0) {
      f32x4* dst = reinterpret_cast<f32x4*>(o + gl * VPL);
#pragma unroll
      for (int j = 0; j < VPL / 4; ++j)
        __builtin_nontemporal_store(f32x4{a[4 * j] * inv, a[4 * j + 1] * inv, a[4 * j + 2] * inv,
                                          a[4 * j + 3] * inv},
                                    dst + j);
    }
    if (p.lse != nullptr && lane == 0) p.lse[row] = (M + log2f(den)) * kLn2;
  }
}

template <int D, bool kStream>
__global__ __launch_bounds__(256) void attn_combine(AttnParams p, StreamParams sp) {
  if constexpr (kStream) {
    if (sp.piece_rows) combine_stream_rows<D>(p, sp, blockIdx.x, gridDim.x, blockDim.x >> 6);
    else combine_rows_grouped<D, true>(p, sp, blockIdx.x, gridDim.x, blockDim.x >> 6);
  }
  else if (grouped_split_combine(p.max_splits, (long)p.B * p.W * p.Hq))
    combine_rows_grouped<D, false>(p, sp, blockIdx.x, gridDim.x, blockDim.x >> 6);
  else
    combine_rows<D>(p, blockIdx.x, blockDim.x >> 6);
}

// The step's second launch: one acceptance + commit workgroup per sequence
// (first, so that they are dispatched first: they hold the longest chain of
// dependent loads), then combine workgroups for every output row
// (combine_rows_per_block combine waves each).  The two
// parts touch disjoint data (the commit writes cache slots at or past each
// context length and ctx_lens_out, which must not alias the ctx_lens the
// combine reads), so they run side by side.  A combine workgroup takes
// combine_rows_per_block rows, chosen so that all workgroups fit on the
// compute units at once when the rows are few: the combine is bound by load
// latency, and a compute unit keeps only so many loads in flight.
template <int D, bool kStream>
__global__ __launch_bounds__(kAcceptThreads) void finish_kernel(AttnParams p, StreamParams sp, AcceptParams ap,
                                                     CommitParams cp, int combine_rows_per_block) {
  __shared__ int sm[kAcceptScratchInts];
  if ((int)blockIdx.x < p.B)
    accept_commit_seq(ap, cp, (int)blockIdx.x, sm);
  else if constexpr (kStream) {
    if (sp.piece_rows)
      combine_stream_rows<D>(p, sp, blockIdx.x - p.B, gridDim.x - p.B, combine_rows_per_block);
    else
      combine_rows_grouped<D, true>(p, sp, blockIdx.x - p.B, gridDim.x - p.B, combine_rows_per_block);
  }
  else
    combine_rows<D>(p, blockIdx.x - p.B, combine_rows_per_block);
}

}  // namespace mtpv
