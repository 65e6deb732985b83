// Split-K combine: merges the per-split partial softmax states of one output
// row (b, w, h) into out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s and
// lse = ln 2 * (M + log2 sum_s 2^(m_s - M) l_s).  Sequences with a malformed
// mask or context length get NaN rows.
//
// One wave per row.  Pass 1 spreads the splits over the lanes (one split per
// lane) for M and the denominator.  Pass 2 splits the wave into four groups of
// sixteen lanes: group q takes splits q, q+4, ..., each lane D/16 consecutive
// accumulators, so every load is 16-byte wide and many are in flight; the
// four group sums are folded with two shuffles.
#pragma once

#include "common.hpp"

namespace mtpv {

template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnParams p) {
  constexpr int VPL = D / 16;  // accumulators per lane per split
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4, gl = lane & 15;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)p.B * p.W * p.Hq) return;
  const int h = (int)(row % p.Hq);
  const size_t bw = row / p.Hq;
  const int w = (int)(bw % p.W);
  const int b = (int)(bw / p.W);
  const int kvh = h / p.g;
  const int rho = w * p.g + (h - kvh * p.g);

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
  const int ns = num_splits(L, p.S);
  const size_t base = (((size_t)b * p.max_splits) * p.Hkv + kvh) * (size_t)p.R + rho;
  const size_t sstride = (size_t)p.Hkv * p.R;

  // pass 1: reference max and denominator, one split per lane
  float M = neg_inf();
  for (int s = lane; s < ns; s += kWave) M = fmaxf(M, p.part_ml[2 * (base + s * sstride)]);
  M = wave_max(M);
  float wl = 0.f, wlane = 0.f;  // weight of split `lane` (first 64 splits)
  for (int s = lane; s < ns; s += kWave) {
    const size_t i = base + s * sstride;
    const float wt = fast_exp2(p.part_ml[2 * i] - M);
    if (s == lane) wlane = wt;
    wl += wt * p.part_ml[2 * i + 1];
  }
  const float den = wave_sum(wl);

  // pass 2: weighted accumulator sums, four groups of sixteen lanes
  float a[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) a[j] = 0.f;
  const int nfast = ns < kWave ? ns : kWave;
  for (int s0 = 0; s0 < nfast; s0 += 4) {  // splits whose weight sits in a lane
    const int s = s0 + gq;
    const float wt = __shfl(wlane, s & 63);
    if (s < nfast) {
      const float4* src = reinterpret_cast<const float4*>(p.part_acc + (base + s * sstride) * D + gl * VPL);
#pragma unroll
      for (int j = 0; j < VPL / 4; ++j) {
        const float4 v = src[j];
        a[4 * j] = fmaf(wt, v.x, a[4 * j]);
        a[4 * j + 1] = fmaf(wt, v.y, a[4 * j + 1]);
        a[4 * j + 2] = fmaf(wt, v.z, a[4 * j + 2]);
        a[4 * j + 3] = fmaf(wt, v.w, a[4 * j + 3]);
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
    a[j] += __shfl_xor(a[j], 16);
    a[j] += __shfl_xor(a[j], 32);
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

}  // namespace mtpv
