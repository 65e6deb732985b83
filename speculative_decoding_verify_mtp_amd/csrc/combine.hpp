// Split-K combine: merges the per-split partial softmax states of one output
// row (b, w, h) into out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s and
// lse = ln 2 * (M + log2 sum_s 2^(m_s - M) l_s).  One wave per row; lanes
// span d.  Sequences with a malformed mask or context length get NaN rows.
#pragma once

#include "common.hpp"

namespace mtpv {

template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnParams p) {
  constexpr int PER = D / kWave;
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (size_t)p.B * p.W * p.Hq) return;
  const int h = (int)(row % p.Hq);
  const size_t bw = row / p.Hq;
  const int w = (int)(bw % p.W);
  const int b = (int)(bw / p.W);
  const int kvh = h / p.g;
  const int rho = w * p.g + (h - kvh * p.g);
  float* o = p.out + row * D + lane * PER;

  const int L = p.ctx_lens[b];
  bool ok;
  node_visibility(p.mask_kind[b], p.mask_ids + (size_t)b * p.W, p.W, p.lookback, lane, ok);
  const bool ctx_ok = L >= 0 && L <= p.max_ctx;
  if (!ok || !ctx_ok) {
    if (lane == 0 && w == 0 && h == 0) raise_status((ok ? 0u : MTP_DEV_BAD_MASK) | (ctx_ok ? 0u : MTP_DEV_BAD_CTX));
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = qnan();
    if (p.lse != nullptr && lane == 0) p.lse[row] = qnan();
    return;
  }
  const int ns = num_splits(L, p.S);
  const size_t base = (((size_t)b * p.max_splits) * p.Hkv + kvh) * (size_t)p.R + rho;
  const size_t sstride = (size_t)p.Hkv * p.R;

  float M = neg_inf();
  for (int s = lane; s < ns; s += kWave) M = fmaxf(M, p.part_ml[2 * (base + s * sstride)]);
  M = wave_max(M);
  float den = 0.f;
  for (int s = lane; s < ns; s += kWave) {
    const size_t i = base + s * sstride;
    den += fast_exp2(p.part_ml[2 * i] - M) * p.part_ml[2 * i + 1];
  }
  den = wave_sum(den);

  float a[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) a[i] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t i = base + s * sstride;
    const float wgt = fast_exp2(p.part_ml[2 * i] - M);
    const float* src = p.part_acc + i * D + lane * PER;
#pragma unroll
    for (int k = 0; k < PER; ++k) a[k] = fmaf(wgt, src[k], a[k]);
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = a[i] * inv;
  if (p.lse != nullptr && lane == 0) p.lse[row] = (M + log2f(den)) * kLn2;
}

}  // namespace mtpv
