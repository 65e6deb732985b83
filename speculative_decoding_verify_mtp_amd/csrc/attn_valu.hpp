// Split-K verify attention on the vector ALUs, for fp32 inputs and for bf16
// heads whose W * g rows are too few (< 16) to fill an MFMA tile.
//
// One wave = one work item: (sequence, KV head, chunk of RC rows, split).
// The wave is cut into KG key groups of LPK = D/16 lanes; a key group walks
// its own keys (key k0 + kg each step) and each of its lanes owns 16
// consecutive elements of d.  A lane group keeps its own online-softmax state
// per row; the KG states are merged with shuffles at the end of the item.
#pragma once

#include "common.hpp"

namespace mtpv {

template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&x)[16]);

template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&x)[16]) {
  const float4* s = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = s[i];
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
}

template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* p, float (&x)[16]) {
  const uint4* s = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 v = s[i];
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}

constexpr int kValuRows = 4;  // rows per work item

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_partial_valu(AttnParams p) {
  constexpr int LPK = D / 16;
  constexpr int KG = kWave / LPK;
  constexpr int RC = kValuRows;
  const int lane = threadIdx.x & 63;
  const int kg = lane / LPK;
  const int sub = lane % LPK;
  const int b = blockIdx.y;
  const Item it = decode_item(blockIdx.x * 4 + (threadIdx.x >> 6), p);
  if (it.split >= p.max_splits) return;
  const int start = split_start(p, it.split);
  // Loads that do not depend on the context length go out together with it:
  // the split's page indices (lane i holding entries i and 64 + i; a split
  // spans at most 128 pages; bounded by the block table, not by the
  // context), the mask description and, below, Q.
  const int32_t* btrow = p.block_table + (size_t)b * p.max_pages;
  const int pbase = start >> 4;
  const int pavail = p.max_pages - pbase;
  const int pr0 = lane < pavail ? btrow[pbase + lane] : 0;
  const int pr1 = lane + 64 < pavail ? btrow[pbase + lane + 64] : 0;
  const int mkind = p.mask_kind[b];
  const int mid = lane_mask_id(p, b, lane);

  const T* qbase = static_cast<const T*>(p.q);
  const T* kc = static_cast<const T*>(p.k_cache) + (size_t)it.kvh * D + sub * 16;
  const T* vc = static_cast<const T*>(p.v_cache) + (size_t)it.kvh * D + sub * 16;
  const T* kn = static_cast<const T*>(p.k_new) + (size_t)it.kvh * D + sub * 16;
  const T* vn = static_cast<const T*>(p.v_new) + (size_t)it.kvh * D + sub * 16;
  const size_t slot_stride = (size_t)p.Hkv * D;

  float qv[RC][16];
#pragma unroll
  for (int r = 0; r < RC; ++r) {
    const int rho = it.rb * RC + r;
    if (rho < p.R) {
      const int w = rho / p.g;
      const int j = rho - w * p.g;
      load16<T>(qbase + ((size_t)(b * p.W + w) * p.Hq + (size_t)it.kvh * p.g + j) * D + sub * 16,
                qv[r]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) qv[r][i] = 0.f;
    }
  }

  const int L = p.ctx_lens[b];
  if (L < 0 || L > p.max_ctx) return;
  const int ns = num_splits(p, L);
  if (it.split >= ns) return;
  const int end = min(L, split_start(p, it.split + 1));
  const bool last = it.split == ns - 1;

  // In-block visibility rows of this item's rows (last split only).
  int ntail = 0;
  uint64_t vrow[RC];
#pragma unroll
  for (int r = 0; r < RC; ++r) vrow[r] = 0;
  if (last) {
    bool ok;
    const uint64_t vnode =
        node_visibility(mkind, mid, p.W, p.lookback, lane, ok);
    if (ok) {
      ntail = p.W;
#pragma unroll
      for (int r = 0; r < RC; ++r) {
        const int rho = min(it.rb * RC + r, p.R - 1);
        vrow[r] = shfl64(vnode, rho / p.g);
      }
    }
  }

  float m[RC], l[RC], acc[RC][16];
#pragma unroll
  for (int r = 0; r < RC; ++r) {
    m[r] = neg_inf();
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
  }

  const int ncomm = end - start;
  const int n = ncomm + ntail;
  bool bad = false;
  for (int k0 = 0; k0 < n; k0 += KG) {
    const int kk = k0 + kg;
    const bool valid = kk < n;
    // the page of key kk from the split's page list (pr0, pr1 above): one
    // memory round trip per step instead of two.  The shuffle runs with the
    // whole wave active (the list lanes are not those of the key).
    const int pi = ((start + min(kk, max(ncomm - 1, 0))) >> 4) - pbase;
    const int a0 = __shfl(pr0, pi & 63);
    const int a1 = __shfl(pr1, pi & 63);
    const T* kp;
    const T* vp;
    int jb = -1;  // in-block key index, -1 for committed keys
    if (kk < ncomm) {
      const int t = start + kk;
      int pg = pi < 64 ? a0 : a1;
      if ((unsigned)pg >= (unsigned)p.num_pages) {
        bad = true;
        pg = 0;
      }
      const size_t off = ((size_t)pg * kPage + (t & 15)) * slot_stride;
      kp = kc + off;
      vp = vc + off;
    } else {
      const int j = valid ? kk - ncomm : 0;
      jb = j;
      const size_t off = (size_t)(b * p.W + j) * slot_stride;
      kp = kn + off;
      vp = vn + off;
    }
    float kf[16], vf[16];
    load16<T>(kp, kf);
    load16<T>(vp, vf);
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s = fmaf(qv[r][i], kf[i], s);
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) s += __shfl_xor(s, o);
      s = mul_rn(s, p.scale_log2);  // the max and the exponent see the same rounded score
      const bool vis = valid && (jb < 0 || ((vrow[r] >> jb) & 1ull) != 0ull);
      if (vis) {
        const float mn = fmaxf(m[r], s);
        const float cf = fast_exp2(m[r] - mn);
        const float pp = fast_exp2(s - mn);
        l[r] = l[r] * cf + pp;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][i] = fmaf(acc[r][i], cf, pp * vf[i]);
        m[r] = mn;
      }
    }
  }

  // Merge the KG key-group states.
#pragma unroll
  for (int o = LPK; o < kWave; o <<= 1) {
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      const float mo = __shfl_xor(m[r], o);
      const float lo = __shfl_xor(l[r], o);
      const float mm = fmaxf(m[r], mo);
      const float mu = mm == neg_inf() ? 0.f : mm;
      const float c1 = fast_exp2(m[r] - mu);
      const float c2 = fast_exp2(mo - mu);
      l[r] = l[r] * c1 + lo * c2;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][i] = acc[r][i] * c1 + __shfl_xor(acc[r][i], o) * c2;
      m[r] = mm;
    }
  }

  if (__ballot(bad) != 0ull) {
    if (lane == 0) raise_status(MTP_DEV_BAD_PAGE);
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      m[r] = qnan();
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][i] = qnan();
    }
  }

  if (kg == 0) {
#pragma unroll
    for (int r = 0; r < RC; ++r) {
      const int rho = it.rb * RC + r;
      if (rho < p.R) {
        const size_t pidx =
            (((size_t)b * p.max_splits + it.split) * p.Hkv + it.kvh) * (size_t)p.R + rho;
        if (sub == 0) {
          p.part_ml[2 * pidx] = m[r];
          p.part_ml[2 * pidx + 1] = l[r];
        }
        float4* dst = reinterpret_cast<float4*>(p.part_acc + pidx * D + sub * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[i] = make_float4(acc[r][4 * i], acc[r][4 * i + 1], acc[r][4 * i + 2], acc[r][4 * i + 3]);
      }
    }
  }
}

}  // namespace mtpv
