// Confidence-threshold and hybrid acceptance ("BitMTP: When Multi-Token
// Prediction Meets Low-Bit Large Language Models", Sec. 3.3; the threshold
// rule of "Dynamic Multi-Byte Prediction With Hierarchical Language Models",
// Sec. 3.1).  One workgroup per sequence.
//
// The waves take row tasks in turn: the drafter's probability of the drafted
// token at rows 1..W-1 (one pass over the row: online max and sum of 2^x in
// the log2 domain, then the drafted entry), and, when the verifier's logits
// are given, the argmax of rows 0..W-1.  Wave 0 then maps node i to lane i:
// the confidence prefix h is the depth of the deepest node whose whole root
// path is confident; with h >= m the step takes the h drafts (accepted
// length h - 1, path = root path of the deepest confident node's parent,
// bonus = that node's draft), otherwise the greedy verification result.
#pragma once

#include "accept_commit.hpp"

namespace mtpv {

struct HybridParams {
  const float* draft_logits;  // [B, W, V]: the drafter's distribution of each row's draft
  int32_t* conf_len;          // [B]: confidence prefix h (-1 for a malformed mask)
  float tau;                  // confidence threshold
  int min_prefix;             // m
};

// Merges the lanes' running (max, sum of 2^(x - max)) states of a row in the
// log2 domain; every lane returns the row's state.
__device__ __forceinline__ void merge_softmax_state(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float mo = __shfl_xor(m, o);
    const float so = __shfl_xor(s, o);
    const float mn = fmaxf(m, mo);
    const float mu = mn == neg_inf() ? 0.f : mn;  // two lanes without entries
    s = s * fast_exp2(m - mu) + so * fast_exp2(mo - mu);
    m = mn;
  }
}

// Folds four logits (already scaled by log2 e) into a lane's running state.
__device__ __forceinline__ void fold4(float& m, float& s, float a, float b, float c, float e) {
  const float mn = fmaxf(m, fmaxf(fmaxf(a, b), fmaxf(c, e)));
  s = s * fast_exp2(m - mn) + (fast_exp2(a - mn) + fast_exp2(b - mn)) +
      (fast_exp2(c - mn) + fast_exp2(e - mn));
  m = mn;
}

// Softmax probability of entry d of a V-long row, by one wave (0 when d is
// not a token id).  Each lane keeps a running maximum and a sum of 2^(x - max)
// over its entries in the log2 domain; the wave merges the lane states.
__device__ __forceinline__ float wave_row_prob(const float* row, int V, int d, bool vec) {
  const int lane = threadIdx.x & 63;
  float m = neg_inf();
  float s = 0.f;
  if (vec) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    const int n4 = V >> 2;
#pragma unroll 4
    for (int v = lane; v < n4; v += kWave) {
      const float4 x = r4[v];
      fold4(m, s, x.x * kLog2e, x.y * kLog2e, x.z * kLog2e, x.w * kLog2e);
    }
  } else {
    for (int v = lane; v < V; v += kWave) {
      const float a = row[v] * kLog2e;
      const float mn = fmaxf(m, a);
      s = s * fast_exp2(m - mn) + fast_exp2(a - mn);
      m = mn;
    }
  }
  merge_softmax_state(m, s);
  if (d < 0 || d >= V) return 0.f;
  return fast_exp2(row[d] * kLog2e - m) / s;
}

// The same for a row held in registers by load_reg_row; the drafted entry
// is taken from the lane that holds it.
__device__ __forceinline__ float reg_row_prob(const RegRow& r, int V, int d) {
  const int lane = threadIdx.x & 63;
  float m = neg_inf();
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kRegVec4; ++u) {
    if (lane + u * kWave < (V >> 2))
      fold4(m, s, r.x[u].x * kLog2e, r.x[u].y * kLog2e, r.x[u].z * kLog2e, r.x[u].w * kLog2e);
  }
  merge_softmax_state(m, s);
  if (d < 0 || d >= V) return 0.f;
  // float4 chunk c = d / 4 sits in lane c % 64, register c / 64; every
  // register is shuffled (no run-time register index, which would move the
  // row to scratch memory) and the one holding the chunk is kept.
  const int c = d >> 2;
  const int e = d & 3;
  float xe = 0.f;
#pragma unroll
  for (int u = 0; u < kRegVec4; ++u) {
    const float4 x = r.x[u];
    const float xu = __shfl(e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w, c % kWave);
    if (c / kWave == u) xe = xu;
  }
  return fast_exp2(xe * kLog2e - m) / s;
}

__global__ __launch_bounds__(kAcceptThreads) void accept_hybrid_kernel(AcceptParams ap, HybridParams hp) {
  __shared__ int s_conf[MTP_MAX_W];  // row i's draft is confident
  __shared__ int s_tgt[MTP_MAX_W];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int W = ap.W;
  Prefetch f{};
  if (threadIdx.x < kWave) f = prefetch_inputs(ap, nullptr, b);

  // Row tasks: t < W-1 is the confidence of row t+1; then (with logits) the
  // argmax of row t-(W-1).  Task t runs on wave t % waves.
  const int nconf = W - 1;
  const int ntask = nconf + (ap.logits != nullptr ? W : 0);
  const float* drows = hp.draft_logits + (size_t)b * W * ap.V;
  const float* lrows = ap.logits != nullptr ? ap.logits + (size_t)b * W * ap.V : nullptr;
  const int32_t* drafts = ap.draft_ids + (size_t)b * W;
  const bool dvec = rows_vec(hp.draft_logits, ap.V);
  const bool lvec = ap.logits != nullptr && rows_vec(ap.logits, ap.V);
  if (dvec && (ap.logits == nullptr || lvec) && ap.V <= kRegV) {
    constexpr int kRows = 2 * kRegRows;  // up to 2W - 1 tasks: twice the rows of a pass
    for (int t0 = wv; t0 < ntask; t0 += nw * kRows) {
      RegRow rr[kRows];
      int dr[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int t = t0 + r * nw;
        dr[r] = t < nconf ? drafts[t + 1] : -1;
        if (t < ntask)
          load_reg_row(t < nconf ? drows + (size_t)(t + 1) * ap.V : lrows + (size_t)(t - nconf) * ap.V,
                       ap.V, rr[r]);
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int t = t0 + r * nw;
        if (t < nconf) {
          const float pr = reg_row_prob(rr[r], ap.V, dr[r]);
          if (lane == 0) s_conf[t + 1] = (dr[r] >= 0 && dr[r] < ap.V && pr >= hp.tau) ? 1 : 0;
        } else if (t < ntask) {
          const int bi = reg_row_argmax(rr[r], ap.V);
          if (lane == 0) s_tgt[t - nconf] = bi;
        }
      }
    }
  } else {
    for (int t = wv; t < ntask; t += nw) {
      if (t < nconf) {
        const int d = drafts[t + 1];
        const float pr = wave_row_prob(drows + (size_t)(t + 1) * ap.V, ap.V, d, dvec);
        if (lane == 0) s_conf[t + 1] = (d >= 0 && d < ap.V && pr >= hp.tau) ? 1 : 0;
      } else {
        const int bi = wave_row_argmax(lrows + (size_t)(t - nconf) * ap.V, ap.V, lvec);
        if (lane == 0) s_tgt[t - nconf] = bi;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;

  const bool in = lane < W;
  const NodeTree tr = node_tree(f.kind, f.id, W);
  int32_t* path = ap.accept_path + (size_t)b * W;
  if (!tr.ok) {
    if (in) path[lane] = -1;
    if (lane == 0) {
      ap.accept_len[b] = -1;
      ap.bonus_id[b] = -1;
      hp.conf_len[b] = -1;
      raise_status(MTP_DEV_BAD_MASK);
    }
    return;
  }
  const bool conf = in && lane >= 1 && s_conf[lane] != 0;
  const int ckey = deepest_good(__ballot(conf), tr, W);
  const int h = ckey >> 6;
  const int cbest = 63 - (ckey & 63);
  if (h >= 1 && h >= hp.min_prefix) {
    const uint64_t ab = shfl64(tr.anc, cbest) & ~(1ull << cbest);  // root path of the parent
    const int dbest = __shfl(f.draft, cbest);
    write_path(ab, h - 1, W, path, nullptr);
    if (lane == 0) {
      ap.accept_len[b] = h - 1;
      ap.bonus_id[b] = dbest;
      hp.conf_len[b] = h;
    }
    return;
  }
  if (lane == 0) hp.conf_len[b] = h;
  if (ap.logits == nullptr) {  // the verifier is needed but its logits are absent
    if (in) path[lane] = -1;
    if (lane == 0) {
      ap.accept_len[b] = -1;
      ap.bonus_id[b] = -1;
    }
    return;
  }
  const bool match = in && lane >= 1 && f.draft >= 0 && f.draft == s_tgt[tr.par];
  const int key = deepest_good(__ballot(match), tr, W);
  const int best = 63 - (key & 63);
  const int len = key >> 6;
  write_path(shfl64(tr.anc, best), len, W, path, nullptr);
  if (lane == 0) {
    ap.accept_len[b] = len;
    ap.bonus_id[b] = s_tgt[best];
  }
}

}  // namespace mtpv
