// Dynamic token tree for the next verify block ("Efficient Training-Free
// Multi-Token Prediction via Embedding-Space Probing", Sec. 2.C and 2.D).
// One workgroup per sequence.
//
// 1. Ranked lists: the waves take the probed depths in turn; for depth d a
//    wave extracts the first n = slots + 1 tokens of p_d in the order
//    (probability descending, id ascending) into LDS.  One token of a list
//    may be the parent's and is skipped later, so slots + 1 entries always
//    suffice.  Each round takes every lane's best entry ranked below the
//    previous pick, then the wave's best of those; with V <= 1024 the lane's
//    16 entries (ids lane + 64 j) stay in registers, larger vocabularies
//    rescan the row.
// 2. Spine: wave 0 walks the depths in order: the top-1 token of depth d is
//    the first list entry that differs from the spine token above, and
//    c_d = c_{d-1} * p_d(spine) (fp32, in this order).
// 3. Best-first expansion without rounds: a parent's cumulative probability
//    is never below its children's (and ties go to the shallower), so the
//    best-first order is one global order of all candidates by (c_{d-1} * p,
//    depth, rank).  Each thread takes candidates and counts the candidates
//    above them (a bisection per depth list: the keys of a list decrease
//    along it); the count is the candidate's row - 1.  Rows past the
//    prediction budget or below min_cum_prob are dropped.
// 4. Parents (the row of the top-1 node of the depth above), the root row and
//    the mask-token rows, chained from the deepest chosen top-1 node.
#pragma once

#include "common.hpp"

namespace mtpv {

constexpr int kTreeMaxK = 64;
constexpr int kTreeMaxList = MTP_MAX_W;  // slots + 1 <= W <= 64
constexpr int kTreeRegElems = 16;        // entries per lane on the register path
constexpr int kTreeRegV = kWave * kTreeRegElems;

struct TreeParams {
  const float* probs;      // [B, K, V]
  const int32_t* root;     // [B]
  int32_t* draft;          // [B, W]
  int32_t* parent;         // [B, W]
  int32_t* depth;          // [B, W]
  int32_t* n_nodes;        // [B]
  float min_cum_prob;
  int B, K, V, W, n_mask;
};

// (p, i) ranks above (q, j): more probable, or as probable with a smaller id.
// Bitwise operators: no short-circuit branches in the unrolled scans.
__device__ __forceinline__ bool rank_above(float p, int i, float q, int j) {
  return (p > q) | ((p == q) & (i < j));
}

// Wave argmax of (p, i) by rank (every lane gets the winner).
__device__ __forceinline__ void wave_best(float& p, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float q = __shfl_xor(p, o);
    const int j = __shfl_xor(i, o);
    const bool take = rank_above(q, j, p, i);
    p = take ? q : p;
    i = take ? j : i;
  }
}

// The first n entries of one probability row by rank into (tok, prb);
// entries past the vocabulary get token -1, probability -1.
template <bool kRegs>
__device__ __forceinline__ void ranked_list(const float* row, int V, int n, int* tok, float* prb) {
  const int lane = threadIdx.x & 63;
  if constexpr (kRegs) {
    float p[kTreeRegElems];
#pragma unroll
    for (int j = 0; j < kTreeRegElems; ++j) {
      const int i = lane + kWave * j;
      p[j] = row[min(i, V - 1)];  // unconditional (in-bounds) load, then select
      p[j] = i < V ? p[j] : -1.f;
    }
    // each round: every lane's best entry below the previous pick, then the
    // wave's best of those
    float pp = __builtin_inff();
    int pi = -1;
    for (int r = 0; r < n; ++r) {
      float bp = -1.f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kTreeRegElems; ++j) {
        const int i = lane + kWave * j;
        const bool take = (p[j] >= 0.f) & rank_above(pp, pi, p[j], i) & rank_above(p[j], i, bp, bi);
        bp = take ? p[j] : bp;
        bi = take ? i : bi;
      }
      wave_best(bp, bi);
      if (lane == 0) {
        tok[r] = bp >= 0.f ? bi : -1;
        prb[r] = bp >= 0.f ? bp : -1.f;
      }
      pp = bp;
      pi = bi;
    }
  } else {
    float pp = __builtin_inff();
    int pi = -1;
    for (int r = 0; r < n; ++r) {
      float bp = -1.f;
      int bi = 0x7fffffff;
      for (int i = lane; i < V; i += kWave) {
        const float x = row[i];
        const bool below = rank_above(pp, pi, x, i);
        if (below && rank_above(x, i, bp, bi)) {
          bp = x;
          bi = i;
        }
      }
      wave_best(bp, bi);
      if (lane == 0) {
        tok[r] = bp >= 0.f ? bi : -1;
        prb[r] = bp >= 0.f ? bp : -1.f;
      }
      pp = bp;
      pi = bi;
    }
  }
}

// Number of entries of depth list e (sorted, most probable first) whose key
// (cumulative probability c * prb, then depth, then rank among the unpruned
// entries) is above the target's; the pruned entry (index `pi`, n if none)
// does not count.  The keys of a list decrease along it, so the entries
// above form a prefix, found by bisection.
__device__ __forceinline__ int count_above(const int* tok, const float* prb, int n, int e, float c,
                                           int pi, float tcp, int td, int tr) {
  int lo = 0, hi = n;  // entries [0, lo) are above, [hi, n) are not
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const float cp = tok[mid] >= 0 ? c * prb[mid] : -1.f;
    bool above;
    if (cp != tcp)
      above = cp > tcp;
    else if (e != td)
      above = e < td;
    else
      above = mid - (pi < mid ? 1 : 0) < tr;
    if (above)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo - (pi < lo ? 1 : 0);
}

__global__ __launch_bounds__(1024) void tree_build_kernel(TreeParams p) {
  __shared__ int s_tok[kTreeMaxK][kTreeMaxList];
  __shared__ float s_prb[kTreeMaxK][kTreeMaxList];
  __shared__ int s_skip[kTreeMaxK];    // the pruned token of depth d + 1 (the spine above)
  __shared__ int s_pidx[kTreeMaxK];    // its index in the list (n if absent)
  __shared__ float s_cpar[kTreeMaxK];  // c of the depth above
  __shared__ int s_spine_row[kTreeMaxK];
  __shared__ int s_row_depth[MTP_MAX_W];
  __shared__ int s_nsel, s_deep;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int W = p.W;
  const int slots = W - 1 - p.n_mask;
  const int n = slots + 1;
  const int K = p.K;
  const int root = p.root[b];

  // 1. ranked lists
  if (slots > 0) {
    for (int d = wv; d < K; d += nw) {
      const float* row = p.probs + ((size_t)b * K + d) * p.V;
      if (p.V <= kTreeRegV)
        ranked_list<true>(row, p.V, n, s_tok[d], s_prb[d]);
      else
        ranked_list<false>(row, p.V, n, s_tok[d], s_prb[d]);
    }
  }
  if (threadIdx.x < kTreeMaxK) s_spine_row[threadIdx.x] = -1;
  if (threadIdx.x == 0) {
    s_nsel = 0;
    s_deep = 0;
  }
  __syncthreads();

  // 2. spine tokens and cumulative probabilities: lane l of wave 0 walks the
  //    depths in order (all lanes alike) and keeps what depth l + 1 needs
  if (threadIdx.x < kWave && slots > 0) {
    const int d = lane + 1;
    int sp = root;
    float c = 1.f;
    for (int e = 1; e <= K && e <= d; ++e) {
      const int first = s_tok[e - 1][0] == sp ? 1 : 0;
      const int t = first < n ? s_tok[e - 1][first] : -1;
      const float q = first < n ? s_prb[e - 1][first] : -1.f;
      if (e == d) {
        s_skip[d - 1] = sp;
        s_cpar[d - 1] = c;  // -1 when a depth above has no top-1 node
        int pidx = n;
        for (int k = 0; k < n; ++k)
          if (s_tok[d - 1][k] == sp && sp >= 0) pidx = k;
        s_pidx[d - 1] = pidx;
      }
      sp = t;
      c = t >= 0 && c >= 0.f ? c * q : -1.f;
    }
  }
  __syncthreads();

  // 3. every candidate's place in the best-first order = the number of
  //    candidates above it (best first by cumulative probability equals one
  //    global sort: a parent is never below its children)
  const int ncand = slots > 0 ? K * n : 0;
  for (int ci = threadIdx.x; ci < ncand; ci += blockDim.x) {
    const int d = ci / n, j = ci - d * n;
    const int t = s_tok[d][j];
    const float c = s_cpar[d];
    if (t < 0 || t == s_skip[d] || c < 0.f) continue;
    const float cp = c * s_prb[d][j];
    if (cp < p.min_cum_prob) continue;
    const int r = j - (s_pidx[d] < j ? 1 : 0);
    int rank = 0;
    for (int e = 0; e < K; ++e)
      if (s_cpar[e] >= 0.f) rank += count_above(s_tok[e], s_prb[e], n, e, s_cpar[e], s_pidx[e], cp, d, r);
    if (rank >= slots) continue;
    const int row = 1 + rank;
    atomicMax(&s_nsel, row);
    if (r == 0) {  // the top-1 node of depth d + 1: its children's parent
      s_spine_row[d] = row;
      atomicMax(&s_deep, d + 1);
    }
    p.draft[(size_t)b * W + row] = t;
    p.depth[(size_t)b * W + row] = d + 1;
    s_row_depth[row] = d + 1;
  }
  __syncthreads();

  // 4. parents of the chosen rows, the root, the mask-token chain
  const int nsel = s_nsel;  // the last chosen row
  for (int row = 1 + threadIdx.x; row <= nsel; row += blockDim.x) {
    const int d = s_row_depth[row];
    p.parent[(size_t)b * W + row] = d == 1 ? 0 : s_spine_row[d - 2];
  }
  if (threadIdx.x == 0) {
    int32_t* dr = p.draft + (size_t)b * W;
    int32_t* pr = p.parent + (size_t)b * W;
    int32_t* dp = p.depth + (size_t)b * W;
    dr[0] = root;
    pr[0] = -1;
    dp[0] = 0;
    const int deep = s_deep;
    int tail = deep > 0 ? s_spine_row[deep - 1] : 0;
    int tdepth = deep;
    for (int i = nsel + 1; i < W; ++i) {
      dr[i] = -1;
      pr[i] = tail;
      dp[i] = tdepth + 1;
      tail = i;
      tdepth += 1;
    }
    p.n_nodes[b] = nsel + 1;
  }
}

}  // namespace mtpv
