// Dynamic token tree for the next verify block ("Efficient Training-Free
// Multi-Token Prediction via Embedding-Space Probing", Sec. 2.C and 2.D).
// One workgroup per sequence.
//
// 1. Ranked lists (tree_lists_kernel, one workgroup per depth and
//    sequence): the first n = slots + 1 tokens of p_d in the order
//    (probability descending, id ascending).  One token of a list may be the
//    parent's and is skipped later, so slots + 1 entries always suffice.
//    A radix selection of the n-th largest (probability, -id) key, then the
//    n keys above it ordered by counting (see tree_lists_kernel; V <= 4096).
//    The lists go through a workspace to tree_build_kernel (one workgroup
//    per sequence), which does 2-4.
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

struct TreeParams {
  const float* probs;      // [B, K, V]
  const int32_t* root;     // [B]
  int32_t* draft;          // [B, W]
  int32_t* parent;         // [B, W]
  int32_t* depth;          // [B, W]
  int32_t* n_nodes;        // [B]
  int* list_tok;           // workspace [B, K, n]
  float* list_prb;         // workspace [B, K, n]
  float min_cum_prob;
  int B, K, V, W, n_mask;
};

constexpr int kTreeListThreads = 256;
constexpr int kTreeListElems = 16;  // entries per thread: V <= 4096
constexpr int kTreeMaxV = kTreeListThreads * kTreeListElems;

// Ranked list of one (sequence, depth) by radix selection, one workgroup
// per (depth, sequence).  Entry (p, i) gets the 64-bit key
// (bits of p) << 32 | ~i: p >= 0, so a larger key ranks higher (more
// probable, then smaller id) and every key is distinct and non-zero.  Eight
// passes over 8-bit digits, most significant first, find the k-th largest
// key (k = min(n, V)): each pass histograms the digit of the keys that match
// the digits found so far (LDS atomics) and wave 0 walks the bins from the
// top.  The passes stop early once the selected bin holds exactly the keys
// still to be taken (the lower digits then change nothing: every key with
// the prefix is among the k).  The k keys at or above the prefix are then
// appended to LDS and put in order by counting, for each, the keys above it.
__global__ __launch_bounds__(kTreeListThreads) void tree_lists_kernel(TreeParams p) {
  __shared__ int s_hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_k, s_cnt, s_cbin;
  __shared__ unsigned long long s_key[kTreeMaxList];
  const int d = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = p.W - p.n_mask;  // slots + 1
  const float* row = p.probs + ((size_t)b * p.K + d) * p.V;
  unsigned long long key[kTreeListElems];
#pragma unroll
  for (int j = 0; j < kTreeListElems; ++j) {
    const int i = tid + kTreeListThreads * j;
    const float x = row[min(i, p.V - 1)];
    key[j] = i < p.V ? ((unsigned long long)__float_as_uint(x) << 32) | (unsigned)(~i) : 0ull;
  }
  const int kk = min(n, p.V);
  unsigned long long prefix = 0ull;
  int k = kk;
  for (int pass = 7; pass >= 0; --pass) {
    s_hist[tid] = 0;
    __syncthreads();
    const int sh = 8 * pass;
    const unsigned long long hmask = pass == 7 ? 0ull : (~0ull << (sh + 8));
#pragma unroll
    for (int j = 0; j < kTreeListElems; ++j)
      if (key[j] != 0ull && (key[j] & hmask) == (prefix & hmask))
        atomicAdd(&s_hist[(int)((key[j] >> sh) & 255ull)], 1);
    __syncthreads();
    if (tid < kWave) {
      // lane l takes bins 255 - 4l, ..., 252 - 4l (from the top)
      int c[4], sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c[u] = s_hist[255 - 4 * lane - u];
        sum += c[u];
      }
      int incl = sum;  // inclusive scan over lanes
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const int before = incl - sum;
      if (before < k && k <= incl) {
        int acc = before;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (acc < k && k <= acc + c[u]) {
            s_prefix = prefix | ((unsigned long long)(255 - 4 * lane - u) << sh);
            s_k = k - acc;
            s_cbin = c[u];
          }
          acc += c[u];
        }
      }
    }
    __syncthreads();
    prefix = s_prefix;
    k = s_k;
    if (k == s_cbin) break;  // the whole bin is taken (uniform: read from LDS)
  }
  // the kk keys at or above the kk-th largest
  if (tid == 0) s_cnt = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTreeListElems; ++j)
    if (key[j] != 0ull && key[j] >= prefix) s_key[atomicAdd(&s_cnt, 1)] = key[j];
  __syncthreads();
  int* out_tok = p.list_tok + ((size_t)b * p.K + d) * n;
  float* out_prb = p.list_prb + ((size_t)b * p.K + d) * n;
  if (tid < kk) {
    const unsigned long long mine = s_key[tid];
    int r = 0;
    for (int t = 0; t < kk; ++t) r += s_key[t] > mine ? 1 : 0;
    out_tok[r] = (int)(~(unsigned)(mine & 0xffffffffull));
    out_prb[r] = __uint_as_float((unsigned)(mine >> 32));
  } else if (tid < n) {
    out_tok[tid] = -1;
    out_prb[tid] = -1.f;
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
  const int W = p.W;
  const int slots = W - 1 - p.n_mask;
  const int n = slots + 1;
  const int K = p.K;
  const int root = p.root[b];

  // 1. ranked lists (tree_lists_kernel) into LDS
  if (slots > 0) {
    for (int e = threadIdx.x; e < K * n; e += blockDim.x) {
      const int d = e / n, r = e - d * n;
      s_tok[d][r] = p.list_tok[((size_t)b * K + d) * n + r];
      s_prb[d][r] = p.list_prb[((size_t)b * K + d) * n + r];
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
