// Greedy acceptance and KV commit.  One workgroup per sequence.
//
// Acceptance: the waves take the block rows in turn and reduce the argmax
// of each row's logits (smallest id on ties).  Wave 0 then maps block node i
// to lane i: match_i = (draft_i >= 0 and draft_i == target[parent_i]); the
// node is accepted when every node on its root path matches, i.e. when its
// ancestor-or-self bit row has no non-matching node; the accepted node is the
// deepest such node (smallest index on ties), found by one wave max over
// depth * 64 + (63 - i).  The root path is the bit row of that node, so lane
// i writes itself to path position popcount(bits below i).
//
// Commit: lanes of wave 0 validate one path position each (row index, page
// mapping); then all threads copy the accepted rows in 16-byte chunks.  A
// K/V row of one token is Hkv * D contiguous elements both in k_new and in a
// cache slot, so each accepted position is one contiguous copy.
#pragma once

#include "common.hpp"

namespace mtpv {

struct AcceptParams {
  const float* logits;  // [B, W, V]
  const int32_t* tgt = nullptr;  // [B, W] row argmaxes already found (nullptr: from logits)
  const int32_t* draft_ids;
  const uint8_t* mask_kind;
  const int32_t* mask_ids;
  int32_t* accept_len;
  int32_t* accept_path;
  int32_t* bonus_id;
  int B, W, V;
};

struct CommitParams {
  const void* k_new;
  const void* v_new;
  const int32_t* accept_len;   // read when the acceptance is not fused
  const int32_t* accept_path;  // read when the acceptance is not fused
  const int32_t* block_table;
  const int32_t* ctx_in;
  int32_t* ctx_out;
  void* k_cache;
  void* v_cache;
  int skip_root;
  int W, max_pages, num_pages;
  int row_bytes;  // Hkv * D * element size, a multiple of 16
};

// Inputs of wave 0 loaded before the argmax, so that their latency overlaps
// the logits stream: this lane's mask id and draft id, the mask kind, and for
// the commit the context length; the page of slot ctx + lane follows once the
// context length is back (commit_page).
struct Prefetch {
  int kind, id, draft, L, page;
};

__device__ __forceinline__ Prefetch prefetch_inputs(const AcceptParams& ap, const CommitParams* cp, int b) {
  const int lane = threadIdx.x & 63;
  const int W = ap.W;
  Prefetch f;
  f.kind = ap.mask_kind[b];
  f.id = lane < W ? ap.mask_ids[(size_t)b * W + lane] : 0;
  f.draft = lane < W ? ap.draft_ids[(size_t)b * W + lane] : -1;
  f.L = cp != nullptr ? cp->ctx_in[b] : 0;
  f.page = -1;
  return f;
}

// Page of the commit slot ctx + lane (-1 past the block, the table or for a
// negative context length).
__device__ __forceinline__ int commit_page(const CommitParams& cp, int b, int L) {
  const int lane = threadIdx.x & 63;
  const int pi = (L + lane) >> 4;
  return (lane < cp.W && L >= 0 && pi < cp.max_pages) ? cp.block_table[(size_t)b * cp.max_pages + pi] : -1;
}

// Argmax of one logits row by one wave (smallest id on ties); 16-byte
// loads when `vec` (V % 4 == 0 and a 16-byte aligned base).
__device__ __forceinline__ int wave_row_argmax(const float* row, int V, bool vec) {
  const int lane = threadIdx.x & 63;
  float bv = neg_inf();
  int bi = 0x7fffffff;
  if (vec) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    const int n4 = V >> 2;
#pragma unroll 4
    for (int v = lane; v < n4; v += kWave) {
      const float4 x = r4[v];
      const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (xs[e] > bv || bi == 0x7fffffff) {
          bv = xs[e];
          bi = 4 * v + e;
        }
      }
    }
  } else {
    for (int v = lane; v < V; v += kWave) {
      const float x = row[v];
      if (x > bv || bi == 0x7fffffff) {
        bv = x;
        bi = v;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  return bi;
}

__device__ __forceinline__ bool rows_vec(const float* base, int V) {
  return (V & 3) == 0 && ((uintptr_t)base & 15) == 0;
}

// Rows of at most kRegV floats (16-byte aligned, V % 4 == 0) are reduced from
// registers: a wave first issues the loads of up to kRegRows rows (lane l
// holds the float4 chunks l, l + 64, ...), then reduces them one by one, so
// that the load latency is paid once per pass instead of once per row.
constexpr int kRegVec4 = 4;
constexpr int kRegV = kWave * 4 * kRegVec4;
constexpr int kRegRows = 2;

// Threads of the acceptance workgroups: 16 waves, so that one register pass
// (16 x kRegRows rows) covers blocks of up to 32 rows.
constexpr int kAcceptThreads = 1024;

struct RegRow {
  float4 x[kRegVec4];
};

__device__ __forceinline__ void load_reg_row(const float* row, int V, RegRow& r) {
  const int lane = threadIdx.x & 63;
  const float4* r4 = reinterpret_cast<const float4*>(row);
#pragma unroll
  for (int u = 0; u < kRegVec4; ++u) {
    const int v = lane + u * kWave;
    if (v < (V >> 2)) r.x[u] = r4[v];
  }
}

// Argmax of a row held by load_reg_row (smallest id on ties).
__device__ __forceinline__ int reg_row_argmax(const RegRow& r, int V) {
  const int lane = threadIdx.x & 63;
  float bv = neg_inf();
  int bi = 0x7fffffff;
#pragma unroll
  for (int u = 0; u < kRegVec4; ++u) {
    const int v = lane + u * kWave;
    if (v < (V >> 2)) {
      const float xs[4] = {r.x[u].x, r.x[u].y, r.x[u].z, r.x[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (xs[e] > bv || bi == 0x7fffffff) {
          bv = xs[e];
          bi = 4 * v + e;
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  return bi;
}

// Argmax of every block row into s_tgt[0..W).  All waves take part, row i
// on wave i % waves.  `mid()` runs once per thread, right after the loads of
// the thread's first register pass are issued (at the start otherwise): loads
// it issues queue behind the logits, not in front of them.
template <typename Mid>
__device__ __forceinline__ void block_argmax(const AcceptParams& p, int b, int* s_tgt, Mid mid) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  if (p.tgt != nullptr) {  // found by the launch before (the step's target prologue)
    int t = 0;
    if (wv == 0 && lane < p.W) t = p.tgt[(size_t)b * p.W + lane];
    mid();
    if (wv == 0 && lane < p.W) s_tgt[lane] = t;
    return;
  }
  const bool vec = rows_vec(p.logits, p.V);
  const float* base = p.logits + (size_t)b * p.W * p.V;
  if (vec && p.V <= kRegV) {
    bool mid_done = false;  // wave-uniform
    for (int i0 = wv; i0 < p.W; i0 += nw * kRegRows) {
      RegRow rr[kRegRows];
#pragma unroll
      for (int r = 0; r < kRegRows; ++r) {
        const int i = i0 + r * nw;
        if (i < p.W) load_reg_row(base + (size_t)i * p.V, p.V, rr[r]);
      }
      if (!mid_done) {
        mid();
        mid_done = true;
      }
#pragma unroll
      for (int r = 0; r < kRegRows; ++r) {
        const int i = i0 + r * nw;
        if (i < p.W) {
          const int bi = reg_row_argmax(rr[r], p.V);
          if (lane == 0) s_tgt[i] = bi;
        }
      }
    }
    if (!mid_done) mid();
    return;
  }
  mid();
  for (int i = wv; i < p.W; i += nw) {
    const int bi = wave_row_argmax(base + (size_t)i * p.V, p.V, vec);
    if (lane == 0) s_tgt[i] = bi;
  }
}

__device__ __forceinline__ void block_argmax(const AcceptParams& p, int b, int* s_tgt) {
  block_argmax(p, b, s_tgt, [] {});
}

// Acceptance structure of block node `lane` (wave 0, lane = node): its
// ancestor-or-self bit row and its parent (0 for the root and for lanes past
// the block).  CHAIN and SEGMENT blocks accept by index order, TREE blocks
// along parent pointers.  `ok` is false for a malformed mask description.
struct NodeTree {
  uint64_t anc;
  int par;
  bool ok;
};

__device__ __forceinline__ NodeTree node_tree(int kind, int id, int W) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < W;
  NodeTree t;
  if (kind == MTP_MASK_TREE) {
    t.anc = node_visibility(kind, id, W, -1, lane, t.ok);
    t.par = (in && lane >= 1 && t.ok) ? id : 0;
  } else {
    node_visibility(kind, id, W, -1, lane, t.ok);  // validates the description
    t.anc = in ? (~0ull >> (63 - lane)) : 0ull;
    t.par = lane >= 1 ? lane - 1 : 0;
  }
  return t;
}

// Deepest node whose whole root path is in `good_bits` (bit 0, the root, is
// always taken), smallest index on ties, packed as depth * 64 + (63 - node).
__device__ __forceinline__ int deepest_good(uint64_t good_bits, const NodeTree& t, int W) {
  const int lane = threadIdx.x & 63;
  const bool good = lane < W && (t.anc & ~(good_bits | 1ull)) == 0ull;
  return wave_max_int(good ? (__popcll(t.anc) - 1) * 64 + (63 - lane) : -1);
}

// Writes the nodes of bit row `ab` (a root path) to path[0..len], root
// first, and -1 to path[len+1..W).  Path nodes write themselves to their
// depth; positions past len are padded by the lane of the same index (a
// different address even when that lane is itself a path node: its depth is
// <= len < lane).
__device__ __forceinline__ void write_path(uint64_t ab, int len, int W, int32_t* path, int* s_path) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < W;
  if (in && ((ab >> lane) & 1ull)) {
    const int pos = __popcll(ab & ((1ull << lane) - 1ull));
    path[pos] = lane;
    if (s_path != nullptr) s_path[pos] = lane;
  }
  if (in && lane > len) path[lane] = -1;
}

// Acceptance of sequence b by wave 0 (lane = node).  Returns the accepted
// length (-1 for a malformed mask) and fills s_path[0..len] with the path.
__device__ __forceinline__ int wave_accept(const AcceptParams& p, int b, const Prefetch& f, const int* s_tgt,
                                  int* s_path) {
  const int lane = threadIdx.x & 63;
  const int W = p.W;
  const bool in = lane < W;
  const NodeTree t = node_tree(f.kind, f.id, W);
  int32_t* path = p.accept_path + (size_t)b * W;
  if (!t.ok) {
    if (in) path[lane] = -1;
    if (lane == 0) {
      p.accept_len[b] = -1;
      p.bonus_id[b] = -1;
      raise_status(MTP_DEV_BAD_MASK);
    }
    return -1;
  }
  const bool match = in && lane >= 1 && f.draft >= 0 && f.draft == s_tgt[t.par];
  const int key = deepest_good(__ballot(match), t, W);
  const int best = 63 - (key & 63);
  const int len = key >> 6;
  write_path(shfl64(t.anc, best), len, W, path, s_path);
  if (lane == 0) {
    p.accept_len[b] = len;
    p.bonus_id[b] = s_tgt[best];
  }
  return len;
}

// Commit plan of sequence b: wave 0 validates one path position per lane
// (row index, page mapping) and publishes the source rows (s_src), the
// destination slots page * 16 + slot (s_dst) and the range (s_meta: last
// position or -1, first position) in LDS; it writes the new context length.
// Ends with a workgroup barrier.  When fused, `a_fused` and s_path come from
// the acceptance; otherwise they are read from memory.
template <bool kFused>
__device__ __forceinline__ void commit_plan(const CommitParams& p, int b, const Prefetch& f, int a_fused,
                                   const int* s_path, int* s_src, int* s_dst, int* s_meta) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < kWave) {
    const int a = kFused ? a_fused : p.accept_len[b];
    const int L = f.L;
    const int first = p.skip_root ? 1 : 0;
    const bool a_ok = a >= 0 && a <= p.W - 1 && L >= 0;
    bool bad_k = false;
    if (a_ok && lane >= first && lane <= a) {
      const int row = kFused ? s_path[lane] : p.accept_path[(size_t)b * p.W + lane];
      const int pg = f.page;
      bad_k = row < 0 || row >= p.W || pg < 0 || pg >= p.num_pages;
      s_src[lane] = row;
      s_dst[lane] = pg * kPage + ((L + lane) & 15);
    }
    const bool bad = __ballot(bad_k) != 0ull;
    if (lane == 0) {
      const bool good = a_ok && !bad;
      s_meta[0] = good ? a : -1;
      s_meta[1] = first;
      p.ctx_out[b] = good ? L + a + 1 : L;  // L was read before any write of ctx_out
      if (!good) raise_status(a_ok ? MTP_DEV_BAD_PAGE : MTP_DEV_BAD_ACCEPT);
    }
  }
  __syncthreads();
}

// Commit of sequence b: the plan, then all threads copy the accepted rows.
template <bool kFused>
__device__ __forceinline__ void block_commit(const CommitParams& p, int b, const Prefetch& f, int a_fused,
                                    const int* s_path, int* s_src, int* s_dst, int* s_meta) {
  commit_plan<kFused>(p, b, f, a_fused, s_path, s_src, s_dst, s_meta);
  const int a = s_meta[0];
  const int first = s_meta[1];
  if (a < first) return;
  const int chunks = p.row_bytes >> 4;
  const int total = (a - first + 1) * chunks;
  const char* kn = static_cast<const char*>(p.k_new);
  const char* vn = static_cast<const char*>(p.v_new);
  char* kc = static_cast<char*>(p.k_cache);
  char* vc = static_cast<char*>(p.v_cache);
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int k = first + idx / chunks;
    const size_t ch = (size_t)(idx % chunks) * 16;
    const size_t src = ((size_t)b * p.W + s_src[k]) * p.row_bytes + ch;
    const size_t dst = (size_t)s_dst[k] * p.row_bytes + ch;
    *reinterpret_cast<uint4*>(kc + dst) = *reinterpret_cast<const uint4*>(kn + src);
    *reinterpret_cast<uint4*>(vc + dst) = *reinterpret_cast<const uint4*>(vn + src);
  }
}

__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(AcceptParams p) {
  __shared__ int s_tgt[MTP_MAX_W];
  __shared__ int s_path[MTP_MAX_W];
  const int b = blockIdx.x;
  Prefetch f{};
  if (threadIdx.x < kWave) f = prefetch_inputs(p, nullptr, b);
  block_argmax(p, b, s_tgt);
  __syncthreads();
  if (threadIdx.x < kWave) wave_accept(p, b, f, s_tgt, s_path);
}

// Commit inputs of wave 0 (only wave 0 reads ctx_in: ctx_out may alias it).
__device__ __forceinline__ Prefetch commit_prefetch(const CommitParams& p, int b) {
  const int lane = threadIdx.x & 63;
  Prefetch f{};
  f.page = -1;
  if (threadIdx.x < kWave) {
    f.L = p.ctx_in[b];
    const int pi = (f.L + lane) >> 4;
    if (lane < p.W && f.L >= 0 && pi < p.max_pages)
      f.page = p.block_table[(size_t)b * p.max_pages + pi];
  }
  return f;
}

__global__ __launch_bounds__(256) void commit_kernel(CommitParams p) {
  __shared__ int s_src[MTP_MAX_W];
  __shared__ int s_dst[MTP_MAX_W];
  __shared__ int s_meta[2];
  const int b = blockIdx.x;
  block_commit<false>(p, b, commit_prefetch(p, b), 0, nullptr, s_src, s_dst, s_meta);
}

// Positions of the block rows: ctx_lens[b] + the row's depth below the
// anchor (chain / segment: the row index; tree: ancestors counted from the
// ancestor-or-self bit row).  One wave per sequence; a malformed mask gives
// -1 for the sequence and sets the status bit.
__global__ __launch_bounds__(256) void positions_kernel(const int32_t* ctx_lens, const uint8_t* mask_kind,
                                                        const int32_t* mask_ids, int32_t* positions,
                                                        int B, int W) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;
  const int lane = threadIdx.x & 63;
  const int kind = mask_kind[b];
  const int id = lane < W ? mask_ids[(size_t)b * W + lane] : 0;
  const int L = ctx_lens[b];
  const NodeTree t = node_tree(kind, id, W);
  if (lane < W) positions[(size_t)b * W + lane] = t.ok ? L + __popcll(t.anc) - 1 : -1;
  if (!t.ok && lane == 0) raise_status(MTP_DEV_BAD_MASK);
}

// LDS scratch of one fused acceptance + commit, in ints.
constexpr int kAcceptScratchInts = 4 * MTP_MAX_W + 2;

// Acceptance then commit of sequence b by one workgroup (any number of
// waves; wave 0 does the per-node work).  `sm` is kAcceptScratchInts ints of
// LDS.  Load order, heads of the dependency chains first: wave 0's per-node
// inputs and the context length, then the logits rows, then the block's new
// K/V rows (into registers when they fit, kPre 16-byte chunks per thread and
// tensor, up to kPreMaxBytes: the commit is then only stores) and the commit
// pages, which need the context length and are only used after the acceptance.
__device__ __forceinline__ void accept_commit_seq(const AcceptParams& ap, const CommitParams& cp, int b,
                                         int* sm) {
  constexpr int kPre = 4;
  constexpr int kPreMaxBytes = 32 * 1024;
  int* s_tgt = sm;
  int* s_path = sm + MTP_MAX_W;
  int* s_pos = sm + 2 * MTP_MAX_W;  // path position of a block row, -1 if not committed
  int* s_dst = sm + 3 * MTP_MAX_W;  // destination slot of a path position
  int* s_meta = sm + 4 * MTP_MAX_W;
  const int lane = threadIdx.x & 63;
  const int chunks = cp.row_bytes >> 4;
  const int all = ap.W * chunks;
  // one compute unit streams everything this workgroup loads: the rows of a
  // large block are fetched after the acceptance instead, and only if accepted
  const bool pre = all <= kPre * (int)blockDim.x && 2 * all * 16 <= kPreMaxBytes;
  const char* kn = static_cast<const char*>(cp.k_new);
  const char* vn = static_cast<const char*>(cp.v_new);
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 pk[kPre], pv[kPre];
  Prefetch f{};
  if (threadIdx.x < kWave) f = prefetch_inputs(ap, &cp, b);
  block_argmax(ap, b, s_tgt, [&] {
    if (pre) {
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        const int idx = threadIdx.x + u * blockDim.x;
        if (idx < all) {
          const int row = idx / chunks;
          const size_t src = ((size_t)b * ap.W + row) * cp.row_bytes + (size_t)(idx - row * chunks) * 16;
          pk[u] = *reinterpret_cast<const u32x4*>(kn + src);
          pv[u] = *reinterpret_cast<const u32x4*>(vn + src);
        }
      }
    }
    if (threadIdx.x < kWave) f.page = commit_page(cp, b, f.L);
  });
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int a = wave_accept(ap, b, f, s_tgt, s_path);
    // validate the commit: one path position per lane
    const int L = f.L;
    const int first = cp.skip_root ? 1 : 0;
    const bool a_ok = a >= 0 && a <= ap.W - 1 && L >= 0;
    bool bad_k = false;
    int row = -1;
    if (a_ok && lane >= first && lane <= a) {
      row = s_path[lane];
      bad_k = row < 0 || row >= ap.W || f.page < 0 || f.page >= cp.num_pages;
      s_dst[lane] = f.page * kPage + ((L + lane) & 15);
    }
    const bool good = a_ok && __ballot(bad_k) == 0ull;
    if (lane < ap.W) s_pos[lane] = -1;
    if (good && row >= 0) s_pos[row] = lane;  // after the reset: LDS writes of a wave stay in order
    if (lane == 0) {
      s_meta[0] = good ? a : -1;
      s_meta[1] = first;
      cp.ctx_out[b] = good ? L + a + 1 : L;  // L was read before any write of ctx_out
      if (!good) raise_status(a_ok ? MTP_DEV_BAD_PAGE : MTP_DEV_BAD_ACCEPT);
    }
  }
  __syncthreads();
  const int a = s_meta[0];
  const int first = s_meta[1];
  if (a < first) return;
  char* kc = static_cast<char*>(cp.k_cache);
  char* vc = static_cast<char*>(cp.v_cache);
  if (pre) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int idx = threadIdx.x + u * blockDim.x;
      if (idx < all) {
        const int row = idx / chunks;
        const int k = s_pos[row];
        if (k >= 0) {
          const size_t dst = (size_t)s_dst[k] * cp.row_bytes + (size_t)(idx - row * chunks) * 16;
          *reinterpret_cast<u32x4*>(kc + dst) = pk[u];
          *reinterpret_cast<u32x4*>(vc + dst) = pv[u];
        }
      }
    }
  } else {
    const int total = (a - first + 1) * chunks;
    for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
      const int k = first + idx / chunks;
      const size_t ch = (size_t)(idx % chunks) * 16;
      const size_t src = ((size_t)b * ap.W + s_path[k]) * cp.row_bytes + ch;
      const size_t dst = (size_t)s_dst[k] * cp.row_bytes + ch;
      *reinterpret_cast<uint4*>(kc + dst) = *reinterpret_cast<const uint4*>(kn + src);
      *reinterpret_cast<uint4*>(vc + dst) = *reinterpret_cast<const uint4*>(vn + src);
    }
  }
}

__global__ __launch_bounds__(kAcceptThreads) void accept_commit_kernel(AcceptParams ap, CommitParams cp) {
  __shared__ int sm[kAcceptScratchInts];
  accept_commit_seq(ap, cp, blockIdx.x, sm);
}

}  // namespace mtpv
