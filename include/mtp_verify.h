/*
 * mtp_verify.h -- C ABI of the multi-token verify step on MI355X (gfx950).
 *
 * The verify step of multi-token / speculative decoding, as the pages state
 * the problem:
 *
 *   1. verify attention: a width-W block (row 0 = the committed anchor, rows
 *      1..W-1 = drafted or mask tokens) attends over the sequence's committed
 *      paged KV cache plus the block's own K/V under an in-block mask
 *      ("BitMTP: When Multi-Token Prediction Meets Low-Bit Large Language
 *      Models", Sec. 3.3 and Sec. 3.4 M3: width-(D+1) verifier block with the
 *      anchor and an AR-causal mask; "Efficient Training-Free Multi-Token
 *      Prediction via Embedding-Space Probing", Sec. 2 Methodology: block =
 *      last token + predicted tokens + mask tokens, tree verification with
 *      static tree masks; "Dynamic Multi-Byte Prediction With Hierarchical
 *      Language Models", Fig. 2 and Sec. 3: the Latent Causal Attention mask);
 *   2. acceptance: the greedy verifier's argmax at every block row decides
 *      the accepted prefix (chain) or root path (tree) and one
 *      verifier-origin ("bonus") token (BitMTP Sec. 3.3, speculative-only
 *      decoding; Multi-Byte Prediction Sec. 3.1 and Sec. 6.2);
 *   3. KV commit: only the accepted rows' K/V are written into the cache, as
 *      consecutive rows after the committed boundary, and the boundary
 *      advances (BitMTP Sec. 3.4 M2; "BitNest: Bit-Nested Speculative
 *      Decoding for Memory-Efficient LLM Inference Acceleration", Sec. 3.4:
 *      keep accepted entries, discard the rejected suffix).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers owned by the caller, row-major
 *   and densely packed in the layouts given below.  The library allocates
 *   no device memory; verify attention takes a caller-provided workspace.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream) and returns once the kernels are enqueued.  The functions are
 *   stateless and reentrant; calls that write the same buffers must be
 *   ordered by the caller (same stream or events).
 * - Host-checkable argument errors return a non-zero mtp_status and enqueue
 *   nothing.  Data errors found on the device (bad mask ids, a context length
 *   out of range, an unmapped page) never fault: they poison the affected
 *   outputs as documented per call and OR a bit into a per-device sticky
 *   status word read by mtp_get_device_status().
 * - Context length ctx_lens[b] counts the committed tokens strictly before
 *   block row 0.  Logical token t of sequence b lives in page
 *   block_table[b][t / 16], slot t % 16.
 * - Mask description per sequence: mask_kind[b] (uint8) and mask_ids[b][W]
 *   (int32):
 *     MTP_MASK_CHAIN   : ids ignored; row i sees block rows 0..i.
 *     MTP_MASK_TREE    : ids = parent array, ids[0] ignored (root), and
 *                        0 <= ids[i] < i for i >= 1; row i sees itself and
 *                        its ancestors.
 *     MTP_MASK_SEGMENT : ids = segment ids, ids[0] == 0, each step 0 or +1;
 *                        row i sees earlier rows of its own segment, itself,
 *                        and the seg_lookback previous segments (-1 = all
 *                        earlier segments; 1 = the LCA mask of Fig. 2).
 *   Every committed token is visible to every block row.
 */
#ifndef MTP_VERIFY_H
#define MTP_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_ABI_VERSION 1
#define MTP_PAGE_SIZE 16
#define MTP_MAX_W 64

typedef enum {
  MTP_OK = 0,
  MTP_ERR_NULL = 1,        /* a required pointer is NULL */
  MTP_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  MTP_ERR_UNSUPPORTED = 3, /* valid but not implemented (D, dtype, page size) */
  MTP_ERR_WORKSPACE = 4,   /* workspace too small */
  MTP_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  MTP_ERR_CONFLICT = 6,    /* mtp_check_commit_slots: a commit slot is not the sequence's own */
  MTP_ERR_SCRATCH = 7      /* mtp_verify_step_noalloc: the shape exceeds the fixed scratch */
} mtp_status;

typedef enum { MTP_F32 = 0, MTP_BF16 = 1 } mtp_dtype;

typedef enum { MTP_MASK_CHAIN = 0, MTP_MASK_TREE = 1, MTP_MASK_SEGMENT = 2 } mtp_mask_kind;

/* Bits of the device status word. */
#define MTP_DEV_BAD_MASK 0x1u   /* mask_kind unknown or mask_ids malformed */
#define MTP_DEV_BAD_CTX 0x2u    /* ctx_lens[b] < 0 or > max_ctx_len */
#define MTP_DEV_BAD_PAGE 0x4u   /* block_table entry outside [0, num_pages) where read or written */
#define MTP_DEV_BAD_ACCEPT 0x8u /* commit given accept_len / accept_path out of range */

/* Sizes of one verify step. */
typedef struct mtp_shape {
  int32_t B;                 /* sequences in the batch, >= 0 (0 = no-op) */
  int32_t W;                 /* block width, 1..64 (row 0 = anchor) */
  int32_t Hq;                /* query heads; Hq % Hkv == 0, group g = Hq / Hkv */
  int32_t Hkv;               /* KV heads, >= 1 */
  int32_t D;                 /* head dim: 64 or 128 */
  int32_t page_size;         /* tokens per page: must be 16 */
  int32_t num_pages;         /* pages in each of k_cache / v_cache */
  int32_t max_pages_per_seq; /* columns of block_table */
  int32_t max_ctx_len;       /* upper bound of every ctx_lens[b]; <= 16 * max_pages_per_seq */
  int32_t dtype;             /* mtp_dtype of q, k_cache, v_cache, k_new, v_new */
  float scale;               /* softmax scale; 0 selects 1/sqrt(D) */
  int32_t seg_lookback;      /* SEGMENT masks: -1 = all earlier segments, k >= 0 = k previous */
  int32_t split_tokens;      /* committed tokens per split-K work item; 0 = automatic,
                                else a positive multiple of 32 */
} mtp_shape;

/* Returns MTP_ABI_VERSION. */
int32_t mtp_abi_version(void);

/* Static text for a status code (never NULL). */
const char* mtp_status_string(int32_t status);

/* Bytes of device workspace mtp_verify_attn and mtp_verify_step need for
 * `shape` (split-K partials: per sequence, split, KV head and block-row x
 * group-member row, D accumulators plus running max and sum, fp32; then
 * B * W int32 row targets, which mtp_verify_step may hand from its partial
 * launch to its acceptance).  Depends on B, W, Hq, Hkv, D, dtype,
 * max_ctx_len and split_tokens only. */
mtp_status mtp_verify_attn_workspace_size(const mtp_shape* shape, size_t* bytes);

/* Verify attention (the step's attention over committed + in-block keys).
 *
 *   q            [B, W, Hq, D]           dtype
 *   k_cache      [num_pages, 16, Hkv, D] dtype (read only)
 *   v_cache      [num_pages, 16, Hkv, D] dtype (read only)
 *   block_table  [B, max_pages_per_seq]  int32
 *   ctx_lens     [B]                     int32
 *   k_new, v_new [B, W, Hkv, D]          dtype (the block's own K/V)
 *   mask_kind    [B] uint8, mask_ids [B, W] int32 (see above)
 *   out          [B, W, Hq, D]           fp32  (written)
 *   lse          [B, W, Hq]              fp32 natural-log sum-exp of the
 *                                        scaled scores, or NULL
 *   workspace    >= mtp_verify_attn_workspace_size bytes, 16-byte aligned
 *
 * Query head h reads KV head h / (Hq / Hkv).  out[b,i,h] =
 * sum_t softmax_t(scale * q.k_t) v_t over the visible keys.  Data errors:
 * a sequence with a malformed mask or a context length outside
 * [0, max_ctx_len] gets NaN in all of its out / lse rows; a block-table
 * entry outside [0, num_pages) inside the committed range makes the rows
 * that read it NaN.  Both set the corresponding status bit. */
mtp_status mtp_verify_attn(const mtp_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* ctx_lens, const void* k_new, const void* v_new,
                           const uint8_t* mask_kind, const int32_t* mask_ids, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* The two launches mtp_verify_attn makes, for callers that time or order
 * them separately: the split-K partial kernel (writes only the workspace)
 * and the combine kernel (reads the workspace, writes out / lse).  Same
 * arguments and checks as mtp_verify_attn; partial must precede combine on
 * the same workspace. */
mtp_status mtp_verify_attn_partial(const mtp_shape* shape, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* ctx_lens, const void* k_new,
                                   const void* v_new, const uint8_t* mask_kind,
                                   const int32_t* mask_ids, float* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);
mtp_status mtp_verify_attn_combine(const mtp_shape* shape, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* ctx_lens, const void* k_new,
                                   const void* v_new, const uint8_t* mask_kind,
                                   const int32_t* mask_ids, float* out, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Greedy acceptance (uses B and W of `shape` only).
 *
 *   logits      [B, W, V] fp32: the verifier's logits at each block row
 *   draft_ids   [B, W] int32: drafted token of each row (row 0 ignored;
 *               < 0 marks a mask token, which is never accepted)
 *   accept_len  [B] int32 (written): accepted drafts, 0..W-1
 *   accept_path [B, W] int32 (written): block rows of the accepted path,
 *               root first, padded with -1
 *   bonus_id    [B] int32 (written): the verifier-origin token
 *
 * target[i] = argmax_v logits[b,i,v] (smallest id on ties).  Row i >= 1
 * matches when draft_ids[b,i] >= 0 and equals target[parent(i)], where
 * parent(i) is the tree parent (TREE) or i-1 (CHAIN, SEGMENT).  The accepted
 * node is the deepest node whose whole root path matches (smallest index
 * on ties); the root is always accepted; bonus = target[accepted node].
 * A malformed mask writes -1 to all three outputs of that sequence.
 * Logits must be finite (NaN handling is unspecified). */
mtp_status mtp_accept(const mtp_shape* shape, const float* logits, int32_t V,
                      const int32_t* draft_ids, const uint8_t* mask_kind,
                      const int32_t* mask_ids, int32_t* accept_len, int32_t* accept_path,
                      int32_t* bonus_id, void* stream);

/* Confidence-threshold and hybrid acceptance ("BitMTP: When Multi-Token
 * Prediction Meets Low-Bit Large Language Models", Sec. 3.3, with the
 * threshold rule of "Dynamic Multi-Byte Prediction With Hierarchical
 * Language Models", Sec. 3.1).  Uses B and W of `shape` only.
 *
 *   draft_logits [B, W, V] fp32: row i is the drafter's distribution that
 *                produced draft i (row 0 unused)
 *   logits       [B, W, V] fp32 or NULL: the verifier's logits (as for
 *                mtp_accept); NULL when the verifier has not run
 *   tau          confidence threshold (NaN rejected); min_prefix = m
 *   conf_len     [B] int32 (written): confidence prefix h
 *   other arguments and outputs as for mtp_accept.
 *
 * A draft is confident when it is a token (0 <= id < V) and its softmax
 * probability under draft_logits reaches tau (fp32 arithmetic).  h is the
 * depth of the deepest node whose whole root path is confident (chains: the
 * number of leading confident drafts), smallest index on ties.  When h >= 1
 * and h >= m the h drafts are taken without the verifier: accept_len = h - 1,
 * accept_path = root path of the deepest confident node's parent, bonus_id =
 * that node's draft (the next anchor).  Otherwise the outputs are those of
 * mtp_accept, or -1 (accept_len, bonus_id, whole path) when logits is NULL.
 * A malformed mask writes -1 to all four outputs.  The outputs feed
 * mtp_kv_commit unchanged. */
mtp_status mtp_accept_hybrid(const mtp_shape* shape, const float* draft_logits,
                             const float* logits, int32_t V, const int32_t* draft_ids,
                             const uint8_t* mask_kind, const int32_t* mask_ids, float tau,
                             int32_t min_prefix, int32_t* accept_len, int32_t* accept_path,
                             int32_t* bonus_id, int32_t* conf_len, void* stream);

/* KV commit.  For path position k = (skip_root ? 1 : 0) .. accept_len[b],
 * copies the bytes of k_new/v_new[b, accept_path[b][k], :, :] to logical
 * position ctx_lens_in[b] + k of k_cache/v_cache, then writes
 * ctx_lens_out[b] = ctx_lens_in[b] + accept_len[b] + 1 (may alias
 * ctx_lens_in).  skip_root = 1 leaves the anchor's slot untouched (callers
 * whose anchor K/V is already cached).  The caller maps every page the
 * commit writes.  A sequence whose accept_len is outside [0, W-1], whose
 * path holds a row outside [0, W), whose context length is negative or
 * whose target slots are unmapped is not written at all and keeps its
 * context length (status bit set). */
mtp_status mtp_kv_commit(const mtp_shape* shape, const void* k_new, const void* v_new,
                         const int32_t* accept_len, const int32_t* accept_path,
                         const int32_t* block_table, const int32_t* ctx_lens_in,
                         int32_t* ctx_lens_out, int32_t skip_root, void* k_cache,
                         void* v_cache, void* stream);

/* mtp_accept followed by mtp_kv_commit in one launch (one workgroup per
 * sequence); same arguments, same results. */
mtp_status mtp_accept_commit(const mtp_shape* shape, const float* logits, int32_t V,
                             const int32_t* draft_ids, const uint8_t* mask_kind,
                             const int32_t* mask_ids, int32_t* accept_len,
                             int32_t* accept_path, int32_t* bonus_id, const void* k_new,
                             const void* v_new, const int32_t* block_table,
                             const int32_t* ctx_lens_in, int32_t* ctx_lens_out,
                             int32_t skip_root, void* k_cache, void* v_cache, void* stream);

/* The whole verify step in two launches: the split-K partial kernel, then
 * one launch that runs the combine (out, lse) side by side with acceptance
 * and commit (they do not depend on each other: the combine reads partial
 * results and ctx_lens_in, the commit writes cache slots >= ctx_len and
 * ctx_lens_out).  Arguments as for mtp_verify_attn and mtp_accept_commit;
 * attention reads ctx_lens_in and the cache as they are before the commit.
 * When ctx_lens_out aliases ctx_lens_in the combine and the commit run as
 * two ordered launches instead.  Results are those of mtp_verify_attn
 * followed by mtp_accept_commit. */
mtp_status mtp_verify_step(const mtp_shape* shape, const void* q, void* k_cache, void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens_in,
                           const void* k_new, const void* v_new, const uint8_t* mask_kind,
                           const int32_t* mask_ids, const float* logits, int32_t V,
                           const int32_t* draft_ids, float* out, float* lse,
                           int32_t* accept_len, int32_t* accept_path, int32_t* bonus_id,
                           int32_t* ctx_lens_out, int32_t skip_root, void* workspace,
                           size_t workspace_bytes, void* stream);

/* mtp_verify_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same launches and results, with the split-K partials in a fixed
 * 64 MiB array the library keeps in device memory (each GPU the library
 * runs on holds its own copy until the process ends) instead of a caller
 * workspace.  The caller still passes every input and output; nothing is
 * allocated and no part of the array needs clearing.  A shape whose
 * mtp_verify_attn_workspace_size exceeds 64 MiB returns MTP_ERR_SCRATCH and
 * enqueues nothing (the five reference workloads need at most 34 MB).  All
 * calls on one GPU share its array: calls that may overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.
 * Arguments and errors otherwise as for mtp_verify_step. */
mtp_status mtp_verify_step_noalloc(const mtp_shape* shape, const void* q, void* k_cache,
                                   void* v_cache, const int32_t* block_table,
                                   const int32_t* ctx_lens_in, const void* k_new,
                                   const void* v_new, const uint8_t* mask_kind,
                                   const int32_t* mask_ids, const float* logits, int32_t V,
                                   const int32_t* draft_ids, float* out, float* lse,
                                   int32_t* accept_len, int32_t* accept_path, int32_t* bonus_id,
                                   int32_t* ctx_lens_out, int32_t skip_root, void* stream);

/* ---- Nested KV4 / KV8 cache ("BitNest: Bit-Nested Speculative Decoding for
 * Memory-Efficient LLM Inference Acceleration", Sec. 3.4 and Sec. A.2) ----
 *
 * Each committed K or V vector x (one token, one KV head, D elements) is
 * quantized once, when written: s = max|x| / 7, t = x / s,
 * q4 = rint(t), qr = clamp(rint(16 t) - 16 q4, -8, 7) (fp32, rint = round half
 * to even; s = 0 and zero codes for a zero vector).  KV4 = s * q4 (the base
 * plane alone), KV8 = (s / 16) * (16 q4 + qr) (base + refinement).  Layout
 * (all device memory, owned by the caller, 16-byte aligned):
 *   *_base, *_ref  [num_pages, Hkv, 16, D/2] bytes: code + 8 in nibbles, two
 *                  per byte, even element in the low nibble;
 *   *_scale        [num_pages, Hkv, 16] fp32.
 * Slots never written hold arbitrary bytes; no call reads them as data. */
typedef struct mtp_nested_kv {
  uint8_t* k_base;
  uint8_t* k_ref;
  float* k_scale;
  uint8_t* v_base;
  uint8_t* v_ref;
  float* v_scale;
} mtp_nested_kv;

/* Quantizes n_rows K and V rows ([n_rows, Hkv, D] in shape->dtype, fp32 or
 * bf16, finite) into the nested planes at slots[r] = page * 16 + slot (the
 * prefill path).  Uses Hkv, D, dtype and num_pages of `shape`.  A slot
 * outside [0, 16 * num_pages) is skipped (MTP_DEV_BAD_PAGE).  Rows sharing a
 * slot race. */
mtp_status mtp_kv_quantize(const mtp_shape* shape, const void* k_rows, const void* v_rows,
                           int32_t n_rows, const int32_t* slots, const mtp_nested_kv* kv,
                           void* stream);

/* mtp_kv_commit into a nested cache: each accepted row of k_new / v_new is
 * quantized into its slot (same validation and context update as
 * mtp_kv_commit; `kv` is a host pointer to device plane pointers). */
mtp_status mtp_kv_commit_nested(const mtp_shape* shape, const void* k_new, const void* v_new,
                                const int32_t* accept_len, const int32_t* accept_path,
                                const int32_t* block_table, const int32_t* ctx_lens_in,
                                int32_t* ctx_lens_out, int32_t skip_root,
                                const mtp_nested_kv* kv, void* stream);

/* Workspace of mtp_verify_attn_nested (its split plan differs from the
 * bf16-cache one). */
mtp_status mtp_verify_attn_nested_workspace_size(const mtp_shape* shape, size_t* bytes);

/* Verify attention over a nested cache (bf16 queries and block rows,
 * D = 128).  Arguments as for mtp_verify_attn, with the committed cache given
 * as planes.  Committed token t of a sequence with context length L is read
 * in KV8 when kv8_recent < 0 (verification: the full cache) or
 * t >= L - kv8_recent ("Recent-N"), else in KV4; kv8_recent = 0 reads the
 * base plane only (drafting), and then k_ref / v_ref may be NULL.  The
 * block's own rows (k_new, v_new) are used unquantized.  Results match
 * attention over the dequantized cache within the bf16 tolerance for
 * committed V scales s below 2^60 (max|v| below about 8e18; beyond, the
 * scaled weights overflow and the row comes out non-finite). */
mtp_status mtp_verify_attn_nested(const mtp_shape* shape, const void* q, const mtp_nested_kv* kv,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  const void* k_new, const void* v_new, const uint8_t* mask_kind,
                                  const int32_t* mask_ids, int32_t kv8_recent, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* The two launches of mtp_verify_attn_nested on their own (the partial
 * kernel over the planes, then the combine); same arguments and checks. */
mtp_status mtp_verify_attn_nested_partial(const mtp_shape* shape, const void* q,
                                          const mtp_nested_kv* kv, const int32_t* block_table,
                                          const int32_t* ctx_lens, const void* k_new,
                                          const void* v_new, const uint8_t* mask_kind,
                                          const int32_t* mask_ids, int32_t kv8_recent,
                                          float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream);
mtp_status mtp_verify_attn_nested_combine(const mtp_shape* shape, const void* q,
                                          const mtp_nested_kv* kv, const int32_t* block_table,
                                          const int32_t* ctx_lens, const void* k_new,
                                          const void* v_new, const uint8_t* mask_kind,
                                          const int32_t* mask_ids, int32_t kv8_recent,
                                          float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Dynamic token tree for the next block ("Efficient Training-Free Multi-Token
 * Prediction via Embedding-Space Probing", Sec. 2.C: expansion by cumulative
 * probability, only the top-1 token of each depth expanded, a fixed budget,
 * consecutive repeated tokens pruned; Sec. 2.D: block = last token +
 * predicted tokens + mask tokens, positions by offsets).
 *
 *   probs      [B, K, V] fp32 (device): the drafter's probabilities for
 *              depths 1..K (finite, >= 0); K in [1, 64]
 *   root_token [B] int32: the last committed token (block row 0)
 *   W, n_mask  block width (1..64) and mask-token rows (0..W-1); W - 1 -
 *              n_mask rows hold predicted tokens
 *   outputs    draft_ids, parents, depth [B, W] int32; n_nodes [B] int32
 *
 * At depth d the parent's token is dropped; the most probable remaining
 * token (smallest id on ties) is the depth's top-1 node, the parent of every
 * depth-(d+1) candidate; a candidate's cumulative probability is
 * c_{d-1} * p_d(v), c_0 = 1, c_d = c_{d-1} * p_d(top-1) (fp32 products in this
 * order).  Nodes are chosen best first (ties: shallower, then more probable
 * at its depth, then smaller id) while predicted rows remain and the best
 * reaches min_cum_prob (NaN rejected).  Row 0 = root (draft = root token,
 * parent -1), then the chosen nodes in the order chosen, then mask-token rows
 * (draft -1) chained from the deepest chosen top-1 node.  parents is a valid
 * TREE mask description and depth the position offset of each row;
 * n_nodes = 1 + chosen nodes.  V <= 4096.  Two launches: the ranked lists
 * (a workgroup per depth and sequence), then the placement (a workgroup per
 * sequence); `workspace` carries the lists between them. */
mtp_status mtp_build_tree(int32_t B, int32_t K, int32_t V, int32_t W, int32_t n_mask,
                          const float* probs, const int32_t* root_token, float min_cum_prob,
                          int32_t* draft_ids, int32_t* parents, int32_t* depth,
                          int32_t* n_nodes, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace of mtp_build_tree (the ranked candidate lists, caller-owned,
 * 16-byte aligned; contents need no initialisation). */
mtp_status mtp_build_tree_workspace_size(int32_t B, int32_t K, int32_t V, int32_t W,
                                         int32_t n_mask, size_t* bytes);

/* Positions of the block rows for the verifier's inputs, prepared on the
 * device ("BitMTP" Sec. 3.4 M3: verifier inputs follow the materialized KV
 * boundary and are prepared before the host reads the acceptance; "Efficient
 * Training-Free Multi-Token Prediction via Embedding-Space Probing" Sec. 2.D:
 * position indices by offsets).  Uses B and W of `shape`.
 *   positions [B, W] int32 (written): ctx_lens[b] + the row's depth below the
 *   anchor: the row index for CHAIN and SEGMENT blocks, the number of
 *   ancestors for TREE blocks.  A malformed mask writes -1 for the sequence
 *   (MTP_DEV_BAD_MASK).
 * With ctx_lens = the previous step's ctx_lens_out this needs no host
 * round trip between steps. */
mtp_status mtp_block_positions(const mtp_shape* shape, const int32_t* ctx_lens,
                               const uint8_t* mask_kind, const int32_t* mask_ids,
                               int32_t* positions, void* stream);

/* Host-side check of a block table before commits (no device work; the
 * arguments are HOST pointers).  The accepted rows of sequence b are written
 * to the slots of logical positions ctx_lens[b] .. ctx_lens[b] + W - 1, which
 * the sequence must own alone ("BitMTP" Sec. 3.4 M2: accepted rows are
 * promoted into the sequence's own workspace slots).  A table that maps one
 * of those slots a second time, anywhere in logical positions
 * 0 .. ctx_lens[b'] + W - 1 of any sequence b' (b included), is a caller
 * error: the commit would race with another sequence's commit or overwrite
 * history that attention reads, and the device does not detect it.  Pages
 * shared read-only between sequences (a common prefix) are fine as long as
 * no commit range reaches them.
 *   block_table [B, max_pages_per_seq] int32, ctx_lens [B] int32 (host)
 *   bad_seq     (may be NULL) receives the smallest sequence index involved
 *               in a conflict, or -1.
 * Returns MTP_OK, or MTP_ERR_CONFLICT when a conflict exists.  Uses B, W,
 * num_pages and max_pages_per_seq of `shape`; positions past the table,
 * unmapped entries and negative contexts are skipped (the device reports
 * those as data errors).  Time and memory: O(sum of ctx_lens + B W) and
 * 64 bytes per page. */
mtp_status mtp_check_commit_slots(const mtp_shape* shape, const int32_t* block_table,
                                  const int32_t* ctx_lens, int32_t* bad_seq);

/* Reads (and with clear != 0 resets) the current device's sticky status word
 * into *bits.  Synchronous: waits for all work on the device. */
mtp_status mtp_get_device_status(uint32_t* bits, int32_t clear);

#ifdef __cplusplus
}
#endif

#endif /* MTP_VERIFY_H */
