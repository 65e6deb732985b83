"""fp64 CPU oracle for the multi-token verify step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module; the library's
product path never does.  It shares no code with the HIP path.

What it computes, step by step, in the notation of the pages:

* The verifier block.  A width-W block whose row 0 is the committed anchor
  (the last committed token) and whose rows 1..W-1 are drafted tokens or mask
  tokens.  "BitMTP: When Multi-Token Prediction Meets Low-Bit Large Language
  Models", §3.3 (draft block d_1:D, accepted length a_i, one verifier-origin
  token) and §3.4 M3 (width-(D+1) verifier block with the anchor);
  "Efficient Training-Free Multi-Token Prediction via Embedding-Space
  Probing", §2.D (block = last token + predicted tokens + mask tokens).

* In-block visibility (``block_visibility``).
  - CHAIN: the AR-causal verifier mask, row i sees rows 0..i (BitMTP §3.4 M3).
  - TREE: a node sees itself and its ancestors (tree attention; BitMTP §2 on
    Medusa's tree verification; Embedding-Space Probing §2.C-D, dynamic tree
    with static tree masks).  The tree is a parent array with parent[i] < i.
  - SEGMENT: Latent Causal Attention ("Dynamic Multi-Byte Prediction With
    Hierarchical Language Models", Fig. 2 and §3): a position sees itself,
    earlier positions of its own segment and the segments before it.  The
    figure restricts the earlier segments to the immediately preceding one;
    the workload statement lets a query see all earlier segments.  Both are
    covered by ``seg_lookback`` (k >= 0 previous segments, or -1 = all).

* Attention (``verify_attention``).  Every committed position 0..L-1 is
  visible to every block row; block rows are visible per the mask above.
  s = scale * q.k, p = softmax over the visible keys, out = sum p v,
  lse = log sum exp s.  GQA: query head h uses KV head h // (Hq/Hkv).  The
  committed cache is paged: logical token t lives in page
  block_table[t // 16], slot t % 16.  Everything is done in fp64 over an
  explicit dense [W, L+W] boolean mask.

* Acceptance (``accept``).  The target token of row i is the argmax of its
  logits (smallest id on ties).  Row 0 (the anchor) is always accepted
  (Multi-Byte Prediction, Alg. 1: the next-byte head's output is always
  accepted).  A drafted row i matches when its draft equals the target of its
  parent (chain: row i-1), i.e. the verifier's prediction at the parent;
  mask-token rows (draft < 0) never match.  The accepted path is the deepest
  node whose whole root path matches (chain: the longest matching prefix,
  BitMTP §3.3 speculative-only decoding; Multi-Byte Prediction §3.1 and §6.2,
  left-to-right acceptance); ties go to the smaller node index.  The bonus
  (verifier-origin) token is the target at the accepted node (BitMTP §3.3).

* Hybrid acceptance (``accept_hybrid``).  The drafter's probability of each
  drafted token decides a confidence prefix h; h >= m commits the h drafts
  without the verifier, otherwise the greedy verification above decides
  (BitMTP §3.3 hybrid decoding; Multi-Byte Prediction §3.1 byte acceptance).

* Nested KV4 / KV8 cache (``quantize_nested``, ``verify_attention_nested``,
  ``kv_commit_nested``): BitNest §3.4 / §A.2, see its section below.

* Dynamic token tree (``dynamic_tree``): the next block built from the
  drafter's probabilities ("Efficient Training-Free Multi-Token Prediction
  via Embedding-Space Probing" §2.C-D), see its section below.

* Block positions (``block_positions``): committed length + the row's depth
  (BitMTP §3.4 M3; Embedding-Space Probing §2.D).

* Commit (``kv_commit``).  The K/V rows of the accepted path, root first, are
  copied to logical positions L, L+1, ..., L+a; rejected rows are never
  written and the KV boundary advances by a+1 (BitMTP §3.4 M2: accepted draft
  rows are promoted as consecutive rows; "BitNest: Bit-Nested Speculative
  Decoding for Memory-Efficient LLM Inference Acceleration", §3.4 / §A.2:
  retain accepted entries, discard the rejected suffix).  ``skip_root``
  leaves the anchor's slot untouched, for callers whose anchor KV is already
  in the cache (BitMTP §3.4 M2: promotion excludes the repeated anchor).

Data errors (a parent index outside [0, i), segment ids that do not start at
0 or step by other than 0/+1, an unknown mask kind, or an unmapped page for a
slot the commit must write) are handled as the library's contract states:
the sequence's attention output and log-sum-exp are NaN, its acceptance
outputs are -1, and its commit is skipped (context length unchanged).
"""
from __future__ import annotations

import numpy as np

PAGE = 16
CHAIN, TREE, SEGMENT = 0, 1, 2


# ----------------------------------------------------------------------------
# in-block structure
# ----------------------------------------------------------------------------

def mask_is_valid(kind: int, ids: np.ndarray) -> bool:
    """Whether a block's mask description is well formed."""
    W = ids.shape[0]
    if kind == CHAIN:
        return True
    if kind == TREE:
        return all(0 <= int(ids[i]) < i for i in range(1, W))
    if kind == SEGMENT:
        if int(ids[0]) != 0:
            return False
        return all(int(ids[i]) - int(ids[i - 1]) in (0, 1) for i in range(1, W))
    return False


def acceptance_parents(kind: int, ids: np.ndarray) -> np.ndarray:
    """Parent of every block row for acceptance: the tree's parent array, or
    the previous row for a chain / segment block (left-to-right acceptance)."""
    W = ids.shape[0]
    if kind == TREE:
        par = np.array(ids, dtype=np.int64)
        par[0] = -1
        return par
    return np.arange(-1, W - 1, dtype=np.int64)


def block_visibility(kind: int, ids: np.ndarray, seg_lookback: int) -> np.ndarray:
    """[W, W] bool: vis[i, j] = block row i may attend to block row j."""
    W = ids.shape[0]
    vis = np.zeros((W, W), dtype=bool)
    if kind == CHAIN:
        for i in range(W):
            for j in range(i + 1):
                vis[i, j] = True
    elif kind == TREE:
        for i in range(W):
            j = i
            while j >= 0:
                vis[i, j] = True
                j = int(ids[j]) if j > 0 else -1
    elif kind == SEGMENT:
        for i in range(W):
            si = int(ids[i])
            for j in range(W):
                sj = int(ids[j])
                own = (sj == si) and (j <= i)
                earlier = sj < si and (seg_lookback < 0 or si - sj <= seg_lookback)
                vis[i, j] = own or earlier
    else:
        raise ValueError(f"unknown mask kind {kind}")
    return vis


def dense_mask(ctx_len: int, vis: np.ndarray) -> np.ndarray:
    """[W, L+W] bool over (committed keys, block keys)."""
    W = vis.shape[0]
    m = np.zeros((W, ctx_len + W), dtype=bool)
    m[:, :ctx_len] = True
    m[:, ctx_len:] = vis
    return m


# ----------------------------------------------------------------------------
# paged cache
# ----------------------------------------------------------------------------

def page_slot(block_row: np.ndarray, t: int) -> tuple[int, int]:
    """Physical (page, slot) of logical token t of one sequence."""
    return int(block_row[t // PAGE]), t % PAGE


def gather_committed(cache: np.ndarray, block_row: np.ndarray, ctx_len: int) -> np.ndarray:
    """Committed rows 0..L-1 of one sequence as a dense [L, Hkv, D] fp64 array."""
    Hkv, D = cache.shape[2], cache.shape[3]
    out = np.empty((ctx_len, Hkv, D), dtype=np.float64)
    for t in range(ctx_len):
        page, slot = page_slot(block_row, t)
        out[t] = cache[page, slot]
    return out


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, mask: np.ndarray,
           scale: float):
    """Masked softmax attention of W query rows over N keys, fp64.

    q [W, D], keys/values [N, D], mask [W, N] -> out [W, D], lse [W], p [W, N]."""
    s = scale * (q @ keys.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    out = p @ values
    lse = m[:, 0] + np.log(z[:, 0])
    return out, lse, p


def attention_over(q, committed, k_new, v_new, mask_kind, mask_ids, scale=None, seg_lookback=-1):
    """Verify attention for a batch whose committed rows come from
    ``committed(b, L) -> (keys [L,Hkv,D], values [L,Hkv,D])`` (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    B, W, Hq, D = q.shape
    Hkv = k_new.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, W, Hq, D), np.nan)
    lse = np.full((B, W, Hq), np.nan)
    for b in range(B):
        kind, ids = int(mask_kind[b]), np.asarray(mask_ids[b])
        if not mask_is_valid(kind, ids):
            continue
        ck, cv = committed(b)
        L = ck.shape[0]
        keys = np.concatenate([ck, k_new[b]], axis=0)
        vals = np.concatenate([cv, v_new[b]], axis=0)
        mask = dense_mask(L, block_visibility(kind, ids, seg_lookback))
        for h in range(Hq):
            kvh = h // g
            o, l, _ = attend(q[b, :, h, :], keys[:, kvh, :], vals[:, kvh, :], mask, scale)
            out[b, :, h, :] = o
            lse[b, :, h] = l
    return out, lse


def verify_attention(q, k_cache, v_cache, block_table, ctx_lens, k_new, v_new,
                     mask_kind, mask_ids, scale=None, seg_lookback=-1):
    """Verify attention for a batch.

    q [B,W,Hq,D]; k_cache/v_cache [pages,16,Hkv,D]; block_table [B,max_pages];
    ctx_lens [B]; k_new/v_new [B,W,Hkv,D]; mask_kind [B]; mask_ids [B,W].
    Returns out [B,W,Hq,D] and lse [B,W,Hq] in fp64."""
    def committed(b):
        L = int(ctx_lens[b])
        return (gather_committed(k_cache, block_table[b], L),
                gather_committed(v_cache, block_table[b], L))
    return attention_over(q, committed, k_new, v_new, mask_kind, mask_ids, scale, seg_lookback)


# ----------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------

def target_ids(logits: np.ndarray) -> np.ndarray:
    """Greedy verifier prediction per row: argmax, smallest id on ties."""
    return np.argmax(np.asarray(logits), axis=-1).astype(np.int64)


def accept(logits, draft_ids, mask_kind, mask_ids):
    """Returns accept_len [B], accept_path [B,W] (-1 padded), bonus_id [B]."""
    logits = np.asarray(logits)
    B, W = logits.shape[0], logits.shape[1]
    tgt = target_ids(logits)
    acc_len = np.full(B, -1, dtype=np.int64)
    path = np.full((B, W), -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        kind, ids = int(mask_kind[b]), np.asarray(mask_ids[b])
        if not mask_is_valid(kind, ids):
            continue
        par = acceptance_parents(kind, ids)
        ok = np.zeros(W, dtype=bool)
        depth = np.zeros(W, dtype=np.int64)
        ok[0] = True
        for i in range(1, W):
            d = int(draft_ids[b, i])
            p = int(par[i])
            depth[i] = depth[p] + 1
            ok[i] = ok[p] and d >= 0 and d == tgt[b, p]
        best = 0
        for i in range(1, W):
            if ok[i] and depth[i] > depth[best]:
                best = i
        chain = []
        j = best
        while j >= 0:
            chain.append(j)
            j = int(par[j])
        chain.reverse()
        acc_len[b] = depth[best]
        path[b, :len(chain)] = chain
        bonus[b] = tgt[b, best]
    return acc_len, path, bonus


# ----------------------------------------------------------------------------
# commit
# ----------------------------------------------------------------------------

def commit_writes(accept_len, accept_path, block_table, ctx_lens, num_pages, skip_root=False):
    """The commit's writes as (b, page, slot, block row) and the new context
    lengths.  A sequence whose accepted length or path is out of range, or
    one of whose target slots is unmapped, writes nothing and keeps its
    length."""
    ctx = np.array(ctx_lens, dtype=np.int64, copy=True)
    B, W = accept_path.shape
    out = []
    for b in range(B):
        a = int(accept_len[b])
        if a < 0 or a > W - 1:
            continue
        L = int(ctx_lens[b])
        first = 1 if skip_root else 0
        writes = []
        for k in range(first, a + 1):
            t = L + k
            row = int(accept_path[b, k])
            if t // PAGE >= block_table.shape[1] or not (0 <= row < W):
                writes = None
                break
            page, slot = page_slot(block_table[b], t)
            if not (0 <= page < num_pages):
                writes = None
                break
            writes.append((b, page, slot, row))
        if writes is None:
            continue
        out.extend(writes)
        ctx[b] = L + a + 1
    return out, ctx


def kv_commit(k_cache, v_cache, k_new, v_new, accept_len, accept_path, block_table,
              ctx_lens, skip_root=False):
    """Copies the accepted rows' K/V bytes into the cache pages.

    Works on the raw element arrays (any dtype: the copy is exact).  Returns
    (k_cache', v_cache', ctx_lens') as new arrays; the inputs are not
    modified."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    writes, ctx = commit_writes(accept_len, accept_path, block_table, ctx_lens, kc.shape[0],
                                skip_root)
    for b, page, slot, row in writes:
        kc[page, slot] = k_new[b, row]
        vc[page, slot] = v_new[b, row]
    return kc, vc, ctx


# ----------------------------------------------------------------------------
# confidence-threshold and hybrid acceptance
# ----------------------------------------------------------------------------

def draft_confidence(draft_logits, draft_ids):
    """[B, W] fp64: the drafter's softmax probability of each drafted token
    (row i of draft_logits is the distribution that produced draft i;
    "Dynamic Multi-Byte Prediction With Hierarchical Language Models" Sec. 3.1:
    a predicted byte is accepted when the model's probability for it reaches
    the threshold).  Mask tokens (draft < 0) and row 0 get confidence 0."""
    x = np.asarray(draft_logits, dtype=np.float64)
    B, W, V = x.shape
    conf = np.zeros((B, W))
    for b in range(B):
        for i in range(1, W):
            d = int(draft_ids[b, i])
            if d < 0 or d >= V:
                continue
            row = x[b, i]
            m = row.max()
            e = np.exp(row - m)
            conf[b, i] = e[d] / e.sum()
    return conf


def accept_hybrid(draft_logits, logits, draft_ids, mask_kind, mask_ids, tau, min_prefix):
    """Hybrid acceptance ("BitMTP: When Multi-Token Prediction Meets Low-Bit
    Large Language Models", Sec. 3.3): the confidence prefix h is the number of
    leading drafts whose confidence reaches tau (mask tokens never count; a tree takes the deepest root
    path of confident nodes, smallest index on ties; Sec. 3.1 of the
    multi-byte page: left to right, the first below the threshold and
    everything after it discarded).  If h >= min_prefix the h draft tokens are
    committed without the verifier: the step emits h tokens, the last of which
    becomes the next anchor, so accept_len = h - 1 (drafts committed besides
    the anchor), the path is the root path of the h-th token's parent and the
    bonus is the h-th draft token.  Otherwise the greedy verification result
    (``accept``) is used; ``logits`` may be None, and then those sequences get
    -1 outputs.  Returns accept_len, accept_path, bonus_id, conf_len (h)."""
    draft_logits = np.asarray(draft_logits)
    B, W = draft_logits.shape[0], draft_logits.shape[1]
    conf = draft_confidence(draft_logits, draft_ids)
    if logits is not None:
        v_len, v_path, v_bonus = accept(logits, draft_ids, mask_kind, mask_ids)
    acc_len = np.full(B, -1, dtype=np.int64)
    path = np.full((B, W), -1, dtype=np.int64)
    bonus = np.full(B, -1, dtype=np.int64)
    conf_len = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        kind, ids = int(mask_kind[b]), np.asarray(mask_ids[b])
        if not mask_is_valid(kind, ids):
            continue
        par = acceptance_parents(kind, ids)
        ok = np.zeros(W, dtype=bool)
        depth = np.zeros(W, dtype=np.int64)
        ok[0] = True
        for i in range(1, W):
            p = int(par[i])
            depth[i] = depth[p] + 1
            token = 0 <= int(draft_ids[b, i]) < draft_logits.shape[2]
            ok[i] = ok[p] and token and conf[b, i] >= tau
        best = 0
        for i in range(1, W):
            if ok[i] and depth[i] > depth[best]:
                best = i
        h = int(depth[best])
        conf_len[b] = h
        if h >= min_prefix and h >= 1:
            chain = []
            j = int(par[best])
            while j >= 0:
                chain.append(j)
                j = int(par[j])
            chain.reverse()
            acc_len[b] = h - 1
            path[b, :len(chain)] = chain
            bonus[b] = int(draft_ids[b, best])
        elif logits is not None:
            acc_len[b], path[b], bonus[b] = v_len[b], v_path[b], v_bonus[b]
    return acc_len, path, bonus, conf_len


# ----------------------------------------------------------------------------
# nested KV4 / KV8 cache
# ----------------------------------------------------------------------------
#
# "BitNest: Bit-Nested Speculative Decoding for Memory-Efficient LLM Inference
# Acceleration", §3.4 and §A.2.  Every cached K or V vector of one token and
# one KV head is quantized once, when it is written: symmetric round-to-nearest
# at a per-vector scale s gives the 4-bit base codes (the KV4 view, s * q4);
# the base's residual is quantized again at the sixteen-times finer scale s/16
# into 4-bit refinement codes, and base + refinement is the KV8 view,
# (s/16) * (16 q4 + qr).  The two code planes are stored separately, so a
# reader takes the base alone (KV4) or both (KV8).
#
# The pages leave the scale rule and the rounding open; the reading used here:
#   s = max|x| / 7 (so the base uses codes -7..7), t = x / s, q4 = rint(t),
#   qr = clamp(rint(16 t) - 16 q4, -8, 7), rint = round half to even, all in
#   fp32 (the codes are integers decided by floating point: both sides decide
#   in fp32).  A zero vector has s = 0 and zero codes.
# Storage: codes + 8 as unsigned nibbles, two per byte, the even element in
# the low nibble; planes [pages, Hkv, 16, D/2] bytes; scales [pages, Hkv, 16]
# fp32 (the 16 slots of one page and head are contiguous).
# Reading policy (§3.4, §A.2): verification reads KV8; drafting reads KV4;
# "Recent-N" reads the N most recent committed tokens in KV8 and older ones
# in KV4.  kv8_recent = -1 means all KV8, 0 all KV4, N > 0 Recent-N.

NEST_OFFSET = 8


def quantize_nested(x):
    """x [..., D] (finite) -> base codes q4, refinement codes qr (int64, in
    [-8, 7]) and the fp32 scale s [...]."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    s = (amax / np.float32(7.0)).astype(np.float32)
    live = s > 0
    t = (x / np.where(live, s, np.float32(1.0))[..., None]).astype(np.float32)
    q4 = np.rint(t)
    qr = np.clip(np.rint(t * np.float32(16.0)) - 16.0 * q4, -8, 7)
    q4 = np.where(live[..., None], q4, 0).astype(np.int64)
    qr = np.where(live[..., None], qr, 0).astype(np.int64)
    return q4, qr, s


def pack_nibbles(codes):
    """[..., D] codes in [-8, 7] -> [..., D/2] bytes (code + 8, even element low)."""
    u = (np.asarray(codes) + NEST_OFFSET).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int64)
    out[..., 0::2] = (packed & 15).astype(np.int64) - NEST_OFFSET
    out[..., 1::2] = (packed >> 4).astype(np.int64) - NEST_OFFSET
    return out


def nested_planes(cache):
    """Quantizes a whole [pages, 16, Hkv, D] cache into its nested planes."""
    q4, qr, s = quantize_nested(cache)
    return {"base": np.ascontiguousarray(pack_nibbles(q4).transpose(0, 2, 1, 3)),
            "ref": np.ascontiguousarray(pack_nibbles(qr).transpose(0, 2, 1, 3)),
            "scale": np.ascontiguousarray(s.transpose(0, 2, 1))}


def dequantize_nested(planes, level):
    """KV8 (level 8) or KV4 (level 4) view of nested planes as a
    [pages, 16, Hkv, D] fp64 cache (exact)."""
    q4 = unpack_nibbles(planes["base"]).astype(np.float64)
    s = np.asarray(planes["scale"], dtype=np.float64)[..., None]
    if level == 4:
        v = s * q4
    elif level == 8:
        qr = unpack_nibbles(planes["ref"]).astype(np.float64)
        v = s * (16.0 * q4 + qr) / 16.0
    else:
        raise ValueError("level must be 4 or 8")
    return v.transpose(0, 2, 1, 3)


def verify_attention_nested(q, k_planes, v_planes, block_table, ctx_lens, k_new, v_new,
                            mask_kind, mask_ids, scale=None, seg_lookback=-1, kv8_recent=-1):
    """Verify attention over a nested cache: committed token t of a sequence
    with context L is read in KV8 when kv8_recent < 0 or t >= L - kv8_recent,
    else in KV4; the block's own rows (k_new, v_new) are used as given."""
    views = {lvl: (dequantize_nested(k_planes, lvl), dequantize_nested(v_planes, lvl))
             for lvl in (4, 8)}

    def committed(b):
        L = int(ctx_lens[b])
        k8 = gather_committed(views[8][0], block_table[b], L)
        v8 = gather_committed(views[8][1], block_table[b], L)
        if kv8_recent < 0:
            return k8, v8
        k4 = gather_committed(views[4][0], block_table[b], L)
        v4 = gather_committed(views[4][1], block_table[b], L)
        old = np.arange(L) < L - kv8_recent
        return np.where(old[:, None, None], k4, k8), np.where(old[:, None, None], v4, v8)

    return attention_over(q, committed, k_new, v_new, mask_kind, mask_ids, scale, seg_lookback)


def kv_commit_nested(k_planes, v_planes, k_new, v_new, accept_len, accept_path, block_table,
                     ctx_lens, skip_root=False):
    """The commit of ``kv_commit`` into a nested cache: each accepted row is
    quantized (``quantize_nested``) into its slot's codes and scale.  Returns
    new plane dicts and the new context lengths."""
    kp = {k: np.array(v, copy=True) for k, v in k_planes.items()}
    vp = {k: np.array(v, copy=True) for k, v in v_planes.items()}
    writes, ctx = commit_writes(accept_len, accept_path, block_table, ctx_lens,
                                kp["scale"].shape[0], skip_root)
    for b, page, slot, row in writes:
        for planes, src in ((kp, k_new), (vp, v_new)):
            q4, qr, sc = quantize_nested(np.asarray(src[b, row], dtype=np.float32))
            planes["base"][page, :, slot] = pack_nibbles(q4)
            planes["ref"][page, :, slot] = pack_nibbles(qr)
            planes["scale"][page, :, slot] = sc
    return kp, vp, ctx


# ----------------------------------------------------------------------------
# dynamic token tree (block construction for the next verify step)
# ----------------------------------------------------------------------------
#
# "Efficient Training-Free Multi-Token Prediction via Embedding-Space
# Probing", §2.C (dynamic tree: expansion by cumulative probability, only the
# top-1 token of each depth expanded, a fixed block-complexity budget, pruning
# of consecutive repeated tokens) and §2.D (block = last token + predicted
# tokens + mask tokens; masks and positions by offsets).  Reading used here:
#   * inputs: the drafter's probabilities p_d over the vocabulary for depths
#     d = 1..K (fp32), the last committed token (the root), the block width W
#     and the number of mask-token rows n_mask; W - 1 - n_mask rows hold
#     predicted tokens;
#   * pruning: at depth d a token equal to its parent's token is dropped;
#   * the top-1 (spine) token s_d of depth d is the most probable remaining
#     token (smallest id on ties); only spine nodes get children, so every
#     depth-d candidate is a child of s_{d-1} with cumulative probability
#     c_{d-1} * p_d(v), c_0 = 1, c_d = c_{d-1} * p_d(s_d) (fp32 products, in
#     this order: the comparisons are taken in the kernel's precision);
#   * expansion: best first by cumulative probability (ties: shallower, then
#     more probable at its depth, then smaller id) while prediction rows remain
#     and the best candidate reaches min_cum_prob;
#   * rows: 0 = root (draft = root token, parent -1), then the chosen nodes in
#     the order chosen (parents always come earlier), then mask-token rows
#     (draft -1): a chain hanging from the deepest chosen spine node (the
#     root if none).  depth = the row's distance from the root, the position
#     offset of the row.

def depth_candidates(p_row, parent_token):
    """Tokens of one depth, most probable first (smallest id on ties),
    without the parent's token (no consecutive repeats)."""
    return sorted((v for v in range(len(p_row)) if v != parent_token),
                  key=lambda v: (-float(p_row[v]), v))


def dynamic_tree(probs, root_token, W, n_mask, min_cum_prob=0.0):
    """probs [B, K, V] fp32 -> draft_ids, parents, depth [B, W] and n_nodes [B]
    (root + chosen predicted tokens)."""
    probs = np.asarray(probs, dtype=np.float32)
    B, K, V = probs.shape
    slots = W - 1 - n_mask
    thr = np.float32(min_cum_prob)
    draft = np.full((B, W), -1, dtype=np.int64)
    parent = np.full((B, W), -1, dtype=np.int64)
    depth = np.zeros((B, W), dtype=np.int64)
    n_nodes = np.zeros(B, dtype=np.int64)
    for b in range(B):
        # candidates of every depth, most probable first, without the repeat
        spine_tok = [int(root_token[b])]
        c = [np.float32(1.0)]
        lists = []
        for d in range(1, K + 1):
            order = depth_candidates(probs[b, d - 1], spine_tok[d - 1])
            if not order:  # a one-token vocabulary: nothing below the root
                break
            lists.append(order)
            spine_tok.append(order[0])
            c.append(np.float32(c[d - 1] * probs[b, d - 1, order[0]]))
        # best-first expansion: the frontier holds the next unused candidate
        # of every depth whose parent (the spine node above) is in the tree
        draft[b, 0], parent[b, 0], depth[b, 0] = spine_tok[0], -1, 0
        spine_row = {0: 0}
        nxt = {1: 0} if lists else {}
        rows = 1
        while rows - 1 < slots and nxt:
            best = None
            for d, r in nxt.items():
                v = lists[d - 1][r]
                cp = np.float32(c[d - 1] * probs[b, d - 1, v])
                key = (-float(cp), d, r)
                if best is None or key < best[0]:
                    best = (key, d, r, v, cp)
            _, d, r, v, cp = best
            if cp < thr:
                break
            draft[b, rows], parent[b, rows], depth[b, rows] = v, spine_row[d - 1], d
            if r == 0:  # the spine node of depth d: its children become candidates
                spine_row[d] = rows
                if d + 1 <= len(lists):
                    nxt[d + 1] = 0
            rows += 1
            if r + 1 < len(lists[d - 1]):
                nxt[d] = r + 1
            else:
                del nxt[d]
        n_nodes[b] = rows
        tail = spine_row[max(spine_row)]
        for i in range(rows, W):
            draft[b, i], parent[b, i], depth[b, i] = -1, tail, depth[b, tail] + 1
            tail = i
    return draft, parent, depth, n_nodes


# ----------------------------------------------------------------------------
# block positions (verifier-input preparation on the device)
# ----------------------------------------------------------------------------

def block_positions(ctx_lens, mask_kind, mask_ids):
    """[B, W] position of every block row: the committed length plus the
    row's depth below the anchor ("BitMTP" §3.4 M3: the verifier's positions
    follow the materialized KV boundary; "Efficient Training-Free Multi-Token
    Prediction via Embedding-Space Probing" §2.D: position indices by
    offsets).  Chain and segment blocks are sequential (depth = row index);
    a tree row's depth is its number of ancestors.  A malformed mask gives -1
    for the whole sequence."""
    mask_ids = np.asarray(mask_ids)
    B, W = mask_ids.shape
    pos = np.full((B, W), -1, dtype=np.int64)
    for b in range(B):
        kind, ids = int(mask_kind[b]), mask_ids[b]
        if not mask_is_valid(kind, ids):
            continue
        for i in range(W):
            depth, j = 0, i
            if kind == TREE:
                while j > 0:
                    j = int(ids[j])
                    depth += 1
            else:
                depth = i
            pos[b, i] = int(ctx_lens[b]) + depth
    return pos
