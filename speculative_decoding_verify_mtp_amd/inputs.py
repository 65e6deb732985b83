"""Seeded synthetic inputs for the multi-token verify step.

This module only *draws* inputs: shapes, page tables, context lengths, draft
trees, segment ids, token ids and random tensor values.  It holds none of the
verify step's arithmetic (no attention, no argmax, no acceptance, no commit),
so both the fp64 oracle and the HIP path can consume exactly the same bytes.

Workload shapes follow the problem statement shared by the pages: a width-W
block of drafted or mask positions (row 0 is the last committed token, the
"anchor"/root) verified against a paged KV cache of 16-token pages with GQA,
with the in-block mask given as a parent-index array (chain or tree) or a
segment-id array.

Recipe (all drawn from one seed):
  * structure (context lengths, page permutation, parents, segment ids,
    target/draft ids) from ``numpy.random.default_rng(seed)``;
  * tensor values (Q, cached K/V, in-block K/V, logits) i.i.d. N(0,1) from a
    ``torch.Generator`` seeded with ``seed`` on the device that holds them,
    rounded to bf16 (round-to-nearest-even) or kept fp32;
  * cache slots that hold no committed token (the tail of a sequence's last
    page, the commit workspace slots, spare pages) are NaN, so that a kernel
    reading outside the committed range poisons its output;
  * target ids uniform in [0, vocab); the logits row of a position is
    N(0,1) with its target lifted to (row max + 1), so the argmax is unique;
  * a drafted child of node p equals target[p] with probability ``match_p``
    (first child; if it misses, one other child matches with probability
    1/2); other siblings get distinct non-matching ids, so the accepted path
    is unique;
  * drafter logits (for confidence acceptance): N(0, 0.1^2) per entry, with
    the drafted token's logit set to log(p / (1 - p)) + log(vocab - 1), where
    the intended probability p is drawn from CONFIDENT_PROBS with probability
    ``conf_p``, else from DOUBTFUL_PROBS; the drafted token's softmax
    probability is then p up to the noise of the other entries (a few
    thousandths of the odds), so with 7 or more tokens every confidence
    stays at least 0.04 away from a 0.9 threshold.  Drawn after every other input, so the other
    inputs do not depend on these.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace, asdict

import numpy as np
import torch

PAGE_SIZE = 16
MASK_CHAIN, MASK_TREE, MASK_SEGMENT = 0, 1, 2


CONFIDENT_PROBS = (0.95, 0.99, 0.999)
DOUBTFUL_PROBS = (0.05, 0.3, 0.75)


@dataclass(frozen=True)
class Workload:
    """One synthetic verify-step workload."""

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    W: int
    dtype: str  # "f32" or "bf16"
    ctx_lo: int
    ctx_hi: int  # context lengths uniform integers in [ctx_lo, ctx_hi]
    masks: str  # "chain" | "tree" | "segment" | "mixed" (even b chain, odd b tree)
    seg_lookback: int = -1  # SEGMENT: -1 = all earlier segments, k >= 0 = k previous
    tree_depth: int = 8  # TREE: maximum depth (edges from the root)
    seg_max: int = 6  # SEGMENT: segment lengths uniform in [1, seg_max]
    match_p: float = 0.7
    shuffle_pages: bool = True
    spare_pages: int = 64
    vocab: int = 1000
    mask_token_rows: int = 0  # trailing rows whose draft id is -1 (never accepted)
    conf_p: float = 0.8  # probability that a draft's logit lift is a confident one
    commit_steps: int = 1  # pages are mapped for this many steps of W committed rows

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


# The five synthetic workloads of the verify step (sizes and distributions as
# stated for the method's problem; seeds are 1000 + index).
WORKLOADS = {
    "tiny_chain": Workload("tiny_chain", B=1, Hq=4, Hkv=4, D=64, W=4, dtype="f32",
                           ctx_lo=256, ctx_hi=256, masks="chain", shuffle_pages=False),
    "bitnet2b_chain": Workload("bitnet2b_chain", B=1, Hq=20, Hkv=5, D=128, W=8,
                               dtype="bf16", ctx_lo=4096, ctx_hi=4096, masks="chain"),
    "llama3_8b_tree": Workload("llama3_8b_tree", B=1, Hq=32, Hkv=8, D=128, W=32,
                               dtype="bf16", ctx_lo=8192, ctx_hi=8192, masks="tree"),
    "lca_segments": Workload("lca_segments", B=4, Hq=16, Hkv=16, D=64, W=16,
                             dtype="bf16", ctx_lo=16384, ctx_hi=16384, masks="segment",
                             seg_lookback=-1),
    "ragged_batch": Workload("ragged_batch", B=64, Hq=32, Hkv=8, D=128, W=16,
                             dtype="bf16", ctx_lo=512, ctx_hi=32768, masks="mixed"),
}
WORKLOAD_ORDER = ["tiny_chain", "bitnet2b_chain", "llama3_8b_tree", "lca_segments",
                  "ragged_batch"]


def workload_seed(name: str) -> int:
    return 1000 + WORKLOAD_ORDER.index(name) + 1


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


# ----------------------------------------------------------------------------
# structure
# ----------------------------------------------------------------------------

def chain_parents(W: int) -> np.ndarray:
    p = np.arange(-1, W - 1, dtype=np.int32)
    return p


def random_tree_parents(rng: np.random.Generator, W: int, max_depth: int) -> np.ndarray:
    """Nodes 0..min(W-1, max_depth) form the top-1 chain; every later node takes
    a uniform parent among the existing nodes shallower than ``max_depth``.
    Parents always precede children (parent[i] < i)."""
    parent = np.full(W, -1, dtype=np.int32)
    depth = np.zeros(W, dtype=np.int32)
    chain_len = min(W, max_depth + 1)
    for i in range(1, chain_len):
        parent[i] = i - 1
        depth[i] = i
    for i in range(chain_len, W):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(rng.choice(cand))
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def random_segments(rng: np.random.Generator, W: int, seg_max: int) -> np.ndarray:
    """Segment ids for W positions: lengths uniform in [1, seg_max] until the
    block is covered, the last segment truncated.  ids start at 0 and step by
    0 or +1."""
    seg = np.zeros(W, dtype=np.int32)
    pos, sid = 0, 0
    while pos < W:
        n = int(rng.integers(1, seg_max + 1))
        seg[pos:pos + n] = sid
        pos += n
        sid += 1
    return seg


def draw_drafts(rng: np.random.Generator, parent: np.ndarray, tgt: np.ndarray, vocab: int,
                match_p: float, mask_token_rows: int) -> np.ndarray:
    """Draft ids for one block.  ``parent`` gives, per node, the node whose
    prediction the draft is compared with (chain: i-1)."""
    W = parent.shape[0]
    draft = np.full(W, -1, dtype=np.int32)
    children: dict[int, list[int]] = {}
    for i in range(1, W):
        children.setdefault(int(parent[i]), []).append(i)
    for p, kids in children.items():
        want = int(tgt[p])
        matched = -1
        if rng.random() < match_p:
            matched = kids[0]
        elif len(kids) > 1 and rng.random() < 0.5:
            matched = kids[int(rng.integers(1, len(kids)))]
        # distinct non-matching ids for the siblings
        pool = rng.choice(vocab - 1, size=len(kids), replace=False)
        pool = np.where(pool >= want, pool + 1, pool)  # skip the target id
        for c, alt in zip(kids, pool):
            draft[c] = want if c == matched else int(alt)
    if mask_token_rows:
        draft[W - mask_token_rows:] = -1
    draft[0] = -1  # the root carries no draft
    return draft


def make_structure(wl: Workload, seed: int) -> dict:
    """All integer inputs of one workload (host numpy arrays)."""
    rng = np.random.default_rng(seed)
    B, W = wl.B, wl.W
    if wl.ctx_lo == wl.ctx_hi:
        ctx = np.full(B, wl.ctx_lo, dtype=np.int32)
    else:
        ctx = rng.integers(wl.ctx_lo, wl.ctx_hi + 1, size=B).astype(np.int32)

    kinds = np.zeros(B, dtype=np.uint8)
    ids = np.zeros((B, W), dtype=np.int32)
    accept_parent = np.zeros((B, W), dtype=np.int32)
    for b in range(B):
        kind = {"chain": MASK_CHAIN, "tree": MASK_TREE, "segment": MASK_SEGMENT,
                "mixed": MASK_CHAIN if b % 2 == 0 else MASK_TREE}[wl.masks]
        kinds[b] = kind
        if kind == MASK_CHAIN:
            ids[b] = chain_parents(W)
            accept_parent[b] = chain_parents(W)
        elif kind == MASK_TREE:
            ids[b] = random_tree_parents(rng, W, wl.tree_depth)
            accept_parent[b] = ids[b]
        else:
            ids[b] = random_segments(rng, W, wl.seg_max)
            accept_parent[b] = chain_parents(W)

    # pages: every logical slot up to ctx + commit_steps * W - 1 is mapped
    # (commit workspace)
    n_pages = [(int(L) + wl.commit_steps * W + PAGE_SIZE - 1) // PAGE_SIZE for L in ctx]
    pool = int(sum(n_pages)) + wl.spare_pages
    order = rng.permutation(pool).astype(np.int32) if wl.shuffle_pages else \
        np.arange(pool, dtype=np.int32)
    max_pages = max(n_pages)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    cur = 0
    for b in range(B):
        table[b, :n_pages[b]] = order[cur:cur + n_pages[b]]
        cur += n_pages[b]

    tgt = rng.integers(0, wl.vocab, size=(B, W)).astype(np.int32)
    draft = np.stack([draw_drafts(rng, accept_parent[b], tgt[b], wl.vocab, wl.match_p,
                                  wl.mask_token_rows) for b in range(B)])
    confident = rng.random((B, W)) < wl.conf_p
    p = np.where(confident, rng.choice(CONFIDENT_PROBS, size=(B, W)),
                 rng.choice(DOUBTFUL_PROBS, size=(B, W)))
    lift = (np.log(p / (1 - p)) + math.log(max(wl.vocab - 1, 1))).astype(np.float32)
    lift_tok = np.where(draft >= 0, draft, rng.integers(0, wl.vocab, size=(B, W))).astype(np.int32)
    return dict(ctx_lens=ctx, mask_kind=kinds, mask_ids=ids, block_table=table,
                num_pages=pool, target_ids=tgt, draft_ids=draft, draft_lift=lift,
                draft_lift_token=lift_tok)


def valid_slots(block_table: np.ndarray, ctx_lens: np.ndarray, num_pages: int) -> np.ndarray:
    """[num_pages, PAGE_SIZE] bool: True where a slot holds a committed token."""
    valid = np.zeros((num_pages, PAGE_SIZE), dtype=bool)
    for b in range(block_table.shape[0]):
        L = int(ctx_lens[b])
        full, rem = divmod(L, PAGE_SIZE)
        pages = block_table[b]
        valid[pages[:full]] = True
        if rem:
            valid[pages[full], :rem] = True
    return valid


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------

def _randn(shape, gen, device, dtype, chunk_rows: int | None = None) -> torch.Tensor:
    """N(0,1) drawn in fp32 and rounded to ``dtype``; drawn in chunks along
    dim 0 so multi-GB pools never need an fp32 copy."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    step = rows if chunk_rows is None else max(1, chunk_rows)
    for s in range(0, rows, step):
        e = min(rows, s + step)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                               dtype=torch.float32).to(dtype)
    return out


def make_inputs(wl: Workload, seed: int, device: str | torch.device = "cpu",
                poison: bool = True) -> dict:
    """Every input of one verify step as tensors on ``device`` (integer
    structure is also returned as host numpy under ``host``)."""
    device = torch.device(device)
    st = make_structure(wl, seed)
    B, W, Hq, Hkv, D = wl.B, wl.W, wl.Hq, wl.Hkv, wl.D
    dt = torch_dtype(wl.dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    npages = st["num_pages"]
    per_page = PAGE_SIZE * Hkv * D
    chunk = max(1, (64 << 20) // per_page)
    q = _randn((B, W, Hq, D), gen, device, dt)
    k_cache = _randn((npages, PAGE_SIZE, Hkv, D), gen, device, dt, chunk)
    v_cache = _randn((npages, PAGE_SIZE, Hkv, D), gen, device, dt, chunk)
    k_new = _randn((B, W, Hkv, D), gen, device, dt)
    v_new = _randn((B, W, Hkv, D), gen, device, dt)
    logits = torch.randn((B, W, wl.vocab), generator=gen, device=device, dtype=torch.float32)
    tgt = torch.from_numpy(st["target_ids"]).to(device=device, dtype=torch.int64)
    lift = logits.amax(dim=-1, keepdim=True) + 1.0
    logits.scatter_(-1, tgt.unsqueeze(-1), lift)
    draft_logits = 0.1 * torch.randn((B, W, wl.vocab), generator=gen, device=device,
                                     dtype=torch.float32)
    lt = torch.from_numpy(st["draft_lift_token"]).to(device=device, dtype=torch.int64)
    draft_logits.scatter_(-1, lt.unsqueeze(-1),
                          torch.from_numpy(st["draft_lift"]).to(device).unsqueeze(-1))
    if poison:
        valid = torch.from_numpy(valid_slots(st["block_table"], st["ctx_lens"], npages))
        invalid = (~valid).to(device)
        k_cache[invalid] = float("nan")
        v_cache[invalid] = float("nan")

    def it(a, dtype=torch.int32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)

    return dict(
        workload=wl, seed=seed, host=st,
        q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
        block_table=it(st["block_table"]), ctx_lens=it(st["ctx_lens"]),
        mask_kind=it(st["mask_kind"], torch.uint8), mask_ids=it(st["mask_ids"]),
        logits=logits, draft_ids=it(st["draft_ids"]), draft_logits=draft_logits,
        seg_lookback=wl.seg_lookback, scale=1.0 / math.sqrt(D),
    )


def kv_bytes(wl: Workload, ctx_lens: np.ndarray) -> int:
    """Committed K+V bytes one verify step must read (the headline numerator)."""
    elem = 4 if wl.dtype == "f32" else 2
    return int(np.sum(ctx_lens.astype(np.int64))) * wl.Hkv * wl.D * 2 * elem


def make_tree_inputs(B: int, K: int, V: int, seed: int, peak: float = 8.0, device="cpu") -> dict:
    """Drafter probabilities for the tree builder: per (sequence, depth) a
    heavy-tailed distribution (uniform draws to the power `peak`, normalised
    in fp32), and a root token per sequence."""
    rng = np.random.default_rng(seed)
    w = rng.random((B, K, V)) ** peak
    probs = (w / w.sum(axis=-1, keepdims=True)).astype(np.float32)
    root = rng.integers(0, V, size=B).astype(np.int32)
    return dict(probs=torch.from_numpy(probs).to(device), root=torch.from_numpy(root).to(device),
                host=dict(probs=probs, root=root))
