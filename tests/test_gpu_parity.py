"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Attention within |d| <= 1e-3 + 1e-2 |ref| elementwise (bf16 inputs) or
1e-4 + 1e-4 |ref| (fp32 inputs); acceptance, paths, bonus ids, context
lengths and committed K/V bytes bit-exact.  Cases span several 32-key
tiles, several splits and ragged tails, more than 64 splits per row, equal-
depth tree ties and the finish launch with more sequences than compute units
can take beside it.  The five full-size workloads are in test_gpu_full_size.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_common import (I, O, lib, assert_accept_equal, assert_attn_close, f64, gpu_inputs,
                              ints, oracle_accept, oracle_attn, raw, run_attn, tol_for)

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore::RuntimeWarning"),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def W_(name, **kw) -> I.Workload:
    base = dict(name=name, B=2, Hq=8, Hkv=2, D=128, W=8, dtype="bf16", ctx_lo=100, ctx_hi=700,
                masks="chain")
    base.update(kw)
    return I.Workload(**base)


SMALL = [
    I.WORKLOADS["tiny_chain"],
    W_("chain_g4", Hq=20, Hkv=5, W=8, ctx_lo=300, ctx_hi=700),
    W_("tree_w32", Hq=32, Hkv=8, W=32, ctx_lo=500, ctx_hi=1100, masks="tree"),
    W_("segment_all", Hq=16, Hkv=16, D=64, W=16, ctx_lo=200, ctx_hi=600, masks="segment"),
    W_("segment_lca", Hq=16, Hkv=16, D=64, W=16, ctx_lo=200, ctx_hi=600, masks="segment",
       seg_lookback=1),
    W_("segment_own", Hq=4, Hkv=1, D=64, W=20, ctx_lo=0, ctx_hi=90, masks="segment",
       seg_lookback=0),
    W_("mixed_b6", B=6, Hq=32, Hkv=8, W=16, ctx_lo=0, ctx_hi=900, masks="mixed"),
    W_("valu_bf16_r3", Hq=4, Hkv=4, W=3, ctx_lo=50, ctx_hi=333, masks="tree"),
    W_("valu_bf16_d64", Hq=6, Hkv=3, D=64, W=7, ctx_lo=17, ctx_hi=81, masks="mixed"),
    W_("fp32_d128_tree", Hq=8, Hkv=2, W=5, dtype="f32", ctx_lo=40, ctx_hi=300, masks="tree"),
    W_("fp32_d64_seg", Hq=3, Hkv=1, D=64, W=9, dtype="f32", ctx_lo=0, ctx_hi=64,
       masks="segment", seg_lookback=1),
    W_("w1_decode", B=3, Hq=16, Hkv=2, W=1, ctx_lo=1, ctx_hi=500),
    W_("w1_decode_d64", B=3, Hq=32, Hkv=2, D=64, W=1, ctx_lo=0, ctx_hi=200),
    W_("w64_tree", Hq=4, Hkv=2, W=64, ctx_lo=90, ctx_hi=400, masks="tree", tree_depth=63),
    W_("w64_chain_d64", Hq=2, Hkv=2, D=64, W=64, ctx_lo=1, ctx_hi=130),
    W_("w33_mixed_g8", B=3, Hq=64, Hkv=8, W=33, ctx_lo=31, ctx_hi=97, masks="mixed"),
    # 192 rows per KV head: three row blocks per (split, head), 18 such units,
    # so both the XCD-paired groups of eight units and the tail are used
    W_("row_blocks3_hkv3", B=3, Hq=36, Hkv=3, W=16, ctx_lo=100, ctx_hi=1500, masks="mixed"),
    W_("ctx0", B=3, Hq=8, Hkv=8, W=16, ctx_lo=0, ctx_hi=0, masks="mixed"),
    W_("ctx_page_edges", B=4, Hq=8, Hkv=1, W=4, ctx_lo=15, ctx_hi=17),
    W_("mask_tokens", Hq=16, Hkv=4, W=12, ctx_lo=64, ctx_hi=64, mask_token_rows=4),
    # 4096 output rows with few splits: the combine takes four rows per wave
    W_("grouped_d64", B=4, Hq=64, Hkv=16, D=64, W=16, ctx_lo=50, ctx_hi=700, masks="mixed"),
    W_("grouped_fp32", B=2, Hq=64, Hkv=64, D=64, W=32, dtype="f32", ctx_lo=20, ctx_hi=300,
       masks="tree"),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_attention_matches_oracle_small(wl):
    inp = gpu_inputs(wl, 7)
    out, lse = run_attn(inp)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=wl.name)


# Magnitudes far from N(0, 1).  Very large scores used to overflow the
# exponential (an fma's exact product against the rounded reference max left
# a residual of half an ulp, above 2^31 more than the exponent range) and gave
# NaN rows; tiny ones must not vanish.  Attention is linear in V and the
# softmax sees only q.k, so each case compares out / (V scale).  One
# workload per kernel family: the stream kernel (nine sequences), the
# per-split LDS kernel (two), the D = 64 direct-load kernel and the fp32 VALU
# kernel.
EXTREME = [(1e-30, 1.0, 1.0), (1e30, 1.0, 1.0), (1.0, 1e-20, 1.0), (1.0, 1e12, 1.0),
           (1.0, 1.0, 1e-20), (1.0, 1.0, 1e20)]
EXTREME_WL = [
    W_("x_stream", B=9, Hq=16, Hkv=4, W=8, ctx_lo=20, ctx_hi=900, masks="mixed"),
    W_("x_lds", B=2, Hq=16, Hkv=4, W=8, ctx_lo=20, ctx_hi=900, masks="mixed"),
    W_("x_d64", B=2, Hq=16, Hkv=16, D=64, W=16, ctx_lo=20, ctx_hi=600, masks="segment",
       seg_lookback=1),
    W_("x_fp32", B=2, Hq=4, Hkv=4, D=64, W=4, dtype="f32", ctx_lo=20, ctx_hi=300),
]


@pytest.mark.parametrize("qs,ks,vs", EXTREME, ids=[f"q{a:g}_k{b:g}_v{c:g}" for a, b, c in EXTREME])
@pytest.mark.parametrize("wl", EXTREME_WL, ids=[w.name for w in EXTREME_WL])
def test_extreme_magnitudes(wl, qs, ks, vs):
    inp = gpu_inputs(wl, 33)
    inp["q"].mul_(qs)
    for key, f in (("k_cache", ks), ("k_new", ks), ("v_cache", vs), ("v_new", vs)):
        inp[key].mul_(f)
    out, lse = run_attn(inp)
    assert lib.device_status(clear=True) == 0
    ref_out, ref_lse = oracle_attn(inp)
    assert np.isfinite(out.cpu().numpy()).all(), f"{wl.name} q{qs} k{ks} v{vs}: non-finite output"
    assert_attn_close(out / vs, lse, ref_out / vs, ref_lse, *tol_for(wl),
                      what=f"{wl.name} q{qs} k{ks} v{vs}")


@pytest.mark.parametrize("split", [32, 64, 96, 128, 2048])
def test_split_size_does_not_change_the_result(split):
    wl = W_("splits", B=3, Hq=16, Hkv=4, W=8, ctx_lo=1, ctx_hi=700, masks="mixed")
    inp = gpu_inputs(wl, 3)
    out, lse = run_attn(inp, split_tokens=split)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"split {split}")


@pytest.mark.parametrize("split", [64, 1024, 2048])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_valu_long_splits_match_oracle(split, dtype):
    # fewer than 16 rows per KV head: the vector-ALU kernel, whose splits
    # span up to 128 pages and end on ragged steps of the key groups
    wl = W_("valu_long", B=3, Hq=4, Hkv=2, W=3, dtype=dtype, ctx_lo=1500, ctx_hi=2600,
            masks="mixed")
    inp = gpu_inputs(wl, 11)
    out, lse = run_attn(inp, split_tokens=split)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"valu split {split} {dtype}")


@pytest.mark.parametrize("B", [1024, 1100])
def test_batch_at_and_above_the_stream_table(B):
    """1024 sequences fill the stream schedule's stage table exactly; more
    run the per-split LDS kernel instead."""
    wl = W_(f"b{B}", B=B, Hq=4, Hkv=1, W=4, ctx_lo=0, ctx_hi=40, masks="mixed", spare_pages=8)
    inp = gpu_inputs(wl, 6)
    out, lse = run_attn(inp)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"B={B}")
    assert lib.device_status(clear=True) == 0


@pytest.mark.parametrize("split", [32, 256, 1024])
def test_stream_work_split_does_not_change_the_result(split):
    """Workgroups of 1, 8 or 32 stages: ranges start and end inside
    segments, pieces per segment vary."""
    wl = W_("stream", B=9, Hq=32, Hkv=8, W=16, ctx_lo=0, ctx_hi=1500, masks="mixed")
    inp = gpu_inputs(wl, 13)
    out, lse = run_attn(inp, split_tokens=split)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"stream split {split}")


STREAM_HEADS = [
    W_("stream_hkv5", B=9, Hq=20, Hkv=5, W=8, ctx_lo=0, ctx_hi=1500, masks="chain"),
    W_("stream_hkv1_rb2", B=8, Hq=16, Hkv=1, W=16, ctx_lo=40, ctx_hi=900, masks="mixed"),
    W_("stream_hkv16", B=10, Hq=32, Hkv=16, W=8, ctx_lo=0, ctx_hi=700, masks="tree"),
    # more KV heads than persistent workgroups: one range per head
    W_("stream_hkv600", B=8, Hq=600, Hkv=600, W=16, ctx_lo=0, ctx_hi=100, masks="chain"),
    # 33 rows per sequence: the combine's four-row waves straddle sequences
    W_("stream_rows_straddle", B=9, Hq=3, Hkv=1, W=11, ctx_lo=0, ctx_hi=400, masks="mixed"),
]


@pytest.mark.parametrize("split", [0, 64])
@pytest.mark.parametrize("wl", STREAM_HEADS, ids=[w.name for w in STREAM_HEADS])
def test_stream_ranges_per_kv_head(wl, split):
    """The stream grid is Hkv workgroups per range: head counts that do and
    do not divide the slot count, one or two row blocks per head."""
    inp = gpu_inputs(wl, 17)
    out, lse = run_attn(inp, split_tokens=split)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"{wl.name} split {split}")


# Two workgroups per CU and at least 32 stages per range: the ranges of the
# first dispatch round are longer than the rest (Hkv = 8: 32 + 32 ranges per
# head; Hkv = 5: 51 + 51).
STREAM_WEIGHTED = [
    W_("stream_weighted_hkv8", B=20, Hq=32, Hkv=8, W=16, ctx_lo=3500, ctx_hi=5500, masks="mixed"),
    W_("stream_weighted_hkv5", B=24, Hq=20, Hkv=5, W=8, ctx_lo=5000, ctx_hi=6000, masks="chain"),
]


# Few sequences over the whole grid: 256 ranges per KV head cross each
# segment, and the combine takes one row per wave.
STREAM_MANY_PIECES = [
    W_("stream_pieces_hkv2", B=8, Hq=32, Hkv=2, W=4, ctx_lo=2000, ctx_hi=4000, masks="mixed"),
    W_("stream_pieces_w16", B=9, Hq=16, Hkv=1, W=4, ctx_lo=100, ctx_hi=3000, masks="tree"),
]


@pytest.mark.parametrize("wl", STREAM_MANY_PIECES, ids=[w.name for w in STREAM_MANY_PIECES])
def test_stream_many_pieces_per_segment(wl):
    inp = gpu_inputs(wl, 29)
    out, lse = run_attn(inp)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=wl.name)


# Fewer than eight sequences, one row tile per wave, ranges of at least four
# stages: the stream kernel (and its row-per-wave combine).
SMALL_BATCH_STREAM = [
    W_("stream_b1", B=1, Hq=32, Hkv=8, W=16, ctx_lo=9000, ctx_hi=9000, masks="chain"),
    W_("stream_b2_hkv5", B=2, Hq=20, Hkv=5, W=8, ctx_lo=8000, ctx_hi=8000, masks="tree"),
    W_("stream_b3_mixed", B=3, Hq=32, Hkv=8, W=16, ctx_lo=3000, ctx_hi=6000, masks="mixed"),
]


@pytest.mark.parametrize("wl", SMALL_BATCH_STREAM, ids=[w.name for w in SMALL_BATCH_STREAM])
def test_small_batch_stream(wl):
    inp = gpu_inputs(wl, 31)
    out, lse = run_attn(inp)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=wl.name)


@pytest.mark.parametrize("wl", STREAM_WEIGHTED, ids=[w.name for w in STREAM_WEIGHTED])
def test_stream_weighted_ranges(wl):
    inp = gpu_inputs(wl, 19)
    out, lse = run_attn(inp)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=wl.name)


# One sequence, 128 rows per KV head (two row blocks of 64), 288 to 512
# items: the splits of the first dispatch round hold 288 tokens, the rest
# 224.  The last case bounds the context at 8192 tokens but holds 3000, so it
# ends inside the long splits.
WEIGHTED_SPLITS = [
    (W_("wsplit_6000", B=1, Hq=32, Hkv=8, W=32, ctx_lo=6000, ctx_hi=6000, masks="tree"), None),
    (W_("wsplit_5000", B=1, Hq=32, Hkv=8, W=32, ctx_lo=5000, ctx_hi=5000, masks="chain"), None),
    (W_("wsplit_bound", B=1, Hq=32, Hkv=8, W=32, ctx_lo=3000, ctx_hi=3000, masks="tree"), 8192),
]


@pytest.mark.parametrize("wl,bound", WEIGHTED_SPLITS, ids=[w.name for w, _ in WEIGHTED_SPLITS])
def test_single_sequence_weighted_splits(wl, bound):
    inp = gpu_inputs(wl, 23)
    if bound is not None:  # a table wide enough for the bound (unmapped entries past the context)
        bt = inp["block_table"]
        pad = torch.full((bt.shape[0], bound // 16 - bt.shape[1]), -1, dtype=bt.dtype, device=bt.device)
        inp["block_table"] = torch.cat([bt, pad], dim=1).contiguous()
    out, lse = run_attn(inp, max_ctx_len=bound)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=wl.name)


PHASES = [
    W_("phase_split", B=3, Hq=20, Hkv=5, W=8, ctx_lo=100, ctx_hi=900),
    W_("phase_stream", B=9, Hq=32, Hkv=8, W=16, ctx_lo=0, ctx_hi=900, masks="mixed"),
    W_("phase_grouped", B=4, Hq=64, Hkv=16, D=64, W=16, ctx_lo=50, ctx_hi=700, masks="mixed"),
]


@pytest.mark.parametrize("wl", PHASES, ids=[w.name for w in PHASES])
def test_partial_then_combine_equals_the_fused_call(wl):
    """mtp_verify_attn_partial then mtp_verify_attn_combine on one workspace
    give exactly what mtp_verify_attn gives (the same kernels in order)."""
    inp = gpu_inputs(wl, 23)
    mc = int(inp["host"]["ctx_lens"].max())
    args = (inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["ctx_lens"],
            inp["k_new"], inp["v_new"], inp["mask_kind"], inp["mask_ids"])
    kw = dict(max_ctx_len=mc, scale=inp["scale"], seg_lookback=inp["seg_lookback"])
    out, lse = lib.verify_attn(*args, **kw)
    ws = torch.empty(max(lib.workspace_bytes(lib.shape_of(inp["q"], inp["k_cache"],
                                                          inp["block_table"], **kw)), 16),
                     dtype=torch.uint8, device=out.device)
    o2 = torch.full_like(out, float("nan"))
    l2 = torch.full_like(lse, float("nan"))
    lib.verify_attn(*args, out=o2, lse=l2, workspace=ws, phase="partial", **kw)
    lib.verify_attn(*args, out=o2, lse=l2, workspace=ws, phase="combine", **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_loose_max_ctx_len_bound():
    """max_ctx_len only sizes the split plan; a loose bound gives the same result."""
    wl = W_("loose", B=2, Hq=8, Hkv=2, W=8, ctx_lo=10, ctx_hi=300, masks="tree")
    inp = gpu_inputs(wl, 4)
    out, lse = run_attn(inp, max_ctx_len=inp["block_table"].shape[1] * 16)
    ref_out, ref_lse = oracle_attn(inp)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl))


# More than 64 splits per row: the combines' loop past their first 64 splits
# (the automatic plan reaches it for one sequence of 64K tokens, as 128
# splits of 512).  ctx 5000 with 64-token splits gives 79 splits.
MANY_SPLITS = [
    W_("splits79_lds", B=1, Hq=20, Hkv=5, W=8, ctx_lo=5000, ctx_hi=5000),
    W_("splits79_d64", B=1, Hq=16, Hkv=4, D=64, W=16, ctx_lo=5000, ctx_hi=5000,
       masks="segment", seg_lookback=1),
    W_("splits79_valu", B=1, Hq=4, Hkv=2, W=3, ctx_lo=5000, ctx_hi=5000, masks="tree"),
    W_("splits79_fp32", B=2, Hq=4, Hkv=4, D=64, W=4, dtype="f32", ctx_lo=4990, ctx_hi=5000),
]


@pytest.mark.parametrize("wl", MANY_SPLITS, ids=[w.name for w in MANY_SPLITS])
def test_more_than_64_splits(wl):
    inp = gpu_inputs(wl, 19)
    ref_out, ref_lse = oracle_attn(inp)
    out, lse = run_attn(inp, split_tokens=64)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"{wl.name} attn")
    n_ref, path_ref, bonus_ref = oracle_accept(inp)
    kc_ref, vc_ref, ctx_ref = O.kv_commit(raw(inp["k_cache"]), raw(inp["v_cache"]),
                                          raw(inp["k_new"]), raw(inp["v_new"]), n_ref, path_ref,
                                          ints(inp["block_table"]), ints(inp["ctx_lens"]))
    out, lse, n, path, bonus, ctx_out = lib.verify_step(
        inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["ctx_lens"],
        inp["k_new"], inp["v_new"], inp["mask_kind"], inp["mask_ids"], inp["logits"],
        inp["draft_ids"], max_ctx_len=int(inp["host"]["ctx_lens"].max()), scale=inp["scale"],
        seg_lookback=inp["seg_lookback"], split_tokens=64)
    torch.cuda.synchronize()
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"{wl.name} step")
    assert_accept_equal((n, path, bonus), (n_ref, path_ref, bonus_ref))
    assert np.array_equal(ints(ctx_out), ctx_ref)
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)


# ----------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------

ACCEPT = [
    W_("acc_chain", B=16, W=8, ctx_lo=1, ctx_hi=1),
    W_("acc_tree", B=16, W=32, ctx_lo=1, ctx_hi=1, masks="tree"),
    W_("acc_tree_w64", B=8, W=64, ctx_lo=1, ctx_hi=1, masks="tree", tree_depth=63, match_p=0.9),
    W_("acc_segment", B=16, W=16, ctx_lo=1, ctx_hi=1, masks="segment"),
    W_("acc_mixed_v7", B=16, W=16, ctx_lo=1, ctx_hi=1, masks="mixed", vocab=7),
    W_("acc_reject_all", B=8, W=16, ctx_lo=1, ctx_hi=1, masks="mixed", match_p=0.0),
    W_("acc_accept_all", B=8, W=16, ctx_lo=1, ctx_hi=1, masks="chain", match_p=1.0),
    W_("acc_mask_tokens", B=8, W=12, ctx_lo=1, ctx_hi=1, masks="chain", match_p=1.0,
       mask_token_rows=5),
    W_("acc_w1", B=4, W=1, ctx_lo=1, ctx_hi=1),
    W_("acc_vocab_big", B=2, W=8, ctx_lo=1, ctx_hi=1, vocab=50000),
]


@pytest.mark.parametrize("wl", ACCEPT, ids=[w.name for w in ACCEPT])
def test_accept_bit_exact(wl):
    inp = gpu_inputs(wl.scaled(D=64, Hq=2, Hkv=2), 11)
    got = lib.accept(inp["logits"], inp["draft_ids"], inp["mask_kind"], inp["mask_ids"])
    assert_accept_equal(got, oracle_accept(inp))


def test_accept_argmax_ties_take_the_smallest_id():
    B, W, V = 3, 4, 300
    logits = torch.zeros((B, W, V), dtype=torch.float32)
    tgt = np.array([[5, 299, 0, 77], [64, 128, 192, 256], [1, 2, 3, 4]])
    for b in range(B):
        for i in range(W):
            logits[b, i, tgt[b, i]] = 2.0
            logits[b, i, tgt[b, i] + 1:][::7] = 2.0  # later ids tie with it
    draft = torch.tensor([[-1, 5, 299, 0], [-1, 64, 7, 192], [-1, 1, 2, 3]], dtype=torch.int32)
    kinds = torch.zeros(B, dtype=torch.uint8)
    ids = torch.tensor(np.tile(np.arange(-1, W - 1), (B, 1)), dtype=torch.int32)
    ref = O.accept(logits.numpy(), draft.numpy(), kinds.numpy(), ids.numpy())
    got = lib.accept(logits.cuda(), draft.cuda(), kinds.cuda(), ids.cuda())
    assert_accept_equal(got, ref)
    assert list(ints(got[0])) == [3, 1, 3]


STEP_TARGETS = [
    # the partial launch finds the row targets (V <= 1024, V % 4 == 0) ...
    W_("targets_v1000", B=2, Hq=32, Hkv=8, W=32, ctx_lo=300, ctx_hi=900, masks="tree"),
    W_("targets_v4", B=1, Hq=20, Hkv=5, W=8, ctx_lo=500, ctx_hi=500, vocab=4),
    # ... or the acceptance reduces the rows itself
    W_("targets_v1001", B=1, Hq=20, Hkv=5, W=8, ctx_lo=500, ctx_hi=500, vocab=1001),
    W_("targets_v3000", B=2, Hq=16, Hkv=4, W=16, ctx_lo=200, ctx_hi=600, masks="mixed",
       vocab=3000),
]


@pytest.mark.parametrize("wl", STEP_TARGETS, ids=[w.name for w in STEP_TARGETS])
@pytest.mark.parametrize("ties", [False, True])
def test_step_targets_match_oracle(wl, ties):
    """Acceptance through the whole step, on both routes of the row targets;
    with ties, every logits row repeats its maximum at later ids, so the
    smallest id must win on either route."""
    inp = gpu_inputs(wl, 25)
    if ties:
        lg = inp["logits"]
        mx = lg.max(dim=2, keepdim=True).values
        am = lg.argmax(dim=2, keepdim=True)
        ids = torch.arange(lg.shape[2], device=lg.device).view(1, 1, -1)
        lg[:] = torch.where(((ids - am) % 3 == 0) & (ids > am), mx.expand_as(lg), lg)
    n_ref, path_ref, bonus_ref = oracle_accept(inp)
    kc_ref, vc_ref, ctx_ref = O.kv_commit(raw(inp["k_cache"]), raw(inp["v_cache"]),
                                          raw(inp["k_new"]), raw(inp["v_new"]), n_ref, path_ref,
                                          ints(inp["block_table"]), ints(inp["ctx_lens"]))
    out, lse, n, path, bonus, ctx_out = lib.verify_step(
        inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["ctx_lens"],
        inp["k_new"], inp["v_new"], inp["mask_kind"], inp["mask_ids"], inp["logits"],
        inp["draft_ids"], ctx_lens_out=torch.full_like(inp["ctx_lens"], -3),
        max_ctx_len=int(inp["host"]["ctx_lens"].max()), scale=inp["scale"])
    torch.cuda.synchronize()
    assert_accept_equal((n, path, bonus), (n_ref, path_ref, bonus_ref))
    assert np.array_equal(ints(ctx_out), ctx_ref)
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)


def tie_block(tgt: np.ndarray, V: int):
    """Four tree blocks of width 8 whose siblings share drafted ids, so that
    several equally deep nodes are accepted.  Returns (parents, drafts,
    expected paths).  A draft that must not match takes its parent's target
    + 1 (mod V)."""
    par = np.array([[-1, 0, 0, 1, 2, 1, 2, 3],
                    [-1, 0, 0, 1, 2, 1, 2, 3],
                    [-1, 0, 0, 1, 2, 1, 2, 3],
                    [-1, 0, 0, 2, 1, 4, 3, 6]], dtype=np.int32)
    # per block: the nodes whose draft equals their parent's target
    match = [{1, 2, 3, 4},        # depth-2 nodes 3 and 4 tie: node 3
             {1, 2, 4, 6},        # depth-2 nodes 4 and 6 tie: node 4
             {1, 2, 3, 4, 7},     # node 7 is deeper: depth 3 beats the tie
             {1, 2, 3, 4, 6}]     # 3 (under 2) and 4 (under 1) tie at depth 2,
    #                               6 under 3 is deeper: node 6
    paths = [[0, 1, 3], [0, 2, 4], [0, 1, 3, 7], [0, 2, 3, 6]]
    draft = np.full(par.shape, -1, dtype=np.int32)
    for b in range(par.shape[0]):
        for i in range(1, par.shape[1]):
            want = int(tgt[b, par[b, i]])
            draft[b, i] = want if i in match[b] else (want + 1) % V
    return par, draft, paths


def test_accept_equal_depth_ties_take_the_smallest_node():
    """Siblings sharing a drafted id both match; of equally deep accepted
    nodes the one with the smallest index wins (acceptance alone, and inside
    the step's finish launch with its commit)."""
    wl = W_("acc_ties", B=4, Hq=8, Hkv=2, W=8, ctx_lo=20, ctx_hi=60, masks="tree")
    inp = gpu_inputs(wl, 31)
    par, draft, paths = tie_block(inp["host"]["target_ids"], wl.vocab)
    inp["mask_ids"] = torch.from_numpy(par).cuda()
    inp["draft_ids"] = torch.from_numpy(draft).cuda()
    ref = oracle_accept(inp)
    for b, p in enumerate(paths):
        assert list(ref[1][b][:len(p)]) == p and ref[0][b] == len(p) - 1
    assert_accept_equal(lib.accept(inp["logits"], inp["draft_ids"], inp["mask_kind"],
                                   inp["mask_ids"]), ref)
    ref_out, ref_lse = oracle_attn(inp)
    kc_ref, vc_ref, ctx_ref = O.kv_commit(raw(inp["k_cache"]), raw(inp["v_cache"]),
                                          raw(inp["k_new"]), raw(inp["v_new"]), ref[0], ref[1],
                                          ints(inp["block_table"]), ints(inp["ctx_lens"]))
    out, lse, n, path, bonus, ctx_out = lib.verify_step(
        inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["ctx_lens"],
        inp["k_new"], inp["v_new"], inp["mask_kind"], inp["mask_ids"], inp["logits"],
        inp["draft_ids"], max_ctx_len=int(inp["host"]["ctx_lens"].max()), scale=inp["scale"])
    torch.cuda.synchronize()
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what="ties")
    assert_accept_equal((n, path, bonus), ref)
    assert np.array_equal(ints(ctx_out), ctx_ref)
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)


# ----------------------------------------------------------------------------
# confidence-threshold / hybrid acceptance
# ----------------------------------------------------------------------------

HYBRID = [
    W_("hyb_chain", B=16, W=8, ctx_lo=1, ctx_hi=1, conf_p=0.85),
    W_("hyb_tree", B=16, W=32, ctx_lo=1, ctx_hi=1, masks="tree", conf_p=0.9),
    W_("hyb_tree_w64", B=8, W=64, ctx_lo=1, ctx_hi=1, masks="tree", tree_depth=63,
       match_p=0.9, conf_p=0.97),
    W_("hyb_mixed_v7", B=16, W=16, ctx_lo=1, ctx_hi=1, masks="mixed", vocab=7),
    W_("hyb_mask_tokens", B=8, W=12, ctx_lo=1, ctx_hi=1, conf_p=1.0, mask_token_rows=5),
    W_("hyb_w1", B=4, W=1, ctx_lo=1, ctx_hi=1),
    W_("hyb_vocab_odd", B=6, W=9, ctx_lo=1, ctx_hi=1, masks="segment", vocab=1001),
    W_("hyb_vocab_big", B=2, W=8, ctx_lo=1, ctx_hi=1, vocab=50000),
]


def oracle_hybrid(inp, tau, m, with_logits=True):
    host = inp["host"]
    return O.accept_hybrid(f64(inp["draft_logits"]), f64(inp["logits"]) if with_logits else None,
                           host["draft_ids"], host["mask_kind"], host["mask_ids"], tau, m)


def assert_hybrid_equal(got, ref, tau, conf):
    live = conf[:, 1:]
    assert np.all(np.abs(live - tau) > 1e-4), "a confidence lies on the threshold"
    assert_accept_equal(got[:3], ref[:3])
    assert np.array_equal(ints(got[3]), ref[3]), f"conf_len {ints(got[3])} != {ref[3]}"


@pytest.mark.parametrize("with_logits", [True, False])
@pytest.mark.parametrize("tau,m", [(0.9, 1), (0.9, 3), (0.5, 2), (0.97, 1), (1.5, 1), (0.0, 4)])
@pytest.mark.parametrize("wl", HYBRID, ids=[w.name for w in HYBRID])
def test_hybrid_accept_bit_exact(wl, tau, m, with_logits):
    inp = gpu_inputs(wl.scaled(D=64, Hq=2, Hkv=2), 13)
    got = lib.accept_hybrid(inp["draft_logits"], inp["logits"] if with_logits else None,
                            inp["draft_ids"], inp["mask_kind"], inp["mask_ids"], tau, m)
    torch.cuda.synchronize()
    conf = O.draft_confidence(f64(inp["draft_logits"]), inp["host"]["draft_ids"])
    conf[inp["host"]["draft_ids"] < 0] = 2.0  # mask tokens decide nothing near tau
    assert_hybrid_equal(got, oracle_hybrid(inp, tau, m, with_logits), tau, conf)


def test_hybrid_confident_outputs_feed_the_commit():
    """A confidence-branch acceptance commits through mtp_kv_commit like a
    verified one: the h drafts' rows (root first) land in the cache."""
    wl = W_("hyb_commit", B=6, Hq=4, Hkv=2, W=12, ctx_lo=3, ctx_hi=90, masks="mixed",
            conf_p=0.95)
    inp = gpu_inputs(wl, 17)
    n, path, bonus, h = lib.accept_hybrid(inp["draft_logits"], None, inp["draft_ids"],
                                          inp["mask_kind"], inp["mask_ids"], 0.9, 1)
    ref = oracle_hybrid(inp, 0.9, 1, with_logits=False)
    assert np.array_equal(ints(n), ref[0]) and np.array_equal(ints(path), ref[1])
    keep = ints(n) >= 0
    n = torch.where(n >= 0, n, torch.zeros_like(n))  # unconfident sequences: the root only
    path = path.clone()
    path[:, 0] = 0
    kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()
    ctx_out = lib.kv_commit(inp["k_new"], inp["v_new"], n, path, inp["block_table"],
                            inp["ctx_lens"], kc, vc)
    torch.cuda.synchronize()
    host = inp["host"]
    rk, rv, rctx = O.kv_commit(raw(inp["k_cache"]), raw(inp["v_cache"]), raw(inp["k_new"]),
                               raw(inp["v_new"]), ints(n), ints(path), host["block_table"],
                               host["ctx_lens"], False)
    assert np.array_equal(ints(ctx_out), rctx)
    assert np.array_equal(raw(kc), rk) and np.array_equal(raw(vc), rv)
    assert keep.any() and (ints(n)[keep] >= 1).any()


# ----------------------------------------------------------------------------
# commit
# ----------------------------------------------------------------------------

COMMIT = [
    W_("com_mixed", B=6, Hq=8, Hkv=2, W=16, ctx_lo=0, ctx_hi=200, masks="mixed"),
    W_("com_full_accept", B=4, Hq=4, Hkv=4, D=64, W=20, ctx_lo=5, ctx_hi=40, match_p=1.0),
    W_("com_fp32", B=3, Hq=4, Hkv=2, W=9, dtype="f32", ctx_lo=14, ctx_hi=18, masks="tree"),
]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("skip_root", [False, True])
@pytest.mark.parametrize("wl", COMMIT, ids=[w.name for w in COMMIT])
def test_commit_bit_exact(wl, skip_root, fused):
    inp = gpu_inputs(wl, 5)
    n_ref, path_ref, bonus_ref = oracle_accept(inp)
    kc0, vc0 = raw(inp["k_cache"]), raw(inp["v_cache"])
    kc_ref, vc_ref, ctx_ref = O.kv_commit(kc0, vc0, raw(inp["k_new"]), raw(inp["v_new"]), n_ref,
                                          path_ref, ints(inp["block_table"]),
                                          ints(inp["ctx_lens"]), skip_root)
    ctx_out = torch.full_like(inp["ctx_lens"], -7)
    if fused:
        n, path, bonus, ctx_out = lib.accept_commit(
            inp["logits"], inp["draft_ids"], inp["mask_kind"], inp["mask_ids"], inp["k_new"],
            inp["v_new"], inp["block_table"], inp["ctx_lens"], inp["k_cache"], inp["v_cache"],
            ctx_lens_out=ctx_out, skip_root=skip_root)
        assert_accept_equal((n, path, bonus), (n_ref, path_ref, bonus_ref))
    else:
        n = torch.from_numpy(n_ref.astype(np.int32)).cuda()
        path = torch.from_numpy(path_ref.astype(np.int32)).cuda()
        lib.kv_commit(inp["k_new"], inp["v_new"], n, path, inp["block_table"], inp["ctx_lens"],
                      inp["k_cache"], inp["v_cache"], ctx_lens_out=ctx_out, skip_root=skip_root)
    torch.cuda.synchronize()
    assert np.array_equal(ints(ctx_out), ctx_ref)
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)


def test_commit_in_place_context_update_and_idempotence():
    wl = W_("com_inplace", B=5, Hq=8, Hkv=2, W=8, ctx_lo=3, ctx_hi=100, masks="mixed")
    inp = gpu_inputs(wl, 9)
    n_ref, path_ref, _ = oracle_accept(inp)
    ctx0 = inp["ctx_lens"].clone()
    kc_ref, vc_ref, ctx_ref = O.kv_commit(raw(inp["k_cache"]), raw(inp["v_cache"]),
                                          raw(inp["k_new"]), raw(inp["v_new"]), n_ref, path_ref,
                                          ints(inp["block_table"]), ints(ctx0))
    # the same commit twice from the same boundary, then once in place
    for _ in range(2):
        out = lib.accept_commit(inp["logits"], inp["draft_ids"], inp["mask_kind"],
                                inp["mask_ids"], inp["k_new"], inp["v_new"], inp["block_table"],
                                ctx0, inp["k_cache"], inp["v_cache"])[3]
    ctx = ctx0.clone()
    lib.accept_commit(inp["logits"], inp["draft_ids"], inp["mask_kind"], inp["mask_ids"],
                      inp["k_new"], inp["v_new"], inp["block_table"], ctx, inp["k_cache"],
                      inp["v_cache"], ctx_lens_out=ctx)
    torch.cuda.synchronize()
    assert np.array_equal(ints(out), ctx_ref) and np.array_equal(ints(ctx), ctx_ref)
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)


def test_commit_then_attend_equals_verify_rows():
    """After committing an accepted chain, decoding accepted row i as a
    one-row block at context L+i reproduces row i of the verify output."""
    wl = W_("com_decode", B=2, Hq=8, Hkv=2, W=6, ctx_lo=20, ctx_hi=60, match_p=1.0)
    inp = gpu_inputs(wl, 12)
    out, _ = run_attn(inp)
    lib.accept_commit(inp["logits"], inp["draft_ids"], inp["mask_kind"], inp["mask_ids"],
                      inp["k_new"], inp["v_new"], inp["block_table"], inp["ctx_lens"],
                      inp["k_cache"], inp["v_cache"])
    for i in range(wl.W):
        ctx_i = inp["ctx_lens"] + i
        o1, _ = lib.verify_attn(inp["q"][:, i:i + 1].contiguous(), inp["k_cache"], inp["v_cache"],
                                inp["block_table"], ctx_i, inp["k_new"][:, i:i + 1].contiguous(),
                                inp["v_new"][:, i:i + 1].contiguous(),
                                torch.zeros_like(inp["mask_kind"]),
                                torch.full((wl.B, 1), -1, dtype=torch.int32, device="cuda"),
                                max_ctx_len=int(ints(ctx_i).max()), scale=inp["scale"])
        torch.cuda.synchronize()
        np.testing.assert_allclose(o1[:, 0].cpu().numpy(), out[:, i].cpu().numpy(),
                                   atol=2e-3, rtol=2e-2)


# ----------------------------------------------------------------------------
# data errors: poisoned outputs and the sticky status word, never a fault
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("B", [3, 9], ids=["split", "stream"])
def test_malformed_mask_poisons_only_that_sequence(B):
    wl = W_("bad_mask", B=B, Hq=8, Hkv=2, W=8, ctx_lo=30, ctx_hi=90, masks="tree")
    inp = gpu_inputs(wl, 2)
    lib.device_status(clear=True)
    ids = inp["mask_ids"].clone()
    ids[1, 5] = 6  # a parent after its child
    inp["mask_ids"] = ids
    out, lse = run_attn(inp)
    assert torch.isnan(out[1]).all() and torch.isnan(lse[1]).all()
    ref_out, ref_lse = oracle_attn(inp)
    rest = [b for b in range(B) if b != 1]
    keep = torch.tensor(rest, device=out.device)
    assert_attn_close(out[keep], lse[keep], ref_out[rest], ref_lse[rest], *tol_for(wl))
    n, path, bonus = lib.accept(inp["logits"], inp["draft_ids"], inp["mask_kind"], ids)
    assert_accept_equal((n, path, bonus), oracle_accept(inp))
    assert lib.device_status(clear=True) & lib.DEV_BAD_MASK


def test_context_above_bound_poisons_that_sequence():
    wl = W_("bad_ctx", B=2, Hq=8, Hkv=2, W=4, ctx_lo=40, ctx_hi=40)
    inp = gpu_inputs(wl, 2)
    lib.device_status(clear=True)
    out, lse = run_attn(inp, max_ctx_len=39)
    assert torch.isnan(out).all() and torch.isnan(lse).all()
    assert lib.device_status(clear=True) & lib.DEV_BAD_CTX


def test_stream_context_above_bound_poisons_only_that_sequence():
    """Stream schedule: sequences past max_ctx_len get no stages and NaN rows;
    the others are unaffected."""
    wl = W_("bad_ctx_stream", B=9, Hq=8, Hkv=2, W=8, ctx_lo=20, ctx_hi=300, masks="mixed")
    inp = gpu_inputs(wl, 3)
    ctx = [int(x) for x in inp["host"]["ctx_lens"]]
    bound = max(ctx) - 1
    lib.device_status(clear=True)
    out, lse = run_attn(inp, max_ctx_len=bound)
    bad = [b for b in range(wl.B) if ctx[b] > bound]
    rest = [b for b in range(wl.B) if ctx[b] <= bound]
    assert bad and rest
    assert torch.isnan(out[bad]).all() and torch.isnan(lse[bad]).all()
    ref_out, ref_lse = oracle_attn(inp)
    keep = torch.tensor(rest, device=out.device)
    assert_attn_close(out[keep], lse[keep], ref_out[rest], ref_lse[rest], *tol_for(wl))
    assert lib.device_status(clear=True) & lib.DEV_BAD_CTX


def test_unmapped_committed_page_poisons_the_rows_that_read_it():
    wl = W_("bad_page", B=2, Hq=8, Hkv=2, W=4, ctx_lo=100, ctx_hi=100)
    inp = gpu_inputs(wl, 2)
    lib.device_status(clear=True)
    bt = inp["block_table"].clone()
    bt[0, 2] = inp["k_cache"].shape[0] + 5
    inp["block_table"] = bt
    out, lse = run_attn(inp)
    assert torch.isnan(out[0]).all()
    assert torch.isfinite(out[1]).all()
    assert lib.device_status(clear=True) & lib.DEV_BAD_PAGE


def test_commit_with_unmapped_target_slot_writes_nothing():
    wl = W_("bad_commit", B=3, Hq=4, Hkv=2, W=8, ctx_lo=30, ctx_hi=30, match_p=1.0)
    inp = gpu_inputs(wl, 2)
    lib.device_status(clear=True)
    bt = inp["block_table"].clone()
    bt[1, (30 + 7) // 16] = -1
    kc0, vc0 = raw(inp["k_cache"]), raw(inp["v_cache"])
    n_ref, path_ref, _ = oracle_accept(inp)
    kc_ref, vc_ref, ctx_ref = O.kv_commit(kc0, vc0, raw(inp["k_new"]), raw(inp["v_new"]), n_ref,
                                          path_ref, ints(bt), ints(inp["ctx_lens"]))
    _, _, _, ctx = lib.accept_commit(inp["logits"], inp["draft_ids"], inp["mask_kind"],
                                     inp["mask_ids"], inp["k_new"], inp["v_new"], bt,
                                     inp["ctx_lens"], inp["k_cache"], inp["v_cache"])
    torch.cuda.synchronize()
    assert np.array_equal(ints(ctx), ctx_ref) and ctx_ref[1] == 30
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)
    assert lib.device_status(clear=True) & lib.DEV_BAD_PAGE


def test_empty_batch_is_a_no_op():
    wl = W_("empty", B=1, Hq=4, Hkv=2, W=4, ctx_lo=10, ctx_hi=10)
    inp = gpu_inputs(wl, 1)
    e = lambda t: t[:0]
    out, lse = lib.verify_attn(e(inp["q"]), inp["k_cache"], inp["v_cache"], e(inp["block_table"]),
                               e(inp["ctx_lens"]), e(inp["k_new"]), e(inp["v_new"]),
                               e(inp["mask_kind"]), e(inp["mask_ids"]), max_ctx_len=10)
    torch.cuda.synchronize()
    assert out.numel() == 0


# ----------------------------------------------------------------------------
# the whole step in two launches
# ----------------------------------------------------------------------------

STEP = [
    W_("step_mixed_b9", B=9, Hq=32, Hkv=8, W=16, ctx_lo=0, ctx_hi=700, masks="mixed"),
    W_("step_stream_straddle", B=9, Hq=3, Hkv=1, W=11, ctx_lo=10, ctx_hi=400, masks="mixed"),
    # 256 ranges per KV head over 8 sequences: the finish launch's combine
    # takes one row per wave
    W_("step_stream_pieces", B=8, Hq=32, Hkv=2, W=4, ctx_lo=1500, ctx_hi=3000, masks="mixed"),
    # one long sequence on the stream kernel
    W_("step_stream_b1", B=1, Hq=32, Hkv=8, W=16, ctx_lo=9000, ctx_hi=9000, masks="tree"),
    W_("step_grouped_b4", B=4, Hq=64, Hkv=8, W=16, ctx_lo=50, ctx_hi=600, masks="mixed"),
    W_("step_chain_b1", B=1, Hq=20, Hkv=5, W=8, ctx_lo=600, ctx_hi=600),
    # one sequence of 4000 tokens on the per-split kernel with key slices
    # (32 splits of 128 tokens); 38 and 47 splits of 32 tokens on the D = 64
    # and fp32 kernels (the finish launch's combine takes a second batch)
    W_("step_chain_b1_long", B=1, Hq=20, Hkv=5, W=8, ctx_lo=4000, ctx_hi=4000),
    W_("step_segment_d64_38_splits", B=1, Hq=16, Hkv=16, D=64, W=16, ctx_lo=1200, ctx_hi=1200,
       masks="segment", seg_lookback=1),
    W_("step_fp32_47_splits", B=1, Hq=4, Hkv=4, W=4, dtype="f32", ctx_lo=1500, ctx_hi=1500),
    W_("step_segment_d64", B=3, Hq=16, Hkv=16, D=64, W=16, ctx_lo=30, ctx_hi=300,
       masks="segment", seg_lookback=1),
    W_("step_fp32", B=2, Hq=4, Hkv=4, D=64, W=4, dtype="f32", ctx_lo=100, ctx_hi=256),
    # more sequences than half the compute units: the finish launch keeps one
    # combine workgroup per compute unit behind the acceptance workgroups
    W_("step_b300", B=300, Hq=8, Hkv=2, W=16, ctx_lo=0, ctx_hi=64, masks="mixed",
       spare_pages=8),
]


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("wl", STEP, ids=[w.name for w in STEP])
def test_verify_step_matches_attention_then_accept_commit(wl, in_place):
    inp = gpu_inputs(wl, 21)
    ref_out, ref_lse = oracle_attn(inp)
    n_ref, path_ref, bonus_ref = oracle_accept(inp)
    kc_ref, vc_ref, ctx_ref = O.kv_commit(raw(inp["k_cache"]), raw(inp["v_cache"]),
                                          raw(inp["k_new"]), raw(inp["v_new"]), n_ref, path_ref,
                                          ints(inp["block_table"]), ints(inp["ctx_lens"]))
    ctx = inp["ctx_lens"].clone()
    ctx_out = ctx if in_place else torch.full_like(ctx, -3)
    out, lse, n, path, bonus, ctx_out = lib.verify_step(
        inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], ctx, inp["k_new"],
        inp["v_new"], inp["mask_kind"], inp["mask_ids"], inp["logits"], inp["draft_ids"],
        ctx_lens_out=ctx_out, max_ctx_len=int(inp["host"]["ctx_lens"].max()), scale=inp["scale"],
        seg_lookback=inp["seg_lookback"])
    torch.cuda.synchronize()
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=wl.name)
    assert_accept_equal((n, path, bonus), (n_ref, path_ref, bonus_ref))
    assert np.array_equal(ints(ctx_out), ctx_ref)
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)
