"""GPU parity of the nested KV4 / KV8 cache: quantization and the quantizing
commit bit-exact against the oracle (codes and scales), verify attention over
the planes within the bf16 tolerance of the oracle's attention over the
dequantized cache (KV8, KV4 and Recent-N reads).

The GPU path quantizes the bf16 pool with its own kernel; the oracle
quantizes the same bf16 values with its own code."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_common import (ATOL, RTOL, I, O, lib, assert_attn_close, banner, f64, gpu_inputs,
                              ints, oracle_accept)

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore::RuntimeWarning"),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def W_(name, **kw) -> I.Workload:
    base = dict(name=name, B=2, Hq=8, Hkv=2, D=128, W=8, dtype="bf16", ctx_lo=100, ctx_hi=700,
                masks="chain")
    base.update(kw)
    return I.Workload(**base)


def finite_slots(cache) -> np.ndarray:
    """[pages, 16] bool: slots whose K row holds no NaN (written rows)."""
    c = cache.float().cpu().numpy()
    return np.isfinite(c).all(axis=(2, 3))


def quantized(inp):
    pages, _, Hkv, D = inp["k_cache"].shape
    kv = lib.NestedKV(pages, Hkv, D)
    lib.kv_quantize_cache(inp["k_cache"], inp["v_cache"], kv)
    torch.cuda.synchronize()
    return kv


def oracle_planes(inp):
    return (O.nested_planes(inp["k_cache"].float().cpu().numpy()),
            O.nested_planes(inp["v_cache"].float().cpu().numpy()))


def assert_planes_equal(got: dict, ref: dict, where: np.ndarray, what: str):
    """Planes equal at the [pages, 16] slots selected by `where`."""
    for key in ("base", "ref", "scale"):
        g = np.swapaxes(got[key], 1, 2)[where]
        r = np.swapaxes(ref[key], 1, 2)[where]
        if key == "scale":
            g, r = g.view(np.int32), r.astype(np.float32).view(np.int32)
        assert np.array_equal(g, r), f"{what} {key} plane differs"


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_quantize_bit_exact(dtype, D):
    banner(f"quantize dtype={dtype} D={D}")
    n, Hkv, pages = 300, 3, 40
    g = torch.Generator().manual_seed(3)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rows = (torch.randn((n, Hkv, D), generator=g) *
            torch.tensor([1e-3, 1.0, 40.0])[torch.randint(0, 3, (n, 1, 1), generator=g)])
    rows[0].zero_()  # s = 0
    rows[1, 0] = torch.tensor([7.0, -3.5, 2.96875, -0.5] * (D // 4))  # ties of both roundings
    rows = rows.to(tdt)
    vrows = torch.randn((n, Hkv, D), generator=g).to(tdt)
    slots = torch.randperm(pages * 16, generator=g)[:n].to(torch.int32)
    kv = lib.NestedKV(pages, Hkv, D)
    lib.kv_quantize(rows.cuda(), vrows.cuda(), slots.cuda(), kv)
    torch.cuda.synchronize()
    assert lib.device_status(clear=True) == 0
    for which, src in (("k", rows), ("v", vrows)):
        q4, qr, sc = O.quantize_nested(src.float().numpy())
        got = kv.planes(which)
        pg, sl = (slots // 16).numpy(), (slots % 16).numpy()
        assert np.array_equal(got["base"][pg, :, sl], O.pack_nibbles(q4)), f"{which} base"
        assert np.array_equal(got["ref"][pg, :, sl], O.pack_nibbles(qr)), f"{which} ref"
        assert np.array_equal(got["scale"][pg, :, sl].view(np.int32), sc.view(np.int32)), \
            f"{which} scale"


def test_quantize_rejects_slots_outside_the_pool():
    wl = W_("quant_bad", B=1, Hq=2, Hkv=2, D=128, ctx_lo=20, ctx_hi=20)
    inp = gpu_inputs(wl, 4)
    pages = inp["k_cache"].shape[0]
    kv = lib.NestedKV(pages, 2, 128)
    rows = inp["k_new"][0, :3].contiguous()
    slots = torch.tensor([5, pages * 16, -1], dtype=torch.int32, device="cuda")
    lib.kv_quantize(rows, rows, slots, kv)
    torch.cuda.synchronize()
    assert lib.device_status(clear=True) & lib.DEV_BAD_PAGE
    assert kv.k_scale.view(-1)[5].item() > 0


NESTED = [
    W_("n_chain_g4", Hq=20, Hkv=5, W=8, ctx_lo=300, ctx_hi=700),
    W_("n_tree_w32", Hq=32, Hkv=8, W=32, ctx_lo=200, ctx_hi=600, masks="tree"),
    W_("n_mixed_b5", B=5, Hq=32, Hkv=8, W=16, ctx_lo=0, ctx_hi=900, masks="mixed"),
    W_("n_r4_padded", B=3, Hq=4, Hkv=4, W=4, ctx_lo=1, ctx_hi=333, masks="tree"),
    W_("n_r48", B=2, Hq=12, Hkv=2, W=8, ctx_lo=33, ctx_hi=517, masks="mixed"),
    W_("n_w64", Hq=4, Hkv=2, W=64, ctx_lo=90, ctx_hi=400, masks="tree", tree_depth=63),
    # 192 rows per KV head: three row blocks, XCD-paired groups and a tail
    W_("n_row_blocks3", B=3, Hq=36, Hkv=3, W=16, ctx_lo=100, ctx_hi=1500, masks="mixed"),
    W_("n_segment", Hq=16, Hkv=4, W=16, ctx_lo=15, ctx_hi=260, masks="segment", seg_lookback=1),
    W_("n_ctx_edges", B=4, Hq=8, Hkv=1, W=4, ctx_lo=15, ctx_hi=17),
]


def oracle_nested(inp, kp, vp, recent):
    return O.verify_attention_nested(f64(inp["q"]), kp, vp, ints(inp["block_table"]),
                                     ints(inp["ctx_lens"]), f64(inp["k_new"]), f64(inp["v_new"]),
                                     ints(inp["mask_kind"]), ints(inp["mask_ids"]), inp["scale"],
                                     inp["seg_lookback"], recent)


@pytest.mark.parametrize("recent", [-1, 0, 37])
@pytest.mark.parametrize("wl", NESTED, ids=[w.name for w in NESTED])
def test_nested_attention_matches_oracle(wl, recent):
    inp = gpu_inputs(wl, 9)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    mc = max(int(inp["host"]["ctx_lens"].max()), 0)
    out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], kv8_recent=recent, max_ctx_len=mc,
                                      scale=inp["scale"], seg_lookback=inp["seg_lookback"])
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_nested(inp, kp, vp, recent)
    assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, f"{wl.name} recent={recent}")
    assert lib.device_status(clear=True) == 0


# Eight or more sequences: the nested stream-K kernel (ranges of the list of
# 32-key stages of every segment; pieces per range and segment).
NESTED_STREAM = [
    W_("ns_mixed", B=9, Hq=32, Hkv=8, W=16, ctx_lo=0, ctx_hi=900, masks="mixed"),
    # 128 rows per KV head: two row blocks of 64 (two segments per sequence and head)
    W_("ns_rows128", B=8, Hq=32, Hkv=8, W=32, ctx_lo=40, ctx_hi=700, masks="tree"),
    W_("ns_hkv5", B=9, Hq=20, Hkv=5, W=8, ctx_lo=0, ctx_hi=1100, masks="chain"),
    W_("ns_r16", B=10, Hq=8, Hkv=4, W=8, ctx_lo=15, ctx_hi=300, masks="mixed"),
    # 33 rows per sequence and head (a padded tile), segments with lookback 1
    W_("ns_r33", B=8, Hq=3, Hkv=1, W=11, ctx_lo=0, ctx_hi=500, masks="segment", seg_lookback=1),
    # fewer sequences whose ranges hold four or more stages
    W_("ns_b1", B=1, Hq=32, Hkv=8, W=16, ctx_lo=9000, ctx_hi=9000, masks="chain"),
    W_("ns_b2", B=2, Hq=32, Hkv=8, W=16, ctx_lo=5000, ctx_hi=8000, masks="mixed"),
]


@pytest.mark.parametrize("recent", [-1, 0, 37])
@pytest.mark.parametrize("wl", NESTED_STREAM, ids=[w.name for w in NESTED_STREAM])
def test_nested_stream_attention_matches_oracle(wl, recent):
    inp = gpu_inputs(wl, 14)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], kv8_recent=recent,
                                      max_ctx_len=int(inp["host"]["ctx_lens"].max()),
                                      scale=inp["scale"], seg_lookback=inp["seg_lookback"])
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_nested(inp, kp, vp, recent)
    assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, f"{wl.name} recent={recent}")
    assert lib.device_status(clear=True) == 0


# Magnitudes far from N(0, 1): the stream kernel scales Q by a power of two
# per row and P by 2^60 so that its products with the code bytes (operand bit
# patterns 0x00uu = u 2^-133) stay in the normal fp32 range.  Attention is
# linear in V and the softmax sees only q.k, so each case compares out / v
# scale with the standard tolerance.  Two workloads: the stream kernel (nine
# sequences) and the per-split kernel (two).
EXTREME = [(1e-30, 1.0, 1.0), (1e30, 1.0, 1.0), (1.0, 1e-20, 1.0), (1.0, 1e12, 1.0),
           (1.0, 1.0, 1e-12), (1.0, 1.0, 1e16)]


@pytest.mark.parametrize("qs,ks,vs", EXTREME, ids=[f"q{a:g}_k{b:g}_v{c:g}" for a, b, c in EXTREME])
@pytest.mark.parametrize("B", [9, 2])
def test_nested_extreme_magnitudes(B, qs, ks, vs):
    wl = W_("n_extreme", B=B, Hq=16, Hkv=4, W=8, ctx_lo=20, ctx_hi=900, masks="mixed")
    inp = gpu_inputs(wl, 31)
    inp["q"].mul_(qs)
    for key, f in (("k_cache", ks), ("k_new", ks), ("v_cache", vs), ("v_new", vs)):
        inp[key].mul_(f)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    for recent in (-1, 0):
        out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                          inp["k_new"], inp["v_new"], inp["mask_kind"],
                                          inp["mask_ids"], kv8_recent=recent,
                                          max_ctx_len=int(inp["host"]["ctx_lens"].max()),
                                          scale=inp["scale"], seg_lookback=inp["seg_lookback"])
        torch.cuda.synchronize()
        assert lib.device_status(clear=True) == 0
        ref_out, ref_lse = oracle_nested(inp, kp, vp, recent)
        assert np.isfinite(out.cpu().numpy()).all(), f"B={B} q{qs} k{ks} v{vs}: non-finite output"
        assert_attn_close(out / vs, lse, ref_out / vs, ref_lse, ATOL, RTOL,
                          f"B={B} q{qs} k{ks} v{vs} recent={recent}")


@pytest.mark.parametrize("B", [1024, 1100])
def test_nested_batch_at_and_above_the_stream_table(B):
    """1024 sequences fill the nested stream kernel's stage table exactly;
    more run the per-split nested kernel."""
    wl = W_(f"n_b{B}", B=B, Hq=4, Hkv=1, W=4, ctx_lo=0, ctx_hi=40, masks="mixed", spare_pages=8)
    inp = gpu_inputs(wl, 16)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    for recent in (-1, 0):
        out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                          inp["k_new"], inp["v_new"], inp["mask_kind"],
                                          inp["mask_ids"], kv8_recent=recent,
                                          max_ctx_len=int(inp["host"]["ctx_lens"].max()),
                                          scale=inp["scale"], seg_lookback=inp["seg_lookback"])
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle_nested(inp, kp, vp, recent)
        assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, f"B={B} recent={recent}")
        assert lib.device_status(clear=True) == 0


@pytest.mark.parametrize("split", [32, 96, 1024])
def test_nested_stream_work_split_does_not_change_the_result(split):
    """Workgroups of 1, 3 or 32 stages: ranges start and end inside
    committed stages and inside the in-block stage."""
    wl = W_("ns_split", B=9, Hq=32, Hkv=8, W=16, ctx_lo=0, ctx_hi=1500, masks="mixed")
    inp = gpu_inputs(wl, 15)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], kv8_recent=600, scale=inp["scale"],
                                      split_tokens=split)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_nested(inp, kp, vp, 600)
    assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, f"stream split={split}")


@pytest.mark.parametrize("split", [32, 64, 2048])
def test_nested_split_size_does_not_change_the_result(split):
    wl = W_("n_split", B=3, Hq=16, Hkv=4, W=8, ctx_lo=500, ctx_hi=1300, masks="mixed")
    inp = gpu_inputs(wl, 12)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], scale=inp["scale"], split_tokens=split)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_nested(inp, kp, vp, -1)
    assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, f"split={split}")


def test_kv4_reads_need_no_refinement_planes():
    wl = W_("n_kv4", B=2, Hq=8, Hkv=2, W=8, ctx_lo=100, ctx_hi=300)
    inp = gpu_inputs(wl, 13)
    kv = quantized(inp)
    base_only = lib.NestedKV(kv.num_pages, kv.Hkv, kv.D, with_ref=False)
    for name in ("k_base", "v_base", "k_scale", "v_scale"):
        getattr(base_only, name).copy_(getattr(kv, name))
    kp, vp = oracle_planes(inp)
    out, lse = lib.verify_attn_nested(inp["q"], base_only, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], kv8_recent=0, scale=inp["scale"])
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_nested(inp, kp, vp, 0)
    assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, "kv4 base only")
    with pytest.raises(lib.MtpError):
        lib.verify_attn_nested(inp["q"], base_only, inp["block_table"], inp["ctx_lens"],
                               inp["k_new"], inp["v_new"], inp["mask_kind"], inp["mask_ids"],
                               kv8_recent=-1)


def test_nested_full_size_bitnet2b_chain():
    wl = I.WORKLOADS["bitnet2b_chain"]
    inp = gpu_inputs(wl, I.workload_seed("bitnet2b_chain"))
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    mc = int(inp["host"]["ctx_lens"].max())
    out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], max_ctx_len=mc, scale=inp["scale"])
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_nested(inp, kp, vp, -1)
    assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, "bitnet2b_chain nested")


@pytest.mark.parametrize("skip_root", [False, True])
def test_nested_commit_bit_exact(skip_root):
    wl = W_("n_commit", B=6, Hq=8, Hkv=2, W=16, ctx_lo=0, ctx_hi=200, masks="mixed")
    inp = gpu_inputs(wl, 21)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    n, path, _ = lib.accept(inp["logits"], inp["draft_ids"], inp["mask_kind"], inp["mask_ids"])
    ctx_out = lib.kv_commit_nested(inp["k_new"], inp["v_new"], n, path, inp["block_table"],
                                   inp["ctx_lens"], kv, skip_root=skip_root)
    torch.cuda.synchronize()
    rn, rpath, _ = oracle_accept(inp)
    assert np.array_equal(ints(n), rn)
    kp2, vp2, rctx = O.kv_commit_nested(kp, vp, inp["k_new"].float().cpu().numpy(),
                                        inp["v_new"].float().cpu().numpy(), rn, rpath,
                                        ints(inp["block_table"]), ints(inp["ctx_lens"]), skip_root)
    assert np.array_equal(ints(ctx_out), rctx)
    # every slot that holds a finite row before or after the commit
    where = finite_slots(inp["k_cache"]) & finite_slots(inp["v_cache"])
    for b in range(wl.B):
        for k in range(int(rn[b]) + 1):
            t = int(inp["host"]["ctx_lens"][b]) + k
            where[inp["host"]["block_table"][b, t // 16], t % 16] = True
    assert_planes_equal(kv.planes("k"), kp2, where, "K")
    assert_planes_equal(kv.planes("v"), vp2, where, "V")
    assert lib.device_status(clear=True) == 0


# ----------------------------------------------------------------------------
# data errors of the nested kernels: poisoned rows and the sticky status word
# ----------------------------------------------------------------------------

def nested_attn(inp, kv, recent=-1, max_ctx_len=None):
    out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], kv8_recent=recent,
                                      max_ctx_len=max_ctx_len, scale=inp["scale"])
    torch.cuda.synchronize()
    return out, lse


def assert_rest_close(inp, kp, vp, out, lse, rest, recent=-1):
    ref_out, ref_lse = oracle_nested(inp, kp, vp, recent)
    keep = torch.tensor(rest, device=out.device)
    assert_attn_close(out[keep], lse[keep], ref_out[rest], ref_lse[rest], ATOL, RTOL, "rest")


@pytest.mark.parametrize("B", [3, 9], ids=["split", "stream"])
def test_nested_malformed_mask_poisons_only_that_sequence(B):
    wl = W_("n_bad_mask", B=B, Hq=8, Hkv=2, W=8, ctx_lo=30, ctx_hi=300, masks="tree")
    inp = gpu_inputs(wl, 21)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    lib.device_status(clear=True)
    ids = inp["mask_ids"].clone()
    ids[1, 5] = 6  # a parent after its child
    inp["mask_ids"] = ids
    out, lse = nested_attn(inp, kv)
    assert torch.isnan(out[1]).all() and torch.isnan(lse[1]).all()
    assert_rest_close(inp, kp, vp, out, lse, [b for b in range(B) if b != 1])
    assert lib.device_status(clear=True) & lib.DEV_BAD_MASK


@pytest.mark.parametrize("B", [3, 9], ids=["split", "stream"])
def test_nested_unmapped_committed_page_poisons_that_sequence(B):
    wl = W_("n_bad_page", B=B, Hq=8, Hkv=2, W=8, ctx_lo=100, ctx_hi=400, masks="mixed")
    inp = gpu_inputs(wl, 22)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    lib.device_status(clear=True)
    good = dict(inp)  # the oracle reads the unchanged table (sequence 0 is not compared)
    bt = inp["block_table"].clone()
    bt[0, 2] = kv.num_pages + 5
    inp["block_table"] = bt
    out, lse = nested_attn(inp, kv)
    assert torch.isnan(out[0]).all()
    assert_rest_close(good, kp, vp, out, lse, list(range(1, B)))
    assert lib.device_status(clear=True) & lib.DEV_BAD_PAGE


def test_nested_stream_context_above_bound_poisons_only_that_sequence():
    wl = W_("n_bad_ctx", B=9, Hq=8, Hkv=2, W=8, ctx_lo=20, ctx_hi=300, masks="mixed")
    inp = gpu_inputs(wl, 23)
    kv = quantized(inp)
    kp, vp = oracle_planes(inp)
    ctx = [int(x) for x in inp["host"]["ctx_lens"]]
    bound = max(ctx) - 1
    lib.device_status(clear=True)
    out, lse = nested_attn(inp, kv, recent=0, max_ctx_len=bound)
    bad = [b for b in range(wl.B) if ctx[b] > bound]
    rest = [b for b in range(wl.B) if ctx[b] <= bound]
    assert bad and rest
    assert torch.isnan(out[bad]).all() and torch.isnan(lse[bad]).all()
    assert_rest_close(inp, kp, vp, out, lse, rest, recent=0)
    assert lib.device_status(clear=True) & lib.DEV_BAD_CTX
