"""GPU parity over seeded random shapes.

The launch plan chooses among the fp32/VALU kernel, the direct-load D = 64
MFMA kernel, the per-split LDS kernel (with key slices, weighted splits, row
blocks) and the stream-K kernel (with and without the small-batch routing)
from the shape alone.  These cases draw batch, width, head counts, head
dimension, dtype, mask kind and context lengths from one fixed seed, so they
reach plan routes and tile edges that no hand-picked case fixes.  Each case
runs the whole step (mtp_verify_step: attention, then acceptance and commit
in the finish launch) and compares every output with the oracle: attention
within the stated tolerance, acceptance, context lengths and the committed
cache bytes bit-exact.  A second set draws shapes for the nested KV4 / KV8
cache (bf16, D = 128) and its KV8, KV4 and Recent-N reads, a third for the
dynamic token tree builder (draft ids, parents, depths and node counts
bit-exact).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_common import (I, O, lib, assert_accept_equal, assert_attn_close, gpu_inputs,
                              ints, oracle_accept, oracle_attn, raw, tol_for)

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore::RuntimeWarning"),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def random_workloads(n: int, seed: int) -> list[I.Workload]:
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        D = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        Hkv = int(rng.choice([1, 2, 4, 5, 8]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        W = int(rng.choice([1, 2, 4, 5, 8, 11, 16, 23, 32, 40, 64]))
        B = int(rng.choice([1, 2, 3, 5, 8, 9, 13]))
        ctx_hi = int(rng.choice([0, 17, 300, 1000, 3000]))
        ctx_lo = int(rng.integers(0, ctx_hi + 1))
        masks = str(rng.choice(["chain", "tree", "segment", "mixed"])) if W > 1 else "chain"
        kw = dict(name=f"rand{k}", B=B, Hq=Hkv * g, Hkv=Hkv, D=D, W=W, dtype=dtype,
                  ctx_lo=ctx_lo, ctx_hi=ctx_hi, masks=masks,
                  tree_depth=int(min(8, W - 1)) if W > 1 else 1)
        if masks == "segment":
            kw["seg_lookback"] = int(rng.choice([-1, 0, 1, 2]))
        out.append(I.Workload(**kw))
    return out


RANDOM = random_workloads(64, 2026)


@pytest.mark.parametrize("wl", RANDOM, ids=[f"{w.name}-B{w.B}-W{w.W}-h{w.Hq}x{w.Hkv}-D{w.D}-{w.dtype}-"
                                            f"{w.masks}-ctx{w.ctx_lo}_{w.ctx_hi}" for w in RANDOM])
def test_random_shape_step_matches_oracle(wl):
    inp = gpu_inputs(wl, 77)
    ref_out, ref_lse = oracle_attn(inp)
    n_ref, path_ref, bonus_ref = oracle_accept(inp)
    kc_ref, vc_ref, ctx_ref = O.kv_commit(raw(inp["k_cache"]), raw(inp["v_cache"]),
                                          raw(inp["k_new"]), raw(inp["v_new"]), n_ref, path_ref,
                                          ints(inp["block_table"]), ints(inp["ctx_lens"]))
    ctx_out = torch.full_like(inp["ctx_lens"], -3)
    out, lse, n, path, bonus, ctx_out = lib.verify_step(
        inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["ctx_lens"],
        inp["k_new"], inp["v_new"], inp["mask_kind"], inp["mask_ids"], inp["logits"],
        inp["draft_ids"], ctx_lens_out=ctx_out,
        max_ctx_len=int(inp["host"]["ctx_lens"].max()), scale=inp["scale"],
        seg_lookback=inp["seg_lookback"])
    torch.cuda.synchronize()
    assert lib.device_status(clear=True) == 0
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=wl.name)
    assert_accept_equal((n, path, bonus), (n_ref, path_ref, bonus_ref))
    assert np.array_equal(ints(ctx_out), ctx_ref)
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)


def random_nested(n: int, seed: int) -> list[tuple[I.Workload, int]]:
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        Hkv = int(rng.choice([1, 2, 4, 5, 8]))
        g = int(rng.choice([1, 2, 4, 8]))
        W = int(rng.choice([1, 4, 8, 11, 16, 32, 64]))
        B = int(rng.choice([1, 2, 5, 8, 9, 12]))
        ctx_hi = int(rng.choice([0, 40, 500, 2000]))
        ctx_lo = int(rng.integers(0, ctx_hi + 1))
        masks = str(rng.choice(["chain", "tree", "mixed"])) if W > 1 else "chain"
        wl = I.Workload(name=f"nrand{k}", B=B, Hq=Hkv * g, Hkv=Hkv, D=128, W=W, dtype="bf16",
                        ctx_lo=ctx_lo, ctx_hi=ctx_hi, masks=masks,
                        tree_depth=int(min(8, W - 1)) if W > 1 else 1)
        recent = int(rng.choice([-1, 0, int(rng.integers(1, max(2, ctx_hi + 1)))]))
        out.append((wl, recent))
    return out


NESTED = random_nested(24, 4052)


@pytest.mark.parametrize("wl,recent", NESTED,
                         ids=[f"{w.name}-B{w.B}-W{w.W}-h{w.Hq}x{w.Hkv}-{w.masks}-ctx{w.ctx_lo}_{w.ctx_hi}"
                              f"-recent{r}" for w, r in NESTED])
def test_random_shape_nested_attention_matches_oracle(wl, recent):
    inp = gpu_inputs(wl, 78)
    pages, _, Hkv, D = inp["k_cache"].shape
    kv = lib.NestedKV(pages, Hkv, D)
    lib.kv_quantize_cache(inp["k_cache"], inp["v_cache"], kv)
    kp = O.nested_planes(inp["k_cache"].float().cpu().numpy())
    vp = O.nested_planes(inp["v_cache"].float().cpu().numpy())
    out, lse = lib.verify_attn_nested(inp["q"], kv, inp["block_table"], inp["ctx_lens"],
                                      inp["k_new"], inp["v_new"], inp["mask_kind"],
                                      inp["mask_ids"], kv8_recent=recent,
                                      max_ctx_len=int(inp["host"]["ctx_lens"].max()),
                                      scale=inp["scale"], seg_lookback=inp["seg_lookback"])
    torch.cuda.synchronize()
    assert lib.device_status(clear=True) == 0
    ref_out, ref_lse = O.verify_attention_nested(
        inp["q"].double().cpu().numpy(), kp, vp, ints(inp["block_table"]), ints(inp["ctx_lens"]),
        inp["k_new"].double().cpu().numpy(), inp["v_new"].double().cpu().numpy(),
        ints(inp["mask_kind"]), ints(inp["mask_ids"]), inp["scale"], inp["seg_lookback"], recent)
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"{wl.name} recent={recent}")


def random_trees(n: int, seed: int) -> list[tuple]:
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 7))
        K = int(rng.choice([1, 2, 5, 8, 13, 32, 64]))
        V = int(rng.choice([1, 2, 9, 100, 1000, 4096]))
        W = int(rng.choice([1, 2, 7, 16, 33, 64]))
        n_mask = int(rng.integers(0, min(W, 9)))
        thr = float(rng.choice([0.0, 0.0, 1e-4, 1e-2]))
        peak = float(rng.choice([0.5, 2.0, 8.0]))
        out.append((B, K, V, W, n_mask, thr, peak))
    return out


TREES = random_trees(24, 6077)


@pytest.mark.parametrize("case", TREES, ids=[str(c) for c in TREES])
def test_random_shape_tree_matches_oracle(case):
    B, K, V, W, n_mask, thr, peak = case
    inp = I.make_tree_inputs(B, K, V, 57 + K + V + W, peak=peak, device="cuda")
    got = lib.build_tree(inp["probs"], inp["root"], W, n_mask, thr)
    torch.cuda.synchronize()
    ref = O.dynamic_tree(inp["host"]["probs"], inp["host"]["root"], W, n_mask, thr)
    for g, r, name in zip(got, ref, ("draft", "parents", "depth", "n_nodes")):
        assert np.array_equal(ints(g), r), f"{case} {name}: {ints(g)} != {r}"
