"""A device-resident decode loop: N verify steps captured in one HIP graph,
each step's context lengths written by the previous step's commit
(ping-pong buffers), block positions prepared on the device from them, no
host synchronisation in between.  Checked against the oracle applied step
by step (attention within tolerance; acceptance, positions, committed cache
bytes and context lengths exact), and replayed twice from the same state."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_common import ATOL, RTOL, I, O, assert_attn_close, banner, f64, ints, lib, raw

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore::RuntimeWarning"),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

N = 4


def bf16_from_raw(r: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(r)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("masks", ["mixed", "chain"])
def test_graph_captured_decode_loop(masks):
    wl = I.Workload(name="loop", B=4, Hq=8, Hkv=2, D=128, W=8, dtype="bf16", ctx_lo=20,
                    ctx_hi=150, masks=masks, commit_steps=N, match_p=0.8)
    banner(f"loop N={N} {wl}")
    base = I.make_inputs(wl, 41, device="cuda")
    steps = [I.make_inputs(wl, 41 + 100 * (k + 1), device="cuda") for k in range(N)]
    bt = base["block_table"]
    kc0, vc0 = base["k_cache"].clone(), base["v_cache"].clone()
    kc, vc = base["k_cache"].clone(), base["v_cache"].clone()
    ctx = [base["ctx_lens"].clone(), torch.empty_like(base["ctx_lens"])]
    ctx0 = base["ctx_lens"].clone()
    mc = int(base["host"]["ctx_lens"].max()) + N * wl.W
    shape = lib.shape_of(steps[0]["q"], kc, bt, max_ctx_len=mc, scale=base["scale"])
    ws = torch.empty(max(lib.workspace_bytes(shape), 16), dtype=torch.uint8, device="cuda")
    B, W, Hq, D = steps[0]["q"].shape
    outs = [dict(out=torch.empty((B, W, Hq, D), device="cuda"),
                 lse=torch.empty((B, W, Hq), device="cuda"),
                 alen=torch.empty(B, dtype=torch.int32, device="cuda"),
                 apath=torch.empty((B, W), dtype=torch.int32, device="cuda"),
                 bonus=torch.empty(B, dtype=torch.int32, device="cuda"),
                 pos=torch.empty((B, W), dtype=torch.int32, device="cuda")) for _ in range(N)]

    def loop():
        for k in range(N):
            s, o = steps[k], outs[k]
            cin, cout = ctx[k % 2], ctx[(k + 1) % 2]
            lib.block_positions(cin, s["mask_kind"], s["mask_ids"], positions=o["pos"])
            lib.verify_step(s["q"], kc, vc, bt, cin, s["k_new"], s["v_new"], s["mask_kind"],
                            s["mask_ids"], s["logits"], s["draft_ids"], out=o["out"], lse=o["lse"],
                            accept_len=o["alen"], accept_path=o["apath"], bonus_id=o["bonus"],
                            ctx_lens_out=cout, workspace=ws, shape=shape)

    loop()  # eager once (loads the code objects)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    results = []
    for rep in range(2):
        kc.copy_(kc0)
        vc.copy_(vc0)
        ctx[0].copy_(ctx0)
        torch.cuda.synchronize()
        if rep == 0:
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    loop()
            torch.cuda.synchronize()
            kc.copy_(kc0)
            vc.copy_(vc0)
            ctx[0].copy_(ctx0)
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        results.append(([{k: v.clone() for k, v in o.items()} for o in outs], raw(kc), raw(vc),
                        ints(ctx[N % 2])))
    assert lib.device_status(clear=True) == 0

    # the oracle, step by step
    host = base["host"]
    rk, rv, rctx = raw(kc0), raw(vc0), host["ctx_lens"].astype(np.int64)
    for k in range(N):
        s = steps[k]
        sh = s["host"]
        ref_out, ref_lse = O.verify_attention(f64(s["q"]), bf16_from_raw(rk), bf16_from_raw(rv),
                                              host["block_table"], rctx, f64(s["k_new"]),
                                              f64(s["v_new"]), sh["mask_kind"], sh["mask_ids"],
                                              base["scale"])
        ref_acc = O.accept(s["logits"].cpu().numpy(), sh["draft_ids"], sh["mask_kind"],
                           sh["mask_ids"])
        ref_pos = O.block_positions(rctx, sh["mask_kind"], sh["mask_ids"])
        for rep in range(2):
            o = results[rep][0][k]
            assert_attn_close(o["out"], o["lse"], ref_out, ref_lse, ATOL, RTOL, f"step {k}")
            assert np.array_equal(ints(o["alen"]), ref_acc[0]), f"step {k} accept_len"
            assert np.array_equal(ints(o["apath"]), ref_acc[1]), f"step {k} accept_path"
            assert np.array_equal(ints(o["bonus"]), ref_acc[2]), f"step {k} bonus"
            assert np.array_equal(ints(o["pos"]), ref_pos), f"step {k} positions"
        rk, rv, rctx = O.kv_commit(rk, rv, raw(s["k_new"]), raw(s["v_new"]), ref_acc[0],
                                   ref_acc[1], host["block_table"], rctx)
    for rep in range(2):
        _, gk, gv, gctx = results[rep]
        assert np.array_equal(gctx, rctx)
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    assert (rctx - host["ctx_lens"] >= N).all()


def test_tree_builder_feeds_the_step_on_the_device():
    """Drafter probabilities -> dynamic tree (block of the next step) ->
    positions -> verify step (tree mask from the builder) -> commit, all on
    the device; the oracle takes the same path on the CPU."""
    B, W, n_mask, K = 3, 16, 3, 6
    wl = I.Workload(name="tree_step", B=B, Hq=8, Hkv=2, D=128, W=W, dtype="bf16", ctx_lo=40,
                    ctx_hi=300, masks="tree")
    banner(f"tree -> step {wl}")
    base = I.make_inputs(wl, 61, device="cuda")
    tin = I.make_tree_inputs(B, K, wl.vocab, 62, device="cuda")
    root = base["draft_ids"][:, 0].contiguous()  # any token: the anchor
    draft, parents, depth, n_nodes = lib.build_tree(tin["probs"], root, W, n_mask)
    kinds = torch.full((B,), lib.MASK_TREE, dtype=torch.uint8, device="cuda")
    pos = lib.block_positions(base["ctx_lens"], kinds, parents)
    kc, vc = base["k_cache"].clone(), base["v_cache"].clone()
    out, lse, alen, apath, bonus, ctx_out = lib.verify_step(
        base["q"], kc, vc, base["block_table"], base["ctx_lens"], base["k_new"], base["v_new"],
        kinds, parents, base["logits"], draft, scale=base["scale"])
    torch.cuda.synchronize()
    assert lib.device_status(clear=True) == 0
    h = base["host"]
    rd, rp, rdep, rn = O.dynamic_tree(tin["host"]["probs"], ints(root), W, n_mask)
    assert np.array_equal(ints(draft), rd) and np.array_equal(ints(parents), rp)
    assert np.array_equal(ints(pos), O.block_positions(h["ctx_lens"], ints(kinds), rp))
    assert np.array_equal(ints(pos), h["ctx_lens"][:, None] + rdep)
    ref_out, ref_lse = O.verify_attention(f64(base["q"]), f64(base["k_cache"]),
                                          f64(base["v_cache"]), h["block_table"], h["ctx_lens"],
                                          f64(base["k_new"]), f64(base["v_new"]), ints(kinds), rp,
                                          base["scale"])
    assert_attn_close(out, lse, ref_out, ref_lse, ATOL, RTOL, "tree step")
    ra = O.accept(base["logits"].cpu().numpy(), rd, ints(kinds), rp)
    assert np.array_equal(ints(alen), ra[0]) and np.array_equal(ints(apath), ra[1])
    assert np.array_equal(ints(bonus), ra[2])
    rk, rv, rctx = O.kv_commit(raw(base["k_cache"]), raw(base["v_cache"]), raw(base["k_new"]),
                               raw(base["v_new"]), ra[0], ra[1], h["block_table"], h["ctx_lens"])
    assert np.array_equal(ints(ctx_out), rctx)
    assert np.array_equal(raw(kc), rk) and np.array_equal(raw(vc), rv)
