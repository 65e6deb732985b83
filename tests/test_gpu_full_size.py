"""GPU parity of the whole verify step at the five workloads' full sizes, in
the launch configuration the benchmark times: mtp_verify_step with the
automatic plan (the partial kernel, then one launch running the combine
beside acceptance and commit), and mtp_verify_attn (the partial kernel, then
the combine launch on its own).

Attention is compared with the fp64 oracle on every output row within
|d| <= 1e-3 + 1e-2 |ref| (bf16 inputs) or 1e-4 + 1e-4 |ref| (fp32 inputs);
acceptance, paths, bonus ids, context lengths and the committed cache bytes
are compared bit for bit.  The ragged batch (64 sequences, 4.9 GB of paged
K/V) is compared on all of its sequences, eight at a time: the oracle's
dense fp64 copy of the whole pool would need about 20 GB of host memory.
The nested KV8 / KV4 cache is compared the same way on the ragged batch.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_common import (ATOL, RTOL, I, O, lib, assert_accept_equal, assert_attn_close,
                              banner, f64, gpu_inputs, ints, oracle_accept, oracle_attn,
                              oracle_attn_sub, raw, sub_problem, tol_for)

pytestmark = [pytest.mark.gpu,
              pytest.mark.filterwarnings("ignore::RuntimeWarning"),
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_step(inp: dict, ctx_out: torch.Tensor):
    """mtp_verify_step as the benchmark launches it (automatic split plan,
    bound = the longest context, separate ctx_lens_out)."""
    mc = int(inp["host"]["ctx_lens"].max())
    return lib.verify_step(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                           inp["ctx_lens"], inp["k_new"], inp["v_new"], inp["mask_kind"],
                           inp["mask_ids"], inp["logits"], inp["draft_ids"], ctx_lens_out=ctx_out,
                           max_ctx_len=mc, scale=inp["scale"], seg_lookback=inp["seg_lookback"])


FULL = [("tiny_chain", -1), ("bitnet2b_chain", -1), ("llama3_8b_tree", -1),
        ("lca_segments", -1), ("lca_segments", 1)]


@pytest.mark.parametrize("name,lookback", FULL, ids=[f"{n}_lb{lb}" for n, lb in FULL])
def test_full_size_step(name, lookback):
    """The whole step on one workload: attention rows, acceptance, the new
    context lengths and every byte of both caches after the commit."""
    wl = I.WORKLOADS[name].scaled(seg_lookback=lookback)
    inp = gpu_inputs(wl, I.workload_seed(name))
    kc0, vc0 = raw(inp["k_cache"]), raw(inp["v_cache"])
    ref_out, ref_lse = oracle_attn(inp)
    n_ref, path_ref, bonus_ref = oracle_accept(inp)
    kc_ref, vc_ref, ctx_ref = O.kv_commit(kc0, vc0, raw(inp["k_new"]), raw(inp["v_new"]), n_ref,
                                          path_ref, ints(inp["block_table"]),
                                          ints(inp["ctx_lens"]), False)
    del kc0, vc0
    # the attention on its own first (it reads the cache before the commit)
    mc = int(inp["host"]["ctx_lens"].max())
    out_a, lse_a = lib.verify_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                                   inp["ctx_lens"], inp["k_new"], inp["v_new"], inp["mask_kind"],
                                   inp["mask_ids"], max_ctx_len=mc, scale=inp["scale"],
                                   seg_lookback=inp["seg_lookback"])
    ctx_out = torch.full_like(inp["ctx_lens"], -3)
    out, lse, n, path, bonus, ctx_out = run_step(inp, ctx_out)
    torch.cuda.synchronize()
    assert lib.device_status(clear=True) == 0
    assert_attn_close(out_a, lse_a, ref_out, ref_lse, *tol_for(wl), what=f"{name} attn")
    assert_attn_close(out, lse, ref_out, ref_lse, *tol_for(wl), what=f"{name} step")
    assert_accept_equal((n, path, bonus), (n_ref, path_ref, bonus_ref))
    assert np.array_equal(ints(ctx_out), ctx_ref)
    assert np.array_equal(ints(inp["ctx_lens"]), inp["host"]["ctx_lens"])  # input untouched
    assert np.array_equal(raw(inp["k_cache"]), kc_ref)
    assert np.array_equal(raw(inp["v_cache"]), vc_ref)


# ----------------------------------------------------------------------------
# the ragged batch: one step on the GPU, compared eight sequences at a time
# ----------------------------------------------------------------------------

RAGGED_CHUNK = 8
RAGGED_B = I.WORKLOADS["ragged_batch"].B


@pytest.fixture(scope="module")
def ragged():
    name = "ragged_batch"
    wl = I.WORKLOADS[name]
    inp = gpu_inputs(wl, I.workload_seed(name))
    pre_k, pre_v = inp["k_cache"].clone(), inp["v_cache"].clone()
    mc = int(inp["host"]["ctx_lens"].max())
    out_a, lse_a = lib.verify_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                                   inp["ctx_lens"], inp["k_new"], inp["v_new"], inp["mask_kind"],
                                   inp["mask_ids"], max_ctx_len=mc, scale=inp["scale"],
                                   seg_lookback=inp["seg_lookback"])
    ctx_out = torch.full_like(inp["ctx_lens"], -3)
    out, lse, n, path, bonus, ctx_out = run_step(inp, ctx_out)
    torch.cuda.synchronize()
    status = lib.device_status(clear=True)
    res = dict(inp=inp, pre=dict(inp, k_cache=pre_k, v_cache=pre_v), status=status,
               attn=(out_a.cpu(), lse_a.cpu()), step=(out.cpu(), lse.cpu()),
               accept=(n.cpu(), path.cpu(), bonus.cpu()), ctx_out=ctx_out.cpu())
    yield res
    res.clear()
    del inp, pre_k, pre_v
    torch.cuda.empty_cache()


def test_ragged_step_acceptance_and_context(ragged):
    assert ragged["status"] == 0
    inp = ragged["inp"]
    n_ref, path_ref, bonus_ref = oracle_accept(inp)
    assert_accept_equal(ragged["accept"], (n_ref, path_ref, bonus_ref))
    assert np.array_equal(ints(ragged["ctx_out"]), inp["host"]["ctx_lens"] + n_ref + 1)


def test_ragged_step_writes_only_the_accepted_slots(ragged):
    """Every slot the commit changed is one of the accepted rows' target
    slots, and every such slot changed (it held NaN before)."""
    inp, pre = ragged["inp"], ragged["pre"]
    changed = torch.zeros(inp["k_cache"].shape[:2], dtype=torch.bool, device="cuda")
    for post, before in ((inp["k_cache"], pre["k_cache"]), (inp["v_cache"], pre["v_cache"])):
        changed |= (post.view(torch.int16) != before.view(torch.int16)).any(dim=3).any(dim=2)
    changed = changed.cpu().numpy()
    n = ints(ragged["accept"][0])
    host = inp["host"]
    want = np.zeros_like(changed)
    for b in range(RAGGED_B):
        for k in range(int(n[b]) + 1):
            t = int(host["ctx_lens"][b]) + k
            want[host["block_table"][b, t // 16], t % 16] = True
    assert np.array_equal(changed, want)


@pytest.mark.parametrize("chunk", range(RAGGED_B // RAGGED_CHUNK))
def test_ragged_step_chunk(ragged, chunk):
    """Eight sequences of the ragged batch: attention rows of both launch
    paths against the oracle, and the committed pages byte for byte."""
    seqs = list(range(chunk * RAGGED_CHUNK, (chunk + 1) * RAGGED_CHUNK))
    inp, pre = ragged["inp"], ragged["pre"]
    wl = inp["workload"]
    ctx = inp["host"]["ctx_lens"]
    banner(f"ragged chunk {chunk}: sequences {seqs} ctx {[int(ctx[b]) for b in seqs]}")
    sub = sub_problem(pre, seqs)
    ref_out, ref_lse = oracle_attn_sub(sub)
    for what, (out, lse) in (("attn", ragged["attn"]), ("step", ragged["step"])):
        assert_attn_close(out[seqs], lse[seqs], ref_out, ref_lse, *tol_for(wl),
                          what=f"ragged chunk {chunk} {what}")
    n_ref, path_ref, _ = oracle_accept(inp)
    kc_ref, vc_ref, _ = O.kv_commit(raw(sub["k_cache"]), raw(sub["v_cache"]),
                                    raw(sub["k_new"]), raw(sub["v_new"]), n_ref[seqs],
                                    path_ref[seqs], sub["block_table"], sub["ctx_lens"], False)
    post = sub_problem(inp, seqs)  # the same pages after the step
    assert np.array_equal(raw(post["k_cache"]), kc_ref)
    assert np.array_equal(raw(post["v_cache"]), vc_ref)


# ----------------------------------------------------------------------------
# nested KV8 / KV4 cache on the full ragged batch
# ----------------------------------------------------------------------------

NESTED_READS = {"kv8": -1, "kv4": 0, "recent1024": 1024}


@pytest.fixture(scope="module")
def ragged_nested(ragged):
    pre = ragged["pre"]
    pages, _, Hkv, D = pre["k_cache"].shape
    kv = lib.NestedKV(pages, Hkv, D)
    lib.kv_quantize_cache(pre["k_cache"], pre["v_cache"], kv)
    mc = int(pre["host"]["ctx_lens"].max())
    outs = {}
    for key, recent in NESTED_READS.items():
        out, lse = lib.verify_attn_nested(pre["q"], kv, pre["block_table"], pre["ctx_lens"],
                                          pre["k_new"], pre["v_new"], pre["mask_kind"],
                                          pre["mask_ids"], kv8_recent=recent, max_ctx_len=mc,
                                          scale=pre["scale"], seg_lookback=pre["seg_lookback"])
        torch.cuda.synchronize()
        outs[key] = (out.cpu(), lse.cpu())
    status = lib.device_status(clear=True)
    del kv
    torch.cuda.empty_cache()
    return dict(outs=outs, status=status)


@pytest.mark.parametrize("chunk", range(RAGGED_B // RAGGED_CHUNK))
def test_ragged_nested_chunk(ragged, ragged_nested, chunk):
    """KV8, KV4 and Recent-1024 reads of the nested cache on eight sequences
    against the oracle's attention over its own dequantized planes."""
    assert ragged_nested["status"] == 0
    seqs = list(range(chunk * RAGGED_CHUNK, (chunk + 1) * RAGGED_CHUNK))
    banner(f"ragged nested chunk {chunk}: sequences {seqs}")
    sub = sub_problem(ragged["pre"], seqs)
    kp = O.nested_planes(sub["k_cache"].float().numpy())
    vp = O.nested_planes(sub["v_cache"].float().numpy())
    for key, recent in NESTED_READS.items():
        ref_out, ref_lse = O.verify_attention_nested(
            f64(sub["q"]), kp, vp, sub["block_table"], sub["ctx_lens"], f64(sub["k_new"]),
            f64(sub["v_new"]), sub["mask_kind"], sub["mask_ids"], sub["scale"],
            sub["seg_lookback"], recent)
        out, lse = ragged_nested["outs"][key]
        assert_attn_close(out[seqs], lse[seqs], ref_out, ref_lse, ATOL, RTOL,
                          what=f"ragged nested chunk {chunk} {key}")
