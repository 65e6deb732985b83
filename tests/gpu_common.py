"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare it with the fp64 oracle on the same input bytes."""
from __future__ import annotations

import numpy as np
import torch

from oracle import verify_oracle as O
from speculative_decoding_verify_mtp_amd import inputs as I
from speculative_decoding_verify_mtp_amd import lib
from tests.helpers import f64, ints, raw, within_tol

ATOL, RTOL = 1e-3, 1e-2  # bf16 inputs, fp32 outputs
ATOL32, RTOL32 = 1e-4, 1e-4  # fp32 inputs


def tol_for(wl: I.Workload):
    return (ATOL32, RTOL32) if wl.dtype == "f32" else (ATOL, RTOL)


def banner(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def gpu_inputs(wl: I.Workload, seed: int) -> dict:
    banner(f"{wl.name} B={wl.B} W={wl.W} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} dtype={wl.dtype} "
           f"ctx=[{wl.ctx_lo},{wl.ctx_hi}] masks={wl.masks} lookback={wl.seg_lookback} seed={seed}")
    return I.make_inputs(wl, seed, device="cuda")


def run_attn(inp: dict, split_tokens: int = 0, max_ctx_len: int | None = None):
    host = inp["host"]
    mc = int(host["ctx_lens"].max()) if max_ctx_len is None else max_ctx_len
    mc = max(mc, 0)
    out, lse = lib.verify_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                               inp["ctx_lens"], inp["k_new"], inp["v_new"], inp["mask_kind"],
                               inp["mask_ids"], max_ctx_len=mc, scale=inp["scale"],
                               seg_lookback=inp["seg_lookback"], split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out, lse


def assert_attn_close(out, lse, ref_out, ref_lse, atol, rtol, what=""):
    got = out.detach().cpu().double().numpy()
    ok, worst = within_tol(got, ref_out, atol, rtol)
    assert ok, f"{what} out: worst excess over tolerance {worst:.3e}"
    if lse is not None:
        gl = lse.detach().cpu().double().numpy()
        ok, worst = within_tol(gl, ref_lse, atol, rtol)
        assert ok, f"{what} lse: worst excess over tolerance {worst:.3e}"


def sub_problem(inp: dict, seqs: list[int]) -> dict:
    """The sequences `seqs` of a batch as a small stand-alone problem: only
    their pages are copied (to the host, exactly) and the block table is
    renumbered.  Input preparation for the oracle; no arithmetic."""
    host = inp["host"]
    W = inp["q"].shape[1]
    tables, pages = [], []
    for b in seqs:
        L = int(host["ctx_lens"][b])
        n = (L + W + 15) // 16
        pages.append(host["block_table"][b, :n])
    flat = np.concatenate(pages)
    idx = torch.from_numpy(flat.astype(np.int64)).to(inp["k_cache"].device)
    kc = inp["k_cache"].index_select(0, idx).cpu()
    vc = inp["v_cache"].index_select(0, idx).cpu()
    maxp = max(len(p) for p in pages)
    table = np.full((len(seqs), maxp), -1, dtype=np.int64)
    cur = 0
    for i, p in enumerate(pages):
        table[i, :len(p)] = np.arange(cur, cur + len(p))
        cur += len(p)
    sel = torch.tensor(seqs, dtype=torch.int64)
    return dict(q=inp["q"].cpu()[sel], k_cache=kc, v_cache=vc, block_table=table,
                ctx_lens=host["ctx_lens"][seqs], k_new=inp["k_new"].cpu()[sel],
                v_new=inp["v_new"].cpu()[sel], mask_kind=host["mask_kind"][seqs],
                mask_ids=host["mask_ids"][seqs], scale=inp["scale"],
                seg_lookback=inp["seg_lookback"])


def oracle_attn_sub(sub: dict):
    return O.verify_attention(f64(sub["q"]), f64(sub["k_cache"]), f64(sub["v_cache"]),
                              sub["block_table"], sub["ctx_lens"], f64(sub["k_new"]),
                              f64(sub["v_new"]), sub["mask_kind"], sub["mask_ids"], sub["scale"],
                              sub["seg_lookback"])


def oracle_attn(inp: dict):
    return O.verify_attention(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                              ints(inp["block_table"]), ints(inp["ctx_lens"]), f64(inp["k_new"]),
                              f64(inp["v_new"]), ints(inp["mask_kind"]), ints(inp["mask_ids"]),
                              inp["scale"], inp["seg_lookback"])


def oracle_accept(inp: dict):
    return O.accept(inp["logits"].detach().cpu().numpy(), ints(inp["draft_ids"]),
                    ints(inp["mask_kind"]), ints(inp["mask_ids"]))


def assert_accept_equal(got, ref):
    n, path, bonus = (ints(t) for t in got)
    rn, rpath, rbonus = ref
    assert np.array_equal(n, rn), f"accept_len {n} != {rn}"
    assert np.array_equal(path, rpath), "accept_path differs"
    assert np.array_equal(bonus, rbonus), f"bonus {bonus} != {rbonus}"


__all__ = ["I", "O", "lib", "raw", "f64", "ints", "np", "torch"]
