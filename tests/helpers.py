"""Shared test helpers: fixture parsing and tensor conversion."""
from __future__ import annotations

import json
import os
import re

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    text = open(os.path.join(GOLDEN, name)).read()
    body = " ".join(line.split("#", 1)[0] for line in text.splitlines())
    parts = re.split(r"(\b[A-Za-z_]\w*)\s*=\s*", body)
    out = {}
    for i in range(1, len(parts), 2):
        out[parts[i]] = json.loads(parts[i + 1].strip())
    return out


def f64(t) -> np.ndarray:
    """Exact fp64 copy of a float tensor (bf16 and fp32 embed exactly)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def ints(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.int64)
    return t.detach().to("cpu", torch.int64).numpy()


def raw(t) -> np.ndarray:
    """Bit pattern of a tensor as a numpy integer array (bf16 -> int16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def oracle_attention(oracle, inp: dict):
    return oracle.verify_attention(
        f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), ints(inp["block_table"]),
        ints(inp["ctx_lens"]), f64(inp["k_new"]), f64(inp["v_new"]), ints(inp["mask_kind"]),
        ints(inp["mask_ids"]), inp["scale"], inp["seg_lookback"])


def oracle_accept(oracle, inp: dict):
    return oracle.accept(inp["logits"].detach().cpu().numpy(), ints(inp["draft_ids"]),
                         ints(inp["mask_kind"]), ints(inp["mask_ids"]))


def within_tol(got: np.ndarray, ref: np.ndarray, atol=1e-3, rtol=1e-2):
    """Elementwise |got - ref| <= atol + rtol*|ref|; returns (ok, worst excess)."""
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    return (not bad.any()), float(np.max(err - bound)) if err.size else 0.0
