"""GPU parity of the dynamic token tree builder: draft ids, parent array,
depths and node counts bit-exact against the oracle (the comparisons are
fp32 products and compares on both sides)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_common import I, O, banner, ints, lib

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [  # B, K, V, W, n_mask, min_cum_prob, peak
    (4, 8, 1000, 32, 4, 0.0, 8.0),
    (4, 8, 1000, 32, 4, 1e-3, 8.0),
    (3, 4, 1000, 64, 0, 0.0, 4.0),
    (2, 16, 50, 20, 3, 0.0, 2.0),
    (2, 1, 30, 10, 2, 0.0, 8.0),
    (5, 20, 7, 40, 5, 0.0, 1.0),
    (2, 3, 4096, 24, 2, 0.0, 8.0),   # the largest vocabulary
    (2, 64, 200, 64, 8, 0.0, 8.0),
    (3, 6, 100, 1, 0, 0.0, 8.0),     # W = 1: the root only
    (3, 6, 100, 8, 7, 0.0, 8.0),     # no predicted rows
    (2, 5, 1, 6, 1, 0.0, 8.0),       # one-token vocabulary
]


def check(inp, W, n_mask, thr):
    got = lib.build_tree(inp["probs"], inp["root"], W, n_mask, thr)
    torch.cuda.synchronize()
    ref = O.dynamic_tree(inp["host"]["probs"], inp["host"]["root"], W, n_mask, thr)
    for g, r, name in zip(got, ref, ("draft", "parents", "depth", "n_nodes")):
        assert np.array_equal(ints(g), r), f"{name}: {ints(g)} != {r}"


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_tree_matches_oracle(case):
    B, K, V, W, n_mask, thr, peak = case
    banner(f"tree B={B} K={K} V={V} W={W} n_mask={n_mask} thr={thr}")
    inp = I.make_tree_inputs(B, K, V, 31 + K + V, peak=peak, device="cuda")
    check(inp, W, n_mask, thr)


def test_tree_ties_and_zero_probabilities():
    banner("tree ties")
    p = np.zeros((2, 4, 64), dtype=np.float32)
    p[0] = 1.0 / 64          # every token ties
    p[1, :, :8] = 0.125      # eight tokens tie, the rest are 0
    inp = dict(probs=torch.from_numpy(p).cuda(),
               root=torch.tensor([3, 70], dtype=torch.int32).cuda(),
               host=dict(probs=p, root=np.array([3, 70])))
    check(inp, 40, 2, 0.0)
    check(inp, 40, 2, 1.0 / 64)


def test_tree_output_feeds_the_verify_step():
    """The block the builder emits is a valid TREE description for the
    acceptance kernel, whose result matches the oracle's on it."""
    banner("tree -> accept")
    inp = I.make_tree_inputs(3, 8, 1000, 77, device="cuda")
    d, par, dep, n = lib.build_tree(inp["probs"], inp["root"], 24, 4)
    B, W, V = 3, 24, 1000
    g = torch.Generator().manual_seed(5)
    logits = torch.randn((B, W, V), generator=g)
    kinds = torch.full((B,), lib.MASK_TREE, dtype=torch.uint8)
    got = lib.accept(logits.cuda(), d, kinds.cuda(), par)
    torch.cuda.synchronize()
    ref = O.accept(logits.numpy(), ints(d), kinds.numpy(), ints(par))
    assert all(np.array_equal(ints(a), b) for a, b in zip(got, ref))
    assert lib.device_status(clear=True) == 0


@pytest.mark.parametrize("masks", ["chain", "tree", "segment", "mixed"])
def test_block_positions_match_oracle(masks):
    banner(f"positions {masks}")
    wl = I.Workload(name="pos", B=9, Hq=2, Hkv=2, D=64, W=24, dtype="bf16", ctx_lo=0,
                    ctx_hi=500, masks=masks)
    inp = I.make_inputs(wl, 3, device="cuda")
    got = lib.block_positions(inp["ctx_lens"], inp["mask_kind"], inp["mask_ids"])
    torch.cuda.synchronize()
    h = inp["host"]
    assert np.array_equal(ints(got), O.block_positions(h["ctx_lens"], h["mask_kind"],
                                                        h["mask_ids"]))


def test_tree_rejects_vocabularies_above_4096():
    inp = I.make_tree_inputs(1, 2, 4097, 5, device="cuda")
    with pytest.raises(lib.MtpError):
        lib.build_tree(inp["probs"], inp["root"], 8, 1)
