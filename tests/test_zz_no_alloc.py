"""mtp_verify_step_noalloc, the step for callers that cannot allocate device
memory (its split-K partials in the library's fixed device scratch), against
mtp_verify_step with a caller workspace on the same inputs: out / lse bit for
bit (same kernels, same plan), acceptance, context lengths and the
committed cache bytes equal.  Two calls in a row, the second smaller and on
the other workspace layout, so it runs on what the first left in the
scratch.  (Shapes beyond the scratch are rejected before any device work;
test_abi_host.py checks that on the host.)"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_common import I, lib, gpu_inputs, ints, raw

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CALLS = [
    # stream-K layout (12 sequences), then the per-split layout (3 sequences)
    I.Workload("noalloc_stream", B=12, Hq=32, Hkv=8, D=128, W=16, dtype="bf16", ctx_lo=100,
               ctx_hi=3000, masks="mixed"),
    I.Workload("noalloc_split", B=3, Hq=20, Hkv=5, D=128, W=8, dtype="bf16", ctx_lo=50,
               ctx_hi=900, masks="chain"),
]


def step(inp, kc, vc, noalloc):
    ctx_out = torch.full_like(inp["ctx_lens"], -3)
    res = lib.verify_step(inp["q"], kc, vc, inp["block_table"], inp["ctx_lens"], inp["k_new"],
                          inp["v_new"], inp["mask_kind"], inp["mask_ids"], inp["logits"],
                          inp["draft_ids"], ctx_lens_out=ctx_out,
                          max_ctx_len=int(inp["host"]["ctx_lens"].max()), scale=inp["scale"],
                          noalloc=noalloc)
    torch.cuda.synchronize()
    return res


def test_noalloc_step_equals_the_workspace_step():
    for call, wl in enumerate(CALLS):
        print(f"[gpu-case] noalloc call {call}: {wl.name} B={wl.B}", flush=True)
        inp = gpu_inputs(wl, 40 + call)
        kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()
        ref = step(inp, inp["k_cache"], inp["v_cache"], noalloc=False)
        got = step(inp, kc, vc, noalloc=True)
        assert lib.device_status(clear=True) == 0
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"call {call} out/lse"
        for g, r in zip(got[2:], ref[2:]):
            assert np.array_equal(ints(g), ints(r)), f"call {call} acceptance / context"
        assert np.array_equal(raw(kc), raw(inp["k_cache"])), f"call {call} K cache"
        assert np.array_equal(raw(vc), raw(inp["v_cache"])), f"call {call} V cache"
