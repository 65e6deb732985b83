"""Pins of the oracle's nested KV4 / KV8 cache against facts it does not
define: hand-worked vectors, brute-force nearest codes, error bounds of
round-to-nearest, exact scaling and sign symmetry, and reduction of the
nested attention to the dense (already pinned) attention on grid-exact data."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import verify_oracle as O
from speculative_decoding_verify_mtp_amd import inputs as I
from tests.helpers import load_golden


def test_golden_rows():
    g = load_golden("nested_kv_rows.txt")
    q4, qr, s = O.quantize_nested(np.array(g["a_x"]))
    assert s == g["a_scale"]
    assert list(q4) == g["a_q4"] and list(qr) == g["a_qr"]
    assert list(O.pack_nibbles(q4)) == g["a_base_bytes"]
    assert list(O.pack_nibbles(qr)) == g["a_ref_bytes"]
    planes = {"base": O.pack_nibbles(q4)[None, None, None], "ref": O.pack_nibbles(qr)[None, None, None],
              "scale": np.array([[[s]]], dtype=np.float32)}
    assert list(O.dequantize_nested(planes, 8)[0, 0, 0]) == g["a_kv8"]
    assert list(O.dequantize_nested(planes, 4)[0, 0, 0]) == g["a_kv4"]
    q4, qr, s = O.quantize_nested(np.array(g["b_x"]))
    assert s == g["b_scale"] and list(q4) == g["b_q4"] and list(qr) == g["b_qr"]
    assert list(s * (16 * q4 + qr) / 16) == g["b_kv8"]
    q4, qr, s = O.quantize_nested(np.array(g["c_x"]))
    assert s == 0 and not q4.any() and not qr.any()


def _rows(seed, n=400, D=128):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)) * rng.choice([1e-3, 1.0, 30.0], size=(n, 1))
    return x.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("seed", range(3))
def test_codes_are_the_nearest_grid_points(seed):
    """Brute force over all 16 base codes, then all 16 refinement codes."""
    x = _rows(seed)
    q4, qr, s = O.quantize_nested(x)
    s64 = s.astype(np.float64)[:, None]
    ks = np.arange(-8, 8)
    d4 = np.abs(x[..., None] - s64[..., None] * ks)          # [n, D, 16]
    best4 = ks[np.argmin(d4, axis=-1)]
    srt = np.sort(d4, axis=-1)
    clear = srt[..., 1] - srt[..., 0] > 1e-5 * s64          # skip near-ties
    assert np.array_equal(q4[clear], best4[clear])
    resid = x - s64 * q4
    dr = np.abs(resid[..., None] - (s64 / 16)[..., None] * ks)
    bestr = ks[np.argmin(dr, axis=-1)]
    srt = np.sort(dr, axis=-1)
    clear = srt[..., 1] - srt[..., 0] > 1e-5 * s64
    assert np.array_equal(qr[clear], bestr[clear])


@pytest.mark.parametrize("seed", range(3))
def test_round_to_nearest_error_bounds(seed):
    x = _rows(seed)
    q4, qr, s = O.quantize_nested(x)
    s64 = s.astype(np.float64)[:, None]
    amax = np.abs(x).max(axis=1)
    assert np.all(np.abs(s.astype(np.float64) * 7 - amax) <= 1e-6 * amax)
    assert q4.min() >= -7 and q4.max() <= 7 and qr.min() >= -8 and qr.max() <= 7
    kv4, kv8 = s64 * q4, s64 * (16 * q4 + qr) / 16
    tol = 1e-6 * s64
    assert np.all(np.abs(x - kv4) <= s64 / 2 + tol)
    clamped = qr == 7
    assert np.all(np.abs(x - kv8)[~clamped] <= s64.repeat(x.shape[1], 1)[~clamped] / 32 + tol.repeat(x.shape[1], 1)[~clamped])
    assert np.all(np.abs(x - kv8) <= s64 / 16 + tol)
    # the largest element is on both grids
    i = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q4[np.arange(len(x)), i]) == 7) and np.all(qr[np.arange(len(x)), i] == 0)


def test_power_of_two_scaling_and_sign_symmetry():
    x = _rows(7, n=200)
    q4, qr, s = O.quantize_nested(x)
    for k in (-6, 3):
        q4k, qrk, sk = O.quantize_nested(x * 2.0 ** k)
        assert np.array_equal(q4k, q4) and np.array_equal(qrk, qr)
        assert np.array_equal(sk, (s * np.float32(2.0 ** k)).astype(np.float32))
    q4n, qrn, sn = O.quantize_nested(-x)
    assert np.array_equal(sn, s) and np.array_equal(q4n, -q4)
    free = (qr != 7) & (qr != -8)
    assert np.array_equal(qrn[free], -qr[free])


def test_pack_round_trip():
    rng = np.random.default_rng(3)
    c = rng.integers(-8, 8, size=(5, 3, 64))
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(c)), c)


def _grid_cache(rng, pages, Hkv, D, refine=True):
    """A cache whose every row lies on its own KV8 grid (so KV8 reproduces it
    exactly): integer codes times s/16 with the largest element +-7 s."""
    s = rng.choice([0.125, 0.25, 0.5], size=(pages, 16, Hkv, 1))
    q4 = rng.integers(-7, 8, size=(pages, 16, Hkv, D))
    # |qr| < 8: a refinement of -8 is a tie of the base rounding
    qr = rng.integers(-7, 8, size=(pages, 16, Hkv, D)) if refine else np.zeros_like(q4)
    q4[..., 0], qr[..., 0] = 7, 0
    qr = np.where(np.abs(16 * q4 + qr) > 112, 0, qr)  # stay within max |x| = 7 s
    return s * (16 * q4 + qr) / 16


@pytest.mark.parametrize("masks", ["chain", "tree", "mixed"])
def test_grid_exact_cache_reduces_to_dense_attention(masks):
    wl = I.Workload(name="n", B=3, Hq=4, Hkv=2, D=32, W=6, dtype="f32", ctx_lo=5, ctx_hi=40,
                    masks=masks)
    inp = I.make_inputs(wl, 5)
    st = inp["host"]
    rng = np.random.default_rng(11)
    pages = inp["k_cache"].shape[0]
    for refine, recent in ((True, -1), (False, 0), (False, 7)):
        kc, vc = _grid_cache(rng, pages, 2, 32, refine), _grid_cache(rng, pages, 2, 32, refine)
        kp, vp = O.nested_planes(kc), O.nested_planes(vc)
        args = (inp["q"].numpy(), st["block_table"], st["ctx_lens"], inp["k_new"].numpy(),
                inp["v_new"].numpy(), st["mask_kind"], st["mask_ids"])
        ref = O.verify_attention(args[0], kc, vc, *args[1:])
        got = O.verify_attention_nested(args[0], kp, vp, *args[1:], kv8_recent=recent)
        np.testing.assert_allclose(got[0], ref[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got[1], ref[1], rtol=1e-12, atol=1e-12)


def test_recent_window_reads_kv8_only_for_the_newest_tokens():
    wl = I.Workload(name="n", B=2, Hq=2, Hkv=1, D=16, W=3, dtype="f32", ctx_lo=30, ctx_hi=50,
                    masks="chain")
    inp = I.make_inputs(wl, 6)
    st = inp["host"]
    kc, vc = inp["k_cache"].numpy(), inp["v_cache"].numpy()
    kc, vc = np.nan_to_num(kc), np.nan_to_num(vc)
    kp, vp = O.nested_planes(kc), O.nested_planes(vc)
    k8, k4 = O.dequantize_nested(kp, 8), O.dequantize_nested(kp, 4)
    v8, v4 = O.dequantize_nested(vp, 8), O.dequantize_nested(vp, 4)
    args = (st["mask_kind"], st["mask_ids"])
    for N in (0, 1, 17, 10**6):
        for b in range(wl.B):
            L = int(st["ctx_lens"][b])
            mk, mv = k8.copy(), v8.copy()
            for t in range(max(0, L - N)):  # older tokens, KV4, by hand
                page, slot = st["block_table"][b, t // 16], t % 16
                mk[page, slot], mv[page, slot] = k4[page, slot], v4[page, slot]
            one = slice(b, b + 1)
            ref = O.verify_attention(inp["q"].numpy()[one], mk, mv, st["block_table"][one],
                                     st["ctx_lens"][one], inp["k_new"].numpy()[one],
                                     inp["v_new"].numpy()[one], args[0][one], args[1][one])
            got = O.verify_attention_nested(inp["q"].numpy()[one], kp, vp, st["block_table"][one],
                                            st["ctx_lens"][one], inp["k_new"].numpy()[one],
                                            inp["v_new"].numpy()[one], args[0][one], args[1][one],
                                            kv8_recent=N)
            np.testing.assert_allclose(got[0], ref[0], rtol=1e-12, atol=1e-12)
    assert not np.allclose(k8, k4)


@pytest.mark.parametrize("skip_root", [False, True])
def test_nested_commit_quantizes_exactly_the_accepted_rows(skip_root):
    wl = I.Workload(name="n", B=4, Hq=4, Hkv=2, D=32, W=8, dtype="bf16", ctx_lo=3, ctx_hi=60,
                    masks="mixed")
    inp = I.make_inputs(wl, 8)
    st = inp["host"]
    kc = np.nan_to_num(inp["k_cache"].float().numpy())
    vc = np.nan_to_num(inp["v_cache"].float().numpy())
    kp, vp = O.nested_planes(kc), O.nested_planes(vc)
    n, path, _ = O.accept(inp["logits"].numpy(), st["draft_ids"], st["mask_kind"], st["mask_ids"])
    kn, vn = inp["k_new"].float().numpy(), inp["v_new"].float().numpy()
    kp2, vp2, ctx = O.kv_commit_nested(kp, vp, kn, vn, n, path, st["block_table"], st["ctx_lens"],
                                       skip_root)
    assert np.array_equal(ctx, st["ctx_lens"] + n + 1)
    touched = np.zeros(kp["scale"].shape[::2], dtype=bool)  # [pages, 16]
    for b in range(wl.B):
        for k in range(1 if skip_root else 0, int(n[b]) + 1):
            t = int(st["ctx_lens"][b]) + k
            page, slot = st["block_table"][b, t // 16], t % 16
            touched[page, slot] = True
            for planes, src in ((kp2, kn), (vp2, vn)):
                x = src[b, path[b, k]]  # [Hkv, D]
                dq = O.dequantize_nested({key: planes[key][page:page + 1, :, slot:slot + 1]
                                          for key in planes}, 8)[0, 0]
                s = np.abs(x).max(axis=1, keepdims=True) / 7
                assert np.all(np.abs(dq - x) <= s / 16 + 1e-6 * s)
    for old, new in ((kp, kp2), (vp, vp2)):
        keep = ~touched
        assert np.array_equal(old["scale"].transpose(0, 2, 1)[keep], new["scale"].transpose(0, 2, 1)[keep])
        assert np.array_equal(old["base"].transpose(0, 2, 1, 3)[keep], new["base"].transpose(0, 2, 1, 3)[keep])
