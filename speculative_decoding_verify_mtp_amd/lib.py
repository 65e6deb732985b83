"""Thin ctypes binding of libmtpverify.so (include/mtp_verify.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks their dtype / shape / contiguity, and passes raw
device pointers plus the current HIP stream to the C ABI.  All computation
happens in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmtpverify.so")

MTP_F32, MTP_BF16 = 0, 1
MASK_CHAIN, MASK_TREE, MASK_SEGMENT = 0, 1, 2
DEV_BAD_MASK, DEV_BAD_CTX, DEV_BAD_PAGE, DEV_BAD_ACCEPT = 1, 2, 4, 8
MTP_ERR_CONFLICT, MTP_ERR_SCRATCH = 6, 7

EXPORTS = ("mtp_abi_version", "mtp_status_string", "mtp_verify_attn_workspace_size",
           "mtp_verify_attn", "mtp_verify_attn_partial", "mtp_verify_attn_combine",
           "mtp_accept", "mtp_accept_hybrid", "mtp_kv_commit", "mtp_accept_commit",
           "mtp_verify_step", "mtp_kv_quantize", "mtp_kv_commit_nested",
           "mtp_verify_attn_nested_workspace_size", "mtp_verify_attn_nested",
           "mtp_verify_attn_nested_partial", "mtp_verify_attn_nested_combine",
           "mtp_build_tree", "mtp_build_tree_workspace_size", "mtp_block_positions",
           "mtp_check_commit_slots", "mtp_verify_step_noalloc", "mtp_get_device_status")
_ATTN_FN = {"both": "mtp_verify_attn", "partial": "mtp_verify_attn_partial",
            "combine": "mtp_verify_attn_combine"}
_NESTED_FN = {"both": "mtp_verify_attn_nested", "partial": "mtp_verify_attn_nested_partial",
              "combine": "mtp_verify_attn_nested_combine"}


class MtpError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: status {status} ({text})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("W", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("max_ctx_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("seg_lookback", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32)]


class NestedKVStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("k_base", "k_ref", "k_scale",
                                                "v_base", "v_ref", "v_scale")]


_lib = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Loads the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m speculative_decoding_verify_mtp_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sp = ctypes.POINTER(Shape)
    lib.mtp_abi_version.restype = _i32
    lib.mtp_abi_version.argtypes = []
    lib.mtp_status_string.restype = ctypes.c_char_p
    lib.mtp_status_string.argtypes = [_i32]
    lib.mtp_verify_attn_workspace_size.restype = _i32
    lib.mtp_verify_attn_workspace_size.argtypes = [sp, ctypes.POINTER(_sz)]
    for fn in _ATTN_FN.values():
        getattr(lib, fn).restype = _i32
        getattr(lib, fn).argtypes = [sp] + [_vp] * 11 + [_vp, _sz, _vp]
    lib.mtp_accept.restype = _i32
    lib.mtp_accept.argtypes = [sp, _vp, _i32] + [_vp] * 6 + [_vp]
    lib.mtp_accept_hybrid.restype = _i32
    lib.mtp_accept_hybrid.argtypes = ([sp, _vp, _vp, _i32] + [_vp] * 3
                                      + [ctypes.c_float, _i32] + [_vp] * 4 + [_vp])
    lib.mtp_kv_commit.restype = _i32
    lib.mtp_kv_commit.argtypes = [sp] + [_vp] * 7 + [_i32, _vp, _vp, _vp]
    lib.mtp_accept_commit.restype = _i32
    lib.mtp_accept_commit.argtypes = ([sp, _vp, _i32] + [_vp] * 6 + [_vp] * 5
                                      + [_i32, _vp, _vp, _vp])
    lib.mtp_verify_step.restype = _i32
    lib.mtp_verify_step.argtypes = ([sp] + [_vp] * 10 + [_i32] + [_vp] * 7 + [_i32, _vp, _sz, _vp])
    lib.mtp_verify_step_noalloc.restype = _i32
    lib.mtp_verify_step_noalloc.argtypes = [sp] + [_vp] * 10 + [_i32] + [_vp] * 7 + [_i32, _vp]
    npp = ctypes.POINTER(NestedKVStruct)
    lib.mtp_kv_quantize.restype = _i32
    lib.mtp_kv_quantize.argtypes = [sp, _vp, _vp, _i32, _vp, npp, _vp]
    lib.mtp_kv_commit_nested.restype = _i32
    lib.mtp_kv_commit_nested.argtypes = [sp] + [_vp] * 7 + [_i32, npp, _vp]
    lib.mtp_verify_attn_nested_workspace_size.restype = _i32
    lib.mtp_verify_attn_nested_workspace_size.argtypes = [sp, ctypes.POINTER(_sz)]
    for fn in _NESTED_FN.values():
        getattr(lib, fn).restype = _i32
        getattr(lib, fn).argtypes = [sp, _vp, npp] + [_vp] * 6 + [_i32, _vp, _vp, _vp, _sz, _vp]
    lib.mtp_build_tree.restype = _i32
    lib.mtp_build_tree.argtypes = [_i32] * 5 + [_vp, _vp, ctypes.c_float] + [_vp] * 5 + [_sz, _vp]
    lib.mtp_build_tree_workspace_size.restype = _i32
    lib.mtp_build_tree_workspace_size.argtypes = [_i32] * 5 + [ctypes.POINTER(_sz)]
    lib.mtp_block_positions.restype = _i32
    lib.mtp_block_positions.argtypes = [sp] + [_vp] * 4 + [_vp]
    lib.mtp_check_commit_slots.restype = _i32
    lib.mtp_check_commit_slots.argtypes = [sp, _vp, _vp, ctypes.POINTER(_i32)]
    lib.mtp_get_device_status.restype = _i32
    lib.mtp_get_device_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), _i32]
    if lib.mtp_abi_version() != 1:
        raise RuntimeError("libmtpverify ABI version mismatch")
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MtpError(fn, status, load().mtp_status_string(status).decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmtpverify must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MTP_F32
    if t.dtype == torch.bfloat16:
        return MTP_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


@dataclass
class VerifyShape:
    """Python mirror of mtp_shape."""

    B: int
    W: int
    Hq: int
    Hkv: int
    D: int
    num_pages: int
    max_pages_per_seq: int
    max_ctx_len: int
    dtype: int
    scale: float = 0.0
    seg_lookback: int = -1
    split_tokens: int = 0

    def c(self) -> Shape:
        return Shape(self.B, self.W, self.Hq, self.Hkv, self.D, 16, self.num_pages,
                     self.max_pages_per_seq, self.max_ctx_len, self.dtype, self.scale,
                     self.seg_lookback, self.split_tokens)


def shape_of(q: torch.Tensor, k_cache: torch.Tensor, block_table: torch.Tensor, *,
             max_ctx_len: int | None = None, scale: float = 0.0, seg_lookback: int = -1,
             split_tokens: int = 0) -> VerifyShape:
    B, W, Hq, D = q.shape
    num_pages, page, Hkv, D2 = k_cache.shape
    if page != 16 or D2 != D:
        raise ValueError("k_cache must be [num_pages, 16, Hkv, D]")
    maxp = block_table.shape[1]
    return VerifyShape(B, W, Hq, Hkv, D, num_pages, maxp,
                       maxp * 16 if max_ctx_len is None else int(max_ctx_len),
                       _dtype_code(q), float(scale), int(seg_lookback), int(split_tokens))


def workspace_bytes(shape: VerifyShape) -> int:
    n = ctypes.c_size_t(0)
    cs = shape.c()
    _check("mtp_verify_attn_workspace_size",
           load().mtp_verify_attn_workspace_size(ctypes.byref(cs), ctypes.byref(n)))
    return int(n.value)


def verify_attn(q, k_cache, v_cache, block_table, ctx_lens, k_new, v_new, mask_kind, mask_ids,
                *, out=None, lse=None, want_lse=True, workspace=None, shape=None,
                max_ctx_len=None, scale=0.0, seg_lookback=-1, split_tokens=0, stream=None,
                phase="both"):
    """Verify attention; returns (out [B,W,Hq,D] fp32, lse [B,W,Hq] fp32 or None).

    phase "partial" / "combine" launches only one of the two kernels (the
    combine must follow a partial launch on the same workspace)."""
    lib = load()
    if shape is None:
        shape = shape_of(q, k_cache, block_table, max_ctx_len=max_ctx_len, scale=scale,
                         seg_lookback=seg_lookback, split_tokens=split_tokens)
    B, W, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, W, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, W, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(shape), 16), dtype=torch.uint8,
                                device=q.device)
    for t in (block_table, ctx_lens, mask_ids):
        if t.dtype != torch.int32:
            raise ValueError("block_table, ctx_lens and mask_ids must be int32")
    if mask_kind.dtype != torch.uint8:
        raise ValueError("mask_kind must be uint8")
    cs = shape.c()
    fn = _ATTN_FN[phase]
    _check(fn, getattr(lib, fn)(
        ctypes.byref(cs), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(ctx_lens), _ptr(k_new), _ptr(v_new), _ptr(mask_kind), _ptr(mask_ids), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def _accept_shape(draft_ids: torch.Tensor) -> Shape:
    B, W = draft_ids.shape
    return Shape(B, W, 1, 1, 64, 16, 0, 0, 0, MTP_F32, 0.0, -1, 0)


def accept(logits, draft_ids, mask_kind, mask_ids, *, accept_len=None, accept_path=None,
           bonus_id=None, stream=None):
    """Greedy acceptance; returns (accept_len [B], accept_path [B,W], bonus_id [B]) int32."""
    lib = load()
    B, W, V = logits.shape
    dev = logits.device
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    accept_path = (torch.empty((B, W), dtype=torch.int32, device=dev) if accept_path is None
                   else accept_path)
    bonus_id = torch.empty(B, dtype=torch.int32, device=dev) if bonus_id is None else bonus_id
    cs = _accept_shape(draft_ids)
    _check("mtp_accept", lib.mtp_accept(
        ctypes.byref(cs), _ptr(logits), V, _ptr(draft_ids), _ptr(mask_kind), _ptr(mask_ids),
        _ptr(accept_len), _ptr(accept_path), _ptr(bonus_id), _stream(stream)))
    return accept_len, accept_path, bonus_id


def accept_hybrid(draft_logits, logits, draft_ids, mask_kind, mask_ids, tau, min_prefix, *,
                  accept_len=None, accept_path=None, bonus_id=None, conf_len=None, stream=None):
    """Confidence-threshold / hybrid acceptance; ``logits`` may be None.  Returns
    (accept_len [B], accept_path [B,W], bonus_id [B], conf_len [B]) int32."""
    lib = load()
    B, W, V = draft_logits.shape
    dev = draft_logits.device
    if logits is not None and tuple(logits.shape) != (B, W, V):
        raise ValueError("logits and draft_logits must have the same shape")
    new = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)  # noqa: E731
    accept_len = new(B) if accept_len is None else accept_len
    accept_path = new(B, W) if accept_path is None else accept_path
    bonus_id = new(B) if bonus_id is None else bonus_id
    conf_len = new(B) if conf_len is None else conf_len
    cs = _accept_shape(draft_ids)
    _check("mtp_accept_hybrid", lib.mtp_accept_hybrid(
        ctypes.byref(cs), _ptr(draft_logits), _ptr(logits), V, _ptr(draft_ids), _ptr(mask_kind),
        _ptr(mask_ids), float(tau), int(min_prefix), _ptr(accept_len), _ptr(accept_path),
        _ptr(bonus_id), _ptr(conf_len), _stream(stream)))
    return accept_len, accept_path, bonus_id, conf_len


def _commit_shape(k_new, k_cache, block_table) -> Shape:
    B, W, Hkv, D = k_new.shape
    maxp = block_table.shape[1]
    return Shape(B, W, Hkv, Hkv, D, 16, k_cache.shape[0], maxp, 0, _dtype_code(k_new), 0.0, -1, 0)


def kv_commit(k_new, v_new, accept_len, accept_path, block_table, ctx_lens_in, k_cache, v_cache,
              *, ctx_lens_out=None, skip_root=False, stream=None):
    """Writes the accepted rows into the cache (in place); returns ctx_lens_out."""
    lib = load()
    if ctx_lens_out is None:
        ctx_lens_out = torch.empty_like(ctx_lens_in)
    cs = _commit_shape(k_new, k_cache, block_table)
    _check("mtp_kv_commit", lib.mtp_kv_commit(
        ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _ptr(accept_len), _ptr(accept_path),
        _ptr(block_table), _ptr(ctx_lens_in), _ptr(ctx_lens_out), int(bool(skip_root)),
        _ptr(k_cache), _ptr(v_cache), _stream(stream)))
    return ctx_lens_out


def accept_commit(logits, draft_ids, mask_kind, mask_ids, k_new, v_new, block_table, ctx_lens_in,
                  k_cache, v_cache, *, accept_len=None, accept_path=None, bonus_id=None,
                  ctx_lens_out=None, skip_root=False, stream=None):
    """Fused acceptance + commit; returns (accept_len, accept_path, bonus_id, ctx_lens_out)."""
    lib = load()
    B, W, V = logits.shape
    dev = logits.device
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    accept_path = (torch.empty((B, W), dtype=torch.int32, device=dev) if accept_path is None
                   else accept_path)
    bonus_id = torch.empty(B, dtype=torch.int32, device=dev) if bonus_id is None else bonus_id
    if ctx_lens_out is None:
        ctx_lens_out = torch.empty_like(ctx_lens_in)
    cs = _commit_shape(k_new, k_cache, block_table)
    _check("mtp_accept_commit", lib.mtp_accept_commit(
        ctypes.byref(cs), _ptr(logits), V, _ptr(draft_ids), _ptr(mask_kind), _ptr(mask_ids),
        _ptr(accept_len), _ptr(accept_path), _ptr(bonus_id), _ptr(k_new), _ptr(v_new),
        _ptr(block_table), _ptr(ctx_lens_in), _ptr(ctx_lens_out), int(bool(skip_root)),
        _ptr(k_cache), _ptr(v_cache), _stream(stream)))
    return accept_len, accept_path, bonus_id, ctx_lens_out


def verify_step(q, k_cache, v_cache, block_table, ctx_lens_in, k_new, v_new, mask_kind, mask_ids,
                logits, draft_ids, *, out=None, lse=None, want_lse=True, accept_len=None,
                accept_path=None, bonus_id=None, ctx_lens_out=None, skip_root=False,
                workspace=None, shape=None, max_ctx_len=None, scale=0.0, seg_lookback=-1,
                split_tokens=0, stream=None, noalloc=False):
    """The whole verify step (attention, acceptance, commit) in two launches.

    noalloc=True calls mtp_verify_step_noalloc (the library's fixed device
    scratch instead of a workspace; `workspace` must then be None).
    Returns (out, lse, accept_len, accept_path, bonus_id, ctx_lens_out)."""
    lib = load()
    if shape is None:
        shape = shape_of(q, k_cache, block_table, max_ctx_len=max_ctx_len, scale=scale,
                         seg_lookback=seg_lookback, split_tokens=split_tokens)
    B, W, Hq, D = q.shape
    dev = q.device
    V = logits.shape[2]
    if out is None:
        out = torch.empty((B, W, Hq, D), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, W, Hq), dtype=torch.float32, device=dev)
    if noalloc and workspace is not None:
        raise ValueError("noalloc=True takes no workspace")
    if workspace is None and not noalloc:
        workspace = torch.empty(max(workspace_bytes(shape), 16), dtype=torch.uint8, device=dev)
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    accept_path = (torch.empty((B, W), dtype=torch.int32, device=dev) if accept_path is None
                   else accept_path)
    bonus_id = torch.empty(B, dtype=torch.int32, device=dev) if bonus_id is None else bonus_id
    if ctx_lens_out is None:
        ctx_lens_out = torch.empty_like(ctx_lens_in)
    cs = shape.c()
    args = (ctypes.byref(cs), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(ctx_lens_in), _ptr(k_new), _ptr(v_new), _ptr(mask_kind), _ptr(mask_ids),
            _ptr(logits), V, _ptr(draft_ids), _ptr(out), _ptr(lse), _ptr(accept_len),
            _ptr(accept_path), _ptr(bonus_id), _ptr(ctx_lens_out), int(bool(skip_root)))
    if noalloc:
        _check("mtp_verify_step_noalloc", lib.mtp_verify_step_noalloc(*args, _stream(stream)))
    else:
        _check("mtp_verify_step", lib.mtp_verify_step(*args, _ptr(workspace), workspace.numel(),
                                                      _stream(stream)))
    return out, lse, accept_len, accept_path, bonus_id, ctx_lens_out


def check_commit_slots(block_table, ctx_lens, W: int, num_pages: int) -> int:
    """Host-side ownership check of the commit slots (mtp_check_commit_slots)
    on host arrays (numpy or CPU tensors).  Returns the smallest sequence
    index involved in a conflict, or -1 when every commit slot is its
    sequence's own."""
    import numpy as np

    bt = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    ctx = np.ascontiguousarray(np.asarray(ctx_lens), dtype=np.int32)
    if bt.ndim != 2 or ctx.shape != (bt.shape[0],):
        raise ValueError("block_table must be [B, max_pages] and ctx_lens [B]")
    cs = Shape(bt.shape[0], W, 1, 1, 64, 16, num_pages, bt.shape[1], 0, MTP_F32, 0.0, -1, 0)
    bad = ctypes.c_int32(-2)
    st = load().mtp_check_commit_slots(ctypes.byref(cs), bt.ctypes.data, ctx.ctypes.data,
                                       ctypes.byref(bad))
    if st not in (0, MTP_ERR_CONFLICT):
        _check("mtp_check_commit_slots", st)
    return int(bad.value)


def device_status(clear: bool = True) -> int:
    """Sticky device status bits (MTP_DEV_*); synchronises the device."""
    v = ctypes.c_uint32(0)
    _check("mtp_get_device_status", load().mtp_get_device_status(ctypes.byref(v), int(clear)))
    return int(v.value)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


# ----------------------------------------------------------------------------
# nested KV4 / KV8 cache
# ----------------------------------------------------------------------------

class NestedKV:
    """The six planes of a nested cache as torch tensors (allocation only):
    base / ref [num_pages, Hkv, 16, D/2] uint8 and scale [num_pages, Hkv, 16]
    fp32, for K and for V."""

    def __init__(self, num_pages: int, Hkv: int, D: int, device="cuda", with_ref: bool = True):
        def codes():
            return torch.zeros((num_pages, Hkv, 16, D // 2), dtype=torch.uint8, device=device)
        self.num_pages, self.Hkv, self.D = num_pages, Hkv, D
        self.k_base, self.v_base = codes(), codes()
        self.k_ref = codes() if with_ref else None
        self.v_ref = codes() if with_ref else None
        self.k_scale = torch.zeros((num_pages, Hkv, 16), dtype=torch.float32, device=device)
        self.v_scale = torch.zeros((num_pages, Hkv, 16), dtype=torch.float32, device=device)

    def c(self) -> NestedKVStruct:
        return NestedKVStruct(*(_ptr(t) for t in (self.k_base, self.k_ref, self.k_scale,
                                                    self.v_base, self.v_ref, self.v_scale)))

    def planes(self, which: str) -> dict:
        """Host numpy copies of the K ("k") or V ("v") planes."""
        return {"base": getattr(self, which + "_base").cpu().numpy(),
                "ref": getattr(self, which + "_ref").cpu().numpy(),
                "scale": getattr(self, which + "_scale").cpu().numpy()}


def kv_quantize(k_rows, v_rows, slots, kv: NestedKV, *, stream=None):
    """Quantizes rows [n, Hkv, D] (fp32 or bf16) into slots [n] (page * 16 + slot)."""
    lib = load()
    n, Hkv, D = k_rows.shape
    cs = Shape(0, 1, Hkv, Hkv, D, 16, kv.num_pages, 0, 0, _dtype_code(k_rows), 0.0, -1, 0)
    ckv = kv.c()
    _check("mtp_kv_quantize", lib.mtp_kv_quantize(
        ctypes.byref(cs), _ptr(k_rows), _ptr(v_rows), n, _ptr(slots), ctypes.byref(ckv),
        _stream(stream)))


def kv_quantize_cache(k_cache, v_cache, kv: NestedKV, *, stream=None):
    """Quantizes every slot of a [pages, 16, Hkv, D] cache (prefill helper)."""
    pages, _, Hkv, D = k_cache.shape
    slots = torch.arange(pages * 16, dtype=torch.int32, device=k_cache.device)
    kv_quantize(k_cache.reshape(pages * 16, Hkv, D), v_cache.reshape(pages * 16, Hkv, D), slots,
                kv, stream=stream)


def kv_commit_nested(k_new, v_new, accept_len, accept_path, block_table, ctx_lens_in,
                     kv: NestedKV, *, ctx_lens_out=None, skip_root=False, stream=None):
    """Quantizing commit into a nested cache; returns ctx_lens_out."""
    lib = load()
    if ctx_lens_out is None:
        ctx_lens_out = torch.empty_like(ctx_lens_in)
    B, W, Hkv, D = k_new.shape
    cs = Shape(B, W, Hkv, Hkv, D, 16, kv.num_pages, block_table.shape[1], 0, _dtype_code(k_new),
               0.0, -1, 0)
    ckv = kv.c()
    _check("mtp_kv_commit_nested", lib.mtp_kv_commit_nested(
        ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _ptr(accept_len), _ptr(accept_path),
        _ptr(block_table), _ptr(ctx_lens_in), _ptr(ctx_lens_out), int(bool(skip_root)),
        ctypes.byref(ckv), _stream(stream)))
    return ctx_lens_out


def nested_workspace_bytes(shape: VerifyShape) -> int:
    n = ctypes.c_size_t(0)
    cs = shape.c()
    _check("mtp_verify_attn_nested_workspace_size",
           load().mtp_verify_attn_nested_workspace_size(ctypes.byref(cs), ctypes.byref(n)))
    return int(n.value)


def verify_attn_nested(q, kv: NestedKV, block_table, ctx_lens, k_new, v_new, mask_kind, mask_ids,
                       *, kv8_recent=-1, out=None, lse=None, want_lse=True, workspace=None,
                       shape=None, max_ctx_len=None, scale=0.0, seg_lookback=-1, split_tokens=0,
                       stream=None, phase="both"):
    """Verify attention over a nested cache; returns (out, lse).  phase
    "partial" / "combine" launches only one of the two kernels."""
    lib = load()
    B, W, Hq, D = q.shape
    if shape is None:
        maxp = block_table.shape[1]
        shape = VerifyShape(B, W, Hq, kv.Hkv, D, kv.num_pages, maxp,
                            maxp * 16 if max_ctx_len is None else int(max_ctx_len),
                            _dtype_code(q), float(scale), int(seg_lookback), int(split_tokens))
    if out is None:
        out = torch.empty((B, W, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, W, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(nested_workspace_bytes(shape), 16), dtype=torch.uint8,
                                device=q.device)
    cs = shape.c()
    ckv = kv.c()
    fn = _NESTED_FN[phase]
    _check(fn, getattr(lib, fn)(
        ctypes.byref(cs), _ptr(q), ctypes.byref(ckv), _ptr(block_table), _ptr(ctx_lens),
        _ptr(k_new), _ptr(v_new), _ptr(mask_kind), _ptr(mask_ids), int(kv8_recent), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def build_tree(probs, root_token, W, n_mask, min_cum_prob=0.0, *, workspace=None, out=None,
               stream=None):
    """Dynamic token tree; returns (draft_ids, parents, depth [B, W], n_nodes [B]) int32."""
    lib = load()
    B, K, V = probs.shape
    dev = probs.device
    if out is None:
        out = (torch.empty((B, W), dtype=torch.int32, device=dev),
               torch.empty((B, W), dtype=torch.int32, device=dev),
               torch.empty((B, W), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    draft, parents, depth, n_nodes = out
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check("mtp_build_tree_workspace_size",
               lib.mtp_build_tree_workspace_size(B, K, V, W, n_mask, ctypes.byref(n)))
        workspace = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=dev)
    _check("mtp_build_tree", lib.mtp_build_tree(
        B, K, V, W, n_mask, _ptr(probs), _ptr(root_token), float(min_cum_prob), _ptr(draft),
        _ptr(parents), _ptr(depth), _ptr(n_nodes), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return draft, parents, depth, n_nodes


def block_positions(ctx_lens, mask_kind, mask_ids, *, positions=None, stream=None):
    """Positions [B, W] int32 of the block rows (ctx_lens + depth)."""
    lib = load()
    B, W = mask_ids.shape
    if positions is None:
        positions = torch.empty((B, W), dtype=torch.int32, device=mask_ids.device)
    cs = Shape(B, W, 1, 1, 64, 16, 0, 0, 0, MTP_F32, 0.0, -1, 0)
    _check("mtp_block_positions", lib.mtp_block_positions(
        ctypes.byref(cs), _ptr(ctx_lens), _ptr(mask_kind), _ptr(mask_ids),
        _ptr(positions), _stream(stream)))
    return positions
