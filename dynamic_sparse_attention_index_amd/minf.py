"""Python binding of libminf.so: argument marshalling only.

Each function has the name of the C entry point it calls. Tensors are torch
tensors on the GPU (bf16 for Q/K/V/O, int32 for indices); outputs and
workspaces are allocated with torch (device memory plumbing) unless the
caller passes them in. Every step of the computation runs in the library's
HIP kernels; there is no fallback path. Importing this module raises if the
library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libminf.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "minf.h")

MINF_OK = 0
KIND = {"dense": 0, "ashape": 1, "vs": 2, "block": 3, "vs_window": 4}


class MinfError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class HeadPlan(ctypes.Structure):
    """Mirror of minf_head_plan."""
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("sink", ctypes.c_int32),
        ("local", ctypes.c_int32),
        ("k_v", ctypes.c_int32),
        ("k_s", ctypes.c_int32),
        ("k_b", ctypes.c_int32),
        ("v_idx", ctypes.c_void_p),
        ("s_idx", ctypes.c_void_p),
        ("blk_idx", ctypes.c_void_p),
        ("blk_cnt", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m dynamic_sparse_attention_index_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    ip = ctypes.POINTER(ctypes.c_int32)
    sigs = {
        "minf_status_string": (ctypes.c_char_p, [i32]),
        "minf_last_error_detail": (ctypes.c_char_p, []),
        "minf_abi_version": (i32, []),
        "minf_vs_index_workspace_size": (sz, [i64, i32]),
        "minf_build_vs_index": (i32, [vp, vp, i64, i32, i32, i32, ip, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp]),
        "minf_vs_scores": (i32, [vp, vp, i64, i32, i32, i32, ip, i32, i32, f32, vp, vp, vp, sz, vp]),
        "minf_block_index_workspace_size": (sz, [i64, i32, i32, i32]),
        "minf_build_block_index": (i32, [vp, vp, i64, i32, i32, i32, ip, i32, i32, vp, vp, vp, sz, vp]),
        "minf_block_pool": (i32, [vp, i64, i32, i32, ip, i32, vp, vp]),
        "minf_sparse_attn_workspace_size": (sz, [i64, i32]),
        "minf_sparse_attn": (i32, [vp, vp, vp, vp, vp, i64, i32, i32, i32, f32, ctypes.POINTER(HeadPlan), vp, sz, vp]),
        "minf_dense_attn": (i32, [vp, vp, vp, vp, vp, i64, i32, i32, i32, f32, i32, vp]),
        "minf_build_permuted_block_index": (i32, [vp, vp, i64, i32, i32, i32, ip, i32, i32, vp, vp, vp, vp, sz, vp]),
        "minf_permute_rows": (i32, [vp, vp, i32, i64, i32, vp, i32, vp]),
        "minf_decode_pool_keys": (i32, [vp, i64, i32, i32, i32, vp, vp]),
        "minf_decode_workspace_size": (sz, [i64, i32, i32]),
        "minf_sparse_decode": (i32, [vp, vp, vp, vp, i64, i32, i32, i32, f32, i32, vp, vp, vp, vp, sz, vp]),
        "minf_dense_decode": (i32, [vp, vp, vp, i64, i32, i32, i32, f32, vp, vp, vp, sz, vp]),
        "minf_plan_work": (i32, [ctypes.POINTER(HeadPlan), i64, i32, vp, vp, sz, vp]),
        "minf_attention_recall": (i32, [vp, vp, i64, i32, vp, i32, vp, vp]),
        "minf_decode_noalloc_max_bytes": (sz, []),
        "minf_sparse_decode_noalloc": (i32, [vp, vp, vp, vp, i64, i32, i32, i32, f32, i32, vp, vp, vp, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def header_functions() -> list:
    """Names of the functions include/minf.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(minf_[a-z_0-9]+)\s*\(", text)) - {"minf_head_plan"})


def library():
    return _lib


def _check(status: int):
    if status != MINF_OK:
        name = _lib.minf_status_string(status).decode()
        detail = _lib.minf_last_error_detail().decode()
        raise MinfError(status, name, detail)


def _stream_of(stream=None):
    """The stream the call is enqueued on (torch's current stream by default)."""
    return torch.cuda.current_stream() if stream is None else stream


def _stream(s):
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name, shape=None, device=None):
    """t must be a contiguous GPU tensor of `dtype` (and of `shape` / on `device` when given)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on the GPU")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")


def _empty(shape, dtype, device, s):
    """A new tensor whose memory the caching allocator ties to stream s, the stream the
    library's kernels use it on (so it is not handed out again before they finish)."""
    with torch.cuda.stream(s):
        return torch.empty(shape, dtype=dtype, device=device)


def _qkv(q, k, v=None):
    """Shapes of Q [hq, n, d] and K (and V) [hkv, n, d], all bf16 on one device."""
    _need(q, torch.bfloat16, "q")
    if q.dim() != 3:
        raise ValueError(f"q must be [hq, n, d] (got {tuple(q.shape)})")
    hq, n, d = q.shape
    _need(k, torch.bfloat16, "k", device=q.device)
    if k.dim() != 3 or k.shape[1] != n or k.shape[2] != d:
        raise ValueError(f"k must be [hkv, {n}, {d}] (got {tuple(k.shape)})")
    if v is not None:
        _need(v, torch.bfloat16, "v", shape=tuple(k.shape), device=q.device)
    return hq, n, d, k.shape[0]


def _heads_arr(heads):
    heads = [int(h) for h in heads]
    arr = (ctypes.c_int32 * max(1, len(heads)))(*heads)
    return arr, len(heads)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _need_out(t, shape, name, device=None):
    _need(t, torch.int32, name, shape=shape, device=device)


def _workspace(nbytes, device, workspace, s):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        if workspace.device != device:
            raise ValueError(f"workspace must be on {device} (got {workspace.device})")
        return workspace, workspace.numel() * workspace.element_size()
    return _empty((nbytes,), torch.uint8, device, s), nbytes


def minf_build_vs_index(q, k, heads, last_q=64, k_v=1000, k_s=6096, scale=None, workspace=None, stream=None,
                        out=None):
    """VS index for query heads `heads`: (v_idx [n_heads, min(k_v, n)], s_idx [n_heads, min(k_s, n)]).

    out: optional preallocated (v_idx, s_idx) of those shapes, contiguous int32.
    """
    hq, n, d, hkv = _qkv(q, k)
    s = _stream_of(stream)
    arr, nh = _heads_arr(heads)
    kv_eff, ks_eff = min(k_v, n), min(k_s, n)
    if out is None:
        v_idx = _empty((nh, kv_eff), torch.int32, q.device, s)
        s_idx = _empty((nh, ks_eff), torch.int32, q.device, s)
    else:
        v_idx, s_idx = out
        _need_out(v_idx, (nh, kv_eff), "v_idx", q.device)
        _need_out(s_idx, (nh, ks_eff), "s_idx", q.device)
    ws, wsb = _workspace(_lib.minf_vs_index_workspace_size(n, nh), q.device, workspace, s)
    _check(_lib.minf_build_vs_index(_ptr(q), _ptr(k), n, hq, hkv, d, arr, nh, last_q, k_v, k_s, _scale(scale, d),
                                    _ptr(v_idx), _ptr(s_idx), _ptr(ws), wsb, _stream(s)))
    return v_idx, s_idx


def minf_vs_scores(q, k, heads, last_q=64, scale=None, workspace=None, stream=None):
    """Column sums and diagonal sums of the last-query softmax: (v [n_heads, n], sl [n_heads, n])."""
    hq, n, d, hkv = _qkv(q, k)
    s = _stream_of(stream)
    arr, nh = _heads_arr(heads)
    v = _empty((nh, n), torch.float32, q.device, s)
    sl = _empty((nh, n), torch.float32, q.device, s)
    ws, wsb = _workspace(_lib.minf_vs_index_workspace_size(n, nh), q.device, workspace, s)
    _check(_lib.minf_vs_scores(_ptr(q), _ptr(k), n, hq, hkv, d, arr, nh, last_q, _scale(scale, d), _ptr(v), _ptr(sl),
                               _ptr(ws), wsb, _stream(s)))
    return v, sl


def _block_outputs(out, nh, nb, k_b, device, s):
    if out is None:
        return _empty((nh, nb, k_b), torch.int32, device, s), _empty((nh, nb), torch.int32, device, s)
    bi, bc = out
    _need_out(bi, (nh, nb, k_b), "blk_idx", device)
    _need_out(bc, (nh, nb), "blk_cnt", device)
    return bi, bc


def minf_build_block_index(q, k, heads, k_b=256, workspace=None, stream=None, out=None):
    """Block index: (blk_idx [n_heads, n_b, k_b] padded with -1, blk_cnt [n_heads, n_b]).

    out: optional preallocated (blk_idx, blk_cnt) of those shapes, contiguous int32.
    """
    hq, n, d, hkv = _qkv(q, k)
    s = _stream_of(stream)
    arr, nh = _heads_arr(heads)
    nb = (n + 63) // 64
    blk_idx, blk_cnt = _block_outputs(out, nh, nb, int(k_b), q.device, s)
    ws, wsb = _workspace(_lib.minf_block_index_workspace_size(n, hq, hkv, nh), q.device, workspace, s)
    _check(_lib.minf_build_block_index(_ptr(q), _ptr(k), n, hq, hkv, d, arr, nh, int(k_b), _ptr(blk_idx),
                                       _ptr(blk_cnt), _ptr(ws), wsb, _stream(s)))
    return blk_idx, blk_cnt


def minf_build_permuted_block_index(q, k, heads, pos, k_b=256, workspace=None, stream=None, out=None):
    """Block index of a permuted sequence (q, k in permuted order, pos[t] = original position of row t).

    Returns (blk_idx [n_heads, n_b, k_b] int32, blk_cnt [n_heads, n_b] int32); out: optional
    preallocated pair of those shapes.
    """
    hq, n, d, hkv = _qkv(q, k)
    _need(pos, torch.int32, "pos", shape=(n,), device=q.device)
    s = _stream_of(stream)
    arr, nh = _heads_arr(heads)
    nb = (n + 63) // 64
    bi, bc = _block_outputs(out, nh, nb, int(k_b), q.device, s)
    ws, wsb = _workspace(_lib.minf_block_index_workspace_size(n, hq, hkv, nh), q.device, workspace, s)
    _check(_lib.minf_build_permuted_block_index(_ptr(q), _ptr(k), n, hq, hkv, d, arr, nh, int(k_b), _ptr(pos),
                                                _ptr(bi), _ptr(bc), _ptr(ws), wsb, _stream(s)))
    return bi, bc


def minf_permute_rows(x, src, scatter=False, out=None, stream=None):
    """Rows of x [h, n, ...] (contiguous) permuted by src: gather out[:, t] = x[:, src[t]], or scatter
    out[:, src[t]] = x[:, t]."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda or not x.is_contiguous() or x.dim() < 2:
        raise ValueError("x must be a contiguous GPU tensor [h, n, ...]")
    h, n = x.shape[0], x.shape[1]
    _need(src, torch.int32, "src", shape=(n,), device=x.device)
    s = _stream_of(stream)
    row_bytes = x[0, 0].numel() * x.element_size()
    if out is None:
        out = _empty(tuple(x.shape), x.dtype, x.device, s)
    else:
        _need(out, x.dtype, "out", shape=tuple(x.shape), device=x.device)
    _check(_lib.minf_permute_rows(_ptr(x), _ptr(out), h, n, row_bytes, _ptr(src), 1 if scatter else 0, _stream(s)))
    return out


def minf_block_pool(x, heads, stream=None):
    """64-row block means of x [h, n, d] for the listed heads: [n_heads, n_b, d] float32."""
    _need(x, torch.bfloat16, "x")
    if x.dim() != 3:
        raise ValueError(f"x must be [h, n, d] (got {tuple(x.shape)})")
    h, n, d = x.shape
    s = _stream_of(stream)
    arr, nh = _heads_arr(heads)
    out = _empty((nh, (n + 63) // 64, d), torch.float32, x.device, s)
    _check(_lib.minf_block_pool(_ptr(x), n, h, d, arr, nh, _ptr(out), _stream(s)))
    return out


def make_plans(plans, n=None, device=None):
    """Convert per-head plan dicts into the C struct array (keeps tensor references alive).

    With n (the sequence length) the index tensors' shapes are checked against it: v_idx and
    s_idx 1-D, blk_idx [n_b, k_b], blk_cnt [n_b], pos [n]; with device, their device too.
    """
    arr = (HeadPlan * len(plans))()
    keep = []
    nb = None if n is None else (int(n) + 63) // 64
    for h, p in enumerate(plans):
        kind = p["kind"]
        e = arr[h]
        if kind not in KIND:
            raise ValueError(f"unknown plan kind {kind!r}")
        e.kind = KIND[kind]
        if kind == "ashape":
            e.sink, e.local = int(p["sink"]), int(p["local"])
        elif kind in ("vs", "vs_window"):
            vi, si = p["v_idx"], p["s_idx"]
            for t, nm in ((vi, "v_idx"), (si, "s_idx")):
                _need(t, torch.int32, f"head {h} {nm}", device=device)
                if t.dim() != 1:
                    raise ValueError(f"head {h} {nm} must be 1-D (got {tuple(t.shape)})")
            e.k_v, e.k_s = vi.numel(), si.numel()
            e.v_idx, e.s_idx = vi.data_ptr(), si.data_ptr()
            keep += [vi, si]
        elif kind == "block":
            bi, bc = p["blk_idx"], p["blk_cnt"]
            _need(bi, torch.int32, f"head {h} blk_idx", device=device)
            if bi.dim() != 2 or (nb is not None and bi.shape[0] != nb):
                raise ValueError(f"head {h} blk_idx must be [n_b, k_b] (got {tuple(bi.shape)})")
            _need(bc, torch.int32, f"head {h} blk_cnt", shape=(bi.shape[0],), device=device)
            e.k_b = bi.shape[-1]
            e.blk_idx, e.blk_cnt = bi.data_ptr(), bc.data_ptr()
            keep += [bi, bc]
            if p.get("pos") is not None:
                _need(p["pos"], torch.int32, f"head {h} pos", shape=None if n is None else (int(n),), device=device)
                e.pos = p["pos"].data_ptr()
                keep.append(p["pos"])
    return arr, keep


def _attn_outputs(q, out, lse, with_lse, s):
    hq, n, _ = q.shape
    if out is None:
        o = _empty(tuple(q.shape), torch.bfloat16, q.device, s)
    else:
        _need(out, torch.bfloat16, "out", shape=tuple(q.shape), device=q.device)
        o = out
    if lse is None and with_lse:
        lse = _empty((hq, n), torch.float32, q.device, s)
    elif lse is not None:
        _need(lse, torch.float32, "lse", shape=(hq, n), device=q.device)
    return o, lse


def minf_sparse_attn(q, k, v, plans, scale=None, out=None, lse=None, with_lse=True, workspace=None, stream=None):
    """Sparse attention over per-head plans: (o [hq, n, d] bf16, lse [hq, n] float32 or None).

    plans: a list of per-head plan dicts (checked against q's length and device), or the
    (array, keep) pair that make_plans returned.
    """
    hq, n, d, hkv = _qkv(q, k, v)
    s = _stream_of(stream)
    arr, keep = plans if isinstance(plans, tuple) else make_plans(plans, n=n, device=q.device)
    if len(arr) != hq:
        raise ValueError("one plan per query head is required")
    o, lse = _attn_outputs(q, out, lse, with_lse, s)
    ws, wsb = _workspace(_lib.minf_sparse_attn_workspace_size(n, hq), q.device, workspace, s)
    _check(_lib.minf_sparse_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), n, hq, hkv, d, _scale(scale, d), arr,
                                 _ptr(ws), wsb, _stream(s)))
    del keep
    return o, lse


def minf_dense_attn(q, k, v, scale=None, causal=True, out=None, lse=None, with_lse=True, stream=None):
    """Dense FlashAttention baseline: (o [hq, n, d] bf16, lse [hq, n] float32 or None)."""
    hq, n, d, hkv = _qkv(q, k, v)
    s = _stream_of(stream)
    o, lse = _attn_outputs(q, out, lse, with_lse, s)
    _check(_lib.minf_dense_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), n, hq, hkv, d, _scale(scale, d),
                                1 if causal else 0, _stream(s)))
    return o, lse


def minf_decode_pool_keys(k, first_block=0, out=None, stream=None):
    """Block means of K for decoding: float32 [hkv, d, n_b] (blocks >= first_block recomputed)."""
    _need(k, torch.bfloat16, "k")
    if k.dim() != 3:
        raise ValueError(f"k must be [hkv, n, d] (got {tuple(k.shape)})")
    hkv, n, d = k.shape
    s = _stream_of(stream)
    nb = (n + 63) // 64
    if out is None:
        kbar_t = _empty((hkv, d, nb), torch.float32, k.device, s)
    else:
        _need(out, torch.float32, "out", shape=(hkv, d, nb), device=k.device)
        kbar_t = out
    _check(_lib.minf_decode_pool_keys(_ptr(k), n, hkv, d, int(first_block), _ptr(kbar_t), _stream(s)))
    return kbar_t


def _decode_args(q, k, v):
    _need(q, torch.bfloat16, "q")
    if q.dim() != 2:
        raise ValueError(f"q must be [hq, d] (got {tuple(q.shape)})")
    hq, d = q.shape
    _need(k, torch.bfloat16, "k", device=q.device)
    if k.dim() != 3 or k.shape[2] != d:
        raise ValueError(f"k must be [hkv, n, {d}] (got {tuple(k.shape)})")
    _need(v, torch.bfloat16, "v", shape=tuple(k.shape), device=q.device)
    return hq, d, k.shape[0], k.shape[1]


def _decode_outputs(q, out, lse, s):
    hq = q.shape[0]
    if out is None:
        out = _empty(tuple(q.shape), torch.bfloat16, q.device, s)
    else:
        _need(out, torch.bfloat16, "out", shape=tuple(q.shape), device=q.device)
    if lse is None:
        lse = _empty((hq,), torch.float32, q.device, s)
    else:
        _need(lse, torch.float32, "lse", shape=(hq,), device=q.device)
    return out, lse


def minf_sparse_decode(q, k, v, kbar_t, k_b, scale=None, out=None, lse=None, blk_idx=None, with_index=True,
                       workspace=None, stream=None):
    """One decode step: q [hq, d] against the cache k/v [hkv, n, d].

    Returns (o [hq, d] bf16, lse [hq] float32, blk_idx [hq, min(k_b, n_b)] int32 or None).
    """
    hq, d, hkv, n = _decode_args(q, k, v)
    s = _stream_of(stream)
    nb = (n + 63) // 64
    kk = min(int(k_b), nb)
    if kbar_t is not None:
        _need(kbar_t, torch.float32, "kbar_t", shape=(hkv, d, nb), device=q.device)
    o, lse = _decode_outputs(q, out, lse, s)
    if blk_idx is None and with_index:
        blk_idx = _empty((hq, kk), torch.int32, q.device, s)
    elif blk_idx is not None:
        _need_out(blk_idx, (hq, kk), "blk_idx", q.device)
    ws, wsb = _workspace(_lib.minf_decode_workspace_size(n, hq, int(k_b)), q.device, workspace, s)
    _check(_lib.minf_sparse_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(kbar_t), n, hq, hkv, d, _scale(scale, d),
                                   int(k_b), _ptr(blk_idx), _ptr(o), _ptr(lse), _ptr(ws), wsb, _stream(s)))
    return o, lse, blk_idx


def minf_dense_decode(q, k, v, scale=None, out=None, lse=None, workspace=None, stream=None):
    """Dense decoding baseline: (o [hq, d] bf16, lse [hq] float32)."""
    hq, d, hkv, n = _decode_args(q, k, v)
    s = _stream_of(stream)
    o, lse = _decode_outputs(q, out, lse, s)
    ws, wsb = _workspace(_lib.minf_decode_workspace_size(n, hq, (n + 63) // 64), q.device, workspace, s)
    _check(_lib.minf_dense_decode(_ptr(q), _ptr(k), _ptr(v), n, hq, hkv, d, _scale(scale, d), _ptr(o), _ptr(lse),
                                  _ptr(ws), wsb, _stream(s)))
    return o, lse


def minf_plan_work(plans, n, workspace=None, stream=None):
    """Work of each head's plan in the sparse kernel's unit (64x64 blocks, gathered columns at
    1/64): float64 [hq] on the plans' device. plans: per-head plan dicts (as for
    minf_sparse_attn) or the pair make_plans returned; n: the sequence length."""
    if isinstance(plans, tuple):
        arr, keep = plans
        device = torch.device("cuda", torch.cuda.current_device())
    else:
        device = next((t.device for p in plans for t in p.values() if isinstance(t, torch.Tensor)),
                      torch.device("cuda", torch.cuda.current_device()))
        arr, keep = make_plans(plans, n=n, device=device)
    hq = len(arr)
    s = _stream_of(stream)
    work = _empty((hq,), torch.float64, device, s)
    ws, wsb = _workspace(_lib.minf_sparse_attn_workspace_size(int(n), hq), device, workspace, s)
    _check(_lib.minf_plan_work(arr, int(n), hq, _ptr(work), _ptr(ws), wsb, _stream(s)))
    del keep
    return work


def minf_attention_recall(lse_mask, lse_dense, rows=None, stream=None):
    """Mean over rows of exp(lse_mask - lse_dense) per head (0 for an empty mask row):
    float64 [hq]. lse_mask, lse_dense: float32 [hq, n]; rows: int32 row ids or None (all)."""
    _need(lse_mask, torch.float32, "lse_mask")
    if lse_mask.dim() != 2:
        raise ValueError(f"lse_mask must be [hq, n] (got {tuple(lse_mask.shape)})")
    hq, n = lse_mask.shape
    _need(lse_dense, torch.float32, "lse_dense", shape=(hq, n), device=lse_mask.device)
    nr = n
    if rows is not None:
        _need(rows, torch.int32, "rows", device=lse_mask.device)
        if rows.dim() != 1 or rows.numel() < 1:
            raise ValueError("rows must be a non-empty 1-D int32 tensor")
        nr = rows.numel()
    s = _stream_of(stream)
    out = _empty((hq,), torch.float64, lse_mask.device, s)
    _check(_lib.minf_attention_recall(_ptr(lse_mask), _ptr(lse_dense), n, hq, _ptr(rows), nr, _ptr(out), _stream(s)))
    return out


def minf_sparse_decode_noalloc(q, k, v, kbar_t, k_b, out, lse, blk_idx=None, scale=None, stream=None):
    """minf_sparse_decode with the library's static scratch: no allocation by the library or here.

    out [hq, d] bf16, lse [hq] float32 and the optional blk_idx [hq, min(k_b, n_b)] int32 are the
    caller's (preallocated) tensors; returns (out, lse, blk_idx).
    """
    hq, d, hkv, n = _decode_args(q, k, v)
    s = _stream_of(stream)
    nb = (n + 63) // 64
    if kbar_t is not None:
        _need(kbar_t, torch.float32, "kbar_t", shape=(hkv, d, nb), device=q.device)
    _need(out, torch.bfloat16, "out", shape=tuple(q.shape), device=q.device)
    _need(lse, torch.float32, "lse", shape=(hq,), device=q.device)
    if blk_idx is not None:
        _need_out(blk_idx, (hq, min(int(k_b), nb)), "blk_idx", q.device)
    _check(_lib.minf_sparse_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(kbar_t), n, hq, hkv, d, _scale(scale, d),
                                           int(k_b), _ptr(blk_idx), _ptr(out), _ptr(lse), _stream(s)))
    return out, lse, blk_idx
