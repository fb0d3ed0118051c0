"""ctypes binding of ``libattn_mi355x.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors into pointers, strides and sizes, allocates outputs
through torch, passes torch's current stream, and raises on a negative
status.  There is no fallback: if the library is missing, the first call
raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# Another build of the same library (for instance the host-sanitized one of
# build.build_sanitized) can be named by ATTN_MI355X_LIBRARY.
LIB_PATH = os.environ.get("ATTN_MI355X_LIBRARY") or os.path.join(_HERE, "libattn_mi355x.so")

ATTN_F32, ATTN_BF16 = 0, 1
ATTN_E_HIP = -7
_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}

EXPORTED = ("attn_params_sizeof", "attn_abi_version", "attn_strerror", "attn_fwd",
            "attn_decode_workspace_bytes", "attn_decode_splitkv", "attn_decode_splitkv_noalloc",
            "attn_merge_states", "attn_bwd_workspace_bytes", "attn_bwd")
DECODE_SCRATCH_BYTES = 32 << 20   # ATTN_DECODE_SCRATCH_BYTES


class Params(ctypes.Structure):
    """Mirror of attn_params_t (field order and types as in the header)."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads_q", ctypes.c_int64), ("heads_kv", ctypes.c_int64),
        ("t_q", ctypes.c_int64), ("t_k", ctypes.c_int64), ("d_h", ctypes.c_int64),
        ("d_v", ctypes.c_int64), ("q_offset", ctypes.c_int64),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("bias_stride", ctypes.c_int64 * 4), ("bias", ctypes.c_void_p),
        ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("n_seqs", ctypes.c_int64), ("max_seqlen_q", ctypes.c_int64),
        ("seqlens_k", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: Optional[str] = None):
    """Load the HIP library (once) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP attention library not built: {p} is missing "
                           "(run __graft_entry__.build() or python -m online_softmax_exact_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    pp = ctypes.POINTER(Params)
    lib.attn_params_sizeof.restype = sz
    lib.attn_params_sizeof.argtypes = []
    lib.attn_abi_version.restype = ctypes.c_int
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode_workspace_bytes.argtypes = [pp, i64]
    lib.attn_decode_splitkv.restype = ctypes.c_int
    lib.attn_decode_splitkv.argtypes = [pp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_decode_splitkv_noalloc.restype = ctypes.c_int
    lib.attn_decode_splitkv_noalloc.argtypes = [pp, i64, vp, vp, vp, vp, vp, vp]
    lib.attn_merge_states.restype = ctypes.c_int
    lib.attn_merge_states.argtypes = [i64, i64, i64, vp, i64, i64, vp, i64, i64,
                                      ctypes.c_int32, vp, i64, vp, vp]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [pp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    if lib.attn_params_sizeof() != ctypes.sizeof(Params):
        raise RuntimeError("attn_params_t layout mismatch between header and binding")
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().attn_strerror(status).decode()


def _check(status: int):
    if status == 0:
        return
    msg = strerror(status)
    if status == ATTN_E_HIP:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _outer_strides(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, T, D]")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous innermost dimension")
    return tuple(int(x) for x in t.stride()[:3])


def _same_device(device, **tensors):
    """Every named tensor (None skipped) lives on ``device``."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, not on {device} with the other operands")


def _require_gpu(q, **tensors):
    """The kernels read and write device memory: q must be a GPU tensor and
    every other operand must be on its device (a host pointer handed to a
    kernel would fault)."""
    if q.device.type != "cuda":
        raise ValueError(f"operands must be GPU tensors (got {q.device})")
    _same_device(q.device, **tensors)


def _int32_vector(t, n, name, device):
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != n or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name} must be a contiguous int32 vector of {n} entries on the device of q")
    return t.data_ptr()


def make_params(q, k, v, o, *, scale, causal, q_offset, bias, window=0, cu_seqlens_q=None,
                cu_seqlens_k=None, max_seqlen_q=None, seqlens_k=None) -> Params:
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    b, hq, tq, dh = q.shape
    p = Params()
    p.batch, p.heads_q, p.heads_kv = b, hq, k.shape[1]
    p.t_q, p.t_k, p.d_h, p.d_v = tq, k.shape[2], dh, v.shape[3]
    if k.shape[0] != b or v.shape[0] != b or v.shape[1] != k.shape[1] or v.shape[2] != k.shape[2]:
        raise ValueError("k and v must be [B, H_kv, T_k, *] with the batch of q")
    if k.shape[3] != dh:
        raise ValueError("q and k must share d_h")
    _same_device(q.device, k=k, v=v, o=None if o.device.type == "meta" else o)
    p.q_offset = int(q_offset)
    p.q_stride[:] = _outer_strides(q, "q")
    p.k_stride[:] = _outer_strides(k, "k")
    p.v_stride[:] = _outer_strides(v, "v")
    p.o_stride[:] = _outer_strides(o, "o")
    p.scale = float(1.0 / math.sqrt(dh) if scale is None else scale)
    p.dtype = _DTYPES[q.dtype]
    p.causal = 1 if causal else 0
    if window is None or int(window) < 0 or int(window) >= 1 << 31:
        raise ValueError("window must be an int in [0, 2^31)")
    p.window = int(window)
    if bias is not None:
        if bias.dtype != torch.float32 or bias.device != q.device:
            raise ValueError("bias must be a float32 tensor on the device of q")
        full = bias.expand(b, hq, tq, k.shape[2])
        p.bias_stride[:] = tuple(int(x) for x in full.stride())
        p.bias = full.data_ptr() if full.numel() else None
    if cu_seqlens_q is not None or cu_seqlens_k is not None:
        if cu_seqlens_q is None or cu_seqlens_k is None or b != 1:
            raise ValueError("packed sequences need cu_seqlens_q and cu_seqlens_k and batch 1")
        n = cu_seqlens_q.shape[0] - 1 if cu_seqlens_q.dim() == 1 else -1
        if n < 0:
            raise ValueError("cu_seqlens_q must hold n_seqs + 1 offsets")
        p.cu_seqlens_q = _int32_vector(cu_seqlens_q, n + 1, "cu_seqlens_q", q.device)
        p.cu_seqlens_k = _int32_vector(cu_seqlens_k, n + 1, "cu_seqlens_k", q.device)
        p.n_seqs = n
        # Without a caller's bound the grid covers the longest possible sequence.
        p.max_seqlen_q = tq if max_seqlen_q is None else int(max_seqlen_q)
    if seqlens_k is not None:
        p.seqlens_k = _int32_vector(seqlens_k, b, "seqlens_k", q.device)
    return p


def _outputs(q, d_v, out, lse):
    """The output and LSE tensors: allocated here, or the caller's after
    checking that the kernels' writes stay inside them (shape, dtype and
    device; any outer strides of out, a contiguous LSE)."""
    b, hq, tq, _ = q.shape
    if out is None:
        out = torch.empty((b, hq, tq, d_v), dtype=q.dtype, device=q.device)
    elif out.dtype != q.dtype or tuple(out.shape) != (b, hq, tq, d_v) or out.device != q.device:
        raise ValueError(f"out must be a [B, H_q, T_q, d_v] = {(b, hq, tq, d_v)} {q.dtype} tensor "
                         f"on {q.device}")
    if lse is None:
        lse = torch.empty((b, hq, tq), dtype=torch.float32, device=q.device)
    elif (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (b, hq, tq)
          or lse.device != q.device):
        raise ValueError("lse must be a contiguous [B, H_q, T_q] float32 tensor on the device of q")
    return out, lse


def attn_fwd(q, k, v, *, scale=None, causal=True, q_offset=0, bias=None, window=0,
             out=None, lse=None, return_n_legal=False, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, seqlens_k=None, stream=None):
    """Exact attention; returns (o, lse) or (o, lse, n_legal).  ``window`` > 0
    keeps only keys j >= q_offset + i - window + 1 for row i.

    Packed sequences: q, k, v of batch 1 with ``cu_seqlens_q`` /
    ``cu_seqlens_k`` (int32 device offsets, n_seqs + 1 each); row i of a
    sequence sits at q_offset + (L_k - L_q) + i and sees only its own keys.
    ``max_seqlen_q`` (a host int) sizes the grid; it defaults to T_q.
    Per-batch KV lengths: ``seqlens_k`` (int32 device, one per batch); batch b
    uses keys [0, L_b) and its row i sits at q_offset + L_b - T_q + i."""
    lib = load_library()
    out, lse = _outputs(q, v.shape[3], out, lse)
    _require_gpu(q, k=k, v=v, bias=bias, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                 seqlens_k=seqlens_k)
    p = make_params(q, k, v, out, scale=scale, causal=causal, q_offset=q_offset, bias=bias,
                    window=window, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                    max_seqlen_q=max_seqlen_q, seqlens_k=seqlens_k)
    n_legal = None
    if return_n_legal:
        n_legal = torch.empty(lse.shape, dtype=torch.int32, device=q.device)
    _check(lib.attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                        _ptr(n_legal), _stream(q.device, stream)))
    return (out, lse, n_legal) if return_n_legal else (out, lse)


def _decode_offset(q, k_cache, q_offset, seqlens_k):
    """Default query position: the newest T_q positions of the cache (with
    per-batch lengths the library already places rows at the end of each)."""
    if q_offset is not None:
        return q_offset
    return 0 if seqlens_k is not None else k_cache.shape[2] - q.shape[2]


def attn_decode_workspace_bytes(q, k_cache, v_cache, *, split_size, scale=None,
                                causal=True, q_offset=None, bias=None, window=0,
                                seqlens_k=None) -> int:
    lib = load_library()
    o = torch.empty((q.shape[0], q.shape[1], q.shape[2], v_cache.shape[3]),
                    dtype=q.dtype, device="meta")
    off = _decode_offset(q, k_cache, q_offset, seqlens_k)
    p = make_params(q, k_cache, v_cache, o, scale=scale, causal=causal, q_offset=off, bias=bias,
                    window=window, seqlens_k=seqlens_k)
    return int(lib.attn_decode_workspace_bytes(ctypes.byref(p), int(split_size)))


def attn_decode_splitkv(q, k_cache, v_cache, *, split_size, scale=None, causal=True,
                        q_offset=None, bias=None, window=0, seqlens_k=None, workspace=None,
                        out=None, lse=None, stream=None):
    """Split-KV decode + merge; returns (o, lse, workspace).

    ``q_offset`` defaults to T_k - T_q (the queries are the newest positions),
    or to 0 with ``seqlens_k`` (int32 device KV length per batch: batch b
    uses keys [0, L_b), its rows at q_offset + L_b - T_q + i).
    ``workspace`` is a uint8 device tensor of at least
    ``attn_decode_workspace_bytes`` bytes; allocated here when None."""
    lib = load_library()
    out, lse = _outputs(q, v_cache.shape[3], out, lse)
    _require_gpu(q, k_cache=k_cache, v_cache=v_cache, bias=bias, seqlens_k=seqlens_k,
                 workspace=workspace)
    off = _decode_offset(q, k_cache, q_offset, seqlens_k)
    p = make_params(q, k_cache, v_cache, out, scale=scale, causal=causal, q_offset=off, bias=bias,
                    window=window, seqlens_k=seqlens_k)
    need = int(lib.attn_decode_workspace_bytes(ctypes.byref(p), int(split_size)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _check(lib.attn_decode_splitkv(ctypes.byref(p), int(split_size), _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(out), _ptr(lse),
                                   ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                   _stream(q.device, stream)))
    return out, lse, workspace


def attn_decode_splitkv_noalloc(q, k_cache, v_cache, *, split_size, scale=None, causal=True,
                                q_offset=None, bias=None, window=0, seqlens_k=None, out=None,
                                lse=None, stream=None):
    """attn_decode_splitkv with the library's fixed per-GPU workspace instead
    of a caller's (the C entry point allocates nothing; outputs are allocated
    here when not given).  Returns (o, lse).  Problems whose workspace would
    exceed DECODE_SCRATCH_BYTES raise ValueError; calls that overlap on one
    GPU race on that workspace."""
    lib = load_library()
    out, lse = _outputs(q, v_cache.shape[3], out, lse)
    _require_gpu(q, k_cache=k_cache, v_cache=v_cache, bias=bias, seqlens_k=seqlens_k)
    off = _decode_offset(q, k_cache, q_offset, seqlens_k)
    p = make_params(q, k_cache, v_cache, out, scale=scale, causal=causal, q_offset=off, bias=bias,
                    window=window, seqlens_k=seqlens_k)
    with torch.cuda.device(q.device):   # the library works on the current device
        _check(lib.attn_decode_splitkv_noalloc(ctypes.byref(p), int(split_size), _ptr(q),
                                               _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                               _stream(q.device, stream)))
    return out, lse


def attn_bwd(q, k, v, o, lse, d_o, *, scale=None, causal=True, q_offset=0, bias=None, window=0,
             cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, seqlens_k=None,
             d_q=None, d_k=None, d_v=None, workspace=None, stream=None):
    """Gradients (d_q, d_k, d_v) of attn_fwd's attention for the upstream
    gradient ``d_o``, recomputed from the forward's ``o`` and ``lse``.  Each
    gradient gets the shape, strides and dtype of its forward tensor; ``d_o``
    must have the strides of ``o``.

    Packed sequences take the forward's ``cu_seqlens_q`` / ``cu_seqlens_k`` /
    ``max_seqlen_q``; the library leaves rows and keys outside every sequence
    unwritten, so gradients allocated here start at zero.  Per-batch KV
    lengths take the forward's ``seqlens_k``; keys past a batch's length get
    zero gradients."""
    lib = load_library()
    _require_gpu(q, k=k, v=v, o=o, lse=lse, d_o=d_o, bias=bias, cu_seqlens_q=cu_seqlens_q,
                 cu_seqlens_k=cu_seqlens_k, seqlens_k=seqlens_k, d_q=d_q, d_k=d_k, d_v=d_v,
                 workspace=workspace)
    if d_o.shape != o.shape or d_o.stride() != o.stride() or d_o.dtype != o.dtype:
        raise ValueError("d_o must have the shape, strides and dtype of o")
    if not lse.is_contiguous() or lse.shape != o.shape[:3] or lse.dtype != torch.float32:
        raise ValueError("lse must be the contiguous float32 [B, H_q, T_q] LSE of the forward")
    p = make_params(q, k, v, o, scale=scale, causal=causal, q_offset=q_offset, bias=bias,
                    window=window, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                    max_seqlen_q=max_seqlen_q, seqlens_k=seqlens_k)
    grads = []
    for t, g in ((q, d_q), (k, d_k), (v, d_v)):
        if g is None:
            g = torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)
            if cu_seqlens_q is not None:
                g.zero_()
        elif g.shape != t.shape or g.stride() != t.stride() or g.dtype != t.dtype:
            raise ValueError("gradients must have the shape, strides and dtype of their tensors")
        grads.append(g)
    need = int(lib.attn_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _check(lib.attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o),
                        _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]),
                        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                        _stream(q.device, stream)))
    return tuple(grads)


def split_workspace_views(workspace, q, v_cache, split_size):
    """(o_parts [B, H_q, T_q, S, d_v], lse_parts [B, H_q, T_q, S]) views of a
    decode workspace, in the layout the header documents."""
    b, hq, tq, _ = q.shape
    t_k, d_v = v_cache.shape[2], v_cache.shape[3]
    n_splits = max(1, -(-t_k // split_size))
    rows = b * hq * tq
    o_bytes = rows * n_splits * d_v * 4
    lse_off = (o_bytes + 255) // 256 * 256
    o = workspace[:o_bytes].view(torch.float32).view(b, hq, tq, n_splits, d_v)
    l = workspace[lse_off:lse_off + rows * n_splits * 4].view(torch.float32).view(b, hq, tq, n_splits)
    return o, l


def attn_merge_states(o_states, lse_states, *, out_dtype=torch.float32, out=None,
                      lse_out=None, stream=None):
    """Merge partials o_states [R, S, d_v] / lse_states [R, S] (fp32) into
    (o [R, d_v], lse [R])."""
    lib = load_library()
    if o_states.dtype != torch.float32 or lse_states.dtype != torch.float32:
        raise ValueError("partials must be float32")
    if o_states.dim() != 3 or lse_states.dim() != 2:
        raise ValueError("o_states must be [R, S, d_v] and lse_states [R, S]")
    r, s, d_v = o_states.shape
    if lse_states.shape != (r, s):
        raise ValueError("lse_states must be [R, S]")
    if d_v > 1 and o_states.stride(2) != 1:
        raise ValueError("o_states must have a contiguous innermost dimension")
    if out is None:
        if out_dtype not in _DTYPES:
            raise ValueError("out_dtype must be float32 or bfloat16")
        out = torch.empty((r, d_v), dtype=out_dtype, device=o_states.device)
    if lse_out is None:
        lse_out = torch.empty((r,), dtype=torch.float32, device=o_states.device)
    if out.dtype not in _DTYPES or tuple(out.shape) != (r, d_v) or (d_v > 1 and out.stride(1) != 1):
        raise ValueError(f"out must be a float32 or bfloat16 [R, d_v] = {(r, d_v)} tensor with "
                         "contiguous rows")
    if lse_out.dtype != torch.float32 or lse_out.numel() != r or not lse_out.is_contiguous():
        raise ValueError(f"lse_out must be a contiguous float32 tensor of R = {r} elements")
    _require_gpu(o_states, lse_states=lse_states, out=out, lse_out=lse_out)
    _check(lib.attn_merge_states(r, s, d_v, _ptr(o_states), o_states.stride(0),
                                 o_states.stride(1), _ptr(lse_states), lse_states.stride(0),
                                 lse_states.stride(1), _DTYPES[out.dtype], _ptr(out),
                                 out.stride(0), _ptr(lse_out), _stream(o_states.device, stream)))
    return out, lse_out
