"""Dynamic Bifocal RoPE attention (Jet-Long) for MI355X: Python binding of libbifocal.so.

Thin ctypes layer over the C ABI declared in include/bifocal.h: it checks tensor
dtypes/devices, allocates outputs with torch, and passes raw device pointers and the
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no fallback path.  If the shared library is missing, importing
this package succeeds but the first call raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "lib", "lib_path", "rope_apply", "bifocal_prefill", "bifocal_prefill_ie", "bifocal_decode",
    "bifocal_decode_batch", "workspace_bytes", "group_size", "Workspace", "BifocalError",
    "OP_PREFILL", "OP_DECODE", "OP_PREFILL_IE", "VARIANTS", "bifocal_prefill_variant",
    "bifocal_decode_variant", "bifocal_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libbifocal.so")

OP_ROPE, OP_PREFILL, OP_DECODE, OP_PREFILL_IE = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 4 << 20  # BIFOCAL_NOALLOC_SCRATCH_BYTES
VARIANTS = {"bifocal": 0, "interp": 1, "window": 2}
_F32, _BF16 = 0, 1


class BifocalError(RuntimeError):
    pass


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is missing: build it with `python -m dynamic_rope_context_amd.build`")
    lib = ctypes.CDLL(lib_path)
    vp, i32, i64, sz, f32, f64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_size_t, ctypes.c_float, ctypes.c_double)
    lib.rope_apply.argtypes = [vp, vp, i32, i32, i32, i32, f64, i32, i32, vp]
    lib.rope_apply.restype = i32
    lib.bifocal_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64,
                                    f32, i32, vp, sz, vp]
    lib.bifocal_prefill.restype = i32
    lib.bifocal_prefill_ie.argtypes = lib.bifocal_prefill.argtypes
    lib.bifocal_prefill_ie.restype = i32
    lib.bifocal_prefill_variant.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            f64, f32, i32, i32, vp, sz, vp]
    lib.bifocal_prefill_variant.restype = i32
    lib.bifocal_decode_variant.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           i32, f64, f32, i32, i32, vp, sz, vp]
    lib.bifocal_decode_variant.restype = i32
    lib.bifocal_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64, f32,
                                   i32, vp, sz, vp]
    lib.bifocal_decode.restype = i32
    lib.bifocal_decode_batch.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, f64, f32, i32, vp, sz, vp]
    lib.bifocal_decode_batch.restype = i32
    lib.bifocal_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64,
                                           f32, i32, vp]
    lib.bifocal_decode_noalloc.restype = i32
    lib.bifocal_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32]
    lib.bifocal_workspace_bytes.restype = sz
    lib.bifocal_status_string.argtypes = [i32]
    lib.bifocal_status_string.restype = ctypes.c_char_p
    lib.bifocal_group_size.argtypes = [i64, i32]
    lib.bifocal_group_size.restype = i32
    return lib


_lib_handle = None


def lib():
    """The loaded libbifocal.so (loaded on first use; raises if it was not built)."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


def _check(status: int, what: str) -> None:
    if status != 0:
        raise BifocalError(f"{what}: {lib().bifocal_status_string(status).decode()} ({status})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise BifocalError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _outputs(ref: torch.Tensor, out, lse, want_lse: bool, lse_shape):
    """Allocate or check the output tensors: out like ``ref``, lse float32 of lse_shape on
    the same device.  A caller-provided buffer of the wrong shape, dtype or device is an
    error (the library writes through raw pointers)."""
    if out is None:
        out = torch.empty_like(ref)
    elif out.shape != ref.shape or out.dtype != ref.dtype or out.device != ref.device:
        raise BifocalError(f"out must be {tuple(ref.shape)} {ref.dtype} on {ref.device}")
    if lse is None and want_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=ref.device)
    elif lse is not None and (tuple(lse.shape) != tuple(lse_shape) or lse.dtype != torch.float32
                              or lse.device != ref.device):
        raise BifocalError(f"lse must be {tuple(lse_shape)} float32 on {ref.device}")
    return out, lse


def _same(ref: torch.Tensor, *ts) -> None:
    for t in ts:
        if t.dtype != ref.dtype or t.device != ref.device:
            raise BifocalError("inputs must share one dtype and one device")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise BifocalError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise BifocalError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _stream_obj(stream, device):
    """The torch stream object of a launch: the current stream, a torch stream, or a raw
    HIP stream handle wrapped as an external stream."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


class _CallWorkspace:
    """A workspace for one call that owns none: allocated (and its header cleared) on the
    launch stream, and marked as used by that stream afterwards, so that the caching
    allocator hands the memory to nobody else before the call's kernels are done."""

    def __init__(self, workspace, stream, device, make):
        self.given = workspace
        self.stream = stream
        self.device = device
        self.make = make
        self.ws = None

    def __enter__(self):
        if self.given is not None:
            return self.given
        s = _stream_obj(self.stream, self.device)
        with torch.cuda.stream(s):
            self.ws = self.make()
        self._s = s
        return self.ws

    def __exit__(self, *exc):
        if self.ws is not None:
            self.ws.buf.record_stream(self._s)
        return False


def group_size(L: int, w_pretrained: int) -> int:
    """G = max(1, ceil(L / w_pretrained)) as the kernels compute it."""
    return int(lib().bifocal_group_size(int(L), int(w_pretrained)))


def workspace_bytes(op: int, max_len: int, Hq: int, Hkv: int, D: int,
                    total_tokens: Optional[int] = None, num_seqs: int = 1) -> int:
    """Workspace bytes for an operation; prefill also needs the largest token count and
    batch size of the calls (defaults: one sequence of max_len tokens)."""
    total = max_len if total_tokens is None else total_tokens
    return int(lib().bifocal_workspace_bytes(op, max_len, total, num_seqs, Hq, Hkv, D))


class Workspace:
    """Caller-owned device workspace, 256-byte aligned.  Only its first 256 bytes (the
    position table's header) are cleared, on the current stream: every other byte is
    written by the library before it is read."""

    def __init__(self, nbytes: int, device="cuda"):
        if nbytes <= 0:
            raise BifocalError("workspace size must be positive")
        self.buf = torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.ptr = self.buf.data_ptr() + off
        self.nbytes = int(nbytes)
        self.buf[off:off + 256].zero_()

    @classmethod
    def for_op(cls, op: int, max_len: int, Hq: int, Hkv: int, D: int, device="cuda",
               total_tokens: Optional[int] = None, num_seqs: int = 1):
        n = workspace_bytes(op, max_len, Hq, Hkv, D, total_tokens, num_seqs)
        if n == 0:
            raise BifocalError("invalid workspace request")
        return cls(n, device)


def rope_apply(x: torch.Tensor, theta: float, pos: Optional[torch.Tensor] = None, pos0: int = 0,
               G: int = 1, stream=None) -> torch.Tensor:
    """In place: x[t, h, :] <- R(floor(p_t / G)) x[t, h, :] (G = 1: standard RoPE)."""
    if x.dim() != 3:
        raise BifocalError("x must be [T, H, D]")
    T, H, D = x.shape
    pp = 0
    if pos is not None:
        if pos.dtype != torch.int32 or pos.numel() != T:
            raise BifocalError("pos must be int32 [T]")
        pp = _dev(pos, "pos")
    _check(lib().rope_apply(_dev(x, "x"), pp, int(pos0), T, H, D, float(theta), int(G),
                           _dtype_code(x), _stream(stream)), "rope_apply")
    return x


def _prefill(fn, op, Q, K, V, cu_seqlens, w0, w_pretrained, theta, softmax_scale, out, lse,
             want_lse, workspace, stream, what):
    if Q.dim() != 3 or K.dim() != 3 or V.shape != K.shape:
        raise BifocalError("expected Q [T,Hq,D], K and V [T,Hkv,D]")
    T, Hq, D = Q.shape
    Hkv = K.shape[1]
    if K.shape[0] != T or K.shape[2] != D or K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise BifocalError("Q, K, V shapes or dtypes disagree")
    cu = [int(c) for c in cu_seqlens]
    B = len(cu) - 1
    cu_arr = (ctypes.c_int32 * len(cu))(*cu)
    _same(Q, K, V)
    out, lse = _outputs(Q, out, lse, want_lse, (Hq, T))
    max_len = max([cu[b + 1] - cu[b] for b in range(B)] + [0])
    make = lambda: Workspace.for_op(op, max(max_len, 1), Hq, Hkv, D, Q.device,
                                    total_tokens=max(T, max_len, 1), num_seqs=max(B, 1))
    with _CallWorkspace(workspace, stream, Q.device, make) as ws:
        _check(fn(
            _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(out, "out"),
            _dev(lse, "lse") if lse is not None else 0,
            ctypes.cast(cu_arr, ctypes.c_void_p), B, Hq, Hkv, D, int(w0), int(w_pretrained),
            float(theta), float(softmax_scale), _dtype_code(Q), ws.ptr, ws.nbytes,
            _stream(stream)), what)
    return out, lse


def bifocal_prefill(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                    cu_seqlens: Sequence[int], w0: int, w_pretrained: int, theta: float,
                    softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                    workspace: Optional[Workspace] = None, stream=None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Bifocal causal attention over packed sequences.  Q [T,Hq,D], K/V [T,Hkv,D] carry
    standard RoPE at local positions.  Returns (O [T,Hq,D], LSE [Hq,T] float32 or None)."""
    return _prefill(lib().bifocal_prefill, OP_PREFILL, Q, K, V, cu_seqlens, w0, w_pretrained,
                    theta, softmax_scale, out, lse, want_lse, workspace, stream,
                    "bifocal_prefill")


def bifocal_prefill_ie(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                       cu_seqlens: Sequence[int], w0: int, w_pretrained: int, theta: float,
                       softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                       workspace: Optional[Workspace] = None, stream=None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The same attention computed as three passes (local/window, remote/causal,
    remote/window) merged by inclusion-exclusion of their LSEs (bf16 only)."""
    return _prefill(lib().bifocal_prefill_ie, OP_PREFILL_IE, Q, K, V, cu_seqlens, w0,
                    w_pretrained, theta, softmax_scale, out, lse, want_lse, workspace, stream,
                    "bifocal_prefill_ie")


def bifocal_decode(q: torch.Tensor, Kcache: torch.Tensor, Vcache: torch.Tensor, pos: int,
                   w0: int, w_pretrained: int, theta: float, softmax_scale: float = 0.0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   want_lse: bool = True, workspace: Optional[Workspace] = None, stream=None
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One decode step: q [Hq,D] at position pos over cache entries 0..pos of
    Kcache/Vcache [S,Hkv,D] (standard RoPE).  Returns (o [Hq,D], LSE [Hq] or None)."""
    if q.dim() != 2 or Kcache.dim() != 3 or Vcache.shape != Kcache.shape:
        raise BifocalError("expected q [Hq,D], Kcache and Vcache [S,Hkv,D]")
    Hq, D = q.shape
    S, Hkv = Kcache.shape[0], Kcache.shape[1]
    if pos + 1 > S:
        raise BifocalError("the cache holds fewer than pos + 1 entries")
    _same(q, Kcache, Vcache)
    out, lse = _outputs(q, out, lse, want_lse, (Hq,))
    make = lambda: Workspace.for_op(OP_DECODE, pos + 1, Hq, Hkv, D, q.device)
    with _CallWorkspace(workspace, stream, q.device, make) as ws:
        _check(lib().bifocal_decode(
            _dev(q, "q"), _dev(Kcache, "Kcache"), _dev(Vcache, "Vcache"), _dev(out, "out"),
            _dev(lse, "lse") if lse is not None else 0, int(pos), Hq, Hkv, D, int(w0),
            int(w_pretrained), float(theta), float(softmax_scale), _dtype_code(q), ws.ptr,
            ws.nbytes, _stream(stream)), "bifocal_decode")
    return out, lse


def bifocal_decode_batch(q: torch.Tensor, Kcache: torch.Tensor, Vcache: torch.Tensor,
                         pos: Sequence[int], w0: int, w_pretrained: int, theta: float,
                         softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                         workspace: Optional[Workspace] = None, stream=None
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One decode step per sequence of a ragged batch: q [B,Hq,D], sequence b at position
    pos[b] over entries 0..pos[b] of Kcache/Vcache [B,S,Hkv,D] (standard RoPE), each with
    its own G.  Returns (o [B,Hq,D], LSE [B,Hq] or None)."""
    if q.dim() != 3 or Kcache.dim() != 4 or Vcache.shape != Kcache.shape:
        raise BifocalError("expected q [B,Hq,D], Kcache and Vcache [B,S,Hkv,D]")
    B, Hq, D = q.shape
    S, Hkv = Kcache.shape[1], Kcache.shape[2]
    pl = [int(p) for p in pos]
    if len(pl) != B or Kcache.shape[0] != B or Kcache.shape[3] != D:
        raise BifocalError("q, caches and pos disagree on the batch")
    _same(q, Kcache, Vcache)
    out, lse = _outputs(q, out, lse, want_lse, (B, Hq))
    make = lambda: Workspace.for_op(OP_DECODE, max(pl + [0]) + 1, Hq, Hkv, D, q.device,
                                    num_seqs=max(B, 1))
    pos_arr = (ctypes.c_int32 * max(B, 1))(*pl)
    with _CallWorkspace(workspace, stream, q.device, make) as ws:
        _check(lib().bifocal_decode_batch(
            _dev(q, "q"), _dev(Kcache, "Kcache"), _dev(Vcache, "Vcache"), _dev(out, "out"),
            _dev(lse, "lse") if lse is not None else 0, ctypes.cast(pos_arr, ctypes.c_void_p),
            B, S, Hq, Hkv, D, int(w0), int(w_pretrained), float(theta), float(softmax_scale),
            _dtype_code(q), ws.ptr, ws.nbytes, _stream(stream)), "bifocal_decode_batch")
    return out, lse


def _variant_code(variant) -> int:
    if variant not in VARIANTS:
        raise BifocalError(f"unknown variant {variant!r}; one of {sorted(VARIANTS)}")
    return VARIANTS[variant]


def bifocal_prefill_variant(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                            cu_seqlens: Sequence[int], w0: int, w_pretrained: int, theta: float,
                            variant: str = "bifocal", softmax_scale: float = 0.0,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            want_lse: bool = True, workspace: Optional[Workspace] = None,
                            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """bifocal_prefill for a variant: "bifocal", "interp" (remote positions x/G, continuous)
    or "window" (local window only)."""
    code = _variant_code(variant)
    f = lib().bifocal_prefill_variant

    def fn(*a):  # insert the variant before the dtype argument
        return f(*a[:14], code, *a[14:])
    return _prefill(fn, OP_PREFILL, Q, K, V, cu_seqlens, w0, w_pretrained, theta, softmax_scale,
                    out, lse, want_lse, workspace, stream, "bifocal_prefill_variant")


def bifocal_decode_variant(q: torch.Tensor, Kcache: torch.Tensor, Vcache: torch.Tensor,
                           pos: Sequence[int], w0: int, w_pretrained: int, theta: float,
                           variant: str = "bifocal", softmax_scale: float = 0.0,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           want_lse: bool = True, workspace: Optional[Workspace] = None,
                           stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """bifocal_decode_batch for a variant (see bifocal_prefill_variant)."""
    code = _variant_code(variant)
    if q.dim() != 3 or Kcache.dim() != 4 or Vcache.shape != Kcache.shape:
        raise BifocalError("expected q [B,Hq,D], Kcache and Vcache [B,S,Hkv,D]")
    B, Hq, D = q.shape
    S, Hkv = Kcache.shape[1], Kcache.shape[2]
    pl = [int(p) for p in pos]
    if len(pl) != B or Kcache.shape[0] != B or Kcache.shape[3] != D:
        raise BifocalError("q, caches and pos disagree on the batch")
    _same(q, Kcache, Vcache)
    out, lse = _outputs(q, out, lse, want_lse, (B, Hq))
    make = lambda: Workspace.for_op(OP_DECODE, max(pl + [0]) + 1, Hq, Hkv, D, q.device,
                                    num_seqs=max(B, 1))
    pos_arr = (ctypes.c_int32 * max(B, 1))(*pl)
    with _CallWorkspace(workspace, stream, q.device, make) as ws:
        _check(lib().bifocal_decode_variant(
            _dev(q, "q"), _dev(Kcache, "Kcache"), _dev(Vcache, "Vcache"), _dev(out, "out"),
            _dev(lse, "lse") if lse is not None else 0, ctypes.cast(pos_arr, ctypes.c_void_p),
            B, S, Hq, Hkv, D, int(w0), int(w_pretrained), float(theta), float(softmax_scale),
            code, _dtype_code(q), ws.ptr, ws.nbytes, _stream(stream)), "bifocal_decode_variant")
    return out, lse


def bifocal_decode_noalloc(q: torch.Tensor, Kcache: torch.Tensor, Vcache: torch.Tensor, pos: int,
                           w0: int, w_pretrained: int, theta: float, softmax_scale: float = 0.0,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           want_lse: bool = True, stream=None
                           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """bifocal_decode without a workspace (bf16, D = 128): the library keeps the split
    partials in a fixed device array of its own per GPU; calls that overlap on one GPU
    race.  Pass out (and lse) to allocate nothing here either."""
    if q.dim() != 2 or Kcache.dim() != 3 or Vcache.shape != Kcache.shape:
        raise BifocalError("expected q [Hq,D], Kcache and Vcache [S,Hkv,D]")
    Hq, D = q.shape
    S, Hkv = Kcache.shape[0], Kcache.shape[1]
    if pos + 1 > S:
        raise BifocalError("the cache holds fewer than pos + 1 entries")
    _same(q, Kcache, Vcache)
    out, lse = _outputs(q, out, lse, want_lse, (Hq,))
    _check(lib().bifocal_decode_noalloc(
        _dev(q, "q"), _dev(Kcache, "Kcache"), _dev(Vcache, "Vcache"), _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else 0, int(pos), Hq, Hkv, D, int(w0),
        int(w_pretrained), float(theta), float(softmax_scale), _dtype_code(q), _stream(stream)),
        "bifocal_decode_noalloc")
    return out, lse
