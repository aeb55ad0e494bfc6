"""Python binding of libfa2.so, the gfx950 FlashAttention-2 library.

Argument marshalling only: every step of the forward and backward passes runs
in the HIP kernels behind the C ABI declared in ``include/fa2.h``.  PyTorch is
used for device memory and the current stream.  There is no fallback: if the
library is not built, importing works but every call raises ``Fa2Error``.

Functions with the C names (``fa2_forward``, ``fa2_backward``,
``fa2_backward_stage``, their ``_ex`` forms with a key/value head count for
grouped-query attention, ``fa2_backward_workspace_size`` (``_ex``),
``fa2_forward_varlen``, ``fa2_backward_varlen`` (packed ragged batches),
``fa2_backward_noalloc`` (the backward with the library's static workspace),
``fa2_decode``, ``fa2_decode_workspace_size``, ``fa2_status_string``) take
caller-allocated tensors like the C ABI; ``forward`` / ``backward`` /
``decode`` allocate the outputs (K and V may have fewer heads than Q: H_kv
dividing H); ``attention`` is the same forward and backward as a
``torch.autograd.Function``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

FA2_F32 = 0
FA2_BF16 = 1
FA2_F16 = 2
FA2_OK = 0
FA2_ERR_INVALID_ARG = 1
FA2_ERR_UNSUPPORTED = 2
FA2_ERR_WORKSPACE = 3
FA2_ERR_LAUNCH = 4
FA2_ERR_SCRATCH = 5
# Bytes of the static workspace behind fa2_backward_noalloc (FA2_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa2.so")

_lib = None


class Fa2Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s" % (what, fa2_status_string(status)))


def lib() -> ctypes.CDLL:
    """The loaded libfa2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Fa2Error(FA2_ERR_LAUNCH, "libfa2.so is not built (python -m tiled_attention_fwd_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.fa2_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
        L.fa2_forward.restype = i
        L.fa2_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp,
                                   ctypes.c_size_t, vp]
        L.fa2_backward.restype = i
        L.fa2_backward_stage.argtypes = [i] + L.fa2_backward.argtypes
        L.fa2_backward_stage.restype = i
        L.fa2_forward_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.fa2_forward_ex.restype = i
        L.fa2_backward_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp,
                                      ctypes.c_size_t, vp]
        L.fa2_backward_ex.restype = i
        L.fa2_backward_stage_ex.argtypes = [i] + L.fa2_backward_ex.argtypes
        L.fa2_backward_stage_ex.restype = i
        L.fa2_backward_workspace_size.argtypes = [i, i, i, i, i]
        L.fa2_backward_workspace_size.restype = ctypes.c_size_t
        L.fa2_backward_workspace_size_ex.argtypes = [i, i, i, i, i, i]
        L.fa2_backward_workspace_size_ex.restype = ctypes.c_size_t
        L.fa2_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
        L.fa2_backward_noalloc.restype = i
        L.fa2_forward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        L.fa2_forward_varlen.restype = i
        L.fa2_backward_varlen.argtypes = [vp] * 10 + [i, i, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
        L.fa2_backward_varlen.restype = i
        L.fa2_backward_stage_varlen.argtypes = [i] + L.fa2_backward_varlen.argtypes
        L.fa2_backward_stage_varlen.restype = i
        L.fa2_backward_workspace_size_varlen.argtypes = [i, i, i, i, i, i, i]
        L.fa2_backward_workspace_size_varlen.restype = ctypes.c_size_t
        L.fa2_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
        L.fa2_decode.restype = i
        L.fa2_decode_workspace_size.argtypes = [i, i, i, i, i, i, i]
        L.fa2_decode_workspace_size.restype = ctypes.c_size_t
        L.fa2_status_string.argtypes = [i]
        L.fa2_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def fa2_status_string(status: int) -> str:
    try:
        return lib().fa2_status_string(int(status)).decode()
    except Fa2Error:
        return "status %d" % status


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return FA2_F32
    if t == torch.bfloat16:
        return FA2_BF16
    if t == torch.float16:
        return FA2_F16
    raise TypeError("unsupported dtype %s (float32, bfloat16 or float16)" % t)


def _check_tensors(ref: torch.Tensor, *ts: torch.Tensor):
    if ref.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors, got %s" % (tuple(ref.shape),))
    for t in (ref,) + ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
        if t.device != ref.device:
            raise ValueError("tensors must be on one device")


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _scratch(nbytes: int, device, stream) -> torch.Tensor:
    """A device buffer that the library's kernels use on ``stream``.

    torch's caching allocator ties a block to the stream current at
    allocation; when the launch stream is another one, the block is also
    recorded on it, so that freeing the tensor (at the end of the call that
    allocated it) cannot hand the memory to new work while the kernels
    enqueued on ``stream`` still use it."""
    t = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    _record(t, stream)
    return t


def _record(t: torch.Tensor, stream) -> None:
    if stream is None:
        return
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=t.device)
    if stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _heads(q, k, v, *qlike):
    """(B, H, H_kv, N, d) after checking q-shaped and k-shaped arguments."""
    B, H, N, d = q.shape
    if k.dim() != 4:
        raise ValueError("expected [B, H_kv, N, d] keys, got %s" % (tuple(k.shape),))
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d) or v.shape != k.shape or H_kv == 0 and H != 0 or H_kv and H % H_kv:
        raise ValueError("k, v must be [B, H_kv, N, d] with H_kv dividing H = %d" % H)
    for t in (k, v) + tuple(qlike):
        if t.dtype != q.dtype:
            raise ValueError("all tensors must share one dtype")
    for t in qlike:
        if t.shape != q.shape:
            raise ValueError("o, dO, dq must have q's shape")
    return B, H, H_kv, N, d


def fa2_forward(q, k, v, o, lse, causal: bool = True, scale: float | None = None, stream=None) -> None:
    """Enqueue the forward pass into caller-allocated ``o`` and ``lse``."""
    _forward_call(False, q, k, v, o, lse, causal, scale, stream)


def fa2_forward_ex(q, k, v, o, lse, causal: bool = True, scale: float | None = None, stream=None) -> None:
    """As ``fa2_forward`` with k, v of H_kv heads ([B, H_kv, N, d])."""
    _forward_call(True, q, k, v, o, lse, causal, scale, stream)


def _forward_call(ex, q, k, v, o, lse, causal, scale, stream):
    _check_tensors(q, k, v, o, lse)
    B, H, H_kv, N, d = _heads(q, k, v, o)
    if not ex and H_kv != H:
        raise ValueError("fa2_forward needs H_kv == H; use fa2_forward_ex")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    tail = (N, d, _scale(scale, d), int(bool(causal)), _dtype_code(q.dtype), _stream(stream, q.device))
    if ex:
        st = lib().fa2_forward_ex(*ptrs, B, H, H_kv, *tail)
    else:
        st = lib().fa2_forward(*ptrs, B, H, *tail)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_forward_ex" if ex else "fa2_forward")


def fa2_backward_workspace_size(B: int, H: int, N: int, d: int, dtype) -> int:
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().fa2_backward_workspace_size(B, H, N, d, code))


def fa2_backward_workspace_size_ex(B: int, H: int, H_kv: int, N: int, d: int, dtype) -> int:
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().fa2_backward_workspace_size_ex(B, H, H_kv, N, d, code))


def fa2_backward(q, k, v, o, dO, lse, dq, dk, dv, causal: bool = True, scale: float | None = None,
                 workspace: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue the backward pass into caller-allocated ``dq``, ``dk``, ``dv``."""
    _backward_call(False, 0, q, k, v, o, dO, lse, dq, dk, dv, causal, scale, workspace, stream)


def fa2_backward_ex(q, k, v, o, dO, lse, dq, dk, dv, causal: bool = True, scale: float | None = None,
                    workspace: torch.Tensor | None = None, stream=None) -> None:
    """As ``fa2_backward`` with k, v, dk, dv of H_kv heads."""
    _backward_call(True, 0, q, k, v, o, dO, lse, dq, dk, dv, causal, scale, workspace, stream)


def fa2_backward_stage(stage: int, q, k, v, o, dO, lse, dq, dk, dv, causal: bool = True,
                       scale: float | None = None, workspace: torch.Tensor | None = None,
                       stream=None) -> None:
    """Enqueue one backward stage: 1 the dQ kernel (which also writes D and
    LSE*log2(e) to the workspace), 2 the dK/dV kernel; 1 then 2 is
    ``fa2_backward``."""
    if workspace is None:
        raise ValueError("the stages share state through the workspace: pass one")
    _backward_call(False, int(stage), q, k, v, o, dO, lse, dq, dk, dv, causal, scale, workspace, stream)


def fa2_backward_stage_ex(stage: int, q, k, v, o, dO, lse, dq, dk, dv, causal: bool = True,
                          scale: float | None = None, workspace: torch.Tensor | None = None,
                          stream=None) -> None:
    """As ``fa2_backward_stage`` with k, v, dk, dv of H_kv heads."""
    if workspace is None:
        raise ValueError("the stages share state through the workspace: pass one")
    _backward_call(True, int(stage), q, k, v, o, dO, lse, dq, dk, dv, causal, scale, workspace, stream)


def fa2_backward_noalloc(q, k, v, o, dO, lse, dq, dk, dv, causal: bool = True, scale: float | None = None,
                         stream=None) -> None:
    """``fa2_backward_ex`` without a workspace argument: the library's static
    per-GPU buffer serves as the workspace and nothing is allocated (for
    callers that cannot allocate).  Problems needing more than
    NOALLOC_SCRATCH_BYTES raise (FA2_ERR_SCRATCH); calls whose work overlaps
    on one GPU share that buffer and race."""
    _check_tensors(q, k, v, o, dO, lse, dq, dk, dv)
    B, H, H_kv, N, d = _heads(q, k, v, o, dO, dq)
    if dk.shape != k.shape or dv.shape != k.shape or dk.dtype != q.dtype or dv.dtype != q.dtype:
        raise ValueError("dk, dv must have k's shape and q's dtype")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    st = lib().fa2_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d,
                                    _scale(scale, d), int(bool(causal)), _dtype_code(q.dtype),
                                    _stream(stream, q.device))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_backward_noalloc")


def _backward_call(ex, stage, q, k, v, o, dO, lse, dq, dk, dv, causal, scale, workspace, stream):
    _check_tensors(q, k, v, o, dO, lse, dq, dk, dv)
    B, H, H_kv, N, d = _heads(q, k, v, o, dO, dq)
    if dk.shape != k.shape or dv.shape != k.shape or dk.dtype != q.dtype or dv.dtype != q.dtype:
        raise ValueError("dk, dv must have k's shape and q's dtype")
    if not ex and H_kv != H:
        raise ValueError("fa2_backward needs H_kv == H; use fa2_backward_ex")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N]")
    need = fa2_backward_workspace_size_ex(B, H, H_kv, N, d, q.dtype)
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    tail = (N, d, _scale(scale, d), int(bool(causal)), _dtype_code(q.dtype), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    heads = (B, H, H_kv) if ex else (B, H)
    L = lib()
    if stage == 0:
        st = (L.fa2_backward_ex if ex else L.fa2_backward)(*ptrs, *heads, *tail)
    else:
        st = (L.fa2_backward_stage_ex if ex else L.fa2_backward_stage)(stage, *ptrs, *heads, *tail)
    if st != FA2_OK:
        name = ("fa2_backward" if stage == 0 else "fa2_backward_stage(%d)" % stage) + ("_ex" if ex else "")
        raise Fa2Error(st, name)


def _varlen_shapes(q, k, v, cu_seqlens, max_seqlen, *qlike):
    """(B, H, H_kv, T, d) of a packed ragged batch after checking shapes."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed tensors are [H, T, d]")
    H, T, d = q.shape
    H_kv = k.shape[0]
    if k.shape != (H_kv, T, d) or v.shape != k.shape or H_kv == 0 and H != 0 or H_kv and H % H_kv:
        raise ValueError("k, v must be [H_kv, T, d] with H_kv dividing H = %d" % H)
    for t in (k, v) + tuple(qlike):
        if t.dtype != q.dtype:
            raise ValueError("all tensors must share one dtype")
    for t in qlike:
        if t.shape != q.shape:
            raise ValueError("o, dO, dq must have q's shape")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda \
            or not cu_seqlens.is_contiguous() or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be a contiguous int32 GPU tensor [B + 1]")
    return cu_seqlens.numel() - 1, H, H_kv, T, d


def fa2_forward_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen: int, causal: bool = True,
                       scale: float | None = None, stream=None) -> None:
    """Forward pass of a packed ragged batch: q, o [H, T, d]; k, v
    [H_kv, T, d]; lse float32 [H, T]; sequence b is rows cu_seqlens[b] ..
    cu_seqlens[b+1]-1 of every head."""
    _check_tensors_any(q, k, v, o, lse)
    B, H, H_kv, T, d = _varlen_shapes(q, k, v, cu_seqlens, max_seqlen, o)
    if lse.shape != (H, T) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [H, T]")
    st = lib().fa2_forward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  cu_seqlens.data_ptr(), B, H, H_kv, T, int(max_seqlen), d, _scale(scale, d),
                                  int(bool(causal)), _dtype_code(q.dtype), _stream(stream, q.device))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_forward_varlen")


def fa2_backward_workspace_size_varlen(B: int, H: int, H_kv: int, T: int, max_seqlen: int, d: int, dtype) -> int:
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().fa2_backward_workspace_size_varlen(B, H, H_kv, T, max_seqlen, d, code))


def fa2_backward_varlen(q, k, v, o, dO, lse, dq, dk, dv, cu_seqlens, max_seqlen: int, causal: bool = True,
                        scale: float | None = None, workspace: torch.Tensor | None = None, stream=None,
                        stage: int = 0) -> None:
    """Backward pass of a packed ragged batch (stage 0: both stages,
    else ``fa2_backward_stage_varlen``); dk, dv have k's shape."""
    _check_tensors_any(q, k, v, o, dO, lse, dq, dk, dv)
    B, H, H_kv, T, d = _varlen_shapes(q, k, v, cu_seqlens, max_seqlen, o, dO, dq)
    if dk.shape != k.shape or dv.shape != k.shape or dk.dtype != q.dtype or dv.dtype != q.dtype:
        raise ValueError("dk, dv must have k's shape and q's dtype")
    if lse.shape != (H, T) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [H, T]")
    need = fa2_backward_workspace_size_varlen(B, H, H_kv, T, int(max_seqlen), d, q.dtype)
    if workspace is None:
        if stage:
            raise ValueError("the stages share state through the workspace: pass one")
        workspace = _scratch(need, q.device, stream)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(), lse.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), cu_seqlens.data_ptr(), B, H, H_kv, T, int(max_seqlen), d,
            _scale(scale, d), int(bool(causal)), _dtype_code(q.dtype), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    if stage:
        st = lib().fa2_backward_stage_varlen(int(stage), *args)
    else:
        st = lib().fa2_backward_varlen(*args)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_backward_varlen" if not stage else "fa2_backward_stage_varlen(%d)" % stage)


def _check_tensors_any(*ts: torch.Tensor):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.device != ts[0].device:
            raise ValueError("tensors must be on one device")


def fa2_decode_workspace_size(B: int, H: int, H_kv: int, N_q: int, N_k: int, d: int, dtype) -> int:
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().fa2_decode_workspace_size(B, H, H_kv, N_q, N_k, d, code))


def fa2_decode(q, k, v, o, lse, causal: bool = False, scale: float | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue decoding of q [B, H, N_q, d] against the cache k, v
    [B, H_kv, N_k, d] into caller-allocated ``o`` (q's shape) and ``lse``
    (float32 [B, H, N_q]); causal places the queries at the cache's last
    N_q positions."""
    _check_tensors(q, k, v, o, lse)
    B, H, Nq, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k, v must be [B, H_kv, N_k, d] with q's B and d")
    H_kv, Nk = k.shape[1], k.shape[2]
    for t in (k, v, o):
        if t.dtype != q.dtype:
            raise ValueError("all tensors must share one dtype")
    if o.shape != q.shape:
        raise ValueError("o must have q's shape")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, N_q]")
    code = _dtype_code(q.dtype)
    need = int(lib().fa2_decode_workspace_size(B, H, H_kv, Nq, Nk, d, code))
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fa2_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv, Nq,
                          Nk, d, _scale(scale, d), int(bool(causal)), code, ws_ptr, ws_bytes,
                          _stream(stream, q.device))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_decode")


def decode(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Return (o, lse) of q [B, H, N_q, d] against the cache k, v
    [B, H_kv, N_k, d] (float32, bfloat16 or float16; d = 16, 32, 64, 128)."""
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    for t in (o, lse):
        _record(t, stream)
    fa2_decode(q, k, v, o, lse, causal, scale, None, stream)
    return o, lse


def forward(q, k, v, causal: bool = True, scale: float | None = None, stream=None):
    """Return (o, lse) for q [B, H, N, d] and k, v [B, H_kv, N, d] (H_kv
    dividing H) float32, bfloat16 or float16 GPU tensors."""
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    for t in (o, lse):
        _record(t, stream)
    fa2_forward_ex(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def backward(q, k, v, o, lse, dO, causal: bool = True, scale: float | None = None,
             workspace: torch.Tensor | None = None, stream=None):
    """Return (dq, dk, dv) of L = sum(o * dO); o, lse come from ``forward``;
    dk, dv have k's shape."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for t in (dq, dk, dv):
        _record(t, stream)
    fa2_backward_ex(q, k, v, o, dO, lse, dq, dk, dv, causal, scale, workspace, stream)
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """torch.autograd bridge: the forward pass runs ``forward`` (keeping o and
    lse for the backward), the backward pass ``backward``; both on the current
    stream."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = forward(q, k, v, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, dO.contiguous(), ctx.causal, ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal: bool = True, scale: float | None = None):
    """O = softmax(scale * q k^T + mask) v for contiguous q [B, H, N, d] and
    k, v [B, H_kv, N, d] on the GPU, differentiable in q, k and v through
    torch.autograd (the library's forward and backward kernels; scale
    defaults to 1/sqrt(d))."""
    return _Attention.apply(q, k, v, causal, scale)
