"""ctypes binding of libdiffattn (include/diffattn.h), same entry-point names.

Argument marshalling only: tensor checks, pointers, strides and the current
torch stream go in; every step of the computation runs in the library's HIP
kernels.  PyTorch provides device memory and streams.  If the library is not
built, every call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdiffattn.so")

DIFFATTN_FP32 = 0
DIFFATTN_BF16 = 1

STATUS = {0: "DIFFATTN_OK", 1: "DIFFATTN_ERR_INVALID_ARGUMENT", 2: "DIFFATTN_ERR_UNSUPPORTED",
          3: "DIFFATTN_ERR_WORKSPACE", 4: "DIFFATTN_ERR_HIP"}

EXPORTS = ("diffattn_lambda_init", "diffattn_lambda", "diffattn_prefill", "diffattn_prefill_v2",
           "diffattn_attention", "diffattn_combine",
           "diffattn_decode_workspace_bytes", "diffattn_decode", "diffattn_attention_decode",
           "diffattn_decode_noalloc",
           "diffattn_decode_v1_workspace_bytes",
           "diffattn_decode_v1", "diffattn_status_string",
           "diffattn_last_error")


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("%s: %s" % (STATUS.get(status, str(status)), detail))


_lib = None


def load_library():
    """Load libdiffattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libdiffattn.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.diffattn_lambda_init.restype = ctypes.c_double
    lib.diffattn_lambda_init.argtypes = [I]
    lib.diffattn_lambda.restype = I
    lib.diffattn_lambda.argtypes = [P, P, P, P, I, I, I, P, P]
    lib.diffattn_prefill.restype = I
    lib.diffattn_prefill.argtypes = [P, P, P, P, P, L, L, L, I, I, I, I, I, I, I, P, I, F, F, P,
                                     P, P]
    lib.diffattn_prefill_v2.restype = I
    lib.diffattn_prefill_v2.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, P]
    lib.diffattn_attention.restype = I
    lib.diffattn_attention.argtypes = [P, P, P, L, L, L, I, I, I, I, I, I, I, P, P]
    lib.diffattn_combine.restype = I
    lib.diffattn_combine.argtypes = [P, P, P, I, I, I, I, I, F, F, P, P, P]
    lib.diffattn_decode_workspace_bytes.restype = S
    lib.diffattn_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.diffattn_decode.restype = I
    lib.diffattn_decode.argtypes = [P, P, P, P, I, I, I, I, I, P, P, S, P, P]
    lib.diffattn_attention_decode.restype = I
    lib.diffattn_attention_decode.argtypes = [P, P, P, P, I, I, I, I, I, P, S, P, P]
    lib.diffattn_decode_noalloc.restype = I
    lib.diffattn_decode_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P]
    lib.diffattn_decode_v1_workspace_bytes.restype = S
    lib.diffattn_decode_v1_workspace_bytes.argtypes = [I, I, I]
    lib.diffattn_decode_v1.restype = I
    lib.diffattn_decode_v1.argtypes = [P, P, P, P, I, I, I, I, I, P, I, F, F, P, P, S, P, P]
    lib.diffattn_status_string.restype = ctypes.c_char_p
    lib.diffattn_status_string.argtypes = [I]
    lib.diffattn_last_error.restype = ctypes.c_char_p
    lib.diffattn_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise DiffAttnError(status, load_library().diffattn_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _same_device(*named):
    """All tensors on one device (the kernels address them from one GPU)."""
    dev = None
    for t, name in named:
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, expected %s like the other tensors" % (name, t.device, dev))


def _check_lambda(lam, n: int, what: str = "H"):
    if not isinstance(lam, torch.Tensor) or lam.dtype != torch.float32 or lam.numel() != n \
            or not lam.is_contiguous():
        raise ValueError("lambda must be a contiguous fp32 tensor of %s = %d entries" % (what, n))


def _token_stride(t: torch.Tensor, name: str) -> int:
    """ld of a [B, H, N, w] tensor laid out as [B][H][N][ld] with unit channel stride."""
    if t.dim() != 4:
        raise ValueError("%s must be [B, H, N, width]" % name)
    B, H, N, w = t.shape
    sb, sh, sn, sc = t.stride()
    if sc != 1 and w > 1:
        raise ValueError("%s must have unit stride along its last dimension" % name)
    ld = sn
    if (H > 1 and sh != N * ld) or (B > 1 and sb != H * N * ld):
        raise ValueError("%s must be laid out [B][H][N][ld] (head stride N*ld)" % name)
    return ld


# --------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------

def diffattn_lambda_init(layer: int) -> float:
    return float(load_library().diffattn_lambda_init(int(layer)))


def diffattn_lambda(lq1, lk1, lq2, lk2, layer: int, out=None, stream=None) -> torch.Tensor:
    """Per-head lambda, fp32 [H]; inputs fp32 [H, dim] on the GPU."""
    lib = load_library()
    for t in (lq1, lk1, lq2, lk2):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != lq1.shape:
            raise ValueError("lq1, lk1, lq2, lk2 must be contiguous fp32 tensors of one shape")
    if lq1.dim() not in (1, 2):
        raise ValueError("lq1, lk1, lq2, lk2 must be [H, dim] or [dim]")
    H, dim = (1, lq1.shape[0]) if lq1.dim() == 1 else lq1.shape
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=lq1.device)
    if out.dtype != torch.float32 or out.numel() != H or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor of H = %d entries" % H)
    _same_device((lq1, "lq1"), (lk1, "lk1"), (lq2, "lq2"), (lk2, "lk2"), (out, "out"))
    _check(lib.diffattn_lambda(_ptr(lq1), _ptr(lk1), _ptr(lq2), _ptr(lk2), H, dim, int(layer),
                               _ptr(out), _stream(stream)))
    return out


def diffattn_prefill(q1, q2, k1, k2, v, lam, *, causal: bool = True, rmsnorm: bool = False,
                     eps: float = 1e-5, norm_scale: float = 1.0, norm_weight=None, out=None,
                     stream=None) -> torch.Tensor:
    """Fused differential-attention prefill; returns fp32 [B, H, N, dv].

    q1, q2, k1, k2: [B, H, N, d] views (e.g. halves of a packed [B, H, N, 2d]
    tensor), v: [B, H, N, dv], all fp32 or all bf16; lam: fp32 [H].
    """
    lib = load_library()
    if q1.dtype == torch.bfloat16:
        dt = DIFFATTN_BF16
    elif q1.dtype == torch.float32:
        dt = DIFFATTN_FP32
    else:
        raise ValueError("prefill inputs must be bf16 or fp32")
    for t in (q2, k1, k2, v):
        if t.dtype != q1.dtype:
            raise ValueError("q1, q2, k1, k2, v must share one dtype")
    B, H, N, d = q1.shape
    dv = v.shape[-1]
    for t, name in ((q2, "q2"), (k1, "k1"), (k2, "k2")):
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError("%s must be [B, H, N, d] like q1" % name)
    if tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("v must be [B, H, N, dv]")
    ldq, ldq2 = _token_stride(q1, "q1"), _token_stride(q2, "q2")
    ldk, ldk2 = _token_stride(k1, "k1"), _token_stride(k2, "k2")
    ldv = _token_stride(v, "v")
    if ldq != ldq2 or ldk != ldk2:
        raise ValueError("q1/q2 and k1/k2 must share their token strides")
    _check_lambda(lam, H)
    if rmsnorm and norm_weight is not None and (norm_weight.dtype != torch.float32
                                                or norm_weight.numel() != dv):
        raise ValueError("norm_weight must be fp32 [dv]")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=torch.float32, device=q1.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H, N, dv) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, H, N, dv]")
    _same_device((q1, "q1"), (q2, "q2"), (k1, "k1"), (k2, "k2"), (v, "v"), (lam, "lambda"),
                 (norm_weight if rmsnorm else None, "norm_weight"), (out, "out"))
    _check(lib.diffattn_prefill(_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), ldq, ldk, ldv, dt,
                                B, H, N, d, dv, int(bool(causal)), _ptr(lam), int(bool(rmsnorm)),
                                float(eps), float(norm_scale), _ptr(norm_weight), _ptr(out),
                                _stream(stream)))
    return out


def diffattn_prefill_packed(q, k, v, lam, **kw) -> torch.Tensor:
    """Prefill on packed V1 tensors q, k: [B, H, N, 2d] (halves Q1|Q2, K1|K2)."""
    d = q.shape[-1] // 2
    return diffattn_prefill(q[..., :d], q[..., d:], k[..., :d], k[..., d:], v, lam, **kw)


def diffattn_prefill_v2(q, k, v, lam, *, causal: bool = True, out=None, stream=None) -> torch.Tensor:
    """V2-layout prefill; returns fp32 [B, Hq/2, N, D].

    q: [B, Hq, N, D]; k, v: [B, Hkv, N, D] (bf16 or fp32, contiguous);
    lam: fp32 [Hq/2].  Pair p uses query heads 2p and 2p+1 over K/V head
    p // (Hq // (2*Hkv)).
    """
    lib = load_library()
    if q.dtype == torch.bfloat16:
        dtype = DIFFATTN_BF16
    elif q.dtype == torch.float32:
        dtype = DIFFATTN_FP32
    else:
        raise ValueError("q must be bf16 or fp32")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != q.dtype or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("%s must be a contiguous 4-d tensor of q's dtype" % name)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, D) or v.shape != (B, Hkv, N, D):
        raise ValueError("k and v must be [B, Hkv, N, D]")
    _check_lambda(lam, Hq // 2, "Hq/2")
    if out is None:
        out = torch.empty((B, Hq // 2, N, D), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq // 2, N, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, Hq/2, N, D]")
    _same_device((q, "q"), (k, "k"), (v, "v"), (lam, "lambda"), (out, "out"))
    _check(lib.diffattn_prefill_v2(_ptr(q), _ptr(k), _ptr(v), dtype, B, Hq, Hkv, N, D,
                                   1 if causal else 0, _ptr(lam), _ptr(out), _stream(stream)))
    return out


def diffattn_attention(q, k, v, *, causal: bool = True, out=None, stream=None) -> torch.Tensor:
    """Plain softmax attention softmax(q k^T / sqrt d) v; q, k: [B, H, N, d]
    and v: [B, H, N, dv] bf16 views with unit channel stride; returns fp32
    [B, H, N, dv]."""
    lib = load_library()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16:
            raise ValueError("%s must be bf16" % name)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("k must be [B, H, N, d] like q and v [B, H, N, dv]")
    ldq, ldk, ldv = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H, N, dv) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, H, N, dv]")
    _same_device((q, "q"), (k, "k"), (v, "v"), (out, "out"))
    _check(lib.diffattn_attention(_ptr(q), _ptr(k), _ptr(v), ldq, ldk, ldv, DIFFATTN_BF16, B, H, N,
                                  d, dv, 1 if causal else 0, _ptr(out), _stream(stream)))
    return out


def diffattn_combine(o1, o2, lam, *, rmsnorm: bool = False, eps: float = 1e-5,
                     norm_scale: float = 1.0, norm_weight=None, out=None,
                     stream=None) -> torch.Tensor:
    """out = o1 - lambda_h o2 (+ optional RMS norm) on contiguous fp32 [B, H, N, dv]."""
    lib = load_library()
    for t, name in ((o1, "o1"), (o2, "o2")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != o1.shape:
            raise ValueError("%s must be contiguous fp32 of one shape" % name)
    B, H, N, dv = o1.shape
    _check_lambda(lam, H)
    if out is None:
        out = torch.empty_like(o1)
    if out.dtype != torch.float32 or out.shape != o1.shape or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 of o1's shape")
    if rmsnorm and norm_weight is not None and (norm_weight.dtype != torch.float32
                                                or norm_weight.numel() != dv):
        raise ValueError("norm_weight must be fp32 [dv]")
    _same_device((o1, "o1"), (o2, "o2"), (lam, "lambda"),
                 (norm_weight if rmsnorm else None, "norm_weight"), (out, "out"))
    _check(lib.diffattn_combine(_ptr(o1), _ptr(o2), _ptr(lam), B, H, N, dv, 1 if rmsnorm else 0,
                                eps, norm_scale, _ptr(norm_weight), _ptr(out), _stream(stream)))
    return out


def diffattn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, max_len: int) -> int:
    return int(load_library().diffattn_decode_workspace_bytes(B, Hq, Hkv, D, max_len))


def diffattn_decode(q, k_cache, v_cache, seq_lens, lam, *, workspace=None, out=None,
                    stream=None) -> torch.Tensor:
    """V2-layout decode; returns fp32 [B, Hq/2, D].

    q: bf16 [B, Hq, D]; k_cache, v_cache: bf16 [B, Hkv, max_len, D]; seq_lens:
    int32 [B]; lam: fp32 [Hq/2]; workspace: optional uint8 device tensor of at
    least diffattn_decode_workspace_bytes(...) bytes.
    """
    lib = load_library()
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be contiguous bf16" % name)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and the caches [B, Hkv, max_len, D]")
    B, Hq, D = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_len, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [B, Hkv, max_len, D] for q [B, Hq, D]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of B = %d entries" % B)
    _check_lambda(lam, Hq // 2, "Hq/2")
    need = diffattn_decode_workspace_bytes(B, Hq, Hkv, D, max_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq // 2, D), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq // 2, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, Hq/2, D]")
    _same_device((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens"),
                 (lam, "lambda"), (workspace, "workspace"), (out, "out"))
    _check(lib.diffattn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, Hq, Hkv,
                               D, max_len, _ptr(lam), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(out),
                               _stream(stream)))
    return out


def diffattn_attention_decode(q, k_cache, v_cache, seq_lens, *, workspace=None, out=None,
                              stream=None) -> torch.Tensor:
    """Plain single-map GQA attention decode (the baseline the V2 layout is
    compared with); returns fp32 [B, Hq, D].

    q: bf16 [B, Hq, D]; k_cache, v_cache: bf16 [B, Hkv, max_len, D]; seq_lens:
    int32 [B].  Query head h attends over KV head h // (Hq // Hkv).
    """
    lib = load_library()
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be contiguous bf16" % name)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and the caches [B, Hkv, max_len, D]")
    B, Hq, D = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_len, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [B, Hkv, max_len, D] for q [B, Hq, D]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of B = %d entries" % B)
    need = diffattn_decode_workspace_bytes(B, Hq, Hkv, D, max_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, Hq, D]")
    _same_device((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens"),
                 (workspace, "workspace"), (out, "out"))
    _check(lib.diffattn_attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B,
                                         Hq, Hkv, D, max_len, _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(out),
                                         _stream(stream)))
    return out


DECODE_SCRATCH_BYTES = 16 << 20   # DIFFATTN_DECODE_SCRATCH_BYTES


def diffattn_decode_noalloc(q, k_cache, v_cache, seq_lens, lam, out, stream=None) -> torch.Tensor:
    """V2-layout decode through the allocation-free entry point: partial
    states in the library's fixed per-device scratch, so the caller passes
    ``out`` (fp32 [B, Hq/2, D]) and nothing is allocated.  Calls that overlap
    on one device race on that scratch.  Same tensors as diffattn_decode."""
    lib = load_library()
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be contiguous bf16" % name)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and the caches [B, Hkv, max_len, D]")
    B, Hq, D = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, max_len, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [B, Hkv, max_len, D] for q [B, Hq, D]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of B = %d entries" % B)
    _check_lambda(lam, Hq // 2, "Hq/2")
    if out is None or out.dtype != torch.float32 or tuple(out.shape) != (B, Hq // 2, D) \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [B, Hq/2, D] tensor")
    _same_device((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens"),
                 (lam, "lambda"), (out, "out"))
    _check(lib.diffattn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, Hq,
                                       Hkv, D, max_len, _ptr(lam), _ptr(out), _stream(stream)))
    return out


def diffattn_decode_v1_workspace_bytes(B: int, H: int, max_len: int) -> int:
    return int(load_library().diffattn_decode_v1_workspace_bytes(B, H, max_len))


def diffattn_decode_v1(q, k_cache, v_cache, seq_lens, lam, *, rmsnorm: bool = True,
                       eps: float = 1e-5, norm_scale: float = 1.0, norm_weight=None,
                       workspace=None, out=None, stream=None) -> torch.Tensor:
    """V1-layout decode; returns fp32 [B, H, dv].

    q: bf16 [B, H, 2d] packed [q1 | q2]; k_cache: bf16 [B, H, max_len, 2d]
    packed [k1 | k2]; v_cache: bf16 [B, H, max_len, dv]; seq_lens: int32 [B];
    lam: fp32 [H].  With ``rmsnorm`` the output rows are RMS-normalised and
    scaled by ``norm_scale`` (1 - lambda_init for the V1 head norm).
    """
    lib = load_library()
    B, H, d2 = q.shape
    max_len, dv = k_cache.shape[2], v_cache.shape[-1]
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be contiguous bf16" % name)
    if k_cache.shape != (B, H, max_len, d2) or v_cache.shape[:3] != (B, H, max_len):
        raise ValueError("cache shapes must be [B, H, max_len, 2d] and [B, H, max_len, dv]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 tensor of B = %d entries" % B)
    _check_lambda(lam, H)
    if rmsnorm and norm_weight is not None and (norm_weight.dtype != torch.float32
                                                or norm_weight.numel() != dv):
        raise ValueError("norm_weight must be fp32 [dv]")
    need = diffattn_decode_v1_workspace_bytes(B, H, max_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H, dv) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, H, dv]")
    _same_device((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens"),
                 (lam, "lambda"), (norm_weight if rmsnorm else None, "norm_weight"),
                 (workspace, "workspace"), (out, "out"))
    _check(lib.diffattn_decode_v1(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, H,
                                  d2 // 2, dv, max_len, _ptr(lam), 1 if rmsnorm else 0, eps,
                                  norm_scale, _ptr(norm_weight), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _ptr(out),
                                  _stream(stream)))
    return out
