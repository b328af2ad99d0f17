"""Double-precision CPU oracle for differential attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
built from ``oracle.c`` with gcc) and shares no code with the GPU library.

Every function takes host arrays (numpy, or CPU torch tensors via ``.numpy()``)
holding fp32 values or bf16 bit patterns (uint16), exactly the bytes the GPU
path receives, and returns float64 results.

Pages followed (each function repeats the passage it implements):
  * "差分注意力" (aiknowledge.cn): part 一 "Softmax 的噪声底" and "差分思路",
    part 二 Steps 2-4.
  * "【架构革新】Differential Transformer：用“差分降噪”重塑LLM注意力机制"
    (mcipr.com), section 3: the lambda_init depth schedule.
  * "Understanding Differential Transformer Unchains Pretrained Self-Attentions"
    (Paper-Notes), 关键设计: A_diff = A1 - lambda A2, rows of a softmax sum to 1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .snr import snr_from_weights, snr_closed_form  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# A test may point the wrapper at another build of oracle.c (the mutation
# test builds deliberately broken copies to show the pins catch them).
_LIB_PATH = os.environ.get("DIFFATTN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

FP32 = 0
BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (IEEE double arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_int64
    D = ctypes.c_double
    lib.oracle_lambda_init.restype = D
    lib.oracle_lambda_init.argtypes = [I]
    lib.oracle_lambda.restype = None
    lib.oracle_lambda.argtypes = [P, P, P, P, I, I, I, P]
    lib.oracle_prefill.restype = I
    lib.oracle_prefill.argtypes = [I, P, P, P, P, P, L, L, L, I, I, I, I, I, I, P,
                                   I, D, D, P, P, L, P, I]
    lib.oracle_prefill_weights.restype = I
    lib.oracle_prefill_weights.argtypes = [I, P, P, P, P, L, L, I, I, I, I, I, I, I, I, P, P]
    lib.oracle_decode.restype = I
    lib.oracle_decode.argtypes = [I, P, P, P, P, I, I, I, I, I, P, P, I]
    lib.oracle_default_threads.restype = I
    lib.oracle_default_threads.argtypes = []
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses when asked for 0 (all online host CPUs)."""
    return int(_load().oracle_default_threads())


# --------------------------------------------------------------------------
# Array plumbing (no arithmetic of the method).
# --------------------------------------------------------------------------

def _as_host(x):
    """numpy view of a CPU array-like; torch bf16 tensors become uint16 bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must be host (CPU) arrays")
            if x.dtype == torch.bfloat16:
                return x.contiguous().view(torch.int16).numpy().view(np.uint16)
            return x.contiguous().numpy()
    except ImportError:  # pragma: no cover - torch is present in this image
        pass
    return np.ascontiguousarray(x)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return FP32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle element type must be float32 or bf16 bits (uint16), got %s" % a.dtype)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# --------------------------------------------------------------------------
# lambda
# --------------------------------------------------------------------------

def lambda_init(layer: int) -> float:
    """lambda_init = 0.8 - 0.6 exp(-0.3 (layer - 1)) in double.

    Page "【架构革新】Differential Transformer..." (mcipr.com), section 3.
    """
    return float(_load().oracle_lambda_init(int(layer)))


def compute_lambda(lq1, lk1, lq2, lk2, layer: int) -> np.ndarray:
    """Per-head lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init(layer), fp32 [H].

    Page "差分注意力", part 二 Step 4.  Inputs fp32 [H, dim] (or [dim] for one
    head); dots and exps in double, one rounding to fp32.
    """
    arrs = [np.ascontiguousarray(_as_host(a), dtype=np.float32) for a in (lq1, lk1, lq2, lk2)]
    if arrs[0].ndim == 1:
        arrs = [a.reshape(1, -1) for a in arrs]
    H, dim = arrs[0].shape
    for a in arrs:
        if a.shape != (H, dim):
            raise ValueError("lq1, lk1, lq2, lk2 must share one [H, dim] shape")
    out = np.zeros(H, dtype=np.float32)
    _load().oracle_lambda(*[_ptr(a) for a in arrs], H, dim, int(layer), _ptr(out))
    return out


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

def prefill(q1, q2, k1, k2, v, lam, *, causal: bool = True, rmsnorm: bool = False,
            eps: float = 1e-5, norm_scale: float = 1.0, norm_weight=None, rows=None,
            nthreads: int = 0) -> np.ndarray:
    """Differential attention out = (A1 - lambda A2) V, optionally RMS-normalised.

    q1, q2, k1, k2: [B, H, N, d]; v: [B, H, N, dv]; fp32 or bf16 bits; lam: fp32 [H].
    A1 = softmax(Q1 K1^T / sqrt d), A2 = softmax(Q2 K2^T / sqrt d) -- page
    "差分注意力", part 一 "差分思路" and part 二 Step 2.  With ``rmsnorm`` each
    output row (one head, dv channels) becomes o / sqrt(mean o^2 + eps) * w *
    norm_scale (page "差分注意力", "V1 到 V2 的 diff": per-head RMSNorm after the
    difference; the caller passes norm_scale = 1 - lambda_init).

    rows: None for all [B, H, N] rows (returns [B, H, N, dv]), or flat row
    indices (b*H + h)*N + i (returns [len(rows), dv]).
    """
    q1, q2, k1, k2, v = (_as_host(a) for a in (q1, q2, k1, k2, v))
    dt = _dtype_code(q1)
    for a in (q2, k1, k2, v):
        if _dtype_code(a) != dt:
            raise TypeError("all of q1, q2, k1, k2, v must share one element type")
    B, H, N, d = q1.shape
    dv = v.shape[-1]
    for a in (q2, k1, k2):
        if a.shape != (B, H, N, d):
            raise ValueError("q1, q2, k1, k2 must be [B, H, N, d]")
    if v.shape != (B, H, N, dv):
        raise ValueError("v must be [B, H, N, dv]")
    lam = np.ascontiguousarray(_as_host(lam), dtype=np.float32).reshape(-1)
    if lam.shape != (H,):
        raise ValueError("lambda must have H entries")
    w = None if norm_weight is None else np.ascontiguousarray(_as_host(norm_weight), dtype=np.float32)
    if rows is None:
        r_arr = None
        nrows = B * H * N
        out = np.zeros((B, H, N, dv), dtype=np.float64)
    else:
        r_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = r_arr.size
        out = np.zeros((nrows, dv), dtype=np.float64)
    if nrows == 0:
        return out
    rc = _load().oracle_prefill(dt, _ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v),
                                d, d, dv, B, H, N, d, dv, int(bool(causal)), _ptr(lam),
                                int(bool(rmsnorm)), float(eps), float(norm_scale),
                                None if w is None else _ptr(w),
                                None if r_arr is None else _ptr(r_arr), nrows,
                                _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments (code %d)" % rc)
    return out


def prefill_weights(q1, q2, k1, k2, b: int, h: int, i: int, *, causal: bool = True):
    """The softmax rows A1[i, :] and A2[i, :] of query (b, h, i) as float64 [N] each.

    Used for the signal-to-noise measurement of page "差分注意力", part 二 Step 3.
    """
    q1, q2, k1, k2 = (_as_host(a) for a in (q1, q2, k1, k2))
    dt = _dtype_code(q1)
    B, H, N, d = q1.shape
    a1 = np.zeros(N, dtype=np.float64)
    a2 = np.zeros(N, dtype=np.float64)
    rc = _load().oracle_prefill_weights(dt, _ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), d, d,
                                        B, H, N, d, int(bool(causal)), b, h, i,
                                        _ptr(a1), _ptr(a2))
    if rc != 0:
        raise ValueError("oracle_prefill_weights rejected its arguments (code %d)" % rc)
    return a1, a2


# --------------------------------------------------------------------------
# decode (V2 layout)
# --------------------------------------------------------------------------

def decode(q, k_cache, v_cache, seq_lens, lam, *, nthreads: int = 0) -> np.ndarray:
    """One-token differential attention over a KV cache in the V2 layout.

    q: [B, Hq, D]; k_cache, v_cache: [B, Hkv, Lmax, D]; seq_lens: int32 [B];
    lam: fp32 [Hq/2].  Pair p uses query heads 2p (A1) and 2p+1 (A2) over KV
    head floor(2p / (Hq/Hkv)); key positions 0..L_b-1 are visible.  Returns
    float64 [B, Hq/2, D].  Page "差分注意力", "V1 到 V2 的 diff" (twice the query
    heads over the same KV heads) and part 二 Step 2.
    """
    q, k_cache, v_cache = (_as_host(a) for a in (q, k_cache, v_cache))
    dt = _dtype_code(q)
    if _dtype_code(k_cache) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("q, k_cache, v_cache must share one element type")
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    if k_cache.shape != (B, Hkv, Lmax, D) or v_cache.shape != (B, Hkv, Lmax, D):
        raise ValueError("caches must be [B, Hkv, Lmax, D]")
    lens = np.ascontiguousarray(_as_host(seq_lens), dtype=np.int32).reshape(-1)
    lam = np.ascontiguousarray(_as_host(lam), dtype=np.float32).reshape(-1)
    if lens.shape != (B,) or lam.shape != (Hq // 2,):
        raise ValueError("seq_lens must be [B] and lambda [Hq/2]")
    out = np.zeros((B, Hq // 2, D), dtype=np.float64)
    rc = _load().oracle_decode(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens),
                               B, Hq, Hkv, D, Lmax, _ptr(lam), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments (code %d)" % rc)
    return out
