"""Seeded synthetic inputs for differential attention.

This module only draws and lays out inputs; it holds none of the operator's
arithmetic.  Both the GPU library's callers and the CPU oracle receive the
bytes it produces.

Shapes and structure follow the pages' workloads:
  * unit-variance queries, keys and values, split into two halves per head
    (V1 layout) or twice the query heads over shared KV heads (V2 layout) --
    page "差分注意力" (aiknowledge.cn), "V1 到 V2 的 diff";
  * one strongly matching key per head, built as 5x the probing query --
    page "差分注意力", part 二 Step 1 (the noise-floor probe);
  * many answer positions scattered over a 64k context -- page
    "【架构革新】Differential Transformer..." (mcipr.com), section 4 (20 needles
    at 64k);
  * lambda parameters lq1, lk1, lq2, lk2 drawn with standard deviation 0.1.

Random numbers come from torch's seeded generator on the requested device,
in the fixed order q, k, v, lq1, lk1, lq2, lk2, then the structure (needle
positions, sequence lengths).  bf16 values are fp32 draws rounded to nearest
even.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class PrefillCase:
    """A V1-layout prefill workload: Q and K packed as [B, H, N, 2d] halves."""
    name: str
    dtype: str          # "fp32" or "bf16"
    B: int
    H: int
    N: int
    d: int              # width of each query/key half (the softmax dot length)
    dv: int             # value width
    layer: int          # 1-based layer index for lambda_init
    rmsnorm: bool
    seed: int
    causal: bool = True
    eps: float = 1e-5
    needle: str = "none"   # "none" | "last_query" | "mean_query"
    n_needles: int = 0
    needle_scale: float = 5.0   # needle key = needle_scale x (probing query half)
    # If set, "last_query" needles are instead scaled so that the first-map
    # score q1 . k1 / sqrt(d) of the probing query equals this value in every
    # head (a controlled signal strength for noise-floor sweeps).
    needle_score: Optional[float] = None

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def pairs(self) -> int:
        """Causal (query, key) pairs over all heads (or all pairs if not causal)."""
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * self.H * per_head


@dataclasses.dataclass(frozen=True)
class DecodeCase:
    """A V2-layout decode workload: one query token per sequence over a KV cache."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    Lmin: int
    Lmax: int
    layer: int
    seed: int
    dtype: str = "bf16"

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


@dataclasses.dataclass(frozen=True)
class V2PrefillCase:
    """A V2-layout prefill workload: Hq query heads (pairs 2p, 2p+1) over Hkv
    shared K/V heads, full head width D for both maps, no per-head norm."""
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    layer: int
    seed: int
    causal: bool = True

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def pairs_per_kv(self) -> int:
        return self.Hq // (2 * self.Hkv)

    def pairs(self) -> int:
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * (self.Hq // 2) * per_head


@dataclasses.dataclass(frozen=True)
class V1DecodeCase:
    """A V1-layout decode workload: per head one packed query [q1 | q2] over a
    cache of packed keys [k1 | k2] and values, RMS-normalised output."""
    name: str
    B: int
    H: int
    d: int
    dv: int
    Lmin: int
    Lmax: int
    layer: int
    seed: int
    rmsnorm: bool = True
    eps: float = 1e-5
    dtype: str = "bf16"

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


# The five workloads the operator is specified on.
TINY_FP32 = PrefillCase("tiny_fp32_b1_h2_n128_d32_dv64", "fp32", B=1, H=2, N=128, d=32, dv=64,
                        layer=1, rmsnorm=False, seed=1)
V1_NORM = PrefillCase("v1_norm_bf16_b4_h16_n2048_d64_dv128", "bf16", B=4, H=16, N=2048, d=64,
                      dv=128, layer=6, rmsnorm=True, seed=2)
NEEDLE_32K = PrefillCase("needle_bf16_b1_h16_n32768_d64_dv128", "bf16", B=1, H=16, N=32768,
                         d=64, dv=128, layer=1, rmsnorm=False, seed=3, needle="last_query",
                         n_needles=1)
V2_DECODE = DecodeCase("v2_decode_bf16_b32_hq32_hkv8_d128_l4096_65536", B=32, Hq=32, Hkv=8,
                       D=128, Lmin=4096, Lmax=65536, layer=1, seed=4)
MULTI_NEEDLE_64K = PrefillCase("multineedle_bf16_b1_h32_n65536_d64_dv128", "bf16", B=1, H=32,
                               N=65536, d=64, dv=128, layer=12, rmsnorm=True, seed=5,
                               needle="mean_query", n_needles=20)

# The V2 (production) prefill layout at long context: 16 pairs over 8 K/V
# heads, head width 128 for both maps.
V2_PREFILL_32K = V2PrefillCase("v2_prefill_bf16_b1_hq32_hkv8_n32768_d128", "bf16", B=1, Hq=32,
                               Hkv=8, N=32768, D=128, layer=1, seed=6)

# V1-layout decode: 16 diff heads with their own half-width K1|K2 and V
# caches (twice the cache bytes of the V2 layout's 8 shared KV heads).
V1_DECODE = V1DecodeCase("v1_decode_bf16_b16_h16_d64_dv128_l4096_65536", B=16, H=16, d=64, dv=128,
                         Lmin=4096, Lmax=65536, layer=12, seed=7)

# The V1 layout with the 64k workload's norm at other lengths (no needles), for
# the fused kernel's rate against N: from below the long workloads to twice the
# longest.  Each length takes a different head count, so every launch has its
# own workgroup count (N/256 row tiles per head).
V1_LENGTH_SWEEP = tuple(
    PrefillCase("v1_sweep_bf16_b1_h%d_n%d_d64_dv128" % (h, n), "bf16", B=1, H=h, N=n, d=64,
                dv=128, layer=12, rmsnorm=True, seed=8)
    for n, h in ((4096, 48), (8192, 32), (16384, 24), (131072, 8)))

PREFILL_CASES = {c.name: c for c in (TINY_FP32, V1_NORM, NEEDLE_32K, MULTI_NEEDLE_64K)}
DECODE_CASES = {V2_DECODE.name: V2_DECODE}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device, dtype, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def make_prefill(case: PrefillCase, device="cpu") -> dict:
    """Inputs of one prefill workload.

    Returns q, k: [B, H, N, 2d] (first half Q1/K1, second half Q2/K2), v:
    [B, H, N, dv] in the case's dtype; lq1, lk1, lq2, lk2: fp32 [H, d];
    needles: int64 [H, n] positions (empty if none).
    """
    g = _gen(case.seed, device)
    dt = case.torch_dtype
    B, H, N, d, dv = case.B, case.H, case.N, case.d, case.dv
    q = _normal((B, H, N, 2 * d), g, device, dt)
    k = _normal((B, H, N, 2 * d), g, device, dt)
    v = _normal((B, H, N, dv), g, device, dt)
    lam = [_normal((H, d), g, device, torch.float32, std=0.1) for _ in range(4)]
    needles = torch.zeros((H, 0), dtype=torch.int64)
    if case.needle == "last_query":
        # One position per head whose first-map key is needle_scale x the last
        # query's first-map half (the strong match of the noise-floor probe;
        # the pages use 5x).
        pos = torch.randint(0, N - 1, (H,), generator=g, device=device, dtype=torch.int64)
        for h in range(H):
            p = int(pos[h])
            qh = q[:, h, N - 1, :d].float()
            if case.needle_score is None:
                scale = case.needle_scale
            else:
                scale = case.needle_score * (d ** 0.5) / (qh * qh).sum(dim=-1, keepdim=True)
            k[:, h, p, :d] = (qh * scale).to(dt)
        needles = pos.cpu().reshape(H, 1)
    elif case.needle == "mean_query":
        # n positions shared by every head; first-map key rows = 5x the mean of
        # that head's first-map query rows.
        perm = torch.randperm(N, generator=g, device=device)[: case.n_needles]
        pos = torch.sort(perm).values
        for b in range(B):
            for h in range(H):
                m = q[b, h, :, :d].double().mean(dim=0)
                k[b, h, pos, :d] = (m * case.needle_scale).to(dt).unsqueeze(0).expand(pos.numel(), d)
        needles = pos.cpu().reshape(1, -1).expand(H, -1).contiguous()
    return {"q": q, "k": k, "v": v, "lq1": lam[0], "lk1": lam[1], "lq2": lam[2],
            "lk2": lam[3], "needles": needles}


def make_decode(case: DecodeCase, device="cpu", fill_unused: Optional[float] = None) -> dict:
    """Inputs of one decode workload.

    Returns q: [B, Hq, D]; k_cache, v_cache: [B, Hkv, Lmax, D]; seq_lens: int32
    [B] uniform in [Lmin, Lmax]; lq1, lk1, lq2, lk2: fp32 [Hq/2, D].  With
    ``fill_unused`` the cache slots at positions >= L_b hold that value (e.g.
    NaN, to show they are never read).
    """
    g = _gen(case.seed, device)
    dt = case.torch_dtype
    B, Hq, Hkv, D, L = case.B, case.Hq, case.Hkv, case.D, case.Lmax
    q = _normal((B, Hq, D), g, device, dt)
    kc = torch.empty((B, Hkv, L, D), dtype=dt, device=device)
    vc = torch.empty((B, Hkv, L, D), dtype=dt, device=device)
    for b in range(B):          # per sequence, to bound the fp32 temporaries
        kc[b] = _normal((Hkv, L, D), g, device, dt)
    for b in range(B):
        vc[b] = _normal((Hkv, L, D), g, device, dt)
    lam = [_normal((Hq // 2, D), g, device, torch.float32, std=0.1) for _ in range(4)]
    lens = torch.randint(case.Lmin, case.Lmax + 1, (B,), generator=g, device=device,
                         dtype=torch.int64).to(torch.int32)
    if fill_unused is not None:
        for b in range(B):
            kc[b, :, int(lens[b]):, :] = fill_unused
            vc[b, :, int(lens[b]):, :] = fill_unused
    return {"q": q, "k_cache": kc, "v_cache": vc, "seq_lens": lens, "lq1": lam[0],
            "lk1": lam[1], "lq2": lam[2], "lk2": lam[3]}


def make_prefill_v2(case: V2PrefillCase, device="cpu") -> dict:
    """Inputs of one V2 prefill workload: q [B, Hq, N, D]; k, v [B, Hkv, N, D];
    lq1, lk1, lq2, lk2 fp32 [Hq/2, D]."""
    g = _gen(case.seed, device)
    dt = case.torch_dtype
    q = _normal((case.B, case.Hq, case.N, case.D), g, device, dt)
    k = _normal((case.B, case.Hkv, case.N, case.D), g, device, dt)
    v = _normal((case.B, case.Hkv, case.N, case.D), g, device, dt)
    lam = [_normal((case.Hq // 2, case.D), g, device, torch.float32, std=0.1) for _ in range(4)]
    return {"q": q, "k": k, "v": v, "lq1": lam[0], "lk1": lam[1], "lq2": lam[2], "lk2": lam[3]}


def make_decode_v1(case: V1DecodeCase, device="cpu") -> dict:
    """Inputs of one V1 decode workload: q [B, H, 2d]; k_cache [B, H, Lmax, 2d];
    v_cache [B, H, Lmax, dv]; seq_lens int32 [B] uniform in [Lmin, Lmax];
    lq1, lk1, lq2, lk2 fp32 [H, d]."""
    g = _gen(case.seed, device)
    dt = case.torch_dtype
    B, H, d, dv, L = case.B, case.H, case.d, case.dv, case.Lmax
    q = _normal((B, H, 2 * d), g, device, dt)
    kc = torch.empty((B, H, L, 2 * d), dtype=dt, device=device)
    vc = torch.empty((B, H, L, dv), dtype=dt, device=device)
    for b in range(B):
        kc[b] = _normal((H, L, 2 * d), g, device, dt)
    for b in range(B):
        vc[b] = _normal((H, L, dv), g, device, dt)
    lam = [_normal((H, d), g, device, torch.float32, std=0.1) for _ in range(4)]
    lens = torch.randint(case.Lmin, case.Lmax + 1, (B,), generator=g, device=device,
                         dtype=torch.int64).to(torch.int32)
    return {"q": q, "k_cache": kc, "v_cache": vc, "seq_lens": lens, "lq1": lam[0],
            "lk1": lam[1], "lq2": lam[2], "lk2": lam[3]}


def scaled_prefill(case: PrefillCase, **changes) -> PrefillCase:
    """A copy of a workload with some fields changed (smaller parity sizes)."""
    return dataclasses.replace(case, **changes)


def scaled_decode(case: DecodeCase, **changes) -> DecodeCase:
    return dataclasses.replace(case, **changes)
