"""Signal-to-noise of differential vs plain attention, read off the fused
prefill kernel (page "差分注意力" (aiknowledge.cn), part 二 Step 3 and the
exercises of part 五: the noise floor of softmax attention and how the
difference lowers it as the context grows).

The kernel is run with probe values instead of real ones: column c of V is
the indicator of marked position c and the last column is all ones.  Row i of
the output is then sum_j w_ij v_j, i.e. the weight of query i on each marked
position, and the row's total weight (1 - lambda for A1 - lambda A2, 1 for a
softmax).  Running it once with the head's lambda and once with lambda = 0
(plain softmax A1) gives both sides of the comparison for the last query:

    SNR = w[signal] * (n_visible - 1) / (total - w[signal])

(the signal weight over the mean weight of the other visible positions).
Everything here is argument marshalling around diffattn_prefill.
"""
from __future__ import annotations

import torch

from . import api

PROBE_DV = 64     # value width of the probe (a supported (d, dv) = (64, 64) shape)


def probe_weights(q, k, lam, positions, *, causal: bool = True) -> dict:
    """Weights of the last query of every head on the marked positions.

    q, k: bf16 [1, H, N, 2d] packed V1 tensors (d = 64); lam: fp32 [H];
    positions: int64 [H, n] (n <= 63) marked key positions per head.
    Returns dict of fp64 CPU tensors: ``diff`` [H, n] and ``diff_total`` [H]
    for A1 - lambda A2, ``plain`` [H, n] and ``plain_total`` [H] for A1.
    """
    B, H, N, d2 = q.shape
    if B != 1 or d2 != 128:
        raise ValueError("probe expects B = 1 and d = 64")
    n = positions.shape[1]
    if n > PROBE_DV - 1:
        raise ValueError("at most %d marked positions" % (PROBE_DV - 1))
    v = torch.zeros((1, H, N, PROBE_DV), dtype=torch.bfloat16, device=q.device)
    pos = positions.to(q.device)
    for h in range(H):
        v[0, h, pos[h], torch.arange(n, device=q.device)] = 1.0
    v[..., PROBE_DV - 1] = 1.0
    res = {}
    for name, lam_used in (("diff", lam), ("plain", torch.zeros_like(lam))):
        out = api.diffattn_prefill_packed(q, k, v, lam_used, causal=causal)
        last = out[0, :, N - 1, :].double().cpu()
        res[name] = last[:, :n]
        res[name + "_total"] = last[:, PROBE_DV - 1]
    return res


def snr_last_query(q, k, lam, signal, *, causal: bool = True) -> dict:
    """SNR of the last query towards one signal position per head.

    signal: int64 [H].  Returns fp64 CPU tensors ``plain`` and ``diff`` [H].
    """
    N = q.shape[2]
    w = probe_weights(q, k, lam, signal.reshape(-1, 1), causal=causal)
    out = {}
    for name in ("plain", "diff"):
        s = w[name][:, 0]
        out[name] = s * (N - 1) / (w[name + "_total"] - s)
    return out


def noise_sweep_point(q, k, lam, signal, *, causal: bool = True) -> dict:
    """One point of the noise-floor sweep for the last query of every head:
    the share of the row's total weight on the signal position and on all
    other positions (the noise floor), for A1 - lambda A2 and for A1, and
    the SNRs.  Fp64 CPU tensors [H] keyed plain_signal, plain_noise, diff_signal,
    diff_noise, plain_snr, diff_snr."""
    N = q.shape[2]
    w = probe_weights(q, k, lam, signal.reshape(-1, 1), causal=causal)
    out = {}
    for name in ("plain", "diff"):
        s = w[name][:, 0]
        t = w[name + "_total"]
        out[name + "_signal"] = s / t
        out[name + "_noise"] = (t - s) / t
        out[name + "_snr"] = s * (N - 1) / (t - s)
    return out


def needle_mass(q, k, lam, needles, *, causal: bool = True) -> dict:
    """Fraction of the last query's total weight that falls on the needles,
    per head, for A1 - lambda A2 and for A1.  needles: int64 [H, n]."""
    w = probe_weights(q, k, lam, needles, causal=causal)
    return {name: w[name].sum(dim=1) / w[name + "_total"] for name in ("plain", "diff")}
