"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these re-types the oracle's formula: each checks it against a
hand-worked rational example, a textbook routine it must reduce to (torch's
float64 scaled-dot-product attention), a closed form, an invariant, or a brute
force computed a different way.  All run on the CPU.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _num(x):
    if isinstance(x, str):
        return {"ln2": math.log(2.0), "ln4": math.log(4.0), "ln8": math.log(8.0)}[x]
    return float(x)


def _frac(s: str) -> float:
    if "sqrt" in s:
        coef, rest = s.split("*sqrt(")
        num, den = rest.rstrip(")").split("/")
        return float(coef) * math.sqrt(float(num) / float(den))
    return float(Fraction(s))


def _arr(nested, dtype=np.float32):
    return np.array([[_num(x) for x in row] for row in nested], dtype=dtype)


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * scale).astype(np.float32)


def _sdpa(q, k, v, causal, scale):
    """torch float64 SDPA on [B, H, N, *] numpy arrays."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal,
                                          scale=scale).numpy()


# ---------------------------------------------------------------------------
# lambda_init and lambda
# ---------------------------------------------------------------------------

def test_lambda_init_first_layer_and_limit(oracle_mod):
    # 0.8 - 0.6 * exp(0) = 0.2 at the first layer; tends to 0.8 with depth.
    assert abs(oracle_mod.lambda_init(1) - 0.2) < 1e-15
    assert abs(oracle_mod.lambda_init(400) - 0.8) < 1e-15
    vals = [oracle_mod.lambda_init(l) for l in range(1, 40)]
    assert all(b > a for a, b in zip(vals, vals[1:]))


def test_lambda_init_decay_rate(oracle_mod):
    # The gap to 0.8 shrinks by exp(-0.3) per layer.
    for layer in (1, 2, 6, 11):
        gap0 = 0.8 - oracle_mod.lambda_init(layer)
        gap1 = 0.8 - oracle_mod.lambda_init(layer + 1)
        assert abs(gap1 / gap0 - math.exp(-0.3)) < 1e-12


def test_lambda_equal_halves_give_lambda_init(oracle_mod):
    a = _rand((5, 32), 1, 0.1)
    b = _rand((5, 32), 2, 0.1)
    lam = oracle_mod.compute_lambda(a, b, a, b, layer=6)
    assert np.all(lam == np.float32(oracle_mod.lambda_init(6)))


def test_lambda_hand_values_and_sign(oracle_mod):
    # head 0: lq1.lk1 = ln 3, lq2.lk2 = 0      -> 3 - 1 + 0.2 = 2.2
    # head 1: lq1.lk1 = 0,    lq2.lk2 = ln 3   -> 1 - 3 + 0.2 = -1.8 (negative allowed)
    # head 2: lq1.lk1 = ln 2, lq2.lk2 = ln 1.5 -> 2 - 1.5 + 0.2 = 0.7; each vector
    #         lives on its own coordinate so a mis-paired dot product gives 0.
    lq1 = np.zeros((3, 4), np.float32); lk1 = np.zeros((3, 4), np.float32)
    lq2 = np.zeros((3, 4), np.float32); lk2 = np.zeros((3, 4), np.float32)
    lq1[0, 0], lk1[0, 0] = 1.0, math.log(3.0)
    lq2[1, 1], lk2[1, 1] = 1.0, math.log(3.0)
    lq1[2, 0], lk1[2, 0] = 0.5, 2 * math.log(2.0)
    lq2[2, 2], lk2[2, 2] = 2.0, 0.5 * math.log(1.5)
    lam = oracle_mod.compute_lambda(lq1, lk1, lq2, lk2, layer=1)
    np.testing.assert_allclose(lam, [2.2, -1.8, 0.7], atol=1e-6)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_hand_worked(oracle_mod, causal):
    g = _golden()["prefill"]
    r = lambda a: _arr(a).reshape(1, 1, 3, -1)
    out = oracle_mod.prefill(r(g["q1"]), r(g["q2"]), r(g["k1"]), r(g["k2"]), r(g["v"]),
                             np.array([g["lambda"]], np.float32), causal=causal)
    key = "causal_out" if causal else "noncausal_out"
    want = np.array([[_frac(x) for x in row] for row in g[key]])
    np.testing.assert_allclose(out[0, 0], want, atol=1e-7)


def test_prefill_hand_worked_rmsnorm(oracle_mod):
    g = _golden()["prefill"]
    r = lambda a: _arr(a).reshape(1, 1, 3, -1)
    out = oracle_mod.prefill(r(g["q1"]), r(g["q2"]), r(g["k1"]), r(g["k2"]), r(g["v"]),
                             np.array([g["lambda"]], np.float32), causal=True,
                             rmsnorm=True, eps=0.0, norm_scale=1.0)
    want = [_frac(x) for x in g["causal_rmsnorm_row2"]]
    np.testing.assert_allclose(out[0, 0, 2], want, atol=1e-7)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_lambda_zero_is_softmax_attention(oracle_mod, causal):
    # lambda = 0 leaves A1 V: torch's float64 SDPA with scale 1/sqrt(d).
    B, H, N, d, dv = 2, 3, 37, 16, 24
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (1, 2, 3, 4))
    v = _rand((B, H, N, dv), 5)
    out = oracle_mod.prefill(q1, q2, k1, k2, v, np.zeros(H, np.float32), causal=causal)
    ref = _sdpa(q1, k1, v, causal, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_is_difference_of_two_attentions(oracle_mod, causal):
    # (A1 - lam A2) V = A1 V - lam (A2 V) by linearity; each term is SDPA.
    B, H, N, d, dv = 2, 4, 29, 8, 12
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (11, 12, 13, 14))
    v = _rand((B, H, N, dv), 15)
    lam = np.array([0.3, -0.7, 1.5, 0.0], np.float32)
    out = oracle_mod.prefill(q1, q2, k1, k2, v, lam, causal=causal)
    sc = 1.0 / math.sqrt(d)
    ref = _sdpa(q1, k1, v, causal, sc) - lam.astype(np.float64)[None, :, None, None] * \
        _sdpa(q2, k2, v, causal, sc)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_prefill_identical_maps_lambda_one_is_zero(oracle_mod):
    B, H, N, d, dv = 1, 2, 33, 16, 16
    q, k = _rand((B, H, N, d), 21), _rand((B, H, N, d), 22)
    v = _rand((B, H, N, dv), 23)
    out = oracle_mod.prefill(q, q, k, k, v, np.ones(H, np.float32), causal=True)
    assert np.all(out == 0.0)


def test_prefill_rows_sum_to_one_minus_lambda(oracle_mod):
    # A value column of ones reads off the row sums of A1 - lam A2: 1 - lam.
    B, H, N, d = 2, 3, 40, 16
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (31, 32, 33, 34))
    v = np.ones((B, H, N, 4), np.float32)
    lam = np.array([0.2, 0.9, -0.4], np.float32)
    out = oracle_mod.prefill(q1, q2, k1, k2, v, lam, causal=True)
    want = (1.0 - lam.astype(np.float64))[None, :, None, None]
    np.testing.assert_allclose(out, np.broadcast_to(want, out.shape), atol=1e-12)


def test_prefill_single_token(oracle_mod):
    # N = 1: both maps put weight 1 on the only key: out = (1 - lam) v0.
    q1, q2, k1, k2 = (_rand((1, 2, 1, 8), s) for s in (41, 42, 43, 44))
    v = _rand((1, 2, 1, 8), 45)
    lam = np.array([0.25, -2.0], np.float32)
    out = oracle_mod.prefill(q1, q2, k1, k2, v, lam)
    np.testing.assert_allclose(out[0, :, 0], (1 - lam[:, None]) * v[0, :, 0].astype(np.float64),
                               atol=1e-15)


def test_prefill_two_tokens_sigmoid(oracle_mod):
    # Row 1 of a causal 2-token head: softmax over two scores is a logistic.
    d = 8
    q1, q2, k1, k2 = (_rand((1, 1, 2, d), s) for s in (51, 52, 53, 54))
    v = _rand((1, 1, 2, 3), 55)
    lam = np.float32(0.6)
    out = oracle_mod.prefill(q1, q2, k1, k2, v, np.array([lam]))
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    dot = lambda a, b: float(np.dot(a.astype(np.float64), b.astype(np.float64)))
    s1 = [dot(q1[0, 0, 1], k1[0, 0, j]) / math.sqrt(d) for j in (0, 1)]
    s2 = [dot(q2[0, 0, 1], k2[0, 0, j]) / math.sqrt(d) for j in (0, 1)]
    w0 = sig(s1[0] - s1[1]) - float(lam) * sig(s2[0] - s2[1])
    w1 = sig(s1[1] - s1[0]) - float(lam) * sig(s2[1] - s2[0])
    want = w0 * v[0, 0, 0].astype(np.float64) + w1 * v[0, 0, 1].astype(np.float64)
    np.testing.assert_allclose(out[0, 0, 1], want, atol=1e-14)


def test_prefill_brute_force_longdouble(oracle_mod):
    # Explicit full matrices in extended precision, no maximum shift.
    B, H, N, d, dv = 1, 2, 7, 4, 5
    q1, q2, k1, k2 = (_rand((B, H, N, d), s, 0.7) for s in (61, 62, 63, 64))
    v = _rand((B, H, N, dv), 65)
    lam = np.array([0.45, -0.3], np.float32)
    out = oracle_mod.prefill(q1, q2, k1, k2, v, lam, causal=True)
    L = np.longdouble
    mask = np.tril(np.ones((N, N), dtype=bool))
    for h in range(H):
        def amap(q, k):
            e = np.exp(q[0, h].astype(L) @ k[0, h].astype(L).T / np.sqrt(L(d)))
            e = np.where(mask, e, L(0))
            return e / e.sum(axis=1, keepdims=True)
        w = amap(q1, k1) - L(lam[h]) * amap(q2, k2)
        ref = w @ v[0, h].astype(L)
        np.testing.assert_allclose(out[0, h].astype(L), ref, atol=1e-13)


def test_prefill_causality(oracle_mod):
    # Changing keys/values after position i leaves rows <= i bit-identical.
    B, H, N, d, dv = 1, 2, 24, 8, 8
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (71, 72, 73, 74))
    v = _rand((B, H, N, dv), 75)
    lam = np.array([0.5, 0.1], np.float32)
    base = oracle_mod.prefill(q1, q2, k1, k2, v, lam)
    i = 11
    k1b, k2b, vb = k1.copy(), k2.copy(), v.copy()
    k1b[:, :, i + 1:] += 3.0
    k2b[:, :, i + 1:] -= 2.0
    vb[:, :, i + 1:] *= -5.0
    pert = oracle_mod.prefill(q1, q2, k1b, k2b, vb, lam)
    assert np.array_equal(base[:, :, : i + 1], pert[:, :, : i + 1])
    assert not np.array_equal(base[:, :, i + 1:], pert[:, :, i + 1:])


def test_prefill_rmsnorm_invariants(oracle_mod):
    # RMS of y = |s| sqrt(ms / (ms + eps)); y parallel to o (times weight).
    B, H, N, d, dv = 1, 2, 19, 8, 32
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (81, 82, 83, 84))
    v = _rand((B, H, N, dv), 85)
    lam = np.array([0.3, 0.7], np.float32)
    wgt = (1.0 + 0.5 * _rand((dv,), 86)).astype(np.float32)
    o = oracle_mod.prefill(q1, q2, k1, k2, v, lam)
    scale, eps = 0.3338780, 1e-5
    y = oracle_mod.prefill(q1, q2, k1, k2, v, lam, rmsnorm=True, eps=eps, norm_scale=scale)
    ms = (o ** 2).mean(axis=-1)
    rms_y = np.sqrt((y ** 2).mean(axis=-1))
    np.testing.assert_allclose(rms_y, abs(scale) * np.sqrt(ms / (ms + eps)), rtol=1e-12)
    ratio = y / o
    np.testing.assert_allclose(ratio, np.broadcast_to(ratio[..., :1], ratio.shape), rtol=1e-12)
    yw = oracle_mod.prefill(q1, q2, k1, k2, v, lam, rmsnorm=True, eps=eps, norm_scale=scale,
                            norm_weight=wgt)
    np.testing.assert_allclose(yw, y * wgt.astype(np.float64), rtol=1e-12, atol=1e-15)


def test_prefill_bf16_bits_equal_widened_fp32(oracle_mod):
    # bf16 inputs are read as the exact fp32 values they encode.
    B, H, N, d, dv = 1, 2, 21, 16, 16
    t = [torch.from_numpy(_rand((B, H, N, d if i < 4 else dv), 90 + i)).to(torch.bfloat16)
         for i in range(5)]
    lam = np.array([0.4, -0.1], np.float32)
    out_bf = oracle_mod.prefill(*t, lam)
    out_f32 = oracle_mod.prefill(*[x.float() for x in t], lam)
    assert np.array_equal(out_bf, out_f32)


def test_prefill_row_subset_matches_full(oracle_mod):
    B, H, N, d, dv = 2, 3, 17, 8, 8
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (101, 102, 103, 104))
    v = _rand((B, H, N, dv), 105)
    lam = np.array([0.1, 0.2, 0.3], np.float32)
    full = oracle_mod.prefill(q1, q2, k1, k2, v, lam)
    rows = np.array([0, 5, 16, 17, 40, B * H * N - 1], np.int64)
    sub = oracle_mod.prefill(q1, q2, k1, k2, v, lam, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, dv)[rows])


def test_prefill_weights_rows(oracle_mod):
    # Weights rows match torch's float64 softmax and zero out masked keys.
    B, H, N, d = 1, 2, 30, 8
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (111, 112, 113, 114))
    a1, a2 = oracle_mod.prefill_weights(q1, q2, k1, k2, 0, 1, 12)
    s = torch.from_numpy(k1[0, 1, :13].astype(np.float64)) @ \
        torch.from_numpy(q1[0, 1, 12].astype(np.float64)) / math.sqrt(d)
    np.testing.assert_allclose(a1[:13], torch.softmax(s, 0).numpy(), atol=1e-15)
    assert np.all(a1[13:] == 0) and np.all(a2[13:] == 0)
    assert abs(a2.sum() - 1.0) < 1e-14


# ---------------------------------------------------------------------------
# decode (V2 layout)
# ---------------------------------------------------------------------------

def test_decode_hand_worked(oracle_mod):
    g = _golden()["decode"]
    s = g["shape"]
    q = _arr(g["q"]).reshape(1, s["Hq"], s["D"])
    kc = np.stack([_arr(x) for x in g["k_cache"]]).reshape(1, s["Hkv"], s["Lmax"], s["D"])
    vc = np.stack([_arr(x) for x in g["v_cache"]]).reshape(1, s["Hkv"], s["Lmax"], s["D"])
    out = oracle_mod.decode(q, kc, vc, np.array([s["L"]], np.int32),
                            np.array(g["lambda"], np.float32))
    want = np.array([[[_frac(x) for x in row] for row in pair] for pair in g["out"]])
    np.testing.assert_allclose(out, want, atol=1e-7)


def test_decode_is_difference_of_two_attentions(oracle_mod):
    # Per pair: SDPA(q_2p, K_g, V_g) - lam_p SDPA(q_2p+1, K_g, V_g) over L_b keys.
    B, Hq, Hkv, D, Lmax = 3, 8, 2, 16, 23
    q = _rand((B, Hq, D), 121)
    kc, vc = _rand((B, Hkv, Lmax, D), 122), _rand((B, Hkv, Lmax, D), 123)
    lens = np.array([23, 1, 9], np.int32)
    lam = np.array([0.2, -0.5, 0.9, 1.3], np.float32)
    out = oracle_mod.decode(q, kc, vc, lens, lam)
    grp = Hq // Hkv
    for b in range(B):
        for p in range(Hq // 2):
            gidx = (2 * p) // grp
            K = kc[b, gidx, : lens[b]][None, None]
            V = vc[b, gidx, : lens[b]][None, None]
            a = _sdpa(q[b, 2 * p][None, None, None], K, V, False, 1 / math.sqrt(D))
            c = _sdpa(q[b, 2 * p + 1][None, None, None], K, V, False, 1 / math.sqrt(D))
            np.testing.assert_allclose(out[b, p], (a - float(lam[p]) * c).reshape(-1),
                                       atol=1e-12)


def test_decode_equals_last_prefill_row(oracle_mod):
    # A decode query at position L-1 over the cache is the last row of a causal
    # prefill whose query halves are the pair's two heads.
    B, Hq, Hkv, D, L = 1, 4, 1, 8, 13
    q = _rand((B, Hq, D), 131)
    kc, vc = _rand((B, Hkv, L, D), 132), _rand((B, Hkv, L, D), 133)
    lam = np.array([0.35, -0.25], np.float32)
    out = oracle_mod.decode(q, kc, vc, np.array([L], np.int32), lam)
    for p in range(2):
        q1 = np.zeros((1, 1, L, D), np.float32); q2 = np.zeros_like(q1)
        q1[0, 0, -1], q2[0, 0, -1] = q[0, 2 * p], q[0, 2 * p + 1]
        k = kc[:, :1]
        row = oracle_mod.prefill(q1, q2, k, k, vc[:, :1], lam[p:p + 1],
                                 rows=[L - 1])
        np.testing.assert_allclose(out[0, p], row[0], atol=1e-14)


# ---------------------------------------------------------------------------
# signal-to-noise (page part 二 Step 3)
# ---------------------------------------------------------------------------

def test_snr_closed_form_matches_direct(oracle_mod):
    B, H, N, d = 1, 1, 50, 16
    q1, q2, k1, k2 = (_rand((B, H, N, d), s) for s in (141, 142, 143, 144))
    a1, a2 = oracle_mod.prefill_weights(q1, q2, k1, k2, 0, 0, N - 1)
    direct = oracle_mod.snr_from_weights(a1, a2, 0.4, signal=7, visible=N)
    closed = oracle_mod.snr_closed_form(a1[7], a2[7], 0.4, visible=N)
    assert abs(direct["plain"] / closed["plain"] - 1) < 1e-10
    assert abs(direct["diff"] / closed["diff"] - 1) < 1e-10


def test_snr_signal_plus_noise_improves(oracle_mod):
    # One signal among 999 noise positions; both maps share the noise keys and
    # only the first map's key at the signal position matches the query.  The
    # second map then carries the shared noise floor, and subtracting it raises
    # the signal-to-noise ratio for every lam in (0, lam*), lam* = (1-a)/(1-b);
    # at lam* the mean noise weight vanishes.
    N, d = 1000, 64
    g = np.random.default_rng(7)
    q = g.standard_normal(d).astype(np.float32)
    keys = g.standard_normal((N, d)).astype(np.float32)
    k1 = keys.copy()
    k1[0] = (1.4 * q).astype(np.float32)   # noise mass ~17%, inside the page's 8-30% band
    shape = (1, 1, N, d)
    qq = np.zeros(shape, np.float32); qq[0, 0, -1] = q
    a1, a2 = oracle_mod.prefill_weights(qq, qq, k1.reshape(shape), keys.reshape(shape),
                                        0, 0, N - 1, causal=False)
    a, b = a1[0], a2[0]
    assert 0.08 < 1 - a < 0.30        # a visible noise floor
    lam_star = (1 - a) / (1 - b)
    for frac in (0.1, 0.5, 0.9):
        s = oracle_mod.snr_from_weights(a1, a2, frac * lam_star, signal=0, visible=N)
        assert s["diff"] > s["plain"] > 0
    w = a1 - lam_star * a2
    assert abs(w[1:].mean()) < 1e-12
