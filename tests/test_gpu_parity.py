"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs, element by element, plus invariants that hold at any
size.  Every test prints its case before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import oracle
from differential_attention_prefill_amd import api
from differential_attention_prefill_amd import workloads as W

from parity_util import (compare, gpu_lambda, run_prefill_gpu, run_prefill_oracle, say)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.load_library()


# ---------------------------------------------------------------------------
# lambda: bit-identical in fp32
# ---------------------------------------------------------------------------

def assert_lambda_bitwise(inp, layer, lam_gpu):
    want = oracle.compute_lambda(inp["lq1"].cpu(), inp["lk1"].cpu(), inp["lq2"].cpu(),
                                 inp["lk2"].cpu(), layer)
    got = lam_gpu.cpu().numpy()
    assert got.view(np.uint32).tolist() == want.view(np.uint32).tolist()


def test_lambda_bitwise_many_heads_and_layers():
    g = torch.Generator().manual_seed(99)
    for layer in (1, 2, 6, 12, 24):
        for dim in (1, 7, 32, 64, 128, 1000):
            lq = [torch.randn((64, dim), generator=g) * 0.1 for _ in range(4)]
            say("lambda layer=%d dim=%d" % (layer, dim))
            want = oracle.compute_lambda(*lq, layer)
            got = api.diffattn_lambda(*(t.to(DEV) for t in lq), layer=layer).cpu().numpy()
            assert got.view(np.uint32).tolist() == want.view(np.uint32).tolist()


# ---------------------------------------------------------------------------
# fp32 prefill
# ---------------------------------------------------------------------------

def _prefill_case_check(case, rows=None, **over):
    inp = W.make_prefill(case, device=DEV)
    lam_gpu = gpu_lambda(inp, case.layer)
    assert_lambda_bitwise(inp, case.layer, lam_gpu)
    lam = lam_gpu.cpu().numpy()
    out = run_prefill_gpu(case, inp, lam_gpu, **over)
    torch.cuda.synchronize()
    ref = run_prefill_oracle(case, inp, lam, rows=rows, **over)
    got = out.cpu().numpy()
    if rows is not None:
        got = got.reshape(-1, case.dv)[rows]
    return compare(got, ref, case.dtype, case.name)


def test_prefill_fp32_tiny_workload():
    say("fp32 prefill %s" % W.TINY_FP32.name)
    _prefill_case_check(W.TINY_FP32)


@pytest.mark.parametrize("d,dv,N,causal,rms", [
    (32, 64, 1, True, False), (32, 64, 77, True, True), (64, 128, 100, False, False),
    (64, 64, 33, True, True), (128, 128, 50, True, False), (128, 64, 65, False, True),
    (32, 128, 129, True, False),
])
def test_prefill_fp32_shapes(d, dv, N, causal, rms):
    case = W.PrefillCase("fp32_d%d_dv%d_n%d" % (d, dv, N), "fp32", B=2, H=3, N=N, d=d, dv=dv,
                         layer=3, rmsnorm=rms, seed=1000 + N, causal=causal)
    say("fp32 prefill %s causal=%s rms=%s" % (case.name, causal, rms))
    _prefill_case_check(case)


# ---------------------------------------------------------------------------
# bf16 prefill (the fused MFMA kernel)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,dv,N,causal,rms", [
    (64, 128, 1, True, False), (64, 128, 31, True, True), (64, 128, 32, True, False),
    (64, 128, 33, True, False), (64, 128, 300, True, True), (64, 128, 517, False, False),
    (64, 128, 257, False, True), (64, 64, 200, True, True), (32, 64, 160, True, False),
    (128, 128, 190, True, False), (128, 128, 64, False, True), (128, 128, 1, True, True),
    (128, 128, 33, True, False), (128, 128, 128, True, True), (128, 128, 257, False, True),
])
def test_prefill_bf16_shapes(d, dv, N, causal, rms):
    case = W.PrefillCase("bf16_d%d_dv%d_n%d" % (d, dv, N), "bf16", B=2, H=3, N=N, d=d, dv=dv,
                         layer=4, rmsnorm=rms, seed=2000 + N, causal=causal)
    say("bf16 prefill %s causal=%s rms=%s" % (case.name, causal, rms))
    _prefill_case_check(case)


@pytest.mark.parametrize("d,dv,mode,causal", [
    (64, 128, "wide", True), (64, 128, "growing", True), (64, 128, "growing", False),
    (128, 128, "wide", False), (128, 128, "growing", True),
])
def test_prefill_bf16_rescale_stress(d, dv, mode, causal):
    """Logits far wider than the unit-variance workloads, so that row maxima
    keep growing past the lazy-rescale threshold: "wide" scales the queries
    by 6 (scaled scores with a spread of about 6); "growing" adds to key j of
    each map (j/N) * A * u_m along a fixed unit direction u_m (A = 30 sqrt(d)
    for map 1, 20 sqrt(d) for map 2), so a query's scores drift by up to about
    30 over the sequence, upward for half the queries (a new maximum in most
    sub-tiles, at different times in the two maps) and downward for the rest
    (probabilities that underflow)."""
    N = 700
    case = W.PrefillCase("bf16_%s_d%d" % (mode, d), "bf16", B=1, H=2, N=N, d=d, dv=dv, layer=3,
                         rmsnorm=True, seed=4100 + d, causal=causal)
    say("bf16 prefill rescale stress %s d=%d causal=%s" % (mode, d, causal))
    inp = W.make_prefill(case, device="cpu")
    g = torch.Generator().manual_seed(4200 + d)
    if mode == "wide":
        inp["q"] = (inp["q"].float() * 6.0).to(torch.bfloat16)
    else:
        ramp = (torch.arange(N, dtype=torch.float32) / N).reshape(1, 1, N, 1)
        k = inp["k"].float()
        for m, amp in ((0, 30.0), (1, 20.0)):
            u = torch.randn(d, generator=g)
            u = u / u.norm()
            k[..., m * d:(m + 1) * d] += ramp * (amp * math.sqrt(d)) * u
        inp["k"] = k.to(torch.bfloat16)
    lam_gpu = gpu_lambda(inp, case.layer)
    out = run_prefill_gpu(case, inp, lam_gpu).cpu().numpy()
    ref = run_prefill_oracle(case, inp, lam_gpu.cpu().numpy())
    compare(out, ref, "bf16", case.name)


def test_prefill_bf16_norm_weight():
    case = W.PrefillCase("bf16_weighted_norm", "bf16", B=1, H=2, N=130, d=64, dv=128, layer=6,
                         rmsnorm=True, seed=77)
    w = (1.0 + 0.5 * torch.randn(128, generator=torch.Generator().manual_seed(5))).float()
    say("bf16 prefill with a norm weight")
    inp = W.make_prefill(case, device=DEV)
    lam_gpu = gpu_lambda(inp, case.layer)
    out = run_prefill_gpu(case, inp, lam_gpu, norm_weight=w.to(DEV)).cpu().numpy()
    ref = run_prefill_oracle(case, inp, lam_gpu.cpu().numpy(), norm_weight=w)
    compare(out, ref, "bf16", case.name)


def test_prefill_v1_norm_workload_full():
    # B=4, H=16, N=2048, d=64, dv=128, RMS norm x (1 - lambda_init(6)): every row.
    say("bf16 prefill %s (all rows)" % W.V1_NORM.name)
    _prefill_case_check(W.V1_NORM)


def _sample_rows(case, needles, per_head=24, seed=0):
    """Rows to check at full size: first/last rows, needle rows, random rows."""
    g = np.random.default_rng(seed)
    rows = []
    for b in range(case.B):
        for h in range(case.H):
            base = (b * case.H + h) * case.N
            pick = set([0, 1, 31, 32, 127, 128, case.N - 1, case.N - 2, case.N - 33])
            for p in np.asarray(needles[h]).reshape(-1)[:4]:
                pick.update([int(p), min(case.N - 1, int(p) + 1)])
            pick.update(g.integers(0, case.N, size=per_head).tolist())
            rows.extend(base + r for r in sorted(pick) if 0 <= r < case.N)
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("case", [W.NEEDLE_32K, W.MULTI_NEEDLE_64K], ids=lambda c: c.name)
def test_prefill_long_workloads_sampled(case):
    say("bf16 prefill %s (sampled rows, full size)" % case.name)
    inp = W.make_prefill(case, device=DEV)
    rows = _sample_rows(case, inp["needles"])
    lam_gpu = gpu_lambda(inp, case.layer)
    assert_lambda_bitwise(inp, case.layer, lam_gpu)
    out = run_prefill_gpu(case, inp, lam_gpu)
    torch.cuda.synchronize()
    got = out.reshape(-1, case.dv)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del out
    ref = run_prefill_oracle(case, inp, lam_gpu.cpu().numpy(), rows=rows)
    compare(got, ref, "bf16", case.name + " sampled")


def test_prefill_longest_sequence_sampled():
    # The longest context any workload here runs through the fused kernel (the
    # noise-floor sweep's 256k), one head pair, the 64k workload's layer and
    # norm: sampled rows at full size, including the last rows.
    case = W.scaled_prefill(W.MULTI_NEEDLE_64K, N=262144, H=1)
    say("bf16 prefill, multi-needle recipe at H=1 N=%d (sampled rows)" % case.N)
    inp = W.make_prefill(case, device=DEV)
    g = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 65535, 65536, case.N - 257, case.N - 256,
                                      case.N - 2, case.N - 1], g.integers(0, case.N, 20)]))
    lam_gpu = gpu_lambda(inp, case.layer)
    out = run_prefill_gpu(case, inp, lam_gpu)
    torch.cuda.synchronize()
    got = out.reshape(-1, case.dv)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del out
    ref = run_prefill_oracle(case, inp, lam_gpu.cpu().numpy(), rows=rows.astype(np.int64))
    compare(got, ref, "bf16", "multi-needle recipe, H=1 N=%d, sampled" % case.N)


# ---------------------------------------------------------------------------
# V2-layout prefill: doubled query heads over shared K/V heads
# ---------------------------------------------------------------------------

def _v2_pair_tensors(inp, case):
    """Per-pair tensors [B, Hq/2, N, D]: q1 = heads 2p, q2 = heads 2p+1, k1 = k2
    and v the K/V head p // (Hq / (2 Hkv)) (test-side marshalling only)."""
    q = inp["q"]
    g = case.pairs_per_kv
    k = inp["k"].repeat_interleave(g, dim=1)
    v = inp["v"].repeat_interleave(g, dim=1)
    return (q[:, 0::2].contiguous(), q[:, 1::2].contiguous(), k.contiguous(), k.contiguous(),
            v.contiguous())


def _v2_check(case, rows=None):
    inp = W.make_prefill_v2(case, device=DEV)
    lam_gpu = gpu_lambda(inp, case.layer)
    out = api.diffattn_prefill_v2(inp["q"], inp["k"], inp["v"], lam_gpu, causal=case.causal)
    torch.cuda.synchronize()
    q1, q2, k1, k2, v = (t.cpu() for t in _v2_pair_tensors(inp, case))
    got = out.cpu().numpy()
    if rows is not None:
        got = got.reshape(-1, case.D)[rows]
    ref = oracle.prefill(q1, q2, k1, k2, v, lam_gpu.cpu().numpy(), causal=case.causal, rows=rows)
    return compare(got, ref, case.dtype, case.name)


@pytest.mark.parametrize("dtype,Hq,Hkv,N,D,causal", [
    ("bf16", 8, 2, 300, 128, True), ("bf16", 8, 4, 200, 64, True), ("bf16", 4, 1, 129, 128, False),
    ("bf16", 16, 2, 97, 128, True), ("fp32", 4, 1, 130, 64, True), ("fp32", 8, 2, 65, 128, False),
])
def test_prefill_v2_shapes(dtype, Hq, Hkv, N, D, causal):
    case = W.V2PrefillCase("v2_%s_hq%d_hkv%d_n%d_d%d" % (dtype, Hq, Hkv, N, D), dtype, B=2, Hq=Hq,
                           Hkv=Hkv, N=N, D=D, layer=2, seed=3000 + N, causal=causal)
    say("v2 prefill %s causal=%s" % (case.name, causal))
    _v2_check(case)


def test_prefill_v2_long_sampled():
    case = W.scaled_prefill(W.V2_PREFILL_32K, N=8192)
    say("v2 prefill %s (sampled rows)" % case.name)
    g = np.random.default_rng(1)
    H = case.Hq // 2
    rows = np.concatenate([h * case.N + np.unique(np.concatenate(
        [[0, 1, 127, 128, case.N - 1], g.integers(0, case.N, 12)])) for h in range(H)])
    _v2_check(case, rows=rows.astype(np.int64))


def test_prefill_v2_equals_v1_entry_on_expanded_tensors():
    # The V2 entry point is the V1 kernel with head strides; on materialised
    # per-pair tensors both entries give bit-identical results.
    for D in (64, 128):
        case = W.V2PrefillCase("v2_vs_v1_d%d" % D, "bf16", B=2, Hq=8, Hkv=2, N=333, D=D, layer=3,
                               seed=41 + D)
        say("v2 vs v1 entry D=%d" % D)
        inp = W.make_prefill_v2(case, device=DEV)
        lam = gpu_lambda(inp, case.layer)
        a = api.diffattn_prefill_v2(inp["q"], inp["k"], inp["v"], lam)
        q1, q2, k1, k2, v = _v2_pair_tensors(inp, case)
        b = api.diffattn_prefill(q1, q2, k1, k2, v, lam, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# Unfused two-pass path: plain attention twice, then the combine pass
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dv,N,causal", [(128, 300, True), (64, 200, False), (128, 64, False)])
def test_attention_single_map(dv, N, causal):
    case = W.PrefillCase("attn_dv%d_n%d" % (dv, N), "bf16", B=2, H=3, N=N, d=64, dv=dv, layer=1,
                         rmsnorm=False, seed=4000 + N, causal=causal)
    say("single-map attention %s causal=%s" % (case.name, causal))
    inp = W.make_prefill(case, device=DEV)
    q1, k1 = inp["q"][..., :64], inp["k"][..., :64]
    out = api.diffattn_attention(q1, k1, inp["v"], causal=causal)
    torch.cuda.synchronize()
    # lambda = 0 turns the oracle's difference into A1 V.
    ref = run_prefill_oracle(case, inp, np.zeros(case.H, dtype=np.float32))
    compare(out.cpu().numpy(), ref, "bf16", case.name)


def test_unfused_two_pass_matches_oracle_and_fused():
    case = W.scaled_prefill(W.V1_NORM, B=2, H=4, N=700)
    say("unfused two-pass %s" % case.name)
    inp = W.make_prefill(case, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    q, k, v = inp["q"], inp["k"], inp["v"]
    scale = 1.0 - api.diffattn_lambda_init(case.layer)
    o1 = api.diffattn_attention(q[..., :64], k[..., :64], v)
    o2 = api.diffattn_attention(q[..., 64:], k[..., 64:], v)
    out = api.diffattn_combine(o1, o2, lam, rmsnorm=True, eps=case.eps, norm_scale=scale)
    fused = run_prefill_gpu(case, inp, lam)
    torch.cuda.synchronize()
    ref = run_prefill_oracle(case, inp, lam.cpu().numpy())
    compare(out.cpu().numpy(), ref, "bf16", case.name + " unfused")
    compare(out.cpu().numpy(), fused.cpu().numpy().astype(np.float64), "bf16",
            case.name + " unfused vs fused")


# ---------------------------------------------------------------------------
# bf16 prefill invariants
# ---------------------------------------------------------------------------

def _rand_bf16(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_rows_sum_to_one_minus_lambda(d):
    # A value tensor of ones reads off the row sums of A1 - lam A2 = 1 - lam.
    B, H, N, dv = 1, 4, 700, 128
    say("bf16 row-sum invariant N=%d d=%d" % (N, d))
    q, k = _rand_bf16((B, H, N, 2 * d), 1), _rand_bf16((B, H, N, 2 * d), 2)
    v = torch.ones((B, H, N, dv), dtype=torch.bfloat16, device=DEV)
    lam = torch.tensor([0.2, 0.8, -0.5, 1.3], device=DEV)
    out = api.diffattn_prefill_packed(q, k, v, lam).cpu().double()
    want = (1 - lam.cpu().double()).view(1, H, 1, 1).expand_as(out)
    assert (out - want).abs().max().item() < 1e-2


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_identical_maps_cancel(d):
    B, H, N, dv = 2, 2, 333, 128
    say("bf16 identical maps with lambda=1, d=%d" % d)
    qh, kh = _rand_bf16((B, H, N, d), 3), _rand_bf16((B, H, N, d), 4)
    v = _rand_bf16((B, H, N, dv), 5)
    lam = torch.ones(H, device=DEV)
    out = api.diffattn_prefill(qh, qh, kh, kh, v, lam)
    assert out.abs().max().item() <= 1e-6


@pytest.mark.parametrize("B,H,N,causal,d", [(2, 4, 1000, True, 64), (1, 3, 777, False, 64),
                                            (2, 2, 900, True, 128)])
def test_prefill_bitwise_deterministic(B, H, N, causal, d):
    # Many workgroups, repeated launches: results must be bit-identical, and
    # with identical maps and lambda = 1 every output must vanish.
    say("bf16 determinism B=%d H=%d N=%d causal=%s d=%d" % (B, H, N, causal, d))
    dv = 128
    qh, kh, v = _rand_bf16((B, H, N, d), 31), _rand_bf16((B, H, N, d), 32), _rand_bf16((B, H, N, dv), 33)
    q, k = _rand_bf16((B, H, N, 2 * d), 34), _rand_bf16((B, H, N, 2 * d), 35)
    lam = torch.linspace(-0.5, 1.5, H, device=DEV)
    first = api.diffattn_prefill_packed(q, k, v, lam, causal=causal)
    for _ in range(3):
        assert torch.equal(first, api.diffattn_prefill_packed(q, k, v, lam, causal=causal))
    ones = torch.ones(H, device=DEV)
    for _ in range(3):
        z = api.diffattn_prefill(qh, qh, kh, kh, v, ones, causal=causal)
        assert z.abs().max().item() <= 1e-6


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_causality_and_determinism(d):
    B, H, N, dv = 1, 2, 400, 128
    say("bf16 causality / determinism d=%d" % d)
    q, k, v = _rand_bf16((B, H, N, 2 * d), 6), _rand_bf16((B, H, N, 2 * d), 7), _rand_bf16((B, H, N, dv), 8)
    lam = torch.tensor([0.3, 0.6], device=DEV)
    a = api.diffattn_prefill_packed(q, k, v, lam)
    b = api.diffattn_prefill_packed(q, k, v, lam)
    assert torch.equal(a, b)
    i = 170
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i + 1:] = _rand_bf16((B, H, N - i - 1, 2 * d), 9)
    v2[:, :, i + 1:] = _rand_bf16((B, H, N - i - 1, dv), 10)
    c = api.diffattn_prefill_packed(q, k2, v2, lam)
    assert torch.equal(a[:, :, : i + 1], c[:, :, : i + 1])
    assert not torch.equal(a[:, :, i + 1:], c[:, :, i + 1:])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_prefill_nonfinite_key_row_is_causal(d, bad):
    # Causal masking replaces the scores of keys after a query before they are
    # used, so a non-finite key row j leaves every output row i < j exactly as
    # it was (page "差分注意力", part 二 Step 2: query i attends to keys 0..i).
    # Rows at the start, inside and at the end of 32-key sub-tiles and of
    # 256-row tiles.
    B, H, N, dv = 1, 2, 600, 128
    q, k, v = _rand_bf16((B, H, N, 2 * d), 16), _rand_bf16((B, H, N, 2 * d), 17), _rand_bf16((B, H, N, dv), 18)
    lam = torch.tensor([0.3, 0.6], device=DEV)
    clean = api.diffattn_prefill_packed(q, k, v, lam)
    for j in (1, 31, 32, 170, 255, 256, 511, 599):
        say("bf16 non-finite key row d=%d bad=%s j=%d" % (d, bad, j))
        kb = k.clone()
        kb[:, :, j] = bad
        out = api.diffattn_prefill_packed(q, kb, v, lam)
        assert torch.equal(out[:, :, :j], clean[:, :, :j]), j
        torch.cuda.synchronize()


def test_prefill_separate_tensors_match_packed():
    B, H, N, d, dv = 1, 2, 96, 64, 128
    say("bf16 separate Q1/Q2/K1/K2 tensors")
    q, k, v = _rand_bf16((B, H, N, 2 * d), 11), _rand_bf16((B, H, N, 2 * d), 12), _rand_bf16((B, H, N, dv), 13)
    lam = torch.tensor([0.4, 0.1], device=DEV)
    a = api.diffattn_prefill_packed(q, k, v, lam)
    b = api.diffattn_prefill(q[..., :d].contiguous(), q[..., d:].contiguous(),
                             k[..., :d].contiguous(), k[..., d:].contiguous(), v, lam)
    assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_one_key_tensor_for_both_maps(d):
    # K1 and K2 the same tensor (one pointer): at d = 128 this selects the
    # stage layout that holds the keys once; against the oracle and against
    # the same keys passed as two distinct tensors (bitwise).
    B, H, N, dv = 2, 3, 300, 128
    say("bf16 prefill, K1 = K2 (one tensor), d=%d N=%d" % (d, N))
    q1, q2 = _rand_bf16((B, H, N, d), 21), _rand_bf16((B, H, N, d), 22)
    k, v = _rand_bf16((B, H, N, d), 23), _rand_bf16((B, H, N, dv), 24)
    lam = torch.tensor([0.4, -0.2, 0.9], device=DEV)
    shared = api.diffattn_prefill(q1, q2, k, k, v, lam)
    separate = api.diffattn_prefill(q1, q2, k, k.clone(), v, lam)
    torch.cuda.synchronize()
    assert torch.equal(shared, separate)
    ref = oracle.prefill(q1.cpu(), q2.cpu(), k.cpu(), k.cpu(), v.cpu(), lam.cpu().numpy(), causal=True)
    compare(shared.cpu().numpy(), ref, "bf16", "one key tensor d=%d" % d)


def test_prefill_rejects_host_pointer():
    lib = api.load_library()
    host = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16)
    dev = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((1, 1, 16, 128), device=DEV)
    lam = torch.zeros(1, device=DEV)
    st = lib.diffattn_prefill(host.data_ptr(), dev.data_ptr() + 128, dev.data_ptr(),
                              dev.data_ptr() + 128, dev.data_ptr(), 128, 128, 128, 1, 1, 1, 16,
                              64, 128, 1, lam.data_ptr(), 0, 1e-5, 1.0, None, out.data_ptr(), None)
    assert st == 1
    assert torch.count_nonzero(out).item() == 0


# ---------------------------------------------------------------------------
# decode (V2 layout)
# ---------------------------------------------------------------------------

def _decode_check(case, fill_unused=None):
    inp = W.make_decode(case, device=DEV, fill_unused=fill_unused)
    lam_gpu = gpu_lambda(inp, case.layer)
    assert_lambda_bitwise(inp, case.layer, lam_gpu)
    out = api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam_gpu)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.decode(inp["q"].cpu(), inp["k_cache"].cpu(), inp["v_cache"].cpu(),
                        inp["seq_lens"].cpu(), lam_gpu.cpu().numpy())
    return compare(got, ref, "bf16", case.name)


@pytest.mark.parametrize("lens", [[1, 2, 31, 33], [1023, 1024, 1025, 3000], [4096, 777, 4095, 64],
                                  [2047, 2048, 2049, 4097], [8191, 8192, 8193, 12289]])
def test_decode_ragged_lengths(lens):
    case = W.DecodeCase("decode_small_%d" % lens[0], B=len(lens), Hq=8, Hkv=2, D=128,
                        Lmin=1, Lmax=max(lens), layer=2, seed=sum(lens))
    say("decode lens=%s" % lens)
    inp = W.make_decode(case, device=DEV)
    inp["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for b, L in enumerate(lens):   # unused cache slots hold NaN: they must not be read
        inp["k_cache"][b, :, L:] = float("nan")
        inp["v_cache"][b, :, L:] = float("nan")
    lam_gpu = gpu_lambda(inp, case.layer)
    out = api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam_gpu)
    ref = oracle.decode(inp["q"].cpu(), inp["k_cache"].cpu(), inp["v_cache"].cpu(),
                        inp["seq_lens"].cpu(), lam_gpu.cpu().numpy())
    compare(out.cpu().numpy(), ref, "bf16", case.name)


@pytest.mark.parametrize("mode", ["wide", "growing"])
def test_decode_rescale_stress(mode):
    """Decode over several pieces per sequence with logits far wider than the
    workload's: "wide" scales the queries by 6; "growing" adds (j/L) * 30
    sqrt(D) * u to cached key j along a fixed unit direction u, so a head's
    scores drift by up to about 30 across the sequence (new maxima inside and
    across pieces, or underflowing probabilities), which exercises the lazy
    rescale in the split kernel and the log-sum-exp weights of the merge."""
    lens = [9000, 4097, 2500, 1]
    case = W.DecodeCase("decode_stress_%s" % mode, B=len(lens), Hq=8, Hkv=2, D=128,
                        Lmin=1, Lmax=max(lens), layer=5, seed=4300 + len(mode))
    say("decode rescale stress %s lens=%s" % (mode, lens))
    inp = W.make_decode(case, device="cpu")
    inp["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    if mode == "wide":
        inp["q"] = (inp["q"].float() * 6.0).to(torch.bfloat16)
    else:
        g = torch.Generator().manual_seed(4400)
        u = torch.randn(case.D, generator=g)
        u = u / u.norm()
        k = inp["k_cache"].float()
        for b, L in enumerate(lens):
            ramp = (torch.arange(L, dtype=torch.float32) / L).reshape(1, L, 1)
            k[b, :, :L] += ramp * (30.0 * math.sqrt(case.D)) * u
        inp["k_cache"] = k.to(torch.bfloat16)
    dev = {x: inp[x].to(DEV) for x in ("q", "k_cache", "v_cache", "seq_lens")}
    lam_gpu = gpu_lambda(inp, case.layer)
    out = api.diffattn_decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["seq_lens"], lam_gpu)
    ref = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                        lam_gpu.cpu().numpy())
    compare(out.cpu().numpy(), ref, "bf16", case.name)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (16, 2), (32, 8), (8, 4), (32, 2)])
def test_decode_group_sizes(hq, hkv):
    case = W.DecodeCase("decode_g%d" % (hq // hkv), B=2, Hq=hq, Hkv=hkv, D=128, Lmin=500,
                        Lmax=2500, layer=1, seed=hq * 10 + hkv)
    say("decode Hq=%d Hkv=%d" % (hq, hkv))
    _decode_check(case, fill_unused=float("nan"))


def test_decode_invalid_device_length_gives_zeros():
    case = W.DecodeCase("decode_badlen", B=3, Hq=8, Hkv=2, D=128, Lmin=10, Lmax=300, layer=1,
                        seed=5)
    say("decode with an out-of-range device length")
    inp = W.make_decode(case, device=DEV)
    inp["seq_lens"] = torch.tensor([100, 0, 301], dtype=torch.int32, device=DEV)
    lam = gpu_lambda(inp, 1)
    out = api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam)
    assert torch.count_nonzero(out[1:]).item() == 0
    ref = oracle.decode(inp["q"][:1].cpu(), inp["k_cache"][:1].cpu(), inp["v_cache"][:1].cpu(),
                        np.array([100], np.int32), lam.cpu().numpy())
    compare(out[:1].cpu().numpy(), ref, "bf16", "decode valid row")


@pytest.mark.parametrize("layout", ["v2", "v1"])
def test_decode_bitwise_repeatable_over_stale_workspace(layout):
    # Two calls on one workspace, the second after the workspace was filled
    # with 0xFF bytes (NaN states, piece counts of -1): every call rewrites
    # every state and count the merge reads, and the fixed merge order makes
    # the output bitwise identical.
    lens = torch.tensor([20000, 4096, 1, 9001, 12345, 8192], dtype=torch.int32)
    if layout == "v2":
        case = W.DecodeCase("decode_repeat", B=len(lens), Hq=32, Hkv=8, D=128, Lmin=1,
                            Lmax=20000, layer=4, seed=1234)
        inp = W.make_decode(case, device=DEV)
        nbytes = api.diffattn_decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, case.Lmax)
    else:
        case = W.V1DecodeCase("decode_v1_repeat", B=len(lens), H=8, d=64, dv=128, Lmin=1,
                              Lmax=20000, layer=4, seed=1235)
        inp = W.make_decode_v1(case, device=DEV)
        nbytes = api.diffattn_decode_v1_workspace_bytes(case.B, case.H, case.Lmax)
    say("decode %s repeatability over a stale workspace" % layout)
    inp["seq_lens"] = lens.to(DEV)
    lam = gpu_lambda(inp, case.layer)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    run = (lambda: api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam,
                                       workspace=ws)) if layout == "v2" else \
          (lambda: api.diffattn_decode_v1(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam,
                                          workspace=ws))
    first = run().clone()
    ws.fill_(0xFF)
    second = run()
    torch.cuda.synchronize()
    assert torch.isfinite(first).all()
    assert torch.equal(first, second)


def test_decode_many_short_sequences_in_one_range():
    # 300 sequences of 1 .. 40 keys over 8 KV heads: about 49k keys in about
    # 12 ranges of the minimum length, so each workgroup walks some 200
    # segments (whole ones, plus a cut one at each end of its range) and skips
    # the sequences without keys.
    B, max_len = 300, 40
    case = W.DecodeCase("decode_short", B=B, Hq=16, Hkv=8, D=128, Lmin=1, Lmax=max_len, layer=2,
                        seed=91)
    say("decode %d short sequences in one key range" % B)
    inp = W.make_decode(case, device=DEV)
    lens = torch.randint(1, max_len + 1, (B,), generator=torch.Generator().manual_seed(12),
                         dtype=torch.int32)
    bad = [0, 1, 150, 299]
    for i, v in zip(bad, [0, max_len + 1, -1, 0]):
        lens[i] = v
    inp["seq_lens"] = lens.to(DEV)
    lam = gpu_lambda(inp, case.layer)
    out = api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[bad]).item() == 0
    good = [b for b in range(B) if b not in bad]
    ref = oracle.decode(inp["q"][good].cpu(), inp["k_cache"][good].cpu(), inp["v_cache"][good].cpu(),
                        lens[good].numpy(), lam.cpu().numpy())
    compare(out[good].cpu().numpy(), ref, "bf16", case.name)


def test_decode_many_items_with_invalid_lengths():
    # Key ranges of about 6k keys over segments of 1 .. 12288: most ranges
    # cover pieces of several segments and skip the out-of-range lengths in
    # between.
    B, max_len = 64, 12288
    case = W.DecodeCase("decode_items", B=B, Hq=16, Hkv=8, D=128, Lmin=1, Lmax=max_len, layer=3,
                        seed=77)
    say("decode %d sequences, several pieces each, invalid lengths interleaved" % B)
    inp = W.make_decode(case, device=DEV)
    lens = torch.randint(1, max_len + 1, (B,), generator=torch.Generator().manual_seed(11),
                         dtype=torch.int32)
    bad = [3, 17, 18, 40, 63]
    for i, v in zip(bad, [0, -5, max_len + 1, 0, max_len + 100]):
        lens[i] = v
    inp["seq_lens"] = lens.to(DEV)
    lam = gpu_lambda(inp, case.layer)
    out = api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[bad]).item() == 0
    good = [b for b in range(B) if b not in bad]
    ref = oracle.decode(inp["q"][good].cpu(), inp["k_cache"][good].cpu(), inp["v_cache"][good].cpu(),
                        lens[good].numpy(), lam.cpu().numpy())
    compare(out[good].cpu().numpy(), ref, "bf16", case.name)


def test_decode_v2_workload_full():
    # B=32, Hq=32 (16 pairs), Hkv=8, D=128, lengths uniform in [4096, 65536].
    say("decode %s (all outputs)" % W.V2_DECODE.name)
    _decode_check(W.V2_DECODE)


# ---------------------------------------------------------------------------
# Plain single-map GQA decode (the baseline the V2 layout is compared with)
# ---------------------------------------------------------------------------

def _plain_decode_oracle(q, k_cache, v_cache, lens):
    """Plain attention of every query head through the oracle's decode: a
    query tensor of 2*Hq heads whose even heads are the plain heads and odd
    heads zero, lambda = 0 (the oracle's pair p over KV head
    2p // (2Hq/Hkv) = p // (Hq/Hkv) then gives A1 V of head p)."""
    B, Hq, D = q.shape
    q2 = torch.zeros((B, 2 * Hq, D), dtype=q.dtype)
    q2[:, 0::2] = q
    return oracle.decode(q2, k_cache, v_cache, lens, np.zeros(Hq, np.float32))


@pytest.mark.parametrize("B,Hq,Hkv,lens", [
    (4, 16, 8, [4096, 20000, 1, 9001]), (3, 8, 8, [1, 700, 333]), (2, 6, 2, [5000, 100]),
    (3, 3, 3, [257, 1, 4100]), (2, 16, 1, [12289, 8191]),
])
def test_attention_decode_single_map(B, Hq, Hkv, lens):
    case = W.DecodeCase("plain_decode_hq%d_hkv%d" % (Hq, Hkv), B=B, Hq=Hq, Hkv=Hkv, D=128,
                        Lmin=1, Lmax=max(lens), layer=1, seed=B * 100 + Hq)
    say("plain decode B=%d Hq=%d Hkv=%d lens=%s" % (B, Hq, Hkv, lens))
    inp = W.make_decode(case, device=DEV)
    inp["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for b, L in enumerate(lens):   # unused cache slots hold NaN: they must not be read
        inp["k_cache"][b, :, L:] = float("nan")
        inp["v_cache"][b, :, L:] = float("nan")
    out = torch.full((B, Hq, 128), float("nan"), device=DEV)
    api.diffattn_attention_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], out=out)
    torch.cuda.synchronize()
    ref = _plain_decode_oracle(inp["q"].cpu(), inp["k_cache"].cpu(), inp["v_cache"].cpu(),
                               inp["seq_lens"].cpu())
    compare(out.cpu().numpy(), ref, "bf16", case.name)


def test_attention_decode_invalid_length_gives_zeros():
    case = W.DecodeCase("plain_decode_badlen", B=3, Hq=8, Hkv=2, D=128, Lmin=10, Lmax=300,
                        layer=1, seed=6)
    say("plain decode with out-of-range device lengths")
    inp = W.make_decode(case, device=DEV)
    inp["seq_lens"] = torch.tensor([120, 0, 301], dtype=torch.int32, device=DEV)
    out = torch.full((3, 8, 128), float("nan"), device=DEV)
    api.diffattn_attention_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[1:]).item() == 0
    ref = _plain_decode_oracle(inp["q"][:1].cpu(), inp["k_cache"][:1].cpu(), inp["v_cache"][:1].cpu(),
                               np.array([120], np.int32))
    compare(out[:1].cpu().numpy(), ref, "bf16", "plain decode valid row")


def test_v2_decode_equals_two_plain_decodes_combined():
    # The differential decode of pair p is the plain decode of query head 2p
    # minus lambda_p times that of head 2p+1 over the same KV head: both run
    # the same split kernel, so the pieces are identical and only the final
    # fp32 combination can differ.
    case = W.scaled_decode(W.V2_DECODE, B=6, Lmin=1000, Lmax=30000, seed=81)
    say("v2 decode against two plain decodes combined, %s B=%d" % (case.name, case.B))
    inp = W.make_decode(case, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    v2 = api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam)
    plain = api.diffattn_attention_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"])
    torch.cuda.synchronize()
    combined = plain[:, 0::2] - lam.view(1, -1, 1) * plain[:, 1::2]
    assert (v2 - combined).abs().max().item() <= 1e-6


# ---------------------------------------------------------------------------
# V1-layout decode: half-width maps, value cache read once, RMS norm
# ---------------------------------------------------------------------------

def _decode_v1_oracle(inp, case, lam, rows_of=None, norm_weight=None):
    """Oracle by definition: the decode query of sequence b is the last row of
    a causal prefill over its L_b cached positions (test-side marshalling)."""
    q, kc, vc = (inp[x].cpu() for x in ("q", "k_cache", "v_cache"))
    lens = inp["seq_lens"].cpu().tolist()
    d = case.d
    out = np.zeros((case.B, case.H, case.dv))
    for b in range(case.B):
        L = int(lens[b])
        q1 = torch.zeros((1, case.H, L, d), dtype=q.dtype)
        q2 = torch.zeros((1, case.H, L, d), dtype=q.dtype)
        q1[0, :, L - 1] = q[b, :, :d]
        q2[0, :, L - 1] = q[b, :, d:]
        k1 = kc[b, :, :L, :d].unsqueeze(0).contiguous()
        k2 = kc[b, :, :L, d:].unsqueeze(0).contiguous()
        v = vc[b, :, :L].unsqueeze(0).contiguous()
        rows = np.array([h * L + L - 1 for h in range(case.H)], dtype=np.int64)
        out[b] = oracle.prefill(q1, q2, k1, k2, v, lam, causal=True, rmsnorm=case.rmsnorm,
                                eps=case.eps, norm_scale=(1.0 - oracle.lambda_init(case.layer))
                                if case.rmsnorm else 1.0, norm_weight=norm_weight, rows=rows)
    return out


def _decode_v1_run(case, inp, lam, norm_weight=None):
    return api.diffattn_decode_v1(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam,
                                  rmsnorm=case.rmsnorm, eps=case.eps,
                                  norm_scale=(1.0 - api.diffattn_lambda_init(case.layer))
                                  if case.rmsnorm else 1.0, norm_weight=norm_weight)


@pytest.mark.parametrize("lens,rms", [([1, 2, 31, 33], True), ([1023, 1024, 1025, 3000], True),
                                      ([4096, 777, 64, 2049], False), ([2047, 2048, 6000, 4097], True)])
def test_decode_v1_ragged_lengths(lens, rms):
    case = W.V1DecodeCase("v1_decode_small_%d" % lens[-1], B=len(lens), H=3, d=64, dv=128,
                          Lmin=1, Lmax=max(lens), layer=5, seed=900 + lens[-1], rmsnorm=rms)
    say("v1 decode %s lens=%s rms=%s" % (case.name, lens, rms))
    inp = W.make_decode_v1(case, device=DEV)
    inp["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    got = _decode_v1_run(case, inp, lam).cpu().numpy()
    ref = _decode_v1_oracle(inp, case, lam.cpu().numpy())
    compare(got, ref, "bf16", case.name)


def test_decode_v1_norm_weight_and_bad_length():
    case = W.V1DecodeCase("v1_decode_weighted", B=3, H=2, d=64, dv=128, Lmin=100, Lmax=600,
                          layer=8, seed=31)
    say("v1 decode with a norm weight and an invalid length")
    inp = W.make_decode_v1(case, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    w = (1.0 + 0.5 * torch.randn(128, generator=torch.Generator().manual_seed(9))).float()
    got = _decode_v1_run(case, inp, lam, norm_weight=w.to(DEV)).cpu().numpy()
    ref = _decode_v1_oracle(inp, case, lam.cpu().numpy(), norm_weight=w)
    compare(got, ref, "bf16", case.name)
    inp["seq_lens"][1] = 0
    got = _decode_v1_run(case, inp, lam).cpu().numpy()
    assert np.all(got[1] == 0.0)


def test_decode_v1_workload_scaled():
    case = W.scaled_decode(W.V1_DECODE, B=4)
    say("v1 decode %s (B=4, full lengths)" % case.name)
    inp = W.make_decode_v1(case, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    got = _decode_v1_run(case, inp, lam).cpu().numpy()
    ref = _decode_v1_oracle(inp, case, lam.cpu().numpy())
    compare(got, ref, "bf16", case.name)


# ---------------------------------------------------------------------------
# Signal-to-noise read off the kernel with probe values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1024, 4096, 16384, 65536])
def test_snr_probe_matches_oracle(N):
    from differential_attention_prefill_amd import snr
    # A score of 10 keeps the signal weight well inside (0, 1) at these lengths.
    case = W.scaled_prefill(W.NEEDLE_32K, N=N, H=4, dv=64, needle_score=10.0)
    say("snr probe %s N=%d" % (case.name, N))
    inp = W.make_prefill(case, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    sig = inp["needles"][:, 0]
    got = snr.snr_last_query(inp["q"], inp["k"], lam, sig)
    q, k = inp["q"].cpu(), inp["k"].cpu()
    q1, q2, k1, k2 = (t.contiguous() for t in (q[..., :64], q[..., 64:], k[..., :64], k[..., 64:]))
    lam_h = lam.cpu().numpy()
    for h in range(case.H):
        a1, a2 = oracle.prefill_weights(q1, q2, k1, k2, 0, h, N - 1)
        ref = oracle.snr_from_weights(a1, a2, float(lam_h[h]), int(sig[h]), N)
        for name in ("plain", "diff"):
            g, r = float(got[name][h]), ref[name]
            say("  head %d %s: kernel %.4g oracle %.4g" % (h, name, g, r))
            assert abs(g - r) <= 2e-2 * abs(r), (h, name, g, r)


def test_needle_mass_probe_matches_oracle():
    from differential_attention_prefill_amd import snr
    case = W.scaled_prefill(W.MULTI_NEEDLE_64K, N=4096, H=3, dv=64)
    say("needle mass probe %s" % case.name)
    inp = W.make_prefill(case, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    got = snr.needle_mass(inp["q"], inp["k"], lam, inp["needles"])
    q, k = inp["q"].cpu(), inp["k"].cpu()
    q1, q2, k1, k2 = (t.contiguous() for t in (q[..., :64], q[..., 64:], k[..., :64], k[..., 64:]))
    lam_h = lam.cpu().numpy()
    for h in range(case.H):
        a1, a2 = oracle.prefill_weights(q1, q2, k1, k2, 0, h, case.N - 1)
        pos = inp["needles"][h].numpy()
        w = a1 - float(lam_h[h]) * a2
        ref = {"plain": a1[pos].sum(), "diff": w[pos].sum() / w.sum()}
        for name in ("plain", "diff"):
            g = float(got[name][h])
            say("  head %d %s: kernel %.5f oracle %.5f" % (h, name, g, ref[name]))
            assert abs(g - ref[name]) <= 1e-2 * max(abs(ref[name]), 1e-3), (h, name)


def test_needle_32k_snr_regime():
    # The 32k needle workload at full size (16 heads, one needle per head whose
    # first-map key is 5x the last query's first half): the last query's SNRs
    # from the oracle's fp64 softmax rows on the bytes the GPU generated.  At
    # d = 64 the needle scores about 40 above the noise, so A1's noise mass is
    # ~1e-12 to ~1e-8: the plain SNR is huge and, whenever lambda exceeds that mass,
    # the signed differential SNR is negative (over-subtracted noise).  The
    # kernel's own rows for these queries are checked by the sampled parity
    # test; here the kernel's read of the signal's weight share must match.
    from oracle import snr as osnr
    from differential_attention_prefill_amd import snr
    case = W.NEEDLE_32K
    say("snr regime %s (last query of every head)" % case.name)
    inp = W.make_prefill(case, device=DEV)
    lam = gpu_lambda(inp, case.layer)
    sig = inp["needles"][:, 0]
    got = snr.noise_sweep_point(inp["q"], inp["k"], lam, sig)
    q, k = inp["q"].cpu(), inp["k"].cpu()
    q1, q2, k1, k2 = (t.contiguous() for t in (q[..., :64], q[..., 64:], k[..., :64], k[..., 64:]))
    lam_h = lam.cpu().numpy()
    N = case.N
    plain, diff, diff_abs = [], [], []
    for h in range(case.H):
        a1, a2 = oracle.prefill_weights(q1, q2, k1, k2, 0, h, N - 1)
        s = int(sig[h])
        r = oracle.snr_from_weights(a1, a2, float(lam_h[h]), s, N)
        plain.append(r["plain"])
        diff.append(r["diff"])
        diff_abs.append(r["diff_abs"])
        # The needle's score is 5|q1|^2/8 with |q1|^2 ~ chi^2(64): at least ~25
        # above the noise for any plausible draw, so A1's noise mass stays
        # below ~1e-5 even over 32767 noise keys.
        assert a1[s] > 1 - 1e-5, (h, a1[s])
        assert r["plain"] > 1e8, (h, r["plain"])
        say("  head %d: A1 noise mass %.3g, lambda %.4f, SNR plain %.3g diff %.3g"
            % (h, 1 - a1[s], lam_h[h], r["plain"], r["diff"]))
        # Signed differential SNR: negative exactly when lambda outweighs the
        # noise mass left after subtraction.
        noise_diff = (1 - a1[s]) - lam_h[h] * (1 - a2[s])
        assert np.sign(r["diff"]) == np.sign(noise_diff), (h, r["diff"], noise_diff)
        if a1[s] < 1.0:   # the closed form's plain ratio needs 1 - a > 0 in fp64
            cf = osnr.snr_closed_form(float(a1[s]), float(a2[s]), float(lam_h[h]), N)
            assert abs(cf["diff"] - r["diff"]) <= 1e-3 * abs(r["diff"]), (h, cf["diff"], r["diff"])
        # Kernel: the signal's share of the row weight, plain and differential.
        w = a1 - lam_h[h] * a2
        for name, ref in (("plain", a1[s] / a1.sum()), ("diff", w[s] / w.sum())):
            g = float(got[name + "_signal"][h])
            assert abs(g - ref) <= 1e-2 * abs(ref), (h, name, g, ref)
    say("  SNR medians over heads: plain %.3g, diff (signed) %.3g, diff (|noise|) %.3g"
        % (np.median(plain), np.median(diff), np.median(diff_abs)))
