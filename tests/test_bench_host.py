"""bench.py's host-side contract, CPU only: it refuses more than one GPU
before touching any device, and its algorithmic work counts equal brute-force
counts on small cases (the counts every throughput and roofline fraction it
prints is divided by)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from differential_attention_prefill_amd import workloads as W  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for an unsupported run


def _brute_pairs(N, causal):
    return sum(1 for i in range(N) for j in range(N) if (j <= i or not causal))


def test_prefill_flops_count_visible_pairs():
    for N, causal in ((1, True), (7, True), (33, True), (5, False)):
        case = W.PrefillCase("t", "bf16", B=2, H=3, N=N, d=64, dv=128, layer=1, rmsnorm=False,
                             seed=0, causal=causal)
        pairs = 2 * 3 * _brute_pairs(N, causal)
        assert bench.prefill_flops(case) == pairs * (4 * 64 + 2 * 128)
        assert bench.executed_prefill_flops(case) == pairs * (4 * 64 + 4 * 128)


def test_full_size_prefill_flops():
    c = W.MULTI_NEEDLE_64K
    assert bench.prefill_flops(c) == 32 * 65536 * 65537 // 2 * 512
    assert abs(bench.prefill_flops(c) - 3.5184908959744e13) < 1


def test_decode_bytes_and_flops_count_every_row_once():
    c = W.V2_DECODE
    lens = np.array([1, 5, 4096, 65536] + [100] * (c.B - 4))
    kv = sum(int(L) * c.Hkv * (c.D + c.D) * 2 for L in lens)      # K and V rows, bf16
    extra = c.B * c.Hq * c.D * 2 + (c.Hq // 2) * 4 + c.B * 4 + c.B * (c.Hq // 2) * c.D * 4
    assert bench.decode_bytes(c, lens) == kv + extra
    assert bench.decode_flops(c, lens) == sum(int(L) for L in lens) * (c.Hq // 2) * 6 * c.D


def test_ranges_nest_and_do_nothing_without_the_roctx_library(monkeypatch):
    # With the library the ranges push and pop in pairs; without it (no ROCm
    # profiler SDK under ROCM_PATH) every range is a no-op and the body runs.
    calls = []

    class FakeLib:
        def roctxRangePushA(self, name):
            calls.append(("push", name))
            return 0

        def roctxRangePop(self):
            calls.append(("pop",))
            return 0

    r = bench.Ranges()
    r._lib = FakeLib()
    with r("outer"):
        with r("inner"):
            pass
    assert calls == [("push", b"outer"), ("push", b"inner"), ("pop",), ("pop",)]
    try:
        with r("raises"):
            raise KeyError("x")
    except KeyError:
        pass
    assert calls[-1] == ("pop",)          # popped on the way out of an exception

    monkeypatch.setenv("ROCM_PATH", "/nonexistent-rocm")
    empty = bench.Ranges()
    assert empty._lib is None
    ran = []
    with empty("anything"):
        ran.append(1)
    assert ran == [1]


def test_every_extra_has_a_runner():
    # measure_extras runs each name in EXTRAS; a name with no runner would be
    # silently skipped.
    import inspect
    src = inspect.getsource(bench.measure_extras)
    for name in bench.EXTRAS:
        assert '"%s"' % name in src, name
