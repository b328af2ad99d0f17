"""Full-size parity of the long prefill workloads against the CPU oracle.

The operator is the one of page "差分注意力", part 二 Step 2 (with the
per-head norm of "V1 到 V2 的 diff" on the 64k workload).  Each workload runs
once through the C ABI, in the launch configuration the benchmark times,
into an output buffer filled with NaN beforehand: every element must come
back finite (a tile that no workgroup writes cannot pass).  Then:

  * 32k needle workload: every row of every head against the oracle;
  * 64k multi-needle workload: at least four rows of every 256-row tile of
    every head (the tile's first and last rows and two random rows), plus
    the needle rows, against the oracle;
  * V2 prefill at 32k, D = 128: the first, last and one random row of every
    128-row tile of every pair.
  * the length-sweep workloads at 8k (every row) and 128k (the first, last
    and one random row of every 256-row tile of every head).

The oracle runs on all host threads; each test prints its case first.
"""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_prefill_amd import api
from differential_attention_prefill_amd import workloads as W

from parity_util import compare, gpu_lambda, run_prefill_gpu, run_prefill_oracle, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.load_library()


def _run_nan_filled(case, inp, lam_gpu):
    out = torch.full((case.B, case.H, case.N, case.dv), float("nan"), dtype=torch.float32,
                     device=DEV)
    run_prefill_gpu(case, inp, lam_gpu, out=out)
    torch.cuda.synchronize()
    bad = int((~torch.isfinite(out)).sum().item())
    assert bad == 0, "%s: %d output elements not written or not finite" % (case.name, bad)
    return out


@pytest.fixture(scope="module")
def needle_32k():
    _require_gpu()
    case = W.NEEDLE_32K
    say("32k needle workload %s: GPU run into a NaN-filled output" % case.name)
    inp = W.make_prefill(case, device=DEV)
    lam_gpu = gpu_lambda(inp, case.layer)
    out = _run_nan_filled(case, inp, lam_gpu)
    host = {k: inp[k].cpu() for k in ("q", "k", "v")}
    return case, host, lam_gpu.cpu().numpy(), out.cpu().numpy().reshape(-1, case.dv)


@pytest.mark.parametrize("h", range(W.NEEDLE_32K.H))
def test_needle_32k_every_row(needle_32k, h):
    case, host, lam, got = needle_32k
    rows = np.arange(h * case.N, (h + 1) * case.N, dtype=np.int64)
    say("32k needle workload, head %d: all %d rows against the oracle" % (h, case.N))
    ref = run_prefill_oracle(case, host, lam, rows=rows)
    compare(got[rows], ref, "bf16", "%s head %d (every row)" % (case.name, h))


@pytest.fixture(scope="module")
def multi_needle_64k():
    _require_gpu()
    case = W.MULTI_NEEDLE_64K
    say("64k multi-needle workload %s: GPU run into a NaN-filled output" % case.name)
    inp = W.make_prefill(case, device=DEV)
    lam_gpu = gpu_lambda(inp, case.layer)
    out = _run_nan_filled(case, inp, lam_gpu)
    rows = _tile_rows(case.B * case.H, case.N, 256, per_tile=2, seed=64)
    needles = np.unique(np.asarray(inp["needles"]).reshape(-1))
    extra = np.concatenate([h * case.N + needles for h in range(case.H)])
    rows = np.unique(np.concatenate([rows, extra])).astype(np.int64)
    got = out.reshape(-1, case.dv)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del out
    host = {k: inp[k].cpu() for k in ("q", "k", "v")}
    return case, host, lam_gpu.cpu().numpy(), rows, got


def _tile_rows(heads, N, tile, per_tile, seed):
    """Flat rows (head * N + i): for every tile of every head its first and
    last row and `per_tile` random rows inside it."""
    g = np.random.default_rng(seed)
    out = []
    for hh in range(heads):
        for t0 in range(0, N, tile):
            t1 = min(N, t0 + tile)
            pick = {t0, t1 - 1}
            pick.update(g.integers(t0, t1, size=per_tile).tolist())
            out.extend(hh * N + r for r in sorted(pick))
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("group", range(4))
def test_multi_needle_64k_every_tile(multi_needle_64k, group):
    case, host, lam, rows, got = multi_needle_64k
    per = case.H // 4
    lo, hi = group * per * case.N, (group + 1) * per * case.N
    sel = (rows >= lo) & (rows < hi)
    tiles = np.unique(rows[sel] // 256)
    assert tiles.size == per * case.N // 256
    say("64k multi-needle workload, heads %d..%d: %d rows covering all %d tiles"
        % (group * per, (group + 1) * per - 1, int(sel.sum()), tiles.size))
    ref = run_prefill_oracle(case, host, lam, rows=rows[sel])
    compare(got[sel], ref, "bf16", "%s heads %d..%d (every tile)"
            % (case.name, group * per, (group + 1) * per - 1))


def test_v2_prefill_32k_every_tile():
    _require_gpu()
    case = W.V2_PREFILL_32K
    H = case.Hq // 2
    say("v2 prefill %s: first/last/random row of every 128-row tile of every pair" % case.name)
    inp = W.make_prefill_v2(case, device=DEV)
    lam_gpu = gpu_lambda(inp, case.layer)
    out = torch.full((case.B, H, case.N, case.D), float("nan"), dtype=torch.float32, device=DEV)
    api.diffattn_prefill_v2(inp["q"], inp["k"], inp["v"], lam_gpu, causal=case.causal, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all().item()), "v2 prefill: unwritten or non-finite outputs"
    rows = _tile_rows(case.B * H, case.N, 128, per_tile=1, seed=32)
    got = out.reshape(-1, case.D)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del out
    # Per-pair tensors for the oracle: q1 = query heads 2p, q2 = heads 2p+1,
    # keys and values of K/V head p // (Hq / (2 Hkv)).
    g = case.pairs_per_kv
    q = inp["q"].cpu()
    k = inp["k"].cpu().repeat_interleave(g, dim=1).contiguous()
    v = inp["v"].cpu().repeat_interleave(g, dim=1).contiguous()
    ref = oracle.prefill(q[:, 0::2].contiguous(), q[:, 1::2].contiguous(), k, k, v,
                         lam_gpu.cpu().numpy(), causal=case.causal, rows=rows)
    compare(got, ref, "bf16", case.name + " (every tile)")


@pytest.mark.parametrize("n", [8192, 131072])
def test_length_sweep_against_oracle(n):
    """The length-sweep workloads the benchmark times beside the step: at 8k
    every row of every head, at 128k the first, last and one random row of
    every 256-row tile of every head."""
    _require_gpu()
    case = next(c for c in W.V1_LENGTH_SWEEP if c.N == n)
    say("length sweep %s: GPU run into a NaN-filled output" % case.name)
    inp = W.make_prefill(case, device=DEV)
    lam_gpu = gpu_lambda(inp, case.layer)
    out = _run_nan_filled(case, inp, lam_gpu)
    heads = case.B * case.H
    if n <= 8192:
        rows = np.arange(heads * case.N, dtype=np.int64)
    else:
        rows = _tile_rows(heads, case.N, 256, per_tile=1, seed=n)
        assert np.unique(rows // 256).size == heads * case.N // 256
    got = out.reshape(-1, case.dv)[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del out
    host = {k: inp[k].cpu() for k in ("q", "k", "v")}
    say("length sweep %s: %d rows against the oracle" % (case.name, rows.size))
    ref = run_prefill_oracle(case, host, lam_gpu.cpu().numpy(), rows=rows)
    compare(got, ref, "bf16", "%s (%s)" % (case.name, "every row" if n <= 8192 else "every tile"))
