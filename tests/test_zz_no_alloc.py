"""The allocation-free decode entry point against the workspace entry point.

diffattn_decode_noalloc keeps its partial states in the library's fixed
per-device scratch array instead of a caller workspace; with the same inputs
it runs the same kernels with the same grid, so its output must equal
diffattn_decode's bit for bit.  Two calls in a row, the second on a smaller
input (the scratch still holds the first call's states), then sizes beyond
the scratch, which are refused with nothing launched.  Also checked against
the oracle within the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_prefill_amd import api
from differential_attention_prefill_amd import workloads as W

from parity_util import compare, gpu_lambda, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.load_library()


def _both(case, fill_unused=None):
    inp = W.make_decode(case, device=DEV, fill_unused=fill_unused)
    lam = gpu_lambda(inp, case.layer)
    ref_ws = api.diffattn_decode(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam)
    out = torch.full((case.B, case.Hq // 2, case.D), float("nan"), device=DEV)
    api.diffattn_decode_noalloc(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], lam, out)
    torch.cuda.synchronize()
    return inp, lam, ref_ws, out


def test_noalloc_decode_matches_workspace_entry_twice():
    # First call: 8 sequences of 4k..20k keys, 32 query heads over 8 KV heads.
    big = W.scaled_decode(W.V2_DECODE, B=8, Lmin=4096, Lmax=20000, seed=71)
    need = api.diffattn_decode_workspace_bytes(big.B, big.Hq, big.Hkv, big.D, big.Lmax)
    assert need <= api.DECODE_SCRATCH_BYTES
    say("no-alloc decode, call 1: %s B=%d Lmax=%d (%d workspace bytes)" % (big.name, big.B, big.Lmax, need))
    inp, lam, ref_ws, out = _both(big)
    assert torch.equal(out, ref_ws), "call 1: differs from the workspace entry point"
    ref = oracle.decode(inp["q"].cpu(), inp["k_cache"].cpu(), inp["v_cache"].cpu(),
                        inp["seq_lens"].cpu(), lam.cpu().numpy())
    compare(out.cpu().numpy(), ref, "bf16", "no-alloc decode call 1")

    # Second call, smaller: 3 sequences, 8 query heads over 2 KV heads, unused
    # cache slots NaN; the scratch still holds call 1's partial states.
    small = W.scaled_decode(W.V2_DECODE, B=3, Hq=8, Hkv=2, Lmin=100, Lmax=1500, seed=72)
    say("no-alloc decode, call 2: B=%d Hq=%d Hkv=%d Lmax=%d" % (small.B, small.Hq, small.Hkv, small.Lmax))
    inp2, lam2, ref_ws2, out2 = _both(small, fill_unused=float("nan"))
    assert torch.equal(out2, ref_ws2), "call 2: differs from the workspace entry point"
    ref2 = oracle.decode(inp2["q"].cpu(), inp2["k_cache"].cpu(), inp2["v_cache"].cpu(),
                         inp2["seq_lens"].cpu(), lam2.cpu().numpy())
    compare(out2.cpu().numpy(), ref2, "bf16", "no-alloc decode call 2")


def test_noalloc_decode_refuses_sizes_beyond_scratch():
    lib = api.load_library()
    B, Hq, Hkv, D, L = 64, 32, 8, 128, 1 << 20
    need = api.diffattn_decode_workspace_bytes(B, Hq, Hkv, D, L)
    assert need > api.DECODE_SCRATCH_BYTES
    say("no-alloc decode refuses %d bytes of partial states" % need)
    small = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    lam = torch.zeros(Hq // 2, device=DEV)
    out = torch.full((B, Hq // 2, D), 7.0, device=DEV)
    # Only the sizes are read before the refusal: no kernel runs on these buffers.
    st = lib.diffattn_decode_noalloc(small.data_ptr(), small.data_ptr(), small.data_ptr(),
                                     lens.data_ptr(), B, Hq, Hkv, D, L, lam.data_ptr(),
                                     out.data_ptr(), None)
    assert st == 3, st
    assert "scratch" in lib.diffattn_last_error().decode()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all().item())
