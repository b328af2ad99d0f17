"""Host model of every global address the fused bf16 prefill kernels form
(prefill_pp.hip: both maps per wave for d <= 64 and its single-map form; the
one-map-per-wave kernel for d = 128), checked against the bounds of the tensor
it points into, for every supported shape, several token strides and the V2
head layout.  CPU only: the kernels' address arithmetic is restated here
lane by lane.

What the kernels address:
  * Key/value tiles through raw buffer descriptors (copies that write LDS):
    copy block `id` of a tile is 1 KB; lane l fetches 16 bytes at byte offset
    coff(id, l) from the descriptor base src + head offset + t * TK * ld; the
    descriptor's extent is rows * ld * 2 bytes (rows = keys left in the tile),
    so the hardware returns zeros for offsets at or beyond it.  Property: every
    offset below the extent lies inside its tensor (for the K2 half of a packed
    tensor: inside the whole [.., 2d] tensor), and all of it fits the kernels'
    32-bit offset arithmetic.
  * Query fragments: flat 16-byte loads of the lane's own row (rows past N
    are not loaded).
  * Outputs: flat 16-byte stores of rows below N.

Also the index of the first 32-key sub-tile a wave masks, which the d <= 64
kernel computes once per wave: it must select exactly the sub-tiles the
masking rule names, for every length and row block.
"""
import itertools

import numpy as np
import pytest

TK = 64          # keys per LDS tile
WAVE = 64


def k_swz(d, row):
    kc, rpb = d // 8, 256 // (d * 2)
    return (row // rpb) % kc


def v_swz(dv, row):
    return 4 * (row & 3) if dv == 128 else 2 * ((row >> 1) & 1)


def copy_blocks(d, dv, nk, waves):
    """(id, region, lane offsets without the tile stride) of every copy block
    of a tile: region 0/1 = the two key halves, 2 = values."""
    kc, vc = d // 8, dv // 8
    krowb, vrowb = d * 2, dv * 2
    kblk = TK * krowb // 1024
    stage = nk * TK * krowb + TK * vrowb
    ncopy = stage // 1024
    assert ncopy % waves == 0
    lane = np.arange(WAVE)
    out = []
    for cid in range(ncopy):
        if cid < nk * kblk:
            row = (cid % kblk) * (1024 // krowb) + lane // kc
            chunk = (lane % kc) ^ np.array([k_swz(d, r) for r in row])
            out.append((cid, cid // kblk, row, chunk))
        else:
            row = (cid - nk * kblk) * (1024 // vrowb) + lane // vc
            chunk = (lane % vc) ^ np.array([v_swz(dv, r) for r in row])
            out.append((cid, 2, row, chunk))
    return out


def check_copies(d, dv, nk, waves, N, B, H, ld, heads):
    """heads: list of (tensor sizes in elements, element offsets of the key
    and value head bases, element offsets of K1/K2 pointers)."""
    blocks = copy_blocks(d, dv, nk, waves)
    ntile = -(-N // TK)
    for (k_len, v_len, k1_ptr, k2_ptr, koff, voff) in heads:
        for cid, region, row, chunk in blocks:
            ldr = ld["v"] if region == 2 else ld["k"]
            width = dv if region == 2 else d
            ptr = 0 if region == 2 else (k1_ptr if region == 0 else k2_ptr)
            hoff = voff if region == 2 else koff
            tlen = v_len if region == 2 else k_len
            coff = row * ldr * 2 + chunk * 16                      # bytes, per lane
            assert coff.max() < 2 ** 31
            assert TK * ldr * 2 < 2 ** 32                          # unsigned tile stride
            for t in range(ntile):
                rows = min(N - t * TK, TK)
                extent = rows * ldr * 2
                assert extent < 2 ** 31
                base = (ptr + hoff + t * TK * ldr) * 2             # bytes from the tensor start
                live = coff < extent
                # each live 16-byte fetch lies inside its row's `width`
                # elements and inside the tensor
                assert np.all(row[live] < rows)
                assert np.all(chunk[live] * 16 + 16 <= width * 2)
                end = base + coff[live] + 16
                assert end.max(initial=0) <= tlen * 2, (d, dv, N, cid, t)
                assert (base + coff[live]).min(initial=0) >= 0


def v1_heads(B, H, N, d, dv, ldk, ldv, packed):
    heads = []
    k_len = B * H * N * ldk
    v_len = B * H * N * ldv
    for b, h in itertools.product(range(B), range(H)):
        koff = (b * H + h) * N * ldk
        voff = (b * H + h) * N * ldv
        heads.append((k_len, v_len, 0, d if packed else 0, koff, voff))
    return heads


def outputs_and_queries(B, H, N, d, dv, bm, ldq, q_len, qoff_of, q2_ptr):
    """Query loads and output stores of every lane of every workgroup; q2_ptr
    is the q2 pointer's element offset in its tensor (d in a packed tensor, 0
    for a tensor of its own)."""
    row_tiles = -(-N // bm)
    lane = np.arange(WAVE)
    col, half = lane & 31, lane >> 5
    for bh in range(B * H):
        for tile in range(row_tiles):
            for rb in range(bm // 32):
                my_row = tile * bm + rb * 32 + col
                ok = my_row < N
                for st in range(d // 16):
                    for qptr in (0, q2_ptr):       # q1, then q2
                        off = qoff_of(bh) + my_row[ok] * ldq + half[ok] * 8 + st * 16 + qptr
                        assert np.all(off >= 0) and np.all(off + 8 <= q_len)
                # output rows: dv fp32 channels per row, 16-byte stores
                orow = (bh * N + my_row[ok]) * dv
                assert np.all(orow + dv <= B * H * N * dv)


@pytest.mark.parametrize("d,dv", [(64, 128), (64, 64), (32, 64)])
@pytest.mark.parametrize("layout", ["packed", "separate", "padded"])
def test_two_map_kernel_addresses(d, dv, layout):
    for N in (1, 31, 33, 63, 64, 65, 127, 257, 300):
        B, H = 2, 3
        if layout == "packed":
            ldq = ldk = 2 * d
            ldv = dv
        elif layout == "separate":
            ldq = ldk = d
            ldv = dv
        else:
            ldq = ldk = 2 * d + 8
            ldv = dv + 24
        heads = v1_heads(B, H, N, d, dv, ldk, ldv, packed=layout != "separate")
        if layout == "separate":   # K2 is its own tensor: same shape, its own base
            heads = [(k, v, 0, 0, ko, vo) for (k, v, _, _, ko, vo) in heads]
        check_copies(d, dv, 2, 8, N, B, H, {"k": ldk, "v": ldv}, heads)
        outputs_and_queries(B, H, N, d, dv, 256, ldq, B * H * N * ldq,
                            lambda bh: bh * N * ldq, 0 if layout == "separate" else d)


@pytest.mark.parametrize("d,dv", [(64, 128), (64, 64)])
def test_single_map_kernel_addresses(d, dv):
    for N in (1, 65, 300):
        heads = v1_heads(2, 2, N, d, dv, 2 * d, dv, packed=False)
        check_copies(d, dv, 1, 8, N, 2, 2, {"k": 2 * d, "v": dv}, heads)


@pytest.mark.parametrize("shared_keys", [True, False])
def test_one_map_per_wave_kernel_addresses_v2(shared_keys):
    # V2 layout at D = 128: q [B][Hq][N][D], k, v [B][Hkv][N][D]; pair p uses
    # query heads 2p, 2p+1 and K/V head p // (Hq / (2 Hkv)).
    D = 128
    for (B, Hq, Hkv, N) in ((2, 8, 2, 1), (1, 8, 4, 129), (2, 4, 1, 300), (1, 16, 2, 64)):
        g = Hq // (2 * Hkv)
        heads = []
        for b, p in itertools.product(range(B), range(Hq // 2)):
            kv = p // g
            off = (b * Hkv + kv) * N * D
            heads.append((B * Hkv * N * D, B * Hkv * N * D, 0, 0, off, off))
        check_copies(D, D, 1 if shared_keys else 2, 8, N, B, Hq // 2, {"k": D, "v": D}, heads)
        # q2 = q + N*D: the odd query head of the pair, one head further on
        outputs_and_queries(B, Hq // 2, N, D, D, 128, D, B * Hq * N * D,
                            lambda bh: ((bh // (Hq // 2)) * Hq + 2 * (bh % (Hq // 2))) * N * D, N * D)


def test_largest_bf16_stride_fits_32_bit_offsets():
    # The C ABI refuses bf16 token strides of 2^24 elements and more; at the
    # largest accepted stride every offset, tile stride and extent of a 64-row
    # tile still fits the kernels' 32-bit arithmetic.
    ld = (1 << 24) - 8
    for d, dv in ((64, 128), (32, 64)):
        for cid, region, row, chunk in copy_blocks(d, dv, 2, 8):
            assert (row * ld * 2 + chunk * 16).max() < 2 ** 31
        assert TK * ld * 2 < 2 ** 31
    assert TK * (1 << 24) * 2 >= 2 ** 31        # the first refused stride would not fit


def first_masked_subtile(N, wrow0, causal, bn=32):
    """The kernels' precomputed index of the first 32-key sub-tile that needs
    masking, as they form it."""
    j_end = (N - bn) // bn + 1 if N >= bn else 0
    if not causal:
        return j_end
    x = wrow0 - bn + 1
    return min(j_end, 0 if x < 0 else x // bn + 1)


@pytest.mark.parametrize("causal", [False, True])
def test_first_masked_subtile_matches_the_masking_rule(causal):
    # A sub-tile j needs masking iff it reaches past the sequence end
    # (32j + 32 > N) or, causally, past the row block's first row
    # (32j + 31 > first row); the kernels test j >= the precomputed index.
    for N in list(range(1, 300)) + [4095, 4096, 4097]:
        nsub = -(-N // 32)
        for wrow0 in range(0, N, 32):
            jm = first_masked_subtile(N, wrow0, causal)
            for j in range(nsub + 1):
                masked = (32 * j + 32 > N) or (causal and 32 * j + 31 > wrow0)
                assert masked == (j >= jm), (N, wrow0, causal, j)
