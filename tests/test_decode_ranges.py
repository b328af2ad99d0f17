"""Model of the split-KV decode's key ranges (host-side check of the index
arithmetic in csrc/decode.hip, no GPU).

The split kernel lays the (sequence, KV head) segments of the cache end to
end and gives workgroup w the keys [w*R, (w+1)*R); it writes one partial state
per segment it touches, into slot w - seg0 // R of that segment, and the
workgroup holding a segment's last piece writes the segment's piece count,
which the merge kernel reads.  The model below follows the split kernel step
by step and checks, for many length mixes and grid sizes, that every key of
every valid sequence is streamed exactly once, that every slot the merge reads
(below the count) was written exactly once, that every valid segment gets a
count, and that no slot index reaches the workspace bound the host sizes.
"""
import random

import pytest

STEP = 128          # keys per loop step of a workgroup (4 waves x 32 keys)
RANGE_MIN = 4096    # shortest range


def valid_len(lens, b, max_len):
    L = lens[b]
    return 0 if (L < 1 or L > max_len) else L


def range_len(total, nranges):
    r = -(-total // nranges)
    r = -(-r // STEP) * STEP
    return max(r, RANGE_MIN)


def max_splits(max_len):
    return -(-max_len // RANGE_MIN) + 1


def grid(B, Hkv, max_len, cus=256):
    return min(2 * cus, B * Hkv * -(-max_len // RANGE_MIN))


def split_kernel(lens, Hkv, max_len, G):
    """Pieces (b, g, c0, cend, slot) written by each workgroup, in its order."""
    B = len(lens)
    total = sum(valid_len(lens, b, max_len) * Hkv for b in range(B))
    R = range_len(total, G)
    out = []
    for w in range(G):
        r0 = w * R
        if r0 >= total:
            continue
        r1 = min(total, r0 + R)
        b, L, base = 0, valid_len(lens, 0, max_len), 0
        while base + L * Hkv <= r0:
            base += L * Hkv
            b += 1
            assert b < B
            L = valid_len(lens, b, max_len)
        g = (r0 - base) // L
        seg0 = base + g * L
        pos = r0
        while pos < r1:
            c0 = pos - seg0
            cend = min(L, r1 - seg0)
            assert 0 <= c0 < cend <= L
            out.append((w, b, g, c0, cend, w - seg0 // R))
            pos = seg0 + cend
            if pos < r1:
                assert cend == L
                seg0 += L
                g += 1
                if g == Hkv:
                    g = 0
                    while True:
                        b += 1
                        assert b < B
                        L = valid_len(lens, b, max_len)
                        if L:
                            break
    return out, R


def check(lens, Hkv, max_len, G):
    pieces, R = split_kernel(lens, Hkv, max_len, G)
    S = max_splits(max_len)
    seen = {}
    slots = {}
    counts = {}
    for (w, b, g, c0, cend, slot) in pieces:
        assert 0 <= slot < S
        if cend == valid_len(lens, b, max_len):
            assert (b, g) not in counts
            counts[(b, g)] = slot + 1
        key = (b, g, slot)
        assert key not in slots, "slot written twice"
        slots[key] = (c0, cend)
        for k in range(c0, cend, 97):       # sampled, plus both ends below
            seen[(b, g, k)] = seen.get((b, g, k), 0) + 1
        for k in (c0, cend - 1):
            seen.setdefault((b, g, k, "end"), 0)
            seen[(b, g, k, "end")] += 1
    for b in range(len(lens)):
        L = valid_len(lens, b, max_len)
        for g in range(Hkv):
            if L == 0:
                assert not any(k[:2] == (b, g) for k in slots)
                continue
            n = counts[(b, g)]
            got = sorted((s, slots[(b, g, s)]) for s in range(n))
            # Slots 0..n-1 written, nothing beyond, pieces tile [0, L) in order.
            assert not any(k[:2] == (b, g) and k[2] >= n for k in slots)
            edge = 0
            for s, (c0, cend) in got:
                assert c0 == edge
                edge = cend
            assert edge == L
    for k, cnt in seen.items():
        assert cnt == 1 or (len(k) == 4 and cnt <= 2), k   # an end key of a 1-key piece counts twice


@pytest.mark.parametrize("seed", range(40))
def test_ranges_random_mixes(seed):
    rng = random.Random(seed)
    B = rng.choice([1, 2, 3, 7, 16, 32])
    Hkv = rng.choice([1, 2, 8, 16])
    max_len = rng.choice([1, 100, 2048, 4097, 65536])
    lens = [rng.randint(1, max_len) for _ in range(B)]
    # Some sequences without keys (zero, negative, too long): skipped.
    for b in range(B):
        if rng.random() < 0.15:
            lens[b] = rng.choice([0, -5, max_len + 1])
    if all(valid_len(lens, b, max_len) == 0 for b in range(B)):
        lens[0] = max_len
    G = grid(B, Hkv, max_len, cus=rng.choice([1, 8, 256]))
    check(lens, Hkv, max_len, G)


def test_ranges_bench_shape():
    # 32 sequences, 8 KV heads, lengths in [4096, 65536], 512 workgroups.
    rng = random.Random(7)
    lens = [rng.randint(4096, 65536) for _ in range(32)]
    G = grid(32, 8, 65536)
    assert G == 512
    pieces, R = split_kernel(lens, 8, 65536, G)
    check(lens, 8, 65536, G)
    per_wg = {}
    for (w, b, g, c0, cend, slot) in pieces:
        per_wg[w] = per_wg.get(w, 0) + cend - c0
    loads = list(per_wg.values())
    # Every workgroup but the last streams exactly R keys.
    assert max(loads) == R and sorted(loads)[1] == R


def test_ranges_degenerate():
    check([1], 1, 1, 1)
    check([5, 0, 7], 2, 8, grid(3, 2, 8))
    check([2048] * 4, 8, 2048, grid(4, 8, 2048))
    check([65536] * 2, 1, 65536, 1)      # one workgroup: every segment in pieces of one range
