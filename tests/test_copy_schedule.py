"""Model of the fused prefill kernels' global->LDS copy schedule (the
ping-pong kernels: two wave groups, three LDS stages of 64-key tiles), checked
over many key extents.

Rule under test, per wave of either group: before the loop, tiles 0 and 1 are
issued and the wave waits for tile 0; at the end of its matrix phase of every
odd step j it issues tile (j+3)/2 (if it exists) and then waits until at most
CPW copies (tile (j+1)/2 + 1's, if that tile exists) are in flight.  The loop
has one workgroup barrier per step: group 0 places it after its softmax phase
and group 1 between its matrix and softmax phases, so interval j (ending with
the j-th loop barrier) holds the matrix phase of step j of both groups.
Invariants: every copy is issued once, into a stage whose previous tile (t-3)
was last read in an earlier interval; a tile's copies of every wave are
complete in an interval before its first read; nothing is in flight at the
end.  Host-side logic only: no GPU.
"""
import pytest


def simulate(kv_end, cpw, tk=64, bn=32):
    ntile = -(-kv_end // tk)
    nsub = -(-kv_end // bn)
    last_read = {}          # tile -> last global phase that reads it
    first_read = {}
    issue_phase = {}        # (group, tile) -> phase
    done_phase = {}         # (group, tile) -> phase of the wait that completed it
    for g in (0, 1):
        issued = [0] * cpw + ([1] * cpw if ntile > 1 else [])
        complete = len(issued) - (cpw if ntile > 1 else 0)
        seen = [0]          # copies already credited to their tile

        def mark(ph):
            # copies complete in issue order: credit those newly complete
            while seen[0] < complete:
                t = issued[seen[0]]
                seen[0] += 1
                if seen[0] == len(issued) or issued[seen[0]] != t:
                    done_phase.setdefault((g, t), ph)
        mark(-1)
        for j in range(nsub + 1):
            p = j                   # the interval of both groups' M(j)
            # The matrix phase of step j reads the keys of sub-tile j and the
            # values of sub-tile max(j-1, 0) (taking every step as visible).
            for t in {j // 2, max(j - 1, 0) // 2}:
                if t < ntile:
                    last_read[t] = max(last_read.get(t, -1), p)
                    first_read[t] = min(first_read.get(t, 1 << 30), p)
            if j & 1:
                ti, tw = (j + 3) >> 1, (j + 1) >> 1
                if ti < ntile:
                    assert (g, ti) not in issue_phase
                    issue_phase[(g, ti)] = p
                    issued += [ti] * cpw
                n = cpw if tw + 1 < ntile else 0
                assert sum(1 for t in issued if t > tw) <= n
                complete = max(complete, len(issued) - n)
                mark(p)
        assert complete == len(issued), "copies still in flight at the end"
    return ntile, last_read, first_read, issue_phase, done_phase


# Copies per wave and tile in the kernels built: 2 (d = 32, dv = 64), 3
# (d = 64, dv = 64; single map d = 64, dv = 128), 4 (d = 64, dv = 128; d = 128
# with one shared key tensor) and 6 (d = 128 with two key tensors).
@pytest.mark.parametrize("cpw", [2, 3, 4, 6])
def test_copy_schedule_invariants(cpw):
    extents = list(range(1, 64 * 40 + 1)) + [4095, 4096, 4097, 32768, 65536]
    for kv_end in extents:
        ntile, last_read, first_read, issue_phase, done_phase = simulate(kv_end, cpw)
        assert sorted(issue_phase) == sorted((g, t) for g in (0, 1) for t in range(2, ntile))
        for (g, t), ph in issue_phase.items():
            # the stage's previous tile has no read at or after this phase
            assert last_read.get(t - 3, -1) < ph, (kv_end, g, t)
        for t in range(ntile):
            for g in (0, 1):
                assert done_phase[(g, t)] < first_read[t], (kv_end, g, t)
