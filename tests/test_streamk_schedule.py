"""The stream-K partition as the kernels compute it, checked on the CPU.

The stream-K kernels (hgemm_streamk_kernel, hgemm_dma_streamk_kernel,
sgemm_streamk_kernel) and their fix-up kernels share one piece of integer
arithmetic, restated here from their source: the cut tiles' W = T_r * S
(tile, k step) iterations are split over Gs workgroups, workgroup w taking
[w*W/Gs, (w+1)*W/Gs); a piece that does not cover a whole tile goes to slot
2w (it holds the range's last iteration) or 2w + 1; the fix-up of cut tile t
sums the pieces of workgroups owner(t*S) .. owner(t*S + S - 1) in that order,
reading slot 2g + side with side = 0 iff g's last iteration lies in t.  The
piece count comes from streamk_groups (gemm_problem.hpp).  These tests check
the invariants the kernels rely on: every iteration is computed exactly once,
no workgroup writes more than its two slots, the fix-up finds exactly the
pieces that were written, and a tile inside one range is stored whole.
"""
import math

import pytest


def streamk_groups(G, cut, steps, ratio):
    W = cut * steps
    s = int(math.sqrt(steps * ratio / cut) + 0.5)
    s = max(1, min(s, steps))
    return min(cut * s, G, W)


def pieces(W, S, Gs):
    """(workgroup, local tile, kb, ke, slot or None) as the main kernel walks them."""
    out = []
    for w in range(Gs):
        begin, end = w * W // Gs, (w + 1) * W // Gs
        it = begin
        while it < end:
            local = it // S
            kb = it - local * S
            ke = min(end - local * S, S)
            it = local * S + ke
            if kb == 0 and ke == S:
                out.append((w, local, kb, ke, None))
            else:
                side = 0 if end - 1 < (local + 1) * S else 1
                out.append((w, local, kb, ke, 2 * w + side))
    return out


def fixup_reads(local, W, S, Gs):
    """Slots the fix-up of cut tile `local` adds, in order (empty: not cut)."""
    g0 = ((local * S + 1) * Gs - 1) // W
    g1 = ((local * S + S) * Gs - 1) // W
    if g0 == g1:
        return []
    reads = []
    for g in range(g0, g1 + 1):
        end = (g + 1) * W // Gs
        side = 0 if end - 1 < (local + 1) * S else 1
        reads.append(2 * g + side)
    return reads


CASES = [(cut, S, G) for G in (256, 1024) for cut in (1, 4, 16, 32, 100, 255)
         for S in (1, 2, 16, 63, 129)]


@pytest.mark.parametrize("cut,S,G", CASES)
@pytest.mark.parametrize("ratio", [14, 40, 140, 1e9])
def test_partition_covers_every_iteration_once(cut, S, G, ratio):
    W = cut * S
    Gs = streamk_groups(G, cut, S, ratio)
    assert 1 <= Gs <= min(G, W)
    ps = pieces(W, S, Gs)
    seen = [0] * W
    for w, local, kb, ke, _ in ps:
        assert 0 <= kb < ke <= S
        for k in range(kb, ke):
            seen[local * S + k] += 1
    assert seen == [1] * W
    # at most two partial pieces per workgroup, in distinct slots of its own
    slots = [slot for *_, slot in ps if slot is not None]
    assert len(slots) == len(set(slots))
    assert all(slot // 2 == w for w, *_, slot in ps if slot is not None)


@pytest.mark.parametrize("cut,S,G", CASES)
@pytest.mark.parametrize("ratio", [14, 40, 140, 1e9])
def test_fixup_reads_exactly_the_written_pieces(cut, S, G, ratio):
    W = cut * S
    Gs = streamk_groups(G, cut, S, ratio)
    ps = pieces(W, S, Gs)
    for local in range(cut):
        written = sorted((w, slot) for w, t, kb, ke, slot in ps if t == local and slot is not None)
        whole = [p for p in ps if p[1] == local and p[4] is None]
        reads = fixup_reads(local, W, S, Gs)
        if whole:
            # stored whole by one workgroup: no partial pieces, no fix-up
            assert not written and not reads and len(whole) == 1
        else:
            # the fix-up adds the written slots in increasing workgroup order
            assert reads == [slot for _, slot in written]
            assert len(reads) >= 2
            # and their k ranges tile [0, S) in that order
            ranges = sorted((kb, ke) for w, t, kb, ke, slot in ps if t == local)
            assert ranges[0][0] == 0 and ranges[-1][1] == S
            assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))


def test_balanced_split_examples():
    # the cases the measurements quote: 16 cut tiles of 16 steps on the general
    # kernel, 16 of 64 on the direct-load one, 32 of 63 on the fp32 one
    assert streamk_groups(256, 16, 16, 40) == 96
    assert streamk_groups(256, 16, 64, 14) == 112
    assert streamk_groups(1024, 32, 63, 140) == 544
    # a huge ratio spreads over every workgroup (or every iteration)
    assert streamk_groups(256, 16, 16, 1e9) == 256
    assert streamk_groups(256, 4, 3, 1e9) == 12
