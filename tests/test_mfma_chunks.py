"""The matrix-core kernel's chunk bookkeeping, restated on the CPU (no GPU).

gemv_mfma_lds_kernel cuts each row into chunks of CB blocks (8 for Q8_0, 16
for Q4_0 and MXFP4), gives wave w of WT the chunks w, w + WT, ..., moves a
row's last chunk back to end at the row's end when nb is not a multiple of
CB, and zeroes the blocks of that chunk that the chunk before already
counted.  Each lane reads granules 64 v + lane of a chunk (16 bytes each,
row-major over the workgroup's 16 RT rows) into LDS at an odd granule stride
per row.  These checks walk the same index arithmetic for every lane and
show that every block of a row is counted exactly once, that every load
stays inside its row and every LDS write inside the wave's region, and that
the x prefetch past a wave's last chunk reads a valid block and is zeroed.
"""
from __future__ import annotations

import pytest

# bytes per 32-weight unit, units per chunk (Q4_K: one 144-byte super-block)
FORMATS = {"Q8_0": (34, 8), "Q4_0": (18, 16), "MXFP4": (17, 16), "Q4_K": (18, 8)}


def walk(kbytes, cb, nb, wt, rt):
    cbytes = cb * kbytes
    assert cbytes % 16 == 0
    gr = cbytes // 16
    grp = gr | 1
    rows = 16 * rt
    ng = rows * gr
    nv = (ng + 63) // 64
    rb = nb * kbytes
    nch = (nb + cb - 1) // cb

    def chunk_base(c):
        return min(cb * c, nb - cb)

    counted = [0] * nb
    for w in range(wt):
        mine = (nch - w + wt - 1) // wt if nch > w else 0
        for n in range(mine):
            c = w + wt * n
            off = chunk_base(c) * kbytes
            for lane in range(64):
                for v in range(nv):
                    g = 64 * v + lane
                    on = g < ng
                    row, q = divmod(g, gr)
                    goff = 16 * q if on else 0
                    assert 0 <= off + goff and off + goff + 16 <= rb  # the load stays in the row
                    if on:
                        assert 16 * (row * grp + q) + 16 <= rows * grp * 16  # the write stays in the wave's region
            for cc in range(cb):
                b = chunk_base(c) + cc
                assert 0 <= b < nb and cc * kbytes + kbytes <= grp * 16
                if b >= cb * c:
                    counted[b] += 1
        for u in range(mine * cb, mine * cb + 2):  # x prefetch past the wave's last chunk
            c = w + wt * (u // cb)
            bb = chunk_base(c) + u % cb
            assert 0 <= bb < nb and not bb >= cb * c
    assert counted == [1] * nb, (nb, counted)


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_every_block_once_and_every_access_in_bounds(fmt):
    kbytes, cb = FORMATS[fmt]
    nbs = list(range(cb, cb + 70)) + [192, 768, 1536]
    if fmt == "Q4_K":  # k is a multiple of 256: whole super-blocks, no chunk moved back
        nbs = [nb for nb in nbs if nb % 8 == 0]
    for nb in nbs:
        walk(kbytes, cb, nb, 8, 2)
