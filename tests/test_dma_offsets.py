"""Host-side check of the invariant the scalar-offset DMA relies on.

A buffer load's range check compares only the per-lane offset with the
buffer's byte size; the instruction's scalar offset is added after the check.
The kernels pass a stage's advance as that scalar offset (dma16_so / dma4_so)
only for stages that lie wholly inside every row: all stages of a reduction
range but its last, which is issued with per-lane checked offsets.  So for
every unchecked stage, every lane whose per-lane offset passes the check must
end inside the buffer with the scalar offset added, and every masked lane
(per-lane offset kOobOffset) must stay out of range whatever is added to it.

The per-lane offsets are formed here the way the kernels form them (the
lane -> row / chunk maps of the K-major and MN-major DMA and of the block-scale
words), for ragged and aligned shapes; nothing runs on a GPU.
"""
import itertools

import pytest

KROW = 128             # bytes of one row per K-major stage
BK = 64                # reduction rows per MN-major stage
OOB = 0x80000000       # per-lane offset of a masked lane
LIMIT = 1 << 31        # every buffer handed to a call is smaller than this


def _stages(red_bytes, stage_bytes):
    return -(-red_bytes // stage_bytes)


def _check_lane(voff, soff, size, num_records):
    """voff passes the check -> the access ends inside the buffer; a masked
    lane stays masked with or without the scalar part (no 32-bit wrap)."""
    if voff == OOB:
        assert num_records <= OOB and voff + soff < (1 << 32)
        return
    assert voff < num_records
    assert voff + soff + size <= num_records, (voff, soff, size, num_records)


@pytest.mark.parametrize("rows,row_elems,esz", [
    (1, 8, 2), (3, 64, 2), (5, 72, 2), (17, 136, 2), (4096, 2048, 2), (7, 200, 2),
    (9, 16, 1), (3, 144, 1), (33, 2048, 1), (2, 4160, 1),
])
def test_kmajor_operand_stages(rows, row_elems, esz):
    """K-major operand tiles (x / W rows, dY rows in dX; 2-byte or 8-bit
    elements, rows a multiple of 16 bytes): lane p of an instruction loads row
    chunk c = (p % 8) ^ ((row >> 1) & 7) of its row, 16 bytes at
    row_offset + 16 c; an unchecked stage kt adds kt * 128 as the scalar
    offset, the last stage is checked per lane (chunk live when
    kt * 128 + 16 c < row bytes)."""
    rowbytes = row_elems * esz
    assert rowbytes % 16 == 0
    nrec = rows * rowbytes
    KI = _stages(rowbytes, KROW)
    for row in {0, rows // 2, rows - 1}:
        for lane_row in range(16):                 # the swizzle repeats every 16 rows
            for p in range(8):
                c = p ^ ((lane_row >> 1) & 7)
                base = row * rowbytes + c * 16
                for kt in range(KI - 1):           # unchecked: every stage but the last
                    _check_lane(base, kt * KROW, 16, nrec)
                kt = KI - 1
                off = base + kt * KROW if kt * KROW + c * 16 < rowbytes else OOB
                _check_lane(off, 0, 16, nrec)
    # a masked row keeps kOobOffset in every stage
    for kt in range(KI):
        _check_lane(OOB, kt * KROW, 16, nrec)


@pytest.mark.parametrize("N,K", [(64, 8), (72, 64), (136, 200), (1408, 4096), (2048, 2048),
                                 (65, 24), (128, 256), (17, 520)])
def test_mnmajor_weight_stages(N, K):
    """dX's weight operand, MN-major: lane p of instruction i loads reduction
    row r = 2 (w * 32/NW + i) + p // 32 of the stage and column chunk
    ch = (p % 32) ^ ((r & 3) << 2), i.e. W[e] byte r * 2K + 2 (kc0 + 8 ch),
    masked when the column is past K; stage kt adds kt * 64 * 2K."""
    rowbytes = 2 * K
    nrec = N * rowbytes                            # one expert's slice
    KI = _stages(N, BK)
    NW = 4
    for kc0 in range(0, K, 256):
        for w, i, p in itertools.product(range(NW), range(32 // NW), range(64)):
            r = 2 * (w * (32 // NW) + i) + p // 32
            ch = (p % 32) ^ ((r & 3) << 2)
            col = kc0 + 8 * ch
            voff = r * rowbytes + 2 * col if col < K else OOB
            for kt in range(KI - 1):
                _check_lane(voff, kt * BK * rowbytes, 16, nrec)
            kt = KI - 1                            # checked: row and column both in range
            n = kt * BK + r
            off = n * rowbytes + 2 * col if (n < N and col < K) else OOB
            _check_lane(off, 0, 16, nrec)


@pytest.mark.parametrize("rows,K", [(1, 128), (9, 256), (4096, 2048), (3, 7168), (5, 384)])
def test_block_scale_words(rows, K):
    """Block scales (one byte per 32 reduction elements): a row's 4 scale bytes
    of stage kt (128 elements) at row * K/32 + 4 kt; the row offset per lane,
    4 kt as the scalar offset."""
    kblk = K // 32
    nrec = rows * kblk
    KI = _stages(K, 128)
    for row in {0, rows - 1}:
        for kt in range(KI - 1):
            _check_lane(row * kblk, 4 * kt, 4, nrec)
        _check_lane(row * kblk + 4 * (KI - 1), 0, 4, nrec)
    for kt in range(KI):
        _check_lane(OOB, 4 * kt, 4, nrec)


@pytest.mark.parametrize("rows,K", [(1, 512), (9, 1024), (4096, 2048), (3, 7168), (64, 7168)])
def test_block_scale_groups_of_four_stages(rows, K):
    """The masked decode's scale ring with K a multiple of 512: a row's 16
    bytes of four stages (512 elements) at row * K/32 + 16 g, the row offset
    per lane and 16 g as the scalar offset for every group g, the last one
    included (K/32 is a multiple of 16, so a group never crosses a row end);
    without that multiple, 4 kt per stage for every stage, the last included."""
    assert K % 512 == 0
    kblk = K // 32
    nrec = rows * kblk
    for row in {0, rows - 1}:
        assert (row * kblk) % 16 == 0
        for g in range(K // 512):
            _check_lane(row * kblk, 16 * g, 16, nrec)
        for kt in range(K // 128):
            _check_lane(row * kblk, 4 * kt, 4, nrec)
    for g in range(K // 512):
        _check_lane(OOB, 16 * g, 16, nrec)


def test_size_limit_keeps_masked_lanes_masked():
    """With every buffer below 2^31 bytes, kOobOffset is out of range of all
    of them, and adding any in-buffer advance to it cannot wrap to a small
    offset."""
    for nrec in (1, 4096, LIMIT - 1):
        for soff in (0, 128, LIMIT - 1):
            _check_lane(OOB, soff, 16, nrec)
