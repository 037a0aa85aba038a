"""Offset arithmetic of the GEMM's K-contiguous stage copy (csrc/gemm.hip, CopyKC),
replayed on the host for ragged tiles.

A raw buffer load checks only its per-lane offset against the descriptor's
record count; the scalar offset is added after the check.  So every row a load
reaches must be reachable through the per-lane offset alone: a load whose
per-lane offset passes the check must stay inside the operand once the scalar
offset is added, and a load for a row past the operand must fail the check.
The replay mirrors prepare() / issue() of CopyKC: every copy instruction has its
own per-lane offset (its row and chunk), and a step adds only the K position
as the scalar offset.
"""
from __future__ import annotations

import itertools

import pytest

KBK = 64            # K depth of one stage (bf16 elements)
ROW_BYTES = KBK * 2
OOB = 0x80000000


def swz(row):
    return (row & 7) ^ ((row >> 3) & 7)


def copy_loads(R, NW, ld, rows, K, kt, rowstep_in_soff=False):
    """Yield (row, chunk, voffset, soffset, records) for every lane load of step kt.

    rowstep_in_soff replays a wrong variant (one per-lane offset for every
    instruction, the row step added through the scalar offset)."""
    n_instr = R // 8 // NW
    records = min(rows * ld * 2, 0x7FFFFFFF)
    step = NW * 8 * ld * 2
    kbytes = kt * ROW_BYTES
    tail = (K % KBK) != 0 and kt == (K + KBK - 1) // KBK - 1
    for wave, lane in itertools.product(range(NW), range(64)):
        for i in range(n_instr):
            row = (wave + i * NW) * 8 + (lane >> 3)
            kc = (lane & 7) ^ swz(row)
            if rowstep_in_soff:
                row0 = wave * 8 + (lane >> 3)
                o = row0 * ld * 2 + ((lane & 7) ^ swz(row0)) * 16
                kc = (lane & 7) ^ swz(row0)
                soff = kbytes + i * step
            else:
                o = (row * ld * 2 + kc * 16) & 0xFFFFFFFF
                soff = kbytes
            if tail and kt * KBK + kc * 8 >= K:
                o = OOB
            yield row, kc, o, soff, records


def violations(R, NW, ld, rows, K, **kw):
    bad = []
    for kt in range((K + KBK - 1) // KBK):
        for row, kc, o, soff, records in copy_loads(R, NW, ld, rows, K, kt, **kw):
            checked_ok = o < records
            if not checked_ok:
                continue          # reads zeros: fine whatever the row
            byte = o + soff
            if row >= rows or byte >= rows * ld * 2:
                bad.append((kt, row, kc, o, soff))
                continue
            # inside the operand the load reads its own row's chunk at k < K
            k = kt * KBK + kc * 8
            assert byte == row * ld * 2 + k * 2, (row, kc, o, soff)
            assert k < K
    return bad


CASES = [
    # (R, NW, ld, rows, K): eight-wave tiles (kOne) and four-wave tiles, full and ragged
    (256, 8, 512, 256, 512),
    (256, 8, 512, 5, 512),         # T = 4097 on a 256-row tile: 5 rows in the last tile
    (256, 8, 520, 133, 520),       # ragged rows and a partial K step
    (256, 8, 72, 64, 72),          # exactly the first instruction's rows
    (256, 8, 72, 65, 72),
    (128, 8, 264, 100, 264),
    (256, 4, 512, 77, 512),
    (128, 4, 136, 9, 136),
    (64, 4, 64, 1, 64),
]


@pytest.mark.parametrize("R,NW,ld,rows,K", CASES)
def test_every_checked_load_stays_inside_the_operand(R, NW, ld, rows, K):
    assert violations(R, NW, ld, rows, K) == []


def test_row_step_in_the_scalar_offset_reads_past_a_ragged_tile():
    """A copy that puts the row step into the scalar offset reads rows past the
    operand on a ragged tile; the replay sees it (and nothing on a full tile)."""
    bad = violations(256, 8, 512, 5, 512, rowstep_in_soff=True)
    assert bad and max(b[1] for b in bad) >= 64
    assert violations(256, 8, 512, 256, 512, rowstep_in_soff=True) == []


def test_per_lane_offsets_fit_32_bits_on_the_widest_tiles():
    """Per-lane offsets reach (R - 1) * ld * 2 + 112; the planner keeps R * ld * 2
    below 2^31, which for 384-row tiles allows strides up to 2^21 elements."""
    for R, ld in ((256, (1 << 22) - 8), (384, (1 << 21) - 8)):
        assert R * ld * 2 < (1 << 31)
        assert (R - 1) * ld * 2 + 7 * 16 < (1 << 32)
