"""Host model of the matrix-core kernels' index maps (no GPU).

The GPU parity tests check results; these check the layout invariants the
kernels rely on, for every lane:
- the code words each lane hands to an MFMA after the two cross-half swaps
  cover every column of a 128-column segment exactly once, and each MFMA sees
  columns of one 64-column group only (its scale is per group);
- the activation slots of the A operand name the same columns as the codes;
- line loads: the LDS slots the lanes write (rows 0-7 and 8-15 of a 128-byte
  window) and read (their row and quarter of either segment) form a bijection
  that returns the right bytes, and no 16-lane pass of a write or a read hits
  one 16-byte bank slot twice.
"""
from __future__ import annotations

import itertools


def slot_columns(h, t, g):
    """Columns (within a segment) of MFMA slot (h, t) for lane group g, as the kernel lays them out."""
    c0 = 64 * h + 32 * (g % 2) + 8 * (t + 2 * (g // 2))
    return list(range(c0, c0 + 8))


def loaded_words(g):
    """Columns of the 4 words a lane of group g loads: quarter g of the segment (32 columns)."""
    return [list(range(32 * g + 8 * j, 32 * g + 8 * j + 8)) for j in range(4)]


def permlane32_swap(a, b):
    """v_permlane32_swap on per-lane values: returns (new a, new b).

    New a holds a's low half and b's low half (moved up); new b holds a's high
    half (moved down) and b's high half.
    """
    na = [a[l] if l < 32 else b[l - 32] for l in range(64)]
    nb = [a[l + 32] if l < 32 else b[l] for l in range(64)]
    return na, nb


def test_code_words_cover_each_segment_once_per_group():
    # word j of lane l: columns of its own quarter (lane group l // 16)
    words = [[loaded_words(l // 16)[j] for l in range(64)] for j in range(4)]
    s02 = permlane32_swap(words[0], words[2])
    s13 = permlane32_swap(words[1], words[3])
    # slot (h, t): (0,0) = new word 0, (1,0) = new word 2, (0,1) = new word 1, (1,1) = new word 3
    slots = {(0, 0): s02[0], (1, 0): s02[1], (0, 1): s13[0], (1, 1): s13[1]}
    for n in range(16):                       # weight row of the B operand (lane % 16)
        seen = []
        for (h, t), per_lane in slots.items():
            cols = [c for g in range(4) for c in per_lane[n + 16 * g]]
            assert len(set(cols)) == 32
            assert all(64 * h <= c < 64 * h + 64 for c in cols), (h, t)    # one group per MFMA
            for g in range(4):
                assert per_lane[n + 16 * g] == slot_columns(h, t, g)          # the A operand's columns
            seen += cols
        assert sorted(seen) == list(range(128))                              # each column exactly once


def test_line_load_transpose_is_a_conflict_free_bijection():
    def f(sg, q):
        return 2 * (sg * 4 + q)

    data = {}                                 # LDS slot -> (row, segment, quarter) of the 16 bytes it holds
    for inst, base in ((0, 0), (1, 8)):        # even unit: rows 0-7; odd unit: rows 8-15
        slots = []
        for l in range(64):
            row, sg, q = base + l // 8, (l % 8) // 4, l % 4    # lane's 16 bytes: window bytes 16*(l%8)
            slot = sg * 64 + q * 16 + (row ^ f(sg, q))
            assert 0 <= slot < 128 and slot not in data
            data[slot] = (row, sg, q)
            slots.append(slot)
        for p in range(4):                     # 16-lane passes of a 16-byte write
            assert len({s % 16 for s in slots[16 * p:16 * p + 16]}) == 16
    assert len(data) == 128
    for sg in range(2):
        reads = []
        for l in range(64):
            n, g = l % 16, l // 16
            slot = sg * 64 + g * 16 + (n ^ f(sg, g))
            assert data[slot] == (n, sg, g)                # the lane's own row and quarter of segment sg
            reads.append(slot)
        for p in range(4):
            assert len({s % 16 for s in reads[16 * p:16 * p + 16]}) == 16


def test_load_offsets_cover_each_tile_window_once():
    """Line loads of a segment pair read every byte of a 16-row, 128-byte window once."""
    for rowbytes in (2048, 7168, 256):
        seen = set()
        for hi, l in itertools.product((0, 1), range(64)):
            off = (l // 8) * rowbytes + 16 * (l % 8) + hi * 8 * rowbytes
            row, col = divmod(off, rowbytes)
            for b in range(16):
                seen.add((row, col + b))
        assert seen == {(r, c) for r in range(16) for c in range(128)}


def dpp_row_ror(vals, n):
    """DPP row_ror:n on per-lane values: lane i of each 16-lane row receives lane (i - n) mod 16."""
    return [vals[16 * (l // 16) + (l % 16 - n) % 16] for l in range(64)]


def test_compact_activation_loads_fill_every_slot_of_the_pass_rows():
    """Compact x loads (XQ row sets per 16 lanes) plus row rotations give lane r < 16/XQ
    of every lane group slots 0-3 of pass row r, the words the full 4-load form reads."""
    rotations = {1: [None, None, None, None], 2: [None, None, 8, 8], 4: [None, 12, 8, 4]}
    for xq, rots in rotations.items():
        R, L = 16 // xq, 4 // xq
        # load j of lane l: (row, slot, lane group) it fetched
        loads = []
        for j in range(L):
            per_lane = []
            for l in range(64):
                m, g = l % 16, l // 16
                per_lane.append((m % R, (m // R) * L + j, g))
            loads.append(per_lane)
        for i in range(4):
            src = loads[i % L]
            got = src if rots[i] is None else dpp_row_ror(src, rots[i])
            for l in range(64):
                m, g = l % 16, l // 16
                if m < R:
                    assert got[l] == (m, i, g), (xq, i, l, got[l])
                # the word's columns are those of the codes in slot i of the lane's group
                row, slot, gg = got[l]
                assert gg == g


def test_staged_activations_are_a_conflict_free_exchange():
    """Staged activation form (up to 8 rows): load k of lane l reads word l % 16 of row
    4k + l // 16; LDS slot of (row, word) is row*16 + (word ^ row). Every (row, word) of a
    segment lands in its own slot, each lane reads back the words of its A operand slots,
    and no 16-lane pass of a write or a read hits one 16-byte bank slot twice (lanes m and
    m + 8 read one address, a broadcast)."""
    data = {}
    for k in range(2):
        slots = []
        for l in range(64):
            row, word = 4 * k + l // 16, l % 16
            slot = row * 16 + (word ^ row)
            assert 0 <= slot < 128 and slot not in data
            data[slot] = (row, word)
            slots.append(slot)
        for p in range(4):
            assert len({s % 16 for s in slots[16 * p:16 * p + 16]}) == 16
    assert len(data) == 128
    for i in range(4):
        h, t = i >> 1, i & 1
        reads = []
        for l in range(64):
            m, g = l % 16, l // 16
            row = m & 7
            word = 8 * h + 4 * (g & 1) + t + 2 * (g >> 1)
            slot = row * 16 + (word ^ row)
            assert data[slot] == (row, word)
            assert list(range(8 * word, 8 * word + 8)) == slot_columns(h, t, g)
            reads.append(slot)
        for p in range(4):
            part = reads[16 * p:16 * p + 16]
            assert len({s % 16 for s in part}) == len(set(part)) == 8
