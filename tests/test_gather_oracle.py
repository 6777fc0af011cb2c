"""Pins of the hashed multi-table gather oracle (oracle.engram_gather): the
retrieval step of the Engram memory (zhichai.net TileKernels page, section
"5. Engram": N-gram hashed embedding tables with O(1) lookup). The gather is
an exact copy, so it is pinned by a hand-built example, the out-of-range
rule, and agreement of the table pattern generators."""

import numpy as np
import torch

import oracle
import synth


def test_hand_example():
    # two tables packed in one buffer: table 0 = rows 0..2, table 1 = rows 3..6
    data = np.arange(7 * 2, dtype=np.uint16).reshape(7, 2)      # row r = [2r, 2r+1]
    idx = np.array([[2, 0], [0, 3], [1, 1]])
    out = oracle.engram_gather(idx, data, [0, 3], [3, 4])
    want = np.array([[[4, 5], [6, 7]],        # t0: table0 row2, table1 row0 (= row 3)
                     [[0, 1], [12, 13]],      # t1: table0 row0, table1 row3 (= row 6)
                     [[2, 3], [8, 9]]],       # t2: table0 row1, table1 row1 (= row 4)
                    dtype=np.uint16)
    assert np.array_equal(out, want)


def test_out_of_range_gives_zero_rows():
    data = np.arange(7 * 2, dtype=np.uint16).reshape(7, 2) + 1
    idx = np.array([[3, -1], [-5, 4], [2, 3]])
    out = oracle.engram_gather(idx, data, [0, 3], [3, 4])
    assert np.all(out[0, 0] == 0) and np.all(out[0, 1] == 0)
    assert np.all(out[1, 0] == 0) and np.all(out[1, 1] == 0)
    assert np.array_equal(out[2, 0], data[2]) and np.array_equal(out[2, 1], data[6])


def test_table_pattern_generators_agree_and_are_distinct():
    d = 40
    t = torch.empty((50, d), dtype=torch.bfloat16)
    synth.fill_table_bits_torch(t, 7, 10, 40, d)
    got = t.view(torch.int16).numpy().view(np.uint16)[10:50]
    want = synth.table_bits_np(7, np.arange(40), d)
    assert np.array_equal(got, want)
    vals = (want.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(vals)) and np.all((np.abs(vals) >= 1) & (np.abs(vals) < 2))
    # rows differ from each other and from the same rows of another table
    assert len({r.tobytes() for r in want}) == 40
    assert not np.array_equal(want, synth.table_bits_np(8, np.arange(40), d))
