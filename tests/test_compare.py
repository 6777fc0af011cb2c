"""Pins of the comparison helpers (oracle/compare.cpp) that every GPU parity
verdict rests on: relative L2 against bf16(reference), bf16 ulp distance,
per-class splits, non-finite counts and the forward-output rule."""

import numpy as np

import oracle
import synth


def bits(v):
    return synth.round_bf16(np.asarray(v, dtype=np.float64))


def test_rel_l2_and_ulps_match_a_direct_computation():
    r = np.random.default_rng(0)
    ref = r.standard_normal((20, 64))
    gpu = bits(ref).copy()
    gpu[3, 5] += 1        # one ulp away
    gpu[7, 9] += 3        # three ulps away
    st = oracle.BF16Stats()
    st.add(gpu, ref)
    # the expected figures use synth's rounding, not the comparator's own
    rb = synth.bf16_to_f64(synth.round_bf16(ref))
    g = synth.bf16_to_f64(gpu)
    want = np.linalg.norm(g - rb) / np.linalg.norm(rb)
    assert abs(st.rel_l2() - want) <= 1e-12 * want
    assert st.max_ulp() == 3 and st.count_over_1ulp() == 1 and st.nonfinite() == 0
    rows = np.linalg.norm(g - rb, axis=1) / np.linalg.norm(rb, axis=1)
    assert abs(st.max_row_rel() - rows.max()) <= 1e-12 * rows.max()


def test_ulp_distance_crosses_zero_and_counts_nan():
    ref = np.array([[1e-40, -1e-40, 0.0, 1.0]])
    gpu = np.array([[0x8001, 0x0001, 0x8000, 0x7FC0]], dtype=np.uint16)  # -tiny, +tiny, -0, NaN
    st = oracle.BF16Stats()
    st.add(gpu, ref)
    # bf16(1e-40) is the subnormal 0x0001 (about 9.2e-41); -0x0001 is 2 ulps
    # away through zero; -0 and +0 share a position; NaN counts as non-finite
    assert st.nonfinite() == 1
    st2 = oracle.BF16Stats()
    st2.add(gpu[:, :3], ref[:, :3])
    assert st2.max_ulp() == 2


def test_row_classes_are_kept_apart():
    r = np.random.default_rng(1)
    ref = r.standard_normal((6, 32))
    gpu = bits(ref).copy()
    gpu[4] = bits(ref[4] * 1.5)          # a badly wrong row in class 2
    cls = np.array([0, 0, 0, 0, 2, 0], dtype=np.uint8)
    st = oracle.BF16Stats()
    st.add(gpu, ref, cls)
    assert st.rel_l2([0]) == 0.0
    assert st.rel_l2([2]) > 0.3 and st.rel_l2() > 0.1


def test_forward_output_rule():
    # x + gate * v with heavy cancellation: a result within the tolerance
    # the gate error allows passes even when it is many ulps off
    x = np.array([[1.0, 0.5, 3.0]])
    v = np.array([[-2.0, 1.0, 1.0]])
    gate = np.array([0.5 + 1e-7])
    ref = x + gate[:, None] * v                  # [-2e-7, 1.0000001, 3.5000001]
    xb, vb = bits(x), bits(v)
    exact = bits(ref)
    res = oracle.check_out(exact, ref, xb, vb, gate)
    assert res.tolist() == [0, 0, 0, 0]
    off = exact.copy()
    off[0, 0] = bits([[0.0]])[0, 0]              # 0 instead of -2e-7: many ulps
    res = oracle.check_out(off, ref, xb, vb, gate)
    # |0 - (-2e-7)| <= 1e-5 |v| + 2^-24 (|x| + |gate v|): passes by the bound
    assert res[1] == 1 and res[2] == 1 and res[3] == 0
    bad = exact.copy()
    bad[0, 1] = bits([[1.25]])[0, 0]             # a real error on an ordinary element
    res = oracle.check_out(bad, ref, xb, vb, gate)
    assert res[3] == 1
