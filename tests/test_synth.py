"""The seeded input generator: known answers, determinism, the stated recipes."""

import numpy as np
import pytest

import synth


def test_philox_known_answers():
    # Known-answer vectors published with Random123 for Philox-4x32-10
    # (Salmon et al., SC'11): counter, key -> output.
    cases = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2,
         [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in cases:
        assert list(synth.philox4x32_10(ctr, key)) == want


def test_round_bf16_nearest_even():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3e38, -1e-40]])
    bits = synth.round_bf16(v)
    got = synth.bf16_to_f64(bits)
    # the two bf16 neighbours of got bracket v and got is the nearer one
    up = synth.bf16_to_f64((bits.astype(np.int32) + 1).astype(np.uint16))
    dn = synth.bf16_to_f64((bits.astype(np.int32) - 1).astype(np.uint16))
    nz = np.abs(got) > 0
    err = np.abs(got - v)
    # no bf16 neighbour is nearer to v
    assert np.all(err[nz] <= np.abs(up - v)[nz])
    assert np.all(err[nz] <= np.abs(dn - v)[nz])
    # ties go to the even significand
    assert synth.round_bf16(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert synth.round_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82


def test_deterministic_and_row_ranges_agree():
    a = synth.make_inputs(1)
    b = synth.make_inputs(1)
    for name in ("x", "k", "v", "grad_out", "wh", "we"):
        assert np.array_equal(a[name], b[name])
    # a row range of a workload is the same rows of the whole workload
    for cfg in (1, 3):
        full = synth.make_inputs(cfg, rows=(0, 96)) if cfg == 3 else synth.make_inputs(cfg)
        part = synth.make_inputs(cfg, rows=(17, 53))
        for name in ("x", "k", "v", "grad_out"):
            assert np.array_equal(full[name][17:53], part[name])


def test_streams_differ():
    d = synth.make_inputs(1)
    assert not np.array_equal(d["x"], d["k"])
    assert not np.array_equal(d["x"], d["v"])
    assert not np.array_equal(d["wh"], d["we"])


def test_normal_moments_and_weights():
    d = synth.make_inputs(2, rows=(0, 64))
    x = synth.bf16_to_f64(d["x"])
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    for w in (d["wh"], d["we"]):
        assert w.dtype == np.float32
        assert abs(w.mean() - 1.0) < 0.01 and abs(w.std() - 0.1) < 0.01


def test_correlated_k_recipe():
    d = synth.make_inputs(3, rows=(0, 256))
    x = synth.bf16_to_f64(d["x"])
    k = synth.bf16_to_f64(d["k"])
    rho = d["rho"]
    assert rho.min() >= -1 and rho.max() <= 1
    c = np.array([np.corrcoef(x[t], k[t])[0, 1] for t in range(256)])
    assert np.max(np.abs(c - rho)) < 0.06
    assert abs(k.std() - 1.0) < 0.02


def test_stress_row_classes():
    T = 65537
    for name in ("x", "k", "v"):
        s = synth.stress_row_scales(0, T, name)
        assert np.sum(s == 1e3) == 66 and np.sum(s == 0.0) == 66
    sx = synth.stress_row_scales(0, T, "x")
    sk = synth.stress_row_scales(0, T, "k")
    assert not np.array_equal(sx, sk)
    # the stress workload honours the row classes
    zr = int(np.nonzero(sx == 0)[0][0])
    br = int(np.nonzero(sx == 1e3)[0][0])
    for r, want_zero in ((zr, True), (br, False)):
        d = synth.make_inputs(5, rows=(r, r + 1), with_grad=False)
        row = synth.bf16_to_f64(d["x"])[0]
        assert np.all(row == 0) == want_zero
        if not want_zero:
            assert np.median(np.abs(row)) > 100
    # Student-t(3) rows at a small width: zero rows are zero, scaled rows large
    t = synth.student_t3_bf16(0, synth.STREAM_X, 4, 4096, np.array([1.0, 1e3, 0.0, 1.0]))
    tf = synth.bf16_to_f64(t)
    assert np.all(tf[2] == 0)
    assert np.median(np.abs(tf[1])) > 300 * np.median(np.abs(tf[0]))
    # heavy tails: kurtosis of t(3) is infinite; sample excess kurtosis is large
    z = tf[[0, 3]].ravel()
    kurt = np.mean((z - z.mean()) ** 4) / np.var(z) ** 2
    assert kurt > 6
    # variance of t(3) is 3
    big = synth.student_t3_bf16(0, synth.STREAM_V, 64, 4096, np.ones(64))
    bf = synth.bf16_to_f64(big)
    assert 2.0 < bf.var() < 4.5 and abs(np.median(bf)) < 0.02


def test_zipf_ranks_small_vocabulary_exact():
    # vocab 4, s = 1: weights 1, 1/2, 1/3, 1/4 (sum 25/12), so the CDF is
    # 12/25, 18/25, 22/25, 1; uniforms just below and just above each step
    # land on either side of it
    cuts = np.array([12, 18, 22]) / 25
    u = np.concatenate([cuts - 1e-12, cuts + 1e-12, [0.0, 0.999999]])
    assert synth.zipf_ranks(u, 4, 1.0).tolist() == [0, 1, 2, 1, 2, 3, 0, 3]


def test_zipf_id_map_is_a_bijection():
    V = synth.HASH_CONFIGS["b8s4096_zipf"].vocab
    ids = synth.zipf_rank_to_id(np.arange(V), V)
    assert ids.min() == 0 and ids.max() == V - 1 and len(np.unique(ids)) == V


def test_zipf_token_frequencies():
    c = synth.HASH_CONFIGS["b8s4096_zipf"]
    t = synth.hash_tokens(c).ravel()
    assert np.array_equal(t, synth.hash_tokens(c).ravel())           # seeded
    assert t.min() >= 0 and t.max() < c.vocab
    n = t.size
    harmonic = np.sum(1.0 / np.arange(1, c.vocab + 1))
    for r in range(4):
        p = 1.0 / ((r + 1) * harmonic)
        tok = int(synth.zipf_rank_to_id(r, c.vocab))
        cnt = int(np.sum(t == tok))
        assert abs(cnt - n * p) < 5 * np.sqrt(n * p * (1 - p)), (r, cnt, n * p)
    # the uniform recipe stays uniform: no id carries more than a few tokens
    u = synth.hash_tokens(synth.HASH_CONFIGS["b8s4096"]).ravel()
    assert np.bincount(u, minlength=c.vocab).max() < 10
