"""Pins of the N-gram hash oracle (oracle/engram_hash_oracle.cpp).

The hash of the zhichai.net TileKernels page, section "5. Engram", combines
an N-gram's token ids with XOR and multiplication and maps the result to a
table index. The page gives no constants or examples, so the oracle is pinned
by hand-derived known answers (tests/golden/engram_hash_known_answers.txt,
including 64-bit wrap-around and the pad id), by the special case N = 1, and
by properties a wrong window, a wrong pad rule or a leak between sequences
would break."""

import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "engram_hash_known_answers.txt")


def known_answers():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, toks, n, a, M, pad, want = (p.strip() for p in line.split("|"))
        yield (name, [int(t) for t in toks.split()], int(n), [int(x) for x in a.split()],
               int(M), int(pad), [int(w) for w in want.split()])


@pytest.mark.parametrize("case", list(known_answers()), ids=lambda c: c[0])
def test_known_answers(case):
    name, toks, n, a, M, pad, want = case
    mult = np.zeros((1, 1, 4), dtype=np.uint64)
    mult[0, 0, :n] = a
    tokens = np.array([toks], dtype=np.uint32).view(np.int32)
    got = oracle.engram_hash(tokens, [n], mult, np.array([[M]], dtype=np.uint32), pad)
    assert got[0, :, 0, 0].tolist() == want


def test_splitmix64_published_vector():
    # first outputs of SplitMix64 seeded with 1234567 (the reference
    # implementation's test vector)
    assert synth.splitmix64(1234567, 5) == [6457827717110365317, 3203168211198807973,
                                            9817491932198370423, 4593380528125082431,
                                            16408922859458223821]


def test_range_and_shape():
    c = synth.HASH_CONFIGS["tiny"]
    p = synth.hash_params(c)
    t = synth.hash_tokens(c)
    out = oracle.engram_hash(t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    assert out.shape == (c.B, c.S, 2, 8)
    assert np.all(out >= 0) and np.all(out < p["table_size"][None, None])


def test_unigram_reduces_to_modular_product():
    # N = 1 with products below 2^64: index = (tok * a) mod M, plain integers
    r = np.random.default_rng(0)
    tokens = r.integers(0, 1 << 20, size=(2, 50)).astype(np.int32)
    a = r.integers(1, 1 << 40, size=(1, 3)).astype(np.uint64) | np.uint64(1)
    mult = np.zeros((1, 3, 4), dtype=np.uint64)
    mult[0, :, 0] = a[0]
    M = np.array([[97, 65536, 1000003]], dtype=np.uint32)
    out = oracle.engram_hash(tokens, [1], mult, M, 0)
    for j in range(3):
        want = [(int(t) * int(a[0, j])) % int(M[0, j]) for t in tokens.ravel()]
        assert out[..., 0, j].ravel().tolist() == want


def test_window_is_exactly_n_tokens():
    # changing a token n or more positions back leaves position s unchanged;
    # changing any of the last n tokens changes (almost surely) the index
    c = synth.HASH_CONFIGS["tiny"]
    p = synth.hash_params(c)
    t = synth.hash_tokens(c)[:1].copy()
    base = oracle.engram_hash(t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    s = 20
    for back in range(0, 5):
        t2 = t.copy()
        t2[0, s - back] = (t2[0, s - back] + 1) % c.vocab
        out = oracle.engram_hash(t2, p["ngram"], p["mult"], p["table_size"], p["pad"])
        for l, n in enumerate(p["ngram"]):
            same = np.array_equal(out[0, s, l], base[0, s, l])
            assert same == (back >= n), (back, n)


def test_sequences_are_independent_and_pad_starts_each():
    c = synth.HASH_CONFIGS["tiny"]
    p = synth.hash_params(c)
    t = synth.hash_tokens(c)
    out = oracle.engram_hash(t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    for b in range(c.B):
        alone = oracle.engram_hash(t[b:b + 1], p["ngram"], p["mult"], p["table_size"], p["pad"])
        assert np.array_equal(out[b], alone[0])
    # prepending pad tokens explicitly gives the same indices as the pad rule
    padded = np.concatenate([np.full((c.B, 3), p["pad"], dtype=np.int32), t], axis=1)
    out_p = oracle.engram_hash(padded, p["ngram"], p["mult"], p["table_size"], p["pad"])
    assert np.array_equal(out_p[:, 3:], out)


def test_order_matters_through_the_multipliers():
    # with distinct multipliers, (u, w) and (w, u) hash differently (a hash
    # that forgot the per-position multiplier would make them equal)
    mult = np.zeros((1, 1, 4), dtype=np.uint64)
    mult[0, 0, :2] = [0x9E3779B97F4A7C15, 0xC2B2AE3D27D4EB4F]
    M = np.array([[(1 << 31) - 1]], dtype=np.uint32)
    a = oracle.engram_hash(np.array([[11, 22]], dtype=np.int32), [2], mult, M, 0)
    b = oracle.engram_hash(np.array([[22, 11]], dtype=np.int32), [2], mult, M, 0)
    assert a[0, 1, 0, 0] != b[0, 1, 0, 0]


def test_indices_spread_over_the_table():
    # multiplicative hashing of distinct N-grams fills a prime-sized table
    # close to uniformly (chi-square with M - 1 degrees of freedom)
    mult = np.zeros((1, 1, 4), dtype=np.uint64)
    mult[0, 0, :2] = [0x9E3779B97F4A7C15 | 1, 0xBF58476D1CE4E5B9 | 1]
    M = 1021
    r = np.random.default_rng(5)
    t = r.integers(0, 1 << 17, size=(1, 200000)).astype(np.int32)
    out = oracle.engram_hash(t, [2], mult, np.array([[M]], dtype=np.uint32), 0)
    counts = np.bincount(out.ravel(), minlength=M)
    expect = out.size / M
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < M - 1 + 6 * np.sqrt(2 * (M - 1))
