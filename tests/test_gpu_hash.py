"""GPU parity of the N-gram hash (tk_engram_hash through the C ABI) against
the integer oracle: bit-exact on every index."""

import random

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eg(cuda_device):
    import engram_conditional_memory_amd as m
    m.load_library()
    return m


def gpu_hash(eg, dev, tokens, ngram, mult, table_size, pad):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to(dev)
    out = eg.tk_engram_hash(t, ngram, mult, table_size, pad)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "b8s4096", "b8s4096_zipf", "b64s4096", "b1024s4096"])
def test_hash_workloads(eg, cuda_device, name):
    # every index of every workload, the 4.2 M-token throughput one included
    c = synth.HASH_CONFIGS[name]
    p = synth.hash_params(c)
    t = synth.hash_tokens(c)
    want = oracle.engram_hash(t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    got = gpu_hash(eg, cuda_device, t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("B,S,L,K,ngram", [
    (1, 1, 1, 1, (1,)),          # one token, generic path
    (5, 1000, 2, 8, (2, 3)),      # ragged S (not a block multiple)
    (3, 257, 3, 3, (1, 2, 4)),    # 9 tables: 4-byte stores
    (2, 300, 4, 8, (4, 3, 2, 1)), # 32 tables
    (7, 33, 1, 4, (4,)),
    (2, 300, 2, 2, (1, 1)),       # N = 1 everywhere, 16-byte stores
    (4, 513, 1, 5, (3,)),         # 5 tables: 4-byte stores, N = 3
    (3, 129, 3, 4, (2, 1, 2)),    # 12 tables, largest N = 2
])
def test_hash_shapes_and_orders(eg, cuda_device, B, S, L, K, ngram):
    r = np.random.default_rng(B * 1000 + S)
    tokens = r.integers(-(1 << 31), (1 << 31) - 1, size=(B, S), dtype=np.int64).astype(np.int32)
    mult = r.integers(0, 1 << 63, size=(L, K, 4), dtype=np.int64).astype(np.uint64)
    mult = mult * np.uint64(2) + np.uint64(1)
    sizes = r.integers(1, 1 << 31, size=(L, K), dtype=np.int64).astype(np.uint32)
    sizes.flat[0] = 1
    sizes.flat[-1] = 1 << 31                       # the largest supported size
    pad = 0xFFFFFFFF
    want = oracle.engram_hash(tokens, ngram, mult, sizes, pad)
    got = gpu_hash(eg, cuda_device, tokens, ngram, mult, sizes, pad)
    assert np.array_equal(got, want)
    if L * K > 1:
        assert np.all(got[..., 0, 0] == 0)         # table of size 1


@pytest.mark.parametrize("ngram", [(1, 2), (2, 1), (1, 3), (3, 1), (2, 3), (3, 2), (1, 4),
                                   (4, 1), (2, 4), (4, 2), (3, 4), (4, 3), (3, 3)])
def test_hash_two_layers_of_eight_tables(eg, cuda_device, ngram):
    """Two layers of eight tables, the pages' layout, run an instance with
    each layer's order fixed at compile time, one per ordered pair of
    orders (and the shared one when both are equal): every pair, on a ragged
    batch, bit-exact against the oracle."""
    r = np.random.default_rng(1000 + 10 * ngram[0] + ngram[1])
    B, S = 3, 777
    tokens = r.integers(-(1 << 31), (1 << 31) - 1, size=(B, S), dtype=np.int64).astype(np.int32)
    mult = r.integers(0, 1 << 63, size=(2, 8, 4), dtype=np.int64).astype(np.uint64)
    mult = mult * np.uint64(2) + np.uint64(1)
    sizes = r.integers(1, 1 << 31, size=(2, 8), dtype=np.int64).astype(np.uint32)
    sizes[1, 7] = 1 << 31
    pad = int(r.integers(0, 1 << 32))
    want = oracle.engram_hash(tokens, ngram, mult, sizes, pad)
    got = gpu_hash(eg, cuda_device, tokens, ngram, mult, sizes, pad)
    assert np.array_equal(got, want)


def test_hash_empty(eg, cuda_device):
    import torch
    c = synth.HASH_CONFIGS["tiny"]
    p = synth.hash_params(c)
    t = torch.empty((0, 5), dtype=torch.int32, device=cuda_device)
    out = eg.tk_engram_hash(t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    assert out.shape == (0, 5, 2, 8)


def test_hash_modulus_at_its_edges(eg, cuda_device):
    """The reduction h mod M at hashes chosen next to multiples of M, at the
    top of the 64-bit range, and at table sizes 1, 2, powers of two, 2^31 - 1
    and 2^31. With N = 1 the hash of table q at position 0 is tok * mult[q]
    mod 2^64; an odd token is invertible modulo 2^64, so mult[q] =
    target * tok^-1 puts that hash at any chosen target."""
    r = np.random.default_rng(2024)
    big = random.Random(2024)          # for integers beyond 64-bit numpy ranges
    M64 = (1 << 64) - 1
    sizes_all = [1, 2, 3, 7, 1 << 16, 524287, 524288, (1 << 30) + 1, (1 << 31) - 1, 1 << 31]
    sizes_all += [int(x) for x in r.integers(1, 1 << 31, size=22)]
    checked = 0
    for call in range(24):
        K = 32
        sizes = np.array([sizes_all[(call + q) % len(sizes_all)] for q in range(K)],
                         dtype=np.uint64)
        tok0 = int(r.integers(0, 1 << 31)) * 2 + 1          # odd, as an unsigned 32-bit id
        inv = pow(tok0, -1, 1 << 64)
        targets = []
        for q in range(K):
            M = int(sizes[q])
            top = M64 // M
            k = big.randrange(max(top - 3, 0), top + 1) if call % 3 == 0 else \
                big.randrange(0, top + 1)
            cand = [M64, M64 - 1, k * M, k * M - 1, k * M + M - 1, 0, M - 1]
            targets.append(cand[(call + q) % len(cand)] % (1 << 64))
        mult = np.zeros((1, K, 4), dtype=np.uint64)
        for q in range(K):
            mult[0, q, 0] = np.uint64((targets[q] * inv) % (1 << 64))
        S = 5
        tokens = r.integers(0, 1 << 32, size=(1, S), dtype=np.int64)
        tokens[0, 0] = tok0
        tokens = tokens.astype(np.uint32).view(np.int32)
        want = oracle.engram_hash(tokens, (1,), mult, sizes.astype(np.uint32).reshape(1, K), 0)
        got = gpu_hash(eg, cuda_device, tokens, (1,), mult,
                       sizes.astype(np.uint32).reshape(1, K), 0)
        assert np.array_equal(got, want), call
        # position 0 hashes to the targets; check those against Python integers
        row = got.reshape(S, K)[0].astype(np.int64)
        assert [int(v) for v in row] == [t % int(M) for t, M in zip(targets, sizes)], call
        checked += K
    assert checked == 24 * 32


@pytest.mark.timeout(300)
def test_hash_output_beyond_2_31_elements(eg, cuda_device):
    """One sequence of 2^27 + 1000 tokens: its 2 x 8 indices per token pass
    the 32-bit element range (2^31 + 16000 of them, 8.6 GB), so the offsets
    of the last waves need 64 bits. The first, a middle and the last 4096
    positions are compared with the oracle, run on those positions and the
    two tokens before them (the 3-gram window)."""
    import torch
    c = synth.HASH_CONFIGS["b8s4096"]
    p = synth.hash_params(c)
    S = (1 << 27) + 1000
    r = np.random.default_rng(27)
    tokens = r.integers(0, c.vocab, size=(1, S), dtype=np.int32)
    t = torch.from_numpy(tokens).to(cuda_device)
    out = eg.tk_engram_hash(t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    torch.cuda.synchronize()
    assert out.numel() > (1 << 31)
    back = max(p["ngram"]) - 1
    for a in (0, S // 2, S - 4096):
        lo = max(0, a - back)
        want = oracle.engram_hash(tokens[:, lo:a + 4096], p["ngram"], p["mult"],
                                  p["table_size"], p["pad"])[:, a - lo:]
        got = out[:, a:a + 4096].cpu().numpy()
        assert np.array_equal(got, want), a
    del out, t
    torch.cuda.empty_cache()
