"""GPU parity of the N-gram hash (tk_engram_hash through the C ABI) against
the integer oracle: bit-exact on every index."""

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


@pytest.mark.parametrize("name", ["tiny", "b8s4096", "b8s4096_zipf", "b64s4096"])
def test_hash_workloads(eg, cuda_device, name):
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


def test_hash_empty(eg, cuda_device):
    import torch
    c = synth.HASH_CONFIGS["tiny"]
    p = synth.hash_params(c)
    t = torch.empty((0, 5), dtype=torch.int32, device=cuda_device)
    out = eg.tk_engram_hash(t, p["ngram"], p["mult"], p["table_size"], p["pad"])
    assert out.shape == (0, 5, 2, 8)
