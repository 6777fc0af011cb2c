"""GPU parity of the hashed multi-table gather (tk_engram_gather through the
C ABI) against the oracle, and of the whole memory-read step (hash, then
gather) against oracle hash then oracle gather: bit-exact."""

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


def say(msg):
    print(msg, flush=True)


def bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def packed_tables(dev, Q, rows, d):
    """Device buffer with table q in rows [q * max_rows, q * max_rows + rows[q])."""
    import torch
    stride = int(max(rows))
    data = torch.empty((Q * stride, d), dtype=torch.bfloat16, device=dev)
    for q in range(Q):
        synth.fill_table_bits_torch(data, q, q * stride, int(rows[q]), d)
    offsets = np.arange(Q, dtype=np.int64) * stride
    return data, offsets


def expected_rows(idx, rows, d):
    """Expected gather from the table pattern, recomputed on the host."""
    T, Q = idx.shape
    out = np.zeros((T, Q, d), dtype=np.uint16)
    for q in range(Q):
        ok = (idx[:, q] >= 0) & (idx[:, q] < rows[q])
        out[ok, q] = synth.table_bits_np(q, idx[ok, q], d)
    return out


def test_gather_tiny_against_oracle(eg, cuda_device):
    import torch
    c = synth.GATHER_CONFIGS["tiny"]
    rows = np.array(synth.primes_below(c.rows, c.tables), dtype=np.uint32)
    data, off = packed_tables(cuda_device, c.tables, rows, c.d)
    r = np.random.default_rng(1)
    idx = r.integers(0, rows.min(), size=(c.T, c.tables)).astype(np.int32)
    idx[0, 0] = -1                         # out of range: zero row
    idx[1, 3] = int(rows[3])               # one past the end: zero row
    idx[2, 5] = -(1 << 31)
    out = eg.tk_engram_gather(torch.from_numpy(idx).to(cuda_device), data, off, rows)
    torch.cuda.synchronize()
    want = oracle.engram_gather(idx, bits(data), off, rows)
    assert np.array_equal(bits(out), want)
    assert np.array_equal(want, expected_rows(idx, rows, c.d))


@pytest.mark.parametrize("T,Q,d", [(1, 1, 8), (3, 3, 8), (5, 7, 200), (2, 32, 64), (2, 2, 8192)])
def test_gather_shapes(eg, cuda_device, T, Q, d):
    import torch
    rows = np.array([17 + 3 * q for q in range(Q)], dtype=np.uint32)
    data, off = packed_tables(cuda_device, Q, rows, d)
    r = np.random.default_rng(T * 100 + Q)
    idx = r.integers(-3, int(rows.max()) + 3, size=(T, Q)).astype(np.int32)
    out = eg.tk_engram_gather(torch.from_numpy(idx).to(cuda_device), data, off, rows)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.engram_gather(idx, bits(data), off, rows))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tokens_recipe", ["b8s4096", "b8s4096_zipf"])
def test_memory_read_full_size(eg, cuda_device, tokens_recipe):
    """tokens -> tk_engram_hash -> tk_engram_gather at the H=7168 workload's
    size (32768 tokens, 16 tables of ~2^19 rows x 448 bf16), with uniform
    and with Zipf(1) token frequencies: every index is compared with the
    oracle hash, every gathered row with the table pattern recomputed on
    the host."""
    import torch
    hc = synth.HASH_CONFIGS[tokens_recipe]
    gc = synth.GATHER_CONFIGS["t32768_d448"]
    p = synth.hash_params(hc)
    tokens = synth.hash_tokens(hc)
    sizes = p["table_size"].reshape(-1)
    say(f"[memory read] tables: {gc.tables} x {1 << 19} rows x {gc.d}")
    data, off = packed_tables(cuda_device, gc.tables, np.full(gc.tables, 1 << 19), gc.d)
    t_dev = torch.from_numpy(tokens).to(cuda_device)
    idx_dev = eg.tk_engram_hash(t_dev, p["ngram"], p["mult"], p["table_size"], p["pad"])
    out = eg.tk_engram_gather(idx_dev.view(hc.B, hc.S, -1), data, off, sizes)
    torch.cuda.synchronize()
    idx = idx_dev.cpu().numpy().reshape(gc.T, gc.tables)
    want_idx = oracle.engram_hash(tokens, p["ngram"], p["mult"], p["table_size"], p["pad"])
    assert np.array_equal(idx, want_idx.reshape(gc.T, gc.tables))
    got = bits(out).reshape(gc.T, gc.tables, gc.d)
    del out, data
    torch.cuda.empty_cache()
    say("[memory read] comparing rows")
    for a in range(0, gc.T, 4096):
        sl = slice(a, a + 4096)
        assert np.array_equal(got[sl], expected_rows(idx[sl], sizes, gc.d)), sl


@pytest.mark.timeout(300)
def test_gather_output_beyond_2_31_elements(eg, cuda_device):
    """300000 tokens x 16 tables x 448 bf16: the output's 2.15e9 elements
    pass the 32-bit range, so the offsets of the last tokens need 64 bits.
    Indices are uniform over each table plus a few out of range; the first,
    a middle and the last 4096 tokens are compared with the table pattern."""
    import torch
    T, Q, d = 300000, 16, 448
    rows = np.full(Q, 1 << 19, dtype=np.uint32)
    data, off = packed_tables(cuda_device, Q, rows, d)
    r = np.random.default_rng(31)
    idx = r.integers(-2, (1 << 19) + 2, size=(T, Q)).astype(np.int32)
    out = eg.tk_engram_gather(torch.from_numpy(idx).to(cuda_device), data, off, rows)
    torch.cuda.synchronize()
    assert out.numel() > (1 << 31)
    for a in (0, T // 2, T - 4096):
        got = bits(out[a:a + 4096])
        assert np.array_equal(got, expected_rows(idx[a:a + 4096], rows, d)), a
    del out, data
    torch.cuda.empty_cache()


def test_memory_read_tiny_against_oracles(eg, cuda_device):
    import torch
    hc = synth.HASH_CONFIGS["tiny"]
    p = synth.hash_params(hc)
    tokens = synth.hash_tokens(hc)
    sizes = p["table_size"].reshape(-1)
    d = 16
    data, off = packed_tables(cuda_device, len(sizes), sizes, d)
    idx_dev = eg.tk_engram_hash(torch.from_numpy(tokens).to(cuda_device), p["ngram"],
                                p["mult"], p["table_size"], p["pad"])
    out = eg.tk_engram_gather(idx_dev.view(hc.B, hc.S, -1), data, off, sizes)
    torch.cuda.synchronize()
    assert out.shape == (hc.B, hc.S, len(sizes), d)
    idx = oracle.engram_hash(tokens, p["ngram"], p["mult"], p["table_size"], p["pad"])
    want = oracle.engram_gather(idx.reshape(-1, len(sizes)), bits(data), off, sizes)
    assert np.array_equal(bits(out).reshape(want.shape), want)


def test_gather_rejects_a_non_contiguous_index_tensor(eg, cuda_device):
    import torch
    rows = np.array([5, 5], dtype=np.uint32)
    data, off = packed_tables(cuda_device, 2, rows, 8)
    idx = torch.zeros((2, 4), dtype=torch.int32, device=cuda_device)[:, ::2]
    assert not idx.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        eg.tk_engram_gather(idx, data, off, rows)
    out = eg.tk_engram_gather(idx.contiguous(), data, off, rows)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.engram_gather(np.zeros((2, 2), np.int32),
                                                          bits(data), off, rows))


def test_memory_read_in_a_hip_graph(eg, cuda_device):
    """The hash and the gather allocate nothing either: hash -> gather captured
    in a HIP graph replays bit for bit like the eager calls, with eager
    writes to the outputs between the replays."""
    import torch
    dev = cuda_device
    hc = synth.HASH_CONFIGS["tiny"]
    hp = synth.hash_params(hc)
    tokens = torch.from_numpy(synth.hash_tokens(hc)).to(dev)
    sizes = hp["table_size"].reshape(-1)
    Q, width = len(sizes), 24
    table = torch.empty((Q * int(sizes.max()), width), dtype=torch.bfloat16, device=dev)
    offsets = np.arange(Q, dtype=np.int64) * int(sizes.max())
    for q in range(Q):
        synth.fill_table_bits_torch(table, q, int(offsets[q]), int(sizes[q]), width)
    idx = torch.empty((hc.B, hc.S, len(hc.ngram), hc.tables), dtype=torch.int32, device=dev)
    rows = torch.empty((hc.B, hc.S, Q, width), dtype=torch.bfloat16, device=dev)

    def read():
        eg.tk_engram_hash(tokens, hp["ngram"], hp["mult"], hp["table_size"], hp["pad"], idx)
        eg.tk_engram_gather(idx.view(hc.B, hc.S, Q), table, offsets, sizes, rows)

    read()
    torch.cuda.synchronize()
    ref = [idx.clone(), rows.clone()]
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        read()                                   # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        read()
    for i in range(4):
        idx.fill_(-7)                            # eager work between replays
        rows.view(torch.int16).fill_(0x7FC1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), i
        assert torch.equal(rows.view(torch.int16), ref[1].view(torch.int16)), i
