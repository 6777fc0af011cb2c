"""No call writes outside its outputs. Every output (and the backward's
workspace) is a window into a larger buffer whose margins hold a fixed bit
pattern; after the calls the margins must be unchanged, and the windows must
equal the outputs of an ordinary run. The shapes are ragged: T off the grid,
widths with masked tail chunks, sequences that end inside a wave."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

MARGIN = 4096          # elements on each side; keeps every window 16-byte aligned


@pytest.fixture(scope="module")
def eg(cuda_device):
    import engram_conditional_memory_amd as m
    m.load_library()
    return m


def padded(n, dtype, dev, fill_bits):
    """A buffer of n + 2 * MARGIN elements filled with `fill_bits`; returns the
    buffer and the window of n elements in its middle."""
    import torch
    itype = {torch.bfloat16: torch.int16, torch.float32: torch.int32,
             torch.int32: torch.int32}[dtype]
    buf = torch.full((n + 2 * MARGIN,), fill_bits, dtype=itype, device=dev).view(dtype)
    return buf, buf[MARGIN:MARGIN + n]


def margins_intact(buf, fill_bits):
    import torch
    itype = {torch.bfloat16: torch.int16, torch.float32: torch.int32,
             torch.int32: torch.int32}[buf.dtype]
    b = buf.view(itype)
    return bool(torch.all(b[:MARGIN] == fill_bits)) and bool(torch.all(b[-MARGIN:] == fill_bits))


def same_bits(a, b):
    import torch
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("T,H", [(1001, 7168), (37, 520), (4099, 4096), (3, 8), (257, 2048),
                                 (129, 6144), (20003, 7168), (35001, 4096)])
def test_gate_calls_write_only_their_outputs(eg, cuda_device, T, H):
    # the last two shapes walk their rows in two launches, the second short
    import torch
    dev = cuda_device
    r = np.random.default_rng(T * 31 + H)

    def up(a):
        return torch.from_numpy(synth.round_bf16(a).view(np.int16)).view(torch.bfloat16).to(dev)
    x, k, v, g = (up(r.standard_normal((T, H))) for _ in range(4))
    wh = torch.from_numpy((1 + 0.1 * r.standard_normal(H)).astype(np.float32)).to(dev)
    we = torch.from_numpy((1 + 0.1 * r.standard_normal(H)).astype(np.float32)).to(dev)
    P = eg.tk_engram_num_partials(T, H)
    fill_b, fill_f = 0x7FC1, 0x7FC00001                     # NaN patterns, never written
    bufs = {}
    for name, n, dt, fill in (("out", T * H, torch.bfloat16, fill_b),
                              ("gate", T, torch.float32, fill_f),
                              ("dx", T * H, torch.bfloat16, fill_b),
                              ("dk", T * H, torch.bfloat16, fill_b),
                              ("dv", T * H, torch.bfloat16, fill_b),
                              ("ws", P * H, torch.float32, fill_f),
                              ("dwh", H, torch.float32, fill_f),
                              ("dwe", H, torch.float32, fill_f)):
        bufs[name] = (*padded(n, dt, dev, fill), fill)
    view = {n: b[1] for n, b in bufs.items()}
    eg.tk_engram_gate_fwd(x, k, v, wh, we, out=view["out"].view(T, H), gate=view["gate"])
    eg.tk_engram_gate_bwd(g, x, k, v, wh, we, dx=view["dx"].view(T, H),
                          dk=view["dk"].view(T, H), dv=view["dv"].view(T, H),
                          workspace=view["ws"].view(P, H))
    eg.tk_engram_grad_w_reduce(view["ws"], P, H, wh, we, dwh=view["dwh"], dwe=view["dwe"])
    torch.cuda.synchronize()
    for name, (buf, _, fill) in bufs.items():
        assert margins_intact(buf, fill), f"{name}: a write landed outside the output"
    out, gate = eg.tk_engram_gate_fwd(x, k, v, wh, we)
    dx, dk, dv, ws, P2 = eg.tk_engram_gate_bwd(g, x, k, v, wh, we)
    dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P2, H, wh, we)
    torch.cuda.synchronize()
    assert P2 == P
    for name, want in (("out", out), ("gate", gate), ("dx", dx), ("dk", dk), ("dv", dv),
                       ("dwh", dwh), ("dwe", dwe)):
        assert same_bits(view[name], want.reshape(-1)), name
    assert same_bits(view["ws"], ws[:P].reshape(-1))


@pytest.mark.parametrize("T,H", [(20003, 7168), (37, 520), (1001, 7168)])
def test_fused_and_noalloc_calls_write_only_their_outputs(eg, cuda_device, T, H):
    # the fused-weight forward and backward, and the backward + reduction
    # with library-owned partials, into windows of marked buffers; each must
    # equal the plain calls bit for bit
    import torch
    dev = cuda_device
    r = np.random.default_rng(T * 7 + H)

    def up(a):
        return torch.from_numpy(synth.round_bf16(a).view(np.int16)).view(torch.bfloat16).to(dev)
    x, k, v, g = (up(r.standard_normal((T, H))) for _ in range(4))
    wh = torch.from_numpy((1 + 0.1 * r.standard_normal(H)).astype(np.float32)).to(dev)
    we = torch.from_numpy((1 + 0.1 * r.standard_normal(H)).astype(np.float32)).to(dev)
    w = eg.tk_engram_fused_weight(wh, we)
    P = eg.tk_engram_num_partials(T, H)
    fill_b, fill_f = 0x7FC1, 0x7FC00001
    bufs = {}
    for name, n, dt, fill in (("out", T * H, torch.bfloat16, fill_b),
                              ("gate", T, torch.float32, fill_f),
                              ("dx", T * H, torch.bfloat16, fill_b),
                              ("dk", T * H, torch.bfloat16, fill_b),
                              ("dv", T * H, torch.bfloat16, fill_b),
                              ("ws", P * H, torch.float32, fill_f),
                              ("ndx", T * H, torch.bfloat16, fill_b),
                              ("ndk", T * H, torch.bfloat16, fill_b),
                              ("ndv", T * H, torch.bfloat16, fill_b),
                              ("ndwh", H, torch.float32, fill_f),
                              ("ndwe", H, torch.float32, fill_f)):
        bufs[name] = (*padded(n, dt, dev, fill), fill)
    view = {n: b[1] for n, b in bufs.items()}
    eg.tk_engram_gate_fwd_fused(x, k, v, w, out=view["out"].view(T, H), gate=view["gate"])
    eg.tk_engram_gate_bwd_fused(g, x, k, v, w, dx=view["dx"].view(T, H),
                                dk=view["dk"].view(T, H), dv=view["dv"].view(T, H),
                                workspace=view["ws"].view(P, H))
    eg.tk_engram_gate_bwd_reduce_noalloc(g, x, k, v, wh, we, dx=view["ndx"].view(T, H),
                                         dk=view["ndk"].view(T, H), dv=view["ndv"].view(T, H),
                                         dwh=view["ndwh"], dwe=view["ndwe"])
    torch.cuda.synchronize()
    for name, (buf, _, fill) in bufs.items():
        assert margins_intact(buf, fill), f"{name}: a write landed outside the output"
    out, gate = eg.tk_engram_gate_fwd(x, k, v, wh, we)
    dx, dk, dv, ws, _ = eg.tk_engram_gate_bwd(g, x, k, v, wh, we)
    dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P, H, wh, we)
    torch.cuda.synchronize()
    for name, want in (("out", out), ("gate", gate), ("dx", dx), ("dk", dk), ("dv", dv),
                       ("ndx", dx), ("ndk", dk), ("ndv", dv), ("ndwh", dwh), ("ndwe", dwe)):
        assert same_bits(view[name], want.reshape(-1)), name
    assert same_bits(view["ws"], ws[:P].reshape(-1))


@pytest.mark.parametrize("B,S,L,K", [(3, 1000, 2, 8), (2, 33, 3, 3), (1, 64, 1, 4),
                                     (5, 65, 4, 8), (2, 1, 2, 8)])
def test_hash_writes_only_its_output(eg, cuda_device, B, S, L, K):
    import torch
    dev = cuda_device
    r = np.random.default_rng(B * 100 + S)
    tokens = torch.from_numpy(r.integers(0, 129280, size=(B, S)).astype(np.int32)).to(dev)
    ngram = tuple(int(n) for n in r.integers(1, 5, size=L))
    mult = (r.integers(0, 1 << 62, size=(L, K, 4), dtype=np.int64).astype(np.uint64)
            * np.uint64(2) + np.uint64(1))
    sizes = r.integers(1, 1 << 20, size=(L, K)).astype(np.uint32)
    fill = 0x5A5A5A5A
    buf, win = padded(B * S * L * K, torch.int32, dev, fill)
    eg.tk_engram_hash(tokens, ngram, mult, sizes, 7, out=win.view(B, S, L, K))
    torch.cuda.synchronize()
    assert margins_intact(buf, fill)
    want = oracle.engram_hash(tokens.cpu().numpy(), ngram, mult, sizes, 7)
    assert np.array_equal(win.view(B, S, L, K).cpu().numpy(), want)


@pytest.mark.parametrize("T,Q,d", [(33, 16, 448), (5, 3, 8), (130, 7, 200)])
def test_gather_writes_only_its_output(eg, cuda_device, T, Q, d):
    import torch
    dev = cuda_device
    r = np.random.default_rng(T + Q + d)
    rows = r.integers(1, 50, size=Q).astype(np.uint32)
    offsets = np.concatenate([[0], np.cumsum(rows[:-1])]).astype(np.int64)
    total = int(rows.sum())
    table = torch.from_numpy(r.integers(-30000, 30000, size=(total, d)).astype(np.int16)
                             ).view(torch.bfloat16).to(dev)
    idx = torch.from_numpy(r.integers(-2, 55, size=(T, Q)).astype(np.int32)).to(dev)
    fill = 0x7FC1
    buf, win = padded(T * Q * d, torch.bfloat16, dev, fill)
    eg.tk_engram_gather(idx, table, offsets, rows, out=win.view(T, Q, d))
    torch.cuda.synchronize()
    assert margins_intact(buf, fill)
    want = oracle.engram_gather(idx.cpu().numpy(), table.view(torch.int16).cpu().numpy()
                                .view(np.uint16), offsets, rows)
    got = win.view(torch.int16).cpu().numpy().view(np.uint16).reshape(want.shape)
    assert np.array_equal(got, want)
