"""The autograd wrapper (engram_conditional_memory_amd.autograd) on the GPU:
it must return exactly what the three C-ABI calls return, match the fp64
oracle within the parity tolerances, accumulate into .grad, and accept
[..., H] shapes."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

REL_TOL = 1e-3


@pytest.fixture(scope="module")
def eg(cuda_device):
    import engram_conditional_memory_amd as m
    m.load_library()
    return m


def case(T, H, seed):
    r = np.random.default_rng(seed)
    d = {n: synth.round_bf16(r.standard_normal((T, H))) for n in ("x", "k", "v", "grad_out")}
    d["k"] = synth.round_bf16(synth.bf16_to_f64(d["k"]) + 0.5 * synth.bf16_to_f64(d["x"]))
    d["wh"] = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    d["we"] = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    return d


def dev_bf16(bits, dev, requires_grad=False):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    return t.requires_grad_(requires_grad)


def bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_module_matches_c_abi_and_oracle(eg, cuda_device):
    import torch
    T, H = 300, 4096
    d = case(T, H, seed=1)
    dev = cuda_device
    x, k, v = (dev_bf16(d[n], dev, True) for n in ("x", "k", "v"))
    gout = dev_bf16(d["grad_out"], dev)
    m = eg.EngramGate(H, device=dev)
    with torch.no_grad():
        m.wh.copy_(torch.from_numpy(d["wh"]))
        m.we.copy_(torch.from_numpy(d["we"]))
    out = m(x, k, v)
    out.backward(gout)
    torch.cuda.synchronize()

    # exactly the C-ABI calls
    xr, kr, vr = (dev_bf16(d[n], dev) for n in ("x", "k", "v"))
    o2, g2 = eg.tk_engram_gate_fwd(xr, kr, vr, m.wh.detach(), m.we.detach())
    dx, dk, dv, ws, P = eg.tk_engram_gate_bwd(gout, xr, kr, vr, m.wh.detach(), m.we.detach())
    dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P, H, m.wh.detach(), m.we.detach())
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(o2))
    assert torch.equal(m.last_gate, g2)
    for a, b in ((x.grad, dx), (k.grad, dk), (v.grad, dv)):
        assert np.array_equal(bits(a), bits(b))
    assert torch.equal(m.wh.grad, dwh) and torch.equal(m.we.grad, dwe)

    # and the oracle
    o_dx, o_dk, o_dv, o_dwh, o_dwe, _ = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"],
                                                        d["wh"], d["we"])
    for got, ref in ((x.grad, o_dx), (k.grad, o_dk), (v.grad, o_dv)):
        st = oracle.BF16Stats()
        st.add(bits(got), ref)
        assert st.rel_l2() <= REL_TOL and st.nonfinite() == 0
    for got, ref in ((m.wh.grad, o_dwh), (m.we.grad, o_dwe)):
        g = got.cpu().numpy().astype(np.float64)
        assert np.linalg.norm(g - ref) / np.linalg.norm(ref) <= REL_TOL


def test_grad_accumulates_and_leading_shape(eg, cuda_device):
    import torch
    B, S, H = 2, 37, 7168
    d = case(B * S, H, seed=2)
    dev = cuda_device
    x, k, v = (dev_bf16(d[n], dev).view(B, S, H).requires_grad_(True) for n in ("x", "k", "v"))
    gout = dev_bf16(d["grad_out"], dev).view(B, S, H)
    wh = torch.from_numpy(d["wh"]).to(dev).requires_grad_(True)
    we = torch.from_numpy(d["we"]).to(dev).requires_grad_(True)
    out, gate = eg.engram_gate(x, k, v, wh, we)
    assert out.shape == (B, S, H) and gate.shape == (B, S) and not gate.requires_grad
    out.backward(gout)
    first = [t.grad.clone() for t in (x, k, v, wh, we)]
    out, _ = eg.engram_gate(x, k, v, wh, we)
    out.backward(gout)
    torch.cuda.synchronize()
    for t, g1 in zip((x, k, v, wh, we), first):
        assert torch.equal(t.grad, 2 * g1)       # doubling is exact in bf16 and fp32


def test_frozen_weights_skip_the_reduction(eg, cuda_device):
    import torch
    T, H = 64, 256
    d = case(T, H, seed=3)
    dev = cuda_device
    x = dev_bf16(d["x"], dev, True)
    k, v = dev_bf16(d["k"], dev), dev_bf16(d["v"], dev)
    wh = torch.from_numpy(d["wh"]).to(dev)
    we = torch.from_numpy(d["we"]).to(dev)
    out, _ = eg.engram_gate(x, k, v, wh, we)
    out.float().sum().backward()
    torch.cuda.synchronize()
    assert x.grad is not None and wh.grad is None and k.grad is None


def test_module_at_the_main_workload_shape(eg, cuda_device):
    """At 32768 tokens x 7168 (each call two launches), the shape the
    autograd line of the benchmark times, the module's outputs and all five
    gradients equal the C-ABI calls' bit for bit. The inputs are drawn on the
    GPU; the C-ABI calls themselves are checked against the oracle at this
    shape by the full-size parity tests."""
    import torch
    T, H = 32768, 7168
    dev = cuda_device
    g = torch.Generator(device=dev).manual_seed(32768)
    x0, k0, v0, gout = (torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)
                        for _ in range(4))
    wh0 = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    we0 = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    m = eg.EngramGate(H, device=dev)
    with torch.no_grad():
        m.wh.copy_(wh0)
        m.we.copy_(we0)
    x, k, v = (t.clone().requires_grad_(True) for t in (x0, k0, v0))
    out = m(x, k, v)
    out.backward(gout)
    o2, g2 = eg.tk_engram_gate_fwd(x0, k0, v0, wh0, we0)
    dx, dk, dv, ws, P = eg.tk_engram_gate_bwd(gout, x0, k0, v0, wh0, we0)
    dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P, H, wh0, we0)
    torch.cuda.synchronize()
    assert eg.tk_engram_gate_launches(T, H, 1) == 2
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(m.last_gate, g2)
    for a, b in ((x.grad, dx), (k.grad, dk), (v.grad, dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(m.wh.grad, dwh) and torch.equal(m.we.grad, dwe)
