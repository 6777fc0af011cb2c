"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances, and where they come from:
  gate            max |gpu - oracle| <= 1e-5
  out             within 1 bf16 ulp of bf16(oracle), or, where x and gate*v
                  cancel, |gpu - oracle| <= 1e-5 |v| + 2^-24 (|x| + |gate v|):
                  a gate within 1e-5 and one fp32 rounding of x + gate*v
                  allow exactly that much where the result is tiny
  dx, dk, dv      relative L2 error <= 1e-3 against bf16(oracle): the
                  outputs are bf16, whose rounding alone is ~1.7e-3 relative
                  L2 against unrounded fp64, so they are compared with the
                  oracle's value rounded once to bf16
  dwh, dwe        relative L2 error <= 1e-3 against the oracle (fp32 outputs)
  reruns          bit-identical
Full-size workloads are compared on every element, streaming the oracle over
chunks of rows.
"""

import math
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

GATE_TOL = 1e-5
REL_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def eg(cuda_device):
    import engram_conditional_memory_amd as m
    m.load_library()
    return m


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def to_host_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def same_bits(a, b):
    import torch
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


def run_gpu(eg, d, dev, backward=True, rerun=False, fused=False, eps=oracle.EPS):
    """Forward (+ backward + reduction) on the GPU; returns host arrays. With
    `rerun`, every call runs a second time into fresh outputs, and each
    output must equal the first run's bit for bit. With `fused`, the forward
    and the backward take the fused weight w = wh * we from
    tk_engram_fused_weight instead of wh and we."""
    import torch
    T, H = d["x"].shape
    x, k, v = to_dev(d["x"], dev), to_dev(d["k"], dev), to_dev(d["v"], dev)
    wh = torch.from_numpy(d["wh"]).to(dev)
    we = torch.from_numpy(d["we"]).to(dev)
    if fused:
        w = eg.tk_engram_fused_weight(wh, we)
        fwd = lambda: eg.tk_engram_gate_fwd_fused(x, k, v, w, eps=eps)  # noqa: E731
        bwd = lambda g: eg.tk_engram_gate_bwd_fused(g, x, k, v, w, eps=eps)  # noqa: E731
    else:
        fwd = lambda: eg.tk_engram_gate_fwd(x, k, v, wh, we, eps=eps)  # noqa: E731
        bwd = lambda g: eg.tk_engram_gate_bwd(g, x, k, v, wh, we, eps=eps)  # noqa: E731
    out, gate = fwd()
    if rerun:
        out2, gate2 = fwd()
        torch.cuda.synchronize()
        assert same_bits(out, out2) and same_bits(gate, gate2), "forward rerun differs"
        del out2, gate2
    res = {}
    if backward:
        g = to_dev(d["grad_out"], dev)
        dx, dk, dv, ws, P = bwd(g)
        dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P, H, wh, we)
        if rerun:
            again = bwd(g)
            again_w = eg.tk_engram_grad_w_reduce(again[3], P, H, wh, we)
            torch.cuda.synchronize()
            for name, a, b in (("dx", dx, again[0]), ("dk", dk, again[1]), ("dv", dv, again[2]),
                               ("partials", ws, again[3]), ("dwh", dwh, again_w[0]),
                               ("dwe", dwe, again_w[1])):
                assert same_bits(a, b), f"backward rerun differs in {name}"
            say(f"  rerun bit-identical (T={T} H={H}): out, gate, dx, dk, dv, partials, "
                "dwh, dwe")
            del again, again_w
        torch.cuda.synchronize()
        del g
        res.update(dx=to_host_bits(dx), dk=to_host_bits(dk), dv=to_host_bits(dv),
                   dwh=dwh.cpu().numpy(), dwe=dwe.cpu().numpy(), P=P)
        del dx, dk, dv, ws
    torch.cuda.synchronize()
    res.update(out=to_host_bits(out), gate=gate.cpu().numpy())
    del x, k, v, out, gate
    torch.cuda.empty_cache()
    return res


def row_classes(d):
    """0 = regular row, 1 = some input row of the token is all zero,
    2 = some input row is scaled by 1e3 (stress workload only)."""
    T = d["x"].shape[0]
    cls = np.zeros(T, dtype=np.uint8)
    if d["config"].kind != "stress":
        return cls
    for name in ("x", "k", "v"):
        s = synth.stress_row_scales(0, d["T"], name)[d["r0"]:d["r0"] + T]
        cls[s == 1e3] = np.maximum(cls[s == 1e3], 2)
        cls[s == 0.0] = 1
    return cls


def compare(d, g, backward=True, chunk=2048, eps=oracle.EPS):
    """Stream the oracle over the rows and collect every statistic."""
    T, H = d["x"].shape
    cls = row_classes(d)
    out_res = np.zeros(4)
    gate_err = 0.0
    st = {n: oracle.BF16Stats() for n in ("dx", "dk", "dv")}
    dwh = np.zeros(H)
    dwe = np.zeros(H)
    min_abs_z = np.inf
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        sl = slice(a, b)
        o_out, o_gate, o_z = oracle.fwd_bf16(d["x"][sl], d["k"][sl], d["v"][sl],
                                             d["wh"], d["we"], eps=eps)
        gate_err = max(gate_err, float(np.max(np.abs(g["gate"][sl] - o_gate))))
        nz = np.abs(o_z[o_z != 0])
        if nz.size:
            min_abs_z = min(min_abs_z, float(nz.min()))
        oracle.check_out(g["out"][sl], o_out, d["x"][sl], d["v"][sl], o_gate, out_res)
        del o_out
        if backward:
            o_dx, o_dk, o_dv, p_wh, p_we, _ = oracle.bwd_bf16(
                d["grad_out"][sl], d["x"][sl], d["k"][sl], d["v"][sl], d["wh"], d["we"],
                eps=eps)
            st["dx"].add(g["dx"][sl], o_dx, cls[sl])
            st["dk"].add(g["dk"][sl], o_dk, cls[sl])
            st["dv"].add(g["dv"][sl], o_dv, cls[sl])
            dwh += p_wh
            dwe += p_we
            del o_dx, o_dk, o_dv
    rep = {"gate_err": gate_err, "out": out_res, "min_abs_z": min_abs_z}
    if backward:
        rep.update(st=st, dwh_rel=float(np.linalg.norm(g["dwh"] - dwh) / np.linalg.norm(dwh)),
                   dwe_rel=float(np.linalg.norm(g["dwe"] - dwe) / np.linalg.norm(dwe)))
    return rep


def assert_dv_is_gate_times_grad(d, g, chunk=4096):
    """The backward recomputes the forward's gate bit for bit, so dv must be
    the fp32 product gate * grad_out (gate from the forward) rounded once to
    bf16, element for element."""
    T = d["x"].shape[0]
    for a in range(0, T, chunk):
        sl = slice(a, min(T, a + chunk))
        gout = oracle.bf16_to_f64(d["grad_out"][sl]).astype(np.float32)
        prod = g["gate"][sl].astype(np.float32)[:, None] * gout      # fp32 multiply
        want = oracle.round_bf16(prod.astype(np.float64))
        assert np.array_equal(g["dv"][sl], want), f"dv rows {sl}"


def assert_report(rep, backward=True, name=""):
    out = rep["out"]
    say(f"[{name}] gate max err {rep['gate_err']:.3e} (min |z| {rep['min_abs_z']:.2e}); "
        f"out max ulp {out[0]:.0f}, >1ulp {out[1]:.0f}, by cancellation bound "
        f"{out[2]:.0f}, failing {out[3]:.0f}")
    assert rep["gate_err"] <= GATE_TOL
    assert out[3] == 0
    if backward:
        for n, s in rep["st"].items():
            say(f"[{name}] {n}: rel L2 {s.rel_l2():.3e} (regular rows {s.rel_l2([0]):.3e}), "
                f"max row rel {s.max_row_rel():.3e}, max ulp {s.max_ulp():.0f}, "
                f"non-finite {s.nonfinite()}")
            assert s.nonfinite() == 0
            assert s.rel_l2() <= REL_TOL, n
            assert s.rel_l2([0]) <= REL_TOL, n
        say(f"[{name}] dwh rel L2 {rep['dwh_rel']:.3e}, dwe rel L2 {rep['dwe_rel']:.3e}")
        assert rep["dwh_rel"] <= REL_TOL and rep["dwe_rel"] <= REL_TOL


# ---------------------------------------------------------------- workloads

def test_config1_tiny(eg, cuda_device):
    d = synth.make_inputs(1)
    g = run_gpu(eg, d, cuda_device)
    rep = compare(d, g)
    assert_report(rep, name="tiny T=64 H=256")
    assert_dv_is_gate_times_grad(d, g)
    # the tiny workload is small enough for a strict elementwise check too
    assert rep["st"]["dv"].max_ulp() <= 1


def test_config2_forward(eg, cuda_device):
    d = synth.make_inputs(2, with_grad=False)
    g = run_gpu(eg, d, cuda_device, backward=False)
    assert_report(compare(d, g, backward=False), backward=False, name="fwd T=1024 H=4096")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_full_size(eg, cuda_device, cfg):
    c = synth.CONFIGS[cfg]
    say(f"[config {cfg}] {c.name}: generating T={c.T} H={c.H}")
    d = synth.make_inputs(cfg)
    g = run_gpu(eg, d, cuda_device, rerun=True)
    say(f"[config {cfg}] GPU done (P={g['P']}), comparing with the oracle")
    assert_report(compare(d, g), name=c.name)
    assert_dv_is_gate_times_grad(d, g)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 4])
def test_fused_weight_calls_match_the_oracle_and_the_unfused_calls(eg, cuda_device, cfg):
    # engram_fused_weight of the "5. Engram" section feeding the gate: the
    # forward and the backward that read w = wh * we give the unfused calls'
    # results bit for bit, and so meet the oracle's tolerances
    c = synth.CONFIGS[cfg]
    say(f"[config {cfg}] {c.name}: fused-weight calls, T={c.T} H={c.H}")
    d = synth.make_inputs(cfg)
    gf = run_gpu(eg, d, cuda_device, fused=True)
    gu = run_gpu(eg, d, cuda_device)
    for name in ("out", "gate", "dx", "dk", "dv", "dwh", "dwe"):
        assert np.array_equal(gf[name].view(np.uint8), gu[name].view(np.uint8)), name
    assert_report(compare(d, gf), name=c.name + " (fused weight)")


@pytest.mark.timeout(900)
def test_tensors_beyond_2_31_elements(eg, cuda_device):
    """T * H = 2,150,400,000 > 2^31 (4.3 GB per bf16 tensor): every offset
    past 2^31 elements must still land on its own row. Each input tensor
    repeats a seeded tile of rows with its own prime period, so no two of the
    300,000 tokens share all four input rows, and every element of every
    output is compared with the oracle, streamed over chunks of rows."""
    import torch
    dev = cuda_device
    H, T = 7168, 300_000
    assert T * H > 2 ** 31
    periods = {"x": 4099, "k": 4111, "v": 4127, "grad_out": 4129}
    r = np.random.default_rng(23)
    tiles = {n: synth.round_bf16(r.standard_normal((p, H))) for n, p in periods.items()}
    wh = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    we = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    say(f"[T={T} H={H}] building {T * H * 2 / 1e9:.1f} GB device tensors")
    ar = torch.arange(T, device=dev)
    t = {}
    for n, p in periods.items():
        tile = to_dev(tiles[n], dev)
        t[n] = tile[ar % p]
        del tile
    del ar
    whd, wed = torch.from_numpy(wh).to(dev), torch.from_numpy(we).to(dev)
    out, gate = eg.tk_engram_gate_fwd(t["x"], t["k"], t["v"], whd, wed)
    dx, dk, dv, ws, P = eg.tk_engram_gate_bwd(t["grad_out"], t["x"], t["k"], t["v"], whd, wed)
    dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P, H, whd, wed)
    torch.cuda.synchronize()
    del t, ws
    say(f"[T={T} H={H}] GPU done (P={P}), comparing every element with the oracle")
    gate_h = gate.cpu().numpy()
    st = {n: oracle.BF16Stats() for n in ("dx", "dk", "dv")}
    out_res = np.zeros(4)
    gate_err, min_abs_z = 0.0, np.inf
    o_dwh, o_dwe = np.zeros(H), np.zeros(H)
    chunk = 4096
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        rows = np.arange(a, b)
        h = {n: tiles[n][rows % p] for n, p in periods.items()}
        o_out, o_gate, o_z = oracle.fwd_bf16(h["x"], h["k"], h["v"], wh, we)
        gate_err = max(gate_err, float(np.max(np.abs(gate_h[a:b] - o_gate))))
        nz = np.abs(o_z[o_z != 0])
        if nz.size:
            min_abs_z = min(min_abs_z, float(nz.min()))
        oracle.check_out(to_host_bits(out[a:b]), o_out, h["x"], h["v"], o_gate, out_res)
        del o_out
        o_dx, o_dk, o_dv, p_wh, p_we, _ = oracle.bwd_bf16(h["grad_out"], h["x"], h["k"],
                                                          h["v"], wh, we)
        st["dx"].add(to_host_bits(dx[a:b]), o_dx)
        st["dk"].add(to_host_bits(dk[a:b]), o_dk)
        st["dv"].add(to_host_bits(dv[a:b]), o_dv)
        o_dwh += p_wh
        o_dwe += p_we
        del o_dx, o_dk, o_dv
        if (a // chunk) % 16 == 15:
            say(f"[T={T} H={H}] compared rows < {b}")
    g_dwh, g_dwe = dwh.cpu().numpy(), dwe.cpu().numpy()
    rep = {"gate_err": gate_err, "out": out_res, "min_abs_z": min_abs_z, "st": st,
           "dwh_rel": float(np.linalg.norm(g_dwh - o_dwh) / np.linalg.norm(o_dwh)),
           "dwe_rel": float(np.linalg.norm(g_dwe - o_dwe) / np.linalg.norm(o_dwe))}
    del out, gate, dx, dk, dv, dwh, dwe
    torch.cuda.empty_cache()
    assert_report(rep, name=f"T={T} H={H}, beyond 2^31 elements")


# ------------------------------------------------------------- determinism

def test_reruns_are_bit_identical(eg, cuda_device):
    d = synth.make_inputs(3, rows=(0, 4099))     # ragged: not a block multiple
    a = run_gpu(eg, d, cuda_device)
    b = run_gpu(eg, d, cuda_device)
    for n in ("out", "gate", "dx", "dk", "dv", "dwh", "dwe"):
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), n


# -------------------------------------------------------------- edge cases

def make_case(T, H, seed=0, fill=None):
    r = np.random.default_rng(seed)
    d = {"T": T, "H": H, "r0": 0, "config": synth.CONFIGS[1]}
    for n in ("x", "k", "v", "grad_out"):
        d[n] = synth.round_bf16(r.standard_normal((T, H)))
    d["wh"] = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    d["we"] = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    if fill:
        fill(d)
    return d


@pytest.mark.parametrize("T,H", [(1, 8), (3, 64), (5, 72), (7, 520), (9, 1032),
                                 (33, 2048), (17, 4096), (11, 7168), (6, 8192),
                                 (1000, 4096), (513, 7168), (4099, 256)])
def test_shapes(eg, cuda_device, T, H):
    d = make_case(T, H, seed=T * 7 + H)
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name=f"T={T} H={H}")
    assert_dv_is_gate_times_grad(d, g)


def _random_shapes(n=30, seed=8192):
    r = np.random.default_rng(seed)
    return [(int(r.integers(1, 3001)), 8 * int(r.integers(1, 1025))) for _ in range(n)]


@pytest.mark.parametrize("T,H", _random_shapes())
def test_random_shapes(eg, cuda_device, T, H):
    # seeded random widths (any multiple of 8 up to 8192, so mostly the
    # generic plans with masked tail chunks) and token counts, every element
    # against the oracle, the forward's gate reused bit for bit by dv
    d = make_case(T, H, seed=T * 13 + H)
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name=f"T={T} H={H}")
    assert_dv_is_gate_times_grad(d, g)


def test_special_rows(eg, cuda_device):
    T, H = 12, 4096

    def fill(d):
        z = np.zeros(H, dtype=np.uint16)
        d["x"][0] = z                            # zero hidden row
        d["k"][1] = z                            # zero key row
        d["x"][2] = d["k"][2] = d["v"][2] = z    # everything zero
        d["v"][3] = z                            # no gradient reaches the gate
        d["x"][4] = d["k"][4]                    # k = x
        d["x"][5] = d["x"][4]                    # same x, k = -x: mirrored gate
        d["k"][5] = d["x"][4] ^ 0x8000
        d["x"][6, 1::2] = 0                      # orthogonal supports: gate 1/2
        d["k"][6, 0::2] = 0
        big = synth.round_bf16(synth.bf16_to_f64(d["x"][7]) * 1e3)
        d["x"][7] = big                          # scaled row
    d = make_case(T, H, seed=5, fill=fill)
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name="special rows")
    gate = g["gate"]
    assert gate[0] == 0.5 and gate[1] == 0.5 and gate[2] == 0.5 and gate[6] == 0.5
    # orthogonal supports: out = bf16(x + v / 2), bit for bit
    want = oracle.round_bf16(oracle.bf16_to_f64(d["x"][6]) + 0.5 * oracle.bf16_to_f64(d["v"][6]))
    assert np.array_equal(g["out"][6], want)
    # zero row everywhere: dx = grad_out exactly, dk = 0, dv = grad_out / 2
    assert np.array_equal(g["dx"][2], d["grad_out"][2])
    assert np.all(oracle.bf16_to_f64(g["dk"][2]) == 0)
    # v = 0: no gradient through the gate
    assert np.array_equal(g["dx"][3], d["grad_out"][3])
    assert np.all(oracle.bf16_to_f64(g["dk"][3]) == 0)
    # mirrored gate: sigmoid(-s) = 1 - sigmoid(s)
    assert abs(gate[4] + gate[5] - 1.0) < 2e-6


@pytest.mark.parametrize("H", [4096, 7168])
def test_smallest_eps(eg, cuda_device, H):
    # eps = 2^-126, the smallest the calls accept: rows of zeros and rows far
    # below eps get a normalising scale near 2^63, which the backward's fp32
    # elementwise work must hold without overflow (a zero row stays zero)
    T = 16

    def fill(d):
        z = np.zeros(H, dtype=np.uint16)
        d["x"][0] = z
        d["k"][1] = z
        d["x"][2] = d["k"][2] = z
        for t in (3, 4, 5):
            d["x"][t] = synth.round_bf16(synth.bf16_to_f64(d["x"][t]) * 2.0 ** -120)
        for t in (4, 6):
            d["k"][t] = synth.round_bf16(synth.bf16_to_f64(d["k"][t]) * 2.0 ** -120)
    d = make_case(T, H, seed=H + 126, fill=fill)
    eps = 2.0 ** -126
    g = run_gpu(eg, d, cuda_device, eps=eps)
    assert_report(compare(d, g, eps=eps), name=f"eps 2^-126 H={H}")
    for n in ("dx", "dk", "dv"):
        assert np.all(np.isfinite(oracle.bf16_to_f64(g[n]))), n
    assert np.all(np.isfinite(g["dwh"])) and np.all(np.isfinite(g["dwe"]))
    # the row with x and k both zero: dx = grad_out and dk = 0 exactly
    assert np.array_equal(g["dx"][2], d["grad_out"][2])
    assert np.all(oracle.bf16_to_f64(g["dk"][2]) == 0)


def test_derivative_clamp_region(eg, cuda_device):
    """Rows whose z sits on both sides of the derivative clamp. x lives on
    the even columns and k on the odd ones, except k[0] = c: the weighted
    dot is then the single exact product x[0] c wh[0] we[0], so z is known
    to fp32 rounding of the two norms and each row lands where it is meant
    to, below, near or above the clamp."""
    H = 4096
    cs = [s * 2.0 ** -e for e in range(4, 15) for s in (1, -1)]
    T = len(cs)

    def fill(d):
        d["x"][:, 1::2] = 0
        d["k"][:, 0::2] = 0
        d["k"][:, 0] = synth.round_bf16(np.array(cs))
    d = make_case(T, H, seed=11, fill=fill)
    _, _, z = oracle.fwd_bf16(d["x"], d["k"], d["v"], d["wh"], d["we"], want_out=False)
    az = np.abs(z)
    assert np.sum(az < 0.5 * oracle.CLAMP) >= 4 and np.sum(az > 2 * oracle.CLAMP) >= 4
    assert np.sum((az > 0.5 * oracle.CLAMP) & (az < 2 * oracle.CLAMP)) >= 2
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name="clamp region")
    assert_dv_is_gate_times_grad(d, g)
    # row by row as well: a wrong branch on one row would hide in the totals
    o_dx, o_dk, _, _, _, _ = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"],
                                             d["wh"], d["we"])
    for name, o in (("dx", o_dx), ("dk", o_dk)):
        ref = oracle.bf16_to_f64(oracle.round_bf16(o))
        got = oracle.bf16_to_f64(g[name])
        rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
        say(f"[clamp region] {name} worst row rel L2 {rel.max():.3e}")
        assert np.all(rel <= REL_TOL), (name, np.flatnonzero(rel > REL_TOL), z)


@pytest.mark.parametrize("T,H", [(1000, 4096), (500, 7168), (37, 256), (40000, 4096),
                                 (20000, 7168)])
def test_workspace_holds_the_documented_partials(eg, cuda_device, T, H):
    """The header's contract for the backward's workspace: partial row p is
    c_p[i] = sum over t = p, p + P, ... of dd_t r_x,t r_k,t x_t,i k_t,i,
    rebuilt here in fp64 from the oracle's per-token scalars. The last two
    shapes walk their rows in two launches each, the second one short
    (157 = 120 + 37 rows per block at H = 4096, 90 = 78 + 12 at H = 7168), so
    the partial sums carry over a launch boundary."""
    import torch
    d = make_case(T, H, seed=T + H)
    dev = cuda_device
    x, k, v = to_dev(d["x"], dev), to_dev(d["k"], dev), to_dev(d["v"], dev)
    g = to_dev(d["grad_out"], dev)
    wh, we = torch.from_numpy(d["wh"]).to(dev), torch.from_numpy(d["we"]).to(dev)
    _, _, _, ws, P = eg.tk_engram_gate_bwd(g, x, k, v, wh, we)
    torch.cuda.synchronize()
    assert P == eg.tk_engram_num_partials(T, H) and 1 <= P <= T
    got = ws.cpu().numpy()[:P]
    xf, kf = oracle.bf16_to_f64(d["x"]), oracle.bf16_to_f64(d["k"])
    _, _, fst = oracle.fwd_f64(xf, kf, oracle.bf16_to_f64(d["v"]), d["wh"], d["we"])
    _, _, _, _, _, dd = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"], d["wh"],
                                        d["we"], want_grads=False)
    A = dd * fst[:, 2] * fst[:, 3]                    # dd r_x r_k per token
    want = np.zeros((P, H))
    for p in range(P):
        want[p] = (A[p::P, None] * xf[p::P] * kf[p::P]).sum(axis=0)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    say(f"[workspace T={T} H={H} P={P}] rel L2 {rel:.3e}")
    assert rel <= 1e-5


@pytest.mark.parametrize("H", [4096, 7168, 2048, 6144])
def test_row_magnitudes_across_the_bf16_range(eg, cuda_device, H):
    """Rows of x, of k, of both, or of v scaled by 2^e, from far below eps
    (where the gate is 1/2) to 2^125, near the top of the bf16 range. The
    sums are fp64 and every coefficient is formed from normalised rows, so
    nothing overflows on the way; every row of every output is compared with
    the oracle on its own. The widths cover each kind of plan: 2 x 4 and
    1 x 4 with weights in registers, 7 x 2 and 2 x 6 with weights in LDS."""
    exps = (-120, -64, -40, -20, 0, 20, 40, 56, 60, 64, 80, 100, 120, 125)
    cases = [(e, w) for e in exps for w in ("x", "k", "both", "v")]

    def fill(d):
        for t, (e, w) in enumerate(cases):
            for n in ("x", "k", "v"):
                if w == n or (w == "both" and n != "v"):
                    d[n][t] = synth.round_bf16(synth.bf16_to_f64(d[n][t]) * 2.0 ** e)
    d = make_case(len(cases), H, seed=29 + H, fill=fill)
    for n in ("x", "k", "v"):
        assert np.all(np.isfinite(synth.bf16_to_f64(d[n])))
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name=f"row magnitudes 2^-120 .. 2^125, H={H}")
    assert_dv_is_gate_times_grad(d, g)
    o_dx, o_dk, o_dv, _, _, _ = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"],
                                                d["wh"], d["we"])
    worst = 0.0
    for name, o in (("dx", o_dx), ("dk", o_dk), ("dv", o_dv)):
        ref = oracle.bf16_to_f64(oracle.round_bf16(o))
        got = oracle.bf16_to_f64(g[name])
        assert np.all(np.isfinite(got)), name
        rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
        worst = max(worst, float(rel.max()))
        assert np.all(rel <= REL_TOL), (name, [cases[i] for i in np.flatnonzero(rel > REL_TOL)])
    say(f"[row magnitudes H={H}] worst row rel L2 {worst:.3e}")


@pytest.mark.parametrize("H", [4096, 7168, 2048, 6144, 520])
def test_saturated_gates(eg, cuda_device, H):
    """Gates from 1/2 to within e^-45 of 0 and of 1. The weights are scaled so
    that a row with k = x reaches s = 45; k = rho x + sqrt(1 - rho^2) n puts
    the other rows at s of about 45 sqrt|rho|, of either sign. Where the gate
    saturates, its derivative g (1 - g) is e^-|s| and the whole dk row (and
    the gate's share of dx) scales with it, so every row is compared with
    the oracle on its own: g (1 - g) formed from a gate rounded to fp32
    would be off by up to 100% there."""
    targets = np.array([0.5, 2, 5, 8, 10, 12, 15, 17, 20, 25, 30, 35, 40, 45.0])
    rho = np.concatenate([targets, -targets]) ** 2 / 45.0 ** 2 * np.repeat([1, -1], 14)
    T = rho.size
    c = math.sqrt(45.0 ** 2 / math.sqrt(H))

    def fill(d):
        r = np.random.default_rng(H)
        x = synth.bf16_to_f64(d["x"])
        n = r.standard_normal((T, H))
        d["k"] = synth.round_bf16(rho[:, None] * x + np.sqrt(1 - rho[:, None] ** 2) * n)
        d["wh"] = (c * (1 + 0.05 * r.standard_normal(H))).astype(np.float32)
        d["we"] = (c * (1 + 0.05 * r.standard_normal(H))).astype(np.float32)
    d = make_case(T, H, seed=97 + H, fill=fill)
    _, o_gate, o_z = oracle.fwd_bf16(d["x"], d["k"], d["v"], d["wh"], d["we"], want_out=False)
    s = np.sign(o_z) * np.sqrt(np.abs(o_z))
    assert s.max() > 40 and s.min() < -40 and np.sum(np.abs(s) > 17) >= 8
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name=f"saturated gates H={H}")
    assert_dv_is_gate_times_grad(d, g)
    o_dx, o_dk, o_dv, _, _, _ = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"],
                                                d["wh"], d["we"])
    worst = 0.0
    for name, o in (("dx", o_dx), ("dk", o_dk), ("dv", o_dv)):
        ref = oracle.bf16_to_f64(oracle.round_bf16(o))
        got = oracle.bf16_to_f64(g[name])
        assert np.all(np.isfinite(got)), name
        rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
        worst = max(worst, float(rel.max()))
        assert np.all(rel <= REL_TOL), (name, s[rel > REL_TOL])
    say(f"[saturated gates H={H}] |s| up to {np.abs(s).max():.1f}, "
        f"worst row rel L2 {worst:.3e}")


def test_empty_and_zero_partials(eg, cuda_device):
    import torch
    dev = cuda_device
    H = 256
    x = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    wh = torch.ones(H, device=dev)
    out, gate = eg.tk_engram_gate_fwd(x, x, x, wh, wh)
    assert out.shape == (0, H) and gate.shape == (0,)
    dx, dk, dv, ws, P = eg.tk_engram_gate_bwd(x, x, x, x, wh, wh)
    assert P == 0
    dwh = torch.full((H,), 7.0, device=dev)
    dwe = torch.full((H,), 7.0, device=dev)
    eg.tk_engram_grad_w_reduce(ws, 0, H, wh, wh, dwh, dwe)
    torch.cuda.synchronize()
    assert torch.all(dwh == 0) and torch.all(dwe == 0)


def test_side_stream_and_identity(eg, cuda_device):
    import torch
    d = make_case(300, 4096, seed=11)
    s = torch.cuda.Stream(cuda_device)
    with torch.cuda.stream(s):
        g = run_gpu(eg, d, cuda_device)
    torch.cuda.synchronize()
    rep = compare(d, g)
    assert_report(rep, name="side stream")
    # wh * dwh == we * dwe up to fp32 rounding of the two products
    lhs = d["wh"].astype(np.float64) * g["dwh"]
    rhs = d["we"].astype(np.float64) * g["dwe"]
    assert np.max(np.abs(lhs - rhs)) <= 1e-6 * np.max(np.abs(lhs))


def test_stream_probe(eg, cuda_device):
    import torch
    n = (1 << 20) + 12                  # not a whole tile: exercises the tail
    srcs = [torch.randint(-(1 << 31), (1 << 31) - 1, (n,), dtype=torch.int32,
                          device=cuda_device) for _ in range(3)]
    dsts = [torch.zeros_like(srcs[0]) for _ in range(2)]
    eg.tk_engram_stream_probe(srcs, dsts)
    torch.cuda.synchronize()
    x = srcs[0] ^ srcs[1] ^ srcs[2]
    assert torch.equal(dsts[0], x)
    assert torch.equal(dsts[1], srcs[0] ^ (srcs[1] + 1) ^ (srcs[2] + 1))


def test_copy_probe(eg, cuda_device):
    import torch
    src = torch.arange(1 << 20, dtype=torch.int32, device=cuda_device)
    dst = torch.zeros_like(src)
    eg.tk_engram_copy_probe(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# --------------------------------------------------------------- fused weight

@pytest.mark.parametrize("H", [1, 7, 256, 7168, 100003])
def test_fused_weight_is_the_exact_product(eg, cuda_device, H):
    import torch
    r = np.random.default_rng(H)
    wh = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    we = (r.standard_normal(H) * 10.0 ** r.integers(-30, 30, H)).astype(np.float32)
    whd, wed = torch.from_numpy(wh).to(cuda_device), torch.from_numpy(we).to(cuda_device)
    w = eg.tk_engram_fused_weight(whd, wed)
    w2 = torch.full((H,), float("nan"), dtype=torch.float64, device=cuda_device)
    eg.bind_fused_weight(whd, wed, w2)()                  # the pre-marshalled form
    torch.cuda.synchronize()
    want = oracle.fused_weight(wh, we)
    assert np.array_equal(w.cpu().numpy(), want)
    assert np.array_equal(w2.cpu().numpy(), want)


# ----------------------------------------------------------------- HIP graphs

@pytest.mark.parametrize("T,H,form", [(1000, 7168, "plain"), (20003, 7168, "plain"),
                                      (20003, 7168, "fused+noalloc"), (1000, 4096,
                                                                        "fused+noalloc")])
def test_graph_capture_and_replay(eg, cuda_device, T, H, form):
    """The gate calls allocate nothing and write no memset, so a step
    captured into a HIP graph replays bit for bit like the eager calls: the
    three plain calls, or the fused-weight forward and the backward +
    reduction with library-owned partials (for callers that cannot allocate,
    such as code under graph capture). At 20003 x 7168 each gate call is two
    launches (epochs)."""
    import torch
    d = make_case(T, H, seed=21)
    dev = cuda_device
    x, k, v, gout = (to_dev(d[n], dev) for n in ("x", "k", "v", "grad_out"))
    wh = torch.from_numpy(d["wh"]).to(dev)
    we = torch.from_numpy(d["we"]).to(dev)
    bf = torch.bfloat16
    out, dx, dk, dv = (torch.empty((T, H), dtype=bf, device=dev) for _ in range(4))
    gate = torch.empty((T,), dtype=torch.float32, device=dev)
    P = eg.tk_engram_num_partials(T, H)
    ws = torch.empty((P, H), dtype=torch.float32, device=dev)
    dwh = torch.empty((H,), dtype=torch.float32, device=dev)
    dwe = torch.empty((H,), dtype=torch.float32, device=dev)

    w = eg.tk_engram_fused_weight(wh, we)

    def step():
        if form == "plain":
            eg.tk_engram_gate_fwd(x, k, v, wh, we, out, gate)
            eg.tk_engram_gate_bwd(gout, x, k, v, wh, we, dx, dk, dv, ws)
            eg.tk_engram_grad_w_reduce(ws, P, H, wh, we, dwh, dwe)
        else:
            eg.tk_engram_gate_fwd_fused(x, k, v, w, out, gate)
            eg.tk_engram_gate_bwd_reduce_noalloc(gout, x, k, v, wh, we, dx, dk, dv, dwh, dwe)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, gate, dx, dk, dv, dwh, dwe)]
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in (out, gate, dx, dk, dv, dwh, dwe):
            t.fill_(float("nan"))                # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, gate, dx, dk, dv, dwh, dwe), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), i


# ------------------------------------------------ other widths at volume

@pytest.mark.parametrize("T,H", [(20001, 3072), (8192, 8192), (24001, 2048), (9001, 5120),
                                 (6001, 6144)])
def test_other_widths_many_rows_per_block(eg, cuda_device, T, H):
    # the plans of the other widths (H=2048: 1 wave x 4 chunks on 512
    # workgroups; H=3072: 3 waves x 2 chunks; H=5120 and 6144: 5 and 6 waves
    # x 2 chunks, the backward with three rows in flight and its weights in
    # LDS; H=8192: 8 waves x 2 chunks with the tail mask) with ~25-80 rows
    # per workgroup, compared on every element
    d = make_case(T, H, seed=T + H)
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name=f"T={T} H={H}")
    assert_dv_is_gate_times_grad(d, g)


@pytest.mark.parametrize("T,H", [(61441, 2048), (49153, 3072), (24577, 5120), (20481, 6144),
                                 (16385, 8192)])
def test_other_widths_across_epochs(eg, cuda_device, T, H):
    # the same plans past what one launch covers (by a single row at 2048,
    # 5120 and 6144): each call runs as two launches, the second carrying
    # each workgroup's weight-gradient sum on from the first, compared on
    # every element
    assert eg.tk_engram_gate_launches(T, H, 0) == 2
    assert eg.tk_engram_gate_launches(T, H, 1) == 2
    d = make_case(T, H, seed=T + H)
    g = run_gpu(eg, d, cuda_device)
    assert_report(compare(d, g), name=f"T={T} H={H}")
    assert_dv_is_gate_times_grad(d, g)


@pytest.mark.parametrize("H", [8, 256, 520, 1032, 2048, 2056, 3072, 4096, 4104, 5120, 6144, 7168,
                               8192])
def test_fused_and_noalloc_forms_at_every_plan(eg, cuda_device, H):
    """Every width's launch plan has its own kernels, in a plain and a
    fused-weight form: the fused-weight forward and backward, and the
    allocation-free backward + reduction, must give the plain calls' outputs
    bit for bit at each of them (planned widths, generic plans, masked tail
    chunks)."""
    import torch
    dev = cuda_device
    T = 600
    d = make_case(T, H, seed=H + 5)
    x, k, v, g = (to_dev(d[n], dev) for n in ("x", "k", "v", "grad_out"))
    wh, we = torch.from_numpy(d["wh"]).to(dev), torch.from_numpy(d["we"]).to(dev)
    out, gate = eg.tk_engram_gate_fwd(x, k, v, wh, we)
    dx, dk, dv, ws, P = eg.tk_engram_gate_bwd(g, x, k, v, wh, we)
    dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P, H, wh, we)
    w = eg.tk_engram_fused_weight(wh, we)
    f_out, f_gate = eg.tk_engram_gate_fwd_fused(x, k, v, w)
    f_dx, f_dk, f_dv, f_ws, _ = eg.tk_engram_gate_bwd_fused(g, x, k, v, w)
    n_dx, n_dk, n_dv, n_dwh, n_dwe = eg.tk_engram_gate_bwd_reduce_noalloc(g, x, k, v, wh, we)
    torch.cuda.synchronize()
    for name, a, b in (("out", out, f_out), ("gate", gate, f_gate), ("dx", dx, f_dx),
                       ("dk", dk, f_dk), ("dv", dv, f_dv), ("partials", ws, f_ws),
                       ("noalloc dx", dx, n_dx), ("noalloc dk", dk, n_dk),
                       ("noalloc dv", dv, n_dv), ("noalloc dwh", dwh, n_dwh),
                       ("noalloc dwe", dwe, n_dwe)):
        assert same_bits(a, b), f"{name} differs at H={H}"


def test_nan_row_stays_in_its_row(eg, cuda_device):
    # rows are independent in the forward: a NaN in one token's hidden row
    # gives that token a NaN gate and output and leaves every other row as
    # the oracle computes it
    T, H = 300, 4096
    d = make_case(T, H, seed=99)
    d["x"][17, 5] = 0x7FC0                       # bf16 quiet NaN
    g = run_gpu(eg, d, cuda_device, backward=False)
    assert np.isnan(g["gate"][17])
    keep = np.ones(T, dtype=bool)
    keep[17] = False
    sub = {n: d[n][keep] for n in ("x", "k", "v")}
    _, o_gate, _ = oracle.fwd_bf16(sub["x"], sub["k"], sub["v"], d["wh"], d["we"])
    assert np.max(np.abs(g["gate"][keep] - o_gate)) <= GATE_TOL
