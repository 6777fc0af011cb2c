"""Pins of the fp64 oracle against what the formula itself fixes.

The gate is defined on the zhichai.net TileKernels page, section "5. Engram"
(gate formula): per token the two RMSNorm outputs of x (weight wh) and k
(weight we) are dotted, the dot is scaled by 1/sqrt(H), passed through the
signed square root and a sigmoid to give the gate, and out = x + gate * v.
The pages print no worked example, so the oracle is pinned by closed forms,
exact special cases, invariances, a library RMSNorm, and finite differences
and automatic differentiation of its forward for the backward.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

EPS = oracle.EPS


def sigmoid(s):
    return 1.0 / (1.0 + math.exp(-s))


def rng_rows(T, H, seed=0, scale=1.0):
    r = np.random.default_rng(seed)
    return r.standard_normal((T, H)) * scale


def weights(H, seed=1):
    r = np.random.default_rng(seed)
    return 1.0 + 0.1 * r.standard_normal(H), 1.0 + 0.1 * r.standard_normal(H)


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("H", [256, 4096, 7168])
def test_closed_form_k_equals_x(H):
    # With k = x and wh = we = 1: d = H m/(m+eps), m = mean(x^2), so
    # gate = sigmoid(H^(1/4) sqrt(m/(m+eps))).
    x = rng_rows(6, H, seed=H)
    x[1] *= 1e-3          # m comparable to eps
    x[2] *= 1e3
    x[3] = 0.0            # zero row: gate = 1/2
    ones = np.ones(H)
    _, gate, _ = oracle.fwd_f64(x, x, x, ones, ones)
    for t in range(6):
        m = float(np.mean(x[t] ** 2))
        want = 0.5 if m == 0 else sigmoid(H ** 0.25 * math.sqrt(m / (m + EPS)))
        assert abs(gate[t] - want) <= 1e-15


def test_closed_form_unit_mean_square_values():
    # x = +-1 has m = 1 exactly: gate = sigmoid(H^(1/4)/sqrt(1+eps)).
    for H, approx in ((256, 0.982013790), (4096, 0.999664650), (7168, 0.999899103)):
        x = np.where(np.arange(H) % 3 == 0, -1.0, 1.0)[None, :]
        ones = np.ones(H)
        _, gate, _ = oracle.fwd_f64(x, x, x, ones, ones)
        exact = sigmoid(H ** 0.25 / math.sqrt(1 + EPS))
        assert abs(gate[0] - exact) < 1e-15
        # the eps-free values sigmoid(H^(1/4)) differ by sigmoid'(s) s eps / 2
        assert abs(gate[0] - approx) < 1e-7


def test_mirror_k_minus_x():
    H = 512
    x = rng_rows(8, H, seed=3)
    k = rng_rows(8, H, seed=4) + 0.5 * x
    v = rng_rows(8, H, seed=5)
    wh, we = weights(H)
    _, g, _ = oracle.fwd_f64(x, k, v, wh, we)
    _, gm, _ = oracle.fwd_f64(x, -k, v, wh, we)
    assert np.max(np.abs(g + gm - 1.0)) < 1e-15


def test_orthogonal_supports_give_half():
    H = 256
    x = rng_rows(4, H, seed=6)
    k = rng_rows(4, H, seed=7)
    v = rng_rows(4, H, seed=8)
    x[:, 1::2] = 0.0
    k[:, 0::2] = 0.0
    wh, we = weights(H)
    out, g, st = oracle.fwd_f64(x, k, v, wh, we)
    assert np.all(st[:, 4] == 0.0) and np.all(g == 0.5)
    assert np.array_equal(out, x + 0.5 * v)


def test_gate_bounds_cauchy_schwarz():
    H = 1024
    x = rng_rows(64, H, seed=9)
    k = np.repeat(rng_rows(1, H, seed=10), 64, axis=0) * np.linspace(-2, 2, 64)[:, None]
    k += 0.01 * rng_rows(64, H, seed=11)
    wh, we = weights(H, seed=12)
    _, g, st = oracle.fwd_f64(x, k, x, wh, we)
    B = H ** 0.25 * math.sqrt(np.max(np.abs(wh)) * np.max(np.abs(we)))
    assert np.all(np.abs(st[:, 6]) < B)
    assert np.all((g > sigmoid(-B)) & (g < sigmoid(B)))
    assert np.all((g > 0) & (g < 1))


def test_invariances():
    H = 768
    x = rng_rows(5, H, seed=13)
    k = rng_rows(5, H, seed=14) + 0.3 * x
    v = rng_rows(5, H, seed=15)
    wh, we = weights(H, seed=16)
    out, g, st = oracle.fwd_f64(x, k, v, wh, we)
    # joint permutation of the hidden axis
    p = np.random.default_rng(17).permutation(H)
    out_p, g_p, _ = oracle.fwd_f64(x[:, p], k[:, p], v[:, p], wh[p], we[p])
    assert np.max(np.abs(g_p - g)) < 1e-14
    assert np.max(np.abs(out_p - out[:, p])) < 1e-13
    # wh -> 2 wh, we -> we / 2 (exact in binary)
    _, g2, _ = oracle.fwd_f64(x, k, v, 2 * wh, we / 2)
    assert np.max(np.abs(g2 - g)) < 1e-15
    # x -> c x changes only the eps term
    _, g3, _ = oracle.fwd_f64(7.0 * x, k, v, wh, we)
    assert np.max(np.abs(g3 - g)) < 1e-6


def test_forward_against_library_rmsnorm():
    # RMSNorm from torch (y = x / sqrt(mean(x^2) + eps) * weight), in fp64.
    H = 384
    x = rng_rows(16, H, seed=18)
    k = rng_rows(16, H, seed=19) - 0.4 * x
    v = rng_rows(16, H, seed=20)
    wh, we = weights(H, seed=21)
    out, g, st = oracle.fwd_f64(x, k, v, wh, we)
    tx, tk, tv = (torch.from_numpy(a) for a in (x, k, v))
    a = torch.nn.functional.rms_norm(tx, (H,), torch.from_numpy(wh), EPS)
    b = torch.nn.functional.rms_norm(tk, (H,), torch.from_numpy(we), EPS)
    d = (a * b).sum(-1)
    z = d / math.sqrt(H)
    gt = torch.sigmoid(torch.sign(z) * torch.sqrt(torch.abs(z)))
    assert np.max(np.abs(st[:, 4] - d.numpy()) / np.abs(d.numpy())) < 1e-12
    assert np.max(np.abs(g - gt.numpy())) < 1e-15
    assert np.max(np.abs(out - (tx + gt[:, None] * tv).numpy())) < 1e-14


# --------------------------------------------------------------- backward pins

def _config1_f64():
    d = synth.make_inputs(1)
    f = oracle.bf16_to_f64
    return (f(d["grad_out"]), f(d["x"]), f(d["k"]), f(d["v"]),
            d["wh"].astype(np.float64), d["we"].astype(np.float64))


def _row_loss(gout_row, x, k, v, wh, we):
    out, _, _ = oracle.fwd_f64(x, k, v, wh, we)
    return out @ gout_row


def test_backward_finite_differences_config1():
    gout, x, k, v, wh, we = _config1_f64()
    T, H = x.shape
    _, _, st = oracle.fwd_f64(x, k, v, wh, we)
    keep = np.abs(st[:, 5]) >= 1e-2      # FD is not valid across the clamp / kink
    assert keep.sum() >= T - 2
    gout = gout * keep[:, None]
    dx, dk, dv, dwh, dwe, _ = oracle.bwd_f64(gout, x, k, v, wh, we)

    def fd_row(which, t):
        base = [x[t:t + 1], k[t:t + 1], v[t:t + 1]]
        h = 1e-6 * np.maximum(1.0, np.abs(base[which][0]))
        plus = [np.repeat(b, H, 0) for b in base]
        minus = [np.repeat(b, H, 0) for b in base]
        plus[which] = plus[which] + np.diag(h)
        minus[which] = minus[which] - np.diag(h)
        lp = _row_loss(gout[t], *plus, wh, we)
        lm = _row_loss(gout[t], *minus, wh, we)
        return (lp - lm) / (2 * h)

    for which, ana in ((0, dx), (1, dk), (2, dv)):
        num = np.stack([fd_row(which, t) for t in range(T)])
        num[~keep] = ana[~keep]
        rel = np.linalg.norm(num - ana) / np.linalg.norm(ana)
        assert rel < 1e-7, (which, rel)

    def total_loss(wh_, we_):
        out, _, _ = oracle.fwd_f64(x, k, v, wh_, we_)
        return float(np.sum(gout * out))

    for which, ana in ((0, dwh), (1, dwe)):
        num = np.empty(H)
        for i in range(H):
            w = [wh.copy(), we.copy()]
            h = 1e-6 * max(1.0, abs(w[which][i]))
            w[which][i] += h
            lp = total_loss(*w)
            w[which][i] -= 2 * h
            lm = total_loss(*w)
            num[i] = (lp - lm) / (2 * h)
        rel = np.linalg.norm(num - ana) / np.linalg.norm(ana)
        assert rel < 1e-6, (which, rel)


def test_backward_against_autograd():
    # Automatic differentiation of the forward written with library ops.
    H = 512
    T = 24
    x = rng_rows(T, H, seed=22)
    k = rng_rows(T, H, seed=23) + np.linspace(-1, 1, T)[:, None] * x
    v = rng_rows(T, H, seed=24)
    gout = rng_rows(T, H, seed=25)
    wh, we = weights(H, seed=26)
    _, _, st = oracle.fwd_f64(x, k, v, wh, we)
    assert np.all(np.abs(st[:, 5]) > oracle.CLAMP)   # clamp inactive here
    dx, dk, dv, dwh, dwe, _ = oracle.bwd_f64(gout, x, k, v, wh, we)
    tx, tk, tv, twh, twe = (torch.tensor(a, requires_grad=True) for a in (x, k, v, wh, we))
    a = torch.nn.functional.rms_norm(tx, (H,), twh, EPS)
    b = torch.nn.functional.rms_norm(tk, (H,), twe, EPS)
    z = (a * b).sum(-1) / math.sqrt(H)
    g = torch.sigmoid(torch.sign(z) * torch.sqrt(torch.abs(z)))
    out = tx + g[:, None] * tv
    (out * torch.from_numpy(gout)).sum().backward()
    for ana, ref in ((dx, tx.grad), (dk, tk.grad), (dv, tv.grad), (dwh, twh.grad),
                     (dwe, twe.grad)):
        ref = ref.numpy()
        assert np.linalg.norm(ana - ref) / np.linalg.norm(ref) < 1e-13


def test_backward_invariants():
    gout, x, k, v, wh, we = _config1_f64()
    T, H = x.shape
    dx, dk, dv, dwh, dwe, bst = oracle.bwd_f64(gout, x, k, v, wh, we)
    _, g, st = oracle.fwd_f64(x, k, v, wh, we)
    dd, d = bst[:, 3], st[:, 4]
    scale = np.max(np.abs(wh * dwh))
    # wh * dwh = we * dwe, element by element
    assert np.max(np.abs(wh * dwh - we * dwe)) <= 1e-14 * scale
    # sum_i wh_i dwh_i = sum_t dd_t d_t
    assert abs(np.sum(wh * dwh) - np.sum(dd * d)) <= 1e-12 * np.sum(np.abs(dd * d))
    # scale-freeness of RMSNorm: x . (dx - gout) = dd d eps / (m_x + eps) per row
    ex = np.sum(x * (dx - gout), 1)
    assert np.allclose(ex, dd * d * EPS / (st[:, 0] + EPS), rtol=1e-6, atol=1e-12)
    ek = np.sum(k * dk, 1)
    assert np.allclose(ek, dd * d * EPS / (st[:, 1] + EPS), rtol=1e-6, atol=1e-12)
    # dv = gate * grad_out
    assert np.array_equal(dv, g[:, None] * gout)


def test_backward_special_cases():
    H = 256
    x = rng_rows(6, H, seed=27)
    k = rng_rows(6, H, seed=28)
    v = rng_rows(6, H, seed=29)
    gout = rng_rows(6, H, seed=30)
    wh, we = weights(H, seed=31)
    # v = 0: no gradient reaches the gate
    dx, dk, dv, dwh, dwe, _ = oracle.bwd_f64(gout, x, k, 0 * v, wh, we)
    assert np.array_equal(dx, gout) and np.all(dk == 0)
    assert np.all(dwh == 0) and np.all(dwe == 0)
    # grad_out orthogonal to v (disjoint supports): same
    g2, v2 = gout.copy(), v.copy()
    g2[:, ::2] = 0
    v2[:, 1::2] = 0
    dx, dk, _, dwh, dwe, _ = oracle.bwd_f64(g2, x, k, v2, wh, we)
    assert np.array_equal(dx, g2) and np.all(dk == 0) and np.all(dwh == 0)
    # an x = 0 row: dk row is exactly 0, dx row is grad_out + dd/sqrt(eps) wh*b
    x0 = x.copy()
    x0[2] = 0
    dx, dk, dv, dwh, dwe, bst = oracle.bwd_f64(gout, x0, k, v, wh, we)
    assert np.all(dk[2] == 0) and np.all(np.isfinite(dx))
    _, _, st = oracle.fwd_f64(x0, k, v, wh, we)
    b = k[2] * st[2, 3] * we
    want = gout[2] + bst[2, 3] / math.sqrt(EPS) * wh * b
    assert np.allclose(dx[2], want, rtol=1e-12, atol=1e-12)
    # x = k = v = 0 rows: everything finite, no gate gradient
    z = np.zeros((3, H))
    dx, dk, dv, dwh, dwe, _ = oracle.bwd_f64(gout[:3], z, z, z, wh, we)
    assert np.array_equal(dx, gout[:3]) and np.all(dk == 0)
    assert np.all(np.isfinite(dwh)) and np.all(dwh == 0)


def test_backward_mirror_in_saturation():
    # sigmoid' is even, and so is 1/(2 sqrt|z|): k -> -k flips d, z and s but
    # leaves ds, dz and dd unchanged; d is odd in k, so dk is unchanged and
    # dx - grad_out changes sign. With large weights s reaches about 36,
    # where the gate lies within 1e-15 of 1 and its derivative must still
    # keep full relative precision on both sides.
    H = 256
    x = rng_rows(6, H, seed=40)
    n = rng_rows(6, H, seed=41)
    rho = np.array([1.0, 0.9, 0.6, 0.3, 0.1, 0.02])[:, None]
    k = rho * x + np.sqrt(1.0 - rho ** 2) * n
    v = rng_rows(6, H, seed=42)
    gout = rng_rows(6, H, seed=43)
    c = np.full(H, 9.0)
    dx, dk, _, _, _, bst = oracle.bwd_f64(gout, x, k, v, c, c)
    mdx, mdk, _, _, _, mbst = oracle.bwd_f64(gout, x, -k, v, c, c)
    s = oracle.fwd_f64(x, k, v, c, c)[2][:, 6]
    assert s.max() > 34 and s.min() < 8
    assert np.all(bst[:, 1] != 0)
    assert np.allclose(mbst[:, 1:], bst[:, 1:], rtol=1e-12, atol=0)
    # row by row: the saturated rows' gradients are many orders smaller
    kscale = np.max(np.abs(dk), 1, keepdims=True)
    assert np.all(kscale > 0)
    assert np.all(np.abs(mdk - dk) <= 1e-10 * kscale)
    xscale = np.max(np.abs(dx - gout), 1, keepdims=True)
    assert np.all(np.abs((mdx - gout) + (dx - gout)) <= 1e-10 * xscale)


def test_clamp_bounds_the_derivative():
    # rows with |z| below the clamp use 1/(2 sqrt(clamp)); above, 1/(2 sqrt|z|)
    H = 256
    x = rng_rows(3, H, seed=32)
    k = rng_rows(3, H, seed=33)
    k[:, 1::2] = 0
    x[:, 0::2] = 0          # d = 0 exactly
    gout = rng_rows(3, H, seed=34)
    v = rng_rows(3, H, seed=35)
    wh, we = weights(H, seed=36)
    bst = oracle.bwd_f64(gout, x, k, v, wh, we)[5]
    dg = np.sum(gout * v, 1)
    want_dd = dg * 0.25 * 0.5 / math.sqrt(oracle.CLAMP) / math.sqrt(H)
    assert np.allclose(bst[:, 3], want_dd, rtol=1e-14)


# -------------------------------------------------- bf16 front end and rounding

def test_bf16_front_end_matches_f64():
    d = synth.make_inputs(1)
    f = oracle.bf16_to_f64
    out, g, z = oracle.fwd_bf16(d["x"], d["k"], d["v"], d["wh"], d["we"], threads=3)
    out2, g2, st = oracle.fwd_f64(f(d["x"]), f(d["k"]), f(d["v"]), d["wh"], d["we"])
    assert np.array_equal(out, out2) and np.array_equal(g, g2)
    assert np.array_equal(z, st[:, 5])
    dx, dk, dv, dwh, dwe, dd = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"],
                                               d["wh"], d["we"], threads=5)
    r = oracle.bwd_f64(f(d["grad_out"]), f(d["x"]), f(d["k"]), f(d["v"]), d["wh"], d["we"])
    assert np.array_equal(dx, r[0]) and np.array_equal(dk, r[1])
    assert np.array_equal(dv, r[2]) and np.array_equal(dd, r[5][:, 3])
    assert np.allclose(dwh, r[3], rtol=1e-13, atol=1e-15)
    assert np.allclose(dwe, r[4], rtol=1e-13, atol=1e-15)


def test_round_bf16_matches_torch_on_fp32_values():
    # fp32 -> bf16 in torch is round-to-nearest-even; on fp32-representable
    # inputs the oracle's fp64 -> bf16 rounding must agree bit for bit.
    r = np.random.default_rng(37)
    v = (r.standard_normal(200000) * 10.0 ** r.integers(-20, 20, 200000)).astype(np.float32)
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_brute_force_on_doubles():
    r = np.random.default_rng(38)
    v = r.standard_normal(50000) * 10.0 ** r.integers(-35, 35, 50000)
    bits = oracle.round_bf16(v)
    got = oracle.bf16_to_f64(bits)
    up = oracle.bf16_to_f64((bits.astype(np.int32) + 1).astype(np.uint16))
    dn = oracle.bf16_to_f64((bits.astype(np.int32) - 1).astype(np.uint16))
    err = np.abs(got - v)
    # no bf16 neighbour is nearer to v (ties are checked against torch above)
    assert np.all(err <= np.abs(up - v)) and np.all(err <= np.abs(dn - v))


def _nearest_bf16(v):
    """bf16 bits of fp64 values by IEEE 754 round-to-nearest-even, found by
    searching the table of every finite bf16 value: the nearest one wins,
    a tie goes to the pattern with an even last bit, and a magnitude of at
    least 2^128 - 2^119 (halfway from the largest finite value, 0x7F7F, to
    2^128) rounds to infinity. NaN is not handled."""
    pats = np.arange(0, 0x7F80, dtype=np.uint32)            # +0 up to 0x7F7F
    vals = (pats << 16).view(np.float32).astype(np.float64)  # increasing
    a = np.abs(np.asarray(v, dtype=np.float64))
    hi = np.minimum(np.searchsorted(vals, a), len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = np.abs(a - vals[lo]), np.abs(vals[hi] - a)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(a == vals[hi], hi, pick)
    out = pats[pick].astype(np.uint32)
    out = np.where(a >= 2.0 ** 128 - 2.0 ** 119, 0x7F80, out)
    return (out | np.where(np.signbit(v), 0x8000, 0)).astype(np.uint16)


def test_nearest_bf16_reference_on_known_values():
    # the search above, on values whose bf16 patterns follow from the format
    vals = [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 ** -133, 1.5 * 2 ** -133,
            2.5 * 2 ** -133, 0.5 * 2 ** -133, 0.75 * 2 ** -133, 2.0 ** -126 - 2 ** -134,
            2.0 ** 127 * (2 - 2 ** -7), 2.0 ** 128 - 2.0 ** 119, 2.0 ** 130, -0.0, -1.0]
    want = [0x3F80, 0x3F80, 0x3F82, 0x0001, 0x0002, 0x0002, 0x0000, 0x0001, 0x0080,
            0x7F7F, 0x7F80, 0x7F80, 0x8000, 0xBF80]
    assert _nearest_bf16(np.array(vals)).tolist() == want


def test_round_bf16_across_the_whole_range():
    # |v| from 2^-140 to 2^129: the subnormal bf16 range (multiples of
    # 2^-133, their exact ties and the values next to them), every binade of
    # the normal range, and the top: the largest finite bf16 (0x7F7F), the
    # midpoint to infinity and what lies on either side of both.
    r = np.random.default_rng(43)
    e = np.arange(-140, 130)
    sig = np.concatenate([[1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2 - 2 ** -8, 2 - 2 ** -9],
                          1.0 + r.random(60), 1.0 + r.integers(0, 2 ** 23, 60) * 2.0 ** -23])
    v = (sig[None, :] * 2.0 ** e[:, None]).ravel()
    q = 2.0 ** -133
    j = np.arange(0, 129, dtype=np.float64)
    sub = np.concatenate([j * q, (j + 0.5) * q, (j + 0.25) * q, (j + 0.75) * q])
    top_max = 2.0 ** 127 * (2 - 2 ** -7)           # 0x7F7F
    top_mid = 2.0 ** 128 - 2.0 ** 119                # halfway to 2^128
    top = np.array([top_max, top_mid, 2.0 ** 128, 2.0 ** 129, np.finfo(np.float64).max])
    v = np.concatenate([v, sub, top])
    with np.errstate(over="ignore"):
        near = np.concatenate([np.nextafter(v, 0.0), np.nextafter(v, np.inf)])
    v = np.concatenate([v, near])
    v = v[(v >= 2.0 ** -141) | (v == 0.0)]
    v = np.concatenate([v, -v])
    got = oracle.round_bf16(v)
    assert np.array_equal(got, _nearest_bf16(v))
    assert got[np.argmax(v == top_mid)] == 0x7F80
    assert got[np.argmax(v == np.nextafter(top_mid, 0.0))] == 0x7F7F
    # torch's fp32 -> bf16 on the values fp32 holds exactly, ties included
    with np.errstate(over="ignore"):
        f32 = v.astype(np.float32)
    exact = np.isfinite(f32) & (f32.astype(np.float64) == v)
    want = (torch.from_numpy(f32[exact]).to(torch.bfloat16).view(torch.int16).numpy()
            .view(np.uint16))
    assert exact.sum() > 20000
    assert np.array_equal(got[exact], want)
    # infinities keep their sign, and NaN gives the quiet NaN
    special = oracle.round_bf16(np.array([np.inf, -np.inf, np.nan]))
    assert special.tolist() == [0x7F80, 0xFF80, 0x7FC0]


def test_oracle_snapshot_config1():
    # Regression record written by tests/golden/make_oracle_snapshot.py.
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "config1_oracle_snapshot.txt")
    rows, cols = {}, {}
    for line in open(path):
        p = line.split()
        if p and p[0] == "row":
            rows[int(p[1])] = [float(s) for s in p[2:]]
        elif p and p[0] == "col":
            cols[int(p[1])] = [float(s) for s in p[2:]]
    d = synth.make_inputs(1)
    _, gate, z = oracle.fwd_bf16(d["x"], d["k"], d["v"], d["wh"], d["we"])
    dx, dk, dv, dwh, dwe, dd = oracle.bwd_bf16(d["grad_out"], d["x"], d["k"], d["v"],
                                               d["wh"], d["we"])
    assert len(rows) == 64 and len(cols) == 32
    for t, want in rows.items():
        got = [gate[t], z[t], dd[t], dx[t].sum(), dk[t].sum(), dv[t].sum()]
        assert np.allclose(got, want, rtol=1e-12, atol=1e-14)
    for i, want in cols.items():
        assert np.allclose([dwh[i], dwe[i]], want, rtol=1e-12, atol=1e-14)


def test_fused_weight_is_exact():
    # the fused weight of the "5. Engram" section's weight preprocessing:
    # wh * we formed in fp64 equals the exact rational product
    from fractions import Fraction
    r = np.random.default_rng(41)
    wh = (r.standard_normal(500) * 10.0 ** r.integers(-20, 20, 500)).astype(np.float32)
    we = (r.standard_normal(500) * 10.0 ** r.integers(-20, 20, 500)).astype(np.float32)
    w = oracle.fused_weight(wh, we)
    for a, b, c in zip(wh, we, w):
        assert Fraction(float(a)) * Fraction(float(b)) == Fraction(float(c))
