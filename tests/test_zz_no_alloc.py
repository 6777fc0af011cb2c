"""The allocation-free backward, tk_engram_gate_bwd_reduce_noalloc, against
the backward and the reduction it combines (tk_engram_gate_bwd, then
tk_engram_grad_w_reduce with a caller's workspace).

Both run the same kernels with the same number of partials, so every output
must be bit-identical. Calls follow one another on one GPU with shrinking
inputs, so each later call finds the earlier call's partials in the
library's array and must not be affected by them.
"""

import sys

import pytest

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def eg(cuda_device):
    import engram_conditional_memory_amd as m
    m.load_library()
    return m


def inputs(T, H, dev, seed):
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)

    def rows():
        return torch.randn((T, H), device=dev, generator=g).to(torch.bfloat16)

    x, go, v = rows(), rows(), rows()
    rho = torch.rand((T, 1), device=dev, generator=g) * 2 - 1
    k = (rho * x.float() + (1 - rho * rho).sqrt() * torch.randn((T, H), device=dev,
                                                                  generator=g)).to(torch.bfloat16)
    wh = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    we = 1 + 0.1 * torch.randn(H, device=dev, generator=g)
    return go, x, k, v, wh, we


def same_bits(a, b):
    import torch
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


def check_against_workspace_path(eg, dev, T, H, seed):
    import torch
    say(f"[no-alloc] T={T} H={H} seed={seed}")
    go, x, k, v, wh, we = inputs(T, H, dev, seed)
    dx, dk, dv, ws, P = eg.tk_engram_gate_bwd(go, x, k, v, wh, we)
    dwh, dwe = eg.tk_engram_grad_w_reduce(ws, P, H, wh, we)
    ndx, ndk, ndv, ndwh, ndwe = eg.tk_engram_gate_bwd_reduce_noalloc(go, x, k, v, wh, we)
    torch.cuda.synchronize()
    for name, a, b in (("dx", dx, ndx), ("dk", dk, ndk), ("dv", dv, ndv),
                       ("dwh", dwh, ndwh), ("dwe", dwe, ndwe)):
        assert same_bits(a, b), f"{name} differs at T={T} H={H}"
    if T > 0:
        assert torch.isfinite(dwh).all() and dwh.abs().sum() > 0


@pytest.mark.parametrize("shapes", [
    [(20003, 7168), (4099, 7168), (1000, 7168)],   # the tuned width: two launches (epochs),
                                                   # then one, ragged, then fewer rows
    [(3000, 2048), (700, 4096), (33, 256)],  # most partials (P = 512 at H = 2048), then
                                             # other widths over the leftovers
])
def test_noalloc_matches_workspace_path_on_successive_calls(eg, cuda_device, shapes):
    for i, (T, H) in enumerate(shapes):
        check_against_workspace_path(eg, cuda_device, T, H, seed=100 + i)


def test_noalloc_largest_partials_then_smaller(eg, cuda_device):
    # the largest partial array any shape uses (P = 256 at H = 8192, the whole
    # 8 MiB array), then a smaller shape
    check_against_workspace_path(eg, cuda_device, 600, 8192, seed=7)
    check_against_workspace_path(eg, cuda_device, 65, 1024, seed=8)


def test_noalloc_empty_batch_writes_zero_weight_gradients(eg, cuda_device):
    import torch
    H = 512
    go, x, k, v, wh, we = inputs(0, H, cuda_device, 9)
    dwh = torch.full((H,), 3.0, device=cuda_device)
    dwe = torch.full((H,), 3.0, device=cuda_device)
    eg.tk_engram_gate_bwd_reduce_noalloc(go, x, k, v, wh, we, dwh=dwh, dwe=dwe)
    torch.cuda.synchronize()
    assert torch.equal(dwh, torch.zeros_like(dwh)) and torch.equal(dwe, torch.zeros_like(dwe))
