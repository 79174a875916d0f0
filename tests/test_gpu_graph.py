"""GPU checks of HIP graph capture.

Under stream capture a call enqueues only kernels on the caller's stream: no
allocation, no synchronisation and no event (the automatic NS schedule and
tile choice reuse what earlier calls settled, else take the per-product
launches and the estimated tiling, which give bitwise the same results).  So
a captured call replays to the eager result bit for bit.  Each graph is
replayed several times with eager work and synchronisations in between (that
work uses the same library state: workspaces, the static scratch of the
allocation-free entry point), and every replay is checked.
"""
import numpy as np
import pytest

import workloads
from parity import torch_bf16_to_bits

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    yield m
    m.muon_set_ns_schedule("auto")
    m.muon_set_gemm_tiling(0)


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("shape", [(3, 300, 700), (4, 512, 1024), (2, 1000, 260)])
def test_noalloc_graph_replays(nsm, shape):
    import torch
    print(f"[graph] noalloc {shape}", flush=True)
    x = workloads.to_device_bf16(workloads.gaussian_bits(shape, seed=sum(shape)))
    y = workloads.to_device_bf16(workloads.gaussian_bits(shape, seed=sum(shape) + 1))
    out = torch.empty_like(x)
    other = torch.empty_like(x)
    nsm.ns_orthogonalize_batched_noalloc(x, out)     # first call on the device: resolves the scratch address
    torch.cuda.synchronize()
    want = torch_bf16_to_bits(out)
    g = _capture(lambda: nsm.ns_orthogonalize_batched_noalloc(x, out))
    for r in range(REPLAYS):
        out.zero_()
        nsm.ns_orthogonalize_batched_noalloc(y, other)   # eager work on the same scratch in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(torch_bf16_to_bits(out), want, err_msg=f"replay {r}")


@pytest.mark.parametrize("schedule", ["auto", "per_product", "persistent"])
def test_ns_graph_replays(nsm, schedule):
    # the settled automatic schedule (and the cached loop queue) are reused under capture
    import torch
    print(f"[graph] ns_orthogonalize_batched 8 x 512x1024 schedule={schedule}", flush=True)
    nsm.muon_set_ns_schedule(schedule)
    try:
        x = workloads.to_device_bf16(workloads.gaussian_bits((8, 512, 1024), seed=77))
        out = torch.empty_like(x)
        for _ in range(12):                      # lets the automatic choices settle
            nsm.ns_orthogonalize_batched(x, out)
        torch.cuda.synchronize()
        want = torch_bf16_to_bits(out)
        g = _capture(lambda: nsm.ns_orthogonalize_batched(x, out))
        for r in range(REPLAYS):
            out.zero_()
            nsm.ns_orthogonalize_batched(x, torch.empty_like(x))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(torch_bf16_to_bits(out), want, err_msg=f"replay {r}")
    finally:
        nsm.muon_set_ns_schedule("auto")


def test_ns_graph_first_call_captured(nsm):
    # a shape set never seen before: under capture it takes the per-product
    # launches with the estimated tiling (no queue built, nothing timed)
    import torch
    print("[graph] first call under capture 6 x 384x1280", flush=True)
    x = workloads.to_device_bf16(workloads.gaussian_bits((6, 384, 1280), seed=5))
    out = torch.empty_like(x)
    g = _capture(lambda: nsm.ns_orthogonalize_batched(x, out))
    g.replay()
    torch.cuda.synchronize()
    got = torch_bf16_to_bits(out)
    nsm.muon_set_ns_schedule("per_product")
    try:
        ref = torch.empty_like(x)
        nsm.ns_orthogonalize_batched(x, ref)
        torch.cuda.synchronize()
    finally:
        nsm.muon_set_ns_schedule("auto")
    np.testing.assert_array_equal(got, torch_bf16_to_bits(ref))


def test_step_graph_replays(nsm):
    # in-place Muon steps: each replay advances params and momentum exactly as an eager step
    import torch
    print("[graph] muon_step_batched 4 x 640x1280", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    P0 = torch.randn((4, 640, 1280), generator=gen, device="cuda") / 1280 ** 0.5
    G = (torch.randn((4, 640, 1280), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
    M0 = torch.randn((4, 640, 1280), generator=gen, device="cuda") * 1e-3
    kw = dict(lr=0.02, weight_decay=0.01, momentum=0.95)
    Pe, Me = P0.clone(), M0.clone()
    for _ in range(12):                          # settle the automatic choices on a scratch copy
        nsm.muon_step_batched(P0.clone(), G, M0.clone(), **kw)
    Pg, Mg = P0.clone(), M0.clone()
    g = _capture(lambda: nsm.muon_step_batched(Pg, G, Mg, **kw))
    # capturing does not run the step: Pg, Mg still hold the initial state
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Pg.cpu().numpy().view(np.int32), P0.cpu().numpy().view(np.int32))
    for r in range(REPLAYS):
        nsm.muon_step_batched(Pe, G, Me, **kw)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Pg.cpu().numpy().view(np.int32), Pe.cpu().numpy().view(np.int32),
                                      err_msg=f"params after replay {r}")
        np.testing.assert_array_equal(Mg.cpu().numpy().view(np.int32), Me.cpu().numpy().view(np.int32),
                                      err_msg=f"momentum after replay {r}")
