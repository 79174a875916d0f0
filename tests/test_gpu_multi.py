"""GPU checks of muon_step_multi, the pointer-array step over matrices of any
shapes: each matrix's parameters, momentum buffer and NS output must be
bitwise the ones muon_step_batched gives it (whose parity with the fp64
oracle the other GPU tests establish), whatever the grouping and launch
sharing.  Cases: the 124M custom-sizing set (gates, attn view, mlp: B'X and
the polynomial of attn and mlp share launches), mixed shapes with per-matrix
lr_mul / wd_mul and tall blocks, ACCURATE precision, and a shape group larger
than one pointer table.  The 124M set, in the call the benchmark times (one
muon_step_multi over all 43 matrices), is also checked against the fp64
oracle directly."""
import pytest

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    return m


def _state(shapes, seed):
    """Separate per-matrix tensors (each its own allocation) for a list of
    (rows, cols, view_blocks, lr_mul, wd_mul)."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    mats = []
    for r, c, v, lm, wm in shapes:
        P = torch.randn((r, c), generator=gen, device="cuda") / c ** 0.5
        G = (torch.randn((r, c), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
        M = torch.randn((r, c), generator=gen, device="cuda") * 1e-3
        mats.append(dict(params=P, grads=G, momentum_buf=M, update_out=torch.empty_like(G),
                         view_blocks=v, lr_mul=lm, wd_mul=wm))
    return mats


def _clone(mats):
    return [{k: (v.clone() if hasattr(v, "clone") else v) for k, v in m.items()} for m in mats]


def _reference(nsm, mats, steps, **kw):
    """muon_step_batched on each matrix alone (a batch of one)."""
    for _ in range(steps):
        for m in mats:
            nsm.muon_step_batched(m["params"], m["grads"], m["momentum_buf"], view_blocks=m["view_blocks"],
                                  lr_mul=m["lr_mul"], wd_mul=m["wd_mul"], update_out=m["update_out"], **kw)


def _check_equal(got, ref, label):
    import torch
    torch.cuda.synchronize()
    for i, (g, r) in enumerate(zip(got, ref)):
        for k in ("params", "momentum_buf", "update_out"):
            assert torch.equal(g[k].view(torch.int16) if g[k].dtype == torch.bfloat16 else g[k].view(torch.int32),
                               r[k].view(torch.int16) if r[k].dtype == torch.bfloat16 else r[k].view(torch.int32)), \
                f"{label}: matrix {i} ({tuple(g['params'].shape)}, view {g['view_blocks']}) differs in {k}"


def _run_case(nsm, shapes, seed, steps=2, precision="fast", label=""):
    print(f"[multi] {label}: {len(shapes)} matrices, precision={precision}", flush=True)
    mats = _state(shapes, seed)
    ref = _clone(mats)
    kw = dict(lr=0.02, weight_decay=0.01, momentum=0.95, precision=precision)
    for _ in range(steps):
        nsm.muon_step_multi(mats, **kw)
    _reference(nsm, ref, steps, **kw)
    _check_equal(mats, ref, label)


def test_multi_gpt124m_set(nsm):
    wl = workloads.get_workload("gpt124m")
    shapes = []
    for g in wl.groups:
        shapes += [(g.rows, g.cols, g.view_blocks, 1.0, 1.0)] * g.count
    _run_case(nsm, shapes, seed=1, label="124M custom sizing")


def test_multi_mixed_shapes_and_multipliers(nsm):
    shapes = [(512, 512, 1, 1.0, 1.0), (512, 256, 1, 0.5, 2.0), (256, 512, 1, 1.0, 0.0), (512, 512, 1, 2.0, 1.0),
              (1024, 512, 1, 1.0, 1.0), (512, 1024, 1, 1.5, 0.5), (1, 12, 1, 1.0, 1.0), (96, 384, 4, 1.0, 1.0),
              (300, 700, 1, 1.0, 1.0), (700, 300, 1, 0.7, 1.3), (33, 70, 1, 1.0, 1.0), (1536, 768, 1, 1.0, 1.0),
              (768, 1536, 1, 1.0, 1.0)]
    _run_case(nsm, shapes, seed=2, label="mixed")


def test_multi_accurate(nsm):
    shapes = [(256, 640, 1, 1.0, 1.0), (640, 256, 1, 1.0, 1.0), (256, 640, 1, 0.5, 2.0), (256, 256, 1, 1.0, 1.0)]
    _run_case(nsm, shapes, seed=3, precision="accurate", label="accurate")


def test_multi_many_matrices_one_shape(nsm):
    # 40 matrices of one shape: the shape group spans two pointer tables (32 + 8)
    shapes = [(64, 128, 1, 1.0 + 0.01 * i, 1.0) for i in range(40)] + [(1, 12, 1, 1.0, 1.0)] * 35
    _run_case(nsm, shapes, seed=4, label="many")


def test_multi_merged_conv_kernels_match_oracle(nsm):
    """>2-D parameters are stepped as the 2-D matrix merge_small_dims gives
    (threshold 8192): a (32, 3, 64, 64) convolution kernel as 96 x 4096 (the
    pages' example, matrix-core path), (8, 4, 5, 5) as 8 x 100 and
    (16, 1, 3, 3) as 16 x 9 (small-block path).  Checked against the fp64
    oracle's step on the oracle's own merged view."""
    import numpy as np
    import torch
    import oracle
    from oracle.shape_oracle import merge_small_dims
    from parity import (MOMENTUM_TOL, NS_REL_TOL, assert_ns_close, bits_to_f64, rel_fro,
                        torch_bf16_to_bits)
    shapes = [(32, 3, 64, 64), (8, 4, 5, 5), (16, 1, 3, 3)]
    rng = np.random.default_rng(31)
    mats, host = [], []
    for k, shp in enumerate(shapes):
        P0 = (rng.standard_normal(shp) * 0.02).astype(np.float32)
        gb = workloads.gaussian_bits(shp, seed=700 + k, std=1e-2)
        P = torch.from_numpy(P0).cuda()
        mats.append(dict(params=P, grads=workloads.to_device_bf16(gb), momentum_buf=torch.zeros_like(P),
                         update_out=torch.empty(shp, dtype=torch.bfloat16, device="cuda")))
        host.append((P0, gb))
    print("[multi merge] conv-shaped parameters", flush=True)
    nsm.muon_step_multi(mats, lr=0.02, weight_decay=0.01, momentum=0.95)
    torch.cuda.synchronize()
    for shp, m, (P0, gb) in zip(shapes, mats, host):
        r, c = merge_small_dims(shp, 8192, 2)
        assert nsm.muon_merge_small_dims(shp, 8192, 2) == (r, c)
        P_ref, M_ref, O_ref = oracle.muon_step(P0.reshape(1, r, c), bits_to_f64(gb).reshape(1, r, c),
                                               np.zeros((1, r, c)), lr=0.02, weight_decay=0.01, momentum=0.95)
        O_got = bits_to_f64(torch_bf16_to_bits(m["update_out"])).reshape(r, c)
        assert_ns_close(O_got, O_ref[0], label=f"{shp} as {r}x{c}")
        assert rel_fro(m["momentum_buf"].cpu().numpy().reshape(r, c), M_ref[0]) <= MOMENTUM_TOL
        lr_eff = float(np.float32(0.02)) * oracle.aspect_factor(r, c)
        bound = NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_ref)
        assert np.linalg.norm(m["params"].cpu().numpy().reshape(r, c) - P_ref[0]) <= bound
    # a tensor that cannot merge to 2-D at this threshold is rejected before any work
    bad = torch.zeros((4096, 3, 4096), device="cuda")
    with pytest.raises(ValueError):
        nsm.muon_step_multi([dict(params=bad, grads=bad.to(torch.bfloat16), momentum_buf=bad.clone())],
                            lr=0.02, weight_decay=0.0, momentum=0.95)


@pytest.mark.timeout(600)
def test_multi_gpt124m_set_matches_oracle(nsm):
    """One muon_step_multi over the 43 matrices of the 124M custom-sizing set
    (11 gates 1x12, 10 attn 768x3072 with view 4, 22 mlp 768x3072), 3 steps of
    the workload's settings, every matrix against the fp64 oracle after every
    step: NS output (update_out), momentum buffer and parameters."""
    import numpy as np
    import torch
    import oracle
    from parity import MOMENTUM_TOL, NS_REL_TOL, assert_ns_close, bits_to_f64, rel_fro, torch_bf16_to_bits
    wl = workloads.get_workload("gpt124m")
    mats, refs = [], []
    for grp in wl.groups:
        P_host = workloads.param_init_host(wl, grp)
        for i in range(grp.count):
            P = torch.from_numpy(P_host[i].copy()).cuda()
            mats.append(dict(params=P, grads=None, momentum_buf=torch.zeros_like(P),
                             update_out=torch.empty(P.shape, dtype=torch.bfloat16, device="cuda"),
                             view_blocks=grp.view_blocks))
            refs.append(dict(grp=grp, i=i, P=P_host[i].astype(np.float64), M=np.zeros(P.shape), bound=0.0))
    worst = 0.0
    for t in range(wl.steps):
        print(f"[multi oracle] 124M set step {t}", flush=True)
        bits = {}
        for grp in wl.groups:
            bits[grp.name] = workloads.grad_bits_host(wl, grp, t)
        for m, r in zip(mats, refs):
            m["grads"] = workloads.to_device_bf16(bits[r["grp"].name][r["i"]])
        nsm.muon_step_multi(mats, lr=wl.lr, weight_decay=wl.weight_decay, momentum=wl.momentum,
                            ns_steps=wl.ns_steps, precision="fast")
        torch.cuda.synchronize()
        for m, r in zip(mats, refs):
            grp = r["grp"]
            g = bits_to_f64(bits[grp.name][r["i"]])
            P_new, M_new, O_ref = oracle.muon_step(r["P"][None], g[None], r["M"][None], lr=wl.lr,
                                                   weight_decay=wl.weight_decay, momentum=wl.momentum,
                                                   view_blocks=grp.view_blocks, ns_steps=wl.ns_steps)
            label = f"{grp.name}[{r['i']}] step {t}"
            rel, _ = assert_ns_close(bits_to_f64(torch_bf16_to_bits(m["update_out"])), O_ref[0], grp.view_blocks,
                                     sigma=(t == 0), label=label)
            worst = max(worst, rel)
            em = rel_fro(m["momentum_buf"].cpu().numpy(), M_new[0])
            assert em <= MOMENTUM_TOL, f"momentum {label}: {em:.3e}"
            lr_eff = float(np.float32(wl.lr)) * oracle.aspect_factor(grp.rows, grp.cols)
            r["bound"] += NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_new)
            ep = np.linalg.norm(m["params"].cpu().numpy() - P_new[0])
            assert ep <= r["bound"], f"params {label}: {ep:.3e} > {r['bound']:.3e}"
            r["P"], r["M"] = P_new[0], M_new[0]
    print(f"[multi oracle] worst NS relative error over 43 matrices x {wl.steps} steps: {worst:.3e}", flush=True)
