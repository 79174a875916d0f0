"""GPU parity of adamw_step_multi (the AdamW step of the non-matrix parameters)
against the fp64 oracle, element by element.

Tolerance (derived from the fp32 arithmetic of the kernel): each of m, v and p
is a handful of fp32 operations on the previous values, so its error is a few
units of 2^-24 of the magnitudes involved.  Per element:
  |m - m_ref| <= 1e-6 (|m_ref| + (1 - beta1) |g|)
  |v - v_ref| <= 1e-6 (|v_ref| + (1 - beta2) g^2)
  |p - p_ref| <= 1e-6 (|p_ref| + step (|m_ref| + (1 - beta1) |g|) / (sqrt(v_ref) + eps))
(the momentum bound 1e-6 relative of the Muon step, applied per element with
the scale of the terms that form each value; states carry across steps on
both sides).  Cases: ragged sizes around the 8-element vector groups and the
8192-element chunks, a 3-D tensor, an unaligned tensor (element path), empty
tensors, per-tensor step counts and multipliers, weight decay on and off,
several steps, more tensors than one launch takes, the 124M record's
embedding + head + scalars at full size (sampled), and bitwise repeatability."""
import numpy as np
import pytest

import oracle
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


def _check(name, got, ref, scale):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bound = 1e-6 * scale + 1e-30
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (f"{name}: {bad.size} elements out of tolerance, first {bad[:5]}, "
                           f"err {err[bad[:5]]}, bound {bound[bad[:5]]}")


def _ref_step(p, g, m, v, t, *, lr, betas, eps, wd, lr_mul, wd_mul):
    pn, mn, vn = oracle.adamw_step(p, g, m, v, t=t, lr=lr, beta1=betas[0], beta2=betas[1], eps=eps,
                                   weight_decay=wd, lr_mul=lr_mul, wd_mul=wd_mul)
    _, step = oracle.adam_scalars(t, lr=lr, beta1=betas[0], beta2=betas[1], weight_decay=wd,
                                  lr_mul=lr_mul, wd_mul=wd_mul)
    b1, b2 = float(np.float32(betas[0])), float(np.float32(betas[1]))
    scales = dict(m=np.abs(mn) + (1 - b1) * np.abs(g), v=np.abs(vn) + (1 - b2) * g * g,
                  p=np.abs(pn) + step * (np.abs(mn) + (1 - b1) * np.abs(g)) / (np.sqrt(vn) + float(np.float32(eps))))
    return (pn, mn, vn), scales


SPECS = [  # (shape, step t, lr_mul, wd_mul, start moments nonzero, unaligned)
    ((1000, 768), 1, 1.0, 1.0, False, False),
    ((48,), 1, 1.0, 1.0, False, False),
    ((13,), 4, 2.0, 0.5, True, False),
    ((8191,), 1, 1.0, 1.0, False, False),
    ((8192 + 7,), 2, 0.5, 1.0, True, False),
    ((3, 5, 7), 7, 1.0, 3.0, True, False),
    ((3001,), 1, 1.0, 1.0, True, True),
    ((0,), 1, 1.0, 1.0, False, False),
    ((64, 129), 10, 1.0, 1.0, True, False),
]


def _make(specs, seed):
    import torch
    rng = np.random.default_rng(seed)
    host, dev = [], []
    for i, (shape, t, lm, wm, warm, unal) in enumerate(specs):
        n = int(np.prod(shape))
        p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-3).astype(np.float32) if warm else np.zeros(n, np.float32)
        v = (rng.random(n) * 1e-6).astype(np.float32) if warm else np.zeros(n, np.float32)
        host.append(dict(p=p.astype(np.float64), m=m.astype(np.float64), v=v.astype(np.float64), t=t, lm=lm, wm=wm))
        off = 1 if unal else 0

        def put(a, dtype=torch.float32):
            buf = torch.zeros(n + off, dtype=dtype, device="cuda")
            view = buf[off:off + n]
            view.copy_(torch.from_numpy(a).to(dtype))
            return view.view(shape)
        dev.append(dict(params=put(p), exp_avg=put(m), exp_avg_sq=put(v), step=t, lr_mul=lm, wd_mul=wm,
                        grads=torch.zeros(shape, dtype=torch.bfloat16, device="cuda")))
    return host, dev


@pytest.mark.parametrize("wd", [0.0, 0.05])
def test_adamw_parity_mixed(nsm, wd):
    import torch
    print(f"[adamw parity] mixed tensors wd={wd}", flush=True)
    lr, betas, eps = 0.008, (0.8, 0.95), 1e-8
    host, dev = _make(SPECS, seed=11)
    for step in range(3):
        gb = []
        for i, (shape, *_r) in enumerate(SPECS):
            n = int(np.prod(shape))
            bits = workloads.gaussian_bits((n,), seed=1000 * step + i, std=1e-3)
            gb.append(bits)
            if n:
                dev[i]["grads"] = workloads.to_device_bf16(bits).view(shape)
        nsm.adamw_step_multi(dev, lr=lr, betas=betas, eps=eps, weight_decay=wd)
        torch.cuda.synchronize()
        for i, h in enumerate(host):
            g = workloads.bf16_bits_to_f32(gb[i]).astype(np.float64)
            (pn, mn, vn), sc = _ref_step(h["p"], g, h["m"], h["v"], h["t"], lr=lr, betas=betas, eps=eps, wd=wd,
                                         lr_mul=h["lm"], wd_mul=h["wm"])
            d = dev[i]
            got_p = d["params"].reshape(-1).cpu().numpy()
            got_m = d["exp_avg"].reshape(-1).cpu().numpy()
            got_v = d["exp_avg_sq"].reshape(-1).cpu().numpy()
            _check(f"step{step} t{i} exp_avg", got_m, mn, sc["m"])
            _check(f"step{step} t{i} exp_avg_sq", got_v, vn, sc["v"])
            _check(f"step{step} t{i} params", got_p, pn, sc["p"])
            # carry the GPU state forward on both sides (the oracle starts each step from it)
            h["p"], h["m"], h["v"] = got_p.astype(np.float64), got_m.astype(np.float64), got_v.astype(np.float64)
            h["t"] += 1
            d["step"] = h["t"]


def test_adamw_zero_decay_and_zero_grad_keep_params(nsm):
    import torch
    p = torch.randn(5000, device="cuda")
    p0 = p.clone()
    t = dict(params=p, grads=torch.zeros(5000, dtype=torch.bfloat16, device="cuda"),
             exp_avg=torch.zeros(5000, device="cuda"), exp_avg_sq=torch.zeros(5000, device="cuda"), step=1)
    nsm.adamw_step_multi([t], lr=0.008, betas=(0.8, 0.95), eps=1e-8, weight_decay=0.0)
    torch.cuda.synchronize()
    assert torch.equal(p, p0)
    assert not t["exp_avg"].any() and not t["exp_avg_sq"].any()


def test_adamw_many_tensors_two_launches(nsm):
    import torch
    specs = [((100 + 37 * i,), 1 + i % 3, 1.0 + 0.1 * i, 1.0, i % 2 == 0, i % 5 == 0) for i in range(30)]
    host, dev = _make(specs, seed=12)
    lr, betas, eps, wd = 0.01, (0.9, 0.99), 1e-6, 0.1
    gb = []
    for i, (shape, *_r) in enumerate(specs):
        bits = workloads.gaussian_bits(shape, seed=500 + i, std=1e-2)
        gb.append(bits)
        dev[i]["grads"] = workloads.to_device_bf16(bits)
    nsm.muon_timing_enable(["adamw"])
    nsm.adamw_step_multi(dev, lr=lr, betas=betas, eps=eps, weight_decay=wd)
    kt = nsm.muon_timing_collect()
    nsm.muon_timing_enable([])
    assert kt["adamw"][0] == 2     # 30 tensors: 24 + 6
    for i, h in enumerate(host):
        g = workloads.bf16_bits_to_f32(gb[i]).astype(np.float64)
        (pn, mn, vn), sc = _ref_step(h["p"], g, h["m"], h["v"], h["t"], lr=lr, betas=betas, eps=eps, wd=wd,
                                     lr_mul=h["lm"], wd_mul=h["wm"])
        _check(f"t{i} params", dev[i]["params"].cpu().numpy(), pn, sc["p"])
        _check(f"t{i} exp_avg", dev[i]["exp_avg"].cpu().numpy(), mn, sc["m"])
        _check(f"t{i} exp_avg_sq", dev[i]["exp_avg_sq"].cpu().numpy(), vn, sc["v"])


def _full_state(wl):
    import torch
    out = []
    for i, (name, shape) in enumerate(wl.tensors):
        P = workloads.adam_params_device(wl, i)
        out.append(dict(params=P, grads=workloads.adam_grads_device(wl, i, 0),
                        exp_avg=torch.zeros_like(P), exp_avg_sq=torch.zeros_like(P), step=1))
    return out


def test_adamw_gpt124m_full_size_sampled(nsm):
    """The 124M record's embedding, head and scalars at full size, three steps;
    100k sampled elements per tensor (and every scalar) checked against the
    oracle run on those elements' own histories."""
    import torch
    wl = workloads.ADAM_WORKLOADS["gpt124m_adam"]
    print(f"[adamw parity] {wl.name} full size", flush=True)
    state = _full_state(wl)
    rng = np.random.default_rng(7)
    samples, hist = [], []
    for i, d in enumerate(state):
        n = d["params"].numel()
        idx = np.arange(n) if n <= 100_000 else np.unique(np.concatenate(
            [rng.choice(n, 100_000, replace=False), [0, n - 1, n - 8, 8191, 8192]]))
        samples.append(torch.from_numpy(idx).cuda())
        p0 = d["params"].reshape(-1)[samples[-1]].cpu().numpy().astype(np.float64)
        hist.append(dict(p=p0, m=np.zeros(idx.size), v=np.zeros(idx.size)))
    for step in range(3):
        if step:
            for i, d in enumerate(state):
                d["grads"] = workloads.adam_grads_device(wl, i, step)
        gs = [d["grads"].reshape(-1)[samples[i]].float().cpu().numpy().astype(np.float64)
              for i, d in enumerate(state)]
        nsm.adamw_step_multi(state, lr=wl.lr, betas=wl.betas, eps=wl.eps, weight_decay=wl.weight_decay)
        torch.cuda.synchronize()
        for i, d in enumerate(state):
            h = hist[i]
            (pn, mn, vn), sc = _ref_step(h["p"], gs[i], h["m"], h["v"], step + 1, lr=wl.lr, betas=wl.betas,
                                         eps=wl.eps, wd=wl.weight_decay, lr_mul=1.0, wd_mul=1.0)
            gp = d["params"].reshape(-1)[samples[i]].cpu().numpy()
            gm = d["exp_avg"].reshape(-1)[samples[i]].cpu().numpy()
            gv = d["exp_avg_sq"].reshape(-1)[samples[i]].cpu().numpy()
            _check(f"{wl.tensors[i][0]} step{step} params", gp, pn, sc["p"])
            _check(f"{wl.tensors[i][0]} step{step} exp_avg", gm, mn, sc["m"])
            _check(f"{wl.tensors[i][0]} step{step} exp_avg_sq", gv, vn, sc["v"])
            h["p"], h["m"], h["v"] = gp.astype(np.float64), gm.astype(np.float64), gv.astype(np.float64)
            d["step"] = step + 2


def test_adamw_bitwise_repeatable(nsm):
    import torch
    wl = workloads.ADAM_WORKLOADS["gpt124m_adam"]
    a = _full_state(wl)
    b = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()} for d in a]
    for s in (a, b):
        nsm.adamw_step_multi(s, lr=wl.lr, betas=wl.betas, eps=wl.eps, weight_decay=0.01)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        for k in ("params", "exp_avg", "exp_avg_sq"):
            assert torch.equal(x[k], y[k])
