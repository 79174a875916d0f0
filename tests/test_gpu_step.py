"""GPU parity of muon_step_batched against the fp64 oracle on the seeded
workloads: the tiny 4 x 64x128 batch, the 9-layer d=512 GQA matrices, the
124M custom-sizing set (gates + attn view + mlp), and a sampled check of the
96-matrix GPT-2-medium-like batch with heavy-tailed rows (stored wide and
tall)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import (MOMENTUM_TOL, NS_REL_TOL, assert_ns_close, bits_to_f64, rel_fro,
                    torch_bf16_to_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    return m


def _run_host_workload(nsm, wl, steps=None, sigma_every=True):
    """Runs `steps` optimizer steps of every group on the GPU and in the oracle,
    checking O, M and P after every step."""
    import torch
    steps = wl.steps if steps is None else steps
    worst = {"ns": 0.0, "mom": 0.0, "param": 0.0}
    for grp in wl.groups:
        P_host = workloads.param_init_host(wl, grp)
        P = torch.from_numpy(P_host).cuda()
        M = torch.zeros_like(P)
        O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
        P_ref = P_host.astype(np.float64)
        M_ref = np.zeros_like(P_ref)
        bound = 0.0
        for t in range(steps):
            mu = wl.momentum_at(t)
            gbits = workloads.grad_bits_host(wl, grp, t)
            print(f"[step parity] {wl.name}/{grp.name} {grp.count}x{grp.rows}x{grp.cols} "
                  f"view={grp.view_blocks} step={t}", flush=True)
            G = workloads.to_device_bf16(gbits)
            nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay, momentum=mu,
                                  view_blocks=grp.view_blocks, ns_steps=wl.ns_steps,
                                  precision=grp.precision, update_out=O)
            torch.cuda.synchronize()
            P_new, M_new, O_ref = oracle.muon_step(P_ref, bits_to_f64(gbits), M_ref, lr=wl.lr,
                                                   weight_decay=wl.weight_decay, momentum=mu,
                                                   view_blocks=grp.view_blocks, ns_steps=wl.ns_steps)
            O_got = bits_to_f64(torch_bf16_to_bits(O))
            M_got = M.cpu().numpy().astype(np.float64)
            P_got = P.cpu().numpy().astype(np.float64)
            lr_eff = float(np.float32(wl.lr)) * oracle.aspect_factor(grp.rows, grp.cols)
            for i in range(grp.count):
                r, s = assert_ns_close(O_got[i], O_ref[i], grp.view_blocks, sigma=sigma_every or t == 0,
                                       label=f"{grp.name}[{i}] step {t}")
                worst["ns"] = max(worst["ns"], r)
                em = rel_fro(M_got[i], M_new[i])
                assert em <= MOMENTUM_TOL, f"momentum {grp.name}[{i}] step {t}: {em:.3e}"
                worst["mom"] = max(worst["mom"], em)
            bound += NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_new)
            ep = np.linalg.norm(P_got - P_new)
            assert ep <= bound, f"params {grp.name} step {t}: {ep:.3e} > {bound:.3e}"
            worst["param"] = max(worst["param"], ep / bound)
            P_ref, M_ref = P_new, M_new
    print(f"[step parity] {wl.name} worst: {worst}", flush=True)
    return worst


def test_step_tiny(nsm):
    _run_host_workload(nsm, workloads.get_workload("tiny"))


def test_step_tiny_plain_momentum_and_multipliers(nsm):
    import torch
    wl = workloads.get_workload("tiny")
    grp = wl.groups[0]
    P_host = workloads.param_init_host(wl, grp)
    P = torch.from_numpy(P_host).cuda()
    M = torch.full_like(P, 0.25)
    gbits = workloads.grad_bits_host(wl, grp, 0)
    O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
    nsm.muon_step_batched(P, workloads.to_device_bf16(gbits), M, lr=0.1, weight_decay=0.3,
                          momentum=0.9, nesterov=False, lr_mul=0.5, wd_mul=2.0, update_out=O)
    torch.cuda.synchronize()
    P_ref, M_ref, O_ref = oracle.muon_step(P_host, bits_to_f64(gbits), np.full(P_host.shape, 0.25),
                                           lr=0.1, weight_decay=0.3, momentum=0.9, nesterov=False,
                                           lr_mul=0.5, wd_mul=2.0)
    for i in range(grp.count):
        assert_ns_close(bits_to_f64(torch_bf16_to_bits(O))[i], O_ref[i], label=f"plain[{i}]")
        assert rel_fro(M.cpu().numpy()[i], M_ref[i]) <= MOMENTUM_TOL
    bound = NS_REL_TOL * 0.05 * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_ref)
    assert np.linalg.norm(P.cpu().numpy() - P_ref) <= bound


def test_step_gqa_small(nsm):
    _run_host_workload(nsm, workloads.get_workload("gqa_small"), sigma_every=False)


def test_step_gpt124m(nsm):
    _run_host_workload(nsm, workloads.get_workload("gpt124m"), sigma_every=False)


def test_step_gpt2_medium_sampled(nsm):
    """96 matrices (48 wide 1024x4096, 48 stored tall 4096x1024), heavy-tailed
    rows, 20 steps on the GPU; the oracle follows one wide and one tall matrix
    through all 20 steps (momentum and parameters every step, NS output at the
    first and the last step)."""
    import torch
    wl = workloads.get_workload("gpt2_medium")
    sample = {0: [17], 1: [30]}
    for gi, grp in enumerate(wl.groups):
        P = workloads.params_device(wl, grp)
        M = torch.zeros_like(P)
        O = torch.empty(P.shape, dtype=torch.bfloat16, device="cuda")
        idx = sample[gi]
        P_ref = P[idx].cpu().numpy().astype(np.float64)
        M_ref = np.zeros_like(P_ref)
        bound = 0.0
        for t in range(wl.steps):
            print(f"[step parity] gpt2_medium/{grp.name} step={t}", flush=True)
            G = workloads.grads_device(wl, grp, t)
            g_host = bits_to_f64(torch_bf16_to_bits(G[idx]))
            nsm.muon_step_batched(P, G, M, lr=wl.lr, weight_decay=wl.weight_decay,
                                  momentum=wl.momentum, update_out=O)
            torch.cuda.synchronize()
            need_ns = t in (0, wl.steps - 1)
            M_new, U = oracle.nesterov_momentum(g_host, M_ref, wl.momentum)
            O_ref = np.stack([oracle.newton_schulz(u) for u in U])
            P_new = np.stack([oracle.muon_update(P_ref[k], O_ref[k], wl.lr, wl.weight_decay)
                              for k in range(len(idx))])
            M_got = M[idx].cpu().numpy()
            for k in range(len(idx)):
                assert rel_fro(M_got[k], M_new[k]) <= MOMENTUM_TOL
                if need_ns:
                    assert_ns_close(bits_to_f64(torch_bf16_to_bits(O[idx[k]])), O_ref[k],
                                    label=f"{grp.name}[{idx[k]}] step {t}")
            lr_eff = float(np.float32(wl.lr)) * oracle.aspect_factor(grp.rows, grp.cols)
            bound += NS_REL_TOL * lr_eff * np.linalg.norm(O_ref) + 4 * 2.0 ** -24 * np.linalg.norm(P_new)
            ep = np.linalg.norm(P[idx].cpu().numpy() - P_new)
            assert ep <= bound, (t, ep, bound)
            P_ref, M_ref = P_new, M_new
            del G
