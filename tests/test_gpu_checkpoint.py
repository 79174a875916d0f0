"""Checkpoint / resume of the Muon step.  The optimizer's only state is the
momentum buffer, a caller-owned tensor (the pages' optimizer saves it with
its state dict and restores it in place).  Running k steps, saving params
and momentum to a torch checkpoint, reloading them into fresh device
allocations (a new workspace too) and running the remaining steps must give
bitwise the same params, momentum and last update as the uninterrupted run:
the step reads nothing but its arguments and keeps no device state between
calls.  Cases: muon_step_multi on a mixed set (wide, tall, attn view,
per-matrix multipliers, a small gate on the fp32 small-block path) and
muon_step_batched in ACCURATE precision."""
import io

import pytest

pytestmark = pytest.mark.gpu

STEPS, SPLIT = 6, 3
HYPER = dict(lr=0.05, weight_decay=0.01)


@pytest.fixture(scope="module")
def nsm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests must run on an MI355X")
    import newton_schulz_muon_amd as m
    m.load_library()
    return m


def _grads(shapes, steps, seed):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return [[(torch.randn((r, c), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
             for (r, c, *_rest) in shapes] for _ in range(steps)]


def _save_load(tensors):
    """Round trip through a torch checkpoint on the host (weights only)."""
    import torch
    buf = io.BytesIO()
    torch.save([t.cpu() for t in tensors], buf)
    buf.seek(0)
    return [t.cuda() for t in torch.load(buf, weights_only=True)]


def _momentum(t):
    return 0.85 + 0.1 * min(t / 4, 1.0)    # a warm-up schedule, so the step index matters


def test_resume_multi_is_bitwise(nsm):
    import torch
    shapes = [(768, 3072, 1, 1.0, 1.0), (3072, 768, 1, 1.0, 0.5), (768, 3072, 4, 0.5, 1.0),
              (512, 512, 1, 2.0, 0.0), (1, 12, 1, 1.0, 1.0)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    P0 = [torch.randn((r, c), generator=gen, device="cuda") / c ** 0.5 for (r, c, *_r) in shapes]
    grads = _grads(shapes, STEPS, 12)

    def run(P, M, t0, t1):
        outs = [torch.empty((r, c), dtype=torch.bfloat16, device="cuda") for (r, c, *_r) in shapes]
        for t in range(t0, t1):
            mats = [dict(params=P[i], grads=grads[t][i], momentum_buf=M[i], update_out=outs[i],
                         view_blocks=v, lr_mul=lm, wd_mul=wm) for i, (_r, _c, v, lm, wm) in enumerate(shapes)]
            print(f"[resume multi] step {t}", flush=True)
            nsm.muon_step_multi(mats, momentum=_momentum(t), **HYPER)
        torch.cuda.synchronize()
        return outs

    Pa, Ma = [p.clone() for p in P0], [torch.zeros_like(p) for p in P0]
    Oa = run(Pa, Ma, 0, STEPS)

    Pb, Mb = [p.clone() for p in P0], [torch.zeros_like(p) for p in P0]
    run(Pb, Mb, 0, SPLIT)
    state = _save_load(Pb + Mb)
    del Pb, Mb
    torch.cuda.empty_cache()
    Pc, Mc = state[:len(shapes)], state[len(shapes):]
    Oc = run(Pc, Mc, SPLIT, STEPS)
    for i in range(len(shapes)):
        assert torch.equal(Pa[i], Pc[i]), f"params {shapes[i]}"
        assert torch.equal(Ma[i], Mc[i]), f"momentum {shapes[i]}"
        assert torch.equal(Oa[i], Oc[i]), f"update {shapes[i]}"


def test_resume_batched_accurate_is_bitwise(nsm):
    import torch
    B, R, C = 4, 1024, 2048
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    P0 = torch.randn((B, R, C), generator=gen, device="cuda") / C ** 0.5
    grads = [(torch.randn((B, R, C), generator=gen, device="cuda") * 1e-2).to(torch.bfloat16)
             for _ in range(STEPS)]

    def run(P, M, t0, t1):
        out = torch.empty((B, R, C), dtype=torch.bfloat16, device="cuda")
        for t in range(t0, t1):
            print(f"[resume batched accurate] step {t}", flush=True)
            nsm.muon_step_batched(P, grads[t], M, momentum=_momentum(t), precision="accurate",
                                  update_out=out, **HYPER)
        torch.cuda.synchronize()
        return out

    Pa, Ma = P0.clone(), torch.zeros_like(P0)
    Oa = run(Pa, Ma, 0, STEPS)
    Pb, Mb = P0.clone(), torch.zeros_like(P0)
    run(Pb, Mb, 0, SPLIT)
    Pc, Mc = _save_load([Pb, Mb])
    del Pb, Mb
    Oc = run(Pc, Mc, SPLIT, STEPS)
    assert torch.equal(Pa, Pc) and torch.equal(Ma, Mc) and torch.equal(Oa, Oc)
