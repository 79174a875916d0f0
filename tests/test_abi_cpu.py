"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/muon_hip.h declares, and rejects bad arguments before it
touches the device."""
import ctypes
import os
import re

import pytest

import newton_schulz_muon_amd as nsm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_hip.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nsm.LIB_PATH):
        pytest.fail("libmuon_hip.so is not built: run `python -m newton_schulz_muon_amd.build`")
    return nsm.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert "muon_step_batched" in names and "ns_orthogonalize_batched" in names
    assert set(names) == set(nsm.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_matches_header(lib):
    ver = int(re.search(r"#define MUON_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert nsm.muon_abi_version() == ver


def test_default_config(lib):
    cfg = nsm.muon_ns_config_default()
    assert cfg.ns_steps == 5
    assert (cfg.a, cfg.b, cfg.c) == pytest.approx((3.4445, -4.7750, 2.0315), abs=1e-6)
    assert cfg.eps == pytest.approx(1e-7)
    assert cfg.precision == 0


def _up(x, a):
    return (x + a - 1) // a * a


def _regions(nb, m, n, split=False):
    """Bytes of one block batch's plan regions (no header, no loop queue)."""
    mp, np_ = _up(m, 128), _up(n, 128)
    xb = _up(nb * mp * np_ * 2, 256)
    ab = _up(nb * mp * mp * 2, 256)
    tiles = (mp // 64) * (np_ // 64)
    trace = _up(mp // 32, 32)          # floats per block: a 128-byte multiple
    # iterate ping-pong (and lo planes when split); A; B (+ lo); sums of squares; scales;
    # trace partials of the norm; counters of the persistent NS loop (9 + one per block,
    # each on a 128-byte line)
    return ((4 if split else 2) * xb + (3 if split else 2) * ab + _up(nb * tiles * 4, 256) + _up(nb * 8, 256)
            + _up(nb * trace * 4, 256) + _up((9 + nb) * 128, 256))


def _queue_entries(nb, m, n, steps=5, split=False):
    """Entries of the persistent loop's queue region (one per 256-wide tile at most)."""
    mp, np_ = _up(m, 128), _up(n, 128)
    if split or mp % 256 or np_ % 256:
        return 0
    t, tn = mp // 256, np_ // 256
    return nb * steps * (t * (t + 1) + t * tn)


def _expected_ws(nb, m, n, split=False, steps=5):
    # a 256-byte status header, the plan regions, the loop queue (8 bytes per entry)
    return 256 + _regions(nb, m, n, split) + _up(8 * _queue_entries(nb, m, n, steps, split), 256)


def test_workspace_bytes(lib):
    assert nsm.muon_workspace_bytes(0, 768, 3072) == 0
    assert nsm.muon_workspace_bytes(32, 768, 3072) == _expected_ws(32, 768, 3072)
    # attn view: 10 stored 768x3072 -> 40 blocks of 768x768
    assert nsm.muon_workspace_bytes(10, 768, 3072, 4) == _expected_ws(40, 768, 768)
    # tall blocks are stored oriented: 4096x1024 -> 1024x4096
    assert nsm.muon_workspace_bytes(3, 4096, 1024) == _expected_ws(3, 1024, 4096)
    # ragged shapes pad to 128
    assert nsm.muon_workspace_bytes(2, 300, 700) == _expected_ws(2, 300, 700)
    acc = nsm.make_config(precision="accurate")
    assert nsm.muon_workspace_bytes(2, 300, 700, 1, acc) == _expected_ws(2, 300, 700, split=True)
    # small blocks need no workspace
    assert nsm.muon_workspace_bytes(11, 1, 12) == 0


@pytest.mark.parametrize("shape", [(1, 0, 5), (1, 5, 0), (1, 8, 10, 4), (-1, 4, 4), (1, 8, 8, 0)])
def test_workspace_bytes_rejects_bad_shapes(lib, shape):
    b, r, c, *v = shape
    with pytest.raises(nsm.MuonError) as e:
        nsm.muon_workspace_bytes(b, r, c, v[0] if v else 1)
    assert e.value.status == 2
    assert nsm.muon_last_error()


def _cfg(**kw):
    cfg = nsm.muon_ns_config_default()
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


def test_ns_validation_before_device(lib):
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails validation
    # batch 0 is a no-op even with null pointers
    assert lib.ns_orthogonalize_batched(None, None, 0, 4, 4, 1, None, None, 0, None) == 0
    assert lib.ns_orthogonalize_batched(None, fake, 2, 128, 128, 1, None, None, 0, None) == 1
    assert "non-null" in nsm.muon_last_error()
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 0, 1, None, None, 0, None) == 2
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 66, 4, None, None, 0, None) == 2
    assert lib.ns_orthogonalize_batched(ctypes.c_void_p((1 << 20) + 2), fake, 2, 128, 128, 1,
                                        None, None, 0, None) == 3
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 128, 1, ctypes.byref(_cfg(ns_steps=-1)),
                                        None, 0, None) == 1
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 128, 1, ctypes.byref(_cfg(precision=7)),
                                        None, 0, None) == 1
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 128, 1, ctypes.byref(_cfg(eps=-1.0)),
                                        None, 0, None) == 1
    # workspace missing or too small
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 128, 1, None, None, 0, None) == 4
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 128, 1, None, fake, 100, None) == 4
    need = nsm.muon_workspace_bytes(2, 128, 128)
    assert lib.ns_orthogonalize_batched(fake, fake, 2, 128, 128, 1, None,
                                        ctypes.c_void_p((1 << 20) + 16), need, None) == 3
    # partial overlap of out and x
    assert lib.ns_orthogonalize_batched(fake, ctypes.c_void_p((1 << 20) + 16), 2, 128, 128, 1, None,
                                        fake, need, None) == 1


def test_step_validation_before_device(lib):
    fake = ctypes.c_void_p(1 << 20)
    other = ctypes.c_void_p(1 << 32)
    third = ctypes.c_void_p(1 << 34)
    f = ctypes.c_float
    args = dict(lr=0.02, wd=0.01, mu=0.95)

    def call(p, g, m, b=2, r=128, c=128, v=1, lr=0.02, wd=0.01, mu=0.95, out=None, ws=None, wsb=0):
        return lib.muon_step_batched(p, g, m, b, r, c, v, f(lr), f(wd), f(mu), 1, f(1.0), f(1.0),
                                     None, out, ws, wsb, None)
    assert call(None, None, None, b=0) == 0
    assert call(None, other, third) == 1
    assert call(fake, other, third, mu=1.5) == 1
    assert call(fake, other, third, lr=float("nan")) == 1
    assert call(fake, other, third, wd=float("inf")) == 1
    assert call(fake, fake, third) == 1        # params and grads overlap
    assert call(fake, other, third, out=other) == 1
    assert call(fake, other, third, c=0) == 2
    assert call(fake, other, third) == 4       # no workspace
    del args


def _mat(p, g, m, rows, cols, v=1, out=None, lr_mul=1.0, wd_mul=1.0):
    e = nsm.MuonMatrix()
    e.params, e.grads, e.momentum_buf, e.update_out = p, g, m, out
    e.rows, e.cols, e.view_blocks, e.lr_mul, e.wd_mul = rows, cols, v, lr_mul, wd_mul
    return e


def _mats(*entries):
    arr = (nsm.MuonMatrix * len(entries))()
    for i, e in enumerate(entries):
        arr[i] = e
    return arr


def test_multi_workspace_bytes(lib):
    base = 1 << 30
    # 3 mlp-like, 2 attn (view 4), 1 gate: groups by (rows, cols, view)
    es = [_mat(base + i * (1 << 26), base + i * (1 << 26) + (1 << 24), base + i * (1 << 26) + (1 << 25), 768, 3072)
          for i in range(3)]
    es += [_mat(base + (3 + i) * (1 << 26), base + (3 + i) * (1 << 26) + (1 << 24),
                base + (3 + i) * (1 << 26) + (1 << 25), 768, 3072, 4) for i in range(2)]
    es += [_mat(base + 6 * (1 << 26), base + 6 * (1 << 26) + 4096, base + 6 * (1 << 26) + 8192, 1, 12)]
    arr = _mats(*es)
    got = lib.muon_step_multi_workspace_bytes(arr, len(es), None)
    # one wave (equal padded side): header, both groups' regions, one queue for both
    q = _queue_entries(3, 768, 3072) + _queue_entries(8, 768, 768)
    assert got == 256 + _regions(3, 768, 3072) + _regions(8, 768, 768) + _up(8 * q, 256)
    assert lib.muon_step_multi_workspace_bytes(arr, 0, None) == 0
    bad = _mats(_mat(base, base + 4096, base + 8192, 8, 10, 4))
    assert lib.muon_step_multi_workspace_bytes(bad, 1, None) == ctypes.c_size_t(-1).value


def test_multi_validation_before_device(lib):
    f = ctypes.c_float
    base = 1 << 30

    def call(arr, n, lr=0.02, ws=None, wsb=0):
        return lib.muon_step_multi(arr, n, f(lr), f(0.01), f(0.95), 1, None, ws, wsb, None)
    good = _mats(_mat(base, base + (1 << 20), base + (1 << 21), 128, 128),
                 _mat(base + (1 << 22), base + (1 << 22) + (1 << 20), base + (1 << 22) + (1 << 21), 128, 128))
    assert call(None, 0) == 0
    assert call(None, 2) == 1                                  # null array
    assert call(good, 2, lr=float("nan")) == 1
    assert call(good, 2) == 4                                  # no workspace
    # the second matrix's params overlap the first one's momentum buffer
    ov = _mats(_mat(base, base + (1 << 20), base + (1 << 21), 128, 128),
               _mat(base + (1 << 21) + 64, base + (1 << 23), base + (1 << 24), 128, 128))
    assert call(ov, 2) == 1
    assert "overlap" in nsm.muon_last_error()
    mis = _mats(_mat(base + 4, base + (1 << 20), base + (1 << 21), 128, 128))
    assert call(mis, 1) == 3
    inf = _mats(_mat(base, base + (1 << 20), base + (1 << 21), 128, 128, lr_mul=float("inf")))
    assert call(inf, 1) == 1
    shp = _mats(_mat(base, base + (1 << 20), base + (1 << 21), 0, 128))
    assert call(shp, 1) == 2
    nul = _mats(_mat(None, base + (1 << 20), base + (1 << 21), 128, 128))
    assert call(nul, 1) == 1


def test_multi_alignment_by_path(lib):
    # A 1x12 gate takes the element-wise small path: 8-byte offsets are fine
    # (they are what slices of a stacked [n, 1, 12] batch give).  The call
    # still fails, on the overlap planted in the second and third matrices,
    # before any device work.
    f = ctypes.c_float
    base = 1 << 30
    arr = _mats(_mat(base + 48, base + 4096 + 24, base + 8192 + 48, 1, 12),
                _mat(base + (1 << 20), base + (1 << 21), base + (1 << 22), 128, 128),
                _mat(base + (1 << 20) + 64, base + (1 << 23), base + (1 << 24), 128, 128))
    assert lib.muon_step_multi(arr, 3, f(0.02), f(0.01), f(0.95), 1, None, None, 0, None) == 1
    assert "overlap" in nsm.muon_last_error()
    # the same offset on a vector-path matrix is rejected
    arr = _mats(_mat(base + (1 << 20) + 8, base + (1 << 21), base + (1 << 22), 128, 128))
    assert lib.muon_step_multi(arr, 1, f(0.02), f(0.01), f(0.95), 1, None, None, 0, None) == 3


def _adam(p, g, m, v, numel, step=1, lr_mul=1.0, wd_mul=1.0):
    e = nsm.MuonAdamTensor()
    e.params, e.grads, e.exp_avg, e.exp_avg_sq = p, g, m, v
    e.numel, e.step, e.lr_mul, e.wd_mul = numel, step, lr_mul, wd_mul
    return e


def _adams(*entries):
    arr = (nsm.MuonAdamTensor * len(entries))()
    for i, e in enumerate(entries):
        arr[i] = e
    return arr


def test_adamw_validation_before_device(lib):
    f = ctypes.c_float
    base = 1 << 30
    mb = 1 << 20

    def call(arr, n, lr=0.008, b1=0.8, b2=0.95, eps=1e-8, wd=0.0):
        return lib.adamw_step_multi(arr, n, f(lr), f(b1), f(b2), f(eps), f(wd), None)
    good = _adams(_adam(base, base + mb, base + 2 * mb, base + 3 * mb, 1000),
                  _adam(base + 4 * mb, base + 5 * mb, base + 6 * mb, base + 7 * mb, 768, step=3))
    assert call(None, 0) == 0
    assert call(None, 2) == 1                                   # null array
    assert call(good, -1) == 2
    assert call(good, 2, lr=float("nan")) == 1
    assert call(good, 2, wd=float("inf")) == 1
    assert call(good, 2, eps=-1.0) == 1
    assert call(good, 2, b1=1.0) == 1
    assert call(good, 2, b2=-0.1) == 1
    # tensors with numel 0 are skipped (null pointers allowed): nothing to do, no device work
    assert call(_adams(_adam(None, None, None, None, 0), _adam(None, None, None, None, 0)), 2) == 0
    assert call(_adams(_adam(base, base + mb, base + 2 * mb, base + 3 * mb, -5)), 1) == 2
    assert call(_adams(_adam(None, base + mb, base + 2 * mb, base + 3 * mb, 10)), 1) == 1
    assert call(_adams(_adam(base, base + mb, base + 2 * mb, base + 3 * mb, 10, step=0)), 1) == 1
    assert call(_adams(_adam(base, base + mb, base + 2 * mb, base + 3 * mb, 10, lr_mul=float("nan"))), 1) == 1
    assert call(_adams(_adam(base + 2, base + mb, base + 2 * mb, base + 3 * mb, 10)), 1) == 3
    assert call(_adams(_adam(base, base + mb + 1, base + 2 * mb, base + 3 * mb, 10)), 1) == 3
    # exp_avg of the second tensor overlaps params of the first
    ov = _adams(_adam(base, base + mb, base + 2 * mb, base + 3 * mb, 1000),
                _adam(base + 4 * mb, base + 5 * mb, base + 400, base + 7 * mb, 10))
    assert call(ov, 2) == 1
    assert "overlap" in nsm.muon_last_error()
    # params and grads of one tensor overlap
    assert call(_adams(_adam(base, base + 1000, base + 2 * mb, base + 3 * mb, 1000)), 1) == 1


def test_workspace_must_not_overlap_data(lib):
    # Valid calls in every other respect; each fails on the overlap before any device work.
    f = ctypes.c_float
    base = 1 << 32
    need = nsm.muon_workspace_bytes(2, 128, 128)
    n = 2 * 128 * 128
    P, G, M = base, base + 8 * n, base + 16 * n
    ws = base + 24 * n
    # workspace starting inside momentum_buf
    assert lib.muon_step_batched(P, G, M, 2, 128, 128, 1, f(0.02), f(0.01), f(0.95), 1, f(1.0), f(1.0),
                                 None, None, ctypes.c_void_p(M + 256), need, None) == 1
    assert "workspace" in nsm.muon_last_error()
    # ns: workspace covering x
    assert lib.ns_orthogonalize_batched(ctypes.c_void_p(G), ctypes.c_void_p(ws), 2, 128, 128, 1, None,
                                        ctypes.c_void_p(G - 256), need, None) == 1
    # multi: workspace overlapping the second matrix's grads
    arr = _mats(_mat(base, base + (1 << 20), base + (1 << 21), 128, 128),
                _mat(base + (1 << 22), base + (1 << 23), base + (1 << 24), 128, 128))
    wsb = lib.muon_step_multi_workspace_bytes(arr, 2, None)
    assert lib.muon_step_multi(arr, 2, f(0.02), f(0.01), f(0.95), 1, None, ctypes.c_void_p(base + (1 << 23) - 256),
                               wsb, None) == 1
    assert "workspace overlaps" in nsm.muon_last_error()


def test_ns_schedule_modes(lib):
    # Host-only: the process-wide schedule switch takes modes 0, 1, 2 and
    # rejects others; the binding maps names to them.
    for mode in (1, 2, 0):
        assert lib.muon_set_ns_schedule(mode) == 0
    assert lib.muon_set_ns_schedule(3) == 1
    assert "schedule mode" in nsm.muon_last_error()
    assert lib.muon_set_ns_schedule(-1) == 1
    for name in ("per_product", "persistent", "auto"):
        nsm.muon_set_ns_schedule(name)
    with pytest.raises(ValueError):
        nsm.muon_set_ns_schedule("fast")


def test_gemm_tiling_widths(lib):
    # Host-only: the process-wide tile width takes 0, 64, 128, 256
    for w in (64, 128, 256, 0):
        assert lib.muon_set_gemm_tiling(w) == 0
    for bad in (-1, 1, 32, 96, 512):
        assert lib.muon_set_gemm_tiling(bad) == 1
        assert "tile width" in nsm.muon_last_error()
        with pytest.raises(ValueError):
            nsm.muon_set_gemm_tiling(bad)
    nsm.muon_set_gemm_tiling(0)


def test_workspace_status_validation(lib):
    # host-side checks only (no copy is enqueued)
    assert lib.muon_workspace_status(None, ctypes.c_void_p(1 << 30), None) == 1
    assert lib.muon_workspace_status(ctypes.c_void_p(1 << 30), None, None) == 1
    assert lib.muon_workspace_status(ctypes.c_void_p((1 << 30) + 16), ctypes.c_void_p(1 << 30), None) == 3
    assert lib.muon_workspace_status(ctypes.c_void_p(1 << 30), ctypes.c_void_p((1 << 30) + 2), None) == 3


def test_loop_fault_modes(lib):
    for mode in (1, 2, 0):
        assert lib.muon_debug_set_loop_fault(mode) == 0
    assert lib.muon_debug_set_loop_fault(3) == 1
    assert lib.muon_debug_set_loop_fault(-1) == 1
    assert "loop fault mode" in nsm.muon_last_error()
