"""muon_merge_small_dims (host code of the C library) against the shape oracle,
exactly, on every shape of up to 5 extents from a small alphabet, plus large
extents (no overflow) and argument validation.  Needs the built library, no GPU."""
import ctypes
import math
import os

import pytest

import newton_schulz_muon_amd as nsm
from oracle.shape_oracle import merge_small_dims
from test_oracle_shape import THRESHOLDS, all_shapes, golden_cases


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nsm.LIB_PATH):
        pytest.fail("libmuon_hip.so is not built: run `python -m newton_schulz_muon_amd.build`")
    return nsm.load_library()


def test_matches_oracle_exhaustive(lib):
    n = 0
    for shape in all_shapes():
        for thr in THRESHOLDS:
            for tgt in (1, 2, 3, math.inf):
                got = nsm.muon_merge_small_dims(shape, thr, 0 if tgt == math.inf else tgt)
                assert got == merge_small_dims(shape, thr, tgt), (shape, thr, tgt)
                n += 1
    assert n > 100_000


@pytest.mark.parametrize("case", golden_cases())
def test_page_examples(lib, case):
    shape, thr, tgt, merged = case
    assert nsm.muon_merge_small_dims(shape, thr, tgt) == merged


def test_large_extents_and_ranks(lib):
    big = 1 << 40
    for shape, thr, tgt in [((big, big), (1 << 62), 1), ((big, 3, big), (1 << 63) - 1, 1),
                            ((2,) * 16, 1 << 20, 2), ((3,) * 16, 10, 4), ((1,) * 16, 5, 1)]:
        assert nsm.muon_merge_small_dims(shape, thr, tgt) == merge_small_dims(shape, thr, tgt)


def test_validation(lib):
    out = (ctypes.c_int64 * 16)()
    nd = ctypes.c_int32()
    shp = (ctypes.c_int64 * 17)(*([2] * 17))
    assert lib.muon_merge_small_dims(shp, 17, 10, 2, out, ctypes.byref(nd)) == 2      # too many dims
    assert lib.muon_merge_small_dims(shp, -1, 10, 2, out, ctypes.byref(nd)) == 2
    assert lib.muon_merge_small_dims(shp, 2, 0, 2, out, ctypes.byref(nd)) == 1        # threshold
    assert lib.muon_merge_small_dims(shp, 2, 10, -1, out, ctypes.byref(nd)) == 1      # target
    assert lib.muon_merge_small_dims(None, 2, 10, 2, out, ctypes.byref(nd)) == 1
    assert lib.muon_merge_small_dims(shp, 2, 10, 2, None, ctypes.byref(nd)) == 1
    neg = (ctypes.c_int64 * 2)(3, -4)
    assert lib.muon_merge_small_dims(neg, 2, 10, 2, out, ctypes.byref(nd)) == 2
    assert "negative" in nsm.muon_last_error()
    assert lib.muon_merge_small_dims(None, 0, 10, 2, out, ctypes.byref(nd)) == 0 and nd.value == 1
