"""Pins of the shape-merging oracle: the page's printed examples, invariants
over every shape of up to 5 extents from a small alphabet, and planted
mistakes the pins must reject.  No GPU."""
import itertools
import math
import os

import pytest

from oracle.shape_oracle import merge_small_dims

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "merge_small_dims.txt")
ALPHABET = (0, 1, 2, 3, 5, 64)
THRESHOLDS = (1, 6, 64, 1000, 1 << 40)
TARGETS = (1, 2, 3, math.inf)


def golden_cases():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        shape, thr, tgt, merged = (x.strip() for x in line.split("|"))
        out.append((tuple(int(v) for v in shape.split(",")), int(thr), int(tgt),
                    tuple(int(v) for v in merged.split(","))))
    return out


def all_shapes(max_len=5):
    for n in range(max_len + 1):
        yield from itertools.product(ALPHABET, repeat=n)


def check_invariants(fn, shape, thr, tgt):
    """Properties the page's description fixes, independent of how the walk is written."""
    r = fn(shape, thr, tgt)
    if len(shape) == 0:
        return r == (1,)
    if 0 in shape:
        return r == (0,)
    sq = [s for s in shape if s != 1]
    if not sq:
        return r == (1,)
    if tgt == math.inf:
        return r == tuple(sq)
    # r partitions the squeezed extents into contiguous runs, in order
    runs, i = [], 0
    for x in r:
        j, p = i, 1
        while j < len(sq) and p < x:
            p *= sq[j]
            j += 1
        if p != x or j == i:
            return False
        runs.append(sq[i:j])
        i = j
    if i != len(sq):
        return False
    # a merged run stays within the threshold; a single extent may exceed it
    if any(len(run) > 1 and x > thr for run, x in zip(runs, r)):
        return False
    # never below the target; no adjacent pair left mergeable while above it
    if len(r) < min(tgt, len(sq)):
        return False
    if len(r) > tgt and any(a * b <= thr for a, b in zip(r, r[1:])):
        return False
    return True


@pytest.mark.parametrize("case", golden_cases())
def test_page_examples(case):
    shape, thr, tgt, merged = case
    assert merge_small_dims(shape, thr, tgt) == merged


def test_invariants_exhaustive():
    n = 0
    for shape in all_shapes():
        for thr in THRESHOLDS:
            for tgt in TARGETS:
                assert check_invariants(merge_small_dims, shape, thr, tgt), (shape, thr, tgt)
                n += 1
    assert n > 100_000


def test_special_cases():
    assert merge_small_dims((), 10) == (1,)
    assert merge_small_dims((7,), 1) == (7,)
    assert merge_small_dims((4, 0, 5), 100) == (0,)
    assert merge_small_dims((1, 1, 1), 100, 1) == (1,)
    assert merge_small_dims((1, 768, 1), 100, 2) == (768,)
    # the walk runs from the last extent: (2, 3, 4) at threshold 12 merges 3*4 first
    assert merge_small_dims((2, 3, 4), 12, 1) == (2, 12)
    with pytest.raises(ValueError):
        merge_small_dims((2, 3), 10, 2.5)
    with pytest.raises(ValueError):
        merge_small_dims((2, -1), 10, 2)


def _left_to_right(shape, thr, tgt=2):
    sq = [s for s in shape if s != 1]
    if not shape:
        return (1,)
    if 0 in shape:
        return (0,)
    if not sq:
        return (1,)
    out = [sq[0]]
    for k, x in enumerate(sq[1:], start=1):
        if len(out) + (len(sq) - k) > tgt and out[-1] * x <= thr:
            out[-1] *= x
        else:
            out.append(x)
    return tuple(out)


def _no_early_stop(shape, thr, tgt=2):
    return merge_small_dims(shape, thr, 1)


def _no_squeeze(shape, thr, tgt=2):
    if not shape:
        return (1,)
    if 0 in shape:
        return (0,)
    cur, done = shape[-1], []
    for i in range(len(shape) - 2, -1, -1):
        if (i + 2 + len(done)) > tgt and shape[i] * cur <= thr:
            cur *= shape[i]
        else:
            done.append(cur)
            cur = shape[i]
    done.append(cur)
    return tuple(reversed(done))


@pytest.mark.parametrize("mutant", [_left_to_right, _no_early_stop, _no_squeeze])
def test_pins_reject_mutants(mutant):
    failed = any(mutant(s, t, g) != m for s, t, g, m in golden_cases())
    if not failed:
        failed = any(not check_invariants(mutant, s, t, g)
                     for s in all_shapes(4) for t in THRESHOLDS for g in (1, 2, 3))
    assert failed, f"{mutant.__name__} not detected"
