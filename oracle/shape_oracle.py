"""Oracle of the shape merging that turns a >2-D parameter into the 2-D matrix
Muon orthogonalises (plain Python, integer arithmetic).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the test suite calls it.  It shares no code with the C library.

Source: [SH] the guide to the utils module of distributed_shampoo in
modded-nanogpt's optimization track, section "tensor math utilities:
dimension merging, blocking and distributed allocation" (merge_small_dims):
  * a 0-D shape is treated as 1-D: () -> (1,);
  * a shape with a zero extent is empty: -> (0,);
  * extents equal to 1 are squeezed out first; if every extent is 1 the
    result is (1,);
  * adjacent extents are merged while their product stays within the
    threshold, walking from the last extent towards the first (row-major
    layout keeps merged extents contiguous, so the result is a view);
  * merging stops as soon as the shape has the target number of extents,
    even where the threshold would allow more;
  * a target of infinity leaves the squeezed shape unmerged.

Readings (each also listed in the design doc):
  S1  The walk keeps a current (last-formed) extent: the next extent to the
      left is folded into it when the product is within the threshold and
      the shape still has more extents than the target; otherwise it starts
      a new extent.  This reproduces the page's (1, 2, 5, 1) -> (10,) with
      threshold 10, target 1, and (32, 3, 64, 64) -> (96, 4096) with
      threshold 8192, target 2.  The page prints the same (96, 4096) for
      threshold 1024 as well, which no threshold-bounded merge can give
      (4096 > 1024); that printout is taken to be an error on the page.
  S2  An extent larger than the threshold is never split; it stays as it is.

Pinned by the page's printed examples (tests/golden/merge_small_dims.txt)
and by invariants checked over every shape up to 5 extents of a small
alphabet (tests/test_oracle_shape.py); not parity unpinned.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple, Union


def merge_small_dims(shape: Sequence[int], threshold: int,
                     target: Union[int, float] = 2) -> Tuple[int, ...]:
    """[SH] merged shape of a contiguous tensor of `shape`."""
    if isinstance(target, float):
        if target != math.inf:
            raise ValueError("a float target must be math.inf")
    elif target < 1:
        raise ValueError("target must be >= 1")
    shape = tuple(int(s) for s in shape)
    if any(s < 0 for s in shape):
        raise ValueError("extents must be >= 0")
    if len(shape) == 0:
        return (1,)
    if any(s == 0 for s in shape):
        return (0,)
    squeezed = [s for s in shape if s != 1]
    if not squeezed:
        return (1,)
    if target == math.inf:
        return tuple(squeezed)
    # walk from the last extent to the first; `done` holds the merged extents
    # to the right (in reverse), `cur` the extent being formed
    cur = squeezed[-1]
    done = []
    for i in range(len(squeezed) - 2, -1, -1):
        nxt = squeezed[i]
        count = (i + 1) + 1 + len(done)     # extents of the shape as it stands
        if count > target and nxt * cur <= threshold:
            cur = nxt * cur
        else:
            done.append(cur)
            cur = nxt
    done.append(cur)
    return tuple(reversed(done))
