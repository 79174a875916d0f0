"""The library's ownership contract, checked on its sources (no GPU):

* no device memory is allocated or freed by the library (no hipMalloc /
  hipMallocAsync / hipFree / hipExtMallocWithFlags / hipMallocManaged),
* no call synchronises the host with the device (no hipMemcpy without Async,
  no hipDeviceSynchronize / hipStreamSynchronize), except the timing
  diagnostics' documented wait for their events,
* every kernel launch names the caller's stream: no launch on the null
  stream (`0, nullptr>>>`, `0, 0>>>`, or a launch without a stream argument),
* host memory the library keeps is pinned (hipHostMalloc) and never freed
  while a copy from it may be pending (no hipHostFree).
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_muon_amd", "csrc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".hpp")))


def _code(path):
    """Source text with comments and string literals removed."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r'"(?:\\.|[^"\\])*"', '""', text)


@pytest.mark.parametrize("src", SOURCES)
def test_no_device_allocation(src):
    code = _code(os.path.join(CSRC, src))
    for name in ("hipMalloc", "hipMallocAsync", "hipFree", "hipFreeAsync", "hipExtMallocWithFlags",
                 "hipMallocManaged", "hipHostFree", "hipHostRegister"):
        assert not re.search(r"\b%s\s*\(" % name, code), f"{src} calls {name}"


@pytest.mark.parametrize("src", SOURCES)
def test_no_synchronising_calls(src):
    code = _code(os.path.join(CSRC, src))
    assert not re.search(r"\bhipMemcpy\s*\(", code), f"{src} calls the synchronous hipMemcpy"
    assert not re.search(r"\bhipMemset\s*\(", code), f"{src} calls the synchronous hipMemset"
    assert not re.search(r"\bhipDeviceSynchronize\s*\(", code), f"{src} synchronises the device"
    assert not re.search(r"\bhipStreamSynchronize\s*\(", code), f"{src} synchronises a stream"
    # the one documented wait: muon_timing_collect waits for its own timing events
    waits = re.findall(r"\bhipEventSynchronize\s*\(", code)
    if waits:
        assert src == "muon_api.hip" and len(waits) == 1
        body = code[code.index("muon_status muon_timing_collect("):]
        assert "hipEventSynchronize" in body[:body.index("\n}\n")]


def _top_level_args(text):
    """Comma-separated arguments of a launch configuration, outside parentheses."""
    out, depth, cur = [], 0, ""
    for ch in text:
        if ch in "([{":
            depth += 1
        elif ch in ")]}":
            depth -= 1
        if ch == "," and depth == 0:
            out.append(cur.strip())
            cur = ""
        else:
            cur += ch
    out.append(cur.strip())
    return out


@pytest.mark.parametrize("src", SOURCES)
def test_every_launch_names_a_stream(src):
    code = _code(os.path.join(CSRC, src))
    for m in re.finditer(r"<<<(.*?)>>>", code, flags=re.S):
        args = _top_level_args(m.group(1))
        assert len(args) == 4, f"{src}: launch <<<{m.group(1)}>>> has no stream argument"
        assert args[3] not in ("0", "nullptr", "NULL", "hipStreamDefault"), \
            f"{src}: launch <<<{m.group(1)}>>> on the null stream"


def test_pinned_host_copy_only_for_queues():
    # the only host allocation: the persistent loop's queue cache (pinned, kept)
    hits = {src: len(re.findall(r"\bhipHostMalloc\s*\(", _code(os.path.join(CSRC, src)))) for src in SOURCES}
    assert {k: v for k, v in hits.items() if v} == {"ns_gemm.hip": 1}
