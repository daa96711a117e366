"""Host-side check of the emitted gfx950 code: no workgroup barrier is reached while this wave's
own LDS stores may still be in flight.

The copy loops of the prefill kernels end an iteration with LDS stores (list slots, row
statistics) that other waves read after the next iteration's barrier.  The barrier only orders
them if the wave has waited for its LDS counter (lgkmcnt) first.  That wait was once missing at
a loop header reached over the back edge, and the backward then gave different bits from call
to call.  This test compiles the kernels to assembly (no GPU needed) and walks every kernel, in
program order and over each backward branch, from every LDS store to the next barrier."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from top_chunk_sparse_amd import build as B

SOURCES = ["prefill.hip", "prefill_bwd.hip", "gist_prefill.hip"]


def _asm(src, outdir):
    out = os.path.join(outdir, src + ".s")
    cmd = [B.HIPCC] + B.COMMON + ["--cuda-device-only", "-S", "-x", "hip",
                                  os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _kernels(text):
    ks, name = {}, None
    for raw in text.split("\n"):
        m = re.match(r"^(_Z\w+):", raw)
        if m:
            name = m.group(1)
            ks[name] = []
        elif name is not None:
            ks[name].append(raw.strip())
            if raw.strip().startswith("s_endpgm"):
                name = None
    return ks


def _step(line, pending):
    """LDS-store state after one instruction: set by a ds_write, cleared by lgkmcnt(0)."""
    if line.startswith("ds_write"):
        return True
    if line.startswith("s_waitcnt") and "lgkmcnt(0)" in line:
        return False
    return pending


def _unwaited_barriers(lines):
    labels = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):", l)
        if m:
            labels[m.group(1)] = i
    bad = []
    pending = False
    for i, l in enumerate(lines):
        pending = _step(l, pending)
        if l.startswith("s_barrier") and pending:
            bad.append(("in order", i))
        m = re.match(r"^s_c?branch\w*\s+(\.LBB\w+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i and pending:
            # over the back edge: from the loop header to its first barrier
            p = pending
            for j in range(labels[m.group(1)], i):
                p = _step(lines[j], p)
                if lines[j].startswith("s_barrier"):
                    if p:
                        bad.append(("back edge", j))
                    break
    return bad


@pytest.mark.skipif(not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC),
                    reason="hipcc not installed")
def test_no_barrier_with_lds_stores_in_flight(tmp_path):
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _asm(s, str(tmp_path)), SOURCES))
    found = {}
    for src, text in zip(SOURCES, texts):
        ks = _kernels(text)
        assert ks, src
        for name, lines in ks.items():
            bad = _unwaited_barriers(lines)
            if bad:
                found[f"{src}:{name}"] = bad
    assert not found, found


def test_scanner_sees_a_missing_wait():
    """The scanner itself: a loop whose stores reach the header's barrier unwaited is caught,
    and the same loop with lgkmcnt(0) before the branch is not."""
    loop = [".LBB0_1:", "s_waitcnt vmcnt(0)", "s_barrier", "ds_read_b128 v[0:3], v4",
            "s_waitcnt lgkmcnt(0)", "ds_write_b32 v5, v6", "s_cbranch_scc1 .LBB0_1",
            "s_endpgm"]
    assert _unwaited_barriers(loop) == [("back edge", 2)]
    fixed = loop[:6] + ["s_waitcnt lgkmcnt(0)"] + loop[6:]
    assert _unwaited_barriers(fixed) == []
    straight = ["ds_write_b32 v5, v6", "s_barrier"]
    assert _unwaited_barriers(straight) == [("in order", 1)]
