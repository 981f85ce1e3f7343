"""Static check of the generated gfx950 code: no LDS read is in flight at a workgroup barrier.

Several kernels refill an LDS buffer with direct-to-LDS loads right after the barrier that ends
its use. A fragment read that one wave still has in flight at that barrier could then return
data another wave's refill has already overwritten. The compiler may move MFMAs, and with them
the waits for their operands, past `s_barrier`, so the kernels wait for their own reads
explicitly before such barriers. This test compiles every source to gfx950 assembly (device
code only, the library's own flags) and checks, for every kernel, that along every path to every
`s_barrier` each `ds_read` issued has been covered by an `lgkmcnt` wait. LDS operations of one
wave complete in order, so after `s_waitcnt lgkmcnt(N)` at most N of them are outstanding.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from mamba_selective_scan_mixer_amd import build as B

CAP = 64   # outstanding-read counts are capped so the fixed point below terminates


def _device_asm(src: str, out: str) -> str:
    flags = [f for f in B.CFLAGS if f != "-fPIC"]
    cmd = [B.HIPCC, *flags, "--offload-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    return open(out).read()


def _functions(asm: str):
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end].split("\n")


def _blocks(lines):
    """Basic blocks: (label, instructions, successor labels)."""
    blocks, cur_label, cur = [], "<entry>", []
    for ln in lines:
        lab = re.match(r"^(\.LBB\w+):", ln)
        if lab:
            blocks.append([cur_label, cur])
            cur_label, cur = lab.group(1), []
            continue
        t = ln.split(";")[0].strip()
        if t and not t.startswith("."):
            cur.append(t)
    blocks.append([cur_label, cur])
    out = []
    for i, (label, ins) in enumerate(blocks):
        succ, falls = [], True
        for t in ins:
            op = t.split()[0]
            m = re.match(r"s_c?branch\w*\s+(\.LBB\w+)", t)
            if m:
                succ.append(m.group(1))
            if op in ("s_branch", "s_endpgm", "s_setpc_b64"):
                falls = False
        if falls and i + 1 < len(blocks):
            succ.append(blocks[i + 1][0])
        out.append((label, ins, succ))
    return out


def _step(pending: int, t: str, on_barrier=None) -> int:
    op = t.split()[0]
    if op.startswith("ds_read") or op.startswith("ds_load"):
        return min(pending + 1, CAP)
    if op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", t)
        if m:
            return min(pending, int(m.group(1)))
        return pending
    if op == "s_barrier" and on_barrier is not None:
        on_barrier(pending)
    return pending


def _barrier_violations(lines):
    blocks = _blocks(lines)
    index = {b[0]: i for i, b in enumerate(blocks)}
    entry = [0] * len(blocks)           # max outstanding reads on entry, over all paths
    changed = True
    while changed:
        changed = False
        for i, (_, ins, succ) in enumerate(blocks):
            p = entry[i]
            for t in ins:
                p = _step(p, t)
            for s in succ:
                j = index.get(s)
                if j is not None and p > entry[j]:
                    entry[j] = p
                    changed = True
    bad = []
    for i, (label, ins, _) in enumerate(blocks):
        p = entry[i]
        for t in ins:
            p = _step(p, t, on_barrier=lambda n, label=label: n and bad.append((label, n)))
    return bad


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                    reason="hipcc not available")
def test_no_lds_read_in_flight_at_any_barrier(tmp_path):
    srcs = B.sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        asms = list(ex.map(lambda s: _device_asm(s, str(tmp_path / (os.path.basename(s) + ".s"))), srcs))
    checked, problems = 0, []
    for src, asm in zip(srcs, asms):
        for name, lines in _functions(asm):
            if not any("s_barrier" in ln for ln in lines):
                continue
            checked += 1
            for label, n in _barrier_violations(lines):
                problems.append(f"{os.path.basename(src)} {name} block {label}: {n} LDS read(s) in flight")
    assert checked >= 10, checked      # the GEMM, decode, scan, conv, norm and backward kernels
    assert not problems, "\n".join(problems)


def test_checker_flags_a_read_left_in_flight():
    """The analysis itself: a read waited for only after the barrier is reported, also when it
    reaches the barrier around a loop back edge; one waited for before it is not."""
    bad = ["ds_read_b128 v[0:3], v4", "s_barrier", "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    good = ["ds_read_b128 v[0:3], v4", "s_waitcnt lgkmcnt(0)", "s_barrier", "s_endpgm"]
    loop = [".LBB0_1:", "s_waitcnt vmcnt(0)", "s_barrier", "ds_read_b128 v[0:3], v4",
            "v_mfma_f32_32x32x16_bf16 v[0:15], v[0:3], v[0:3], v[0:15]",
            "s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    partial = ["ds_read_b128 v[0:3], v4", "ds_read_b128 v[4:7], v4", "s_waitcnt lgkmcnt(1)",
               "s_barrier", "s_endpgm"]
    assert _barrier_violations(bad)
    assert not _barrier_violations(good)
    assert _barrier_violations(loop)
    assert _barrier_violations(partial)
