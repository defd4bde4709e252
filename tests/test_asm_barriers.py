"""Every workgroup barrier in the gfx950 kernels is reached with no LDS read of
the wave still in flight.

The kernels overwrite an LDS buffer (direct global->LDS copies) right after
the barrier that ends the last reads of it.  If a wave's read of that buffer
were still outstanding at the barrier, another wave's copy could land first.
``__syncthreads`` does not always make hipcc wait for outstanding LDS reads
(seen with reads issued at the end of a loop body and a barrier at the loop
head), so this checks the generated code: each kernel source is compiled to
gfx950 assembly and a dataflow pass over each function's control-flow graph
tracks the number of outstanding LDS reads (raised by ``ds_read*``, lowered by
``s_waitcnt lgkmcnt(n)``) at every ``s_barrier``.  CPU only: hipcc
cross-compiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_95_amd", "csrc")
KERNEL_SOURCES = ["fa_fwd16.hip", "fa_fwd8.hip", "fa_fwd32.hip", "fa_bwd16.hip"]
CAP = 64


def split_functions(text: str):
    """(name, body lines) of every function in an AMDGPU assembly listing."""
    funcs, cur = [], None
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", line)
        if m:
            cur = (m.group(1), [])
            funcs.append(cur)
            continue
        if cur is not None:
            cur[1].append(line)
            if line.strip().startswith("s_endpgm"):
                cur = None
    return funcs


def barrier_hazards(body):
    """Barriers (block label, index in block) that some path reaches with LDS
    reads outstanding."""
    blocks, labels = [["entry", []]], {}
    for line in body:
        t = line.strip()
        m = re.match(r"^(\.LBB\w+):", t)
        if m or t.startswith("; %bb."):
            lab = m.group(1) if m else t.split()[1].rstrip(":")
            blocks.append([lab, []])
            labels[lab] = len(blocks) - 1
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        blocks[-1][1].append(t)
        if re.match(r"s_c?branch", t):  # a branch always ends its block
            blocks.append(["after_%d" % len(blocks), []])
    succ = []
    for i, (_, ins) in enumerate(blocks):
        s, last = [], ins[-1] if ins else ""
        m = re.match(r"s_(c?branch\w*)\s+(\.LBB\w+)", last)
        if m:
            if m.group(2) in labels:
                s.append(labels[m.group(2)])
            if m.group(1) != "branch" and i + 1 < len(blocks):
                s.append(i + 1)
        elif not (last.startswith("s_endpgm") or last.startswith("s_setpc")) and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    def walk(i, hazards=None):
        p = entry[i]
        for j, t in enumerate(blocks[i][1]):
            if t.startswith("ds_read") or t.startswith("ds_load"):
                p = min(CAP, p + 1)
            elif t.startswith("s_waitcnt"):
                m = re.search(r"lgkmcnt\((\d+)\)", t)
                if m:
                    p = min(p, int(m.group(1)))
            elif t.startswith("s_barrier") and p > 0 and hazards is not None:
                hazards.add((blocks[i][0], j))
        return p

    # outstanding reads at each block's entry: the maximum over its predecessors
    entry = [0] * len(blocks)
    changed = True
    while changed:
        changed = False
        for i in range(len(blocks)):
            p = walk(i)
            for k in succ[i]:
                if p > entry[k]:
                    entry[k] = p
                    changed = True
    hazards = set()
    for i in range(len(blocks)):
        walk(i, hazards)
    return sorted(hazards)


LOOP_TEMPLATE = """\
_Zfoo:
\ts_mov_b32 s0, 0
.LBB0_1:
{wait}\ts_barrier
\tds_read_b128 v[0:3], v4
\tv_mfma_f32_32x32x16_bf16 v[8:23], v[0:3], v[0:3], v[8:23]
\tds_read_b64_tr_b16 v[4:5], v6
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
"""


def test_analyser_sees_a_read_carried_around_a_loop_to_its_barrier():
    # the read at the end of the body reaches the barrier at the loop head
    (_, body), = split_functions(LOOP_TEMPLATE.format(wait=""))
    assert barrier_hazards(body) == [(".LBB0_1", 0)]
    (_, body), = split_functions(LOOP_TEMPLATE.format(wait="\ts_waitcnt lgkmcnt(1)\n"))
    assert barrier_hazards(body) == [(".LBB0_1", 1)]
    (_, body), = split_functions(LOOP_TEMPLATE.format(wait="\ts_waitcnt vmcnt(0) lgkmcnt(0)\n"))
    assert barrier_hazards(body) == []


def _assembly(src: str, out_dir: str) -> str:
    from exact_attention_95_amd import build
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [build.hipcc(), *build.COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(cmd), r.stderr[-2000:]))
    return out


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_no_kernel_reaches_a_barrier_with_lds_reads_in_flight(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
        paths = list(ex.map(lambda s: _assembly(s, str(tmp_path)), KERNEL_SOURCES))
    found, n_funcs, n_barriers = [], 0, 0
    for path in paths:
        text = open(path).read()
        for name, body in split_functions(text):
            n_funcs += 1
            n_barriers += sum(1 for line in body if line.strip().startswith("s_barrier"))
            for h in barrier_hazards(body):
                found.append((os.path.basename(path), name, h))
    assert n_funcs > 20 and n_barriers > 20  # the listing was parsed
    assert not found, found
