"""The realigning kernels take a neighbouring lane's word with a DPP wave
shift (wave_shl:1), which reads nothing useful from a lane that is switched
off.  This test compiles rr_kernels.hip for gfx950 to assembly (no GPU
needed) and walks the control-flow graph of every realigning kernel: on every
path, each instruction carrying the wave shift (the DPP move, or a VALU
operation the compiler folded it into) must run outside any divergent region
(no s_*_saveexec without its restore), i.e. with every lane of the wave
active.  No ds_bpermute remains."""
import os
import re
import shutil
import subprocess

import pytest

from pack_rr_helper_amd import build as B

KERNELS = ("copy_mixed_kernel", "copy_mixed_uniform_kernel", "reduce_shifted_kernel",
           "reduce_shifted_uniform_kernel")


def _asm(tmp_path):
    if not shutil.which(B.HIPCC) and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / "rr_kernels.s"
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), B.SOURCES[0]],
                   check=True, capture_output=True)
    return out.read_text().split("\n")


def _functions(lines):
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S+:", l)]
    for st in starts:
        end = next((i for i in range(st + 1, len(lines)) if lines[i].strip().startswith(".Lfunc_end")),
                   len(lines))
        yield lines[st].split(":")[0], lines[st + 1:end]


def _blocks(body):
    order, blocks, cur = ["entry"], {"entry": []}, "entry"
    for t in (l.strip() for l in body):
        m = re.match(r"^(\.LBB\d+_\d+):", t) or re.match(r"^; %(bb\.\d+):", t)
        if m:
            cur = m.group(1)
            order.append(cur)
            blocks[cur] = []
        elif t and not t.startswith((";", ".")):
            blocks[cur].append(t)
    succ = {}
    for i, b in enumerate(order):
        s, falls = [], True
        for t in blocks[b]:
            m = re.match(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", t)
            if m:
                s.append(m.group(1))
            m = re.match(r"s_branch\s+(\.LBB\d+_\d+)", t)
            if m:
                s.append(m.group(1))
                falls = False
            if t.startswith("s_endpgm"):
                falls = False
        if falls and i + 1 < len(order):
            s.append(order[i + 1])
        succ[b] = s
    return order, blocks, succ


def _is_exchange(t):
    return "wave_shl:1" in t


def _exchanges_in_divergent_code(body):
    """(lane-exchange count, those reachable at a nonzero exec nesting depth)."""
    order, blocks, succ = _blocks(body)
    seen = {b: set() for b in order}
    seen["entry"].add(0)
    work, bad = ["entry"], set()
    while work:
        b = work.pop()
        for d0 in list(seen[b]):
            d = d0
            for j, t in enumerate(blocks[b]):
                if re.match(r"s_\w+_saveexec_b64", t):
                    d += 1
                elif re.match(r"s_or_b64\s+exec,\s*exec,", t) or re.match(r"s_mov_b64\s+exec,\s*s", t):
                    d = max(0, d - 1)
                if _is_exchange(t) and d:
                    bad.add((b, j))
            for s in succ[b]:
                if d not in seen[s] and d < 8:
                    seen[s].add(d)
                    work.append(s)
    total = sum(1 for b in order for t in blocks[b] if _is_exchange(t))
    return total, len(bad)


def test_lane_exchanges_run_with_every_lane_active(tmp_path):
    lines = _asm(tmp_path)
    checked = set()
    for name, body in _functions(lines):
        kern = next((k for k in KERNELS if re.search(rf"\d{k}[EI]", name)), None)
        if kern is None:
            continue
        total, bad = _exchanges_in_divergent_code(body)
        assert total > 0, f"{name}: no wave_shl:1 exchange found (the realignment changed shape)"
        assert bad == 0, f"{name}: {bad} of {total} lane exchanges run inside a divergent region"
        assert not any(t.strip().startswith("ds_bpermute") for t in body), f"{name}: ds_bpermute is back"
        checked.add(kern)
    assert checked == set(KERNELS)
