"""The grouped GEMM issues its weight loads as inline assembly, which the
compiler does not count: it neither waits for them nor knows that their
destination registers are still being written.  The kernel's own explicit
waits must therefore retire every such load before anything touches its
registers (an MFMA reading the operand, a copy, or another value placed in
them after the compiler considers them dead).

This test compiles gemm.hip for gfx950 to assembly, exactly as the library
build does, and walks every bf16 register-fed kernel: it keeps the queue of
loads in flight (all vector-memory loads count towards vmcnt, in issue
order), retires the oldest ones at each `s_waitcnt vmcnt(N)`, and fails on
any instruction that names a register of an untracked load still in the
queue.  Loop bodies are walked twice, so loads issued for the next
iteration meet their uses; a new path (after s_branch / s_endpgm) starts
with an empty queue."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_sparse_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# the untracked weight load: 16 bytes per lane, VGPR offset + SGPR base
UNTRACKED = re.compile(r"global_load_dwordx4 v\[\d+:\d+\], v\d+, s\[")


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _walk_order(raw):
    """Line indices in walk order: straight-line code once, each loop body
    (from its header to the branch back to it) twice."""
    seq, i = [], 0
    while i < len(raw):
        if "Loop Header" in raw[i]:
            lab = raw[i].split(":")[0]
            back = re.compile(r"s_cbranch\w*\s+" + re.escape(lab) + r"\b")
            e = next(k for k in range(i + 1, len(raw)) if back.search(raw[k]))
            seq += list(range(i, e + 1)) * 2
            i = e + 1
        else:
            seq.append(i)
            i += 1
    return seq


def violations(func_text):
    raw = func_text.split("\n")
    lines = [l.split(";")[0].strip() for l in raw]
    queue, bad = [], []
    for i in _walk_order(raw):
        l = lines[i]
        if not l or l.startswith(".") or l.endswith(":"):
            continue
        op = l.split()[0]
        if op in ("s_endpgm", "s_branch"):
            queue = []
            continue
        if op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", l)
            if m and len(queue) > int(m.group(1)):
                queue = queue[len(queue) - int(m.group(1)):]
            continue
        operands = l.split(None, 1)[1] if " " in l else ""
        pending = set()
        for untracked, dest in queue:
            if untracked:
                pending |= dest
        hit = _regs(operands) & pending
        if hit:
            bad.append(f"line {i}: {l} (registers {sorted(hit)[:4]} still loading)")
        if op.startswith(("global_load", "buffer_load", "flat_load")):
            dest = set() if "lds" in op else _regs(operands.split(",")[0])
            queue.append((bool(UNTRACKED.match(l)), dest))
    return bad


@pytest.fixture(scope="module")
def gemm_isa():
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "gemm.s")
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-x", "hip", "--cuda-device-only", "-S",
               os.path.join(CSRC, "gemm.hip"), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            pytest.fail(f"hipcc failed:\n{r.stderr[-2000:]}")
        with open(out) as f:
            return f.read()


def _kernels(isa):
    funcs = re.split(r"\n(?=_ZN3moe[^\n]*:\s*;)", isa)
    found = {}
    for f in funcs:
        name = f.split(":")[0]
        # bf16 (unsigned short) register-fed kernels: the FP8 form (F8 = true,
        # "Lb1E") and the fp32-output form keep compiler-tracked loads
        if "k_gemm_wideIt" in name and "Lb0E" in name:
            found[name] = f
    return found


def test_untracked_weight_loads_are_waited_for(gemm_isa):
    kernels = _kernels(gemm_isa)
    assert len(kernels) >= 4, sorted(kernels)
    for name, text in kernels.items():
        assert sum(1 for l in text.split("\n") if UNTRACKED.search(l)) > 0, name
        bad = violations(text)
        assert not bad, f"{name}: " + "; ".join(bad[:5])


def test_the_walk_catches_a_missing_wait():
    # a register read right after its untracked load, with no wait between
    text = "\n".join([
        "k:",
        "\tglobal_load_dwordx4 v[4:7], v1, s[2:3]",
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]",
        "\ts_endpgm",
    ])
    assert len(violations(text)) == 1
    # ... and accepts it once the wait retires the load
    ok = text.replace("\tv_mfma", "\ts_waitcnt vmcnt(0)\n\tv_mfma")
    assert violations(ok) == []
    # a loop whose next-iteration load is used before the wait at its top
    loop = "\n".join([
        "k:",
        "\tglobal_load_dwordx4 v[4:7], v1, s[2:3]",
        "\ts_waitcnt vmcnt(0)",
        ".LBB0_1:                                ; =>This Inner Loop Header: Depth=1",
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]",
        "\tglobal_load_dwordx4 v[4:7], v1, s[2:3]",
        "\ts_cbranch_scc0 .LBB0_1",
        "\ts_waitcnt vmcnt(0)",
        "\ts_endpgm",
    ])
    assert violations(loop)
