"""Static checks of the row-wave kernels' gfx950 assembly (no GPU needed):
mla_rowwave_kernel (bf16 cache), mla_rowwave_f8_kernel (FP8 cache) and
their sparse-mode versions mla_rowwave_sparse_kernel and
mla_rowwave_f8_sparse_kernel.

The kernels keep their 512-dim output accumulators in AGPRs a0-a255 that only
inline asm touches, and issue some matrix products as inline asm, which the
compiler does not see as matrix products.  That design holds only if the
compiled code keeps these properties, which these tests read off the
assembly that hipcc emits for the library source:

* no AGPR is named outside the inline asm blocks (the compiler never spills
  to, or allocates in, the accumulator file);
* no VGPR spills and no scratch memory (SGPRs spilled into VGPR lanes are
  harmless here: they never touch the accumulators);
* no instruction other than a matrix product reads or writes the VGPR
  result of a matrix product within the wait states that a 32x32x16 bf16
  product needs before its result may be read (12 on gfx950; the compiler
  itself inserts 12);
* no VALU instruction writes an operand register of a matrix product within
  the two wait states before it, along every control-flow path (the bf16
  kernels' products take their operands from loads and carry no wait states
  of their own; the FP8 kernels convert operands with VALU instructions and
  their product asm starts with s_nop 1).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_paged_kv_04_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
KERNELS = ["_ZN3mla18mla_rowwave_kernelENS_10DecodeArgsE",
           "_ZN3mla25mla_rowwave_sparse_kernelENS_10DecodeArgsE",
           "_ZN3mla21mla_rowwave_f8_kernelENS_10DecodeArgsE",
           "_ZN3mla28mla_rowwave_f8_sparse_kernelENS_10DecodeArgsE"]
RESULT_WAIT_STATES = 12


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    out = str(tmp_path_factory.mktemp("asm") / "mla_kernels.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, "mla_kernels.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read()


def _body(text, kernel):
    start = text.index("\n" + kernel + ":")
    end = text.index("s_endpgm", start)
    return text[start:end].split("\n")


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


@pytest.mark.parametrize("kernel", KERNELS)
def test_no_agpr_outside_inline_asm(asm, kernel):
    inside = False
    bad = []
    for ln in _body(asm, kernel):
        t = ln.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
        elif t.startswith(";;#ASMEND"):
            inside = False
        elif t and not t.startswith((";", ".")) and re.search(r"\ba\[?\d", t) and not inside:
            bad.append(t)
    assert not bad, bad[:10]


@pytest.mark.parametrize("kernel", KERNELS)
def test_no_spills(asm, kernel):
    i = asm.index(".name:           " + kernel)
    start = asm.rfind("\n  - ", 0, i)      # the kernel's metadata record
    end = asm.find("\n  - ", i)
    meta = asm[start:end if end > 0 else i + 4000]
    assert re.search(r"\.vgpr_spill_count:\s+0\b", meta)
    assert re.search(r"\.private_segment_fixed_size:\s+0\b", meta)


@pytest.mark.parametrize("kernel", KERNELS)
def test_mfma_results_not_touched_early(asm, kernel):
    lines = [l.strip() for l in _body(asm, kernel)]
    bad = []
    for i, l in enumerate(lines):
        if not l.startswith("v_mfma"):
            continue
        dst = _vregs(l.split(None, 1)[1].split(",")[0].strip())
        if not dst:
            continue   # AGPR result
        states = 0
        for l2 in lines[i + 1:]:
            if not l2 or l2.startswith((";", ".")) or l2.endswith(":"):
                continue
            m = re.match(r"s_nop (\d+)", l2)
            states += int(m.group(1)) + 1 if m else 1
            if states > RESULT_WAIT_STATES:
                break
            if l2.startswith("v_mfma"):
                ops = [o.strip() for o in l2.split(None, 1)[1].split(",")]
                if (_vregs(ops[1]) | _vregs(ops[2])) & dst:
                    bad.append((l, l2))
                continue
            parts = l2.split(None, 1)
            if len(parts) < 2:
                continue
            regs = set()
            for tok in re.split(r",\s*", parts[1].split(";")[0]):
                if tok:
                    regs |= _vregs(tok.split()[0])
            if regs & dst:
                bad.append((l, l2))
    assert not bad, bad[:10]


OPERAND_WAIT_STATES = 2   # a VALU write of a matrix product's operand, then the product


def _cfg(asm_text, kernel):
    """The kernel's instructions and labels in order, with each label's
    branch sources (as ('label', name) / ('ins', text) items)."""
    items = []
    for ln in _body(asm_text, kernel):
        t = ln.split(";")[0].strip()
        if not t or t.startswith("."):
            m = re.match(r"^(\.LBB\w+):", ln.strip())
            if m:
                items.append(("label", m.group(1)))
            continue
        if t.endswith(":"):
            continue
        items.append(("ins", t))
    preds = {}
    for i, (kind, x) in enumerate(items):
        m = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", x) if kind == "ins" else None
        if m:
            preds.setdefault(m.group(1), []).append(i)
    return items, preds


def _valu_dst(ins):
    op = ins.split()[0]
    if not op.startswith("v_") or op.startswith("v_mfma"):
        return set()
    if op.startswith("v_cmp") and "_e64" not in op:
        return set()   # VOPC writes vcc only
    args = ins[len(op):].split(",")
    return _regs(args[0]) if args and args[0].strip() else set()


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


@pytest.mark.parametrize("kernel", KERNELS)
def test_products_wait_for_valu_written_operands(asm, kernel):
    """No VALU instruction writes a register that a matrix product reads
    (A, B or C operand, VGPR or AGPR) within the two wait states before it,
    along every control-flow path into the product (branch sources and
    fall-through alike; each instruction counts one wait state, s_nop N
    counts N + 1)."""
    items, preds = _cfg(asm, kernel)
    n = 0
    bad = []
    for i, (kind, x) in enumerate(items):
        if kind != "ins" or not x.startswith("v_mfma"):
            continue
        n += 1
        ops = [o.strip() for o in x.split(None, 1)[1].split(",")]
        srcs = set()
        for o in ops[1:4]:
            srcs |= _regs(o)
        work, seen = [(i - 1, OPERAND_WAIT_STATES)], set()
        while work:
            p, rem = work.pop()
            if rem <= 0 or (p, rem) in seen:
                continue
            seen.add((p, rem))
            if p < 0:
                continue
            kind2, y = items[p]
            if kind2 == "label":
                work.extend((b, rem) for b in preds.get(y, []))
                q = p - 1
                while q >= 0 and items[q][0] == "label":
                    q -= 1
                if q >= 0 and not items[q][1].startswith(("s_branch", "s_endpgm")):
                    work.append((p - 1, rem))
                continue
            if _valu_dst(y) & srcs:
                bad.append((x, y))
                continue
            m = re.match(r"s_nop (\d+)", y)
            work.append((p - 1, rem - (int(m.group(1)) + 1 if m else 1)))
    assert n > 0
    assert not bad, bad[:10]
