"""Static checks of the library's gfx950 machine code (CPU; built here from the sources).

The attention kernels and the k-major GEMM layouts read fragments with the transposing LDS read
`ds_read_b64_tr_b16` written as inline assembly: the compiler does not know these reads are in
flight, so it inserts no wait for them, and the kernels wait explicitly (`s_waitcnt lgkmcnt`)
before the fragments are used. That is only correct if no instruction reads or writes a
register of such a read while it is outstanding, the compiler's own register reuse included
(a mistake of this kind faults the GPU or corrupts results silently). This test compiles every
HIP source of the library to assembly and follows every path through each kernel's control flow
(a dataflow analysis over its basic blocks, loops iterated to a fixpoint), keeping the queue of
LDS operations that may be outstanding (`lgkmcnt(N)` leaves at most the newest N of them
outstanding: LDS operations complete in order), and reports every instruction that names a
register an outstanding LDS read may still write.

It also lists each kernel's register spills and requires none in the kernels of the forward
layer path.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_depth_token_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

REG_RE = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
LGKM_RE = re.compile(r"lgkmcnt\((\d+)\)")


def _regs(text):
    out = set()
    for m in REG_RE.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def _compile(src):
    from sparse_depth_token_amd import build as b
    fd, out = tempfile.mkstemp(suffix=".s")
    os.close(fd)
    cmd = [HIPCC, *[f for f in b.FLAGS if f != "-fPIC"], "--offload-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    try:
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return f.read()
    finally:
        os.remove(out)


def _kernels(asm):
    """{kernel symbol: [instructions and labels]} for every kernel in an assembly file."""
    out = {}
    for m in re.finditer(r"^(_Z\w+):\s*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        if end < 0 or f"\t.type\t{name},@function" not in asm:
            continue
        lines = []
        for ln in asm[m.end():end].splitlines():
            t = ln.split(";")[0].strip()
            if not t:
                continue
            if t.endswith(":") and t.startswith(".LBB"):
                lines.append(t)
            elif not t.startswith("."):
                lines.append(t)
        out[name] = lines
    return out


MAXQ = 64          # LDS operations tracked per path (the lgkmcnt field counts at most 15)


def _ds_operands(ins):
    op = ins.split()[0]
    operands = ins.split(None, 1)[1] if " " in ins else ""
    is_read = op.startswith(("ds_read", "ds_load", "ds_bpermute", "ds_permute",
                             "ds_swizzle")) or "_rtn_" in op
    if is_read:
        first, _, rest = operands.partition(",")
        return _regs(first), _regs(rest)
    return set(), _regs(operands)


def _step(state, ins, problems=None):
    """Transfer one instruction over the outstanding-LDS state: a tuple of register sets, newest
    first (position i: what the (i+1)-th newest outstanding LDS operation may still write)."""
    op = ins.split()[0]
    if op == "s_waitcnt":
        m = LGKM_RE.search(ins)
        return state[:int(m.group(1))] if m else state
    busy = set().union(*state) if state else set()
    if op.startswith("ds_"):
        dest, srcs = _ds_operands(ins)
        hit = (dest | srcs) & busy
        if hit and problems is not None:
            problems.append((ins, sorted(hit)))
        new = (frozenset(dest),) + state
        if len(new) > MAXQ:
            new = new[:MAXQ - 1] + (frozenset().union(*new[MAXQ - 1:]),)
        return new
    hit = _regs(ins) & busy
    if hit and problems is not None:
        problems.append((ins, sorted(hit)))
    return state


def _merge(a, b):
    n = max(len(a), len(b))
    return tuple((a[i] if i < len(a) else frozenset()) | (b[i] if i < len(b) else frozenset())
                 for i in range(n))


def check_kernel(lines):
    """Instructions that touch a register an outstanding LDS read may still write, on any path
    through the kernel's control flow: [(instruction, regs)]. A forward may-analysis over the
    basic blocks, iterated to a fixpoint (loops included)."""
    # basic blocks: split at labels and after branches
    blocks, labels, cur = [], {}, []
    for ins in lines:
        if ins.endswith(":"):
            if cur:
                blocks.append(cur)
            cur = []
            labels[ins[:-1]] = len(blocks)
            continue
        cur.append(ins)
        if ins.split()[0].startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    succ = []
    for i, b in enumerate(blocks):
        last = b[-1] if b else ""
        op = last.split()[0] if last else ""
        tgt = last.split()[1] if op.startswith(("s_branch", "s_cbranch")) else None
        out = []
        if tgt is not None:
            assert tgt in labels, f"branch to an unknown label: {last}"
            out.append(labels[tgt])
        if not op.startswith(("s_branch", "s_endpgm", "s_setpc")) and i + 1 < len(blocks):
            out.append(i + 1)
        succ.append(out)
    entry = [None] * len(blocks)
    entry[0] = ()
    work = [0]
    while work:
        i = work.pop()
        st = entry[i]
        for ins in blocks[i]:
            st = _step(st, ins)
        for j in succ[i]:
            m = st if entry[j] is None else _merge(entry[j], st)
            if m != entry[j]:
                entry[j] = m
                work.append(j)
    problems = []
    for i, b in enumerate(blocks):
        if entry[i] is None:
            continue
        st = entry[i]
        for ins in b:
            st = _step(st, ins, problems)
    return problems


SOURCES = ["attention.hip", "attention_bwd.hip", "gemm.hip", "rows.hip", "rows_bwd.hip",
           "route.hip", "probe.hip", "xmod_api.hip"]


@pytest.fixture(scope="module")
def asm():
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(zip(SOURCES, ex.map(_compile, SOURCES)))


def test_no_register_touched_by_an_outstanding_lds_read(asm):
    checked, with_tr = 0, 0
    report = {}
    for src, text in asm.items():
        for name, lines in _kernels(text).items():
            checked += 1
            with_tr += any("ds_read_b64_tr_b16" in l for l in lines)
            p = check_kernel(lines)
            if p:
                report[name] = p[:5]
    print(f"{checked} kernels checked, {with_tr} with transposing LDS reads")
    assert with_tr >= 8 and checked >= 40
    assert not report, report


def test_the_check_finds_a_planted_hazard():
    lines = ["ds_read_b64_tr_b16 v[10:11], v2 offset:64",
             "v_mov_b32 v3, v4",
             "v_add_f32 v5, v10, v6",           # reads v10 before the wait
             "s_waitcnt lgkmcnt(0)",
             "v_add_f32 v7, v11, v6"]
    assert [p[0] for p in check_kernel(lines)] == ["v_add_f32 v5, v10, v6"]
    # across a loop's back edge: the read issued at the end of the body is pending at its top
    loop = [".LBB0_1:", "v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[24:27], a[0:15]",
            "ds_read_b128 v[20:23], v1", "s_cbranch_scc1 .LBB0_1"]
    assert check_kernel(loop)
    ok = [".LBB0_1:", "s_waitcnt lgkmcnt(0)",
          "v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[24:27], a[0:15]",
          "ds_read_b128 v[20:23], v1", "s_cbranch_scc1 .LBB0_1"]
    assert not check_kernel(ok)


def _template_ints(name):
    """The integer template arguments of a mangled kernel name (Li<n>E), in order."""
    return [int(v) for v in re.findall(r"Li(\d+)E", name)]


def forward_kernel(name):
    """Kernels of the forward layer path: attention, router, top-k (both selects), the row
    kernels and the GEMM instances with a forward epilogue (store, SwiGLU, gated residual, fp32
    store) in the NT layout. The one-workgroup top-k instances for sequences of more than 16384
    tokens (32 and 64 keys per thread) are left out: they hold every key in registers and
    spill, and only the stand-alone top-k entry points called without a workspace run them
    (the layers take the chunked select for every sequence longer than 8192 tokens)."""
    if "gemm_kernel" in name:
        # <BM, BN, WM, WN, BK, NS, EPI, LAY, NL, SCHED>: forward epilogues, NT layout
        t = _template_ints(name)
        return len(t) == 10 and t[6] in (0, 1, 2, 3) and t[7] == 0
    if "topk_kernel" in name:
        return _template_ints(name) not in ([32], [64])
    return any(f in name for f in ("attn_kernel", "router_kernel", "gather_rows_kernel",
                                   "residual_rmsnorm_kernel", "scatter_kernel",
                                   "topk_chunk_hist_kernel", "topk_threshold_kernel",
                                   "topk_emit_kernel"))


def test_spills(asm):
    spills = {}
    for src, text in asm.items():
        for m in re.finditer(r"\.name:\s+(\S+)\n(?:.*\n)*?\s+\.vgpr_spill_count:\s+(\d+)", text):
            spills[m.group(1)] = int(m.group(2))
    print("kernels with spills:", {k: v for k, v in spills.items() if v})
    fwd = {k: v for k, v in spills.items() if forward_kernel(k)}
    assert len(fwd) >= 18
    assert sum("gemm_kernel" in k for k in fwd) >= 8, "forward GEMM instances checked"
    assert not any(fwd.values()), {k: v for k, v in fwd.items() if v}
