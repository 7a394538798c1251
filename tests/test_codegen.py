"""Code generation of the HIP kernels for gfx950 (no GPU needed: hipcc cross-compiles): every kernel
compiles without VGPR spills or scratch memory, and without a blown-up instruction count. A loop the
unroller leaves rolled turns a register ring indexed by the loop counter into select chains over
every slot (a paged prefill variant once compiled to 48K instructions and ran 50x slower), and a
spill turns a register access into a memory access."""

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_online_amd", "csrc")
MAX_INSTRUCTIONS = 12000
# Kernels allowed a few spills, each with the reason; their scratch accesses must still stay out of
# every inner loop (loop depth >= 2 in the compiler's annotations).
SPILLS_ALLOWED = {
    # O^T of 32 heads x 512 channels takes all 256 AGPRs and q, scores and fragments all 256 VGPRs:
    # the compiler keeps one or two prologue values in scratch and reloads them in the epilogue or at
    # the start of a pass (outside the block loop)
    "decode_mla_kernel": 4,
    # the fp32 path for the tiny configuration; its spills go to AGPRs (no scratch)
    "prefill_f32_kernel": 4,
}


_XDL_AGPR = re.compile(r"\s+v_mfma\S*\s+a\[")          # matrix product writing accumulation registers
_AGPR_OTHER = re.compile(r"\s+(?!v_mfma)\S+\s.*\ba(\d+|\[)")  # any other instruction touching them
_NOP = re.compile(r"\s+s_nop\s+(\w+)")
# Wait states required between a 32x32x16 bf16 product (8 passes) writing registers and a VALU, memory
# or LDS instruction reading or overwriting them: 11 in the CDNA3/CDNA4 hazard tables; checked against
# the 16-pass figure (19) to leave a margin.
XDL_WAIT_STATES = 19


def _instructions(body):
    """(instruction, written as inline assembly) pairs and the label -> instruction index map."""
    ins, labels, in_asm = [], {}, False
    for line in body:
        lab = re.match(r"^(\.LBB\d+_\d+):", line)
        if lab:
            labels[lab.group(1)] = len(ins)
        elif ";;#ASMSTART" in line:
            in_asm = True
        elif ";;#ASMEND" in line:
            in_asm = False
        elif line.startswith("\t") and not line.lstrip().startswith((";", ".")) and line.strip():
            ins.append((line.split(";")[0].rstrip(), in_asm))
    return ins, labels


def _asm_xdl_agpr(body):
    return any(a and _XDL_AGPR.match(t) for t, a in _instructions(body)[0])


def _agpr_hazards(body):
    """Minimum wait states, over every path through the kernel's control flow, between a matrix product
    written as inline assembly that writes accumulation registers (AGPRs) and the next instruction,
    other than a matrix product, that reads or writes any AGPR. The compiler tracks this hazard for
    the products it emits itself, but not for inline assembly, so only those products start the count.
    Returns the accesses whose minimum is below XDL_WAIT_STATES, and the products not preceded by an
    s_nop of at least 2 wait states (a VALU write of a product's operands needs 2)."""
    pairs, labels = _instructions(body)
    ins = [t for t, _ in pairs]
    xdl = [a and bool(_XDL_AGPR.match(t)) for t, a in pairs]
    n = len(ins)
    succ = []
    for i, t in enumerate(ins):
        f = t.split()
        if f[0] == "s_endpgm" or f[0].startswith("s_setpc"):
            succ.append([])
        elif f[0] == "s_branch":
            succ.append([labels[f[1]]])
        elif f[0].startswith("s_cbranch"):
            succ.append([labels[f[1]]] + ([i + 1] if i + 1 < n else []))
        else:
            succ.append([i + 1] if i + 1 < n else [])
    cost = [int(_NOP.match(t).group(1), 0) + 1 if _NOP.match(t) else 1 for t in ins]
    INF = 1 << 20
    before = [INF] * n            # min wait states since the last such product, on entry to instruction i
    work = list(range(n))
    while work:
        i = work.pop()
        out = 0 if xdl[i] else min(INF, before[i] + cost[i])
        for j in succ[i]:
            if out < before[j]:
                before[j] = out
                work.append(j)
    short = [(i, before[i], ins[i].strip()) for i in range(n)
             if not _XDL_AGPR.match(ins[i]) and _AGPR_OTHER.match(ins[i]) and before[i] < XDL_WAIT_STATES]
    unpadded = [(i, ins[i].strip()) for i in range(n)
                if xdl[i] and not (i > 0 and _NOP.match(ins[i - 1]) and cost[i - 1] >= 2)]
    return short, unpadded


def _kernels(path):
    from long_context_online_amd import build as b
    name = os.path.basename(path)
    out = f"/tmp/blasst_codegen_{os.getpid()}_{name}.s"
    cmd = [b.HIPCC, *[f for f in b.COMMON if f != "-fPIC"], *b.EXTRA.get(name, []), "-x", "hip",
           "--cuda-device-only", "-S", path, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read()
    os.remove(out)
    res = {}
    for block in text.split("- .agpr_count")[1:]:   # one metadata block per kernel
        sym = re.search(r"\.name:\s+(\S+)", block).group(1)
        m = re.search(r"^" + re.escape(sym) + r":", text, flags=re.M)
        j = text.index(".Lfunc_end", m.end())
        n = sum(1 for line in text[m.end():j].splitlines()
                if line.startswith("\t") and not line.lstrip().startswith((";", ".")))
        depth, deep_scratch = 0, 0
        for line in text[m.end():j].splitlines():
            d = re.search(r"Depth=(\d+)", line)
            if re.match(r"^\.LBB\d+_\d+:", line) or line.startswith("; %bb."):
                depth = int(d.group(1)) if d else 0
            if depth >= 2 and re.match(r"\s+(scratch_|buffer_(load|store)_dword\w* \S+, off, s\[0:3\])", line):
                deep_scratch += 1
        body = text[m.end():j].splitlines()
        res[sym] = {"instructions": n, "scratch_in_inner_loops": deep_scratch,
                    "xdl_agpr_body": body if _asm_xdl_agpr(body) else None,
                    "vgpr_spills": int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1)),
                    "scratch": int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))}
    return name, res


@pytest.fixture(scope="module")
def codegen():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        return dict(ex.map(_kernels, srcs))


def test_every_source_has_kernels(codegen):
    for name, kernels in codegen.items():
        if name != "noalloc.hip":
            assert kernels, f"no kernel found in {name}"


def test_no_spills_no_scratch_no_blowup(codegen):
    bad = []
    for name, kernels in codegen.items():
        for sym, k in kernels.items():
            allowed = next((n for key, n in SPILLS_ALLOWED.items() if key in sym), 0)
            spills = max(k["vgpr_spills"], k["scratch"] // 4)
            if spills > allowed or k["scratch_in_inner_loops"] or k["instructions"] > MAX_INSTRUCTIONS:
                bad.append((name, sym[:90], k))
    assert not bad, "\n".join(map(str, bad))


def test_inline_assembly_products_keep_their_wait_states(codegen):
    """The latent decode's P.V products accumulate in AGPRs through inline assembly, which the
    compiler's hazard tracking does not see: every path from such a product to a VALU, memory or LDS
    access of an AGPR (the zeroing at the start of a pass, the epilogue's reads and stores, any copy
    the register allocator adds) must carry the wait states written around the products."""
    checked = 0
    for name, kernels in codegen.items():
        for sym, k in kernels.items():
            if k["xdl_agpr_body"] is None:
                continue
            checked += 1
            short, unpadded = _agpr_hazards(k["xdl_agpr_body"])
            assert not short, (name, sym[:90], short[:5])
            assert not unpadded, (name, sym[:90], unpadded[:5])
    assert checked >= 2   # the latent decode kernel with and without diagnostics


def test_agpr_hazard_check_finds_a_missing_pad():
    """The check itself: a product followed too closely by a read of its accumulators, directly and
    around a loop back edge, is reported; padded enough, it is not."""
    mf = "\t;;#ASMSTART\n\ts_nop 3\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n\t;;#ASMEND"
    rd = "\tv_accvgpr_read_b32 v8, a0"
    body = (mf + "\n\ts_nop 7\n" + rd + "\n\ts_endpgm").splitlines()
    assert len(_agpr_hazards(body)[0]) == 1
    body = (mf + "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n" + rd + "\n\ts_endpgm").splitlines()
    assert _agpr_hazards(body) == ([], [])
    loop = (".LBB0_1:\n\tv_accvgpr_write_b32 a0, 0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n" + mf +
            "\n\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm").splitlines()
    assert len(_agpr_hazards(loop)[0]) == 1            # the back edge reaches the write 1 state later
    assert len(_agpr_hazards(["\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
                               "\t;;#ASMEND", "\ts_endpgm"])[1]) == 1  # no s_nop before the product
    # a product the compiler emitted itself (outside inline assembly) is left to its hazard tracking
    assert _agpr_hazards(["\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]", rd,
                          "\ts_endpgm"]) == ([], [])
