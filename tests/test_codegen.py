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
        res[sym] = {"instructions": n, "scratch_in_inner_loops": deep_scratch,
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
