"""The C ABI without a GPU: the library loads, exports every declared entry point, matches the binding's
struct layout, rejects invalid arguments before any HIP call, and its host-only calibration agrees
with the oracle's."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blasst.h")


@pytest.fixture(scope="module")
def m():
    import long_context_online_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        from long_context_online_amd import build
        build.build()
    pkg.lib()
    return pkg


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(blasst_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(m):
    names = _declared_functions()
    assert "blasst_prefill" in names and "blasst_decode" in names and "blasst_calibrate" in names
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in blasst.h but not exported"
    assert set(names) == set(m.blasst.EXPORTED)


def test_struct_layout_matches_binding(m):
    lib = m.lib()
    assert lib.blasst_prefill_params_size() == ctypes.sizeof(m.blasst.PrefillParams)
    assert lib.blasst_decode_params_size() == ctypes.sizeof(m.blasst.DecodeParams)
    assert lib.blasst_prefill_backward_params_size() == ctypes.sizeof(m.blasst.BackwardParams)
    assert lib.blasst_prefill_paged_params_size() == ctypes.sizeof(m.blasst.PagedPrefillParams)
    assert lib.blasst_version() >= 10000


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case below fails validation first


def _prefill(**over):
    from long_context_online_amd.blasst import PrefillParams, Threshold
    p = PrefillParams()
    p.struct_size = ctypes.sizeof(PrefillParams)
    p.q = p.k = p.v = p.o = FAKE
    p.q_stride[:] = [128 * 256 * 128, 256 * 128, 128]
    p.k_stride[:] = p.v_stride[:] = p.o_stride[:] = p.q_stride[:]
    p.thr = Threshold(0, 0, 0.5, 0.0)
    p.in_dtype = p.out_dtype = 0
    p.batch, p.seqlen_q, p.seqlen_k = 1, 256, 256
    p.num_q_heads, p.num_kv_heads, p.head_dim_qk, p.head_dim_v = 4, 2, 128, 128
    p.causal, p.block_q, p.block_k, p.num_splits = 1, 128, 128, 1
    for k, v in over.items():
        if k == "thr":
            p.thr = Threshold(*v)
        else:
            setattr(p, k, v)
    return p


PREFILL_BAD = [
    ({"k_stride": (1 << 40, 1 << 30, 1 << 22)}, 2),
    ({"q": None}, 1), ({"o": None}, 1), ({"batch": 0}, 1), ({"num_kv_heads": 3}, 1),
    ({"num_splits": 0}, 1), ({"in_dtype": 7}, 1), ({"causal": 2}, 1), ({"block_k": 0}, 1),
    ({"thr": (0, 0, 1.5, 0.0)}, 1), ({"thr": (0, 0, -0.1, 0.0)}, 1), ({"thr": (1, 0, 0.0, -2.0)}, 1),
    ({"thr": (5, 0, 0.0, 0.0)}, 1), ({"thr": (0, 1, 0.5, 0.0)}, 1), ({"struct_size": 8}, 1),
    ({"softmax_scale": float("nan")}, 1),
    ({"thr": (2, 0, 0.0, 0.0), "skip_mask": FAKE}, 1), ({"thr": (2, 0, 0.0, 0.0), "crit": FAKE}, 1),
    ({"thr": (2, 0, 0.0, 0.0), "stats_only": 1}, 1),
    ({"head_dim_qk": 96, "head_dim_v": 96}, 2), ({"block_q": 64}, 2), ({"block_q": 32, "block_k": 32}, 2),
    ({"q": FAKE + 2}, 2), ({"in_dtype": 1, "out_dtype": 0}, 2), ({"in_dtype": 1, "out_dtype": 1}, 2),
    # bf16 K/V rows must not overlap (token stride >= head_dim): an expanded tensor (stride 0) and a
    # stride below the row length are refused
    ({"k_stride": (128 * 256 * 128, 256 * 128, 0)}, 2), ({"v_stride": (128 * 256 * 128, 256 * 128, 64)}, 2),
    ({"v_staging": 2}, 1), ({"v_staging": -1}, 1),
]


@pytest.mark.parametrize("over,status", PREFILL_BAD, ids=[str(x[0]) for x in PREFILL_BAD])
def test_prefill_rejects_invalid_arguments(m, over, status):
    lib = m.lib()
    p = _prefill(**over)
    assert lib.blasst_prefill(ctypes.byref(p), None) == status
    assert lib.blasst_last_error()
    assert lib.blasst_prefill(None, None) == 1


def test_prefill_workspace_size(m):
    """The prefill keeps every partial result on chip: 0 bytes for valid params with the last error
    cleared; invalid params give 0 with a message (pointers are not checked)."""
    lib = m.lib()
    lib.blasst_prefill(None, None)                       # leaves a message behind
    assert lib.blasst_prefill_workspace_size(ctypes.byref(_prefill(num_splits=4))) == 0
    assert lib.blasst_last_error() == b""
    assert lib.blasst_prefill_workspace_size(ctypes.byref(_prefill(q=None, k=None, v=None, o=None))) == 0
    assert lib.blasst_last_error() == b""
    assert lib.blasst_prefill_workspace_size(ctypes.byref(_prefill(num_kv_heads=3))) == 0
    assert b"multiple" in lib.blasst_last_error()
    assert lib.blasst_prefill_workspace_size(None) == 0 and lib.blasst_last_error()


def _decode(**over):
    from long_context_online_amd.blasst import DecodeParams, Threshold
    p = DecodeParams()
    p.struct_size = ctypes.sizeof(DecodeParams)
    p.q = p.k_cache = p.v_cache = p.block_table = p.seq_lens = p.o = FAKE
    p.thr = Threshold(1, 0, 0.0, 2.0)
    p.in_dtype = 0
    p.out_dtype = 1
    p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim_qk, p.head_dim_v = 4, 32, 8, 128, 128
    p.page_size, p.max_pages_per_seq, p.num_pages = 16, 64, 300
    p.block_k, p.num_splits, p.tile_rows = 64, 16, 0
    for k, v in over.items():
        if k == "thr":
            p.thr = Threshold(*v)
        else:
            setattr(p, k, v)
    return p


DECODE_BAD = [
    ({"q": None}, 1), ({"seq_lens": None}, 1), ({"num_kv_heads": 5}, 1), ({"block_k": 40}, 1),
    ({"num_splits": 0}, 1), ({"tile_rows": 3}, 1), ({"thr": (0, 0, 2.0, 0.0)}, 1), ({"num_q_tokens": -1}, 1),
    ({"page_size": 0}, 1), ({"struct_size": 4}, 1),
    ({"in_dtype": 1}, 2), ({"page_size": 32, "block_k": 64}, 2), ({"block_k": 128}, 2),
    ({"head_dim_qk": 64, "head_dim_v": 64}, 2), ({"v_cache": None}, 2),
    ({"workspace": None}, 4),
    ({"num_q_tokens": 5}, 2), ({"num_q_tokens": 9, "tile_rows": 2}, 2),
    ({"v_cache": None, "num_kv_heads": 1, "num_q_heads": 128, "head_dim_qk": 576, "head_dim_v": 512,
      "tile_rows": 128, "num_q_tokens": 2}, 2),
    ({"v_cache": None, "num_kv_heads": 1, "num_q_heads": 128, "head_dim_qk": 576, "head_dim_v": 512,
      "tile_rows": 32, "num_q_tokens": 3}, 2),
    ({"v_cache": None, "num_kv_heads": 1, "num_q_heads": 128, "head_dim_qk": 576, "head_dim_v": 512,
      "tile_rows": 16, "num_q_tokens": 2}, 2),
    # threshold mode NONE (no decisions) takes no decision diagnostics, whatever `a` holds
    ({"thr": (2, 0, 0.0, 5.0), "skip_mask": FAKE}, 1), ({"thr": (2, 0, 0.0, 5.0), "crit": FAKE}, 1),
    ({"thr": (2, 0, 0.0, float("nan")), "stats_only": 1}, 1),
    # 32-bit indexing in the kernels: context length, workgroup count and mask rows
    ({"max_pages_per_seq": 1 << 28}, 2), ({"batch": 1 << 12, "num_splits": 1 << 16}, 2),
    ({"batch": 1 << 12, "max_pages_per_seq": 1 << 16}, 2),
]


@pytest.mark.parametrize("over,status", DECODE_BAD, ids=[str(x[0]) for x in DECODE_BAD])
def test_decode_rejects_invalid_arguments(m, over, status):
    lib = m.lib()
    p = _decode(**over)
    assert lib.blasst_decode(ctypes.byref(p), None) == status
    assert lib.blasst_last_error()


def test_decode_no_alloc_rejects_before_any_hip_call(m):
    """The allocation-free decode checks its arguments like blasst_decode (no GPU needed to reach
    them), and refuses params whose split partials exceed the library's scratch array."""
    lib = m.lib()
    cap = 64 << 20
    for over, status in DECODE_BAD:
        if over == {"workspace": None}:
            continue          # ignored here: there is no workspace
        p = _decode(**over)
        assert lib.blasst_decode_no_alloc(ctypes.byref(p), None) == status
        assert lib.blasst_last_error()
    big = _decode(batch=512, num_splits=16)       # 512 x 32 x 16 partials of 129 floats > 64 MiB
    assert lib.blasst_decode_workspace_size(ctypes.byref(big)) > cap
    assert lib.blasst_decode_no_alloc(ctypes.byref(big), None) == 4
    assert b"scratch" in lib.blasst_last_error()
    latent = _decode(v_cache=None, batch=64, num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                     tile_rows=128, num_splits=8)
    assert lib.blasst_decode_no_alloc(ctypes.byref(latent), None) == 4


def test_decode_workspace_size(m):
    lib = m.lib()
    p = _decode()
    n = lib.blasst_decode_workspace_size(ctypes.byref(p))
    parts = 4 * 32 * 16
    assert n >= parts * (128 + 1) * 4 and n % 256 == 0
    p1 = _decode(num_splits=1)
    assert lib.blasst_decode_workspace_size(ctypes.byref(p1)) == 0
    p4 = _decode(num_q_tokens=4, tile_rows=4)
    assert lib.blasst_decode_workspace_size(ctypes.byref(p4)) >= 4 * parts * (128 + 1) * 4
    bad = _decode(num_kv_heads=5)
    assert lib.blasst_decode_workspace_size(ctypes.byref(bad)) == 0 and lib.blasst_last_error()


def test_calibration_matches_oracle(m):
    import oracle
    rng = np.random.default_rng(3)
    crit = np.concatenate([-np.abs(rng.standard_normal(997)) * 4, [np.inf] * 20, [np.nan] * 5]).astype(np.float32)
    for s in [0.0, 0.2, 0.5, 0.7, 0.75, 0.99]:
        got = m.blasst_calib_quantile(crit, s)
        want = oracle.quantile_ln_lambda(crit.astype(np.float64), s)
        assert got == pytest.approx(want, abs=1e-6) or (math.isinf(got) and math.isinf(want))
    L = np.array([4096, 8192, 16384, 32768, 65536, 131072] * 3, dtype=np.float64)
    s = np.repeat([0.3, 0.5, 0.7], 6)
    lam = np.exp(1.2 + 5.0 * s + 0.05 * rng.standard_normal(18)) / L
    a1, b1, r1 = m.blasst_calibrate(L, s, lam)
    a2, b2, r2 = oracle.fit_alpha_beta(L, s, lam)
    assert a1 == pytest.approx(a2, rel=1e-12) and b1 == pytest.approx(b2, rel=1e-12) and r1 == pytest.approx(r2, rel=1e-9)
    assert m.blasst_lambda_for(a1, b1, 0.5, 8192) == pytest.approx(oracle.lambda_for(a2, b2, 0.5, 8192), rel=1e-12)
    with pytest.raises(m.BlasstError):
        m.blasst_calibrate([1, 2], [0.5, 0.5], [0.1, 0.1])


def test_calibration_errors_set_the_message(m):
    """Every error return of the host calibration calls sets the calling thread's message, and a
    success clears it."""
    lib = m.lib()
    dp = ctypes.POINTER(ctypes.c_double)
    out = ctypes.c_double()
    c = np.array([-1.0, -2.0, np.nan], dtype=np.float32)
    cp = c.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    nan3 = np.full(3, np.nan, dtype=np.float32)
    cases = [
        (lambda: lib.blasst_calib_quantile(None, 3, 0.5, ctypes.byref(out)), b"non-NULL"),
        (lambda: lib.blasst_calib_quantile(cp, 0, 0.5, ctypes.byref(out)), b"n must"),
        (lambda: lib.blasst_calib_quantile(cp, 3, 1.5, ctypes.byref(out)), b"target_s"),
        (lambda: lib.blasst_calib_quantile(nan3.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 3, 0.5,
                                           ctypes.byref(out)), b"NaN"),
    ]
    L = np.array([4096.0, 8192.0]); s2 = np.array([0.5, 0.5]); lam = np.array([0.1, 0.1])
    args = [x.ctypes.data_as(dp) for x in (L, s2, lam)]
    a_, b_, r_ = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    outs = (ctypes.byref(a_), ctypes.byref(b_), ctypes.byref(r_))
    cases += [
        (lambda: lib.blasst_calibrate(*args, 1, *outs), b"two points"),
        (lambda: lib.blasst_calibrate(*args, 2, *outs), b"distinct"),
        (lambda: lib.blasst_calibrate(args[0], args[1], None, 2, *outs), b"non-NULL"),
    ]
    bad = np.array([0.1, -0.1])
    cases.append((lambda: lib.blasst_calibrate(args[0], np.array([0.3, 0.5]).ctypes.data_as(dp),
                                                bad.ctypes.data_as(dp), 2, *outs), b"point 1"))
    for call, text in cases:
        lib.blasst_calib_quantile(cp, 3, 0.5, ctypes.byref(out))   # a success clears the message
        assert lib.blasst_last_error() == b""
        assert call() == 1
        assert text in lib.blasst_last_error(), (text, lib.blasst_last_error())
    with pytest.raises(m.BlasstError, match="distinct"):
        m.blasst_calibrate([1, 2], [0.5, 0.5], [0.1, 0.1])


def _backward(**over):
    from long_context_online_amd.blasst import BackwardParams
    p = BackwardParams()
    p.struct_size = ctypes.sizeof(BackwardParams)
    p.q = p.k = p.v = p.o = p.dout = p.lse = p.dq = p.dk = p.dv = FAKE
    st = [32 * 4096 * 128, 4096 * 128, 128]
    for name in ("q_stride", "k_stride", "v_stride", "o_stride", "dout_stride", "dq_stride", "dk_stride",
                 "dv_stride"):
        getattr(p, name)[:] = st
    p.in_dtype, p.grad_dtype, p.o_dtype = 0, 1, 0
    p.batch, p.seqlen_q, p.seqlen_k, p.num_q_heads, p.num_kv_heads = 1, 4096, 4096, 32, 8
    p.head_dim_qk = p.head_dim_v = 128
    p.causal, p.block_q, p.block_k = 1, 128, 128
    for k, v in over.items():
        setattr(p, k, v)
    return p


BACKWARD_BAD = [
    ({"q": None}, 1), ({"lse": None}, 1), ({"dv": None}, 1), ({"num_kv_heads": 5}, 1), ({"seqlen_q": 0}, 1),
    ({"grad_dtype": 7}, 1), ({"o_dtype": 3}, 1), ({"causal": 2}, 1), ({"struct_size": 8}, 1), ({"softmax_scale": float("nan")}, 1),
    ({"in_dtype": 1}, 2), ({"head_dim_qk": 64, "head_dim_v": 64}, 2), ({"block_q": 64, "block_k": 64}, 2),
    ({"dq": FAKE + 8}, 2),
    ({}, 4),   # no workspace
]


@pytest.mark.parametrize("over,status", BACKWARD_BAD, ids=[str(x[0]) for x in BACKWARD_BAD])
def test_backward_rejects_invalid_arguments(m, over, status):
    lib = m.lib()
    p = _backward(**over)
    assert lib.blasst_prefill_backward(ctypes.byref(p), None) == status
    assert lib.blasst_last_error()


def test_backward_workspace_size(m):
    lib = m.lib()
    assert lib.blasst_prefill_backward_workspace_size(ctypes.byref(_backward())) == 32 * 4096 * 4
    odd = _backward(seqlen_q=1000, seqlen_k=1000)
    assert lib.blasst_prefill_backward_workspace_size(ctypes.byref(odd)) == (32 * 1000 * 4 + 255) // 256 * 256
    assert lib.blasst_prefill_backward_workspace_size(ctypes.byref(_backward(num_kv_heads=5))) == 0


def _paged(**over):
    from long_context_online_amd.blasst import PagedPrefillParams, Threshold
    p = PagedPrefillParams()
    p.struct_size = ctypes.sizeof(PagedPrefillParams)
    p.q = p.k_cache = p.v_cache = p.block_table = p.seq_lens = p.o = FAKE
    p.q_stride[:] = [32 * 512 * 128, 512 * 128, 128]
    p.o_stride[:] = p.q_stride[:]
    p.thr = Threshold(1, 0, 0.0, 4.0)
    p.in_dtype, p.out_dtype = 0, 0
    p.batch, p.seqlen_q, p.num_q_heads, p.num_kv_heads = 2, 512, 32, 8
    p.head_dim_qk = p.head_dim_v = 128
    p.page_size, p.max_pages_per_seq, p.num_pages = 16, 256, 600
    p.block_q = p.block_k = 128
    p.num_splits = 1
    for k, v in over.items():
        if k == "thr":
            p.thr = Threshold(*v)
        else:
            setattr(p, k, v)
    return p


PAGED_BAD = [
    ({"q": None}, 1), ({"seq_lens": None}, 1), ({"v_cache": None}, 1), ({"o": None}, 1), ({"num_kv_heads": 5}, 1),
    ({"num_splits": 0}, 1), ({"thr": (0, 0, 1.5, 0.0)}, 1), ({"struct_size": 16}, 1), ({"page_size": 0}, 1),
    ({"in_dtype": 1}, 2), ({"page_size": 32}, 2), ({"block_q": 64, "block_k": 64}, 2),
    ({"head_dim_qk": 64, "head_dim_v": 64}, 2), ({"q": FAKE + 4}, 2),
    ({"thr": (2, 0, 0.0, 0.0), "skip_mask": FAKE}, 1), ({"thr": (2, 0, 0.0, 0.0), "stats_only": 1}, 1),
    ({"max_pages_per_seq": 1 << 28}, 2), ({"num_pages": 1 << 30}, 2),
]


@pytest.mark.parametrize("over,status", PAGED_BAD, ids=[str(x[0]) for x in PAGED_BAD])
def test_paged_prefill_rejects_invalid_arguments(m, over, status):
    lib = m.lib()
    p = _paged(**over)
    assert lib.blasst_prefill_paged(ctypes.byref(p), None) == status
    assert lib.blasst_last_error()
