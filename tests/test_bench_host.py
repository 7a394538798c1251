"""Host-side behaviour of bench.py (no GPU): the one-GPU contract and the lookup of committed profile
records, which the benchmark reports only while the kernel sources hash to what was profiled."""

import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def _record(tmp_path, src_text):
    src = tmp_path / "k.hip"
    src.write_text(src_text)
    (tmp_path / "profiles").mkdir()
    rec = {"kern<1>": {"sources": ["k.hip"], "source_sha256": hashlib.sha256(src_text.encode()).hexdigest(),
                       "traffic_bytes": 1234,
                       "sq": {"mfma_instructions": 10, "mfma_flops": 327680, "mfma_busy": 0.5,
                              "lds_bank_conflict_frac": 0.0}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    return src


def test_profile_record_follows_the_source_hash(tmp_path, monkeypatch):
    src = _record(tmp_path, "kernel source\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("kern<1>") == 1234
    assert bench.profiled_counters("kern<1>")["mfma_busy"] == 0.5
    assert bench.profiled_traffic("other<2>") is None
    src.write_text("kernel source, changed\n")
    assert bench.profiled_traffic("kern<1>") is None
    assert bench.profiled_counters("kern<1>") is None


def test_profile_record_missing_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("kern<1>") is None


def test_ceiling_library_exports_and_rejects_bad_arguments():
    """The streaming-ceiling probe library the benchmark loads: its three entry points exist, and
    invalid arguments are refused before any launch (so this needs no GPU)."""
    import ctypes
    path = os.path.join(ROOT, "long_context_online_amd", "libblasst_ceiling.so")
    if not os.path.exists(path):
        from long_context_online_amd import build
        build.build()
    lib = ctypes.CDLL(path)
    assert lib.blasst_ceiling_page_bytes() == 4096
    lib.blasst_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_void_p]
    lib.blasst_ceiling_stream_pages.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int, ctypes.c_void_p]
    assert lib.blasst_ceiling_stream_read(None, 1024, 16, 8, None) == -1        # no source
    assert lib.blasst_ceiling_stream_read(16, 1000, 16, 8, None) == -1          # not whole 16-byte vectors
    assert lib.blasst_ceiling_stream_read(24, 1024, 16, 8, None) == -1          # misaligned
    assert lib.blasst_ceiling_stream_read(16, 1024, 16, 0, None) == -1          # empty grid
    assert lib.blasst_ceiling_stream_pages(16, None, 4, 16, 8, None) == -1      # no table
    assert lib.blasst_ceiling_stream_pages(16, 16, 0, 16, 8, None) == -1        # no pages
