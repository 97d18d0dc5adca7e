"""CPU-side checks of the C ABI: the library loads, exports every function the
public header declares, and rejects bad arguments before touching a device."""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spectra.h")


def _lib():
    from dequant_gemv_spectra_amd import spectra
    if not os.path.exists(spectra.LIB_PATH):
        from dequant_gemv_spectra_amd import build
        build.build()
    return spectra


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spectra_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for required in ("spectra_pack", "spectra_gemm", "spectra_free", "spectra_info", "spectra_export",
                     "spectra_last_error", "spectra_gemm_ex", "spectra_gemm_grouped", "spectra_pack_device",
                     "spectra_version"):
        assert required in names


def test_library_exports_every_declared_symbol():
    sp = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", sp.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(spectra_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    L = sp.lib()
    for n in declared_functions():
        getattr(L, n)
    assert set(sp.EXPORTED) == set(declared_functions())


def test_status_codes_match_header():
    sp = _lib()
    text = open(HEADER).read()
    for name, val in re.findall(r"(SPECTRA_E_\w+|SPECTRA_OK)\s*=\s*(-?\d+)", text):
        assert getattr(sp, name) == int(val), name
    kernels = dict(re.findall(r"SPECTRA_KERNEL_(\w+)\s*=\s*(\d+)", text))
    assert {k.lower(): int(v) for k, v in kernels.items()} == sp.KERNELS
    plans = {int(v): k for k, v in re.findall(r"SPECTRA_PLAN_(\w+)\s*=\s*(\d+)", text)}
    assert plans == {1: "GEMV", 2: "MFMA_TILED", 3: "MFMA", 4: "MFMA_SPLITK"}
    assert sp.PLANS == {1: "k_gemv_m1", 2: "k_mfma_ks", 3: "k_mfma", 4: "k_mfma_sk"}


def test_host_argument_checks_without_a_device():
    sp = _lib()
    L = sp.lib()
    P = ctypes.c_void_p
    assert L.spectra_version() == 1
    info = sp.spectra_info_t()
    assert L.spectra_info(None, ctypes.byref(info)) == sp.SPECTRA_E_INVAL
    assert L.spectra_gemm(None, P(16), P(16), 1) == sp.SPECTRA_E_INVAL
    assert L.spectra_gemm_ex(P(0x1000), P(16), P(16), 1, None, 0) == sp.SPECTRA_E_INVAL  # not a live handle
    assert L.spectra_gemm_plan(None, 1, 0) == sp.SPECTRA_E_INVAL
    assert L.spectra_gemm_plan(P(0x1000), 1, 0) == sp.SPECTRA_E_INVAL
    assert L.spectra_export(None, None, 0) == sp.SPECTRA_E_INVAL
    assert L.spectra_gemm_grouped(None, 1, None, None, 1, None) == sp.SPECTRA_E_INVAL
    L.spectra_free(None)
    L.spectra_free(P(0x1000))  # unknown handles are ignored, never dereferenced
    buf = (ctypes.c_uint16 * 16)()
    for K, N in ((0, 4), (4, 0), (-1, 4), (1 << 25, 1), (1 << 21, 1 << 20)):
        assert not L.spectra_pack(buf, buf, K, N)
        assert "out of range" in sp.spectra_last_error() or "2^40" in sp.spectra_last_error()
    assert not L.spectra_pack(None, buf, 4, 4)
    assert "null" in sp.spectra_last_error()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from dequant_gemv_spectra_amd import spectra
    monkeypatch.setattr(spectra, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(spectra, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        spectra.lib()
