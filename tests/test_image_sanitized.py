"""The library's host-side container-image checks (csrc/image.cpp), built on
the CPU with the address and undefined-behaviour sanitizers and run on well
formed images and on images corrupted field by field and byte by byte: every
check must come back with a status and no sanitizer report (no read past a
buffer, no overflow, no misaligned access).  CPU only: the checks make no
device calls."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from dequant_gemv_spectra_amd import synth
from oracle import spectra_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cxx():
    for c in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no host C++ compiler")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    d = tmp_path_factory.mktemp("imgsan")
    exe = str(d / "image_harness")
    srcs = [os.path.join(ROOT, "dequant_gemv_spectra_amd", "csrc", "image.cpp"),
            os.path.join(ROOT, "tests", "image_sanitizer_harness.cpp")]
    # host code only (the HIP headers in their host-compiler mode)
    cmd = [_cxx(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *srcs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"sanitizer build unavailable: {r.stderr[-400:]}")
    return exe


def _images():
    out = []
    for N, K, n_out, seed in ((3, 31, 1, 1), (40, 200, 9, 2), (17, 33, 2, 3), (9, 5, 0, 4), (64, 96, 3, 5)):
        W, g, _ = synth.random_case(N, K, n_out, seed)
        out.append(O.pack(W, g))
    W, g, _ = synth.random_case(9, 5, 0, 6)
    out.append(O.pack(W, g, mask=np.ones(5, bool)))  # every channel heavy-tailed (G = 0)
    return out


def _corruptions(img, rng):
    """(label, bytes, expected-valid) variants of one image."""
    b = bytearray(img)
    yield "whole", bytes(b), True
    yield "empty", b"", False
    yield "header only", bytes(b[:128]), False
    yield "truncated", bytes(b[:-256]), False
    yield "one byte short", bytes(b[:-1]), False
    yield "extended", bytes(b) + b"\0" * 256, False
    for off, val in ((8, 1 << 40), (8, 0), (16, 0), (16, 1 << 62), (24, 3), (32, 1 << 20), (40, 1 << 30),
                     (48, 7), (56, 1 << 33), (64, 1 << 63), (96, 16), (96, (1 << 64) - 1)):
        c = bytearray(b)
        c[off:off + 8] = int(val).to_bytes(8, "little")
        yield f"header field {off} = {val}", bytes(c), False
    c = bytearray(b)
    c[0] ^= 1
    yield "magic", bytes(c), False
    for i in range(40):  # random byte flips past the header
        c = bytearray(b)
        pos = int(rng.integers(128, len(b)))
        c[pos] ^= int(rng.integers(1, 256))
        yield f"flip at {pos}", bytes(c), None  # either verdict, never a sanitizer report


@pytest.mark.parametrize("chunk", [256, 4096, 1 << 20])
def test_image_checks_are_memory_safe(harness, tmp_path, chunk):
    rng = np.random.default_rng(chunk)
    files, expect = [], []
    for i, img in enumerate(_images()):
        for j, (label, data, valid) in enumerate(_corruptions(img, rng)):
            p = tmp_path / f"img{i}_{j}.bin"
            p.write_bytes(data)
            files.append(str(p))
            expect.append((label, valid))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([harness, str(chunk), *files], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitizer or harness failure:\n{r.stderr[-3000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    lines = r.stdout.split()
    assert len(lines) == 2 * len(files)
    for k, (label, valid) in enumerate(expect):
        whole, streamed = int(lines[2 * k]), int(lines[2 * k + 1])
        assert whole == streamed, f"{label}: whole {whole} vs streamed {streamed}"
        if valid is True:
            assert whole == 0, f"{label}: a well formed image was rejected"
        elif valid is False:
            assert whole == -1, f"{label}: a malformed image was accepted"
        else:
            assert whole in (0, -1)
