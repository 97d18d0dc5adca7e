"""Container files and host images on the GPU: save / load round trips through
the chunked staging path, import of oracle-packed images, and rejection of
malformed files while they stream."""
import hashlib
import struct

import numpy as np
import pytest

from dequant_gemv_spectra_amd import synth
from oracle import spectra_oracle as O

pytestmark = pytest.mark.gpu


def _sp():
    from dequant_gemv_spectra_amd import spectra
    return spectra


def _torch():
    import torch
    return torch


def _same_products(c1, c2, K, M=1, seed=0):
    sp, torch = _sp(), _torch()
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal((M, K)).astype(np.float16)).cuda()
    y1 = sp.spectra_gemm(c1, x)
    y2 = sp.spectra_gemm(c2, x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("N,K,n_out,seed,chunk", [(300, 1000, 10, 1, 4096), (2049, 1536, 15, 2, 0),
                                                  (9, 97, 5, 3, 4096), (64, 9728, 120, 4, 65536)])
def test_save_load_round_trip(tmp_path, N, K, n_out, seed, chunk):
    sp = _sp()
    W, g, _ = synth.random_case(N, K, n_out, seed)
    c = sp.spectra_pack(W, g)
    img = sp.spectra_export(c)
    path = str(tmp_path / "c.spectra")
    sp.spectra_save(c, path, chunk)
    with open(path, "rb") as fh:
        assert fh.read() == img
    c2 = sp.spectra_load(path, chunk)
    assert sp.spectra_export(c2) == img
    _same_products(c, c2, K)


def test_import_oracle_image_runs_the_product_and_gather():
    sp, torch = _sp(), _torch()
    W, g, x = synth.random_case(257, 2560, 30, 5, M=2)
    img = O.pack(W, g)
    c = sp.spectra_import(img)
    assert sp.spectra_export(c) == img
    y = sp.spectra_gemm(c, torch.from_numpy(x).cuda()).cpu().numpy().astype(np.float64)
    W_hat = O.unpack(img)["W_hat"]
    assert np.all(np.abs(y - O.matmul_ref(W_hat, x)) <= O.tolerance(W_hat, x))
    ids = np.arange(0, 257, 5)
    e = sp.spectra_embed(c, torch.from_numpy(ids.astype(np.int32)).cuda()).cpu().numpy()
    assert np.array_equal(e.view(np.uint16), O.embed_ref(img, ids).view(np.uint16))


def test_load_rejects_malformed_files(tmp_path):
    sp = _sp()
    W, g, _ = synth.random_case(200, 3000, 30, 6)
    img = O.pack(W, g)
    u = O.unpack(img)
    off = u["offsets"]
    with pytest.raises(sp.SpectraError) as ei:
        sp.spectra_load(str(tmp_path / "missing.spectra"))
    assert ei.value.status == sp.SPECTRA_E_IO
    cases = {"truncated": img[:-256]}
    b = bytearray(img)
    struct.pack_into("<H", b, off["scales"] + 2 * (u["N"] * u["G"] - 3), 0x7E00)  # NaN late in the file
    cases["nan scale"] = bytes(b)
    b = bytearray(img)
    p = np.frombuffer(img, "<i4", 3000, off["perm"]).copy()
    p[[10, 11]] = p[[11, 10]]
    b[off["perm"]:off["perm"] + 12000] = p.tobytes()
    cases["perm order"] = bytes(b)
    for what, data in cases.items():
        path = str(tmp_path / (what.replace(" ", "_") + ".spectra"))
        with open(path, "wb") as fh:
            fh.write(data)
        with pytest.raises(sp.SpectraError) as ei:
            sp.spectra_load(path, 4096)
        assert ei.value.status == sp.SPECTRA_E_INVAL, what
    with pytest.raises(sp.SpectraError):
        sp.spectra_import(cases["nan scale"])


@pytest.mark.timeout(900)
def test_save_load_lm_head_container(tmp_path):
    """The 131072 x 3072 container (241 MB) through 8 MiB chunks."""
    sp = _sp()
    wl = synth.workload(4)
    lin = wl.linears[0]
    c = sp.spectra_pack(synth.weights(lin, 4), synth.gamma(lin, 4))
    path = str(tmp_path / "lm_head.spectra")
    sp.spectra_save(c, path)
    c2 = sp.spectra_load(path)
    h1 = hashlib.sha256(sp.spectra_export(c)).hexdigest()
    h2 = hashlib.sha256(sp.spectra_export(c2)).hexdigest()
    assert h1 == h2
    _same_products(c, c2, lin.K, M=1, seed=7)
