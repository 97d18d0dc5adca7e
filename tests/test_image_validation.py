"""Host-side checks of container images (spectra_validate_image): no device is
touched, so these run on the CPU.  Images come from the oracle's packer; each
corruption must be rejected with SPECTRA_E_INVAL."""
import struct

import numpy as np
import pytest

from dequant_gemv_spectra_amd import synth
from oracle import spectra_oracle as O


def _sp():
    from dequant_gemv_spectra_amd import spectra
    return spectra


def _image(N, K, n_out, seed):
    W, g, _ = synth.random_case(N, K, n_out, seed)
    return O.pack(W, g)


def _rejects(img, what):
    sp = _sp()
    with pytest.raises(sp.SpectraError) as ei:
        sp.spectra_validate_image(bytes(img))
    assert ei.value.status == sp.SPECTRA_E_INVAL, what
    return str(ei.value)


@pytest.mark.parametrize("N,K,n_out,seed", [(1, 1, 0, 0), (3, 31, 1, 2), (17, 33, 2, 3),
                                            (9, 97, 5, 6), (100, 130, 129, 7), (33, 300, 0, 8)])
def test_oracle_images_are_valid(N, K, n_out, seed):
    _sp().spectra_validate_image(_image(N, K, n_out, seed))


def test_all_heavy_tailed_image_is_valid():
    W = np.zeros((9, 5), np.float16)
    for k in range(5):
        W[k, k] = 1.0 + k
    _sp().spectra_validate_image(O.pack(W, np.ones(5, np.float16)))


def _field(img, i):
    return struct.unpack_from("<Q", img, 8 * i)[0]


def _set_field(img, i, v):
    b = bytearray(img)
    struct.pack_into("<Q", b, 8 * i, v)
    return b


def test_header_corruptions_rejected():
    img = _image(40, 200, 6, 1)
    _rejects(img[:100], "shorter than the header")
    b = bytearray(img)
    b[0] ^= 0x01
    assert "magic" in _rejects(b, "magic")
    assert "version" in _rejects(_set_field(img, 0, (_field(img, 0) & 0xFFFFFFFF) | (2 << 32)), "version")
    _rejects(img[:-1], "truncated")
    _rejects(img + b"\0", "one byte too long")
    _rejects(_set_field(img, 1, 0), "K = 0")
    _rejects(_set_field(img, 3, _field(img, 3) + 1), "K_b")
    _rejects(_set_field(img, 4, _field(img, 4) + 1), "G")
    _rejects(_set_field(img, 5, 201), "n_out > K")
    for i in range(6, 13):
        _rejects(_set_field(img, i, _field(img, i) + 256), f"offset field {i}")


def test_mask_and_perm_corruptions_rejected():
    img = _image(40, 200, 6, 2)
    u = O.unpack(img)
    off = u["offsets"]
    # a bulk channel flagged: n_out no longer matches the mask
    k = int(u["perm"][0])
    b = bytearray(img)
    b[off["mask"] + 4 * (k // 32) + (k % 32) // 8] ^= 1 << (k % 8)
    assert "n_out" in _rejects(b, "extra mask bit")
    # a bit past K in the last mask word (K = 200: bits 8..31 of word 6)
    b = bytearray(img)
    b[off["mask"] + 4 * 6 + 3] |= 0x80
    _rejects(b, "mask bit past K")
    # two bulk perm entries swapped
    b = bytearray(img)
    p = np.frombuffer(img, "<i4", 200, off["perm"]).copy()
    p[[3, 4]] = p[[4, 3]]
    b[off["perm"]:off["perm"] + 800] = p.tobytes()
    assert "perm" in _rejects(b, "perm order")


def test_payload_corruptions_rejected():
    img = _image(41, 97, 5, 3)  # N*G = 41*3, odd: one unused zero nibble
    u = O.unpack(img)
    off = u["offsets"]
    N, G, n_out = u["N"], u["G"], u["n_out"]
    assert n_out > 0 and (N * G) % 2 == 1
    for bits, what in [(0x7E00, "NaN"), (0x7C00, "inf"), (0x8001, "negative")]:
        b = bytearray(img)
        struct.pack_into("<H", b, off["scales"] + 2 * 17, bits)
        assert "scale" in _rejects(b, f"scale {what}")
    b = bytearray(img)
    struct.pack_into("<H", b, off["outliers"] + 2 * (N * n_out - 1), 0xFC00)
    assert "heavy-tailed" in _rejects(b, "outlier -inf")
    b = bytearray(img)
    b[off["zeros"] + (N * G) // 2] |= 0x50
    assert "nibble" in _rejects(b, "unused zero nibble")
    # the codes section has no invalid values: any bits are a valid code
    b = bytearray(img)
    b[off["codes"] + 5] ^= 0xFF
    _sp().spectra_validate_image(bytes(b))
