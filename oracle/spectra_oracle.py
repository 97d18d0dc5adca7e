"""CPU oracle for the SPECTRA sparse-precision dequant-GEMV path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the entry module
and the CPU-baseline leg of the benchmark may import this module.  The GPU
library never calls it, and it shares no code with the GPU library: it is
written from the method's description and from the container layout as the
library's public header states it in prose.

Method (SPECTRA page, "SPECTRA: Sparse-Precision Exact Channel Tensor
Reconstruction Architecture", abstract): channel saliency from the upstream
normalization gain, a fourth-moment kurtosis test (> 3.0) that routes
heavy-tailed input channels to exact floating point, and microscaled
Group-32 4-bit codes with bit-packed zero points for the Gaussian bulk.  The
page gives no formulas; the readings this oracle takes are:

  * kurtosis is the excess kurtosis m4/m2^2 - 3 with population moments of
    s = W[:, k] * gamma[k], flagged iff > 3.0 and m2 > 0;
  * flagged channels leave the 4-bit grid entirely (the bulk is compacted,
    ascending), and are kept as their original fp16 bits;
  * each group of 32 consecutive bulk channels of one output row is quantized
    asymmetrically over [min(0, min w), max(0, max w)] with 15 steps, scale
    rounded to fp16, integer zero point and codes by round-half-even;
  * the product is y = x W_hat^T, here evaluated in float64.

All floating-point work is IEEE binary64 (numpy float64) except the single
fp16 rounding of the scale, done by numpy's float64 -> float16 conversion
(round to nearest even).  No blocking or fusion beyond what the definition
states: column blocks in `channel_kurtosis` and row blocks in `matmul_ref`
only bound memory; every column's and every output's arithmetic is the plain
definition.

Parity status of each function (what pins it, in tests/test_oracle_pins.py):
  channel_kurtosis   closed forms (single spike, symmetric two-point,
                     Bernoulli), scipy.stats.kurtosis, exact gain scaling
  outlier_mask       threshold placement via the single-spike closed form
  permutation        invariants (bulk ascending, then flagged ascending)
  quantize_groups    exact round trip of grid-valued groups, all-zero and
                     one-signed groups, error bound, monotonicity; hand-valued
                     ties: codes and zero points round half to even ({0, 15,
                     2.5} -> code 2; {-6.5, 8.5} -> z 6, codes 0 and 14), and
                     so does the fp16 scale (1 + 2^-11 -> 1, 1 + 3*2^-11 ->
                     1 + 2^-9)
  pack / unpack      hand-written byte fixtures in tests/golden, round trip,
                     footprint closed form, outlier bits
  matmul_ref         pure-Python brute force on tiny shapes, one-hot inputs
  tolerance          hand-computed bounds on a 3 x 2 W_hat and two rows of x
                     (signs on both operands), and the 1e-6 floor
  embed_ref          grid-valued tables gather back bit-exact (bulk and
                     heavy-tailed channels), out-of-range ids give zero rows
  kv_quantize        grid-valued head vectors round-trip exactly; the same
                     groups through quantize_groups directly
  kv_attend_ref      pure-Python brute force (math.exp, explicit sums) on tiny
                     caches; one-token cache returns V; equal keys average V;
                     a two-token cache with hand-computed softmax weights
  kv_attend_tolerance  the same two-token cache: 1e-3 * p|V| + 1e-6 by hand
"""
from __future__ import annotations

import numpy as np

MAGIC = 0x31435053
VERSION = 1
HEADER_BYTES = 128
ALIGN = 256
GROUP = 32
KURTOSIS_THRESHOLD = 3.0


# ---------------------------------------------------------------------------
# Step 1: saliency and the kurtosis split
# ---------------------------------------------------------------------------
def channel_kurtosis(W16: np.ndarray, gamma16: np.ndarray, col_block: int = 256):
    """Excess kurtosis of each gain-scaled input channel.

    s[n] = W[n, k] * gamma[k] (binary64, exact); population moments about the
    mean.  Returns (kappa, m2) as float64 arrays of length K; kappa is NaN
    where m2 == 0 (a constant channel).
    """
    W16 = np.asarray(W16, dtype=np.float16)
    N, K = W16.shape
    g = np.asarray(gamma16, dtype=np.float16).astype(np.float64)
    kappa = np.empty(K, dtype=np.float64)
    m2_out = np.empty(K, dtype=np.float64)
    for k0 in range(0, K, col_block):
        k1 = min(K, k0 + col_block)
        S = W16[:, k0:k1].astype(np.float64) * g[k0:k1]
        mean = S.sum(axis=0) / N
        D2 = S - mean
        D2 *= D2
        m2 = D2.sum(axis=0) / N
        D2 *= D2
        m4 = D2.sum(axis=0) / N
        with np.errstate(divide="ignore", invalid="ignore"):
            kap = np.where(m2 > 0, m4 / (m2 * m2) - 3.0, np.nan)
        kappa[k0:k1] = kap
        m2_out[k0:k1] = m2
    return kappa, m2_out


def outlier_mask(W16, gamma16) -> np.ndarray:
    """Boolean [K]: True where the channel is heavy-tailed (kappa > 3.0, m2 > 0)."""
    kappa, m2 = channel_kurtosis(W16, gamma16)
    return (m2 > 0) & (np.nan_to_num(kappa, nan=-np.inf) > KURTOSIS_THRESHOLD)


# ---------------------------------------------------------------------------
# Step 2: order (compaction of the bulk)
# ---------------------------------------------------------------------------
def permutation(mask: np.ndarray) -> np.ndarray:
    """Bulk channels ascending, then heavy-tailed channels ascending (int32)."""
    mask = np.asarray(mask, dtype=bool)
    idx = np.arange(mask.size)
    return np.concatenate([idx[~mask], idx[mask]]).astype(np.int32)


# ---------------------------------------------------------------------------
# Step 3: Group-32 asymmetric 4-bit quantization
# ---------------------------------------------------------------------------
def quantize_groups(Wb: np.ndarray):
    """Quantize bulk rows.

    Wb: float64 [N][K_b] (bulk channels in bulk order).  Returns
    (q uint8 [N][G][32], z uint8 [N][G], s16 float16 [N][G]); padding members
    (bulk position >= K_b) carry q = z.
    """
    Wb = np.asarray(Wb, dtype=np.float64)
    N, K_b = Wb.shape
    G = -(-K_b // GROUP)
    pad = G * GROUP - K_b
    Wp = np.concatenate([Wb, np.zeros((N, pad))], axis=1).reshape(N, G, GROUP)
    real = (np.arange(G * GROUP) < K_b).reshape(G, GROUP)[None, :, :]

    lo = np.minimum(0.0, np.where(real, Wp, np.inf).min(axis=2))
    hi = np.maximum(0.0, np.where(real, Wp, -np.inf).max(axis=2))
    s = (hi - lo) / 15.0
    s16 = s.astype(np.float16)
    s16d = s16.astype(np.float64)
    nz = s16d > 0
    safe = np.where(nz, s16d, 1.0)
    z = np.where(nz, np.minimum(15.0, np.rint(-lo / safe)), 0.0)
    qf = np.rint(Wp / safe[:, :, None]) + z[:, :, None]
    qf = np.clip(qf, 0.0, 15.0)
    qf = np.where(nz[:, :, None], qf, 0.0)
    qf = np.where(real, qf, z[:, :, None])
    return qf.astype(np.uint8), z.astype(np.uint8), s16


def dequantize_groups(q, z, s16, K_b: int) -> np.ndarray:
    """w_hat = (q - z) * s16 in binary64, bulk order, padding dropped: [N][K_b]."""
    q = np.asarray(q, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    N, G, _ = q.shape
    return ((q - z[:, :, None]) * s[:, :, None]).reshape(N, G * GROUP)[:, :K_b]


# ---------------------------------------------------------------------------
# Container image (layout as written in the public header)
# ---------------------------------------------------------------------------
def _align(v: int) -> int:
    return (v + ALIGN - 1) // ALIGN * ALIGN


def section_sizes(K: int, N: int, n_out: int) -> dict:
    K_b = K - n_out
    G = -(-K_b // GROUP)
    return {
        "mask": 4 * (-(-K // 32)),
        "perm": 4 * K,
        "codes": 16 * N * G,
        "scales": 2 * N * G,
        "zeros": -(-(N * G) // 2),
        "outliers": 2 * N * n_out,
    }


def footprint(K: int, N: int, n_out: int) -> int:
    """Payload bytes: 4 + 16/32 + 4/32 bits per bulk weight (K_b rounded up to
    a multiple of 32) plus 16 bits per heavy-tailed weight."""
    K_b = K - n_out
    G = -(-K_b // GROUP)
    bulk_slots = N * G * GROUP
    bits = bulk_slots * 4 + (bulk_slots // 32) * 16 + (bulk_slots // 32) * 4 + N * n_out * 16
    # zero points pack two per byte: an odd group count leaves half a byte
    return -(-bits // 8)


def layout(K: int, N: int, n_out: int) -> dict:
    sz = section_sizes(K, N, n_out)
    off = {}
    pos = HEADER_BYTES
    for name in ("mask", "perm", "codes", "scales", "zeros", "outliers"):
        pos = _align(pos)
        off[name] = pos
        pos += sz[name]
    off["total"] = _align(pos)
    return off


def encode_codes(q: np.ndarray) -> np.ndarray:
    """q uint8 [N][G][32] -> uint32 words [N][G][4] per the member bit placement:
    member e sits in word e//8 at bit 16*(e%2) + 4*((e%8)//2)."""
    q = np.asarray(q, dtype=np.uint32)
    e = np.arange(GROUP)
    word = e // 8
    bit = 16 * (e % 2) + 4 * ((e % 8) // 2)
    N, G, _ = q.shape
    out = np.zeros((N, G, 4), dtype=np.uint32)
    for m in range(GROUP):
        out[:, :, word[m]] |= q[:, :, m] << np.uint32(bit[m])
    return out


def decode_codes(words: np.ndarray) -> np.ndarray:
    """Inverse of encode_codes: uint32 [N][G][4] -> uint8 [N][G][32]."""
    words = np.asarray(words, dtype=np.uint32)
    e = np.arange(GROUP)
    word = e // 8
    bit = 16 * (e % 2) + 4 * ((e % 8) // 2)
    N, G, _ = words.shape
    q = np.empty((N, G, GROUP), dtype=np.uint8)
    for m in range(GROUP):
        q[:, :, m] = (words[:, :, word[m]] >> np.uint32(bit[m])) & np.uint32(0xF)
    return q


def pack(W16: np.ndarray, gamma16: np.ndarray, mask: np.ndarray | None = None,
         row_block: int = 8192) -> bytes:
    """Build the full container image for W (fp16 [N][K]) and gamma (fp16 [K]).

    `mask` overrides the kurtosis decision (used only to re-derive the rest of
    the image when a channel sits within rounding of the threshold).
    """
    W16 = np.ascontiguousarray(W16, dtype=np.float16)
    gamma16 = np.asarray(gamma16, dtype=np.float16)
    N, K = W16.shape
    if not (np.isfinite(W16).all() and np.isfinite(gamma16).all()):
        raise ValueError("non-finite input")
    if mask is None:
        mask = outlier_mask(W16, gamma16)
    mask = np.asarray(mask, dtype=bool)
    perm = permutation(mask)
    n_out = int(mask.sum())
    K_b = K - n_out
    G = -(-K_b // GROUP)

    O = W16[:, perm[K_b:]]
    off = layout(K, N, n_out)
    img = bytearray(off["total"])
    hdr = np.zeros(HEADER_BYTES // 8, dtype=np.uint64)
    hdr[0] = np.uint64(MAGIC | (VERSION << 32))
    hdr[1:6] = [K, N, K_b, G, n_out]
    hdr[6:13] = [off["mask"], off["perm"], off["codes"], off["scales"], off["zeros"],
                 off["outliers"], off["total"]]
    img[0:HEADER_BYTES] = hdr.astype("<u8").tobytes()

    mwords = np.zeros(-(-K // 32), dtype=np.uint32)
    for k in np.nonzero(mask)[0]:
        mwords[k // 32] |= np.uint32(1) << np.uint32(k % 32)
    _put(img, off["mask"], mwords.astype("<u4"))
    _put(img, off["perm"], perm.astype("<i4"))
    # Groups are independent, so rows are quantized in blocks only to bound memory.
    zf = np.zeros(N * G + (N * G) % 2, dtype=np.uint8)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        q, z, s16 = quantize_groups(W16[r0:r1][:, perm[:K_b]].astype(np.float64))
        _put(img, off["codes"] + 16 * r0 * G, encode_codes(q).astype("<u4"))
        _put(img, off["scales"] + 2 * r0 * G, s16.astype("<f2"))
        zf[r0 * G:r1 * G] = z.reshape(-1)
    _put(img, off["zeros"], (zf[0::2] | (zf[1::2] << 4)).astype(np.uint8))
    _put(img, off["outliers"], O.astype("<f2"))
    return bytes(img)


def _put(img: bytearray, pos: int, arr: np.ndarray):
    b = np.ascontiguousarray(arr).tobytes()
    img[pos:pos + len(b)] = b


def unpack(img: bytes) -> dict:
    """Parse a container image back into its fields and the reconstruction.

    Returns dict with K, N, K_b, G, n_out, mask, perm, q, z, s16, O (fp16) and
    W_hat (float64 [N][K] in original channel order: bulk entries are
    (q - z) * s16, heavy-tailed entries are O).
    """
    hdr = np.frombuffer(img, dtype="<u8", count=HEADER_BYTES // 8)
    if int(hdr[0]) & 0xFFFFFFFF != MAGIC or int(hdr[0]) >> 32 != VERSION:
        raise ValueError("bad magic/version")
    K, N, K_b, G, n_out = (int(v) for v in hdr[1:6])
    o_mask, o_perm, o_codes, o_scales, o_zeros, o_out, total = (int(v) for v in hdr[6:13])
    mw = np.frombuffer(img, "<u4", -(-K // 32), o_mask)
    mask = ((mw[np.arange(K) // 32] >> (np.arange(K) % 32).astype(np.uint32)) & 1).astype(bool)
    perm = np.frombuffer(img, "<i4", K, o_perm).astype(np.int64)
    words = np.frombuffer(img, "<u4", N * G * 4, o_codes).reshape(N, G, 4)
    q = decode_codes(words)
    s16 = np.frombuffer(img, "<f2", N * G, o_scales).reshape(N, G)
    zb = np.frombuffer(img, np.uint8, -(-(N * G) // 2), o_zeros)
    zf = np.empty(zb.size * 2, dtype=np.uint8)
    zf[0::2] = zb & 0xF
    zf[1::2] = zb >> 4
    z = zf[:N * G].reshape(N, G)
    O = np.frombuffer(img, "<f2", N * n_out, o_out).reshape(N, n_out)
    W_hat = np.empty((N, K), dtype=np.float64)
    W_hat[:, perm[:K_b]] = dequantize_groups(q, z, s16, K_b)
    W_hat[:, perm[K_b:]] = O.astype(np.float64)
    return dict(K=K, N=N, K_b=K_b, G=G, n_out=n_out, mask=mask, perm=perm, q=q, z=z,
                s16=s16, O=O, W_hat=W_hat, total=total,
                offsets=dict(mask=o_mask, perm=o_perm, codes=o_codes, scales=o_scales,
                             zeros=o_zeros, outliers=o_out))


# ---------------------------------------------------------------------------
# Step 5: the product and its accuracy contract
# ---------------------------------------------------------------------------
def matmul_ref(W_hat: np.ndarray, x16: np.ndarray, row_block: int = 8192) -> np.ndarray:
    """y_ref = x W_hat^T in binary64.  x: fp16 [M][K]; returns float64 [M][N]."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    N = W_hat.shape[0]
    y = np.empty((x.shape[0], N), dtype=np.float64)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        y[:, r0:r1] = x @ np.asarray(W_hat[r0:r1], dtype=np.float64).T
    return y


def tolerance(W_hat: np.ndarray, x16: np.ndarray, row_block: int = 8192) -> np.ndarray:
    """Per-element bound 1e-3 * (|W_hat| |x|^T)[m][n] + 1e-6."""
    ax = np.abs(np.asarray(x16, dtype=np.float16).astype(np.float64))
    N = W_hat.shape[0]
    t = np.empty((ax.shape[0], N), dtype=np.float64)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        t[:, r0:r1] = ax @ np.abs(np.asarray(W_hat[r0:r1], dtype=np.float64)).T
    return 1e-3 * t + 1e-6


def reconstruct_rows(img: bytes, rows: np.ndarray) -> np.ndarray:
    """W_hat restricted to the given output rows (float64 [len(rows)][K]),
    for sampled checks on shapes too large to reconstruct whole."""
    hdr = np.frombuffer(img, dtype="<u8", count=HEADER_BYTES // 8)
    K, N, K_b, G, n_out = (int(v) for v in hdr[1:6])
    o_mask, o_perm, o_codes, o_scales, o_zeros, o_out, total = (int(v) for v in hdr[6:13])
    rows = np.asarray(rows, dtype=np.int64)
    perm = np.frombuffer(img, "<i4", K, o_perm).astype(np.int64)
    words_all = np.frombuffer(img, "<u4", N * G * 4, o_codes).reshape(N, G, 4)
    q = decode_codes(words_all[rows])
    s16 = np.frombuffer(img, "<f2", N * G, o_scales).reshape(N, G)[rows]
    zb = np.frombuffer(img, np.uint8, -(-(N * G) // 2), o_zeros)
    flat = rows[:, None] * G + np.arange(G)[None, :]
    z = ((zb[flat >> 1] >> ((flat & 1) * 4).astype(np.uint8)) & 0xF).astype(np.uint8)
    O = np.frombuffer(img, "<f2", N * n_out, o_out).reshape(N, n_out)[rows]
    W_hat = np.empty((rows.size, K), dtype=np.float64)
    W_hat[:, perm[:K_b]] = dequantize_groups(q, z, s16, K_b)
    W_hat[:, perm[K_b:]] = O.astype(np.float64)
    return W_hat


# ---------------------------------------------------------------------------
# Step 6: row gather (the fused embedding)
# ---------------------------------------------------------------------------
def embed_ref(img: bytes, ids) -> np.ndarray:
    """Rows W_hat[ids[i]] in channel order, each entry rounded once to fp16
    (round to nearest even); an id outside [0, N) gives a row of zeros.

    SPECTRA page ("SPECTRA: Sparse-Precision Exact Channel Tensor
    Reconstruction Architecture", abstract and highlight 5, the fused
    embedding): a vocabulary table is kept in the same Group-32 4-bit format
    and the rows a forward pass needs are gathered and dequantized on the fly.
    Reading: the table E [V][D] is packed as W with N = V rows and K = D
    channels, and a gathered row is that row of W_hat (bulk entries
    (q - z) * s16, heavy-tailed entries their fp16 bits).  The bulk value is
    exact in binary64, so one rounding to fp16 is the only one.
    """
    hdr = np.frombuffer(img, dtype="<u8", count=HEADER_BYTES // 8)
    K, N = int(hdr[1]), int(hdr[2])
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    ok = (ids >= 0) & (ids < N)
    out = np.zeros((ids.size, K), dtype=np.float16)
    if ok.any():
        out[ok] = reconstruct_rows(img, ids[ok]).astype(np.float16)
    return out


# ---------------------------------------------------------------------------
# Step 7: the Group-32 4-bit KV cache (quantize on append, attend)
# ---------------------------------------------------------------------------
def kv_quantize(x16: np.ndarray):
    """Quantize key or value vectors on append.

    SPECTRA page ("SPECTRA: Sparse-Precision Exact Channel Tensor
    Reconstruction Architecture", abstract): the key-value cache is kept in
    microscaled Group-32 4-bit form.  Reading: each head's vector of D = 32G
    channels is split into G groups of 32 consecutive channels and quantized
    exactly as a bulk weight group (same range, scale, zero point and codes;
    no heavy-tailed split, which the page states for weights only).
    x16: fp16 [T][H][D].  Returns (q uint8 [T][H][G][32], z uint8 [T][H][G],
    s16 float16 [T][H][G]).
    """
    x = np.asarray(x16, dtype=np.float16)
    T, H, D = x.shape
    if D % GROUP:
        raise ValueError("head dimension must be a multiple of 32")
    q, z, s16 = quantize_groups(x.reshape(T * H, D).astype(np.float64))
    G = D // GROUP
    return q.reshape(T, H, G, GROUP), z.reshape(T, H, G), s16.reshape(T, H, G)


def kv_dequantize(q, z, s16) -> np.ndarray:
    """(q - z) * s16 in binary64: float64 [T][H][D]."""
    q = np.asarray(q)
    T, H, G, _ = q.shape
    w = dequantize_groups(q.reshape(T * H, G, GROUP), np.asarray(z).reshape(T * H, G),
                          np.asarray(s16).reshape(T * H, G), G * GROUP)
    return w.reshape(T, H, G * GROUP)


def kv_attend_ref(q16: np.ndarray, K_hat: np.ndarray, V_hat: np.ndarray) -> np.ndarray:
    """Decode-step attention over the dequantized cache, in binary64.

    q16: fp16 [Hq][D] (one query per head); K_hat, V_hat: float64 [L][Hkv][D]
    with Hq a multiple of Hkv (query head h reads cache head h // (Hq/Hkv)).
    out[h] = softmax(q_h K_hat^T / sqrt(D)) V_hat, the plain definition
    (max subtracted before exp only to keep exp finite).
    """
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    Hq, D = q.shape
    L, Hkv, _ = K_hat.shape
    rep = Hq // Hkv
    out = np.empty((Hq, D), dtype=np.float64)
    for h in range(Hq):
        kv = h // rep
        s = K_hat[:, kv, :] @ q[h] / np.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ V_hat[:, kv, :]
    return out


def kv_attend_tolerance(q16: np.ndarray, K_hat: np.ndarray, V_hat: np.ndarray) -> np.ndarray:
    """Per-element bound 1e-3 * (sum_t p_t |V_hat[t]|)[h][d] + 1e-6: the GEMM
    bound with the weights read as V_hat and the input as the softmax
    weights (fp16 output rounding spends 2^-11 of it)."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    Hq, D = q.shape
    L, Hkv, _ = K_hat.shape
    rep = Hq // Hkv
    t = np.empty((Hq, D), dtype=np.float64)
    for h in range(Hq):
        kv = h // rep
        s = K_hat[:, kv, :] @ q[h] / np.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        t[h] = p @ np.abs(V_hat[:, kv, :])
    return 1e-3 * t + 1e-6
