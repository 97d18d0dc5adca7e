"""Seeded synthetic inputs for the SPECTRA dequant-GEMV path.

This module draws weights, norm gains and activations only. It holds none of
the method's arithmetic (no kurtosis, no quantization, no packing), so both the
CPU oracle and the GPU path can take their inputs from it.

Workload shapes follow the five layer configurations the path is measured on:
a single 2048x2048 linear; the seven linears of a 1.5B-class decoder layer
(hidden 1536, 12 query / 2 KV heads of dim 128, MLP 8960); 36 layers of a
4B-class decoder (hidden 2560, MLP 9728; 32 query / 8 KV heads of dim 128 is
this module's reading of the attention widths); a 131072x3072 LM head; and a
28672x8192 MLP projection swept over M.

Value recipe (the SPECTRA page, abstract, describes heavy-tailed input
channels inside an otherwise Gaussian bulk; the numbers below are the
workload definitions):
  * W[n, k] ~ N(0, 0.02^2), drawn in float32 and rounded to fp16 (RNE);
  * round(f*K) input channels, chosen without replacement, have their whole
    column replaced by Student-t(df=3) * 0.2, drawn in float64, rounded to fp16;
  * gamma[k] ~ U(0.5, 1.5) rounded to fp16;
  * x[m, k] ~ N(0, 1) rounded to fp16.

Every draw comes from numpy's PCG64 seeded by a SeedSequence whose entropy
is (config id, layer, linear id, role[, row block]), so a matrix does not
depend on which other matrices were drawn, nor on the number of threads used.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

ROW_BLOCK = 4096  # rows drawn per independent stream (parallel generation)

_ROLE_W, _ROLE_COLS, _ROLE_T, _ROLE_GAMMA, _ROLE_X, _ROLE_FRAC = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Linear:
    """One linear layer y = x W^T with W of shape [N][K]."""
    name: str
    N: int
    K: int
    n_out: int          # number of heavy-tailed input channels planted
    layer: int = 0
    lin_id: int = 0


@dataclass
class Workload:
    name: str
    cfg_id: int
    linears: list = field(default_factory=list)
    Ms: tuple = (1,)
    description: str = ""


def _n_out(frac: float, K: int) -> int:
    return int(round(frac * K))


def _decoder_layer(cfg_id, layer, hidden, mlp, q_heads, kv_heads, head_dim, frac):
    q = q_heads * head_dim
    kv = kv_heads * head_dim
    shapes = [("q", q, hidden), ("k", kv, hidden), ("v", kv, hidden),
              ("o", hidden, q), ("gate", mlp, hidden), ("up", mlp, hidden),
              ("down", hidden, mlp)]
    return [Linear(f"L{layer}.{nm}", N, K, _n_out(frac, K), layer, i)
            for i, (nm, N, K) in enumerate(shapes)]


def layer_outlier_fraction(cfg_id: int, layer: int) -> float:
    """Per-layer heavy-tailed fraction f ~ U(0.5 %, 2 %) for the 4B-class stack."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, layer, 0, _ROLE_FRAC])))
    return float(rng.uniform(0.005, 0.02))


def workload(cfg_id: int, layers: int | None = None) -> Workload:
    """The five measured layer configurations (1-based ids)."""
    if cfg_id == 1:
        return Workload("linear-2048x2048", 1, [Linear("W", 2048, 2048, 16)], (1,),
                        "single linear K=2048 N=2048, 16 heavy-tailed channels (0.8 %)")
    if cfg_id == 2:
        return Workload("decoder-1.5B-layer", 2,
                        _decoder_layer(2, 0, 1536, 8960, 12, 2, 128, 0.01), (1,),
                        "1.5B-class decoder layer q/k/v/o/gate/up/down, 1 % heavy-tailed")
    if cfg_id == 3:
        nl = 36 if layers is None else layers
        lins = []
        for l in range(nl):
            lins += _decoder_layer(3, l, 2560, 9728, 32, 8, 128, layer_outlier_fraction(3, l))
        return Workload("decoder-4B-36-layers", 3, lins, (1,),
                        "4B-class decoder stack, 36 layers x 7 linears, f ~ U(0.5 %, 2 %) per layer")
    if cfg_id == 4:
        return Workload("lm-head-131072x3072", 4, [Linear("lm_head", 131072, 3072, 31)], (1, 4),
                        "LM head N=131072 K=3072, 1 % heavy-tailed")
    if cfg_id == 5:
        return Workload("mlp-28672x8192", 5, [Linear("mlp", 28672, 8192, 82)],
                        (1, 2, 4, 8, 16, 32, 64, 128),
                        "MLP projection N=28672 K=8192 swept over M, 1 % heavy-tailed")
    raise ValueError(f"unknown config {cfg_id}")


def _rng(*entropy) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def _fill_block(W, r0, r1, seed_key, std):
    rng = _rng(*seed_key, r0 // ROW_BLOCK)
    blk = rng.standard_normal((r1 - r0, W.shape[1]), dtype=np.float32)
    blk *= np.float32(std)
    W[r0:r1] = blk.astype(np.float16)


def outlier_channels(lin: Linear, cfg_id: int) -> np.ndarray:
    """Indices of the planted heavy-tailed input channels (sorted)."""
    rng = _rng(cfg_id, lin.layer, lin.lin_id, _ROLE_COLS)
    return np.sort(rng.choice(lin.K, size=lin.n_out, replace=False)).astype(np.int64)


def weights(lin: Linear, cfg_id: int, threads: int | None = None) -> np.ndarray:
    """fp16 W [N][K] for one linear (row blocks drawn in parallel, deterministically)."""
    W = np.empty((lin.N, lin.K), dtype=np.float16)
    key = (cfg_id, lin.layer, lin.lin_id, _ROLE_W)
    blocks = [(r, min(r + ROW_BLOCK, lin.N)) for r in range(0, lin.N, ROW_BLOCK)]
    nthr = threads or min(16, os.cpu_count() or 1)
    if len(blocks) == 1 or nthr == 1:
        for r0, r1 in blocks:
            _fill_block(W, r0, r1, key, 0.02)
    else:
        with _cf.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(lambda b: _fill_block(W, b[0], b[1], key, 0.02), blocks))
    cols = outlier_channels(lin, cfg_id)
    if cols.size:
        rng = _rng(cfg_id, lin.layer, lin.lin_id, _ROLE_T)
        t = rng.standard_t(3.0, size=(lin.N, cols.size)) * 0.2
        W[:, cols] = t.astype(np.float16)
    return W


def gamma(lin: Linear, cfg_id: int) -> np.ndarray:
    rng = _rng(cfg_id, lin.layer, lin.lin_id, _ROLE_GAMMA)
    return rng.uniform(0.5, 1.5, size=lin.K).astype(np.float16)


def activations(lin: Linear, cfg_id: int, M: int, salt: int = 0) -> np.ndarray:
    rng = _rng(cfg_id, lin.layer, lin.lin_id, _ROLE_X, M, salt)
    return rng.standard_normal((M, lin.K)).astype(np.float16)


def random_case(N: int, K: int, n_out: int, seed: int, M: int = 1, std: float = 0.02):
    """A small arbitrary-shape case: (W, gamma, x) drawn with the same recipe."""
    lin = Linear("case", N, K, min(n_out, K), layer=seed, lin_id=N * 7919 + K)
    cfg = 1000 + seed
    return weights(lin, cfg, threads=1), gamma(lin, cfg), activations(lin, cfg, M)
