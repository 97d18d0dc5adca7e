"""Decode-step plans for a stack of decoder layers (host-side plumbing only).

A layer's seven projections run as four dependent phases: q/k/v share the
layer input, o reads the q output (it has the attention output's width),
gate/up share o's output, and down reads the gate output; the next layer's
q/k/v read down's output.  The attention, residual, normalization and
activation a real decoder applies between them are outside this library's
path: here each phase reads the previous projection's output directly, scaled
by a power of two (exact in fp16) that keeps the chain's magnitudes near 1.
Every product runs in the library's persistent decode-step kernel
(spectra_step_*); this module only builds the phase list.
"""
from __future__ import annotations

import math

QKV, O, GATE_UP, DOWN = "qkv", "o", "gate_up", "down"


def pow2_near(v: float) -> float:
    """The power of two nearest to v > 0 on a log scale."""
    return float(2.0 ** round(math.log2(v)))


def chain_scales(gains, rms_in: float = 1.0):
    """Input scales for a chain whose phase p multiplies the rms of its input
    by gains[p]: phase 0 takes 1.0, and phase p + 1 the power of two that
    brings the expected rms of phase p's output back near 1."""
    scales, rms = [1.0], rms_in
    for g in gains[:-1]:
        out = rms * g
        s = 1.0 / pow2_near(out)
        scales.append(s)
        rms = out * s
    return scales


def layer_phases(layers, x0, scales=None):
    """Phases of a decoder stack.

    layers: list of dicts with the keys q, k, v, o, gate, up, down, each a
    (Container, y tensor) pair.  x0: CUDA fp16 [K] input of the first q/k/v.
    scales: one input scale per phase (4 per layer), default 1.0.
    """
    phases = []
    for li, L in enumerate(layers):
        base = 4 * li
        groups = [(QKV, ("q", "k", "v"), -1 if li == 0 else base - 1),
                  (O, ("o",), base),
                  (GATE_UP, ("gate", "up"), base + 1),
                  (DOWN, ("down",), base + 2)]
        for kind, names, inp in groups:
            p = len(phases)
            phases.append({"kind": kind, "layer": li, "names": names,
                           "containers": [L[n][0] for n in names], "ys": [L[n][1] for n in names],
                           "input": inp, "x": x0 if inp < 0 else None,
                           "x_scale": 1.0 if scales is None else float(scales[p])})
    return phases
