"""Writes cfg3_image_sha256.txt: the SHA-256 of the oracle's container image
for every linear of the 36-layer 4B-class decoder workload (hidden 2560,
MLP 9728; q/k/v/o/gate/up/down per layer, seeded synthetic weights).

    python tests/golden/make_cfg3_image_hashes.py

Calls only the CPU oracle (oracle/spectra_oracle.py: kurtosis split, Group-32
quantization, container image) and the seeded input generators; nothing here
runs the GPU path.  Each line: name, N, K, the oracle's heavy-tailed channel
count, the number of channels whose kurtosis lies within 1e-9 of the 3.0
threshold (where two mask decisions are valid; none in this workload), the
image size in bytes and its SHA-256.  About 6 minutes on 8 cores.
"""
import hashlib
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from dequant_gemv_spectra_amd import synth  # noqa: E402
from oracle import spectra_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cfg3_image_sha256.txt")


def main():
    wl = synth.workload(3)
    lines = ["# name N K n_out borderline bytes sha256 (oracle images, 4B-class decoder workload)"]
    t0 = time.time()
    for lin in wl.linears:
        W, g = synth.weights(lin, 3), synth.gamma(lin, 3)
        kap, m2 = O.channel_kurtosis(W, g)
        border = int(((m2 > 0) & (np.abs(np.nan_to_num(kap, nan=0.0) - 3.0) < 1e-9)).sum())
        mask = O.outlier_mask(W, g)
        img = O.pack(W, g, mask)
        lines.append(f"{lin.name} {lin.N} {lin.K} {int(mask.sum())} {border} {len(img)} "
                     f"{hashlib.sha256(img).hexdigest()}")
        if lin.name.endswith("down"):
            print(f"{lin.name}: {time.time() - t0:.0f}s", flush=True)
    with open(OUT, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {OUT}: {len(lines) - 1} linears")


if __name__ == "__main__":
    main()
