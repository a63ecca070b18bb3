"""Writes vq_codebook_256x8_cos.txt: the k-means fixture codebook
(vq_codebook_256x8.txt) after the oracle's cosine refinement (NSNQuant page,
Metodologia sec. 3: the k-means codebook is refined to minimise the cosine
distance between vectors and their quantised versions).

Recipe: the same 2^18 samples of seed 4 as the k-means fixture, 20 passes.
Run from the repository root:  python tests/golden/make_vq_codebook_cos.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from calibration_free_kv_amd import synth  # noqa: E402

N = 1 << 18
SEED = 4
PASSES = 20

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    cb0 = np.loadtxt(os.path.join(here, "vq_codebook_256x8.txt"), dtype=np.float32).reshape(256, 8)
    s = synth.gaussian_samples(SEED, N)
    cb, mc = O.cosine_refine(s, cb0, passes=PASSES)
    with open(os.path.join(here, "vq_codebook_256x8_cos.txt"), "w") as f:
        f.write("# cosine-refined codebook, 256 x 8, float32; from vq_codebook_256x8.txt, %d samples, seed %d, "
                "%d passes, mean cosine %.6f -> %.6f\n" % (N, SEED, PASSES, mc[0], mc[-1]))
        for row in cb.astype(np.float32):
            f.write(" ".join("%.9g" % v for v in row) + "\n")
    print("mean cosine per pass", np.array2string(mc, precision=6))
