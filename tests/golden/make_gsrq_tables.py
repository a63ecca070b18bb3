"""Writes gsrq_tables_256x32.txt: the two stages of the GSRQ reading (GSRQ
page: gain-shape k-means inside a residual quantisation pipeline), trained by
the oracle on N(0, I_32) samples, as the NSN codebook is trained on standard
normal samples (NSNQuant page, Metodologia sec. 3).

Recipe: 2^16 samples of seed 7 (32-dim), GSKM with 256 shapes per stage
started from 256 distinct samples (seeds 8 and 9), 20 passes; 16 gain levels
per stage by Lloyd's algorithm on the best projections.  File layout: stage 1
shapes (256 lines of 32), stage 1 levels (one line of 16), stage 2 shapes,
stage 2 levels, all float32.
Run from the repository root:  python tests/golden/make_gsrq_tables.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from calibration_free_kv_amd import synth  # noqa: E402

N = 1 << 16
M = 32
K = 256
PASSES = 20

if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    s = synth.gaussian_samples(7, N, dim=M)
    tab = O.gsrq_train(s, [synth.kmeans_init(7, N, K), synth.kmeans_init(8, N, K)], passes=PASSES)
    with open(os.path.join(here, "gsrq_tables_256x32.txt"), "w") as f:
        f.write("# GSRQ tables: stage 1 shapes 256 x 32, levels 16; stage 2 shapes 256 x 32, levels 16; float32; "
                "%d samples, seed 7, %d passes, mean best projection %.6f -> %.6f (stage 1), %.6f -> %.6f "
                "(stage 2)\n" % (N, PASSES, tab["objective1"][0], tab["objective1"][-1], tab["objective2"][0],
                                 tab["objective2"][-1]))
        for k in (1, 2):
            for row in tab["S%d" % k].astype(np.float32):
                f.write(" ".join("%.9g" % v for v in row) + "\n")
            f.write(" ".join("%.9g" % v for v in tab["G%d" % k].astype(np.float32)) + "\n")
    print("objective per pass", tab["objective1"], tab["objective2"])
