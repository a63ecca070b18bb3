"""Helpers for the GPU parity tests (comparison only; no method arithmetic)."""
import numpy as np
import pytest
import torch

import oracle as O

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def unpack_np(codes, bits, d=128):
    """LSB-first records [..., 16*bits] -> indices [..., d] (layout spec, vectorised)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    b = np.unpackbits(codes, axis=-1, bitorder="little").reshape(codes.shape[:-1] + (d, bits))
    return (b.astype(np.int64) << np.arange(bits)).sum(-1)


def to_np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def check_codes(x, signs, bits, gpu_codes, gpu_norms, where=None, label=""):
    """Compare GPU codes/norms of vectors x [B,H,T,d] (or the subset `where` =
    (b_idx, h_idx, t_idx) arrays) against the oracle.  Index mismatches are
    allowed only at coordinates within 1e-5 of a threshold; returns counts."""
    B, H, T, d = x.shape
    if where is None:
        bb, hh, tt = [a.ravel() for a in np.meshgrid(np.arange(B), np.arange(H), np.arange(T), indexing="ij")]
    else:
        bb, hh, tt = where
    gi = unpack_np(gpu_codes[bb, hh, tt], bits)
    gn = gpu_norms[bb, hh, tt]
    mism = flagged = 0
    for h in np.unique(hh):
        sel = hh == h
        xs = x[bb[sel], h, tt[sel]][None, None]
        ref = O.quantize(xs, signs[h:h + 1], bits)
        oi = ref["idx"][0, 0]
        fl = ref["flags"][0, 0].astype(bool)
        bad = oi != gi[sel]
        assert not np.any(bad & ~fl), "%s: %d code mismatches outside the 1e-5 band (head %d)" % (
            label, int(np.sum(bad & ~fl)), h)
        mism += int(np.sum(bad))
        flagged += int(np.sum(fl))
        on = ref["norms"][0, 0]
        np.testing.assert_allclose(gn[sel], on, rtol=1e-5, atol=1e-30, err_msg=label + " norms")
    return dict(mismatch_at_boundary=mism, flagged=flagged, compared=int(gi.size))
