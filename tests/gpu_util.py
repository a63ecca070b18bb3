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


def boundary_mismatches(gi, ref, t, label=""):
    """Validity of GPU indices gi [..., d] against the oracle's quantisation
    `ref` (a dict with idx, flags and the rotated coordinates y) and the
    thresholds t it used.  Equal except at flagged coordinates (within 1e-5
    of a threshold); there the GPU may hold only the neighbouring cell across
    that threshold.  Returns (mismatches, flagged)."""
    oi, fl, y = ref["idx"], ref["flags"].astype(bool), ref["y"]
    t = np.asarray(t, np.float64)
    mism = gi != oi
    assert not np.any(mism & ~fl), "%s: %d code mismatches outside the 1e-5 band" % (label, int(np.sum(mism & ~fl)))
    if mism.any():
        g, o = gi[mism].astype(np.int64), oi[mism].astype(np.int64)
        assert np.all(np.abs(g - o) == 1), label + ": a flagged coordinate moved by more than one cell"
        near = np.abs(y[mism] - t[np.minimum(g, o)])
        assert near.max() < O.BAND, (label, "mismatch not at the threshold between the two cells", near.max())
    return int(mism.sum()), int(fl.sum())


def bound_mismatches(mism, flagged, label=""):
    """The GPU's rotated coordinates carry fp32 rounding (~1e-6), so it can
    disagree on only a fraction of the flagged (1e-5 band) decisions."""
    assert mism <= flagged // 2 + 2, (label, "too many boundary mismatches", mism, flagged)


def check_codes(x, signs, bits, gpu_codes, gpu_norms, where=None, label=""):
    """Compare GPU codes/norms of vectors x [B,H,T,d] (or the subset `where` =
    (b_idx, h_idx, t_idx) arrays) against the oracle.  Index mismatches are
    allowed only at coordinates within 1e-5 of a threshold, only to the
    neighbouring cell, and only on a bounded share of them; returns counts."""
    B, H, T, d = x.shape
    if where is None:
        bb, hh, tt = [a.ravel() for a in np.meshgrid(np.arange(B), np.arange(H), np.arange(T), indexing="ij")]
    else:
        bb, hh, tt = where
    gi = unpack_np(gpu_codes[bb, hh, tt], bits)
    gn = gpu_norms[bb, hh, tt]
    _, t = O.tables_f32(bits)
    mism = flagged = 0
    for h in np.unique(hh):
        sel = hh == h
        xs = x[bb[sel], h, tt[sel]][None, None]
        ref = O.quantize(xs, signs[h:h + 1], bits, want_y=True)
        m, f = boundary_mismatches(gi[sel], {k: v[0, 0] for k, v in ref.items()}, t, "%s head %d" % (label, h))
        mism += m
        flagged += f
        on = ref["norms"][0, 0]
        np.testing.assert_allclose(gn[sel], on, rtol=1e-5, atol=1e-30, err_msg=label + " norms")
    bound_mismatches(mism, flagged, label)
    return dict(mismatch_at_boundary=mism, flagged=flagged, compared=int(gi.size))
