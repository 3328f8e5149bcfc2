"""The parity gate: the span-02 GPU test page's bound, rel-RMS below 1e-2
against the f64 reference, applied to every (row, head) output vector on its
own, so that one wrong key in one row cannot hide in the average over the
whole output.  A NaN anywhere fails."""
import numpy as np

import oracle

TOL = 1e-2


def per_head(got, ref):
    """(whole-output rel-RMS, worst per-(row, head) rel-RMS with NaN counted
    as inf, (row, head) of the worst)."""
    e = oracle.rel_rms_each(got, ref)
    e = np.where(np.isnan(e), np.inf, e)
    idx = np.unravel_index(int(np.argmax(e)), e.shape)
    return oracle.rel_rms(got, ref), float(e[idx]), tuple(int(i) for i in idx)


def passes(got, ref, tol=TOL):
    return per_head(got, ref)[1] < tol
