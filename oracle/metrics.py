"""The pages' two measures, in fp64 -- TEST INFRASTRUCTURE ONLY (part of the oracle).

* Orthogonality (thelatestinai.com listing, Table 1 caption): ||O||_* / (sqrt(min(m,n)) ||O||_F) for a
  nonzero m x n matrix O; it equals 1 exactly when all singular values are equal.  The singular
  values come from LAPACK's SVD (numpy), used here as a library primitive.
* Effective rank (Figure 2 caption): exp(-sum_i p_i log p_i) as a fraction of the dimension, with
  p_i the normalised eigenvalues of a second moment (Table 1(a) applies it to the singular values of
  the matrix Y instead).
"""
from __future__ import annotations

import numpy as np


def orthogonality(O) -> float:
    O = np.asarray(O, dtype=np.float64)
    s = np.linalg.svd(O, compute_uv=False)
    fro = float(np.sqrt(np.sum(O * O)))
    if fro == 0.0:
        raise ValueError("orthogonality is defined for a nonzero matrix")
    return float(np.sum(s) / (np.sqrt(min(O.shape)) * fro))


def effective_rank(values) -> float:
    """exp(entropy of the normalised nonnegative values) / len(values)."""
    v = np.asarray(values, dtype=np.float64)
    if np.any(v < 0):
        raise ValueError("effective rank needs nonnegative values")
    p = v / v.sum()
    nz = p[p > 0]
    return float(np.exp(-np.sum(nz * np.log(nz))) / len(v))
