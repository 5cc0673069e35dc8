"""Block-diagonal Hadamard rotation (SAW-INT4, section 2: the vector is cut into
blocks of size h and each block gets its own Hadamard transform; KV4-RL,
"Methodology in Plain English": keys are stored rotated and queries are rotated
to match, which leaves q.k unchanged).

Readings where the pages are silent: the Hadamard matrix is Sylvester's
(natural order), there is no random sign diagonal (the method is described as
calibration-free), and the transform is normalised by 1/sqrt(h) so that it is
orthogonal.

Two forms are given:

* ``rotate_f64`` -- the mathematical definition, a dense fp64 matrix product;
* ``fwht_f32``  -- the fp32 evaluation that feeds the quantizer.  Its operation
  order is fixed so that integer codes derived from it are reproducible:
  butterfly stages with strides 1, 2, 4, ..., h/2 in that order, each pair
  (a, b) -> (a + b, a - b) rounded to fp32, then one fp32 multiply by the fp32
  value nearest to 1/sqrt(h).

Pinned by tests: H.H^T = h.I, equality with scipy.linalg.hadamard, q.k
preservation, h = 1 is the identity, and fp32 vs fp64 agreement.
"""

from __future__ import annotations

import numpy as np


def sylvester(h: int) -> np.ndarray:
    """Integer Sylvester-Hadamard matrix, H[i, j] = (-1)^popcount(i & j)."""
    assert h >= 1 and (h & (h - 1)) == 0, "h must be a power of two"
    H = np.empty((h, h), dtype=np.int64)
    for i in range(h):
        for j in range(h):
            H[i, j] = -1 if bin(i & j).count("1") % 2 else 1
    return H


def block_rotation_f64(d: int, h: int) -> np.ndarray:
    """The d x d orthogonal matrix blockdiag(H_h, ..., H_h) / sqrt(h)."""
    assert d % h == 0
    return np.kron(np.eye(d // h), sylvester(h).astype(np.float64)) / np.sqrt(h)


def rotate_f64(x, h: int) -> np.ndarray:
    """y = blockdiag(H_h) x / sqrt(h) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    M = block_rotation_f64(x.shape[-1], h)
    return x @ M.T


def inv_sqrt_f32(h: int) -> np.float32:
    """The fp32 value nearest to 1/sqrt(h)."""
    return np.float32(1.0 / np.sqrt(np.float64(h)))


def fwht_f32(x, h: int) -> np.ndarray:
    """fp32 block Walsh-Hadamard transform with the fixed stage order (see module doc)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    assert d % h == 0
    lead = y.shape[:-1]
    length = 1
    while length < h:
        # pairs (i, i + length) with (i & length) == 0, inside aligned blocks of 2*length
        z = y.reshape(lead + (d // (2 * length), 2, length))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(lead + (d,))
        length *= 2
    return y * inv_sqrt_f32(h)
