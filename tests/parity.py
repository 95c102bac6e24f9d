"""Comparison helpers shared by the GPU parity tests (test code, CPU side)."""

from __future__ import annotations

import numpy as np

from oracle import commvq_oracle as O

NEAR_TIE_REL = 1e-5   # codes may differ only where the top-2 distance gap is below this
ATTN_TOL = 2e-3       # max |out - ref| / max |ref| per (sequence, query head)


def check_encoding(x, cb, gpu_packed, n_entries, rel_tol=NEAR_TIE_REL):
    """Compare GPU-packed records with the oracle's.

    Bytes must match exactly, except for groups where the GPU picked a different
    entry whose oracle (float64) distance is within rel_tol of the minimum; the
    later rounds of such a group are then checked from the GPU's pick onwards.
    Returns (hard_mismatches, near_ties) as lists of (token, head, round, group, rel)."""
    x = np.asarray(x)
    cb = np.asarray(cb)
    H, G, R, Nc, g = cb.shape
    codes, _ = O.encode(x, cb)
    ref = O.pack_codes(codes, n_entries)
    gpu_packed = np.asarray(gpu_packed)
    if gpu_packed.shape != ref.shape:
        return [("shape", gpu_packed.shape, ref.shape)], []
    if np.array_equal(gpu_packed, ref):
        return [], []
    gcodes = O.unpack_codes(gpu_packed, R, G, n_entries)
    hard, ties = [], []
    # padding bits of a record must be zero
    nbits = R * G * O.field_bits(n_entries)
    if nbits % 8:
        last = gpu_packed[..., -1].astype(np.int64) >> (nbits % 8)
        for n, h in np.argwhere(last != 0):
            hard.append((int(n), int(h), -1, -1, "nonzero padding"))
    for n, h, j in np.argwhere((gcodes != codes).any(axis=2)):
        e = x[n, h, j * g:(j + 1) * g].astype(np.float64)
        for r in range(R):
            d = O.sq_distances(e, cb[h, j, r].astype(np.float64))
            gi = int(gcodes[n, h, r, j])
            dmin = float(d.min())
            if gi != int(np.argmin(d)):
                rel = (float(d[gi]) - dmin) / max(dmin, 1e-12 * float(e @ e), 1e-300)
                item = (int(n), int(h), r, int(j), rel)
                if rel < rel_tol:
                    ties.append(item)
                else:
                    hard.append(item)
                    break
            e = e - cb[h, j, r, gi].astype(np.float64)
    return hard, ties


def row_errors(gpu, ref):
    """Per-row max |gpu - ref| / max |ref| over the last axis (rows of zeros must be exact)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(gpu - ref).max(-1)
    den = np.abs(ref).max(-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
