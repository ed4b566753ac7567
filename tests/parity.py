"""Comparison rules for GPU-vs-oracle parity (test infrastructure).

Tolerances (the band definitions are readings of the stated tolerance; see the
design notes of the repository):
  * codes: bit-exact, except coordinates whose float64 rotated value z lies
    within 1e-6 * max(|t_j|, 1) of the threshold t_j separating the two
    indices; such mismatches are counted and must be <= 1e-5 of all codes.
  * half norms / gamma: exact, except values within 1e-6 relative of a half
    rounding midpoint.
  * QJL bits: exact, except |(S r)_j| <= 1e-6 ||S_j|| ||r||; vectors with a
    band code mismatch are excluded (their residual differs).
  * reconstructions: |x_gpu - x_ref| <= 1e-5 * n16 elementwise.
  * attention: per output row ||o_gpu - o_ref|| / ||o_ref|| <= 2e-3.
  * search estimates: |est_gpu - est_ref| <= 1e-5 (unit vectors).
"""
from __future__ import annotations

import numpy as np

from oracle import tq_oracle as o

CODE_BAND = 1e-6
CODE_MISMATCH_FRAC = 1e-5
HALF_BAND = 1e-6
QJL_BAND = 1e-6
RECON_TOL = 1e-5
ATTN_TOL = 2e-3
SEARCH_TOL = 1e-5


def compare_codes(gpu_codes: np.ndarray, ref: dict, codec: o.Codec):
    """Returns (n_mismatch, mismatch_rows_mask); asserts every mismatch is in band."""
    gi = o.unpack_indices(gpu_codes, codec.d, codec.bits)
    ri = ref["idx"]
    bad = gi != ri
    n_bad = int(bad.sum())
    rows = np.zeros(gi.shape[0], dtype=bool)
    if n_bad:
        t = codec.threshold.astype(np.float64)
        rr, cc = np.nonzero(bad)
        z = ref["z"][rr, cc]
        lo = np.minimum(gi[rr, cc], ri[rr, cc])
        hi = np.maximum(gi[rr, cc], ri[rr, cc])
        assert np.all(hi - lo == 1), "code mismatch by more than one cell"
        tj = t[lo]  # threshold between cells lo and lo+1
        band = CODE_BAND * np.maximum(np.abs(tj), 1.0)
        out = np.abs(z - tj) > band
        assert not np.any(out), (
            f"{int(out.sum())} code mismatches outside the band; worst |z-t| = {np.abs(z - tj)[out].max():.3e}")
        rows[rr] = True
    total = gi.size
    assert n_bad <= max(CODE_MISMATCH_FRAC * total, 0), f"{n_bad} band mismatches of {total} codes"
    return n_bad, rows


def _half_midpoint_distance(x: np.ndarray) -> np.ndarray:
    """Relative distance of each float64 value to the nearest half rounding midpoint."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    h = x.astype(np.float16)
    hb = h.view(np.uint16).astype(np.int64)
    up = np.minimum(hb + 1, 0x7BFF).astype(np.uint16).view(np.float16).astype(np.float64)
    dn = np.maximum(hb - 1, 0).astype(np.uint16).view(np.float16).astype(np.float64)
    hv = h.astype(np.float64)
    mid = np.where(x >= hv, 0.5 * (hv + up), 0.5 * (hv + dn))
    return np.abs(x - mid) / np.maximum(x, 1e-30)


def compare_halves(gpu_bits: np.ndarray, ref_values64: np.ndarray, ref_half: np.ndarray, skip=None):
    g = np.asarray(gpu_bits).view(np.uint16)
    r = np.asarray(ref_half).view(np.uint16)
    bad = g != r
    if skip is not None:
        bad &= ~skip
    if bad.any():
        dist = _half_midpoint_distance(ref_values64[bad])
        assert np.all(dist <= HALF_BAND), f"{int((dist > HALF_BAND).sum())} half mismatches outside the band"
    return int(bad.sum())


def compare_qjl(gpu_bits: np.ndarray, ref: dict, S: np.ndarray, codec: o.Codec, skip_rows: np.ndarray):
    m = codec.qjl_m
    g = o.unpack_signs(gpu_bits, m)
    r = o.unpack_signs(ref["qjl"], m)
    bad = (g != r) & ~skip_rows[:, None]
    n_bad = int(bad.sum())
    if n_bad:
        rr, jj = np.nonzero(bad)
        u = np.abs(ref["u"][rr, jj])
        sn = np.linalg.norm(np.asarray(S, np.float64), axis=1)[jj]
        rn = np.linalg.norm(ref["r"][rr], axis=1)
        band = QJL_BAND * sn * rn
        assert np.all(u <= band), f"{int((u > band).sum())} QJL sign mismatches outside the band"
    return n_bad


def rel_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.linalg.norm(a - b, axis=-1)
    den = np.linalg.norm(b, axis=-1)
    return np.where(den > 0, num / np.maximum(den, 1e-300), num)


def assert_topk_ids(gpu_ids: np.ndarray, ref_scores_all: np.ndarray, k: int):
    """GPU top-k id sets equal the oracle's, except swaps across rank k/k+1
    when the oracle's score gap there is <= 2e-5."""
    for i in range(gpu_ids.shape[0]):
        sc = ref_scores_all[i]
        order = np.lexsort((np.arange(sc.size), -sc))
        want = set(order[:k].tolist())
        got = set(int(v) for v in gpu_ids[i] if v >= 0)
        if got != want:
            kth = sc[order[k - 1]]
            for v in got ^ want:
                assert abs(sc[v] - kth) <= 2e-5, f"query {i}: id {v} differs beyond the tie band"
