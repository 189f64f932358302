"""Parity rule between the GPU codes and the CPU oracle.

(i)   Index and sign bits must equal the oracle's, except where the oracle's
      fp64 pre-decision value (y_i or z_j, unit domain) lies within 1e-6 of
      the crossed boundary. After an excused index mismatch the oracle
      recomputes r, gamma and z from the GPU's indices before the vector's
      signs are compared.
(ii)  fp16 scalars may differ by one ulp only where the fp64 value lies
      within 1e-6 (relative) of an fp16 rounding midpoint.
(iii) Excused mismatches number at most 1e-5 of the coded items.
(iv)  Logits and outputs, given identical codes:
      |gpu - ref| <= 1e-4 + 1e-3 |ref| elementwise.
"""
from __future__ import annotations

import numpy as np

import oracle as O

BOUNDARY_EPS = 1e-6
EXCUSED_FRACTION = 1e-5
ATOL = 1e-4
RTOL = 1e-3


def _fp16_excusable(gpu_h: np.ndarray, ref64: np.ndarray) -> np.ndarray:
    """True where gpu_h (fp16) is the fp16 neighbour of round(ref64) and ref64
    sits within 1e-6 relative of the midpoint between the two."""
    ref_h = ref64.astype(np.float16)
    a = ref_h.astype(np.float64)
    b = gpu_h.astype(np.float64)
    adjacent = (np.nextafter(ref_h, np.float16(np.inf)) == gpu_h) | (np.nextafter(ref_h, np.float16(-np.inf)) == gpu_h)
    mid = 0.5 * (a + b)
    return adjacent & (np.abs(ref64 - mid) <= BOUNDARY_EPS * np.maximum(np.abs(ref64), 1e-30))


def check_scalars(gpu_h, ref64, ref_h, what):
    gpu_h = np.asarray(gpu_h, dtype=np.float16)
    bad = gpu_h.view(np.uint16) != np.asarray(ref_h, dtype=np.float16).view(np.uint16)
    excused = bad & _fp16_excusable(gpu_h, np.asarray(ref64, dtype=np.float64))
    hard = bad & ~excused
    assert not np.any(hard), f"{what}: {int(hard.sum())} fp16 scalars differ beyond the midpoint rule " \
                             f"(first at {np.argwhere(hard)[:3].tolist()})"
    return int(excused.sum())


def check_index(gpu_idx, enc, thresholds, what):
    """Returns (excused count, mask of vectors with an excused index mismatch)."""
    gpu_idx = np.asarray(gpu_idx)
    ref = enc["idx"]
    y = enc["y"]
    t = np.asarray(thresholds, dtype=np.float32).astype(np.float64)
    bad = gpu_idx != ref
    if not np.any(bad):
        return 0, np.zeros(ref.shape[:-1], dtype=bool)
    diff = np.abs(gpu_idx.astype(np.int64) - ref)
    upper = np.maximum(gpu_idx, ref)           # crossed threshold is t[upper-1]
    crossed = t[np.clip(upper - 1, 0, len(t) - 1)]
    excused = bad & (diff == 1) & (np.abs(y - crossed) <= BOUNDARY_EPS)
    hard = bad & ~excused
    assert not np.any(hard), f"{what}: {int(hard.sum())} index mismatches away from a boundary " \
                             f"(first at {np.argwhere(hard)[:3].tolist()}, gpu {gpu_idx[hard][:3]}, " \
                             f"ref {ref[hard][:3]}, y {y[hard][:3]})"
    return int(excused.sum()), np.any(excused, axis=-1)


def check_key_codes(gpu_codes, gpu_scal, enc, lm_bits, centroids, thresholds, sketch, d, what="keys"):
    """Full parity rule for key records of shape [..., (w+1)d/8] and scalars [..., 2] (fp16 bits)."""
    gidx, gsig = O.unpack_key_codes(np.asarray(gpu_codes), d, lm_bits)
    gsc = np.asarray(gpu_scal).view(np.float16)
    n_items = gidx.size * 2 + gsc.size
    ex_idx, vec_mask = check_index(gidx, enc, thresholds, what + " idx")
    z = enc["z"].copy()
    gamma = enc["gamma"].copy()
    ghat = enc["ghat"].copy()
    sigma = enc["sigma"].copy()
    if np.any(vec_mask):
        rq = O.requantize_key(enc["y"][vec_mask], gidx[vec_mask], centroids, sketch)
        z[vec_mask] = rq["z"]
        gamma[vec_mask] = rq["gamma"]
        ghat[vec_mask] = rq["ghat"]
        sigma[vec_mask] = rq["sigma"]
    bad = gsig != sigma
    excused = bad & (np.abs(z) <= BOUNDARY_EPS)
    hard = bad & ~excused
    assert not np.any(hard), f"{what} sign: {int(hard.sum())} sign mismatches away from zero " \
                             f"(first at {np.argwhere(hard)[:3].tolist()}, z {z[hard][:3]})"
    ex = ex_idx + int(excused.sum())
    ex += check_scalars(gsc[..., 0], enc["n"], enc["nhat"], what + " norm")
    ex += check_scalars(gsc[..., 1], gamma, ghat, what + " gamma")
    assert ex <= max(1, EXCUSED_FRACTION * n_items), f"{what}: {ex} excused mismatches of {n_items} items"
    return dict(excused=ex, items=n_items, exact=(ex == 0))


def check_value_codes(gpu_words, gpu_scal, enc, lm_bits, thresholds, n_tok, what="values", t0=0):
    """Value codes of slots [t0, t0 + n_tok) against the oracle's encoding of those tokens."""
    gidx = O.unpack_value_codes(np.asarray(gpu_words).view(np.uint32), t0 + n_tok)[:, t0:]
    gsc = np.asarray(gpu_scal).view(np.float16)[..., t0:t0 + n_tok]
    n_items = gidx.size + gsc.size
    ex, _ = check_index(gidx, enc, thresholds, what + " idx")
    ex += check_scalars(gsc, enc["n"], enc["nhat"], what + " norm")
    assert ex <= max(1, EXCUSED_FRACTION * n_items), f"{what}: {ex} excused mismatches of {n_items} items"
    return dict(excused=ex, items=n_items, exact=(ex == 0))


def assert_close(gpu, ref, what, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    tol = atol + rtol * np.abs(ref)
    bad = ~(err <= tol)
    assert not np.any(bad), f"{what}: {int(bad.sum())}/{bad.size} outside atol={atol} rtol={rtol}; " \
                            f"worst err {err.max():.3g} at {np.unravel_index(np.argmax(err - tol), err.shape)}"
    return float(np.max(err / tol)) if err.size else 0.0
