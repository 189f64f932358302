"""CPU oracle of the TurboQuant KV-cache codec (numpy, float64).

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously correct
statement of what the GPU path computes. Only the tests, the smoke check and
the CPU-baseline leg of the benchmark may import it; the library itself never
does, and it shares no code, table or constant with the GPU path. Random
parameters of the method (rotation signs, QJL sketch) are passed in as data.

What the method computes, and where the pages say so (page title, section):

* Two stages: scramble (rotate) the vector and scalar-quantize it, then fix
  the remaining error with one bit per coordinate
  ("TurboQuant と RotorQuant を DGX Spark で試してみた", PolarQuant + QJL の
  2 段階圧縮; English version "I tried TurboQuant and RotorQuant on DGX
  Spark", Two-stage compression: PolarQuant + QJL).
* Stage 1 in the vLLM/MLX implementations is a randomized Hadamard rotation
  followed by per-coordinate Lloyd-Max quantization, with no per-block scale
  ("TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況",
  第1段：PolarQuantによる回転とスカラー量子化).
* Stage 2 applies the 1-bit sign of a Johnson-Lindenstrauss random projection
  to the residual so that inner-product estimates become unbiased (same page,
  第2段：QJLの1ビット残差による内積バイアス除去; "メモリの壁を砕く圧縮革命、
  TurboQuant始動", QJL section).
* No calibration data and no training: everything depends only on (d, bits,
  seed) (same page, キャリブレーション不要が効く場面).

Where the pages are silent the plainest reading is taken; each such reading
is named in the function that relies on it:

  rotation      R = H diag(s) / sqrt(d), H the Sylvester Hadamard matrix
                H[i][j] = (-1)^popcount(i & j) (natural order), s iid +-1.
  norm          n = ||x|| stored as fp16 (round to nearest even); the unit
                vector u = x / n is quantized (u = 0 when n = 0).
  codebook      Lloyd-Max for the exact marginal density of one coordinate
                of a uniform unit vector in R^d.
  decisions     idx_i = #{j : y_i >= t_j}, taken on fp32(y_i) against fp32
                thresholds; sigma_j = [fp32(z_j) >= 0].
  residual      r = y - c[idx] in the rotated unit domain; gamma = ||r||
                stored as fp16.
  sketch        S in R^{d x d}, iid N(0,1) rounded once to fp16.
  estimator     <q, k> ~ n (sum_i q'_i c[idx_i]
                           + sqrt(pi/2)/d * gamma * sum_j p_j (2 sigma_j - 1)),
                q' = R q, p = S q'.
  softmax       exact, max-subtracted, scale sm_scale; GQA head h reads KV
                head h // G; a query attends to t < ctx_len tokens.
  value decode  acc = sum_t a_t n_t c_v[idx_t] in the rotated domain, then
                out = R_v^T acc.
  MSE-only keys the ablation without the QJL stage (same page, 第2段: the
                MSE-optimal quantizer alone biases inner products): a key
                keeps its index planes and norm only, and its logit is the
                estimator's first term n sum_i q'_i c[idx_i].

The pages print no worked logit values. The estimator is pinned instead by
what they state about it and by independent restatements: its mean over
fresh sketches equals <q, k> (unbiasedness over 1e5 pairs, with a negative
control that drops the QJL term and the variance in closed form), and
key_logits equals the formula written with scipy's Hadamard matrix and
explicit products.
"""
from __future__ import annotations

import functools
import math

import numpy as np
from scipy import special

__all__ = [
    "sphere_coord_density", "coord_cdf", "interval_mass", "interval_moment",
    "make_codebook", "hadamard", "rotate", "rotate_inverse",
    "encode", "pack_key_codes", "unpack_key_codes", "pack_mse_key_codes", "unpack_mse_key_codes", "pack_value_codes",
    "unpack_value_codes", "prepare_query", "key_logits", "key_logits_mse", "pair_logits", "decode_attend",
    "append_decode_attend", "prefill_attend", "rate_plan", "e4m3_value", "e4m3_encode", "decode_attend_k8",
    "top_k", "search",
    "QJL_CONST",
]

# --------------------------------------------------------------------------
# (a0) Lloyd-Max codebook for one coordinate of a random unit vector
# --------------------------------------------------------------------------


def sphere_coord_density(x, d: int):
    """Density f_d(x) of one coordinate of a uniform unit vector in R^d.

    f_d(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2) on
    [-1, 1]. After a random rotation every coordinate of a unit vector has
    this law, whatever the input distribution, which is what makes the
    quantizer data-oblivious.
    """
    x = np.asarray(x, dtype=np.float64)
    logc = special.gammaln(d / 2) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2)
    inside = np.abs(x) < 1
    out = np.zeros_like(x)
    out[inside] = np.exp(logc + (d - 3) / 2 * np.log1p(-x[inside] ** 2))
    return out


def coord_cdf(t, d: int):
    """P(X <= t) for X ~ f_d.  X^2 ~ Beta(1/2, (d-1)/2), so
    P(|X| <= a) = I_{a^2}(1/2, (d-1)/2) and F(t) = 1/2 + sign(t)/2 P(|X| <= |t|).
    Returned as a pair (F(t), 1 - F(t)) so tails keep full precision."""
    t = np.asarray(t, dtype=np.float64)
    a2 = np.minimum(t * t, 1.0)
    inner = special.betainc(0.5, (d - 1) / 2, a2)          # P(|X| <= |t|)
    outer = special.betaincc(0.5, (d - 1) / 2, a2)         # P(|X| >  |t|)
    lower = np.where(t >= 0, 0.5 + 0.5 * inner, 0.5 * outer)
    upper = np.where(t >= 0, 0.5 * outer, 0.5 + 0.5 * inner)
    return lower, upper


def interval_mass(a, b, d: int):
    """Integral of f_d over [a, b] (a <= b), via the incomplete beta function."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    la, ua = coord_cdf(a, d)
    lb, ub = coord_cdf(b, d)
    # use whichever difference is the difference of small numbers
    return np.where(b <= 0, lb - la, np.where(a >= 0, ua - ub, lb - la))


def interval_moment(a, b, d: int):
    """Integral of x f_d(x) over [a, b]: an antiderivative of x (1-x^2)^((d-3)/2)
    is -(1-x^2)^((d-1)/2) / (d-1)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    logc = special.gammaln(d / 2) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2)

    def prim(x):
        return -np.power(np.maximum(1.0 - x * x, 0.0), (d - 1) / 2) / (d - 1)

    return math.exp(logc) * (prim(b) - prim(a))


def make_codebook(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000,
                  return_fp64: bool = False):
    """Lloyd-Max quantizer with L = 2^bits levels for the density f_d.

    The two Lloyd conditions are iterated to their fixed point:
      thresholds are midpoints of neighbouring centroids,
      each centroid is the conditional mean of f_d on its cell,
    with t_0 = -1 and t_L = +1. The density is symmetric, so the iteration is
    kept exactly symmetric (c_{L-1-j} = -c_j; the middle threshold of an even
    L is 0). For d >= 3 f_d is log-concave and the fixed point is unique.

    Returns (centroids fp32 [L] ascending, thresholds fp32 [L-1]); thresholds
    are the fixed point's exact midpoints rounded once to fp32. With
    return_fp64 the unrounded fp64 arrays are returned instead.
    """
    if d < 3 or bits < 1 or bits > 8:
        raise ValueError("make_codebook: need d >= 3 and 1 <= bits <= 8")
    L = 1 << bits
    # start from equal-probability cells (quantiles of f_d)
    probs = (np.arange(L) + 0.5) / L
    # invert the CDF by bisection (vectorized)
    lo = -np.ones(L)
    hi = np.ones(L)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        f, _u = coord_cdf(mid, d)
        lo = np.where(f < probs, mid, lo)
        hi = np.where(f < probs, hi, mid)
    c = 0.5 * (lo + hi)
    c = 0.5 * (c - c[::-1])
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        m0 = interval_mass(edges[:-1], edges[1:], d)
        m1 = interval_moment(edges[:-1], edges[1:], d)
        c_new = m1 / m0
        c_new = 0.5 * (c_new - c_new[::-1])
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    if L % 2 == 0:
        t[L // 2 - 1] = 0.0
    if return_fp64:
        return c, t
    return c.astype(np.float32), t.astype(np.float32)


# --------------------------------------------------------------------------
# (a2) rotation R = H diag(s) / sqrt(d)
# --------------------------------------------------------------------------


@functools.lru_cache(maxsize=None)
def _hadamard_cached(d: int) -> np.ndarray:
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    a = i & j
    pop = np.zeros_like(a)
    while np.any(a):
        pop += a & 1
        a = a >> 1
    h = np.where(pop % 2 == 0, 1.0, -1.0)
    h.setflags(write=False)
    return h


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix in natural order: H[i][j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("hadamard: d must be a power of two")
    return _hadamard_cached(d)


def rotate(x, signs):
    """y = R x with R = H diag(s) / sqrt(d); rows of x are vectors."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    return (x * s) @ hadamard(d).T / math.sqrt(d)


def rotate_inverse(y, signs):
    """x = R^T y = diag(s) H^T y / sqrt(d)."""
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = y.shape[-1]
    return (y @ hadamard(d)) * s / math.sqrt(d)


# --------------------------------------------------------------------------
# (a1)-(a5), (a7) encode
# --------------------------------------------------------------------------


def encode(x, signs, centroids, thresholds, sketch=None):
    """Encode rows of x (any float dtype, converted exactly to fp64).

    Steps, in the pages' order: store the norm, rotate the unit vector,
    quantize each coordinate with the Lloyd-Max thresholds; for keys (sketch
    given) take the residual, its norm and the signs of its projection by S.

    Returns a dict with
      idx    int64 [..., d]   Lloyd-Max indices
      nhat   float16 [...]    stored norm
      sigma  uint8 [..., d]   QJL sign bits            (keys)
      ghat   float16 [...]    stored residual norm     (keys)
    and, for the parity rule, the fp64 pre-decision values
      y      float64 [..., d] rotated unit vector
      z      float64 [..., d] projected residual        (keys)
      n, gamma  float64 norms before fp16 rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    t32 = np.asarray(thresholds, dtype=np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1))
    safe = np.where(n > 0, n, 1.0)
    u = np.where((n > 0)[..., None], x / safe[..., None], 0.0)
    y = rotate(u, signs)
    yf = y.astype(np.float32)
    idx = np.sum(yf[..., None] >= t32, axis=-1).astype(np.int64)
    out = dict(idx=idx, nhat=n.astype(np.float16), y=y, n=n)
    if sketch is not None:
        S = np.asarray(sketch, dtype=np.float16).astype(np.float64)
        r = y - c[idx]
        gamma = np.sqrt(np.sum(r * r, axis=-1))
        z = _project(S, r)
        sigma = (z.astype(np.float32) >= 0).astype(np.uint8)
        out.update(sigma=sigma, ghat=gamma.astype(np.float16), z=z, gamma=gamma, r=r)
    return out


def _project(S, v):
    """S v for every row v. S is one [d, d] sketch shared by all rows, or a
    stack [..., d, d] holding one sketch per row (used by statistical tests
    that redraw S for every key)."""
    if S.ndim == 2:
        return v @ S.T
    return np.einsum("...jk,...k->...j", S, v)


def requantize_key(y, idx, centroids, sketch):
    """Residual, gamma and projection of a key for GIVEN indices (used by the
    parity rule after an excused index mismatch)."""
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    S = np.asarray(sketch, dtype=np.float16).astype(np.float64)
    r = np.asarray(y, dtype=np.float64) - c[np.asarray(idx)]
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    z = _project(S, r)
    return dict(r=r, gamma=gamma, z=z, sigma=(z.astype(np.float32) >= 0).astype(np.uint8),
                ghat=gamma.astype(np.float16))


# --------------------------------------------------------------------------
# (a6) packing
# --------------------------------------------------------------------------


def _plane_bytes(bits01):
    """[..., d] of 0/1 -> [..., d/8] bytes, coordinate i at byte i//8, bit i%8."""
    b = np.asarray(bits01, dtype=np.uint8)
    d = b.shape[-1]
    b = b.reshape(b.shape[:-1] + (d // 8, 8))
    weights = (1 << np.arange(8)).astype(np.uint8)
    return np.sum(b * weights, axis=-1, dtype=np.uint64).astype(np.uint8)


def pack_key_codes(idx, sigma, lm_bits: int):
    """Key record: lm_bits index planes (plane p holds bit p of idx), then the
    QJL sign plane; each plane is d/8 bytes, coordinate i at byte i//8, bit
    i%8. Returns uint8 [..., (lm_bits+1)*d/8]."""
    idx = np.asarray(idx, dtype=np.int64)
    planes = [_plane_bytes((idx >> p) & 1) for p in range(lm_bits)]
    planes.append(_plane_bytes(sigma))
    return np.concatenate(planes, axis=-1)


def unpack_key_codes(codes, d: int, lm_bits: int):
    codes = np.asarray(codes, dtype=np.uint8)
    nb = d // 8
    bits = np.unpackbits(codes, axis=-1, bitorder="little").astype(np.int64)
    idx = np.zeros(codes.shape[:-1] + (d,), dtype=np.int64)
    for p in range(lm_bits):
        idx |= bits[..., p * d:(p + 1) * d] << p
    sigma = bits[..., lm_bits * d:(lm_bits + 1) * d].astype(np.uint8)
    assert codes.shape[-1] == (lm_bits + 1) * nb
    return idx, sigma


def pack_mse_key_codes(idx, lm_bits: int):
    """MSE-only key record (the ablation without the QJL stage): the lm_bits
    index planes of a key record and nothing else, plane p holding bit p of
    idx, coordinate i at byte i//8, bit i%8. Returns uint8 [..., lm_bits*d/8]."""
    idx = np.asarray(idx, dtype=np.int64)
    return np.concatenate([_plane_bytes((idx >> p) & 1) for p in range(lm_bits)], axis=-1)


def unpack_mse_key_codes(codes, d: int, lm_bits: int):
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] == lm_bits * (d // 8)
    bits = np.unpackbits(codes, axis=-1, bitorder="little").astype(np.int64)
    idx = np.zeros(codes.shape[:-1] + (d,), dtype=np.int64)
    for p in range(lm_bits):
        idx |= bits[..., p * d:(p + 1) * d] << p
    return idx


VALUE_BLOCK = 32   # tokens per value-code block


def pack_value_codes(idx, lm_bits: int, cap: int | None = None):
    """Value codes, token-major: for each sequence, tokens are grouped in
    blocks of 32; for block B, plane p and coordinate i one 32-bit word holds
    bit p of idx[32B + j, i] at bit j. idx: [n_seq, n_tok, d] ->
    uint32 [n_seq, cap/32, lm_bits, d] (tokens >= n_tok are zero)."""
    idx = np.asarray(idx, dtype=np.int64)
    n_seq, n_tok, d = idx.shape
    if cap is None:
        cap = -(-n_tok // VALUE_BLOCK) * VALUE_BLOCK
    nblk = cap // VALUE_BLOCK
    full = np.zeros((n_seq, cap, d), dtype=np.int64)
    full[:, :n_tok] = idx
    full = full.reshape(n_seq, nblk, VALUE_BLOCK, d)
    out = np.zeros((n_seq, nblk, lm_bits, d), dtype=np.uint64)
    for p in range(lm_bits):
        bit = (full >> p) & 1                                  # [s, B, 32, d]
        for j in range(VALUE_BLOCK):
            out[:, :, p, :] |= bit[:, :, j, :].astype(np.uint64) << np.uint64(j)
    return out.astype(np.uint32)


def unpack_value_codes(words, n_tok: int):
    words = np.asarray(words, dtype=np.uint64)
    n_seq, nblk, lm_bits, d = words.shape
    idx = np.zeros((n_seq, nblk, VALUE_BLOCK, d), dtype=np.int64)
    for p in range(lm_bits):
        for j in range(VALUE_BLOCK):
            idx[:, :, j, :] |= (((words[:, :, p, :] >> np.uint64(j)) & np.uint64(1))
                                .astype(np.int64) << p)
    return idx.reshape(n_seq, nblk * VALUE_BLOCK, d)[:, :n_tok]


# --------------------------------------------------------------------------
# (a8)-(a11) logits and decode attention
# --------------------------------------------------------------------------

QJL_CONST = math.sqrt(math.pi / 2.0)   # divided by m = d sketch rows


def prepare_query(q, signs, sketch):
    """q' = R q and p = S q' (fp64)."""
    qr = rotate(np.asarray(q, dtype=np.float64), signs)
    S = np.asarray(sketch, dtype=np.float16).astype(np.float64)
    return qr, qr @ S.T


def key_logits(q, signs, centroids, sketch, idx, sigma, nhat, ghat):
    """Estimated <q, k> for every query row of q against every key.

    q: [nq, d]; idx, sigma: [N, d]; nhat, ghat: [N] (stored fp16 values).
    Returns fp64 [nq, N]:
      n (sum_i q'_i c[idx_i] + sqrt(pi/2)/d * gamma * sum_j p_j (2 sigma_j - 1)).
    """
    d = np.asarray(q).shape[-1]
    qr, p = prepare_query(q, signs, sketch)
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    khat = c[np.asarray(idx)]                                  # [N, d]
    lm = qr @ khat.T                                           # [nq, N]
    pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0       # [N, d]
    qjl = p @ pm.T                                             # [nq, N]
    n = np.asarray(nhat, dtype=np.float16).astype(np.float64)
    g = np.asarray(ghat, dtype=np.float16).astype(np.float64)
    return n[None, :] * (lm + (QJL_CONST / d) * g[None, :] * qjl)


def key_logits_mse(q, signs, centroids, idx, nhat):
    """The MSE-only estimate of <q, k>: the first term of key_logits alone,
    n sum_i q'_i c[idx_i] with q' = R q -- the biased estimate that the QJL
    bit corrects ("TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況",
    第2段). q: [nq, d]; idx: [N, d]; nhat: [N]. Returns fp64 [nq, N]."""
    qr = rotate(np.asarray(q, dtype=np.float64), signs)
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    n = np.asarray(nhat, dtype=np.float16).astype(np.float64)
    return n[None, :] * (qr @ c[np.asarray(idx)].T)


def pair_logits(q, signs, centroids, sketch, idx, sigma, nhat, ghat):
    """Estimated <q_i, k_i> for row-aligned pairs (query i against key i).

    Same estimator as key_logits; the sketch may be one [d, d] matrix or one
    per pair ([N, d, d]). Returns fp64 [N]."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    S = np.asarray(sketch, dtype=np.float16).astype(np.float64)
    qr = rotate(q, signs)
    p = _project(S, qr)
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    lm = np.sum(qr * c[np.asarray(idx)], axis=-1)
    qjl = np.sum(p * (2.0 * np.asarray(sigma, dtype=np.float64) - 1.0), axis=-1)
    n = np.asarray(nhat, dtype=np.float16).astype(np.float64)
    g = np.asarray(ghat, dtype=np.float16).astype(np.float64)
    return n * (lm + (QJL_CONST / d) * g * qjl)


def value_rows(vidx, vnhat, v_centroids):
    """Reconstructed values in the rotated domain: n_t c_v[idx_t]."""
    cv = np.asarray(v_centroids, dtype=np.float32).astype(np.float64)
    return np.asarray(vnhat, dtype=np.float16).astype(np.float64)[..., None] * cv[np.asarray(vidx)]


def decode_attend(q, k_signs, k_centroids, sketch, kidx, ksigma, knhat, kghat,
                  v_signs, v_centroids, vidx, vnhat, ctx_lens, sm_scale, group: int):
    """Fused decode attention over the coded cache.

    q: [B, Hq, d]; key/value arrays indexed [B*Hkv, T, ...]; ctx_lens [B].
    Query head h of batch b reads KV sequence b*Hkv + h // group, tokens
    t < ctx_lens[b]. Returns fp64 [B, Hq, d]; rows with ctx_len <= 0 are 0.
    sketch None: MSE-only keys (no QJL stage; ksigma and kghat unused), whose
    logits are the estimator's first term (key_logits_mse).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = Hq // group
    out = np.zeros((B, Hq, d))
    for b in range(B):
        T = int(ctx_lens[b])
        if T <= 0:
            continue
        for hk in range(Hkv):
            s = b * Hkv + hk
            qs = q[b, hk * group:(hk + 1) * group]
            if sketch is None:
                lg = key_logits_mse(qs, k_signs, k_centroids, kidx[s, :T], knhat[s, :T])
            else:
                lg = key_logits(qs, k_signs, k_centroids, sketch, kidx[s, :T], ksigma[s, :T],
                                knhat[s, :T], kghat[s, :T])    # [G, T]
            z = sm_scale * lg
            z = z - z.max(axis=1, keepdims=True)
            a = np.exp(z)
            a = a / a.sum(axis=1, keepdims=True)
            vr = value_rows(vidx[s, :T], vnhat[s, :T], v_centroids)   # [T, d]
            acc = a @ vr                                       # [G, d] rotated domain
            out[b, hk * group:(hk + 1) * group] = rotate_inverse(acc, v_signs)
    return out


def prefill_attend(q, k_signs, k_centroids, sketch, kidx, ksigma, knhat, kghat, v_signs, v_centroids, vidx,
                   vnhat, pos0, sm_scale, group: int):
    """Causal attention of a prefill chunk over the coded cache (whose slots
    already hold the chunk's own tokens): q [B, C, Hq, d]; query position i
    of batch row b attends to the tokens t <= pos0[b] + i (clamped to the
    cache arrays' length). Long prefills sit at the high end of the pages'
    measured throughput range ("TurboQuantとは？仕組み・実測精度・2026年7月
    時点の実装状況", section 「精度劣化ゼロ」の出所と、マージ後に判明した実測値).
    sketch None: MSE-only keys, as in decode_attend. Returns fp64 [B, C, Hq, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, C, Hq, d = q.shape
    T = np.asarray(kidx).shape[1]
    out = np.zeros((B, C, Hq, d))
    Hkv = Hq // group
    for b in range(B):
        rows = lambda a: None if a is None else a[b * Hkv:(b + 1) * Hkv]
        for i in range(C):
            n = min(int(pos0[b]) + i + 1, T)
            out[b, i] = decode_attend(q[b, i][None], k_signs, k_centroids, sketch, rows(kidx), rows(ksigma),
                                      rows(knhat), rows(kghat), v_signs, v_centroids, rows(vidx), rows(vnhat),
                                      [n], sm_scale, group)[0]
    return out


def append_decode_attend(q, k_new, v_new, k_signs, k_centroids, k_thresholds, sketch, kidx, ksigma, knhat,
                         kghat, v_signs, v_centroids, v_thresholds, vidx, vnhat, ctx_lens, sm_scale, group: int):
    """One decoding step: the new token's key and value (k_new, v_new
    [B, Hkv, d]) are encoded and stored in slot ctx_lens[b] - 1 of every KV
    sequence of batch row b (ctx_lens counts the new token; rows with
    ctx_lens <= 0 append nothing), then decode_attend runs over the updated
    cache. The encode step sits beside decode on the serving path: the pages
    place decode-heavy serving at the low end of the measured throughput
    ("TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況", section
    「精度劣化ゼロ」の出所と、マージ後に判明した実測値).

    The cache arrays are [B*Hkv, T, ...] as in decode_attend and are not
    modified; returns (out [B, Hq, d], updated cache dict, key encoding and
    value encoding of the new rows, each [B, Hkv, ...]). sketch None:
    MSE-only keys (ksigma and kghat unused and returned as None)."""
    k_new = np.asarray(k_new, dtype=np.float64)
    B, Hkv, d = k_new.shape
    ek = encode(k_new.reshape(B * Hkv, d), k_signs, k_centroids, k_thresholds, sketch)
    ev = encode(np.asarray(v_new, dtype=np.float64).reshape(B * Hkv, d), v_signs, v_centroids, v_thresholds)
    qjl = sketch is not None
    cache = {"kidx": np.array(kidx), "ksigma": np.array(ksigma) if qjl else None, "knhat": np.array(knhat),
             "kghat": np.array(kghat) if qjl else None, "vidx": np.array(vidx), "vnhat": np.array(vnhat)}
    for b in range(B):
        t = int(ctx_lens[b]) - 1
        if t < 0:
            continue
        for hk in range(Hkv):
            s = b * Hkv + hk
            cache["kidx"][s, t] = ek["idx"][s]
            cache["knhat"][s, t] = ek["nhat"][s]
            if qjl:
                cache["ksigma"][s, t] = ek["sigma"][s]
                cache["kghat"][s, t] = ek["ghat"][s]
            cache["vidx"][s, t] = ev["idx"][s]
            cache["vnhat"][s, t] = ev["nhat"][s]
    out = decode_attend(q, k_signs, k_centroids, sketch, cache["kidx"], cache["ksigma"], cache["knhat"],
                        cache["kghat"], v_signs, v_centroids, cache["vidx"], cache["vnhat"], ctx_lens, sm_scale,
                        group)
    shape = lambda e: {k: v.reshape((B, Hkv) + v.shape[1:]) for k, v in e.items()}
    return out, cache, shape(ek), shape(ev)


# --------------------------------------------------------------------------
# fp8 keys (the k8v4 cache shape)
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of OCP e4m3fn byte(s): sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent field 0 is subnormal (m/8 * 2^-6), the two
    codes with all exponent and mantissa bits set are NaN, there is no
    infinity."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def e4m3_encode(x, scale=1.0):
    """e4m3fn bytes of x / scale: the quotient in float32 (both operands as
    float32, correctly rounded), finite values beyond +-448 saturated, then
    rounded to the nearest e4m3 value with ties to an even mantissa; NaN gives
    0xff. Reading for the k8v4 preset the pages name (fp8 keys with 4-bit
    values, "TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況", section
    vLLM：–kv-cache-dtypeの切り替えだけで利用可能): the pages do not give the
    fp8 format or its scaling; OCP e4m3fn with one per-tensor scale is the
    common fp8 KV-cache form."""
    y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float64)
    nan = np.isnan(y)
    y = np.where(nan, 0.0, np.clip(y, -E4M3_MAX, E4M3_MAX))
    sign = np.signbit(y)
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                          # subnormals share the quantum 2^-9
    q = 2.0 ** (e - 3.0)
    r = np.rint(a / q) * q                           # round half to even on the mantissa
    # fields of the rounded magnitude
    normal = r >= 2.0 ** -6
    er = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    ef = np.where(normal, er + 7.0, 0.0)
    mf = np.where(normal, (r / 2.0 ** er - 1.0) * 8.0, r / 2.0 ** -9)
    code = (sign.astype(np.int64) << 7) | (ef.astype(np.int64) << 3) | mf.astype(np.int64)
    return np.where(nan, 0xFF, code).astype(np.uint8)


def decode_attend_k8(q, kcodes, k_scale, v_signs, v_centroids, vidx, vnhat, ctx_lens, sm_scale, group: int):
    """Decode attention over fp8 keys and coded values: logit = k_scale *
    q . e4m3(k) (no rotation on the key side), softmax, values as in
    decode_attend. q [B, Hq, d]; kcodes uint8 [B*Hkv, T, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = Hq // group
    K = e4m3_value(kcodes) * float(k_scale)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        T = int(ctx_lens[b])
        if T <= 0:
            continue
        for hk in range(Hkv):
            s = b * Hkv + hk
            lg = q[b, hk * group:(hk + 1) * group] @ K[s, :T].T
            z = sm_scale * lg
            z = z - z.max(axis=1, keepdims=True)
            a = np.exp(z)
            a = a / a.sum(axis=1, keepdims=True)
            out[b, hk * group:(hk + 1) * group] = rotate_inverse(a @ value_rows(vidx[s, :T], vnhat[s, :T],
                                                                                v_centroids), v_signs)
    return out


# --------------------------------------------------------------------------
# fractional rates
# --------------------------------------------------------------------------

def rate_plan(bits: float, n_layers: int, is_key: bool):
    """Per-layer Lloyd-Max widths for an average of `bits` per channel (keys:
    the QJL sign bit included). The pages name 2.5- and 3.5-bit operating
    points ("TurboQuantとは？仕組み・実測精度・2026年7月時点の実装状況",
    section 「精度劣化ゼロ」の出所と、マージ後に判明した実測値) and a serving
    fork that sets the quantization parameters per layer for those presets
    ("TurboQuant と RotorQuant を DGX Spark で試してみた", section DGX Spark
    専用の vLLM フォーク); how the bits are allocated is not stated. Reading
    taken: the two neighbouring integer widths, the wider one on
    round(frac * n_layers) layers spread evenly over the depth (layer l when
    the proportional count floor(l * n_hi / n_layers) steps up at l + 1).
    Returns a list of ints, or raises ValueError outside widths 1..4."""
    avg = bits - (1.0 if is_key else 0.0)
    w = math.floor(avg)
    n_hi = math.floor((avg - w) * n_layers + 0.5)
    plan = [w + (1 if (l + 1) * n_hi // n_layers > l * n_hi // n_layers else 0) for l in range(n_layers)]
    if min(plan) < 1 or max(plan) > 4:
        raise ValueError("widths outside 1..4")
    return plan


# --------------------------------------------------------------------------
# inner-product search over a coded database
# --------------------------------------------------------------------------

def top_k(scores, k: int):
    """The k largest entries of every row of scores [n_rows, n], ranked by
    score descending and, among equal scores, by column ascending (-0.0 and
    +0.0 are equal). Returns (values [n_rows, k], columns [n_rows, k]).

    The ranking step of inner-product search over a coded database: the
    pages name vector-search indexes as a target of the same codes and
    estimator, ranked by inner product ("メモリの壁を砕く圧縮革命、TurboQuant
    始動", sections TurboQuantの全体像 and 仕組みをほどく)."""
    s = np.asarray(scores)
    n_rows, n = s.shape
    cols = np.arange(n)
    vals = np.empty((n_rows, k), dtype=s.dtype)
    idx = np.empty((n_rows, k), dtype=np.int64)
    for r in range(n_rows):
        order = np.lexsort((cols, -s[r]))[:k]        # primary: -score, then column
        idx[r] = order
        vals[r] = s[r, order]
    return vals, idx


def search(q, signs, centroids, sketch, idx, sigma, nhat, ghat, k: int):
    """Inner-product search of the query rows q [nq, d] over a database of
    coded vectors (key records idx, sigma, nhat, ghat): the estimated inner
    products (key_logits), then their top k per query (top_k)."""
    return top_k(key_logits(q, signs, centroids, sketch, idx, sigma, nhat, ghat), k)

