"""Property tests (hypothesis) of the oracle and the host side of libtq.

- Packing: key, MSE-only key and value records round-trip for random shapes
  (d a multiple of 8 up to 256, w 1..4, ragged token counts) and keep every
  plane's bits where the layout puts them.
- Decisions: idx = #{j : t_j <= y} is monotone in y, lands in [0, L), and a
  value exactly on a threshold takes the upper cell.
- Encoding: for random (n, d in {4, ..., 256} powers of two, w) the rotated
  unit vector has norm 1 (0 for the zero vector), indices stay in range, the
  centroid of each coordinate's cell brackets it between the cell's
  thresholds, and a single-token input encodes like the same row in a batch.
- The host codebook (tq_make_codebook) equals the oracle's for random
  (d, w), and tq_rate_plan's widths average to the requested rate.
- Argument validation: malformed requests return TQ_EINVAL / TQ_EUNSUPPORTED
  before anything is launched (no GPU is needed to run these).
"""
import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import kv_cache_vector_rht_amd as tq
import oracle as O

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])

dims8 = st.sampled_from([8, 16, 24, 32, 64, 96, 128, 256])
widths = st.integers(min_value=1, max_value=4)


@SETTINGS
@given(d=dims8, w=widths, n=st.integers(1, 5), t=st.integers(1, 70), seed=st.integers(0, 2**31 - 1))
def test_pack_roundtrips(d, w, n, t, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, 1 << w, size=(n, t, d))
    sig = rng.integers(0, 2, size=(n, t, d))
    rec = O.pack_key_codes(idx, sig, w)
    assert rec.shape == (n, t, (w + 1) * d // 8)
    i2, s2 = O.unpack_key_codes(rec, d, w)
    np.testing.assert_array_equal(i2, idx)
    np.testing.assert_array_equal(s2, sig)
    # plane p, coordinate i: byte p*d/8 + i//8, bit i%8
    b, tk, i, p = rng.integers(n), rng.integers(t), rng.integers(d), rng.integers(w)
    assert (rec[b, tk, p * d // 8 + i // 8] >> (i % 8)) & 1 == (idx[b, tk, i] >> p) & 1
    assert (rec[b, tk, w * d // 8 + i // 8] >> (i % 8)) & 1 == sig[b, tk, i]
    mrec = O.pack_mse_key_codes(idx, w)
    np.testing.assert_array_equal(mrec, rec[..., :w * d // 8])
    np.testing.assert_array_equal(O.unpack_mse_key_codes(mrec, d, w), idx)
    words = O.pack_value_codes(idx, w)
    assert words.shape[1] == (t + 31) // 32
    np.testing.assert_array_equal(O.unpack_value_codes(words, t), idx)
    # value word (block t//32, plane p, coordinate i) holds token t's bit p at bit t%32
    assert (int(words[b, tk // 32, p, i]) >> (tk % 32)) & 1 == (idx[b, tk, i] >> p) & 1


@SETTINGS
@given(d=st.sampled_from([4, 8, 64, 128, 256]), w=widths, seed=st.integers(0, 2**31 - 1))
def test_decisions_are_monotone_with_ties_up(d, w, seed):
    c, t = O.make_codebook(d, w)
    rng = np.random.default_rng(seed)
    y = np.sort(rng.uniform(-1, 1, size=200))
    # plant exact ties on every threshold
    y = np.sort(np.concatenate([y, t.astype(np.float64)]))
    idx = np.sum(y.astype(np.float32)[:, None] >= t.astype(np.float32), axis=1)
    assert np.all(np.diff(idx) >= 0) and idx.min() >= 0 and idx.max() <= (1 << w) - 1
    for j, tj in enumerate(t):
        k = np.searchsorted(y, tj)
        assert idx[k] == j + 1                  # y == t_j: the upper cell


@SETTINGS
@given(logd=st.integers(2, 8), w=widths, n=st.integers(1, 6), seed=st.integers(0, 2**31 - 1),
       zero_row=st.booleans())
def test_encode_invariants(logd, w, n, seed, zero_row):
    d = 1 << logd
    rng = np.random.default_rng(seed)
    s = rng.choice([-1.0, 1.0], size=d)
    S = rng.standard_normal((d, d)).astype(np.float16)
    c, t = O.make_codebook(d, w)
    x = rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))
    if zero_row:
        x[0] = 0.0
    e = O.encode(x, s, c, t, S)
    ny = np.sqrt(np.sum(e["y"] ** 2, axis=1))
    want = np.where(e["n"] > 0, 1.0, 0.0)
    np.testing.assert_allclose(ny, want, atol=1e-12)
    assert e["idx"].min() >= 0 and e["idx"].max() < (1 << w)
    lo = np.concatenate([[-np.inf], t])[e["idx"]]
    hi = np.concatenate([t, [np.inf]])[e["idx"]]
    yf = e["y"].astype(np.float32).astype(np.float64)
    assert np.all(lo <= yf) and np.all(yf < hi)
    if zero_row:
        # norm 0, y = 0 on the middle threshold (upper cell), residual -c[L/2]
        assert e["nhat"][0] == 0 and np.all(e["idx"][0] == (1 << w) // 2)
        np.testing.assert_allclose(e["gamma"][0], np.sqrt(d) * abs(float(c[(1 << w) // 2])), rtol=1e-12)
    # one row alone encodes like the same row in the batch
    e1 = O.encode(x[-1:], s, c, t, S)
    for k in ("idx", "sigma", "nhat", "ghat"):
        np.testing.assert_array_equal(e1[k][0], e[k][-1])


@settings(max_examples=20, deadline=None)
@given(d=st.integers(3, 256), w=st.integers(1, 4))
def test_host_codebook_equals_oracle(d, w):
    c, t = tq.make_codebook(d, w)
    oc, ot = O.make_codebook(d, w)
    np.testing.assert_array_max_ulp(c.numpy(), oc.astype(np.float32), maxulp=1)
    np.testing.assert_array_max_ulp(t.numpy(), ot.astype(np.float32), maxulp=1)


@pytest.mark.parametrize("w", [1, 2, 3, 4, 5, 6, 7, 8])
def test_host_codebook_d3_is_the_uniform_grid_at_every_width(w):
    """At d = 3 one coordinate of a uniform unit vector is uniform on [-1, 1],
    whose Lloyd-Max quantizer is the uniform grid: c_j = -1 + (2 j + 1) / L.
    (The host solver once returned NaN here from 6 bits up: its start left
    (0, 1).)"""
    L = 1 << w
    c, t = tq.make_codebook(3, w)
    want = -1.0 + (2.0 * np.arange(L) + 1.0) / L
    np.testing.assert_array_max_ulp(c.numpy(), want.astype(np.float32), maxulp=1)
    np.testing.assert_array_max_ulp(t.numpy(), (-1.0 + 2.0 * np.arange(1, L) / L).astype(np.float32), maxulp=1)


@SETTINGS
@given(bits=st.floats(0.5, 6.0), n_layers=st.integers(1, 64), is_key=st.booleans())
def test_rate_plan_average(bits, n_layers, is_key):
    try:
        ref = O.rate_plan(bits, n_layers, is_key)
    except ValueError:
        ref = None
    if ref is None:
        with pytest.raises(tq.TQError) as e:
            tq.rate_plan(bits, n_layers, is_key)
        assert e.value.status == tq.TQ_EUNSUPPORTED
        return
    plan = tq.rate_plan(bits, n_layers, is_key)
    assert plan == ref
    avg = bits - (1.0 if is_key else 0.0)
    assert set(plan) <= {int(np.floor(avg)), int(np.floor(avg)) + 1}
    assert abs(sum(plan) / n_layers - avg) <= 0.5 / n_layers + 1e-12


FAKE = 1 << 20      # an aligned address that is never dereferenced


def _codec(d, w, key):
    c = tq._Codec()
    c.d, c.lm_bits, c.is_key, c.reserved = d, w, key, 0
    c.signs = c.centroids = c.thresholds = FAKE
    c.sketch = FAKE if key == 1 else None
    return c


@SETTINGS
@given(d=st.integers(-4, 300), w=st.integers(-1, 9), key=st.integers(-1, 3))
def test_malformed_codecs_are_rejected_before_launch(d, w, key):
    valid = d in (64, 128) and 1 <= w <= 4 and key in (0, 1, 2)
    if valid:
        return
    c = _codec(d, w, key)
    st_ = tq.lib.tq_encode_kv(ctypes.byref(c), ctypes.c_void_p(FAKE), tq.TQ_BF16, 1, 64, 64 * max(d, 1), max(d, 1),
                              ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 64, 0, None)
    assert st_ in (tq.TQ_EINVAL, tq.TQ_EUNSUPPORTED)
    assert tq.lib.tq_last_error().decode()
