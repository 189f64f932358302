"""Exact ties on the Lloyd-Max thresholds, through both encoding entry points.

The C header states one decision rule for every encoding entry point: the
sign of the rotated coordinate gives the top index bit (either zero counts
as positive) and its magnitude is compared with the upper half's thresholds,
so a positive coordinate equal to a threshold takes the upper cell and a
negative one the lower cell. Both tq_encode_kv and the append inside
tq_append_decode_attend must follow it bit for bit.

Exact ties are made with a codebook whose thresholds are dyadic
({-0.5, 0, 0.5}, centroids {+-0.25, +-0.75}) and inputs built backwards from
a rotated vector v with small integer entries and ||v|| = 8: x = diag(s) H v / d
is exact in fp32 and bf16, every step of the rotation is exact, and v_i = +-4
sits exactly on the scaled threshold 0.5 * ||v||. The oracle (whose reading
sends every exact tie to the upper cell) then differs from the GPU exactly on
the negative ties, which the parity rule excuses because they lie on a
boundary."""
import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import say, to_f64
from tq_parity import BOUNDARY_EPS, check_index, check_scalars

pytestmark = pytest.mark.gpu

C = np.array([-0.75, -0.25, 0.25, 0.75], dtype=np.float32)
T = np.array([-0.5, 0.0, 0.5], dtype=np.float32)


def _rotated_rows(d):
    """Rotated vectors v (rows), every one with ||v|| = 8 and ties at +-4."""
    rows = []
    v = np.zeros(d); v[[0, 1, 2, 3]] = [-4, 4, 4, -4]; rows.append(v)
    v = np.zeros(d); v[5], v[9] = 4, -4; v[10:18] = [2, -2, 2, -2, 2, -2, 2, -2]; rows.append(v)
    v = np.zeros(d); v[[d // 2, d - 1, d - 28, 33]] = [-4, -4, 4, 4]; rows.append(v)
    v = np.zeros(d); v[[7, 8]] = [-4, -4]; v[20:28] = [-2, -2, -2, -2, 2, 2, 2, 2]; rows.append(v)
    return np.stack(rows)


def _expected_idx(v):
    """The header's rule on y = v / ||v|| (exact here): sign, then |y| against 0.5."""
    y = v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    j = (np.abs(y) >= 0.5).astype(np.int64)
    return np.where(y >= 0, 2 + j, 1 - j)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_exact_ties_same_cells_in_encode_and_append(d, dt):
    say(f"exact ties d={d} dtype={dt}: tq_encode_kv and tq_append_decode_attend, 4 rows")
    rng = np.random.default_rng(4242 + d)
    s = rng.choice([-1.0, 1.0], size=d)
    sv = rng.choice([-1.0, 1.0], size=d)
    S = rng.standard_normal((d, d)).astype(np.float16)
    H = O.hadamard(d)
    v = _rotated_rows(d)
    n_rows = v.shape[0]
    xk = (v @ H.T) * s / d              # diag(s) H v / d (H symmetric)
    xv = (v @ H.T) * sv / d
    assert np.all(np.asarray(torch.from_numpy(xk).to(dt).double()) == xk)    # exact in the input type
    want = _expected_idx(v)
    assert np.any(want == 0) and np.any(want == 3)                           # ties on both sides

    kc = tq.Codec.make(d, 2, True, s, torch.from_numpy(S), device="cuda", centroids=C, thresholds=T)
    vc = tq.Codec.make(d, 2, False, sv, device="cuda", centroids=C, thresholds=T)
    xk_t = torch.from_numpy(xk).to(dt).cuda()
    xv_t = torch.from_numpy(xv).to(dt).cuda()

    # tq_encode_kv: one token per sequence at slot 0
    cap = 64
    kcodes, kscal = tq.alloc_key_cache(n_rows, cap, kc)
    vcodes, vscal = tq.alloc_value_cache(n_rows, cap, vc)
    tq.encode_kv(kc, xk_t.view(n_rows, 1, d), kcodes, kscal)
    tq.encode_kv(vc, xv_t.view(n_rows, 1, d), vcodes, vscal)

    # the append: sequence b's new token into slot ctx_lens[b] - 1
    lens = [1, 17, 40, 64]
    group = 4
    akc, aks = tq.alloc_key_cache(n_rows, cap, kc)
    avc, avs = tq.alloc_value_cache(n_rows, cap, vc)
    g = torch.Generator(device="cpu")
    g.manual_seed(d)
    q = torch.randn((n_rows, group, d), generator=g).to(dt).cuda()
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    tq.append_decode_attend(kc, vc, q, xk_t.view(n_rows, 1, d), xv_t.view(n_rows, 1, d), akc, aks, avc, avs, ctx,
                            n_kv_heads=1, group=group, max_ctx=cap)
    torch.cuda.synchronize()

    rows = np.arange(n_rows)
    slots = np.array(lens) - 1
    e_idx, e_sig = O.unpack_key_codes(kcodes[:, 0].cpu().numpy(), d, 2)
    a_idx, a_sig = O.unpack_key_codes(akc.cpu().numpy()[rows, slots], d, 2)
    np.testing.assert_array_equal(e_idx, want)
    np.testing.assert_array_equal(a_idx, want)
    ev_idx = O.unpack_value_codes(vcodes.cpu().numpy().view(np.uint32), cap)[:, 0]
    av_idx = O.unpack_value_codes(avc.cpu().numpy().view(np.uint32), cap)[rows, slots]
    np.testing.assert_array_equal(ev_idx, want)
    np.testing.assert_array_equal(av_idx, want)
    # the stored scalars agree between the two entry points
    np.testing.assert_array_equal(kscal[:, 0].cpu().numpy(), aks.cpu().numpy()[rows, slots])
    np.testing.assert_array_equal(vscal[:, 0].cpu().numpy(), avs.cpu().numpy()[rows, slots])

    # against the oracle: the negative ties are the only index differences
    # (the oracle sends them to the upper cell), each on its threshold; the
    # rest of each key (residual norm, sign bits) is checked with the GPU's
    # indices
    enc_k = O.encode(to_f64(xk_t), s, C, T, S)
    enc_v = O.encode(to_f64(xv_t), sv, C, T)
    # (coordinates where v = 0 may come out of the oracle's fp64 rotation as
    # a tiny number of either sign instead of zero, on the middle threshold)
    neg_tie = v == -4
    for e in (enc_k, enc_v):
        diff = e["idx"] != want
        assert np.all(diff[neg_tie]) and np.all(e["idx"][neg_tie] == 1)
        assert not np.any(diff & ~neg_tie & (v != 0))
    for name, codes, scal in (("encode", kcodes[:, 0].cpu().numpy(), kscal[:, 0].cpu().numpy()),
                              ("append", akc.cpu().numpy()[rows, slots], aks.cpu().numpy()[rows, slots])):
        gidx, gsig = O.unpack_key_codes(codes, d, 2)
        ex, _ = check_index(gidx, enc_k, T, f"{name} keys idx")
        assert ex == int((enc_k["idx"] != want).sum())
        rq = O.requantize_key(enc_k["y"], gidx, C, S)
        hard = (gsig != rq["sigma"]) & (np.abs(rq["z"]) > BOUNDARY_EPS)
        assert not np.any(hard), f"{name}: sign bits away from zero differ"
        gsc = scal.view(np.float16)
        check_scalars(gsc[:, 0], enc_k["n"], enc_k["nhat"], f"{name} keys norm")
        check_scalars(gsc[:, 1], rq["gamma"], rq["ghat"], f"{name} keys gamma")
        say(f"   {name} keys vs oracle: {ex} excused ties")
    for name, vi in (("encode", ev_idx), ("append", av_idx)):
        ex, _ = check_index(vi, enc_v, T, f"{name} values idx")
        assert ex == int((enc_v["idx"] != want).sum())
