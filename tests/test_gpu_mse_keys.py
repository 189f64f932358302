"""GPU parity of the MSE-only key cache format (codec is_key = 2: key records
of w index planes and an fp16 norm, no QJL sign plane and no residual norm),
through every call that reads or writes keys.

- tq_encode_kv: the records against the oracle under the parity rule, and
  equal bit for bit to the first w planes and the norm of the full key
  records that the same input encodes to (the same decisions).
- tq_logits / tq_prepare_queries + tq_logits_prepared: given the oracle's
  codes, against the oracle's first-term estimate (key_logits_mse).
- tq_decode_attend, tq_prefill_attend, tq_append_decode_attend: against the
  oracle's attention over MSE-only keys (sketch None), given the GPU's codes.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import (bf16_rne, key_codec, mse_key_codec, pack_mse_keys_into, pack_values_into, say, to_f64,
                        value_codec)
from tq_parity import EXCUSED_FRACTION, assert_close, check_index, check_scalars

pytestmark = pytest.mark.gpu


def _keys(shape, seed, dtype):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    x *= torch.exp(torch.randn((shape[-1],), generator=g))          # lognormal channel scales
    return x.to(dtype)


def _check_mse_records(codes, scal, enc, kc, what):
    gidx = O.unpack_mse_key_codes(codes, kc.d, kc.lm_bits)
    ex, _ = check_index(gidx, enc, kc.thresholds, what + " idx")
    ex += check_scalars(np.asarray(scal).view(np.float16)[..., 0], enc["n"], enc["nhat"], what + " norm")
    n_items = gidx.size + gidx.shape[0] * gidx.shape[1]
    assert ex <= max(1, EXCUSED_FRACTION * n_items), f"{what}: {ex} excused of {n_items}"
    return ex


@pytest.mark.parametrize("d,w,dt", [(128, 3, torch.bfloat16), (128, 2, torch.float32), (64, 2, torch.bfloat16),
                                    (64, 4, torch.float16), (128, 1, torch.bfloat16)])
def test_mse_key_encode_against_oracle_and_full_records(d, w, dt):
    n_seq, n_tok, t0 = 3, 1995, 5
    cap = 2016
    say(f"MSE-only key encode d={d} w={w} {dt}: {n_seq} x {n_tok} tokens at t0={t0}")
    full = key_codec(1500 + d + w, d, w)
    mse = mse_key_codec(1500 + d + w, d, w)
    assert mse.gpu.record_bytes == w * d // 8 and mse.gpu.key_scalars == 1
    x = _keys((n_seq, n_tok, d), d + w, dt)
    xd = x.to("cuda")
    mcodes, mscal = tq.alloc_key_cache(n_seq, cap, mse.gpu)
    fcodes, fscal = tq.alloc_key_cache(n_seq, cap, full.gpu)
    mcodes.fill_(0x5A)
    mscal.fill_(0x1234)
    tq.encode_kv(mse.gpu, xd, mcodes, mscal, t0=t0)
    tq.encode_kv(full.gpu, xd, fcodes, fscal, t0=t0)
    torch.cuda.synchronize()
    mc, ms = mcodes.cpu().numpy(), mscal.cpu().numpy()
    fc, fs = fcodes.cpu().numpy(), fscal.cpu().numpy()
    sl = slice(t0, t0 + n_tok)
    np.testing.assert_array_equal(mc[:, sl], fc[:, sl, :w * d // 8])
    np.testing.assert_array_equal(ms[:, sl, 0], fs[:, sl, 0])
    # slots outside the range untouched
    assert np.all(mc[:, :t0] == 0x5A) and np.all(mc[:, t0 + n_tok:] == 0x5A)
    assert np.all(ms[:, :t0] == 0x1234) and np.all(ms[:, t0 + n_tok:] == 0x1234)
    enc = mse.encode(to_f64(x))
    ex = _check_mse_records(mc[:, sl], ms[:, sl], enc, mse, "MSE-only keys")
    say(f"   {ex} excused boundary items")


@pytest.mark.parametrize("d,w,group,batch,n_kv,n_keys", [
    (128, 3, 4, 1, 8, 1999),        # the decode-layer shape, ragged tail
    (128, 2, 1, 1, 1, 4096),        # single head
    (128, 4, 8, 2, 1, 700),
    (64, 3, 4, 2, 2, 333),
    (64, 1, 16, 1, 1, 64),
    (128, 3, 32, 1, 1, 515),        # four head chunks
])
def test_mse_key_logits_given_oracle_codes(d, w, group, batch, n_kv, n_keys):
    say(f"MSE-only key logits d={d} w={w} G={group} batch={batch} n_kv={n_kv} n_keys={n_keys}")
    kc = mse_key_codec(1600 + d + w, d, w)
    cap = (n_keys + 31) // 32 * 32
    g = torch.Generator(device="cpu")
    g.manual_seed(d * w + group)
    k = torch.randn((batch * n_kv, n_keys, d), generator=g, dtype=torch.float64)
    q = torch.randn((batch, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    enc = kc.encode(k.numpy())
    codes, scal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    pack_mse_keys_into(enc, w, codes, scal)
    qd = q.to("cuda")
    out = tq.logits(kc.gpu, qd, codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys)
    prep = tq.prepare_queries(kc.gpu, qd, n_kv_heads=n_kv, group=group)
    outp = tq.logits_prepared(kc.gpu, prep, batch, codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys)
    torch.cuda.synchronize()
    qn = to_f64(q)
    ref = np.zeros((batch, n_kv * group, n_keys))
    for b in range(batch):
        for h in range(n_kv):
            s = b * n_kv + h
            ref[b, h * group:(h + 1) * group] = O.key_logits_mse(qn[b, h * group:(h + 1) * group], kc.signs,
                                                                 kc.centroids, enc["idx"][s], enc["nhat"][s])
    worst = assert_close(out.cpu().numpy(), ref, "MSE-only key logits")
    say("   worst err/tol", worst)
    np.testing.assert_array_equal(outp.cpu().numpy(), out.cpu().numpy())


def _mse_cache(d, kw, vw, batch, n_kv, T, seed, cap_extra=0):
    kc, vc = mse_key_codec(1700 + d + kw, d, kw), value_codec(1701 + d + vw, d, vw)
    cap = ((T + 31) // 32) * 32 + cap_extra
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    k = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float64)
    k *= torch.exp(torch.randn((d,), generator=g, dtype=torch.float64))
    v = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float64)
    ek, ev = kc.encode(k.numpy()), vc.encode(v.numpy())
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    pack_mse_keys_into(ek, kw, kcodes, kscal)
    pack_values_into(ev, vw, vcodes, vscal)
    return kc, vc, ek, ev, (kcodes, kscal, vcodes, vscal), g, cap


@pytest.mark.parametrize("d,kw,vw,group,batch,n_kv,T,lens", [
    (128, 3, 4, 4, 2, 2, 1500, [1500, 777]),
    (128, 4, 4, 8, 2, 1, 2100, [2100, 1]),          # two row groups of 4 heads
    (64, 2, 4, 4, 3, 2, 600, [600, 0, 313]),        # an empty row
    (128, 2, 3, 1, 2, 1, 96, [96, 40]),
])
def test_mse_key_decode_given_oracle_codes(d, kw, vw, group, batch, n_kv, T, lens):
    say(f"MSE-only key decode d={d} kw={kw} vw={vw} G={group} batch={batch} n_kv={n_kv} T={T} lens={lens}")
    kc, vc, ek, ev, cache, g, cap = _mse_cache(d, kw, vw, batch, n_kv, T, seed=d + kw + group)
    q = torch.randn((batch, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out32 = tq.decode_attend(kc.gpu, vc.gpu, q.to("cuda"), *cache, ctx, n_kv_heads=n_kv, group=group, max_ctx=T,
                             sm_scale=scale, out_dtype=torch.float32)
    outb = tq.decode_attend(kc.gpu, vc.gpu, q.to("cuda"), *cache, ctx, n_kv_heads=n_kv, group=group, max_ctx=T,
                            sm_scale=scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = O.decode_attend(to_f64(q), kc.signs, kc.centroids, None, ek["idx"], None, ek["nhat"], None, vc.signs,
                          vc.centroids, ev["idx"], ev["nhat"], lens, scale, group)
    worst = assert_close(out32.cpu().numpy(), ref, "MSE-only key decode f32")
    say("   worst err/tol", worst)
    np.testing.assert_array_equal(outb.to(torch.float64).cpu().numpy(), bf16_rne(out32.cpu().numpy()))


@pytest.mark.parametrize("d,kw,vw,group,batch,n_kv,T,chunk,pos0", [
    (128, 3, 4, 4, 2, 2, 700, 16, [600, 100]),
    (64, 2, 4, 8, 1, 2, 300, 5, [0]),
])
def test_mse_key_prefill_given_oracle_codes(d, kw, vw, group, batch, n_kv, T, chunk, pos0):
    say(f"MSE-only key prefill d={d} kw={kw} vw={vw} G={group} batch={batch} T={T} chunk={chunk} pos0={pos0}")
    kc, vc, ek, ev, cache, g, cap = _mse_cache(d, kw, vw, batch, n_kv, T, seed=3 * d + kw)
    q = torch.randn((batch, chunk, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    p0 = torch.tensor(pos0, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = tq.prefill_attend(kc.gpu, vc.gpu, q.to("cuda"), *cache, p0, n_kv_heads=n_kv, group=group, max_ctx=T,
                            sm_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.prefill_attend(to_f64(q), kc.signs, kc.centroids, None, ek["idx"], None, ek["nhat"], None, vc.signs,
                           vc.centroids, ev["idx"], ev["nhat"], pos0, scale, group)
    say("   worst err/tol", assert_close(out.cpu().numpy(), ref, "MSE-only key prefill"))


@pytest.mark.parametrize("d,kw,vw,group,batch,n_kv,T,lens", [
    (128, 3, 4, 4, 2, 2, 900, [900, 33]),
    (64, 2, 3, 8, 2, 1, 200, [1, 0]),
])
def test_mse_key_append_step(d, kw, vw, group, batch, n_kv, T, lens):
    """The appended key record equals tq_encode_kv's for the same row, bit for
    bit; the other slots stay; the output matches the oracle's attention over
    the cache the GPU left."""
    say(f"MSE-only key append d={d} kw={kw} vw={vw} G={group} batch={batch} n_kv={n_kv} lens={lens}")
    kc, vc, ek, ev, cache, g, cap = _mse_cache(d, kw, vw, batch, n_kv, T, seed=5 * d + kw, cap_extra=32)
    kcodes, kscal, vcodes, vscal = cache
    before_k, before_s = kcodes.cpu().numpy().copy(), kscal.cpu().numpy().copy()
    q = torch.randn((batch, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k_new = torch.randn((batch, n_kv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v_new = torch.randn((batch, n_kv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = tq.append_decode_attend(kc.gpu, vc.gpu, q.to("cuda"), k_new.to("cuda"), v_new.to("cuda"), kcodes, kscal,
                                  vcodes, vscal, ctx, n_kv_heads=n_kv, group=group, max_ctx=cap, sm_scale=scale,
                                  out_dtype=torch.float32)
    # the same rows through tq_encode_kv into a scratch cache
    ecodes, escal = tq.alloc_key_cache(batch * n_kv, 32, kc.gpu)
    tq.encode_kv(kc.gpu, k_new.to("cuda").view(batch * n_kv, 1, d), ecodes, escal)
    torch.cuda.synchronize()
    after_k, after_s = kcodes.cpu().numpy(), kscal.cpu().numpy()
    keep = np.ones(after_s.shape[:2], dtype=bool)
    for b in range(batch):
        if lens[b] < 1:
            continue
        for h in range(n_kv):
            s, t = b * n_kv + h, lens[b] - 1
            np.testing.assert_array_equal(after_k[s, t], ecodes.cpu().numpy()[s, 0])
            np.testing.assert_array_equal(after_s[s, t], escal.cpu().numpy()[s, 0])
            keep[s, t] = False
    np.testing.assert_array_equal(after_k[keep], before_k[keep])
    np.testing.assert_array_equal(after_s[keep], before_s[keep])
    kidx = O.unpack_mse_key_codes(after_k, d, kw)
    vidx = O.unpack_value_codes(vcodes.cpu().numpy().view(np.uint32), cap)
    ref = O.decode_attend(to_f64(q), kc.signs, kc.centroids, None, kidx, None, after_s.view(np.float16)[..., 0],
                          None, vc.signs, vc.centroids, vidx, vscal.cpu().numpy().view(np.float16), lens, scale,
                          group)
    say("   worst err/tol", assert_close(out.cpu().numpy(), ref, "MSE-only key append"))
