"""GPU parity of causal prefill-chunk attention over the coded cache
(tq_prefill_attend): given the oracle's codes for every cached token
(including the chunk's own), outputs against the oracle's masked softmax
attention within the logit tolerance; a one-position chunk against
tq_decode_attend bit for bit (the same kernels)."""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import bf16_rne, key_codec, pack_keys_into, pack_values_into, say, to_f64, value_codec
from tq_parity import assert_close

pytestmark = pytest.mark.gpu


def _cache(d, kw, vw, batch, n_kv, T, seed):
    kc, vc = key_codec(1400 + d + kw, d, kw), value_codec(1401 + d + vw, d, vw)
    cap = ((T + 31) // 32) * 32
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    k = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float64)
    k *= torch.exp(torch.randn((d,), generator=g, dtype=torch.float64))
    v = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float64)
    ek, ev = kc.encode(k.numpy()), vc.encode(v.numpy())
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    pack_keys_into(ek, kw, kcodes, kscal)
    pack_values_into(ev, vw, vcodes, vscal)
    return kc, vc, ek, ev, (kcodes, kscal, vcodes, vscal), g


@pytest.mark.parametrize("d,kw,vw,group,batch,n_kv,T,chunk,pos0", [
    (128, 3, 4, 4, 2, 2, 700, 16, [600, 100]),      # 64 (position, head) pairs: 8 launches
    (128, 2, 4, 8, 1, 2, 1100, 7, [1000]),          # 56 pairs: a ragged last launch
    (64, 2, 4, 4, 2, 2, 300, 5, [0, 250]),          # a sequence's first chunk
    (128, 2, 3, 1, 3, 1, 96, 33, [0, 40, 63]),      # one head per KV head
    (128, 4, 4, 2, 1, 1, 1300, 12, [1200]),         # 5-bit keys: 256-token splits
    (64, 3, 4, 8, 2, 1, 1600, 9, [1591, 513]),
])
def test_prefill_attend_given_oracle_codes(d, kw, vw, group, batch, n_kv, T, chunk, pos0):
    say(f"prefill d={d} kw={kw} vw={vw} G={group} batch={batch} n_kv={n_kv} T={T} chunk={chunk} pos0={pos0}")
    kc, vc, ek, ev, cache, g = _cache(d, kw, vw, batch, n_kv, T, seed=d + kw + 10 * chunk)
    q = torch.randn((batch, chunk, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    p0 = torch.tensor(pos0, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    qd = q.to("cuda")
    out32 = tq.prefill_attend(kc.gpu, vc.gpu, qd, *cache, p0, n_kv_heads=n_kv, group=group, max_ctx=T,
                              sm_scale=scale, out_dtype=torch.float32)
    outb = tq.prefill_attend(kc.gpu, vc.gpu, qd, *cache, p0, n_kv_heads=n_kv, group=group, max_ctx=T,
                             sm_scale=scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = O.prefill_attend(to_f64(q), kc.signs, kc.centroids, kc.sketch, ek["idx"], ek["sigma"], ek["nhat"],
                           ek["ghat"], vc.signs, vc.centroids, ev["idx"], ev["nhat"], pos0, scale, group)
    worst = assert_close(out32.cpu().numpy(), ref, "prefill f32")
    say("   worst err/tol", worst)
    np.testing.assert_array_equal(outb.to(torch.float64).cpu().numpy(), bf16_rne(out32.cpu().numpy()))


def test_one_position_chunk_is_decode():
    """chunk = 1 runs the decode kernels with the same heads and context
    (ctx_lens = pos0 + 1): outputs identical bit for bit."""
    d, kw, vw, group, batch, n_kv, T = 128, 3, 4, 4, 4, 2, 900
    pos0 = [899, 0, 511, 300]
    say(f"prefill chunk=1 vs decode: pos0={pos0}")
    kc, vc, ek, ev, cache, g = _cache(d, kw, vw, batch, n_kv, T, seed=3)
    q = torch.randn((batch, 1, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16).to("cuda")
    pre = tq.prefill_attend(kc.gpu, vc.gpu, q, *cache, torch.tensor(pos0, dtype=torch.int32, device="cuda"),
                            n_kv_heads=n_kv, group=group, max_ctx=T)
    dec = tq.decode_attend(kc.gpu, vc.gpu, q[:, 0], *cache,
                           torch.tensor([p + 1 for p in pos0], dtype=torch.int32, device="cuda"), n_kv_heads=n_kv,
                           group=group, max_ctx=T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pre[:, 0].cpu().numpy(), dec.cpu().numpy())


@pytest.mark.parametrize("d,kw,vw,group,batch,n_kv,T,chunk,pos0", [
    (128, 2, 4, 4, 2, 2, 1000, 16, [984, 0]),       # 64 pairs; the chunk ends at max_ctx
    (128, 3, 4, 4, 1, 1, 500, 25, [475]),           # 100 pairs: blocks of 64 and 36 pairs
    (64, 1, 2, 16, 1, 2, 300, 4, [100]),            # 1-bit keys, 2-bit values
    (128, 4, 3, 8, 1, 1, 257, 8, [249]),            # 5-bit keys, 3-bit values
    (64, 4, 1, 2, 2, 1, 130, 11, [0, 119]),         # 1-bit values
])
def test_single_pass_prefill_given_oracle_codes(d, kw, vw, group, batch, n_kv, T, chunk, pos0):
    """More than 8 (position, head) pairs per KV head: one scan of the context
    per 64 pairs (values on the fp16 matrix cores), against the oracle."""
    say(f"single-pass prefill d={d} kw={kw} vw={vw} G={group} batch={batch} n_kv={n_kv} T={T} chunk={chunk} "
        f"pos0={pos0}")
    kc, vc, ek, ev, cache, g = _cache(d, kw, vw, batch, n_kv, T, seed=7 * d + kw + chunk)
    q = torch.randn((batch, chunk, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    p0 = torch.tensor(pos0, dtype=torch.int32, device="cuda")
    scale = 0.7 / math.sqrt(d)
    out = tq.prefill_attend(kc.gpu, vc.gpu, q.to("cuda"), *cache, p0, n_kv_heads=n_kv, group=group, max_ctx=T,
                            sm_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.prefill_attend(to_f64(q), kc.signs, kc.centroids, kc.sketch, ek["idx"], ek["sigma"], ek["nhat"],
                           ek["ghat"], vc.signs, vc.centroids, ev["idx"], ev["nhat"], pos0, scale, group)
    say("   worst err/tol", assert_close(out.cpu().numpy(), ref, "single-pass prefill"))


def test_prefill_batched_decode_shape_sampled():
    """The batched-decode cache shape (16 x 8 KV heads x 8192 tokens, 32 query
    heads, 3-bit keys, 4-bit values) with a 16-token chunk at its end, caches
    encoded on the GPU: two sampled (batch row, KV head) groups against the
    oracle over the GPU's codes."""
    import synthetic as syn
    w = syn.WORKLOADS[3]
    d, chunk = w.d, 16
    say(f"prefill chunk {chunk} on {w.name}")
    s, S = syn.key_codec_randoms(w.cfg, d)
    kc = tq.Codec.make(d, w.key_lm_bits, True, s, S, device="cuda")
    vc = tq.Codec.make(d, w.val_bits, False, syn.value_codec_randoms(w.cfg, d), device="cuda")
    kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
    vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc)
    x = syn.keys(w, device="cuda")
    tq.encode_kv(kc, x, kcodes, kscal)
    del x
    x = syn.values(w, device="cuda")
    tq.encode_kv(vc, x, vcodes, vscal)
    del x
    g = torch.Generator(device="cpu")
    g.manual_seed(33)
    q = torch.randn((w.batch, chunk, w.n_q, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    pos0 = [w.n_tok - chunk - 37 * b for b in range(w.batch)]
    p0 = torch.tensor(pos0, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = tq.prefill_attend(kc, vc, q.to("cuda"), kcodes, kscal, vcodes, vscal, p0, n_kv_heads=w.n_kv,
                            group=w.group, max_ctx=w.n_tok, sm_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cs, cv = O.make_codebook(d, w.key_lm_bits), O.make_codebook(d, w.val_bits)
    for b, kvh in ((0, 0), (w.batch - 1, w.n_kv - 1)):
        sq = b * w.n_kv + kvh
        kidx, ksig = O.unpack_key_codes(kcodes[sq].cpu().numpy(), d, w.key_lm_bits)
        ks = kscal[sq].cpu().numpy().view(np.float16)
        vidx = O.unpack_value_codes(vcodes[sq:sq + 1].cpu().numpy().view(np.uint32), w.n_tok)
        vn = vscal[sq:sq + 1].cpu().numpy().view(np.float16)
        heads = slice(kvh * w.group, (kvh + 1) * w.group)
        ref = O.prefill_attend(to_f64(q[b:b + 1, :, heads]), s.numpy(), cs[0], S.numpy(), kidx[None], ksig[None],
                               ks[None, :, 0], ks[None, :, 1], syn.value_codec_randoms(w.cfg, d).numpy(), cv[0],
                               vidx, vn, [pos0[b]], scale, w.group)
        say(f"   group (b={b}, kv={kvh}) worst err/tol",
            assert_close(out[b:b + 1, :, heads].cpu().numpy(), ref, f"prefill b={b} kv={kvh}"))
