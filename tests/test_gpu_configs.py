"""Parity on the five benchmark workloads at their full sizes, launched as the
benchmark launches them. Where the oracle cannot follow every output in
seconds, it checks deterministic samples (named in each test)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
import synthetic as syn
from gpu_common import key_codec, pack_keys_into, pack_values_into, say, to_f64, value_codec
from tq_parity import assert_close, check_key_codes, check_value_codes

pytestmark = pytest.mark.gpu


def _codecs(w):
    kc = key_codec(w.cfg, w.d, w.key_lm_bits)
    vc = value_codec(w.cfg, w.d, w.val_bits) if w.val_bits else None
    return kc, vc


def _oracle_logits(kc, q, enc, n_kv, group):
    batch = q.shape[0]
    ref = np.zeros((batch, n_kv * group, enc["idx"].shape[1]))
    for b in range(batch):
        for h in range(n_kv):
            s = b * n_kv + h
            ref[b, h * group:(h + 1) * group] = O.key_logits(
                q[b, h * group:(h + 1) * group], kc.signs, kc.centroids, kc.sketch, enc["idx"][s], enc["sigma"][s],
                enc["nhat"][s], enc["ghat"][s])
    return ref


def test_cfg1_single_head_encode_and_logits():
    w = syn.WORKLOADS[1]
    say(f"cfg1: {w.name}")
    kc, _ = _codecs(w)
    x = syn.keys(w, device="cuda")
    q = syn.queries(w, device="cuda")
    codes, scal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc.gpu)
    tq.encode_kv(kc.gpu, x, codes, scal)
    lg_gpu_codes = tq.logits(kc.gpu, q, codes, scal, n_kv_heads=1, group=w.group, n_keys=w.n_tok)
    torch.cuda.synchronize()
    enc = kc.encode(to_f64(x))
    r = check_key_codes(codes.cpu().numpy(), scal.cpu().numpy(), enc, w.key_lm_bits, kc.centroids, kc.thresholds,
                        kc.sketch, w.d)
    say("   codes:", r)
    ref = _oracle_logits(kc, to_f64(q), enc, 1, w.group)
    # given identical codes: the oracle's codes uploaded
    c2, s2 = tq.alloc_key_cache(w.n_seq, w.n_tok, kc.gpu)
    pack_keys_into(enc, w.key_lm_bits, c2, s2)
    lg = tq.logits(kc.gpu, q, c2, s2, n_kv_heads=1, group=w.group, n_keys=w.n_tok)
    torch.cuda.synchronize()
    say("   logits worst err/tol:", assert_close(lg.cpu().numpy(), ref, "cfg1 logits"))
    if r["exact"]:
        assert_close(lg_gpu_codes.cpu().numpy(), ref, "cfg1 logits from GPU codes")


def test_cfg2_decode_layer_encode_and_logits():
    w = syn.WORKLOADS[2]
    say(f"cfg2: {w.name}")
    kc, _ = _codecs(w)
    x = syn.keys(w, device="cuda")
    q = syn.queries(w, device="cuda")
    codes, scal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc.gpu)
    tq.encode_kv(kc.gpu, x, codes, scal)
    torch.cuda.synchronize()
    enc = kc.encode(to_f64(x))
    r = check_key_codes(codes.cpu().numpy(), scal.cpu().numpy(), enc, w.key_lm_bits, kc.centroids, kc.thresholds,
                        kc.sketch, w.d)
    say("   codes:", r)
    c2, s2 = tq.alloc_key_cache(w.n_seq, w.n_tok, kc.gpu)
    pack_keys_into(enc, w.key_lm_bits, c2, s2)
    lg = tq.logits(kc.gpu, q, c2, s2, n_kv_heads=w.n_kv, group=w.group, n_keys=w.n_tok)
    torch.cuda.synchronize()
    ref = _oracle_logits(kc, to_f64(q), enc, w.n_kv, w.group)
    say("   logits worst err/tol:", assert_close(lg.cpu().numpy(), ref, "cfg2 logits"))


def _decode_ref(kc, vc, q, ek, ev, lens, group):
    return O.decode_attend(q, kc.signs, kc.centroids, kc.sketch, ek["idx"], ek["sigma"], ek["nhat"], ek["ghat"],
                           vc.signs, vc.centroids, ev["idx"], ev["nhat"], lens, 1.0 / math.sqrt(kc.d), group)


def test_cfg3_batched_decode():
    w = syn.WORKLOADS[3]
    say(f"cfg3: {w.name}")
    kc, vc = _codecs(w)
    xk = syn.keys(w, device="cuda")
    xv = syn.values(w, device="cuda")
    q = syn.queries(w, device="cuda")
    kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc.gpu)
    tq.encode_kv(kc.gpu, xk, kcodes, kscal)
    tq.encode_kv(vc.gpu, xv, vcodes, vscal)
    torch.cuda.synchronize()
    ek = kc.encode(to_f64(xk))
    say("   key codes:", check_key_codes(kcodes.cpu().numpy(), kscal.cpu().numpy(), ek, w.key_lm_bits,
                                         kc.centroids, kc.thresholds, kc.sketch, w.d))
    ev = vc.encode(to_f64(xv))
    say("   value codes:", check_value_codes(vcodes.cpu().numpy(), vscal.cpu().numpy(), ev, w.val_bits,
                                             vc.thresholds, w.n_tok))
    pack_keys_into(ek, w.key_lm_bits, kcodes, kscal)
    pack_values_into(ev, w.val_bits, vcodes, vscal)
    ctx = torch.full((w.batch,), w.n_tok, dtype=torch.int32, device="cuda")
    out = tq.decode_attend(kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=w.n_kv, group=w.group,
                           max_ctx=w.n_tok, out_dtype=torch.float32)
    outb = tq.decode_attend(kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=w.n_kv,
                            group=w.group, max_ctx=w.n_tok, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = _decode_ref(kc, vc, to_f64(q), ek, ev, [w.n_tok] * w.batch, w.group)
    say("   decode worst err/tol:", assert_close(out.cpu().numpy(), ref, "cfg3 decode"))
    assert torch.equal(outb.cpu(), out.to(torch.bfloat16).cpu())


def test_cfg4_full_cache_encode_sampled():
    """The whole 22-layer cache is encoded on the GPU; the oracle checks the
    sequences of layers {0, 21} x batch rows {0, 63} x all 32 heads."""
    w = syn.WORKLOADS[4]
    say(f"cfg4: {w.name}")
    kc, vc = _codecs(w)
    xk = syn.keys(w, device="cuda")
    kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc.gpu)
    tq.encode_kv(kc.gpu, xk, kcodes, kscal)
    torch.cuda.synchronize()
    seqs = [(layer * w.batch + b) * w.n_kv + h for layer in (0, w.layers - 1) for b in (0, w.batch - 1)
            for h in range(w.n_kv)]
    sel = torch.tensor(seqs, device="cuda")
    xs = to_f64(xk[sel])
    gk, gs = kcodes[sel].cpu().numpy(), kscal[sel].cpu().numpy()
    del xk, kcodes, kscal
    torch.cuda.empty_cache()
    ek = kc.encode(xs)
    say("   key codes:", check_key_codes(gk, gs, ek, w.key_lm_bits, kc.centroids, kc.thresholds, kc.sketch, w.d))
    del ek, xs
    xv = syn.values(w, device="cuda")
    vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc.gpu)
    tq.encode_kv(vc.gpu, xv, vcodes, vscal)
    torch.cuda.synchronize()
    xs = to_f64(xv[sel])
    gv, gvs = vcodes[sel].cpu().numpy(), vscal[sel].cpu().numpy()
    del xv, vcodes, vscal
    torch.cuda.empty_cache()
    ev = vc.encode(xs)
    say("   value codes:", check_value_codes(gv, gvs, ev, w.val_bits, vc.thresholds, w.n_tok))


def test_cfg5_long_context_decode_sampled():
    """Full-size encode and decode on the GPU; the oracle checks the codes of
    sequences (b, h) in {(0, 0), (3, 7)} and the 8 query heads reading each."""
    w = syn.WORKLOADS[5]
    say(f"cfg5: {w.name}")
    kc, vc = _codecs(w)
    kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc.gpu)
    xk = syn.keys(w, device="cuda")
    tq.encode_kv(kc.gpu, xk, kcodes, kscal)
    samples = [(0, 0), (w.batch - 1, w.n_kv - 1)]
    seqs = [b * w.n_kv + h for b, h in samples]
    xks = to_f64(xk[seqs])
    del xk
    xv = syn.values(w, device="cuda")
    tq.encode_kv(vc.gpu, xv, vcodes, vscal)
    xvs = to_f64(xv[seqs])
    del xv
    q = syn.queries(w, device="cuda")
    torch.cuda.synchronize()
    ek, ev = kc.encode(xks), vc.encode(xvs)
    say("   key codes:", check_key_codes(kcodes[seqs].cpu().numpy(), kscal[seqs].cpu().numpy(), ek, w.key_lm_bits,
                                         kc.centroids, kc.thresholds, kc.sketch, w.d))
    say("   value codes:", check_value_codes(vcodes[seqs].cpu().numpy(), vscal[seqs].cpu().numpy(), ev, w.val_bits,
                                             vc.thresholds, w.n_tok))
    # identical codes for the sampled sequences, then the full launch
    pack_keys_into(ek, w.key_lm_bits, kcodes, kscal, seqs=seqs)
    pack_values_into(ev, w.val_bits, vcodes, vscal, seqs=seqs)
    ctx = torch.full((w.batch,), w.n_tok, dtype=torch.int32, device="cuda")
    out = tq.decode_attend(kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=w.n_kv, group=w.group,
                           max_ctx=w.n_tok, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qn = to_f64(q)
    for i, (b, h) in enumerate(samples):
        sub = lambda e: {k: v[i:i + 1] for k, v in e.items()}
        ref = _decode_ref(kc, vc, qn[b:b + 1, h * w.group:(h + 1) * w.group], sub(ek), sub(ev), [w.n_tok], w.group)
        got = out[b:b + 1, h * w.group:(h + 1) * w.group].cpu().numpy()
        say(f"   decode (b={b}, h={h}) worst err/tol:", assert_close(got, ref, f"cfg5 decode b={b} h={h}"))
