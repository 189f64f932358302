"""GPU parity of the fused decoding step (tq_append_decode_attend): the new
token's key and value are encoded inside the decode launch into slot
ctx_lens[b] - 1, and attention runs over the whole context.

Checked against the oracle: the new records under the parity rule (the
oracle encodes k_new / v_new), every other slot of both caches unchanged
(including the other 31 tokens of the new value's 32-token block), and the
output against the oracle's attention over the cache as the GPU left it."""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import bf16_rne, key_codec, pack_keys_into, pack_values_into, say, to_f64, value_codec
from tq_parity import EXCUSED_FRACTION, assert_close, check_index, check_key_codes, check_scalars

pytestmark = pytest.mark.gpu

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _randn(shape, seed, scale_channels=False):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if scale_channels:
        x *= torch.exp(torch.randn((shape[-1],), generator=g))
    return x


def _setup(d, kw, vw, group, batch, n_kv, T, seed):
    kc, vc = key_codec(1300 + d + kw, d, kw), value_codec(1301 + d + vw, d, vw)
    cap = ((T + 31) // 32) * 32 + 32
    k = _randn((batch * n_kv, T, d), seed, scale_channels=True).to(torch.float64)
    v = _randn((batch * n_kv, T, d), seed + 1).to(torch.float64)
    ek, ev = kc.encode(k.numpy()), vc.encode(v.numpy())
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    pack_keys_into(ek, kw, kcodes, kscal)
    pack_values_into(ev, vw, vcodes, vscal)
    return kc, vc, cap, kcodes, kscal, vcodes, vscal


def _gpu_cache(kcodes, kscal, vcodes, vscal, d, kw, cap):
    kidx, ksig = O.unpack_key_codes(kcodes.cpu().numpy(), d, kw)
    ks = kscal.cpu().numpy().view(np.float16)
    vidx = O.unpack_value_codes(vcodes.cpu().numpy().view(np.uint32), cap)
    vn = vscal.cpu().numpy().view(np.float16)
    return dict(kidx=kidx, ksigma=ksig, knhat=ks[..., 0], kghat=ks[..., 1], vidx=vidx, vnhat=vn)


def _check_step(kc, vc, kw, vw, d, n_kv, group, q, k_new, v_new, lens, before, after, out32, scale):
    """New records against the oracle encoding, other slots unchanged, the
    output against the oracle's attention over the cache after the step."""
    assert len(lens) == q.shape[0]
    batch = len(lens)
    slots = [(b * n_kv + h, lens[b] - 1) for b in range(batch) if lens[b] >= 1 for h in range(n_kv)]
    enc_k = kc.encode(to_f64(k_new).reshape(batch * n_kv, d))
    enc_v = vc.encode(to_f64(v_new).reshape(batch * n_kv, d))
    if slots:
        rows = np.array([s for s, _ in slots])
        ts = np.array([t for _, t in slots])
        sub = lambda e: {key: val[rows] for key, val in e.items()}
        kcodes, kscal = after["kcodes"], after["kscal"]
        r = check_key_codes(kcodes[rows, ts], kscal[rows, ts], sub(enc_k), kw, kc.centroids, kc.thresholds,
                            kc.sketch, d, "appended keys")
        say("   appended keys:", r)
        vidx = O.unpack_value_codes(after["vcodes"].view(np.uint32), after["vscal"].shape[1])
        ev = sub(enc_v)
        ex, _ = check_index(vidx[rows, ts], ev, vc.thresholds, "appended values idx")
        ex += check_scalars(after["vscal"].view(np.float16)[rows, ts], ev["n"], ev["nhat"], "appended values norm")
        assert ex <= max(1, EXCUSED_FRACTION * (vidx[rows, ts].size + len(rows)))
    # every other slot unchanged
    keep = np.ones(after["kscal"].shape[:2], dtype=bool)
    for s, t in slots:
        keep[s, t] = False
    np.testing.assert_array_equal(after["kcodes"][keep], before["kcodes"][keep])
    np.testing.assert_array_equal(after["kscal"][keep], before["kscal"][keep])
    np.testing.assert_array_equal(after["vscal"][keep], before["vscal"][keep])
    cap = after["vscal"].shape[1]
    vb = O.unpack_value_codes(before["vcodes"].view(np.uint32), cap)
    va = O.unpack_value_codes(after["vcodes"].view(np.uint32), cap)
    np.testing.assert_array_equal(va[keep], vb[keep])
    # output given the GPU's cache
    kidx, ksig = O.unpack_key_codes(after["kcodes"], d, kw)
    ks = after["kscal"].view(np.float16)
    ref = O.decode_attend(to_f64(q), kc.signs, kc.centroids, kc.sketch, kidx, ksig, ks[..., 0], ks[..., 1],
                          vc.signs, vc.centroids, va, after["vscal"].view(np.float16), lens, scale, group)
    return assert_close(out32.cpu().numpy(), ref, "append + decode")


def _snapshot(kcodes, kscal, vcodes, vscal):
    return dict(kcodes=kcodes.cpu().numpy(), kscal=kscal.cpu().numpy(), vcodes=vcodes.cpu().numpy(),
                vscal=vscal.cpu().numpy())


@pytest.mark.parametrize("d,kw,vw,group,batch,n_kv,T,lens,kvdt", [
    (128, 3, 4, 4, 3, 2, 700, [700, 1, 333], "bf16"),
    (128, 2, 4, 8, 2, 2, 1100, [0, 1100], "f32"),
    (64, 2, 4, 4, 2, 2, 300, [300, 65], "bf16"),
    (64, 1, 2, 1, 1, 3, 96, [96], "f16"),
    # 16 heads per KV head: two head-chunk launches, each appending the same bytes
    (128, 2, 3, 16, 1, 1, 64, [37], "bf16"),
    # 256 (batch, kv-head) groups, ragged, empty and one-token rows
    (128, 3, 4, 4, 32, 8, 1100, [1100, 1, 700, 0, 257, 1024, 1099, 513] * 4, "bf16"),
    # 5-bit keys: 256-token splits
    (128, 4, 4, 8, 2, 2, 900, [900, 512], "f32"),
    (64, 3, 4, 8, 2, 1, 1600, [1600, 1025], "bf16"),
])
def test_append_decode_attend(d, kw, vw, group, batch, n_kv, T, lens, kvdt):
    say(f"append+decode d={d} kw={kw} vw={vw} G={group} batch={batch} n_kv={n_kv} T={T} lens={lens} kv={kvdt}")
    kc, vc, cap, kcodes, kscal, vcodes, vscal = _setup(d, kw, vw, group, batch, n_kv, T, seed=d + 10 * kw + vw)
    q = _randn((batch, n_kv * group, d), 77 + group).to(torch.bfloat16)
    k_new = _randn((batch, n_kv, d), 78, scale_channels=True).to(DTYPES[kvdt])
    v_new = _randn((batch, n_kv, d), 79).to(DTYPES[kvdt])
    before = _snapshot(kcodes, kscal, vcodes, vscal)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = q.to("cuda"), k_new.to("cuda"), v_new.to("cuda")
    out32 = tq.append_decode_attend(kc.gpu, vc.gpu, qd, kd, vd, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv,
                                    group=group, max_ctx=T, sm_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    after = _snapshot(kcodes, kscal, vcodes, vscal)
    worst = _check_step(kc, vc, kw, vw, d, n_kv, group, q, k_new, v_new, lens, before, after, out32, scale)
    say("   worst err/tol", worst)
    # the same step again with bf16 output: the same bytes are appended, and
    # the output is the RNE of the fp32 one
    outb = tq.append_decode_attend(kc.gpu, vc.gpu, qd, kd, vd, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv,
                                   group=group, max_ctx=T, sm_scale=scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    again = _snapshot(kcodes, kscal, vcodes, vscal)
    for key in after:
        np.testing.assert_array_equal(again[key], after[key])
    np.testing.assert_array_equal(outb.to(torch.float64).cpu().numpy(), bf16_rne(out32.cpu().numpy()))


def test_append_matches_encode_then_decode():
    """The fused step against the two-call path (tq_encode_kv of the new token,
    then tq_decode_attend) on the same inputs: the same records wherever the
    oracle's decisions are clear of a boundary, outputs within the tolerance."""
    d, kw, vw, group, batch, n_kv, T = 128, 3, 4, 4, 4, 2, 800
    lens = [800, 513, 64, 2]
    say(f"append+decode vs encode_kv + decode_attend: batch={batch} n_kv={n_kv} lens={lens}")
    kc, vc, cap, kc1, ks1, vc1, vs1 = _setup(d, kw, vw, group, batch, n_kv, T, seed=5)
    kc2, ks2, vc2, vs2 = kc1.clone(), ks1.clone(), vc1.clone(), vs1.clone()
    q = _randn((batch, n_kv * group, d), 81).to(torch.bfloat16).to("cuda")
    k_new = _randn((batch, n_kv, d), 82, scale_channels=True).to(torch.bfloat16).to("cuda")
    v_new = _randn((batch, n_kv, d), 83).to(torch.bfloat16).to("cuda")
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    fused = tq.append_decode_attend(kc.gpu, vc.gpu, q, k_new, v_new, kc1, ks1, vc1, vs1, ctx, n_kv_heads=n_kv,
                                    group=group, max_ctx=T)
    for b in range(batch):
        t = lens[b] - 1
        sl = slice(b * n_kv, (b + 1) * n_kv)
        tq.encode_kv(kc.gpu, k_new[b][:, None, :], kc2[sl], ks2[sl], t0=t)
        tq.encode_kv(vc.gpu, v_new[b][:, None, :], vc2[sl], vs2[sl], t0=t)
    two = tq.decode_attend(kc.gpu, vc.gpu, q, kc2, ks2, vc2, vs2, ctx, n_kv_heads=n_kv, group=group, max_ctx=T)
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in ((kc1, kc2), (ks1, ks2), (vc1, vc2), (vs1, vs2)))
    say("   identical caches:", same)
    if same:
        assert_close(fused.cpu().numpy(), two.cpu().numpy(), "fused vs two calls")
    else:
        # decisions may differ only at excused boundaries: then each output
        # is checked against the oracle over its own cache instead
        for kcx, ksx, vcx, vsx, out in ((kc1, ks1, vc1, vs1, fused), (kc2, ks2, vc2, vs2, two)):
            c = _gpu_cache(kcx, ksx, vcx, vsx, d, kw, cap)
            ref = O.decode_attend(to_f64(q), kc.signs, kc.centroids, kc.sketch, c["kidx"], c["ksigma"], c["knhat"],
                                  c["kghat"], vc.signs, vc.centroids, c["vidx"], c["vnhat"], lens, 1 / math.sqrt(d),
                                  group)
            assert_close(out.cpu().numpy(), ref, "append + decode (own cache)")


def test_append_steps_replayed_in_a_hip_graph():
    """A decoding loop as a server would run it: one captured step replayed
    three times, ctx_lens advanced by one on the device between replays and
    new key/value rows written eagerly; each replay against the oracle."""
    d, kw, vw, group, batch, n_kv, T = 128, 3, 4, 4, 2, 2, 300
    lens0 = [200, 37]
    say(f"append+decode in a HIP graph: 3 steps from lens {lens0}")
    kc, vc, cap, kcodes, kscal, vcodes, vscal = _setup(d, kw, vw, group, batch, n_kv, T, seed=9)
    q = torch.empty((batch, n_kv * group, d), dtype=torch.bfloat16, device="cuda")
    k_new = torch.empty((batch, n_kv, d), dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    ctx = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    out = torch.empty((batch, n_kv * group, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.append_decode_attend_workspace(batch, n_kv, group, T, d), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(d)
    step = lambda: tq.append_decode_attend(kc.gpu, vc.gpu, q, k_new, v_new, kcodes, kscal, vcodes, vscal, ctx,
                                           n_kv_heads=n_kv, group=group, max_ctx=T, sm_scale=scale, out=out,
                                           workspace=ws)
    q.zero_(); k_new.zero_(); v_new.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up (writes slot lens0 - 1; rewritten below)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    lens = list(lens0)
    for it in range(3):
        qh = _randn((batch, n_kv * group, d), 90 + it).to(torch.bfloat16)
        kh = _randn((batch, n_kv, d), 100 + it, scale_channels=True).to(torch.bfloat16)
        vh = _randn((batch, n_kv, d), 110 + it).to(torch.bfloat16)
        q.copy_(qh.to("cuda")); k_new.copy_(kh.to("cuda")); v_new.copy_(vh.to("cuda"))
        torch.cuda.synchronize()
        before = _snapshot(kcodes, kscal, vcodes, vscal)
        g.replay()
        torch.cuda.synchronize()
        after = _snapshot(kcodes, kscal, vcodes, vscal)
        worst = _check_step(kc, vc, kw, vw, d, n_kv, group, qh, kh, vh, lens, before, after, out, scale)
        say(f"   step {it}: lens {lens} worst err/tol {worst}")
        ctx.add_(1)
        lens = [x + 1 for x in lens]


def test_prompt_chunks_then_decode_steps():
    """A serving sequence end to end: a prompt written by chunks
    (tq_encode_kv of each chunk's keys and values, then tq_prefill_attend of
    its queries), then decode steps that append one token each; every
    output against the oracle over the cache the GPU holds at that point."""
    d, kw, vw, group, batch, n_kv = 128, 3, 4, 4, 2, 2
    chunks, C, steps = 3, 24, 3
    cap = 128
    n_q = n_kv * group
    say(f"prompt of {chunks} chunks of {C} tokens, then {steps} decode steps (batch {batch})")
    kc, vc = key_codec(2100, d, kw), value_codec(2101, d, vw)
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    scale = 1.0 / math.sqrt(d)
    T = chunks * C + steps

    def oracle_cache():
        c = _snapshot(kcodes, kscal, vcodes, vscal)
        kidx, ksig = O.unpack_key_codes(c["kcodes"], d, kw)
        ks = c["kscal"].view(np.float16)
        vidx = O.unpack_value_codes(c["vcodes"].view(np.uint32), cap)
        return (kidx, ksig, ks[..., 0], ks[..., 1], vidx, c["vscal"].view(np.float16))

    for ch in range(chunks):
        t0 = ch * C
        k = _randn((batch * n_kv, C, d), 300 + ch, scale_channels=True).to(torch.bfloat16)
        v = _randn((batch * n_kv, C, d), 400 + ch).to(torch.bfloat16)
        q = _randn((batch, C, n_q, d), 500 + ch).to(torch.bfloat16)
        tq.encode_kv(kc.gpu, k.to("cuda"), kcodes, kscal, t0=t0)
        tq.encode_kv(vc.gpu, v.to("cuda"), vcodes, vscal, t0=t0)
        pos0 = torch.full((batch,), t0, dtype=torch.int32, device="cuda")
        out = tq.prefill_attend(kc.gpu, vc.gpu, q.to("cuda"), kcodes, kscal, vcodes, vscal, pos0, n_kv_heads=n_kv,
                                group=group, max_ctx=T, sm_scale=scale)
        torch.cuda.synchronize()
        kidx, ksig, kn, kg, vidx, vn = oracle_cache()
        ref = O.prefill_attend(to_f64(q), kc.signs, kc.centroids, kc.sketch, kidx, ksig, kn, kg, vc.signs,
                               vc.centroids, vidx, vn, [t0] * batch, scale, group)
        say(f"   chunk {ch}: worst err/tol {assert_close(out.cpu().numpy(), ref, 'prefill chunk')}")
    for st in range(steps):
        lens = [chunks * C + st + 1] * batch
        q = _randn((batch, n_q, d), 600 + st).to(torch.bfloat16)
        k_new = _randn((batch, n_kv, d), 700 + st, scale_channels=True).to(torch.bfloat16)
        v_new = _randn((batch, n_kv, d), 800 + st).to(torch.bfloat16)
        before = _snapshot(kcodes, kscal, vcodes, vscal)
        out = tq.append_decode_attend(kc.gpu, vc.gpu, q.to("cuda"), k_new.to("cuda"), v_new.to("cuda"), kcodes, kscal,
                                      vcodes, vscal, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                      n_kv_heads=n_kv, group=group, max_ctx=T, sm_scale=scale)
        torch.cuda.synchronize()
        after = _snapshot(kcodes, kscal, vcodes, vscal)
        worst = _check_step(kc, vc, kw, vw, d, n_kv, group, q, k_new, v_new, lens, before, after, out, scale)
        say(f"   step {st}: worst err/tol {worst}")
