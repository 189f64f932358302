"""GPU parity against the CPU oracle on small, ragged and edge-case inputs.

Sizes span several 64-token tiles and value blocks with ragged tails; each
test names its case before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
import synthetic as syn
from gpu_common import CodecPair, bf16_rne, key_codec, pack_keys_into, pack_values_into, say, to_f64, \
    value_codec
from tq_parity import assert_close, check_key_codes, check_value_codes

pytestmark = pytest.mark.gpu

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _inputs(n_seq, n_tok, d, dtype, seed, stream=1, scale_channels=False):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed * 7919 + stream)
    x = torch.randn((n_seq, n_tok, d), generator=g, device="cuda", dtype=torch.float32)
    if scale_channels:
        x *= torch.exp(torch.randn((1, 1, d), generator=g, device="cuda"))
    return x.to(dtype)


# ------------------------------------------------------------------ encode


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w", [1, 2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_encode_keys(d, w, dt):
    # 3 x 2000 tokens: about 1e6 coded items at d = 128, so that the parity
    # rule's budget of 1e-5 excused boundary cases is more than one item
    say(f"encode keys d={d} w={w} dtype={dt} n_seq=3 n_tok=2000 t0=37")
    kc = key_codec(100 + d + w, d, w)
    n_seq, n_tok, t0, cap = 3, 2000, 37, 2080
    x = _inputs(n_seq, n_tok, d, DTYPES[dt], seed=d * 10 + w, scale_channels=True)
    codes, scal = tq.alloc_key_cache(n_seq, cap, kc.gpu)
    tq.encode_kv(kc.gpu, x, codes, scal, t0=t0)
    torch.cuda.synchronize()
    enc = kc.encode(to_f64(x))
    r = check_key_codes(codes[:, t0:t0 + n_tok].cpu().numpy(), scal[:, t0:t0 + n_tok].cpu().numpy(), enc, w,
                        kc.centroids, kc.thresholds, kc.sketch, d)
    say("  ", r)
    # slots outside the written range stay untouched
    assert not codes[:, :t0].any() and not codes[:, t0 + n_tok:].any()
    assert not scal[:, :t0].any() and not scal[:, t0 + n_tok:].any()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w", [1, 2, 3, 4])
def test_encode_values_merges_partial_blocks(d, w):
    say(f"encode values d={d} w={w} n_seq=2 n_tok=150 t0=45 over a random cache")
    vc = value_codec(200 + d + w, d, w)
    n_seq, n_tok, t0, cap = 2, 150, 45, 256
    x = _inputs(n_seq, n_tok, d, torch.bfloat16, seed=d + w, stream=2)
    codes, scal = tq.alloc_value_cache(n_seq, cap, vc.gpu)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    before = torch.randint(-2 ** 31, 2 ** 31 - 1, codes.shape, generator=g, device="cuda", dtype=torch.int64)
    codes.copy_(before.to(torch.int32))
    before = codes.clone()
    tq.encode_kv(vc.gpu, x, codes, scal, t0=t0)
    torch.cuda.synchronize()
    enc = vc.encode(to_f64(x))
    words = codes.cpu().numpy().view(np.uint32)
    r = check_value_codes(words, scal.cpu().numpy(), enc, w, vc.thresholds, n_tok, t0=t0)
    say("  ", r)
    # bits of slots outside [t0, t0 + n_tok) are preserved
    old = O.unpack_value_codes(before.cpu().numpy().view(np.uint32), cap)
    new = O.unpack_value_codes(words, cap)
    np.testing.assert_array_equal(new[:, :t0], old[:, :t0])
    np.testing.assert_array_equal(new[:, t0 + n_tok:], old[:, t0 + n_tok:])


def test_append_one_token_per_call_equals_prefill():
    say("append: 70 single-token encodes vs one prefill, keys w=2 and values w=4, d=128")
    d = 128
    kc, vc = key_codec(300, d, 2), value_codec(301, d, 4)
    x = _inputs(2, 70, d, torch.bfloat16, seed=9)
    cap = 96
    k1, ks1 = tq.alloc_key_cache(2, cap, kc.gpu)
    k2, ks2 = tq.alloc_key_cache(2, cap, kc.gpu)
    v1, vs1 = tq.alloc_value_cache(2, cap, vc.gpu)
    v2, vs2 = tq.alloc_value_cache(2, cap, vc.gpu)
    tq.encode_kv(kc.gpu, x, k1, ks1)
    tq.encode_kv(vc.gpu, x, v1, vs1)
    for t in range(70):
        tq.encode_kv(kc.gpu, x[:, t:t + 1], k2, ks2, t0=t)
        tq.encode_kv(vc.gpu, x[:, t:t + 1], v2, vs2, t0=t)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(ks1, ks2)
    assert torch.equal(v1, v2) and torch.equal(vs1, vs2)


def test_encode_zero_and_structured_vectors():
    """Zero rows (norm 0) and rows with exact ties after the transform
    (e1 + e2 rotates to coordinates that are exactly 0 or +-2/sqrt(2d))."""
    say("encode edge rows: zeros, e1, e1+e2, constant rows; keys w=2, values w=2, d=64")
    d = 64
    kc, vc = key_codec(400, d, 2), value_codec(401, d, 2)
    rows = np.zeros((1, 6, d), dtype=np.float32)
    rows[0, 1, 0] = 1.0
    rows[0, 2, 0] = rows[0, 2, 1] = 1.0
    rows[0, 3, :] = 1.0
    rows[0, 4, :] = -3.5
    rows[0, 5, 5] = 1e-3
    x = torch.from_numpy(rows).cuda()
    codes, scal = tq.alloc_key_cache(1, 64, kc.gpu)
    tq.encode_kv(kc.gpu, x, codes, scal)
    vcodes, vscal = tq.alloc_value_cache(1, 64, vc.gpu)
    tq.encode_kv(vc.gpu, x, vcodes, vscal)
    torch.cuda.synchronize()
    enc = kc.encode(rows.astype(np.float64))
    check_key_codes(codes[:, :6].cpu().numpy(), scal[:, :6].cpu().numpy(), enc, 2, kc.centroids, kc.thresholds,
                    kc.sketch, d)
    encv = vc.encode(rows.astype(np.float64))
    check_value_codes(vcodes.cpu().numpy(), vscal.cpu().numpy(), encv, 2, vc.thresholds, 6)
    assert scal[0, 0, 0].item() == 0 and vscal[0, 0].item() == 0


def test_encode_is_deterministic():
    say("determinism: two encodes of the same 4x1000 keys, d=128 w=3")
    kc = key_codec(500, 128, 3)
    x = _inputs(4, 1000, 128, torch.bfloat16, seed=3)
    a = tq.alloc_key_cache(4, 1024, kc.gpu)
    b = tq.alloc_key_cache(4, 1024, kc.gpu)
    tq.encode_kv(kc.gpu, x, *a)
    tq.encode_kv(kc.gpu, x, *b)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------ logits


@pytest.mark.parametrize("d,w,group,batch,n_kv,n_keys", [
    (128, 2, 16, 1, 1, 1000), (128, 3, 4, 2, 3, 777), (64, 2, 4, 2, 2, 513), (64, 1, 1, 1, 2, 65),
    (128, 1, 8, 1, 1, 1), (64, 3, 5, 1, 1, 200),
    # 256 (batch, kv-head) groups: one block per group walks all 4 splits
    (128, 3, 4, 4, 64, 1000),
    # 16 blocks per group, several head chunks (the last one short): the
    # chunks interleaved into the grid's x dimension
    (128, 2, 24, 1, 1, 4001), (64, 3, 20, 1, 2, 4096),
])
def test_logits_given_oracle_codes(d, w, group, batch, n_kv, n_keys):
    say(f"logits d={d} w={w} G={group} batch={batch} n_kv={n_kv} n_keys={n_keys}")
    kc = key_codec(600 + d + w, d, w)
    cap = (n_keys + 11 + 31) // 32 * 32
    k = _inputs(batch * n_kv, n_keys, d, torch.float32, seed=w, scale_channels=True)
    q = _inputs(batch, n_kv * group, d, torch.bfloat16, seed=w, stream=3)
    enc = kc.encode(to_f64(k))
    codes, scal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    pack_keys_into(enc, w, codes, scal)
    out = tq.logits(kc.gpu, q, codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys)
    torch.cuda.synchronize()
    qn = to_f64(q)
    ref = np.zeros((batch, n_kv * group, n_keys))
    for b in range(batch):
        for h in range(n_kv):
            s = b * n_kv + h
            ref[b, h * group:(h + 1) * group] = O.key_logits(
                qn[b, h * group:(h + 1) * group], kc.signs, kc.centroids, kc.sketch, enc["idx"][s],
                enc["sigma"][s], enc["nhat"][s], enc["ghat"][s])
    worst = assert_close(out.cpu().numpy(), ref, "logits")
    say("   worst err/tol", worst)


# ------------------------------------------------------------ decode attend


@pytest.mark.parametrize("d,kw,vw,group,batch,n_kv,T,lens", [
    (128, 2, 4, 4, 3, 2, 700, [700, 1, 333]),
    (128, 3, 4, 8, 2, 1, 1100, [0, 1100]),
    (64, 2, 4, 4, 2, 2, 300, [300, 64]),
    (64, 1, 2, 1, 1, 3, 96, [95]),
    (128, 2, 3, 16, 1, 1, 64, [37]),
    # 256 (batch, kv-head) groups: one block per group walks up to 3 splits
    # through the staging ring (ragged lengths, one empty row)
    (128, 2, 4, 4, 32, 8, 1100, [1100, 1, 700, 0, 257, 1024, 1099, 513] * 4),
    # 5-bit keys, 8 heads: stages of 512 tokens do not fit in LDS, 256-token splits
    (128, 4, 4, 8, 1, 2, 900, [900, 511]),
    # 8 heads, several 512-token splits per block and a ragged last one
    (128, 3, 4, 8, 1, 1, 2100, [2100]),
    (64, 3, 4, 8, 2, 1, 1600, [1600, 1025]),
    # 8 blocks per group and two or three head chunks (the last one short):
    # the chunks interleaved into the grid's x dimension
    (128, 2, 4, 16, 2, 1, 4096, [4096, 2900]),
    (64, 3, 4, 20, 1, 2, 4096, [4096]),
])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_decode_attend_given_oracle_codes(d, kw, vw, group, batch, n_kv, T, lens, out_dtype):
    say(f"decode d={d} kw={kw} vw={vw} G={group} batch={batch} n_kv={n_kv} T={T} lens={lens} out={out_dtype}")
    kc, vc = key_codec(700 + d, d, kw), value_codec(701 + d, d, vw)
    cap = ((T + 31) // 32) * 32 + 32
    k = _inputs(batch * n_kv, T, d, torch.float32, seed=kw, stream=1, scale_channels=True)
    v = _inputs(batch * n_kv, T, d, torch.float32, seed=vw, stream=2)
    q = _inputs(batch, n_kv * group, d, torch.bfloat16, seed=group, stream=3)
    ek, ev = kc.encode(to_f64(k)), vc.encode(to_f64(v))
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    pack_keys_into(ek, kw, kcodes, kscal)
    pack_values_into(ev, vw, vcodes, vscal)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out32 = tq.decode_attend(kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                             max_ctx=T, sm_scale=scale, out_dtype=torch.float32)
    outx = tq.decode_attend(kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                            max_ctx=T, sm_scale=scale, out_dtype=DTYPES[out_dtype])
    torch.cuda.synchronize()
    ref = O.decode_attend(to_f64(q), kc.signs, kc.centroids, kc.sketch, ek["idx"], ek["sigma"], ek["nhat"],
                          ek["ghat"], vc.signs, vc.centroids, ev["idx"], ev["nhat"], lens, scale, group)
    worst = assert_close(out32.cpu().numpy(), ref, "decode f32")
    say("   worst err/tol", worst)
    if out_dtype == "bf16":
        got = outx.to(torch.float64).cpu().numpy()
        expect = bf16_rne(out32.cpu().numpy())
        # identical kernels up to the final rounding: RNE of the fp32 result
        np.testing.assert_array_equal(got, expect)


# ------------------------------------------------------------------ graphs


@pytest.mark.parametrize("group,T,chunk", [
    (4, 600, 2),
    # 16 logit and 8 decode blocks per group, three head chunks: the chunks
    # interleaved into the grid's x dimension; a 96-pair single-pass prefill
    (24, 4000, 4),
])
def test_calls_replay_in_a_hip_graph(group, T, chunk):
    """encode + logits + decode + a prefill chunk captured in one HIP graph:
    every replay, with eager work and synchronisations in between,
    reproduces the eager results bit for bit (the benchmark times such
    replays)."""
    say(f"graph capture: encode + logits + decode + prefill, G={group} T={T} chunk={chunk}, 3 replays")
    d, kw, vw, batch, n_kv = 128, 3, 4, 2, 2
    kc, vc = key_codec(801, d, kw), value_codec(802, d, vw)
    cap = (T + 31) // 32 * 32 + 32
    k = _inputs(batch * n_kv, T, d, torch.bfloat16, seed=11, stream=1, scale_channels=True)
    v = _inputs(batch * n_kv, T, d, torch.bfloat16, seed=12, stream=2)
    q = _inputs(batch, n_kv * group, d, torch.bfloat16, seed=13, stream=3)
    ctx = torch.tensor([T, 333], dtype=torch.int32, device="cuda")
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    lg = torch.empty((batch, n_kv * group, T), dtype=torch.float32, device="cuda")
    out = torch.empty((batch, n_kv * group, d), dtype=torch.float32, device="cuda")
    lws = torch.empty(max(256, tq.logits_workspace(batch, n_kv, group, d)), dtype=torch.uint8, device="cuda")
    dws = torch.empty(tq.decode_attend_workspace(batch, n_kv, group, T, d), dtype=torch.uint8, device="cuda")
    qp = _inputs(batch * chunk, n_kv * group, d, torch.bfloat16, seed=14, stream=3).view(batch, chunk, n_kv * group, d)
    p0 = torch.tensor([T - chunk, T // 2], dtype=torch.int32, device="cuda")
    pout = torch.empty((batch, chunk, n_kv * group, d), dtype=torch.float32, device="cuda")
    pws = torch.empty(tq.prefill_attend_workspace(batch, chunk, n_kv, group, T, d), dtype=torch.uint8, device="cuda")

    def calls():
        tq.encode_kv(kc.gpu, k, kcodes, kscal)
        tq.encode_kv(vc.gpu, v, vcodes, vscal)
        tq.logits(kc.gpu, q, kcodes, kscal, n_kv_heads=n_kv, group=group, n_keys=T, out=lg, workspace=lws)
        tq.decode_attend(kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                         max_ctx=T, out=out, workspace=dws)
        tq.prefill_attend(kc.gpu, vc.gpu, qp, kcodes, kscal, vcodes, vscal, p0, n_kv_heads=n_kv, group=group,
                          max_ctx=T, out=pout, workspace=pws)

    calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (kcodes, kscal, vcodes, vscal, lg, out, pout)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        calls()
    scratch = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    for rep in range(3):
        for t in (kcodes, kscal, vcodes, vscal, lg, out, pout):
            t.zero_()
        tq.encode_kv(kc.gpu, k, *scratch)            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((kcodes, kscal, vcodes, vscal, lg, out, pout), ref):
            assert torch.equal(a, b), f"replay {rep} differs"


def test_explicit_side_stream_owns_the_temporaries():
    """A call given an explicit stream (not the current one) with no
    workspace, no output and a non-contiguous query: the binding's copy,
    output and workspace belong to that stream, so work allocated and
    written on the current stream right after the call cannot reuse them
    while the kernels still run. The result equals the same call on the
    current stream, bit for bit."""
    say("side stream: decode with workspace=None, then allocations on the current stream")
    d, kw, vw, batch, n_kv, group, T = 128, 3, 4, 4, 8, 4, 4096
    kc, vc = key_codec(811, d, kw), value_codec(812, d, vw)
    k = _inputs(batch * n_kv, T, d, torch.bfloat16, seed=21, stream=1)
    v = _inputs(batch * n_kv, T, d, torch.bfloat16, seed=22, stream=2)
    qt = _inputs(n_kv * group, batch, d, torch.bfloat16, seed=23, stream=3).transpose(0, 1)   # not contiguous
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, T, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, T, vc.gpu)
    tq.encode_kv(kc.gpu, k, kcodes, kscal)
    tq.encode_kv(vc.gpu, v, vcodes, vscal)
    ctx = torch.full((batch,), T, dtype=torch.int32, device="cuda")
    ref = tq.decode_attend(kc.gpu, vc.gpu, qt, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(tq.decode_attend(kc.gpu, vc.gpu, qt, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv,
                                     group=group, stream=side))
        junk = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        junk.fill_(0xA5)
        del junk
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
