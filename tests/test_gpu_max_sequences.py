"""The largest call the scan launches take: 65,535 (batch, kv-head) sequences,
the launch grid's y dimension. Short contexts (40 tokens in slots of 64) are
encoded on the GPU; the logits and the decode attention of every sequence
are computed in one call each, and sampled sequences (the first, the last,
an empty and a one-token row, and random others) are checked against the
oracle over the codes the GPU wrote."""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import key_codec, say, to_f64, value_codec
from tq_parity import assert_close

pytestmark = pytest.mark.gpu


def test_max_sequences_logits_and_decode():
    d, kw, vw, group, T, cap = 64, 2, 2, 2, 40, 64
    n = 65535
    say(f"max sequences: {n} sequences x {T} tokens, d={d}, G={group}")
    kc, vc = key_codec(2300, d, kw), value_codec(2301, d, vw)
    g = torch.Generator(device="cuda")
    g.manual_seed(2302)
    k = torch.randn((n, T, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((n, T, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((n, group, d), generator=g, device="cuda").to(torch.bfloat16)
    lens = torch.randint(0, T + 1, (n,), generator=g, device="cuda", dtype=torch.int32)
    lens[0], lens[5], lens[6], lens[n - 1] = T, 0, 1, T
    kcodes, kscal = tq.alloc_key_cache(n, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(n, cap, vc.gpu)
    tq.encode_kv(kc.gpu, k, kcodes, kscal)
    tq.encode_kv(vc.gpu, v, vcodes, vscal)
    del k, v
    scale = 1.0 / math.sqrt(d)
    lg = tq.logits(kc.gpu, q, kcodes, kscal, n_kv_heads=1, group=group, n_keys=T)
    att = tq.decode_attend(kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, lens, n_kv_heads=1, group=group,
                           max_ctx=T, sm_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2303)
    samples = sorted({0, 1, 5, 6, n // 2, n - 2, n - 1, *rng.integers(0, n, size=6).tolist()})
    lens_h = lens.cpu().numpy()
    for sq in samples:
        qn = to_f64(q[sq:sq + 1])
        kidx, ksig = O.unpack_key_codes(kcodes[sq].cpu().numpy(), d, kw)
        ks = kscal[sq].cpu().numpy().view(np.float16)
        vidx = O.unpack_value_codes(vcodes[sq:sq + 1].cpu().numpy().view(np.uint32), cap)
        vn = vscal[sq:sq + 1].cpu().numpy().view(np.float16)
        ref_lg = O.key_logits(qn[0], kc.signs, kc.centroids, kc.sketch, kidx[:T], ksig[:T], ks[:T, 0], ks[:T, 1])
        worst_l = assert_close(lg[sq].cpu().numpy(), ref_lg, f"logits seq {sq}")
        ref = O.decode_attend(qn, kc.signs, kc.centroids, kc.sketch, kidx[None], ksig[None], ks[None, :, 0],
                              ks[None, :, 1], vc.signs, vc.centroids, vidx, vn, [int(lens_h[sq])], scale, group)
        worst_d = assert_close(att[sq:sq + 1].cpu().numpy(), ref, f"decode seq {sq}")
        say(f"   seq {sq} (len {lens_h[sq]}): worst err/tol logits {worst_l:.3f} decode {worst_d:.3f}")
