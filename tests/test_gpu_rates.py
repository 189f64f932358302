"""GPU parity of fractional rates: a small multi-layer cache whose layers use
the widths of tq_rate_plan (3.5-bit keys, 2.5-bit values: two neighbouring
Lloyd-Max widths spread over the layers). Every layer's codes against the
oracle's encoding under the parity rule, and its decode attention against
the oracle given the GPU's codes; the cache's bits per channel as planned."""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import key_codec, say, to_f64, value_codec
from tq_parity import assert_close, check_key_codes, check_value_codes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,key_bits,val_bits,layers", [(128, 3.5, 2.5, 4), (64, 2.5, 3.5, 3)])
def test_fractional_rate_cache(d, key_bits, val_bits, layers):
    batch, n_kv, group, T = 2, 2, 4, 300
    kplan = tq.rate_plan(key_bits, layers, True)
    vplan = tq.rate_plan(val_bits, layers, False)
    assert kplan == O.rate_plan(key_bits, layers, True) and vplan == O.rate_plan(val_bits, layers, False)
    say(f"fractional rates d={d}: keys {key_bits} bits -> {kplan}, values {val_bits} bits -> {vplan}")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(10 * key_bits + val_bits) + d)
    cap = 320
    scale = 1.0 / math.sqrt(d)
    lens = [300, 129]
    key_bits_total = val_bits_total = 0
    for layer in range(layers):
        kw, vw = kplan[layer], vplan[layer]
        kc, vc = key_codec(1500 + layer, d, kw), value_codec(1600 + layer, d, vw)
        k = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
        v = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
        q = torch.randn((batch, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
        kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
        vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
        tq.encode_kv(kc.gpu, k.to("cuda"), kcodes, kscal)
        tq.encode_kv(vc.gpu, v.to("cuda"), vcodes, vscal)
        out = tq.decode_attend(kc.gpu, vc.gpu, q.to("cuda"), kcodes, kscal, vcodes, vscal,
                               torch.tensor(lens, dtype=torch.int32, device="cuda"), n_kv_heads=n_kv, group=group,
                               max_ctx=T, sm_scale=scale)
        torch.cuda.synchronize()
        ek, ev = kc.encode(to_f64(k)), vc.encode(to_f64(v))
        check_key_codes(kcodes[:, :T].cpu().numpy(), kscal[:, :T].cpu().numpy(), ek, kw, kc.centroids,
                        kc.thresholds, kc.sketch, d, f"layer {layer} keys")
        check_value_codes(vcodes.cpu().numpy(), vscal.cpu().numpy(), ev, vw, vc.thresholds, T,
                          f"layer {layer} values")
        kidx, ksig = O.unpack_key_codes(kcodes.cpu().numpy(), d, kw)
        ks = kscal.cpu().numpy().view(np.float16)
        vidx = O.unpack_value_codes(vcodes.cpu().numpy().view(np.uint32), cap)
        ref = O.decode_attend(to_f64(q), kc.signs, kc.centroids, kc.sketch, kidx, ksig, ks[..., 0], ks[..., 1],
                              vc.signs, vc.centroids, vidx, vscal.cpu().numpy().view(np.float16), lens, scale,
                              group)
        assert_close(out.cpu().numpy(), ref, f"layer {layer} decode")
        key_bits_total += kcodes.shape[-1] * 8
        val_bits_total += vcodes.shape[2] * d
    # code bits per channel (scalars aside): the planned average
    assert key_bits_total / (layers * d) == pytest.approx(sum(w + 1 for w in kplan) / layers)
    assert val_bits_total / (layers * d) == pytest.approx(sum(vplan) / layers)
    assert abs(sum(w + 1 for w in kplan) / layers - key_bits) <= 0.5 / layers + 1e-12
