"""GPU parity of the LDS-table formulation of the logit scan (tq_logits_table,
a measurement path beside the matrix-core scan): given the oracle's codes,
logits against the oracle's estimator within the logit tolerance, and
against tq_logits on the same codes."""
import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import key_codec, pack_keys_into, say, to_f64
from tq_parity import assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,w,group,batch,n_kv,n_keys", [
    (128, 3, 4, 1, 8, 1999),        # the decode-layer shape, ragged tail
    (128, 2, 1, 1, 1, 4096),        # single head
    (128, 4, 8, 2, 1, 700),         # two chunks of 4 heads
    (64, 2, 6, 2, 2, 333),          # a ragged head chunk
    (64, 1, 4, 1, 1, 64),
    (128, 1, 3, 1, 2, 257),
])
def test_table_scan_given_oracle_codes(d, w, group, batch, n_kv, n_keys):
    say(f"table scan d={d} w={w} G={group} batch={batch} n_kv={n_kv} n_keys={n_keys}")
    kc = key_codec(1800 + d + w, d, w)
    cap = (n_keys + 31) // 32 * 32
    g = torch.Generator(device="cpu")
    g.manual_seed(d * 7 + w + group)
    k = torch.randn((batch * n_kv, n_keys, d), generator=g, dtype=torch.float64)
    k *= torch.exp(torch.randn((d,), generator=g, dtype=torch.float64))
    q = torch.randn((batch, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    enc = kc.encode(k.numpy())
    codes, scal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    pack_keys_into(enc, w, codes, scal)
    qd = q.to("cuda")
    tab = tq.logits_table(kc.gpu, qd, codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys)
    mf = tq.logits(kc.gpu, qd, codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys)
    torch.cuda.synchronize()
    qn = to_f64(q)
    ref = np.zeros((batch, n_kv * group, n_keys))
    for b in range(batch):
        for h in range(n_kv):
            s = b * n_kv + h
            ref[b, h * group:(h + 1) * group] = O.key_logits(qn[b, h * group:(h + 1) * group], kc.signs, kc.centroids,
                                                             kc.sketch, enc["idx"][s], enc["sigma"][s], enc["nhat"][s],
                                                             enc["ghat"][s])
    say("   worst err/tol vs oracle", assert_close(tab.cpu().numpy(), ref, "table scan"))
    assert_close(tab.cpu().numpy(), mf.cpu().numpy(), "table scan vs matrix-core scan", atol=2e-4, rtol=2e-3)
