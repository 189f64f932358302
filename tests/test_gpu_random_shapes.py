"""Seeded random shapes through the scan calls: GPU parity against the oracle.

Each case draws, from a fixed seed, the head dimension, the key and value
widths, the group size (1 to 32 query heads per KV head, so one to four
chunks of 8 heads), the batch, the KV heads, the context length and ragged
per-row lengths, the query dtype, and a prefill chunk with its first
positions, and in a third of the cases MSE-only keys (index planes and
norm, no QJL part) instead of full TurboQuant keys. Given the oracle's
codes, tq_logits, tq_decode_attend and tq_prefill_attend are checked
against the oracle within the logit tolerance. The draws give block counts per group that are and are not
multiples of 8, so both launch layouts of several head chunks (chunks on
the grid's z dimension, or interleaved into x) are exercised, as are the
single-pass prefill (more than 8 position-head pairs) and the decode-kernel
prefill."""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import (key_codec, mse_key_codec, pack_keys_into, pack_mse_keys_into, pack_values_into, say, to_f64,
                        value_codec)
from tq_parity import assert_close

pytestmark = pytest.mark.gpu

QDT = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}


def _draw(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        kw = int(rng.integers(1, 5))
        vw = int(rng.integers(1, 5))
        group = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 20, 24, 32]))
        batch = int(rng.integers(1, 3))
        n_kv = int(rng.integers(1, 3))
        # long contexts in half the cases, just below 4096 or 2048 tokens: 16
        # or 8 logit splits (and 8 or 4 decode splits), so 8 or 16 blocks per
        # group; short ragged ones in the others
        if i % 2 == 0:
            T = (4096 if i % 4 == 0 else 2048) - int(rng.integers(0, 256))
        else:
            T = int(rng.integers(1, 1200))
        lens = [T] + [int(x) for x in rng.integers(0, T + 1, size=batch - 1)]
        chunk = int(rng.integers(1, min(8, T) + 1))
        pos0 = [int(x) for x in rng.integers(0, T - chunk + 1, size=batch)]
        qdt = str(rng.choice(list(QDT)))
        mse = i % 3 == 2
        cases.append((i, d, kw, vw, group, batch, n_kv, T, lens, chunk, pos0, qdt, mse))
    return cases


@pytest.mark.parametrize("case", _draw(16), ids=lambda c: f"case{c[0]}")
def test_random_shape_scans(case):
    i, d, kw, vw, group, batch, n_kv, T, lens, chunk, pos0, qdt, mse = case
    say(f"random case {i}: d={d} kw={kw} vw={vw} G={group} batch={batch} n_kv={n_kv} T={T} lens={lens} "
        f"chunk={chunk} pos0={pos0} q={qdt} mse_only_keys={mse}")
    kc = mse_key_codec(2100 + i, d, kw) if mse else key_codec(2100 + i, d, kw)
    vc = value_codec(2200 + i, d, vw)
    cap = ((T + 31) // 32) * 32
    g = torch.Generator(device="cpu")
    g.manual_seed(3000 + i)
    k = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float64)
    k *= torch.exp(torch.randn((d,), generator=g, dtype=torch.float64))
    v = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float64)
    ek, ev = kc.encode(k.numpy()), vc.encode(v.numpy())
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    if mse:
        pack_mse_keys_into(ek, kw, kcodes, kscal)
    else:
        pack_keys_into(ek, kw, kcodes, kscal)
    pack_values_into(ev, vw, vcodes, vscal)
    scale = 1.0 / math.sqrt(d)
    # the oracle's key side: no sketch, sign bits or residual norms for MSE-only keys
    sk, ksig, kgh = (None, None, None) if mse else (kc.sketch, ek["sigma"], ek["ghat"])

    # logits over all T keys
    q = torch.randn((batch, n_kv * group, d), generator=g, dtype=torch.float32).to(QDT[qdt])
    qd = q.to("cuda")
    lg = tq.logits(kc.gpu, qd, kcodes, kscal, n_kv_heads=n_kv, group=group, n_keys=T)
    # decode attention over the ragged lengths
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    att = tq.decode_attend(kc.gpu, vc.gpu, qd, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                           max_ctx=T, sm_scale=scale, out_dtype=torch.float32)
    # a prefill chunk at the drawn positions
    qp = torch.randn((batch, chunk, n_kv * group, d), generator=g, dtype=torch.float32).to(QDT[qdt])
    p0 = torch.tensor(pos0, dtype=torch.int32, device="cuda")
    pre = tq.prefill_attend(kc.gpu, vc.gpu, qp.to("cuda"), kcodes, kscal, vcodes, vscal, p0, n_kv_heads=n_kv,
                            group=group, max_ctx=T, sm_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()

    qn = to_f64(q)
    ref = np.zeros((batch, n_kv * group, T))
    for b in range(batch):
        for h in range(n_kv):
            s = b * n_kv + h
            qh = qn[b, h * group:(h + 1) * group]
            if mse:
                ref[b, h * group:(h + 1) * group] = O.key_logits_mse(qh, kc.signs, kc.centroids, ek["idx"][s],
                                                                     ek["nhat"][s])
            else:
                ref[b, h * group:(h + 1) * group] = O.key_logits(qh, kc.signs, kc.centroids, kc.sketch, ek["idx"][s],
                                                                 ek["sigma"][s], ek["nhat"][s], ek["ghat"][s])
    say("   logits worst err/tol", assert_close(lg.cpu().numpy(), ref, "logits"))
    ref = O.decode_attend(qn, kc.signs, kc.centroids, sk, ek["idx"], ksig, ek["nhat"], kgh, vc.signs, vc.centroids,
                          ev["idx"], ev["nhat"], lens, scale, group)
    say("   decode worst err/tol", assert_close(att.cpu().numpy(), ref, "decode"))
    ref = O.prefill_attend(to_f64(qp), kc.signs, kc.centroids, sk, ek["idx"], ksig, ek["nhat"], kgh, vc.signs,
                           vc.centroids, ev["idx"], ev["nhat"], pos0, scale, group)
    say("   prefill worst err/tol", assert_close(pre.cpu().numpy(), ref, "prefill"))
