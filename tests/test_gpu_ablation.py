"""GPU parity of the MSE-only ablation (tq_logits_mse: the estimator's first
term alone, from the same key records) and the bias it shows next to the
full estimator on correlated pairs, on the GPU and in the oracle alike."""
import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import key_codec, pack_keys_into, say, to_f64
from tq_parity import assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,w,group,batch,n_kv,n_keys", [
    (128, 3, 4, 1, 2, 777),
    (64, 2, 8, 2, 1, 300),
])
def test_logits_mse_given_oracle_codes(d, w, group, batch, n_kv, n_keys):
    say(f"logits_mse d={d} w={w} G={group} batch={batch} n_kv={n_kv} n_keys={n_keys}")
    kc = key_codec(700 + d + w, d, w)
    cap = (n_keys + 31) // 32 * 32
    g = torch.Generator(device="cpu")
    g.manual_seed(d + w)
    k = torch.randn((batch * n_kv, n_keys, d), generator=g, dtype=torch.float64)
    q = torch.randn((batch, n_kv * group, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    enc = kc.encode(k.numpy())
    codes, scal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    pack_keys_into(enc, w, codes, scal)
    out = tq.logits(kc.gpu, q.to("cuda"), codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys,
                    mse_only=True)
    torch.cuda.synchronize()
    qn = to_f64(q)
    ref = np.zeros((batch, n_kv * group, n_keys))
    for b in range(batch):
        for h in range(n_kv):
            s = b * n_kv + h
            ref[b, h * group:(h + 1) * group] = O.key_logits_mse(qn[b, h * group:(h + 1) * group], kc.signs,
                                                                 kc.centroids, enc["idx"][s], enc["nhat"][s])
    assert_close(out.cpu().numpy(), ref, "logits_mse")


def test_mse_bias_and_qjl_correction_on_pairs():
    """16384 correlated pairs (k ~ N(0, I), q = k + N(0, I)), d 128, 2-bit
    Lloyd-Max keys: each pair is one sequence of one key with one query head.
    The MSE-only estimate shrinks inner products by about the per-coordinate
    distortion D(2) = 0.116; the full estimator removes the shrinkage. The
    GPU's mean relative errors equal the oracle's on the same codes."""
    d, w, n = 128, 2, 16384
    say(f"bias on {n} pairs, d={d}, w={w}")
    kc = key_codec(811, d, w)
    rng = np.random.default_rng(17)
    k = rng.standard_normal((n, 1, d))
    q = (k[:, 0] + rng.standard_normal((n, d))).astype(np.float32)
    enc = kc.encode(k)
    codes, scal = tq.alloc_key_cache(n, 32, kc.gpu)
    pack_keys_into(enc, w, codes, scal)
    qd = torch.from_numpy(q).to("cuda").view(n, 1, d)
    full = tq.logits(kc.gpu, qd, codes, scal, n_kv_heads=1, group=1, n_keys=1).view(n).cpu().numpy()
    mse = tq.logits(kc.gpu, qd, codes, scal, n_kv_heads=1, group=1, n_keys=1, mse_only=True).view(n).cpu().numpy()
    true = np.sum(q.astype(np.float64) * k[:, 0], axis=1)
    rel_full = full.astype(np.float64).mean() / true.mean() - 1
    rel_mse = mse.astype(np.float64).mean() / true.mean() - 1
    # the oracle on the same codes
    o_full = O.pair_logits(q, kc.signs, kc.centroids, kc.sketch, enc["idx"][:, 0], enc["sigma"][:, 0],
                           enc["nhat"][:, 0], enc["ghat"][:, 0])
    o_mse = O.pair_logits(q, kc.signs, kc.centroids, kc.sketch, enc["idx"][:, 0], enc["sigma"][:, 0],
                          enc["nhat"][:, 0], np.zeros(n, dtype=np.float16))
    say(f"   relative bias: full {rel_full:+.4f} (oracle {o_full.mean() / true.mean() - 1:+.4f}), "
        f"MSE-only {rel_mse:+.4f} (oracle {o_mse.mean() / true.mean() - 1:+.4f})")
    assert abs(rel_full - (o_full.mean() / true.mean() - 1)) < 1e-4
    assert abs(rel_mse - (o_mse.mean() / true.mean() - 1)) < 1e-4
    assert abs(rel_mse - (-0.116)) < 0.01
    assert abs(rel_full) < 0.02
