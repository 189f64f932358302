"""tq_prepare_queries + tq_logits_prepared against tq_logits: the same
kernels' arithmetic split over two launches, so the logits must agree bit
for bit (several head chunks, both head sizes, every key width, fp32 and
bf16 queries); and tq_logits itself is checked against the oracle
elsewhere."""
import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
from gpu_common import key_codec, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,w,group,batch,n_kv,n_keys,qdt", [
    (128, 3, 4, 1, 8, 32768, torch.bfloat16),      # the decode-layer workload's shape
    (128, 1, 20, 2, 2, 1000, torch.float32),       # three head chunks, ragged keys
    (64, 2, 8, 3, 1, 777, torch.bfloat16),
    (64, 4, 5, 1, 3, 4096, torch.float16),
    (128, 4, 1, 4, 2, 300, torch.float32),
    # 16 blocks per group: the three head chunks interleaved into the grid's x
    (128, 2, 24, 1, 2, 4001, torch.bfloat16),
])
def test_prepared_logits_equal_one_call_logits(d, w, group, batch, n_kv, n_keys, qdt):
    say(f"prepared logits d={d} w={w} G={group} batch={batch} n_kv={n_kv} keys={n_keys} q={qdt}")
    kc = key_codec(1900 + d + w, d, w)
    cap = (n_keys + 31) // 32 * 32
    g = torch.Generator(device="cuda")
    g.manual_seed(d + w + group)
    x = torch.randn((batch * n_kv, n_keys, d), generator=g, device="cuda").to(torch.bfloat16)
    codes, scal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    tq.encode_kv(kc.gpu, x, codes, scal)
    q = torch.randn((batch, n_kv * group, d), generator=g, device="cuda").to(qdt)
    one = tq.logits(kc.gpu, q, codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys)
    prep = tq.prepare_queries(kc.gpu, q, n_kv_heads=n_kv, group=group)
    two = tq.logits_prepared(kc.gpu, prep, batch, codes, scal, n_kv_heads=n_kv, group=group, n_keys=n_keys)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(two.cpu().numpy(), one.cpu().numpy())
