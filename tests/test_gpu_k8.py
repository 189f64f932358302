"""GPU parity of the k8v4 cache shape (fp8 keys, TurboQuant values): the
fp8 key encode bit-exact against the oracle's e4m3 rounding, and decode
attention over fp8 keys against the oracle given the GPU's key bytes and
the oracle's value codes."""
import math

import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
from gpu_common import bf16_rne, pack_values_into, say, to_f64, value_codec
from tq_parity import assert_close

pytestmark = pytest.mark.gpu

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("scale,layout", [(1.0, "contiguous"), (0.6, "contiguous"), (0.25, "contiguous"),
                                          (0.6, "offset"), (4.0, "offset")])
def test_encode_fp8_keys_bit_exact(d, dt, scale, layout):
    """Scales 1, 0.25 and 4 take the reciprocal product (exact for powers of
    two), 0.6 the correctly rounded quotient; rows that start one element
    into a wider buffer take the element-wise loads."""
    say(f"fp8 key encode d={d} dtype={dt} scale={scale} layout={layout}")
    n_seq, n_tok, t0, cap = 3, 257, 5, 300
    g = torch.Generator(device="cpu")
    g.manual_seed(d + int(10 * scale))
    x = torch.randn((n_seq, n_tok, d), generator=g) * torch.exp(2.5 * torch.randn((d,), generator=g))
    x[0, 0, :4] = torch.tensor([600.0, -1e4, 1e-7, -0.0])       # saturation, subnormal range, -0
    x = x.to(DTYPES[dt])
    codes = tq.alloc_fp8_key_cache(n_seq, cap, d)
    if layout == "offset":
        wide = torch.zeros((n_seq, n_tok, d + 1), dtype=x.dtype, device="cuda")
        wide[:, :, 1:] = x.to("cuda")
        xd = wide[:, :, 1:]
    else:
        xd = x.to("cuda")
    tq.encode_fp8_keys(xd, codes, scale=scale, t0=t0)
    torch.cuda.synchronize()
    ref = O.e4m3_encode(x.to(torch.float32).numpy(), scale)
    got = codes.cpu().numpy()
    np.testing.assert_array_equal(got[:, t0:t0 + n_tok], ref)
    assert not got[:, :t0].any() and not got[:, t0 + n_tok:].any()


@pytest.mark.parametrize("d,vw,group,batch,n_kv,T,lens,qdt", [
    (128, 4, 4, 3, 2, 700, [700, 1, 333], "bf16"),
    (128, 4, 8, 2, 1, 1100, [0, 1100], "f32"),
    (64, 4, 4, 2, 2, 300, [300, 64], "bf16"),
    (64, 2, 1, 1, 3, 96, [95], "f16"),
    (128, 3, 16, 1, 1, 64, [37], "bf16"),
    (128, 4, 4, 32, 8, 600, [600, 1, 300, 0, 257, 512, 599, 513] * 4, "bf16"),
    # 8 blocks per group and two or three head chunks: the chunks
    # interleaved into the grid's x dimension
    (128, 4, 16, 1, 1, 4096, [4000], "bf16"),
    (64, 2, 24, 2, 1, 4096, [4096, 1500], "f32"),
])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_decode_attend_k8_given_codes(d, vw, group, batch, n_kv, T, lens, qdt, out_dtype):
    say(f"k8 decode d={d} vw={vw} G={group} batch={batch} n_kv={n_kv} T={T} lens={lens} q={qdt} out={out_dtype}")
    vc = value_codec(1700 + d + vw, d, vw)
    cap = ((T + 31) // 32) * 32
    g = torch.Generator(device="cpu")
    g.manual_seed(d * 7 + vw + group)
    k = torch.randn((batch * n_kv, T, d), generator=g) * torch.exp(torch.randn((d,), generator=g))
    v = torch.randn((batch * n_kv, T, d), generator=g, dtype=torch.float64)
    q = torch.randn((batch, n_kv * group, d), generator=g).to(DTYPES[qdt])
    k_scale = 0.25
    kcodes = tq.alloc_fp8_key_cache(batch * n_kv, cap, d)
    tq.encode_fp8_keys(k.to(torch.bfloat16).to("cuda"), kcodes, scale=k_scale)
    ev = vc.encode(v.numpy())
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    pack_values_into(ev, vw, vcodes, vscal)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out32 = tq.decode_attend_k8(vc.gpu, q.to("cuda"), kcodes, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                                k_scale=k_scale, max_ctx=T, sm_scale=scale, out_dtype=torch.float32)
    outx = tq.decode_attend_k8(vc.gpu, q.to("cuda"), kcodes, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                               k_scale=k_scale, max_ctx=T, sm_scale=scale, out_dtype=DTYPES[out_dtype])
    torch.cuda.synchronize()
    ref = O.decode_attend_k8(to_f64(q), kcodes.cpu().numpy(), k_scale, vc.signs, vc.centroids, ev["idx"],
                             ev["nhat"], lens, scale, group)
    worst = assert_close(out32.cpu().numpy(), ref, "k8 decode f32")
    say("   worst err/tol", worst)
    if out_dtype == "bf16":
        np.testing.assert_array_equal(outx.to(torch.float64).cpu().numpy(), bf16_rne(out32.cpu().numpy()))
