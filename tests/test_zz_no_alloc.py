"""tq_decode_attend_noalloc: decode attention with the split partials in the
library's fixed device scratch instead of a caller workspace.

GPU: two calls in a row through the C ABI, the second on a smaller input,
each equal bit for bit to tq_decode_attend on the same inputs (the same
kernels; only where the partials live differs). CPU: the size limit and the
argument checks are host-side and reject before anything touches a device."""

import pytest
import torch

import kv_cache_vector_rht_amd as tq
from gpu_common import key_codec, say, value_codec


def _case(d, kw, vw, batch, n_kv, group, T, lens, seed):
    kc, vc = key_codec(900 + seed, d, kw), value_codec(901 + seed, d, vw)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    k = (torch.randn((batch * n_kv, T, d), generator=g) * torch.exp(torch.randn((d,), generator=g))).to(torch.bfloat16)
    v = torch.randn((batch * n_kv, T, d), generator=g).to(torch.bfloat16)
    q = torch.randn((batch, n_kv * group, d), generator=g).to(torch.bfloat16).cuda()
    cap = (T + 31) // 32 * 32
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc.gpu)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc.gpu)
    tq.encode_kv(kc.gpu, k.cuda(), kcodes, kscal)
    tq.encode_kv(vc.gpu, v.cuda(), vcodes, vscal)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return kc.gpu, vc.gpu, q, kcodes, kscal, vcodes, vscal, ctx


@pytest.mark.gpu
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_equals_workspace_call_twice_second_smaller(out_dtype):
    cases = [
        # 16 x 8 groups of 4 heads at 4096 tokens (two blocks per group)
        (128, 2, 4, 16, 8, 4, 4096, [4096, 1, 4000, 0, 2049, 4095, 512, 3333] * 2, 31),
        # then a smaller one: 2 x 2 groups of 8 heads, ragged
        (64, 3, 4, 2, 2, 8, 700, [700, 129], 32),
    ]
    for d, kw, vw, batch, n_kv, group, T, lens, seed in cases:
        say(f"no-alloc decode d={d} kw={kw} vw={vw} batch={batch} n_kv={n_kv} G={group} T={T} out={out_dtype}")
        kc, vc, q, kcodes, kscal, vcodes, vscal, ctx = _case(d, kw, vw, batch, n_kv, group, T, lens, seed)
        need = tq.decode_attend_workspace(batch, n_kv, group, T, d)
        assert need <= tq.decode_attend_noalloc_max_workspace()
        ref = tq.decode_attend(kc, vc, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                               max_ctx=T, out_dtype=out_dtype)
        out = torch.full_like(ref, float("nan"))
        tq.decode_attend_noalloc(kc, vc, q, kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=n_kv, group=group,
                                 out=out, max_ctx=T)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"max diff {(out.float() - ref.float()).abs().max().item()}"


def test_noalloc_rejects_calls_beyond_the_fixed_scratch_before_any_launch():
    """Host-side: a call whose partials exceed the fixed scratch is refused
    with TQ_EUNSUPPORTED, and malformed arguments with TQ_EINVAL, without a
    device (null device pointers are never dereferenced on the host)."""
    import ctypes
    cap = tq.decode_attend_noalloc_max_workspace()
    assert cap == 16 << 20
    d, n_kv, group = 128, 8, 32
    # 16 MiB / (d + 2) / 4 bytes / group: the most (batch, kv-head) groups of one block each
    batch = 4096
    assert tq.decode_attend_workspace(batch, n_kv, group, 512, d) > cap
    kc = tq._Codec()
    kc.d, kc.lm_bits, kc.is_key = d, 3, 1
    kc.signs = kc.centroids = kc.thresholds = kc.sketch = 16
    vc = tq._Codec()
    vc.d, vc.lm_bits, vc.is_key = d, 4, 0
    vc.signs = vc.centroids = vc.thresholds = 16
    P = ctypes.c_void_p
    st = tq.lib.tq_decode_attend_noalloc(ctypes.byref(kc), ctypes.byref(vc), P(16), tq.TQ_BF16, batch, n_kv, group,
                                         P(16), P(16), P(16), P(16), 512, P(16), 512, 0.1, P(16), tq.TQ_F32, None)
    assert st == tq.TQ_EUNSUPPORTED
    assert b"scratch" in tq.lib.tq_last_error()
    st = tq.lib.tq_decode_attend_noalloc(ctypes.byref(kc), ctypes.byref(vc), None, tq.TQ_BF16, 2, n_kv, 4,
                                         P(16), P(16), P(16), P(16), 512, P(16), 512, 0.1, P(16), tq.TQ_F32, None)
    assert st == tq.TQ_EINVAL
    st = tq.lib.tq_decode_attend_noalloc(ctypes.byref(kc), ctypes.byref(vc), P(16), tq.TQ_BF16, 2, n_kv, 4,
                                         P(16), P(16), P(16), P(16), 500, P(16), 500, 0.1, P(16), tq.TQ_F32, None)
    assert st == tq.TQ_EINVAL                      # cap not a multiple of 32
