"""Host-side tests of libtq (no GPU): exported symbols, the host codebook
solver against the oracle, and argument validation, which must reject bad
calls before anything is launched."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import kv_cache_vector_rht_amd as tq
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    import glob
    src = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", tq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines()}
    declared = _declared()
    assert declared, "no declarations found in include/*.h"
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    assert set(declared) == set(tq.EXPORTED)
    for s in declared:
        getattr(tq.lib, s)          # resolvable through ctypes


@pytest.mark.parametrize("d", [3, 4, 16, 64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_host_codebook_matches_oracle(d, bits):
    c, t = tq.make_codebook(d, bits)
    co, to = O.make_codebook(d, bits)
    # both solve the same fixed point to ~1e-15; fp32 rounding must agree
    cu = c.numpy().view(np.int32).astype(np.int64)
    tu = t.numpy().view(np.int32).astype(np.int64)
    assert np.max(np.abs(cu - co.view(np.int32))) <= 1
    assert np.max(np.abs(tu - to.view(np.int32))) <= 1
    assert np.all(c.numpy() == -c.numpy()[::-1])
    assert t.numpy()[(1 << bits) // 2 - 1] == 0.0


@pytest.mark.parametrize("d,bits", [(2, 2), (0, 1), (64, 0), (64, 9)])
def test_codebook_rejects_bad_arguments(d, bits):
    with pytest.raises(tq.TQError) as e:
        tq.make_codebook(d, bits)
    assert e.value.status == tq.TQ_EINVAL


def test_record_sizes():
    assert tq.key_record_bytes(128, 3) == 64
    assert tq.key_record_bytes(128, 2) == 48
    assert tq.key_record_bytes(64, 2) == 24
    assert tq.value_block_bytes(128, 4) == 2048
    assert tq.key_record_bytes(96, 2) == 0
    assert tq.mse_key_record_bytes(128, 3) == 48          # + a 2-byte norm: 50 B against 68 B with QJL
    assert tq.mse_key_record_bytes(64, 4) == 32
    assert tq.mse_key_record_bytes(96, 2) == 0


# ---------------------------------------------------------------- validation

FAKE = 1 << 20      # an aligned, never-dereferenced address


def _codec(d=128, w=2, key=1, sketch=True):
    c = tq._Codec()
    c.d, c.lm_bits, c.is_key, c.reserved = d, w, key, 0
    c.signs = c.centroids = c.thresholds = FAKE
    c.sketch = FAKE if sketch else None
    return c


def _p(v=FAKE):
    return ctypes.c_void_p(v)


def _encode(c, xt=tq.TQ_BF16, n_seq=1, n_tok=64, seq_stride=64 * 128, tok_stride=128, codes=FAKE,
            scal=FAKE, cap=64, t0=0, x=FAKE):
    return tq.lib.tq_encode_kv(ctypes.byref(c) if c is not None else None, _p(x), xt, n_seq, n_tok,
                               seq_stride, tok_stride, _p(codes), _p(scal), cap, t0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(c=None), tq.TQ_EINVAL),
    (dict(c="d96"), tq.TQ_EINVAL),
    (dict(c="d256"), tq.TQ_EUNSUPPORTED),
    (dict(c="w0"), tq.TQ_EINVAL),
    (dict(c="w5"), tq.TQ_EUNSUPPORTED),
    (dict(c="nosketch"), tq.TQ_EINVAL),
    (dict(c="kind3"), tq.TQ_EINVAL),
    (dict(c="mse", n_tok=-1), tq.TQ_EINVAL),                # an MSE-only key codec needs no sketch
    (dict(xt=7), tq.TQ_EINVAL),
    (dict(n_tok=-1), tq.TQ_EINVAL),
    (dict(t0=32, n_tok=64, cap=64), tq.TQ_EINVAL),
    (dict(c="value", cap=48, n_tok=16), tq.TQ_EINVAL),
    (dict(x=0), tq.TQ_EINVAL),
    (dict(codes=0), tq.TQ_EINVAL),
    (dict(tok_stride=64), tq.TQ_EINVAL),
    (dict(x=FAKE + 2), tq.TQ_EUNSUPPORTED),
    (dict(tok_stride=129, seq_stride=129 * 64), tq.TQ_EUNSUPPORTED),
    (dict(codes=FAKE + 4), tq.TQ_EINVAL),
])
def test_encode_validation(kwargs, status):
    c = kwargs.pop("c", "key")
    codec = {"key": _codec(), "d96": _codec(d=96), "d256": _codec(d=256), "w0": _codec(w=0),
             "w5": _codec(w=5), "nosketch": _codec(sketch=False), "value": _codec(key=0),
             "kind3": _codec(key=3), "mse": _codec(key=2, sketch=False), None: None}[c]
    assert _encode(codec, **kwargs) == status
    assert tq.lib.tq_last_error().decode()


def test_encode_empty_is_noop():
    assert _encode(_codec(), n_seq=0) == tq.TQ_OK
    assert _encode(_codec(), n_tok=0) == tq.TQ_OK


def _logits(c, batch=1, n_kv=8, group=4, cap=1024, n_keys=1024, ws=None, ws_ptr=FAKE, q=FAKE, qt=tq.TQ_BF16):
    if ws is None:
        ws = tq.logits_workspace(batch, n_kv, group, 128)
    return tq.lib.tq_logits(ctypes.byref(c), _p(q), qt, batch, n_kv, group, _p(), _p(), cap, n_keys, _p(),
                            _p(ws_ptr), ws, None)


def test_logits_validation():
    assert _logits(_codec(key=0)) == tq.TQ_EINVAL
    assert _logits(_codec(), n_keys=2048) == tq.TQ_EINVAL
    assert _logits(_codec(), group=33) == tq.TQ_EUNSUPPORTED
    assert _logits(_codec(), cap=1000, n_keys=1000) == tq.TQ_EINVAL        # cap not a multiple of 32
    assert _logits(_codec(), cap=1 << 27, n_keys=64) == tq.TQ_EUNSUPPORTED  # a sequence above 4 GiB
    assert _logits(_codec(), q=0) == tq.TQ_EINVAL
    assert _logits(_codec(), qt=9) == tq.TQ_EINVAL
    assert _logits(_codec(), batch=-1) == tq.TQ_EINVAL
    assert _logits(_codec(), n_keys=0) == tq.TQ_OK
    # MSE-only key records: no sketch needed; the 4 GiB bound uses their w d/8 bytes
    assert _logits(_codec(key=2, sketch=False), n_keys=0) == tq.TQ_OK
    assert _logits(_codec(key=2, sketch=False, w=4), cap=1 << 27, n_keys=64) == tq.TQ_EUNSUPPORTED
    assert tq.logits_workspace(1, 8, 4, 128) == 0                           # queries are prepared in LDS
    # the MSE-only ablation validates exactly like tq_logits
    cs = _codec()
    assert tq.lib.tq_logits_mse(ctypes.byref(cs), _p(), tq.TQ_BF16, 1, 8, 33, _p(), _p(), 256, 64, _p(), None, 0,
                                None) == tq.TQ_EUNSUPPORTED
    assert tq.lib.tq_logits_mse(ctypes.byref(cs), _p(), tq.TQ_BF16, 1, 8, 4, _p(), _p(), 256, 512, _p(), None, 0,
                                None) == tq.TQ_EINVAL
    assert tq.lib.tq_logits_mse(ctypes.byref(cs), _p(), tq.TQ_BF16, 1, 8, 4, _p(), _p(), 256, 0, _p(), None, 0,
                                None) == tq.TQ_OK


def _decode(kc, vc, batch=2, n_kv=2, group=4, cap=256, max_ctx=256, scale=0.1, out_t=tq.TQ_F32, ws=None,
            ctx=FAKE):
    if ws is None:
        ws = tq.decode_attend_workspace(batch, n_kv, group, max_ctx, 128)
    return tq.lib.tq_decode_attend(ctypes.byref(kc), ctypes.byref(vc), _p(), tq.TQ_BF16, batch, n_kv, group,
                                   _p(), _p(), _p(), _p(), cap, _p(ctx), max_ctx, scale, _p(), out_t, _p(), ws,
                                   None)


def test_decode_validation():
    k, v = _codec(), _codec(w=4, key=0, sketch=False)
    assert _decode(v, v) == tq.TQ_EINVAL                       # key codec expected
    assert _decode(k, k) == tq.TQ_EINVAL                       # value codec expected
    assert _decode(k, _codec(d=64, w=4, key=0)) == tq.TQ_EINVAL
    assert _decode(k, v, out_t=tq.TQ_F16) == tq.TQ_EUNSUPPORTED
    assert _decode(k, v, max_ctx=512) == tq.TQ_EINVAL
    assert _decode(k, v, cap=250, max_ctx=200) == tq.TQ_EINVAL
    assert _decode(k, v, group=33) == tq.TQ_EUNSUPPORTED
    assert _decode(k, v, scale=float("nan")) == tq.TQ_EINVAL
    assert _decode(k, v, ws=64) == tq.TQ_EINVAL
    assert _decode(k, v, cap=1 << 27, max_ctx=256) == tq.TQ_EUNSUPPORTED   # a sequence above 4 GiB
    assert _decode(k, v, ctx=0) == tq.TQ_EINVAL
    assert _decode(k, v, batch=0) == tq.TQ_OK
    assert tq.decode_attend_workspace(4, 8, 8, 131072, 128) > 0


def _append(kc, vc, batch=2, n_kv=2, group=4, cap=256, max_ctx=256, out_t=tq.TQ_F32, kvt=tq.TQ_BF16, ws=None,
            knew=FAKE, ctx=FAKE):
    if ws is None:
        ws = tq.append_decode_attend_workspace(batch, n_kv, group, max_ctx, 128)
    return tq.lib.tq_append_decode_attend(ctypes.byref(kc), ctypes.byref(vc), _p(), tq.TQ_BF16, _p(knew), _p(),
                                          kvt, batch, n_kv, group, _p(), _p(), _p(), _p(), cap, _p(ctx), max_ctx,
                                          0.1, _p(), out_t, _p(), ws, None)


def test_append_decode_validation():
    k, v = _codec(), _codec(w=4, key=0, sketch=False)
    assert _append(v, v) == tq.TQ_EINVAL                       # key codec expected
    assert _append(k, v, out_t=tq.TQ_F16) == tq.TQ_EUNSUPPORTED
    assert _append(k, v, max_ctx=512) == tq.TQ_EINVAL            # max_ctx > cap
    assert _append(k, v, group=33) == tq.TQ_EUNSUPPORTED
    assert _append(k, v, kvt=7) == tq.TQ_EINVAL                  # bad k_new/v_new dtype
    assert _append(k, v, knew=0) == tq.TQ_EINVAL                 # NULL k_new
    assert _append(k, v, ctx=0) == tq.TQ_EINVAL
    # one more partial per group than tq_decode_attend
    small = tq.decode_attend_workspace(2, 2, 4, 256, 128)
    assert tq.append_decode_attend_workspace(2, 2, 4, 256, 128) > small
    assert _append(k, v, ws=small) == tq.TQ_EINVAL
    assert _append(k, v, batch=0) == tq.TQ_OK


def _prefill(kc, vc, batch=2, chunk=8, n_kv=2, group=4, cap=256, max_ctx=256, ws=None, pos0=FAKE):
    if ws is None:
        ws = tq.prefill_attend_workspace(batch, chunk, n_kv, group, max_ctx, 128)
    return tq.lib.tq_prefill_attend(ctypes.byref(kc), ctypes.byref(vc), _p(), tq.TQ_BF16, batch, chunk, n_kv, group,
                                    _p(), _p(), _p(), _p(), cap, _p(pos0), max_ctx, 0.1, _p(), tq.TQ_F32, _p(), ws,
                                    None)


def test_prefill_validation():
    k, v = _codec(), _codec(w=4, key=0, sketch=False)
    assert _prefill(v, v) == tq.TQ_EINVAL
    assert _prefill(k, v, chunk=-1) == tq.TQ_EINVAL
    assert _prefill(k, v, chunk=257, group=4) == tq.TQ_EUNSUPPORTED      # more than 1024 (position, head) pairs
    assert _prefill(k, v, group=33) == tq.TQ_EUNSUPPORTED
    assert _prefill(k, v, pos0=0) == tq.TQ_EINVAL
    assert _prefill(k, v, max_ctx=512) == tq.TQ_EINVAL
    # the partials of every (position, head) pair
    # up to 8 (position, head) pairs per KV head: the decode kernels' partials
    # (1 block per group here); more: the single-pass kernel's partials (2
    # blocks of 128-token splits per group) and one prepared query record per
    # 8 pairs (sized for 4-bit keys: 2 row groups x 9 fragments x 2 KiB + 128)
    assert tq.prefill_attend_workspace(2, 2, 2, 4, 256, 128) == 2 * 2 * 1 * (2 * 4) * (128 + 2) * 4
    assert tq.prefill_attend_workspace(2, 8, 2, 4, 256, 128) == (2 * 2 * 2 * (8 * 4) * (128 + 2) * 4 +
                                                                 2 * 2 * 4 * (2 * 9 * 2 * 1024 + 128))
    assert _prefill(k, v, ws=tq.decode_attend_workspace(2, 2, 4, 256, 128)) == tq.TQ_EINVAL
    assert _prefill(k, v, chunk=0) == tq.TQ_OK
    assert _prefill(k, v, batch=0) == tq.TQ_OK


def test_fp8_key_calls_validation():
    x = _p(FAKE)
    enc = lambda **kw: tq.lib.tq_encode_fp8_keys(kw.get("x", x), kw.get("xt", tq.TQ_BF16), kw.get("d", 128), 2, 10,
                                                 10 * 128, 128, kw.get("scale", 1.0), kw.get("codes", x),
                                                 kw.get("cap", 32), kw.get("t0", 0), None)
    assert enc(d=60) == tq.TQ_EINVAL
    assert enc(scale=0.0) == tq.TQ_EINVAL
    assert enc(scale=float("inf")) == tq.TQ_EINVAL
    assert enc(t0=30) == tq.TQ_EINVAL                              # t0 + n_tok > cap
    assert enc(xt=5) == tq.TQ_EINVAL
    assert enc(codes=None) == tq.TQ_EINVAL
    v = _codec(w=4, key=0, sketch=False)
    ws = tq.decode_attend_workspace(2, 2, 4, 256, 128)
    dec = lambda **kw: tq.lib.tq_decode_attend_k8(ctypes.byref(kw.get("vc", v)), _p(), tq.TQ_BF16, 2, 2,
                                                  kw.get("group", 4), _p(), kw.get("ks", 1.0), _p(), _p(), 256, _p(),
                                                  kw.get("max_ctx", 256), 0.1, _p(), tq.TQ_F32, _p(),
                                                  kw.get("ws", ws), None)
    assert dec(ks=-1.0) == tq.TQ_EINVAL
    assert dec(vc=_codec()) == tq.TQ_EINVAL                        # a key codec where values are expected
    assert dec(max_ctx=512) == tq.TQ_EINVAL
    assert dec(group=33) == tq.TQ_EUNSUPPORTED
    assert dec(ws=64) == tq.TQ_EINVAL
    assert tq.lib.tq_decode_attend_k8(None, _p(), tq.TQ_BF16, 2, 2, 4, _p(), 1.0, _p(), _p(), 256, _p(), 256, 0.1,
                                      _p(), tq.TQ_F32, _p(), ws, None) == tq.TQ_EINVAL


def test_header_is_plain_c_and_links(tmp_path):
    """include/tq.h compiles as strict C99 and a C program links against
    libtq and calls its host entry points (no GPU needed)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "use_tq.c"
    src.write_text(
        '#include <stdio.h>\n#include "tq.h"\n'
        "int main(void) {\n"
        "  float c[4], t[3];\n"
        "  if (tq_make_codebook(128, 2, c, t) != TQ_OK) return 1;\n"
        "  if (!(c[0] < c[1] && c[1] < 0 && t[1] == 0.0f)) return 2;\n"
        "  if (tq_key_record_bytes(128, 3) != 64) return 3;\n"
        "  int32_t w[4];\n"
        "  if (tq_rate_plan(3.5, 4, 1, w) != TQ_OK || w[0] + w[1] + w[2] + w[3] != 10) return 4;\n"
        "  printf(\"%s\\n\", tq_status_string(TQ_EINVAL));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "use_tq"
    lib_dir = os.path.join(root, "kv_cache_vector_rht_amd")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(root, "include"),
                        str(src), "-o", str(exe), "-L", lib_dir, "-ltq", f"-Wl,-rpath,{lib_dir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.startswith("TQ_EINVAL")


def test_sequence_count_limit():
    """(batch, kv-head) sequences ride on the grid's y dimension: above 65535
    per call is rejected before any launch."""
    k, v = _codec(), _codec(w=4, key=0, sketch=False)
    assert _logits(k, batch=65536, n_kv=1) == tq.TQ_EUNSUPPORTED
    assert _decode(k, v, batch=65536, n_kv=1, ws=1 << 40) == tq.TQ_EUNSUPPORTED
    assert _append(k, v, batch=32768, n_kv=2, ws=1 << 40) == tq.TQ_EUNSUPPORTED
    assert _prefill(k, v, batch=70000, n_kv=1, ws=1 << 40) == tq.TQ_EUNSUPPORTED


def test_prepared_logits_validation():
    k = _codec()
    cs = ctypes.byref(k)
    need = tq.prepared_queries_bytes(2, 8, 4, 128, 2)
    assert need == 2 * 8 * 1 * (2 * (2 + 1) * 2 * 1024 + 128)
    assert tq.prepared_queries_bytes(2, 8, 4, 96, 2) == 0
    prep = lambda **kw: tq.lib.tq_prepare_queries(cs, _p(), kw.get("qt", tq.TQ_BF16), 2, 8, kw.get("group", 4),
                                                  kw.get("buf", _p()), kw.get("bytes", need), None)
    assert prep(bytes=need - 1) == tq.TQ_EINVAL
    assert prep(buf=None) == tq.TQ_EINVAL
    assert prep(qt=9) == tq.TQ_EINVAL
    assert prep(group=33) == tq.TQ_EUNSUPPORTED
    assert prep(group=0) == tq.TQ_OK
    lg = lambda **kw: tq.lib.tq_logits_prepared(cs, kw.get("buf", _p()), kw.get("bytes", need), 2, 8, 4, _p(), _p(),
                                                kw.get("cap", 256), kw.get("n", 256), _p(), None)
    assert lg(bytes=need - 1) == tq.TQ_EINVAL
    assert lg(n=300) == tq.TQ_EINVAL                                    # n_keys > cap
    assert lg(cap=250, n=200) == tq.TQ_EINVAL
    assert lg(n=0) == tq.TQ_OK


def test_rate_plan_matches_oracle():
    for n in (1, 3, 22, 64):
        for bits in (1.0, 1.5, 2.5, 3.25, 3.5, 4.0, 4.5):
            for is_key in (False, True):
                try:
                    ref = O.rate_plan(bits, n, is_key)
                except ValueError:
                    with pytest.raises(tq.TQError):
                        tq.rate_plan(bits, n, is_key)
                    continue
                assert tq.rate_plan(bits, n, is_key) == ref
    out = (ctypes.c_int32 * 4)()
    assert tq.lib.tq_rate_plan(3.5, 0, 1, out) == tq.TQ_EINVAL
    assert tq.lib.tq_rate_plan(float("nan"), 4, 1, out) == tq.TQ_EINVAL
    assert tq.lib.tq_rate_plan(3.5, 4, 2, out) == tq.TQ_EINVAL
    assert tq.lib.tq_rate_plan(3.5, 4, 1, None) == tq.TQ_EINVAL
    assert tq.lib.tq_rate_plan(1.5, 4, 1, out) == tq.TQ_EUNSUPPORTED     # 0.5 Lloyd-Max bits
    assert tq.lib.tq_rate_plan(5.5, 4, 0, out) == tq.TQ_EUNSUPPORTED


def _topk(n_rows=4, n_cols=5000, ld=5000, k=10, ws=None, scores=FAKE, out=FAKE):
    if ws is None:
        ws = tq.topk_workspace(n_rows, n_cols, k)
    return tq.lib.tq_topk(_p(scores), n_rows, n_cols, ld, k, _p(out), _p(out), _p(FAKE), ws, None)


def test_topk_validation():
    assert _topk(ld=4000) == tq.TQ_EINVAL                      # ld < n_cols
    assert _topk(k=5001) == tq.TQ_EINVAL                       # k > n_cols
    assert _topk(k=-1) == tq.TQ_EINVAL
    assert _topk(n_rows=-1) == tq.TQ_EINVAL
    assert _topk(k=1025, n_cols=5000) == tq.TQ_EUNSUPPORTED
    assert _topk(n_cols=1 << 31, ld=1 << 31) == tq.TQ_EUNSUPPORTED
    assert _topk(ws=8) == tq.TQ_EINVAL                         # workspace too small
    assert _topk(scores=0) == tq.TQ_EINVAL
    assert _topk(k=0) == tq.TQ_OK                              # no-ops launch nothing
    assert _topk(n_rows=0) == tq.TQ_OK
    # 8-byte candidates: k per 4096-column chunk, then k per 4096 candidates
    assert tq.topk_workspace(32, 1 << 20, 100) == 32 * (256 * 100 + 7 * 100) * 8
    assert tq.topk_workspace(1, 4097, 10) >= (2 * 10 + 10) * 8


def test_status_strings():
    for s in (tq.TQ_OK, tq.TQ_EINVAL, tq.TQ_EUNSUPPORTED, tq.TQ_EHIP):
        assert tq.lib.tq_status_string(s).decode().startswith("TQ_")


def _cpu_codecs(d=64):
    """Codecs whose arrays live on the host: every device call must refuse them."""
    rng = np.random.default_rng(3)
    s = rng.choice([-1.0, 1.0], size=d)
    S = rng.standard_normal((d, d)).astype(np.float16)
    return tq.Codec.make(d, 2, True, s, S, device="cpu"), tq.Codec.make(d, 4, False, s, device="cpu")


def test_binding_rejects_bad_tensors_before_any_launch():
    """The binding checks dtypes, shapes and devices before a pointer reaches
    the library: int64 context lengths (which the kernels would read as
    interleaved low and high words), queries of the wrong head size or head
    count, and host tensors."""
    import torch
    kc, vc = _cpu_codecs()
    batch, n_kv, group, cap, d = 2, 2, 4, 64, 64
    kcodes, kscal = tq.alloc_key_cache(batch * n_kv, cap, kc)
    vcodes, vscal = tq.alloc_value_cache(batch * n_kv, cap, vc)
    q = torch.zeros((batch, n_kv * group, d), dtype=torch.bfloat16)
    call = lambda **kw: tq.decode_attend(kc, vc, kw.get("q", q), kcodes, kscal, vcodes, vscal,
                                         kw.get("lens", torch.tensor([5, 7], dtype=torch.int32)),
                                         n_kv_heads=n_kv, group=group, max_ctx=cap)
    with pytest.raises(ValueError, match="int32"):
        call(lens=torch.tensor([5, 7]))                       # int64
    with pytest.raises(ValueError, match="at least 2"):
        call(lens=torch.tensor([5], dtype=torch.int32))
    with pytest.raises(ValueError, match="CUDA"):
        call()                                                # every tensor on the host
    with pytest.raises(ValueError, match="shape"):
        tq.logits(kc, torch.zeros((batch, n_kv * group, d // 2)), kcodes, kscal, n_kv_heads=n_kv, group=group,
                  n_keys=cap)
    with pytest.raises(ValueError, match="shape"):
        tq.logits(kc, torch.zeros((batch, n_kv * group + 1, d)), kcodes, kscal, n_kv_heads=n_kv, group=group,
                  n_keys=cap)
    with pytest.raises(ValueError, match="int32"):
        tq.prefill_attend(kc, vc, torch.zeros((batch, 3, n_kv * group, d)), kcodes, kscal, vcodes, vscal,
                          torch.zeros(batch, dtype=torch.int64), n_kv_heads=n_kv, group=group)
    with pytest.raises(ValueError, match="int32"):
        tq.append_decode_attend(kc, vc, q, torch.zeros((batch, n_kv, d)), torch.zeros((batch, n_kv, d)), kcodes,
                                kscal, vcodes, vscal, torch.tensor([5, 7]), n_kv_heads=n_kv, group=group)
    with pytest.raises(ValueError, match=f"\\[n_seq, n_tok, {d}\\]"):
        tq.encode_kv(kc, torch.zeros((n_kv, 10, d + 8)), kcodes, kscal)
    with pytest.raises(ValueError, match="CUDA"):
        tq.encode_kv(kc, torch.zeros((n_kv, 10, d)), kcodes, kscal)
