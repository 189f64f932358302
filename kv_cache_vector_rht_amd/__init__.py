"""Python binding of libtq, the TurboQuant KV-cache codec for MI355X (gfx950).

Argument marshalling only: every step of the codec runs in the HIP kernels of
libtq.so, called through its C ABI (include/tq.h). PyTorch provides device
memory and the current stream. There is no fallback: if the library is not
built, the first call raises.

    import kv_cache_vector_rht_amd as tq
    kc = tq.Codec.make(d=128, lm_bits=2, is_key=True, signs=s, sketch=S, device="cuda")
    kcodes, kscal = tq.alloc_key_cache(n_seq, cap, kc)
    tq.encode_kv(kc, x, kcodes, kscal)                     # x [n_seq, n_tok, d]
    logits = tq.logits(kc, q, kcodes, kscal, n_kv_heads=8, group=4, n_keys=n_tok)
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP = 0, -1, -2, -3
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
VALUE_BLOCK = 32

_DTYPE = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _Codec(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("lm_bits", ctypes.c_int32), ("is_key", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("signs", ctypes.c_void_p), ("centroids", ctypes.c_void_p),
                ("thresholds", ctypes.c_void_p), ("sketch", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libtq.so is not built ({LIB_PATH}); run "
                          "`python -m kv_cache_vector_rht_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    CP = ctypes.POINTER(_Codec)
    sig = {
        "tq_make_codebook": ([I32, I32, P, P], I32),
        "tq_rate_plan": ([ctypes.c_double, I32, I32, P], I32),
        "tq_key_record_bytes": ([I32, I32], SZ),
        "tq_mse_key_record_bytes": ([I32, I32], SZ),
        "tq_value_block_bytes": ([I32, I32], SZ),
        "tq_encode_kv": ([CP, P, I32, I64, I64, I64, I64, P, P, I64, I64, P], I32),
        "tq_logits": ([CP, P, I32, I32, I32, I32, P, P, I64, I64, P, P, SZ, P], I32),
        "tq_logits_workspace": ([I32, I32, I32, I32], SZ),
        "tq_logits_mse": ([CP, P, I32, I32, I32, I32, P, P, I64, I64, P, P, SZ, P], I32),
        "tq_prepared_queries_bytes": ([I32, I32, I32, I32, I32], SZ),
        "tq_prepare_queries": ([CP, P, I32, I32, I32, I32, P, SZ, P], I32),
        "tq_logits_prepared": ([CP, P, SZ, I32, I32, I32, P, P, I64, I64, P, P], I32),
        "tq_decode_attend": ([CP, CP, P, I32, I32, I32, I32, P, P, P, P, I64, P, I64, F, P, I32, P, SZ, P], I32),
        "tq_decode_attend_workspace": ([I32, I32, I32, I64, I32], SZ),
        "tq_decode_attend_noalloc": ([CP, CP, P, I32, I32, I32, I32, P, P, P, P, I64, P, I64, F, P, I32, P], I32),
        "tq_decode_attend_noalloc_max_workspace": ([], SZ),
        "tq_append_decode_attend": ([CP, CP, P, I32, P, P, I32, I32, I32, I32, P, P, P, P, I64, P, I64, F, P, I32, P,
                                     SZ, P], I32),
        "tq_append_decode_attend_workspace": ([I32, I32, I32, I64, I32], SZ),
        "tq_prefill_attend": ([CP, CP, P, I32, I32, I32, I32, I32, P, P, P, P, I64, P, I64, F, P, I32, P, SZ, P], I32),
        "tq_prefill_attend_workspace": ([I32, I32, I32, I32, I64, I32], SZ),
        "tq_encode_fp8_keys": ([P, I32, I32, I64, I64, I64, I64, F, P, I64, I64, P], I32),
        "tq_decode_attend_k8": ([CP, P, I32, I32, I32, I32, P, F, P, P, I64, P, I64, F, P, I32, P, SZ, P], I32),
        "tq_topk": ([P, I64, I64, I64, I32, P, P, P, SZ, P], I32),
        "tq_topk_workspace": ([I64, I64, I32], SZ),
        "tq_probe_read": ([P, SZ, P, P], I32),
        "tq_logits_table": ([CP, P, I32, I32, I32, I32, P, P, I64, I64, P, P, SZ, P], I32),
        "tq_logits_table_workspace": ([I32, I32, I32, I32], SZ),
        "tq_status_string": ([I32], ctypes.c_char_p),
        "tq_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


class _Lazy:
    """The loaded libtq; loaded on first use so that the build module can be
    imported before the library exists. Any use without a built library raises."""
    _lib = None

    def __getattr__(self, name):
        if _Lazy._lib is None:
            _Lazy._lib = _load()
        return getattr(_Lazy._lib, name)


lib = _Lazy()


def load():
    """Load libtq now (raises ImportError if it is not built)."""
    return lib.tq_status_string

EXPORTED = ("tq_make_codebook", "tq_rate_plan", "tq_key_record_bytes", "tq_mse_key_record_bytes",
            "tq_value_block_bytes", "tq_encode_kv",
            "tq_logits", "tq_logits_workspace", "tq_logits_mse", "tq_prepared_queries_bytes", "tq_prepare_queries",
            "tq_logits_prepared", "tq_decode_attend", "tq_decode_attend_workspace", "tq_decode_attend_noalloc",
            "tq_decode_attend_noalloc_max_workspace",
            "tq_append_decode_attend", "tq_append_decode_attend_workspace", "tq_prefill_attend",
            "tq_prefill_attend_workspace", "tq_encode_fp8_keys", "tq_decode_attend_k8",
            "tq_topk", "tq_topk_workspace", "tq_probe_read", "tq_logits_table", "tq_logits_table_workspace",
            "tq_status_string", "tq_last_error")


def _check(status: int, what: str):
    if status != TQ_OK:
        msg = lib.tq_last_error().decode()
        raise TQError(status, f"{what}: {lib.tq_status_string(status).decode()} ({msg})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run a device call with `stream` (when given) as torch's current stream,
    so that the binding's own copies (contiguous queries) and allocations
    (outputs, workspaces) are ordered on, and owned by, the stream the
    kernels run on."""
    import functools

    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, stream=None, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)
    return wrapper


# Argument checks of the device calls: shapes, dtypes and devices are
# validated here, before any pointer reaches the library (which sees only
# pointers and sizes). Errors are ValueError.

def _tensor(name, t):
    if not torch.is_tensor(t):
        raise ValueError(f"{name} must be a torch tensor")


def _device(name, t, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor (got one on {t.device})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the codec on {device}")


def _check_lens(name, t, batch, device):
    """int32 [>= batch], contiguous, on the codec's device."""
    _tensor(name, t)
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32 (got {t.dtype})")
    if t.dim() != 1 or t.numel() < batch:
        raise ValueError(f"{name} must be 1-D with at least {batch} entries (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _device(name, t, device)


def _check_queries(name, q, codec, lead, device):
    """q [*lead, d] in f32/bf16/f16 on the codec's device (made contiguous by the caller)."""
    _tensor(name, q)
    if q.dtype not in _DTYPE:
        raise ValueError(f"{name} must be float32, bfloat16 or float16 (got {q.dtype})")
    if tuple(q.shape) != tuple(lead) + (codec.d,):
        raise ValueError(f"{name} must have shape {tuple(lead) + (codec.d,)} (got {tuple(q.shape)})")
    _device(name, q, device)


def _check_out(out, shape, dtypes, device):
    _tensor("out", out)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)} (got {tuple(out.shape)})")
    if out.dtype not in dtypes:
        raise ValueError(f"out must be one of {dtypes} (got {out.dtype})")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _device("out", out, device)


def _check_key_cache(codec, codes, scal, n_seq, device):
    """Key cache of at least n_seq sequences: codes uint8 [S, cap, rec], scalars int16 [S, cap, 2]
    ([S, cap, 1] for MSE-only keys)."""
    _tensor("key codes", codes)
    _tensor("key scalars", scal)
    if codes.dtype != torch.uint8 or scal.dtype != torch.int16:
        raise ValueError("key codes must be uint8 and key scalars int16 (fp16 bits)")
    ns = codec.key_scalars
    if codes.dim() != 3 or scal.dim() != 3 or scal.shape[2] != ns:
        raise ValueError(f"key cache must be codes [n_seq, cap, rec] and scalars [n_seq, cap, {ns}]")
    if codes.shape[2] != codec.record_bytes:
        raise ValueError(f"key records must be {codec.record_bytes} bytes (got {codes.shape[2]})")
    if codes.shape[:2] != scal.shape[:2]:
        raise ValueError("key codes and scalars disagree in sequences or capacity")
    if codes.shape[0] < n_seq:
        raise ValueError(f"key cache holds {codes.shape[0]} sequences, the call needs {n_seq}")
    if not (codes.is_contiguous() and scal.is_contiguous()):
        raise ValueError("key cache tensors must be contiguous")
    _device("key codes", codes, device)
    _device("key scalars", scal, device)
    return scal.shape[1]


def _check_value_cache(codec, codes, scal, n_seq, cap, device):
    """Value cache: codes int32 [S, cap/32, w, d], scalars int16 [S, cap], the key cache's cap."""
    _tensor("value codes", codes)
    _tensor("value scalars", scal)
    if codes.dtype != torch.int32 or scal.dtype != torch.int16:
        raise ValueError("value codes must be int32 (uint32 words) and value scalars int16 (fp16 bits)")
    if codes.dim() != 4 or scal.dim() != 2:
        raise ValueError("value cache must be codes [n_seq, cap/32, w, d] and scalars [n_seq, cap]")
    if tuple(codes.shape[1:]) != (cap // VALUE_BLOCK, codec.lm_bits, codec.d) or scal.shape[1] != cap:
        raise ValueError(f"value cache must have {cap} slots of {codec.lm_bits}-bit, d={codec.d} codes "
                         f"(got codes {tuple(codes.shape)}, scalars {tuple(scal.shape)})")
    if codes.shape[0] != scal.shape[0] or codes.shape[0] < n_seq:
        raise ValueError(f"value cache holds {min(codes.shape[0], scal.shape[0])} sequences, the call needs {n_seq}")
    if not (codes.is_contiguous() and scal.is_contiguous()):
        raise ValueError("value cache tensors must be contiguous")
    _device("value codes", codes, device)
    _device("value scalars", scal, device)


def _check_workspace(ws, need, device):
    _tensor("workspace", ws)
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the call needs {need}")
    _device("workspace", ws, device)


# ---------------------------------------------------------------- codebook


def make_codebook(d: int, lm_bits: int):
    """Lloyd-Max codebook (host): (centroids float32 [2^w], thresholds float32 [2^w - 1])."""
    L = 1 << lm_bits
    c = torch.zeros(L, dtype=torch.float32)
    t = torch.zeros(max(L - 1, 1), dtype=torch.float32)
    _check(lib.tq_make_codebook(d, lm_bits, _ptr(c), _ptr(t)), "tq_make_codebook")
    return c, t[:L - 1]


def key_record_bytes(d: int, lm_bits: int) -> int:
    return int(lib.tq_key_record_bytes(d, lm_bits))


def mse_key_record_bytes(d: int, lm_bits: int) -> int:
    return int(lib.tq_mse_key_record_bytes(d, lm_bits))


def value_block_bytes(d: int, lm_bits: int) -> int:
    return int(lib.tq_value_block_bytes(d, lm_bits))


# ---------------------------------------------------------------- codec


@dataclass
class Codec:
    """Device-resident codec parameters (see tq_codec in include/tq.h).
    mse_only: key records without the QJL part (is_key = 2 in the C ABI)."""
    d: int
    lm_bits: int
    is_key: bool
    signs: torch.Tensor          # float32 [d]
    centroids: torch.Tensor      # float32 [2^w]
    thresholds: torch.Tensor     # float32 [2^w - 1]
    sketch: Optional[torch.Tensor] = None   # float16 [d, d] (keys with the QJL stage)
    mse_only: bool = False

    @staticmethod
    def make(d, lm_bits, is_key, signs, sketch=None, device="cuda", centroids=None, thresholds=None,
             mse_only=False):
        """Codec from rotation signs (+ sketch for keys with the QJL stage); the
        codebook comes from tq_make_codebook unless given."""
        if centroids is None or thresholds is None:
            centroids, thresholds = make_codebook(d, lm_bits)
        if mse_only and not is_key:
            raise ValueError("mse_only applies to key codecs")
        dev = torch.device(device)
        sk = None
        if is_key and not mse_only:
            if sketch is None:
                raise ValueError("a key codec needs a sketch")
            sk = torch.as_tensor(sketch).to(torch.float16).contiguous().to(dev)
        return Codec(d, lm_bits, bool(is_key),
                     torch.as_tensor(signs, dtype=torch.float32).contiguous().to(dev),
                     torch.as_tensor(centroids, dtype=torch.float32).contiguous().to(dev),
                     torch.as_tensor(thresholds, dtype=torch.float32).contiguous().to(dev), sk,
                     bool(mse_only))

    def struct(self) -> _Codec:
        s = _Codec()
        kind = (2 if self.mse_only else 1) if self.is_key else 0
        s.d, s.lm_bits, s.is_key, s.reserved = self.d, self.lm_bits, kind, 0
        s.signs = self.signs.data_ptr()
        s.centroids = self.centroids.data_ptr()
        s.thresholds = self.thresholds.data_ptr()
        s.sketch = self.sketch.data_ptr() if self.sketch is not None else None
        return s

    @property
    def record_bytes(self) -> int:
        if self.mse_only:
            return mse_key_record_bytes(self.d, self.lm_bits)
        return key_record_bytes(self.d, self.lm_bits)

    @property
    def key_scalars(self) -> int:
        """fp16 scalars stored per key token: {norm, residual norm}, or {norm} (MSE-only)."""
        return 1 if self.mse_only else 2


def rate_plan(bits: float, n_layers: int, is_key: bool) -> list:
    """Per-layer Lloyd-Max widths for a fractional rate of `bits` per channel (keys: QJL bit
    included): the two neighbouring integer widths spread evenly over the layers."""
    out = (ctypes.c_int32 * n_layers)() if n_layers > 0 else None
    _check(lib.tq_rate_plan(float(bits), n_layers, int(bool(is_key)), out), "tq_rate_plan")
    return list(out)


def alloc_key_cache(n_seq: int, cap: int, codec: Codec, device=None):
    """(codes uint8 [n_seq, cap, (w+1)d/8], scalars int16 [n_seq, cap, 2] holding fp16 bits);
    MSE-only keys: codes [n_seq, cap, w d/8], scalars [n_seq, cap, 1]."""
    dev = device or codec.signs.device
    codes = torch.zeros((n_seq, cap, codec.record_bytes), dtype=torch.uint8, device=dev)
    scal = torch.zeros((n_seq, cap, codec.key_scalars), dtype=torch.int16, device=dev)
    return codes, scal


def alloc_value_cache(n_seq: int, cap: int, codec: Codec, device=None):
    """(codes int32 [n_seq, cap/32, w, d] (uint32 words), scalars int16 [n_seq, cap] fp16 bits)."""
    if cap % VALUE_BLOCK:
        raise ValueError("value cache capacity must be a multiple of 32")
    dev = device or codec.signs.device
    codes = torch.zeros((n_seq, cap // VALUE_BLOCK, codec.lm_bits, codec.d), dtype=torch.int32, device=dev)
    scal = torch.zeros((n_seq, cap), dtype=torch.int16, device=dev)
    return codes, scal


# ---------------------------------------------------------------- device calls


def encode_kv(codec: Codec, x: torch.Tensor, codes: torch.Tensor, scalars: torch.Tensor,
              t0: int = 0, stream=None):
    """Encode x [n_seq, n_tok, d] (rows contiguous) into cache slots [t0, t0+n_tok)."""
    return _encode_kv(codec, x, codes, scalars, t0, stream=stream)


@_on_stream
def _encode_kv(codec, x, codes, scalars, t0, stream=None):
    _tensor("x", x)
    if x.dim() != 3 or x.stride(2) != 1 or x.shape[2] != codec.d:
        raise ValueError(f"x must be [n_seq, n_tok, {codec.d}] with contiguous rows (got {tuple(x.shape)})")
    if x.dtype not in _DTYPE:
        raise ValueError(f"x must be float32, bfloat16 or float16 (got {x.dtype})")
    n_seq, n_tok, d = x.shape
    dev = codec.signs.device
    _device("x", x, dev)
    if codec.is_key:
        cap = _check_key_cache(codec, codes, scalars, n_seq, dev)
    else:
        _tensor("value scalars", scalars)
        cap = scalars.shape[1] if scalars.dim() == 2 else -1
        _check_value_cache(codec, codes, scalars, n_seq, cap, dev)
    if t0 < 0 or t0 + n_tok > cap:
        raise ValueError(f"slots [{t0}, {t0 + n_tok}) exceed the cache capacity {cap}")
    cs = codec.struct()
    st = lib.tq_encode_kv(ctypes.byref(cs), _ptr(x), _DTYPE[x.dtype], n_seq, n_tok, x.stride(0), x.stride(1),
                          _ptr(codes), _ptr(scalars), cap, t0, _stream(stream))
    _check(st, "tq_encode_kv")


def logits_workspace(batch: int, n_kv_heads: int, group: int, d: int) -> int:
    return int(lib.tq_logits_workspace(batch, n_kv_heads, group, d))


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


@_on_stream
def logits(codec: Codec, q: torch.Tensor, codes: torch.Tensor, scalars: torch.Tensor, n_kv_heads: int,
           group: int, n_keys: int, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None, mse_only: bool = False) -> torch.Tensor:
    """Estimated q.k logits, float32 [batch, n_kv_heads*group, n_keys]. q: [batch, n_q, d].
    mse_only: the estimator's first term alone (tq_logits_mse, the ablation without the QJL bit)."""
    dev = codec.signs.device
    _tensor("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [batch, n_kv_heads*group, d]")
    batch = q.shape[0]
    n_q = n_kv_heads * group
    _check_queries("q", q, codec, (batch, n_q), dev)
    q = q.contiguous()
    cap = _check_key_cache(codec, codes, scalars, batch * n_kv_heads, dev)
    if n_keys < 0 or n_keys > cap:
        raise ValueError(f"n_keys={n_keys} outside [0, {cap}]")
    if out is None:
        out = torch.empty((batch, n_q, n_keys), dtype=torch.float32, device=dev)
    _check_out(out, (batch, n_q, n_keys), (torch.float32,), dev)
    need = logits_workspace(batch, n_kv_heads, group, codec.d)
    if workspace is None:
        workspace = _workspace(need, dev)
    _check_workspace(workspace, need, dev)
    cs = codec.struct()
    fn = lib.tq_logits_mse if mse_only else lib.tq_logits
    st = fn(ctypes.byref(cs), _ptr(q), _DTYPE[q.dtype], batch, n_kv_heads, group, _ptr(codes),
            _ptr(scalars), cap, n_keys, _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "tq_logits_mse" if mse_only else "tq_logits")
    return out


def decode_attend_workspace(batch: int, n_kv_heads: int, group: int, max_ctx: int, d: int) -> int:
    return int(lib.tq_decode_attend_workspace(batch, n_kv_heads, group, max_ctx, d))


def _attend_common(kc, vc, q, lead, kcodes, kscalars, vcodes, vscalars, lens, lens_name, batch, n_kv_heads,
                   max_ctx, sm_scale, out, out_dtype, key_codec=True):
    """Checks shared by the attention calls; returns (q, cap, max_ctx, sm_scale, out, out dtype code)."""
    dev = vc.signs.device
    _check_lens(lens_name, lens, batch, dev)
    if key_codec and kc.signs.device != dev:
        raise ValueError("key and value codecs are on different devices")
    if key_codec and kc.d != vc.d:
        raise ValueError(f"key d={kc.d} and value d={vc.d} differ")
    _check_queries("q", q, vc, lead, dev)
    q = q.contiguous()
    n_seq = batch * n_kv_heads
    if key_codec:
        cap = _check_key_cache(kc, kcodes, kscalars, n_seq, dev)
    else:
        _tensor("fp8 key codes", kcodes)
        if kcodes.dtype != torch.uint8 or kcodes.dim() != 3 or kcodes.shape[2] != vc.d:
            raise ValueError(f"fp8 key cache must be uint8 [n_seq, cap, {vc.d}]")
        if kcodes.shape[0] < n_seq or not kcodes.is_contiguous():
            raise ValueError(f"fp8 key cache must be contiguous with at least {n_seq} sequences")
        _device("fp8 key codes", kcodes, dev)
        cap = kcodes.shape[1]
    _check_value_cache(vc, vcodes, vscalars, n_seq, cap, dev)
    if max_ctx is None:
        max_ctx = cap
    if max_ctx < 0 or max_ctx > cap:
        raise ValueError(f"max_ctx={max_ctx} outside [0, {cap}]")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(vc.d)
    if out is None:
        out = torch.empty(tuple(lead) + (vc.d,), dtype=out_dtype, device=dev)
    _check_out(out, tuple(lead) + (vc.d,), (torch.float32, torch.bfloat16), dev)
    ot = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[out.dtype]
    return q, cap, max_ctx, sm_scale, out, ot


def _batch_of(q, dims, what):
    _tensor("q", q)
    if q.dim() != dims:
        raise ValueError(f"q must be {what}")
    return q.shape[0]


@_on_stream
def decode_attend(kc: Codec, vc: Codec, q: torch.Tensor, kcodes, kscalars, vcodes, vscalars, ctx_lens: torch.Tensor,
                  n_kv_heads: int, group: int, max_ctx: Optional[int] = None, sm_scale: Optional[float] = None,
                  out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Fused decode attention over the coded cache: [batch, n_q, d] in out_dtype."""
    batch = _batch_of(q, 3, "[batch, n_kv_heads*group, d]")
    n_q = n_kv_heads * group
    q, cap, max_ctx, sm_scale, out, ot = _attend_common(kc, vc, q, (batch, n_q), kcodes, kscalars, vcodes, vscalars,
                                                        ctx_lens, "ctx_lens", batch, n_kv_heads, max_ctx, sm_scale,
                                                        out, out_dtype)
    need = decode_attend_workspace(batch, n_kv_heads, group, max_ctx, kc.d)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check_workspace(workspace, need, q.device)
    ks, vs = kc.struct(), vc.struct()
    st = lib.tq_decode_attend(ctypes.byref(ks), ctypes.byref(vs), _ptr(q), _DTYPE[q.dtype], batch, n_kv_heads,
                              group, _ptr(kcodes), _ptr(kscalars), _ptr(vcodes), _ptr(vscalars), cap,
                              _ptr(ctx_lens), max_ctx, float(sm_scale), _ptr(out), ot, _ptr(workspace),
                              workspace.numel(), _stream(stream))
    _check(st, "tq_decode_attend")
    return out


@_on_stream
def decode_attend_noalloc(kc: Codec, vc: Codec, q: torch.Tensor, kcodes, kscalars, vcodes, vscalars,
                          ctx_lens: torch.Tensor, n_kv_heads: int, group: int, out: torch.Tensor,
                          max_ctx: Optional[int] = None, sm_scale: Optional[float] = None,
                          stream=None) -> torch.Tensor:
    """decode_attend with the split partials in the library's fixed device scratch (no workspace):
    q must be contiguous and `out` given, so that the call allocates nothing. Calls that overlap on
    one GPU share the scratch and must be serialized."""
    batch = _batch_of(q, 3, "[batch, n_kv_heads*group, d]")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous (the call makes no copies)")
    n_q = n_kv_heads * group
    q, cap, max_ctx, sm_scale, out, ot = _attend_common(kc, vc, q, (batch, n_q), kcodes, kscalars, vcodes, vscalars,
                                                        ctx_lens, "ctx_lens", batch, n_kv_heads, max_ctx, sm_scale,
                                                        out, out.dtype if torch.is_tensor(out) else None)
    ks, vs = kc.struct(), vc.struct()
    st = lib.tq_decode_attend_noalloc(ctypes.byref(ks), ctypes.byref(vs), _ptr(q), _DTYPE[q.dtype], batch,
                                      n_kv_heads, group, _ptr(kcodes), _ptr(kscalars), _ptr(vcodes), _ptr(vscalars),
                                      cap, _ptr(ctx_lens), max_ctx, float(sm_scale), _ptr(out), ot, _stream(stream))
    _check(st, "tq_decode_attend_noalloc")
    return out


def decode_attend_noalloc_max_workspace() -> int:
    return int(lib.tq_decode_attend_noalloc_max_workspace())


def prepared_queries_bytes(batch: int, n_kv_heads: int, group: int, d: int, lm_bits: int) -> int:
    return int(lib.tq_prepared_queries_bytes(batch, n_kv_heads, group, d, lm_bits))


@_on_stream
def prepare_queries(codec: Codec, q: torch.Tensor, n_kv_heads: int, group: int,
                    prepared: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The query preparation of tq_logits alone: an opaque uint8 buffer for logits_prepared."""
    dev = codec.signs.device
    batch = _batch_of(q, 3, "[batch, n_kv_heads*group, d]")
    _check_queries("q", q, codec, (batch, n_kv_heads * group), dev)
    q = q.contiguous()
    need = prepared_queries_bytes(batch, n_kv_heads, group, codec.d, codec.lm_bits)
    if prepared is None:
        prepared = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _tensor("prepared", prepared)
    if prepared.dtype != torch.uint8 or not prepared.is_contiguous() or prepared.numel() < need:
        raise ValueError(f"prepared must be a contiguous uint8 tensor of at least {need} bytes")
    _device("prepared", prepared, dev)
    cs = codec.struct()
    st = lib.tq_prepare_queries(ctypes.byref(cs), _ptr(q), _DTYPE[q.dtype], batch, n_kv_heads, group, _ptr(prepared),
                                prepared.numel(), _stream(stream))
    _check(st, "tq_prepare_queries")
    return prepared


@_on_stream
def logits_prepared(codec: Codec, prepared: torch.Tensor, batch: int, codes: torch.Tensor, scalars: torch.Tensor,
                    n_kv_heads: int, group: int, n_keys: int, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """tq_logits from prepared queries: float32 [batch, n_kv_heads*group, n_keys]."""
    dev = codec.signs.device
    _tensor("prepared", prepared)
    need = prepared_queries_bytes(batch, n_kv_heads, group, codec.d, codec.lm_bits)
    if prepared.dtype != torch.uint8 or not prepared.is_contiguous() or prepared.numel() < need:
        raise ValueError(f"prepared must be a contiguous uint8 tensor of at least {need} bytes")
    _device("prepared", prepared, dev)
    cap = _check_key_cache(codec, codes, scalars, batch * n_kv_heads, dev)
    if n_keys < 0 or n_keys > cap:
        raise ValueError(f"n_keys={n_keys} outside [0, {cap}]")
    n_q = n_kv_heads * group
    if out is None:
        out = torch.empty((batch, n_q, n_keys), dtype=torch.float32, device=dev)
    _check_out(out, (batch, n_q, n_keys), (torch.float32,), dev)
    cs = codec.struct()
    st = lib.tq_logits_prepared(ctypes.byref(cs), _ptr(prepared), prepared.numel(), batch, n_kv_heads, group,
                                _ptr(codes), _ptr(scalars), cap, n_keys, _ptr(out), _stream(stream))
    _check(st, "tq_logits_prepared")
    return out


def append_decode_attend_workspace(batch: int, n_kv_heads: int, group: int, max_ctx: int, d: int) -> int:
    return int(lib.tq_append_decode_attend_workspace(batch, n_kv_heads, group, max_ctx, d))


@_on_stream
def append_decode_attend(kc: Codec, vc: Codec, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, kcodes,
                         kscalars, vcodes, vscalars, ctx_lens: torch.Tensor, n_kv_heads: int, group: int,
                         max_ctx: Optional[int] = None, sm_scale: Optional[float] = None, out_dtype=torch.float32,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """One decoding step in one launch: k_new / v_new [batch, n_kv_heads, d] are encoded into slot
    ctx_lens[b] - 1 of the caches (ctx_lens counts the new token) and the queries attend over the whole
    context: [batch, n_q, d] in out_dtype."""
    batch = _batch_of(q, 3, "[batch, n_kv_heads*group, d]")
    n_q = n_kv_heads * group
    q, cap, max_ctx, sm_scale, out, ot = _attend_common(kc, vc, q, (batch, n_q), kcodes, kscalars, vcodes, vscalars,
                                                        ctx_lens, "ctx_lens", batch, n_kv_heads, max_ctx, sm_scale,
                                                        out, out_dtype)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _tensor(name, t)
        if t.dtype not in _DTYPE or tuple(t.shape) != (batch, n_kv_heads, kc.d):
            raise ValueError(f"{name} must be float32/bfloat16/float16 [{batch}, {n_kv_heads}, {kc.d}]")
        _device(name, t, q.device)
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    k_new, v_new = k_new.contiguous(), v_new.contiguous()
    need = append_decode_attend_workspace(batch, n_kv_heads, group, max_ctx, kc.d)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check_workspace(workspace, need, q.device)
    ks, vs = kc.struct(), vc.struct()
    st = lib.tq_append_decode_attend(ctypes.byref(ks), ctypes.byref(vs), _ptr(q), _DTYPE[q.dtype], _ptr(k_new),
                                     _ptr(v_new), _DTYPE[k_new.dtype], batch, n_kv_heads, group, _ptr(kcodes),
                                     _ptr(kscalars), _ptr(vcodes), _ptr(vscalars), cap, _ptr(ctx_lens), max_ctx,
                                     float(sm_scale), _ptr(out), ot, _ptr(workspace), workspace.numel(),
                                     _stream(stream))
    _check(st, "tq_append_decode_attend")
    return out


def prefill_attend_workspace(batch: int, chunk: int, n_kv_heads: int, group: int, max_ctx: int, d: int) -> int:
    return int(lib.tq_prefill_attend_workspace(batch, chunk, n_kv_heads, group, max_ctx, d))


@_on_stream
def prefill_attend(kc: Codec, vc: Codec, q: torch.Tensor, kcodes, kscalars, vcodes, vscalars, pos0: torch.Tensor,
                   n_kv_heads: int, group: int, max_ctx: Optional[int] = None, sm_scale: Optional[float] = None,
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal attention of a prefill chunk q [batch, chunk, n_q, d] over the coded cache, whose slots
    [pos0[b], pos0[b] + chunk) already hold the chunk's keys and values: position i of row b attends to
    the tokens t <= pos0[b] + i. Returns [batch, chunk, n_q, d] in out_dtype."""
    batch = _batch_of(q, 4, "[batch, chunk, n_kv_heads*group, d]")
    chunk = q.shape[1]
    n_q = n_kv_heads * group
    q, cap, max_ctx, sm_scale, out, ot = _attend_common(kc, vc, q, (batch, chunk, n_q), kcodes, kscalars, vcodes,
                                                        vscalars, pos0, "pos0", batch, n_kv_heads, max_ctx,
                                                        sm_scale, out, out_dtype)
    need = prefill_attend_workspace(batch, chunk, n_kv_heads, group, max_ctx, kc.d)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check_workspace(workspace, need, q.device)
    ks, vs = kc.struct(), vc.struct()
    st = lib.tq_prefill_attend(ctypes.byref(ks), ctypes.byref(vs), _ptr(q), _DTYPE[q.dtype], batch, chunk, n_kv_heads,
                               group, _ptr(kcodes), _ptr(kscalars), _ptr(vcodes), _ptr(vscalars), cap, _ptr(pos0),
                               max_ctx, float(sm_scale), _ptr(out), ot, _ptr(workspace), workspace.numel(),
                               _stream(stream))
    _check(st, "tq_prefill_attend")
    return out


def alloc_fp8_key_cache(n_seq: int, cap: int, d: int, device="cuda") -> torch.Tensor:
    """fp8 key cache: uint8 [n_seq, cap, d] of OCP e4m3fn bytes."""
    return torch.zeros((n_seq, cap, d), dtype=torch.uint8, device=device)


@_on_stream
def encode_fp8_keys(x: torch.Tensor, codes: torch.Tensor, scale: float = 1.0, t0: int = 0, stream=None):
    """Encode keys x [n_seq, n_tok, d] (rows contiguous) as e4m3fn(x / scale) into slots [t0, t0 + n_tok)."""
    _tensor("x", x)
    _tensor("codes", codes)
    if x.dim() != 3 or x.stride(2) != 1 or x.dtype not in _DTYPE:
        raise ValueError("x must be a float32/bfloat16/float16 [n_seq, n_tok, d] tensor with contiguous rows")
    n_seq, n_tok, d = x.shape
    if codes.dtype != torch.uint8 or codes.dim() != 3 or codes.shape[2] != d or codes.shape[0] < n_seq \
            or not codes.is_contiguous():
        raise ValueError(f"codes must be a contiguous uint8 [>= {n_seq}, cap, {d}] tensor")
    if t0 < 0 or t0 + n_tok > codes.shape[1]:
        raise ValueError(f"slots [{t0}, {t0 + n_tok}) exceed the cache capacity {codes.shape[1]}")
    _device("x", x, codes.device)
    _device("codes", codes, x.device)
    st = lib.tq_encode_fp8_keys(_ptr(x), _DTYPE[x.dtype], d, n_seq, n_tok, x.stride(0), x.stride(1), float(scale),
                                _ptr(codes), codes.shape[1], t0, _stream(stream))
    _check(st, "tq_encode_fp8_keys")


@_on_stream
def decode_attend_k8(vc: Codec, q: torch.Tensor, kcodes: torch.Tensor, vcodes, vscalars, ctx_lens: torch.Tensor,
                     n_kv_heads: int, group: int, k_scale: float = 1.0, max_ctx: Optional[int] = None,
                     sm_scale: Optional[float] = None, out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention over fp8 keys and TurboQuant values (the k8v4 shape): [batch, n_q, d]."""
    batch = _batch_of(q, 3, "[batch, n_kv_heads*group, d]")
    n_q = n_kv_heads * group
    q, cap, max_ctx, sm_scale, out, ot = _attend_common(None, vc, q, (batch, n_q), kcodes, None, vcodes, vscalars,
                                                        ctx_lens, "ctx_lens", batch, n_kv_heads, max_ctx, sm_scale,
                                                        out, out_dtype, key_codec=False)
    need = decode_attend_workspace(batch, n_kv_heads, group, max_ctx, vc.d)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check_workspace(workspace, need, q.device)
    vs = vc.struct()
    st = lib.tq_decode_attend_k8(ctypes.byref(vs), _ptr(q), _DTYPE[q.dtype], batch, n_kv_heads, group, _ptr(kcodes),
                                 float(k_scale), _ptr(vcodes), _ptr(vscalars), cap, _ptr(ctx_lens), max_ctx,
                                 float(sm_scale), _ptr(out), ot, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "tq_decode_attend_k8")
    return out


def topk_workspace(n_rows: int, n_cols: int, k: int) -> int:
    return int(lib.tq_topk_workspace(n_rows, n_cols, k))


@_on_stream
def topk(scores: torch.Tensor, k: int, n_cols: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
         stream=None):
    """The k largest entries of each row of a float32 [n_rows, >= n_cols] matrix (rows may be padded:
    stride(0) is the leading dimension): (values [n_rows, k] descending, columns int32 [n_rows, k]);
    ties go to the smaller column."""
    _tensor("scores", scores)
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be a float32 [n_rows, n] matrix with unit column stride")
    if not scores.is_cuda:
        raise ValueError("scores must be a CUDA tensor")
    n_rows = scores.shape[0]
    if n_cols is None:
        n_cols = scores.shape[1]
    if n_cols < 0 or n_cols > scores.shape[1]:
        raise ValueError(f"n_cols={n_cols} outside [0, {scores.shape[1]}]")
    vals = torch.empty((n_rows, k), dtype=torch.float32, device=scores.device)
    idx = torch.empty((n_rows, k), dtype=torch.int32, device=scores.device)
    need = topk_workspace(n_rows, n_cols, k)
    if workspace is None:
        workspace = _workspace(need, scores.device)
    _check_workspace(workspace, need, scores.device)
    st = lib.tq_topk(_ptr(scores), n_rows, n_cols, scores.stride(0), k, _ptr(vals), _ptr(idx), _ptr(workspace),
                     workspace.numel(), _stream(stream))
    _check(st, "tq_topk")
    return vals, idx


@_on_stream
def probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Measurement only: one read-and-reduce pass over the bytes of a contiguous CUDA tensor
    (tq_probe_read); sink is a CUDA int32/uint32 tensor of at least one element."""
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda):
        raise ValueError("src must be a contiguous CUDA tensor and sink a CUDA tensor")
    st = lib.tq_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream))
    _check(st, "tq_probe_read")


@_on_stream
def logits_table(codec: Codec, q: torch.Tensor, codes: torch.Tensor, scalars: torch.Tensor, n_kv_heads: int,
                 group: int, n_keys: int, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """Measurement path: the logits of tq_logits from the LDS-table formulation of the scan
    (tq_logits_table); float32 [batch, n_kv_heads*group, n_keys]."""
    dev = codec.signs.device
    _tensor("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [batch, n_kv_heads*group, d]")
    batch = q.shape[0]
    n_q = n_kv_heads * group
    _check_queries("q", q, codec, (batch, n_q), dev)
    q = q.contiguous()
    cap = _check_key_cache(codec, codes, scalars, batch * n_kv_heads, dev)
    if n_keys < 0 or n_keys > cap:
        raise ValueError(f"n_keys={n_keys} outside [0, {cap}]")
    if out is None:
        out = torch.empty((batch, n_q, n_keys), dtype=torch.float32, device=dev)
    _check_out(out, (batch, n_q, n_keys), (torch.float32,), dev)
    need = int(lib.tq_logits_table_workspace(batch, n_kv_heads, group, codec.d))
    if workspace is None:
        workspace = _workspace(need, dev)
    _check_workspace(workspace, need, dev)
    cs = codec.struct()
    st = lib.tq_logits_table(ctypes.byref(cs), _ptr(q), _DTYPE[q.dtype], batch, n_kv_heads, group, _ptr(codes),
                             _ptr(scalars), cap, n_keys, _ptr(out), _ptr(workspace), workspace.numel(),
                             _stream(stream))
    _check(st, "tq_logits_table")
    return out


@_on_stream
def search(codec: Codec, q: torch.Tensor, codes: torch.Tensor, scalars: torch.Tensor, n_db: int, k: int,
           scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Inner-product search of up to 32 queries [n_q, d] over a coded database (the keys of one
    sequence: codes/scalars of a key cache with one sequence, its first n_db slots): the
    estimated scores by the logit scan, then their top k per query.
    Returns (values [n_q, k], columns int32 [n_q, k])."""
    _tensor("q", q)
    if q.dim() != 2:
        raise ValueError("q must be [n_q, d]")
    n_q = q.shape[0]
    if scores is None:
        scores = torch.empty((1, n_q, n_db), dtype=torch.float32, device=q.device)
    logits(codec, q.unsqueeze(0), codes, scalars, n_kv_heads=1, group=n_q, n_keys=n_db, out=scores, stream=stream)
    return topk(scores.view(n_q, n_db), k, workspace=workspace, stream=stream)
