"""Seeded synthetic workloads for the TurboQuant KV-cache codec.

This module only draws random numbers and lays them out; it holds none of
the codec's arithmetic. Both the GPU path (tests, bench) and the CPU oracle
are fed from here, so the two always see identical arrays.

Every array is drawn from a ``torch.Generator`` seeded with
``seed(cfg, stream, copy)``. Streams:

  0  key codec randomness: rotation signs s_k (d), then QJL sketch S (d x d)
  1  keys
  2  values
  3  queries
  4  channel scales and outlier masks
  5  value codec randomness: rotation signs s_v (d)
  6  context lengths (ragged batches in tests)

Codec randomness (signs, sketch) is always drawn on the CPU so that it is the
same on every machine. Bulk tensors (K, V, Q) are drawn on the device that
asks for them; the CPU generator and the GPU generator are different
algorithms, so a parity test draws on the GPU and copies the slice it checks
back to the host for the oracle.

The workloads stand in for the model shapes the pages mention (Llama-3.1-8B,
Qwen3-4B and TinyLlama-1.1B attention layers, contexts up to 128K tokens);
no dataset or weight file is involved.
"""
from __future__ import annotations

import dataclasses
import torch

# --------------------------------------------------------------------------
# workload table
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    d: int
    batch: int
    n_kv: int            # KV heads (per layer)
    group: int           # query heads per KV head (0: no queries / encode only)
    n_tok: int           # context length (tokens per sequence)
    key_bits: int        # b: (b-1) Lloyd-Max bits + 1 QJL bit
    val_bits: int        # Lloyd-Max bits of values (0: no values)
    in_dtype: torch.dtype
    layers: int = 1
    timed: str = ""      # the operation the bench times on this workload

    @property
    def key_lm_bits(self) -> int:
        return self.key_bits - 1

    @property
    def n_q(self) -> int:
        return self.n_kv * self.group

    @property
    def n_seq(self) -> int:
        """Number of (layer, batch, kv-head) sequences in the cache."""
        return self.layers * self.batch * self.n_kv

    @property
    def n_vec(self) -> int:
        return self.n_seq * self.n_tok


WORKLOADS = {
    1: Workload(1, "single-head d128 N4096 fp32 keys with 4 outlier channels x20, 16 queries",
                d=128, batch=1, n_kv=1, group=16, n_tok=4096, key_bits=3, val_bits=0,
                in_dtype=torch.float32, timed="encode+logits"),
    2: Workload(2, "Llama-3.1-8B-shaped decode layer: 8 KV / 32 Q heads, d128, batch 1, ctx 32768",
                d=128, batch=1, n_kv=8, group=4, n_tok=32768, key_bits=4, val_bits=0,
                in_dtype=torch.bfloat16, timed="logits"),
    3: Workload(3, "Qwen3-4B-shaped batched decode: 8 KV / 32 Q heads, d128, batch 16 x ctx 8192",
                d=128, batch=16, n_kv=8, group=4, n_tok=8192, key_bits=3, val_bits=4,
                in_dtype=torch.bfloat16, timed="decode_attend"),
    4: Workload(4, "TinyLlama-1.1B-shaped prefill encode: 22 layers x 32 heads, d64, batch 64 x 4096",
                d=64, batch=64, n_kv=32, group=0, n_tok=4096, key_bits=3, val_bits=4,
                in_dtype=torch.bfloat16, layers=22, timed="encode"),
    5: Workload(5, "long-context decode: 8 KV / 64 Q heads, d128, batch 4 x ctx 131072",
                d=128, batch=4, n_kv=8, group=8, n_tok=131072, key_bits=4, val_bits=4,
                in_dtype=torch.bfloat16, timed="decode_attend"),
}

STREAM_KEY_CODEC = 0
STREAM_K = 1
STREAM_V = 2
STREAM_Q = 3
STREAM_SCALES = 4
STREAM_VAL_CODEC = 5
STREAM_CTX = 6


def seed(cfg: int, stream: int, copy: int = 0) -> int:
    """Deterministic 63-bit seed for (config, stream, copy)."""
    return (cfg * 1_000_003 + stream * 10_007 + copy * 101) & ((1 << 63) - 1)


def generator(cfg: int, stream: int, copy: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed(cfg, stream, copy))
    return g


# --------------------------------------------------------------------------
# codec randomness (always CPU)
# --------------------------------------------------------------------------


def rademacher(n: int, g: torch.Generator) -> torch.Tensor:
    """n iid +-1 values as float32."""
    bits = torch.randint(0, 2, (n,), generator=g, dtype=torch.int64)
    return (bits * 2 - 1).to(torch.float32)


def key_codec_randoms(cfg: int, d: int):
    """Rotation signs s_k [d] (float32 +-1) and QJL sketch S [d, d] (float16).

    S is drawn as float32 N(0, 1) and rounded once to float16: the sketch is
    fp16-representable by construction, and both the oracle and the GPU use
    exactly these values.
    """
    g = generator(cfg, STREAM_KEY_CODEC)
    signs = rademacher(d, g)
    sketch = torch.randn((d, d), generator=g, dtype=torch.float32).to(torch.float16)
    return signs, sketch


def value_codec_randoms(cfg: int, d: int) -> torch.Tensor:
    """Rotation signs s_v [d] of the value codec."""
    return rademacher(d, generator(cfg, STREAM_VAL_CODEC))


# --------------------------------------------------------------------------
# bulk tensors
# --------------------------------------------------------------------------


def _randn_into(out: torch.Tensor, g, scale_fn=None, chunk_elems=1 << 27):
    """Fill ``out`` (any float dtype, dim 0 = sequences) with N(0,1) draws.

    Draws are made in float32, chunk by chunk along dim 0, optionally scaled
    by ``scale_fn(r0, r1, x)`` in float32, then rounded to ``out.dtype``.
    """
    per_row = out[0].numel() if out.shape[0] else 1
    rows = max(1, chunk_elems // max(1, per_row))
    for r0 in range(0, out.shape[0], rows):
        r1 = min(out.shape[0], r0 + rows)
        x = torch.randn((r1 - r0,) + tuple(out.shape[1:]), generator=g,
                        dtype=torch.float32, device=out.device)
        if scale_fn is not None:
            scale_fn(r0, r1, x)
        out[r0:r1] = x.to(out.dtype)
    return out


def channel_scales(cfg: int, n_kv: int, d: int, which: int) -> torch.Tensor:
    """Per (kv-head, channel) lognormal(0,1) scales [n_kv, d]; which=0 keys, 1 values."""
    g = generator(cfg, STREAM_SCALES, copy=which)
    return torch.exp(torch.randn((n_kv, d), generator=g, dtype=torch.float32))


def outlier_channels_cfg1(d: int = 128, count: int = 4) -> torch.Tensor:
    """The 4 fixed outlier channels of the single-head workload (without replacement)."""
    g = generator(1, STREAM_SCALES)
    return torch.randperm(d, generator=g)[:count].sort().values


def outlier_mask_cfg4(which: int, layers=22, heads=32, d=64, p=0.02) -> torch.Tensor:
    """Boolean [layers, heads, d]: each (layer, head, channel) is an outlier w.p. p."""
    g = generator(4, STREAM_SCALES, copy=which)
    return torch.rand((layers, heads, d), generator=g) < p


def keys(w: Workload, device="cpu", copy: int = 0) -> torch.Tensor:
    """Key cache input.

    Shape [layers*batch*n_kv, n_tok, d] (one row block per sequence), in the
    workload's input dtype. Sequence index = (layer*batch + b)*n_kv + h.
    """
    return _kv(w, STREAM_K, 0, device, copy)


def values(w: Workload, device="cpu", copy: int = 0) -> torch.Tensor:
    assert w.val_bits > 0
    return _kv(w, STREAM_V, 1, device, copy)


def _kv(w: Workload, stream: int, which: int, device, copy: int) -> torch.Tensor:
    g = generator(w.cfg, stream, copy, device=device)
    out = torch.empty((w.n_seq, w.n_tok, w.d), dtype=w.in_dtype, device=device)
    scale_fn = None
    if w.cfg == 1:
        ch = outlier_channels_cfg1(w.d).to(device)

        def scale_fn(r0, r1, x):
            x[:, :, ch] *= 20.0
    elif w.cfg in (2, 5):
        sc = channel_scales(w.cfg, w.n_kv, w.d, which).to(device)       # [n_kv, d]

        def scale_fn(r0, r1, x):
            head = torch.arange(r0, r1, device=device) % w.n_kv
            x.mul_(sc[head][:, None, :])
    elif w.cfg == 4:
        m = outlier_mask_cfg4(which, w.layers, w.n_kv, w.d).to(device)  # [L, H, d]
        sc = torch.where(m, 10.0, 1.0).to(torch.float32)

        def scale_fn(r0, r1, x):
            seqs = torch.arange(r0, r1, device=device)
            layer = seqs // (w.batch * w.n_kv)
            head = seqs % w.n_kv
            x.mul_(sc[layer, head][:, None, :])
    return _randn_into(out, g, scale_fn)


def kv_slice(w: Workload, which: int, layer: int = 0, b: int = 0, device="cpu") -> torch.Tensor:
    """The n_kv sequences of one (layer, batch row) of a workload, [n_kv, n_tok, d]
    in its input dtype, drawn from a generator of their own (copy 1000 + the
    slice's index) with the same law as ``keys``/``values`` (which = 0 / 1):
    the layer's outlier mask, the channel scales, the outlier channels. The
    draws differ from those of the full cache; a stand-in of the same law for
    timing samples of caches too large to draw whole."""
    g = generator(w.cfg, STREAM_K if which == 0 else STREAM_V, 1000 + layer * w.batch + b, device=device)
    out = torch.empty((w.n_kv, w.n_tok, w.d), dtype=w.in_dtype, device=device)
    scale_fn = None
    if w.cfg == 1:
        ch = outlier_channels_cfg1(w.d).to(device)

        def scale_fn(r0, r1, x):
            x[:, :, ch] *= 20.0
    elif w.cfg in (2, 5):
        sc = channel_scales(w.cfg, w.n_kv, w.d, which).to(device)

        def scale_fn(r0, r1, x):
            x.mul_(sc[r0:r1][:, None, :])
    elif w.cfg == 4:
        m = outlier_mask_cfg4(which, w.layers, w.n_kv, w.d)[layer].to(device)   # [H, d]
        sc = torch.where(m, 10.0, 1.0).to(torch.float32)

        def scale_fn(r0, r1, x):
            x.mul_(sc[r0:r1][:, None, :])
    return _randn_into(out, g, scale_fn)


def queries(w: Workload, device="cpu", copy: int = 0) -> torch.Tensor:
    """Query input [batch, n_q, d] N(0, 1) in the workload's input dtype."""
    g = generator(w.cfg, STREAM_Q, copy, device=device)
    q = torch.randn((w.batch, w.n_q, w.d), generator=g, dtype=torch.float32, device=device)
    return q.to(w.in_dtype)


def ragged_ctx_lens(batch: int, max_ctx: int, cfg: int = 0) -> torch.Tensor:
    """int32 context lengths in [1, max_ctx] for ragged-batch tests."""
    g = generator(cfg, STREAM_CTX)
    return torch.randint(1, max_ctx + 1, (batch,), generator=g, dtype=torch.int32)


def small(d=128, n_seq=2, n_tok=300, key_bits=3, val_bits=4, group=4, in_dtype=torch.float32,
          cfg=0) -> Workload:
    """A small ad-hoc workload for tests (sizes the oracle finishes in seconds)."""
    return Workload(cfg, f"small d{d} seq{n_seq} tok{n_tok}", d=d, batch=n_seq, n_kv=1,
                    group=group, n_tok=n_tok, key_bits=key_bits, val_bits=val_bits,
                    in_dtype=in_dtype)


def gaussian_rows(n: int, d: int, cfg: int, stream: int, device="cpu", dtype=torch.float32,
                  copy: int = 0) -> torch.Tensor:
    """n iid N(0, I_d) rows."""
    g = generator(cfg, stream, copy, device=device)
    return torch.randn((n, d), generator=g, dtype=torch.float32, device=device).to(dtype)


# --------------------------------------------------------------------------
# inner-product search over a coded database
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class SearchWorkload:
    cfg: int
    name: str
    d: int
    n_db: int            # database vectors (one coded sequence)
    n_q: int             # queries per scan (<= 32: the query heads of one KV head)
    k: int               # results per query
    key_bits: int        # b: (b-1) Lloyd-Max bits + 1 QJL bit
    in_dtype: torch.dtype

    @property
    def key_lm_bits(self) -> int:
        return self.key_bits - 1


SEARCH = SearchWorkload(6, "inner-product search: 32 queries over 1,048,576 coded vectors, d128, 4-bit codes, top 100",
                        d=128, n_db=1 << 20, n_q=32, k=100, key_bits=4, in_dtype=torch.bfloat16)


def search_database(w: SearchWorkload, device="cpu") -> torch.Tensor:
    """Database rows [1, n_db, d]: N(0, 1) with per-channel lognormal(0, 1)
    scales (the key recipe of the decode-layer workloads), in w.in_dtype."""
    sc = channel_scales(w.cfg, 1, w.d, 0).to(device)            # [1, d]
    out = torch.empty((1, w.n_db, w.d), dtype=w.in_dtype, device=device)

    def scale_fn(r0, r1, x):
        x.mul_(sc[None, :, :])
    return _randn_into(out, generator(w.cfg, STREAM_K, device=device), scale_fn, chunk_elems=1 << 24)


def search_queries(w: SearchWorkload, device="cpu") -> torch.Tensor:
    """Queries [n_q, d] N(0, 1) in w.in_dtype."""
    g = generator(w.cfg, STREAM_Q, device=device)
    return torch.randn((w.n_q, w.d), generator=g, dtype=torch.float32, device=device).to(w.in_dtype)
