"""Shared setup for the GPU parity tests: codecs from the seeded generators,
oracle-side encodings, and packing of oracle codes into the cache layout so
that logits and attention can be compared given identical codes."""
from __future__ import annotations

import sys

import numpy as np
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
import synthetic as syn


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class CodecPair:
    """GPU codec + the same parameters as numpy arrays for the oracle.

    The GPU side takes its codebook from tq_make_codebook, the oracle side
    from oracle.make_codebook; the two are checked equal elsewhere."""

    def __init__(self, d, lm_bits, is_key, signs, sketch=None, device="cuda", mse_only=False):
        self.d, self.lm_bits, self.is_key = d, lm_bits, is_key
        self.gpu = tq.Codec.make(d, lm_bits, is_key, signs, sketch, device=device, mse_only=mse_only)
        self.signs = np.asarray(signs, dtype=np.float64)
        self.sketch = None if sketch is None else np.asarray(sketch.numpy() if torch.is_tensor(sketch) else sketch,
                                                             dtype=np.float16)
        self.centroids, self.thresholds = O.make_codebook(d, lm_bits)

    def encode(self, x):
        return O.encode(np.asarray(x, dtype=np.float64), self.signs, self.centroids, self.thresholds,
                        self.sketch if self.is_key else None)


def key_codec(cfg, d, lm_bits, device="cuda"):
    s, S = syn.key_codec_randoms(cfg, d)
    return CodecPair(d, lm_bits, True, s.numpy(), S, device)


def mse_key_codec(cfg, d, lm_bits, device="cuda"):
    """MSE-only keys: the key codec's rotation and codebook, no sketch."""
    s, _ = syn.key_codec_randoms(cfg, d)
    return CodecPair(d, lm_bits, True, s.numpy(), None, device, mse_only=True)


def value_codec(cfg, d, lm_bits, device="cuda"):
    return CodecPair(d, lm_bits, False, syn.value_codec_randoms(cfg, d).numpy(), None, device)


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu").to(torch.float64).numpy()


def pack_keys_into(enc, lm_bits, codes: torch.Tensor, scal: torch.Tensor, seqs=None, t0=0):
    """Write oracle key codes [n, T, ...] into GPU cache tensors at sequences `seqs`, slots t0.."""
    rec = O.pack_key_codes(enc["idx"], enc["sigma"], lm_bits)                  # [n, T, R]
    sc = np.stack([enc["nhat"], enc["ghat"]], axis=-1).astype(np.float16)      # [n, T, 2]
    n, T = rec.shape[:2]
    idx = torch.arange(n) if seqs is None else torch.as_tensor(seqs)
    codes[idx.to(codes.device), t0:t0 + T] = torch.from_numpy(rec).to(codes.device)
    scal[idx.to(scal.device), t0:t0 + T] = torch.from_numpy(sc.view(np.int16)).to(scal.device)


def pack_mse_keys_into(enc, lm_bits, codes: torch.Tensor, scal: torch.Tensor):
    """Write oracle MSE-only key codes [n, T, ...] into GPU cache tensors at slots 0.."""
    rec = O.pack_mse_key_codes(enc["idx"], lm_bits)                           # [n, T, R]
    n, T = rec.shape[:2]
    codes[:n, :T] = torch.from_numpy(rec).to(codes.device)
    sc = np.asarray(enc["nhat"], dtype=np.float16)[..., None]                 # [n, T, 1]
    scal[:n, :T] = torch.from_numpy(sc.view(np.int16)).to(scal.device)


def pack_values_into(enc, lm_bits, codes: torch.Tensor, scal: torch.Tensor, seqs=None):
    """Write oracle value codes for tokens [0, T) of sequences `seqs`."""
    cap = scal.shape[1]
    words = O.pack_value_codes(enc["idx"], lm_bits, cap=cap)                  # [n, cap/32, w, d]
    n, T = enc["idx"].shape[:2]
    idx = torch.arange(n) if seqs is None else torch.as_tensor(seqs)
    codes[idx.to(codes.device)] = torch.from_numpy(words.view(np.int32)).to(codes.device)
    sc = np.zeros((n, cap), dtype=np.float16)
    sc[:, :T] = enc["nhat"]
    scal[idx.to(scal.device)] = torch.from_numpy(sc.view(np.int16)).to(scal.device)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (round to nearest even) -> float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
