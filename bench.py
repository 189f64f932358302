"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]
    python bench.py --pmc-pass      # eager launches for rocprofv3 --pmc runs

Headline workload: the Llama-3.1-8B-shaped decode layer (8 KV heads, 32
query heads, d = 128, batch 1, context 32768, 4-bit keys = 3 Lloyd-Max bits
+ 1 QJL bit, bf16 inputs with lognormal channel scales). One step encodes
the whole 32768-token key prefill of the layer into the packed cache and
then computes every q.k logit of the 32 query heads from the packed codes.
Inputs are resident in HBM before timing starts; each step uses a different
one of `--copies` independent input/cache sets (together > 1 GiB) so that
the 256 MB Infinity Cache cannot hold the working set.

The step's logit scan reads codes its own encode has just written; at 17.8
MB they are resident in the 256 MB Infinity Cache, so the step is partly
served from cache, and the per-kernel roofline figures (graphs of
back-to-back calls of one kind over the rotated copies) are the ones to
price against HBM.

Printed: one JSON line. `value` is q.k logits per second over whole steps
(encode + logit scan with its query preparation); the K timed steps (the
two library calls per step, each step on a fresh input copy) are captured
as one HIP graph and timed with HIP events around its replay. Per-kernel times come from graphs of
back-to-back calls of one kind (HIP events around their replays);
`roofline` prices the kernel with the largest share of the step against
HBM's 8 TB/s with the algorithmic bytes it must move (also against a
measured 4 GiB device copy), and carries the HBM bytes the counters saw
(FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size) from the
committed profile summary while the kernel sources are unchanged. The extras time the
fused decode attention on the batched (16 x 8192) and long-context
(4 x 131072) decode workloads and the full-cache encode of the 22-layer
TinyLlama-shaped prefill, the search scan (32 queries over 1,048,576
coded vectors, then the top 100 of each), the MSE-only key ablation (the
logit scan over 68 B TurboQuant records, 50 B and 66 B MSE-only records, and
the estimator's first term alone on the 68 B records: time, bytes and error
against exact q.k), and the
single-head workload (4096 fp32 keys, 16 queries; launch-latency bound,
absolute numbers only). Every scan's HBM fraction is also given against a
read-only stream measured on the same part (`tq_probe_read`, 4 GiB).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X datasheet
# VALU issue: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 instruction per 4 cycles
# per SIMD (16 lanes per cycle; the packed fp32 forms that double it are not
# used by this library)
VALU_PEAK = 256 * 4 * 2.4e9 / 4        # wave instructions per second (614.4 G)
MFMA_F16_PEAK = 2.5e15                 # dense fp16 FLOP/s
METRIC = "q·k logits/s + encode tokens/s over packed TurboQuant KV; % of HBM roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=16)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on the batched and long-context decode workloads in full (minutes) "
                         "and on the 22-layer encode's layer {0, 21} x row {0, 63} slices")
    ap.add_argument("--only", default="", help="comma list of extra sections: "
                                               "dec3,app3,pre3,k8v4,dec5,enc4,search,ablation,formulations,single")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="launch each timed kernel a few times eagerly, after a 1 GiB calibration copy, "
                         "for hardware-counter runs; prints no JSON line")
    return ap.parse_args()


def capture(torch, fns):
    """One HIP graph that replays the library calls `fns` in order. The calls
    are asynchronous launches on the current stream with preallocated
    outputs; they run once eagerly on the capture stream first."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_replays(torch, graphs, reps):
    """Seconds per replay, HIP events on the replay stream around `reps`
    rounds over `graphs`."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for g in graphs:
            g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * len(graphs))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the library sources that define each timed kernel
KERNEL_SOURCES = {
    "encode": ["tq_encode.inc.h", "tq_qjl.h", "tq_device.h", "tq_kernels.h", "tq_encode_d128.hip",
               "tq_encode_d64.hip"],
    "logits": ["tq_decode.inc.h", "tq_mfma.h", "tq_qjl.h", "tq_device.h", "tq_kernels.h", "tq_decode_d128.hip",
               "tq_decode_d64.hip"],
}
KERNEL_SOURCES["decode"] = KERNEL_SOURCES["logits"]
KERNEL_SOURCES["topk"] = ["tq_topk.hip", "tq_kernels.h"]


def kernel_sources_digest(kernel):
    """sha256 over the sources that define `kernel`, so that counter figures
    taken from an older build of it are recognised as stale."""
    import hashlib
    d = os.path.join(ROOT, "kv_cache_vector_rht_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[kernel]):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


# kernel -> committed rocprofv3 summary that holds its FETCH_SIZE / WRITE_SIZE
# figures ("traffic_bytes_per_launch" and "kernel_sources_sha256" lines)
PROFILE_OF = {
    "encode": "profiles/encode_kernel_llama8b_prefill32k.txt",
    "logits": "profiles/logits_kernel_llama8b_ctx32k.txt",
}


def profile_field(kernel, name):
    """A figure (first number of the line `name: ...`) from the committed
    counter summary of `kernel`, or None when there is none or the kernel's
    sources changed since it was taken."""
    path = os.path.join(ROOT, PROFILE_OF.get(kernel, ""))
    if not os.path.isfile(path):
        return None
    fields = {}
    for line in open(path):
        k, sep, v = line.partition(":")
        if sep:
            fields[k.strip()] = v.strip()
    try:
        if fields.get("kernel_sources_sha256") != kernel_sources_digest(kernel):
            return None
        return float(fields[name].split()[0])
    except (KeyError, ValueError, IndexError):
        return None


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary (None if stale)."""
    return profile_field(kernel, "traffic_bytes_per_launch")


def copy_probe(torch, gib=4, reps=5):
    """Device-to-device copy of `gib` GiB (torch's copy kernel): HBM bytes
    moved (read + write) per second, the bandwidth a plain stream reaches."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": 2 * n, "GBps": 2 * n / sec / 1e9, "what": f"{gib} GiB device-to-device copy, torch copy kernel"}


def read_probe(torch, tq, gib=4, reps=5):
    """Read-only stream over `gib` GiB (tq_probe_read): bytes per second a
    kernel that only reads gets from HBM on this part."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    tq.probe_read(src, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        tq.probe_read(src, sink)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src
    torch.cuda.empty_cache()
    return {"bytes": n, "GBps": n / sec / 1e9, "what": f"{gib} GiB read-and-reduce stream (tq_probe_read)"}


PROBE_GBPS = None   # set by main() once the read probe has run


def hbm(bytes_, seconds):
    return bytes_ / seconds / HBM_PEAK if seconds > 0 else 0.0


def of_probe(bytes_, seconds):
    """Fraction of the measured read-only stream (None before the probe ran)."""
    if PROBE_GBPS is None or seconds <= 0:
        return None
    return bytes_ / seconds / (PROBE_GBPS * 1e9)


# ------------------------------------------------------------------ workloads


def setup_codecs(torch, tq, syn, w, device):
    s, S = syn.key_codec_randoms(w.cfg, w.d)
    kc = tq.Codec.make(w.d, w.key_lm_bits, True, s, S, device=device)
    vc = None
    if w.val_bits:
        vc = tq.Codec.make(w.d, w.val_bits, False, syn.value_codec_randoms(w.cfg, w.d), device=device)
    return kc, vc, (s, S)


def main_decode_layer(args, torch, tq, syn):
    """Workload 2: encode prefill + logits, rotated over independent copies."""
    w = syn.WORKLOADS[2]
    dev = "cuda"
    kc, _, _ = setup_codecs(torch, tq, syn, w, dev)
    C = args.copies
    log(f"[main] generating {C} copies of {w.name}")
    xs = [syn.keys(w, device=dev, copy=c) for c in range(C)]
    qs = [syn.queries(w, device=dev, copy=c) for c in range(C)]
    caches = [tq.alloc_key_cache(w.n_seq, w.n_tok, kc) for _ in range(C)]
    outs = [torch.empty((w.batch, w.n_q, w.n_tok), dtype=torch.float32, device=dev) for _ in range(C)]
    ws = torch.empty(tq.logits_workspace(w.batch, w.n_kv, w.group, w.d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def enc(c):
        codes, scal = caches[c]
        return lambda: tq.encode_kv(kc, xs[c], codes, scal)

    def lgt(c):
        codes, scal = caches[c]
        return lambda: tq.logits(kc, qs[c], codes, scal, n_kv_heads=w.n_kv, group=w.group, n_keys=w.n_tok,
                                 out=outs[c], workspace=ws)

    # the warmup steps and the K timed steps each captured as one graph:
    # step i encodes copy i % C's prefill, then computes all its logits, so
    # the timed region holds exactly K whole steps and no host launch gaps
    # (one graph launch per step would leave the GPU idle between steps)
    def steps_graph(n):
        return capture(torch, [f for i in range(n) for f in (enc(i % C), lgt(i % C))]) if n > 0 else None
    warm_g = steps_graph(args.warmup)
    timed_g = steps_graph(args.steps)
    if warm_g is not None:
        warm_g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    timed_g.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total = t0.elapsed_time(t1) * 1e-3
    # per kernel: graphs of C back-to-back calls of one kind, over all copies
    enc_s = time_replays(torch, [capture(torch, [enc(c) for c in range(C)])], 3) / C
    lgt_s = time_replays(torch, [capture(torch, [lgt(c) for c in range(C)])], 3) / C
    ks = {"encode": {"avg_s": enc_s}, "logits": {"avg_s": lgt_s}}
    n_vec = w.n_vec
    rec = kc.record_bytes + 4
    bytes_encode = n_vec * (w.d * 2 + rec)                       # bf16 in, codes + scalars out
    bytes_logits = n_vec * rec + w.batch * w.n_q * w.n_tok * 4   # codes + scalars in, fp32 logits out
    logits_per_step = w.batch * w.n_q * w.n_tok
    kern = {
        "encode": dict(avg_us=ks["encode"]["avg_s"] * 1e6, bytes_per_launch=bytes_encode,
                       unit="key vectors", units_per_launch=n_vec,
                       tokens_per_s=n_vec / ks["encode"]["avg_s"],
                       hbm_frac=hbm(bytes_encode, ks["encode"]["avg_s"]),
                       mfma_flops_per_launch=n_vec * 2 * w.d * w.d),
        "logits": dict(avg_us=ks["logits"]["avg_s"] * 1e6, bytes_per_launch=bytes_logits,
                       unit="keys (x32 query heads)", units_per_launch=n_vec,
                       logits_per_s=logits_per_step / ks["logits"]["avg_s"],
                       hbm_frac=hbm(bytes_logits, ks["logits"]["avg_s"]),
                       frac_of_read_probe=of_probe(bytes_logits, ks["logits"]["avg_s"])),
    }
    return dict(w=w, total_s=total, wall_s=wall, steps=args.steps, kernels=kern,
                value=logits_per_step * args.steps / total, unit="logits/s",
                encode_tokens_per_s=n_vec * args.steps / total)


def decode_workload(torch, tq, syn, cfg, copies, steps):
    """Fused decode attention over a prefilled coded cache (workloads 3 and 5)."""
    w = syn.WORKLOADS[cfg]
    dev = "cuda"
    kc, vc, _ = setup_codecs(torch, tq, syn, w, dev)
    log(f"[dec{cfg}] encoding {copies} cache copies of {w.name}")
    caches = []
    for c in range(copies):
        kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
        vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc)
        x = syn.keys(w, device=dev, copy=c)
        tq.encode_kv(kc, x, kcodes, kscal)
        del x
        x = syn.values(w, device=dev, copy=c)
        tq.encode_kv(vc, x, vcodes, vscal)
        del x
        caches.append((kcodes, kscal, vcodes, vscal))
    qs = [syn.queries(w, device=dev, copy=c) for c in range(copies)]
    ctx = torch.full((w.batch,), w.n_tok, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.decode_attend_workspace(w.batch, w.n_kv, w.group, w.n_tok, w.d), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty((w.batch, w.n_q, w.d), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()

    def dec(c):
        kcodes, kscal, vcodes, vscal = caches[c]
        return lambda: tq.decode_attend(kc, vc, qs[c], kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=w.n_kv,
                                        group=w.group, max_ctx=w.n_tok, out=outs[c], workspace=ws,
                                        out_dtype=torch.bfloat16)

    g = capture(torch, [dec(c) for c in range(copies)])
    g.replay()
    avg = time_replays(torch, [g], max(1, steps // copies)) / copies
    th = w.n_seq * w.n_tok
    bytes_ = th * (kc.record_bytes + 4 + vc.lm_bits * w.d // 8 + 2) + w.batch * w.n_q * w.d * 4
    return dict(workload=w.name, avg_us=avg * 1e6, bytes_per_launch=bytes_, unit="token-heads",
                units_per_launch=th, attended_logits_per_s=w.batch * w.n_q * w.n_tok / avg,
                hbm_frac=hbm(bytes_, avg), frac_of_read_probe=of_probe(bytes_, avg), copies=copies)


def append_step_workload(torch, tq, syn, cfg, copies, steps):
    """A whole decoding step on workload 3: the new token's key and value
    encoded into slot n_tok - 1 of every sequence and attention over all
    n_tok tokens, as one fused call (tq_append_decode_attend) and as the
    two-call path (tq_encode_kv of the new key and value, tq_decode_attend)."""
    w = syn.WORKLOADS[cfg]
    dev = "cuda"
    kc, vc, _ = setup_codecs(torch, tq, syn, w, dev)
    log(f"[app{cfg}] encoding {copies} cache copies of {w.name}")
    caches, news = [], []
    for c in range(copies):
        kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
        vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc)
        x = syn.keys(w, device=dev, copy=c)
        tq.encode_kv(kc, x, kcodes, kscal)
        news.append([x[:, -1:].clone()])
        del x
        x = syn.values(w, device=dev, copy=c)
        tq.encode_kv(vc, x, vcodes, vscal)
        news[-1].append(x[:, -1:].clone())
        del x
        caches.append((kcodes, kscal, vcodes, vscal))
    qs = [syn.queries(w, device=dev, copy=c) for c in range(copies)]
    ctx = torch.full((w.batch,), w.n_tok, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.append_decode_attend_workspace(w.batch, w.n_kv, w.group, w.n_tok, w.d), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty((w.batch, w.n_q, w.d), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()

    def fused(c):
        kcodes, kscal, vcodes, vscal = caches[c]
        kn, vn = (t.view(w.batch, w.n_kv, w.d) for t in news[c])
        return lambda: tq.append_decode_attend(kc, vc, qs[c], kn, vn, kcodes, kscal, vcodes, vscal, ctx,
                                               n_kv_heads=w.n_kv, group=w.group, max_ctx=w.n_tok, out=outs[c],
                                               workspace=ws, out_dtype=torch.bfloat16)

    def two_calls(c):
        kcodes, kscal, vcodes, vscal = caches[c]
        kn, vn = news[c]

        def run():
            tq.encode_kv(kc, kn, kcodes, kscal, t0=w.n_tok - 1)
            tq.encode_kv(vc, vn, vcodes, vscal, t0=w.n_tok - 1)
            tq.decode_attend(kc, vc, qs[c], kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=w.n_kv, group=w.group,
                             max_ctx=w.n_tok, out=outs[c], workspace=ws, out_dtype=torch.bfloat16)
        return run

    res = {}
    for name, mk in (("fused_us", fused), ("two_calls_us", two_calls)):
        g = capture(torch, [mk(c) for c in range(copies)])
        g.replay()
        res[name] = time_replays(torch, [g], max(1, steps // copies)) / copies * 1e6
    th = w.n_seq * w.n_tok
    return dict(workload=w.name + ", new token appended each step", unit="token-heads", units_per_launch=th,
                attended_logits_per_s=w.batch * w.n_q * w.n_tok / (res["fused_us"] * 1e-6), copies=copies, **res)


def prefill_chunk_workload(torch, tq, syn, cfg, chunk, copies, steps):
    """Causal attention of a `chunk`-token prefill chunk at the end of the
    workload's context (positions n_tok - chunk .. n_tok - 1), over a cache
    that already holds the chunk."""
    w = syn.WORKLOADS[cfg]
    dev = "cuda"
    kc, vc, _ = setup_codecs(torch, tq, syn, w, dev)
    log(f"[pre{cfg}] encoding {copies} cache copies of {w.name}")
    caches = []
    for c in range(copies):
        kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
        vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc)
        x = syn.keys(w, device=dev, copy=c)
        tq.encode_kv(kc, x, kcodes, kscal)
        del x
        x = syn.values(w, device=dev, copy=c)
        tq.encode_kv(vc, x, vcodes, vscal)
        del x
        caches.append((kcodes, kscal, vcodes, vscal))
    g = torch.Generator(device=dev)
    g.manual_seed(cfg * 1000 + chunk)
    qs = [torch.randn((w.batch, chunk, w.n_q, w.d), generator=g, device=dev).to(w.in_dtype) for _ in range(copies)]
    pos0 = torch.full((w.batch,), w.n_tok - chunk, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.prefill_attend_workspace(w.batch, chunk, w.n_kv, w.group, w.n_tok, w.d), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty((w.batch, chunk, w.n_q, w.d), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()

    def pre(c):
        kcodes, kscal, vcodes, vscal = caches[c]
        return lambda: tq.prefill_attend(kc, vc, qs[c], kcodes, kscal, vcodes, vscal, pos0, n_kv_heads=w.n_kv,
                                         group=w.group, max_ctx=w.n_tok, out=outs[c], workspace=ws,
                                         out_dtype=torch.bfloat16)

    gr = capture(torch, [pre(c) for c in range(copies)])
    gr.replay()
    avg = time_replays(torch, [gr], max(1, steps // copies)) / copies
    pairs = w.batch * w.n_q * sum(w.n_tok - chunk + i + 1 for i in range(chunk))
    heads = chunk * w.group                               # (position, head) pairs per KV head
    scans = (heads + 63) // 64 if heads > 8 else (heads + 7) // 8   # passes over each context
    nbytes = w.n_seq * w.n_tok * ((kc.record_bytes + 4) + (w.val_bits * w.d // 8 + 2))
    return dict(workload=f"{w.name}, causal prefill chunk of {chunk} tokens at the end of the context",
                avg_us=avg * 1e6, attended_logits_per_s=pairs / avg, chunk=chunk, pairs_per_kv_head=heads,
                context_scans=scans, cache_bytes=nbytes, hbm_frac=hbm(nbytes * scans, avg),
                frac_of_read_probe=of_probe(nbytes * scans, avg), copies=copies)


def k8v4_ablation(torch, tq, syn, copies, steps):
    """Workload 3 with fp8 keys (the k8v4 shape) beside its own TurboQuant
    keys (3-bit, the k3v4 shape), both with the same 4-bit values: decode
    time, bytes per token-head, and the attention output's relative RMS
    error against exact attention over the unquantized bf16 keys and values
    (first two batch rows, all heads)."""
    w = syn.WORKLOADS[3]
    dev = "cuda"
    kc, vc, _ = setup_codecs(torch, tq, syn, w, dev)
    log(f"[k8v4] encoding {copies} cache copies of {w.name} (TurboQuant and fp8 keys)")
    tqc, k8c, exact = [], [], None
    for c in range(copies):
        kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
        vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc)
        k8 = tq.alloc_fp8_key_cache(w.n_seq, w.n_tok, w.d)
        xk = syn.keys(w, device=dev, copy=c)
        tq.encode_kv(kc, xk, kcodes, kscal)
        tq.encode_fp8_keys(xk, k8)
        xv = syn.values(w, device=dev, copy=c)
        tq.encode_kv(vc, xv, vcodes, vscal)
        if c == 0:
            exact = (xk[:2 * w.n_kv].float(), xv[:2 * w.n_kv].float())
        del xk, xv
        tqc.append((kcodes, kscal, vcodes, vscal))
        k8c.append(k8)
    qs = [syn.queries(w, device=dev, copy=c) for c in range(copies)]
    ctx = torch.full((w.batch,), w.n_tok, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.decode_attend_workspace(w.batch, w.n_kv, w.group, w.n_tok, w.d), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty((w.batch, w.n_q, w.d), dtype=torch.float32, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()

    def dec_tq(c):
        kcodes, kscal, vcodes, vscal = tqc[c]
        return lambda: tq.decode_attend(kc, vc, qs[c], kcodes, kscal, vcodes, vscal, ctx, n_kv_heads=w.n_kv,
                                        group=w.group, max_ctx=w.n_tok, out=outs[c], workspace=ws)

    def dec_k8(c):
        _, _, vcodes, vscal = tqc[c]
        return lambda: tq.decode_attend_k8(vc, qs[c], k8c[c], vcodes, vscal, ctx, n_kv_heads=w.n_kv,
                                           group=w.group, max_ctx=w.n_tok, out=outs[c], workspace=ws)

    res = {}
    scale = 1.0 / math.sqrt(w.d)
    K, V = exact
    q0 = qs[0][:2].float().reshape(2, w.n_kv, w.group, w.d)
    Kb, Vb = K.reshape(2, w.n_kv, w.n_tok, w.d), V.reshape(2, w.n_kv, w.n_tok, w.d)
    ref = torch.softmax(torch.matmul(q0, Kb.transpose(-1, -2).contiguous()) * scale, dim=-1)
    ref = torch.matmul(ref, Vb).reshape(2, w.n_q, w.d)
    for name, mk, key_bytes in (("k3v4", dec_tq, kc.record_bytes + 4), ("k8v4", dec_k8, w.d)):
        mk(0)()
        torch.cuda.synchronize()
        err = (outs[0][:2] - ref).pow(2).mean().sqrt() / ref.pow(2).mean().sqrt()
        g = capture(torch, [mk(c) for c in range(copies)])
        g.replay()
        t = time_replays(torch, [g], max(1, steps // copies)) / copies
        bytes_ = w.n_seq * w.n_tok * (key_bytes + vc.lm_bits * w.d // 8 + 2) + w.batch * w.n_q * w.d * 4
        res[name] = dict(avg_us=t * 1e6, bytes_per_token_head=key_bytes + vc.lm_bits * w.d // 8 + 2,
                         hbm_frac=hbm(bytes_, t), frac_of_read_probe=of_probe(bytes_, t),
                         rel_rms_error_vs_exact=float(err))
        del g
    return dict(workload=w.name, copies=copies, **res)


def encode_full_cache(torch, tq, syn, steps):
    """Workload 4: encode every K and V vector of the 22-layer prefill."""
    w = syn.WORKLOADS[4]
    dev = "cuda"
    kc, vc, _ = setup_codecs(torch, tq, syn, w, dev)
    log(f"[enc4] generating inputs for {w.name} ({w.n_vec * 2} vectors)")
    xk = syn.keys(w, device=dev)
    xv = syn.values(w, device=dev)
    kcodes, kscal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
    vcodes, vscal = tq.alloc_value_cache(w.n_seq, w.n_tok, vc)
    torch.cuda.synchronize()

    gk = capture(torch, [lambda: tq.encode_kv(kc, xk, kcodes, kscal)])
    gv = capture(torch, [lambda: tq.encode_kv(vc, xv, vcodes, vscal)])
    tk = time_replays(torch, [gk], steps)
    tv = time_replays(torch, [gv], steps)
    bk = w.n_vec * (w.d * 2 + kc.record_bytes + 4)
    bv = w.n_vec * (w.d * 2 + vc.lm_bits * w.d // 8 + 2)
    out = dict(workload=w.name, keys_avg_us=tk * 1e6, values_avg_us=tv * 1e6,
               tokens_per_s=(2 * w.n_vec) / (tk + tv), bytes_per_pass=bk + bv,
               hbm_frac=hbm(bk + bv, tk + tv), keys_hbm_frac=hbm(bk, tk), values_hbm_frac=hbm(bv, tv))
    del kcodes, kscal, vcodes, vscal, gk, gv
    torch.cuda.empty_cache()
    # fractional rates: per-layer widths from tq_rate_plan, one cache per layer
    per_layer = w.batch * w.n_kv
    s, S = syn.key_codec_randoms(w.cfg, w.d)
    sv = syn.value_codec_randoms(w.cfg, w.d)
    out["fractional"] = []
    for rate in (2.5, 3.5):
        kplan, vplan = tq.rate_plan(rate, w.layers, True), tq.rate_plan(rate, w.layers, False)
        calls, nbytes = [], 0
        for layer in range(w.layers):
            kcl = tq.Codec.make(w.d, kplan[layer], True, s, S, device=dev)
            vcl = tq.Codec.make(w.d, vplan[layer], False, sv, device=dev)
            kc_l, ks_l = tq.alloc_key_cache(per_layer, w.n_tok, kcl)
            vc_l, vs_l = tq.alloc_value_cache(per_layer, w.n_tok, vcl)
            sl = slice(layer * per_layer, (layer + 1) * per_layer)
            calls.append(lambda a=kcl, x=xk[sl], c=kc_l, sc=ks_l: tq.encode_kv(a, x, c, sc))
            calls.append(lambda a=vcl, x=xv[sl], c=vc_l, sc=vs_l: tq.encode_kv(a, x, c, sc))
            nbytes += per_layer * w.n_tok * (2 * w.d * 2 + kcl.record_bytes + 4 + vcl.lm_bits * w.d // 8 + 2)
        gf = capture(torch, calls)
        tf = time_replays(torch, [gf], steps)
        out["fractional"].append(dict(
            bits_per_channel=rate, key_lm_bits=kplan, value_lm_bits=vplan,
            key_bits_achieved=sum(b + 1 for b in kplan) / w.layers, value_bits_achieved=sum(vplan) / w.layers,
            avg_us=tf * 1e6, tokens_per_s=(2 * w.n_vec) / tf, bytes_per_pass=nbytes, hbm_frac=hbm(nbytes, tf)))
        del calls, gf
        torch.cuda.empty_cache()
    del xk, xv
    return out


def search_workload(torch, tq, syn, copies, steps):
    """Inner-product search: 32 queries scanned over 1,048,576 coded vectors
    (the logit scan with the queries as the query heads of one KV head),
    then the top 100 per query; `copies` independent databases and score
    buffers rotated so that the working set exceeds the Infinity Cache."""
    w = syn.SEARCH
    dev = "cuda"
    s, S = syn.key_codec_randoms(w.cfg, w.d)
    kc = tq.Codec.make(w.d, w.key_lm_bits, True, s, S, device=dev)
    log(f"[search] encoding {copies} database copies of {w.name}")
    dbs = []
    for c in range(copies):
        codes, scal = tq.alloc_key_cache(1, w.n_db, kc)
        x = syn.search_database(w, device=dev)
        if c:
            x = x[:, torch.randperm(w.n_db, device=dev)]       # another database of the same law
        tq.encode_kv(kc, x, codes, scal)
        del x
        dbs.append((codes, scal))
    q = syn.search_queries(w, device=dev)
    scores = [torch.empty((1, w.n_q, w.n_db), dtype=torch.float32, device=dev) for _ in range(copies)]
    ws = torch.empty(tq.topk_workspace(w.n_q, w.n_db, w.k), dtype=torch.uint8, device=dev)
    vals = torch.empty((w.n_q, w.k), dtype=torch.float32, device=dev)
    idx = torch.empty((w.n_q, w.k), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def scan(c):
        codes, scal = dbs[c]
        return lambda: tq.logits(kc, q.unsqueeze(0), codes, scal, n_kv_heads=1, group=w.n_q, n_keys=w.n_db,
                                 out=scores[c])

    def rank(c):
        return lambda: tq.lib.tq_topk(tq._ptr(scores[c]), w.n_q, w.n_db, w.n_db, w.k, tq._ptr(vals), tq._ptr(idx),
                                      tq._ptr(ws), ws.numel(), tq._stream(None))

    g_all = capture(torch, [f for c in range(copies) for f in (scan(c), rank(c))])
    g_scan = capture(torch, [scan(c) for c in range(copies)])
    g_rank = capture(torch, [rank(c) for c in range(copies)])
    g_all.replay()
    reps = max(1, steps // copies)
    t_all = time_replays(torch, [g_all], reps) / copies
    t_scan = time_replays(torch, [g_scan], reps) / copies
    t_rank = time_replays(torch, [g_rank], reps) / copies
    rec = kc.record_bytes + 4
    b_scan = w.n_db * rec + w.n_q * w.n_db * 4          # coded database in, scores out
    b_rank = w.n_q * w.n_db * 4                         # scores in (candidates are a few MB)
    return dict(workload=w.name, search_avg_us=t_all * 1e6, scan_avg_us=t_scan * 1e6, topk_avg_us=t_rank * 1e6,
                scores_per_s=w.n_q * w.n_db / t_all, queries_per_s=w.n_q / t_all,
                scan_bytes_per_launch=b_scan, scan_hbm_frac=hbm(b_scan, t_scan),
                scan_frac_of_read_probe=of_probe(b_scan, t_scan),
                topk_bytes_per_launch=b_rank, topk_hbm_frac=hbm(b_rank, t_rank),
                topk_frac_of_read_probe=of_probe(b_rank, t_rank), k=w.k, copies=copies)


def mse_keys_ablation(torch, tq, syn, copies, steps):
    """The MSE-only key ablation on the decode-layer workload (8 KV / 32 Q
    heads, 32768 keys, bf16 keys with lognormal channel scales), one logit
    scan per key cache format, each over `copies` cache copies rotated so
    that the working set exceeds the Infinity Cache:
      tq_b4        4-bit TurboQuant keys (3 Lloyd-Max bits + QJL), 68 B/key
      mse_b3       MSE-only keys, 3 Lloyd-Max bits (codec is_key = 2), 50 B/key
      mse_b4       MSE-only keys, 4 Lloyd-Max bits, 66 B/key (the same bits
                   per channel as tq_b4)
      tq_b4_first_term  the estimator's first term alone over the 68 B records
                   (tq_logits_mse: the bias on identical codes)
    For each: time per call, algorithmic bytes, HBM fractions, and the logits
    against the exact q.k of the unquantized keys: least-squares slope (the
    shrinkage the QJL bit removes) and RMS error relative to the exact
    logits' RMS."""
    w = syn.WORKLOADS[2]
    dev = "cuda"
    s, S = syn.key_codec_randoms(w.cfg, w.d)
    codecs = {
        "tq_b4": (tq.Codec.make(w.d, w.key_lm_bits, True, s, S, device=dev), False),
        "mse_b3": (tq.Codec.make(w.d, w.key_lm_bits, True, s, device=dev, mse_only=True), False),
        "mse_b4": (tq.Codec.make(w.d, w.key_lm_bits + 1, True, s, device=dev, mse_only=True), False),
    }
    codecs["tq_b4_first_term"] = (codecs["tq_b4"][0], True)
    x = syn.keys(w, device=dev)
    q = syn.queries(w, device=dev)
    log(f"[ablation] encoding {copies} copies of {w.name} in three key formats")
    caches = {}
    for name in ("tq_b4", "mse_b3", "mse_b4"):
        kc = codecs[name][0]
        caches[name] = []
        for _ in range(copies):
            codes, scal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
            tq.encode_kv(kc, x, codes, scal)
            caches[name].append((codes, scal))
    caches["tq_b4_first_term"] = caches["tq_b4"]
    outs = [torch.empty((w.batch, w.n_q, w.n_tok), dtype=torch.float32, device=dev) for _ in range(copies)]
    # exact logits: query head h against the keys of KV head h // group
    qf = q[0].float().view(w.n_kv, w.group, w.d)
    ex = torch.bmm(qf, x.float().transpose(1, 2).contiguous()).view(1, w.n_q, w.n_tok).double()
    torch.cuda.synchronize()
    res = dict(workload=w.name, copies=copies)
    for name, (kc, first_term) in codecs.items():
        def call(c, kc=kc, first_term=first_term, name=name):
            codes, scal = caches[name][c]
            return lambda: tq.logits(kc, q, codes, scal, n_kv_heads=w.n_kv, group=w.group, n_keys=w.n_tok,
                                     out=outs[c], mse_only=first_term)
        t = time_replays(torch, [capture(torch, [call(c) for c in range(copies)])], max(1, steps // copies)) / copies
        rec = kc.record_bytes + 2 * kc.key_scalars
        nbytes = w.n_vec * rec + w.batch * w.n_q * w.n_tok * 4
        call(0)()
        e = outs[0].double()
        res[name] = dict(avg_us=t * 1e6, record_bytes=rec, bytes_per_call=nbytes, hbm_frac=hbm(nbytes, t),
                         frac_of_read_probe=of_probe(nbytes, t), logits_per_s=w.batch * w.n_q * w.n_tok / t,
                         slope=float((e * ex).sum() / (ex * ex).sum()),
                         rel_rms_err=float(((e - ex) ** 2).mean().sqrt() / (ex ** 2).mean().sqrt()))
    del x, caches
    torch.cuda.empty_cache()
    return res


def scan_formulations(torch, tq, syn, copies, steps):
    """The logit scan of the decode-layer workload (8 KV / 32 Q heads, 32768
    4-bit keys) in its two formulations, over `copies` rotated cache copies:
    the bit planes on the matrix cores (tq_logits, each block preparing its
    queries; and tq_prepare_queries + tq_logits_prepared, the preparation in
    a launch of its own) and the codebook in LDS (tq_logits_table: nibble
    tables per head, one lane per key, after a preparation launch). Times per
    call; the counters that split them per kernel come from rocprofv3."""
    w = syn.WORKLOADS[2]
    dev = "cuda"
    kc, _, _ = setup_codecs(torch, tq, syn, w, dev)
    x = syn.keys(w, device=dev)
    q = syn.queries(w, device=dev)
    caches = []
    for _ in range(copies):
        codes, scal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
        tq.encode_kv(kc, x, codes, scal)
        caches.append((codes, scal))
    del x
    outs = [torch.empty((w.batch, w.n_q, w.n_tok), dtype=torch.float32, device=dev) for _ in range(copies)]
    prep = tq.prepare_queries(kc, q, n_kv_heads=w.n_kv, group=w.group)
    tws = torch.empty(max(256, int(tq.lib.tq_logits_table_workspace(w.batch, w.n_kv, w.group, w.d))),
                      dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    calls = {
        "matrix_cores": lambda c: (lambda: tq.logits(kc, q, caches[c][0], caches[c][1], n_kv_heads=w.n_kv,
                                                     group=w.group, n_keys=w.n_tok, out=outs[c])),
        "matrix_cores_prepared": lambda c: (lambda: (tq.prepare_queries(kc, q, n_kv_heads=w.n_kv, group=w.group,
                                                                        prepared=prep),
                                                     tq.logits_prepared(kc, prep, w.batch, caches[c][0], caches[c][1],
                                                                        n_kv_heads=w.n_kv, group=w.group,
                                                                        n_keys=w.n_tok, out=outs[c]))),
        "lds_table": lambda c: (lambda: tq.logits_table(kc, q, caches[c][0], caches[c][1], n_kv_heads=w.n_kv,
                                                        group=w.group, n_keys=w.n_tok, out=outs[c], workspace=tws)),
    }
    nbytes = w.n_vec * (kc.record_bytes + 4) + w.batch * w.n_q * w.n_tok * 4
    res = dict(workload=w.name, copies=copies, bytes_per_call=nbytes)
    ref = None
    for name, mk in calls.items():
        t = time_replays(torch, [capture(torch, [mk(c) for c in range(copies)])], max(1, steps // copies)) / copies
        mk(0)()
        torch.cuda.synchronize()
        if ref is None:
            ref = outs[0].clone()
        err = float((outs[0] - ref).abs().max() / ref.abs().max())
        res[name] = dict(avg_us=t * 1e6, hbm_frac=hbm(nbytes, t), frac_of_read_probe=of_probe(nbytes, t),
                         max_rel_diff_vs_matrix_cores=err)
    del caches
    torch.cuda.empty_cache()
    return res


def single_head_workload(torch, tq, syn, reps=50):
    """The single-head workload: encode of 4096 fp32 keys (d 128, 2 Lloyd-Max
    bits + QJL) and all 16 x 4096 logits. Its 2.8 MB fit any cache and a call
    is a few microseconds of launch latency, so the figures are absolute
    rates (graphs of back-to-back calls, HIP events), not HBM fractions."""
    w = syn.WORKLOADS[1]
    dev = "cuda"
    kc, _, _ = setup_codecs(torch, tq, syn, w, dev)
    x = syn.keys(w, device=dev)
    q = syn.queries(w, device=dev)
    codes, scal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
    out = torch.empty((w.batch, w.n_q, w.n_tok), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    enc = lambda: tq.encode_kv(kc, x, codes, scal)
    lgt = lambda: tq.logits(kc, q, codes, scal, n_kv_heads=w.n_kv, group=w.group, n_keys=w.n_tok, out=out)
    n = 16
    t_enc = time_replays(torch, [capture(torch, [enc] * n)], reps) / n
    t_lgt = time_replays(torch, [capture(torch, [lgt] * n)], reps) / n
    t_step = time_replays(torch, [capture(torch, [f for _ in range(n) for f in (enc, lgt)])], reps) / n
    return dict(workload=w.name, encode_us=t_enc * 1e6, logits_us=t_lgt * 1e6, step_us=t_step * 1e6,
                encode_tokens_per_s=w.n_vec / t_enc, logits_per_s=w.n_q * w.n_tok / t_lgt,
                step_logits_per_s=w.n_q * w.n_tok / t_step)


# ------------------------------------------------------------------ CPU baseline


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def _oracle_decode(O, np, syn, torch, w, kvs, q, lens, s, S, sv, ck, tk, cv, tv):
    """Encode a sample's keys and values with the oracle, then its decode attention."""
    k, v = kvs
    ek = O.encode(k, s, ck, tk, S)
    ev = O.encode(v, sv, cv, tv)
    return O.decode_attend(q, s, ck, S, ek["idx"], ek["sigma"], ek["nhat"], ek["ghat"], sv, cv, ev["idx"],
                           ev["nhat"], lens, 1.0 / math.sqrt(w.d), w.group)


def cpu_baseline(w, syn, torch, full=False):
    """The oracle (numpy fp64) on the host cores.

    Headline (`value`): the decode-layer step (encode of the 262144-key
    prefill + all 1,048,576 logits), median of 3 runs with every thread
    numpy's BLAS has. Beside it: the single-head workload at 1 thread and at
    all threads (median of 3), and one run per sample of the batched-decode
    and long-context workloads (encode of the sample's K and V + its decode
    attention) and of the 22-layer encode, each scaled linearly to its
    whole workload and labelled extrapolated unless it is the whole workload
    (`full`: the two decode workloads in full, chunked by batch row, and the
    22-layer encode on layers {0, 21} x batch rows {0, 63})."""
    import dataclasses
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_limits
    threads = blas_threads()

    def med3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[1]

    # headline: the decode-layer step, all 8 KV heads
    s, S = syn.key_codec_randoms(w.cfg, w.d)
    sn, Sn = s.numpy(), S.numpy()
    c, t = O.make_codebook(w.d, w.key_lm_bits)
    ws = dataclasses.replace(w, batch=1)
    x = syn.keys(ws).double().numpy()          # [n_kv, n_tok, d]
    q = syn.queries(ws).double().numpy()[0]    # [n_q, d]
    encs = {}

    def enc_all():
        encs["e"] = [O.encode(x[h], sn, c, t, Sn) for h in range(w.n_kv)]

    def lg_all():
        for h, e in enumerate(encs["e"]):
            O.key_logits(q[h * w.group:(h + 1) * w.group], sn, c, Sn, e["idx"], e["sigma"], e["nhat"], e["ghat"])
    enc_s = med3(enc_all)
    lg_s = med3(lg_all)
    step_s = enc_s + lg_s
    del x, encs
    out = {"value": w.batch * w.n_q * w.n_tok / step_s, "unit": "logits/s", "cores": int(threads), "kind": "oracle",
           "sample": f"numpy fp64 oracle, median of 3 runs, {threads} BLAS threads: the whole decode-layer step "
                     f"(encode of {w.n_vec} keys + {w.batch * w.n_q * w.n_tok} logits)",
           "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": threads,
           "step_s": step_s, "encode_keys_per_s": w.n_vec / enc_s, "logits_per_s": w.batch * w.n_q * w.n_tok / lg_s}

    # the single-head workload, 1 thread and all threads
    w1 = syn.WORKLOADS[1]
    s1, S1 = syn.key_codec_randoms(w1.cfg, w1.d)
    c1, t1 = O.make_codebook(w1.d, w1.key_lm_bits)
    x1 = syn.keys(w1).double().numpy()[0]
    q1 = syn.queries(w1).double().numpy()[0]

    def step1():
        e = O.encode(x1, s1.numpy(), c1, t1, S1.numpy())
        O.key_logits(q1, s1.numpy(), c1, S1.numpy(), e["idx"], e["sigma"], e["nhat"], e["ghat"])
    single = {}
    for label, lim in (("1_thread", 1), ("all_threads", threads)):
        with threadpool_limits(limits=lim):
            sec = med3(step1)
        single[label] = {"threads": lim, "step_s": sec, "encode_tokens_per_s_incl_logits": w1.n_vec / sec,
                         "logits_per_s": w1.n_q * w1.n_tok / sec}
    out["single_head"] = single

    # decode-attention workloads: samples (or, full, every batch row)
    work = {}
    for cfg in (3, 5):
        wc = syn.WORKLOADS[cfg]
        sk, Sk = syn.key_codec_randoms(cfg, wc.d)
        sv = syn.value_codec_randoms(cfg, wc.d).numpy()
        ck, tk = O.make_codebook(wc.d, wc.key_lm_bits)
        cv, tv = O.make_codebook(wc.d, wc.val_bits)
        rows = list(range(wc.batch)) if full else [0]
        n_kv_sample = wc.n_kv if (full or cfg == 3) else 1
        ws1 = dataclasses.replace(wc, batch=1, n_kv=n_kv_sample)
        qa = syn.queries(wc).double().numpy()
        sec = 0.0
        for b in rows:
            kv = (syn.kv_slice(ws1, 0, 0, b).double().numpy(), syn.kv_slice(ws1, 1, 0, b).double().numpy())
            qb = qa[b:b + 1, :n_kv_sample * wc.group]
            t0 = time.perf_counter()
            _oracle_decode(O, np, syn, torch, ws1, kv, qb, [wc.n_tok], sk.numpy(), Sk.numpy(), sv, ck, tk, cv, tv)
            sec += time.perf_counter() - t0
            del kv
        done = len(rows) * n_kv_sample
        whole = wc.batch * wc.n_kv
        work[f"decode_attend_cfg{cfg}"] = {
            "workload": wc.name, "sample": f"{len(rows)} batch row(s) x {n_kv_sample} KV head(s) of "
                                           f"{wc.batch} x {wc.n_kv}: encode of K and V + decode attention",
            "sample_s": sec, "extrapolated": done < whole, "whole_s": sec * whole / done,
            "attended_logits_per_s": wc.batch * wc.n_q * wc.n_tok / (sec * whole / done)}
    # 22-layer encode: (layer, batch row) slices of 32 heads x 4096 tokens, K and V
    w4 = syn.WORKLOADS[4]
    sk4, Sk4 = syn.key_codec_randoms(4, w4.d)
    sv4 = syn.value_codec_randoms(4, w4.d).numpy()
    ck4, tk4 = O.make_codebook(w4.d, w4.key_lm_bits)
    cv4, tv4 = O.make_codebook(w4.d, w4.val_bits)
    slices = [(0, 0), (0, 63), (21, 0), (21, 63)] if full else [(0, 0)]
    sec = 0.0
    for layer, b in slices:
        k = syn.kv_slice(w4, 0, layer, b).double().numpy()
        v = syn.kv_slice(w4, 1, layer, b).double().numpy()
        t0 = time.perf_counter()
        O.encode(k, sk4.numpy(), ck4, tk4, Sk4.numpy())
        O.encode(v, sv4, cv4, tv4)
        sec += time.perf_counter() - t0
        del k, v
    per_vec = sec / (2 * len(slices) * w4.n_kv * w4.n_tok)
    work["encode_cfg4"] = {"workload": w4.name, "sample": f"(layer, batch row) slices {slices}: 32 heads x 4096 "
                                                          f"tokens each, K and V (same-law stand-in draws)",
                           "sample_s": sec, "extrapolated": True, "whole_s": per_vec * 2 * w4.n_vec,
                           "vectors_per_s": 1.0 / per_vec}
    out["workloads"] = work
    return out


# ------------------------------------------------------------------ counters


def pmc_pass(torch, tq, syn):
    """Launches for hardware-counter runs: a 1 GiB device copy (the
    calibration kernel: 1 GiB read, 1 GiB written), each kernel of the
    headline step three times eagerly, the prepared and LDS-table logit
    scans, then the decode-attention workloads, the prefill chunk and the
    fused append step (one cache copy each) and the search scan (one
    database)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    w = syn.WORKLOADS[2]
    kc, _, _ = setup_codecs(torch, tq, syn, w, "cuda")
    x = syn.keys(w, device="cuda")
    q = syn.queries(w, device="cuda")
    codes, scal = tq.alloc_key_cache(w.n_seq, w.n_tok, kc)
    out = torch.empty((w.batch, w.n_q, w.n_tok), dtype=torch.float32, device="cuda")
    for _ in range(3):
        tq.encode_kv(kc, x, codes, scal)
    for _ in range(3):
        tq.logits(kc, q, codes, scal, n_kv_heads=w.n_kv, group=w.group, n_keys=w.n_tok, out=out)
    # the two formulations of the scan with their preparation launches
    prep = tq.prepare_queries(kc, q, n_kv_heads=w.n_kv, group=w.group)
    for _ in range(3):
        tq.prepare_queries(kc, q, n_kv_heads=w.n_kv, group=w.group, prepared=prep)
        tq.logits_prepared(kc, prep, w.batch, codes, scal, n_kv_heads=w.n_kv, group=w.group, n_keys=w.n_tok, out=out)
        tq.logits_table(kc, q, codes, scal, n_kv_heads=w.n_kv, group=w.group, n_keys=w.n_tok, out=out)
    torch.cuda.synchronize()
    del x, q, codes, scal, out, prep
    torch.cuda.empty_cache()
    for cfg in (3, 5):
        decode_workload(torch, tq, syn, cfg, copies=1, steps=3)
        torch.cuda.empty_cache()
    prefill_chunk_workload(torch, tq, syn, 3, chunk=16, copies=1, steps=2)
    torch.cuda.empty_cache()
    append_step_workload(torch, tq, syn, 3, copies=1, steps=2)
    torch.cuda.empty_cache()
    search_workload(torch, tq, syn, copies=1, steps=2)
    torch.cuda.empty_cache()
    log("[pmc] done: copy 1 GiB x2, encode x3, logits x3, prepared and LDS-table scans x3, decode attention of "
        "workloads 3 and 5, the 16-token prefill chunk and the fused append step of workload 3, search scan")


# ------------------------------------------------------------------ main


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the codec path has no "
                                   "multi-GPU component (shard batch x KV heads across GPUs instead)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)
    import torch
    import kv_cache_vector_rht_amd as tq
    import synthetic as syn
    tq.load()
    torch.cuda.set_device(0)
    only = set(filter(None, args.only.split(",")))
    if args.pmc_pass:
        pmc_pass(torch, tq, syn)
        return

    global PROBE_GBPS
    log("[probe] read-only stream")
    rp = read_probe(torch, tq)
    PROBE_GBPS = rp["GBps"]
    res = main_decode_layer(args, torch, tq, syn)
    w = res["w"]
    kern = res["kernels"]
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    kd = kern[dom]
    log("[copy] device copy bandwidth probe")
    cp = copy_probe(torch)
    t_dom = kd["avg_us"] * 1e-6
    # the roofs of the dominant kernel: HBM (algorithmic bytes), the matrix
    # cores (algorithmic flops of its dense products, fp16 peak) and vector
    # ALU issue, "alu" (wave instructions the counters saw per launch, while the
    # committed counter summary is current); the binding roof is the one the
    # kernel comes closest to
    roofs = {"hbm": {"achieved": kd["bytes_per_launch"] / t_dom / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": kd["hbm_frac"], "per_unit": kd["bytes_per_launch"] / kd["units_per_launch"],
                     "per_unit_what": "algorithmic bytes per " + kd["unit"].rstrip("s").split(" (")[0]}}
    if kd.get("mfma_flops_per_launch"):
        f = kd["mfma_flops_per_launch"] / t_dom
        roofs["mfma"] = {"achieved": f / 1e12, "peak": MFMA_F16_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": f / MFMA_F16_PEAK,
                         "per_unit": kd["mfma_flops_per_launch"] / kd["units_per_launch"],
                         "per_unit_what": "algorithmic flops per key (the d x d QJL projection)"}
    valu = profile_field(dom, "valu_instructions_per_launch")
    if valu:
        roofs["alu"] = {"achieved": valu / t_dom / 1e9, "peak": VALU_PEAK / 1e9, "unit": "G wave-instructions/s",
                        "frac": valu / t_dom / VALU_PEAK, "per_unit": valu / kd["units_per_launch"],
                        "per_unit_what": "VALU wave instructions per key (counter SQ_INSTS_VALU)"}
    bound = max(roofs, key=lambda r: roofs[r]["frac"])
    rb = roofs[bound]
    roof = {"kernel": dom, "bound": bound, "achieved": rb["achieved"], "peak": rb["peak"], "unit": rb["unit"],
            "frac": rb["frac"], "traffic": measured_traffic(dom),
            "bytes_per_unit": kd["bytes_per_launch"] / kd["units_per_launch"],
            "units_per_launch": kd["units_per_launch"], "roofs": roofs,
            "copy_probe_GBps": cp["GBps"], "read_probe_GBps": rp["GBps"],
            "hbm_frac_of_copy": roofs["hbm"]["achieved"] / cp["GBps"],
            "hbm_frac_of_read_probe": roofs["hbm"]["achieved"] / rp["GBps"]}
    extras = {}
    if not args.no_extras:
        if not only or "single" in only:
            extras["single_head"] = single_head_workload(torch, tq, syn)
        torch.cuda.empty_cache()
        if not only or "dec3" in only:
            extras["decode_attend_batched"] = decode_workload(torch, tq, syn, 3, copies=9, steps=20)
        torch.cuda.empty_cache()
        if not only or "app3" in only:
            extras["append_decode_step"] = append_step_workload(torch, tq, syn, 3, copies=9, steps=20)
        torch.cuda.empty_cache()
        if not only or "pre3" in only:
            extras["prefill_chunk"] = prefill_chunk_workload(torch, tq, syn, 3, chunk=16, copies=4, steps=8)
        torch.cuda.empty_cache()
        if not only or "k8v4" in only:
            extras["k8v4_ablation"] = k8v4_ablation(torch, tq, syn, copies=4, steps=20)
        torch.cuda.empty_cache()
        if not only or "dec5" in only:
            extras["decode_attend_long_context"] = decode_workload(torch, tq, syn, 5, copies=2, steps=10)
        torch.cuda.empty_cache()
        if not only or "enc4" in only:
            extras["encode_full_cache"] = encode_full_cache(torch, tq, syn, steps=2)
        torch.cuda.empty_cache()
        if not only or "search" in only:
            extras["search_scan"] = search_workload(torch, tq, syn, copies=4, steps=20)
        torch.cuda.empty_cache()
        if not only or "ablation" in only:
            extras["mse_keys_ablation"] = mse_keys_ablation(torch, tq, syn, copies=16, steps=32)
        torch.cuda.empty_cache()
        if not only or "formulations" in only:
            extras["logit_scan_formulations"] = scan_formulations(torch, tq, syn, copies=16, steps=32)
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        log("[cpu] timing the oracle" + (" in full (minutes)" if args.cpu_full else " on samples"))
        cpu = cpu_baseline(w, syn, torch, full=args.cpu_full)
    line = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["total_s"] / res["steps"] * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped decode layer: encode 32768-token key prefill + all q.k "
                               "logits", "kv_heads": w.n_kv, "q_heads": w.n_q, "head_dim": w.d, "batch": w.batch,
                   "context": w.n_tok, "key_bits": w.key_bits, "input_dtype": "bf16",
                   "compute": "fp32 vector arithmetic, int8/fp16/bf16 matrix cores with exact operands",
                   "copies_rotated": args.copies},
        "encode_tokens_per_s": kern["encode"]["tokens_per_s"],
        "step_encode_tokens_per_s": res["encode_tokens_per_s"],
        "roofline": roof, "cpu_baseline": cpu, "kernels": kern, "extras": extras,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
