"""GPU parity of the search scan: row-wise top-k (bit-exact against the
oracle's ranking of the same scores) and inner-product search over a coded
database (scores within the logit tolerance given identical codes, ranking
exact on the GPU's own scores, and membership equal to the oracle's wherever
the oracle score is clear of the k-th by more than the tolerance)."""
import numpy as np
import pytest
import torch

import kv_cache_vector_rht_amd as tq
import oracle as O
import synthetic as syn
from gpu_common import key_codec, pack_keys_into, say, to_f64
from tq_parity import ATOL, RTOL, assert_close

pytestmark = pytest.mark.gpu


def _scores(n_rows, n_cols, kind, seed, ld=None):
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 + seed)
    if kind == "ties":
        x = torch.randint(-20, 21, (n_rows, n_cols), generator=g).to(torch.float32)
    else:
        x = torch.randn((n_rows, n_cols), generator=g, dtype=torch.float32)
    if kind == "specials" and n_cols >= 8:
        x[:, 0] = -0.0
        x[:, 1] = 0.0
        x[:, 2] = float("inf")
        x[:, 3] = float("-inf")
        x[:, 5] = float("inf")
    if ld is not None and ld > n_cols:
        pad = torch.full((n_rows, ld), 7.0e30)          # padding must never be read
        pad[:, :n_cols] = x
        return pad
    return x


@pytest.mark.parametrize("n_rows,n_cols,k,kind,ld", [
    (3, 100, 1, "normal", None),
    (5, 4096, 10, "ties", None),          # exactly one chunk
    (2, 4097, 100, "ties", None),         # a one-column second chunk
    (4, 20000, 1000, "normal", None),
    (1, 9000, 1024, "ties", None),        # the largest k
    (7, 1, 1, "normal", None),
    (3, 333, 333, "ties", None),          # k = n_cols
    (2, 70001, 64, "specials", None),
    (3, 5000, 17, "normal", 5003),        # padded rows (ld > n_cols)
    (2, 100000, 1024, "ties", None),      # three select passes (25600 -> 7168 -> 2048 candidates)
])
def test_topk_matches_oracle_ranking(n_rows, n_cols, k, kind, ld):
    say(f"topk rows={n_rows} cols={n_cols} k={k} {kind} ld={ld}")
    host = _scores(n_rows, n_cols, kind, n_cols + k, ld)
    dev = host.to("cuda")
    vals, idx = tq.topk(dev, k, n_cols=n_cols)
    torch.cuda.synchronize()
    rv, ri = O.top_k(host[:, :n_cols].numpy(), k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(vals.cpu().numpy(), rv)


def test_topk_more_rows_than_one_launch_grid():
    say("topk rows=70001 cols=64 k=5 (rows in launches of 65535)")
    host = _scores(70001, 64, "ties", 3)
    vals, idx = tq.topk(host.to("cuda"), 5)
    torch.cuda.synchronize()
    rv, ri = O.top_k(host.numpy(), 5)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(vals.cpu().numpy(), rv)


def test_topk_twice_same_workspace():
    say("topk: two calls share one workspace, the second smaller")
    ws = torch.empty(tq.topk_workspace(4, 50000, 200), dtype=torch.uint8, device="cuda")
    for n_rows, n_cols, k in ((4, 50000, 200), (2, 3000, 5)):
        host = _scores(n_rows, n_cols, "ties", n_cols)
        vals, idx = tq.topk(host.to("cuda"), k, workspace=ws)
        torch.cuda.synchronize()
        rv, ri = O.top_k(host.numpy(), k)
        np.testing.assert_array_equal(idx.cpu().numpy(), ri)
        np.testing.assert_array_equal(vals.cpu().numpy(), rv)


def _check_membership(gpu_idx, ref, k):
    """Wherever the oracle score is clear of the oracle's k-th score by more
    than twice the tolerance, membership in the top k must agree."""
    for r in range(ref.shape[0]):
        kth = np.sort(ref[r])[::-1][k - 1]
        tol = 2 * (ATOL + RTOL * max(abs(kth), 1.0))
        chosen = set(gpu_idx[r].tolist())
        surely_in = np.nonzero(ref[r] > kth + tol)[0]
        surely_out = np.nonzero(ref[r] < kth - tol)[0]
        assert set(surely_in.tolist()) <= chosen, f"row {r}: a clear winner is missing"
        assert not (set(surely_out.tolist()) & chosen), f"row {r}: a clear loser was chosen"


@pytest.mark.parametrize("d,w,n_q,n_db,k", [
    (128, 3, 32, 5000, 10),
    (128, 2, 5, 4096 + 77, 100),
    (64, 3, 9, 3001, 16),
])
def test_search_given_oracle_codes(d, w, n_q, n_db, k):
    say(f"search d={d} w={w} queries={n_q} database={n_db} k={k}")
    kc = key_codec(900 + d + w, d, w)
    cap = (n_db + 31) // 32 * 32
    g = torch.Generator(device="cpu")
    g.manual_seed(d * 31 + w)
    db = torch.randn((1, n_db, d), generator=g, dtype=torch.float64)
    q = torch.randn((n_q, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    enc = kc.encode(db.numpy())
    codes, scal = tq.alloc_key_cache(1, cap, kc.gpu)
    pack_keys_into(enc, w, codes, scal)
    qd = q.to("cuda")
    scores = torch.empty((1, n_q, n_db), dtype=torch.float32, device="cuda")
    vals, idx = tq.search(kc.gpu, qd, codes, scal, n_db, k, scores=scores)
    torch.cuda.synchronize()
    ref = O.key_logits(to_f64(q), kc.signs, kc.centroids, kc.sketch, enc["idx"][0], enc["sigma"][0],
                       enc["nhat"][0], enc["ghat"][0])
    got = scores[0].cpu().numpy()
    assert_close(got, ref, "search scores")
    rv, ri = O.top_k(got, k)                              # exact ranking of the GPU's own scores
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(vals.cpu().numpy(), rv)
    _check_membership(idx.cpu().numpy(), ref, k)


def test_search_full_database_size():
    """The benchmark's search workload: 32 queries over 1,048,576 coded
    vectors (d 128, 4-bit keys), top 100. Ranking exact on the GPU scores;
    scores of 4096 sampled vectors against the oracle given the GPU's codes."""
    w = syn.SEARCH
    say(f"search full size: {w.n_q} queries x {w.n_db} vectors, k={w.k}")
    s, S = syn.key_codec_randoms(w.cfg, w.d)
    kc = tq.Codec.make(w.d, w.key_lm_bits, True, s, S)
    codes, scal = tq.alloc_key_cache(1, w.n_db, kc)
    tq.encode_kv(kc, syn.search_database(w, device="cuda"), codes, scal)
    q = syn.search_queries(w, device="cuda")
    scores = torch.empty((1, w.n_q, w.n_db), dtype=torch.float32, device="cuda")
    vals, idx = tq.search(kc, q, codes, scal, w.n_db, w.k, scores=scores)
    torch.cuda.synchronize()
    got = scores[0].cpu().numpy()
    rv, ri = O.top_k(got, w.k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(vals.cpu().numpy(), rv)
    # sampled scores against the oracle, from the GPU's own codes
    cols = np.random.default_rng(5).choice(w.n_db, 4096, replace=False)
    rec = codes[0, torch.as_tensor(cols, device="cuda")].cpu().numpy()
    sc = scal[0, torch.as_tensor(cols, device="cuda")].cpu().numpy().view(np.float16)
    kidx, ksig = O.unpack_key_codes(rec, w.d, w.key_lm_bits)
    cent, _ = O.make_codebook(w.d, w.key_lm_bits)
    ref = O.key_logits(to_f64(q.cpu()), s.numpy().astype(np.float64), cent, S.numpy().astype(np.float16), kidx,
                       ksig, sc[:, 0], sc[:, 1])
    assert_close(got[:, cols], ref, "search scores (sampled)")


def test_topk_in_hip_graph_replays():
    """tq_topk captured in a HIP graph and replayed three times, the scores
    rewritten eagerly between replays; every replay against the oracle."""
    say("topk in a HIP graph: 3 replays over changing scores")
    n_rows, n_cols, k = 4, 30000, 50
    scores = torch.empty((n_rows, n_cols), dtype=torch.float32, device="cuda")
    vals = torch.empty((n_rows, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((n_rows, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(tq.topk_workspace(n_rows, n_cols, k), dtype=torch.uint8, device="cuda")
    call = lambda: tq.lib.tq_topk(tq._ptr(scores), n_rows, n_cols, n_cols, k, tq._ptr(vals), tq._ptr(idx),
                                  tq._ptr(ws), ws.numel(), tq._stream(None))
    scores.copy_(_scores(n_rows, n_cols, "ties", 0).to("cuda"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert call() == tq.TQ_OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert call() == tq.TQ_OK
    torch.cuda.synchronize()
    for rep in range(3):
        host = _scores(n_rows, n_cols, "ties" if rep % 2 else "normal", 10 + rep)
        scores.copy_(host.to("cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rv, ri = O.top_k(host.numpy(), k)
        np.testing.assert_array_equal(idx.cpu().numpy(), ri)
        np.testing.assert_array_equal(vals.cpu().numpy(), rv)
