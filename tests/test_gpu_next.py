"""GPU parity of the ops beyond the four-op hot path, through the C ABI,
against the fp64 oracle: M-RoPE fused with the KV-cache append, fused
softmax + top-k sampling, and LayerNorm with its fused residual add."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import norm_rope_swiglu_amd as nrs
import oracle
import workloads as W
from numerics import ln_scale
from parity import check, check_exact

pytestmark = pytest.mark.gpu

SENTINEL = -7.0


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    nrs.lib()


def _v_for(w, seed=5):
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(w.layer.k.shape, generator=g, dtype=torch.float64).to(torch.float32)
    return v.to(w.layer.k.dtype).to(w.layer.k.device)


def kv_parity(w, seq_idx, slot, n_seqs, max_seq, tag, rows=None):
    """Run nrs.mrope_kv_append on the workload's q/k (v drawn here) and check
    q, every written cache entry, and that every other entry is untouched."""
    L = w.layer
    dev = "cuda"
    dt = L.q.dtype
    q, k = L.q.to(dev).clone(), L.k.to(dev)
    v = _v_for(w).to(dev)
    pos = w.pos.to(dev)
    seq_idx = torch.as_tensor(seq_idx, dtype=torch.int32).to(dev)
    slot = torch.as_tensor(slot, dtype=torch.int32).to(dev)
    T, nkv, D = k.shape
    kc = torch.full((n_seqs, nkv, max_seq, D), SENTINEL, dtype=dt, device=dev)
    vc = torch.full_like(kc, SENTINEL)
    q0 = q.clone()
    nrs.mrope_kv_append(q, k, v, pos, w.sections, w.theta, kc, vc, seq_idx, slot)
    torch.cuda.synchronize()

    valid = (seq_idx >= 0) & (seq_idx < n_seqs) & (slot >= 0) & (slot < max_seq)
    # untouched entries keep the sentinel bit for bit
    written = torch.zeros(n_seqs, max_seq, dtype=torch.bool, device=dev)
    written[seq_idx[valid].long(), slot[valid].long()] = True
    keep = ~written[:, None, :, None].expand_as(kc)
    assert torch.all(kc[keep] == SENTINEL) and torch.all(vc[keep] == SENTINEL), f"{tag}: stray writes"

    sel = torch.arange(T, device=dev) if rows is None else rows.to(dev)
    sel = sel[valid[sel]]
    # the oracle with each selected token in its own one-slot cache
    n = int(sel.numel())
    qs_, ks_, vs_ = q0[sel].cpu(), k[sel].cpu(), v[sel].cpu()
    ps_ = pos[:, sel].cpu().contiguous()
    ident = torch.arange(n, dtype=torch.int32)
    rq, rkc, rvc = oracle.mrope_kv_append(qs_, ks_, vs_, ps_, w.sections, w.theta, ident,
                                          torch.zeros(n, dtype=torch.int32),
                                          np.zeros((n, nkv, 1, D)), torch.zeros(n, nkv, 1, D, dtype=dt))
    b, s = seq_idx[sel].long(), slot[sel].long()
    check(f"{tag}/q", q[sel], rq, pairs=True)
    check(f"{tag}/k_cache", kc[b, :, s, :], rkc[:, :, 0, :], pairs=True)
    check_exact(f"{tag}/v_cache", vc[b, :, s, :], rvc[:, :, 0, :])


def test_kv_append_decode_step():
    w = W.decode(n_layers=1)
    p = w.pos[0]
    kv_parity(w, seq_idx=list(range(5)), slot=p, n_seqs=5, max_seq=2048, tag="kv/decode")


def test_kv_append_prefill():
    w = W.prefill()
    kv_parity(w, seq_idx=[0] * w.tokens, slot=list(range(w.tokens)), n_seqs=1, max_seq=4096,
              tag="kv/prefill")


def test_kv_append_ragged():
    w = W.ragged(device="cuda")
    seq, slot = [], []
    for i, L in enumerate(w.seq_lens):
        seq += [i] * L
    slot = w.pos[0].cpu().tolist()            # each sequence's own positions (offset + index)
    kv_parity(w, seq_idx=seq, slot=slot, n_seqs=len(w.seq_lens), max_seq=2560, tag="kv/ragged")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_append_skips_out_of_range(dtype):
    w = W.sweep(dtype=dtype, hidden=512, head_dim=64, tokens=40)
    seq = [t % 3 for t in range(40)]
    slot = [t for t in range(40)]
    seq[3], seq[7], slot[11], slot[13] = -1, 3, -2, 40     # nonexistent sequence / slot
    kv_parity(w, seq_idx=seq, slot=slot, n_seqs=3, max_seq=40, tag=f"kv/skip/{dtype}")


@pytest.mark.parametrize("D,sec,nq,nkv", [(16, (2, 3, 3), 3, 1), (32, (4, 6, 6), 2, 3),
                                          (64, (8, 12, 12), 100, 40), (128, (16, 24, 24), 16, 8),
                                          (256, (32, 48, 48), 4, 2)])
def test_kv_append_head_shapes(D, sec, nq, nkv):
    # half-heads of 1, 2 or 4 chunks take one lane per chunk with the pair partner swizzled
    # in; 100 q + 2 x 40 kv heads of 64 give more chunks per token than a block has threads
    for dt in (torch.float32, torch.bfloat16):
        g = torch.Generator().manual_seed(D)
        T = 37
        w = W.Workload("kvshape", "f32" if dt == torch.float32 else "bf16", T, nq * D, 0, nq, nkv, D,
                       sec, 1e4, 1e-6, torch.randint(0, 9000, (3, T), generator=g, dtype=torch.int32))
        q = torch.randn(T, nq, D, generator=g).to(dt)
        k = torch.randn(T, nkv, D, generator=g).to(dt)
        w.layers.append(W.Layer(None, None, None, q, k, None))
        perm = torch.randperm(T, generator=g)
        kv_parity(w, seq_idx=(perm % 2).tolist(), slot=(perm // 2).tolist(), n_seqs=2, max_seq=19,
                  tag=f"kv/shape{D}/{dt}")


def test_kv_append_narrow_heads_streaming():
    # head_dim 64 at a streaming size (two chunks per thread, several tokens per block, a
    # part-filled last block), slots in reverse order, checked on sampled tokens
    w = W.sweep(dtype="bf16", hidden=1024, head_dim=64, tokens=8192 + 3, device="cuda")
    T = w.tokens
    g = torch.Generator().manual_seed(5)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, T - 2, T - 1]),
                                   torch.randint(0, T, (60,), generator=g)]))
    kv_parity(w, seq_idx=[0] * T, slot=list(range(T - 1, -1, -1)), n_seqs=1, max_seq=T,
              tag="kv/narrow_stream", rows=rows)


def test_kv_append_small_tokens_streaming():
    # 4 q + 2 kv heads of 128 (64 items a token) at a streaming size: 4 tokens per ~256-thread
    # block with a part-filled last block, slots scattered over two sequences
    w = W.sweep(dtype="bf16", hidden=512, head_dim=128, tokens=8195, device="cuda")
    T = w.tokens
    g = torch.Generator().manual_seed(6)
    perm = torch.randperm(T, generator=g)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, 2, 3, T - 3, T - 2, T - 1]),
                                   torch.randint(0, T, (57,), generator=g)]))
    kv_parity(w, seq_idx=(perm % 2).tolist(), slot=(perm // 2).tolist(), n_seqs=2,
              max_seq=(T + 1) // 2, tag="kv/small_tokens_stream", rows=rows)


@pytest.mark.parametrize("hidden,T", [(1024, 8195), (2048, 8197)])
def test_kv_append_1024_thread_blocks_streaming(hidden, T):
    # tokens of 128 and 256 items at a streaming size: 8 and 4 tokens per 1024-thread block,
    # a part-filled last block, slots shuffled over two sequences
    w = W.sweep(dtype="bf16", hidden=hidden, head_dim=128, tokens=T, device="cuda")
    g = torch.Generator().manual_seed(8)
    perm = torch.randperm(T, generator=g)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, 2, 3, 4, T - 5, T - 3, T - 2, T - 1]),
                                   torch.randint(0, T, (55,), generator=g)]))
    kv_parity(w, seq_idx=(perm % 2).tolist(), slot=(perm // 2).tolist(), n_seqs=2,
              max_seq=(T + 1) // 2, tag=f"kv/blocks1024/H{hidden}", rows=rows)


def test_kv_append_full_size_sampled():
    w = W.sweep(dtype="bf16", hidden=2048, head_dim=128, tokens=32768, device="cuda")
    g = torch.Generator().manual_seed(3)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, 32766, 32767]),
                                   torch.randint(0, 32768, (60,), generator=g)]))
    kv_parity(w, seq_idx=[0] * 32768, slot=list(range(32768)), n_seqs=1, max_seq=32768,
              tag="kv/32k", rows=rows)


# ------------------------------------------------------------ fused softmax + top-k sampling

DELTA = 1e-5   # fp32 prefix-sum error allowance on the sampling CDF (k <= 1024 terms)


def _logits(rows, vocab, scale, dt, seed, ties=False):
    key = W.stream_key(seed, f"logits/{rows}/{vocab}/{scale}/{ties}")
    v = W.normal(key, rows * vocab).reshape(rows, vocab) * scale
    if ties:
        v = torch.round(v)
    return W.store(v, dt)


def _u(rows, seed):
    return W.uniform(W.stream_key(seed, f"u/{rows}"), rows).to(torch.float32)


def sample_parity(logits, T, k, u, tag, want_probs=True):
    """Check the full softmax (when asked for), and that every sampled token
    lies in the oracle's kept set with u inside its exact CDF interval (to
    DELTA); where u is farther than DELTA from every boundary the token must be
    the oracle's."""
    if want_probs:
        tok, probs = nrs.softmax_topk_sample(logits.cuda(), T, k, u.cuda(), probs=True)
    else:
        tok = nrs.softmax_topk_sample(logits.cuda(), T, k, u.cuda())
    otok, oprobs, kept, cdf = oracle.softmax_topk_sample(logits, T, k, u.numpy(),
                                                         want_probs=want_probs)
    if want_probs:
        check(f"{tag}/probs", probs, oprobs)
    tok = tok.cpu().numpy()
    uu = u.numpy().astype(np.float64)
    for r in range(logits.shape[0]):
        where = np.nonzero(kept[r] == tok[r])[0]
        assert where.size == 1, f"{tag}: row {r} token {tok[r]} not in the oracle's top {k}"
        j = int(where[0])
        lo = cdf[r, j - 1] if j > 0 else 0.0
        assert lo - DELTA <= uu[r] < cdf[r, j] + DELTA, f"{tag}: row {r} u {uu[r]} outside [{lo}, {cdf[r, j]})"
        if np.min(np.abs(cdf[r] - uu[r])) > DELTA:
            assert tok[r] == otok[r], f"{tag}: row {r}"
    return tok, otok


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("vocab,k,scale,T", [(3072, 50, 4.0, 0.9), (3072, 1024, 0.5, 1.0),
                                             (4104, 7, 2.0, 0.7), (8, 8, 1.0, 1.3),
                                             (151936, 50, 3.0, 1.0)])
def test_sample_decode_rows(dt, vocab, k, scale, T):
    rows = 5 if vocab > 50000 else 33
    lg = _logits(rows, vocab, scale, dt, 1)
    sample_parity(lg, T, k, _u(rows, 2), f"sample/{dt}/V{vocab}/k{k}")


@pytest.mark.parametrize("dt,vocab", [("bf16", 16384), ("bf16", 32000), ("bf16", 65536),
                                      ("f32", 8192), ("f32", 16384), ("f32", 32000),
                                      ("bf16", 65544), ("f32", 32776)])
def test_sample_register_held_rows(dt, vocab):
    # rows held in registers at 2, 4 and 8 chunks per thread, and just past the
    # largest held row (streamed by every pass)
    lg = _logits(6, vocab, 3.0, dt, 11)
    sample_parity(lg, 0.8, 64, _u(6, 12), f"sample/{dt}/held{vocab}")


@pytest.mark.parametrize("dt,vocab,k", [("bf16", 8192, 64), ("f32", 4096, 64), ("bf16", 3080, 33),
                                        ("f32", 260, 5), ("bf16", 520, 64)])
def test_sample_partial_chunk_rounds(dt, vocab, k):
    # rows whose chunks leave the last round of the 1024 threads partly filled
    # (or fill it exactly), with k up to one wave's width
    lg = _logits(9, vocab, 3.0, dt, 21)
    sample_parity(lg, 0.9, k, _u(9, 22), f"sample/rounds/{dt}/V{vocab}/k{k}")
    # many ties at the k-th value: the lowest indices are kept
    t = _logits(4, vocab, 1.0, dt, 23, ties=True)
    sample_parity(t, 1.0, k, _u(4, 24), f"sample/rounds_ties/{dt}/V{vocab}/k{k}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("vocab,k", [(3072, 65), (3072, 128), (32000, 256), (151936, 200)])
def test_sample_mid_k(dt, vocab, k):
    # k past one wave: the counting sort (up to 256 gathered entries) with the
    # block-wide scan, and a streamed row gathering more than one wave
    rows = 4 if vocab > 50000 else 12
    lg = _logits(rows, vocab, 3.0, dt, 31)
    sample_parity(lg, 1.1, k, _u(rows, 32), f"sample/midk/{dt}/V{vocab}/k{k}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sample_ties(dt):
    # integer-valued logits: many equal values, the k-th often tied
    lg = _logits(40, 3072, 2.0, dt, 3, ties=True)
    sample_parity(lg, 1.0, 100, _u(40, 4), f"sample/ties/{dt}")
    lg = torch.zeros(3, 1024).to(lg.dtype)                # all equal: lowest indices kept
    tok, _ = sample_parity(lg, 1.0, 16, torch.tensor([0.0, 0.5, 0.99], dtype=torch.float32),
                           f"sample/flat/{dt}")
    assert tok.tolist() == [0, 8, 15]
    # ties at the k-th value outnumbering the 1024-entry gather buffer: the ordered
    # compaction must keep the lowest indices (a few larger logits sit above them)
    lg = torch.zeros(3, 8192)
    lg[:, [5000, 7, 8191]] = torch.tensor([3.0, 2.0, 1.0])
    lg = lg.to(W.store(torch.zeros(1), dt).dtype)
    tok, _ = sample_parity(lg, 1.0, 20, torch.tensor([0.0, 0.9999, 0.97], dtype=torch.float32),
                           f"sample/many_ties/{dt}")
    assert tok[0] == 5000


@pytest.mark.parametrize("dt,vocab,k,rows", [("bf16", 151936, 50, 7), ("bf16", 151936, 200, 3),
                                             ("bf16", 151936, 1024, 2), ("bf16", 65544, 64, 5),
                                             ("bf16", 70000, 7, 257), ("f32", 40000, 64, 6),
                                             ("f32", 32776, 1, 4), ("f32", 151936, 33, 3)])
def test_sample_long_rows_token_only(dt, vocab, k, rows):
    # rows longer than a workgroup holds in registers, sampled without the softmax output
    lg = _logits(rows, vocab, 3.0, dt, 41)
    sample_parity(lg, 0.9, k, _u(rows, 42), f"sample/long/{dt}/V{vocab}/k{k}", want_probs=False)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sample_long_rows_ties(dt):
    # ties in a streamed row, and equal maxima at scattered places (each 65536 logits apart
    # in bf16, 32768 in fp32: a register-held row's length)
    V = 151936
    seg = 65536 if dt == "bf16" else 32768
    n_seg = -(-V // seg)
    # integer-valued rows: many ties at the k-th value
    lg = _logits(5, V, 2.0, dt, 43, ties=True)
    sample_parity(lg, 1.0, 100, _u(5, 44), f"sample/long_ties/{dt}", want_probs=False)
    # equal maxima around every multiple of that length, fewer than k of them above a flat
    # row: the kept set is every maximum plus the lowest-index zeros
    lg = torch.zeros(4, V)
    for b in range(1, n_seg):
        lg[:, b * seg - 3: b * seg + 3] = 5.0
    lg[:, V - 2:] = 5.0
    lg = lg.to(W.store(torch.zeros(1), dt).dtype)
    u = torch.tensor([0.0, 0.3, 0.7, 0.999999], dtype=torch.float32)
    tok, otok = sample_parity(lg, 1.0, 64, u, f"sample/long_scattered_max/{dt}", want_probs=False)
    assert tok[0] == seg - 3                                # the lowest-index maximum first
    # all equal: the lowest indices are kept
    lg = torch.zeros(3, V).to(lg.dtype)
    tok, _ = sample_parity(lg, 1.0, 16, torch.tensor([0.0, 0.5, 0.99], dtype=torch.float32),
                           f"sample/long_flat/{dt}", want_probs=False)
    assert tok.tolist() == [0, 8, 15]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sample_long_rows_one_read_cases(dt):
    # rows longer than the registers hold are read once: the held first part's k-th largest
    # logit bounds the row's from below, and only logits at or above it are kept from the rest
    V = 151936
    ramp = torch.linspace(-8.0, 8.0, V)
    # ascending: the whole rest of the row passes the bound (the buffer overflows, and the
    # row is selected again over every logit); descending: none of it does
    lg = W.store(torch.stack([ramp, ramp.flip(0), ramp, ramp.flip(0)]), dt)
    tok, _ = sample_parity(lg, 1.0, 50, torch.tensor([0.0, 0.0, 0.6, 0.6], dtype=torch.float32),
                           f"sample/long_ramp/{dt}", want_probs=False)
    assert tok[1] == 0                                      # the largest logit comes first
    # the largest logits all in the streamed part, below the buffer's size
    lg = _logits(6, V, 3.0, dt, 47).float()
    lg[:, V - 40:] = 20.0 + 0.01 * torch.arange(40, dtype=torch.float32)
    sample_parity(W.store(lg, dt), 1.0, 50, _u(6, 48), f"sample/long_late_peaks/{dt}",
                  want_probs=False)
    # k = 300: more kept entries than the counting sort takes
    lg = _logits(4, V, 3.0, dt, 49)
    sample_parity(lg, 1.0, 300, _u(4, 50), f"sample/long_k300/{dt}", want_probs=False)


def test_sample_benchmark_batch_every_row():
    # the benchmark's sampler launch: 256 rows x 151936 bf16 logits, k 50, token only; every
    # row against the oracle's full sort
    lg = _logits(256, 151936, 3.0, "bf16", 51)
    sample_parity(lg, 1.0, 50, _u(256, 52), "sample/bench256x151936", want_probs=False)


def test_sample_long_rows_greedy_tied_maximum():
    lg = _logits(8, 151936, 4.0, "bf16", 45).float()
    top = lg.max(dim=1).values + 2.0
    lg[:, 120000] = top
    lg[:, 140000] = top                                    # tied maximum: lower index wins
    tok = nrs.softmax_topk_sample(lg.to(torch.bfloat16).cuda(), 1.0, 1, _u(8, 46).cuda()).cpu()
    assert torch.all(tok == 120000)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sample_long_rows_equal_maxima_in_few_threads(dt):
    # 200 equal maxima packed into the chunks of a few threads (thread t holds chunks t,
    # t + 1024, ...; 8 or 4 logits a chunk), k = 30: the bound, taken from each thread's
    # largest logit, counts each such thread once, and the kept set is the 30 lowest-index
    # maxima
    V = 151936
    vec = 8 if dt == "bf16" else 4
    lg = _logits(4, V, 1.0, dt, 61).float()
    nch = V // vec
    idx = sorted((t + 1024 * j) * vec + e for t in (3, 700) for j in range(nch // 1024 + 1)
                 for e in range(vec) if t + 1024 * j < nch)[:200]
    assert len(idx) == 200
    lg[:, idx] = 5.0
    lg = W.store(lg, dt)
    u = torch.tensor([0.0, 0.25, 0.5, 0.999], dtype=torch.float32)
    tok, _ = sample_parity(lg, 1.0, 30, u, f"sample/long_packed_maxima/{dt}", want_probs=False)
    assert tok[0] == min(idx)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sample_long_rows_many_equal_maxima(dt):
    # 400 equal maxima spread over the row, k = 50: all of them pass the bound, and the
    # sort keeps the 50 lowest-index maxima
    V = 151936
    g = torch.Generator().manual_seed(62)
    lg = _logits(3, V, 1.0, dt, 63).float()
    for r in range(3):
        lg[r, torch.randperm(V, generator=g)[:400]] = 6.0
    lg = W.store(lg, dt)
    u = torch.tensor([0.0, 0.5, 0.9999], dtype=torch.float32)
    tok, _ = sample_parity(lg, 1.0, 50, u, f"sample/long_equal_maxima/{dt}", want_probs=False)
    first = [int(torch.nonzero(lg[r].float() == 6.0)[0]) for r in range(3)]
    assert tok[0] == first[0]


@pytest.mark.parametrize("dt,vocab,k,rows", [("bf16", 65544, 128, 5), ("bf16", 151936, 1, 6),
                                             ("bf16", 65544, 50, 600), ("f32", 151936, 50, 3),
                                             ("bf16", 262144, 20, 3)])
def test_sample_long_rows_shapes(dt, vocab, k, rows):
    # k = 128 (the bound from each wave's 16 leading maxima), greedy, 600 rows, fp32, and
    # a 262,144-logit row (several streamed batches past the held part)
    lg = _logits(rows, vocab, 3.0, dt, 64)
    sample_parity(lg, 0.8, k, _u(rows, 65), f"sample/long/{dt}/V{vocab}/k{k}/R{rows}",
                  want_probs=False)


def test_sample_long_rows_back_to_back_calls():
    # long-row calls of different shapes and k in a row on one stream, then again, every
    # one checked
    cases = [("bf16", 151936, 50, 8), ("bf16", 65544, 64, 20), ("f32", 151936, 40, 4),
             ("bf16", 151936, 3, 8)]
    for rep in range(2):
        for i, (dt, V, k, R) in enumerate(cases):
            lg = _logits(R, V, 3.0, dt, 70 + i)
            sample_parity(lg, 1.0, k, _u(R, 80 + i + rep), f"sample/b2b/{rep}/{i}",
                          want_probs=False)


def test_sample_long_rows_graph_replays():
    # long-row calls captured in a graph and replayed several times with eager calls
    # between: every replay gives the eager tokens
    R, V = 64, 151936
    lgs = [_logits(R, V, 3.0, "bf16", 90 + i).cuda() for i in range(3)]
    us = [_u(R, 95 + i).cuda() for i in range(3)]
    toks = [torch.empty(R, dtype=torch.int32, device="cuda") for _ in range(3)]
    want = [nrs.softmax_topk_sample(lgs[i], 1.0, 50, us[i]).cpu() for i in range(3)]
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        nrs.softmax_topk_sample(lgs[0], 1.0, 50, us[0], token=toks[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        for i in range(3):
            nrs.softmax_topk_sample(lgs[i], 1.0, 50, us[i], token=toks[i])
    for rep in range(4):
        for t in toks:
            t.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(toks[i].cpu(), want[i]), f"replay {rep} call {i}"
        other = nrs.softmax_topk_sample(lgs[(rep + 1) % 3], 1.0, 50, us[(rep + 1) % 3]).cpu()
        assert torch.equal(other, want[(rep + 1) % 3]), f"eager call after replay {rep}"
    # and against the oracle once
    otok, _, kept, _ = oracle.softmax_topk_sample(lgs[0].cpu(), 1.0, 50, us[0].cpu().numpy(),
                                                  want_probs=False)
    for r in range(R):
        assert int(want[0][r]) in kept[r].tolist()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sample_long_rows_bound_at_or_below_zero(dt):
    # the long-row filter tests loaded values against a bound above zero and compares order
    # keys otherwise: rows of negative logits (log-probabilities), and rows whose k-th value
    # is exactly zero with +0 and -0 both present (equal logits, kept by index)
    V = 151936
    neg = -(_logits(3, V, 2.0, dt, 71).float().abs() + 0.5)
    sample_parity(W.store(neg, dt), 1.0, 50, _u(3, 72), f"sample/long_negative/{dt}",
                  want_probs=False)
    z = torch.zeros(3, V)
    z[:, 1::2] = -0.0                                  # signed zeros interleaved
    z[:, [100, 5000, 90000, 150000]] = torch.tensor([3.0, 2.0, 1.0, 0.5])
    z[:, 7] = -1.0
    tok, _ = sample_parity(W.store(z, dt), 1.0, 20, torch.tensor([0.0, 0.99, 0.9999], dtype=torch.float32),
                           f"sample/long_zero_bound/{dt}", want_probs=False)
    assert tok[0] == 100


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_sample_long_rows_non_finite_logits_give_a_valid_index(dt):
    # NaN logits, and infinite ones (exp(inf - inf) is NaN here as in fp64), give an
    # unspecified token, but always one of the row's indices
    V = 151936
    lg = _logits(6, V, 3.0, dt, 74).float()
    lg[0, ::3] = float("nan")
    lg[1, :] = float("nan")
    lg[2, 12345] = float("nan")
    lg[3, [40000, 20]] = float("inf")
    lg[4, :] = -float("inf")
    lg[5, ::2] = float("inf")
    tok = nrs.softmax_topk_sample(W.store(lg, dt).cuda(), 1.0, 50, _u(6, 75).cuda()).cpu()
    assert torch.all((tok >= 0) & (tok < V))


@pytest.mark.parametrize("dt,vocab", [("bf16", 8192), ("bf16", 16384), ("bf16", 32000),
                                      ("bf16", 65528), ("bf16", 65536), ("f32", 4096),
                                      ("f32", 8200), ("f32", 32000), ("f32", 32768)])
def test_sample_held_rows_token_only(dt, vocab):
    # token-only rows of one to eight chunks per thread (the whole row held) with top_k <= 128
    # are filtered against a bound from the threads' maxima: exactly one chunk per thread,
    # partial last rounds, k = 1, 50 and 128, ties, all-equal rows (every entry passes the
    # bound: the buffer overflows and the row is selected again), ramps, negative rows (the
    # bound below zero: compared on order keys)
    rows = 5
    for k, seed in ((50, 81), (1, 82), (128, 83)):
        lg = _logits(rows, vocab, 3.0, dt, seed)
        sample_parity(lg, 0.9, k, _u(rows, seed + 10), f"sample/held/{dt}/V{vocab}/k{k}",
                      want_probs=False)
    t = _logits(rows, vocab, 2.0, dt, 84, ties=True)
    sample_parity(t, 1.0, 64, _u(rows, 85), f"sample/held_ties/{dt}/V{vocab}", want_probs=False)
    ramp = torch.linspace(-8.0, 8.0, vocab)
    other = torch.stack([torch.zeros(vocab), ramp, ramp.flip(0), -(ramp.abs() + 1.0)])
    stored = W.store(other, dt)
    tok, _ = sample_parity(stored, 1.0, 40, torch.tensor([0.5, 0.0, 0.0, 0.3], dtype=torch.float32),
                           f"sample/held_shapes/{dt}/V{vocab}", want_probs=False)
    for r in (1, 2):   # u = 0: the first of the largest logits (bf16 rounding ties the ramp's ends)
        row = stored[r].float()
        assert tok[r] == int(torch.nonzero(row == row.max())[0])


def test_sample_greedy_is_first_argmax():
    lg = _logits(64, 3072, 4.0, "f32", 5)
    lg[:, 1234] = lg.max(dim=1).values + 1.0
    lg[:, 2222] = lg[:, 1234]                              # tied maximum: lower index wins
    tok = nrs.softmax_topk_sample(lg.cuda(), 1.0, 1, _u(64, 6).cuda()).cpu()
    assert torch.all(tok == 1234)


def test_sample_inverse_cdf_frequencies():
    lg = _logits(1, 64, 2.0, "f32", 7).repeat(20000, 1)
    N = lg.shape[0]
    u = ((torch.arange(N, dtype=torch.float64) + 0.5) / N).to(torch.float32)
    tok = nrs.softmax_topk_sample(lg.cuda(), 1.0, 64, u.cuda()).cpu().numpy()
    _, probs, _, _ = oracle.softmax_topk_sample(lg[:1], 1.0, 64, np.zeros(1, np.float32))
    counts = np.bincount(tok, minlength=64)
    assert np.all(np.abs(counts - N * probs[0]) <= 2.0)


# ------------------------------------------------------------ LayerNorm

def _f32(v):
    return float(np.float32(v))


def _ln_inputs(rows, hidden, dt, seed=0, offset=3.0, bias=True):
    """Rows with their own mean and spread (LayerNorm's inputs are not
    centred), gamma ~ 1 + 0.1 N, beta ~ 0.1 N."""
    def key(n):
        return W.stream_key(seed, f"ln/{n}/{rows}/{hidden}/{offset}")
    mu = W.normal(key("mu"), rows).reshape(rows, 1) * offset
    sd = torch.exp(W.normal(key("sd"), rows).reshape(rows, 1) * 0.5)
    x = W.normal(key("x"), rows * hidden).reshape(rows, hidden) * sd + mu
    gamma = 1 + 0.1 * W.normal(key("g"), hidden)
    beta = 0.1 * W.normal(key("b"), hidden) if bias else None
    return W.store(x, dt), W.store(gamma, dt), None if beta is None else W.store(beta, dt)


def ln_parity(x, gamma, beta, eps, tag, residual=None, rows=None):
    """nrs.layernorm / nrs.add_layernorm against the oracle, on every row or
    on the sampled `rows` of a full-size launch."""
    cu = (lambda t: None if t is None else t.cuda())
    if residual is None:
        y = nrs.layernorm(cu(x), cu(gamma), cu(beta), eps).cpu()
        ro = None
    else:
        y, ro = nrs.add_layernorm(cu(x), cu(residual), cu(gamma), cu(beta), eps)
        y, ro = y.cpu(), ro.cpu()
    sel = slice(None) if rows is None else rows
    xs = x[sel].contiguous()
    if residual is None:
        ry, h = oracle.layernorm(xs, gamma, beta, _f32(eps)), xs
    else:
        ry, h = oracle.add_layernorm(xs, residual[sel].contiguous(), gamma, beta, _f32(eps))
        check_exact(f"{tag}/residual_out", ro[sel], h)
    sc = ln_scale(oracle.widen(h).reshape(h.shape), oracle.widen(gamma),
                  None if beta is None else oracle.widen(beta), _f32(eps))
    check(f"{tag}/y", y[sel], ry, scale=sc)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("hidden", [8, 24, 200, 1024, 1280, 1600, 2048, 5120, 8192, 12288, 32768])
def test_layernorm_widths(dt, hidden):
    if dt == "f32" and hidden in (8, 24):
        hidden //= 2                               # fp32 rows need multiples of 4 only
    rows = 37 if hidden <= 8192 else 5
    bias = hidden % 3 != 1
    x, g, b = _ln_inputs(rows, hidden, dt, 1, bias=bias)
    ln_parity(x, g, b, 1e-5, f"ln/{dt}/H{hidden}")
    r, _, _ = _ln_inputs(rows, hidden, dt, 2, offset=1.0)
    ln_parity(x, g, b, 1e-5, f"add_ln/{dt}/H{hidden}", residual=r)


def test_layernorm_widest_rows():
    x, g, b = _ln_inputs(3, 65536, "bf16", 3)
    ln_parity(x, g, b, 1e-5, "ln/bf16/H65536")
    ln_parity(x, g, b, 1e-5, "add_ln/bf16/H65536", residual=x.flip(0).contiguous())


@pytest.mark.parametrize("rows", [1, 3, 4, 5, 255, 257])
def test_layernorm_row_counts(rows):
    x, g, b = _ln_inputs(rows, 1024, "bf16", 4)
    ln_parity(x, g, b, 1e-6, f"ln/rows{rows}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_layernorm_cancellation_and_degenerate_rows(dt):
    # far-off means (|mean| / sigma ~ 1e3), constant rows (variance 0: y = beta
    # up to the mean's rounding), eps dominating a tiny variance
    x, g, b = _ln_inputs(16, 2048, dt, 5, offset=1000.0)
    ln_parity(x, g, b, 1e-5, f"ln/{dt}/offset")
    c = torch.full((4, 2048), 0.0)
    c[0] = 3.0
    c[1] = -0.15625
    c[2] = 7.1
    c[3, ::2], c[3, 1::2] = 1e-4, -1e-4
    ln_parity(W.store(c, dt), g, b, 1e-5, f"ln/{dt}/degenerate")
    y = nrs.layernorm(W.store(c, dt)[:2].cuda(), g.cuda(), b.cuda(), 1e-5).cpu()
    assert torch.equal(y, b.expand(2, -1))        # sums and means of c[0], c[1] are exact


def test_layernorm_strided_in_place_and_empty():
    big, g, b = _ln_inputs(9, 3072, "bf16", 6)
    xd = big.cuda()[:, 512:2560]                  # rows of stride 3072
    y = nrs.layernorm(xd, g[:2048].contiguous().cuda(), b[:2048].contiguous().cuda(), 1e-5)
    ry = oracle.layernorm(big[:, 512:2560], g[:2048].contiguous(), b[:2048].contiguous(), _f32(1e-5))
    check("ln/strided", y, ry, scale=ln_scale(oracle.widen(big[:, 512:2560].contiguous()).reshape(9, 2048),
                                               oracle.widen(g[:2048].contiguous()),
                                               oracle.widen(b[:2048].contiguous()), _f32(1e-5)))
    z = big[:, 512:2560].contiguous().cuda()     # the same rows, in place
    nrs.layernorm(z, g[:2048].contiguous().cuda(), b[:2048].contiguous().cuda(), 1e-5, out=z)
    check_exact("ln/in_place", z, y.cpu())
    e = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    gg = torch.ones(256, dtype=torch.bfloat16, device="cuda")
    assert nrs.layernorm(e, gg).shape == (0, 256)
    yy, rr = nrs.add_layernorm(e, e.clone(), gg, gg)
    assert yy.shape == rr.shape == (0, 256)


def test_add_layernorm_in_place():
    x, g, b = _ln_inputs(64, 1024, "bf16", 7)
    r, _, _ = _ln_inputs(64, 1024, "bf16", 8)
    y, ro = nrs.add_layernorm(x.cuda(), r.cuda(), g.cuda(), b.cuda(), 1e-5)
    xd, rd = x.cuda(), r.cuda()
    nrs.add_layernorm(xd, rd, g.cuda(), b.cuda(), 1e-5, out=xd, residual_out=rd)
    check_exact("add_ln/in_place.y", xd, y.cpu())
    check_exact("add_ln/in_place.residual_out", rd, ro.cpu())


@pytest.mark.parametrize("add", [False, True])
@pytest.mark.parametrize("dt,H,T", [("bf16", 1544, 8195), ("bf16", 3080, 8195), ("f32", 1000, 8195),
                                    ("f32", 1540, 2051)])
def test_layernorm_streaming_ragged_width(add, dt, H, T):
    # streaming-size calls whose rows (193 or 385 bf16 chunks, 250 or 385 fp32 chunks) take one
    # wave each with 4 or 8 chunks per thread (8: plain LayerNorm only; fp32 in calls up to
    # 32 MiB), the last only partly filled, over a row count that leaves a part-filled block
    x, g, b = _ln_inputs(T, H, dt, 12)
    r = _ln_inputs(T, H, dt, 13, offset=1.0)[0] if add else None
    gen = torch.Generator().manual_seed(14)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, 2, 3, T - 3, T - 2, T - 1]),
                                   torch.randint(0, T, (57,), generator=gen)]))
    ln_parity(x, g, b, 1e-5, f"{'add_' if add else ''}ln/stream/{dt}/{H}", residual=r, rows=rows)


@pytest.mark.parametrize("add", [False, True])
def test_layernorm_full_size_sampled(add):
    # the benchmark's launch: 32768 rows x 2048, bf16, streaming stores
    T, H = 32768, 2048
    x, g, b = _ln_inputs(T, H, "bf16", 9)
    r = _ln_inputs(T, H, "bf16", 10, offset=1.0)[0] if add else None
    gen = torch.Generator().manual_seed(11)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, 2, 3, T - 2, T - 1]),
                                   torch.randint(0, T, (58,), generator=gen)]))
    ln_parity(x, g, b, 1e-5, f"{'add_' if add else ''}ln/32k", residual=r, rows=rows)
