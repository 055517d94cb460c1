"""The ops beyond the four-op step recorded into a graph (torch's CUDA-graph
capture of the C-ABI launches on the capturing stream) and replayed several
times, with eager work and synchronisations between replays: every replay
must reproduce the eager result bit for bit."""
from __future__ import annotations

import pytest
import torch

import norm_rope_swiglu_amd as nrs
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    nrs.lib()


def _replays_match(run, outputs, reps=4, reset=None):
    """run() writes `outputs` in place; compare eager vs each graph replay.
    Between replays every output is overwritten (reset() for outputs the op
    writes only in part: it restores what the op does not write)."""
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    for o in outputs:
        o.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for i in range(reps):
        if reset is None:
            for o in outputs:
                o.fill_(-3.0 if o.is_floating_point() else -3)   # eager work between replays
        else:
            reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"


def _bf16(shape, seed, scale=1.0):
    n = 1
    for d in shape:
        n *= d
    return W.store(W.normal(W.stream_key(seed, f"graph/{shape}"), n).reshape(shape) * scale,
                   "bf16").cuda()


def test_graph_layernorm_and_add_layernorm():
    x, r = _bf16((5, 2048), 1), _bf16((5, 2048), 2)
    g, b = _bf16((2048,), 3, 0.1) + 1, _bf16((2048,), 4, 0.1)
    y, y2, ro = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)

    def run():
        nrs.layernorm(x, g, b, 1e-5, out=y)
        nrs.add_layernorm(x, r, g, b, 1e-5, out=y2, residual_out=ro)
    _replays_match(run, [y, y2, ro])


def test_graph_rmsnorm_linear_every_path():
    # 5 rows: the GEMV; 20 rows: the 16-row matrix-core tiles; 300 rows: the tiled GEMM
    x5, x20, x300 = _bf16((5, 2048), 5), _bf16((20, 2048), 9), _bf16((300, 512), 6)
    w1, w2 = _bf16((4096, 2048), 7, 0.02), _bf16((384, 512), 8, 0.05)
    y1 = torch.empty(5, 4096, dtype=torch.bfloat16, device="cuda")
    y3 = torch.empty(20, 4096, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty(300, 384, dtype=torch.bfloat16, device="cuda")

    def run():
        nrs.rmsnorm_linear(x5, w1, 1e-6, out=y1)
        nrs.rmsnorm_linear(x20, w1, 1e-6, out=y3)
        nrs.rmsnorm_linear(x300, w2, 1e-6, out=y2)
    _replays_match(run, [y1, y3, y2])


def test_graph_softmax_topk_sample():
    lg = _bf16((5, 3072), 9, 4.0)
    u = torch.rand(5, device="cuda")
    tok = torch.empty(5, dtype=torch.int32, device="cuda")
    probs = torch.empty_like(lg)

    def run():
        nrs.softmax_topk_sample(lg, 0.9, 50, u, token=tok, probs=probs)
    _replays_match(run, [tok, probs])


def test_graph_mrope_kv_append():
    w = W.decode(n_layers=1)
    L = w.layer
    q0, k, v = L.q.cuda(), L.k.cuda(), _bf16(tuple(L.k.shape), 10)
    pos = w.pos.cuda()
    kc = torch.zeros(5, 8, 64, 128, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    seq = torch.arange(5, dtype=torch.int32, device="cuda")
    slot = (torch.arange(5, dtype=torch.int32, device="cuda") * 7) % 64
    q = torch.empty_like(q0)

    def run():
        q.copy_(q0)                             # mrope rotates q in place
        nrs.mrope_kv_append(q, k, v, pos, w.sections, w.theta, kc, vc, seq, slot)
    def reset():
        q.fill_(-3.0)
        kc.zero_()
        vc.zero_()
    _replays_match(run, [q, kc, vc], reset=reset)
