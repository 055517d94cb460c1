"""GPU parity of the HIP kernels (through the C ABI) against the fp64 oracle.

Every workload recipe is covered: the tiny fp32 layer, all 28 layers of the
bf16 decode step, the bf16 prefill with outliers and mixed position streams,
the packed ragged batch, and the width/numerics sweep (reduced token counts
element by element; full 32768-token launches on sampled rows).  Edge cases:
empty calls, ragged lane tails, the block-per-row path for wide rows, strided
and in-place calls, packed qkv, extreme gates, subnormal results.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import norm_rope_swiglu_amd as nrs
import oracle
import workloads as W
from parity import check, check_exact, dump

pytestmark = pytest.mark.gpu
# where the per-check parity report (every comparison's worst error and cosine) is written:
# the file named by NRS_PARITY_REPORT, if set
REPORT = os.environ.get("NRS_PARITY_REPORT")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    nrs.lib()  # raises if the HIP library is missing: no fallback
    yield
    if REPORT:
        dump(REPORT)


def f32(v):
    return float(np.float32(v))


def cuda(t):
    return t.to("cuda", copy=True)


def layer_parity(w: W.Workload, L: W.Layer, tag: str, rows=None):
    """Run the four ops on the GPU over the whole layer; compare all rows, or
    only `rows` (an index tensor) against the oracle."""
    dev = L.x.device.type == "cuda"
    g = (lambda t: t) if dev else cuda
    x, res, gamma, q, k, gu, pos = (g(L.x), g(L.residual), g(L.gamma), g(L.q.clone()),
                                    g(L.k.clone()), g(L.gate_up), g(w.pos))
    h_in = (lambda t: t.cpu()) if rows is None else (lambda t: t[rows].cpu())
    eps = f32(w.eps)
    torch.cuda.synchronize()

    y = nrs.rmsnorm(x, gamma, w.eps)
    check(f"{tag}/rmsnorm", h_in(y), oracle.rmsnorm(h_in(x), gamma.cpu(), eps))

    y, ro = nrs.add_rmsnorm(x, res, gamma, w.eps)
    ry, rro = oracle.add_rmsnorm(h_in(x), h_in(res), gamma.cpu(), eps)
    check_exact(f"{tag}/add_rmsnorm.residual_out", h_in(ro), rro)
    check(f"{tag}/add_rmsnorm.y", h_in(y), ry)

    q0, k0 = h_in(q), h_in(k)
    nrs.mrope(q, k, pos, w.sections, w.theta)
    p_sel = w.pos.cpu() if rows is None else w.pos.cpu()[:, rows.cpu()].contiguous()
    rq, rk = oracle.mrope(q0, k0, p_sel, w.sections, w.theta)
    check(f"{tag}/mrope.q", h_in(q), rq, pairs=True)
    check(f"{tag}/mrope.k", h_in(k), rk, pairs=True)

    out = nrs.swiglu(gu)
    check(f"{tag}/swiglu", h_in(out), oracle.swiglu(h_in(gu)))


# ------------------------------------------------------------ the workloads

def test_tiny_layer_f32():
    w = W.tiny()
    layer_parity(w, w.layer, "tiny_f32")


def test_decode_step_all_layers():
    w = W.decode(n_layers=28, second_norm=True)
    for li, L in enumerate(w.layers):
        layer_parity(w, L, f"decode/L{li}")
        # the post-attention norm of the four-op layer
        y, ro = nrs.add_rmsnorm(cuda(L.x2), cuda(L.residual), cuda(L.gamma2), w.eps)
        ry, rro = oracle.add_rmsnorm(L.x2, L.residual, L.gamma2, f32(w.eps))
        check_exact(f"decode/L{li}/post_norm.residual_out", ro, rro)
        check(f"decode/L{li}/post_norm.y", y, ry)


def test_prefill_outliers_and_streams():
    w = W.prefill()
    assert not torch.equal(w.pos[0], w.pos[1])   # distinct t and h/w streams
    layer_parity(w, w.layer, "prefill")


def test_ragged_packed_batch():
    w = W.ragged(device="cuda")
    layer_parity(w, w.layer, "ragged")


def test_ragged_rows_stay_local():
    # perturbing one token changes that token's outputs only
    w = W.ragged(n_seqs=8, device="cuda")
    L = w.layer
    t = w.seq_lens[0] + w.seq_lens[1] - 1          # last token of sequence 1
    outs = []
    for bump in (False, True):
        x, q, k, gu = L.x.clone(), L.q.clone(), L.k.clone(), L.gate_up.clone()
        pos = w.pos.clone()
        if bump:
            x[t] += 1.0
            q[t] += 1.0
            k[t] += 1.0
            gu[t] += 1.0
            pos[:, t] += 3
        y, ro = nrs.add_rmsnorm(x, L.residual, L.gamma, w.eps)
        nrs.mrope(q, k, pos, w.sections, w.theta)
        outs.append((y, ro, q, k, nrs.swiglu(gu)))
    for a, b in zip(*outs):
        diff = (a != b).reshape(a.shape[0], -1).any(dim=1)
        assert diff[t] and int(diff.sum()) == 1


SWEEP_H = [512, 1024, 1536, 2048, 4096]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hidden", SWEEP_H)
@pytest.mark.parametrize("head_dim", [64, 128])
def test_sweep_reduced_tokens(dtype, hidden, head_dim):
    w = W.sweep(dtype=dtype, hidden=hidden, head_dim=head_dim, tokens=333)
    layer_parity(w, w.layer, f"sweep333/{dtype}/h{hidden}/d{head_dim}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hidden", SWEEP_H)
@pytest.mark.parametrize("eps", [1e-6, 1e-5])
def test_sweep_scaled_rows(dtype, hidden, eps):
    w = W.sweep(dtype=dtype, hidden=hidden, head_dim=128, tokens=257, scaled=True, eps=eps)
    layer_parity(w, w.layer, f"scaled257/{dtype}/h{hidden}/eps{eps}")


def _sample_rows(T, n=48, seed=0):
    g = torch.Generator().manual_seed(seed)
    idx = torch.cat([torch.tensor([0, 1, T // 2, T - 2, T - 1]), torch.randint(0, T, (n,), generator=g)])
    return torch.unique(idx).to("cuda")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hidden", SWEEP_H)
def test_sweep_full_size_sampled(dtype, hidden):
    # the full 32768-token launches (the benchmark's configuration), checked on sampled rows
    w = W.sweep(dtype=dtype, hidden=hidden, head_dim=128, tokens=32768, device="cuda")
    layer_parity(w, w.layer, f"sweep32k/{dtype}/h{hidden}", rows=_sample_rows(32768))


def test_sweep_full_size_scaled_sampled():
    w = W.sweep(dtype="bf16", hidden=2048, head_dim=128, tokens=32768, scaled=True,
                eps=1e-5, device="cuda")
    layer_parity(w, w.layer, "sweep32k_scaled/bf16/h2048", rows=_sample_rows(32768, seed=1))


# ------------------------------------------------------------ edge cases

def _rand(shape, dt, seed=0, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float64) * scale).to(torch.float32).to(dt)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("hidden", [8, 64, 520, 1032, 8 * (3 * 64 + 5), 4096 + 8, 8192, 16384,
                                    65536])
def test_norm_widths(dt, hidden):
    # lane tails, every wave-path width class (bf16 rows with a residual of
    # 65-256 chunks: one wave per row, 2 or 4 chunks per thread, part-empty
    # last chunk), and the block-per-row path
    if dt == torch.float32 and hidden > 32768:
        hidden = 32768
    rows = 37
    x, r = _rand((rows, hidden), dt, 1), _rand((rows, hidden), dt, 2)
    gamma = (1 + 0.1 * _rand((hidden,), torch.float32, 3)).to(dt)
    y = nrs.rmsnorm(cuda(x), cuda(gamma), 1e-6)
    check(f"width{hidden}/rmsnorm", y, oracle.rmsnorm(x, gamma, f32(1e-6)))
    y, ro = nrs.add_rmsnorm(cuda(x), cuda(r), cuda(gamma), 1e-6)
    ry, rro = oracle.add_rmsnorm(x, r, gamma, f32(1e-6))
    check_exact(f"width{hidden}/add.residual_out", ro, rro)
    check(f"width{hidden}/add.y", y, ry)


@pytest.mark.parametrize("dt,rows,hidden", [(torch.bfloat16, 2051, 3080), (torch.bfloat16, 2048, 4096),
                                             (torch.bfloat16, 4099, 1544), (torch.float32, 2051, 1540),
                                             (torch.float32, 2051, 1000)])
def test_norm_streaming_shapes(dt, rows, hidden):
    # streaming-size calls (>= 16 MiB) in the shapes chosen for them: bf16 rows of 257-512
    # chunks over 2 waves x 4 chunks and fp32 ones over one wave x 8 (RMSNorm, calls up to
    # 32 MiB), rows of 65-256 chunks over one wave (with the residual add), part-filled
    # chunk groups and blocks
    x, r = _rand((rows, hidden), dt, 21), _rand((rows, hidden), dt, 22)
    gamma = (1 + 0.1 * _rand((hidden,), torch.float32, 23)).to(dt)
    y = nrs.rmsnorm(cuda(x), cuda(gamma), 1e-6)
    check(f"stream{rows}x{hidden}/rmsnorm", y, oracle.rmsnorm(x, gamma, f32(1e-6)))
    y, ro = nrs.add_rmsnorm(cuda(x), cuda(r), cuda(gamma), 1e-6)
    ry, rro = oracle.add_rmsnorm(x, r, gamma, f32(1e-6))
    check_exact(f"stream{rows}x{hidden}/add.residual_out", ro, rro)
    check(f"stream{rows}x{hidden}/add.y", y, ry)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("hidden", [16, 40, 128, 136, 256])
@pytest.mark.parametrize("rows", [1, 37, 1000])
def test_norm_short_rows_share_waves(dt, hidden, rows):
    # rows of at most 32 chunks take an aligned lane group each, several per wave
    if dt == torch.float32 and hidden == 136:
        hidden = 132
    x, r = _rand((rows, hidden), dt, 11), _rand((rows, hidden), dt, 12)
    gamma = (1 + 0.1 * _rand((hidden,), torch.float32, 13)).to(dt)
    y = nrs.rmsnorm(cuda(x), cuda(gamma), 1e-6)
    check(f"short{hidden}x{rows}/rmsnorm", y, oracle.rmsnorm(x, gamma, f32(1e-6)))
    y, ro = nrs.add_rmsnorm(cuda(x), cuda(r), cuda(gamma), 1e-6)
    ry, rro = oracle.add_rmsnorm(x, r, gamma, f32(1e-6))
    check_exact(f"short{hidden}x{rows}/add.residual_out", ro, rro)
    check(f"short{hidden}x{rows}/add.y", y, ry)


def test_per_head_norm_shape():
    # a per-head RMSNorm over head_dim 128: 2048 tokens x 16 heads as 32768 rows of 128,
    # strided inside a packed qkv row (token stride 32 heads x 128)
    big = _rand((2048, 32 * 128), torch.bfloat16, 14)
    q = cuda(big)[:, : 16 * 128].reshape(2048, 16, 128)
    gamma = (1 + 0.1 * _rand((128,), torch.float32, 15)).to(torch.bfloat16)
    y = nrs.rmsnorm(q.reshape(-1, 128) if q.is_contiguous() else q.contiguous().view(-1, 128),
                    cuda(gamma), 1e-6)
    ref = oracle.rmsnorm(big[:, : 16 * 128].reshape(-1, 128).contiguous(), gamma, f32(1e-6))
    check("per_head128/rmsnorm", y, ref)


@pytest.mark.parametrize("rows", [1, 3, 4, 5, 4095, 9000])
def test_norm_row_counts(rows):
    x = _rand((rows, 2048), torch.bfloat16, rows)
    gamma = (1 + 0.1 * _rand((2048,), torch.float32, 5)).to(torch.bfloat16)
    y = nrs.rmsnorm(cuda(x), cuda(gamma), 1e-5)
    check(f"rows{rows}/rmsnorm", y, oracle.rmsnorm(x, gamma, f32(1e-5)))


def test_empty_calls_launch_nothing():
    e = torch.empty(0, 256, device="cuda", dtype=torch.bfloat16)
    g = torch.ones(256, device="cuda", dtype=torch.bfloat16)
    assert nrs.rmsnorm(e, g).shape == (0, 256)
    y, ro = nrs.add_rmsnorm(e, e.clone(), g)
    assert y.shape == (0, 256)
    assert nrs.swiglu(torch.empty(0, 512, device="cuda", dtype=torch.bfloat16)).shape == (0, 256)
    q = torch.empty(0, 4, 64, device="cuda", dtype=torch.bfloat16)
    nrs.mrope(q, q.clone(), torch.zeros(3, 1, dtype=torch.int32, device="cuda"), (8, 12, 12))
    torch.cuda.synchronize()


def test_rmsnorm_strided_rows_and_in_place():
    big = _rand((50, 3072), torch.bfloat16, 7)
    gamma = (1 + 0.1 * _rand((2048,), torch.float32, 8)).to(torch.bfloat16)
    xd = cuda(big)[:, 512:2560]                      # rows of stride 3072
    y = nrs.rmsnorm(xd, cuda(gamma), 1e-6)
    check("strided/rmsnorm", y, oracle.rmsnorm(big[:, 512:2560], gamma, f32(1e-6)))
    out = torch.full((50, 4096), 7.0, dtype=torch.bfloat16, device="cuda")[:, 1024:3072]
    nrs.rmsnorm(xd, cuda(gamma), 1e-6, out=out)      # strided output rows too
    check_exact("strided/rmsnorm.out", out, y.cpu())
    z = xd.contiguous()
    nrs.rmsnorm(z, cuda(gamma), 1e-6, out=z)          # y == x
    check_exact("in_place/rmsnorm", z, y.cpu())


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_add_rmsnorm_in_place(dt):
    x, r = _rand((300, 1536), dt, 9), _rand((300, 1536), dt, 10)
    gamma = (1 + 0.1 * _rand((1536,), torch.float32, 11)).to(dt)
    y, ro = nrs.add_rmsnorm(cuda(x), cuda(r), cuda(gamma), 1e-6)
    xd, rd = cuda(x), cuda(r)
    nrs.add_rmsnorm(xd, rd, cuda(gamma), 1e-6, out=xd, residual_out=rd)
    check_exact("in_place/add.y", xd, y.cpu())
    check_exact("in_place/add.residual_out", rd, ro.cpu())


def test_mrope_packed_qkv_streams_and_extremes():
    T, nq, nkv, D = 131, 16, 8, 128
    qkv = _rand((T, (nq + 2 * nkv) * D), torch.bfloat16, 12)
    g = torch.Generator().manual_seed(13)
    pos = torch.randint(-5000, 5000, (3, T), generator=g, dtype=torch.int32)
    pos[:, :3] = torch.tensor([[0, (1 << 24) - 1, -(1 << 24) + 1]] * 3, dtype=torch.int32)
    pos_wide = torch.zeros(3, T + 9, dtype=torch.int32)
    pos_wide[:, :T] = pos
    d = cuda(qkv)
    q = d[:, : nq * D].view(T, nq, D)
    k = d[:, nq * D : (nq + nkv) * D].view(T, nkv, D)
    v_before = d[:, (nq + nkv) * D :].clone()
    nrs.mrope(q, k, cuda(pos_wide)[:, :T], (16, 24, 24), 1e6)
    rq, rk = oracle.mrope(qkv[:, : nq * D].view(T, nq, D), qkv[:, nq * D : (nq + nkv) * D].view(T, nkv, D),
                          pos, (16, 24, 24), 1e6)
    check("qkv/mrope.q", q, rq, pairs=True)
    check("qkv/mrope.k", k, rk, pairs=True)
    assert torch.equal(d[:, (nq + nkv) * D :], v_before)     # v untouched


@pytest.mark.parametrize("dt,D", [(torch.bfloat16, 64), (torch.float32, 32), (torch.bfloat16, 16)])
def test_mrope_narrow_heads_in_packed_qkv(dt, D):
    # narrow half-heads (chunk per lane, partner swizzled in) inside a packed qkv row, with
    # the extreme positions; v must stay untouched
    T, nq, nkv = 45, 6, 2
    sec = (D // 8, D // 8, D // 2 - D // 4)
    qkv = _rand((T, (nq + 2 * nkv) * D), dt, 41)
    g = torch.Generator().manual_seed(42)
    pos = torch.randint(-5000, 5000, (3, T), generator=g, dtype=torch.int32)
    pos[:, :3] = torch.tensor([[0, (1 << 24) - 1, -(1 << 24) + 1]] * 3, dtype=torch.int32)
    d = cuda(qkv)
    q = d[:, : nq * D].view(T, nq, D)
    k = d[:, nq * D : (nq + nkv) * D].view(T, nkv, D)
    v_before = d[:, (nq + nkv) * D :].clone()
    nrs.mrope(q, k, cuda(pos), sec, 1e6)
    rq, rk = oracle.mrope(qkv[:, : nq * D].view(T, nq, D), qkv[:, nq * D : (nq + nkv) * D].view(T, nkv, D),
                          pos, sec, 1e6)
    check(f"qkv_narrow{D}/mrope.q", q, rq, pairs=True)
    check(f"qkv_narrow{D}/mrope.k", k, rk, pairs=True)
    assert torch.equal(d[:, (nq + nkv) * D :], v_before)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D,sec,nq,nkv", [(16, (2, 3, 3), 3, 0), (32, (4, 6, 6), 2, 3),
                                          (48, (8, 8, 8), 3, 1), (64, (32, 0, 0), 1, 1),
                                          (64, (8, 12, 12), 100, 40), (128, (0, 0, 64), 2, 5),
                                          (256, (32, 48, 48), 4, 2), (512, (64, 96, 96), 2, 1)])
def test_mrope_shapes(dt, D, sec, nq, nkv):
    # power-of-two half-heads of up to 32 chunks take one lane per chunk with the partner
    # chunk swizzled in from another lane (waves straddling tokens where a token's heads
    # are not whole waves); fp32 D 512 and D 48 the thread-per-pair kernel; 140 heads of
    # 64 give more chunks per token than a block has threads
    T = 77
    q, k = _rand((T, nq, D), dt, 14), _rand((T, max(nkv, 0), D), dt, 15)
    g = torch.Generator().manual_seed(16)
    pos = torch.randint(0, 40000, (3, T), generator=g, dtype=torch.int32)
    qd, kd = cuda(q), cuda(k)
    nrs.mrope(qd, kd, cuda(pos), sec, 1e4)
    rq, rk = oracle.mrope(q, k, pos, sec, 1e4)
    check(f"mrope{D}/q", qd, rq, pairs=True)
    if nkv:
        check(f"mrope{D}/k", kd, rk, pairs=True)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_mrope_narrow_heads_streaming(dt):
    # a streaming-size call (>= 16 MiB: several tokens per block, nontemporal) with
    # head_dim 64, 8 q / 4 kv heads, and a part-filled last block, checked on sampled tokens
    T, nq, nkv, D = 16384 + 4, 8, 4, 64
    q, k = _rand((T, nq, D), dt, 31), _rand((T, nkv, D), dt, 32)
    pos = torch.arange(T, dtype=torch.int32).repeat(3, 1).contiguous()
    qd, kd = cuda(q), cuda(k)
    nrs.mrope(qd, kd, cuda(pos), (8, 12, 12), 1e6)
    g = torch.Generator().manual_seed(33)
    sel = torch.cat([torch.arange(8), torch.arange(T - 8, T), torch.randint(0, T, (200,), generator=g)])
    rq, rk = oracle.mrope(q[sel].contiguous(), k[sel].contiguous(), pos[:, sel].contiguous(),
                          (8, 12, 12), 1e6)
    check("mrope_narrow_stream/q", qd.cpu()[sel], rq, pairs=True)
    check("mrope_narrow_stream/k", kd.cpu()[sel], rk, pairs=True)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_swiglu_extreme_gates(dt):
    gates = [0.0, -0.0, 1.0, -1.0, 20.0, 100.0, 1e4, -20.0, -79.9, -80.0, -80.1, -87.0, -88.8,
             -89.0, -95.0, -100.0, -104.0, -110.0, -120.0, -149.9, -150.0, -150.1, -180.0,
             -200.0, -213.9, -214.0, -214.1, -300.0, -1e4, 3.0e38 / 1e30]
    ups = [1.0, -1.0, 1e3, 1e10, 1e30, 2.0**-20, -3.5e3]
    G = torch.tensor([g for g in gates for _ in ups], dtype=torch.float64)
    U = torch.tensor([u for _ in gates for u in ups], dtype=torch.float64)
    n = G.numel()
    pad = (-n) % 8
    G = torch.cat([G, torch.zeros(pad, dtype=torch.float64)])
    U = torch.cat([U, torch.ones(pad, dtype=torch.float64)])
    gu = torch.cat([G, U]).to(torch.float32).to(dt).view(1, -1)
    out = nrs.swiglu(cuda(gu))
    check(f"swiglu_extremes/{dt}", out, oracle.swiglu(gu))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_swiglu_gate_sweep_no_low_gate(dt):
    # chunks whose gates are all >= -80 take the kernel's branch-free path
    # (a hardware base-2 exponential on an exactly split exponent): a dense
    # sweep of that range, its edge at -80 and just above, large and
    # infinite gates (clamped there), and a NaN gate, each in chunks with no
    # gate below -80
    rng = np.random.default_rng(23)
    n = 1 << 16
    g = np.linspace(-80.0, 100.0, n)
    edge = np.array([-80.0, np.nextafter(np.float32(-80.0), np.float32(0)), -79.5, 100.0,
                     np.nextafter(np.float32(100.0), np.float32(200)), 150.0, 1e4, 3e38,
                     np.inf, np.nan, 0.0, -0.0, 1e-30, -1e-30, 88.7, 89.0, 104.0, 127.0])
    edge = np.repeat(edge, 8)            # whole chunks of one gate in either dtype
    G = np.concatenate([g, edge])
    U = rng.uniform(-1.0, 1.0, G.size)     # |g u| stays inside fp32's range
    U[:n] = rng.standard_normal(n) * np.exp(rng.uniform(-20.0, 20.0, n))
    U[:1024] = 1.0
    gu = torch.from_numpy(np.concatenate([G, U])).to(torch.float32).to(dt).view(1, -1)
    out = nrs.swiglu(cuda(gu))
    check(f"swiglu_sweep/{dt}", out, oracle.swiglu(gu))


def test_swiglu_strided_rows():
    big = _rand((40, 2 * 768 + 64), torch.bfloat16, 17, scale=4.0)
    gu = cuda(big)[:, 32 : 32 + 1536]
    out = torch.zeros(40, 1024, dtype=torch.bfloat16, device="cuda")[:, 128:896]
    nrs.swiglu(gu, out=out)
    check("strided/swiglu", out, oracle.swiglu(big[:, 32 : 32 + 1536]))


# ------------------------------------------------------------ decode graph

def _decode_buffers(w, four_op):
    layers = []
    R = cuda(w.layers[0].residual)
    for L in w.layers:
        d = {"in_x": cuda(L.x), "in_residual": R, "in_gamma": cuda(L.gamma),
             "in_y": torch.empty_like(cuda(L.x)), "in_residual_out": torch.empty_like(R),
             "q": cuda(L.q), "k": cuda(L.k), "gate_up": cuda(L.gate_up),
             "act_out": torch.empty(w.tokens, w.inter, dtype=L.x.dtype, device="cuda")}
        R = d["in_residual_out"]
        if four_op:
            d.update(post_x=cuda(L.x2), post_residual=R, post_gamma=cuda(L.gamma2),
                     post_y=torch.empty_like(R), post_residual_out=torch.empty_like(R))
            R = d["post_residual_out"]
        layers.append(d)
    return layers


@pytest.mark.parametrize("four_op", [False, True])
def test_decode_graph_matches_eager_and_oracle(four_op):
    w = W.decode(n_layers=28, second_norm=True)
    pos = cuda(w.pos)
    eager = _decode_buffers(w, four_op)
    for d in eager:   # the same calls, one by one, on torch's stream
        nrs.add_rmsnorm(d["in_x"], d["in_residual"], d["in_gamma"], w.eps, out=d["in_y"],
                        residual_out=d["in_residual_out"])
        nrs.mrope(d["q"], d["k"], pos, w.sections, w.theta)
        if four_op:
            nrs.add_rmsnorm(d["post_x"], d["post_residual"], d["post_gamma"], w.eps,
                            out=d["post_y"], residual_out=d["post_residual_out"])
        nrs.swiglu(d["gate_up"], out=d["act_out"])
    bufs = _decode_buffers(w, four_op)
    g = nrs.decode_graph(bufs, pos, w.sections, w.theta, w.eps)
    assert g.nodes == (4 if four_op else 3) * 28
    g.launch()
    torch.cuda.synchronize()
    for a, b in zip(eager, bufs):
        for key in ("in_y", "in_residual_out", "q", "k", "act_out") + (
                ("post_y", "post_residual_out") if four_op else ()):
            assert torch.equal(a[key], b[key]), key
    # the residual chain through all layers, against the oracle
    R = w.layers[0].residual
    for li, (L, b) in enumerate(zip(w.layers, bufs)):
        ry, R = oracle.add_rmsnorm(L.x, R, L.gamma, f32(w.eps))
        check_exact(f"graph/L{li}/residual_out", b["in_residual_out"], R)
        check(f"graph/L{li}/y", b["in_y"], ry)
        if four_op:
            ry, R = oracle.add_rmsnorm(L.x2, R, L.gamma2, f32(w.eps))
            check_exact(f"graph/L{li}/post_residual_out", b["post_residual_out"], R)
            check(f"graph/L{li}/post_y", b["post_y"], ry)
        rq, rk = oracle.mrope(L.q, L.k, w.pos, w.sections, w.theta)
        check(f"graph/L{li}/q", b["q"], rq, pairs=True)
        check(f"graph/L{li}/k", b["k"], rk, pairs=True)
        check(f"graph/L{li}/act", b["act_out"], oracle.swiglu(L.gate_up))
    # replays re-run the same nodes: norm and swiglu outputs are unchanged, and
    # q/k turn once more per replay (eager again for comparison)
    y0 = [b["in_y"].clone() for b in bufs]
    for _ in range(3):
        g.launch()
        torch.cuda.synchronize()
        for d in eager:
            nrs.mrope(d["q"], d["k"], pos, w.sections, w.theta)
    torch.cuda.synchronize()
    for a, b, y in zip(eager, bufs, y0):
        assert torch.equal(b["in_y"], y)
        assert torch.equal(a["q"], b["q"]) and torch.equal(a["k"], b["k"])
    g.close()


def test_null_graph():
    g = nrs.null_graph(84)
    assert g.nodes == 84
    for _ in range(3):
        g.launch()
    torch.cuda.synchronize()
    g.close()
