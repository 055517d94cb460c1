"""GPU parity of the fused RMSNorm + Linear (through the C ABI) against the
fp64 oracle: decode-sized rows at the projection shapes of the decode step,
row counts across the 16-row tiles and 64-row launches, input widths with
ragged matrix-core steps, output widths off the 16-column tiles, strided
operands, eps-dominated and zero rows, and sampled rows of a prefill-sized
call."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import norm_rope_swiglu_amd as nrs
import oracle
import workloads as W
from numerics import dot_scale
from parity import check

pytestmark = pytest.mark.gpu

U = 2.0**-24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    nrs.lib()


def _f32(v):
    return float(np.float32(v))


def lin_inputs(rows, n_in, n_out, dt, seed=0, x_scale=1.0):
    """x rows with their own scales; w ~ N(0, 1/n_in) so outputs are O(1)."""
    def key(n):
        return W.stream_key(seed, f"lin/{n}/{rows}/{n_in}/{n_out}")
    sc = torch.exp(W.normal(key("s"), rows).reshape(rows, 1)) * x_scale
    x = W.normal(key("x"), rows * n_in).reshape(rows, n_in) * sc
    w = W.normal(key("w"), n_out * n_in).reshape(n_out, n_in) / np.sqrt(n_in)
    return W.store(x, dt), W.store(w, dt)


def lin_parity(x, w, eps, tag, rows=None, out=None):
    """Run nrs.rmsnorm_linear on the GPU (all rows of x) and compare all rows,
    or the sampled `rows`, with the oracle under the fp32 chain bound."""
    xd, wd = x.cuda(), w.cuda()
    y = nrs.rmsnorm_linear(xd, wd, eps, out=out)
    torch.cuda.synchronize()
    y = y.cpu()
    sel = slice(None) if rows is None else rows
    xs = x[sel].contiguous() if x.stride(1) == 1 and rows is not None else x[sel]
    ref = oracle.rmsnorm_linear(xs, w, _f32(eps))
    xw = oracle.widen(xs.contiguous()).reshape(xs.shape)
    ww = oracle.widen(w.contiguous()).reshape(w.shape)
    n_in = x.shape[1]
    bound = (n_in / 8 + 64) * U
    check(tag, y[sel], ref, scale=dot_scale(xw, ww, _f32(eps)), tol=bound, abs_frac=bound)
    return y


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n_out", [4096, 12288, 3072])
def test_decode_projections(dt, n_out):
    # 5 sequences x 1 token, hidden 2048: qkv (16 + 8 + 8 heads x 128), gate_up (2 x 6144),
    # and a 3072-entry codec head
    x, w = lin_inputs(5, 2048, n_out, dt, 1)
    lin_parity(x, w, 1e-6, f"lin/{dt}/5x2048x{n_out}")


@pytest.mark.parametrize("rows", [1, 15, 16, 17, 31, 32, 33, 48, 64, 65, 130])
def test_row_counts(rows):
    # 16-row tiles (1, 2 or 4 per launch) and 64-row launches
    x, w = lin_inputs(rows, 256, 100, "bf16", 2)
    lin_parity(x, w, 1e-5, f"lin/rows{rows}")


@pytest.mark.parametrize("dt,n_in", [("bf16", 8), ("bf16", 24), ("bf16", 40), ("bf16", 264),
                                     ("bf16", 1600), ("bf16", 8192), ("f32", 4), ("f32", 12),
                                     ("f32", 20), ("f32", 1028), ("f32", 4096)])
def test_input_widths(dt, n_in):
    # widths that leave a partial matrix-core step and uneven wave shares
    x, w = lin_inputs(7, n_in, 48, dt, 3)
    lin_parity(x, w, 1e-6, f"lin/{dt}/in{n_in}")


@pytest.mark.parametrize("n_out", [1, 15, 17, 33, 250])
def test_output_widths(n_out):
    x, w = lin_inputs(9, 512, n_out, "bf16", 4)
    lin_parity(x, w, 1e-6, f"lin/out{n_out}")


@pytest.mark.parametrize("rows,n_in,n_out", [(1, 8, 1), (3, 4096, 40), (4, 2056, 9), (8, 800, 17),
                                             (8, 2048, 7), (2, 520, 4099),
                                             (1, 8192, 33), (2, 6144, 70), (1, 16384, 9),
                                             (3, 5456, 17), (1, 12296, 5), (2, 4104, 12),
                                             (1, 4104, 3), (1, 2048, 8200), (8, 1600, 8197),
                                             (3, 1032, 8195), (5, 2048, 8192)])
def test_gemv_shapes(rows, n_in, n_out):
    # bf16 decode rows (<= 8, x within 2048 chunks): one wave per pair of weight rows,
    # 1, 2, 4 or 8 chunks per lane with part-filled last chunk groups, blocks of 8 weight
    # rows with part-filled last blocks, and the largest x staged in LDS; rows of more
    # than 512 chunks (over 4096 inputs) in 2, 3 or 4 passes of 8 chunks per lane, with
    # part-filled last passes; outputs from 8192 on at 1032-2048 inputs take 8-wave blocks
    # (16 weight rows a block), with part-filled last blocks
    x, w = lin_inputs(rows, n_in, n_out, "bf16", 11)
    lin_parity(x, w, 1e-6, f"lin/gemv/{rows}x{n_in}x{n_out}")


def test_gemv_strided_operands():
    xb, wb = lin_inputs(6, 640, 96, "bf16", 12)
    x, w = xb[:, 64:576], wb[:, 128:640]            # rows of stride 640, 512 wide
    y = lin_parity(x, w, 1e-6, "lin/gemv/strided")
    big = torch.zeros(6, 128, dtype=x.dtype, device="cuda")
    nrs.rmsnorm_linear(x.cuda(), w.cuda(), 1e-6, out=big[:, 16:112])
    torch.cuda.synchronize()
    assert torch.equal(big[:, 16:112].cpu(), y)
    assert torch.all(big[:, :16] == 0) and torch.all(big[:, 112:] == 0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_strided_operands(dt):
    xb, wb = lin_inputs(12, 640, 96, dt, 5)
    x, w = xb[:, 64:576], wb[:, 128:640]            # rows of stride 640, 512 wide
    y = lin_parity(x, w, 1e-6, f"lin/{dt}/strided")
    # a strided output: rows of stride 128 in a wider buffer
    big = torch.zeros(12, 128, dtype=x.dtype, device="cuda")
    nrs.rmsnorm_linear(x.cuda(), w.cuda(), 1e-6, out=big[:, 16:112])
    torch.cuda.synchronize()
    assert torch.equal(big[:, 16:112].cpu(), y)
    assert torch.all(big[:, :16] == 0) and torch.all(big[:, 112:] == 0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_eps_dominated_and_zero_rows(dt):
    # mean(x^2) ~ 1e-4 against eps = 0.5: dropping eps or the mean changes every output
    x, w = lin_inputs(6, 1024, 64, dt, 6, x_scale=0.01)
    x[2] = 0                                              # zero row: output exactly 0
    y = lin_parity(x, w, 0.5, f"lin/{dt}/eps")
    assert torch.all(y[2] == 0)
    lin_parity(x, w, 0.0, f"lin/{dt}/eps0_nonzero_rows", rows=torch.tensor([0, 1, 3, 4, 5]))


@pytest.mark.parametrize("rows,n_in,n_out", [(65, 64, 128), (129, 200, 200), (300, 1000, 130),
                                             (257, 8, 16), (512, 2048, 384)])
def test_gemm_tile_tails(rows, n_in, n_out):
    # the many-row (tiled) path: row, input and output counts off the 128 x 128 x 64 tiles
    x, w = lin_inputs(rows, n_in, n_out, "bf16", 10)
    lin_parity(x, w, 1e-6, f"lin/gemm/{rows}x{n_in}x{n_out}")


def test_gemm_big_tiles_with_tails():
    # >= 256 tiles of 256 x 256 (the large-tile path), row and column counts off the tile
    x, w = lin_inputs(4100, 1000, 4100, "bf16", 12)
    g = torch.Generator().manual_seed(13)
    rows = torch.unique(torch.cat([torch.tensor([0, 255, 256, 4095, 4096, 4099]),
                                   torch.randint(0, 4100, (40,), generator=g)]))
    lin_parity(x, w, 1e-6, "lin/gemm/big4100", rows=rows)


@pytest.mark.parametrize("n_in", [8, 40, 72, 104, 168, 232, 264])
def test_gemm_big_tiles_short_inputs(n_in):
    # the large-tile path with 1-9 stages of 32 inputs: fewer stages than the
    # ring's prologue fills, the tail alone, and one steady pass before it
    x, w = lin_inputs(4096, n_in, 4096, "bf16", 16)
    g = torch.Generator().manual_seed(17)
    rows = torch.unique(torch.cat([torch.tensor([0, 255, 256, 4095]),
                                   torch.randint(0, 4096, (12,), generator=g)]))
    lin_parity(x, w, 1e-6, f"lin/gemm/big_short{n_in}", rows=rows)


def test_gemm_benchmark_shape_sampled_rows():
    # the benchmark's large GEMM launch: 32768 x 2048 -> 4096 (256 x 256 tiles, 64 stages),
    # 64 rows against the oracle, the first and last of the first and last tiles among them
    x, w = lin_inputs(32768, 2048, 4096, "bf16", 18)
    g = torch.Generator().manual_seed(19)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, 255, 256, 32511, 32512, 32766, 32767]),
                                   torch.randint(0, 32768, (56,), generator=g)]))
    lin_parity(x, w, 1e-6, "lin/gemm/bench32768", rows=rows)


def test_gemm_strided_operands():
    xb, wb = lin_inputs(200, 640, 96, "bf16", 11)
    lin_parity(xb[:, 64:576], wb[:, 128:640], 1e-6, "lin/gemm/strided")


def test_wide_vocab_head():
    x, w = lin_inputs(2, 1024, 32000, "bf16", 7)
    lin_parity(x, w, 1e-6, "lin/vocab32000")


def test_prefill_sampled_rows():
    # 2048 tokens x 2048 -> 4096 in one call (32 launches of 64 rows); 64 rows checked
    x, w = lin_inputs(2048, 2048, 4096, "bf16", 8)
    g = torch.Generator().manual_seed(9)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, 63, 64, 2046, 2047]),
                                   torch.randint(0, 2048, (58,), generator=g)]))
    lin_parity(x, w, 1e-6, "lin/prefill2048", rows=rows)


def test_empty_and_rejects():
    e = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(64, 256, dtype=torch.bfloat16, device="cuda")
    assert nrs.rmsnorm_linear(e, w).shape == (0, 64)
    with pytest.raises(ValueError):
        nrs.rmsnorm_linear(torch.empty(4, 256, dtype=torch.bfloat16, device="cuda"),
                           torch.empty(64, 128, dtype=torch.bfloat16, device="cuda"))


def test_fp32_many_rows_in_64_row_passes():
    # fp32 rows beyond 64 go through the few-row kernel 64 rows at a time
    x, w = lin_inputs(150, 512, 80, "f32", 14)
    lin_parity(x, w, 1e-6, "lin/f32/rows150")


def test_gemm_long_row_stride():
    # rows 2^22 elements apart exceed the tiled path's 32-bit tile offsets and
    # take the 64-row passes instead; both must agree with the oracle
    x, w = lin_inputs(66, 64, 40, "bf16", 15)
    stride = 1 << 22
    big = torch.zeros(66 * stride, dtype=torch.bfloat16, device="cuda")
    xs = big.as_strided((66, 64), (stride, 1))
    xs.copy_(x.cuda())
    y = nrs.rmsnorm_linear(xs, w.cuda(), 1e-6)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_linear(x, w, _f32(1e-6))
    bound = (64 / 8 + 64) * U
    check("lin/gemm/stride2^22", y.cpu(), ref, scale=dot_scale(oracle.widen(x).reshape(x.shape),
                                                              oracle.widen(w).reshape(w.shape), _f32(1e-6)),
          tol=bound, abs_frac=bound)
