"""The calibration kernel (nrs_stream_probe) writes what its header says, in
every variant, at cached and streaming sizes and with a ragged last
workgroup; and M-RoPE on tokens whose rows are 4 MiB apart (a streaming call
of 8 tokens) stays in parity with the oracle."""
from __future__ import annotations

import pytest
import torch

import norm_rope_swiglu_amd as nrs
import oracle
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    nrs.lib()


def _words(nbytes, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), generator=g, dtype=torch.int32)


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
@pytest.mark.parametrize("nbytes", [16, 1024 + 48, 3 << 20, (24 << 20) + 16 * 37])
@pytest.mark.parametrize("n_read,n_write", [(0, 1), (0, 2), (1, 0), (1, 1), (1, 2), (2, 0), (2, 1),
                                            (2, 2)])
def test_stream_probe_outputs(nbytes, n_read, n_write, variant):
    src = [_words(nbytes, 7 + i) for i in range(n_read)]
    dsrc = [s.cuda() for s in src]
    ddst = [torch.full((nbytes // 4,), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
            for _ in range(n_write)]
    nrs.stream_probe(n_read, n_write, dsrc, ddst, nbytes, variant)
    torch.cuda.synchronize()
    got = [d.cpu() for d in ddst]
    if n_read == 0:
        # the counter pattern: chunk i holds (i mod 2^32, i >> 32, 0x5A5A5A5A, 0xA5A5A5A5)
        i = torch.arange(nbytes // 16, dtype=torch.int64)
        want0 = torch.stack([i & 0xFFFFFFFF, i >> 32, torch.full_like(i, 0x5A5A5A5A),
                             torch.full_like(i, 0xA5A5A5A5)], dim=1).reshape(-1)
        want0 = (want0 - ((want0 >> 31) << 32)).to(torch.int32)     # as signed 32-bit words
    else:
        want0 = src[0] if n_read == 1 else src[0] ^ src[1]
    if n_write >= 1:
        assert torch.equal(got[0], want0)
    if n_write == 2:
        assert torch.equal(got[1], ~(src[0] if n_read >= 1 else want0))
    for s, d in zip(src, dsrc):      # sources are only read
        assert torch.equal(d.cpu(), s)


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("kib,rows", [(1, 5), (2, 3), (3, 9), (4, 7), (6, 2), (8, 5), (12, 1),
                                      (16, 6), (4, 4096 + 3)])
@pytest.mark.parametrize("n", [1, 2])
def test_stream_probe_rows(kib, rows, n, variant):
    nbytes = rows * kib * 1024
    src = [_words(nbytes, 20 + i) for i in range(n)]
    ddst = [torch.full((nbytes // 4,), 0x3C3C3C3C, dtype=torch.int32, device="cuda")
            for _ in range(n)]
    nrs.stream_probe(n, n, [t.cuda() for t in src], ddst, nbytes, variant, row_bytes=kib * 1024)
    torch.cuda.synchronize()
    assert torch.equal(ddst[0].cpu(), src[0] if n == 1 else src[0] ^ src[1])
    if n == 2:
        assert torch.equal(ddst[1].cpu(), ~src[0])


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("row_bytes,rows", [(16, 7), (1008, 3), (16384 * 16 + 48, 2),
                                            (151936 * 2, 5), (8 * 1024 * 16, 3)])
def test_stream_probe_row_read(row_bytes, rows, variant):
    # the row-granular read (the sampler's shape) completes, leaves its source
    # untouched and writes nothing: rows shorter than, equal to and longer than
    # the 8 chunks per thread it issues first, with a partial last batch
    nbytes = rows * row_bytes
    src = _words(nbytes, 31)
    d = src.cuda()
    nrs.stream_probe(1, 0, [d], [], nbytes, variant, row_bytes=row_bytes)
    torch.cuda.synchronize()
    assert torch.equal(d.cpu(), src)


def test_stream_probe_empty_call():
    nrs.stream_probe(1, 1, [torch.empty(16, dtype=torch.uint8, device="cuda")],
                     [torch.empty(16, dtype=torch.uint8, device="cuda")], 0)


def test_mrope_wide_token_stride():
    # 8 tokens whose q rows are 4 MiB apart; 25 MB of q and k are moved, above
    # the streaming threshold
    T, nq, nkv, D = 8, 4096, 2048, 128
    qs = (1 << 21) + 64                      # elements per token row of q (bf16: ~4 MiB)
    g = torch.Generator().manual_seed(3)
    qbuf = (torch.randn(T, qs, generator=g) * 1.0).to(torch.bfloat16)
    k = torch.randn(T, nkv, D, generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 30000, (3, T), generator=g, dtype=torch.int32)
    dq = qbuf.cuda()
    q = dq[:, : nq * D].view(T, nq, D)
    dk = k.cuda()
    nrs.mrope(q, dk, pos.cuda(), (16, 24, 24), 1e6)
    rq, rk = oracle.mrope(qbuf[:, : nq * D].view(T, nq, D), k, pos, (16, 24, 24), 1e6)
    check("mrope/wide-stride.q", q, rq, pairs=True)
    check("mrope/wide-stride.k", dk, rk, pairs=True)
    # the rest of each q row is untouched
    assert torch.equal(dq[:, nq * D:].cpu(), qbuf[:, nq * D:])
