"""GPU parity of the paged split-KV entry point (decode against a paged cache:
"FlashAttention and inference kernels", sections "A paged decode attention
kernel (with GQA)" and "Parallelism during decode: Flash-Decoding and
split-K") against the oracle's paged gather.

The handbook's paged decode test runs context lengths 1, 17, 1000 and 4096
over a shuffled block table of 16-position pages; here they run (plus 131072)
for one fp32 token (the FMA kernel) and one bf16 token (the tiled MFMA kernel
in split mode), and short chunks over long prefixes.  Every slot that holds no
cache position, spare pages included, is NaN, and so is the workspace before
each call, so reading a wrong page, slot or partial poisons the output.
Tolerances as in test_parity_gpu.py.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import oracle
import synth

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 64


def to_gpu(x, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def widen(x, dtype):
    return x if dtype == "f32" else synth.bf16_bits_to_f32(synth.to_bf16_bits(x))


def run(q, kp, vp, table, P, dtype):
    C = q.shape[0]
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    need, splits = cpf.splitkv_workspace(C, P, tdt)
    ws = torch.full((need // 4 + 4,), float("nan"), device="cuda")
    out = torch.full((C, HQ, D), float("nan"), device="cuda")
    cpf.attn_prefill_paged_splitkv(to_gpu(q, dtype), to_gpu(kp, dtype), to_gpu(vp, dtype),
                                   torch.from_numpy(table).cuda(), P, out=out, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), splits


def check(got, q, kp, vp, table, P, dtype, what):
    qo, kpo, vpo = widen(q, dtype), widen(kp, dtype), widen(vp, dtype)
    ref = oracle.attn_prefill_paged(qo, kpo, vpo, table, P).astype(np.float64)
    err = np.abs(got.astype(np.float64) - ref)
    if dtype == "f32":
        tol = 1e-4 + 1e-3 * np.abs(ref)
    else:
        tol = 1e-5 + 2.0 ** -8 * oracle.attn_prefill_paged(qo, kpo, np.abs(vpo), table, P).astype(np.float64)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d bad, first %s, max err %g" % (what, bad.sum(), tuple(np.argwhere(bad)[0]),
                                                                 float(np.nanmax(err)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ctx", [1, 17, 1000, 4096, 131072])
def test_paged_decode_context_lengths(ctx, dtype):
    P = ctx - 1
    q, k, v = synth.case_plain(1, P, 8800 + ctx)
    kp, vp, table = synth.to_pages(k, v, 16, 8900 + ctx)
    got, splits = run(q, kp, vp, table, P, dtype)
    check(got, q, kp, vp, table, P, dtype, "paged decode ctx=%d %s" % (ctx, dtype))
    if ctx >= 4096:
        assert splits > 1
    if ctx == 1:   # one visible key: its value row, bitwise
        for h in range(HQ):
            assert np.array_equal(got[0, h], widen(v, dtype)[0, h // 4]), h


@pytest.mark.parametrize("page_size", [1, 17, 64, 1000])
def test_paged_decode_page_sizes(page_size):
    """Pages that do not divide the 64-key split grain or the wave's 8-key
    chunks, single-position pages, and pages longer than a split."""
    P = 5000
    q, k, v, plants = synth.case_planted_chunk(1, P, 8700 + page_size, 1)
    kp, vp, table = synth.to_pages(k, v, page_size, 8600 + page_size)
    got, _ = run(q, kp, vp, table, P, "f32")
    check(got, q, kp, vp, table, P, "f32", "paged decode page=%d" % page_size)
    assert np.all(got[0, 0] == np.float32(4.0))   # the token's own key is planted


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("C,P,page_size", [(4, 4000, 16), (17, 3000, 17), (64, 20000, 16), (300, 3000, 64)])
def test_paged_splitkv_chunks(C, P, page_size, dtype):
    q, k, v, plants = synth.case_planted_chunk(C, P, 8500 + C + P, 3)
    kp, vp, table = synth.to_pages(k, v, page_size, 8400 + page_size)
    got, splits = run(q, kp, vp, table, P, dtype)
    check(got, q, kp, vp, table, P, dtype, "paged split C=%d P=%d page=%d %s" % (C, P, page_size, dtype))
    if dtype == "f32":
        for p in plants:
            assert np.all(got[p - P, 0] == np.float32(4.0))


def test_paged_decode_matches_contiguous_decode_bitwise():
    """The same plan over the same positions: the paged and contiguous
    split-KV calls give the same bits."""
    P = 16383
    q, k, v = synth.case_plain(1, P, 8300)
    kp, vp, table = synth.to_pages(k, v, 16, 8301)
    got, _ = run(q, kp, vp, table, P, "f32")
    contig = cpf.attn_prefill_splitkv(to_gpu(q, "f32"), to_gpu(k, "f32"), to_gpu(v, "f32"), P=P).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), contig.view(np.uint32))


@pytest.mark.parametrize("C", [1, 24])
def test_out_of_range_table_entries_read_as_zero_rows(C):
    """As for attn_prefill_paged: entries outside [0, numBlocks) read as zero
    keys and values, which the oracle reproduces by zeroing those positions."""
    P, ps = 3000, 16
    q, k, v = synth.case_plain(C, P, 8200 + C)
    kp, vp, table = synth.to_pages(k, v, ps, 8201)
    bad = table.copy()
    bad[2] = kp.shape[0]
    bad[100] = -7
    got, _ = run(q, kp, vp, bad, P, "f32")
    k0, v0 = k.copy(), v.copy()
    for b in (2, 100):
        k0[b * ps:(b + 1) * ps] = 0.0
        v0[b * ps:(b + 1) * ps] = 0.0
    ref = oracle.attn_prefill(q, k0, v0, P).astype(np.float64)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= 1e-4 + 1e-3 * np.abs(ref)), float(np.nanmax(err))
