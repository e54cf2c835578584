"""GPU parity of the paged-cache entry point against the oracle's paged gather.

The cache is scattered into seeded, shuffled pages ("FlashAttention and
inference kernels", section PagedAttention); every slot that holds no cache
position, including whole spare pages, is NaN, so reading a wrong page or
slot poisons the output.  Tolerances as in test_parity_gpu.py.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import oracle
import synth

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 64


def dev():
    return torch.device("cuda", 0)


def to_gpu(x, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev())


def widen(x, dtype):
    return x if dtype == "f32" else synth.bf16_bits_to_f32(synth.to_bf16_bits(x))


def check(got, ref, dtype, absref=None, what=""):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    if dtype == "f32":
        tol = 1e-4 + 1e-3 * np.abs(ref.astype(np.float64))
    else:
        tol = 1e-5 + 2.0 ** -8 * absref.astype(np.float64)
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d bad, first %s got %r ref %r" % (
        what, bad.sum(), tuple(np.argwhere(bad)[0]), got[tuple(np.argwhere(bad)[0])],
        ref[tuple(np.argwhere(bad)[0])])


def run_paged(q, kp, vp, table, P, dtype):
    out = torch.full((q.shape[0], HQ, D), float("nan"), device=dev())
    cpf.attn_prefill_paged(to_gpu(q, dtype), to_gpu(kp, dtype), to_gpu(vp, dtype),
                           torch.from_numpy(table).to(dev()), P, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("page_size", [1, 16, 17, 64])
@pytest.mark.parametrize("C,P", [(17, 31), (300, 1000), (1030, 77)])
def test_paged_fp32(page_size, C, P):
    q, k, v, plants = synth.case_planted_chunk(C, P, 5000 + C + P, 3)
    kp, vp, table = synth.to_pages(k, v, page_size, 5100 + page_size)
    got = run_paged(q, kp, vp, table, P, "f32")
    ref = oracle.attn_prefill_paged(q, kp, vp, table, P)
    check(got, ref, "f32", what="paged C=%d P=%d page=%d" % (C, P, page_size))
    for p in plants:
        assert np.all(got[p - P, 0] == np.float32(4.0))


def test_paged_one_stage_over_several_rounds():
    """The 8-row one-staging-buffer kernel over pages, in more rounds than
    the 512 resident workgroups (1300 rows against a prefix of 10C), every
    element against the oracle."""
    C, P = 1300, 13000
    assert cpf.plan(C, P, torch.float32, paged=True)["lds_bytes"] < 81920   # two workgroups per CU
    q, k, v, plants = synth.case_planted_chunk(C, P, 5300, 3)
    kp, vp, table = synth.to_pages(k, v, 16, 5301)
    got = run_paged(q, kp, vp, table, P, "f32")
    ref = oracle.attn_prefill_paged(q, kp, vp, table, P)
    check(got, ref, "f32", what="paged C=%d P=%d page=16" % (C, P))
    for p in plants:
        assert np.all(got[p - P, 0] == np.float32(4.0))


@pytest.mark.parametrize("page_size", [16, 33])
def test_paged_bf16(page_size):
    C, P = 300, 1000
    q, k, v = synth.case_plain(C, P, 5200)
    kp, vp, table = synth.to_pages(k, v, page_size, 5201)
    got = run_paged(q, kp, vp, table, P, "bf16")
    qo, kpo, vpo = widen(q, "bf16"), widen(kp, "bf16"), widen(vp, "bf16")
    ref = oracle.attn_prefill_paged(qo, kpo, vpo, table, P)
    absref = oracle.attn_prefill_paged(qo, kpo, np.abs(vpo), table, P)
    check(got, ref, "bf16", absref, "paged bf16 page=%d" % page_size)


def test_paged_full_size_c2048_p2048():
    C, P = 2048, 2048
    q, k, v = synth.case_plain(C, P, 200)
    kp, vp, table = synth.to_pages(k, v, 16, 5301)
    got = run_paged(q, kp, vp, table, P, "f32")
    ref = oracle.attn_prefill_paged(q, kp, vp, table, P)
    check(got, ref, "f32", what="paged C=P=2048")


@pytest.mark.parametrize("C,P,dtype", [(600, 200, "f32"), (1800, 900, "f32"), (384, 1000, "f32"), (512, 0, "f32"),
                                     (1100, 8800, "f32"),
                                     (2048, 500, "bf16"), (4096, 300, "bf16")])
def test_paged_equals_contiguous_bitwise(C, P, dtype):
    """Same launch plan, same arithmetic: the paged path must reproduce the
    contiguous path bit for bit (fp32 16-row and 32-row work items with two
    staging buffers and 8-row ones with one, in the heavy/light order and
    heaviest first;
    bf16 32-row and 64-row ones)."""
    q, k, v = synth.case_plain(C, P, 5400 + C)
    kp, vp, table = synth.to_pages(k, v, 16, 5401 + C)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    pp, pc = cpf.plan(C, P, tdt, paged=True), cpf.plan(C, P, tdt)
    lp, lc = pp.pop("lds_bytes"), pc.pop("lds_bytes")
    offsets = 2 * 4 * pc["keys_per_tile"]                  # the row offsets of two tiles
    qrows = 1024 * pc["rows_per_item"] if dtype == "f32" else 0
    # fp32 Q rows that no longer fit after the offsets move into a staging tile
    assert lp == lc + offsets or (lc + offsets > 160 * 1024 and lp == lc - qrows + offsets), (lp, lc)
    assert pp == pc
    paged = run_paged(q, kp, vp, table, P, dtype)
    contig = cpf.attn_prefill(to_gpu(q, dtype), to_gpu(k, dtype), to_gpu(v, dtype), P=P).cpu().numpy()
    assert np.array_equal(paged.view(np.uint32), contig.view(np.uint32))


def test_out_of_range_table_entries_read_as_zero_rows():
    """Table entries outside [0, numBlocks) do not fault: their positions read
    as zero keys and values (the kernel's own range check), which the oracle
    reproduces by zeroing those positions of the logical cache."""
    C, P, ps = 40, 200, 16
    q, k, v = synth.case_plain(C, P, 5500)
    kp, vp, table = synth.to_pages(k, v, ps, 5501)
    bad = table.copy()
    bad[2] = kp.shape[0]          # one past the pool
    bad[5] = -7
    got = run_paged(q, kp, vp, bad, P, "f32")
    k0, v0 = k.copy(), v.copy()
    for b in (2, 5):
        k0[b * ps:(b + 1) * ps] = 0.0
        v0[b * ps:(b + 1) * ps] = 0.0
    ref = oracle.attn_prefill(q, k0, v0, P)
    check(got, ref, "f32", what="out-of-range table entries")
