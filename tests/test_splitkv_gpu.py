"""GPU parity of the split-KV entry point (key range split across workgroups,
partials merged by the log-sum-exp rule of "FlashAttention and inference
kernels", Flash-Decoding and Exercises, exercise 2) against the oracle.

The workspace is filled with NaN before every call, so a partial the merge
reads but no workgroup wrote shows up.  Tolerances as in test_parity_gpu.py.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import oracle
import synth

pytestmark = pytest.mark.gpu


def gpu(x, dtype="f32"):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def widen(x):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(x))


def run(q, k, v, P, dtype="f32"):
    C = q.shape[0]
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    need, splits = cpf.splitkv_workspace(C, P, tdt)
    ws = torch.full((need // 4 + 4,), float("nan"), device="cuda")
    out = torch.full((C, 32, 64), float("nan"), device="cuda")
    cpf.attn_prefill_splitkv(gpu(q, dtype), gpu(k, dtype), gpu(v, dtype), out=out, P=P, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), splits


def close_f32(got, ref):
    err = np.abs(got.astype(np.float64) - ref)
    bad = ~(err <= 1e-4 + 1e-3 * np.abs(ref))
    assert not bad.any(), "%d bad, max err %g" % (bad.sum(), np.nanmax(err))


@pytest.mark.parametrize("C,P", [(1, 31), (1, 1000), (1, 16383), (4, 4000), (17, 31), (33, 1000), (64, 20000),
                                 (300, 3000)])
def test_splitkv_fp32(C, P):
    q, k, v, plants = synth.case_planted_chunk(C, P, 7000 + C + P, 3)
    got, splits = run(q, k, v, P)
    ref = oracle.attn_prefill(q, k, v, P)
    close_f32(got, ref)
    for p in plants:
        assert np.all(got[p - P, 0] == np.float32(4.0))
    if P + C > 2048:
        assert splits > 1


def test_splitkv_single_key_exact():
    q, k, v = synth.case_plain(1, 0, 7100)
    got, _ = run(q, k, v, 0)
    for h in range(32):
        assert np.array_equal(got[0, h], v[0, h // 4])


def test_splitkv_last_key_plant():
    C, P = 8, 30000
    q, k, v, _ = synth.case_last_key(C, P, 7200)
    got, splits = run(q, k, v, P)
    assert splits > 1
    assert np.all(got[C - 1, 0] == np.float32(4.0))
    close_f32(got, oracle.attn_prefill(q, k, v, P))


@pytest.mark.parametrize("C,P", [(1, 32767), (16, 8000)])
def test_splitkv_bf16(C, P):
    q, k, v = synth.case_plain(C, P, 7300 + C)
    got, _ = run(q, k, v, P, "bf16")
    qo, ko, vo = widen(q), widen(k), widen(v)
    ref = oracle.attn_prefill(qo, ko, vo, P)
    a = oracle.attn_prefill(qo, ko, np.abs(vo), P)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= 1e-5 + 2.0 ** -8 * a)


def test_splitkv_matches_single_pass():
    C, P = 12, 9000
    q, k, v = synth.case_plain(C, P, 7400)
    got, _ = run(q, k, v, P)
    one = cpf.attn_prefill(gpu(q), gpu(k), gpu(v), P=P).cpu().numpy()
    assert np.max(np.abs(got - one)) < 1e-5


@pytest.mark.parametrize("P", [0, 7, 8, 62, 63, 64, 65, 511, 4095, 100000])
def test_decode_one_token_fp32(P):
    """One token (the FMA decode kernel): split edges at multiples of 64 keys,
    waves and key slots with no keys, and a cache longer than 64 splits'
    worth of the minimum split."""
    q, k, v = synth.case_plain(1, P, 7500 + P)
    got, splits = run(q, k, v, P)
    close_f32(got, oracle.attn_prefill(q, k, v, P))
    assert 1 <= splits <= 32


@pytest.mark.parametrize("P", [5, 1000, 50000])
def test_decode_one_token_bf16(P):
    q, k, v = synth.case_plain(1, P, 7600 + P)
    got, _ = run(q, k, v, P, "bf16")
    qo, ko, vo = widen(q), widen(k), widen(v)
    ref = oracle.attn_prefill(qo, ko, vo, P)
    a = oracle.attn_prefill(qo, ko, np.abs(vo), P)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 1e-5 + 2.0 ** -8 * a)


def test_decode_planted_maximum_in_last_split():
    """The row's dominant key is its last one (the token itself), so the
    running maximum jumps in the last split and the merge must rescale."""
    P = 20000
    q, k, v, pos = synth.case_last_key(1, P, 7700)
    got, splits = run(q, k, v, P)
    assert splits > 1 and pos == [P]
    assert np.all(got[0, 0] == np.float32(4.0))
    close_f32(got, oracle.attn_prefill(q, k, v, P))


def test_decode_deterministic():
    q, k, v = synth.case_plain(1, 9999, 7800)
    a, _ = run(q, k, v, 9999)
    b, _ = run(q, k, v, 9999)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_side_stream_without_context_keeps_its_allocations_on_that_stream():
    """A call on an explicit side stream, made outside any stream context,
    with out and workspace allocated by the binding: both must be allocated on
    the side stream, so torch's caching allocator does not hand the freed
    workspace to the current stream while the side stream's kernels may still
    use it.  The side stream is held back by a spin first, so the kernels run
    after the binding has returned and freed the workspace."""
    C, P = 17, 3000
    q, k, v, plants = synth.case_planted_chunk(C, P, 7400, 3)
    qd, kd, vd = gpu(q), gpu(k), gpu(v)
    need, _ = cpf.splitkv_workspace(C, P, torch.float32)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)
    out = cpf.attn_prefill_splitkv(qd, kd, vd, P=P, stream=s)
    junk = torch.full((need // 4 + 64,), float("nan"), device="cuda")   # current stream, runs at once
    snap = torch.cuda.memory_snapshot()
    s.synchronize()
    torch.cuda.synchronize()
    streams = {seg["stream"] for seg in snap if seg.get("total_size", 0) >= need}
    assert s.cuda_stream in streams
    close_f32(out.cpu().numpy(), oracle.attn_prefill(q, k, v, P))
    del junk
