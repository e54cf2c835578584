"""GPU parity of the three-kernel pipeline with the full score matrix
("Inference Attention 1: The Full Score Matrix", Lesson) against the oracle,
on prompt prefill (P = 0).  Tolerance as for the fp32 fused path: the scores,
exponentials and sums are fp32, the oracle's are double."""
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


def g(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def check(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = 1e-4 + 1e-3 * np.abs(ref.astype(np.float64))
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d bad, first %s" % (what, bad.sum(), tuple(np.argwhere(bad)[0]))


@pytest.mark.parametrize("T", [1, 17, 33, 64, 65, 257, 512])
def test_naive_matches_oracle(T):
    q, k, v, plants = synth.case_planted_chunk(T, 0, 6000 + T, 3)
    out = torch.full((T, HQ, D), float("nan"), device=dev())
    cpf.attn_naive(g(q), g(k), g(v), out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    check(got, oracle.attn_prefill(q, k, v, 0), "naive T=%d" % T)
    for p in plants:
        assert np.all(got[p, 0] == np.float32(4.0))


def test_naive_workspace_holds_the_causal_probability_matrix():
    """After the call the workspace is the row-normalised causal matrix:
    zeros above the diagonal, rows summing to 1."""
    T = 130
    q, k, v = synth.case_plain(T, 0, 6100)
    ws = torch.full((cpf.naive_workspace(T) // 4,), float("nan"), device=dev())
    cpf.attn_naive(g(q), g(k), g(v), workspace=ws)
    torch.cuda.synchronize()
    Pm = ws.view(HQ, T, T).cpu().numpy().astype(np.float64)
    upper = np.triu(np.ones((T, T), dtype=bool), 1)
    assert np.all(Pm[:, upper] == 0.0)
    assert np.allclose(Pm.sum(axis=2), 1.0, atol=1e-5)
    assert np.all(Pm[:, 0, 0] == 1.0)


def test_naive_full_size_t2048_sampled():
    T = 2048
    q, k, v = synth.case_plain(T, 0, 200)
    got = cpf.attn_naive(g(q), g(k), g(v)).cpu().numpy()
    rows = np.array([0, 1, 63, 64, 1000, 2046, 2047] * 2, dtype=np.int32)
    heads = np.array([0, 31, 5, 6, 17, 3, 30, 1, 2, 4, 8, 9, 10, 11], dtype=np.int32)
    ref = oracle.attn_rows(q, k, v, 0, rows, heads)
    check(got[rows, heads], ref, "naive T=2048 sampled")


def test_naive_agrees_with_fused():
    T = 700
    q, k, v = synth.case_plain(T, 0, 6200)
    a = cpf.attn_naive(g(q), g(k), g(v)).cpu().numpy()
    b = cpf.attn_prefill(g(q), g(k), g(v), P=0).cpu().numpy()
    assert np.allclose(a, b, rtol=1e-4, atol=1e-5)


def test_side_stream_without_context_keeps_its_allocations_on_that_stream():
    """The score-matrix workspace and out that the binding allocates for a
    call on an explicit side stream (outside any stream context) belong to
    that stream (see the split-KV test of the same name)."""
    T = 300
    q, k, v, _ = synth.case_planted_chunk(T, 0, 6400, 3)
    qd, kd, vd = g(q), g(k), g(v)
    need = cpf.naive_workspace(T)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)
    out = cpf.attn_naive(qd, kd, vd, stream=s)
    junk = torch.full((need // 4 + 64,), float("nan"), device=dev())
    snap = torch.cuda.memory_snapshot()
    s.synchronize()
    torch.cuda.synchronize()
    assert s.cuda_stream in {seg["stream"] for seg in snap if seg.get("total_size", 0) >= need}
    check(out.cpu().numpy(), oracle.attn_prefill(q, k, v, 0), "naive on a side stream")
    del junk
