"""The entry points can be captured in a HIP graph and replayed: they enqueue
kernels on the caller's stream and allocate, synchronise and memset nothing.
Each replay is checked bit for bit against an eager call on the same inputs,
with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import synth

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda", 0)


def g(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def replay_and_compare(graph, out, want, refill):
    for _ in range(3):
        out.fill_(float("nan"))
        refill()                      # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32))


def test_prefill_in_a_graph():
    C, P = 300, 1000
    q, k, v = synth.case_plain(C, P, 8100)
    qd, kd, vd = g(q), g(k), g(v)
    want = cpf.attn_prefill(qd, kd, vd, P=P).clone()
    out = torch.empty_like(want)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm the binding on the capture stream's device
        cpf.attn_prefill(qd, kd, vd, out=out, P=P)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cpf.attn_prefill(qd, kd, vd, out=out, P=P)
    scratch = torch.empty(1 << 20, device=dev())
    replay_and_compare(graph, out, want, lambda: scratch.uniform_())


def test_splitkv_decode_in_a_graph():
    C, P = 1, 9000
    q, k, v = synth.case_plain(C, P, 8200)
    qd, kd, vd = g(q), g(k), g(v)
    need, _ = cpf.splitkv_workspace(C, P)
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    want = cpf.attn_prefill_splitkv(qd, kd, vd, P=P, workspace=ws).clone()
    out = torch.empty_like(want)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cpf.attn_prefill_splitkv(qd, kd, vd, out=out, P=P, workspace=ws)
    scratch = torch.empty(1 << 20, device=dev())
    replay_and_compare(graph, out, want, lambda: scratch.normal_())


def test_noalloc_decode_in_a_graph():
    """The no-alloc entry point is meant for callers that capture graphs: its
    partials live in the library's fixed array, so capture needs no buffer
    but the inputs and out."""
    C, P = 1, 12000
    q, k, v = synth.case_plain(C, P, 8300)
    qd, kd, vd = g(q), g(k), g(v)
    want = torch.empty((C, 32, 64), device=dev())
    cpf.attn_prefill_splitkv_noalloc(qd, kd, vd, want, P=P)
    torch.cuda.synchronize()
    out = torch.empty_like(want)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cpf.attn_prefill_splitkv_noalloc(qd, kd, vd, out, P=P)
    scratch = torch.empty(1 << 20, device=dev())
    replay_and_compare(graph, out, want, lambda: scratch.normal_())


def test_paged_splitkv_decode_in_a_graph():
    C, P = 1, 7000
    q, k, v = synth.case_plain(C, P, 8400)
    kp, vp, table = synth.to_pages(k, v, 16, 8401)
    qd, kpd, vpd, tabd = g(q), g(kp), g(vp), torch.from_numpy(table).to(dev())
    need, _ = cpf.splitkv_workspace(C, P)
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    want = cpf.attn_prefill_paged_splitkv(qd, kpd, vpd, tabd, P, workspace=ws).clone()
    out = torch.empty_like(want)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cpf.attn_prefill_paged_splitkv(qd, kpd, vpd, tabd, P, out=out, workspace=ws)
    scratch = torch.empty(1 << 20, device=dev())
    replay_and_compare(graph, out, want, lambda: scratch.uniform_())
