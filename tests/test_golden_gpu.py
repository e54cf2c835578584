"""The handbook's worked online-softmax example ("FlashAttention and inference
kernels", Exercises, exercise 1: scores [1, 3] then [2, 5], values 10, 20, 30,
40, printed result 36.88) through every GPU entry point.

Embedded as in tests/golden/g1_online_softmax_example.json: one query row
whose head vectors are 8 e_0, so the score of key j is K[j][g][0].  Two
placements of the example's four keys:
  * P = 3, keys 0..3: the page's own shape;
  * P = 200, keys 126..129: the example straddles a 128-key staged tile, a
    key-split wave boundary and a decode split boundary, so the running (m, l,
    O) of the first pair must be carried or merged into the second.  Every
    other key scores -1000, whose weight e^-1005 underflows to exactly 0 in
    float and in double, and carries V = 4096, so any leak shows.
The expected value is the closed form sum(v e^s) / sum(e^s) in double.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import synth

pytestmark = pytest.mark.gpu

G = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                "g1_online_softmax_example.json")))
SCORES, VALUES = G["scores"], G["values"]
EXPECT = sum(v * math.exp(s) for s, v in zip(SCORES, VALUES)) / sum(math.exp(s) for s in SCORES)
PLACEMENTS = {"page": (3, [0, 1, 2, 3]), "straddle": (200, [126, 127, 128, 129])}


def inputs(P, positions):
    q = np.zeros((1, 32, 64), dtype=np.float32)
    q[:, :, 0] = 8.0
    k = np.zeros((P + 1, 8, 64), dtype=np.float32)
    k[:, :, 0] = -1000.0
    v = np.full((P + 1, 8, 64), 4096.0, dtype=np.float32)
    for pos, s_, val in zip(positions, SCORES, VALUES):
        k[pos, :, 0] = s_
        v[pos] = val
    return q, k, v


def gpu(x, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def run(entry, dtype, q, k, v, P):
    out = torch.full((1, 32, 64), float("nan"), device="cuda")
    qd, kd, vd = gpu(q, dtype), gpu(k, dtype), gpu(v, dtype)
    if entry == "prefill":
        cpf.attn_prefill(qd, kd, vd, out=out, P=P)
    elif entry == "rowwise":
        cpf.attn_prefill_rowwise(qd, kd, vd, out=out, P=P)
    elif entry == "splitkv":
        need, _ = cpf.splitkv_workspace(1, P, torch.float32 if dtype == "f32" else torch.bfloat16)
        ws = torch.full((need // 4 + 4,), float("nan"), device="cuda")
        cpf.attn_prefill_splitkv(qd, kd, vd, out=out, P=P, workspace=ws)
    else:
        kp, vp, table = synth.to_pages(k, v, 16, 4242)
        cpf.attn_prefill_paged(qd, gpu(kp, dtype), gpu(vp, dtype), torch.from_numpy(table).cuda(), P, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_closed_form_matches_print():
    assert round(EXPECT, 2) == G["printed"]["final"]


@pytest.mark.parametrize("placement", sorted(PLACEMENTS))
@pytest.mark.parametrize("entry", ["prefill", "paged", "splitkv", "rowwise"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example(placement, entry, dtype):
    P, positions = PLACEMENTS[placement]
    q, k, v = inputs(P, positions)
    got = run(entry, dtype, q, k, v, P)
    err = np.abs(got - EXPECT)
    if dtype == "f32":
        assert np.all(err <= 1e-4 + 1e-3 * EXPECT), (err.max(), got.flat[0])
        assert np.all(np.round(got, 2) == G["printed"]["final"])
    else:
        # bf16 bound with A = sum_j w_j |V_j| = EXPECT (all values positive); scores and values are exact in bf16
        assert np.all(err <= 1e-5 + 2.0 ** -8 * EXPECT), (err.max(), got.flat[0])
