"""GPU parity of the per-row baseline (no tiling, every row streams its whole
K/V prefix, as the starter of "Inference Attention 2" does; Lesson) against
the oracle; tolerances as in test_parity_gpu.py.  Shapes cover partial and
several 64-key blocks, rows of one key and the bf16 path."""
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


def close(got, ref, atol=1e-4, rtol=1e-3):
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= atol + rtol * np.abs(ref)), float(np.nanmax(err))


@pytest.mark.parametrize("C,P", [(17, 31), (1, 0), (33, 1000), (65, 7), (300, 200)])
def test_rowwise_fp32(C, P):
    q, k, v, plants = synth.case_planted_chunk(C, P, 6000 + C + P, 3)
    got = cpf.attn_prefill_rowwise(gpu(q), gpu(k), gpu(v), P=P).cpu().numpy()
    ref = oracle.attn_prefill(q, k, v, P)
    close(got, ref)
    for p in plants:
        assert np.all(got[p - P, 0] == np.float32(4.0))
    if P == 0:
        for h in range(32):
            assert np.array_equal(got[0, h], v[0, h // 4])


def test_rowwise_bf16():
    C, P = 40, 500
    q, k, v = synth.case_plain(C, P, 6100)
    got = cpf.attn_prefill_rowwise(gpu(q, "bf16"), gpu(k, "bf16"), gpu(v, "bf16"), P=P).cpu().numpy()
    qo, ko, vo = widen(q), widen(k), widen(v)
    ref = oracle.attn_prefill(qo, ko, vo, P)
    a = oracle.attn_prefill(qo, ko, np.abs(vo), P)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= 1e-5 + 2.0 ** -8 * a)


def test_rowwise_full_size_sampled_rows():
    C, P = 2048, 2048
    q, k, v = synth.case_plain(C, P, 200)
    got = cpf.attn_prefill_rowwise(gpu(q), gpu(k), gpu(v), P=P).cpu().numpy()
    rows = np.array([0, 1, 63, 64, 1000, 2046, 2047])
    rr, hh = np.repeat(rows, 32), np.tile(np.arange(32), len(rows))
    ref = oracle.attn_rows(q, k, v, P, rr, hh)
    close(got[rr, hh], ref)
