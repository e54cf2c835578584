"""GPU check of attn_prefill_splitkv_noalloc, the split-KV entry point whose
key-split partials live in the library's fixed per-device scratch array: its
output must equal attn_prefill_splitkv's (same kernels, caller workspace)
bit for bit, and the oracle's within the stated tolerances, on two calls in a
row, the second smaller than the first (the array keeps the first call's
partials, which must not leak into the second)."""
import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import oracle
import synth

pytestmark = pytest.mark.gpu


def gpu(x, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def widen(x, dtype):
    return x if dtype == "f32" else synth.bf16_bits_to_f32(synth.to_bf16_bits(x))


def one_call(C, P, dtype, seed):
    q, k, v, plants = synth.case_planted_chunk(C, P, seed, 3)
    qd, kd, vd = gpu(q, dtype), gpu(k, dtype), gpu(v, dtype)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    need, _ = cpf.splitkv_workspace(C, P, tdt)
    assert need <= cpf.NOALLOC_SCRATCH_BYTES
    out = torch.full((C, 32, 64), float("nan"), device="cuda")
    cpf.attn_prefill_splitkv_noalloc(qd, kd, vd, out, P=P)
    ws = torch.full((need // 4 + 4,), float("nan"), device="cuda")
    want = torch.full((C, 32, 64), float("nan"), device="cuda")
    cpf.attn_prefill_splitkv(qd, kd, vd, out=want, P=P, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.cpu().numpy().view(np.uint32)), (C, P, dtype)
    qo, ko, vo = widen(q, dtype), widen(k, dtype), widen(v, dtype)
    ref = oracle.attn_prefill(qo, ko, vo, P).astype(np.float64)
    err = np.abs(got.astype(np.float64) - ref)
    if dtype == "f32":
        tol = 1e-4 + 1e-3 * np.abs(ref)
    else:
        tol = 1e-5 + 2.0 ** -8 * oracle.attn_prefill(qo, ko, np.abs(vo), P).astype(np.float64)
    assert np.all(err <= tol), (C, P, dtype, float(np.nanmax(err)))
    for p in plants:
        if dtype == "f32":
            assert np.all(got[p - P, 0] == np.float32(4.0))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    # first call: 64 rows over a 20000-position prefix (several key splits of
    # the MFMA kernel); second call smaller: one token (fp32: the FMA decode
    # kernel) over a 5000-position prefix
    one_call(64, 20000, dtype, 9100)
    one_call(1, 5000, dtype, 9200)


def test_noalloc_rejects_calls_beyond_the_scratch_array():
    C, P = 4096, 100
    need, _ = cpf.splitkv_workspace(C, P, torch.float32)
    assert need > cpf.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(C, 32, 64, device="cuda")
    k = torch.zeros(P + C, 8, 64, device="cuda")
    out = torch.zeros(C, 32, 64, device="cuda")
    with pytest.raises(cpf.AttnError) as e:
        cpf.attn_prefill_splitkv_noalloc(q, k, k.clone(), out, P=P)
    assert e.value.code == 8
    # the array is untouched by a rejected call: a valid call still matches
    one_call(17, 31, "f32", 9300)
