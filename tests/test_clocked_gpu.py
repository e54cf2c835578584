"""GPU check of attn_prefill_clocked, the entry point the benchmark reads its
clock and phase times from: the same result as attn_prefill bit for bit, and a
clock log in which every workgroup started before it ended, ran at a plausible
MI355X shader clock (a few hundred MHz idle to about 2.4 GHz), and wrote its
phase marks in order (a second item's mark only where it has one)."""
import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("C,P,dtype", [(2048, 2048, torch.float32), (512, 0, torch.float32),
                                       (100, 3000, torch.float32), (4096, 100, torch.bfloat16)])
def test_clocked_call_matches_and_logs_a_plausible_clock(C, P, dtype):
    q, k, v = synth.case_plain(C, P, 9500 + C)
    qd, kd, vd = (torch.from_numpy(x).cuda().to(dtype) for x in (q, k, v))
    want = cpf.attn_prefill(qd, kd, vd, P=P)
    got, clocks = cpf.attn_prefill_clocked(qd, kd, vd, P=P)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    c = clocks.cpu().numpy().astype(np.int64)
    plan = cpf.plan(C, P, dtype)
    assert c.shape == (plan["grid"], cpf.CLOCK_WORDS)
    assert np.all(c[:, 2] > c[:, 0]) and np.all(c[:, 3] > c[:, 1])
    mhz = (c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * 100.0
    assert np.all((mhz > 100) & (mhz < 2600)), (mhz.min(), mhz.max())
    # phase marks in order: start <= first tile in <= loop done <= stored <= end
    assert np.all(c[:, 0] <= c[:, 4]) and np.all(c[:, 4] <= c[:, 5]) and np.all(c[:, 5] <= c[:, 6])
    assert np.all(c[:, 6] <= c[:, 2])
    two = c[:, 7] != 0
    assert np.all(c[two, 6] <= c[two, 7]) and np.all(c[two, 7] <= c[two, 2])
    if plan["items_per_workgroup"] == 1:
        assert not two.any()
    else:   # paired items: every workgroup but the middle one of an odd count has two
        assert two.sum() >= plan["grid"] - 8


def test_clocked_rejects_a_short_clock_buffer():
    lib = cpf.load_library()
    C, P = 64, 64
    q = torch.zeros(C, 32, 64, device="cuda")
    k = torch.zeros(P + C, 8, 64, device="cuda")
    out = torch.zeros(C, 32, 64, device="cuda")
    grid = cpf.plan(C, P)["grid"]
    n = cpf.CLOCK_WORDS * grid
    buf = torch.zeros(n, dtype=torch.int64, device="cuda")
    args = (q.data_ptr(), k.data_ptr(), k.data_ptr(), out.data_ptr(), C, P, 0)
    assert lib.attn_prefill_clocked(*args, buf.data_ptr(), n - 1, None) == 7
    assert lib.attn_prefill_clocked(*args, None, n, None) == 2
    assert lib.attn_prefill_clocked(*args, buf.data_ptr() + 4, n, None) == 4
    assert lib.attn_prefill_clocked(*args, out.data_ptr(), n, None) == 6
    torch.cuda.synchronize()


def test_clocked_writes_a_given_buffer_in_place():
    """The form the benchmark times: a clock buffer allocated beforehand is
    written in place (nothing allocated or cleared by the call), rows past the
    launch's workgroups are left alone, and the output is attn_prefill's."""
    C, P = 300, 1000
    q, k, v = synth.case_plain(C, P, 9700)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    grid = cpf.plan(C, P)["grid"]
    buf = torch.full((grid + 3, cpf.CLOCK_WORDS), -1, dtype=torch.int64, device="cuda")
    want = cpf.attn_prefill(qd, kd, vd, P=P)
    for _ in range(2):
        got, clocks = cpf.attn_prefill_clocked(qd, kd, vd, P=P, clocks=buf)
        torch.cuda.synchronize()
        assert clocks.data_ptr() == buf.data_ptr() and clocks.shape == (grid, cpf.CLOCK_WORDS)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))
        c = buf.cpu().numpy()
        assert np.all(c[grid:] == -1)
        assert np.all(c[:grid, 2] > c[:grid, 0]) and np.all(c[:grid, 3] > c[:grid, 1])
    with pytest.raises(ValueError):
        cpf.attn_prefill_clocked(qd, kd, vd, P=P, clocks=buf[:grid - 1])
    with pytest.raises(ValueError):
        cpf.attn_prefill_clocked(qd, kd, vd, P=P, clocks=buf.to(torch.int32))
