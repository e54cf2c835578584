"""Pins for the CPU oracle, checked against facts fixed by the pages and by
mathematics rather than against the oracle itself.

Each pin is a function of `run(q, k, v, P) -> out`, so the same suite is also
run against deliberately broken copies of the oracle (compiled on the CPU in a
temporary directory) to show that each plausible mistake fails some pin.

Sources:
* "FlashAttention and inference kernels", Exercises, exercise 1 (worked
  online-softmax example, printed values in tests/golden/).
* "Inference Attention 2: Flash Prefill Against a Cached Prefix", Lesson:
  causal edge j <= P + i, head mapping h -> h/4, scale 1/8, planted 4.0
  hazards scoring 128, last-key plant.
* "Inference Attention 1: The Full Score Matrix", Lesson: the single-token
  row whose probability must be exactly 1; stable softmax.
"""
import ctypes
import json
import math
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
HQ, HKV, D = 32, 8, 64


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def _g1_inputs():
    g = json.load(open(os.path.join(GOLDEN, "g1_online_softmax_example.json")))
    scores, values = g["scores"], g["values"]
    q = np.zeros((1, HQ, D), np.float32)
    q[0, :, 0] = 8.0
    k = np.zeros((4, HKV, D), np.float32)
    v = np.zeros((4, HKV, D), np.float32)
    for j in range(4):
        k[j, :, 0] = scores[j]
        v[j, :, :] = values[j]
    return g, q, k, v


def pin_golden_worked_example(run):
    """The page's worked example: the printed final value 36.88 (2 decimals),
    the printed intermediates O/l = 44.384/1.2034, and the page's direct
    softmax-weighted sum written in closed form."""
    g, q, k, v = _g1_inputs()
    out = run(q, k, v, 3)
    pr = g["printed"]
    assert np.all(np.abs(out - pr["final"]) <= 0.005 + 1e-9), out.ravel()[:4]
    assert np.all(np.abs(out - pr["tile2"]["O"] / pr["tile2"]["l"]) <= 0.01)
    s, vals = g["scores"], g["values"]
    closed = sum(math.exp(a) * b for a, b in zip(s, vals)) / sum(math.exp(a) for a in s)
    assert np.all(out == np.float32(closed)), (out.ravel()[0], closed)


def pin_single_visible_key(run):
    """A row that sees one key has probability exactly 1 on it, so its
    output is that key's value row, bit for bit (T=1, and row 0 of P=0)."""
    q, k, v = synth.case_plain(1, 0, 9100)
    out = run(q, k, v, 0)
    for h in range(HQ):
        assert np.array_equal(out[0, h], v[0, h // 4])
    q, k, v = synth.case_plain(5, 0, 9200)
    out = run(q, k, v, 0)
    for h in range(HQ):
        assert np.array_equal(out[0, h], v[0, h // 4])


def pin_planted_rows_exact(run):
    """Planted 4.0 in query head 0 and KV head 0: planted scores are 128,
    every other weight is below e^-90, so planted rows of head 0 are exactly
    4.0 in float32."""
    q, k, v, pos = synth.case_planted_chunk(17, 31, 100, 3)
    out = run(q, k, v, 31)
    for p in pos:
        assert np.all(out[p - 31, 0] == np.float32(4.0)), (p, out[p - 31, 0, :4])


def pin_huge_scores_stable(run):
    """Planting 12.0 makes scores of 12*12*64/8 = 1152, beyond double exp
    overflow (about 709): only a max-subtracted softmax returns the planted
    value (exactly 12.0) instead of inf/NaN."""
    q, k, v = synth.case_plain(9, 20, 9300)
    synth.plant(q, k, v, 20, [24, 27], value=12.0)
    out = run(q, k, v, 20)
    assert np.all(np.isfinite(out))
    for p in (24, 27):
        assert np.all(out[p - 20, 0] == np.float32(12.0)), out[p - 20, 0, :4]


def pin_last_key_plant(run):
    """Only the final cache position is planted: the last chunk row of head 0
    meets its maximum at its last key and must be exactly 4.0."""
    C, P = 40, 300
    q, k, v, pos = synth.case_last_key(C, P, 9400)
    out = run(q, k, v, P)
    assert np.all(out[C - 1, 0] == np.float32(4.0))


def pin_zero_keys_prefix_mean(run):
    """K = 0 makes every score 0, so each output is the plain mean of the
    visible value rows j <= P+i: exact prefix averages of V."""
    C, P = 7, 13
    q, k, v = synth.case_plain(C, P, 9500)
    k[:] = 0.0
    out = run(q, k, v, P)
    v64 = v.astype(np.float64)
    for i in range(C):
        n = P + i + 1
        for h in range(HQ):
            ref = v64[:n, h // 4, :].mean(axis=0)
            np.testing.assert_allclose(out[i, h], ref, rtol=2e-7, atol=1e-7)


def pin_logistic_two_keys(run):
    """Two keys whose scores are 0 and 1, with the 1 spread evenly over all
    64 dims (q = 1, K[1] = 1/8): the weight on key 1 is the logistic
    e/(1+e).  With V[0] = 0 and V[1] = 1 that is the output."""
    q = np.ones((1, HQ, D), np.float32)
    k = np.zeros((2, HKV, D), np.float32)
    k[1] = 0.125
    v = np.zeros((2, HKV, D), np.float32)
    v[1] = 1.0
    out = run(q, k, v, 1)
    ref = math.e / (1.0 + math.e)
    assert np.all(out == np.float32(ref)), (out.ravel()[0], ref)


def pin_convex_hull(run):
    """Each output is a convex combination of the visible value rows."""
    C, P = 17, 31
    q, k, v, _ = synth.case_planted_chunk(C, P, 9600, 2)
    out = run(q, k, v, P).astype(np.float64)
    for i in range(C):
        n = P + i + 1
        for h in range(HQ):
            vv = v[:n, h // 4, :].astype(np.float64)
            assert np.all(out[i, h] >= vv.min(axis=0) - 1e-6)
            assert np.all(out[i, h] <= vv.max(axis=0) + 1e-6)


def pin_prefix_permutation(run):
    """Permuting the prefix positions 0..P-1 (keys with their values) does
    not change any output: every row sees the whole prefix."""
    C, P = 6, 25
    q, k, v = synth.case_plain(C, P, 9700)
    out = run(q, k, v, P)
    perm = np.random.default_rng(5).permutation(P)
    k2, v2 = k.copy(), v.copy()
    k2[:P], v2[:P] = k[perm], v[perm]
    out2 = run(q, k2, v2, P)
    np.testing.assert_allclose(out2, out, rtol=1e-6, atol=1e-7)


def pin_future_keys_ignored(run):
    """Row i must not depend on cache positions beyond P+i."""
    C, P = 8, 10
    q, k, v = synth.case_plain(C, P, 9800)
    out = run(q, k, v, P)
    for i in (0, 3, C - 2):
        k2, v2 = k.copy(), v.copy()
        k2[P + i + 1:] = 50.0
        v2[P + i + 1:] = -77.0
        out2 = run(q, k2, v2, P)
        assert np.array_equal(out2[i], out[i]), i
        assert not np.array_equal(out2[i + 1], out[i + 1])


def pin_gqa_mapping(run):
    """Heads 4g..4g+3 read KV head g: identical query rows across a group
    give identical outputs, and changing KV head g changes only those four
    heads."""
    C, P = 5, 9
    q, k, v = synth.case_plain(C, P, 9900)
    for g in range(HKV):
        q[:, 4 * g + 1:4 * g + 4, :] = q[:, 4 * g:4 * g + 1, :]
    out = run(q, k, v, P)
    for g in range(HKV):
        for t in range(1, 4):
            assert np.array_equal(out[:, 4 * g + t], out[:, 4 * g])
    for g in (0, 5):
        k2, v2 = k.copy(), v.copy()
        k2[:, g] *= -1.0
        v2[:, g] += 1.0
        out2 = run(q, k2, v2, P)
        for h in range(HQ):
            same = np.array_equal(out2[:, h], out[:, h])
            assert same == (h // 4 != g), (g, h)


def numpy_reference(q, k, v, P):
    """softmax(Q K^T / 8 + causal mask) V in float64 with KV heads repeated
    four times: the matrix form of the same definition, by numpy."""
    C = q.shape[0]
    T = P + C
    kk = np.repeat(k.astype(np.float64), 4, axis=1)      # [T][32][64]
    vv = np.repeat(v.astype(np.float64), 4, axis=1)
    qq = q.astype(np.float64)
    s = np.matmul(qq.transpose(1, 0, 2), kk.transpose(1, 2, 0)) / 8.0   # [32][C][T]
    mask = np.arange(T)[None, :] > (P + np.arange(C))[:, None]
    s[:, mask] = -np.inf
    s -= s.max(axis=2, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=2, keepdims=True)
    o = np.matmul(w, vv.transpose(1, 0, 2))              # [32][C][64]
    return o.transpose(1, 0, 2).astype(np.float32)


def pin_numpy_formulation(run):
    """Random tiny shapes against the numpy matrix formulation."""
    for (C, P, sb) in [(1, 3, 8100), (17, 31, 8200), (33, 0, 8300), (5, 40, 8400)]:
        q, k, v = synth.case_plain(C, P, sb)
        out = run(q, k, v, P)
        ref = numpy_reference(q, k, v, P)
        np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


PINS = [pin_golden_worked_example, pin_single_visible_key, pin_planted_rows_exact,
        pin_huge_scores_stable, pin_last_key_plant, pin_zero_keys_prefix_mean,
        pin_logistic_two_keys, pin_convex_hull, pin_prefix_permutation,
        pin_future_keys_ignored, pin_gqa_mapping, pin_numpy_formulation]


def _oracle_run(q, k, v, P):
    return oracle.attn_prefill(q, k, v, P)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(_oracle_run)


def test_rows_entry_matches_full():
    C, P = 17, 31
    q, k, v, _ = synth.case_planted_chunk(C, P, 100, 3)
    full = oracle.attn_prefill(q, k, v, P)
    rows = np.array([0, 5, 16, 16, 3])
    heads = np.array([0, 31, 0, 7, 12])
    sel = oracle.attn_rows(q, k, v, P, rows, heads)
    for t in range(len(rows)):
        assert np.array_equal(sel[t], full[rows[t], heads[t]])


@pytest.mark.parametrize("page_size", [1, 16, 17, 64])
def test_paged_gather_matches_contiguous_cache(page_size):
    """A paged cache built by scattering the contiguous cache into shuffled
    pages (the unused slots hold NaN) gives bit-identical outputs: the gather
    reproduces the logical cache exactly."""
    C, P = 17, 70
    q, k, v, _ = synth.case_planted_chunk(C, P, 9910, 3)
    kp, vp, table = synth.to_pages(k, v, page_size, 9917)
    got = oracle.attn_prefill_paged(q, kp, vp, table, P)
    ref = oracle.attn_prefill(q, k, v, P)
    assert np.array_equal(got, ref)
    assert sorted(set(table.tolist())) == sorted(table.tolist())   # a permutation prefix


def test_paged_rejects_bad_table():
    q, k, v = synth.case_plain(3, 5, 9920)
    kp, vp, table = synth.to_pages(k, v, 4, 9921)
    bad = table.copy()
    bad[0] = kp.shape[0]
    with pytest.raises(RuntimeError):
        oracle.attn_prefill_paged(q, kp, vp, bad, 5)


def test_oracle_rejects_bad_shapes():
    q, k, v = synth.case_plain(3, 4, 7000)
    with pytest.raises(ValueError):
        oracle.attn_prefill(q, k, v, 5)
    out = oracle.attn_prefill(q[:0], k[:4], v[:4], 4)
    assert out.shape == (0, HQ, D)


# ----------------------------------------------------------------------------
# planted mistakes: each broken copy of the oracle must fail at least one pin
# ----------------------------------------------------------------------------

MUTANTS = {
    "scale_dropped": ("s[j] = dot * 0.125;", "s[j] = dot;"),
    "causal_short": ("const int n = P + i + 1;", "const int n = P + i;"),
    "causal_long": ("const int n = P + i + 1;", "const int n = P + i + 2;"),
    "no_max_subtraction": ("s[j] = exp(s[j] - M);", "s[j] = exp(s[j]);"),
    "max_sign_flip": ("s[j] = exp(s[j] - M);", "s[j] = exp(M - s[j]);"),
    "gqa_modulo": ("const int g = h / OR_GROUP;", "const int g = h % OR_HKV;"),
    "k_for_v": ("const float* vrow = vc +", "const float* vrow = kc +"),
    "half_the_dims": ("for (int k = 0; k < OR_D; ++k) dot +=", "for (int k = 0; k < OR_D / 2; ++k) dot +="),
    "no_normalisation": ("orow[d] = (float)(acc[d] / L);", "orow[d] = (float)(acc[d]);"),
    "neighbour_head": ("const float* qrow = q + ((size_t)i * OR_HQ + h) * OR_D;",
                       "const float* qrow = q + ((size_t)i * OR_HQ + (h ^ 1)) * OR_D;"),
    "first_max_only": ("if (s[j] > M) M = s[j];", "if (s[j] > M && j < 2) M = s[j];"),
    "value_row_shift": ("const float* vrow = vc + ((size_t)j * OR_HKV + g) * OR_D;",
                        "const float* vrow = vc + ((size_t)(j > 0 ? j - 1 : 0) * OR_HKV + g) * OR_D;"),
    "paged_slot_shift": ("(size_t)(t % pageSize)) * row;", "(size_t)((t + 1) % pageSize)) * row;"),
    "paged_block_shift": ("blockTable[t / pageSize] * pageSize", "blockTable[(t + 1) / pageSize] * pageSize"),
}


def _mutant_runner(so_path):
    lib = ctypes.CDLL(so_path)
    f = ctypes.POINTER(ctypes.c_float)
    lib.oracle_attn_prefill.argtypes = [f, f, f, f, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_attn_prefill.restype = ctypes.c_int

    def run(q, k, v, P):
        # K/V get four rows of NaN past the cache, so a mutant that reads past
        # the visible range sees NaN instead of leaving the buffer.
        q = np.ascontiguousarray(q, np.float32)
        T = k.shape[0]
        kp = np.full((T + 4,) + k.shape[1:], np.nan, np.float32)
        vp = np.full((T + 4,) + v.shape[1:], np.nan, np.float32)
        kp[:T], vp[:T] = k, v
        k, v = kp, vp
        out = np.empty_like(q)
        with np.errstate(all="ignore"):
            rc = lib.oracle_attn_prefill(q.ctypes.data_as(f), k.ctypes.data_as(f),
                                         v.ctypes.data_as(f), out.ctypes.data_as(f),
                                         q.shape[0], P, 2)
        assert rc == 0
        return out
    return run


def run_pins_on(so_path):
    """Run every pin against the library at so_path; return the names of the
    pins it fails.  Called in a child process by the mutation test."""
    run = _mutant_runner(so_path)
    caught = []
    pins = list(PINS) + [_paged_pin(so_path)]
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(run)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    return caught


def _paged_pin(so_path):
    """The paged gather pin, run on the library at so_path."""
    lib = ctypes.CDLL(so_path)
    f = ctypes.POINTER(ctypes.c_float)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_attn_prefill_paged.argtypes = [f, f, f, ip, ctypes.c_int, ctypes.c_int, f, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int]
    lib.oracle_attn_prefill_paged.restype = ctypes.c_int
    contiguous = _mutant_runner(so_path)

    def pin_paged_gather(run):
        C, P = 9, 30
        q, k, v = synth.case_plain(C, P, 9930)
        kp, vp, table = synth.to_pages(k, v, 16, 9931)
        out = np.empty_like(q)
        with np.errstate(all="ignore"):
            rc = lib.oracle_attn_prefill_paged(q.ctypes.data_as(f), kp.ctypes.data_as(f), vp.ctypes.data_as(f),
                                               table.ctypes.data_as(ip), kp.shape[0], 16, out.ctypes.data_as(f),
                                               C, P, 2)
        assert rc == 0
        assert np.array_equal(out, contiguous(q, k, v, P))
    return pin_paged_gather


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    """A broken copy of the oracle must fail some pin.  It runs in a child
    process: a mutant that crashes (e.g. by writing past its scratch) is
    caught too."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor not found: " + old
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as tmp:
        c_path = os.path.join(tmp, "m.c")
        so_path = os.path.join(tmp, "m.so")
        open(c_path, "w").write(mutated)
        subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", so_path, c_path, "-lm"],
                       check=True)
        code = ("import sys, json; sys.path[:0] = [%r, %r]; import test_oracle as t; "
                "print('CAUGHT=' + json.dumps(t.run_pins_on(%r)))"
                % (HERE, os.path.dirname(HERE), so_path))
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("CAUGHT=")]
        if r.returncode < 0:
            return  # the mutant was killed by a signal (e.g. a segfault): caught
        assert r.returncode == 0 and lines, r.stderr[-2000:]
        caught = json.loads(lines[-1][len("CAUGHT="):])
        print(name, "caught by", caught)
        assert caught, "mutant %s passed every pin" % name
