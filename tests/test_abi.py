"""The C-ABI library loads and exports every function include/*.h declares;
argument validation and the launch plan behave as documented.  Nothing here
touches a GPU: only host-side entry points are called."""
import ctypes
import glob
import os
import re
import subprocess

import pytest
import torch

import chunked_prefill_flash_amd as cpf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, NULLP, DTYPE, MISAL, LAUNCH, ALIAS, WORKSPACE = range(8)
F32, BF16 = 0, 1
A = 0x10000000          # fake, 16-byte aligned addresses: never dereferenced
MB = 1 << 20


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cpf.library_path()):
        pytest.fail("library not built: run `python -m chunked_prefill_flash_amd.build`")
    return cpf.load_library()


def test_header_declares_the_binding_symbols():
    assert declared_functions() == set(cpf.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", cpf.library_path()], capture_output=True, text=True)
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if ln.strip()}
    assert declared_functions() <= exported


def test_binding_constants_match_the_header():
    src = open(os.path.join(os.path.dirname(__file__), "..", "include", "attn_prefill.h")).read()
    defs = dict(re.findall(r"#define (ATTN_\w+) \(?([^)\n]*)\)?", src))
    assert int(defs["ATTN_CLOCK_WORDS"]) == cpf.CLOCK_WORDS
    base, shift = re.fullmatch(r"(\d+)u << (\d+)", defs["ATTN_NOALLOC_SCRATCH_BYTES"]).groups()
    assert int(base) << int(shift) == cpf.NOALLOC_SCRATCH_BYTES


def test_library_contains_gfx950_code():
    blob = open(cpf.library_path(), "rb").read()
    assert b"gfx950" in blob


def test_version(lib):
    assert lib.attn_prefill_version() >= 100


def test_status_strings(lib):
    for code, name in cpf.STATUS.items():
        assert cpf.status_string(code) == name
    assert cpf.status_string(99) == "ATTN_ERR_UNKNOWN"


def v(q=A, k=A + 64 * MB, vv=A + 128 * MB, out=A + 192 * MB, C=17, P=31, dt=F32):
    return cpf.validate(q, k, vv, out, C, P, dt)


def test_validate_accepts_good_arguments():
    assert v() == OK
    assert v(dt=BF16) == OK
    assert v(C=1, P=0) == OK


def test_validate_codes():
    assert v(dt=2) == DTYPE
    assert v(dt=-1) == DTYPE
    assert v(C=-1) == INVALID
    assert v(P=-1) == INVALID
    assert v(C=2 ** 31 - 10, P=100) == INVALID          # P + C overflows int
    assert v(q=0) == NULLP
    assert v(k=0) == NULLP
    assert v(vv=0) == NULLP
    assert v(out=0) == NULLP
    assert v(q=A + 4) == MISAL
    assert v(out=A + 192 * MB + 8) == MISAL
    assert v(k=A + 64 * MB + 2, dt=BF16) == MISAL


def test_validate_zero_chunk_is_noop_even_without_pointers():
    assert v(q=0, k=0, vv=0, out=0, C=0, P=5) == OK


def test_validate_alias():
    # out overlapping q, k or v is rejected; adjacent buffers are fine
    C, P = 17, 31
    qbytes = C * 32 * 64 * 4
    assert v(out=A, q=A) == ALIAS
    assert v(out=A + qbytes - 16, q=A) == ALIAS
    assert v(out=A + qbytes, q=A) == OK
    assert v(out=A + 64 * MB + 1024, k=A + 64 * MB) == ALIAS
    assert v(out=A + 128 * MB, vv=A + 128 * MB) == ALIAS


def test_plan_shapes():
    p = cpf.plan(2048, 2048)
    assert p["threads"] == 64 * (p["rows_per_item"] // 8) * p["key_splits"]
    assert p["grid"] % 8 == 0
    # every row tile of every KV group is covered exactly once
    tiles = -(-2048 // p["rows_per_item"])
    assert p["grid"] // 8 * p["items_per_workgroup"] >= tiles
    assert p["lds_bytes"] <= 160 * 1024
    for C in (1, 17, 33, 255, 256, 511, 512, 1023, 1024, 2047, 2048, 4096, 65536):
        for dt in (torch_f32(), torch_bf16()):
            pp = cpf.plan(C, 100, dt)
            t = -(-C // pp["rows_per_item"])
            per = pp["items_per_workgroup"]
            assert pp["grid"] == 8 * (-(-t // per) if per == 2 else t)
            assert pp["lds_bytes"] <= 160 * 1024
    assert cpf.plan(0, 5)["grid"] == 0


def pv(q=A, kp=A + 64 * MB, vp=A + 128 * MB, tab=A + 192 * MB, nb=10, ps=16, out=A + 256 * MB, C=17, P=31,
       dt=F32):
    return cpf.paged_validate(q, kp, vp, tab, nb, ps, out, C, P, dt)


def test_paged_validate_codes():
    assert pv() == OK
    assert pv(dt=BF16) == OK
    assert pv(dt=5) == DTYPE
    assert pv(ps=0) == INVALID
    assert pv(nb=0) == INVALID
    assert pv(C=-1) == INVALID
    assert pv(nb=1 << 20, ps=16) == INVALID            # pool beyond 32-bit offsets (16M rows x 2 KiB)
    big_tab = dict(C=1, ps=1, tab=A + 320 * MB)          # table placed after out: no overlap
    assert pv(P=(1 << 30) - 1, **big_tab) == INVALID     # 2^30 entries: 4 GiB, beyond 32-bit offsets
    assert pv(P=(1 << 30) - 2, **big_tab) == OK          # 2^30 - 1 entries fit
    assert pv(q=0, kp=0, vp=0, tab=0, out=0, C=0) == OK
    assert pv(tab=0) == NULLP
    assert pv(tab=A + 192 * MB + 2) == MISAL
    assert pv(tab=A + 192 * MB + 4) == OK              # the table needs 4-byte alignment only
    assert pv(kp=A + 64 * MB + 8) == MISAL
    assert pv(out=A + 192 * MB, tab=A + 192 * MB) == ALIAS
    assert pv(out=A + 64 * MB, kp=A + 64 * MB) == ALIAS


def test_paged_splitkv_rejections():
    """The paged checks of attn_prefill_paged plus the workspace checks of
    attn_prefill_splitkv, before any device call (fake pointers)."""
    lib = cpf.load_library()
    need, _ = cpf.splitkv_workspace(4, 1000)
    f = lib.attn_prefill_paged_splitkv
    base = dict(q=A, kp=A + 64 * MB, vp=A + 128 * MB, tab=A + 192 * MB, nb=80, ps=16, out=A + 196 * MB, C=4, P=1000)

    def call(ws, nbytes, **kw):
        a = dict(base, **kw)
        return f(a["q"], a["kp"], a["vp"], a["tab"], a["nb"], a["ps"], a["out"], a["C"], a["P"], F32, ws, nbytes,
                 None)
    ws = A + 256 * MB
    assert call(ws, need - 16) == WORKSPACE
    assert call(None, need) == NULLP
    assert call(ws + 4, need) == MISAL
    assert call(A + 64 * MB, need) == ALIAS            # workspace on the K pool
    assert call(A + 192 * MB, need) == ALIAS           # workspace on the table
    assert call(ws, need, ps=0) == INVALID             # the paged checks come first
    assert call(ws, need, tab=None) == NULLP
    assert call(ws, need, C=0) == OK                   # nothing to do


def test_fp32_plans_balance_causal_work():
    """Row-tile height and pairing per shape (see the planner's makespan
    estimate): (rows per item, workgroups, items per workgroup)."""
    want = {(2048, 2048): (32, 256, 2), (2048, 0): (32, 256, 2), (512, 15872): (16, 256, 1),
            (1024, 0): (16, 512, 1), (1536, 0): (8, 1536, 1), (512, 0): (8, 512, 1), (600, 0): (16, 304, 1),
            (255, 3): (8, 256, 1), (1000, 13): (16, 504, 1), (1500, 100): (8, 1504, 1), (2049, 7): (16, 1032, 1),
            (1024, 16384): (32, 256, 1), (1100, 0): (16, 552, 1),
            (17, 31): (8, 24, 1), (768, 0): (16, 384, 1), (1530, 0): (8, 1536, 1), (768, 2000): (8, 768, 1),
            (1100, 4400): (8, 1104, 1), (300, 3000): (8, 304, 1), (1400, 0): (16, 704, 1),
            (2560, 1000): (16, 1280, 1), (4096, 0): (32, 512, 2), (900, 1000): (16, 456, 1)}
    for (C, P), w in want.items():
        p = cpf.plan(C, P)
        assert (p["rows_per_item"], p["grid"], p["items_per_workgroup"]) == w, (C, P, p)


def test_one_staging_buffer_only_where_its_items_fill_whole_rounds():
    """The one-stage shapes (64 KiB of K/V tiles and 1 KiB per Q row of LDS,
    two workgroups per CU: 512 slots) are planned for plain chunks: 8-row
    items below 1800 rows whose workgroups (one per 8 rows and KV group) fill
    one round, whole rounds or more than two rounds and most of a third of the
    slots, or whose prefix (P >= C) makes the items alike, except past P = 8C
    where 16- or 32-row items fill exactly 256 workgroups (paged caches, with
    the row offsets of two tiles in LDS: one round, or more rounds from 1025
    rows against prefixes of 8C); 16-row items at
    C = 961..1024 with P <= 4C, and at C = 880..960 with C <= P <= 4C (plain
    caches only)."""
    ONE_STAGE, ONE_STAGE16 = 7, 8
    for C, P in [(512, 0), (1024 + 512, 0), (1530, 0), (1500, 100), (512, 128), (512, 129), (257, 0),
                 (100, 0), (384, 1000), (768, 2000), (1536, 1536), (1100, 8800), (1100, 12000), (640, 10000),
                 (1792, 1792)]:
        p = cpf.plan(C, P)
        assert p["variant"] == ONE_STAGE and p["lds_bytes"] == 65536 + 1024 * 8, (C, P, p)
        pp = cpf.plan(C, P, paged=True)   # paged: one round, or more from 1025 rows against P >= 8C
        if p["grid"] <= 512 or (C > 1024 and P >= 8 * C):
            assert pp["variant"] == ONE_STAGE and pp["lds_bytes"] == 65536 + 1024 * 8 + 2 * 4 * 128, (C, P, pp)
        else:
            assert pp["variant"] != ONE_STAGE, (C, P, pp)
    for C, P in [(768, 0), (896, 0), (960, 0), (1024, 0), (512, 15872), (512, 8000), (1024, 16000), (2048, 0),
                 (2048, 2048), (1792, 1000), (1900, 1900), (2000, 1000)]:
        assert cpf.plan(C, P)["variant"] != ONE_STAGE, (C, P)
    for C, P in [(880, 880), (896, 896), (960, 3840), (961, 0), (1000, 13), (1024, 0), (1024, 4096)]:
        p = cpf.plan(C, P)
        assert p["variant"] == ONE_STAGE16 and p["lds_bytes"] == 65536 + 1024 * 16 and p["grid"] <= 512, (C, P, p)
        assert cpf.plan(C, P, paged=True)["variant"] != ONE_STAGE16
    for C, P in [(879, 879), (880, 0), (960, 959), (1025, 0), (1024, 4097), (768, 0)]:
        assert cpf.plan(C, P)["variant"] != ONE_STAGE16, (C, P)


def test_long_chunk_workgroup_shapes():
    for paged in (False, True):
        assert cpf.plan(2048, 2048, paged=paged)["threads"] == 1024          # fp32: 32 rows, 16 waves
        bf = cpf.plan(2048, 2048, dtype=torch.bfloat16, paged=paged)            # bf16: 32 rows, unpaired,
        assert (bf["threads"], bf["grid"], bf["items_per_workgroup"]) == (512, 512, 1)   # two per CU
    for paged in (False, True):                                             # bf16: 64 rows, paired
        bf = cpf.plan(4096, 28672, dtype=torch.bfloat16, paged=paged)
        assert (bf["rows_per_item"], bf["threads"], bf["grid"], bf["items_per_workgroup"]) == (64, 1024, 256, 2)


def test_splitkv_workspace_sizes():
    nb, ns = cpf.splitkv_workspace(1, 32767)
    assert ns > 1 and nb == ns * 1 * 32 * 66 * 4
    nb, ns = cpf.splitkv_workspace(17, 31)
    assert ns >= 1 and nb == ns * 17 * 32 * 66 * 4
    assert cpf.splitkv_workspace(0, 10) == (0, 0)
    # splits never exceed the cache length in staged tiles, and always cover it
    for C, P in [(1, 0), (1, 100), (5, 4000), (64, 100000), (300, 3000)]:
        nb, ns = cpf.splitkv_workspace(C, P)
        assert 1 <= ns <= max(1, (P + C + 63) // 64)
    with pytest.raises(cpf.AttnError):
        cpf.splitkv_workspace(-1, 0)


def test_noalloc_rejects_before_any_device_call(lib):
    """Argument errors and calls whose partials exceed the fixed scratch array
    return before any HIP call (fake pointers, never dereferenced)."""
    TOO_LARGE = 8
    f = lib.attn_prefill_splitkv_noalloc
    assert f(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, -1, 0, F32, None) == INVALID
    assert f(None, A + 64 * MB, A + 128 * MB, A + 192 * MB, 4, 10, F32, None) == NULLP
    assert f(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 4, 10, 7, None) == DTYPE
    assert f(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 0, 10, F32, None) == OK      # C == 0: nothing to do
    for C, P in [(4096, 100), (2048, 0), (1990, 5000)]:
        need, _ = cpf.splitkv_workspace(C, P)
        assert need > cpf.NOALLOC_SCRATCH_BYTES
        assert f(A, A + 64 * MB, A + 128 * MB, A + 256 * MB, C, P, F32, None) == TOO_LARGE
    assert cpf.status_string(TOO_LARGE) == "ATTN_ERR_TOO_LARGE"


def test_splitkv_rejects_small_or_missing_workspace():
    import ctypes
    lib = cpf.load_library()
    need, _ = cpf.splitkv_workspace(4, 1000)
    args = (A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 4, 1000, F32)
    assert lib.attn_prefill_splitkv(*args, A + 256 * MB, need - 16, None) == WORKSPACE
    assert lib.attn_prefill_splitkv(*args, None, need, None) == NULLP
    assert lib.attn_prefill_splitkv(*args, A + 256 * MB + 4, need, None) == MISAL
    assert lib.attn_prefill_splitkv(*args, A + 192 * MB, need, None) == ALIAS    # workspace on out


def test_naive_workspace_and_rejections():
    lib = cpf.load_library()
    assert cpf.naive_workspace(0) == 0
    assert cpf.naive_workspace(17) == 32 * 17 * 17 * 4
    assert cpf.naive_workspace(2048) == 32 * 2048 * 2048 * 4 == 512 * MB
    with pytest.raises(cpf.AttnError):
        cpf.naive_workspace(-1)
    with pytest.raises(cpf.AttnError):
        cpf.naive_workspace(46341)
    T = 100
    need = cpf.naive_workspace(T)
    args = (A, A + 64 * MB, A + 128 * MB, A + 192 * MB, T)
    assert lib.attn_naive(*args, A + 256 * MB, need - 4, None) == WORKSPACE
    assert lib.attn_naive(*args, None, need, None) == NULLP
    assert lib.attn_naive(*args, A + 256 * MB + 4, need, None) == MISAL
    assert lib.attn_naive(*args, A + 128 * MB, need, None) == ALIAS       # workspace on v
    assert lib.attn_naive(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, -1, A + 256 * MB, need, None) == 1
    assert lib.attn_naive(None, None, None, None, 0, None, 0, None) == 0  # T = 0 is a no-op


def test_plan_errors():
    with pytest.raises(cpf.AttnError):
        cpf.plan(-1, 0)
    with pytest.raises(cpf.AttnError):
        cpf.plan(1, 0, 7)


def test_chunk_length_limit():
    """Chunks up to 2^25 rows and caches up to 2^30 positions (more than any
    GPU's memory holds) are planned with positive, exact grids in every mode;
    larger ones are rejected before any launch arithmetic could overflow."""
    big = 1 << 25
    for dt in (torch.float32, torch.bfloat16):
        for paged in (False, True):
            for P in (0, 2 ** 30 - big):
                p = cpf.plan(big, P, dt, paged)
                items = (big + p["rows_per_item"] - 1) // p["rows_per_item"]
                assert p["grid"] * p["items_per_workgroup"] >= items * 8 > 0
            with pytest.raises(cpf.AttnError):
                cpf.plan(big + 1, 0, dt, paged)
            with pytest.raises(cpf.AttnError):
                cpf.plan(2 ** 31 - 1, 0, dt, paged)
            with pytest.raises(cpf.AttnError):
                cpf.plan(big, 2 ** 30 - big + 1, dt, paged)
    far = dict(q=A, k=A + (1 << 40), vv=A + (2 << 40), out=A + (3 << 40))   # no overlap at 2^25 rows
    assert v(C=big, P=0, **far) == OK
    assert v(C=big + 1, P=0, **far) == INVALID
    nb, ns = cpf.splitkv_workspace(big, 1000)
    assert ns >= 1 and nb == ns * big * 32 * 66 * 4
    with pytest.raises(cpf.AttnError):
        cpf.splitkv_workspace(big + 1, 0)


def torch_f32():
    import torch
    return torch.float32


def torch_bf16():
    import torch
    return torch.bfloat16


def test_flop_count():
    # 4*d FLOPs per visible (row, key) pair per query head
    assert cpf.visible_pairs(1, 0) == 1
    assert cpf.visible_pairs(2048, 2048) == 2048 * 2048 + 2048 * 2049 // 2
    assert cpf.flops(2048, 2048) == 8192 * 6_292_480 == 51_547_996_160


def test_binding_rejects_bad_tensors_without_gpu():
    import torch
    q = torch.zeros(3, 32, 64)
    k = torch.zeros(5, 8, 64)
    with pytest.raises(ValueError):      # CPU tensors are refused before any library call
        cpf.attn_prefill(q, k, k)
    with pytest.raises(TypeError):
        cpf.attn_prefill(q.double(), k.double(), k.double())
    with pytest.raises(ValueError):
        cpf.attn_prefill(q, torch.zeros(4, 8, 64), torch.zeros(4, 8, 64), P=2)


def test_every_binding_rejects_host_tensors_and_bad_shapes():
    """Each wrapper checks dtypes, shapes and placement before it calls the
    library (none of these reach a kernel)."""
    import torch
    q = torch.zeros(3, 32, 64)
    k = torch.zeros(5, 8, 64)
    table = torch.zeros(1, dtype=torch.int32)
    pages = torch.zeros(2, 16, 8, 64)
    with pytest.raises(ValueError):
        cpf.attn_prefill_paged(q, pages, pages, table, 2)
    with pytest.raises(TypeError):
        cpf.attn_prefill_paged(q, pages.double(), pages.double(), table, 2)
    with pytest.raises(ValueError):
        cpf.attn_prefill_paged(q, pages, pages, table.long(), 2)
    with pytest.raises(ValueError):
        cpf.attn_prefill_splitkv(q, k, k)
    with pytest.raises(ValueError):
        cpf.attn_prefill_rowwise(q, k, k)
    with pytest.raises(TypeError):
        cpf.attn_naive(q.bfloat16(), k.bfloat16(), k.bfloat16())
    with pytest.raises(ValueError):
        cpf.attn_naive(q, torch.zeros(3, 8, 64), torch.zeros(3, 8, 64))
    with pytest.raises(ValueError):
        cpf.attn_naive(q, torch.zeros(4, 8, 64), torch.zeros(4, 8, 64))
    with pytest.raises(ValueError):   # pages of no positions
        cpf.attn_prefill_paged(q, torch.zeros(2, 0, 8, 64), torch.zeros(2, 0, 8, 64), table, 2)
    with pytest.raises(TypeError):    # dtype checked before the plan lookup
        cpf.attn_prefill_clocked(q.double(), k.double(), k.double(), P=2)
    with pytest.raises(ValueError):
        cpf.attn_prefill_clocked(q, torch.zeros(4, 8, 64), torch.zeros(4, 8, 64), P=2)
