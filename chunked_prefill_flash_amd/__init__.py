"""Causal grouped-query flash-attention prefill against a cached prefix, for
AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of libattn_prefill.so (declared in
include/attn_prefill.h).  This module only checks and marshals arguments: it
passes device pointers, sizes and the current HIP stream to the library, and
every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and streams only.

The operation ("Inference Attention 2: Flash Prefill Against a Cached Prefix",
Lesson): q[C][32][64] holds a chunk of C query tokens at positions P..P+C-1;
kCache and vCache [P+C][8][64] hold every visible position; out[C][32][64]
(float32) receives causal attention with query head h reading KV head h/4 and
scale 1/8.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported first so the library binds to torch's HIP runtime

__all__ = ["attn_prefill", "attn_prefill_paged", "attn_prefill_paged_splitkv", "attn_prefill_rowwise",
           "attn_prefill_splitkv", "attn_prefill_splitkv_noalloc", "NOALLOC_SCRATCH_BYTES", "splitkv_workspace",
           "attn_naive", "naive_workspace", "validate", "paged_validate", "plan", "attn_prefill_clocked", "status_string",
           "library_path", "load_library", "flops", "visible_pairs", "AttnError", "EXPORTED_SYMBOLS", "HQ", "HKV",
           "D"]

HQ, HKV, D = 32, 8, 64
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn_prefill.so")
_lib = None

# Every function include/attn_prefill.h declares.
EXPORTED_SYMBOLS = ("attn_prefill", "attn_status_string", "attn_prefill_validate", "attn_prefill_plan",
                    "attn_prefill_version", "attn_prefill_paged", "attn_prefill_paged_validate",
                    "attn_prefill_rowwise", "attn_prefill_splitkv", "attn_prefill_splitkv_workspace",
                    "attn_naive", "attn_naive_workspace", "attn_prefill_splitkv_noalloc",
                    "attn_prefill_paged_splitkv", "attn_prefill_clocked")

# ATTN_NOALLOC_SCRATCH_BYTES of include/attn_prefill.h
NOALLOC_SCRATCH_BYTES = 16 << 20
CLOCK_WORDS = 8                  # ATTN_CLOCK_WORDS: clock-log words per workgroup

DTYPES = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_NULL_PTR", 3: "ATTN_ERR_UNSUPPORTED_DTYPE",
          4: "ATTN_ERR_MISALIGNED", 5: "ATTN_ERR_LAUNCH", 6: "ATTN_ERR_ALIAS", 7: "ATTN_ERR_WORKSPACE",
          8: "ATTN_ERR_TOO_LARGE"}


class AttnError(RuntimeError):
    """A nonzero attn_status_t from the library."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s returned %s (%d)" % (where, STATUS.get(code, "?"), code))


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libattn_prefill.so (built by __graft_entry__.build() or
    `python -m chunked_prefill_flash_amd.build`).  Raises if it is missing:
    there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libattn_prefill.so is not built (%s); run "
                           "`python -m chunked_prefill_flash_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.attn_prefill.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.attn_prefill.restype = i
    lib.attn_prefill_splitkv.argtypes = [vp, vp, vp, vp, i, i, i, vp, ctypes.c_size_t, vp]
    lib.attn_prefill_splitkv.restype = i
    lib.attn_prefill_splitkv_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.attn_prefill_splitkv_noalloc.restype = i
    lib.attn_prefill_splitkv_workspace.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int)]
    lib.attn_prefill_splitkv_workspace.restype = i
    lib.attn_naive.argtypes = [vp, vp, vp, vp, i, vp, ctypes.c_size_t, vp]
    lib.attn_naive.restype = i
    lib.attn_naive_workspace.argtypes = [i, ctypes.POINTER(ctypes.c_size_t)]
    lib.attn_naive_workspace.restype = i
    lib.attn_prefill_rowwise.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.attn_prefill_rowwise.restype = i
    lib.attn_prefill_validate.argtypes = [vp, vp, vp, vp, i, i, i]
    lib.attn_prefill_validate.restype = i
    lib.attn_prefill_plan.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_int)]
    lib.attn_prefill_plan.restype = i
    lib.attn_prefill_paged.argtypes = [vp, vp, vp, vp, i, i, vp, i, i, i, vp]
    lib.attn_prefill_paged.restype = i
    lib.attn_prefill_paged_splitkv.argtypes = [vp, vp, vp, vp, i, i, vp, i, i, i, vp, ctypes.c_size_t, vp]
    lib.attn_prefill_paged_splitkv.restype = i
    lib.attn_prefill_paged_validate.argtypes = [vp, vp, vp, vp, i, i, vp, i, i, i]
    lib.attn_prefill_paged_validate.restype = i
    lib.attn_prefill_clocked.argtypes = [vp, vp, vp, vp, i, i, i, vp, ctypes.c_size_t, vp]
    lib.attn_prefill_clocked.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_prefill_version.argtypes = []
    lib.attn_prefill_version.restype = i
    _lib = lib
    return lib


def _gpu_tensors(device, **tensors):
    """Every tensor contiguous and on `device` (a GPU)."""
    for name, t in tensors.items():
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
        if t.device != device:
            raise ValueError("%s is on %s, expected %s (all tensors on one device)" % (name, t.device, device))


def _out_tensor(out, C: int, device, stream) -> torch.Tensor:
    """The caller's out (checked) or a new float32 [C][32][64] on `device`,
    allocated on `stream` (the stream the kernels write it on)."""
    if out is None:
        with torch.cuda.stream(stream):
            return torch.empty((C, HQ, D), dtype=torch.float32, device=device)
    if out.dtype != torch.float32 or tuple(out.shape) != (C, HQ, D):
        raise ValueError("out must be float32 [C][32][64] = [%d][32][64], got %s %s"
                         % (C, out.dtype, tuple(out.shape)))
    _gpu_tensors(device, out=out)
    return out


def _workspace(workspace, need: int, device, stream) -> torch.Tensor:
    """The caller's workspace (checked for device and contiguity; the library
    checks its size) or a new one of `need` bytes.  A new one is allocated on
    `stream`, the stream the kernels use it on: torch's caching allocator then
    hands its memory to no other stream when it is freed on return, while the
    kernels may still be running."""
    if workspace is None:
        with torch.cuda.stream(stream):
            return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _gpu_tensors(device, workspace=workspace)
    return workspace


def _stream(stream, device):
    return stream if stream is not None else torch.cuda.current_stream(device)


def status_string(code: int) -> str:
    return load_library().attn_status_string(int(code)).decode()


def validate(q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, C: int, P: int, dtype_code: int) -> int:
    """Raw argument check of the C ABI (no GPU work); returns the status code."""
    return int(load_library().attn_prefill_validate(q_ptr, k_ptr, v_ptr, out_ptr, C, P, dtype_code))


def paged_validate(q_ptr: int, kp_ptr: int, vp_ptr: int, table_ptr: int, num_blocks: int, page_size: int,
                   out_ptr: int, C: int, P: int, dtype_code: int) -> int:
    """Raw argument check of attn_prefill_paged (no GPU work); returns the status code."""
    return int(load_library().attn_prefill_paged_validate(q_ptr, kp_ptr, vp_ptr, table_ptr, num_blocks,
                                                          page_size, out_ptr, C, P, dtype_code))


def plan(C: int, P: int, dtype=torch.float32, paged: bool = False) -> dict:
    """The launch decomposition the library uses for (C, P, dtype)."""
    code = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    arr = (ctypes.c_int * 8)()
    st = load_library().attn_prefill_plan(C, P, code, int(bool(paged)), arr)
    if st != 0:
        raise AttnError(st, "attn_prefill_plan")
    keys = ("rows_per_item", "key_splits", "grid", "threads", "items_per_workgroup", "keys_per_tile",
            "lds_bytes", "variant")
    return dict(zip(keys, list(arr)))


def visible_pairs(C: int, P: int) -> int:
    """(query row, key) pairs inside the causal edge, per query head."""
    return C * P + C * (C + 1) // 2


def flops(C: int, P: int) -> int:
    """Attention FLOPs of one call: 4*d per visible pair per query head."""
    return 4 * D * HQ * visible_pairs(C, P)


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
                 P: int | None = None, stream: torch.cuda.Stream | None = None, _entry: str = "attn_prefill"
                 ) -> torch.Tensor:
    """out[C][32][64] = causal GQA attention of q against the cache (k, v).

    q [C][32][64], k and v [P+C][8][64], all float32 or all bfloat16, contiguous,
    on one GPU.  out is float32 [C][32][64] (allocated if None).  P defaults to
    k.shape[0] - C.  Runs asynchronously on `stream` (default: current stream).
    """
    if q.dtype not in DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype in %s" % list(DTYPES))
    if q.dim() != 3 or q.shape[1:] != (HQ, D):
        raise ValueError("q must be [C][32][64], got %s" % tuple(q.shape))
    C = q.shape[0]
    if P is None:
        P = k.shape[0] - C
    if k.shape != (P + C, HKV, D) or v.shape != k.shape:
        raise ValueError("k and v must be [P+C][8][64] = [%d][8][64], got %s and %s"
                         % (P + C, tuple(k.shape), tuple(v.shape)))
    _gpu_tensors(q.device, q=q, k=k, v=v)
    s = _stream(stream, q.device)
    out = _out_tensor(out, C, q.device, s)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = getattr(lib, _entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), C, P, DTYPES[q.dtype],
                                  s.cuda_stream)
    if st != 0:
        raise AttnError(st, _entry)
    return out


def attn_prefill_clocked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
                         P: int | None = None, stream: torch.cuda.Stream | None = None,
                         clocks: torch.Tensor | None = None):
    """attn_prefill that also logs the clock: returns (out, clocks) with
    clocks an int64 [workgroups][CLOCK_WORDS] device tensor (not yet
    synchronised, zero where a mark was not written): (shader clock, 100 MHz
    counter) at each workgroup's start [0, 1] and end [2, 3], and the shader
    clock when its first work item's first tile is in LDS [4], when that
    item's key loop is done [5] and its output stored [6], and when a second
    item's first tile is in LDS [7].  A workgroup's clock in MHz is
    (c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * 100.  `clocks` may be given:
    a contiguous int64 device tensor of at least that many rows, written in
    place with nothing allocated or cleared (a mark not written keeps its old
    value), so that a timed loop can log one of its calls."""
    if q.dtype not in DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype in %s" % list(DTYPES))
    C = q.shape[0]
    if P is None:
        P = k.shape[0] - C
    if q.dim() != 3 or q.shape[1:] != (HQ, D) or k.shape != (P + C, HKV, D) or v.shape != k.shape:
        raise ValueError("bad shapes q %s k %s v %s for P=%d" % (tuple(q.shape), tuple(k.shape), tuple(v.shape), P))
    _gpu_tensors(q.device, q=q, k=k, v=v)
    grid = plan(C, P, q.dtype)["grid"] if C > 0 else 0
    s = _stream(stream, q.device)
    if clocks is None:
        with torch.cuda.stream(s):
            clocks = torch.zeros((max(grid, 1), CLOCK_WORDS), dtype=torch.int64, device=q.device)
    elif (clocks.dtype != torch.int64 or clocks.device != q.device or not clocks.is_contiguous()
          or clocks.dim() != 2 or clocks.shape[1] != CLOCK_WORDS or clocks.shape[0] < grid):
        raise ValueError("clocks must be a contiguous int64 [>= %d][%d] tensor on %s" % (grid, CLOCK_WORDS, q.device))
    out = _out_tensor(out, C, q.device, s)
    with torch.cuda.device(q.device):
        st = load_library().attn_prefill_clocked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), C, P,
                                                 DTYPES[q.dtype], clocks.data_ptr(), clocks.numel(), s.cuda_stream)
    if st != 0:
        raise AttnError(st, "attn_prefill_clocked")
    return out, clocks[:grid]


def attn_prefill_rowwise(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
                         P: int | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Same result as attn_prefill by the per-row starter algorithm (a timing
    baseline: every row re-reads its prefix).  Same arguments."""
    return attn_prefill(q, k, v, out=out, P=P, stream=stream, _entry="attn_prefill_rowwise")


def _paged_args(q, k_pages, v_pages, block_table, P):
    """Checks of the paged entry points; returns (C, numBlocks, pageSize)."""
    if q.dtype not in DTYPES or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q, k_pages, v_pages must share one dtype in %s" % list(DTYPES))
    if q.dim() != 3 or q.shape[1:] != (HQ, D):
        raise ValueError("q must be [C][32][64], got %s" % tuple(q.shape))
    if k_pages.dim() != 4 or k_pages.shape[2:] != (HKV, D) or v_pages.shape != k_pages.shape:
        raise ValueError("pages must be [numBlocks][pageSize][8][64], got %s and %s"
                         % (tuple(k_pages.shape), tuple(v_pages.shape)))
    C = q.shape[0]
    num_blocks, page_size = k_pages.shape[0], k_pages.shape[1]
    if num_blocks < 1 or page_size < 1:
        raise ValueError("pages must hold at least one page of at least one position, got %s" % (tuple(k_pages.shape),))
    if block_table.dtype != torch.int32 or block_table.dim() != 1 or \
            block_table.shape[0] < -(-(P + C) // page_size):
        raise ValueError("block_table must be int32 with at least ceil((P+C)/pageSize) entries")
    _gpu_tensors(q.device, q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table)
    return C, num_blocks, page_size


def attn_prefill_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                       P: int, out: torch.Tensor | None = None,
                       stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Causal GQA attention of q [C][32][64] against a paged cache.

    k_pages, v_pages: [numBlocks][pageSize][8][64], same dtype as q;
    block_table: int32 with at least ceil((P+C)/pageSize) physical page indices.
    Cache position t lives at slot t % pageSize of page block_table[t // pageSize].
    """
    C, num_blocks, page_size = _paged_args(q, k_pages, v_pages, block_table, P)
    s = _stream(stream, q.device)
    out = _out_tensor(out, C, q.device, s)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_prefill_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                    num_blocks, page_size, out.data_ptr(), C, P, DTYPES[q.dtype], s.cuda_stream)
    if st != 0:
        raise AttnError(st, "attn_prefill_paged")
    return out


def attn_prefill_paged_splitkv(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                               block_table: torch.Tensor, P: int, out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None,
                               stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """attn_prefill_paged with the key range split across workgroups and the
    partials merged (decode against a paged cache).  Arguments as for
    attn_prefill_paged; workspace as for attn_prefill_splitkv (at least
    splitkv_workspace(C, P, dtype)[0] bytes; allocated if None)."""
    C, num_blocks, page_size = _paged_args(q, k_pages, v_pages, block_table, P)
    s = _stream(stream, q.device)
    out = _out_tensor(out, C, q.device, s)
    workspace = _workspace(workspace, splitkv_workspace(C, P, q.dtype)[0], q.device, s)
    nbytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_prefill_paged_splitkv(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                            block_table.data_ptr(), num_blocks, page_size, out.data_ptr(), C, P,
                                            DTYPES[q.dtype], workspace.data_ptr(), nbytes, s.cuda_stream)
    if st != 0:
        raise AttnError(st, "attn_prefill_paged_splitkv")
    return out


def splitkv_workspace(C: int, P: int, dtype=torch.float32):
    """(bytes, splits): the workspace attn_prefill_splitkv needs and its key splits."""
    code = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    nbytes = ctypes.c_size_t()
    splits = ctypes.c_int()
    st = load_library().attn_prefill_splitkv_workspace(C, P, code, ctypes.byref(nbytes), ctypes.byref(splits))
    if st != 0:
        raise AttnError(st, "attn_prefill_splitkv_workspace")
    return int(nbytes.value), int(splits.value)


def attn_prefill_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
                         P: int | None = None, workspace: torch.Tensor | None = None,
                         stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Same result as attn_prefill with the key range split across workgroups
    and merged (for short chunks / decode against long prefixes).  workspace:
    a GPU tensor of at least splitkv_workspace(C, P, dtype)[0] bytes (allocated
    if None)."""
    if q.dtype not in DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype in %s" % list(DTYPES))
    C = q.shape[0]
    if P is None:
        P = k.shape[0] - C
    if q.dim() != 3 or q.shape[1:] != (HQ, D) or k.shape != (P + C, HKV, D) or v.shape != k.shape:
        raise ValueError("bad shapes q %s k %s v %s for P=%d" % (tuple(q.shape), tuple(k.shape), tuple(v.shape), P))
    _gpu_tensors(q.device, q=q, k=k, v=v)
    s = _stream(stream, q.device)
    out = _out_tensor(out, C, q.device, s)
    workspace = _workspace(workspace, splitkv_workspace(C, P, q.dtype)[0], q.device, s)
    nbytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_prefill_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), C, P, DTYPES[q.dtype],
                                      workspace.data_ptr(), nbytes, s.cuda_stream)
    if st != 0:
        raise AttnError(st, "attn_prefill_splitkv")
    return out


def attn_prefill_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                                 P: int | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """attn_prefill_splitkv with the key-split partials in the library's fixed
    per-device scratch array (NOALLOC_SCRATCH_BYTES) instead of a workspace:
    neither this call nor the library allocates anything, so `out` must be
    given.  Calls on one device share the array and must be ordered on one
    stream.  Raises AttnError (ATTN_ERR_TOO_LARGE) when the call's partials do
    not fit the array."""
    if q.dtype not in DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype in %s" % list(DTYPES))
    if out is None:
        raise ValueError("attn_prefill_splitkv_noalloc allocates nothing: pass out")
    C = q.shape[0]
    if P is None:
        P = k.shape[0] - C
    if q.dim() != 3 or q.shape[1:] != (HQ, D) or k.shape != (P + C, HKV, D) or v.shape != k.shape:
        raise ValueError("bad shapes q %s k %s v %s for P=%d" % (tuple(q.shape), tuple(k.shape), tuple(v.shape), P))
    _gpu_tensors(q.device, q=q, k=k, v=v)
    s = _stream(stream, q.device)
    out = _out_tensor(out, C, q.device, s)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_prefill_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), C, P,
                                              DTYPES[q.dtype], s.cuda_stream)
    if st != 0:
        raise AttnError(st, "attn_prefill_splitkv_noalloc")
    return out


def naive_workspace(T: int) -> int:
    """Bytes of score-matrix workspace attn_naive needs (32*T*T*4)."""
    nbytes = ctypes.c_size_t()
    st = load_library().attn_naive_workspace(T, ctypes.byref(nbytes))
    if st != 0:
        raise AttnError(st, "attn_naive_workspace")
    return int(nbytes.value)


def attn_naive(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Causal prompt prefill (P = 0) by the three-kernel pipeline with the full
    32 x T x T score matrix in `workspace` (allocated if None).  fp32 only."""
    if q.dtype != torch.float32 or k.dtype != torch.float32 or v.dtype != torch.float32:
        raise TypeError("attn_naive takes float32 tensors")
    T = q.shape[0]
    if q.shape != (T, HQ, D) or k.shape != (T, HKV, D) or v.shape != k.shape:
        raise ValueError("q [T][32][64], k and v [T][8][64] expected")
    _gpu_tensors(q.device, q=q, k=k, v=v)
    s = _stream(stream, q.device)
    out = _out_tensor(out, T, q.device, s)
    workspace = _workspace(workspace, naive_workspace(T), q.device, s)
    nbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = load_library().attn_naive(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), T,
                                       workspace.data_ptr(), nbytes, s.cuda_stream)
    if st != 0:
        raise AttnError(st, "attn_naive")
    return out
