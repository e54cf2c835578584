"""Calls the host-side entry points of a library build (plan, split-KV
workspace, argument validation, paged validation, naive workspace) over
extreme and seeded random sizes.  Run by test_host_ubsan.py against a build
whose host code is instrumented with UndefinedBehaviorSanitizer; no GPU call
is made.  Usage: python host_fuzz.py LIBRARY N_RANDOM"""
import ctypes
import random
import sys

lib = ctypes.CDLL(sys.argv[1])
n_random = int(sys.argv[2])
vp, i = ctypes.c_void_p, ctypes.c_int
lib.attn_prefill_plan.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_int)]
lib.attn_prefill_validate.argtypes = [vp, vp, vp, vp, i, i, i]
lib.attn_prefill_splitkv_workspace.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int)]
lib.attn_prefill_paged_validate.argtypes = [vp, vp, vp, vp, i, i, vp, i, i, i]
lib.attn_naive_workspace.argtypes = [i, ctypes.POINTER(ctypes.c_size_t)]
plan = (ctypes.c_int * 8)()
nbytes, nsplits = ctypes.c_size_t(), ctypes.c_int()
IMAX = 2 ** 31 - 1
A = 0x10000000                       # fake, aligned, far-apart addresses: never dereferenced
q, k, v, out, table = A, A + (1 << 40), A + (2 << 40), A + (3 << 40), A + (4 << 40)
edges = [0, 1, 2, 7, 8, 31, 32, 63, 64, 127, 128, 255, 256, 879, 880, 960, 961, 1024, 1025, 1100, 1599, 1600,
         1800, 2047, 2048, 4095, 4096, 2 ** 20, 2 ** 25 - 1, 2 ** 25, 2 ** 25 + 1, 2 ** 26, 2 ** 30 - 1, 2 ** 30, IMAX, -1,
         -IMAX - 1]
rng = random.Random(7)
chunks = edges + [int(2 ** rng.uniform(0, 31)) for _ in range(n_random)]
calls = 0
for C in chunks:
    lim = (1 << 30) - C if 0 <= C <= (1 << 25) else 0
    prefixes = rng.sample(edges, 8) + [int(2 ** rng.uniform(0, 31)) for _ in range(4)]
    if lim > 0:
        prefixes += [lim, lim - 1, lim // 2, rng.randrange(lim)]
    for P in prefixes:
        for dt in (0, 1, 2, -1):
            for paged in (0, 1):
                lib.attn_prefill_plan(C, P, dt, paged, plan)
            lib.attn_prefill_splitkv_workspace(C, P, dt, ctypes.byref(nbytes), ctypes.byref(nsplits))
            lib.attn_prefill_validate(q, k, v, out, C, P, dt)
            for page, blocks in ((16, 1 << 20), (1, 3), (rng.randrange(1, 5000), rng.randrange(1, 1 << 24)),
                                 (IMAX, IMAX), (0, 5), (5, 0)):
                lib.attn_prefill_paged_validate(q, k, v, table, blocks, page, out, C, P, dt)
            calls += 9
    lib.attn_naive_workspace(C, ctypes.byref(nbytes))
    calls += 1
print("host_fuzz: %d calls" % calls)
