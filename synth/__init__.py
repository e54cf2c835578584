"""Seeded synthetic inputs for causal GQA attention over a cached prefix.

This module only draws numbers and places them in arrays.  It holds none of
the attention arithmetic, so both the CPU oracle and the GPU path can be fed
from it without sharing any of the method.

Random numbers
--------------
* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state_n = seed + n * 0x9E3779B97F4A7C15, output
  mixed by the published 30/27/31 shift-xor-multiply finaliser.
* 53-bit uniforms in (0, 1]: ((x >> 11) + 1) * 2**-53.
* Normal deviates by the Box-Muller transform (Box and Muller, 1958): each
  pair of uniforms (u1, u2) yields sqrt(-2 ln u1) * cos(2 pi u2) and
  sqrt(-2 ln u1) * sin(2 pi u2).
* Everything is computed in float64 and rounded once to float32.

Shapes follow the tensor contract of "Inference Attention 2: Flash Prefill
Against a Cached Prefix" (Lesson): q is [C][32][64], the K and V caches are
[P+C][8][64], out is [C][32][64].

Hazards ("Inference Attention 2", Lesson, the paragraph on planted hazards):
a planted position carries 4.0 in query head 0 and KV head 0, so a planted
query against a planted key scores 4*4*64/8 = 128.
"""
from __future__ import annotations

import numpy as np

HQ = 32          # query heads
HKV = 8          # key/value heads
D = 64           # head dimension
PLANT_VALUE = 4.0

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start+1 .. start+n of the SplitMix64 stream for `seed` (uint64)."""
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def uniform53(seed: int, n: int, start: int = 0) -> np.ndarray:
    """n float64 uniforms in (0, 1], 53 random bits each."""
    x = splitmix64(seed, n, start) >> np.uint64(11)
    return (x.astype(np.float64) + 1.0) * (2.0 ** -53)


def normal_f32(seed: int, n: int) -> np.ndarray:
    """n N(0,1) deviates (Box-Muller in float64, one rounding to float32)."""
    m = (n + 1) // 2
    u = uniform53(seed, 2 * m)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * np.pi * u2
    z = np.empty(2 * m, dtype=np.float64)
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    return z[:n].astype(np.float32)


def draw_distinct(seed: int, lo: int, hi: int, k: int) -> list[int]:
    """k distinct integers from [lo, hi), by a partial Fisher-Yates shuffle
    driven by SplitMix64 (modulo reduction; the bias is below 2**-40 here)."""
    n = hi - lo
    if k > n:
        raise ValueError("cannot draw %d distinct values from %d" % (k, n))
    pool = list(range(lo, hi))
    r = splitmix64(seed, k)
    for t in range(k):
        j = t + int(r[t] % np.uint64(n - t))
        pool[t], pool[j] = pool[j], pool[t]
    return sorted(pool[:k])


def qkv_normal(C: int, P: int, seed_q: int, seed_k: int, seed_v: int):
    """q [C][32][64] and K/V caches [P+C][8][64], i.i.d. N(0,1), float32."""
    T = P + C
    q = normal_f32(seed_q, C * HQ * D).reshape(C, HQ, D)
    k = normal_f32(seed_k, T * HKV * D).reshape(T, HKV, D)
    v = normal_f32(seed_v, T * HKV * D).reshape(T, HKV, D)
    return q, k, v


def plant(q: np.ndarray, k: np.ndarray, v: np.ndarray, P: int, positions,
          value: float = PLANT_VALUE, plant_q: bool = True) -> None:
    """Write `value` into all 64 dims of query head 0 (chunk row pos-P) and
    of KV head 0 of the K and V caches, at every absolute position `pos`."""
    C = q.shape[0]
    for pos in positions:
        if not (0 <= pos < k.shape[0]):
            raise ValueError("plant position %d outside the cache" % pos)
        k[pos, 0, :] = value
        v[pos, 0, :] = value
        if plant_q:
            if not (P <= pos < P + C):
                raise ValueError("query plant %d outside the chunk" % pos)
            q[pos - P, 0, :] = value


def poison_bits() -> int:
    """Quiet-NaN bit pattern written into every output element before a call."""
    return 0x7FC00000


# --------------------------------------------------------------------------
# Named workloads.  Seeds follow one rule: 100*case + 1/2/3 for q/k/v and
# 100*case + 7 for plant positions.
# --------------------------------------------------------------------------

def case_planted_chunk(C: int = 17, P: int = 31, seed_base: int = 100, n_plants: int = 3):
    """Chunk C at prefix P with n_plants 4.0 plants drawn from the chunk's
    own positions [P, P+C) (so a planted query meets its planted key)."""
    q, k, v = qkv_normal(C, P, seed_base + 1, seed_base + 2, seed_base + 3)
    pos = draw_distinct(seed_base + 7, P, P + C, min(n_plants, C))
    plant(q, k, v, P, pos)
    return q, k, v, pos


def case_plain(C: int, P: int, seed_base: int):
    """q/k/v i.i.d. N(0,1), no plants."""
    return qkv_normal(C, P, seed_base + 1, seed_base + 2, seed_base + 3)


def case_last_key(C: int = 512, P: int = 15872, seed_base: int = 400):
    """Only the final cache position P+C-1 is planted (query row C-1 head 0,
    K/V head 0), so that row's maximum first appears in its last tile."""
    q, k, v = qkv_normal(C, P, seed_base + 1, seed_base + 2, seed_base + 3)
    pos = [P + C - 1]
    plant(q, k, v, P, pos)
    return q, k, v, pos


def case_monotone(C: int, P: int, seed_base: int = 900):
    """Query head 0 rows all ones and K head 0 row j equal to 0.01*j, so every
    head-0 score grows with the key position and each row's maximum is its own
    diagonal key, met in that row's last tile."""
    q, k, v = qkv_normal(C, P, seed_base + 1, seed_base + 2, seed_base + 3)
    q[:, 0, :] = 1.0
    T = P + C
    k[:, 0, :] = (0.01 * np.arange(T, dtype=np.float64)).astype(np.float32)[:, None]
    return q, k, v


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even), returned as uint16
    bit patterns.  Inputs here are finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_pages(k: np.ndarray, v: np.ndarray, page_size: int, seed: int, spare_pages: int = 3,
             fill: float = float("nan")):
    """Scatter a contiguous cache [T][8][64] into pages [numBlocks][page_size][8][64]
    in a seeded shuffled order ("FlashAttention and inference kernels",
    PagedAttention: position t lives at slot t % page_size of physical page
    table[t // page_size]).  spare_pages unused pages are added; every slot not
    holding a cache position is `fill` (NaN by default), so reading a wrong page
    or slot shows up.  Returns (k_pages, v_pages, table int32)."""
    T = k.shape[0]
    nlog = -(-T // page_size)
    nb = nlog + spare_pages
    order = list(range(nb))
    r = splitmix64(seed, nb)
    for t in range(nb - 1, 0, -1):            # Fisher-Yates over the physical pages
        j = int(r[t] % np.uint64(t + 1))
        order[t], order[j] = order[j], order[t]
    table = np.array(order[:nlog], dtype=np.int32)
    kp = np.full((nb, page_size) + k.shape[1:], fill, dtype=np.float32)
    vp = np.full((nb, page_size) + v.shape[1:], fill, dtype=np.float32)
    for b in range(nlog):
        lo, hi = b * page_size, min(T, (b + 1) * page_size)
        kp[table[b], : hi - lo] = k[lo:hi]
        vp[table[b], : hi - lo] = v[lo:hi]
    return kp, vp, table


def case_long_cache(C: int, P: int, seed_base: int = 1100, k_scale: float = 6.0, band: int = 4096):
    """A cache too long to fill with i.i.d. draws cheaply (P+C positions,
    typically past 2^20 so fp32 byte offsets pass 2^31).

    q is i.i.d. N(0,1).  Three bands of positions hold i.i.d. draws, K scaled
    by k_scale so their scores dominate the softmax: [0, band), `band`
    positions centred on position 2^20 (the first position whose fp32 K/V
    rows start at byte 2^31), and the last 2*band positions (the chunk and
    the keys just before it).  Elsewhere K is zero (score 0) and V repeats a
    17-position pattern of multiples of 1/8 in [-1, 1]; 2^20 is not a
    multiple of 17, so a row read from a wrapped offset differs."""
    T = P + C
    q = normal_f32(seed_base + 1, C * HQ * D).reshape(C, HQ, D)
    k = np.zeros((T, HKV, D), dtype=np.float32)
    period = 17
    j = np.arange(period, dtype=np.int64)[:, None, None]
    g = np.arange(HKV, dtype=np.int64)[None, :, None]
    d = np.arange(D, dtype=np.int64)[None, None, :]
    pattern = (((5 * j + 3 * g + d) % 17) - 8).astype(np.float32) / 8.0
    v = pattern[np.arange(T, dtype=np.int64) % period]
    mid = 1 << 20
    bands = [(0, band), (mid - band // 2, mid + band // 2), (T - 2 * band, T)]
    for t, (lo, hi) in enumerate(bands):
        lo, hi = max(0, lo), min(T, hi)
        if hi <= lo:
            continue
        n = (hi - lo) * HKV * D
        k[lo:hi] = (k_scale * normal_f32(seed_base + 2 + 10 * t, n).astype(np.float64)).astype(
            np.float32).reshape(hi - lo, HKV, D)
        v[lo:hi] = normal_f32(seed_base + 3 + 10 * t, n).reshape(hi - lo, HKV, D)
    return q, k, v, bands
