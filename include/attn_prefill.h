/*
 * attn_prefill.h -- C ABI of the causal grouped-query flash-attention prefill
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operation ("Inference Attention 2: Flash Prefill Against a Cached
 * Prefix", Lesson): a chunk of C new query tokens at absolute positions
 * P .. P+C-1 attends causally to a key/value cache holding positions
 * 0 .. P+C-1, so chunk row i sees cache positions j <= P + i.  There are 32
 * query heads and 8 key/value heads of size 64; query head h reads KV head
 * h / 4; the score scale is exactly 1/8.  For every row i, head h (g = h/4)
 * and dim d:
 *
 *     s_j          = (1/8) * sum_k q[i][h][k] * kCache[j][g][k],  j <= P + i
 *     out[i][h][d] = sum_j softmax_j(s)_j * vCache[j][g][d]
 *
 * computed in one pass over key/value tiles with an online softmax (running
 * maximum, running denominator, accumulator rescaled when the maximum moves,
 * one division at the end), with no score matrix and no workspace ("Inference
 * Attention 2", Lesson, the four update equations; "FlashAttention and
 * inference kernels", section "FlashAttention: tiling plus online softmax").
 *
 * Layout (all dense, row-major, no padding, element offsets fit in 64 bits):
 *     q      [C][32][64]      dtype         (token-major, then head, then dim)
 *     kCache [P+C][8][64]     dtype
 *     vCache [P+C][8][64]     dtype
 *     out    [C][32][64]      float32 for every dtype
 *
 * Ownership: every pointer is device memory owned by the caller.  The library
 * allocates nothing and may be called from any host thread.  It keeps no state
 * between calls, except that attn_prefill_splitkv_noalloc uses one fixed
 * scratch array per device (see there).  Work is enqueued on `stream` and the
 * call returns without waiting; the caller synchronises.  `out` must not overlap the inputs; every
 * element of out[0..C) is overwritten.
 *
 * Every entry point only enqueues kernels on `stream`: it allocates,
 * synchronises and memsets nothing, so calls can be captured in a HIP graph
 * and replayed (with the same pointers and sizes).
 *
 * Errors: nothing is thrown across the ABI; each call returns an
 * attn_status_t and enqueues no work unless it returns ATTN_OK.
 */
#ifndef ATTN_PREFILL_H
#define ATTN_PREFILL_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed shape of the tensor contract ("Inference Attention 2", Lesson). */
#define ATTN_NUM_Q_HEADS 32
#define ATTN_NUM_KV_HEADS 8
#define ATTN_HEAD_DIM 64

/* Element type of q, kCache and vCache.  out is always float32.  Any other
 * value is rejected with ATTN_ERR_UNSUPPORTED_DTYPE; in C++ the enum takes int
 * as its underlying type, so that such a value is still a representable
 * attn_dtype_t when the library checks it. */
typedef enum
#ifdef __cplusplus
    : int
#endif
{
    ATTN_DTYPE_F32 = 0,  /* IEEE binary32; scores and PV products in fp32 MFMA */
    ATTN_DTYPE_BF16 = 1  /* bfloat16; bf16 MFMA with fp32 accumulation, fp32 softmax state */
} attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,      /* C < 0, C > 2^25, P < 0, or P + C > 2^30 */
    ATTN_ERR_NULL_PTR = 2,         /* a tensor pointer is NULL while C > 0 */
    ATTN_ERR_UNSUPPORTED_DTYPE = 3,/* dtype is not an attn_dtype_t value */
    ATTN_ERR_MISALIGNED = 4,       /* a tensor pointer is not 16-byte aligned */
    ATTN_ERR_LAUNCH = 5,           /* the HIP runtime rejected the launch */
    ATTN_ERR_ALIAS = 6,            /* out (or a workspace) overlaps another argument */
    ATTN_ERR_WORKSPACE = 7,        /* workspace smaller than attn_prefill_splitkv_workspace() */
    ATTN_ERR_TOO_LARGE = 8         /* the call needs more than ATTN_NOALLOC_SCRATCH_BYTES of scratch */
} attn_status_t;

/*
 * attn_prefill -- out = causal GQA attention of the chunk q against the cache.
 *
 *   q       device pointer, [C][32][64] of dtype, 16-byte aligned
 *   kCache  device pointer, [P+C][8][64] of dtype, 16-byte aligned
 *   vCache  device pointer, [P+C][8][64] of dtype, 16-byte aligned
 *   out     device pointer, [C][32][64] float32, 16-byte aligned, written
 *   C       chunk length (number of query rows), 0 <= C <= 2^25 (33,554,432);
 *           C == 0 is a no-op
 *   P       prefix length already in the cache, 0 <= P <= 2^30 - C (no GPU's memory
 *           holds a larger cache)
 *   dtype   element type of q, kCache, vCache
 *   stream  HIP stream to enqueue on (0 = the null stream)
 *
 * Returns ATTN_OK once the kernel is enqueued, or an error code (see
 * attn_status_t) with nothing enqueued.  Asynchronous: errors raised while
 * the kernel runs surface at the caller's next synchronisation.
 */
attn_status_t attn_prefill(const void* q, const void* kCache, const void* vCache, float* out,
                           int C, int P, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_prefill_clocked -- attn_prefill (the same kernels, launch plan and
 * result) that also logs the clock it runs at and where each workgroup's time
 * goes, for reporting throughput against the peak at that clock as well as
 * the nominal one: thread 0 of every workgroup stores counters at fixed marks.
 *
 *   clocks      device memory of at least clockCount unsigned 64-bit values,
 *               8-byte aligned, not overlapping any tensor; workgroup w writes
 *               the ATTN_CLOCK_WORDS values from clocks[ATTN_CLOCK_WORDS * w]:
 *                 [0] shader clock at start      [1] 100 MHz counter at start
 *                 [2] shader clock at end        [3] 100 MHz counter at end
 *                 [4] shader clock when its first work item's first K/V tile
 *                     is in LDS (the item's Q and tile loads have landed)
 *                 [5] shader clock when that item's key loop is done
 *                 [6] shader clock when that item's output is stored
 *                 [7] shader clock when the second work item's first tile
 *                     is in LDS; not written when there is no second item
 *   clockCount  at least ATTN_CLOCK_WORDS x the workgroups of the launch
 *               (plan[2] of attn_prefill_plan for the same C, P, dtype with
 *               paged = 0)
 *   other arguments as for attn_prefill
 *
 * The clock of workgroup w over its life is ([2] - [0]) / ([3] - [1]) *
 * 100 MHz; a phase in seconds is its shader-clock difference over that clock.
 * Returns as attn_prefill, plus ATTN_ERR_NULL_PTR / ATTN_ERR_MISALIGNED /
 * ATTN_ERR_ALIAS for clocks and ATTN_ERR_WORKSPACE when clockCount is too
 * small.
 */
#define ATTN_CLOCK_WORDS 8
attn_status_t attn_prefill_clocked(const void* q, const void* kCache, const void* vCache, float* out,
                                   int C, int P, attn_dtype_t dtype, unsigned long long* clocks,
                                   size_t clockCount, hipStream_t stream);

/* Static, NUL-terminated name of a status code ("ATTN_OK", ...). */
const char* attn_status_string(attn_status_t status);

/*
 * attn_prefill_validate -- the argument checks of attn_prefill alone, with no
 * HIP call and no launch.  Same arguments and return codes; ATTN_OK means
 * attn_prefill would try to launch.  Host-only; safe without a GPU.
 */
attn_status_t attn_prefill_validate(const void* q, const void* kCache, const void* vCache,
                                    const float* out, int C, int P, attn_dtype_t dtype);

/*
 * attn_prefill_paged -- the same operation with the key/value cache held in
 * fixed-size pages ("FlashAttention and inference kernels", section
 * PagedAttention: cache position t lives at slot t % pageSize of physical page
 * blockTable[t / pageSize]).
 *
 *   kPages, vPages  device pointers, [numBlocks][pageSize][8][64] of dtype,
 *                   16-byte aligned; numBlocks*pageSize*8*64*sizeof(dtype)
 *                   must not exceed 2^32-1 bytes
 *   blockTable      device pointer, int32, at least ceil((P+C)/pageSize)
 *                   entries, 4-byte aligned; entries are physical page indices
 *   numBlocks       pages in the pool, > 0
 *   pageSize        positions per page, > 0
 *   q, out, C, P, dtype, stream as for attn_prefill
 *
 * A table entry outside [0, numBlocks) does not fault: the positions it maps
 * read as zeros (the result is then not the attention of any cache).  Returns
 * as attn_prefill; ATTN_ERR_INVALID_ARG also for pageSize <= 0, numBlocks <= 0,
 * or a pool or table too large for 32-bit byte offsets (a pool above 4 GiB, or
 * 2^30 or more table entries); ATTN_ERR_ALIAS if out overlaps q, the pools or
 * the table.
 */
attn_status_t attn_prefill_paged(const void* q, const void* kPages, const void* vPages, const int* blockTable,
                                 int numBlocks, int pageSize, float* out, int C, int P, attn_dtype_t dtype,
                                 hipStream_t stream);

/*
 * attn_prefill_rowwise -- the same result as attn_prefill with no tiling
 * ("Inference Attention 2", Lesson: the starter serves each (row, head) on its
 * own and every row streams its whole K/V prefix from memory).  One 64-lane
 * wave per (row, head), keys in blocks of 64: scores with one lane per key,
 * the weighted sum of V with one lane per dim, one online softmax update per
 * block.  A baseline to time the tiled kernel against (the page's SPEEDUP),
 * not a fast path.  Same arguments, layout, ownership and return codes as
 * attn_prefill.
 */
attn_status_t attn_prefill_rowwise(const void* q, const void* kCache, const void* vCache, float* out,
                                   int C, int P, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_prefill_splitkv -- the same result as attn_prefill, with the key range
 * of each row tile split across workgroups ("FlashAttention and inference
 * kernels", Flash-Decoding / split-K): every split writes an unnormalised
 * partial (O_s, m_s, l_s) per (row, head) to `workspace`, and a second kernel
 * merges them with weights e^(m_s - m) over the splits each row reaches.  For
 * short chunks (decode, C = 1..64) against long prefixes, where row tiles x KV
 * groups alone cannot fill the GPU.  A single fp32 token (C = 1) is split by
 * a kernel built on plain FMAs (no MFMA tile to fill); everything else uses
 * the tiled MFMA kernel with a key range per workgroup.
 *
 *   workspace       device memory of at least attn_prefill_splitkv_workspace()
 *                   bytes, 16-byte aligned, not overlapping any argument;
 *                   owned by the caller; its contents on entry do not matter
 *                   and are garbage on return.  Calls that share a workspace
 *                   must be ordered on one stream.
 *   workspaceBytes  its size in bytes
 *   other arguments as for attn_prefill
 *
 * Returns as attn_prefill; ATTN_ERR_WORKSPACE if workspaceBytes is too small,
 * ATTN_ERR_NULL_PTR / ATTN_ERR_MISALIGNED / ATTN_ERR_ALIAS for the workspace.
 */
attn_status_t attn_prefill_splitkv(const void* q, const void* kCache, const void* vCache, float* out,
                                   int C, int P, attn_dtype_t dtype, void* workspace, size_t workspaceBytes,
                                   hipStream_t stream);

/* Size of the per-device scratch array behind attn_prefill_splitkv_noalloc. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * attn_prefill_splitkv_noalloc -- attn_prefill_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and result, with the
 * key-split partials in a fixed scratch array of ATTN_NOALLOC_SCRATCH_BYTES
 * that the library holds on each device it runs on until the process ends,
 * instead of a caller workspace.  The call allocates nothing and calls no
 * allocating routine.
 *
 *   q, kCache, vCache, out, C, P, dtype, stream as for attn_prefill; the
 *   current device must be the device of the tensors and of `stream`.
 *
 * All calls on one device share that device's array and leave it holding the
 * last call's partials; nothing in it needs to start at any value.  Calls
 * whose kernels can overlap on one device race on the array: order them on
 * one stream (or otherwise serialise them).  The first call on a device looks
 * up the array's device address (hipGetSymbolAddress) once.
 *
 * Returns as attn_prefill_splitkv; ATTN_ERR_TOO_LARGE, with nothing enqueued,
 * when attn_prefill_splitkv_workspace() for (C, P, dtype) exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES (for example C above about 1980 rows); use
 * attn_prefill or attn_prefill_splitkv there.  ATTN_ERR_LAUNCH also when the
 * array's address cannot be obtained, and ATTN_ERR_INVALID_ARG (nothing
 * enqueued) when `stream` belongs to another device than the current one.
 */
attn_status_t attn_prefill_splitkv_noalloc(const void* q, const void* kCache, const void* vCache, float* out,
                                           int C, int P, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_prefill_splitkv_workspace -- bytes of workspace attn_prefill_splitkv
 * needs for (C, P, dtype), and (if splits != NULL) how many key splits it
 * uses.  Host-only, no HIP call.  C == 0 needs 0 bytes.
 */
attn_status_t attn_prefill_splitkv_workspace(int C, int P, attn_dtype_t dtype, size_t* bytes, int* splits);

/*
 * attn_prefill_paged_splitkv -- attn_prefill_splitkv over a paged cache: the
 * key range of each row tile split across workgroups, the partials merged
 * ("FlashAttention and inference kernels", sections "Parallelism during
 * decode: Flash-Decoding and split-K" and "A paged decode attention kernel
 * (with GQA)"), with every K/V row found through the block table as in
 * attn_prefill_paged (section PagedAttention).  The decode shape against a
 * paged cache: one token (or a short chunk) over a long prefix, where row
 * tiles x KV groups alone would leave most of the GPU idle.  One fp32 token
 * runs on the FMA kernel, everything else on the tiled MFMA kernel.
 *
 *   q, kPages, vPages, blockTable, numBlocks, pageSize, out, C, P, dtype as
 *   for attn_prefill_paged; workspace and workspaceBytes as for
 *   attn_prefill_splitkv, sized by attn_prefill_splitkv_workspace(C, P, dtype)
 *   (the same plan); stream as for attn_prefill.
 *
 * A table entry outside [0, numBlocks) reads as zeros, as in
 * attn_prefill_paged.  Returns as attn_prefill_paged, and as
 * attn_prefill_splitkv for the workspace (ATTN_ERR_ALIAS also when it overlaps
 * the pools or the table).
 */
attn_status_t attn_prefill_paged_splitkv(const void* q, const void* kPages, const void* vPages,
                                         const int* blockTable, int numBlocks, int pageSize, float* out, int C, int P,
                                         attn_dtype_t dtype, void* workspace, size_t workspaceBytes,
                                         hipStream_t stream);

/*
 * attn_naive -- causal prompt prefill (P = 0) by the three-kernel pipeline of
 * "Inference Attention 1: The Full Score Matrix" (Lesson): a scores kernel
 * writes the 32 x T x T fp32 score matrix (-inf above the diagonal) into
 * `workspace`, a softmax kernel normalises each row in place, a weighted-sum
 * kernel multiplies it by V.  A baseline that shows the memory cost the fused
 * path removes; fp32 only.
 *
 *   q [T][32][64], k and v [T][8][64], out [T][32][64]: fp32 device memory as
 *   for attn_prefill with C = T, P = 0
 *   workspace       at least attn_naive_workspace(T) bytes (32*T*T floats),
 *                   16-byte aligned, not overlapping any argument
 *   T               prompt length, 0 <= T <= 46340
 *
 * Returns as attn_prefill; ATTN_ERR_WORKSPACE if the workspace is too small.
 */
attn_status_t attn_naive(const float* q, const float* k, const float* v, float* out, int T, void* workspace,
                         size_t workspaceBytes, hipStream_t stream);

/* Bytes of workspace attn_naive needs for T (32*T*T*4). Host-only. */
attn_status_t attn_naive_workspace(int T, size_t* bytes);

/* The argument checks of attn_prefill_paged alone; host-only, no HIP call. */
attn_status_t attn_prefill_paged_validate(const void* q, const void* kPages, const void* vPages,
                                          const int* blockTable, int numBlocks, int pageSize, const float* out,
                                          int C, int P, attn_dtype_t dtype);

/*
 * attn_prefill_plan -- the launch decomposition attn_prefill (paged == 0) or
 * attn_prefill_paged (paged != 0) would use for (C, P, dtype), written to the
 * caller's int array plan[8]:
 *   plan[0] rows per work item (query rows of one KV group per item)
 *   plan[1] waves splitting the key range inside a workgroup
 *   plan[2] workgroups in the grid
 *   plan[3] threads per workgroup
 *   plan[4] work items per workgroup (1, or 2 when rows are paired)
 *   plan[5] keys per staged K/V tile
 *   plan[6] LDS bytes per workgroup
 *   plan[7] kernel variant id
 * Host-only, no HIP call.  Returns ATTN_OK or ATTN_ERR_INVALID_ARG /
 * ATTN_ERR_UNSUPPORTED_DTYPE / ATTN_ERR_NULL_PTR (plan == NULL).
 */
attn_status_t attn_prefill_plan(int C, int P, attn_dtype_t dtype, int paged, int* plan);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int attn_prefill_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PREFILL_H */
