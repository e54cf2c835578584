// attn_prefill.hip -- causal grouped-query flash-attention prefill of a query
// chunk against a cached prefix, for AMD Instinct MI355X (gfx950, CDNA4).
//
// What is computed ("Inference Attention 2: Flash Prefill Against a Cached
// Prefix", Lesson): chunk row i (absolute position P+i) attends to cache
// positions j <= P+i; 32 query heads, 8 KV heads, head size 64, query head h
// reads KV head h/4, scale exactly 1/8.  Query rows are tiled and held in
// registers, each K/V tile is staged in LDS once and consumed by every resident
// row, and the online softmax (running max m, running denominator l,
// accumulator rescaled by exp(m_old - m_new), one division by l at the end) is
// carried across tiles (same page, the four update equations).  Tiles wholly
// past the causal edge are never visited and only tiles that straddle it are
// masked elementwise ("FlashAttention and inference kernels", the paragraph on
// the causal mask).  One workgroup serves all four query heads of a KV group so
// each K/V tile is read once for them (same handbook, Exercises, exercise 3).
//
// Mapping onto CDNA4
// ------------------
// * A wave owns 32 queries: 8 consecutive chunk rows x the 4 query heads of
//   one KV group.  Query slot n = lane % 32 is (row 8w + n/4, head 4g + n%4).
// * Scores are computed transposed, S^T[key][query] = K . Q^T, with the
//   32x32 MFMA (fp32: v_mfma_f32_32x32x2_f32; bf16: v_mfma_f32_32x32x16_bf16).
//   Its accumulator layout puts query n in lanes n and n+32 and 16 of the 32
//   keys of a sub-block in each lane's registers (key 8(r/4) + 4(lane/32) +
//   r%4 in register r).  The softmax state of a query therefore lives in two
//   lanes, row maxima are in-register reductions plus one exchange between
//   the two half-waves, and the rescale factor is per lane.
// * The output is accumulated transposed too, O^T[dim][query] = V^T . P^T,
//   so the probabilities feed the B operand straight from the score
//   registers (the key order inside a sub-block is free because PV sums over
//   keys; V is read in the matching order).
// * K/V tiles go from HBM straight into LDS (bounds-checked buffer loads with
//   an LDS destination), rows unpadded with their 16-byte chunks XOR-permuted
//   per row so the MFMA operand reads avoid bank conflicts; the next tile's
//   loads are in flight while the current tile is consumed (two stages), or,
//   in the one-stage plans for short and mid-size chunks, two workgroups share
//   a CU and one computes while the other's loads land.  fp32 Q rows take the
//   same path into LDS, once per work item for all its waves.
// * A workgroup is NW row-waves x KS key-split waves.  Key-split waves take
//   alternate 32-key sub-blocks of each tile and are merged once at the end
//   with the log-sum-exp rule ("FlashAttention and inference kernels",
//   Flash-Decoding section and Exercises, exercise 2), skipping empty splits.
// * blockIdx.x % 8 selects the KV group: consecutive workgroups go to the 8
//   XCDs round-robin, so every XCD's L2 holds the K/V of one group only.
// * Row tiles i and n-1-i can be paired in one workgroup so every workgroup
//   does the same causal work.
// * exp is evaluated as exp2 with log2(e)/8 folded in (into Q for fp32, into an
//   FMA for bf16).  The running maximum is only moved when a sub-block's
//   maximum exceeds it by more than 8 in log2 units; any reference value
//   gives the same softmax because it cancels in O/l, and p stays <= 2^8.
//   The weights are formed against the current maximum first: a lane's sum
//   bounds each of its weights, so one compare of that sum with 2^8 replaces
//   the block maximum, which is only formed (and the weights redone) in a wave
//   where some sum passes it.  The maximum starts at -1e30, finite and below
//   any score, so a masked (-inf) score gives a zero weight with no special
//   case.
//
// Other kernels in this file: the same kernel in paged-cache and key-split
// modes, an FMA kernel for one fp32 decode token, the merge of key-split
// partials, and two baselines timed against the fused kernel (the per-row
// starter algorithm and the three-kernel pipeline with the full score matrix).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

#include <mutex>
#include <type_traits>

#include "attn_prefill.h"

// Fixed device scratch for attn_prefill_splitkv_noalloc (callers that cannot
// allocate): the key-split partials live here instead of in a caller
// workspace.  Each device the library runs on holds its own copy for the life
// of the process.  Host code never passes this name to a kernel (on the host
// it is only a stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kHQ = ATTN_NUM_Q_HEADS;   // 32
constexpr int kHKV = ATTN_NUM_KV_HEADS; // 8
constexpr int kD = ATTN_HEAD_DIM;       // 64
constexpr int kGroup = kHQ / kHKV;      // 4
constexpr int kClockWords = ATTN_CLOCK_WORDS;   // clock-log words per workgroup

// log2(e) / 8: scores become base-2 exponents with the 1/8 scale applied.
constexpr float kScaleLog2 = 0.18033688011112042f;
// Move the running maximum only when a tile raises it by more than this many
// powers of two.
constexpr float kRescaleSlack = 8.0f;
constexpr float kSlackWeight = 256.0f;                // 2^kRescaleSlack
constexpr float kInvScaleLog2 = 5.545177444479562f;   // 8 / log2(e)

typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
};
template <> struct Elem<__bf16> {
    static constexpr int kBytes = 2;
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Tile geometry for a workgroup of NW row-waves x KS key-split waves with ST
// staging buffers (2: the next tile loads while the current one is consumed;
// 1: half the LDS, so two workgroups share a CU and overlap each other).
//
// LDS holds each staged K and V tile as unpadded key-major rows (256 B fp32,
// 128 B bf16), in ST stages, laid out V0 V1 K0 K1: every V operand then sits
// below 64 KiB and every K operand below 64 KiB of a per-lane base, so each
// LDS read is one base register plus an immediate offset (the DS offset field
// is 16 bits).  Inside a row the 16-byte chunks are permuted by XOR with a
// per-row code, one for K rows and one for V rows, so that the operand reads
// spread over all LDS banks: a 16-byte K read serves 16 lanes (16 keys, the
// same logical chunk) per LDS cycle, whose 16-byte slots must then all differ
// modulo 256 bytes; the V reads (fp32: 8 bytes per lane; bf16: transposed
// 4-key x 16-dim blocks) have their own pattern.  Unpadded rows let each
// direct global->LDS load instruction fill 1 KiB of whole rows.
template <typename T, int NW, int KS, int ST = 2>
struct Geo {
    static constexpr int kNB = KS > 2 ? KS : 2;      // 32-key sub-blocks per staged tile
    static constexpr int kBK = 32 * kNB;             // keys per staged tile
    static constexpr int kThreads = 64 * NW * KS;
    static constexpr int kWaves = NW * KS;
    static constexpr int kRows = 8 * NW;             // chunk rows per work item
    static constexpr int kRowBytes = kD * Elem<T>::kBytes;
    static constexpr int kTileBytes = kBK * kRowBytes;                // one tensor, one stage
    static constexpr int kStageBytes = 2 * kTileBytes;                // K and V of one stage
    static constexpr int kKBase = ST * kTileBytes;                    // K0 follows the V stages
    static constexpr int kKSpan = ST * kTileBytes;                    // the K stages
    static_assert(2 * kTileBytes <= 65536 && kKSpan <= 65536, "LDS operand offsets must fit 16 bits");
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;             // rows per 64-lane 16 B load
    static constexpr int kLoadsPerTile = 2 * kBK / kRowsPerLoad;      // K and V
    static constexpr int kLoadsPerWave = (kLoadsPerTile + kWaves - 1) / kWaves;
    // Merge buffer for key splits: per (row-wave, split>0) wave, 34 floats/lane.
    static constexpr int kMergeBytes = KS > 1 ? NW * (KS - 1) * 34 * 64 * 4 : 0;
    static constexpr int kLdsBytes = ST * kStageBytes > kMergeBytes ? ST * kStageBytes : kMergeBytes;
    // Paged cache: the row offsets of two tiles follow the tiles.  fp32: a work
    // item's Q rows (the group's 4 heads, 1 KiB per row) are staged in LDS,
    // after the tiles where they fit in the 160 KiB of a workgroup (half that
    // when two one-stage workgroups share a CU), else in the second stage's V
    // tile, which is free until the item's second tile is issued.
    static constexpr int kQRowBytes = kGroup * kD * 4;
    static constexpr int kQBytes = kRows * kQRowBytes;
    static constexpr int kLdsLimit = ST == 2 ? 163840 : 81920;
    static constexpr int q_offset(bool paged) { return kLdsBytes + (paged ? 2 * kBK * 4 : 0); }
    static constexpr bool q_after(bool paged) { return sizeof(T) == 4 && q_offset(paged) + kQBytes <= kLdsLimit; }
    static constexpr bool q_in_stage1(bool paged) {
        return sizeof(T) == 4 && !q_after(paged) && ST == 2 && kQBytes <= kTileBytes;
    }
    static constexpr int lds_total(bool paged) { return q_offset(paged) + (q_after(paged) ? kQBytes : 0); }
};

// Row-dependent chunk permutations (XOR codes) of staged rows.  A 16-byte
// K operand read serves 16 lanes (16 keys at the same logical chunk) per LDS
// cycle of 256 bytes, so their 16-byte slots must all differ modulo 256
// bytes.  fp32: a row is one such cycle of 16 chunks, so each row of a
// 16-key group gets its own code.  bf16: two 128-byte rows share a cycle, in
// its two halves, so each row pair gets its own code.  Both depend on the row
// modulo 16, and every stage, tile and sub-block offset is a multiple of 16
// rows.
template <typename T>
__device__ __forceinline__ int k_code(int r) {
    if constexpr (sizeof(T) == 4) {
        return r & 15;
    } else {
        return (r >> 1) & 7;
    }
}

// V rows: the code of the operand reads' row within an 8-row block.
template <typename T>
__device__ __forceinline__ int chunk_code(int r) {
    if constexpr (sizeof(T) == 4) {
        return r & 7;                                   // 16 chunks per row; low 3 bits permuted
    } else {
        return ((r & 3) << 1) | ((r >> 2) & 1);         // 8 chunks per row
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes n and n+32 of a wave hold different keys of the same query.  One
// v_permlane32_swap with x in both operands (it exchanges the upper half of
// the first with the lower half of the second) leaves, in every lane, the
// lower half's x of that query in one result and the upper half's in the
// other, so both lanes combine the same two values and agree bitwise.
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// n / d for 0 <= n < 2^32 and a divisor d >= 1 fixed for the launch, as one
// high multiply, a subtract, an add and two shifts (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994, section 4:
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// q = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0) with t = mulhi(m, n)).
struct FastDiv {
    uint32_t m;
    int s1, s2;
};

FastDiv make_fastdiv(uint32_t d) {
    int l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l < 1 ? l : 1, l > 1 ? l - 1 : 0};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
    const uint32_t t = __umulhi(f.m, n);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

// Paged cache description ("FlashAttention and inference kernels", section
// PagedAttention): position t lives at slot t % page_size of physical page
// table[t / page_size]; kc/vc then point at [num_blocks][page_size][8][64].
// `div` divides by page_size; `shift` is log2(page_size) when that is a
// power of two (then a shift and a mask replace the division), else -1.
struct PagedCache {
    const int* table;
    int page_size;
    int num_blocks;
    FastDiv div;
    int shift;
};

PagedCache make_paged(const int* table, int page_size, int num_blocks) {
    int shift = -1;
    if ((page_size & (page_size - 1)) == 0) {
        shift = 0;
        while ((1 << shift) < page_size) ++shift;
    }
    return PagedCache{table, page_size, num_blocks, make_fastdiv((uint32_t)page_size), shift};
}

// Page index, in-page slot and first position of a page's slot (page * page_size + slot).
__device__ __forceinline__ uint32_t page_index(uint32_t key, const PagedCache& pg) {
    return pg.shift >= 0 ? key >> pg.shift : fast_div(key, pg.div);
}
__device__ __forceinline__ uint32_t page_slot(uint32_t key, uint32_t blk, const PagedCache& pg) {
    return pg.shift >= 0 ? key & (uint32_t)(pg.page_size - 1) : key - blk * (uint32_t)pg.page_size;
}
__device__ __forceinline__ uint32_t pool_position(uint32_t page, uint32_t slot, const PagedCache& pg) {
    return pg.shift >= 0 ? (page << pg.shift) | slot : page * (uint32_t)pg.page_size + slot;
}

// Key-range split across workgroups (Flash-Decoding, "FlashAttention and
// inference kernels"): workgroup split s covers keys [s*len, (s+1)*len) of
// its row tile and writes unnormalised partials (O, m, l) to `part`, which a
// merge kernel combines.  n == 0: no split, the kernel writes `out` itself.
struct KeySplit {
    float* part;    // [n][C][32][64] O, then [n][C][32][2] (m in log2 units, l)
    int len;        // keys per split, a multiple of the staged tile
    int n;          // number of splits
};

// Kernel modes, as bits: a paged cache, a key-range split, or both.
enum Mode { kPlain = 0, kPaged = 1, kSplit = 2, kPagedSplit = 3 };

// ---------------------------------------------------------------------------
// The kernel.  One workgroup = one KV group g and one or two row tiles.
// ---------------------------------------------------------------------------

// One staging buffer: two workgroups per CU, so at least 2 * NW * KS / 4 waves
// per SIMD (the second bound is waves per execution unit).
template <typename T, int NW, int KS, int MODE, int ST = 2>
__global__ void __launch_bounds__(64 * NW * KS, ST == 1 ? NW * KS / 2 : 1)
attn_prefill_kernel(const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
                    float* __restrict__ out, int C, int P, int n_row_tiles, int paired, PagedCache pg,
                    KeySplit ks, unsigned long long* __restrict__ clk) {
    static_assert(ST == 2 || (ST == 1 && (MODE & kSplit) == 0), "one staging buffer: no key splits");
    // Clock log (attn_prefill_clocked; null otherwise): thread 0 stores, with
    // ordinary vector stores, the shader-clock counter and the fixed 100 MHz
    // counter at the workgroup's start and end, and the shader clock at the
    // phase marks of its first two work items, so that the clock the kernel
    // runs at and where its time goes can be read from the kernel itself.
    // Only the plain kernels are ever launched with a log.
    constexpr bool kLog = MODE == kPlain;
    auto mark = [&](int slot) {
        if (kLog && clk != nullptr && threadIdx.x == 0)
            clk[kClockWords * blockIdx.x + slot] = __builtin_amdgcn_s_memtime();
    };
    if (kLog && clk != nullptr && threadIdx.x == 0) {
        clk[kClockWords * blockIdx.x] = __builtin_amdgcn_s_memtime();
        clk[kClockWords * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
    }
    using G = Geo<T, NW, KS, ST>;
    constexpr int kBK = G::kBK, kNB = G::kNB, kRows = G::kRows, kRB = G::kRowBytes;
    constexpr bool kF32 = sizeof(T) == 4;
    constexpr bool PAGED = (MODE & kPaged) != 0;
    constexpr bool SPLIT = (MODE & kSplit) != 0;

    // One LDS object: K/V stages (reused by the key-split merge), then, for a
    // paged cache, the row offsets of two tiles, then (fp32, where it fits)
    // the Q rows of one work item.  A second __shared__ array would make the
    // compiler wait for every HBM->LDS load in flight before each LDS read of
    // the staged tiles.
    constexpr int kQRowBytes = G::kQRowBytes;
    constexpr bool kQAfter = G::q_after(PAGED);          // Q rows after the tiles (and row offsets)
    constexpr bool kQInStage1 = G::q_in_stage1(PAGED);   // else in the second stage's V tile
    constexpr bool kQLds = kQAfter || kQInStage1;
    __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[G::lds_total(PAGED)];
    unsigned char* const qbuf = lds_raw + (kQInStage1 ? G::kTileBytes : G::q_offset(PAGED));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps load descriptors scalar
    const int wr = wid % NW;   // row sub-tile of this wave
    const int wp = wid / NW;   // key split of this wave
    if constexpr (sizeof(T) == 2) {
        // bf16 is bound by the softmax arithmetic: waves of even key split win
        // issue ties, so the two waves sharing a SIMD drift out of phase and
        // one's exponentials overlap the other's MFMAs
        if ((wp & 1) == 0) __builtin_amdgcn_s_setprio(1);
    }
    const int n = lane & 31;   // query slot
    const int hh = lane >> 5;  // half-wave
    const int g = blockIdx.x % kHKV;
    const int split = SPLIT ? (blockIdx.x / kHKV) % ks.n : 0;
    const int slot = SPLIT ? blockIdx.x / kHKV / ks.n : blockIdx.x / kHKV;
    int kb = 0;                // first key of this work item's key range
    const int total = P + C;   // cache positions

    int items[2];
    int nitems = 1;
    if (paired == 1) {
        items[0] = n_row_tiles - 1 - slot;  // the heavier tile first
        items[1] = slot;
        nitems = items[1] != items[0] ? 2 : 1;
    } else if (paired == 2) {
        // one item per workgroup, all resident at once two per CU: the first
        // half of the slots takes the heavy tiles in descending order and the
        // second half the light ones ascending, so a CU's two workgroups (slots
        // s and s + half) carry tiles n-1-s and s
        const int half = (n_row_tiles + 1) / 2;
        items[0] = slot < half ? n_row_tiles - 1 - slot : slot - half;
        items[1] = items[0];
    } else {
        items[0] = n_row_tiles - 1 - slot;  // heaviest tiles are launched first
        items[1] = items[0];
    }

    // ---- K/V tile staging: bounds-checked buffer loads straight into LDS ----
    // Load instruction i of a tile covers rows (i % (BK/rpl))*rpl .. +rpl-1 of
    // K (i < BK/rpl) or V; lane L fetches the chunk that belongs at position
    // L % cpr of row L / cpr.  Contiguous cache: the descriptor's range is the
    // tile's valid rows, so rows past the cache end read as zero.  Paged cache:
    // the descriptor spans the page pool and a row past the cache end, or one
    // whose page index is out of range, is given an offset past the range and
    // reads as zero.
    constexpr int kCPR = kRB / 16;                  // 16-byte chunks per row
    constexpr int kRPL = G::kRowsPerLoad;
    constexpr int kLPW = G::kLoadsPerWave;
    const int rl = lane / kCPR;                     // row within one load
    const int pc = lane % kCPR;                     // chunk position within the row
    auto load_row = [&](int u) { return ((wid + u * G::kWaves) % (kBK / kRPL)) * kRPL + rl; };
    // Paged cache: the byte offset of every K/V row of tile t sits in LDS slot
    // t & 1, written two tiles ahead by the first kBK threads, so a lane that
    // issues a row's loads holds no page state.  Those threads load the table
    // entry of their row of tile t+2 into a register while tile t is consumed
    // and store the row's byte offset after the tile's vmcnt(0).
    uint32_t* const pofs = reinterpret_cast<uint32_t*>(lds_raw + G::kLdsBytes);   // [2][kBK]
    constexpr uint32_t kNoRow = 0xffffffffu;        // past the cache, or a bad table entry
    // The table is read through a buffer descriptor (scalar base, 32-bit lane
    // offset), and row offsets are formed in 32 bits: the host rejects pools
    // and tables whose byte sizes do not fit them.
    const __amdgpu_buffer_rsrc_t rtab = __builtin_amdgcn_make_buffer_rsrc(
        (void*)pg.table, (short)0, PAGED ? (uint32_t)((total + pg.page_size - 1) / pg.page_size) * 4u : 0u,
        0x00020000);
    // The thread index is made opaque in both helpers so that nothing derived
    // from it is hoisted out of the key loop and held in registers throughout.
    auto fetch_entry = [&](int t) {                 // table entry of row tid of tile t (first kBK threads)
        int ent = 0;
        if (tid < kBK) {                            // whole waves (kBK is a multiple of 64)
            int r = tid;
            asm volatile("" : "+v"(r));
            const int key = kb + t * kBK + r;       // past the table: the load reads zero
            ent = (int)__builtin_amdgcn_raw_buffer_load_b32(rtab, page_index((uint32_t)key, pg) * 4u, 0, 0);
        }
        return ent;
    };
    auto store_offset = [&](int t, int ent) {       // after the vmcnt(0) that covers fetch_entry(t)
        if (tid < kBK) {
            int r = tid;
            asm volatile("" : "+v"(r));
            const int key = kb + t * kBK + r;
            const uint32_t in_page = page_slot((uint32_t)key, page_index((uint32_t)key, pg), pg);
            pofs[(t & 1) * kBK + r] =
                key < total && (uint32_t)ent < (uint32_t)pg.num_blocks
                    ? pool_position((uint32_t)ent, in_page, pg) * (uint32_t)(kHKV * kRB) + (uint32_t)(g * kRB)
                    : kNoRow;
        }
    };
    // fp32 Q through LDS: the rows of work item i0q go from memory straight
    // into LDS (one 1 KiB row per load instruction: the group's 4 heads), once
    // for the workgroup instead of once per key-split wave, and each wave reads
    // its 8 rows from there.  Position p of a row holds logical chunk
    // p ^ ((4 * (row % 4) + head) % 16) (the head being p / 16, which the XOR
    // keeps), so the 16 lanes of an LDS cycle (4 rows x 4 heads at one chunk)
    // read 16 different bank groups.
    auto issue_q = [&](int i0q) {
        const int rows_q = min(kRows, C - i0q);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + (size_t)i0q * kHQ * kD), (short)0, (uint32_t)rows_q * kHQ * kD * 4, 0x00020000);
        int L = lane;
        asm volatile("" : "+v"(L));
#pragma unroll
        for (int u = 0; u < (kRows + G::kWaves - 1) / G::kWaves; ++u) {
            const int r = wid + u * G::kWaves;      // item row of this instruction; past the chunk it reads zero
            if (kRows % G::kWaves != 0 && r >= kRows) break;
            const int lc = L ^ ((4 * (r & 3) + (L >> 4)) & 15);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t*)(qbuf + r * kQRowBytes), 16,
                                                     (uint32_t)((r * kHQ + g * kGroup) * kD * 4 + lc * 16), 0, 0, 0);
        }
    };
    bool q_staged = false;     // qbuf already holds the next work item's Q

    auto issue_tile = [&](int t, int stage) {
        const int key0 = kb + t * kBK;
        uint32_t range;
        size_t base;
        if constexpr (PAGED) {
            range = (uint32_t)((size_t)pg.num_blocks * pg.page_size * kHKV * kRB);
            base = 0;
        } else {
            range = (uint32_t)min(kBK, total - key0) * kHKV * kRB;   // bytes of this tile's rows, all groups
            base = (size_t)key0 * kHKV * kD;
        }
        __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + base), (short)0, range, 0x00020000);
        __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + base), (short)0, range, 0x00020000);
#pragma unroll
        for (int u = 0; u < kLPW; ++u) {
            const int i = wid + u * G::kWaves;
            if (G::kLoadsPerTile % G::kWaves != 0 && i >= G::kLoadsPerTile) break;
            const int tensor = i / (kBK / kRPL);
            const int row = load_row(u);
            const int lc = pc ^ (tensor ? chunk_code<T>(row) : k_code<T>(row));   // logical chunk at position pc
            uint32_t voff;
            if constexpr (PAGED) {
                const uint32_t ro = pofs[(t & 1) * kBK + row];
                voff = ro == kNoRow ? range : ro + lc * 16;   // ro + lc*16 < range for a valid row
            } else {
                voff = (uint32_t)(row * kHKV + g) * kRB + lc * 16;
            }
            unsigned char* dst = lds_raw + (tensor ? 0 : G::kKBase) + stage * G::kTileBytes + (row - rl) * kRB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(tensor ? rv : rk, (lds_void_t*)dst, 16, voff, 0, 0, 0);
        }
    };

    for (int it = 0; it < nitems; ++it) {
        const int tile = items[it];
        const int i0 = tile * kRows;
        const int i0w = i0 + 8 * wr;
        const int rows_end = min(i0 + kRows, C);
        if constexpr (SPLIT) kb = split * ks.len;
        if constexpr (PAGED) {
            // An opaque copy per work item: the page lookups of its first tiles
            // are then recomputed here instead of being hoisted out of the item
            // loop and kept live (spilled) across the whole kernel.
            asm volatile("" : "+s"(kb));
        }
        const int kv_end = SPLIT ? min(P + rows_end, kb + ks.len) : P + rows_end;
        const int ntiles = kv_end > kb ? (kv_end - kb + kBK - 1) / kBK : 0;
        if (ntiles == 0) continue;                  // this split lies past every row of the item
        const bool wave_active = i0w < C;
        const int w_first = P + i0w;                // visible limit of the wave's first row
        const int w_last = P + min(i0w + 7, C - 1); // visible limit of its last valid row
        // from an opaque lane copy, so that nothing lane-derived is held
        // across the item loop
        int lane0 = lane;
        asm volatile("" : "+v"(lane0));
        const int row = i0w + ((lane0 & 31) >> 2);
        const int head = g * kGroup + (lane0 & 3);
        const int lim = P + row;                    // this lane's query sees keys <= lim

        if constexpr (PAGED) {
            const int e0 = fetch_entry(0);
            const int e1 = ntiles > 1 ? fetch_entry(1) : 0;
            store_offset(0, e0);
            if (ntiles > 1) store_offset(1, e1);
            __syncthreads();
        }
        if constexpr (kQLds) {
            if (!q_staged) issue_q(i0);
            q_staged = false;
        }
        issue_tile(0, 0);

        // ---- Q operand (B of S^T = K Q^T), held for the whole key loop ----
        // fp32: qf[s] = q[row][head][32*hh + s] * log2(e)/8, s = 0..31
        // bf16: qb[s] = q[row][head][16*s + 8*hh .. +7], s = 0..3
        // Loaded through a buffer descriptor over this work item's rows (a
        // scalar base and a 32-bit lane offset instead of a 64-bit address per
        // lane); rows past the chunk read as zero.  The output is stored the
        // same way.
        const int item_rows = min(kRows, C - i0);
        // element offset of this lane's (row, head) in the item, formed from an
        // opaque lane copy so it is recomputed per item rather than held
        int lane1 = lane;
        asm volatile("" : "+v"(lane1));
        const uint32_t lane_vec =
            (uint32_t)((8 * wr + ((lane1 & 31) >> 2)) * kHQ + g * kGroup + (lane1 & 3)) * kD;
        float qf[kF32 ? 32 : 1];
        bf8 qb[kF32 ? 1 : 4];
        {
            const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(q + (size_t)i0 * kHQ * kD), (short)0, (uint32_t)item_rows * kHQ * kD * sizeof(T), 0x00020000);
            if constexpr (kQLds) {
                (void)rq;                           // read from LDS once the item's first tile is in
            } else if constexpr (kF32) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const f4 x = __builtin_bit_cast(
                        f4, __builtin_amdgcn_raw_buffer_load_b128(rq, (lane_vec + 32 * hh + 4 * c) * 4, 0, 0));
#pragma unroll
                    for (int e = 0; e < 4; ++e) qf[4 * c + e] = x[e] * kScaleLog2;
                }
            } else {
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    qb[st] = __builtin_bit_cast(
                        bf8, __builtin_amdgcn_raw_buffer_load_b128(rq, (lane_vec + 8 * hh + 16 * st) * 2, 0, 0));
            }
        }

        // O^T accumulators.  bf16: o0 holds dims 0..31 and o1 dims 32..63; fp32:
        // o0 holds the even dims and o1 the odd ones (row m of each is dim 2m or
        // 2m+1), so one 8-byte LDS read gives a lane both of its V operands.
        f16v o0 = {}, o1 = {};
        float m = -1e30f;        // running max (log2 units); finite, below any score
        float thr = -1e30f;      // rescale when a block maximum exceeds this
        float l = 0.f;           // this lane's share of the running denominator

        // ---- per-lane LDS offsets of the MFMA operands (swizzle folded in) ----
        // The XOR codes depend only on the row index mod 16 (K) or mod 8 (V),
        // and every stage, tile and sub-block offset is a multiple of 16 rows
        // (V reads step by 8 rows), so each lane's operand addresses are a
        // handful of fixed offsets plus immediates.
        //  fp32 K: chunk 8*hh + c of row n           (c = 0..7)
        //  fp32 V: dwords 2n, 2n+1 of row 4*hh + q   (q = 0..3; row + 8*(t/4))
        //  bf16 K: chunk 2*st + hh of row n          (st = 0..3)
        //  bf16 V: transposed 4-key x 16-dim blocks, one offset per 32-dim half
        int koff[kF32 ? 8 : 4];
        int voff[kF32 ? 4 : 2];
        if constexpr (kF32) {
#pragma unroll
            for (int c = 0; c < 8; ++c) koff[c] = G::kKBase + n * kRB + (((8 * hh + c) ^ k_code<T>(n)) * 16);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int r = 4 * hh + q4;
                voff[q4] = r * kRB + (((n >> 1) ^ chunk_code<T>(r)) * 16) + (n & 1) * 8;
            }
        } else {
#pragma unroll
            for (int st = 0; st < 4; ++st) koff[st] = G::kKBase + n * kRB + (((2 * st + hh) ^ k_code<T>(n)) * 16);
            const int grp = (lane >> 4) & 1;
            const int j = lane & 15;
            const int r = 4 * hh + (j >> 2);            // row within an 8-row block
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int dim = 32 * nt + 16 * grp + 4 * (j & 3);
                voff[nt] = r * kRB + (((dim >> 3) ^ chunk_code<T>(r)) * 16) + (dim & 4) * 2;
            }
        }

        // ---- bf16 V operands of a sub-block, read ahead ----
        // Transposed LDS reads: within each 16-lane group, lane j points at 4 dims
        // of key K0 + j/4 and receives dim D0 + j of keys K0..K0+3, which is the A
        // operand V^T[dim][key] of the PV MFMA.  The compiler cannot tell these
        // reads apart from the LDS writes of loads in flight and would wait for
        // every outstanding load before them, so each tile's are made before the
        // next tile's loads are issued.
        struct VOpsBf16 {
            bf8 a[2][2];                         // [key half u][dim half nt]
        };
        struct NoVOps {};                        // fp32 reads V inside the sub-block
        using VOps = std::conditional_t<kF32, NoVOps, VOpsBf16>;
        auto read_v = [&](auto stage_c, auto sbc) {
            constexpr int kStage = decltype(stage_c)::value;
            constexpr int sb = decltype(sbc)::value;
            const unsigned char* Vs = lds_raw + kStage * G::kTileBytes + 32 * sb * kRB;
            VOpsBf16 vo;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const unsigned char* a = Vs + 16 * u * kRB + voff[nt];
                    const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a);
                    const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a + 8 * kRB));
                    vo.a[u][nt] = __builtin_shufflevector(__builtin_bit_cast(bf4, h0), __builtin_bit_cast(bf4, h1),
                                                          0, 1, 2, 3, 4, 5, 6, 7);
                }
            return vo;
        };

        // ---- one 32-key sub-block: scores, mask, online softmax, PV ----
        // `stage_c` and `sb` are compile-time constants at every call; the K
        // offsets koff[] carry the K region's base.
        auto sub_block = [&](auto stage_c, auto sbc, int jb, const VOps& vo) {
            constexpr int kStage = decltype(stage_c)::value;
            constexpr int sb = decltype(sbc)::value;
            const unsigned char* Ks = lds_raw + kStage * G::kTileBytes + 32 * sb * kRB;
            const unsigned char* Vs = lds_raw + kStage * G::kTileBytes + 32 * sb * kRB;
            f16v s = {};
            if constexpr (kF32) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const f4 kx = *reinterpret_cast<const f4*>(Ks + koff[c]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kx[e], qf[4 * c + e], s, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const bf8 kx = __builtin_bit_cast(bf8, *reinterpret_cast<const u16x8*>(Ks + koff[st]));
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx, qb[st], s, 0, 0, 0);
                }
            }
            // causal mask, only where the sub-block crosses the wave's first row edge
            if (jb + 31 > w_first) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = jb + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key > lim) s[r] = -INFINITY;
                }
            }
            // Lazy rescale: m moves only when a block maximum exceeds it by more
            // than kRescaleSlack (log2 units), so every weight stays within
            // 2^slack.  The block maximum uses the NaN-propagating v_maximum3_f32,
            // which unlike fmaxf needs no quieting of the MFMA results first.
            auto block_max = [&]() {
                float bm = s[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) bm = __builtin_elementwise_maximum(bm, s[r]);
                return half_max(bm);
            };
            auto rescale = [&](float bl, bool upd) {   // bl: block maximum, log2 units
                const float alpha = upd ? fast_exp2(m - bl) : 1.0f;
                if (upd) {
                    m = bl;
                    thr = kF32 ? m + kRescaleSlack : (m + kRescaleSlack) * kInvScaleLog2;
                }
                l *= alpha;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    o0[r] *= alpha;
                    o1[r] *= alpha;
                }
            };
            float p[16];
            if constexpr (kF32) {
                // Weights first, against the current m.  Their lane sum bounds each
                // of them, so the block maximum is formed only in a wave where some
                // lane's sum exceeds 2^slack; there the rescale test is the usual
                // one (a lane whose maximum passes it always has such a sum).
                auto weights = [&]() {
#pragma unroll
                    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(s[r] - m);
                    float ps = p[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) ps += p[r];
                    return ps;
                };
                float ps = weights();
                if (__ballot(ps > kSlackWeight)) {
                    const float bm = block_max();
                    rescale(bm, bm > thr);
                    ps = weights();
                }
                l += ps;
            }
            bf8 pbv[2];   // bf16: the weights rounded to nearest even, PV operand B
            if constexpr (!kF32) {
                // Same scheme on the rounded weights (bf16 scores are raw dot
                // products: thr is in raw units); the denominator sums exactly
                // the weights the PV product uses.
                constexpr bf2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};
                auto weights = [&]() {
                    const float mu = m;
#pragma unroll
                    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(s[r], kScaleLog2, -mu));
                    float ps = 0.f;
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) pbv[u][e] = (__bf16)p[8 * u + e];
#pragma unroll
                        for (int e = 0; e < 8; e += 2)
                            ps = __builtin_amdgcn_fdot2_f32_bf16(bf2{pbv[u][e], pbv[u][e + 1]}, kOnes, ps, false);
                    }
                    return ps;
                };
                float ps = weights();
                if (__ballot(ps > kSlackWeight)) {
                    const float bm = block_max();
                    rescale(bm * kScaleLog2, bm > thr);
                    ps = weights();
                }
                l += ps;
            }
            if constexpr (kF32) {
                // key 8(t/4) + 4hh + t%4 of the sub-block: V[key][2n] and V[key][2n+1]
#pragma unroll
                for (int t4 = 0; t4 < 16; ++t4) {
                    const f2 vr = *reinterpret_cast<const f2*>(Vs + 8 * (t4 >> 2) * kRB + voff[t4 & 3]);
                    o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[0], p[t4], o0, 0, 0, 0);
                    o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[1], p[t4], o1, 0, 0, 0);
                }
            } else {
                (void)Vs;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vo.a[u][0], pbv[u], o0, 0, 0, 0);
                    o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vo.a[u][1], pbv[u], o1, 0, 0, 0);
                }
            }
        };

        // This wave's sub-block of tile t (sub-block wp: one per wave), read from
        // stage kStage; the dispatch on the runtime split index
        // keeps every LDS offset an immediate.
        static_assert(kNB == KS, "each wave takes exactly one 32-key sub-block of a tile");
        auto active = [&](int t) { return wave_active && kb + t * kBK + 32 * wp <= w_last; };
        auto prefetch_v = [&](auto stage_off, int t) {
            VOps vo{};
            if constexpr (!kF32) {
                if (active(t)) {
                    [&]<int... W>(std::integer_sequence<int, W...>) {
                        ((wp == W ? (vo = read_v(stage_off, std::integral_constant<int, W>{}), 0) : 0), ...);
                    }(std::make_integer_sequence<int, KS>{});
                }
            }
            return vo;
        };
        auto consume = [&](auto stage_off, int t, const VOps& vo) {
            if (!active(t)) return;
            const int jb = kb + t * kBK + 32 * wp;
            [&]<int... W>(std::integer_sequence<int, W...>) {
                ((wp == W ? (sub_block(stage_off, std::integral_constant<int, W>{}, jb, vo), 0) : 0), ...);
            }(std::make_integer_sequence<int, KS>{});
        };

        // ---- key loop over staged tiles (double-buffered, unrolled by two) ----
        // Tile t+1's loads go to the other stage while tile t is consumed; that
        // stage was last read before the previous barrier.
        __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): tile 0 (and Q) have landed in LDS
        __syncthreads();
        if (it < 2) mark(it == 0 ? 4 : 7);       // the item's first tile is in LDS
        if constexpr (kQLds) {
            // qf[s] = q[row][head][32*hh + s] * log2(e)/8 from this wave's rows of qbuf
            int lane3 = lane;
            asm volatile("" : "+v"(lane3));
            const int qr = 8 * wr + ((lane3 & 31) >> 2);   // row within the item
            const int qh = lane3 & 3;
            const int qhh = lane3 >> 5;
            const unsigned char* qrow = qbuf + qr * kQRowBytes;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int pos = (qh * 16 + qhh * 8 + c) ^ ((4 * (qr & 3) + qh) & 15);
                const f4 x = *reinterpret_cast<const f4*>(qrow + pos * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) qf[4 * c + e] = x[e] * kScaleLog2;
            }
        }
        // The next work item's Q goes into qbuf once every wave has read this
        // one's, i.e. after the barrier that ends tile 0; it lands with tile 1.
        auto stage_next_q = [&](int t) {
            if constexpr (kQAfter && ST == 2) {    // one-stage plans have one item per workgroup
                if (t == 0 && it + 1 < nitems) {
                    issue_q(items[it + 1] * kRows);
                    q_staged = true;
                }
            } else {
                (void)t;
            }
        };
        // One staging buffer: every tile is consumed, then the next is loaded
        // into the same buffer; the other workgroup on the CU computes meanwhile.
        // Paged: the table entries of tile t+2 are read while tile t is
        // consumed and their offsets stored while tile t+1's loads are in
        // flight, into the slot tile t's loads used (read before the barrier
        // that ends tile t); the barrier after those loads publishes them.
        if constexpr (ST == 1) {
            for (int t = 0; t < ntiles; ++t) {
                const VOps vo = prefetch_v(std::integral_constant<int, 0>{}, t);
                int ent = 0;
                if constexpr (PAGED) {
                    if (t + 2 < ntiles) ent = fetch_entry(t + 2);
                }
                consume(std::integral_constant<int, 0>{}, t, vo);
                __syncthreads();                      // every wave is done with the tile
                if (t + 1 < ntiles) {
                    issue_tile(t + 1, 0);
                    if constexpr (PAGED) {
                        if (t + 2 < ntiles) store_offset(t + 2, ent);
                    }
                    stage_next_q(t);
                    __builtin_amdgcn_s_waitcnt(0x3f70);
                    __syncthreads();
                }
            }
        }
        // Paged: the table entries of tile t+2 are read during tile t and their
        // offsets stored after its vmcnt(0), into the slot tile t's loads used
        // (every wave issued those before the previous barrier).
        for (int t = 0; ST == 2 && t < ntiles; t += 2) {
            VOps vo = prefetch_v(std::integral_constant<int, 0>{}, t);
            if constexpr (kQInStage1) {
                if (t == 0) __syncthreads();          // every wave has read its Q out of the second stage
            }
            if (t + 1 < ntiles) issue_tile(t + 1, 1);
            int ent = 0;
            if constexpr (PAGED) {
                if (t + 2 < ntiles) ent = fetch_entry(t + 2);
            }
            consume(std::integral_constant<int, 0>{}, t, vo);
            __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): tile t+1 has landed
            if constexpr (PAGED) {
                if (t + 2 < ntiles) store_offset(t + 2, ent);
            }
            __syncthreads();
            if (t + 1 < ntiles) {
                vo = prefetch_v(std::integral_constant<int, 1>{}, t + 1);
                if (t + 2 < ntiles) issue_tile(t + 2, 0);
                stage_next_q(t);
                if constexpr (PAGED) {
                    if (t + 3 < ntiles) ent = fetch_entry(t + 3);
                }
                consume(std::integral_constant<int, 1>{}, t + 1, vo);
                __builtin_amdgcn_s_waitcnt(0x3f70);
                if constexpr (PAGED) {
                    if (t + 3 < ntiles) store_offset(t + 3, ent);
                }
                __syncthreads();
            }
        }

        if (it == 0) mark(5);                    // the first item's key loop is done
        // Lane offsets used after the key loop are formed again from an opaque
        // copy of the lane index, so they are not held (or spilled) through it.
        int lane2 = lane;
        asm volatile("" : "+v"(lane2));
        const uint32_t out_vec = (uint32_t)((8 * wr + ((lane2 & 31) >> 2)) * kHQ + g * kGroup + (lane2 & 3)) * kD;
        const int hh2 = lane2 >> 5;              // the half-wave, from the same copy

        // ---- merge key splits (log-sum-exp), in LDS ----
        if constexpr (KS > 1) {
            float* mb = reinterpret_cast<float*>(lds_raw);
            if (wp > 0 && wave_active) {
                float* dst = mb + (size_t)((wr * (KS - 1) + wp - 1) * 34) * 64 + lane2;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    dst[r * 64] = o0[r];
                    dst[(16 + r) * 64] = o1[r];
                }
                dst[32 * 64] = m;
                dst[33 * 64] = l;
            }
            __syncthreads();
            if (wp == 0 && wave_active) {
#pragma unroll
                for (int sp = 1; sp < KS; ++sp) {
                    const float* src = mb + (size_t)((wr * (KS - 1) + sp - 1) * 34) * 64 + lane2;
                    const float m2 = src[32 * 64];
                    const float l2 = src[33 * 64];
                    const float mx = fmaxf(m, m2);
                    const float a = fast_exp2(m - mx);
                    const float b = fast_exp2(m2 - mx);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        o0[r] = a * o0[r] + b * src[r * 64];
                        o1[r] = a * o1[r] + b * src[(16 + r) * 64];
                    }
                    l = a * l + b * l2;
                    m = mx;
                }
            }
        }

        // ---- epilogue: one division per query, fp32 stores ----
        // This lane's 32 values of its (row, head) output vector, times sc, in
        // dim order; accumulator element r sits in row 8(r/4) + 4hh + r%4 of
        // its 32-row block.
        // `item` points at the output of row i0, head 0; rows past the chunk
        // fall outside the descriptor and are not written.
        auto store_o = [&](float* item, float sc) {
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                (void*)item, (short)0, (uint32_t)item_rows * kHQ * kD * 4, 0x00020000);
            auto st4 = [&](uint32_t elem, f4 x) {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), ro, (out_vec + elem) * 4, 0, 0);
            };
            if constexpr (kF32) {
                // rows 8a+4hh+j: dims 16a+8hh+2j (o0), +1 (o1)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    st4(8 * hh2 + 16 * a, f4{o0[4 * a] * sc, o1[4 * a] * sc, o0[4 * a + 1] * sc, o1[4 * a + 1] * sc});
                    st4(8 * hh2 + 16 * a + 4,
                        f4{o0[4 * a + 2] * sc, o1[4 * a + 2] * sc, o0[4 * a + 3] * sc, o1[4 * a + 3] * sc});
                }
            } else {
                // rows 8a+4hh+j: dims 8a+4hh+j (o0), +32 (o1)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    st4(4 * hh2 + 8 * a, f4{o0[4 * a] * sc, o0[4 * a + 1] * sc, o0[4 * a + 2] * sc, o0[4 * a + 3] * sc});
                    st4(4 * hh2 + 32 + 8 * a,
                        f4{o1[4 * a] * sc, o1[4 * a + 1] * sc, o1[4 * a + 2] * sc, o1[4 * a + 3] * sc});
                }
            }
        };
        if constexpr (SPLIT) {
            // key split: unnormalised partial O, running max m and denominator l
            if (wp == 0 && wave_active && row < C) {
                const float lt = half_sum(l);
                const size_t qi = ((size_t)split * C + row) * kHQ + head;
                store_o(ks.part + ((size_t)split * C + i0) * kHQ * kD, 1.0f);
                if (hh == 0) {
                    float* ml = ks.part + (size_t)ks.n * C * kHQ * kD + qi * 2;
                    ml[0] = m;
                    ml[1] = lt;
                }
            }
        } else if constexpr (KS > 1 && NW > 1) {
            // Items of 16 rows or more: normalised rows through LDS, then
            // full-line stores.  Wave (wr, 0) writes its 8 rows x 4 heads x 64
            // dims into its own merge slots (read only by itself above), 16-byte
            // chunks XOR-permuted by (row * 4 + head) % 16 so that a write
            // instruction spreads over all banks; after a barrier every wave
            // stores whole 1 KiB rows, four lanes per 64-byte line, as
            // non-temporal writes.  (8-row items store from registers: there
            // the extra barrier costs more than the whole lines gain.)
            (void)ks;
            (void)store_o;
            float* const stg0 = reinterpret_cast<float*>(lds_raw);
            constexpr int kSlotFloats = (KS - 1) * 34 * 64;       // one row-wave's merge slots
            if (wp == 0 && wave_active) {
                const float lt = half_sum(l);
                const float inv = 1.0f / lt;
                const int rw = (lane2 & 31) >> 2, hd = lane2 & 3;
                const int f = (rw * 4 + hd) & 15;
                float* const base = stg0 + wr * kSlotFloats + rw * 256 + hd * 64;
                auto put = [&](int dim, f4 x) {   // dim: a multiple of 4
                    const int c = dim >> 2;
                    *reinterpret_cast<f4*>(base + ((c ^ f) << 2)) = x;
                };
                if constexpr (kF32) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        put(8 * hh2 + 16 * a, f4{o0[4 * a] * inv, o1[4 * a] * inv, o0[4 * a + 1] * inv, o1[4 * a + 1] * inv});
                        put(8 * hh2 + 16 * a + 4,
                            f4{o0[4 * a + 2] * inv, o1[4 * a + 2] * inv, o0[4 * a + 3] * inv, o1[4 * a + 3] * inv});
                    }
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        put(4 * hh2 + 8 * a, f4{o0[4 * a] * inv, o0[4 * a + 1] * inv, o0[4 * a + 2] * inv, o0[4 * a + 3] * inv});
                        put(4 * hh2 + 32 + 8 * a,
                            f4{o1[4 * a] * inv, o1[4 * a + 1] * inv, o1[4 * a + 2] * inv, o1[4 * a + 3] * inv});
                    }
                }
            }
            __syncthreads();
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(out + (size_t)i0 * kHQ * kD), (short)0, (uint32_t)item_rows * kHQ * kD * 4, 0x00020000);
            int L = lane;
            asm volatile("" : "+v"(L));
            const int hd = L >> 4, c = L & 15;
#pragma unroll
            for (int u = 0; u < kRows / G::kWaves; ++u) {
                const int r = wid + u * G::kWaves;               // item row; rows past the chunk are not written
                const int rw = r & 7;
                const float* src = stg0 + (r >> 3) * kSlotFloats + rw * 256 + hd * 64 + ((c ^ ((rw * 4 + hd) & 15)) << 2);
                const f4 x = *reinterpret_cast<const f4*>(src);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), ro,
                                                       (uint32_t)((r * kHQ + g * kGroup) * kD * 4 + L * 16), 0, 2);
            }
        } else if (wp == 0 && wave_active) {
            (void)ks;
            const float lt = half_sum(l);
            const float inv = 1.0f / lt;
            if (row < C) store_o(out + (size_t)i0 * kHQ * kD, inv);
        }
        __syncthreads();   // LDS is reused by the next work item
        if (it == 0) mark(6);                    // the first item's output is stored
    }
    if (kLog && clk != nullptr && threadIdx.x == 0) {
        clk[kClockWords * blockIdx.x + 2] = __builtin_amdgcn_s_memtime();
        clk[kClockWords * blockIdx.x + 3] = __builtin_amdgcn_s_memrealtime();
    }
}

// ---------------------------------------------------------------------------
// Per-row baseline ("Inference Attention 2: Flash Prefill Against a Cached
// Prefix", Lesson: the starter serves each (query row, head) on its own and
// every row streams its whole K/V prefix from memory; nothing is staged or
// shared between rows).  One 64-lane wave per (row, head), keys in blocks of
// 64: for the scores lane j takes key j0 + j (its whole K row against the
// query, which every lane holds), for the weighted sum lane d takes output dim
// d (one coalesced V row per key, each key's weight broadcast from its lane).
// The online softmax state moves once per block: block maximum, one rescale
// of the denominator and accumulator, the block's weights.  The traffic per
// row is its whole prefix, which is what the tiled kernel is timed against.
// ---------------------------------------------------------------------------
constexpr int kRowWaves = 4;     // waves (rows) per workgroup

template <typename T>
__device__ __forceinline__ float load_elem(const T* p) {
    if constexpr (sizeof(T) == 4) {
        return *reinterpret_cast<const float*>(p);
    } else {
        return (float)*p;
    }
}

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// 8 consecutive elements as floats (one 16-byte load in bf16, two in fp32)
template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&x)[8]) {
    if constexpr (sizeof(T) == 4) {
        const f4 a = *reinterpret_cast<const f4*>(p);
        const f4 b = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    } else {
        const bf8 a = *reinterpret_cast<const bf8*>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
    }
}

template <typename T>
__global__ void __launch_bounds__(64 * kRowWaves)
attn_rowwise_kernel(const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
                    float* __restrict__ out, int C, int P) {
    const int lane = threadIdx.x & 63;
    const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowWaves + (threadIdx.x >> 6));
    const int h = blockIdx.y;
    if (row >= C) return;                              // whole waves leave together
    const int g = h / kGroup;
    float qv[kD];                                      // the query, scaled; the same in every lane
    const T* qrow = q + ((size_t)row * kHQ + h) * kD;
#pragma unroll
    for (int c = 0; c < kD; c += 8) {
        float x[8];
        load8f(qrow + c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[c + e] = x[e] * kScaleLog2;
    }
    constexpr size_t kPos = (size_t)kHKV * kD;         // elements between positions
    const T* kg = kc + (size_t)g * kD;                 // KV head g at position 0
    const T* vg = vc + (size_t)g * kD + lane;          // dim `lane` of KV head g at position 0
    const int n = P + row + 1;                         // visible keys
    float run_max = -INFINITY, denom = 0.f, acc = 0.f;
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int last = n - 1 - j0;                   // lanes past it hold no key
        const T* krow = kg + (size_t)(j0 + min(lane, last)) * kPos;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < kD; c += 8) {
            float x[8];
            load8f(krow + c, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) s = __builtin_fmaf(qv[c + e], x[e], s);
        }
        if (lane > last) s = -INFINITY;
        const float next = fmaxf(run_max, wave_max64(s));
        const float keep = fast_exp2(run_max - next);  // 0 on the first block (run_max = -inf)
        const float w = fast_exp2(s - next);           // 0 for a lane with no key
        denom = denom * keep + wave_sum64(w);
        acc *= keep;
        const int cnt = min(64, last + 1);
#pragma unroll 8
        for (int b = 0; b < 64; ++b) {                 // weights past cnt are 0; their loads stay in range
            const float vb = load_elem(vg + (size_t)(j0 + min(b, cnt - 1)) * kPos);
            acc = __builtin_fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), b)), vb, acc);
        }
        run_max = next;
    }
    out[((size_t)row * kHQ + h) * kD + lane] = acc / denom;
}

// ---------------------------------------------------------------------------
// Merge of key-split partials ("FlashAttention and inference kernels",
// Exercises, exercise 2): m = max_s m_s, w_s = 2^(m_s - m), out = sum_s w_s O_s /
// sum_s w_s l_s over the splits a row reaches (s*len <= P + row), so no empty
// segment takes part.  One wave per (row, head), one lane per dim.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
attn_merge_splits_kernel(const float* __restrict__ part, float* __restrict__ out, int C, int P, int len, int n) {
    // (row, head) index, wave-uniform: split offsets below stay scalar
    const int qi = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (qi >= C * kHQ) return;                           // whole waves leave together
    const int row = qi / kHQ;
    const int lane = threadIdx.x & 63;                   // output dim; also a split index below
    const int ns = min(n, (P + row) / len + 1);
    const float* ml = part + (size_t)n * C * kHQ * kD;
    const size_t stride = (size_t)C * kHQ;              // between splits, in (row, head) units
    // 32 splits at a time (the planners make at most 32), all their loads
    // issued together (indices clamped into range; the weight of a clamped
    // slot, and of lanes 32..63, is 0), combined online; the weighted sum of a
    // chunk in four independent FMA chains
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 32) {
        const int cnt = min(32, ns - s0);
        const int sl = s0 + min(lane & 31, cnt - 1);
        const float ms = ml[(sl * stride + qi) * 2];
        const float ls = ml[(sl * stride + qi) * 2 + 1];
        const float* src = part + ((size_t)s0 * stride + qi) * kD + lane;
        float x[32];
#pragma unroll
        for (int t = 0; t < 32; ++t) x[t] = src[(size_t)min(t, cnt - 1) * stride * kD];
        const bool valid = lane < cnt;                    // lanes 32..63 repeat 0..31
        const float mc = wave_max64(valid ? ms : -INFINITY);
        const float mn = fmaxf(M, mc);                   // finite: every reached split saw a key
        const float scale = fast_exp2(M - mn);           // 0 on the first chunk
        const float w = valid ? fast_exp2(ms - mn) : 0.f;
        L = L * scale + wave_sum64(w * ls);
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 32; ++t)
            a[t & 3] = __builtin_fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), t)), x[t], a[t & 3]);
        O = O * scale + ((a[0] + a[1]) + (a[2] + a[3]));
        M = mn;
    }
    out[(size_t)qi * kD + lane] = O / L;
}

// ---------------------------------------------------------------------------
// Single fp32 token (C = 1) for the split-KV entry point ("FlashAttention and
// inference kernels", Flash-Decoding: split the key range, one partial
// (O, m, l) per split, merged afterwards).  One token leaves 31 of the 32
// query slots of an MFMA tile empty, and fp32 MFMAs cost as much time as the
// loads here, so this kernel uses plain FMAs instead:
// lane = 8 * key slot + dim slice; the 8 lanes of a key slot each hold 8 dims
// of q (4 heads of the group) and of the key's K and V rows.  Every key slot
// runs its own online softmax over the keys it visits (no cross-lane traffic
// in the loop beyond the 3-step sum of the dot products); the slots, then the
// waves, are merged at the end by the log-sum-exp rule.  Partials use the
// layout and log2 units of the MFMA split kernel, so the same merge kernel
// finishes the job.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 4;        // waves per workgroup
constexpr int kDecUnroll = 4;       // key chunks (8 keys per wave) loaded together
constexpr float kDecFloor = -1e30f; // running-max start: finite, below any score

__device__ __forceinline__ void load_row8(const float* p, float (&x)[8]) {
    const f4 a = *reinterpret_cast<const f4*>(p);
    const f4 b = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[4 + e] = b[e];
    }
}

__device__ __forceinline__ void load_row8(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[8]) {
    const f4 a = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    const f4 b = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[4 + e] = b[e];
    }
}

// sum over the 8 consecutive lanes of a key slot; every lane ends with the
// same bits (each step adds the same two values in either order)
__device__ __forceinline__ float slot_sum8(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // lane ^ 1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // lane ^ 2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // 7 - lane
    return x;
}

// PAGED: kc and vc are the page pools [numBlocks][pageSize][8][64] and a
// position's row is found through the block table ("FlashAttention and
// inference kernels", section PagedAttention); the table entries of a chunk's
// keys are read one chunk ahead, so a row load waits on no table read.
template <bool PAGED>
__global__ void __launch_bounds__(64 * kDecWaves)
attn_decode_split_kernel(const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
                         float* __restrict__ part, int P, int len, int n, PagedCache pg) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = lane >> 3;         // key slot 0..7
    const int ds = lane & 7;            // dims 8*ds .. 8*ds+7
    const int g = blockIdx.x % kHKV;
    const int split = blockIdx.x / kHKV;
    const int total = P + 1;
    const int kbeg = split * len;
    const int kend = min(total, kbeg + len);

    float qf[4][8];                     // q of heads 4g..4g+3, scaled by log2(e)/8
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        load_row8(q + (size_t)(kGroup * g + h) * kD + 8 * ds, qf[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[h][e] *= kScaleLog2;
    }
    float m[4], l[4], acc[4][8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        m[h] = kDecFloor;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    // Paged cache: the pools and the table are read through buffer
    // descriptors, so a row whose table entry is out of range (given an
    // offset past the pool) reads as zero keys and values, as in the tiled
    // kernel; row offsets are 32-bit (the host bounds pool and table sizes).
    constexpr uint32_t kRowBytes = kD * 4;
    const uint32_t pool_bytes = PAGED ? (uint32_t)((size_t)pg.num_blocks * pg.page_size * kHKV * kRowBytes) : 0u;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kc, (short)0, pool_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vc, (short)0, pool_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rtab = __builtin_amdgcn_make_buffer_rsrc(
        (void*)pg.table, (short)0, PAGED ? (uint32_t)((total + pg.page_size - 1) / pg.page_size) * 4u : 0u,
        0x00020000);
    // byte offset of this lane's 8 dims of position `key` in the pools
    auto row_offset = [&](int key, int entry) -> uint32_t {
        const uint32_t in_page = page_slot((uint32_t)key, page_index((uint32_t)key, pg), pg);
        return (uint32_t)entry < (uint32_t)pg.num_blocks
                   ? (pool_position((uint32_t)entry, in_page, pg) * kHKV + g) * kRowBytes + 32u * ds
                   : pool_bytes;
    };
    auto table_entry = [&](int key) -> int {   // key < kend, or the entry is not used
        return (int)__builtin_amdgcn_raw_buffer_load_b32(rtab, page_index((uint32_t)min(key, kend - 1), pg) * 4u, 0, 0);
    };

    constexpr int kStep = 8 * kDecWaves;    // keys between a wave's consecutive chunks
    int ent[kDecUnroll] = {};               // paged: table entries of this iteration's keys
    if constexpr (PAGED) {
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) ent[u] = table_entry(kbeg + 8 * w + kStep * u + slot);
    }
    for (int c0 = kbeg + 8 * w; c0 < kend; c0 += kStep * kDecUnroll) {
        float kx[kDecUnroll][8], vx[kDecUnroll][8];
        bool ok[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const int key = c0 + kStep * u + slot;
            ok[u] = key < kend;
            if constexpr (PAGED) {
                const uint32_t off = row_offset(ok[u] ? key : kbeg, ok[u] ? ent[u] : -1);
                load_row8(rk, off, kx[u]);
                load_row8(rv, off, vx[u]);
            } else {
                const size_t off = ((size_t)(ok[u] ? key : kbeg) * kHKV + g) * kD + 8 * ds;   // in range either way
                load_row8(kc + off, kx[u]);
                load_row8(vc + off, vx[u]);
            }
        }
        if constexpr (PAGED) {
            // the next iteration's table entries, in flight during this one's math
#pragma unroll
            for (int u = 0; u < kDecUnroll; ++u) ent[u] = table_entry(c0 + kStep * kDecUnroll + kStep * u + slot);
        }
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qf[h][e], kx[u][e], d);
                d = slot_sum8(d);
                const float sv = ok[u] ? d : -INFINITY;
                if (sv > m[h] + kRescaleSlack) {    // rare after the first keys
                    const float alpha = fast_exp2(m[h] - sv);
                    m[h] = sv;
                    l[h] *= alpha;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
                }
                const float pr = fast_exp2(sv - m[h]);   // 0 for a key past the range
                l[h] += pr;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(pr, vx[u][e], acc[h][e]);
            }
        }
    }

    // merge the 8 key slots of the wave (lanes 8 apart hold the same dims):
    // slots 8 apart by a DPP rotate within 16-lane rows, then rows and halves
    // by permlane swaps; every step combines the same two partials in both
    // lanes, in either order
    auto merge_with = [&](auto other) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float m0, m1, l0, l1;
            other(m[h], m0, m1);
            other(l[h], l0, l1);
            const float mm = fmaxf(m0, m1);
            const float a = fast_exp2(m0 - mm), b = fast_exp2(m1 - mm);
            l[h] = a * l0 + b * l1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x0, x1;
                other(acc[h][e], x0, x1);
                acc[h][e] = a * x0 + b * x1;
            }
            m[h] = mm;
        }
    };
    merge_with([](float x, float& a, float& b) {
        a = x;
        b = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));   // row_ror 8
    });
    merge_with([](float x, float& a, float& b) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    });
    merge_with([](float x, float& a, float& b) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    });
    // merge the waves through LDS: per wave and head, 64 dims + m + l
    __shared__ float sm[kDecWaves][4][kD + 2];
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm[w][h][8 * ds + e] = acc[h][e];
            if (ds == 0) {
                sm[w][h][kD] = m[h];
                sm[w][h][kD + 1] = l[h];
            }
        }
    }
    __syncthreads();
    if (tid >= 4 * kD) return;              // the first 256 threads: 4 heads x 64 dims
    const int h = tid >> 6, d = tid & 63;
    float mm = sm[0][h][kD];
#pragma unroll
    for (int v = 1; v < kDecWaves; ++v) mm = fmaxf(mm, sm[v][h][kD]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) {
        const float wt = fast_exp2(sm[v][h][kD] - mm);
        O += wt * sm[v][h][d];
        L += wt * sm[v][h][kD + 1];
    }
    const size_t qi = (size_t)split * kHQ + kGroup * g + h;   // C = 1: (split, row 0, head)
    part[qi * kD + d] = O;
    if (d == 0) {
        float* ml = part + (size_t)n * kHQ * kD + qi * 2;
        ml[0] = mm;
        ml[1] = L;
    }
}

// ---------------------------------------------------------------------------
// Naive three-kernel pipeline ("Inference Attention 1: The Full Score Matrix",
// Lesson): prompt prefill (P = 0) as an eager framework runs it, with the whole
// 32 x T x T fp32 score matrix in a caller workspace between the kernels.
//  1. scores: S[h][i][j] = q[i][h] . k[j][h/4] / 8, -inf above the diagonal
//  2. row softmax in place (max subtracted; 0 above the diagonal)
//  3. weighted sum: out[i][h] = sum_j S[h][i][j] v[j][h/4]
// It exists to be measured against the fused path: it moves the T x T matrix
// through memory four times.
// ---------------------------------------------------------------------------
constexpr int kNT = 64;   // tile edge of the two matrix products

__global__ void __launch_bounds__(256)
naive_scores_kernel(const float* __restrict__ q, const float* __restrict__ k, float* __restrict__ S, int T) {
    const int h = blockIdx.z, g = h / kGroup;
    const int i0 = blockIdx.y * kNT, j0 = blockIdx.x * kNT;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;   // 4 x 4 outputs per thread
    float* Sh = S + (size_t)h * T * T;
    if (j0 > i0 + kNT - 1) {                                   // wholly above the diagonal
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int i = i0 + 4 * ty + a, j = j0 + 4 * tx + b;
                if (i < T && j < T) Sh[(size_t)i * T + j] = -INFINITY;
            }
        return;
    }
    __shared__ float qs[kNT][kNT + 1];
    __shared__ float ks[kNT][kNT + 1];
    for (int e = threadIdx.x; e < kNT * kNT; e += 256) {
        const int r = e / kNT, c = e % kNT;
        qs[r][c] = i0 + r < T ? q[((size_t)(i0 + r) * kHQ + h) * kD + c] : 0.f;
        ks[r][c] = j0 + r < T ? k[((size_t)(j0 + r) * kHKV + g) * kD + c] : 0.f;
    }
    __syncthreads();
    float acc[4][4] = {};
    for (int c = 0; c < kD; ++c) {
        float qa[4], kb4[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) qa[a] = qs[4 * ty + a][c];
#pragma unroll
        for (int b = 0; b < 4; ++b) kb4[b] = ks[4 * tx + b][c];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] += qa[a] * kb4[b];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = i0 + 4 * ty + a, j = j0 + 4 * tx + b;
            if (i < T && j < T) Sh[(size_t)i * T + j] = j <= i ? acc[a][b] * 0.125f : -INFINITY;
        }
}

__global__ void __launch_bounds__(256)
naive_softmax_kernel(float* __restrict__ S, int T) {
    float* row = S + ((size_t)blockIdx.y * T + blockIdx.x) * T;
    __shared__ float red[4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float mx = -INFINITY;
    for (int j = threadIdx.x; j < T; j += 256) mx = fmaxf(mx, row[j]);
    mx = wave_max64(mx);
    if (lane == 0) red[w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.f;
    for (int j = threadIdx.x; j < T; j += 256) {
        const float e = __expf(row[j] - mx);
        row[j] = e;
        sum += e;
    }
    sum = wave_sum64(sum);
    if (lane == 0) red[w] = sum;
    __syncthreads();
    const float inv = 1.0f / (red[0] + red[1] + red[2] + red[3]);
    for (int j = threadIdx.x; j < T; j += 256) row[j] *= inv;
}

__global__ void __launch_bounds__(256)
naive_pv_kernel(const float* __restrict__ S, const float* __restrict__ v, float* __restrict__ out, int T) {
    const int h = blockIdx.y, g = h / kGroup;
    const int i0 = blockIdx.x * kNT;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;   // rows 4*ty+a, dims 4*tx+b
    const float* Sh = S + (size_t)h * T * T;
    __shared__ float ps[kNT][kNT + 1];
    __shared__ float vs[kNT][kNT + 1];
    float acc[4][4] = {};
    for (int j0 = 0; j0 < T; j0 += kNT) {
        for (int e = threadIdx.x; e < kNT * kNT; e += 256) {
            const int r = e / kNT, c = e % kNT;
            ps[r][c] = (i0 + r < T && j0 + c < T) ? Sh[(size_t)(i0 + r) * T + j0 + c] : 0.f;
            vs[r][c] = j0 + r < T ? v[((size_t)(j0 + r) * kHKV + g) * kD + c] : 0.f;
        }
        __syncthreads();
        for (int c = 0; c < kNT; ++c) {
            float pa[4], vb[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) pa[a] = ps[4 * ty + a][c];
#pragma unroll
            for (int b = 0; b < 4; ++b) vb[b] = vs[c][4 * tx + b];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] += pa[a] * vb[b];
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int i = i0 + 4 * ty + a;
        if (i >= T) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) out[((size_t)i * kHQ + h) * kD + 4 * tx + b] = acc[a][b];
    }
}

// ---------------------------------------------------------------------------
// Host side: argument checks, launch plan, dispatch.
// ---------------------------------------------------------------------------
enum Variant { kV_4x2 = 0, kV_2x4 = 1, kV_1x4 = 2, kV_4x4 = 3, kV_decode = 4, kV_8x2 = 5, kV_1x4s1 = 7, kV_2x4s1 = 8 };

struct Plan {
    int rows, ks, grid, threads, per_wg, bk, lds, variant, n_row_tiles;
    int paired;   // 0: one item per workgroup, heaviest first; 1: tiles i and n-1-i; 2: heavy/light halves
    int splits, split_len;   // key-range splits across workgroups (0: none)
};

// pair < 0: pair tiles i and n-1-i when that still leaves a workgroup per CU;
// otherwise pair iff pair != 0.
template <typename T, int NW, int KS, int ST = 2>
Plan make_plan(int C, int variant, int pair = -1, bool paged = false) {
    using G = Geo<T, NW, KS, ST>;
    Plan p{};
    p.rows = G::kRows;
    p.ks = KS;
    p.threads = G::kThreads;
    p.bk = G::kBK;
    p.lds = G::lds_total(paged);
    p.variant = variant;
    p.n_row_tiles = (C + G::kRows - 1) / G::kRows;
    const int pairs = (p.n_row_tiles + 1) / 2;
    p.paired = pair < 0 ? (pairs * kHKV >= 256 ? 1 : 0) : (pair != 0);
    p.per_wg = p.paired ? 2 : 1;
    p.grid = (p.paired ? pairs : p.n_row_tiles) * kHKV;
    return p;
}

// Makespan estimate for work items of H rows where a CU runs one workgroup at a
// time (every fp32 shape takes 128 KiB of LDS; the 64-row bf16 shape 16 waves).
// An item of H rows over k keys costs H*k/eff + item, eff the shape's measured
// relative efficiency and item the fixed cost of an item (Q load, first tile,
// merge and stores: about 3 us, the time a 32-row fp32 item spends on 52 keys
// and a 64-row bf16 item on 177).  Unpaired workgroups
// are launched heaviest first, so their makespan is about the larger of the
// heaviest item and the mean load per CU; paired ones (tiles i and n-1-i) all
// cost about the same and run in ceil(workgroups/256) rounds.  The mean load is
// what an ideal heaviest-first schedule reaches; pairing wins ties (within 2%):
// fewer workgroups, no scheduling tail (C=2048 P=0: 4% faster).
struct ShapeCost {
    double t;
    int paired;
};
inline ShapeCost shape_cost(int C, int P, int H, double eff, double item) {
    constexpr double kCUs = 256.0;
    const double n = (double)((C + H - 1) / H);
    // keys of tile i: P + min(H(i+1), C); only the last tile is capped
    const double work = (double)H * (n * P + (double)H * (n - 1) * n / 2 + C) / eff;
    const double tu = fmax((double)H * ((double)P + C) / eff + item, (work + n * item) * kHKV / kCUs);
    const double tp = ceil(ceil(n / 2) * kHKV / kCUs) * ((double)H * (2.0 * P + C + H) / eff + 2 * item);
    return tp <= 1.02 * tu ? ShapeCost{tp, 1} : ShapeCost{tu, 0};
}

// fp32 (contiguous or paged): 32, 16 or 8 rows x 4 heads per work item (16-,
// 8- or 4-wave workgroups, 4 key-split waves over 128-key tiles), paired or
// not, whichever the estimate above makes fastest (relative efficiencies 1,
// 0.92, 0.68, measured on balanced grids), unless one of the one-stage rules
// below applies (plain caches: 8- or 16-row items with one staging buffer, two
// workgroups per CU, where measured plan sweeps put them ahead).  Long chunks
// take 32 rows in pairs; a short prompt (P small against C) takes smaller
// items so that causal work evens out over the CUs.  bf16: 64-key tiles over 2 waves, 64 rows per work item (16
// waves) from 4096 rows on, where row tiles still pair into 256 workgroups
// (each staged tile then serves twice the queries: ~3% faster on long
// prefixes, whose K/V exceed the L2), 32 rows (8-wave workgroups, two per CU)
// from 2048 rows or for paged caches, then 16 rows unpaired (C=1024: 7% faster
// than 32 rows at P=0, 13% at P=1024) and 8 rows below 256.
template <typename T>
Plan choose_plan(int C, int P, bool paged) {
    Plan p;
    if constexpr (sizeof(T) == 4) {
        constexpr double kItem = 32.0 * 52.0;
        const ShapeCost c32 = shape_cost(C, P, 32, 1.0, kItem), c16 = shape_cost(C, P, 16, 0.92, kItem),
                        c8 = shape_cost(C, P, 8, 0.68, kItem);
        // One staging buffer with 8-row items, unpaired: two workgroups share a
        // CU (512 slots), each nearly as fast as alone since the other computes
        // while it waits on its loads.  Measured against the two-stage plans
        // it wins where its workgroups (one per 8 rows and KV group) fill one
        // round of the 512 slots, whole rounds, or more than two rounds and
        // most of a third (T=512 +16%; T=1536, C=1500 P=100 +4%; C=384 P=1000
        // +22%; C=1536 P=1536 +10%; T=960, 1.9 rounds: -10%) or where a long
        // prefix makes the items alike so a partial round costs little (C=768
        // P=2000 +17%, C=1100 P=12000 +31%: there the 32-row items take two
        // rounds of 256 workgroups for 280).  It loses with a partial round of
        // causal items (T=768 -11%), near 2048 rows to the 32-row items (C=1900
        // to 2000: -4 to -7%) and on prefixes past 8C where 16- or 32-row
        // items fill exactly the 256 CUs (C=512 P=15872 -3%, C=1024 P=16000
        // -4%).  Paged caches take it in one round (C=512 P=0 and C=384 P=1000
        // 20% faster) and over more rounds only from 1025 rows against
        // prefixes of 8C (C=1100 P=8800 16%, C=1536 P=12288 6% faster; 3-11%
        // slower at C=768 P=2000..12000 and C=1536 P=1536, where each tile's
        // row offsets weigh more); the 16-row one-stage plans below have no
        // LDS left for the offsets and stay plain.
        const int wgs = 8 * ((C + 7) / 8);
        const int rem = wgs % 512;
        const bool exact_fit = 8 * ((C + 31) / 32) == 256 || 8 * ((C + 15) / 16) == 256;
        const bool os16_shape = C >= 880 && C <= 1024 && P <= 4 * C && (C > 960 || P >= C);
        const bool one_stage = !os16_shape && C < 1800 && !(P > 8 * C && exact_fit) &&
                               (wgs <= 512 || (paged ? C > 1024 && P >= 8 * C
                                                     : rem == 0 || (rem >= 440 && wgs > 1024) || P >= C));
        // 16-row items with one staging buffer, two workgroups per CU (four
        // waves per SIMD instead of the two of a 16-row workgroup alone), where
        // they fill the 512 slots in one round: C = 961..1024 (+4-9% over the
        // paired two-stage 16-row items at P = 0..4096; -2% at P = 16384), and
        // C = 880..960 with P >= C (+2-6% over the 8-row one-stage items; at
        // P = 0 the two-stage 16-row items there are 8% faster)
        const bool one_stage16 = !paged && os16_shape;   // paged: the two-stage plans
        // The same 16-row items, unpaired over several rounds of the 512
        // slots, heaviest first: for causal chunks of 1100..1599 rows (T=1400
        // +10%, T=1200 +4%) and from 2048 rows wherever the 32-row items would
        // run unpaired, i.e. could not pair into one round of 256 workgroups
        // (C=2560 P=1000 +12%, C=2100 P=12000 +13%, T=2300 +5%).
        const bool c32_unpaired = c32.t <= c16.t && c32.t <= c8.t && !c32.paired;
        const bool one_stage16u = !paged && !one_stage16 && !one_stage &&
                                  ((C >= 1100 && C < 1600 && P < C) || (C >= 2048 && c32_unpaired));
        if (one_stage16) p = make_plan<T, 2, 4, 1>(C, kV_2x4s1, 0);
        else if (one_stage) p = make_plan<T, 1, 4, 1>(C, kV_1x4s1, 0, paged);
        else if (one_stage16u) p = make_plan<T, 2, 4, 1>(C, kV_2x4s1, 0);
        else if (c32.t <= c16.t && c32.t <= c8.t) p = make_plan<T, 4, 4>(C, kV_4x4, c32.paired, paged);
        else if (c16.t <= c8.t) p = make_plan<T, 2, 4>(C, kV_2x4, c16.paired, paged);
        else p = make_plan<T, 1, 4>(C, kV_1x4, c8.paired, paged);
    } else {
        // two (4,2) or (2,4) workgroups fit a CU, so pairing their items into
        // 256 workgroups would leave half the slots empty: they stay unpaired
        // (C=2048 P=2048: 69.1 -> 62.5 us, P=500: 39.8 -> 36.9 us against
        // paired (4,2) items, with the heavy/light placement below)
        // 32-row items also for 1025..2047 rows against long prefixes, where
        // 16-row ones would take more than one round of 512 workgroups (C=1100
        // P=12000 6%, C=1536 P=1536 4%, C=1800 P=3000 8%, C=2000 P=2000 8%
        // faster; at C=1100..1200 P=C and at P=0 the 16-row items stay 11-13%
        // ahead)
        p = C >= 2048 || (C > 1024 && (P >= 4 * C || (C >= 1400 && P >= C)))
                ? (C >= 4096 ? make_plan<T, 8, 2>(C, kV_8x2, shape_cost(C, P, 64, 1.0, 64.0 * 177.0).paired, paged)
                             : make_plan<T, 4, 2>(C, kV_4x2, 0, paged))
            : C >= 256 ? make_plan<T, 2, 4>(C, kV_2x4, 0, paged)
                       : make_plan<T, 1, 4>(C, kV_1x4, -1, paged);
    }
    // Unpaired plans that run two workgroups per CU (fp32 with one staging
    // buffer, every bf16 shape but the 64-row one) and fit in one round of
    // 512 resident workgroups: heavy and light tiles side by side on each CU
    // (T=512 fp32 +7%, C=1024 P=0 bf16 +8%, P=1024 +3.5%); over several
    // rounds the heaviest-first order does better (T=1536 fp32: -6%).
    const bool two_per_cu = sizeof(T) == 4 ? (p.variant == kV_1x4s1 || p.variant == kV_2x4s1) : p.variant != kV_8x2;
    if (!p.paired && two_per_cu && p.grid <= 2 * 256) p.paired = 2;
    return p;
}

Plan plan_for(int C, int P, attn_dtype_t dtype, bool paged) {
    return dtype == ATTN_DTYPE_BF16 ? choose_plan<__bf16>(C, P, paged) : choose_plan<float>(C, P, paged);
}

template <typename T, int NW, int KS, int MODE, int ST = 2>
hipError_t launch(const Plan& p, const void* q, const void* k, const void* v, float* out, int C, int P,
                  PagedCache pg, KeySplit ksp, unsigned long long* clk, hipStream_t stream) {
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    int n_row_tiles = p.n_row_tiles, paired = p.paired;
    void* args[] = {&qq, &kk, &vv, &out, &C, &P, &n_row_tiles, &paired, &pg, &ksp, &clk};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_prefill_kernel<T, NW, KS, MODE, ST>), dim3(p.grid),
                           dim3(p.threads), args, 0, stream);
}

template <typename T, int MODE>
hipError_t dispatch(const Plan& p, const void* q, const void* k, const void* v, float* out, int C, int P,
                    PagedCache pg, KeySplit ksp, hipStream_t stream, unsigned long long* clk = nullptr) {
    switch (p.variant) {
        case kV_4x2:
            if constexpr ((MODE & kSplit) != 0) return hipErrorInvalidValue;   // never planned
            else return launch<T, 4, 2, MODE>(p, q, k, v, out, C, P, pg, ksp, clk, stream);
        case kV_2x4: return launch<T, 2, 4, MODE>(p, q, k, v, out, C, P, pg, ksp, clk, stream);
        case kV_1x4s1:   // planned for fp32 only, never with key splits
            if constexpr ((MODE & kSplit) != 0 || sizeof(T) != 4) return hipErrorInvalidValue;
            else return launch<T, 1, 4, MODE, 1>(p, q, k, v, out, C, P, pg, ksp, clk, stream);
        case kV_2x4s1:   // planned for fp32 plain caches only
            if constexpr (MODE != kPlain || sizeof(T) != 4) return hipErrorInvalidValue;
            else return launch<T, 2, 4, MODE, 1>(p, q, k, v, out, C, P, pg, ksp, clk, stream);
        case kV_8x2:   // planned for bf16 only, never with key splits
            if constexpr ((MODE & kSplit) != 0 || sizeof(T) != 2) return hipErrorInvalidValue;
            else return launch<T, 8, 2, MODE>(p, q, k, v, out, C, P, pg, ksp, clk, stream);
        case kV_4x4:   // planned for fp32 only, never with key splits
            if constexpr ((MODE & kSplit) != 0 || sizeof(T) != 4) return hipErrorInvalidValue;
            else return launch<T, 4, 4, MODE>(p, q, k, v, out, C, P, pg, ksp, clk, stream);
        default: return launch<T, 1, 4, MODE>(p, q, k, v, out, C, P, pg, ksp, clk, stream);
    }
}

// Key splits for the workspace variant: about one workgroup per CU (row tiles
// x KV groups x splits >= 256; measured faster than 512 or 1024 because each
// split then streams more tiles), each split at least two staged tiles long;
// split length a multiple of the staged tile.
Plan split_plan(int C, int P, attn_dtype_t dtype) {
    if (C == 1 && dtype == ATTN_DTYPE_F32) {
        // one fp32 token: the FMA decode kernel, splits of a multiple of 64
        // keys, at most 32 of them (up to 256 four-wave workgroups; measured
        // faster than 16, 24, 64 or 128 at 16384 keys).  bf16 stays on the MFMA
        // kernel below: with twice the keys per byte the FMA work is no longer
        // hidden behind the loads, and bf16 MFMAs are cheap enough.
        Plan p{};
        const long long total = (long long)P + 1;   // sums below in 64 bits: P may be near INT_MAX
        const int len = (int)max(64LL, ((total + 31) / 32 + 63) / 64 * 64);
        p.rows = 1;
        p.ks = kDecWaves;
        p.threads = 64 * kDecWaves;
        p.bk = 8;
        p.lds = kDecWaves * 4 * (kD + 2) * 4;
        p.variant = kV_decode;
        p.n_row_tiles = 1;
        p.per_wg = 1;
        p.split_len = len;
        p.splits = (int)((total + len - 1) / len);
        p.grid = kHKV * p.splits;
        return p;
    }
    // short chunks: 8-row work items; longer ones: 16 rows (both 4 key-split waves)
    Plan p = C < 256 ? (dtype == ATTN_DTYPE_BF16 ? make_plan<__bf16, 1, 4>(C, kV_1x4) : make_plan<float, 1, 4>(C, kV_1x4))
                     : (dtype == ATTN_DTYPE_BF16 ? make_plan<__bf16, 2, 4>(C, kV_2x4) : make_plan<float, 2, 4>(C, kV_2x4));
    p.paired = 0;
    p.per_wg = 1;
    const long long total = (long long)P + C;   // sums below in 64 bits: P + C may be near INT_MAX
    const int base = p.n_row_tiles * kHKV;
    constexpr int kTargetWorkgroups = 256;
    const long long most = (total + 2 * p.bk - 1) / (2 * p.bk);
    const long long s = max(1LL, min((long long)(kTargetWorkgroups + base - 1) / base, most));
    const long long len = ((total + s - 1) / s + p.bk - 1) / p.bk * p.bk;
    p.splits = (int)((total + len - 1) / len);
    p.split_len = len;
    p.grid = base * p.splits;
    return p;
}

size_t split_workspace_bytes(const Plan& p, int C) {
    return (size_t)p.splits * C * kHQ * (kD + 2) * sizeof(float);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

attn_status_t scratch_address(hipStream_t stream, void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
    // the kernels run on the stream's device: it must be the current one,
    // whose copy of the array is the one looked up here
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (sdev != dev) return ATTN_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_LAUNCH;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return ATTN_OK;
}

// The two kernels of a split-KV call: split partials into `part`, then merge
// them into `out`.  pg.table == nullptr: contiguous cache; otherwise kCache and
// vCache are page pools read through pg.  Arguments are already checked.
attn_status_t launch_splitkv(const Plan& p, const void* q, const void* kCache, const void* vCache, float* out,
                             int C, int P, attn_dtype_t dtype, float* part, PagedCache pg, hipStream_t stream) {
    const bool paged = pg.table != nullptr;
    const KeySplit ksp{part, p.split_len, p.splits};
    int len = p.split_len, n = p.splits;
    hipError_t e;
    if (p.variant == kV_decode) {
        void* dargs[] = {const_cast<void**>(&q), const_cast<void**>(&kCache), const_cast<void**>(&vCache), &part, &P,
                         &len, &n, &pg};
        const void* fn = paged ? reinterpret_cast<const void*>(&attn_decode_split_kernel<true>)
                               : reinterpret_cast<const void*>(&attn_decode_split_kernel<false>);
        e = hipLaunchKernel(fn, dim3(p.grid), dim3(p.threads), dargs, 0, stream);
    } else if (paged) {
        e = dtype == ATTN_DTYPE_BF16
                ? dispatch<__bf16, kPagedSplit>(p, q, kCache, vCache, out, C, P, pg, ksp, stream)
                : dispatch<float, kPagedSplit>(p, q, kCache, vCache, out, C, P, pg, ksp, stream);
    } else {
        e = dtype == ATTN_DTYPE_BF16 ? dispatch<__bf16, kSplit>(p, q, kCache, vCache, out, C, P, pg, ksp, stream)
                                     : dispatch<float, kSplit>(p, q, kCache, vCache, out, C, P, pg, ksp, stream);
    }
    if (e != hipSuccess) return ATTN_ERR_LAUNCH;
    const float* pc = part;
    void* args[] = {&pc, &out, &C, &P, &len, &n};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_merge_splits_kernel), dim3((C * kHQ + 3) / 4),
                        dim3(256), args, 0, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

// Chunk and cache sizes the launch arithmetic is planned for: row, tile, split
// and grid counts, key offsets plus a split's length, and the planner's
// comparisons stay within int (the merge kernel's (row, head) count
// C * 32 among them).  The q and output rows of a chunk past kMaxChunkRows
// (at least 12 KiB per row), or the K/V of a cache past kMaxPositions (at
// least 2 KiB per position), would exceed a GPU's memory.
constexpr int kMaxChunkRows = 1 << 25;
constexpr int kMaxPositions = 1 << 30;
static bool sizes_ok(int C, int P) {
    return C >= 0 && C <= kMaxChunkRows && P >= 0 && P <= kMaxPositions - C;
}

extern "C" {

attn_status_t attn_prefill_validate(const void* q, const void* kCache, const void* vCache, const float* out,
                                    int C, int P, attn_dtype_t dtype) {
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (!sizes_ok(C, P)) return ATTN_ERR_INVALID_ARG;
    if (C == 0) return ATTN_OK;
    if (!q || !kCache || !vCache || !out) return ATTN_ERR_NULL_PTR;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kCache) |
                          reinterpret_cast<uintptr_t>(vCache) | reinterpret_cast<uintptr_t>(out);
    if (mis & 15u) return ATTN_ERR_MISALIGNED;
    const size_t esz = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
    const size_t nq = (size_t)C * kHQ * kD, nkv = ((size_t)P + C) * kHKV * kD;
    const size_t out_bytes = nq * 4;
    if (overlaps(out, out_bytes, q, nq * esz) || overlaps(out, out_bytes, kCache, nkv * esz) ||
        overlaps(out, out_bytes, vCache, nkv * esz))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn_status_t attn_prefill_plan(int C, int P, attn_dtype_t dtype, int paged, int* plan) {
    if (!plan) return ATTN_ERR_NULL_PTR;
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (!sizes_ok(C, P)) return ATTN_ERR_INVALID_ARG;
    const Plan p = plan_for(C > 0 ? C : 1, P, dtype, paged != 0);
    plan[0] = p.rows;
    plan[1] = p.ks;
    plan[2] = C > 0 ? p.grid : 0;
    plan[3] = p.threads;
    plan[4] = p.per_wg;
    plan[5] = p.bk;
    plan[6] = p.lds;
    plan[7] = p.variant;
    return ATTN_OK;
}

attn_status_t attn_prefill(const void* q, const void* kCache, const void* vCache, float* out, int C, int P,
                           attn_dtype_t dtype, hipStream_t stream) {
    const attn_status_t st = attn_prefill_validate(q, kCache, vCache, out, C, P, dtype);
    if (st != ATTN_OK || C == 0) return st;
    const Plan p = plan_for(C, P, dtype, false);
    const PagedCache none = make_paged(nullptr, 1, 0);
    const KeySplit nosplit{nullptr, 0, 0};
    const hipError_t e = dtype == ATTN_DTYPE_BF16
                             ? dispatch<__bf16, kPlain>(p, q, kCache, vCache, out, C, P, none, nosplit, stream)
                             : dispatch<float, kPlain>(p, q, kCache, vCache, out, C, P, none, nosplit, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_prefill_clocked(const void* q, const void* kCache, const void* vCache, float* out, int C, int P,
                                   attn_dtype_t dtype, unsigned long long* clocks, size_t clockCount,
                                   hipStream_t stream) {
    const attn_status_t st = attn_prefill_validate(q, kCache, vCache, out, C, P, dtype);
    if (st != ATTN_OK || C == 0) return st;
    const Plan p = plan_for(C, P, dtype, false);
    if (!clocks) return ATTN_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(clocks) & 7u) return ATTN_ERR_MISALIGNED;
    if (clockCount < kClockWords * (size_t)p.grid) return ATTN_ERR_WORKSPACE;
    const size_t esz = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
    const size_t nq = (size_t)C * kHQ * kD, nkv = ((size_t)P + C) * kHKV * kD, nc = 8 * kClockWords * (size_t)p.grid;
    if (overlaps(clocks, nc, q, nq * esz) || overlaps(clocks, nc, kCache, nkv * esz) ||
        overlaps(clocks, nc, vCache, nkv * esz) || overlaps(clocks, nc, out, nq * 4))
        return ATTN_ERR_ALIAS;
    const PagedCache none = make_paged(nullptr, 1, 0);
    const KeySplit nosplit{nullptr, 0, 0};
    const hipError_t e = dtype == ATTN_DTYPE_BF16
                             ? dispatch<__bf16, kPlain>(p, q, kCache, vCache, out, C, P, none, nosplit, stream, clocks)
                             : dispatch<float, kPlain>(p, q, kCache, vCache, out, C, P, none, nosplit, stream, clocks);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_prefill_splitkv_workspace(int C, int P, attn_dtype_t dtype, size_t* bytes, int* splits) {
    if (!bytes) return ATTN_ERR_NULL_PTR;
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (!sizes_ok(C, P)) return ATTN_ERR_INVALID_ARG;
    if (C == 0) {
        *bytes = 0;
        if (splits) *splits = 0;
        return ATTN_OK;
    }
    const Plan p = split_plan(C, P, dtype);
    *bytes = split_workspace_bytes(p, C);
    if (splits) *splits = p.splits;
    return ATTN_OK;
}

attn_status_t attn_prefill_splitkv(const void* q, const void* kCache, const void* vCache, float* out, int C, int P,
                                   attn_dtype_t dtype, void* workspace, size_t workspaceBytes,
                                   hipStream_t stream) {
    const attn_status_t st = attn_prefill_validate(q, kCache, vCache, out, C, P, dtype);
    if (st != ATTN_OK || C == 0) return st;
    const Plan p = split_plan(C, P, dtype);
    const size_t need = split_workspace_bytes(p, C);
    if (!workspace) return ATTN_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return ATTN_ERR_MISALIGNED;
    if (workspaceBytes < need) return ATTN_ERR_WORKSPACE;
    const size_t esz = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
    const size_t nq = (size_t)C * kHQ * kD, nkv = ((size_t)P + C) * kHKV * kD;
    if (overlaps(workspace, need, q, nq * esz) || overlaps(workspace, need, kCache, nkv * esz) ||
        overlaps(workspace, need, vCache, nkv * esz) || overlaps(workspace, need, out, nq * 4))
        return ATTN_ERR_ALIAS;
    return launch_splitkv(p, q, kCache, vCache, out, C, P, dtype, static_cast<float*>(workspace),
                          make_paged(nullptr, 1, 0), stream);
}

attn_status_t attn_prefill_splitkv_noalloc(const void* q, const void* kCache, const void* vCache, float* out,
                                           int C, int P, attn_dtype_t dtype, hipStream_t stream) {
    const attn_status_t st = attn_prefill_validate(q, kCache, vCache, out, C, P, dtype);
    if (st != ATTN_OK || C == 0) return st;
    const Plan p = split_plan(C, P, dtype);
    if (split_workspace_bytes(p, C) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_TOO_LARGE;
    void* ws = nullptr;
    const attn_status_t sa = scratch_address(stream, &ws);
    if (sa != ATTN_OK) return sa;
    return launch_splitkv(p, q, kCache, vCache, out, C, P, dtype, static_cast<float*>(ws), make_paged(nullptr, 1, 0),
                          stream);
}

attn_status_t attn_naive_workspace(int T, size_t* bytes) {
    if (!bytes) return ATTN_ERR_NULL_PTR;
    if (T < 0 || T > 46340) return ATTN_ERR_INVALID_ARG;       // T*T fits int
    *bytes = (size_t)kHQ * T * T * sizeof(float);
    return ATTN_OK;
}

attn_status_t attn_naive(const float* q, const float* k, const float* v, float* out, int T, void* workspace,
                         size_t workspaceBytes, hipStream_t stream) {
    if (T < 0 || T > 46340) return ATTN_ERR_INVALID_ARG;
    const attn_status_t st = attn_prefill_validate(q, k, v, out, T, 0, ATTN_DTYPE_F32);
    if (st != ATTN_OK || T == 0) return st;
    const size_t need = (size_t)kHQ * T * T * sizeof(float);
    if (!workspace) return ATTN_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return ATTN_ERR_MISALIGNED;
    if (workspaceBytes < need) return ATTN_ERR_WORKSPACE;
    const size_t nq = (size_t)T * kHQ * kD * 4, nkv = (size_t)T * kHKV * kD * 4;
    if (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nkv) || overlaps(workspace, need, v, nkv) ||
        overlaps(workspace, need, out, nq))
        return ATTN_ERR_ALIAS;
    float* S = static_cast<float*>(workspace);
    const int nt = (T + kNT - 1) / kNT;
    {
        void* args[] = {&q, &k, &S, &T};
        if (hipLaunchKernel(reinterpret_cast<const void*>(&naive_scores_kernel), dim3(nt, nt, kHQ), dim3(256), args,
                            0, stream) != hipSuccess)
            return ATTN_ERR_LAUNCH;
    }
    {
        void* args[] = {&S, &T};
        if (hipLaunchKernel(reinterpret_cast<const void*>(&naive_softmax_kernel), dim3(T, kHQ), dim3(256), args, 0,
                            stream) != hipSuccess)
            return ATTN_ERR_LAUNCH;
    }
    {
        const float* Sc = S;
        void* args[] = {&Sc, &v, &out, &T};
        if (hipLaunchKernel(reinterpret_cast<const void*>(&naive_pv_kernel), dim3(nt, kHQ), dim3(256), args, 0,
                            stream) != hipSuccess)
            return ATTN_ERR_LAUNCH;
    }
    return ATTN_OK;
}

attn_status_t attn_prefill_rowwise(const void* q, const void* kCache, const void* vCache, float* out, int C, int P,
                                   attn_dtype_t dtype, hipStream_t stream) {
    const attn_status_t st = attn_prefill_validate(q, kCache, vCache, out, C, P, dtype);
    if (st != ATTN_OK || C == 0) return st;
    const dim3 grid((C + kRowWaves - 1) / kRowWaves, kHQ);
    hipError_t e;
    if (dtype == ATTN_DTYPE_BF16) {
        const __bf16 *qq = static_cast<const __bf16*>(q), *kk = static_cast<const __bf16*>(kCache),
                     *vv = static_cast<const __bf16*>(vCache);
        void* args[] = {&qq, &kk, &vv, &out, &C, &P};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_rowwise_kernel<__bf16>), grid, dim3(64 * kRowWaves),
                            args, 0,
                            stream);
    } else {
        const float *qq = static_cast<const float*>(q), *kk = static_cast<const float*>(kCache),
                    *vv = static_cast<const float*>(vCache);
        void* args[] = {&qq, &kk, &vv, &out, &C, &P};
        e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_rowwise_kernel<float>), grid, dim3(64 * kRowWaves),
                            args, 0,
                            stream);
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_prefill_paged_validate(const void* q, const void* kPages, const void* vPages,
                                          const int* blockTable, int numBlocks, int pageSize, const float* out,
                                          int C, int P, attn_dtype_t dtype) {
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (!sizes_ok(C, P) || pageSize <= 0 || numBlocks <= 0) return ATTN_ERR_INVALID_ARG;
    const size_t esz = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
    const size_t pool = (size_t)numBlocks * (size_t)pageSize * kHKV * kD * esz;
    if (pool > 0xFFFFFFFFull) return ATTN_ERR_INVALID_ARG;     // page pool addressed with 32-bit offsets
    if (C == 0) return ATTN_OK;
    if (!q || !kPages || !vPages || !blockTable || !out) return ATTN_ERR_NULL_PTR;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kPages) |
                          reinterpret_cast<uintptr_t>(vPages) | reinterpret_cast<uintptr_t>(out);
    if ((mis & 15u) || (reinterpret_cast<uintptr_t>(blockTable) & 3u)) return ATTN_ERR_MISALIGNED;
    const size_t nq = (size_t)C * kHQ * kD, out_bytes = nq * 4;
    const size_t ntab = ((size_t)P + C + pageSize - 1) / pageSize;
    if (ntab * 4 > 0xFFFFFFFFull) return ATTN_ERR_INVALID_ARG;   // table addressed with 32-bit offsets
    if (overlaps(out, out_bytes, q, nq * esz) || overlaps(out, out_bytes, kPages, pool) ||
        overlaps(out, out_bytes, vPages, pool) || overlaps(out, out_bytes, blockTable, ntab * 4))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn_status_t attn_prefill_paged(const void* q, const void* kPages, const void* vPages, const int* blockTable,
                                 int numBlocks, int pageSize, float* out, int C, int P, attn_dtype_t dtype,
                                 hipStream_t stream) {
    const attn_status_t st =
        attn_prefill_paged_validate(q, kPages, vPages, blockTable, numBlocks, pageSize, out, C, P, dtype);
    if (st != ATTN_OK || C == 0) return st;
    const Plan p = plan_for(C, P, dtype, true);
    const PagedCache pg = make_paged(blockTable, pageSize, numBlocks);
    const KeySplit nosplit{nullptr, 0, 0};
    const hipError_t e = dtype == ATTN_DTYPE_BF16
                             ? dispatch<__bf16, kPaged>(p, q, kPages, vPages, out, C, P, pg, nosplit, stream)
                             : dispatch<float, kPaged>(p, q, kPages, vPages, out, C, P, pg, nosplit, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_prefill_paged_splitkv(const void* q, const void* kPages, const void* vPages,
                                         const int* blockTable, int numBlocks, int pageSize, float* out, int C, int P,
                                         attn_dtype_t dtype, void* workspace, size_t workspaceBytes,
                                         hipStream_t stream) {
    const attn_status_t st =
        attn_prefill_paged_validate(q, kPages, vPages, blockTable, numBlocks, pageSize, out, C, P, dtype);
    if (st != ATTN_OK || C == 0) return st;
    const Plan p = split_plan(C, P, dtype);
    const size_t need = split_workspace_bytes(p, C);
    if (!workspace) return ATTN_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return ATTN_ERR_MISALIGNED;
    if (workspaceBytes < need) return ATTN_ERR_WORKSPACE;
    const size_t esz = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
    const size_t nq = (size_t)C * kHQ * kD;
    const size_t pool = (size_t)numBlocks * (size_t)pageSize * kHKV * kD * esz;
    const size_t ntab = ((size_t)P + C + pageSize - 1) / pageSize;
    if (overlaps(workspace, need, q, nq * esz) || overlaps(workspace, need, kPages, pool) ||
        overlaps(workspace, need, vPages, pool) || overlaps(workspace, need, blockTable, ntab * 4) ||
        overlaps(workspace, need, out, nq * 4))
        return ATTN_ERR_ALIAS;
    return launch_splitkv(p, q, kPages, vPages, out, C, P, dtype, static_cast<float*>(workspace),
                          make_paged(blockTable, pageSize, numBlocks), stream);
}

const char* attn_status_string(attn_status_t s) {
    switch (s) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
        case ATTN_ERR_NULL_PTR: return "ATTN_ERR_NULL_PTR";
        case ATTN_ERR_UNSUPPORTED_DTYPE: return "ATTN_ERR_UNSUPPORTED_DTYPE";
        case ATTN_ERR_MISALIGNED: return "ATTN_ERR_MISALIGNED";
        case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
        case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS";
        case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
        case ATTN_ERR_TOO_LARGE: return "ATTN_ERR_TOO_LARGE";
    }
    return "ATTN_ERR_UNKNOWN";
}

int attn_prefill_version(void) { return 200; }

}  // extern "C"
