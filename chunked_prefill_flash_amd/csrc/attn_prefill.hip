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
// * K/V tiles are staged in LDS with padded rows so the MFMA operand reads are
//   free of bank conflicts; the next tile's global loads are issued before the
//   current tile's math and written to the other LDS buffer after it.
// * A workgroup is NW row-waves x KS key-split waves.  Key-split waves take
//   alternate 32-key sub-blocks of each tile and are merged once at the end
//   with the log-sum-exp rule ("FlashAttention and inference kernels",
//   Flash-Decoding section and Exercises, exercise 2), skipping empty splits.
// * blockIdx.x % 8 selects the KV group: consecutive workgroups go to the 8
//   XCDs round-robin, so every XCD's L2 holds the K/V of one group only.
// * Rows tiles i and n-1-i can be paired in one workgroup so every workgroup
//   does the same causal work.
// * exp is evaluated as exp2 with log2(e)/8 folded in (into Q for fp32, into an
//   FMA for bf16).  The running maximum is only moved when a tile's maximum
//   exceeds it by more than 2^8 (log2 units); any reference value gives the
//   same softmax because it cancels in O/l, and p stays <= 256.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

#include "attn_prefill.h"

namespace {

constexpr int kHQ = ATTN_NUM_Q_HEADS;   // 32
constexpr int kHKV = ATTN_NUM_KV_HEADS; // 8
constexpr int kD = ATTN_HEAD_DIM;       // 64
constexpr int kGroup = kHQ / kHKV;      // 4

// log2(e) / 8: scores become base-2 exponents with the 1/8 scale applied.
constexpr float kScaleLog2 = 0.18033688011112042f;
// Move the running maximum only when a tile raises it by more than this many
// powers of two.
constexpr float kRescaleSlack = 8.0f;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
};
template <> struct Elem<__bf16> {
    static constexpr int kBytes = 2;
};

// Tile geometry for a workgroup of NW row-waves x KS key-split waves.
template <typename T, int NW, int KS>
struct Geo {
    static constexpr int kNB = KS > 2 ? KS : 2;      // 32-key sub-blocks per staged tile
    static constexpr int kBK = 32 * kNB;             // keys per staged tile
    static constexpr int kThreads = 64 * NW * KS;
    static constexpr int kRows = 8 * NW;             // chunk rows per work item
    static constexpr int kElemsPerChunk = 16 / Elem<T>::kBytes;   // 16-byte global loads
    static constexpr int kChunksPerRow = kD / kElemsPerChunk;
    static constexpr int kChunks = kBK * kChunksPerRow / kThreads; // per tensor per thread
    static_assert(kBK * kChunksPerRow % kThreads == 0, "tile load must divide evenly");
    // LDS layout, in elements of T.
    //  fp32: K[BK][68] and V[BK][68], both key-major (row padding of 16 B).
    //  bf16: K[BK][72] key-major (padding 16 B) and V^T[64][BK+4] dim-major
    //        (padding 8 B), so a lane's eight PV operands are two 8-byte reads.
    static constexpr int kKStride = kD + 16 / Elem<T>::kBytes;
    static constexpr bool kVT = sizeof(T) == 2;
    static constexpr int kVStride = kVT ? kBK + 4 : kD + 4;
    static constexpr int kKElems = kBK * kKStride;
    static constexpr int kVElems = kVT ? kD * kVStride : kBK * kVStride;
    static constexpr int kStageBytes = (kKElems + kVElems) * Elem<T>::kBytes;
    // Merge buffer for key splits: per (row-wave, split>0) wave, 34 floats/lane.
    static constexpr int kMergeBytes = KS > 1 ? NW * (KS - 1) * 34 * 64 * 4 : 0;
    static constexpr int kLdsBytes =
        2 * kStageBytes > kMergeBytes ? 2 * kStageBytes : kMergeBytes;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xchg_half(float x) {
    // value of the lane 32 positions away (the other half-wave)
    return __shfl_xor(x, 32, 64);
}

// ---------------------------------------------------------------------------
// The kernel.  One workgroup = one KV group g and one or two row tiles.
// ---------------------------------------------------------------------------
template <typename T, int NW, int KS>
__global__ void __launch_bounds__(64 * NW * KS)
attn_prefill_kernel(const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
                    float* __restrict__ out, int C, int P, int n_row_tiles, int paired) {
    using G = Geo<T, NW, KS>;
    constexpr int kBK = G::kBK, kNB = G::kNB, kThreads = G::kThreads, kRows = G::kRows;
    constexpr int kEPC = G::kElemsPerChunk, kCPR = G::kChunksPerRow, kCH = G::kChunks;
    constexpr bool kF32 = sizeof(T) == 4;

    __shared__ __attribute__((aligned(16))) unsigned char lds_raw[G::kLdsBytes];
    T* const stage0 = reinterpret_cast<T*>(lds_raw);
    T* const stage1 = reinterpret_cast<T*>(lds_raw + G::kStageBytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wr = wid % NW;   // row sub-tile of this wave
    const int wp = wid / NW;   // key split of this wave
    const int n = lane & 31;   // query slot
    const int hh = lane >> 5;  // half-wave
    const int g = blockIdx.x % kHKV;
    const int slot = blockIdx.x / kHKV;
    const int total = P + C;   // cache positions

    int items[2];
    int nitems = 1;
    if (paired) {
        items[0] = n_row_tiles - 1 - slot;  // the heavier tile first
        items[1] = slot;
        nitems = items[1] != items[0] ? 2 : 1;
    } else {
        items[0] = n_row_tiles - 1 - slot;  // heaviest tiles are launched first
        items[1] = items[0];
    }

    for (int it = 0; it < nitems; ++it) {
        const int tile = items[it];
        const int i0 = tile * kRows;
        const int i0w = i0 + 8 * wr;
        const int rows_end = min(i0 + kRows, C);
        const int kv_end = P + rows_end;
        const int ntiles = (kv_end + kBK - 1) / kBK;
        const bool wave_active = i0w < C;
        const int w_first = P + i0w;                // visible limit of the wave's first row
        const int w_last = P + min(i0w + 7, C - 1); // visible limit of its last valid row
        const int row = i0w + (n >> 2);
        const int head = g * kGroup + (n & 3);
        const int lim = P + row;                    // this lane's query sees keys <= lim

        // ---- Q operand (B of S^T = K Q^T), held for the whole key loop ----
        // fp32: qf[s] = q[row][head][32*hh + s] * log2(e)/8, s = 0..31
        // bf16: qb[s] = q[row][head][16*s + 8*hh .. +7], s = 0..3
        float qf[kF32 ? 32 : 1];
        bf8 qb[kF32 ? 1 : 4];
        if constexpr (kF32) {
            const float* src = reinterpret_cast<const float*>(q) + ((size_t)row * kHQ + head) * kD + 32 * hh;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                f4 x = row < C ? *reinterpret_cast<const f4*>(src + 4 * c) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) qf[4 * c + e] = x[e] * kScaleLog2;
            }
        } else {
            const uint16_t* src = reinterpret_cast<const uint16_t*>(q) + ((size_t)row * kHQ + head) * kD + 8 * hh;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                u16x8 x = row < C ? *reinterpret_cast<const u16x8*>(src + 16 * s) : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                qb[s] = __builtin_bit_cast(bf8, x);
            }
        }

        f16v o0 = {}, o1 = {};   // O^T for dims 0..31 and 32..63
        float m = -INFINITY;     // running max (log2 units)
        float l = 0.f;           // this lane's share of the running denominator

        // ---- K/V tile staging: global -> registers -> LDS ----
        f4 kreg[kCH], vreg[kCH];
        auto load_tile = [&](int t) {
#pragma unroll
            for (int u = 0; u < kCH; ++u) {
                const int c = tid + u * kThreads;
                const int key = t * kBK + c / kCPR;
                const int col = (c % kCPR) * kEPC;
                if (key < total) {
                    const size_t off = ((size_t)key * kHKV + g) * kD + col;
                    kreg[u] = *reinterpret_cast<const f4*>(kc + off);
                    vreg[u] = *reinterpret_cast<const f4*>(vc + off);
                } else {
                    kreg[u] = f4{0.f, 0.f, 0.f, 0.f};
                    vreg[u] = f4{0.f, 0.f, 0.f, 0.f};
                }
            }
        };
        auto store_tile = [&](T* stage) {
            T* Ks = stage;
            T* Vs = stage + G::kKElems;
#pragma unroll
            for (int u = 0; u < kCH; ++u) {
                const int c = tid + u * kThreads;
                const int key = c / kCPR;
                const int col = (c % kCPR) * kEPC;
                *reinterpret_cast<f4*>(Ks + key * G::kKStride + col) = kreg[u];
                if constexpr (!G::kVT) {
                    *reinterpret_cast<f4*>(Vs + key * G::kVStride + col) = vreg[u];
                } else {
                    const u16x8 x = __builtin_bit_cast(u16x8, vreg[u]);
                    uint16_t* vt = reinterpret_cast<uint16_t*>(Vs);
#pragma unroll
                    for (int e = 0; e < 8; ++e) vt[(col + e) * G::kVStride + key] = x[e];
                }
            }
        };

        // ---- one 32-key sub-block: scores, mask, online softmax, PV ----
        auto sub_block = [&](const T* stage, int sb, int jb) {
            const T* Ks = stage;
            const T* Vs = stage + G::kKElems;
            f16v s = {};
            if constexpr (kF32) {
                const float* kr = reinterpret_cast<const float*>(Ks) + (32 * sb + n) * G::kKStride + 32 * hh;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const f4 kx = *reinterpret_cast<const f4*>(kr + 4 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kx[e], qf[4 * c + e], s, 0, 0, 0);
                }
            } else {
                const uint16_t* kr = reinterpret_cast<const uint16_t*>(Ks) + (32 * sb + n) * G::kKStride + 8 * hh;
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const bf8 kx = __builtin_bit_cast(bf8, *reinterpret_cast<const u16x8*>(kr + 16 * st));
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx, qb[st], s, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] *= kScaleLog2;
            }
            // causal mask, only where the sub-block crosses the wave's first row edge
            if (jb + 31 > w_first) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = jb + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key > lim) s[r] = -INFINITY;
                }
            }
            float bm = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) bm = fmaxf(bm, s[r]);
            bm = fmaxf(bm, xchg_half(bm));
            const bool upd = bm > m + kRescaleSlack;
            if (__ballot(upd)) {
                const float alpha = upd ? fast_exp2(m - bm) : 1.0f;
                if (upd) m = bm;
                l *= alpha;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    o0[r] *= alpha;
                    o1[r] *= alpha;
                }
            }
            const float mu = m == -INFINITY ? 0.f : m;
            float p[16];
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = fast_exp2(s[r] - mu);
                ps += p[r];
            }
            l += ps;
            if constexpr (kF32) {
                const float* vr = reinterpret_cast<const float*>(Vs) + (32 * sb) * G::kVStride + n;
#pragma unroll
                for (int t4 = 0; t4 < 16; ++t4) {
                    const int key = 8 * (t4 >> 2) + 4 * hh + (t4 & 3);
                    const float v0 = vr[key * G::kVStride];
                    const float v1 = vr[key * G::kVStride + 32];
                    o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(v0, p[t4], o0, 0, 0, 0);
                    o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(v1, p[t4], o1, 0, 0, 0);
                }
            } else {
                const uint16_t* vt = reinterpret_cast<const uint16_t*>(Vs);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    bf8 pb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pb[e] = (__bf16)p[8 * u + e];
                    const int kofs = 32 * sb + 16 * u + 4 * hh;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const uint16_t* vrow = vt + (32 * nt + n) * G::kVStride + kofs;
                        const uint64_t lo = *reinterpret_cast<const uint64_t*>(vrow);
                        const uint64_t hi = *reinterpret_cast<const uint64_t*>(vrow + 8);
                        const bf4 a0 = __builtin_bit_cast(bf4, lo);
                        const bf4 a1 = __builtin_bit_cast(bf4, hi);
                        const bf8 va = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
                        if (nt == 0)
                            o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o0, 0, 0, 0);
                        else
                            o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o1, 0, 0, 0);
                    }
                }
            }
        };

        // ---- key loop over staged tiles (double-buffered) ----
        load_tile(0);
        store_tile(stage0);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            T* cur = (t & 1) ? stage1 : stage0;
            T* nxt = (t & 1) ? stage0 : stage1;
            const bool more = t + 1 < ntiles;
            if (more) load_tile(t + 1);
            if (wave_active) {
#pragma unroll
                for (int sb = wp; sb < kNB; sb += KS) {
                    const int jb = t * kBK + 32 * sb;
                    if (jb <= w_last) sub_block(cur, sb, jb);
                }
            }
            if (more) store_tile(nxt);
            __syncthreads();
        }

        // ---- merge key splits (log-sum-exp), in LDS ----
        if constexpr (KS > 1) {
            float* mb = reinterpret_cast<float*>(lds_raw);
            if (wp > 0 && wave_active) {
                float* dst = mb + (size_t)((wr * (KS - 1) + wp - 1) * 34) * 64 + lane;
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
                    const float* src = mb + (size_t)((wr * (KS - 1) + sp - 1) * 34) * 64 + lane;
                    const float m2 = src[32 * 64];
                    const float l2 = src[33 * 64];
                    const float mx = fmaxf(m, m2);           // m is finite: split 0 sees key 0
                    const float a = fast_exp2(m - mx);
                    const float b = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mx);
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
        if (wp == 0 && wave_active) {
            const float lt = l + xchg_half(l);
            const float inv = 1.0f / lt;
            if (row < C) {
                float* dst = out + ((size_t)row * kHQ + head) * kD + 4 * hh;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    *reinterpret_cast<f4*>(dst + 8 * a) =
                        f4{o0[4 * a] * inv, o0[4 * a + 1] * inv, o0[4 * a + 2] * inv, o0[4 * a + 3] * inv};
                    *reinterpret_cast<f4*>(dst + 32 + 8 * a) =
                        f4{o1[4 * a] * inv, o1[4 * a + 1] * inv, o1[4 * a + 2] * inv, o1[4 * a + 3] * inv};
                }
            }
        }
        __syncthreads();   // LDS is reused by the next work item
    }
}

// ---------------------------------------------------------------------------
// Host side: argument checks, launch plan, dispatch.
// ---------------------------------------------------------------------------
enum Variant { kV_4x2 = 0, kV_2x4 = 1, kV_1x4 = 2 };

struct Plan {
    int rows, ks, grid, threads, per_wg, bk, lds, variant, n_row_tiles, paired;
};

template <typename T, int NW, int KS>
Plan make_plan(int C, int variant) {
    using G = Geo<T, NW, KS>;
    Plan p{};
    p.rows = G::kRows;
    p.ks = KS;
    p.threads = G::kThreads;
    p.bk = G::kBK;
    p.lds = G::kLdsBytes;
    p.variant = variant;
    p.n_row_tiles = (C + G::kRows - 1) / G::kRows;
    // Pair tiles i and n-1-i when that still leaves a workgroup per CU.
    const int pairs = (p.n_row_tiles + 1) / 2;
    p.paired = pairs * kHKV >= 256 ? 1 : 0;
    p.per_wg = p.paired ? 2 : 1;
    p.grid = (p.paired ? pairs : p.n_row_tiles) * kHKV;
    return p;
}

template <typename T>
Plan choose_plan(int C) {
    if (C >= 1024) return make_plan<T, 4, 2>(C, kV_4x2);
    if (C >= 256) return make_plan<T, 2, 4>(C, kV_2x4);
    return make_plan<T, 1, 4>(C, kV_1x4);
}

Plan plan_for(int C, attn_dtype_t dtype) {
    return dtype == ATTN_DTYPE_BF16 ? choose_plan<__bf16>(C) : choose_plan<float>(C);
}

template <typename T, int NW, int KS>
hipError_t launch(const Plan& p, const void* q, const void* k, const void* v, float* out, int C, int P,
                  hipStream_t stream) {
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    int n_row_tiles = p.n_row_tiles, paired = p.paired;
    void* args[] = {&qq, &kk, &vv, &out, &C, &P, &n_row_tiles, &paired};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_prefill_kernel<T, NW, KS>), dim3(p.grid),
                           dim3(p.threads), args, 0, stream);
}

template <typename T>
hipError_t dispatch(const Plan& p, const void* q, const void* k, const void* v, float* out, int C, int P,
                    hipStream_t stream) {
    switch (p.variant) {
        case kV_4x2: return launch<T, 4, 2>(p, q, k, v, out, C, P, stream);
        case kV_2x4: return launch<T, 2, 4>(p, q, k, v, out, C, P, stream);
        default: return launch<T, 1, 4>(p, q, k, v, out, C, P, stream);
    }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

attn_status_t attn_prefill_validate(const void* q, const void* kCache, const void* vCache, const float* out,
                                    int C, int P, attn_dtype_t dtype) {
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (C < 0 || P < 0 || P > INT_MAX - C) return ATTN_ERR_INVALID_ARG;
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

attn_status_t attn_prefill_plan(int C, int P, attn_dtype_t dtype, int* plan) {
    if (!plan) return ATTN_ERR_NULL_PTR;
    if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_UNSUPPORTED_DTYPE;
    if (C < 0 || P < 0 || P > INT_MAX - C) return ATTN_ERR_INVALID_ARG;
    const Plan p = plan_for(C > 0 ? C : 1, dtype);
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
    const Plan p = plan_for(C, dtype);
    const hipError_t e = dtype == ATTN_DTYPE_BF16 ? dispatch<__bf16>(p, q, kCache, vCache, out, C, P, stream)
                                                  : dispatch<float>(p, q, kCache, vCache, out, C, P, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
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
    }
    return "ATTN_ERR_UNKNOWN";
}

int attn_prefill_version(void) { return 100; }

}  // extern "C"
