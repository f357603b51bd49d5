// libpagedattn: paged-KV decode attention and KV append for MI355X (gfx950).
//
// The operations are the ones the ForgeLLM README (LLM-inference-server)
// lists among its features: a KV cache of physical blocks reached through
// per-request logical block tables, and decode attention that reads those
// blocks through the table with an online softmax instead of building a padded
// K/V; grouped-query heads share a kv-head.  The LLM-Inference-Engine README
// ("why dynamic injection" paragraph) notes that decode is memory-bound, and
// that is the bound these kernels are built for: every K/V byte is read from
// HBM exactly once, with 16-byte coalesced loads, and the arithmetic runs on
// the matrix cores so that it stays off the critical path.
//
// Design (one workgroup = one worker, one wavefront per kv-head of a slice):
//  * The kv-heads are taken in slices of up to 2 (the largest divisor of
//    their count that fits).  Work unit = one (sequence, slice, logical
//    block).  All units of the batch are laid end to end, sequence-major then
//    slice then block, and dealt to the workers in equal contiguous runs
//    ("stream-K"), so every worker streams the same number of blocks whatever
//    the length mix.  Wave i of a worker takes kv-head i of the slice over the
//    worker's blocks: the waves of a workgroup read the neighbouring tiles of
//    the same physical block together (one block's kv-heads are contiguous in
//    the pool), and a split of a sequence is shared by all of its heads
//    instead of multiplying the partial results.  A run that covers a whole
//    (sequence, kv-head) writes the output directly; one that covers part of
//    it stores (o, log-sum-exp), and the wave that stores the last part of a
//    pair merges the parts, inside the same launch.  The split depends only
//    on the lengths and the worker count, so results are bitwise
//    reproducible and independent of physical placement.
//  * Per 16-token tile, the G query heads of a kv-head form the columns of
//    one 16x16 MFMA tile: S = K * Q^T (tokens x heads), then O^T += V^T * P^T
//    (dims x heads).  P comes out of the first product in exactly the lane
//    layout the second needs as an operand, and every head's softmax state
//    stays in the lanes of that head's column, so no data crosses lanes
//    except for the row maximum.
//  * The cache layout (see pagedattn.h) makes each MFMA operand fragment one
//    contiguous 16-byte (K) or 8/16-byte (V) piece per lane, with consecutive
//    lanes reading consecutive bytes: the loads go straight from HBM to
//    registers, no LDS staging.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "pagedattn.h"

namespace {

constexpr int kWave = 64;
#ifndef PA_MAX_SLICE
#define PA_MAX_SLICE 2
#endif
constexpr int kMaxSlice = PA_MAX_SLICE;            // kv-heads (waves) of one decode workgroup, at most
constexpr int kGroupThreads = kWave * kMaxSlice;  // the largest decode workgroup
constexpr int kWriteThreads = 256;
// Sequences one call takes: each decode workgroup keeps 8 (several query
// tokens: 16) bytes a sequence in LDS, at most 128 KB at this count; the host
// also checks the device's LDS limit before a launch.
constexpr int kMaxSeqs = 8192;
constexpr int kMaxGroup = 16;
#ifndef PA_WAVES_PER_CU
#define PA_WAVES_PER_CU 2
#endif
constexpr int kWavesPerCU = PA_WAVES_PER_CU;  // automatic split: decode waves per compute unit
#ifndef PA_MIN_BLOCKS_PER_WORKER
#define PA_MIN_BLOCKS_PER_WORKER 16
#endif
constexpr int kMinBlocksPerWorker = PA_MIN_BLOCKS_PER_WORKER;
// Synchronisation words at the start of every workspace (zero before the first
// call, and left zero by every call): kSyncHeader counters (the prompt-chunk
// kernel's item counters, one per XCD, and its count of workgroups done), then
// one arrival word per (range, wave) of a split.
constexpr int kSyncWords = PA_WORKSPACE_SYNC_BYTES / 8;
constexpr int kSyncHeader = 16;
// XCDs of an MI355X; the dispatcher deals workgroups to them in turn (workgroup b
// runs on XCD b % kXcds).
constexpr int kXcds = 8;
constexpr int kMaxWorkers = 1 << 20;
constexpr int kMaxRopePairs = 64;  // head_dim / 2
#ifndef PA_RUN_COST_BYTES
#define PA_RUN_COST_BYTES 49152
#endif
constexpr size_t kRunCostBytes = PA_RUN_COST_BYTES;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- shapes

template <int DT, int D, int B>
struct Cfg {
    static constexpr int kElt = DT == PA_F32 ? 4 : 2;
    static constexpr int kKFrag = D * kElt / 64;  // 16-byte K pieces per lane per 16-token tile
    static constexpr int kVChunk = D / 16;        // 16-dim chunks of the output
    static constexpr int kVPiece = D * kElt / 64;  // 16-byte V pieces per lane per tile (4/kElt chunks each)
    static constexpr int kSub = B / 16;           // 16-token tiles per block
    static constexpr int kTileBytes = B * D * kElt;
    static constexpr int kSlabBytes = 16 * D * kElt;  // one 16-token slab of a tile
};


// ---------------------------------------------------------------- MFMA steps

// S (16 tokens x 16 heads) += K piece x Q piece.
template <int DT>
__device__ inline f32x4 qk_step(uint4 k, uint4 q, f32x4 acc) {
    if constexpr (DT == PA_BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), __builtin_bit_cast(bf16x8, q),
                                                        acc, 0, 0, 0);
    } else if constexpr (DT == PA_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k), __builtin_bit_cast(f16x8, q), acc,
                                                       0, 0, 0);
    } else {
        f32x4 kf = __builtin_bit_cast(f32x4, k);
        f32x4 qf = __builtin_bit_cast(f32x4, q);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], qf[e], acc, 0, 0, 0);
        return acc;
    }
}

// Probabilities of 4 tokens for this lane's head, in the operand form of the PV product.
template <int DT>
struct PPack;
template <>
struct PPack<PA_BF16> {
    i16x4 v;
};
template <>
struct PPack<PA_F16> {
    f16x4 v;
};
template <>
struct PPack<PA_F32> {
    f32x4 v;
};

template <int DT>
__device__ inline PPack<DT> pack_p(const float p[4]) {
    PPack<DT> r;
    if constexpr (DT == PA_BF16) {
        bf16x4 b = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
        r.v = __builtin_bit_cast(i16x4, b);
    } else if constexpr (DT == PA_F16) {
        r.v = f16x4{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    } else {
        r.v = f32x4{p[0], p[1], p[2], p[3]};
    }
    return r;
}

// O^T (16 dims x 16 heads) += V^T (16 dims x 4 tokens per lane group) x P^T, for
// the chunks in one 16-byte V piece: two 16-dim chunks (halves .xy, .zw) for
// 16-bit types, one (all of it) for f32.
template <int DT>
__device__ inline void pv_piece(uint4 v, PPack<DT> p, f32x4* O) {
    if constexpr (DT == PA_BF16) {
        O[0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, make_uint2(v.x, v.y)), p.v, O[0], 0, 0, 0);
        O[1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, make_uint2(v.z, v.w)), p.v, O[1], 0, 0, 0);
    } else if constexpr (DT == PA_F16) {
        O[0] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, make_uint2(v.x, v.y)), p.v, O[0], 0, 0, 0);
        O[1] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, make_uint2(v.z, v.w)), p.v, O[1], 0, 0, 0);
    } else {
        f32x4 vf = __builtin_bit_cast(f32x4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) O[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[e], p.v[e], O[0], 0, 0, 0);
    }
}

// Zero the V entries of tokens at or past the context end (their P is 0, but
// 0 * NaN would still poison the sum).  Token first_tok + e is element e of
// each 4-token group in the piece.
template <int ELT>
__device__ inline void mask_v(uint4& v, int first_tok, int ctx) {
    if constexpr (ELT == 2) {
        const uint32_t m01 = (first_tok + 0 >= ctx ? 0u : 0x0000ffffu) | (first_tok + 1 >= ctx ? 0u : 0xffff0000u);
        const uint32_t m23 = (first_tok + 2 >= ctx ? 0u : 0x0000ffffu) | (first_tok + 3 >= ctx ? 0u : 0xffff0000u);
        v.x &= m01;
        v.z &= m01;
        v.y &= m23;
        v.w &= m23;
    } else {
        if (first_tok + 0 >= ctx) v.x = 0;
        if (first_tok + 1 >= ctx) v.y = 0;
        if (first_tok + 2 >= ctx) v.z = 0;
        if (first_tok + 3 >= ctx) v.w = 0;
    }
}

// Store 4 consecutive fp32 values as the storage type (round to nearest even).
template <int DT>
__device__ inline void store4(uint8_t* dst, f32x4 x) {
    if constexpr (DT == PA_BF16) {
        bf16x4 b = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
        *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, b);
    } else if constexpr (DT == PA_F16) {
        f16x4 h = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
        *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, h);
    } else {
        *reinterpret_cast<f32x4*>(dst) = x;
    }
}

// Store 2 consecutive fp32 values as the storage type (round to nearest even).
template <int DT>
__device__ inline void store2(uint8_t* dst, float2 x) {
    if constexpr (DT == PA_BF16) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 b = {(__bf16)x.x, (__bf16)x.y};
        *reinterpret_cast<uint32_t*>(dst) = __builtin_bit_cast(uint32_t, b);
    } else if constexpr (DT == PA_F16) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        f16x2 h = {(_Float16)x.x, (_Float16)x.y};
        *reinterpret_cast<uint32_t*>(dst) = __builtin_bit_cast(uint32_t, h);
    } else {
        *reinterpret_cast<float2*>(dst) = x;
    }
}

// ---------------------------------------------------------------- arguments

struct DecodeArgs {
    const uint8_t* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    uint8_t* out;
    unsigned long long* sync;      // the workspace's synchronisation words (see kSyncWords)
    float* part_lse;               // [workers * slice][2][cols]: per wave, two slots
    float* part_o;                 // [workers * slice][2][cols][D]
    const uint8_t* k_new;          // append: [num_seqs][Hkv][D], the token at position ctx-1
    const uint8_t* v_new;
    uint8_t* k_cache_w;            // append: the same pools, written
    uint8_t* v_cache_w;
    float scale_log2;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t num_workers;  // attention workgroups
    int32_t slice;        // kv-heads side by side in a worker: its waves
    int32_t chunks;       // num_kv_heads / slice
    int32_t per_segment;  // 1: worker w owns (sequence, slice) w entirely
    int32_t attn_groups;  // append: workgroups [attn_groups, grid) store the new rows
    int32_t run_cost;     // extra units counted per (sequence, slice) with context (see load_lengths)
    int32_t cols;         // columns of a pair: G heads, or (several query tokens) tpc tokens x G heads
    const int32_t* query_start;  // several query tokens: [num_seqs + 1] query rows of each sequence
    int32_t num_q_rows;   // several query tokens: rows of q and out (query_start values are clamped to it)
    int32_t chunk;        // several query tokens: this launch takes tokens [chunk*tpc, (chunk+1)*tpc) of each
    int32_t tpc;          // several query tokens: tokens per pair (16 / G)
    int32_t chunk_min;    // several query tokens: sequences with more tokens than this go to chunk_kernel
    double rope_w[kMaxRopePairs];  // append with rotary embedding: frequencies theta^(-2i/D), i < D/2
};

// What a decode_kernel instantiation computes: one query token per sequence,
// the same with the KV append fused in, or several query tokens per sequence;
// kModeAppendRope is the append with the rotary embedding of q and the new K
// rows fused in as well (16-bit caches).
enum { kModeDecode = 0, kModeAppend = 1, kModeMulti = 2, kModeAppendRope = 3 };
constexpr bool mode_appends(int mode) { return mode == kModeAppend || mode == kModeAppendRope; }

// Element offset (in q or out) of column c of pair (s, kvh).  One token per
// sequence: head kvh*G + c of row s.  Several: the pair holds query rows
// row0 .. row0 + tpc - 1, column c being head kvh*G + c % G of row row0 + c / G.
template <bool MQ>
__device__ inline size_t col_offset(const DecodeArgs& a, int s, int kvh, int row0, int c, int D) {
    const int G = a.group;
    if constexpr (MQ)
        return ((size_t)(row0 + c / G) * a.num_q_heads + kvh * G + c % G) * D;
    else
        return ((size_t)s * a.num_q_heads + kvh * G + c) * D;
}

__device__ inline int clamp_ctx(int ctx, int B, int max_blocks) {
    ctx = ctx < 0 ? 0 : ctx;
    return ctx > max_blocks * B ? max_blocks * B : ctx;
}

// Context lengths (clamped) and the exclusive prefix over sequences of their
// unit counts, into LDS: ctx[S], pre[S + 1].  A sequence with nb > 0 blocks
// counts nb + run_cost units per slice of kv-heads: the work split deals out
// units, and the first run_cost units of a (sequence, slice) stand for the
// cost of starting a run on it (loading Q, waiting for the first tile) and
// hold no blocks.  Every wave of the workgroup takes part.
//
// With several query tokens per sequence (MQ), this launch's pair of sequence
// s holds its query tokens i in [i0, i0 + rows), i0 = chunk * tpc; they see
// positions up to L - n + i0 + rows - 1, so the pair's context is
// L - n + i0 + rows; row0[s] is the query row of token i0, rows[s] the count
// (0: no work for s in this launch).
template <int B, bool MQ>
__device__ __attribute__((always_inline)) void load_lengths(const DecodeArgs& a, int32_t* ctx, int32_t* pre, int32_t* row0, int32_t* rows,
                             int32_t* wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = a.num_seqs, nthreads = blockDim.x;
    const int per = (S + nthreads - 1) / nthreads;
    const int lo = min(S, tid * per), hi = min(S, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) {
        int c = clamp_ctx(a.context_lens[i], B, a.max_blocks);
        if constexpr (MQ) {
            // Rows outside [0, num_q_rows) are never touched, whatever query_start holds.
            const int q0 = min(max(a.query_start[i], 0), a.num_q_rows);
            const int n = min(max(a.query_start[i + 1], q0), a.num_q_rows) - q0;
            const int i0 = a.chunk * a.tpc;
            // (a sequence with more than chunk_min tokens is chunk_kernel's)
            const int nr = (i0 < n && n <= a.chunk_min) ? min(a.tpc, n - i0) : 0;
            c = nr > 0 ? max(0, min(c, c - n + i0 + nr)) : 0;
            row0[i] = q0 + i0;
            rows[i] = nr;
        }
        ctx[i] = c;
        sum += c > 0 ? (c + B - 1) / B + a.run_cost : 0;
    }
    int x = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) wave_tot[wave] = x;
    __syncthreads();
    int run = x - sum;
    for (int w = 0; w < wave; ++w) run += wave_tot[w];
    for (int i = lo; i < hi; ++i) {
        pre[i] = run;
        run += ctx[i] > 0 ? (ctx[i] + B - 1) / B + a.run_cost : 0;
    }
    if (tid == nthreads - 1) pre[S] = run;
    __syncthreads();
}

// Largest s in [0, S) with pre[s] <= v.
__device__ inline int find_seq(const int32_t* pre, int S, int v) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= v)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Runs: worker w streams units [w*U/W, (w+1)*U/W).
__device__ inline int64_t run_start(int64_t w, int64_t U, int64_t W) { return w * U / W; }

// The worker whose run holds unit u.
__device__ inline int64_t owner_of(int64_t u, int64_t U, int64_t W) { return ((u + 1) * W + U - 1) / U - 1; }

// Partial results cross workgroups (and the XCDs' separate L2 caches) inside
// one launch.  They are written and read only with device-coherent accesses
// (relaxed agent-scope atomics: they go to, and come from, the device's
// coherence point rather than a possibly stale XCD-local L2 line), so a writer
// needs only to wait for its stores to complete before it counts its part,
// and the last wave reads the parts after its count returns.  This is what an
// agent-scope release/acquire pair amounts to when every shared access is
// itself coherent, without writing back and invalidating whole L2 caches.
__device__ inline void coherent_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this wave's outstanding vector-memory operations (stores included) complete.
// s_waitcnt immediate for vmcnt(0) alone (expcnt 7 and lgkmcnt 15 wait for
// nothing).  Issued through the builtin, the compiler sees the wait and knows
// that no vector-memory access is outstanding after it.
constexpr int kWaitVmcnt0 = 0x0F70;
__device__ inline void wait_vmem_done() { __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); }
__device__ inline void wait_stores_done() { wait_vmem_done(); }
// Vector-memory operations complete in the order they were issued: wait until
// at most N (< 64) of this wave's are still outstanding.
template <int N>
__device__ inline void wait_vmem_upto() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Count this wave's part of a split (sequence, kv-head); true for the wave
// that stores the last part.  The word counts the parts stored so far: it is
// zero when the call starts (the workspace contract), every part adds one, and
// the last part puts it back to zero before it merges, so the next call on the
// same workspace (or a graph replay) finds it zero again.  Nothing depends on
// what the rest of the workspace holds.
__device__ inline bool arrive(unsigned long long* word, int parts) {
    const unsigned long long prev = atomicAdd(word, 1ull);
    if ((int)prev + 1 != parts) return false;
    atomicExch(word, 0ull);
    return true;
}

// ---------------------------------------------------------------- decode: one run of blocks

// A pointer through which uniform loads become scalar-memory loads.
typedef const int32_t __attribute__((address_space(4)))* ScalarPtr;


#ifndef PA_TILE_BUFFERS
#define PA_TILE_BUFFERS 2  // 16-token tiles in registers: one being consumed, the rest in flight
#endif
#ifndef PA_PREFETCH_RUNS
#define PA_PREFETCH_RUNS 1  // a run loads the next run's first tile and Q while it consumes its last tile
#endif
#ifndef PA_KV_NONTEMPORAL
#define PA_KV_NONTEMPORAL 1  // K/V are read once: hint the caches not to keep them
#endif

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// K/V loads.  The decode reads each K/V byte once, so its loads carry the
// non-temporal hint; the prompt-chunk kernel reads a sequence's K/V once per
// block of query tokens, and those blocks run side by side, so its loads are
// plain and the repeats come from L2 (REUSE).
template <typename T, bool REUSE = false>
__device__ inline T load_kv(const uint8_t* p) {
    if constexpr (PA_KV_NONTEMPORAL && !REUSE)
        return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
    else
        return *reinterpret_cast<const T*>(p);
}

// Put one token's entries (token e of the piece's 4-token groups) into a V piece:
// 16-bit types hold two dims per piece (halves .xy and .zw), f32 one.
template <int ELT>
__device__ inline void put_v_row(uint4& v, int e, const uint32_t* vals) {
    if constexpr (ELT == 2) {
        const int sh = (e & 1) * 16;
        const uint32_t keep = ~(0xffffu << sh);
        if (e < 2) {
            v.x = (v.x & keep) | (vals[0] << sh);
            v.z = (v.z & keep) | (vals[1] << sh);
        } else {
            v.y = (v.y & keep) | (vals[0] << sh);
            v.w = (v.w & keep) | (vals[1] << sh);
        }
    } else {
        if (e == 0) v.x = vals[0];
        if (e == 1) v.y = vals[0];
        if (e == 2) v.z = vals[0];
        if (e == 3) v.w = vals[0];
    }
}

// ---------------------------------------------------------------- rotary embedding

// Rotary embedding, rotate-half pairing: dims i and i + D/2 turn by pos * w_i.
// Every operation is spelled out (no contraction, no library call whose code
// could differ between call sites), so every kernel that rotates produces the
// same bits.  The angle (up to 10^5 radians for the first pairs at long
// contexts) is formed in double and reduced there by multiples of pi/2; sin
// and cos of the remainder r in [-pi/4, pi/4] come from their Taylor series to
// the r^11 and r^12 terms in float (Horner form; the remainder is below 2e-9,
// under float's resolution there), and the rotation is single precision.
__device__ inline void rope_cs(double w, int pos, float& c, float& s) {
#pragma clang fp contract(off)
    constexpr double kHalfPi = 1.5707963267948966;
    const double ang = (double)pos * w;
    const double k = rint(ang * (1.0 / kHalfPi));
    const float r = (float)fma(-kHalfPi, k, ang);
    const float r2 = r * r;
    float ps = -1.0f / 5040.0f + r2 * (1.0f / 362880.0f - r2 * (1.0f / 39916800.0f));
    ps = 1.0f / 120.0f + r2 * ps;
    ps = -1.0f / 6.0f + r2 * ps;
    const float sr = r + (r * r2) * ps;
    float pc = 1.0f / 40320.0f + r2 * (-1.0f / 3628800.0f + r2 * (1.0f / 479001600.0f));
    pc = -1.0f / 720.0f + r2 * pc;
    pc = 1.0f / 24.0f + r2 * pc;
    pc = -0.5f + r2 * pc;
    const float cr = 1.0f + r2 * pc;
    // angle = r + q pi/2 with q = k mod 4: (sin, cos) is (sr, cr), (cr, -sr),
    // (-sr, -cr) or (-cr, sr); selects rather than a branch on q.
    const int q = (int)(((int64_t)k) & 3);
    const float sa = (q & 1) ? cr : sr, ca = (q & 1) ? sr : cr;
    s = (q & 2) ? -sa : sa;
    c = ((q + 1) & 2) ? -ca : ca;
}
__device__ inline void rope_rot(float& x, float& y, float c, float s) {
#pragma clang fp contract(off)
    const float nx = x * c - y * s;
    const float ny = y * c + x * s;
    x = nx;
    y = ny;
}

// The X = 16 / ELT values of a 16-byte piece, widened to float, and back (RNE).
template <int DT>
__device__ inline void piece_to_float(uint4 v, float* f) {
    if constexpr (DT == PA_BF16) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (float)b[j];
    } else if constexpr (DT == PA_F16) {
        const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (float)h[j];
    } else {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
}
template <int DT>
__device__ inline uint4 float_to_piece(const float* f) {
    if constexpr (DT == PA_BF16) {
        bf16x8 b;
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = (__bf16)f[j];
        return __builtin_bit_cast(uint4, b);
    } else if constexpr (DT == PA_F16) {
        f16x8 h;
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = (_Float16)f[j];
        return __builtin_bit_cast(uint4, h);
    } else {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
}

// Rotate a row held as pieces: pieces[f] holds dims (4f + r) * X .. + X - 1 for
// f < NF, so piece f and piece f + NF/2 hold the dims i and i + D/2 of the
// same pairs (the fragments the QK product uses).
template <int DT, int NF>
__device__ __attribute__((always_inline)) inline void rope_fragments(uint4* pieces, int r, int pos, const double* w) {
    constexpr int X = DT == PA_F32 ? 4 : 8;
#pragma unroll
    for (int f = 0; f < NF / 2; ++f) {
        float x[X], y[X];
        piece_to_float<DT>(pieces[f], x);
        piece_to_float<DT>(pieces[f + NF / 2], y);
#pragma unroll
        for (int j = 0; j < X; ++j) {
            float c, sn;
            rope_cs(w[(4 * f + r) * X + j], pos, c, sn);
            rope_rot(x[j], y[j], c, sn);
        }
        pieces[f] = float_to_piece<DT>(x);
        pieces[f + NF / 2] = float_to_piece<DT>(y);
    }
}

// The same rotation for up to 16 rows (columns of the QK product) held as
// operand pieces, through a per-wave LDS buffer: the lanes spread over the
// pairs of the rows that need it instead of each turning all of its own
// pieces.  Lane (n, r) holds pieces[f] = dims (4f + r) * 8 .. + 7 of a row;
// lanes with `has` put theirs in row `wrow` of the buffer, rows [0, nrows)
// (a wave-uniform count) are rotated, and those lanes take back row `rrow`.
// 16-bit types only.
template <int DT, int D, int NF>
__device__ __attribute__((always_inline)) inline void rope_rows_lds(uint4* pieces, int wrow, int rrow, bool has, int nrows,
                                                                    int r, int pos, const double* w, uint8_t* buf) {
    static_assert(DT != PA_F32, "16-bit rows");
    const int lane = threadIdx.x & 63;
    uint4* b = reinterpret_cast<uint4*>(buf);  // [row][D / 8] 16-byte units
    if (has) {
#pragma unroll
        for (int f = 0; f < NF; ++f) b[wrow * (D / 8) + 4 * f + r] = pieces[f];
    }
    __builtin_amdgcn_wave_barrier();
    typedef typename std::conditional<DT == PA_BF16, __bf16, _Float16>::type T;
    T* e = reinterpret_cast<T*>(buf);
    const int pairs = nrows * (D / 2);
#pragma unroll 1
    for (int p0 = 0; p0 < pairs; p0 += kWave) {
        const int p = p0 + lane;
        const int rw = p / (D / 2), i = p % (D / 2);
        if (p < pairs) {
            float x = (float)e[rw * D + i], y = (float)e[rw * D + i + D / 2];
            float c, sn;
            rope_cs(w[i], pos, c, sn);
            rope_rot(x, y, c, sn);
            e[rw * D + i] = (T)x;
            e[rw * D + i + D / 2] = (T)y;
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (has) {
#pragma unroll
        for (int f = 0; f < NF; ++f) pieces[f] = b[rrow * (D / 8) + 4 * f + r];
    }
    __builtin_amdgcn_wave_barrier();
}

// Vector loads of a prefetched run start: its first tile (K and V pieces) and its Q pieces.
template <int DT, int D>
constexpr int kPrefetchLoads = 2 * Cfg<DT, D, 16>::kKFrag + Cfg<DT, D, 16>::kVPiece;

template <int DT, int D, int B>
struct Tile {
    uint4 k[Cfg<DT, D, B>::kKFrag];
    uint4 v[Cfg<DT, D, B>::kVPiece];
};

// Where a wave's partial result for one split (sequence, kv-head) lives: wave
// wid = worker * slice + (kv-head within the slice), slot 0 for the worker's
// first run and 1 for its last.
__device__ inline size_t part_index(int64_t wid, int slot, int G, int h) { return ((size_t)wid * 2 + slot) * G + h; }

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48:
// one head's four row groups).  permlane16/32_swap leave, in the two halves of
// their result, a lane's own value and that of its partner 16 (32) lanes away,
// in some order; both are plain VALU operations.
__device__ inline float row_group_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float row_group_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Per-wave LDS used by a merge: the weights of a pass's parts, and per column
// the running denominator and rescale factor.
struct MergeLds {
    float w[kWave][kMaxGroup];  // weight of part k for column h (relative to the running max)
    float den[kMaxGroup];       // running sum of weights
    float rescale[kMaxGroup];   // factor applied to earlier chunks when the running max grows
};
// (Before a run's first tile is consumed, the area also holds the 16 rows of
// Q being rotated: 16 x 128 16-bit values.)
static_assert(sizeof(MergeLds) >= 16 * 128 * 2, "rotation buffer");

// Lane x of the same 16-lane row, by DPP: quad_perm [1,0,3,2] (xor 1),
// quad_perm [2,3,0,1] (xor 2), row_ror 4 and row_ror 8.
template <int CTRL>
__device__ inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Max and sum over the lanes that share lane % NCp (NCp a power of two up to
// 16): rotations inside each 16-lane row (xor 1, xor 2 by quad_perm; row_ror
// 4 and 8), as many as NCp leaves, then across the four rows by the swaps.
__device__ inline float parts_max(float x, int NCp) {
    if (NCp < 2) x = fmaxf(x, dpp<0xB1>(x));
    if (NCp < 4) x = fmaxf(x, dpp<0x4E>(x));
    if (NCp < 8) x = fmaxf(x, dpp<0x124>(x));
    if (NCp < 16) x = fmaxf(x, dpp<0x128>(x));
    return row_group_max(x);
}
__device__ inline float parts_sum(float x, int NCp) {
    if (NCp < 2) x += dpp<0xB1>(x);
    if (NCp < 4) x += dpp<0x4E>(x);
    if (NCp < 8) x += dpp<0x124>(x);
    if (NCp < 16) x += dpp<0x128>(x);
    return row_group_sum(x);
}

// Whole-wave reductions without LDS: all-reduce within each 16-lane row by DPP,
// then across the four rows with the permlane swaps.
__device__ inline float wave_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x124>(x));
    x = fmaxf(x, dpp<0x128>(x));
    return row_group_max(x);
}
__device__ inline float wave_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x124>(x);
    x += dpp<0x128>(x);
    return row_group_sum(x);
}

// Partial results go through buffer resources: accesses are bounds-checked to
// the resource (a load past its end returns 0) and carry the agent-coherence
// bit (the cache-policy operand's SC1, 16), like the relaxed agent-scope
// accesses above.  Word 3 is the gfx9-family raw-buffer format.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCoherentPolicy = 16;
__device__ inline f32x4 coherent_load4(__amdgpu_buffer_rsrc_t r, int byte_offset) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, kCoherentPolicy));
}
__device__ inline void coherent_store4(__amdgpu_buffer_rsrc_t r, int byte_offset, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_offset, 0, kCoherentPolicy);
}
__device__ inline float coherent_load1(__amdgpu_buffer_rsrc_t r, int byte_offset) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_offset, 0, kCoherentPolicy));
}

// The log-sum-exp merge of a pair's parts, by the wave that stored the last
// one.  A pair has NC = a.cols columns (heads, or query token x head); its
// NC x D outputs are cut into 16-byte units; in a pass over units
// [unit0, unit0 + 64 UPL), lane l owns units unit0 + l + 64 i (i < UPL) and
// keeps their float4 accumulators in registers.  Parts are taken 64 / NCp at a
// time (NCp: NC rounded up to a power of two), one log-sum-exp per lane, and
// one reduction over the lanes of each column forms the running maximum M, the
// weights 2^(lse - M) and their sum for all columns at once.
// The outputs are read PB = kMergeLoads/UPL parts per batch, kMergeLoads
// 16-byte loads in flight per lane; the first batch is issued before the
// log-sum-exps, so a merge of up to PB parts costs one round trip to memory.  Only the first
// `active` columns are stored (the rest pad the last token group).
#ifndef PA_MERGE_LOADS
#define PA_MERGE_LOADS 8
#endif
// 16-byte loads per lane in one batch of a merge.  Larger batches shorten
// merges of many parts but raise the kernel's register count everywhere.
constexpr int kMergeLoads = PA_MERGE_LOADS;
static_assert(kMergeLoads >= 8, "a batch must hold at least one part at 8 units per lane");

template <int DT, int D, int UPL, bool MQ>
__device__ __attribute__((always_inline)) void merge_body(const DecodeArgs& a, int s, int kvh, int row0, int active, int64_t F, int parts,
                           int64_t wa, int first_slot, bool unit_runs, int64_t U, int64_t W, int hs, int wi,
                           int unit0, MergeLds& L) {
    constexpr int E = DT == PA_F32 ? 4 : 2;
    constexpr int PB = kMergeLoads / UPL;
    // A part holds a.cols columns (the stride of the layout); only the pair's
    // first `active` ones hold a query, and only those are read and merged.
    const int lane = threadIdx.x & 63, NS = a.cols, NC = active;
    const int NU = NC * D / 4;
    const int part_bytes = NC * D * 4;
    const int lse_bytes = (int)(W * hs * 2 * NS * 4);  // every wave's two slots of NS log-sum-exps
    const __amdgpu_buffer_rsrc_t lse_r =
        __builtin_amdgcn_make_buffer_rsrc(a.part_lse, (short)0, lse_bytes, kBufferWord3);

    f32x4 acc[UPL];
    int hu[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        hu[i] = min((unit0 + lane + kWave * i) * 4 / D, NC - 1);
    }
    // Index of part k's first log-sum-exp (part_index(wave, slot, NC, 0)): the
    // part's worker, and in it the wave of this pair's kv-head.
    auto part_loc = [&](int k) -> int64_t {
        const int64_t wk = unit_runs ? owner_of(F + k, U, W) : wa + k;
        return (int64_t)part_index(wk * hs + wi, k == 0 ? first_slot : 0, NS, 0);
    };
    // Every slot of v is defined and read on every path (unused slots are zero
    // and weigh 0), so no load of the merge can be left pending where the
    // next run reuses its register.
    f32x4 v[PB][UPL];
    auto issue = [&](int kb, int n) {  // parts kb .. kb + n - 1 (n <= PB), uniform
#pragma unroll
        for (int p = 0; p < PB; ++p) {
#pragma unroll
            for (int i = 0; i < UPL; ++i) v[p][i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p < n) {
                const float* base = a.part_o + part_loc(kb + p) * D;
                const __amdgpu_buffer_rsrc_t r =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, part_bytes, kBufferWord3);
#pragma unroll
                for (int i = 0; i < UPL; ++i) v[p][i] = coherent_load4(r, (unit0 + lane + kWave * i) * 16);
            }
        }
    };
    auto consume = [&](int kb, int n, int k0) {
#pragma unroll
        for (int p = 0; p < PB; ++p) {
#pragma unroll
            for (int i = 0; i < UPL; ++i) acc[i] += (p < n ? L.w[kb + p - k0][hu[i]] : 0.f) * v[p][i];
        }
    };

    // A pass takes PPP parts: lane (kk, hh) = (lane / NCp, lane % NCp) holds
    // part k0 + kk's log-sum-exp of column hh (NCp: the columns rounded up to a
    // power of two), so the maxima and sums over the parts of every column come
    // from one reduction across the lanes of that column.  Mh and Dh are the
    // column's running maximum and denominator (the same in all its lanes).
    const int NCp = NC <= 1 ? 1 : NC <= 2 ? 2 : NC <= 4 ? 4 : NC <= 8 ? 8 : 16;
    const int PPP = kWave / NCp;
    const int kk = lane / NCp, hh = lane % NCp;
    float Mh = -INFINITY, Dh = 0.f;
    for (int k0 = 0; k0 < parts; k0 += PPP) {
        const int cnt = min(PPP, parts - k0);
        issue(k0, min(PB, cnt));
        // The load is not under a lane mask (a lane without a part reads past
        // the end and gets 0), so the compiler sees every one consumed.
        const bool has = kk < cnt && hh < NC;
        const int lse_off = has ? (int)(part_loc(k0 + kk) * 4) + 4 * hh : lse_bytes;
        const float x0 = coherent_load1(lse_r, lse_off);
        const float x = has ? x0 : -INFINITY;
        const float mn = fmaxf(Mh, parts_max(x, NCp));
        // (0 while Mh is -inf; a padding column, all -inf, keeps 1)
        const float sc = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(Mh - mn);
        const float wt = has ? __builtin_amdgcn_exp2f(x - mn) : 0.f;
        Dh = Dh * sc + parts_sum(wt, NCp);
        Mh = mn;
        L.w[kk][hh] = wt;
        if (kk == 0) {
            L.den[hh] = Dh;
            L.rescale[hh] = sc;
        }
        __builtin_amdgcn_wave_barrier();
        if (k0 > 0) {
#pragma unroll
            for (int i = 0; i < UPL; ++i) acc[i] *= L.rescale[hu[i]];
        }
        consume(k0, min(PB, cnt), k0);
        for (int kb = k0 + PB; kb < k0 + cnt; kb += PB) {
            const int n = min(PB, k0 + cnt - kb);
            issue(kb, n);
            consume(kb, n, k0);
        }
        __builtin_amdgcn_wave_barrier();
    }
    // Every load above has been consumed by now; saying so (vmcnt 0, before
    // the stores) keeps the compiler from draining the next run's loads at its
    // start for a load it cannot prove done.
    wait_vmem_done();
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = unit0 + lane + kWave * i;
        const int h = u * 4 / D, d = u * 4 % D;
        if (u < NU && h < active) {
            uint8_t* dst = a.out + (col_offset<MQ>(a, s, kvh, row0, h, D) + d) * E;
            store4<DT>(dst, acc[i] * (1.f / L.den[h]));
        }
    }
    __builtin_amdgcn_wave_barrier();
}

template <int DT, int D, bool MQ>
__device__ __attribute__((always_inline)) void merge_parts(const DecodeArgs& a, int s, int kvh, int row0, int active, int64_t F, int64_t Fv, int nb,
                            int64_t U, int64_t W, int hs, int wi, MergeLds& L) {
    const bool unit_runs = W >= U;
    const int64_t wa = owner_of(F, U, W);
    const int parts = unit_runs ? nb : (int)(owner_of(F + nb - 1, U, W) - wa + 1);
    // The owner of the first block used slot 0 if this pair was its first run,
    // i.e. its units begin at or after the pair's first unit Fv.
    const int first_slot = run_start(wa, U, W) >= Fv ? 0 : 1;
    const int units = active * D / 4;  // 16-byte output units of the pair's active columns
    if (units <= kWave)
        merge_body<DT, D, 1, MQ>(a, s, kvh, row0, active, F, parts, wa, first_slot, unit_runs, U, W, hs, wi, 0, L);
    else if (units <= 2 * kWave)
        merge_body<DT, D, 2, MQ>(a, s, kvh, row0, active, F, parts, wa, first_slot, unit_runs, U, W, hs, wi, 0, L);
    else if (units <= 4 * kWave)
        merge_body<DT, D, 4, MQ>(a, s, kvh, row0, active, F, parts, wa, first_slot, unit_runs, U, W, hs, wi, 0, L);
    else if (MQ && units <= 8 * kWave)  // 16 columns of D = 128: one pass, 2 parts a batch
        merge_body<DT, D, 8, MQ>(a, s, kvh, row0, active, F, parts, wa, first_slot, unit_runs, U, W, hs, wi, 0, L);
    else
        for (int u0 = 0; u0 < units; u0 += 4 * kWave)  // up to 256 units per pass
            merge_body<DT, D, 4, MQ>(a, s, kvh, row0, active, F, parts, wa, first_slot, unit_runs, U, W, hs, wi, u0, L);
}

// One run of a worker: logical blocks [j0, j1) of pair (s, kvh), whose
// (sequence, slice) occupies units [Fv, F + nb) of the split (the units before
// F hold no block).  Every field is the same in all lanes of the wave.
struct Run {
    int s, kvh, ctx, row0, rows, j0, j1, nb, slot;
    int64_t F, Fv;
};

// What a run starts from when it was prefetched: its first tile, its Q
// pieces, the id of its first block (checked) and that of its second (raw),
// all loaded while the run before it consumed its last tile.
template <int DT, int D, int B>
struct Prefetch {
    Tile<DT, D, B> tile;
    uint4 q[Cfg<DT, D, B>::kKFrag];
    int phys;
    int next_id;
};

// Q of the lane's column, in the B-operand form of the QK product.  Columns
// n >= active are padding: they take column 0's row, so they only repeat its
// scores (and its rescale decisions) and are never stored.  Every lane loads,
// so the load is not under a lane mask.
template <int DT, int D, bool MQ>
__device__ inline void load_q(const DecodeArgs& a, const Run& r, uint4* qf) {
    constexpr int E = DT == PA_F32 ? 4 : 2;
    const int lane = threadIdx.x & 63, n = lane & 15, rg = lane >> 4;
    const int active = MQ ? r.rows * a.group : a.group;
    const int qc = n < active ? n : 0;
    const uint8_t* qrow = a.q + col_offset<MQ>(a, r.s, r.kvh, r.row0, qc, D) * E;
#pragma unroll
    for (int f = 0; f < Cfg<DT, D, 16>::kKFrag; ++f) qf[f] = *reinterpret_cast<const uint4*>(qrow + 64 * f + 16 * rg);
}

// The loads of tile `tau` of a run whose current block id is `phys`: the
// 16-token slab tau % kSub of (block, kv-head), 16 * D contiguous elements of
// either pool.
template <int DT, int D, int B, bool REUSE = false>
__device__ inline void load_tile(const DecodeArgs& a, int phys, int kvh, int u, Tile<DT, D, B>& t) {
    using C = Cfg<DT, D, B>;
    const int lane = threadIdx.x & 63, n = lane & 15, r = lane >> 4;
    const size_t slab = (size_t)phys * a.num_kv_heads * C::kTileBytes + (size_t)kvh * C::kTileBytes +
                        (size_t)u * C::kSlabBytes;
    const uint8_t* kt = a.k_cache + slab;
    const uint8_t* vt = a.v_cache + slab;
#pragma unroll
    for (int f = 0; f < C::kKFrag; ++f)
        t.k[f] = __builtin_bit_cast(uint4, load_kv<u32x4, REUSE>(kt + ((4 * f + r) * 16 + n) * 16));
#pragma unroll
    for (int c = 0; c < C::kVPiece; ++c)
        t.v[c] = __builtin_bit_cast(uint4, load_kv<u32x4, REUSE>(vt + ((r * C::kVPiece + c) * 16 + n) * 16));
}

// Start run r early: its first block id (already read: id0) and the one after,
// its first tile and its Q.
template <int DT, int D, int B, bool MQ>
__device__ __attribute__((always_inline)) inline void prefetch_run(const DecodeArgs& a, const Run& r, int id0,
                                                                   Prefetch<DT, D, B>& pf) {
    const ScalarPtr bt = (ScalarPtr)(a.block_tables + (size_t)r.s * a.max_blocks);
    pf.phys = ((unsigned)id0 < (unsigned)a.num_blocks) ? id0 : 0;
    // (read unconditionally: j0 + 1 is inside the row unless j0 is its last entry,
    // and then the value is never used)
    pf.next_id = bt[r.j0 + 1 < a.max_blocks ? r.j0 + 1 : r.j0];
    load_tile<DT, D, B>(a, pf.phys, r.kvh, 0, pf.tile);
    load_q<DT, D, MQ>(a, r, pf.q);
}

// Attend pair (s, kvh) of run r over its blocks [j0, j1).  A run over the
// whole context writes out; otherwise the run stores a partial in slot
// r.slot of wave wid (wave wi of its worker, which has hs waves), and the wave
// that stores the pair's last partial merges them.  With several query tokens
// (MODE kModeMulti) the pair's columns are its `rows` query tokens (from query
// row row0) times the G heads, and column (i, h) sees positions up to
// ctx - rows + i; otherwise the columns are the G heads of sequence s's one
// token, which sees positions up to ctx - 1.
// With PF, the run's first tile and Q are already in flight in pf, and when
// `more` is set the run loads the next run's (nx) into pf while it consumes
// its own last tile, so that the next run never waits a full memory latency
// for its first tile.
template <int DT, int D, int B, int MODE, bool PF>
__device__ __attribute__((always_inline)) void attend_run(const DecodeArgs& a, const Run& rn, bool more, const Run& nx,
                                                          Prefetch<DT, D, B>& pf, int64_t U, int64_t W, int wid,
                                                          int hs, int wi, MergeLds& mlds, const double* rw) {
    const int s = rn.s, kvh = rn.kvh, ctx = rn.ctx, row0 = rn.row0, rows = rn.rows, j0 = rn.j0, j1 = rn.j1,
              nb = rn.nb, slot = rn.slot;
    const int64_t F = rn.F, Fv = rn.Fv;
    using C = Cfg<DT, D, B>;
    constexpr int E = C::kElt;
    constexpr int NBUF = PA_TILE_BUFFERS;
    constexpr bool APPEND = mode_appends(MODE), MQ = MODE == kModeMulti, ROPE = MODE == kModeAppendRope;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // this lane's column (and row within a 16-row piece)
    const int r = lane >> 4;  // this lane's group of 4 rows / k-range
    const int G = a.group;
    const int active = MQ ? rows * G : G;  // columns that hold a query
    const int qc = n < active ? n : 0;     // the column whose query this lane uses
    // Last position this lane's column sees; a tile reaching past lim0 needs masking.
    const int lim0 = MQ ? ctx - rows : ctx - 1;
    const int lim = MQ ? lim0 + qc / G : lim0;

    // Block ids are read with scalar loads (the row of the table is the same for
    // the whole wave), one block ahead, so waiting for one never waits on the
    // K/V loads in flight.
    const ScalarPtr bt = (ScalarPtr)(a.block_tables + (size_t)s * a.max_blocks);
    int next_id = PF ? pf.next_id : bt[j0];
    // The next run's first block id, read now so that it is at hand when this
    // run issues the next run's first tile.
    int nx_id0 = 0;
    if constexpr (PF) {
        if (more) nx_id0 = ((ScalarPtr)(a.block_tables + (size_t)nx.s * a.max_blocks))[nx.j0];
    }

    uint4 qf[C::kKFrag];
    if constexpr (PF) {
#pragma unroll
        for (int f = 0; f < C::kKFrag; ++f) qf[f] = pf.q[f];
    } else {
        load_q<DT, D, MQ>(a, rn, qf);
    }

    f32x4 O[C::kVChunk];
#pragma unroll
    for (int c = 0; c < C::kVChunk; ++c) O[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;  // running max (log2 domain) of this lane's head
    float lsum = 0.f;     // this lane's share of the running denominator

    const int ntiles = (j1 - j0) * C::kSub;

    // Fused append: the run that holds the sequence's last block owns the new
    // token (position ctx - 1).  It loads the token's K/V rows for this kv-head
    // into the registers where its tile holds them and attends to them from
    // there, so it never depends on the cache store of those rows, which
    // other waves of the launch make (its tile load may see the slot before
    // or after that store).  No other run reads that slot.
    const bool owns_new = APPEND && j1 == nb && ctx > 0;
    const int tl = ctx - 1;                        // position of the new token
    const int tl_tile = (tl / B - j0) * C::kSub + (tl % B) / 16;  // its tile in this run
    const int tt = tl % 16;                        // its row within that tile
    uint4 k_sub[C::kKFrag];                        // lanes n == tt: the K pieces of the new row
    uint32_t v_sub[C::kVPiece][4 / E];             // lanes r == tt/4: its V entries for this lane's dims
    if constexpr (APPEND) {
        if (owns_new) {
            const size_t row = ((size_t)s * a.num_kv_heads + kvh) * (size_t)(D * E);
            const uint8_t* kn = a.k_new + row;
            const uint8_t* vn = a.v_new + row;
#pragma unroll
            for (int f = 0; f < C::kKFrag; ++f)
                k_sub[f] = n == tt ? *reinterpret_cast<const uint4*>(kn + (4 * f + r) * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int c = 0; c < C::kVPiece; ++c)
#pragma unroll
                for (int h = 0; h < 4 / E; ++h) {
                    const int d = c * (64 / E) + 16 * h + n;  // dim of this lane's row in half h of piece c
                    v_sub[c][h] = r == tt / 4 ? (E == 2 ? (uint32_t)reinterpret_cast<const uint16_t*>(vn)[d]
                                                        : reinterpret_cast<const uint32_t*>(vn)[d])
                                              : 0u;
                }
        }
    }

    int phys = PF ? pf.phys : 0;
    auto issue = [&](int tau, Tile<DT, D, B>& t) {
        const int j = j0 + tau / C::kSub, u = tau % C::kSub;
        if (u == 0) {  // first tile of block j: take its id, fetch the next one
            phys = ((unsigned)next_id < (unsigned)a.num_blocks) ? next_id : 0;
            if (j + 1 < j1) next_id = bt[j + 1];
        }
        load_tile<DT, D, B>(a, phys, kvh, u, t);
    };
    // The next run's first tile and Q, in place of the tile after this run's last.
    // (With no next run pf is cleared instead, so that on every path its old
    // contents -- this run's first tile and Q -- are dead once copied out.)
    auto prefetch_next = [&]() {
        if constexpr (PF) {
            if (more) {
                prefetch_run<DT, D, B, MQ>(a, nx, nx_id0, pf);
            } else {
#pragma unroll
                for (int f = 0; f < C::kKFrag; ++f) pf.tile.k[f] = pf.q[f] = make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int c = 0; c < C::kVPiece; ++c) pf.tile.v[c] = make_uint4(0, 0, 0, 0);
            }
        }
    };

    // m is a reference maximum, not necessarily the running one: weights are
    // exp2(z - m), and m (with O and lsum) is moved up only when some head's
    // tile maximum exceeds it by more than kLazy, so most tiles skip the
    // rescale.  Weights then stay below 2^kLazy, far inside fp32 and the
    // 16-bit P operand's range, and O / lsum is unchanged by the choice of m.
    constexpr float kLazy = 8.f;
    auto consume = [&](int tau, Tile<DT, D, B>& t, bool may_be_partial) {
        const int j = j0 + tau / C::kSub, u = tau % C::kSub;
        const int tok0 = j * B + 16 * u + 4 * r;  // position of this lane's first row
        const bool partial = may_be_partial && j * B + 16 * u + 16 > lim0 + 1;
        if constexpr (APPEND) {
            if (may_be_partial && owns_new && tau == tl_tile) {  // the tile holding the new token
                if (n == tt) {
#pragma unroll
                    for (int f = 0; f < C::kKFrag; ++f) t.k[f] = k_sub[f];
                }
                if (r == tt / 4) {
#pragma unroll
                    for (int c = 0; c < C::kVPiece; ++c) put_v_row<E>(t.v[c], tt % 4, v_sub[c]);
                }
            }
        }

        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < C::kKFrag; ++f) sc = qk_step<DT>(t.k[f], qf[f], sc);

        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = sc[e] * a.scale_log2;
            if (partial && tok0 + e > lim) z[e] = -INFINITY;
        }
        const float tmax = row_group_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
        if (__builtin_amdgcn_read_exec() & __ballot(tmax > m + kLazy)) {
            const float m_new = fmaxf(m, tmax);
            const float alpha = (m == m_new) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int c = 0; c < C::kVChunk; ++c) O[c] *= alpha;
            m = m_new;
        }
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = (z[e] > -INFINITY) ? __builtin_amdgcn_exp2f(z[e] - m) : 0.f;
        lsum += (p[0] + p[1]) + (p[2] + p[3]);

        if (partial) {
#pragma unroll
            for (int c = 0; c < C::kVPiece; ++c) mask_v<E>(t.v[c], tok0, ctx);
        }
        const PPack<DT> pp = pack_p<DT>(p);
#pragma unroll
        for (int c = 0; c < C::kVPiece; ++c) pv_piece<DT>(t.v[c], pp, &O[c * (4 / E)]);
    };

    // Ring of NBUF tiles: tile tau lives in buf[tau % NBUF]; NBUF - 1 tiles are
    // in flight while one is consumed.  The steady-state loop issues exactly one
    // tile per step on every path, so the wait before consuming a tile counts
    // only the loads issued after it and never drains the ring; the first and
    // last steps are peeled.
    // Only the last kSub tiles of a sequence can reach past its end (with
    // several query tokens, up to 15 more positions are masked for some
    // columns: one tile more); the steady loop stops early enough that those
    // always fall in the peeled tail, so it never pays for masking.
    constexpr int kMasked = MQ ? C::kSub + 1 : C::kSub;
    constexpr int kTail = (NBUF - 1 > kMasked ? NBUF - 1 : kMasked);
    // With the rotary embedding fused in, Q and the new K row are rotated (at
    // the token's position, ctx - 1) once the first tiles are on their way, so
    // the rotation overlaps their latency instead of delaying their issue.
    auto rotate_inputs = [&]() {
        if constexpr (ROPE) {
            uint8_t* lbuf = reinterpret_cast<uint8_t*>(&mlds);  // free until the merge
            // Only the active columns are turned; padding columns take column 0's result.
            rope_rows_lds<DT, D, C::kKFrag>(qf, n, qc, true, active, r, ctx - 1, rw, lbuf);
            if (owns_new) rope_rows_lds<DT, D, C::kKFrag>(k_sub, 0, 0, n == tt, 1, r, tl, rw, lbuf);
        }
    };
    Tile<DT, D, B> buf[NBUF];
    // The run's first tile: already in flight when it was prefetched.
    auto first = [&]() {
        if constexpr (PF)
            buf[0] = pf.tile;
        else
            issue(0, buf[0]);
    };
    if (ntiles < NBUF) {
        first();
#pragma unroll
        for (int i = 1; i < NBUF; ++i)
            if (i < ntiles) issue(i, buf[i]);
        prefetch_next();
        rotate_inputs();
#pragma unroll
        for (int i = 0; i < NBUF; ++i)
            if (i < ntiles) consume(i, buf[i], true);
    } else {
        first();
#pragma unroll
        for (int i = 1; i < NBUF - 1; ++i) issue(i, buf[i]);
        rotate_inputs();
        int tau0 = 0;
        for (; tau0 + NBUF - 1 + kTail < ntiles; tau0 += NBUF) {
#pragma unroll
            for (int k = 0; k < NBUF; ++k) {
                issue(tau0 + k + NBUF - 1, buf[(k + NBUF - 1) % NBUF]);
                consume(tau0 + k, buf[k], false);
            }
        }
#pragma unroll
        for (int k = 0; k < NBUF + kTail; ++k) {
            const int tau = tau0 + k;
            if (tau < ntiles) {
                if (tau + NBUF - 1 < ntiles)
                    issue(tau + NBUF - 1, buf[(k + NBUF - 1) % NBUF]);
                else if (tau + NBUF - 1 == ntiles)
                    prefetch_next();
                consume(tau, buf[k % NBUF], true);
            }
        }
    }

    // Every tile load of this run has been consumed; only the next run's
    // prefetch (issued last) may still be in flight.  Saying so before the
    // stores below keeps the compiler from draining loads for a register it
    // cannot prove written.
    wait_vmem_upto<PF ? kPrefetchLoads<DT, D> : 0>();

    // Full denominator of the lane's head: the four row groups hold disjoint tokens.
    lsum = row_group_sum(lsum);
    // (A column that sees no position can only come from lengths that break
    // the preconditions; it then gets 0 rather than 0/0.)
    const float inv = MQ ? (lsum > 0.f ? 1.f / lsum : 0.f) : 1.f / lsum;
    if (j0 == 0 && j1 == nb) {
        if (n < active) {
            uint8_t* orow = a.out + col_offset<MQ>(a, s, kvh, row0, n, D) * E;
#pragma unroll
            for (int c = 0; c < C::kVChunk; ++c) store4<DT>(orow + (16 * c + 4 * r) * E, O[c] * inv);
        }
        return;
    }
    {
        // The partial's outputs as 16-byte stores with the agent-coherence bit
        // (through a resource bounded to the part's active columns, so lanes of
        // padding columns store nothing).
        const size_t part0 = part_index(wid, slot, a.cols, 0);
        const __amdgpu_buffer_rsrc_t po = __builtin_amdgcn_make_buffer_rsrc(a.part_o + part0 * D, (short)0,
                                                                             active * D * 4, kBufferWord3);
#pragma unroll
        for (int c = 0; c < C::kVChunk; ++c) coherent_store4(po, (n * D + 16 * c + 4 * r) * 4, O[c] * inv);
        if (n < active && r == 0) coherent_store(a.part_lse + part0 + n, m + __log2f(lsum));
    }
    // Publish the partial (wait until its device-coherent stores are done),
    // then count it; the wave that stores the last part merges.
    wait_stores_done();
    const int parts = W >= U ? nb : (int)(owner_of(F + nb - 1, U, W) - owner_of(F, U, W) + 1);
    int last = 0;
    // The pair's arrival word belongs to the range holding its first block: a
    // pair is split only when it runs past the end of that range, and only the
    // last pair that starts in a range can, so the word is the pair's alone.
    const int64_t first_owner = owner_of(F, U, W);
    if (lane == 0) last = arrive(a.sync + kSyncHeader + first_owner * hs + wi, parts) ? 1 : 0;
    if (__shfl(last, 0)) merge_parts<DT, D, MQ>(a, s, kvh, row0, active, F, Fv, nb, U, W, hs, wi, mlds);
}

// Fused append, the store side: wave `wi` of the writer workgroups copies the
// new K/V rows of RPW consecutive (sequence, kv-head) rows into their slots,
// the same bytes pa_write_kv stores.  It runs beside the attention waves, so
// their loads never wait behind these stores (a wave's loads and stores share
// one counter).  Each row touches one line per 16-byte K piece and one per V
// line of its slab.  These partial-line stores are what the append costs the
// reads around them.  Plain stores cost the most; the non-temporal hint less;
// the agent-coherence bit (SC1), used here, a little less again.  A row with
// no context, or whose block id or length lies outside the table or pool, is
// skipped.
template <int DT, int D, int B, bool ROPE>
__device__ __attribute__((always_inline)) void store_new_rows(const DecodeArgs& a, int wi, const double* rw) {
    using C = Cfg<DT, D, B>;
    constexpr int E = C::kElt;
    constexpr int KP = D * E / 16;  // 16-byte pieces per row
    constexpr int RPW = 64 / KP;    // rows per wave: one piece per lane
    constexpr int NV = RPW * D / 64;  // V elements per lane; element k of a lane is in row 64k / D
    const int lane = threadIdx.x & 63;
    // Stores go through a resource over the row's 16-token slab, with the
    // agent-coherence bit.
    auto slab_rsrc = [](uint8_t* p) {
        return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, Cfg<DT, D, B>::kSlabBytes, kBufferWord3);
    };
    const int Hkv = a.num_kv_heads;
    const int rows = a.num_seqs * Hkv;
    const int r0 = wi * RPW;
    if (r0 >= rows) return;

    // Byte offset of row `row`'s slab in either pool and the token's place in
    // it, or -1 when the row has nothing to store.
    auto locate = [&](int row, int& tt, int& pos) -> int64_t {
        if (row >= rows) return -1;
        const int sq = row / Hkv, g = row % Hkv;
        const int L = clamp_ctx(a.context_lens[sq], B, a.max_blocks);
        if (L == 0) return -1;
        pos = L - 1;
        const int pl = a.block_tables[(size_t)sq * a.max_blocks + pos / B];
        if ((unsigned)pl >= (unsigned)a.num_blocks) return -1;
        tt = pos % 16;
        return ((int64_t)pl * Hkv + g) * C::kTileBytes + (int64_t)((pos % B) / 16) * C::kSlabBytes;
    };

    // Loads first, so they are all in flight together.
    const uint8_t* kn = a.k_new + (size_t)r0 * (D * E);
    const uint8_t* vn = a.v_new + (size_t)r0 * (D * E);
    const int kq = lane / KP, ki = lane % KP;
    uint4 kv = make_uint4(0, 0, 0, 0);
    if (r0 + kq < rows) kv = *reinterpret_cast<const uint4*>(kn + (size_t)lane * 16);
    uint32_t vv[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        vv[k] = 0;
        if (r0 + 64 * k / D < rows)
            vv[k] = E == 2 ? (uint32_t)reinterpret_cast<const uint16_t*>(vn)[64 * k + lane]
                           : reinterpret_cast<const uint32_t*>(vn)[64 * k + lane];
    }

    // K: lane (kq, ki) holds piece ki of row r0 + kq.  With the rotary
    // embedding, piece ki pairs with piece ki ^ KP/2 (dims i and i + D/2) of
    // the same row, in lane lane ^ KP/2.
    {
        int tt = 0, pos = 0;
        const int64_t slab = locate(r0 + kq, tt, pos);
        if constexpr (ROPE) {
            uint4 pv;
            pv.x = __shfl_xor(kv.x, KP / 2);
            pv.y = __shfl_xor(kv.y, KP / 2);
            pv.z = __shfl_xor(kv.z, KP / 2);
            pv.w = __shfl_xor(kv.w, KP / 2);
            const bool lo = ki < KP / 2;
            uint4 pr[2] = {lo ? kv : pv, lo ? pv : kv};  // (dims i, dims i + D/2)
            constexpr int X = 16 / E;
            float x[X], y[X];
            piece_to_float<DT>(pr[0], x);
            piece_to_float<DT>(pr[1], y);
#pragma unroll
            for (int j = 0; j < X; ++j) {
                float c, sn;
                rope_cs(rw[(ki % (KP / 2)) * X + j], pos, c, sn);
                rope_rot(x[j], y[j], c, sn);
            }
            kv = lo ? float_to_piece<DT>(x) : float_to_piece<DT>(y);
        }
        if (slab >= 0)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, kv), slab_rsrc(a.k_cache_w + slab),
                                                   (ki * 16 + tt) * 16, 0, kCoherentPolicy);
    }
    // V: element k of the lane is dim (64k) % D + lane of row r0 + 64k / D.
    constexpr int Y = 4 / E;
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        int tt = 0, pos = 0;
        const int64_t slab = locate(r0 + q, tt, pos);
        if (slab < 0) continue;
#pragma unroll
        for (int k = q * D / 64; k < (q + 1) * D / 64; ++k) {
            const int d = (64 * k) % D + lane;
            const int e = ((((tt / 4) * (D / (16 * Y)) + d / (16 * Y)) * 16 + d % 16) * Y + (d / 16) % Y) * 4 + tt % 4;
            if constexpr (E == 2)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)vv[k], slab_rsrc(a.v_cache_w + slab), e * 2, 0,
                                                      kCoherentPolicy);
            else
                __builtin_amdgcn_raw_buffer_store_b32(vv[k], slab_rsrc(a.v_cache_w + slab), e * 4, 0,
                                                      kCoherentPolicy);
        }
    }
}

// Static LDS of a decode workgroup: the per-wave totals of the length prefix
// and the rotary frequencies.  The merge areas, one per wave, follow the
// length arrays in the dynamic part (decode_len_words 32-bit words, a
// multiple of 4 so that the areas start on a 16-byte boundary).
constexpr size_t kDecodeStaticLds = sizeof(int32_t) * kMaxSlice + sizeof(double) * kMaxRopePairs;
__host__ __device__ inline int decode_len_words(int num_seqs, bool multi) {
    return (2 * num_seqs + 1 + (multi ? 2 * num_seqs : 0) + 3) & ~3;
}

#ifndef PA_MIN_WAVES_PER_SIMD
#define PA_MIN_WAVES_PER_SIMD 1
#endif

// One launch: workgroups [0, num_workers) are the workers of the split, each
// with `slice` waves; with the append fused in, the workgroups after them
// store the new K/V rows.
template <int DT, int D, int B, int MODE>
__global__ __launch_bounds__(kGroupThreads, PA_MIN_WAVES_PER_SIMD) void decode_kernel(DecodeArgs a) {
    using C = Cfg<DT, D, B>;
    constexpr bool APPEND = mode_appends(MODE), MQ = MODE == kModeMulti;
    // ctx[num_seqs], pre[num_seqs + 1]; several query tokens: row0[num_seqs], rows[num_seqs];
    // then the merge areas.
    extern __shared__ __attribute__((aligned(16))) int32_t s_lds[];
    __shared__ int32_t s_wave_tot[kMaxSlice];
    // Rotary frequencies in LDS: lanes index them by their own dims, and a
    // lane-dependent index into the argument block would copy it to scratch.
    constexpr bool ROPE = MODE == kModeAppendRope;
    __shared__ double s_rope_w[ROPE ? kMaxRopePairs : 1];
    if constexpr (ROPE) {
        if (threadIdx.x == 0) {  // one lane, constant indices: scalar loads of the argument block
#pragma unroll
            for (int i = 0; i < kMaxRopePairs; ++i) s_rope_w[i] = a.rope_w[i];
        }
        __syncthreads();
    }
    const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave in the workgroup
    if constexpr (APPEND) {
        if ((int)blockIdx.x >= a.attn_groups) {
            store_new_rows<DT, D, B, ROPE>(a, (blockIdx.x - a.attn_groups) * (blockDim.x >> 6) + wi, s_rope_w);
            return;
        }
    }
    int32_t* s_ctx = s_lds;
    int32_t* s_pre = s_lds + a.num_seqs;
    int32_t* s_row0 = s_pre + a.num_seqs + 1;
    int32_t* s_rows = s_row0 + a.num_seqs;
    MergeLds* s_merge = reinterpret_cast<MergeLds*>(s_lds + decode_len_words(a.num_seqs, MQ));
    load_lengths<B, MQ>(a, s_ctx, s_pre, s_row0, s_rows, s_wave_tot);

    const int lane = threadIdx.x & 63;
    if ((int)blockIdx.x >= a.num_workers) return;
    // This worker.  Workgroup b runs on XCD b % 8; numbering the workers so that
    // each XCD holds consecutive ranges keeps the two parts of a pair cut at a
    // range boundary on one XCD (measured: 0.3-0.8 us off every workload).
    const int g = [&]() {
        const int per = a.num_workers / kXcds, extra = a.num_workers % kXcds;
        const int x = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
        return (x < extra ? x * (per + 1) : extra * (per + 1) + (x - extra) * per) + i;
    }();
    const int S = a.num_seqs, Hkv = a.num_kv_heads, G = a.group;
    const int W = a.num_workers, hs = a.slice, hc = a.chunks;
    const int wid = g * hs + wi;  // this wave among all workers' waves

    // Query rows with no context get out = 0; wave wid takes the pairs z = wid (mod W * hs).
    for (int z = wid; z < S * Hkv; z += W * hs) {
        const int s = z / Hkv, kvh = z % Hkv;
        if (s_ctx[s] != 0) continue;
        const int nrows = MQ ? s_rows[s] : 1;
        for (int i = 0; i < nrows; ++i) {
            uint8_t* orow = a.out + col_offset<MQ>(a, s, kvh, MQ ? s_row0[s] : 0, i * G, D) * C::kElt;
            for (int k = lane; k < G * D * C::kElt / 16; k += kWave)
                reinterpret_cast<uint4*>(orow)[k] = make_uint4(0, 0, 0, 0);
        }
    }

    const int64_t U = (int64_t)__builtin_amdgcn_readfirstlane(s_pre[S]) * hc;  // uniform: a scalar loop
    int64_t start, end;
    if (a.per_segment) {
        if (g >= S * hc) return;
        const int s = g / hc, c = g % hc;
        const int nb = s_pre[s + 1] - s_pre[s];
        start = (int64_t)s_pre[s] * hc + (int64_t)c * nb;
        end = start + nb;
    } else {
        start = (int64_t)g * U / W;
        end = (int64_t)(g + 1) * U / W;
    }
    // The worker's runs in unit order, one at a time; a range that ends inside
    // a pair's leading units holds no block and is skipped.
    int64_t u = start;
    auto next_run = [&](Run& run) -> bool {
      while (u < end) {
        // Every lane holds the same values; readfirstlane lets them live in scalar registers.
        const int s = __builtin_amdgcn_readfirstlane(find_seq(s_pre, S, (int)(u / hc)));
        const int base = __builtin_amdgcn_readfirstlane(s_pre[s]);
        const int nbv = __builtin_amdgcn_readfirstlane(s_pre[s + 1]) - base;  // units of each slice
        const int ctx = __builtin_amdgcn_readfirstlane(s_ctx[s]);
        const int nb = (ctx + B - 1) / B;  // its blocks
        const int cost = nbv - nb;         // its leading units that hold no block
        const int off = (int)(u - (int64_t)base * hc);
        const int c = off / nbv, jv0 = off % nbv;
        const int kvh = c * hs + wi;  // this wave's kv-head
        const int64_t left = end - u;
        const int jv1 = left < (int64_t)(nbv - jv0) ? jv0 + (int)left : nbv;
        const int j0 = jv0 > cost ? jv0 - cost : 0, j1 = jv1 - cost;
        const int64_t Fv = (int64_t)base * hc + (int64_t)c * nbv;  // the (sequence, slice)'s first unit
        const int row0 = MQ ? __builtin_amdgcn_readfirstlane(s_row0[s]) : 0;
        const int rows = MQ ? __builtin_amdgcn_readfirstlane(s_rows[s]) : 1;
        const int slot = u == start ? 0 : 1;
        u += jv1 - jv0;
        if (j1 > j0) {
            run = Run{s, kvh, ctx, row0, rows, j0, j1, nb, slot, Fv + cost, Fv};
            return true;
        }
      }
      return false;
    };
    // Each run after the first starts from what the run before it prefetched.
    // (Measured: 1.7 us off the ragged 256-sequence decode, none elsewhere; with
    // the append's registers on top it made the fused step slower, so only the
    // plain decode does it, and only for 16-bit caches: a third f32 tile of
    // 128-dim rows does not fit beside the ring without spilling.)
    constexpr bool PF = PA_PREFETCH_RUNS && MODE == kModeDecode && DT != PA_F32;
    Prefetch<DT, D, B> pf;
    Run cur{};
    bool have = next_run(cur);
    if constexpr (PF) {
        if (have)
            prefetch_run<DT, D, B, MQ>(a, cur, ((ScalarPtr)(a.block_tables + (size_t)cur.s * a.max_blocks))[cur.j0],
                                       pf);
    }
    while (have) {
        Run nx{};
        const bool more = next_run(nx);
        attend_run<DT, D, B, MODE, PF>(a, cur, more, nx, pf, U, W, wid, hs, wi, s_merge[wi], s_rope_w);
        cur = nx;
        have = more;
    }
}

// ---------------------------------------------------------------- prompt chunks

// Causal attention of many query tokens of a sequence at once (a prompt split
// into chunks that run beside decode steps: ForgeLLM README, feature list and
// the paragraph under its architecture flowchart).  A workgroup takes one
// (sequence, kv-head, block of query tokens): NT matrix-core column tiles of
// tpc tokens x G heads, so every K/V tile feeds NT QK and NT PV products.  Its
// four waves hold the same columns and split the positions those tokens see
// into four contiguous ranges of 16-token tiles, each read once, with the
// online softmax of the split path per column; the four partial states are
// merged through LDS at the end (the same log-sum-exp identity as the split
// merge).  The grid is persistent, as many workgroups per compute unit as
// stay resident (chunk_occupancy): each builds
// the per-sequence prefix of item counts in LDS once and then takes items
// from counters in the workspace's synchronisation words, one per XCD (the
// last workgroup to finish puts them back to zero).  Sequences with at most chunk_min
// tokens are left to decode_kernel's several-token mode.
constexpr int kChunkThreads = 256;
constexpr int kChunkWaves = kChunkThreads / kWave;

#ifndef PA_CHUNK_TILES
#define PA_CHUNK_TILES 0  // 0: by row size
#endif
#ifndef PA_CHUNK_REUSE
#define PA_CHUNK_REUSE 1  // K/V loads without the non-temporal hint (query blocks share them in L2)
#endif
#ifndef PA_CHUNK_OCC
#define PA_CHUNK_OCC 0  // resident workgroups per compute unit; 0: by row size
#endif
// Column tiles per workgroup and resident workgroups per compute unit: as many
// tiles as fit, beside the K/V tile ring, in the registers of two waves per
// SIMD (one wave per SIMD cannot overlap one wave's matrix products, softmax
// and load waits: on the Llama-3-8B-shaped prompt chunks, 4 tiles at one wave
// per SIMD took 235 us, 2 tiles at two 179 us).  f32 rows of 128 dims leave
// room for two tiles at one wave per SIMD only.
template <int DT, int D>
constexpr int chunk_tiles() {
    return PA_CHUNK_TILES > 0 ? PA_CHUNK_TILES : (D * (DT == PA_F32 ? 4 : 2) <= 128 ? 4 : 2);
}
template <int DT, int D>
constexpr int chunk_occupancy() {
    return PA_CHUNK_OCC > 0 ? PA_CHUNK_OCC : (D * (DT == PA_F32 ? 4 : 2) <= 256 ? 2 : 1);
}

// Query rows of sequence i (query_start clamped into [0, num_q_rows]).
__device__ inline void query_rows(const DecodeArgs& a, int i, int& q0, int& nq) {
    q0 = min(max(a.query_start[i], 0), a.num_q_rows);
    nq = min(max(a.query_start[i + 1], q0), a.num_q_rows) - q0;
}

// The attention of one item: sequence s, kv-head g, query block qb.  REUSE:
// other query blocks of the sequence read the same K/V (plain loads, kept in
// L2); otherwise the loads carry the non-temporal hint, as in the decode.
template <int DT, int D, int B, bool REUSE>
__device__ __attribute__((always_inline)) void chunk_item(const DecodeArgs& a, int s, int g, int qb, int q0, int nq,
                                                          int L, f32x4 (*s_o)[Cfg<DT, D, B>::kVChunk][kWave],
                                                          float (*s_m)[kWave], float (*s_l)[kWave],
                                                          unsigned long long* ctr, int lo_item, int32_t* s_item) {
    using C = Cfg<DT, D, B>;
    constexpr int E = C::kElt;
    constexpr int NT = chunk_tiles<DT, D>();
    constexpr float kLazy = 8.f;
    const int lane = threadIdx.x & 63, n = lane & 15, r = lane >> 4;
    const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.group, tpc = a.tpc;
    const int QB = NT * tpc;  // query tokens of a workgroup
    const int i_begin = qb * QB;  // the item's first token
    const int ntok = min(QB, nq - i_begin);

    // Per column tile: the lane's token (padding columns and tokens past the
    // sequence's take the tile's first column, or the block's first token:
    // same scores, never stored), the last position it sees, and its Q pieces.
    const bool col_real = n < tpc * G;
    int lim[NT];
    uint4 qf[NT][C::kKFrag];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const int first = min(i_begin + ct * tpc, nq - 1);
        const int t = col_real ? first + n / G : first;
        const bool ok = col_real && t < nq;
        const int tk = ok ? t : first;
        lim[ct] = L - nq + tk;
        const int h = ok ? n % G : 0;
        const uint8_t* qrow = a.q + ((size_t)(q0 + tk) * a.num_q_heads + g * G + h) * (size_t)(D * E);
#pragma unroll
        for (int f = 0; f < C::kKFrag; ++f) qf[ct][f] = *reinterpret_cast<const uint4*>(qrow + 64 * f + 16 * r);
    }
    // Positions the block's tokens see: tiles [0, T); this wave takes
    // [tau_lo, tau_hi).  Tiles before tau_mask are seen whole by every column.
    const int lim_last = L - nq + i_begin + ntok - 1;
    const int lim_first = L - nq + i_begin;
    const int T = lim_last >= 0 ? lim_last / 16 + 1 : 0;
    const int tau_lo = wi * T / kChunkWaves, tau_hi = (wi + 1) * T / kChunkWaves;
    const int tau_mask = lim_first >= 0 ? (lim_first + 1) / 16 : 0;
    const int nblk = (T + C::kSub - 1) / C::kSub;

    f32x4 O[NT][C::kVChunk];
    float m[NT], lsum[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
        for (int c = 0; c < C::kVChunk; ++c) O[ct][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[ct] = -INFINITY;
        lsum[ct] = 0.f;
    }

    const ScalarPtr bt = (ScalarPtr)(a.block_tables + (size_t)s * a.max_blocks);
    int next_id = tau_lo < tau_hi ? bt[tau_lo / C::kSub] : 0;
    int phys = 0;
    auto issue = [&](int tau, Tile<DT, D, B>& t) {
        const int j = tau / C::kSub, u = tau % C::kSub;
        if (u == 0 || tau == tau_lo) {
            phys = ((unsigned)next_id < (unsigned)a.num_blocks) ? next_id : 0;
            if (j + 1 < nblk) next_id = bt[j + 1];
        }
        load_tile<DT, D, B, REUSE && (bool)PA_CHUNK_REUSE>(a, phys, g, u, t);
    };
    // One tile: all NT score tiles first (independent products the matrix core
    // can overlap), then the softmax of every column with one rarely taken
    // branch for the rescales, then all NT PV products.  Only the tiles from
    // tau_mask on hold positions some column must not see (past its token, or
    // past the context); the others take the form without masks (`partial`
    // false), where every score is finite and so is the running maximum after
    // the first tile.
    auto consume = [&](int tau, Tile<DT, D, B>& t, auto partial_tag) {
        constexpr bool partial = decltype(partial_tag)::value;
        const int tok0 = 16 * tau + 4 * r;  // position of this lane's first row
        f32x4 sc[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            sc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int f = 0; f < C::kKFrag; ++f) sc[ct] = qk_step<DT>(t.k[f], qf[ct][f], sc[ct]);
        }
        if constexpr (partial) {
#pragma unroll
            for (int c = 0; c < C::kVPiece; ++c) mask_v<E>(t.v[c], tok0, L);
        }
        float z[NT][4], tmax[NT];
        bool up = false;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[ct][e] = sc[ct][e] * a.scale_log2;
                if constexpr (partial) {
                    if (tok0 + e > lim[ct]) z[ct][e] = -INFINITY;
                }
            }
            tmax[ct] = row_group_max(fmaxf(fmaxf(z[ct][0], z[ct][1]), fmaxf(z[ct][2], z[ct][3])));
            up = up || tmax[ct] > m[ct] + kLazy;
        }
        if (__builtin_amdgcn_read_exec() & __ballot(up)) {
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const float m_new = fmaxf(m[ct], tmax[ct]);
                if (m_new > m[ct] + kLazy) {
                    const float alpha = __builtin_amdgcn_exp2f(m[ct] - m_new);  // 0 while m is -inf
                    lsum[ct] *= alpha;
#pragma unroll
                    for (int c = 0; c < C::kVChunk; ++c) O[ct][c] *= alpha;
                    m[ct] = m_new;
                }
            }
        }
        PPack<DT> pp[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (partial)
                    p[e] = (z[ct][e] > -INFINITY) ? __builtin_amdgcn_exp2f(z[ct][e] - m[ct]) : 0.f;
                else
                    p[e] = __builtin_amdgcn_exp2f(z[ct][e] - m[ct]);
            }
            lsum[ct] += (p[0] + p[1]) + (p[2] + p[3]);
            pp[ct] = pack_p<DT>(p);
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
#pragma unroll
            for (int c = 0; c < C::kVPiece; ++c) pv_piece<DT>(t.v[c], pp[ct], &O[ct][c * (4 / E)]);
        }
    };

    // Two tiles in registers: the next one's loads are in flight while one is
    // consumed.  Every step issues a load (the last tile again at the very
    // end, unused), so no load sits under a branch.
    // Pairs of tiles that lie before tau_mask take the form without masks; the
    // rest (the masked form is exact for any tile) follow in the same ring.
    Tile<DT, D, B> buf[2];
    if (tau_lo < tau_hi) {
        issue(tau_lo, buf[0]);
        int tau = tau_lo;
        for (; tau + 1 < tau_mask && tau + 1 < tau_hi; tau += 2) {
            issue(tau + 1, buf[1]);
            consume(tau, buf[0], std::false_type{});
            issue(min(tau + 2, tau_hi - 1), buf[0]);
            consume(tau + 1, buf[1], std::false_type{});
        }
        for (; tau + 1 < tau_hi; tau += 2) {
            issue(tau + 1, buf[1]);
            consume(tau, buf[0], std::true_type{});
            issue(min(tau + 2, tau_hi - 1), buf[0]);
            consume(tau + 1, buf[1], std::true_type{});
        }
        if (tau < tau_hi) consume(tau, buf[0], std::true_type{});
    }
    wait_vmem_done();

    // The workgroup's next item is claimed now, so that the claim's round trip
    // overlaps the merge below; it is published with the merge's last barrier.
    unsigned long long nxt = 0;
    if (threadIdx.x == 0) nxt = atomicAdd(ctr, 1ull);

    // Merge the four waves' states, one column tile at a time: waves 1..3 put
    // theirs in LDS, wave 0 combines them with its own and stores the output.
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        if (wi > 0) {
#pragma unroll
            for (int c = 0; c < C::kVChunk; ++c) s_o[wi - 1][c][lane] = O[ct][c];
            s_m[wi - 1][lane] = m[ct];
            s_l[wi - 1][lane] = lsum[ct];
        }
        __syncthreads();
        if (wi == 0) {
            float M = m[ct];
#pragma unroll
            for (int w = 0; w < kChunkWaves - 1; ++w) M = fmaxf(M, s_m[w][lane]);
            // (M is -inf only for a column that sees no position: nq > L)
            const float a0 = M > -INFINITY ? __builtin_amdgcn_exp2f(m[ct] - M) : 0.f;
            float l = lsum[ct] * a0;
            f32x4 acc[C::kVChunk];
#pragma unroll
            for (int c = 0; c < C::kVChunk; ++c) acc[c] = O[ct][c] * a0;
#pragma unroll
            for (int w = 0; w < kChunkWaves - 1; ++w) {
                const float aw = M > -INFINITY ? __builtin_amdgcn_exp2f(s_m[w][lane] - M) : 0.f;
                l += s_l[w][lane] * aw;
#pragma unroll
                for (int c = 0; c < C::kVChunk; ++c) acc[c] += s_o[w][c][lane] * aw;
            }
            l = row_group_sum(l);
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const int t = i_begin + ct * tpc + n / G;
            if (col_real && t < nq) {
                uint8_t* orow = a.out + ((size_t)(q0 + t) * a.num_q_heads + g * G + n % G) * (size_t)(D * E);
#pragma unroll
                for (int c = 0; c < C::kVChunk; ++c) store4<DT>(orow + (16 * c + 4 * r) * E, acc[c] * inv);
            }
        }
        if (ct == NT - 1 && threadIdx.x == 0) *s_item = lo_item + (int)nxt;
        __syncthreads();
    }
}

template <int DT, int D, int B>
__global__ __launch_bounds__(kChunkThreads, (chunk_occupancy<DT, D>())) void chunk_kernel(DecodeArgs a) {
    using C = Cfg<DT, D, B>;
    constexpr int NT = chunk_tiles<DT, D>();
    // The merge area: waves 1..3 hand one column tile's state to wave 0 at a time.
    __shared__ f32x4 s_o[kChunkWaves - 1][C::kVChunk][kWave];
    __shared__ float s_m[kChunkWaves - 1][kWave], s_l[kChunkWaves - 1][kWave];
    __shared__ int32_t s_wave_tot[kChunkWaves];
    __shared__ int32_t s_item;
    extern __shared__ __attribute__((aligned(16))) int32_t s_pre[];  // [num_seqs + 1]: items before sequence s
    int32_t* s_q0 = s_pre + a.num_seqs + 1;  // [num_seqs + 1]: first query row (clamped)
    int32_t* s_len = s_q0 + a.num_seqs + 1;  // [num_seqs]: context length (clamped)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = a.num_seqs, Hkv = a.num_kv_heads, QB = NT * a.tpc;
    // Items of a sequence: its query blocks times the kv-heads, when it has
    // more than chunk_min tokens.  Exclusive prefix over sequences into LDS,
    // beside each sequence's first query row and length, so that an item
    // starts from LDS rather than from memory.
    auto items_of = [&](int i) {
        int q0, nq;
        query_rows(a, i, q0, nq);
        return nq > a.chunk_min ? (nq + QB - 1) / QB * Hkv : 0;
    };
    const int per = (S + kChunkThreads - 1) / kChunkThreads;
    const int lo = min(S, tid * per), hi = min(S, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) {
        int q0, nq;
        query_rows(a, i, q0, nq);
        s_q0[i] = q0;
        s_len[i] = clamp_ctx(a.context_lens[i], B, a.max_blocks);
        sum += items_of(i);
    }
    if (tid == 0) s_q0[S] = min(max(a.query_start[S], 0), a.num_q_rows);
    int x = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wave_tot[wave] = x;
    __syncthreads();
    int run = x - sum;
    for (int w = 0; w < wave; ++w) run += s_wave_tot[w];
    for (int i = lo; i < hi; ++i) {
        s_pre[i] = run;
        run += items_of(i);
    }
    if (tid == kChunkThreads - 1) s_pre[S] = run;
    __syncthreads();
    const int nitems = s_pre[S];

    // Items in order (sequence, kv-head, query block).  The items are cut into
    // kXcds contiguous ranges, one per XCD (workgroups are dealt to the XCDs in
    // turn, blockIdx % kXcds), each with a counter in the synchronisation words:
    // a workgroup takes items from its own XCD's range, so the blocks of one
    // (sequence, kv-head) run side by side and share K/V in that XCD's L2; when
    // its range is used up it takes what is left of the others'.
    static_assert(kXcds + 1 <= kSyncHeader, "the counters lie in the header of the synchronisation words");
    unsigned long long* counter = a.sync;  // [kXcds] item counters, then the count of workgroups done
    const int home = (int)(blockIdx.x % kXcds);
    for (int v = 0; v < kXcds; ++v) {
        const int x = (home + v) % kXcds;
        const int lo_item = (int)((int64_t)nitems * x / kXcds), hi_item = (int)((int64_t)nitems * (x + 1) / kXcds);
        if (tid == 0) s_item = lo_item + (int)atomicAdd(counter + x, 1ull);
        __syncthreads();
        for (;;) {
            const int item = __builtin_amdgcn_readfirstlane(s_item);
            __syncthreads();
            if (item >= hi_item) break;
            const int s = __builtin_amdgcn_readfirstlane(find_seq(s_pre, S, item));
            const int nqb = (s_pre[s + 1] - s_pre[s]) / Hkv;
            const int local = item - s_pre[s];
            const int q0 = __builtin_amdgcn_readfirstlane(s_q0[s]);
            const int nq = max(__builtin_amdgcn_readfirstlane(s_q0[s + 1]), q0) - q0;
            const int L = __builtin_amdgcn_readfirstlane(s_len[s]);
            if (nqb > 1)
                chunk_item<DT, D, B, true>(a, s, local / nqb, local % nqb, q0, nq, L, s_o, s_m, s_l, counter + x,
                                           lo_item, &s_item);
            else
                chunk_item<DT, D, B, false>(a, s, local / nqb, local % nqb, q0, nq, L, s_o, s_m, s_l, counter + x,
                                            lo_item, &s_item);
        }
    }
    // The last workgroup out puts the counters (and the count) back to zero.
    if (tid == 0) {
        if (atomicAdd(counter + kXcds, 1ull) + 1 == gridDim.x) {
#pragma unroll
            for (int x = 0; x <= kXcds; ++x) atomicExch(counter + x, 0ull);
        }
    }
}

// ---------------------------------------------------------------- KV append

struct WriteArgs {
    const uint8_t* k_new;
    const uint8_t* v_new;
    const int64_t* slots;
    uint8_t* k_cache;
    uint8_t* v_cache;
    int64_t pool_slots;  // num_blocks * block_size
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
};

// One workgroup per token.  K moves in 16-byte pieces (a piece of a row is
// contiguous in the pool); V moves element by element into its slab.
template <int ELT>
__global__ __launch_bounds__(kWriteThreads) void write_kernel(WriteArgs a) {
    const int i = blockIdx.x;
    const int64_t slot = a.slots[i];
    if (slot < 0 || slot >= a.pool_slots) return;
    const int B = a.block_size, Hkv = a.num_kv_heads, D = a.head_dim;
    const int64_t p = slot / B;
    const int o = (int)(slot % B);
    const int pieces = D * ELT / 16;
    const int slabs = B / 16, sl = o / 16, os = o % 16;
    // K slab: the 16-byte piece dc of token t at (dc*16 + t)*16 bytes.
    for (int c = threadIdx.x; c < Hkv * pieces; c += kWriteThreads) {
        const int g = c / pieces, dc = c % pieces;
        const uint4 v = *reinterpret_cast<const uint4*>(a.k_new + ((size_t)i * Hkv + g) * (size_t)(D * ELT) + dc * 16);
        const size_t slab = ((size_t)p * Hkv + g) * slabs + sl;
        *reinterpret_cast<uint4*>(a.k_cache + ((slab * pieces + dc) * 16 + os) * 16) = v;
    }
    // V slab: element (t, d) at ((((t/4)*(D/16Y) + d/16Y)*16 + d%16)*Y + (d/16)%Y)*4 + t%4, Y = 4/ELT.
    using U = typename std::conditional<ELT == 4, uint32_t, uint16_t>::type;
    constexpr int Y = 4 / ELT;
    for (int e = threadIdx.x; e < Hkv * D; e += kWriteThreads) {
        const int g = e / D, d = e % D;
        const U v = reinterpret_cast<const U*>(a.v_new)[((size_t)i * Hkv + g) * D + d];
        const size_t slab = ((size_t)p * Hkv + g) * slabs + sl;
        const int in_slab = ((((os / 4) * (D / (16 * Y)) + d / (16 * Y)) * 16 + d % 16) * Y + (d / 16) % Y) * 4 + os % 4;
        reinterpret_cast<U*>(a.v_cache)[slab * 16 * D + in_slab] = v;
    }
}

// ---------------------------------------------------------------- rotary embedding, standalone

struct RopeArgs {
    uint8_t* q;
    uint8_t* k;
    const int32_t* positions;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    double w[kMaxRopePairs];
};

// One workgroup per token; thread j rotates pair j % (D/2) of head j / (D/2),
// over the q heads and then the k heads, in place.
template <int DT>
__global__ __launch_bounds__(kWriteThreads) void rope_kernel(RopeArgs a) {
    constexpr int E = DT == PA_F32 ? 4 : 2;
    const int t = blockIdx.x, D = a.head_dim, half = D / 2;
    const int pos = a.positions[t];
    const int pairs = (a.num_q_heads + a.num_kv_heads) * half;
    for (int j = threadIdx.x; j < pairs; j += kWriteThreads) {
        const int h = j / half, i = j % half;
        uint8_t* row = h < a.num_q_heads ? a.q + ((size_t)t * a.num_q_heads + h) * (size_t)(D * E)
                                         : a.k + ((size_t)t * a.num_kv_heads + (h - a.num_q_heads)) * (size_t)(D * E);
        float x, y;
        if constexpr (DT == PA_BF16) {
            x = (float)reinterpret_cast<const __bf16*>(row)[i];
            y = (float)reinterpret_cast<const __bf16*>(row)[i + half];
        } else if constexpr (DT == PA_F16) {
            x = (float)reinterpret_cast<const _Float16*>(row)[i];
            y = (float)reinterpret_cast<const _Float16*>(row)[i + half];
        } else {
            x = reinterpret_cast<const float*>(row)[i];
            y = reinterpret_cast<const float*>(row)[i + half];
        }
        float c, sn;
        rope_cs(a.w[i], pos, c, sn);
        rope_rot(x, y, c, sn);
        if constexpr (DT == PA_BF16) {
            reinterpret_cast<__bf16*>(row)[i] = (__bf16)x;
            reinterpret_cast<__bf16*>(row)[i + half] = (__bf16)y;
        } else if constexpr (DT == PA_F16) {
            reinterpret_cast<_Float16*>(row)[i] = (_Float16)x;
            reinterpret_cast<_Float16*>(row)[i + half] = (_Float16)y;
        } else {
            reinterpret_cast<float*>(row)[i] = x;
            reinterpret_cast<float*>(row)[i + half] = y;
        }
    }
}

// ---------------------------------------------------------------- host side

// Rotary frequencies theta^(-2i/D) for i < D/2, in double.
bool rope_frequencies(float theta, int D, double* w) {
    if (!std::isfinite(theta) || theta <= 1.f || D / 2 > kMaxRopePairs) return false;
    for (int i = 0; i < D / 2; ++i) w[i] = std::pow((double)theta, -2.0 * i / D);
    return true;
}

std::atomic<int> g_cu_count[64];

pa_status_t cu_count(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    if (dev >= 0 && dev < 64) {
        int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return PA_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
        return PA_ERR_HIP;
    if (dev >= 0 && dev < 64) g_cu_count[dev].store(c, std::memory_order_relaxed);
    *out = c;
    return PA_OK;
}

std::atomic<int> g_lds_limit[64];

// Largest LDS allocation (bytes) one workgroup may make on the current device.
pa_status_t lds_limit(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    if (dev >= 0 && dev < 64) {
        int c = g_lds_limit[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return PA_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || c <= 0)
        return PA_ERR_HIP;
    if (dev >= 0 && dev < 64) g_lds_limit[dev].store(c, std::memory_order_relaxed);
    *out = c;
    return PA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

pa_status_t check_cache(const pa_cache_desc_t* c) {
    if (c == nullptr) return PA_ERR_INVALID_ARG;
    if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0)
        return PA_ERR_INVALID_ARG;
    if (c->dtype != PA_F32 && c->dtype != PA_F16 && c->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (c->block_size != 16 && c->block_size != 32) return PA_ERR_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

struct Plan {
    int workers;  // workgroups of the split
    int slice;    // kv-heads per worker, one wave each
    int chunks;   // num_kv_heads / slice
    int per_segment;
    size_t bytes;
    size_t off_lse;
    size_t off_o;
};

pa_status_t check_decode_shapes(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                                const pa_cache_desc_t* cache) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || num_q_heads <= 0 || max_blocks < 0) return PA_ERR_INVALID_ARG;
    if (num_q_heads % cache->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    const int G = num_q_heads / cache->num_kv_heads;
    if (G > kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (num_seqs > kMaxSeqs) return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_seqs * cache->num_kv_heads * max_blocks >= (int64_t)INT32_MAX) return PA_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks * cache->block_size >= (int64_t)INT32_MAX) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Kv-heads a decode worker takes side by side (one wave each): the largest
// divisor of their count that is at most kMaxSlice.
int head_slice(int num_kv_heads) {
    for (int h = kMaxSlice; h > 1; --h)
        if (num_kv_heads % h == 0) return h;
    return 1;
}

// Worker count and workspace layout; needs the device only for the automatic choice.
// Workspace: the synchronisation words (PA_WORKSPACE_SYNC_BYTES, a fixed size so
// that calls of any shape find them in the same place), then part_lse
// [W * slice][2][cols], then part_o [W * slice][2][cols][D], where cols is a
// pair's column count (G, or tokens x G).
pa_status_t make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks, const pa_cache_desc_t* cache,
                      int32_t num_workers, int cols, Plan* plan) {
    const int Hkv = cache->num_kv_heads, G = cols, D = cache->head_dim;
    *plan = Plan{0, 1, 1, 0, 0, 0, 0};
    plan->slice = head_slice(Hkv);
    plan->chunks = Hkv / plan->slice;
    if (num_workers == -1) {
        plan->workers = num_seqs * plan->chunks;
        plan->per_segment = 1;
        return PA_OK;
    }
    if (num_workers < -1 || num_workers > kMaxWorkers) return PA_ERR_INVALID_ARG;
    int W = num_workers;
    if (W == 0) {
        int cus = 0;
        pa_status_t st = cu_count(&cus);
        if (st != PA_OK) return st;
        // At least kMinBlocksPerWorker blocks per worker, counted on the widest
        // table; but never fewer workers than (sequence, slice) items, since a
        // worker that walks several sequences pays a run start (a Q load and a
        // first tile that waits a full memory latency) for each in turn.
        const int64_t units_bound = (int64_t)num_seqs * plan->chunks * max_blocks;
        int64_t want = (units_bound + kMinBlocksPerWorker - 1) / kMinBlocksPerWorker;
        const int64_t items = (int64_t)num_seqs * plan->chunks;
        if (want < items) want = items;
        const int64_t per_cu = kWavesPerCU / plan->slice;
        const int64_t cap = (int64_t)cus * (per_cu < 1 ? 1 : per_cu);
        W = (int)(want < 1 ? 1 : (want > cap ? cap : want));
    }
    // One arrival word per wave of every range must fit the synchronisation words.
    if ((int64_t)W * plan->slice > kSyncWords - kSyncHeader) return PA_ERR_UNSUPPORTED;
    plan->workers = W;
    const size_t waves = (size_t)W * plan->slice;
    const size_t sync = PA_WORKSPACE_SYNC_BYTES;
    const size_t lse = round_up(sizeof(float) * waves * 2 * G, 256);
    const size_t o = sizeof(float) * waves * 2 * G * D;
    plan->off_lse = sync;
    plan->off_o = sync + lse;
    plan->bytes = sync + lse + o;
    return PA_OK;
}

// Dynamic LDS bytes of one decode workgroup: the per-sequence arrays and a
// merge area per wave.
size_t decode_dynamic_lds(int num_seqs, bool multi, int slice) {
    return sizeof(int32_t) * (size_t)decode_len_words(num_seqs, multi) + sizeof(MergeLds) * (size_t)slice;
}

template <int DT, int D, int B, int MODE>
hipError_t launch_decode(const DecodeArgs& a, const Plan& plan, hipStream_t stream) {
    using C = Cfg<DT, D, B>;
    constexpr bool APPEND = mode_appends(MODE);
    const int groups = plan.workers;
    if (groups == 0) return hipSuccess;
    DecodeArgs args_copy = a;
    args_copy.attn_groups = groups;
    int writer_groups = 0;
    if (APPEND) {
        constexpr int rows_per_wave = 64 / (D * C::kElt / 16);
        const int waves = (a.num_seqs * a.num_kv_heads + rows_per_wave - 1) / rows_per_wave;
        writer_groups = (waves + plan.slice - 1) / plan.slice;
    }
    void* args[] = {&args_copy};
    const size_t lds = decode_dynamic_lds(a.num_seqs, MODE == kModeMulti, plan.slice);
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_kernel<DT, D, B, MODE>),
                           dim3(groups + writer_groups), dim3(kWave * plan.slice), args, lds, stream);
}

template <int DT, int MODE>
hipError_t dispatch_decode(const DecodeArgs& a, const Plan& plan, int D, int B, hipStream_t stream) {
    if (D == 64)
        return B == 16 ? launch_decode<DT, 64, 16, MODE>(a, plan, stream)
                       : launch_decode<DT, 64, 32, MODE>(a, plan, stream);
    return B == 16 ? launch_decode<DT, 128, 16, MODE>(a, plan, stream)
                   : launch_decode<DT, 128, 32, MODE>(a, plan, stream);
}

template <int MODE>
hipError_t dispatch_dtype(const DecodeArgs& a, const Plan& plan, const pa_cache_desc_t* cache, hipStream_t stream) {
    const int D = cache->head_dim, B = cache->block_size;
    switch (cache->dtype) {
        case PA_F32:
            return dispatch_decode<PA_F32, MODE>(a, plan, D, B, stream);
        case PA_F16:
            return dispatch_decode<PA_F16, MODE>(a, plan, D, B, stream);
        default:
            return dispatch_decode<PA_BF16, MODE>(a, plan, D, B, stream);
    }
}

// Query tokens per pair when a sequence has several: as many as fit 16 columns.
int tokens_per_pair(int num_q_heads, const pa_cache_desc_t* cache) {
    const int G = num_q_heads / cache->num_kv_heads;
    return G >= 16 ? 1 : 16 / G;
}

// Query tokens of one chunk_kernel item (its column tiles x tpc).
int chunk_block_tokens(const pa_cache_desc_t* cache, int tpc) {
    const int row_bytes = cache->head_dim * (cache->dtype == PA_F32 ? 4 : 2);
    return (PA_CHUNK_TILES > 0 ? PA_CHUNK_TILES : (row_bytes <= 128 ? 4 : 2)) * tpc;
}

// LDS of one prompt-chunk workgroup: its merge area (static, bounded here from
// above) and the per-sequence prefix, first query rows and lengths (dynamic).
size_t chunk_lds_bytes(int num_seqs, int head_dim) {
    const size_t merge = (size_t)(kChunkWaves - 1) * (head_dim / 16) * kWave * 16 + 2 * (kChunkWaves - 1) * kWave * 4;
    return merge + 256 + sizeof(int32_t) * (size_t)(3 * num_seqs + 2);
}

// The persistent grid: resident workgroups per CU times the CUs, or fewer when
// there are fewer items than that.
template <int DT, int D, int B>
hipError_t launch_chunk(const DecodeArgs& a, int64_t items, int cus, hipStream_t stream) {
    const int grid = (int)std::min<int64_t>(items, (int64_t)cus * chunk_occupancy<DT, D>());
    static_assert(PA_CHUNK_TILES > 0 || chunk_tiles<DT, D>() == (D * (DT == PA_F32 ? 4 : 2) <= 128 ? 4 : 2),
                  "chunk_block_tokens");
    DecodeArgs args_copy = a;
    void* args[] = {&args_copy};
    return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_kernel<DT, D, B>), dim3(grid), dim3(kChunkThreads),
                           args, sizeof(int32_t) * (size_t)(3 * a.num_seqs + 2), stream);
}

hipError_t dispatch_chunk(const DecodeArgs& a, const pa_cache_desc_t* cache, int64_t items, int cus,
                          hipStream_t stream) {
    const int D = cache->head_dim, B = cache->block_size;
#define PA_CHUNK_CASE(DT)                                                                              \
    return D == 64 ? (B == 16 ? launch_chunk<DT, 64, 16>(a, items, cus, stream) : launch_chunk<DT, 64, 32>(a, items, cus, stream)) \
                   : (B == 16 ? launch_chunk<DT, 128, 16>(a, items, cus, stream)                           \
                              : launch_chunk<DT, 128, 32>(a, items, cus, stream));
    switch (cache->dtype) {
        case PA_F32:
            PA_CHUNK_CASE(PA_F32)
        case PA_F16:
            PA_CHUNK_CASE(PA_F16)
        default:
            PA_CHUNK_CASE(PA_BF16)
    }
#undef PA_CHUNK_CASE
}

// Shared by pa_decode_ex, pa_decode_append (mode kModeAppend: k_new/v_new) and
// pa_attend (mode kModeMulti: query_start and max_query_len).
pa_status_t decode_impl(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                        int32_t max_query_len, int32_t num_q_rows, float scale, float rope_theta, void* out,
                        int32_t num_seqs,
                        int32_t num_q_heads, int32_t max_blocks_per_seq, const pa_cache_desc_t* cache,
                        void* workspace, size_t workspace_bytes, int32_t num_workers, int mode,
                        pa_stream_t stream) {
    pa_status_t st = check_decode_shapes(num_seqs, num_q_heads, max_blocks_per_seq, cache);
    if (st != PA_OK) return st;
    const bool append = mode_appends(mode), multi = mode == kModeMulti;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    if (num_workers < -1 || num_workers > kMaxWorkers) return PA_ERR_INVALID_ARG;
    if (multi && (max_query_len < 0 || num_q_rows < 0)) return PA_ERR_INVALID_ARG;
    double rope_w[kMaxRopePairs] = {};
    if (rope_theta != 0.f && !rope_frequencies(rope_theta, cache->head_dim, rope_w)) return PA_ERR_INVALID_ARG;
    // nothing is touched, so empty tensors may pass null pointers
    if (num_seqs == 0 || (multi && (max_query_len == 0 || num_q_rows == 0))) return PA_OK;
    if (!q || !k_cache || !v_cache || !context_lens || !out) return PA_ERR_INVALID_ARG;
    if (max_blocks_per_seq > 0 && !block_tables) return PA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(context_lens, 4) || (block_tables && !aligned(block_tables, 4)))
        return PA_ERR_INVALID_ARG;
    if (append && (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))) return PA_ERR_INVALID_ARG;
    if (multi && (!query_start || !aligned(query_start, 4))) return PA_ERR_INVALID_ARG;
    const int G = num_q_heads / cache->num_kv_heads;
    const int tpc = multi ? tokens_per_pair(num_q_heads, cache) : 1;
    Plan plan;
    st = make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, num_workers, tpc * G, &plan);
    if (st != PA_OK) return st;
    // (several query tokens: chunk_kernel's item counter needs the synchronisation words in any case)
    const size_t need = multi ? std::max(plan.bytes, (size_t)PA_WORKSPACE_SYNC_BYTES) : plan.bytes;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)))
        return PA_ERR_WORKSPACE;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    DecodeArgs a{};
    a.q = static_cast<const uint8_t*>(q);
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = static_cast<uint8_t*>(out);
    a.sync = plan.per_segment ? nullptr : reinterpret_cast<unsigned long long*>(ws);
    a.part_lse = plan.per_segment ? nullptr : reinterpret_cast<float*>(ws + plan.off_lse);
    a.part_o = plan.per_segment ? nullptr : reinterpret_cast<float*>(ws + plan.off_o);
    a.k_new = static_cast<const uint8_t*>(k_new);
    a.v_new = static_cast<const uint8_t*>(v_new);
    a.k_cache_w = static_cast<uint8_t*>(k_cache);
    a.v_cache_w = static_cast<uint8_t*>(v_cache);
    a.scale_log2 = scale * kLog2e;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache->num_kv_heads;
    a.group = num_q_heads / cache->num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = cache->num_blocks;
    a.num_workers = plan.workers;
    a.slice = plan.slice;
    a.chunks = plan.chunks;
    a.per_segment = plan.per_segment;
    a.cols = tpc * G;
    a.query_start = query_start;
    a.num_q_rows = num_q_rows;
    a.tpc = tpc;
    for (int i = 0; i < kMaxRopePairs; ++i) a.rope_w[i] = rope_w[i];
    // A run start costs about as much as streaming kRunCostBytes of K/V: count
    // it as that many units so that workers with many short runs get fewer blocks.
    const size_t unit_bytes = (size_t)cache->block_size * cache->head_dim * (cache->dtype == PA_F32 ? 4 : 2) * 2;
    a.run_cost = plan.per_segment ? 0 : (int32_t)(kRunCostBytes / unit_bytes);

    // LDS of one decode workgroup: lengths and prefix (dynamic) plus the merge areas (static).
    int lds_max = 0;
    st = lds_limit(&lds_max);
    if (st != PA_OK) return st;
    if (decode_dynamic_lds(num_seqs, multi, plan.slice) + kDecodeStaticLds > (size_t)lds_max) return PA_ERR_UNSUPPORTED;
    if (multi && max_query_len > tpc && chunk_lds_bytes(num_seqs, cache->head_dim) > (size_t)lds_max)
        return PA_ERR_UNSUPPORTED;

    hipStream_t sm = static_cast<hipStream_t>(stream);
    if (!multi) {
        if (mode == kModeAppendRope) {
            if (cache->dtype == PA_F32) return PA_ERR_UNSUPPORTED;
            const hipError_t e = cache->dtype == PA_F16
                                     ? dispatch_decode<PA_F16, kModeAppendRope>(a, plan, cache->head_dim,
                                                                                 cache->block_size, sm)
                                     : dispatch_decode<PA_BF16, kModeAppendRope>(a, plan, cache->head_dim,
                                                                                  cache->block_size, sm);
            return e == hipSuccess ? PA_OK : PA_ERR_HIP;
        }
        const hipError_t e = append ? dispatch_dtype<kModeAppend>(a, plan, cache, sm)
                                    : dispatch_dtype<kModeDecode>(a, plan, cache, sm);
        return e == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    // Several query tokens.  Sequences with more tokens than one 16-column tile
    // holds (tpc) go to chunk_kernel, one launch: on the split path they would
    // take one launch, and one pass over their K/V, per group of tpc tokens.
    // The others take the split path, one launch, a pair per 16-column tile.
    a.chunk_min = tpc;
    if (max_query_len > a.chunk_min) {
        // Items: at most (rows / QB + num_seqs) x kv-heads; a workgroup per compute unit.
        const int qb = chunk_block_tokens(cache, tpc);  // an item's query tokens
        const int64_t bound = ((int64_t)num_q_rows / qb + num_seqs) * cache->num_kv_heads;
        if (bound >= (int64_t)INT32_MAX) return PA_ERR_UNSUPPORTED;
        int cus = 0;
        st = cu_count(&cus);
        if (st != PA_OK) return st;
        a.sync = reinterpret_cast<unsigned long long*>(ws);
        if (dispatch_chunk(a, cache, bound, cus, sm) != hipSuccess) return PA_ERR_HIP;
    }
    const int chunks = (std::min(max_query_len, a.chunk_min) + tpc - 1) / tpc;
    for (int c = 0; c < chunks; ++c) {
        a.chunk = c;
        if (dispatch_dtype<kModeMulti>(a, plan, cache, sm) != hipSuccess) return PA_ERR_HIP;
    }
    return PA_OK;
}

// ---------------------------------------------------------------- the allocation-free decode

// The workspace of pa_decode_noalloc: a device array of the library's own, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in); it uses the
// device address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

__global__ __launch_bounds__(256) void zero_words_kernel(uint4* p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = make_uint4(0, 0, 0, 0);
}

// This device's copy of `scratch`, set up on the first call on the device:
// its address, and its synchronisation words cleared by a small kernel on the
// caller's stream (a kernel rather than a memset node, in case the call is
// being captured into a graph).
pa_status_t noalloc_scratch(hipStream_t stream, uint8_t** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (p == nullptr) {
            void* ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return PA_ERR_HIP;
            const int words = PA_WORKSPACE_SYNC_BYTES / 16;
            void* args[] = {&ptr, const_cast<int*>(&words)};
            if (hipLaunchKernel(reinterpret_cast<const void*>(&zero_words_kernel), dim3(words / 256), dim3(256), args,
                                0, stream) != hipSuccess)
                return PA_ERR_HIP;
            p = static_cast<uint8_t*>(ptr);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status_t status) {
    // A caller may pass any integer; read its bits rather than the enum, whose
    // out-of-range values C++ leaves undefined.
    int32_t code = 0;
    static_assert(sizeof(status) == sizeof(code), "pa_status_t is an int");
    std::memcpy(&code, &status, sizeof(code));
    switch (code) {
        case PA_OK:
            return "ok";
        case PA_ERR_INVALID_ARG:
            return "invalid argument";
        case PA_ERR_UNSUPPORTED:
            return "unsupported shape or dtype";
        case PA_ERR_WORKSPACE:
            return "workspace missing or too small";
        case PA_ERR_HIP:
            return "HIP runtime error";
        case PA_ERR_CAPACITY:
            return "block pool capacity exceeded";
    }
    return "unknown status";
}

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

size_t pa_workspace_sync_bytes(void) { return PA_WORKSPACE_SYNC_BYTES; }

pa_status_t pa_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping, void* k_cache,
                        void* v_cache, int32_t num_tokens, const pa_cache_desc_t* cache, pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (num_tokens < 0) return PA_ERR_INVALID_ARG;
    if (num_tokens == 0) return PA_OK;  // nothing is touched, so empty tensors may pass null pointers
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(slot_mapping, 8))
        return PA_ERR_INVALID_ARG;
    WriteArgs a{static_cast<const uint8_t*>(k_new),
                static_cast<const uint8_t*>(v_new),
                slot_mapping,
                static_cast<uint8_t*>(k_cache),
                static_cast<uint8_t*>(v_cache),
                (int64_t)cache->num_blocks * cache->block_size,
                cache->block_size,
                cache->num_kv_heads,
                cache->head_dim};
    void* args[] = {&a};
    const void* fn = cache->dtype == PA_F32 ? reinterpret_cast<const void*>(&write_kernel<4>)
                                            : reinterpret_cast<const void*>(&write_kernel<2>);
    hipError_t e = hipLaunchKernel(fn, dim3(num_tokens), dim3(kWriteThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                    const pa_cache_desc_t* cache, int32_t num_workers) {
    if (check_decode_shapes(num_seqs, num_q_heads, max_blocks_per_seq, cache) != PA_OK) return 0;
    Plan plan;
    const int G = num_q_heads / cache->num_kv_heads;
    if (make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, num_workers, G, &plan) != PA_OK) return 0;
    return plan.bytes;
}

size_t pa_attend_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 const pa_cache_desc_t* cache, int32_t num_workers) {
    if (check_decode_shapes(num_seqs, num_q_heads, max_blocks_per_seq, cache) != PA_OK) return 0;
    Plan plan;
    const int cols = tokens_per_pair(num_q_heads, cache) * (num_q_heads / cache->num_kv_heads);
    if (make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, num_workers, cols, &plan) != PA_OK) return 0;
    return std::max(plan.bytes, (size_t)PA_WORKSPACE_SYNC_BYTES);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 const pa_cache_desc_t* cache) {
    return pa_decode_workspace_bytes_ex(num_seqs, num_q_heads, max_blocks_per_seq, cache, 0);
}

pa_status_t pa_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                         size_t workspace_bytes, int32_t num_workers, pa_stream_t stream) {
    return decode_impl(q, nullptr, nullptr, const_cast<void*>(k_cache), const_cast<void*>(v_cache), block_tables,
                       context_lens, nullptr, 1, num_seqs, scale, 0.f, out, num_seqs, num_q_heads,
                       max_blocks_per_seq, cache, workspace, workspace_bytes, num_workers, kModeDecode, stream);
}

pa_status_t pa_attend(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, const int32_t* query_start, float scale, void* out,
                      int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t max_query_len,
                      int32_t num_q_rows, const pa_cache_desc_t* cache, void* workspace, size_t workspace_bytes,
                      int32_t num_workers, pa_stream_t stream) {
    return decode_impl(q, nullptr, nullptr, const_cast<void*>(k_cache), const_cast<void*>(v_cache), block_tables,
                       context_lens, query_start, max_query_len, num_q_rows, scale, 0.f, out, num_seqs, num_q_heads,
                       max_blocks_per_seq, cache, workspace, workspace_bytes, num_workers, kModeMulti, stream);
}

pa_status_t pa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                             int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                             const pa_cache_desc_t* cache, void* workspace, size_t workspace_bytes,
                             int32_t num_workers, pa_stream_t stream) {
    return decode_impl(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, nullptr, 1, num_seqs, scale,
                       0.f, out, num_seqs, num_q_heads, max_blocks_per_seq, cache, workspace, workspace_bytes,
                       num_workers, kModeAppend, stream);
}

pa_status_t pa_decode_rope_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, float scale,
                                  float rope_theta, void* out, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                                  size_t workspace_bytes, int32_t num_workers, pa_stream_t stream) {
    if (rope_theta == 0.f) return PA_ERR_INVALID_ARG;  // 0 means "no rotation" inside
    if (cache && cache->dtype == PA_F32) return PA_ERR_UNSUPPORTED;  // f32: pa_rope, then pa_decode_append
    return decode_impl(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, nullptr, 1, num_seqs, scale,
                       rope_theta, out, num_seqs, num_q_heads, max_blocks_per_seq, cache, workspace,
                       workspace_bytes, num_workers, kModeAppendRope, stream);
}

pa_status_t pa_rope(void* q, void* k, const int32_t* positions, int32_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype, float rope_theta, pa_stream_t stream) {
    if (num_tokens < 0 || num_q_heads < 0 || num_kv_heads < 0) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    RopeArgs a{};
    if (!rope_frequencies(rope_theta, head_dim, a.w)) return PA_ERR_INVALID_ARG;
    if (num_tokens == 0 || num_q_heads + num_kv_heads == 0) return PA_OK;  // nothing is touched
    if (!positions || !aligned(positions, 4) || (num_q_heads > 0 && (!q || !aligned(q, 16))) ||
        (num_kv_heads > 0 && (!k || !aligned(k, 16))))
        return PA_ERR_INVALID_ARG;
    a.q = static_cast<uint8_t*>(q);
    a.k = static_cast<uint8_t*>(k);
    a.positions = positions;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    void* args[] = {&a};
    const void* fn = dtype == PA_F32   ? reinterpret_cast<const void*>(&rope_kernel<PA_F32>)
                     : dtype == PA_F16 ? reinterpret_cast<const void*>(&rope_kernel<PA_F16>)
                                       : reinterpret_cast<const void*>(&rope_kernel<PA_BF16>);
    hipError_t e = hipLaunchKernel(fn, dim3(num_tokens), dim3(kWriteThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                      size_t workspace_bytes, pa_stream_t stream) {
    return pa_decode_ex(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                        max_blocks_per_seq, cache, workspace, workspace_bytes, 0, stream);
}

pa_status_t pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                              int32_t num_q_heads, int32_t max_blocks_per_seq, const pa_cache_desc_t* cache,
                              pa_stream_t stream) {
    // The plan pa_decode would take; 0 for arguments it rejects (pa_decode_ex then
    // reports why) or when no split needs a workspace.
    const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, max_blocks_per_seq, cache);
    if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
    uint8_t* ws = nullptr;
    if (need > 0 && num_seqs > 0) {
        const pa_status_t st = noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
        if (st != PA_OK) return st;
    }
    return pa_decode_ex(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                        max_blocks_per_seq, cache, ws, ws ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, 0, stream);
}

}  // extern "C"
