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
// Design (one wavefront = one worker):
//  * Work unit = one (sequence, kv-head, logical block).  All units of the
//    batch are laid end to end, sequence-major then kv-head then block, and
//    dealt to the workers in equal contiguous runs ("stream-K"), so every
//    worker streams the same number of blocks whatever the length mix.  A
//    run that covers a whole (sequence, kv-head) writes the output directly;
//    one that covers part of it writes (o, log-sum-exp) and a merge kernel
//    combines the parts.  The split depends only on the lengths and the
//    worker count, so results are bitwise reproducible and independent of
//    physical placement.
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
#include <type_traits>

#include "pagedattn.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kGroupThreads = kWave * kWavesPerGroup;
constexpr int kMaxSeqs = 4096;
constexpr int kMaxGroup = 16;
constexpr int kWorkersPerCU = 8;
constexpr int kMinBlocksPerWorker = 4;
constexpr int kMaxWorkers = 1 << 20;
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
    static constexpr int kSub = B / 16;           // 16-token tiles per block
    static constexpr int kTileBytes = B * D * kElt;
};

template <int ELT>
struct VPiece;  // the V bytes one lane feeds to one PV product: 4 tokens
template <>
struct VPiece<2> {
    using type = uint2;
};
template <>
struct VPiece<4> {
    using type = uint4;
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

// O^T (16 dims x 16 heads) += V^T piece (16 dims x 4k tokens) x P^T.
template <int DT>
__device__ inline f32x4 pv_step(typename VPiece<DT == PA_F32 ? 4 : 2>::type v, PPack<DT> p, f32x4 acc) {
    if constexpr (DT == PA_BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, v), p.v, acc, 0, 0, 0);
    } else if constexpr (DT == PA_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, v), p.v, acc, 0, 0, 0);
    } else {
        f32x4 vf = __builtin_bit_cast(f32x4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[e], p.v[e], acc, 0, 0, 0);
        return acc;
    }
}

// Zero the V entries of tokens at or past the context end (their P is 0, but
// 0 * NaN would still poison the sum).
template <int ELT>
__device__ inline void mask_v(typename VPiece<ELT>::type& v, int first_tok, int ctx) {
    if constexpr (ELT == 2) {
        uint32_t lo = v.x, hi = v.y;
        if (first_tok + 0 >= ctx) lo &= 0xffff0000u;
        if (first_tok + 1 >= ctx) lo &= 0x0000ffffu;
        if (first_tok + 2 >= ctx) hi &= 0xffff0000u;
        if (first_tok + 3 >= ctx) hi &= 0x0000ffffu;
        v.x = lo;
        v.y = hi;
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

// ---------------------------------------------------------------- arguments

struct DecodeArgs {
    const uint8_t* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    uint8_t* out;
    int32_t* seq_prefix;  // [num_seqs + 1] blocks before each sequence, or null
    float* part_lse;      // [workers][2][G]
    float* part_o;        // [workers][2][G][D]
    float scale_log2;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t max_blocks;
    int32_t num_blocks;
    int32_t num_workers;
    int32_t per_segment;  // 1: worker w owns (sequence, kv-head) w entirely
};

__device__ inline int blocks_of(int ctx, int B, int max_blocks) {
    ctx = ctx < 0 ? 0 : ctx;
    int nb = (ctx + B - 1) / B;
    return nb > max_blocks ? max_blocks : nb;
}

__device__ inline int clamp_ctx(int ctx, int B, int max_blocks) {
    ctx = ctx < 0 ? 0 : ctx;
    return ctx > max_blocks * B ? max_blocks * B : ctx;
}

// Exclusive prefix over sequences of their block counts, into LDS [num_seqs + 1].
template <int B>
__device__ void build_prefix(const DecodeArgs& a, int32_t* pre, int32_t* wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = a.num_seqs;
    const int per = (S + kGroupThreads - 1) / kGroupThreads;
    const int lo = min(S, tid * per), hi = min(S, lo + per);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += blocks_of(a.context_lens[i], B, a.max_blocks);
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
        run += blocks_of(a.context_lens[i], B, a.max_blocks);
    }
    if (tid == kGroupThreads - 1) pre[S] = run;
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

// ---------------------------------------------------------------- decode: one run of blocks

template <int DT, int D, int B>
struct Tile {
    uint4 k[Cfg<DT, D, B>::kKFrag];
    typename VPiece<Cfg<DT, D, B>::kElt>::type v[Cfg<DT, D, B>::kVChunk];
};

// Attend query group (s, kvh) over logical blocks [j0, j1) of sequence s.
// whole: the run is the sequence's entire context (write out), otherwise
// write a partial into slot `slot` of worker `w`.
template <int DT, int D, int B>
__device__ void attend_run(const DecodeArgs& a, int s, int kvh, int j0, int j1, bool whole, int w, int slot) {
    using C = Cfg<DT, D, B>;
    constexpr int E = C::kElt;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // this lane's head column (and row within a 16-row piece)
    const int r = lane >> 4;  // this lane's group of 4 rows / k-range
    const int G = a.group;
    const int ctx = __builtin_amdgcn_readfirstlane(clamp_ctx(a.context_lens[s], B, a.max_blocks));

    // Q of the lane's head, in the B-operand form of the QK product.
    uint4 qf[C::kKFrag];
    {
        const int hq = kvh * G + (n < G ? n : 0);
        const uint8_t* qrow = a.q + ((size_t)s * a.num_q_heads + hq) * (size_t)(D * E);
#pragma unroll
        for (int f = 0; f < C::kKFrag; ++f) {
            uint4 v = *reinterpret_cast<const uint4*>(qrow + 64 * f + 16 * r);
            qf[f] = n < G ? v : make_uint4(0, 0, 0, 0);
        }
    }

    f32x4 O[C::kVChunk];
#pragma unroll
    for (int c = 0; c < C::kVChunk; ++c) O[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;  // running max (log2 domain) of this lane's head
    float lsum = 0.f;     // this lane's share of the running denominator

    const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks;
    const size_t blk_stride = (size_t)a.num_kv_heads * C::kTileBytes;
    const size_t head_off = (size_t)kvh * C::kTileBytes;
    const int ntiles = (j1 - j0) * C::kSub;

    int id_base = j0;
    int ids = (j0 + lane < j1) ? bt[j0 + lane] : 0;

    auto issue = [&](int tau, Tile<DT, D, B>& t) {
        const int j = j0 + tau / C::kSub, u = tau % C::kSub;
        if (j - id_base >= kWave) {
            id_base += kWave;
            ids = (id_base + lane < j1) ? bt[id_base + lane] : 0;
        }
        int phys = __builtin_amdgcn_readlane(ids, j - id_base);
        phys = ((unsigned)phys < (unsigned)a.num_blocks) ? phys : 0;
        const uint8_t* kt = a.k_cache + (size_t)phys * blk_stride + head_off;
        const uint8_t* vt = a.v_cache + (size_t)phys * blk_stride + head_off;
#pragma unroll
        for (int f = 0; f < C::kKFrag; ++f)
            t.k[f] = *reinterpret_cast<const uint4*>(kt + ((4 * f + r) * B + 16 * u + n) * 16);
#pragma unroll
        for (int c = 0; c < C::kVChunk; ++c)
            t.v[c] = *reinterpret_cast<const typename VPiece<E>::type*>(vt + ((16 * c + n) * B + 16 * u + 4 * r) * E);
    };

    auto consume = [&](int tau, Tile<DT, D, B>& t) {
        const int j = j0 + tau / C::kSub, u = tau % C::kSub;
        const int tok0 = j * B + 16 * u + 4 * r;  // position of this lane's first row
        const bool partial = j * B + 16 * u + 16 > ctx;

        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < C::kKFrag; ++f) sc = qk_step<DT>(t.k[f], qf[f], sc);

        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = sc[e] * a.scale_log2;
            if (partial && tok0 + e >= ctx) z[e] = -INFINITY;
        }
        float tmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float alpha = (m == m_new) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = (z[e] > -INFINITY) ? __builtin_amdgcn_exp2f(z[e] - m_new) : 0.f;
        lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m = m_new;
#pragma unroll
        for (int c = 0; c < C::kVChunk; ++c) O[c] *= alpha;

        if (partial) {
#pragma unroll
            for (int c = 0; c < C::kVChunk; ++c) mask_v<E>(t.v[c], tok0, ctx);
        }
        const PPack<DT> pp = pack_p<DT>(p);
#pragma unroll
        for (int c = 0; c < C::kVChunk; ++c) O[c] = pv_step<DT>(t.v[c], pp, O[c]);
    };

    Tile<DT, D, B> t0, t1;
    issue(0, t0);
    for (int tau = 0; tau < ntiles; tau += 2) {
        if (tau + 1 < ntiles) issue(tau + 1, t1);
        consume(tau, t0);
        if (tau + 1 < ntiles) {
            if (tau + 2 < ntiles) issue(tau + 2, t0);
            consume(tau + 1, t1);
        }
    }

    // Full denominator of the lane's head: the four row groups hold disjoint tokens.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (n >= G) return;
    const float inv = 1.f / lsum;
    if (whole) {
        uint8_t* orow = a.out + ((size_t)s * a.num_q_heads + kvh * G + n) * (size_t)(D * E);
#pragma unroll
        for (int c = 0; c < C::kVChunk; ++c) store4<DT>(orow + (16 * c + 4 * r) * E, O[c] * inv);
    } else {
        const size_t part = ((size_t)w * 2 + slot) * G + n;
        float* po = a.part_o + part * D;
#pragma unroll
        for (int c = 0; c < C::kVChunk; ++c) *reinterpret_cast<f32x4*>(po + 16 * c + 4 * r) = O[c] * inv;
        if (r == 0) a.part_lse[part] = m + __log2f(lsum);
    }
}

template <int DT, int D, int B>
__global__ __launch_bounds__(kGroupThreads) void decode_kernel(DecodeArgs a) {
    using C = Cfg<DT, D, B>;
    extern __shared__ int32_t s_prefix[];  // [num_seqs + 1]
    __shared__ int32_t s_wave_tot[kWavesPerGroup];
    build_prefix<B>(a, s_prefix, s_wave_tot);
    if (blockIdx.x == 0 && a.seq_prefix != nullptr)
        for (int i = threadIdx.x; i <= a.num_seqs; i += kGroupThreads) a.seq_prefix[i] = s_prefix[i];

    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    if (w >= a.num_workers) return;
    const int S = a.num_seqs, Hkv = a.num_kv_heads, G = a.group;
    const int W = a.num_workers;

    // Sequences with no context get out = 0; worker w takes the pairs z = w (mod W).
    for (int z = w; z < S * Hkv; z += W) {
        const int s = z / Hkv, kvh = z % Hkv;
        if (s_prefix[s + 1] != s_prefix[s]) continue;
        uint8_t* orow = a.out + ((size_t)s * a.num_q_heads + (size_t)kvh * G) * (size_t)(D * C::kElt);
        for (int i = lane; i < G * D * C::kElt / 16; i += kWave)
            reinterpret_cast<uint4*>(orow)[i] = make_uint4(0, 0, 0, 0);
    }

    const int64_t U = (int64_t)s_prefix[S] * Hkv;
    int64_t start, end;
    if (a.per_segment) {
        if (w >= S * Hkv) return;
        const int s = w / Hkv, kvh = w % Hkv;
        const int nb = s_prefix[s + 1] - s_prefix[s];
        start = (int64_t)s_prefix[s] * Hkv + (int64_t)kvh * nb;
        end = start + nb;
    } else {
        start = (int64_t)w * U / W;
        end = (int64_t)(w + 1) * U / W;
    }
    for (int64_t u = start; u < end;) {
        // Every lane holds the same values; readfirstlane lets them live in scalar registers.
        const int s = __builtin_amdgcn_readfirstlane(find_seq(s_prefix, S, (int)(u / Hkv)));
        const int base = __builtin_amdgcn_readfirstlane(s_prefix[s]);
        const int nb = __builtin_amdgcn_readfirstlane(s_prefix[s + 1]) - base;
        const int off = (int)(u - (int64_t)base * Hkv);
        const int kvh = off / nb, j0 = off % nb;
        const int64_t left = end - u;
        const int j1 = left < (int64_t)(nb - j0) ? j0 + (int)left : nb;
        attend_run<DT, D, B>(a, s, kvh, j0, j1, j0 == 0 && j1 == nb, w, u == start ? 0 : 1);
        u += j1 - j0;
    }
}

// ---------------------------------------------------------------- merge of split runs

struct MergeArgs {
    const int32_t* seq_prefix;
    const float* part_lse;
    const float* part_o;
    uint8_t* out;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t num_workers;
};

__device__ inline int64_t run_start(int64_t w, int64_t U, int64_t W) { return w * U / W; }

// The worker whose run holds unit u.
__device__ inline int64_t owner_of(int64_t u, int64_t U, int64_t W) { return ((u + 1) * W + U - 1) / U - 1; }

template <int DT, int D>
__global__ __launch_bounds__(kGroupThreads) void merge_kernel(MergeArgs a) {
    constexpr int E = DT == PA_F32 ? 4 : 2;
    const int z = blockIdx.x;
    const int Hkv = a.num_kv_heads, G = a.group, S = a.num_seqs;
    const int s = z / Hkv, kvh = z % Hkv;
    const int nb = a.seq_prefix[s + 1] - a.seq_prefix[s];
    if (nb == 0) return;
    const int64_t U = (int64_t)a.seq_prefix[S] * Hkv, W = a.num_workers;
    const int64_t first = (int64_t)a.seq_prefix[s] * Hkv + (int64_t)kvh * nb;
    const int64_t last = first + nb - 1;
    const int64_t wa = owner_of(first, U, W), wb = owner_of(last, U, W);
    if (wa == wb) return;  // one worker held the whole context and wrote out

    // Each thread merges 4 consecutive dims of one head across the parts.
    for (int i = threadIdx.x; i < G * D / 4; i += kGroupThreads) {
        const int h = i / (D / 4), d4 = (i % (D / 4)) * 4;
        float M = -INFINITY;
        for (int64_t w = wa; w <= wb; ++w) {
            if (run_start(w, U, W) == run_start(w + 1, U, W)) continue;
            const int slot = (w == wa && run_start(w, U, W) != first) ? 1 : 0;
            M = fmaxf(M, a.part_lse[((size_t)w * 2 + slot) * G + h]);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
        for (int64_t w = wa; w <= wb; ++w) {
            if (run_start(w, U, W) == run_start(w + 1, U, W)) continue;
            const int slot = (w == wa && run_start(w, U, W) != first) ? 1 : 0;
            const size_t part = ((size_t)w * 2 + slot) * G + h;
            const float wt = __builtin_amdgcn_exp2f(a.part_lse[part] - M);
            acc += wt * *reinterpret_cast<const f32x4*>(a.part_o + part * D + d4);
            den += wt;
        }
        uint8_t* dst = a.out + (((size_t)s * a.num_q_heads + kvh * G + h) * D + d4) * E;
        store4<DT>(dst, acc * (1.f / den));
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
// contiguous in the pool); V moves element by element into its transposed tile.
template <int ELT>
__global__ __launch_bounds__(kGroupThreads) void write_kernel(WriteArgs a) {
    const int i = blockIdx.x;
    const int64_t slot = a.slots[i];
    if (slot < 0 || slot >= a.pool_slots) return;
    const int B = a.block_size, Hkv = a.num_kv_heads, D = a.head_dim;
    const int64_t p = slot / B;
    const int o = (int)(slot % B);
    const int pieces = D * ELT / 16;
    for (int c = threadIdx.x; c < Hkv * pieces; c += kGroupThreads) {
        const int g = c / pieces, dc = c % pieces;
        const uint4 v = *reinterpret_cast<const uint4*>(a.k_new + ((size_t)i * Hkv + g) * (size_t)(D * ELT) + dc * 16);
        *reinterpret_cast<uint4*>(a.k_cache + (((size_t)p * Hkv + g) * pieces + dc) * (size_t)(B * 16) + o * 16) = v;
    }
    using U = typename std::conditional<ELT == 4, uint32_t, uint16_t>::type;
    for (int e = threadIdx.x; e < Hkv * D; e += kGroupThreads) {
        const int g = e / D, d = e % D;
        const U v = reinterpret_cast<const U*>(a.v_new)[((size_t)i * Hkv + g) * D + d];
        reinterpret_cast<U*>(a.v_cache)[(((size_t)p * Hkv + g) * D + d) * B + o] = v;
    }
}

// ---------------------------------------------------------------- host side

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
    int workers;
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

// Worker count and workspace layout; needs the device only for the automatic choice.
pa_status_t make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks, const pa_cache_desc_t* cache,
                      int32_t num_workers, Plan* plan) {
    const int Hkv = cache->num_kv_heads, G = num_q_heads / Hkv, D = cache->head_dim;
    *plan = Plan{0, 0, 0, 0, 0};
    if (num_workers == -1) {
        plan->workers = num_seqs * Hkv;
        plan->per_segment = 1;
        return PA_OK;
    }
    if (num_workers < -1 || num_workers > kMaxWorkers) return PA_ERR_INVALID_ARG;
    int W = num_workers;
    if (W == 0) {
        int cus = 0;
        pa_status_t st = cu_count(&cus);
        if (st != PA_OK) return st;
        const int64_t units_bound = (int64_t)num_seqs * Hkv * max_blocks;
        int64_t want = (units_bound + kMinBlocksPerWorker - 1) / kMinBlocksPerWorker;
        const int64_t cap = (int64_t)cus * kWorkersPerCU;
        W = (int)(want < 1 ? 1 : (want > cap ? cap : want));
    }
    plan->workers = W;
    const size_t prefix = round_up(sizeof(int32_t) * ((size_t)num_seqs + 1), 256);
    const size_t lse = round_up(sizeof(float) * (size_t)W * 2 * G, 256);
    const size_t o = sizeof(float) * (size_t)W * 2 * G * D;
    plan->off_lse = prefix;
    plan->off_o = prefix + lse;
    plan->bytes = prefix + lse + o;
    return PA_OK;
}

template <int DT, int D, int B>
hipError_t launch_decode(const DecodeArgs& a, const Plan& plan, hipStream_t stream) {
    const int groups = (plan.workers + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups == 0) return hipSuccess;
    void* args[] = {const_cast<DecodeArgs*>(&a)};
    const size_t lds = sizeof(int32_t) * ((size_t)a.num_seqs + 1);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_kernel<DT, D, B>), dim3(groups),
                                   dim3(kGroupThreads), args, lds, stream);
    if (e != hipSuccess || plan.per_segment) return e;
    MergeArgs m{a.seq_prefix, a.part_lse, a.part_o, a.out, a.num_seqs, a.num_q_heads, a.num_kv_heads, a.group,
                a.num_workers};
    void* margs[] = {&m};
    return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<DT, D>), dim3(a.num_seqs * a.num_kv_heads),
                           dim3(kGroupThreads), margs, 0, stream);
}

template <int DT>
hipError_t dispatch_decode(const DecodeArgs& a, const Plan& plan, int D, int B, hipStream_t stream) {
    if (D == 64) return B == 16 ? launch_decode<DT, 64, 16>(a, plan, stream) : launch_decode<DT, 64, 32>(a, plan, stream);
    return B == 16 ? launch_decode<DT, 128, 16>(a, plan, stream) : launch_decode<DT, 128, 32>(a, plan, stream);
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status_t status) {
    switch (status) {
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
    }
    return "unknown status";
}

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

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
    hipError_t e = hipLaunchKernel(fn, dim3(num_tokens), dim3(kGroupThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                    const pa_cache_desc_t* cache, int32_t num_workers) {
    if (check_decode_shapes(num_seqs, num_q_heads, max_blocks_per_seq, cache) != PA_OK) return 0;
    Plan plan;
    if (make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, num_workers, &plan) != PA_OK) return 0;
    return plan.bytes;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 const pa_cache_desc_t* cache) {
    return pa_decode_workspace_bytes_ex(num_seqs, num_q_heads, max_blocks_per_seq, cache, 0);
}

pa_status_t pa_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                         size_t workspace_bytes, int32_t num_workers, pa_stream_t stream) {
    pa_status_t st = check_decode_shapes(num_seqs, num_q_heads, max_blocks_per_seq, cache);
    if (st != PA_OK) return st;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    if (num_workers < -1 || num_workers > kMaxWorkers) return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return PA_OK;  // nothing is touched, so empty tensors may pass null pointers
    if (!q || !k_cache || !v_cache || !context_lens || !out) return PA_ERR_INVALID_ARG;
    if (max_blocks_per_seq > 0 && !block_tables) return PA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(context_lens, 4) || (block_tables && !aligned(block_tables, 4)))
        return PA_ERR_INVALID_ARG;
    Plan plan;
    st = make_plan(num_seqs, num_q_heads, max_blocks_per_seq, cache, num_workers, &plan);
    if (st != PA_OK) return st;
    if (plan.bytes > 0 && (workspace == nullptr || workspace_bytes < plan.bytes || !aligned(workspace, 256)))
        return PA_ERR_WORKSPACE;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    DecodeArgs a{};
    a.q = static_cast<const uint8_t*>(q);
    a.k_cache = static_cast<const uint8_t*>(k_cache);
    a.v_cache = static_cast<const uint8_t*>(v_cache);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = static_cast<uint8_t*>(out);
    a.seq_prefix = plan.per_segment ? nullptr : reinterpret_cast<int32_t*>(ws);
    a.part_lse = plan.per_segment ? nullptr : reinterpret_cast<float*>(ws + plan.off_lse);
    a.part_o = plan.per_segment ? nullptr : reinterpret_cast<float*>(ws + plan.off_o);
    a.scale_log2 = scale * kLog2e;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache->num_kv_heads;
    a.group = num_q_heads / cache->num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = cache->num_blocks;
    a.num_workers = plan.workers;
    a.per_segment = plan.per_segment;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (cache->dtype) {
        case PA_F32:
            e = dispatch_decode<PA_F32>(a, plan, cache->head_dim, cache->block_size, s);
            break;
        case PA_F16:
            e = dispatch_decode<PA_F16>(a, plan, cache->head_dim, cache->block_size, s);
            break;
        default:
            e = dispatch_decode<PA_BF16>(a, plan, cache->head_dim, cache->block_size, s);
            break;
    }
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                      size_t workspace_bytes, pa_stream_t stream) {
    return pa_decode_ex(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                        max_blocks_per_seq, cache, workspace, workspace_bytes, 0, stream);
}

}  // extern "C"
