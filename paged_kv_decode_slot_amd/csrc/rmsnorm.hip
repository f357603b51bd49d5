// RMSNorm of token rows, optionally fused with the residual add that comes
// before it in a decoder (ForgeLLM README, feature list: RMSNorm in the
// Llama-family decoder, with a reference, a fused and a compiled kernel).
//
//   h = x                       or  h = round(x + residual), stored back to residual
//   out_d = round(h_d * w_d / sqrt(mean_d(h_d^2) + eps))
//
// One wavefront per row: lane l holds the row's 16-byte pieces l, l + 64, ...
// in registers (NP of them), so the row is read once, every load of the row is
// in flight together, and the sum of squares is a lane sum plus a butterfly
// over the wave (every lane ends with the same bits: each step adds the same
// two values, in either order).  The weight stays in registers across the
// rows a wave takes.  Arithmetic is float32; the output is rounded once.
// Rows are streamed with the non-temporal hint (loads and stores): a row is
// touched once, and keeping it out of the caches left more of the memory
// system to the stream (16384 x 4096 bf16: 46.5 -> 44.6 us plain,
// 102 -> 91 us with the residual, against 51 us for a plain device copy of
// the plain form's bytes).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedattn.h"

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormWaves = kNormThreads / 64;

struct NormArgs {
    const uint8_t* x;
    uint8_t* residual;  // null: plain RMSNorm
    const uint8_t* w;
    uint8_t* out;
    int64_t rows;
    int32_t pieces;  // 16-byte pieces per row
    float eps;
    float h;  // row length, as a float
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ inline uint4 load_stream(const uint8_t* base, int64_t idx) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base) + idx));
}
__device__ inline void store_stream(uint8_t* base, int64_t idx, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(base) + idx);
}
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

template <int DT>
__device__ inline void widen8(uint4 v, float* f) {
    if constexpr (DT == PA_BF16) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (float)b[j];
    } else if constexpr (DT == PA_F16) {
        const f16x8_t b = __builtin_bit_cast(f16x8_t, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (float)b[j];
    } else {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
}

template <int DT>
__device__ inline uint4 narrow8(const float* f) {
    if constexpr (DT == PA_BF16) {
        bf16x8_t b;
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = (__bf16)f[j];
        return __builtin_bit_cast(uint4, b);
    } else if constexpr (DT == PA_F16) {
        f16x8_t b;
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = (_Float16)f[j];
        return __builtin_bit_cast(uint4, b);
    } else {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
}

template <int DT, int NP, bool ADD>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(NormArgs a) {
#pragma clang fp contract(off)
    constexpr int X = DT == PA_F32 ? 4 : 8;  // elements per piece
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * kNormWaves;
    if (wave >= a.rows) return;

    uint4 w[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k)
        w[k] = lane + 64 * k < a.pieces ? reinterpret_cast<const uint4*>(a.w)[lane + 64 * k] : make_uint4(0, 0, 0, 0);

    const size_t row_bytes = (size_t)a.pieces * 16;
    for (int64_t row = wave; row < a.rows; row += waves) {
        const uint8_t* xr = a.x + row * row_bytes;
        uint8_t* rr = ADD ? a.residual + row * row_bytes : nullptr;
        uint4 v[NP], r[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const bool in = lane + 64 * k < a.pieces;
            v[k] = in ? load_stream(xr, lane + 64 * k) : make_uint4(0, 0, 0, 0);
            if constexpr (ADD) r[k] = in ? load_stream(rr, lane + 64 * k) : make_uint4(0, 0, 0, 0);
        }
        if constexpr (ADD) {  // h = round(x + residual): the new residual, and the row to normalise
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                float f[X], g[X];
                widen8<DT>(v[k], f);
                widen8<DT>(r[k], g);
#pragma unroll
                for (int j = 0; j < X; ++j) f[j] = f[j] + g[j];
                v[k] = narrow8<DT>(f);
                if (lane + 64 * k < a.pieces) store_stream(rr, lane + 64 * k, v[k]);
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            float f[X];
            widen8<DT>(v[k], f);
#pragma unroll
            for (int j = 0; j < X; ++j) ss = ss + f[j] * f[j];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss = ss + __shfl_xor(ss, o);
        const float rs = 1.0f / sqrtf(ss / a.h + a.eps);
        uint8_t* orow = a.out + row * row_bytes;
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            float f[X], g[X];
            widen8<DT>(v[k], f);
            widen8<DT>(w[k], g);
#pragma unroll
            for (int j = 0; j < X; ++j) f[j] = (f[j] * rs) * g[j];
            if (lane + 64 * k < a.pieces) store_stream(orow, lane + 64 * k, narrow8<DT>(f));
        }
    }
}

template <int DT, int NP>
const void* pick_add(bool add) {
    return add ? reinterpret_cast<const void*>(&rmsnorm_kernel<DT, NP, true>)
               : reinterpret_cast<const void*>(&rmsnorm_kernel<DT, NP, false>);
}

template <int DT>
const void* pick(int np, bool add) {
    switch (np) {
        case 1: return pick_add<DT, 1>(add);
        case 2: return pick_add<DT, 2>(add);
        case 4: return pick_add<DT, 4>(add);
        case 8: return pick_add<DT, 8>(add);
        default: return pick_add<DT, 16>(add);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" pa_status_t pa_rmsnorm(const void* x, void* residual, const void* weight, void* out, int64_t rows,
                                  int32_t hidden, float eps, int32_t dtype, pa_stream_t stream) {
    if (rows < 0 || hidden <= 0 || !(eps >= 0.f) || !(eps < INFINITY)) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
    const int X = dtype == PA_F32 ? 4 : 8;
    if (hidden % X) return PA_ERR_UNSUPPORTED;
    const int pieces = hidden / X;
    if (pieces > 64 * 16) return PA_ERR_UNSUPPORTED;
    if (rows == 0) return PA_OK;
    if (!x || !weight || !out || !aligned16(x) || !aligned16(weight) || !aligned16(out)) return PA_ERR_INVALID_ARG;
    if (residual && !aligned16(residual)) return PA_ERR_INVALID_ARG;
    int np = 1;
    while (64 * np < pieces) np *= 2;
    const void* fn = dtype == PA_BF16 ? pick<PA_BF16>(np, residual != nullptr)
                     : dtype == PA_F16 ? pick<PA_F16>(np, residual != nullptr)
                                       : pick<PA_F32>(np, residual != nullptr);
    NormArgs a{static_cast<const uint8_t*>(x), static_cast<uint8_t*>(residual), static_cast<const uint8_t*>(weight),
               static_cast<uint8_t*>(out), rows, pieces, eps, (float)hidden};
    // One wave per row (the hardware hands rows to CUs as they free up; a grid
    // capped at the resident waves ran 7% slower); past 2^20 rows a wave
    // takes several.
    const int64_t max_groups = (int64_t)1 << 18;
    int64_t groups = (rows + kNormWaves - 1) / kNormWaves;
    if (groups > max_groups) groups = max_groups;
    void* args[] = {&a};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)groups), dim3(kNormThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}
