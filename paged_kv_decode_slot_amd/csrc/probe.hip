// Read-bandwidth probe: the ceilings the decode kernel is measured against.
//
// Decode attention over a paged cache is a scan of K/V tiles scattered over a
// pool, so its bound is HBM bandwidth (LLM-Inference-Engine README, "why
// dynamic injection" paragraph and key learnings: decode is memory-bound).
// This kernel reads tiles of a buffer and nothing else, either in address
// order (the streaming-read ceiling) or in a given order (for 4 KB tiles in a
// shuffled order, the ceiling of reading a paged pool whole-tile by whole-tile).
// Each wavefront takes tiles in a grid-stride loop with 16-byte non-temporal
// loads, every lane a contiguous 16 bytes of each 1 KB run, and folds what it
// reads into an XOR it stores at the end, so no load can be dropped and the
// result is checkable.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedattn.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kTilesInFlight = 4;  // tiles a wavefront has loads in flight for at once
constexpr int kRunsPerBatch = 4;   // 1 KB runs of each of those tiles per batch: 16 loads per lane

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct ProbeArgs {
    const uint8_t* src;
    const int32_t* tile_ids;  // NULL: tile i is at i * tile_bytes
    uint32_t* sink;           // [waves * 64][4]
    int64_t num_tiles;
    int32_t tile_bytes;       // a multiple of 1024
};

// Wavefront w takes tiles w, w + waves, w + 2 waves, ... kTilesInFlight at a
// time; the ids of its next group are fetched while the current group's data
// is in flight.
template <bool LISTED>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(ProbeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
    const int64_t waves = ((int64_t)gridDim.x * kProbeThreads) >> 6;
    const int runs = a.tile_bytes / 1024;  // 1 KB runs per tile: one 16-byte load per lane each
    // Id of tile t, or -1 past the end; the id load is not under a branch (it reads
    // the last entry instead), so it never waits for the data loads in flight.
    auto tile_id = [&](int64_t t) -> int64_t {
        int64_t id = t;
        if constexpr (LISTED) id = a.tile_ids[t < a.num_tiles ? t : a.num_tiles - 1];
        return t < a.num_tiles ? id : -1;
    };
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t ids[kTilesInFlight];
#pragma unroll
    for (int i = 0; i < kTilesInFlight; ++i) ids[i] = tile_id(wave + i * waves);
    for (int64_t t0 = wave; t0 < a.num_tiles; t0 += kTilesInFlight * waves) {
        int64_t cur[kTilesInFlight];
#pragma unroll
        for (int i = 0; i < kTilesInFlight; ++i) cur[i] = ids[i];
        for (int r0 = 0; r0 < runs; r0 += kRunsPerBatch) {
            // Every load is issued (a missing tile or run reads tile 0's first run, which
            // lies in src whenever any tile does) and only the valid ones are folded in,
            // so no load sits under a branch.
            u32x4 v[kTilesInFlight][kRunsPerBatch];
#pragma unroll
            for (int i = 0; i < kTilesInFlight; ++i)
#pragma unroll
                for (int r = 0; r < kRunsPerBatch; ++r) {
                    const bool ok = cur[i] >= 0 && r0 + r < runs;
                    const int64_t off = ok ? cur[i] * a.tile_bytes + (int64_t)(r0 + r) * 1024 : 0;
                    v[i][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.src + off + lane * 16));
                }
            if (r0 + kRunsPerBatch >= runs) {  // the group's last batch: fetch the next group's ids
#pragma unroll
                for (int i = 0; i < kTilesInFlight; ++i) ids[i] = tile_id(t0 + (kTilesInFlight + i) * waves);
            }
#pragma unroll
            for (int i = 0; i < kTilesInFlight; ++i)
#pragma unroll
                for (int r = 0; r < kRunsPerBatch; ++r)
                    if (cur[i] >= 0 && r0 + r < runs) acc ^= v[i][r];
        }
    }
    reinterpret_cast<u32x4*>(a.sink)[wave * 64 + lane] = acc;
}

}  // namespace

extern "C" {

pa_status_t pa_read_probe(const void* src, const int32_t* tile_ids, int64_t num_tiles, int32_t tile_bytes,
                          uint32_t* sink, int32_t num_waves, pa_stream_t stream) {
    if (num_tiles < 0 || tile_bytes <= 0 || tile_bytes % 1024 != 0 || num_waves <= 0 || num_waves % 4 != 0)
        return PA_ERR_INVALID_ARG;
    if (!sink || ((uintptr_t)sink % 16) != 0) return PA_ERR_INVALID_ARG;
    if (num_tiles > 0 && (!src || ((uintptr_t)src % 16) != 0)) return PA_ERR_INVALID_ARG;
    if (tile_ids && ((uintptr_t)tile_ids % 4) != 0) return PA_ERR_INVALID_ARG;
    ProbeArgs a{static_cast<const uint8_t*>(src), tile_ids, sink, num_tiles, tile_bytes};
    void* args[] = {&a};
    const void* fn = tile_ids ? reinterpret_cast<const void*>(&read_probe_kernel<true>)
                              : reinterpret_cast<const void*>(&read_probe_kernel<false>);
    const hipError_t e = hipLaunchKernel(fn,
                                         dim3(num_waves / (kProbeThreads / 64)), dim3(kProbeThreads), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
