// Block pool for the paged KV cache: a stack of free physical block ids in
// device memory, the kernel that gives each step's new tokens their blocks
// and slots, the kernel that returns a finished sequence's blocks, and the
// host-side worst-case reservation and telemetry.
//
// What the pages fix: the cache is a preallocated pool of fixed-size physical
// blocks; a request owns a logical block table and is handed blocks on demand
// as it grows; admission reserves for the worst case, finished requests give
// their blocks back, a request that cannot be served is refused with a
// capacity error, and occupancy and bytes are reported (ForgeLLM README,
// feature list; LLM-Inference-Engine README, the "why paged KV cache"
// paragraph and the request-journey figure, where the block pool allocates
// for the engine).
//
// The device part runs on the step's stream without a host round trip: the
// stack and its counters live in device memory, sequences are served in
// order (so the result is deterministic and does not depend on which
// workgroup runs first), and every index is bounded by the stack's capacity,
// so a corrupt state record cannot send a store out of the arrays.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedattn.h"

namespace {

constexpr int kPoolThreads = 256;      // one sequence (or release entry) per thread of a workgroup
constexpr int kRowsPerGroup = 1024;    // token rows one workgroup fills before the rows are split further
constexpr int kMaxRowSplit = 1024;

// Fields of the state record (int32[8]); [4..5] hold a 64-bit arrival word:
// (workgroups arrived << 32) | blocks popped, zero between calls.
enum { kTop = 0, kRefusedSeqs = 1, kLowWater = 2, kRefusedReleases = 3, kArrive = 4 };

__device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct SeqSpan {
    int64_t L, first, have, need, row0, n;
};

// Sequence s's length after the call (clamped to its table), its new rows and
// the blocks it holds and needs.
__device__ inline SeqSpan seq_span(const int32_t* ctx, const int32_t* qs, int s, int M, int B) {
    SeqSpan q;
    int64_t L = ctx[s];
    L = L < 0 ? 0 : (L > (int64_t)M * B ? (int64_t)M * B : L);
    q.L = L;
    q.row0 = qs ? qs[s] : s;
    q.n = qs ? (int64_t)qs[s + 1] - qs[s] : 1;
    if (q.n < 0) q.n = 0;
    q.first = L - q.n;
    q.have = q.first > 0 ? cdiv(q.first, B) : 0;
    q.need = cdiv(L, B) - q.have;
    return q;
}

// Workgroup-wide sum and inclusive scan of 64-bit values (256 threads).
__device__ inline int64_t group_sum(int64_t v, int64_t* red) {
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
    for (int o = kPoolThreads / 2; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    const int64_t r = red[0];
    __syncthreads();
    return r;
}
__device__ inline int64_t group_inclusive_scan(int64_t v, int64_t* buf) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int o = 1; o < kPoolThreads; o <<= 1) {
        const int64_t add = tid >= o ? buf[tid - o] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    const int64_t r = buf[tid];
    __syncthreads();
    return r;
}

// The last workgroup to arrive gets true.  `popped` is this workgroup's share
// of the blocks taken; the caller of a true result gets the call's total.
__device__ inline bool arrive_last(int32_t* state, uint32_t popped, uint32_t* total_popped) {
    const uint32_t groups = gridDim.x * gridDim.y;
    if (groups == 1) {  // alone: no count to keep
        *total_popped = popped;
        return true;
    }
    auto* word = reinterpret_cast<unsigned long long*>(state + kArrive);
    const unsigned long long old = atomicAdd(word, (1ull << 32) | popped);
    *total_popped = (uint32_t)old + popped;
    return (uint32_t)(old >> 32) == groups - 1;
}

struct InitArgs {
    int32_t* free_ids;
    int32_t* state;
    int32_t num_free;
    int32_t capacity;
};

__global__ __launch_bounds__(kPoolThreads) void pool_init_kernel(InitArgs a) {
    const int i = blockIdx.x * kPoolThreads + threadIdx.x;
    if (i < a.capacity) a.free_ids[i] = i < a.num_free ? a.num_free - 1 - i : -1;
    if (i < 8) a.state[i] = (i == kTop || i == kLowWater) ? a.num_free : 0;
}

struct AssignArgs {
    const int32_t* ctx;
    const int32_t* qs;  // may be null: one row per sequence
    int32_t* bt;
    const int32_t* free_ids;
    int32_t* state;
    int64_t* slots;
    int32_t S, M, B, num_tokens, capacity;
};

// Grid (ceil(S / 256), row splits).  Workgroup x serves sequences
// [256x, 256x + 256): it computes their needs, the blocks popped before them
// (a sum over the earlier sequences, so no workgroup waits for another), and
// which are served; the workgroups with y = 0 write the new table entries,
// and all of them fill the slots of the group's rows, split over y.
__global__ __launch_bounds__(kPoolThreads) void assign_kernel(AssignArgs a) {
    __shared__ int64_t red[kPoolThreads];
    __shared__ int64_t s_first[kPoolThreads], s_len[kPoolThreads], s_have[kPoolThreads], s_off[kPoolThreads];
    __shared__ int64_t s_row0[kPoolThreads + 1];
    __shared__ int8_t s_served[kPoolThreads];
    const int tid = threadIdx.x;
    const int s0 = blockIdx.x * kPoolThreads;
    const int cnt = min(kPoolThreads, a.S - s0);
    int64_t top0 = a.state[kTop];
    top0 = top0 < 0 ? 0 : (top0 > a.capacity ? a.capacity : top0);

    // Blocks needed by the sequences before this group.
    int64_t before = 0;
    for (int r = tid; r < s0; r += kPoolThreads) before += seq_span(a.ctx, a.qs, r, a.M, a.B).need;
    const int64_t base = group_sum(before, red);

    const int s = s0 + tid;
    SeqSpan q{0, 0, 0, 0, 0, 0};
    if (tid < cnt) q = seq_span(a.ctx, a.qs, s, a.M, a.B);
    const int64_t incl = base + group_inclusive_scan(q.need, red);  // blocks popped up to and including s
    const bool served = q.need == 0 || incl <= top0;
    const int64_t off = incl - q.need;  // ids taken before s's
    if (tid < cnt) {
        s_first[tid] = q.first;
        s_len[tid] = q.L;
        s_have[tid] = q.have;
        s_off[tid] = off;
        s_served[tid] = served;
        s_row0[tid] = q.row0;
    }
    if (tid == 0) {
        const int last = s0 + cnt;  // rows of the group end where the next sequence's begin
        s_row0[cnt] = a.qs ? (int64_t)a.qs[last] : (int64_t)last;
    }
    // The new blocks: the first popped (free_ids[top0 - 1 - off]) becomes block `have`.
    uint32_t popped = 0;
    if (blockIdx.y == 0 && tid < cnt && served && q.need > 0) {
        for (int64_t k = 0; k < q.need; ++k)
            a.bt[(size_t)s * a.M + q.have + k] = a.free_ids[top0 - 1 - off - k];
    }
    const int64_t refused = group_sum(tid < cnt && !served ? 1 : 0, red);  // also orders the LDS writes
    const int64_t pops = group_sum(tid < cnt && served ? q.need : 0, red);
    if (blockIdx.y == 0) popped = (uint32_t)pops;

    // Slots of the group's rows.  Rows before the first sequence's or past
    // num_tokens are left alone (a malformed query_start).
    int64_t R0 = s_row0[0] < 0 ? 0 : s_row0[0];
    int64_t R1 = s_row0[cnt] > a.num_tokens ? a.num_tokens : s_row0[cnt];
    for (int64_t r = R0 + (int64_t)blockIdx.y * kPoolThreads + tid; r < R1; r += (int64_t)gridDim.y * kPoolThreads) {
        int lo = 0, hi = cnt - 1;  // the last sequence whose rows start at or before r
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_row0[mid] <= r) lo = mid;
            else hi = mid - 1;
        }
        const int64_t p = s_first[lo] + (r - s_row0[lo]);
        int64_t slot = -1;
        if (s_served[lo] && p >= 0 && p < s_len[lo]) {  // p < L unless query_start is malformed
            const int64_t j = p / a.B;
            const int64_t have = s_have[lo];
            const int32_t id = j < have ? a.bt[(size_t)(s0 + lo) * a.M + j]
                                        : a.free_ids[top0 - 1 - s_off[lo] - (j - have)];
            slot = (int64_t)id * a.B + p % a.B;
        }
        a.slots[r] = slot;
    }

    __syncthreads();
    if (tid == 0) {
        if (blockIdx.y == 0 && refused) atomicAdd(a.state + kRefusedSeqs, (int)refused);
        uint32_t total = 0;
        if (arrive_last(a.state, popped, &total)) {
            const int32_t new_top = (int32_t)(top0 - total);
            a.state[kTop] = new_top;
            if (new_top < a.state[kLowWater]) a.state[kLowWater] = new_top;
            if (gridDim.x * gridDim.y > 1) *reinterpret_cast<unsigned long long*>(a.state + kArrive) = 0ull;
        }
    }
}

struct ReleaseArgs {
    const int32_t* ids;
    const int32_t* ctx;
    int32_t* bt;
    int32_t* free_ids;
    int32_t* state;
    int32_t R, S, M, B, capacity;
};

__device__ inline int64_t release_count(const ReleaseArgs& a, int r) {
    const int s = a.ids[r];
    if (s < 0 || s >= a.S) return 0;
    int64_t L = a.ctx[s];
    L = L < 0 ? 0 : (L > (int64_t)a.M * a.B ? (int64_t)a.M * a.B : L);
    return cdiv(L, a.B);
}

// Grid ceil(R / 256).  Entry r pushes its sequence's blocks at stack
// positions top0 + (blocks of the entries before it) + j.
__global__ __launch_bounds__(kPoolThreads) void release_kernel(ReleaseArgs a) {
    __shared__ int64_t red[kPoolThreads];
    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * kPoolThreads;
    int64_t top0 = a.state[kTop];
    top0 = top0 < 0 ? 0 : (top0 > a.capacity ? a.capacity : top0);
    int64_t before = 0, all = 0;
    for (int r = tid; r < a.R; r += kPoolThreads) {
        const int64_t c = release_count(a, r);
        all += c;
        if (r < r0) before += c;
    }
    const int64_t base = group_sum(before, red);
    const int64_t total = group_sum(all, red);
    const int r = r0 + tid;
    const int64_t nb = r < a.R ? release_count(a, r) : 0;
    const int64_t pos = top0 + base + group_inclusive_scan(nb, red) - nb;
    const bool ok = top0 + total <= a.capacity;
    if (ok && nb > 0) {
        const int s = a.ids[r];
        for (int64_t j = 0; j < nb; ++j) {
            a.free_ids[pos + j] = a.bt[(size_t)s * a.M + j];
            a.bt[(size_t)s * a.M + j] = -1;
        }
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t unused = 0;
        if (arrive_last(a.state, 0, &unused)) {
            if (ok) a.state[kTop] = (int32_t)(top0 + total);
            else a.state[kRefusedReleases] += 1;
            if (gridDim.x > 1) *reinterpret_cast<unsigned long long*>(a.state + kArrive) = 0ull;
        }
    }
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int64_t host_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

pa_status_t pa_pool_init(int32_t* free_ids, int32_t* pool_state, int32_t num_free, int32_t capacity,
                         pa_stream_t stream) {
    if (capacity < 0 || num_free < 0 || num_free > capacity || !pool_state || !aligned(pool_state, 8))
        return PA_ERR_INVALID_ARG;
    if (capacity > 0 && !free_ids) return PA_ERR_INVALID_ARG;
    InitArgs a{free_ids, pool_state, num_free, capacity};
    void* args[] = {&a};
    const int groups = capacity > 8 ? (capacity + kPoolThreads - 1) / kPoolThreads : 1;
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pool_init_kernel), dim3(groups),
                                   dim3(kPoolThreads), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_assign_slots(const int32_t* context_lens, const int32_t* query_start, int32_t* block_tables,
                            const int32_t* free_ids, int32_t* pool_state, int64_t* slot_mapping, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t num_tokens, int32_t capacity,
                            pa_stream_t stream) {
    if (num_seqs < 0 || num_tokens < 0 || block_size <= 0 || capacity < 0) return PA_ERR_INVALID_ARG;
    if (!query_start && num_tokens != num_seqs) return PA_ERR_INVALID_ARG;
    if (num_seqs == 0) return num_tokens == 0 ? PA_OK : PA_ERR_INVALID_ARG;
    if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_INVALID_ARG;
    if (!context_lens || !block_tables || !free_ids || !pool_state || !aligned(pool_state, 8))
        return PA_ERR_INVALID_ARG;
    if (num_tokens > 0 && (!slot_mapping || !aligned(slot_mapping, 8))) return PA_ERR_INVALID_ARG;
    AssignArgs a{context_lens, query_start, block_tables, free_ids, pool_state, slot_mapping,
                 num_seqs, max_blocks_per_seq, block_size, num_tokens, capacity};
    void* args[] = {&a};
    const int gx = (num_seqs + kPoolThreads - 1) / kPoolThreads;
    int64_t gy = host_cdiv(host_cdiv(num_tokens, gx), kRowsPerGroup);
    gy = gy < 1 ? 1 : (gy > kMaxRowSplit ? kMaxRowSplit : gy);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&assign_kernel), dim3(gx, (unsigned)gy),
                                   dim3(kPoolThreads), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_release_seqs(const int32_t* seq_ids, int32_t num_release, const int32_t* context_lens,
                            int32_t* block_tables, int32_t* free_ids, int32_t* pool_state, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t capacity, pa_stream_t stream) {
    if (num_release < 0 || num_seqs < 0 || block_size <= 0 || capacity < 0) return PA_ERR_INVALID_ARG;
    if (num_release == 0) return PA_OK;
    if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_INVALID_ARG;
    if (!seq_ids || !pool_state || !aligned(pool_state, 8)) return PA_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!context_lens || !block_tables)) return PA_ERR_INVALID_ARG;
    if (capacity > 0 && !free_ids) return PA_ERR_INVALID_ARG;
    ReleaseArgs a{seq_ids, context_lens, block_tables, free_ids, pool_state,
                  num_release, num_seqs, max_blocks_per_seq, block_size, capacity};
    void* args[] = {&a};
    const int gx = (num_release + kPoolThreads - 1) / kPoolThreads;
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&release_kernel), dim3(gx), dim3(kPoolThreads),
                                   args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status_t pa_acct_init(pa_pool_acct_t* acct, int64_t num_blocks, int32_t block_size, int64_t bytes_per_block) {
    if (!acct || num_blocks < 0 || block_size <= 0 || bytes_per_block < 0) return PA_ERR_INVALID_ARG;
    *acct = pa_pool_acct_t{};
    acct->num_blocks = num_blocks;
    acct->block_size = block_size;
    acct->bytes_per_block = bytes_per_block;
    return PA_OK;
}

pa_status_t pa_acct_admit(pa_pool_acct_t* acct, int64_t max_tokens) {
    if (!acct || max_tokens < 0 || acct->block_size <= 0) return PA_ERR_INVALID_ARG;
    const int64_t need = host_cdiv(max_tokens, acct->block_size);
    if (acct->reserved_blocks + need > acct->num_blocks) {
        acct->refused += 1;
        return PA_ERR_CAPACITY;
    }
    acct->reserved_blocks += need;
    acct->admitted += 1;
    if (acct->reserved_blocks > acct->peak_reserved_blocks) acct->peak_reserved_blocks = acct->reserved_blocks;
    return PA_OK;
}

pa_status_t pa_acct_retire(pa_pool_acct_t* acct, int64_t max_tokens) {
    if (!acct || max_tokens < 0 || acct->block_size <= 0) return PA_ERR_INVALID_ARG;
    const int64_t need = host_cdiv(max_tokens, acct->block_size);
    if (acct->admitted <= 0 || need > acct->reserved_blocks) return PA_ERR_INVALID_ARG;
    acct->reserved_blocks -= need;
    acct->admitted -= 1;
    return PA_OK;
}

pa_status_t pa_pool_telemetry(const pa_pool_acct_t* acct, const int32_t* state_host, int64_t tokens_stored,
                              pa_pool_telemetry_t* out) {
    if (!acct || !state_host || !out || tokens_stored < 0) return PA_ERR_INVALID_ARG;
    pa_pool_telemetry_t t{};
    t.capacity_blocks = acct->num_blocks;
    t.free_blocks = state_host[0];
    t.used_blocks = acct->num_blocks - state_host[0];
    t.peak_used_blocks = acct->num_blocks - state_host[2];
    t.capacity_bytes = acct->num_blocks * acct->bytes_per_block;
    t.used_bytes = t.used_blocks * acct->bytes_per_block;
    t.reserved_blocks = acct->reserved_blocks;
    t.peak_reserved_blocks = acct->peak_reserved_blocks;
    t.admitted = acct->admitted;
    t.tokens_stored = tokens_stored;
    t.empty_slots = t.used_blocks * acct->block_size - tokens_stored;
    t.occupancy = acct->num_blocks > 0 ? (double)t.used_blocks / (double)acct->num_blocks : 0.0;
    t.refused_admissions = acct->refused;
    t.refused_sequences = state_host[1];
    t.refused_releases = state_host[3];
    *out = t;
    return (t.used_blocks < 0 || t.empty_slots < 0) ? PA_ERR_INVALID_ARG : PA_OK;
}

}  // extern "C"
