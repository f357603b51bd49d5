/*
 * libpagedattn: decode-step attention over a paged (block-table) KV cache,
 * and the KV-append write that places each new token's K/V in its slot,
 * for AMD Instinct MI355X (gfx950).
 *
 * Where the operations come from:
 *  - ForgeLLM README (LLM-inference-server), feature list: the KV cache is a
 *    pool of physical blocks, each request owns a logical block table that
 *    maps its j-th block to a physical one, and decode attention reads the
 *    physical blocks straight through that table with an online softmax,
 *    never assembling a padded batch-wide K/V; the decoder uses grouped-query
 *    attention.
 *  - LLM-Inference-Engine README, request-journey figure and the "why paged
 *    KV cache" paragraph: fixed-size blocks are preallocated and handed to a
 *    request on demand as it grows; the "why dynamic injection" paragraph:
 *    decode is memory-bound.
 *
 * Conventions shared by every call
 *  - All pointers to tensors are DEVICE pointers; descriptors are HOST
 *    pointers.  Every tensor is dense and row-major.
 *  - One element type (pa_dtype_t) for q, out, the caches and new K/V rows.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *    void*; NULL is the null stream).  They never synchronise the host,
 *    never allocate, keep no pointer after returning and hold no state
 *    beyond a per-device compute-unit count, so they are reentrant.
 *  - The caller owns every buffer.  Errors come back as pa_status_t; nothing
 *    is thrown across the ABI.  Arguments are checked on the host before any
 *    launch; device data (slots, block ids, lengths) cannot be checked
 *    without a synchronisation and is a precondition.  Out-of-range device
 *    values are clamped inside the kernels so they cannot fault, but the
 *    results are then unspecified.
 *
 * Cache layout.  A block keeps its tokens in slabs of 16 consecutive tokens
 * (block_size / 16 slabs per block).  Each (block, kv-head, slab) is
 * 16 * head_dim contiguous elements; in either pool, the slab of token `o` of
 * physical block `p`, kv-head `g` starts at element
 *    ((p * num_kv_heads + g) * (block_size / 16) + o / 16) * 16 * head_dim.
 * Inside a slab, with t = o % 16, X = 16 / element bytes (4 for f32, 8 for
 * f16/bf16) and Y = 4 / element bytes (1 for f32, 2 for f16/bf16), dim `d` is
 *    K: (d / X) * 16 * X + t * X + d % X
 *    V: ((((t / 4) * (D / (16*Y)) + d / (16*Y)) * 16 + d % 16) * Y + (d / 16) % Y) * 4 + t % 4
 * (for f32: ((t / 4) * D + d) * 4 + t % 4).  This places each 16-byte piece
 * that a matrix-core operand needs in one load, with consecutive lanes
 * reading consecutive bytes, and keeps a token's V row inside one quarter of
 * its slab.  A slot is p * block_size + o.
 * The geometry per (block, kv-head) is that of a plain
 * [num_blocks][num_kv_heads][block_size][head_dim] pool -- the same bytes,
 * the same tile per (block, kv-head) -- but the order of the elements inside
 * each 16-token slab is this one, not token-major rows: with token-major
 * rows a V operand (4 consecutive tokens of one dim) would take 4 separate
 * 2- or 4-byte loads per lane.  Pools are therefore written only through
 * pa_write_kv / pa_decode_append (or code that follows the formulas above);
 * a caller holding token-major pools must convert them once.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 3

/*
 * Every workspace begins with this many bytes of synchronisation words (the
 * counters by which the parts of a split are merged inside one launch).
 * They must hold zero before the workspace is first used -- one hipMemset
 * (or a zero-filled allocation) when it is created -- and every call leaves
 * them zero again when it completes, so a workspace may then be reused by
 * calls of any shape, and captured in a graph, without clearing it again.
 * The bytes after them need no initialisation.  Calls that share a workspace
 * must not run at the same time (issue them on one stream).
 */
#define PA_WORKSPACE_SYNC_BYTES (256 * 1024)

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, Hq not a multiple of Hkv */
    PA_ERR_UNSUPPORTED = 2, /* a valid request outside what the library implements */
    PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    PA_ERR_HIP = 4,         /* a HIP runtime call or a launch failed */
    PA_ERR_CAPACITY = 5     /* the block pool cannot promise what an admission asks for */
} pa_status_t;

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype_t;

/* Geometry of a K/V pool pair. */
typedef struct pa_cache_desc {
    int32_t num_blocks;   /* physical blocks in each pool, > 0 */
    int32_t block_size;   /* tokens per block: 16 or 32 */
    int32_t num_kv_heads; /* Hkv > 0 */
    int32_t head_dim;     /* D: 64 or 128 */
    int32_t dtype;        /* a pa_dtype_t */
} pa_cache_desc_t;

typedef void* pa_stream_t; /* a hipStream_t */

/*
 * KV append: for every token i < num_tokens with slot_mapping[i] >= 0, copy
 * k_new[i][g][:] and v_new[i][g][:] (every kv-head g) into physical block
 * slot / block_size at offset slot % block_size of k_cache / v_cache, bit for
 * bit.  A negative slot marks a padding token: nothing is written for it.
 * No other cache byte changes.
 *   k_new, v_new : [num_tokens][num_kv_heads][head_dim], 16-byte aligned
 *   slot_mapping : int64 [num_tokens], 8-byte aligned
 *   k_cache, v_cache : pools in the layout above, 16-byte aligned
 * Preconditions (unchecked): slot < num_blocks * block_size; no two tokens
 * of one call share a non-negative slot.  A slot past the pool is skipped.
 * num_tokens == 0 is a no-op (pointers are then not looked at).
 */
pa_status_t pa_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping, void* k_cache,
                        void* v_cache, int32_t num_tokens, const pa_cache_desc_t* cache, pa_stream_t stream);

/*
 * Decode attention, one query token per sequence: for sequence s < num_seqs
 * and query head h < num_q_heads, with G = num_q_heads / num_kv_heads,
 * kv-head g = h / G and L = context_lens[s],
 *   out[s][h][:] = sum_{t<L} softmax_t(scale * q[s][h][:] . K_t) * V_t
 * where K_t, V_t are the rows of logical position t, found in physical block
 * block_tables[s][t / block_size] at offset t % block_size.  L counts the
 * token being decoded (its K/V must already be written), and only positions
 * t < L are read: block-table entries past ceil(L / block_size) and slots
 * past L in the last block may hold anything, NaN included.  L == 0 gives
 * out = 0.  Arithmetic is fp32; out is rounded to nearest-even once.
 *   q, out        : [num_seqs][num_q_heads][head_dim], 16-byte aligned; out
 *                   must not overlap any input
 *   block_tables  : int32 [num_seqs][max_blocks_per_seq], 4-byte aligned
 *   context_lens  : int32 [num_seqs], 4-byte aligned
 *   workspace     : device scratch of at least pa_decode_workspace_bytes(...)
 *                   bytes, 256-byte aligned (may be NULL when that is 0);
 *                   its first PA_WORKSPACE_SYNC_BYTES bytes must be zero
 *                   before its first use and are left zero by every call;
 *                   the rest needs no initialisation and is clobbered
 * Supported: 1 <= G <= 16, head_dim 64/128, block_size 16/32, num_seqs <= 8192
 * (and per-sequence tables of 8 bytes a sequence within the device's LDS per
 * workgroup: 160 KB on MI355X), else PA_ERR_UNSUPPORTED.
 * Preconditions (unchecked): 0 <= L <= max_blocks_per_seq * block_size and
 * 0 <= block_tables[s][j] < num_blocks for j < ceil(L / block_size).
 * The result depends only on logical positions: it is bitwise the same
 * for any physical placement and from run to run.  num_seqs == 0 is a no-op
 * (pointers are then not looked at).
 */
pa_status_t pa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                      size_t workspace_bytes, pa_stream_t stream);

/*
 * pa_decode for callers that cannot allocate device memory -- code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation: the same computation with the same automatic split (bitwise
 * the same output as pa_decode), with its workspace taken from a device
 * array of PA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends.  It calls no allocator.  The first call on
 * a device looks up that array's address and clears its synchronisation
 * words with a small kernel on `stream`.
 * All calls on one GPU share the one array: calls that overlap in time on a
 * GPU (other streams, other host threads) race and give undefined results;
 * issue them on one stream.  A plan larger than the array (not reached on
 * MI355X: at most 2 wavefronts per compute unit, G <= 16, head_dim <= 128)
 * returns PA_ERR_WORKSPACE.  Arguments as in pa_decode.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
pa_status_t pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                              int32_t num_q_heads, int32_t max_blocks_per_seq, const pa_cache_desc_t* cache,
                              pa_stream_t stream);

/*
 * Workspace bytes pa_decode needs for these shapes on the current device
 * (0 means none).  Returns 0 as well for arguments pa_decode would reject.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 const pa_cache_desc_t* cache);

/*
 * pa_decode with the work split chosen by the caller:
 *   num_workers == 0  : automatic (what pa_decode does)
 *   num_workers == -1 : one worker per (sequence, kv-head slice) over its
 *                       whole context; no partial results, no merge
 *   num_workers  > 0  : the logical blocks of all sequences are dealt to that
 *                       many workers in equal contiguous runs; pairs cut
 *                       between runs are merged by a log-sum-exp reduction
 * A worker is one workgroup with a wavefront per kv-head of a slice of the
 * kv-heads (the slice is the largest divisor of num_kv_heads up to 2), so
 * every wave of a worker covers the same logical blocks.  num_workers times
 * the slice may be at most PA_WORKSPACE_SYNC_BYTES / 8 - 16 (the arrival words
 * of the split), else PA_ERR_UNSUPPORTED.
 * Every choice computes the same function; results agree within rounding.
 */
pa_status_t pa_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                         int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                         size_t workspace_bytes, int32_t num_workers, pa_stream_t stream);

/*
 * One decode step in one launch: the KV append of each sequence's new token
 * followed by decode attention, with the same results as
 *    pa_write_kv(k_new, v_new, slots, k_cache, v_cache, num_seqs, ...)
 *    pa_decode_ex(q, k_cache, v_cache, block_tables, context_lens, ...)
 * where the new token of sequence s is its last position, L - 1 with
 * L = context_lens[s], so slots[s] = block_tables[s][(L-1)/block_size] *
 * block_size + (L-1) % block_size (no slot when L == 0).  The decode output
 * is bitwise the same as that pair of calls with the same num_workers, and
 * so are the caches afterwards.
 *   k_new, v_new : [num_seqs][num_kv_heads][head_dim], 16-byte aligned
 *   other arguments as in pa_decode_ex; the caches are written.
 * Precondition (unchecked): no sequence's new-token slot lies in a block
 * another sequence of the call reads (distinct last blocks).
 */
pa_status_t pa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                             int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                             const pa_cache_desc_t* cache, void* workspace, size_t workspace_bytes,
                             int32_t num_workers, pa_stream_t stream);

/*
 * Rotary position embedding in place, the rotate-half pairing of the Llama
 * family (ForgeLLM README, feature list: RoPE in the Llama-family decoder;
 * the paragraph after its quick start: RoPE scaling is not supported, so this
 * is the plain form).  For every token t and head, with p = positions[t] and
 * w_i = rope_theta^(-2i/D), i < D/2, dims i and i + D/2 of the row become
 *   x_i cos(p w_i) - x_{i+D/2} sin(p w_i),   x_{i+D/2} cos(p w_i) + x_i sin(p w_i)
 * rounded to nearest-even into the dtype.  The angle is formed and reduced in
 * double; sin, cos and the rotation are single precision.
 *   q : [num_tokens][num_q_heads][head_dim], k : [num_tokens][num_kv_heads][head_dim],
 *       16-byte aligned, rotated in place (NULL allowed when its head count is 0)
 *   positions : int32 [num_tokens], device
 *   rope_theta : finite, > 1;  head_dim 64 or 128;  dtype a pa_dtype_t
 */
pa_status_t pa_rope(void* q, void* k, const int32_t* positions, int32_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype, float rope_theta, pa_stream_t stream);

/*
 * One decoder step's attention in one launch, rotary embedding included:
 * bitwise the same output and caches as
 *    pa_rope(q', k_new', positions = context_lens - 1, ...)   on copies q', k_new'
 *    pa_decode_append(q', k_new', v_new, ...)
 * with the same num_workers; q and k_new are only read.  16-bit caches only
 * (PA_ERR_UNSUPPORTED for f32: call the pair above).  Arguments as in
 * pa_decode_append, plus rope_theta as in pa_rope.
 */
pa_status_t pa_decode_rope_append(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, float scale,
                                  float rope_theta, void* out, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_blocks_per_seq, const pa_cache_desc_t* cache, void* workspace,
                                  size_t workspace_bytes, int32_t num_workers, pa_stream_t stream);

/*
 * Attention of several query tokens per sequence over the paged cache: the
 * causal extension of pa_decode, for prompts split into chunks that run
 * alongside decode steps and for checking speculative draft tokens (ForgeLLM
 * README: feature list, causal masking and chunked prefill; the paragraph
 * under its architecture flowchart; TokenForge post: speculative decoding).
 * Sequence s owns query rows query_start[s] .. query_start[s+1] - 1, its
 * n = query_start[s+1] - query_start[s] newest positions: with
 * L = context_lens[s], query token i (row query_start[s] + i) sits at position
 * L - n + i and, for every head h (kv-head h / G),
 *   out[row][h][:] = sum_{t <= L-n+i} softmax_t(scale * q[row][h][:] . K_t) * V_t
 * The K/V of all L positions, the query tokens' own included, must already be
 * in the cache (pa_write_kv).  n = 1 for every sequence is exactly pa_decode_ex.
 *   q, out         : [num_q_rows][num_q_heads][head_dim], 16-byte aligned
 *   query_start    : int32 [num_seqs + 1], device, non-decreasing from 0 to
 *                    at most num_q_rows; values outside [0, num_q_rows] are
 *                    clamped into it, so no row outside q/out is touched
 *   max_query_len  : host value >= every n (0: nothing to do)
 *   num_q_rows     : host value, the rows of q and out
 *   other arguments as in pa_decode_ex; the workspace must hold
 *   pa_attend_workspace_bytes(...) bytes
 * Two paths, chosen per sequence on the device, two launches on `stream`.
 * A sequence with at most floor(16 / G) tokens takes the split path of
 * pa_decode_ex: its tokens and heads are the columns of one matrix-core tile
 * that reads the K/V they see once.  A longer one (draft tokens, a prompt
 * chunk) is cut into blocks of C = 4 x floor(16 / G) tokens for 64-dim 16-bit
 * rows and 2 x floor(16 / G) otherwise, each attended by one workgroup whose
 * four waves split the positions and merge at the end: its K/V is read once
 * per block (mostly from L2, the blocks of a sequence running side by side).
 * Preconditions (unchecked): n <= L, and those of pa_decode.  A column whose
 * tokens see no position (only possible when n > L) gives 0.  Limits as in
 * pa_decode; PA_ERR_UNSUPPORTED also when a workgroup's per-sequence tables
 * (16 bytes a sequence, and for prompt chunks 12 beside a 25 KB merge area)
 * exceed the device's LDS.
 */
pa_status_t pa_attend(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, const int32_t* query_start, float scale, void* out,
                      int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t max_query_len,
                      int32_t num_q_rows, const pa_cache_desc_t* cache, void* workspace, size_t workspace_bytes,
                      int32_t num_workers, pa_stream_t stream);

/* Workspace bytes pa_attend needs for these shapes and num_workers (0 for arguments it rejects);
 * at least PA_WORKSPACE_SYNC_BYTES, whose words also count the prompt-chunk work items. */
size_t pa_attend_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 const pa_cache_desc_t* cache, int32_t num_workers);

/* Workspace bytes pa_decode_ex and pa_decode_append need for that num_workers. */
size_t pa_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                    const pa_cache_desc_t* cache, int32_t num_workers);

/* PA_WORKSPACE_SYNC_BYTES of the built library. */
size_t pa_workspace_sync_bytes(void);

/* Static, human-readable name of a status. */
const char* pa_status_string(pa_status_t status);

/*
 * Block pool (ForgeLLM README, feature list: physical KV blocks behind
 * per-request logical block tables, worst-case admission reservation,
 * reclamation, capacity errors and occupancy/byte telemetry;
 * LLM-Inference-Engine README, the "why paged KV cache" paragraph and the
 * request-journey figure: fixed-size blocks from a preallocated pool, handed
 * to a request on demand as it grows).
 *
 * The free blocks are a stack of ids in device memory, free_ids[0 .. top),
 * with the top at index top - 1, and a device state record pool_state of 8
 * int32 (8-byte aligned):
 *   [0] top: free blocks          [1] sequences refused for lack of blocks
 *   [2] lowest top since init     [3] releases refused (the stack would overflow)
 *   [4..7] internal, zero between calls
 * `capacity` is the length of free_ids.  The calls below keep the stack and
 * the tables on the device and run on `stream` with no host synchronisation;
 * calls on one pool must not overlap (use one stream).  Every index they form
 * is bounded by capacity, the table width and num_tokens, so malformed device
 * values give unspecified ids, never an access outside those arrays.
 */

/* Stack the ids 0 .. num_free - 1 so that pops yield them in increasing
 * order; the rest of free_ids becomes -1 and the counters start at zero.
 * 0 <= num_free <= capacity. */
pa_status_t pa_pool_init(int32_t* free_ids, int32_t* pool_state, int32_t num_free, int32_t capacity,
                         pa_stream_t stream);

/*
 * Give each sequence's new tokens their blocks and slots.  Sequence s has
 * L = context_lens[s] positions after this step, the newest
 * n = query_start[s+1] - query_start[s] of them new (n = 1 for every sequence
 * when query_start is NULL, and then num_tokens = num_seqs); it already holds
 * blocks 0 .. ceil((L - n) / B) - 1 of its table row and needs the blocks up
 * to ceil(L / B) - 1.  Sequences are served in order: one needing no block
 * is always served; one needing k blocks is served when k ids remain and no
 * earlier sequence was refused, and pops them, the first popped becoming its
 * lowest new block.  Row query_start[s] + i (position p = L - n + i) gets
 * slot_mapping = block_tables[s][p / B] * B + p % B, ready for pa_write_kv;
 * a refused sequence's rows get -1, its table row is left alone and
 * pool_state[1] counts it.
 *   context_lens : int32 [num_seqs], device; query_start : int32 [num_seqs + 1]
 *       non-decreasing from 0 to num_tokens, device, or NULL
 *   block_tables : int32 [num_seqs][max_blocks_per_seq], device, updated
 *   slot_mapping : int64 [num_tokens], device, written
 *   block_size   : B, the pool's tokens per block
 * Preconditions (unchecked): L <= max_blocks_per_seq * B (longer lengths are
 * clamped), n >= 0.  Rows whose position would be below 0 get -1.
 */
pa_status_t pa_assign_slots(const int32_t* context_lens, const int32_t* query_start, int32_t* block_tables,
                            const int32_t* free_ids, int32_t* pool_state, int64_t* slot_mapping, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t num_tokens, int32_t capacity,
                            pa_stream_t stream);

/*
 * Reclaim finished sequences: for r = 0 .. num_release - 1 in order, sequence
 * seq_ids[r] pushes blocks 0 .. ceil(context_lens[s] / B) - 1 of its table
 * row, in that order, and those entries become -1.  Ids outside
 * [0, num_seqs) hold nothing.  If the stack would then exceed capacity,
 * nothing changes and pool_state[3] counts the refusal.
 * Precondition (unchecked): the ids are distinct.
 */
pa_status_t pa_release_seqs(const int32_t* seq_ids, int32_t num_release, const int32_t* context_lens,
                            int32_t* block_tables, int32_t* free_ids, int32_t* pool_state, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t capacity, pa_stream_t stream);

/*
 * Host-side admission accounting, worst case: a request is admitted only if
 * the blocks for its largest possible length (prompt plus the most tokens it
 * may generate) fit beside every admitted request's, so the device pool can
 * never run dry for admitted requests.  Plain host memory, no GPU calls.
 */
typedef struct pa_pool_acct {
    int64_t num_blocks;           /* blocks in the pool */
    int64_t block_size;           /* tokens per block */
    int64_t bytes_per_block;      /* K and V bytes of one block, all kv-heads */
    int64_t reserved_blocks;      /* promised to admitted requests */
    int64_t peak_reserved_blocks;
    int64_t admitted;             /* admitted and not yet retired */
    int64_t refused;              /* admissions refused with PA_ERR_CAPACITY */
} pa_pool_acct_t;

pa_status_t pa_acct_init(pa_pool_acct_t* acct, int64_t num_blocks, int32_t block_size, int64_t bytes_per_block);
/* Reserve ceil(max_tokens / block_size) blocks, or PA_ERR_CAPACITY (nothing reserved). */
pa_status_t pa_acct_admit(pa_pool_acct_t* acct, int64_t max_tokens);
/* Give back an admitted request's reservation (the same max_tokens). */
pa_status_t pa_acct_retire(pa_pool_acct_t* acct, int64_t max_tokens);

/* Occupancy and bytes, from the accounting and a host copy of pool_state. */
typedef struct pa_pool_telemetry {
    int64_t capacity_blocks, free_blocks, used_blocks, peak_used_blocks;
    int64_t capacity_bytes, used_bytes;
    int64_t reserved_blocks, peak_reserved_blocks, admitted;
    int64_t tokens_stored; /* as given: the sum of the live sequences' lengths */
    int64_t empty_slots;   /* slots of used blocks that hold no token */
    double occupancy;      /* used_blocks / capacity_blocks */
    int64_t refused_admissions, refused_sequences, refused_releases;
} pa_pool_telemetry_t;

/* state_host: the 8 int32 of pool_state copied to the host.  PA_ERR_INVALID_ARG
 * when the figures contradict each other (more tokens than used slots). */
pa_status_t pa_pool_telemetry(const pa_pool_acct_t* acct, const int32_t* state_host, int64_t tokens_stored,
                              pa_pool_telemetry_t* out);

/*
 * RMSNorm of token rows (ForgeLLM README, feature list: RMSNorm in the
 * Llama-family decoder, with reference, fused and compiled kernels checked
 * against each other), optionally fused with the residual add before it:
 *   h = x, or, when residual is not NULL, h = round(x + residual), which is
 *       also stored back into residual;
 *   out[t][d] = round(h[t][d] * weight[d] / sqrt(mean_d(h[t][d]^2) + eps))
 * with float32 arithmetic and one rounding (nearest-even) into the dtype.
 *   x, residual, out : [rows][hidden], weight : [hidden], one pa_dtype_t,
 *       16-byte aligned, device; out may be x (each row is read before it is
 *       written)
 *   hidden : a multiple of 8 (16-bit) or 4 (f32), at most 8192 (16-bit) or
 *       4096 (f32), else PA_ERR_UNSUPPORTED;  eps >= 0, finite
 */
pa_status_t pa_rmsnorm(const void* x, void* residual, const void* weight, void* out, int64_t rows, int32_t hidden,
                       float eps, int32_t dtype, pa_stream_t stream);

/*
 * Read-bandwidth probe (a measurement aid, not part of the attention path):
 * the decode is a scan of K/V tiles, memory-bound (LLM-Inference-Engine
 * README, "why dynamic injection" paragraph and key learnings), and this call
 * measures the ceilings it is judged against.  It reads num_tiles tiles of
 * tile_bytes bytes from src -- tile i at (tile_ids ? tile_ids[i] : i) *
 * tile_bytes -- with 16-byte loads, and stores into sink, per lane of each of
 * num_waves wavefronts, the XOR of the 16-byte pieces it read (the XOR over
 * all of sink is the XOR over all pieces read).
 *   src      : device, 16-byte aligned;  tile_ids : int32 [num_tiles], device, or NULL
 *   sink     : device, num_waves * 64 * 16 bytes, 16-byte aligned, written
 *   tile_bytes : a positive multiple of 1024;  num_waves : a positive multiple of 4
 * Precondition (unchecked): every tile lies inside src.
 */
pa_status_t pa_read_probe(const void* src, const int32_t* tile_ids, int64_t num_tiles, int32_t tile_bytes,
                          uint32_t* sink, int32_t num_waves, pa_stream_t stream);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
