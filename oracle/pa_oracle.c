/*
 * Plain, slow, float64 CPU oracle for paged-KV decode attention, for the
 * KV-append slot write and for the block pool that hands out the slots.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the CPU-baseline leg of the benchmark call it; the library never does.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes (the plain definition, not the fast algorithm):
 *
 *  write: every token i with slot >= 0 goes to physical block slot / B at
 *    offset slot % B, for every kv-head: its K row and V row are copied there
 *    bit for bit; nothing else in the pools changes.  Tokens are taken in
 *    index order.  (ForgeLLM README, feature list: physical KV blocks owned
 *    through per-request logical block tables; LLM-Inference-Engine README,
 *    request-journey figure: fixed-size blocks handed out per request.)
 *
 *  decode: for sequence s and query head h, with kv-head g = h / G
 *    (grouped-query attention, ForgeLLM README feature list: query heads share
 *    a kv-head in contiguous groups of G) and L = context_lens[s]:
 *      for every logical position t < L, the K and V rows live in physical
 *      block block_tables[s][t / B] at offset t % B (ForgeLLM README, feature
 *      list: decode attention reads the physical blocks through the block
 *      table, never a padded K/V);
 *      z_t = scale * sum_d q[d] * k_t[d]          (sum over d in order)
 *      m   = max_t z_t,  w_t = exp(z_t - m)
 *      out = (sum_t w_t * v_t) / (sum_t w_t)      (sums over t in order)
 *    and out = 0 when L = 0.  Only positions t < L are read (the decode token
 *    is the newest position, so the causal mask is exactly t < L).  All
 *    arithmetic is double; stored values are widened exactly.
 *
 *  attend (several query tokens per sequence): the same sum for each of a
 *    sequence's n newest positions, with the causal mask of a decoder
 *    (ForgeLLM README, feature list: causal masking; the paragraph under the
 *    architecture flowchart: long prompts are split into bounded chunks and
 *    interleaved with decode; TokenForge post: speculative decoding, whose
 *    draft tokens are checked by exactly this attention).  Query token i of
 *    sequence s sits at position L - n + i and sees positions t <= L - n + i,
 *    so it is the decode sum over the first L - n + i + 1 positions.
 *
 * Pool layout.  The pages fix none; this is the layout documented for the
 * library's caller.  A block keeps its tokens in slabs of 16 consecutive
 * tokens (B a multiple of 16); each (block, kv-head, slab) holds 16 * D
 * contiguous elements.  With X = 16 / element_bytes and Y = 4 / element_bytes,
 * token t (0..15) and dim d of a slab sit at
 *    K: (d / X) * 16 * X + t * X + d % X
 *    V: ((((t / 4) * (D / (16*Y)) + d / (16*Y)) * 16 + d % 16) * Y + (d / 16) % Y) * 4 + t % 4
 * (for f32, Y = 1 and V is ((t / 4) * D + d) * 4 + t % 4), and slab
 * (p, g, o / 16) starts at element ((p * Hkv + g) * (B / 16) + o / 16) * 16 * D.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

static int elt_bytes(int dtype) { return dtype == OR_F32 ? 4 : 2; }

/* IEEE 754 binary16 -> double, from the format's definition. */
static double half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the top half of an IEEE binary32. */
static double bf16_to_double(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

static double widen(const void* base, size_t idx, int dtype) {
    if (dtype == OR_F32) return (double)((const float*)base)[idx];
    uint16_t raw = ((const uint16_t*)base)[idx];
    return dtype == OR_F16 ? half_to_double(raw) : bf16_to_double(raw);
}

static size_t slab_base(int64_t p, int g, int o, int Hkv, int B, int D) {
    return (((size_t)p * Hkv + g) * (size_t)(B / 16) + (size_t)(o / 16)) * 16 * (size_t)D;
}

static size_t k_index(int64_t p, int g, int o, int d, int Hkv, int B, int D, int X) {
    int t = o % 16;
    return slab_base(p, g, o, Hkv, B, D) + (size_t)(d / X) * 16 * X + (size_t)t * X + (size_t)(d % X);
}

static size_t v_index(int64_t p, int g, int o, int d, int Hkv, int B, int D, int Y) {
    int t = o % 16;
    size_t q = (size_t)(t / 4) * (size_t)(D / (16 * Y)) + (size_t)(d / (16 * Y)); /* (token quad, 16Y-dim group) */
    size_t in_slab = ((q * 16 + (size_t)(d % 16)) * Y + (size_t)((d / 16) % Y)) * 4 + (size_t)(t % 4);
    return slab_base(p, g, o, Hkv, B, D) + in_slab;
}

/* Geometry the layout is defined for. */
static int layout_ok(int B, int D, int dtype) {
    int eb = elt_bytes(dtype);
    return B > 0 && B % 16 == 0 && D > 0 && D % (16 * (4 / eb)) == 0;
}

/* Returns 0, or -1 on a bad argument. */
int oracle_write_kv(const void* k_new, const void* v_new, const int64_t* slot, void* k_pool, void* v_pool,
                    int64_t num_tokens, int64_t num_blocks, int B, int Hkv, int D, int dtype) {
    int eb = elt_bytes(dtype);
    int X = 16 / eb, Y = 4 / eb;
    if (Hkv <= 0 || !layout_ok(B, D, dtype)) return -1;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t sl = slot[i];
        if (sl < 0) continue;
        int64_t p = sl / B;
        int o = (int)(sl % B);
        if (p >= num_blocks) return -1;
        for (int g = 0; g < Hkv; ++g) {
            for (int d = 0; d < D; ++d) {
                size_t src = ((size_t)i * Hkv + g) * (size_t)D + (size_t)d;
                memcpy((char*)k_pool + k_index(p, g, o, d, Hkv, B, D, X) * eb, (const char*)k_new + src * eb, eb);
                memcpy((char*)v_pool + v_index(p, g, o, d, Hkv, B, D, Y) * eb, (const char*)v_new + src * eb, eb);
            }
        }
    }
    return 0;
}

typedef struct {
    const void *q, *k_pool, *v_pool;
    const int32_t *bt, *ctx;
    double scale;
    int S, Hq, Hkv, D, B, maxblk, dtype;
    const int32_t* pairs; /* (s, h) pairs to compute, or NULL for all */
    int64_t npairs;
    const int32_t* qstart;  /* several query tokens per sequence: [S + 1], else NULL */
    const int32_t* row_seq; /* with qstart: the sequence of each query row */
    double* out;            /* [npairs][D], [S][Hq][D], or [query rows][Hq][D] */
    int64_t first, last;
    int status;
} job_t;

/*
 * One output row: query row qrow (of q's [rows][Hq][D]), head h, over the
 * first L positions of sequence s, gathered through its block table.  The
 * definition written out.
 */
static int attend_one(const job_t* J, int s, int qrow, int h, int L, double* out_row) {
    int G = J->Hq / J->Hkv;
    int g = h / G;
    int X = 16 / elt_bytes(J->dtype), Y = 4 / elt_bytes(J->dtype);
    int D = J->D;
    if (L < 0 || L > J->maxblk * J->B) return -1;
    for (int d = 0; d < D; ++d) out_row[d] = 0.0;
    if (L == 0) return 0;

    double* q = malloc(sizeof(double) * D);
    double* z = malloc(sizeof(double) * L);
    if (!q || !z) {
        free(q);
        free(z);
        return -1;
    }
    for (int d = 0; d < D; ++d) q[d] = widen(J->q, ((size_t)qrow * J->Hq + h) * D + d, J->dtype);

    /* logits through the block table */
    for (int t = 0; t < L; ++t) {
        int64_t p = J->bt[(size_t)s * J->maxblk + t / J->B];
        int o = t % J->B;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[d] * widen(J->k_pool, k_index(p, g, o, d, J->Hkv, J->B, D, X), J->dtype);
        z[t] = J->scale * dot;
    }
    double m = z[0];
    for (int t = 1; t < L; ++t)
        if (z[t] > m) m = z[t];

    double den = 0.0;
    for (int t = 0; t < L; ++t) {
        double w = exp(z[t] - m);
        den += w;
        int64_t p = J->bt[(size_t)s * J->maxblk + t / J->B];
        int o = t % J->B;
        for (int d = 0; d < D; ++d) out_row[d] += w * widen(J->v_pool, v_index(p, g, o, d, J->Hkv, J->B, D, Y), J->dtype);
    }
    for (int d = 0; d < D; ++d) out_row[d] /= den;
    free(q);
    free(z);
    return 0;
}

static void* run_job(void* arg) {
    job_t* J = (job_t*)arg;
    for (int64_t k = J->first; k < J->last; ++k) {
        int s, h, qrow, L;
        if (J->qstart) {
            /* query row qrow is token i of sequence s: position ctx - n + i, so it
               sees the first ctx - n + i + 1 positions (causal) */
            qrow = (int)(k / J->Hq);
            h = (int)(k % J->Hq);
            s = J->row_seq[qrow];
            int n = J->qstart[s + 1] - J->qstart[s];
            int i = qrow - J->qstart[s];
            L = J->ctx[s] - n + i + 1;
            if (n > J->ctx[s]) {
                J->status = -1;
                return NULL;
            }
        } else {
            if (J->pairs) {
                s = J->pairs[2 * k];
                h = J->pairs[2 * k + 1];
            } else {
                s = (int)(k / J->Hq);
                h = (int)(k % J->Hq);
            }
            if (s < 0 || s >= J->S) {
                J->status = -1;
                return NULL;
            }
            qrow = s;
            L = J->ctx[s];
        }
        if (h < 0 || h >= J->Hq || attend_one(J, s, qrow, h, L, J->out + (size_t)k * J->D)) {
            J->status = -1;
            return NULL;
        }
    }
    return NULL;
}

static int run_jobs(job_t proto, int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = n > 0 ? (int)n : 1;
    job_t* jobs = calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].first = n * i / nthreads;
        jobs[i].last = n * (i + 1) / nthreads;
        jobs[i].status = 0;
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, run_job, &jobs[i])) break;
        started = i;
    }
    run_job(&jobs[0]);
    int status = jobs[0].status;
    for (int i = 1; i <= started; ++i) {
        pthread_join(th[i], NULL);
        if (jobs[i].status) status = jobs[i].status;
    }
    /* threads that failed to start: run their share here */
    for (int i = started + 1; i < nthreads; ++i) {
        run_job(&jobs[i]);
        if (jobs[i].status) status = jobs[i].status;
    }
    free(jobs);
    free(th);
    return status;
}

/*
 * Decode: one query token per sequence.  out: double [npairs][D] for the
 * listed (s, h) pairs (pairs = int32 [npairs][2]), or [S][Hq][D] when pairs is
 * NULL (npairs ignored).  Work is split over nthreads threads by output row;
 * each row is computed by one thread in the fixed order above, so the result
 * does not depend on nthreads.
 */
int oracle_decode(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                  const int32_t* context_lens, float scale, double* out, int S, int Hq, int Hkv, int D, int B,
                  int max_blocks_per_seq, int dtype, const int32_t* pairs, int64_t npairs, int nthreads) {
    if (Hkv <= 0 || Hq % Hkv || !layout_ok(B, D, dtype)) return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q;
    J.k_pool = k_pool;
    J.v_pool = v_pool;
    J.bt = block_tables;
    J.ctx = context_lens;
    J.scale = (double)scale;
    J.S = S;
    J.Hq = Hq;
    J.Hkv = Hkv;
    J.D = D;
    J.B = B;
    J.maxblk = max_blocks_per_seq;
    J.dtype = dtype;
    J.pairs = pairs;
    J.npairs = npairs;
    J.out = out;
    return run_jobs(J, pairs ? npairs : (int64_t)S * Hq, nthreads);
}

/*
 * Several query tokens per sequence (the causal extension of decode: chunked
 * prefill, speculative verification).  Sequence s owns query rows
 * [query_start[s], query_start[s + 1]) of q ([rows][Hq][D]); they are its
 * newest n = query_start[s+1] - query_start[s] positions of context_lens[s],
 * and row i sees positions t <= context_lens[s] - n + i.  out: double
 * [rows][Hq][D].  -1 on a bad argument (n > context_lens[s] included).
 */
int oracle_attend(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                  const int32_t* context_lens, const int32_t* query_start, float scale, double* out, int S, int Hq,
                  int Hkv, int D, int B, int max_blocks_per_seq, int dtype, int nthreads) {
    if (Hkv <= 0 || Hq % Hkv || !layout_ok(B, D, dtype) || query_start[0] != 0) return -1;
    for (int s = 0; s < S; ++s)
        if (query_start[s + 1] < query_start[s]) return -1;
    int rows = query_start[S];
    int32_t* row_seq = malloc(sizeof(int32_t) * (size_t)(rows > 0 ? rows : 1));
    if (!row_seq) return -1;
    for (int s = 0; s < S; ++s)
        for (int r = query_start[s]; r < query_start[s + 1]; ++r) row_seq[r] = s;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q;
    J.k_pool = k_pool;
    J.v_pool = v_pool;
    J.bt = block_tables;
    J.ctx = context_lens;
    J.scale = (double)scale;
    J.S = S;
    J.Hq = Hq;
    J.Hkv = Hkv;
    J.D = D;
    J.B = B;
    J.maxblk = max_blocks_per_seq;
    J.dtype = dtype;
    J.qstart = query_start;
    J.row_seq = row_seq;
    J.out = out;
    int status = run_jobs(J, (int64_t)rows * Hq, nthreads);
    free(row_seq);
    return status;
}

/*
 * Rotary position embedding, the rotate-half pairing of the Llama family
 * (ForgeLLM README, feature list: RoPE in the Llama-family decoder; the
 * paragraph after its quick start: RoPE scaling is not supported, so the
 * plain form is the one to compute).  For a row x of D values at position p,
 * with w_i = theta^(-2i/D) for i < D/2:
 *   x'_i       = x_i cos(p w_i) - x_{i+D/2} sin(p w_i)
 *   x'_{i+D/2} = x_{i+D/2} cos(p w_i) + x_i sin(p w_i)
 * x: [T][H][D] in the storage dtype, pos: int32 [T]; out: double [T][H][D],
 * the rotated values before any rounding.
 */
int oracle_rope(const void* x, const int32_t* pos, double* out, int64_t T, int H, int D, int dtype, double theta) {
    if (D <= 0 || D % 2 || H <= 0 || theta <= 1.0) return -1;
    int half = D / 2;
    for (int64_t t = 0; t < T; ++t) {
        double p = (double)pos[t];
        for (int h = 0; h < H; ++h) {
            size_t row = ((size_t)t * H + h) * (size_t)D;
            for (int i = 0; i < half; ++i) {
                double w = pow(theta, -2.0 * i / D);
                double c = cos(p * w), sn = sin(p * w);
                double a = widen(x, row + i, dtype), b = widen(x, row + i + half, dtype);
                out[row + i] = a * c - b * sn;
                out[row + i + half] = b * c + a * sn;
            }
        }
    }
    return 0;
}

/*
 * Round doubles to the nearest value of the storage dtype, ties to even, in
 * one step (no intermediate float): out holds doubles that the dtype
 * represents exactly.  For a type with m mantissa bits, minimum normal
 * exponent emin and largest finite value vmax, |x| = q * 2^e with
 * q in [2^m, 2^(m+1)) (or e = emin - m below the normal range) is rounded by
 * rounding q to an integer.
 */
int oracle_round(const double* in, int64_t n, int dtype, double* out) {
    int m, emin;
    double vmax;
    if (dtype == 0) {
        for (int64_t k = 0; k < n; ++k) out[k] = (double)(float)in[k];
        return 0;
    } else if (dtype == 1) {
        m = 10;
        emin = -14;
        vmax = 65504.0;
    } else if (dtype == 2) {
        m = 7;
        emin = -126;
        vmax = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    } else {
        return -1;
    }
    for (int64_t k = 0; k < n; ++k) {
        double x = in[k], ax = fabs(x);
        if (isnan(x) || isinf(x) || ax == 0.0) {
            out[k] = x;
            continue;
        }
        int e2;
        frexp(ax, &e2); /* ax = f * 2^e2, f in [0.5, 1) */
        int e = e2 - 1 - m;
        if (e2 - 1 < emin) e = emin - m;
        double r = nearbyint(ldexp(ax, -e)) ; /* round half to even in the default mode */
        double v = ldexp(r, e);
        /* values at or above the midpoint between vmax and the next power step overflow */
        if (v > vmax) v = INFINITY;
        out[k] = x < 0 ? -v : v;
    }
    return 0;
}

/* Exposes the element widening on its own, so it can be checked against other converters. */
void oracle_widen(const void* src, int64_t n, int dtype, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = widen(src, (size_t)i, dtype);
}

/*
 * Block pool (ForgeLLM README, feature list: physical KV blocks behind
 * per-request logical block tables, worst-case admission reservation,
 * reclamation and capacity errors; LLM-Inference-Engine README, the "why
 * paged KV cache" paragraph and the request-journey figure: fixed-size blocks
 * from a preallocated pool, handed to a request on demand as it grows).
 *
 * The pool is a stack of free block ids, free_ids[0 .. top), the top at
 * index top - 1, and a state record of 8 int32:
 *   [0] top: free blocks        [1] sequences refused for lack of blocks
 *   [2] lowest top since init   [3] release calls refused (stack would overflow)
 *   [4..7] zero between calls
 *
 * init: the ids 0 .. num_free - 1, stacked so that pops yield them in
 *   increasing order.
 * assign: sequences are taken in order.  Sequence s has L = context_lens[s]
 *   positions after the call, the newest n of them new (n = query_start[s+1] -
 *   query_start[s], or 1 without query_start), so it already holds
 *   have = ceil((L - n) / B) blocks and needs ceil(L / B) - have more.  A
 *   sequence needing none is always served; otherwise it is served when the
 *   stack still holds what it needs and no earlier sequence was refused, and
 *   takes that many ids off the top, the first one popped becoming its block
 *   `have`.  Each new token's slot is block_table[s][p / B] * B + p % B for its
 *   position p = L - n + i; a refused sequence's tokens (and positions below
 *   0) get -1 and its table is left alone.
 * release: the listed sequences (in list order; ids outside [0, S) hold
 *   nothing) push blocks 0 .. ceil(L / B) - 1 of their tables, in that order,
 *   and those table entries become -1; if the stack would then hold more than
 *   `capacity` ids, nothing changes and state[3] counts the refusal.
 */
void oracle_pool_init(int32_t* free_ids, int32_t* state, int32_t num_free) {
    for (int32_t i = 0; i < num_free; ++i) free_ids[i] = num_free - 1 - i;
    for (int k = 0; k < 8; ++k) state[k] = 0;
    state[0] = num_free;
    state[2] = num_free;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int oracle_assign_slots(const int32_t* ctx, const int32_t* qs, int32_t* bt, const int32_t* free_ids, int32_t* state,
                        int64_t* slots, int S, int M, int B) {
    if (S < 0 || M < 0 || B <= 0) return 1;
    int refusing = 0;
    for (int s = 0; s < S; ++s) {
        int64_t L = ctx[s];
        if (L < 0) L = 0;
        if (L > (int64_t)M * B) L = (int64_t)M * B;
        const int64_t row0 = qs ? qs[s] : s;
        const int64_t n = qs ? qs[s + 1] - qs[s] : 1;
        const int64_t first = L - n;
        const int64_t have = first > 0 ? ceil_div(first, B) : 0;
        const int64_t need = ceil_div(L, B) - have;
        int served = 1;
        if (need > 0) {
            if (refusing || need > state[0]) {
                refusing = 1;
                served = 0;
                state[1] += 1;
            } else {
                for (int64_t k = 0; k < need; ++k) {
                    state[0] -= 1;
                    bt[(size_t)s * M + have + k] = free_ids[state[0]];
                }
            }
        }
        for (int64_t i = 0; i < n; ++i) {
            const int64_t p = first + i;
            slots[row0 + i] = (served && p >= 0) ? (int64_t)bt[(size_t)s * M + p / B] * B + p % B : -1;
        }
    }
    if (state[0] < state[2]) state[2] = state[0];
    return 0;
}

int oracle_release_seqs(const int32_t* ids, int R, const int32_t* ctx, int32_t* bt, int32_t* free_ids, int32_t* state,
                        int S, int M, int B, int32_t capacity) {
    if (R < 0 || S < 0 || M < 0 || B <= 0) return 1;
    int64_t total = 0;
    for (int r = 0; r < R; ++r) {
        const int s = ids[r];
        if (s < 0 || s >= S) continue;
        int64_t L = ctx[s] < 0 ? 0 : ctx[s];
        if (L > (int64_t)M * B) L = (int64_t)M * B;
        total += ceil_div(L, B);
    }
    if (state[0] + total > capacity) {
        state[3] += 1;
        return 0;
    }
    for (int r = 0; r < R; ++r) {
        const int s = ids[r];
        if (s < 0 || s >= S) continue;
        int64_t L = ctx[s] < 0 ? 0 : ctx[s];
        if (L > (int64_t)M * B) L = (int64_t)M * B;
        for (int64_t j = 0; j < ceil_div(L, B); ++j) {
            free_ids[state[0]] = bt[(size_t)s * M + j];
            state[0] += 1;
            bt[(size_t)s * M + j] = -1;
        }
    }
    return 0;
}

/*
 * RMSNorm (ForgeLLM README, feature list: RMSNorm in the Llama-family decoder,
 * with a reference, a fused and a compiled kernel checked against each
 * other).  For each row x of H values and the weight w:
 *   ms = (1/H) * sum_d x_d^2,   y_d = x_d * w_d / sqrt(ms + eps)
 * in double, sums in index order; out holds y before any rounding.  With a
 * residual (the fused form a decoder uses between sublayers), the row first
 * becomes h = round_to_dtype(x + residual), which is stored back as the new
 * residual (res_out, doubles the dtype holds exactly), and h is normalised.
 * x, residual: [T][H], w: [H], all in the storage dtype; eps is the float
 * value the caller passes, widened exactly.
 */
int oracle_rmsnorm(const void* x, const void* residual, const void* w, double* out, double* res_out, int64_t T,
                   int H, int dtype, double eps) {
    if (H <= 0 || T < 0 || eps < 0) return -1;
    double* h = (double*)malloc(sizeof(double) * (size_t)H);
    if (!h) return -2;
    for (int64_t t = 0; t < T; ++t) {
        const size_t row = (size_t)t * H;
        for (int d = 0; d < H; ++d) h[d] = widen(x, row + d, dtype);
        if (residual) {
            for (int d = 0; d < H; ++d) h[d] += widen(residual, row + d, dtype);
            oracle_round(h, H, dtype, h);
            for (int d = 0; d < H; ++d) res_out[row + d] = h[d];
        }
        double ss = 0.0;
        for (int d = 0; d < H; ++d) ss += h[d] * h[d];
        const double r = 1.0 / sqrt(ss / H + eps);
        for (int d = 0; d < H; ++d) out[row + d] = h[d] * widen(w, (size_t)d, dtype) * r;
    }
    free(h);
    return 0;
}
