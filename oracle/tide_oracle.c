/*
 * CPU oracle for the layout-aware FSDP2 reduce-scatter local stage, the
 * all-gather copy-out and the all-gather copy-in.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file.  Only the test suite, the package's smoke check and
 * the benchmark's CPU-baseline leg use it.  It shares no source with the HIP
 * library: the shard geometry, the bf16 widening and the summation are all
 * written out again here, in plain loops, from the definitions in
 *
 *   "The Endgame of FSDP Communication: Layout-Aware Collectives on Copy
 *    Engines, RDMA, and NVSwitch" (Wang et al.)
 *     - Section 2.1 "The Layout Mismatch in FSDP2": the dimension-0 shard
 *       geometry, the rank-major all-gather buffer, the parameter-major
 *       landing offset (Equation 2) and the rows each destination owns;
 *     - Section 4 "TIDE-RS": the reduce-scatter result (Equation 5);
 *     - Section 4.3 "Numerical Semantics and Determinism": fp32 accumulation
 *       that never narrows a partial;
 *     - Section 3.1 "In-Place Shards and Paced Doubling": mixed-precision
 *       groups cast their fp32 shards to bf16 on the way into the all-gather;
 *     - Section 2.2 and Table 4: the memory-bound elementwise victim of the
 *       interference measurements.
 *
 * Readings taken where the pages leave a step open (each is also listed with
 * the design notes of this repository):
 *   - sizes are counted in elements, not bytes (the pages' byte sizes are the
 *     element counts times the item size);
 *   - contributions are summed in rank order 0, 1, ..., W-1 for every
 *     destination, the accumulator starting from rank 0's widened value;
 *   - each addition is one IEEE-754 binary32 addition, round to nearest even,
 *     subnormals kept, no fused operations;
 *   - alpha = 1 and accumulate = 0 (Equation 5's defaults): the finished sum
 *     is stored as is, with no added +0;
 *   - otherwise alpha scales the finished fp32 sum once (one binary32
 *     multiplication) and accumulate adds the scaled sum to the existing
 *     output (one binary32 addition); padding rows count as rows of zeros;
 *   - fp32 gradients are taken as is (no widening);
 *   - output elements of padding rows (rows at or past D_p) are +0.0f;
 *   - the copy-out writes the unpadded per-parameter tensor of D_p * K_p
 *     elements and never reads the padding of a shard;
 *   - the copy-in takes each rank's local shard as its n_real(p, r) elements
 *     (unpadded rows), casts fp32 to bf16 by round to nearest even (a NaN
 *     stays a quiet NaN of the same sign and top payload bits), and writes
 *     bf16 +0 into the padding;
 *   - a parameter must have at least one dimension; a 1-D parameter has
 *     K_p = 1; zero-sized dimensions are allowed;
 *   - the pages name their elementwise victim without its operation; here it
 *     is y = a * x + b over fp32 arrays, the product and the sum each rounded
 *     to binary32 (no fused multiply-add).
 *
 * Pins: every function here is checked against hand-derived values, closed
 * forms, invariants and brute force by the CPU tests of this repository.
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float arithmetic evaluated in binary32"
#endif

#define ORACLE_OK 0
#define ORACLE_INVALID (-1)
#define ORACLE_NOMEM (-4)

/* ------------------------------------------------------------------------
 * Shard geometry (Section 2.1).
 *
 * Parameter p, of shape (d_0, d_1, ..., d_{m-1}), is viewed as D_p rows of
 * K_p elements: D_p = d_0 and K_p = d_1 * ... * d_{m-1} (1 when m = 1).
 * Each of the W ranks owns R_p = ceil(D_p / W) rows, padded: rank r owns
 * rows [r R_p, (r+1) R_p) and rows at or past D_p are padding.
 * A rank's shard of p has n_p = R_p K_p elements; shards of the P
 * parameters sit one after the other, p's at offset o_p = sum_{i<p} n_i,
 * and a rank's whole shard has S = sum_p n_p elements.
 * ------------------------------------------------------------------------ */
typedef struct {
    int32_t W, P;
    int64_t *D, *K, *R, *n, *o;
    int64_t S;
} geometry;

static void geometry_free(geometry* g) {
    free(g->D);
    free(g->K);
    free(g->R);
    free(g->n);
    free(g->o);
    memset(g, 0, sizeof(*g));
}

/* Fill g from the shapes; ORACLE_INVALID on a bad shape or int64 overflow. */
static int geometry_build(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, geometry* g) {
    memset(g, 0, sizeof(*g));
    if (W < 1 || P < 1 || ndims == NULL || dims == NULL) return ORACLE_INVALID;
    g->W = W;
    g->P = P;
    g->D = calloc((size_t)P, sizeof(int64_t));
    g->K = calloc((size_t)P, sizeof(int64_t));
    g->R = calloc((size_t)P, sizeof(int64_t));
    g->n = calloc((size_t)P, sizeof(int64_t));
    g->o = calloc((size_t)P, sizeof(int64_t));
    if (!g->D || !g->K || !g->R || !g->n || !g->o) {
        geometry_free(g);
        return ORACLE_NOMEM;
    }
    int64_t pos = 0; /* position of parameter p's first dimension in dims */
    int64_t offset = 0;
    for (int32_t p = 0; p < P; ++p) {
        if (ndims[p] < 1) {
            geometry_free(g);
            return ORACLE_INVALID;
        }
        int64_t D = dims[pos];
        int64_t K = 1;
        for (int32_t j = 1; j < ndims[p]; ++j) {
            if (dims[pos + j] < 0 || __builtin_mul_overflow(K, dims[pos + j], &K)) {
                geometry_free(g);
                return ORACLE_INVALID;
            }
        }
        int64_t total;
        if (D < 0 || __builtin_mul_overflow(D, K, &total)) {
            geometry_free(g);
            return ORACLE_INVALID;
        }
        pos += ndims[p];
        int64_t R = (D + W - 1) / W; /* ceil(D / W); 0 when D = 0 */
        int64_t n;
        if (__builtin_mul_overflow(R, K, &n)) {
            geometry_free(g);
            return ORACLE_INVALID;
        }
        g->D[p] = D;
        g->K[p] = K;
        g->R[p] = R;
        g->n[p] = n;
        g->o[p] = offset;
        if (__builtin_add_overflow(offset, n, &offset)) {
            geometry_free(g);
            return ORACLE_INVALID;
        }
    }
    int64_t whole;
    if (__builtin_mul_overflow(offset, (int64_t)W, &whole)) {
        geometry_free(g);
        return ORACLE_INVALID;
    }
    g->S = offset;
    return ORACLE_OK;
}

/* Number of real (non-padding) rows of parameter p held by rank r. */
static int64_t real_rows(const geometry* g, int32_t p, int32_t r) {
    int64_t first = (int64_t)r * g->R[p];
    int64_t rows = g->D[p] - first;
    if (rows < 0) rows = 0;
    if (rows > g->R[p]) rows = g->R[p];
    return rows;
}

/*
 * oracle_plan: the shard geometry and the per-(parameter, rank) placement.
 *
 * Outputs (caller-allocated):
 *   D, K, R, n, o      [P]     as defined above
 *   S                  [1]     per-rank shard elements
 *   n_real             [P*W]   index p*W + r: real elements of p held by r
 *   rank_major_offset  [P*W]   element offset of r's shard of p in the
 *                              rank-major all-gather buffer: r S + o_p
 *   landing_offset     [P*W]   element offset of the same shard in the
 *                              parameter-major landing buffer (Equation 2):
 *                              W o_p + r n_p
 */
int oracle_plan(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, int64_t* D, int64_t* K,
                int64_t* R, int64_t* n, int64_t* o, int64_t* S, int64_t* n_real, int64_t* rank_major_offset,
                int64_t* landing_offset) {
    geometry g;
    int rc = geometry_build(W, P, ndims, dims, &g);
    if (rc != ORACLE_OK) return rc;
    for (int32_t p = 0; p < P; ++p) {
        D[p] = g.D[p];
        K[p] = g.K[p];
        R[p] = g.R[p];
        n[p] = g.n[p];
        o[p] = g.o[p];
        for (int32_t r = 0; r < W; ++r) {
            n_real[(int64_t)p * W + r] = real_rows(&g, p, r) * g.K[p];
            rank_major_offset[(int64_t)p * W + r] = (int64_t)r * g.S + g.o[p];
            landing_offset[(int64_t)p * W + r] = (int64_t)W * g.o[p] + (int64_t)r * g.n[p];
        }
    }
    *S = g.S;
    geometry_free(&g);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * bf16 -> fp32.  A bf16 value is the upper half of a binary32 value, so the
 * widening is exact: put the 16 bits in the high half, zeros below.
 * ------------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t bits) {
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return f;
}

/* The x86 SSE control word must say: round to nearest even, no flush of
 * subnormal results (FTZ), no treating of subnormal inputs as zero (DAZ).
 * It is per thread, so each worker sets it for itself and restores it. */
#define MXCSR_FTZ 0x8000u
#define MXCSR_DAZ 0x0040u
#define MXCSR_RC 0x6000u

static unsigned ieee_mode_enter(void) {
    unsigned saved = _mm_getcsr();
    _mm_setcsr(saved & ~(MXCSR_FTZ | MXCSR_DAZ | MXCSR_RC));
    return saved;
}

static void ieee_mode_leave(unsigned saved) { _mm_setcsr(saved); }

/* ------------------------------------------------------------------------
 * Work split for the threaded runs.  Tasks are the (rank, parameter) pairs;
 * every output element is computed by exactly one task, the same way for
 * any thread count, so the result does not depend on the thread count.
 * ------------------------------------------------------------------------ */
typedef struct {
    const geometry* g;
    const void* const* shards;    /* [W*P], index r*P + p */
    int32_t shard_dtype;          /* 0 = bf16 bits, 1 = fp32 */
    const void* const* grads_any; /* [W*P], index u*P + p, bf16 bits or fp32 */
    int32_t grad_dtype;           /* 0 = bf16, 1 = fp32 */
    float alpha;
    int32_t accumulate;
    const uint16_t* const* grads_one; /* [P]: one rank's gradients */
    float* packed;                /* [W*S] */
    const uint16_t* const* grads; /* [W*P], index u*P + p */
    float* const* out;            /* [W] */
    const uint16_t* rank_major;   /* [W*S] */
    uint16_t* const* params;      /* [P] */
    uint16_t* rank_major_out;     /* [W*S] */
    const uint16_t* const* params_in; /* [P] */
    int32_t nthreads;
    int32_t tid;
} job;

/*
 * Reduce-scatter, one task: destination rank r, parameter p (Equation 5 with
 * alpha = 1, accumulate = 0):
 *   out_r[o_p + e] = G_p^(0)[i] + G_p^(1)[i] + ... + G_p^(W-1)[i],
 *   i = r R_p K_p + e, for e below the real element count; +0.0f past it.
 */
static void rs_task(const job* j, int32_t r, int32_t p) {
    const geometry* g = j->g;
    int64_t real = real_rows(g, p, r) * g->K[p];
    int64_t first = (int64_t)r * g->R[p] * g->K[p];
    float* dst = j->out[r] + g->o[p];
    for (int64_t e = 0; e < g->n[p]; ++e) {
        if (e < real) {
            int64_t i = first + e;
            float acc = bf16_to_f32(j->grads[(int64_t)0 * g->P + p][i]);
            for (int32_t u = 1; u < g->W; ++u) acc = acc + bf16_to_f32(j->grads[(int64_t)u * g->P + p][i]);
            dst[e] = acc;
        } else {
            dst[e] = 0.0f;
        }
    }
}

/* Contribution of rank u to element i of parameter p, widened to fp32 (an
 * fp32 gradient is taken as is). */
static float grad_value(const job* j, int32_t u, int32_t p, int64_t i) {
    const void* t = j->grads_any[(int64_t)u * j->g->P + p];
    if (j->grad_dtype == 1) return ((const float*)t)[i];
    return bf16_to_f32(((const uint16_t*)t)[i]);
}

/*
 * Reduce-scatter in the general form of Equation 5, one task (r, p):
 *   out_r[o_p + e] <- (accumulate ? out_r[o_p + e] : 0) + alpha * sum_u g_u
 * with the sum taken in rank order as in rs_task, alpha applied once to the
 * finished fp32 sum (one binary32 multiplication), and the accumulation one
 * binary32 addition; with accumulate off the scaled sum is stored as is.
 * Padding rows are rows of zeros in every rank (Section 2.1), so their sum
 * is +0.  rs_task is the alpha = 1, accumulate off, bf16 case on its own.
 */
static void rs_general_task(const job* j, int32_t r, int32_t p) {
    const geometry* g = j->g;
    int64_t real = real_rows(g, p, r) * g->K[p];
    int64_t first = (int64_t)r * g->R[p] * g->K[p];
    float* dst = j->out[r] + g->o[p];
    for (int64_t e = 0; e < g->n[p]; ++e) {
        float sum = 0.0f;
        if (e < real) {
            sum = grad_value(j, 0, p, first + e);
            for (int32_t u = 1; u < g->W; ++u) sum = sum + grad_value(j, u, p, first + e);
        }
        float v = j->alpha * sum;
        dst[e] = j->accumulate ? dst[e] + v : v;
    }
}

/* Stock FSDP2's gradient packing for one source rank (Section 2.1, Equation
 * 3: slice, zero-pad, upcast, pack): rank u's bf16 gradient rows that
 * destination r owns go, widened to fp32, to packed[r S + o_p + e]; padding
 * rows are +0.0f. */
static void chunk_cat_task(const job* j, int32_t r, int32_t p) {
    const geometry* g = j->g;
    int64_t real = real_rows(g, p, r) * g->K[p];
    const uint16_t* src = j->grads_one[p] + (int64_t)r * g->R[p] * g->K[p];
    float* dst = j->packed + (int64_t)r * g->S + g->o[p];
    for (int64_t e = 0; e < g->n[p]; ++e) dst[e] = (e < real) ? bf16_to_f32(src[e]) : 0.0f;
}

/* Copy-out, one task: rank r's shard of parameter p lands in the parameter's
 * own storage at the rows that rank owns; padding is not read. */
static void copyout_task(const job* j, int32_t r, int32_t p) {
    const geometry* g = j->g;
    int64_t real = real_rows(g, p, r) * g->K[p];
    const uint16_t* src = j->rank_major + (int64_t)r * g->S + g->o[p];
    uint16_t* dst = j->params[p] + (int64_t)r * g->R[p] * g->K[p];
    for (int64_t e = 0; e < real; ++e) dst[e] = src[e];
}

/* fp32 -> bf16, round to nearest, ties to even, done on the bit pattern:
 * add half of the dropped 16-bit tail (minus one unless the kept part is
 * odd) and truncate; overflow carries into the exponent and gives +-inf.
 * A NaN stays a NaN of the same sign with its top payload bits and the quiet
 * bit set. */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_odd = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + keep_odd) >> 16);
}

/* All-gather copy-in, one task: rank r's local shard of parameter p (its
 * n_real(p, r) elements, fp32 master weights cast to bf16, or bf16 as is) is
 * written into the rank-major buffer at r S + o_p, the padding of the slot as
 * bf16 +0.  (FSDP2's copy-in, Section 2.1; the cast is the mixed-precision
 * one of Section 3.1.) */
static void copyin_task(const job* j, int32_t r, int32_t p) {
    const geometry* g = j->g;
    int64_t real = real_rows(g, p, r) * g->K[p];
    uint16_t* dst = j->rank_major_out + (int64_t)r * g->S + g->o[p];
    const void* src = j->shards[(int64_t)r * g->P + p];
    for (int64_t e = 0; e < g->n[p]; ++e) {
        if (e >= real) {
            dst[e] = 0;
        } else if (j->shard_dtype == 1) {
            dst[e] = f32_to_bf16_rne(((const float*)src)[e]);
        } else {
            dst[e] = ((const uint16_t*)src)[e];
        }
    }
}

/* Pack (the inverse of the copy-out; FSDP2's all-gather copy-in): rank r's
 * shard of parameter p is written into the rank-major buffer, padding as
 * bf16 +0 (0x0000). */
static void pack_task(const job* j, int32_t r, int32_t p) {
    const geometry* g = j->g;
    int64_t real = real_rows(g, p, r) * g->K[p];
    const uint16_t* src = j->params_in[p] + (int64_t)r * g->R[p] * g->K[p];
    uint16_t* dst = j->rank_major_out + (int64_t)r * g->S + g->o[p];
    for (int64_t e = 0; e < g->n[p]; ++e) dst[e] = (e < real) ? src[e] : (uint16_t)0;
}

typedef void (*task_fn)(const job*, int32_t, int32_t);

typedef struct {
    job j;
    task_fn fn;
} worker_arg;

static void* worker(void* arg) {
    worker_arg* a = (worker_arg*)arg;
    unsigned saved = ieee_mode_enter();
    int64_t ntasks = (int64_t)a->j.g->W * a->j.g->P;
    for (int64_t t = a->j.tid; t < ntasks; t += a->j.nthreads) {
        int32_t r = (int32_t)(t / a->j.g->P);
        int32_t p = (int32_t)(t % a->j.g->P);
        a->fn(&a->j, r, p);
    }
    ieee_mode_leave(saved);
    return NULL;
}

static int run_tasks(job base, task_fn fn, int32_t nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    worker_arg* args = calloc((size_t)nthreads, sizeof(worker_arg));
    pthread_t* th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!args || !th) {
        free(args);
        free(th);
        return ORACLE_NOMEM;
    }
    int32_t started = 0;
    for (int32_t t = 0; t < nthreads; ++t) {
        args[t].j = base;
        args[t].j.nthreads = nthreads;
        args[t].j.tid = t;
        args[t].fn = fn;
    }
    if (nthreads == 1) {
        worker(&args[0]);
    } else {
        for (int32_t t = 0; t < nthreads; ++t) {
            if (pthread_create(&th[t], NULL, worker, &args[t]) != 0) break;
            ++started;
        }
        for (int32_t t = 0; t < started; ++t) pthread_join(th[t], NULL);
        /* A thread that could not be started: do its share here. */
        for (int32_t t = started; t < nthreads; ++t) worker(&args[t]);
    }
    free(args);
    free(th);
    return ORACLE_OK;
}

/*
 * oracle_rs_local: the reduce-scatter local stage over W simulated ranks.
 *   grads  [W*P]  grads[u*P + p] is rank u's bf16 gradient of parameter p,
 *                 D_p * K_p elements, row-major (bf16 bit patterns)
 *   out    [W]    out[r] receives rank r's packed fp32 shard, S elements
 *   nthreads      host threads to use (>= 1); the result does not depend on it
 */
int oracle_rs_local(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* const* grads,
                    float* const* out, int32_t nthreads) {
    geometry g;
    int rc = geometry_build(W, P, ndims, dims, &g);
    if (rc != ORACLE_OK) return rc;
    if (grads == NULL || out == NULL) {
        geometry_free(&g);
        return ORACLE_INVALID;
    }
    job j;
    memset(&j, 0, sizeof j);
    j.g = &g;
    j.grads = grads;
    j.out = out;
    rc = run_tasks(j, rs_task, nthreads);
    geometry_free(&g);
    return rc;
}

/*
 * oracle_copyout: all-gather copy-out.
 *   rank_major  [W*S]  rank r's shard of p at element r S + o_p
 *   params      [P]    params[p] receives D_p * K_p bf16 elements
 */
int oracle_copyout(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* rank_major,
                   uint16_t* const* params, int32_t nthreads) {
    geometry g;
    int rc = geometry_build(W, P, ndims, dims, &g);
    if (rc != ORACLE_OK) return rc;
    if (rank_major == NULL || params == NULL) {
        geometry_free(&g);
        return ORACLE_INVALID;
    }
    job j;
    memset(&j, 0, sizeof j);
    j.g = &g;
    j.rank_major = rank_major;
    j.params = params;
    rc = run_tasks(j, copyout_task, nthreads);
    geometry_free(&g);
    return rc;
}

/*
 * oracle_pack: the rank-major all-gather buffer holding every rank's shard,
 * padding zero (a test helper: builds copy-out inputs from known tensors).
 *   params      [P]    D_p * K_p bf16 elements each
 *   rank_major  [W*S]  written in full
 */
int oracle_pack(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* const* params,
                uint16_t* rank_major, int32_t nthreads) {
    geometry g;
    int rc = geometry_build(W, P, ndims, dims, &g);
    if (rc != ORACLE_OK) return rc;
    if (rank_major == NULL || params == NULL) {
        geometry_free(&g);
        return ORACLE_INVALID;
    }
    job j;
    memset(&j, 0, sizeof j);
    j.g = &g;
    j.params_in = params;
    j.rank_major_out = rank_major;
    rc = run_tasks(j, pack_task, nthreads);
    geometry_free(&g);
    return rc;
}

/*
 * oracle_copyin: every rank's all-gather copy-in, giving the rank-major buffer
 * the all-gather would produce.
 *   shards       [W*P]  shards[r*P + p] is rank r's local shard of parameter p:
 *                       n_real(p, r) elements (its rows of the parameter)
 *   shard_dtype  0 = bf16 bit patterns (copied), 1 = fp32 (cast to bf16)
 *   rank_major   [W*S]  written in full
 */
int oracle_copyin(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const void* const* shards,
                  int32_t shard_dtype, uint16_t* rank_major, int32_t nthreads) {
    geometry g;
    int rc = geometry_build(W, P, ndims, dims, &g);
    if (rc != ORACLE_OK) return rc;
    if (rank_major == NULL || shards == NULL || (shard_dtype != 0 && shard_dtype != 1)) {
        geometry_free(&g);
        return ORACLE_INVALID;
    }
    job j;
    memset(&j, 0, sizeof j);
    j.g = &g;
    j.shards = shards;
    j.shard_dtype = shard_dtype;
    j.rank_major_out = rank_major;
    rc = run_tasks(j, copyin_task, nthreads);
    geometry_free(&g);
    return rc;
}

/* oracle_cast_bf16: the element cast on its own (n values), for pinning. */
int oracle_cast_bf16(const float* x, int64_t n, uint16_t* out) {
    if ((x == NULL || out == NULL) && n > 0) return ORACLE_INVALID;
    unsigned saved = ieee_mode_enter();
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(x[i]);
    ieee_mode_leave(saved);
    return ORACLE_OK;
}

/*
 * oracle_rs_local_ex: Equation 5 in full.
 *   grads       [W*P]  bf16 bits (grad_dtype 0) or fp32 (grad_dtype 1),
 *                      grads[u*P + p] of D_p * K_p elements
 *   alpha       scale of the finished sum
 *   accumulate  0: out is written; 1: the scaled sum is added to out
 *   out         [W]    S fp32 elements each (read when accumulating)
 */
int oracle_rs_local_ex(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const void* const* grads,
                       int32_t grad_dtype, float alpha, int32_t accumulate, float* const* out, int32_t nthreads) {
    geometry g;
    int rc = geometry_build(W, P, ndims, dims, &g);
    if (rc != ORACLE_OK) return rc;
    if (grads == NULL || out == NULL || (grad_dtype != 0 && grad_dtype != 1)) {
        geometry_free(&g);
        return ORACLE_INVALID;
    }
    job j;
    memset(&j, 0, sizeof j);
    j.g = &g;
    j.grads_any = grads;
    j.grad_dtype = grad_dtype;
    j.alpha = alpha;
    j.accumulate = accumulate != 0;
    j.out = out;
    rc = run_tasks(j, rs_general_task, nthreads);
    geometry_free(&g);
    return rc;
}

/*
 * oracle_chunk_cat: stock FSDP2's packed fp32 reduce-scatter input of one
 * source rank.
 *   grads   [P]    that rank's bf16 gradients, D_p * K_p elements each
 *   packed  [W*S]  written in full
 */
int oracle_chunk_cat(int32_t W, int32_t P, const int32_t* ndims, const int64_t* dims, const uint16_t* const* grads,
                     float* packed, int32_t nthreads) {
    geometry g;
    int rc = geometry_build(W, P, ndims, dims, &g);
    if (rc != ORACLE_OK) return rc;
    if (grads == NULL || packed == NULL) {
        geometry_free(&g);
        return ORACLE_INVALID;
    }
    job j;
    memset(&j, 0, sizeof j);
    j.g = &g;
    j.grads_one = grads;
    j.packed = packed;
    rc = run_tasks(j, chunk_cat_task, nthreads);
    geometry_free(&g);
    return rc;
}

/*
 * oracle_axpb: the elementwise victim of the interference measurements
 * (Section 2.2; Table 4's 256 MiB elementwise kernel), y[i] = a * x[i] + b,
 * the product rounded to binary32 and then the sum rounded to binary32.
 *   n  elements (>= 0); x, y  [n] (may be NULL only when n = 0)
 */
int oracle_axpb(int64_t n, const float* x, float a, float b, float* y) {
    if (n < 0 || (n > 0 && (x == NULL || y == NULL))) return ORACLE_INVALID;
    unsigned saved = ieee_mode_enter();
    for (int64_t i = 0; i < n; ++i) {
        volatile float prod = a * x[i]; /* one rounding, kept apart from the sum */
        y[i] = prod + b;
    }
    ieee_mode_leave(saved);
    return ORACLE_OK;
}
