/*
 * Plain CPU oracle for the table-batched embedding (TBE) forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls this code;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no code, header or table with the GPU library.
 *
 * Everything is the plain definition written out, in fp64, one loop at a time:
 *
 *  - forward: PyTorch blog "Modernizing Table Batched Embeddings with FBTriton",
 *    section 2 (each bag gathers its rows, scales each by its per-sample weight
 *    if any, and sums them into one D-wide output row) and the layout of
 *    "Table-Batched Embeddings in Triton", section 1 (table-major offsets of
 *    length T*B+1, tables concatenated, output B x sum_t D_t);
 *  - transpose: same blog, section 3 (transpose_embedding_input turns the
 *    batch into runs, one per unique (table, row)); the tutorial's section 2
 *    uses a stable sort of the linearized row id, which fixes the order of
 *    lookups inside a run;
 *  - backward: same blog, section 3 (sum the upstream gradient rows of every
 *    lookup of a run, then exactly one optimizer step per touched row; with
 *    per-sample weights a lookup's gradient row is multiplied by its weight
 *    before it is added);
 *    SGD as in the blog's backward-pass goal (w - lr*grad); row-wise Adagrad
 *    as in the tutorial's section 5 (one fp32 state per row, state += mean of
 *    g^2 over the row, w -= lr*g/(sqrt(state)+eps), using the new state);
 *  - bounds check: the blog's "Bounds checking" paragraph says invalid inputs
 *    are validated and repaired but gives no rule; the rule used here is:
 *    offsets become a clamped running maximum with o[0]=0 and o[T*B]=N, and
 *    an index outside [0, E_t) becomes 0; each repaired entry is counted.
 *
 * Rounding to the storage dtype (fp32 / fp16 / bf16) is round-to-nearest-even
 * of the fp64 result, written from the IEEE 754 encodings.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_SGD = 0, OR_ROWWISE_ADAGRAD = 1 };

/* ------------------------------------------------------------------------ */
/* rounding of a double to the storage formats (round to nearest, ties even) */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormal quantum 2^-24 */
uint16_t oracle_round_f16(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return sign | 0x7e00;
    if (a < 0x1p-14) {                       /* subnormal (or zero): count quanta of 2^-24 */
        double r = nearbyint(a * 0x1p24);    /* r <= 1024; 1024 encodes the smallest normal */
        return sign | (uint16_t)r;
    }
    int e;
    frexp(a, &e);                            /* a = m * 2^e, 0.5 <= m < 1 */
    int E = e - 1;                           /* a = 1.f * 2^E */
    double r = nearbyint(ldexp(a, 10 - E));  /* significand in units of 2^(E-10): [1024, 2048] */
    if (r == 2048.0) { r = 1024.0; E += 1; }
    if (E > 15) return sign | 0x7c00;        /* overflow to infinity */
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024);
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits; subnormal quantum 2^-133 */
uint16_t oracle_round_bf16(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return sign | 0x7fc0;
    if (a < 0x1p-126) {
        double r = nearbyint(a * 0x1p133);   /* r <= 128; 128 encodes the smallest normal */
        return sign | (uint16_t)r;
    }
    int e;
    frexp(a, &e);
    int E = e - 1;
    double r = nearbyint(ldexp(a, 7 - E));   /* [128, 256] */
    if (r == 256.0) { r = 128.0; E += 1; }
    if (E > 127) return sign | 0x7f80;
    return sign | (uint16_t)((E + 127) << 7) | (uint16_t)((int)r - 128);
}

/* bits of x rounded to the storage dtype, widened to 32 bits */
uint32_t oracle_round_bits(int dtype, double x) {
    if (dtype == OR_F16) return oracle_round_f16(x);
    if (dtype == OR_BF16) return oracle_round_bf16(x);
    float f = (float)x;                      /* C conversion: nearest, ties to even */
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

void oracle_round_array(int dtype, const double* x, int64_t n, uint32_t* bits) {
    for (int64_t i = 0; i < n; ++i) bits[i] = oracle_round_bits(dtype, x[i]);
}

/* ------------------------------------------------------------------------ */
/* layout helpers                                                           */
/* ------------------------------------------------------------------------ */

/* first element of table t in the flat weight buffer: sum_{t'<t} E_t' * D_t' */
static int64_t weight_base(const int64_t* E, const int64_t* D, int64_t t) {
    int64_t s = 0;
    for (int64_t u = 0; u < t; ++u) s += E[u] * D[u];
    return s;
}
/* first column of table t in an output row: sum_{t'<t} D_t' */
static int64_t column_base(const int64_t* D, int64_t t) {
    int64_t s = 0;
    for (int64_t u = 0; u < t; ++u) s += D[u];
    return s;
}
/* first linearized row id of table t: sum_{t'<t} E_t' */
static int64_t row_base(const int64_t* E, int64_t t) {
    int64_t s = 0;
    for (int64_t u = 0; u < t; ++u) s += E[u];
    return s;
}

/* ------------------------------------------------------------------------ */
/* forward                                                                  */
/* ------------------------------------------------------------------------ */

/*
 * out[b][col_t + d] = sum_{j in bag(t, b)} psw_j * W_t[indices[j]][d]   (psw = 1 if NULL)
 * out_abs holds the same sum of absolute values (for the error bound).
 * W holds every table as double, concatenated.  Returns 0, or -1 on an index
 * outside its table, or -2 on a bag with decreasing offsets.
 */
int oracle_forward(int64_t T, int64_t B, const int64_t* E, const int64_t* D,
                   const double* W, const int64_t* indices, const int64_t* offsets,
                   const double* psw, double* out, double* out_abs) {
    int64_t width = column_base(D, T);
    for (int64_t t = 0; t < T; ++t) {
        const double* Wt = W + weight_base(E, D, t);
        int64_t col = column_base(D, t);
        for (int64_t b = 0; b < B; ++b) {
            int64_t s = offsets[t * B + b], e = offsets[t * B + b + 1];
            if (e < s) return -2;
            double* o = out + b * width + col;
            double* oa = out_abs + b * width + col;
            for (int64_t d = 0; d < D[t]; ++d) { o[d] = 0.0; oa[d] = 0.0; }
            for (int64_t j = s; j < e; ++j) {
                int64_t r = indices[j];
                if (r < 0 || r >= E[t]) return -1;
                double wgt = psw ? psw[j] : 1.0;
                for (int64_t d = 0; d < D[t]; ++d) {
                    double term = wgt * Wt[r * D[t] + d];
                    o[d] += term;
                    oa[d] += fabs(term);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* transpose: linearize, stable sort, run-length encode                     */
/* ------------------------------------------------------------------------ */

typedef struct { int64_t key, pos; } key_pos;

static int cmp_key_pos(const void* a, const void* b) {
    const key_pos* x = (const key_pos*)a;
    const key_pos* y = (const key_pos*)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;  /* ties keep storage order: stable */
    return 0;
}

/*
 * Lookup j of bag (t, b) gets key = sum_{t'<t} E_t' + indices[j] and bag id
 * t*B + b.  Lookups are sorted by (key, j); runs are maximal equal-key
 * stretches.  Outputs (each sized N): sorted_key, sorted_pos, sorted_bag,
 * run_key / run_start / run_len (first num_runs entries used).
 * Returns num_runs, or -1 on an index outside its table, -2 on bad offsets,
 * -3 on allocation failure.
 */
int64_t oracle_transpose(int64_t T, int64_t B, const int64_t* E,
                         const int64_t* indices, const int64_t* offsets,
                         int64_t* sorted_key, int64_t* sorted_pos, int64_t* sorted_bag,
                         int64_t* run_key, int64_t* run_start, int64_t* run_len) {
    int64_t N = T * B > 0 ? offsets[T * B] : 0;
    if (N == 0) return 0;
    key_pos* kp = (key_pos*)malloc(sizeof(key_pos) * (size_t)N);
    int64_t* bag_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (!kp || !bag_of) { free(kp); free(bag_of); return -3; }
    for (int64_t t = 0; t < T; ++t) {
        int64_t base = row_base(E, t);
        for (int64_t b = 0; b < B; ++b) {
            int64_t s = offsets[t * B + b], e = offsets[t * B + b + 1];
            if (e < s || s < 0 || e > N) { free(kp); free(bag_of); return -2; }
            for (int64_t j = s; j < e; ++j) {
                if (indices[j] < 0 || indices[j] >= E[t]) { free(kp); free(bag_of); return -1; }
                kp[j].key = base + indices[j];
                kp[j].pos = j;
                bag_of[j] = t * B + b;
            }
        }
    }
    qsort(kp, (size_t)N, sizeof(key_pos), cmp_key_pos);
    int64_t runs = 0;
    for (int64_t i = 0; i < N; ++i) {
        sorted_key[i] = kp[i].key;
        sorted_pos[i] = kp[i].pos;
        sorted_bag[i] = bag_of[kp[i].pos];
        if (i == 0 || kp[i].key != kp[i - 1].key) {
            run_key[runs] = kp[i].key;
            run_start[runs] = i;
            run_len[runs] = 0;
            ++runs;
        }
        run_len[runs - 1] += 1;
    }
    free(kp);
    free(bag_of);
    return runs;
}

/* table that owns linearized row `key` */
static int64_t table_of_key(int64_t T, const int64_t* E, int64_t key) {
    int64_t base = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (key < base + E[t]) return t;
        base += E[t];
    }
    return -1;
}

static int64_t next_pow2(int64_t x) {
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

/*
 * Segment-length routing (blog section 3 and section 4, problems 1 and 3):
 * a run is long iff run_len >= threshold, and then covers ceil(len / chunk)
 * chunks; a short run goes to bucket next_pow2(D_t) of its table.
 * is_long[r] in {0,1}, bucket[r] = next_pow2(D) for short runs and 0 for long,
 * nchunks[r] = chunks of a long run (0 for short).  Returns total chunks.
 */
int64_t oracle_classify(int64_t T, const int64_t* E, const int64_t* D, int64_t num_runs,
                        const int64_t* run_key, const int64_t* run_len,
                        int64_t threshold, int64_t chunk,
                        int8_t* is_long, int64_t* bucket, int64_t* nchunks) {
    int64_t total = 0;
    for (int64_t r = 0; r < num_runs; ++r) {
        int64_t t = table_of_key(T, E, run_key[r]);
        if (run_len[r] >= threshold) {
            is_long[r] = 1;
            bucket[r] = 0;
            nchunks[r] = (run_len[r] + chunk - 1) / chunk;
            total += nchunks[r];
        } else {
            is_long[r] = 0;
            bucket[r] = next_pow2(D[t]);
            nchunks[r] = 0;
        }
    }
    return total;
}

/* ------------------------------------------------------------------------ */
/* backward                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * For every run (unique key k of table t, row r = k - rowbase_t):
 *   g[d] = sum_{j in run} psw_j * grad_out[bag_j][col_t + d]        (fp64)
 *   SGD:       w' = w - lr * g
 *   Adagrad:   m' = m + (sum_d g[d]^2) / D_t ;  w' = w - lr * g / (sqrt(m') + eps)
 * Untouched rows keep w and m.  Inputs: W (double, flat), momentum (double,
 * one per row; may be NULL for SGD), grad_out (double, B x width).
 * Outputs (flat like W unless noted): g, g_abs (sum of |psw_j*grad|),
 * w_new (unrounded), w_bits (w_new rounded to w_dtype), m_new / m_f32 (one per
 * row), touched (one per row).  Returns number of runs, or < 0 on error.
 */
int64_t oracle_backward(int64_t T, int64_t B, const int64_t* E, const int64_t* D, int w_dtype,
                        const double* W, const int64_t* indices, const int64_t* offsets,
                        const double* psw, const double* grad_out, int optimizer,
                        double lr, double eps, const double* momentum,
                        double* g, double* g_abs, double* w_new, uint32_t* w_bits,
                        double* m_new, float* m_f32, int8_t* touched) {
    int64_t N = T * B > 0 ? offsets[T * B] : 0;
    int64_t width = column_base(D, T);
    int64_t rows = row_base(E, T);
    int64_t elems = weight_base(E, D, T);
    for (int64_t i = 0; i < elems; ++i) {
        g[i] = 0.0;
        g_abs[i] = 0.0;
        w_new[i] = W[i];
        w_bits[i] = oracle_round_bits(w_dtype, W[i]);
    }
    for (int64_t r = 0; r < rows; ++r) {
        double m = momentum ? momentum[r] : 0.0;
        m_new[r] = m;
        m_f32[r] = (float)m;
        touched[r] = 0;
    }
    if (N == 0) return 0;
    int64_t* sk = (int64_t*)malloc(sizeof(int64_t) * (size_t)N * 6);
    if (!sk) return -3;
    int64_t *sp = sk + N, *sb = sk + 2 * N, *rk = sk + 3 * N, *rs = sk + 4 * N, *rl = sk + 5 * N;
    int64_t runs = oracle_transpose(T, B, E, indices, offsets, sk, sp, sb, rk, rs, rl);
    if (runs < 0) { free(sk); return runs; }
    for (int64_t q = 0; q < runs; ++q) {
        int64_t t = table_of_key(T, E, rk[q]);
        int64_t row = rk[q] - row_base(E, t);
        int64_t Dt = D[t];
        int64_t wb = weight_base(E, D, t) + row * Dt;
        int64_t col = column_base(D, t);
        /* 1. sum the gradient rows of every lookup of the run */
        for (int64_t i = rs[q]; i < rs[q] + rl[q]; ++i) {
            int64_t j = sp[i];
            int64_t b = sb[i] % B;
            double wgt = psw ? psw[j] : 1.0;
            for (int64_t d = 0; d < Dt; ++d) {
                double term = wgt * grad_out[b * width + col + d];
                g[wb + d] += term;
                g_abs[wb + d] += fabs(term);
            }
        }
        /* 2. exactly one optimizer step on the summed gradient */
        touched[rk[q]] = 1;
        if (optimizer == OR_SGD) {
            for (int64_t d = 0; d < Dt; ++d) w_new[wb + d] = W[wb + d] - lr * g[wb + d];
        } else {
            double ss = 0.0;
            for (int64_t d = 0; d < Dt; ++d) ss += g[wb + d] * g[wb + d];
            double m = (momentum ? momentum[rk[q]] : 0.0) + ss / (double)Dt;
            m_new[rk[q]] = m;
            m_f32[rk[q]] = (float)m;
            double denom = sqrt(m) + eps;
            for (int64_t d = 0; d < Dt; ++d) w_new[wb + d] = W[wb + d] - lr * g[wb + d] / denom;
        }
        for (int64_t d = 0; d < Dt; ++d) w_bits[wb + d] = oracle_round_bits(w_dtype, w_new[wb + d]);
    }
    (void)rows;
    free(sk);
    return runs;
}

/* ------------------------------------------------------------------------ */
/* bounds check and repair                                                  */
/* ------------------------------------------------------------------------ */

/*
 * offsets (length T*B+1) and indices (length N) are repaired in place:
 *   o'[0] = 0, o'[T*B] = N, o'[i] = max(o'[i-1], min(max(o[i], 0), N));
 *   then for each table t, every index in [o'[t*B], o'[(t+1)*B]) outside
 *   [0, E_t) becomes 0.
 * counts[0] = indices repaired, counts[1] = offsets entries changed.
 */
void oracle_bounds_check(int64_t T, int64_t B, const int64_t* E, int64_t* indices, int64_t N,
                         int64_t* offsets, int64_t* counts) {
    int64_t nb = T * B;
    counts[0] = 0;
    counts[1] = 0;
    int64_t prev = 0;
    for (int64_t i = 0; i <= nb; ++i) {
        int64_t v;
        if (i == 0) v = 0;
        else if (i == nb) v = N;
        else {
            v = offsets[i];
            if (v < 0) v = 0;
            if (v > N) v = N;
            if (v < prev) v = prev;
        }
        if (i == nb && v < prev) v = prev;  /* cannot happen: prev <= N */
        if (v != offsets[i]) counts[1] += 1;
        offsets[i] = v;
        prev = v;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = offsets[t * B]; j < offsets[(t + 1) * B]; ++j) {
            if (indices[j] < 0 || indices[j] >= E[t]) {
                indices[j] = 0;
                counts[0] += 1;
            }
        }
    }
}
