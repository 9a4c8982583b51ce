/*
 * ja_oracle.c -- plain fp64 CPU oracle for jagged attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. It shares no code
 * with the HIP library. The definitions it follows are quoted by section in
 * ja_oracle.h; every loop below is the textbook definition written out, with
 * no blocking, fusion or reordering.
 */
#include "ja_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- element decoding (exact widening to double) ---------------------- */

static double elem(const void* p, int dtype, int64_t idx) {
    if (dtype == ORA_F64) return ((const double*)p)[idx];
    if (dtype == ORA_F32) return (double)((const float*)p)[idx];
    /* bf16: the 16 stored bits are the upper half of an IEEE binary32. */
    uint32_t bits = (uint32_t)((const uint16_t*)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---- activations ---------------------------------------------------------
 * GDPA section: an element-wise activation (GELU or SiLU) replaces softmax.
 * SiLU is x * sigmoid(x); GELU is the tanh form named in the same section. */

static double act_silu(double x) { return x / (1.0 + exp(-x)); }

static double act_gelu_tanh(double x) {
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* Derivatives, used by the pointwise backward. */
static double dact_silu(double x) {
    double s = 1.0 / (1.0 + exp(-x));
    return s + x * s * (1.0 - s);
}

static double dact_gelu_tanh(double x) {
    const double c = sqrt(2.0 / M_PI);
    double u = c * (x + 0.044715 * x * x * x);
    double t = tanh(u);
    double du = c * (1.0 + 3.0 * 0.044715 * x * x);
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du;
}

/* GDPA section, ALU-only activation: GELU replaced by its Taylor expansion of
 * order 6 about 0, for inputs kept small by QK-norm. With c = sqrt(2/pi),
 * a = 0.044715 and u = c (x + a x^3):
 *   tanh u = c x + (c a - c^3/3) x^3 + (2 c^5/15 - c^3 a) x^5 + O(x^7),
 * so 0.5 x (1 + tanh u) = x/2 + k2 x^2 + k4 x^4 + k6 x^6 + O(x^8) with
 *   k2 = c/2, k4 = (c a - c^3/3)/2, k6 = (2 c^5/15 - c^3 a)/2. */
static void gelu_taylor_coeffs(double* k2, double* k4, double* k6) {
    const double c = sqrt(2.0 / M_PI), a = 0.044715;
    const double c3 = c * c * c, c5 = c3 * c * c;
    *k2 = c / 2.0;
    *k4 = (c * a - c3 / 3.0) / 2.0;
    *k6 = (2.0 * c5 / 15.0 - c3 * a) / 2.0;
}

static double act_gelu_taylor(double x) {
    double k2, k4, k6;
    gelu_taylor_coeffs(&k2, &k4, &k6);
    const double x2 = x * x;
    return 0.5 * x + k2 * x2 + k4 * x2 * x2 + k6 * x2 * x2 * x2;
}

static double dact_gelu_taylor(double x) {
    double k2, k4, k6;
    gelu_taylor_coeffs(&k2, &k4, &k6);
    const double x2 = x * x;
    return 0.5 + 2.0 * k2 * x + 4.0 * k4 * x2 * x + 6.0 * k6 * x2 * x2 * x;
}

static double act_apply(int act, double x) {
    if (act == ORA_SILU) return act_silu(x);
    if (act == ORA_GELU_TAYLOR) return act_gelu_taylor(x);
    return act_gelu_tanh(x);
}

static double act_deriv(int act, double x) {
    if (act == ORA_SILU) return dact_silu(x);
    if (act == ORA_GELU_TAYLOR) return dact_gelu_taylor(x);
    return dact_gelu_tanh(x);
}

/* ---- MXFP8 ("Mixed Ultra-Low-Precision Training" section) -----------------
 * E4M3 in its "fn" form (no infinities; the top code is NaN; largest finite
 * 448 = 1.75 * 2^8): 1 sign bit, 4 exponent bits biased by 7, 3 mantissa bits;
 * exponent field 0 holds subnormals m * 2^-9. */
double ora_e4m3_decode(uint8_t b) {
    const int sgn = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* Nearest E4M3 value, ties to even, of x in [-448, 448]. */
uint8_t ora_e4m3_encode(double x) {
    const uint8_t sgn = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a < ldexp(1.0, -6)) {                 /* subnormal step 2^-9; 8 steps = 2^-6 = code 0x08 */
        const double mi = nearbyint(ldexp(a, 9));
        return (uint8_t)(sgn | (uint8_t)mi);
    }
    int ex;
    (void)frexp(a, &ex);                      /* a = f 2^ex, f in [0.5, 1) */
    int e = ex - 1;                           /* a in [2^e, 2^(e+1)) */
    double mi = nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (mi == 8.0) { mi = 0.0; ++e; }
    return (uint8_t)(sgn | (uint8_t)((e + 7) << 3) | (uint8_t)mi);
}

/* Scale exponent of one [32 x 32] block with largest magnitude amax: the shared
 * exponent floor(log2(amax)) minus E4M3's largest exponent 8, limited to the
 * E8M0 range [-127, 127]; an all-zero block takes -127. */
static int mx_block_exponent(double amax) {
    if (!(amax > 0.0)) return -127;
    int ex;
    (void)frexp(amax, &ex);
    int e = (ex - 1) - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

int ora_mxfp8_quantize(const void* x, int dtype, const int32_t* off, int32_t B, int32_t H, int32_t d,
                       uint8_t* x8, uint8_t* scales, int32_t* soff) {
    if (!x || !off || !x8 || !scales || !soff || B < 0 || H < 1 || d < 32 || d % 32 != 0) return -1;
    if (dtype != ORA_F32 && dtype != ORA_BF16 && dtype != ORA_F64) return -1;
    if (off[0] != 0) return -1;
    soff[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        if (off[b + 1] < off[b]) return -1;
        soff[b + 1] = soff[b] + (off[b + 1] - off[b] + 31) / 32;
    }
    const int32_t nd = d / 32;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t r0 = off[b], L = off[b + 1] - off[b];
        for (int64_t jb = 0; jb * 32 < L; ++jb)
            for (int32_t h = 0; h < H; ++h)
                for (int32_t c = 0; c < nd; ++c) {
                    const int64_t rows = L - jb * 32 < 32 ? L - jb * 32 : 32;
                    double amax = 0.0;
                    for (int64_t r = 0; r < rows; ++r)
                        for (int32_t e = 0; e < 32; ++e) {
                            const double a = fabs(elem(x, dtype, ((r0 + jb * 32 + r) * H + h) * d + c * 32 + e));
                            if (a > amax) amax = a;
                        }
                    const int ex = mx_block_exponent(amax);
                    scales[((int64_t)(soff[b] + jb) * H + h) * nd + c] = (uint8_t)(ex + 127);
                    for (int64_t r = 0; r < rows; ++r)
                        for (int32_t e = 0; e < 32; ++e) {
                            const int64_t i = ((r0 + jb * 32 + r) * H + h) * d + c * 32 + e;
                            double v = ldexp(elem(x, dtype, i), -ex);
                            if (v > 448.0) v = 448.0;
                            if (v < -448.0) v = -448.0;
                            x8[i] = ora_e4m3_encode(v);
                        }
                }
    }
    return 0;
}

/* Dequantized tensor: x = e4m3(x8) * 2^(scale - 127) of its [32 x 32] block. */
static double* mx_dequantize(const uint8_t* x8, const uint8_t* scales, const int32_t* soff,
                             const int32_t* off, int32_t B, int32_t H, int32_t d) {
    const int64_t T = off[B], nd = d / 32;
    double* x = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T * H * d : 1));
    if (!x) return NULL;
    for (int32_t b = 0; b < B; ++b)
        for (int64_t r = off[b]; r < off[b + 1]; ++r)
            for (int32_t h = 0; h < H; ++h)
                for (int32_t c = 0; c < d; ++c) {
                    const int64_t jb = soff[b] + (r - off[b]) / 32;
                    const int sc = scales[(jb * H + h) * nd + c / 32];
                    const int64_t i = (r * H + h) * d + c;
                    x[i] = ldexp(ora_e4m3_decode(x8[i]), sc - 127);
                }
    return x;
}

/* ---- visibility ----------------------------------------------------------
 * Query i sees key j (both local to their sequence) iff j < Lk, and
 * causal => j <= i, and window W > 0 => (causal ? i - j < W : |i - j| < W),
 * and block size G > 0 => i and j lie in the same G-token block of the
 * sequence (floor(i / G) == floor(j / G)): "BlockAttention" section, each
 * query block attends only to its own key/value block. */
static int visible(int64_t i, int64_t j, int64_t Lk, int causal, int32_t window, int32_t block) {
    if (j < 0 || j >= Lk) return 0;
    if (causal && j > i) return 0;
    if (block > 0 && i / block != j / block) return 0;
    if (window > 0) {
        int64_t diff = i - j;
        if (!causal && diff < 0) diff = -diff;
        if (diff >= window) return 0;
    }
    return 1;
}

/* ---- work distribution over (b, h) pairs ------------------------------ */

typedef struct {
    const void *q, *k, *v, *dout;
    int dtype;
    const int32_t *q_off, *k_off;
    int32_t B, H, d;
    int act, causal;
    int32_t window;
    int32_t block;
    int pquant; /* softmax: P rounded to MXFP8 (E4M3 at the fixed scale 2^-8) in P V */
    double scale;
    const uint8_t* pair_mask;
    double *out, *lse, *dq, *dk, *dv;
    int64_t next; /* next work unit to claim */
    int64_t* rbase; /* forward: [B+1] first 64-row block of each sequence */
} job_t;

static int64_t claim(job_t* J) { return __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED); }

/* s_ij = scale * sum_c Q[qo+i,h,c] K[ko+j,h,c], summed in ascending c. */
static double score(const job_t* J, int64_t qrow, int64_t krow, int32_t h) {
    const int64_t H = J->H, d = J->d;
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c)
        acc += elem(J->q, J->dtype, (qrow * H + h) * d + c) *
               elem(J->k, J->dtype, (krow * H + h) * d + c);
    return J->scale * acc;
}

/* Forward of rows [i0, i1) of one (b, h) pair: the plain definition, row by row. */
static void fwd_rows(job_t* J, int32_t b, int32_t h, int64_t i0, int64_t i1) {
    const int64_t H = J->H, d = J->d;
    const int64_t qo = J->q_off[b], ko = J->k_off[b];
    const int64_t Lk = J->k_off[b + 1] - ko;
    double* s = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    for (int64_t i = i0; i < i1; ++i) {
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        double lse_i = NAN;
        if (J->act == ORA_SOFTMAX) {
            double m = -INFINITY;
            int64_t n = 0;
            for (int64_t j = 0; j < Lk; ++j) {
                if (!visible(i, j, Lk, J->causal, J->window, J->block)) continue;
                s[j] = score(J, qo + i, ko + j, (int32_t)h);
                if (s[j] > m) m = s[j];
                ++n;
            }
            if (n == 0) {
                lse_i = -INFINITY;
            } else {
                double l = 0.0;
                for (int64_t j = 0; j < Lk; ++j)
                    if (visible(i, j, Lk, J->causal, J->window, J->block)) l += exp(s[j] - m);
                for (int64_t j = 0; j < Lk; ++j) {
                    if (!visible(i, j, Lk, J->causal, J->window, J->block)) continue;
                    double p = exp(s[j] - m);
                    if (J->pquant) p = ldexp(ora_e4m3_decode(ora_e4m3_encode(ldexp(p, 8))), -8);
                    for (int64_t c = 0; c < d; ++c)
                        o[c] += p * elem(J->v, J->dtype, ((ko + j) * H + h) * d + c);
                }
                for (int64_t c = 0; c < d; ++c) o[c] /= l;
                lse_i = m + log(l);
            }
        } else {
            for (int64_t j = 0; j < Lk; ++j) {
                if (!visible(i, j, Lk, J->causal, J->window, J->block)) continue;
                double a = act_apply(J->act, score(J, qo + i, ko + j, (int32_t)h));
                for (int64_t c = 0; c < d; ++c)
                    o[c] += a * elem(J->v, J->dtype, ((ko + j) * H + h) * d + c);
            }
            if (Lk > 0)
                for (int64_t c = 0; c < d; ++c) o[c] /= (double)Lk;
        }
        for (int64_t c = 0; c < d; ++c) J->out[((qo + i) * H + h) * d + c] = o[c];
        if (J->lse) J->lse[(qo + i) * H + h] = lse_i;
    }
    free(s);
    free(o);
}

static void fwd_pair(job_t* J, int32_t b, int32_t h) {
    fwd_rows(J, b, h, 0, (int64_t)J->q_off[b + 1] - J->q_off[b]);
}

/* Backward of one (b, h) pair. Softmax: P_ij = exp(s_ij - lse_i),
 * D_i = sum_c dO_ic O_ic, dV_j = sum_i P_ij dO_i, dP_ij = dO_i . V_j,
 * dS_ij = P_ij (dP_ij - D_i), dQ_i = scale sum_j dS_ij K_j,
 * dK_j = scale sum_i dS_ij Q_i. Pointwise: the weight is act(s_ij)/Lk, and
 * dS_ij = act'(s_ij) dP_ij / Lk. O and lse are the oracle's own. */
static void bwd_pair(job_t* J, int32_t b, int32_t h) {
    const int64_t H = J->H, d = J->d;
    const int64_t qo = J->q_off[b], ko = J->k_off[b];
    const int64_t Lq = J->q_off[b + 1] - qo, Lk = J->k_off[b + 1] - ko;
    fwd_pair(J, b, h); /* writes out and lse rows of this pair */
    double* lse_local = (double*)malloc(sizeof(double) * (size_t)(Lq > 0 ? Lq : 1));
    /* The softmax backward needs lse; when the caller passed no lse buffer
     * recompute it row by row here. */
    for (int64_t i = 0; i < Lq; ++i) {
        if (J->act != ORA_SOFTMAX) { lse_local[i] = NAN; continue; }
        if (J->lse) { lse_local[i] = J->lse[(qo + i) * H + h]; continue; }
        double m = -INFINITY;
        for (int64_t j = 0; j < Lk; ++j)
            if (visible(i, j, Lk, J->causal, J->window, J->block)) {
                double sj = score(J, qo + i, ko + j, (int32_t)h);
                if (sj > m) m = sj;
            }
        double l = 0.0;
        for (int64_t j = 0; j < Lk; ++j)
            if (visible(i, j, Lk, J->causal, J->window, J->block))
                l += exp(score(J, qo + i, ko + j, (int32_t)h) - m);
        lse_local[i] = (m == -INFINITY) ? -INFINITY : m + log(l);
    }
    for (int64_t i = 0; i < Lq; ++i)
        for (int64_t c = 0; c < d; ++c) J->dq[((qo + i) * H + h) * d + c] = 0.0;
    for (int64_t j = 0; j < Lk; ++j)
        for (int64_t c = 0; c < d; ++c) {
            J->dk[((ko + j) * H + h) * d + c] = 0.0;
            J->dv[((ko + j) * H + h) * d + c] = 0.0;
        }
    for (int64_t i = 0; i < Lq; ++i) {
        const int64_t qi = ((qo + i) * H + h) * d;
        double Di = 0.0;
        if (J->act == ORA_SOFTMAX)
            for (int64_t c = 0; c < d; ++c) Di += elem(J->dout, J->dtype, qi + c) * J->out[qi + c];
        for (int64_t j = 0; j < Lk; ++j) {
            if (!visible(i, j, Lk, J->causal, J->window, J->block)) continue;
            const int64_t kj = ((ko + j) * H + h) * d;
            double sij = score(J, qo + i, ko + j, (int32_t)h);
            double p, dsfac;
            double dp = 0.0;
            for (int64_t c = 0; c < d; ++c)
                dp += elem(J->dout, J->dtype, qi + c) * elem(J->v, J->dtype, kj + c);
            if (J->act == ORA_SOFTMAX) {
                p = exp(sij - lse_local[i]);
                dsfac = p * (dp - Di);
            } else {
                p = act_apply(J->act, sij) / (double)Lk;
                dsfac = act_deriv(J->act, sij) * dp / (double)Lk;
            }
            for (int64_t c = 0; c < d; ++c) {
                J->dv[kj + c] += p * elem(J->dout, J->dtype, qi + c);
                J->dq[qi + c] += J->scale * dsfac * elem(J->k, J->dtype, kj + c);
                J->dk[kj + c] += J->scale * dsfac * elem(J->q, J->dtype, qi + c);
            }
        }
    }
    free(lse_local);
}

/* Forward work units are (head, 64-row block of the batch); rbase[b] is the first
 * row block of sequence b. Backward units are whole (b, h) pairs, since dK and dV
 * of a key gather over every row of its sequence. */
#define ORA_ROWS 64

static int32_t seq_of_block(const int64_t* rbase, int32_t B, int64_t rb) {
    int32_t lo = 0, hi = B; /* rbase[lo] <= rb < rbase[hi] */
    while (hi - lo > 1) {
        int32_t mid = (lo + hi) / 2;
        if (rbase[mid] <= rb) lo = mid;
        else hi = mid;
    }
    return lo;
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    if (J->dq) {
        const int64_t npairs = (int64_t)J->B * J->H;
        for (;;) {
            int64_t p = claim(J);
            if (p >= npairs) break;
            if (J->pair_mask && !J->pair_mask[p]) continue;
            bwd_pair(J, (int32_t)(p / J->H), (int32_t)(p % J->H));
        }
        return NULL;
    }
    const int64_t nrb = J->rbase[J->B];
    const int64_t nunits = nrb * J->H;
    for (;;) {
        int64_t u = claim(J);
        if (u >= nunits) break;
        const int32_t h = (int32_t)(u / nrb);
        const int64_t rb = u % nrb;
        const int32_t b = seq_of_block(J->rbase, J->B, rb);
        if (J->pair_mask && !J->pair_mask[(int64_t)b * J->H + h]) continue;
        const int64_t Lq = (int64_t)J->q_off[b + 1] - J->q_off[b];
        const int64_t i0 = (rb - J->rbase[b]) * ORA_ROWS;
        const int64_t i1 = i0 + ORA_ROWS < Lq ? i0 + ORA_ROWS : Lq;
        fwd_rows(J, b, h, i0, i1);
    }
    return NULL;
}

int ora_num_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int run(job_t* J, int nthreads) {
    if (nthreads <= 0) nthreads = ora_num_threads();
    if (nthreads < 1) nthreads = 1;
    int64_t* rbase = NULL;
    if (!J->dq) {
        rbase = (int64_t*)malloc(sizeof(int64_t) * ((size_t)J->B + 1));
        rbase[0] = 0;
        for (int32_t b = 0; b < J->B; ++b) {
            int64_t Lq = (int64_t)J->q_off[b + 1] - J->q_off[b];
            rbase[b + 1] = rbase[b] + (Lq + ORA_ROWS - 1) / ORA_ROWS;
        }
        J->rbase = rbase;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int t = 0; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, worker, J) == 0) ++started;
    if (started == 0) worker(J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    free(th);
    free(rbase);
    return 0;
}

static int check_common(const int32_t* q_off, const int32_t* k_off, int32_t B, int32_t H,
                        int32_t d, int act, int32_t window) {
    if (!q_off || !k_off || B < 0 || H < 1 || d < 1 || window < 0) return -1;
    if (act != ORA_SOFTMAX && act != ORA_SILU && act != ORA_GELU_TANH && act != ORA_GELU_TAYLOR) return -1;
    if (q_off[0] != 0 || k_off[0] != 0) return -1;
    for (int32_t b = 0; b < B; ++b)
        if (q_off[b + 1] < q_off[b] || k_off[b + 1] < k_off[b]) return -1;
    return 0;
}

int ora_fwd_block(const void* q, const void* k, const void* v, int dtype,
                  const int32_t* q_off, const int32_t* k_off,
                  int32_t B, int32_t H, int32_t d,
                  int act, int causal, int32_t window, int32_t block, double scale,
                  const uint8_t* pair_mask, double* out, double* lse, int nthreads) {
    if (check_common(q_off, k_off, B, H, d, act, window) || !out || block < 0) return -1;
    if (dtype != ORA_F32 && dtype != ORA_BF16 && dtype != ORA_F64) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype;
    J.q_off = q_off; J.k_off = k_off; J.B = B; J.H = H; J.d = d;
    J.act = act; J.causal = causal != 0; J.window = window; J.block = block; J.scale = scale;
    J.pair_mask = pair_mask; J.out = out; J.lse = lse;
    return run(&J, nthreads);
}

int ora_fwd(const void* q, const void* k, const void* v, int dtype,
            const int32_t* q_off, const int32_t* k_off,
            int32_t B, int32_t H, int32_t d,
            int act, int causal, int32_t window, double scale,
            const uint8_t* pair_mask, double* out, double* lse, int nthreads) {
    return ora_fwd_block(q, k, v, dtype, q_off, k_off, B, H, d, act, causal, window, 0, scale,
                         pair_mask, out, lse, nthreads);
}

int ora_fwd_mxfp8(const uint8_t* q8, const uint8_t* qs, const int32_t* q_soff,
                  const uint8_t* k8, const uint8_t* ks, const int32_t* k_soff,
                  const uint8_t* v8, const uint8_t* vs,
                  const int32_t* q_off, const int32_t* k_off, int32_t B, int32_t H, int32_t d,
                  int causal, int32_t window, double scale, int pquant,
                  const uint8_t* pair_mask, double* out, double* lse, int nthreads) {
    if (check_common(q_off, k_off, B, H, d, ORA_SOFTMAX, window) || !out || d % 32 != 0) return -1;
    if (!q8 || !qs || !q_soff || !k8 || !ks || !k_soff || !v8 || !vs) return -1;
    double* q = mx_dequantize(q8, qs, q_soff, q_off, B, H, d);
    double* k = mx_dequantize(k8, ks, k_soff, k_off, B, H, d);
    double* v = mx_dequantize(v8, vs, k_soff, k_off, B, H, d);
    int rc = -1;
    if (q && k && v) {
        job_t J;
        memset(&J, 0, sizeof J);
        J.q = q; J.k = k; J.v = v; J.dtype = ORA_F64;
        J.q_off = q_off; J.k_off = k_off; J.B = B; J.H = H; J.d = d;
        J.act = ORA_SOFTMAX; J.causal = causal != 0; J.window = window; J.scale = scale;
        J.pquant = pquant != 0;
        J.pair_mask = pair_mask; J.out = out; J.lse = lse;
        rc = run(&J, nthreads);
    }
    free(q);
    free(k);
    free(v);
    return rc;
}

int ora_bwd_block(const void* q, const void* k, const void* v, const void* dout, int dtype,
                  const int32_t* q_off, const int32_t* k_off,
                  int32_t B, int32_t H, int32_t d,
                  int act, int causal, int32_t window, int32_t block, double scale,
                  const uint8_t* pair_mask, double* out, double* lse,
                  double* dq, double* dk, double* dv, int nthreads) {
    if (check_common(q_off, k_off, B, H, d, act, window) || block < 0) return -1;
    if (!out || !dq || !dk || !dv || !dout) return -1;
    if (dtype != ORA_F32 && dtype != ORA_BF16 && dtype != ORA_F64) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dout = dout; J.dtype = dtype;
    J.q_off = q_off; J.k_off = k_off; J.B = B; J.H = H; J.d = d;
    J.act = act; J.causal = causal != 0; J.window = window; J.block = block; J.scale = scale;
    J.pair_mask = pair_mask; J.out = out; J.lse = lse;
    J.dq = dq; J.dk = dk; J.dv = dv;
    return run(&J, nthreads);
}

int ora_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
            const int32_t* q_off, const int32_t* k_off,
            int32_t B, int32_t H, int32_t d,
            int act, int causal, int32_t window, double scale,
            const uint8_t* pair_mask, double* out, double* lse,
            double* dq, double* dk, double* dv, int nthreads) {
    return ora_bwd_block(q, k, v, dout, dtype, q_off, k_off, B, H, d, act, causal, window, 0, scale,
                         pair_mask, out, lse, dq, dk, dv, nthreads);
}

/* ---- reference work list ---------------------------------------------- */

typedef struct { int32_t b, t, cost, key; } item_t;

static int item_cmp(const void* pa, const void* pb) {
    const item_t* a = (const item_t*)pa;
    const item_t* c = (const item_t*)pb;
    if (a->key != c->key) return a->key > c->key ? -1 : 1; /* descending */
    if (a->b != c->b) return a->b < c->b ? -1 : 1;
    if (a->t != c->t) return a->t < c->t ? -1 : 1;
    return 0;
}

int64_t ora_tile_list_block(const int32_t* row_off, const int32_t* col_off, int32_t B,
                            int32_t BM, int32_t BN, int causal, int32_t window, int32_t block,
                            int transposed, int32_t cap,
                            int32_t* items, int32_t* costs, int64_t max_items) {
    if (!row_off || !col_off || B < 0 || BM < 1 || BN < 1 || window < 0 || block < 0 || cap < 1) return -1;
    int64_t n = 0;
    for (int32_t b = 0; b < B; ++b) {
        int64_t L = row_off[b + 1] - row_off[b];
        if (L < 0) return -1;
        n += (L + BM - 1) / BM;
    }
    if (n > max_items) return -1;
    item_t* it = (item_t*)malloc(sizeof(item_t) * (size_t)(n > 0 ? n : 1));
    int64_t m = 0;
    for (int32_t b = 0; b < B; ++b) {
        int64_t Lr = row_off[b + 1] - row_off[b], Lc = col_off[b + 1] - col_off[b];
        for (int64_t t = 0; t * BM < Lr; ++t) {
            int64_t r0 = t * BM, r1 = r0 + BM < Lr ? r0 + BM : Lr; /* rows [r0, r1) */
            /* Visible columns of any row in [r0, r1): brute force over the
             * definition, so this reference does not rely on a closed form. */
            int64_t lo = -1, hi = -1;
            for (int64_t c = 0; c < Lc; ++c) {
                int any = 0;
                for (int64_t r = r0; r < r1 && !any; ++r) {
                    /* not transposed: rows are queries i, columns keys j;
                     * transposed: rows are keys j, columns queries i. */
                    any = transposed ? visible(c, r, Lr, causal, window, block)
                                     : visible(r, c, Lc, causal, window, block);
                }
                if (any) {
                    if (lo < 0) lo = c;
                    hi = c + 1;
                }
            }
            int32_t cost = 0;
            if (lo >= 0) cost = (int32_t)((hi + BN - 1) / BN - lo / BN);
            it[m].b = b;
            it[m].t = (int32_t)t;
            it[m].cost = cost;
            it[m].key = cost < cap ? cost : cap;
            ++m;
        }
    }
    qsort(it, (size_t)m, sizeof(item_t), item_cmp);
    for (int64_t i = 0; i < m; ++i) {
        items[2 * i] = it[i].b;
        items[2 * i + 1] = it[i].t;
        costs[i] = it[i].cost;
    }
    free(it);
    return m;
}

int64_t ora_tile_list(const int32_t* row_off, const int32_t* col_off, int32_t B,
                      int32_t BM, int32_t BN, int causal, int32_t window,
                      int transposed, int32_t cap,
                      int32_t* items, int32_t* costs, int64_t max_items) {
    return ora_tile_list_block(row_off, col_off, B, BM, BN, causal, window, 0, transposed, cap,
                               items, costs, max_items);
}
