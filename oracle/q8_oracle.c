/*
 * q8_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for exact chunked causal attention over a
 * Q8_0-quantised KV cache.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no source, header, table or helper with the HIP
 * library under chunked_flashattention_q8_amd/; the product path never calls it.
 *
 * Sources (the web pages this method is described on):
 *   [OOC]  "Out-of-Core Flash Streaming & Speculative Decode (1M Context)", m4-prefill-engine.
 *          Sec. 3 "Chunked FlashAttention: Exact Mathematical Derivation" gives the recurrence;
 *          Sec. 1 "The Context Memory Wall" gives the Q8_0 row size (2 blocks x 34 bytes per
 *          64-dim head row); Sec. 4 "Mode A vs. Mode B" gives the triangular causal mask.
 *   [ARCH] "Core Architecture & The 4-Brick Pipeline", m4-prefill-engine.
 *          Sec. 5 "Brick 4" defines block_q8_0: 32 int8 values plus one FP16 scale, 34 bytes,
 *          8-bit symmetric quantisation.
 *
 * Readings taken where the pages are silent (each is listed in the design doc):
 *   - the scale is d = amax/127 in IEEE single precision, stored as binary16 (round to nearest
 *     even); values are quantised against the STORED scale: q = round(x / d16), ties away from
 *     zero, clamped to [-127, 127]; an all-zero block stores d16 = 0 and q = 0;
 *   - block bytes are the scale (little-endian binary16) followed by the 32 int8 values; a 64-dim
 *     row is block 0 (dims 0..31) then block 1 (dims 32..63);
 *   - a query at absolute position p sees keys at positions <= p (diagonal included);
 *   - the state starts as m = -inf, l = 0, O = 0, and a chunk in which a row sees no key leaves
 *     that row's state untouched;
 *   - all attention arithmetic is IEEE binary64, one rounding per operation, no contraction.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------
 * binary16 codec.  Written from the IEEE 754 definition of the format: 1 sign bit, 5 exponent
 * bits (bias 15), 10 fraction bits; exponent field 0 holds zero and the subnormals (value
 * F * 2^-24), field 31 holds infinities and NaNs.
 * ---------------------------------------------------------------------------------------- */

double orc_f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25);
    return sign ? -mag : mag;
}

/* Round a float to the nearest binary16 value, ties to even.  The binary16 values in the binade
 * [2^e, 2^(e+1)) are the multiples of 2^(e-10); below 2^-14 the grid is that of the
 * subnormals, 2^-24.  a / quantum is exact (division by a power of two of a value with 24
 * significant bits), so nearbyint() (round half to even in the default rounding mode) picks the
 * correctly rounded grid point. */
uint16_t orc_f32_to_f16(float xf)
{
    double x = (double)xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7e00;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7c00;
    int e;
    frexp(a, &e); /* a = frac * 2^e, frac in [0.5, 1)  =>  binade exponent is e - 1 */
    e -= 1;
    if (e < -14)
        e = -14;
    double quantum = ldexp(1.0, e - 10);
    double n = nearbyint(a / quantum);
    double v = n * quantum;
    if (v > 65504.0)
        return sign | 0x7c00; /* beyond the largest finite binary16 after rounding */
    if (v < ldexp(1.0, -14))  /* subnormal (or zero) */
        return sign | (uint16_t)(v / ldexp(1.0, -24));
    int ev;
    frexp(v, &ev); /* rounding may have carried v into the next binade */
    ev -= 1;
    uint16_t frac = (uint16_t)(v / ldexp(1.0, ev - 10) - 1024.0);
    return sign | (uint16_t)((ev + 15) << 10) | frac;
}

void orc_f32_to_f16_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f64_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f64(h[i]);
}

/* ------------------------------------------------------------------------------------------
 * Q8_0 block codec ([ARCH] Sec. 5, block_q8_0; [OOC] Sec. 1 row size).
 * ---------------------------------------------------------------------------------------- */

#define QK 32          /* values per block */
#define BLOCK_BYTES 34 /* 2-byte binary16 scale + 32 int8 */

/* Returns 0 on success, 1 if the block's scale is not a finite binary16 value. */
static int pack_block(const float *x, uint8_t *out)
{
    float amax = 0.0f;
    for (int t = 0; t < QK; ++t) {
        float a = fabsf(x[t]);
        if (a > amax)
            amax = a;
    }
    float d = amax / 127.0f; /* IEEE single-precision division */
    uint16_t d16 = orc_f32_to_f16(d);
    float dh = (float)orc_f16_to_f64(d16); /* exact: every binary16 value is a float */
    out[0] = (uint8_t)(d16 & 0xff);
    out[1] = (uint8_t)(d16 >> 8);
    for (int t = 0; t < QK; ++t) {
        int q = 0;
        if (dh != 0.0f) {
            float r = x[t] / dh;  /* IEEE single-precision division */
            float rq = roundf(r); /* nearest integer, halves away from zero */
            if (rq > 127.0f)
                rq = 127.0f;
            if (rq < -127.0f)
                rq = -127.0f;
            q = (int)rq;
        }
        out[2 + t] = (uint8_t)(int8_t)q;
    }
    return isfinite(dh) ? 0 : 1;
}

typedef struct {
    const float *x;
    uint8_t *dst;
    int64_t b0, b1;
    int64_t bad;
} pack_job;

static void *pack_worker(void *arg)
{
    pack_job *j = (pack_job *)arg;
    int64_t bad = 0;
    for (int64_t b = j->b0; b < j->b1; ++b)
        bad += pack_block(j->x + b * QK, j->dst + b * BLOCK_BYTES);
    j->bad = bad;
    return NULL;
}

/* Packs n_blocks consecutive blocks of 32 floats into n_blocks * 34 bytes.  Returns the number
 * of blocks whose scale overflowed binary16 (their bytes are still written). */
int64_t orc_q8_0_pack(const float *x, uint8_t *dst, int64_t n_blocks, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (n_blocks < (int64_t)nthreads * 64)
        nthreads = 1;
    pthread_t th[256];
    pack_job jobs[256];
    int64_t per = (n_blocks + nthreads - 1) / nthreads;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i].x = x;
        jobs[i].dst = dst;
        jobs[i].b0 = (int64_t)i * per < n_blocks ? (int64_t)i * per : n_blocks;
        jobs[i].b1 = (int64_t)(i + 1) * per < n_blocks ? (int64_t)(i + 1) * per : n_blocks;
        jobs[i].bad = 0;
        if (nthreads > 1)
            pthread_create(&th[i], NULL, pack_worker, &jobs[i]);
        else
            pack_worker(&jobs[i]);
    }
    int64_t bad = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (nthreads > 1)
            pthread_join(th[i], NULL);
        bad += jobs[i].bad;
    }
    return bad;
}

/* Value t of a block is q_t * d16, exact in binary64. */
void orc_q8_0_dequant(const uint8_t *src, double *y, int64_t n_blocks)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t *blk = src + b * BLOCK_BYTES;
        double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int t = 0; t < QK; ++t)
            y[b * QK + t] = (double)(int8_t)blk[2 + t] * d;
    }
}

/* ------------------------------------------------------------------------------------------
 * Attention.  Problem layout (head-major):
 *   Q      binary16 bits [B][H][M][D]; query row i of every sequence sits at absolute position
 *          q_pos0 + i;
 *   K, V   key j of head (b, h) at absolute position j, either Q8_0 rows of D/32 blocks
 *          ([B][H][N][D/32*34] bytes) or binary16 bits ([B][H][N][D]).
 * ---------------------------------------------------------------------------------------- */

enum { ORC_KV_Q8_0 = 0, ORC_KV_F16 = 1 };

typedef struct {
    const uint16_t *q;
    const uint8_t *k;
    const uint8_t *v;
    int32_t kv_fmt;
    int32_t B, H, M, N, D;
    int64_t q_pos0;
    int32_t causal;
} orc_problem;

/* Dequantises keys [j0, j0 + n) of head (b, h) of K (which = 0) or V (which = 1) to [n][D]. */
static void load_kv_rows(const orc_problem *p, int b, int h, int which, int64_t j0, int64_t n,
                         double *out)
{
    const uint8_t *base = which ? p->v : p->k;
    int64_t head = (int64_t)b * p->H + h;
    if (p->kv_fmt == ORC_KV_Q8_0) {
        int64_t row_bytes = (int64_t)(p->D / QK) * BLOCK_BYTES;
        const uint8_t *src = base + (head * p->N + j0) * row_bytes;
        orc_q8_0_dequant(src, out, n * (p->D / QK));
    } else {
        const uint16_t *src = (const uint16_t *)base + (head * p->N + j0) * p->D;
        for (int64_t i = 0; i < n * p->D; ++i)
            out[i] = orc_f16_to_f64(src[i]);
    }
}

static void load_q_row(const orc_problem *p, int64_t row, double *qv)
{
    const uint16_t *src = p->q + row * p->D;
    for (int t = 0; t < p->D; ++t)
        qv[t] = orc_f16_to_f64(src[t]);
}

/* Number of keys among [j0, j0 + n) that a query at absolute position pos may see: with the
 * triangular causal mask those at positions <= pos, otherwise all of them. */
static int64_t visible_count(const orc_problem *p, int64_t pos, int64_t j0, int64_t n)
{
    if (!p->causal)
        return n;
    int64_t last = pos - j0; /* last visible index relative to j0 */
    if (last < 0)
        return 0;
    return last + 1 < n ? last + 1 : n;
}

static double score(const double *qv, const double *krow, int D)
{
    double s = 0.0;
    for (int t = 0; t < D; ++t)
        s += qv[t] * krow[t];
    return s / sqrt((double)D);
}

/* Single pass: softmax(q K^T / sqrt(D)) V over the visible keys, plus the log-sum-exp of the
 * scaled logits.  A row that sees no key gets O = 0 and LSE = -inf. */
static void attn_row_single(const orc_problem *p, const double *Kd, const double *Vd,
                            const double *qv, int64_t pos, double *o, double *lse, double *w)
{
    int D = p->D;
    int64_t nv = visible_count(p, pos, 0, p->N);
    for (int t = 0; t < D; ++t)
        o[t] = 0.0;
    if (nv == 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nv; ++j) {
        w[j] = score(qv, Kd + j * D, D);
        if (w[j] > m)
            m = w[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nv; ++j) {
        w[j] = exp(w[j] - m);
        l += w[j];
    }
    for (int64_t j = 0; j < nv; ++j)
        for (int t = 0; t < D; ++t)
            o[t] += w[j] * Vd[j * D + t];
    for (int t = 0; t < D; ++t)
        o[t] /= l;
    *lse = m + log(l);
}

/* One chunk of the [OOC] Sec. 3 recurrence for one query row.  Chunk keys are [j0, j0 + n).
 * State (m, l, O) is updated in place; a row with no visible key in the chunk is untouched. */
static void attn_row_chunk(const orc_problem *p, const double *Kc, const double *Vc,
                           const double *qv, int64_t pos, int64_t j0, int64_t n, double *m,
                           double *l, double *O, double *S)
{
    int D = p->D;
    int64_t nv = visible_count(p, pos, j0, n);
    if (nv == 0)
        return;
    /* step 1: local tile scores S_ij = Q_i . K_cj / sqrt(D) */
    for (int64_t j = 0; j < nv; ++j)
        S[j] = score(qv, Kc + j * D, D);
    /* step 2: local maximum */
    double mt = -INFINITY;
    for (int64_t j = 0; j < nv; ++j)
        if (S[j] > mt)
            mt = S[j];
    /* step 3: updated running maximum */
    double mn = *m > mt ? *m : mt;
    /* step 4: rescale factor alpha = e^(m_old - m_new); beta_j = e^(S_ij - m_new), stored
     * over S */
    double alpha = exp(*m - mn); /* e^(-inf) = 0 for a row that had seen nothing */
    for (int64_t j = 0; j < nv; ++j)
        S[j] = exp(S[j] - mn);
    /* step 5: normaliser */
    double sb = 0.0;
    for (int64_t j = 0; j < nv; ++j)
        sb += S[j];
    *l = *l * alpha + sb;
    /* step 6: unnormalised output */
    for (int t = 0; t < D; ++t) {
        double acc = 0.0;
        for (int64_t j = 0; j < nv; ++j)
            acc += S[j] * Vc[j * D + t];
        O[t] = O[t] * alpha + acc;
    }
    *m = mn;
}

/* ---- threading over the rows of one head ---- */

typedef struct {
    const orc_problem *p;
    const double *Kd, *Vd;
    const int64_t *rows; /* flat row ids (b*H + h)*M + i, all of one head */
    const int64_t *slot; /* output slot of each row */
    int64_t n;
    int mode; /* 0 = single pass, 1 = chunk list */
    /* single pass outputs */
    double *O, *lse;
    /* chunk mode */
    const int64_t *c_start;
    const int64_t *c_len;
    int n_chunks;
    int64_t kv_lo; /* first key position held in Kd/Vd */
    double *sm, *sl;
    int tid, nthreads;
} row_job;

static void *row_worker(void *arg)
{
    row_job *j = (row_job *)arg;
    const orc_problem *p = j->p;
    int D = p->D;
    double *qv = (double *)malloc(sizeof(double) * D);
    double *w = (double *)malloc(sizeof(double) * (p->N > 0 ? p->N : 1));
    for (int64_t r = j->tid; r < j->n; r += j->nthreads) {
        int64_t row = j->rows[r];
        int64_t i = row % p->M;
        int64_t pos = p->q_pos0 + i;
        int64_t s = j->slot[r];
        load_q_row(p, row, qv);
        if (j->mode == 0) {
            attn_row_single(p, j->Kd, j->Vd, qv, pos, j->O + s * D, j->lse + s, w);
        } else {
            for (int c = 0; c < j->n_chunks; ++c) {
                int64_t off = j->c_start[c] - j->kv_lo;
                attn_row_chunk(p, j->Kd + off * D, j->Vd + off * D, qv, pos, j->c_start[c],
                               j->c_len[c], j->sm + s, j->sl + s, j->O + s * D, w);
            }
        }
    }
    free(qv);
    free(w);
    return NULL;
}

/* Groups rows by head (rows must be sorted by head), dequantises each head's keys
 * [kv_lo, kv_hi) once, and runs the rows of that head on nthreads threads. */
static int run_rows(const orc_problem *p, const int64_t *rows, int64_t n_rows, int mode,
                    double *O, double *lse, const int64_t *c_start, const int64_t *c_len,
                    int n_chunks, double *sm, double *sl, int nthreads)
{
    int D = p->D;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    int64_t kv_lo = 0, kv_hi = p->N;
    if (mode == 1 && n_chunks > 0) {
        kv_lo = c_start[0];
        kv_hi = c_start[0] + c_len[0];
        for (int c = 1; c < n_chunks; ++c) {
            if (c_start[c] < kv_lo)
                kv_lo = c_start[c];
            if (c_start[c] + c_len[c] > kv_hi)
                kv_hi = c_start[c] + c_len[c];
        }
    }
    int64_t nk = kv_hi - kv_lo;
    double *Kd = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
    double *Vd = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * D);
    int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_rows > 0 ? n_rows : 1));
    if (!Kd || !Vd || !slot) {
        free(Kd);
        free(Vd);
        free(slot);
        return 1;
    }
    for (int64_t r = 0; r < n_rows; ++r)
        slot[r] = r;
    int64_t r0 = 0;
    while (r0 < n_rows) {
        int64_t head = rows[r0] / p->M;
        int64_t r1 = r0;
        while (r1 < n_rows && rows[r1] / p->M == head)
            ++r1;
        int b = (int)(head / p->H), h = (int)(head % p->H);
        if (nk > 0) {
            load_kv_rows(p, b, h, 0, kv_lo, nk, Kd);
            load_kv_rows(p, b, h, 1, kv_lo, nk, Vd);
        }
        int nt = (int64_t)nthreads < r1 - r0 ? nthreads : (int)(r1 - r0);
        pthread_t th[256];
        row_job jobs[256];
        for (int t = 0; t < nt; ++t) {
            row_job *j = &jobs[t];
            j->p = p;
            j->Kd = Kd;
            j->Vd = Vd;
            j->rows = rows + r0;
            j->slot = slot + r0;
            j->n = r1 - r0;
            j->mode = mode;
            j->O = O;
            j->lse = lse;
            j->c_start = c_start;
            j->c_len = c_len;
            j->n_chunks = n_chunks;
            j->kv_lo = kv_lo;
            j->sm = sm;
            j->sl = sl;
            j->tid = t;
            j->nthreads = nt;
            if (nt > 1)
                pthread_create(&th[t], NULL, row_worker, j);
            else
                row_worker(j);
        }
        if (nt > 1)
            for (int t = 0; t < nt; ++t)
                pthread_join(th[t], NULL);
        r0 = r1;
    }
    free(Kd);
    free(Vd);
    free(slot);
    return 0;
}

/* Single-pass attention for the listed rows (flat ids (b*H + h)*M + i, sorted by head).
 * O: [n_rows][D] binary64, lse: [n_rows].  Returns 0 on success. */
int orc_attention_rows(const orc_problem *p, const int64_t *rows, int64_t n_rows, double *O,
                       double *lse, int nthreads)
{
    return run_rows(p, rows, n_rows, 0, O, lse, NULL, NULL, 0, NULL, NULL, nthreads);
}

/* Applies the chunks [c_start[c], c_start[c] + c_len[c]) in the given order to the state of the
 * listed rows, following the recurrence of [OOC] Sec. 3.  m, l: [n_rows]; O: [n_rows][D] (the
 * unnormalised running output), all updated in place.  Returns 0 on success. */
int orc_attention_chunks(const orc_problem *p, const int64_t *rows, int64_t n_rows,
                         const int64_t *c_start, const int64_t *c_len, int n_chunks, double *m,
                         double *l, double *O, int nthreads)
{
    return run_rows(p, rows, n_rows, 1, O, NULL, c_start, c_len, n_chunks, m, l, nthreads);
}

/* Merge two partial states of the same rows, over disjoint key sets, into the first: the state
 * a single pass over both key sets would have reached.  A partial state (m, l, O) summarises its
 * keys exactly as a chunk's (local maximum, sum of e^(S - max), sum of e^(S - max) V) do, so this
 * is steps 3-6 of the [OOC] Sec. 3 recurrence with the second state in the chunk's place:
 * m' = max(m_a, m_b), l' = l_a e^(m_a - m') + l_b e^(m_b - m'), O' likewise.  An empty state
 * (m = -inf) contributes nothing; two empty states stay empty. */
void orc_merge_states(double *m_a, double *l_a, double *O_a, const double *m_b,
                      const double *l_b, const double *O_b, int64_t n_rows, int D)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        if (m_b[r] == -INFINITY)
            continue;
        if (m_a[r] == -INFINITY) {
            m_a[r] = m_b[r];
            l_a[r] = l_b[r];
            for (int t = 0; t < D; ++t)
                O_a[r * D + t] = O_b[r * D + t];
            continue;
        }
        double mn = m_a[r] > m_b[r] ? m_a[r] : m_b[r];
        double fa = exp(m_a[r] - mn), fb = exp(m_b[r] - mn);
        l_a[r] = l_a[r] * fa + l_b[r] * fb;
        for (int t = 0; t < D; ++t)
            O_a[r * D + t] = O_a[r * D + t] * fa + O_b[r * D + t] * fb;
        m_a[r] = mn;
    }
}

/* After the last chunk the output is O / l ([OOC] Sec. 3) and the log-sum-exp is m + ln l.
 * A row that never saw a key (l = 0) yields O = 0 and LSE = -inf. */
void orc_finalize(const double *m, const double *l, const double *O, int64_t n_rows, int D,
                  double *out, double *lse)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        if (l[r] == 0.0) {
            for (int t = 0; t < D; ++t)
                out[r * D + t] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        for (int t = 0; t < D; ++t)
            out[r * D + t] = O[r * D + t] / l[r];
        lse[r] = m[r] + log(l[r]);
    }
}
