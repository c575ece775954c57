/*
 * pa_oracle.c -- plain CPU float64 reference for paged KV append and paged attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file; only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code with the HIP library: the pool layout, the dtype decoders, the fp8
 * encoder and the attention arithmetic are all written out here from their definitions.
 *
 * What it computes (sources are the four scraped pages on paged KV caches):
 *   - attention is softmax(Q K^T / sqrt(d)) V                (page 1, section 2 "what the
 *     KV cache stores", the Attention(Q,K,V) formula);
 *   - each sequence's KV lives in fixed-size physical blocks reached through a per-sequence
 *     block table that maps logical block i to a physical block  (page 1, section 4
 *     "PagedAttention", the logical->physical mapping figure; page 3, section 2.1, which
 *     gives 16 tokens as the default block size and says the kernel reads KV block by
 *     block through the table instead of assuming contiguity);
 *   - several query heads share one KV head (GQA)            (page 1, section 10);
 *   - the KV cache may be stored as 8-bit floats, e4m3 preferred over e5m2 (which can drift
 *     numerically on long sequences), with
 *     per-tensor or per-head scales                          (page 1, section 15; page 2,
 *     "quantisation"; page 3, section 2.4);
 *   - or as 8-bit integers: a tuning step brings the KV cache from 16-bit floats down to INT8
 *     (page 4, section 4.5, step 4; page 2, "quantisation", which names KV-cache quantisation
 *     beside weight and activation quantisation).  The pages give no encoding; the reading
 *     taken here is the plain symmetric one: one fp32 scale per (layer, kv head), the stored
 *     code is the nearest integer (ties to even) to fl32(x / scale), saturated to [-127, 127]
 *     (NaN stores 0), and the cached value is code * scale.
 * Each decode step produces the new token's K/V and stores it in the cache, and the new
 * query attends over all stored positions including that one (page 1, section 1, the
 * prefill/decode diagram).
 *
 * The attention is evaluated token by token, walking the block table: for each query row
 * the scores z_t = scale * <q, K_t> are formed for every visible position t, then the plain
 * two-pass softmax  w_t = exp(z_t - max z),  out = sum_t w_t V_t / sum_t w_t  is applied.
 * There is no online-softmax trick, no blocking and no reordering.
 *
 * Pool layout (a format both sides must agree on; the pages give none).  Let e be the
 * element size in bytes (4 fp32, 2 bf16, 1 fp8), W = 64 / e, T = min(16 / e, B) and B the
 * block size.  The K pool and the V pool are each [num_blocks][num_kv_heads][B * D]
 * elements; inside one (block, kv head) tile of B*D elements, token o (0 <= o < B) and
 * channel d are at
 *     K:  (d / W) * (B * W) + o * W + (d % W)
 *     V:  ((o / T) * D + d) * T + (o % T)
 * i.e. K is split into 64-byte channel slices stored token-major, and V into groups of T
 * consecutive tokens stored channel-major, the T tokens of one channel side by side.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8_E4M3 = 2, OR_FP8_E5M2 = 3, OR_INT8 = 4 };

enum {
    OR_OK = 0,
    OR_ERR_ARG = 1,
    OR_ERR_DTYPE = 2,
    OR_ERR_BOUNDS = 3,
    OR_ERR_NOMEM = 4,
};

static int elem_bytes(int dtype)
{
    switch (dtype) {
    case OR_F32: return 4;
    case OR_BF16: return 2;
    case OR_FP8_E4M3: return 1;
    case OR_FP8_E5M2: return 1;
    case OR_INT8: return 1;
    default: return 0;
    }
}

/* ---- layout ----------------------------------------------------------------------- */

int64_t oracle_k_elem_index(int64_t block, int kv_head, int token, int d,
                            int num_kv_heads, int head_dim, int block_size, int dtype)
{
    int e = elem_bytes(dtype);
    if (e == 0) return -1;
    int64_t W = 64 / e;
    int64_t tile = ((int64_t)block * num_kv_heads + kv_head) * (int64_t)block_size * head_dim;
    return tile + (d / W) * ((int64_t)block_size * W) + (int64_t)token * W + (d % W);
}

int64_t oracle_v_elem_index(int64_t block, int kv_head, int token, int d,
                            int num_kv_heads, int head_dim, int block_size, int dtype)
{
    int e = elem_bytes(dtype);
    if (e == 0) return -1;
    int64_t T = 16 / e < block_size ? 16 / e : block_size;
    int64_t tile = ((int64_t)block * num_kv_heads + kv_head) * (int64_t)block_size * head_dim;
    return tile + ((int64_t)(token / T) * head_dim + d) * T + (token % T);
}

/* The layout needs whole 64-byte channel slices (K) and whole token groups (V). */
static int layout_ok(int head_dim, int block_size, int dtype)
{
    int e = elem_bytes(dtype);
    if (e == 0 || head_dim <= 0 || block_size <= 0) return 0;
    int T = 16 / e < block_size ? 16 / e : block_size;
    return (head_dim % (64 / e)) == 0 && (block_size % T) == 0;
}

/* ---- element decoders ------------------------------------------------------------- */

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an IEEE binary32 */
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double f32_bits_to_double(const unsigned char* p)
{
    float f;
    memcpy(&f, p, 4);
    return (double)f;
}

/* OCP 8-bit float E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 is subnormal (m * 2^-9); no infinities; S.1111.111 is NaN; max 448. */
double oracle_e4m3_to_double(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* OCP 8-bit float E5M2: 1 sign bit, 5 exponent bits (bias 15), 2 mantissa bits; exponent 0
 * is subnormal (m * 2^-16); exponent 31 holds the infinities (m = 0) and NaNs (m != 0);
 * largest finite value 57344. */
double oracle_e5m2_to_double(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);
    else
        v = ldexp((double)(4 + m), e - 17); /* (1 + m/4) * 2^(e-15) */
    return s ? -v : v;
}

/* Nearest code to a (finite, 0 <= a < value(top)) among codes 0..top, ties to the even code
 * (the code's low bit is the mantissa's low bit).  Codes 0..top are increasing in value. */
static int nearest_code(double a, int top, double (*value)(uint8_t))
{
    int lo = 0, hi = top; /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - value((uint8_t)lo); /* exact: both have few bits */
    double dhi = value((uint8_t)hi) - a;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo % 2 == 0) ? lo : hi;
}

/* Round a binary32 value to E4M3 with round-to-nearest-even, saturating finite
 * magnitudes above the largest finite value (448) to +-448; NaN keeps its sign bit and
 * maps to S.1111.111.  Found by comparing |y| against the sorted table of the 127
 * non-negative finite magnitudes (codes 0..126 are increasing in value). */
uint8_t oracle_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return sign | 0x7f;
    double a = fabs((double)y);
    if (a >= 448.0) return sign | 0x7e;
    return sign | (uint8_t)nearest_code(a, 0x7e, oracle_e4m3_to_double);
}

/* The same rule for E5M2: round to nearest even, finite magnitudes (and infinities) at or
 * above the largest finite value saturate to +-57344 (S.11110.11), NaN keeps its sign and
 * maps to S.11111.11. */
uint8_t oracle_e5m2_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return sign | 0x7f;
    double a = fabs((double)y);
    if (a >= 57344.0) return sign | 0x7b;
    return sign | (uint8_t)nearest_code(a, 0x7b, oracle_e5m2_to_double);
}

/* INT8 cache code: a two's-complement byte c; its value (before the scale) is the integer c. */
double oracle_int8_to_double(uint8_t c) { return (double)(int8_t)c; }

/* Nearest integer to a binary32 value, ties to the even integer, saturated to [-127, 127]
 * (the symmetric range: +x and -x get opposite codes); NaN stores 0.  Written out: n is the
 * integer part below y, r = y - n is exact (|y| < 127 has at most 24 significant bits), and
 * r > 1/2, or r = 1/2 with n odd, rounds up. */
uint8_t oracle_int8_encode(float y)
{
    if (isnan(y)) return 0;
    if (y >= 127.0f) return 127;
    if (y <= -127.0f) return (uint8_t)(int8_t)-127;
    double a = (double)y;
    double f = floor(a);
    double r = a - f;
    long n = (long)f;
    if (r > 0.5 || (r == 0.5 && n % 2 != 0)) n += 1;
    return (uint8_t)(int8_t)n;
}

static int is_fp8(int dtype) { return dtype == OR_FP8_E4M3 || dtype == OR_FP8_E5M2; }

/* A quantised cache (fp8 or INT8): codes times a per-head scale. */
static int is_quant(int dtype) { return is_fp8(dtype) || dtype == OR_INT8; }

static double load_elem(const unsigned char* base, int64_t idx, int dtype)
{
    switch (dtype) {
    case OR_F32: return f32_bits_to_double(base + idx * 4);
    case OR_BF16: {
        uint16_t b;
        memcpy(&b, base + idx * 2, 2);
        return bf16_bits_to_double(b);
    }
    case OR_FP8_E4M3: return oracle_e4m3_to_double(base[idx]);
    case OR_FP8_E5M2: return oracle_e5m2_to_double(base[idx]);
    case OR_INT8: return oracle_int8_to_double(base[idx]);
    default: return NAN;
    }
}

/* ---- paged KV append --------------------------------------------------------------- */

/* For every token i with slot_mapping[i] >= 0 the token goes to physical block
 * slot / block_size at offset slot % block_size, for every kv head and channel.  Same
 * source and cache dtype: the element's bits are copied.  fp32/bf16 source into an E4M3 (E5M2,
 * INT8) cache: the stored code is e4m3(fl32(x / scale[h])) (e5m2(...), int8(...)) -- one IEEE
 * binary32 division by that head's scale, then the rounding above. */
int oracle_kv_cache_write(const void* key, const void* value, int src_dtype,
                          void* k_pool, void* v_pool, int cache_dtype, int64_t num_blocks,
                          const int64_t* slot_mapping, int64_t num_tokens,
                          int num_kv_heads, int head_dim, int block_size,
                          const float* k_scale, const float* v_scale)
{
    int es = elem_bytes(src_dtype), ec = elem_bytes(cache_dtype);
    if (!es || !ec) return OR_ERR_DTYPE;
    if (is_quant(src_dtype)) return OR_ERR_DTYPE;
    if (src_dtype != cache_dtype && !is_quant(cache_dtype)) return OR_ERR_DTYPE;
    if (is_quant(cache_dtype) && (!k_scale || !v_scale)) return OR_ERR_ARG;
    if (!layout_ok(head_dim, block_size, cache_dtype)) return OR_ERR_ARG;
    const unsigned char* src[2] = {(const unsigned char*)key, (const unsigned char*)value};
    unsigned char* dst[2] = {(unsigned char*)k_pool, (unsigned char*)v_pool};
    const float* scl[2] = {k_scale, v_scale};
    for (int64_t i = 0; i < num_tokens; i++) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        int64_t b = slot / block_size;
        int o = (int)(slot % block_size);
        if (b >= num_blocks) return OR_ERR_BOUNDS;
        for (int kv = 0; kv < 2; kv++) {
            for (int h = 0; h < num_kv_heads; h++) {
                for (int d = 0; d < head_dim; d++) {
                    int64_t si = ((int64_t)i * num_kv_heads + h) * head_dim + d;
                    int64_t di = kv == 0
                        ? oracle_k_elem_index(b, h, o, d, num_kv_heads, head_dim, block_size, cache_dtype)
                        : oracle_v_elem_index(b, h, o, d, num_kv_heads, head_dim, block_size, cache_dtype);
                    if (src_dtype == cache_dtype) {
                        memcpy(dst[kv] + di * ec, src[kv] + si * es, (size_t)es);
                    } else {
                        float x;
                        if (src_dtype == OR_F32) {
                            memcpy(&x, src[kv] + si * 4, 4);
                        } else {
                            uint16_t bb;
                            memcpy(&bb, src[kv] + si * 2, 2);
                            x = (float)bf16_bits_to_double(bb);
                        }
                        float y = x / scl[kv][h]; /* binary32 division, round to nearest */
                        dst[kv][di] = cache_dtype == OR_FP8_E4M3   ? oracle_e4m3_encode(y)
                                      : cache_dtype == OR_FP8_E5M2 ? oracle_e5m2_encode(y)
                                                                   : oracle_int8_encode(y);
                    }
                }
            }
        }
    }
    return OR_OK;
}

/* ---- paged attention ---------------------------------------------------------------- */

typedef struct {
    double* out;
    const unsigned char* q;
    int q_dtype;
    const unsigned char* kp;
    const unsigned char* vp;
    int cache_dtype;
    int64_t num_blocks;
    const int32_t* tables;
    int mbps;
    const int32_t* ctx;
    const int32_t* cu_q;
    int num_seqs, hq, hkv, d, bs;
    double scale;
    const float* k_scale;
    const float* v_scale;
    int64_t total_rows;
    int nthreads, tid;
    int status;
} job_t;

/* One query row (sequence s, row i of its q_len rows, query head h). */
static int attend_row(const job_t* J, int s, int64_t row, int i, int q_len, int h)
{
    const int G = J->hq / J->hkv;
    const int g = h / G; /* query head h reads kv head floor(h / G) */
    const int D = J->d, B = J->bs;
    double* out = J->out + (row * J->hq + h) * (int64_t)D;
    int pos = J->ctx[s] - q_len + i; /* the chunk is the last q_len positions of ctx */
    int n = pos + 1;                 /* visible positions 0..pos */
    for (int dd = 0; dd < D; dd++) out[dd] = 0.0;
    if (n <= 0) return OR_OK;
    if ((n + B - 1) / B > J->mbps) return OR_ERR_BOUNDS;
    double ks = 1.0, vs = 1.0;
    if (is_quant(J->cache_dtype)) {
        ks = (double)J->k_scale[g];
        vs = (double)J->v_scale[g];
    }
    double* qv = (double*)malloc(sizeof(double) * D);
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    if (!qv || !z) {
        free(qv);
        free(z);
        return OR_ERR_NOMEM;
    }
    for (int dd = 0; dd < D; dd++)
        qv[dd] = load_elem(J->q, (row * J->hq + h) * (int64_t)D + dd, J->q_dtype);
    /* scores, token by token through the block table */
    for (int t = 0; t < n; t++) {
        int64_t b = J->tables[(int64_t)s * J->mbps + t / B];
        int o = t % B;
        if (b < 0 || b >= J->num_blocks) {
            free(qv);
            free(z);
            return OR_ERR_BOUNDS;
        }
        double dot = 0.0;
        for (int dd = 0; dd < D; dd++) {
            int64_t ki = oracle_k_elem_index(b, g, o, dd, J->hkv, D, B, J->cache_dtype);
            dot += qv[dd] * (ks * load_elem(J->kp, ki, J->cache_dtype));
        }
        z[t] = J->scale * dot;
    }
    /* two-pass softmax */
    double m = -INFINITY;
    for (int t = 0; t < n; t++)
        if (z[t] > m) m = z[t];
    double den = 0.0;
    for (int t = 0; t < n; t++) {
        z[t] = exp(z[t] - m);
        den += z[t];
    }
    for (int t = 0; t < n; t++) {
        int64_t b = J->tables[(int64_t)s * J->mbps + t / B];
        int o = t % B;
        for (int dd = 0; dd < D; dd++) {
            int64_t vi = oracle_v_elem_index(b, g, o, dd, J->hkv, D, B, J->cache_dtype);
            out[dd] += z[t] * (vs * load_elem(J->vp, vi, J->cache_dtype));
        }
    }
    for (int dd = 0; dd < D; dd++) out[dd] /= den;
    free(qv);
    free(z);
    return OR_OK;
}

static void* worker(void* arg)
{
    job_t* J = (job_t*)arg;
    int64_t items = J->total_rows * J->hq;
    for (int64_t it = J->tid; it < items; it += J->nthreads) {
        int64_t row = it / J->hq;
        int h = (int)(it % J->hq);
        /* sequence owning this row: cu_q is a non-decreasing prefix sum */
        int s = 0;
        while (s + 1 < J->num_seqs && J->cu_q[s + 1] <= row) s++;
        int q_len = J->cu_q[s + 1] - J->cu_q[s];
        int i = (int)(row - J->cu_q[s]);
        int st = attend_row(J, s, row, i, q_len, h);
        if (st != OR_OK) {
            J->status = st;
            return NULL;
        }
    }
    return NULL;
}

/* out: float64 [total_rows][num_heads][head_dim], total_rows = cu_q[num_seqs].
 * query: [total_rows][num_heads][head_dim] in q_dtype.  context_lens[s] counts every
 * position of sequence s including its q_len new rows.  Decode is cu_q = 0,1,2,...,S. */
int oracle_paged_attention(double* out, const void* query, int q_dtype,
                           const void* k_pool, const void* v_pool, int cache_dtype,
                           int64_t num_blocks, const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, const int32_t* cu_q, int num_seqs,
                           int num_heads, int num_kv_heads, int head_dim, int block_size,
                           double scale, const float* k_scale, const float* v_scale, int nthreads)
{
    if (!elem_bytes(q_dtype) || is_quant(q_dtype) || !elem_bytes(cache_dtype)) return OR_ERR_DTYPE;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads) return OR_ERR_ARG;
    if (!layout_ok(head_dim, block_size, cache_dtype)) return OR_ERR_ARG;
    if (is_quant(cache_dtype) && (!k_scale || !v_scale)) return OR_ERR_ARG;
    if (num_seqs == 0) return OR_OK;
    for (int s = 0; s < num_seqs; s++)
        if (cu_q[s + 1] < cu_q[s]) return OR_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    job_t base = {out, (const unsigned char*)query, q_dtype, (const unsigned char*)k_pool,
                  (const unsigned char*)v_pool, cache_dtype, num_blocks, block_tables,
                  max_blocks_per_seq, context_lens, cu_q, num_seqs, num_heads, num_kv_heads,
                  head_dim, block_size, scale, k_scale, v_scale, cu_q[num_seqs], nthreads, 0, OR_OK};
    job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nthreads);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return OR_ERR_NOMEM;
    }
    char* running = (char*)calloc((size_t)nthreads, 1);
    if (!running) {
        free(jobs);
        free(th);
        return OR_ERR_NOMEM;
    }
    for (int k = 0; k < nthreads; k++) {
        jobs[k] = base;
        jobs[k].tid = k;
    }
    for (int k = 1; k < nthreads; k++)
        running[k] = pthread_create(&th[k], NULL, worker, &jobs[k]) == 0;
    worker(&jobs[0]);
    for (int k = 1; k < nthreads; k++) {
        if (running[k])
            pthread_join(th[k], NULL);
        else
            worker(&jobs[k]); /* thread could not be started: do its share here */
    }
    free(running);
    int st = OR_OK;
    for (int k = 0; k < nthreads; k++)
        if (jobs[k].status != OR_OK) st = jobs[k].status;
    free(jobs);
    free(th);
    return st;
}

/* Closed form for the KV footprint per token: layers x kv_heads x head_dim x 2 (K and V)
 * x bytes per element (page 1, section 2.1; page 3, section 2.1). */
int64_t oracle_kv_bytes_per_token(int num_layers, int num_kv_heads, int head_dim, int dtype)
{
    return (int64_t)num_layers * num_kv_heads * head_dim * 2 * elem_bytes(dtype);
}

/* Array forms of the E4M3 codec, for exhaustive tests. */
void oracle_e4m3_encode_array(const float* y, uint8_t* codes, int64_t n)
{
    for (int64_t i = 0; i < n; i++) codes[i] = oracle_e4m3_encode(y[i]);
}

void oracle_e4m3_decode_array(const uint8_t* codes, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_to_double(codes[i]);
}

void oracle_e5m2_encode_array(const float* y, uint8_t* codes, int64_t n)
{
    for (int64_t i = 0; i < n; i++) codes[i] = oracle_e5m2_encode(y[i]);
}

void oracle_e5m2_decode_array(const uint8_t* codes, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e5m2_to_double(codes[i]);
}

void oracle_int8_encode_array(const float* y, uint8_t* codes, int64_t n)
{
    for (int64_t i = 0; i < n; i++) codes[i] = oracle_int8_encode(y[i]);
}

void oracle_int8_decode_array(const uint8_t* codes, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = oracle_int8_to_double(codes[i]);
}
