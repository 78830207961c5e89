/*
 * oracle.c -- plain, slow fp64 reference for attention over a block-paged
 * KV cache whose keys are Q8_0 and whose values are Q4_0, and the reference
 * quantiser of the KV writer (binary32 decisions, see its section below).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  It shares
 * no code, header, table or constant with the HIP library: the page layout,
 * the page-table entry encoding and the fp16 format are decoded here from
 * their written definitions.
 *
 * What is computed (per layer):
 *   Exact softmax attention of each query row over the complete, logically
 *   ordered KV history.  Streaming and residency change only where a page
 *   physically lives, never the result ("Adaptive KV Streaming for
 *   llama.cpp", section "Adaptive KV streaming"; "troed's fork of Raymond's
 *   adaptive KV streaming", section "Keep the stock attention order").
 *   Pages hold 256 token positions ("troed's fork ...", section "KV data
 *   movement and attention").
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - Q8_0 block: 32 values, one IEEE binary16 scale d, 32 int8 codes c;
 *     value = d * c.  Q4_0 block: 32 values, one binary16 scale d, 32 4-bit
 *     codes n; value = d * (n - 8).
 *   - Query rows are the last W positions of the N-token history; row r sits
 *     at position N - W + r and sees keys 0 .. N - W + r (causal among the
 *     rows).
 *   - Grouped-query attention: query head h reads KV head floor(h / G),
 *     G = n_q_heads / n_kv_heads.
 *   - Element types: Q8_0 (8), Q4_0 (2), F16 (1, plain IEEE binary16, no
 *     scales).  Supported pairs (K, V): (Q8_0, Q4_0), (Q8_0, Q8_0),
 *     (Q4_0, Q4_0), (F16, F16).
 *   - Page layout (head_dim 128, T tokens per page, H KV heads), four
 *     sections in this order (scales only for the block types):
 *       K codes   H * T * kc bytes (kc = 128 Q8_0, 64 Q4_0, 256 F16)
 *       K scales  binary16 H * T * 4
 *       V codes   H * T * vc bytes (vc = 128 Q8_0, 64 Q4_0, 256 F16)
 *       V scales  binary16 H * T * 4
 *     K scales are stored [head][token][block].  V scales of head h start at
 *     h*T*8 bytes into their section, in 32-token tiles of 256 bytes; inside
 *     a tile, token j (jj = j%32) and block b sit at
 *         (b*4 + (jj%16)/4)*16 + ((jj/16)*4 + jj%4)*2.
 *     K codes of head h start at h*T*kc in 16-token tiles of 16*kc bytes;
 *     inside a tile, for token j and dim t:
 *       Q8_0  byte (t/64)*1024 + (((t%32)/8)*16 + j%16)*16 + ((t/32)%2)*8 + t%8
 *       Q4_0  byte (((t%32)/8)*16 + j%16)*16 + (t/32)*4 + (t%8)%4, the low
 *             nibble when t%8 < 4, else the high nibble
 *       F16   bytes at (t/32)*1024 + (((t%32)/8)*16 + j%16)*16 + (t%8)*2
 *     V codes of head h start at h*T*vc in 32-token tiles of 32*vc bytes;
 *     with jj = j%32, g = (jj%16)/4 and s = (jj/16)*4 + jj%4:
 *       Q4_0  byte (t/64)*1024 + (g*16 + t%16)*16 + ((t/16)%4)*4 + jj%4, the
 *             low nibble when jj < 16, else the high nibble
 *       Q8_0  byte (t/32)*1024 + (g*16 + t%16)*16 + ((t/16)%2)*8 + s
 *       F16   bytes at (t/16)*1024 + (g*16 + t%16)*16 + s*2
 *     binary16 values are little-endian.
 *   - Page-table entry: an id below 0x80000000 names a pool page;
 *     0x80000000|s names ring slot s; 0xFFFFFFFF means "in the host
 *     history", i.e. logical page P is page P of the layer's host copy.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HEAD_DIM 128
#define BLOCK 32
#define N_BLOCKS (HEAD_DIM / BLOCK)

/* ---------------------------------------------------------------------- */
/* IEEE 754 binary16 -> double, from the format's definition.              */
/* ---------------------------------------------------------------------- */
double oracle_f16_to_f64(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int exponent = (bits >> 10) & 0x1F;
    int mantissa = bits & 0x3FF;
    double v;
    if (exponent == 0) {
        v = ldexp((double)mantissa, -24); /* subnormal: m * 2^-14 * 2^-10 */
    } else if (exponent == 31) {
        v = mantissa ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + mantissa), exponent - 25); /* 1.m * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* ---------------------------------------------------------------------- */
/* Page layout reading                                                     */
/* ---------------------------------------------------------------------- */
#define T_F16 1
#define T_Q4_0 2
#define T_Q8_0 8

static int code_bytes(int type) { return type == T_Q8_0 ? HEAD_DIM : type == T_Q4_0 ? HEAD_DIM / 2 : 2 * HEAD_DIM; }
static int scale_bytes(int type) { return type == T_F16 ? 0 : N_BLOCKS * 2; }

static size_t sec_k_codes(int kt, int vt, int H, int T) { (void)kt; (void)vt; (void)H; (void)T; return 0; }
static size_t sec_k_scales(int kt, int vt, int H, int T) { (void)vt; return (size_t)H * T * code_bytes(kt); }
static size_t sec_v_codes(int kt, int vt, int H, int T) {
    return sec_k_scales(kt, vt, H, T) + (size_t)H * T * scale_bytes(kt);
}
static size_t sec_v_scales(int kt, int vt, int H, int T) {
    return sec_v_codes(kt, vt, H, T) + (size_t)H * T * code_bytes(vt);
}

int oracle_pair_supported(int kt, int vt) {
    return (kt == T_Q8_0 && vt == T_Q4_0) || (kt == T_Q8_0 && vt == T_Q8_0) || (kt == T_Q4_0 && vt == T_Q4_0) ||
           (kt == T_F16 && vt == T_F16);
}

size_t oracle_page_bytes(int kt, int vt, int n_kv_heads, int page_tokens) {
    return sec_v_scales(kt, vt, n_kv_heads, page_tokens) + (size_t)n_kv_heads * page_tokens * scale_bytes(vt);
}

static uint16_t read_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* The code of (head, token j, dim t): Q8_0 the signed int8, Q4_0 the nibble
 * n (0..15), F16 the binary16 bits. */
int oracle_k_code(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int t) {
    const int kc = code_bytes(kt);
    const size_t base = sec_k_codes(kt, vt, H, T) + (size_t)head * T * kc + (size_t)(j / 16) * 16 * kc;
    const size_t lane = (size_t)(((t % 32) / 8) * 16 + j % 16);
    if (kt == T_Q8_0) {
        size_t off = (size_t)(t / 64) * 1024 + lane * 16 + (size_t)((t / 32) % 2) * 8 + (size_t)(t % 8);
        return (int)(int8_t)page[base + off];
    }
    if (kt == T_Q4_0) {
        uint8_t byte = page[base + lane * 16 + (size_t)(t / 32) * 4 + (size_t)((t % 8) % 4)];
        return (t % 8) < 4 ? (byte & 0x0F) : (byte >> 4);
    }
    return (int)read_u16(page + base + (size_t)(t / 32) * 1024 + lane * 16 + (size_t)(t % 8) * 2);
}

int oracle_v_code(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int t) {
    const int vc = code_bytes(vt);
    const int jj = j % 32, g = (jj % 16) / 4, slot = (jj / 16) * 4 + jj % 4;
    const size_t base = sec_v_codes(kt, vt, H, T) + (size_t)head * T * vc + (size_t)(j / 32) * 32 * vc;
    const size_t lane = (size_t)(g * 16 + t % 16);
    if (vt == T_Q4_0) {
        uint8_t byte = page[base + (size_t)(t / 64) * 1024 + lane * 16 + (size_t)((t / 16) % 4) * 4 + (size_t)(jj % 4)];
        return jj < 16 ? (byte & 0x0F) : (byte >> 4);
    }
    if (vt == T_Q8_0) {
        return (int)(int8_t)page[base + (size_t)(t / 32) * 1024 + lane * 16 + (size_t)((t / 16) % 2) * 8 + (size_t)slot];
    }
    return (int)read_u16(page + base + (size_t)(t / 16) * 1024 + lane * 16 + (size_t)slot * 2);
}

static uint16_t k_scale_bits(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int block) {
    size_t off = sec_k_scales(kt, vt, H, T) + (((size_t)head * T + j) * N_BLOCKS + block) * 2;
    return read_u16(page + off);
}

static uint16_t v_scale_bits(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int block) {
    int jj = j % 32;
    size_t off = sec_v_scales(kt, vt, H, T) + (size_t)head * T * N_BLOCKS * 2 + (size_t)(j / 32) * 256 +
                 (size_t)(block * 4 + (jj % 16) / 4) * 16 + (size_t)((jj / 16) * 4 + jj % 4) * 2;
    return read_u16(page + off);
}

double oracle_k_scale(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int block) {
    return kt == T_F16 ? 1.0 : oracle_f16_to_f64(k_scale_bits(page, kt, vt, H, T, head, j, block));
}

double oracle_v_scale(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int block) {
    return vt == T_F16 ? 1.0 : oracle_f16_to_f64(v_scale_bits(page, kt, vt, H, T, head, j, block));
}

/* Element value of a code of the given type (exact in fp64). */
static double value_of(int type, double scale, int code) {
    if (type == T_Q8_0) return scale * (double)code;
    if (type == T_Q4_0) return scale * (double)(code - 8);
    return oracle_f16_to_f64((uint16_t)code);
}

/* Dequantised key / value element (exact in fp64). */
double oracle_k_value(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int t) {
    return value_of(kt, oracle_k_scale(page, kt, vt, H, T, head, j, t / BLOCK),
                    oracle_k_code(page, kt, vt, H, T, head, j, t));
}

double oracle_v_value(const uint8_t *page, int kt, int vt, int H, int T, int head, int j, int t) {
    return value_of(vt, oracle_v_scale(page, kt, vt, H, T, head, j, t / BLOCK),
                    oracle_v_code(page, kt, vt, H, T, head, j, t));
}

/* ---------------------------------------------------------------------- */
/* Page-table resolution                                                   */
/* ---------------------------------------------------------------------- */
typedef struct {
    const uint8_t *pool;    size_t n_pool;   /* pool pages */
    const uint8_t *ring;    size_t n_ring;   /* ring slots */
    const uint8_t *history;                  /* layer's host copy, logical order (may be NULL) */
    size_t page_bytes;
} oracle_store;

/* Returns the page's bytes, or NULL when the entry names nothing valid. */
static const uint8_t *resolve(const oracle_store *st, uint32_t entry, size_t logical_page) {
    if (entry == 0xFFFFFFFFu) {
        return st->history ? st->history + logical_page * st->page_bytes : NULL;
    }
    if (entry & 0x80000000u) {
        size_t slot = entry & 0x7FFFFFFFu;
        return slot < st->n_ring ? st->ring + slot * st->page_bytes : NULL;
    }
    return entry < st->n_pool ? st->pool + (size_t)entry * st->page_bytes : NULL;
}

/* ---------------------------------------------------------------------- */
/* Attention over one row / head: scores, softmax, weighted sum.           */
/* A "key source" gives K-hat and V-hat rows of one KV head.               */
/* ---------------------------------------------------------------------- */
typedef struct {
    /* paged */
    const uint8_t *const *pages; int H; int T; int kt; int vt;
    /* logical (unpaged, Q8_0 K / Q4_0 V): [N][H][128] codes, [N][H][4] scales */
    const int8_t *kc; const uint16_t *kd; const uint8_t *vc; const uint16_t *vd;
    /* plain values: [N][H][128] fp64 (any type, dequantised by the caller) */
    const double *kv; const double *vv;
} key_source;

static void k_row(const key_source *src, int g, int j, double *out) {
    if (src->pages) {
        const uint8_t *pg = src->pages[j / src->T];
        for (int t = 0; t < HEAD_DIM; t++)
            out[t] = oracle_k_value(pg, src->kt, src->vt, src->H, src->T, g, j % src->T, t);
    } else if (src->kv) {
        memcpy(out, src->kv + ((size_t)j * src->H + g) * HEAD_DIM, sizeof(double) * HEAD_DIM);
    } else {
        size_t row = ((size_t)j * src->H + g);
        for (int t = 0; t < HEAD_DIM; t++)
            out[t] = oracle_f16_to_f64(src->kd[row * N_BLOCKS + t / BLOCK]) * (double)src->kc[row * HEAD_DIM + t];
    }
}

static void v_row(const key_source *src, int g, int j, double *out) {
    if (src->pages) {
        const uint8_t *pg = src->pages[j / src->T];
        for (int t = 0; t < HEAD_DIM; t++)
            out[t] = oracle_v_value(pg, src->kt, src->vt, src->H, src->T, g, j % src->T, t);
    } else if (src->vv) {
        memcpy(out, src->vv + ((size_t)j * src->H + g) * HEAD_DIM, sizeof(double) * HEAD_DIM);
    } else {
        size_t row = ((size_t)j * src->H + g);
        for (int t = 0; t < HEAD_DIM; t++)
            out[t] = oracle_f16_to_f64(src->vd[row * N_BLOCKS + t / BLOCK]) * ((double)src->vc[row * HEAD_DIM + t] - 8.0);
    }
}

/* Softmax attention of query q (fp32, 128) over keys [k0, k1) of KV head g.
 * Writes the un-normalised partial (m, l, acc) of the split: m = max score,
 * l = sum exp(s - m), acc = sum exp(s - m) * v.  An empty range gives
 * m = -inf, l = 0, acc = 0. */
static void attend_range(const key_source *src, int g, const float *q, double scale, int k0, int k1,
                         double *m_out, double *l_out, double *acc) {
    double krow[HEAD_DIM], vrow[HEAD_DIM];
    int n = k1 - k0;
    memset(acc, 0, sizeof(double) * HEAD_DIM);
    if (n <= 0) { *m_out = -INFINITY; *l_out = 0.0; return; }
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = k0; j < k1; j++) {
        k_row(src, g, j, krow);
        double dot = 0.0;
        for (int t = 0; t < HEAD_DIM; t++) dot += (double)q[t] * krow[t];
        s[j - k0] = scale * dot;
        if (s[j - k0] > m) m = s[j - k0];
    }
    double l = 0.0;
    for (int j = k0; j < k1; j++) {
        double w = exp(s[j - k0] - m);
        l += w;
        v_row(src, g, j, vrow);
        for (int t = 0; t < HEAD_DIM; t++) acc[t] += w * vrow[t];
    }
    free(s);
    *m_out = m; *l_out = l;
}

/* Full attention for a list of rows. q: [W][Hq][128] fp32.  rows: which of
 * the W rows to compute (NULL = all); out: [n_rows][Hq][128]; lse:
 * [n_rows][Hq] natural-log sum-exp of the scaled scores. */
static int attend_rows(const key_source *src, int n_tokens, int Hq, int Hkv, const float *q, int W,
                       double scale, const int *rows, int n_rows, double *out, double *lse, int n_threads) {
    if (Hkv <= 0 || Hq % Hkv != 0 || W <= 0 || W > n_tokens) return -1;
    int G = Hq / Hkv;
    if (!rows) n_rows = W;
    int units = n_rows * Hq;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int u = 0; u < units; u++) {
        int ri = u / Hq, h = u % Hq;
        int r = rows ? rows[ri] : ri;
        if (r < 0 || r >= W) { bad = 1; continue; }
        int pos = n_tokens - W + r;               /* row's own position */
        double m, l, acc[HEAD_DIM];
        attend_range(src, h / G, q + ((size_t)r * Hq + h) * HEAD_DIM, scale, 0, pos + 1, &m, &l, acc);
        double *o = out + ((size_t)ri * Hq + h) * HEAD_DIM;
        for (int t = 0; t < HEAD_DIM; t++) o[t] = acc[t] / l;
        if (lse) lse[(size_t)ri * Hq + h] = m + log(l);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------- */
/* Public entry points                                                     */
/* ---------------------------------------------------------------------- */

/* Attention through a page table.  page_table[P] for P < ceil(N / T). */
int oracle_attend_paged(const uint8_t *pool, size_t n_pool, const uint8_t *ring, size_t n_ring,
                        const uint8_t *history, const uint32_t *page_table, int n_tokens, int page_tokens,
                        int kt, int vt, int Hq, int Hkv, const float *q, int W, double scale, const int *rows,
                        int n_rows, double *out, double *lse, int n_threads) {
    if (n_tokens <= 0 || page_tokens <= 0 || page_tokens % 32 != 0 || !oracle_pair_supported(kt, vt)) return -1;
    oracle_store st = {pool, n_pool, ring, n_ring, history, oracle_page_bytes(kt, vt, Hkv, page_tokens)};
    int n_pages = (n_tokens + page_tokens - 1) / page_tokens;
    const uint8_t **pages = (const uint8_t **)malloc(sizeof(uint8_t *) * (size_t)n_pages);
    for (int p = 0; p < n_pages; p++) {
        pages[p] = resolve(&st, page_table[p], (size_t)p);
        if (!pages[p]) { free(pages); return -2; }
    }
    key_source src = {pages, Hkv, page_tokens, kt, vt, NULL, NULL, NULL, NULL, NULL, NULL};
    int rc = attend_rows(&src, n_tokens, Hq, Hkv, q, W, scale, rows, n_rows, out, lse, n_threads);
    free(pages);
    return rc;
}

/* Attention over unpaged logical arrays (the quantiser's own output). */
int oracle_attend_logical(const int8_t *kc, const uint16_t *kd, const uint8_t *vc, const uint16_t *vd,
                          int n_tokens, int Hq, int Hkv, const float *q, int W, double scale, const int *rows,
                          int n_rows, double *out, double *lse, int n_threads) {
    key_source src = {NULL, Hkv, 0, T_Q8_0, T_Q4_0, kc, kd, vc, vd, NULL, NULL};
    return attend_rows(&src, n_tokens, Hq, Hkv, q, W, scale, rows, n_rows, out, lse, n_threads);
}

/* Attention over plain fp64 keys and values [N][Hkv][128] (any element type,
 * dequantised by the caller). */
int oracle_attend_values(const double *kv, const double *vv, int n_tokens, int Hq, int Hkv, const float *q, int W,
                         double scale, const int *rows, int n_rows, double *out, double *lse, int n_threads) {
    key_source src = {NULL, Hkv, 0, 0, 0, NULL, NULL, NULL, NULL, kv, vv};
    return attend_rows(&src, n_tokens, Hq, Hkv, q, W, scale, rows, n_rows, out, lse, n_threads);
}

/* Split partials: keys of row r (0 .. pos_r) cut at the given boundaries
 * (bounds[0] = 0 < ... < bounds[n_splits] >= n_tokens), each split reduced
 * on its own to (m, l, acc).  Layout: m, l [n_splits][W][Hq]; acc
 * [n_splits][W][Hq][128].  Keys beyond a row's position are excluded. */
int oracle_split_partials(const uint8_t *const *pages, int page_tokens, int kt, int vt, int n_tokens, int Hq,
                          int Hkv, const float *q, int W, double scale, const int *bounds, int n_splits,
                          double *m, double *l, double *acc) {
    if (Hkv <= 0 || Hq % Hkv != 0 || W <= 0 || W > n_tokens || !oracle_pair_supported(kt, vt)) return -1;
    int G = Hq / Hkv;
    key_source src = {pages, Hkv, page_tokens, kt, vt, NULL, NULL, NULL, NULL, NULL, NULL};
    for (int s = 0; s < n_splits; s++)
        for (int r = 0; r < W; r++)
            for (int h = 0; h < Hq; h++) {
                int pos = n_tokens - W + r;
                int k0 = bounds[s], k1 = bounds[s + 1] < pos + 1 ? bounds[s + 1] : pos + 1;
                size_t u = ((size_t)s * W + r) * Hq + h;
                attend_range(&src, h / G, q + ((size_t)r * Hq + h) * HEAD_DIM, scale, k0, k1, &m[u], &l[u],
                             acc + u * HEAD_DIM);
            }
    return 0;
}

/* Log-sum-exp merge of split partials, splits taken in index order:
 *   M = max_s m_s;  L = sum_s e^(m_s - M) l_s;  O = sum_s e^(m_s - M) acc_s / L.
 * Empty splits (l = 0) are skipped.  units = W * Hq. */
int oracle_merge(const double *m, const double *l, const double *acc, int n_splits, int units, double *out) {
    for (int u = 0; u < units; u++) {
        double M = -INFINITY;
        for (int s = 0; s < n_splits; s++)
            if (l[(size_t)s * units + u] > 0.0 && m[(size_t)s * units + u] > M) M = m[(size_t)s * units + u];
        double L = 0.0, o[HEAD_DIM];
        memset(o, 0, sizeof(o));
        for (int s = 0; s < n_splits; s++) {
            size_t i = (size_t)s * units + u;
            if (l[i] <= 0.0) continue;
            double w = exp(m[i] - M);
            L += w * l[i];
            for (int t = 0; t < HEAD_DIM; t++) o[t] += w * acc[i * HEAD_DIM + t];
        }
        if (L <= 0.0) return -1;
        for (int t = 0; t < HEAD_DIM; t++) out[(size_t)u * HEAD_DIM + t] = o[t] / L;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * KV writer reference: quantise fp32 rows into Q8_0 / Q4_0 blocks.
 *
 * The pages name the block types and say the KV writer quantises the new
 * rows before attention reads them ("troed's fork ...", section "KV data
 * movement and attention"); they do not spell out the quantiser.  Reading
 * (the common one for these block types):
 *   Q8_0: d = amax / 127 rounded to binary16; code = round-half-even(x / d)
 *         clamped to [-127, 127]; d = 0 gives codes 0.
 *   Q4_0: m = the element of largest magnitude (first on ties, sign kept);
 *         d = m / -8 rounded to binary16; code = round-half-even(x / d) + 8
 *         clamped to [0, 15]; d = 0 gives codes 8.
 * The code of each element is a decision taken in binary32 arithmetic (the
 * division x / d and the rounding), so this reference takes it in binary32
 * too; the scale is the binary32 quotient amax / 127 (or m / -8) rounded to
 * binary16.
 * ---------------------------------------------------------------------- */

/* binary32 -> binary16, round to nearest, ties to even, from the two
 * formats' bit definitions (IEEE 754): 1 + 5 + 10 bits, exponent bias 15,
 * subnormals of 2^-24 units, overflow to infinity, NaN stays NaN. */
uint16_t oracle_f32_to_f16(float x) {
    uint32_t f;
    memcpy(&f, &x, 4);
    const uint32_t sign = (f >> 16) & 0x8000u;
    const uint32_t a = f & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) return (uint16_t)(sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u));
    if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520: past the largest finite */
    if (a >= 0x38800000u) {                                 /* >= 2^-14: a normal binary16 */
        const uint32_t e = (a >> 23) - 127 + 15;
        const uint32_t m = a & 0x7FFFFFu;
        uint32_t h = (e << 10) | (m >> 13);
        const uint32_t rest = m & 0x1FFFu;
        if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h++; /* a carry moves into the exponent */
        return (uint16_t)(sign | h);
    }
    if (a <= 0x33000000u) return (uint16_t)sign; /* <= 2^-25: rounds to zero (2^-25 is a tie, to even) */
    /* subnormal binary16: value = M * 2^(E - 150); units of 2^-24 */
    const uint32_t E = a >> 23;
    const uint32_t M = (a & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126 - E; /* 14 .. 24 here */
    uint32_t q = M >> shift;
    const uint32_t rem = M & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    return (uint16_t)(sign | q);
}

static float f16_to_f32_exact(uint16_t h) { return (float)oracle_f16_to_f64(h); }

/* n_blocks blocks of 32 values: codes[32 * n], scales[n] (binary16 bits). */
void oracle_quantize_q8_0(const float *x, int n_blocks, int8_t *codes, uint16_t *scales) {
    for (int b = 0; b < n_blocks; b++) {
        const float *xb = x + (size_t)b * BLOCK;
        float amax = 0.0f;
        for (int i = 0; i < BLOCK; i++) {
            const float v = fabsf(xb[i]);
            if (v > amax) amax = v;
        }
        const uint16_t d16 = oracle_f32_to_f16(amax / 127.0f);
        const float d = f16_to_f32_exact(d16);
        scales[b] = d16;
        for (int i = 0; i < BLOCK; i++) {
            float c = 0.0f;
            if (d != 0.0f) {
                c = rintf(xb[i] / d);
                if (c > 127.0f) c = 127.0f;
                if (c < -127.0f) c = -127.0f;
            }
            codes[(size_t)b * BLOCK + i] = (int8_t)c;
        }
    }
}

/* codes are the 4-bit values 0..15, one per byte. */
void oracle_quantize_q4_0(const float *x, int n_blocks, uint8_t *codes, uint16_t *scales) {
    for (int b = 0; b < n_blocks; b++) {
        const float *xb = x + (size_t)b * BLOCK;
        int imax = 0;
        float amax = fabsf(xb[0]);
        for (int i = 1; i < BLOCK; i++) {
            if (fabsf(xb[i]) > amax) {
                amax = fabsf(xb[i]);
                imax = i;
            }
        }
        const uint16_t d16 = oracle_f32_to_f16(xb[imax] / -8.0f);
        const float d = f16_to_f32_exact(d16);
        scales[b] = d16;
        for (int i = 0; i < BLOCK; i++) {
            float c = 8.0f;
            if (d != 0.0f) {
                c = rintf(xb[i] / d) + 8.0f;
                if (c > 15.0f) c = 15.0f;
                if (c < 0.0f) c = 0.0f;
            }
            codes[(size_t)b * BLOCK + i] = (uint8_t)c;
        }
    }
}

/* Every code and scale of one page, in logical order: kcode, vcode int32
 * [T][H][128] (Q8_0 the signed code, Q4_0 the nibble, F16 the binary16
 * bits); kd, vd binary16 [T][H][4] (zero for F16). */
void oracle_unpack_page(const uint8_t *page, int kt, int vt, int H, int T, int32_t *kcode, uint16_t *kd,
                        int32_t *vcode, uint16_t *vd) {
    for (int j = 0; j < T; j++)
        for (int h = 0; h < H; h++) {
            const size_t row = (size_t)j * H + h;
            for (int t = 0; t < HEAD_DIM; t++) {
                kcode[row * HEAD_DIM + t] = oracle_k_code(page, kt, vt, H, T, h, j, t);
                vcode[row * HEAD_DIM + t] = oracle_v_code(page, kt, vt, H, T, h, j, t);
            }
            for (int b = 0; b < N_BLOCKS; b++) {
                kd[row * N_BLOCKS + b] = kt == T_F16 ? 0 : k_scale_bits(page, kt, vt, H, T, h, j, b);
                vd[row * N_BLOCKS + b] = vt == T_F16 ? 0 : v_scale_bits(page, kt, vt, H, T, h, j, b);
            }
        }
}
