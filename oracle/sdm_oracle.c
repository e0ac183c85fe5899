/*
 * Oracle for the sparse-delta-memory (SDM) decode step and token gather.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path never
 * calls it, and it shares no code, header, table or helper with the HIP
 * kernels.
 *
 * It is the plain definition written out as sequential loops, one stream (or
 * token) at a time, in the order the method states it:
 *
 *   decode (page "sparse_delta_memory/decode.py", docstring of sdm_decode_step):
 *     d = exp(g);  retrieved = sum_w k_val[w] d[w] memory[k_idx[w]]
 *     delta_v = beta (v - retrieved)
 *     memory[k_idx[w]] = d[w] memory[k_idx[w]] + k_val[w] delta_v   (written rows only)
 *     readings = sum_r q_val[r] memory[q_idx[r]]                      (after the write)
 *   with k_val, v, q_val rounded to the bank dtype, beta and g used in float32,
 *   rows stored and readings returned in the bank dtype (same docstring, and the
 *   casts of _sdm_decode_kernel on that page).
 *
 *   token gather (page "sparse_delta_memory/cuda/gather_cuda.py", module docstring):
 *     out_o[t] = sum_n w_o[t,n] bank[idx_o[t,n]]   (float32 accumulation)
 *     stash[t,n] = bank[idx_0[t,n]]                (raw rows of operand 0)
 *   token t is padding when (t mod chunk) >= valid: zero outputs, zero stash rows.
 *   Group g sums entries g, g+groups, ... in ascending order from +0; the group
 *   partials are then summed in group order from +0 (same docstring).
 *
 * Readings of the pages taken here where they leave a step open:
 *   - float32 -> bfloat16 is round-to-nearest-even (NaN stays NaN);
 *   - d = exp(g) is the correctly rounded float of exp((double)g);
 *   - the float32 decode sums over w (and r) use the same grouped order as the
 *     gather, with groups = 1 meaning one ascending fused multiply-add chain;
 *     any grouping is a correct result (the pages fix no order for the decode);
 *   - the update is fma(k_val[w], delta_v, row * d[w]) with row * d[w] rounded;
 *   - the reads see the rows as stored, i.e. already rounded to the bank dtype.
 *
 * The *_f64 functions are the brute-force references used to pin the float32
 * functions: every operation in double, with only the input roundings to the
 * bank dtype and the final store rounding (taken directly from double).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -o libsdm_oracle.so sdm_oracle.c -lm
 * (no contraction, so every a*b+c written here is two roundings and every
 * fmaf() one).
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_WIDTH 256

enum {
    ORACLE_OK = 0,
    ORACLE_E_ARG = -1,        /* bad sizes or widths */
    ORACLE_E_SLOT = -2,       /* slot outside [0, num_slots) */
    ORACLE_E_DUP = -3,        /* repeated write slot within one stream */
    ORACLE_E_NOMEM = -4,
    ORACLE_E_POS = -5,        /* compact-stash position past its block, or named by two slots */
};

/* ---------------------------------------------------------------- bfloat16 */

static float bits_to_float(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t float_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* A bfloat16 is the high half of a float32, so widening is exact. */
float oracle_bf16_to_float(uint16_t b) { return bits_to_float((uint32_t)b << 16); }

/* Round a float32 to bfloat16, to nearest, ties to even. */
uint16_t oracle_float_to_bf16(float f) {
    uint32_t u = float_to_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep sign, force quiet */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t low = u & 0xffffu, keep = u >> 16;
    if (low > 0x8000u || (low == 0x8000u && (keep & 1u))) keep += 1u; /* carries into the exponent on overflow */
    return (uint16_t)keep;
}

/* oracle_float_to_bf16 over an array (for checking a conversion over many inputs). */
void oracle_float_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_float_to_bf16(in[i]);
}

/* Round a double straight to bfloat16 (one rounding, to nearest, ties to even). */
uint16_t oracle_double_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0u;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7f80u);
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int q = e - 1 - 7;            /* bfloat16 spacing there: 8 significant bits */
    if (q < -133) q = -133;       /* subnormal spacing 2^-133 */
    double r = nearbyint(ldexp(a, -q)); /* exact scaling, then ties-to-even */
    double y = ldexp(r, q);
    if (y >= 0x1p128) return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | (float_to_bits((float)y) >> 16)); /* y is a bfloat16 value: exact */
}

/* Round a float32 to the bank dtype and widen back. */
static float round_to_bank(float x, int bank_bf16) {
    return bank_bf16 ? oracle_bf16_to_float(oracle_float_to_bf16(x)) : x;
}

static float bank_load(const void* bank, int bank_bf16, int64_t hd, int64_t row, int64_t c) {
    if (bank_bf16) return oracle_bf16_to_float(((const uint16_t*)bank)[row * hd + c]);
    return ((const float*)bank)[row * hd + c];
}

static void bank_store_f32(void* bank, int bank_bf16, int64_t hd, int64_t row, int64_t c, float x) {
    if (bank_bf16) ((uint16_t*)bank)[row * hd + c] = oracle_float_to_bf16(x);
    else ((float*)bank)[row * hd + c] = x;
}

static void bank_store_f64(void* bank, int bank_bf16, int64_t hd, int64_t row, int64_t c, double x) {
    if (bank_bf16) ((uint16_t*)bank)[row * hd + c] = oracle_double_to_bf16(x);
    else ((float*)bank)[row * hd + c] = (float)x;
}

/* ------------------------------------------------------------ shared checks */

static int check_decode_args(int64_t num_slots, int64_t hd, int64_t streams, int W, int R, int G,
                             int groups, const int64_t* k_idx, const int64_t* q_idx) {
    if (num_slots < 1 || hd < 1 || streams < 0) return ORACLE_E_ARG;
    if (W < 1 || W > ORACLE_MAX_WIDTH || R < 1 || R > ORACLE_MAX_WIDTH) return ORACLE_E_ARG;
    if (G != 1 && G != W) return ORACLE_E_ARG;
    if (groups < 1) return ORACLE_E_ARG;
    for (int64_t i = 0; i < streams * W; ++i)
        if (k_idx[i] < 0 || k_idx[i] >= num_slots) return ORACLE_E_SLOT;
    for (int64_t i = 0; i < streams * R; ++i)
        if (q_idx[i] < 0 || q_idx[i] >= num_slots) return ORACLE_E_SLOT;
    /* Write slots are distinct within a stream: a precondition of the method. */
    for (int64_t s = 0; s < streams; ++s)
        for (int a = 0; a < W; ++a)
            for (int b = a + 1; b < W; ++b)
                if (k_idx[s * W + a] == k_idx[s * W + b]) return ORACLE_E_DUP;
    return ORACLE_OK;
}

/* Sum over i < n of a[i] * x[i * stride]: group g takes i = g, g + groups, ...
 * ascending as one fused multiply-add chain from +0; the partials are then
 * added in group order from +0. */
static float grouped_dot(const float* a, const float* x, int64_t stride, int n, int groups) {
    float total = 0.0f;
    for (int g = 0; g < groups; ++g) {
        float p = 0.0f;
        for (int i = g; i < n; i += groups) p = fmaf(a[i], x[(int64_t)i * stride], p);
        total = total + p;
    }
    return total;
}

/* ----------------------------------------------------- decode, float32 path */

int sdm_oracle_decode_step(void* bank, int bank_bf16, int64_t num_slots, int64_t hd, int64_t streams,
                           int W, int R, int G, int groups, const int64_t* k_idx, const float* k_val,
                           const float* v, const float* beta, const float* g, const int64_t* q_idx,
                           const float* q_val, void* readings) {
    int rc = check_decode_args(num_slots, hd, streams, W, R, G, groups, k_idx, q_idx);
    if (rc != ORACLE_OK) return rc;
    const int64_t n_rows = (W > R ? W : R);
    float* rows = (float*)malloc(sizeof(float) * (size_t)(n_rows * hd));
    float* kv = (float*)malloc(sizeof(float) * ORACLE_MAX_WIDTH);
    float* d = (float*)malloc(sizeof(float) * ORACLE_MAX_WIDTH);
    float* coef = (float*)malloc(sizeof(float) * ORACLE_MAX_WIDTH);
    float* qv = (float*)malloc(sizeof(float) * ORACLE_MAX_WIDTH);
    float* dv = (float*)malloc(sizeof(float) * (size_t)hd);
    if (!rows || !kv || !d || !coef || !qv || !dv) {
        free(rows); free(kv); free(d); free(coef); free(qv); free(dv);
        return ORACLE_E_NOMEM;
    }
    for (int64_t s = 0; s < streams; ++s) {
        const int64_t* ks = k_idx + s * W;
        const int64_t* qs = q_idx + s * R;
        /* Per-write weight (rounded to the bank dtype), decay and coefficient. */
        for (int w = 0; w < W; ++w) {
            kv[w] = round_to_bank(k_val[s * W + w], bank_bf16);
            d[w] = (float)exp((double)g[s * G + (G == 1 ? 0 : w)]);
            coef[w] = kv[w] * d[w];
        }
        /* The written rows as they are before this step's writes. */
        for (int w = 0; w < W; ++w)
            for (int64_t c = 0; c < hd; ++c) rows[w * hd + c] = bank_load(bank, bank_bf16, hd, ks[w], c);
        /* retrieved and delta_v, column by column. */
        const float b = beta[s];
        for (int64_t c = 0; c < hd; ++c) {
            float retrieved = grouped_dot(coef, rows + c, hd, W, groups);
            float vc = round_to_bank(v[s * hd + c], bank_bf16);
            dv[c] = b * (vc - retrieved);
        }
        /* Decay-and-write of the W rows; no other slot changes. */
        for (int w = 0; w < W; ++w)
            for (int64_t c = 0; c < hd; ++c) {
                float decayed = rows[w * hd + c] * d[w];
                bank_store_f32(bank, bank_bf16, hd, ks[w], c, fmaf(kv[w], dv[c], decayed));
            }
        /* Read after the write: rows as stored in the bank dtype. */
        for (int r = 0; r < R; ++r) {
            qv[r] = round_to_bank(q_val[s * R + r], bank_bf16);
            for (int64_t c = 0; c < hd; ++c) rows[r * hd + c] = bank_load(bank, bank_bf16, hd, qs[r], c);
        }
        for (int64_t c = 0; c < hd; ++c) {
            float out = grouped_dot(qv, rows + c, hd, R, groups);
            bank_store_f32(readings, bank_bf16, hd, s, c, out);
        }
    }
    free(rows); free(kv); free(d); free(coef); free(qv); free(dv);
    return ORACLE_OK;
}

/* ------------------------------------------------ decode, float64 brute force */

/* Same step in double. row_exact/row_mag ([streams, W, hd]) receive the unrounded
 * new rows and the magnitude |row d| + |kv| |beta| (|v| + sum_w |kv d row|);
 * read_exact/read_mag ([streams, hd]) the unrounded readings and sum_r |qv row|.
 * Any of the four may be NULL. */
int sdm_oracle_decode_step_f64(void* bank, int bank_bf16, int64_t num_slots, int64_t hd, int64_t streams,
                               int W, int R, int G, const int64_t* k_idx, const float* k_val,
                               const float* v, const float* beta, const float* g, const int64_t* q_idx,
                               const float* q_val, void* readings, double* row_exact, double* row_mag,
                               double* read_exact, double* read_mag) {
    int rc = check_decode_args(num_slots, hd, streams, W, R, G, 1, k_idx, q_idx);
    if (rc != ORACLE_OK) return rc;
    const int64_t n_rows = (W > R ? W : R);
    double* rows = (double*)malloc(sizeof(double) * (size_t)(n_rows * hd));
    double* kv = (double*)malloc(sizeof(double) * ORACLE_MAX_WIDTH);
    double* d = (double*)malloc(sizeof(double) * ORACLE_MAX_WIDTH);
    double* dv = (double*)malloc(sizeof(double) * (size_t)hd);
    double* dvmag = (double*)malloc(sizeof(double) * (size_t)hd);
    if (!rows || !kv || !d || !dv || !dvmag) {
        free(rows); free(kv); free(d); free(dv); free(dvmag);
        return ORACLE_E_NOMEM;
    }
    for (int64_t s = 0; s < streams; ++s) {
        const int64_t* ks = k_idx + s * W;
        const int64_t* qs = q_idx + s * R;
        for (int w = 0; w < W; ++w) {
            kv[w] = (double)round_to_bank(k_val[s * W + w], bank_bf16);
            d[w] = exp((double)g[s * G + (G == 1 ? 0 : w)]);
            for (int64_t c = 0; c < hd; ++c) rows[w * hd + c] = (double)bank_load(bank, bank_bf16, hd, ks[w], c);
        }
        const double b = (double)beta[s];
        for (int64_t c = 0; c < hd; ++c) {
            double retrieved = 0.0, mag = 0.0;
            for (int w = 0; w < W; ++w) {
                retrieved += kv[w] * d[w] * rows[w * hd + c];
                mag += fabs(kv[w] * d[w] * rows[w * hd + c]);
            }
            double vc = (double)round_to_bank(v[s * hd + c], bank_bf16);
            dv[c] = b * (vc - retrieved);
            dvmag[c] = fabs(b) * (fabs(vc) + mag);
        }
        for (int w = 0; w < W; ++w)
            for (int64_t c = 0; c < hd; ++c) {
                double x = d[w] * rows[w * hd + c] + kv[w] * dv[c];
                int64_t o = (s * W + w) * hd + c;
                if (row_exact) row_exact[o] = x;
                if (row_mag) row_mag[o] = fabs(d[w] * rows[w * hd + c]) + fabs(kv[w]) * dvmag[c];
                bank_store_f64(bank, bank_bf16, hd, ks[w], c, x);
            }
        for (int64_t c = 0; c < hd; ++c) {
            double acc = 0.0, mag = 0.0;
            for (int r = 0; r < R; ++r) {
                double qv = (double)round_to_bank(q_val[s * R + r], bank_bf16);
                double x = (double)bank_load(bank, bank_bf16, hd, qs[r], c);
                acc += qv * x;
                mag += fabs(qv * x);
            }
            if (read_exact) read_exact[s * hd + c] = acc;
            if (read_mag) read_mag[s * hd + c] = mag;
            bank_store_f64(readings, bank_bf16, hd, s, c, acc);
        }
    }
    free(rows); free(kv); free(d); free(dv); free(dvmag);
    return ORACLE_OK;
}

/* ------------------------------------------------------------- token gather */

static int token_live(int64_t t, int64_t chunk, int64_t valid, const int32_t* chunk_valid) {
    int64_t lim = chunk_valid ? (int64_t)chunk_valid[t / chunk] : valid;
    return (t % chunk) < lim;
}

/* Slots are checked for live tokens only: a padding token reads no row (its
 * outputs and stash rows are zeros), so its slots may hold anything. */
static int check_gather_args(int64_t num_slots, int64_t hd, int64_t tokens, int64_t chunk, int64_t valid,
                             const int32_t* chunk_valid, const int64_t* idx0, int width0,
                             const int64_t* idx1, int width1, int groups) {
    if (num_slots < 1 || hd < 1 || tokens < 0 || chunk < 1 || tokens % chunk != 0) return ORACLE_E_ARG;
    if (valid < 0 || valid > chunk) return ORACLE_E_ARG;
    if (width0 < 1 || width0 > ORACLE_MAX_WIDTH) return ORACLE_E_ARG;
    if (idx1 && (width1 < 1 || width1 > ORACLE_MAX_WIDTH)) return ORACLE_E_ARG;
    if (groups < 1) return ORACLE_E_ARG;
    if (chunk_valid)
        for (int64_t k = 0; k < tokens / chunk; ++k)
            if (chunk_valid[k] < 0 || chunk_valid[k] > chunk) return ORACLE_E_ARG;
    for (int64_t t = 0; t < tokens; ++t) {
        if (!token_live(t, chunk, valid, chunk_valid)) continue;
        for (int n = 0; n < width0; ++n)
            if (idx0[t * width0 + n] < 0 || idx0[t * width0 + n] >= num_slots) return ORACLE_E_SLOT;
        if (idx1)
            for (int n = 0; n < width1; ++n)
                if (idx1[t * width1 + n] < 0 || idx1[t * width1 + n] >= num_slots) return ORACLE_E_SLOT;
    }
    return ORACLE_OK;
}

/* One or two operands (idx1 == NULL: one). Weights come widened to float
 * (a bfloat16 weight widens exactly); the gather does not round them. */
int sdm_oracle_gather(const void* bank, int bank_bf16, int64_t num_slots, int64_t hd, int64_t tokens,
                      int64_t chunk, int64_t valid, const int32_t* chunk_valid, const int64_t* idx0,
                      const float* w0, int width0, float* out0, void* stash, const int64_t* idx1,
                      const float* w1, int width1, float* out1, int groups) {
    int rc = check_gather_args(num_slots, hd, tokens, chunk, valid, chunk_valid, idx0, width0, idx1, width1,
                               groups);
    if (rc != ORACLE_OK) return rc;
    const int es = bank_bf16 ? 2 : 4;
    const int max_w = (idx1 && width1 > width0) ? width1 : width0;
    float* rows = (float*)malloc(sizeof(float) * (size_t)max_w * (size_t)hd);
    if (!rows) return ORACLE_E_NOMEM;
    for (int64_t t = 0; t < tokens; ++t) {
        const int live = token_live(t, chunk, valid, chunk_valid);
        for (int o = 0; o < (idx1 ? 2 : 1); ++o) {
            const int64_t* idx = o ? idx1 : idx0;
            const float* w = o ? w1 : w0;
            float* out = o ? out1 : out0;
            const int width = o ? width1 : width0;
            if (!live) {
                for (int64_t c = 0; c < hd; ++c) out[t * hd + c] = 0.0f;
                continue;
            }
            for (int n = 0; n < width; ++n)
                for (int64_t c = 0; c < hd; ++c)
                    rows[n * hd + c] = bank_load(bank, bank_bf16, hd, idx[t * width + n], c);
            for (int64_t c = 0; c < hd; ++c) out[t * hd + c] = grouped_dot(w + t * width, rows + c, hd, width, groups);
        }
        if (stash) {
            unsigned char* dst = (unsigned char*)stash + (size_t)(t * width0 * hd * es);
            for (int n = 0; n < width0; ++n) {
                unsigned char* row = dst + (size_t)(n * hd * es);
                if (live) memcpy(row, (const unsigned char*)bank + (size_t)(idx0[t * width0 + n] * hd * es), (size_t)(hd * es));
                else memset(row, 0, (size_t)(hd * es));
            }
        }
    }
    free(rows);
    return ORACLE_OK;
}

/* The compact stash (page "sparse_delta_memory/cuda/gather_cuda.py": the
 * kernel's snapshot addressing when a position map kpos is given, and the host
 * checks of token_gather_dc). The stash holds one block of chunk * width0 rows
 * per chunk; entry n of a live token t of chunk k, with p = kpos[t, n] >= 0,
 * copies the raw row bank[idx0[t, n]] to row p of block k. Entries with a
 * negative position and every entry of a padding token copy nothing, and rows
 * that no entry names keep their contents. Two live entries of one chunk that
 * name one position must name one slot (which row would land there is not
 * defined otherwise); both that and a position past the block are ORACLE_E_POS. The
 * outputs are those of sdm_oracle_gather. */
int sdm_oracle_gather_compact_stash(const void* bank, int bank_bf16, int64_t num_slots, int64_t hd, int64_t tokens,
                                    int64_t chunk, int64_t valid, const int32_t* chunk_valid, const int64_t* idx0,
                                    int width0, const int32_t* kpos, void* stash) {
    int rc = check_gather_args(num_slots, hd, tokens, chunk, valid, chunk_valid, idx0, width0, NULL, 0, 1);
    if (rc != ORACLE_OK) return rc;
    const int es = bank_bf16 ? 2 : 4;
    const int64_t crow = chunk * width0;
    int64_t* owner = (int64_t*)malloc(sizeof(int64_t) * (size_t)crow);  /* slot stored at each position */
    if (!owner) return ORACLE_E_NOMEM;
    for (int64_t k = 0; k < tokens / chunk; ++k) {
        for (int64_t p = 0; p < crow; ++p) owner[p] = -1;
        for (int64_t t = k * chunk; t < (k + 1) * chunk; ++t) {
            if (!token_live(t, chunk, valid, chunk_valid)) continue;
            for (int n = 0; n < width0; ++n) {
                const int64_t p = kpos[t * width0 + n];
                if (p < 0) continue;
                if (p >= crow) { free(owner); return ORACLE_E_POS; }
                const int64_t slot = idx0[t * width0 + n];
                if (owner[p] >= 0 && owner[p] != slot) { free(owner); return ORACLE_E_POS; }
                owner[p] = slot;
                memcpy((unsigned char*)stash + (size_t)((k * crow + p) * hd * es),
                       (const unsigned char*)bank + (size_t)(slot * hd * es), (size_t)(hd * es));
            }
        }
    }
    free(owner);
    return ORACLE_OK;
}

/* The gather's sums in double, with sum |w row| per output (NULL to skip). */
int sdm_oracle_gather_f64(const void* bank, int bank_bf16, int64_t num_slots, int64_t hd, int64_t tokens,
                          int64_t chunk, int64_t valid, const int32_t* chunk_valid, const int64_t* idx,
                          const float* w, int width, double* out, double* mag) {
    int rc = check_gather_args(num_slots, hd, tokens, chunk, valid, chunk_valid, idx, width, NULL, 0, 1);
    if (rc != ORACLE_OK) return rc;
    for (int64_t t = 0; t < tokens; ++t) {
        const int live = token_live(t, chunk, valid, chunk_valid);
        for (int64_t c = 0; c < hd; ++c) {
            double acc = 0.0, m = 0.0;
            if (live)
                for (int n = 0; n < width; ++n) {
                    double x = (double)w[t * width + n] * (double)bank_load(bank, bank_bf16, hd, idx[t * width + n], c);
                    acc += x;
                    m += fabs(x);
                }
            out[t * hd + c] = acc;
            if (mag) mag[t * hd + c] = m;
        }
    }
    return ORACLE_OK;
}
