/*
 * Oracle for the per-layer n-gram embedding (PLE) lookup path.
 * TEST INFRASTRUCTURE ONLY (see ple_oracle.h): plain, single-threaded, slow.
 * Floating point is carried in double; the storage roundings to bfloat16 are
 * the ones the path itself stores (rows, kv, gated value, conv output).
 */
#include "ple_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

/* OCP 8-bit floating point, E4M3 "fn" flavour: sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; there
 * is no infinity, so the largest finite value is 1.75 * 2^8 = 448. */
double orc_e4m3fn_value(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits, so 8
 * significant bits for normal numbers; subnormal spacing 2^-133.  Rounds the
 * real value x to the nearest representable value, ties to even. */
uint16_t orc_bf16_from_double(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return 0x7FC0u;
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                      /* a in [2^(e-1), 2^e) */
    int qexp = e - 8;                  /* spacing of 8-significant-bit numbers */
    if (qexp < -133) qexp = -133;      /* subnormal spacing */
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);  /* default mode: nearest-even */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;                /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

double orc_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* n-gram IDs                                                                */
/* ------------------------------------------------------------------------ */

static int64_t as_signed64(uint64_t u) {
    int64_t s;
    memcpy(&s, &u, 8);
    return s;
}

static uint64_t as_unsigned64(int64_t s) {
    uint64_t u;
    memcpy(&u, &s, 8);
    return u;
}

/* The request that owns token t: qsl[r] <= t < qsl[r+1]. */
static int32_t request_of(const int32_t* qsl, int32_t num_reqs, int64_t t) {
    for (int32_t r = 0; r < num_reqs; ++r)
        if (qsl[r] <= t && t < qsl[r + 1]) return r;
    return -1;
}

int orc_ngram_ids(const int32_t* input_ids, const int32_t* qsl, int64_t num_tokens, int32_t num_reqs,
                  const int32_t* ngram_context, int32_t C, int32_t heads_per_ngram, int32_t first_head,
                  int32_t num_heads, int32_t eos, const int64_t* mult, const int64_t* vocab,
                  const int64_t* offsets, int32_t* ids, int32_t* ngram_context_out) {
    if (C < 1 || C > 7 || heads_per_ngram < 1 || num_heads < 1 || first_head < 0 ||
        first_head + num_heads > C * heads_per_ngram || num_reqs < 0 || num_tokens < 0)
        return 1;
    for (int32_t h = 0; h < num_heads; ++h)
        if (vocab[h] <= 0) return 1;
    if (num_reqs == 0 && num_tokens > 0) return 1;
    if (num_reqs > 0 && (qsl[0] != 0 || qsl[num_reqs] != num_tokens)) return 1;

    for (int64_t t = 0; t < num_tokens; ++t) {
        int32_t r = request_of(qsl, num_reqs, t);
        if (r < 0) return 1;
        int64_t a = qsl[r];

        /* the window, current token first */
        int64_t s[8];
        s[0] = input_ids[t];
        int crossed_eos = 0;
        for (int32_t j = 1; j <= C; ++j) {
            int64_t p = t - j;
            int64_t raw;
            if (p >= a)
                raw = input_ids[p];
            else if (ngram_context != NULL)
                raw = ngram_context[(int64_t)r * C + (C - (a - p))];
            else
                raw = eos;
            if (raw == eos) crossed_eos = 1;
            s[j] = crossed_eos ? eos : raw;
        }

        for (int32_t h = 0; h < num_heads; ++h) {
            int32_t order = 2 + (first_head + h) / heads_per_ngram;
            uint64_t acc = 0;  /* unsigned arithmetic wraps mod 2^64 */
            for (int32_t j = 0; j < order; ++j)
                acc += as_unsigned64(s[j]) * as_unsigned64(mult[(int64_t)h * (C + 1) + j]);
            int64_t x = as_signed64(acc);
            int64_t V = vocab[h];
            int64_t m = ((x % V) + V) % V;  /* floor modulo: result in [0, V) */
            ids[t * num_heads + h] = (int32_t)(offsets[h] + m);
        }
    }

    if (ngram_context_out != NULL) {
        for (int32_t r = 0; r < num_reqs; ++r) {
            int64_t a = qsl[r], len = qsl[r + 1] - qsl[r];
            for (int32_t i = 0; i < C; ++i) {
                int64_t q = len + i; /* index into ctx[r] ++ tok[a:b], of length C + len */
                int32_t v;
                if (q >= C)
                    v = input_ids[a + (q - C)];
                else if (ngram_context != NULL)
                    v = ngram_context[(int64_t)r * C + q];
                else
                    v = eos;
                ngram_context_out[(int64_t)r * C + i] = v;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* gathers                                                                   */
/* ------------------------------------------------------------------------ */

void orc_gather_bf16(const uint16_t* table, int32_t dim, const int32_t* ids, int64_t n, uint16_t* rows) {
    for (int64_t k = 0; k < n; ++k)
        for (int32_t c = 0; c < dim; ++c) rows[k * dim + c] = table[(int64_t)ids[k] * dim + c];
}

void orc_gather_fp8(const uint8_t* codes, const float* scales, int32_t dim, const int32_t* ids, int64_t n,
                    uint16_t* rows) {
    for (int64_t k = 0; k < n; ++k) {
        int64_t id = ids[k];
        float scale = scales[id];
        for (int32_t c = 0; c < dim; ++c) {
            float value = (float)orc_e4m3fn_value(codes[id * dim + c]); /* exact in fp32 */
            float product = value * scale;                              /* one fp32 multiply */
            rows[k * dim + c] = orc_bf16_from_double((double)product);
        }
    }
}

void orc_gather_fp8_global(const uint8_t* codes, float scale, int32_t dim, const int32_t* ids, int64_t n,
                           uint16_t* rows) {
    for (int64_t k = 0; k < n; ++k) {
        int64_t id = ids[k];
        for (int32_t c = 0; c < dim; ++c) {
            float value = (float)orc_e4m3fn_value(codes[id * dim + c]); /* exact in fp32 */
            float product = value * scale;                              /* one fp32 multiply */
            rows[k * dim + c] = orc_bf16_from_double((double)product);
        }
    }
}

double orc_e2m1_value(uint8_t code) {
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

void orc_gather_nvfp4(const uint8_t* codes, const uint8_t* block_scales, float tensor_scale, int32_t dim,
                      const int32_t* ids, int64_t n, uint16_t* rows) {
    const int64_t row_bytes = dim / 2, row_blocks = dim / 16;
    for (int64_t k = 0; k < n; ++k) {
        int64_t id = ids[k];
        for (int32_t c = 0; c < dim; ++c) {
            uint8_t byte = codes[id * row_bytes + c / 2];
            uint8_t code = (c % 2 == 0) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4);
            double block = orc_e4m3fn_value(block_scales[id * row_blocks + c / 16]);
            float scaled = (float)(orc_e2m1_value(code) * block); /* exact: 2 x 4 significant bits */
            float value = scaled * tensor_scale;                  /* one fp32 multiply */
            rows[k * dim + c] = orc_bf16_from_double((double)value);
        }
    }
}

void orc_select_rows(const uint16_t* gathered, int32_t num_shards, int64_t slot, int32_t rank, int64_t n,
                     int32_t width, uint16_t* out) {
    for (int64_t t = 0; t < n; ++t)
        for (int32_t k = 0; k < num_shards; ++k)
            for (int32_t c = 0; c < width; ++c)
                out[(t * num_shards + k) * width + c] =
                    gathered[((int64_t)k * num_shards * slot + (int64_t)rank * slot + t) * width + c];
}

/* ------------------------------------------------------------------------ */
/* merged key/value projection                                               */
/* ------------------------------------------------------------------------ */

void orc_kv_proj(const uint16_t* x, const uint16_t* w, int64_t T, int32_t K, int32_t O, uint16_t* kv) {
    /* the operands widened to double once (exact), then plain dot products */
    double* wd = (double*)malloc(sizeof(double) * (size_t)O * (size_t)K);
    double* xd = (double*)malloc(sizeof(double) * (size_t)K);
    if (wd == NULL || xd == NULL) {
        free(wd);
        free(xd);
        return;
    }
    for (int64_t i = 0; i < (int64_t)O * K; ++i) wd[i] = orc_bf16_value(w[i]);
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) xd[k] = orc_bf16_value(x[t * K + k]);
        for (int32_t o = 0; o < O; ++o) {
            const double* wr = wd + (int64_t)o * K;
            double acc = 0.0;
            for (int32_t k = 0; k < K; ++k) acc += xd[k] * wr[k];
            kv[t * O + o] = orc_bf16_from_double(acc);
        }
    }
    free(wd);
    free(xd);
}

/* ------------------------------------------------------------------------ */
/* gate                                                                      */
/* ------------------------------------------------------------------------ */

void orc_gate(const uint16_t* hidden, const uint16_t* kv, int64_t T, int32_t N, double eps, uint16_t* out,
              double* gate) {
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* h = hidden + t * N;
        const uint16_t* k = kv + t * 2 * (int64_t)N;
        const uint16_t* v = k + N;
        double hh = 0.0, kk = 0.0, hk = 0.0;
        for (int32_t c = 0; c < N; ++c) {
            double hc = orc_bf16_value(h[c]), kc = orc_bf16_value(k[c]);
            hh += hc * hc;
            kk += kc * kc;
            hk += hc * kc;
        }
        double rms_h = sqrt(hh / N + eps);
        double rms_k = sqrt(kk / N + eps);
        double s = hk / (rms_h * rms_k * sqrt((double)N));
        double g = 1.0 / (1.0 + exp(-s));
        if (gate != NULL) gate[t] = g;
        for (int32_t c = 0; c < N; ++c) out[t * N + c] = orc_bf16_from_double(g * orc_bf16_value(v[c]));
    }
}

/* ------------------------------------------------------------------------ */
/* dilated causal short convolution                                          */
/* ------------------------------------------------------------------------ */

int orc_conv(const uint16_t* x, const int32_t* qsl, int64_t T, int32_t R, const uint16_t* state,
             const uint16_t* w, int32_t N, int32_t K, int32_t d, uint16_t* y, uint16_t* state_out) {
    if (K < 1 || d < 1 || N < 1 || R < 0 || T < 0) return 1;
    if (R == 0 && T > 0) return 1;
    if (R > 0 && (qsl[0] != 0 || qsl[R] != T)) return 1;
    int64_t S = (int64_t)(K - 1) * d;

    for (int64_t t = 0; t < T; ++t) {
        int32_t r = request_of(qsl, R, t);
        if (r < 0) return 1;
        int64_t a = qsl[r];
        for (int32_t c = 0; c < N; ++c) {
            double acc = 0.0;
            for (int32_t i = 0; i < K; ++i) {
                int64_t p = t - (int64_t)i * d;
                double xv;
                if (p >= a)
                    xv = orc_bf16_value(x[p * N + c]);
                else if (state != NULL)
                    xv = orc_bf16_value(state[((int64_t)r * S + (S - (a - p))) * N + c]);
                else
                    xv = 0.0;
                acc += orc_bf16_value(w[(int64_t)c * K + (K - 1 - i)]) * xv;
            }
            y[t * N + c] = orc_bf16_from_double(acc);
        }
    }

    if (state_out != NULL && S > 0) {
        for (int32_t r = 0; r < R; ++r) {
            int64_t a = qsl[r], len = qsl[r + 1] - qsl[r];
            for (int64_t m = 0; m < S; ++m) {
                int64_t q = len + m; /* index into state[r] ++ x[a:b], of length S + len */
                for (int32_t c = 0; c < N; ++c) {
                    uint16_t v;
                    if (q >= S)
                        v = x[(a + (q - S)) * N + c];
                    else if (state != NULL)
                        v = state[((int64_t)r * S + q) * N + c];
                    else
                        v = 0; /* +0.0 */
                    state_out[((int64_t)r * S + m) * N + c] = v;
                }
            }
        }
    }
    return 0;
}
