/*
 * Oracle for the per-layer n-gram embedding (PLE) lookup path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, single-threaded CPU
 * statement of what the path computes, written from the defining pages.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code with the GPU library and the GPU library never
 * calls it.
 *
 * Sources (cited by page title and section):
 *   [P1] "PR #54371 [Qwen4Exp] Support UVA PLE-offload and Engram tensor
 *        parallelism" - sections 功能与动机 (motivation) and 关键源码片段
 *        (key source snippets: the pinned-host embedding and its lookup).
 *   [P3] "PR #54517 [Qwen3.8-Flash-Next] Fuse Qwen4Exp PLE kernels" -
 *        sections 实现拆解 (implementation breakdown: ids, gate, conv kernels,
 *        merged kv_proj) and 关键源码片段 (compute_ngram_ids, the ids kernel's
 *        arguments and its per-shift loop).
 *   [P4] "Support PLE-Offload for Qwen3.8-Flash-Next - #53899" - the report
 *        on FP8 PLE tables (float8_e4m3fn with a weight scale; the review
 *        thread on one global weight scale) and the walkthrough naming NVFP4
 *        embedding support.
 * Where the pages leave a step open the readings are listed per function.
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * brute force, closed forms or library routines; none is "parity unpinned".
 */
#ifndef PLE_ORACLE_H
#define PLE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * N-gram hash IDs ([P3] 实现拆解 item 2, 关键源码片段 compute_ngram_ids and the
 * ids kernel).  For token t of request r (tokens [a, b) = [qsl[r], qsl[r+1])):
 *   raw(j), 1 <= j <= C:  tok[t-j] if t-j >= a, else ngram_context[r][C-(a-(t-j))]
 *                         when a context is given, else eos.
 *   s_0 = tok[t]; s_j = eos once some raw(j'), 1 <= j' <= j, is eos, else raw(j).
 *   head h (global head g = first_head + h) has order n = 2 + g / heads_per_ngram.
 *   ids[t][h] = offsets[h] + floormod(int64(sum_{j<n} s_j * mult[h][j] mod 2^64), vocab[h]).
 * ngram_context_out[r][i] (if non-NULL) = the (C-i)-th most recent raw token of
 * ngram_context[r] ++ tok[a:b].
 * Returns 0, or 1 on an argument outside the documented ranges.
 */
int orc_ngram_ids(const int32_t* input_ids, const int32_t* qsl, int64_t num_tokens, int32_t num_reqs,
                  const int32_t* ngram_context, int32_t context_len, int32_t heads_per_ngram,
                  int32_t first_head, int32_t num_heads, int32_t eos_token_id,
                  const int64_t* multipliers, const int64_t* vocab_sizes, const int64_t* offsets,
                  int32_t* ids, int32_t* ngram_context_out);

/* rows[k][:] = table[ids[k]][:], bf16 bit copy ([P1] 关键源码片段, F.embedding). */
void orc_gather_bf16(const uint16_t* table, int32_t dim, const int32_t* ids, int64_t n, uint16_t* rows);

/* rows[k][c] = bf16(float(e4m3fn(codes[ids[k]][c])) * scales[ids[k]]) with one
 * fp32 multiply, both roundings to nearest even ([P4] FP8 PLE table). */
void orc_gather_fp8(const uint8_t* codes, const float* scales, int32_t dim, const int32_t* ids, int64_t n,
                    uint16_t* rows);

/* The same with one scale for the whole table ([P4] review thread: an FP8
 * PLE table with one global weight scale). */
void orc_gather_fp8_global(const uint8_t* codes, float scale, int32_t dim, const int32_t* ids, int64_t n,
                           uint16_t* rows);

/* OCP float8 e4m3fn value of a code (NaN for 0x7F and 0xFF). */
double orc_e4m3fn_value(uint8_t code);

/* OCP MX FP4 e2m1 value of a 4-bit code: sign bit 3, exponent bits 2..1
 * (bias 1), mantissa bit 0; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double orc_e2m1_value(uint8_t code);

/* NVFP4 rows ([P4] walkthrough names NVFP4 embedding support; the layout is
 * the plain reading of the public format, the pages print none): a row of dim
 * elements is dim/2 bytes, element c in byte c/2 (low nibble for even c); its
 * 16-element block b has the e4m3fn scale block_scales[row][b]; one fp32
 * tensor_scale for the table.
 * rows[k][c] = bf16(float(e2m1(code) * e4m3fn(block scale)) * tensor_scale):
 * the first product is exact, then one fp32 multiply, then nearest-even. */
void orc_gather_nvfp4(const uint8_t* codes, const uint8_t* block_scales, float tensor_scale, int32_t dim,
                      const int32_t* ids, int64_t n, uint16_t* rows);

/* bfloat16 nearest-even rounding of a real value; NaN -> 0x7FC0. */
uint16_t orc_bf16_from_double(double x);
double orc_bf16_value(uint16_t bits);

/* Rank-major row selection ([P1] 实现拆解 item 3, selecting a replica's token
 * window after the gather; [P2] 实现拆解 item 4, the rank-major select-rows
 * kernel): out[t][k*width + c] = gathered[k][rank*slot + t][c] for t < n,
 * gathered [E][E*slot][width], out [n][E*width]; a bit copy. */
void orc_select_rows(const uint16_t* gathered, int32_t num_shards, int64_t slot, int32_t rank, int64_t n,
                     int32_t width, uint16_t* out);

/* kv[t][o] = bf16(sum_k x[t][k] * w[o][k]) with the sum in double ([P3] merged kv_proj). */
void orc_kv_proj(const uint16_t* x, const uint16_t* w, int64_t num_tokens, int32_t k_dim, int32_t out_dim,
                 uint16_t* kv);

/*
 * Gate ([P3] 实现拆解 item 2, "PLE gating and normalisation"), per token t with
 * h = hidden[t], k = kv[t][0:N], v = kv[t][N:2N]:
 *   s = <h, k> / (sqrt(mean(h^2) + eps) * sqrt(mean(k^2) + eps) * sqrt(N))
 *   g = 1 / (1 + exp(-s));  out[t] = bf16(g * v);  gate[t] = g (if non-NULL).
 */
void orc_gate(const uint16_t* hidden, const uint16_t* kv, int64_t num_tokens, int32_t n, double eps,
              uint16_t* out, double* gate);

/*
 * Dilated causal depthwise short convolution ([P3] 实现拆解 item 2):
 *   y[t][c] = bf16(sum_{i<K} w[c][K-1-i] * xt(t - i*d, c)),
 *   xt(p, c) = x[p][c] for p >= a (start of t's request), else
 *              state[r][S-(a-p)][c] if a state is given, else 0;  S = (K-1)*d.
 * state_out[r][m] (if non-NULL) = the (S-m)-th most recent input of state[r] ++ x[a:b].
 */
int orc_conv(const uint16_t* x, const int32_t* qsl, int64_t num_tokens, int32_t num_reqs,
             const uint16_t* state, const uint16_t* w, int32_t n, int32_t kernel, int32_t dilation,
             uint16_t* y, uint16_t* state_out);

#ifdef __cplusplus
}
#endif

#endif
