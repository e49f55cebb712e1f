// libple C ABI: argument validation, launch configuration, error reporting.
// Every check runs before the first HIP call of an entry point, so a rejected
// call never touches a device.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "ple.h"
#include "ple_launch.h"

using namespace ple;

#ifndef PLE_FUSED_GATED_CONV
#define PLE_FUSED_GATED_CONV 1  // the fused path forms the gated value inside the conv
#endif

namespace {

thread_local char g_msg[512];

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_msg[0] = '\0';
    return PLE_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(PLE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// The current device must be gfx950 (checked once per device).
int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    static std::mutex mu;
    static signed char state[256];  // 0 unknown, 1 gfx950, -1 other
    if (dev < 0 || dev >= 256) return fail(PLE_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        if (state[dev] < 0)
            return fail(PLE_ERR_UNSUPPORTED, "device %d is %s; libple is built for gfx950 only", dev,
                        prop.gcnArchName);
    }
    if (state[dev] < 0) return fail(PLE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return PLE_OK;
}

int validate_hash(const ple_hash_desc* h, HashParams* hp) {
    if (h == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "hash descriptor is NULL");
    if (h->num_heads == 0) return fail(PLE_ERR_INVALID_ARGUMENT, "num_heads == 0 (empty head shard)");
    if (h->num_heads < 0 || h->num_heads > PLE_MAX_HEADS)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_heads %d outside 1..%d", h->num_heads, PLE_MAX_HEADS);
    if (h->context_len < 1 || h->context_len > PLE_MAX_CONTEXT)
        return fail(PLE_ERR_INVALID_ARGUMENT, "context_len %d outside 1..%d", h->context_len, PLE_MAX_CONTEXT);
    if (h->heads_per_ngram < 1) return fail(PLE_ERR_INVALID_ARGUMENT, "heads_per_ngram must be >= 1");
    if (h->first_head < 0 || (int64_t)h->first_head + h->num_heads > (int64_t)h->context_len * h->heads_per_ngram)
        return fail(PLE_ERR_INVALID_ARGUMENT, "heads [%d, %d) outside the %d heads of orders 2..%d",
                    h->first_head, h->first_head + h->num_heads, h->context_len * h->heads_per_ngram,
                    h->context_len + 1);
    if (h->multipliers == nullptr || h->vocab_sizes == nullptr || h->offsets == nullptr)
        return fail(PLE_ERR_INVALID_ARGUMENT, "multipliers, vocab_sizes and offsets must be non-NULL");
    memset(hp, 0, sizeof(*hp));
    hp->num_heads = h->num_heads;
    hp->context_len = h->context_len;
    hp->eos = h->eos_token_id;
    const int W = h->context_len + 1;
    for (int k = 0; k < h->num_heads; ++k) {
        const int64_t V = h->vocab_sizes[k], off = h->offsets[k];
        if (V < 1 || V > INT32_MAX)
            return fail(PLE_ERR_INVALID_ARGUMENT, "vocab_sizes[%d] = %lld outside 1..2^31-1", k, (long long)V);
        if (off < 0 || off + V > ((int64_t)1 << 31))
            return fail(PLE_ERR_UNSUPPORTED, "head %d rows [%lld, %lld) do not fit int32 row ids", k,
                        (long long)off, (long long)(off + V));
        HeadHash& hh = hp->head[k];
        hh.vocab = (uint32_t)V;
        hh.offset = (uint32_t)off;
        hh.barrett = UINT64_MAX / (uint64_t)V;
        hh.wrap_mod = (uint32_t)((UINT64_MAX % (uint64_t)V + 1u) % (uint64_t)V);
        hh.order = (uint32_t)(2 + (h->first_head + k) / h->heads_per_ngram);
        // shifts at or beyond the head's order contribute nothing (zero multiplier)
        for (int j = 0; j < W; ++j) {
            const uint64_t m = j < (int)hh.order ? (uint64_t)h->multipliers[(int64_t)k * W + j] : 0u;
            if (j < 4)
                hh.mult[j] = m;
            else
                hp->mult_hi[k][j - 4] = m;
        }
    }
    return PLE_OK;
}

// table elements per 16-byte chunk of a stored row
int table_elems_per_chunk(int dtype) {
    return dtype == PLE_DTYPE_BF16 ? 8 : (dtype == PLE_DTYPE_NVFP4 ? 32 : 16);
}

int validate_table(const ple_table_desc* t, int* cpr_log2) {
    if (t == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "table descriptor is NULL");
    if (t->dtype != PLE_DTYPE_BF16 && t->dtype != PLE_DTYPE_FP8_E4M3 && t->dtype != PLE_DTYPE_FP8_E4M3_GLOBAL &&
        t->dtype != PLE_DTYPE_NVFP4)
        return fail(PLE_ERR_UNSUPPORTED, "table dtype %d is not one of the PLE_DTYPE_* formats", t->dtype);
    if (t->table == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "table pointer is NULL");
    if (!aligned16(t->table)) return fail(PLE_ERR_INVALID_ARGUMENT, "table pointer is not 16-byte aligned");
    if (t->num_rows < 1 || t->num_rows > ((int64_t)1 << 31))
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_rows %lld outside 1..2^31", (long long)t->num_rows);
    if (t->dim < 1 || t->dim > 8192) return fail(PLE_ERR_INVALID_ARGUMENT, "dim %d outside 1..8192", t->dim);
    const int elem_per_chunk = table_elems_per_chunk(t->dtype);
    if (t->dim % elem_per_chunk != 0)
        return fail(PLE_ERR_UNSUPPORTED, "row of %d elements is not a multiple of 16 bytes (%d elements)", t->dim,
                    elem_per_chunk);
    if (t->dtype != PLE_DTYPE_BF16) {
        if (t->row_scales == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "a quantised table needs row_scales");
        if (!aligned4(t->row_scales)) return fail(PLE_ERR_INVALID_ARGUMENT, "row_scales is not 4-byte aligned");
    }
    if (t->dtype == PLE_DTYPE_NVFP4) {
        if (t->block_scales == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "an NVFP4 table needs block_scales");
        if (((uintptr_t)t->block_scales & 1) != 0)
            return fail(PLE_ERR_INVALID_ARGUMENT, "block_scales is not 2-byte aligned");
    }
    const int cpr = t->dim / 8;  // 16-byte output chunks per row
    *cpr_log2 = -1;
    if ((cpr & (cpr - 1)) == 0)
        for (int s = 0; s < 31; ++s)
            if ((1 << s) == cpr) *cpr_log2 = s;
    return PLE_OK;
}

int validate_heads_in_table(const ple_hash_desc* h, const ple_table_desc* t) {
    for (int k = 0; k < h->num_heads; ++k)
        if (h->offsets[k] + h->vocab_sizes[k] > t->num_rows)
            return fail(PLE_ERR_INVALID_ARGUMENT, "head %d rows [%lld, %lld) exceed the table's %lld rows", k,
                        (long long)h->offsets[k], (long long)(h->offsets[k] + h->vocab_sizes[k]),
                        (long long)t->num_rows);
    return PLE_OK;
}

// Checks of the batch fields used by the ids / lookup calls.
int validate_batch_tokens(const ple_batch_desc* b) {
    if (b == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "batch descriptor is NULL");
    if (b->num_tokens < 0 || b->num_tokens > PLE_MAX_TOKENS)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens %lld outside 0..%d", (long long)b->num_tokens,
                    PLE_MAX_TOKENS);
    if (b->num_reqs < 0) return fail(PLE_ERR_INVALID_ARGUMENT, "num_reqs < 0");
    if (b->num_reqs == 0 && b->num_tokens > 0)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens > 0 with num_reqs == 0");
    if (b->max_request_tokens < 0) return fail(PLE_ERR_INVALID_ARGUMENT, "max_request_tokens < 0");
    if (b->num_reqs > 0 && (b->query_start_loc == nullptr || !aligned4(b->query_start_loc)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "query_start_loc is NULL or misaligned");
    if (b->num_tokens > 0 && (b->input_ids == nullptr || !aligned4(b->input_ids)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "input_ids is NULL or misaligned");
    if (b->ngram_context != nullptr && !aligned4(b->ngram_context))
        return fail(PLE_ERR_INVALID_ARGUMENT, "ngram_context is misaligned");
    if (b->ngram_context_out != nullptr) {
        if (!aligned4(b->ngram_context_out)) return fail(PLE_ERR_INVALID_ARGUMENT, "ngram_context_out is misaligned");
        if ((const void*)b->ngram_context_out == (const void*)b->ngram_context)
            return fail(PLE_ERR_INVALID_ARGUMENT, "ngram_context_out must not alias ngram_context");
    }
    return PLE_OK;
}

int validate_batch_conv(const ple_batch_desc* b) {
    if (b == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "batch descriptor is NULL");
    if (b->num_tokens < 0 || b->num_tokens > PLE_MAX_TOKENS)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens %lld outside 0..%d", (long long)b->num_tokens,
                    PLE_MAX_TOKENS);
    if (b->num_reqs < 0) return fail(PLE_ERR_INVALID_ARGUMENT, "num_reqs < 0");
    if (b->num_reqs == 0 && b->num_tokens > 0)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens > 0 with num_reqs == 0");
    if (b->num_reqs > 0 && (b->query_start_loc == nullptr || !aligned4(b->query_start_loc)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "query_start_loc is NULL or misaligned");
    if (b->conv_state != nullptr && !aligned16(b->conv_state))
        return fail(PLE_ERR_INVALID_ARGUMENT, "conv_state is not 16-byte aligned");
    if (b->conv_state_out != nullptr) {
        if (!aligned16(b->conv_state_out))
            return fail(PLE_ERR_INVALID_ARGUMENT, "conv_state_out is not 16-byte aligned");
        if ((const void*)b->conv_state_out == (const void*)b->conv_state)
            return fail(PLE_ERR_INVALID_ARGUMENT, "conv_state_out must not alias conv_state");
    }
    return PLE_OK;
}

int validate_conv_shape(const uint16_t* w, int N, int K, int d) {
    if (w == nullptr || !aligned16(w)) return fail(PLE_ERR_INVALID_ARGUMENT, "conv weight is NULL or not 16-byte aligned");
    if (N < 8 || N % 8 != 0) return fail(PLE_ERR_UNSUPPORTED, "hidden size %d is not a positive multiple of 8", N);
    if (K < 1 || K > 16) return fail(PLE_ERR_INVALID_ARGUMENT, "conv kernel %d outside 1..16", K);
    if (d < 1) return fail(PLE_ERR_INVALID_ARGUMENT, "conv dilation %d < 1", d);
    if ((int64_t)(K - 1) * d > 4096) return fail(PLE_ERR_INVALID_ARGUMENT, "conv span (K-1)*d exceeds 4096");
    return PLE_OK;
}

int validate_gemm_shape(int K, int O) {
    if (K < 64 || K % 64 != 0) return fail(PLE_ERR_UNSUPPORTED, "kv_proj input width %d is not a multiple of 64", K);
    if (O < 16 || O % 16 != 0) return fail(PLE_ERR_UNSUPPORTED, "kv_proj output width %d is not a multiple of 16", O);
    if (K > (1 << 20)) return fail(PLE_ERR_UNSUPPORTED, "kv_proj input width %d exceeds 2^20", K);
    return PLE_OK;
}

int validate_gemm(const uint16_t* x, const uint16_t* w, int64_t T, int K, int O, const uint16_t* kv) {
    if (T < 0 || T > PLE_MAX_TOKENS) return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens outside 0..%d", PLE_MAX_TOKENS);
    int rc = validate_gemm_shape(K, O);
    if (rc) return rc;
    if (((T + 127) / 128) * (int64_t)((O + 127) / 128) > ((int64_t)1 << 24))
        return fail(PLE_ERR_UNSUPPORTED, "kv_proj of %lld x %d outputs exceeds 2^24 tiles", (long long)T, O);
    if (x == nullptr || w == nullptr || kv == nullptr)
        return fail(PLE_ERR_INVALID_ARGUMENT, "kv_proj pointers must be non-NULL");
    if (!aligned16(x) || !aligned16(w) || !aligned16(kv))
        return fail(PLE_ERR_INVALID_ARGUMENT, "kv_proj pointers must be 16-byte aligned");
    return PLE_OK;
}

int validate_gate(const uint16_t* hidden, const uint16_t* kv, int64_t T, int N, float eps, const uint16_t* out,
                  const float* gate) {
    if (T < 0 || T > PLE_MAX_TOKENS) return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens outside 0..%d", PLE_MAX_TOKENS);
    if (N < 8 || N % 8 != 0) return fail(PLE_ERR_UNSUPPORTED, "hidden size %d is not a positive multiple of 8", N);
    if (!(eps >= 0.0f) || eps > 1.0f) return fail(PLE_ERR_INVALID_ARGUMENT, "eps must be in [0, 1]");
    if (hidden == nullptr || kv == nullptr || out == nullptr)
        return fail(PLE_ERR_INVALID_ARGUMENT, "gate pointers must be non-NULL");
    if (!aligned16(hidden) || !aligned16(kv) || !aligned16(out))
        return fail(PLE_ERR_INVALID_ARGUMENT, "gate pointers must be 16-byte aligned");
    if (gate != nullptr && !aligned4(gate)) return fail(PLE_ERR_INVALID_ARGUMENT, "gate output is misaligned");
    return PLE_OK;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

LookupArgs lookup_args(const ple_table_desc* t, int H, int cpr_log2, const ple_batch_desc* b, const int32_t* ids_in,
                       int64_t T, int32_t* ids_out, uint16_t* rows) {
    LookupArgs g;
    memset(&g, 0, sizeof(g));
    g.tok = b ? b->input_ids : nullptr;
    g.qsl = b ? b->query_start_loc : nullptr;
    g.ctx = b ? b->ngram_context : nullptr;
    g.num_reqs = b ? b->num_reqs : 0;
    g.ids_in = ids_in;
    g.ids_out = ids_out;
    g.table = t->table;
    g.scales = t->row_scales;
    g.block_scales = t->block_scales;
    g.scale_stride = t->dtype == PLE_DTYPE_FP8_E4M3 ? 1 : 0;
    g.rows = rows;
    g.num_tokens = T;
    g.num_rows = t->num_rows;
    g.num_heads = H;
    g.dim = t->dim;
    g.tokens_per_wave = lookup_tokens_per_wave(H, t->dim / 8, t->dtype, T);
    g.cpr_log2 = cpr_log2;
    return g;
}

int run_context_out(const ple_hash_desc* h, const ple_batch_desc* b, hipStream_t s) {
    if (b->ngram_context_out == nullptr || b->num_reqs == 0) return PLE_OK;
    hipError_t e = launch_context_out(b->input_ids, b->query_start_loc, b->num_tokens, b->num_reqs, h->context_len,
                                      h->eos_token_id, b->ngram_context, b->ngram_context_out, s);
    return e == hipSuccess ? PLE_OK : hip_fail(e, "context_out launch");
}

int run_conv(const uint16_t* x, const ple_batch_desc* b, const uint16_t* w, int N, int K, int d, uint16_t* y,
             hipStream_t s) {
    if (b->num_tokens > 0) {
        hipError_t e = launch_conv(x, b->query_start_loc, b->num_tokens, b->num_reqs, b->conv_state, w, N, K, d, y, s);
        if (e != hipSuccess) return hip_fail(e, "conv launch");
    }
    const int S = (K - 1) * d;
    if (b->conv_state_out != nullptr && b->num_reqs > 0 && S > 0) {
        hipError_t e = launch_conv_state_out(x, b->query_start_loc, b->num_tokens, b->num_reqs, b->conv_state, N, S,
                                             b->conv_state_out, s);
        if (e != hipSuccess) return hip_fail(e, "conv state launch");
    }
    return PLE_OK;
}

int validate_layer(const ple_layer_desc* L, HashParams* hp, int* cpr_log2) {
    if (L == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
    int rc = validate_hash(&L->hash, hp);
    if (rc) return rc;
    rc = validate_table(&L->table, cpr_log2);
    if (rc) return rc;
    return validate_heads_in_table(&L->hash, &L->table);
}

}  // namespace

extern "C" {

const char* ple_error_message(void) { return g_msg; }

const char* ple_version(void) { return "libple 0.1.0 (gfx950)"; }

int ple_ngram_ids(const ple_hash_desc* hash, const ple_batch_desc* batch, int32_t* ids, void* stream) {
    HashParams hp;
    int rc = validate_hash(hash, &hp);
    if (rc) return rc;
    rc = validate_batch_tokens(batch);
    if (rc) return rc;
    if (batch->num_tokens > 0 && (ids == nullptr || !aligned4(ids)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "ids output is NULL or misaligned");
    if (batch->num_tokens == 0 && (batch->ngram_context_out == nullptr || batch->num_reqs == 0)) return ok();
    rc = check_device();
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (batch->num_tokens > 0) {
        hipError_t e = launch_ngram_ids(hp, batch->input_ids, batch->query_start_loc, batch->num_tokens,
                                        batch->num_reqs, batch->ngram_context, ids, s);
        if (e != hipSuccess) return hip_fail(e, "ngram_ids launch");
    }
    rc = run_context_out(hash, batch, s);
    return rc ? rc : ok();
}

int ple_gather(const ple_table_desc* table, const int32_t* ids, int64_t num_tokens, int32_t num_heads,
               uint16_t* rows, void* stream) {
    int cpr_log2 = -1;
    int rc = validate_table(table, &cpr_log2);
    if (rc) return rc;
    if (num_heads < 1 || num_heads > PLE_MAX_HEADS)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_heads %d outside 1..%d", num_heads, PLE_MAX_HEADS);
    if (num_tokens < 0 || num_tokens > PLE_MAX_TOKENS)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens outside 0..%d", PLE_MAX_TOKENS);
    if (num_tokens == 0) return ok();
    if (ids == nullptr || !aligned4(ids)) return fail(PLE_ERR_INVALID_ARGUMENT, "ids is NULL or misaligned");
    if (rows == nullptr || !aligned16(rows)) return fail(PLE_ERR_INVALID_ARGUMENT, "rows is NULL or not 16-byte aligned");
    rc = check_device();
    if (rc) return rc;
    HashParams hp;
    memset(&hp, 0, sizeof(hp));
    LookupArgs g = lookup_args(table, num_heads, cpr_log2, nullptr, ids, num_tokens, nullptr, rows);
    hipError_t e = launch_lookup(hp, g, table->dtype, kModeIds, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "gather launch");
}

int ple_lookup(const ple_hash_desc* hash, const ple_table_desc* table, const ple_batch_desc* batch,
               int32_t* ids_out, uint16_t* rows, void* stream) {
    HashParams hp;
    int cpr_log2 = -1;
    int rc = validate_hash(hash, &hp);
    if (rc) return rc;
    rc = validate_table(table, &cpr_log2);
    if (rc) return rc;
    rc = validate_heads_in_table(hash, table);
    if (rc) return rc;
    rc = validate_batch_tokens(batch);
    if (rc) return rc;
    if (batch->num_tokens > 0 && (rows == nullptr || !aligned16(rows)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "rows is NULL or not 16-byte aligned");
    if (ids_out != nullptr && !aligned4(ids_out)) return fail(PLE_ERR_INVALID_ARGUMENT, "ids_out is misaligned");
    if (batch->num_tokens == 0 && (batch->ngram_context_out == nullptr || batch->num_reqs == 0)) return ok();
    rc = check_device();
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (batch->num_tokens > 0) {
        LookupArgs g = lookup_args(table, hash->num_heads, cpr_log2, batch, nullptr, batch->num_tokens, ids_out, rows);
        hipError_t e = launch_lookup(hp, g, table->dtype, kModeHash, s);
        if (e != hipSuccess) return hip_fail(e, "lookup launch");
    }
    rc = run_context_out(hash, batch, s);
    return rc ? rc : ok();
}

int ple_prefetch(const ple_layer_desc* layer, const ple_batch_desc* batch, uint16_t* staging, void* stream) {
    if (layer == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
    return ple_lookup(&layer->hash, &layer->table, batch, nullptr, staging, stream);
}

namespace {
constexpr int64_t kDedupMaxRows = (int64_t)1 << 22;

// log2 of the hash-set capacity: a power of two >= 2 n (at least 256)
int dedup_log2cap(int64_t n) {
    int l = 8;
    while (((int64_t)1 << l) < 2 * n) ++l;
    return l;
}

// The workspace of n = T*H positions: ids, slot_of, list (distinct) and
// repeats [n], the two lists' counts, keys and rep [cap].
struct DedupWorkspace {
    int log2cap;
    size_t cap;
    int32_t* ids;
    int32_t* slot_of;
    int32_t* list;
    int32_t* repeats;
    int32_t* counts;  // [0] distinct positions, [1] repeats
    int32_t* keys;
    int32_t* rep;
};

DedupWorkspace dedup_workspace(void* workspace, int64_t n) {
    DedupWorkspace w;
    w.log2cap = dedup_log2cap(n);
    w.cap = (size_t)1 << w.log2cap;
    const size_t nb = round256((size_t)n * 4);
    char* ws = (char*)workspace;
    w.ids = (int32_t*)ws;
    w.slot_of = (int32_t*)(ws + nb);
    w.list = (int32_t*)(ws + 2 * nb);
    w.repeats = (int32_t*)(ws + 3 * nb);
    w.counts = (int32_t*)(ws + 4 * nb);
    w.keys = (int32_t*)(ws + 4 * nb + 256);
    w.rep = (int32_t*)(ws + 4 * nb + 256 + round256(w.cap * 4));
    return w;
}

// Checks shared by the plan and the fetch: the layer's hash and table, the
// row limit and the workspace (needed when T > 0).
int dedup_checks(const ple_layer_desc* layer, int64_t T, const void* workspace, size_t workspace_bytes,
                 HashParams* hp, int* cpr_log2) {
    if (layer == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
    int rc = validate_hash(&layer->hash, hp);
    if (rc) return rc;
    rc = validate_table(&layer->table, cpr_log2);
    if (rc) return rc;
    rc = validate_heads_in_table(&layer->hash, &layer->table);
    if (rc) return rc;
    if (T < 0 || T > PLE_MAX_TOKENS)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens %lld outside 0..%d", (long long)T, PLE_MAX_TOKENS);
    const int64_t n = T * layer->hash.num_heads;
    if (n > kDedupMaxRows)
        return fail(PLE_ERR_UNSUPPORTED, "dedup prefetch takes at most %lld rows (T*H = %lld)",
                    (long long)kDedupMaxRows, (long long)n);
    const size_t need = ple_prefetch_dedup_workspace_bytes(T, layer->hash.num_heads);
    if (T > 0 && (workspace == nullptr || ((uintptr_t)workspace & 255) != 0 || workspace_bytes < need))
        return fail(PLE_ERR_WORKSPACE, "dedup workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                    workspace_bytes);
    return PLE_OK;
}
}  // namespace

size_t ple_prefetch_dedup_workspace_bytes(int64_t max_tokens, int32_t num_heads) {
    if (max_tokens <= 0 || num_heads <= 0) return 0;
    const int64_t n = max_tokens * num_heads;
    if (n > kDedupMaxRows) return 0;
    const size_t cap = (size_t)1 << dedup_log2cap(n);
    // ids, slot_of, list and repeats [n], the lists' counts, keys and rep [cap]
    return 4 * round256((size_t)n * 4) + 256 + 2 * round256(cap * 4);
}

int ple_prefetch_dedup_plan(const ple_layer_desc* layer, const ple_batch_desc* batch, void* workspace,
                            size_t workspace_bytes, void* stream) {
    HashParams hp;
    int cpr_log2 = -1;
    int rc = validate_batch_tokens(batch);
    if (rc) return rc;
    rc = dedup_checks(layer, batch->num_tokens, workspace, workspace_bytes, &hp, &cpr_log2);
    if (rc) return rc;
    const int64_t T = batch->num_tokens;
    if (T == 0 && (batch->ngram_context_out == nullptr || batch->num_reqs == 0)) return ok();
    rc = check_device();
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (T > 0) {
        const int64_t n = T * layer->hash.num_heads;
        const DedupWorkspace w = dedup_workspace(workspace, n);
        // IDs, with the hash set's keys and the lists' counts cleared by the same launch
        hipError_t e = launch_ngram_ids(hp, batch->input_ids, batch->query_start_loc, T, batch->num_reqs,
                                        batch->ngram_context, w.ids, s, w.keys, (int64_t)w.cap, w.counts, 2);
        if (e == hipSuccess)
            e = launch_dedup_insert(w.ids, n, w.keys, w.rep, w.log2cap, w.slot_of, w.list, w.repeats, w.counts, s);
        if (e != hipSuccess) return hip_fail(e, "dedup plan launch");
    }
    rc = run_context_out(&layer->hash, batch, s);
    return rc ? rc : ok();
}

int ple_prefetch_dedup_fetch(const ple_layer_desc* layer, int64_t num_tokens, void* workspace,
                             size_t workspace_bytes, uint16_t* staging, int32_t* num_unique, void* stream) {
    HashParams hp;
    int cpr_log2 = -1;
    int rc = dedup_checks(layer, num_tokens, workspace, workspace_bytes, &hp, &cpr_log2);
    if (rc) return rc;
    const int64_t T = num_tokens;
    if (T > 0 && (staging == nullptr || !aligned16(staging)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "staging is NULL or not 16-byte aligned");
    if (num_unique != nullptr && !aligned4(num_unique)) return fail(PLE_ERR_INVALID_ARGUMENT, "num_unique misaligned");
    if (T == 0 && num_unique == nullptr) return ok();
    rc = check_device();
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    const ple_table_desc* table = &layer->table;
    hipError_t e;
    if (T > 0) {
        const int64_t n = T * layer->hash.num_heads;
        const DedupWorkspace w = dedup_workspace(workspace, n);
        // the distinct rows from the table: one "token" per list entry, one head
        HashParams none;
        memset(&none, 0, sizeof(none));
        LookupArgs g = lookup_args(table, 1, cpr_log2, nullptr, w.ids, n, nullptr, staging);
        g.list = w.list;
        g.list_count = w.counts;
        g.count_out = num_unique;
        e = launch_lookup(none, g, table->dtype, kModeList, s);
        if (e == hipSuccess) {
            // then each repeat from its first read: the same walk over the
            // repeats, with the staging rows as a bf16 table of n rows and
            // row rep[slot_of[i]] for position i
            ple_table_desc st;
            memset(&st, 0, sizeof(st));
            st.table = staging;
            st.num_rows = n;
            st.dim = table->dim;
            st.dtype = PLE_DTYPE_BF16;
            LookupArgs c = lookup_args(&st, 1, cpr_log2, nullptr, w.slot_of, n, nullptr, staging);
            c.list = w.repeats;
            c.list_count = w.counts + 1;
            c.rep = w.rep;
            c.rep_len = (int64_t)w.cap;
            e = launch_lookup(none, c, PLE_DTYPE_BF16, kModeList, s);
        }
    } else {
        // nothing to look up: report zero distinct rows
        e = launch_dedup_count(nullptr, num_unique, s);
    }
    return e == hipSuccess ? ok() : hip_fail(e, "dedup fetch launch");
}

int ple_prefetch_dedup(const ple_layer_desc* layer, const ple_batch_desc* batch, uint16_t* staging,
                       void* workspace, size_t workspace_bytes, int32_t* num_unique, void* stream) {
    HashParams hp;
    int cpr_log2 = -1;
    int rc = validate_batch_tokens(batch);
    if (rc) return rc;
    // every check of both calls before either launches
    rc = dedup_checks(layer, batch->num_tokens, workspace, workspace_bytes, &hp, &cpr_log2);
    if (rc) return rc;
    if (batch->num_tokens > 0 && (staging == nullptr || !aligned16(staging)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "staging is NULL or not 16-byte aligned");
    if (num_unique != nullptr && !aligned4(num_unique)) return fail(PLE_ERR_INVALID_ARGUMENT, "num_unique misaligned");
    rc = ple_prefetch_dedup_plan(layer, batch, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return ple_prefetch_dedup_fetch(layer, batch->num_tokens, workspace, workspace_bytes, staging, num_unique, stream);
}

int ple_dp_gather_slot(const int64_t* token_counts, int32_t dp_size, int32_t group_size, int32_t dp_rank,
                       int64_t* slot, int64_t* offset) {
    if (token_counts == nullptr || slot == nullptr || offset == nullptr)
        return fail(PLE_ERR_INVALID_ARGUMENT, "dp_gather_slot pointers must be non-NULL");
    if (dp_size < 1 || group_size < 1 || dp_size % group_size != 0)
        return fail(PLE_ERR_INVALID_ARGUMENT, "group size %d must divide dp size %d", group_size, dp_size);
    if (dp_rank < 0 || dp_rank >= dp_size) return fail(PLE_ERR_INVALID_ARGUMENT, "dp rank %d outside 0..%d", dp_rank, dp_size - 1);
    const int32_t g0 = dp_rank - dp_rank % group_size;
    int64_t mx = 0;
    for (int32_t r = g0; r < g0 + group_size; ++r) {
        if (token_counts[r] < 0) return fail(PLE_ERR_INVALID_ARGUMENT, "negative token count at rank %d", r);
        mx = token_counts[r] > mx ? token_counts[r] : mx;
    }
    *slot = mx;
    *offset = (int64_t)(dp_rank - g0) * mx;
    return ok();
}

int ple_head_shard(int32_t num_heads, int32_t tp_size, int32_t tp_rank, int32_t dp_size, int32_t dp_rank,
                   int32_t* first_head, int32_t* shard_heads) {
    if (first_head == nullptr || shard_heads == nullptr)
        return fail(PLE_ERR_INVALID_ARGUMENT, "head_shard outputs must be non-NULL");
    if (tp_size < 1 || dp_size < 1 || tp_rank < 0 || tp_rank >= tp_size || dp_rank < 0 || dp_rank >= dp_size)
        return fail(PLE_ERR_INVALID_ARGUMENT, "tp/dp ranks outside their sizes");
    if (num_heads < 1 || num_heads > PLE_MAX_HEADS)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_heads %d outside 1..%d", num_heads, PLE_MAX_HEADS);
    const int64_t shards = (int64_t)tp_size * dp_size;
    if (num_heads % shards != 0)
        return fail(PLE_ERR_UNSUPPORTED, "%d heads do not split evenly over %lld shards (an empty or uneven head shard)",
                    num_heads, (long long)shards);
    const int32_t per = (int32_t)(num_heads / shards);
    const int32_t s = tp_rank * dp_size + dp_rank;  // TP-major
    *first_head = s * per;
    *shard_heads = per;
    return ok();
}

int ple_select_rows(const uint16_t* gathered, int32_t num_shards, int64_t slot, int32_t rank, int64_t num_tokens,
                    int32_t width, uint16_t* out, void* stream) {
    if (num_shards < 1 || num_shards > 1024) return fail(PLE_ERR_INVALID_ARGUMENT, "num_shards %d outside 1..1024", num_shards);
    if (rank < 0 || rank >= num_shards) return fail(PLE_ERR_INVALID_ARGUMENT, "rank %d outside 0..%d", rank, num_shards - 1);
    if (slot < 0 || num_tokens < 0 || num_tokens > slot)
        return fail(PLE_ERR_INVALID_ARGUMENT, "num_tokens %lld must lie in 0..slot %lld", (long long)num_tokens,
                    (long long)slot);
    if (width < 8 || width % 8 != 0) return fail(PLE_ERR_UNSUPPORTED, "width %d is not a positive multiple of 8", width);
    if ((int64_t)num_shards * slot > PLE_MAX_TOKENS * (int64_t)64)
        return fail(PLE_ERR_INVALID_ARGUMENT, "gathered buffer of %lld rows per shard is too large",
                    (long long)((int64_t)num_shards * slot));
    if (num_tokens == 0) return ok();
    if (gathered == nullptr || out == nullptr || !aligned16(gathered) || !aligned16(out))
        return fail(PLE_ERR_INVALID_ARGUMENT, "gathered and out must be non-NULL and 16-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_select_rows(gathered, num_shards, slot, rank, num_tokens, width, out, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "select_rows launch");
}

int ple_kv_proj(const uint16_t* x, const uint16_t* w, int64_t num_tokens, int32_t k_dim, int32_t out_dim,
                uint16_t* kv, void* stream) {
    int rc = validate_gemm(x, w, num_tokens, k_dim, out_dim, kv);
    if (rc) return rc;
    if (num_tokens == 0) return ok();
    rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_kv_proj(x, w, num_tokens, k_dim, out_dim, kv, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "kv_proj launch");
}

int ple_gate(const uint16_t* hidden, const uint16_t* kv, int64_t num_tokens, int32_t n, float eps, uint16_t* out,
             float* gate, void* stream) {
    int rc = validate_gate(hidden, kv, num_tokens, n, eps, out, gate);
    if (rc) return rc;
    if (num_tokens == 0) return ok();
    rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_gate(hidden, kv, num_tokens, n, eps, out, gate, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "gate launch");
}

int ple_conv(const uint16_t* x, const ple_batch_desc* batch, const uint16_t* w, int32_t n, int32_t kernel,
             int32_t dilation, uint16_t* y, void* stream) {
    int rc = validate_batch_conv(batch);
    if (rc) return rc;
    rc = validate_conv_shape(w, n, kernel, dilation);
    if (rc) return rc;
    if (batch->num_tokens > 0) {
        if (x == nullptr || y == nullptr || !aligned16(x) || !aligned16(y))
            return fail(PLE_ERR_INVALID_ARGUMENT, "conv x and y must be non-NULL and 16-byte aligned");
        if (x == y) return fail(PLE_ERR_INVALID_ARGUMENT, "conv output must not alias its input");
    }
    const bool state_work = batch->conv_state_out != nullptr && batch->num_reqs > 0 && kernel > 1;
    if (batch->num_tokens == 0 && !state_work) return ok();
    rc = check_device();
    if (rc) return rc;
    rc = run_conv(x, batch, w, n, kernel, dilation, y, (hipStream_t)stream);
    return rc ? rc : ok();
}

int ple_spec_commit(const ple_hash_desc* hash, const ple_batch_desc* batch, const int32_t* accepted,
                    const uint16_t* x, int32_t n, int32_t conv_kernel, int32_t conv_dilation, void* stream) {
    if (batch == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "batch descriptor is NULL");
    const bool ctx_work = batch->ngram_context_out != nullptr;
    const bool conv_work = batch->conv_state_out != nullptr;
    int rc = validate_batch_conv(batch);
    if (rc) return rc;
    if (ctx_work) {
        HashParams hp;
        rc = validate_hash(hash, &hp);
        if (rc) return rc;
        rc = validate_batch_tokens(batch);
        if (rc) return rc;
    }
    int S = 0;
    if (conv_work) {
        if (n < 8 || n % 8 != 0) return fail(PLE_ERR_UNSUPPORTED, "hidden size %d is not a positive multiple of 8", n);
        if (conv_kernel < 1 || conv_kernel > 16)
            return fail(PLE_ERR_INVALID_ARGUMENT, "conv kernel %d outside 1..16", conv_kernel);
        if (conv_dilation < 1) return fail(PLE_ERR_INVALID_ARGUMENT, "conv dilation %d < 1", conv_dilation);
        if ((int64_t)(conv_kernel - 1) * conv_dilation > 4096)
            return fail(PLE_ERR_INVALID_ARGUMENT, "conv span (K-1)*d exceeds 4096");
        S = (conv_kernel - 1) * conv_dilation;
        if (batch->num_tokens > 0 && (x == nullptr || !aligned16(x)))
            return fail(PLE_ERR_INVALID_ARGUMENT, "conv input x is NULL or not 16-byte aligned");
    }
    if (batch->num_reqs > 0 && (accepted == nullptr || !aligned4(accepted)))
        return fail(PLE_ERR_INVALID_ARGUMENT, "accepted is NULL or misaligned");
    const bool do_ctx = ctx_work && batch->num_reqs > 0 && hash->context_len > 0;
    const bool do_conv = conv_work && batch->num_reqs > 0 && S > 0;
    if (!do_ctx && !do_conv) return ok();
    rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_spec_commit(batch->input_ids, x, batch->query_start_loc, batch->num_tokens,
                                      batch->num_reqs, accepted, batch->conv_state, n, S,
                                      do_conv ? batch->conv_state_out : nullptr, batch->ngram_context,
                                      do_ctx ? hash->context_len : 0, do_ctx ? hash->eos_token_id : 0,
                                      do_ctx ? batch->ngram_context_out : nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "spec commit launch");
    return ok();
}

size_t ple_prefill_workspace_bytes(const ple_layer_desc* layer, int64_t max_tokens) {
    if (layer == nullptr || max_tokens <= 0) return 0;
    const size_t T = (size_t)max_tokens;
    const size_t HD = (size_t)layer->hash.num_heads * (size_t)layer->table.dim;
    const size_t N = (size_t)layer->hidden;
    return round256(T * HD * 2) + round256(T * 2 * N * 2) + round256(T * N * 2) + round256(T * 4);
}

}  // extern "C"

namespace {

// Checks of a fused prefill call apart from its workspace.
int prefill_checks(const ple_layer_desc* layer, const ple_batch_desc* batch, const uint16_t* hidden,
                   const uint16_t* prefetched_rows, const uint16_t* out, const float* gate, HashParams* hp,
                   int* cpr_log2) {
    int rc = validate_layer(layer, hp, cpr_log2);
    if (rc) return rc;
    rc = validate_batch_tokens(batch);
    if (rc) return rc;
    rc = validate_batch_conv(batch);
    if (rc) return rc;
    const int N = layer->hidden;
    const int HD = layer->hash.num_heads * layer->table.dim;
    rc = validate_conv_shape(layer->conv_weight, N, layer->conv_kernel, layer->conv_dilation);
    if (rc) return rc;
    const int64_t T = batch->num_tokens;
    rc = validate_gemm_shape(HD, 2 * N);
    if (rc) return rc;
    if (!(layer->eps >= 0.0f) || layer->eps > 1.0f) return fail(PLE_ERR_INVALID_ARGUMENT, "eps must be in [0, 1]");
    if (T > 0) {
        if (layer->kv_weight == nullptr || !aligned16(layer->kv_weight))
            return fail(PLE_ERR_INVALID_ARGUMENT, "kv_weight is NULL or not 16-byte aligned");
        if (prefetched_rows != nullptr && !aligned16(prefetched_rows))
            return fail(PLE_ERR_INVALID_ARGUMENT, "prefetched_rows is not 16-byte aligned");
        if (hidden == nullptr || out == nullptr || !aligned16(hidden) || !aligned16(out))
            return fail(PLE_ERR_INVALID_ARGUMENT, "hidden and out must be non-NULL and 16-byte aligned");
        if (gate != nullptr && !aligned4(gate)) return fail(PLE_ERR_INVALID_ARGUMENT, "gate output is misaligned");
    }
    return PLE_OK;
}

// Whether a checked fused prefill call has any work (T == 0 still carries
// the state and context).
bool prefill_has_work(const ple_layer_desc* layer, const ple_batch_desc* batch, const uint16_t* prefetched_rows) {
    const bool state_work = batch->conv_state_out != nullptr && batch->num_reqs > 0 && layer->conv_kernel > 1;
    const bool ctx_work = prefetched_rows == nullptr && batch->ngram_context_out != nullptr && batch->num_reqs > 0;
    return batch->num_tokens > 0 || state_work || ctx_work;
}

// The launches of a checked fused prefill call, with its intermediates in ws.
int prefill_run(const ple_layer_desc* layer, const ple_batch_desc* batch, const HashParams& hp, int cpr_log2,
                const uint16_t* hidden, const uint16_t* prefetched_rows, uint16_t* out, float* gate, char* ws,
                hipStream_t s) {
    const int N = layer->hidden;
    const int HD = layer->hash.num_heads * layer->table.dim;
    const int64_t T = batch->num_tokens;
    const bool state_work = batch->conv_state_out != nullptr && batch->num_reqs > 0 && layer->conv_kernel > 1;
    const bool ctx_work = prefetched_rows == nullptr && batch->ngram_context_out != nullptr && batch->num_reqs > 0;
    uint16_t* rows = (uint16_t*)ws;
    uint16_t* kv = (uint16_t*)(ws + round256((size_t)T * HD * 2));
    uint16_t* gated = (uint16_t*)((char*)kv + round256((size_t)T * 2 * N * 2));
    hipError_t e;
    if (T > 0) {
        const uint16_t* x = prefetched_rows;
        if (x == nullptr) {
            LookupArgs g = lookup_args(&layer->table, layer->hash.num_heads, cpr_log2, batch, nullptr, T, nullptr, rows);
            e = launch_lookup(hp, g, layer->table.dtype, kModeHash, s);
            if (e != hipSuccess) return hip_fail(e, "lookup launch");
            x = rows;
        }
        e = launch_kv_proj(x, layer->kv_weight, T, HD, 2 * N, kv, s);
        if (e != hipSuccess) return hip_fail(e, "kv_proj launch");
    }
    // decode batches and verify windows (at most 4 tokens per request): gate,
    // conv and the carried state and context in one launch
    if (decode_tail_supported(batch->max_request_tokens, layer->conv_kernel, N)) {
        DecodeTailArgs a;
        a.hidden = hidden;
        a.kv = kv;
        a.qsl = batch->query_start_loc;
        a.tok = batch->input_ids;
        a.T = T;
        a.R = batch->num_reqs;
        a.N = N;
        a.eps = layer->eps;
        a.d = layer->conv_dilation;
        a.conv_w = layer->conv_weight;
        a.state = batch->conv_state;
        a.state_out = state_work ? batch->conv_state_out : nullptr;
        a.ctx = batch->ngram_context;
        a.ctx_out = ctx_work ? batch->ngram_context_out : nullptr;
        a.C = ctx_work ? layer->hash.context_len : 0;
        a.eos = layer->hash.eos_token_id;
        a.gated = gated;
        a.y = out;
        a.gate = gate;
        e = launch_decode_tail(a, layer->conv_kernel, s);
        if (e != hipSuccess) return hip_fail(e, "decode tail launch");
        return PLE_OK;
    }
    if (T > 0 && PLE_FUSED_GATED_CONV && conv_rows_supported(layer->conv_kernel, N)) {
        // the gate alone, then the conv on the value half of kv, gated as it
        // is read: the gated value makes no round trip through memory; only
        // the conv inputs the carried state or a verify commit may take are
        // written to the workspace
        float* g = (float*)((char*)gated + round256((size_t)T * N * 2));
        e = launch_gate_only(hidden, kv, T, N, layer->eps, g, gate, s);
        if (e != hipSuccess) return hip_fail(e, "gate launch");
        ConvRowsArgs ca = {};
        ca.x = kv + N;
        ca.x_stride = 2 * (int64_t)N;
        ca.g = g;
        ca.qsl = batch->query_start_loc;
        ca.T = T;
        ca.R = batch->num_reqs;
        ca.state = batch->conv_state;
        ca.w = layer->conv_weight;
        ca.N = N;
        ca.d = layer->conv_dilation;
        ca.y = out;
        ca.gated_out = gated;
        e = launch_conv_gated(ca, layer->conv_kernel, s);
        if (e != hipSuccess) return hip_fail(e, "conv launch");
    } else if (T > 0) {
        e = launch_gate(hidden, kv, T, N, layer->eps, gated, gate, s);
        if (e != hipSuccess) return hip_fail(e, "gate launch");
        e = launch_conv(gated, batch->query_start_loc, T, batch->num_reqs, batch->conv_state, layer->conv_weight, N,
                        layer->conv_kernel, layer->conv_dilation, out, s);
        if (e != hipSuccess) return hip_fail(e, "conv launch");
    }
    // the carried context and conv state in one launch (the commit kernel
    // over every request's whole window)
    if (ctx_work || state_work) {
        const int S = (layer->conv_kernel - 1) * layer->conv_dilation;
        e = launch_spec_commit(batch->input_ids, gated, batch->query_start_loc, T, batch->num_reqs, nullptr,
                               batch->conv_state, N, S, state_work ? batch->conv_state_out : nullptr,
                               batch->ngram_context, ctx_work ? layer->hash.context_len : 0,
                               layer->hash.eos_token_id, ctx_work ? batch->ngram_context_out : nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "state launch");
    }
    return PLE_OK;
}

}  // namespace

extern "C" {

int ple_prefill_fused(const ple_layer_desc* layer, const ple_batch_desc* batch, const uint16_t* hidden,
                      const uint16_t* prefetched_rows, uint16_t* out, float* gate, void* workspace,
                      size_t workspace_bytes, void* stream) {
    HashParams hp;
    int cpr_log2 = -1;
    int rc = prefill_checks(layer, batch, hidden, prefetched_rows, out, gate, &hp, &cpr_log2);
    if (rc) return rc;
    const int64_t T = batch->num_tokens;
    if (T > 0) {
        if (workspace == nullptr) return fail(PLE_ERR_WORKSPACE, "workspace is NULL");
        const size_t need = ple_prefill_workspace_bytes(layer, T);
        if (workspace_bytes < need)
            return fail(PLE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                        workspace_bytes, need);
        if (((uintptr_t)workspace & 255u) != 0)
            return fail(PLE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    }
    if (!prefill_has_work(layer, batch, prefetched_rows)) return ok();
    rc = check_device();
    if (rc) return rc;
    rc = prefill_run(layer, batch, hp, cpr_log2, hidden, prefetched_rows, out, gate, (char*)workspace,
                     (hipStream_t)stream);
    return rc ? rc : ok();
}

int ple_prefill_fused_noalloc(const ple_layer_desc* layer, const ple_batch_desc* batch, const uint16_t* hidden,
                              const uint16_t* prefetched_rows, uint16_t* out, float* gate, void* stream) {
    HashParams hp;
    int cpr_log2 = -1;
    int rc = prefill_checks(layer, batch, hidden, prefetched_rows, out, gate, &hp, &cpr_log2);
    if (rc) return rc;
    const size_t need = ple_prefill_workspace_bytes(layer, batch->num_tokens);
    if (need > (size_t)PLE_NOALLOC_SCRATCH_BYTES)
        return fail(PLE_ERR_WORKSPACE,
                    "ple_prefill_fused_noalloc: %lld tokens need %zu bytes of intermediates, more than the "
                    "library's %zu-byte scratch array (use ple_prefill_fused with a workspace)",
                    (long long)batch->num_tokens, need, (size_t)PLE_NOALLOC_SCRATCH_BYTES);
    if (!prefill_has_work(layer, batch, prefetched_rows)) return ok();
    rc = check_device();
    if (rc) return rc;
    void* scratch = nullptr;
    hipError_t e = noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
    rc = prefill_run(layer, batch, hp, cpr_log2, hidden, prefetched_rows, out, gate, (char*)scratch,
                     (hipStream_t)stream);
    return rc ? rc : ok();
}

int ple_host_alloc(size_t bytes, void** host, void** device) {
    if (bytes == 0 || host == nullptr || device == nullptr)
        return fail(PLE_ERR_INVALID_ARGUMENT, "ple_host_alloc needs bytes > 0 and non-NULL outputs");
    *host = nullptr;
    *device = nullptr;
    void* h = nullptr;
    hipError_t e = hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocPortable);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, h, 0);
    if (e != hipSuccess) {
        (void)hipHostFree(h);
        return hip_fail(e, "hipHostGetDevicePointer");
    }
    *host = h;
    *device = d;
    return ok();
}

int ple_host_free(void* host) {
    if (host == nullptr) return ok();
    hipError_t e = hipHostFree(host);
    return e == hipSuccess ? ok() : hip_fail(e, "hipHostFree");
}

int ple_stream_create_cu_masked(int32_t num_cus, void** stream) {
    if (stream == nullptr) return fail(PLE_ERR_INVALID_ARGUMENT, "stream output is NULL");
    if (num_cus < 1) return fail(PLE_ERR_INVALID_ARGUMENT, "num_cus must be >= 1");
    int rc = check_device();
    if (rc) return rc;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    if (num_cus > cus) num_cus = cus;
    uint32_t mask[16] = {0};
    const int words = (cus + 31) / 32 > 16 ? 16 : (cus + 31) / 32;
    for (int c = 0; c < num_cus && c < 32 * words; ++c) mask[c >> 5] |= 1u << (c & 31);
    hipStream_t s = nullptr;
    e = hipExtStreamCreateWithCUMask(&s, (uint32_t)words, mask);
    if (e != hipSuccess) return hip_fail(e, "hipExtStreamCreateWithCUMask");
    *stream = (void*)s;
    return ok();
}

int ple_stream_destroy(void* stream) {
    if (stream == nullptr) return ok();
    hipError_t e = hipStreamDestroy((hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hipStreamDestroy");
}

}  // extern "C"
