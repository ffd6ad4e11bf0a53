// kvq_api.hip -- the extern "C" boundary of libkvq.so (declared in include/kvq.h).
// Every argument is checked on the host before the first HIP call, so a rejected
// call launches nothing and writes nothing.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kvq_internal.h"

namespace {

using namespace kvq;

const uint16_t h_levels[510] = {KVQ_LEVELS_FP16_LIST};
const float h_thresholds[510] = {KVQ_THRESHOLDS_LIST};
const float h_gain_dd[8] = {KVQ_GAIN_DD_LIST};

bool debug_on() {
    static const bool on = getenv("KVQ_DEBUG") != nullptr;
    return on;
}

int32_t fail(int32_t st, const char* fn, const char* why) {
    if (debug_on()) fprintf(stderr, "kvq: %s rejected: %s (%s)\n", fn, why, kvq_status_string(st));
    return st;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// head_dim rule: exact128 for quantize/attention, any even 2..128 for energy/allocation
int32_t check_geom(const kvq_geom* g, bool exact128, const char* fn) {
    if (!g) return fail(KVQ_ERR_ARG, fn, "null geometry");
    if (g->layout_version != KVQ_LAYOUT_VERSION) return fail(KVQ_ERR_VERSION, fn, "layout_version");
    const int d = g->head_dim;
    if (exact128 ? d != kHeadDim : (d < 2 || d > kHeadDim || (d & 1))) return fail(KVQ_ERR_SHAPE, fn, "head_dim");
    if (g->n_kv_heads < 1 || g->n_kv_heads > 65535) return fail(KVQ_ERR_SHAPE, fn, "n_kv_heads");
    if (g->rope_pairing != KVQ_PAIR_HALF && g->rope_pairing != KVQ_PAIR_INTERLEAVED)
        return fail(KVQ_ERR_ARG, fn, "rope_pairing");
    const int nb = d / 2;
    if (!((g->k_budget >= 0 && g->k_budget <= 8 * nb) || g->k_budget == 16 * nb))
        return fail(KVQ_ERR_BUDGET, fn, "k_budget");
    if (!((g->v_bits >= 1 && g->v_bits <= 8) || g->v_bits == 16)) return fail(KVQ_ERR_BUDGET, fn, "v_bits");
    if (g->capacity_tokens < 0 || g->capacity_tokens % kTile) return fail(KVQ_ERR_CAPACITY, fn, "capacity_tokens");
    return KVQ_OK;
}

int32_t hip_status(hipError_t e, const char* fn) {
    if (e == hipSuccess) return KVQ_OK;
    if (debug_on()) fprintf(stderr, "kvq: %s: HIP error %s\n", fn, hipGetErrorString(e));
    return KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t kvq_version(void) { return KVQ_LAYOUT_VERSION; }

const char* kvq_status_string(int32_t status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_ARG: return "invalid argument";
        case KVQ_ERR_SHAPE: return "unsupported shape";
        case KVQ_ERR_BUDGET: return "invalid bit budget";
        case KVQ_ERR_ALIGN: return "misaligned pointer or stride";
        case KVQ_ERR_CAPACITY: return "capacity exceeded or not a multiple of 64";
        case KVQ_ERR_WORKSPACE: return "workspace too small";
        case KVQ_ERR_HIP: return "HIP launch failed";
        case KVQ_ERR_VERSION: return "unsupported layout version";
        default: return "unknown status";
    }
}

int64_t kvq_tile_bytes(const kvq_geom* g) {
    const int32_t st = check_geom(g, true, "kvq_tile_bytes");
    if (st) return st;
    return tile_bytes(g->head_dim, g->k_budget, g->v_bits);
}

int64_t kvq_cache_bytes(const kvq_geom* g) {
    const int32_t st = check_geom(g, true, "kvq_cache_bytes");
    if (st) return st;
    return (int64_t)g->n_kv_heads * (g->capacity_tokens / kTile) * tile_bytes(g->head_dim, g->k_budget, g->v_bits);
}

int32_t kvq_get_codebook(int32_t w, uint16_t* levels_fp16, float* thresholds, float* gain_dd) {
    if (w < 1 || w > 8) return fail(KVQ_ERR_ARG, "kvq_get_codebook", "width");
    const int off = KVQ_CB_OFF(w), n = 1 << w;
    if (levels_fp16) memcpy(levels_fp16, h_levels + off, sizeof(uint16_t) * n);
    if (thresholds) memcpy(thresholds, h_thresholds + off, sizeof(float) * n);
    if (gain_dd) memcpy(gain_dd, h_gain_dd, sizeof(float) * 8);
    return KVQ_OK;
}

int32_t kvq_block_energy(const kvq_geom* g, const void* x, int64_t n_tok, int64_t stride_tok, int64_t stride_head,
                         uint64_t* energy, void* stream) {
    const char* fn = "kvq_block_energy";
    int32_t st = check_geom(g, false, fn);
    if (st) return st;
    if (n_tok < 0) return fail(KVQ_ERR_ARG, fn, "n_tok < 0");
    if (!energy || (n_tok > 0 && !x)) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (stride_tok < 0 || stride_head < 0) return fail(KVQ_ERR_ARG, fn, "negative stride");
    if (!aligned(x, 4) || (stride_tok & 1) || (stride_head & 1) || !aligned(energy, 16))
        return fail(KVQ_ERR_ALIGN, fn, "x 4-byte / strides even / energy 16-byte");
    if (n_tok == 0) return KVQ_OK;
    return hip_status(launch_block_energy((const uint16_t*)x, n_tok, stride_tok, stride_head, g->n_kv_heads,
                                          g->head_dim, g->rope_pairing, energy, (hipStream_t)stream),
                      fn);
}

int32_t kvq_allocate_bits(const kvq_geom* g, const uint64_t* energy, int32_t n_units, int32_t budget, int32_t mode,
                          uint8_t* bits, float* sigma, void* stream) {
    const char* fn = "kvq_allocate_bits";
    int32_t st = check_geom(g, false, fn);
    if (st) return st;
    const int nb = g->head_dim / 2;
    if (n_units < 0) return fail(KVQ_ERR_ARG, fn, "n_units < 0");
    if (mode != KVQ_GREEDY && mode != KVQ_UNIFORM) return fail(KVQ_ERR_ARG, fn, "mode");
    if (!((budget >= 0 && budget <= 8 * nb) || budget == 16 * nb)) return fail(KVQ_ERR_BUDGET, fn, "budget");
    if (mode == KVQ_UNIFORM && budget != 16 * nb && budget % nb) return fail(KVQ_ERR_BUDGET, fn, "uniform budget");
    if (n_units > 0 && (!energy || !bits || !sigma)) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(energy, 16) || !aligned(sigma, 4)) return fail(KVQ_ERR_ALIGN, fn, "energy 16-byte / sigma 4-byte");
    if (n_units == 0) return KVQ_OK;
    return hip_status(launch_allocate(energy, n_units, nb, budget, mode, bits, sigma, (hipStream_t)stream), fn);
}

int32_t kvq_quantize_pack(const kvq_geom* g, const void* k, const void* v, int64_t stride_tok, int64_t stride_head,
                          int32_t n_seq, const int64_t* first_slot, const int32_t* n_new, const int64_t* src_row0,
                          int32_t max_new, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                          uint8_t* cache, const int64_t* seq_byte_off, void* stream) {
    const char* fn = "kvq_quantize_pack";
    int32_t st = check_geom(g, true, fn);
    if (st) return st;
    if (n_seq < 0 || max_new < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if (n_seq > 65535) return fail(KVQ_ERR_SHAPE, fn, "n_seq");
    if (max_new > g->capacity_tokens) return fail(KVQ_ERR_CAPACITY, fn, "max_new > capacity");
    if (stride_tok < 0 || stride_head < 0) return fail(KVQ_ERR_ARG, fn, "negative stride");
    if (n_seq == 0 || max_new == 0) return KVQ_OK;
    if (!k || !v || !first_slot || !n_new || !src_row0 || !k_bits || !k_sigma || !v_sigma || !cache || !seq_byte_off)
        return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(k, 4) || !aligned(v, 4) || (stride_tok & 1) || (stride_head & 1) || !aligned(cache, 16) ||
        !aligned(first_slot, 8) || !aligned(src_row0, 8) || !aligned(seq_byte_off, 8) || !aligned(n_new, 4) ||
        !aligned(k_sigma, 4) || !aligned(v_sigma, 4))
        return fail(KVQ_ERR_ALIGN, fn, "alignment");
    return hip_status(launch_quantize_pack(*g, (const uint16_t*)k, (const uint16_t*)v, stride_tok, stride_head, n_seq,
                                           first_slot, n_new, src_row0, max_new, k_bits, k_sigma, v_sigma, cache,
                                           seq_byte_off, (hipStream_t)stream),
                      fn);
}

int64_t kvq_decode_workspace_bytes_ex(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, int64_t max_len,
                                      int32_t kernel, int32_t tiles_per_split) {
    const char* fn = "kvq_decode_workspace_bytes";
    int32_t st = check_geom(g, true, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0 || max_len < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if (max_len > g->capacity_tokens) return fail(KVQ_ERR_CAPACITY, fn, "max_len > capacity");
    DecodePlan plan;
    st = plan_decode(*g, n_q_heads, n_seq, max_len, kernel, tiles_per_split, &plan);
    if (st) return fail(st, fn, "no kernel for this geometry");
    return plan.workspace;
}

int64_t kvq_decode_workspace_bytes(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, int64_t max_len) {
    return kvq_decode_workspace_bytes_ex(g, n_q_heads, n_seq, max_len, KVQ_DECODE_AUTO, 0);
}

namespace {
// shared validation of the decode calls; fills the plan
int32_t check_decode(const kvq_geom* g, int32_t n_q_heads, const void* q, const uint8_t* cache,
                     const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq, int64_t max_len,
                     const uint8_t* k_bits, const float* k_sigma, const float* v_sigma, const void* ws,
                     size_t ws_bytes, int32_t kernel, int32_t tiles_per_split, DecodePlan* plan, const char* fn,
                     bool ws_owned_by_library = false) {
    int32_t st = check_geom(g, true, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0 || max_len < 0 || tiles_per_split < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if ((int64_t)n_seq * n_q_heads > 2147483647LL) return fail(KVQ_ERR_SHAPE, fn, "n_seq * n_q_heads");
    if (n_seq > 65535) return fail(KVQ_ERR_SHAPE, fn, "n_seq");
    if (max_len > g->capacity_tokens) return fail(KVQ_ERR_CAPACITY, fn, "max_len > capacity");
    st = plan_decode(*g, n_q_heads, n_seq, max_len, kernel, tiles_per_split, plan);
    if (st) return fail(st, fn, "no kernel for this geometry");
    if (n_seq == 0) return KVQ_OK;
    if (!q || !cache || !seq_byte_off || !seq_len || !k_bits || !k_sigma || !v_sigma || (!ws && !ws_owned_by_library))
        return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(ws, 16) || !aligned(seq_byte_off, 8) ||
        !aligned(seq_len, 4) || !aligned(k_sigma, 4) || !aligned(v_sigma, 4))
        return fail(KVQ_ERR_ALIGN, fn, "alignment");
    if ((int64_t)ws_bytes < plan->workspace) return fail(KVQ_ERR_WORKSPACE, fn, "workspace/partials bytes");
    return KVQ_OK;
}
}  // namespace

int32_t kvq_decode_plan(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, int64_t max_len, int32_t kernel,
                        int32_t tiles_per_split, int32_t* kernel_out, int32_t* tiles_out, int32_t* n_split_out,
                        int64_t* workspace_out) {
    const char* fn = "kvq_decode_plan";
    int32_t st = check_geom(g, true, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0 || max_len < 0 || tiles_per_split < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if (max_len > g->capacity_tokens) return fail(KVQ_ERR_CAPACITY, fn, "max_len > capacity");
    DecodePlan plan;
    st = plan_decode(*g, n_q_heads, n_seq, max_len, kernel, tiles_per_split, &plan);
    if (st) return fail(st, fn, "no kernel for this geometry");
    if (kernel_out) *kernel_out = plan.kernel;
    if (tiles_out) *tiles_out = plan.tiles_per_split;
    if (n_split_out) *n_split_out = plan.n_split;
    if (workspace_out) *workspace_out = plan.workspace;
    return KVQ_OK;
}

int32_t kvq_decode_n_split(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, int64_t max_len, int32_t kernel,
                           int32_t tiles_per_split) {
    const char* fn = "kvq_decode_n_split";
    int32_t st = check_geom(g, true, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0 || max_len < 0 || tiles_per_split < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if (max_len > g->capacity_tokens) return fail(KVQ_ERR_CAPACITY, fn, "max_len > capacity");
    DecodePlan plan;
    st = plan_decode(*g, n_q_heads, n_seq, max_len, kernel, tiles_per_split, &plan);
    if (st) return fail(st, fn, "no kernel for this geometry");
    return plan.n_split;
}

int32_t kvq_decode_partials(const kvq_geom* g, int32_t n_q_heads, const void* q, const uint8_t* cache,
                            const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq, int64_t max_len,
                            const uint8_t* k_bits, const float* k_sigma, const float* v_sigma, float softmax_scale,
                            float* partials, size_t partials_bytes, int32_t kernel, int32_t tiles_per_split,
                            void* stream) {
    const char* fn = "kvq_decode_partials";
    DecodePlan plan;
    int32_t st = check_decode(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma,
                              partials, partials_bytes, kernel, tiles_per_split, &plan, fn);
    if (st || n_seq == 0) return st;
    return hip_status(launch_decode_partials(*g, plan, n_q_heads, (const uint16_t*)q, (uint8_t*)cache, seq_byte_off,
                                             seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma, softmax_scale,
                                             partials, (hipStream_t)stream),
                      fn);
}

int32_t kvq_merge_partials(int32_t n_seq, int32_t n_q_heads, int32_t n_split, const float* partials, float* out,
                           void* stream) {
    const char* fn = "kvq_merge_partials";
    if (n_seq < 0 || n_q_heads < 0 || n_split < 1) return fail(KVQ_ERR_ARG, fn, "counts");
    if ((int64_t)n_seq * n_q_heads > 2147483647LL) return fail(KVQ_ERR_SHAPE, fn, "n_seq * n_q_heads");
    if (n_seq == 0 || n_q_heads == 0) return KVQ_OK;
    if (!partials || !out) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(partials, 16) || !aligned(out, 16)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    return hip_status(launch_merge(n_seq * n_q_heads, n_split, partials, out, (hipStream_t)stream), fn);
}

int32_t kvq_packed_decode_attn_ex(const kvq_geom* g, int32_t n_q_heads, const void* q, const uint8_t* cache,
                                  const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq, int64_t max_len,
                                  const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                                  float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                                  int32_t kernel, int32_t tiles_per_split, void* stream) {
    const char* fn = "kvq_packed_decode_attn";
    DecodePlan plan;
    int32_t st = check_decode(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma,
                              workspace, workspace_bytes, kernel, tiles_per_split, &plan, fn);
    if (st || n_seq == 0) return st;
    if (!out) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(out, 16)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    hipError_t e = launch_decode_partials(*g, plan, n_q_heads, (const uint16_t*)q, (uint8_t*)cache, seq_byte_off,
                                          seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma, softmax_scale,
                                          (float*)workspace, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(launch_merge(n_seq * n_q_heads, plan.n_split, (const float*)workspace, out, (hipStream_t)stream),
                      fn);
}

int32_t kvq_packed_decode_attn(const kvq_geom* g, int32_t n_q_heads, const void* q, const uint8_t* cache,
                               const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq, int64_t max_len,
                               const uint8_t* k_bits, const float* k_sigma, const float* v_sigma, float softmax_scale,
                               float* out, void* workspace, size_t workspace_bytes, void* stream) {
    return kvq_packed_decode_attn_ex(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma,
                                     v_sigma, softmax_scale, out, workspace, workspace_bytes, KVQ_DECODE_AUTO, 0,
                                     stream);
}

// ---------------------------------------------------------------- allocation-free decode
// The split partials of kvq_packed_decode_attn_noalloc live in a library-owned device
// array (one per GPU, alive until the process ends) instead of a caller workspace.
// The array's name is a host-side stand-in: its device address is looked up once per
// device with hipGetSymbolAddress, and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// the current device's copy of `scratch` (looked up on the device's first call)
int32_t scratch_address(void** out, const char* fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_ARG, fn, "device ordinal beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, fn);
        if (ptr == nullptr || !aligned(ptr, 256)) return fail(KVQ_ERR_HIP, fn, "scratch symbol address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}
}  // namespace

int32_t kvq_packed_decode_attn_noalloc(const kvq_geom* g, int32_t n_q_heads, const void* q, const uint8_t* cache,
                                       const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq,
                                       int64_t max_len, const uint8_t* k_bits, const float* k_sigma,
                                       const float* v_sigma, float softmax_scale, float* out, void* stream) {
    const char* fn = "kvq_packed_decode_attn_noalloc";
    DecodePlan plan;
    int32_t st = check_decode(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma,
                              nullptr, (size_t)KVQ_NOALLOC_SCRATCH_BYTES, KVQ_DECODE_AUTO, 0, &plan, fn, true);
    if (st == KVQ_ERR_WORKSPACE)
        return fail(st, fn, "the plan's partials exceed KVQ_NOALLOC_SCRATCH_BYTES; use kvq_packed_decode_attn");
    if (st || n_seq == 0) return st;
    if (!out) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(out, 16)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    void* ws = nullptr;
    st = scratch_address(&ws, fn);
    if (st) return st;
    hipError_t e = launch_decode_partials(*g, plan, n_q_heads, (const uint16_t*)q, (uint8_t*)cache, seq_byte_off,
                                          seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma, softmax_scale,
                                          (float*)ws, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(launch_merge(n_seq * n_q_heads, plan.n_split, (const float*)ws, out, (hipStream_t)stream), fn);
}

namespace {
int32_t check_step_rows(const void* k_new, const void* v_new, int64_t stride_seq, int64_t stride_head, const char* fn) {
    if (!k_new || !v_new) return fail(KVQ_ERR_ARG, fn, "null new-token pointer");
    if (stride_seq < 0 || stride_head < 0) return fail(KVQ_ERR_ARG, fn, "negative stride");
    if (!aligned(k_new, 4) || !aligned(v_new, 4) || (stride_seq & 1) || (stride_head & 1))
        return fail(KVQ_ERR_ALIGN, fn, "new-token alignment");
    return KVQ_OK;
}
}  // namespace

int32_t kvq_decode_step_partials(const kvq_geom* g, int32_t n_q_heads, const void* q, const void* k_new,
                                 const void* v_new, int64_t new_stride_seq, int64_t new_stride_head, uint8_t* cache,
                                 const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq, int64_t max_len,
                                 const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                                 float softmax_scale, float* partials, size_t partials_bytes, int32_t kernel,
                                 int32_t tiles_per_split, void* stream) {
    const char* fn = "kvq_decode_step_partials";
    DecodePlan plan;
    int32_t st = check_decode(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma,
                              partials, partials_bytes, kernel, tiles_per_split, &plan, fn);
    if (st || n_seq == 0) return st;
    st = check_step_rows(k_new, v_new, new_stride_seq, new_stride_head, fn);
    if (st) return st;
    const AppendArgs app{(const uint16_t*)k_new, (const uint16_t*)v_new, new_stride_seq, new_stride_head};
    return hip_status(launch_decode_partials(*g, plan, n_q_heads, (const uint16_t*)q, cache, seq_byte_off, seq_len,
                                             n_seq, max_len, k_bits, k_sigma, v_sigma, softmax_scale, partials,
                                             (hipStream_t)stream, app),
                      fn);
}

int32_t kvq_decode_step(const kvq_geom* g, int32_t n_q_heads, const void* q, const void* k_new, const void* v_new,
                        int64_t new_stride_seq, int64_t new_stride_head, uint8_t* cache, const int64_t* seq_byte_off,
                        const int32_t* seq_len, int32_t n_seq, int64_t max_len, const uint8_t* k_bits,
                        const float* k_sigma, const float* v_sigma, float softmax_scale, float* out, void* workspace,
                        size_t workspace_bytes, int32_t kernel, int32_t tiles_per_split, void* stream) {
    const char* fn = "kvq_decode_step";
    DecodePlan plan;
    int32_t st = check_decode(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma,
                              workspace, workspace_bytes, kernel, tiles_per_split, &plan, fn);
    if (st || n_seq == 0) return st;
    st = check_step_rows(k_new, v_new, new_stride_seq, new_stride_head, fn);
    if (st) return st;
    if (!out) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(out, 16)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    const AppendArgs app{(const uint16_t*)k_new, (const uint16_t*)v_new, new_stride_seq, new_stride_head};
    hipError_t e = launch_decode_partials(*g, plan, n_q_heads, (const uint16_t*)q, cache, seq_byte_off, seq_len,
                                          n_seq, max_len, k_bits, k_sigma, v_sigma, softmax_scale, (float*)workspace,
                                          (hipStream_t)stream, app);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(launch_merge(n_seq * n_q_heads, plan.n_split, (const float*)workspace, out, (hipStream_t)stream),
                      fn);
}

namespace {
constexpr int kWindowLimit = 1024;  // window tokens per (sequence, KV head): one merge thread each

int32_t check_window(const kvq_geom* g, int32_t window, const void* win_k, const void* win_v, int64_t max_len,
                     const char* fn) {
    if (window < 1 || window > kWindowLimit) return fail(KVQ_ERR_ARG, fn, "window outside 1..1024");
    if (!win_k || !win_v) return fail(KVQ_ERR_ARG, fn, "null window pointer");
    if (!aligned(win_k, 16) || !aligned(win_v, 16)) return fail(KVQ_ERR_ALIGN, fn, "window alignment");
    if (max_len < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    (void)g;
    return KVQ_OK;
}

int32_t window_decode(const kvq_geom* g, int32_t window, int32_t n_q_heads, const void* q, const void* k_new,
                      const void* v_new, int64_t new_stride_seq, int64_t new_stride_head, void* win_k, void* win_v,
                      uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq,
                      int64_t max_len, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                      float softmax_scale, float* out, void* workspace, size_t workspace_bytes, int32_t kernel,
                      int32_t tiles_per_split, void* stream, const char* fn) {
    int32_t st = check_window(g, window, win_k, win_v, max_len, fn);
    if (st) return st;
    const int64_t packed_max = max_len > window ? max_len - window : 0;
    DecodePlan plan;
    st = check_decode(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, packed_max, k_bits, k_sigma, v_sigma,
                      workspace, (size_t)INT64_MAX, kernel, tiles_per_split, &plan, fn);
    if (st || n_seq == 0) return st;
    const int n_chunks = plan.n_split + window_chunks(window);  // the packed chunks and the window's
    if (n_chunks > 65535) return fail(KVQ_ERR_CAPACITY, fn, "chunks");
    const int64_t ws_need = plan_workspace(plan, n_chunks);
    if ((int64_t)workspace_bytes < ws_need) return fail(KVQ_ERR_WORKSPACE, fn, "workspace bytes");
    if (k_new) {
        if (!v_new) return fail(KVQ_ERR_ARG, fn, "null new-token pointer");
        if (new_stride_seq < 0 || new_stride_head < 0) return fail(KVQ_ERR_ARG, fn, "negative stride");
        if (!aligned(k_new, 16) || !aligned(v_new, 16) || (new_stride_seq & 7) || (new_stride_head & 7))
            return fail(KVQ_ERR_ALIGN, fn, "new-token rows must be 16-byte aligned");
    }
    if (!out) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(out, 16)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    // one launch: the packed chunks (the token leaving the window packed by the tail
    // tile's wave, which then writes the new token to its ring row) and the window chunk
    AppendArgs app{};
    app.k = k_new ? (const uint16_t*)win_k : nullptr;
    app.v = k_new ? (const uint16_t*)win_v : nullptr;
    app.stride_seq = (int64_t)g->n_kv_heads * window * kHeadDim;
    app.stride_head = (int64_t)window * kHeadDim;
    app.window = window;
    app.ring_k = (uint16_t*)win_k;
    app.ring_v = (uint16_t*)win_v;
    app.k_new = (const uint16_t*)k_new;
    app.v_new = (const uint16_t*)v_new;
    app.new_stride_seq = new_stride_seq;
    app.new_stride_head = new_stride_head;
    hipError_t e = launch_decode_partials(*g, plan, n_q_heads, (const uint16_t*)q, cache, seq_byte_off, seq_len,
                                          n_seq, packed_max, k_bits, k_sigma, v_sigma, softmax_scale,
                                          (float*)workspace, (hipStream_t)stream, app);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(launch_merge(n_seq * n_q_heads, n_chunks, (const float*)workspace, out,
                                   (hipStream_t)stream),
                      fn);
}
}  // namespace

int64_t kvq_window_workspace_bytes(const kvq_geom* g, int32_t window, int32_t n_q_heads, int32_t n_seq,
                                   int64_t max_len, int32_t kernel, int32_t tiles_per_split) {
    const char* fn = "kvq_window_workspace_bytes";
    if (window < 1 || window > kWindowLimit) return fail(KVQ_ERR_ARG, fn, "window outside 1..1024");
    if (max_len < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    const int64_t packed_max = max_len > window ? max_len - window : 0;
    const int64_t ws = kvq_decode_workspace_bytes_ex(g, n_q_heads, n_seq, packed_max, kernel, tiles_per_split);
    if (ws < 0) return ws;
    DecodePlan plan;
    if (plan_decode(*g, n_q_heads, n_seq, packed_max, kernel, tiles_per_split, &plan))
        return fail(KVQ_ERR_SHAPE, fn, "no kernel for this geometry");
    return plan_workspace(plan, plan.n_split + window_chunks(window));
}

int32_t kvq_window_decode_attn(const kvq_geom* g, int32_t window, int32_t n_q_heads, const void* q,
                               const void* win_k, const void* win_v, const uint8_t* cache,
                               const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq, int64_t max_len,
                               const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                               float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                               int32_t kernel, int32_t tiles_per_split, void* stream) {
    return window_decode(g, window, n_q_heads, q, nullptr, nullptr, 0, 0, (void*)win_k, (void*)win_v,
                         (uint8_t*)cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma,
                         softmax_scale, out, workspace, workspace_bytes, kernel, tiles_per_split, stream,
                         "kvq_window_decode_attn");
}

int32_t kvq_window_decode_step(const kvq_geom* g, int32_t window, int32_t n_q_heads, const void* q,
                               const void* k_new, const void* v_new, int64_t new_stride_seq,
                               int64_t new_stride_head, void* win_k, void* win_v, uint8_t* cache,
                               const int64_t* seq_byte_off, const int32_t* seq_len, int32_t n_seq, int64_t max_len,
                               const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                               float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                               int32_t kernel, int32_t tiles_per_split, void* stream) {
    if (!k_new) return fail(KVQ_ERR_ARG, "kvq_window_decode_step", "null new-token pointer");
    return window_decode(g, window, n_q_heads, q, k_new, v_new, new_stride_seq, new_stride_head, win_k, win_v, cache,
                         seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma, softmax_scale, out,
                         workspace, workspace_bytes, kernel, tiles_per_split, stream, "kvq_window_decode_step");
}


// ---------------------------------------------------------------- chunked prefill
namespace {
int32_t check_prefill_shape(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, int32_t max_q, int64_t max_len,
                            int32_t n_split, PrefillPlan* plan, const char* fn) {
    int32_t st = check_geom(g, true, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0 || max_q < 0 || max_len < 0 || n_split < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if (n_seq > 65535) return fail(KVQ_ERR_SHAPE, fn, "n_seq");
    if ((int64_t)n_seq * max_q * n_q_heads > 2147483647LL) return fail(KVQ_ERR_SHAPE, fn, "n_seq * max_q * n_q_heads");
    if (max_len > g->capacity_tokens) return fail(KVQ_ERR_CAPACITY, fn, "max_len > capacity");
    st = plan_prefill(*g, n_q_heads, n_seq, max_q, max_len, n_split, plan);
    if (st) return fail(st, fn, "geometry not served by the prefill kernel (K16, V16 or group > 128)");
    if ((int64_t)plan->n_qb * g->n_kv_heads > 2147483647LL) return fail(KVQ_ERR_SHAPE, fn, "grid");
    return KVQ_OK;
}
}  // namespace

int32_t kvq_prefill_plan(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, int32_t max_q, int64_t max_len,
                         int32_t n_split, int32_t* n_split_out, int64_t* workspace_out) {
    PrefillPlan plan;
    const int32_t st = check_prefill_shape(g, n_q_heads, n_seq, max_q, max_len, n_split, &plan, "kvq_prefill_plan");
    if (st) return st;
    if (n_split_out) *n_split_out = plan.n_split;
    if (workspace_out) *workspace_out = plan.workspace;
    return KVQ_OK;
}

int64_t kvq_prefill_workspace_bytes(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, int32_t max_q,
                                    int64_t max_len, int32_t n_split) {
    PrefillPlan plan;
    const int32_t st =
        check_prefill_shape(g, n_q_heads, n_seq, max_q, max_len, n_split, &plan, "kvq_prefill_workspace_bytes");
    return st ? st : plan.workspace;
}

int32_t kvq_packed_prefill_attn(const kvq_geom* g, int32_t n_q_heads, const void* q, const uint8_t* cache,
                                const int64_t* seq_byte_off, const int32_t* q_start, const int32_t* n_q,
                                int32_t n_seq, int32_t max_q, int64_t max_len, const uint8_t* k_bits,
                                const float* k_sigma, const float* v_sigma, float softmax_scale, float* out,
                                void* workspace, size_t workspace_bytes, int32_t n_split, void* stream) {
    const char* fn = "kvq_packed_prefill_attn";
    PrefillPlan plan;
    int32_t st = check_prefill_shape(g, n_q_heads, n_seq, max_q, max_len, n_split, &plan, fn);
    if (st) return st;
    if (n_seq == 0 || max_q == 0) return KVQ_OK;
    if (!q || !cache || !seq_byte_off || !q_start || !n_q || !k_bits || !k_sigma || !v_sigma || !out)
        return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (plan.workspace > 0 && !workspace) return fail(KVQ_ERR_ARG, fn, "null workspace");
    if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16) || !aligned(workspace, 16) ||
        !aligned(seq_byte_off, 8) || !aligned(q_start, 4) || !aligned(n_q, 4) || !aligned(k_sigma, 4) ||
        !aligned(v_sigma, 4))
        return fail(KVQ_ERR_ALIGN, fn, "alignment");
    if ((int64_t)workspace_bytes < plan.workspace) return fail(KVQ_ERR_WORKSPACE, fn, "workspace bytes");
    return hip_status(launch_prefill(*g, plan, n_q_heads, (const uint16_t*)q, cache, seq_byte_off, q_start, n_q, n_seq,
                                     max_q, max_len, k_bits, k_sigma, v_sigma, softmax_scale, out, (float*)workspace,
                                     (hipStream_t)stream),
                      fn);
}

// ---------------------------------------------------------------- rotation variant
namespace {
int32_t check_rot_geom(const kvq_geom* g, const char* fn) {
    int32_t st = check_geom(g, true, fn);
    if (st) return st;
    if (g->k_budget % kMaxBlocks || g->k_budget < kMaxBlocks || g->k_budget > 8 * kMaxBlocks)
        return fail(KVQ_ERR_BUDGET, fn, "rotated keys need a uniform width 1..8 (k_budget a multiple of 64)");
    if (g->v_bits > 8) return fail(KVQ_ERR_BUDGET, fn, "v_bits 1..8");
    return KVQ_OK;
}
}  // namespace

int32_t kvq_rot_quantize_pack(const kvq_geom* g, const void* k, const void* v, int64_t stride_tok,
                              int64_t stride_head, int32_t n_seq, const int64_t* first_slot, const int32_t* n_new,
                              const int64_t* src_row0, int32_t max_new, const uint8_t* k_signs,
                              const uint8_t* v_signs, const float* v_sigma, uint8_t* cache,
                              const int64_t* seq_byte_off, void* stream) {
    const char* fn = "kvq_rot_quantize_pack";
    int32_t st = check_rot_geom(g, fn);
    if (st) return st;
    if (n_seq < 0 || max_new < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if (n_seq > 65535) return fail(KVQ_ERR_SHAPE, fn, "n_seq");
    if (max_new > g->capacity_tokens) return fail(KVQ_ERR_CAPACITY, fn, "max_new > capacity");
    if (stride_tok < 0 || stride_head < 0) return fail(KVQ_ERR_ARG, fn, "negative stride");
    if (n_seq == 0 || max_new == 0) return KVQ_OK;
    if (!k || !v || !first_slot || !n_new || !src_row0 || !k_signs || (!v_signs && !v_sigma) || !cache ||
        !seq_byte_off)
        return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(k, 4) || !aligned(v, 4) || (stride_tok & 1) || (stride_head & 1) || !aligned(cache, 16) ||
        !aligned(first_slot, 8) || !aligned(src_row0, 8) || !aligned(seq_byte_off, 8) || !aligned(n_new, 4) ||
        !aligned(v_sigma, 4))
        return fail(KVQ_ERR_ALIGN, fn, "alignment");
    return hip_status(launch_rot_quantize(*g, (const uint16_t*)k, (const uint16_t*)v, stride_tok, stride_head, n_seq,
                                          first_slot, n_new, src_row0, max_new, k_signs, v_signs, v_sigma, cache,
                                          seq_byte_off, (hipStream_t)stream),
                      fn);
}

int32_t kvq_rot_queries(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, const void* q, void* q_rot,
                        const uint8_t* k_signs, void* stream) {
    const char* fn = "kvq_rot_queries";
    int32_t st = check_rot_geom(g, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if ((int64_t)n_seq * n_q_heads > 2147483647LL) return fail(KVQ_ERR_SHAPE, fn, "n_seq * n_q_heads");
    if (n_seq == 0) return KVQ_OK;
    if (!q || !q_rot || !k_signs) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(q, 4) || !aligned(q_rot, 4)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    return hip_status(launch_rot_queries((const uint16_t*)q, (uint16_t*)q_rot, k_signs, n_seq * n_q_heads, n_q_heads,
                                         n_q_heads / g->n_kv_heads, (hipStream_t)stream),
                      fn);
}

int32_t kvq_rot_back(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, float* out, const uint8_t* v_signs,
                     void* stream) {
    const char* fn = "kvq_rot_back";
    int32_t st = check_rot_geom(g, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if ((int64_t)n_seq * n_q_heads > 2147483647LL) return fail(KVQ_ERR_SHAPE, fn, "n_seq * n_q_heads");
    if (n_seq == 0) return KVQ_OK;
    if (!out || !v_signs) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(out, 8)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    return hip_status(launch_rot_back(out, v_signs, n_seq * n_q_heads, n_q_heads, n_q_heads / g->n_kv_heads,
                                      (hipStream_t)stream),
                      fn);
}

extern "C++" namespace kvq {
// kvq_rotate.hip (C++ linkage inside this extern "C" block)
hipError_t launch_rot_step(const kvq_geom& g, int n_q_heads, int n_seq, const uint16_t* q, uint16_t* qr,
                           const uint16_t* k_new, const uint16_t* v_new, int64_t stride_seq, int64_t stride_head,
                           uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                           const uint8_t* k_signs, const uint8_t* v_signs, const float* v_sigma, hipStream_t st);
}  // namespace kvq

int32_t kvq_rot_decode_prepare(const kvq_geom* g, int32_t n_q_heads, int32_t n_seq, const void* q, void* q_rot,
                               const void* k_new, const void* v_new, int64_t new_stride_seq, int64_t new_stride_head,
                               uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                               const uint8_t* k_signs, const uint8_t* v_signs, const float* v_sigma, void* stream) {
    const char* fn = "kvq_rot_decode_prepare";
    int32_t st = check_rot_geom(g, fn);
    if (st) return st;
    if (n_q_heads < 1 || n_q_heads % g->n_kv_heads) return fail(KVQ_ERR_SHAPE, fn, "n_q_heads");
    if (n_seq < 0) return fail(KVQ_ERR_ARG, fn, "negative count");
    if (n_seq > 65535 || g->n_kv_heads + n_q_heads > 65535) return fail(KVQ_ERR_SHAPE, fn, "n_seq or heads");
    if (n_seq == 0) return KVQ_OK;
    if (!q || !q_rot || !k_new || !v_new || !cache || !seq_byte_off || !seq_len || !k_signs ||
        (!v_signs && !v_sigma))
        return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (new_stride_seq < 0 || new_stride_head < 0) return fail(KVQ_ERR_ARG, fn, "negative stride");
    if (!aligned(q, 4) || !aligned(q_rot, 4) || !aligned(k_new, 4) || !aligned(v_new, 4) || (new_stride_seq & 1) ||
        (new_stride_head & 1) || !aligned(cache, 16) || !aligned(seq_byte_off, 8) || !aligned(seq_len, 4) ||
        !aligned(v_sigma, 4))
        return fail(KVQ_ERR_ALIGN, fn, "alignment");
    return hip_status(launch_rot_step(*g, n_q_heads, n_seq, (const uint16_t*)q, (uint16_t*)q_rot,
                                      (const uint16_t*)k_new, (const uint16_t*)v_new, new_stride_seq, new_stride_head,
                                      cache, seq_byte_off, seq_len, k_signs, v_signs, v_sigma, (hipStream_t)stream),
                      fn);
}

int32_t kvq_rot_decode_step_partials(const kvq_geom* g, int32_t n_q_heads, const void* q, const void* k_new,
                                     const void* v_new, int64_t new_stride_seq, int64_t new_stride_head,
                                     uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                                     int32_t n_seq, int64_t max_len, const uint8_t* k_bits, const float* k_sigma,
                                     const float* v_sigma, const uint8_t* k_signs, const uint8_t* v_signs,
                                     float softmax_scale, float* partials, size_t partials_bytes,
                                     int32_t tiles_per_split, void* stream) {
    const char* fn = "kvq_rot_decode_step_partials";
    int32_t st = check_rot_geom(g, fn);
    if (st) return st;
    DecodePlan plan;
    st = check_decode(g, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits, k_sigma, v_sigma,
                      partials, partials_bytes, KVQ_DECODE_MFMA, tiles_per_split, &plan, fn);
    if (st || n_seq == 0) return st;
    st = check_step_rows(k_new, v_new, new_stride_seq, new_stride_head, fn);
    if (st) return st;
    if (!k_signs) return fail(KVQ_ERR_ARG, fn, "null pointer");
    AppendArgs app{(const uint16_t*)k_new, (const uint16_t*)v_new, new_stride_seq, new_stride_head};
    app.k_signs = k_signs;
    app.v_signs = v_signs;
    return hip_status(launch_decode_partials(*g, plan, n_q_heads, (const uint16_t*)q, cache, seq_byte_off, seq_len,
                                             n_seq, max_len, k_bits, k_sigma, v_sigma, softmax_scale, partials,
                                             (hipStream_t)stream, app),
                      fn);
}

// ---------------------------------------------------------------- measurement helper
int32_t kvq_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t n_blocks, void* stream) {
    const char* fn = "kvq_read_probe";
    if (bytes < 0 || n_blocks < 1 || n_blocks > (1 << 24)) return fail(KVQ_ERR_ARG, fn, "counts");
    if (bytes == 0) return KVQ_OK;
    if (!src || !sink) return fail(KVQ_ERR_ARG, fn, "null pointer");
    if (!aligned(src, 16) || (bytes & 15) || !aligned(sink, 4)) return fail(KVQ_ERR_ALIGN, fn, "alignment");
    return hip_status(launch_read_probe(src, bytes, sink, n_blocks, (hipStream_t)stream), fn);
}

}  // extern "C"
