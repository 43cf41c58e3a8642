// C ABI of libekv (declared in include/ekv.h).  Validates every argument on
// the host before enqueuing anything, sizes workspaces, and dispatches to the
// kernel launchers.  Holds no state besides the thread-local error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/ekv.h"
#include "ekv_internal.h"

namespace {

thread_local char g_err[512] = "";

ekv_status fail(ekv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ekv_status fail(ekv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

ekv_status ok() {
    g_err[0] = '\0';
    return EKV_OK;
}

ekv_status hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ok();
    return fail(EKV_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

ekv_status check_shape(const ekv_shape* s, ekv::Dims* d) {
    if (!s) return fail(EKV_ERR_INVALID_ARG, "shape is NULL");
    if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_groups < 1 || s->head_dim < 1 ||
        s->page_size < 1 || s->max_pages_per_seq < 1 || s->num_phys_pages < 1)
        return fail(EKV_ERR_INVALID_ARG, "shape fields must be positive");
    if (s->num_q_heads % s->num_kv_groups != 0)
        return fail(EKV_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_groups (%d)",
                    s->num_q_heads, s->num_kv_groups);
    const int r = s->num_q_heads / s->num_kv_groups;
    if (r != 1 && r != 2 && r != 4 && r != 8)
        return fail(EKV_ERR_UNSUPPORTED, "heads per group r=%d not in {1,2,4,8}", r);
    if (s->num_kv_groups > 16) return fail(EKV_ERR_UNSUPPORTED, "num_kv_groups=%d > 16", s->num_kv_groups);
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(EKV_ERR_UNSUPPORTED, "head_dim=%d not in {64,128}", s->head_dim);
    if (s->page_size != 16) return fail(EKV_ERR_UNSUPPORTED, "page_size=%d (only 16 is built)", s->page_size);
    if (s->kv_dtype != EKV_F32 && s->kv_dtype != EKV_BF16)
        return fail(EKV_ERR_UNSUPPORTED, "kv_dtype=%d", s->kv_dtype);
    if (s->stat_dtype != EKV_F32 && s->stat_dtype != EKV_BF16 && s->stat_dtype != EKV_FP8_E4M3)
        return fail(EKV_ERR_UNSUPPORTED, "stat_dtype=%d", s->stat_dtype);
    if ((long long)s->max_pages_per_seq * 16 > 0x7fffffffLL)
        return fail(EKV_ERR_UNSUPPORTED, "max_pages_per_seq=%d too large", s->max_pages_per_seq);
    if ((long long)s->batch * s->num_kv_groups > 65535)
        return fail(EKV_ERR_UNSUPPORTED, "batch*num_kv_groups > 65535");
    d->B = s->batch;
    d->HQ = s->num_q_heads;
    d->G = s->num_kv_groups;
    d->R = r;
    d->D = s->head_dim;
    d->MP = s->max_pages_per_seq;
    d->NP = s->num_phys_pages;
    d->kv_bf16 = s->kv_dtype == EKV_BF16;
    d->stat = s->stat_dtype == EKV_BF16 ? ekv::kStatBF16 : (s->stat_dtype == EKV_FP8_E4M3 ? ekv::kStatFP8 : ekv::kStatF32);
    return EKV_OK;
}

bool gauss_alpha_ok(float alpha) {
    return fabsf(alpha - 1.5f) < 1e-6f || fabsf(alpha - 2.0f) < 1e-6f || fabsf(alpha - 4.0f / 3.0f) < 1e-6f;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Argument checks shared by ekv_entmax_decode and ekv_entmax_decode_noalloc
// that do not involve the workspace; fills the workspace plan.
ekv_status check_decode(const ekv_shape* shape, int sparse, int32_t sel_stride, const int32_t* sel_count,
                        float alpha, const float* tau_ref, const float* delta, const int32_t* support_ref,
                        ekv::Dims* d, ekv::DecodePlan* pl) {
    ekv_status st = check_shape(shape, d);
    if (st != EKV_OK) return st;
    if (!(alpha >= 1.0f) || !(alpha < 1e6f)) return fail(EKV_ERR_INVALID_ARG, "alpha must be >= 1 (got %g)", alpha);
    if (sparse && sel_stride < 1) return fail(EKV_ERR_INVALID_ARG, "sel_stride=%d < 1", sel_stride);
    if (sparse && !sel_count) return fail(EKV_ERR_INVALID_ARG, "sel_count is required with sel_pages");
    if (delta && !tau_ref) return fail(EKV_ERR_INVALID_ARG, "delta needs tau_ref");
    if (support_ref && !tau_ref) return fail(EKV_ERR_INVALID_ARG, "support_ref needs tau_ref");
    *pl = ekv::plan_decode(*d, sparse, sparse ? sel_stride : 0, alpha);
    if (pl->too_long)
        return fail(EKV_ERR_UNSUPPORTED, "rows of %d pages are longer than the decode is built for",
                    sparse ? sel_stride : d->MP);
    return EKV_OK;
}

// Scratch memory of ekv_entmax_decode_noalloc: one copy of this array per GPU
// the library runs on, held until the process ends.  Host code never uses
// the array's name as an address (on the host it names a stand-in, not
// device memory): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept in g_scratch.
constexpr size_t kNoallocScratchBytes = (size_t)EKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call per device; concurrent first calls store the same address).
hipError_t scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

int32_t ekv_abi_version(void) { return EKV_ABI_VERSION; }

const char* ekv_last_error(void) { return g_err; }

ekv_status ekv_build_page_stats(const ekv_shape* shape, const void* k_cache, const int32_t* page_table,
                                const int32_t* seq_lens, const int32_t* page_list, int32_t n_list,
                                void* kmin, void* kmax, void* kmean, void* kvar, void* stream) {
    ekv::Dims d;
    ekv_status st = check_shape(shape, &d);
    if (st != EKV_OK) return st;
    if (!k_cache || !page_table || !seq_lens) return fail(EKV_ERR_INVALID_ARG, "k_cache, page_table and seq_lens are required");
    if ((kmin == nullptr) != (kmax == nullptr)) return fail(EKV_ERR_INVALID_ARG, "kmin and kmax must both be given or both NULL");
    if ((kmean == nullptr) != (kvar == nullptr)) return fail(EKV_ERR_INVALID_ARG, "kmean and kvar must both be given or both NULL");
    if (!kmin && !kmean) return fail(EKV_ERR_INVALID_ARG, "no statistic requested");
    if (page_list && n_list < 0) return fail(EKV_ERR_INVALID_ARG, "n_list < 0");
    if ((long long)d.B * d.MP > 0x7fffffffLL) return fail(EKV_ERR_UNSUPPORTED, "batch*max_pages too large");
    return hip_status(ekv::launch_page_stats(d, k_cache, page_table, seq_lens, page_list, n_list, kmin, kmax,
                                             kmean, kvar, (hipStream_t)stream),
                      "ekv_build_page_stats");
}

ekv_status ekv_append_kv(const ekv_shape* shape, const void* k_new, const void* v_new,
                         const int32_t* page_table, const int32_t* seq_lens, void* k_cache, void* v_cache,
                         void* kmin, void* kmax, void* kmean, void* kvar, int32_t* new_lens, void* stream) {
    ekv::Dims d;
    ekv_status st = check_shape(shape, &d);
    if (st != EKV_OK) return st;
    if (!k_new || !v_new || !page_table || !seq_lens || !k_cache || !v_cache)
        return fail(EKV_ERR_INVALID_ARG, "k_new, v_new, page_table, seq_lens, k_cache and v_cache are required");
    if ((kmin == nullptr) != (kmax == nullptr)) return fail(EKV_ERR_INVALID_ARG, "kmin and kmax must both be given or both NULL");
    if ((kmean == nullptr) != (kvar == nullptr)) return fail(EKV_ERR_INVALID_ARG, "kmean and kvar must both be given or both NULL");
    if (new_lens && (const void*)new_lens == (const void*)seq_lens)
        return fail(EKV_ERR_INVALID_ARG, "new_lens must not alias seq_lens");
    if ((long long)d.B * d.MP > 0x7fffffffLL) return fail(EKV_ERR_UNSUPPORTED, "batch*max_pages too large");
    return hip_status(ekv::launch_append_kv(d, k_new, v_new, page_table, seq_lens, k_cache, v_cache, kmin, kmax,
                                            kmean, kvar, new_lens, (hipStream_t)stream),
                      "ekv_append_kv");
}

ekv_status ekv_score_pages(const ekv_shape* shape, int32_t selector, const void* q, const int32_t* page_table,
                           const int32_t* seq_lens, const void* kmin, const void* kmax, const void* kmean,
                           const void* kvar, float* score, float* mu, float* sigma, float* head_score,
                           void* stream) {
    ekv::Dims d;
    ekv_status st = check_shape(shape, &d);
    if (st != EKV_OK) return st;
    if (!q || !page_table || !seq_lens) return fail(EKV_ERR_INVALID_ARG, "q, page_table and seq_lens are required");
    if (selector == EKV_SEL_TOPK) {
        if (!kmin || !kmax || !score) return fail(EKV_ERR_INVALID_ARG, "top-k scoring needs kmin, kmax and score");
        hipError_t e = ekv::launch_box_score(d, q, page_table, seq_lens, kmin, kmax, score, (hipStream_t)stream);
        if (e == hipSuccess && head_score)
            e = ekv::launch_head_box_score(d, q, page_table, seq_lens, kmin, kmax, head_score, (hipStream_t)stream);
        return hip_status(e, "ekv_score_pages");
    }
    if (selector == EKV_SEL_GAUSS) {
        if (!kmean || !kvar || !mu || !sigma) return fail(EKV_ERR_INVALID_ARG, "Gaussian scoring needs kmean, kvar, mu and sigma");
        if (head_score) return fail(EKV_ERR_INVALID_ARG, "head_score is an output of top-k scoring only");
        return hip_status(ekv::launch_gauss_score(d, q, page_table, seq_lens, kmean, kvar, mu, sigma,
                                                  (hipStream_t)stream),
                          "ekv_score_pages");
    }
    return fail(EKV_ERR_INVALID_ARG, "unknown selector %d", selector);
}

ekv_status ekv_select(const ekv_shape* shape, int32_t selector, const int32_t* seq_lens, float alpha,
                      int32_t budget_pages, float z, const float* score, const float* mu, const float* sigma,
                      int32_t* sel_pages, int32_t* sel_count, float* tau_hat, void* workspace,
                      size_t* workspace_bytes, void* stream) {
    ekv::Dims d;
    ekv_status st = check_shape(shape, &d);
    if (st != EKV_OK) return st;
    if (!workspace_bytes) return fail(EKV_ERR_INVALID_ARG, "workspace_bytes is NULL");
    if (budget_pages < 1) return fail(EKV_ERR_INVALID_ARG, "budget_pages=%d < 1", budget_pages);
    if (selector != EKV_SEL_TOPK && selector != EKV_SEL_GAUSS && selector != EKV_SEL_SUPERSET)
        return fail(EKV_ERR_INVALID_ARG, "unknown selector %d", selector);
    const bool gauss = selector == EKV_SEL_GAUSS;
    const bool superset = selector == EKV_SEL_SUPERSET;
    if (gauss) {
        if (!(alpha > 1.0f)) return fail(EKV_ERR_INVALID_ARG, "Gaussian selection needs alpha > 1 (got %g)", alpha);
        if (!gauss_alpha_ok(alpha))
            return fail(EKV_ERR_UNSUPPORTED, "Gaussian selection built for alpha in {2, 3/2, 4/3} (got %g)", alpha);
        if (!(z == z)) return fail(EKV_ERR_INVALID_ARG, "z is NaN");
    }
    if (superset && !(alpha > 1.0f)) return fail(EKV_ERR_INVALID_ARG, "superset selection needs alpha > 1 (got %g)", alpha);
    if (superset && !(alpha < 1e6f)) return fail(EKV_ERR_INVALID_ARG, "alpha out of range (got %g)", alpha);
    const size_t keys_bytes = align256(ekv::select_keys_bytes(d, budget_pages));
    const size_t tau_bytes = gauss ? align256((size_t)d.B * d.HQ * sizeof(float)) : 0;
    const size_t need = keys_bytes + tau_bytes;
    if (!workspace) {
        *workspace_bytes = need;
        return ok();
    }
    if (*workspace_bytes < need)
        return fail(EKV_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", *workspace_bytes, need);
    if (((uintptr_t)workspace & 255) != 0) return fail(EKV_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    if (!seq_lens || !sel_pages || !sel_count) return fail(EKV_ERR_INVALID_ARG, "seq_lens, sel_pages and sel_count are required");
    if (gauss ? (!mu || !sigma) : !score) return fail(EKV_ERR_INVALID_ARG, "missing page scores for the selector");
    if (superset && !tau_hat) return fail(EKV_ERR_INVALID_ARG, "superset selection needs tau_hat (per-head lower bounds)");
    uint32_t* keys = (uint32_t*)workspace;
    float* th = tau_hat ? tau_hat : (float*)((char*)workspace + keys_bytes);
    hipStream_t s = (hipStream_t)stream;
    if (gauss) {
        hipError_t e = ekv::launch_gauss_tau(d, mu, sigma, seq_lens, alpha, th, s);
        if (e != hipSuccess) return hip_status(e, "ekv_select (threshold estimate)");
    }
    return hip_status(ekv::launch_select(d, selector, seq_lens, alpha, budget_pages, z, score, mu, sigma,
                                         th, keys, sel_pages, sel_count, s),
                      "ekv_select");
}

ekv_status ekv_entmax_decode(const ekv_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* page_table, const int32_t* seq_lens, const int32_t* sel_pages,
                             const int32_t* sel_count, int32_t sel_stride, float alpha, const float* tau_hint,
                             const float* tau_ref,
                             float* out, float* tau, int32_t* support, float* delta, int32_t* support_ref,
                             void* workspace,
                             size_t* workspace_bytes, void* stream) {
    ekv::Dims d;
    ekv::DecodePlan pl;
    const int sparse = sel_pages != nullptr;
    ekv_status st = check_decode(shape, sparse, sel_stride, sel_count, alpha, tau_ref, delta, support_ref, &d, &pl);
    if (st != EKV_OK) return st;
    if (!workspace_bytes) return fail(EKV_ERR_INVALID_ARG, "workspace_bytes is NULL");
    if (!workspace) {
        *workspace_bytes = pl.bytes;
        return ok();
    }
    if (*workspace_bytes < pl.bytes)
        return fail(EKV_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", *workspace_bytes, pl.bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(EKV_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out || !tau)
        return fail(EKV_ERR_INVALID_ARG, "q, k_cache, v_cache, page_table, seq_lens, out and tau are required");
    const ekv::DecodeHeads io = {tau_hint, tau_ref, out, tau, support, delta, support_ref};
    return hip_status(ekv::launch_decode(d, pl, q, k_cache, v_cache, page_table, seq_lens, sel_pages, sel_count,
                                         sel_stride, alpha, io, (char*)workspace, (hipStream_t)stream),
                      "ekv_entmax_decode");
}

ekv_status ekv_entmax_decode_noalloc(const ekv_shape* shape, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                                     const int32_t* sel_pages, const int32_t* sel_count, int32_t sel_stride,
                                     float alpha, const float* tau_hint, const float* tau_ref, float* out,
                                     float* tau, int32_t* support, float* delta, int32_t* support_ref,
                                     void* stream) {
    ekv::Dims d;
    ekv::DecodePlan pl;
    const int sparse = sel_pages != nullptr;
    ekv_status st = check_decode(shape, sparse, sel_stride, sel_count, alpha, tau_ref, delta, support_ref, &d, &pl);
    if (st != EKV_OK) return st;
    if (pl.bytes > kNoallocScratchBytes)
        return fail(EKV_ERR_WORKSPACE,
                    "this decode needs %zu bytes of scratch, more than the %zu bytes the no-allocation entry "
                    "point holds per GPU; use ekv_entmax_decode with a caller workspace",
                    pl.bytes, kNoallocScratchBytes);
    if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out || !tau)
        return fail(EKV_ERR_INVALID_ARG, "q, k_cache, v_cache, page_table, seq_lens, out and tau are required");
    void* ws = nullptr;
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return hip_status(e, "ekv_entmax_decode_noalloc (scratch address)");
    const ekv::DecodeHeads io = {tau_hint, tau_ref, out, tau, support, delta, support_ref};
    return hip_status(ekv::launch_decode(d, pl, q, k_cache, v_cache, page_table, seq_lens, sel_pages, sel_count,
                                         sel_stride, alpha, io, (char*)ws, (hipStream_t)stream),
                      "ekv_entmax_decode_noalloc");
}

ekv_status ekv_probe_read(const void* buf, size_t bytes, const int32_t* order, int32_t unroll, int32_t blocks,
                          uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(EKV_ERR_INVALID_ARG, "buf and sink are required");
    if (bytes == 0 || bytes % 4096 != 0) return fail(EKV_ERR_INVALID_ARG, "bytes=%zu is not a positive multiple of 4096", bytes);
    if (((uintptr_t)buf & 15) != 0) return fail(EKV_ERR_INVALID_ARG, "buf not 16-byte aligned");
    if (bytes / 4096 > 0x7fffffffull) return fail(EKV_ERR_UNSUPPORTED, "more than 2^31 - 1 chunks");
    if (unroll != 2 && unroll != 4 && unroll != 8) return fail(EKV_ERR_UNSUPPORTED, "unroll=%d not in {2,4,8}", unroll);
    if (blocks < 1 || blocks > (1 << 20)) return fail(EKV_ERR_INVALID_ARG, "blocks=%d not in [1, 2^20]", blocks);
    return hip_status(ekv::launch_probe_read(buf, (long)(bytes / 4096), order, unroll, blocks, sink,
                                             (hipStream_t)stream),
                      "ekv_probe_read");
}

}  // extern "C"
