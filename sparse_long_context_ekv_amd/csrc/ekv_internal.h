// Host-side interface between the C ABI layer (api.hip) and the kernel
// launchers (stats.hip, score.hip, select.hip, decode.hip).  Each launcher
// enqueues its kernels on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ekv {

enum { kStatF32 = 0, kStatBF16 = 1, kStatFP8 = 2 };

struct Dims {
    int B, HQ, G, R, D, MP, NP;
    int kv_bf16;     // 1 = bf16 KV, 0 = fp32
    int stat;        // mean/var storage: kStatF32, kStatBF16, kStatFP8
};

// Page statistics.
hipError_t launch_page_stats(const Dims& d, const void* k_cache, const int32_t* page_table,
                             const int32_t* seq_lens, const int32_t* page_list, int n_list,
                             void* kmin, void* kmax, void* kmean, void* kvar, hipStream_t s);

// Append one token per sequence (+ statistics of its page).
hipError_t launch_append_kv(const Dims& d, const void* k_new, const void* v_new, const int32_t* page_table,
                            const int32_t* seq_lens, void* k_cache, void* v_cache, void* kmin, void* kmax,
                            void* kmean, void* kvar, int32_t* new_lens, hipStream_t s);

// Page scores.
hipError_t launch_box_score(const Dims& d, const void* q, const int32_t* page_table,
                            const int32_t* seq_lens, const void* kmin, const void* kmax,
                            float* score, hipStream_t s);
hipError_t launch_head_box_score(const Dims& d, const void* q, const int32_t* page_table, const int32_t* seq_lens,
                                 const void* kmin, const void* kmax, float* head_score, hipStream_t s);
hipError_t launch_gauss_score(const Dims& d, const void* q, const int32_t* page_table,
                              const int32_t* seq_lens, const void* kmean, const void* kvar,
                              float* mu, float* sigma, hipStream_t s);

// Selection.  mode: 0 top-k, 1 Gaussian, 2 support superset (ekv_selector).
// `keys` is workspace of select_keys_bytes(d, budget) bytes (256-byte aligned).
hipError_t launch_gauss_tau(const Dims& d, const float* mu, const float* sigma,
                            const int32_t* seq_lens, float alpha, float* tau_hat, hipStream_t s);
size_t select_keys_bytes(const Dims& d, int budget);
hipError_t launch_select(const Dims& d, int mode, const int32_t* seq_lens, float alpha,
                         int budget, float z, const float* score, const float* mu,
                         const float* sigma, const float* tau_hat, uint32_t* keys,
                         int32_t* sel_pages, int32_t* sel_count, hipStream_t s);

// Decode.
struct DecodePlan {
    int sparse;      // selection given
    int fused;       // sparse entmax within kFusedMaxSlots: logits kernel + one tau/PV kernel per (b, g)
    int stream;      // entmax otherwise: candidate stream, threshold, PV over the support
    int smx1;        // softmax over bf16 keys: one pass (streamed blocks), then a merge
    int nslot;       // slots per (b, h): selected (or all) pages x page size
    // fused and softmax paths: logits kernel blocks
    int lg_ppb;      // log2 of ppb
    int ppb;         // pages per logits block
    int nchunk1;     // logits blocks per (b, g)
    // softmax path: PV blocks over all slots
    int spb;         // slots per PV block (multiple of 256)
    int nchunk3;     // PV blocks per (b, g)
    // stream path
    int cpb_s;       // chunks (of 32 pages) per candidate-stream block
    int nsplit_s;    // candidate-stream blocks per (b, g)
    int too_long;    // rows longer than the stream path is built for
    size_t off_logits, off_part1, off_part3;
    size_t off_cands, off_ccount, off_cmax, off_sup, off_supcnt, off_order;
    size_t bytes;
};
DecodePlan plan_decode(const Dims& d, int sparse, int sel_stride, float alpha);

// Per-(sequence, head) inputs and outputs of one decode, each [B][HQ]
// (out [B][HQ][D]); the optional ones may be NULL.
struct DecodeHeads {
    const float* tau_hint;   // start of the threshold iteration (x units), or NULL
    const float* tau_ref;    // threshold of the reference distribution (delta, supref), or NULL
    float* out;
    float* tau;
    int32_t* support;
    float* delta;
    int32_t* supref;
};

hipError_t launch_decode(const Dims& d, const DecodePlan& pl, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* sel_pages, const int32_t* sel_count, int sel_stride,
                         float alpha, const DecodeHeads& io, char* ws, hipStream_t s);

// Per-dtype decode launches (decode_bf16.hip, decode_f32.hip); mode is the
// entmax mode of decode_kernels.h and beta = 1/(alpha-1).
hipError_t launch_decode_bf16(const Dims& d, const DecodePlan& pl, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                              const int32_t* sel_pages, const int32_t* sel_count, int sel_stride, float alpha,
                              int mode, float beta, const DecodeHeads& io, char* ws, hipStream_t s);
hipError_t launch_decode_f32(const Dims& d, const DecodePlan& pl, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                             const int32_t* sel_pages, const int32_t* sel_count, int sel_stride, float alpha,
                             int mode, float beta, const DecodeHeads& io, char* ws, hipStream_t s);


// Streaming-read probe (probe.hip).
hipError_t launch_probe_read(const void* buf, long n_chunks, const int32_t* order, int unroll, int blocks,
                             uint32_t* sink, hipStream_t s);

}  // namespace ekv
