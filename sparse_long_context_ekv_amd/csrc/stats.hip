// Page key statistics: per (physical page, group, channel) min / max / mean /
// population variance over the page's valid tokens; and the append path that
// writes one new token per sequence and refreshes its page's statistics.
//
// Follows "EntmaxKV: Support-Aware Decoding for Entmax Attention" section 4.2
// and Appendix B.1 (per-channel page min/max of the keys) and section 4.3
// (per-page mean/variance read by the Gaussian selector).
//
// Mapping: one 16-lane row per (page, group) tile; lane l owns channels
// [l*CH, (l+1)*CH) and walks the page's 16 token rows, so each token row is
// one contiguous D*sizeof(T)-byte read by the 16 lanes.  The whole tile stays
// in registers: min/max are exact selections of stored values, the mean is an
// fp32 sum in token order divided by n_p, the variance a second pass over the
// registers (sum of squared deviations / n_p).
#include "ekv_device.h"
#include "ekv_internal.h"

namespace ekv {

// Statistics of one (page, group) tile held by a 16-lane row: v[t] holds this
// lane's CH channels of token t, tokens 0..np-1 valid.  Writes this lane's
// slice of kmin/kmax (exact selections of stored values, KV dtype) and
// kmean/kvar (fp32 sum in token order / n_p; population variance by a second
// pass over the registers; rounded to the statistics dtype: fp32, bf16 or
// FP8 E4M3, each round to nearest even, FP8 saturating at 448) at `out`.
// Shared by the whole-cache build and the append path, so the two agree bit
// for bit.
template <typename T, int CH, typename S>
__device__ __forceinline__ void tile_stats_store(const Vec<T, CH> (&v)[kPage], int np, size_t out,
                                                 T* __restrict__ kmin, T* __restrict__ kmax,
                                                 S* __restrict__ kmean, S* __restrict__ kvar) {
    float mn[CH], mx[CH], sm[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        mn[c] = v[0].get(c);
        mx[c] = mn[c];
        sm[c] = mn[c];
    }
#pragma unroll
    for (int t = 1; t < kPage; ++t) {
        if (t < np) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float x = v[t].get(c);
                mn[c] = fminf(mn[c], x);
                mx[c] = fmaxf(mx[c], x);
                sm[c] += x;
            }
        }
    }
    float mean[CH], var[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        mean[c] = sm[c] / (float)np;
        var[c] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
        if (t < np) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float dlt = v[t].get(c) - mean[c];
                var[c] = fmaf(dlt, dlt, var[c]);
            }
        }
    }
    if (kmin) {
        Vec<T, CH> a, c2;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            a.set_exact(c, mn[c]);
            c2.set_exact(c, mx[c]);
        }
        a.store(kmin + out);
        c2.store(kmax + out);
    }
    if (kmean) {
        if constexpr (std::is_same<S, float>::value) {
#pragma unroll
            for (int c = 0; c < CH; c += 4) {
                *reinterpret_cast<float4*>(kmean + out + c) = make_float4(mean[c], mean[c + 1], mean[c + 2], mean[c + 3]);
                *reinterpret_cast<float4*>(kvar + out + c) =
                    make_float4(var[c] / (float)np, var[c + 1] / (float)np, var[c + 2] / (float)np, var[c + 3] / (float)np);
            }
        } else if constexpr (std::is_same<S, bf16_t>::value) {
            Vec<bf16_t, CH> a, c2;
#pragma unroll
            for (int c = 0; c < CH; c += 2) {
                a.w[c >> 1] = f32_to_bf16_rne(mean[c]) | (f32_to_bf16_rne(mean[c + 1]) << 16);
                c2.w[c >> 1] = f32_to_bf16_rne(var[c] / (float)np) | (f32_to_bf16_rne(var[c + 1] / (float)np) << 16);
            }
            a.store(kmean + out);
            c2.store(kvar + out);
        } else {
            Vec<fp8_t, CH> a, c2;
#pragma unroll
            for (int c = 0; c < CH; c += 4) {
                uint32_t wm = 0, wv = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    wm |= f32_to_e4m3_sat(mean[c + k]) << (8 * k);
                    wv |= f32_to_e4m3_sat(var[c + k] / (float)np) << (8 * k);
                }
                a.w[c >> 2] = wm;
                c2.w[c >> 2] = wv;
            }
            a.store(kmean + out);
            c2.store(kvar + out);
        }
    }
}

template <typename T, int D, typename S>
__global__ __launch_bounds__(256) void page_stats_kernel(
    const T* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_list, int n_items,
    int B, int G, int MP, int NP, T* __restrict__ kmin, T* __restrict__ kmax, S* __restrict__ kmean,
    S* __restrict__ kvar) {
    constexpr int CH = D / kRow;
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;
    const int per_iter = kRow / G;               // (page) items per block iteration
    if (row >= per_iter * G) return;             // whole idle rows only
    const int g = row % G;
    for (int item = blockIdx.x * per_iter + row / G; item < n_items; item += gridDim.x * per_iter) {
        int e = page_list ? page_list[item] : item;
        if (e < 0) continue;                      // a negative entry would divide to b = 0, p < 0
        int b = e / MP, p = e - b * MP;
        if (b >= B) continue;
        int n = seq_len_at(seq_lens, b, MP);
        if (p >= num_pages(n)) continue;
        int np = min(kPage, n - p * kPage);
        int phys = page_table[(size_t)b * MP + p];
        if (phys < 0 || phys >= NP) continue;     // corrupt table entry: never read outside the cache
        const T* tile = k_cache + ((size_t)phys * G + g) * kPage * D + lane * CH;

        Vec<T, CH> v[kPage];
#pragma unroll
        for (int t = 0; t < kPage; ++t)
            if (t < np) v[t].load(tile + (size_t)t * D);
        tile_stats_store<T, CH, S>(v, np, ((size_t)phys * G + g) * D + lane * CH, kmin, kmax, kmean, kvar);
    }
}

// Append one token per sequence and refresh the statistics of the page it
// lands in.  One 16-lane row per (sequence, group): the new key and value are
// written at position n = seq_lens[b] (logical page n/16, slot n%16); the
// page's earlier tokens are read back, the new key joins them from registers,
// and tile_stats_store recomputes the page's statistics exactly as the
// whole-cache build would.  A sequence whose position has no valid physical
// page (n at capacity, or a bad table entry) is left untouched.
template <typename T, int D, typename S>
__global__ __launch_bounds__(256) void append_kv_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int B, int G, int MP, int NP, T* __restrict__ k_cache,
    T* __restrict__ v_cache, T* __restrict__ kmin, T* __restrict__ kmax, S* __restrict__ kmean,
    S* __restrict__ kvar, int32_t* __restrict__ new_lens) {
    constexpr int CH = D / kRow;
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;
    const int per_iter = kRow / G;
    if (row >= per_iter * G) return;             // whole idle rows only (no barrier in this kernel)
    const int g = row % G;
    for (int b = blockIdx.x * per_iter + row / G; b < B; b += gridDim.x * per_iter) {
        const int n = seq_lens[b];
        const int p = n >> 4, t = n & (kPage - 1);
        const int phys = (n >= 0 && p < MP) ? page_table[(size_t)b * MP + p] : -1;
        const bool ok = phys >= 0 && phys < NP;
        if (new_lens && g == 0 && lane == 0) new_lens[b] = ok ? n + 1 : n;
        if (!ok) continue;
        const size_t src = ((size_t)b * G + g) * D + lane * CH;
        const size_t tile = ((size_t)phys * G + g) * kPage * D + lane * CH;
        Vec<T, CH> kn, vn;
        kn.load(k_new + src);
        vn.load(v_new + src);
        kn.store(k_cache + tile + (size_t)t * D);
        vn.store(v_cache + tile + (size_t)t * D);
        if (!kmin && !kmean) continue;
        Vec<T, CH> v[kPage];
#pragma unroll
        for (int i = 0; i < kPage; ++i) {
            if (i < t) v[i].load(k_cache + tile + (size_t)i * D);
            else if (i == t) v[i] = kn;
        }
        tile_stats_store<T, CH, S>(v, t + 1, ((size_t)phys * G + g) * D + lane * CH, kmin, kmax, kmean, kvar);
    }
}

template <typename T, int D, typename S>
static hipError_t run_stats(const Dims& d, const void* k, const int32_t* pt, const int32_t* sl,
                            const int32_t* pl, int n_items, void* kmin, void* kmax, void* kmean,
                            void* kvar, hipStream_t s) {
    const int per_iter = kRow / d.G;
    long blocks = ((long)n_items + per_iter - 1) / per_iter;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    page_stats_kernel<T, D, S><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        (const T*)k, pt, sl, pl, n_items, d.B, d.G, d.MP, d.NP, (T*)kmin, (T*)kmax, (S*)kmean, (S*)kvar);
    return hipGetLastError();
}

hipError_t launch_page_stats(const Dims& d, const void* k_cache, const int32_t* page_table,
                             const int32_t* seq_lens, const int32_t* page_list, int n_list,
                             void* kmin, void* kmax, void* kmean, void* kvar, hipStream_t s) {
    const int n_items = page_list ? n_list : d.B * d.MP;
    if (n_items <= 0) return hipSuccess;
#define EKV_STATS(T, DD, S) return run_stats<T, DD, S>(d, k_cache, page_table, seq_lens, page_list, n_items, kmin, kmax, kmean, kvar, s)
    if (d.kv_bf16) {
        if (d.D == 128) { switch (d.stat) { case kStatBF16: EKV_STATS(bf16_t, 128, bf16_t); case kStatFP8: EKV_STATS(bf16_t, 128, fp8_t); default: EKV_STATS(bf16_t, 128, float); } }
        else            { switch (d.stat) { case kStatBF16: EKV_STATS(bf16_t, 64, bf16_t); case kStatFP8: EKV_STATS(bf16_t, 64, fp8_t); default: EKV_STATS(bf16_t, 64, float); } }
    } else {
        if (d.D == 128) { switch (d.stat) { case kStatBF16: EKV_STATS(float, 128, bf16_t); case kStatFP8: EKV_STATS(float, 128, fp8_t); default: EKV_STATS(float, 128, float); } }
        else            { switch (d.stat) { case kStatBF16: EKV_STATS(float, 64, bf16_t); case kStatFP8: EKV_STATS(float, 64, fp8_t); default: EKV_STATS(float, 64, float); } }
    }
#undef EKV_STATS
}

template <typename T, int D, typename S>
static hipError_t run_append(const Dims& d, const void* kn, const void* vn, const int32_t* pt, const int32_t* sl,
                             void* kc, void* vc, void* kmin, void* kmax, void* kmean, void* kvar, int32_t* nl,
                             hipStream_t s) {
    const int per_iter = kRow / d.G;
    long blocks = ((long)d.B + per_iter - 1) / per_iter;
    if (blocks > 65536) blocks = 65536;
    append_kv_kernel<T, D, S><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        (const T*)kn, (const T*)vn, pt, sl, d.B, d.G, d.MP, d.NP, (T*)kc, (T*)vc, (T*)kmin, (T*)kmax, (S*)kmean,
        (S*)kvar, nl);
    return hipGetLastError();
}

hipError_t launch_append_kv(const Dims& d, const void* k_new, const void* v_new, const int32_t* page_table,
                            const int32_t* seq_lens, void* k_cache, void* v_cache, void* kmin, void* kmax,
                            void* kmean, void* kvar, int32_t* new_lens, hipStream_t s) {
#define EKV_APP(T, DD, S) return run_append<T, DD, S>(d, k_new, v_new, page_table, seq_lens, k_cache, v_cache, kmin, kmax, kmean, kvar, new_lens, s)
    if (d.kv_bf16) {
        if (d.D == 128) { switch (d.stat) { case kStatBF16: EKV_APP(bf16_t, 128, bf16_t); case kStatFP8: EKV_APP(bf16_t, 128, fp8_t); default: EKV_APP(bf16_t, 128, float); } }
        else            { switch (d.stat) { case kStatBF16: EKV_APP(bf16_t, 64, bf16_t); case kStatFP8: EKV_APP(bf16_t, 64, fp8_t); default: EKV_APP(bf16_t, 64, float); } }
    } else {
        if (d.D == 128) { switch (d.stat) { case kStatBF16: EKV_APP(float, 128, bf16_t); case kStatFP8: EKV_APP(float, 128, fp8_t); default: EKV_APP(float, 128, float); } }
        else            { switch (d.stat) { case kStatBF16: EKV_APP(float, 64, bf16_t); case kStatFP8: EKV_APP(float, 64, fp8_t); default: EKV_APP(float, 64, float); } }
    }
#undef EKV_APP
}

}  // namespace ekv
