// Candidate page selection ("EntmaxKV: Support-Aware Decoding for Entmax
// Attention", section 4.3).
//
// gauss_tau_kernel: per (sequence, query head), the distributional entmax
// threshold of Appendix C.2 Eq. (18),
//     F(tau) = sum_p n_p E[[(alpha-1) S_p - tau]_+^beta] - 1 = 0,
//     S_p ~ N(mu_p, sigma_p^2),
// with the closed-form truncated-normal expectations (beta = 1, 2, 3; with
// m = (alpha-1) mu - tau, v = (alpha-1) sigma, z = m/v):
//     E1 = m Phi + v phi,  E2 = (m^2 + v^2) Phi + m v phi,
//     E3 = (m^3 + 3 m v^2) Phi + v (m^2 + 2 v^2) phi,   v = 0: [m]_+^beta.
// F is convex and decreasing in tau and F(max_p (alpha-1) mu_p - 1) >= 0
// (Jensen on the page with the largest mean), so Newton steps taken from that
// point increase monotonically to the root; dF/dtau = -beta sum n_p E_{beta-1}.
// The page moments are staged in LDS when they fit.
//
// select_kernel: one block per (sequence, KV group).  Keys are the pooled box
// score (top-k) or the pooled Gaussian margin
//     t_p = max_h (mu_{h,p} - tau_hat_h/(alpha-1)) / sigma_{h,p}
// (Gaussian; sigma = 0 gives +inf when mu > theta, else -inf).  Pages with a
// key at or above the cutoff (-inf for top-k, -z for Gaussian) are candidates;
// the min(budget, #candidates) largest keys are kept (at least one page),
// ties going to the lower page index.  The k-th largest key is found by an
// 8-bit radix select over order-preserving 32-bit keys; the kept pages are
// then compacted in index order, which yields ascending output.
#include "ekv_device.h"
#include "ekv_internal.h"

namespace ekv {

constexpr int kTauThreads = 256;
constexpr int kTauLdsPages = 8192;     // 64 KiB of LDS for (a*mu, a*sigma)

__device__ __forceinline__ void gauss_terms(int beta, float m, float v, float& e_b, float& e_bm1) {
    if (v > 0.0f) {
        const float z = m / v;
        const float Phi = 0.5f * erfcf(-z * 0.70710678118654752f);
        const float phi = 0.39894228040143268f * expf(-0.5f * z * z);
        const float e1 = fmaf(m, Phi, v * phi);
        if (beta == 1) {
            e_b = e1;
            e_bm1 = Phi;
        } else {
            const float e2 = fmaf(fmaf(m, m, v * v), Phi, m * v * phi);
            if (beta == 2) {
                e_b = e2;
                e_bm1 = e1;
            } else {
                e_b = fmaf(m * fmaf(m, m, 3.0f * v * v), Phi, v * fmaf(m, m, 2.0f * v * v) * phi);
                e_bm1 = e2;
            }
        }
    } else {
        const float mp = fmaxf(m, 0.0f);
        e_bm1 = beta == 1 ? (m > 0.0f ? 1.0f : 0.0f) : (beta == 2 ? mp : mp * mp);
        e_b = e_bm1 * mp;
    }
}

__global__ __launch_bounds__(kTauThreads) void gauss_tau_kernel(
    const float* __restrict__ mu, const float* __restrict__ sigma, const int32_t* __restrict__ seq_lens,
    int HQ, int MP, float a, int beta, int lds_pages, float* __restrict__ tau_hat) {
    extern __shared__ float lds[];                 // [2][kTauLdsPages] when staged
    __shared__ float red[16];
    int phase = 0;
    const int h = blockIdx.x, b = blockIdx.y;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    float* out = tau_hat + (size_t)b * HQ + h;
    if (M == 0) {
        if (threadIdx.x == 0) *out = -INFINITY;
        return;
    }
    const int last_np = n - (M - 1) * kPage;
    const float* mrow = mu + ((size_t)b * HQ + h) * MP;
    const float* srow = sigma + ((size_t)b * HQ + h) * MP;
    const bool staged = M <= lds_pages;
    float* lm = lds;
    float* ls = lds + lds_pages;

    float xmax = -INFINITY;
    for (int p = threadIdx.x; p < M; p += kTauThreads) {
        float xm = a * mrow[p];
        xmax = fmaxf(xmax, xm);
        if (staged) {
            lm[p] = xm;
            ls[p] = a * srow[p];
        }
    }
    xmax = block_max<kTauThreads / 64>(xmax, red, phase);   // barrier also publishes LDS
    float tau = xmax - 1.0f;
    for (int it = 0; it < 64; ++it) {
        float f = 0.0f, df = 0.0f;
        for (int p = threadIdx.x; p < M; p += kTauThreads) {
            const float xm = staged ? lm[p] : a * mrow[p];
            const float v = staged ? ls[p] : a * srow[p];
            const float np = (p == M - 1) ? (float)last_np : (float)kPage;
            float eb, ebm1;
            gauss_terms(beta, xm - tau, v, eb, ebm1);
            f = fmaf(np, eb, f);
            df = fmaf(np, ebm1, df);
        }
        f = block_sum<kTauThreads / 64>(f, red, phase) - 1.0f;
        df = block_sum<kTauThreads / 64>(df, red, phase) * (float)beta;
        if (!(f > 0.0f) || !(df > 0.0f)) break;     // at the root (to rounding)
        const float nt = tau + f / df;
        if (!(nt > tau)) break;                       // no further fp32 progress
        const bool done = (nt - tau) <= 1e-7f * fmaxf(1.0f, fabsf(nt));
        tau = nt;
        if (done) break;
    }
    if (threadIdx.x == 0) *out = tau;
}

// --------------------------------------------------------------- select ----
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Inclusive-exclusive block scan of one flag per thread, in thread order.
// Returns the number of set flags below this thread; *total gets the block
// total.  `wsum` is LDS of kSelWaves ints.
__device__ __forceinline__ int block_excl_scan(bool flag, int* wsum, int* total) {
    const uint64_t m = __ballot(flag);
    const int wid = threadIdx.x >> 6;
    const int below = lanes_below(m);
    if ((threadIdx.x & 63) == 0) wsum[wid] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int c = wsum[i];
        off += (i < wid) ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return off + below;
}

template <int GAUSS, int R>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const int32_t* __restrict__ seq_lens, int G, int MP, int budget, const float* __restrict__ score,
    const float* __restrict__ mu, const float* __restrict__ sigma, const float* __restrict__ tau_hat,
    float inv_a, float zcut, uint32_t* __restrict__ keys_ws, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ sel_count) {
    __shared__ int hist[256];
    __shared__ int wsum[kSelWaves];
    __shared__ float red[2 * kSelWaves];
    __shared__ int sh_digit, sh_above;
    int phase = 0;
    const int g = blockIdx.x, b = blockIdx.y;
    const int HQ = G * R;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    uint32_t* keys = keys_ws + ((size_t)b * G + g) * MP;
    int32_t* out = sel_pages + ((size_t)b * G + g) * budget;

    // Pass A: keys, and the count of candidates at or above the cutoff.
    const uint32_t cut = GAUSS ? ord_key(-zcut) : 0u;
    float theta[R];
    if constexpr (GAUSS) {
#pragma unroll
        for (int j = 0; j < R; ++j) theta[j] = tau_hat[(size_t)b * HQ + g * R + j] * inv_a;
    }
    float cnt = 0.0f;
    for (int p = threadIdx.x; p < M; p += kSelThreads) {
        float f;
        if constexpr (GAUSS) {
            f = -INFINITY;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const size_t o = ((size_t)b * HQ + g * R + j) * MP + p;
                const float dm = mu[o] - theta[j];
                const float sg = sigma[o];
                const float t = sg > 0.0f ? dm / sg : (dm > 0.0f ? INFINITY : -INFINITY);
                f = fmaxf(f, t);
            }
        } else {
            f = score[((size_t)b * G + g) * MP + p];
        }
        const uint32_t k = ord_key(f);
        keys[p] = k;
        cnt += (k >= cut) ? 1.0f : 0.0f;
    }
    const int ncand = (int)block_sum<kSelWaves>(cnt, red, phase);   // barrier: keys visible
    int keep = M == 0 ? 0 : max(1, min(budget, ncand));

    uint32_t T;
    int need_eq;
    if (ncand >= 1 && ncand <= budget) {
        T = cut;              // every candidate, nothing else
        need_eq = M;
    } else if (keep > 0) {
        // Radix select of the keep-th largest key.
        uint32_t prefix = 0;
        int remaining = keep;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
            __syncthreads();
            const uint32_t hmask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
            for (int p = threadIdx.x; p < M; p += kSelThreads) {
                const uint32_t k = keys[p];
                if ((k & hmask) == (prefix & hmask)) atomicAdd(&hist[(k >> shift) & 255u], 1);
            }
            __syncthreads();
            if (threadIdx.x < 64) {
                // Wave 0: lane l holds digits 255-4l .. 252-4l (descending); an
                // inclusive scan over lanes gives the count of keys at or above
                // each lane's lowest digit; the first lane reaching `remaining`
                // walks its four digits.
                const int l = threadIdx.x;
                int c4[4], sum = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    c4[i] = hist[255 - 4 * l - i];
                    sum += c4[i];
                }
                int incl = sum;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int o = __shfl_up(incl, off, 64);
                    if (l >= off) incl += o;
                }
                const uint64_t hit = __ballot(incl >= remaining);
                const int L = hit ? (int)__builtin_ctzll(hit) : 63;
                if (l == L) {
                    int above = incl - sum, dgt = 255 - 4 * l - 3;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (above + c4[i] >= remaining) { dgt = 255 - 4 * l - i; break; }
                        above += c4[i];
                    }
                    sh_digit = dgt;
                    sh_above = above;
                }
            }
            __syncthreads();
            prefix |= (uint32_t)sh_digit << shift;
            remaining -= sh_above;
        }
        T = prefix;
        need_eq = remaining;
    } else {
        T = 0xffffffffu;
        need_eq = 0;
    }

    // Compaction in page order: keys > T, then the first need_eq keys == T.
    int written = 0, eq_seen = 0;
    for (int base = 0; base < M; base += kSelThreads) {
        const int p = base + threadIdx.x;
        const uint32_t k = p < M ? keys[p] : 0u;
        const bool eq = p < M && k == T;
        int eq_tot;
        const int eq_rank = eq_seen + block_excl_scan(eq, wsum, &eq_tot);
        const bool take = p < M && (k > T || (eq && eq_rank < need_eq));
        int tot;
        const int pos = written + block_excl_scan(take, wsum, &tot);
        if (take && pos < budget) out[pos] = p;
        written += tot;
        eq_seen += eq_tot;
    }
    for (int i = written + threadIdx.x; i < budget; i += kSelThreads) out[i] = -1;
    if (threadIdx.x == 0) sel_count[(size_t)b * G + g] = min(written, budget);
}

hipError_t launch_gauss_tau(const Dims& d, const float* mu, const float* sigma,
                            const int32_t* seq_lens, float alpha, float* tau_hat, hipStream_t s) {
    const float a = alpha - 1.0f;
    const int beta = (int)lrintf(1.0f / a);
    // Stage (a*mu, a*sigma) in LDS for sequences of up to kTauLdsPages pages
    // (64 KiB; gfx950 gives a workgroup up to 160 KiB of LDS).
    int lds_pages = d.MP < kTauLdsPages ? d.MP : kTauLdsPages;
    size_t lds = (size_t)2 * lds_pages * sizeof(float);
    static bool attr_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (lds > 48 * 1024 && !attr_set[dev]) {
        if (hipFuncSetAttribute((const void*)gauss_tau_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) == hipSuccess) {
            attr_set[dev] = true;
        } else {
            (void)hipGetLastError();
            lds_pages = 0;
            lds = 0;
        }
    }
    gauss_tau_kernel<<<dim3(d.HQ, d.B), dim3(kTauThreads), lds, s>>>(mu, sigma, seq_lens, d.HQ, d.MP,
                                                                      a, beta, lds_pages, tau_hat);
    return hipGetLastError();
}

hipError_t launch_select(const Dims& d, int gauss, const int32_t* seq_lens, float alpha,
                         int budget, float z, const float* score, const float* mu,
                         const float* sigma, const float* tau_hat, uint32_t* keys,
                         int32_t* sel_pages, int32_t* sel_count, hipStream_t s) {
    const float inv_a = alpha > 1.0f ? 1.0f / (alpha - 1.0f) : 0.0f;
    dim3 grid(d.G, d.B);
#define EKV_SEL(RR, GG)                                                                              \
    select_kernel<GG, RR><<<grid, dim3(kSelThreads), 0, s>>>(seq_lens, d.G, d.MP, budget, score, mu, \
                                                             sigma, tau_hat, inv_a, z, keys,          \
                                                             sel_pages, sel_count);                   \
    return hipGetLastError();
    if (gauss) {
        switch (d.R) {
            case 1: { EKV_SEL(1, 1) }
            case 2: { EKV_SEL(2, 1) }
            case 4: { EKV_SEL(4, 1) }
            case 8: { EKV_SEL(8, 1) }
            default: return hipErrorInvalidValue;
        }
    }
    EKV_SEL(1, 0)
#undef EKV_SEL
}

}  // namespace ekv
