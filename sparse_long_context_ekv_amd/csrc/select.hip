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
// F is decreasing in tau, dF/dtau = -beta sum n_p E_{beta-1}, and
// F(max_p (alpha-1) mu_p - 1) >= 1 (Jensen on the page with the largest mean),
// which starts a bracketed Newton iteration on log F (see gauss_tau_kernel).
// The page moments are staged in LDS when they fit.
//
// select_reg_kernel / select_kernel: one block per (sequence, KV group).
// Keys are the pooled box
// score (top-k) or the pooled Gaussian margin
//     t_p = max_h (mu_{h,p} - tau_hat_h/(alpha-1)) / sigma_{h,p}
// (Gaussian; sigma = 0 gives +inf when mu > theta, else -inf).  Pages with a
// key at or above the cutoff (-inf for top-k, -z for Gaussian) are candidates;
// the min(budget, #candidates) largest keys are kept (at least one page),
// ties going to the lower page index.  The k-th largest key is found by an
// 8-bit radix select over order-preserving 32-bit keys; the kept pages are
// then compacted in index order, which yields ascending output.
#include <atomic>

#include "ekv_device.h"
#include "ekv_internal.h"

namespace ekv {

constexpr int kTauThreads = 512;
constexpr int kTauWaves = kTauThreads / 64;
constexpr int kTauLdsPages = 8192;     // 64 KiB of LDS for the (a*mu, a*sigma) pairs
constexpr int kTauMaxIter = 40;
constexpr float kTauTol = 1e-5f;       // stop once a step is below this (relative)
constexpr int kTauSub = 16;            // warm start: every 16th page ...
constexpr int kTauSubMin = 2048;       // ... for sequences of at least this many pages
constexpr float kTauSubTol = 1e-3f;     // below the subsample's own error (about 1e-2)
// Early stop of the passes over all pages (see gauss_tau_solve).  Measured on
// the clustered 128K workload (fp64 replay of the iteration): from the
// warm start (relative error ~1e-2) one Halley step leaves ~1e-7 and one
// Newton step ~4e-5.
constexpr float kTauAcceptHalley = 3e-2f;
constexpr float kTauAcceptNewton = 1e-3f;

// Standard normal upper tail Q(x) = 1 - Phi(x), x >= 0, as phi(x) R(x) with
// the Mills ratio R(x) ~ t h(t), t = 1/(1 + kMillsK x), h the polynomial
// below (fitted by fit_mills_ratio.py beside this file; relative error of R
// about 3e-7 in fp32 over all x >= 0).
constexpr float kMillsK = 0.4f;
constexpr float kMillsC[12] = {
    4.000000060e-01f, 3.999997675e-01f, 3.360165060e-01f, 2.075455040e-01f,
    5.289435759e-02f, -1.341597885e-01f, 1.025012210e-01f, -7.160952091e-01f,
    1.344201684e+00f, -1.132010460e+00f, 4.732496738e-01f, -8.082909137e-02f};
constexpr float kTinyV = 1e-30f;       // v at or below this: the page is a point mass

// n_p-free terms of page p at threshold tau, with m = (alpha-1) mu_p - tau,
// v = (alpha-1) sigma_p, z = m/v: e_b = E[Y_+^beta], e_b1 = E[Y_+^(beta-1)],
// e_b2 = E[Y_+^(beta-2)] for Y ~ N(m, v^2), where E[Y_+^0] = P(Y > 0) = Phi(z)
// and E[Y_+^-1] stands for the density of Y at 0, phi(z)/v (the derivative of
// Phi(z) in m).  A page with v <= kTinyV is a point mass at m: E[Y_+^k] =
// [m]_+^k (and 0 for the density).  Branch-free: both forms are computed and
// one is selected.
template <int BETA>
__device__ __forceinline__ void gauss_terms(float m, float v, float& e_b, float& e_b1, float& e_b2) {
    const bool point = !(v > kTinyV);
    const float vs = point ? 1.0f : v;
    const float rv = __builtin_amdgcn_rcpf(vs);
    const float z = m * rv;
    const float t = __builtin_amdgcn_rcpf(fmaf(kMillsK, fabsf(z), 1.0f));
    float h = kMillsC[11];
#pragma unroll
    for (int i = 10; i >= 0; --i) h = fmaf(h, t, kMillsC[i]);
    // phi(z) = exp(-z^2/2) / sqrt(2 pi), through 2^x
    const float phi = 0.39894228040143268f * __builtin_amdgcn_exp2f(-0.72134752044448170f * z * z);
    const float q = phi * t * h;
    const float Phi = z < 0.0f ? q : 1.0f - q;
    const float mp = fmaxf(m, 0.0f);
    const float e1 = fmaf(m, Phi, vs * phi);
    if constexpr (BETA == 1) {
        e_b = point ? mp : e1;
        e_b1 = point ? (m > 0.0f ? 1.0f : 0.0f) : Phi;
        e_b2 = point ? 0.0f : phi * rv;
    } else {
        const float e2 = fmaf(fmaf(m, m, vs * vs), Phi, m * vs * phi);
        if constexpr (BETA == 2) {
            e_b = point ? mp * mp : e2;
            e_b1 = point ? mp : e1;
            e_b2 = point ? (m > 0.0f ? 1.0f : 0.0f) : Phi;
        } else {
            const float e3 = fmaf(m * fmaf(m, m, 3.0f * vs * vs), Phi, vs * fmaf(m, m, 2.0f * vs * vs) * phi);
            e_b = point ? mp * mp * mp : e3;
            e_b1 = point ? mp * mp : e2;
            e_b2 = point ? mp : e1;
        }
    }
}

// Sums over pages p = first, first + step, ... < count of `src`:
// f += w_p e_beta, d1 += w_p e_(beta-1), d2 += w_p e_(beta-2), with w_p = w
// except for index `last`, which weighs w_last.  Two pages per trip.
template <int BETA, bool STAGED>
__device__ __forceinline__ void gauss_sums(const float2* __restrict__ src, const float* __restrict__ mrow,
                                           const float* __restrict__ srow, int first, int step, int count,
                                           int last, float w, float w_last, float a, float t, float& f, float& d1,
                                           float& d2) {
    auto page = [&](int p) {
        const float2 e = STAGED ? src[p] : make_float2(a * mrow[p], a * srow[p]);
        const float wp = (p == last) ? w_last : w;
        float eb, eb1, eb2;
        gauss_terms<BETA>(e.x - t, e.y, eb, eb1, eb2);
        f = fmaf(wp, eb, f);
        d1 = fmaf(wp, eb1, d1);
        d2 = fmaf(wp, eb2, d2);
    };
    int p = first;
    for (; p + step < count; p += 2 * step) {
        page(p);
        page(p + step);
    }
    if (p < count) page(p);
}

// Root of F(tau) = 1 for one (sequence, head).  Every iteration evaluates,
// in one pass over the pages, F = sum_p n_p E_beta, D1 = sum_p n_p E_(beta-1)
// and D2 = sum_p n_p E_(beta-2), so that dF/dtau = -beta D1 and
// d2F/dtau2 = beta (beta-1) D2 (beta = 1: F'' = D2, the density sum).
// It keeps a bracket [lo, hi] with F(lo) >= 1 >= F(hi) and steps on
// L = log F: log F is close to linear or concave over the Gaussian tails that
// dominate F, so these steps are accurate from afar, where Newton on F itself
// creeps (F behaves like a high power of the distance to the largest page
// means).  beta >= 2 takes Halley steps on L (third order; D2 costs no extra
// exp or rcp per page); beta = 1 takes Newton steps, since there the Halley
// step on L stays bounded while F >> 1.  While F > 1 a step is capped at four
// times the Newton step on F^(1/beta), which is convex (an L^beta norm of
// (Y - tau)_+ over the page mixture) and so never passes the root.  A step
// that leaves the bracket is replaced by its midpoint.
// The iteration stops after a step below `tol` (relative), or after an
// unmodified Halley / Newton step below `accept`: the error left after such a
// step is of order C step^3 (Halley) or C step^2 (Newton), far below `tol`
// for the `accept` values used (kTauAcceptHalley, kTauAcceptNewton), so the
// confirming pass over all pages is skipped.
// WAVE: one wave runs the whole iteration with wave-level sums and no block
// barrier; otherwise the block shares the pages and sums across waves.
template <int BETA, bool WAVE, bool STAGED>
__device__ float gauss_tau_solve(const float2* __restrict__ src, const float* __restrict__ mrow,
                                 const float* __restrict__ srow, int count, int last, float w, float w_last,
                                 float a, float lo, float t, float tol, float accept, float* red, int& phase) {
    constexpr float fb = (float)BETA;
    float hi = INFINITY;
    const int first = WAVE ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    const int step = WAVE ? 64 : kTauThreads;
    for (int it = 0; it < kTauMaxIter; ++it) {
        float f = 0.0f, d1 = 0.0f, d2 = 0.0f;
        gauss_sums<BETA, STAGED>(src, mrow, srow, first, step, count, last, w, w_last, a, t, f, d1, d2);
        if constexpr (WAVE) {
            f = wave_sum(f);
            d1 = wave_sum(d1);
            d2 = wave_sum(d2);
        } else {
            block_sum3<kTauWaves>(f, d1, d2, red, phase);   // block-uniform from here on
        }
        if (f >= 1.0f) lo = fmaxf(lo, t); else hi = fminf(hi, t);
        if (f == 1.0f) break;
        float step_t = NAN;
        bool pure = false;                                      // an unmodified Halley / Newton step
        if (d1 > 0.0f && f > 0.0f) {
            // step arithmetic in single-instruction approximations (hw_*): it
            // decides where a step lands, not the root F(t) = 1 converges to
            const float rf = hw_rcp(f);
            const float L = hw_log2(f) * 0.69314718055994531f;  // log F
            const float dL = -fb * d1 * rf;                     // d log F / d tau
            step_t = -L * hw_rcp(dL);
            pure = BETA == 1;
            if constexpr (BETA >= 2) {
                const float d2L = fb * (fb - 1.0f) * d2 * rf - dL * dL;
                const float den = 2.0f * dL * dL - L * d2L;
                if (den > 0.0f) {
                    step_t = -2.0f * L * dL * hw_rcp(den);
                    pure = true;
                }
            }
            if (f > 1.0f) {
                const float gr = BETA == 1 ? f : (BETA == 2 ? hw_sqrt(f) : hw_exp2(hw_log2(f) * (1.0f / 3.0f)));
                const float cap = 4.0f * (1.0f - hw_rcp(gr)) * f * hw_rcp(d1);
                if (cap < step_t) {
                    step_t = cap;
                    pure = false;
                }
            }
        }
        float nt = t + step_t;
        if (!(nt >= lo && nt <= hi)) {
            if (!(hi < INFINITY) || !(lo > -INFINITY)) break;   // no usable step, no finite bracket
            nt = 0.5f * (lo + hi);
            step_t = nt - t;
            pure = false;
        }
        const float scale = fmaxf(1.0f, fabsf(t));
        const bool done = fabsf(step_t) <= tol * scale || (pure && fabsf(step_t) <= accept * scale);
        t = nt;
        if (done) break;
    }
    return t;
}

// One block per (sequence, head).  Staging copies (a mu, a sigma) of every
// page into LDS (16-byte loads) and every kTauSub-th page into a compact
// array; the iteration first runs on that subsample (weights x kTauSub, in
// one wave) to a loose tolerance, and the passes over all pages start
// from its estimate: 2 full passes instead of 5 to 6 on 8192-page sequences.
// The full passes keep the exact lower end max_p (alpha-1) mu_p - 1.
template <int BETA>
__global__ __launch_bounds__(kTauThreads) void gauss_tau_kernel(
    const float* __restrict__ mu, const float* __restrict__ sigma, const int32_t* __restrict__ seq_lens,
    int HQ, int MP, float a, int lds_pages, float* __restrict__ tau_hat) {
    extern __shared__ float2 lds2[];               // [lds_pages] pages, then [lds_pages / kTauSub] subsample
    __shared__ float red[6 * kTauWaves];
    int phase = 0;
    const int h = blockIdx.x, b = blockIdx.y;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    float* out = tau_hat + (size_t)b * HQ + h;
    if (M == 0) {
        if (threadIdx.x == 0) *out = -INFINITY;
        return;
    }
    const float last_np = (float)(n - (M - 1) * kPage);
    const float* mrow = mu + ((size_t)b * HQ + h) * MP;
    const float* srow = sigma + ((size_t)b * HQ + h) * MP;
    const bool staged = M <= lds_pages;
    float2* sub2 = lds2 + lds_pages;
    const int msub = (M + kTauSub - 1) / kTauSub;

    float xmax = -INFINITY;
    const bool vec = staged && ((((uintptr_t)mrow) | ((uintptr_t)srow)) & 15) == 0;
    if (vec) {
        // All 16-byte loads first (at most kTauLdsPages / (4 kTauThreads) = 4
        // per row and thread), with no branch between them, so that they are
        // in flight together; chunks past the full ones read chunk 0 and are
        // dropped.  Then the < 4 trailing pages one by one.
        constexpr int NV = kTauLdsPages / (4 * kTauThreads);
        const int nv = M >> 2;                   // full 4-page chunks
        float4 m4[NV], s4[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int c = (int)threadIdx.x + k * kTauThreads;
            const int cc = c < nv ? c : 0;
            if (nv > 0) {                        // block-uniform
                m4[k] = *reinterpret_cast<const float4*>(mrow + 4 * cc);
                s4[k] = *reinterpret_cast<const float4*>(srow + 4 * cc);
            }
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int c = (int)threadIdx.x + k * kTauThreads;
            if (c < nv) {
                const float xm[4] = {a * m4[k].x, a * m4[k].y, a * m4[k].z, a * m4[k].w};
                const float xs[4] = {a * s4[k].x, a * s4[k].y, a * s4[k].z, a * s4[k].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = 4 * c + i;
                    xmax = fmaxf(xmax, xm[i]);
                    lds2[p] = make_float2(xm[i], xs[i]);
                    if ((p & (kTauSub - 1)) == 0) sub2[p / kTauSub] = make_float2(xm[i], xs[i]);
                }
            }
        }
        const int p = 4 * nv + (int)threadIdx.x;
        if (p < M) {
            const float xm = a * mrow[p];
            xmax = fmaxf(xmax, xm);
            lds2[p] = make_float2(xm, a * srow[p]);
            if ((p & (kTauSub - 1)) == 0) sub2[p / kTauSub] = lds2[p];
        }
    } else {
        for (int p = threadIdx.x; p < M; p += kTauThreads) {
            const float xm = a * mrow[p];
            xmax = fmaxf(xmax, xm);
            if (staged) {
                lds2[p] = make_float2(xm, a * srow[p]);
                if ((p & (kTauSub - 1)) == 0) sub2[p / kTauSub] = lds2[p];
            }
        }
    }
    xmax = block_max<kTauWaves>(xmax, red, phase);   // barrier also publishes LDS
    const float lo = xmax - 1.0f;                    // F(lo) >= 1 (Jensen on the top page)
    float t = lo;
    const float wsub = (float)(kTauSub * kPage);
    if (staged && M >= kTauSubMin) {                 // no lower end known for the subsample
        __shared__ float sh_t;
        if (threadIdx.x < 64) {                      // wave 0 alone; the others wait at the barrier
            const float ts = gauss_tau_solve<BETA, true, true>(sub2, mrow, srow, msub, -1, wsub, wsub, a,
                                                               -INFINITY, lo, kTauSubTol, 0.0f, red, phase);
            if (threadIdx.x == 0) sh_t = ts;
        }
        __syncthreads();
        t = sh_t;
    }
    const float accept = BETA == 1 ? kTauAcceptNewton : kTauAcceptHalley;
    if (staged)
        t = gauss_tau_solve<BETA, false, true>(lds2, mrow, srow, M, M - 1, (float)kPage, last_np, a, lo, t,
                                               kTauTol, accept, red, phase);
    else
        t = gauss_tau_solve<BETA, false, false>(lds2, mrow, srow, M, M - 1, (float)kPage, last_np, a, lo, t,
                                                kTauTol, accept, red, phase);
    if (threadIdx.x == 0) *out = t;
}

// --------------------------------------------------------------- select ----
enum { kSelTopk = 0, kSelGauss = 1, kSelSuperset = 2 };

// Cutoff key of a (sequence, group): candidates are keys >= cut.
//  top-k: every page;  Gaussian: margin >= -z;
//  superset: box score >= min over the group's heads of tau_lo / (alpha-1),
//  lowered by 1e-5 relative so that fp32 rounding of the scores and of the
//  lower bound can only add pages, never drop one the exact rule keeps.
template <int MODE, int R>
__device__ __forceinline__ uint32_t select_cut(const float* __restrict__ tau_hat, size_t head0, float inv_a,
                                               float zcut) {
    if constexpr (MODE == kSelGauss) {
        return ord_key(-zcut);
    } else if constexpr (MODE == kSelSuperset) {
        float th = INFINITY;
#pragma unroll
        for (int j = 0; j < R; ++j) th = fminf(th, tau_hat[head0 + j]);
        th *= inv_a;
        th -= 1e-5f * fmaxf(1.0f, fabsf(th));
        return th > -INFINITY ? ord_key(th) : 0u;    // -inf or NaN: every page
    } else {
        return 0u;
    }
}


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

template <int MODE, int R>
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
    const uint32_t cut = select_cut<MODE, R>(tau_hat, (size_t)b * HQ + g * R, inv_a, zcut);
    float theta[R];
    if constexpr (MODE == kSelGauss) {
#pragma unroll
        for (int j = 0; j < R; ++j) theta[j] = tau_hat[(size_t)b * HQ + g * R + j] * inv_a;
    }
    float cnt = 0.0f;
    for (int p = threadIdx.x; p < M; p += kSelThreads) {
        float f;
        if constexpr (MODE == kSelGauss) {
            f = -INFINITY;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const size_t o = ((size_t)b * HQ + g * R + j) * MP + p;
                const float dm = mu[o] - theta[j];
                const float sg = sigma[o];
                const float t = sg > 0.0f ? dm * __builtin_amdgcn_rcpf(sg) : (dm > 0.0f ? INFINITY : -INFINITY);
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
                const int incl = wave_incl_scan(sum);
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

// KPT consecutive floats of `row` starting at p0 (entries at or past M read
// as 0 and are never used); 16-byte loads when the whole span is valid and
// aligned.
template <int KPT>
__device__ __forceinline__ void load_span(const float* __restrict__ row, int p0, int M, float (&v)[KPT]) {
    if (p0 + KPT <= M && ((uintptr_t)(row + p0) & 15) == 0) {
#pragma unroll
        for (int j = 0; j < KPT; j += 4) {
            const float4 x = *reinterpret_cast<const float4*>(row + p0 + j);
            v[j] = x.x;
            v[j + 1] = x.y;
            v[j + 2] = x.z;
            v[j + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) v[j] = p0 + j < M ? row[p0 + j] : 0.0f;
    }
}

// Keys of the KPT consecutive pages [p0, p0 + KPT) of row (b, g): the pooled
// box score (top-k, superset) or the pooled Gaussian margin.  Entries at or
// past M are filled but never used.
template <int MODE, int R, int KPT>
__device__ __forceinline__ void page_keys(const float* __restrict__ score, const float* __restrict__ mu,
                                          const float* __restrict__ sigma, const float* __restrict__ tau_hat,
                                          float inv_a, int b, int g, int G, int MP, int M, int p0,
                                          uint32_t (&key)[KPT]) {
    const int HQ = G * R;
    if constexpr (MODE == kSelGauss) {
        constexpr int C = KPT < 8 ? KPT : 8;      // pages per sub-chunk (bounds registers)
#pragma unroll
        for (int c0 = 0; c0 < KPT; c0 += C) {
            float f[C];
#pragma unroll
            for (int i = 0; i < C; ++i) f[i] = -INFINITY;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const size_t o = ((size_t)b * HQ + g * R + j) * MP;
                const float theta = tau_hat[(size_t)b * HQ + g * R + j] * inv_a;
                float m[C], sg[C];
                load_span<C>(mu + o, p0 + c0, M, m);
                load_span<C>(sigma + o, p0 + c0, M, sg);
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const float dm = m[i] - theta;
                    const float t = sg[i] > 0.0f ? dm * __builtin_amdgcn_rcpf(sg[i])
                                                 : (dm > 0.0f ? INFINITY : -INFINITY);
                    f[i] = fmaxf(f[i], t);
                }
            }
#pragma unroll
            for (int i = 0; i < C; ++i) key[c0 + i] = ord_key(f[i]);
        }
    } else {
        float f[KPT];
        load_span<KPT>(score + ((size_t)b * G + g) * MP, p0, M, f);
#pragma unroll
        for (int i = 0; i < KPT; ++i) key[i] = ord_key(f[i]);
    }
}

// The cutoff (T, need_eq) of a block-wide selection over keys in registers:
// the kept entries are those with key > T, then the first need_eq with
// key == T in entry order.  `ok(i)` tells which register entries exist.
// `ncand` is the number of keys at or above `cut` (the candidates) and
// `keep` the number to keep; with 1 <= ncand <= keep every candidate is kept.
// Otherwise the keep-th largest key is found by an 8-bit radix select; when
// ncand > keep the answer is a candidate, so only candidates are
// histogrammed, as offsets from the smallest (cmin; cmax the largest), and
// the first pass takes the top 8 bits of the candidates' own range.
// (ncand == 0: over every key.)
template <int KPT, typename Ok>
__device__ __forceinline__ void block_kth_key(const uint32_t (&key)[KPT], Ok ok, uint32_t cut, int ncand, int keep,
                                              uint32_t cmin, uint32_t cmax, int* hist, int* sh_digit,
                                              int* sh_above, uint32_t& T, int& need_eq) {
    if (ncand >= 1 && ncand <= keep) {
        T = cut;              // every candidate, nothing else
        need_eq = 0x7fffffff;
        return;
    }
    if (keep <= 0) {
        T = 0xffffffffu;
        need_eq = 0;
        return;
    }
    const bool all = ncand == 0;
    const uint32_t base = all ? 0u : cmin;
    const uint32_t span = all ? 0xffffffffu : cmax - cmin;
    const int nbits = span ? 32 - __builtin_clz(span) : 0;
    uint32_t prefix = 0;     // determined high bits of (key - base)
    int remaining = keep;
    int shift = nbits > 8 ? nbits - 8 : 0;
    int width = nbits > 8 ? 8 : nbits;
    while (width > 0) {
        for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        const int top = shift + width;
        const uint32_t hmask = top >= 32 ? 0u : (0xffffffffu << top);
        const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const uint32_t rel = key[i] - base;
            if (ok(i) && (all || key[i] >= cut) && (rel & hmask) == prefix)
                atomicAdd(&hist[(rel >> shift) & dmask], 1);
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            // Lane l holds digits 255-4l .. 252-4l (descending); the first
            // lane whose inclusive count reaches `remaining` walks its four.
            const int l = threadIdx.x;
            int c4[4], sum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c4[i] = hist[255 - 4 * l - i];
                sum += c4[i];
            }
            const int incl = wave_incl_scan(sum);
            const uint64_t hit = __ballot(incl >= remaining);
            const int L = hit ? (int)__builtin_ctzll(hit) : 63;
            if (l == L) {
                int above = incl - sum, dgt = 255 - 4 * l - 3;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (above + c4[i] >= remaining) { dgt = 255 - 4 * l - i; break; }
                    above += c4[i];
                }
                *sh_digit = dgt;
                *sh_above = above;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)*sh_digit << shift;
        remaining -= *sh_above;
        width = shift >= 8 ? 8 : shift;
        shift -= width;
    }
    T = base + prefix;
    need_eq = remaining;
}

// Compaction of the kept entries in entry order (thread t owns entries
// [t*KPT, (t+1)*KPT)): one block-wide scan of per-thread counts gives each
// kept entry its position; put(i, pos) is called for every kept entry with
// pos < cap.  Returns min(kept, cap) (block-uniform).
template <int KPT, typename Ok, typename Put>
__device__ __forceinline__ int block_compact(const uint32_t (&key)[KPT], Ok ok, uint32_t T, int need_eq, int cap,
                                             int* wsum, Put put) {
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (ok(i)) {
            ngt += key[i] > T ? 1 : 0;
            neq += key[i] == T ? 1 : 0;
        }
    }
    int egt, eeq, tgt, teq;
    block_excl_scan2<kSelWaves>(ngt, neq, egt, eeq, &tgt, &teq, wsum);
    int pos = egt + min(eeq, need_eq);
    int eq_rank = eeq;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (ok(i)) {
            const bool eq = key[i] == T;
            const bool take = key[i] > T || (eq && eq_rank < need_eq);
            eq_rank += eq ? 1 : 0;
            if (take) {
                if (pos < cap) put(i, pos);
                ++pos;
            }
        }
    }
    return min(tgt + min(teq, need_eq), cap);
}

// Candidates among the valid register keys (key >= cut): their count (block
// total, every thread) and key range.
template <int KPT, typename Ok>
__device__ __forceinline__ int block_candidates(const uint32_t (&key)[KPT], Ok ok, uint32_t cut, uint32_t& cmin,
                                                uint32_t& cmax, int* wsum) {
    int cnt = 0;
    cmin = 0xffffffffu;
    cmax = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (ok(i) && key[i] >= cut) {
            ++cnt;
            cmin = min(cmin, key[i]);
            cmax = max(cmax, key[i]);
        }
    }
    int ncand;
    block_count_range<kSelWaves>(cnt, cmin, cmax, &ncand, wsum);
    return ncand;
}

// Same selection as select_kernel with the keys held in registers: thread t
// owns the KPT consecutive pages [t*KPT, (t+1)*KPT), so one block-wide scan of
// per-thread counts places every kept page in ascending order.  Needs
// M <= KPT * kSelThreads.
template <int MODE, int R, int KPT>
__global__ __launch_bounds__(kSelThreads) void select_reg_kernel(
    const int32_t* __restrict__ seq_lens, int G, int MP, int budget, const float* __restrict__ score,
    const float* __restrict__ mu, const float* __restrict__ sigma, const float* __restrict__ tau_hat,
    float inv_a, float zcut, int32_t* __restrict__ sel_pages, int32_t* __restrict__ sel_count) {
    __shared__ int hist[256];
    __shared__ int wsum[3 * kSelWaves];
    __shared__ int sh_digit, sh_above;
    const int g = blockIdx.x, b = blockIdx.y;
    const int HQ = G * R;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    int32_t* out = sel_pages + ((size_t)b * G + g) * budget;
    const int p0 = threadIdx.x * KPT;
    auto ok = [&](int i) { return p0 + i < M; };

    uint32_t key[KPT];
    page_keys<MODE, R, KPT>(score, mu, sigma, tau_hat, inv_a, b, g, G, MP, M, p0, key);
    const uint32_t cut = select_cut<MODE, R>(tau_hat, (size_t)b * HQ + g * R, inv_a, zcut);
    uint32_t cmin, cmax;
    const int ncand = block_candidates<KPT>(key, ok, cut, cmin, cmax, wsum);
    const int keep = M == 0 ? 0 : max(1, min(budget, ncand));
    uint32_t T;
    int need_eq;
    block_kth_key<KPT>(key, ok, cut, ncand, keep, cmin, cmax, hist, &sh_digit, &sh_above, T, need_eq);
    const int written = block_compact<KPT>(key, ok, T, need_eq, budget, wsum,
                                           [&](int i, int pos) { out[pos] = p0 + i; });
    for (int i = written + threadIdx.x; i < budget; i += kSelThreads) out[i] = -1;
    if (threadIdx.x == 0) sel_count[(size_t)b * G + g] = written;
}

// Two-level selection for rows of many pages when there are few (sequence,
// group) rows to spread over the chip.  Under the order "larger key first,
// then lower page index", a page among the row's top `keep` is also among
// the top `keep` of any subset that contains it, in particular of its own
// chunk of kChunkPages pages.  So:
//  select_chunk_kernel (grid: chunks x G x B) keeps the top min(budget,
//    chunk) pages of each chunk, whatever the cutoff, as (key, page) entries
//    in page order, and counts the chunk's candidates (keys at or above the
//    cutoff);
//  select_merge_kernel (grid: G x B) applies the one-level rule (keep =
//    max(1, min(budget, candidates of the row))) to the union of the chunks'
//    entries.  The union is in page order, so ties still go to the lower page
//    and the output is ascending.
// The result is the one-level selection exactly.  Workspace per row:
// nchunk x budget entries (uint32 key, uint32 page), then nchunk counts
// (entries kept, candidates).
constexpr int kChunkPages = 4 * kSelThreads;
constexpr int kMergeMaxChunks = 256;       // chunks per row at most
constexpr int kMergeMaxEntries = 64 * kSelThreads;
constexpr int kTwoLevelRows = 256;         // two-level only below this many rows ...
constexpr int kTwoLevelMinPages = 8192;    // ... of more than this many pages

template <int MODE, int R>
__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(
    const int32_t* __restrict__ seq_lens, int G, int MP, int budget, const float* __restrict__ score,
    const float* __restrict__ mu, const float* __restrict__ sigma, const float* __restrict__ tau_hat,
    float inv_a, float zcut, int nchunk, uint2* __restrict__ entries, int2* __restrict__ counts) {
    constexpr int KPT = kChunkPages / kSelThreads;
    __shared__ int hist[256];
    __shared__ int wsum[3 * kSelWaves];
    __shared__ int sh_digit, sh_above;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int HQ = G * R;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    const size_t row = ((size_t)b * G + g) * nchunk + c;
    uint2* out = entries + row * budget;
    const int p0 = c * kChunkPages + threadIdx.x * KPT;
    auto ok = [&](int i) { return p0 + i < M; };

    uint32_t key[KPT];
    page_keys<MODE, R, KPT>(score, mu, sigma, tau_hat, inv_a, b, g, G, MP, M, p0, key);
    const uint32_t cut = select_cut<MODE, R>(tau_hat, (size_t)b * HQ + g * R, inv_a, zcut);
    uint32_t cmin, cmax;
    const int ncand = block_candidates<KPT>(key, ok, cut, cmin, cmax, wsum);
    // The chunk's own top pages: here every valid page counts as a candidate.
    uint32_t amin, amax;
    const int nvalid = block_candidates<KPT>(key, ok, 0u, amin, amax, wsum);
    const int keep = min(budget, nvalid);
    uint32_t T;
    int need_eq;
    block_kth_key<KPT>(key, ok, 0u, nvalid, keep, amin, amax, hist, &sh_digit, &sh_above, T, need_eq);
    const int written = block_compact<KPT>(key, ok, T, need_eq, budget, wsum, [&](int i, int pos) {
        out[pos] = make_uint2(key[i], (uint32_t)(p0 + i));
    });
    if (threadIdx.x == 0) counts[row] = make_int2(written, ncand);
}

template <int MODE, int R, int KPT>
__global__ __launch_bounds__(kSelThreads) void select_merge_kernel(
    const int32_t* __restrict__ seq_lens, int G, int MP, int budget, const float* __restrict__ tau_hat,
    float inv_a, float zcut, int nchunk, const uint2* __restrict__ entries, const int2* __restrict__ counts,
    int32_t* __restrict__ sel_pages, int32_t* __restrict__ sel_count) {
    __shared__ int hist[256];
    __shared__ int wsum[3 * kSelWaves];
    __shared__ int sh_digit, sh_above;
    __shared__ int sh_kept[kMergeMaxChunks];
    __shared__ int sh_ncand;
    const int g = blockIdx.x, b = blockIdx.y;
    const int HQ = G * R;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    const size_t row0 = ((size_t)b * G + g) * nchunk;
    int32_t* out = sel_pages + ((size_t)b * G + g) * budget;
    if (threadIdx.x < 64) {
        int nc = 0;
        for (int c = threadIdx.x; c < nchunk; c += 64) {
            const int2 k = counts[row0 + c];
            sh_kept[c] = k.x;
            nc += k.y;
        }
        nc = wave_isum(nc);
        if (threadIdx.x == 0) sh_ncand = nc;
    }
    __syncthreads();
    // Entry e = c * budget + i (chunk c, its i-th kept page): thread t owns
    // entries [t*KPT, (t+1)*KPT); slots past a chunk's kept count are empty.
    const int e0 = threadIdx.x * KPT;
    uint32_t key[KPT], page[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int e = e0 + i;
        const int c = e / budget;
        const bool v = c < nchunk && e - c * budget < sh_kept[c < nchunk ? c : 0];
        const uint2 x = v ? entries[row0 * budget + e] : make_uint2(0u, 0u);
        key[i] = x.x;
        page[i] = v ? x.y : 0xffffffffu;
    }
    auto ok = [&](int i) { return page[i] != 0xffffffffu; };
    const uint32_t cut = select_cut<MODE, R>(tau_hat, (size_t)b * HQ + g * R, inv_a, zcut);
    uint32_t cmin, cmax;
    (void)block_candidates<KPT>(key, ok, cut, cmin, cmax, wsum);
    const int ncand = sh_ncand;
    const int keep = M == 0 ? 0 : max(1, min(budget, ncand));
    uint32_t T;
    int need_eq;
    block_kth_key<KPT>(key, ok, cut, ncand, keep, cmin, cmax, hist, &sh_digit, &sh_above, T, need_eq);
    const int written = block_compact<KPT>(key, ok, T, need_eq, budget, wsum,
                                           [&](int i, int pos) { out[pos] = (int32_t)page[i]; });
    for (int i = written + threadIdx.x; i < budget; i += kSelThreads) out[i] = -1;
    if (threadIdx.x == 0) sel_count[(size_t)b * G + g] = written;
}

template <int BETA>
static hipError_t run_gauss_tau(const Dims& d, const float* mu, const float* sigma, const int32_t* seq_lens,
                                float a, float* tau_hat, hipStream_t s) {
    // (a*mu, a*sigma) are staged in LDS for sequences of up to kTauLdsPages
    // pages (64 KiB of the 160 KiB a gfx950 workgroup may use).  The kernel
    // attribute allowing that much dynamic LDS is set once per device.
    // The flag is atomic: concurrent first calls from several host threads
    // are well defined (setting the attribute twice is harmless).
    static std::atomic<bool> attr_ok[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const size_t max_lds = (size_t)(kTauLdsPages + kTauLdsPages / kTauSub) * sizeof(float2);
    if (!attr_ok[dev].load(std::memory_order_acquire)) {
        if (hipFuncSetAttribute((const void*)gauss_tau_kernel<BETA>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)max_lds) == hipSuccess)
            attr_ok[dev].store(true, std::memory_order_release);
        else
            (void)hipGetLastError();
    }
    const bool big = attr_ok[dev].load(std::memory_order_acquire);
    // lds_pages is a multiple of kTauSub: the subsample array follows the pages.
    int lds_pages = big ? (d.MP < kTauLdsPages ? d.MP : kTauLdsPages) : 0;
    if (!big && (size_t)d.MP * sizeof(float2) * (kTauSub + 1) / kTauSub <= 48 * 1024) lds_pages = d.MP;
    lds_pages = (lds_pages + kTauSub - 1) / kTauSub * kTauSub;
    const size_t lds = (size_t)(lds_pages + lds_pages / kTauSub) * sizeof(float2);
    gauss_tau_kernel<BETA><<<dim3(d.HQ, d.B), dim3(kTauThreads), lds, s>>>(
        mu, sigma, seq_lens, d.HQ, d.MP, a, lds_pages, tau_hat);
    return hipGetLastError();
}

hipError_t launch_gauss_tau(const Dims& d, const float* mu, const float* sigma,
                            const int32_t* seq_lens, float alpha, float* tau_hat, hipStream_t s) {
    const float a = alpha - 1.0f;
    switch ((int)lrintf(1.0f / a)) {
        case 1: return run_gauss_tau<1>(d, mu, sigma, seq_lens, a, tau_hat, s);
        case 2: return run_gauss_tau<2>(d, mu, sigma, seq_lens, a, tau_hat, s);
        case 3: return run_gauss_tau<3>(d, mu, sigma, seq_lens, a, tau_hat, s);
        default: return hipErrorInvalidValue;
    }
}

// Two-level selection (see select_chunk_kernel) when there are fewer rows
// than half the compute units' worth and rows are long: one block per row
// would leave most of the chip idle (65536-page rows of 8 groups took 71 us
// in one level, measured).  Needs a budget well below the chunk, and the
// chunks' entries of a row within the merge kernel's registers.
static int two_level_chunks(const Dims& d, int budget) {
    if ((long)d.B * d.G >= kTwoLevelRows || d.MP <= kTwoLevelMinPages || budget * 4 > kChunkPages) return 0;
    const int nchunk = (d.MP + kChunkPages - 1) / kChunkPages;
    if (nchunk > kMergeMaxChunks || (long)nchunk * budget > kMergeMaxEntries) return 0;
    return nchunk;
}

size_t select_keys_bytes(const Dims& d, int budget) {
    const size_t one = (size_t)d.B * d.G * d.MP * sizeof(uint32_t);
    const int nchunk = two_level_chunks(d, budget);
    const size_t rows = (size_t)d.B * d.G * nchunk;
    const size_t two = nchunk ? ((rows * budget * sizeof(uint2) + 255) & ~(size_t)255) + rows * sizeof(int2) : 0;
    return one > two ? one : two;
}

hipError_t launch_select(const Dims& d, int mode, const int32_t* seq_lens, float alpha,
                         int budget, float z, const float* score, const float* mu,
                         const float* sigma, const float* tau_hat, uint32_t* keys,
                         int32_t* sel_pages, int32_t* sel_count, hipStream_t s) {
    const float inv_a = alpha > 1.0f ? 1.0f / (alpha - 1.0f) : 0.0f;
    dim3 grid(d.G, d.B);
    const int nchunk = two_level_chunks(d, budget);
    if (nchunk) {
        const size_t rows = (size_t)d.B * d.G * nchunk;
        uint2* entries = reinterpret_cast<uint2*>(keys);
        int2* counts = reinterpret_cast<int2*>(reinterpret_cast<char*>(keys) +
                                               ((rows * budget * sizeof(uint2) + 255) & ~(size_t)255));
        int kpt = 4;
        while ((long)kpt * kSelThreads < (long)nchunk * budget) kpt *= 2;
        const dim3 grid1(nchunk, d.G, d.B);
#define EKV_TWO(MM, RR)                                                                                        \
    {                                                                                                          \
        select_chunk_kernel<MM, RR><<<grid1, dim3(kSelThreads), 0, s>>>(seq_lens, d.G, d.MP, budget, score,    \
                                                                        mu, sigma, tau_hat, inv_a, z, nchunk,  \
                                                                        entries, counts);                      \
        switch (kpt) {                                                                                         \
            case 4: select_merge_kernel<MM, RR, 4><<<grid, dim3(kSelThreads), 0, s>>>(                         \
                        seq_lens, d.G, d.MP, budget, tau_hat, inv_a, z, nchunk, entries, counts, sel_pages,    \
                        sel_count); break;                                                                     \
            case 8: select_merge_kernel<MM, RR, 8><<<grid, dim3(kSelThreads), 0, s>>>(                         \
                        seq_lens, d.G, d.MP, budget, tau_hat, inv_a, z, nchunk, entries, counts, sel_pages,    \
                        sel_count); break;                                                                     \
            case 16: select_merge_kernel<MM, RR, 16><<<grid, dim3(kSelThreads), 0, s>>>(                       \
                        seq_lens, d.G, d.MP, budget, tau_hat, inv_a, z, nchunk, entries, counts, sel_pages,    \
                        sel_count); break;                                                                     \
            case 32: select_merge_kernel<MM, RR, 32><<<grid, dim3(kSelThreads), 0, s>>>(                       \
                        seq_lens, d.G, d.MP, budget, tau_hat, inv_a, z, nchunk, entries, counts, sel_pages,    \
                        sel_count); break;                                                                     \
            default: select_merge_kernel<MM, RR, 64><<<grid, dim3(kSelThreads), 0, s>>>(                       \
                        seq_lens, d.G, d.MP, budget, tau_hat, inv_a, z, nchunk, entries, counts, sel_pages,    \
                        sel_count); break;                                                                     \
        }                                                                                                      \
        return hipGetLastError();                                                                              \
    }
#define EKV_TWOM(MM)                                         \
    switch (d.R) {                                           \
        case 1: EKV_TWO(MM, 1)                               \
        case 2: EKV_TWO(MM, 2)                               \
        case 4: EKV_TWO(MM, 4)                               \
        case 8: EKV_TWO(MM, 8)                               \
        default: return hipErrorInvalidValue;                \
    }
        if (mode == kSelGauss) { EKV_TWOM(kSelGauss) }
        if (mode == kSelSuperset) { EKV_TWOM(kSelSuperset) }
        EKV_TWO(kSelTopk, 1)
#undef EKV_TWOM
#undef EKV_TWO
    }
    // Keys in registers when every sequence fits KPT * kSelThreads pages.
    int kpt = 0;
    for (int k = 4; k <= 64; k *= 2)
        if ((long)k * kSelThreads >= d.MP) { kpt = k; break; }
#define EKV_SELR(MM, RR, KK)                                                                              \
    select_reg_kernel<MM, RR, KK><<<grid, dim3(kSelThreads), 0, s>>>(seq_lens, d.G, d.MP, budget, score,  \
                                                                     mu, sigma, tau_hat, inv_a, z,        \
                                                                     sel_pages, sel_count);               \
    return hipGetLastError();
#define EKV_SELK(MM, RR)                                     \
    switch (kpt) {                                           \
        case 4: { EKV_SELR(MM, RR, 4) }                      \
        case 8: { EKV_SELR(MM, RR, 8) }                      \
        case 16: { EKV_SELR(MM, RR, 16) }                    \
        case 32: { EKV_SELR(MM, RR, 32) }                    \
        case 64: { EKV_SELR(MM, RR, 64) }                    \
        default: break;                                      \
    }
#define EKV_SEL(MM, RR)                                                                              \
    select_kernel<MM, RR><<<grid, dim3(kSelThreads), 0, s>>>(seq_lens, d.G, d.MP, budget, score, mu, \
                                                             sigma, tau_hat, inv_a, z, keys,          \
                                                             sel_pages, sel_count);                   \
    return hipGetLastError();
#define EKV_SELM(MM)                                         \
    switch (d.R) {                                           \
        case 1: { EKV_SELK(MM, 1) EKV_SEL(MM, 1) }           \
        case 2: { EKV_SELK(MM, 2) EKV_SEL(MM, 2) }           \
        case 4: { EKV_SELK(MM, 4) EKV_SEL(MM, 4) }           \
        case 8: { EKV_SELK(MM, 8) EKV_SEL(MM, 8) }           \
        default: return hipErrorInvalidValue;                \
    }
    if (mode == kSelGauss) { EKV_SELM(kSelGauss) }
    if (mode == kSelSuperset) { EKV_SELM(kSelSuperset) }
    EKV_SELK(kSelTopk, 1)
    EKV_SEL(kSelTopk, 1)
#undef EKV_SELM
#undef EKV_SEL
#undef EKV_SELK
#undef EKV_SELR
}

}  // namespace ekv
