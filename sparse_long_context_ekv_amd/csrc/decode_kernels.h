// Kernels of the alpha-entmax decode over the selected pages ("EntmaxKV:
// Support-Aware Decoding for Entmax Attention", section 4.1; alpha-entmax of
// section 2.2; dropped mass of section 3.1).  x = (alpha - 1) s, and only
// x > max(x) - 1 can be in the support (the top term alone is at most 1).
// Three paths:
//
//  fused (alpha > 1, at most kFusedMaxSlots selected slots per head):
//   logits_kernel         grid (chunks of 8 selected pages, B*G): gathers each
//                         page-group K tile (16 tokens x D, contiguous)
//                         through the page table, one token per 16-lane row,
//                         and writes s = q.k/sqrt(D) for the group's r heads
//                         into a [B][HQ][slots] workspace (invalid slots -inf);
//   sparse_tau_pv_kernel  one block per (b, g): candidates, threshold
//                         (TauIter), support, PV over the support rows.
//  streamed (alpha > 1 otherwise: full cache, long selections): no logits are
//   kept; cand_stream_mfma_kernel (bf16 keys) or cand_stream_kernel ->
//   stream_tau_kernel -> support_pv_kernel -> reduce_kernel (see "streamed
//   entmax" below).
//  softmax (alpha = 1): bf16 keys in one pass, softmax_stream_kernel (keys
//   and values read once; running max and max-shifted sums per block) ->
//   softmax_merge_kernel; fp32 keys: logits_kernel with per-chunk (max,
//   sum exp(s - max), count) -> softmax_tau_kernel (log-partition) ->
//   pv_kernel (every slot, p = exp(s - tau)) -> reduce_kernel (fixed-order
//   sum of chunk partials).
// Bitwise reproducible: the one atomic (the bf16 candidate stream's running
// max, shared by a block's waves in LDS) only decides which extra entries
// below the final filter its lists hold, and the threshold kernel orders the
// candidates it keeps by list and slot.  (Past kCandCap candidates per head,
// where the threshold kernel reads the lists directly, sums may round
// differently from run to run.)
//
// This header is compiled once per KV element type (decode_bf16.hip,
// decode_f32.hip), so that the two sets of instantiations build in parallel.
#pragma once

#include "ekv_device.h"
#include "ekv_internal.h"

namespace ekv {

enum { kModeSoftmax = 0, kModeBeta1 = 1, kModeBeta2 = 2, kModeGeneral = 3 };
constexpr int kLogitUnroll = 4;
constexpr int kMaxLogitPpb = 64;       // pages per logits block at most (plan_decode: 8, 32 or 64)
constexpr int kCandCap = 8192;        // threshold candidates per head gathered in LDS (streamed path)

// -------------------------------------------------------------- logits ----
// Logits of a block's selected pages i0 .. i1-1, whose logical page and
// physical tile were resolved into sh_lp / sh_phys (indexed from i0; -1 =
// not readable): one token row per 16-lane row, the r heads' dot products
// by fixed-order row sums, s = q.k/sqrt(D) stored at st[(i - i0) * kPage]
// by lane j < R for head j (st already offset by the head and the row),
// -inf for tokens past the sequence end or on unreadable pages.  PART also
// keeps the row's running (max, sum exp(s - max), count) for head `lane`.
// UNROLL pages' tiles per row are in flight at once.
template <typename T, int D, int R, bool PART, int UNROLL = kLogitUnroll>
__device__ __forceinline__ void chunk_logits(const Vec<T, D / kRow> (&qv)[R], const T* __restrict__ k_cache,
                                             const int* sh_lp, const int* sh_phys, int i0, int i1, int ppb, int n,
                                             int G, int g, int lane, int row, float inv_sqrt_d, float* st,
                                             float& run_m, float& run_l, float& run_c) {
    constexpr int CH = D / kRow;
    constexpr int NW = Vec<T, CH>::NW;
    for (int i = i0; i < i1; i += UNROLL) {
        Vec<T, CH> kv[UNROLL];
        int lp[UNROLL], phys[UNROLL];
        bool ok[UNROLL];
        // Branch-free, so that all loads of the unroll are in flight at once
        // (a load under a per-page branch waits for the previous ones); an
        // empty slot reads page 0 and is ignored.
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int t = min(i + u - i0, ppb - 1);
            lp[u] = i + u < i1 ? sh_lp[t] : -1;
            phys[u] = sh_phys[t];
            ok[u] = lp[u] >= 0;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            kv[u].load(k_cache + (((size_t)(ok[u] ? phys[u] : 0) * G + g) * kPage + row) * D + lane * CH);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int ii = i + u;
            if (ii >= i1) break;                       // block-uniform
            float mine = -INFINITY;
            if (ok[u]) {                               // block-uniform
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    float acc = 0.0f;
                    if constexpr (std::is_same<T, float>::value) {
#pragma unroll
                        for (int c = 0; c < CH; ++c) acc = fmaf(qv[j].get(c), kv[u].get(c), acc);
                    } else {
#pragma unroll
                        for (int w = 0; w < NW; ++w)
                            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kv[u].w[w]),
                                                                  __builtin_bit_cast(bf16x2_t, qv[j].w[w]),
                                                                  acc, false);
                    }
                    acc = row_sum16(acc) * inv_sqrt_d;
                    mine = (lane == j) ? acc : mine;
                }
                if (lp[u] * kPage + row >= n) mine = -INFINITY;   // past the sequence end
            }
            if (lane < R) {
                st[(ii - i0) * kPage] = mine;
                if (PART && mine > -INFINITY) {
                    if (mine > run_m) {
                        run_l = run_l * expf(run_m - mine) + 1.0f;
                        run_m = mine;
                    } else {
                        run_l += expf(mine - run_m);
                    }
                    run_c += 1.0f;
                }
            }
        }
    }
}


// The same logits on the matrix cores, for bf16 keys: a page's 16 tokens
// against the group's r <= 8 queries is a small dense contraction,
// logits[head][token] = sum_c q[head][c] k[token][c], done by D/32
// v_mfma_f32_16x16x32_bf16 per page (rows = heads, padded to 16 with
// zeros; columns = the page's tokens).  In the MFMA's operand layout lane
// l (token or head t = l % 16, quarter h = l / 16) supplies the 8 channels
// 32 i + 8 h .. 32 i + 8 h + 7 of instruction i, so one load instruction
// of the wave reads 64 contiguous bytes of each of the page's 16 tokens,
// and the result leaves heads 4h .. 4h + 3 of token t in lane l.  Each
// wave takes every 4th page of the chunk, UNROLL pages in flight; results
// go to stage[head * stride + (page - i0) * 16 + token] (-inf past the
// sequence end or on an unreadable page).  Needs 256-thread blocks.
// The query operand: lane l holds channels 32 i + 8 (l / 16) .. + 7 of head
// l % 16 for instruction i (zeros for rows past the group's R heads).
template <int D, int R>
struct MfmaQ {
    bf16x8_t a[D / 32];
    __device__ __forceinline__ void load(const bf16_t* __restrict__ qrow) {
        static_assert(R <= 16 && D % 32 == 0, "one 16-row tile of heads, whole 32-channel slices");
        const int l = threadIdx.x & 63, tq = l & 15, hq = l >> 4;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
            const uint4 v = tq < R ? *reinterpret_cast<const uint4*>(qrow + (size_t)tq * D + 32 * t + 8 * hq)
                                   : make_uint4(0u, 0u, 0u, 0u);
            a[t] = __builtin_bit_cast(bf16x8_t, v);
        }
    }
};

// UNROLL pages of one wave in registers: pages i, i + NW, ..., i + NW (UNROLL
// - 1) of the chunk [i0, i1), NW = the waves that share the chunk.  load() issues every read without branches (a
// page past the chunk or unreadable reads page 0 and is ignored); logits()
// contracts them with the query tile and writes stage[head * stride +
// (page - i0) * 16 + token].
template <int D, int UNROLL, int NW = 4>
struct MfmaKPages {
    bf16x8_t kb[UNROLL][D / 32];
    bool ok[UNROLL];
    int lp[UNROLL];

    __device__ __forceinline__ void load(const bf16_t* __restrict__ k_cache, const int* sh_lp, const int* sh_phys,
                                         int i, int i0, int i1, int G, int g) {
        const int l = threadIdx.x & 63, tq = l & 15, hq = l >> 4;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int ii = i + NW * u;
            const int t = ii < i1 ? ii - i0 : 0;
            const int ph = sh_phys[t];
            lp[u] = sh_lp[t];
            ok[u] = ii < i1 && ph >= 0;
            const bf16_t* src = k_cache + (((size_t)(ok[u] ? ph : 0) * G + g) * kPage + tq) * D + 8 * hq;
#pragma unroll
            for (int t2 = 0; t2 < D / 32; ++t2)
                kb[u][t2] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(src + 32 * t2));
        }
    }

    // Every page's 16 x 16 product (pages past the chunk too: their reads
    // were of page 0 and the caller ignores them), no branches.
    template <int R>
    __device__ __forceinline__ void contract(const MfmaQ<D, R>& q, f32x4_t (&acc)[UNROLL]) const {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            acc[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t2 = 0; t2 < D / 32; ++t2)
                acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[t2], kb[u][t2], acc[u], 0, 0, 0);
        }
    }

    template <int R>
    __device__ __forceinline__ void logits(const MfmaQ<D, R>& q, int i, int i0, int i1, int n, float inv_sqrt_d,
                                           float* stage, int stride) const {
        const int l = threadIdx.x & 63, tq = l & 15, hq = l >> 4;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int ii = i + NW * u;
            if (ii < i1) {                                          // wave-uniform
                f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t2 = 0; t2 < D / 32; ++t2)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[t2], kb[u][t2], acc, 0, 0, 0);
                const bool live = ok[u] && lp[u] * kPage + tq < n;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int head = 4 * hq + j;
                    if (head < R)
                        stage[head * stride + (ii - i0) * kPage + tq] = live ? acc[j] * inv_sqrt_d : -INFINITY;
                }
            }
        }
    }
};

template <int D, int R, int UNROLL, int NW = 4>
__device__ __forceinline__ void chunk_logits_mfma(const bf16_t* __restrict__ qrow, const bf16_t* __restrict__ k_cache,
                                                  const int* sh_lp, const int* sh_phys, int i0, int i1, int n, int G,
                                                  int g, float inv_sqrt_d, float* stage, int stride) {
    MfmaQ<D, R> qa;
    qa.load(qrow);
    for (int i = i0 + (int)(threadIdx.x >> 6); i < i1; i += NW * UNROLL) {    // wave-uniform
        MfmaKPages<D, UNROLL, NW> kp;
        kp.load(k_cache, sh_lp, sh_phys, i, i0, i1, G, g);
        kp.template logits<R>(qa, i, i0, i1, n, inv_sqrt_d, stage, stride);
    }
}

// PART: also keep per-chunk (max, sum exp(s - max), valid count) per head,
// which the general threshold kernel reads (softmax, full cache).  NWV: waves
// per block; 8 (64 pages, four per wave per round on the matrix cores, two
// blocks per CU) only for bf16 keys without partials, so that the selected
// logits of a 128-unit batch take one round of blocks: a block's time is its
// chain of dependent loads (selection -> page table -> K tile), and 64 pages
// per block amortise it.
template <typename T, int D, int R, bool PART, int NWV = 4>
__global__ __launch_bounds__(64 * NWV) void logits_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_count, int sel_stride, int G, int MP, int NP, int lg_ppb,
    int nslot, int nchunk1, float inv_sqrt_d, float* __restrict__ logits, float* __restrict__ part1) {
    constexpr int CH = D / kRow;
    extern __shared__ float stage[];           // [R][ppb * kPage] logits of this chunk
    __shared__ float sh_m[kRow][R], sh_l[kRow][R], sh_c[kRow][R];
    __shared__ int sh_lp[kMaxLogitPpb], sh_phys[kMaxLogitPpb];
    const int ppb = 1 << lg_ppb;
    const int unit = blockIdx.y;
    const int b = unit / G, g = unit - b * G;
    const int HQ = G * R;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    const int cnt = sel_pages ? min(max(sel_count[unit], 0), sel_stride) : M;
    const int i0 = blockIdx.x * ppb;
    const int i1 = min(cnt, i0 + ppb);
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;          // token within the page

    Vec<T, CH> qv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qv[j].load(q + ((size_t)b * HQ + g * R + j) * D + lane * CH);

    float* st = stage + ((lane < R ? lane : 0) << (lg_ppb + 4)) + row;   // lane j < R: head j
    float run_m = -INFINITY, run_l = 0.0f, run_c = 0.0f;
    const int32_t* sel = sel_pages ? sel_pages + (size_t)unit * sel_stride : nullptr;

    // The chunk's pages: logical index and physical tile, resolved once (one
    // selection -> page-table chain per block instead of one per page and row).
    for (int t = threadIdx.x; t < ppb; t += blockDim.x) {
        const int ii = i0 + t;
        const int lp = ii < i1 ? (sel ? sel[ii] : ii) : -1;
        const int phys = (lp >= 0 && lp < M) ? page_table[(size_t)b * MP + lp] : -1;
        const bool ok = phys >= 0 && phys < NP;
        sh_lp[t] = ok ? lp : -1;
        sh_phys[t] = ok ? phys : -1;
    }
    __syncthreads();

    static_assert(NWV == 4 || (!PART && std::is_same<T, bf16_t>::value), "8-wave blocks: bf16 keys, no partials");
    if constexpr (!PART && std::is_same<T, bf16_t>::value) {
        chunk_logits_mfma<D, R, (NWV == 4 ? 2 : 4), NWV>(q + ((size_t)b * HQ + g * R) * D, k_cache, sh_lp, sh_phys,
                                                          i0, i1, n, G, g, inv_sqrt_d, stage, ppb * kPage);
    } else {
        chunk_logits<T, D, R, PART>(qv, k_cache, sh_lp, sh_phys, i0, i1, ppb, n, G, g, lane, row, inv_sqrt_d, st,
                                    run_m, run_l, run_c);
    }
    if (PART && lane < R) {
        sh_m[row][lane] = run_m;
        sh_l[row][lane] = run_l;
        sh_c[row][lane] = run_c;
    }
    __syncthreads();
    // One contiguous run of (i1 - i0) * 16 slots per head.
    const int nsl = max(i1 - i0, 0) * kPage;
    const int per_head = ppb * kPage;
    for (int t = threadIdx.x; t < R * per_head; t += blockDim.x) {
        const int j = t >> (lg_ppb + 4), r = t & (per_head - 1);
        if (r < nsl) logits[((size_t)b * HQ + g * R + j) * nslot + i0 * kPage + r] = stage[t];
    }
    if (PART && threadIdx.x < R) {
        const int j = threadIdx.x;
        float m = -INFINITY;
        for (int r2 = 0; r2 < kRow; ++r2) m = fmaxf(m, sh_m[r2][j]);
        float l = 0.0f, c = 0.0f;
        for (int r2 = 0; r2 < kRow; ++r2) {
            if (sh_m[r2][j] > -INFINITY) l += sh_l[r2][j] * expf(sh_m[r2][j] - m);
            c += sh_c[r2][j];
        }
        float* o = part1 + (((size_t)b * HQ + g * R + j) * nchunk1 + blockIdx.x) * 3;
        o[0] = m;
        o[1] = l;
        o[2] = c;
    }
}

// ----------------------------------------------------------------- tau ----
__device__ __forceinline__ float powb(float d, int mode, float beta) {
    return mode == kModeBeta1 ? d : (mode == kModeBeta2 ? d * d : powf(d, beta));
}

// State of the threshold iteration of one head for beta >= 1, where
// F(t) = sum_j [x_j - t]_+^beta is decreasing and G = F^(1/beta), the L^beta
// norm of (x - t)_+, is convex, so that:
//  * from a point left of the root (F >= 1) a Newton step on G rises and
//    never passes the root;
//  * from a point right of the root (F < 1) the Newton (tangent) step on G
//    lands at or left of the root.
// The iteration may therefore start anywhere in [max - 1, max) (e.g. at the
// Gaussian threshold estimate of the full cache); it keeps the best point
// known to lie left of the root (tl) and right of it (tr).  For beta = 1 and
// 2 every step first tries the closed form on the current support
// S = {x > t}: with d = x - t over S, s1 = sum d^beta, s0 = sum d^(beta-1),
// k = |S|,
//     beta = 1:  tau = t + (s1 - 1)/k,
//     beta = 2:  tau = t + m - sqrt((1 - V)/k),  m = s0/k, V = s1 - s0 m
//                (V the centred sum of squares of S, which must be <= 1),
// and accepts it when it is consistent with S (min_S x > tau >= every other
// candidate): the threshold is unique, so a consistent value is exact.
struct TauIter {
    float t, tl, tr, tau;
    bool done;
};

__device__ __forceinline__ TauIter tau_iter_start(float lo, float xmax, float hint, bool empty) {
    TauIter st;
    st.t = (hint > lo && hint < xmax) ? hint : lo;   // a NaN or out-of-bracket hint starts at lo
    st.tl = -INFINITY;
    st.tr = INFINITY;
    st.tau = lo;
    st.done = empty;
    return st;
}

// One step, given at st.t the sums over the candidates x > lo: s1, s0, k as
// above, mn = min of the candidates above t, rest = max of those at or below.
template <int MODE>
__device__ __forceinline__ void tau_iter_step(TauIter& st, float lo, float beta, float s1, float s0, float k,
                                              float mn, float rest) {
    const float t = st.t;
    if constexpr (MODE == kModeBeta1 || MODE == kModeBeta2) {
        if (k > 0.0f) {
            const float rk = hw_rcp(k);
            float tcf;
            if constexpr (MODE == kModeBeta1) {
                tcf = t + (s1 - 1.0f) * rk;
            } else {
                const float m = s0 * rk;
                const float v = fmaf(-s0, m, s1);
                tcf = v <= 1.0f ? t + m - hw_sqrt((1.0f - v) * rk) : NAN;
            }
            if (mn > tcf && !(rest > tcf)) {
                st.tau = tcf;
                st.done = true;
                return;
            }
        }
    }
    if (!(s1 > 0.0f) || !(s0 > 0.0f)) {
        // nothing above t: a start at or above every candidate; restart at lo
        if (t > lo) {
            st.t = lo;
        } else {
            st.tau = t;
            st.done = true;
        }
        return;
    }
    const float g = MODE == kModeBeta1 ? s1 : (MODE == kModeBeta2 ? hw_sqrt(s1) : hw_pow(s1, hw_rcp(beta)));
    const float nt = t + (1.0f - hw_rcp(g)) * s1 * hw_rcp(s0);
    if (s1 >= 1.0f) {                       // at or left of the root
        st.tl = t;
        if (!(nt > t)) {                    // no progress at fp32 resolution
            st.tau = t;
            st.done = true;
        } else if (!(nt < st.tr)) {         // the root lies in [t, tr] and the step says it is at tr
            st.tau = st.tr;
            st.done = true;
        } else {
            st.t = nt;
        }
    } else {                                // right of the root: the tangent step lands at or left of it
        st.tr = t;
        const float nl = fmaxf(nt, fmaxf(lo, st.tl));
        if (st.tl > -INFINITY || !(nl < t)) {
            // a step from the left passed the root by rounding (the only way
            // back to the right side), or no step is left: the tangent point,
            // or the last left point if that is nearer, is within rounding of
            // the root
            st.tau = nl < t ? nl : t;
            st.done = true;
        } else {
            st.t = nl;
        }
    }
}

// Softmax (alpha = 1): the log-partition log sum_j exp(s_j) from the
// logits kernel's chunk partials (max, sum exp(s - max), count), combined in
// a fixed order; every valid token is in the support, and the kept mass
// under tau_ref is sum_j exp(s_j - tau_ref).  grid (HQ, B).
static __global__ __launch_bounds__(256) void softmax_tau_kernel(
    const float* __restrict__ part1, int HQ, int nchunk1, const float* __restrict__ tau_ref,
    float* __restrict__ tau_out, int32_t* __restrict__ support_out, float* __restrict__ delta_out,
    int32_t* __restrict__ supref_out) {
    __shared__ float red[8];
    int phase = 0;
    const int h = blockIdx.x, b = blockIdx.y;
    const size_t oh = (size_t)b * HQ + h;
    const float* pm = part1 + oh * nchunk1 * 3;
    float mx = -INFINITY;
    for (int c = threadIdx.x; c < nchunk1; c += 256) mx = fmaxf(mx, pm[c * 3]);
    mx = block_max<4>(mx, red, phase);
    float L = 0.0f, C = 0.0f;
    for (int c = threadIdx.x; c < nchunk1; c += 256) {
        const float m = pm[c * 3];
        if (m > -INFINITY) L += pm[c * 3 + 1] * expf(m - mx);
        C += pm[c * 3 + 2];
    }
    L = block_sum<4>(L, red, phase);
    C = block_sum<4>(C, red, phase);
    if (!(C > 0.0f)) {
        if (threadIdx.x == 0) {
            tau_out[oh] = -INFINITY;
            if (support_out) support_out[oh] = 0;
            if (delta_out) delta_out[oh] = 1.0f;
            if (supref_out) supref_out[oh] = 0;
        }
        return;
    }
    const float tref = tau_ref ? tau_ref[oh] : 0.0f;
    float kept = 0.0f;
    if (delta_out) {
        for (int c = threadIdx.x; c < nchunk1; c += 256) {
            const float m = pm[c * 3];
            if (m > -INFINITY) kept += pm[c * 3 + 1] * expf(m - tref);
        }
        kept = block_sum<4>(kept, red, phase);
    }
    if (threadIdx.x == 0) {
        tau_out[oh] = mx + logf(L);
        if (support_out) support_out[oh] = (int32_t)C;
        if (delta_out) delta_out[oh] = 1.0f - kept;
        if (supref_out) supref_out[oh] = (int32_t)C;      // softmax: every token has p > 0
    }
}

// --------------------------------------------- streamed entmax (general) ----
// alpha > 1 over the full cache or over a selection past the fused kernel's
// slots.  No logits are kept: only x > max(x) - 1 can be in the support (the
// top term alone is at most 1), so
//   cand_stream_kernel  grid (splits * B*G): a block walks a contiguous range
//                       of up to kStreamMaxChunks chunks of kStreamPpb pages,
//                       computes the r heads' logits of each chunk in LDS and
//                       keeps, per head, the chunk's x > (running max) - 1,
//                       the running max being the largest x of the block's
//                       chunks so far: every x > (global max) - 1 is kept,
//                       and the filter tightens as the block goes.  Output per
//                       (b, h, split): the list (x, slot) in slot order, its
//                       count and the block's max;
//   cand_stream_mfma_kernel  the same for bf16 keys, on the matrix cores, one
//                       list per wave (described at the kernel);
//   stream_tau_kernel   grid (HQ, B): global max from the list maxima; the
//                       lists read by flat index (all threads, independent
//                       loads), candidates above (global max) - 1 gathered
//                       into LDS (or read from the lists when they do not
//                       fit); the threshold by TauIter, support size, dropped
//                       mass, and the support list (p, slot);
//   support_pv_kernel   grid (kSupSplit, HQ, B): V rows of the support only,
//                       partial sums per split, summed by reduce_kernel.
constexpr int kStreamPpb = 32;                        // pages per chunk
constexpr int kStreamSlots = kStreamPpb * kPage;      // 512 slots per chunk
constexpr int kStreamMaxChunks = 64;                  // chunks per candidate-stream block at most
constexpr int kStreamMaxLists = 2048;                 // candidate lists per (b, h) at most (4 per block)
constexpr int kStreamStage = 1536;                    // candidates staged in LDS per wave (bf16 stream; 65 KiB per block)
constexpr int kTauT = 512;                            // threads of the streamed threshold kernel (2 blocks per CU)
constexpr int kTauWaveCands = 2048;                   // at most this many candidates: one wave iterates
constexpr int kTauW = kTauT / 64;
constexpr int kStreamBlocks = 512;                    // aim: about this many candidate-stream blocks (2 per CU)
constexpr int kStreamRaggedChunks = 24;               // chunks per block at most on a ragged batch
constexpr int kSupSplit = 8;                          // PV blocks per head over its support
constexpr int kStreamUnroll = 8;                      // pages' tiles in flight per row while streaming

// The batch's sequences by length, longest first (ties: lower index first):
// order[rank] = b, where rank_b counts the sequences that go before b.
// Batches of at most kOrderLdsB sequences: every candidate-stream block
// computes the order itself into LDS (B^2 / 256 steps per thread);
// larger ones: this one-block kernel, once (B^2 / 1024 steps per thread, so
// batches past kOrderMaxB keep their order).
constexpr int kOrderLdsB = 256;
constexpr int kOrderMaxB = 4096;

// The b of rank `rank`: from `order` (device, larger batches) or computed
// into `sh` by the block (ends with a barrier).
__device__ __forceinline__ int stream_seq(const int32_t* __restrict__ seq_lens, int B, int MP,
                                          const int32_t* __restrict__ order, int rank, int* sh) {
    if (B > kOrderLdsB) return order[rank];
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int nb = seq_len_at(seq_lens, b, MP);
        int r = 0;
        for (int c = 0; c < B; ++c) {
            const int nc = seq_len_at(seq_lens, c, MP);
            r += (nc > nb || (nc == nb && c < b)) ? 1 : 0;
        }
        sh[r] = b;
    }
    __syncthreads();
    return sh[rank];
}
static __global__ __launch_bounds__(1024) void order_by_length_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                                      int MP, int32_t* __restrict__ order) {
    if (B > kOrderMaxB) {
        for (int b = threadIdx.x; b < B; b += blockDim.x) order[b] = b;
        return;
    }
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int nb = seq_len_at(seq_lens, b, MP);
        int rank = 0;
        for (int c = 0; c < B; ++c) {
            const int nc = seq_len_at(seq_lens, c, MP);
            rank += (nc > nb || (nc == nb && c < b)) ? 1 : 0;
        }
        order[rank] = b;
    }
}

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void cand_stream_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_count, int sel_stride, int B, int G, int MP, int NP, int cpb, int nsplit,
    const int32_t* __restrict__ order, float inv_sqrt_d, float a, float2* __restrict__ cands,
    int32_t* __restrict__ ccount, float* __restrict__ cmax) {
    constexpr int CH = D / kRow;
    constexpr int JPW = (R + 3) / 4;                     // heads per wave
    constexpr int XPL = kStreamSlots / 64;
    __shared__ float stage[R * kStreamSlots];            // [R][slots] logits of the current chunk
    __shared__ int sh_lp[kStreamMaxChunks * kStreamPpb], sh_phys[kStreamMaxChunks * kStreamPpb];
    // Block order: group fastest, then split, then sequence, so the G blocks
    // that run side by side read the same logical pages of one sequence (the
    // G tiles of a physical page are adjacent in the cache); sequences
    // longest first (`order`), so that on a ragged batch the long sequences'
    // blocks start first and the short ones fill in behind them.
    __shared__ int sh_order[kOrderLdsB];
    const int g = blockIdx.x % G, rest = blockIdx.x / G;
    const int split = rest % nsplit, b = stream_seq(seq_lens, B, MP, order, rest / nsplit, sh_order);
    const int unit = b * G + g;
    const int HQ = G * R;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    const int cnt = sel_pages ? min(max(sel_count[unit], 0), sel_stride) : M;
    const int span = cpb * kStreamPpb;              // <= kStreamMaxChunks * kStreamPpb (the plan's cap)
    const int p0 = split * span;
    const int p1 = span <= kStreamMaxChunks * kStreamPpb ? min(cnt, p0 + span) : p0;   // else: an empty range
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;
    const int wv = threadIdx.x >> 6, l64 = threadIdx.x & 63;
    const size_t lcap = (size_t)span * kPage;             // list capacity: every slot of the range

    Vec<T, CH> qv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qv[j].load(q + ((size_t)b * HQ + g * R + j) * D + lane * CH);
    // Every page of the range resolved at once (selection -> page table).
    const int32_t* sel = sel_pages ? sel_pages + (size_t)unit * sel_stride : nullptr;
    for (int t = threadIdx.x; t < min(span, kStreamMaxChunks * kStreamPpb); t += blockDim.x) {
        const int ii = p0 + t;
        const int lp = ii < p1 ? (sel ? sel[ii] : ii) : -1;
        const int phys = (lp >= 0 && lp < M) ? page_table[(size_t)b * MP + lp] : -1;
        const bool ok = phys >= 0 && phys < NP;
        sh_lp[t] = ok ? lp : -1;
        sh_phys[t] = ok ? phys : -1;
    }
    __syncthreads();

    float rmax[JPW];
    int rcnt[JPW];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
        rmax[jj] = -INFINITY;
        rcnt[jj] = 0;
    }
    float* st = stage + (lane < R ? lane : 0) * kStreamSlots + row;
    for (int c = 0; c < cpb; ++c) {
        const int i0 = p0 + c * kStreamPpb;
        if (i0 >= p1) break;                                 // block-uniform
        const int i1 = min(p1, i0 + kStreamPpb);
        float rm = -INFINITY, rl = 0.0f, rc = 0.0f;
        chunk_logits<T, D, R, false, kStreamUnroll>(qv, k_cache, sh_lp + c * kStreamPpb, sh_phys + c * kStreamPpb,
                                                    i0, i1, kStreamPpb, n, G, g, lane, row, inv_sqrt_d, st, rm, rl,
                                                    rc);
        __syncthreads();
        const int nsl = (i1 - i0) * kPage;
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            const int j = wv + 4 * jj;
            if (j >= R) break;                               // wave-uniform
            const float* sj = stage + j * kStreamSlots;
            float xs[XPL];
            float m = -INFINITY;
#pragma unroll
            for (int k = 0; k < XPL; ++k) {
                const int idx = k * 64 + l64;
                xs[k] = idx < nsl ? a * sj[idx] : -INFINITY;
                m = fmaxf(m, xs[k]);
            }
            rmax[jj] = fmaxf(rmax[jj], wave_max(m));
            const float lo = rmax[jj] - 1.0f;               // -inf: nothing valid yet
            float2* dst = cands + (((size_t)b * HQ + g * R + j) * nsplit + split) * lcap;
#pragma unroll
            for (int k = 0; k < XPL; ++k) {
                const bool f = xs[k] > lo;
                const uint64_t bal = __ballot(f);
                if (f) dst[rcnt[jj] + lanes_below(bal)] = make_float2(xs[k], __int_as_float(i0 * kPage + k * 64 + l64));
                rcnt[jj] += __popcll(bal);
            }
        }
        __syncthreads();                                     // the stage is rewritten by the next chunk
    }
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
        const int j = wv + 4 * jj;
        if (j < R && l64 == 0) {
            const size_t rcx = ((size_t)b * HQ + g * R + j) * nsplit + split;
            ccount[rcx] = rcnt[jj];
            cmax[rcx] = rmax[jj];
        }
    }
}

// bf16 keys: the same filter with every wave on its own pages (pages
// p0 + w, p0 + w + 4, ... of the block's range, in steps of 8 pages, on the
// matrix cores) and its own list per head, so that after the page table is
// resolved no barrier couples the block's waves: each keeps its next
// step's reads in flight while it takes this step's candidates.  The
// candidates are staged in LDS (kStreamStage entries per wave, split over
// the r heads) and copied out only when this step could overflow a buffer
// (before the next step's reads are issued, so that the wait for those
// reads does not also wait for fresh stores) and at the end.  The running
// max is shared by the block's waves through an LDS atomic max (any value
// read is a logit of the block, so still every x > (global max) - 1 is
// kept).  Lists per (b, h, split, wave) of capacity cpb * 128 slots, in
// slot order.
template <int D, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void cand_stream_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_count, int sel_stride, int B, int G, int MP, int NP, int cpb, int nsplit,
    const int32_t* __restrict__ order, float inv_sqrt_d, float a, float2* __restrict__ cands,
    int32_t* __restrict__ ccount, float* __restrict__ cmax) {
    constexpr int KPW = R <= 4 ? 8 : 4;                  // pages per wave per step (32 or 16 KiB in flight)
    constexpr int SP = 4 * KPW;                          // pages per block step
    constexpr int CB = kStreamStage / R;                 // staged candidates per (wave, head)
    constexpr int NR = (R + 3) / 4;                      // rows of lanes that hold heads
    static_assert(CB >= 2 * KPW * kPage, "a step adds at most KPW * 16 candidates per head");
    static_assert(kStreamPpb % (4 * KPW) == 0, "whole steps per chunk");
    __shared__ float2 stage[4][kStreamStage];
    __shared__ uint32_t smax[R];                         // the block's running max per head (ord_key)
    __shared__ int sh_lp[kStreamMaxChunks * kStreamPpb], sh_phys[kStreamMaxChunks * kStreamPpb];
    // Block order: group fastest, then split, then sequence, longest first
    // (see cand_stream_kernel).
    __shared__ int sh_order[kOrderLdsB];
    const int g = blockIdx.x % G, rest = blockIdx.x / G;
    const int split = rest % nsplit, b = stream_seq(seq_lens, B, MP, order, rest / nsplit, sh_order);
    const int unit = b * G + g;
    const int HQ = G * R;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    const int cnt = sel_pages ? min(max(sel_count[unit], 0), sel_stride) : M;
    const int span = cpb * kStreamPpb;              // <= kStreamMaxChunks * kStreamPpb (the plan's cap)
    const int p0 = split * span;
    const int p1 = span <= kStreamMaxChunks * kStreamPpb ? min(cnt, p0 + span) : p0;   // else: an empty range
    const int32_t* sel = sel_pages ? sel_pages + (size_t)unit * sel_stride : nullptr;
    for (int t = threadIdx.x; t < min(span, kStreamMaxChunks * kStreamPpb); t += blockDim.x) {
        const int ii = p0 + t;
        const int lp = ii < p1 ? (sel ? sel[ii] : ii) : -1;
        const int phys = (lp >= 0 && lp < M) ? page_table[(size_t)b * MP + lp] : -1;
        const bool ok = phys >= 0 && phys < NP;
        sh_lp[t] = ok ? lp : -1;
        sh_phys[t] = ok ? phys : -1;
    }
    if (threadIdx.x < R) smax[threadIdx.x] = ord_key(-INFINITY);
    __syncthreads();

    // Lane l: token tq = l % 16 of a page, heads 4 hq .. 4 hq + 3 (hq = l / 16).
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, tq = l & 15, hq = l >> 4;
    const size_t lcap = (size_t)cpb * (kStreamPpb / 4) * kPage;   // a quarter of the range's slots
    const uint32_t below = (1u << tq) - 1u;
    float rmax[4];
    int rcnt[4], scnt[4];                                  // copied out / staged (the row's head)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        rmax[j] = -INFINITY;
        rcnt[j] = 0;
        scnt[j] = 0;
    }
    // the row's staging buffers: head 4 hq + j at buf + j * CB
    float2* const buf = &stage[wv][min(4 * hq, R - 1) * CB];
    // A full stage (or the end): by the whole wave, head by head (only this
    // wave touches its stage; head h's counts live in row h / 4, register
    // h % 4), first drop the staged x <= (block max so far) - 1, compacting
    // in place; then, at the end or if the stage is still too full, copy it
    // out to the wave's list.
    auto flush = [&](bool last) {
#pragma unroll
        for (int h = 0; h < R; ++h) {
            const int jr = h & 3, rl = 16 * (h >> 2);
            const int c = __builtin_amdgcn_readlane(scnt[jr], rl);
            const float m = fmaxf(readlane(rmax[jr], rl),
                                  ord_unkey(__hip_atomic_load(&smax[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)));
            const float lo = m - 1.0f;
            float2* const src = &stage[wv][h * CB];
            int keep = 0;
            for (int e0 = 0; e0 < c; e0 += 4 * 64) {        // wave-uniform
                float2 v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int e = e0 + k * 64 + l;
                    v[k] = src[e < c ? e : 0];
                }
                // every read of the batch is issued before its first write,
                // and a kept entry only moves down
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const bool kf = e0 + k * 64 + l < c && v[k].x > lo;
                    const uint64_t bal = __ballot(kf);
                    if (kf) src[keep + lanes_below(bal)] = v[k];
                    keep += __popcll(bal);
                }
            }
            int r0 = __builtin_amdgcn_readlane(rcnt[jr], rl);
            if (last || keep > CB - KPW * kPage) {               // wave-uniform
                float2* dst = cands + ((((size_t)b * HQ + g * R + h) * nsplit + split) * 4 + wv) * lcap + r0;
                for (int e0 = 0; e0 < keep; e0 += 4 * 64) {
                    float2 v[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int e = e0 + k * 64 + l;
                        v[k] = src[e < keep ? e : 0];
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (e0 + k * 64 + l < keep) dst[e0 + k * 64 + l] = v[k];
                }
                r0 += keep;
                keep = 0;
            }
            if ((l >> 4) == (h >> 2)) {
                scnt[jr] = keep;
                rcnt[jr] = r0;
                rmax[jr] = fmaxf(rmax[jr], m);
            }
        }
    };
    MfmaQ<D, R> mq;
    mq.load(q + ((size_t)b * HQ + g * R) * D);
    MfmaKPages<D, KPW> kp;
    if (p0 < p1) kp.load(k_cache, sh_lp, sh_phys, p0 + wv, p0, min(p1, p0 + SP), G, g);
    for (int i0 = p0; i0 < p1; i0 += SP) {                  // block-uniform
        const int i1 = min(p1, i0 + SP);
        f32x4_t acc[KPW];
        kp.template contract<R>(mq, acc);
        bool full = false;
#pragma unroll
        // rows of lanes that hold heads only: the other rows' counts follow
        // row 0's but a flush never resets them
        for (int j = 0; j < 4; ++j) full |= hq < NR && scnt[j] > CB - KPW * kPage;
        if (__ballot(full)) flush(false);                    // wave-uniform
        bool live[KPW];
#pragma unroll
        for (int u = 0; u < KPW; ++u) live[u] = i0 + wv + 4 * u < i1 && kp.ok[u] && kp.lp[u] * kPage + tq < n;
        // the next step's reads go out as soon as this step's tiles are
        // contracted (after any copy-out), before its candidates are taken
        if (i1 < p1) kp.load(k_cache, sh_lp + (i1 - p0), sh_phys + (i1 - p0), i1 + wv, i1, min(p1, i1 + SP), G, g);
        float x[KPW][4];
        float lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float m = -INFINITY;
#pragma unroll
            for (int u = 0; u < KPW; ++u) {
                x[u][j] = live[u] ? a * (acc[u][j] * inv_sqrt_d) : -INFINITY;
                m = fmaxf(m, x[u][j]);
            }
            rmax[j] = fmaxf(rmax[j], row_max16(m));          // the row's head 4 hq + j, in all 16 lanes
        }
        // the block's running max: the first lane of each row of heads
        // publishes its row's maxima (one LDS round trip for all four) and the
        // result goes back to the row's lanes
        uint32_t got[4] = {0u, 0u, 0u, 0u};
        if (tq == 0 && 4 * hq < R) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < R) got[j] = atomicMax(&smax[4 * hq + j], ord_key(rmax[j]));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < R) {
                float gb = ord_unkey(got[j]);
                gb = NR == 1 ? readlane(gb, 0) : (hq == 0 ? readlane(gb, 0) : readlane(gb, 16));
                if (4 * hq + j < R) rmax[j] = fmaxf(rmax[j], gb);
            }
            lo[j] = rmax[j] - 1.0f;                          // -inf: nothing valid yet
        }
#pragma unroll
        for (int u = 0; u < KPW; ++u) {
            const float slot = __int_as_float((i0 + wv + 4 * u) * kPage + tq);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool f = 4 * hq + j < R && x[u][j] > lo[j];
                // this row's lanes (one row of heads: row 0, the same for every lane)
                const uint32_t rb = (uint32_t)(__ballot(f) >> (NR == 1 ? 0 : 16 * hq)) & 0xffffu;
                if (f) buf[j * CB + scnt[j] + __popc(rb & below)] = make_float2(x[u][j], slot);
                scnt[j] += __popc(rb);
            }
        }
    }
    flush(true);
    if (tq == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int head = 4 * hq + j;
            if (head < R) {
                const size_t rcx = (((size_t)b * HQ + g * R + head) * nsplit + split) * 4 + wv;
                ccount[rcx] = rcnt[j];
                cmax[rcx] = rmax[j];
            }
        }
    }
}

// --------------------------------------------- one-pass softmax (bf16) ----
// alpha = 1 over bf16 keys (full cache or a selection): keys and values are
// read once.  The streamed path's blocks (ranges of one (b, g), longest
// sequences first); every wave takes its own pages, 4 per step (2 at r = 8): logits on
// the matrix cores, then per head a running max m, a running sum
// l = sum exp(s - m) and o = sum exp(s - m) v over the wave's tokens, both
// rescaled by exp(m_old - m_new) when m grows (the max-shifted sums of the
// log-partition, so nothing overflows).  The next step's K tiles are read
// before this step's softmax arithmetic, its V tiles after this step's PV.
// Lane l owns value channels [D/64 l, D/64 (l + 1)) of every token; a
// token's weight comes from the lane that holds its logit (v_readlane).
// The block's four waves combine (m, l, o) by rescaling to the larger max;
// softmax_merge_kernel combines the blocks of a row the same way:
// out = o / l, tau = m + log l.

// Word 3 of a raw buffer resource on CDNA (32-bit data format, stride 0):
// with it, a buffer load whose byte offset is at or past the resource's
// range returns zero and reads nothing.
constexpr int kBufferRsrcWord3 = 0x00020000;

template <int D, int KPW>
struct VRows {
    static constexpr int VC = D / 64;                 // channels per lane
    uint32_t w[KPW][kPage];                           // VC bf16 of each token (low half when VC = 1)
    // Each page is read through a buffer resource (the page's tile as base,
    // its valid tokens x D x 2 bytes as the range), so rows of tokens that
    // are not in the sequence (past its end, on an unreadable page, past the
    // range) come back as zero without being read: their zero weights never
    // meet whatever those slots hold (0 x NaN), at no cost in instructions.
    // The page is the same for the whole wave, so the resource is scalar.
    __device__ __forceinline__ void load(const bf16_t* __restrict__ v_cache, const int* sh_lp, const int* sh_phys,
                                         int i, int i0, int i1, int G, int g, int n) {
        const int l = threadIdx.x & 63;
#pragma unroll
        for (int u = 0; u < KPW; ++u) {
            const int ii = i + 4 * u;
            const int t = ii < i1 ? ii - i0 : 0;
            const int ph = sh_phys[t];
            const bool ok = ii < i1 && ph >= 0;
            const int ntok = ok ? min(n - sh_lp[t] * kPage, kPage) : 0;
            const int phs = __builtin_amdgcn_readfirstlane(ok ? ph : 0);
            const int nbytes = __builtin_amdgcn_readfirstlane(max(ntok, 0)) * D * 2;
            const bf16_t* base = v_cache + ((size_t)phs * G + g) * kPage * D;
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nbytes, kBufferRsrcWord3);
#pragma unroll
            for (int tk = 0; tk < kPage; ++tk) {
                if constexpr (VC == 2) w[u][tk] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * l + tk * D * 2, 0, 0);
                else w[u][tk] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, 2 * l + tk * D * 2, 0, 0);
            }
        }
    }
    __device__ __forceinline__ float get(int u, int tk, int c) const {
        return c == 0 ? __uint_as_float(w[u][tk] << 16) : __uint_as_float(w[u][tk] & 0xffff0000u);
    }
};

template <int D, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void softmax_stream_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache, const bf16_t* __restrict__ v_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_pages, const int32_t* __restrict__ sel_count, int sel_stride, int B, int G,
    int MP, int NP, int cpb, int nsplit, const int32_t* __restrict__ order, float inv_sqrt_d,
    float* __restrict__ part) {
    constexpr int KPW = R <= 4 ? 4 : 2;                  // pages per wave per step
    constexpr int SP = 4 * KPW;
    constexpr int VC = D / 64;
    __shared__ int sh_order[kOrderLdsB];
    __shared__ int sh_lp[kStreamMaxChunks * kStreamPpb], sh_phys[kStreamMaxChunks * kStreamPpb];
    __shared__ float wm[4][R], wl[4][R], wc[4];
    __shared__ float wo[4][R][D];
    // block order as in the candidate stream: group fastest, then split, then
    // sequence, longest first
    const int g = blockIdx.x % G, rest = blockIdx.x / G;
    const int split = rest % nsplit, b = stream_seq(seq_lens, B, MP, order, rest / nsplit, sh_order);
    const int unit = b * G + g;
    const int HQ = G * R;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    const int cnt = sel_pages ? min(max(sel_count[unit], 0), sel_stride) : M;
    const int span = cpb * kStreamPpb;
    const int p0 = split * span;
    const int p1 = span <= kStreamMaxChunks * kStreamPpb ? min(cnt, p0 + span) : p0;   // else: an empty range
    const int32_t* sel = sel_pages ? sel_pages + (size_t)unit * sel_stride : nullptr;
    for (int t = threadIdx.x; t < min(span, kStreamMaxChunks * kStreamPpb); t += blockDim.x) {
        const int ii = p0 + t;
        const int lp = ii < p1 ? (sel ? sel[ii] : ii) : -1;
        const int phys = (lp >= 0 && lp < M) ? page_table[(size_t)b * MP + lp] : -1;
        const bool ok = phys >= 0 && phys < NP;
        sh_lp[t] = ok ? lp : -1;
        sh_phys[t] = ok ? phys : -1;
    }
    __syncthreads();

    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, tq = l & 15, hq = l >> 4;
    float m[R], ls[R], o[R][VC];
#pragma unroll
    for (int h = 0; h < R; ++h) {
        m[h] = -INFINITY;
        ls[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < VC; ++c) o[h][c] = 0.0f;
    }
    float valid = 0.0f;
    MfmaQ<D, R> mq;
    mq.load(q + ((size_t)b * HQ + g * R) * D);
    MfmaKPages<D, KPW> kp;
    VRows<D, KPW> vr;
    if (p0 < p1) {
        kp.load(k_cache, sh_lp, sh_phys, p0 + wv, p0, min(p1, p0 + SP), G, g);
        vr.load(v_cache, sh_lp, sh_phys, p0 + wv, p0, min(p1, p0 + SP), G, g, n);
    }
    for (int i0 = p0; i0 < p1; i0 += SP) {                  // block-uniform
        const int i1 = min(p1, i0 + SP);
        f32x4_t acc[KPW];
        kp.template contract<R>(mq, acc);
        float sv[KPW][4];
#pragma unroll
        for (int u = 0; u < KPW; ++u) {
            const bool live = i0 + wv + 4 * u < i1 && kp.ok[u] && kp.lp[u] * kPage + tq < n;
            valid += (float)__popcll(__ballot(live) & 0xffffull);
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[u][j] = live ? acc[u][j] * inv_sqrt_d : -INFINITY;
        }
        // the next step's key tiles go out before this step's arithmetic
        if (i1 < p1) kp.load(k_cache, sh_lp + (i1 - p0), sh_phys + (i1 - p0), i1 + wv, i1, min(p1, i1 + SP), G, g);
        // new running maxima (uniform per head) and the rescaling of l and o
#pragma unroll
        for (int h = 0; h < R; ++h) {
            const int jr = h & 3, rw = 16 * (h >> 2);
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < KPW; ++u) mx = fmaxf(mx, sv[u][jr]);
            const float mstep = readlane(row_max16(mx), rw);
            const float mnew = fmaxf(m[h], mstep);
            const float sc = m[h] > -INFINITY ? expf(m[h] - mnew) : 0.0f;
            m[h] = mnew;
            ls[h] *= sc;
#pragma unroll
            for (int c = 0; c < VC; ++c) o[h][c] *= sc;
        }
        // weights exp(s - m) in the lanes that hold the logits
        float pw[KPW][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float mh = (R <= 4 || hq == 0) ? m[j < R ? j : 0] : m[(4 + j) < R ? 4 + j : 0];
            float rs = 0.0f;
#pragma unroll
            for (int u = 0; u < KPW; ++u) {
                pw[u][j] = sv[u][j] > -INFINITY ? expf(sv[u][j] - mh) : 0.0f;
                rs += pw[u][j];
            }
            rs = row_sum16(rs);
#pragma unroll
            for (int h = j; h < R; h += 4) ls[h] += readlane(rs, 16 * (h >> 2));
        }
        // PV: every token's weight from its lane, this lane's value channels
#pragma unroll
        for (int u = 0; u < KPW; ++u) {
#pragma unroll
            for (int tk = 0; tk < kPage; ++tk) {
#pragma unroll
                for (int h = 0; h < R; ++h) {
                    const float w = readlane(pw[u][h & 3], 16 * (h >> 2) + tk);
#pragma unroll
                    for (int c = 0; c < VC; ++c) o[h][c] = fmaf(w, vr.get(u, tk, c), o[h][c]);
                }
            }
        }
        // the next step's value tiles
        if (i1 < p1) vr.load(v_cache, sh_lp + (i1 - p0), sh_phys + (i1 - p0), i1 + wv, i1, min(p1, i1 + SP), G, g, n);
    }
    // the block's four waves -> one (m, l, o, count) per head
    if (l == 0) {
#pragma unroll
        for (int h = 0; h < R; ++h) {
            wm[wv][h] = m[h];
            wl[wv][h] = ls[h];
        }
        wc[wv] = valid;
    }
#pragma unroll
    for (int h = 0; h < R; ++h)
#pragma unroll
        for (int c = 0; c < VC; ++c) wo[wv][h][VC * l + c] = o[h][c];
    __syncthreads();
    for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
        const int h = idx / D, c = idx - h * D;
        float mm = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) mm = fmaxf(mm, wm[w2][h]);
        float oo = 0.0f, ll = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const float e = wm[w2][h] > -INFINITY ? expf(wm[w2][h] - mm) : 0.0f;
            oo += wo[w2][h][c] * e;
            ll += wl[w2][h] * e;
        }
        float* dst = part + (((size_t)b * HQ + g * R + h) * nsplit + split) * (D + 4);
        dst[c] = oo;
        if (c == 0) {
            dst[D] = mm;
            dst[D + 1] = ll;
            dst[D + 2] = ((wc[0] + wc[1]) + wc[2]) + wc[3];
        }
    }
}

// The row's blocks, combined: weights exp(m_s - max m), summed in block
// order.  One 256-thread block per (b, h): the splits' maxima, weights and
// sums first (a thread per split), then every channel over the splits in
// 256 / D interleaved parts (independent loads, several in flight), the
// parts added in a fixed order.  At most kStreamMaxLists / 4 splits (the
// plan's row limit).
template <int D>
static __global__ __launch_bounds__(256) void softmax_merge_kernel(
    const float* __restrict__ part, int HQ, int nsplit, const float* __restrict__ tau_ref,
    float* __restrict__ out, float* __restrict__ tau_out, int32_t* __restrict__ support_out,
    float* __restrict__ delta_out, int32_t* __restrict__ supref_out) {
    constexpr int NP = 256 / D;                       // parts per channel
    __shared__ float sw[kStreamMaxLists / 4];
    __shared__ float osum[NP][D];
    __shared__ float red[4 * 4];                     // block_sum2: two phases of 2 x 4 waves
    int phase = 0;
    const int h = blockIdx.x, b = blockIdx.y;
    const size_t oh = (size_t)b * HQ + h;
    const float* pr = part + oh * nsplit * (D + 4);
    const int ns = min(nsplit, kStreamMaxLists / 4);
    float mx = -INFINITY;
    for (int s2 = threadIdx.x; s2 < ns; s2 += 256) mx = fmaxf(mx, pr[(size_t)s2 * (D + 4) + D]);
    mx = block_max<4>(mx, red, phase);
    float L = 0.0f, C = 0.0f;
    for (int s2 = threadIdx.x; s2 < ns; s2 += 256) {
        const float* e = pr + (size_t)s2 * (D + 4);
        const float w = e[D] > -INFINITY ? expf(e[D] - mx) : 0.0f;
        sw[s2] = w;
        L += e[D + 1] * w;
        C += e[D + 2];
    }
    block_sum2<4>(L, C, red, phase);                  // barriers: the weights are visible
    const int c = threadIdx.x % D, pt = threadIdx.x / D;
    float o = 0.0f;
#pragma unroll 8
    for (int s2 = pt; s2 < ns; s2 += NP) o = fmaf(pr[(size_t)s2 * (D + 4) + c], sw[s2], o);
    osum[pt][c] = o;
    __syncthreads();
    if (threadIdx.x < D) {
        float oo = osum[0][c];
#pragma unroll
        for (int k = 1; k < NP; ++k) oo += osum[k][c];
        const bool any = C > 0.0f;
        out[oh * D + c] = any ? oo / L : 0.0f;
        if (c == 0) {
            tau_out[oh] = any ? mx + logf(L) : -INFINITY;
            if (support_out) support_out[oh] = (int32_t)C;
            const float tref = tau_ref ? tau_ref[oh] : 0.0f;
            if (delta_out) delta_out[oh] = any ? 1.0f - L * expf(mx - tref) : 1.0f;
            if (supref_out) supref_out[oh] = (int32_t)C;   // softmax: every token has p > 0
        }
    }
}

template <int MODE>
static __global__ __launch_bounds__(kTauT) void stream_tau_kernel(
    const float2* __restrict__ cands, const int32_t* __restrict__ ccount, const float* __restrict__ cmax,
    int nsplit, int lcap, int HQ, int nslot, float beta, const float* __restrict__ tau_hint,
    const float* __restrict__ tau_ref, float* __restrict__ tau_out, int32_t* __restrict__ support_out,
    float* __restrict__ delta_out, int32_t* __restrict__ supref_out, float2* __restrict__ sup_list,
    int32_t* __restrict__ sup_count) {
    constexpr int mode = MODE;                            // compile-time: no powf where beta is 1 or 2
    constexpr int UNR = 8;                                // flat entries in flight per thread
    __shared__ float cand[kCandCap];
    __shared__ float cslot[kCandCap];                     // slot bits of each candidate
    __shared__ int loff[kStreamMaxLists + 1];             // flat offset of each list
    __shared__ float red[2 * kTauW];
    __shared__ int wsum[2 * kTauW];
    __shared__ float red5[2][kTauW][5];
    int phase = 0, p5 = 0;
    const int h = blockIdx.x, b = blockIdx.y;
    const size_t oh = (size_t)b * HQ + h;
    const float2* lists = cands + oh * nsplit * (size_t)lcap;
    const int32_t* counts = ccount + oh * nsplit;

    float xmax = -INFINITY;
    for (int c = threadIdx.x; c < nsplit; c += kTauT) xmax = fmaxf(xmax, cmax[oh * nsplit + c]);
    xmax = block_max<kTauW>(xmax, red, phase);
    if (!(xmax > -INFINITY)) {                             // no valid token
        if (threadIdx.x == 0) {
            tau_out[oh] = -INFINITY;
            if (support_out) support_out[oh] = 0;
            if (delta_out) delta_out[oh] = 1.0f;
            if (supref_out) supref_out[oh] = 0;
            sup_count[oh] = 0;
        }
        return;
    }
    const float lo = xmax - 1.0f;

    // Flat offsets of the lists: thread t scans splits [t*per, (t+1)*per).
    {
        const int per = (nsplit + kTauT - 1) / kTauT;
        int local = 0;
        for (int i = 0; i < per; ++i) {
            const int c = threadIdx.x * per + i;
            local += c < nsplit ? counts[c] : 0;
        }
        int ex, ex2, tot, tot2;
        block_excl_scan2<kTauW>(local, 0, ex, ex2, &tot, &tot2, wsum);
        for (int i = 0; i < per; ++i) {
            const int c = threadIdx.x * per + i;
            if (c < nsplit) {
                loff[c] = ex;
                ex += counts[c];
            }
        }
        if (threadIdx.x == 0) loff[nsplit] = tot;
        __syncthreads();
    }
    const int T = loff[nsplit];
    // Every list entry, by flat index f = tid, tid + kTauT, ... (UNR loads in
    // flight), in a fixed order: fn(x, slot bits).
    auto each_flat = [&](auto&& fn) {
        int sidx = 0;                                      // list of the current f, moved forward
        for (int f0 = threadIdx.x; f0 < T; f0 += kTauT * UNR) {
            float2 e[UNR];
            bool ok[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int f = f0 + u * kTauT;
                ok[u] = f < T;
                const int ff = ok[u] ? f : T - 1;        // past the end: the last entry (ignored); keeps sidx monotone
                while (loff[sidx + 1] <= ff) ++sidx;
                e[u] = lists[(size_t)sidx * lcap + (ff - loff[sidx])];
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u)
                if (ok[u]) fn(e[u]);
        }
    };
    // Candidates x > lo into LDS in one pass over the lists: rounds of
    // kTauT * GUNR entries (all in flight at once; entry f0 + kTauT u + t read by
    // thread t), each candidate placed at its rank in flat order: the
    // candidates of earlier rounds, of the round's earlier u, of earlier
    // waves at this u, and of lower lanes (wave ballot).  So they land in
    // list order and, within a list, in slot order, whatever else the lists
    // hold: the set x > lo and that order fix every sum below.  If they do
    // not all fit, the later passes read the lists instead.
    constexpr int GUNR = 64 / kTauW;                      // GUNR * kTauW (u, wave) pairs: one per lane of a wave
    __shared__ int gbase[GUNR * kTauW + 1];               // per (u, wave): rank of its first candidate; round total
    int total = 0;
    {
        const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
        int sidx = 0;
        for (int f0 = 0; f0 < T; f0 += kTauT * GUNR) {    // block-uniform
            float2 e[GUNR];
            uint64_t bal[GUNR];
#pragma unroll
            for (int u = 0; u < GUNR; ++u) {
                const int f = f0 + u * kTauT + (int)threadIdx.x;
                const int ff = f < T ? f : T - 1;          // past the end: the last entry (ignored); keeps sidx monotone
                while (loff[sidx + 1] <= ff) ++sidx;
                e[u] = lists[(size_t)sidx * lcap + (ff - loff[sidx])];
            }
#pragma unroll
            for (int u = 0; u < GUNR; ++u) {
                bal[u] = __ballot(f0 + u * kTauT + (int)threadIdx.x < T && e[u].x > lo);
                if (ln == 0) gbase[u * kTauW + wv] = __popcll(bal[u]);
            }
            __syncthreads();
            if (wv == 0) {                                 // exclusive scan in (u, wave) order
                const int c = gbase[ln];
                const int inc = wave_incl_scan(c);
                gbase[ln] = inc - c;
                if (ln == 63) gbase[GUNR * kTauW] = inc;
            }
            __syncthreads();
            const int tot = gbase[GUNR * kTauW];
            if (total + tot <= kCandCap) {                 // block-uniform
#pragma unroll
                for (int u = 0; u < GUNR; ++u) {
                    if ((bal[u] >> ln) & 1u) {
                        const int pos = total + gbase[u * kTauW + wv] + lanes_below(bal[u]);
                        cand[pos] = e[u].x;
                        cslot[pos] = e[u].y;
                    }
                }
            }
            total += tot;
            __syncthreads();                               // gbase is rewritten by the next round
        }
    }
    const bool in_lds = total <= kCandCap;
    __syncthreads();

    // Three block sums (fixed order), a minimum and a maximum, one barrier.
    auto block5 = [&](float v0, float v1, float v2, float vmin, float vmax, float* r) {
        const float a0 = wave_sum(v0), a1 = wave_sum(v1), a2 = wave_sum(v2);
        const float a3 = -wave_max(-vmin), a4 = wave_max(vmax);
        const int wid = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            red5[p5][wid][0] = a0;
            red5[p5][wid][1] = a1;
            red5[p5][wid][2] = a2;
            red5[p5][wid][3] = a3;
            red5[p5][wid][4] = a4;
        }
        __syncthreads();
        r[0] = r[1] = r[2] = 0.0f;
        r[3] = INFINITY;
        r[4] = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < kTauW; ++w2) {
            r[0] += red5[p5][w2][0];
            r[1] += red5[p5][w2][1];
            r[2] += red5[p5][w2][2];
            r[3] = fminf(r[3], red5[p5][w2][3]);
            r[4] = fmaxf(r[4], red5[p5][w2][4]);
        }
        p5 ^= 1;
    };
    // Every candidate x > lo, from LDS or from the lists.
    auto each_cand = [&](auto&& fn) {
        if (in_lds) {
            for (int i = threadIdx.x; i < total; i += kTauT) fn(cand[i]);
        } else {
            each_flat([&](float2 e) {
                if (e.x > lo) fn(e.x);
            });
        }
    };

    float tau = lo;
    if (beta >= 1.0f && in_lds && total <= kTauWaveCands) {
        // Few candidates: one wave iterates over them in LDS with wave-level
        // sums, so a step costs no block barrier (about 2 us of barrier
        // latency per step otherwise, whatever the candidate count); the
        // other waves wait at the barrier below.  Many candidates: the block
        // shares them (a single wave's serial LDS reads would cost more).
        __shared__ float sh_tau;
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            TauIter st = tau_iter_start(lo, xmax, tau_hint ? tau_hint[oh] : NAN, false);
            for (int it = 0; it < 100 && !st.done; ++it) {   // wave-uniform state
                const float t = st.t;
                float s1 = 0.0f, s0 = 0.0f, kk = 0.0f, mn = INFINITY, rest = -INFINITY;
                for (int i0 = 0; i0 < total; i0 += 4 * 64) {
                    float xs[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int i = i0 + u * 64 + lane;
                        xs[u] = i < total ? cand[i] : -INFINITY;
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float x = xs[u];
                        const float d = x - t;
                        if (d > 0.0f) {
                            s1 += powb(d, mode, beta);
                            s0 += mode == kModeBeta1 ? 1.0f : (mode == kModeBeta2 ? d : powf(d, beta - 1.0f));
                            kk += 1.0f;
                            mn = fminf(mn, x);
                        } else {
                            rest = fmaxf(rest, x);
                        }
                    }
                }
                s1 = wave_sum(s1);
                s0 = wave_sum(s0);
                kk = wave_sum(kk);
                mn = -wave_max(-mn);
                rest = wave_max(rest);
                if (mode == kModeBeta1) tau_iter_step<kModeBeta1>(st, lo, beta, s1, s0, kk, mn, rest);
                else if (mode == kModeBeta2) tau_iter_step<kModeBeta2>(st, lo, beta, s1, s0, kk, mn, rest);
                else tau_iter_step<kModeGeneral>(st, lo, beta, s1, s0, kk, mn, rest);
            }
            if (lane == 0) sh_tau = st.done ? st.tau : st.t;
        }
        __syncthreads();
        tau = sh_tau;
    } else if (beta >= 1.0f) {
        TauIter st = tau_iter_start(lo, xmax, tau_hint ? tau_hint[oh] : NAN, false);
        for (int it = 0; it < 100 && !st.done; ++it) {   // block-uniform state
            const float t = st.t;
            float s1 = 0.0f, s0 = 0.0f, kk = 0.0f, mn = INFINITY, rest = -INFINITY;
            each_cand([&](float x) {
                const float d = x - t;
                if (d > 0.0f) {
                    s1 += powb(d, mode, beta);
                    s0 += mode == kModeBeta1 ? 1.0f : (mode == kModeBeta2 ? d : powf(d, beta - 1.0f));
                    kk += 1.0f;
                    mn = fminf(mn, x);
                } else {
                    rest = fmaxf(rest, x);
                }
            });
            float r[5];
            block5(s1, s0, kk, mn, rest, r);
            if (mode == kModeBeta1) tau_iter_step<kModeBeta1>(st, lo, beta, r[0], r[1], r[2], r[3], r[4]);
            else if (mode == kModeBeta2) tau_iter_step<kModeBeta2>(st, lo, beta, r[0], r[1], r[2], r[3], r[4]);
            else tau_iter_step<kModeGeneral>(st, lo, beta, r[0], r[1], r[2], r[3], r[4]);
        }
        tau = st.done ? st.tau : st.t;
    } else {
        // beta < 1 (alpha > 2): bisection on [max - 1, max], where
        // F(max - 1) >= 1 > 0 = F(max)
        float l2 = lo, hi = xmax;
        for (int it = 0; it < 60; ++it) {
            const float mid = 0.5f * (l2 + hi);
            float s1 = 0.0f;
            each_cand([&](float x) {
                const float d = x - mid;
                if (d > 0.0f) s1 += powf(d, beta);
            });
            float r[5];
            block5(s1, 0.0f, 0.0f, 0.0f, 0.0f, r);
            if (r[0] >= 1.0f) l2 = mid; else hi = mid;
        }
        tau = 0.5f * (l2 + hi);
    }

    // Support size, dropped mass w.r.t. tau_ref (>= tau >= lo, so only
    // candidates count), and the support list (p, slot) at per-thread offsets;
    // from LDS, or from the lists when the candidates did not fit.
    auto each_cand2 = [&](auto&& fn) {
        if (in_lds) {
            for (int i = threadIdx.x; i < total; i += kTauT) fn(make_float2(cand[i], cslot[i]));
        } else {
            each_flat([&](float2 e) {
                if (e.x > lo) fn(e);
            });
        }
    };
    const float tref = tau_ref ? tau_ref[oh] : 0.0f;
    const bool want_ref = delta_out || supref_out;
    int ns = 0;
    float kept = 0.0f, nref = 0.0f;
    each_cand2([&](float2 e) {
        if (e.x > tau) ++ns;
        if (want_ref && e.x > tref) {
            kept += powb(e.x - tref, mode, beta);
            nref += 1.0f;
        }
    });
    int soff, soff2, stotal, st2;
    block_excl_scan2<kTauW>(ns, 0, soff, soff2, &stotal, &st2, wsum);
    float2* sl_out = sup_list + oh * (size_t)nslot;
    each_cand2([&](float2 e) {
        if (e.x > tau) sl_out[soff++] = make_float2(powb(e.x - tau, mode, beta), e.y);
    });
    if (want_ref) {
        kept = block_sum<kTauW>(kept, red, phase);
        nref = block_sum<kTauW>(nref, red, phase);
    }
    if (threadIdx.x == 0) {
        tau_out[oh] = tau;
        if (support_out) support_out[oh] = stotal;
        if (delta_out) delta_out[oh] = 1.0f - kept;
        if (supref_out) supref_out[oh] = (int32_t)nref;
        sup_count[oh] = stotal;
    }
}

// V rows of the support list of head (b, h), split over kSupSplit blocks
// (entries [count*split/kSupSplit, count*(split+1)/kSupSplit)): each 16-lane
// row takes every 16th entry, PVU entries in flight (entry -> page of the
// selection -> physical tile -> V row), then the rows and the block's waves
// are summed in a fixed order into part3[(b, h)][split][D].
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void support_pv_kernel(
    const T* __restrict__ v_cache, const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel_pages, const int32_t* __restrict__ sel_count, int sel_stride, int G, int MP,
    int NP, int nslot, const float2* __restrict__ sup_list, const int32_t* __restrict__ sup_count,
    float* __restrict__ part3) {
    constexpr int CH = D / kRow;
    constexpr int PVU = 4;
    __shared__ float wred[4][D];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int HQ = gridDim.y;
    const int g = h / R;
    const int unit = b * G + g;
    const size_t oh = (size_t)b * HQ + h;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    const int cnt = sel_pages ? min(max(sel_count[unit], 0), sel_stride) : M;
    const int32_t* sel = sel_pages ? sel_pages + (size_t)unit * sel_stride : nullptr;
    const int32_t* pt = page_table + (size_t)b * MP;
    const long total = sup_count[oh];
    const int k0 = (int)(total * split / kSupSplit), k1 = (int)(total * (split + 1) / kSupSplit);
    const float2* list = sup_list + oh * (size_t)nslot;
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;
    float acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
    for (int e0 = k0 + row; e0 < k1; e0 += PVU * kRow) {
        Vec<T, CH> vv[PVU];
        float pp[PVU];
        bool ok[PVU];
        // branch-free, so that the PVU chains are in flight together; an
        // entry past the range re-reads entry e0 and is ignored
#pragma unroll
        for (int u = 0; u < PVU; ++u) {
            const int e = e0 + u * kRow;
            const float2 en = list[e < k1 ? e : e0];
            const int slot = __float_as_int(en.y);
            const int ip = slot >> 4;
            const int lp = (ip >= 0 && ip < cnt) ? (sel ? sel[ip] : ip) : -1;
            const int phys = (lp >= 0 && lp < M) ? pt[lp] : -1;
            ok[u] = e < k1 && phys >= 0 && phys < NP;
            pp[u] = ok[u] ? en.x : 0.0f;
            vv[u].load(v_cache + (((size_t)(ok[u] ? phys : 0) * G + g) * kPage + (slot & (kPage - 1))) * D + lane * CH);
        }
#pragma unroll
        for (int u = 0; u < PVU; ++u)
            if (ok[u])
#pragma unroll
                for (int c = 0; c < CH; ++c) acc[c] = fmaf(pp[u], vv[u].get(c), acc[c]);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        float v = acc[c];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[c] = v;
    }
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) < kRow) {
#pragma unroll
        for (int c = 0; c < CH; ++c) wred[wid][lane * CH + c] = acc[c];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += 256)
        part3[(oh * kSupSplit + split) * D + c] = ((wred[0][c] + wred[1][c]) + wred[2][c]) + wred[3][c];
}

// ------------------------------------------------------------------ PV ----
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void pv_kernel(
    const T* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_count, int sel_stride, const float* __restrict__ logits,
    const float* __restrict__ tau, int G, int MP, int NP, int nslot, int spb, int nchunk3, int mode,
    float alpha, float beta, float* __restrict__ part3) {
    constexpr int CH = D / kRow;
    __shared__ int list_slot[256];
    __shared__ float list_p[256][R];
    __shared__ int pg_phys[256 / kPage];    // physical tile of each page of the current 256-slot batch
    __shared__ int wsum[4];
    __shared__ float wred[4][R][D];
    const int unit = blockIdx.y;
    const int b = unit / G, g = unit - b * G;
    const int HQ = G * R;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    const int cnt = sel_pages ? min(max(sel_count[unit], 0), sel_stride) : M;
    const int nused = cnt * kPage;
    const int s0 = blockIdx.x * spb;
    const int s1 = min(nused, s0 + spb);
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;
    const float a = alpha - 1.0f;
    const int32_t* sel = sel_pages ? sel_pages + (size_t)unit * sel_stride : nullptr;

    float tj[R];
#pragma unroll
    for (int j = 0; j < R; ++j) tj[j] = tau[(size_t)b * HQ + g * R + j];

    float acc[R][CH];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[j][c] = 0.0f;

    for (int base = s0; base < s1; base += 256) {
        // The batch's 16 pages resolved once (selection -> page table), so
        // that the V row loads below depend on nothing but LDS.  base is a
        // multiple of 256 (s0 is a multiple of spb).
        if (threadIdx.x < 256 / kPage) {
            const int ip = (base >> 4) + (int)threadIdx.x;
            int phys = -1;
            if (ip * kPage < s1) {
                const int lp = sel ? sel[ip] : ip;
                if (lp >= 0 && lp < M) {
                    const int ph = page_table[(size_t)b * MP + lp];
                    phys = (ph >= 0 && ph < NP) ? ph : -1;
                }
            }
            pg_phys[threadIdx.x] = phys;
        }
        const int sl = base + threadIdx.x;
        float pj[R];
        bool any = false;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            float p = 0.0f;
            if (sl < s1 && tj[j] > -INFINITY) {
                const float s = logits[((size_t)b * HQ + g * R + j) * nslot + sl];
                if (mode == kModeSoftmax) {
                    p = s > -INFINITY ? expf(s - tj[j]) : 0.0f;
                } else {
                    const float dd = a * s - tj[j];
                    p = dd > 0.0f ? powb(dd, mode, beta) : 0.0f;
                }
            }
            pj[j] = p;
            any = any || p > 0.0f;
        }
        const uint64_t m = __ballot(any);
        const int wid = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) wsum[wid] = __popcll(m);
        __syncthreads();
        int off = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            off += i < wid ? wsum[i] : 0;
            tot += wsum[i];
        }
        if (any) {
            const int pos = off + lanes_below(m);
            list_slot[pos] = sl;
#pragma unroll
            for (int j = 0; j < R; ++j) list_p[pos][j] = pj[j];
        }
        __syncthreads();
        // Each row takes entries row, row + 16, ... in order, four V rows in
        // flight at a time, without branches between the loads (an empty or
        // invalid entry reads row 0 of tile 0 and is ignored).
        constexpr int PVB = 4;
        for (int e0 = row; e0 < tot; e0 += PVB * kRow) {
            Vec<T, CH> vv[PVB];
            bool ok[PVB];
            int ent[PVB];
#pragma unroll
            for (int u = 0; u < PVB; ++u) {
                const int e = e0 + u * kRow;
                ent[u] = e < tot ? e : e0;
                const int slot = list_slot[ent[u]];
                const int phys = pg_phys[(slot - base) >> 4];
                ok[u] = e < tot && phys >= 0;
                vv[u].load(v_cache + (((size_t)(ok[u] ? phys : 0) * G + g) * kPage + (slot & (kPage - 1))) * D +
                           lane * CH);
            }
#pragma unroll
            for (int u = 0; u < PVB; ++u) {
                if (!ok[u]) continue;
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const float p = list_p[ent[u]][j];
#pragma unroll
                    for (int c = 0; c < CH; ++c) acc[j][c] = fmaf(p, vv[u].get(c), acc[j][c]);
                }
            }
        }
        __syncthreads();
    }

    // Reduce the 16 rows: rows of a wave by cross-lane adds (fixed order),
    // then the 4 waves through LDS.
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            float v = acc[j][c];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc[j][c] = v;
        }
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) < kRow) {
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int c = 0; c < CH; ++c) wred[wid][j][lane * CH + c] = acc[j][c];
    }
    __syncthreads();
    for (int o = threadIdx.x; o < R * D; o += 256) {
        const int j = o / D, c = o - j * D;
        const float v = ((wred[0][j][c] + wred[1][j][c]) + wred[2][j][c]) + wred[3][j][c];
        part3[(((size_t)b * HQ + g * R + j) * nchunk3 + blockIdx.x) * D + c] = v;
    }
}

// kReduceThreads threads per (b, h): thread (slice, c) sums the chunks
// k = slice, slice + S, ... (S = kReduceThreads / D slices) of channel c in
// order, then slice 0 adds the S slice sums in slice order: a fixed order,
// with S independent load streams per channel instead of one (one stream took
// 80 us over the 256 chunks of a 1M-token row).
constexpr int kReduceThreads = 1024;
static __global__ __launch_bounds__(kReduceThreads) void reduce_kernel(const float* __restrict__ part3, int HQ, int D,
                                                                      int nchunk3, float* __restrict__ out) {
    __shared__ float red[kReduceThreads];
    const int h = blockIdx.x, b = blockIdx.y;
    const size_t oh = (size_t)b * HQ + h;
    const int S = kReduceThreads / D;
    const int slice = threadIdx.x / D, c = threadIdx.x - slice * D;
    const float* src = part3 + oh * nchunk3 * D + c;
    float s = 0.0f;
    int k = slice;
    for (; k + 3 * S < nchunk3; k += 4 * S) {
        const float a0 = src[(size_t)k * D], a1 = src[(size_t)(k + S) * D];
        const float a2 = src[(size_t)(k + 2 * S) * D], a3 = src[(size_t)(k + 3 * S) * D];
        s += a0;
        s += a1;
        s += a2;
        s += a3;
    }
    for (; k < nchunk3; k += S) s += src[(size_t)k * D];
    red[threadIdx.x] = s;
    __syncthreads();
    if (slice == 0) {
        float t = red[c];
        for (int i = 1; i < S; ++i) t += red[i * D + c];
        out[oh * D + c] = t;
    }
}

// ------------------------------------------------- fused tau + PV (sparse) ----
constexpr int kFusedMaxSlots = 4096;   // selected slots per head on the fused path
constexpr int kCandLds = 1024;         // threshold candidates per head kept in LDS
constexpr int kPvList = 512;           // support entries per PV pass

// Orders this wave's LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int MODE>
__device__ __forceinline__ float pw(float d, float beta) {      // d^beta, d > 0
    return MODE == kModeBeta1 ? d : (MODE == kModeBeta2 ? d * d : powf(d, beta));
}
template <int MODE>
__device__ __forceinline__ float pw1(float d, float beta) {     // d^(beta-1), d > 0
    return MODE == kModeBeta1 ? 1.0f : (MODE == kModeBeta2 ? d : powf(d, beta - 1.0f));
}

// One block per (sequence, KV group): the r query heads of the group, each
// split over W waves (W = 16 / r, at most the register chunks available), so
// a wave holds KPLW float4 of logits per lane; slot k*256 + 4*lane + c of the
// wave's part sits in xr[k][c], invalid slots -inf.  Per head:
//  0. the block stages the physical page of every selected page in LDS (its
//     loads overlap the logits loads);
//  1. max(x) over the head's waves (x = (alpha-1) s);
//  2. each wave compacts its threshold candidates x > max(x) - 1 (only those
//     can be in the support: the top term alone is at most 1) with their
//     slots into its own LDS list, lane by lane after one wave scan of
//     per-lane counts (a fixed order, so results are reproducible); past CW
//     candidates the wave keeps working on its registers;
//  3. tau from sum [x - tau]_+^beta = 1 (TauIter): from tau = max(x) - 1, or
//     from the caller's tau_hint (the Gaussian selector's estimate, as the
//     selection hands it to decode) when it lies in (max - 1, max); each step
//     tries the closed form on the current support (beta in {1, 2}) and
//     otherwise takes a Newton step on F^(1/beta), the L^beta norm of
//     (x - tau)_+, convex and decreasing (beta < 1: bisection).  Each step
//     sums per wave, and the head's W partials are combined in a fixed order
//     after one block barrier (partials double-buffered);
//  4. tau, the support size and the dropped mass w.r.t. tau_ref (tau_ref,
//     the threshold over a superset of these tokens, is at least max(x) - 1,
//     so only candidates contribute);
//  5. each wave compacts its part of the support (slot, p = [x - tau]_+^beta)
//     and gathers only those V rows, four per step across the 16-lane rows;
//     the W partial outputs are summed in a fixed order.
template <typename T, int D, int R, int W, int KPLW, int MODE>
__global__ __launch_bounds__(64 * R * W) void sparse_tau_pv_kernel(
    const T* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_pages,
    const int32_t* __restrict__ sel_count, int sel_stride, const float* __restrict__ logits,
    int G, int MP, int NP, float alpha, float beta, const float* __restrict__ tau_hint,
    const float* __restrict__ tau_ref, float* __restrict__ out, float* __restrict__ tau_out,
    int32_t* __restrict__ support_out, float* __restrict__ delta_out, int32_t* __restrict__ supref_out) {
    constexpr int NWV = R * W;                   // waves in the block
    constexpr int CH = D / kRow;
    constexpr int PVU = 4;                       // V rows per 16-lane row in flight
    constexpr int NPG = W * KPLW * 256 / kPage;  // selected pages per head at most
    // candidates per wave kept in LDS: room for twice a wave's even share of
    // the head's kCandLds (a wave may hold more than its share), at most 512
    // so that the block's LDS stays within 160 KiB
    constexpr int CW = (2 * kCandLds / W) < 512 ? (2 * kCandLds / W) : 512;
    constexpr int PW = kPvList / W;              // support entries per wave per pass
    __shared__ float cand_x[NWV][CW + 64];       // + one dump slot per lane
    __shared__ int cand_s[NWV][CW + 64];
    __shared__ int pv_slot[NWV][PW + 64];
    __shared__ float pv_p[NWV][PW + 64];
    __shared__ int phys_of[NPG];
    __shared__ float part[2][NWV][5];
    __shared__ int wave_nc[NWV];                 // candidates of each wave in LDS, -1 if not
    __shared__ float sh_tau[R];
    __shared__ int flag[2][NWV];
    __shared__ float pvout[NWV][D];
    const int unit = blockIdx.x;
    const int b = unit / G, g = unit - b * G;
    const int HQ = G * R;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = wv / W, w = wv - j * W;
    const size_t oh = (size_t)b * HQ + g * R + j;
    const int n = seq_len_at(seq_lens, b, MP);
    const int M = num_pages(n);
    const int cnt = min(max(sel_count[unit], 0), min(sel_stride, NPG));
    const int nused = cnt * kPage;
    const size_t nslot = (size_t)sel_stride * kPage;
    const float a = alpha - 1.0f;
    const int base = w * KPLW * 256;             // first slot of this wave's part
    const float* lrow = logits + oh * nslot;
    float* o = out + oh * D;

    // 0. selected logical pages -> physical pages (loads first), then the logits
    const int32_t* sel = sel_pages + (size_t)unit * sel_stride;
    const int32_t* pt = page_table + (size_t)b * MP;
    constexpr int NPL = (NPG + 64 * NWV - 1) / (64 * NWV);
    int lpg[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int ip = i * 64 * NWV + (int)threadIdx.x;
        lpg[i] = ip < cnt ? sel[ip] : -1;
    }
    float xr[KPLW][4];
#pragma unroll
    for (int k = 0; k < KPLW; ++k) {
        const int s0 = base + k * 256 + 4 * lane;
        float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (s0 < nused) v = *reinterpret_cast<const float4*>(lrow + s0);
        xr[k][0] = v.x;
        xr[k][1] = v.y;
        xr[k][2] = v.z;
        xr[k][3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int ip = i * 64 * NWV + (int)threadIdx.x;
        if (ip < NPG) {
            const int lp = lpg[i];
            const int ph = (lp >= 0 && lp < M) ? pt[lp] : -1;
            phys_of[ip] = (ph >= 0 && ph < NP) ? ph : -1;
        }
    }

    // 1. max over the head (and the valid count, for the bisection bracket)
    float xm = -INFINITY;
    int nv = 0;
#pragma unroll
    for (int k = 0; k < KPLW; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            xr[k][c] *= a;
            xm = fmaxf(xm, xr[k][c]);
            nv += xr[k][c] > -INFINITY ? 1 : 0;
        }
    xm = wave_max(xm);
    nv = wave_isum(nv);
    if (lane == 0) {
        part[0][wv][0] = xm;
        part[0][wv][1] = (float)nv;
    }
    __syncthreads();
    float xmax = -INFINITY, nvalid = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) {
        xmax = fmaxf(xmax, part[0][j * W + w2][0]);
        nvalid += part[0][j * W + w2][1];
    }
    // A head without a finite logit (no valid slot, or non-finite inputs) does
    // no work but still takes part in every barrier below.
    const bool empty = !(xmax > -INFINITY);
    const float lo = empty ? 0.0f : xmax - 1.0f;

    // 2. this wave's candidates x > lo
    int mine = 0;
#pragma unroll
    for (int k = 0; k < KPLW; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c) mine += xr[k][c] > lo ? 1 : 0;
    const int incl = wave_incl_scan(mine);
    const int ncand = __builtin_amdgcn_readlane(incl, 63);
    const bool in_lds = ncand <= CW;
    float* cx = cand_x[wv];
    int* cs = cand_s[wv];
    if (in_lds) {
        int pos = incl - mine;
        const int dump = CW + lane;
#pragma unroll
        for (int k = 0; k < KPLW; ++k)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool f = xr[k][c] > lo;
                const int at = f ? pos : dump;
                cx[at] = xr[k][c];
                cs[at] = base + k * 256 + 4 * lane + c;
                pos += f ? 1 : 0;
            }
        wave_lds_sync();
    }
    auto each_cand = [&](auto&& fn) {
        if (in_lds) {
            for (int i = lane; i < ncand; i += 64) fn(cx[i], cs[i]);
        } else {
#pragma unroll
            for (int k = 0; k < KPLW; ++k)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (xr[k][c] > lo) fn(xr[k][c], base + k * 256 + 4 * lane + c);
        }
    };
    // The head's W wave partials after a barrier: three sums (fixed order), a
    // minimum and a maximum.  The partials alternate between part[0] and
    // part[1]: a call writes the buffer that the call before the previous
    // one read, and the previous call's barrier lies between those reads and
    // this write.  Step 1 above read part[0] with no barrier after it, so the
    // first call must write part[1] (pb starts at 0 and is flipped before the
    // write).  `any` tells whether any wave of the block passed fl != 0.
    int pb = 0;
    auto head_sums = [&](float v0, float v1, float v2, float vmin, float vmax, int fl, float* r, bool& any) {
        pb ^= 1;
        if (lane == 0) {
            part[pb][wv][0] = v0;
            part[pb][wv][1] = v1;
            part[pb][wv][2] = v2;
            part[pb][wv][3] = vmin;
            part[pb][wv][4] = vmax;
            flag[pb][wv] = fl;
        }
        __syncthreads();
        r[0] = r[1] = r[2] = 0.0f;
        r[3] = INFINITY;
        r[4] = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < W; ++w2) {
            const float* pw = part[pb][j * W + w2];
            r[0] += pw[0];
            r[1] += pw[1];
            r[2] += pw[2];
            r[3] = fminf(r[3], pw[3]);
            r[4] = fmaxf(r[4], pw[4]);
        }
        any = false;
#pragma unroll
        for (int v2 = 0; v2 < NWV; ++v2) any = any || flag[pb][v2] != 0;
    };

    // 3. tau.  Every step of the iteration is a pass over the head's
    // candidates, a handful of reductions and scalar-like arithmetic that
    // every wave of the head would repeat; with 16 waves on a CU that
    // repeated work is what the iteration costs.  So when every wave's
    // candidates are in LDS (the usual case), one wave per head gathers the
    // head's candidates (at most kCandLds) into registers and iterates alone,
    // with wave-level sums and no block barrier, and a single barrier hands
    // tau to the head's other waves.  Otherwise every wave iterates on its
    // own candidates and the head's partials meet after a barrier per step.
    // Both start from max - 1, or from the caller's estimate (tau_hint, e.g.
    // the Gaussian threshold estimate of the full cache) when it lies in
    // (max - 1, max); see TauIter (beta < 1: bisection).
    if (lane == 0) wave_nc[wv] = in_lds ? ncand : -1;
    __syncthreads();
    bool all_lds = true;                         // every wave in LDS, every head within kCandLds
#pragma unroll
    for (int j2 = 0; j2 < R; ++j2) {
        int tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < W; ++w2) {
            const int c = wave_nc[j2 * W + w2];
            all_lds = all_lds && c >= 0;
            tot += c;
        }
        all_lds = all_lds && tot <= kCandLds;
    }
    const float hint = (tau_hint && !empty) ? tau_hint[oh] : NAN;
    float tau = lo;
    if (all_lds) {                                           // block-uniform
        if (w == j % W) {                                    // the head's iterating wave
            constexpr int NH = kCandLds / 64;
            int off[W + 1];
            off[0] = 0;
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2) off[w2 + 1] = off[w2] + wave_nc[j * W + w2];
            const int nh = off[W];
            float hx[NH];
#pragma unroll
            for (int i = 0; i < NH; ++i) {
                // element e of the concatenated lists: list w2, entry e - off[w2]
                // (a select chain, so that no register array is indexed at run time)
                const int e = lane + 64 * i;
                int w2 = 0, base = 0;
#pragma unroll
                for (int u = 1; u < W; ++u) {
                    const bool past = e >= off[u];
                    w2 = past ? u : w2;
                    base = past ? off[u] : base;
                }
                hx[i] = e < nh ? cand_x[j * W + w2][e - base] : -INFINITY;
            }
            // (guards, not breaks, so that the loops unroll and hx stays in registers)
            auto each_h = [&](auto&& fn) {
#pragma unroll
                for (int i = 0; i < NH; ++i)
                    if (i * 64 < nh && hx[i] > lo) fn(hx[i]);      // first test wave-uniform
            };
            if (MODE != kModeGeneral || beta >= 1.0f) {
                TauIter st = tau_iter_start(lo, xmax, hint, empty);
                for (int it = 0; it < 100 && !st.done; ++it) {   // wave-uniform
                    const float t = st.t;                        // t >= lo
                    float s1 = 0.0f, s0 = 0.0f, mn = INFINITY, rest = -INFINITY;
                    int kk = 0;
                    // Branch-free: selects instead of divergent paths per element
                    // (entries past the list are -inf: not above t, not above lo).
#pragma unroll
                    for (int i = 0; i < NH; ++i) {
                        if (i * 64 >= nh) continue;              // wave-uniform
                        const float x = hx[i];
                        const float d = x - t;
                        const bool in = d > 0.0f;
                        const float dp = in ? d : 0.0f;
                        s1 += in ? pw<MODE>(dp, beta) : 0.0f;
                        s0 += in ? pw1<MODE>(dp, beta) : 0.0f;
                        kk += in ? 1 : 0;
                        mn = in ? fminf(mn, x) : mn;
                        rest = (!in && x > lo) ? fmaxf(rest, x) : rest;
                    }
                    tau_iter_step<MODE>(st, lo, beta, wave_sum(s1), wave_sum(s0), (float)wave_isum(kk),
                                        -wave_max(-mn), wave_max(rest));
                }
                tau = st.done ? st.tau : st.t;
            } else {
                float l2 = lo, hi = xmax - powf(nvalid, 1.0f - alpha);
                for (int it = 0; it < 60 && !empty; ++it) {
                    const float mid = 0.5f * (l2 + hi);
                    float s1 = 0.0f;
                    each_h([&](float x) {
                        const float d = x - mid;
                        if (d > 0.0f) s1 += pw<MODE>(d, beta);
                    });
                    if (wave_sum(s1) >= 1.0f) l2 = mid; else hi = mid;
                }
                tau = 0.5f * (l2 + hi);
            }
            if (lane == 0) sh_tau[j] = tau;
        }
        __syncthreads();
        tau = sh_tau[j];
    } else if (MODE != kModeGeneral || beta >= 1.0f) {
        TauIter it_st = tau_iter_start(lo, xmax, hint, empty);
        for (int it = 0; it < 100; ++it) {
            float s1 = 0.0f, s0 = 0.0f, mn = INFINITY, rest = -INFINITY;
            int kk = 0;
            if (!it_st.done) {
                const float t = it_st.t;
                each_cand([&](float x, int) {
                    const float d = x - t;
                    if (d > 0.0f) {
                        s1 += pw<MODE>(d, beta);
                        s0 += pw1<MODE>(d, beta);
                        ++kk;
                        mn = fminf(mn, x);
                    } else {
                        rest = fmaxf(rest, x);
                    }
                });
            }
            float r[5];
            bool any;
            head_sums(wave_sum(s1), wave_sum(s0), (float)wave_isum(kk), -wave_max(-mn), wave_max(rest),
                      it_st.done ? 0 : 1, r, any);
            if (!any) break;                                 // block-uniform
            if (!it_st.done) tau_iter_step<MODE>(it_st, lo, beta, r[0], r[1], r[2], r[3], r[4]);
        }
        tau = it_st.done ? it_st.tau : it_st.t;
    } else {
        // beta < 1 (alpha > 2): bisection on [max - 1, max - n^(1-alpha)]
        float l2 = lo, hi = xmax - powf(nvalid, 1.0f - alpha);
        for (int it = 0; it < 60; ++it) {
            const float mid = 0.5f * (l2 + hi);
            float s1 = 0.0f;
            each_cand([&](float x, int) {
                const float d = x - mid;
                if (d > 0.0f) s1 += pw<MODE>(d, beta);
            });
            s1 = wave_sum(s1);
            float r[5];
            bool any;
            head_sums(s1, 0.0f, 0.0f, 0.0f, 0.0f, 0, r, any);
            if (r[0] >= 1.0f) l2 = mid; else hi = mid;
        }
        tau = 0.5f * (l2 + hi);
    }

    // 4. support size and dropped mass with respect to tau_ref
    // (every token above tau_ref is a candidate: tau_ref >= tau >= max - 1)
    int ns = 0, nref = 0;
    float kept = 0.0f;
    const float tref = tau_ref ? tau_ref[oh] : 0.0f;
    const bool want_ref = delta_out || supref_out;
    if (!empty) each_cand([&](float x, int) {
        ns += x > tau ? 1 : 0;
        if (want_ref && x > tref) {
            kept += pw<MODE>(x - tref, beta);
            ++nref;
        }
    });
    const int sinc = wave_incl_scan(ns);
    const int nsw = __builtin_amdgcn_readlane(sinc, 63);      // this wave's support
    {
        float r[5];
        bool any;
        head_sums((float)nsw, want_ref ? wave_sum(kept) : 0.0f, want_ref ? (float)wave_isum(nref) : 0.0f, 0.0f, 0.0f,
                  0, r, any);
        if (w == 0 && lane == 0) {
            tau_out[oh] = empty ? -INFINITY : tau;
            if (support_out) support_out[oh] = empty ? 0 : (int32_t)r[0];
            if (delta_out) delta_out[oh] = empty ? 1.0f : 1.0f - r[1];
            if (supref_out) supref_out[oh] = empty ? 0 : (int32_t)r[2];
        }
    }

    // 5. PV over this wave's part of the support, in passes of PW entries.
    const int rg = lane >> 4, l16 = lane & (kRow - 1);
    int* ls = pv_slot[wv];
    float* lpv = pv_p[wv];
    float acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
    for (int start = 0; start < nsw; start += PW) {
        if (start > 0) wave_lds_sync();          // the previous pass has read its list
        int pos = sinc - ns - start;
        const int dump = PW + lane;
        each_cand([&](float x, int slot) {
            if (x > tau) {
                const int at = (pos >= 0 && pos < PW) ? pos : dump;
                ls[at] = slot;
                lpv[at] = pw<MODE>(x - tau, beta);
                ++pos;
            }
        });
        wave_lds_sync();
        const int nent = min(nsw - start, PW);
        for (int e0 = 0; e0 < nent; e0 += 4 * PVU) {
            Vec<T, CH> vv[PVU];
            float pp[PVU];
            bool okv[PVU];
            // Branch-free, so that the PVU row loads are in flight together
            // (a load under a branch waits for the earlier ones); a slot past
            // the list reads entry 0's row of page 0 and is ignored.
#pragma unroll
            for (int u = 0; u < PVU; ++u) {
                const int e = e0 + 4 * u + rg;
                const int ec = e < nent ? e : 0;
                const int slot = ls[ec];
                const int phys = phys_of[slot >> 4];
                okv[u] = e < nent && phys >= 0;
                pp[u] = okv[u] ? lpv[ec] : 0.0f;
                vv[u].load(v_cache + (((size_t)(okv[u] ? phys : 0) * G + g) * kPage + (slot & (kPage - 1))) * D +
                           l16 * CH);
            }
#pragma unroll
            for (int u = 0; u < PVU; ++u)
                if (okv[u])
#pragma unroll
                    for (int c = 0; c < CH; ++c) acc[c] = fmaf(pp[u], vv[u].get(c), acc[c]);
        }
    }
    // Fixed-order sums: the four 16-lane rows of the wave, then the head's waves.
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        float v = acc[c];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[c] = v;
    }
    if (lane < kRow) {
#pragma unroll
        for (int c = 0; c < CH; ++c) pvout[wv][l16 * CH + c] = acc[c];
    }
    __syncthreads();
    if (w == 0) {
        for (int c = lane; c < D; c += 64) {
            float v = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2) v += pvout[j * W + w2][c];
            o[c] = v;
        }
    }
}

template <typename T, int D, int R, int MODE>
static hipError_t run_fused(const Dims& d, const DecodePlan& pl, const void* v_cache, const int32_t* pt,
                            const int32_t* sl, const int32_t* sel_pages, const int32_t* sel_count, int sel_stride,
                            float alpha, float beta, const float* logits, const DecodeHeads& io, hipStream_t s) {
    const int units = d.B * d.G;
    // KPL float4 of logits per lane in all; W = 16 / R waves per head, at most KPL.
    constexpr int WMAX = 16 / R;
#define EKV_FUSED(KPL)                                                                                      \
    {                                                                                                       \
        constexpr int W = WMAX < KPL ? WMAX : KPL;                                                          \
        sparse_tau_pv_kernel<T, D, R, W, KPL / W, MODE><<<dim3(units), dim3(64 * R * W), 0, s>>>(           \
            (const T*)v_cache, pt, sl, sel_pages, sel_count, sel_stride, logits, d.G, d.MP, d.NP, alpha, beta, \
            io.tau_hint, io.tau_ref, io.out, io.tau, io.support, io.delta, io.supref);                      \
        return hipGetLastError();                                                                           \
    }
    if (pl.nslot <= 256) EKV_FUSED(1)
    if (pl.nslot <= 512) EKV_FUSED(2)
    if (pl.nslot <= 1024) EKV_FUSED(4)
    if (pl.nslot <= 2048) EKV_FUSED(8)
    EKV_FUSED(16)
#undef EKV_FUSED
}

template <typename T, int D, int R>
static hipError_t run_decode(const Dims& d, const DecodePlan& pl, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* pt, const int32_t* sl,
                             const int32_t* sel_pages, const int32_t* sel_count, int sel_stride,
                             float alpha, int mode, float beta, const DecodeHeads& io, char* ws,
                             hipStream_t s) {
    float* logits = (float*)(ws + pl.off_logits);
    float* part1 = (float*)(ws + pl.off_part1);
    float* part3 = (float*)(ws + pl.off_part3);
    const int units = d.B * d.G;
    const size_t lds = ((size_t)R * pl.ppb * kPage) * sizeof(float);
    if (pl.fused) {
        bool wide = false;                                   // 64-page, 8-wave blocks (bf16 keys)
        if constexpr (std::is_same<T, bf16_t>::value) {
            if (pl.lg_ppb == 6) {
                logits_kernel<T, D, R, false, 8><<<dim3(pl.nchunk1, units), dim3(512), lds, s>>>(
                    (const T*)q, (const T*)k_cache, pt, sl, sel_pages, sel_count, sel_stride, d.G, d.MP, d.NP,
                    pl.lg_ppb, pl.nslot, pl.nchunk1, 1.0f / sqrtf((float)D), logits, nullptr);
                wide = true;
            }
        }
        if (!wide)
            logits_kernel<T, D, R, false><<<dim3(pl.nchunk1, units), dim3(256), lds, s>>>(
                (const T*)q, (const T*)k_cache, pt, sl, sel_pages, sel_count, sel_stride, d.G, d.MP, d.NP,
                pl.lg_ppb, pl.nslot, pl.nchunk1, 1.0f / sqrtf((float)D), logits, nullptr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        switch (mode) {
            case kModeBeta1:
                return run_fused<T, D, R, kModeBeta1>(d, pl, v_cache, pt, sl, sel_pages, sel_count, sel_stride,
                                                      alpha, beta, logits, io, s);
            case kModeBeta2:
                return run_fused<T, D, R, kModeBeta2>(d, pl, v_cache, pt, sl, sel_pages, sel_count, sel_stride,
                                                      alpha, beta, logits, io, s);
            default:
                return run_fused<T, D, R, kModeGeneral>(d, pl, v_cache, pt, sl, sel_pages, sel_count,
                                                        sel_stride, alpha, beta, logits, io, s);
        }
    }
    if (pl.stream) {
        float2* cands = (float2*)(ws + pl.off_cands);
        int32_t* ccount = (int32_t*)(ws + pl.off_ccount);
        float* cmax = (float*)(ws + pl.off_cmax);
        float2* sup = (float2*)(ws + pl.off_sup);
        int32_t* supcnt = (int32_t*)(ws + pl.off_supcnt);
        int32_t* order = (int32_t*)(ws + pl.off_order);
        if (d.B > kOrderLdsB) {
            order_by_length_kernel<<<dim3(1), dim3(1024), 0, s>>>(sl, d.B, d.MP, order);
            hipError_t e0 = hipGetLastError();
            if (e0 != hipSuccess) return e0;
        }
        // lists per split: one per wave on bf16 keys, one per block otherwise
        int lps = 1;
        if constexpr (std::is_same<T, bf16_t>::value) {
            lps = 4;
            cand_stream_mfma_kernel<D, R><<<dim3(pl.nsplit_s * units), dim3(256), 0, s>>>(
                (const T*)q, (const T*)k_cache, pt, sl, sel_pages, sel_count, sel_stride, d.B, d.G, d.MP, d.NP,
                pl.cpb_s, pl.nsplit_s, order, 1.0f / sqrtf((float)D), alpha - 1.0f, cands, ccount, cmax);
        } else {
            cand_stream_kernel<T, D, R><<<dim3(pl.nsplit_s * units), dim3(256), 0, s>>>(
                (const T*)q, (const T*)k_cache, pt, sl, sel_pages, sel_count, sel_stride, d.B, d.G, d.MP, d.NP,
                pl.cpb_s, pl.nsplit_s, order, 1.0f / sqrtf((float)D), alpha - 1.0f, cands, ccount, cmax);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
#define EKV_STREAM_TAU(M)                                                                                        \
    stream_tau_kernel<M><<<dim3(d.HQ, d.B), dim3(kTauT), 0, s>>>(cands, ccount, cmax, pl.nsplit_s * lps,           \
                                                                 pl.cpb_s * kStreamSlots / lps, d.HQ, pl.nslot,  \
                                                                 beta, io.tau_hint, io.tau_ref, io.tau,          \
                                                                 io.support, io.delta, io.supref, sup, supcnt)
        if (mode == kModeBeta1) EKV_STREAM_TAU(kModeBeta1);
        else if (mode == kModeBeta2) EKV_STREAM_TAU(kModeBeta2);
        else EKV_STREAM_TAU(kModeGeneral);
#undef EKV_STREAM_TAU
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        support_pv_kernel<T, D, R><<<dim3(kSupSplit, d.HQ, d.B), dim3(256), 0, s>>>(
            (const T*)v_cache, pt, sl, sel_pages, sel_count, sel_stride, d.G, d.MP, d.NP, pl.nslot, sup, supcnt, part3);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        reduce_kernel<<<dim3(d.HQ, d.B), dim3(kReduceThreads), 0, s>>>(part3, d.HQ, D, kSupSplit, io.out);
        return hipGetLastError();
    }
    if constexpr (std::is_same<T, bf16_t>::value) {
        if (pl.smx1) {
            float* part = (float*)(ws + pl.off_part3);
            int32_t* order = (int32_t*)(ws + pl.off_order);
            if (d.B > kOrderLdsB) {
                order_by_length_kernel<<<dim3(1), dim3(1024), 0, s>>>(sl, d.B, d.MP, order);
                hipError_t e0 = hipGetLastError();
                if (e0 != hipSuccess) return e0;
            }
            softmax_stream_kernel<D, R><<<dim3(pl.nsplit_s * units), dim3(256), 0, s>>>(
                (const bf16_t*)q, (const bf16_t*)k_cache, (const bf16_t*)v_cache, pt, sl, sel_pages, sel_count,
                sel_stride, d.B, d.G, d.MP, d.NP, pl.cpb_s, pl.nsplit_s, order, 1.0f / sqrtf((float)D), part);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            softmax_merge_kernel<D><<<dim3(d.HQ, d.B), dim3(256), 0, s>>>(part, d.HQ, pl.nsplit_s, io.tau_ref,
                                                                       io.out, io.tau, io.support, io.delta,
                                                                       io.supref);
            return hipGetLastError();
        }
    }
    // softmax: logits with chunk partials, log-partition, PV over every slot
    logits_kernel<T, D, R, true><<<dim3(pl.nchunk1, units), dim3(256), lds, s>>>(
        (const T*)q, (const T*)k_cache, pt, sl, sel_pages, sel_count, sel_stride, d.G, d.MP, d.NP,
        pl.lg_ppb, pl.nslot, pl.nchunk1, 1.0f / sqrtf((float)D), logits, part1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    softmax_tau_kernel<<<dim3(d.HQ, d.B), dim3(256), 0, s>>>(part1, d.HQ, pl.nchunk1, io.tau_ref, io.tau,
                                                             io.support, io.delta, io.supref);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    pv_kernel<T, D, R><<<dim3(pl.nchunk3, units), dim3(256), 0, s>>>(
        (const T*)v_cache, pt, sl, sel_pages, sel_count, sel_stride, logits, io.tau, d.G, d.MP, d.NP,
        pl.nslot, pl.spb, pl.nchunk3, mode, alpha, beta, part3);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    reduce_kernel<<<dim3(d.HQ, d.B), dim3(kReduceThreads), 0, s>>>(part3, d.HQ, D, pl.nchunk3, io.out);
    return hipGetLastError();
}


// Kernel launches for one KV element type (decode_bf16.hip, decode_f32.hip).
template <typename T>
static hipError_t launch_decode_typed(const Dims& d, const DecodePlan& pl, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                                      const int32_t* sel_pages, const int32_t* sel_count, int sel_stride,
                                      float alpha, int mode, float beta, const DecodeHeads& io, char* ws,
                                      hipStream_t s) {
#define EKV_DEC(RR, DD)                                                                          \
    return run_decode<T, DD, RR>(d, pl, q, k_cache, v_cache, page_table, seq_lens, sel_pages,    \
                                 sel_count, sel_stride, alpha, mode, beta, io, ws, s)
#define EKV_RSW(DD)                             \
    switch (d.R) {                              \
        case 1: EKV_DEC(1, DD);                 \
        case 2: EKV_DEC(2, DD);                 \
        case 4: EKV_DEC(4, DD);                 \
        case 8: EKV_DEC(8, DD);                 \
        default: return hipErrorInvalidValue;   \
    }
    if (d.D == 128) { EKV_RSW(128) } else { EKV_RSW(64) }
#undef EKV_RSW
#undef EKV_DEC
}

}  // namespace ekv
