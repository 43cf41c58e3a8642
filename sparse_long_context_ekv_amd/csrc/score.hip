// Query-aware page scores.
//
// Box score ("EntmaxKV: Support-Aware Decoding for Entmax Attention",
// section 4.2 and Appendix B.1): the largest q.k/sqrt(D) over the
// axis-aligned box spanned by the page's keys,
//     u_{h,p} = (1/sqrt(D)) sum_i max(q_i kmax_i, q_i kmin_i),
// pooled per KV group by the maximum over the group's r query heads, so one
// page set serves every head of the group.
//
// Gaussian moments (section 4.3, "score moments per head and batch element"
// of section 4.4), channels treated as independent:
//     mu_{h,p} = (1/sqrt(D)) sum_i q_i mean_i,  sigma_{h,p}^2 = (1/D) sum_i q_i^2 var_i.
//
// Both kernels are pure streams over the page statistics: one 16-lane row
// per (page, group), lane l owning channels [l*CH, (l+1)*CH), the r query
// slices of the group in registers, one fixed-order DPP row sum per head.
// A block covers 2^lg_ppb consecutive logical pages of one sequence (up to
// 256); each row issues the loads of UNROLL pages before using any of them.
// Results are staged in LDS and written once, at the end of the block, one
// contiguous run of pages per output row, four floats per store: single-float stores scattered over
// the [B][.][MP] rows (one per page and head) cost the statistics stream a
// third of its speed, and stores interleaved with the stream cost twice what
// they cost alone.
#include <atomic>

#include "ekv_device.h"
#include "ekv_internal.h"

namespace ekv {

constexpr int kUnroll = 4;
constexpr int kMfmaLgPpb = 8;          // pages per matrix-core moments block, at most (256)

// Writes a block's staged results, rows of 2^lg floats in LDS, to output
// rows starting at column p_begin, np columns of each.  One thread moves four
// consecutive columns (a 16-byte LDS read and, where the destination is
// 16-byte aligned, one 16-byte store): the flush is the tail of every block,
// and single-float copies made it several times longer.  The stores are
// non-temporal: the outputs are read once, by the next kernel, and stores
// left dirty in L2 cost a write-back at the end of the kernel (about 3 us of
// the step on the 128K batched workload, measured).
template <typename RowPtr>
__device__ __forceinline__ void flush_rows(const float* stage, int nrows, int lg, int p_begin, int np,
                                           bool vec, RowPtr row_ptr) {
    const int lq = lg - 2;                     // quads per row, log2 (lg >= 2)
    for (int i = threadIdx.x; i < (nrows << lq); i += blockDim.x) {
        const int rr = i >> lq, pp = (i & ((1 << lq) - 1)) << 2;
        if (pp >= np) continue;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + (i << 2));
        float* o = row_ptr(rr) + p_begin + pp;
        if (vec && pp + 4 <= np) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(o));
        } else {
            __builtin_nontemporal_store(v.x, o);
            if (pp + 1 < np) __builtin_nontemporal_store(v.y, o + 1);
            if (pp + 2 < np) __builtin_nontemporal_store(v.z, o + 2);
            if (pp + 3 < np) __builtin_nontemporal_store(v.w, o + 3);
        }
    }
}

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void box_score_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const T* __restrict__ kmin, const T* __restrict__ kmax,
    float* __restrict__ score, int G, int MP, int NP, int lg_ppb, float inv_sqrt_d, bool vec) {
    constexpr int CH = D / kRow;
    extern __shared__ float stage[];           // [G][ppb]
    const int ppb = 1 << lg_ppb;
    const int b = blockIdx.y;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    const int p_begin = blockIdx.x * ppb;
    if (p_begin >= M) return;                  // block-uniform
    const int p_end = min(M, p_begin + ppb);
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;
    const int per_iter = kRow / G;
    const bool active = row < per_iter * G;    // idle rows still reach the barrier
    const int slot = row / G, g = active ? row % G : 0;
    const int HQ = G * R;

    Vec<T, CH> qv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) qv[j].load(q + ((size_t)b * HQ + g * R + j) * D + lane * CH);

    // For bf16: per head and 32-bit word, a mask picking kmax where q >= 0
    // and kmin where q < 0 (bitwise select), so max(q*kmax, q*kmin) is one
    // select and one packed dot product per channel pair.
    constexpr int NW = Vec<T, CH>::NW;
    uint32_t pick_max[std::is_same<T, float>::value ? 1 : R][NW];
    if constexpr (!std::is_same<T, float>::value) {
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                uint32_t x = qv[j].w[w];
                pick_max[j][w] = ((x & 0x8000u) ? 0u : 0x0000ffffu) | ((x & 0x80000000u) ? 0u : 0xffff0000u);
            }
    }
    (void)pick_max;

    const int32_t* pt = page_table + (size_t)b * MP;
    for (int p0 = p_begin + slot; active && p0 < p_end; p0 += kUnroll * per_iter) {
        Vec<T, CH> lo[kUnroll], hi[kUnroll];
        bool ok[kUnroll];
        int phys[kUnroll];
        // All table entries, then all statistics loads, without branches, so
        // that every load of the unroll is in flight at once (a load under a
        // per-page branch waits for the previous ones).  Past the block's end
        // or on a bad entry, page 0 is read and ignored.
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) phys[u] = pt[min(p0 + u * per_iter, p_end - 1)];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            ok[u] = p0 + u * per_iter < p_end && phys[u] >= 0 && phys[u] < NP;
            const size_t off = ((size_t)(ok[u] ? phys[u] : 0) * G + g) * D + lane * CH;
            lo[u].load(kmin + off);
            hi[u].load(kmax + off);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!ok[u]) {
                // a page of the block whose table entry maps outside the
                // cache: defined result -inf (never selected ahead of a
                // readable page), not a stale stage slot
                if (p0 + u * per_iter < p_end && lane == 0)
                    stage[(g << lg_ppb) + p0 + u * per_iter - p_begin] = -INFINITY;
                continue;
            }
            float best = -INFINITY;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float acc = 0.0f;
                if constexpr (std::is_same<T, float>::value) {
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        float qc = qv[j].get(c);
                        acc = fmaf(qc, qc >= 0.0f ? hi[u].get(c) : lo[u].get(c), acc);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        uint32_t m = pick_max[j][w];
                        uint32_t sel = (m & hi[u].w[w]) | (~m & lo[u].w[w]);
                        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, sel),
                                                              __builtin_bit_cast(bf16x2_t, qv[j].w[w]),
                                                              acc, false);
                    }
                }
                best = fmaxf(best, row_sum16(acc));
            }
            if (lane == 0) stage[(g << lg_ppb) + p0 + u * per_iter - p_begin] = best * inv_sqrt_d;
        }
    }
    __syncthreads();
    flush_rows(stage, G, lg_ppb, p_begin, p_end - p_begin, vec,
               [&](int gg) { return score + ((size_t)b * G + gg) * MP; });
}

template <typename T, typename S, int D, int R>
__global__ __launch_bounds__(256) void gauss_score_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const S* __restrict__ kmean, const S* __restrict__ kvar,
    float* __restrict__ mu, float* __restrict__ sigma, int G, int MP, int NP, int lg_ppb,
    float inv_sqrt_d, float inv_d, bool vec) {
    constexpr int CH = D / kRow;
    extern __shared__ float stage[];           // [2][HQ][ppb]: mu, then sigma
    const int ppb = 1 << lg_ppb;
    const int b = blockIdx.y;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    const int p_begin = blockIdx.x * ppb;
    if (p_begin >= M) return;                  // block-uniform
    const int p_end = min(M, p_begin + ppb);
    const int lane = threadIdx.x & (kRow - 1);
    const int row = threadIdx.x >> 4;
    const int per_iter = kRow / G;
    const bool active = row < per_iter * G;    // idle rows still reach the barrier
    const int slot = row / G, g = active ? row % G : 0;
    const int HQ = G * R;

    float qf[R][CH], q2[R][CH];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        Vec<T, CH> v;
        v.load(q + ((size_t)b * HQ + g * R + j) * D + lane * CH);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            qf[j][c] = v.get(c);
            q2[j][c] = qf[j][c] * qf[j][c];
        }
    }

    const int32_t* pt = page_table + (size_t)b * MP;
    // lane j < R holds mu of head g*R+j, lane R+j its sigma
    const int jh = lane < R ? lane : lane - R;
    float* dst = stage + ((lane < R ? 0 : HQ) + g * R + jh) * ppb;
    const bool writer = lane < 2 * R;
    for (int p0 = p_begin + slot; active && p0 < p_end; p0 += kUnroll * per_iter) {
        Vec<S, CH> mv[kUnroll], vv[kUnroll];
        bool ok[kUnroll];
        int phys[kUnroll];
        // as in box_score_kernel: all loads of the unroll in flight at once
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) phys[u] = pt[min(p0 + u * per_iter, p_end - 1)];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            ok[u] = p0 + u * per_iter < p_end && phys[u] >= 0 && phys[u] < NP;
            const size_t off = ((size_t)(ok[u] ? phys[u] : 0) * G + g) * D + lane * CH;
            mv[u].load(kmean + off);
            vv[u].load(kvar + off);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!ok[u]) {
                // table entry outside the cache: mu = -inf, sigma = 0, a point
                // mass that adds nothing to the threshold equation and has
                // the lowest margin (never a stale stage slot)
                if (p0 + u * per_iter < p_end && writer)
                    dst[p0 + u * per_iter - p_begin] = lane < R ? -INFINITY : 0.0f;
                continue;
            }
            float mine = 0.0f;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float am = 0.0f, av = 0.0f;
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    am = fmaf(qf[j][c], mv[u].get(c), am);
                    av = fmaf(q2[j][c], vv[u].get(c), av);
                }
                am = row_sum16(am);
                av = row_sum16(av);
                mine = (lane == j) ? am * inv_sqrt_d : mine;
                mine = (lane == R + j) ? sqrtf(fmaxf(av, 0.0f) * inv_d) : mine;
            }
            if (writer) dst[p0 + u * per_iter - p_begin] = mine;
        }
    }
    __syncthreads();
    flush_rows(stage, 2 * HQ, lg_ppb, p_begin, p_end - p_begin, vec, [&](int hh) {
        return hh < HQ ? mu + ((size_t)b * HQ + hh) * MP : sigma + ((size_t)b * HQ + hh - HQ) * MP;
    });
}

// ------------------------------------------------- matrix-core moments ----
// The Gaussian moments with bf16 queries over 16-bit or FP8 statistics, as
// small dense contractions on v_mfma_f32_16x16x32_bf16: rows = the group's r
// query heads (zero-padded to 16), columns = 16 consecutive pages, k = 32
// channels per instruction.  Every product is exact in the fp32 accumulator:
//   mu      = q . mean                                  (D/32 instructions)
//   sigma^2 = (q^2)_hi . var + (q^2)_lo . var, with q^2 (exact in fp32, at
//             most 16 significant bits) split into two bf16 parts that sum
//             to it exactly                           (2 D/32 instructions)
// and FP8 codes widen to bf16 exactly.  The 2r row sums per page of the
// lane-per-channel kernel above are what limits it on 16-bit statistics
// (half the bytes per page, the same arithmetic); here a 16-page tile of one
// group costs 3 D/32 instructions.  (Box scores, q+ . kmax + q- . kmin, ran
// no faster this way on the ragged batch, 252 us against 245 us: the
// lane-per-channel box kernel does one select and one packed dot product per
// channel pair and is not bound by its arithmetic.)
//
// Operand layout of the instruction: lane l (t = l % 16, h = l / 16) holds
// 8 channels of instruction i (mfma_chan) of query head t (A) and of page t
// (B); the result holds heads 4 h .. 4 h + 3 of page t.  A block covers
// 2^lg_ppb pages of one sequence and GB groups (GB = 4, 2 or 1, dividing G;
// grid x = G / GB); wave w takes group w % GB and every (4/GB)-th 16-page
// tile, kMfmaTiles tiles' loads in flight at once.
// Measured on the 128K batched workload: bf16 statistics 104-108 us with
// 256-page blocks (5.0-5.1 TB/s of reads), 112 us with 128, 119 us with 64,
// 175 us with 16; FP8 54-65 us.  The same kernel with the contractions
// replaced by a fold of the loaded words runs within 2% of this: the reads
// (two 256-byte rows per page and group at random physical pages), not the
// arithmetic, bound it.
constexpr int kMfmaTiles = 4;

// First channel of lane quarter h's 8-channel slice in instruction i.  The
// contraction does not depend on which channels an instruction takes, as
// long as the query and statistics operands agree: 16-bit statistics use
// 32 i + 8 h (one 16-byte load per instruction), FP8 statistics
// 64 (i / 2) + 16 h + 8 (i % 2), so one 16-byte load of 16 codes feeds two
// instructions.
template <typename S>
__device__ __forceinline__ int mfma_chan(int i, int h) {
    return std::is_same<S, fp8_t>::value ? 64 * (i >> 1) + 16 * h + 8 * (i & 1) : 32 * i + 8 * h;
}

// Sixteen FP8 codes (one 16-byte load) as two bf16 operands, exactly.
__device__ __forceinline__ void load16_fp8_bf16(const fp8_t* p, bf16x8_t& lo8, bf16x8_t& hi8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const auto f = (k & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)rw[k >> 1], true)
                               : __builtin_amdgcn_cvt_pk_f32_fp8((int)rw[k >> 1], false);
        // E4M3 values have 3 fraction bits: the top 16 bits are exact
        w[k] = (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
    }
    lo8 = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    hi8 = __builtin_bit_cast(bf16x8_t, make_uint4(w[4], w[5], w[6], w[7]));
}

// Eight bf16 lanes of a query operand from fp32 values that bf16 holds exactly.
__device__ __forceinline__ bf16x8_t pack8_bf16(const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xffff0000u);
    return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

template <typename S, int D, int R, int GB>
__global__ __launch_bounds__(256) void gauss_mfma_kernel(
    const bf16_t* __restrict__ q, const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const S* __restrict__ kmean, const S* __restrict__ kvar, float* __restrict__ mu, float* __restrict__ sigma,
    int G, int MP, int NP, int lg_ppb, float inv_sqrt_d, float inv_d, bool vec) {
    constexpr int NT = D / 32;
    static_assert(NT % 2 == 0, "FP8 statistics feed instructions in pairs");
    static_assert(std::is_same<S, bf16_t>::value || std::is_same<S, fp8_t>::value, "16-bit or FP8 statistics");
    extern __shared__ float stage[];               // [2][GB*R][ppb]: mu, then sigma
    const int ppb = 1 << lg_ppb;
    const int b = blockIdx.z, g0 = blockIdx.x * GB;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    const int p_begin = blockIdx.y * ppb;
    if (p_begin >= M) return;                      // block-uniform
    const int p_end = min(M, p_begin + ppb);
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, tq = l & 15, hq = l >> 4;
    const int gl = wv % GB, g = g0 + gl;
    const int HQ = G * R;

    // the query operands of this wave's group (rows past R are zero)
    bf16x8_t qa[3][NT];                            // q, (q^2)_hi, (q^2)_lo
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        float v[8];
        const uint4 raw = tq < R ? *reinterpret_cast<const uint4*>(q + ((size_t)b * HQ + g * R + tq) * D +
                                                                   mfma_chan<S>(i, hq))
                                 : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(rw[k] << 16);
            v[2 * k + 1] = __uint_as_float(rw[k] & 0xffff0000u);
        }
        float hi[8], lo[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float q2 = v[k] * v[k];                                       // exact
            hi[k] = __uint_as_float(__float_as_uint(q2) & 0xffff0000u);         // top 8 significant bits
            lo[k] = q2 - hi[k];                                                 // the rest, exact in bf16
        }
        qa[0][i] = pack8_bf16(v);
        qa[1][i] = pack8_bf16(hi);
        qa[2][i] = pack8_bf16(lo);
    }

    // the block's table entries, read once (-1: past the block or outside the cache)
    __shared__ int sh_phys[1 << kMfmaLgPpb];
    const int32_t* pt = page_table + (size_t)b * MP;
    for (int t = threadIdx.x; t < ppb; t += blockDim.x) {
        const int ph = p_begin + t < p_end ? pt[p_begin + t] : -1;
        sh_phys[t] = ph >= 0 && ph < NP ? ph : -1;
    }
    __syncthreads();
    const int ntile = (p_end - p_begin + kPage - 1) / kPage;
    constexpr int WPG = 4 / GB;                     // waves per group
    for (int t0 = wv / GB; t0 < ntile; t0 += WPG * kMfmaTiles) {   // wave-uniform
        bf16x8_t s0[kMfmaTiles][NT], s1[kMfmaTiles][NT];
        bool ok[kMfmaTiles];
        // every tile's loads first, without branches (a page past the block
        // or with a bad table entry reads page 0 and is ignored)
#pragma unroll
        for (int u = 0; u < kMfmaTiles; ++u) {
            const int pi = (t0 + u * WPG) * kPage + tq;   // page within the block
            const int ph = sh_phys[pi < ppb ? pi : 0];
            ok[u] = pi < ppb && ph >= 0;
            const size_t off = ((size_t)(ok[u] ? ph : 0) * G + g) * D;
            if constexpr (std::is_same<S, fp8_t>::value) {
#pragma unroll
                for (int i = 0; i < NT; i += 2) {
                    load16_fp8_bf16(kmean + off + mfma_chan<S>(i, hq), s0[u][i], s0[u][i + 1]);
                    load16_fp8_bf16(kvar + off + mfma_chan<S>(i, hq), s1[u][i], s1[u][i + 1]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    s0[u][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kmean + off + mfma_chan<S>(i, hq)));
                    s1[u][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kvar + off + mfma_chan<S>(i, hq)));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kMfmaTiles; ++u) {
            const int tile = t0 + u * WPG;
            if (tile < ntile) {                                       // wave-uniform
                const int p = p_begin + tile * kPage + tq;
                f32x4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0][i], s0[u][i], a0, 0, 0, 0);
                    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1][i], s1[u][i], a1, 0, 0, 0);
                    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[2][i], s1[u][i], a1, 0, 0, 0);
                }
                if (p < p_end) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int head = 4 * hq + j;
                        if (head < R) {
                            // bad table entry: mu = -inf, sigma = 0 (a point mass that adds nothing)
                            stage[(gl * R + head) * ppb + p - p_begin] = ok[u] ? a0[j] * inv_sqrt_d : -INFINITY;
                            stage[((GB + gl) * R + head) * ppb + p - p_begin] =
                                ok[u] ? sqrtf(fmaxf(a1[j], 0.0f) * inv_d) : 0.0f;
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    flush_rows(stage, 2 * GB * R, lg_ppb, p_begin, p_end - p_begin, vec, [&](int rr) {
        return rr < GB * R ? mu + ((size_t)b * HQ + g0 * R + rr) * MP
                           : sigma + ((size_t)b * HQ + g0 * R + rr - GB * R) * MP;
    });
}

template <typename S, int D, int R>
static hipError_t run_gauss_mfma(const Dims& d, const void* q, const int32_t* pt, const int32_t* sl,
                                 const void* kmean, const void* kvar, float* mu, float* sigma, hipStream_t s) {
    const int GB = d.G % 4 == 0 ? 4 : (d.G % 2 == 0 ? 2 : 1);
    // (all G groups of a page in one 8-wave block measured slower than two
    // 4-group blocks side by side)
    int lg = kMfmaLgPpb;
    // at most 32 KiB of staged outputs, and at least 1024 blocks where the batch allows
    while (lg > 4 && ((((size_t)2 * GB * R) << lg) * sizeof(float) > 32768 ||
                      (((long)d.B * d.MP) >> lg) * (d.G / GB) < 1024))
        --lg;
    const size_t lds = (((size_t)2 * GB * R) << lg) * sizeof(float);
    // group blocks of the same pages side by side in launch order: the G rows
    // of a physical page's statistics are adjacent in memory
    const dim3 grid(d.G / GB, (d.MP + (1 << lg) - 1) >> lg, d.B);
    const bool vec = d.MP % 4 == 0 && ((uintptr_t)mu & 15) == 0 && ((uintptr_t)sigma & 15) == 0;
#define EKV_LAUNCH_MFMA(GBV)                                                                                      \
    gauss_mfma_kernel<S, D, R, GBV><<<grid, dim3(256), lds, s>>>((const bf16_t*)q, pt, sl, (const S*)kmean,       \
                                                                 (const S*)kvar, mu, sigma, d.G, d.MP, d.NP, lg,  \
                                                                 1.0f / sqrtf((float)D), 1.0f / (float)D, vec)
    if (GB == 4) EKV_LAUNCH_MFMA(4);
    else if (GB == 2) EKV_LAUNCH_MFMA(2);
    else EKV_LAUNCH_MFMA(1);
#undef EKV_LAUNCH_MFMA
    return hipGetLastError();
}

// log2 of the pages per block of the lane-per-channel kernels.  Measured on
// the 128K batched workload: with fp32 statistics (1 KiB per page and group)
// 256-page blocks, whose staged outputs go out in long runs at the end, beat
// 16-page blocks by ~3%; with 16-bit statistics (half the bytes per page)
// the 512 large blocks keep too few loads in flight and 16-page blocks are
// 25% faster.  Box scores over bf16 min/max on the ragged 64-sequence batch:
// 64-page blocks 245 us, 16-page 260 us, 256-page 270 us.  (bf16 queries
// over 16-bit or FP8 statistics now take the matrix-core kernels.)  Fewer
// pages when that leaves under 512 blocks for 256 CUs or the block's outputs
// (`out_per_page` floats per page) would pass 64 KiB of LDS.
static int score_lg_ppb(const Dims& d, int out_per_page, int lg_max) {
    const long units = (long)d.B * d.MP;
    int lg = lg_max;
    while (lg > 2 && ((units >> lg) < 512 || ((long)out_per_page << lg) * 4 > 65536)) --lg;
    return lg;
}

// Raises the kernel's dynamic LDS limit to 64 KiB, once per device.  The flag
// is atomic so that concurrent first calls from several host threads are
// well defined (setting the attribute twice is harmless).
template <typename K>
static bool allow_64k_lds(K kernel) {
    static std::atomic<bool> ok[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!ok[dev].load(std::memory_order_acquire)) {
        if (hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 65536) == hipSuccess)
            ok[dev].store(true, std::memory_order_release);
        else
            (void)hipGetLastError();
    }
    return ok[dev].load(std::memory_order_acquire);
}

template <typename T, int D, int R>
static hipError_t run_box(const Dims& d, const void* q, const int32_t* pt, const int32_t* sl,
                          const void* kmin, const void* kmax, float* score, hipStream_t s) {
    int lg = score_lg_ppb(d, d.G, d.kv_bf16 ? 6 : 8);
    if (((size_t)d.G << lg) * sizeof(float) > 48 * 1024 && !allow_64k_lds(box_score_kernel<T, D, R>)) lg = 2;
    dim3 grid((d.MP + (1 << lg) - 1) >> lg, d.B);
    const size_t lds = ((size_t)d.G << lg) * sizeof(float);
    const bool vec = d.MP % 4 == 0 && ((uintptr_t)score & 15) == 0;
    box_score_kernel<T, D, R><<<grid, dim3(256), lds, s>>>((const T*)q, pt, sl, (const T*)kmin, (const T*)kmax,
                                                           score, d.G, d.MP, d.NP, lg, 1.0f / sqrtf((float)D), vec);
    return hipGetLastError();
}

template <typename T, typename S, int D, int R>
static hipError_t run_gauss(const Dims& d, const void* q, const int32_t* pt, const int32_t* sl,
                            const void* kmean, const void* kvar, float* mu, float* sigma, hipStream_t s) {
    int lg = score_lg_ppb(d, 2 * d.HQ, d.stat == kStatF32 ? 8 : 4);
    if (((size_t)2 * d.HQ << lg) * sizeof(float) > 48 * 1024 && !allow_64k_lds(gauss_score_kernel<T, S, D, R>))
        lg = 2;
    dim3 grid((d.MP + (1 << lg) - 1) >> lg, d.B);
    const size_t lds = ((size_t)2 * d.HQ << lg) * sizeof(float);
    const bool vec = d.MP % 4 == 0 && ((uintptr_t)mu & 15) == 0 && ((uintptr_t)sigma & 15) == 0;
    gauss_score_kernel<T, S, D, R><<<grid, dim3(256), lds, s>>>((const T*)q, pt, sl, (const S*)kmean,
                                                                (const S*)kvar, mu, sigma, d.G, d.MP, d.NP, lg,
                                                                1.0f / sqrtf((float)D), 1.0f / (float)D, vec);
    return hipGetLastError();
}

#define EKV_R_SWITCH(MACRO, ...)                          \
    switch (d.R) {                                        \
        case 1: MACRO(1, __VA_ARGS__);                    \
        case 2: MACRO(2, __VA_ARGS__);                    \
        case 4: MACRO(4, __VA_ARGS__);                    \
        case 8: MACRO(8, __VA_ARGS__);                    \
        default: return hipErrorInvalidValue;             \
    }

hipError_t launch_box_score(const Dims& d, const void* q, const int32_t* page_table,
                            const int32_t* seq_lens, const void* kmin, const void* kmax,
                            float* score, hipStream_t s) {
#define EKV_BOX(RR, T, DD) return run_box<T, DD, RR>(d, q, page_table, seq_lens, kmin, kmax, score, s)
    if (d.kv_bf16) {
        if (d.D == 128) { EKV_R_SWITCH(EKV_BOX, bf16_t, 128) } else { EKV_R_SWITCH(EKV_BOX, bf16_t, 64) }
    } else {
        if (d.D == 128) { EKV_R_SWITCH(EKV_BOX, float, 128) } else { EKV_R_SWITCH(EKV_BOX, float, 64) }
    }
#undef EKV_BOX
}

// Per-head box scores u_{h,p} before the pooling over the group's heads (an
// optional output of top-k scoring, for inspection; not on the step's path):
// one 16-lane row per page, every head of the batch row in turn, fp32 sums.
// Pages past the sequence end are not written; an unreadable table entry
// gives -inf.
template <typename T, int D>
__global__ __launch_bounds__(256) void head_box_kernel(const T* __restrict__ q, const int32_t* __restrict__ page_table,
                                                       const int32_t* __restrict__ seq_lens, const T* __restrict__ kmin,
                                                       const T* __restrict__ kmax, float* __restrict__ head_score,
                                                       int HQ, int G, int MP, int NP, float inv_sqrt_d) {
    constexpr int CH = D / kRow;
    const int b = blockIdx.y;
    const int M = num_pages(seq_len_at(seq_lens, b, MP));
    const int p = blockIdx.x * kRow + (threadIdx.x >> 4);
    const int lane = threadIdx.x & (kRow - 1);
    if (blockIdx.x * kRow >= M) return;            // block-uniform
    const bool live = p < M;                        // rows past the end still take part in the row sums
    const int ph = live ? page_table[(size_t)b * MP + p] : -1;
    const bool ok = ph >= 0 && ph < NP;
    const int R = HQ / G;
    for (int h = 0; h < HQ; ++h) {
        const int g = h / R;
        Vec<T, CH> qv, lo, hi;
        qv.load(q + ((size_t)b * HQ + h) * D + lane * CH);
        const size_t off = ((size_t)(ok ? ph : 0) * G + g) * D + lane * CH;
        lo.load(kmin + off);
        hi.load(kmax + off);
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float qc = qv.get(c);
            acc += fmaxf(qc * hi.get(c), qc * lo.get(c));
        }
        acc = row_sum16(acc);
        if (live && lane == 0) head_score[((size_t)b * HQ + h) * MP + p] = ok ? acc * inv_sqrt_d : -INFINITY;
    }
}

hipError_t launch_head_box_score(const Dims& d, const void* q, const int32_t* page_table, const int32_t* seq_lens,
                                 const void* kmin, const void* kmax, float* head_score, hipStream_t s) {
    const dim3 grid((d.MP + kRow - 1) / kRow, d.B);
    const float isd = 1.0f / sqrtf((float)d.D);
#define EKV_HB(T, DD)                                                                                              \
    head_box_kernel<T, DD><<<grid, dim3(256), 0, s>>>((const T*)q, page_table, seq_lens, (const T*)kmin,          \
                                                      (const T*)kmax, head_score, d.HQ, d.G, d.MP, d.NP, isd)
    if (d.kv_bf16) {
        if (d.D == 128) EKV_HB(bf16_t, 128); else EKV_HB(bf16_t, 64);
    } else {
        if (d.D == 128) EKV_HB(float, 128); else EKV_HB(float, 64);
    }
#undef EKV_HB
    return hipGetLastError();
}

hipError_t launch_gauss_score(const Dims& d, const void* q, const int32_t* page_table,
                              const int32_t* seq_lens, const void* kmean, const void* kvar,
                              float* mu, float* sigma, hipStream_t s) {
#define EKV_GS(RR, T, S, DD) return run_gauss<T, S, DD, RR>(d, q, page_table, seq_lens, kmean, kvar, mu, sigma, s)
#define EKV_GSM(RR, S, DD) \
    return run_gauss_mfma<S, DD, RR>(d, q, page_table, seq_lens, kmean, kvar, mu, sigma, s)
    if (d.kv_bf16) {
        if (d.stat == kStatBF16) {
            if (d.D == 128) { EKV_R_SWITCH(EKV_GSM, bf16_t, 128) } else { EKV_R_SWITCH(EKV_GSM, bf16_t, 64) }
        } else if (d.stat == kStatFP8) {
            if (d.D == 128) { EKV_R_SWITCH(EKV_GSM, fp8_t, 128) } else { EKV_R_SWITCH(EKV_GSM, fp8_t, 64) }
        } else {
            if (d.D == 128) { EKV_R_SWITCH(EKV_GS, bf16_t, float, 128) } else { EKV_R_SWITCH(EKV_GS, bf16_t, float, 64) }
        }
    } else {
        if (d.stat == kStatBF16) {
            if (d.D == 128) { EKV_R_SWITCH(EKV_GS, float, bf16_t, 128) } else { EKV_R_SWITCH(EKV_GS, float, bf16_t, 64) }
        } else if (d.stat == kStatFP8) {
            if (d.D == 128) { EKV_R_SWITCH(EKV_GS, float, fp8_t, 128) } else { EKV_R_SWITCH(EKV_GS, float, fp8_t, 64) }
        } else {
            if (d.D == 128) { EKV_R_SWITCH(EKV_GS, float, float, 128) } else { EKV_R_SWITCH(EKV_GS, float, float, 64) }
        }
    }
#undef EKV_GS
#undef EKV_GSM
}

}  // namespace ekv
