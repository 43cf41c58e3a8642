// Device-side helpers for the libekv kernels (gfx950, wave64).
//
// Conventions used by every kernel:
//  * a "row" is 16 consecutive lanes of a wavefront (one DPP row); a row
//    covers one D-wide vector (a key, a value or a statistic) with each lane
//    owning CH = D/16 consecutive channels, so a row reads D*sizeof(T)
//    contiguous bytes;
//  * reductions use fixed-order DPP rotations within a row and readlane /
//    LDS across rows, never atomics, so every result is reproducible run to
//    run;
//  * bf16 values are carried as their 16-bit patterns (the upper half of an
//    fp32), widened exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace ekv {

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint8_t fp8_t;        // OCP FP8 E4M3 code (statistics storage only)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));   // a 16x16x32 bf16 MFMA operand (8 per lane)
typedef float f32x4_t __attribute__((ext_vector_type(4)));     // a 16x16 MFMA accumulator (4 per lane)

constexpr int kPage = 16;     // tokens per page (the only page size built)
constexpr int kRow = 16;      // lanes per DPP row

// ---------------------------------------------------------------- loads ----
// CH channels of element type T as 32-bit words.
template <typename T, int CH>
struct Vec {
    static constexpr int NW = CH * (int)sizeof(T) / 4;
    static_assert(NW == 1 || NW == 2 || NW == 4 || NW == 8, "row slice must be 4, 8, 16 or 32 bytes");
    uint32_t w[NW];

    __device__ __forceinline__ void load(const T* p) {
        if constexpr (NW == 1) {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        } else if constexpr (NW == 2) {
            uint2 a = *reinterpret_cast<const uint2*>(p);
            w[0] = a.x; w[1] = a.y;
        } else if constexpr (NW == 4) {
            uint4 a = *reinterpret_cast<const uint4*>(p);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        } else {
            const uint4* p4 = reinterpret_cast<const uint4*>(p);
            uint4 a = p4[0], b = p4[1];
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        }
    }
    __device__ __forceinline__ void store(T* p) const {
        if constexpr (NW == 1) {
            *reinterpret_cast<uint32_t*>(p) = w[0];
        } else if constexpr (NW == 2) {
            *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        } else if constexpr (NW == 4) {
            *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            uint4* p4 = reinterpret_cast<uint4*>(p);
            p4[0] = make_uint4(w[0], w[1], w[2], w[3]);
            p4[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
    // Channel i widened to fp32 (exact).  FP8 codes go through the packed
    // hardware conversion (checked against the E4M3 definition on all 256
    // codes on gfx950).
    __device__ __forceinline__ float get(int i) const {
        if constexpr (std::is_same<T, float>::value) {
            return __uint_as_float(w[i]);
        } else if constexpr (std::is_same<T, fp8_t>::value) {
            const int word = (int)w[i >> 2];
            const auto pair = ((i >> 1) & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true)
                                             : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
            return pair[i & 1];
        } else {
            return (i & 1) ? __uint_as_float(w[i >> 1] & 0xffff0000u)
                           : __uint_as_float(w[i >> 1] << 16);
        }
    }
    // Set channel i from an fp32 value that is exactly representable in T.
    __device__ __forceinline__ void set_exact(int i, float v) {
        if constexpr (std::is_same<T, float>::value) {
            w[i] = __float_as_uint(v);
        } else {
            uint32_t h = __float_as_uint(v) >> 16;
            if (i & 1) w[i >> 1] = (w[i >> 1] & 0x0000ffffu) | (h << 16);
            else       w[i >> 1] = (w[i >> 1] & 0xffff0000u) | h;
        }
    }
};

// fp32 -> OCP FP8 E4M3 code (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits; no infinities; S.1111.111 is NaN): round to nearest even, finite
// magnitudes beyond the largest finite value 448 saturate to 448, NaN stays
// NaN.  Below 2^-6 the grid is the subnormal step 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float f) {
    const uint32_t s = (__float_as_uint(f) >> 24) & 0x80u;
    const float a = fabsf(f);
    if (!(a == a)) return s | 0x7fu;
    if (a >= 448.0f) return s | 0x7eu;
    if (a < 0.015625f) return s | (uint32_t)rintf(a * 512.0f);   // 0..8; 8 is the smallest normal
    uint32_t u = __float_as_uint(a);
    u += 0x7ffffu + ((u >> 20) & 1u);                             // round the 23-bit mantissa to 3 bits
    const uint32_t e = (u >> 23) - 120u;                          // biased 7 instead of 127
    return s | (e << 3) | ((u >> 20) & 7u);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---------------------------------------------------- hardware math ----
// Single-instruction approximations (about 1 ulp) for the arithmetic of
// iteration steps, where rounding only changes how a step lands and never
// the value the iteration converges to: the IEEE-exact division, sqrtf and
// logf expand to long dependent instruction chains, which a one-wave
// iteration pays on every step.
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_pow(float x, float y) { return hw_exp2(y * hw_log2(x)); }   // x > 0

// ------------------------------------------------------- cross-lane ops ----
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP controls: row_ror:k = 0x120 + k.
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0x128>(v);
    v += dpp<0x124>(v);
    v += dpp<0x122>(v);
    v += dpp<0x121>(v);
    return v;
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0x128>(v));
    v = fmaxf(v, dpp<0x124>(v));
    v = fmaxf(v, dpp<0x122>(v));
    v = fmaxf(v, dpp<0x121>(v));
    return v;
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Wave-uniform sum / max over 64 lanes (fixed order: rows 0,1,2,3).
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum16(v);
    return ((readlane(v, 0) + readlane(v, 16)) + readlane(v, 32)) + readlane(v, 48);
}
__device__ __forceinline__ float wave_max(float v) {
    v = row_max16(v);
    return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}

// Number of set bits of a 64-bit lane mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Block-uniform reductions for blocks of NW waves.  `red` is an LDS array
// of at least 2*NW floats; `phase` alternates so that back-to-back calls need
// one barrier each.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red, int& phase) {
    float w = wave_sum(v);
    const int wid = threadIdx.x >> 6;
    float* r = red + phase * NW;
    if ((threadIdx.x & 63) == 0) r[wid] = w;
    __syncthreads();
    float s = r[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) s += r[i];
    phase ^= 1;
    return s;
}
template <int NW>
__device__ __forceinline__ float block_max(float v, float* red, int& phase) {
    float w = wave_max(v);
    const int wid = threadIdx.x >> 6;
    float* r = red + phase * NW;
    if ((threadIdx.x & 63) == 0) r[wid] = w;
    __syncthreads();
    float s = r[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) s = fmaxf(s, r[i]);
    phase ^= 1;
    return s;
}

// Two block-uniform sums with one barrier.  `red` holds at least 4*NW floats.
template <int NW>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red, int& phase) {
    const float wa = wave_sum(a), wb = wave_sum(b);
    const int wid = threadIdx.x >> 6;
    float* r = red + phase * 2 * NW;
    if ((threadIdx.x & 63) == 0) {
        r[wid] = wa;
        r[NW + wid] = wb;
    }
    __syncthreads();
    float sa = r[0], sb = r[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        sa += r[i];
        sb += r[NW + i];
    }
    phase ^= 1;
    a = sa;
    b = sb;
}

// Three block-uniform sums with one barrier.  `red` holds at least 6*NW floats.
template <int NW>
__device__ __forceinline__ void block_sum3(float& a, float& b, float& c, float* red, int& phase) {
    const float wa = wave_sum(a), wb = wave_sum(b), wc = wave_sum(c);
    const int wid = threadIdx.x >> 6;
    float* r = red + phase * 3 * NW;
    if ((threadIdx.x & 63) == 0) {
        r[wid] = wa;
        r[NW + wid] = wb;
        r[2 * NW + wid] = wc;
    }
    __syncthreads();
    float sa = r[0], sb = r[NW], sc = r[2 * NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
        sa += r[i];
        sb += r[NW + i];
        sc += r[2 * NW + i];
    }
    phase ^= 1;
    a = sa;
    b = sb;
    c = sc;
}

// Integer DPP move: lanes whose source is outside the row read 0 when BC.
template <int CTRL, int ROWMASK = 0xf, bool BC = true>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xf, BC);
}

// Inclusive prefix sum over the 64 lanes of a wave, all in registers:
// Hillis-Steele within each 16-lane row (row_shr 1, 2, 4, 8), then lane 15
// of rows 0 and 2 is added into rows 1 and 3 (row_bcast:15), and lane 31
// into rows 2 and 3 (row_bcast:31).  Integer, so exact.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_i<0x111>(v);
    v += dpp_i<0x112>(v);
    v += dpp_i<0x114>(v);
    v += dpp_i<0x118>(v);
    v += dpp_i<0x142, 0xa, false>(v);
    v += dpp_i<0x143, 0xc, false>(v);
    return v;
}

// Wave-uniform integer sum (exact).
__device__ __forceinline__ int wave_isum(int v) {
    return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

// Wave-uniform unsigned min / max (row rotations, then the four rows).
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
    v = min(v, (uint32_t)dpp_i<0x128, 0xf, false>((int)v));
    v = min(v, (uint32_t)dpp_i<0x124, 0xf, false>((int)v));
    v = min(v, (uint32_t)dpp_i<0x122, 0xf, false>((int)v));
    v = min(v, (uint32_t)dpp_i<0x121, 0xf, false>((int)v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<0x128, 0xf, false>((int)v));
    v = max(v, (uint32_t)dpp_i<0x124, 0xf, false>((int)v));
    v = max(v, (uint32_t)dpp_i<0x122, 0xf, false>((int)v));
    v = max(v, (uint32_t)dpp_i<0x121, 0xf, false>((int)v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// Block-wide exclusive prefix sums of two per-thread counts, in thread
// order, for blocks of NW waves; totals are returned in *ta, *tb.  `wsum`
// is LDS of at least 2*NW ints.  Ends with a barrier, so `wsum` may be
// reused right after.
template <int NW>
__device__ __forceinline__ void block_excl_scan2(int a, int b, int& ea, int& eb, int* ta, int* tb, int* wsum) {
    const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) {
        wsum[wid] = ia;
        wsum[NW + wid] = ib;
    }
    __syncthreads();
    int oa = 0, ob = 0, sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int ca = wsum[i], cb = wsum[NW + i];
        oa += i < wid ? ca : 0;
        ob += i < wid ? cb : 0;
        sa += ca;
        sb += cb;
    }
    __syncthreads();
    ea = oa + ia - a;
    eb = ob + ib - b;
    *ta = sa;
    *tb = sb;
}

// Block-wide total of a per-thread count and min / max of per-thread uint32
// values, for blocks of NW waves; every thread gets the results.  `wsum` is
// LDS of at least 3*NW ints.  Ends with a barrier.
template <int NW>
__device__ __forceinline__ void block_count_range(int c, uint32_t& mn, uint32_t& mx, int* total, int* wsum) {
    c = wave_isum(c);
    mn = wave_umin(mn);
    mx = wave_umax(mx);
    const int wid = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        wsum[wid] = c;
        wsum[NW + wid] = (int)mn;
        wsum[2 * NW + wid] = (int)mx;
    }
    __syncthreads();
    int t = 0;
    uint32_t a = 0xffffffffu, b = 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        t += wsum[i];
        a = min(a, (uint32_t)wsum[NW + i]);
        b = max(b, (uint32_t)wsum[2 * NW + i]);
    }
    __syncthreads();
    *total = t;
    mn = a;
    mx = b;
}

// Order-preserving map float -> uint32 (larger float, larger key); -0 == +0.
__device__ __forceinline__ uint32_t ord_key(float f) {
    if (f == 0.0f) f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ord_key.
__device__ __forceinline__ float ord_unkey(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int num_pages(int n) { return (n + kPage - 1) / kPage; }

// Sequence length clamped to what its page-table row can address, so that a
// bad length never sends a kernel outside the table, the cache or an output row.
__device__ __forceinline__ int seq_len_at(const int32_t* seq_lens, int b, int MP) {
    const int n = seq_lens[b];
    const int cap = MP * kPage;
    return n < 0 ? 0 : (n > cap ? cap : n);
}

}  // namespace ekv
