// Sparse alpha-entmax decode: the workspace plan and the dispatch to the
// per-dtype kernel launches (decode_bf16.hip, decode_f32.hip); the kernels
// and what they compute are described in decode_kernels.h.
#include <algorithm>

#include "decode_kernels.h"

namespace ekv {

// ---------------------------------------------------------------- host ----
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodePlan plan_decode(const Dims& d, int sparse, int sel_stride, float alpha) {
    DecodePlan pl = {};
    pl.sparse = sparse;
    const int maxp = sparse ? sel_stride : d.MP;
    pl.nslot = maxp * kPage;
    pl.fused = sparse && alpha > 1.0f && pl.nslot <= kFusedMaxSlots;
    pl.stream = !pl.fused && alpha > 1.0f;
    const size_t bh = (size_t)d.B * d.HQ;
    // pages per logits block: 64 for the fused path's bf16 keys (8-wave
    // blocks on the matrix cores) where that still gives 256 blocks or more,
    // 8 for other selections (and for few rows: a small batch's blocks are
    // latency chains, so more and shorter ones), 32 over the cache
    const long wide_blocks = (long)d.B * d.G * ((maxp + 63) / 64);
    pl.lg_ppb = pl.fused && d.kv_bf16 && wide_blocks >= 256 ? 6 : (sparse ? 3 : 5);
    pl.ppb = 1 << pl.lg_ppb;
    pl.nchunk1 = (maxp + pl.ppb - 1) / pl.ppb;
    if (pl.nchunk1 < 1) pl.nchunk1 = 1;
    // one-pass softmax for bf16 keys (alpha = 1): the streamed path's block split
    pl.smx1 = !(alpha > 1.0f) && d.kv_bf16;
    if (pl.stream || pl.smx1) {
        // Chunks per block: about kStreamBlocks blocks in all, at most
        // kStreamMaxChunks chunks per block; each block keeps up to 4 lists
        // per head (one per wave on bf16 keys), kStreamMaxLists per (b, h).
        // The work is estimated from the pages the cache holds where that is
        // less than B * max pages (sequences shorter than the table's width):
        // about kStreamBlocks working blocks either way.  Where it is less
        // than 3/4 of it (a ragged batch, most likely), blocks are capped at
        // 24 chunks, so that the longest-first order can balance the CUs.
        const long nchunk = maxp > 0 ? (maxp + kStreamPpb - 1) / kStreamPpb : 1;
        const long cap_pages = (long)d.B * maxp;
        const long work_pages = sparse ? cap_pages : std::min<long>(cap_pages, d.NP);
        const long work_chunks = std::max<long>((work_pages + kStreamPpb - 1) / kStreamPpb, 1) * d.G;
        long cpb = (work_chunks + kStreamBlocks - 1) / kStreamBlocks;
        if (cpb < 1) cpb = 1;
        if (cpb > kStreamMaxChunks) cpb = kStreamMaxChunks;
        if (4 * work_pages < 3 * cap_pages && cpb > kStreamRaggedChunks) cpb = kStreamRaggedChunks;
        // never fewer chunks per block than the longest row needs to fit its lists
        const long cpb_need = (nchunk + kStreamMaxLists / 4 - 1) / (kStreamMaxLists / 4);
        if (cpb < cpb_need) cpb = std::min<long>(cpb_need, kStreamMaxChunks);
        pl.cpb_s = (int)cpb;
        pl.nsplit_s = (int)((nchunk + cpb - 1) / cpb);
        // rows past kStreamMaxLists / 4 * kStreamMaxChunks chunks (16M tokens) are not built
        pl.too_long = 4L * pl.nsplit_s > kStreamMaxLists;
    } else if (!pl.fused) {
        // the same row limit on the softmax path of fp32 keys
        pl.too_long = (long)maxp > (long)(kStreamMaxLists / 4) * kStreamMaxChunks * kStreamPpb;
    }
    if (pl.fused) {
        // selected logits [B][HQ][nslot]
        pl.off_logits = 0;
        pl.bytes = align256(bh * pl.nslot * sizeof(float));
    } else if (pl.stream) {
        // per (b, h, split, wave): candidate list (x, slot), count, max; per
        // (b, h): support list (p, slot), its count, kSupSplit partial outputs
        const size_t rows = bh * pl.nsplit_s * 4;              // list counts and maxima
        pl.off_cands = 0;
        pl.off_ccount = pl.off_cands + align256(bh * pl.nsplit_s * pl.cpb_s * kStreamSlots * sizeof(float2));
        pl.off_cmax = pl.off_ccount + align256(rows * sizeof(int32_t));
        pl.off_sup = pl.off_cmax + align256(rows * sizeof(float));
        pl.off_supcnt = pl.off_sup + align256(bh * pl.nslot * sizeof(float2));
        pl.off_part3 = pl.off_supcnt + align256(bh * sizeof(int32_t));
        pl.off_order = pl.off_part3 + align256(bh * kSupSplit * d.D * sizeof(float));   // sequences by length
        pl.bytes = pl.off_order + align256((size_t)d.B * sizeof(int32_t));
    } else if (pl.smx1) {
        // per (b, h, split): o [D], running max, sum of exp, valid count
        pl.off_part3 = 0;
        pl.off_order = align256(bh * pl.nsplit_s * (d.D + 4) * sizeof(float));
        pl.bytes = pl.off_order + align256((size_t)d.B * sizeof(int32_t));
    } else {
        // softmax: logits, chunk partials (max, sum exp, count), PV partials
        pl.spb = sparse ? 256 : 4096;
        pl.nchunk3 = (pl.nslot + pl.spb - 1) / pl.spb;
        if (pl.nchunk3 < 1) pl.nchunk3 = 1;
        pl.off_logits = 0;
        pl.off_part1 = align256(bh * pl.nslot * sizeof(float));
        pl.off_part3 = pl.off_part1 + align256(bh * pl.nchunk1 * 3 * sizeof(float));
        pl.bytes = pl.off_part3 + align256(bh * pl.nchunk3 * d.D * sizeof(float));
    }
    return pl;
}

hipError_t launch_decode(const Dims& d, const DecodePlan& pl, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* sel_pages, const int32_t* sel_count, int sel_stride,
                         float alpha, const DecodeHeads& io, char* ws, hipStream_t s) {
    int mode;
    float beta = 0.0f;
    if (alpha == 1.0f) {
        mode = kModeSoftmax;
    } else {
        beta = 1.0f / (alpha - 1.0f);
        mode = (beta == 1.0f) ? kModeBeta1 : (beta == 2.0f ? kModeBeta2 : kModeGeneral);
    }
    return (d.kv_bf16 ? launch_decode_bf16 : launch_decode_f32)(d, pl, q, k_cache, v_cache, page_table, seq_lens,
                                                               sel_pages, sel_count, sel_stride, alpha, mode, beta,
                                                               io, ws, s);
}

}  // namespace ekv
