// Sparse alpha-entmax decode: the workspace plan and the dispatch to the
// per-dtype kernel launches (decode_bf16.hip, decode_f32.hip); the kernels
// and what they compute are described in decode_kernels.h.
#include "decode_kernels.h"

namespace ekv {

// ---------------------------------------------------------------- host ----
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodePlan plan_decode(const Dims& d, int sparse, int sel_stride, float alpha) {
    DecodePlan pl;
    pl.sparse = sparse;
    const int maxp = sparse ? sel_stride : d.MP;
    pl.nslot = maxp * kPage;
    pl.fused = sparse && alpha > 1.0f && pl.nslot <= kFusedMaxSlots;
    pl.lg_ppb = sparse ? 3 : 5;
    pl.ppb = 1 << pl.lg_ppb;
    pl.nchunk1 = (maxp + pl.ppb - 1) / pl.ppb;
    if (pl.nchunk1 < 1) pl.nchunk1 = 1;
    pl.spb = sparse ? 256 : 4096;
    pl.nchunk3 = (pl.nslot + pl.spb - 1) / pl.spb;
    if (pl.nchunk3 < 1) pl.nchunk3 = 1;
    const size_t bh = (size_t)d.B * d.HQ;
    pl.off_logits = 0;
    pl.off_part1 = align256(bh * pl.nslot * sizeof(float));
    pl.ncc = 0;
    pl.off_cand = pl.off_ccnt = 0;
    if (pl.fused) {
        pl.off_part3 = pl.off_part1;
        pl.bytes = pl.off_part1;
    } else {
        pl.off_part3 = pl.off_part1 + align256(bh * pl.nchunk1 * 3 * sizeof(float));
        pl.bytes = pl.off_part3 + align256(bh * pl.nchunk3 * d.D * sizeof(float));
        // Entmax over many slots: the threshold candidates are compacted by
        // many blocks (cand_kernel) instead of inside the one block per head.
        const int ncc = (pl.nslot + kCandChunk - 1) / kCandChunk;
        if (alpha > 1.0f && ncc >= 2 && ncc <= kCandMaxChunks) {
            pl.ncc = ncc;
            pl.off_cand = pl.bytes;
            pl.off_ccnt = pl.off_cand + align256(bh * ncc * kCandPerChunk * sizeof(float));
            pl.bytes = pl.off_ccnt + align256(bh * ncc * sizeof(int));
        }
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
