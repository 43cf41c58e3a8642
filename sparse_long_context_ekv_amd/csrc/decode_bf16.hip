// Sparse alpha-entmax decode kernels for bf16 KV caches (see decode_kernels.h).
#include "decode_kernels.h"

namespace ekv {

hipError_t launch_decode_bf16(const Dims& d, const DecodePlan& pl, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                              const int32_t* sel_pages, const int32_t* sel_count, int sel_stride, float alpha,
                              int mode, float beta, const DecodeHeads& io, char* ws, hipStream_t s) {
    return launch_decode_typed<bf16_t>(d, pl, q, k_cache, v_cache, page_table, seq_lens, sel_pages, sel_count,
                                       sel_stride, alpha, mode, beta, io, ws, s);
}

}  // namespace ekv
