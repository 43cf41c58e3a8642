/*
 * ekv.h -- C ABI of libekv: support-aware sparse alpha-entmax decode over a
 * paged, GQA-shared KV cache on AMD MI355X (gfx950).
 *
 * Method: "EntmaxKV: Support-Aware Decoding for Entmax Attention" (Duarte,
 * Couceiro, Treviso; arXiv 2605.21649), below [EKV].  One decode step for a
 * batch of single-token queries is
 *
 *     ekv_score_pages  ->  ekv_select  ->  ekv_entmax_decode
 *
 * on page statistics that ekv_build_page_stats writes once per page (at
 * prefill, or when a page fills).  [EKV] section 4.1 is the pipeline,
 * section 4.2 the page scoring, section 4.3 the two selection policies,
 * section 4.4 the hand-off of selected page indices (and the threshold
 * estimate) from selection to decode without a host round trip.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every pointer argument other than `shape`, `workspace_bytes` and the
 *    returned strings is a DEVICE pointer on the current HIP device.  The
 *    library never allocates, frees, copies to or from the host, or
 *    synchronises; every kernel is enqueued on `stream` (a hipStream_t passed
 *    as void*, NULL = the legacy default stream).  The caller owns all memory.
 *  - Argument checks run on the host before anything is enqueued; a failed
 *    check returns an error code and leaves every buffer untouched.
 *    ekv_last_error() then returns a message (thread-local).
 *  - Launch failures return EKV_ERR_HIP.  Outputs are undefined after any
 *    error.
 *  - Non-finite inputs are not detected; they propagate.
 *  - Calls on one stream may be enqueued back to back; the library is
 *    stateless and reentrant.  Calls that share a workspace buffer must be
 *    ordered (same stream, or synchronised by the caller).
 *  - Workspace: an entry point that takes `workspace` reports the bytes it
 *    needs in *workspace_bytes and returns EKV_OK without enqueuing anything
 *    when `workspace` is NULL; when `workspace` is not NULL, *workspace_bytes
 *    must hold its size and a size below the need returns EKV_ERR_WORKSPACE.
 *    The workspace must be 256-byte aligned.
 *
 * Layout (row-major, innermost index last)
 * -----------------------------------------
 *   B = batch, HQ = num_q_heads, G = num_kv_groups, r = HQ/G, D = head_dim,
 *   P = page_size, MP = max_pages_per_seq, NP = num_phys_pages.
 *   q           [B][HQ][D]          kv_dtype
 *   k_cache     [NP][G][P][D]       kv_dtype   (one page-group tile contiguous)
 *   v_cache     [NP][G][P][D]       kv_dtype
 *   page_table  [B][MP]             int32, logical page -> physical page
 *   seq_lens    [B]                 int32, tokens of each sequence (0..MP*P)
 *   kmin, kmax  [NP][G][D]          kv_dtype   (exact per-channel min / max)
 *   kmean, kvar [NP][G][D]          stat_dtype (per-channel mean / variance)
 * Sequence b has M_b = ceil(seq_lens[b]/P) logical pages; logical page p holds
 * tokens [pP, min((p+1)P, seq_lens[b])).  Query head h reads group
 * floor(h / r) (consecutive heads share a group).  Slots of a last page beyond
 * the sequence end are never read.
 */
#ifndef EKV_H
#define EKV_H

#include <stddef.h>
#include <stdint.h>

/* ABI version of this header (ekv_abi_version() returns it). */
#define EKV_ABI_VERSION 6

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EKV_OK = 0,
    EKV_ERR_INVALID_ARG = 1,   /* null pointer, inconsistent shape, bad value */
    EKV_ERR_UNSUPPORTED = 2,   /* valid request outside what is built        */
    EKV_ERR_WORKSPACE = 3,     /* workspace smaller than reported need       */
    EKV_ERR_HIP = 4            /* a HIP launch or runtime call failed        */
} ekv_status;

/* EKV_FP8_E4M3 (statistics storage only): OCP FP8 E4M3 -- 1 sign, 4 exponent
 * bits (bias 7), 3 mantissa bits, no infinities, S.1111.111 = NaN, largest
 * finite 448.  Written by rounding the fp32 statistic to nearest even;
 * finite magnitudes beyond 448 saturate to 448. */
typedef enum { EKV_F32 = 0, EKV_BF16 = 1, EKV_FP8_E4M3 = 2 } ekv_dtype;

typedef enum {
    EKV_SEL_TOPK = 0,     /* [EKV] section 4.3 "Top-k page selection"            */
    EKV_SEL_GAUSS = 1,    /* [EKV] section 4.3 "Gaussian-aware entmax selection"  */
    EKV_SEL_SUPERSET = 2  /* [EKV] Appendix B.2 support-superset selection        */
} ekv_selector;

/* Problem shape.  Supported: D in {64, 128}; P == 16; r in {1, 2, 4, 8};
 * G <= 16; kv_dtype in {EKV_F32, EKV_BF16}; stat_dtype in {EKV_F32, EKV_BF16,
 * EKV_FP8_E4M3}. */
typedef struct {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_groups;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages_per_seq;
    int32_t num_phys_pages;
    int32_t kv_dtype;     /* ekv_dtype of q, k_cache, v_cache, kmin, kmax (F32/BF16) */
    int32_t stat_dtype;   /* ekv_dtype of kmean, kvar                      */
} ekv_shape;

/* Page key statistics ([EKV] section 4.2 and Appendix B.1 for the per-channel
 * min/max; mean and variance are the page statistics the Gaussian selector of
 * section 4.3 reads).  For each listed logical page of each sequence, over
 * the page's valid tokens only, per group and channel:
 *   kmin/kmax = exact min/max of the stored keys (same dtype, bit-exact),
 *   kmean     = (1/n_p) sum k,   kvar = (1/n_p) sum (k - kmean)^2
 *               (fp32 accumulation in token order; rounded to stat_dtype).
 * Results are written at the page's PHYSICAL index.
 *   page_list : NULL = every logical page of every sequence; otherwise n_list
 *               device entries b*MP + p (negative entries, entries with
 *               b >= B or p >= M_b, and pages whose page_table entry lies
 *               outside [0, NP) are skipped).
 *   kmin,kmax : may both be NULL (not written); kmean,kvar likewise; not all
 *               four NULL.
 * Not on the per-step path: run at prefill or when a page fills.          */
ekv_status ekv_build_page_stats(const ekv_shape* shape, const void* k_cache,
                                const int32_t* page_table, const int32_t* seq_lens,
                                const int32_t* page_list, int32_t n_list,
                                void* kmin, void* kmax, void* kmean, void* kvar,
                                void* stream);

/* Append one decoded token per sequence and refresh the statistics of the
 * page it lands in (the step on the other side of the path: every decode
 * step writes one key/value per sequence into the writable page, whose
 * metadata must then cover it; [EKV] section 4.1 costs page metadata per page,
 * and section 4.2 defines it).
 *   k_new, v_new [B][G][D] kv_dtype: the new token's key and value per group.
 *   For each sequence b with n = seq_lens[b]: the token is written at
 *   logical position n (page n/P, slot n%P, through page_table, which must
 *   already map that page); then the statistics of that page are recomputed
 *   from its n%P + 1 tokens with the same arithmetic as ekv_build_page_stats,
 *   so they equal a full rebuild bit for bit.  kmin/kmax and kmean/kvar may
 *   each be NULL (in pairs) to skip them.
 *   new_lens [B] int32 (NULL ok, must not alias seq_lens): n + 1, or n for a
 *   sequence that was left untouched because page n/P is beyond the table
 *   (n >= MP*P) or maps outside [0, NP).
 * seq_lens itself is not modified.                                          */
ekv_status ekv_append_kv(const ekv_shape* shape, const void* k_new, const void* v_new,
                         const int32_t* page_table, const int32_t* seq_lens, void* k_cache, void* v_cache,
                         void* kmin, void* kmax, void* kmean, void* kvar, int32_t* new_lens, void* stream);

/* Query-aware page scores ([EKV] section 4.2 and Appendix B.1; section 4.3).
 * EKV_SEL_TOPK (reads kmin, kmax; writes score [B][G][MP] fp32):
 *   u_{h,p} = (1/sqrt(D)) sum_i max(q_{h,i} kmax_{p,i}, q_{h,i} kmin_{p,i}),
 *   score_{g,p} = max over the r heads of group g of u_{h,p}.
 * EKV_SEL_GAUSS (reads kmean, kvar; writes mu, sigma [B][HQ][MP] fp32):
 *   mu_{h,p} = (1/sqrt(D)) sum_i q_{h,i} kmean_{p,i},
 *   sigma_{h,p} = sqrt((1/D) sum_i q_{h,i}^2 kvar_{p,i})
 *   (per-head moments of the page's token scores, channels treated as
 *   independent).
 * head_score [B][HQ][MP] fp32 (NULL ok; EKV_SEL_TOPK only, else
 *   EKV_ERR_INVALID_ARG): the per-head box scores u_{h,p} before the pooling
 *   over the group's heads, for inspection (a second, unoptimised launch;
 *   score_{g,p} = max over the group's heads of them, up to fp32 rounding).
 * Entries for p >= M_b are not written.  A page p < M_b whose page_table
 * entry lies outside [0, NP) is not read: it gets score -inf (head_score
 * likewise), or mu -inf and sigma 0 (a point mass below every threshold).
 * Accumulation is fp32.                                                    */
ekv_status ekv_score_pages(const ekv_shape* shape, int32_t selector, const void* q,
                           const int32_t* page_table, const int32_t* seq_lens,
                           const void* kmin, const void* kmax,
                           const void* kmean, const void* kvar,
                           float* score, float* mu, float* sigma, float* head_score,
                           void* stream);

/* Candidate page selection, one page set per (sequence, KV group)
 * ([EKV] section 4.3; Appendix B.2).
 * EKV_SEL_TOPK: the min(budget_pages, M_b) pages with the largest score;
 *   ties go to the lower logical page index.  `alpha`, `z`, mu, sigma unused.
 * EKV_SEL_GAUSS: per head, tau_hat solves the distributional threshold
 *   equation ([EKV] Appendix C.2, Eq. (18))
 *       sum_p n_p E[[(alpha-1) S_p - tau_hat]_+^beta] = 1,
 *       S_p ~ N(mu_{h,p}, sigma_{h,p}^2), beta = 1/(alpha-1),
 *   with the closed-form truncated-normal expectations (alpha in
 *   {2, 3/2, 4/3}; other alpha -> EKV_ERR_UNSUPPORTED).  Page p of group g is
 *   a candidate when max_h (mu_{h,p} - tau_hat_h/(alpha-1)) / sigma_{h,p} >= -z
 *   (the page rule of Eq. (21) is not legible on the page; this is the reading
 *   this library takes); candidates are ranked by that margin (ties to the
 *   lower index) and at most budget_pages are kept; at least one page is kept.
 * EKV_SEL_SUPERSET (alpha > 1): `score` holds the box scores of
 *   EKV_SEL_TOPK scoring (upper bounds on every token score of a page) and
 *   tau_hat is an INPUT: per head, a threshold (x units) no larger than that
 *   head's full-cache entmax threshold -- e.g. the tau that
 *   ekv_entmax_decode returns for any subset of the tokens, which can only be
 *   smaller.  Page p of group g is a candidate when
 *       score_{g,p} >= min_{h in g} tau_hat_h / (alpha-1) - 1e-5 |.|
 *   (the relative slack absorbs fp32 rounding, so it only ever adds pages);
 *   candidates are ranked by score (ties to the lower index), at most
 *   budget_pages kept, at least one.  Whenever no candidate is cut by the
 *   budget, the selection contains every token of the entmax support of every
 *   head of the group, and decoding on it is exact (dropped mass 0).
 * Outputs: sel_pages [B][G][budget_pages] int32 logical indices in ascending
 *   order, unused tail = -1; sel_count [B][G] int32; tau_hat [B][HQ] fp32
 *   (GAUSS: output, may be NULL; SUPERSET: required input).  Needs a
 *   workspace (see conventions).                                            */
ekv_status ekv_select(const ekv_shape* shape, int32_t selector, const int32_t* seq_lens,
                      float alpha, int32_t budget_pages, float z,
                      const float* score, const float* mu, const float* sigma,
                      int32_t* sel_pages, int32_t* sel_count, float* tau_hat,
                      void* workspace, size_t* workspace_bytes, void* stream);

/* Exact alpha-entmax attention over the tokens of the selected pages
 * ([EKV] section 4.1; alpha-entmax of section 2.2):
 *   s_{h,j} = q_h . k_{g(h),j} / sqrt(D) for j in C_tok (valid tokens of the
 *   group's selected pages), x = (alpha-1) s, beta = 1/(alpha-1),
 *   tau_h from sum_j [x_j - tau_h]_+^beta = 1,
 *   p_j = [x_j - tau_h]_+^beta (exact zeros), out_h = sum_j p_j v_{g(h),j}.
 *   alpha == 1 is softmax over C_tok and tau is then the log-partition
 *   log sum_j exp(s_j).  alpha > 1 may be any value; 1.5 and 2 use a closed
 *   form on the support found.
 * sel_pages == NULL selects every page (full-cache decode); otherwise
 *   sel_pages [B][G][sel_stride] logical page indices (ascending not
 *   required) and sel_count [B][G] of them are used.  An index outside
 *   [0, pages of the sequence), or a page whose table entry lies outside
 *   [0, num_phys_pages), contributes no token; a page named twice
 *   contributes its tokens twice (ekv_select never names one twice).
 * tau_hint [B][HQ] fp32 (NULL ok; alpha > 1): a start for the threshold
 *   iteration, in x units -- the selection's threshold estimate, which
 *   [EKV] section 4.4 hands to decode with the selected pages (ekv_select's
 *   EKV_SEL_GAUSS tau_hat).  It is used only where it lies strictly between
 *   max(x) - 1 and max(x) over the head's candidate tokens; the threshold
 *   found is the same, up to fp32 rounding, with or without it.
 * Outputs: out [B][HQ][D] fp32; tau [B][HQ] fp32 (x units; log-partition for
 *   alpha == 1); support [B][HQ] int32 nonzero count (NULL ok);
 *   delta [B][HQ] fp32 (NULL ok; needs tau_ref): dropped mass
 *   1 - sum_{j in C_tok} p_ref_j of the distribution whose threshold is
 *   tau_ref [B][HQ] (e.g. a full-cache decode's tau) ([EKV] section 3.1);
 *   support_ref [B][HQ] int32 (NULL ok; needs tau_ref): the number of tokens
 *   of C_tok with p_ref > 0 (x_j > tau_ref; every token for alpha == 1).
 *   Divided by the full-cache decode's support it is the support recall rho
 *   of [EKV] section 3.1 and Appendix E.1.
 * An empty candidate set (seq_lens[b] == 0 or sel_count == 0) gives
 *   out = 0, tau = -inf, support = 0, delta = 1, support_ref = 0.
 * Rows of more than 2^20 pages (16M tokens: max_pages_per_seq for
 *   sel_pages == NULL, else sel_stride) return EKV_ERR_UNSUPPORTED.
 * Cache slots that hold no token of a sequence (the tail of its last page,
 *   pages no table entry names) may hold any bits, NaN included: no output
 *   depends on them.
 * Needs a workspace (see conventions); its size depends on the shape, on
 * alpha (1 or not), on sel_pages being NULL or not and on sel_stride.      */
ekv_status ekv_entmax_decode(const ekv_shape* shape, const void* q,
                             const void* k_cache, const void* v_cache,
                             const int32_t* page_table, const int32_t* seq_lens,
                             const int32_t* sel_pages, const int32_t* sel_count,
                             int32_t sel_stride, float alpha, const float* tau_hint,
                             const float* tau_ref, float* out, float* tau, int32_t* support,
                             float* delta, int32_t* support_ref,
                             void* workspace, size_t* workspace_bytes, void* stream);

/* Bytes of device scratch that ekv_entmax_decode_noalloc holds per GPU. */
#define EKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/* ekv_entmax_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, computation, outputs
 * and errors as ekv_entmax_decode; it calls no hipMalloc/hipFree and no
 * allocating library routine.  Its scratch is a static device array of
 * EKV_NOALLOC_SCRATCH_BYTES per GPU (one copy per device, held until the
 * process ends, its address looked up on the first call on each device).
 *   - A decode whose workspace need (as ekv_entmax_decode would report it)
 *     exceeds EKV_NOALLOC_SCRATCH_BYTES returns EKV_ERR_WORKSPACE before
 *     enqueuing anything.
 *   - Every call on one GPU uses that GPU's one array: calls whose kernels
 *     overlap on one GPU (different streams, or different host threads
 *     without ordering) race on it and give undefined results.  Calls on one
 *     stream are ordered and safe.  The kernels write every scratch byte
 *     they read, so nothing needs to start at zero.                        */
ekv_status ekv_entmax_decode_noalloc(const ekv_shape* shape, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* page_table, const int32_t* seq_lens,
                                     const int32_t* sel_pages, const int32_t* sel_count,
                                     int32_t sel_stride, float alpha, const float* tau_hint,
                                     const float* tau_ref, float* out, float* tau, int32_t* support,
                                     float* delta, int32_t* support_ref, void* stream);

/* Streaming-read probe (measurement only, not part of a decode step): reads
 * `bytes` of device memory at `buf` (a positive multiple of 4096, 16-byte
 * aligned) in 4 KiB chunks, in order (order == NULL) or in the order of the
 * bytes/4096 device int32 chunk indices in `order` (an entry outside
 * [0, bytes/4096) reads chunk 0).  It gives the read bandwidth the chip
 * achieves for a linear stream and for 4 KiB pieces gathered through an
 * index (the access pattern of page statistics and K tiles reached through
 * a page table), against which the kernels' roofline fractions are read.
 * `blocks` 256-thread blocks each keep `unroll` chunks (2, 4 or 8) in
 * flight.  `sink` is one device uint32, written only if the folded data
 * happens to equal a fixed constant (it keeps the loads live).           */
ekv_status ekv_probe_read(const void* buf, size_t bytes, const int32_t* order, int32_t unroll,
                          int32_t blocks, uint32_t* sink, void* stream);

/* Message describing the last error returned on this thread ("" if none). */
const char* ekv_last_error(void);

/* Library ABI version; equals EKV_ABI_VERSION of the header it was built
 * with. */
int32_t ekv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EKV_H */
