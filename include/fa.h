/*
 * fa.h -- C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention tile by tile with an
 * online softmax, so the N x N score matrix never reaches device memory
 * (tiling and online softmax: "FlashAttention-4 Conquers Asymmetric GPU
 * Hardware Scaling", podcast.app episode page, second paragraph of the
 * description). The forward pass writes O and the per-row log-sum-exp; the
 * backward pass recomputes the softmax and writes dQ, dK and dV (backward pass:
 * abstract on the zhuanzhiai.com page). Causal masking and packed
 * variable-length batches follow the daily.dev "Summary" of the Together AI
 * post; grouped K/V heads (Hq a multiple of Hkv) are supported as well.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees or synchronises. Work is enqueued on `stream`
 *    (a hipStream_t; NULL means the default stream) and the call returns at
 *    once. Device faults surface at the caller's next synchronisation.
 *  - bf16 tensors hold IEEE bfloat16 bit patterns; fp32 tensors hold IEEE
 *    binary32. Every tensor is contiguous and 16-byte aligned.
 *  - Uniform batch (cu_seqlens == NULL), "BSHD" layout:
 *        Q, O, dO, dQ : [B, N, Hq, d]      K, V, dK, dV : [B, N, Hkv, d]
 *        LSE          : [B, Hq, N] fp32
 *  - Packed variable-length batch (cu_seqlens != NULL): B sequences of length
 *    L_s = cu_seqlens[s+1] - cu_seqlens[s], packed along the token axis:
 *        Q, O, dO, dQ : [T, Hq, d]         K, V, dK, dV : [T, Hkv, d]
 *        LSE          : [Hq, T] fp32       T = cu_seqlens[B]
 *    cu_seqlens is a device int32 array of B+1 entries with cu_seqlens[0] = 0,
 *    non-decreasing, and every L_s <= N (N is the maximum length). Its contents
 *    are not checked (that would need a synchronisation); breaking these
 *    preconditions is undefined behaviour.
 *  - Query head h reads K/V head h / (Hq / Hkv).
 *  - Causal: key j is masked for query i when j > i (positions within the
 *    sequence; queries and keys have the same length).
 *  - Scores are S = softmax_scale * Q K^T; LSE_i = ln(sum_j exp(S_ij)).
 *  - All arguments are validated on the host before anything is launched; an
 *    invalid argument returns a status code and enqueues nothing.
 *  - Supported head sizes: d = 64 and d = 128.
 *  - Size limits (beyond them a call returns FA_ERR_UNSUPPORTED): at most 2^31
 *    tokens per tensor (B * N, or T), at most 2^24 work items
 *    (B * Hq * ceil(N / 128)), and Hkv * d <= 32768 (Hkv <= 256 at d = 128).
 *  - Entry points are stateless and may be called concurrently from several
 *    host threads.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned pointer, Hq % Hkv != 0, scale not
                                    finite or negative */
    FA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head size other than 64 or 128,
                                    sizes beyond the limits below) */
    FA_ERR_WORKSPACE = 3,        /* backward workspace missing or smaller than fa_bwd_workspace_size() */
    FA_ERR_HIP = 4               /* the HIP runtime reported an error at launch */
} fa_status;

/* Exponential used for the softmax numerators. */
typedef enum {
    FA_EXP_HW = 0,   /* the hardware v_exp_f32 instruction */
    FA_EXP_POLY = 1  /* polynomial on the FMA pipe after an exact split x = n + f
                        (software exponential with Cody-Waite range reduction:
                        daily.dev "Summary") */
} fa_exp_mode;

/* Optional tuning knobs of the forward pass; pass NULL for the defaults. */
typedef struct {
    int exp_mode;        /* fa_exp_mode; default FA_EXP_HW */
    float rescale_tau;   /* conditional rescaling threshold in log2 units ("conditional
                            online softmax rescaling", daily.dev "Summary"): each row
                            keeps its first key tile's max, and only a row whose sum of
                            exp2 terms relative to that max exceeds 2^tau (or is not
                            finite) is recomputed with its exact max. Default 32, which
                            bounds every P by 2^32. Any tau >= 0 gives the same result
                            up to rounding; small values only cost extra passes. */
    int lpt_order;       /* 1 (default): heaviest query tiles first (longest-processing-
                            time-first, daily.dev "Summary"); 0: plain order. */
} fa_fwd_options;

/*
 * Forward attention.
 *   q, k, v      bf16 inputs (layouts above)
 *   o            bf16 output, same shape as q
 *   lse          fp32 output, per-row natural-log log-sum-exp of the scaled scores
 *   B            batch size (uniform) or number of sequences (packed); B >= 0
 *   Hq, Hkv      query and key/value head counts, Hq % Hkv == 0
 *   N            sequence length (uniform) or maximum sequence length (packed); N >= 0
 *   d            head size (64 or 128)
 *   causal       0 or 1
 *   softmax_scale finite scale >= 0 applied to Q K^T (the kernels take the row maxima of
 *                the raw products Q K^T and fold the scale into the exponent, which is
 *                exact only for a non-negative scale; a negative one returns
 *                FA_ERR_INVALID_ARGUMENT)
 *   cu_seqlens   NULL (uniform) or device int32[B+1] (packed)
 *   stream       hipStream_t or NULL
 * B == 0 or N == 0 is a valid empty call and enqueues nothing.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                 const int32_t* cu_seqlens, void* stream);

/* fa_fwd with explicit options (NULL = defaults). */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                    const int32_t* cu_seqlens, const fa_fwd_options* options, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (for packed batches
 * pass the number of sequences as B and the maximum length as N; the bound
 * B * N >= T is used). Returns 0 for empty problems.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int causal, int varlen);

/*
 * Backward attention.
 *   q, k, v, o   bf16 forward inputs and the forward output O
 *   lse          fp32 LSE written by fa_fwd for the same inputs
 *   dout         bf16 upstream gradient dO, same shape as q
 *   dq, dk, dv   bf16 outputs, shaped like q, k, v; dK/dV of a K/V head sum over its
 *                Hq/Hkv query heads
 *   workspace    device scratch of at least fa_bwd_workspace_size(...) bytes, 256-byte
 *                aligned; its contents on entry do not matter and on return are undefined
 * Other arguments as for fa_fwd. Returns FA_ERR_WORKSPACE if the workspace is
 * NULL or too small for a non-empty problem.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                 const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Arguments and
 * results as for fa_bwd, without the workspace: the library keeps it in a fixed
 * device array of fa_bwd_noalloc_max_workspace() bytes (64 MiB), one per GPU,
 * held until the process ends. No call allocates or frees anything.
 *   - Returns FA_ERR_WORKSPACE when fa_bwd_workspace_size(...) for these sizes
 *     exceeds that maximum (for packed batches the bound uses B * N tokens).
 *   - Every call on one GPU uses that GPU's single array: calls that overlap on
 *     one GPU (on different streams, or from several host threads without
 *     ordering) race on it and give undefined results. Calls ordered on one
 *     stream are safe; nothing in the array needs clearing between calls.
 *   - FA_ERR_HIP if the array's device address cannot be obtained.
 */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                         const int32_t* cu_seqlens, void* stream);

/* Size in bytes of fa_bwd_noalloc's fixed workspace array. */
size_t fa_bwd_noalloc_max_workspace(void);

/* Stages of the backward pass, for fa_bwd_ex. */
typedef enum {
    FA_BWD_PREPROCESS = 1,  /* D_i = rowsum(dO o O) and LSE_i * log2(e) into the workspace; for
                               packed batches also the order in which DKDV takes its work */
    FA_BWD_DKDV = 2,        /* dK and dV (read the workspace) */
    FA_BWD_DQ = 4,          /* dQ (reads the workspace) */
    FA_BWD_ALL = 7
} fa_bwd_stage;

/*
 * fa_bwd restricted to the stages in `stages` (a mask of fa_bwd_stage), run in
 * the order PREPROCESS, DKDV, DQ. DKDV and DQ read what PREPROCESS wrote into the
 * same workspace and do not depend on each other, so once PREPROCESS has run
 * they may be enqueued separately (for instance on two streams, ordered after
 * PREPROCESS by the caller). fa_bwd(...) is fa_bwd_ex(..., FA_BWD_ALL, stream).
 * Returns FA_ERR_INVALID_ARGUMENT for a mask outside 1..7.
 */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv,
                    int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                    const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes, int stages,
                    void* stream);

/*
 * Forward attention with 8-bit Q and K (the low-precision variant of
 * FlashAttention's lineage; podcast.app episode page, source list). Q and K
 * hold OCP E4M3 codes (1 byte each, layouts as for fa_fwd); element values are
 * code * q_descale[s, h] and code * k_descale[s, hkv] (fp32, one per sequence
 * and head; s is the batch index, or the sequence index of a packed batch).
 * V is bf16 and O, LSE are as for fa_fwd: the exact attention of the
 * dequantised Q and K, computed with the scores from the 8-bit matrix cores
 * (the products of E4M3 values are exact in the fp32 accumulation).
 *   q_descale  fp32 [B, Hq], device
 *   k_descale  fp32 [B, Hkv], device
 *   d          128 only (other sizes return FA_ERR_UNSUPPORTED)
 * Other arguments and errors as for fa_fwd.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                     void* o, float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                     const int32_t* cu_seqlens, void* stream);

/*
 * fa_fwd_fp8 with explicit options (NULL = defaults). rescale_tau and lpt_order
 * act as for fa_fwd_ex; exp_mode must be FA_EXP_HW (FA_EXP_POLY returns
 * FA_ERR_UNSUPPORTED for the 8-bit kernel).
 */
fa_status fa_fwd_fp8_ex(const void* q, const void* k, const void* v, const float* q_descale,
                        const float* k_descale, void* o, float* lse, int B, int Hq, int Hkv, int N, int d,
                        int causal, float softmax_scale, const int32_t* cu_seqlens,
                        const fa_fwd_options* options, void* stream);

/* Tokens per descale block of fa_fwd_fp8_blockscale, and its largest block count. */
#define FA_FP8_SCALE_BLOCK 64
#define FA_FP8_MAX_BLOCKS 4096

/*
 * fa_fwd_fp8 with one descale per block of 64 tokens of every (sequence,
 * head) instead of one per (sequence, head): finer scaling of the 8-bit
 * inputs (the low-precision variant of FlashAttention's lineage; podcast.app
 * episode page, source list). With nb = ceil(N / FA_FP8_SCALE_BLOCK), N the
 * (maximum) sequence length, the element of token t (position local to its
 * sequence s) and head h has the value
 *   q: code * q_descale[s, h, t / 64]      k: code * k_descale[s, hkv, t / 64]
 *   q_descale  fp32 [B, Hq, nb], device
 *   k_descale  fp32 [B, Hkv, nb], device
 * Descales must be finite and > 0. The exp2 factor of each 32-key tile is
 * softmax_scale * log2(e) times the query's and the tile's descales, folded in
 * once per tile; the result is the exact attention of the dequantised Q and
 * K. Returns FA_ERR_UNSUPPORTED when nb > FA_FP8_MAX_BLOCKS (N > 262144) or
 * d != 128; options, other arguments and errors as for fa_fwd_fp8_ex.
 */
fa_status fa_fwd_fp8_blockscale(const void* q, const void* k, const void* v, const float* q_descale,
                                const float* k_descale, void* o, float* lse, int B, int Hq, int Hkv, int N,
                                int d, int causal, float softmax_scale, const int32_t* cu_seqlens,
                                const fa_fwd_options* options, void* stream);

/*
 * Split-KV partial attention (uniform batches). The keys of every sequence are
 * cut into n_splits contiguous chunks of C = ceil(Nk / n_splits) keys (chunk p:
 * keys p*C .. min((p+1)*C, Nk) - 1; chunks past the end are empty). For every
 * query i and chunk p it writes the attention over that chunk's keys alone:
 *   LSE_p(i) = ln sum_{j in chunk p, visible} exp(scale * q_i . k_j)
 *   O_p(i)   = sum_{j in chunk p, visible} exp(scale * q_i . k_j - LSE_p(i)) v_j
 * and LSE_p(i) = -inf, O_p(i) = 0 where query i sees no key of the chunk.
 * fa_merge of the parts gives the attention over all keys. This is the
 * combination step of the online softmax applied across key chunks
 * (podcast.app episode page, description; Ring Attention in its source list),
 * for long key ranges with few queries (decoding, chunked prefill) and for the
 * per-chunk results of sequence-parallel attention.
 *   q         bf16 [B, Nq, Hq, d]
 *   k, v      bf16 [B, Nk, Hkv, d]
 *   o_part    fp32 [n_splits, B, Nq, Hq, d]   device memory owned by the caller
 *   lse_part  fp32 [n_splits, B, Hq, Nq]      device memory owned by the caller
 *   causal    query i sits at key position i + Nk - Nq (the last query sees
 *             every key); requires Nq <= Nk
 *   n_splits  1 .. 1024
 * Other arguments as for fa_fwd. Returns FA_ERR_INVALID_ARGUMENT for bad
 * sizes, flags or pointers, FA_ERR_UNSUPPORTED for other head sizes.
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale,
                       int n_splits, void* stream);

/*
 * fa_fwd_split with explicit options (NULL = defaults). rescale_tau and
 * lpt_order act as for fa_fwd_ex; exp_mode must be FA_EXP_HW (FA_EXP_POLY
 * returns FA_ERR_UNSUPPORTED for the split kernel).
 */
fa_status fa_fwd_split_ex(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale,
                          int n_splits, const fa_fwd_options* options, void* stream);

/*
 * Merge of partial attention results (the combination step of the online
 * softmax, podcast.app episode page, description), row by row:
 *   LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p
 * Rows whose every part has LSE_p = -inf get LSE = -inf and O = 0.
 *   o_part    fp32 [n_parts, B, N, H, d]   (fa_fwd_split's layout, any producer)
 *   lse_part  fp32 [n_parts, B, H, N]
 *   o         bf16 [B, N, H, d] (output)
 *   lse       fp32 [B, H, N]    (output)
 * A packed [T, H, d] / [H, T] pair is B = 1, N = T. d in {64, 128},
 * n_parts 1 .. 1024. Device pointers, caller-owned; o_part and o, or lse_part
 * and lse, must not overlap. Returns FA_ERR_INVALID_ARGUMENT for bad sizes or
 * pointers, FA_ERR_UNSUPPORTED for other d.
 */
fa_status fa_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                   int n_parts, int B, int H, int N, int d, void* stream);

/*
 * The element-wise exponential the softmax uses, on its own (a check of the
 * kernels' software exponential with range reduction, phantomic12 summary,
 * co-design list; daily.dev Summary): y[i] = 2^x[i] computed by the same
 * device function as the forward pass selects with fa_fwd_options.exp_mode,
 * FA_EXP_HW (v_exp_f32) or FA_EXP_POLY (exact split x = n + f, polynomial in f
 * on the FMA pipe, 2^n applied by v_ldexp_f32; inputs below -125 give 0,
 * inputs at or above 128 give +inf, NaN stays NaN). The backward pass always
 * uses v_exp_f32.
 *   x, y      fp32 [n], device, caller-owned, 4-byte aligned (may not overlap)
 *   n         >= 0 (0 launches nothing)
 * Returns FA_ERR_INVALID_ARGUMENT for n < 0, another mode or bad pointers.
 */
fa_status fa_exp2_eval(const float* x, float* y, int64_t n, int exp_mode, void* stream);

/* Static, human-readable description of a status code. */
const char* fa_status_string(fa_status s);

/* Library version string. */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
