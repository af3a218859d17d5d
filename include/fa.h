/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * Exact attention O = softmax(scale * Q K^T) V, computed in one streaming
 * pass with an online softmax so that the score matrix S and the
 * probability matrix P never reach device memory, in the forms below (the
 * last one, the unfused contrast, is the exception and writes both):
 *
 *   fa_fwd           prefill / training forward over contiguous Q, K, V.
 *   fa_bwd           training backward: dQ, dK, dV from the forward's O and
 *                    LSE, with P re-computed on chip (never stored).
 *   fa_paged_decode  one query token per request against a paged KV cache,
 *                    split over workgroups and merged by log-sum-exp.
 *   fa_paged_decode_noalloc  the same with the library's built-in
 *                    workspace, for callers that cannot allocate.
 *   fa_paged_decode_fp8kv  the same over a cache stored as e4m3 codes with
 *                    per-tensor scales (half the bytes to read).
 *   fa_paged_prefill chunked prefill: a block of new query tokens per
 *                    request against its paged KV cache.
 *   fa_naive_attention  the pages' three-kernel contrast: S and P
 *                    materialised in device memory (for measurement).
 *
 * Sources (cited by page and section):
 *   [FA3-guide]  "Flash Attention 3 指南：GPU IO 优化的终极武器"
 *                (guijiagi.com): the fp8 forward listing.
 *   [FA3-paged]  "FlashAttention V3 实战：Hopper 架构下的 Paged KV Cache
 *                协同优化" (ybb.press): §一 (the attention definition),
 *                §3.1 (online softmax with tiling), §3.2 (paged KV cache).
 *   [Capstone]   "项目三：榨干片上 SRAM——CUDA Softmax 与 Attention 算子
 *                极致性能调优" (lilinji.mintlify.site): §1.1 (definition),
 *                §2.2 (online softmax and the two-block merge), §4.1-4.2
 *                (Q-outer loop order, deferred normalisation), §7.3 Q2
 *                (causal tile skipping), appendix A Q1 (merge proof).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory on the current HIP device,
 *   allocated and owned by the caller, contiguous in the layout stated,
 *   16-byte aligned (4-byte for fp32 LSE and the int32 tables).
 *   The library never allocates, frees or keeps a pointer, and keeps no
 *   state between calls: calls from several host threads are safe. (The
 *   one exception, fa_paged_decode_noalloc, uses a workspace built into the
 *   library and documents the rules that come with it.)
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *   stream) and runs asynchronously: outputs are valid once the stream has
 *   reached the call. Nothing inside synchronises with the host, allocates
 *   or records a memset, so the calls may be captured into a HIP graph
 *   (replays read the captured pointers; workspace contents on entry never
 *   matter).
 * - Inputs are read-only. Outputs are fully overwritten.
 * - Return value: FA_OK (0) on success. A negative FA_E* code means the
 *   arguments were rejected before anything was launched and nothing was
 *   written. A positive value is a hipError_t reported by the launch.
 *   No C++ exception or abort crosses this boundary.
 * - LSE is the natural-log log-sum-exp of the scaled scores of a row,
 *   LSE = m + ln(l) with m the row maximum and l = sum exp(s - m): the pair
 *   (m, l) the pages keep per row ([Capstone §6.1], the row about not
 *   writing P), folded into one fp32 number. A row that sees no key gets
 *   O = 0 and LSE = -inf.
 * - Head dimension d is 64 or 128.
 */
#ifndef EXACT_ATTENTION_FA_H
#define EXACT_ATTENTION_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of Q, K, V (fa_fwd `dtype`). */
#define FA_DTYPE_F32 0      /* fp32 in, fp32 O                              */
#define FA_DTYPE_BF16 1     /* bf16 in, bf16 O (fp32 accumulation)          */
#define FA_DTYPE_FP8_E4M3 2 /* OCP float8 e4m3fn in + per-tensor fp32
                               scales, bf16 O                               */

/* Return codes. */
#define FA_OK 0
#define FA_EINVAL_NULL (-1)     /* a required pointer is NULL               */
#define FA_EINVAL_DIM (-2)      /* a size is <= 0, or a product overflows   */
#define FA_EUNSUPPORTED_D (-3)  /* head dimension not 64 or 128             */
#define FA_EGQA (-4)            /* Hq not a multiple of Hkv, or group too big*/
#define FA_EDTYPE (-5)          /* unknown dtype                            */
#define FA_EDESCALE (-6)        /* fp8 without descales, or descales given
                                   for another dtype, or a descale <= 0     */
#define FA_ESCALE (-7)          /* softmax scale not finite or not > 0      */
#define FA_EPAGE (-8)           /* unsupported page size / page count       */
#define FA_EWORKSPACE (-9)      /* workspace missing or too small           */
#define FA_ESPLITS (-10)        /* num_splits < 0 or > 65536                */
#define FA_EALIGN (-11)         /* a tensor pointer is not 16-byte aligned
                                   (4-byte for lse, block_table, seq_lens) */
#define FA_ESCRATCH (-12)       /* fa_paged_decode_noalloc: the sizes need
                                   more than the built-in workspace        */

/*
 * fa_fwd - exact attention forward, prefill / training shape.
 *
 * Computes, for every batch b, query head h and query row i,
 *   S_ij = scale * <Q[b,h,i,:], K[b,h/(Hq/Hkv),j,:]>     ([Capstone §1.1])
 *   O[b,h,i,:] = sum_j softmax_j(S_i.) V[b,h/(Hq/Hkv),j,:]
 *   LSE[b,h,i] = ln sum_j exp(S_ij)
 * in a single pass over K/V tiles with the online-softmax recurrence of
 * [Capstone §2.2] in the Q-outer order with deferred 1/l of [Capstone
 * §4.1-4.2]. S and P stay on chip.
 *
 * q      [B, Hq,  Nq, d]  element type `dtype`
 * k, v   [B, Hkv, Nk, d]  element type `dtype`
 * o      [B, Hq,  Nq, d]  fp32 for FA_DTYPE_F32, bf16 otherwise
 * lse    [B, Hq,  Nq]     fp32; may be NULL when LSE is not wanted
 * Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv) (grouped-query
 *   attention; Hq == Hkv is plain multi-head attention).
 * scale  finite and > 0 (the pages use 1/sqrt(d)).
 * causal non-zero: key j is visible to query i iff j <= i + (Nk - Nq)
 *   (bottom-right aligned; the lower triangle when Nq == Nk, [Capstone
 *   §7.3 Q2]). KV tiles wholly above the diagonal are skipped. Rows that
 *   see no key (only possible when Nq > Nk) get O = 0, LSE = -inf.
 * qkv_descale  HOST pointer to three floats (s_q, s_k, s_v), each > 0:
 *   the real inputs are code * s ([FA3-guide] fp8 listing, with a
 *   per-tensor scale). Required for FA_DTYPE_FP8_E4M3, must be NULL for the
 *   other dtypes. Read during the call only.
 *   In the fp8 path, P is rounded to e4m3 (unscaled) before the P.V
 *   product, as in the [FA3-guide] fp8 listing; l is summed in fp32.
 * stream hipStream_t or NULL.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
           int causal, int dtype, const float* qkv_descale, void* stream);

/*
 * fa_bwd_workspace_size - bytes of device workspace fa_bwd needs for
 * B * Hq * Nq query rows (two fp32 values per row plus padding); 0 when a
 * size is not positive. Contents on entry do not matter.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Nq);

/*
 * fa_bwd - exact attention backward ([Capstone §6.1], the row about writing
 * P to HBM, and §7.3 question 1: the forward keeps no P, so the backward
 * re-computes it on chip from Q, K and the saved row statistics).
 *
 * With S, P the scaled scores and probabilities of fa_fwd (same mask) and
 * dO = dL/dO, computes the gradient of the definition:
 *   dV[b,g] = sum over the query heads h of group g of P^T dO
 *   dQ[b,h] = scale * dS K,   dK[b,g] = scale * sum_h dS^T Q,
 *   dS = P * (dP - D),  dP = dO V^T,  D_i = sum_d dO[i,d] * O[i,d]
 * where P_ij = exp(S_ij - LSE_i) is re-computed from Q, K and the LSE that
 * fa_fwd returned. Deterministic (no atomics).
 *
 * q, o, dout  [B, Hq,  Nq, d] bf16 (o: the forward's output)
 * k, v        [B, Hkv, Nk, d] bf16
 * lse         [B, Hq,  Nq] fp32, the forward's LSE (-inf rows get zero
 *             gradients)
 * dq          [B, Hq,  Nq, d] bf16, written (fp32 accumulation, rounded once)
 * dk, dv      [B, Hkv, Nk, d] bf16, written
 * Hq % Hkv == 0; scale finite and > 0; causal as in fa_fwd.
 * dtype       FA_DTYPE_BF16 (the only one supported; others -> FA_EDTYPE)
 * workspace   device memory of at least fa_bwd_workspace_size(B, Hq, Nq)
 *             bytes, 256-byte aligned; workspace_bytes its true size.
 * stream      hipStream_t or NULL.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
           int causal, int dtype, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * fa_paged_decode_workspace_size - bytes of device workspace that
 * fa_paged_decode needs for these arguments (always > 0 for valid ones).
 * num_splits: 0 = let the library choose (the same choice fa_paged_decode
 * makes for the same arguments on the same current device), else the
 * number of page ranges (see fa_paged_decode). The size grows linearly with
 * B + ranges. Returns 0 for arguments fa_paged_decode would reject.
 */
size_t fa_paged_decode_workspace_size(int B, int Hq, int Hkv, int d,
                                      int max_pages_per_seq, int page_size,
                                      int num_splits);

/*
 * fa_paged_decode - one query token per request against a paged KV cache
 * ([FA3-paged §3.2]: each request's cache lives in fixed-size pages that a
 * per-request table maps to physical slots, like virtual memory).
 *
 * For request b with L = seq_lens[b] cached tokens, logical page p holds
 * tokens p*page_size .. p*page_size+page_size-1 in physical page
 * block_table[b, p]. The query attends to all L tokens (no mask inside the
 * context; slots of the last page at or past L are ignored).
 *
 * Split-KV: the pages of all requests, in request order, are cut into R
 * ranges of equal page count, and each (range, KV head) is processed by
 * one wave. A request that lies inside one range gets its output from that
 * wave directly; a request cut by range borders gets a normalised partial
 * output and its LSE from each range, merged with the log-sum-exp form of
 * the two-block merge identity ([Capstone §2.2 step 4], appendix A Q1).
 *
 * q            [B, Hq, d] bf16 (one token per request)
 * k_pool,
 * v_pool       [num_pages, page_size, Hkv, d] bf16 (token-major pages)
 * block_table  [B, max_pages_per_seq] int32, row-major, device memory.
 *              Entries past ceil(L/page_size) are never read.
 * seq_lens     [B] int32, device memory. Values are clamped to
 *              [0, max_pages_per_seq*page_size]. L = 0 gives O = 0 and
 *              LSE = -inf for that request.
 *              A referenced page id outside [0, num_pages) is never
 *              dereferenced: that request's O and LSE become NaN.
 * page_size    16.
 * num_pages    number of pages in each pool (for the bounds check above).
 * Hq % Hkv == 0 and Hq / Hkv <= 16; B * max_pages_per_seq <= 2^31 - 1.
 * scale        finite and > 0.
 * o            [B, Hq, d] bf16; lse [B, Hq] fp32 or NULL.
 * workspace    device memory of at least
 *              fa_paged_decode_workspace_size(B, Hq, Hkv, d,
 *              max_pages_per_seq, page_size, num_splits) bytes, 256-byte
 *              aligned. Its contents on entry do not matter. Two calls that
 *              run concurrently must not share a workspace.
 * workspace_bytes  the true size of the buffer `workspace` points to. The
 *              library checks it against the size it needs and cannot check
 *              it against the allocation: a value larger than the buffer
 *              lets the kernels write past its end.
 * num_splits   0 = auto (about one wave per (range, KV head) for every
 *              wave the GPU holds at once), else R, the number of page
 *              ranges, 1..65536 (rounded up to a multiple of the ranges one
 *              workgroup holds). Any R gives the same result up to fp32
 *              rounding.
 * stream       hipStream_t or NULL.
 */
int fa_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int page_size, int num_pages, int B, int Hq, int Hkv,
                    int d, int max_pages_per_seq, float scale, void* o,
                    float* lse, void* workspace, size_t workspace_bytes,
                    int num_splits, void* stream);

/*
 * fa_paged_decode_noalloc - fa_paged_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. It calls no allocating routine;
 * the split partials live in a workspace built into the library instead of
 * a caller buffer: a 16 MiB array that every device the library runs on
 * holds once, from the first call on that device until the process ends.
 *
 * Arguments, results and errors as fa_paged_decode, without `workspace`
 * and `workspace_bytes`, plus:
 * num_splits   0 = auto: the range count fa_paged_decode would choose,
 *              lowered (to a multiple of the ranges one workgroup holds)
 *              until the partials fit the built-in workspace; the result is
 *              the same up to fp32 rounding. An explicit count whose
 *              partials do not fit -> FA_ESCRATCH.
 * FA_ESCRATCH  the sizes need more than the built-in workspace even with
 *              the fewest ranges (about (B + ranges) * Hq * (d + 1) * 4
 *              bytes must fit in 16 MiB).
 * All calls on one device share its built-in workspace, which keeps the
 * last call's contents (a call never reads what an earlier call left):
 * calls that may run at the same time on one device (from different
 * streams or host threads) race on it and must be serialised by the
 * caller. A positive return is also possible from the first call on a
 * device, when the workspace's device address cannot be looked up.
 */
int fa_paged_decode_noalloc(const void* q, const void* k_pool,
                            const void* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, int page_size,
                            int num_pages, int B, int Hq, int Hkv, int d,
                            int max_pages_per_seq, float scale, void* o,
                            float* lse, int num_splits, void* stream);

/*
 * fa_paged_decode_fp8kv - fa_paged_decode over a KV cache stored as OCP
 * e4m3 codes with one fp32 scale per pool: the cached values are
 * K = code_k * s_k and V = code_v * s_v (the per-tensor scaling of the
 * [FA3-guide] fp8 listing applied to the paged cache of [FA3-paged §3.2]).
 * The query stays bf16 and the result is exact attention over those
 * values: the codes are widened exactly in registers, s_k is folded into
 * the score scale and s_v into the final normalisation.
 *
 * Arguments as fa_paged_decode, except:
 * k_pool,
 * v_pool       [num_pages, page_size, Hkv, d] e4m3 codes (one byte each)
 * kv_descale   HOST pointer to two floats (s_k, s_v), finite and > 0;
 *              NULL or a bad value -> FA_EDESCALE. Read during the call.
 * workspace    sized by fa_paged_decode_workspace_size (the same plan).
 */
int fa_paged_decode_fp8kv(const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, int page_size,
                          int num_pages, int B, int Hq, int Hkv, int d,
                          int max_pages_per_seq, float scale,
                          const float* kv_descale, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int num_splits, void* stream);

/*
 * fa_paged_prefill - exact attention of Nq new query tokens per request
 * against the request's paged KV cache (chunked prefill: the serving use
 * of the paged cache of [FA3-paged §3.2]), in the fused single pass of
 * fa_fwd (S and P stay on chip).
 *
 * Request b's cache holds L = seq_lens[b] tokens (clamped to
 * [0, max_pages_per_seq * 16]) in the pages block_table[b, 0..ceil(L/16)),
 * and q holds its last Nq positions, L-Nq .. L-1 (they are already in the
 * cache). causal non-zero: query i sees keys j <= i + L - Nq (bottom-right
 * alignment; rows with i + L - Nq < 0 see no key: O = 0, LSE = -inf);
 * zero: every query sees all L keys.
 *
 * q            [B, Hq, Nq, d] bf16
 * k_pool,
 * v_pool       [num_pages, page_size, Hkv, d] bf16 (as fa_paged_decode)
 * block_table  [B, max_pages_per_seq] int32; entries past ceil(L/16) are
 *              not read; max_pages_per_seq <= 8192. A referenced page id
 *              outside [0, num_pages) is not dereferenced: that request's
 *              O and LSE become NaN.
 * seq_lens     [B] int32
 * page_size    16.  Hq % Hkv == 0; scale finite and > 0.
 * o            [B, Hq, Nq, d] bf16; lse [B, Hq, Nq] fp32 or NULL.
 * No workspace. stream hipStream_t or NULL.
 */
int fa_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int page_size, int num_pages, int B, int Hq, int Hkv,
                     int Nq, int d, int max_pages_per_seq, float scale,
                     int causal, void* o, float* lse, void* stream);

/*
 * fa_naive_workspace_size - bytes of workspace fa_naive_attention needs:
 * the B*Hq*Nq*Nk score matrix at 2 bytes per score. 0 for sizes <= 0.
 */
size_t fa_naive_workspace_size(int B, int Hq, int Nq, int Nk);

/*
 * fa_naive_attention - the same result as fa_fwd (bf16), computed the way
 * the pages' contrast does it ([Capstone §0] and §1.1): three kernels with
 * the score matrix S and the probabilities P written to and read back from
 * device memory, 8*Nq*d + 8*Nq*Nk bytes per head (2-byte elements) instead
 * of the fused kernel's single pass. Kept for measurement; use fa_fwd.
 *   kernel 1: S = scale * Q K^T, stored as fp16 in `workspace`
 *   kernel 2: per row, the three-pass safe softmax ([Capstone §2.1]) with
 *             the causal mask; P (bf16) written over S's row, LSE written
 *   kernel 3: O = P V
 * Arguments as fa_fwd with dtype bf16, plus:
 * Nk           a multiple of 8, at most 16384.
 * workspace    device memory of fa_naive_workspace_size(B, Hq, Nq, Nk)
 *              bytes, 256-byte aligned (contents on entry do not matter);
 *              workspace_bytes its true size.
 */
int fa_naive_attention(const void* q, const void* k, const void* v, void* o,
                       float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                       int d, float scale, int causal, void* workspace,
                       size_t workspace_bytes, void* stream);

/* fa_strerror - static, NUL-terminated description of a return code. */
const char* fa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_FA_H */
