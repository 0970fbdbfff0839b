/*
 * attn.h — C ABI of the MI355X (gfx950) fused-attention library libattn.so.
 *
 * Every entry point computes scaled-dot-product attention with a one-pass
 * online softmax and also returns the per-row log-sum-exp:
 *
 *   O_i   = Σ_j softmax_j(scale · q_i·k_j + mask_ij) · v_j
 *   LSE_i = ln Σ_j exp(scale · q_i·k_j + mask_ij)        (natural log)
 *
 * The pages that define the operation (cited by title and section):
 *  - "05 · Tích vô hướng, Softmax và toán của Attention" (inference-notes):
 *    §1 dot product and the 1/√d scale, §2 softmax, §3 one head one token,
 *    §4 GQA (four query heads share one K/V head), §6 online softmax.
 *  - "AI Infra 入门：RMSNorm、Softmax、Causal Mask、Sampling 的数学与底层优化":
 *    §3 causal mask (−∞ for j > i; tiles above the diagonal skipped, only
 *    diagonal tiles masked), online softmax with running max and running
 *    sum rescaled by exp(m_old − m_new), LSE and split-K merging.
 *  - "Bộ 06 · Bên trong model": Q2 (−∞ not 0; cached K/V are exact),
 *    Q3 (attend only the filled part of a preallocated cache).
 *  - "MLA 矩阵乘法吸收的数值稳定性治理": §一 absorption into the query,
 *    §二 channel scale S and FP32 on-chip accumulation, §五 low-precision
 *    storage with high-precision accumulation.
 *  - "第11节：Attention 实现（Flash vs Fallback）": §3 (the keys are the
 *    cached history followed by the current tokens; the triu(1) causal mask
 *    covers only the current tokens' columns), §4 score shape [B,H,Q,K].
 *
 * Conventions shared by all entry points
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    owned by the caller, contiguous, innermost dimension last (row-major).
 *  - bf16 tensors use the bfloat16 storage format; all products are
 *    accumulated in fp32 and the output is rounded once (round to nearest
 *    even). LSE is fp32.
 *  - Work is enqueued on `stream` (NULL = the default stream) and runs
 *    asynchronously; no entry point synchronises or allocates memory.
 *  - Arguments are validated on the host before anything is enqueued. On
 *    any non-OK status nothing is launched and no output is touched;
 *    attn_last_error() then holds a description (thread-local).
 *  - No C++ exception crosses this interface.
 *  - NaN or Inf in the inputs propagate to the outputs; they are not
 *    detected.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_POINTER = 1, /* a required pointer is NULL                  */
    ATTN_ERR_BAD_SHAPE = 2,    /* a size is out of range or inconsistent      */
    ATTN_ERR_UNSUPPORTED = 3,  /* valid but not implemented (dtype, head dim) */
    ATTN_ERR_WORKSPACE = 4,    /* workspace missing or too small              */
    ATTN_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
} attn_status;

typedef enum attn_dtype {
    ATTN_BF16 = 0,
    ATTN_FP32 = 1
} attn_dtype;

/*
 * Causal prefill: N queries attend to the same N positions with the causal
 * mask (key j is visible to query i iff j <= i).
 *
 *   q   [B, Hq,  N, D]   dtype
 *   k   [B, Hkv, N, D]   dtype
 *   v   [B, Hkv, N, D]   dtype
 *   o   [B, Hq,  N, D]   dtype (output)
 *   lse [B, Hq,  N]      fp32  (output, natural log)
 *
 * Query head hq uses K/V head hq / (Hq/Hkv) (contiguous GQA groups).
 * dtype ATTN_BF16: D in {64, 128}; MFMA bf16 products, fp32 accumulation.
 * dtype ATTN_FP32: D in {64, 128}; fp32 throughout.
 * scale multiplies every score (1/√D for plain attention); it must be finite
 * and > 0.
 * Errors: NULL pointer → ATTN_ERR_NULL_POINTER; B, Hq, Hkv, N < 1 or
 * Hq % Hkv != 0, a tensor above 2^31 elements, or a scale that is not finite
 * and positive → ATTN_ERR_BAD_SHAPE;
 * other D or dtype → ATTN_ERR_UNSUPPORTED; launch failure → ATTN_ERR_HIP.
 */
attn_status attn_prefill_causal(attn_dtype dtype, const void *q, const void *k,
                                const void *v, void *o, float *lse, int B,
                                int Hq, int Hkv, int N, int D, float scale,
                                hipStream_t stream);

/*
 * Backward of attn_prefill_causal (bf16, D = 128): given the forward's
 * inputs, its output o and per-row lse, and the upstream gradient
 * dout = ∂L/∂O, writes
 *   dq = scale·dS·K,  dk = scale·dSᵀ·Q,  dv = Pᵀ·dout,
 * with P = exp(scale·q·k − lse) recomputed from the stored LSE ("AI Infra
 * 入门…", §3: the LSE lets the backward recompute P exactly) and
 * dS = P ∘ (dout·Vᵀ − rowsum(dout ∘ o)); dk and dv sum over the Hq/Hkv query
 * heads sharing each K/V head. All products accumulate in fp32; each
 * gradient is rounded once to bf16. Deterministic (no atomics).
 *
 *   q, o, dout, dq  [B, Hq,  N, D]   bf16 (dq: output)
 *   k, v, dk, dv    [B, Hkv, N, D]   bf16 (dk, dv: outputs)
 *   lse             [B, Hq,  N]      fp32, natural log, as written by the forward
 *   workspace       attn_prefill_causal_backward_workspace_bytes() bytes
 *                   (16-byte aligned; contents on entry do not matter)
 *
 * Errors: NULL pointer → ATTN_ERR_NULL_POINTER; B, Hq, Hkv, N < 1,
 * Hq % Hkv, a tensor above 2^31 elements or a bad scale → ATTN_ERR_BAD_SHAPE;
 * D != 128 or misaligned tensors → ATTN_ERR_UNSUPPORTED; workspace too small
 * → ATTN_ERR_WORKSPACE; launch failure → ATTN_ERR_HIP.
 */
attn_status attn_prefill_causal_backward(const void *q, const void *k,
                                         const void *v, const void *o,
                                         const float *lse, const void *dout,
                                         void *dq, void *dk, void *dv, int B,
                                         int Hq, int Hkv, int N, int D,
                                         float scale, void *workspace,
                                         size_t workspace_bytes,
                                         hipStream_t stream);

/* Bytes of workspace attn_prefill_causal_backward needs (0 if invalid). */
size_t attn_prefill_causal_backward_workspace_bytes(int B, int Hq, int N, int D);

/*
 * Chunked prefill against a K/V cache: for each sequence, Nq new tokens whose
 * K/V are already appended to the cache attend to the whole filled cache.
 * Sequence b's cache holds kv_lens[b] positions; its last Nq are the chunk's
 * own tokens, so chunk row i sits at position P + i with P = kv_lens[b] − Nq,
 * and key j is visible to it iff j <= P + i (every history key, and chunk
 * keys 0..i: the bottom-right-aligned causal mask). Slots at or past
 * kv_lens[b] are never read.
 *
 *   q        [B, Hq, Nq, D]          bf16
 *   k_cache  [B, Hkv, kv_cap, D]     bf16
 *   v_cache  [B, Hkv, kv_cap, D]     bf16
 *   o        [B, Hq, Nq, D]          bf16 (output)
 *   lse      [B, Hq, Nq]             fp32 (output, natural log)
 *   kv_lens  [B]                     int32, DEVICE memory, read by the kernel
 *            at run time (so a captured graph can be replayed with new
 *            lengths); each value must lie in [Nq, kv_cap] — values outside
 *            are clamped into that range, they are not reported.
 *
 *   workspace  attn_prefill_chunked_workspace_bytes() bytes, 16-byte aligned
 *            (contents on entry do not matter). When the chunk's query
 *            tiles alone would leave compute units idle (short chunks), the
 *            keys are split over several workgroups whose fp32 partials go
 *            here and are merged through their log-sum-exp by a second
 *            kernel on the same stream.
 *
 * Query head hq uses K/V head hq / (Hq/Hkv). D must be 128. Nq = 1 is a
 * decode step; Nq = kv_lens[b] with kv_cap = Nq is attn_prefill_causal.
 * Errors: NULL pointer → ATTN_ERR_NULL_POINTER; B, Hq, Hkv, Nq < 1,
 * Hq % Hkv, Nq > kv_cap, a tensor above 2^31 elements, or a scale that is
 * not finite and positive → ATTN_ERR_BAD_SHAPE; other D → ATTN_ERR_UNSUPPORTED;
 * workspace NULL or too small → ATTN_ERR_WORKSPACE; launch failure →
 * ATTN_ERR_HIP.
 */
attn_status attn_prefill_chunked(const void *q, const void *k_cache,
                                 const void *v_cache, void *o, float *lse,
                                 const int *kv_lens, int B, int Hq, int Hkv,
                                 int Nq, int kv_cap, int D, float scale,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Bytes of workspace attn_prefill_chunked needs (0 if invalid). */
size_t attn_prefill_chunked_workspace_bytes(int B, int Hq, int Nq, int kv_cap,
                                            int D);

/*
 * Single-query GQA decode over a bf16 K/V cache (no mask: the one query sees
 * every cached position). Only the first kv_len slots are read; slots
 * kv_len..kv_cap-1 are never touched (they may hold anything). kv_len counts
 * the current token: its K/V must already be in the cache.
 *
 *   q        [B, Hq, D]               bf16
 *   k_cache  [B, Hkv, kv_cap, D]      bf16
 *   v_cache  [B, Hkv, kv_cap, D]      bf16
 *   o        [B, Hq, D]               bf16 (output)
 *   lse      [B, Hq]                  fp32 (output, natural log)
 *   workspace: device memory of at least attn_decode_gqa_workspace_bytes()
 *              bytes (16-byte aligned). Its contents on entry do not matter:
 *              it carries the per-split partial results from the split pass
 *              to the merge pass of the same call. Calls that may run
 *              concurrently must not share a workspace.
 *
 * The cache is split into chunks processed by separate workgroups, each
 * producing a partial (O, running max, running sum); a second kernel on the
 * same stream merges the partials through their log-sum-exp. The split
 * depends only on the shape (and the cache type), so results are bitwise
 * reproducible.
 * D must be 128 and Hq/Hkv at most 16.
 * Errors: NULL pointer → ATTN_ERR_NULL_POINTER; B, Hq, Hkv < 1, Hq % Hkv,
 * kv_len < 1 or kv_len > kv_cap, or a scale that is not finite and positive
 * → ATTN_ERR_BAD_SHAPE; other D or group size
 * → ATTN_ERR_UNSUPPORTED; workspace NULL or too small → ATTN_ERR_WORKSPACE;
 * launch failure → ATTN_ERR_HIP.
 */
attn_status attn_decode_gqa(const void *q, const void *k_cache,
                            const void *v_cache, void *o, float *lse, int B,
                            int Hq, int Hkv, int kv_len, int kv_cap, int D,
                            float scale, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace attn_decode_gqa, attn_decode_gqa_fp8 and
 * attn_decode_gqa_ragged need for this shape (kv_len: the longest sequence
 * for a ragged batch; 0 if invalid); one size serves all three (the plans
 * differ: a ragged batch is cut into pieces of at most 768 keys). */
size_t attn_decode_gqa_workspace_bytes(int B, int Hq, int Hkv, int kv_len,
                                       int D);

/*
 * GQA decode that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Same
 * arguments, kernels, results (bit for bit) and errors as attn_decode_gqa,
 * without the workspace pair: the split partials go to a static device
 * array of 2 MiB inside the library (one per GPU, held until the process
 * ends; its device address is looked up on the first call on each device).
 * That covers every shape whose partials need at most 2 MiB — among them
 * any group size up to 4, and the Llama-3-8B decode (B = 8, 32/8 heads,
 * 4096 keys: 0.5 MiB); a shape needing more returns ATTN_ERR_WORKSPACE,
 * launches nothing and must use attn_decode_gqa. Nothing in the array has
 * to start at any value. All calls on one GPU share the array and it keeps
 * the last call's contents: calls that may overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 */
attn_status attn_decode_gqa_noalloc(const void *q, const void *k_cache,
                                    const void *v_cache, void *o, float *lse, int B,
                                    int Hq, int Hkv, int kv_len, int kv_cap, int D,
                                    float scale, hipStream_t stream);

/*
 * GQA decode over an FP8 K/V cache: as attn_decode_gqa, but k_cache and
 * v_cache hold OCP FP8 E4M3 codes, one byte per element ([B, Hkv, kv_cap, D]
 * bytes; sign, 4-bit exponent with bias 7, 3-bit mantissa, largest finite
 * 448, S.1111.111 = NaN). The cached values enter the products exactly (each
 * E4M3 value is converted to bf16 without rounding) and accumulate in fp32,
 * so only the bytes read from HBM halve ("MLA 矩阵乘法吸收的数值稳定性治理",
 * §五: low-precision cache storage, FP32 accumulation on chip). Any
 * per-channel scaling of the stored values (stored = s·k) is the caller's:
 * fold s⁻¹ into q for K and apply s⁻¹ to O for V. q stays bf16.
 * Workspace: attn_decode_gqa_workspace_bytes() of the same shape.
 * Errors as for attn_decode_gqa.
 */
attn_status attn_decode_gqa_fp8(const void *q, const void *k_cache,
                                const void *v_cache, void *o, float *lse, int B,
                                int Hq, int Hkv, int kv_len, int kv_cap, int D,
                                float scale, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * GQA decode of a ragged batch: as attn_decode_gqa, but sequence b's cache
 * is filled to kv_lens[b] ("Bộ 06 · Bên trong model", Q3: attend to the
 * filled part only; each sequence of a serving batch has its own length).
 *
 *   kv_lens  [B] int32, DEVICE memory, read at run time; each value is
 *            clamped to [0, max_kv_len]. A sequence of length 0 attends to
 *            nothing: its O is 0 and its LSE is −∞ (the empty sums).
 *   max_kv_len  the longest length in the batch (or any bound of it, at
 *            most kv_cap): it fixes the split of the cache (the uniform
 *            call's split, or pieces of at most 768 keys when that is finer,
 *            so short sequences do not leave CUs idle) and the workspace
 *            size, attn_decode_gqa_workspace_bytes(B, Hq, Hkv, max_kv_len,
 *            D). Work for splits past a sequence's length is skipped.
 *
 * Errors as for attn_decode_gqa with max_kv_len in the place of kv_len;
 * kv_lens NULL → ATTN_ERR_NULL_POINTER.
 */
attn_status attn_decode_gqa_ragged(const void *q, const void *k_cache,
                                   const void *v_cache, void *o, float *lse,
                                   const int *kv_lens, int B, int Hq, int Hkv,
                                   int max_kv_len, int kv_cap, int D,
                                   float scale, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Absorbed MLA decode: every query head attends to one shared latent cache.
 * Each cached row is [latent (Dv) | rope (Dqk − Dv)]; the key is the whole
 * row and the value is its latent part, so the value is read from the same
 * bytes as the key. The query is the absorbed query (W_UK folded in) with
 * its rope part appended. Channel balancing (query ·S⁻¹, latent ·S) is done
 * by the caller before storage; O is returned in the same S-scaled latent
 * space (S⁻¹ belongs to the output projection outside this call).
 *
 *   q    [B, Hq, Dqk]         bf16
 *   ckv  [B, kv_cap, Dqk]     bf16 (only the first kv_len rows are read)
 *   o    [B, Hq, Dv]          bf16 (output)
 *   lse  [B, Hq]              fp32 (output, natural log)
 *   workspace: as for attn_decode_gqa, sized by
 *              attn_decode_mla_workspace_bytes().
 *
 * (Dqk, Dv) must be (576, 512); Hq must be a multiple of 16.
 * All products accumulate in fp32; the output is rounded once.
 * Errors as for attn_decode_gqa; other (Dqk, Dv) or Hq → ATTN_ERR_UNSUPPORTED.
 */
attn_status attn_decode_mla_absorbed(const void *q, const void *ckv, void *o,
                                     float *lse, int B, int Hq, int kv_len,
                                     int kv_cap, int Dqk, int Dv, float scale,
                                     void *workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Bytes of workspace attn_decode_mla_absorbed needs (0 if invalid). */
size_t attn_decode_mla_workspace_bytes(int B, int Hq, int kv_len, int Dqk,
                                       int Dv);

/*
 * Absorbed MLA decode over an FP8 latent cache: as attn_decode_mla_absorbed,
 * but ckv holds OCP FP8 E4M3 codes, one byte per element ([B, kv_cap, Dqk]
 * bytes; sign, 4-bit exponent with bias 7, 3-bit mantissa, largest finite
 * 448, S.1111.111 = NaN). The stored rows must be the channel-balanced
 * latent S·c ("MLA 矩阵乘法吸收的数值稳定性治理", §二.1: the static channel
 * scale S brings every latent channel into a common range; raw latent
 * channels span orders of magnitude that E4M3 cannot hold), with the query
 * in bf16 carrying S⁻¹. Each cached value enters the products exactly
 * (converted to bf16 without rounding) and every product accumulates in
 * fp32 (§五: low-precision storage, fp32 accumulation), so only the bytes
 * read from HBM halve. O is returned in the S-scaled latent space.
 * Workspace: attn_decode_mla_workspace_bytes() of the same shape.
 * Errors as for attn_decode_mla_absorbed.
 */
attn_status attn_decode_mla_fp8(const void *q, const void *ckv, void *o,
                                float *lse, int B, int Hq, int kv_len,
                                int kv_cap, int Dqk, int Dv, float scale,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Absorbed MLA decode of a ragged batch: as attn_decode_mla_absorbed, with
 * sequence b's latent cache filled to kv_lens[b] (DEVICE int32 [B], read at
 * run time, clamped to [0, max_kv_len]; length 0 gives O = 0, LSE = −∞).
 * The work is split evenly over the 32-key tiles of all sequences together
 * (equal runs of tiles across sequence boundaries, one workgroup per piece
 * of a run within one sequence), so short and long sequences in one batch
 * keep the whole GPU busy; the split is recomputed on the device from
 * kv_lens on every call. max_kv_len (the longest length, or a bound of it, at most
 * kv_cap) bounds the lengths. Workspace: attn_decode_mla_ragged_workspace_bytes().
 * Errors as for attn_decode_mla_absorbed with max_kv_len in the place of
 * kv_len; kv_lens NULL → ATTN_ERR_NULL_POINTER.
 */
attn_status attn_decode_mla_ragged(const void *q, const void *ckv, void *o,
                                   float *lse, const int *kv_lens, int B,
                                   int Hq, int max_kv_len, int kv_cap,
                                   int Dqk, int Dv, float scale,
                                   void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * Absorbed MLA decode of a ragged batch over an FP8 latent cache: the
 * ragged batch of attn_decode_mla_ragged (kv_lens, max_kv_len, the balanced
 * split over all sequences' tiles) with the E4M3 latent cache of
 * attn_decode_mla_fp8 ([B, kv_cap, Dqk] bytes of the channel-balanced
 * latent S·c, "MLA 矩阵乘法吸收的数值稳定性治理", §二.1; each value enters the
 * products exactly as bf16, every product accumulates in fp32, §五). Given
 * a bf16 copy of the same cached values, the result is bit for bit that of
 * attn_decode_mla_ragged. Workspace: attn_decode_mla_ragged_workspace_bytes().
 * Errors as for attn_decode_mla_ragged.
 */
attn_status attn_decode_mla_ragged_fp8(const void *q, const void *ckv,
                                       void *o, float *lse,
                                       const int *kv_lens, int B, int Hq,
                                       int max_kv_len, int kv_cap, int Dqk,
                                       int Dv, float scale, void *workspace,
                                       size_t workspace_bytes,
                                       hipStream_t stream);

/* Bytes of workspace attn_decode_mla_ragged needs (0 if invalid). */
size_t attn_decode_mla_ragged_workspace_bytes(int B, int Hq, int max_kv_len,
                                              int Dqk, int Dv);

/* Static, human-readable name of a status code. */
const char *attn_status_string(attn_status s);

/* Description of the last non-OK status returned on this thread ("" if none). */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
