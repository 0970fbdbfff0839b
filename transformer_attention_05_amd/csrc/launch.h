// Host-side launchers of the gfx950 kernels (internal to libattn.so). Each
// assumes its arguments were validated by the C-ABI layer in attn_api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// ---- GQA decode ----------------------------------------------------------
struct GqaPlan {
    int splits;      // workgroups per (batch, K/V head)
    int split_keys;  // keys per split (multiple of the 128-key workgroup step)
    size_t ws_ml, ws_part, ws_total;  // workspace byte offsets / size
};
// fp8: plan for an E4M3 cache; ragged: a batch with per-sequence lengths
// (pieces of at most 768 keys when that is finer than the uniform split)
bool gqa_plan(int B, int Hq, int Hkv, int kv_len, GqaPlan *p, bool fp8, bool ragged = false);
// kv_lens: NULL (every sequence holds kv_len keys) or a device array of B
// per-sequence lengths, each clamped to [0, kv_len] by the kernel.
// fp8: the caches hold OCP FP8 E4M3 codes (one byte per element) instead of bf16.
hipError_t launch_decode_gqa(const GqaPlan &p, const void *q, const void *k, const void *v,
                             void *o, float *lse, int B, int Hq, int Hkv, int kv_len,
                             int kv_cap, float scale, void *ws, hipStream_t s,
                             const int *kv_lens, bool fp8);
// The E4M3 split kernel alone (decode_gqa_fp8.hip); xcd: the XCD remap of
// the workgroup ids is on.
hipError_t launch_decode_gqa_split_fp8(const GqaPlan &p, const void *q, const void *k,
                                       const void *v, void *o, float *lse, int B, int Hq,
                                       int Hkv, int kv_len, int kv_cap, float scale, void *ws,
                                       hipStream_t s, const int *kv_lens, int xcd);

// ---- causal prefill ------------------------------------------------------
hipError_t launch_prefill_bf16(const void *q, const void *k, const void *v, void *o,
                               float *lse, int B, int Hq, int Hkv, int N, int D,
                               float scale, hipStream_t s);
hipError_t launch_prefill_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int B, int Hq, int Hkv, int N, float scale,
                                    hipStream_t s);
// N queries per sequence against caches of kv_cap slots filled to kv_lens[b]
// (a device array, clamped to [N, kv_cap]); the queries are the last N
// positions (bottom-right causal mask).
// Short chunks split the keys over several workgroups (fp32 partials in ws,
// prefill_chunked_workspace_bytes(), merged through the LSE).
int prefill_chunked_splits(int B, int Hq, int Nq, int kv_cap);
size_t prefill_chunked_workspace_bytes(int B, int Hq, int Nq, int kv_cap);
hipError_t launch_prefill_chunked_d128(const void *q, const void *k, const void *v, void *o,
                                       float *lse, const int *kv_lens, int B, int Hq, int Hkv,
                                       int N, int kv_cap, float scale, void *ws, hipStream_t s);
// Backward of the causal prefill, d = 128, bf16; ws holds two fp32 arrays
// [B·Hq][N rounded up to 32]: D = dO·O and LSE·log₂e (+∞ past the sequence).
size_t prefill_bwd_workspace_bytes(int B, int Hq, int N);
hipError_t launch_prefill_bwd_d128(const void *q, const void *k, const void *v, const void *o,
                                   const float *lse, const void *dout, void *dq, void *dk,
                                   void *dv, int B, int Hq, int Hkv, int N, float scale,
                                   void *ws, hipStream_t s);
hipError_t launch_prefill_f32(const float *q, const float *k, const float *v, float *o,
                              float *lse, int B, int Hq, int Hkv, int N, int D,
                              float scale, hipStream_t s);

// ---- absorbed MLA decode -------------------------------------------------
struct MlaPlan {
    int splits, split_keys;
    size_t ws_ml, ws_part, ws_total;
};
bool mla_plan(int B, int Hq, int kv_len, MlaPlan *p);
// ragged batch: splits = workers per head group of the balanced split
bool mla_ragged_plan(int B, int Hq, int max_len, MlaPlan *p);
// kv_lens: NULL, or a device array of B lengths (plan from mla_ragged_plan,
// kv_len = the longest sequence).
hipError_t launch_decode_mla(const MlaPlan &p, const void *q, const void *ckv, void *o,
                             float *lse, int B, int Hq, int kv_len, int kv_cap,
                             float scale, void *ws, hipStream_t s, const int *kv_lens, bool fp8);

// ---- split-K merge through the log-sum-exp (shared by both decodes) -------
constexpr int kMaxSplits = 128;  // upper bound the planners respect
// ml [rows][splits] = float4 (m, ℓ, λ, unused) in base 2 (ℓ feeds the LSE,
// λ normalises O); part [rows][splits][dv]: fp32 Õ.
// xcd_group: 0, or the rows per group when group g's partials were written
// on XCD g % 8 (the merge then reads them there).
hipError_t launch_merge(const float *ml, const float *part, void *o, float *lse, int rows,
                        int splits, int dv, hipStream_t s, int xcd_group = 0);
// The merge of the balanced split of a ragged batch (ragged.h): records
// [slot][row of the batch's Hq heads], slot = worker + sequence, `workers`
// workers over tiles of `tile` keys of sequences of length kv_lens[b] (at
// most max_len). A sequence with no key gets O = 0, LSE = −∞.
hipError_t launch_merge_ragged(const float *ml, const float *part, void *o, float *lse,
                               const int *kv_lens, int B, int Hq, int max_len, int workers,
                               int tile, int dv, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace attn
