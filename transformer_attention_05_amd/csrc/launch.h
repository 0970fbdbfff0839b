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
    int split_keys;  // keys per split (multiple of the 256-key chunk)
    size_t ws_ml, ws_part, ws_total;  // workspace byte offsets / size
};
bool gqa_plan(int B, int Hq, int Hkv, int kv_len, GqaPlan *p);
hipError_t launch_decode_gqa(const GqaPlan &p, const void *q, const void *k, const void *v,
                             void *o, float *lse, int B, int Hq, int Hkv, int kv_len,
                             int kv_cap, float scale, void *ws, hipStream_t s);

// ---- causal prefill ------------------------------------------------------
hipError_t launch_prefill_bf16(const void *q, const void *k, const void *v, void *o,
                               float *lse, int B, int Hq, int Hkv, int N, int D,
                               float scale, hipStream_t s);
hipError_t launch_prefill_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int B, int Hq, int Hkv, int N, float scale,
                                    hipStream_t s);
hipError_t launch_prefill_f32(const float *q, const float *k, const float *v, float *o,
                              float *lse, int B, int Hq, int Hkv, int N, int D,
                              float scale, hipStream_t s);

// ---- absorbed MLA decode -------------------------------------------------
struct MlaPlan {
    int splits, split_keys;
    size_t ws_ml, ws_part, ws_total;
};
bool mla_plan(int B, int Hq, int kv_len, MlaPlan *p);
hipError_t launch_decode_mla(const MlaPlan &p, const void *q, const void *ckv, void *o,
                             float *lse, int B, int Hq, int kv_len, int kv_cap,
                             float scale, void *ws, hipStream_t s);

// ---- split-K merge through the log-sum-exp (shared by both decodes) -------
constexpr int kMaxSplits = 128;  // upper bound the planners respect
// ml [rows][splits] = float4 (m, ℓ, λ, unused) in base 2 (ℓ feeds the LSE,
// λ normalises O); part [rows][splits][dv] fp32.
hipError_t launch_merge(const float *ml, const float *part, void *o, float *lse, int rows,
                        int splits, int dv, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace attn
