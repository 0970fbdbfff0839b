// C-ABI entry points of libattn.so: argument validation on the host (nothing
// is enqueued on error), status reporting, and dispatch to the gfx950 kernels.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "../../include/attn.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

attn_status fail(attn_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

attn_status ok()
{
    g_last_error[0] = '\0';
    return ATTN_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
// The kernels take row maxima of unscaled scores, which is only the max of
// the scaled ones for a positive scale.
bool good_scale(float s) { return s > 0.f && s <= 3.4e38f; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

constexpr long long kMaxElems = (1ll << 31) - 1;

attn_status from_hip(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shared by the uniform and the ragged GQA decode: kv_lens NULL means every
// sequence holds kv_len keys; otherwise kv_len is the longest.
attn_status decode_gqa_impl(const char *fn, const void *q, const void *k_cache,
                            const void *v_cache, void *o, float *lse, const int *kv_lens,
                            int B, int Hq, int Hkv, int kv_len, int kv_cap, int D, float scale,
                            void *workspace, size_t workspace_bytes, hipStream_t stream,
                            bool fp8 = false, bool fixed_scratch = false)
{
    const char *len_name = kv_lens ? "max_kv_len" : "kv_len";
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: B, Hq, Hkv, D must be >= 1", fn);
    if (Hq % Hkv)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: Hq (%d) not a multiple of Hkv (%d)", fn, Hq, Hkv);
    if (!good_scale(scale))
        return fail(ATTN_ERR_BAD_SHAPE, "%s: scale must be finite and > 0", fn);
    if (kv_len < 1 || kv_len > kv_cap)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: need 1 <= %s (%d) <= kv_cap (%d)", fn, len_name, kv_len,
                    kv_cap);
    if ((long long)B * Hkv * kv_cap * D > kMaxElems)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: cache exceeds 2^31 elements", fn);
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d (only 128)", fn, D);
    if (Hq / Hkv > 16)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: group size %d above 16", fn, Hq / Hkv);
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(o) || !aligned4(lse) ||
        !aligned4(kv_lens))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: tensors must be 16-byte aligned (o, lse, kv_lens: 4)", fn);
    attn::GqaPlan p;
    attn::gqa_plan(B, Hq, Hkv, kv_len, &p, fp8, kv_lens != nullptr);
    if (fixed_scratch && p.ws_total > workspace_bytes)
        return fail(ATTN_ERR_WORKSPACE,
                    "%s: this shape needs %zu bytes of scratch; the library's static scratch holds "
                    "%zu (use attn_decode_gqa with a caller workspace)", fn, p.ws_total,
                    workspace_bytes);
    if (!workspace || workspace_bytes < p.ws_total || !aligned16(workspace))
        return fail(ATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", fn, p.ws_total,
                    workspace ? workspace_bytes : (size_t)0);
    return from_hip(attn::launch_decode_gqa(p, q, k_cache, v_cache, o, lse, B, Hq, Hkv, kv_len,
                                            kv_cap, scale, workspace, stream, kv_lens, fp8),
                    fn);
}

// Scratch of attn_decode_gqa_noalloc: the split partials between the split
// kernel and the merge kernel live in this fixed device array instead of a
// caller workspace, so the call allocates nothing. Each device holds its own
// copy until the process ends. On the host the name `scratch` is only a
// stand-in for the symbol: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
constexpr size_t kScratchBytes = 2u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

attn_status scratch_of_current_device(const char *fn, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e, fn);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return from_hip(e, fn);
        if (!ptr) return fail(ATTN_ERR_HIP, "%s: no device address for the static scratch", fn);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return ATTN_OK;
}

attn_status decode_mla_impl(const char *fn, const void *q, const void *ckv, void *o, float *lse,
                            const int *kv_lens, int B, int Hq, int kv_len, int kv_cap, int Dqk,
                            int Dv, float scale, void *workspace, size_t workspace_bytes,
                            hipStream_t stream, bool fp8 = false)
{
    const char *len_name = kv_lens ? "max_kv_len" : "kv_len";
    if (B < 1 || Hq < 1 || Dqk < 1 || Dv < 1 || Dv > Dqk)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: bad B, Hq, Dqk or Dv", fn);
    if (!good_scale(scale))
        return fail(ATTN_ERR_BAD_SHAPE, "%s: scale must be finite and > 0", fn);
    if (kv_len < 1 || kv_len > kv_cap)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: need 1 <= %s (%d) <= kv_cap (%d)", fn, len_name, kv_len,
                    kv_cap);
    if ((long long)B * kv_cap * Dqk > kMaxElems)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: cache exceeds 2^31 elements", fn);
    if (Dqk != 576 || Dv != 512)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: (Dqk, Dv) = (%d, %d), only (576, 512)", fn, Dqk, Dv);
    if (Hq % 16)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: Hq (%d) not a multiple of 16", fn, Hq);
    if (!aligned16(q) || !aligned16(ckv) || !aligned16(o) || !aligned4(lse) || !aligned4(kv_lens))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: tensors must be 16-byte aligned (lse, kv_lens: 4)", fn);
    attn::MlaPlan p;
    if (kv_lens)
        attn::mla_ragged_plan(B, Hq, kv_len, &p);
    else
        attn::mla_plan(B, Hq, kv_len, &p);
    if (!workspace || workspace_bytes < p.ws_total || !aligned16(workspace))
        return fail(ATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", fn, p.ws_total,
                    workspace ? workspace_bytes : (size_t)0);
    return from_hip(attn::launch_decode_mla(p, q, ckv, o, lse, B, Hq, kv_len, kv_cap, scale,
                                            workspace, stream, kv_lens, fp8),
                    fn);
}

}  // namespace

extern "C" {

const char *attn_status_string(attn_status s)
{
    switch (s) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_NULL_POINTER: return "ATTN_ERR_NULL_POINTER";
        case ATTN_ERR_BAD_SHAPE: return "ATTN_ERR_BAD_SHAPE";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    }
    return "ATTN_ERR_UNKNOWN";
}

const char *attn_last_error(void) { return g_last_error; }

attn_status attn_prefill_causal(attn_dtype dtype, const void *q, const void *k,
                                const void *v, void *o, float *lse, int B, int Hq,
                                int Hkv, int N, int D, float scale, hipStream_t stream)
{
    if (!q || !k || !v || !o || !lse)
        return fail(ATTN_ERR_NULL_POINTER, "attn_prefill_causal: NULL tensor pointer");
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1)
        return fail(ATTN_ERR_BAD_SHAPE, "attn_prefill_causal: B, Hq, Hkv, N, D must be >= 1");
    if (Hq % Hkv)
        return fail(ATTN_ERR_BAD_SHAPE, "attn_prefill_causal: Hq (%d) not a multiple of Hkv (%d)", Hq, Hkv);
    if (!good_scale(scale))
        return fail(ATTN_ERR_BAD_SHAPE, "attn_prefill_causal: scale must be finite and > 0");
    if ((long long)B * Hq * N * D > kMaxElems)
        return fail(ATTN_ERR_BAD_SHAPE, "attn_prefill_causal: tensor exceeds 2^31 elements");
    if (dtype != ATTN_BF16 && dtype != ATTN_FP32)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_causal: unknown dtype %d", (int)dtype);
    if (D != 64 && D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_causal: head dim %d not in {64, 128}", D);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_causal: tensors must be 16-byte aligned");
    if (dtype == ATTN_BF16)
        return from_hip(attn::launch_prefill_bf16(q, k, v, o, lse, B, Hq, Hkv, N, D, scale, stream),
                        "attn_prefill_causal");
    return from_hip(attn::launch_prefill_f32((const float *)q, (const float *)k, (const float *)v,
                                             (float *)o, lse, B, Hq, Hkv, N, D, scale, stream),
                    "attn_prefill_causal");
}

size_t attn_prefill_chunked_workspace_bytes(int B, int Hq, int Nq, int kv_cap, int D)
{
    if (B < 1 || Hq < 1 || Nq < 1 || kv_cap < Nq || D != 128) return 0;
    return attn::prefill_chunked_workspace_bytes(B, Hq, Nq, kv_cap);
}

attn_status attn_prefill_chunked(const void *q, const void *k_cache, const void *v_cache,
                                 void *o, float *lse, const int *kv_lens, int B, int Hq,
                                 int Hkv, int Nq, int kv_cap, int D, float scale,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    static const char fn[] = "attn_prefill_chunked";
    if (!q || !k_cache || !v_cache || !o || !lse || !kv_lens)
        return fail(ATTN_ERR_NULL_POINTER, "%s: NULL tensor pointer", fn);
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || D < 1)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: B, Hq, Hkv, Nq, D must be >= 1", fn);
    if (Hq % Hkv)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: Hq (%d) not a multiple of Hkv (%d)", fn, Hq, Hkv);
    if (!good_scale(scale))
        return fail(ATTN_ERR_BAD_SHAPE, "%s: scale must be finite and > 0", fn);
    if (Nq > kv_cap)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: need Nq (%d) <= kv_cap (%d)", fn, Nq, kv_cap);
    if ((long long)B * Hq * Nq * D > kMaxElems || (long long)B * Hkv * kv_cap * D > kMaxElems)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: tensor exceeds 2^31 elements", fn);
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d (only 128)", fn, D);
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        !aligned4(lse) || !aligned4(kv_lens))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: tensors must be 16-byte aligned (lse, kv_lens: 4)", fn);
    const size_t need = attn::prefill_chunked_workspace_bytes(B, Hq, Nq, kv_cap);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(ATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return from_hip(attn::launch_prefill_chunked_d128(q, k_cache, v_cache, o, lse, kv_lens, B, Hq,
                                                      Hkv, Nq, kv_cap, scale, workspace, stream),
                    fn);
}

size_t attn_prefill_causal_backward_workspace_bytes(int B, int Hq, int N, int D)
{
    if (B < 1 || Hq < 1 || N < 1 || D != 128) return 0;
    return attn::prefill_bwd_workspace_bytes(B, Hq, N);
}

attn_status attn_prefill_causal_backward(const void *q, const void *k, const void *v,
                                         const void *o, const float *lse, const void *dout,
                                         void *dq, void *dk, void *dv, int B, int Hq, int Hkv,
                                         int N, int D, float scale, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream)
{
    static const char fn[] = "attn_prefill_causal_backward";
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
        return fail(ATTN_ERR_NULL_POINTER, "%s: NULL tensor pointer", fn);
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: B, Hq, Hkv, N, D must be >= 1", fn);
    if (Hq % Hkv)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: Hq (%d) not a multiple of Hkv (%d)", fn, Hq, Hkv);
    if (!good_scale(scale))
        return fail(ATTN_ERR_BAD_SHAPE, "%s: scale must be finite and > 0", fn);
    if ((long long)B * Hq * N * D > kMaxElems)
        return fail(ATTN_ERR_BAD_SHAPE, "%s: tensor exceeds 2^31 elements", fn);
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d (only 128)", fn, D);
    const void *t16[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void *p : t16)
        if (!aligned16(p))
            return fail(ATTN_ERR_UNSUPPORTED, "%s: tensors must be 16-byte aligned", fn);
    if (!aligned4(lse))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: lse must be 4-byte aligned", fn);
    const size_t need = attn::prefill_bwd_workspace_bytes(B, Hq, N);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(ATTN_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    return from_hip(attn::launch_prefill_bwd_d128(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv,
                                                  N, scale, workspace, stream),
                    fn);
}

size_t attn_decode_gqa_workspace_bytes(int B, int Hq, int Hkv, int kv_len, int D)
{
    // one size serves both cache types and ragged batches: the largest plan
    attn::GqaPlan p, p8, pr;
    if (D != 128 || !attn::gqa_plan(B, Hq, Hkv, kv_len, &p, false) ||
        !attn::gqa_plan(B, Hq, Hkv, kv_len, &p8, true) ||
        !attn::gqa_plan(B, Hq, Hkv, kv_len, &pr, false, true))
        return 0;
    size_t m = p.ws_total > p8.ws_total ? p.ws_total : p8.ws_total;
    return m > pr.ws_total ? m : pr.ws_total;
}

attn_status attn_decode_gqa(const void *q, const void *k_cache, const void *v_cache, void *o,
                            float *lse, int B, int Hq, int Hkv, int kv_len, int kv_cap, int D,
                            float scale, void *workspace, size_t workspace_bytes,
                            hipStream_t stream)
{
    if (!q || !k_cache || !v_cache || !o || !lse)
        return fail(ATTN_ERR_NULL_POINTER, "attn_decode_gqa: NULL tensor pointer");
    return decode_gqa_impl("attn_decode_gqa", q, k_cache, v_cache, o, lse, nullptr, B, Hq, Hkv,
                           kv_len, kv_cap, D, scale, workspace, workspace_bytes, stream);
}

attn_status attn_decode_gqa_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                    void *o, float *lse, int B, int Hq, int Hkv, int kv_len,
                                    int kv_cap, int D, float scale, hipStream_t stream)
{
    const char *fn = "attn_decode_gqa_noalloc";
    if (!q || !k_cache || !v_cache || !o || !lse)
        return fail(ATTN_ERR_NULL_POINTER, "%s: NULL tensor pointer", fn);
    void *ws = nullptr;
    const attn_status st = scratch_of_current_device(fn, &ws);
    if (st != ATTN_OK) return st;
    return decode_gqa_impl(fn, q, k_cache, v_cache, o, lse, nullptr, B, Hq, Hkv, kv_len, kv_cap, D,
                           scale, ws, kScratchBytes, stream, false, true);
}

attn_status attn_decode_gqa_fp8(const void *q, const void *k_cache, const void *v_cache,
                                void *o, float *lse, int B, int Hq, int Hkv, int kv_len,
                                int kv_cap, int D, float scale, void *workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    if (!q || !k_cache || !v_cache || !o || !lse)
        return fail(ATTN_ERR_NULL_POINTER, "attn_decode_gqa_fp8: NULL tensor pointer");
    return decode_gqa_impl("attn_decode_gqa_fp8", q, k_cache, v_cache, o, lse, nullptr, B, Hq, Hkv,
                           kv_len, kv_cap, D, scale, workspace, workspace_bytes, stream, true);
}

attn_status attn_decode_gqa_ragged(const void *q, const void *k_cache, const void *v_cache,
                                   void *o, float *lse, const int *kv_lens, int B, int Hq,
                                   int Hkv, int max_kv_len, int kv_cap, int D, float scale,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!q || !k_cache || !v_cache || !o || !lse || !kv_lens)
        return fail(ATTN_ERR_NULL_POINTER, "attn_decode_gqa_ragged: NULL tensor pointer");
    return decode_gqa_impl("attn_decode_gqa_ragged", q, k_cache, v_cache, o, lse, kv_lens, B, Hq,
                           Hkv, max_kv_len, kv_cap, D, scale, workspace, workspace_bytes, stream);
}

size_t attn_decode_mla_workspace_bytes(int B, int Hq, int kv_len, int Dqk, int Dv)
{
    attn::MlaPlan p;
    if (Dqk != 576 || Dv != 512 || !attn::mla_plan(B, Hq, kv_len, &p)) return 0;
    return p.ws_total;
}

attn_status attn_decode_mla_absorbed(const void *q, const void *ckv, void *o, float *lse,
                                     int B, int Hq, int kv_len, int kv_cap, int Dqk, int Dv,
                                     float scale, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream)
{
    if (!q || !ckv || !o || !lse)
        return fail(ATTN_ERR_NULL_POINTER, "attn_decode_mla_absorbed: NULL tensor pointer");
    return decode_mla_impl("attn_decode_mla_absorbed", q, ckv, o, lse, nullptr, B, Hq, kv_len,
                           kv_cap, Dqk, Dv, scale, workspace, workspace_bytes, stream);
}

attn_status attn_decode_mla_fp8(const void *q, const void *ckv, void *o, float *lse, int B,
                                int Hq, int kv_len, int kv_cap, int Dqk, int Dv, float scale,
                                void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!q || !ckv || !o || !lse)
        return fail(ATTN_ERR_NULL_POINTER, "attn_decode_mla_fp8: NULL tensor pointer");
    return decode_mla_impl("attn_decode_mla_fp8", q, ckv, o, lse, nullptr, B, Hq, kv_len, kv_cap,
                           Dqk, Dv, scale, workspace, workspace_bytes, stream, true);
}

size_t attn_decode_mla_ragged_workspace_bytes(int B, int Hq, int max_kv_len, int Dqk, int Dv)
{
    attn::MlaPlan p;
    if (Dqk != 576 || Dv != 512 || !attn::mla_ragged_plan(B, Hq, max_kv_len, &p)) return 0;
    return p.ws_total;
}

attn_status attn_decode_mla_ragged(const void *q, const void *ckv, void *o, float *lse,
                                   const int *kv_lens, int B, int Hq, int max_kv_len, int kv_cap,
                                   int Dqk, int Dv, float scale, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream)
{
    if (!q || !ckv || !o || !lse || !kv_lens)
        return fail(ATTN_ERR_NULL_POINTER, "attn_decode_mla_ragged: NULL tensor pointer");
    return decode_mla_impl("attn_decode_mla_ragged", q, ckv, o, lse, kv_lens, B, Hq, max_kv_len,
                           kv_cap, Dqk, Dv, scale, workspace, workspace_bytes, stream);
}

attn_status attn_decode_mla_ragged_fp8(const void *q, const void *ckv, void *o, float *lse,
                                       const int *kv_lens, int B, int Hq, int max_kv_len,
                                       int kv_cap, int Dqk, int Dv, float scale, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream)
{
    if (!q || !ckv || !o || !lse || !kv_lens)
        return fail(ATTN_ERR_NULL_POINTER, "attn_decode_mla_ragged_fp8: NULL tensor pointer");
    return decode_mla_impl("attn_decode_mla_ragged_fp8", q, ckv, o, lse, kv_lens, B, Hq,
                           max_kv_len, kv_cap, Dqk, Dv, scale, workspace, workspace_bytes, stream,
                           true);
}

}  // extern "C"
