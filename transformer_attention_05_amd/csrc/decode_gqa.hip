// Single-query GQA decode over a bf16 K/V cache, gfx950.
//
// Decode is memory-bound: about 4 flops per byte of K/V read ("05 · Tích vô
// hướng, Softmax và toán của Attention", §4), so the design goal is to stream
// every cached K/V byte from HBM exactly once with enough loads in flight.
//
// Decomposition. Workgroup (split, hkv, b) owns keys
// [split·split_keys, min(kv_len, (split+1)·split_keys)) of one K/V head and
// all G = Hq/Hkv query heads that share it, so each K/V byte is loaded once
// and used G times. Its four waves take 64 keys each per 256-key step.
//
// Per 64-key wave chunk:
//   * S = K·qᵀ on v_mfma_f32_16x16x32_bf16 with keys as MFMA rows and the
//     (zero-padded) heads as MFMA columns: lane l feeds K[key = l%16][8 d]
//     straight from global memory (16 B per lane), fp32 accumulation.
//   * online softmax in base 2 (scores pre-multiplied by scale·log2 e):
//     running max m, running sum ℓ, old sum and output rescaled by
//     2^(m_old − m_new) ("AI Infra 入门…", §3, online softmax).
//   * O += P·V on the VALU in fp32: lane l holds V[key][8 d] of one key
//     (4 keys × 256 B = 1 KiB contiguous per wave load) and gets that key's
//     weights for every head from a per-wave LDS table.
// The waves' (m, ℓ, O) are merged in LDS; with one split the workgroup
// writes O/ℓ and LSE directly, otherwise it writes its partial (m, ℓ, Õ) to
// the workspace and a second kernel merges the partials through their
// log-sum-exp (split-K merge, "AI Infra 入门…", §3). No workgroup waits for
// another and no cross-workgroup fence is needed: the kernel boundary orders
// the partial writes before the merge. Slots at or past kv_len are never read.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kWaveKeys = 64;
constexpr int kChunk = kWaves * kWaveKeys;  // 256 keys per workgroup step
constexpr int kTargetGroups = 1024;         // workgroups per launch the split aims at

template <int GP>
__global__ __launch_bounds__(256, GP >= 16 ? 1 : 2) void decode_gqa_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, uint16_t *__restrict__ o, float *__restrict__ lse,
    int Hq, int Hkv, int G, int kv_len, int kv_cap, float scale_log2, int splits,
    int split_keys, float *__restrict__ ws_ml, float *__restrict__ ws_part)
{
    const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = b * Hkv + hkv;
    const int key_begin = split * split_keys;
    const int key_end = min(kv_len, key_begin + split_keys);
    const uint16_t *kbase = kc + (size_t)bh * kv_cap * kD;
    const uint16_t *vbase = vc + (size_t)bh * kv_cap * kD;

    __shared__ float p_lds[kWaves][kWaveKeys * GP + GP];
    __shared__ float red_o[kWaves][GP][kD];
    __shared__ float red_m[kWaves][GP], red_l[kWaves][GP];

    // qᵀ as the MFMA B operand: column = head (lane % 16), 8 d per lane.
    const int hcol = lane & 15, quad = lane >> 4;
    bf16x8 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (hcol < G)
            w = *(const u32x4 *)(q + (size_t)(b * Hq + hkv * G + hcol) * kD + 32 * s + 8 * quad);
        qf[s] = as<bf16x8>(w);
    }

    float m_run = -INFINITY, l_run = 0.f;  // for head hcol (S layout)
    float oacc[GP][8];                     // O[h][8·(lane%16) + e] for this lane's key slot
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[h][e] = 0.f;

    float *pw = p_lds[wave];
    for (int c0 = key_begin; c0 < key_end; c0 += kChunk) {
        const int w0 = c0 + wave * kWaveKeys;  // this wave's first key
        if (w0 >= key_end) break;              // wave-uniform
        // ---- issue all loads of the chunk (K in MFMA-A layout, V row-major)
        u32x4 kr[4][4], vr[16];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int key = min(w0 + blk * 16 + hcol, key_end - 1);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kr[blk][s] = *(const u32x4 *)(kbase + (size_t)key * kD + 32 * s + 8 * quad);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = min(w0 + 4 * i + quad, key_end - 1);
            vr[i] = *(const u32x4 *)(vbase + (size_t)key * kD + 8 * hcol);
        }
        // ---- S = K qᵀ: row = key (4·quad + i within a 16-key block), col = head
        float sc[16];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma16x16x32(as<bf16x8>(kr[blk][s]), qf[s], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = w0 + blk * 16 + 4 * quad + i;
                sc[blk * 4 + i] = key < key_end ? acc[i] * scale_log2 : -INFINITY;
            }
        }
        // ---- online softmax for head hcol (its 64 keys live in 4 lanes)
        float mx = sc[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sc[j]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast(m_run - m_new);  // m_run = -inf → 0
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            sc[j] = exp2_fast(sc[j] - m_new);
            ps += sc[j];
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
        // ---- publish p[key][head] and alpha[head] to this wave's LDS table
        if (hcol < GP) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pw[(blk * 16 + 4 * quad + i) * GP + hcol] = sc[blk * 4 + i];
            if (quad == 0) pw[kWaveKeys * GP + hcol] = alpha;
        }
        wave_lds_sync();
        // ---- O = alpha·O + Σ_key p·V  (lane: key slot quad, d = 8·hcol..+7)
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            const float a = pw[kWaveKeys * GP + h];
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[h][e] *= a;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float *prow = pw + (4 * i + quad) * GP;
            float v[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = bf16lo(vr[i][j]);
                v[2 * j + 1] = bf16hi(vr[i][j]);
            }
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                const float p = prow[h];
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[h][e] = fmaf(p, v[e], oacc[h][e]);
            }
        }
        wave_lds_sync();
    }

    // ---- merge the four key slots of the wave (lanes l, l^16, l^32, l^48)
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = oacc[h][e];
            x += shfl_xor(x, 16);
            x += shfl_xor(x, 32);
            oacc[h][e] = x;
        }
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    if (quad == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) red_o[wave][h][8 * hcol + e] = oacc[h][e];
    }
    if (lane < GP) {
        red_m[wave][lane] = m_run;
        red_l[wave][lane] = l_run;
    }
    __syncthreads();

    // ---- merge the four waves; write the result or this split's partial
    for (int idx = tid; idx < GP * kD; idx += 256) {
        const int h = idx / kD, d = idx % kD;
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
        float acc = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2_fast(red_m[w][h] - M);  // empty wave: 2^-inf = 0
            acc = fmaf(f, red_o[w][h][d], acc);
            l = fmaf(f, red_l[w][h], l);
        }
        if (h >= G) continue;
        const size_t row = (size_t)b * Hq + hkv * G + h;
        if (splits == 1) {
            o[row * kD + d] = (uint16_t)(pack_bf16x2(acc / l, 0.f) & 0xffffu);
            if (d == 0) lse[row] = (M + log2_fast(l)) * kLn2;
        } else {
            const size_t slot = row * splits + split;
            ws_part[slot * kD + d] = acc;
            if (d == 0) {
                ws_ml[2 * slot] = M;
                ws_ml[2 * slot + 1] = l;
            }
        }
    }
}

}  // namespace

bool gqa_plan(int B, int Hq, int Hkv, int kv_len, GqaPlan *p)
{
    if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || kv_len < 1) return false;
    const int G = Hq / Hkv;
    if (G > 16) return false;
    int gp = 1;
    while (gp < G) gp *= 2;
    const long groups = (long)B * Hkv;
    const int chunks = (kv_len + kChunk - 1) / kChunk;
    int want = (int)((kTargetGroups + groups - 1) / groups);
    int s = want < 1 ? 1 : (want < chunks ? want : chunks);
    const int per = (chunks + s - 1) / s;
    s = (chunks + per - 1) / per;
    p->gp = gp;
    p->splits = s;
    p->split_keys = per * kChunk;
    const size_t rows = (size_t)B * Hq;
    p->ws_ml = 0;
    p->ws_part = align_up(sizeof(float) * 2 * rows * s, 256);
    p->ws_total = s == 1 ? 256 : p->ws_part + align_up(sizeof(float) * kD * rows * s, 256);
    return true;
}

hipError_t launch_decode_gqa(const GqaPlan &p, const void *q, const void *k, const void *v,
                             void *o, float *lse, int B, int Hq, int Hkv, int kv_len,
                             int kv_cap, float scale, void *ws, hipStream_t st)
{
    char *w = (char *)ws;
    float *ws_ml = (float *)(w + p.ws_ml);
    float *ws_part = (float *)(w + p.ws_part);
    const dim3 grid(p.splits, Hkv, B), block(256);
    const float sl2 = scale * kLog2e;
    const int G = Hq / Hkv;
#define ATTN_GQA_CASE(GPV)                                                              \
    case GPV:                                                                            \
        decode_gqa_kernel<GPV><<<grid, block, 0, st>>>(                                 \
            (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, \
            lse, Hq, Hkv, G, kv_len, kv_cap, sl2, p.splits, p.split_keys, ws_ml, ws_part); \
                                                                                      \
        break;
    switch (p.gp) {
        ATTN_GQA_CASE(1)
        ATTN_GQA_CASE(2)
        ATTN_GQA_CASE(4)
        ATTN_GQA_CASE(8)
        ATTN_GQA_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef ATTN_GQA_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_merge(ws_ml, ws_part, o, lse, B * Hq, p.splits, kD, st);
}

}  // namespace attn
