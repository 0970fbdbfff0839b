// Absorbed MLA decode, gfx950: bf16 latent cache, fp32 accumulation.
//
// With W_UK folded into the query ("MLA 矩阵乘法吸收的数值稳定性治理", §一),
// every query head attends to one shared latent cache whose rows are
// [latent 512 | rope 64]. The key is the whole 576-wide row and the value is
// its latent part, so one HBM read of a row serves both products. Storage is
// bf16 but every product accumulates in fp32 and the output is rounded once
// (§二.2, §五).
//
// Decomposition. Workgroup (split, head group, b) has 8 waves and covers 128
// query heads, so each latent tile is loaded from HBM once and shared through
// LDS by all heads. Each wave owns 16 heads as the columns of
// v_mfma_f32_16x16x32_bf16:
//   Sᵀ = C·Qᵀ      keys as MFMA rows, 576-deep contraction, Q fragments held
//                  in registers for the whole pass;
//   online softmax in base 2 (running max and sum, rescale by 2^(m_old−m_new));
//   Oᵀ += Vᵀ·Pᵀ    P stays in registers (the Sᵀ accumulator layout is the
//                  B-operand layout), Vᵀ from a transposed LDS copy of the
//                  tile's first 512 channels written at staging time.
// Latent tiles of 32 rows are double-buffered in LDS. Splits of the cache
// write (O, m, ℓ) partials in fp32; a second small kernel merges them through
// their log-sum-exp ("AI Infra 入门…", §3, split-K with LSE). Rows at or past
// kv_len are never read.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int MD = 576, MV = 512, MBC = 32, MW = 8, MH = 16 * MW;
constexpr int MKS = MD / 32;     // 18 k-steps of the score product
constexpr int MDB = MV / 16;     // 32 row blocks of Oᵀ
constexpr int MKSTR = MD + 8;    // latent tile row stride (elements)
constexpr int MVSTR = MBC + 8;   // Vᵀ tile row stride (elements)
constexpr int MCH = MD / 8;      // 72 sixteen-byte chunks per row
constexpr int MUNITS = (MBC / 4) * MCH;  // staging units of 4 rows × 16 B
constexpr int MTHREADS = 64 * MW;
constexpr int MUPT = (MUNITS + MTHREADS - 1) / MTHREADS;
constexpr int kTargetGroups = 256;

__global__ __launch_bounds__(MTHREADS, 1) void decode_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ ckv,
    uint16_t *__restrict__ o, float *__restrict__ lse, int Hq, int kv_len, int kv_cap,
    float scale_log2, int splits, int split_keys, float *__restrict__ ws_ml,
    float *__restrict__ ws_part)
{
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][MBC * MKSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][MV * MVSTR];

    const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hcol = lane & 15, quad = lane >> 4;
    const int head0 = hg * MH + wave * 16;
    const bool wave_active = head0 < Hq;
    const int head = head0 + hcol;
    const int key_begin = split * split_keys;
    const int key_end = min(kv_len, key_begin + split_keys);
    const uint16_t *cb = ckv + (size_t)b * kv_cap * MD;

    bf16x8 qf[MKS];
    {
        const uint16_t *qr = q + ((size_t)b * Hq + min(head, Hq - 1)) * MD + 8 * quad;
#pragma unroll
        for (int ks = 0; ks < MKS; ++ks) qf[ks] = as<bf16x8>(*(const u32x4 *)(qr + 32 * ks));
    }

    u32x4 sreg[MUPT][4];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int u = 0; u < MUPT; ++u) {
            const int unit = tid + u * MTHREADS;
            if (unit < MUNITS) {
                const int kg = unit / MCH, dc = unit % MCH;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = min(t0 + 4 * kg + r, key_end - 1);
                    sreg[u][r] = *(const u32x4 *)(cb + (size_t)key * MD + 8 * dc);
                }
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < MUPT; ++u) {
            const int unit = tid + u * MTHREADS;
            if (unit < MUNITS) {
                const int kg = unit / MCH, dc = unit % MCH;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *(u32x4 *)&k_lds[buf][(4 * kg + r) * MKSTR + 8 * dc] = sreg[u][r];
                if (dc < MV / 8) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u32x2 a = {__byte_perm(sreg[u][0][j], sreg[u][1][j], 0x5410),
                                         __byte_perm(sreg[u][2][j], sreg[u][3][j], 0x5410)};
                        const u32x2 c = {__byte_perm(sreg[u][0][j], sreg[u][1][j], 0x7632),
                                         __byte_perm(sreg[u][2][j], sreg[u][3][j], 0x7632)};
                        *(u32x2 *)&vt_lds[buf][(8 * dc + 2 * j) * MVSTR + 4 * kg] = a;
                        *(u32x2 *)&vt_lds[buf][(8 * dc + 2 * j + 1) * MVSTR + 4 * kg] = c;
                    }
                }
            }
        }
    };

    f32x4 oacc[MDB];
#pragma unroll
    for (int db = 0; db < MDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int n_t = (key_end - key_begin + MBC - 1) / MBC;
    load_tile(key_begin);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < n_t; ++t) {
        const int cur = t & 1;
        const int t0 = key_begin + t * MBC;
        if (t + 1 < n_t) load_tile(t0 + MBC);
        if (wave_active) {
            float sc[8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const uint16_t *kr = &k_lds[cur][(16 * kb + hcol) * MKSTR + 8 * quad];
#pragma unroll
                for (int ks = 0; ks < MKS; ++ks)
                    acc = mfma16x16x32(as<bf16x8>(*(const u32x4 *)(kr + 32 * ks)), qf[ks], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = t0 + 16 * kb + 4 * quad + i;
                    sc[4 * kb + i] = key < key_end ? acc[i] * scale_log2 : -INFINITY;
                }
            }
            float mx = sc[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);  // finite: each tile has a key < key_end
            const float alpha = exp2_fast(m_run - m_new);
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sc[i] = exp2_fast(sc[i] - m_new);
                ps += sc[i];
            }
            l_run = l_run * alpha + ps;
            m_run = m_new;
            const u32x4 pw = {pack_bf16x2(sc[0], sc[1]), pack_bf16x2(sc[2], sc[3]),
                              pack_bf16x2(sc[4], sc[5]), pack_bf16x2(sc[6], sc[7])};
            const bf16x8 pf = as<bf16x8>(pw);
            // A slot s ↔ key 4·quad + s (s < 4) or 16 + 4·quad + (s − 4)
            const uint16_t *vr = &vt_lds[cur][hcol * MVSTR + 4 * quad];
#pragma unroll
            for (int db = 0; db < MDB; ++db) {
                const u32x2 lo = *(const u32x2 *)(vr + 16 * db * MVSTR);
                const u32x2 hi = *(const u32x2 *)(vr + 16 * db * MVSTR + 16);
                const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                oacc[db] = mfma16x16x32(as<bf16x8>(a), pf, oacc[db] * alpha);
            }
        }
        if (t + 1 < n_t) store_tile(cur ^ 1);
        __syncthreads();
    }

    if (!wave_active) return;
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    if (head >= Hq) return;
    // lane holds Oᵀ[d = 16·db + 4·quad + i][head]
    if (splits == 1) {
        const float inv = 1.f / l_run;
        uint16_t *orow = o + ((size_t)b * Hq + head) * MV;
#pragma unroll
        for (int db = 0; db < MDB; ++db) {
            const u32x2 w = {pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv),
                             pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv)};
            *(u32x2 *)(orow + 16 * db + 4 * quad) = w;
        }
        if (quad == 0) lse[(size_t)b * Hq + head] = (m_run + log2_fast(l_run)) * kLn2;
    } else {
        const size_t slot = ((size_t)b * Hq + head) * splits + split;
        float *prow = ws_part + slot * MV;
#pragma unroll
        for (int db = 0; db < MDB; ++db) *(f32x4 *)(prow + 16 * db + 4 * quad) = oacc[db];
        if (quad == 0) {
            ws_ml[2 * slot] = m_run;
            ws_ml[2 * slot + 1] = l_run;
        }
    }
}

// Merge the split partials of every (b, head) through their log-sum-exp.
// Thread = (row, 4 consecutive channels); summation over splits in order.
__global__ __launch_bounds__(256) void merge_mla_kernel(
    const float *__restrict__ ws_ml, const float *__restrict__ ws_part,
    uint16_t *__restrict__ o, float *__restrict__ lse, int rows, int splits)
{
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int row = gid / (MV / 4), c4 = gid % (MV / 4);
    if (row >= rows) return;
    const float *ml = ws_ml + (size_t)row * splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float f = exp2_fast(ml[2 * s] - M);
        const f32x4 p = *(const f32x4 *)(ws_part + ((size_t)row * splits + s) * MV + 4 * c4);
        acc += f * p;
        l = fmaf(f, ml[2 * s + 1], l);
    }
    const float inv = 1.f / l;
    const u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *(u32x2 *)(o + (size_t)row * MV + 4 * c4) = w;
    if (c4 == 0) lse[row] = (M + log2_fast(l)) * kLn2;
}

}  // namespace

bool mla_plan(int B, int Hq, int kv_len, MlaPlan *p)
{
    if (B < 1 || Hq < 16 || Hq % 16 || kv_len < 1) return false;
    const long hgs = (Hq + MH - 1) / MH;
    const int tiles = (kv_len + MBC - 1) / MBC;
    const long groups = (long)B * hgs;
    int want = (int)((kTargetGroups + groups - 1) / groups);
    int s = want < 1 ? 1 : (want < tiles ? want : tiles);
    const int per = (tiles + s - 1) / s;
    s = (tiles + per - 1) / per;
    p->splits = s;
    p->split_keys = per * MBC;
    p->ws_counters = 0;
    p->ws_ml = 0;
    const size_t rows = (size_t)B * Hq;
    p->ws_part = align_up(sizeof(float) * 2 * rows * s, 256);
    p->ws_total = p->ws_part + align_up(sizeof(float) * MV * rows * s, 256);
    if (s == 1) p->ws_total = 256;  // unused, but keep a non-zero minimum
    return true;
}

hipError_t launch_decode_mla(const MlaPlan &p, const void *q, const void *ckv, void *o,
                             float *lse, int B, int Hq, int kv_len, int kv_cap,
                             float scale, void *ws, hipStream_t st)
{
    char *w = (char *)ws;
    float *ws_ml = (float *)(w + p.ws_ml);
    float *ws_part = (float *)(w + p.ws_part);
    const dim3 grid(p.splits, (Hq + MH - 1) / MH, B);
    decode_mla_kernel<<<grid, dim3(MTHREADS), 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)ckv, (uint16_t *)o, lse, Hq, kv_len, kv_cap,
        scale * kLog2e, p.splits, p.split_keys, ws_ml, ws_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int rows = B * Hq;
    const int threads = rows * (MV / 4);
    merge_mla_kernel<<<dim3((threads + 255) / 256), dim3(256), 0, st>>>(
        ws_ml, ws_part, (uint16_t *)o, lse, rows, p.splits);
    return hipGetLastError();
}

}  // namespace attn
