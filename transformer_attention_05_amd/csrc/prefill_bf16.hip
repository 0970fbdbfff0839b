// Causal prefill in bf16 with fp32 accumulation, gfx950 MFMA.
//
// One workgroup (4 waves) owns a 128-row query tile of one (batch, head);
// each wave owns 32 query rows and keeps their Q fragments in registers for
// the whole pass (Q outer, K/V inner: the loop order "AI Infra 入门…", §3
// credits to FlashAttention-2). K/V tiles of 64 keys are staged through LDS,
// double-buffered, and walked once:
//
//   Sᵀ = K·Qᵀ   v_mfma_f32_32x32x16_bf16, keys as MFMA rows, queries as
//               columns, so each lane holds one query's scores and the row
//               max / row sum are in-lane plus one cross-half exchange.
//   mask        only in tiles that cross the diagonal: key > query → −inf.
//               Tiles wholly above a wave's diagonal are skipped, and the
//               key loop stops at the tile holding the tile's last row
//               ("AI Infra 入门…", §3: tile-level classification).
//   online softmax in base 2 (scale·log2 e folded into one multiply):
//               m_new = max(m, rowmax), α = 2^(m − m_new), ℓ = α·ℓ + Σp,
//               Oᵀ ← α·Oᵀ ("05 · Tích vô hướng…", §6; "Bộ 06…", Q1).
//   Oᵀ += Vᵀ·Pᵀ P rounded to bf16 in registers — the Sᵀ accumulator layout
//               is exactly the B-operand layout, so no data moves — and Vᵀ
//               read from a transposed LDS copy written at staging time.
//   epilogue    O = Oᵀ/ℓ rounded once to bf16; LSE = ln2·(m + log2 ℓ).
//
// S and P never leave registers ("05 · Tích vô hướng…", §5–§6).
// Work items are ordered heaviest first (last query tiles see the most keys).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BR = 128, BC = 64, NW = 4;

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
    int Hq, int Hkv, int N, int n_qtiles, float scale_log2)
{
    constexpr int KS = D / 16;             // 16-wide k steps of Q·Kᵀ
    constexpr int DB = D / 32;             // 32-row blocks of Oᵀ
    constexpr int KSTR = D + 8;            // K tile row stride (elements), 16 B pad
    constexpr int VSTR = BC + 4;           // Vᵀ tile row stride (elements), 8 B pad
    constexpr int CH = D / 8;              // 16-byte chunks per row
    constexpr int RPT = BC * CH / 256;     // tile rows staged per thread (2 or 4)
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BC * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * VSTR];

    const int n_bh = gridDim.x / n_qtiles;
    const int qt = n_qtiles - 1 - (int)(blockIdx.x / n_bh);
    const int bhq = blockIdx.x % n_bh;
    const int b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv);
    const int q0 = qt * BR;

    const uint16_t *Qp = q + (size_t)bhq * N * D;
    const uint16_t *Kp = k + (size_t)(b * Hkv + hkv) * N * D;
    const uint16_t *Vp = v + (size_t)(b * Hkv + hkv) * N * D;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int qrow = q0 + wave * 32 + col;
    const int wrow0 = q0 + wave * 32, wrow1 = wrow0 + 31;

    // Q fragment (B operand of Sᵀ): query qrow, d = 16·ks + 8·half + 0..7
    bf16x8 qf[KS];
    {
        const uint16_t *qr = Qp + (size_t)min(qrow, N - 1) * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = as<bf16x8>(*(const u32x4 *)(qr + 16 * ks));
    }

    // staging assignment: rows sg·RPT + r of the tile, 16-byte chunk sc
    const int sc = tid % CH, sg = tid / CH;
    u32x4 kreg[RPT], vreg[RPT];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int key = min(j * BC + sg * RPT + r, N - 1);
            kreg[r] = *(const u32x4 *)(Kp + (size_t)key * D + 8 * sc);
            vreg[r] = *(const u32x4 *)(Vp + (size_t)key * D + 8 * sc);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            *(u32x4 *)&k_lds[buf][(sg * RPT + r) * KSTR + 8 * sc] = kreg[r];
        // transpose 8 d × RPT keys into Vᵀ rows d = 8·sc + e
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint16_t *lo = &vt_lds[buf][(8 * sc + 2 * j) * VSTR + sg * RPT];
            uint16_t *hi = &vt_lds[buf][(8 * sc + 2 * j + 1) * VSTR + sg * RPT];
            if constexpr (RPT == 4) {
                u32x2 a = {__byte_perm(vreg[0][j], vreg[1][j], 0x5410), __byte_perm(vreg[2][j], vreg[3][j], 0x5410)};
                u32x2 c = {__byte_perm(vreg[0][j], vreg[1][j], 0x7632), __byte_perm(vreg[2][j], vreg[3][j], 0x7632)};
                *(u32x2 *)lo = a;
                *(u32x2 *)hi = c;
            } else {
                *(uint32_t *)lo = __byte_perm(vreg[0][j], vreg[1][j], 0x5410);
                *(uint32_t *)hi = __byte_perm(vreg[0][j], vreg[1][j], 0x7632);
            }
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int n_kt = min(N - 1, q0 + BR - 1) / BC + 1;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const int cur = j & 1;
        if (j + 1 < n_kt) load_tile(j + 1);
        const int kt0 = j * BC;
        if (kt0 <= wrow1 && wrow0 < N) {
            // ---- Sᵀ = K Qᵀ (two 32-key blocks)
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
                const uint16_t *kr = &k_lds[cur][(kb * 32 + col) * KSTR + 8 * half];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    sacc[kb] = mfma32x32x16(as<bf16x8>(*(const u32x4 *)(kr + 16 * ks)), qf[ks], sacc[kb]);
            }
            // ---- scale, diagonal mask; lane's keys: kt0 + 32kb + 8(i/4) + 4half + i%4
            const bool diag = kt0 + BC - 1 > wrow0;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = sacc[kb][i] * scale_log2;
                    if (diag) {
                        const int key = kt0 + kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                        if (key > qrow) x = -INFINITY;
                    }
                    sacc[kb][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);  // finite: key 0 is in tile 0
            const float alpha = exp2_fast(m_run - m_new);
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2_fast(sacc[kb][i] - m_new);
                    sacc[kb][i] = p;
                    ps += p;
                }
            l_run = l_run * alpha + ps;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
            // ---- Pᵀ fragments: 16-key step mm uses S registers 8(mm%2)..+7 of block mm/2
            bf16x8 pf[4];
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                u32x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    w[t] = pack_bf16x2(sacc[mm / 2][8 * (mm % 2) + 2 * t], sacc[mm / 2][8 * (mm % 2) + 2 * t + 1]);
                pf[mm] = as<bf16x8>(w);
            }
            // ---- Oᵀ += Vᵀ Pᵀ; A slot t ↔ key 16mm + 8(t/4) + 4half + t%4
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t *vr = &vt_lds[cur][(db * 32 + col) * VSTR + 4 * half];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const u32x2 lo = *(const u32x2 *)(vr + 16 * mm);
                    const u32x2 hi = *(const u32x2 *)(vr + 16 * mm + 8);
                    const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[db] = mfma32x32x16(as<bf16x8>(a), pf[mm], oacc[db]);
                }
            }
        }
        if (j + 1 < n_kt) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = Oᵀ/ℓ, one rounding; LSE in natural log
    const float l_tot = l_run + shfl_xor(l_run, 32);
    if (qrow < N) {
        const float inv = 1.f / l_tot;
        uint16_t *orow = o + ((size_t)bhq * N + qrow) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                                 pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                *(u32x2 *)(orow + db * 32 + 8 * g + 4 * half) = w;
            }
        if (half == 0) lse[(size_t)bhq * N + qrow] = (m_run + log2_fast(l_tot)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const void *q, const void *k, const void *v, void *o,
                               float *lse, int B, int Hq, int Hkv, int N, int D,
                               float scale, hipStream_t st)
{
    if (D == 128) return launch_prefill_bf16_d128(q, k, v, o, lse, B, Hq, Hkv, N, scale, st);
    const int n_qtiles = (N + BR - 1) / BR;
    const dim3 grid((unsigned)(n_qtiles * B * Hq)), block(256);
    const float sl2 = scale * kLog2e;
    if (D == 64)
        prefill_bf16_kernel<64><<<grid, block, 0, st>>>((const uint16_t *)q, (const uint16_t *)k,
            (const uint16_t *)v, (uint16_t *)o, lse, Hq, Hkv, N, n_qtiles, sl2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
