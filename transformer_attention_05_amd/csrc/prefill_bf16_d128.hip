// Causal prefill for head dimension 128, bf16 in/out, fp32 accumulation, gfx950.
//
// One workgroup (4 waves) owns a 128-row query tile of one (batch, head);
// each wave owns 32 query rows and keeps their Q fragments in registers for
// the whole pass (Q outer, K/V inner: the loop order "AI Infra 入门…", §3
// credits to FlashAttention-2). 64-key K and V tiles stream HBM → LDS with
// global_load_lds_dwordx4 one tile ahead of use (double-buffered, no register
// staging), both kept row-major; 16-byte chunks are XOR-swizzled per row,
// chunk c of row r stored at c ^ (2·(r & 7) | ((r >> 3) & 1)), which keeps the
// 32-row score reads and the 4-row transposed value reads on distinct banks.
//
//   Sᵀ = K·Qᵀ   v_mfma_f32_32x32x16_bf16, keys as MFMA rows, queries as
//               columns: each lane owns one query's scores, so the row max and
//               row sum are in-lane plus one cross-half exchange.
//   mask        only in tiles that cross a wave's diagonal (key > query → −inf);
//               tiles wholly above a wave's rows are skipped and the key loop
//               stops at the tile holding the tile's last row ("AI Infra
//               入门…", §3: tile-level classification).
//   online softmax in base 2: the max is taken on raw scores (scale > 0),
//               p = 2^(s·scale·log2 e − m) in one FMA + v_exp_f32; the output
//               rescale α = 2^(m_old − m_new) is skipped when no lane's max
//               moved (α = 1 exactly) ("05 · Tích vô hướng…", §6).
//   Oᵀ += Vᵀ·Pᵀ P rounded to bf16 in registers (the Sᵀ accumulator layout is
//               the B-operand layout); the Vᵀ operand comes straight from the
//               row-major V tile through ds_read_b64_tr_b16.
//   epilogue    O = Oᵀ/ℓ rounded once to bf16; LSE = ln2·(m + log2 ℓ).
//
// S and P never leave registers ("05 · Tích vô hướng…", §5–§6).
// Work order: the query tiles of one (batch, K/V head) group run on one XCD
// (workgroups are dealt to the 8 XCDs round-robin by id), heaviest first, so
// the concurrently running tiles of a group walk the same K/V through that
// XCD's L2.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int D = 128, BR = 128, BC = 64, NW = 4;
constexpr int ROWB = D * 2;               // bytes per K/V row
constexpr int TILEB = BC * ROWB;          // 16 KiB per tile
constexpr int NLOAD = TILEB / 1024;       // wave-wide 1 KiB loads per tile and tensor
constexpr int KS = D / 16, DB = D / 32;
constexpr int kXcds = 8;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz_x(int r) { return (2 * (r & 7)) | ((r >> 3) & 1); }

__global__ __launch_bounds__(256, 2) void prefill_d128_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
    int Hq, int Hkv, int N, int n_qtiles, float scale_log2)
{
    __shared__ __attribute__((aligned(1024))) char kt[2][TILEB];
    __shared__ __attribute__((aligned(1024))) char vt[2][TILEB];

    // ---- work item: contiguous runs of the (group, heavy-first) list per XCD
    const int G = Hq / Hkv;
    const int T = gridDim.x, id = blockIdx.x;
    const int xcd = id % kXcds, slot = id / kXcds;
    const int per = T / kXcds, rem = T % kXcds;
    const int w = xcd * per + min(xcd, rem) + slot;
    const int per_group = G * n_qtiles;
    const int grp = w / per_group, within = w % per_group;
    const int qt = n_qtiles - 1 - within / G;
    const int b = grp / Hkv, hkv = grp % Hkv;
    const int hq = hkv * G + within % G;
    const int bhq = b * Hq + hq;
    const int q0 = qt * BR;

    const uint16_t *Qp = q + (size_t)bhq * N * D;
    const uint16_t *Kp = k + (size_t)grp * N * D;
    const uint16_t *Vp = v + (size_t)grp * N * D;

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

    // HBM → LDS: wave-wide load idx fills tile bytes [1024·idx, +1024): rows
    // 4·idx + lane/16, physical chunk lane % 16
    auto load_tile = [&](int j, int buf) {
#pragma unroll
        for (int t = 0; t < NLOAD / NW; ++t) {
            const int idx = wave + NW * t;
            const int r = 4 * idx + (lane >> 4);
            const int c = (lane & 15) ^ swz_x(r);
            const size_t off = (size_t)min(j * BC + r, N - 1) * D + 8 * c;
            __builtin_amdgcn_global_load_lds((const void *)(Kp + off), (lds_void *)&kt[buf][1024 * idx], 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(Vp + off), (lds_void *)&vt[buf][1024 * idx], 16, 0, 0);
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    // per-lane LDS offsets (bytes within a tile)
    const int ks_x = swz_x(col);                        // rows 32·kb + col share it
    const int g = lane >> 4, e = (lane >> 2) & 3, cq = lane & 3;
    const int vr1 = 4 * half + e;                       // + 16·mm; read 2 adds 8 rows
    const int vchunk0 = 2 * (g & 1) + (cq >> 1);        // + 4·db
    const int vbyte = 8 * (cq & 1);

    const int n_kt = min(N - 1, q0 + BR - 1) / BC + 1;
    load_tile(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int j = 0; j < n_kt; ++j) {
        const int cur = j & 1;
        if (j + 1 < n_kt) load_tile(j + 1, cur ^ 1);
        const int kt0 = j * BC;
        if (kt0 <= wrow1 && wrow0 < N) {
            const char *kb_ = kt[cur];
            const char *vb_ = vt[cur];
            // ---- Sᵀ = K Qᵀ, the two 32-key blocks interleaved
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 a = *(const u32x4 *)(kb_ + (32 * kb + col) * ROWB + 16 * ((2 * ks + half) ^ ks_x));
                    sacc[kb] = mfma32x32x16(as<bf16x8>(a), qf[ks], sacc[kb]);
                }
            // ---- diagonal mask; lane's keys: kt0 + 32kb + 8(i/4) + 4half + i%4
            float mx = -INFINITY;
            if (kt0 + BC - 1 > wrow0) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kt0 + kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                        if (key > qrow) sacc[kb][i] = -INFINITY;
                    }
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
            mx = half_max(mx);
            const float m_new = fmaxf(m_run, mx * scale_log2);  // finite: key 0 is in tile 0
            const float alpha = exp2_fast(m_run - m_new);
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2_fast(fmaf(sacc[kb][i], scale_log2, -m_new));
                    sacc[kb][i] = p;
                    ps += p;
                }
            l_run = l_run * alpha + ps;
            m_run = m_new;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            }
            // ---- Pᵀ fragments: 16-key step mm uses S registers 8(mm%2)..+7 of block mm/2
            bf16x8 pf[4];
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                u32x4 wv;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    wv[t] = pack_bf16x2(sacc[mm / 2][8 * (mm % 2) + 2 * t], sacc[mm / 2][8 * (mm % 2) + 2 * t + 1]);
                pf[mm] = as<bf16x8>(wv);
            }
            // ---- Oᵀ += Vᵀ Pᵀ; A slot t ↔ key 16mm + 8(t/4) + 4half + t%4
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int r1 = 16 * mm + vr1, r2 = r1 + 8;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int ch = 4 * db + vchunk0;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(vb_ + r1 * ROWB + 16 * (ch ^ swz_x(r1)) + vbyte));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(vb_ + r2 * ROWB + 16 * (ch ^ swz_x(r2)) + vbyte));
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
                    oacc[db] = mfma32x32x16(as<bf16x8>(a), pf[mm], oacc[db]);
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: O = Oᵀ/ℓ, one rounding; LSE in natural log
    const float l_tot = half_sum(l_run);
    if (qrow < N) {
        const float inv = 1.f / l_tot;
        uint16_t *orow = o + ((size_t)bhq * N + qrow) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const u32x2 wv = {pack_bf16x2(oacc[db][4 * gg] * inv, oacc[db][4 * gg + 1] * inv),
                                  pack_bf16x2(oacc[db][4 * gg + 2] * inv, oacc[db][4 * gg + 3] * inv)};
                *(u32x2 *)(orow + db * 32 + 8 * gg + 4 * half) = wv;
            }
        if (half == 0) lse[(size_t)bhq * N + qrow] = (m_run + log2_fast(l_tot)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int B, int Hq, int Hkv, int N, float scale,
                                    hipStream_t st)
{
    const int n_qtiles = (N + BR - 1) / BR;
    const dim3 grid((unsigned)(n_qtiles * B * Hq)), block(256);
    prefill_d128_kernel<<<grid, block, 0, st>>>((const uint16_t *)q, (const uint16_t *)k,
                                                (const uint16_t *)v, (uint16_t *)o, lse, Hq, Hkv, N,
                                                n_qtiles, scale * kLog2e);
    return hipGetLastError();
}

}  // namespace attn
