// Absorbed MLA decode, gfx950: bf16 latent cache, fp32 accumulation.
//
// With W_UK folded into the query ("MLA 矩阵乘法吸收的数值稳定性治理", §一),
// every query head attends to one shared latent cache whose rows are
// [latent 512 | rope 64]. The key is the whole 576-wide row and the value is
// its latent part, so one HBM read of a row serves both products. Storage is
// bf16; every product accumulates in fp32 and the output is rounded once
// (§二.2, §五).
//
// Decomposition. Workgroup (split, head group, b) has 8 waves and covers 128
// query heads, so each latent tile is read from HBM once and shared through
// LDS by all heads. Each wave owns 16 heads as the columns of
// v_mfma_f32_16x16x32_bf16:
//   Sᵀ = C·Qᵀ      keys as MFMA rows, 576-deep contraction; the wave's Q
//                  fragments stay in registers for the whole pass;
//   online softmax in base 2 (running max and sum; the output is rescaled by
//                  2^(m_old − m_new) only when some lane's max moved);
//   Oᵀ += Vᵀ·Pᵀ    P stays in registers (the Sᵀ accumulator layout is the
//                  B-operand layout) as a bf16 pair hi + lo, so the weights
//                  keep about 16 significant bits; the Vᵀ operand is fetched straight from
//                  the row-major latent tile with ds_read_b64_tr_b16, which
//                  hands each lane one column of a 4-row × 16-column block.
// Latent tiles (32 rows × 1152 B) move HBM → LDS with global_load_lds_dwordx4
// (no register staging), double-buffered so the next tile streams in while
// the current one is consumed. 16-byte chunks are XOR-swizzled per row so the
// score reads and the transposed value reads hit distinct LDS banks.
// Splits of the cache write fp32 (m, ℓ, Õ) partials; the shared merge kernel
// combines them through their log-sum-exp. Rows at or past kv_len are never
// read.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int MD = 576, MV = 512, MBC = 32, MW = 8, MH = 16 * MW;
constexpr int MKS = MD / 32;                 // 18 k-steps of the score product
constexpr int MDB = MV / 16;                 // 32 row blocks of Oᵀ
constexpr int MROWB = MD * 2;                // bytes per latent row (1152)
constexpr int MCH = MD / 8;                  // 72 sixteen-byte chunks per row
constexpr int MTILEB = MBC * MROWB;          // 36,864 bytes per tile
constexpr int MLOADS = MTILEB / 1024;        // 36 wave-wide 1 KiB loads per tile
constexpr int MTHREADS = 64 * MW;
constexpr int kTargetGroups = 256;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Physical 16-byte chunk holding logical chunk c of tile row r.
__device__ __forceinline__ int swz(int r, int c) {
    return (c & ~7) | ((c & 7) ^ ((r & 7) ^ ((r >> 3) & 1)));
}

__global__ __launch_bounds__(MTHREADS, 1) void decode_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ ckv,
    uint16_t *__restrict__ o, float *__restrict__ lse, int Hq, int kv_len, int kv_cap,
    float scale_log2, int splits, int split_keys, float *__restrict__ ws_ml,
    float *__restrict__ ws_part)
{
    __shared__ __attribute__((aligned(1024))) char tile[2][MTILEB];

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

    // HBM → LDS: wave-wide load i fills tile bytes [1024 i, 1024 i + 1024);
    // lane l's 16 bytes land at chunk position 64 i + l = (row, physical chunk).
    auto load_tile = [&](int t0, int buf) {
        for (int i = wave; i < MLOADS; i += MW) {
            const int pos = 64 * i + lane;
            const int r = pos / MCH, pc = pos % MCH;
            const int c = swz(r, pc);  // the swizzle is its own inverse
            const int key = min(t0 + r, key_end - 1);
            __builtin_amdgcn_global_load_lds((const void *)(cb + (size_t)key * MD + 8 * c),
                                             (lds_void *)&tile[buf][1024 * i], 16, 0, 0);
        }
    };

    f32x4 oacc[MDB];
#pragma unroll
    for (int db = 0; db < MDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // transposed value reads: lane 16·g + 4·e + c addresses row 4·g + e (and
    // 16 + 4·g + e), columns 4·c .. 4·c + 3 of a 16-column block
    const int vg = quad, ve = (lane >> 2) & 3, vc = lane & 3;
    const int vr1 = 4 * vg + ve, vr2 = 16 + 4 * vg + ve;

    const int n_t = (key_end - key_begin + MBC - 1) / MBC;
    load_tile(key_begin, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int t = 0; t < n_t; ++t) {
        const int cur = t & 1;
        const int t0 = key_begin + t * MBC;
        if (t + 1 < n_t) load_tile(t0 + MBC, cur ^ 1);
        if (wave_active) {
            const char *tb = tile[cur];
            float sc[8];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int r = 16 * kb + hcol;
                const char *rowp = tb + r * MROWB;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < MKS; ++ks) {
                    const u32x4 a = *(const u32x4 *)(rowp + 16 * swz(r, 4 * ks + quad));
                    acc = mfma16x16x32(as<bf16x8>(a), qf[ks], acc);
                }
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
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // exact: α = 1 changes nothing
#pragma unroll
                for (int db = 0; db < MDB; ++db) oacc[db] *= alpha;
            }
            // P as a bf16 pair hi + lo (lo = bf16 of the exact fp32 residual):
            // the weights keep about 16 significant bits in the product
            u32x4 phi, plo;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t h = pack_bf16x2(sc[2 * u], sc[2 * u + 1]);
                phi[u] = h;
                plo[u] = pack_bf16x2(sc[2 * u] - bf16lo(h), sc[2 * u + 1] - bf16hi(h));
            }
            const bf16x8 pf_hi = as<bf16x8>(phi), pf_lo = as<bf16x8>(plo);
            // Vᵀ operand: slots 0..3 ↔ keys 4·quad + e, slots 4..7 ↔ keys 16 + 4·quad + e
            const char *row1 = tb + vr1 * MROWB + 8 * (vc & 1);
            const char *row2 = tb + vr2 * MROWB + 8 * (vc & 1);
#pragma unroll
            for (int db = 0; db < MDB; ++db) {
                const int c = 2 * db + (vc >> 1);
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(row1 + 16 * swz(vr1, c)));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(row2 + 16 * swz(vr2, c)));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
                oacc[db] = mfma16x16x32(as<bf16x8>(a), pf_hi, oacc[db]);
                oacc[db] = mfma16x16x32(as<bf16x8>(a), pf_lo, oacc[db]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

}  // namespace

bool mla_plan(int B, int Hq, int kv_len, MlaPlan *p)
{
    if (B < 1 || Hq < 16 || Hq % 16 || kv_len < 1) return false;
    const long hgs = (Hq + MH - 1) / MH;
    const int tiles = (kv_len + MBC - 1) / MBC;
    const long groups = (long)B * hgs;
    int want = (int)((kTargetGroups + groups - 1) / groups);
    int s = want < 1 ? 1 : (want < tiles ? want : tiles);
    if (s > kMaxSplits) s = kMaxSplits;
    const int per = (tiles + s - 1) / s;
    s = (tiles + per - 1) / per;
    p->splits = s;
    p->split_keys = per * MBC;
    const size_t rows = (size_t)B * Hq;
    p->ws_ml = 0;
    p->ws_part = align_up(sizeof(float) * 2 * rows * s, 256);
    p->ws_total = s == 1 ? 256 : p->ws_part + align_up(sizeof(float) * MV * rows * s, 256);
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
    return launch_merge(ws_ml, ws_part, o, lse, B * Hq, p.splits, MV, st);
}

}  // namespace attn
