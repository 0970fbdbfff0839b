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
//   online softmax in base 2 against a reference max m that moves only when
//                  a score exceeds it by more than kLazy (so the weights
//                  2^(s − m) stay ≤ 2^kLazy and the output is rescaled
//                  rarely); the log-sum-exp comes out exact either way;
//   Oᵀ += Vᵀ·Pᵀ    P stays in registers (the Sᵀ accumulator layout is the
//                  B-operand layout) rounded to bf16; the Vᵀ operand is
//                  fetched straight from the row-major latent tile with
//                  ds_read_b64_tr_b16, which hands each lane one column of a
//                  4-row × 16-column block.
// Weight precision. A bf16 weight carries a relative error of up to 2^-8.
// The output is normalised by the sum of the weights exactly as multiplied,
// so it is a convex combination of the values and a single dominant key
// comes out exact. For short caches (kv_len ≤ kLoMaxKeys) the few weights do
// not average their rounding errors out, so a second product adds
// Vᵀ·bf16(P − bf16(P)) and the weights enter with about 16 significant bits.
// Overlap. For long caches half the waves run their P·V product one tile
// behind their scores, so on each SIMD one wave's softmax (VALU, lane
// exchanges) runs while the other wave keeps the matrix unit busy.
// Latent tiles (32 rows × 1152 B) move HBM → LDS with global_load_lds_dwordx4
// (no register staging, copy_to_lds16) into a ring of MNBUF buffers. The low
// three bits of each row's 16-byte chunk index are XORed with
// (row & 7) ^ (row / 16 & 1), which spreads both the score reads
// (ds_read_b128, 16 rows at one column) and the transposed value reads
// (8 rows × 32 B per 32-lane phase) over all 64 LDS banks. (The row / 16
// term changes no bank; without it the compiler shares address registers
// between the two 16-row halves and runs out of registers.)
// Splits of the cache write fp32 (m, ℓ, λ, Õ) partials, transposed through
// LDS so that every store is a contiguous 1 KiB, with streaming
// (non-temporal) stores that do not stay dirty in L2; the shared merge kernel
// combines them through their log-sum-exp. Rows at or past kv_len are never
// read.
#include "common.h"
#include "launch.h"

#include <type_traits>

#ifndef ATTN_MLA_NBUF
#define ATTN_MLA_NBUF 4  // LDS tile ring depth (3 or 4)
#endif

namespace attn {
namespace {

constexpr int MD = 576, MV = 512, MBC = 32, MW = 8, MH = 16 * MW;
constexpr int MNBUF = ATTN_MLA_NBUF;
constexpr int MKS = MD / 32;                 // 18 k-steps of the score product
constexpr int MDB = MV / 16;                 // 32 row blocks of Oᵀ
constexpr int MROWB = MD * 2;                // bytes per latent row (1152)
constexpr int MCH = MD / 8;                  // 72 sixteen-byte chunks per row
constexpr int MTILEB = MBC * MROWB;          // 36,864 bytes per tile
constexpr int MLOADS = MTILEB / 1024;        // 36 wave-wide 1 KiB loads per tile
constexpr int MLOADS_HI = (MLOADS + MW - 1) / MW;  // loads per tile of waves < MLOADS % MW
constexpr int MLOADS_LO = MLOADS / MW;             // loads per tile of the other waves
constexpr int MTHREADS = 64 * MW;
constexpr int kTargetGroups = 256;
constexpr float kLazy = 8.f;      // reference-max slack, log2 units
constexpr int kLoMaxKeys = 512;   // caches this short get the second P product
constexpr int kOutStride = 260;   // floats per head row of the output transpose
static_assert(MNBUF >= 3 && MNBUF <= 4, "tile ring depth");
static_assert(MNBUF * MTILEB <= 160 * 1024, "LDS");
static_assert(MW * 16 * kOutStride * 4 <= MNBUF * MTILEB, "output transpose fits the ring");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Physical 16-byte chunk holding logical chunk c of tile row r (an involution).
__device__ __forceinline__ int swz(int r, int c) {
    return (c & ~7) | ((c & 7) ^ (r & 7) ^ ((r >> 4) & 1));
}

// Wait until this wave's copies of a tile have landed while the copies of
// `ahead` later tiles (0 or 1) may still be in flight.
__device__ __forceinline__ void wait_tile(int ahead, bool hi_wave) {
    if (ahead > 0) {
        if (hi_wave) wait_vmcnt<MLOADS_HI>(); else wait_vmcnt<MLOADS_LO>();
    } else {
        wait_vmcnt<0>();
    }
}

template <bool LO>
__global__ __launch_bounds__(MTHREADS, 1) void decode_mla_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ ckv,
    uint16_t *__restrict__ o, float *__restrict__ lse, int Hq, int kv_len, int kv_cap,
    float scale_log2, int splits, int split_keys, float *__restrict__ ws_ml,
    float *__restrict__ ws_part)
{
    __shared__ __attribute__((aligned(1024))) char tile[MNBUF][MTILEB];

    const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hcol = lane & 15, quad = lane >> 4;
    const int head0 = hg * MH + wave * 16;
    const bool wave_active = head0 < Hq;
    const bool hi_wave = wave < MLOADS % MW;
    // half the waves run P·V one tile behind their scores (long caches only:
    // the second weight product of short caches leaves no registers for it)
    const bool lag = !LO && wave >= MW / 2;
    const int head = head0 + hcol;
    const int key_begin = split * split_keys;
    const int key_end = min(kv_len, key_begin + split_keys);
    const uint16_t *cb = ckv + (size_t)b * kv_cap * MD;

    bf16x8 qf[MKS];
    {
        const uint16_t *qr = q + ((size_t)b * Hq + min(head, Hq - 1)) * MD + 8 * quad;
#pragma unroll
        for (int ks = 0; ks < MKS; ++ks) qf[ks] = as<bf16x8>(*(const u32x4 *)(qr + 32 * ks));
        // Make the compiler wait for these loads here, before any tile copy is
        // in flight: waited for inside the loop, they would drain the ring.
#pragma unroll
        for (int ks = 0; ks < MKS; ++ks) asm volatile("" :: "v"(qf[ks]));
    }

    // HBM → LDS: wave-wide copy i fills tile bytes [1024 i, 1024 i + 1024);
    // lane l's 16 bytes land at chunk position 64 i + l = (row, physical chunk).
    // Rows past the split's end repeat its last row (their scores are masked).
    auto load_tile = [&](int t0, int buf) {
        for (int i = wave; i < MLOADS; i += MW) {
            const int pos = 64 * i + lane;
            const int r = pos / MCH, pc = pos % MCH;
            const int key = min(t0 + r, key_end - 1);
            copy_to_lds16(cb + (size_t)key * MD + 8 * swz(r, pc), &tile[buf][1024 * i]);
        }
    };

    f32x4 oacc[MDB];
#pragma unroll
    for (int db = 0; db < MDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    // per head (the 4 lanes of a head agree): reference max, fp32 weight sum
    // (for the LSE) and sum of the weights as multiplied (for O); the sums
    // are per lane here and added across the head's lanes at the end
    float m_ref = -INFINITY, l_e = 0.f, l_o = 0.f;
    bf16x8 pf_hi, pf_lo;  // weights of the tile whose P·V is pending

    // transposed value reads: lane 16·g + 4·e + c addresses row 4·g + e (and
    // 16 + 4·g + e), columns 4·c .. 4·c + 3 of a 16-column block
    const int ve = (lane >> 2) & 3, vc = lane & 3;
    const int vr1 = 4 * quad + ve, vr2 = 16 + 4 * quad + ve;

    // ---- scores of one tile, online softmax, weights into pf_hi / pf_lo
    auto scores = [&](const char *tb, int t0) __attribute__((always_inline)) {
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
        mx = fmaxf(mx, shfl_xor(mx, 32));  // finite: each tile has a key < key_end
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + kLazy)) {
            const float m_new = mx > m_ref + kLazy ? mx : m_ref;
            const float alpha = exp2_fast(m_ref - m_new);  // first tile: 2^-inf = 0
            l_e *= alpha;
            l_o *= alpha;
#pragma unroll
            for (int db = 0; db < MDB; ++db) oacc[db] *= alpha;
            m_ref = m_new;
        }
        u32x4 phi, plo;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float p0 = exp2_fast(sc[2 * u] - m_ref), p1 = exp2_fast(sc[2 * u + 1] - m_ref);
            l_e += p0 + p1;
            const uint32_t h = pack_bf16x2(p0, p1);
            phi[u] = h;
            l_o = sum_bf16x2(h, l_o);
            if constexpr (LO) {
                // the residual p − bf16(p) is exact in fp32
                const uint32_t w = pack_bf16x2(p0 - bf16lo(h), p1 - bf16hi(h));
                plo[u] = w;
                l_o = sum_bf16x2(w, l_o);
            }
        }
        pf_hi = as<bf16x8>(phi);
        if constexpr (LO) pf_lo = as<bf16x8>(plo);
    };

    // ---- Oᵀ += Vᵀ Pᵀ for the tile in tb; A slots 0..3 ↔ keys 4·quad + e,
    // slots 4..7 ↔ keys 16 + 4·quad + e
    auto pv = [&](const char *tb) __attribute__((always_inline)) {
        const char *row1 = tb + vr1 * MROWB + 8 * (vc & 1);
        const char *row2 = tb + vr2 * MROWB + 8 * (vc & 1);
#pragma unroll
        for (int db = 0; db < MDB; ++db) {
            const int c = 2 * db + (vc >> 1);
            const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(row1 + 16 * swz(vr1, c)));
            const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(row2 + 16 * swz(vr2, c)));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo4), h2 = __builtin_bit_cast(u32x2, hi4);
            const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
            oacc[db] = mfma16x16x32(as<bf16x8>(a), pf_hi, oacc[db]);
            if constexpr (LO) oacc[db] = mfma16x16x32(as<bf16x8>(a), pf_lo, oacc[db]);
        }
    };

    // Ring: tile t lives in buffer t % MNBUF. Step t waits for tile t, then
    // refills the buffer of tile t − 2 (read last by the lagging waves at step
    // t − 1) with tile t + MNBUF − 2.
    const int n_t = (key_end - key_begin + MBC - 1) / MBC;
#pragma unroll
    for (int p = 0; p < MNBUF - 2; ++p)
        if (p < n_t) load_tile(key_begin + p * MBC, p);

    // The two halves of the workgroup run separate copies of the loop (same
    // waits and barriers), so the weights a lagging wave carries from one
    // step to the next occupy no registers in the other half.
    auto run = [&](auto lag_tag) __attribute__((always_inline)) {
        constexpr bool LAG = decltype(lag_tag)::value;
        for (int t = 0; t < n_t; ++t) {
            const int t0 = key_begin + t * MBC;
            wait_tile(min(MNBUF - 3, n_t - 1 - t), hi_wave);
            __syncthreads();  // tile t visible; tile t − 2 no longer read
            if (t + MNBUF - 2 < n_t) load_tile(t0 + (MNBUF - 2) * MBC, (t + MNBUF - 2) % MNBUF);
            if (!wave_active) continue;
            const char *tb = tile[t % MNBUF];
            if constexpr (LAG) {
                if (t > 0) pv(tile[(t + MNBUF - 1) % MNBUF]);
                scores(tb, t0);
            } else {
                scores(tb, t0);
                pv(tb);
            }
        }
        if constexpr (LAG) {
            if (wave_active && n_t > 0) pv(tile[(n_t - 1) % MNBUF]);
        }
    };
    if constexpr (LO) run(std::false_type{});
    else if (lag) run(std::true_type{});
    else run(std::false_type{});

    // ---- epilogue: per-head sums over the head's four lanes
    l_e += shfl_xor(l_e, 16);
    l_e += shfl_xor(l_e, 32);
    l_o += shfl_xor(l_o, 16);
    l_o += shfl_xor(l_o, 32);
    // lane holds Oᵀ[d = 16·db + 4·quad + i][head]
    if (splits == 1) {
        if (!wave_active || head >= Hq) return;
        const float inv = 1.f / l_o;
        uint16_t *orow = o + ((size_t)b * Hq + head) * MV;
#pragma unroll
        for (int db = 0; db < MDB; ++db) {
            const u32x2 w = {pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv),
                             pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv)};
            *(u32x2 *)(orow + 16 * db + 4 * quad) = w;
        }
        if (quad == 0) lse[(size_t)b * Hq + head] = (m_ref + log2_fast(l_e)) * kLn2;
        return;
    }
    // Partials: each wave transposes its 16 heads × 512 values through LDS
    // (half the values at a time) so that every global store writes 1 KiB of
    // one head's row.
    __syncthreads();  // every wave is done with the ring
    if (!wave_active) return;
    if (quad == 0 && head < Hq)
        *(float4 *)(ws_ml + 4 * (((size_t)b * Hq + head) * splits + split)) =
            make_float4(m_ref, l_e, l_o, 0.f);
    float *st = (float *)&tile[0][0] + wave * 16 * kOutStride;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int j = 0; j < MDB / 2; ++j) {
            const int db = (MDB / 2) * half + j;
            *(f32x4 *)(st + hcol * kOutStride + 16 * j + 4 * quad) = oacc[db];
        }
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const f32x4 v = *(const f32x4 *)(st + r * kOutStride + 4 * lane);
            if (head0 + r < Hq) {
                const size_t slot = ((size_t)b * Hq + head0 + r) * splits + split;
                __builtin_nontemporal_store(v, (f32x4 *)(ws_part + slot * MV + (MV / 2) * half + 4 * lane));
            }
        }
        wave_lds_sync();
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
    p->ws_part = align_up(sizeof(float) * 4 * rows * s, 256);
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
    auto kern = kv_len <= kLoMaxKeys ? decode_mla_kernel<true> : decode_mla_kernel<false>;
    kern<<<grid, dim3(MTHREADS), 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)ckv, (uint16_t *)o, lse, Hq, kv_len, kv_cap,
        scale * kLog2e, p.splits, p.split_keys, ws_ml, ws_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_merge(ws_ml, ws_part, o, lse, B * Hq, p.splits, MV, st);
}

}  // namespace attn
