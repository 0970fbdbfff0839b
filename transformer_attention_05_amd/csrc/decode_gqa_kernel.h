// Single-query GQA decode over a bf16 K/V cache, gfx950.
//
// Decode is memory-bound: about 4 flops per byte of K/V read ("05 · Tích vô
// hướng, Softmax và toán của Attention", §4), so the design goal is to stream
// every cached K/V byte from HBM exactly once and keep the memory pipe full.
//
// Decomposition. Workgroup (split, hkv, b) owns keys
// [split·split_keys, min(kv_len, (split+1)·split_keys)) of one K/V head and
// all G = Hq/Hkv query heads that share it, so each K/V byte is loaded once
// and used G times. The split count aims at one round of about 256
// workgroups, one per CU, for either cache type (no tail); a ragged batch is
// cut into pieces of at most 768 keys instead when that is finer. The four
// waves of a workgroup take 32-key chunks in turn and software-pipeline them:
// the K and V loads of a wave's next chunk are in flight while the current
// chunk is computed.
//
// Per 32-key wave chunk:
//   * Sᵀ = K·qᵀ on v_mfma_f32_16x16x32_bf16, keys as MFMA rows, the
//     (zero-padded) heads as columns; lane l feeds K[key = l%16][8 d] straight
//     from global memory (16 B per lane), fp32 accumulation.
//   * online softmax in base 2 (scores pre-multiplied by scale·log2 e):
//     running max m, running sum ℓ, old sum and output rescaled by
//     2^(m_old − m_new) ("AI Infra 入门…", §3, online softmax); the rescale
//     is skipped when no lane's max moved (α = 1 exactly).
//   * Oᵀ += Vᵀ·Pᵀ on the same MFMA: P stays in registers (the Sᵀ accumulator
//     layout is the B-operand layout) as a bf16 pair hi + lo, so the weights
//     keep about 16 significant bits (one bf16 P would put up to 2^-9
//     relative error on every weight, which a short cache cannot average
//     away); V rows, loaded 1 KiB-contiguous
//     per wave load, pass through a per-wave LDS buffer from which
//     ds_read_b64_tr_b16 hands each lane one column of a 4-row × 16-column
//     block — the transposed A operand.
// The waves' (m, ℓ, Oᵀ) are merged in LDS; with one split the workgroup
// writes O/ℓ and LSE directly, otherwise it writes its partial (m, ℓ, Õ) to
// the workspace and a second kernel merges the partials through their
// log-sum-exp (split-K merge, "AI Infra 入门…", §3). No workgroup waits for
// another; the kernel boundary orders the partial writes before the merge.
// Slots at or past kv_len are never read. The cache loads carry the
// non-temporal hint (each cached byte is read once): 29.0 → 27.0 µs for the
// Llama-3-8B call. A ragged batch is cut into pieces of at most 768 keys
// (below), so its workgroups' ranges are short too; the hint measured
// slower only while each of them streamed a whole sequence (119 → 129 µs).
// When the number of (batch, K/V head) groups is a multiple of 8, the
// workgroup ids are remapped so that all splits of group g run on XCD g % 8
// (workgroups are dealt to the 8 XCDs round-robin by id), and the merge puts
// the group's rows on the same XCD, where the partials were written.
// FP8 cache (OCP E4M3, one byte per element): the same kernel with the K and
// V bytes converted to bf16 in registers right after they arrive
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1, exact: every E4M3 value is a
// bf16 value), so the products and the fp32 accumulation are unchanged and
// only the HBM bytes halve. A lane reads 32 contiguous bytes of its key row
// (d = 32·quad .. 32·quad + 31) and the MFMA k-steps take them in that
// order, the query fragments following the same permutation of d.
// Ragged batches: with a per-sequence length array, workgroup (split, hkv, b)
// clips its key range to its own sequence's length; splits wholly past it do
// no work and write an empty partial (m = −∞, ℓ = λ = 0, Õ = 0), which the
// merge weighs by 2^−∞ = 0. A sequence with no key gets O = 0 and
// LSE = ln 0 = −∞ (the empty sums).
//
// The kernel template sits in this header so that its bf16 and E4M3
// instantiations are compiled in two translation units (decode_gqa.hip and
// decode_gqa_fp8.hip) with different scheduling options (build.py).
#pragma once
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kWaveKeys = 32;
constexpr int kChunk = kWaves * kWaveKeys;  // keys per workgroup step
constexpr int kDB = kD / 16;                // 16-row blocks of Oᵀ

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Physical 16-byte chunk of logical chunk c in row r of a wave's V buffer
// (rows of 256 B): spreads the 4-row transposed reads over all banks.
__device__ __forceinline__ int vswz(int r, int c) { return c ^ (2 * (r & 7)); }

template <bool FP8> struct Chunk;
template <> struct Chunk<false> {
    u32x4 k[2][4];  // [16-key block][32-d step], MFMA A layout
    u32x4 v[8];     // row 4·i + quad, 16-byte chunk hcol
};
template <> struct Chunk<true> {
    u32x4 k[2][2];  // [16-key block][half]: E4M3 bytes d = 32·quad + 16·half .. + 15
    u32x4 v[4];     // row 8·i + lane/8, E4M3 bytes d = 16·(lane%8) .. + 15
};

// Cache loads carry the non-temporal hint (every cache byte is read once).
__device__ __forceinline__ u32x4 ld_cache(const char *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// One wave's chunk of 32 keys from w0 (rows past key_end repeat its last).
// kb, vb: the (b, hkv) cache rows, kD elements of 2 (bf16) or 1 (E4M3) bytes.
__device__ __forceinline__ void load_chunk(Chunk<false> &c, const char *kb, const char *vb,
                                           int w0, int key_end, int hcol, int quad, int)
{
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int key = min(w0 + 16 * blk + hcol, key_end - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            c.k[blk][s] = ld_cache(kb + 2 * ((size_t)key * kD + 32 * s + 8 * quad));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int key = min(w0 + 4 * i + quad, key_end - 1);
        c.v[i] = ld_cache(vb + 2 * ((size_t)key * kD + 8 * hcol));
    }
}
__device__ __forceinline__ void load_chunk(Chunk<true> &c, const char *kb, const char *vb,
                                           int w0, int key_end, int hcol, int quad, int lane)
{
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int key = min(w0 + 16 * blk + hcol, key_end - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            c.k[blk][h] = ld_cache(kb + (size_t)key * kD + 32 * quad + 16 * h);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = min(w0 + 8 * i + (lane >> 3), key_end - 1);
        c.v[i] = ld_cache(vb + (size_t)key * kD + 16 * (lane & 7));
    }
}

// Four E4M3 codes (one dword, lowest byte first) as four bf16, exactly.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// MFMA A operand of k-step s for 16-key block blk.
__device__ __forceinline__ bf16x8 k_operand(const Chunk<false> &c, int blk, int s) {
    return as<bf16x8>(c.k[blk][s]);
}
__device__ __forceinline__ bf16x8 k_operand(const Chunk<true> &c, int blk, int s) {
    const u32x4 w = c.k[blk][s >> 1];
    const u32x2 a = e4m3x4_to_bf16(w[2 * (s & 1)]), b = e4m3x4_to_bf16(w[2 * (s & 1) + 1]);
    return as<bf16x8>(u32x4{a[0], a[1], b[0], b[1]});
}

template <bool FP8>
__global__ __launch_bounds__(256, 2) void decode_gqa_kernel(
    const uint16_t *__restrict__ q, const char *__restrict__ kc,
    const char *__restrict__ vc, uint16_t *__restrict__ o, float *__restrict__ lse,
    int Hq, int Hkv, int G, int kv_len, int kv_cap, float scale_log2, int splits,
    int split_keys, float *__restrict__ ws_ml, float *__restrict__ ws_part,
    const int *__restrict__ kv_lens, int xcd_map)
{
    int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
    if (xcd_map) {
        // workgroups are dealt to the 8 XCDs round-robin by linear id: give
        // every split of group g the XCD g % 8 (group count a multiple of 8),
        // so the merge can find a group's partials in one L2
        const int lin = blockIdx.x + splits * (blockIdx.y + Hkv * blockIdx.z);
        const int x = lin % 8, k = lin / 8;
        const int g = 8 * (k / splits) + x;
        split = k % splits;
        hkv = g % Hkv;
        b = g / Hkv;
    }
    // ragged batch: this sequence's own length, clamped to [0, kv_len]
    if (kv_lens) kv_len = min(max(kv_lens[b], 0), kv_len);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hcol = lane & 15, quad = lane >> 4;
    const int bh = b * Hkv + hkv;
    const int key_begin = split * split_keys;
    const int key_end = min(kv_len, key_begin + split_keys);
    constexpr int kElt = FP8 ? 1 : 2;  // cache bytes per element
    const char *kbase = kc + (size_t)bh * kv_cap * kD * kElt;
    const char *vbase = vc + (size_t)bh * kv_cap * kD * kElt;

    __shared__ __attribute__((aligned(16))) char vbuf[kWaves][kWaveKeys * kD * 2];
    __shared__ float red_o[kWaves][16][kD + 4];
    __shared__ float red_m[kWaves][16], red_l[kWaves][16];

    // qᵀ as the MFMA B operand: column = head (lane % 16), 8 d per lane
    // (k-step s: d = 32·s + 8·quad, or 32·quad + 8·s for the E4M3 cache)
    bf16x8 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        u32x4 w = {0u, 0u, 0u, 0u};
        const int d0 = FP8 ? 32 * quad + 8 * s : 32 * s + 8 * quad;
        if (hcol < G)
            w = *(const u32x4 *)(q + (size_t)(b * Hq + hkv * G + hcol) * kD + d0);
        qf[s] = as<bf16x8>(w);
    }

    float m_run = -INFINITY, l_run = 0.f;  // head hcol
    f32x4 oacc[kDB];                       // Oᵀ[d = 16·db + 4·quad + i][head hcol]
#pragma unroll
    for (int db = 0; db < kDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    char *vb = vbuf[wave];
    // transposed reads: lane 16·g + 4·e + c addresses rows 4·g + e and
    // 16 + 4·g + e, columns 4·c .. 4·c + 3 of a 16-column block
    const int ve = (lane >> 2) & 3, vcol = lane & 3;
    const int vr1 = 4 * quad + ve, vr2 = 16 + 4 * quad + ve;

    auto compute = [&](const Chunk<FP8> &c, int w0) {
        // ---- Sᵀ = K qᵀ (two 16-key blocks)
        float sc[8];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma16x16x32(k_operand(c, blk, s), qf[s], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = w0 + 16 * blk + 4 * quad + i;
                sc[4 * blk + i] = key < key_end ? acc[i] * scale_log2 : -INFINITY;
            }
        }
        // ---- V rows → this wave's LDS buffer as bf16 (rows of 256 B)
        if constexpr (FP8) {
            // row 8·i + lane/8, bf16 chunks 2·(lane%8) and 2·(lane%8) + 1
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 8 * i + (lane >> 3), ch = 2 * (lane & 7);
                const u32x2 a = e4m3x4_to_bf16(c.v[i][0]), b2 = e4m3x4_to_bf16(c.v[i][1]);
                const u32x2 c2 = e4m3x4_to_bf16(c.v[i][2]), d2 = e4m3x4_to_bf16(c.v[i][3]);
                *(u32x4 *)(vb + r * (kD * 2) + 16 * vswz(r, ch)) = u32x4{a[0], a[1], b2[0], b2[1]};
                *(u32x4 *)(vb + r * (kD * 2) + 16 * vswz(r, ch + 1)) = u32x4{c2[0], c2[1], d2[0], d2[1]};
            }
        } else {
            // row 4·i + quad, chunk hcol
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + quad;
                *(u32x4 *)(vb + r * (kD * 2) + 16 * vswz(r, hcol)) = c.v[i];
            }
        }
        // ---- online softmax for head hcol (its 32 keys live in 4 lanes)
        float mx = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;  // chunk wholly past key_end
        const float alpha = exp2_fast(m_run - m_use);
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sc[j] = exp2_fast(sc[j] - m_use);
            ps += sc[j];
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < kDB; ++db) oacc[db] *= alpha;
        }
        // P as a bf16 pair hi + lo (lo = bf16 of the exact fp32 residual), so the
        // weights enter the product with about 16 significant bits, not 8
        u32x4 phi, plo;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t h = pack_bf16x2(sc[2 * t], sc[2 * t + 1]);
            phi[t] = h;
            plo[t] = pack_bf16x2(sc[2 * t] - bf16lo(h), sc[2 * t + 1] - bf16hi(h));
        }
        const bf16x8 pf_hi = as<bf16x8>(phi), pf_lo = as<bf16x8>(plo);
        wave_lds_sync();
        // ---- Oᵀ += Vᵀ Pᵀ; A slot s ↔ key 4·quad + s (s < 4) or 16 + 4·quad + s − 4
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const int ch = 2 * db + (vcol >> 1);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(vb + vr1 * (kD * 2) + 16 * vswz(vr1, ch) + 8 * (vcol & 1)));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(vb + vr2 * (kD * 2) + 16 * vswz(vr2, ch) + 8 * (vcol & 1)));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
            oacc[db] = mfma16x16x32(as<bf16x8>(a), pf_hi, oacc[db]);
            oacc[db] = mfma16x16x32(as<bf16x8>(a), pf_lo, oacc[db]);
        }
        wave_lds_sync();  // the buffer is rewritten by the next chunk
    };

    // ---- software-pipelined chunk loop (ping-pong register buffers; for
    // the E4M3 cache a third buffer, two chunks in flight, measured slower).
    // The next chunk is loaded whether or not it exists (past the end every
    // lane reads the last key row, a cache hit): with a conditional load the
    // compiler's wait for the current chunk has to assume the load was not
    // issued, and then also waits for the next chunk when it was.
    const int first = key_begin + wave * kWaveKeys;
    Chunk<FP8> ca, cb;
    if (first < key_end) load_chunk(ca, kbase, vbase, first, key_end, hcol, quad, lane);
    for (int w0 = first; w0 < key_end; w0 += 2 * kChunk) {
        const int w1 = w0 + kChunk;
        load_chunk(cb, kbase, vbase, w1, key_end, hcol, quad, lane);
        compute(ca, w0);
        if (w1 >= key_end) break;
        const int w2 = w1 + kChunk;
        load_chunk(ca, kbase, vbase, w2, key_end, hcol, quad, lane);
        compute(cb, w1);
    }

    // ---- merge the four waves through LDS
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[wave][hcol][16 * db + 4 * quad + i] = oacc[db][i];
    if (quad == 0) {
        red_m[wave][hcol] = m_run;
        red_l[wave][hcol] = l_run;
    }
    __syncthreads();
    for (int idx = tid; idx < G * kD; idx += 256) {
        const int h = idx / kD, d = idx % kD;
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
        const float Mu = M == -INFINITY ? 0.f : M;  // no key at all: every weight 0
        float acc = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2_fast(red_m[w][h] - Mu);  // idle wave: 2^-inf = 0
            acc = fmaf(f, red_o[w][h][d], acc);
            l = fmaf(f, red_l[w][h], l);
        }
        const size_t row = (size_t)b * Hq + hkv * G + h;
        if (splits == 1) {
            o[row * kD + d] = (uint16_t)(pack_bf16x2(l > 0.f ? acc / l : 0.f, 0.f) & 0xffffu);
            if (d == 0) lse[row] = (M + log2_fast(l)) * kLn2;  // no key: −∞
        } else {
            const size_t slot = row * splits + split;
            ws_part[slot * kD + d] = acc;
            if (d == 0) *(float4 *)(ws_ml + 4 * slot) = make_float4(M, l, l, 0.f);
        }
    }
}


// One launch of the split kernel; launch_decode_gqa adds the merge.
template <bool FP8>
hipError_t launch_gqa_split(const GqaPlan &p, const void *q, const void *k, const void *v,
                            void *o, float *lse, int B, int Hq, int Hkv, int kv_len, int kv_cap,
                            float scale, void *ws, hipStream_t st, const int *kv_lens, int xcd)
{
    char *w = (char *)ws;
    const dim3 grid(p.splits, Hkv, B), block(256);
    decode_gqa_kernel<FP8><<<grid, block, 0, st>>>(
        (const uint16_t *)q, (const char *)k, (const char *)v, (uint16_t *)o, lse, Hq,
        Hkv, Hq / Hkv, kv_len, kv_cap, scale * kLog2e, p.splits, p.split_keys,
        (float *)(w + p.ws_ml), (float *)(w + p.ws_part), kv_lens, xcd);
    return hipGetLastError();
}

}  // namespace
}  // namespace attn
