// Split-K merge through the log-sum-exp ("AI Infra 入门…", §3: LSE makes
// the local reductions of Flash-Decoding mergeable).
//
// Each of `splits` partial results for a row holds, in base 2,
//   m_s  = the split's reference max (any value ≥ its scores minus a few),
//   ℓ_s  = Σ 2^(s_j − m_s) in fp32, the sum the log-sum-exp is made of,
//   λ_s  = Σ of the weights 2^(s_j − m_s) as they entered the product with V
//          (equal to ℓ_s where those weights are exact; the sum of their
//          rounded values otherwise, so that O is a convex combination of the
//          values with exactly the weights used),
//   Õ_s  = Σ 2^(s_j − m_s) · v_j   (not normalised),
// and the merge computes M = max_s m_s, w_s = 2^(m_s − M),
// O = Σ_s w_s Õ_s / Σ_s w_s λ_s (rounded once to bf16) and
// LSE = ln2 · (M + log2 Σ_s w_s ℓ_s). Splits are summed in index order, so
// the result is deterministic. An empty split (no key: m = −∞, sums 0) gets
// weight 0; a row whose splits are all empty gets O = 0 and LSE = −∞.
//
// Layout: ml[row][split] = (m, ℓ, λ, unused) as float4, part[row][split][dv]
// fp32 Õ;
// for the balanced split of a ragged batch (ragged.h), ml[slot][row] and
// part[slot][row][dv] with slot = worker + sequence.
// One 128-thread block per row; each thread reduces dv/128 channels over the
// splits, with the loads of up to 16 splits in flight at once.
#include "common.h"
#include "launch.h"
#include "ragged.h"

namespace attn {
namespace {

// Merge `splits` partial records of one row: record s at ml4[s·mstride]
// (float4) and pr[s·pstride + ...] (dv floats); thread t owns channels
// CPT·t .. CPT·t + CPT − 1.
template <int CPT, int SPT>
__device__ __forceinline__ void merge_row(const float4 *__restrict__ mr, size_t mstride,
                                          const float *__restrict__ pr_, size_t pstride, int splits,
                                          uint16_t *__restrict__ orow, float *__restrict__ lse_out,
                                          int t)
{
    // splits are taken SPT at a time with every load of a pass in flight at
    // once (one memory round trip when splits <= SPT); across passes the
    // running max grows and earlier sums are rescaled, like the online
    // softmax itself
    float M = -INFINITY, l = 0.f, lam = 0.f, acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += SPT) {
        float x[SPT][CPT];
        float4 st[SPT];
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int s = min(s0 + u, splits - 1);
            st[u] = mr[(size_t)s * mstride];
            const float *pr = pr_ + (size_t)s * pstride;
#pragma unroll
            for (int c = 0; c < CPT; ++c) x[u][c] = pr[c];
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < SPT; ++u)
            if (s0 + u < splits) Mn = fmaxf(Mn, st[u].x);
        const float Mu = Mn == -INFINITY ? 0.f : Mn;  // only empty splits so far
        const float a = exp2_fast(M - Mu);  // first pass: 2^-inf = 0
        l *= a;
        lam *= a;
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] *= a;
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            // splits past the end were loaded from a clamped index: weight 0
            const float w = s0 + u < splits ? exp2_fast(st[u].x - Mu) : 0.f;
            l = fmaf(w, st[u].y, l);
            lam = fmaf(w, st[u].z, lam);
#pragma unroll
            for (int c = 0; c < CPT; ++c) acc[c] = fmaf(w, x[u][c], acc[c]);
        }
        M = Mn;
    }
    const float inv = lam > 0.f ? 1.f / lam : 0.f;
    if constexpr (CPT == 1) {
        orow[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
    } else {
#pragma unroll
        for (int c = 0; c < CPT; c += 2) *(uint32_t *)(orow + c) = pack_bf16x2(acc[c] * inv, acc[c + 1] * inv);
    }
    if (t == 0) *lse_out = (M + log2_fast(l)) * kLn2;
}

template <int CPT, int SPT>  // channels per thread (dv / 128), split slots per pass
__global__ __launch_bounds__(128) void merge_kernel(
    const float *__restrict__ ml, const float *__restrict__ part, uint16_t *__restrict__ o,
    float *__restrict__ lse, int splits, int xcd_group)
{
    constexpr int DV = 128 * CPT;
    int row = blockIdx.x;
    if (xcd_group) {
        // rows g·G .. g·G + G − 1 of group g on XCD g % 8, where the
        // group's partials were written (blocks go to XCDs by id % 8)
        const int x = row % 8, k = row / 8;
        row = (8 * (k / xcd_group) + x) * xcd_group + k % xcd_group;
    }
    const int t = threadIdx.x;
    const size_t poff = (size_t)row * splits * DV + CPT * t;
    merge_row<CPT, SPT>((const float4 *)(ml + (size_t)row * splits * 4), 1, part + poff, DV, splits,
                        o + (size_t)row * DV + CPT * t, lse + row, t);
}

// Ragged batch, balanced split: row (b, h) gathers the records of the
// workers whose runs overlap sequence b (slots w + b, consecutive).
template <int CPT, int SPT>
__global__ __launch_bounds__(128) void merge_ragged_kernel(
    const float *__restrict__ ml, const float *__restrict__ part, uint16_t *__restrict__ o,
    float *__restrict__ lse, const int *__restrict__ kv_lens, int B, int Hq, int max_len,
    int workers, int tile)
{
    constexpr int DV = 128 * CPT;
    const int row = blockIdx.x, t = threadIdx.x;
    const int b = row / Hq, h = row % Hq;
    const int n = (ragged_len(kv_lens, b, max_len) + tile - 1) / tile;
    uint16_t *orow = o + (size_t)row * DV + CPT * t;
    if (n == 0) {  // no key: empty sums
#pragma unroll
        for (int c = 0; c < CPT; ++c) orow[c] = 0;
        if (t == 0) lse[row] = -INFINITY;
        return;
    }
    // one pass over the lengths: all tiles (T) and those before sequence b
    int T = 0, first = 0;
    {
        const int lane = __lane_id();
        for (int c = 0; c < B; c += 64) {
            const int m = c + lane < B ? (ragged_len(kv_lens, c + lane, max_len) + tile - 1) / tile : 0;
            int all = m, before = c + lane < b ? m : 0;
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                all += __shfl_xor(all, d);
                before += __shfl_xor(before, d);
            }
            T += all;
            first += before;
        }
    }
    const int P_eff = min(workers, T);
    const int w0 = ragged_owner(first, T, P_eff), w1 = ragged_owner(first + n - 1, T, P_eff);
    const size_t slot0 = (size_t)(w0 + b) * Hq + h;
    const size_t poff = slot0 * DV + CPT * t;
    merge_row<CPT, SPT>((const float4 *)ml + slot0, (size_t)Hq, part + poff, (size_t)Hq * DV,
                        w1 - w0 + 1, orow, lse + row, t);
}

}  // namespace

hipError_t launch_merge(const float *ml, const float *part, void *o, float *lse, int rows,
                        int splits, int dv, hipStream_t st, int xcd_group)
{
    if (splits > kMaxSplits) return hipErrorInvalidValue;
    const dim3 grid((unsigned)rows), block(128);
    if (dv == 128 && splits <= 8)  // one pass, no clamped duplicate loads
        merge_kernel<1, 8><<<grid, block, 0, st>>>(ml, part, (uint16_t *)o, lse, splits, xcd_group);
    else if (dv == 128)
        merge_kernel<1, 16><<<grid, block, 0, st>>>(ml, part, (uint16_t *)o, lse, splits, xcd_group);
    else if (dv == 512)
        merge_kernel<4, 16><<<grid, block, 0, st>>>(ml, part, (uint16_t *)o, lse, splits, xcd_group);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_merge_ragged(const float *ml, const float *part, void *o, float *lse,
                               const int *kv_lens, int B, int Hq, int max_len, int workers,
                               int tile, int dv, hipStream_t st)
{
    const dim3 grid((unsigned)(B * Hq)), block(128);
    // a row of a ragged batch has few records (its sequence's share of
    // the workers, plus one): passes of 4
    if (dv == 128)
        merge_ragged_kernel<1, 4><<<grid, block, 0, st>>>(ml, part, (uint16_t *)o, lse, kv_lens, B,
                                                          Hq, max_len, workers, tile);
    else if (dv == 512)
        merge_ragged_kernel<4, 4><<<grid, block, 0, st>>>(ml, part, (uint16_t *)o, lse, kv_lens, B,
                                                          Hq, max_len, workers, tile);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
