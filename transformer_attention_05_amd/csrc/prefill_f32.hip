// Causal prefill in fp32 throughout (inputs, products, accumulation, output).
//
// One wave per 16-row query tile of one (batch, head); K/V tiles of 16 keys
// are staged in LDS. Lane l owns query row l/4 and a quarter of the keys of
// each tile for the scores and a quarter of the head dimension for O. The
// same tile classification as the bf16 path applies: the key loop stops at
// the tile holding the tile's last row, and the −∞ mask is evaluated only in
// tiles that cross the diagonal ("AI Infra 入门…", §3). Online softmax with
// running max and sum in base 2 ("05 · Tích vô hướng…", §6).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int TR = 16, TC = 16;

// This lane's share of K/V tile rows kt0 .. kt0 + TC − 1 (rows past N repeat
// row N − 1) into registers.
template <int D, int NL>
__device__ __forceinline__ void fetch_kv_tile(f32x4 (&kr)[NL], f32x4 (&vr)[NL], const float *Kp,
                                              const float *Vp, int kt0, int N, int lane)
{
#pragma unroll
    for (int t = 0; t < NL; ++t) {
        const int idx = lane + 64 * t, row = idx / (D / 4), c4 = idx % (D / 4);
        const int src = min(kt0 + row, N - 1);
        kr[t] = *(const f32x4 *)(Kp + (size_t)src * D + 4 * c4);
        vr[t] = *(const f32x4 *)(Vp + (size_t)src * D + 4 * c4);
    }
}

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ o, float *__restrict__ lse, int Hq, int Hkv, int N, int n_qtiles,
    float scale_log2)
{
    constexpr int DQ = D / 4;  // head-dim slice per lane
    __shared__ __attribute__((aligned(16))) float q_lds[TR][D];
    __shared__ __attribute__((aligned(16))) float k_lds[TC][D + 4];
    __shared__ __attribute__((aligned(16))) float v_lds[TC][D];

    const int n_bh = gridDim.x / n_qtiles;
    const int qt = n_qtiles - 1 - (int)(blockIdx.x / n_bh);
    const int bhq = blockIdx.x % n_bh;
    const int b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv);
    const int q0 = qt * TR;
    const float *Qp = q + (size_t)bhq * N * D;
    const float *Kp = k + (size_t)(b * Hkv + hkv) * N * D;
    const float *Vp = v + (size_t)(b * Hkv + hkv) * N * D;

    const int lane = threadIdx.x, r = lane >> 2, sub = lane & 3;
    const int qrow = q0 + r;

    {
        // all of the tile's loads first, then the stores: one round trip
        constexpr int NQ = TR * D / 4 / 64;
        f32x4 qr[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            const int idx = lane + 64 * t, row = idx / (D / 4), c4 = idx % (D / 4);
            qr[t] = *(const f32x4 *)(Qp + (size_t)min(q0 + row, N - 1) * D + 4 * c4);
        }
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            const int idx = lane + 64 * t, row = idx / (D / 4), c4 = idx % (D / 4);
            *(f32x4 *)&q_lds[row][4 * c4] = qr[t];
        }
    }

    float oacc[DQ];
#pragma unroll
    for (int e = 0; e < DQ; ++e) oacc[e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const int n_kt = min(N - 1, q0 + TR - 1) / TC + 1;

    // A tile's K/V loads (and the Q tile's) are all issued before its LDS
    // stores: one round trip per tile instead of one per slice of rows. For
    // d = 64 the K/V loads also run one tile ahead, in flight while the tile
    // before is computed (rows past N repeat row N − 1, so the load after
    // the last tile needs no condition); for d = 128 the 64 extra registers
    // cost more than that overlap gives. Measured together: 12.2 → 10.0 µs
    // for 2 heads × 64 queries (d = 64), 124.8 → 101.1 µs for 8 heads × 777
    // (d = 64), 301.9 → 246.5 µs for 8 heads × 1024 (d = 128; 451 µs with
    // the tile ahead).
    constexpr bool AHEAD = D <= 64;
    constexpr int NL = TC * D / 4 / 64;  // float4 of K (and of V) per lane per tile
    f32x4 kr[NL], vr[NL];
    if constexpr (AHEAD) fetch_kv_tile<D, NL>(kr, vr, Kp, Vp, 0, N, lane);
    for (int j = 0; j < n_kt; ++j) {
        const int kt0 = j * TC;
        __syncthreads();  // previous tile fully consumed
        if constexpr (!AHEAD) fetch_kv_tile<D, NL>(kr, vr, Kp, Vp, kt0, N, lane);
#pragma unroll
        for (int t = 0; t < NL; ++t) {
            const int idx = lane + 64 * t, row = idx / (D / 4), c4 = idx % (D / 4);
            *(f32x4 *)&k_lds[row][4 * c4] = kr[t];
            *(f32x4 *)&v_lds[row][4 * c4] = vr[t];
        }
        if constexpr (AHEAD) fetch_kv_tile<D, NL>(kr, vr, Kp, Vp, kt0 + TC, N, lane);
        __syncthreads();
        // scores for keys kt0 + 4·sub + c
        float s[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) s[c] = 0.f;
        for (int d = 0; d < D; d += 4) {
            const float4 qv = *(const float4 *)&q_lds[r][d];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4 kv = *(const float4 *)&k_lds[4 * sub + c][d];
                s[c] = fmaf(qv.x, kv.x, s[c]);
                s[c] = fmaf(qv.y, kv.y, s[c]);
                s[c] = fmaf(qv.z, kv.z, s[c]);
                s[c] = fmaf(qv.w, kv.w, s[c]);
            }
        }
        const bool diag = kt0 + TC - 1 > q0;
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s[c] *= scale_log2;
            if (diag && kt0 + 4 * sub + c > qrow) s[c] = -INFINITY;
            mx = fmaxf(mx, s[c]);
        }
        mx = fmaxf(mx, shfl_xor(mx, 1));
        mx = fmaxf(mx, shfl_xor(mx, 2));
        const float m_new = fmaxf(m_run, mx);  // finite: key 0 is in tile 0
        const float alpha = exp2_fast(m_run - m_new);
        float ps = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s[c] = exp2_fast(s[c] - m_new);
            ps += s[c];
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
        // gather the row's 16 weights from its four lanes
        float p[TC];
#pragma unroll
        for (int src = 0; src < 4; ++src)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                p[4 * src + c] = __int_as_float(__builtin_amdgcn_ds_bpermute(
                    ((lane & ~3) | src) << 2, __float_as_int(s[c])));
#pragma unroll
        for (int e = 0; e < DQ; ++e) {
            float acc = oacc[e] * alpha;
#pragma unroll
            for (int t = 0; t < TC; ++t) acc = fmaf(p[t], v_lds[t][sub * DQ + e], acc);
            oacc[e] = acc;
        }
    }

    l_run += shfl_xor(l_run, 1);
    l_run += shfl_xor(l_run, 2);
    if (qrow < N) {
        const float inv = 1.f / l_run;
        float *orow = o + ((size_t)bhq * N + qrow) * D + sub * DQ;
#pragma unroll
        for (int e = 0; e < DQ; e += 4)
            *(float4 *)(orow + e) = make_float4(oacc[e] * inv, oacc[e + 1] * inv, oacc[e + 2] * inv, oacc[e + 3] * inv);
        if (sub == 0) lse[(size_t)bhq * N + qrow] = (m_run + log2_fast(l_run)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const float *q, const float *k, const float *v, float *o,
                              float *lse, int B, int Hq, int Hkv, int N, int D,
                              float scale, hipStream_t st)
{
    const int n_qtiles = (N + TR - 1) / TR;
    const dim3 grid((unsigned)(n_qtiles * B * Hq)), block(64);
    const float sl2 = scale * kLog2e;
    if (D == 128)
        prefill_f32_kernel<128><<<grid, block, 0, st>>>(q, k, v, o, lse, Hq, Hkv, N, n_qtiles, sl2);
    else if (D == 64)
        prefill_f32_kernel<64><<<grid, block, 0, st>>>(q, k, v, o, lse, Hq, Hkv, N, n_qtiles, sl2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
