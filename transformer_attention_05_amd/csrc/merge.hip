// Split-K merge through the log-sum-exp ("AI Infra 入门…", §3: LSE makes
// the local reductions of Flash-Decoding mergeable).
//
// Each of `splits` partial results for a row holds, in base 2,
//   m_s  = the split's running max,  ℓ_s = Σ 2^(s_j − m_s),
//   Õ_s  = Σ 2^(s_j − m_s) · v_j   (not normalised),
// and the merge computes M = max_s m_s, ℓ = Σ_s 2^(m_s − M) ℓ_s,
// O = Σ_s 2^(m_s − M) Õ_s / ℓ (rounded once to bf16), LSE = ln2 · (M + log2 ℓ).
// Splits are summed in index order, so the result is deterministic.
//
// Layout: ml[row][split][2] = (m, ℓ), part[row][split][dv]; one thread per
// (row, 4 consecutive channels).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(
    const float *__restrict__ ml, const float *__restrict__ part, uint16_t *__restrict__ o,
    float *__restrict__ lse, int rows, int splits, int dv)
{
    const int per_row = dv / 4;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const int row = (int)(gid / per_row), c4 = (int)(gid % per_row);
    if (row >= rows) return;
    const float *mr = ml + (size_t)row * splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, mr[2 * s]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float f = exp2_fast(mr[2 * s] - M);
        const f32x4 p = *(const f32x4 *)(part + ((size_t)row * splits + s) * dv + 4 * c4);
        acc += f * p;
        l = fmaf(f, mr[2 * s + 1], l);
    }
    const float inv = 1.f / l;
    const u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *(u32x2 *)(o + (size_t)row * dv + 4 * c4) = w;
    if (c4 == 0) lse[row] = (M + log2_fast(l)) * kLn2;
}

}  // namespace

hipError_t launch_merge(const float *ml, const float *part, void *o, float *lse, int rows,
                        int splits, int dv, hipStream_t st)
{
    const long threads = (long)rows * (dv / 4);
    merge_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st>>>(
        ml, part, (uint16_t *)o, lse, rows, splits, dv);
    return hipGetLastError();
}

}  // namespace attn
