// Hardware ceilings the measurements of the attention kernels are read
// against (libattn_probes.so, used by bench.py --ceilings; not part of the
// attention library's C ABI):
//   * attn_probe_stream_read: a plain streaming read of a device buffer, 16
//     bytes per lane per load, several loads in flight per lane, over a grid
//     of the caller's size. Its best rate over a few grid sizes is the read
//     bandwidth a decode kernel can hope for on this GPU (the 8 TB/s HBM
//     figure is the interface peak; a read-only kernel reaches less).
//   * attn_probe_stream_ranges: the same read with each workgroup streaming
//     its own contiguous range, as one split of a decode does, with a given
//     number of workgroups, threads per workgroup and loads per batch: how
//     the rate depends on the CUs in use and on the bytes in flight.
//   * attn_probe_mfma_valu: can one wave hide its own vector work under its
//     matrix work? Shader-clock cycles per step of MF 32×32×16 bf16 MFMAs
//     (independent accumulators) and NV fp32 FMAs (independent chains), one
//     wave per SIMD.
//   * attn_probe_lds_read: LDS read rate per CU of ds_read_b128 (16 bytes per
//     lane) and of the transposing ds_read_b64_tr_b16 (8 bytes per lane), on
//     conflict-free addresses, with 8 or 16 waves per CU and eight reads in
//     flight per wave.
//   * attn_probe_valu: per-wave timing (shader clock) of long runs of
//     independent v_exp_f32 (the transcendental unit the online softmax's
//     2^x uses), of fp32 FMAs, and of a software 2^x built from FMAs
//     (range reduction x = n + f with n = rint(x), a degree-6 polynomial
//     for 2^f on [−½, ½], n added to the exponent), each with eight independent chains
//     per lane and enough waves per SIMD to fill the issue slots.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                          uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; almost never stores
}

// Workgroup b reads elements [b·per, (b + 1)·per) of src in batches of U
// loads of 16 bytes per lane (T threads); every load of a batch is issued
// before any of them is used, so a lane has up to U in flight and the batch
// drains before the next one starts. One workgroup per CU is the use case:
// the waves per SIMD are pinned to T / 256, which leaves the compiler the
// registers for a whole batch (with only the launch bound it trades them for
// occupancy and keeps about a dozen loads in flight).
template <int T, int U>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(T / 256, T / 256)))
void stream_ranges_kernel(const u32x4 *__restrict__ src, size_t per, uint32_t *__restrict__ sink)
{
    const u32x4 *p = src + (size_t)blockIdx.x * per;
    size_t i = threadIdx.x;
    uint32_t acc = 0;
    for (; i + (size_t)(U - 1) * T < per; i += (size_t)U * T) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + (size_t)u * T);
        // the scheduler would otherwise interleave the uses and their waits
        // with the loads
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < per; i += T) {
        const u32x4 v = p[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; almost never stores
}

// One wave per workgroup; each step issues MF MFMAs (32×32×16 bf16 into four
// independent accumulators, round robin) and NV FMAs (eight independent
// chains). cyc[b]: the wave's shader-clock cycles over `iters` × 4 steps.
template <int MF, int NV>
__global__ __launch_bounds__(64) void mfma_valu_kernel(float *__restrict__ out,
                                                       unsigned long long *__restrict__ cyc, int iters)
{
    const int lane = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    f32x16 acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 1.0f + 0.01f * (float)(lane + k);
    const unsigned long long t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int f = 0; f < MF; ++f)
                acc[(m + f) & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[(m + f) & 3], 0, 0, 0);
#pragma unroll
            for (int v = 0; v < NV; ++v) x[v & 7] = fmaf(x[v & 7], 0.999f, 0.0001f);
        }
    }
    const unsigned long long t1 = __builtin_readcyclecounter();
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[k][i];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += x[k];
    out[(size_t)blockIdx.x * 64 + lane] = s;
    if (lane == 0) cyc[blockIdx.x] = t1 - t0;
}

// LDS read rate. The workgroup fills a 64 KiB buffer, then each wave issues
// `iters` rounds of eight reads (all eight issued before any is used) at
// conflict-free addresses: KIND 0 ds_read_b128, lane l at byte 16·l of a
// 1 KiB slot; KIND 1 ds_read_b64_tr_b16, lane l at byte 8·l of a 512-byte
// slot (64 slots either way, all inside the buffer). cyc[w]: wave w's
// shader-clock cycles over the rounds.
template <int KIND, int T>
__global__ __launch_bounds__(T) void lds_read_kernel(uint32_t *__restrict__ out,
                                                     unsigned long long *__restrict__ cyc, int iters)
{
    __shared__ __attribute__((aligned(16))) uint32_t buf[65536 / 4];
    for (int i = threadIdx.x; i < 65536 / 4; i += T) buf[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const char *base = (const char *)buf;
    constexpr int SLOT = KIND == 0 ? 1024 : 512, BYTES = KIND == 0 ? 16 : 8;
    uint32_t acc = 0;
    const unsigned long long t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
        u32x4 v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int off = ((it * 8 + r + wave) & 63) * SLOT + BYTES * lane;
            if constexpr (KIND == 0) {
                v[r] = *(const u32x4 *)(base + off);
            } else {
                const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(const_cast<char *>(base) + off));
                const uint32_t *w = (const uint32_t *)&t;
                v[r] = u32x4{w[0], w[1], 0u, 0u};
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 8; ++r) acc ^= v[r][0] ^ v[r][1] ^ v[r][2] ^ v[r][3];
    }
    const unsigned long long t1 = __builtin_readcyclecounter();
    out[(size_t)blockIdx.x * T + threadIdx.x] = acc;
    if (lane == 0) cyc[(size_t)blockIdx.x * (T / 64) + wave] = t1 - t0;
}

// 2^x from FMAs: x = n + f with n = rint(x), f in [−½, ½]; 2^f by a degree-6
// Taylor polynomial of e^(f·ln2) in Horner form (relative error < 2^-22 on
// [−½, ½]); the exponent n is added to the result's exponent bits.
__device__ __forceinline__ float exp2_poly(float x)
{
    x = fminf(fmaxf(x, -126.f), 126.f);
    const float n = __builtin_rintf(x);
    const float f = x - n;
    float p = 1.5403530e-4f;            // ln2^6 / 720
    p = fmaf(p, f, 1.3333558e-3f);      // ln2^5 / 120
    p = fmaf(p, f, 9.6181291e-3f);      // ln2^4 / 24
    p = fmaf(p, f, 5.5504109e-2f);      // ln2^3 / 6
    p = fmaf(p, f, 2.4022651e-1f);      // ln2^2 / 2
    p = fmaf(p, f, 6.9314718e-1f);      // ln2
    p = fmaf(p, f, 1.0f);
    return __int_as_float(__float_as_int(p) + ((int)n << 23));
}

template <int KIND>  // 0: v_exp_f32, 1: fma, 2: exp2_poly
__global__ __launch_bounds__(256) void valu_kernel(float *__restrict__ out, unsigned long long *__restrict__ cyc,
                                                   int iters)
{
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = -1.0f - 0.01f * (float)(threadIdx.x & 63) - 0.1f * (float)c;
    const unsigned long long t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if (KIND == 0) x[c] = __builtin_amdgcn_exp2f(x[c]);
            else if (KIND == 1) x[c] = fmaf(x[c], 0.999f, -0.5f);
            else x[c] = exp2_poly(x[c]);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) s += x[c];
    const unsigned long long t1 = __builtin_readcyclecounter();
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if ((threadIdx.x & 63) == 0) cyc[(size_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

}  // namespace

extern "C" {

// Reads nbytes (a multiple of 16) from src with `blocks` workgroups of 256
// threads, four 16-byte loads in flight per lane. Returns a hipError_t code.
int attn_probe_stream_read(const void *src, size_t nbytes, int blocks, void *sink, hipStream_t st)
{
    stream_read_kernel<4><<<blocks, 256, 0, st>>>((const u32x4 *)src, nbytes / 16, (uint32_t *)sink);
    return (int)hipGetLastError();
}

// Reads nbytes (a multiple of 16·blocks) from src, workgroup b streaming the
// b-th of `blocks` equal contiguous ranges with `threads` threads in batches
// of `batch` 16-byte loads per lane, each batch issued whole before it is
// used. (threads, batch) is one of (256, 8), (256, 16), (256, 32),
// (1024, 8); anything else returns hipErrorInvalidValue and launches
// nothing. Returns a hipError_t code.
int attn_probe_stream_ranges(const void *src, size_t nbytes, int blocks, int threads, int batch,
                             void *sink, hipStream_t st)
{
    if (blocks < 1 || nbytes % (16 * (size_t)blocks)) return (int)hipErrorInvalidValue;
    const size_t per = nbytes / 16 / (size_t)blocks;
    const u32x4 *s = (const u32x4 *)src;
    uint32_t *k = (uint32_t *)sink;
    if (threads == 256 && batch == 8) stream_ranges_kernel<256, 8><<<blocks, 256, 0, st>>>(s, per, k);
    else if (threads == 256 && batch == 16) stream_ranges_kernel<256, 16><<<blocks, 256, 0, st>>>(s, per, k);
    else if (threads == 256 && batch == 32) stream_ranges_kernel<256, 32><<<blocks, 256, 0, st>>>(s, per, k);
    else if (threads == 1024 && batch == 8) stream_ranges_kernel<1024, 8><<<blocks, 1024, 0, st>>>(s, per, k);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// mf MFMAs and nv FMAs per step, (mf, nv) one of (1, 0), (1, 4), (1, 8),
// (1, 16), (2, 8), (2, 16), (0, 8), (0, 16); `blocks` one-wave workgroups
// (1024 puts one wave on every SIMD); cyc[b] gets workgroup b's cycles over
// iters × 4 steps, out one float per lane. Anything else returns
// hipErrorInvalidValue and launches nothing.
int attn_probe_mfma_valu(int mf, int nv, int blocks, int iters, float *out, unsigned long long *cyc,
                         hipStream_t st)
{
#define ATTN_MV(M, N) \
    if (mf == M && nv == N) { mfma_valu_kernel<M, N><<<blocks, 64, 0, st>>>(out, cyc, iters); return (int)hipGetLastError(); }
    ATTN_MV(1, 0) ATTN_MV(1, 4) ATTN_MV(1, 8) ATTN_MV(1, 16) ATTN_MV(2, 8) ATTN_MV(2, 16) ATTN_MV(0, 8) ATTN_MV(0, 16)
#undef ATTN_MV
    return (int)hipErrorInvalidValue;
}

// kind 0: ds_read_b128, 1: ds_read_b64_tr_b16; threads 512 or 1024 (8 or 16
// waves per workgroup, one workgroup per CU when blocks = 256). cyc gets one
// entry per wave (blocks × threads / 64), out one word per thread. Anything
// else returns hipErrorInvalidValue and launches nothing.
int attn_probe_lds_read(int kind, int threads, int blocks, int iters, uint32_t *out,
                        unsigned long long *cyc, hipStream_t st)
{
    if (kind == 0 && threads == 512) lds_read_kernel<0, 512><<<blocks, 512, 0, st>>>(out, cyc, iters);
    else if (kind == 0 && threads == 1024) lds_read_kernel<0, 1024><<<blocks, 1024, 0, st>>>(out, cyc, iters);
    else if (kind == 1 && threads == 512) lds_read_kernel<1, 512><<<blocks, 512, 0, st>>>(out, cyc, iters);
    else if (kind == 1 && threads == 1024) lds_read_kernel<1, 1024><<<blocks, 1024, 0, st>>>(out, cyc, iters);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// kind 0: v_exp_f32, 1: fp32 FMA, 2: 2^x from FMAs. Each lane runs eight
// independent chains of `iters` steps; cyc[w] receives wave w's shader-clock
// cycles (blocks × 4 waves); out holds one float per thread.
int attn_probe_valu(int kind, int blocks, int iters, float *out, unsigned long long *cyc, hipStream_t st)
{
    if (kind == 0) valu_kernel<0><<<blocks, 256, 0, st>>>(out, cyc, iters);
    else if (kind == 1) valu_kernel<1><<<blocks, 256, 0, st>>>(out, cyc, iters);
    else if (kind == 2) valu_kernel<2><<<blocks, 256, 0, st>>>(out, cyc, iters);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // extern "C"
