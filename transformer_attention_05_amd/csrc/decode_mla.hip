// Absorbed MLA decode, gfx950: bf16 or FP8 E4M3 latent cache, fp32
// accumulation.
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
// LDS by all heads. Per 32-key tile the work is split two ways:
//   scores    wave w owns heads 16w .. 16w + 15 as the columns of
//             v_mfma_f32_16x16x32_bf16: Sᵀ = C·Qᵀ with keys as MFMA rows over
//             the 576-deep row (the two 16-key halves as independent chains,
//             each step's tile operands requested one step ahead); the Q
//             fragments stay resident for the whole pass, 14 of the 18
//             k-steps in registers and the last 4 in LDS (the registers are
//             taken by Q and by the output); then the online softmax of those
//             heads;
//   values    wave w owns latent channels 64w .. 64w + 63 for all 128 heads:
//             Oᵀ[its 64 channels][128 heads] += Vᵀ·Pᵀ.
// The weights cross between the two through LDS: the Sᵀ accumulator of a
// wave already has the lane layout of the Pᵀ B operand (its slots are the
// same keys), so each wave writes its 16 heads' bf16 weights as 1 KiB, one
// 16-byte run per lane, and every wave reads the 8 head blocks back with
// ds_read_b128. The Vᵀ operand comes straight from the row-major latent tile
// through ds_read_b64_tr_b16 (one column of a 4-row × 16-column block per
// lane), but each wave now reads only its 64 channels: transposed reads run
// at half the rate of ds_read_b128 and were the busiest LDS traffic when
// every wave read all 512 channels for its own heads.
// Schedule. For uniform batches without the residual product the loop is
// software-pipelined over tiles: step t scores tile t + 1, then runs the
// P·V MFMAs of tile t with the softmax of tile t + 1 in five stages between
// the head blocks' MFMAs (independent work, so the VALU overlaps the matrix
// cores), one barrier per step. The other kernels score, barrier, multiply
// and barrier again per tile.
// Softmax. Base 2, against a reference max m that moves only when a score
// exceeds it by more than kLazy (so the weights 2^(s − m) stay ≤ 2^kLazy and
// the output is rescaled rarely); the rescale factor of each head goes to
// LDS with its weights. The log-sum-exp comes out exact either way.
// Weight precision. A bf16 weight carries a relative error of up to 2^-8.
// The output is normalised by the sum of the weights exactly as multiplied,
// so it is a convex combination of the values and a single dominant key
// comes out exact. For short caches (kv_len ≤ kLoMaxKeys) the few weights do
// not average their rounding errors out, so a second product adds
// Vᵀ·bf16(P − bf16(P)) and the weights enter with about 16 significant bits.
// Latent tiles (32 rows × 1152 B) move HBM → LDS with global_load_lds_dwordx4
// (no register staging, copy_to_lds16_sv / _v) into a ring of MNBUF buffers. The low
// three bits of each row's 16-byte chunk index are XORed with
// (row & 7) ^ (row / 16 & 1), which spreads both the score reads
// (ds_read_b128, 16 rows at one column) and the transposed value reads
// (8 rows × 32 B per 32-lane phase) over all 64 LDS banks. (The row / 16
// term changes no bank; without it the compiler shares address registers
// between the two 16-row halves and runs out of registers.)
// Splits of the cache write fp32 (m, ℓ, λ, Õ) partials, Õ staged through LDS
// so that every store writes whole 128-byte lines; the shared merge kernel
// combines them through their log-sum-exp. The stores take the default cache
// policy: with whole lines written, the merge then finds part of the records
// on chip (measured against non-temporal stores in one process: 32K call
// 183.3 → 180.0 µs, ragged batch 111.7 → 110.3 µs). Rows at or past kv_len
// are never read.
// E4M3 cache (F8): the stored rows are the channel-balanced latent S·c, so
// every channel fits E4M3's range ("MLA 矩阵乘法吸收的数值稳定性治理", §二.1).
// Tiles of 32 rows × 576 B are copied the same way; a score operand is
// 8 bytes (ds_read_b64) and a value operand one ds_read_b64_tr_b8 (8 rows
// of one 16-channel column block per lane group, row k in byte k), each
// widened to 8 bf16 in registers (v_cvt_scalef32_pk_bf16_fp8 with scale 1:
// exact). The value rows a lane names are chosen so the keys arrive in the
// weights' slot order, and the products, their operands and their order are
// those of the bf16 path: given a bf16 copy of the same values the two give
// the same bits. A different chunk swizzle (swz8) keeps both reads
// conflict-free on the 576-byte rows.
// Ragged batches (per-sequence lengths in device memory): the 32-key tiles of
// all sequences, in batch order, are cut into P equal runs (ragged.h), so a
// mix of short and long sequences keeps every CU busy; each piece of a run
// that lies in one sequence is one workgroup (P + B of them, all resident at
// once) writing one partial, and the merge finds a row's partials from the
// same arithmetic. The residual product is switched on per piece for
// sequences of at most kLoMaxKeys keys. A sequence with no key gets O = 0
// and LSE = −∞.
#include "common.h"
#include "launch.h"
#include "ragged.h"

#include <type_traits>

namespace attn {
namespace {

constexpr int MD = 576, MV = 512, MBC = 32, MW = 8, MH = 16 * MW;
constexpr int MNBUF = 3;                     // LDS tile ring depth
constexpr int MKS = MD / 32;                 // 18 k-steps of the score product
constexpr int MKQ = 4;                       // k-steps whose Q fragments live in LDS
constexpr int MKR = MKS - MKQ;               // k-steps whose Q fragments live in registers
// Score operand reads in flight ahead of the MFMAs: one k-step (two reads).
// Measured on the 32K workloads: three reads spill for bf16; four or six
// for E4M3 take 185 µs against 182.
constexpr int MSD = 2;
constexpr int MHB = MH / 16;                 // 8 head blocks of 16
constexpr int MDW = MV / MW;                 // 64 latent channels per wave in P·V
constexpr int MDBW = MDW / 16;               // 4 row blocks of Oᵀ per wave
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

// Tile geometry of the bf16 cache (F8 = false) and of the E4M3 cache (one
// byte per element: rows, tiles and copies halve).
template <bool F8>
struct MGeo {
    static constexpr int ROWB = F8 ? MD : MROWB;           // bytes per latent row
    static constexpr int CH = ROWB / 16;                   // 16-byte chunks per row
    static constexpr int TILEB = MBC * ROWB;               // bytes per tile
    static constexpr int LOADS = TILEB / 1024;             // wave-wide 1 KiB copies per tile
    static constexpr int LOADS_HI = (LOADS + MW - 1) / MW; // copies of waves < LOADS % MW
    static constexpr int LOADS_LO = LOADS / MW;            // copies of the other waves
};
static_assert(MGeo<true>::LOADS * 1024 == MGeo<true>::TILEB, "whole copies");
// LDS: tile ring, weights (hi and lo), per-head factors, LDS-held Q fragments
static_assert(MNBUF * MTILEB + 2 * MHB * 1024 + MH * 4 + MKQ * MW * 1024 <= 160 * 1024, "LDS");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_v2i32;

// HBM → LDS without registers: global_load_lds_dwordx4 copies 16 bytes per
// lane to LDS byte lds_block + 16·lane (lds_block is wave-uniform and goes
// to M0). Written as asm on purpose: the compiler then does not track the
// copy, and does not put a wait for every copy in flight in front of each
// later LDS read (it cannot tell which buffer a transposed read touches).
// The caller orders each copy with s_waitcnt vmcnt(N) and a barrier before
// any lane reads the block; there is no output register. The non-temporal
// hint (nt) marks the cache bytes as read once (measured: 193 → 189 µs on
// the 32K workload).
// copy_to_lds16_sv: addressed as a wave-uniform base plus a per-lane 32-bit
// byte offset (the scalar-base form of the instruction), so a full tile's
// copies need no per-lane address arithmetic.
// Both forms carry the non-temporal hint: every cache byte is read once.
__device__ __forceinline__ void copy_to_lds16_sv(const void *base, uint32_t off, const void *lds_block) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const lds_char *)lds_block;
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" :: "v"(off), "s"(base), "{m0}"(m0) : "memory");
}
// the per-lane-address form, for partial tiles
__device__ __forceinline__ void copy_to_lds16_v(const void *src, const void *lds_block) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const lds_char *)lds_block;
    asm volatile("global_load_lds_dwordx4 %0, off nt" :: "v"(src), "{m0}"(m0) : "memory");
}

// Physical 16-byte chunk holding logical chunk c of tile row r (an involution).
__device__ __forceinline__ int swz(int r, int c) {
    return (c & ~7) | ((c & 7) ^ (r & 7) ^ ((r >> 4) & 1));
}

// E4M3 tile rows (576 B = 36 chunks): the low two bits of the chunk index
// are XORed with bit 2 of the row and with bit 3 ^ bit 4 of the row. A score
// read takes one chunk of 16 consecutive rows (0–15 or 16–31) per 32-lane
// phase and a transposed value read one chunk of rows {0–7, 16–23} or
// {8–15, 24–31}; in both, the rows that fall on the same banks (equal
// row mod 4, rows being 36 chunks apart) get four different XOR values.
__device__ __forceinline__ int swz8(int r, int c) {
    return c ^ (((r >> 2) & 1) | ((((r >> 3) ^ (r >> 4)) & 1) << 1));
}
template <bool F8>
__device__ __forceinline__ int swz_t(int r, int c) { return F8 ? swz8(r, c) : swz(r, c); }

// 8 E4M3 codes → 8 bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(u32x2 w) {
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.f, true);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, false);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.f, true);
    return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                 __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

// Wait until this wave's copies of a tile have landed while the copies of
// `ahead` later tiles (0 or 1) may still be in flight.
template <bool F8>
__device__ __forceinline__ void wait_tile(int ahead, bool hi_wave) {
    if (ahead > 0) {
        if (hi_wave) wait_vmcnt<MGeo<F8>::LOADS_HI>(); else wait_vmcnt<MGeo<F8>::LOADS_LO>();
    } else {
        wait_vmcnt<0>();
    }
}

// LOM: the weight residual product off (0), on (1), or on for sequences of
// at most kLoMaxKeys keys (2); FULL: every workgroup has all 8 head blocks.
// SK = false: workgroup (split, hg, b) takes keys [split·split_keys, ...) of
// sequence b, every sequence holding kv_len keys. SK = true (ragged batch,
// grid (splits + B, hg, 1)): workgroup j takes piece j of the balanced split
// of ragged.h with `splits` workers over the tiles of all B sequences
// (lengths kv_lens[b], at most kv_len) — one worker's run within one
// sequence — and writes its partial to slot j.
template <int LOM, bool FULL, bool SK, bool F8>
__global__ __launch_bounds__(MTHREADS, 1) void decode_mla_kernel(
    const uint16_t *__restrict__ q, const char *__restrict__ ckv,
    uint16_t *__restrict__ o, float *__restrict__ lse, int Hq, int kv_len, int kv_cap,
    float scale_log2, int splits, int split_keys, float *__restrict__ ws_ml,
    float *__restrict__ ws_part, const int *__restrict__ kv_lens, int B)
{
    using G = MGeo<F8>;
    // PIPE: the software-pipelined schedule (uniform batches without the
    // residual product); its weights and factors are double-buffered
    constexpr bool PIPE = LOM == 0 && !SK;
    constexpr int NPB = PIPE ? 2 : 1;
    static_assert(MNBUF * G::TILEB + NPB * MHB * 1024 + (LOM ? MHB : 1) * 1024 + NPB * MH * 4 +
                      MKQ * MW * 1024 <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) char tile[MNBUF][G::TILEB];
    // weights in B-operand order and per-head α (then λ)
    __shared__ __attribute__((aligned(16))) u32x4 p_hi[NPB][MHB][64];
    __shared__ __attribute__((aligned(16))) u32x4 p_lo[LOM ? MHB : 1][64];
    __shared__ __attribute__((aligned(16))) float hinfo[NPB][16][MHB];
    // Q fragments of the last MKQ k-steps, each wave's own (registers are
    // all taken by the other Q fragments and the output)
    __shared__ __attribute__((aligned(16))) u32x4 q_lds[MKQ][MW][64];

    const int split = blockIdx.x, hg = blockIdx.y;
    int b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hcol = lane & 15, quad = lane >> 4;
    const int nhb = FULL ? MHB : min(MHB, (Hq - hg * MH) / 16);  // head blocks here (Hq % 16 == 0)
    const bool own = wave < nhb;                     // this wave scores heads 16·wave ..
    const int head = hg * MH + wave * 16 + hcol;     // its score head
    const bool hi_wave = wave < G::LOADS % MW;
    int seq_len, key_begin, key_end;
    if constexpr (SK) {
        int t0, t1;
        if (!ragged_piece(kv_lens, B, kv_len, MBC, splits, split, b, seq_len, t0, t1)) return;
        key_begin = t0 * MBC;
        key_end = min(seq_len, t1 * MBC);
    } else {
        seq_len = kv_len;
        key_begin = split * split_keys;
        key_end = min(kv_len, key_begin + split_keys);
    }
    const bool lo_on = LOM == 1 || (LOM == 2 && seq_len <= kLoMaxKeys);  // wave-uniform
    const char *cb = ckv + (size_t)b * kv_cap * G::ROWB;

    bf16x8 qf[MKR];
    {
        const uint16_t *qr = q + ((size_t)b * Hq + min(head, Hq - 1)) * MD + 8 * quad;
#pragma unroll
        for (int ks = 0; ks < MKR; ++ks) qf[ks] = as<bf16x8>(*(const u32x4 *)(qr + 32 * ks));
#pragma unroll
        for (int j = 0; j < MKQ; ++j) q_lds[j][wave][lane] = *(const u32x4 *)(qr + 32 * (MKR + j));
        // Make the compiler wait for these loads here, before any tile copy is
        // in flight: waited for inside the loop, they would drain the ring.
#pragma unroll
        for (int ks = 0; ks < MKR; ++ks) asm volatile("" :: "v"(qf[ks]));
        wave_lds_sync();
    }

    // HBM → LDS: wave-wide copy i = wave + MW·j fills tile bytes
    // [1024 i, 1024 i + 1024); lane l's 16 bytes land at chunk position
    // 64 i + l = (row r, physical chunk pc), and come from row r, logical
    // chunk swz(r, pc). The byte offsets within a full tile are fixed.
    // (each offset is below 2^16: two per register)
    // The copies every wave makes (j < LOADS_LO) keep their offsets packed in
    // registers; the one extra copy of the first LOADS % MW waves computes its
    // offset when issued, from a lane index made there (held across the loop,
    // that offset was spilled, and the reload's wait also waited for every
    // tile copy in flight).
    auto voff_of = [&](int j, int ln) __attribute__((always_inline)) {
        const int pos = 64 * (wave + MW * j) + ln;
        const int r = min(pos / G::CH, MBC - 1), pc = pos % G::CH;
        return (uint32_t)(r * G::ROWB + 16 * swz_t<F8>(r, pc));
    };
    uint32_t voffp[(G::LOADS_LO + 1) / 2] = {};
#pragma unroll
    for (int j = 0; j < G::LOADS_LO; ++j) voffp[j / 2] |= voff_of(j, lane) << (16 * (j & 1));
    static_assert(G::TILEB <= 65536, "tile offsets fit 16 bits");
    auto voff = [&](int j) __attribute__((always_inline)) {
        if (j < G::LOADS_LO) return (voffp[j / 2] >> (16 * (j & 1))) & 0xffffu;
        int ln;  // the lane index, recomputed here (v_mbcnt) rather than kept live
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        return voff_of(j, ln);
    };
    // Ragged batches: made opaque once per tile, so the unpacked offsets are
    // rebuilt (a shift and a mask each) rather than held in registers. There
    // they spilled, and each reload's wait also waited for every tile copy in
    // flight (measured: 125.6 → 106.3 µs for the ragged 32K batch; the
    // uniform kernels do not spill in the loop and are left as they were).
    auto voff_refresh = [&]() __attribute__((always_inline)) {
        if constexpr (SK) {
#pragma unroll
            for (int i = 0; i < (G::LOADS_LO + 1) / 2; ++i) asm volatile("" : "+v"(voffp[i]));
        }
    };
    // Rows past the split's end repeat its last row (their scores are masked).
    auto load_tile = [&](int t0, int buf) __attribute__((always_inline)) {
        if (t0 + MBC <= key_end) {
            voff_refresh();
            const char *base = cb + (size_t)t0 * G::ROWB;
#pragma unroll
            for (int j = 0; j < G::LOADS_HI; ++j)
                if (j < G::LOADS_LO || hi_wave)
                    copy_to_lds16_sv(base, voff(j), &tile[buf][1024 * (wave + MW * j)]);
        } else {
            for (int i = wave; i < G::LOADS; i += MW) {
                const int pos = 64 * i + lane;
                const int r = pos / G::CH, pc = pos % G::CH;
                const int key = min(t0 + r, key_end - 1);
                copy_to_lds16_v(cb + (size_t)key * G::ROWB + 16 * swz_t<F8>(r, pc), &tile[buf][1024 * i]);
            }
        }
    };

    // Oᵀ[d = 64·wave + 16·db + 4·quad + i][head = 16·hb + hcol of the group]
    f32x4 oacc[MDBW][MHB];
#pragma unroll
    for (int db = 0; db < MDBW; ++db)
#pragma unroll
        for (int hb = 0; hb < MHB; ++hb) oacc[db][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // per score head (the 4 lanes of a head agree): reference max, fp32
    // weight sum (for the LSE) and sum of the weights as multiplied (for O);
    // the sums are per lane and added across the head's lanes at the end
    float m_ref = -INFINITY, l_e = 0.f, l_o = 0.f;

    // transposed value reads: lane 16·g + 4·e + c addresses row 4·g + e (and
    // 16 + 4·g + e), columns 4·c .. 4·c + 3 of a 16-column block
    const int ve = (lane >> 2) & 3, vc = lane & 3;
    const int vr1 = 4 * quad + ve, vr2 = 16 + 4 * quad + ve;

    // ---- scores of this wave's 16 heads: raw q·c into sc (the scale is
    // applied in the exponent). PARTIAL: the tile runs past the split's end
    // (its last keys are masked). cbase (if set): the next full tile's
    // copies into buffer cbuf are issued between the score steps instead of
    // in one burst
    auto score_mfma = [&](const char *tb, int t0, float (&sc)[8], const char *cbase, int cbuf,
                          auto partial_tag) __attribute__((always_inline)) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
        {
            // the two 16-key halves of the tile as two independent MFMA chains,
            // the operands of step ks + 1 requested before the MFMAs of step ks
            // A operand of k-step ks: d = 32·ks + 8·quad .. + 7 of the lane's row
            // (bf16: one 16-byte chunk; E4M3: 8 bytes, widened at the MFMA)
            const char *row0 = tb + hcol * G::ROWB, *row1 = row0 + 16 * G::ROWB;
            using Raw = std::conditional_t<F8, u32x2, u32x4>;
            // The swizzled chunk of k-step ks follows one per-lane pattern for
            // even ks and one for odd ks, each moving by a fixed amount every
            // two steps: (ks odd ? po : pe) + STEP2·(ks / 2) is the chunk
            // swz(r, 4ks + quad) (swz8(r, 2ks + quad / 2) for E4M3), so the
            // addresses are two registers per row and immediate offsets.
            constexpr int STEP2 = F8 ? 64 : 128;
            auto ptrs = [&](const char *rowp, int r, const char *&pe, const char *&po)
                __attribute__((always_inline)) {
                if constexpr (F8) {
                    const int x = (quad >> 1) ^ ((r >> 2) & 1) ^ ((((r >> 3) ^ (r >> 4)) & 1) << 1);
                    pe = rowp + 16 * x + 8 * (quad & 1);
                    po = rowp + 16 * (x ^ 2) + 8 * (quad & 1);
                } else {
                    const int y = quad ^ (r & 7) ^ ((r >> 4) & 1);
                    pe = rowp + 16 * y;
                    po = rowp + 16 * (y ^ 4);
                }
            };
            const char *pe0, *po0, *pe1, *po1;
            ptrs(row0, hcol, pe0, po0);
            ptrs(row1, 16 + hcol, pe1, po1);
            auto ld = [&](int half, int ks) __attribute__((always_inline)) {
                const char *p = (ks & 1 ? (half ? po1 : po0) : (half ? pe1 : pe0)) + STEP2 * (ks >> 1);
                if constexpr (F8) return *(const u32x2 *)p;
                else return *(const u32x4 *)p;
            };
            auto opnd = [&](Raw a) __attribute__((always_inline)) {
                if constexpr (F8) return as<bf16x8>(e4m3x8_to_bf16(a));
                else return as<bf16x8>(a);
            };
            if (cbase) voff_refresh();
            // The 2·MKS operand reads in order (k-step ks, half h) = 2ks + h;
            // read u + MSD is requested before the MFMA of read u, from a
            // ring of MSD + 1 registers sets. The Q fragments held in LDS are
            // read one k-step ahead as well.
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            constexpr int NRD = 2 * MKS;
            Raw ring[MSD + 1];
#pragma unroll
            for (int u = 0; u < MSD; ++u) ring[u] = ld(u & 1, u >> 1);
            u32x4 qn = {}, qn_next = {};
            if (MKR == 0) qn_next = q_lds[0][wave][lane];
#pragma unroll
            for (int ks = 0; ks < MKS; ++ks) {
                constexpr int kEvery = (MKS + G::LOADS_HI - 1) / G::LOADS_HI;  // score steps per copy
                if (cbase && ks % kEvery == 0) {
                    const int j = ks / kEvery;
                    if (j < G::LOADS_LO || hi_wave)
                        copy_to_lds16_sv(cbase, voff(j), &tile[cbuf][1024 * (wave + MW * j)]);
                }
                qn = qn_next;
                if (ks + 1 >= MKR && ks + 1 < MKS) qn_next = q_lds[ks + 1 - MKR][wave][lane];
                const bf16x8 qk = ks < MKR ? qf[ks < MKR ? ks : 0] : as<bf16x8>(qn);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int u = 2 * ks + h;
                    if (u + MSD < NRD) ring[(u + MSD) % (MSD + 1)] = ld((u + MSD) & 1, (u + MSD) >> 1);
                    acc[h] = mfma16x16x32(opnd(ring[u % (MSD + 1)]), qk, acc[h]);
                }
                // keep the compiler from hoisting later reads (hoisting spills)
                __builtin_amdgcn_sched_barrier(0);
            }
            const f32x4 acc0 = acc[0], acc1 = acc[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i] = acc0[i];
                sc[4 + i] = acc1[i];
                if (PARTIAL && t0 + 4 * quad + i >= key_end) sc[i] = -INFINITY;
                if (PARTIAL && t0 + 16 + 4 * quad + i >= key_end) sc[4 + i] = -INFINITY;
            }
        }
    };

    // ---- online softmax of the tile's scores, weights and factors to LDS
    // buffer pb, in five stages (the pipelined schedule runs P·V MFMAs of
    // the previous tile between them): 0 the tile max, 1 the reference
    // update, 2 and 3 the weights of the two 16-key halves, 4 the stores.
    // The reference moves only when a score exceeds it by more than kLazy;
    // lanes whose reference stays get α = 2^0 = 1 exactly.
    float sm_mx = 0.f, sm_alpha = 1.f;
    u32x4 sm_phi = {}, sm_plo = {};
    auto softmax_stage = [&](const float (&sc)[8], int pb, int stage) __attribute__((always_inline)) {
        if (stage == 0) {
            float mx = sc[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));  // finite: each tile has a key < key_end
            sm_mx = mx * scale_log2;           // scale > 0: the max commutes with it
        } else if (stage == 1) {
            const bool mv = sm_mx > m_ref + kLazy;
            const float m_new = mv ? sm_mx : m_ref;
            sm_alpha = mv ? exp2_fast(m_ref - m_new) : 1.f;  // first tile: 2^-inf = 0
            l_e *= sm_alpha;
            l_o *= sm_alpha;
            m_ref = m_new;
        } else if (stage == 2 || stage == 3) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int u = 2 * (stage - 2) + v;
                const float p0 = exp2_fast(fmaf(sc[2 * u], scale_log2, -m_ref));
                const float p1 = exp2_fast(fmaf(sc[2 * u + 1], scale_log2, -m_ref));
                l_e += p0 + p1;
                const uint32_t h = pack_bf16x2(p0, p1);
                sm_phi[u] = h;
                l_o = sum_bf16x2(h, l_o);
                if (LOM != 0 && lo_on) {
                    // the residual p − bf16(p) is exact in fp32
                    const uint32_t w = pack_bf16x2(p0 - bf16lo(h), p1 - bf16hi(h));
                    sm_plo[u] = w;
                    l_o = sum_bf16x2(w, l_o);
                }
            }
        } else {
            // B operand of head block `wave`: slots 0..3 ↔ keys 4·quad + e,
            // slots 4..7 ↔ keys 16 + 4·quad + e (the Sᵀ rows this lane holds)
            p_hi[pb][wave][lane] = sm_phi;
            if (LOM != 0 && lo_on) p_lo[wave][lane] = sm_plo;
            // (the four lanes of a head hold the same α: all store it, with no
            // branch around the store)
            hinfo[pb][hcol][wave] = sm_alpha;
        }
    };
    auto scores = [&](const char *tb, int t0, int pb, const char *cbase, int cbuf,
                      auto partial_tag) __attribute__((always_inline)) {
        float sc[8];
        score_mfma(tb, t0, sc, cbase, cbuf, partial_tag);
#pragma unroll
        for (int st = 0; st < 5; ++st) softmax_stage(sc, pb, st);
    };

    // ---- Oᵀ += Vᵀ Pᵀ over this wave's 64 channels and every head block.
    // With sm set (wave-uniform), the softmax stages of the next tile's
    // scores scn (into weight buffer pbn) run between the head blocks' MFMAs:
    // they do not depend on them, so the VALU work overlaps the matrix cores.
    auto values = [&](const char *tb, int pb, const float (&scn)[8], int pbn, bool sm)
        __attribute__((always_inline)) {
        // rescale first: the new weights are relative to the moved references
        {
            const f32x4 a0 = *(const f32x4 *)&hinfo[pb][hcol][0], a1 = *(const f32x4 *)&hinfo[pb][hcol][4];
            const float al[MHB] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            bool moved = false;
#pragma unroll
            for (int hb = 0; hb < MHB; ++hb) moved |= hb < nhb && al[hb] != 1.f;
            if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
                for (int hb = 0; hb < MHB; ++hb)
#pragma unroll
                    for (int db = 0; db < MDBW; ++db) oacc[db][hb] *= al[hb];
            }
        }
        u32x4 va[MDBW];
        if constexpr (F8) {
            // ds_read_b64_tr_b8: lane 16·g + 2·r + h names row r of an 8-row
            // block (bytes 8h .. 8h + 7 of a 16-byte column block) and receives
            // column lane % 16 of the 8 rows, row k in byte k. Rows: keys
            // 4·g + r (r < 4) and 16 + 4·g + r − 4 (r ≥ 4), the slot order of
            // the weights; column block = 16 latent channels.
            const int r8 = (lane >> 1) & 7;
            const int kr = r8 < 4 ? 4 * quad + r8 : 12 + 4 * quad + r8;
            const char *rowp = tb + kr * G::ROWB + 8 * (lane & 1);
#pragma unroll
            for (int db = 0; db < MDBW; ++db) {
                const int c = MDBW * wave + db;
                const auto x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(rowp + 16 * swz8(kr, c)));
                va[db] = e4m3x8_to_bf16(__builtin_bit_cast(u32x2, x));
            }
        } else {
            const char *row1 = tb + vr1 * MROWB + 8 * (vc & 1);
            const char *row2 = tb + vr2 * MROWB + 8 * (vc & 1);
#pragma unroll
            for (int db = 0; db < MDBW; ++db) {
                const int c = 2 * (MDBW * wave + db) + (vc >> 1);
                const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(row1 + 16 * swz(vr1, c)));
                const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(row2 + 16 * swz(vr2, c)));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo4), h2 = __builtin_bit_cast(u32x2, hi4);
                va[db] = u32x4{l2[0], l2[1], h2[0], h2[1]};
            }
        }
        // the weights of head block hb + VPF are requested before the MFMAs of hb
        constexpr int VPF = 2;
        u32x4 pr[VPF + 1];
#pragma unroll
        for (int u = 0; u < VPF; ++u)
            if (u < nhb) pr[u] = p_hi[pb][u][lane];
#pragma unroll
        for (int hb = 0; hb < MHB; ++hb) {
            if (hb < nhb) {
                if (hb + VPF < nhb) pr[(hb + VPF) % (VPF + 1)] = p_hi[pb][hb + VPF][lane];
                const bf16x8 bh = as<bf16x8>(pr[hb % (VPF + 1)]);
#pragma unroll
                for (int db = 0; db < MDBW; ++db) oacc[db][hb] = mfma16x16x32(as<bf16x8>(va[db]), bh, oacc[db][hb]);
                __builtin_amdgcn_sched_barrier(0);
                if (LOM != 0 && lo_on) {
                    const bf16x8 bl = as<bf16x8>(p_lo[hb][lane]);
#pragma unroll
                    for (int db = 0; db < MDBW; ++db) oacc[db][hb] = mfma16x16x32(as<bf16x8>(va[db]), bl, oacc[db][hb]);
                }
            }
            if (hb < 5 && sm) {
                softmax_stage(scn, pbn, hb);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    const int n_t = max(0, key_end - key_begin + MBC - 1) / MBC;  // 0: split past the end
    auto do_scores = [&](const char *tb, int t0, int pb, const char *cbase, int cbuf) __attribute__((always_inline)) {
        if (own) {
            if (t0 + MBC > key_end) scores(tb, t0, pb, cbase, cbuf, std::true_type{});
            else scores(tb, t0, pb, cbase, cbuf, std::false_type{});
        }
    };
    float sc_none[8] = {};  // (no softmax between the P·V MFMAs)
    if constexpr (PIPE) {
        // Software-pipelined over tiles. Step t: wait for tile t + 1, one
        // barrier, then the score MFMAs of tile t + 1, then the P·V MFMAs of
        // tile t with the softmax of tile t + 1 run between them, its
        // weights going to buffer (t + 1) & 1. Tile t lives in buffer
        // t % MNBUF and is read in steps t − 1 and t, so the buffer of tile
        // t − 1 takes tile t + 2 from step t on (its copies spread over the
        // score steps). The barrier of step t publishes tile t + 1 and the
        // weights of tile t, and keeps the buffers step t reuses until every
        // wave has left step t − 1.
        float sc[8] = {};
        auto score_tile = [&](int u, const char *cbase, int cbuf) __attribute__((always_inline)) {
            const int u0 = key_begin + u * MBC;
            if (u0 + MBC > key_end) score_mfma(tile[u % MNBUF], u0, sc, cbase, cbuf, std::true_type{});
            else score_mfma(tile[u % MNBUF], u0, sc, cbase, cbuf, std::false_type{});
        };
        if (n_t > 0) load_tile(key_begin, 0);
        if (n_t > 1) load_tile(key_begin + MBC, 1);
        if (n_t > 0) {
            wait_tile<F8>(min(1, n_t - 1), hi_wave);
            __syncthreads();  // tile 0 visible
            if (own) {
                score_tile(0, nullptr, 0);
#pragma unroll
                for (int st = 0; st < 5; ++st) softmax_stage(sc, 0, st);
            }
        }
        for (int t = 0; t < n_t; ++t) {
            const bool next = t + 1 < n_t;
            if (next) wait_tile<F8>(0, hi_wave);
            __syncthreads();  // tile t + 1 and the weights of tile t visible
            const int tn = key_begin + (t + 2) * MBC, bn = (t + 2) % MNBUF;
            const bool refill = t + 2 < n_t, spread = refill && own && next && tn + MBC <= key_end;
            if (refill && !spread) load_tile(tn, bn);
            if (next && own) score_tile(t + 1, spread ? cb + (size_t)tn * G::ROWB : nullptr, bn);
            // (waves without score heads run the stages on zeros; their
            // weights and factors are never read)
            // (one call with a flag: two calls, with and without the
            // softmax, made the register allocator spill)
            values(tile[t % MNBUF], t & 1, sc, (t + 1) & 1, next);
        }
    } else {
        // Tile t lives in buffer t % MNBUF. Step t waits for tile t, then refills
        // the buffer of tile t − 1 with tile t + MNBUF − 1. The second barrier of
        // a step publishes the weights; the first barrier of the next step keeps
        // them until every wave has used them. (A one-barrier variant with
        // double-buffered weights measured slower: a wave's scores then compete
        // for LDS with the other waves' P·V.)
    #pragma unroll
        for (int p = 0; p < MNBUF - 1; ++p)
            if (p < n_t) load_tile(key_begin + p * MBC, p);
        for (int t = 0; t < n_t; ++t) {
            const int t0 = key_begin + t * MBC;
            wait_tile<F8>(min(MNBUF - 2, n_t - 1 - t), hi_wave);
            __syncthreads();  // tile t visible; tile t − 1 and the last weights no longer read
            // refill: a full next tile is copied from inside the score steps of
            // the waves that score; a partial one (clamped rows), or the copies of
            // a wave without score heads, in one go
            const int tn = t0 + (MNBUF - 1) * MBC, bn = (t + MNBUF - 1) % MNBUF;
            const bool refill = t + MNBUF - 1 < n_t, spread = refill && own && tn + MBC <= key_end;
            if (refill && !spread) load_tile(tn, bn);
            const char *tb = tile[t % MNBUF];
            do_scores(tb, t0, 0, spread ? cb + (size_t)tn * G::ROWB : nullptr, bn);
            __syncthreads();  // weights and rescale factors of every head visible
            values(tb, 0, sc_none, 0, false);
        }
    }

    // ---- epilogue: per-head sums over the head's four lanes
    l_e += shfl_xor(l_e, 16);
    l_e += shfl_xor(l_e, 32);
    l_o += shfl_xor(l_o, 16);
    l_o += shfl_xor(l_o, 32);
    if (!SK && splits == 1) {
        // every wave needs λ of every head: pass it through LDS
        __syncthreads();
        if (own && quad == 0) {
            hinfo[0][hcol][wave] = l_o;
            lse[(size_t)b * Hq + head] = (m_ref + log2_fast(l_e)) * kLn2;
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < MHB; ++hb) {
            if (hb >= nhb) break;
            const float lam = hinfo[0][hcol][hb];
            const float inv = lam > 0.f ? 1.f / lam : 0.f;  // no key: O = 0
            uint16_t *orow = o + ((size_t)b * Hq + hg * MH + 16 * hb + hcol) * MV + MDW * wave + 4 * quad;
#pragma unroll
            for (int db = 0; db < MDBW; ++db) {
                const u32x2 w = {pack_bf16x2(oacc[db][hb][0] * inv, oacc[db][hb][1] * inv),
                                 pack_bf16x2(oacc[db][hb][2] * inv, oacc[db][hb][3] * inv)};
                *(u32x2 *)(orow + 16 * db) = w;
            }
        }
        return;
    }
    // partial records: [row][split] for the uniform split, [slot][row of
    // the batch's heads] (slot = piece = w + b) for the balanced one
    auto rec = [&](int h) __attribute__((always_inline)) {
        return SK ? (size_t)split * Hq + h : ((size_t)b * Hq + h) * splits + split;
    };
    // the partial output Õ is stored in fp32, as accumulated: the merge
    // rounds the output once, and any value bf16 can hold fits
    if (own && quad == 0) *(float4 *)(ws_ml + 4 * rec(head)) = make_float4(m_ref, l_e, l_o, 0.f);
    // Õ goes out one 16-head block at a time through LDS, so that each store
    // instruction writes 1 KiB of one row (whole 128-byte lines): from the
    // accumulators a lane holds 16 bytes of 16 different rows, and stored
    // directly every instruction wrote 64 bytes per row. The block is staged
    // as [head][512 channels] with 16-byte chunk c of row r at c ^ r, which
    // keeps both the writes (16 rows × 4 chunks) and the row reads on all
    // banks; two staging buffers (the tile ring and the LDS-held Q, both
    // free now) alternate, so one barrier per block suffices.
    wait_vmcnt<0>();   // no tile copy may still be landing in the ring
    __syncthreads();   // every wave is done with the ring and its Q fragments
    float *const stage[2] = {(float *)&tile[0][0], (float *)&q_lds[0][0][0]};
    static_assert(sizeof(tile) >= 16 * MV * 4 && sizeof(q_lds) >= 16 * MV * 4, "staging");
#pragma unroll
    for (int hb = 0; hb < MHB; ++hb) {
        if (hb >= nhb) break;
        float *buf = stage[hb & 1];
#pragma unroll
        for (int db = 0; db < MDBW; ++db) {
            const int c = (MDW / 4) * wave + 4 * db + quad;  // chunk of row hcol
            *(f32x4 *)(buf + hcol * MV + 4 * (c ^ hcol)) = oacc[db][hb];
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < 16 / MW; ++rr) {
            const int r = (16 / MW) * wave + rr;
            float *prow = ws_part + rec(hg * MH + 16 * hb + r) * MV;
#pragma unroll
            for (int h = 0; h < MV / 256; ++h) {
                const int c = 64 * h + lane;
                const f32x4 v = *(const f32x4 *)(buf + r * MV + 4 * (c ^ r));
                *(f32x4 *)(prow + 4 * c) = v;
            }
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
    // one workgroup per CU: at most kTargetGroups workgroups, so that none
    // waits for a second round (rounding the split count up would leave a
    // few workgroups running alone after the rest)
    int want = (int)(kTargetGroups / groups);
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

bool mla_ragged_plan(int B, int Hq, int max_len, MlaPlan *p)
{
    if (B < 1 || Hq < 16 || Hq % 16 || max_len < 1) return false;
    const long hgs = (Hq + MH - 1) / MH;
    const long tiles_max = (long)B * ((max_len + MBC - 1) / MBC);
    // workers per head group: the P + B pieces (one workgroup each, one
    // workgroup per CU) should all run at once, or the last pieces, each
    // nearly a whole run, would start only when the first ones end
    long P = kTargetGroups / hgs - B;
    if (P < 16) P = 16;
    if (P > tiles_max) P = tiles_max;
    p->splits = (int)P;
    p->split_keys = 0;
    const size_t recs = (size_t)(P + B) * Hq;        // slots w + b, all heads
    p->ws_ml = 0;
    p->ws_part = align_up(sizeof(float) * 4 * recs, 256);
    p->ws_total = p->ws_part + align_up(sizeof(float) * MV * recs, 256);
    return true;
}

template <bool F8>
static hipError_t launch_decode_mla_t(const MlaPlan &p, const void *q, const void *ckv, void *o,
                                      float *lse, int B, int Hq, int kv_len, int kv_cap,
                                      float scale, void *ws, hipStream_t st, const int *kv_lens)
{
    char *w = (char *)ws;
    float *ws_ml = (float *)(w + p.ws_ml);
    float *ws_part = (float *)(w + p.ws_part);
    const int hgs = (Hq + MH - 1) / MH;
    const bool full = Hq % MH == 0;
    if (kv_lens) {
        // ragged: balanced split over the tiles of all sequences (kv_len is
        // the longest); short sequences switch the residual product on
        const dim3 grid(p.splits + B, hgs, 1);  // one workgroup per slot (piece)
        auto kern = kv_len <= kLoMaxKeys
                        ? (full ? decode_mla_kernel<1, true, true, F8> : decode_mla_kernel<1, false, true, F8>)
                        : (full ? decode_mla_kernel<2, true, true, F8> : decode_mla_kernel<2, false, true, F8>);
        kern<<<grid, dim3(MTHREADS), 0, st>>>(
            (const uint16_t *)q, (const char *)ckv, (uint16_t *)o, lse, Hq, kv_len, kv_cap,
            scale * kLog2e, p.splits, 0, ws_ml, ws_part, kv_lens, B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_merge_ragged(ws_ml, ws_part, o, lse, kv_lens, B, Hq, kv_len, p.splits, MBC,
                                   MV, st);
    }
    const dim3 grid(p.splits, hgs, B);
    auto kern = kv_len <= kLoMaxKeys
                    ? (full ? decode_mla_kernel<1, true, false, F8> : decode_mla_kernel<1, false, false, F8>)
                    : (full ? decode_mla_kernel<0, true, false, F8> : decode_mla_kernel<0, false, false, F8>);
    kern<<<grid, dim3(MTHREADS), 0, st>>>(
        (const uint16_t *)q, (const char *)ckv, (uint16_t *)o, lse, Hq, kv_len, kv_cap,
        scale * kLog2e, p.splits, p.split_keys, ws_ml, ws_part, nullptr, B);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_merge(ws_ml, ws_part, o, lse, B * Hq, p.splits, MV, st);
}

hipError_t launch_decode_mla(const MlaPlan &p, const void *q, const void *ckv, void *o,
                             float *lse, int B, int Hq, int kv_len, int kv_cap,
                             float scale, void *ws, hipStream_t st, const int *kv_lens, bool fp8)
{
    return fp8 ? launch_decode_mla_t<true>(p, q, ckv, o, lse, B, Hq, kv_len, kv_cap, scale, ws, st, kv_lens)
               : launch_decode_mla_t<false>(p, q, ckv, o, lse, B, Hq, kv_len, kv_cap, scale, ws, st, kv_lens);
}

}  // namespace attn
