// Backward of the causal prefill, head dimension 128, bf16 in/out, fp32
// accumulation, gfx950.
//
// The forward keeps the per-row log-sum-exp; the backward recomputes the
// weights from it exactly, P = 2^(s·scale·log2 e − LSE·log2 e), instead of
// storing the N×N matrix ("AI Infra 入门…", §3: the LSE turns the softmax
// division into a subtraction, which is what lets the backward recompute P).
// With dO = ∂L/∂O and D_i = dO_i·O_i (= Σ_j P_ij dP_ij):
//   dV = Pᵀ·dO,  dP = dO·Vᵀ,  dS = P ∘ (dP − D),  dQ = scale·dS·K,
//   dK = scale·dSᵀ·Q,
// dK and dV summed over the query heads that share a K/V head.
//
// Three kernels, no atomics (the result is bitwise reproducible):
//   dot    D_i = dO_i·O_i in fp32 (16 lanes per row).
//   dkdv   workgroup (b, K/V head, 128-key block), 4 waves of 32 keys each
//          with their K and V rows in registers as MFMA B operands. For each
//          query head of the group and each 32-query tile at or after the
//          block (tiles in an LDS ring of four, see below):
//            S  = Q·Kᵀ, dP = dO·Vᵀ          (v_mfma_f32_32x32x16_bf16; the
//                                           lane holds one key's column)
//            P, dS element-wise (masked on the diagonal tiles)
//            dVᵀ += dOᵀ·P, dKᵀ += Qᵀ·dS      (P and dS rounded to bf16 in
//                                           registers: their accumulator
//                                           layout is the B-operand layout;
//                                           dOᵀ and Qᵀ by ds_read_b64_tr_b16)
//   dq     workgroup (b, query head, 128-query block), 4 waves of 32 queries
//          with Qᵀ and dOᵀ fragments in registers; over the 32-key tiles up
//          to the diagonal:
//            Sᵀ = K·Qᵀ, dPᵀ = V·dOᵀ, Pᵀ and dSᵀ, dQᵀ += Kᵀ·dSᵀ
// so S and dP are computed twice (in dkdv and in dq) rather than summed into
// dQ across workgroups with atomics.
// Tiles (Q and dO for dkdv, K and V for dq; 32 rows of 256 B each) move HBM →
// LDS by direct wave-wide copies (global_load_lds_dwordx4, no register
// staging) into a ring of four, three tiles ahead of use: with two buffers
// filled through registers, the next tile's load latency was exposed once
// per tile and took half of dkdv's time. One copy of each tile serves both
// the row reads (ds_read_b128) and the transposed reads (ds_read_b64_tr_b16):
// 16-byte chunk c of row r sits at chunk c ^ (4·(r & 3) + (r / 4 & 3)),
// which puts both patterns on all 64 banks.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace attn {
namespace {

constexpr int D = 128, KS = D / 16, DB = D / 32;
constexpr int T = 32;                       // rows per wave and per tile
constexpr int NWV = 4;                      // waves per workgroup
constexpr int BLK = T * NWV;                // keys (dkdv) or queries (dq) per workgroup

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ int bswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// Reads of a swizzled tile (256-byte rows, chunk c of row r at
// c ^ bswz(r), tile base 256-byte aligned). A lane's three base addresses
// are formed once per tile; each read then takes one XOR with a
// compile-time constant (the field offset of the tile and 4096·mm ride in
// the instruction's offset):
//   row read of k-step ks (chunk 2·ks + half of row col): f = bswz(col),
//     row = col·256 + 16·(half ^ (f & 1)) + 32·(f >> 1), read at row ^ 32·ks;
//   transposed read (mm, db): lo (or hi = lo ^ (8·256 + 32)) ^ 64·db.
// The transposed read is an MFMA A operand (32 rows of d × 16 k) from a tile
// whose rows are the k index. Slot t of lane 16g + 4e + c holds tile row
// 16·mm + 8·(t/4) + 4·half + t%4, the layout the Sᵀ/P accumulator registers
// 8·mm .. 8·mm + 7 match. Rows 16·mm + 4·half + e (and + 8) have swizzle
// 4·e + half (+ 2), so chunk 4·db + low lands at 4·(db ^ e) + (low ^ (half [+ 2])).
struct SwzLane {
    uint32_t row, lo, hi;  // LDS byte addresses
};
struct SwzOff {
    uint32_t row, lo, hi;  // the same relative to the tile
};
__device__ __forceinline__ SwzOff swz_off(int lane) {
    const int col = lane & 31, half = lane >> 5, g = lane >> 4, e = (lane >> 2) & 3, c = lane & 3;
    const int f = bswz(col), low = 2 * (g & 1) + (c >> 1);
    SwzOff z;
    z.row = col * 256 + 16 * (half ^ (f & 1)) + 32 * (f >> 1);
    z.lo = (4 * half + e) * 256 + 64 * e + 16 * (low ^ half) + 8 * (c & 1);
    z.hi = z.lo ^ (8 * 256 + 32);
    return z;
}
__device__ __forceinline__ SwzLane swz_lane(const void *tile, const SwzOff &o) {
    const uint32_t base = (uint32_t)(uintptr_t)(const lds_char *)tile;
    return SwzLane{base + o.row, base + o.lo, base + o.hi};
}
template <int FIELD>
__device__ __forceinline__ u32x4 row_read(const SwzLane &z, int ks) {
    return *(lds_u32x4 *)(uintptr_t)((z.row ^ (32 * ks)) + FIELD);
}
template <int FIELD>
__device__ __forceinline__ bf16x8 tr_read(const SwzLane &z, int mm, int db) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(uintptr_t)((z.lo ^ (64 * db)) + FIELD + 16 * 256 * mm));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(uintptr_t)((z.hi ^ (64 * db)) + FIELD + 16 * 256 * mm));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return as<bf16x8>(u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// B operands of the two 16-row k-steps of a 32×32 accumulator, rounded to bf16.
__device__ __forceinline__ void pack_b(const f32x16 &acc, bf16x8 (&out)[2]) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(acc[8 * mm + 2 * t], acc[8 * mm + 2 * t + 1]);
        out[mm] = as<bf16x8>(w);
    }
}

// ---------------------------------------------------------------- D = dO·O ---
// Row statistics in the workspace, rows of each (b, head) padded to Np, a
// multiple of the 32-row tile: dd = D = dO·O and l2 = LSE·log₂e; a padded
// row gets D = 0 and l2 = +∞, so that its weights 2^(s·scale·log₂e − l2)
// are 0 without a test in the dK/dV loop.
__global__ __launch_bounds__(256) void bwd_dot_kernel(const uint16_t *__restrict__ o,
                                                      const uint16_t *__restrict__ dout,
                                                      const float *__restrict__ lse,
                                                      float *__restrict__ dd, float *__restrict__ l2,
                                                      long rows_p, int N, int Np)
{
    const long rp = (long)blockIdx.x * 16 + threadIdx.x / 16;  // padded row
    const int c = threadIdx.x % 16;  // 8 elements each
    const long bh = rp / Np;
    const int r = (int)(rp - bh * Np);
    const long row = bh * N + r;
    const bool real = rp < rows_p && r < N;
    float acc = 0.f;
    if (real) {
        const u32x4 a = *(const u32x4 *)(o + row * D + 8 * c);
        const u32x4 b = *(const u32x4 *)(dout + row * D + 8 * c);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc += bf16lo(a[t]) * bf16lo(b[t]) + bf16hi(a[t]) * bf16hi(b[t]);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
    if (rp < rows_p && c == 0) {
        dd[rp] = acc;
        l2[rp] = real ? lse[row] * kLog2e : INFINITY;
    }
}

// ------------------------------------------------------------------- dK, dV ---
// One 32-row query tile: Q and dO rows of 256 B, unpadded, 16-byte chunk c
// of row r stored at chunk c ^ bswz(r); then the 32 rows' LSE·log₂e and D
// values (+∞ and 0 for rows past the sequence). The swizzle spreads both reads over all 64 banks: a row
// read (ds_read_b128) takes one chunk of 16 rows per 16-lane phase, a
// transposed read (ds_read_b64_tr_b16) 4 chunks of 4 consecutive rows per
// 32-lane phase. A wave-wide 1 KiB copy fills 4 whole rows.
struct TileBuf {
    uint16_t qs[T * D], ds[T * D];
    float l2[T], dd[T];
};
constexpr int NRING = 4;                                    // tiles in LDS
constexpr int TILE_COPIES = 2 * (T * D * 2 / 1024) + 1;     // 8 + 8 + LSE/D
constexpr int COPIES_MIN = TILE_COPIES / NWV;               // copies every wave issues per tile

__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ dout, const float *__restrict__ l2, const float *__restrict__ dd,
    uint16_t *__restrict__ dk, uint16_t *__restrict__ dv, int Hq, int Hkv, int N, int Np, int n_kblk,
    float scale_log2, float scale)
{
    __shared__ __attribute__((aligned(1024))) TileBuf buf[NRING];

    const int G = Hq / Hkv;
    // Heaviest first (key block 0 sees every query). When the (b, K/V head)
    // groups are a multiple of 8, all key blocks of a group run on one XCD
    // (workgroups are dealt to the 8 XCDs round-robin by id): they read the
    // same Q and dO tiles, and walk them in the same order (below), so the
    // tiles come from that XCD's L2 rather than from HBM once per block.
    int kblk, bh;
    {
        const int groups = (int)gridDim.x / n_kblk, lin = blockIdx.x;
        if (groups % 8 == 0) {
            const int x = lin % 8, kk = lin / 8, per = groups / 8;
            kblk = kk / per;
            bh = 8 * (kk % per) + x;
        } else {
            kblk = lin % n_kblk;
            bh = lin / n_kblk;
        }
    }
    const int b = bh / Hkv, hkv = bh % Hkv;
    const int k0 = kblk * BLK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int kw0 = k0 + T * wave;          // this wave's keys
    const int key = kw0 + col;              // this lane's key (column)
    const size_t kvoff = (size_t)bh * N * D;

    // K and V rows of the wave's keys as B operands (k = d): d = 16·ks + 8·half
    bf16x8 kf[KS], vf[KS];
    {
        const int kr = min(key, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = as<bf16x8>(*(const u32x4 *)(k + kvoff + (size_t)kr * D + 16 * ks + 8 * half));
            vf[ks] = as<bf16x8>(*(const u32x4 *)(v + kvoff + (size_t)kr * D + 16 * ks + 8 * half));
        }
    }
    f32x16 dkacc[DB], dvacc[DB];  // dKᵀ, dVᵀ: rows d = 32·db + row(i), column = key
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dkacc[db][i] = dvacc[db][i] = 0.f;

    // staging: thread tid moves 16-byte chunks (tid, tid + 256) of the
    // 32 × 256 B Q and dO tiles, row r = chunk / 16, column chunk c = chunk % 16
    const int q_first = (k0 / T) * T;                   // first tile with a query >= k0
    const int n_qt = (N - q_first + T - 1) / T;         // query tiles per head
    const int n_it = G * n_qt;
    // Items: the query heads of the group innermost, the tiles from the last
    // one down to the diagonal, so every key block of the group starts on
    // the same tiles and they walk them together. Item it is head
    // hkv·G + it % G, tile n_qt − 1 − it / G; the copy and compute cursors
    // step through them without a division.
    struct Cursor {
        int hh, tt;
    };
    auto advance = [&](Cursor &c) __attribute__((always_inline)) {
        if (++c.hh == G) {
            c.hh = 0;
            --c.tt;
        }
    };
    // copy j of a tile (wave w issues j = w, w + 4, ...): 0..7 Q rows
    // 4j .. 4j + 3, 8..15 dO rows, 16 LSE (lanes 0..31) and D (32..63).
    // Lane l lands at row 4j + l/16, physical chunk l % 16, so it reads
    // logical chunk (l % 16) ^ bswz(row).
    auto issue_tile = [&](const Cursor &c, TileBuf &t) __attribute__((always_inline)) {
        const int h = hkv * G + c.hh, q0 = q_first + T * c.tt;
        const size_t qoff = ((size_t)b * Hq + h) * N;
        for (int j = wave; j < TILE_COPIES; j += NWV) {  // wave-uniform
            if (j == TILE_COPIES - 1) {  // padded rows: q0 + 31 < Np
                const size_t r = ((size_t)b * Hq + h) * Np + q0 + (lane & 31);
                copy4_to_lds(lane < 32 ? l2 + r : dd + r, t.l2);
                continue;
            }
            const bool isd = j >= 8;
            const int i = isd ? j - 8 : j;
            const int r = 4 * i + (lane >> 4), c = (lane & 15) ^ bswz(r);
            const uint16_t *src = (isd ? dout : q) + (qoff + min(q0 + r, N - 1)) * D + 8 * c;
            uint16_t *dst = (isd ? t.ds : t.qs) + 512 * i;
            copy16_to_lds(src, dst);
        }
    };

    Cursor cp = {0, n_qt - 1}, cc = {0, n_qt - 1};  // next item to copy, to compute
    for (int t = 0; t < NRING - 1; ++t)
        if (t < n_it) {
            issue_tile(cp, buf[t]);
            advance(cp);
        }
    wait_vmcnt<0>();
    regs_ready(kf);
    regs_ready(vf);
    __syncthreads();
    // One item: copy ahead, then S, dP, P, dS and the dV, dK products. DIAG:
    // the item may lie on or before a wave's diagonal (the block's first
    // NWV query tiles), so waves whose keys it does not see skip it and
    // the causal mask applies; the tiles after those are visible to every
    // wave in full and take neither test.
    auto step = [&](int it, auto diag_tag) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        // into the buffer of tile it − 1, which every wave is done with
        if (it + NRING - 1 < n_it) {
            issue_tile(cp, buf[(it + NRING - 1) % NRING]);
            advance(cp);
        }
        const int q0 = q_first + T * cc.tt;
        advance(cc);
        const TileBuf &tb = buf[it % NRING];
        // the lane's read addresses; the lane index is made opaque so that they
        // are rebuilt per tile (a few VALU) rather than held in registers
        int lane_x = lane;
        asm volatile("" : "+v"(lane_x));
        const SwzLane z = swz_lane(&tb, swz_off(lane_x));
        if (!DIAG || q0 + T - 1 >= kw0) {  // some query of the tile sees some key of the wave
            // ---- S = Q·Kᵀ and dP = dO·Vᵀ: rows = queries, lane column = key
            f32x16 s, dp;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = as<bf16x8>(row_read<offsetof(TileBuf, qs)>(z, ks));
                const bf16x8 c = as<bf16x8>(row_read<offsetof(TileBuf, ds)>(z, ks));
                s = mfma32x32x16(a, kf[ks], s);
                dp = mfma32x32x16(c, vf[ks], dp);
            }
            // ---- P = 2^(s·scale·log2 e − LSE₂), dS = P ∘ (dP − D); query rows
            // 8·(i/4) + 4·half + i%4 (their LSE and D come as float4 runs)
            // (padded query rows: l2 = +∞ gives P = 0, D = 0 gives dS = 0).
            // Causal mask key > query, i.e. t > 8·(i/4) + i%4 with
            // t = key − q0 − 4·half: it can hold only in the diagonal tile
            // (q0 = kw0); later tiles have t < 0.
            const int t = key - q0 - 4 * half;
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const float4 L4 = *(const float4 *)&tb.l2[8 * gi + 4 * half];
                const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
                const float4 D4 = *(const float4 *)&tb.dd[8 * gi + 4 * half];
                const float Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 4 * gi + j;
                    float p = exp2_fast(fmaf(s[i], scale_log2, -Lr[j]));
                    if (DIAG && t > 8 * gi + j) p = 0.f;
                    s[i] = p;
                    dp[i] = p * (dp[i] - Dr[j]);
                }
            }
            bf16x8 pf[2], sf[2];
            pack_b(s, pf);
            pack_b(dp, sf);
            // ---- dVᵀ += dOᵀ·P, dKᵀ += Qᵀ·dS (k = the tile's queries)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dvacc[db] = mfma32x32x16(tr_read<offsetof(TileBuf, ds)>(z, mm, db), pf[mm], dvacc[db]);
                    dkacc[db] = mfma32x32x16(tr_read<offsetof(TileBuf, qs)>(z, mm, db), sf[mm], dkacc[db]);
                }
        }
        // this wave's copies of tile it + 1 done; those of later tiles may fly
        {
            const int newer = min(it + NRING - 1, n_it - 1) - (it + 1);
            if (newer >= 2) wait_vmcnt<2 * COPIES_MIN>();
            else if (newer == 1) wait_vmcnt<COPIES_MIN>();
            else wait_vmcnt<0>();
        }
        __syncthreads();
    };
    const int n_bulk = max(0, n_qt - NWV) * G;  // items on tiles q0 >= k0 + BLK
    int it = 0;
    for (; it < n_bulk; ++it) step(it, std::false_type{});
    for (; it < n_it; ++it) step(it, std::true_type{});

    // ---- epilogue: dK = scale·(dKᵀ)ᵀ, dV; lane writes column `key`, rows d
    if (key < N) {
        uint16_t *dkr = dk + kvoff + (size_t)key * D, *dvr = dv + kvoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int d0 = 32 * db + 8 * gi + 4 * half;
                const u32x2 wk = {pack_bf16x2(dkacc[db][4 * gi] * scale, dkacc[db][4 * gi + 1] * scale),
                                  pack_bf16x2(dkacc[db][4 * gi + 2] * scale, dkacc[db][4 * gi + 3] * scale)};
                const u32x2 wv = {pack_bf16x2(dvacc[db][4 * gi], dvacc[db][4 * gi + 1]),
                                  pack_bf16x2(dvacc[db][4 * gi + 2], dvacc[db][4 * gi + 3])};
                *(u32x2 *)(dkr + d0) = wk;
                *(u32x2 *)(dvr + d0) = wv;
            }
    }
}

// ----------------------------------------------------------------------- dQ ---
struct KTileBuf {          // one 32-key tile of K and V, 256-byte rows, swizzled (bswz)
    uint16_t ks[T * D], vs[T * D];
};
constexpr int KTILE_COPIES = 2 * (T * D * 2 / 1024);         // 8 + 8
static_assert(KTILE_COPIES % NWV == 0, "every wave issues the same copies per tile");

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dd,
    uint16_t *__restrict__ dq, int Hq, int Hkv, int N, int Np, int n_qblk, float scale_log2, float scale)
{
    __shared__ __attribute__((aligned(1024))) KTileBuf buf[NRING];

    // Heaviest first (the last query block sees every key). When the (b,
    // K/V head) groups are a multiple of 8, every query block of every query
    // head of a group runs on one XCD: they all walk the group's K and V
    // tiles from the first one up, so the tiles come from that XCD's L2.
    int qblk, bhq;
    {
        const int G = Hq / Hkv, groups = (int)gridDim.x / (n_qblk * G), lin = blockIdx.x;
        if (groups % 8 == 0) {
            const int x = lin % 8, kk = lin / 8, per = groups / 8;
            const int rem = kk % (per * G), gr = 8 * (rem / G) + x;
            qblk = n_qblk - 1 - kk / (per * G);
            bhq = (gr / Hkv) * Hq + (gr % Hkv) * G + rem % G;
        } else {
            qblk = n_qblk - 1 - lin % n_qblk;
            bhq = lin / n_qblk;
        }
    }
    const int b = bhq / Hq, hq = bhq % Hq, hkv = hq / (Hq / Hkv);
    const int q0 = qblk * BLK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int qw0 = q0 + T * wave, qrow = qw0 + col;  // this lane's query (column)
    const size_t qoff = (size_t)bhq * N * D, kvoff = ((size_t)b * Hkv + hkv) * N * D;

    // Qᵀ and dOᵀ as B operands (k = d): d = 16·ks + 8·half
    bf16x8 qf[KS], df[KS];
    {
        const int r = min(qrow, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = as<bf16x8>(*(const u32x4 *)(q + qoff + (size_t)r * D + 16 * ks + 8 * half));
            df[ks] = as<bf16x8>(*(const u32x4 *)(dout + qoff + (size_t)r * D + 16 * ks + 8 * half));
        }
    }
    const float lse2 = lse[(size_t)bhq * N + min(qrow, N - 1)] * kLog2e;
    const float dq_d = dd[(size_t)bhq * Np + min(qrow, N - 1)];
    f32x16 acc[DB];  // dQᵀ: rows d, column = query
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    const int n_kt = min(N - 1, q0 + BLK - 1) / T + 1;   // key tiles up to the block's last row
    // copy i of a tile (wave w issues i = w, w + 4, ...): 0..7 K rows
    // 4i .. 4i + 3, 8..15 V rows; lane l lands at row 4i + l/16, physical
    // chunk l % 16, and reads logical chunk (l % 16) ^ bswz(row)
    auto issue_tile = [&](int j, KTileBuf &t) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KTILE_COPIES / NWV; ++u) {
            const int i = wave + NWV * u;
            const bool isv = i >= 8;
            const int ii = isv ? i - 8 : i;
            const int r = 4 * ii + (lane >> 4), c = (lane & 15) ^ bswz(r);
            const uint16_t *src = (isv ? v : k) + kvoff + (size_t)min(T * j + r, N - 1) * D + 8 * c;
            uint16_t *dst = (isv ? t.vs : t.ks) + 512 * ii;
            copy16_to_lds(src, dst);
        }
    };

    for (int t = 0; t < NRING - 1; ++t)
        if (t < n_kt) issue_tile(t, buf[t]);
    wait_vmcnt<0>();
    regs_ready(qf);
    regs_ready(df);
    regs_ready(lse2);
    regs_ready(dq_d);
    __syncthreads();
    const SwzOff zo = swz_off(lane);
    for (int j = 0; j < n_kt; ++j) {
        // into the buffer of tile j − 1, which every wave is done with
        if (j + NRING - 1 < n_kt) issue_tile(j + NRING - 1, buf[(j + NRING - 1) % NRING]);
        const KTileBuf &tb = buf[j % NRING];
        const SwzLane z = swz_lane(&tb, zo);
        const int kt0 = T * j;
        if (kt0 <= qw0 + T - 1 && qw0 < N) {
            // ---- Sᵀ = K·Qᵀ, dPᵀ = V·dOᵀ: rows = keys, lane column = query
            f32x16 s, dp;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = as<bf16x8>(row_read<offsetof(KTileBuf, ks)>(z, ks));
                const bf16x8 c = as<bf16x8>(row_read<offsetof(KTileBuf, vs)>(z, ks));
                s = mfma32x32x16(a, qf[ks], s);
                dp = mfma32x32x16(c, df[ks], dp);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = exp2_fast(fmaf(s[i], scale_log2, -lse2));
            if (kt0 + T - 1 > qw0) {  // keys after some query of the wave (wave-uniform)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kt0 + 8 * (i / 4) + 4 * half + (i % 4) > qrow) s[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) dp[i] = s[i] * (dp[i] - dq_d);
            bf16x8 sf[2];
            pack_b(dp, sf);
            // ---- dQᵀ += Kᵀ·dSᵀ (k = the tile's keys)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = mfma32x32x16(tr_read<offsetof(KTileBuf, ks)>(z, mm, db), sf[mm], acc[db]);
        }
        {   // this wave's copies of tile j + 1 done; those of later tiles may fly
            constexpr int per = KTILE_COPIES / NWV;
            const int newer = min(j + NRING - 1, n_kt - 1) - (j + 1);
            if (newer >= 2) wait_vmcnt<2 * per>();
            else if (newer == 1) wait_vmcnt<per>();
            else wait_vmcnt<0>();
        }
        __syncthreads();
    }

    if (qrow < N) {
        uint16_t *row = dq + qoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const u32x2 w = {pack_bf16x2(acc[db][4 * gi] * scale, acc[db][4 * gi + 1] * scale),
                                 pack_bf16x2(acc[db][4 * gi + 2] * scale, acc[db][4 * gi + 3] * scale)};
                *(u32x2 *)(row + 32 * db + 8 * gi + 4 * half) = w;
            }
    }
}

}  // namespace

// dd then l2, each [B·Hq][Np] fp32 (Np = N rounded up to the 32-row tile)
static size_t bwd_rows_padded(int B, int Hq, int N) { return (size_t)B * Hq * ((N + T - 1) / T * T); }
size_t prefill_bwd_workspace_bytes(int B, int Hq, int N)
{
    return align_up(2 * sizeof(float) * bwd_rows_padded(B, Hq, N), 256);
}

hipError_t launch_prefill_bwd_d128(const void *q, const void *k, const void *v, const void *o,
                                   const float *lse, const void *dout, void *dq, void *dk,
                                   void *dv, int B, int Hq, int Hkv, int N, float scale,
                                   void *ws, hipStream_t st)
{
    const int Np = (N + T - 1) / T * T;
    const long rows_p = (long)bwd_rows_padded(B, Hq, N);
    float *dd = (float *)ws, *l2 = dd + rows_p;
    bwd_dot_kernel<<<dim3((unsigned)((rows_p + 15) / 16)), dim3(256), 0, st>>>(
        (const uint16_t *)o, (const uint16_t *)dout, lse, dd, l2, rows_p, N, Np);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float sl2 = scale * kLog2e;
    const int n_blk = (N + BLK - 1) / BLK;
    bwd_dkdv_kernel<<<dim3((unsigned)(n_blk * B * Hkv)), dim3(256), 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dout, l2,
        dd, (uint16_t *)dk, (uint16_t *)dv, Hq, Hkv, N, Np, n_blk, sl2, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    bwd_dq_kernel<<<dim3((unsigned)(n_blk * B * Hq)), dim3(256), 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dout, lse,
        dd, (uint16_t *)dq, Hq, Hkv, N, Np, n_blk, sl2, scale);
    return hipGetLastError();
}

}  // namespace attn
