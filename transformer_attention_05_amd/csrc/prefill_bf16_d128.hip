// Causal prefill for head dimension 128, bf16 in/out, fp32 accumulation, gfx950.
//
// One workgroup (8 waves) owns a 256-row query tile of one (batch, head);
// each wave owns 32 query rows and keeps their Q fragments in registers for
// the whole pass (Q outer, K/V inner: the loop order "AI Infra 入门…", §3
// credits to FlashAttention-2). 64-key K and V tiles stream HBM → LDS with
// global_load_lds_dwordx4 two tiles ahead of use (a ring of four, no register
// staging; the bulk tiles take one barrier per pair), both row-major in
// unpadded 256-byte rows: 16-byte chunk c of row r sits at chunk
// c ^ (4·(r & 3) + (r / 4 & 3)), which spreads both the score reads (one
// chunk of 16 rows per 16-lane ds_read_b128 phase) and the transposed value
// reads (4 chunks of 4 rows per 32-lane phase) over all 64 banks. A
// wave-wide direct load fills 1 KiB of LDS, 4 whole rows, each lane fetching
// the chunk its slot holds. (Padded rows, 272 B for K and 320 B for V, are
// also conflict-free and give every read a compile-time offset, but take
// 37 KiB per tile against 32 and measured 1–2 % slower.)
//
//   Sᵀ = K·Qᵀ   v_mfma_f32_32x32x16_bf16, keys as MFMA rows, queries as
//               columns: each lane owns one query's scores, so the row max and
//               row sum are in-lane plus one cross-half exchange.
//   mask        only in tiles that cross a wave's diagonal (key > query → −inf);
//               tiles wholly above a wave's rows are skipped and the key loop
//               stops at the tile holding the tile's last row ("AI Infra
//               入门…", §3: tile-level classification).
//   online softmax in base 2: the max is taken on raw scores (scale > 0),
//               p = 2^(s·scale·log2 e − m) in one FMA + v_exp_f32, with the
//               running max m and the rescale of ℓ and O by 2^(m_old − m_new)
//               ("05 · Tích vô hướng…", §6), skipped when no lane's max moved.
//   Oᵀ += Vᵀ·Pᵀ P rounded to bf16 in registers (the Sᵀ accumulator layout is
//               the B-operand layout); the Vᵀ operand comes straight from the
//               row-major V tile through ds_read_b64_tr_b16.
//   epilogue    O = Oᵀ/ℓ rounded once to bf16; LSE = ln2·(m + log2 ℓ).
//
// S and P never leave registers ("05 · Tích vô hướng…", §5–§6).
// Loop split: the key tiles before a workgroup's first row, visible to every
// wave, run in a loop of their own with only the unmasked step; the few
// tiles around the diagonal follow with a per-wave choice of skip, masked
// or unmasked step. (With all three in one loop the compiler kept the output
// in two register sets and copied 64 registers per tile.)
// Work order: the query tiles of one (batch, K/V head) group run on one XCD
// (workgroups are dealt to the 8 XCDs round-robin by id), heaviest first, so
// the concurrently running tiles of a group walk the same K/V through that
// XCD's L2.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace attn {
namespace {

// 8 waves of 32 query rows; a ring of four 64-key K/V tiles in unpadded,
// swizzled 256-byte rows; the bulk tiles two per barrier. (Measured and not
// kept: 4 waves, rings of 2, 3 and 5 tiles, padded rows of 272 and 320
// bytes, one tile per barrier, masks evaluated on every tile, a lazy
// reference max, sched_barrier groups of the transposed reads.)
constexpr int NW = 8, NBUF = 4;
constexpr int D = 128, BR = 32 * NW, BC = 64;
constexpr int ROWB = 256;                 // LDS row stride of the K and V tiles (bytes)
constexpr int KTILEB = BC * ROWB;         // 16 KiB
constexpr int VTILEB = BC * ROWB;         // 16 KiB
constexpr int KLOADS = KTILEB / 1024, VLOADS = VTILEB / 1024;
constexpr int KPW = (KLOADS + NW - 1) / NW, VPW = (VLOADS + NW - 1) / NW;
constexpr int LOADS_MIN = KLOADS / NW + VLOADS / NW;  // loads every wave issues per tile
constexpr int KS = D / 16, DB = D / 32;
constexpr int kXcds = 8;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Global byte offset, within a K/V tile, of the 16 bytes that lane `lane` of
// wave-wide direct load `idx` brings into LDS slot 64·idx + lane (a copy
// fills 4 whole rows of 16 slots). Rows past `rows` (the end of the
// sequence) are clamped to the last valid row. 16-byte chunk c of tile row r
// sits at chunk c ^ bswz(r): a score read takes one chunk of 16 rows per
// 16-lane phase of ds_read_b128, a transposed value read 4 chunks of 4
// consecutive rows per 32-lane phase of ds_read_b64_tr_b16, and the swizzle
// puts both on all 64 banks.
__device__ __forceinline__ int bswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ uint32_t tile_src(int idx, int lane, int rows) {
    const int s = 64 * idx + lane;
    const int r = s / 16, c = (s % 16) ^ bswz(r);
    return (uint32_t)(min(r, rows - 1) * (D * 2) + 16 * c);
}


// N queries per (batch, head). CHUNK = false: K/V hold the same N positions
// (rows of N slots). CHUNK = true: K/V are caches of kv_cap slots per (batch,
// K/V head) filled to kv_lens[b], whose last N entries are the queries' own
// positions, so query i sits at position kv_lens[b] − N + i.
// CHUNK with gridDim.y = S > 1: workgroup (item, s) takes the s-th of S
// contiguous ranges of its query tile's key tiles and writes an fp32 partial
// (m, ℓ, λ, Õ) to ws_ml / ws_part ([row][s], row = bhq·N + query) for the
// LSE merge, instead of O and the LSE.
template <bool CHUNK>
__global__ __launch_bounds__(64 * NW, 2) void prefill_d128_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
    int Hq, int Hkv, int N, int n_qtiles, float scale_log2, int kv_cap,
    const int *__restrict__ kv_lens, float *__restrict__ ws_ml, float *__restrict__ ws_part)
{
    __shared__ __attribute__((aligned(1024))) char kt[NBUF][KTILEB];
    __shared__ __attribute__((aligned(1024))) char vt[NBUF][VTILEB];

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
    // keys of this sequence, their row stride, and the position of query 0
    // (lengths outside [N, kv_cap] are clamped into it)
    int kv_len = N, kv_stride = N, q_off = 0;
    if constexpr (CHUNK) {
        kv_len = min(max(kv_lens[b], N), kv_cap);
        kv_stride = kv_cap;
        q_off = kv_len - N;
    }

    const uint16_t *Qp = q + (size_t)bhq * N * D;
    const char *Kp = (const char *)(k + (size_t)grp * kv_stride * D);
    const char *Vp = (const char *)(v + (size_t)grp * kv_stride * D);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int col = lane & 31, half = lane >> 5;
    const int qrow = q0 + wave * 32 + col;
    const int qpos = qrow + q_off;  // the query's key position
    const int wrow0 = q0 + wave * 32, wrow1 = wrow0 + 31;

    // Q fragment (B operand of Sᵀ): query qrow, d = 16·ks + 8·half + 0..7
    bf16x8 qf[KS];
    {
        const uint16_t *qr = Qp + (size_t)min(qrow, N - 1) * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = as<bf16x8>(*(const u32x4 *)(qr + 16 * ks));
    }

    // this lane's source offsets for its wave's direct loads of a full tile
    uint32_t ksrc[KPW], vsrc[VPW];
#pragma unroll
    for (int t = 0; t < KPW; ++t) ksrc[t] = tile_src(min(wave + NW * t, KLOADS - 1), lane, BC);
#pragma unroll
    for (int t = 0; t < VPW; ++t) vsrc[t] = tile_src(min(wave + NW * t, VLOADS - 1), lane, BC);

    // Loads 0 .. NW·⌊LOADS/NW⌋ − 1 are spread evenly over the waves; the
    // remaining LOADS % NW go to the first waves.
    auto issue = [&](const char *src, char *dst) {
        copy16_to_lds(src, dst);
    };
    auto load_tile = [&](int j, int buf) {
        const char *kb = Kp + (size_t)j * BC * D * 2, *vb = Vp + (size_t)j * BC * D * 2;
        const int rows = kv_len - j * BC;  // valid rows of this tile
        if (rows >= BC) {
#pragma unroll
            for (int t = 0; t < KLOADS / NW; ++t) issue(kb + ksrc[t], &kt[buf][1024 * (wave + NW * t)]);
#pragma unroll
            for (int t = 0; t < VLOADS / NW; ++t) issue(vb + vsrc[t], &vt[buf][1024 * (wave + NW * t)]);
            if (wave < KLOADS % NW)
                issue(kb + ksrc[KPW - 1], &kt[buf][1024 * (wave + NW * (KPW - 1))]);
            if (wave < VLOADS % NW)
                issue(vb + vsrc[VPW - 1], &vt[buf][1024 * (wave + NW * (VPW - 1))]);
        } else {  // last, partial tile: rows past the sequence repeat its last row
            for (int t = 0; t < KPW; ++t)
                if (wave + NW * t < KLOADS)
                    issue(kb + tile_src(wave + NW * t, lane, rows), &kt[buf][1024 * (wave + NW * t)]);
            for (int t = 0; t < VPW; ++t)
                if (wave + NW * t < VLOADS)
                    issue(vb + tile_src(wave + NW * t, lane, rows), &vt[buf][1024 * (wave + NW * t)]);
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    // m_ref: the running max the sums and the output are kept relative to
    float m_ref = -INFINITY, l_run = 0.f;

    // lane coordinates of the transposed V reads
    const int g = lane >> 4, e = (lane >> 2) & 3, cq = lane & 3;

    const int n_kt = min(kv_len - 1, q_off + q0 + BR - 1) / BC + 1;
    // key tiles [t_lo, t_hi) of this workgroup (a split's share, or all)
    int t_lo = 0, t_hi = n_kt;
    const int S = CHUNK ? (int)gridDim.y : 1, split = CHUNK ? (int)blockIdx.y : 0;
    if constexpr (CHUNK) {
        t_lo = (int)((long)split * n_kt / S);
        t_hi = (int)((long)(split + 1) * n_kt / S);
    }
    // the first two tiles resident
    for (int t = 0; t < 2; ++t)
        if (t_lo + t < t_hi) load_tile(t_lo + t, t);
    wait_vmcnt<0>();
    regs_ready(qf);
    __syncthreads();

    // One key tile for this wave: Sᵀ, online softmax, Oᵀ update. MASK is set
    // only for tiles that cross the wave's diagonal.
    auto tile_step = [&](const char *kb_, const char *vb_, int kt0, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
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
                const u32x4 a =
                    *(const u32x4 *)(kb_ + (kb * 32 + col) * ROWB + 16 * ((2 * ks + half) ^ bswz(col)));
                sacc[kb] = mfma32x32x16(as<bf16x8>(a), qf[ks], sacc[kb]);
            }
        // ---- mask (key > query → −inf); lane's keys: kt0 + 32kb + 8(i/4) + 4half + i%4
        if constexpr (MASK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kt0 + kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    if (key > qpos) sacc[kb][i] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        const float m_tile = half_max(mx) * scale_log2;
        const bool move = m_tile > m_ref;  // m_ref = −inf: first visible tile
        if (__builtin_amdgcn_ballot_w64(move)) {
            const float m_new = move ? m_tile : m_ref;
            float alpha = exp2_fast(m_ref - m_new);  // 1 where not moved, 0 at first
            // a split's range can begin at a diagonal tile whose keys all lie
            // after some rows of the wave: those rows have seen no key yet
            // (reference −∞ on both sides), and their empty sums stay empty
            if (CHUNK && m_new == -INFINITY) alpha = 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m_ref = m_new;
        }
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // (rows that have seen no key: every score −∞, weight 0)
                const float p = exp2_fast(fmaf(sacc[kb][i], scale_log2,
                                               CHUNK && m_ref == -INFINITY ? 0.f : -m_ref));
                sacc[kb][i] = p;
                ps += p;
            }
        l_run += ps;
        // ---- Pᵀ fragments: 16-key step mm uses S registers 8(mm%2)..+7 of block
        // mm/2 (the largest weight of a row is exactly 1: the running max
        // defines the reference)
        bf16x8 pf[4];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            u32x4 wv;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                wv[t] = pack_bf16x2(sacc[mm / 2][8 * (mm % 2) + 2 * t], sacc[mm / 2][8 * (mm % 2) + 2 * t + 1]);
            pf[mm] = as<bf16x8>(wv);
        }
        // ---- Oᵀ += Vᵀ Pᵀ; A slot t ↔ key 16mm + 8(t/4) + 4half + t%4.
        // Lane 16g + 4e + c addresses V rows 16mm + 4half + e (and + 8),
        // columns 32db + 16(g&1) + 4c .. + 3.
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                // rows 16mm + 4half + e (+ 8): swizzle 4e + half (+ 2)
                const int low = 2 * (g & 1) + (cq >> 1);
                const char *r0 = vb_ + (16 * mm + 4 * half + e) * ROWB + 64 * (db ^ e) + 8 * (cq & 1);
                const char *p1 = r0 + 16 * (low ^ half);
                const char *p2 = r0 + 8 * ROWB + 16 * (low ^ (half + 2));
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p1);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p2);
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
                oacc[db] = mfma32x32x16(as<bf16x8>(a), pf[mm], oacc[db]);
            }
        }
    };

    // Bulk: the key tiles before the workgroup's first row are wholly visible
    // to every wave. They get a loop of their own with a single unmasked step,
    // so the output registers stay put (where masked, unmasked and skipped
    // tiles meet in one loop, the compiler copies all 64 of them back and
    // forth every tile).
    // (in a ragged last query tile the waves past the last query run the
    // bulk tiles too; their rows are never written)
    const int n_bulk = (q_off + q0 + 1) / BC;
    // Bulk tiles two at a time, one barrier per pair: the next pair's copies
    // go into the two buffers the last barrier freed while this pair is
    // computed (ring of 4).
    int j = t_lo;
    const int bulk_end = min(n_bulk, t_hi);
    for (; j + 1 < bulk_end; j += 2) {
        if (j + 2 < t_hi) load_tile(j + 2, (j + 2 - t_lo) & 3);
        if (j + 3 < t_hi) load_tile(j + 3, (j + 3 - t_lo) & 3);
        tile_step(kt[(j - t_lo) & 3], vt[(j - t_lo) & 3], j * BC, std::false_type{});
        tile_step(kt[(j + 1 - t_lo) & 3], vt[(j + 1 - t_lo) & 3], (j + 1) * BC, std::false_type{});
        wait_vmcnt<0>();
        __syncthreads();
    }
    // The rest (a last bulk tile, then the tiles around the diagonal,
    // classified per wave), one per barrier: tiles j and j + 1 are resident
    // or in flight on entry; tile j + 2 is fetched two steps ahead.
    for (; j < t_hi; ++j) {
        const int cur = (j - t_lo) & 3;
        const bool ahead = j + 2 < t_hi;
        if (ahead) load_tile(j + 2, (j + 2 - t_lo) & 3);
        const int kt0 = j * BC;
        if (j < n_bulk)
            tile_step(kt[cur], vt[cur], kt0, std::false_type{});
        else if (wrow0 < N && kt0 + BC - 1 <= wrow0 + q_off)  // wholly visible to the wave
            tile_step(kt[cur], vt[cur], kt0, std::false_type{});
        else if (wrow0 < N && kt0 <= wrow1 + q_off)      // crosses the wave's diagonal
            tile_step(kt[cur], vt[cur], kt0, std::true_type{});
        // tile j + 1 resident before the barrier; tile j + 2 may stay in flight
        if (ahead) wait_vmcnt<LOADS_MIN>(); else wait_vmcnt<0>();
        __syncthreads();
    }

    // ---- epilogue: O = Oᵀ/ℓ, one rounding; LSE (natural log) from the fp32 sum
    const float l_tot = half_sum(l_run);
    if (CHUNK && S > 1) {
        // partial of this key range: Õ relative to m_ref (rows that saw no
        // key here: m = −∞, sums and Õ zero), merged through the LSE later
        if (qrow < N) {
            const size_t slot = ((size_t)bhq * N + qrow) * S + split;
            float *prow = ws_part + slot * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    const f32x4 w4 = {oacc[db][4 * gg], oacc[db][4 * gg + 1], oacc[db][4 * gg + 2],
                                      oacc[db][4 * gg + 3]};
                    __builtin_nontemporal_store(w4, (f32x4 *)(prow + db * 32 + 8 * gg + 4 * half));
                }
            if (half == 0)
                *(float4 *)(ws_ml + 4 * slot) = make_float4(m_ref, l_tot, l_tot, 0.f);
        }
        return;
    }
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
        if (half == 0) lse[(size_t)bhq * N + qrow] = (m_ref + log2_fast(l_tot)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill_bf16_d128(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int B, int Hq, int Hkv, int N, float scale,
                                    hipStream_t st)
{
    const int n_qtiles = (N + BR - 1) / BR;
    const dim3 grid((unsigned)(n_qtiles * B * Hq)), block(64 * NW);
    prefill_d128_kernel<false><<<grid, block, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, lse, Hq,
        Hkv, N, n_qtiles, scale * kLog2e, N, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

// Key splits of a chunked prefill: one unless the query tiles alone leave
// CUs idle (fewer than 256 workgroups); then as many as fit one round of
// 256 workgroups (one per CU), each keeping at least 8 key tiles of the
// longest cache. (One round measured best: for 64 query tiles against a
// 32K cache, 4 splits 260.5 µs against 279.8 for 8, 324.9 for 6, 297.4
// for 12 and 321.0 for 16.)
int prefill_chunked_splits(int B, int Hq, int Nq, int kv_cap)
{
    const long items = (long)B * Hq * ((Nq + BR - 1) / BR);
    if (items >= 256) return 1;
    const long tiles = (kv_cap + BC - 1) / BC;
    long s = 256 / items;
    s = s < tiles / 8 ? s : tiles / 8;
    s = s < kMaxSplits ? s : kMaxSplits;
    return s < 1 ? 1 : (int)s;
}

size_t prefill_chunked_workspace_bytes(int B, int Hq, int Nq, int kv_cap)
{
    const int S = prefill_chunked_splits(B, Hq, Nq, kv_cap);
    if (S == 1) return 256;
    const size_t slots = (size_t)B * Hq * Nq * S;
    return align_up(16 * slots, 256) + align_up(sizeof(float) * D * slots, 256);
}

hipError_t launch_prefill_chunked_d128(const void *q, const void *k, const void *v, void *o,
                                       float *lse, const int *kv_lens, int B, int Hq, int Hkv,
                                       int Nq, int kv_cap, float scale, void *ws, hipStream_t st)
{
    const int n_qtiles = (Nq + BR - 1) / BR;
    const int S = prefill_chunked_splits(B, Hq, Nq, kv_cap);
    const size_t slots = (size_t)B * Hq * Nq * S;
    float *ws_ml = (float *)ws, *ws_part = (float *)((char *)ws + align_up(16 * slots, 256));
    const dim3 grid((unsigned)(n_qtiles * B * Hq), (unsigned)S), block(64 * NW);
    prefill_d128_kernel<true><<<grid, block, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, lse, Hq,
        Hkv, Nq, n_qtiles, scale * kLog2e, kv_cap, kv_lens, ws_ml, ws_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    return launch_merge(ws_ml, ws_part, o, lse, B * Hq * Nq, S, D, st);
}

}  // namespace attn
