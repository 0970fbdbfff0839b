// Balanced work split of a ragged decode batch (device side).
//
// Sequence b of a batch holds L_b = clamp(kv_lens[b], 0, max_len) keys, cut
// into n_b = ⌈L_b / tile⌉ tiles. Taking the tiles of all sequences in batch
// order (T in total), P_eff = min(P, T) workers receive equal contiguous
// runs: worker w takes tiles [⌈w·T/P_eff⌉, ⌈(w+1)·T/P_eff⌉), at least one
// each, so the work is balanced whatever the length mix. Tile t belongs to
// worker ⌊t·P_eff/T⌋. Worker w writes its partial result for sequence b to
// slot w + b: runs and sequences are both increasing in tile order, so two
// overlapping (worker, sequence) pairs never share a slot, and the slots of
// one sequence are consecutive. The lengths are read on the device, so the
// split follows whatever lengths the array holds when the kernel runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

__device__ __forceinline__ int ragged_len(const int *kv_lens, int b, int max_len) {
    return min(max(kv_lens[b], 0), max_len);
}

// Total tiles of the batch; every lane of the wave returns it.
__device__ __forceinline__ int ragged_total(const int *kv_lens, int B, int max_len, int tile) {
    const int lane = __lane_id();
    int T = 0;
    for (int c = 0; c < B; c += 64) {
        int n = c + lane < B ? (ragged_len(kv_lens, c + lane, max_len) + tile - 1) / tile : 0;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m);
        T += n;
    }
    return __builtin_amdgcn_readfirstlane(T);  // wave-uniform: keep it in a scalar register
}

// The sequence holding tile t (0 <= t < T) and the index of its first tile
// (the tiles of sequences 0 .. b−1); every lane of the wave returns them.
__device__ __forceinline__ void ragged_locate(const int *kv_lens, int B, int max_len, int tile,
                                              int t, int &b_out, int &first_out) {
    const int lane = __lane_id();
    int base = 0;
    for (int c = 0; c < B; c += 64) {
        const int n = c + lane < B ? (ragged_len(kv_lens, c + lane, max_len) + tile - 1) / tile : 0;
        int incl = n;  // inclusive prefix sum over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        const uint64_t hit = __ballot(base + incl > t);
        if (hit) {
            const int l = __ffsll((unsigned long long)hit) - 1;
            b_out = __builtin_amdgcn_readfirstlane(c + l);
            first_out = __builtin_amdgcn_readfirstlane(base + __shfl(incl - n, l));
            return;
        }
        base += __shfl(incl, 63);
    }
    b_out = B;
    first_out = __builtin_amdgcn_readfirstlane(base);
}

// First tile of worker w's run (P_eff workers over T tiles).
__device__ __forceinline__ int ragged_run_begin(int w, int T, int P_eff) {
    return (int)(((int64_t)w * T + P_eff - 1) / P_eff);
}

// Worker owning tile t.
__device__ __forceinline__ int ragged_owner(int t, int T, int P_eff) {
    return (int)((int64_t)t * P_eff / T);
}

// Piece j of the balanced split: the overlap of worker w's run with
// sequence b where w + b = j. The pieces of worker w take the consecutive
// slots w + b_first(w) .. w + b_last(w) (the sequences its run touches), so
// the worker owning slot j is the last one whose first slot is <= j, found
// by bisection; a slot between two workers' ranges holds no piece.
// Returns false if slot j holds no piece; else the sequence, its length and
// the piece's tiles [t0, t1) counted from the sequence's first tile.
__device__ __forceinline__ bool ragged_piece(const int *kv_lens, int B, int max_len, int tile,
                                             int workers, int j, int &b, int &len, int &t0,
                                             int &t1) {
    if (B <= 64) {
        // the whole batch fits one wave: lane l holds sequence l's tile
        // count and inclusive prefix sum, and every lookup is a ballot
        const int lane = __lane_id();
        const int n_l = lane < B ? (ragged_len(kv_lens, lane, max_len) + tile - 1) / tile : 0;
        int incl = n_l;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        const int T = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        if (T == 0) return false;
        const int P = min(workers, T);
        auto seq_of = [&](int t) {  // sequence holding tile t
            return __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)__ballot(incl > t)) - 1);
        };
        int lo = 0, hi = P - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (mid + seq_of(ragged_run_begin(mid, T, P)) <= j) lo = mid; else hi = mid - 1;
        }
        const int w = lo, r0 = ragged_run_begin(w, T, P), r1 = ragged_run_begin(w + 1, T, P);
        b = j - w;
        if (b > seq_of(r1 - 1) || b < seq_of(r0)) return false;
        const int first = __builtin_amdgcn_readfirstlane(__shfl(incl - n_l, b));
        const int n = __builtin_amdgcn_readfirstlane(__shfl(n_l, b));
        len = ragged_len(kv_lens, b, max_len);
        t0 = max(r0, first) - first;
        t1 = min(r1, first + n) - first;
        return t0 < t1;
    }
    const int T = ragged_total(kv_lens, B, max_len, tile);
    if (T == 0) return false;
    const int P = min(workers, T);
    int lo = 0, hi = P - 1, bl, fl;
    while (lo < hi) {  // last w with w + b_first(w) <= j
        const int mid = (lo + hi + 1) / 2;
        ragged_locate(kv_lens, B, max_len, tile, ragged_run_begin(mid, T, P), bl, fl);
        if (mid + bl <= j) lo = mid; else hi = mid - 1;
    }
    const int w = lo, r0 = ragged_run_begin(w, T, P), r1 = ragged_run_begin(w + 1, T, P);
    int b_last, f_last;
    ragged_locate(kv_lens, B, max_len, tile, r1 - 1, b_last, f_last);
    b = j - w;
    if (b > b_last) return false;
    int f_first;
    ragged_locate(kv_lens, B, max_len, tile, r0, bl, f_first);
    if (b < bl) return false;
    // first tile of sequence b: walk from the run's first sequence (few steps)
    int first = f_first;
    for (int s = bl; s < b; ++s) first += (ragged_len(kv_lens, s, max_len) + tile - 1) / tile;
    len = ragged_len(kv_lens, b, max_len);
    const int n = (len + tile - 1) / tile;
    t0 = max(r0, first) - first;
    t1 = min(r1, first + n) - first;
    return t0 < t1;
}

}  // namespace attn
