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

}  // namespace attn
