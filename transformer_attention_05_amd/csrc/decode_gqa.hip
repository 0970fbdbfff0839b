// GQA decode: the split plan, the launcher (split kernel, then the merge),
// and the bf16-cache instantiation of the kernel in decode_gqa_kernel.h,
// whose comment describes the design. The E4M3 instantiation is compiled
// in decode_gqa_fp8.hip: this unit is built with LLVM's max-ILP machine
// scheduler and that one with the default (build.py gives the measurements).
#include "decode_gqa_kernel.h"

namespace attn {
namespace {

// Workgroups per launch the split aims at: one per CU, for a bf16 and for
// an E4M3 cache (both measured best of 256 / 512 / 1024 once the next
// chunk's loads stay in flight during compute).
constexpr long kTargetGroups = 256;
// Ragged batches: the host knows only the longest length, and a split sized
// for it leaves the shorter sequences' workgroups idle. Their keys are cut
// into pieces of at most this many keys (the uniform split when that is
// finer), so many short workgroups are dealt out as CUs free up. Measured on
// 32 sequences of 263–7764 keys (8 K/V heads): one split per (b, K/V head)
// 117.2 µs; pieces of 768 keys (11 splits) 103.2 µs, of 512 keys 107.4 µs,
// of about 1000 keys 113.6 µs, of about 320 keys 112.9 µs.
constexpr int kRaggedSplitKeys = 768;

}  // namespace

bool gqa_plan(int B, int Hq, int Hkv, int kv_len, GqaPlan *p, bool fp8, bool ragged)
{
    if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || kv_len < 1) return false;
    const int G = Hq / Hkv;
    if (G > 16) return false;
    const long groups = (long)B * Hkv;
    const int chunks = (kv_len + kChunk - 1) / kChunk;
    int want = (int)((kTargetGroups + groups - 1) / groups);
    if (ragged) want = max(want, (kv_len + kRaggedSplitKeys - 1) / kRaggedSplitKeys);
    int s = want < 1 ? 1 : (want < chunks ? want : chunks);
    if (s > kMaxSplits) s = kMaxSplits;
    const int per = (chunks + s - 1) / s;
    s = (chunks + per - 1) / per;
    p->splits = s;
    p->split_keys = per * kChunk;
    const size_t rows = (size_t)B * Hq;
    p->ws_ml = 0;
    p->ws_part = align_up(sizeof(float) * 4 * rows * s, 256);
    p->ws_total = s == 1 ? 256 : p->ws_part + align_up(sizeof(float) * kD * rows * s, 256);
    return true;
}

hipError_t launch_decode_gqa(const GqaPlan &p, const void *q, const void *k, const void *v,
                             void *o, float *lse, int B, int Hq, int Hkv, int kv_len,
                             int kv_cap, float scale, void *ws, hipStream_t st,
                             const int *kv_lens, bool fp8)
{
    // a group's splits, and its merge rows, on one XCD (group count a multiple of 8)
    const int xcd = (B * Hkv) % 8 == 0;
    // non-temporal loads throughout (ragged batch in 512-key pieces: 113.3 µs
    // with the default policy, 107.4 with the hint)
    const hipError_t e =
        fp8 ? launch_decode_gqa_split_fp8(p, q, k, v, o, lse, B, Hq, Hkv, kv_len, kv_cap, scale,
                                          ws, st, kv_lens, xcd)
            : launch_gqa_split<false>(p, q, k, v, o, lse, B, Hq, Hkv, kv_len, kv_cap, scale, ws,
                                      st, kv_lens, xcd);
    if (e != hipSuccess || p.splits == 1) return e;
    char *w = (char *)ws;
    return launch_merge((const float *)(w + p.ws_ml), (const float *)(w + p.ws_part), o, lse,
                        B * Hq, p.splits, kD, st, xcd ? Hq / Hkv : 0);
}

}  // namespace attn
