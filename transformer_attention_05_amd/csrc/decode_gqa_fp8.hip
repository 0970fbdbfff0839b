// GQA decode over an FP8 E4M3 cache: the E4M3 instantiation of the kernel
// in decode_gqa_kernel.h, in a translation unit of its own so that it keeps
// the compiler's default scheduling while the bf16 one does not (build.py).
#include "decode_gqa_kernel.h"

namespace attn {

hipError_t launch_decode_gqa_split_fp8(const GqaPlan &p, const void *q, const void *k,
                                       const void *v, void *o, float *lse, int B, int Hq,
                                       int Hkv, int kv_len, int kv_cap, float scale, void *ws,
                                       hipStream_t st, const int *kv_lens, int xcd)
{
    return launch_gqa_split<true>(p, q, k, v, o, lse, B, Hq, Hkv, kv_len, kv_cap, scale, ws, st,
                                  kv_lens, xcd);
}

}  // namespace attn
