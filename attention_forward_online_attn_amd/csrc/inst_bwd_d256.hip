// Backward gradient instances at head dim 256 (bf16 and fp16; no operand,
// additive bias or boolean mask; dense and jagged).  The dQ kernel runs one
// wave per SIMD; dK and dV come from two launches of the dK/dV kernel (K and
// dV, then K, V and dK), since K, V and both accumulators exceed one wave's
// registers.  The prep kernel is enqueued by bwd_run (inst_bwd.hip).
#include "attn_bwd_launch.h"

namespace attn {

int bwd_run_d256(bool f16, int bias_kind, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
                 int64_t items) {
  if (bias_kind == kAddBias)
    return f16 ? bwd_launch_grads<256, true, kAddBias>(st, a, B, H, Nq, Nkv, items)
               : bwd_launch_grads<256, false, kAddBias>(st, a, B, H, Nq, Nkv, items);
  if (bias_kind == kMaskBias)
    return f16 ? bwd_launch_grads<256, true, kMaskBias>(st, a, B, H, Nq, Nkv, items)
               : bwd_launch_grads<256, false, kMaskBias>(st, a, B, H, Nq, Nkv, items);
  return f16 ? bwd_launch_grads<256, true, kNoBias>(st, a, B, H, Nq, Nkv, items)
             : bwd_launch_grads<256, false, kNoBias>(st, a, B, H, Nq, Nkv, items);
}

}  // namespace attn
