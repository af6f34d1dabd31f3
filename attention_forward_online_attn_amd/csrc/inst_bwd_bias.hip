// Backward instances with an additive bias or a boolean mask (dense; bf16
// and fp16): the kernels recompute P with the operand, and the dQ kernel
// writes the bias gradient dS when asked.  The prep kernel is shared with
// the unbiased backward (inst_bwd.hip), which enqueues it first.
#include "attn_bwd_launch.h"

namespace attn {

int bwd_run_bias(bool f16, int D, int bias_kind, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq,
                 int64_t Nkv) {
  return by_dim_qk(D, [&](auto d) {
    constexpr int Dc = decltype(d)::value;
    if (bias_kind == kAddBias)
      return f16 ? bwd_launch_grads<Dc, true, kAddBias>(st, a, B, H, Nq, Nkv, 0)
                 : bwd_launch_grads<Dc, false, kAddBias>(st, a, B, H, Nq, Nkv, 0);
    return f16 ? bwd_launch_grads<Dc, true, kMaskBias>(st, a, B, H, Nq, Nkv, 0)
               : bwd_launch_grads<Dc, false, kMaskBias>(st, a, B, H, Nq, Nkv, 0);
  });
}

}  // namespace attn
