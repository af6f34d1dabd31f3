// Backward instances without a score operand (prep, dQ and dK/dV kernels;
// bf16 and fp16; dense and jagged) and their launches.
#include "attn_bwd_launch.h"

namespace attn {

int bwd_run(bool f16, int D, int bias_kind, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
            int64_t items) {
  int rc = by_dim_bwd(D, [&](auto d) {
    constexpr int Dc = decltype(d)::value;
    constexpr int rpb = 256 / (Dc / 8);
    const int grid = (int)((B * H * Nq + rpb - 1) / rpb);
    return f16 ? bwd_launch_one(attn_bwd_prep_kernel<Dc, true>, grid, 256, 0, st, a)
               : bwd_launch_one(attn_bwd_prep_kernel<Dc, false>, grid, 256, 0, st, a);
  });
  if (rc) return rc;
  if (D == 256) return bwd_run_d256(f16, bias_kind, st, a, B, H, Nq, Nkv, items);
  if (bias_kind != kNoBias) return bwd_run_bias(f16, D, bias_kind, st, a, B, H, Nq, Nkv);
  return by_dim_qk(D, [&](auto d) {
    constexpr int Dc = decltype(d)::value;
    return f16 ? bwd_launch_grads<Dc, true, kNoBias>(st, a, B, H, Nq, Nkv, items)
               : bwd_launch_grads<Dc, false, kNoBias>(st, a, B, H, Nq, Nkv, items);
  });
}

}  // namespace attn
