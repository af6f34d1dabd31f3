// Backward instances without a score operand (prep, dQ and dK/dV kernels;
// bf16 and fp16; dense and jagged) and their launches.
#include <climits>

#include "attn_bwd_launch.h"

namespace attn {

int bwd_run(bool f16, int D, int bias_kind, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
            int64_t items) {
  // Every grid of the backward fits an int, checked before anything is
  // enqueued: the prep kernel's (256 / (D / 8) rows per block: 8 at D = 256)
  // and the gradient kernels' (B H ceil(N / 128) tiles, or items H when
  // jagged).  B H and N are each at most INT_MAX, so no product overflows.
  const int64_t rpb = 256 / (D / 8);
  const int64_t prep_grid = (B * H * Nq + rpb - 1) / rpb;
  const int64_t grid_q = a.offsets ? items * H : B * H * ((Nq + 127) / 128);
  const int64_t grid_k = a.offsets ? items * H : B * H * ((Nkv + 127) / 128);
  if (prep_grid > INT_MAX || grid_q > INT_MAX || grid_k > INT_MAX) return ATTN_ERR_INVALID;
  int rc = by_dim_bwd(D, [&](auto d) {
    constexpr int Dc = decltype(d)::value;
    static_assert(256 / (Dc / 8) >= 8, "prep rows per block");
    const int grid = (int)prep_grid;
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
