// Forward instances with an additive bias or a boolean mask (no JVP, never
// split): one per dtype, head dim and kind.
#include "../../include/attn.h"
#include "attn_instances.h"

namespace attn {
namespace {
template <int BIAS>
KernelChoice pick(int dtype, int D) {
  return by_dim_qk(D, [&](auto d) {
    constexpr int Dc = decltype(d)::value;
    if (dtype == ATTN_BF16) return r32<Dc, kBnDense, false, 4, false, BIAS>();
    if (dtype == ATTN_FP16) return r32<Dc, kBnDense, false, 4, true, BIAS>();
    return f32k<Dc, false, BIAS>();
  });
}
}  // namespace

KernelChoice fwd_bias(int dtype, int kind, int D) {
  return kind == kAddBias ? pick<kAddBias>(dtype, D) : pick<kMaskBias>(dtype, D);
}
}  // namespace attn
