// fp32 forward instances (plain and JVP; any pair of query/key and value head dims).
#include "attn_instances.h"

namespace attn {
KernelChoice fwd_f32(int D, int Dv, bool jvp) {
  return by_dim_qk(D, [&](auto dq) {
    return by_dim_qk(Dv, [&](auto dv) {
      constexpr int A = decltype(dq)::value, V = decltype(dv)::value, DVp = A == V ? 0 : V;
      return jvp ? f32k<A, true, kNoBias, DVp>() : f32k<A, false, kNoBias, DVp>();
    });
  });
}
}  // namespace attn
