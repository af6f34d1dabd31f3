// Instance builders for the forward kernels, included by the inst_*.hip
// translation units only.
#pragma once

#include "attn_dispatch.h"
#include "attn_fwd_bf16.h"
#include "attn_fwd_f32.h"

namespace attn {

template <int D, int BN, bool JVP, int NW = 4, bool F16 = false, int BIAS = kNoBias, int DV = 0>
KernelChoice r32() {
  using C = Bf16Cfg<D, BN, JVP, NW, DV>;
  return {attn_fwd_bf16_kernel<D, BN, JVP, NW, F16, BIAS, DV>, C::BM, BN, C::LDS, C::THREADS};
}

template <int D, bool JVP, int BIAS = kNoBias, int DV = 0>
KernelChoice f32k() {
  using C = F32Cfg<D, JVP, DV>;
  return {attn_fwd_f32_kernel<D, JVP, BIAS, DV>, C::BM, C::BN, C::LDS, 256};
}

// 16-bit forward with equal head dims; `split`: 8-wave workgroups whose two
// halves split a query tile's key range.  The JVP at 128 has no instance
// here: it runs as two launches of the (128, 64) value-dim instance over the
// halves of the value columns.
template <bool F16>
KernelChoice choose16(int D, bool jvp, bool split) {
  return by_dim(D, [&](auto d) {
    constexpr int Dc = decltype(d)::value;
    if constexpr (Dc == 128) {
      if (jvp) return KernelChoice{};
      return split ? r32<Dc, kBnDense, false, 8, F16>() : r32<Dc, kBnDense, false, 4, F16>();
    } else {
      if (split) return !jvp ? r32<Dc, kBnDense, false, 8, F16>() : r32<Dc, kBnJvp, true, 8, F16>();
      return !jvp ? r32<Dc, kBnDense, false, 4, F16>() : r32<Dc, kBnJvp, true, 4, F16>();
    }
  });
}

// 16-bit forward whose value head dim differs from the query/key one (JVP
// page: d_v != d_qk): 4-wave workgroups, never split, no bias.
template <bool F16>
KernelChoice choose_mixed16(int D, int Dv, bool jvp) {
  return by_dim_qk(D, [&](auto dq) {
    return by_dim_qk(Dv, [&](auto dv) {
      constexpr int A = decltype(dq)::value, V = decltype(dv)::value;
      // equal dims other than 16 take choose16 (no instance twice in the library)
      if constexpr (A == V && A != 16) {
        return KernelChoice{};
      } else if constexpr (V == 128) {  // the JVP with 128 value columns runs as two (A, 64) halves
        return jvp ? KernelChoice{} : r32<A, kBnDense, false, 4, F16, kNoBias, V>();
      } else {
        return jvp ? r32<A, kBnJvp, true, 4, F16, kNoBias, V>() : r32<A, kBnDense, false, 4, F16, kNoBias, V>();
      }
    });
  });
}

}  // namespace attn
