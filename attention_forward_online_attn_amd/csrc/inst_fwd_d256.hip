// Head dim 256 (dense, causal, jagged, and with a bias or mask): one wave
// per SIMD, so that the 256-column accumulator (128 registers per lane) and
// the Q fragments fit; bf16, fp16 and fp32.  The plain 16-bit forward
// streams 64-key tiles (two stages take 128 KB of LDS in the split K-side /
// V-side layout; half the barriers per key of 32-key tiles, 4-11% faster);
// with a bias or mask the 64-key instance would spill, so it keeps 32.  The
// 16-bit JVP takes at most 64 value columns per launch (the caller runs it
// once per slice): three accumulators over 128 columns spilled inside the
// key loop beside the Q and tQ fragments.  Narrower value head dims (16 to
// 128; JVP page: _attention.forward takes d_v != d_qk) have instances of their own: the
// 16-bit ones on 64-key tiles (JVP: 32), one wave per SIMD for the 256-wide
// Q fragments, and the fp32 ones, whose JVP also carries 128-wide halves of
// 256-wide values.
#include "../../include/attn.h"
#include "attn_instances.h"

namespace attn {
KernelChoice fwd_d256(int dtype) {
  if (dtype == ATTN_BF16) return r32<256, 64, false, 4, false>();
  if (dtype == ATTN_FP16) return r32<256, 64, false, 4, true>();
  return f32k<256, false>();
}

KernelChoice fwd_d256_dv(int dtype, int Dv, bool jvp) {
  return by_dim_qk(Dv, [&](auto dv) {
    constexpr int V = decltype(dv)::value;
    if (dtype == ATTN_FP32) return jvp ? f32k<256, true, kNoBias, V>() : f32k<256, false, kNoBias, V>();
    if (jvp) {
      if constexpr (V > 64) return KernelChoice{};  // taken in 64-wide slices
      else
        return dtype == ATTN_FP16 ? r32<256, 32, true, 4, true, kNoBias, V>() : r32<256, 32, true, 4, false, kNoBias, V>();
    }
    return dtype == ATTN_FP16 ? r32<256, 64, false, 4, true, kNoBias, V>() : r32<256, 64, false, 4, false, kNoBias, V>();
  });
}

namespace {
template <int BIAS>
KernelChoice d256_bias(int dtype) {
  if (dtype == ATTN_BF16) return r32<256, 32, false, 4, false, BIAS>();
  if (dtype == ATTN_FP16) return r32<256, 32, false, 4, true, BIAS>();
  return f32k<256, false, BIAS>();
}
}  // namespace

KernelChoice fwd_d256_bias(int dtype, int kind) {
  return kind == kAddBias ? d256_bias<kAddBias>(dtype) : d256_bias<kMaskBias>(dtype);
}
}  // namespace attn
