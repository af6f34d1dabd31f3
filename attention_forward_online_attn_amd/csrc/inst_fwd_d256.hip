// Head dim 256, forward without tangents (dense, causal, jagged, and with a
// bias or mask): 32-key tiles and one wave per SIMD, so that the 256-column
// accumulator (128 registers per lane) and the Q fragments fit; bf16, fp16
// and fp32.
#include "../../include/attn.h"
#include "attn_instances.h"

namespace attn {
KernelChoice fwd_d256(int dtype) {
  if (dtype == ATTN_BF16) return r32<256, 32, false, 4, false>();
  if (dtype == ATTN_FP16) return r32<256, 32, false, 4, true>();
  return f32k<256, false>();
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
