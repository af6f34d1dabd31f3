// Head dim 256, plain forward only (dense, causal, jagged): 32-key tiles and
// one wave per SIMD, so that the 256-column accumulator (128 registers per
// lane) and the Q fragments fit; bf16, fp16 and fp32.
#include "../../include/attn.h"
#include "attn_instances.h"

namespace attn {
KernelChoice fwd_d256(int dtype) {
  if (dtype == ATTN_BF16) return r32<256, 32, false, 4, false>();
  if (dtype == ATTN_FP16) return r32<256, 32, false, 4, true>();
  return f32k<256, false>();
}
}  // namespace attn
