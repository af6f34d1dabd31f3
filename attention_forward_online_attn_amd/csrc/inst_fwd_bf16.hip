// bf16 forward instances with equal head dims (plain and JVP, 4 and 8 waves).
#include "attn_instances.h"

namespace attn {
KernelChoice fwd_bf16(int D, bool jvp, bool split) { return choose16<false>(D, jvp, split); }
}  // namespace attn
