// fp16 forward instances with equal head dims (plain and JVP, 4 and 8 waves).
#include "attn_instances.h"

namespace attn {
KernelChoice fwd_fp16(int D, bool jvp, bool split) { return choose16<true>(D, jvp, split); }
}  // namespace attn
