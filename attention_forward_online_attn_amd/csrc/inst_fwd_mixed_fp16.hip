// fp16 forward instances whose value head dim differs from the query/key one.
#include "attn_instances.h"

namespace attn {
KernelChoice fwd_mixed_fp16(int D, int Dv, bool jvp) { return choose_mixed16<true>(D, Dv, jvp); }
}  // namespace attn
