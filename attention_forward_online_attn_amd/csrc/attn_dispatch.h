// Kernel selection shared by the host code (attn_abi.hip) and the
// translation units that instantiate the kernels (inst_*.hip): every
// instance table below is compiled in a source file of its own, so the
// library builds in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"

namespace attn {

// Tile shapes of the 16-bit kernels (query tile 128 rows = 4 waves x 32).
constexpr int kBnDense = 64;  // keys per tile, plain forward
constexpr int kBnJvp = 32;    // keys per tile, JVP (four streamed tensors)
constexpr int kBnBwdDq = 32;  // keys per tile of the backward's dQ kernel

// One compiled forward kernel with its tile shape.
struct KernelChoice {
  void (*fn)(FwdArgs);
  int BM;       // query rows per workgroup
  int BN;       // keys per tile
  int lds;      // dynamic LDS bytes
  int threads;  // workgroup size
};

// Calls f(std::integral_constant<int, D>) for a supported head dim (checked
// before: 32, 64 or 128).
template <class F>
auto by_dim(int64_t D, F&& f) {
  if (D == 32) return f(std::integral_constant<int, 32>{});
  if (D == 64) return f(std::integral_constant<int, 64>{});
  return f(std::integral_constant<int, 128>{});
}

// Head dims that also take 16: the value-dim variants (the JVP page's
// cross-attention test pairs d_qk = 16 with d_v = 32; a 16-wide value tile
// is padded to 32 in LDS), the biased forward and the backward (whose
// gradient kernels run a 16-wide head on the 32-wide tiles).
template <class F>
auto by_dim_qk(int64_t D, F&& f) {
  if (D == 16) return f(std::integral_constant<int, 16>{});
  return by_dim(D, f);
}

// Head dims of the backward's prep kernel: those of by_dim_qk and 256 (whose
// gradient kernels live in inst_bwd_d256.hip).
template <class F>
auto by_dim_bwd(int64_t D, F&& f) {
  if (D == 256) return f(std::integral_constant<int, 256>{});
  return by_dim_qk(D, f);
}

// Forward instance tables (dtype codes of include/attn.h).
KernelChoice fwd_bf16(int D, bool jvp, bool split);             // inst_fwd_bf16.hip
KernelChoice fwd_fp16(int D, bool jvp, bool split);             // inst_fwd_fp16.hip
KernelChoice fwd_f32(int D, int Dv, bool jvp);                  // inst_fwd_f32.hip
KernelChoice fwd_bias(int dtype, int kind, int D);              // inst_fwd_bias.hip
KernelChoice fwd_mixed_bf16(int D, int Dv, bool jvp);           // inst_fwd_mixed_bf16.hip
KernelChoice fwd_mixed_fp16(int D, int Dv, bool jvp);           // inst_fwd_mixed_fp16.hip
KernelChoice fwd_d256(int dtype);                               // inst_fwd_d256.hip (values 256 wide)
KernelChoice fwd_d256_dv(int dtype, int Dv, bool jvp);          // inst_fwd_d256.hip (values 16 to 128 wide)
KernelChoice fwd_d256_bias(int dtype, int kind);                // inst_fwd_d256.hip (bias or mask)

// Backward: enqueues the prep, dQ and dK/dV kernels (inst_bwd.hip).  Dense:
// B*H*Nq rows, grids over (batch, head, tile).  Jagged (a.offsets set): the
// prep kernel sees H*total_len rows as one batch and both gradient kernels
// cover `items` plan items per head.  With a bias kind (dense only) it hands
// the gradient kernels over to the biased instances (bwd_run_bias,
// inst_bwd_bias.hip).
int bwd_run(bool f16, int D, int bias_kind, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
            int64_t items);
int bwd_run_bias(bool f16, int D, int bias_kind, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq,
                 int64_t Nkv);
// The gradient kernels at head dim 256, any score operand (inst_bwd_d256.hip).
int bwd_run_d256(bool f16, int bias_kind, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
                 int64_t items);

}  // namespace attn
