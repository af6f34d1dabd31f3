// Launch sequence of the backward (prep, dQ, dK/dV kernels), included by the
// backward instance translation units.
#pragma once

#include "../../include/attn.h"
#include "attn_bwd_bf16.h"
#include "attn_dispatch.h"

namespace attn {

template <class F>
int bwd_launch_one(F* fn, int grid, int threads, int lds, hipStream_t stream, const BwdArgs& a) {
  if (grid <= 0) return ATTN_OK;
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return ATTN_ERR_HIP;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, stream, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// The dQ and dK/dV kernels (after the prep kernel, which bwd_run enqueues).
template <int D, bool F16, int BIAS>
int bwd_launch_grads(hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t items) {
  int rc = ATTN_OK;
  using Cq = BwdDqCfg<D, kBnBwdDq>;
  using Ck = BwdDkdvCfg<D, BIAS>;
  static_assert(Cq::BM == 128 && Ck::BN == 128, "the jagged plan's tiles are 128 rows");
  a.n_tiles = (int)((Nq + Cq::BM - 1) / Cq::BM);
  const int64_t gq = a.offsets ? items * H : B * H * a.n_tiles;
  rc = bwd_launch_one(attn_bwd_dq_kernel<D, kBnBwdDq, F16, BIAS>, (int)gq, Cq::THREADS, Cq::LDS, st, a);
  if (rc) return rc;
  a.n_tiles = (int)((Nkv + Ck::BN - 1) / Ck::BN);
  const int64_t gk = a.offsets ? items * H : B * H * a.n_tiles;
  if constexpr (D == 256) {  // dV, then dK: the two do not fit one wave's registers together
    rc = bwd_launch_one(attn_bwd_dkdv_kernel<D, F16, BIAS, kDkdvOnlyV>, (int)gk, Ck::THREADS, Ck::LDS, st, a);
    if (rc) return rc;
    return bwd_launch_one(attn_bwd_dkdv_kernel<D, F16, BIAS, kDkdvOnlyK>, (int)gk, Ck::THREADS, Ck::LDS, st, a);
  } else {
    return bwd_launch_one(attn_bwd_dkdv_kernel<D, F16, BIAS>, (int)gk, Ck::THREADS, Ck::LDS, st, a);
  }
}

}  // namespace attn
