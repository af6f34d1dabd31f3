// Backward instances (prep, dQ and dK/dV kernels; bf16 and fp16) and their
// launches.
#include "../../include/attn.h"
#include "attn_bwd_bf16.h"
#include "attn_dispatch.h"

namespace attn {
namespace {

template <class F>
int launch_fn(F* fn, int grid, int threads, int lds, hipStream_t stream, const BwdArgs& a) {
  if (grid <= 0) return ATTN_OK;
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return ATTN_ERR_HIP;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, stream, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <int D, bool F16>
int bwd_launch(hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t items) {
  const int64_t rows = B * H * Nq;
  constexpr int rpb = 256 / (D / 8);
  int rc = launch_fn(attn_bwd_prep_kernel<D, F16>, (int)((rows + rpb - 1) / rpb), 256, 0, st, a);
  if (rc) return rc;
  using Cq = BwdDqCfg<D, kBnBwdDq>;
  using Ck = BwdDkdvCfg<D>;
  static_assert(Cq::BM == 128 && Ck::BN == 128, "the jagged plan's tiles are 128 rows");
  a.n_tiles = (int)((Nq + Cq::BM - 1) / Cq::BM);
  const int64_t gq = a.offsets ? items * H : B * H * a.n_tiles;
  rc = launch_fn(attn_bwd_dq_kernel<D, kBnBwdDq, F16>, (int)gq, Cq::THREADS, Cq::LDS, st, a);
  if (rc) return rc;
  a.n_tiles = (int)((Nkv + Ck::BN - 1) / Ck::BN);
  const int64_t gk = a.offsets ? items * H : B * H * a.n_tiles;
  return launch_fn(attn_bwd_dkdv_kernel<D, F16>, (int)gk, Ck::THREADS, Ck::LDS, st, a);
}

}  // namespace

int bwd_run(bool f16, int D, hipStream_t st, BwdArgs& a, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
            int64_t items) {
  return by_dim(D, [&](auto d) {
    constexpr int Dc = decltype(d)::value;
    return f16 ? bwd_launch<Dc, true>(st, a, B, H, Nq, Nkv, items) : bwd_launch<Dc, false>(st, a, B, H, Nq, Nkv, items);
  });
}

}  // namespace attn
