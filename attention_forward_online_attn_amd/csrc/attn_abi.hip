// Host side of libattn_mi355x.so: argument validation, kernel selection and
// launches behind the C ABI of include/attn.h.  Every check runs on the host
// before anything is enqueued; launches are asynchronous on the caller's
// stream.  With ATTN_MI355X_DEBUG=1 in the environment each call also
// synchronises its stream and reports kernel errors as ATTN_ERR_HIP.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "../../include/attn.h"
#include "attn_common.h"
#include "attn_dispatch.h"
#include "jagged_plan.h"

namespace attn {
namespace {

constexpr int kPlanBmMin = 64;  // smallest query tile of any kernel (workspace bound)

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("ATTN_MI355X_DEBUG");
    return e && e[0] == '1';
  }();
  return on;
}

int finish(hipStream_t stream) {
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  if (debug_sync() && hipStreamSynchronize(stream) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b <= limit for non-negative a, b, without forming the product first
bool mul_within(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

// A stride is usable when its dimension is trivial or it keeps 16-byte rows.
bool stride_ok(int64_t stride, int64_t extent, int64_t vec) {
  if (stride < 0) return false;
  return extent <= 1 || stride % vec == 0;
}

// d16: head dim 16 is allowed (the forward, JVP and backward); d256: head
// dim 256 is allowed (the forward, the JVP and the backward).
int check_common(int dtype, int64_t D, float sm_scale, bool d16 = false, bool d256 = false) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32 && dtype != ATTN_FP16) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale) || sm_scale < 0.f) return ATTN_ERR_INVALID;
  if (D != 32 && D != 64 && D != 128 && !(d16 && D == 16) && !(d256 && D == 256))
    return D <= 0 ? ATTN_ERR_INVALID : ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// The forward kernels address the rows of a key tile (at most 128 rows) with
// 32-bit per-lane byte offsets from a uniform tile base: K and V row strides
// must keep 128 rows of 4-byte elements within 2^31 bytes.
constexpr int64_t kMaxKvRowStride = (int64_t)1 << 22;
bool kv_row_stride_ok(int64_t n_stride) { return n_stride <= kMaxKvRowStride; }

int check_s4(const attn_strides4& s, int64_t B, int64_t H, int64_t N, int64_t vec) {
  if (s.d != 1) return ATTN_ERR_INVALID;
  if (s.b < 0 || s.h < 0 || s.n < 0) return ATTN_ERR_INVALID;
  if (!stride_ok(s.b, B, vec) || !stride_ok(s.h, H, vec) || !stride_ok(s.n, N, vec)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int check_s3(const attn_strides3& s, int64_t H, int64_t T, int64_t vec) {
  if (s.d != 1) return ATTN_ERR_INVALID;
  if (s.h < 0 || s.t < 0) return ATTN_ERR_INVALID;
  if (!stride_ok(s.h, H, vec) || !stride_ok(s.t, T, vec)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Compute units of the current device (queried once per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Dense causal work on a small grid (at most four query tiles per CU) runs
// paired key-split workgroups: 8 waves take q-tiles p and n-1-p of a head in
// turn (equal work for every workgroup), and the two 4-wave groups split
// each tile's key range in halves merged at the end, so that both waves of
// a SIMD stay busy and the heaviest tiles take half as many steps.  Larger
// grids balance well enough by heaviest-first dispatch and keep 4-wave
// workgroups.  The JVP at D = 128 (two launches over the value halves) is
// never split.
bool use_split(int dtype, int D, bool jvp, bool dense_causal, int64_t grid) {
  return dtype != ATTN_FP32 && dense_causal && !(jvp && D == 128) && grid <= 4 * (int64_t)cu_count();
}

// Forward kernel for a dtype, head dims and variant (instance tables in the
// inst_*.hip translation units).
KernelChoice choose(int dtype, int D, bool jvp, bool split, int bias_kind, int Dv) {
  if (D == 256) {
    if (bias_kind != kNoBias) return fwd_d256_bias(dtype, bias_kind);
    return Dv == 256 && !jvp ? fwd_d256(dtype) : fwd_d256_dv(dtype, Dv, jvp);
  }
  if (bias_kind != kNoBias) return fwd_bias(dtype, bias_kind, D);
  if (dtype == ATTN_FP32) return fwd_f32(D, Dv, jvp);
  if (Dv != D || D == 16) return dtype == ATTN_BF16 ? fwd_mixed_bf16(D, Dv, jvp) : fwd_mixed_fp16(D, Dv, jvp);
  return dtype == ATTN_BF16 ? fwd_bf16(D, jvp, split) : fwd_fp16(D, jvp, split);
}

int launch(const KernelChoice& k, int grid, hipStream_t stream, const FwdArgs& a) {
  if (k.fn == nullptr) return ATTN_ERR_UNSUPPORTED;  // no instance for this combination
  if (k.lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(k.fn), hipFuncAttributeMaxDynamicSharedMemorySize, k.lds) != hipSuccess)
    return ATTN_ERR_HIP;
  hipLaunchKernelGGL(k.fn, dim3(grid), dim3(k.threads), k.lds, stream, a);
  return ATTN_OK;
}

// Optional bias / mask operand of the dense forward.
struct BiasOperand {
  const void* ptr = nullptr;
  int kind = kNoBias;
  attn_strides4 strides = {0, 0, 0, 1};
};

int dense(int dtype, const void* q, const void* k, const void* v, const void* tq, const void* tk, const void* tv,
          attn_strides4 sq, attn_strides4 sk, attn_strides4 sv, void* o, void* to, attn_strides4 so, float* lse,
          float* tlse, int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, float sm_scale, int causal,
          void* stream, bool jvp, const BiasOperand& bias = BiasOperand(), int64_t Dv = 0) {
  // query/key and value head dims: any of 16, 32, 64, 128, 256 (a 16-wide
  // value tile is laid out 32 wide in LDS)
  int rc = check_common(dtype, D, sm_scale, true, true);
  if (rc) return rc;
  if (Dv == 0) Dv = D;
  if (Dv != 16 && Dv != 32 && Dv != 64 && Dv != 128 && Dv != 256)
    return Dv < 0 ? ATTN_ERR_INVALID : ATTN_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0) return ATTN_ERR_INVALID;
  if (causal && Nq != Nkv) return ATTN_ERR_CAUSAL_SHAPE;
  if (B == 0 || H == 0 || Nq == 0) return ATTN_OK;
  // (batch, head) indices are 32-bit on the device
  if (Nq > INT_MAX || Nkv > INT_MAX || !mul_within(B, H, INT_MAX)) return ATTN_ERR_INVALID;
  const int64_t vec = dtype == ATTN_FP32 ? 4 : 8;
  if (!q || !o || !lse) return ATTN_ERR_INVALID;
  if (Nkv > 0 && (!k || !v)) return ATTN_ERR_INVALID;
  if (jvp && (!to || !tq || (Nkv > 0 && (!tk || !tv)))) return ATTN_ERR_INVALID;
  if ((rc = check_s4(sq, B, H, Nq, vec)) || (rc = check_s4(so, B, H, Nq, vec))) return rc;
  if (Nkv > 0 && ((rc = check_s4(sk, B, H, Nkv, vec)) || (rc = check_s4(sv, B, H, Nkv, vec)))) return rc;
  if (Nkv > 1 && (!kv_row_stride_ok(sk.n) || !kv_row_stride_ok(sv.n))) return ATTN_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, o, tq, tk, tv, to};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if (bias.kind != kNoBias && Nkv > 0) {
    // additive bias: 16-byte chunks of the input element type; mask: 8-byte chunks
    const int64_t bvec = bias.kind == kAddBias ? vec : 8;
    if (!bias.ptr) return ATTN_ERR_INVALID;
    if ((rc = check_s4(bias.strides, B, H, Nq, bvec))) return rc;
    if ((reinterpret_cast<uintptr_t>(bias.ptr) & (bias.kind == kAddBias ? 15u : 7u)) != 0) return ATTN_ERR_UNSUPPORTED;
  }
  const int bias_kind = Nkv > 0 ? bias.kind : kNoBias;  // no key: nothing to read

  const int64_t n_qtiles = (Nq + 127) / 128;  // every bf16 instance uses 128-row q-tiles
  const bool split =
      bias_kind == kNoBias && Dv == D && D != 256 && D != 16 && use_split(dtype, (int)D, jvp, causal != 0, B * H * n_qtiles);
  // Value columns per launch (the launches cover consecutive slices of V,
  // tV, O and tO; each recomputes the scores, and every output column sees
  // the same products as in one launch, so the bits do not change):
  // * the 16-bit JVP with 128 value columns (query/key dims below 256) runs
  //   as two 64-wide halves: three accumulators over 128 columns hold a wave
  //   to one per SIMD, over 64 two waves share a SIMD; the halves ran 1.2x
  //   to 1.5x faster than one launch;
  // * 256-wide queries and keys: the 16-bit JVP in 64-wide slices of 128 or
  //   256 value columns (the one-wave (256, 128) instance spilled about 580
  //   bytes per lane inside its key loop; the 64-wide slices ran 2.2x
  //   faster), the fp32 JVP with 256 value columns in 128-wide halves
  //   (three 256-wide accumulators would spill);
  // * 256 value columns with narrower queries and keys: 128-wide halves,
  //   the 16-bit JVP 64-wide quarters, on the value-dim instances of those
  //   widths.
  int64_t vs = Dv;
  if (bias_kind == kNoBias) {
    const bool jvp16 = jvp && dtype != ATTN_FP32;
    if (D == 256) {
      if (jvp16 && Dv >= 128) vs = 64;
      else if (Dv == 256 && jvp) vs = 128;
    } else if (Dv == 256) {
      vs = jvp16 ? 64 : 128;
    } else if (Dv == 128 && jvp16) {
      vs = 64;
    }
  }
  const int64_t n_slices = Dv / vs;
  const KernelChoice kc = choose(dtype, (int)D, jvp, split, bias_kind, (int)vs);
  const int BM = kc.BM;
  const int64_t n_qtiles_k = (Nq + BM - 1) / BM;
  const int64_t grid = B * H * (split ? (n_qtiles_k + 1) / 2 : n_qtiles_k);
  if (grid > INT_MAX) return ATTN_ERR_INVALID;

  FwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.tq = tq; a.tk = tk; a.tv = tv; a.o = o; a.to = to; a.lse = lse; a.tlse = tlse;
  a.q_sb = sq.b; a.q_sh = sq.h; a.q_sn = sq.n;
  a.k_sb = sk.b; a.k_sh = sk.h; a.k_sn = sk.n;
  a.v_sb = sv.b; a.v_sh = sv.h; a.v_sn = sv.n;
  a.o_sb = so.b; a.o_sh = so.h; a.o_sn = so.n;
  if (bias_kind != kNoBias) {
    a.bias = bias.ptr;
    a.bias_sb = bias.strides.b; a.bias_sh = bias.strides.h; a.bias_sn = bias.strides.n;
  }
  a.B = (int)B; a.H = (int)H; a.Nq = (int)Nq; a.Nkv = (int)Nkv;
  a.n_qtiles = (int)n_qtiles_k;
  a.paired = split ? 1 : 0;
  a.batch_inner = bias_kind != kNoBias && bias.strides.b == 0 && B > 1 ? 1 : 0;
  a.sm_scale = sm_scale;
  a.c = sm_scale * kLog2e;
  if (a.c == 0.f) a.c = 1.17549435e-38f;  // sm_scale == 0: keep exp2 arguments exactly 0 and -inf masks -inf
  a.causal = causal ? 1 : 0;
  a.offsets = nullptr;
  a.plan = nullptr;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();  // clear a stale error so that finish() reports only ours
  rc = launch(kc, (int)grid, st, a);
  if (rc) return rc;
  for (int64_t sl = 1; sl < n_slices; ++sl) {  // the other value slices; every launch writes the same LSE and tLSE
    const int64_t off = sl * vs * (dtype == ATTN_FP32 ? 4 : 2);  // bytes to slice sl's first column
    a.v = v ? (const char*)v + off : nullptr;  // no keys: V is never read
    a.tv = tv ? (const char*)tv + off : nullptr;
    a.o = (char*)o + off;
    a.to = to ? (char*)to + off : nullptr;
    rc = launch(kc, (int)grid, st, a);
    if (rc) return rc;
  }
  return finish(st);
}


int64_t plan_capacity(int64_t num_seqs, int64_t total_len, int BM) {
  // sum_s ceil(len_s / BM) <= floor((total_len + num_seqs (BM - 1)) / BM)
  return (total_len + num_seqs * (BM - 1)) / BM;
}

}  // namespace
}  // namespace attn

using namespace attn;

extern "C" {

int attn_fwd(attn_dtype dtype, const void* q, attn_strides4 q_strides, const void* k, attn_strides4 k_strides,
             const void* v, attn_strides4 v_strides, void* o, attn_strides4 o_strides, float* lse, int64_t B,
             int64_t H, int64_t Nq, int64_t Nkv, int64_t D, float sm_scale, int causal, void* stream) {
  return dense((int)dtype, q, k, v, nullptr, nullptr, nullptr, q_strides, k_strides, v_strides, o, nullptr,
               o_strides, lse, nullptr, B, H, Nq, Nkv, D, sm_scale, causal, stream, false);
}

int attn_fwd_bias(attn_dtype dtype, const void* q, attn_strides4 q_strides, const void* k, attn_strides4 k_strides,
                  const void* v, attn_strides4 v_strides, void* o, attn_strides4 o_strides, float* lse,
                  const void* bias, attn_bias_kind bias_kind, attn_strides4 bias_strides, int64_t B, int64_t H,
                  int64_t Nq, int64_t Nkv, int64_t D, float sm_scale, int causal, void* stream) {
  if (bias_kind != ATTN_BIAS_ADD && bias_kind != ATTN_BIAS_MASK) return ATTN_ERR_UNSUPPORTED;
  BiasOperand b;
  b.ptr = bias;
  b.kind = bias_kind == ATTN_BIAS_ADD ? kAddBias : kMaskBias;
  b.strides = bias_strides;
  return dense((int)dtype, q, k, v, nullptr, nullptr, nullptr, q_strides, k_strides, v_strides, o, nullptr,
               o_strides, lse, nullptr, B, H, Nq, Nkv, D, sm_scale, causal, stream, false, b);
}

int attn_fwd_dv(attn_dtype dtype, const void* q, const void* k, const void* v, const void* tq, const void* tk,
                const void* tv, attn_strides4 q_strides, attn_strides4 k_strides, attn_strides4 v_strides, void* o,
                void* to, attn_strides4 o_strides, float* lse, float* tlse, int64_t B, int64_t H, int64_t Nq,
                int64_t Nkv, int64_t Dqk, int64_t Dv, float sm_scale, int causal, void* stream) {
  if (Dv <= 0) return ATTN_ERR_INVALID;
  const bool jvp = tq != nullptr;
  if (!jvp && (tk || tv || to || tlse)) return ATTN_ERR_INVALID;
  return dense((int)dtype, q, k, v, tq, tk, tv, q_strides, k_strides, v_strides, o, to, o_strides, lse, tlse, B, H,
               Nq, Nkv, Dqk, sm_scale, causal, stream, jvp, BiasOperand(), Dv);
}

int attn_fwd_jvp(attn_dtype dtype, const void* q, const void* k, const void* v, const void* tq, const void* tk,
                 const void* tv, attn_strides4 q_strides, attn_strides4 k_strides, attn_strides4 v_strides, void* o,
                 void* to, attn_strides4 o_strides, float* lse, float* tlse, int64_t B, int64_t H, int64_t Nq,
                 int64_t Nkv, int64_t D, float sm_scale, int causal, void* stream) {
  return dense((int)dtype, q, k, v, tq, tk, tv, q_strides, k_strides, v_strides, o, to, o_strides, lse, tlse, B, H,
               Nq, Nkv, D, sm_scale, causal, stream, true);
}

size_t jagged_attn_workspace_bytes(int64_t num_seqs, int64_t total_len) {
  if (num_seqs < 0 || total_len < 0 || num_seqs > INT_MAX - 1 || total_len > INT_MAX) return 0;
  const int64_t cap = plan_capacity(num_seqs, total_len, kPlanBmMin);
  return (size_t)(16 + 8 * cap);
}

}  // extern "C"

// Static scratch of jagged_attn_fwd_noalloc: the tile plan of a call lives
// here instead of in a caller's workspace.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device array: every host use goes through
// the device address from scratch_address().
static __device__ __align__(256) int32_t scratch[ATTN_NOALLOC_SCRATCH_BYTES / 4];

namespace attn {
namespace {

// This device's address of `scratch`: hipGetSymbolAddress once per device,
// with that device current (the caller's), then cached.
int scratch_address(void** out) {
  static std::atomic<void*> addr[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_ERR_HIP;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ATTN_OK;
}

// jagged_attn_fwd and jagged_attn_fwd_noalloc: with `noalloc` the plan goes
// to this device's static scratch (workspace and workspace_bytes unused).
int jagged_fwd(attn_dtype dtype, const void* q, attn_strides3 q_strides, const void* k, attn_strides3 k_strides,
               const void* v, attn_strides3 v_strides, void* o, attn_strides3 o_strides, float* lse,
               const int64_t* offsets, int64_t num_seqs, int64_t H, int64_t total_len, int64_t D,
               int64_t max_seq_len, float sm_scale, int causal, void* workspace, size_t workspace_bytes,
               bool noalloc, void* stream) {
  int rc = check_common((int)dtype, D, sm_scale, true, true);
  if (rc) return rc;
  if (num_seqs < 0 || H < 0 || total_len < 0 || max_seq_len < 1) return ATTN_ERR_INVALID;
  if (num_seqs > INT_MAX - 1 || H > INT_MAX || total_len > INT_MAX) return ATTN_ERR_INVALID;
  if (num_seqs == 0 || H == 0 || total_len == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !offsets) return ATTN_ERR_INVALID;
  const int64_t vec = dtype == ATTN_FP32 ? 4 : 8;
  if ((rc = check_s3(q_strides, H, total_len, vec)) || (rc = check_s3(k_strides, H, total_len, vec)) ||
      (rc = check_s3(v_strides, H, total_len, vec)) || (rc = check_s3(o_strides, H, total_len, vec)))
    return rc;
  if (total_len > 1 && (!kv_row_stride_ok(k_strides.t) || !kv_row_stride_ok(v_strides.t))) return ATTN_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  const KernelChoice kc = choose((int)dtype, (int)D, false, false, kNoBias, (int)D);
  const int BM = kc.BM;
  const int64_t cap = plan_capacity(num_seqs, total_len, BM);
  const int64_t grid = cap * H;
  if (grid > INT_MAX) return ATTN_ERR_INVALID;
  if (noalloc) {  // the plan must fit the static scratch
    if (16 + 8 * cap > (int64_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    if ((rc = scratch_address(&workspace))) return rc;
  } else if (!workspace || workspace_bytes < (size_t)(16 + 8 * cap) || ((uintptr_t)workspace & 15u)) {
    return ATTN_ERR_WORKSPACE;
  }
  const int mlen = (int)(max_seq_len < INT_MAX ? max_seq_len : INT_MAX);

  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  int32_t* plan = (int32_t*)workspace;
  hipLaunchKernelGGL(jagged_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, offsets, (int)num_seqs, total_len,
                     mlen, causal ? 1 : 0, BM, kc.BN, plan, (int)cap);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;

  FwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.q_sh = q_strides.h; a.q_sn = q_strides.t;
  a.k_sh = k_strides.h; a.k_sn = k_strides.t;
  a.v_sh = v_strides.h; a.v_sn = v_strides.t;
  a.o_sh = o_strides.h; a.o_sn = o_strides.t;
  a.B = (int)num_seqs; a.H = (int)H; a.Nq = 0; a.Nkv = 0; a.n_qtiles = 0;
  a.sm_scale = sm_scale;
  a.c = sm_scale * kLog2e;
  if (a.c == 0.f) a.c = 1.17549435e-38f;
  a.causal = causal ? 1 : 0;
  a.offsets = offsets;
  a.plan = plan;
  a.total_len = (int)total_len;
  a.max_seq_len = mlen;
  rc = launch(kc, (int)grid, st, a);
  if (rc) return rc;
  return finish(st);
}

}  // namespace
}  // namespace attn

extern "C" {

int jagged_attn_fwd(attn_dtype dtype, const void* q, attn_strides3 q_strides, const void* k, attn_strides3 k_strides,
                    const void* v, attn_strides3 v_strides, void* o, attn_strides3 o_strides, float* lse,
                    const int64_t* offsets, int64_t num_seqs, int64_t H, int64_t total_len, int64_t D,
                    int64_t max_seq_len, float sm_scale, int causal, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return attn::jagged_fwd(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, offsets, num_seqs, H,
                          total_len, D, max_seq_len, sm_scale, causal, workspace, workspace_bytes, false, stream);
}

int jagged_attn_fwd_noalloc(attn_dtype dtype, const void* q, attn_strides3 q_strides, const void* k,
                            attn_strides3 k_strides, const void* v, attn_strides3 v_strides, void* o,
                            attn_strides3 o_strides, float* lse, const int64_t* offsets, int64_t num_seqs, int64_t H,
                            int64_t total_len, int64_t D, int64_t max_seq_len, float sm_scale, int causal,
                            void* stream) {
  return attn::jagged_fwd(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, lse, offsets, num_seqs, H,
                          total_len, D, max_seq_len, sm_scale, causal, nullptr, 0, true, stream);
}

size_t jagged_attn_bwd_workspace_bytes(int64_t num_seqs, int64_t H, int64_t total_len) {
  if (num_seqs < 0 || H < 0 || total_len < 0 || num_seqs > INT_MAX - 1 || total_len > INT_MAX || H > INT_MAX)
    return 0;
  if (!mul_within(H, total_len, (int64_t)1 << 40)) return 0;
  const int64_t plan = (16 + 8 * plan_capacity(num_seqs, total_len, 128) + 15) / 16 * 16;
  return (size_t)(plan + 8 * H * total_len);
}

int jagged_attn_bwd(attn_dtype dtype, const void* q, attn_strides3 q_strides, const void* k, attn_strides3 k_strides,
                    const void* v, attn_strides3 v_strides, const void* o, attn_strides3 o_strides, const void* d_o,
                    attn_strides3 do_strides, const float* lse, void* dq, attn_strides3 dq_strides, void* dk,
                    attn_strides3 dk_strides, void* dv, attn_strides3 dv_strides, const int64_t* offsets,
                    int64_t num_seqs, int64_t H, int64_t total_len, int64_t D, int64_t max_seq_len, float sm_scale,
                    int causal, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common((int)dtype, D, sm_scale, true, true);
  if (rc) return rc;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_UNSUPPORTED;
  if (num_seqs < 0 || H < 0 || total_len < 0 || max_seq_len < 1) return ATTN_ERR_INVALID;
  if (num_seqs > INT_MAX - 1 || H > INT_MAX || total_len > INT_MAX) return ATTN_ERR_INVALID;
  if (num_seqs == 0 || H == 0 || total_len == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv || !offsets) return ATTN_ERR_INVALID;
  const attn_strides3* ss[] = {&q_strides, &k_strides, &v_strides, &o_strides, &do_strides,
                               &dq_strides, &dk_strides, &dv_strides};
  for (const attn_strides3* x : ss)
    if ((rc = check_s3(*x, H, total_len, 8))) return rc;
  const void* ptrs[] = {q, k, v, o, d_o, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if (((uintptr_t)lse & 3u) != 0) return ATTN_ERR_UNSUPPORTED;
  const int64_t cap = plan_capacity(num_seqs, total_len, 128);
  // grids within an int (checked again by bwd_run, after the plan kernel has
  // been enqueued): the gradient kernels' cap H items and the prep kernel's
  // H total_len rows at 8 or more rows per block
  if (cap * H > INT_MAX || H * total_len / 8 > INT_MAX) return ATTN_ERR_INVALID;
  const size_t need = jagged_attn_bwd_workspace_bytes(num_seqs, H, total_len);
  if (need == 0) return ATTN_ERR_INVALID;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u)) return ATTN_ERR_WORKSPACE;
  const int mlen = (int)(max_seq_len < INT_MAX ? max_seq_len : INT_MAX);

  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  int32_t* plan = (int32_t*)workspace;
  hipLaunchKernelGGL(jagged_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, offsets, (int)num_seqs, total_len,
                     mlen, causal ? 1 : 0, 128, kBnBwdDq, plan, (int)cap);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;

  const int64_t plan_bytes = (16 + 8 * cap + 15) / 16 * 16;
  BwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = d_o; a.lse = lse; a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = (float*)((char*)workspace + plan_bytes);
  a.lse2 = a.delta + H * total_len;
  a.q_sh = q_strides.h; a.q_sn = q_strides.t;
  a.k_sh = k_strides.h; a.k_sn = k_strides.t;
  a.v_sh = v_strides.h; a.v_sn = v_strides.t;
  a.o_sh = o_strides.h; a.o_sn = o_strides.t;
  a.do_sh = do_strides.h; a.do_sn = do_strides.t;
  a.dq_sh = dq_strides.h; a.dq_sn = dq_strides.t;
  a.dk_sh = dk_strides.h; a.dk_sn = dk_strides.t;
  a.dv_sh = dv_strides.h; a.dv_sn = dv_strides.t;
  a.B = 1; a.H = (int)H; a.Nq = (int)total_len; a.Nkv = (int)total_len;  // the prep kernel's view
  a.sm_scale = sm_scale;
  a.c = sm_scale * kLog2e;
  if (a.c == 0.f) a.c = 1.17549435e-38f;
  a.causal = causal ? 1 : 0;
  a.offsets = offsets;
  a.plan = plan;
  a.total_len = (int)total_len;
  a.max_seq_len = mlen;
  rc = bwd_run(dtype == ATTN_FP16, (int)D, kNoBias, st, a, 1, H, total_len, total_len, cap);
  if (rc) return rc;
  return finish(st);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq) {
  if (B < 0 || H < 0 || Nq < 0) return 0;
  if (!mul_within(B, H, (int64_t)1 << 40) || !mul_within(B * H, Nq, (int64_t)1 << 40)) return 0;
  return (size_t)(8 * B * H * Nq);
}

}  // extern "C"

namespace attn {
namespace {

// Dense backward, optionally with a score operand and its gradient.
int dense_bwd(attn_dtype dtype, const void* q, attn_strides4 q_strides, const void* k, attn_strides4 k_strides,
              const void* v, attn_strides4 v_strides, const void* o, attn_strides4 o_strides, const void* d_o,
              attn_strides4 do_strides, const float* lse, void* dq, attn_strides4 dq_strides, void* dk,
              attn_strides4 dk_strides, void* dv, attn_strides4 dv_strides, int64_t B, int64_t H, int64_t Nq,
              int64_t Nkv, int64_t D, float sm_scale, int causal, void* workspace, size_t workspace_bytes,
              void* stream, const BiasOperand& bias, void* dbias, attn_strides4 dbias_strides) {
  int rc = check_common((int)dtype, D, sm_scale, true, true);
  if (rc) return rc;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_UNSUPPORTED;
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0) return ATTN_ERR_INVALID;
  if (causal && Nq != Nkv) return ATTN_ERR_CAUSAL_SHAPE;
  if (B == 0 || H == 0 || (Nq == 0 && Nkv == 0)) return ATTN_OK;
  if (Nq > INT_MAX || Nkv > INT_MAX || !mul_within(B, H, INT_MAX)) return ATTN_ERR_INVALID;
  if (Nq > 0 && (!q || !o || !d_o || !lse || !dq)) return ATTN_ERR_INVALID;
  if (Nkv > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_INVALID;
  const int64_t vec = 8;
  if ((rc = check_s4(q_strides, B, H, Nq, vec)) || (rc = check_s4(o_strides, B, H, Nq, vec)) ||
      (rc = check_s4(do_strides, B, H, Nq, vec)) || (rc = check_s4(dq_strides, B, H, Nq, vec)))
    return rc;
  if ((rc = check_s4(k_strides, B, H, Nkv, vec)) || (rc = check_s4(v_strides, B, H, Nkv, vec)) ||
      (rc = check_s4(dk_strides, B, H, Nkv, vec)) || (rc = check_s4(dv_strides, B, H, Nkv, vec)))
    return rc;
  const void* ptrs[] = {q, k, v, o, d_o, dq, dk, dv};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  const int bias_kind = Nq > 0 && Nkv > 0 ? bias.kind : kNoBias;  // nothing to read otherwise
  if (bias_kind != kNoBias) {
    if (!bias.ptr) return ATTN_ERR_INVALID;
    const int64_t bvec = 8;  // 16-bit bias: 16-byte chunks; mask: 8-byte chunks
    if ((rc = check_s4(bias.strides, B, H, Nq, bvec))) return rc;
    if ((reinterpret_cast<uintptr_t>(bias.ptr) & (bias_kind == kAddBias ? 15u : 7u)) != 0) return ATTN_ERR_UNSUPPORTED;
  }
  if (dbias != nullptr && bias_kind != kNoBias) {
    if (bias_kind != kAddBias) return ATTN_ERR_INVALID;  // a mask has no gradient
    if ((rc = check_s4(dbias_strides, B, H, Nq, 8))) return rc;
    // every element is written by one lane: broadcast (stride 0) would race
    if ((B > 1 && dbias_strides.b == 0) || (H > 1 && dbias_strides.h == 0) || (Nq > 1 && dbias_strides.n == 0))
      return ATTN_ERR_INVALID;
    if (!aligned16(dbias)) return ATTN_ERR_UNSUPPORTED;
  }
  const int64_t rows = B * H * Nq;  // B H <= INT_MAX, Nq <= INT_MAX: no overflow
  if (B * H * ((Nq + 127) / 128) > INT_MAX || B * H * ((Nkv + 127) / 128) > INT_MAX || rows / 8 > INT_MAX)
    return ATTN_ERR_INVALID;
  if (rows > 0 && (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, Nq) || ((uintptr_t)workspace & 15u)))
    return ATTN_ERR_WORKSPACE;

  BwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = d_o; a.lse = lse; a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = (float*)workspace;
  a.lse2 = (float*)workspace + rows;
  a.q_sb = q_strides.b; a.q_sh = q_strides.h; a.q_sn = q_strides.n;
  a.k_sb = k_strides.b; a.k_sh = k_strides.h; a.k_sn = k_strides.n;
  a.v_sb = v_strides.b; a.v_sh = v_strides.h; a.v_sn = v_strides.n;
  a.o_sb = o_strides.b; a.o_sh = o_strides.h; a.o_sn = o_strides.n;
  a.do_sb = do_strides.b; a.do_sh = do_strides.h; a.do_sn = do_strides.n;
  a.dq_sb = dq_strides.b; a.dq_sh = dq_strides.h; a.dq_sn = dq_strides.n;
  a.dk_sb = dk_strides.b; a.dk_sh = dk_strides.h; a.dk_sn = dk_strides.n;
  a.dv_sb = dv_strides.b; a.dv_sh = dv_strides.h; a.dv_sn = dv_strides.n;
  if (bias_kind != kNoBias) {
    a.bias = bias.ptr;
    a.bias_sb = bias.strides.b; a.bias_sh = bias.strides.h; a.bias_sn = bias.strides.n;
    if (dbias != nullptr) {
      a.dbias = dbias;
      a.dbias_sb = dbias_strides.b; a.dbias_sh = dbias_strides.h; a.dbias_sn = dbias_strides.n;
    }
  }
  a.B = (int)B; a.H = (int)H; a.Nq = (int)Nq; a.Nkv = (int)Nkv;
  a.batch_inner = bias_kind != kNoBias && bias.strides.b == 0 && B > 1 ? 1 : 0;
  a.sm_scale = sm_scale;
  a.c = sm_scale * kLog2e;
  if (a.c == 0.f) a.c = 1.17549435e-38f;  // sm_scale == 0: masked scores stay -inf (no 0 * inf)
  a.causal = causal ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  rc = bwd_run(dtype == ATTN_FP16, (int)D, bias_kind, st, a, B, H, Nq, Nkv, 0);
  if (rc) return rc;
  return finish(st);
}

}  // namespace
}  // namespace attn

extern "C" {

int attn_bwd(attn_dtype dtype, const void* q, attn_strides4 q_strides, const void* k, attn_strides4 k_strides,
             const void* v, attn_strides4 v_strides, const void* o, attn_strides4 o_strides, const void* d_o,
             attn_strides4 do_strides, const float* lse, void* dq, attn_strides4 dq_strides, void* dk,
             attn_strides4 dk_strides, void* dv, attn_strides4 dv_strides, int64_t B, int64_t H, int64_t Nq,
             int64_t Nkv, int64_t D, float sm_scale, int causal, void* workspace, size_t workspace_bytes,
             void* stream) {
  return dense_bwd(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, d_o, do_strides, lse, dq, dq_strides,
                   dk, dk_strides, dv, dv_strides, B, H, Nq, Nkv, D, sm_scale, causal, workspace, workspace_bytes,
                   stream, BiasOperand(), nullptr, attn_strides4{0, 0, 0, 1});
}

int attn_bwd_bias(attn_dtype dtype, const void* q, attn_strides4 q_strides, const void* k, attn_strides4 k_strides,
                  const void* v, attn_strides4 v_strides, const void* o, attn_strides4 o_strides, const void* d_o,
                  attn_strides4 do_strides, const float* lse, const void* bias, attn_bias_kind bias_kind,
                  attn_strides4 bias_strides, void* dbias, attn_strides4 dbias_strides, void* dq,
                  attn_strides4 dq_strides, void* dk, attn_strides4 dk_strides, void* dv, attn_strides4 dv_strides,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, float sm_scale, int causal,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (bias_kind != ATTN_BIAS_ADD && bias_kind != ATTN_BIAS_MASK) return ATTN_ERR_UNSUPPORTED;
  BiasOperand b;
  b.ptr = bias;
  b.kind = bias_kind == ATTN_BIAS_ADD ? kAddBias : kMaskBias;
  b.strides = bias_strides;
  return dense_bwd(dtype, q, q_strides, k, k_strides, v, v_strides, o, o_strides, d_o, do_strides, lse, dq, dq_strides,
                   dk, dk_strides, dv, dv_strides, B, H, Nq, Nkv, D, sm_scale, causal, workspace, workspace_bytes,
                   stream, b, dbias, dbias_strides);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration (dtype, head dim or alignment)";
    case ATTN_ERR_CAUSAL_SHAPE: return "causal attention requires Nq == Nkv";
    case ATTN_ERR_WORKSPACE:
      return "workspace missing or too small (jagged_attn_fwd_noalloc: the tile plan exceeds the static scratch, "
             "ATTN_NOALLOC_SCRATCH_BYTES)";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
