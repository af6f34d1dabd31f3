// Shared device-side definitions: vector types, kernel arguments and the
// mapping of a workgroup to its (batch|sequence, head, query tile).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attn {

// Compile-time unrolled loop: f(std::integral_constant<int, i>) for i < N,
// so that i can feed immediate operands of inline assembly and index
// compile-time tables.
template <int... Is, class F>
__device__ __forceinline__ void static_for_seq(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(std::make_integer_sequence<int, N>{}, f);
}


typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Optional score operand of the dense forward (flash attention with bias
// page, _attn_fwd_inner): none, an additive bias in the input element type,
// or a uint8 mask (0 removes the key for that query).
enum BiasKind { kNoBias = 0, kAddBias = 1, kMaskBias = 2 };

// Arguments of every forward kernel (passed by value).  Strides are in
// elements; the head-dim stride is 1.  Tangents use the primal strides and
// tO uses the strides of O.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  void* o;
  void* to;
  float* lse;
  float* tlse;  // JVP: tangent of LSE per row (nullptr: not written)
  // optional [B, H, Nq, Nkv] additive bias (element type of q) or uint8 mask
  // (dense only; key stride 1, the other strides may be 0 to broadcast)
  const void* bias;
  int64_t bias_sb, bias_sh, bias_sn;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t B, H, Nq, Nkv;
  int32_t n_qtiles;  // dense: number of query tiles per (batch, head)
  int32_t paired;    // dense (8-wave key-split instances): a workgroup takes q-tiles p and n_qtiles-1-p
  int32_t batch_inner;  // dense: the batch is the fastest work index (a bias shared by the batch)
  float c;           // sm_scale * log2(e): scores go to the exp2 domain
  float sm_scale;
  int32_t causal;
  // jagged layout (offsets != nullptr): q/k/v/o are [H, total_len, D]
  const int64_t* offsets;
  const int32_t* plan;  // [0] item count, items (seq, q-tile) from index 4
  int32_t total_len;
  int32_t max_seq_len;
};

// Arguments of the backward kernels (passed by value).  Strides in elements.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B, H, Nq] natural log, as attn_fwd writes it
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace [B * H * Nq]: rowsum(O dO)
  float* lse2;   // workspace [B * H * Nq]: LSE log2(e); rows without keys +inf
  // dense only: optional [B, H, Nq, Nkv] bias (input element type) or uint8
  // mask (key stride 1), and the bias gradient dS (input element type;
  // nullptr: not written)
  const void* bias;
  int64_t bias_sb, bias_sh, bias_sn;
  void* dbias;
  int64_t dbias_sb, dbias_sh, dbias_sn;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int32_t B, H, Nq, Nkv;
  int32_t n_tiles;  // q-tiles (dQ kernel) or key tiles (dK/dV kernel) per (batch, head)
  int32_t batch_inner;  // dense: the batch is the fastest work index (a bias shared by the batch)
  float c;          // sm_scale * log2(e)
  float sm_scale;
  int32_t causal;
  // jagged layout (offsets != nullptr): tensors are [H, total_len, D], the
  // LSE and the workspace rows [H, total_len]; workgroups follow the plan
  const int64_t* offsets;
  const int32_t* plan;  // [0] item count, items (seq, 128-row tile) from index 4
  int32_t total_len;
  int32_t max_seq_len;
};

// One workgroup's share of the problem.
struct Tile {
  int64_t q_off, k_off, v_off, o_off;  // element offset of row 0 of this (batch|seq, head)
  int64_t lse_off;                     // element offset of row 0 in the fp32 LSE buffer
  int64_t bias_off;                    // element offset of row 0 in the bias / mask (dense)
  int qt;                              // query tile index
  int qt2;                             // second query tile of a paired workgroup, or -1
  int Lstore;                          // rows [0, Lstore) exist and are written
  int Lattend;                         // rows [0, Lattend) attend keys; later rows attend none
  int Lkv;                             // keys [0, Lkv)
  bool valid;
};

// Workgroup -> tile.  Dense: the hardware hands workgroup i to XCD i % 8, so
// each XCD is given a contiguous run of the (batch, head)-major work list:
// the query tiles of a head then run on one XCD and share its L2 copy of
// that head's K and V.  With an operand shared by the batch (bias batch
// stride 0) the list is (head, query tile, batch)-major instead: the batches
// of one query tile run together on one XCD and read each bias row through
// one L2, where the bias (N^2 elements per head) would otherwise be fetched
// from HBM once per batch.  Paired (small causal grids): workgroup p of a
// head takes query tiles p and n-1-p, which hold the same number of key
// tiles in all.  Otherwise, causal tiles run heaviest first within a head.
// Jagged: the device-built plan lists (sequence, query tile) items, most
// key tiles first; the head is the fastest index.
template <int BM>
__device__ __forceinline__ Tile resolve_tile(const FwdArgs& a, int bid) {
  Tile t;
  t.qt2 = -1;
  if (a.offsets == nullptr) {
    const int per_head = a.paired ? (a.n_qtiles + 1) >> 1 : a.n_qtiles;
    const int total = a.B * a.H * per_head;
    int logical = bid;
    if ((total & 7) == 0) logical = (bid & 7) * (total >> 3) + (bid >> 3);
    int b, h, qt;
    if (a.batch_inner) {
      b = logical % a.B;
      const int r = logical / a.B;
      h = r / per_head;
      qt = r - h * per_head;
    } else {
      const int bh0 = logical / per_head;
      qt = logical - bh0 * per_head;
      b = bh0 / a.H;
      h = bh0 - b * a.H;
    }
    const int bh = b * a.H + h;
    if (a.paired) {
      const int other = a.n_qtiles - 1 - qt;
      t.qt2 = other != qt ? other : -1;
    } else if (a.causal) {
      qt = a.n_qtiles - 1 - qt;
    }
    t.q_off = b * a.q_sb + h * a.q_sh;
    t.k_off = b * a.k_sb + h * a.k_sh;
    t.v_off = b * a.v_sb + h * a.v_sh;
    t.o_off = b * a.o_sb + h * a.o_sh;
    t.lse_off = (int64_t)bh * a.Nq;
    t.bias_off = b * a.bias_sb + h * a.bias_sh;
    t.qt = qt;
    t.Lstore = a.Nq;
    t.Lattend = a.Nq;
    t.Lkv = a.Nkv;
    t.valid = true;
  } else {
    const int item = bid / a.H, h = bid - item * a.H;
    t.valid = item < a.plan[0];
    if (!t.valid) return t;
    const int seq = a.plan[4 + 2 * item], qt = a.plan[5 + 2 * item];
    const int64_t T = a.total_len;
    int64_t begin = a.offsets[seq], end = a.offsets[seq + 1];
    begin = begin < 0 ? 0 : (begin > T ? T : begin);
    end = end < begin ? begin : (end > T ? T : end);
    const int len = (int)(end - begin);
    const int used = len < a.max_seq_len ? len : a.max_seq_len;
    t.q_off = h * a.q_sh + begin * a.q_sn;
    t.k_off = h * a.k_sh + begin * a.k_sn;
    t.v_off = h * a.v_sh + begin * a.v_sn;
    t.o_off = h * a.o_sh + begin * a.o_sn;
    t.lse_off = (int64_t)h * a.total_len + begin;
    t.bias_off = 0;
    t.qt = qt;
    t.Lstore = len;
    t.Lattend = used;
    t.Lkv = used;
    t.valid = qt * BM < len;
  }
  return t;
}

// Number of keys row i may attend (keys [0, limit) minus nothing else):
// causal rows stop at the diagonal; rows past Lattend attend none.
__device__ __forceinline__ int kv_limit(const Tile& t, int causal, int i) {
  if (i >= t.Lattend) return 0;
  return causal ? (i + 1 < t.Lkv ? i + 1 : t.Lkv) : t.Lkv;
}

}  // namespace attn
