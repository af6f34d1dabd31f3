// fp32 fused attention forward (dense, causal, jagged, optional JVP).
//
// Same streaming algorithm as the bf16 kernel -- per key tile: scores, running
// row max and sum, rescale by exp2(m_old - m_new), accumulate p V (pages:
// _attn_fwd_inner of the tutorial and JVP pages; the SLL jagged forward
// kernel) -- but every product stays in fp32 on the vector ALUs, so fp32
// callers get fp32 accuracy.  It is the precision path, not the throughput
// path: four lanes share a query row (each owns every 4th head-dim column),
// dot products are reduced across the four lanes, K/V tiles of 32 keys are
// staged in LDS and read as broadcasts.
#pragma once

#include "attn_common.h"

namespace attn {

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  return x;
}

// D: query/key head dim; DV_ (0: the same): value head dim.
template <int D, bool JVP, int DV_ = 0>
struct F32Cfg {
  static constexpr int DQK = D, DV = DV_ ? DV_ : D;
  static constexpr int BM = 64;   // query rows per workgroup (256 threads, 4 per row)
  static constexpr int BN = 32;   // keys per tile
  static constexpr int NTEN = JVP ? 4 : 2;
  static constexpr int LDS = (JVP ? 2 : 1) * BN * (DQK + DV) * 4;
};

template <int D, bool JVP, int BIAS = kNoBias, int DV_ = 0>
__global__ void __launch_bounds__(256) attn_fwd_f32_kernel(FwdArgs a) {
  using C = F32Cfg<D, JVP, DV_>;
  constexpr int BM = C::BM, BN = C::BN, NTEN = C::NTEN, DQK = C::DQK, DV = C::DV;
  constexpr int DQ = DQK / 4;             // query/key columns owned by each lane of a quad
  constexpr int DO_ = DV / 4;             // value / output columns owned by each lane
  static_assert(((BN * DQK / 4) % 256 == 0 || BN * DQK / 4 < 256) && ((BN * DV / 4) % 256 == 0 || BN * DV / 4 < 256),
                "tile must split evenly over 256 threads");
  extern __shared__ __attribute__((aligned(16))) float fsm[];

  const Tile t = resolve_tile<BM>(a, blockIdx.x);
  if (!t.valid) return;
  const int tid = threadIdx.x, u = tid & 3;
  const int my_row = t.qt * BM + (tid >> 2);
  const int rr = my_row < t.Lstore ? my_row : t.Lstore - 1;
  const int my_lim = kv_limit(t, a.causal, rr);
  const int row0 = t.qt * BM;
  const int b1 = min(row0 + BM, t.Lattend) - 1;
  const int blk_max = row0 <= b1 ? kv_limit(t, a.causal, b1) : 0;
  const int n_tiles = (blk_max + BN - 1) / BN;

  const float* Q = (const float*)a.q + t.q_off;
  const float* K = (const float*)a.k + t.k_off;
  const float* V = (const float*)a.v + t.v_off;
  const float* TQ = JVP ? (const float*)a.tq + t.q_off : nullptr;
  const float* TK = JVP ? (const float*)a.tk + t.k_off : nullptr;
  const float* TV = JVP ? (const float*)a.tv + t.v_off : nullptr;
  const float* srcs[4] = {K, V, TK, TV};
  const int64_t sns[4] = {a.k_sn, a.v_sn, a.k_sn, a.v_sn};
  // tiles in LDS: K, V, tK, tV (widths DQK, DV, DQK, DV)
  constexpr int toff[4] = {0, BN * DQK, BN * (DQK + DV), BN * (2 * DQK + DV)};
  constexpr int width[4] = {DQK, DV, DQK, DV};

  float qr[DQ], tqr[JVP ? DQ : 1];
  float acc[DO_], accA[JVP ? DO_ : 1], accB[JVP ? DO_ : 1];
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    qr[i] = Q[rr * a.q_sn + 4 * i + u];
    if constexpr (JVP) tqr[i] = TQ[rr * a.q_sn + 4 * i + u];
  }
#pragma unroll
  for (int i = 0; i < DO_; ++i) {
    acc[i] = 0.f;
    if constexpr (JVP) {
      accA[i] = 0.f;
      accB[i] = 0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f, r_run = 0.f;
  // bias / mask row of this lane's query (every lane of the quad reads it);
  // an additive bias moves the scores to the exp2 domain before the max
  const char* brow = nullptr;
  if constexpr (BIAS != kNoBias)
    brow = (const char*)a.bias + (t.bias_off + (int64_t)rr * a.bias_sn) * (BIAS == kAddBias ? 4 : 1);
  const float cs = BIAS == kAddBias ? 1.f : a.c;

  for (int j = 0; j < n_tiles; ++j) {
    __syncthreads();  // the previous tile is no longer being read
    static_for<NTEN>([&](auto x_tag) {
      constexpr int x = decltype(x_tag)::value, W = width[x];
      constexpr int F4 = BN * W / 4;  // float4 per tile
#pragma unroll
      for (int it = 0; it < (F4 + 255) / 256; ++it) {
        const int id = tid + 256 * it;
        if (F4 < 256 && id >= F4) break;
        const int row = id / (W / 4), c4 = id % (W / 4);
        int key = j * BN + row;
        key = key < t.Lkv ? key : t.Lkv - 1;
        *(f32x4*)(fsm + toff[x] + row * W + 4 * c4) = *(const f32x4*)(srcs[x] + key * sns[x] + 4 * c4);
      }
    });
    __syncthreads();
    const float* kt = fsm + toff[0];
    const float* vt = fsm + toff[1];
    const float* tkt = fsm + toff[2];
    const float* tvt = fsm + toff[3];

    float s[BN], ts[JVP ? BN : 1];
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      float part = 0.f, tpart = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        const float kv = kt[jj * DQK + 4 * i + u];
        part = __builtin_fmaf(qr[i], kv, part);
        if constexpr (JVP) tpart = __builtin_fmaf(tqr[i], kv, __builtin_fmaf(qr[i], tkt[jj * DQK + 4 * i + u], tpart));
      }
      s[jj] = quad_sum(part);
      if constexpr (JVP) ts[jj] = quad_sum(tpart);
      if (j * BN + jj >= my_lim) s[jj] = -INFINITY;
    }
    if constexpr (BIAS != kNoBias) {
      const bool full = j * BN + BN <= t.Lkv;
#pragma unroll
      for (int c = 0; c < BN / 8; ++c) {  // 8 keys per step
        float bv[8];
        if (full) {
          if constexpr (BIAS == kAddBias) {
            const f32x4 x0 = *(const f32x4*)(brow + 4 * (int64_t)(j * BN + 8 * c));
            const f32x4 x1 = *(const f32x4*)(brow + 4 * (int64_t)(j * BN + 8 * c + 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) { bv[e] = x0[e]; bv[4 + e] = x1[e]; }
          } else {
            const u32x2 w = *(const u32x2*)(brow + j * BN + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = (float)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
          }
        } else {  // ragged last tile: keys past the end are already masked
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = j * BN + 8 * c + e;
            bv[e] = 0.f;
            if (key < t.Lkv)
              bv[e] = BIAS == kAddBias ? ((const float*)brow)[key] : (float)((const unsigned char*)brow)[key];
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float& x = s[8 * c + e];
          if constexpr (BIAS == kAddBias) x = __builtin_fmaf(x, a.c, bv[e] * kLog2e);
          else if (bv[e] == 0.f) x = -INFINITY;
        }
      }
    }
    float mx = s[0];
#pragma unroll
    for (int jj = 1; jj < BN; ++jj) mx = fmaxf(mx, s[jj]);
    const float m_new = fmaxf(m_run, mx * cs);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    const float msub = m_new == -INFINITY ? 0.f : m_new;
    l_run *= alpha;
    r_run *= alpha;
#pragma unroll
    for (int i = 0; i < DO_; ++i) {
      acc[i] *= alpha;
      if constexpr (JVP) { accA[i] *= alpha; accB[i] *= alpha; }
    }
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      const float p = exp2f(__builtin_fmaf(s[jj], cs, -msub));
      l_run += p;
      const float hv = JVP ? p * ts[jj] : 0.f;
      r_run += hv;
#pragma unroll
      for (int i = 0; i < DO_; ++i) {
        const float vv = vt[jj * DV + 4 * i + u];
        acc[i] = __builtin_fmaf(p, vv, acc[i]);
        if constexpr (JVP) {
          accB[i] = __builtin_fmaf(hv, vv, accB[i]);
          accA[i] = __builtin_fmaf(p, tvt[jj * DV + 4 * i + u], accA[i]);
        }
      }
    }
    m_run = m_new;
  }

  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  if (my_row < t.Lstore) {
    float* orow = (float*)a.o + t.o_off + my_row * a.o_sn;
    float* torow = JVP ? (float*)a.to + t.o_off + my_row * a.o_sn : nullptr;
    const float r_tot = r_run * a.sm_scale;
#pragma unroll
    for (int i = 0; i < DO_; ++i) {
      const float o = acc[i] * inv;
      orow[4 * i + u] = o;
      if constexpr (JVP) torow[4 * i + u] = (accA[i] + a.sm_scale * accB[i] - r_tot * o) * inv;
    }
    if (u == 0) a.lse[t.lse_off + my_row] = empty ? -INFINITY : (m_run + log2f(l_run)) * kLn2;
    if constexpr (JVP)
      if (u == 0 && a.tlse != nullptr) a.tlse[t.lse_off + my_row] = r_tot * inv;
  }
}

}  // namespace attn
