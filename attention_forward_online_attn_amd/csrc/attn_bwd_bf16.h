// bf16 attention backward for gfx950: the gradients dQ, dK, dV of the fused
// forward for a given dO, from the forward's O and LSE.
//
// What is computed follows the backward of the Triton fused attention
// tutorial with JVP (_attn_bwd_preprocess, _attn_bwd_dkdv, _attn_bwd_dq):
//   delta_i = sum_d O_id dO_id,   P = exp(S - LSE) with S = sm_scale Q K^T,
//   dV = P^T dO,   dP = dO V^T,   dS = P (dP - delta),
//   dQ = sm_scale dS K,   dK = sm_scale dS^T Q,
// with P and dS rounded to bf16 for their products (the page rounds them to
// the input type) and fp32 accumulation.
//
// Three kernels on one stream:
// * attn_bwd_prep_kernel: delta and LSE log2(e) per query row (workspace).
// * attn_bwd_dq_kernel: the forward's layout -- a lane owns one query, Q and
//   dO stay in registers, K and V tiles stream through LDS:
//   S^T = K Q^T and dP^T = V dO^T (scores_section), dS^T in registers, and
//   dQ^T += K^T dS^T through the transposing K reads (pv_section).
// * attn_bwd_dkdv_kernel: the mirror image -- a lane owns one key, K and V
//   stay in registers, Q and dO tiles (with their LSE and delta) stream
//   through LDS: S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//   dK^T += Q^T dS through the transposing Q and dO reads.
// Each output element is written once by one lane: no atomics, and the
// result does not depend on the order of the work.  Head dim 16 runs on the
// 32-wide tiles with a zero upper half; at head dim 256 the dK/dV kernel
// runs twice over the same key tiles (dV, then dK), since K, V and both
// accumulators exceed one wave's registers.
#pragma once

#include "attn_fwd_bf16.h"

namespace attn {

// One workgroup's share: element offsets of row 0 of its (batch|sequence,
// head) in every tensor, and the extents of that slice.
struct BwdTile {
  int64_t q_off, k_off, v_off, do_off, dq_off, dk_off, dv_off;
  int64_t row_base;  // index of row 0 in the LSE and workspace rows
  int64_t bias_off, dbias_off;  // element offsets of row 0 in the bias and its gradient (dense)
  int t;             // query tile (dQ kernel) or key tile (dK/dV kernel)
  int Lstore;        // rows / keys [0, Lstore) exist and are written
  int Lq;            // queries [0, Lq) take part
  int Lkv;           // keys [0, Lkv) take part
  bool valid;
};

// ---- delta_i = sum_d O_id dO_id and LSE_i log2(e), one row per D/8 lanes.
template <int D, bool F16 = false>
__global__ void __launch_bounds__(256) attn_bwd_prep_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;          // lanes per row, 16 bytes each
  constexpr int RPB = 256 / LPR;      // rows per workgroup
  const int64_t rows = (int64_t)a.B * a.H * a.Nq;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const int64_t bh = row / a.Nq;
    const int i = (int)(row - bh * a.Nq);
    const int b = (int)(bh / a.H), h = (int)(bh - (int64_t)b * a.H);
    const bf16* orow = (const bf16*)a.o + b * a.o_sb + h * a.o_sh + i * a.o_sn + part * 8;
    const bf16* drow = (const bf16*)a.dout + b * a.do_sb + h * a.do_sh + i * a.do_sn + part * 8;
    const bf16x8 ov = *(const bf16x8*)orow, dv = *(const bf16x8*)drow;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(from16<F16>(ov[e]), from16<F16>(dv[e]), acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    a.delta[row] = acc;
    const float l = a.lse[row];
    // a row without keys (LSE = -inf) has P = 0: exp2(s c - (+inf)) = 0
    a.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// Workgroup -> tile.  Dense: (batch, head, tile), XCD-aware like the forward
// (a run of consecutive work items per XCD shares that XCD's L2 copy of a
// head); with a bias shared by the batch, (head, tile, batch) as in the
// forward.  Jagged: item bid / H of the device-built plan, head bid % H; a
// sequence's first min(len, max_seq_len) rows take part as queries and keys,
// its later rows get zero gradients (SLL jagged page, backward).
// `store_rows_are_keys` selects which extent Lstore describes (dK/dV: keys).
__device__ __forceinline__ BwdTile bwd_tile(const BwdArgs& a, int bid, bool store_rows_are_keys) {
  BwdTile t;
  if (a.offsets == nullptr) {
    const int per_head = a.n_tiles;
    const int total = a.B * a.H * per_head;
    int logical = bid;
    if ((total & 7) == 0) logical = (bid & 7) * (total >> 3) + (bid >> 3);
    int b, h;
    if (a.batch_inner) {  // (head, tile, batch)-major: the batches of a tile share its bias through one L2
      b = logical % a.B;
      const int r = logical / a.B;
      h = r / per_head;
      t.t = r - h * per_head;
    } else {
      const int bh0 = logical / per_head;
      t.t = logical - bh0 * per_head;
      b = bh0 / a.H;
      h = bh0 - b * a.H;
    }
    const int bh = b * a.H + h;
    t.q_off = b * a.q_sb + h * a.q_sh;
    t.k_off = b * a.k_sb + h * a.k_sh;
    t.v_off = b * a.v_sb + h * a.v_sh;
    t.do_off = b * a.do_sb + h * a.do_sh;
    t.dq_off = b * a.dq_sb + h * a.dq_sh;
    t.dk_off = b * a.dk_sb + h * a.dk_sh;
    t.dv_off = b * a.dv_sb + h * a.dv_sh;
    t.row_base = (int64_t)bh * a.Nq;
    t.bias_off = b * a.bias_sb + h * a.bias_sh;
    t.dbias_off = b * a.dbias_sb + h * a.dbias_sh;
    t.Lq = a.Nq;
    t.Lkv = a.Nkv;
    t.Lstore = store_rows_are_keys ? a.Nkv : a.Nq;
    t.valid = true;
  } else {
    const int item = bid / a.H, h = bid - item * a.H;
    t.valid = item < a.plan[0];
    if (!t.valid) return t;
    const int seq = a.plan[4 + 2 * item];
    t.t = a.plan[5 + 2 * item];
    const int64_t T = a.total_len;
    int64_t begin = a.offsets[seq], end = a.offsets[seq + 1];
    begin = begin < 0 ? 0 : (begin > T ? T : begin);
    end = end < begin ? begin : (end > T ? T : end);
    const int len = (int)(end - begin);
    const int used = len < a.max_seq_len ? len : a.max_seq_len;
    t.q_off = h * a.q_sh + begin * a.q_sn;
    t.k_off = h * a.k_sh + begin * a.k_sn;
    t.v_off = h * a.v_sh + begin * a.v_sn;
    t.do_off = h * a.do_sh + begin * a.do_sn;
    t.dq_off = h * a.dq_sh + begin * a.dq_sn;
    t.dk_off = h * a.dk_sh + begin * a.dk_sn;
    t.dv_off = h * a.dv_sh + begin * a.dv_sn;
    t.row_base = (int64_t)h * T + begin;
    t.bias_off = 0;
    t.dbias_off = 0;
    t.Lq = used;
    t.Lkv = used;
    t.Lstore = len;
    t.valid = t.t * 128 < len;
  }
  return t;
}

// Direct global -> LDS copy of ROWS rows of DA bf16 (row stride sn elements)
// into the swizzled tile of D-element rows (D >= DA) at byte `dst` of LDS:
// instruction i of wave w fills 1 KiB block NW i + w, lane l the 16 bytes at
// l * 16; rows at or past `valid` re-read the last valid row (their results
// are masked or dropped).  With DA < D the lanes whose chunk is padding stay
// inactive: bwd_zero_pad clears those chunks once.
template <int D, int ROWS, int NW, int DA = D>
__device__ __forceinline__ void bwd_dma_rows(const bf16* base, int64_t sn, int row0, int valid, lds_t* dst, int wave,
                                             int lane) {
  constexpr int TILE = ROWS * D * 2, NBLK = TILE / 1024, NI = NBLK >= NW ? NBLK / NW : 1;
  constexpr int RPB = 1024 / (2 * D);
  static_assert(NBLK % NW == 0 || NBLK < NW, "whole 1 KiB blocks per wave");
  if (NBLK < NW && wave >= NBLK) return;
  const int last = valid - 1 - row0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = NW * i + wave;
    const int r = RPB * blk + (lane * 16) / (2 * D);
    const int ch = (lane % (D / 8)) ^ swz_f<D>(r);
    if (DA < D && ch >= DA / 8) continue;
    const int rr = r < last ? r : last;
    const char* src = (const char*)(base + (int64_t)(row0 + rr) * sn) + ch * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(dst + blk * 1024),
                                     16, 0, 0);
  }
}

// The dQ kernel's whole key tiles (all ROWS rows exist, row stride at most
// 2^22 elements) take bwd_dma_tile instead: a uniform base, plus i times the rows
// between a wave's blocks, plus one 32-bit lane offset.  When those blocks lie
// a multiple of 16 rows apart the swizzle, which depends on the row modulo
// 16, is the same for all of them.  The base stays an SGPR pair and the lane
// offset is zero-extended at each use (the saddr form), so a copy costs no
// vector instruction, where bwd_dma_rows computes each lane's clamped 64-bit
// address (36 vector instructions per step at D = 128).  The dK/dV kernel's
// query tiles keep bwd_dma_rows: with the biased kernel at its register
// limit the same change cost it 13%.
template <int D, int ROWS, int NW>
__device__ __forceinline__ constexpr bool bwd_dma_tile_ok() {
  constexpr int NBLK = ROWS * D * 2 / 1024, NI = NBLK >= NW ? NBLK / NW : 1;
  return NI == 1 || (NW * (1024 / (2 * D))) % 16 == 0;
}
__device__ __forceinline__ bool bwd_stride_ok(int64_t sn) { return sn <= ((int64_t)1 << 22); }

template <int D, int ROWS, int NW, int DA = D>
__device__ __forceinline__ void bwd_dma_tile(const bf16* base, int64_t sn, int row0, lds_t* dst, int wave, int lane) {
  constexpr int TILE = ROWS * D * 2, NBLK = TILE / 1024, NI = NBLK >= NW ? NBLK / NW : 1;
  constexpr int RPB = 1024 / (2 * D), RSTEP = NW * RPB;
  static_assert(bwd_dma_tile_ok<D, ROWS, NW>(), "one lane offset for every block of the wave");
  if (NBLK < NW && wave >= NBLK) return;
  const int r = RPB * wave + (lane * 16) / (2 * D);
  const int ch = (lane % (D / 8)) ^ swz_f<D>(r);
  if (DA < D && ch >= DA / 8) return;
  const char* tb = (const char*)(base + (int64_t)row0 * sn);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const char* b = tb + (int64_t)i * RSTEP * sn * 2;
    if constexpr (NI > 1) asm("" : "+s"(b));
    uint32_t lo = (uint32_t)(r * (int)sn + ch * 8) * 2u;
    asm("" : "+v"(lo));
    __builtin_amdgcn_global_load_lds((const void*)(b + lo),
                                     (__attribute__((address_space(3))) void*)(dst + (NW * i + wave) * 1024), 16, 0, 0);
  }
}

// Zero the padding chunks (columns DA .. D-1 of every row) of NT consecutive
// swizzled tiles of ROWS rows of D elements from byte `dst` of LDS: the tile
// copies never write them, so a 16-wide head dim can run on the 32-wide
// layout, its upper half zero (no effect on the scores; the output rows it
// feeds are not stored).  The caller's barrier after its first tile copy
// orders these stores before any read.
template <int D, int DA, int ROWS, int NT>
__device__ __forceinline__ void bwd_zero_pad(lds_t* dst, int tid) {
  constexpr int TILE = ROWS * D * 2, PADC = (D - DA) / 8;
  if constexpr (PADC > 0) {
    for (int id = tid; id < NT * ROWS * PADC; id += 256) {
      const int c = DA / 8 + id % PADC, row = (id / PADC) % ROWS, tl = id / (PADC * ROWS);
      *(__attribute__((address_space(3))) u32x4*)(dst + tl * TILE + swz_off<D>(row, c)) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Layout head dim of the gradient kernels: 16 runs on the 32-wide tiles.
template <int D>
constexpr int bwd_layout_dim() {
  return D < 32 ? 32 : D;
}

// ---------------------------------------------------------------- dQ kernel
template <int D, int BN>
struct BwdDqCfg {
  static constexpr int NW = 4, THREADS = 256, BM = 128;
  static constexpr int WAVES_PER_EU = D == 256 ? 1 : 2;  // D=256 holds Q, dO and dQ: 1 wave per SIMD
  static constexpr int DL = bwd_layout_dim<D>();
  static constexpr int TILE = BN * DL * 2;  // one K or V tile
  static constexpr int STAGE = 2 * TILE;   // K then V
  static constexpr int LDS = 2 * STAGE;
};

template <int D, int BN, bool F16 = false, int BIAS = kNoBias>
__global__ void __launch_bounds__(256, (BwdDqCfg<D, BN>::WAVES_PER_EU)) attn_bwd_dq_kernel(BwdArgs a) {
  using C = BwdDqCfg<D, BN>;
  constexpr int BM = C::BM, TILE = C::TILE, STAGE = C::STAGE, NW = C::NW, DL = C::DL;
  constexpr int NB = BN / 32, KD = DL / 16, DB = DL / 32;
  extern __shared__ __attribute__((aligned(256))) char smem_raw[];
  lds_t* smem = (lds_t*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  const BwdTile t = bwd_tile(a, blockIdx.x, false);
  if (!t.valid) return;
  int qt = t.t;
  if (a.causal && a.offsets == nullptr) qt = a.n_tiles - 1 - qt;  // heaviest first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, h32 = lane >> 5;
  const bf16* Q = (const bf16*)a.q + t.q_off;
  const bf16* K = (const bf16*)a.k + t.k_off;
  const bf16* V = (const bf16*)a.v + t.v_off;
  const bf16* DO = (const bf16*)a.dout + t.do_off;
  const int64_t row_base = t.row_base;

  // rows: this lane's query and the wave's key limits (rows past Lq attend
  // no key and get dQ = 0)
  const int w0 = qt * BM + wave * 32;
  const int my_row = w0 + n32;
  const int r_cl = my_row < t.Lstore ? my_row : t.Lstore - 1;
  auto lim = [&](int i) { return i >= t.Lq ? 0 : (a.causal ? min(i + 1, t.Lkv) : t.Lkv); };
  const int my_lim = lim(r_cl);
  const int w1 = min(w0 + 31, t.Lstore - 1);
  const int wave_max = w0 <= w1 && w0 < t.Lq ? lim(min(w1, t.Lq - 1)) : 0;
  const int wave_min = w0 <= w1 && w1 < t.Lq ? lim(w0) : 0;
  const int b1 = min(qt * BM + BM, t.Lq) - 1;
  const int n_tiles = qt * BM <= b1 ? (lim(b1) + BN - 1) / BN : 0;

  // Q and dO rows of this lane (B operands of S^T = K Q^T and dP^T = V dO^T)
  bf16x8 qf[KD], df[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    if (16 * kk < D) {
      qf[kk] = *(const bf16x8*)(Q + r_cl * a.q_sn + 16 * kk + 8 * h32);
      df[kk] = *(const bf16x8*)(DO + r_cl * a.do_sn + 16 * kk + 8 * h32);
    } else {  // padding columns of a 16-wide head
      qf[kk] = bf16x8{};
      df[kk] = bf16x8{};
    }
  }
  const float lse2 = a.lse2[row_base + r_cl];
  const float delta = a.delta[row_base + r_cl];

  const int krow = kperm(n32);
  uint32_t kaddr[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) kaddr[kk] = lds_base + swz_off<DL>(krow, 2 * kk + h32);
  int vlo[DB], vhi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) v_frag_offsets<DL>(lane, db, vlo[db], vhi[db]);

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  f32x16 dummy_a[1], dummy_b[1];
  bf16x8 dummy_h[1][2];
  bf16x8 dummy_t[1];
  f32x16 dummy_ts[1];

  // bias / mask of this lane's row, loaded one key tile ahead as in the
  // forward; with a bias gradient requested, dS of the row (as rounded for
  // the dQ product) is written for every key, 0 where the row sees none
  constexpr int BCH = 2 * NB;
  constexpr int BEL = BIAS == kAddBias ? 2 : 1;
  unsigned bsl[BIAS ? 2 : 1][BIAS ? BCH : 1][bias_dwords<BIAS>()];
  const char* brow = nullptr;
  bf16* dbrow = nullptr;
  if constexpr (BIAS != kNoBias) {
    brow = (const char*)a.bias + (t.bias_off + (int64_t)r_cl * a.bias_sn) * BEL;
    if (a.dbias != nullptr && my_row < t.Lstore) dbrow = (bf16*)a.dbias + t.dbias_off + (int64_t)my_row * a.dbias_sn;
  }
  const float cs = BIAS == kAddBias ? 1.f : a.c;  // the bias moves the scores to the exp2 domain
  auto bias_load = [&](int j, auto slot_tag) {
    if constexpr (BIAS != kNoBias)
      bias_chunks<BIAS, BCH>(brow, j * BN + 8 * h32, j * BN + BN <= t.Lkv, t.Lkv, bsl[decltype(slot_tag)::value]);
  };
  auto dbias_chunk = [&](int key0, bf16x8 val) {  // keys key0 .. key0 + 7 of this lane's row
    if (key0 + 8 <= t.Lkv) {
      *(bf16x8*)(dbrow + key0) = val;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key0 + e < t.Lkv) dbrow[key0 + e] = val[e];
    }
  };
  auto dbias_zero_tile = [&](int j) {
    if constexpr (BIAS != kNoBias) {
      if (dbrow != nullptr) {
        const bf16x8 z = {};
#pragma unroll
        for (int c = 0; c < BCH; ++c) dbias_chunk(j * BN + 16 * c + 8 * h32, z);
      }
    }
  };

  auto fetch = [&](int j, int stage) {
    if (bwd_dma_tile_ok<DL, BN, NW>() && j * BN <= t.Lkv - BN && bwd_stride_ok(a.k_sn) && bwd_stride_ok(a.v_sn)) {
      if constexpr (bwd_dma_tile_ok<DL, BN, NW>()) {
        bwd_dma_tile<DL, BN, NW, D>(K, a.k_sn, j * BN, smem + stage * STAGE, wave, lane);
        bwd_dma_tile<DL, BN, NW, D>(V, a.v_sn, j * BN, smem + stage * STAGE + TILE, wave, lane);
      }
    } else {
      bwd_dma_rows<DL, BN, NW, D>(K + (int64_t)j * BN * a.k_sn, a.k_sn, 0, t.Lkv - j * BN, smem + stage * STAGE, wave,
                                  lane);
      bwd_dma_rows<DL, BN, NW, D>(V + (int64_t)j * BN * a.v_sn, a.v_sn, 0, t.Lkv - j * BN, smem + stage * STAGE + TILE,
                                  wave, lane);
    }
  };

  auto step = [&](int j, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    if (j + 1 < n_tiles) {
      bias_load(j + 1, std::integral_constant<int, S ^ 1>{});
      fetch(j + 1, S ^ 1);
    }
    if (j * BN < wave_max) {
      f32x16 s[NB], dp[NB];
      scores_section<DL, NB, false, S * STAGE, 0, F16>(kaddr, qf, dummy_t, s, dummy_ts);          // S^T = K Q^T
      scores_section<DL, NB, false, S * STAGE + TILE, 0, F16>(kaddr, df, dummy_t, dp, dummy_ts);  // dP^T = V dO^T
      if (j * BN > wave_min - BN) {  // keys past this row's limit: P = 0
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * BN + 32 * bb + 16 * (r >> 3) + 8 * h32 + (r & 7);
            if (key >= my_lim) s[bb][r] = -INFINITY;
          }
      }
      if constexpr (BIAS != kNoBias) apply_bias<BIAS, F16, NB>(s, bsl[S], a.c);
      // dS^T = P^T (dP^T - delta) as the bf16 B operand (keys 8 per register
      // group = key chunk e / 8); chunk 0 first, chunk c+1 computed after the
      // MFMAs of chunk c of the product below
      bf16x8 dsf[NB][2];
      auto dsel = [&](auto e_tag) {
        constexpr int e = decltype(e_tag)::value, bb = e / 16, r = e % 16;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r], cs, -lse2));
        dsf[bb][r >> 3][r & 7] = to16<F16>(p * (dp[bb][r] - delta));
      };
      static_for<8>(dsel);
      // dQ^T += K^T dS^T (transposing reads of the K tile)
      pv_section<DL, NB, false, S * STAGE, 0, F16>(lds_base, vlo, vhi, dsf, dummy_h, acc, dummy_a, dummy_b, [&](auto i_tag) {
        constexpr int i = decltype(i_tag)::value, c = i / DB, EPS = 8 / DB;
        if constexpr (c + 1 < 2 * NB)
          static_for<EPS>([&](auto k_tag) {
            dsel(std::integral_constant<int, 8 * (c + 1) + (i % DB) * EPS + decltype(k_tag)::value>{});
          });
      });
      if constexpr (BIAS != kNoBias) {
        if (dbrow != nullptr) {
#pragma unroll
          for (int c = 0; c < BCH; ++c) dbias_chunk(j * BN + 16 * c + 8 * h32, dsf[c >> 1][c & 1]);
        }
      }
    } else {
      dbias_zero_tile(j);  // no key of this tile is seen by the wave's rows
    }
    __syncthreads();
  };

  bwd_zero_pad<DL, D, BN, 4>(smem, tid);  // K, V of both stages
  if (n_tiles > 0) {
    bias_load(0, std::integral_constant<int, 0>{});
    fetch(0, 0);
    __syncthreads();
    int j = 0;
    for (; j + 2 <= n_tiles; j += 2) {
      step(j, std::integral_constant<int, 0>{});
      step(j + 1, std::integral_constant<int, 1>{});
    }
    if (j < n_tiles) step(j, std::integral_constant<int, 0>{});
  }
  for (int j = n_tiles; j * BN < t.Lkv; ++j) dbias_zero_tile(j);  // key tiles no row of the workgroup sees

  if (my_row < t.Lstore) {
    bf16* orow = (bf16*)a.dq + t.dq_off + my_row * a.dq_sn;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (8 * g >= D) continue;  // padding rows of a 16-wide head
        const int d = 32 * db + 8 * g + 4 * h32;
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = to16<F16>(acc[db][4 * g + e] * a.sm_scale);
        *(bf16x4*)(orow + d) = ov;
      }
  }
}

// ------------------------------------------------------------- dK/dV kernel
template <int D, int BIAS = kNoBias>
struct BwdDkdvCfg {
  static constexpr int NW = 4, THREADS = 256, BN = 128;  // keys per workgroup, 32 per wave
  static constexpr int WAVES_PER_EU = D >= 128 ? 1 : 2;  // D>=128 holds K, V, dK, dV: 1 wave per SIMD
  // query rows per streamed tile: the one-wave D=128 kernel takes 64 (two
  // independent 32-query blocks per step, half the steps and barriers)
  static constexpr int BMQ = D == 128 ? 64 : 32;
  static constexpr int NBQ = BMQ / 32;                   // 32-query blocks per tile
  static constexpr int DL = bwd_layout_dim<D>();
  static constexpr int TILE = BMQ * DL * 2;              // one Q or dO tile
  // LDS: the two Q stages, the two dO stages, then each stage's lse2 and
  // delta rows (per 32-query block: 32 lse2 then 32 delta) -- grouped by
  // tensor so that every fragment read's offset fits the 16-bit immediate
  static constexpr int OFF_DO = 2 * TILE, OFF_ROWS = 4 * TILE, ROWS = NBQ * 256;
  static constexpr int LDS = 4 * TILE + 2 * ROWS;
  static constexpr bool AGPR_KV = D == 128;  // K and V fragments pinned to AGPRs (below)
};

// PART: kDkdvBoth computes dK and dV; at D = 256, where K, V and both
// accumulators do not fit one wave's registers, kDkdvOnlyV (K and dV: S and
// P only) and kDkdvOnlyK (K, V and dK) run as two launches.
constexpr int kDkdvBoth = 0, kDkdvOnlyV = 1, kDkdvOnlyK = 2;

template <int D, bool F16 = false, int BIAS = kNoBias, int PART = kDkdvBoth>
__global__ void __launch_bounds__(256, (BwdDkdvCfg<D, BIAS>::WAVES_PER_EU)) attn_bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdDkdvCfg<D, BIAS>;
  constexpr int BN = C::BN, BMQ = C::BMQ, NBQ = C::NBQ, TILE = C::TILE, NW = C::NW;
  constexpr int OFF_DO = C::OFF_DO, OFF_ROWS = C::OFF_ROWS, ROWS = C::ROWS;
  constexpr int DL = C::DL, KD = DL / 16, DB = DL / 32;
  constexpr bool DO_DV = PART != kDkdvOnlyK, DO_DK = PART != kDkdvOnlyV;
  extern __shared__ __attribute__((aligned(256))) char smem_raw[];
  lds_t* smem = (lds_t*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  // dense causal: low key tiles see the most queries and run first
  const BwdTile t = bwd_tile(a, blockIdx.x, true);
  if (!t.valid) return;
  const int kt = t.t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31, h32 = lane >> 5;
  const bf16* Q = (const bf16*)a.q + t.q_off;
  const bf16* K = (const bf16*)a.k + t.k_off;
  const bf16* V = (const bf16*)a.v + t.v_off;
  const bf16* DO = (const bf16*)a.dout + t.do_off;
  const int64_t row_base = t.row_base;

  // keys: this lane's key; the queries that can see the wave's keys (keys
  // past Lkv take no part and get dK = dV = 0)
  const int k0 = kt * BN + wave * 32;
  const int my_key = k0 + n32;
  const int k_cl = my_key < t.Lstore ? my_key : t.Lstore - 1;
  const bool wave_keys = k0 < t.Lkv;
  const int q_first = a.causal ? kt * BN : 0;        // first query any key of the workgroup sees
  const int wave_q_first = a.causal ? k0 : 0;        // first query any key of this wave sees
  const int jq0 = q_first / BMQ;
  const int n_qt = (t.Lq + BMQ - 1) / BMQ;

  // K and V rows of this lane (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[KD], vf[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    if (16 * kk < D) {
      kf[kk] = *(const bf16x8*)(K + k_cl * a.k_sn + 16 * kk + 8 * h32);
      vf[kk] = DO_DK ? *(const bf16x8*)(V + k_cl * a.v_sn + 16 * kk + 8 * h32) : bf16x8{};
    } else {  // padding columns of a 16-wide head
      kf[kk] = bf16x8{};
      vf[kk] = bf16x8{};
    }
  }
  // One wave per SIMD: the K and V fragments are pinned to the AGPR half of
  // the register file and feed the MFMAs from there as B operands, which
  // leaves the VGPR half to the accumulators and to the products the vector
  // ALU reads (this unit is built with MFMA results in VGPRs; with the
  // results in AGPRs every score and dP element was copied over first).
  if constexpr (C::AGPR_KV) {
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      u32x4 ku = __builtin_bit_cast(u32x4, kf[kk]), vu = __builtin_bit_cast(u32x4, vf[kk]);
      asm volatile("" : "+a"(ku), "+a"(vu));
      kf[kk] = __builtin_bit_cast(bf16x8, ku);
      vf[kk] = __builtin_bit_cast(bf16x8, vu);
    }
  }

  const int qrow = kperm(n32);
  uint32_t qaddr[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) qaddr[kk] = lds_base + swz_off<DL>(qrow, 2 * kk + h32);
  int vlo[DB], vhi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) v_frag_offsets<DL>(lane, db, vlo[db], vhi[db]);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  f32x16 dummy_a[1], dummy_b[1];
  bf16x8 dummy_h[1][2];
  bf16x8 dummy_t[1];
  f32x16 dummy_ts[1];

  // bias / mask for this lane's key and the 16 queries of each block's
  // registers (register r of block b: query q0 + 32 b + 16 (r / 8) + 8 h32 +
  // r % 8), element loads one query tile ahead; 32 lanes read 64 consecutive
  // bytes of a bias row
  constexpr int BEL = BIAS == kAddBias ? 2 : 1;
  unsigned bq[BIAS ? 2 : 1][BIAS ? 16 * NBQ : 1];  // register r of block b at 16 b + r
  const char* bcol = nullptr;
  if constexpr (BIAS != kNoBias) {
    const int kc = my_key < t.Lkv ? my_key : t.Lkv - 1;
    bcol = (const char*)a.bias + (t.bias_off + kc) * BEL;
  }
  const float cs = BIAS == kAddBias ? 1.f : a.c;  // the bias moves the scores to the exp2 domain
  auto bias_load = [&](int jq, auto slot_tag) {
    if constexpr (BIAS != kNoBias) {
      constexpr int SL = decltype(slot_tag)::value;
#pragma unroll
      for (int r = 0; r < 16 * NBQ; ++r) {
        const int qi = min(jq * BMQ + 32 * (r >> 4) + 16 * ((r >> 3) & 1) + 8 * h32 + (r & 7), t.Lq - 1);
        const char* src = bcol + (int64_t)qi * a.bias_sn * BEL;
        if constexpr (BIAS == kAddBias) bq[SL][r] = *(const unsigned short*)src;
        else bq[SL][r] = *(const unsigned char*)src;
      }
    }
  };

  // tile jq: Q and dO rows, then per 32-query block b 32 lse2 and 32 delta
  // values (4 bytes per lane of wave b: lanes 0-31 lse2, lanes 32-63 delta)
  auto fetch = [&](int jq, int stage) {
    const int q0 = jq * BMQ;
    bwd_dma_rows<DL, BMQ, NW, D>(Q, a.q_sn, q0, t.Lq, smem + stage * TILE, wave, lane);
    bwd_dma_rows<DL, BMQ, NW, D>(DO, a.do_sn, q0, t.Lq, smem + OFF_DO + stage * TILE, wave, lane);
    if (wave < NBQ) {
      const int qi = min(q0 + 32 * wave + n32, t.Lq - 1);
      const float* src = (h32 ? a.delta : a.lse2) + row_base + qi;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)(smem + OFF_ROWS + stage * ROWS + 256 * wave),
                                       4, 0, 0);
    }
  };

  auto step = [&](int jq, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    if (jq + 1 < n_qt) {
      bias_load(jq + 1, std::integral_constant<int, S ^ 1>{});
      fetch(jq + 1, S ^ 1);
    }
    const int q0 = jq * BMQ;
    if (wave_keys && q0 + BMQ > wave_q_first) {  // wave-uniform: some key of the wave sees some query
      f32x16 s[NBQ], dp[NBQ];
      scores_section<DL, NBQ, false, S * TILE, 0, F16>(qaddr, kf, dummy_t, s, dummy_ts);            // S = Q K^T
      if constexpr (DO_DK)
        scores_section<DL, NBQ, false, OFF_DO + S * TILE, 0, F16>(qaddr, vf, dummy_t, dp, dummy_ts);  // dP = dO V^T
      // masked pairs (query past Lq, key past Lkv; causal: key after query) get P = 0
      const bool edge = q0 + BMQ > t.Lq || k0 + 32 > t.Lkv || (a.causal && q0 < k0 + 32);
      if (edge) {
#pragma unroll
        for (int b = 0; b < NBQ; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = q0 + 32 * b + 16 * (r >> 3) + 8 * h32 + (r & 7);
            if (qi >= t.Lq || my_key >= t.Lkv || (a.causal && my_key > qi)) s[b][r] = -INFINITY;
          }
      }
      if constexpr (BIAS == kAddBias) {
#pragma unroll
        for (int b = 0; b < NBQ; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[b][r] = __builtin_fmaf(s[b][r], a.c,
                                     from16<F16>(__builtin_bit_cast(bf16, (unsigned short)bq[S][16 * b + r])) * kLog2e);
      } else if constexpr (BIAS == kMaskBias) {
#pragma unroll
        for (int b = 0; b < NBQ; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (bq[S][16 * b + r] == 0u) s[b][r] = -INFINITY;
      }
      // register r of block b holds query q0 + 32 b + 16 (r / 8) + 8 h32 + r % 8;
      // chunk c (block c / 2, registers 8 (c % 2) .. + 7) needs the lse2 and
      // delta of 8 consecutive queries
      const lds_t* st = smem + OFF_ROWS + S * ROWS;
      bf16x8 pf[NBQ][2], dsf[NBQ][2];
      auto chunk = [&](auto c_tag) {
        constexpr int c = decltype(c_tag)::value, b = c / 2, h = c % 2;
        constexpr int qo = 256 * b + 64 * h;
        const f32x4 a0 = *(const __attribute__((address_space(3))) f32x4*)(st + qo + 32 * h32);
        const f32x4 a1 = *(const __attribute__((address_space(3))) f32x4*)(st + qo + 32 * h32 + 16);
        f32x4 d0 = {}, d1 = {};
        if constexpr (DO_DK) {
          d0 = *(const __attribute__((address_space(3))) f32x4*)(st + qo + 128 + 32 * h32);
          d1 = *(const __attribute__((address_space(3))) f32x4*)(st + qo + 128 + 32 * h32 + 16);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float l2 = e < 4 ? a0[e & 3] : a1[e & 3];
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][8 * h + e], cs, -l2));
          pf[b][h][e] = to16<F16>(p);
          if constexpr (DO_DK) {
            const float dl = e < 4 ? d0[e & 3] : d1[e & 3];
            dsf[b][h][e] = to16<F16>(p * (dp[b][8 * h + e] - dl));
          }
        }
      };
      chunk(std::integral_constant<int, 0>{});
      // dV^T += dO^T P and dK^T += Q^T dS (transposing reads of the dO and Q
      // tiles); chunk c + 1 is formed after the first MFMA that consumes chunk c
      if constexpr (DO_DV)
        pv_section<DL, NBQ, false, OFF_DO + S * TILE, 0, F16>(lds_base, vlo, vhi, pf, dummy_h, dv, dummy_a, dummy_b,
                                                            [&](auto i_tag) {
          constexpr int i = decltype(i_tag)::value;
          if constexpr (i % DB == 0 && i / DB + 1 < 2 * NBQ) chunk(std::integral_constant<int, i / DB + 1>{});
        });
      else
        static_for<2 * NBQ - 1>([&](auto c_tag) { chunk(std::integral_constant<int, decltype(c_tag)::value + 1>{}); });
      if constexpr (DO_DK)
        pv_section<DL, NBQ, false, S * TILE, 0, F16>(lds_base, vlo, vhi, dsf, dummy_h, dk, dummy_a, dummy_b, [](auto) {});
    }
    __syncthreads();
  };

  bwd_zero_pad<DL, D, BMQ, 4>(smem, tid);  // Q, dO of both stages
  if (jq0 < n_qt && kt * BN < t.Lkv) {  // a tile of keys past Lkv only writes zeros
    bias_load(jq0, std::integral_constant<int, 0>{});
    fetch(jq0, 0);
    __syncthreads();
    int jq = jq0;
    for (; jq + 2 <= n_qt; jq += 2) {
      step(jq, std::integral_constant<int, 0>{});
      step(jq + 1, std::integral_constant<int, 1>{});
    }
    if (jq < n_qt) step(jq, std::integral_constant<int, 0>{});
  }

  if (my_key < t.Lstore) {
    bf16* krow_o = (bf16*)a.dk + t.dk_off + my_key * a.dk_sn;
    bf16* vrow_o = (bf16*)a.dv + t.dv_off + my_key * a.dv_sn;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (8 * g >= D) continue;  // padding rows of a 16-wide head
        const int d = 32 * db + 8 * g + 4 * h32;
        bf16x4 kv, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[e] = to16<F16>(dk[db][4 * g + e] * a.sm_scale);
          vv[e] = to16<F16>(dv[db][4 * g + e]);
        }
        if constexpr (DO_DK) *(bf16x4*)(krow_o + d) = kv;
        if constexpr (DO_DV) *(bf16x4*)(vrow_o + d) = vv;
      }
  }
}

}  // namespace attn
