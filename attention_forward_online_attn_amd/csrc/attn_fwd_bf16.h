// bf16 fused attention forward for gfx950 (CDNA4): S = K Q^T and O^T = V^T P^T
// on v_mfma_f32_32x32x16_bf16, online softmax in fp32 registers, K/V tiles
// double-buffered in LDS.  Optional fused forward-mode JVP.
//
// What is computed follows the pages' forward kernels (Triton fused attention
// tutorial with JVP: _attn_fwd_inner / _attn_fwd; Flash Attention v2 with JVP:
// _attn_fwd_inner / _attn_fwd; FBGEMM SLL jagged attention:
// _multi_head_jagged_flash_attention_fwd_kernel): per key tile, scores, a
// running row max m and row sum l, rescale by exp2(m_old - m_new), then
// acc += p V; epilogue O = acc / l, LSE = (m + log2 l) ln 2.  The JVP adds
// tS = tQ K^T + Q tK^T, H = p * tS (from fp32 p, as the JVP page orders it),
// r += rowsum(H), accA += p tV, accB += H V and the epilogue
// tO = (accA + accB - r O) / l.
//
// Layout on the chip (one workgroup = 4 waves = 128 query rows, 32 per wave):
// * Each wave computes S^T for its 32 queries, so a lane owns ONE query
//   (lane % 32) and 16 of every 32 keys; the other 16 sit in lane ^ 32.  Row
//   max/sum are in-lane plus one v_permlane32_swap.
// * The MFMA rows of S^T are keys in a permuted order (kperm below) chosen so
//   that the accumulator registers of S^T are, unchanged, the B operand of the
//   P^T product with 8 CONSECUTIVE keys per lane -- no shuffles between the two
//   products.
// * O^T keeps the same lane = query ownership, so the softmax rescale and the
//   epilogue are lane-local.
// * K and V live in LDS in their natural [key][d] layout with a 16-byte chunk
//   XOR swizzle; K fragments are ds_read_b128, V^T fragments come from the
//   transposing ds_read_b64_tr_b16.  Both are bank-conflict free.
// * Lagged rescaling: the running max used for p only moves when a row's
//   max passes it by more than the row's lag (log2 units), so the O rescale
//   is skipped on almost every tile; m, l and acc always share the same
//   reference, so the result is the same identity up to rounding.  The lag
//   is set after each rescale to log2(l) - 1 (row sum l relative to the new
//   max), clamped to [0, kTau]: a term taken without a rescale then has
//   p <= l / 2, i.e. at most a third of the row's final weight.  A row that
//   one key dominates therefore has that key's p = exp2(0) = 1, exact in the
//   16-bit P, as with the exact running max; spread rows, whose l grows fast,
//   reach the full lag kTau after a tile or two.  The fp16 JVP keeps the
//   exact running max (lag 0), so that |p| <= 1 keeps the fp16
//   H = p * scale * tS within the range of the page's own formulation.
// * Per key tile: the next tile is copied straight from global memory into
//   the other LDS stage (global_load_lds_dwordx4, no staging registers); the
//   copies stay in flight through the tile's two MFMA sections (scores, then
//   PV), whose LDS fragment reads run a fixed distance ahead of their MFMAs,
//   and one barrier ends the tile.  Two workgroups share each CU (two waves
//   per SIMD), so one wave's softmax overlaps the other's MFMAs.
// * Small causal grids use 8-wave workgroups: two 4-wave groups take the same
//   query tile, split its key range in halves (each streaming its own tiles
//   into its own LDS stages) and merge their partial (m, l, O) through LDS;
//   such a workgroup takes q-tiles p and n-1-p of a head in turn.
#pragma once

#include <type_traits>
#include <utility>

#include "attn_common.h"

namespace attn {

constexpr float kTau = 8.0f;  // largest lag of the running max (log2 units): p <= 2^kTau

// Waves whose rows attend at most this many keys add P's bf16 rounding
// residual to the PV product (the lo pass below).  With more keys the
// softmax weights of N(0,1)-like scores spread out, |O| stays well below
// max|v|, and the rounding errors of P average out in O.
constexpr int kSplitKeys = 32;

// 16-bit element formats of the MFMA kernels: bf16, or IEEE fp16 when F16.
// Tiles and fragments move raw 16-bit data in bf16-typed registers either
// way; only the MFMA opcode and the float <-> 16-bit conversions differ.
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Round to the element format (to nearest even); the bits in a bf16 slot.
template <bool F16>
__device__ __forceinline__ bf16 to16(float x) {
  if constexpr (F16) return __builtin_bit_cast(bf16, (f16)x);
  else return (bf16)x;
}

template <bool F16>
__device__ __forceinline__ float from16(bf16 x) {
  if constexpr (F16) return (float)__builtin_bit_cast(f16, x);
  else return (float)x;
}


// 16-byte-chunk XOR swizzle of a [rows][D] bf16 tile in LDS.  Conflict free
// for: 16 lanes reading one chunk of 16 different rows (K fragments), the
// transposing reads of 4 consecutive rows x 64 bytes (V fragments), and
// 16 lanes writing consecutive chunks (tile stores).  The 64 banks span 256
// bytes: a row of D = 128 fills them (the chunk is XORed with a bijection of
// row % 16), D = 64 rows share them in pairs (bijection of (row / 2) % 8),
// D = 32 rows in fours (row 4a + b, chunk c lands in slot 4 b + (c ^ a)),
// D = 16 (K tiles only) rows in eights (rows r and r + 8 swap their two
// chunks).
template <int D>
__device__ __forceinline__ int swz_f(int row) {
  if constexpr (D == 128 || D == 256) {  // D = 256: a row spans the banks twice; XOR on the low 4 chunk bits
    const int u = row & 15;
    return ((u & 3) << 2) | (u >> 2);
  } else if constexpr (D == 64) {
    const int u = (row >> 1) & 7;
    return ((u & 1) << 2) | (u >> 1);
  } else if constexpr (D == 32) {
    return (row >> 2) & 3;
  } else {
    return (row >> 3) & 1;
  }
}

template <int D>
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz_f<D>(row)) << 4);
}

// Key (within a 32-key block) that MFMA row m of S^T holds: swaps bits 2 and 3
// of m, so that accumulator register r of lane half h is key
// 16 (r / 8) + 8 h + (r % 8).
__device__ __forceinline__ int kperm(int m) {
  return (m & 16) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Minimum over lanes 0..31 of a non-negative float, as a wave-uniform
// (scalar) value; every lane active.  Non-negative floats order as their bit
// patterns, so the 16-lane steps (DPP: quad swaps, half-row and row mirrors)
// and the final pick between the two rows are unsigned minima.
__device__ __forceinline__ float wave_min32_nonneg(float x) {
  unsigned u = __float_as_uint(x);
  u = min(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  u = min(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  u = min(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));  // row_half_mirror
  u = min(u, (unsigned)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));  // row_mirror
  const unsigned a = __builtin_amdgcn_readlane(u, 0), b = __builtin_amdgcn_readlane(u, 16);
  return __uint_as_float(min(a, b));
}

// A operand of O^T += V^T P^T for output columns 32*db .. 32*db+31 and keys
// key0 .. key0+15: lane (d = lane % 32, half h) gets V[key0 + 8h + i][32 db + d],
// i = 0..7, from two transposing reads.  Within each 16-lane block the
// transposing read hands lane j element j % 4 of the 8-byte rows addressed by
// lanes 4i + j / 4, so lane s of the block addresses key (key0 + 8h + s / 4)
// (and 4 keys further for the second read) at columns
// 32 db + 16 (block % 2) + 4 (s % 4) .. +3.
//
// The swizzle of a row depends only on the row modulo 16 and key0 is a
// multiple of 16, so the lane-dependent part of the two addresses is computed
// once (v_frag_offsets) and key0 enters as an immediate offset.
template <int D>
__device__ __forceinline__ void v_frag_offsets(int lane, int db, int& lo, int& hi) {
  const int blk = lane >> 4, s = lane & 15;
  const int d = 32 * db + 16 * (blk & 1) + 4 * (s & 3);
  const int key = 8 * (blk >> 1) + (s >> 2);
  const int within = (d & 7) << 1;
  lo = swz_off<D>(key, d >> 3) + within;
  hi = swz_off<D>(key + 4, d >> 3) + within;
}

template <int D>
__device__ __forceinline__ bf16x8 v_frag(const lds_t* vt, int key0, int lo, int hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + lo + key0 * (D * 2)));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vt + hi + key0 * (D * 2)));
  const i16x4 v8[2] = {a, b};
  return __builtin_bit_cast(bf16x8, v8);
}

// V^T fragment read for the main PV product, as inline assembly.  The
// compiler treats the transposing-read builtin as possibly aliasing every
// global->LDS tile copy in flight and waits for all of them (vmcnt(0)) before
// it: that would expose the next tile's prefetch on every tile.  The stage
// read here was completed by the barrier that ended the previous tile, so no
// such wait is needed.  The compiler does not count these reads, so the
// caller waits for them itself (lds_wait) before the fragment is used; a
// count that also covers reads the compiler issued later only waits longer,
// since LDS reads complete in order.
template <int OFF>
__device__ __forceinline__ bf16x8 v_frag_async(uint32_t lo, uint32_t hi) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset is 16 bits");
  i16x4 a, b;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(a) : "v"(lo), "i"(OFF));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(b) : "v"(hi), "i"(OFF));
  const i16x4 v8[2] = {a, b};
  return __builtin_bit_cast(bf16x8, v8);
}

// Wait until at most N LDS reads of this wave are outstanding, before the
// use of the fragments f.  A scheduling fence right after the wait keeps
// those uses below it.  The fragments are not tied to the wait as operands:
// the hazard recognizer takes an inline-asm definition of a register for a
// possible vector-ALU write and pads the MFMA that reads it with a wait
// state, where the actual producers are LDS loads that the wait completes
// (57 fewer s_nop in the D = 128 forward; 0.6-1.3% faster).
template <int N, int F>
__device__ __forceinline__ void lds_wait(bf16x8 (&f)[F]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  (void)f;
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---- MFMA sections with software-pipelined LDS fragment reads.
//
// A section is a fixed list of MFMA steps, each fed by fragments read from
// LDS.  Reads run FD steps ahead of their MFMA through a ring of FD + 1
// fragment buffers, and a scheduling fence after every step keeps exactly
// that order: the MFMA pipe sees back-to-back work while at most FD reads are
// in flight, and the register footprint stays fixed (left alone, the
// scheduler hoists every read of a section to its top and spills).
constexpr int kFragDist = 4;  // FD of every instance but the JVP ones at the register limit
// Raised wave priority while a wave streams MFMAs: when two waves share a
// SIMD the one feeding the matrix core is issued first.
constexpr int kMfmaPrio = 1;

// K fragment read (16 bytes per lane) as inline assembly at a register
// address plus an immediate offset; the caller waits for it (lds_wait).
template <int OFF>
__device__ __forceinline__ bf16x8 k_frag_async(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset is 16 bits");
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// S^T = K Q^T for one [NB*32]-key tile (JVP: plus tS^T = tK Q^T + K tQ^T).
// Step i is key block i / KD, head-dim step i % KD.  K (tK) sits at byte KOFF
// (TKOFF) of LDS; kaddr[kk] is the lane's LDS address of its fragment for
// head-dim step kk in block 0 of a tile at byte 0.  The reads are inline
// assembly for the same reason as the V^T reads (they would otherwise be
// re-addressed every tile), with the same explicit waits.
template <int D, int NB, bool JVP, int KOFF, int TKOFF, bool F16 = false, int FD = kFragDist>
__device__ __forceinline__ void scores_section(const uint32_t (&kaddr)[D / 16], const bf16x8 (&qf)[D / 16],
                                               const bf16x8 (&tqf)[JVP ? D / 16 : 1], f32x16 (&s)[NB],
                                               f32x16 (&ts)[JVP ? NB : 1]) {
  constexpr int KD = D / 16, N = NB * KD, R = FD + 1, F = JVP ? 2 : 1;
  bf16x8 ring[R][F];
  auto issue = [&](auto i_tag) {
    constexpr int i = decltype(i_tag)::value;
    if constexpr (i < N) {
      constexpr int blk = 32 * (i / KD) * (D * 2);
      ring[i % R][0] = k_frag_async<KOFF + blk>(kaddr[i % KD]);
      if constexpr (JVP) ring[i % R][F - 1] = k_frag_async<TKOFF + blk>(kaddr[i % KD]);
    }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    s[b] = f32x16{};
    if constexpr (JVP) ts[b] = f32x16{};
  }
  __builtin_amdgcn_s_setprio(kMfmaPrio);
  static_for<FD>(issue);
  static_for<N>([&](auto i_tag) {
    constexpr int i = decltype(i_tag)::value;
    issue(std::integral_constant<int, i + FD>{});
    constexpr int later = F * ((N - 1 - i) < FD ? (N - 1 - i) : FD);
    lds_wait<(later < 15 ? later : 15), F>(ring[i % R]);
    constexpr int b = i / KD, kk = i % KD;
    const bf16x8* f = ring[i % R];
    s[b] = mfma16<F16>(f[0], qf[kk], s[b]);
    if constexpr (JVP) {
      ts[b] = mfma16<F16>(f[F - 1], qf[kk], ts[b]);
      ts[b] = mfma16<F16>(f[0], tqf[kk], ts[b]);
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  __builtin_amdgcn_s_setprio(0);
}

// O^T += V^T P^T for one tile (JVP: accB += V^T H^T, accA += tV^T P^T).
// Step i is key chunk i / DB (16 keys), output block i % DB: the chunks of P
// are consumed in order, so the caller's softmax for chunk c+1 (inter(i),
// placed after the MFMAs of step i) runs on the vector ALU while the matrix
// core works through chunk c.  V^T (tV^T) sits at byte VOFF (TVOFF) of LDS;
// lds_base is the LDS address of byte 0 and vlo/vhi the lane's offsets.
template <int D, int NB, bool JVP, int VOFF, int TVOFF, bool F16 = false, int FD = kFragDist, class Inter>
__device__ __forceinline__ void pv_section(uint32_t lds_base, const int (&vlo)[D / 32], const int (&vhi)[D / 32],
                                           const bf16x8 (&pf)[NB][2], const bf16x8 (&hf)[JVP ? NB : 1][2],
                                           f32x16 (&acc)[D / 32], f32x16 (&accA)[JVP ? D / 32 : 1],
                                           f32x16 (&accB)[JVP ? D / 32 : 1], Inter&& inter) {
  constexpr int DB = D / 32, KC = 2 * NB, N = DB * KC, R = FD + 1, F = JVP ? 2 : 1;
  constexpr int RPF = 2 * F;  // LDS reads per issued step
  bf16x8 ring[R][F];
  auto issue = [&](auto i_tag) {
    constexpr int i = decltype(i_tag)::value;
    if constexpr (i < N) {
      constexpr int db = i % DB, key0 = 16 * (i / DB);
      const uint32_t lo = lds_base + vlo[db], hi = lds_base + vhi[db];
      ring[i % R][0] = v_frag_async<VOFF + key0 * D * 2>(lo, hi);
      if constexpr (JVP) ring[i % R][F - 1] = v_frag_async<TVOFF + key0 * D * 2>(lo, hi);
    }
  };
  __builtin_amdgcn_s_setprio(kMfmaPrio);
  static_for<FD>(issue);
  static_for<N>([&](auto i_tag) {
    constexpr int i = decltype(i_tag)::value;
    issue(std::integral_constant<int, i + FD>{});
    // reads issued after step i's own: those of steps i+1 .. min(i+FD, N-1)
    constexpr int later = RPF * ((N - 1 - i) < FD ? (N - 1 - i) : FD);
    lds_wait<(later < 15 ? later : 15), F>(ring[i % R]);
    constexpr int db = i % DB, c = i / DB;
    const bf16x8* f = ring[i % R];
    acc[db] = mfma16<F16>(f[0], pf[c >> 1][c & 1], acc[db]);
    if constexpr (JVP) {
      accB[db] = mfma16<F16>(f[0], hf[c >> 1][c & 1], accB[db]);
      accA[db] = mfma16<F16>(f[F - 1], pf[c >> 1][c & 1], accA[db]);
    }
    inter(i_tag);
    __builtin_amdgcn_sched_barrier(0);
  });
  __builtin_amdgcn_s_setprio(0);
}

// O^T += V^T Plo^T over the 32 keys of block b, where Plo = p - bf16(p) is
// the bf16 rounding residual of P (so P enters O to about 16 bits).  Only
// waves whose rows attend a few keys run it, on one or two blocks; the
// compiler schedules its reads.
template <int D, bool F16 = false>
__device__ __forceinline__ void pv_lo_block(const lds_t* vt, const int (&vlo)[D / 32], const int (&vhi)[D / 32],
                                            int b, const bf16x8 (&plo)[2], f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int i = 0; i < 2 * (D / 32); ++i) {
    const bf16x8 f = v_frag<D>(vt, 32 * b + 16 * (i & 1), vlo[i >> 1], vhi[i >> 1]);
    acc[i >> 1] = mfma16<F16>(f, plo[i & 1], acc[i >> 1]);
  }
}

// ---- bias / mask operand (flash attention with bias page, _attn_fwd_inner).
// A lane whose scores sit in accumulator registers s[b][r] (key 32 b +
// 16 (r / 8) + 8 h + r % 8 of a tile, h the lane's half) needs, of its own
// row, the 8-key chunks c = 0 .. 2 NB - 1 at keys kb + 16 c (kb = tile start
// + 8 h): 16 bytes of a 16-bit bias or 8 bytes of a uint8 mask each; chunk c
// is registers 8 (c % 2) .. 8 (c % 2) + 7 of s[c / 2].
template <int BIAS>
constexpr int bias_dwords() { return BIAS == kAddBias ? 4 : 2; }

// Loads the chunks of one row into registers; `full`: every key of the
// chunks exists (vector loads), else element loads of the keys below Lkv.
template <int BIAS, int NCH>
__device__ __forceinline__ void bias_chunks(const char* brow, int kb, bool full, int Lkv,
                                            unsigned (&dst)[NCH][bias_dwords<BIAS>()]) {
  constexpr int BEL = BIAS == kAddBias ? 2 : 1;
  if (full) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const char* src = brow + (int64_t)(kb + 16 * c) * BEL;
      if constexpr (BIAS == kAddBias) {
        const u32x4 w = *(const u32x4*)src;
#pragma unroll
        for (int x = 0; x < 4; ++x) dst[c][x] = w[x];
      } else {
        const u32x2 w = *(const u32x2*)src;
        dst[c][0] = w[0];
        dst[c][1] = w[1];
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int x = 0; x < bias_dwords<BIAS>(); ++x) dst[c][x] = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb + 16 * c + e;
        if (key < Lkv) {
          if constexpr (BIAS == kAddBias)
            dst[c][e >> 1] |= (unsigned)(*(const unsigned short*)(brow + 2 * (int64_t)key)) << (16 * (e & 1));
          else
            dst[c][e >> 2] |= (unsigned)(*(const unsigned char*)(brow + key)) << (8 * (e & 3));
        }
      }
    }
  }
}

// Applies the chunks to the scores: additive bias -> s c + bias log2(e) (the
// exp2 domain, after which the softmax scale is 1), or with LN the logits
// s sm_scale + bias themselves (natural-log units: one FMA per score, the
// softmax then scales by log2(e)); mask -> -inf where 0.
template <int BIAS, bool F16, int NB, bool LN = false>
__device__ __forceinline__ void apply_bias(f32x16 (&s)[NB], const unsigned (&src)[2 * NB][bias_dwords<BIAS>()],
                                           float c) {
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (BIAS == kAddBias) {
        const unsigned w = src[2 * b + (r >> 3)][(r & 7) >> 1];
        const unsigned short h = (unsigned short)((r & 1) ? (w >> 16) : (w & 0xffffu));
        const float bv = from16<F16>(__builtin_bit_cast(bf16, h));
        s[b][r] = LN ? __builtin_fmaf(s[b][r], c, bv) : __builtin_fmaf(s[b][r], c, bv * kLog2e);
      } else {
        const unsigned w = src[2 * b + (r >> 3)][(r & 7) >> 2];
        if (((w >> (8 * (r & 3))) & 0xffu) == 0u) s[b][r] = -INFINITY;
      }
    }
}

// D is the query/key head dim; DV_ (0: the same) the value head dim, which
// sets the width of V, tV, O and tO (JVP page: _attention.forward takes
// d_v != d_qk).
template <int D, int BN, bool JVP, int NW_ = 4, int DV_ = 0>
struct Bf16Cfg {
  static constexpr int DQK = D, DV = DV_ ? DV_ : D;
  // value width in LDS: a 16-wide value tile is laid out 32 wide, its upper
  // half zero, so that the PV product keeps whole 32-row MFMA blocks
  static constexpr int DVL = DV < 32 ? 32 : DV;
  static constexpr int NW = NW_;            // waves per workgroup (32 query rows each)
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 128;            // query rows per q-tile (4 waves)
  // 8 waves: two groups of 4 take the same 128 query rows and split the key
  // range in two halves, each streaming its own tiles; the halves' partial
  // (m, l, O) are merged through LDS at the end
  static constexpr bool SPLIT = NW == 8;
  static constexpr int TILE_K = BN * DQK * 2;  // bytes of one K (or tK) tile
  static constexpr int TILE_V = BN * DVL * 2;  // bytes of one V (or tV) tile
  static constexpr int NTEN = JVP ? 4 : 2;  // tensors streamed per key tile
  static constexpr int STAGE = (JVP ? 2 : 1) * (TILE_K + TILE_V);  // bytes of one pipeline stage
  // Stage layout: K, V, then tK, tV, stage after stage.  When two stages
  // pass the 16-bit offset of the LDS reads (256-wide queries and keys: the
  // plain forward on 64-key tiles and the JVP on 32-key tiles; the biased
  // 256-wide instances keep 32-key tiles and fit) both stages' K-side tiles
  // come first and both stages' V-side tiles after them, and the V-side
  // reads take that region's start as their base: VSPLIT.  KSTR / VSTR: bytes from one stage's K-side / V-side tiles
  // to the next stage's; VBASE: start of the V-side region; OFF_*: a tile's
  // offset from its side's stage start.
  static constexpr bool VSPLIT = !SPLIT && 2 * STAGE > 65536;
  static constexpr int KSTR = VSPLIT ? (JVP ? 2 : 1) * TILE_K : STAGE;
  static constexpr int VSTR = VSPLIT ? (JVP ? 2 : 1) * TILE_V : STAGE;
  static constexpr int VBASE = VSPLIT ? 2 * KSTR : 0;
  static constexpr int OFF_V = VSPLIT ? 0 : TILE_K, OFF_TK = VSPLIT ? TILE_K : TILE_K + TILE_V;
  static constexpr int OFF_TV = VSPLIT ? TILE_V : 2 * TILE_K + TILE_V;
  // one wave per SIMD: 128-wide JVP accumulators (three of 64 registers) or
  // 256-wide queries and keys; the JVP with 128-wide queries and keys and at
  // most 64 value columns keeps two (at 64 with a one-step read-ahead, FDIST)
  static constexpr bool WIDE = (JVP && DV == 128) || DQK == 256;
  // floats per lane handed from group 1 to group 0 at the merge: m, l (r),
  // the O accumulator (and accA, accB)
  static constexpr int NVM = (JVP ? 3 : 2) + (DVL / 32) * 16 * (JVP ? 3 : 1);
  // double-buffered key tiles (per group when split); the merge reuses them
  static constexpr int LDS = SPLIT ? (4 * STAGE > NVM * 1024 ? 4 * STAGE : NVM * 1024) : 2 * STAGE;
  static constexpr int CPR_K = DQK / 8, CPR_V = DVL / 8;  // 16-byte chunks per row (in LDS)
  static constexpr int CPR_VS = DV / 8;                   // of those, chunks that hold data
  static constexpr int WAVES_PER_EU = WIDE ? 1 : 2;
  // The plain 4-wave forward at head dims up to 64 fits 128 registers (four
  // waves per SIMD) with no room for a per-row lag of the running max: its
  // waves share one lag in a scalar register.
  static constexpr bool WAVE_LAG = !JVP && NW == 4 && DQK <= 64;
  static_assert(BN % 32 == 0, "unsupported tile");
  // 256-wide queries and keys: values up to 128 wide, or 256 wide for the
  // plain forward (the JVP is launched on 64-wide value slices)
  static_assert(DQK == 16 || DQK == 32 || DQK == 64 || DQK == 128 || (DQK == 256 && (DV <= 128 || (!JVP && DV == 256))),
                "unsupported head dim");
  static_assert(!VSPLIT || (2 * KSTR <= 65536 && 2 * VSTR <= 65536), "each side's two stages within 16-bit offsets");
  static_assert(DV == 16 || DV == 32 || DV == 64 || DV == 128 || DV == 256, "unsupported head dim");
  static_assert(NW == 4 || (NW == 8 && DV == DVL), "8 waves: key-split workgroups of full-width value tiles");
};

template <int D, int BN, bool JVP, int NW_ = 4, bool F16 = false, int BIAS = kNoBias, int DV_ = 0>
__global__ void __launch_bounds__((Bf16Cfg<D, BN, JVP, NW_, DV_>::THREADS), (Bf16Cfg<D, BN, JVP, NW_, DV_>::WAVES_PER_EU))
attn_fwd_bf16_kernel(FwdArgs a) {
  using C = Bf16Cfg<D, BN, JVP, NW_, DV_>;
  constexpr int DQK = C::DQK, DV = C::DV, DVL = C::DVL, CPR_VS = C::CPR_VS;
  constexpr int BM = C::BM, NTEN = C::NTEN, STAGE = C::STAGE, TILE_K = C::TILE_K, TILE_V = C::TILE_V;
  constexpr int OFF_V = C::OFF_V, OFF_TK = C::OFF_TK, OFF_TV = C::OFF_TV;
  constexpr int KSTR = C::KSTR, VSTR = C::VSTR, VBASE = C::VBASE;
  constexpr int CPR_K = C::CPR_K, CPR_V = C::CPR_V;
  constexpr int THREADS = C::THREADS, NW = C::NW;
  constexpr bool SPLIT = C::SPLIT;
  constexpr int NWD = SPLIT ? 4 : NW;              // waves that fill one tile (a group's)
  static_assert(!SPLIT || BIAS == kNoBias, "no score operand with key-split workgroups");
  constexpr int NB = BN / 32;    // 32-key blocks per tile
  // LDS read-ahead of the MFMA sections: one step for the JVP instances that
  // sit at 256 VGPRs (128-wide queries and keys over 64 value columns, and
  // the key-split JVP at 64): with the full read-ahead their fragment rings
  // spilled, and the reloads inside the score section waited on every
  // outstanding load, the next tile's copies included (D = 128 JVP +10.6%,
  // causal JVP at 64 +3.3% without them)
  constexpr int FDIST = JVP && ((DQK == 128 && DV == 64) || (DQK == 64 && NW_ == 8)) ? 1 : kFragDist;
  constexpr int KD = DQK / 16;   // MFMA steps over the query/key head dim
  constexpr int DB = DVL / 32;   // 32-column output blocks
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  lds_t* smem = (lds_t*)smem_raw;
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

  const Tile t = resolve_tile<BM>(a, blockIdx.x);
  if (!t.valid) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: per-wave branches stay scalar
  const int n32 = lane & 31, h32 = lane >> 5;
  // key-range group of this wave (always 0 with 4 waves), its wave index
  // within the group, and the group's two LDS stages (the stage offset stays
  // an immediate of the LDS reads, which hold 16 bits)
  const int grp = SPLIT ? wave >> 2 : 0;
  const int wd = SPLIT ? wave & 3 : wave;
  lds_t* const smem_g = smem + grp * 2 * STAGE;
  const uint32_t lds_g = lds_base + grp * 2 * STAGE;
  const bf16* Q = (const bf16*)a.q + t.q_off;
  const bf16* K = (const bf16*)a.k + t.k_off;
  const bf16* V = (const bf16*)a.v + t.v_off;
  const bf16* TQ = JVP ? (const bf16*)a.tq + t.q_off : nullptr;
  const bf16* TK = JVP ? (const bf16*)a.tk + t.k_off : nullptr;
  const bf16* TV = JVP ? (const bf16*)a.tv + t.v_off : nullptr;

  // Direct global -> LDS tile loads (global_load_lds_dwordx4): instruction i
  // of this wave fills the 1 KiB block NWD * i + wd of a tile (RPB rows; the
  // NWD waves of a group fill that group's tiles, wd is the wave's index in
  // it), lane
  // l the 16 bytes at l * 16 of it, so lane l fetches the chunk whose swizzled
  // home is that spot (the swizzle is an XOR, its own inverse).  A wave's
  // consecutive blocks lie RSTEP rows apart, a multiple of 16, and the
  // swizzle depends on the row modulo 16 only: one per-lane byte offset
  // serves every instruction, which adds a uniform i * RSTEP rows.  No
  // registers or ds_write instructions are spent on staging.
  // K-side tensors (K, tK) and V-side tensors (V, tV) each have their own
  // row width, hence their own block mapping; with equal head dims the two
  // coincide and the instructions interleave as K, V, tK, tV.
  constexpr int NBLK_K = TILE_K / 1024, NBLK_V = TILE_V / 1024;  // 1 KiB blocks per tile
  constexpr int NI_K = NBLK_K >= NWD ? NBLK_K / NWD : 1;          // DMA instructions per wave per tensor
  constexpr int NI_V = NBLK_V >= NWD ? NBLK_V / NWD : 1;
  constexpr int NIM = NI_K > NI_V ? NI_K : NI_V;
  constexpr int RPB_K = 1024 / (2 * DQK), RPB_V = 1024 / (2 * DVL);  // rows per block
  constexpr int RSTEP_K = NWD * RPB_K, RSTEP_V = NWD * RPB_V;       // rows between a wave's blocks
  static_assert((NBLK_K % NWD == 0 || NBLK_K < NWD) && (NBLK_V % NWD == 0 || NBLK_V < NWD),
                "DMA tiles are whole 1 KiB blocks per wave");
  // The swizzle depends on the row modulo 16.  When a wave's blocks lie a
  // multiple of 16 rows apart one per-lane offset serves every instruction;
  // with fewer rows per block (D = 256: 2 rows, blocks 8 rows apart) the
  // swizzle of instruction i repeats with period NPH = 16 / RSTEP, and each
  // phase has its own per-lane offset.
  static_assert(((NI_K == 1 || RSTEP_K % 16 == 0 || 16 % RSTEP_K == 0) &&
                         (NI_V == 1 || RSTEP_V % 16 == 0 || 16 % RSTEP_V == 0)),
                "per-lane swizzle must repeat with the block step");
  constexpr int NPH_K = (NI_K == 1 || RSTEP_K % 16 == 0) ? 1 : 16 / RSTEP_K;
  constexpr int NPH_V = (NI_V == 1 || RSTEP_V % 16 == 0) ? 1 : 16 / RSTEP_V;
  const bool dma_k = NBLK_K >= NWD || wd < NBLK_K;  // waves past the tile's blocks fetch nothing
  const bool dma_v = NBLK_V >= NWD || wd < NBLK_V;
  const int drow_k = RPB_K * wd + (lane * 16) / (2 * DQK);            // row of instruction 0
  const int drow_v = RPB_V * wd + (lane * 16) / (2 * DVL);
  int dch_k[NPH_K], dch_v[NPH_V];                                     // source chunk per phase
  uint32_t dk0[NPH_K], dv0[NPH_V];                                    // byte offsets per phase
#pragma unroll
  for (int ph = 0; ph < NPH_K; ++ph) {
    dch_k[ph] = (lane % CPR_K) ^ swz_f<DQK>(drow_k + RSTEP_K * ph);
    dk0[ph] = (uint32_t)((drow_k * a.k_sn + dch_k[ph] * 8) * 2);
  }
#pragma unroll
  for (int ph = 0; ph < NPH_V; ++ph) {
    dch_v[ph] = (lane % CPR_V) ^ swz_f<DVL>(drow_v + RSTEP_V * ph);
    dv0[ph] = (uint32_t)((drow_v * a.v_sn + dch_v[ph] * 8) * 2);
  }
  // Head dims 128 and 256, the plain key-split workgroups and the 4-wave
  // JVP: the lane offsets pass through an opaque statement in place once per
  // tile (no copy per use), and the whole-tile branch ends in an empty
  // volatile statement, so that its last copy is not merged with the ragged
  // branch's into one copy with a 64-bit vector address: three fewer vector
  // instructions per tile.  Elsewhere both cost registers (the 4-wave plain
  // D = 64 forward would drop from four waves per SIMD to three, the
  // key-split D = 64 JVP would spill more), and the per-use copy stays.
  constexpr bool OFFS_INPLACE = DQK >= 128 || (NW_ == 8 && !JVP) || (NW_ == 4 && JVP);
  auto dma_tile = [&](int j, int stage) {
    const int64_t k0 = (int64_t)j * BN;
    const char* src[4] = {(const char*)K + k0 * a.k_sn * 2, (const char*)V + k0 * a.v_sn * 2,
                          JVP ? (const char*)TK + k0 * a.k_sn * 2 : nullptr,
                          JVP ? (const char*)TV + k0 * a.v_sn * 2 : nullptr};
    lds_t* const base = smem_g;
    const int toff[4] = {stage * KSTR, VBASE + stage * VSTR + OFF_V, stage * KSTR + OFF_TK,
                         VBASE + stage * VSTR + OFF_TV};
    const int64_t step_b[2] = {(int64_t)RSTEP_K * a.k_sn * 2, (int64_t)RSTEP_V * a.v_sn * 2};
    if constexpr (OFFS_INPLACE) {
#pragma unroll
      for (int ph = 0; ph < NPH_K; ++ph) asm("" : "+v"(dk0[ph]));
#pragma unroll
      for (int ph = 0; ph < NPH_V; ++ph) asm("" : "+v"(dv0[ph]));
    }
    // a whole tile of keys: in 32 bits (j BN < Lkv <= INT_MAX), a scalar
    // compare rather than a 64-bit one on the vector ALU
    if (j * BN <= t.Lkv - BN) {
#pragma unroll
      for (int i = 0; i < NIM; ++i)
#pragma unroll
        for (int x = 0; x < NTEN; ++x) {
          const bool vs = x & 1;
          if (i >= (vs ? NI_V : NI_K) || !(vs ? dma_v : dma_k)) continue;
          // a padded value tile: lanes whose slot is padding stay inactive
          if (vs && DV < DVL && dch_v[i % NPH_V] >= CPR_VS) continue;
          // the uniform part of the address stays an SGPR pair (saddr form:
          // scalar base + 32-bit lane offset); with several instructions per
          // tensor the compiler would otherwise fold it into per-lane 64-bit
          // addresses held across the loop.  Likewise the lane offset: an
          // opaque copy at each use (OFFS_INPLACE: the opaque statement per
          // tile above) keeps its zero-extension next to the load
          // (hoisted out of the key loop, it would turn every copy into a
          // 64-bit vector add and a 64-bit address: 28 more vector
          // instructions per pass over the unrolled loop at D = 128, 1-3%)
          const char* b = src[x] + i * step_b[vs];
          if constexpr (NIM > 1) asm("" : "+s"(b));
          uint32_t lo = vs ? dv0[i % NPH_V] : dk0[i % NPH_K];
          if constexpr (!OFFS_INPLACE) asm("" : "+v"(lo));
          __builtin_amdgcn_global_load_lds((const void*)(b + lo),
                                           (__attribute__((address_space(3))) void*)(base + (NWD * i + wd) * 1024 + toff[x]),
                                           16, 0, 0);
        }
      if constexpr (OFFS_INPLACE) asm volatile("");
    } else {  // ragged last tile: rows past the keys re-read the last key (masked)
      const int last = t.Lkv - 1 - (int)k0;
#pragma unroll
      for (int i = 0; i < NIM; ++i) {
        const int row_k = min(drow_k + RSTEP_K * i, last), row_v = min(drow_v + RSTEP_V * i, last);
        const uint32_t ok = (uint32_t)((row_k * a.k_sn + dch_k[i % NPH_K] * 8) * 2);
        const uint32_t ov = (uint32_t)((row_v * a.v_sn + dch_v[i % NPH_V] * 8) * 2);
#pragma unroll
        for (int x = 0; x < NTEN; ++x) {
          const bool vs = x & 1;
          if (i >= (vs ? NI_V : NI_K) || !(vs ? dma_v : dma_k)) continue;
          if (vs && DV < DVL && dch_v[i % NPH_V] >= CPR_VS) continue;
          __builtin_amdgcn_global_load_lds((const void*)(src[x] + (vs ? ov : ok)),
                                           (__attribute__((address_space(3))) void*)(base + (NWD * i + wd) * 1024 + toff[x]),
                                           16, 0, 0);
        }
      }
    }
  };

  // ---- one query tile per pass: with 8 waves a workgroup takes q-tiles p
  // and n-1-p of a head one after the other (every pair holds the same
  // number of key tiles in all, and each is split between the two groups)
  const int n_pass = SPLIT && t.qt2 >= 0 ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int qt = pass == 0 ? t.qt : t.qt2;

    // ---- row bookkeeping (lane % 32 is this lane's query row; with 8 waves
    // both groups take the same rows)
    const int row0 = qt * BM;
    const int w0 = row0 + (wave & 3) * 32;
    const int my_row = w0 + n32;
    const int my_lim = kv_limit(t, a.causal, my_row < t.Lstore ? my_row : t.Lstore - 1);
    const int w1 = min(w0 + 31, t.Lstore - 1);
    int wave_max = 0, wave_min = 0;  // max / min key limit over the wave's rows
    if (w0 <= w1) {
      wave_max = w0 < t.Lattend ? kv_limit(t, a.causal, min(w1, t.Lattend - 1)) : 0;
      wave_min = w1 >= t.Lattend ? 0 : kv_limit(t, a.causal, w0);
    }
    const int b1 = min(row0 + BM, t.Lattend) - 1;
    const int blk_max = row0 <= b1 ? kv_limit(t, a.causal, b1) : 0;
    const int n_tiles = (blk_max + BN - 1) / BN;
    // key tiles of this wave's group: all of them, or with 8 waves group g
    // takes tiles [g n0, min((g + 1) n0, n_tiles)); every wave runs n0 steps
    const int n0 = SPLIT ? (n_tiles + 1) >> 1 : n_tiles;
    const int jbase = grp * n0;
    const int n_mine = SPLIT ? min(n0, n_tiles - jbase) : n_tiles;

    // ---- Q (and tQ) fragments, resident for the whole key loop: the B operand
    // of S^T = K Q^T, lane (query n32, half h32) holds Q[row][16 kk + 8 h32 + 0..7]
    bf16x8 qf[KD];
    bf16x8 tqf[JVP ? KD : 1];
    {
      const int r = my_row < t.Lstore ? my_row : t.Lstore - 1;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) qf[kk] = *(const bf16x8*)(Q + r * a.q_sn + 16 * kk + 8 * h32);
      if constexpr (JVP) {
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) tqf[kk] = *(const bf16x8*)(TQ + r * a.q_sn + 16 * kk + 8 * h32);
      }
    }

    f32x16 acc[DB];
    f32x16 accA[JVP ? DB : 1], accB[JVP ? DB : 1];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      acc[i] = f32x16{};
      if constexpr (JVP) { accA[i] = f32x16{}; accB[i] = f32x16{}; }
    }
    // ---- bias / mask: lane (query n32, half h32) needs, of each tile, the
    // 8-key chunks c = 0 .. 2 NB - 1 at keys 16 c + 8 h32 of its own row: chunk
    // c is accumulator registers 8 (c % 2) .. 8 (c % 2) + 7 of s[c / 2].  The
    // chunks of tile j + 1 are loaded into register slot (j + 1) % 2 at the start
    // of tile j, ahead of that tile's K/V fetch, so the barrier that ends tile j
    // has also completed them.  With an additive bias the scores become the
    // logits s sm_scale + bias, which the softmax takes to the exp2 domain.
    constexpr int BCH = 2 * NB;                      // chunks per lane per tile
    constexpr int BEL = BIAS == kAddBias ? 2 : 1;    // bytes per element
    unsigned bsl[BIAS ? 2 : 1][BIAS ? BCH : 1][bias_dwords<BIAS>()];
    const char* brow = nullptr;
    if constexpr (BIAS != kNoBias) {
      const int r = my_row < t.Lstore ? my_row : t.Lstore - 1;
      brow = (const char*)a.bias + (t.bias_off + (int64_t)r * a.bias_sn) * BEL;
    }
    auto bias_load = [&](int j, auto slot_tag) {
      if constexpr (BIAS != kNoBias)
        bias_chunks<BIAS, BCH>(brow, j * BN + 8 * h32, j * BN + BN <= t.Lkv, t.Lkv, bsl[decltype(slot_tag)::value]);
    };
    // scale of the scores into the exp2 domain at the softmax (log2(e) once
    // an additive bias has made them logits s sm_scale + bias)
    const float cs = BIAS == kAddBias ? kLog2e : a.c;
    // the scale taken with an additive bias (sm_scale 0 as the smallest
    // normal, so that the -inf of masked keys stays -inf rather than 0 * inf)
    const float bscale = a.sm_scale != 0.f ? a.sm_scale : 1.17549435e-38f;
    // the running max lags (see the header); the fp16 JVP keeps it exact
    constexpr bool LAGGED = !(F16 && JVP);
    // fp16 JVP: H = p * (scale tS), the tangent scores scaled before the
    // product as the JVP pages order it, so H stays within fp16's range
    constexpr bool HS = F16 && JVP;

    float m_run = -INFINITY;  // running max, exp2 domain (scores times c)
    float l_run = 0.f;        // this lane's partial row sum (its 16 of every 32 keys)
    float r_run = 0.f;        // JVP: partial rowsum of p * (tQ K^T + Q tK^T) (HS: times scale)
    // how far a tile's max may pass m_run without a rescale (see the header;
    // with C::WAVE_LAG one value for the wave, the smallest of its rows')
    float lag = 0.f;
    // lane-dependent LDS offsets of the K fragments (per head-dim step) and of
    // the V^T fragments (per output column block); tile, block and stage
    // positions are added as immediates.  The swizzle depends on the row mod 16,
    // which 32-key blocks do not change.
    const int krow = kperm(n32);
    uint32_t kaddr[KD];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) kaddr[kk] = lds_g + swz_off<DQK>(krow, 2 * kk + h32);
    int vlo[DB], vhi[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) v_frag_offsets<DVL>(lane, db, vlo[db], vhi[db]);

    // One key tile on LDS stage S = j % 2: fetch tile j + 1 into the other
    // stage (freed by the barrier that ended the previous tile), compute, then
    // one barrier makes tile j + 1 complete and visible.  S is a compile-time
    // constant so every LDS address is a hoisted register plus an immediate.
    auto step = [&](int j, auto stage_tag) {
      constexpr int S = decltype(stage_tag)::value;
      constexpr int SN = S ^ 1;
      const int jt = jbase + j;  // this group's key tile
      const bool ahead = j + 1 < n_mine;
      if (ahead) {  // in flight while this tile computes
        bias_load(jt + 1, std::integral_constant<int, SN>{});
        dma_tile(jt + 1, SN);
      }

      if (j < n_mine && jt * BN < wave_max) {  // wave-uniform: skip tiles this wave cannot see
        const lds_t* vt = smem_g + VBASE + S * VSTR + OFF_V;  // V tile (the cold residual pass reads it)

        // S^T = K Q^T (and the tangent scores tQ K^T + Q tK^T)
        f32x16 s[NB];
        f32x16 ts[JVP ? NB : 1];
        scores_section<DQK, NB, JVP, S * KSTR, S * KSTR + OFF_TK, F16, FDIST>(kaddr, qf, tqf, s, ts);

        // mask keys past this row's limit (ragged tail, causal diagonal,
        // jagged truncation) -- only on tiles that reach some row's limit
        if (jt * BN > wave_min - BN) {
          // key 32 b + 16 (r / 8) + (r % 8) of the lane's block offset
          // jt BN + 8 h32 against the row's limit: one compare with an inline
          // constant per score
          const int lim = my_lim - (jt * BN + 8 * h32);
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * b + 16 * (r >> 3) + (r & 7) >= lim) s[b][r] = -INFINITY;
        }
        if constexpr (BIAS != kNoBias) apply_bias<BIAS, F16, NB, true>(s, bsl[S], bscale);

        // online softmax: the max over this lane's keys of the tile.  A row
        // moves its running max when its tile max (the larger of its two
        // lanes' maxima) passes m_run + lag, i.e. when one of its lanes'
        // maxima does: the wave tests its lanes' own maxima, and only a wave
        // that rescales takes the other half-wave's.  The IEEE maximum (a NaN
        // score propagates) pairs up as one v_maximum3 per two scores with no
        // quieting of its inputs, which fmaxf's NaN rule needs.
        float mx = s[0][0];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, s[b][r]);
        const bool rescaled = __builtin_amdgcn_ballot_w64(mx * cs > m_run + lag) != 0;  // wave-uniform
        if (rescaled) {
          const float m_new = xhalf_max(mx) * cs;
          const bool upd = m_new > m_run + lag;
          const float m_next = upd ? m_new : m_run;
          const float alpha = m_next == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_next);
#pragma unroll
          for (int i = 0; i < DB; ++i) {
            acc[i] *= alpha;
            if constexpr (JVP) { accA[i] *= alpha; accB[i] *= alpha; }
          }
          l_run *= alpha;
          r_run *= alpha;
          m_run = m_next;
        }
        const float msub = m_run == -INFINITY ? 0.f : m_run;

        // Rows that attend at most kSplitKeys keys (short jagged sequences, the
        // first causal rows) follow few keys closely, so |O| can reach max|v|
        // and P's bf16 rounding (2^-9 relative) shows in O: these waves first
        // add V^T Plo^T, Plo = p - bf16(p) being that rounding's residual.  p
        // is recomputed below bit for bit; this pass stays apart from the main
        // product so the latter's code is the same for every wave.
        if (__builtin_expect(wave_max <= kSplitKeys, 0)) {
          float nm = -msub;
          asm volatile("" : "+v"(nm));  // opaque copy: no value here is shared with the main path
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if (jt * BN + 32 * b >= wave_max) break;  // no row of the wave sees this block
            bf16x8 plo[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], cs, nm));
              plo[r >> 3][r & 7] = to16<F16>(p - from16<F16>(to16<F16>(p)));
            }
            pv_lo_block<DVL, F16>(vt, vlo, vhi, b, plo, acc);
          }
        }

        // p = exp2(s c - m); P (and H = p tS) as bf16 B operands: registers
        // 8 c16 .. 8 c16 + 7 of block b are keys 32 b + 16 c16 + 8 h32 + 0..7,
        // i.e. key chunk 2 b + c16 of the PV product.  Chunk 0 is computed
        // first; chunk c+1 is computed in slices after the MFMAs of chunk c.
        bf16x8 pf[NB][2];
        bf16x8 hf[JVP ? NB : 1][2];
        auto soft = [&](auto e_tag) {  // one element e of this lane's 16 NB scores
          constexpr int e = decltype(e_tag)::value, b = e / 16, r = e % 16;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], cs, -msub));
          l_run += p;
          pf[b][r >> 3][r & 7] = to16<F16>(p);
          if constexpr (JVP) {
            const float hv = HS ? p * (ts[b][r] * a.sm_scale) : p * ts[b][r];
            r_run += hv;
            hf[b][r >> 3][r & 7] = to16<F16>(hv);
          }
        };
        constexpr int EPS = 8 / DB;  // elements of the next chunk per PV step
        static_for<8>(soft);
        // O^T += V^T P^T (JVP: accB += V^T H^T, accA += tV^T P^T)
        pv_section<DVL, NB, JVP, S * VSTR + OFF_V, S * VSTR + OFF_TV, F16, FDIST>(
            lds_g + VBASE, vlo, vhi, pf, hf, acc, accA, accB, [&](auto i_tag) {
              constexpr int i = decltype(i_tag)::value, c = i / DB;
              if constexpr (c + 1 < 2 * NB) {
                static_for<EPS>([&](auto k_tag) {
                  soft(std::integral_constant<int, 8 * (c + 1) + (i % DB) * EPS + decltype(k_tag)::value>{});
                });
              }
            });
        // the row's lag, log2(l) - 1 clamped to [0, kTau] (l = 0, no key yet,
        // gives 0), from l_run as it stands after this tile's terms: after a
        // rescale, and on tiles 0, 1, 3, 7, ... (l grows about linearly with
        // the keys seen, so its log2 by about one per doubling)
        if constexpr (LAGGED) {
          if (rescaled || (j & (j + 1)) == 0) {
            const float g = fminf(kTau, fmaxf(0.f, __log2f(xhalf_sum(l_run)) - 1.f));
            lag = C::WAVE_LAG ? wave_min32_nonneg(g) : g;  // lanes l and l ^ 32 share a row
          }
        }
      }

      __syncthreads();
    };

    // The loop sits inside the prologue's branch: on every path into it the
    // Q-fragment loads have completed, so no wait for the next tile's prefetch
    // is needed inside the loop.
    if constexpr (DV < DVL) {
      // the padding chunks of every value tile (both stages, V and tV) are
      // zeroed once: the tile copies never write them, and the barrier after
      // the prologue orders these stores before any fragment read
      constexpr int NVT = JVP ? 2 : 1, PADC = CPR_V - CPR_VS;
      for (int id = tid; id < 2 * NVT * BN * PADC; id += THREADS) {
        const int c = CPR_VS + id % PADC, row = (id / PADC) % BN, st = id / (PADC * BN);
        const int off = VBASE + (st >> 1) * VSTR + ((st & 1) ? OFF_TV : OFF_V) + swz_off<DVL>(row, c);
        *(__attribute__((address_space(3))) u32x4*)(smem + off) = u32x4{0u, 0u, 0u, 0u};
      }
    }

    if (n0 > 0) {
      bias_load(0, std::integral_constant<int, 0>{});
      if (n_mine > 0) dma_tile(jbase, 0);
      __syncthreads();
      int j = 0;
      for (; j + 2 <= n0; j += 2) {
        step(j, std::integral_constant<int, 0>{});
        step(j + 1, std::integral_constant<int, 1>{});
      }
      if (j < n0) step(j, std::integral_constant<int, 0>{});
    }

    // ---- key-split merge: group 1 hands its partial row state (running max,
    // partial sums, accumulators, all relative to its own max) to group 0
    // through LDS, which the loop's last barrier has freed; lane value e sits
    // at float index (e * 4 + wave % 4) * 64 + lane.  Group 0 rescales both
    // parts to the larger max and adds them (the online-softmax merge of two
    // key ranges), then writes the rows.
    if constexpr (SPLIT) {
      typedef __attribute__((address_space(3))) float lds_f;
      lds_f* X = (lds_f*)smem;
      const int sl = (wave & 3) * 64 + lane;
      constexpr int E0 = JVP ? 3 : 2;  // m, l (, r), then the accumulators
      if (grp == 1) {
        X[sl] = m_run;
        X[256 + sl] = l_run;
        if constexpr (JVP) X[512 + sl] = r_run;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            X[(E0 + 16 * db + r) * 256 + sl] = acc[db][r];
            if constexpr (JVP) {
              X[(E0 + 16 * (DB + db) + r) * 256 + sl] = accA[db][r];
              X[(E0 + 16 * (2 * DB + db) + r) * 256 + sl] = accB[db][r];
            }
          }
      }
      __syncthreads();
      if (grp == 0) {
        const float m1 = X[sl];
        const float mm = fmaxf(m_run, m1);
        const float s0 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
        const float s1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        l_run = l_run * s0 + X[256 + sl] * s1;
        if constexpr (JVP) r_run = r_run * s0 + X[512 + sl] * s1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[db][r] = acc[db][r] * s0 + X[(E0 + 16 * db + r) * 256 + sl] * s1;
            if constexpr (JVP) {
              accA[db][r] = accA[db][r] * s0 + X[(E0 + 16 * (DB + db) + r) * 256 + sl] * s1;
              accB[db][r] = accB[db][r] * s0 + X[(E0 + 16 * (2 * DB + db) + r) * 256 + sl] * s1;
            }
          }
        m_run = mm;
      }
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln2, tO = (accA + accB - r O) / l,
    // tLSE = r / l
    // (with 8 waves, by group 0)
    if (!SPLIT || grp == 0) {
      const float l_tot = xhalf_sum(l_run);
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      const float lse = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
      const float r_tot = JVP ? xhalf_sum(r_run) * (HS ? 1.f : a.sm_scale) : 0.f;
      if (my_row < t.Lstore) {
        bf16* orow = (bf16*)a.o + t.o_off + my_row * a.o_sn;
        bf16* torow = JVP ? (bf16*)a.to + t.o_off + my_row * a.o_sn : nullptr;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (32 * db + 8 * g >= DV) continue;  // padding columns of a 16-wide value tile
            const int d = 32 * db + 8 * g + 4 * h32;  // registers 4g..4g+3 are columns d..d+3
            bf16x4 ov;
            bf16x4 tov;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float o = acc[db][4 * g + e] * inv;
              ov[e] = to16<F16>(o);
              if constexpr (JVP)
                tov[e] = to16<F16>((accA[db][4 * g + e] + (HS ? 1.f : a.sm_scale) * accB[db][4 * g + e] - r_tot * o) * inv);
            }
            *(bf16x4*)(orow + d) = ov;
            if constexpr (JVP) *(bf16x4*)(torow + d) = tov;
          }
        if (h32 == 0) a.lse[t.lse_off + my_row] = lse;
        // tangent of LSE: rowsum(P tS) = r / l (0 for a row without keys)
        if constexpr (JVP)
          if (h32 == 0 && a.tlse != nullptr) a.tlse[t.lse_off + my_row] = r_tot * inv;
      }
    }
    // a second query tile's first copies would overwrite the merge area that
    // group 0 has just read
    if (SPLIT && pass + 1 < n_pass) __syncthreads();
  }  // query tile pass
}

}  // namespace attn
