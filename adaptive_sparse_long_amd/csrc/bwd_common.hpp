// bwd_common.hpp -- operand fragments and MFMA building blocks shared by the
// attention backward kernels (the dense alpha-entmax attention's and the
// DashAttention path's): 32-line row blocks held as MFMA operands, products over
// d, accumulation of X^T W^T with X staged transposed in LDS, block visiting
// with prefetch. bf16 operands use v_mfma_f32_32x32x16_bf16 (weights split into
// bf16 high and low parts for float32 accuracy), float32 operands
// v_mfma_f32_32x32x2_f32.
#pragma once

#include "kernels.hpp"

namespace dash {
namespace bwd {
constexpr int kRowPad = 4;
constexpr int kTRow = 32 + kRowPad;  // LDS row of a transposed 32-line block (elements)

template <bool BF, int D>
struct Frags {
  static constexpr int NS = BF ? D / 16 : D / 2;
  bf16x8 b[BF ? NS : 1];
  float f[BF ? 1 : NS];
};

// Operand fragments of one row (row index valid < n_ok, else zeros): bf16 rows
// give 8 elements per k-step at d = 16 s + 8 (lane / 32); float rows one
// element at d = 2 s + lane / 32. DC: the rows' width in memory when it is
// smaller than the fragments' D (head_dim 64 in a 128-wide layout): the dims
// from DC on are zero.
template <bool BF, int D, int DC = D>
__device__ __forceinline__ void load_frags(Frags<BF, D>& fr, const void* base, int row, bool ok) {
  const int hi32 = lane_id() >> 5;
  if constexpr (BF) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + (size_t)row * DC + 8 * hi32;
#pragma unroll
    for (int s = 0; s < Frags<BF, D>::NS; ++s)
      fr.b[s] = as_bf16x8(ok && 16 * s < DC ? ldg16(p + 16 * s) : u32x4{0, 0, 0, 0});
  } else {
    const float* p = static_cast<const float*>(base) + (size_t)row * DC + hi32;
#pragma unroll
    for (int s = 0; s < Frags<BF, D>::NS; ++s) fr.f[s] = ok && 2 * s < DC ? p[2 * s] : 0.f;
  }
}

// C[m][n] = sum_d A_m[d] B_n[d] for the 32 rows held by A and the 32 held by B.
template <bool BF, int D>
__device__ __forceinline__ f32x16 dot32(const Frags<BF, D>& A, const Frags<BF, D>& B) {
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = 0.f;
#pragma unroll
  for (int s = 0; s < Frags<BF, D>::NS; ++s) {
    if constexpr (BF) c = mfma32x32x16(A.b[s], B.b[s], c);
    else c = mfma32x32x2f32(A.f[s], B.f[s], c);
  }
  return c;
}

// acc[db] (C[m = dim 32 db + .][n = lane's line]) += X^T W^T over the block's 32
// lines, where W^T is this lane's column w (acc layout: line 8 (r/4) + 4 (l/32)
// + r%4 of register r) and X the block's rows: bf16 from the transposed LDS
// copy xt with W split into bf16 high and low parts (float32 accuracy; SPLIT
// false for weights that bf16 holds exactly), float32 straight from memory
// (rows >= n_ok contribute zeros).
template <bool BF, int D, bool SPLIT = true>
__device__ __forceinline__ void acc_xt_w(f32x16 (&acc)[D / 32], const f32x16& w, const uint16_t* xt,
                                         const float* X, int r0, int n_ok) {
  const int lane = lane_id();
  const int hi32 = lane >> 5;
  if constexpr (BF) {
    bf16x8 wh[2], wl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = w[8 * ks + 2 * e], a1 = w[8 * ks + 2 * e + 1];
        h[e] = pack_bf16x2(a0, a1);
        if constexpr (SPLIT) l[e] = pack_bf16x2(a0 - bf16lo(h[e]), a1 - bf16hi(h[e]));
      }
      wh[ks] = as_bf16x8(h);
      wl[ks] = as_bf16x8(l);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint16_t* xrow = xt + (32 * db + (lane & 31)) * kTRow + 4 * hi32;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x2 lo = *reinterpret_cast<const u32x2*>(xrow + 16 * ks);
        u32x2 hi = *reinterpret_cast<const u32x2*>(xrow + 16 * ks + 8);
        const bf16x8 xa = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        acc[db] = mfma32x32x16(xa, wh[ks], acc[db]);
        if constexpr (SPLIT) acc[db] = mfma32x32x16(xa, wl[ks], acc[db]);
      }
    }
  } else {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int line = r0 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
        const float x = line < n_ok ? X[(size_t)line * D + 32 * db + (lane & 31)] : 0.f;
        acc[db] = mfma32x32x2f32(x, w[r], acc[db]);
      }
    }
  }
}

// Write the lane's line of acc (dims 32 db + 8 q4 + 4 (l/32) + 0..3) times mul;
// lines DC wide (dims from DC on are not written).
template <bool BF, int D, int DC = D>
__device__ __forceinline__ void store_line(void* out, size_t line, const f32x16 (&acc)[D / 32], float mul) {
  const int hi32 = lane_id() >> 5;
  if constexpr (BF) {
    uint16_t* op = static_cast<uint16_t*>(out) + line * DC + 4 * hi32;
#pragma unroll
    for (int db = 0; db < DC / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 v = {pack_bf16x2(acc[db][4 * q4] * mul, acc[db][4 * q4 + 1] * mul),
                   pack_bf16x2(acc[db][4 * q4 + 2] * mul, acc[db][4 * q4 + 3] * mul)};
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * q4) = v;
      }
  } else {
    float* op = static_cast<float*>(out) + line * DC + 4 * hi32;
#pragma unroll
    for (int db = 0; db < DC / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v = {acc[db][4 * q4] * mul, acc[db][4 * q4 + 1] * mul, acc[db][4 * q4 + 2] * mul,
                   acc[db][4 * q4 + 3] * mul};
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * q4) = v;
      }
  }
}

// Register-set index of a prefetching pass, as a type so that every access to
// the two sets is static (a run-time index would put them in scratch memory).
template <int S>
struct Slot {
  static constexpr int v = S;
};

// Visit the 32-line blocks b0 <= blk < n of a pass whose 64 x 64 tile is on
// (bit (blk / 2) of the mask row `bits`, or every block when bits is null),
// in order. bfloat16 passes load the next block's operands while the current
// one is computed (load(blk, Slot) fills one of two register sets; a block at n
// loads zeros without touching memory); float32 passes (twice the registers)
// load each block when it is reached.
template <bool PF, typename Load, typename Body>
__device__ __forceinline__ void visit_blocks(int b0, int n, const uint32_t* bits, Load load, Body body) {
  auto next = [&](int blk) {
    if (!bits) return min(blk, n);
    while (blk < n) {
      const int t = blk >> 1;
      const uint32_t w = bits[t >> 5] >> (t & 31);
      if (w & 1u) return blk;
      blk = w ? 2 * (t + (int)__builtin_ctz(w)) : 2 * ((t | 31) + 1);
    }
    return n;
  };
  int blk = next(b0);
  if constexpr (PF) {
    load(blk, Slot<0>{});
    while (blk < n) {
      int nb = next(blk + 1);
      load(nb, Slot<1>{});
      body(blk, Slot<0>{});
      blk = nb;
      if (blk >= n) break;
      nb = next(blk + 1);
      load(nb, Slot<0>{});
      body(blk, Slot<1>{});
      blk = nb;
    }
  } else {
    while (blk < n) {
      load(blk, Slot<0>{});
      body(blk, Slot<0>{});
      blk = next(blk + 1);
    }
  }
}

// Stage a 32-row bf16 block held as fragments (lane: row R = lane % 32, dims
// 16 s + 8 (lane / 32) + e) transposed into xt[D][kTRow]. Neighbouring lanes
// (rows R, R ^ 1) swap each 32-bit pair of dims through DPP, so every store
// writes two rows of one dim: the even lane dim 2e' of rows (R, R + 1), the odd
// lane dim 2e' + 1 of rows (R - 1, R).
template <int D>
__device__ __forceinline__ void stage_t_regs(uint16_t* xt, const Frags<true, D>& fr) {
  const int lane = lane_id();
  const int odd = lane & 1;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
  uint16_t* base = xt + (8 * (lane >> 5) + odd) * kTRow + (lane & 30);
#pragma unroll
  for (int s = 0; s < Frags<true, D>::NS; ++s) {
    const u32x4 v = __builtin_bit_cast(u32x4, fr.b[s]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[e], kDppXor1, 0xF, 0xF, false);
      *reinterpret_cast<uint32_t*>(base + (16 * s + 2 * e) * kTRow) = __builtin_amdgcn_perm(w, v[e], sel);
    }
  }
}

}  // namespace bwd
}  // namespace dash
