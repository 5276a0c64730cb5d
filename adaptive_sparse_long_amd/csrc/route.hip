// route.hip -- stage 2 of the DashAttention hierarchy ("How it works" 2 on the
// DashAttention README page): query-to-summary routing scores, alpha-entmax over
// them (threshold by Halley + bisection, AdaSplash README "Usage: Triton
// Entmax"), the routed set (the entmax support) and the routing prior, packed as
// work lists for the stage-3 attention kernels.
//
// Prefill: k_split_summaries scales the float32 summaries into u units and
// splits them into bf16 high and low parts once per call. k_route_fast, one
// workgroup of four wavefronts (32 rows each) per (b, query head, 128-row
// tile), computes the scores with v_mfma_f32_32x32x16_bf16 on both parts (q is
// exact in bf16, so about 16 mantissa bits reach the fp32 accumulator) in two
// passes over the summaries staged through LDS: the high parts alone bound
// each row's max from below, then the exact scores above that bound - 1 (the
// only ones that can carry weight) go into an LDS list; tau, the routed set and
// the work for stage 3 follow from the list. A 2048-slot form of the same
// kernel serves N up to 131072. Tiles whose list or chunk union does not fit
// are queued for k_route_prefill, the general kernel: eight wavefronts of 16
// rows keep every score (registers up to 512 chunk slots, a per-workgroup
// global scratch beyond), per-row LDS candidate lists, tau in a four-lanes-per-
// row layout.
//
// Decode: a bandwidth-bound score kernel streams the float32 summary cache once
// (eight lanes per summary row, four float4 loads each, all g query heads of a
// KV head at once), then one workgroup per (b, kv head) solves tau for its g
// query heads (one wavefront each, 32+ candidates per lane), takes the union of
// their routed chunks and writes the list with g log2 priors per chunk.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"
#include "tau_solve.hpp"

namespace dash {

namespace {

__device__ __forceinline__ u32x4 zero4() { return u32x4{0, 0, 0, 0}; }

// Split 8 float32 values into bf16 high parts and bf16 low parts (x - hi).
__device__ __forceinline__ void split_hi_lo(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float h0 = round_bf16(x[2 * e]);
    float h1 = round_bf16(x[2 * e + 1]);
    h[e] = pack_bf16x2(h0, h1);
    l[e] = pack_bf16x2(x[2 * e] - h0, x[2 * e + 1] - h1);
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

__device__ __forceinline__ float dot8_bf16(const u32x4& v, const float* w) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = fmaf(bf16lo(v[e]), w[2 * e], s);
    s = fmaf(bf16hi(v[e]), w[2 * e + 1], s);
  }
  return s;
}

}  // namespace

// ============================================================================
// Prefill routing
// ============================================================================
// One workgroup per tile of the grid; the first ones take the tiles the
// list-based kernel queued, the rest return at once.
// One queued tile q. GLB: the scores live in this workgroup's part of a global
// scratch (eight wavefronts x NB blocks x 4 x 64 floats) instead of registers,
// for more chunks than registers hold.
template <int NB, int KIND, bool GLB>
__device__ __forceinline__ void route_general_tile(const RouteArgs& a, int q) {
  constexpr int D = 128;
  constexpr int NS = D / 32;                // k-steps of the 16x16x32 MFMA
  constexpr int NW = (NB * 16 + 31) / 32;   // union words
  constexpr int NBR = GLB ? 1 : NB;         // score blocks in registers
  // Split summaries of 64 chunks per stage, shared by the eight wavefronts:
  // per chunk 128 high parts, 128 low parts and 8 bf16 of padding (a chunk
  // stride of 132 dwords keeps eight consecutive lanes on distinct LDS banks).
  constexpr int SROW = 2 * D + 8;
  // After the scores the same LDS holds the per-row candidate lists: per
  // wavefront 16 rows of LROW scores (float) and LROW chunk ids (uint16).
  constexpr int LROW = kRouteCap + 4;
  constexpr int kStageHalves = 2 * 64 * SROW;
  constexpr int kListHalves = 8 * 16 * LROW * 3;
  __shared__ __attribute__((aligned(16))) uint16_t s_big[kStageHalves > kListHalves ? kStageHalves : kListHalves];
  uint16_t (*const sS)[64 * SROW] = reinterpret_cast<uint16_t (*)[64 * SROW]>(s_big);
  __shared__ uint32_t s_union[NW], s_cunion[NW];  // attended chunks: row-major, chunk-major list
  __shared__ int s_pre[NW + 1], s_cpre[NW + 1];
  __shared__ int s_ecnt[NW * 32];  // chunk-major entries: rows taking the chunk,
  __shared__ int s_cl[NW * 32];    // the chunk,
  __shared__ int s_eoff[NW * 32];  // first record in the tile's pool range,
  __shared__ int s_efill[NW * 32]; // records written so far
  __shared__ int s_wtot[8];        // attended chunks of each wavefront's rows
  __shared__ int s_tmp[8];
  __shared__ long long s_tbase;    // the tile's first pool slot, -1: none

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int tile = a.fb_tiles[q].x;
  const int h = a.fb_tiles[q].y % a.Hq;
  const int b = a.fb_tiles[q].y / a.Hq;
  const int hk = h / a.g;
  const int N = a.Nq;
  const int i0 = tile * kTileRows + w * 16;  // first row of this wavefront
  const int cw = i0 / kChunk;                // own (diagonal) chunk of all 16 rows
  const bool wave_valid = i0 < N;
  const int col = lane % 16;                 // B column / D column: the chunk in a block
  const int grp = lane / 16;                 // D-layout row group: rows grp*4 + r
  const bool causal = a.causal != 0;
  const bool est = causal && a.est != 0;
  const int n_slots = a.n_slots;
  // complete-chunk candidates of this wavefront's rows
  const int ncomp = wave_valid ? (causal ? cw : n_slots) : 0;
  const int nblk = (ncomp + 15) / 16;
  const int ncand = ncomp + (est ? 1 : 0);
  const size_t bh = (size_t)b * a.Hq + h;
  const size_t sbase = ((size_t)b * a.Hkv + hk) * (size_t)n_slots * D;
  for (int e = threadIdx.x; e < NW * 32; e += blockDim.x) {
    s_ecnt[e] = 0;
    s_efill[e] = 0;
  }
  if (threadIdx.x < NW) {
    s_union[threadIdx.x] = 0u;
    s_cunion[threadIdx.x] = 0u;
  }

  // ---- q as A operand: row i0 + col, dims 32 s + 8 grp .. +7
  bf16x8 qa[NS];
  {
    const int qi = min(i0 + col, N - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) qa[s] = as_bf16x8(ldg16_d(a.Q, bh * N + qi, 32 * s + 8 * grp, a.d));
  }

  // ---- routing scores in u units, u[blk][r]: chunk blk*16 + col, row grp*4 + r.
  // Groups of four blocks (64 chunks) pass through LDS: all 512 threads load a
  // group once (the next group's loads in flight while the current one is
  // multiplied), then every wavefront reads its B operands from LDS.
  const float uscale = (a.alpha - 1.f) * a.zscale;
  float u[NBR][4];
  float* const gu = GLB ? a.gscr + ((size_t)blockIdx.x * 8 + w) * (size_t)(NB * 4 * kWave) : nullptr;
  // score of row grp*4 + r for chunk blk*16 + col
  auto UV = [&](int blk, int r) -> float {
    if constexpr (GLB) return gu[(blk * 4 + r) * kWave + lane];
    else return u[blk][r];
  };
  auto USET = [&](int blk, int r, float v) {
    if constexpr (GLB) gu[(blk * 4 + r) * kWave + lane] = v;
    else u[blk][r] = v;
  };
  const int nbl = GLB ? nblk : NB;  // blocks the loops below visit
  const int last_row = min(tile * kTileRows + kTileRows, N) - 1;
  const int ncomp_wg = causal ? last_row / kChunk : n_slots;  // most chunks any wavefront scores
  const int ngrp = (ncomp_wg + 63) / 64;
  const int tid = threadIdx.x;
  u32x4 gl[4];
  auto load_grp = [&](int gi) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = tid + 512 * k;  // 2048 segments of 16 bytes
      const int ch = idx >> 5;        // chunk within the group
      const int part = idx & 31;      // 0..15 high, 16..31 low
      const int c = min(gi * 64 + ch, max(ncomp_wg - 1, 0));
      const uint16_t* src = (part < 16 ? a.s_hi : a.s_lo) + sbase + (size_t)c * D + 8 * (part & 15);
      gl[k] = ldg16(src);
    }
  };
  auto store_grp = [&](int stage) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = tid + 512 * k;
      const int ch = idx >> 5;
      const int part = idx & 31;
      *reinterpret_cast<u32x4*>(&sS[stage][ch * SROW + (part < 16 ? 0 : D) + 8 * (part & 15)]) = gl[k];
    }
  };
  if (ngrp > 0) {
    load_grp(0);
    store_grp(0);
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < (GLB ? ngrp : (NB + 3) / 4); ++gi) {
    if (gi < ngrp) {  // uniform over the workgroup
      const bool more = gi + 1 < ngrp;
      if (more) load_grp(gi + 1);
      const uint16_t* base = &sS[gi & 1][col * SROW + 8 * grp];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = gi * 4 + j;
        if (blk < NB) {
          if (blk < nblk) {
            const uint16_t* bp = base + j * 16 * SROW;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              acc = mfma16x16x32(qa[s], *reinterpret_cast<const bf16x8*>(bp + 32 * s), acc);
              acc = mfma16x16x32(qa[s], *reinterpret_cast<const bf16x8*>(bp + D + 32 * s), acc);
            }
            // the summaries are pre-scaled: acc is u. Only the last block can
            // hold columns past the candidates.
            const bool cval = blk < nblk - 1 || blk * 16 + col < ncomp;
#pragma unroll
            for (int r = 0; r < 4; ++r) USET(blk, r, cval ? acc[r] : -INFINITY);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) USET(blk, r, -INFINITY);
          }
        }
      }
      if (more) store_grp((gi + 1) & 1);
      __syncthreads();
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = gi * 4 + j;
        if (blk < NBR) {
#pragma unroll
          for (int r = 0; r < 4; ++r) u[blk][r] = -INFINITY;
        }
      }
    }
  }

  // ---- own-chunk estimate: score against the summary of tokens [cw*C, i]
  float ud[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (est && wave_valid) {
    const size_t krow0 = ((size_t)b * a.Hkv + hk) * a.Lmax + (size_t)cw * kChunk;
    float wc[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 cv = ldg16_d(a.cls, hk, 32 * s + 8 * grp, a.d);
      for (int e = 0; e < 4; ++e) {
        wc[s][2 * e] = bf16lo(cv[e]);
        wc[s][2 * e + 1] = bf16hi(cv[e]);
      }
    }
    f32x4 qk[4];
    float lc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(kb * 16 + col, N - 1 - cw * kChunk);  // stays inside the sequence
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 kv = ldg16_d(a.K, krow0 + key, 32 * s + 8 * grp, a.d);
        acc = mfma16x16x32(qa[s], as_bf16x8(kv), acc);
        part += dot8_bf16(kv, wc[s]);
      }
      qk[kb] = acc;
      lc[kb] = sum_xor32(sum_xor16(part)) * a.inv_sqrt_d;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pi = i0 + grp * 4 + r - cw * kChunk;  // position of the row in its chunk
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mloc = kb * 16 + col <= pi ? fmaxf(mloc, lc[kb]) : mloc;
      const float M = max16(mloc);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float e = kb * 16 + col <= pi ? fast_exp2((lc[kb] - M) * kLog2e) : 0.f;
        num = fmaf(e, qk[kb][r], num);
        den += e;
      }
      ud[r] = (sum16(num) / sum16(den)) * uscale;
    }
  }

  // ---- tau per row. Only scores above max u - 1 can carry weight (tau >=
  // max u - 1): each row's candidates, usually a handful, are gathered in
  // ascending chunk order into an LDS list (in the summary staging, no longer
  // read). A wavefront whose lists all fit solves tau and emits its rows' work
  // in a row layout, four lanes per row; a wavefront with a row of more than
  // kRouteCap candidates solves tau and emits from all its blocks.
  bool row_ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) row_ok[r] = wave_valid && (i0 + grp * 4 + r < N);
  auto seg_of = [&](unsigned long long m) { return (uint32_t)(m >> (16 * grp)) & 0xffffu; };
  const uint32_t below = (1u << col) - 1u;
  float* const s_cu = reinterpret_cast<float*>(s_big) + (size_t)w * 16 * LROW;
  uint16_t* const s_cc = s_big + 2 * 8 * 16 * LROW + (size_t)w * 16 * LROW;
  float mx[4], lo[4];
  int nc[4] = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float m = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < nbl; ++blk) m = fmaxf(m, UV(blk, r));
    mx[r] = fmaxf(max16(m), ud[r]);  // -inf: no candidate at all
    lo[r] = mx[r] - 1.f;
  }
#pragma unroll
  for (int blk = 0; blk < nbl; ++blk) {
    if (blk < nblk) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ub = UV(blk, r);
        const bool cnd = ub > lo[r];
        const unsigned long long m = __ballot(cnd);
        if (m != 0ull) {
          const uint32_t seg = seg_of(m);
          const int pos = nc[r] + __popc(seg & below);
          if (cnd && pos < kRouteCap) {
            s_cu[(grp * 4 + r) * LROW + pos] = ub;
            s_cc[(grp * 4 + r) * LROW + pos] = (uint16_t)(blk * 16 + col);
          }
          nc[r] += __popc(seg);
        }
      }
    }
  }
  const bool ovf = wave_any(nc[0] > kRouteCap || nc[1] > kRouteCap || nc[2] > kRouteCap || nc[3] > kRouteCap);
  wave_lds_fence();

  // row layout: lanes 4 rr .. 4 rr + 3 hold row i0 + rr, lane sub the list
  // positions 4 k + sub
  const int rr = lane >> 2, sub = lane & 3;
  auto to_row = [&](const float (&x)[4]) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float t = __shfl(x[r], (rr >> 2) * 16);
      v = (rr & 3) == r ? t : v;
    }
    return v;
  };
  float ncf[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) ncf[r] = (float)nc[r];
  const float mx_r = to_row(mx), ud_r = to_row(ud);
  const int nc_r = (int)to_row(ncf);
  const bool row_ok_r = wave_valid && i0 + rr < N;
  int kmax = 0;  // list steps of the wavefront (its longest list / 4)
  auto cand = [&](int k) {  // list position 4 k + sub of the lane's row, -inf past its end
    const int p = 4 * k + sub;
    return p < nc_r ? s_cu[rr * LROW + p] : -INFINITY;
  };
  float tau_r = INFINITY;
  float tau[4];
  auto solve = [&](auto&& terms, float (&t)[4], float (&lo4)[4], float (&hi4)[4], auto&& reduce, int nrows) {
    for (int it = 0; it < a.n_iter; ++it) {
      float f0[4] = {0.f, 0.f, 0.f, 0.f}, f1[4] = {0.f, 0.f, 0.f, 0.f}, f2[4] = {0.f, 0.f, 0.f, 0.f};
      terms(f0, f1, f2);
      bool conv = true;
      for (int r = 0; r < nrows; ++r) {
        f0[r] = reduce(f0[r]);
        f1[r] = reduce(f1[r]);
        if (KIND != 1) f2[r] = reduce(f2[r]);
        const float udr = nrows == 1 ? ud_r : ud[r];
        if (est) tau_terms<KIND>(udr, t[r], a.beta, f0[r], f1[r], f2[r]);
        const float nt = tau_step<KIND>(t[r], f0[r], f1[r], f2[r], a.beta, lo4[r], hi4[r]);
        conv = conv && (tau_converged(t[r], nt) || !(t[r] > -INFINITY));
        t[r] = nt;
      }
      if (wave_all(conv)) break;
    }
  };
  if (!ovf) {
    kmax = (int)wave_max((float)((min(nc_r, kRouteCap) + 3) >> 2));
    // tau <= max - n^-(alpha-1), n the values above tau: all among the candidates
    float t1[4] = {mx_r - 1.f, 0.f, 0.f, 0.f};
    float lo1[4] = {mx_r - 1.f, 0.f, 0.f, 0.f};
    float hi1[4] = {tau_upper(mx_r, max(1, nc_r + ((est && ud_r > mx_r - 1.f) ? 1 : 0)), a.alpha), 0.f, 0.f, 0.f};
    solve([&](float (&f0)[4], float (&f1)[4], float (&f2)[4]) {
            for (int k = 0; k < kmax; ++k) tau_terms<KIND>(cand(k), t1[0], a.beta, f0[0], f1[0], f2[0]);
          },
          t1, lo1, hi1,
          [](float x) {  // sum over the row's four lanes
            const float y = x + dpp_f<kDppXor1>(x);
            return y + dpp_f<kDppXor2>(y);
          },
          1);
    tau_r = mx_r > -INFINITY ? t1[0] : INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) tau[r] = __shfl(tau_r, (grp * 4 + r) * 4);
  } else {
    float hi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hi[r] = tau_upper(mx[r], max(ncand, 1), a.alpha);
      tau[r] = lo[r];
    }
    // blocks holding none of the candidates are left out of the iterations
    uint32_t live = ~0u;
    if constexpr (!GLB) {
      live = 0u;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const bool any = (u[blk][0] > lo[0]) || (u[blk][1] > lo[1]) || (u[blk][2] > lo[2]) || (u[blk][3] > lo[3]);
        live |= wave_any(any) ? (1u << blk) : 0u;
      }
    }
    solve([&](float (&f0)[4], float (&f1)[4], float (&f2)[4]) {
#pragma unroll
            for (int blk = 0; blk < nbl; ++blk) {
              if (GLB || ((live >> blk) & 1u)) {
#pragma unroll
                for (int r = 0; r < 4; ++r) tau_terms<KIND>(UV(blk, r), tau[r], a.beta, f0[r], f1[r], f2[r]);
              }
            }
          },
          tau, lo, hi, [](float x) { return sum16(x); }, 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) tau[r] = mx[r] > -INFINITY ? tau[r] : INFINITY;
  }

  // ---- tau output: lanes 0, 16, 32, 48 hold rows grp*4 .. +3
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row_ok[r]) a.tau[bh * (size_t)N + i0 + grp * 4 + r] = tau[r];
  }

  // ---- own chunk: routed (estimate) or always attended with weight 1
  bool dact[4];
  float lwd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float td = ud[r] - tau[r];
    dact[r] = row_ok[r] && (est ? (td > 0.f) : causal);
    lwd[r] = !row_ok[r] ? -INFINITY : (est ? (td > 0.f ? log2_prior<KIND>(td, a.beta) : -INFINITY) : 0.f);
  }

  // ---- per-row bitmask output, only when asked for (lanes 0..15: row i0 + lane)
  if (a.bits != nullptr) {
    unsigned long long md[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) md[r] = __ballot(dact[r]);
    const bool write_bits = wave_valid && lane < 16 && i0 + lane < N;
    const int rg = lane >> 2, r4 = lane & 3;  // D-layout owner of row `lane`
    const bool dl = ((r4 == 0 ? md[0] : r4 == 1 ? md[1] : r4 == 2 ? md[2] : md[3]) >> (16 * rg)) & 1ull;
    uint32_t* bdst = a.bits + ((bh * (size_t)N) + min(i0 + lane, N - 1)) * (size_t)a.bits_words;
#pragma unroll
    for (int wd = 0; wd < NW; ++wd) {
      uint32_t word = 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int blk = 2 * wd + half;
        if (blk < nbl) {
          unsigned long long mb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) mb[r] = __ballot(row_ok[r] && UV(blk, r) > tau[r]);
          const unsigned long long mr = r4 == 0 ? mb[0] : r4 == 1 ? mb[1] : r4 == 2 ? mb[2] : mb[3];
          word |= (uint32_t)((mr >> (16 * rg)) & 0xffffull) << (16 * half);
        }
      }
      if (causal && dl && (cw >> 5) == wd) word |= 1u << (cw & 31);
      if (write_bits && wd < a.bits_words) bdst[wd] = word;
    }
    if (write_bits)
      for (int wd = NW; wd < a.bits_words; ++wd) bdst[wd] = 0u;
  }

  // ---- the routed past chunks of the wavefront's rows, in ascending chunk
  // order per row, from the lists (row layout) or from all blocks (block
  // layout, wavefronts with an overflowing list). Called by the whole
  // wavefront; afterwards the running counts hold each row's number of routed
  // past chunks.
  //   row layout: fn(chunk, rank, u) for this lane's row rr;
  int run_r = 0;
  auto for_each_routed_row = [&](auto&& fn) {
    run_r = 0;
    for (int k = 0; k < kmax; ++k) {
      const float uk = cand(k);
      const bool act = row_ok_r && uk > tau_r;
      const uint32_t q = (uint32_t)(__ballot(act) >> (4 * rr)) & 0xfu;
      const int rank = run_r + __popc(q & ((1u << sub) - 1u));
      run_r += __popc(q);
      if (act) fn((int)s_cc[rr * LROW + 4 * k + sub], rank, uk);
    }
  };
  //   block layout: fn(r, chunk, rank, u) for this lane's rows grp*4 + r.
  int run4[4] = {0, 0, 0, 0};
  auto for_each_routed_blk = [&](auto&& fn) {
#pragma unroll
    for (int r = 0; r < 4; ++r) run4[r] = 0;
#pragma unroll
    for (int blk = 0; blk < nbl; ++blk) {
      if (blk < nblk) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ub = UV(blk, r);
          const bool act = row_ok[r] && ub > tau[r];
          const uint32_t seg = seg_of(__ballot(act));
          const int rank = run4[r] + __popc(seg & below);
          run4[r] += __popc(seg);
          if (act) fn(r, blk * 16 + col, rank, ub);
        }
      }
    }
  };

  // ---- pool slots: one per attended chunk (routed past chunks, then the own
  // chunk) of every row of the tile, taken with one atomic; the slots of a row
  // are consecutive, in chunk order. Rows are numbered (wavefront, row in
  // wavefront) inside the tile.
  int nsl_r = 0, row_pre = 0;          // row layout: slots of the row, slots of the rows before it
  int nsl4[4] = {0, 0, 0, 0}, pre4[4] = {0, 0, 0, 0};  // block layout
  if (!ovf) {
    for_each_routed_row([](int, int, float) {});
    nsl_r = run_r;
    int x = sub == 0 ? nsl_r : 0;
    const int x0 = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      x += lane >= off ? y : 0;
    }
    row_pre = __shfl(x - x0, 4 * rr);
    if (lane == kWave - 1) s_wtot[w] = x;
  } else {
    for_each_routed_blk([](int, int, int, float) {});
#pragma unroll
    for (int r = 0; r < 4; ++r) nsl4[r] = run4[r];
    const int grp_tot = nsl4[0] + nsl4[1] + nsl4[2] + nsl4[3];
    const int g0 = __builtin_amdgcn_readlane(grp_tot, 0), g1 = __builtin_amdgcn_readlane(grp_tot, 16);
    const int g2 = __builtin_amdgcn_readlane(grp_tot, 32), g3 = __builtin_amdgcn_readlane(grp_tot, 48);
    pre4[0] = (grp > 0 ? g0 : 0) + (grp > 1 ? g1 : 0) + (grp > 2 ? g2 : 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) pre4[r] = pre4[r - 1] + nsl4[r - 1];
    if (lane == 0) s_wtot[w] = g0 + g1 + g2 + g3;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) tot += s_wtot[ww];
    long long base = 0;  // a tile without routed past chunks needs no slots
    if (tot > 0) {
      // the workgroup's part of the pool
      const int part = (int)((tile + (size_t)a.n_tiles * (h + (size_t)a.Hq * b)) % kPools);
      const unsigned long long cap = (unsigned long long)a.pool_cap / kPools;
      const unsigned long long got = atomicAdd(&a.pool[part], (unsigned long long)tot);
      base = got + (unsigned long long)tot <= cap ? (long long)(part * cap + got) : -1;
    }
    s_tbase = base;
    a.tbase[bh * a.n_tiles + tile] = base >= 0 ? (uint32_t)base : 0u;
  }
  __syncthreads();
  const bool pooled = s_tbase >= 0;  // uniform: chunk-major for every routed past chunk
  if (threadIdx.x == 0 && !pooled) atomicAdd(a.n_rm, 1);
  const long long tb = s_tbase;
  int wpre = 0;
#pragma unroll
  for (int ww = 0; ww < 8; ++ww) wpre += ww < w ? s_wtot[ww] : 0;
  // own-chunk log2 weight per row (the merge kernel attends it for pooled tiles)
  if (causal && col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row_ok[r]) a.own_lw[bh * (size_t)N + i0 + grp * 4 + r] = lwd[r];
  }
  if (!ovf) {
    if (sub == 0 && row_ok_r) {
      const size_t ri = bh * (size_t)N + i0 + rr;
      a.cmcnt[ri] = pooled ? (uint16_t)nsl_r : (uint16_t)0;
      a.rslot[ri] = pooled ? (uint32_t)(tb + wpre + row_pre) : 0u;
    }
  } else if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row_ok[r]) {
        const size_t ri = bh * (size_t)N + i0 + grp * 4 + r;
        a.cmcnt[ri] = pooled ? (uint16_t)nsl4[r] : (uint16_t)0;
        a.rslot[ri] = pooled ? (uint32_t)(tb + wpre + pre4[r]) : 0u;
      }
  }

  // ---- the tile's attended chunks: chunk-major list if pooled, else row-major
  uint32_t* const un = pooled ? s_cunion : s_union;
  if (!ovf && pooled) {
    for_each_routed_row([&](int c, int, float) { atomicOr(&un[c >> 5], 1u << (c & 31)); });
  } else {
    for_each_routed_blk([&](int, int c, int, float) { atomicOr(&un[c >> 5], 1u << (c & 31)); });
  }
  if (!pooled && causal && col == 0 && (dact[0] || dact[1] || dact[2] || dact[3])) atomicOr(&un[cw >> 5], 1u << (cw & 31));
  __syncthreads();
  if (threadIdx.x == 0 || threadIdx.x == kWave) {
    const bool cm = threadIdx.x != 0;
    const uint32_t* u2 = cm ? s_cunion : s_union;
    int* pre = cm ? s_cpre : s_pre;
    int acc = 0;
    for (int wd = 0; wd < NW; ++wd) {
      pre[wd] = acc;
      acc += __popc(u2[wd]);
    }
    pre[NW] = acc;
    (cm ? a.ccounts : a.counts)[bh * a.n_tiles + tile] = acc;
  }
  __syncthreads();
  const long long toff = bh * a.per_head + prefill_tile_offset(tile, n_slots, causal);
  if (threadIdx.x < 2 * NW) {
    const bool cm = threadIdx.x >= NW;
    const int wd = threadIdx.x % NW;
    uint32_t bits = cm ? s_cunion[wd] : s_union[wd];
    int pos = cm ? s_cpre[wd] : s_pre[wd];
    int* lst = (cm ? a.clists : a.lists) + toff;
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      if (cm) s_cl[pos] = wd * 32 + bpos;
      lst[pos++] = wd * 32 + bpos;
      bits &= bits - 1u;
    }
  }
  // list position of chunk c
  const int* const pre = pooled ? s_cpre : s_pre;
  auto epos = [&](int c) { return pre[c >> 5] + __popc(un[c >> 5] & ((1u << (c & 31)) - 1u)); };
  const int hh = h % a.g;

  if (pooled) {
    // ---- pair records, grouped by chunk in the tile's pool range: count the
    // rows of every entry, place the entries, then write the records
    if (!ovf) {
      for_each_routed_row([&](int c, int, float) { atomicAdd(&s_ecnt[epos(c)], 1); });
    } else {
      for_each_routed_blk([&](int, int c, int, float) { atomicAdd(&s_ecnt[epos(c)], 1); });
    }
    __syncthreads();
    const int ne = s_cpre[NW];
    int* cmp = a.cmp + ((size_t)b * a.Hkv + hk) * n_slots;
    int first = 0;
    // entries EPT t .. EPT t + EPT - 1 per thread
    constexpr int EPT = (NW * 32 + 511) / 512;
    int esum = 0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = EPT * (int)threadIdx.x + k;
      esum += e < ne ? s_ecnt[e] : 0;
    }
    block_excl_scan<8>(esum, s_tmp, first);
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = EPT * (int)threadIdx.x + k;
      if (e < ne) {
        const int cnt_e = s_ecnt[e];
        s_eoff[e] = first;
        a.ceo[toff + e] = make_int2(first, cnt_e);
        // the entry's pairs among all pairs of its chunk
        a.cbase[toff + e] = atomicAdd(&cmp[s_cl[e]], cnt_e);
        first += cnt_e;
      }
    }
    __syncthreads();
    auto put = [&](int e, int row, long long slot, float lw) {
      const int j = atomicAdd(&s_efill[e], 1);
      a.trec[tb + s_eoff[e] + j] = make_int4(row * a.g + hh, (int)slot, __float_as_int(lw), 0);
    };
    if (!ovf) {
      const long long s0 = tb + wpre + row_pre;
      for_each_routed_row([&](int c, int rank, float uu) {
        put(epos(c), i0 + rr, s0 + rank, log2_prior<KIND>(uu - tau_r, a.beta));
      });
    } else {
      for_each_routed_blk([&](int r, int c, int rank, float uu) {
        put(epos(c), i0 + grp * 4 + r, tb + wpre + pre4[r] + rank, log2_prior<KIND>(uu - tau[r], a.beta));
      });
    }
  } else {
    // ---- row-major tile: the rows' tau and routed past chunks, from which the
    // row-major kernel recomputes their weights
    if (col == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (row_ok[r]) a.rm_tau[bh * (size_t)N + i0 + grp * 4 + r] = tau[r];
    }
    const int rg = lane >> 2, r4 = lane & 3;  // D-layout owner of row `lane` (lanes 0..15)
    uint32_t* bdst = a.rm_bits + ((bh * (size_t)N) + min(i0 + lane, N - 1)) * (size_t)a.rm_words;
    const bool write_rm = wave_valid && lane < 16 && i0 + lane < N;
#pragma unroll
    for (int wd = 0; wd < NW; ++wd) {
      uint32_t word = 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int blk = 2 * wd + half;
        if (blk < nbl) {
          unsigned long long mb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) mb[r] = __ballot(row_ok[r] && UV(blk, r) > tau[r]);
          const unsigned long long mr = r4 == 0 ? mb[0] : r4 == 1 ? mb[1] : r4 == 2 ? mb[2] : mb[3];
          word |= (uint32_t)((mr >> (16 * rg)) & 0xffffull) << (16 * half);
        }
      }
      if (write_rm && wd < a.rm_words) bdst[wd] = word;
    }
    if (write_rm)
      for (int wd = NW; wd < a.rm_words; ++wd) bdst[wd] = 0u;
  }
}

// The general prefill routing for the tiles the list-based kernel queued: a
// grid of workgroups walks the queue.
template <int NB, int KIND, bool GLB>
__global__ __launch_bounds__(512) void k_route_prefill(RouteArgs a) {
  const int nq = *a.fb_count;
  if constexpr (GLB) {
    for (int q = blockIdx.x; q < nq; q += gridDim.x) {
      route_general_tile<NB, KIND, GLB>(a, q);
      __syncthreads();  // the next tile reuses the LDS
    }
  } else {
    // one workgroup per tile of the grid, the first nq of them take one each
    if ((int)blockIdx.x < nq) route_general_tile<NB, KIND, GLB>(a, blockIdx.x);
  }
}

// ============================================================================
// Prefill routing, list-based (the common case). Four wavefronts x 32 query
// rows per 128-row tile and query head. The pre-scaled split summaries pass
// through LDS 32 chunks at a time; S^T = summaries x Q^T with
// v_mfma_f32_32x32x16_bf16 (hi and lo parts into one accumulator) gives each
// lane 16 scores (u units) of its query row per block, lanes l and l ^ 32
// sharing a row. Only scores above max u - 1 can carry weight (tau >= max u -
// 1): a first pass, from the high parts alone, bounds each row's max from
// below (the per-chunk error bound of the split covers the missing low
// parts); a second, exact pass writes every score above that bound - 1 as a
// (distance, row, chunk) entry into the tile's LDS list, a segment per
// wavefront and block, and finds the exact row max. A tile whose entries do
// not fit the list (or whose error bounds leave the entries' range) is queued
// for the general kernel before anything else is written; entries past 16 per
// lane are read back from the list when used.
//
// Everything after that is spread evenly over the entries, whatever their
// rows: each lane takes a contiguous run of its wavefront's entries. The tau
// sums are added per row in fixed point, so their order (and with it the
// result) does not depend on which lane adds what. The routed chunks go into
// per-row bitmasks, from which the tile's chunk union, each pair's rank in its
// row and its place among the pairs of its chunk follow without contended
// atomics.
// ============================================================================
// DC: the caller's head_dim (a template argument: no per-load test at 128)
template <int KIND, int MS, int DC>
__global__ __launch_bounds__(256, MS <= 512 ? 4 : 2) void k_route_fast(RouteArgs a) {
  constexpr int D = 128;
  constexpr int NS = D / 16;  // k-steps of the 32x32x16 MFMA
  constexpr int SROW = D + 8;
  constexpr int NWMAX = MS / 32;  // chunk slots of the tile, in words
  // tile list entries: every slot up to 512; beyond, 1024 (a tile whose
  // chunk union is larger goes to the general kernel), so that two
  // workgroups fit a CU's LDS
  constexpr int NE = MS <= 512 ? MS : 1024;
  constexpr int SH = MS <= 512 ? 9 : 11;  // a run key: tile row << SH | chunk
  constexpr uint32_t CMASK = (1u << SH) - 1u;
  constexpr int EPT = (NE + 255) / 256;   // tile list entries per thread
  constexpr int kListWords = 4096 + 2 * NE;
  constexpr int LCAP = kListWords - 2 * NE;  // entries per tile (the chunk entries take the tail)
  static_assert(MS <= 2048 && (MS & (MS - 1)) == 0, "chunk slots: a power of two up to 2048");
  // summary stage (hi and lo parts of 32 chunks). After the passes: the
  // own-chunk key logits (estimate), then the tau sums (tau loop), then the
  // per-row bitmasks [kTileRows][NWMAX] and the per-entry row masks [NE][4]
  // (emission); the tau iterates and first pool slots per row at its end.
  constexpr int kStageWords = 2 * 32 * SROW / 2;
  constexpr int kLateWords = kTileRows * NWMAX + NE * 4 + 2 * kTileRows;
  __shared__ __attribute__((aligned(16))) uint32_t s_scr[kStageWords > kLateWords ? kStageWords : kLateWords];
  uint16_t* const s_stage = reinterpret_cast<uint16_t*>(s_scr);
  static_assert(kTileRows * NWMAX >= 4 * kChunk + 6 * kTileRows, "early scratch fits");
  uint16_t* const sSh = s_stage;
  uint16_t* const sSl = s_stage + 32 * SROW;
  uint32_t* const s_words = reinterpret_cast<uint32_t*>(s_stage);
  float (*const s_lc)[kChunk] = reinterpret_cast<float (*)[kChunk]>(s_words);  // <k, cls> / sqrt(d)
  // tau sums per row in fixed point: 2^-22 units in 32 bits where every term
  // is at most 1 (a row's sums then stay below 512), 2^-32 units in 64 bits for
  // a general alpha
  using Fx = std::conditional_t<KIND == 0, unsigned long long, uint32_t>;
  // (after the own-chunk logits, which other wavefronts may still be reading)
  Fx (*const s_sum)[kTileRows] = reinterpret_cast<Fx (*)[kTileRows]>(s_words + 4 * kChunk);
  uint32_t (*const s_bits)[NWMAX] = reinterpret_cast<uint32_t (*)[NWMAX]>(s_words);
  // per list entry (per chunk in the 512-slot form, where that is the same
  // size): the rows of each wavefront that take it
  uint32_t (*const s_rm)[4] = reinterpret_cast<uint32_t (*)[4]>(s_words + kTileRows * NWMAX);
  constexpr bool kRmByChunk = NE == MS;
  float* const s_t = reinterpret_cast<float*>(s_words + kTileRows * NWMAX + NE * 4);  // tau iterate per row
  uint32_t* const s_s0 = s_words + kTileRows * NWMAX + NE * 4 + kTileRows;           // first pool slot per row
  // the entry list, an entry a 32-bit word: bits 10.. the distance below the
  // row's reference in units of 2^-21 (< 2), bits 5..9 the row in the wavefront, bits
  // 0..4 the chunk in the block; the tile's chunk entries in its tail
  __shared__ __attribute__((aligned(16))) uint32_t s_list[kListWords];
  int* const s_cl = reinterpret_cast<int*>(s_list + LCAP);
  int* const s_eoff = s_cl + NE;
  __shared__ uint32_t s_wun[4][NWMAX], s_union[NWMAX];
  __shared__ int s_pre[NWMAX + 1];
  __shared__ int s_wtot[4], s_tmp[4];
  __shared__ long long s_tbase;
  __shared__ int s_cnt;                     // entries in the list
  __shared__ int s_ownf[kTileRows];         // the row attends its own chunk
  __shared__ float s_bmax[NWMAX];           // per block of 32 chunks: the largest error bound
  __shared__ int2 s_seg[4][MS / 32];  // per wavefront: (first, count | block << 16)

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int tid = threadIdx.x;
  if (tid == 0) s_cnt = 0;  // ordered before any use by the barriers of the first pass
  const int hi32 = lane >> 5;
  const int row = lane & 31;   // the wavefront's row of this lane
  const int R = w * 32 + row;  // the tile's row of this lane
  const bool owner = hi32 == 0;  // lanes 0..31 keep the per-row state
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = a.g;
  const int hk = h / g;
  const int hh = h % g;
  const int N = a.Nq;
  const size_t bh = (size_t)b * a.Hq + h;
  const int i0 = tile * kTileRows + w * 32;  // first row of this wavefront
  const int qi = i0 + row;
  const int cw = i0 / kChunk;                // own chunk of the wavefront's rows
  const bool wave_valid = i0 < N;
  const bool row_ok = qi < N;
  const bool causal = a.causal != 0;
  const bool est = causal && a.est != 0;
  const int n_slots = a.n_slots;
  const int NW = (n_slots + 31) / 32;
  const int ncomp = wave_valid ? (causal ? cw : n_slots) : 0;  // complete-chunk candidates of the rows
  const int last_row = min(tile * kTileRows + kTileRows, N) - 1;
  const int ncomp_wg = causal ? last_row / kChunk : n_slots;
  const int nblk_wg = (ncomp_wg + 31) / 32;
  const size_t sbase = ((size_t)b * a.Hkv + hk) * (size_t)n_slots * D;

  // ---- passes over the summary blocks of the tile: body(kb, u) with u the
  // row's scores of block kb (-inf past the candidates), for the wavefront's
  // blocks; HI: from the high parts of the summaries alone
  bf16x8 qb[NS];  // q^T as the B operand: column qi, dims 16 s + 8 hi32 .. +7 (loaded below)
  u32x4 gl[4];
  auto load_stage = [&](auto hi_tag, int kb) {  // 32 chunks x (hi[, lo]) x 16 segments of 16 bytes
    constexpr bool HI = decltype(hi_tag)::value;
#pragma unroll
    for (int k = 0; k < (HI ? 2 : 4); ++k) {
      const int idx = tid + 256 * k;
      const int cc = HI ? (idx >> 4) : (idx >> 5);
      const int part = HI ? (idx & 15) : (idx & 31);
      const int c = min(kb * 32 + cc, max(ncomp_wg - 1, 0));
      gl[k] = ldg16((part < 16 ? a.s_hi : a.s_lo) + sbase + (size_t)c * D + 8 * (part & 15));
    }
  };
  auto store_stage = [&](auto hi_tag) {
    constexpr bool HI = decltype(hi_tag)::value;
#pragma unroll
    for (int k = 0; k < (HI ? 2 : 4); ++k) {
      const int idx = tid + 256 * k;
      const int cc = HI ? (idx >> 4) : (idx >> 5);
      const int part = HI ? (idx & 15) : (idx & 31);
      *reinterpret_cast<u32x4*>(&(part < 16 ? sSh : sSl)[cc * SROW + 8 * (part & 15)]) = gl[k];
    }
  };
  // first_loaded: the first block's loads were issued by the caller
  auto scan_blocks = [&](auto hi_tag, bool first_loaded, auto&& body) {
    constexpr bool HI = decltype(hi_tag)::value;
    if (nblk_wg > 0 && !first_loaded) load_stage(hi_tag, 0);
    for (int kb = 0; kb < nblk_wg; ++kb) {
      const bool more = kb + 1 < nblk_wg;
      store_stage(hi_tag);
      __syncthreads();
      if (more) load_stage(hi_tag, kb + 1);
      if (kb * 32 < ncomp) {
        // u of row qi for chunks kb*32 + 8 (r/4) + 4 hi32 + r%4
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const uint16_t* ah = &sSh[row * SROW + 8 * hi32];
        const uint16_t* al = &sSl[row * SROW + 8 * hi32];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          acc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ah + 16 * s), qb[s], acc);
          if (!HI) acc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(al + 16 * s), qb[s], acc);
        }
        if (kb * 32 + 32 > ncomp) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[r] = kb * 32 + 8 * (r >> 2) + 4 * hi32 + (r & 3) < ncomp ? acc[r] : -INFINITY;
        }
        body(kb, acc);
      }
      __syncthreads();
    }
  };
  using HiOnly = std::integral_constant<bool, true>;
  using Full = std::integral_constant<bool, false>;

  // pass 1's first summary loads go out before anything else, so that their
  // latency overlaps the query loads and the set-up below
  if (nblk_wg > 0) load_stage(HiOnly{}, 0);

  // ---- q^T as the B operand
  {
#pragma unroll
    for (int s = 0; s < NS; ++s) qb[s] = as_bf16x8(ldg16_dc<DC>(a.Q, bh * N + min(qi, N - 1), 16 * s + 8 * hi32));
  }


  // per block of 32 chunks, the largest error bound of its chunks (visible
  // after the first barrier of pass 1)
  {
    const int clast = max(ncomp_wg - 1, 0);  // chunks past the tile's candidates repeat the last one
#pragma unroll
    for (int c0 = 0; c0 < MS; c0 += 256) {
      float e = a.s_err[(size_t)(b * a.Hkv + hk) * n_slots + min(c0 + tid, clast)];
      e = max_xor16(max16(e));  // over the 32 chunks of the half wavefront
      if ((lane & 31) == 0) s_bmax[(c0 + tid) >> 5] = e;
    }
  }
  // |q| of the row (bf16 values as the MFMA sees them)
  float qn;
  {
    float q2 = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4 v = __builtin_bit_cast(u32x4, qb[s]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q2 = fmaf(bf16lo(v[e]), bf16lo(v[e]), q2);
        q2 = fmaf(bf16hi(v[e]), bf16hi(v[e]), q2);
      }
    }
    qn = sqrtf(sum_xor32(q2));
  }

  // pass 1, from the high parts: a lower bound of the row's max u, the largest
  // hi-only score less |q| times its block's error bound
  float lbound = -INFINITY;
  float emax = 0.f;  // the largest block error bound the row saw
  scan_blocks(HiOnly{}, true, [&](int kb, const f32x16& u) {
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) lmax = fmaxf(lmax, u[r]);
    const float e = s_bmax[kb];
    lbound = fmaxf(lbound, max_xor32(lmax) - qn * e);
    emax = fmaxf(emax, e);
  });
  // every score above max u - 1 is above lbound - 1; the entries are stored
  // below ref = lbound + 2 |q| emax, which no score exceeds
  const float marg = qn * emax;
  const float ref = lbound + 2.f * marg;
  // pass 2: the scores above max - 1; per block, a segment of the list for the
  // wavefront's entries, lane by lane
  int cnt = 0;   // this lane's entries
  int wcnt = 0;  // the wavefront's entries (uniform)
  int nseg = 0;  // its segments (uniform)
  float m_run = -INFINITY;  // the row's max u (exact scores)
  {
    // rows past the sequence end take no entries
    const float thr = row_ok ? lbound - 1.f : INFINITY;
    scan_blocks(Full{}, false, [&](int kb, const f32x16& u) {
      float lmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) lmax = fmaxf(lmax, u[r]);
      m_run = fmaxf(m_run, lmax);
      // this lane's place among the wavefront's entries of the block (lanes in
      // order, a lane's entries in register order): per register a ballot,
      // its lanes below this one counted with mbcnt
      uint32_t pre = 0u;
      int tot = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint64_t bm = __ballot(u[r] > thr);
        pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, pre));
        tot += __popcll(bm);
      }
      if (tot > 0) {
        int first = 0;
        if (lane == 0) {
          first = atomicAdd(&s_cnt, tot);
          s_seg[w][nseg] = make_int2(first, tot | (kb << 16));
        }
        first = __shfl(first, 0);
        ++nseg;
        if (first + tot <= LCAP) {
          uint32_t* lp = s_list + first + (int)pre;
          uint32_t* const lp0 = lp;
          const uint32_t kbase = (uint32_t)((row << 5) | (4 * hi32));
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (u[r] > thr) {
              // the distance below ref in 2^-21 units, rounded (v_cvt_u32
              // truncates); below 2 (so 22 bits) while the error bound is
              // under 0.5, which the tile needs to stay here
              const uint32_t q = (uint32_t)fmaxf(fmaf(ref - u[r], 2097152.f, 0.5f), 0.f);
              *lp++ = (q << 10) | kbase | (uint32_t)(8 * (r >> 2) + (r & 3));
            }
          cnt += (int)(lp - lp0);
        }
      }
      wcnt += tot;
    });
  }
  m_run = max_xor32(m_run);
  const float m_list = ref;  // what the list entries are stored against
  // uniform: the tile goes to the general kernel if its list overflowed or a
  // row's error bound leaves the entries' range
  if (__syncthreads_or(s_cnt > LCAP || (row_ok && marg >= 0.5f))) {
    if (tid == 0) a.fb_tiles[atomicAdd(a.fb_count, 1)] = make_int2(tile, (int)bh);
    return;
  }

  // ---- own-chunk estimate: score against the summary of tokens [cw*C, i]
  float ud = -INFINITY;
  const float uscale = (a.alpha - 1.f) * a.zscale;
  if (est && wave_valid) {
    const size_t krow0 = ((size_t)b * a.Hkv + hk) * a.Lmax + (size_t)cw * kChunk;
    const int lim = N - 1 - cw * kChunk;  // last key of the chunk inside the sequence
    {
      float l = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const u32x4 kv = ldg16_dc<DC>(a.K, krow0 + min(lane, lim), 8 * c8);
        const u32x4 cv = ldg16_dc<DC>(a.cls, hk, 8 * c8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l = fmaf(bf16lo(kv[e]), bf16lo(cv[e]), l);
          l = fmaf(bf16hi(kv[e]), bf16hi(cv[e]), l);
        }
      }
      s_lc[w][lane] = l * a.inv_sqrt_d;
    }
    f32x16 e0, e1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e0[r] = 0.f;
      e1[r] = 0.f;
    }
    const size_t kr0 = krow0 + min(row, lim), kr1 = krow0 + min(row + 32, lim);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      e0 = mfma32x32x16(as_bf16x8(ldg16_dc<DC>(a.K, kr0, 16 * s + 8 * hi32)), qb[s], e0);
      e1 = mfma32x32x16(as_bf16x8(ldg16_dc<DC>(a.K, kr1, 16 * s + 8 * hi32)), qb[s], e1);
    }
    wave_lds_fence();
    const int pi = qi - cw * kChunk;  // keys 0 .. pi of the chunk are the row's
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * hi32 + (r & 3);
      if (kk <= pi) M = fmaxf(M, s_lc[w][kk]);
      if (kk + 32 <= pi) M = fmaxf(M, s_lc[w][kk + 32]);
    }
    M = max_xor32(M);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 8 * (r >> 2) + 4 * hi32 + (r & 3);
      if (kk <= pi) {
        const float e = fast_exp2((s_lc[w][kk] - M) * kLog2e);
        num = fmaf(e, e0[r], num);
        den += e;
      }
      if (kk + 32 <= pi) {
        const float e = fast_exp2((s_lc[w][kk + 32] - M) * kLog2e);
        num = fmaf(e, e1[r], num);
        den += e;
      }
    }
    num = sum_xor32(num);
    den = sum_xor32(den);
    ud = row_ok ? num / den * uscale : -INFINITY;
    if (row_ok) m_run = fmaxf(m_run, ud);  // list entries at or below the new max - 1 stay inert
  }

  // ---- this lane's run of its wavefront's entries (entry k of the wavefront
  // lies in its segments, in order): the first RUNMAX in registers, the rest
  // (heavy wavefronts only) read from the list when used. Loops over the run
  // go to the uniform run length; fetch must be called by the whole wavefront.
  const int run = (wcnt + kWave - 1) / kWave;
  const int k_beg = min(wcnt, lane * run);
  const int nl = min(wcnt, lane * run + run) - k_beg;
  constexpr int RUNMAX = 16;
  // the segment cursor of a walk over increasing j: (segment, its first entry
  // index in the wavefront's order, its record)
  struct SegCursor {
    int sg, sk;
    int2 v;
  };
  auto cursor = [&]() { return SegCursor{0, 0, s_seg[w][0]}; };
  auto fetch = [&](SegCursor& cur, int j, float& uu, uint32_t& kk) {
    uint32_t e = 0u;
    if (j < nl) {
      const int k = k_beg + j;
      while (k >= cur.sk + (cur.v.y & 0xffff)) {
        cur.sk += cur.v.y & 0xffff;
        cur.v = s_seg[w][++cur.sg];
      }
      e = s_list[cur.v.x + k - cur.sk];
    }
    const int rw = (e >> 5) & 31;
    const float mr = __shfl(m_list, rw);  // the max the distance is taken from
    uu = j < nl ? mr - (float)(e >> 10) * 4.76837158e-7f : -INFINITY;
    kk = (uint32_t)(((w * 32 + rw) << SH) | ((cur.v.y >> 16) * 32 + (e & 31)));
  };
  float eu[RUNMAX];
  uint32_t ek[RUNMAX];
  {
    SegCursor cur = cursor();
#pragma unroll
    for (int j = 0; j < RUNMAX; ++j) {
      if (j >= run) break;
      fetch(cur, j, eu[j], ek[j]);
    }
  }
  // fn(j, u, key) for every j < run: registers, then the list
  auto for_run = [&](auto&& fn) {
#pragma unroll
    for (int j = 0; j < RUNMAX; ++j) {
      if (j >= run) break;
      fn(j, eu[j], ek[j]);
    }
    if (run > RUNMAX) {
      SegCursor cur = cursor();
      for (int j = RUNMAX; j < run; ++j) {
        float uu;
        uint32_t kk;
        fetch(cur, j, uu, kk);
        fn(j, uu, kk);
      }
    }
  };

  // ---- tau: safeguarded Halley on the bracket [m - 1, m - n^-(alpha-1)], the
  // rows of the wavefront together
  const bool has = row_ok && m_run > -INFINITY;
  float tau = INFINITY;
  {
    float lo = m_run - 1.f;
    const int n = cnt + __shfl_xor(cnt, 32) + ((est && ud > lo) ? 1 : 0);
    float hi = has ? tau_upper(m_run, max(1, n), a.alpha) : lo;
    float t = lo;
    // fixed point: terms and sums are >= 0; sums stay far below 2^32
    auto to_fx = [](float x) -> Fx {
      if constexpr (KIND == 0) {
        x = fminf(x, 1.0e9f);
        const float xi = floorf(x);
        const uint32_t hw = (uint32_t)xi;
        const uint32_t lw = (uint32_t)fminf((x - xi) * 4294967296.f, 4294967040.f);
        return ((unsigned long long)hw << 32) | lw;
      } else {
        return (uint32_t)fminf(fmaf(x, 4194304.f, 0.5f), 4294967040.f);
      }
    };
    auto from_fx = [](Fx v) {
      if constexpr (KIND == 0)
        return (float)(uint32_t)(v >> 32) + (float)(uint32_t)v * 2.3283064365386963e-10f;
      else
        return (float)v * 2.384185791015625e-07f;
    };
    if (owner) {
      s_t[R] = has ? t : INFINITY;
      s_sum[0][R] = 0;
      s_sum[1][R] = 0;
      s_sum[2][R] = 0;
    }
    wave_lds_fence();
    if (wave_any(has)) {
      for (int it = 0; it < a.n_iter; ++it) {
        float f0 = 0.f, f1 = 0.f, f2 = 0.f;
        int cur = -1;
        float tc = 0.f;
        auto flush = [&]() {
          atomicAdd(&s_sum[0][cur], to_fx(f0));
          atomicAdd(&s_sum[1][cur], to_fx(f1));
          if (KIND != 1) atomicAdd(&s_sum[2][cur], to_fx(f2));
          f0 = f1 = f2 = 0.f;
        };
        for_run([&](int j, float uu, uint32_t kk) {
          if (j < nl) {
            const int rr = kk >> SH;
            if (rr != cur) {
              if (cur >= 0) flush();
              cur = rr;
              tc = s_t[rr];
            }
            tau_terms<KIND>(uu, tc, a.beta, f0, f1, f2);
          }
        });
        if (cur >= 0) flush();
        wave_lds_fence();
        bool conv = true;
        if (owner && has) {
          float F0 = from_fx(s_sum[0][R]), F1 = from_fx(s_sum[1][R]), F2 = from_fx(s_sum[2][R]);
          if (est) tau_terms<KIND>(ud, t, a.beta, F0, F1, F2);
          const float nt = tau_step<KIND>(t, F0, F1, F2, a.beta, lo, hi);
          conv = tau_converged(t, nt);
          t = nt;
          s_t[R] = t;
          s_sum[0][R] = 0;
          s_sum[1][R] = 0;
          s_sum[2][R] = 0;
        }
        wave_lds_fence();
        if (wave_all(conv)) break;
      }
    }
    if (has) tau = t;
  }
  if (owner && row_ok) a.tau[bh * (size_t)N + qi] = tau;

  // ---- own chunk: routed (estimate) or always attended with weight 1. A
  // pooled tile attends it in the merge kernel (one causal tile per 64 rows),
  // from its log2 weight own_lw; a row-major tile lists it with the others.
  const float td = ud - tau;
  const bool dact = row_ok && (est ? (td > 0.f) : causal);
  const float lwd = !row_ok ? -INFINITY : (est ? (td > 0.f ? log2_prior<KIND>(td, a.beta) : -INFINITY) : 0.f);
  const bool own_pair = owner && causal && dact;  // the lane that owns the row's own-chunk weight
  if (owner && row_ok && causal) a.own_lw[bh * (size_t)N + qi] = lwd;

  // ---- per-row bitmasks of the routed past chunks (over the tau sums)
  __syncthreads();
  for (int x = tid; x < kTileRows * NWMAX; x += blockDim.x) (&s_bits[0][0])[x] = 0u;
  if constexpr (kRmByChunk)
    for (int x = tid; x < NE * 4; x += blockDim.x) (&s_rm[0][0])[x] = 0u;
  if (owner) s_ownf[R] = own_pair ? 1 : 0;
  __syncthreads();
  for_run([&](int j, float uu, uint32_t kk) {
    const int rr = kk >> SH, c = kk & CMASK;
    if (j < nl && uu > s_t[rr]) {
      atomicOr(&s_bits[rr][c >> 5], 1u << (c & 31));
      if constexpr (kRmByChunk) atomicOr(&s_rm[c][rr >> 5], 1u << (rr & 31));
    }
  });
  __syncthreads();
  if (a.bits != nullptr) {
    // attended chunks: the routed past chunks and the own chunk
    for (int x = tid; x < kTileRows * a.bits_words; x += blockDim.x) {
      const int r = x / a.bits_words, wd = x % a.bits_words;
      const int q = tile * kTileRows + r;
      const int cq = q / kChunk;
      uint32_t word = wd < NW ? s_bits[r][wd] : 0u;
      if (s_ownf[r] && (cq >> 5) == wd) word |= 1u << (cq & 31);
      if (q < N) a.bits[(bh * (size_t)N + q) * a.bits_words + wd] = word;
    }
  }
  // routed past chunks of the row (owner lanes)
  int nsl = 0;
  if (owner)
    for (int wd = 0; wd < NW; ++wd) nsl += __popc(s_bits[R][wd]);
  // the wavefront's union
  if constexpr (NWMAX == 16) {
    // lane l ORs word l % 16 of rows 8 (l / 16) .. +7
    const int wd = lane & 15;
    uint32_t x = 0u;
#pragma unroll
    for (int r = 0; r < 8; ++r) x |= s_bits[w * 32 + 8 * (lane >> 4) + r][wd];
    x |= __shfl_xor(x, 16);
    x |= __shfl_xor(x, 32);
    if (lane < NWMAX) s_wun[w][lane] = x;
  } else {
    for (int wd = lane; wd < NWMAX; wd += kWave) {
      uint32_t x = 0u;
      for (int r = 0; r < 32; ++r) x |= s_bits[w * 32 + r][wd];
      s_wun[w][wd] = x;
    }
  }

  // ---- pool slots: one per attended chunk of every row of the tile, taken
  // with one atomic; the slots of a row are consecutive, in chunk order
  int row_pre;
  {
    int x = (owner && row_ok) ? nsl : 0;
    const int x0 = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      x += lane >= off ? y : 0;
    }
    row_pre = x - x0;
    if (lane == kWave - 1) s_wtot[w] = x;
  }
  __syncthreads();
  for (int x = tid; x < NWMAX; x += blockDim.x) s_union[x] = s_wun[0][x] | s_wun[1][x] | s_wun[2][x] | s_wun[3][x];
  if constexpr (NE < MS) {
    // a union (plus a row-major tile's own chunk) past NE entries: the tile
    // goes to the general kernel before the pool is touched (what it wrote so
    // far, tau, own-chunk weights and bits, the general kernel rewrites)
    __syncthreads();
    int ne_tile = 1;
    for (int x = 0; x < NW; ++x) ne_tile += __popc(s_union[x]);
    if (ne_tile > NE) {
      if (tid == 0) a.fb_tiles[atomicAdd(a.fb_count, 1)] = make_int2(tile, (int)bh);
      return;
    }
  }
  if (tid == kWave) {
    const int tot = s_wtot[0] + s_wtot[1] + s_wtot[2] + s_wtot[3];
    long long pbase = 0;  // a tile without routed past chunks needs no slots
    if (tot > 0) {
      const int part = (int)((blockIdx.x + (size_t)gridDim.x * (blockIdx.y + (size_t)gridDim.y * blockIdx.z)) % kPools);
      const unsigned long long cap = (unsigned long long)a.pool_cap / kPools;
      const unsigned long long got = atomicAdd(&a.pool[part], (unsigned long long)tot);
      pbase = got + (unsigned long long)tot <= cap ? (long long)(part * cap + got) : -1;
    }
    s_tbase = pbase;
    a.tbase[bh * a.n_tiles + tile] = pbase >= 0 ? (uint32_t)pbase : 0u;
  }
  __syncthreads();
  const bool pooled = s_tbase >= 0;  // uniform: chunk-major for every routed past chunk
  if (tid == 0 && !pooled) atomicAdd(a.n_rm, 1);
  if (!pooled) {
    // the row-major list holds the own chunk too
    if (own_pair) atomicOr(&s_union[cw >> 5], 1u << (cw & 31));
    __syncthreads();
  }
  const long long tb = s_tbase;
  int wpre = 0;
  for (int ww = 0; ww < w; ++ww) wpre += s_wtot[ww];
  const long long s0 = tb + wpre + row_pre;  // the row's first slot (owner lanes)
  if (owner && row_ok) {
    a.cmcnt[bh * (size_t)N + qi] = pooled ? (uint16_t)nsl : (uint16_t)0;
    a.rslot[bh * (size_t)N + qi] = pooled ? (uint32_t)s0 : 0u;
  }
  if (owner) s_s0[R] = (uint32_t)s0;

  // ---- the tile's attended chunks: chunk-major list if pooled, else row-major
  if (tid == 0) {
    int acc = 0;
    for (int wd = 0; wd < NW; ++wd) {
      s_pre[wd] = acc;
      acc += __popc(s_union[wd]);
    }
    s_pre[NW] = acc;
    a.ccounts[bh * a.n_tiles + tile] = pooled ? acc : 0;
    a.counts[bh * a.n_tiles + tile] = pooled ? 0 : acc;
  }
  __syncthreads();
  const long long toff = bh * a.per_head + prefill_tile_offset(tile, n_slots, causal);
  auto epos = [&](int c) { return s_pre[c >> 5] + __popc(s_union[c >> 5] & ((1u << (c & 31)) - 1u)); };
  {
    // every chunk slot of the union by its own thread, at its list position
    int* lst = (pooled ? a.clists : a.lists) + toff;
    for (int c = tid; c < NW * 32; c += blockDim.x) {
      if ((s_union[c >> 5] >> (c & 31)) & 1u) {
        const int pos = epos(c);
        s_cl[pos] = c;
        lst[pos] = c;
      }
    }
  }
  // rank of chunk c among the attended chunks of tile row rr
  auto rank_in_row = [&](int rr, int c) {
    int k = __popc(s_bits[rr][c >> 5] & ((1u << (c & 31)) - 1u));
    for (int wd = 0; wd < (c >> 5); ++wd) k += __popc(s_bits[rr][wd]);
    return k;
  };
  const int ne = s_pre[NW];
  __syncthreads();

  if (pooled) {
    // ---- row masks of every entry (a lane per entry in each wavefront), the
    // pairs per entry and their place: the pairs of a chunk in row order
    if constexpr (!kRmByChunk) {
      for (int e = lane; e < ne; e += kWave) {
        const int c = s_cl[e];
        uint32_t m = 0u;
#pragma unroll
        for (int r = 0; r < 32; ++r) m |= ((s_bits[w * 32 + r][c >> 5] >> (c & 31)) & 1u) << r;
        s_rm[e][w] = m;
      }
      __syncthreads();
    }
    auto rmask = [&](int e) -> const uint32_t* { return s_rm[kRmByChunk ? s_cl[e] : e]; };
    // entries EPT t .. EPT t + EPT - 1 per thread
    auto ecount = [&](int e) {
      const uint32_t* m = rmask(e);
      return __popc(m[0]) + __popc(m[1]) + __popc(m[2]) + __popc(m[3]);
    };
    int ec[EPT];
    int esum = 0;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      ec[q] = EPT * tid + q < ne ? ecount(EPT * tid + q) : 0;
      esum += ec[q];
    }
    int first = 0;
    block_excl_scan<4>(esum, s_tmp, first);
    int* cmp = a.cmp + ((size_t)b * a.Hkv + hk) * n_slots;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = EPT * tid + q;
      if (e < ne) {
        s_eoff[e] = first;
        a.ceo[toff + e] = make_int2(first, ec[q]);
      }
      first += ec[q];
    }
    __syncthreads();
    // the entries' places among all pairs of their chunks (global atomics with
    // return): requested now, their results stored after the records
    int cb[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = EPT * tid + q;
      cb[q] = e < ne ? atomicAdd(&cmp[s_cl[e]], ec[q]) : 0;
    }
    auto place = [&](int e, int rr) {
      const int wr = rr >> 5;
      const uint32_t* m = rmask(e);
      int j = s_eoff[e] + __popc(m[wr] & ((1u << (rr & 31)) - 1u));
      for (int ww = 0; ww < wr; ++ww) j += __popc(m[ww]);
      return j;
    };
    for_run([&](int j, float uu, uint32_t kk) {
      const int rr = kk >> SH, c = kk & CMASK;
      const float tr = s_t[rr];
      if (j < nl && uu > tr)
        a.trec[tb + place(epos(c), rr)] = make_int4((tile * kTileRows + rr) * g + hh, (int)(s_s0[rr] + rank_in_row(rr, c)),
                                                    __float_as_int(log2_prior<KIND>(uu - tr, a.beta)), 0);
    });
#pragma unroll
    for (int q = 0; q < EPT; ++q)
      if (EPT * tid + q < ne) a.cbase[toff + EPT * tid + q] = cb[q];
  } else {
    // ---- row-major tile: the rows' tau and routed past chunks, from which the
    // row-major kernel recomputes their weights
    if (owner && row_ok) a.rm_tau[bh * (size_t)N + qi] = tau;
    for (int x = tid; x < kTileRows * a.rm_words; x += blockDim.x) {
      const int r = x / a.rm_words, wd = x % a.rm_words;
      const int q = tile * kTileRows + r;
      if (q < N) a.rm_bits[(bh * (size_t)N + q) * a.rm_words + wd] = wd < NW ? s_bits[r][wd] : 0u;
    }
  }
}

// Scale the float32 summaries of the chunks the prefill routing reads into u
// units ((alpha - 1) * scaling_factor / sqrt(d)) and split them into bf16 high
// parts and bf16 low parts (x - high), once per call; also clears the
// per-chunk pair counters and the pool slot counters.
__global__ __launch_bounds__(256) void k_split_summaries(RouteArgs a, int n_need) {
  constexpr int D = 128;
  // the per-chunk pair counters the routing adds to start from zero
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.n_bhc; i += gridDim.x * blockDim.x) a.cmp[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x <= kPools)
    a.pool[threadIdx.x] = threadIdx.x < kPools ? 0ull : (unsigned long long)a.pool_cap;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *a.fb_count = 0;
    *a.n_rm = 0;
  }
  const float uscale = (a.alpha - 1.f) * a.zscale;
  const size_t per_bh = (size_t)n_need * (D / 8);
  const size_t total = (size_t)a.B * a.Hkv * per_bh;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = i / per_bh;
    const size_t rem = i % per_bh;
    const size_t c = rem / (D / 8);
    const int e8 = (int)(rem % (D / 8)) * 8;
    f32x4 x0 = ldf4_d(a.S, bh * a.s_cap + c, e8, a.d);
    f32x4 x1 = ldf4_d(a.S, bh * a.s_cap + c, e8 + 4, a.d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x0[e] *= uscale;
      x1[e] *= uscale;
    }
    bf16x8 hi, lo;
    split_hi_lo(x0, x1, hi, lo);
    const size_t dst = (bh * a.n_slots + c) * D + e8;
    *reinterpret_cast<bf16x8*>(a.s_hi + dst) = hi;
    *reinterpret_cast<bf16x8*>(a.s_lo + dst) = lo;
    // the chunk's error bound: |lo| (what a score from the high parts misses)
    // plus 2^-14 |x| (fp32 rounding of the two dot products, with room to
    // spare); the 16 lanes of a chunk are one DPP row
    const u32x4 lw = __builtin_bit_cast(u32x4, lo);
    float l2 = 0.f, x2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      l2 = fmaf(bf16lo(lw[e]), bf16lo(lw[e]), l2);
      l2 = fmaf(bf16hi(lw[e]), bf16hi(lw[e]), l2);
      x2 = fmaf(x0[e], x0[e], x2);
      x2 = fmaf(x1[e], x1[e], x2);
    }
    l2 = sum16(l2);
    x2 = sum16(x2);
    if (e8 == 0) a.s_err[bh * a.n_slots + c] = sqrtf(l2) + 6.103515625e-05f * sqrtf(x2);
  }
}

// ============================================================================
// Decode routing
// ============================================================================
// Scores of the complete chunks against the g query heads of one KV head:
// eight lanes per summary row (four float4 each), 32 rows per wavefront, all of
// a wavefront's summary loads in flight before any arithmetic.
constexpr int kDecScorePasses = 4;                          // 8 rows per pass
constexpr int kDecScoreRowsPerWg = 4 * 8 * kDecScorePasses;  // four wavefronts
template <int G, int DC>
__global__ __launch_bounds__(256) void k_route_decode_scores(RouteArgs a) {
  constexpr int D = 128;
  constexpr int NP = kDecScorePasses;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int grp_id = blockIdx.y;
  const int b = grp_id / a.Hkv;
  const int hk = grp_id % a.Hkv;
  const int t = min(max(a.seqlens[b], 1), a.Lmax) - 1;  // clamp to the cache
  const int ncomp = t / kChunk;
  const int c0 = blockIdx.x * kDecScoreRowsPerWg + w * 8 * NP;
  if (c0 >= ncomp) return;
  const int sub = lane & 7;
  const size_t srow0 = ((size_t)b * a.Hkv + hk) * (size_t)a.s_cap;
  f32x4 sva[NP][4];
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    const int c = min(c0 + pass * 8 + (lane >> 3), ncomp - 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) sva[pass][k] = ldf4_dc<DC>(a.S, srow0 + c, 32 * k + 4 * sub);
  }
  float q[G][16];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x2 v = ldg8_d(a.Q, (size_t)b * a.Hq + hk * G + hh, 32 * k + 4 * sub, a.d);
      q[hh][4 * k + 0] = bf16lo(v[0]);
      q[hh][4 * k + 1] = bf16hi(v[0]);
      q[hh][4 * k + 2] = bf16lo(v[1]);
      q[hh][4 * k + 3] = bf16hi(v[1]);
    }
  }
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    const int c = c0 + pass * 8 + (lane >> 3);
    const bool val = c < ncomp;
    const f32x4* sv = sva[pass];
    float mine = 0.f;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(q[hh][4 * k + e], sv[k][e], part);
      part += dpp_f<kDppXor1>(part);
      part += dpp_f<kDppXor2>(part);
      part += dpp_f<kDppHalfMirror>(part);
      if (sub == hh) mine = part;
    }
    if (val && sub < G) a.z[((size_t)b * a.Hq + hk * G + sub) * a.n_slots + c] = mine * a.zscale;
  }
}

// tau, routed union and work list for the g query heads of one (b, kv head).
// A wavefront per query head; the routed chunks travel as bitmask words built
// from ballots (word j of a row in lane j % 64, register j / 64), and every
// wavefront forms the group's union words and their prefix counts itself.
template <int G, int KPL, int KIND>
__global__ __launch_bounds__(G * 64) void k_route_decode_tau(RouteArgs a) {
  constexpr int D = 128;
  constexpr int NWD = 2 * KPL + 1;           // bitmask words (the own chunk can sit in the last)
  constexpr int NWL = (NWD + 63) / 64;       // words per lane
  __shared__ uint32_t s_wb[G][64 * NWL];     // each head's words
  __shared__ float s_lc[G][64];
  __shared__ float s_qk[G][64];

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int grp_id = blockIdx.x;
  const int b = grp_id / a.Hkv;
  const int hk = grp_id % a.Hkv;
  const int h = hk * G + w;
  const int t = min(max(a.seqlens[b], 1), a.Lmax) - 1;  // clamp to the cache
  const int ct = t / kChunk;
  const int ncomp = ct;
  const bool est = a.est != 0;
  const int ncand = ncomp + (est ? 1 : 0);

  const size_t bh = (size_t)b * a.Hq + h;
  const float am1 = a.alpha - 1.f;

  // ---- every load first: the estimate's query, head_cls and own-chunk keys,
  // then the scores of complete chunks c = k*64 + lane (unconditional, keys
  // past the sequence read its last key and are masked below)
  const int sub = lane & 15, rg = lane >> 4;
  const int nval = t - ct * kChunk + 1;
  u32x4 qv = {0, 0, 0, 0}, cv = {0, 0, 0, 0}, kvs[16];
  if (est) {
    qv = ldg16_d(a.Q, bh, 8 * sub, a.d);
    cv = ldg16_d(a.cls, hk, 8 * sub, a.d);
    const size_t krow0 = ((size_t)b * a.Hkv + hk) * a.Lmax + (size_t)ct * kChunk;
#pragma unroll
    for (int r = 0; r < 16; ++r) kvs[r] = ldg16_d(a.K, krow0 + min(r * 4 + rg, nval - 1), 8 * sub, a.d);
  }
  float u[KPL];
  const float* zrow = a.z + bh * a.n_slots;
#pragma unroll
  for (int k = 0; k < KPL; ++k) u[k] = zrow[min(k * 64 + lane, max(ncomp - 1, 0))];

  // ---- own-chunk estimate from the tokens [ct*C, t]
  float ud = -INFINITY;
  if (est) {
    float wq[8], wc[8];
    for (int e = 0; e < 4; ++e) {
      wq[2 * e] = bf16lo(qv[e]);
      wq[2 * e + 1] = bf16hi(qv[e]);
      wc[2 * e] = bf16lo(cv[e]);
      wc[2 * e + 1] = bf16hi(cv[e]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = r * 4 + rg;
      const bool val = key < nval;
      const u32x4 kv = kvs[r];
      const float pq = sum16(dot8_bf16(kv, wq));
      const float pc = sum16(dot8_bf16(kv, wc));
      if (sub == 0) {
        s_qk[w][key] = pq;  // raw q.k: the 1/sqrt(d) is inside zscale
        s_lc[w][key] = val ? pc * a.inv_sqrt_d : -INFINITY;
      }
    }
    wave_lds_fence();
    const float lcv = s_lc[w][lane];
    const float qkv = s_qk[w][lane];
    const float M = wave_max(lcv);
    const float e = (lcv > -INFINITY) ? fast_exp2((lcv - M) * kLog2e) : 0.f;
    const float num = wave_sum(e * qkv);
    const float den = wave_sum(e);
    ud = (num / den) * a.zscale * am1;
  }

#pragma unroll
  for (int k = 0; k < KPL; ++k) u[k] = k * 64 + lane < ncomp ? u[k] * am1 : -INFINITY;
  float tau = INFINITY;
  if (ncand > 0) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < KPL; ++k) m = fmaxf(m, u[k]);
    m = fmaxf(wave_max(m), ud);
    float lo = m - 1.f, hi = tau_upper(m, ncand, a.alpha);
    tau = lo;
    for (int it = 0; it < a.n_iter; ++it) {
      float f0 = 0.f, f1 = 0.f, f2 = 0.f;
      if constexpr (KIND == 0) {
#pragma unroll
        for (int k = 0; k < KPL; ++k) tau_terms<KIND>(u[k], tau, a.beta, f0, f1, f2);
        f0 = wave_sum(f0);
        f1 = wave_sum(f1);
        f2 = wave_sum(f2);
      } else {
        // beta = 2 or 1: the support size (f2, resp. f1) is a count, taken
        // from the ballots of the tests (wave-uniform, no reduction)
        int nsup = 0;
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
          const float t = u[k] - tau;
          const float p = fmaxf(t, 0.f);
          if constexpr (KIND == 2) f0 = fmaf(p, p, f0), f1 += p;
          else f0 += p;
          nsup += __popcll(__ballot(t > 0.f));
        }
        f0 = wave_sum(f0);
        if constexpr (KIND == 2) {
          f1 = wave_sum(f1);
          f2 = (float)nsup;
        } else {
          f1 = (float)nsup;
        }
      }
      if (est) tau_terms<KIND>(ud, tau, a.beta, f0, f1, f2);
      const float nt = tau_step<KIND>(tau, f0, f1, f2, a.beta, lo, hi);
      const bool conv = tau_converged(tau, nt);
      tau = nt;
      if (conv) break;  // identical in every lane
    }
  }
  if (lane == 0) a.tau[bh] = tau;

  const float tdg = ud - tau;
  const bool dact = est ? (tdg > 0.f) : true;
  const float lwd = est ? (tdg > 0.f ? log2_prior<KIND>(tdg, a.beta) : -INFINITY) : 0.f;

  // ---- this head's routed chunks as words: chunk k*64 + l is bit l % 32 of
  // word 2k + l / 32; the own chunk ct (attended when dact) is bit ct % 32 of
  // word ct / 32 (ct >= ncomp, so no score test covers it)
  uint32_t myw[NWL];
#pragma unroll
  for (int i = 0; i < NWL; ++i) myw[i] = 0u;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const unsigned long long m64 = __ballot(u[k] - tau > 0.f);
    const int j0 = 2 * k, j1 = 2 * k + 1;
    myw[j0 / 64] = lane == (j0 & 63) ? (uint32_t)m64 : myw[j0 / 64];
    myw[j1 / 64] = lane == (j1 & 63) ? (uint32_t)(m64 >> 32) : myw[j1 / 64];
  }
#pragma unroll
  for (int i = 0; i < NWL; ++i)
    if (dact && (ct >> 5) == i * 64 + lane) myw[i] |= 1u << (ct & 31);
  uint32_t* bdst = a.bits ? a.bits + bh * (size_t)a.bits_words : nullptr;
  if (bdst) {
#pragma unroll
    for (int i = 0; i < NWL; ++i)
      if (i * 64 + lane < a.bits_words) bdst[i * 64 + lane] = myw[i];
    for (int wd = 64 * NWL + lane; wd < a.bits_words; wd += 64) bdst[wd] = 0u;
  }
#pragma unroll
  for (int i = 0; i < NWL; ++i) s_wb[w][i * 64 + lane] = myw[i];
  __syncthreads();

  // ---- the group's union words and their exclusive prefix counts, in every
  // wavefront (word i*64 + lane in register i)
  uint32_t uw[NWL];
  int upre[NWL];
  int acc = 0;
#pragma unroll
  for (int i = 0; i < NWL; ++i) {
    uint32_t x = 0u;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) x |= s_wb[hh][i * 64 + lane];
    uw[i] = x;
    const int c = __popc(x);
    int incl = c;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off);
      incl += lane >= off ? y : 0;
    }
    upre[i] = acc + incl - c;
    acc += __shfl(incl, kWave - 1);
  }
  const size_t gbase = (size_t)grp_id * a.n_slots;
  if (w == 0) {
    if (lane == 0) a.counts[grp_id] = acc;
    // the union list in ascending chunk order
#pragma unroll
    for (int i = 0; i < NWL; ++i) {
      uint32_t bits = uw[i];
      int pos = upre[i];
      while (bits) {
        const int bpos = __ffs(bits) - 1;
        a.lists[gbase + pos++] = (i * 64 + lane) * 32 + bpos;
        bits &= bits - 1u;
      }
    }
  }
  // ---- this head's log2 weight at each union entry it routed (the other
  // heads' entries are written by their wavefronts; an entry no head of the
  // group routed does not exist)
  uint32_t wk[KPL];
  int pk[KPL];
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int j = 2 * k + (lane >> 5);  // this lane's word for chunk k*64 + lane
    wk[k] = __shfl(uw[(2 * k) / 64], j & 63);
    pk[k] = __shfl(upre[(2 * k) / 64], j & 63);
  }
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int c = k * 64 + lane;
    if (c != ct && ((wk[k] >> (c & 31)) & 1u)) {
      const int pos = pk[k] + __popc(wk[k] & ((1u << (c & 31)) - 1u));
      const float tt = u[k] - tau;
      a.bias[(gbase + pos) * G + w] = tt > 0.f ? log2_prior<KIND>(tt, a.beta) : -INFINITY;
    }
  }
  {
    // the own chunk's entry (the shuffles with every lane active)
    const int jc = ct >> 5;
    uint32_t word = 0u;
    int pre = 0;
#pragma unroll
    for (int i = 0; i < NWL; ++i) {
      const uint32_t x = __shfl(uw[i], jc & 63);
      const int y = __shfl(upre[i], jc & 63);
      if (jc / 64 == i) {
        word = x;
        pre = y;
      }
    }
    if (lane == 0 && ((word >> (ct & 31)) & 1u))
      a.bias[(gbase + pre + __popc(word & ((1u << (ct & 31)) - 1u))) * G + w] = lwd;
  }
}

// ============================================================================
// launchers
// ============================================================================
template <int KIND>
static hipError_t route_prefill_kind(const RouteArgs& a, hipStream_t stream) {
  const int n_need = a.causal ? a.Nq / kChunk : a.n_slots;
  {
    const size_t work = std::max((size_t)a.B * a.Hkv * n_need * 16, (size_t)a.n_bhc);
    const int blocks = (int)std::min<size_t>((work + 255) / 256, 4096);
    hipLaunchKernelGGL(k_split_summaries, dim3(blocks), dim3(256), 0, stream, a, n_need);
  }
  dim3 grid(a.n_tiles, a.Hq, a.B);
  const unsigned n_grid_tiles = (unsigned)a.n_tiles * a.Hq * a.B;
  // the list-based kernel, then the general kernel for the tiles it queued
  if (a.n_slots <= kRouteRegSlots) {
    if (a.d == 64) hipLaunchKernelGGL((k_route_fast<KIND, kRouteRegSlots, 64>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_route_fast<KIND, kRouteRegSlots, 128>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.d == 64) hipLaunchKernelGGL((k_route_fast<KIND, kPrefillMaxSlots, 64>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_route_fast<KIND, kPrefillMaxSlots, 128>), grid, dim3(256), 0, stream, a);
  }
  const int nb = (a.n_slots + 15) / 16;
#define DASH_RP(NBV, GLB, GRID)                                                                  \
  if (nb <= NBV) {                                                                               \
    hipLaunchKernelGGL((k_route_prefill<NBV, KIND, GLB>), dim3(GRID), dim3(512), 0, stream, a); \
    return hipGetLastError();                                                                    \
  }
  DASH_RP(2, false, n_grid_tiles) DASH_RP(4, false, n_grid_tiles) DASH_RP(8, false, n_grid_tiles)
  DASH_RP(16, false, n_grid_tiles) DASH_RP(32, false, n_grid_tiles)
  DASH_RP(64, true, kRouteGlbGrid) DASH_RP(128, true, kRouteGlbGrid)
#undef DASH_RP
  return hipErrorInvalidValue;
}

hipError_t launch_route_prefill(const RouteArgs& a, hipStream_t stream) {
  if (a.alpha == 1.5f) return route_prefill_kind<2>(a, stream);
  if (a.alpha == 2.0f) return route_prefill_kind<1>(a, stream);
  return route_prefill_kind<0>(a, stream);
}

template <int G, int KIND>
static hipError_t route_decode_g(const RouteArgs& a, hipStream_t stream) {
  const int ncomp_max = (a.Lmax - 1) / kChunk;
  const int nwg = (ncomp_max + kDecScoreRowsPerWg - 1) / kDecScoreRowsPerWg;
  dim3 g1(nwg > 0 ? nwg : 1, a.B * a.Hkv);
  if (ncomp_max > 0) {
    if (a.d == 64) hipLaunchKernelGGL((k_route_decode_scores<G, 64>), g1, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_route_decode_scores<G, 128>), g1, dim3(256), 0, stream, a);
  }
  const int kpl = (ncomp_max + 63) / 64;
#define DASH_RD(K)                                                                              \
  if (kpl <= K) {                                                                               \
    hipLaunchKernelGGL((k_route_decode_tau<G, K, KIND>), dim3(a.B * a.Hkv), dim3(G * 64), 0, \
                       stream, a);                                                              \
    return hipGetLastError();                                                                   \
  }
  DASH_RD(1) DASH_RD(2) DASH_RD(4) DASH_RD(8) DASH_RD(16) DASH_RD(32) DASH_RD(64)
#undef DASH_RD
  return hipErrorInvalidValue;
}

template <int KIND>
static hipError_t route_decode_kind(const RouteArgs& a, hipStream_t stream) {
  switch (a.g) {
    case 1: return route_decode_g<1, KIND>(a, stream);
    case 2: return route_decode_g<2, KIND>(a, stream);
    case 4: return route_decode_g<4, KIND>(a, stream);
    case 8: return route_decode_g<8, KIND>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_route_decode(const RouteArgs& a, hipStream_t stream) {
  if (a.alpha == 1.5f) return route_decode_kind<2>(a, stream);
  if (a.alpha == 2.0f) return route_decode_kind<1>(a, stream);
  return route_decode_kind<0>(a, stream);
}

}  // namespace dash
