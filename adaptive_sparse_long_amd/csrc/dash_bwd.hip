// dash_bwd.hip -- backward of the DashAttention prefill. The DashAttention
// README calls the router "adaptive, differentiable" and has stage 3 use the
// stage-1 prior "to preserve differentiability through the hierarchy"
// ("Documentation", "How it works" item 3); no formula is printed, so this is
// the chain rule through the forward:
//
//   attention  l_ij = <q_i, k_j>/sqrt(d) + log w_{i,c(j)},  P = softmax_j(l),
//              dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i), D_i = sum_j P_ij dP_ij,
//              dQ_i += sum_j dS_ij k_j / sqrt(d),  dK_j += sum_i dS_ij q_i / sqrt(d),
//              dV_j += sum_i P_ij dO_i;
//   prior      g_ic = sum_{j in c} dS_ij is the gradient of log w_ic; a routed
//              chunk has w = pi (an own chunk attended with weight 1 is not a
//              routing candidate);
//   routing    pi_i = entmax_alpha(z_i): dz_ic = pi^(1-alpha) g - pi^(2-alpha) r_i
//              with r_i = sum_c pi^(1-alpha) g / sum_c pi^(2-alpha) over the
//              support (the published entmax Jacobian applied to d pi = g / pi);
//   scores     z_ic = scaling_factor <q_i, s_c> / sqrt(d): dQ_i += that factor
//              times sum_c dz_ic s_c, ds_c += the same factor times
//              sum_i dz_ic q_i; the own-chunk estimate's summary of tokens
//              [c_i C, i] passes its gradient to those keys and head_cls;
//   summaries  the summary backward of every routed chunk (dash_summarize_backward's kernels).
//
// Kernels (bf16 inputs, head_dim 64 or 128, chunk 64):
//   k_dbwd_prep  per row: the log2 weight of every chunk (log2 pi recomputed
//                from the float32 summaries, tau and the forward's routed-chunk
//                bits; 0 for an own chunk attended with weight 1), stored
//                column-major so that the rows of one chunk are contiguous;
//   k_dbwd_rows  row pass, a wavefront per 32 rows: the chunks any of its rows
//                attends are listed once; one sweep recomputes each row's
//                softmax normaliser (log2 domain) and D_i = sum_j P_ij dP_ij
//                (the exact <dO_i, O_i>, not the rounded output's), a second builds
//                S^T = K Q^T and dP^T = V dO^T by MFMA (a lane owns a row), P,
//                dS, g_c, and dQ^T += K^T dS^T (K staged transposed in LDS, dS
//                split into bf16 high and low parts); then the entmax Jacobian
//                per row gives dz, and dQ gets its routing term;
//   k_dbwd_cols  column pass, a wavefront per 32 keys of one chunk, over the g
//                query heads and the 32-row blocks that attend the chunk:
//                S = Q K^T, dP = dO V^T (a lane owns a key), P and dS from the
//                stored normaliser, dV^T += dO^T P, dK^T += Q^T dS, and the
//                chunk's summary gradient sum_i dz_ic q_i by one more product;
//   k_dbwd_est   (causal, estimate_diagonal) the own-chunk estimate's part of
//                dQ, dK and head_cls, per (b, kv head, chunk), on the vector ALUs;
//   then the summary backward of dS, and k_dbwd_combine (float32 sums to the
//   output dtype; dcls parts added in a fixed order).
// Every sum has a fixed order: the results are deterministic.
#include <algorithm>

#include "bwd_common.hpp"
#include "kernels.hpp"

namespace dash {

using namespace bwd;

namespace {
constexpr int D = 128;
constexpr int kMaxListed = kDashBwdMaxSlots;  // chunk slots a row pass can list
}  // namespace

// ---------------------------------------------------------------------------
// prep: one thread per row
// ---------------------------------------------------------------------------
// Every kernel below takes the caller's head_dim DC (the width of the rows of
// Q, K, V, dO, head_cls, S, the outputs and this backward's own arrays) as a
// template argument; at DC = 64 the 128-wide fragments and LDS layouts hold
// zeros in dims 64..127 and nothing is stored there.
template <int DC>
__global__ __launch_bounds__(256) void k_dbwd_prep(DashBwdArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  const int N = a.N;
  if (i >= N) return;
  const int b = (int)(bh / a.Hq), h = (int)(bh % a.Hq), hk = h / a.g;
  const size_t row = bh * N + i;
  u32x4 q[D / 8];  // the query row, bf16
  {
    const uint16_t* qp = a.Q + row * DC;
#pragma unroll
    for (int k = 0; k < D / 8; ++k) q[k] = 8 * k < DC ? ldg16(qp + 8 * k) : u32x4{0, 0, 0, 0};
  }
  auto qdot_f32 = [&](const float* s) {  // <q_i, s> with s float32
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < DC / 8; ++k) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(s + 8 * k);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + 8 * k + 4);
      z = fmaf(bf16lo(q[k][0]), s0[0], z); z = fmaf(bf16hi(q[k][0]), s0[1], z);
      z = fmaf(bf16lo(q[k][1]), s0[2], z); z = fmaf(bf16hi(q[k][1]), s0[3], z);
      z = fmaf(bf16lo(q[k][2]), s1[0], z); z = fmaf(bf16hi(q[k][2]), s1[1], z);
      z = fmaf(bf16lo(q[k][3]), s1[2], z); z = fmaf(bf16hi(q[k][3]), s1[3], z);
    }
    return z;
  };
  auto bdot = [](const u32x4* x, const uint16_t* y) {  // <x, y>, both bf16
    float z = 0.f;
#pragma unroll 4
    for (int k = 0; k < DC / 8; ++k) {
      const u32x4 v = ldg16(y + 8 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z = fmaf(bf16lo(x[k][e]), bf16lo(v[e]), z);
        z = fmaf(bf16hi(x[k][e]), bf16hi(v[e]), z);
      }
    }
    return z;
  };
  const float tau = a.tau[row];
  const uint32_t* bits = a.bits + row * a.bits_words;
  const int ci = i / kChunk;
  const int c_last = a.causal ? ci : a.n_slots - 1;
  const float* Sb = a.S + ((size_t)b * a.Hkv + hk) * a.s_cap * DC;
  float* wt = a.WT + bh * (size_t)a.n_slots * N + i;
  auto weight = [&](float u) { return u > tau ? a.beta * __log2f(u - tau) : -INFINITY; };
  for (int c = 0; c < a.n_slots; ++c) {
    float w = -INFINITY;
    if (c <= c_last && ((bits[c >> 5] >> (c & 31)) & 1u)) {
      if (a.causal && c == ci) {
        if (!a.est) {
          w = 0.f;  // attended with weight 1
        } else {
          // score against the summary of tokens [ci*C, i]: sum_j a_j <q, k_j>
          // with a = softmax(<k_j, cls> / sqrt(d)) over those tokens
          const uint16_t* kb = a.K + (((size_t)b * a.Hkv + hk) * a.Lmax + (size_t)ci * kChunk) * DC;
          u32x4 cl[D / 8];
#pragma unroll
          for (int k = 0; k < D / 8; ++k) cl[k] = 8 * k < DC ? ldg16(a.cls + (size_t)hk * DC + 8 * k) : u32x4{0, 0, 0, 0};
          const int nj = i - ci * kChunk + 1;
          float m = -INFINITY;
          for (int j = 0; j < nj; ++j) m = fmaxf(m, bdot(cl, kb + (size_t)j * DC) * a.inv_sqrt_d);
          float den = 0.f, num = 0.f;
          for (int j = 0; j < nj; ++j) {
            const float e = __expf(bdot(cl, kb + (size_t)j * DC) * a.inv_sqrt_d - m);
            den += e;
            num = fmaf(e, bdot(q, kb + (size_t)j * DC), num);
          }
          w = weight(a.uscale * (num / den));
        }
      } else {
        w = weight(a.uscale * qdot_f32(Sb + (size_t)c * DC));
      }
    }
    wt[(size_t)c * N] = w;
  }
}

// ---------------------------------------------------------------------------
// row pass
// ---------------------------------------------------------------------------
template <int DC>
__global__ __launch_bounds__(256) void k_dbwd_rows(DashBwdArgs a) {
  constexpr bool BF = true;
  __shared__ __attribute__((aligned(16))) uint16_t sKt[4][D * kTRow];
  __shared__ int s_list[4][kMaxListed];

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hi32 = lane >> 5;
  const size_t bh = blockIdx.y;
  const int b = (int)(bh / a.Hq), h = (int)(bh % a.Hq), hk = h / a.g;
  const int N = a.N;
  const int r0 = blockIdx.x * 128 + w * 32;
  if (r0 >= N) return;  // no row of this wavefront (no block barrier below)
  const int qi = r0 + (lane & 31);
  const bool row_ok = qi < N;
  const bool causal = a.causal != 0;
  const int ci = qi / kChunk;
  const size_t kvb = ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax * DC;
  const uint16_t* Kp = a.K + kvb;
  const uint16_t* Vp = a.V + kvb;
  const float* wt = a.WT + bh * (size_t)a.n_slots * N;
  float* dzt = a.DZT + bh * (size_t)a.n_slots * N;
  const float sc = a.scale_log2;

  Frags<BF, D> fq, fdo, fk, fv;
  load_frags<BF, D, DC>(fq, a.Q + bh * (size_t)N * DC, qi, row_ok);
  load_frags<BF, D, DC>(fdo, a.dO + bh * (size_t)N * DC, qi, row_ok);
  auto wrow = [&](int c) { return row_ok ? wt[(size_t)c * N + qi] : -INFINITY; };

  // ---- the chunks some row of the wavefront attends: the OR of the rows'
  // routed-chunk bits (a listed chunk whose recomputed weight is -inf for every
  // row only costs its visit), words loaded together
  const int c_end = causal ? min(r0 + 31, N - 1) / kChunk + 1 : a.n_slots;
  int* list = s_list[w];
  int nl = 0;
  {
    const uint32_t* brow = a.bits + (bh * N + min(qi, N - 1)) * (size_t)a.bits_words;
    const int nw = (c_end + 31) / 32;
    for (int w0 = 0; w0 < nw; w0 += 8) {
      uint32_t x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = (row_ok && w0 + k < nw) ? brow[w0 + k] : 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t u = x[k];
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) u |= __shfl_xor(u, off);
        const int wd = w0 + k;
        if (wd * 32 + 32 > c_end) u &= wd * 32 >= c_end ? 0u : ((1u << (c_end - wd * 32)) - 1u);
        u = __builtin_amdgcn_readfirstlane(u);
        while (u) {
          const int c = wd * 32 + __ffs(u) - 1;
          if (lane == 0) list[nl] = c;
          ++nl;
          u &= u - 1u;
        }
      }
    }
  }
  wave_lds_fence();

  // logits of the lane's row (exp2 domain) against keys 32 kb + 8 (r/4) + 4 hi32 + r%4
  auto logits = [&](int kb, float wc, const f32x16& s, f32x16& x) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb * 32 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
      const bool ok = row_ok && wc > -INFINITY && key < N && (!causal || key <= qi);
      x[r] = ok ? fmaf(s[r], sc, wc) : -INFINITY;
    }
  };

  // The listed chunks' 32-key halves are visited in order, the next half's K
  // and V fragments loaded while the current one is used (two fragment sets).
  // The row's weight for the chunk comes with them.
  Frags<BF, D> fk2, fv2;
  float wc1 = -INFINITY, wc2 = -INFINITY;
  auto load_half = [&](Frags<BF, D>& k_, Frags<BF, D>& v_, float& wc_, int j) {  // half j % 2 of entry j / 2
    const int c = list[j >> 1];
    const int kr = (2 * c + (j & 1)) * 32 + (lane & 31);
    load_frags<BF, D, DC>(k_, Kp, kr, kr < N);
    load_frags<BF, D, DC>(v_, Vp, kr, kr < N);
    wc_ = wrow(c);
  };
  // fn(k fragments, v fragments, weight, half index j) over every half, prefetching
  auto sweep = [&](auto&& fn) {
    if (nl > 0) load_half(fk, fv, wc1, 0);
    for (int e = 0; e < nl; ++e) {
      load_half(fk2, fv2, wc2, 2 * e + 1);
      fn(fk, fv, wc1, 2 * e);
      if (e + 1 < nl) load_half(fk, fv, wc1, 2 * e + 2);
      fn(fk2, fv2, wc2, 2 * e + 1);
    }
  };

  // ---- sweep 1: the softmax normaliser of every row and D_i = sum_j P_ij dP_ij
  // (= <dO_i, O_i> of the exact output), both online: l and t are rescaled
  // together whenever the running max grows
  float m = -INFINITY, l = 0.f, t = 0.f;
  sweep([&](const Frags<BF, D>& k_, const Frags<BF, D>& v_, float wc, int j) {
    const int c = list[j >> 1];
    const int kb = 2 * c + (j & 1);
    const f32x16 s = dot32<BF, D>(k_, fq);
    const f32x16 dp = dot32<BF, D>(v_, fdo);
    f32x16 x;
    logits(kb, wc, s, x);
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) bm = fmaxf(bm, x[r]);
    const float mn = fmaxf(m, bm);
    if (mn > -INFINITY) {
      float bl = 0.f, bt = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ex = fast_exp2(x[r] - mn);
        bl += ex;
        bt = fmaf(ex, dp[r], bt);
      }
      const float sc_old = fast_exp2(m - mn);
      l = fmaf(l, sc_old, bl);
      t = fmaf(t, sc_old, bt);
      m = mn;
    }
  });
  {
    const float mo = max_xor32(m);
    const float f = (mo > -INFINITY && m > -INFINITY) ? fast_exp2(m - mo) : 0.f;
    l = sum_xor32(l * f);
    t = sum_xor32(t * f);
    m = mo;
  }
  const float lse = (m > -INFINITY && l > 0.f) ? m + fast_log2(l) : INFINITY;
  const float Di = l > 0.f ? t / l : 0.f;
  if (lane < 32 && row_ok) {
    a.lse[bh * N + qi] = lse;
    a.Dd[bh * N + qi] = Di;
  }

  // ---- sweep 2: P, dS, g per chunk and dQ^T += K^T dS^T
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  uint16_t* kt = sKt[w];
  float gs = 0.f;
  sweep([&](const Frags<BF, D>& k_, const Frags<BF, D>& v_, float wc, int j) {
    const int c = list[j >> 1];
    const int kb = 2 * c + (j & 1);
    const f32x16 s = dot32<BF, D>(k_, fq);
    f32x16 dp = dot32<BF, D>(v_, fdo);
    f32x16 x;
    logits(kb, wc, s, x);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(x[r] - lse);  // 0 where masked (x = -inf)
      const float ds = p * (dp[r] - Di);
      gs += ds;
      dp[r] = ds;
    }
    stage_t_regs<D>(kt, k_);
    wave_lds_fence();
    acc_xt_w<BF, D>(acc, dp, kt, nullptr, 0, 0);
    wave_lds_fence();
    if (j & 1) {
      const float g = sum_xor32(gs);
      if (row_ok) dzt[(size_t)c * N + qi] = g;  // both lanes of the row write the same value
      gs = 0.f;
    }
  });

  // ---- routing: the entmax Jacobian over the row's candidates
  // candidate: a past chunk; the own chunk only with the estimate (causal); every chunk (non-causal)
  auto candidate = [&](int c) { return !causal || c < ci || (a.est && c == ci); };
  // (weight, g) of entry e, the next entry's requested before this one is used
  auto wg = [&](int e, float& wc_, float& g_) {
    const int c = list[e];
    wc_ = wrow(c);
    g_ = row_ok ? dzt[(size_t)c * N + qi] : 0.f;
  };
  float A1 = 0.f, A2 = 0.f;
  {
    float wn = -INFINITY, gn = 0.f;
    if (nl > 0) wg(0, wn, gn);
    for (int e = 0; e < nl; ++e) {
      const int c = list[e];
      const float wc = wn, g = gn;
      if (e + 1 < nl) wg(e + 1, wn, gn);
      if (candidate(c) && wc > -INFINITY) {
        A1 = fmaf(fast_exp2((1.f - a.alpha) * wc), g, A1);
        A2 += fast_exp2((2.f - a.alpha) * wc);
      }
    }
  }
  const float ratio = A2 > 0.f ? A1 / A2 : 0.f;
  // dQ = acc / sqrt(d) + rt * sum_c dz_c s_c: the routing term enters acc times sqrt(d) = sf / rt
  const float* Sb = a.S + ((size_t)b * a.Hkv + hk) * a.s_cap * DC;
  float wn = -INFINITY, gn = 0.f;
  if (nl > 0) wg(0, wn, gn);
  for (int e = 0; e < nl; ++e) {
    const int c = list[e];
    const float wc = wn, g = gn;
    if (e + 1 < nl) wg(e + 1, wn, gn);
    float dz = 0.f;
    if (candidate(c) && wc > -INFINITY)
      dz = fmaf(fast_exp2((1.f - a.alpha) * wc), g, -fast_exp2((2.f - a.alpha) * wc) * ratio);
    if (row_ok) dzt[(size_t)c * N + qi] = dz;
    // the own chunk's estimate passes its gradient on in k_dbwd_est
    if (dz != 0.f && !(causal && c == ci)) {
      const float f = a.sf * dz;
      const float* sr = Sb + (size_t)c * DC + 4 * hi32;
#pragma unroll
      for (int db = 0; db < DC / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sr + 32 * db + 8 * q4);
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[db][4 * q4 + k] = fmaf(f, v[k], acc[db][4 * q4 + k]);
        }
    }
  }
  if (row_ok) store_line<false, D, DC>(a.dQf, bh * N + qi, acc, a.inv_sqrt_d);
}

// ---------------------------------------------------------------------------
// column pass
// ---------------------------------------------------------------------------
template <int DC>
__global__ __launch_bounds__(256) void k_dbwd_cols(DashBwdArgs a) {
  constexpr bool BF = true;
  constexpr int LC = 512;  // pair list entries per wavefront
  __shared__ __attribute__((aligned(16))) uint16_t sQt[4][D * kTRow];
  __shared__ __attribute__((aligned(16))) uint16_t sOt[4][D * kTRow];
  __shared__ __attribute__((aligned(16))) float sRow[4][4][32];
  __shared__ int sRowIdx[4][32];
  __shared__ int s_pairs[4][LC];  // (head in group << 20) | row

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hi32 = lane >> 5;
  const int b = blockIdx.z, hk = blockIdx.y;
  const int N = a.N;
  const int k0 = blockIdx.x * 128 + w * 32;
  if (k0 >= N) return;  // no key of this wavefront (no block barrier below)
  const int kj = k0 + (lane & 31);
  const bool key_ok = kj < N;
  const bool causal = a.causal != 0;
  const int c = k0 / kChunk;
  const bool first_half = (k0 % kChunk) == 0;  // this wavefront also sums the chunk's summary gradient
  const size_t kvb = ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax * DC;
  const float sc = a.scale_log2;

  Frags<BF, D> fk, fv, fq, fdo;
  load_frags<BF, D, DC>(fk, a.K + kvb, kj, key_ok);
  load_frags<BF, D, DC>(fv, a.V + kvb, kj, key_ok);
  f32x16 dk[D / 32], dv[D / 32], dsum[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
      dsum[db][r] = 0.f;
    }
  uint16_t* qt = sQt[w];
  uint16_t* ot = sOt[w];
  float* srw = sRow[w][0];
  float* srl = sRow[w][1];
  float* srd = sRow[w][2];
  float* srz = sRow[w][3];
  int* sri = sRowIdx[w];
  int* pairs = s_pairs[w];
  const size_t bh0 = (size_t)b * a.Hq + hk * a.g;

  // ---- 32 listed (head, row) pairs attending chunk c at a time: their query and
  // dO rows gathered (a lane per pair), S^T and dP^T against the wavefront's 32
  // keys, then dV^T += dO^T P, dK^T += Q^T dS and the chunk's summary gradient
  auto process = [&](int e0, int ne) {
    const int m = lane & 31;
    const bool ok = m < ne;
    const int ent = ok ? pairs[e0 + m] : 0;
    const int hh = ent >> 20, row = ent & 0xfffff;
    const size_t bh = bh0 + hh;
    load_frags<BF, D, DC>(fq, a.Q + bh * (size_t)N * DC, row, ok);
    load_frags<BF, D, DC>(fdo, a.dO + bh * (size_t)N * DC, row, ok);
    const f32x16 s = dot32<BF, D>(fq, fk);    // S[pair][key]
    const f32x16 dp = dot32<BF, D>(fdo, fv);  // dP[pair][key]
    if (lane < 32) {
      const float wq = ok ? a.WT[(bh * a.n_slots + c) * (size_t)N + row] : -INFINITY;
      srw[m] = wq;
      srl[m] = ok ? a.lse[bh * N + row] : 0.f;
      srd[m] = ok ? a.Dd[bh * N + row] : 0.f;
      // the summary gradient takes dz of rows that route c as a past (or,
      // non-causal, any) chunk
      srz[m] = (ok && wq > -INFINITY && (!causal || row / kChunk > c))
                   ? a.DZT[(bh * a.n_slots + c) * (size_t)N + row] : 0.f;
      sri[m] = ok ? row : -1;
    }
    wave_lds_fence();
    f32x16 p, ds, z;
    bool any_z = false;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 wv = *reinterpret_cast<const f32x4*>(srw + 8 * g4 + 4 * hi32);
      const f32x4 lv = *reinterpret_cast<const f32x4*>(srl + 8 * g4 + 4 * hi32);
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(srd + 8 * g4 + 4 * hi32);
      const f32x4 zv = *reinterpret_cast<const f32x4*>(srz + 8 * g4 + 4 * hi32);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 4 * g4 + k;
        const int q = sri[8 * g4 + 4 * hi32 + k];
        const bool on = key_ok && q >= 0 && (!causal || kj <= q) && wv[k] > -INFINITY;
        const float pr = on ? fast_exp2(fmaf(s[r], sc, wv[k]) - lv[k]) : 0.f;
        p[r] = pr;
        ds[r] = pr * (dp[r] - dv4[k]);
        z[r] = zv[k];
        any_z = any_z || zv[k] != 0.f;
      }
    }
    stage_t_regs<D>(qt, fq);
    stage_t_regs<D>(ot, fdo);
    wave_lds_fence();
    acc_xt_w<BF, D>(dv, p, ot, nullptr, 0, 0);
    acc_xt_w<BF, D>(dk, ds, qt, nullptr, 0, 0);
    if (first_half && wave_any(any_z)) acc_xt_w<BF, D>(dsum, z, qt, nullptr, 0, 0);
    // the next block overwrites the LDS slots only after every lane has read them
    wave_lds_fence();
  };

  // ---- the pairs: rows (that can see a key of this wavefront) whose weight for
  // chunk c is finite, in (head, row) order, 256 rows of a head per step (four
  // per lane), two steps' loads in flight; full blocks of 32 are processed
  // whenever the list nears its capacity, the rest at the end
  const int r_begin = causal ? k0 : 0;
  int np = 0;
  for (int hh = 0; hh < a.g; ++hh) {
    const float* wtc = a.WT + ((bh0 + hh) * a.n_slots + c) * (size_t)N;
    for (int r = r_begin; r < N; r += 512) {
      float wv[2][4];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int rr = r + 256 * st + 4 * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) wv[st][k] = rr + k < N ? wtc[rr + k] : -INFINITY;
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int rr = r + 256 * st + 4 * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bool on = wv[st][k] > -INFINITY;
          const uint64_t bm = __ballot(on);
          const int pos = np + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
          if (on) pairs[pos] = (hh << 20) | (rr + k);
          np += __popcll(bm);
        }
        if (np > LC - 256) {
          wave_lds_fence();
          const int full = np & ~31;
          for (int e0 = 0; e0 < full; e0 += 32) process(e0, 32);
          const int rest = np - full;
          const int moved = lane < rest ? pairs[full + lane] : 0;
          wave_lds_fence();
          if (lane < rest) pairs[lane] = moved;
          np = rest;
        }
      }
    }
  }
  wave_lds_fence();
  for (int e0 = 0; e0 < np; e0 += 32) process(e0, min(32, np - e0));

  if (key_ok) {
    store_line<false, D, DC>(a.dKf, ((size_t)b * a.Hkv + hk) * N + kj, dk, a.inv_sqrt_d);
    store_line<true, D, DC>(a.dV, ((size_t)b * a.Hkv + hk) * a.Lmax + kj, dv, 1.f);
  }
  // every key column of dsum holds the same vector; lanes 0 and 32 store it
  if (first_half && (lane & 31) == 0) store_line<false, D, DC>(a.dSum, ((size_t)b * a.Hkv + hk) * a.n_slots + c, dsum, a.rt);
}

// ---------------------------------------------------------------------------
// own-chunk estimate (causal, estimate_diagonal): row i's own chunk was scored
// against s^_i = sum_{j <= i} a_ij k_j, a_i = softmax(<k_j, cls> / sqrt(d)) over
// the chunk's tokens up to i. With kappa_i = rt dz_i,own:
//   dQ_i += kappa_i s^_i;  ds^_i = kappa_i q_i, and through the summary
//   de_ij = a_ij (<k_j, ds^_i> - <s^_i, ds^_i>),
//   dK_j += a_ij ds^_i + de_ij cls / sqrt(d),  dcls += sum_j de_ij k_j / sqrt(d).
// One workgroup per (b, kv head, chunk) over the g heads' rows of the chunk.
// ---------------------------------------------------------------------------
template <int DC>
__global__ __launch_bounds__(256) void k_dbwd_est(DashBwdArgs a) {
  __shared__ float sK[kChunk][D + 1];
  __shared__ float sq[D], scl[D], se[kChunk], sa[kChunk], skq[kChunk], sde[kChunk];
  const int c = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int N = a.N;
  const int t = threadIdx.x;
  const int nk = min(kChunk, N - c * kChunk);
  const size_t kvb = ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax * DC;
  for (int x = t; x < kChunk * D; x += 256) {
    const int j = x / D, dd = x % D;
    sK[j][dd] = j < nk && dd < DC ? __uint_as_float(((uint32_t)a.K[kvb + (size_t)(c * kChunk + j) * DC + dd]) << 16) : 0.f;
  }
  if (t < D) scl[t] = t < DC ? __uint_as_float(((uint32_t)a.cls[(size_t)hk * DC + t]) << 16) : 0.f;
  __syncthreads();
  if (t < kChunk) {
    float e = 0.f;
    for (int dd = 0; dd < D; ++dd) e = fmaf(sK[t][dd], scl[dd], e);
    se[t] = e * a.inv_sqrt_d;
  }
  // thread t: key jt = t / 4, dims 32 (t % 4) .. +31 of dk; threads t < D: dim t of dcls
  const int jt = t >> 2, d0 = 32 * (t & 3);
  float dk[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) dk[k] = 0.f;
  float dcl = 0.f;
  for (int hh = 0; hh < a.g; ++hh) {
    const size_t bh = (size_t)b * a.Hq + hk * a.g + hh;
    const float* dztc = a.DZT + (bh * a.n_slots + c) * (size_t)N;
    const float* wtc = a.WT + (bh * a.n_slots + c) * (size_t)N;
    for (int il = 0; il < nk; ++il) {
      const int i = c * kChunk + il;
      // uniform; dz is stored only for rows that attend their own chunk
      const float kappa = wtc[i] > -INFINITY ? a.rt * dztc[i] : 0.f;
      if (kappa == 0.f) continue;
      __syncthreads();  // the previous row's shared values are no longer read
      if (t < D) sq[t] = t < DC ? __uint_as_float(((uint32_t)a.Q[(bh * N + i) * DC + t]) << 16) : 0.f;
      __syncthreads();
      if (t < kChunk) {  // wavefront 0: prefix softmax weights and <k_j, q_i>
        const bool on = t <= il;
        const float e = on ? se[t] : -INFINITY;
        const float mx = wave_max(e);
        const float ex = on ? __expf(e - mx) : 0.f;
        const float den = wave_sum(ex);
        const float aj = ex / den;
        float kq = 0.f;
        for (int dd = 0; dd < D; ++dd) kq = fmaf(sK[t][dd], sq[dd], kq);
        sa[t] = aj;
        skq[t] = kq;
        const float sqv = wave_sum(aj * kq);
        sde[t] = aj * kappa * (kq - sqv);
      }
      __syncthreads();
      if (t < D) {
        float shat = 0.f, dc = 0.f;
        for (int j = 0; j <= il; ++j) {
          shat = fmaf(sa[j], sK[j][t], shat);
          dc = fmaf(sde[j], sK[j][t], dc);
        }
        if (t < DC) a.dQf[(bh * N + i) * DC + t] += kappa * shat;
        dcl = fmaf(dc, a.inv_sqrt_d, dcl);
      }
      if (jt <= il) {
        const float aj = sa[jt] * kappa, dej = sde[jt] * a.inv_sqrt_d;
#pragma unroll
        for (int k = 0; k < 32; ++k) dk[k] = fmaf(aj, sq[d0 + k], fmaf(dej, scl[d0 + k], dk[k]));
      }
    }
  }
  if (jt < nk && d0 < DC) {
    float* dst = a.dKf + (((size_t)b * a.Hkv + hk) * N + (size_t)c * kChunk + jt) * DC + d0;
#pragma unroll
    for (int k = 0; k < 32; ++k) dst[k] += dk[k];
  }
  if (t < DC) a.dcls_p[(((size_t)b * a.Hkv + hk) * a.n_slots + c) * DC + t] = dcl;
}

// ---------------------------------------------------------------------------
// combine: dQ, dK to the output dtype; dcls = summary part + estimate parts (fixed order)
// ---------------------------------------------------------------------------
template <int DC>
__global__ __launch_bounds__(256) void k_dbwd_combine(DashBwdArgs a) {
  const size_t nq = (size_t)a.B * a.Hq * a.N * DC;
  const size_t nk = (size_t)a.B * a.Hkv * a.N * DC;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint16_t* dQ = static_cast<uint16_t*>(a.dQ);
  uint16_t* dK = static_cast<uint16_t*>(a.dK);
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < nq; x += stride)
    dQ[x] = __builtin_bit_cast(uint16_t, (__bf16)a.dQf[x]);
  const int n_sum_rows = a.n_sum * kChunk;
  for (size_t x = blockIdx.x * (size_t)blockDim.x + threadIdx.x; x < nk; x += stride) {
    const size_t line = x / DC;
    const int dd = (int)(x % DC);
    const int j = (int)(line % a.N);
    const size_t bhk = line / a.N;
    float v = a.dKf[x];
    if (j < n_sum_rows) v += a.dKs[(bhk * a.Lmax + j) * DC + dd];
    dK[(bhk * a.Lmax + j) * DC + dd] = __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  if (blockIdx.x < (unsigned)a.Hkv && threadIdx.x < DC) {
    const int hk = blockIdx.x;
    float v = a.dcls_s[(size_t)hk * DC + threadIdx.x];
    if (a.causal && a.est)
      for (int b = 0; b < a.B; ++b)
        for (int c = 0; c < a.n_slots; ++c) v += a.dcls_p[(((size_t)b * a.Hkv + hk) * a.n_slots + c) * DC + threadIdx.x];
    a.dcls[(size_t)hk * DC + threadIdx.x] = v;
  }
}

template <int DC>
static hipError_t dash_bwd_dc(const DashBwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_dbwd_prep<DC>, dim3((a.N + 255) / 256, a.B * a.Hq), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(k_dbwd_rows<DC>, dim3((a.N + 127) / 128, a.B * a.Hq), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(k_dbwd_cols<DC>, dim3((a.N + 127) / 128, a.Hkv, a.B), dim3(256), 0, stream, a);
  if (a.causal && a.est) hipLaunchKernelGGL(k_dbwd_est<DC>, dim3(a.n_slots, a.Hkv, a.B), dim3(256), 0, stream, a);
  // the summaries' backward for dS = dSum
  SummarizeBwdArgs sb{a.K, a.cls, a.dSum, a.dKs, a.dcls_s, a.sb_part, a.B, a.Hkv, a.Lmax, DC, a.N,
                      0, a.n_sum, a.n_slots, kChunk, a.inv_sqrt_d};
  hipError_t e = launch_summarize_bwd(sb, stream);
  if (e != hipSuccess) return e;
  const size_t nq = (size_t)a.B * a.Hq * a.N * DC;
  const unsigned grid = (unsigned)std::min<size_t>((nq + 255) / 256, 8192);
  hipLaunchKernelGGL(k_dbwd_combine<DC>, dim3(std::max<unsigned>(grid, (unsigned)a.Hkv)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dash_bwd(const DashBwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? dash_bwd_dc<64>(a, stream) : dash_bwd_dc<128>(a, stream);
}

}  // namespace dash
