// route.hip -- stage 2 of the DashAttention hierarchy ("How it works" 2 on the
// DashAttention README page): query-to-summary routing scores, alpha-entmax over
// them (threshold by Halley + bisection, AdaSplash README "Usage: Triton
// Entmax"), the routed set (the entmax support) and the routing prior, packed as
// work lists for the stage-3 attention kernels.
//
// Prefill: one workgroup of eight wavefronts per (b, query head, 128-row tile).
// Each wavefront owns 16 query rows and keeps all their routing scores in
// registers (16 rows x up to 512 chunks, the 16x16 MFMA output layout: every
// lane holds 4 rows of one chunk per 16-chunk block), so the tau iterations
// re-read registers, not memory. Scores come from v_mfma_f32_16x16x32_bf16 with
// each float32 summary split into bf16 high and low parts (q is exact in bf16),
// which keeps about 16 mantissa bits at bf16 MFMA rate. Row reductions are DPP
// sums over the 16 lanes of a row group. The routed chunks of the 128 rows are
// OR-ed into an LDS bitmask, compacted into an ascending list, and each row's
// log2 prior for every listed chunk is written next to it.
//
// Decode: a bandwidth-bound score kernel streams the float32 summary cache once
// (eight lanes per summary row, four float4 loads each, all g query heads of a
// KV head at once), then one workgroup per (b, kv head) solves tau for its g
// query heads (one wavefront each, 32+ candidates per lane), takes the union of
// their routed chunks and writes the list with g log2 priors per chunk.
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
template <int NB, int KIND>
__global__ __launch_bounds__(512) void k_route_prefill(RouteArgs a) {
  constexpr int D = 128;
  constexpr int NS = D / 32;                // k-steps of the 16x16x32 MFMA
  constexpr int NW = (NB * 16 + 31) / 32;   // union words
  __shared__ uint32_t s_union[NW];
  __shared__ int s_pre[NW + 1];

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
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
  const int ncomp = causal ? cw : n_slots;
  const int nblk = (ncomp + 15) / 16;
  const int ncand = ncomp + (est ? 1 : 0);

  if (threadIdx.x < NW) s_union[threadIdx.x] = 0u;

  const size_t bh = (size_t)b * a.Hq + h;
  const uint16_t* Qb = a.Q + bh * (size_t)N * D;
  const float* Sb = a.S + ((size_t)b * a.Hkv + hk) * (size_t)a.s_cap * D;

  // ---- q as A operand: row i0 + col, dims 32 s + 8 grp .. +7
  bf16x8 qa[NS];
  {
    const int qi = i0 + col;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qa[s] = as_bf16x8(qi < N ? ldg16(Qb + (size_t)qi * D + 32 * s + 8 * grp) : zero4());
  }

  // ---- routing scores in u units: u[blk][r] for chunk blk*16 + col, row grp*4 + r
  const float uscale = (a.alpha - 1.f) * a.zscale;
  float u[NB][4];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    if (wave_valid && blk < nblk) {
      const int c = blk * 16 + col;
      const bool cval = c < ncomp;
      const float* sp = Sb + (size_t)c * D + 8 * grp;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (cval) {
          x0 = *reinterpret_cast<const f32x4*>(sp + 32 * s);
          x1 = *reinterpret_cast<const f32x4*>(sp + 32 * s + 4);
        }
        bf16x8 hi, lo;
        split_hi_lo(x0, x1, hi, lo);
        acc = mfma16x16x32(qa[s], hi, acc);
        acc = mfma16x16x32(qa[s], lo, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) u[blk][r] = cval ? acc[r] * uscale : -INFINITY;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) u[blk][r] = -INFINITY;
    }
  }

  // ---- own-chunk estimate: score against the summary of tokens [cw*C, i]
  float ud[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (est && wave_valid) {
    const uint16_t* kp = a.K + (((size_t)b * a.Hkv + hk) * a.Lmax + (size_t)cw * kChunk) * D;
    float wc[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 cv = ldg16(a.cls + (size_t)hk * D + 32 * s + 8 * grp);
      for (int e = 0; e < 4; ++e) {
        wc[s][2 * e] = bf16lo(cv[e]);
        wc[s][2 * e + 1] = bf16hi(cv[e]);
      }
    }
    f32x4 qk[4];
    float lc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = kb * 16 + col;
      const bool kval = cw * kChunk + key < N;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        u32x4 kv = kval ? ldg16(kp + (size_t)key * D + 32 * s + 8 * grp) : zero4();
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
      for (int kb = 0; kb < 4; ++kb)
        if (kb * 16 + col <= pi) mloc = fmaxf(mloc, lc[kb]);
      const float M = max16(mloc);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb * 16 + col <= pi) {
          const float e = exp2f((lc[kb] - M) * kLog2e);
          num = fmaf(e, qk[kb][r], num);
          den += e;
        }
      }
      num = sum16(num);
      den = sum16(den);
      ud[r] = (num / den) * uscale;
    }
  }

  // ---- tau per row (all 16 lanes of a row group hold the same values)
  float tau[4];
  bool row_ok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) row_ok[r] = wave_valid && (i0 + grp * 4 + r < N);
  if (wave_valid && ncand > 0) {
    float lo[4], hi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) m = fmaxf(m, u[blk][r]);
      m = fmaxf(max16(m), ud[r]);
      lo[r] = m - 1.f;
      hi[r] = tau_upper(m, ncand, a.alpha);
      tau[r] = lo[r];
    }
    for (int it = 0; it < a.n_iter; ++it) {
      float f0[4] = {0.f, 0.f, 0.f, 0.f}, f1[4] = {0.f, 0.f, 0.f, 0.f}, f2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        if (blk < nblk) {
#pragma unroll
          for (int r = 0; r < 4; ++r) tau_terms<KIND>(u[blk][r], tau[r], a.beta, f0[r], f1[r], f2[r]);
        }
      }
      bool conv = true;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f0[r] = sum16(f0[r]);
        f1[r] = sum16(f1[r]);
        if (KIND != 1) f2[r] = sum16(f2[r]);
        if (est) tau_terms<KIND>(ud[r], tau[r], a.beta, f0[r], f1[r], f2[r]);
        const float nt = tau_step<KIND>(tau[r], f0[r], f1[r], f2[r], a.beta, lo[r], hi[r]);
        conv = conv && tau_converged(tau[r], nt);
        tau[r] = nt;
      }
      if (wave_all(conv)) break;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) tau[r] = INFINITY;
  }

  // ---- tau output: lanes 0, 16, 32, 48 hold rows grp*4 .. +3
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row_ok[r]) a.tau[bh * (size_t)N + i0 + grp * 4 + r] = tau[r];
  }

  // ---- routed flags and log2 weights
  bool dact[4];
  float lwd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float td = ud[r] - tau[r];
    dact[r] = row_ok[r] && (est ? (td > 0.f) : causal);
    lwd[r] = est ? ((row_ok[r] && td > 0.f) ? log2_prior<KIND>(td, a.beta) : -INFINITY)
                 : (row_ok[r] ? 0.f : -INFINITY);
  }

  // ---- union of routed chunks over the 128 rows, and the per-row bitmask
  // output (lanes 0..15 write row i0 + lane). Ballots run with all lanes active.
  __syncthreads();  // s_union cleared
  unsigned long long md[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) md[r] = __ballot(dact[r]);
  const bool write_bits = a.bits != nullptr && wave_valid && lane < 16 && i0 + lane < N;
  const int rg = lane >> 2, rr = lane & 3;  // D-layout owner of row `lane`
  const bool dl = ((rr == 0 ? md[0] : rr == 1 ? md[1] : rr == 2 ? md[2] : md[3]) >> (16 * rg)) & 1ull;
  uint32_t* bdst = a.bits + ((bh * (size_t)N) + i0 + lane) * (size_t)a.bits_words;
#pragma unroll
  for (int wd = 0; wd < NW; ++wd) {
    uint32_t word = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int blk = 2 * wd + half;
      if (blk < NB) {
        unsigned long long mb[4];
        bool any = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool act = row_ok[r] && (u[blk][r] - tau[r] > 0.f);
          mb[r] = __ballot(act);
          any = any || act;
        }
        const unsigned long long ma = __ballot(any);
        const uint32_t m16 = (uint32_t)((ma | (ma >> 16) | (ma >> 32) | (ma >> 48)) & 0xffffull);
        if (lane == 0 && m16) atomicOr(&s_union[blk >> 1], m16 << (16 * (blk & 1)));
        const unsigned long long mr = rr == 0 ? mb[0] : rr == 1 ? mb[1] : rr == 2 ? mb[2] : mb[3];
        word |= (uint32_t)((mr >> (16 * rg)) & 0xffffull) << (16 * half);
      }
    }
    if (causal && dl && (cw >> 5) == wd) word |= 1u << (cw & 31);
    if (write_bits && wd < a.bits_words) bdst[wd] = word;
  }
  if (write_bits)
    for (int wd = NW; wd < a.bits_words; ++wd) bdst[wd] = 0u;
  if (causal && wave_valid) {
    const bool anyd = (md[0] | md[1] | md[2] | md[3]) != 0ull;
    if (lane == 0 && anyd) atomicOr(&s_union[cw >> 5], 1u << (cw & 31));
  }

  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int wd = 0; wd < NW; ++wd) {
      s_pre[wd] = acc;
      acc += __popc(s_union[wd]);
    }
    s_pre[NW] = acc;
    a.counts[bh * a.n_tiles + tile] = acc;
  }
  __syncthreads();

  const long long toff = bh * a.per_head + prefill_tile_offset(tile, n_slots, causal);
  if (threadIdx.x < NW) {
    uint32_t bits = s_union[threadIdx.x];
    int pos = s_pre[threadIdx.x];
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      a.lists[toff + pos++] = threadIdx.x * 32 + bpos;
      bits &= bits - 1u;
    }
  }

  // ---- log2 weights of this wavefront's 16 rows for every listed chunk
  if (wave_valid) {
    float* bias = a.bias + toff * kTileRows + w * 16;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int c = blk * 16 + col;
      const uint32_t word = s_union[c >> 5];
      if (((word >> (c & 31)) & 1u) && !(causal && c == cw)) {
        const int pos = s_pre[c >> 5] + __popc(word & ((1u << (c & 31)) - 1u));
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t = u[blk][r] - tau[r];
          v[r] = (row_ok[r] && t > 0.f) ? log2_prior<KIND>(t, a.beta) : -INFINITY;
        }
        *reinterpret_cast<f32x4*>(bias + (size_t)pos * kTileRows + grp * 4) = v;
      }
    }
    if (causal && col == 0) {
      const uint32_t word = s_union[cw >> 5];
      if ((word >> (cw & 31)) & 1u) {
        const int pos = s_pre[cw >> 5] + __popc(word & ((1u << (cw & 31)) - 1u));
        f32x4 v = {lwd[0], lwd[1], lwd[2], lwd[3]};
        *reinterpret_cast<f32x4*>(bias + (size_t)pos * kTileRows + grp * 4) = v;
      }
    }
  } else {
    // rows past N: every listed chunk gets -inf so the attention pass skips them
    float* bias = a.bias + toff * kTileRows + w * 16;
    const int cnt = s_pre[NW];
    for (int pos = lane; pos < cnt * 16; pos += kWave) bias[(size_t)(pos >> 4) * kTileRows + (pos & 15)] = -INFINITY;
  }
}

// ============================================================================
// Decode routing
// ============================================================================
// Scores of the complete chunks against the g query heads of one KV head:
// eight lanes per summary row (four float4 each), 16 rows per wavefront.
template <int G>
__global__ __launch_bounds__(256) void k_route_decode_scores(RouteArgs a) {
  constexpr int D = 128;
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int grp_id = blockIdx.y;
  const int b = grp_id / a.Hkv;
  const int hk = grp_id % a.Hkv;
  const int t = min(max(a.seqlens[b], 1), a.Lmax) - 1;  // clamp to the cache
  const int ncomp = t / kChunk;
  const int c0 = blockIdx.x * 64 + w * 16;
  if (c0 >= ncomp) return;
  const int sub = lane & 7;
  float q[G][16];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint16_t* qp = a.Q + ((size_t)b * a.Hq + hk * G + hh) * D;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x2 v = *reinterpret_cast<const u32x2*>(qp + 32 * k + 4 * sub);
      q[hh][4 * k + 0] = bf16lo(v[0]);
      q[hh][4 * k + 1] = bf16hi(v[0]);
      q[hh][4 * k + 2] = bf16lo(v[1]);
      q[hh][4 * k + 3] = bf16hi(v[1]);
    }
  }
  const float* Sb = a.S + ((size_t)b * a.Hkv + hk) * (size_t)a.s_cap * D;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = c0 + pass * 8 + (lane >> 3);
    const bool val = c < ncomp;
    f32x4 sv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      sv[k] = val ? *reinterpret_cast<const f32x4*>(Sb + (size_t)c * D + 32 * k + 4 * sub)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
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
template <int G, int KPL, int KIND>
__global__ __launch_bounds__(G * 64) void k_route_decode_tau(RouteArgs a) {
  constexpr int D = 128;
  constexpr int NWD = 2 * KPL + 1;
  __shared__ uint32_t s_union[NWD];
  __shared__ int s_pre[NWD + 1];
  __shared__ float s_lc[G][64];
  __shared__ float s_qk[G][64];

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int grp_id = blockIdx.x;
  const int b = grp_id / a.Hkv;
  const int hk = grp_id % a.Hkv;
  const int h = hk * G + w;
  const int t = min(max(a.seqlens[b], 1), a.Lmax) - 1;  // clamp to the cache
  const int ct = t / kChunk;
  const int ncomp = ct;
  const bool est = a.est != 0;
  const int ncand = ncomp + (est ? 1 : 0);
  for (int i = threadIdx.x; i < NWD; i += blockDim.x) s_union[i] = 0u;

  const size_t bh = (size_t)b * a.Hq + h;
  const float am1 = a.alpha - 1.f;

  // ---- own-chunk estimate from the tokens [ct*C, t]
  float ud = -INFINITY;
  if (est) {
    const int sub = lane & 15, rg = lane >> 4;
    float wq[8], wc[8];
    {
      u32x4 qv = ldg16(a.Q + bh * D + 8 * sub);
      u32x4 cv = ldg16(a.cls + (size_t)hk * D + 8 * sub);
      for (int e = 0; e < 4; ++e) {
        wq[2 * e] = bf16lo(qv[e]);
        wq[2 * e + 1] = bf16hi(qv[e]);
        wc[2 * e] = bf16lo(cv[e]);
        wc[2 * e + 1] = bf16hi(cv[e]);
      }
    }
    const int nval = t - ct * kChunk + 1;
    const uint16_t* kp = a.K + (((size_t)b * a.Hkv + hk) * a.Lmax + (size_t)ct * kChunk) * D;
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int key = r * 4 + rg;
      const bool val = key < nval;
      u32x4 kv = val ? ldg16(kp + (size_t)key * D + 8 * sub) : zero4();
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
    const float e = (lcv > -INFINITY) ? exp2f((lcv - M) * kLog2e) : 0.f;
    const float num = wave_sum(e * qkv);
    const float den = wave_sum(e);
    ud = (num / den) * a.zscale * am1;
  }

  // ---- scores of complete chunks c = k*64 + lane
  float u[KPL];
  const float* zrow = a.z + bh * a.n_slots;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int c = k * 64 + lane;
    u[k] = c < ncomp ? zrow[c] * am1 : -INFINITY;
  }
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
#pragma unroll
      for (int k = 0; k < KPL; ++k) tau_terms<KIND>(u[k], tau, a.beta, f0, f1, f2);
      f0 = wave_sum(f0);
      f1 = wave_sum(f1);
      if (KIND != 1) f2 = wave_sum(f2);
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

  __syncthreads();  // s_union cleared; s_lc/s_qk no longer needed
  uint32_t* bdst = a.bits ? a.bits + bh * (size_t)a.bits_words : nullptr;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const unsigned long long m64 = __ballot(u[k] - tau > 0.f);
    uint32_t w0 = (uint32_t)m64, w1 = (uint32_t)(m64 >> 32);
    if (lane == 0 && w0) atomicOr(&s_union[2 * k], w0);
    if (lane == 0 && w1) atomicOr(&s_union[2 * k + 1], w1);
    if (dact && (ct >> 5) == 2 * k) w0 |= 1u << (ct & 31);
    if (dact && (ct >> 5) == 2 * k + 1) w1 |= 1u << (ct & 31);
    if (bdst && lane == 0 && 2 * k < a.bits_words) bdst[2 * k] = w0;
    if (bdst && lane == 0 && 2 * k + 1 < a.bits_words) bdst[2 * k + 1] = w1;
  }
  if (lane == 0 && dact) atomicOr(&s_union[ct >> 5], 1u << (ct & 31));
  if (bdst && lane == 0)
    for (int wd = 2 * KPL; wd < a.bits_words; ++wd)
      bdst[wd] = (dact && (ct >> 5) == wd) ? (1u << (ct & 31)) : 0u;

  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int wd = 0; wd < NWD; ++wd) {
      s_pre[wd] = acc;
      acc += __popc(s_union[wd]);
    }
    s_pre[NWD] = acc;
    a.counts[grp_id] = acc;
  }
  __syncthreads();
  const size_t gbase = (size_t)grp_id * a.n_slots;
  for (int wd = threadIdx.x; wd < NWD; wd += blockDim.x) {
    uint32_t bits = s_union[wd];
    int pos = s_pre[wd];
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      a.lists[gbase + pos++] = wd * 32 + bpos;
      bits &= bits - 1u;
    }
  }
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int c = k * 64 + lane;
    const uint32_t word = s_union[c >> 5];
    if (c != ct && ((word >> (c & 31)) & 1u)) {
      const int pos = s_pre[c >> 5] + __popc(word & ((1u << (c & 31)) - 1u));
      const float tt = u[k] - tau;
      a.bias[(gbase + pos) * G + w] = tt > 0.f ? log2_prior<KIND>(tt, a.beta) : -INFINITY;
    }
  }
  if (lane == 0) {
    const uint32_t word = s_union[ct >> 5];
    if ((word >> (ct & 31)) & 1u) {
      const int pos = s_pre[ct >> 5] + __popc(word & ((1u << (ct & 31)) - 1u));
      a.bias[(gbase + pos) * G + w] = lwd;
    }
  }
}

// ============================================================================
// launchers
// ============================================================================
template <int KIND>
static hipError_t route_prefill_kind(const RouteArgs& a, hipStream_t stream) {
  dim3 grid(a.n_tiles, a.Hq, a.B);
  const int nb = (a.n_slots + 15) / 16;
#define DASH_RP(NBV)                                                                   \
  if (nb <= NBV) {                                                                     \
    hipLaunchKernelGGL((k_route_prefill<NBV, KIND>), grid, dim3(512), 0, stream, a); \
    return hipGetLastError();                                                          \
  }
  DASH_RP(2) DASH_RP(4) DASH_RP(8) DASH_RP(16) DASH_RP(32)
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
  dim3 g1((ncomp_max + 63) / 64 > 0 ? (ncomp_max + 63) / 64 : 1, a.B * a.Hkv);
  if (ncomp_max > 0) hipLaunchKernelGGL((k_route_decode_scores<G>), g1, dim3(256), 0, stream, a);
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
