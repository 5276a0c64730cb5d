// sparse_prefill.hip -- stage 3 of the DashAttention hierarchy ("How it works"
// 3 on the DashAttention README page, "prior-induced sparse softmax"):
//   O_i = sum_j softmax_j(<q_i, k_j>/sqrt(d) + log w_{i,c(j)}) v_j
// over the tokens of the chunks routed to row i, with w the routing prior.
// Visiting the routed chunks in any order gives the same result (the
// order-invariance of the online softmax, "Axiom ledger" Property 2 on the CoSA
// review page), which is what lets the work be cut by chunk instead of by row.
//
// Rows close together rarely route the same chunks, so a row block's chunk
// union is mostly empty pairs. The main path is chunk-major instead:
//   * k_cm_plan / k_cm_scatter: the (row, routed past chunk) pairs the routing
//     recorded per tile are sorted by (b, kv head, chunk) and cut into work
//     items of up to kCmBlocks blocks of 32 pairs;
//   * k_prefill_cm: a persistent grid walks the items; per item the chunk's K
//     (row-major) and V (transposed) are staged once in LDS and each wavefront
//     attends whole blocks of 32 pairs with v_mfma_f32_32x32x16_bf16 (S^T = K
//     Q^T, a lane owns a pair; O^T = V^T P^T), gathering the pairs' query rows,
//     and leaves one partial result per pair in the pool (log2 of its weight
//     sum, float32; its normalised output, fp16);
//   * k_prefill_merge: per (b, kv head, chunk, query head), the 64 rows' own
//     (diagonal) chunk is attended as one causal 64 x 64 tile
//     (v_mfma_f32_16x16x32_bf16) and merged with each row's partials (an exact
//     online-softmax merge in a fixed order), so the always-attended own chunk
//     never goes through the pool.
// Tiles of 128 rows whose pairs did not fit the pool are attended by the
// row-major fallback k_sparse_prefill: one workgroup (four wavefronts of 32
// rows) per (b, query head, tile) walks the tile's chunk union with K/V chunks
// in a double-buffered LDS ring, recomputing each row's prior weight for a
// listed chunk from its tau and routed-chunk bits (a dot product with the
// chunk's split summary). Work is spread so that the g query heads sharing a
// KV head land on the same XCD and share its L2.
#include <algorithm>

#include "kernels.hpp"
#include "tau_solve.hpp"

namespace dash {

namespace {
constexpr int KPAD = 8;  // bf16 elements of padding per K row in LDS
constexpr int VPAD = 4;  // bf16 elements of padding per V^T row in LDS

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);  // low halves: x | y << 16
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);  // high halves: x | y << 16
}
}  // namespace

template <int D, int KIND>
__global__ __launch_bounds__(256, 2) void k_sparse_prefill(PrefillAttnArgs a) {
  constexpr int NS = D / 16;  // k-steps of S^T = K Q^T
  constexpr int NDB = D / 32; // 32-dim blocks of O^T
  constexpr int KROW = D + KPAD;
  constexpr int VROW = kChunk + VPAD;
  static_assert(D == 128, "staging is laid out for head_dim 128");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kChunk * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VROW];
  __shared__ __attribute__((aligned(16))) uint16_t sU[2][2 * D];  // the chunk's summary: high parts, low parts

  if (*a.n_rm == 0 || *a.bad != 0) return;  // every tile went chunk-major / inconsistent workspace
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int tid = threadIdx.x;

  // ---- work units (tile, b, kv head) x g query heads, walked by a persistent
  // grid whose size is a multiple of 8; the g heads of a unit get work ids that
  // are equal modulo 8 (same XCD)
  const int g = a.g;
  const int n_units = a.n_tiles * a.B * a.Hkv;
  const int n_work = ((n_units + 7) / 8) * 8 * g;
  for (int idx = blockIdx.x; idx < n_work; idx += gridDim.x) {
    const int grp8 = idx / (8 * g);
    const int rem = idx % (8 * g);
    const int gh = rem / 8;
    const int unit = grp8 * 8 + rem % 8;
    if (unit >= n_units) continue;
    const int tile = unit / (a.B * a.Hkv);
    const int bhk = unit % (a.B * a.Hkv);
    const int b = bhk / a.Hkv;
    const int hk = bhk % a.Hkv;
    const int h = hk * g + gh;
    const size_t bh = (size_t)b * a.Hq + h;
    const int N = a.N;
    const bool causal = a.causal != 0;

    const int count = a.counts[bh * a.n_tiles + tile];
    if (count == 0) continue;  // every chunk of the tile went chunk-major
    const long long toff = bh * a.per_head + prefill_tile_offset(tile, a.n_slots, causal);
    const int* list = a.lists + toff;

    const int row0 = tile * kTileRows + w * 32;
    const int cw = row0 / kChunk;
    const int qi = row0 + (lane & 31);
    const int hi32 = lane >> 5;
    // the row's tau, routed past chunks and own-chunk weight
    const size_t rix = bh * N + min(qi, N - 1);
    const float tau_r = a.rm_tau[rix];
    const uint32_t* rbits = a.rm_bits + rix * a.rm_words;
    const float own_lw = causal ? a.own_lw[rix] : -INFINITY;
    const uint16_t* Ub = a.s_hi + ((size_t)b * a.Hkv + hk) * (size_t)a.n_slots * D;
    const size_t lo_off = (size_t)(a.s_lo - a.s_hi);

    // Q^T as the B operand: column qi, dims 16 s + 8 hi32 .. +7
    bf16x8 qb[NS];
    {
      // dims past the head_dim are zero
      const uint16_t* qp = a.Q + (bh * N + min(qi, N - 1)) * (size_t)a.d;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int col = 16 * s + 8 * hi32;
        qb[s] = as_bf16x8(qi < N && col < a.d ? ldg16(qp + col) : u32x4{0, 0, 0, 0});
      }
    }

    // staging roles: K rows t/16 + 16 r at dims (t%16)*8; V keys 4 (t%16) + r at
    // dims 8 (t/16). A thread whose dims lie past the head_dim stages zeros.
    const int k_row = tid >> 4, k_col = (tid & 15) * 8;
    const int v_kg = tid & 15, v_dg = tid >> 4;
    const int n_keys = N;
    const int dd = a.d;
    const size_t kvrow0 = ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax;
    const uint16_t* Kt = a.K + kvrow0 * dd + k_col;
    const uint16_t* Vt = a.V + kvrow0 * dd + 8 * v_dg;
    const bool k_in = k_col < dd, v_in = 8 * v_dg < dd;

    u32x4 kr[4], vr[4], ur;
    // Keys past the sequence end are read from its last row instead (a valid
    // address); their scores are masked, so their weights are exactly zero.
    // Threads 0..31 also stage the chunk's split summary (16 bytes each).
    auto load_chunk = [&](int c) {
      const int base = c * kChunk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(base + k_row + 16 * r, n_keys - 1);
        kr[r] = k_in ? ldg16(Kt + (uint32_t)(key * dd)) : u32x4{0, 0, 0, 0};
        const int vkey = min(base + 4 * v_kg + r, n_keys - 1);
        vr[r] = v_in ? ldg16(Vt + (uint32_t)(vkey * dd)) : u32x4{0, 0, 0, 0};
      }
      if (tid < 2 * D / 8) ur = ldg16(Ub + (tid >= D / 8 ? lo_off : 0) + (size_t)c * D + 8 * (tid % (D / 8)));
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4*>(&sK[buf][(k_row + 16 * r) * KROW + k_col]) = kr[r];
      if (tid < 2 * D / 8) *reinterpret_cast<u32x4*>(&sU[buf][8 * tid]) = ur;
      uint16_t* vt = &sV[buf][(8 * v_dg) * VROW + 4 * v_kg];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims 8 v_dg + 2e (low halves) and + 2e + 1 (high halves), keys 4 v_kg .. +3
        u32x2 lo2 = {perm_lo(vr[0][e], vr[1][e]), perm_lo(vr[2][e], vr[3][e])};
        u32x2 hi2 = {perm_hi(vr[0][e], vr[1][e]), perm_hi(vr[2][e], vr[3][e])};
        *reinterpret_cast<u32x2*>(vt + (2 * e) * VROW) = lo2;
        *reinterpret_cast<u32x2*>(vt + (2 * e + 1) * VROW) = hi2;
      }
    };

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = kNegBig, l_run = 0.f;
    const float sc = a.scale_log2;

    // the row's routed bit for chunk c, from its bitmask word
    auto routed = [&](int c, uint32_t word) { return qi < N && ((word >> (c & 31)) & 1u) != 0u; };
    uint32_t word_next = 0u;
    if (count > 0) {
      load_chunk(list[0]);
      word_next = rbits[list[0] >> 5];
      store_chunk(0);
    }
    __syncthreads();

    for (int it = 0; it < count; ++it) {
      const int buf = it & 1;
      const int c = list[it];
      const uint32_t word = word_next;
      const bool more = it + 1 < count;
      if (more) word_next = rbits[list[it + 1] >> 5];
      // ---- the row's log2 weight for chunk c: the own chunk's from the
      // routing; a routed past chunk's recomputed, log2 of (u - tau)^beta with u
      // = <q, summary> in u units (high parts + low parts, as the routing
      // scored it); -inf otherwise
      float bias = -INFINITY;
      if (causal && c == cw) {
        bias = qi < N ? own_lw : -INFINITY;
      } else if (!(causal && c > cw)) {
        const bool rt = routed(c, word);
        if (wave_any(rt)) {
          const uint16_t* up = &sU[buf][8 * hi32];
          float dot = 0.f;
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const u32x4 q4 = __builtin_bit_cast(u32x4, qb[s]);
            const u32x4 h4 = *reinterpret_cast<const u32x4*>(up + 16 * s);
            const u32x4 l4 = *reinterpret_cast<const u32x4*>(up + D + 16 * s);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dot = fmaf(bf16lo(q4[e]), bf16lo(h4[e]), dot);
              dot = fmaf(bf16hi(q4[e]), bf16hi(h4[e]), dot);
              dot = fmaf(bf16lo(q4[e]), bf16lo(l4[e]), dot);
              dot = fmaf(bf16hi(q4[e]), bf16hi(l4[e]), dot);
            }
          }
          const float t = sum_xor32(dot) - tau_r;
          bias = rt && t > 0.f ? log2_prior<KIND>(t, a.beta) : -INFINITY;
        }
      }
      // the next chunk's loads go out once the weight's registers are free
      if (more) load_chunk(list[it + 1]);
      const bool skip = (causal && c > cw) || wave_all(bias == -INFINITY);
      if (!skip) {
        // ---- S^T = K Q^T
        f32x16 s0, s1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = 0.f;
          s1[r] = 0.f;
        }
        const uint16_t* ka = &sK[buf][(lane & 31) * KROW + 8 * hi32];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ka + 16 * s);
          bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ka + 32 * KROW + 16 * s);
          s0 = mfma32x32x16(a0, qb[s], s0);
          s1 = mfma32x32x16(a1, qb[s], s1);
        }
        // ---- masks (own chunk: causal; non-causal last chunk: sequence end), only
        //      in these uniform branches. Lane owns query qi; block kb holds keys
        //      c*64 + 32 kb + 8 (r/4) + 4 hi32 + r%4.
        if (causal && c == cw) {
          const int lim = qi - c * kChunk;  // keys 0 .. lim of this chunk are visible
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r >> 2) + 4 * hi32 + (r & 3);
            s0[r] = kk <= lim ? s0[r] : -INFINITY;
            s1[r] = kk + 32 <= lim ? s1[r] : -INFINITY;
          }
        } else if (!causal && (c + 1) * kChunk > n_keys) {
          const int lim = n_keys - 1 - c * kChunk;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r >> 2) + 4 * hi32 + (r & 3);
            s0[r] = kk <= lim ? s0[r] : -INFINITY;
            s1[r] = kk + 32 <= lim ? s1[r] : -INFINITY;
          }
        }
        // ---- online softmax in the exp2 domain. The row's bias is constant over
        //      the chunk and the scale is positive, so the max is taken on raw
        //      scores and each weight costs one fma and one v_exp.
        float smax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) smax = fmaxf(smax, fmaxf(s0[r], s1[r]));
        smax = max_xor32(smax);
        const float m_new = fmaxf(m_run, fmaf(smax, sc, bias));
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        const float off = bias - m_new;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = fast_exp2(fmaf(s0[r], sc, off));
          s1[r] = fast_exp2(fmaf(s1[r], sc, off));
          ls += s0[r] + s1[r];
        }
        l_run = fmaf(l_run, alpha, ls);
        if (wave_any(alpha != 1.f)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        // ---- P^T as B operands: k-step (kb, hh) takes registers 8 hh .. 8 hh + 7
        bf16x8 pb[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 p0, p1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p0[e] = pack_bf16x2(s0[8 * hh + 2 * e], s0[8 * hh + 2 * e + 1]);
            p1[e] = pack_bf16x2(s1[8 * hh + 2 * e], s1[8 * hh + 2 * e + 1]);
          }
          pb[hh] = as_bf16x8(p0);
          pb[2 + hh] = as_bf16x8(p1);
        }
        // ---- O^T += V^T P^T; V^T row = dim, keys kb*32 + 16 hh + 4 hi32 + {0..3, 8..11}
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* vrow = &sV[buf][(32 * db + (lane & 31)) * VROW + 4 * hi32];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int k0 = (ks >> 1) * 32 + (ks & 1) * 16;
            u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + k0);
            u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + k0 + 8);
            u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
            o[db] = mfma32x32x16(as_bf16x8(va), pb[ks], o[db]);
          }
        }
      }
      if (more) store_chunk(buf ^ 1);
      __syncthreads();
    }

    // ---- normalise and store O (lane: query qi, dims 32 db + 8 (r/4) + 4 hi32 + r%4)
    const float l_tot = sum_xor32(l_run);
    if (qi < N) {
      const float inv = 1.f / l_tot;
      uint16_t* op = a.O + (bh * N + qi) * (size_t)a.d + 4 * hi32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 v = {pack_bf16x2(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv),
                     pack_bf16x2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv)};
          if (32 * db + 8 * q4 + 4 * hi32 < a.d) *reinterpret_cast<u32x2*>(op + 32 * db + 8 * q4) = v;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk-major part. Every (query head, row) pair that routed a past chunk c
// (in a tile that got pool slots) is attended against c alone, 32 pairs per
// MFMA block, and leaves a partial result in its pool slot:
//   1. k_cm_plan (one workgroup): prefix sums of the per-chunk pair counts that
//      the routing left give every (b, kv head, chunk) its start among all
//      pairs, and its blocks are cut into work items of up to kCmBlocks blocks;
//   2. k_cm_scatter: every chunk-major list entry copies its pairs into the
//      chunk-sorted records (row and head in group, pool slot, log2 weight);
//   3. k_prefill_cm: a persistent grid walks the work items in (b, kv head,
//      chunk) order; per item the K and V of its chunk are staged once in LDS
//      and each wavefront attends whole blocks of 32 pairs, gathering their
//      query rows from Q.
// ---------------------------------------------------------------------------
namespace {
constexpr int kCmWgPerCu = 3;  // resident chunk-major workgroups per CU
}  // namespace

// Workgroup j plans the (b, kv head, chunk) entries [256 j, 256 j + 256): the
// pairs and work items of every entry before its range are summed first (each
// workgroup reads the counts ahead of it, 16 KB at 32K), then its own entries
// are scanned. Also resets the chunk-major kernel's queue head.
__global__ __launch_bounds__(256) void k_cm_plan(PrefillAttnArgs a) {
  __shared__ int s_tmp[4][4];
  if (a.pool[kPools] != (unsigned long long)a.pool_cap) {
    // the routing laid the pool out for another workspace size: no chunk-major
    // work; the merge kernel writes NaN rows
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *a.nitems = 0;
      *a.qhead = 0;
      *a.bad = 1;
    }
    return;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.bad = 0;
  auto n_items = [](int P) { return ((P + 31) / 32 + kCmBlocks - 1) / kCmBlocks; };
  const int base = blockIdx.x * 256;
  int pp = 0, pi = 0;
  for (int j = threadIdx.x; j < base; j += 256) {
    const int P = a.cmp[j];
    pp += P;
    pi += n_items(P);
  }
  int unused;
  const int carry_p = block_excl_scan<4>(pp, s_tmp[0], unused);
  const int carry_i = block_excl_scan<4>(pi, s_tmp[1], unused);
  const int idx = base + threadIdx.x;
  const int P = idx < a.n_bhc ? a.cmp[idx] : 0;
  const int ni = n_items(P);
  int ep, ei;
  block_excl_scan<4>(P, s_tmp[2], ep);
  const int ti = block_excl_scan<4>(ni, s_tmp[3], ei);
  if (idx < a.n_bhc) {
    a.cs[idx] = carry_p + ep;
    for (int j = 0; j < ni; ++j) {
      const long long it = (long long)carry_i + ei + j;
      if (it < a.max_items) a.items[it] = make_int2(idx, j * kCmBlocks);
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) *a.nitems = carry_i + ti;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.qhead = 0;
}

// One workgroup per (tile, query head, b): copies the tile's pair records,
// grouped by chunk in its pool range, to their places among the chunk-sorted
// records (each group after the pairs that other tiles reserved before it in
// the same chunk). Thread q copies record q; its group is found by binary
// search over the groups' first records.
__global__ __launch_bounds__(256) void k_cm_scatter(PrefillAttnArgs a) {
  __shared__ int s_first[kPrefillMaxSlots];
  __shared__ long long s_dst[kPrefillMaxSlots];  // destination of record q: s_dst[group] + q
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const size_t bh = (size_t)b * a.Hq + h;
  if (*a.bad != 0) return;
  const int cnt = min(a.ccounts[bh * a.n_tiles + tile], kPrefillMaxSlots);
  if (cnt == 0) return;
  const long long toff = bh * a.per_head + prefill_tile_offset(tile, a.n_slots, a.causal != 0);
  const int* cs = a.cs + ((size_t)b * a.Hkv + h / a.g) * a.n_slots;
  const long long tb = a.tbase[bh * a.n_tiles + tile];
  for (int e = threadIdx.x; e < cnt; e += blockDim.x) {
    const int2 fe = a.ceo[toff + e];
    s_first[e] = fe.x;
    s_dst[e] = (long long)cs[a.clists[toff + e]] + a.cbase[toff + e] - fe.x;
  }
  __syncthreads();
  const int2 last = a.ceo[toff + cnt - 1];
  const int total = last.x + last.y;
  for (int q = threadIdx.x; q < total; q += blockDim.x) {
    int lo = 0, hi = cnt - 1;  // the last group starting at or before q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_first[mid] <= q) lo = mid;
      else hi = mid - 1;
    }
    const long long dst = s_dst[lo] + q;
    if (dst >= 0 && dst < a.pool_cap && tb + q < a.pool_cap) a.recs[dst] = a.trec[tb + q];
  }
}

// DC: the caller's head_dim (the row width of Q, K, V), a template argument so
// that the 128-dim instance has no per-load head_dim test
template <int D, int DC>
__global__ __launch_bounds__(256, kCmWgPerCu) void k_prefill_cm(PrefillAttnArgs a) {
  constexpr int NS = D / 16;
  constexpr int KROW = D + KPAD;
  constexpr int VROW = kChunk + VPAD;
  constexpr int NBW = kCmBlocks / 4;  // blocks of an item per wavefront
  constexpr int OROW = 64 + 8;        // output staging: 64 dims of a row, padded
  static_assert(D == 128, "staging is laid out for head_dim 128");
  __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VROW];
  __shared__ __attribute__((aligned(16))) uint16_t sO[4][32 * OROW];  // per wavefront

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int tid = threadIdx.x;
  const int g = a.g;
  const int N = a.N;
  const float sc = a.scale_log2;
  const int hi32 = lane >> 5;
  const bool causal = a.causal != 0;
  const int nitems = (int)min((long long)*a.nitems, a.max_items);
  __shared__ int s_item;

  for (;;) {
    // the next item from the queue; the barrier also orders the previous
    // item's LDS reads before this item's staging
    __syncthreads();
    if (tid == 0) s_item = atomicAdd(a.qhead, 1);
    __syncthreads();
    const int item = s_item;
    if (item >= nitems) break;
    const int2 it = a.items[item];
    const int bhc = it.x;
    const int c = bhc % a.n_slots;
    const int bhk = bhc / a.n_slots;
    const int b = bhk / a.Hkv;
    const int hk = bhk % a.Hkv;
    const int P = a.cmp[bhc];
    const size_t start = (size_t)a.cs[bhc];
    const int k1 = min(it.y + kCmBlocks, (P + 31) / 32);
    // this wavefront's blocks: it.y + w + 4 i, i < nb
    const int nb = max(0, (k1 - (it.y + w) + 3) / 4);

    // ---- the pair records of this wavefront's blocks; lane j % 32 takes pair
    // 32 k + j % 32 of block k (lanes past the block's end repeat its last pair)
    int4 rec[NBW];
    auto cnt_of = [&](int i) { return min(32, P - 32 * (it.y + w + 4 * i)); };  // pairs of block i
#pragma unroll
    for (int i = 0; i < NBW; ++i)
      if (i < nb) rec[i] = a.recs[start + 32 * (it.y + w + 4 * i) + min(lane & 31, cnt_of(i) - 1)];
    // a record names a row of the sequence (row * g + head in group) and a pool slot
    auto valid_of = [&](const int4& r, int n) {
      return (lane & 31) < n && r.x >= 0 && r.x < N * g && (long long)(uint32_t)r.y < a.pool_cap;
    };
    auto load_q = [&](const int4& r, int n, bf16x8 (&qb)[NS]) {
      const int qh = valid_of(r, n) ? r.x : 0;
      const int row = qh / g;
      const size_t bh = (size_t)b * a.Hq + hk * g + (qh - row * g);
#pragma unroll
      for (int s = 0; s < NS; ++s) qb[s] = as_bf16x8(ldg16_dc<DC>(a.Q, bh * N + row, 16 * s + 8 * hi32));
    };

    // ---- stage K (row-major) and V (transposed) of chunk c; keys past the
    // sequence end read its last row (masked below). The first block's query
    // rows are fetched meanwhile.
    bf16x8 qbuf[2][NS];
    {
      const size_t kvrow0 = ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax;
      const int k_row = tid >> 4, k_col = (tid & 15) * 8;
      const int v_kg = tid & 15, v_dg = tid >> 4;
      u32x4 kr[4], vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kr[r] = ldg16_dc<DC>(a.K, kvrow0 + min(c * kChunk + k_row + 16 * r, N - 1), k_col);
        vr[r] = ldg16_dc<DC>(a.V, kvrow0 + min(c * kChunk + 4 * v_kg + r, N - 1), 8 * v_dg);
      }
      if (nb > 0) load_q(rec[0], cnt_of(0), qbuf[0]);
#pragma unroll
      for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4*>(&sK[(k_row + 16 * r) * KROW + k_col]) = kr[r];
      uint16_t* vt = &sV[(8 * v_dg) * VROW + 4 * v_kg];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x2 lo2 = {perm_lo(vr[0][e], vr[1][e]), perm_lo(vr[2][e], vr[3][e])};
        u32x2 hi2 = {perm_hi(vr[0][e], vr[1][e]), perm_hi(vr[2][e], vr[3][e])};
        *reinterpret_cast<u32x2*>(vt + (2 * e) * VROW) = lo2;
        *reinterpret_cast<u32x2*>(vt + (2 * e + 1) * VROW) = hi2;
      }
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      if (i < nb) {
        // the next block's query rows are in flight while this one is computed
        if (i + 1 < NBW && i + 1 < nb) load_q(rec[i + 1], cnt_of(i + 1), qbuf[(i + 1) & 1]);
        const bf16x8 (&qb)[NS] = qbuf[i & 1];
        const int cnt_i = cnt_of(i);
        const bool valid = valid_of(rec[i], cnt_i);
        const int qh = valid ? rec[i].x : 0;
        const int row = qh / g;
        const float bias = valid ? __int_as_float(rec[i].z) : -INFINITY;

        // ---- S^T = K Q^T (lane: query row, registers: keys)
        f32x16 s0, s1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = 0.f;
          s1[r] = 0.f;
        }
        const uint16_t* ka = &sK[(lane & 31) * KROW + 8 * hi32];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          s0 = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ka + 16 * s), qb[s], s0);
          s1 = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ka + 32 * KROW + 16 * s), qb[s], s1);
          if (s % 2 == 1) __builtin_amdgcn_sched_barrier(0);  // bounds the operands in flight
        }
        // keys of the chunk visible to the row: up to the row itself (causal: the
        // own chunk is the only one that reaches past it) and the sequence end
        const int lim = min(causal ? row - c * kChunk : kChunk - 1, N - 1 - c * kChunk);
        if (wave_any(lim < kChunk - 1)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r >> 2) + 4 * hi32 + (r & 3);
            s0[r] = kk <= lim ? s0[r] : -INFINITY;
            s1[r] = kk + 32 <= lim ? s1[r] : -INFINITY;
          }
        }
        // ---- softmax over the chunk in the exp2 domain, with the row's bias
        float smax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) smax = fmaxf(smax, fmaxf(s0[r], s1[r]));
        smax = max_xor32(smax);
        const bool live = valid && smax > -INFINITY;
        const float m = live ? fmaf(smax, sc, bias) : 0.f;
        const float off = live ? bias - m : -INFINITY;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = fast_exp2(fmaf(s0[r], sc, off));
          s1[r] = fast_exp2(fmaf(s1[r], sc, off));
          ls += s0[r] + s1[r];
        }
        const float l = sum_xor32(ls);
        bf16x8 pb[4];
#pragma unroll
        for (int hh2 = 0; hh2 < 2; ++hh2) {
          u32x4 p0, p1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            p0[q] = pack_bf16x2(s0[8 * hh2 + 2 * q], s0[8 * hh2 + 2 * q + 1]);
            p1[q] = pack_bf16x2(s1[8 * hh2 + 2 * q], s1[8 * hh2 + 2 * q + 1]);
          }
          pb[hh2] = as_bf16x8(p0);
          pb[2 + hh2] = as_bf16x8(p1);
        }
        // ---- partial result of the pair, stored in its pool slot: log2 of its
        // sum of exp2 weights, and O^T = V^T P^T over that sum in natural dim
        // order. Each 64-dim half passes through this wavefront's LDS rows, so
        // that every store instruction writes whole 128-byte lines.
        const uint32_t slot = valid ? (uint32_t)rec[i].y : 0u;
        if (valid && hi32 == 0) __builtin_nontemporal_store(l > 0.f ? m + fast_log2(l) : -INFINITY, a.plse + slot);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* so = sO[w];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int d2 = 0; d2 < 2; ++d2) {
            f32x16 o;
#pragma unroll
            for (int r = 0; r < 16; ++r) o[r] = 0.f;
            const uint16_t* vrow = &sV[(32 * (2 * half + d2) + (lane & 31)) * VROW + 4 * hi32];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const int k0 = (ks >> 1) * 32 + (ks & 1) * 16;
              u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + k0);
              u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + k0 + 8);
              o = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[ks], o);
            }
            __builtin_amdgcn_sched_barrier(0);
            // row lane % 32, dims 32 d2 + 8 q4 + 4 hi32 + {0..3} of this half
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              *reinterpret_cast<u32x2*>(so + (lane & 31) * OROW + 32 * d2 + 8 * q4 + 4 * hi32) =
                  u32x2{pack_f16x2(o[4 * q4] * inv, o[4 * q4 + 1] * inv), pack_f16x2(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv)};
          }
          wave_lds_fence();
          // 32 rows x 128 bytes: eight lanes per row, eight rows per pass; the
          // slot of row rr is held by lane rr
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = lane + kWave * u;
            const int rr = t >> 3, c16 = t & 7;
            const u32x4 v = *reinterpret_cast<const u32x4*>(so + rr * OROW + 8 * c16);
            const int vr = __shfl((int)valid, rr);
            const size_t sr = (uint32_t)__shfl((int)slot, rr);
            if (vr) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.po + sr * D + 64 * half + 8 * c16));
          }
          wave_lds_fence();
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Own chunk and merge. One workgroup per (b, query head, 64-row chunk c) of a
// tile that got pool slots (row-major tiles are left to k_sparse_prefill):
//   A (causal). The rows' own chunk c as one causal 64 x 64 tile: K and V^T
//     of the chunk staged in LDS, four wavefronts of 16 rows each,
//     S^T = K Q^T and O^T = V^T P^T by v_mfma_f32_16x16x32_bf16, the row's
//     own-chunk log2 weight (own_lw) as bias; the normalised result and the
//     log2 of its weight sum go to LDS.
//   B. Every row combines its own-chunk result with its partials (routed past
//     chunks, consecutive slots in chunk order), eight lanes per row: the
//     largest log2 sum first, then each partial's fp16 output added with its
//     normalised weight (fp32 sums); lane p owns dims 8p .. 8p+7 and
//     64+8p .. 64+8p+7, so every load instruction of the eight lanes reads 128
//     contiguous bytes; four partials are in flight together.
// The order of the adds is fixed (own chunk, then the slots in order), so the
// result is deterministic. Partials are written and read once: their stores
// and loads are non-temporal, so they do not displace the query rows and
// chunks that the caches can still serve. The g heads of one (b, kv head, chunk) get work ids
// that are equal modulo 8 (one XCD), so their K/V reads share that L2.
// ---------------------------------------------------------------------------
// DC: the caller's head_dim (row width of Q, K, V, O), a template argument
template <bool CAUSAL, int DC>
__global__ __launch_bounds__(256) void k_prefill_merge(PrefillAttnArgs a) {
  constexpr int D = 128;
  constexpr int NP = 4;           // partials loaded together
  constexpr int KROW = D + KPAD;  // staged K row (bf16)
  constexpr int VROW = kChunk + VPAD;
  constexpr int OROW = D + 4;     // own-chunk output row (fp32)
  constexpr int kStageBytes = (kChunk * KROW + D * VROW) * 2;
  constexpr int kOutBytes = kChunk * OROW * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[kStageBytes > kOutBytes ? kStageBytes : kOutBytes];
  __shared__ float s_lse[kChunk];

  const int g = a.g;
  const int N = a.N;
  const int nC = (N + kChunk - 1) / kChunk;
  const int n_units = a.B * a.Hkv * nC;
  const int idx = blockIdx.x;
  const int grp8 = idx / (8 * g), rem = idx % (8 * g);
  const int gh = rem / 8;
  const int unit = grp8 * 8 + rem % 8;
  if (unit >= n_units) return;
  const int c = unit % nC;
  const int bhk = unit / nC;
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const size_t bh = (size_t)b * a.Hq + hk * g + gh;
  const int tile = c * kChunk / kTileRows;
  const int tid = threadIdx.x;
  if (*a.bad != 0) {
    // inconsistent workspace: every row of the unit reads NaN
    for (int x = tid; x < kChunk * DC / 2; x += blockDim.x) {
      const int r = c * kChunk + x / (DC / 2);
      if (r < N) reinterpret_cast<uint32_t*>(a.O + (bh * N + r) * (size_t)DC)[x % (DC / 2)] = 0x7fc07fc0u;
    }
    return;
  }
  if (a.counts[bh * a.n_tiles + tile] > 0) return;  // a row-major tile
  const int lane = lane_id();
  const int w = tid / kWave;
  const int row0 = c * kChunk;
  float* const sO = reinterpret_cast<float*>(s_raw);
  // the merge's rows (32 per pass, eight lanes each): partial counts and first
  // slots requested now, so that they arrive while the own chunk is attended
  int n_ps[2];
  uint32_t s0_ps[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int qi = row0 + pass * 32 + tid / 8;
    const size_t ri = bh * (size_t)N + min(qi, N - 1);
    n_ps[pass] = qi < N ? (int)a.cmcnt[ri] : 0;
    s0_ps[pass] = a.rslot[ri];
  }

  if constexpr (CAUSAL) {
    uint16_t* const sK = reinterpret_cast<uint16_t*>(s_raw);
    uint16_t* const sV = sK + kChunk * KROW;
    const size_t kvrow0 = ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax;
    // wavefront w: rows row0 + 16 w + lane % 16; lanes l, l^16, l^32, l^48 share a row
    const int rloc = 16 * w + (lane & 15);
    const int qi = row0 + rloc;
    const int q4 = lane >> 4;
    const float lw = qi < N ? a.own_lw[bh * (size_t)N + qi] : -INFINITY;
    bf16x8 qb[D / 32];  // Q^T as the B operand: column qi, dims 32 s + 8 q4 .. +7
    {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) qb[s] = as_bf16x8(ldg16_dc<DC>(a.Q, bh * N + min(qi, N - 1), 32 * s + 8 * q4));
    }
    {
      // K rows (row-major) and V (transposed) of chunk c; keys past the sequence
      // end read its last row (they lie in every row's future: masked)
      const int k_row = tid >> 4, k_col = (tid & 15) * 8;
      const int v_kg = tid & 15, v_dg = tid >> 4;
      u32x4 kr[4], vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kr[r] = ldg16_dc<DC>(a.K, kvrow0 + min(row0 + k_row + 16 * r, N - 1), k_col);
        vr[r] = ldg16_dc<DC>(a.V, kvrow0 + min(row0 + 4 * v_kg + r, N - 1), 8 * v_dg);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4*>(&sK[(k_row + 16 * r) * KROW + k_col]) = kr[r];
      uint16_t* vt = &sV[(8 * v_dg) * VROW + 4 * v_kg];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x2 lo2 = {perm_lo(vr[0][e], vr[1][e]), perm_lo(vr[2][e], vr[3][e])};
        u32x2 hi2 = {perm_hi(vr[0][e], vr[1][e]), perm_hi(vr[2][e], vr[3][e])};
        *reinterpret_cast<u32x2*>(vt + (2 * e) * VROW) = lo2;
        *reinterpret_cast<u32x2*>(vt + (2 * e + 1) * VROW) = hi2;
      }
    }
    __syncthreads();
    // ---- S^T = K Q^T: key block kb holds keys 16 kb + 4 q4 + r of row qi
    f32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        sacc[kb] = mfma16x16x32(*reinterpret_cast<const bf16x8*>(&sK[(16 * kb + (lane & 15)) * KROW + 32 * s + 8 * q4]),
                                qb[s], sacc[kb]);
    }
    // ---- causal mask inside the chunk, softmax in the exp2 domain with the bias
    float smax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = 16 * kb + 4 * q4 + r <= rloc ? sacc[kb][r] : -INFINITY;
        sacc[kb][r] = v;
        smax = fmaxf(smax, v);
      }
    smax = max_xor32(max_xor16(smax));
    const bool live = lw > -INFINITY;
    const float sc = a.scale_log2;
    const float m = live ? fmaf(smax, sc, lw) : 0.f;
    const float off = live ? lw - m : -INFINITY;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], sc, off));
        ls += sacc[kb][r];
      }
    const float l = sum_xor32(sum_xor16(ls));
    // ---- O^T = V^T P^T. The k slots of step j are relabelled on both operands:
    // slot e < 4 is key 32 j + 4 q4 + e, slot e >= 4 is key 32 j + 16 + 4 q4 + e - 4,
    // which is how the S^T blocks 2j and 2j+1 already lie in this lane.
    bf16x8 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pb[j] = as_bf16x8(u32x4{pack_bf16x2(sacc[2 * j][0], sacc[2 * j][1]), pack_bf16x2(sacc[2 * j][2], sacc[2 * j][3]),
                              pack_bf16x2(sacc[2 * j + 1][0], sacc[2 * j + 1][1]),
                              pack_bf16x2(sacc[2 * j + 1][2], sacc[2 * j + 1][3])});
    f32x4 oacc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint16_t* vrow = &sV[(16 * db + (lane & 15)) * VROW + 32 * j + 4 * q4];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
        oacc[db] = mfma16x16x32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[j], oacc[db]);
      }
    }
    __syncthreads();  // every wavefront is done with the staged K and V
    // row rloc, dims 16 db + 4 q4 + r, normalised
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(&sO[rloc * OROW + 16 * db + 4 * q4]) =
          f32x4{oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
    if (q4 == 0) s_lse[rloc] = l > 0.f ? m + fast_log2(l) : -INFINITY;
    __syncthreads();
  }

  // ---- merge, 32 rows per pass
  auto max8 = [](float x) {
    x = fmaxf(x, dpp_f<kDppXor1>(x));
    x = fmaxf(x, dpp_f<kDppXor2>(x));
    return fmaxf(x, dpp_f<kDppHalfMirror>(x));
  };
  auto sum8 = [](float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    return x + dpp_f<kDppHalfMirror>(x);
  };
  const int p = tid & 7;
#pragma unroll 1
  for (int pass = 0; pass < kChunk / 32; ++pass) {
    const int rloc = pass * 32 + tid / 8;
    const int qi = row0 + rloc;
    if (qi >= N) break;  // uniform over the row's eight lanes; later passes are further out
    const size_t ri = bh * (size_t)N + qi;
    int n = pass == 0 ? n_ps[0] : n_ps[1];
    const size_t s0 = pass == 0 ? s0_ps[0] : s0_ps[1];
    if ((long long)(s0 + n) > a.pool_cap) n = 0;
    const float lse_o = CAUSAL ? s_lse[rloc] : -INFINITY;
    float lse[NP];
    u32x4 v[NP][2];
    auto load = [&](int k0) {
#pragma unroll
      for (int x = 0; x < NP; ++x) {
        const size_t sl = s0 + min(k0 + x, max(n - 1, 0));
        lse[x] = __builtin_nontemporal_load(a.plse + sl);
        v[x][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.po + sl * D + 8 * p));
        v[x][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.po + sl * D + 64 + 8 * p));
      }
    };
    if (n > 0) load(0);
    float lp = p < n ? a.plse[s0 + p] : -INFINITY;
    for (int k = p + 8; k < n; k += 8) lp = fmaxf(lp, a.plse[s0 + k]);
    const float M = fmaxf(max8(lp), lse_o);
    float L = 0.f;
    if (M > -INFINITY)
      for (int k = p; k < n; k += 8) L += fast_exp2(a.plse[s0 + k] - M);
    L = sum8(L);
    const float wo = (M > -INFINITY && lse_o > -INFINITY) ? fast_exp2(lse_o - M) : 0.f;
    L += wo;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float acc[16];
    {
      const float wt = wo * inv;
      const f32x4* orow = reinterpret_cast<const f32x4*>(&sO[rloc * OROW]);
#pragma unroll
      for (int hv = 0; hv < 2; ++hv)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const f32x4 x = CAUSAL ? orow[(64 * hv + 8 * p) / 4 + e] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[8 * hv + 4 * e + k] = x[k] * wt;
        }
    }
    if (L > 0.f) {
      for (int k0 = 0; k0 < n; k0 += NP) {
        if (k0 > 0) load(k0);
#pragma unroll
        for (int x = 0; x < NP; ++x) {
          const float wt = k0 + x < n ? fast_exp2(lse[x] - M) * inv : 0.f;
#pragma unroll
          for (int hv = 0; hv < 2; ++hv)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t u = v[x][hv][e];
              acc[8 * hv + 2 * e] = fmaf(f16lo(u), wt, acc[8 * hv + 2 * e]);
              acc[8 * hv + 2 * e + 1] = fmaf(f16hi(u), wt, acc[8 * hv + 2 * e + 1]);
            }
        }
      }
    }
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(acc[8 * hv + 2 * e], acc[8 * hv + 2 * e + 1]);
      if (8 * p + 64 * hv < DC) __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(a.O + ri * DC + 8 * p + 64 * hv));
    }
  }
}

hipError_t launch_sparse_prefill(const PrefillAttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_cm_plan, dim3((a.n_bhc + 255) / 256), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(k_cm_scatter, dim3(a.n_tiles, a.Hq, a.B), dim3(256), 0, stream, a);
  const long long cm_grid = std::min<long long>(a.max_items, (long long)a.n_cu * kCmWgPerCu);
  if (a.d == 64)
    hipLaunchKernelGGL((k_prefill_cm<128, 64>), dim3((unsigned)cm_grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_prefill_cm<128, 128>), dim3((unsigned)cm_grid), dim3(256), 0, stream, a);
  const int m_units = a.B * a.Hkv * ((a.N + kChunk - 1) / kChunk);
  const unsigned merge_grid = (unsigned)((m_units + 7) / 8) * 8 * a.g;
  if (a.causal) {
    if (a.d == 64) hipLaunchKernelGGL((k_prefill_merge<true, 64>), dim3(merge_grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_prefill_merge<true, 128>), dim3(merge_grid), dim3(256), 0, stream, a);
  } else {
    if (a.d == 64) hipLaunchKernelGGL((k_prefill_merge<false, 64>), dim3(merge_grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_prefill_merge<false, 128>), dim3(merge_grid), dim3(256), 0, stream, a);
  }
  // row-major fallback for tiles without pool slots (a persistent grid that
  // skips every other tile)
  const int n_units = a.n_tiles * a.B * a.Hkv;
  const int n_work = ((n_units + 7) / 8) * 8 * a.g;
  const int rm_grid = std::min(n_work, ((a.n_cu * 2 + 7) / 8) * 8);
  if (a.beta == 2.f)
    hipLaunchKernelGGL((k_sparse_prefill<128, 2>), dim3(rm_grid), dim3(256), 0, stream, a);
  else if (a.beta == 1.f)
    hipLaunchKernelGGL((k_sparse_prefill<128, 1>), dim3(rm_grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_sparse_prefill<128, 0>), dim3(rm_grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dash
