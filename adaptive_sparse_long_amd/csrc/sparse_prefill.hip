// sparse_prefill.hip -- stage 3 of the DashAttention hierarchy ("How it works"
// 3 on the DashAttention README page, "prior-induced sparse softmax"):
//   O_i = sum_j softmax_j(<q_i, k_j>/sqrt(d) + log w_{i,c(j)}) v_j
// over the tokens of the chunks routed to row i, with w the routing prior.
// Visiting the routed chunks in any order gives the same result (the
// order-invariance of the online softmax, "Axiom ledger" Property 2 on the CoSA
// review page), so each tile walks its ascending chunk list.
//
// One workgroup (four wavefronts, 32 query rows each) per (b, query head, 128-row
// tile), walking the union list of chunks routed to any of its rows. Per chunk:
//   * the 64 x 128 K chunk (row-major) and V chunk (transposed) are staged in a
//     double-buffered LDS ring, the next chunk's global loads in flight while
//     the current one is computed;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as A, Q^T held in
//     registers as B) -- in this orientation every lane owns one query row, so
//     its bias, running max and sum are per-lane scalars and the score
//     registers are directly the B operand P^T of the next product;
//   * scores get the row's log2 weight, the causal mask on the own chunk, an
//     online softmax in the exp2 domain, and O^T += V^T P^T accumulates in
//     registers (V^T from LDS as A).
// A wavefront skips a chunk that lies in its rows' future or that none of its
// rows routed, so executed work follows 32-row unions, not 128-row ones.
// Workgroups are issued longest-tile first, and the g query heads sharing a KV
// head are placed on the same XCD so their chunk reads share that XCD's L2.
#include <algorithm>

#include "kernels.hpp"

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

template <int D>
__global__ __launch_bounds__(256, 2) void k_sparse_prefill(PrefillAttnArgs a) {
  constexpr int NS = D / 16;  // k-steps of S^T = K Q^T
  constexpr int NDB = D / 32; // 32-dim blocks of O^T
  constexpr int KROW = D + KPAD;
  constexpr int VROW = kChunk + VPAD;
  static_assert(D == 128, "staging is laid out for head_dim 128");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kChunk * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VROW];

  if (*a.n_rm == 0) return;  // every tile went chunk-major
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
    const float* biasp = a.bias + toff * kTileRows + w * 32 + (lane & 31);

    const int row0 = tile * kTileRows + w * 32;
    const int cw = row0 / kChunk;
    const int qi = row0 + (lane & 31);
    const int hi32 = lane >> 5;

    // Q^T as the B operand: column qi, dims 16 s + 8 hi32 .. +7
    bf16x8 qb[NS];
    {
      const uint16_t* qp = a.Q + (bh * N + qi) * (size_t)D + 8 * hi32;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        qb[s] = as_bf16x8(qi < N ? ldg16(qp + 16 * s) : u32x4{0, 0, 0, 0});
    }

    const uint16_t* Kb = a.K + ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax * D;
    const uint16_t* Vb = a.V + ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax * D;
    // staging roles: K rows t/16 + 16 r at dims (t%16)*8; V keys 4 (t%16) + r at dims 8 (t/16)
    const int k_row = tid >> 4, k_col = (tid & 15) * 8;
    const int v_kg = tid & 15, v_dg = tid >> 4;
    const int n_keys = N;

    u32x4 kr[4], vr[4];
    // Keys past the sequence end are read from its last row instead (a valid
    // address); their scores are masked, so their weights are exactly zero.
    auto load_chunk = [&](int c) {
      const int base = c * kChunk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(base + k_row + 16 * r, n_keys - 1);
        kr[r] = ldg16(Kb + (size_t)key * D + k_col);
        const int vkey = min(base + 4 * v_kg + r, n_keys - 1);
        vr[r] = ldg16(Vb + (size_t)vkey * D + 8 * v_dg);
      }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4*>(&sK[buf][(k_row + 16 * r) * KROW + k_col]) = kr[r];
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

    float bias_next = 0.f;
    if (count > 0) {
      load_chunk(list[0]);
      bias_next = biasp[0];
      store_chunk(0);
    }
    __syncthreads();

    for (int it = 0; it < count; ++it) {
      const int buf = it & 1;
      const int c = list[it];
      const float bias = bias_next;
      const bool more = it + 1 < count;
      if (more) {
        load_chunk(list[it + 1]);
        bias_next = biasp[(size_t)(it + 1) * kTileRows];
      }
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
      uint16_t* op = a.O + (bh * N + qi) * (size_t)D + 4 * hi32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 v = {pack_bf16x2(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv),
                     pack_bf16x2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + 32 * db + 8 * q4) = v;
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

__global__ __launch_bounds__(1024) void k_cm_plan(PrefillAttnArgs a) {
  __shared__ int s_tmp[2][16];
  int carry_p = 0, carry_i = 0;
  for (int base = 0; base < a.n_bhc; base += 1024) {
    const int idx = base + threadIdx.x;
    const int P = idx < a.n_bhc ? a.cmp[idx] : 0;
    const int ni = ((P + 31) / 32 + kCmBlocks - 1) / kCmBlocks;
    int ep, ei;
    const int tp = block_excl_scan<16>(P, s_tmp[0], ep);
    const int ti = block_excl_scan<16>(ni, s_tmp[1], ei);
    if (idx < a.n_bhc) {
      a.cs[idx] = carry_p + ep;
      for (int j = 0; j < ni; ++j) {
        const long long it = (long long)carry_i + ei + j;
        if (it < a.max_items) a.items[it] = make_int2(idx, j * kCmBlocks);
      }
    }
    carry_p += tp;
    carry_i += ti;
  }
  if (threadIdx.x == 0) *a.nitems = carry_i;
}

// One workgroup per (tile, query head, b): copies the tile's pair records,
// grouped by chunk in its pool range, to their places among the chunk-sorted
// records (each group after the pairs that other tiles reserved before it in
// the same chunk). Thread q copies record q; its group is found by binary
// search over the groups' first records.
__global__ __launch_bounds__(256) void k_cm_scatter(PrefillAttnArgs a) {
  __shared__ int s_first[kRoutePrefillMaxSlots];
  __shared__ long long s_dst[kRoutePrefillMaxSlots];  // destination of record q: s_dst[group] + q
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const size_t bh = (size_t)b * a.Hq + h;
  const int cnt = min(a.ccounts[bh * a.n_tiles + tile], kRoutePrefillMaxSlots);
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

template <int D>
__global__ __launch_bounds__(256, kCmWgPerCu) void k_prefill_cm(PrefillAttnArgs a) {
  constexpr int NS = D / 16;
  constexpr int NDB = D / 32;
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

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
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
      const uint16_t* qp = a.Q + (bh * N + row) * (size_t)D + 8 * hi32;
#pragma unroll
      for (int s = 0; s < NS; ++s) qb[s] = as_bf16x8(ldg16(qp + 16 * s));
    };

    // ---- stage K (row-major) and V (transposed) of chunk c; keys past the
    // sequence end read its last row (masked below). The first block's query
    // rows are fetched meanwhile.
    __syncthreads();  // the previous item's LDS reads are done
    bf16x8 qbuf[2][NS];
    {
      const uint16_t* Kb = a.K + ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax * D;
      const uint16_t* Vb = a.V + ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax * D;
      const int k_row = tid >> 4, k_col = (tid & 15) * 8;
      const int v_kg = tid & 15, v_dg = tid >> 4;
      u32x4 kr[4], vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kr[r] = ldg16(Kb + (size_t)min(c * kChunk + k_row + 16 * r, N - 1) * D + k_col);
        vr[r] = ldg16(Vb + (size_t)min(c * kChunk + 4 * v_kg + r, N - 1) * D + 8 * v_dg);
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
        if (valid && hi32 == 0) a.plse[slot] = l > 0.f ? m + fast_log2(l) : -INFINITY;
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
            if (vr) *reinterpret_cast<u32x4*>(a.po + sr * D + 64 * half + 8 * c16) = v;
          }
          wave_lds_fence();
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: every row with partial results (the rows of tiles that got pool
// slots) combines them, in the order of its slots (consecutive, so rows stream
// through memory). Eight lanes per row: first the row's largest log2 sum and
// the sum of 2^(log2 sum - largest) over its partials (the lanes split the
// partials, DPP reductions over the eight), then each partial's fp16 output
// is added with its normalised weight (v_fma_mix: fp16 in, fp32 sums). Lane p
// owns dims 8p .. 8p+7 and 64+8p .. 64+8p+7, so each load instruction of the
// eight lanes reads 128 contiguous bytes; four partials are in flight together.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_prefill_merge(PrefillAttnArgs a) {
  constexpr int D = 128;
  constexpr int NP = 4;  // partials loaded together
  const size_t rows = (size_t)a.B * a.Hq * a.N;
  const size_t ri = (size_t)blockIdx.x * 32 + threadIdx.x / 8;
  const int p = threadIdx.x & 7;
  if (ri >= rows) return;
  const int n = a.cmcnt[ri];
  if (n == 0) return;  // the row was attended row-major
  const size_t s0 = a.rslot[ri];
  if ((long long)(s0 + n) > a.pool_cap) return;
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
  // the first partials' loads go out before the weights are known
  float lse[NP];
  u32x4 v[NP][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const size_t sl = s0 + min(k0 + x, n - 1);
      lse[x] = a.plse[sl];
      v[x][0] = ldg16(a.po + sl * D + 8 * p);
      v[x][1] = ldg16(a.po + sl * D + 64 + 8 * p);
    }
  };
  load(0);
  float lp = p < n ? a.plse[s0 + p] : -INFINITY;
  for (int k = p + 8; k < n; k += 8) lp = fmaxf(lp, a.plse[s0 + k]);
  const float M = max8(lp);
  float L = 0.f;
  if (M > -INFINITY)
    for (int k = p; k < n; k += 8) L += fast_exp2(a.plse[s0 + k] - M);
  L = sum8(L);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
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
            acc[8 * hv + 2 * e] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu)), wt, acc[8 * hv + 2 * e]);
            acc[8 * hv + 2 * e + 1] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)), wt, acc[8 * hv + 2 * e + 1]);
          }
      }
    }
  }
#pragma unroll
  for (int hv = 0; hv < 2; ++hv) {
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(acc[8 * hv + 2 * e], acc[8 * hv + 2 * e + 1]);
    *reinterpret_cast<u32x4*>(a.O + ri * D + 8 * p + 64 * hv) = out;
  }
}

hipError_t launch_sparse_prefill(const PrefillAttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_cm_plan, dim3(1), dim3(1024), 0, stream, a);
  hipLaunchKernelGGL(k_cm_scatter, dim3(a.n_tiles, a.Hq, a.B), dim3(256), 0, stream, a);
  const long long cm_grid = std::min<long long>(a.max_items, (long long)a.n_cu * kCmWgPerCu);
  hipLaunchKernelGGL(k_prefill_cm<128>, dim3((unsigned)cm_grid), dim3(256), 0, stream, a);
  const long long rows = (long long)a.B * a.Hq * a.N;
  hipLaunchKernelGGL(k_prefill_merge, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, stream, a);
  // row-major fallback for tiles without pool slots (a persistent grid that
  // skips every other tile)
  const int n_units = a.n_tiles * a.B * a.Hkv;
  const int n_work = ((n_units + 7) / 8) * 8 * a.g;
  const int rm_grid = std::min(n_work, ((a.n_cu * 2 + 7) / 8) * 8);
  hipLaunchKernelGGL(k_sparse_prefill<128>, dim3(rm_grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dash
