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

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int tid = threadIdx.x;

  // ---- work unit: (tile, b, kv head), heaviest tiles first; the g heads of a
  // unit get workgroup ids that are equal modulo 8 (same XCD)
  const int g = a.g;
  const int n_units = a.n_tiles * a.B * a.Hkv;
  const int idx = blockIdx.x;
  const int grp8 = idx / (8 * g);
  const int rem = idx % (8 * g);
  const int gh = rem / 8;
  const int unit = grp8 * 8 + rem % 8;
  if (unit >= n_units) return;
  const int tile = a.n_tiles - 1 - unit / (a.B * a.Hkv);
  const int bhk = unit % (a.B * a.Hkv);
  const int b = bhk / a.Hkv;
  const int hk = bhk % a.Hkv;
  const int h = hk * g + gh;
  const size_t bh = (size_t)b * a.Hq + h;
  const int N = a.N;
  const bool causal = a.causal != 0;

  const int count = a.counts[bh * a.n_tiles + tile];
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

hipError_t launch_sparse_prefill(const PrefillAttnArgs& a, hipStream_t stream) {
  const int n_units = a.n_tiles * a.B * a.Hkv;
  const int grid = ((n_units + 7) / 8) * 8 * a.g;
  hipLaunchKernelGGL(k_sparse_prefill<128>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dash
