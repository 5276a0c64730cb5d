// sparse_decode.hip -- stage 3 of the DashAttention hierarchy for one new token
// per sequence, reading only the routed chunks of the KV cache (the
// prefill/decoding paragraph of "How it works" on the DashAttention README page:
// decoding reuses the chunk-summary cache).
//
// The g query heads of one KV head share one routed-chunk list (the union of
// their routes), so each listed 16 KB K chunk and 16 KB V chunk is read from HBM
// once for all g heads. Split-KV: a workgroup of four wavefronts takes 24 list
// entries; each wavefront streams its chunks with no block barrier:
//   * scores for the g heads: v_mfma_f32_16x16x32_bf16 with the query rows in A
//     (head hh at row hh * 16/g, so each 16-lane row group of the output holds
//     one head) and the K chunk in B, read straight from global memory as
//     16-byte row segments;
//   * online softmax in the exp2 domain with the head's log2 routing weight;
//   * O += P V on the vector ALUs: each lane owns 8 dims and 16 keys, V read as
//     16-byte row segments; the probabilities go through a small per-wavefront
//     LDS slot.
// The four wavefront partials are merged in LDS, the workgroup partial (max,
// sum, unnormalised output per head) goes to the workspace, and a combine kernel
// merges the splits in a fixed order (deterministic).
#include "kernels.hpp"

namespace dash {

// DC: the caller's head_dim (row width of q, K, V), a template argument so that
// the 128-dim instance has no per-load head_dim test
template <int G, int DC>
__global__ __launch_bounds__(256) void k_sparse_decode(DecodeAttnArgs a) {
  constexpr int D = 128;
  constexpr int NS = D / 32;
  constexpr int RSTEP = 16 / G;      // A-row spacing of the heads
  constexpr int HPG = G > 4 ? G / 4 : 1;  // heads per 16-lane row group
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "g must be 1, 2, 4 or 8");
  __shared__ float sP[4][64 * G];
  __shared__ float sA[4][G];
  __shared__ float sM[4][G], sL[4][G];
  __shared__ float sO[4][G][D];

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int split = blockIdx.x;
  const int grp_id = blockIdx.y;
  const int b = grp_id / a.Hkv;
  const int hk = grp_id % a.Hkv;
  const int count = a.counts[grp_id];
  if (split * kDecodeSplit >= count) return;  // whole workgroup
  const int t = min(max(a.seqlens[b], 1), a.Lmax) - 1;  // clamp to the cache
  const int n_keys = t + 1;
  const size_t gbase = (size_t)grp_id * a.n_slots;
  const int col = lane & 15;
  const int rg = lane >> 4;

  // q rows as A operand: A row m = col; head hh sits at row hh * RSTEP
  bf16x8 qa[NS];
  {
    const bool has = (col % RSTEP) == 0 && col / RSTEP < G;
    const size_t qrow = (size_t)b * a.Hq + hk * G + col / RSTEP;
#pragma unroll
    for (int s = 0; s < NS; ++s) qa[s] = as_bf16x8(has ? ldg16_dc<DC>(a.Q, qrow, 32 * s + 8 * rg) : u32x4{0, 0, 0, 0});
  }
  // heads held by this lane in the score layout: D row 4 rg + j is head (4 rg + j) / RSTEP
  int my_head[HPG];
  bool my_valid[HPG];
#pragma unroll
  for (int q = 0; q < HPG; ++q) {
    const int row = 4 * rg + q * RSTEP;  // j = q * RSTEP (only for G == 8 is HPG 2)
    my_valid[q] = (row % RSTEP) == 0 && row / RSTEP < G && (G > 4 || q == 0);
    my_head[q] = row / RSTEP;
  }

  float m_run[HPG], l_run[HPG];
#pragma unroll
  for (int q = 0; q < HPG; ++q) {
    m_run[q] = kNegBig;
    l_run[q] = 0.f;
  }
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;

  const size_t kvrow0 = ((size_t)b * a.Hkv + hk) * (size_t)a.Lmax;
  const float sc = a.scale_log2;
  const int pos_end = min(count, (split + 1) * kDecodeSplit);

  for (int pos = split * kDecodeSplit + w; pos < pos_end; pos += 4) {
    const int c = a.lists[gbase + pos];
    const int base = c * kChunk;
    // ---- loads: K in MFMA B layout, V rows for the ALU product
    u32x4 kv[4][NS];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = base + kb * 16 + col;
      const bool val = key < n_keys;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        kv[kb][s] = val ? ldg16_dc<DC>(a.K, kvrow0 + key, 32 * s + 8 * rg) : u32x4{0, 0, 0, 0};
    }
    float bias[HPG];
#pragma unroll
    for (int q = 0; q < HPG; ++q) bias[q] = my_valid[q] ? a.bias[(gbase + pos) * G + my_head[q]] : -INFINITY;

    // ---- scores: lane holds key kb*16 + col for D rows 4 rg + j
    f32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) z = mfma16x16x32(qa[s], as_bf16x8(kv[kb][s]), z);
      sacc[kb] = z;
    }
    // V after the scores: K's registers are free by then
    __builtin_amdgcn_sched_barrier(0);
    u32x4 vv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = base + rg + 4 * r;
      vv[r] = key < n_keys ? ldg16_dc<DC>(a.V, kvrow0 + key, 8 * col) : u32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_sched_barrier(0);
    float alpha_h[HPG];
#pragma unroll
    for (int q = 0; q < HPG; ++q) {
      const int j = q * RSTEP;  // D-layout register of this head
      float x[4];
      float mx = kNegBig;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = base + kb * 16 + col;
        float v = fmaf(sacc[kb][j], sc, bias[q]);
        if (key >= n_keys) v = -INFINITY;
        x[kb] = v;
        mx = fmaxf(mx, v);
      }
      mx = max16(mx);
      const float m_new = fmaxf(m_run[q], mx);
      const float al = fast_exp2(m_run[q] - m_new);
      m_run[q] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float p = fast_exp2(x[kb] - m_new);
        ls += p;
        if (my_valid[q]) sP[w][(kb * 16 + col) * G + my_head[q]] = p;
      }
      l_run[q] = fmaf(l_run[q], al, ls);
      alpha_h[q] = al;
      if (my_valid[q] && col == 0) sA[w][my_head[q]] = al;
    }
    wave_lds_fence();
    // ---- O = O * alpha + P V  (lane: dims 8 col .. +7, keys rg + 4 r)
    float al_all[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) al_all[hh] = sA[w][hh];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= al_all[hh];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = rg + 4 * r;
      float p[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) p[hh] = sP[w][kk * G + hh];
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16lo(vv[r][e]);
        vf[2 * e + 1] = bf16hi(vv[r][e]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(p[hh], vf[e], acc[hh][e]);
    }
    wave_lds_fence();
    (void)alpha_h;
  }

  // ---- wavefront partial: sum over the four key groups (lanes l, l^16, l^32, l^48)
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = sum_xor32(sum_xor16(acc[hh][e]));
#pragma unroll
  for (int q = 0; q < HPG; ++q) {
    const float lt = sum16(l_run[q]);
    if (my_valid[q] && col == 0) {
      sM[w][my_head[q]] = m_run[q];
      sL[w][my_head[q]] = lt;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) sO[w][hh][8 * lane + e] = acc[hh][e];
  }
  __syncthreads();
  // ---- merge the four wavefronts; write the split partial
  float* part = a.part + ((size_t)grp_id * a.n_splits + split) * G * (D + 2);
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int hh = i / D, dd = i % D;
    float M = kNegBig;
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sM[ww][hh]);
    float o = 0.f;
    for (int ww = 0; ww < 4; ++ww) o += sO[ww][hh][dd] * fast_exp2(sM[ww][hh] - M);
    part[hh * (D + 2) + 2 + dd] = o;
    if (dd == 0) {
      float L = 0.f;
      for (int ww = 0; ww < 4; ++ww) L += sL[ww][hh] * fast_exp2(sM[ww][hh] - M);
      part[hh * (D + 2)] = M;
      part[hh * (D + 2) + 1] = L;
    }
  }
}

// Merge the split partials of one (b, query head) in split order and store O:
// one workgroup per head, one thread per dim.
template <int G>
__global__ __launch_bounds__(128) void k_decode_combine(DecodeAttnArgs a) {
  constexpr int D = 128;
  const int grp_id = blockIdx.x / G;
  const int hh = blockIdx.x % G;
  const int b = grp_id / a.Hkv;
  const int hk = grp_id % a.Hkv;
  const int dd = threadIdx.x;
  const int count = a.counts[grp_id];
  const int ns = (count + kDecodeSplit - 1) / kDecodeSplit;
  const float* part = a.part + (size_t)grp_id * a.n_splits * G * (D + 2) + hh * (D + 2);
  constexpr int kStride = G * (D + 2);
  // one pass with a running max; eight splits' loads in flight per step
  float M = kNegBig, L = 0.f, o = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float pm[8], pl[8], po[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* p = part + min(s0 + j, ns - 1) * kStride;
      pm[j] = s0 + j < ns ? p[0] : kNegBig;
      pl[j] = p[1];
      po[j] = p[2 + dd];
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < 8; ++j) Mn = fmaxf(Mn, pm[j]);
    const float a = fast_exp2(M - Mn);
    L *= a;
    o *= a;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = s0 + j < ns ? fast_exp2(pm[j] - Mn) : 0.f;
      L = fmaf(pl[j], e, L);
      o = fmaf(po[j], e, o);
    }
    M = Mn;
  }
  if (dd < a.d) a.O[((size_t)b * a.Hq + hk * G + hh) * a.d + dd] = __builtin_bit_cast(uint16_t, (__bf16)(o / L));
}

template <int G>
static hipError_t decode_g(const DecodeAttnArgs& a, hipStream_t stream) {
  if (a.d == 64)
    hipLaunchKernelGGL((k_sparse_decode<G, 64>), dim3(a.n_splits, a.B * a.Hkv), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_sparse_decode<G, 128>), dim3(a.n_splits, a.B * a.Hkv), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(k_decode_combine<G>, dim3(a.B * a.Hkv * G), dim3(128), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sparse_decode(const DecodeAttnArgs& a, hipStream_t stream) {
  switch (a.g) {
    case 1: return decode_g<1>(a, stream);
    case 2: return decode_g<2>(a, stream);
    case 4: return decode_g<4>(a, stream);
    case 8: return decode_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dash
