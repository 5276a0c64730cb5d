// summarize.hip -- stage 1 of the DashAttention hierarchy ("How it works" 1 on
// the DashAttention README page): one key summary per KV chunk, pooled with the
// per-KV-head vector head_cls:
//     a_j = softmax_j(<k_j, cls> / sqrt(d)),   s_c = sum_j a_j k_j   (float32)
//
// One wavefront per (b, kv head, chunk). A 64 x 128 bf16 chunk is 16 KB of
// contiguous memory; each load instruction of the wave reads 1 KB of it (four
// rows, 16 lanes x 16 bytes per row), so every byte of K is read once with full
// coalescing. The kernel is bound by HBM bandwidth.
#include "kernels.hpp"

namespace dash {

template <int D>
__global__ __launch_bounds__(256) void k_summarize(const uint16_t* __restrict__ K,
                                                   const uint16_t* __restrict__ cls,
                                                   float* __restrict__ S, int Hkv, int Lmax,
                                                   int n_tokens, const int* __restrict__ seqlens,
                                                   int chunk_begin, int chunk_end, int s_cap,
                                                   int C, float inv_sqrt_d) {
  constexpr int LPR = D / 8;          // lanes per key row (16 bytes each)
  constexpr int RPI = kWave / LPR;    // rows per load instruction
  static_assert(LPR == 16, "summary kernel is laid out for head_dim 128");
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int c = chunk_begin + blockIdx.x * (blockDim.x / kWave) + wave;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  if (c >= chunk_end) return;
  const int n_b = min(seqlens ? seqlens[b] : n_tokens, Lmax);
  int t0 = c * C;
  int t1 = min(t0 + C, n_b);
  if (seqlens && t0 + C > n_b) return;  // append mode: complete chunks only
  if (t1 <= t0) return;
  const int n_valid = t1 - t0;
  const int col = (lane % LPR) * 8;   // first of this lane's 8 dims
  const int rsub = lane / LPR;        // row within a load instruction

  float w_cls[8];
  {
    u32x4 cv = ldg16(cls + (size_t)h * D + col);
    for (int e = 0; e < 4; ++e) {
      w_cls[2 * e] = bf16lo(cv[e]);
      w_cls[2 * e + 1] = bf16hi(cv[e]);
    }
  }
  const uint16_t* kbase = K + (((size_t)b * Hkv + h) * Lmax + t0) * D;
  // C / RPI rows per lane; C <= 64 keeps this at most 16 registers of 16 bytes.
  constexpr int kMaxIt = 64 / RPI;
  u32x4 kv[kMaxIt];
  float logit[kMaxIt];
  const int n_it = (C + RPI - 1) / RPI;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    int row = it * RPI + rsub;
    if (it < n_it && row < n_valid) {
      kv[it] = ldg16(kbase + (size_t)row * D + col);
    } else {
      kv[it] = u32x4{0, 0, 0, 0};
    }
  }
  float mx = kNegBig;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    float part = 0.f;
    for (int e = 0; e < 4; ++e) {
      part = fmaf(bf16lo(kv[it][e]), w_cls[2 * e], part);
      part = fmaf(bf16hi(kv[it][e]), w_cls[2 * e + 1], part);
    }
    float lg = sum16(part) * inv_sqrt_d;
    int row = it * RPI + rsub;
    lg = (it < n_it && row < n_valid) ? lg : -INFINITY;
    logit[it] = lg;
    mx = fmaxf(mx, lg);
  }
  mx = max_xor32(max_xor16(mx));
  float den = 0.f;
  float acc[8];
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    float a = fast_exp2((logit[it] - mx) * kLog2e);  // 0 for masked rows
    den += a;
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(a, bf16lo(kv[it][e]), acc[2 * e]);
      acc[2 * e + 1] = fmaf(a, bf16hi(kv[it][e]), acc[2 * e + 1]);
    }
  }
  // every lane of a row group saw the same rows: den is per row group
  den = sum_xor32(sum_xor16(den));
  for (int e = 0; e < 8; ++e) acc[e] = sum_xor32(sum_xor16(acc[e]));
  if (lane < LPR) {
    float inv = 1.f / den;
    float* dst = S + (((size_t)b * Hkv + h) * s_cap + c) * D + col;
    f32x4 lo = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    f32x4 hi = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    *reinterpret_cast<f32x4*>(dst) = lo;
    *reinterpret_cast<f32x4*>(dst + 4) = hi;
  }
}

hipError_t launch_summarize(const SummarizeArgs& a, hipStream_t stream) {
  const int n = a.chunk_end - a.chunk_begin;
  dim3 grid((n + 3) / 4, a.Hkv, a.B);
  hipLaunchKernelGGL(k_summarize<128>, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.cls), a.S,
                     a.Hkv, a.Lmax, a.n_tokens, a.seqlens, a.chunk_begin, a.chunk_end, a.s_cap,
                     a.C, a.inv_sqrt_d);
  return hipGetLastError();
}

}  // namespace dash
