// summarize.hip -- stage 1 of the DashAttention hierarchy ("How it works" 1 on
// the DashAttention README page): one key summary per KV chunk, pooled with the
// per-KV-head vector head_cls:
//     a_j = softmax_j(<k_j, cls> / sqrt(d)),   s_c = sum_j a_j k_j   (float32)
//
// One wavefront per (b, kv head, chunk). A 64 x 128 bf16 chunk is 16 KB of
// contiguous memory; each load instruction of the wave reads 1 KB of it (four
// rows, 16 lanes x 16 bytes per row; at head_dim 64, eight rows of 8 lanes), so
// every byte of K is read once with full coalescing. The kernel is bound by HBM
// bandwidth.
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
  static_assert(LPR == 16 || LPR == 8, "head_dim 128 or 64");
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
    float lg = (LPR == 16 ? sum16(part) : sum8(part)) * inv_sqrt_d;
    int row = it * RPI + rsub;
    lg = (it < n_it && row < n_valid) ? lg : -INFINITY;
    logit[it] = lg;
    mx = fmaxf(mx, lg);
  }
  // across the row groups of a load instruction (lanes l ^ LPR, ...)
  if (LPR == 8) mx = max_xor8(mx);
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
  if (LPR == 8) {
    den = sum_xor8(den);
    for (int e = 0; e < 8; ++e) acc[e] = sum_xor8(acc[e]);
  }
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
  if (a.d == 64)
    hipLaunchKernelGGL(k_summarize<64>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.cls), a.S,
                       a.Hkv, a.Lmax, a.n_tokens, a.seqlens, a.chunk_begin, a.chunk_end, a.s_cap,
                       a.C, a.inv_sqrt_d);
  else
    hipLaunchKernelGGL(k_summarize<128>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.cls), a.S,
                       a.Hkv, a.Lmax, a.n_tokens, a.seqlens, a.chunk_begin, a.chunk_end, a.s_cap,
                       a.C, a.inv_sqrt_d);
  return hipGetLastError();
}

}  // namespace dash

// ---------------------------------------------------------------------------
// Backward of the summary: for a cotangent ds of s_c (the pages differentiate
// the whole hierarchy; the steps are the summary's own chain rule),
//     de_j = a_j (<k_j, ds> - <s_c, ds>),
//     dk_j = a_j ds + de_j cls / sqrt(d),   dcls += sum_j de_j k_j / sqrt(d).
// k_summarize_bwd keeps the forward's layout (one wavefront per chunk, the
// chunk's keys read once into registers), recomputes a and s_c, writes dk of
// every token of the chunk and the chunk's dcls term into a partial row;
// k_summarize_bwd_reduce adds the partial rows of each kv head in a fixed order
// (deterministic).
namespace dash {

template <int D>
__global__ __launch_bounds__(256) void k_summarize_bwd(SummarizeBwdArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPI = kWave / LPR;
  static_assert(LPR == 16 || LPR == 8, "head_dim 128 or 64");
  // sums over a row's LPR lanes, and over the row groups of a load instruction
  auto rsum = [](float x) { return LPR == 16 ? sum16(x) : sum8(x); };
  auto gsum = [](float x) {
    if (LPR == 8) x = sum_xor8(x);
    return sum_xor32(sum_xor16(x));
  };
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int c = a.chunk_begin + blockIdx.x * (blockDim.x / kWave) + wave;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  if (c >= a.chunk_end) return;
  const int col = (lane % LPR) * 8;
  const int rsub = lane / LPR;
  const int n_chunks = a.chunk_end - a.chunk_begin;
  float* part = a.partials + (((size_t)b * a.Hkv + h) * n_chunks + (c - a.chunk_begin)) * D + col;
  const int t0 = c * a.C;
  const int t1 = min(t0 + a.C, a.n_tokens);
  if (t1 <= t0) {  // no token in this chunk: a zero term
    if (lane < LPR) {
      *reinterpret_cast<f32x4*>(part) = f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(part + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int n_valid = t1 - t0;

  float w_cls[8], g[8];
  {
    const u32x4 cv = ldg16(static_cast<const uint16_t*>(a.cls) + (size_t)h * D + col);
    for (int e = 0; e < 4; ++e) {
      w_cls[2 * e] = bf16lo(cv[e]);
      w_cls[2 * e + 1] = bf16hi(cv[e]);
    }
    const float* gp = a.dS + (((size_t)b * a.Hkv + h) * a.s_cap + c) * D + col;
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
    for (int e = 0; e < 4; ++e) {
      g[e] = g0[e];
      g[4 + e] = g1[e];
    }
  }
  const uint16_t* kbase = static_cast<const uint16_t*>(a.K) + (((size_t)b * a.Hkv + h) * a.Lmax + t0) * D;
  constexpr int kMaxIt = 64 / RPI;
  u32x4 kv[kMaxIt];
  float logit[kMaxIt], dot[kMaxIt];
  const int n_it = (a.C + RPI - 1) / RPI;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int row = it * RPI + rsub;
    kv[it] = (it < n_it && row < n_valid) ? ldg16(kbase + (size_t)row * D + col) : u32x4{0, 0, 0, 0};
  }
  float mx = kNegBig;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    float pl = 0.f, pd = 0.f;
    for (int e = 0; e < 4; ++e) {
      const float k0 = bf16lo(kv[it][e]), k1 = bf16hi(kv[it][e]);
      pl = fmaf(k0, w_cls[2 * e], pl);
      pl = fmaf(k1, w_cls[2 * e + 1], pl);
      pd = fmaf(k0, g[2 * e], pd);
      pd = fmaf(k1, g[2 * e + 1], pd);
    }
    const int row = it * RPI + rsub;
    const bool ok = it < n_it && row < n_valid;
    logit[it] = ok ? rsum(pl) * a.inv_sqrt_d : -INFINITY;
    dot[it] = rsum(pd);  // <k_j, ds>
    mx = fmaxf(mx, logit[it]);
  }
  if (LPR == 8) mx = max_xor8(mx);
  mx = max_xor32(max_xor16(mx));
  float den = 0.f, sacc[8];
  for (int e = 0; e < 8; ++e) sacc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    logit[it] = fast_exp2((logit[it] - mx) * kLog2e);  // unnormalised weight, 0 for masked rows
    den += logit[it];
    for (int e = 0; e < 4; ++e) {
      sacc[2 * e] = fmaf(logit[it], bf16lo(kv[it][e]), sacc[2 * e]);
      sacc[2 * e + 1] = fmaf(logit[it], bf16hi(kv[it][e]), sacc[2 * e + 1]);
    }
  }
  den = gsum(den);
  const float inv = 1.f / den;
  float sd = 0.f;  // <s_c, ds> over this lane's dims, then over the row
  for (int e = 0; e < 8; ++e) sd = fmaf(gsum(sacc[e]) * inv, g[e], sd);
  sd = rsum(sd);

  float pc[8];
  for (int e = 0; e < 8; ++e) pc[e] = 0.f;
  float* dkbase = a.dK + (((size_t)b * a.Hkv + h) * a.Lmax + t0) * D + col;
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int row = it * RPI + rsub;
    const float aj = logit[it] * inv;
    const float de = aj * (dot[it] - sd);
    const float dc = de * a.inv_sqrt_d;
    float o[8];
    for (int e = 0; e < 4; ++e) {
      const float k0 = bf16lo(kv[it][e]), k1 = bf16hi(kv[it][e]);
      pc[2 * e] = fmaf(de, k0, pc[2 * e]);
      pc[2 * e + 1] = fmaf(de, k1, pc[2 * e + 1]);
      o[2 * e] = fmaf(aj, g[2 * e], dc * w_cls[2 * e]);
      o[2 * e + 1] = fmaf(aj, g[2 * e + 1], dc * w_cls[2 * e + 1]);
    }
    if (it < n_it && row < n_valid) {
      float* dst = dkbase + (size_t)row * D;
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
    }
  }
  for (int e = 0; e < 8; ++e) pc[e] = gsum(pc[e]) * a.inv_sqrt_d;
  if (lane < LPR) {
    *reinterpret_cast<f32x4*>(part) = f32x4{pc[0], pc[1], pc[2], pc[3]};
    *reinterpret_cast<f32x4*>(part + 4) = f32x4{pc[4], pc[5], pc[6], pc[7]};
  }
}

// dcls[h] = sum over b and chunks of the partial rows, in two levels with a
// fixed partition (so the result is deterministic):
//   1. workgroup (j, h, b) adds the partial rows of chunks [j R, (j+1) R) of
//      (b, h) -- 8 row streams x 32 float4 columns, the streams then added in
//      order through LDS -- and writes the sum over the first row of its range
//      (a row only it reads, read before it is written);
//   2. workgroup h adds those range sums in (b, j) order.
constexpr int kRedRows = 256;  // partial rows per first-level workgroup

template <int D>
__global__ __launch_bounds__(256) void k_summarize_bwd_reduce1(SummarizeBwdArgs a) {
  constexpr int kCols = D / 4;           // float4 columns per row
  constexpr int kStreams = 256 / kCols;  // row streams
  __shared__ f32x4 s_acc[kStreams][kCols];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int q = threadIdx.x % kCols;
  const int st = threadIdx.x / kCols;
  const int n_chunks = a.chunk_end - a.chunk_begin;
  const int c0 = j * kRedRows, c1 = min(n_chunks, c0 + kRedRows);
  f32x4* rows = reinterpret_cast<f32x4*>(a.partials + ((size_t)b * a.Hkv + h) * n_chunks * D);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int c = c0 + st; c < c1; c += kStreams) acc += rows[(size_t)c * kCols + q];
  s_acc[st][q] = acc;
  __syncthreads();
  if (threadIdx.x < kCols) {
    f32x4 t = s_acc[0][threadIdx.x];
    for (int i = 1; i < kStreams; ++i) t += s_acc[i][threadIdx.x];
    rows[(size_t)c0 * kCols + threadIdx.x] = t;
  }
}

template <int D>
__global__ __launch_bounds__(D) void k_summarize_bwd_reduce2(SummarizeBwdArgs a) {
  const int h = blockIdx.x;
  const int n_chunks = a.chunk_end - a.chunk_begin;
  float t = 0.f;
  for (int b = 0; b < a.B; ++b) {
    const float* rows = a.partials + ((size_t)b * a.Hkv + h) * n_chunks * D + threadIdx.x;
    for (int c0 = 0; c0 < n_chunks; c0 += kRedRows) t += rows[(size_t)c0 * D];
  }
  a.dcls[(size_t)h * D + threadIdx.x] = t;
}

template <int D>
static hipError_t summarize_bwd_d(const SummarizeBwdArgs& a, hipStream_t stream) {
  const int n = a.chunk_end - a.chunk_begin;
  if (n > 0) {
    dim3 grid((n + 3) / 4, a.Hkv, a.B);
    hipLaunchKernelGGL(k_summarize_bwd<D>, grid, dim3(256), 0, stream, a);
    dim3 g1((n + kRedRows - 1) / kRedRows, a.Hkv, a.B);
    hipLaunchKernelGGL(k_summarize_bwd_reduce1<D>, g1, dim3(256), 0, stream, a);
  }
  hipLaunchKernelGGL(k_summarize_bwd_reduce2<D>, dim3(a.Hkv), dim3(D), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_summarize_bwd(const SummarizeBwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? summarize_bwd_d<64>(a, stream) : summarize_bwd_d<128>(a, stream);
}

}  // namespace dash
