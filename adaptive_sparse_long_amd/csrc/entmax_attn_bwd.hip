// entmax_attn_bwd.hip -- backward of the dense alpha-entmax attention with
// block skipping (the AdaSplash README page: "Usage", "AdaSplash with Block
// Masking", whose kernels run forward and backward; "Key Features", block-sparse
// forward and backward passes).
//
// With s_ij = <q_i, k_j> / sqrt(d), u = (alpha - 1) s, t_ij = u_ij - tau_i and
// beta = 1 / (alpha - 1), the forward weights are P_ij = max(t_ij, 0)^beta and
// O = P V. The alpha-entmax Jacobian (Peters, Niculae & Martins 2019) is
// diag(g) - g g^T / sum(g) with g = P^(2 - alpha) = max(t, 0)^((2 - alpha) beta)
// on the support, so for a cotangent dO:
//   dP_ij = <dO_i, v_j>,  c_i = sum_j g_ij dP_ij / sum_j g_ij,
//   dS_ij = g_ij (dP_ij - c_i),
//   dQ_i = sum_j dS_ij k_j / sqrt(d),  dK_j = sum_i dS_ij q_i / sqrt(d),
//   dV_j = sum_i P_ij dO_i.
// Every term is zero off the support, so a 64 x 64 tile whose block-mask bit
// is 0 contributes nothing and is skipped.
//
// Two kernels, both wavefront-per-32-lines, four wavefronts per workgroup:
//   k_entmax_bwd_dq   (row pass): a wavefront owns 32 query rows. Pass 1 over
//       the key blocks builds S^T = K Q^T and dP^T = V dO^T by MFMA (a lane owns
//       one row) and sums g and g dP per row, giving c (stored for the second
//       kernel). Pass 2 recomputes both products, forms dS and accumulates
//       dQ^T += K^T dS^T, K staged transposed in the wavefront's LDS slot.
//   k_entmax_bwd_dkdv (column pass): a wavefront owns 32 keys. Over the query
//       blocks it builds S = Q K^T and dP = dO V^T (a lane owns one key), forms
//       P and dS from tau and c, and accumulates dV^T += dO^T P and
//       dK^T += Q^T dS with Q and dO staged transposed in LDS.
// bfloat16 operands run on v_mfma_f32_32x32x16_bf16 with the weights split
// into bf16 high and low parts (float32 accuracy); float32 operands on
// v_mfma_f32_32x32x2_f32, transposed operands read straight from memory
// (32 consecutive floats per half-wavefront).
#include "kernels.hpp"
#include "tau_solve.hpp"

namespace dash {

namespace {
constexpr int kRowPad = 4;
constexpr int kTRow = 32 + kRowPad;  // LDS row of a transposed 32-line block (elements)

__device__ __forceinline__ uint32_t perm_lo16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// g = max(t, 0)^((2 - alpha) beta), the entmax Jacobian's weight.
template <int KIND>
__device__ __forceinline__ float jac_weight(float t, float alpha, float beta) {
  if constexpr (KIND == 2) return fmaxf(t, 0.f);           // alpha = 1.5: exponent 1
  else if constexpr (KIND == 1) return t > 0.f ? 1.f : 0.f;  // alpha = 2: exponent 0
  else return t > 0.f ? fast_exp2((2.f - alpha) * beta * fast_log2(t)) : 0.f;
}

template <bool BF, int D>
struct Frags {
  static constexpr int NS = BF ? D / 16 : D / 2;
  bf16x8 b[BF ? NS : 1];
  float f[BF ? 1 : NS];
};

// Operand fragments of one row (row index valid < n_ok, else zeros): bf16 rows
// give 8 elements per k-step at d = 16 s + 8 (lane / 32); float rows one
// element at d = 2 s + lane / 32.
template <bool BF, int D>
__device__ __forceinline__ void load_frags(Frags<BF, D>& fr, const void* base, int row, bool ok) {
  const int hi32 = lane_id() >> 5;
  if constexpr (BF) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + (size_t)row * D + 8 * hi32;
#pragma unroll
    for (int s = 0; s < Frags<BF, D>::NS; ++s) fr.b[s] = as_bf16x8(ok ? ldg16(p + 16 * s) : u32x4{0, 0, 0, 0});
  } else {
    const float* p = static_cast<const float*>(base) + (size_t)row * D + hi32;
#pragma unroll
    for (int s = 0; s < Frags<BF, D>::NS; ++s) fr.f[s] = ok ? p[2 * s] : 0.f;
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

// Stage rows [r0, r0 + 32) of a row-major [*, D] bf16 matrix transposed into
// xt[D][kTRow] (rows >= n_ok as zeros). Lane combos: 4 rows x 8 dims each.
template <int D>
__device__ __forceinline__ void stage_t(uint16_t* xt, const uint16_t* X, int r0, int n_ok) {
  const int lane = lane_id();
  constexpr int NCOMBO = 8 * (D / 8);
#pragma unroll
  for (int pass = 0; pass < NCOMBO / 64; ++pass) {
    const int combo = pass * 64 + lane;
    const int kg = combo & 7, dg = combo >> 3;
    u32x4 vr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * kg + r;
      vr[r] = row < n_ok ? ldg16(X + (size_t)row * D + 8 * dg) : u32x4{0, 0, 0, 0};
    }
    uint16_t* dst = xt + (8 * dg) * kTRow + 4 * kg;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x2 lo2 = {perm_lo16(vr[0][e], vr[1][e]), perm_lo16(vr[2][e], vr[3][e])};
      u32x2 hi2 = {perm_hi16(vr[0][e], vr[1][e]), perm_hi16(vr[2][e], vr[3][e])};
      *reinterpret_cast<u32x2*>(dst + (2 * e) * kTRow) = lo2;
      *reinterpret_cast<u32x2*>(dst + (2 * e + 1) * kTRow) = hi2;
    }
  }
}

// acc[db] (C[m = dim 32 db + .][n = lane's line]) += X^T W^T over the block's 32
// lines, where W^T is this lane's column w (acc layout: line 8 (r/4) + 4 (l/32)
// + r%4 of register r) and X the block's rows: bf16 from the transposed LDS
// copy xt, float32 straight from memory (rows >= n_ok contribute zeros).
template <bool BF, int D>
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
        const float r0f = round_bf16(a0), r1f = round_bf16(a1);
        h[e] = pack_bf16x2(r0f, r1f);
        l[e] = pack_bf16x2(a0 - r0f, a1 - r1f);
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
        acc[db] = mfma32x32x16(xa, wl[ks], acc[db]);
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

// Write the lane's line of acc (dims 32 db + 8 q4 + 4 (l/32) + 0..3) times mul.
template <bool BF, int D>
__device__ __forceinline__ void store_line(void* out, size_t line, const f32x16 (&acc)[D / 32], float mul) {
  const int hi32 = lane_id() >> 5;
  if constexpr (BF) {
    uint16_t* op = static_cast<uint16_t*>(out) + line * D + 4 * hi32;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 v = {pack_bf16x2(acc[db][4 * q4] * mul, acc[db][4 * q4 + 1] * mul),
                   pack_bf16x2(acc[db][4 * q4 + 2] * mul, acc[db][4 * q4 + 3] * mul)};
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * q4) = v;
      }
  } else {
    float* op = static_cast<float*>(out) + line * D + 4 * hi32;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v = {acc[db][4 * q4] * mul, acc[db][4 * q4 + 1] * mul, acc[db][4 * q4 + 2] * mul,
                   acc[db][4 * q4 + 3] * mul};
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * q4) = v;
      }
  }
}

__device__ __forceinline__ bool tile_on(const EntmaxBwdArgs& a, size_t bh, int nT, int I, int J) {
  if (!a.mask) return true;
  return (a.mask[(bh * nT + I) * a.mask_words + (J >> 5)] >> (J & 31)) & 1u;
}
}  // namespace

template <typename T, int D, int KIND>
__global__ __launch_bounds__(256) void k_entmax_bwd_dq(EntmaxBwdArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) uint16_t sKt[BF ? 4 : 1][BF ? D * kTRow : 8];

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int hi32 = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y;
  const int N = a.N;
  const int L = a.varlen ? min(max(a.varlen[b], 0), N) : N;
  const int r0 = blockIdx.x * 128 + w * 32;
  if (r0 >= N) return;  // no row of this wavefront exists (no block barrier below)
  const int qi = r0 + (lane & 31);
  const bool row_ok = qi < L;
  const bool causal = a.causal != 0;
  const size_t bh = (size_t)b * a.H + h;
  const int nT = (N + 63) / 64;
  const T* Qp = static_cast<const T*>(a.Q) + bh * (size_t)N * D;
  const T* Kp = static_cast<const T*>(a.K) + bh * (size_t)N * D;
  const T* Vp = static_cast<const T*>(a.V) + bh * (size_t)N * D;
  const T* dOp = static_cast<const T*>(a.dO) + bh * (size_t)N * D;
  const float tau = row_ok ? a.tau[bh * N + qi] : 0.f;

  int last_key = L - 1;
  if (causal) last_key = min(last_key, r0 + 31);
  const int n_kb = r0 < L ? last_key / 32 + 1 : 0;
  const int I = r0 >> 6;

  Frags<BF, D> fq, fdo;
  load_frags<BF, D>(fq, Qp, qi, row_ok);
  load_frags<BF, D>(fdo, dOp, qi, row_ok);

  // t = u - tau of the lane's row against keys key0 + 8 (r/4) + 4 hi32 + r%4
  auto block_t = [&](int key0, f32x16& t, f32x16& dp) {
    Frags<BF, D> fk, fv;
    const int kr = key0 + (lane & 31);
    load_frags<BF, D>(fk, Kp, kr, kr < L);
    load_frags<BF, D>(fv, Vp, kr, kr < L);
    const f32x16 s = dot32<BF, D>(fk, fq);
    dp = dot32<BF, D>(fv, fdo);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
      const bool ok = row_ok && key < L && (!causal || key <= qi);
      t[r] = ok ? fmaf(s[r], a.scale, -tau) : -1.f;
    }
  };

  // ---- pass 1: sum g and sum g dP per row
  float sg = 0.f, sgd = 0.f;
  for (int kb = 0; kb < n_kb; ++kb) {
    if (!tile_on(a, bh, nT, I, kb >> 1)) continue;
    f32x16 t, dp;
    block_t(kb * 32, t, dp);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float g = jac_weight<KIND>(t[r], a.alpha, a.beta);
      sg += g;
      sgd = fmaf(g, dp[r], sgd);
    }
  }
  sg = sum_xor32(sg);
  sgd = sum_xor32(sgd);
  const float c = sg > 0.f ? sgd / sg : 0.f;
  if (lane < 32 && qi < N) a.coef[bh * N + qi] = row_ok ? c : 0.f;

  // ---- pass 2: dS = g (dP - c); dQ^T += K^T dS^T
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  uint16_t* kt = sKt[BF ? w : 0];
  for (int kb = 0; kb < n_kb; ++kb) {
    if (!tile_on(a, bh, nT, I, kb >> 1)) continue;
    f32x16 t, dp;
    block_t(kb * 32, t, dp);
    bool nz = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float g = jac_weight<KIND>(t[r], a.alpha, a.beta);
      t[r] = g * (dp[r] - c);
      nz = nz || g > 0.f;
    }
    if (!wave_any(nz)) continue;
    if constexpr (BF) {
      stage_t<D>(kt, reinterpret_cast<const uint16_t*>(Kp), kb * 32, L);
      wave_lds_fence();
    }
    acc_xt_w<BF, D>(acc, t, kt, reinterpret_cast<const float*>(Kp), kb * 32, L);
    if constexpr (BF) wave_lds_fence();
  }
  if (qi < N) store_line<BF, D>(a.dQ, bh * N + qi, acc, a.inv_sqrt_d);
}

template <typename T, int D, int KIND>
__global__ __launch_bounds__(256) void k_entmax_bwd_dkdv(EntmaxBwdArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) uint16_t sQt[BF ? 4 : 1][BF ? D * kTRow : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sOt[BF ? 4 : 1][BF ? D * kTRow : 8];

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int hi32 = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y;
  const int N = a.N;
  const int L = a.varlen ? min(max(a.varlen[b], 0), N) : N;
  const int k0 = blockIdx.x * 128 + w * 32;
  if (k0 >= N) return;  // no key of this wavefront exists (no block barrier below)
  const int kj = k0 + (lane & 31);
  const bool key_ok = kj < L;
  const bool causal = a.causal != 0;
  const size_t bh = (size_t)b * a.H + h;
  const int nT = (N + 63) / 64;
  const T* Qp = static_cast<const T*>(a.Q) + bh * (size_t)N * D;
  const T* Kp = static_cast<const T*>(a.K) + bh * (size_t)N * D;
  const T* Vp = static_cast<const T*>(a.V) + bh * (size_t)N * D;
  const T* dOp = static_cast<const T*>(a.dO) + bh * (size_t)N * D;
  const int J = k0 >> 6;

  // the lane's K and V rows: held for the whole loop in bf16; float32 rows
  // (twice the registers) are re-read per block from the cache instead
  Frags<BF, D> fk, fv;
  if constexpr (BF) {
    load_frags<BF, D>(fk, Kp, kj, key_ok);
    load_frags<BF, D>(fv, Vp, kj, key_ok);
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }
  uint16_t* qt = sQt[BF ? w : 0];
  uint16_t* ot = sOt[BF ? w : 0];
  const int qb0 = (causal ? k0 : 0) / 32;
  const int n_qb = k0 < L ? (L + 31) / 32 : 0;
  for (int qb = qb0; qb < n_qb; ++qb) {
    if (!tile_on(a, bh, nT, qb >> 1, J)) continue;
    const int q0 = qb * 32;
    // tau and c of the block's rows, one per lane < 32, read by the others through shuffles
    const int qm = q0 + (lane & 31);
    const float tau_m = qm < L ? a.tau[bh * N + qm] : 0.f;
    const float c_m = qm < L ? a.coef[bh * N + qm] : 0.f;
    Frags<BF, D> fq, fdo;
    if constexpr (!BF) load_frags<BF, D>(fk, Kp, kj, key_ok);
    load_frags<BF, D>(fq, Qp, qm, qm < L);
    const f32x16 s = dot32<BF, D>(fq, fk);  // S[query][key]
    if constexpr (!BF) load_frags<BF, D>(fv, Vp, kj, key_ok);
    load_frags<BF, D>(fdo, dOp, qm, qm < L);
    const f32x16 dp = dot32<BF, D>(fdo, fv);  // dP[query][key]
    f32x16 p, ds;
    bool nz = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * hi32 + (r & 3);
      const float tq = __shfl(tau_m, m);
      const float cq = __shfl(c_m, m);
      const int q = q0 + m;
      const bool ok = key_ok && q < L && (!causal || kj <= q);
      const float t = ok ? fmaf(s[r], a.scale, -tq) : -1.f;
      p[r] = prior_of<KIND>(t, a.beta);
      const float g = jac_weight<KIND>(t, a.alpha, a.beta);
      ds[r] = g * (dp[r] - cq);
      nz = nz || g > 0.f;
    }
    if (!wave_any(nz)) continue;
    if constexpr (BF) {
      stage_t<D>(qt, reinterpret_cast<const uint16_t*>(Qp), q0, L);
      stage_t<D>(ot, reinterpret_cast<const uint16_t*>(dOp), q0, L);
      wave_lds_fence();
    }
    acc_xt_w<BF, D>(dv, p, ot, reinterpret_cast<const float*>(dOp), q0, L);
    acc_xt_w<BF, D>(dk, ds, qt, reinterpret_cast<const float*>(Qp), q0, L);
    if constexpr (BF) wave_lds_fence();
  }
  if (kj < N) {
    store_line<BF, D>(a.dK, bh * N + kj, dk, a.inv_sqrt_d);
    store_line<BF, D>(a.dV, bh * N + kj, dv, 1.f);
  }
}

template <typename T, int D, int KIND>
static hipError_t entmax_bwd_tdk(const EntmaxBwdArgs& a, hipStream_t stream) {
  dim3 grid((a.N + 127) / 128, a.H, a.B);
  hipLaunchKernelGGL((k_entmax_bwd_dq<T, D, KIND>), grid, dim3(256), 0, stream, a);
  hipLaunchKernelGGL((k_entmax_bwd_dkdv<T, D, KIND>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t entmax_bwd_td(const EntmaxBwdArgs& a, hipStream_t stream) {
  if (a.alpha == 1.5f) return entmax_bwd_tdk<T, D, 2>(a, stream);
  if (a.alpha == 2.0f) return entmax_bwd_tdk<T, D, 1>(a, stream);
  return entmax_bwd_tdk<T, D, 0>(a, stream);
}

hipError_t launch_entmax_attn_bwd(const EntmaxBwdArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) return a.d == 64 ? entmax_bwd_td<uint16_t, 64>(a, stream) : entmax_bwd_td<uint16_t, 128>(a, stream);
  return a.d == 64 ? entmax_bwd_td<float, 64>(a, stream) : entmax_bwd_td<float, 128>(a, stream);
}

}  // namespace dash
