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
//   k_entmax_bwd_dq   (row pass): a wavefront owns 32 query rows. One pass over
//       the key blocks builds S^T = K Q^T and dP^T = V dO^T by MFMA (a lane owns
//       one row), sums g and g dP per row and accumulates A^T += K^T (g dP)^T and
//       G^T += K^T g^T (K staged transposed in the wavefront's LDS slot); then
//       c = sum g dP / sum g (stored for the second kernel) and
//       dQ = (A - c G) / sqrt(d).
//   k_entmax_bwd_dkdv (column pass): a wavefront owns 32 keys. Over the query
//       blocks it builds S = Q K^T and dP = dO V^T (a lane owns one key), forms
//       P and dS from tau and c, and accumulates dV^T += dO^T P and
//       dK^T += Q^T dS with Q and dO staged transposed in LDS.
// bfloat16 operands run on v_mfma_f32_32x32x16_bf16 with the weights P and dS
// split into bf16 high and low parts (float32 accuracy); float32 operands on
// v_mfma_f32_32x32x2_f32, transposed operands read straight from memory
// (32 consecutive floats per half-wavefront).
#include "bwd_common.hpp"
#include "kernels.hpp"
#include "tau_solve.hpp"

namespace dash {

namespace {
// g = max(t, 0)^((2 - alpha) beta), the entmax Jacobian's weight.
template <int KIND>
__device__ __forceinline__ float jac_weight(float t, float alpha, float beta) {
  if constexpr (KIND == 2) return fmaxf(t, 0.f);           // alpha = 1.5: exponent 1
  else if constexpr (KIND == 1) return t > 0.f ? 1.f : 0.f;  // alpha = 2: exponent 0
  else return t > 0.f ? fast_exp2((2.f - alpha) * beta * fast_log2(t)) : 0.f;
}

}  // namespace

using namespace bwd;

template <typename T, int D, int KIND>
__global__ __launch_bounds__(256) void k_entmax_bwd_dq(EntmaxBwdArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) uint16_t sKt[BF ? 4 : 1][BF ? D * kTRow : 8];

  const int lane = lane_id();
  // wave-uniform (a scalar for the compiler, so block-level tests are scalar branches)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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
  const uint32_t* bits = a.mask ? a.mask + (bh * nT + (r0 >> 6)) * a.mask_words : nullptr;
  // blocks below kb_full have every (row, key) allowed: no per-entry tests there
  const int kb_full = (r0 + 31 < L) ? (causal ? r0 / 32 : L / 32) : 0;

  Frags<BF, D> fq, fdo;
  load_frags<BF, D>(fq, Qp, qi, row_ok);
  load_frags<BF, D>(fdo, dOp, qi, row_ok);

  Frags<BF, D> fk[BF ? 2 : 1], fv[BF ? 2 : 1];
  auto load = [&](int kb, auto sl) {
    constexpr int slot = decltype(sl)::v;
    const int kr = kb * 32 + (lane & 31);
    const bool ok = kb < n_kb && kr < L;
    load_frags<BF, D>(fk[slot], Kp, kr, ok);
    load_frags<BF, D>(fv[slot], Vp, kr, ok);
  };
  // t = u - tau of the lane's row against keys kb*32 + 8 (r/4) + 4 hi32 + r%4
  // (-1 where the key is not allowed)
  auto block_t = [&](int kb, auto sl, f32x16& t, f32x16& dp) {
    constexpr int slot = decltype(sl)::v;
    const f32x16 s = dot32<BF, D>(fk[slot], fq);
    dp = dot32<BF, D>(fv[slot], fdo);
    if (kb < kb_full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = fmaf(s[r], a.scale, -tau);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
        const bool ok = row_ok && key < L && (!causal || key <= qi);
        t[r] = ok ? fmaf(s[r], a.scale, -tau) : -1.f;
      }
    }
  };

  // ---- one pass: per row sum g and sum g dP, and with K^T as the common
  // operand A^T += K^T (g dP)^T and G^T += K^T g^T; then c = sum g dP / sum g and
  // dQ = (A - c G) / sqrt(d) = sum_j g (dP - c) k_j / sqrt(d)
  f32x16 accA[D / 32], accG[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      accA[db][r] = 0.f;
      accG[db][r] = 0.f;
    }
  float sg = 0.f, sgd = 0.f;
  uint16_t* kt = sKt[BF ? w : 0];
  visit_blocks<BF>(0, n_kb, bits, load, [&](int kb, auto sl) {
    constexpr int slot = decltype(sl)::v;
    f32x16 t, dp;
    block_t(kb, sl, t, dp);
    bool nz = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float g = jac_weight<KIND>(t[r], a.alpha, a.beta);
      const float gd = g * dp[r];
      sg += g;
      sgd += gd;
      t[r] = g;
      dp[r] = gd;
      nz = nz || g > 0.f;
    }
    if (wave_any(nz)) {
      if constexpr (BF) {
        stage_t_regs<D>(kt, fk[slot]);
        wave_lds_fence();
      }
      acc_xt_w<BF, D>(accA, dp, kt, reinterpret_cast<const float*>(Kp), kb * 32, L);
      acc_xt_w<BF, D, KIND != 1>(accG, t, kt, reinterpret_cast<const float*>(Kp), kb * 32, L);
      if constexpr (BF) wave_lds_fence();
    }
  });
  sg = sum_xor32(sg);
  sgd = sum_xor32(sgd);
  const float c = sg > 0.f ? sgd / sg : 0.f;
  if (lane < 32 && qi < N) a.coef[bh * N + qi] = row_ok ? c : 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) accA[db][r] = fmaf(-c, accG[db][r], accA[db][r]);
  f32x16 (&acc)[D / 32] = accA;
  if (qi < N) store_line<BF, D>(a.dQ, bh * N + qi, acc, a.inv_sqrt_d);
}

// bf16 at head_dim 64: registers capped for two waves per SIMD (a few spill at
// alpha != 2), which hides more of the MFMA and load latency than one wave does
template <typename T, int D, int KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 && sizeof(T) == 2 ? 2 : 1)))
void k_entmax_bwd_dkdv(EntmaxBwdArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int kColWords = kEntmaxMaxTiles / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQt[BF ? 4 : 1][BF ? D * kTRow : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sOt[BF ? 4 : 1][BF ? D * kTRow : 8];
  __shared__ uint32_t sCol[4][kColWords];
  __shared__ __attribute__((aligned(16))) float sTC[4][2][32];

  const int lane = lane_id();
  // wave-uniform (a scalar for the compiler, so block-level tests are scalar branches)
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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

  // the column of the block mask for this wavefront's key tile, as bits over
  // the row tiles (read 64 row tiles per step)
  const uint32_t* bits = nullptr;
  if (a.mask) {
    uint32_t* col = sCol[w];
    for (int I0 = 0; I0 < nT; I0 += 64) {
      const int I = I0 + lane;
      const bool on = I < nT && ((a.mask[(bh * nT + I) * a.mask_words + (J >> 5)] >> (J & 31)) & 1u);
      const uint64_t bal = __ballot(on);
      if (lane == 0) {
        col[I0 >> 5] = (uint32_t)bal;
        if ((I0 >> 5) + 1 < kColWords) col[(I0 >> 5) + 1] = (uint32_t)(bal >> 32);
      }
    }
    wave_lds_fence();
    bits = col;
  }

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
  float* stau = sTC[w][0];
  float* sc = sTC[w][1];
  const int qb0 = (causal ? k0 : 0) / 32;
  const int n_qb = k0 < L ? (L + 31) / 32 : 0;
  // blocks from qb_full on have every (row, key) allowed, up to the last full one
  const bool keys_full = k0 + 31 < L;
  const int qb_full = causal ? k0 / 32 + 1 : 0;
  const int qb_last_full = L / 32;  // exclusive

  Frags<BF, D> fq[BF ? 2 : 1], fdo[BF ? 2 : 1];
  float tau_m[BF ? 2 : 1], c_m[BF ? 2 : 1];
  // rows of query block qb; tau and c of row qb*32 + lane % 32
  auto load = [&](int qb, auto sl) {
    constexpr int slot = decltype(sl)::v;
    const int qm = qb * 32 + (lane & 31);
    const bool ok = qb < n_qb && qm < L;
    load_frags<BF, D>(fq[slot], Qp, qm, ok);
    load_frags<BF, D>(fdo[slot], dOp, qm, ok);
    tau_m[slot] = ok ? a.tau[bh * N + qm] : 0.f;
    c_m[slot] = ok ? a.coef[bh * N + qm] : 0.f;
  };
  visit_blocks<BF>(qb0, n_qb, bits, load, [&](int qb, auto sl) {
    constexpr int slot = decltype(sl)::v;
    const int q0 = qb * 32;
    if constexpr (!BF) load_frags<BF, D>(fk, Kp, kj, key_ok);
    const f32x16 s = dot32<BF, D>(fq[slot], fk);  // S[query][key]
    if constexpr (!BF) load_frags<BF, D>(fv, Vp, kj, key_ok);
    const f32x16 dp = dot32<BF, D>(fdo[slot], fv);  // dP[query][key]
    // tau and c of the block's rows through the wavefront's LDS slot: register r
    // of this lane holds row 8 (r/4) + 4 hi32 + r%4
    if (lane < 32) {
      stau[lane] = tau_m[slot];
      sc[lane] = c_m[slot];
    }
    wave_lds_fence();
    f32x4 tq[4], cq[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      tq[g4] = *reinterpret_cast<const f32x4*>(stau + 8 * g4 + 4 * hi32);
      cq[g4] = *reinterpret_cast<const f32x4*>(sc + 8 * g4 + 4 * hi32);
    }
    f32x16 p, ds;
    bool nz = false;
    const bool full = keys_full && qb >= qb_full && qb < qb_last_full;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float tr = tq[r >> 2][r & 3];
      float t;
      if (full) {
        t = fmaf(s[r], a.scale, -tr);
      } else {
        const int q = q0 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
        const bool ok = key_ok && q < L && (!causal || kj <= q);
        t = ok ? fmaf(s[r], a.scale, -tr) : -1.f;
      }
      p[r] = prior_of<KIND>(t, a.beta);
      const float g = jac_weight<KIND>(t, a.alpha, a.beta);
      ds[r] = g * (dp[r] - cq[r >> 2][r & 3]);
      nz = nz || g > 0.f;
    }
    if (wave_any(nz)) {
      if constexpr (BF) {
        stage_t_regs<D>(qt, fq[slot]);
        stage_t_regs<D>(ot, fdo[slot]);
        wave_lds_fence();
      }
      acc_xt_w<BF, D>(dv, p, ot, reinterpret_cast<const float*>(dOp), q0, L);
      acc_xt_w<BF, D>(dk, ds, qt, reinterpret_cast<const float*>(Qp), q0, L);
    }
    // the next block overwrites the LDS slots only after every lane has read them
    wave_lds_fence();
  });
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
