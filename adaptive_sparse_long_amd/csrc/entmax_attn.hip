// entmax_attn.hip -- dense alpha-entmax attention with block skipping (the
// AdaSplash README page: "Usage", "AdaSplash with Block Masking", and "Key
// Features": varlen, alpha, causal masking):
//   s_ij = <q_i, k_j> / sqrt(d),  u = (alpha - 1) s,
//   P_ij = max(u_ij - tau_i, 0)^(1/(alpha-1)) with sum_j P_ij = 1,  O = P V,
// plus one bit per 64 x 64 tile that holds a non-zero weight.
//
// Each wavefront owns 32 query rows; S^T = K Q^T comes from MFMA (bf16:
// v_mfma_f32_32x32x16_bf16; float32: v_mfma_f32_32x32x2_f32) so every lane owns
// one query row and row reductions are one permlane32 swap. Three passes over
// the key tiles of the row block:
//   1. scores and row maxima. Since every weight is at most 1, tau >= max u - 1,
//      so a tile whose row maxima are all <= (running max) - 1 can never hold
//      support; the others are marked in a per-wavefront candidate bitmask
//      (a superset of the true support tiles, because the running max only
//      grows);
//   2. tau by safeguarded Halley + bisection steps ("Triton Entmax"), each step
//      recomputing scores of the candidate tiles only and dropping tiles whose
//      row maxima fall below the bracket's lower end;
//   3. output over candidate tiles: tiles with no positive weight are skipped
//      and leave their mask bit 0; the others accumulate O^T += V^T P^T with V
//      staged transposed in a per-wavefront LDS slot and P split into bf16 high
//      and low parts (float32 accuracy at bf16 MFMA rate).
// Rows at or past varlen[b] get O = 0 and tau = 0.
#include "kernels.hpp"
#include "tau_solve.hpp"

namespace dash {

namespace {
constexpr int kMaxMaskWords = kEntmaxMaxTiles / 32;
constexpr int VPAD = 4;

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

__device__ __forceinline__ size_t bh_of(const EntmaxAttnArgs& a, int b, int h) { return (size_t)b * a.H + h; }

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
  static constexpr bool bf16 = true;
};
template <>
struct Elem<float> {
  static constexpr bool bf16 = false;
};
}  // namespace

// KEEP > 0 (N <= 64 KEEP): the scores of a wavefront's KEEP key tiles stay in
// registers from pass 1 on, instead of being recomputed in every tau step and
// in the output pass (short rows, where the recomputation is most of the time).
template <typename T, int D, int KIND, int KEEP>
__global__ __launch_bounds__(256) void k_entmax_attn(EntmaxAttnArgs a) {
  constexpr bool BF = Elem<T>::bf16;
  constexpr int NS = BF ? D / 16 : D / 2;  // k-steps of S^T = K Q^T
  constexpr int NDB = D / 32;
  constexpr int VROW = 64 + VPAD;
  __shared__ uint32_t s_cand[4][kMaxMaskWords];
  __shared__ uint32_t s_mask[2][kMaxMaskWords];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[BF ? 4 : 1][BF ? D * VROW : 8];

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int hi32 = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y;
  const int N = a.N;
  const int L = a.varlen ? min(max(a.varlen[b], 0), N) : N;
  const int r0 = blockIdx.x * 128 + w * 32;
  const int qi = r0 + (lane & 31);
  const bool row_ok = qi < L;
  const bool causal = a.causal != 0;
  const size_t bh = (size_t)b * a.H + h;
  const T* Qp = static_cast<const T*>(a.Q) + bh * (size_t)N * D;
  const T* Kp = static_cast<const T*>(a.K) + bh * (size_t)N * D;
  const T* Vp = static_cast<const T*>(a.V) + bh * (size_t)N * D;
  const int nT = (N + 63) / 64;

  if (a.only_marked) {
    // redo this row block only if the single-pass kernel left it (tau = NaN)
    const int row = blockIdx.x * 128 + (int)threadIdx.x;
    const bool marked = threadIdx.x < 128 && row < N && isnan(a.tau[bh_of(a, b, h) * (size_t)N + row]);
    if (!__syncthreads_or(marked)) return;
  }
  for (int i = threadIdx.x; i < 4 * kMaxMaskWords; i += blockDim.x) (&s_cand[0][0])[i] = 0u;
  for (int i = threadIdx.x; i < 2 * kMaxMaskWords; i += blockDim.x) (&s_mask[0][0])[i] = 0u;
  __syncthreads();

  // key tiles this wavefront can see
  int last_key = L - 1;
  if (causal) last_key = min(last_key, r0 + 31);
  const int n_kt = (r0 < L) ? last_key / 64 + 1 : 0;
  const int n_valid = causal ? min(qi + 1, L) : L;

  // Q^T as B operand
  bf16x8 qb[BF ? NS : 1];
  float qf[BF ? 1 : NS];
  if constexpr (BF) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(Qp) + (size_t)qi * D + 8 * hi32;
#pragma unroll
    for (int s = 0; s < NS; ++s) qb[s] = as_bf16x8(row_ok ? ldg16(qp + 16 * s) : u32x4{0, 0, 0, 0});
  } else {
    const float* qp = reinterpret_cast<const float*>(Qp) + (size_t)qi * D + hi32;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = row_ok ? qp[2 * s] : 0.f;
  }

  // u of key tile J: lane's query qi; keys J*64 + 32 kb + 8 (r/4) + 4 hi32 + r%4
  auto tile_u = [&](int J, f32x16& u0, f32x16& u1) {
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    const int key0 = J * 64 + (lane & 31);
    const int key1 = key0 + 32;
    if constexpr (BF) {
      const uint16_t* k0 = reinterpret_cast<const uint16_t*>(Kp) + (size_t)key0 * D + 8 * hi32;
      const uint16_t* k1 = reinterpret_cast<const uint16_t*>(Kp) + (size_t)key1 * D + 8 * hi32;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8 a0 = as_bf16x8(key0 < L ? ldg16(k0 + 16 * s) : u32x4{0, 0, 0, 0});
        bf16x8 a1 = as_bf16x8(key1 < L ? ldg16(k1 + 16 * s) : u32x4{0, 0, 0, 0});
        s0 = mfma32x32x16(a0, qb[s], s0);
        s1 = mfma32x32x16(a1, qb[s], s1);
      }
    } else {
      const float* k0 = reinterpret_cast<const float*>(Kp) + (size_t)key0 * D + hi32;
      const float* k1 = reinterpret_cast<const float*>(Kp) + (size_t)key1 * D + hi32;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float a0 = key0 < L ? k0[2 * s] : 0.f;
        const float a1 = key1 < L ? k1[2 * s] : 0.f;
        s0 = mfma32x32x2f32(a0, qf[s], s0);
        s1 = mfma32x32x2f32(a1, qf[s], s1);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = J * 64 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
      float x0 = s0[r] * a.scale, x1 = s1[r] * a.scale;
      const bool v0 = row_ok && kk < L && (!causal || kk <= qi);
      const bool v1 = row_ok && kk + 32 < L && (!causal || kk + 32 <= qi);
      u0[r] = v0 ? x0 : -INFINITY;
      u1[r] = v1 ? x1 : -INFINITY;
    }
  };
  auto tile_max = [&](const f32x16& u0, const f32x16& u1) {
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, fmaxf(u0[r], u1[r]));
    return max_xor32(m);
  };
  uint32_t* cand = s_cand[w];
  // fn(J) for the wavefront's key tiles in order (unrolled when the scores are kept)
  auto for_tiles = [&](auto&& fn) {
    if constexpr (KEEP > 0) {
#pragma unroll
      for (int J = 0; J < KEEP; ++J)
        if (J < n_kt) fn(J);
    } else {
      for (int J = 0; J < n_kt; ++J) fn(J);
    }
  };
  f32x16 uk0[KEEP > 0 ? KEEP : 1], uk1[KEEP > 0 ? KEEP : 1];
  auto get_u = [&](int J, f32x16& u0, f32x16& u1) {
    if constexpr (KEEP > 0) {
      u0 = uk0[J];
      u1 = uk1[J];
    } else {
      tile_u(J, u0, u1);
    }
  };

  // ---- pass 1: row maxima and candidate tiles
  float m_run = -INFINITY;
  for_tiles([&](int J) {
    f32x16 u0, u1;
    tile_u(J, u0, u1);
    if constexpr (KEEP > 0) {
      uk0[J] = u0;
      uk1[J] = u1;
    }
    const float mt = tile_max(u0, u1);
    m_run = fmaxf(m_run, mt);
    if (wave_any(row_ok && mt > m_run - 1.f) && lane == 0) cand[J >> 5] |= 1u << (J & 31);
  });
  wave_lds_fence();

  // ---- pass 2: tau
  float tau = 0.f;
  if (n_kt > 0) {
    float lo = m_run - 1.f;
    float hi = row_ok ? tau_upper(m_run, n_valid, a.alpha) : lo;
    tau = lo;
    for (int it = 0; it < a.n_iter; ++it) {
      float f0 = 0.f, f1 = 0.f, f2 = 0.f;
      for_tiles([&](int J) {
        if (!((cand[J >> 5] >> (J & 31)) & 1u)) return;
        f32x16 u0, u1;
        get_u(J, u0, u1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          tau_terms<KIND>(u0[r], tau, a.beta, f0, f1, f2);
          tau_terms<KIND>(u1[r], tau, a.beta, f0, f1, f2);
        }
        const float mt = tile_max(u0, u1);
        if (!wave_any(row_ok && mt > lo) && lane == 0) cand[J >> 5] &= ~(1u << (J & 31));
      });
      wave_lds_fence();
      f0 = sum_xor32(f0);
      f1 = sum_xor32(f1);
      if (KIND != 1) f2 = sum_xor32(f2);
      float nt = tau;
      if (row_ok) nt = tau_step<KIND>(tau, f0, f1, f2, a.beta, lo, hi);
      const bool conv = tau_converged(tau, nt);
      tau = nt;
      if (wave_all(conv)) break;
    }
  }

  // ---- pass 3: output over candidate tiles with a non-zero weight
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float psum = 0.f;
  uint32_t* mrow = s_mask[w >> 1];
  for_tiles([&](int J) {
    if (!((cand[J >> 5] >> (J & 31)) & 1u)) return;
    f32x16 u0, u1;
    get_u(J, u0, u1);
    bool nz = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      u0[r] = prior_of<KIND>(u0[r] - tau, a.beta);
      u1[r] = prior_of<KIND>(u1[r] - tau, a.beta);
      nz = nz || u0[r] > 0.f || u1[r] > 0.f;
      psum += u0[r] + u1[r];
    }
    if (!wave_any(nz)) return;
    if (lane == 0) atomicOr(&mrow[J >> 5], 1u << (J & 31));
    if constexpr (BF) {
      // stage V tile transposed: combos (kg, dg) = keys 4 kg .. +3, dims 8 dg .. +7
      uint16_t* vt = sVt[w];
      const uint16_t* vbase = reinterpret_cast<const uint16_t*>(Vp) + (size_t)J * 64 * D;
      constexpr int NCOMBO = 16 * (D / 8);
#pragma unroll
      for (int pass = 0; pass < NCOMBO / 64; ++pass) {
        const int combo = pass * 64 + lane;
        const int kg = combo & 15, dg = combo >> 4;
        u32x4 vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = J * 64 + 4 * kg + r;
          vr[r] = key < L ? ldg16(vbase + (size_t)(4 * kg + r) * D + 8 * dg) : u32x4{0, 0, 0, 0};
        }
        uint16_t* dst = vt + (8 * dg) * VROW + 4 * kg;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x2 lo2 = {perm_lo(vr[0][e], vr[1][e]), perm_lo(vr[2][e], vr[3][e])};
          u32x2 hi2 = {perm_hi(vr[0][e], vr[1][e]), perm_hi(vr[2][e], vr[3][e])};
          *reinterpret_cast<u32x2*>(dst + (2 * e) * VROW) = lo2;
          *reinterpret_cast<u32x2*>(dst + (2 * e + 1) * VROW) = hi2;
        }
      }
      wave_lds_fence();
      // P^T as B operands, split into bf16 high and low parts
      bf16x8 ph[4], pl[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 h0, h1, l0, l1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = u0[8 * hh + 2 * e], a1 = u0[8 * hh + 2 * e + 1];
          const float b0 = u1[8 * hh + 2 * e], b1 = u1[8 * hh + 2 * e + 1];
          const float ra0 = round_bf16(a0), ra1 = round_bf16(a1);
          const float rb0 = round_bf16(b0), rb1 = round_bf16(b1);
          h0[e] = pack_bf16x2(ra0, ra1);
          l0[e] = pack_bf16x2(a0 - ra0, a1 - ra1);
          h1[e] = pack_bf16x2(rb0, rb1);
          l1[e] = pack_bf16x2(b0 - rb0, b1 - rb1);
        }
        ph[hh] = as_bf16x8(h0);
        pl[hh] = as_bf16x8(l0);
        ph[2 + hh] = as_bf16x8(h1);
        pl[2 + hh] = as_bf16x8(l1);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vrow = vt + (32 * db + (lane & 31)) * VROW + 4 * hi32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int k0 = (ks >> 1) * 32 + (ks & 1) * 16;
          u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + k0);
          u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + k0 + 8);
          const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
          o[db] = mfma32x32x16(va, ph[ks], o[db]);
          o[db] = mfma32x32x16(va, pl[ks], o[db]);
        }
      }
      wave_lds_fence();
    } else {
      const float* vbase = reinterpret_cast<const float*>(Vp) + (size_t)J * 64 * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const int kk = 8 * (s >> 2) + 4 * hi32 + (s & 3);
          const float v0 = J * 64 + kk < L ? vbase[(size_t)kk * D + 32 * db + (lane & 31)] : 0.f;
          const float v1 = J * 64 + 32 + kk < L ? vbase[(size_t)(kk + 32) * D + 32 * db + (lane & 31)] : 0.f;
          o[db] = mfma32x32x2f32(v0, u0[s], o[db]);
          o[db] = mfma32x32x2f32(v1, u1[s], o[db]);
        }
      }
    }
  });

  // ---- outputs
  psum = sum_xor32(psum);
  if (qi < N) {
    const float inv = (row_ok && psum > 0.f) ? 1.f / psum : 0.f;
    if (lane < 32) a.tau[bh * (size_t)N + qi] = row_ok ? tau : 0.f;
    if constexpr (BF) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.O) + (bh * N + qi) * (size_t)D + 4 * hi32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 v = {pack_bf16x2(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv),
                     pack_bf16x2(o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + 32 * db + 8 * q4) = v;
        }
    } else {
      float* op = reinterpret_cast<float*>(a.O) + (bh * N + qi) * (size_t)D + 4 * hi32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v = {o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                     o[db][4 * q4 + 3] * inv};
          *reinterpret_cast<f32x4*>(op + 32 * db + 8 * q4) = v;
        }
    }
  }
  __syncthreads();
  if (a.mask) {
    for (int i = threadIdx.x; i < 2 * a.mask_words; i += blockDim.x) {
      const int ii = i / a.mask_words, wd = i % a.mask_words;
      const int I = blockIdx.x * 2 + ii;
      if (I < nT) a.mask[(bh * nT + I) * a.mask_words + wd] = s_mask[ii][wd];
    }
  }
}

// ---------------------------------------------------------------------------
// Single-pass kernel (bf16). Four wavefronts x 32 rows per workgroup share each
// 64-key K tile, staged once in a double-buffered LDS ring. A lane keeps, in its
// own LDS list, the scores of its row that lie above the row's running max - 1
// (the only ones that can carry weight, since tau >= max u - 1), pruning the
// list whenever the max grows. After the pass, tau is solved over the row's
// two lists (lanes l and l ^ 32) and the output gathers the V rows of the
// support directly: O_i = sum_j P_ij v_j / sum_j P_ij. A wavefront with a list
// past kEntmaxCap writes tau = NaN for its rows and leaves its row block to
// the general kernel, launched after this one.
// ---------------------------------------------------------------------------
template <int D, int KIND>
__global__ __launch_bounds__(256, 2) void k_entmax_buf(EntmaxAttnArgs a) {
  constexpr int NS = D / 16;
  constexpr int KROW = D + 8;
  constexpr int CAP = kEntmaxCap;
  constexpr int NLD = D / 32;  // 16-byte K loads per thread and tile
  constexpr int HD = D / 2;    // output dims per lane
  // one K tile in LDS (D = 64: four workgroups per CU; two buffers would leave three)
  constexpr int KBUF = D == 64 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t sK[KBUF][64 * KROW];
  __shared__ float s_cu[4][CAP][kWave];     // candidate raw scores: [wavefront][entry][lane]
  __shared__ uint16_t s_ck[4][CAP][kWave];  // their keys
  __shared__ uint32_t s_mask[2][kMaxMaskWords];

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int tid = threadIdx.x;
  const int hi32 = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y;
  const int N = a.N;
  const int L = a.varlen ? min(max(a.varlen[b], 0), N) : N;
  const int r0 = blockIdx.x * 128 + w * 32;
  const int qi = r0 + (lane & 31);
  const bool row_ok = qi < L;
  const bool causal = a.causal != 0;
  const size_t bh = (size_t)b * a.H + h;
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + bh * (size_t)N * D;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + bh * (size_t)N * D;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + bh * (size_t)N * D;
  const int nT = (N + 63) / 64;

  for (int i = tid; i < 2 * kMaxMaskWords; i += blockDim.x) (&s_mask[0][0])[i] = 0u;

  // key tiles of the workgroup (uniform) and of this wavefront
  const int wg_r0 = blockIdx.x * 128;
  const int n_kt_wg = wg_r0 < L ? (causal ? min(L - 1, wg_r0 + 127) : L - 1) / 64 + 1 : 0;
  const int n_kt = r0 < L ? (causal ? min(L - 1, r0 + 31) : L - 1) / 64 + 1 : 0;

  // Q^T as the B operand: column qi, dims 16 s + 8 hi32 .. +7
  bf16x8 qb[NS];
  {
    const uint16_t* qp = Qp + (size_t)qi * D + 8 * hi32;
#pragma unroll
    for (int s = 0; s < NS; ++s) qb[s] = as_bf16x8(row_ok ? ldg16(qp + 16 * s) : u32x4{0, 0, 0, 0});
  }

  // K tiles in flight: registers of NP tiles ahead of the one being computed
  constexpr int NP = 2;
  u32x4 kr[NP][NLD];
  auto load_tile = [&](int J, u32x4 (&dst)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + 256 * i;
      const int key = J * 64 + idx / (D / 8);
      dst[i] = key < L ? ldg16(Kp + (size_t)key * D + (idx % (D / 8)) * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&src)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&sK[buf][(idx / (D / 8)) * KROW + (idx % (D / 8)) * 8]) = src[i];
    }
  };

  // ---- the pass over the key tiles, in raw score units s (u = scale * s,
  // scale > 0): a candidate has s > max s - 1 / scale
  const float inv_scale = 1.f / a.scale;
  const bool rows_full = r0 + 31 < L;  // every row of the wavefront is valid
  float m_run = -INFINITY;
  int cnt = 0;  // candidates of this lane (past CAP: overflow)
  auto process = [&](int J, int buf) {
    // S^T = K Q^T: lane's query qi, keys J*64 + 32 kb + 8 (r/4) + 4 hi32 + r%4
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    const uint16_t* ka = &sK[buf][(lane & 31) * KROW + 8 * hi32];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      s0 = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ka + 16 * s), qb[s], s0);
      s1 = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ka + 32 * KROW + 16 * s), qb[s], s1);
    }
    // masks only where the tile reaches the sequence end or the causal diagonal
    if (!(rows_full && J * 64 + 63 < L && (!causal || J * 64 + 63 <= r0))) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = J * 64 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
        const bool v0 = row_ok && kk < L && (!causal || kk <= qi);
        const bool v1 = row_ok && kk + 32 < L && (!causal || kk + 32 <= qi);
        s0[r] = v0 ? s0[r] : -INFINITY;
        s1[r] = v1 ? s1[r] : -INFINITY;
      }
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) lmax = fmaxf(lmax, fmaxf(s0[r], s1[r]));
    const float tmax = max_xor32(lmax);
    // the row's max only grows; entries that fall below max - 1 / scale stay
    // in the list (they carry no weight) until the list needs their room
    m_run = fmaxf(m_run, tmax);
    const float thr = m_run - inv_scale;
    if (lmax > thr) {
      int nn = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) nn += (s0[r] > thr ? 1 : 0) + (s1[r] > thr ? 1 : 0);
      if (cnt + nn > CAP && cnt <= CAP) {
        int k2 = 0;
        for (int e = 0; e < cnt; ++e) {
          const float v = s_cu[w][e][lane];
          if (v > thr) {
            s_cu[w][k2][lane] = v;
            s_ck[w][k2][lane] = s_ck[w][e][lane];
            ++k2;
          }
        }
        cnt = k2;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = J * 64 + 8 * (r >> 2) + 4 * hi32 + (r & 3);
        if (s0[r] > thr) {
          if (cnt < CAP) {
            s_cu[w][cnt][lane] = s0[r];
            s_ck[w][cnt][lane] = (uint16_t)kk;
          }
          ++cnt;
        }
        if (s1[r] > thr) {
          if (cnt < CAP) {
            s_cu[w][cnt][lane] = s1[r];
            s_ck[w][cnt][lane] = (uint16_t)(kk + 32);
          }
          ++cnt;
        }
      }
    }
  };
#pragma unroll
  for (int p = 0; p < NP; ++p)
    if (p < n_kt_wg) load_tile(p, kr[p]);
  if (n_kt_wg > 0) store_tile(0, kr[0]);
  __syncthreads();
  for (int J0 = 0; J0 < n_kt_wg; J0 += NP) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int J = J0 + q;
      if (J < n_kt_wg) {
        if (J + NP < n_kt_wg) load_tile(J + NP, kr[q]);  // kr[q] (tile J) is already in LDS
        if (J < n_kt) process(J, J % KBUF);
        if (KBUF == 1) __syncthreads();  // the tile is read before the next one lands
        if (J + 1 < n_kt_wg) store_tile((J + 1) % KBUF, kr[(q + 1) % NP]);
        __syncthreads();
      }
    }
  }

  if (wave_any(cnt > CAP)) {
    // leave the row block to the general kernel
    if (lane < 32 && qi < N) a.tau[bh * (size_t)N + qi] = __builtin_nanf("");
  } else {
    // ---- tau over the row's candidates: this lane's list and its partner's
    const int pl = lane ^ 32;
    const int cnt_p = __shfl_xor(cnt, 32);
    float tau = 0.f;
    const float mu = a.scale * m_run;  // max u of the row
    if (wave_any(row_ok)) {
      float lo = mu - 1.f;
      float hi = row_ok ? tau_upper(mu, max(1, cnt + cnt_p), a.alpha) : lo;
      tau = lo;
      float cu[CAP];  // this lane's list in u units
#pragma unroll
      for (int e = 0; e < CAP; ++e) cu[e] = e < cnt ? a.scale * s_cu[w][e][lane] : -INFINITY;
      for (int it = 0; it < a.n_iter; ++it) {
        float f0 = 0.f, f1 = 0.f, f2 = 0.f;
#pragma unroll
        for (int e = 0; e < CAP; ++e) tau_terms<KIND>(cu[e], tau, a.beta, f0, f1, f2);
        f0 = sum_xor32(f0);
        f1 = sum_xor32(f1);
        if (KIND != 1) f2 = sum_xor32(f2);
        float nt = tau;
        if (row_ok) nt = tau_step<KIND>(tau, f0, f1, f2, a.beta, lo, hi);
        const bool conv = !row_ok || tau_converged(tau, nt);
        tau = nt;
        if (wave_all(conv)) break;
      }
    }
    // ---- output: O_i = sum_j P_ij v_j / sum_j P_ij over both lists; this lane
    // accumulates dims hi32 * D/2 .. +D/2
    float acc[HD];
#pragma unroll
    for (int j = 0; j < HD; ++j) acc[j] = 0.f;
    float psum = 0.f;
    const int tile_row = (qi >> 6) - 2 * blockIdx.x;  // 0 or 1: this row's 64-row tile in the workgroup
    for (int side = 0; side < 2; ++side) {
      const int src = side == 0 ? lane : pl;
      const int n = side == 0 ? cnt : cnt_p;
      for (int e = 0; e < n; ++e) {
        const float p = row_ok ? prior_of<KIND>(a.scale * s_cu[w][e][src] - tau, a.beta) : 0.f;
        if (p > 0.f) {
          const int key = s_ck[w][e][src];
          psum += p;
          if (side == 0) atomicOr(&s_mask[tile_row][(key >> 6) >> 5], 1u << ((key >> 6) & 31));
          const uint16_t* vp = Vp + (size_t)key * D + hi32 * HD;
#pragma unroll
          for (int c = 0; c < HD / 8; ++c) {
            const u32x4 v = ldg16(vp + 8 * c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[8 * c + 2 * q] = fmaf(p, bf16lo(v[q]), acc[8 * c + 2 * q]);
              acc[8 * c + 2 * q + 1] = fmaf(p, bf16hi(v[q]), acc[8 * c + 2 * q + 1]);
            }
          }
        }
      }
    }
    if (qi < N) {
      const float inv = psum > 0.f ? 1.f / psum : 0.f;
      if (lane < 32) a.tau[bh * (size_t)N + qi] = row_ok ? tau : 0.f;
      uint16_t* op = static_cast<uint16_t*>(a.O) + (bh * N + qi) * (size_t)D + hi32 * HD;
#pragma unroll
      for (int c = 0; c < HD / 8; ++c) {
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(acc[8 * c + 2 * q] * inv, acc[8 * c + 2 * q + 1] * inv);
        *reinterpret_cast<u32x4*>(op + 8 * c) = v;
      }
    }
  }
  __syncthreads();
  if (a.mask) {
    for (int i = tid; i < 2 * a.mask_words; i += blockDim.x) {
      const int ii = i / a.mask_words, wd = i % a.mask_words;
      const int I = blockIdx.x * 2 + ii;
      if (I < nT) a.mask[(bh * nT + I) * a.mask_words + wd] = s_mask[ii][wd];
    }
  }
}

template <typename T, int D>
static hipError_t entmax_td(const EntmaxAttnArgs& a0, hipStream_t stream) {
  dim3 grid((a0.N + 127) / 128, a0.H, a0.B);
  EntmaxAttnArgs a = a0;
  a.only_marked = 0;
  if constexpr (Elem<T>::bf16) {
    // single pass, then the general kernel for the row blocks it left
    if (a.alpha == 1.5f)
      hipLaunchKernelGGL((k_entmax_buf<D, 2>), grid, dim3(256), 0, stream, a);
    else if (a.alpha == 2.0f)
      hipLaunchKernelGGL((k_entmax_buf<D, 1>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_entmax_buf<D, 0>), grid, dim3(256), 0, stream, a);
    a.only_marked = 1;
  }
  // rows of at most 128 keys keep their scores in registers
  if (a.N <= 128) {
    if (a.alpha == 1.5f)
      hipLaunchKernelGGL((k_entmax_attn<T, D, 2, 2>), grid, dim3(256), 0, stream, a);
    else if (a.alpha == 2.0f)
      hipLaunchKernelGGL((k_entmax_attn<T, D, 1, 2>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_entmax_attn<T, D, 0, 2>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (a.alpha == 1.5f)
    hipLaunchKernelGGL((k_entmax_attn<T, D, 2, 0>), grid, dim3(256), 0, stream, a);
  else if (a.alpha == 2.0f)
    hipLaunchKernelGGL((k_entmax_attn<T, D, 1, 0>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_entmax_attn<T, D, 0, 0>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_entmax_attn(const EntmaxAttnArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) return a.d == 64 ? entmax_td<uint16_t, 64>(a, stream) : entmax_td<uint16_t, 128>(a, stream);
  return a.d == 64 ? entmax_td<float, 64>(a, stream) : entmax_td<float, 128>(a, stream);
}

}  // namespace dash
