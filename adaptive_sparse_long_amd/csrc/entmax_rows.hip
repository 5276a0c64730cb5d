// entmax_rows.hip -- row-wise alpha-entmax, the activation the AdaSplash README
// ("Usage", "Triton Entmax (Optimized Entmax Activation)") applies over the
// last dimension of a 2-D tensor with its alpha and n_iter arguments, the
// threshold found by Halley's method plus bisection. For every row x of n:
//   u = (alpha - 1) x,  p_j = max(u_j - tau, 0)^(1/(alpha - 1)),  sum_j p_j = 1.
//
// The row stays in registers for the whole solve, so it is read from HBM once
// and written once: one wavefront per row up to 2048 entries (four wavefronts
// per workgroup, no barrier), one 1024-thread workgroup per row up to 32768.
// The grid walks the rows (a few workgroups per CU), each wavefront or
// workgroup loading its next row while it solves the current one. Entry
// j * STRIDE + t of the row belongs to thread t, so every load and store
// instruction of a wavefront covers 64 consecutive entries.
// Only entries above max u - 1 can be in the support (tau >= max u - 1); a
// wavefront row of more than 256 entries first compacts them into an LDS list
// and iterates over that when it holds at most 256. Each Halley step is one
// pass over the entries and one reduction of (f, f', f''): DPP and permlane
// swaps within the wavefront, then, for the workgroup variant, the 16
// wavefront sums through LDS in a fixed order (so every thread holds the same
// sums and takes the same step). The outputs are divided by their sum, so
// they sum to one up to rounding also when n_iter ends the solve before it
// converges.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"
#include "tau_solve.hpp"

namespace dash {

namespace {

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = __builtin_bit_cast(uint16_t, (__bf16)v); }

}  // namespace

// WAVES = 4: a row per wavefront; WAVES = 16: a row per workgroup. VPL entries
// per thread (n <= VPL * 64, resp. VPL * 1024).
template <typename T, int VPL, int KIND, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_entmax_rows(EntmaxRowsArgs a) {
  constexpr bool WG = WAVES == 16;
  constexpr int STRIDE = WG ? WAVES * kWave : kWave;
  __shared__ float s_red[2][3][WAVES];  // wavefront sums, two parities
  __shared__ float s_max[WAVES];
  constexpr int NCAND = 4 * kWave;  // compacted candidates per wavefront row
  __shared__ float s_cand[WG ? 1 : WAVES][WG ? 1 : NCAND];

  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int n = a.n;
  const int t = WG ? (int)threadIdx.x : lane;
  const float am1 = a.alpha - 1.f;
  // rows of this wavefront (workgroup): a grid-stride walk; the next row's
  // entries are loaded while the current one is solved
  const long long step = WG ? (long long)gridDim.x : (long long)gridDim.x * WAVES;
  long long row = WG ? (long long)blockIdx.x : (long long)blockIdx.x * WAVES + w;
  float xn[VPL];
  auto load_row = [&](long long r) {
    const T* x = static_cast<const T*>(a.X) + r * (long long)n;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = j * STRIDE + t;
      xn[j] = e < n ? load_elem(x + e) : -INFINITY;
    }
  };
  if (row < a.rows) load_row(row);
  for (; row < a.rows; row += step) {  // uniform over the row's threads
    T* y = static_cast<T*>(a.Y) + row * (long long)n;
    float u[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) u[j] = am1 * xn[j];
    if (row + step < a.rows) load_row(row + step);

    int par = 0;
    // (f0, f1, f2) summed over the row, the same in every thread of the row
    auto row_sum3 = [&](float& f0, float& f1, float& f2) {
      f0 = wave_sum(f0);
      f1 = wave_sum(f1);
      f2 = wave_sum(f2);
      if constexpr (WG) {
        if (lane == 0) {
          s_red[par][0][w] = f0;
          s_red[par][1][w] = f1;
          s_red[par][2][w] = f2;
        }
        __syncthreads();  // also orders the reads of this parity two reductions back
        f0 = f1 = f2 = 0.f;
#pragma unroll
        for (int k = 0; k < WAVES; ++k) {
          f0 += s_red[par][0][k];
          f1 += s_red[par][1][k];
          f2 += s_red[par][2][k];
        }
        par ^= 1;
      }
    };

    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < VPL; ++j) mx = fmaxf(mx, u[j]);
    mx = wave_max(mx);
    if constexpr (WG) {
      if (lane == 0) s_max[w] = mx;
      __syncthreads();
      mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < WAVES; ++k) mx = fmaxf(mx, s_max[k]);
    }

    // ---- tau on the bracket [max u - 1, max u - n^-(alpha-1)]. Since tau >=
    // max u - 1, only entries above max u - 1 add to the sums: a wavefront row
    // compacts them into an LDS list (lanes in order, per register a ballot)
    // and iterates over at most four per lane; a row with more keeps them all.
    float tau = INFINITY;  // a row without a finite entry
    if (mx > -INFINITY) {
      float lo = mx - 1.f;
      float hi = tau_upper(mx, n, a.alpha);
      float tt = lo;
      auto solve = [&](const float* v, auto nv) {
        for (int it = 0; it < a.n_iter; ++it) {
          float f0 = 0.f, f1 = 0.f, f2 = 0.f;
#pragma unroll
          for (int j = 0; j < decltype(nv)::value; ++j) tau_terms<KIND>(v[j], tt, a.beta, f0, f1, f2);
          row_sum3(f0, f1, f2);
          const float nt = tau_step<KIND>(tt, f0, f1, f2, a.beta, lo, hi);
          const bool conv = tau_converged(tt, nt);
          tt = nt;
          if (conv) break;  // the same decision in every thread of the row
        }
      };
      bool done = false;
      if constexpr (!WG) {
        if (VPL > 4) {
          int cnt = 0;
#pragma unroll
          for (int j = 0; j < VPL; ++j) {
            const bool c = u[j] > lo;
            const uint64_t bm = __ballot(c);
            const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
            if (c && pos < NCAND) s_cand[w][pos] = u[j];
            cnt += __popcll(bm);
          }
          if (cnt <= NCAND) {
            wave_lds_fence();
            float cu[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) cu[k] = k * kWave + lane < cnt ? s_cand[w][k * kWave + lane] : -INFINITY;
            if (cnt <= kWave) solve(cu, std::integral_constant<int, 1>{});
            else solve(cu, std::integral_constant<int, 4>{});
            done = true;
          }
        }
      }
      if (!done) solve(u, std::integral_constant<int, VPL>{});
      tau = tt;
    }

    // ---- p = max(u - tau, 0)^beta, divided by its sum
    float ps = 0.f, dummy1 = 0.f, dummy2 = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      u[j] = prior_of<KIND>(u[j] - tau, a.beta);
      ps += u[j];
    }
    row_sum3(ps, dummy1, dummy2);
    const float inv = ps > 0.f ? 1.f / ps : 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = j * STRIDE + t;
      if (e < n) store_elem(y + e, u[j] * inv);
    }
    if (a.tau != nullptr && t == 0) a.tau[row] = tau;
  }
}

// Backward: dX = g * dY - g * (g . dY) / sum(g), g = Y^(2 - alpha) on the
// support (Y > 0) and 0 off it: the vector-Jacobian product of the row's
// entmax, from its output alone. One pass: the row's Y and dY in registers,
// two row sums, dX written; the next row is loaded meanwhile.
template <typename T, int VPL, int KIND, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_entmax_rows_bwd(EntmaxRowsArgs a) {
  constexpr bool WG = WAVES == 16;
  constexpr int STRIDE = WG ? WAVES * kWave : kWave;
  __shared__ float s_red[2][2][WAVES];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int n = a.n;
  const int t = WG ? (int)threadIdx.x : lane;
  const long long step = WG ? (long long)gridDim.x : (long long)gridDim.x * WAVES;
  long long row = WG ? (long long)blockIdx.x : (long long)blockIdx.x * WAVES + w;
  float yn[VPL], dn[VPL];
  auto load_row = [&](long long r) {
    const T* y = static_cast<const T*>(a.X) + r * (long long)n;
    const T* dy = static_cast<const T*>(a.dY) + r * (long long)n;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = j * STRIDE + t;
      yn[j] = e < n ? load_elem(y + e) : 0.f;
      dn[j] = e < n ? load_elem(dy + e) : 0.f;
    }
  };
  if (row < a.rows) load_row(row);
  int par = 0;
  const float gexp = 2.f - a.alpha;
  for (; row < a.rows; row += step) {  // uniform over the row's threads
    T* dx = static_cast<T*>(a.Y) + row * (long long)n;
    float g[VPL], dy[VPL];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const float y = yn[j];
      if constexpr (KIND == 2) g[j] = y > 0.f ? __builtin_sqrtf(y) : 0.f;
      else if constexpr (KIND == 1) g[j] = y > 0.f ? 1.f : 0.f;
      else g[j] = y > 0.f ? fast_exp2(gexp * fast_log2(y)) : 0.f;
      dy[j] = dn[j];
      s0 += g[j];
      s1 = fmaf(g[j], dy[j], s1);
    }
    if (row + step < a.rows) load_row(row + step);
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if constexpr (WG) {
      if (lane == 0) {
        s_red[par][0][w] = s0;
        s_red[par][1][w] = s1;
      }
      __syncthreads();  // also orders the reads of this parity two rows back
      s0 = s1 = 0.f;
#pragma unroll
      for (int k = 0; k < WAVES; ++k) {
        s0 += s_red[par][0][k];
        s1 += s_red[par][1][k];
      }
      par ^= 1;
    }
    const float c = s0 > 0.f ? s1 / s0 : 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = j * STRIDE + t;
      if (e < n) store_elem(dx + e, g[j] * (dy[j] - c));
    }
  }
}

namespace {

template <typename T, int KIND>
hipError_t entmax_rows_bwd_t(const EntmaxRowsArgs& a, hipStream_t stream) {
  if (a.n <= 64 * 32) {
    const dim3 grid((unsigned)std::min<long long>((a.rows + 3) / 4, (long long)a.n_cu * 8));
    const int v = (a.n + 63) / 64;
#define DASH_ER(V)                                                                               \
  if (v <= V) {                                                                                  \
    hipLaunchKernelGGL((k_entmax_rows_bwd<T, V, KIND, 4>), grid, dim3(4 * kWave), 0, stream, a); \
    return hipGetLastError();                                                                    \
  }
    DASH_ER(1) DASH_ER(2) DASH_ER(4) DASH_ER(8) DASH_ER(16) DASH_ER(32)
#undef DASH_ER
  }
  const dim3 grid((unsigned)std::min<long long>(a.rows, (long long)a.n_cu * 2));
  const int v = (a.n + 1023) / 1024;
#define DASH_ER(V)                                                                                 \
  if (v <= V) {                                                                                    \
    hipLaunchKernelGGL((k_entmax_rows_bwd<T, V, KIND, 16>), grid, dim3(16 * kWave), 0, stream, a); \
    return hipGetLastError();                                                                      \
  }
  DASH_ER(4) DASH_ER(8) DASH_ER(16) DASH_ER(32)
#undef DASH_ER
  return hipErrorInvalidValue;
}

template <typename T, int KIND>
hipError_t entmax_rows_t(const EntmaxRowsArgs& a, hipStream_t stream) {
  if (a.n <= 64 * 32) {
    const dim3 grid((unsigned)std::min<long long>((a.rows + 3) / 4, (long long)a.n_cu * 8));
    const int v = (a.n + 63) / 64;
#define DASH_ER(V)                                                                           \
  if (v <= V) {                                                                              \
    hipLaunchKernelGGL((k_entmax_rows<T, V, KIND, 4>), grid, dim3(4 * kWave), 0, stream, a); \
    return hipGetLastError();                                                                \
  }
    DASH_ER(1) DASH_ER(2) DASH_ER(4) DASH_ER(8) DASH_ER(16) DASH_ER(32)
#undef DASH_ER
  }
  const dim3 grid((unsigned)std::min<long long>(a.rows, (long long)a.n_cu * 2));
  const int v = (a.n + 1023) / 1024;
#define DASH_ER(V)                                                                             \
  if (v <= V) {                                                                                \
    hipLaunchKernelGGL((k_entmax_rows<T, V, KIND, 16>), grid, dim3(16 * kWave), 0, stream, a); \
    return hipGetLastError();                                                                  \
  }
  DASH_ER(4) DASH_ER(8) DASH_ER(16) DASH_ER(32)
#undef DASH_ER
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t entmax_rows_kind(const EntmaxRowsArgs& a, hipStream_t stream) {
  if (a.alpha == 1.5f) return entmax_rows_t<T, 2>(a, stream);
  if (a.alpha == 2.0f) return entmax_rows_t<T, 1>(a, stream);
  return entmax_rows_t<T, 0>(a, stream);
}

}  // namespace

template <typename T>
hipError_t entmax_rows_bwd_kind(const EntmaxRowsArgs& a, hipStream_t stream) {
  if (a.alpha == 1.5f) return entmax_rows_bwd_t<T, 2>(a, stream);
  if (a.alpha == 2.0f) return entmax_rows_bwd_t<T, 1>(a, stream);
  return entmax_rows_bwd_t<T, 0>(a, stream);
}

hipError_t launch_entmax_rows(const EntmaxRowsArgs& a, bool bf16, hipStream_t stream) {
  if (a.dY != nullptr) return bf16 ? entmax_rows_bwd_kind<uint16_t>(a, stream) : entmax_rows_bwd_kind<float>(a, stream);
  return bf16 ? entmax_rows_kind<uint16_t>(a, stream) : entmax_rows_kind<float>(a, stream);
}

}  // namespace dash
