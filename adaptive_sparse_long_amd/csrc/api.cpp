// api.cpp -- the C ABI of libdash.so (declared in include/dash.h): argument
// validation on the host, workspace sizing, and kernel launches on the caller's
// stream. Nothing here allocates device memory or synchronises the host.
#include "dash.h"

#include <math.h>

#include <mutex>
#include <vector>

#include "kernels.hpp"

using namespace dash;

namespace {

bool finite_gt1(float a) { return isfinite(a) && a > 1.f; }

dash_status check_params(const dash_params& p) {
  if (p.chunk_size <= 0) return DASH_ERR_INVALID_ARG;
  if (!finite_gt1(p.alpha) || p.n_iter < 1 || !isfinite(p.scaling_factor)) return DASH_ERR_INVALID_ARG;
  if ((p.causal != 0 && p.causal != 1) || (p.estimate_diagonal != 0 && p.estimate_diagonal != 1))
    return DASH_ERR_INVALID_ARG;
  if (p.chunk_size != kChunk) return DASH_ERR_UNSUPPORTED;
  return DASH_OK;
}

bool gqa_ok(int Hq, int Hkv) { return Hq > 0 && Hkv > 0 && Hq % Hkv == 0; }
bool g_supported(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

dash_status from_hip(hipError_t e) { return e == hipSuccess ? DASH_OK : DASH_ERR_HIP; }

// Compute units of the current device (sizes persistent grids).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

// Pool slots are addressed with 32 bits.

// Scratch of the allocation-free decode step: a file-scope device array (each
// GPU holds its own copy from the time the library is loaded until the process
// ends). Host code never uses the array's name as an address: its device
// address is looked up once per device (hipGetSymbolAddress, with the device
// current) and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dash_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DASH_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DASH_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DASH_OK;
}

}  // namespace

extern "C" {

void dash_default_params(dash_params* p) {
  if (!p) return;
  p->chunk_size = 64;
  p->alpha = 1.5f;
  p->n_iter = 10;
  p->scaling_factor = 1.0f;
  p->causal = 1;
  p->estimate_diagonal = 1;
}

const char* dash_status_string(int status) {
  // an int, not dash_status: any value a caller passes is valid to read
  switch (status) {
    case DASH_OK: return "ok";
    case DASH_ERR_INVALID_ARG: return "invalid argument";
    case DASH_ERR_UNSUPPORTED: return "unsupported configuration";
    case DASH_ERR_WORKSPACE: return "workspace too small";
    case DASH_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

dash_status dash_summarize(const void* K, const void* head_cls, float* S, dash_dtype dt, int B,
                           int Hkv, int Lmax, int d, int n_tokens, const int* seqlens,
                           int chunk_begin, int chunk_end, int s_cap, dash_params p,
                           hipStream_t stream) {
  if (!K || !head_cls || !S) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || Hkv <= 0 || Lmax <= 0 || d <= 0 || s_cap <= 0) return DASH_ERR_INVALID_ARG;
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > s_cap) return DASH_ERR_INVALID_ARG;
  if (!seqlens && (n_tokens <= 0 || n_tokens > Lmax)) return DASH_ERR_INVALID_ARG;
  if (p.chunk_size <= 0) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  if (p.chunk_size != kChunk || dt != DASH_BF16 || !dash_head_dim_ok(d)) return DASH_ERR_UNSUPPORTED;
  if ((long long)chunk_end * kChunk > (long long)Lmax + kChunk - 1) return DASH_ERR_INVALID_ARG;
  if (chunk_end == chunk_begin) return DASH_OK;
  SummarizeArgs a{K, head_cls, S, B, Hkv, Lmax, d, n_tokens, seqlens, chunk_begin, chunk_end,
                  s_cap, kChunk, 1.f / sqrtf((float)d)};
  return from_hip(launch_summarize(a, stream));
}

dash_status dash_summarize_backward(const void* K, const void* head_cls, const float* dS,
                                    dash_dtype dt, int B, int Hkv, int Lmax, int d, int n_tokens,
                                    int chunk_begin, int chunk_end, int s_cap, dash_params p,
                                    float* dK, float* dcls, float* partials, hipStream_t stream) {
  if (!K || !head_cls || !dS || !dK || !dcls || !partials) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || Hkv <= 0 || Lmax <= 0 || d <= 0 || s_cap <= 0) return DASH_ERR_INVALID_ARG;
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > s_cap) return DASH_ERR_INVALID_ARG;
  if (n_tokens <= 0 || n_tokens > Lmax || p.chunk_size <= 0) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  if (p.chunk_size != kChunk || dt != DASH_BF16 || !dash_head_dim_ok(d)) return DASH_ERR_UNSUPPORTED;
  if ((long long)chunk_end * kChunk > (long long)Lmax + kChunk - 1) return DASH_ERR_INVALID_ARG;
  SummarizeBwdArgs a{K, head_cls, dS, dK, dcls, partials, B, Hkv, Lmax, d, n_tokens,
                     chunk_begin, chunk_end, s_cap, kChunk, 1.f / sqrtf((float)d)};
  return from_hip(launch_summarize_bwd(a, stream));
}

size_t dash_workspace_size(int B, int Hq, int Hkv, int Nq, int Lmax, int d, int decode,
                           dash_params p) {
  if (B <= 0 || !gqa_ok(Hq, Hkv) || Lmax <= 0 || d <= 0 || p.chunk_size != kChunk) return 0;
  // the kernels' own arrays are kDashD wide whatever the head_dim
  if (decode) return decode_layout(B, Hq, Hkv, Lmax, kDashD).total;
  if (Nq <= 0 || Nq > Lmax) return 0;
  return prefill_layout(B, Hq, Hkv, Nq, kDashD, p.causal != 0, prefill_default_pairs(B, Hq, Nq)).total;
}

size_t dash_prefill_workspace_size(int B, int Hq, int Hkv, int Nq, int Lmax, int d, dash_params p,
                                   long long pool_pairs) {
  if (B <= 0 || !gqa_ok(Hq, Hkv) || Lmax <= 0 || d <= 0 || p.chunk_size != kChunk) return 0;
  if (Nq <= 0 || Nq > Lmax || pool_pairs < 0 || pool_pairs > kPoolMaxPairs) return 0;
  return prefill_layout(B, Hq, Hkv, Nq, kDashD, p.causal != 0, pool_pairs).total;
}

dash_status dash_route(const void* Q, const void* K, const void* head_cls, const float* S,
                       dash_dtype dt, int B, int Hq, int Hkv, int Nq, int Lmax, int d, int s_cap,
                       const int* seqlens, dash_params p, float* tau, uint32_t* active_bits,
                       int bits_words, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!Q || !K || !head_cls || !S || !tau || !workspace) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || Nq <= 0 || Lmax <= 0 || d <= 0 || s_cap <= 0 || !gqa_ok(Hq, Hkv))
    return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  dash_status st = check_params(p);
  if (st != DASH_OK) return st;
  if (dt != DASH_BF16 || !dash_head_dim_ok(d)) return DASH_ERR_UNSUPPORTED;
  const int g = Hq / Hkv;
  const bool decode = seqlens != nullptr;
  RouteArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.cls = static_cast<const uint16_t*>(head_cls);
  a.S = S;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.g = g; a.Nq = Nq; a.Lmax = Lmax; a.d = d; a.s_cap = s_cap;
  a.seqlens = seqlens;
  a.alpha = p.alpha;
  a.beta = 1.f / (p.alpha - 1.f);
  a.inv_sqrt_d = 1.f / sqrtf((float)d);
  a.zscale = p.scaling_factor * a.inv_sqrt_d;
  a.n_iter = p.n_iter;
  a.causal = p.causal;
  a.est = p.causal ? p.estimate_diagonal : 0;
  a.tau = tau;
  a.bits = active_bits;
  a.bits_words = bits_words;
  char* ws = static_cast<char*>(workspace);
  if (decode) {
    if (Nq != 1 || p.causal != 1) return DASH_ERR_INVALID_ARG;
    if ((Lmax - 1) / kChunk > kRouteDecodeMaxComplete || !g_supported(g)) return DASH_ERR_UNSUPPORTED;
    if (s_cap < (Lmax - 1) / kChunk) return DASH_ERR_INVALID_ARG;
    const DecodeLayout L = decode_layout(B, Hq, Hkv, Lmax, kDashD);
    if (active_bits && bits_words < (L.n_slots + 31) / 32) return DASH_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return DASH_ERR_WORKSPACE;
    a.n_slots = L.n_slots;
    a.z = reinterpret_cast<float*>(ws + L.off_z);
    a.counts = reinterpret_cast<int*>(ws + L.off_counts);
    a.lists = reinterpret_cast<int*>(ws + L.off_lists);
    a.bias = reinterpret_cast<float*>(ws + L.off_bias);
    return from_hip(launch_route_decode(a, stream));
  }
  if (Nq > Lmax) return DASH_ERR_INVALID_ARG;
  const int n_slots = (Nq + kChunk - 1) / kChunk;
  if (n_slots > kPrefillMaxSlots) return DASH_ERR_UNSUPPORTED;
  if (s_cap < (p.causal ? Nq / kChunk : n_slots)) return DASH_ERR_INVALID_ARG;
  if (active_bits && bits_words < (n_slots + 31) / 32) return DASH_ERR_INVALID_ARG;
  const long long pool = prefill_pool_from_bytes(B, Hq, Hkv, Nq, kDashD, p.causal != 0, ws_bytes);
  if (pool < 0) return DASH_ERR_WORKSPACE;
  const PrefillLayout L = prefill_layout(B, Hq, Hkv, Nq, kDashD, p.causal != 0, pool);
  if (ws_bytes < L.total) return DASH_ERR_WORKSPACE;
  a.n_tiles = L.n_tiles;
  a.n_slots = L.n_slots;
  a.per_head = L.per_head;
  a.counts = reinterpret_cast<int*>(ws + L.off_counts);
  a.lists = reinterpret_cast<int*>(ws + L.off_lists);
  a.bias = nullptr;
  a.rm_tau = reinterpret_cast<float*>(ws + L.off_rmtau);
  a.rm_bits = reinterpret_cast<uint32_t*>(ws + L.off_rmbits);
  a.rm_words = L.words;
  a.ccounts = reinterpret_cast<int*>(ws + L.off_ccounts);
  a.clists = reinterpret_cast<int*>(ws + L.off_clists);
  a.ceo = reinterpret_cast<int2*>(ws + L.off_ceo);
  a.trec = reinterpret_cast<int4*>(ws + L.off_trec);
  a.cbase = reinterpret_cast<int*>(ws + L.off_cbase);
  a.cmp = reinterpret_cast<int*>(ws + L.off_cmp);
  a.n_bhc = L.n_bhc;
  a.pool = reinterpret_cast<unsigned long long*>(ws + L.off_pool);
  a.pool_cap = L.pool_cap;
  a.tbase = reinterpret_cast<uint32_t*>(ws + L.off_tbase);
  a.rslot = reinterpret_cast<uint32_t*>(ws + L.off_rslot);
  a.cmcnt = reinterpret_cast<uint16_t*>(ws + L.off_cmcnt);
  a.own_lw = reinterpret_cast<float*>(ws + L.off_own);
  a.fb_tiles = reinterpret_cast<int2*>(ws + L.off_fb);
  a.fb_count = reinterpret_cast<int*>(ws + L.off_fb_count);
  a.n_rm = a.fb_count + 1;
  a.s_hi = reinterpret_cast<uint16_t*>(ws + L.off_split);
  a.s_lo = a.s_hi + (size_t)B * Hkv * L.n_slots * kDashD;
  a.s_err = reinterpret_cast<float*>(ws + L.off_serr);
  a.gscr = reinterpret_cast<float*>(ws + L.off_gscr);
  return from_hip(launch_route_prefill(a, stream));
}

dash_status dash_sparse_attn_prefill(const void* Q, const void* K, const void* V, dash_dtype dt,
                                     int B, int Hq, int Hkv, int N, int Lmax, int d,
                                     dash_params p, void* O, void* workspace,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!Q || !K || !V || !O || !workspace) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || N <= 0 || Lmax <= 0 || N > Lmax || d <= 0 || !gqa_ok(Hq, Hkv))
    return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  dash_status st = check_params(p);
  if (st != DASH_OK) return st;
  if (dt != DASH_BF16 || !dash_head_dim_ok(d)) return DASH_ERR_UNSUPPORTED;
  if ((N + kChunk - 1) / kChunk > kPrefillMaxSlots) return DASH_ERR_UNSUPPORTED;
  const long long pool = prefill_pool_from_bytes(B, Hq, Hkv, N, kDashD, p.causal != 0, ws_bytes);
  if (pool < 0) return DASH_ERR_WORKSPACE;
  const PrefillLayout L = prefill_layout(B, Hq, Hkv, N, kDashD, p.causal != 0, pool);
  if (ws_bytes < L.total) return DASH_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  PrefillAttnArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.O = static_cast<uint16_t*>(O);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.g = Hq / Hkv; a.N = N; a.Lmax = Lmax;
  a.causal = p.causal;
  a.d = d;
  a.scale_log2 = kLog2e / sqrtf((float)d);
  a.n_tiles = L.n_tiles;
  a.n_slots = L.n_slots;
  a.per_head = L.per_head;
  a.counts = reinterpret_cast<const int*>(ws + L.off_counts);
  a.lists = reinterpret_cast<const int*>(ws + L.off_lists);
  a.rm_tau = reinterpret_cast<const float*>(ws + L.off_rmtau);
  a.rm_bits = reinterpret_cast<const uint32_t*>(ws + L.off_rmbits);
  a.rm_words = L.words;
  a.s_hi = reinterpret_cast<const uint16_t*>(ws + L.off_split);
  a.s_lo = a.s_hi + (size_t)B * Hkv * L.n_slots * kDashD;
  a.beta = 1.f / (p.alpha - 1.f);
  a.ccounts = reinterpret_cast<const int*>(ws + L.off_ccounts);
  a.clists = reinterpret_cast<const int*>(ws + L.off_clists);
  a.ceo = reinterpret_cast<const int2*>(ws + L.off_ceo);
  a.trec = reinterpret_cast<const int4*>(ws + L.off_trec);
  a.cmp = reinterpret_cast<const int*>(ws + L.off_cmp);
  a.cs = reinterpret_cast<int*>(ws + L.off_cs);
  a.cbase = reinterpret_cast<const int*>(ws + L.off_cbase);
  a.nitems = reinterpret_cast<int*>(ws + L.off_nitems);
  a.items = reinterpret_cast<int2*>(ws + L.off_items);
  a.recs = reinterpret_cast<int4*>(ws + L.off_recs);
  a.n_bhc = L.n_bhc;
  a.max_items = L.max_items;
  a.pool_cap = L.pool_cap;
  a.n_cu = device_cus();
  a.tbase = reinterpret_cast<const uint32_t*>(ws + L.off_tbase);
  a.rslot = reinterpret_cast<const uint32_t*>(ws + L.off_rslot);
  a.cmcnt = reinterpret_cast<const uint16_t*>(ws + L.off_cmcnt);
  a.own_lw = reinterpret_cast<const float*>(ws + L.off_own);
  a.qhead = reinterpret_cast<int*>(ws + L.off_qhead);
  a.bad = a.qhead + 1;
  a.pool = reinterpret_cast<const unsigned long long*>(ws + L.off_pool);
  a.n_rm = reinterpret_cast<const int*>(ws + L.off_fb_count) + 1;
  a.plse = reinterpret_cast<float*>(ws + L.off_plse);
  a.po = reinterpret_cast<uint16_t*>(ws + L.off_po);
  return from_hip(launch_sparse_prefill(a, stream));
}

dash_status dash_prefill_counters(const void* workspace, size_t ws_bytes, int B, int Hq, int Hkv, int N,
                                  int d, dash_params p, long long* out, hipStream_t stream) {
  if (!workspace || !out) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || N <= 0 || d <= 0 || !gqa_ok(Hq, Hkv)) return DASH_ERR_INVALID_ARG;
  const long long pool = prefill_pool_from_bytes(B, Hq, Hkv, N, kDashD, p.causal != 0, ws_bytes);
  if (pool < 0) return DASH_ERR_WORKSPACE;
  const PrefillLayout L = prefill_layout(B, Hq, Hkv, N, kDashD, p.causal != 0, pool);
  const char* ws = static_cast<const char*>(workspace);
  std::vector<int> cmp((size_t)L.n_bhc);
  int fb[2] = {0, 0};
  hipError_t e = hipMemcpyAsync(cmp.data(), ws + L.off_cmp, cmp.size() * sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(fb, ws + L.off_fb_count, sizeof(fb), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return DASH_ERR_HIP;
  long long pairs = 0;
  for (int c : cmp) pairs += c;
  out[0] = pairs;
  out[1] = L.pool_cap;
  out[2] = fb[0];
  out[3] = fb[1];
  return DASH_OK;
}

dash_status dash_sparse_attn_decode(const void* Q, const void* Kc, const void* Vc, dash_dtype dt,
                                    int B, int Hq, int Hkv, const int* seqlens, int Lmax, int d,
                                    dash_params p, void* O, void* workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!Q || !Kc || !Vc || !O || !workspace || !seqlens) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || Lmax <= 0 || d <= 0 || !gqa_ok(Hq, Hkv)) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  dash_status st = check_params(p);
  if (st != DASH_OK) return st;
  if (p.causal != 1) return DASH_ERR_INVALID_ARG;
  const int g = Hq / Hkv;
  if (dt != DASH_BF16 || !dash_head_dim_ok(d) || !g_supported(g)) return DASH_ERR_UNSUPPORTED;
  if ((Lmax - 1) / kChunk > kRouteDecodeMaxComplete) return DASH_ERR_UNSUPPORTED;
  const DecodeLayout L = decode_layout(B, Hq, Hkv, Lmax, kDashD);
  if (ws_bytes < L.total) return DASH_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  DecodeAttnArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(Kc);
  a.V = static_cast<const uint16_t*>(Vc);
  a.O = static_cast<uint16_t*>(O);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.g = g; a.Lmax = Lmax;
  a.d = d;
  a.seqlens = seqlens;
  a.scale_log2 = kLog2e / sqrtf((float)d);
  a.n_slots = L.n_slots;
  a.n_splits = L.n_splits;
  a.counts = reinterpret_cast<const int*>(ws + L.off_counts);
  a.lists = reinterpret_cast<const int*>(ws + L.off_lists);
  a.bias = reinterpret_cast<const float*>(ws + L.off_bias);
  a.part = reinterpret_cast<float*>(ws + L.off_part);
  return from_hip(launch_sparse_decode(a, stream));
}

size_t dash_backward_workspace_size(int B, int Hq, int Hkv, int N, int Lmax, int d, dash_params p) {
  if (B <= 0 || !gqa_ok(Hq, Hkv) || N <= 0 || Lmax < N || d <= 0 || p.chunk_size != kChunk) return 0;
  return dash_bwd_layout(B, Hq, Hkv, N, Lmax, d, p.causal != 0).total;
}

dash_status dash_sparse_attn_prefill_backward(const void* Q, const void* K, const void* V,
                                              const void* head_cls, const float* S,
                                              const void* dO, const float* tau,
                                              const uint32_t* active_bits, int bits_words,
                                              dash_dtype dt, int B, int Hq, int Hkv, int N, int Lmax,
                                              int d, int s_cap, dash_params p, void* dQ, void* dK,
                                              void* dV, float* dcls, void* workspace,
                                              size_t ws_bytes, hipStream_t stream) {
  if (!Q || !K || !V || !head_cls || !S || !dO || !tau || !active_bits || !dQ || !dK || !dV || !dcls || !workspace)
    return DASH_ERR_INVALID_ARG;
  if (B <= 0 || N <= 0 || Lmax < N || d <= 0 || s_cap <= 0 || !gqa_ok(Hq, Hkv)) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  dash_status st = check_params(p);
  if (st != DASH_OK) return st;
  if (dt != DASH_BF16 || !dash_head_dim_ok(d)) return DASH_ERR_UNSUPPORTED;
  const DashBwdLayout L = dash_bwd_layout(B, Hq, Hkv, N, Lmax, d, p.causal != 0);
  if (L.n_slots > kDashBwdMaxSlots) return DASH_ERR_UNSUPPORTED;
  if (bits_words < (L.n_slots + 31) / 32) return DASH_ERR_INVALID_ARG;
  if (s_cap < L.n_sum) return DASH_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return DASH_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  DashBwdArgs a{};
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.dO = static_cast<const uint16_t*>(dO);
  a.cls = static_cast<const uint16_t*>(head_cls);
  a.S = S;
  a.tau = tau;
  a.bits = active_bits;
  a.bits_words = bits_words;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.g = Hq / Hkv; a.N = N; a.Lmax = Lmax; a.s_cap = s_cap;
  a.d = d;
  a.n_slots = L.n_slots;
  a.n_sum = L.n_sum;
  a.causal = p.causal;
  a.est = p.causal ? p.estimate_diagonal : 0;
  a.alpha = p.alpha;
  a.beta = 1.f / (p.alpha - 1.f);
  a.inv_sqrt_d = 1.f / sqrtf((float)d);
  a.rt = p.scaling_factor * a.inv_sqrt_d;
  a.sf = p.scaling_factor;
  a.uscale = (p.alpha - 1.f) * a.rt;
  a.scale_log2 = kLog2e * a.inv_sqrt_d;
  a.WT = reinterpret_cast<float*>(ws + L.off_wt);
  a.DZT = reinterpret_cast<float*>(ws + L.off_dzt);
  a.lse = reinterpret_cast<float*>(ws + L.off_lse);
  a.Dd = reinterpret_cast<float*>(ws + L.off_dd);
  a.dQf = reinterpret_cast<float*>(ws + L.off_dqf);
  a.dKf = reinterpret_cast<float*>(ws + L.off_dkf);
  a.dSum = reinterpret_cast<float*>(ws + L.off_dsum);
  a.dKs = reinterpret_cast<float*>(ws + L.off_dks);
  a.sb_part = reinterpret_cast<float*>(ws + L.off_sbp);
  a.dcls_s = reinterpret_cast<float*>(ws + L.off_dcs);
  a.dcls_p = reinterpret_cast<float*>(ws + L.off_dcp);
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.dcls = dcls;
  return from_hip(launch_dash_bwd(a, stream));
}

size_t dash_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

dash_status dash_decode_step_noalloc(const void* Q, const void* Kc, const void* Vc, const void* head_cls,
                                     const float* S, dash_dtype dt, int B, int Hq, int Hkv,
                                     const int* seqlens, int Lmax, int d, int s_cap, dash_params p,
                                     void* O, float* tau, uint32_t* active_bits, int bits_words,
                                     hipStream_t stream) {
  if (!Q || !Kc || !Vc || !head_cls || !S || !seqlens || !O || !tau) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || Lmax <= 0 || d <= 0 || s_cap <= 0 || !gqa_ok(Hq, Hkv)) return DASH_ERR_INVALID_ARG;
  const size_t need = dash_workspace_size(B, Hq, Hkv, 1, Lmax, d, 1, p);
  if (need == 0) return DASH_ERR_INVALID_ARG;
  if (need > kNoAllocScratchBytes) return DASH_ERR_WORKSPACE;  // beyond the static scratch
  // the same host checks as the two calls below, before anything is launched
  dash_status st = check_params(p);
  if (st != DASH_OK) return st;
  if (p.causal != 1) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 || !dash_head_dim_ok(d) || !g_supported(Hq / Hkv)) return DASH_ERR_UNSUPPORTED;
  if ((Lmax - 1) / kChunk > kRouteDecodeMaxComplete) return DASH_ERR_UNSUPPORTED;
  if (s_cap < (Lmax - 1) / kChunk) return DASH_ERR_INVALID_ARG;
  if (active_bits && bits_words < (decode_layout(B, Hq, Hkv, Lmax, kDashD).n_slots + 31) / 32) return DASH_ERR_INVALID_ARG;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != DASH_OK) return st;
  st = dash_route(Q, Kc, head_cls, S, dt, B, Hq, Hkv, 1, Lmax, d, s_cap, seqlens, p, tau, active_bits,
                  bits_words, ws, kNoAllocScratchBytes, stream);
  if (st != DASH_OK) return st;
  return dash_sparse_attn_decode(Q, Kc, Vc, dt, B, Hq, Hkv, seqlens, Lmax, d, p, O, ws, kNoAllocScratchBytes,
                                 stream);
}

dash_status entmax_attn(const void* Q, const void* K, const void* V, dash_dtype dt, int B, int H,
                        int Nmax, int d, const int* varlen, float alpha, int n_iter, int causal,
                        void* O, float* tau, uint32_t* block_mask, hipStream_t stream) {
  if (!Q || !K || !V || !O || !tau) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Nmax <= 0 || d <= 0) return DASH_ERR_INVALID_ARG;
  if (!finite_gt1(alpha) || n_iter < 1 || (causal != 0 && causal != 1)) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return DASH_ERR_UNSUPPORTED;
  const int nT = (Nmax + 63) / 64;
  if (nT > kEntmaxMaxTiles) return DASH_ERR_UNSUPPORTED;
  EntmaxAttnArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.O = O;
  a.B = B; a.H = H; a.N = Nmax; a.d = d;
  a.varlen = varlen;
  a.alpha = alpha;
  a.beta = 1.f / (alpha - 1.f);
  a.scale = (alpha - 1.f) / sqrtf((float)d);
  a.n_iter = n_iter;
  a.causal = causal;
  a.tau = tau;
  a.mask = block_mask;
  a.mask_words = (nT + 31) / 32;
  return from_hip(launch_entmax_attn(a, dt == DASH_BF16, stream));
}

dash_status entmax_attn_backward(const void* Q, const void* K, const void* V, const void* dO,
                                 const float* tau, const uint32_t* block_mask, dash_dtype dt,
                                 int B, int H, int Nmax, int d, const int* varlen, float alpha,
                                 int causal, void* dQ, void* dK, void* dV, float* coef,
                                 hipStream_t stream) {
  if (!Q || !K || !V || !dO || !tau || !dQ || !dK || !dV || !coef) return DASH_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Nmax <= 0 || d <= 0) return DASH_ERR_INVALID_ARG;
  if (!finite_gt1(alpha) || (causal != 0 && causal != 1)) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return DASH_ERR_UNSUPPORTED;
  const int nT = (Nmax + 63) / 64;
  if (nT > kEntmaxMaxTiles) return DASH_ERR_UNSUPPORTED;
  EntmaxBwdArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.dO = dO;
  a.tau = tau;
  a.mask = block_mask;
  a.mask_words = (nT + 31) / 32;
  a.B = B; a.H = H; a.N = Nmax; a.d = d;
  a.varlen = varlen;
  a.alpha = alpha;
  a.beta = 1.f / (alpha - 1.f);
  a.scale = (alpha - 1.f) / sqrtf((float)d);
  a.inv_sqrt_d = 1.f / sqrtf((float)d);
  a.causal = causal;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.coef = coef;
  return from_hip(launch_entmax_attn_bwd(a, dt == DASH_BF16, stream));
}

dash_status entmax_rows(const void* X, void* Y, dash_dtype dt, int rows, int n, float alpha,
                        int n_iter, float* tau, hipStream_t stream) {
  if (!X || !Y) return DASH_ERR_INVALID_ARG;
  if (rows <= 0 || n <= 0 || !finite_gt1(alpha) || n_iter < 1) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  if (n > kEntmaxRowsMax) return DASH_ERR_UNSUPPORTED;
  EntmaxRowsArgs a{};
  a.X = X;
  a.Y = Y;
  a.rows = rows;
  a.n = n;
  a.alpha = alpha;
  a.beta = 1.f / (alpha - 1.f);
  a.n_iter = n_iter;
  a.tau = tau;
  a.n_cu = device_cus();
  return from_hip(launch_entmax_rows(a, dt == DASH_BF16, stream));
}

dash_status entmax_rows_backward(const void* Y, const void* dY, void* dX, dash_dtype dt, int rows,
                                 int n, float alpha, hipStream_t stream) {
  if (!Y || !dY || !dX) return DASH_ERR_INVALID_ARG;
  if (rows <= 0 || n <= 0 || !finite_gt1(alpha)) return DASH_ERR_INVALID_ARG;
  if (dt != DASH_BF16 && dt != DASH_F32) return DASH_ERR_INVALID_ARG;
  if (n > kEntmaxRowsMax) return DASH_ERR_UNSUPPORTED;
  EntmaxRowsArgs a{};
  a.X = Y;
  a.dY = dY;
  a.Y = dX;
  a.rows = rows;
  a.n = n;
  a.alpha = alpha;
  a.beta = 1.f / (alpha - 1.f);
  a.n_cu = device_cus();
  return from_hip(launch_entmax_rows(a, dt == DASH_BF16, stream));
}

}  // extern "C"
