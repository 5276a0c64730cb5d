/*
 * dash.h -- C ABI of libdash.so: hierarchical adaptive sparse attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The operations follow two pages:
 *   - "DashAttention: Differentiable and Adaptive Sparse Hierarchical Attention"
 *     (README page), sections "Usage", "How it works" (items 1-3 and the
 *     prefill/decoding paragraph) and "Core API";
 *   - "AdaSplash: Adaptive Sparse Flash Attention" (README page), sections
 *     "Usage" (Triton Entmax; AdaSplash with Block Masking) and "Key Features"
 *     (varlen, alpha, causal masking).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a device pointer owned by the caller (for example
 *     a torch tensor's data_ptr()). The library never allocates device memory
 *     and keeps no state between calls except cached device properties and the
 *     one static scratch array of dash_decode_step_noalloc, so calls are
 *     thread safe; calls that share a workspace (or that scratch array) must be
 *     ordered by the caller (same stream).
 *   - Tensors are contiguous row-major. q/k/v use [batch, heads, seq, head_dim]
 *     ("Usage" of both pages); head_cls is [kv_heads, head_dim].
 *   - head_dim: 64 or 128 for every entry point. The forward DashAttention
 *     kernels keep their own arrays 128 wide, so dash_workspace_size gives the
 *     same size for head_dim 64 as for 128.
 *   - Work is enqueued on `stream` (NULL = the null stream); nothing
 *     synchronises the host. Outputs are valid once the stream reaches them.
 *   - All argument checks run on the host before any HIP call, so a bad call
 *     returns an error code, writes nothing and launches nothing. No C++
 *     exception crosses this boundary.
 *   - Status codes: DASH_ERR_INVALID_ARG for null pointers, non-positive sizes,
 *     Hq not a multiple of Hkv, alpha <= 1, n_iter < 1 and inconsistent sizes;
 *     DASH_ERR_UNSUPPORTED for a head_dim, dtype, chunk size or length outside
 *     what the kernels are built for; DASH_ERR_WORKSPACE when ws_bytes is below
 *     the matching *_workspace_size(); DASH_ERR_HIP when a launch fails.
 *
 * Notation: B batch, Hq query heads, Hkv KV heads (Hq % Hkv == 0, query head h
 * reads KV head h / (Hq / Hkv): the "enable_gqa" behaviour of "Core API"),
 * d head_dim, C chunk_size, alpha > 1, u = (alpha - 1) * score.
 */
#ifndef DASH_H_
#define DASH_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARG = 1,
  DASH_ERR_UNSUPPORTED = 2,
  DASH_ERR_WORKSPACE = 3,
  DASH_ERR_HIP = 4
} dash_status;

/* The two sentinels give the type the range of int, so that validation can
 * read (and reject) any value a caller passes. */
typedef enum {
  DASH_F32 = 0,
  DASH_BF16 = 1,
  DASH_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  DASH_DTYPE_RANGE_MAX_ = 2147483647
} dash_dtype;

/* Arguments of the DashAttention wrapper ("Core API": chunk_size,
 * estimate_diagonal, scaling_factor) plus the entmax alpha and iteration
 * count of the AdaSplash "Usage" section. Passed by value. */
typedef struct {
  int chunk_size;        /* C; the kernels are built for 64 */
  float alpha;           /* entmax alpha for chunk routing, > 1 (default 1.5) */
  int n_iter;            /* maximum Halley/bisection steps for tau (default 10) */
  float scaling_factor;  /* multiplies the routing scores (default 1.0) */
  int causal;            /* 1: query i sees keys j <= i; 0: all keys */
  int estimate_diagonal; /* causal only. 1: the query's own, still incomplete
                            chunk is routed like the others, scored against the
                            summary of its tokens seen so far; 0: it is not
                            routed and always attended with weight 1 */
} dash_params;

/* Fills p with the defaults of "Core API": C = 64, alpha = 1.5, n_iter = 10,
 * scaling_factor = 1, causal = 1, estimate_diagonal = 1. */
void dash_default_params(dash_params* p);

/* ---------------------------------------------------------------------------
 * dash_summarize -- stage 1, "Local chunk summarization" ("How it works" 1):
 * one key summary per KV chunk built with head_cls. For every (b, kv head h)
 * and chunk c in [chunk_begin, chunk_end):
 *     a_j = softmax_j(<k_j, head_cls[h]> / sqrt(d)) over the chunk's tokens,
 *     S[b, h, c, :] = sum_j a_j k_j          (float32)
 * Chunk c holds tokens [c*C, min((c+1)*C, n_b)) where n_b = seqlens[b] if
 * seqlens is given, else n_tokens. A chunk with no token in a batch entry is
 * skipped; with seqlens given, only chunks complete in that entry
 * ((c+1)*C <= seqlens[b]) are written -- the decode-time "append newly
 * completed chunks" of the prefill/decoding paragraph.
 *   K        [B, Hkv, Lmax, d]   dtype dt
 *   head_cls [Hkv, d]            dtype dt
 *   S        [B, Hkv, s_cap, d]  float32, chunk_end <= s_cap
 *   seqlens  [B] int32 on the device, or NULL
 * --------------------------------------------------------------------------- */
dash_status dash_summarize(const void* K, const void* head_cls, float* S, dash_dtype dt,
                           int B, int Hkv, int Lmax, int d, int n_tokens,
                           const int* seqlens, int chunk_begin, int chunk_end, int s_cap,
                           dash_params p, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * dash_summarize_backward -- gradients through stage 1 (the DashAttention
 * README calls the hierarchy differentiable, "How it works"; the steps are the
 * summary's own chain rule). For a cotangent dS of the summaries S written by
 * dash_summarize over tokens [0, n_tokens), for every (b, kv head h) and chunk
 * c in [chunk_begin, chunk_end) holding tokens j (recomputing a and s_c):
 *     de_j = a_j (<k_j, dS[b,h,c]> - <s_c, dS[b,h,c]>),
 *     dK[b, h, j, :] = a_j dS[b,h,c] + de_j head_cls[h] / sqrt(d),
 *     dcls[h, :]     = sum over b and the chunks of sum_j de_j k_j / sqrt(d).
 *   K        [B, Hkv, Lmax, d]  dtype dt;   head_cls [Hkv, d] dtype dt
 *   dS       [B, Hkv, s_cap, d] float32 (rows of the listed chunks are read)
 *   dK       [B, Hkv, Lmax, d]  float32, written for the tokens of the listed
 *            chunks only (other rows untouched)
 *   dcls     [Hkv, d] float32, written (zeros for an empty chunk range)
 *   partials [B, Hkv, chunk_end - chunk_begin, d] float32 scratch, caller-owned
 * dcls is reduced in a fixed order (deterministic). Device memory is the
 * caller's; nothing is allocated; no host sync. Errors: NULL pointers, sizes
 * <= 0, a chunk range outside [0, s_cap] or past Lmax, n_tokens outside
 * [1, Lmax] -> DASH_ERR_INVALID_ARG; dt other than DASH_BF16, d not 64 or 128
 * or chunk_size != 64 -> DASH_ERR_UNSUPPORTED; a launch failure -> DASH_ERR_HIP.
 * --------------------------------------------------------------------------- */
dash_status dash_summarize_backward(const void* K, const void* head_cls, const float* dS,
                                    dash_dtype dt, int B, int Hkv, int Lmax, int d, int n_tokens,
                                    int chunk_begin, int chunk_end, int s_cap, dash_params p,
                                    float* dK, float* dcls, float* partials, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * dash_route -- stage 2, "Entmax block routing" ("How it works" 2): routing
 * scores z = scaling_factor * <q_i, s_c> / sqrt(d) against every candidate
 * chunk summary, alpha-entmax over them with the threshold tau found by
 * safeguarded Halley steps with bisection (AdaSplash "Usage": Triton Entmax),
 * the routed set (the support) and the prior pi_c = (u_c - tau)_+^(1/(alpha-1)).
 *
 * Candidates of query row i with chunk c_i = i / C:
 *   causal:     complete chunks c < c_i, plus (estimate_diagonal) c_i scored
 *               against the summary of tokens [c_i*C, i] computed on the fly;
 *               without estimate_diagonal c_i is attended with weight 1.
 *   non-causal: every chunk; S must then also hold the partial last chunk.
 *
 * Two modes:
 *   prefill (seqlens == NULL): rows i = 0 .. Nq-1 of Q [B, Hq, Nq, d];
 *       keys K [B, Hkv, Lmax, d] with Nq <= Lmax, n_tokens = Nq.
 *   decode  (seqlens != NULL): Nq must be 1; Q [B, Hq, 1, d] is the new token
 *       at position t_b = seqlens[b] - 1, whose key/value are already in the
 *       caches; causal must be 1.
 * S [B, Hkv, s_cap, d] float32 holds the chunk summaries (dash_summarize).
 *
 * Outputs
 *   tau         [B, Hq, Nq] float32, in u units; +inf for a row without any
 *               candidate (causal, estimate_diagonal = 0, first chunk).
 *   active_bits [B, Hq, Nq, bits_words] uint32 or NULL; bit c % 32 of word
 *               c / 32 is set iff chunk c is attended by the row (the kernel
 *               form of "return_active_blocks", "Usage"/"Core API").
 *               bits_words >= ceil(ceil(Lmax / C) / 32).
 *   workspace   the routed work lists and log2 priors read by the matching
 *               dash_sparse_attn_* call; size from dash_workspace_size().
 *               Prefill: the part beyond the fixed lists is the partial-result
 *               pool of dash_sparse_attn_prefill, one slot per (row, routed
 *               past chunk) pair (292 bytes each, whatever the head_dim), so a larger workspace
 *               buys a larger pool (dash_prefill_workspace_size); the same
 *               ws_bytes must then be passed to dash_sparse_attn_prefill.
 * --------------------------------------------------------------------------- */
dash_status dash_route(const void* Q, const void* K, const void* head_cls, const float* S,
                       dash_dtype dt, int B, int Hq, int Hkv, int Nq, int Lmax, int d,
                       int s_cap, const int* seqlens, dash_params p, float* tau,
                       uint32_t* active_bits, int bits_words, void* workspace,
                       size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace that dash_route and dash_sparse_attn_* need for these
 * sizes (decode = 1 for the seqlens mode). 0 for invalid sizes. Prefill: the
 * fixed part plus a pool of max(5, min(16, 2048 / ceil(Nq / 64))) pairs per
 * query row (16 up to Nq = 8192, 5 from Nq = 32768 on; the routed past chunks
 * per row at the 32K workload average about 3.4). */
size_t dash_workspace_size(int B, int Hq, int Hkv, int Nq, int Lmax, int d, int decode,
                           dash_params p);

/* Bytes of prefill workspace with a partial-result pool of exactly pool_pairs
 * (row, chunk) pairs; 0 for invalid sizes or pool_pairs outside
 * [0, 0xffffff00]. Tiles whose pairs do not fit the pool are attended by the
 * row-major kernel (correct, slower), so any pool size is valid: 0 sends every
 * tile there. A workspace smaller than the pool-free part is rejected with
 * DASH_ERR_WORKSPACE. */
size_t dash_prefill_workspace_size(int B, int Hq, int Hkv, int Nq, int Lmax, int d, dash_params p,
                                   long long pool_pairs);

/* Counters of the last prefill routing in `workspace` (same sizes, params and
 * ws_bytes as that dash_route call), written to out[0..3]: the (row, past
 * chunk) pairs placed in the partial-result pool, the pool's capacity, the
 * 128-row tiles the list-based routing kernel left to the general one, and
 * the tiles attended row-major (their pairs did not fit the pool). Copies
 * them to the host: the call synchronises `stream`. */
dash_status dash_prefill_counters(const void* workspace, size_t ws_bytes, int B, int Hq, int Hkv, int N,
                                  int d, dash_params p, long long* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * dash_sparse_attn_prefill -- stage 3, "Prior-induced sparse softmax" ("How it
 * works" 3) over rows 0 .. N-1:
 *   O_i = sum_j softmax_j(<q_i, k_j> / sqrt(d) + log w_{i, c(j)}) v_j
 * over the tokens j of the chunks routed to row i (j <= i when causal), w the
 * routing prior (1 for an always-attended own chunk). Reads the work that
 * dash_route (prefill mode, same sizes and params) left in `workspace` and
 * uses the rest of it for partial results. Every attended (row, chunk) pair is
 * computed chunk by chunk -- all pairs of a chunk share one pass over its keys
 * and values -- into a partial result (the log of its weight sum and its
 * normalised output), and each row's partials are then merged (the
 * online-softmax merge is exact in any order). Tiles of 128 rows whose pairs
 * did not fit the partial-result pool (its size set by ws_bytes, see
 * dash_route) are attended row by row instead, with each row's prior weights
 * recomputed from its tau, its routed-chunk bits and the summaries; their
 * results match up to rounding, so only then can two identical calls differ
 * in the last bits. ws_bytes must equal dash_route's: a workspace laid out for
 * another pool size is detected on the device and every row of O is set to
 * NaN.
 *   Q [B, Hq, N, d], K/V [B, Hkv, Lmax, d], O [B, Hq, N, d], all dtype dt.
 * --------------------------------------------------------------------------- */
dash_status dash_sparse_attn_prefill(const void* Q, const void* K, const void* V,
                                     dash_dtype dt, int B, int Hq, int Hkv, int N, int Lmax,
                                     int d, dash_params p, void* O, void* workspace,
                                     size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * dash_sparse_attn_prefill_backward -- gradients of the whole prefill
 * (dash_summarize -> dash_route -> dash_sparse_attn_prefill) for a cotangent dO
 * of O. The DashAttention README calls the router "adaptive, differentiable"
 * and has stage 3 use the stage-1 prior "to preserve differentiability through
 * the hierarchy" ("Documentation", "How it works" item 3); the steps are the
 * chain rule through the forward:
 *   attention: dP_ij = <dO_i, v_j>, dS_ij = P_ij (dP_ij - D_i) with
 *     D_i = sum_j P_ij dP_ij (recomputed exactly, not from a rounded output),
 *     dQ_i += sum_j dS_ij k_j / sqrt(d), dK_j += sum_i dS_ij q_i / sqrt(d),
 *     dV_j += sum_i P_ij dO_i;
 *   prior: g_ic = sum_{j in chunk c} dS_ij is the gradient of log pi_ic;
 *   routing (the entmax Jacobian over the row's support, s = pi^(2-alpha)):
 *     dz_ic = s_c g_ic / pi_ic - s_c (sum_c' s_c' g_ic' / pi_ic') / sum_c' s_c';
 *   scores z = scaling_factor <q, s_c> / sqrt(d): dQ_i and the summaries'
 *     gradients, and through dash_summarize's definition dK and head_cls (the
 *     own-chunk estimate's prefix summary likewise).
 * An own chunk attended with weight 1 (estimate_diagonal = 0) is not a routing
 * candidate and takes no routing gradient.
 *   Q, K, V, head_cls, S, tau, p, B, Hq, Hkv, N, Lmax, s_cap: exactly as given
 *       to the forward's dash_summarize / dash_route (prefill mode, rows
 *       0 .. N-1) / dash_sparse_attn_prefill;
 *   active_bits [B, Hq, N, bits_words]: dash_route's attended-chunk bits (the
 *       forward must be run with them);
 *   dO [B, Hq, N, d]: the cotangent of the forward's output;
 *   dQ [B, Hq, N, d], dK / dV [B, Hkv, Lmax, d]: written for rows < N (rows
 *       N .. Lmax-1 untouched), dtype dt; dcls [Hkv, d] float32, written.
 * The routing weights are recomputed from S, tau and the bits (a chunk the
 * forward routed whose recomputed score does not exceed tau, a last-bit
 * disagreement at the edge of the support, gets weight 0). Every sum has a
 * fixed order (deterministic). Device memory is the caller's, the scratch is
 * `workspace` (dash_backward_workspace_size bytes: about 2 * B * Hq * N *
 * ceil(N/64) * 4 + 3 * B * Hq * N * d * 4 bytes), nothing is allocated, no
 * host sync. Errors: NULL pointers, sizes <= 0, N > Lmax, Hq % Hkv != 0, bad
 * params, bits_words too small, s_cap below the summarised chunks ->
 * DASH_ERR_INVALID_ARG; dt other than DASH_BF16, d not 64 or 128, chunk_size != 64,
 * N > 65536 -> DASH_ERR_UNSUPPORTED; ws_bytes too small -> DASH_ERR_WORKSPACE;
 * a launch failure -> DASH_ERR_HIP.
 * --------------------------------------------------------------------------- */
dash_status dash_sparse_attn_prefill_backward(const void* Q, const void* K, const void* V,
                                              const void* head_cls, const float* S,
                                              const void* dO, const float* tau,
                                              const uint32_t* active_bits, int bits_words,
                                              dash_dtype dt, int B, int Hq, int Hkv, int N, int Lmax,
                                              int d, int s_cap, dash_params p, void* dQ, void* dK,
                                              void* dV, float* dcls, void* workspace,
                                              size_t ws_bytes, hipStream_t stream);

/* Bytes of workspace dash_sparse_attn_prefill_backward needs (0 for invalid sizes). */
size_t dash_backward_workspace_size(int B, int Hq, int Hkv, int N, int Lmax, int d, dash_params p);

/* ---------------------------------------------------------------------------
 * dash_sparse_attn_decode -- stage 3 for one new token per sequence, reading
 * only the routed chunks of the caches (prefill/decoding paragraph of "How it
 * works": decoding reuses the chunk-summary cache). Query row t_b =
 * seqlens[b] - 1. Split over the routed chunk list, then merged.
 *   Q [B, Hq, 1, d], Kc/Vc [B, Hkv, Lmax, d], O [B, Hq, 1, d], dtype dt.
 * Reads the lists that dash_route (decode mode) left in `workspace` and uses
 * the rest of it for per-split partial results.
 * --------------------------------------------------------------------------- */
dash_status dash_sparse_attn_decode(const void* Q, const void* Kc, const void* Vc,
                                    dash_dtype dt, int B, int Hq, int Hkv,
                                    const int* seqlens, int Lmax, int d, dash_params p,
                                    void* O, void* workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * dash_decode_step_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): one decode step, exactly dash_route in decode mode followed by
 * dash_sparse_attn_decode (same kernels, same results), with the workspace
 * taken from a scratch array that the library holds in device memory instead
 * of a caller buffer.
 *   Q, Kc, Vc, head_cls, S, seqlens, Lmax, s_cap, p: as for dash_route
 *   (decode mode, causal = 1) and dash_sparse_attn_decode.
 *   O [B, Hq, 1, d], tau [B, Hq, 1], active_bits (NULL or [B, Hq, 1,
 *   bits_words]): the outputs of those two calls.
 * The scratch holds dash_decode_noalloc_max_bytes() bytes (64 MiB) on every
 * GPU the library runs on, from the time it is loaded until the process ends;
 * sizes whose dash_workspace_size(B, Hq, Hkv, 1, Lmax, d, 1, p) exceeds it
 * return DASH_ERR_WORKSPACE before anything is launched. Nothing is allocated:
 * no hipMalloc/hipFree, on any call. Every call on one GPU uses that GPU's one
 * scratch array, so calls that overlap on one GPU (different streams or host
 * threads without ordering) race; calls ordered on one stream are safe. The
 * first call on a device looks up the scratch address (hipGetSymbolAddress)
 * with that device current. Errors: as dash_route and dash_sparse_attn_decode.
 * --------------------------------------------------------------------------- */
dash_status dash_decode_step_noalloc(const void* Q, const void* Kc, const void* Vc,
                                     const void* head_cls, const float* S, dash_dtype dt, int B,
                                     int Hq, int Hkv, const int* seqlens, int Lmax, int d,
                                     int s_cap, dash_params p, void* O, float* tau,
                                     uint32_t* active_bits, int bits_words, hipStream_t stream);

/* Size in bytes of the scratch array dash_decode_step_noalloc uses. */
size_t dash_decode_noalloc_max_bytes(void);

/* ---------------------------------------------------------------------------
 * entmax_attn -- dense alpha-entmax attention with block skipping (AdaSplash
 * "Usage": AdaSplash with Block Masking; "Key Features"). For each (b, h) and
 * row i < len_b (len_b = varlen[b], or Nmax when varlen is NULL):
 *   s_ij = <q_i, k_j> / sqrt(d) over j < len_b (and j <= i when causal),
 *   tau_i : sum_j ((alpha-1) s_ij - tau_i)_+^(1/(alpha-1)) = 1,
 *   O_i = sum_j ((alpha-1) s_ij - tau_i)_+^(1/(alpha-1)) v_j.
 * Rows i >= len_b get O = 0 and tau = 0.
 *   Q/K/V/O    [B, H, Nmax, d] dtype dt (DASH_F32 or DASH_BF16)
 *   varlen     [B] int32 on the device, 1 <= varlen[b] <= Nmax, or NULL
 *   tau        [B, H, Nmax] float32, in u units
 *   block_mask [B, H, nT, ceil(nT / 32)] uint32 or NULL, nT = ceil(Nmax / 64):
 *              bit J % 32 of word J / 32 of row-tile I is set iff the 64 x 64
 *              tile (I, J) holds a non-zero weight ("binary mask per block").
 *              Tiles that are all zero are skipped in the output pass.
 * n_iter bounds the tau iterations (Halley + bisection, "Triton Entmax").
 * --------------------------------------------------------------------------- */
dash_status entmax_attn(const void* Q, const void* K, const void* V, dash_dtype dt, int B,
                        int H, int Nmax, int d, const int* varlen, float alpha, int n_iter,
                        int causal, void* O, float* tau, uint32_t* block_mask,
                        hipStream_t stream);

/* ---------------------------------------------------------------------------
 * entmax_attn_backward -- gradients of entmax_attn (the AdaSplash README runs
 * its attention kernels forward and backward, "Usage", and lists block-sparse
 * forward and backward passes under "Key Features"; the entmax Jacobian is the
 * published one). For a cotangent dO of O, with t_ij = (alpha-1) s_ij - tau_i,
 * P_ij = max(t_ij, 0)^(1/(alpha-1)) and g_ij = P_ij^(2 - alpha) on the support:
 *   dP_ij = <dO_i, v_j>,   coef_i = sum_j g_ij dP_ij / sum_j g_ij,
 *   dS_ij = g_ij (dP_ij - coef_i),
 *   dQ_i = sum_j dS_ij k_j / sqrt(d),  dK_j = sum_i dS_ij q_i / sqrt(d),
 *   dV_j = sum_i P_ij dO_i.
 * Rows and keys at or past len_b get zero gradients.
 *   Q/K/V/dO       [B, H, Nmax, d] dtype dt, the forward's inputs and the cotangent
 *   tau            [B, H, Nmax] float32, the forward's tau output
 *   block_mask     the forward's block mask (tiles with bit 0 are skipped), or
 *                  NULL (every allowed tile is visited; same result)
 *   varlen, alpha, causal: as given to the forward
 *   dQ/dK/dV       [B, H, Nmax, d] dtype dt, written; must not overlap any input
 *   coef           [B, H, Nmax] float32 scratch written with coef_i (row terms
 *                  shared by the two kernels); caller-owned
 * All device memory owned by the caller; work enqueued on stream, no host sync,
 * nothing allocated. Errors: NULL pointers (other than varlen, block_mask), any
 * size <= 0, alpha not a finite value > 1, causal not 0/1 ->
 * DASH_ERR_INVALID_ARG; d not 64 or 128, Nmax > 65536 -> DASH_ERR_UNSUPPORTED;
 * a launch failure -> DASH_ERR_HIP.
 * --------------------------------------------------------------------------- */
dash_status entmax_attn_backward(const void* Q, const void* K, const void* V, const void* dO,
                                 const float* tau, const uint32_t* block_mask, dash_dtype dt,
                                 int B, int H, int Nmax, int d, const int* varlen, float alpha,
                                 int causal, void* dQ, void* dK, void* dV, float* coef,
                                 hipStream_t stream);

/* ---------------------------------------------------------------------------
 * entmax_rows -- row-wise alpha-entmax (AdaSplash README, "Usage": "Triton
 * Entmax (Optimized Entmax Activation)", the activation over the last
 * dimension with alpha and n_iter). For each row r < rows of X:
 *   u = (alpha - 1) x_r,
 *   tau_r : sum_j max(u_j - tau_r, 0)^(1/(alpha-1)) = 1   (Halley + bisection,
 *           at most n_iter steps),
 *   Y_r  = max(u - tau_r, 0)^(1/(alpha-1)), divided by its sum.
 * Entries equal to -inf get 0; a row with no finite entry gets Y = 0 and
 * tau = +inf.
 *   X, Y  [rows, n] row-major, dtype dt (DASH_F32 or DASH_BF16), device
 *         memory owned by the caller; Y may be X (each entry is read before
 *         it is written, by the same thread)
 *   tau   [rows] float32 on the device, in u units, or NULL
 * Errors: NULL X or Y, rows or n <= 0, alpha not a finite value > 1 or
 * n_iter < 1 -> DASH_ERR_INVALID_ARG; n > 32768 -> DASH_ERR_UNSUPPORTED; a
 * launch failure -> DASH_ERR_HIP. Nothing is allocated; no host sync.
 * --------------------------------------------------------------------------- */
dash_status entmax_rows(const void* X, void* Y, dash_dtype dt, int rows, int n, float alpha,
                        int n_iter, float* tau, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * entmax_rows_backward -- the gradient of entmax_rows with respect to its
 * scores (the AdaSplash README runs its entmax kernels forward and backward,
 * "Usage"; the Jacobian is the published one of alpha-entmax): for each row,
 *   g  = Y^(2 - alpha) where Y > 0, 0 elsewhere,
 *   dX = g * dY - g * (sum g * dY) / (sum g)      (dX = 0 for a row with Y = 0).
 *   Y   [rows, n] the forward's output, dtype dt (DASH_F32 or DASH_BF16)
 *   dY  [rows, n] the cotangent, dtype dt
 *   dX  [rows, n] dtype dt; may be dY or Y (each entry is read before it is
 *       written, by the same thread)
 * All device memory owned by the caller. Errors: NULL pointers, rows or n <= 0,
 * alpha not a finite value > 1 -> DASH_ERR_INVALID_ARG; n > 32768 ->
 * DASH_ERR_UNSUPPORTED; a launch failure -> DASH_ERR_HIP.
 * --------------------------------------------------------------------------- */
dash_status entmax_rows_backward(const void* Y, const void* dY, void* dX, dash_dtype dt, int rows,
                                 int n, float alpha, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* dash_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H_ */
