// kernels.hpp -- launch arguments, workspace layouts and launcher declarations
// shared by the HIP kernels and the host API (api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cdna4.hpp"

namespace dash {

// Query rows per prefill workgroup (four wavefronts of 32 rows) and keys per chunk.
constexpr int kTileRows = 128;
constexpr int kChunk = 64;
// Routed chunks handled by one decode split (one workgroup, four wavefronts).
constexpr int kDecodeSplit = 24;
// Partial-result pool of the chunk-major kernel: one slot per (row, routed
// past chunk) pair. Every routed past chunk of a row is attended by the
// chunk-major kernel into a slot of its own; the merge kernel attends the row's
// own chunk (causal) and combines it with the row's partials. A tile whose rows
// find the pool exhausted has all its chunks attended by the row-major kernel
// instead. The pool takes whatever the caller's workspace holds beyond the
// fixed part; the workspace query sizes it to kCmSlotsMax pairs per row at
// short lengths, shrinking to kCmSlotsMin at long ones.
constexpr int kCmSlotsMax = 16;
constexpr int kCmSlotsMin = 5;
// Chunk-major work item: up to kCmBlocks blocks of 32 (row, chunk) pairs of one
// (b, kv head, chunk).
constexpr int kCmBlocks = 24;
// The partial-result pool is split into kPools equal parts, each with its own
// allocation counter (workgroup id modulo kPools picks the part).
constexpr int kPools = 8;
// Beyond 512 chunk slots the general routing kernel keeps its scores in a
// global scratch: kRouteGlbGrid workgroups walk the queued tiles, each with
// its own part (eight wavefronts x up to 128 blocks x 4 x 64 floats).
constexpr int kRouteGlbGrid = 256;
inline size_t route_glb_scratch_bytes(int n_slots) {
  if (n_slots <= 512) return 0;
  const size_t nb = n_slots <= 1024 ? 64 : 128;
  return (size_t)kRouteGlbGrid * 8 * nb * 4 * 64 * sizeof(float);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Head dimension. The DashAttention kernels are laid out for 128 dims; at
// head_dim 64 they run the same layouts with dims 64..127 zero: the caller's
// rows (Q, K, V, head_cls, the summary cache, O) are d elements wide, every
// load of them goes through the helpers below (zeros at and past d, which leave
// dot products, softmax sums and scores unchanged) and every store of O or S
// writes dims below d only. The kernels' own arrays (split summaries, partial
// results) stay 128 wide.
// ---------------------------------------------------------------------------
constexpr int kDashD = 128;
inline bool dash_head_dim_ok(int d) { return d == 64 || d == 128; }
// 8 bf16 at element col (a multiple of 8, below 128) of row `row` of d-wide
// rows. The load itself always goes to col modulo d (inside the row: d is a
// power of two) and is then zeroed past d, so that no load is predicated.
__device__ __forceinline__ u32x4 ldg16_d(const uint16_t* base, size_t row, int col, int d) {
  const u32x4 v = ldg16(base + row * (size_t)d + (col & (d - 1)));
  return col < d ? v : u32x4{0, 0, 0, 0};
}
// The same with the head_dim a compile-time constant (no test at d = 128).
template <int DC>
__device__ __forceinline__ u32x4 ldg16_dc(const uint16_t* base, size_t row, int col) {
  if constexpr (DC == kDashD) {
    return ldg16(base + row * (size_t)DC + col);
  } else {
    const u32x4 v = ldg16(base + row * (size_t)DC + (col & (DC - 1)));
    return col < DC ? v : u32x4{0, 0, 0, 0};
  }
}
template <int DC>
__device__ __forceinline__ f32x4 ldf4_dc(const float* base, size_t row, int col) {
  if constexpr (DC == kDashD) {
    return *reinterpret_cast<const f32x4*>(base + row * (size_t)DC + col);
  } else {
    const f32x4 v = *reinterpret_cast<const f32x4*>(base + row * (size_t)DC + (col & (DC - 1)));
    return col < DC ? v : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}
// 4 bf16 at element col (a multiple of 4)
__device__ __forceinline__ u32x2 ldg8_d(const uint16_t* base, size_t row, int col, int d) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(base + row * (size_t)d + (col & (d - 1)));
  return col < d ? v : u32x2{0, 0};
}
// 4 floats at element col (a multiple of 4)
__device__ __forceinline__ f32x4 ldf4_d(const float* base, size_t row, int col, int d) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(base + row * (size_t)d + (col & (d - 1)));
  return col < d ? v : f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------
// Prefill work lists, per (b, query head) and 128-row tile, each an ascending
// list of chunk ids:
//   row-major list ("rm", tiles without pool slots): every attended chunk; the
//     row-major kernel recomputes each row's prior weight for a listed chunk
//     from the row's tau and routed-chunk bits (rm_tau, rm_bits, written by the
//     routing for these tiles only) and the split summaries;
//   chunk-major list ("cm", tiles with pool slots): every attended chunk, with
//     the (row, chunk) pair records of the rows attending it -- (row * g + head
//     in group, pool slot, log2 weight) -- grouped by chunk in the tile's own
//     pool range (trec, at [tbase + first, + count) for list entry e, (first,
//     count) in ceo).
// Causal tile t can only list chunks 0 .. 2t+1, so tiles are packed in a
// triangle: tile t starts at slot t*(t+1). Non-causal tiles hold n_slots each.
// Per chunk-major list entry: the offset of its pairs among all pairs of its
// chunk (cbase, reserved by the routing). Per (b, kv head, chunk) "bhc": the
// number of its pairs (cmp) and their start in the chunk-sorted pair records
// (cs). Work items list (bhc, first block); recs hold one pair each.
// Per tile: its first pool slot (tbase). Per row: its first slot (rslot), its
// number of partials (cmcnt) and the log2 weight of its own chunk (own_lw,
// causal; -inf when not attended); a row's slots follow its routed past
// chunks in ascending order. pool: kPools slot allocation counters, then the
// pool capacity the routing laid the workspace out for (checked by the
// attention call, which must be given the same workspace size). Per slot: the
// log2 of the partial's sum of exp2 weights (its max included) in float32 and
// its output normalised by that sum in fp16, dims in natural order. qhead: the
// chunk-major kernel's work queue head; bad: set when the attention call finds
// a pool capacity other than the routing's.
// The per-slot arrays (and the work items, whose number follows the pool) come
// last, so that everything before them depends on the shapes alone.
// ---------------------------------------------------------------------------
struct PrefillLayout {
  int n_tiles = 0;
  int n_slots = 0;        // chunk slots = ceil(N / 64)
  int words = 0;          // bitmask words per row = ceil(n_slots / 32)
  long long per_head = 0; // list slots per (b, head)
  int n_bhc = 0;          // B * Hkv * n_slots
  long long max_items = 0;
  size_t off_counts = 0, off_lists = 0;                                // row-major list
  size_t off_ccounts = 0, off_clists = 0, off_ceo = 0, off_cbase = 0;  // chunk-major list
  size_t off_cmp = 0, off_cs = 0, off_nitems = 0;                      // chunk-major pairs
  size_t off_pool = 0, off_tbase = 0, off_rslot = 0, off_cmcnt = 0;    // slots
  size_t off_fb = 0, off_fb_count = 0;  // tiles left to the general routing kernel
  size_t off_own = 0, off_qhead = 0, off_rmtau = 0, off_rmbits = 0;
  size_t off_split = 0;
  size_t off_serr = 0;  // per chunk: bound on |hi-only score - full score| / |q|
  size_t off_gscr = 0;  // scores of the general routing kernel beyond 512 chunk slots
  size_t off_items = 0, off_recs = 0, off_trec = 0, off_plse = 0, off_po = 0;  // per pool slot
  long long pool_cap = 0;
  size_t fixed = 0, total = 0;
};

__host__ __device__ inline long long prefill_tile_offset(int tile, int n_slots, bool causal) {
  return causal ? (long long)tile * (tile + 1) : (long long)tile * n_slots;
}
__host__ __device__ inline int prefill_tile_cap(int tile, int n_slots, bool causal) {
  return causal ? min(n_slots, 2 * tile + 2) : n_slots;
}

// Pool slots are 32-bit indices.
constexpr long long kPoolMaxPairs = 0xffffff00ll;

// off_split: the summaries split into bf16 high and low parts, [B, Hkv, n_slots, d] each.
inline PrefillLayout prefill_layout(int B, int Hq, int Hkv, int N, int d, bool causal, long long pool_pairs) {
  PrefillLayout L;
  L.n_tiles = (N + kTileRows - 1) / kTileRows;
  L.n_slots = (N + kChunk - 1) / kChunk;
  L.words = (L.n_slots + 31) / 32;
  const int t = L.n_tiles - 1;
  L.per_head = prefill_tile_offset(t, L.n_slots, causal) + prefill_tile_cap(t, L.n_slots, causal);
  const size_t heads = (size_t)B * Hq;
  const size_t rows = heads * (size_t)N;
  const size_t pairs = (size_t)(pool_pairs < 0 ? 0 : pool_pairs);
  L.pool_cap = (long long)pairs;
  L.n_bhc = B * Hkv * L.n_slots;
  L.max_items = (long long)((pairs + 32 * kCmBlocks - 1) / (32 * kCmBlocks)) + L.n_bhc;
  size_t o = 0;
  L.off_counts = o;  o += align256(heads * L.n_tiles * sizeof(int));
  L.off_lists = o;   o += align256(heads * (size_t)L.per_head * sizeof(int));
  L.off_ccounts = o; o += align256(heads * L.n_tiles * sizeof(int));
  L.off_clists = o;  o += align256(heads * (size_t)L.per_head * sizeof(int));
  L.off_ceo = o;     o += align256(heads * (size_t)L.per_head * 2 * sizeof(int));
  L.off_cbase = o;   o += align256(heads * (size_t)L.per_head * sizeof(int));
  L.off_cmp = o;     o += align256((size_t)L.n_bhc * sizeof(int));
  L.off_cs = o;      o += align256((size_t)L.n_bhc * sizeof(int));
  L.off_nitems = o;  o += align256(sizeof(int));
  L.off_pool = o;    o += align256((kPools + 1) * sizeof(unsigned long long));
  L.off_tbase = o;   o += align256(heads * L.n_tiles * sizeof(uint32_t));
  L.off_fb = o;      o += align256(heads * L.n_tiles * 2 * sizeof(int));
  L.off_fb_count = o; o += align256(2 * sizeof(int));  // queued tiles, row-major tiles
  L.off_rslot = o;   o += align256(rows * sizeof(uint32_t));
  L.off_cmcnt = o;   o += align256(rows * sizeof(uint16_t));
  L.off_own = o;     o += align256(rows * sizeof(float));
  L.off_qhead = o;   o += align256(2 * sizeof(int));  // queue head, bad
  L.off_rmtau = o;   o += align256(rows * sizeof(float));
  L.off_rmbits = o;  o += align256(rows * L.words * sizeof(uint32_t));
  L.off_split = o;   o += align256((size_t)2 * B * Hkv * L.n_slots * d * sizeof(uint16_t));
  L.off_serr = o;    o += align256((size_t)B * Hkv * L.n_slots * sizeof(float));
  L.off_gscr = o;    o += align256(route_glb_scratch_bytes(L.n_slots));
  L.fixed = o;
  L.off_items = o;   o += align256((size_t)L.max_items * 2 * sizeof(int));
  L.off_recs = o;    o += align256(pairs * 4 * sizeof(int));
  L.off_trec = o;    o += align256(pairs * 4 * sizeof(int));
  L.off_plse = o;    o += align256(pairs * sizeof(float));
  L.off_po = o;      o += align256(pairs * (size_t)d * sizeof(uint16_t));
  L.total = o;
  return L;
}

// Pool pairs the workspace query provides: 2048 / n_slots per row, within
// [kCmSlotsMin, kCmSlotsMax] (16 up to N = 8192, 5 from N = 32768 on).
inline long long prefill_default_pairs(int B, int Hq, int N) {
  const int n_slots = (N + kChunk - 1) / kChunk;
  int per_row = 2048 / n_slots;
  if (per_row > kCmSlotsMax) per_row = kCmSlotsMax;
  if (per_row < kCmSlotsMin) per_row = kCmSlotsMin;
  const long long p = (long long)B * Hq * N * per_row;
  return p < kPoolMaxPairs ? p : kPoolMaxPairs;
}

// The largest pool a workspace of ws_bytes holds (-1: not even the fixed part
// fits). Deterministic in its arguments, so the routing and the attention call
// agree when given the same workspace size.
inline long long prefill_pool_from_bytes(int B, int Hq, int Hkv, int N, int d, bool causal, size_t ws_bytes) {
  const PrefillLayout L0 = prefill_layout(B, Hq, Hkv, N, d, causal, 0);
  if (ws_bytes < L0.total) return -1;
  const size_t per_pair = 36 + 2 * (size_t)d + 1;
  long long p = (long long)((ws_bytes - L0.total) / per_pair);
  if (p > kPoolMaxPairs) p = kPoolMaxPairs;
  while (p > 0 && prefill_layout(B, Hq, Hkv, N, d, causal, p).total > ws_bytes) p -= p / 4096 + 1;
  return p;
}

// ---------------------------------------------------------------------------
// Decode workspace, per (b, kv head) group of g query heads: routing scores of
// every query head, the union list of routed chunks, g log2 weights per listed
// chunk, and per-split partial results (max, sum, unnormalised output).
// ---------------------------------------------------------------------------
struct DecodeLayout {
  int n_slots = 0;   // ceil(Lmax / 64): chunk slots, own chunk included
  int n_splits = 0;  // ceil(n_slots / kDecodeSplit)
  int g = 0;
  size_t off_z = 0, off_counts = 0, off_lists = 0, off_bias = 0, off_part = 0, total = 0;
};

inline DecodeLayout decode_layout(int B, int Hq, int Hkv, int Lmax, int d) {
  DecodeLayout L;
  L.g = Hq / Hkv;
  L.n_slots = (Lmax + kChunk - 1) / kChunk;
  L.n_splits = (L.n_slots + kDecodeSplit - 1) / kDecodeSplit;
  const size_t groups = (size_t)B * Hkv;
  L.off_z = 0;
  L.off_counts = align256((size_t)B * Hq * L.n_slots * sizeof(float));
  L.off_lists = L.off_counts + align256(groups * sizeof(int));
  L.off_bias = L.off_lists + align256(groups * L.n_slots * sizeof(int));
  L.off_part = L.off_bias + align256(groups * L.n_slots * L.g * sizeof(float));
  L.total = L.off_part + align256(groups * L.n_splits * L.g * (size_t)(d + 2) * sizeof(float));
  return L;
}

// --------------------------------------------------------------------------- args
struct SummarizeArgs {
  const void* K;
  const void* cls;
  float* S;
  int B, Hkv, Lmax, d, n_tokens;
  const int* seqlens;
  int chunk_begin, chunk_end, s_cap, C;
  float inv_sqrt_d;
};

struct SummarizeBwdArgs {
  const void* K;
  const void* cls;
  const float* dS;   // [B, Hkv, s_cap, d] cotangent of the summaries
  float* dK;         // [B, Hkv, Lmax, d]
  float* dcls;       // [Hkv, d]
  float* partials;   // [B, Hkv, chunk_end - chunk_begin, d]
  int B, Hkv, Lmax, d, n_tokens;
  int chunk_begin, chunk_end, s_cap, C;
  float inv_sqrt_d;
};

struct RouteArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* cls;
  const float* S;
  int B, Hq, Hkv, g, Nq, Lmax, d, s_cap;
  const int* seqlens;
  float alpha, beta, zscale, inv_sqrt_d;
  int n_iter, causal, est;
  float* tau;
  uint32_t* bits;
  int bits_words;
  // prefill lists (row-major and chunk-major, see PrefillLayout)
  int n_tiles, n_slots;
  long long per_head;
  int* counts;
  int* lists;
  float* bias;       // decode: g log2 weights per listed chunk
  int* ccounts;
  int* clists;
  int2* ceo;
  int4* trec;
  int* cbase;
  int* cmp;  // zeroed by the summary split, counted by the routing
  int n_bhc;
  unsigned long long* pool;  // kPools counters, zeroed by the summary split, then the capacity
  long long pool_cap;
  uint32_t* tbase;
  uint32_t* rslot;
  uint16_t* cmcnt;
  float* own_lw;     // per row: log2 weight of its own chunk (causal)
  float* rm_tau;     // per row of a row-major tile: tau
  uint32_t* rm_bits; // per row of a row-major tile: routed past chunks, rm_words words
  int rm_words;
  int2* fb_tiles;   // tiles the list-based kernel left: (tile, b * Hq + h)
  int* fb_count;     // their number, zeroed by the summary split
  int* n_rm;         // tiles without pool slots (row-major), zeroed by the summary split
  // summaries split into bf16 high / low parts (prefill), [B, Hkv, n_slots, d] each
  uint16_t* s_hi;
  uint16_t* s_lo;
  // per chunk: |s_lo| + 2^-14 |s| (u units), so that |q| times it bounds the
  // difference between a score from the high parts alone and the full one
  float* s_err;
  float* gscr;  // general kernel's score scratch beyond 512 chunk slots
  // decode scratch
  float* z;
};

struct PrefillAttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  int B, Hq, Hkv, g, N, Lmax, causal;
  int d;  // the caller's head_dim (row width of Q, K, V, O): 64 or 128
  float scale_log2;
  int n_tiles, n_slots;
  long long per_head;
  const int* counts;
  const int* lists;
  // row-major part: per row tau and routed-chunk bits, the split summaries
  // (u units), alpha as beta = 1 / (alpha - 1)
  const float* rm_tau;
  const uint32_t* rm_bits;
  int rm_words;
  const uint16_t* s_hi;
  const uint16_t* s_lo;
  float beta;
  // chunk-major part
  const int* ccounts;
  const int* clists;
  const int2* ceo;
  const int4* trec;
  const int* cbase;
  const int* cmp;
  int* cs;
  int* nitems;
  int2* items;
  int4* recs;
  int n_bhc;
  long long max_items, pool_cap;
  int n_cu;
  const uint32_t* tbase;
  const uint32_t* rslot;
  const uint16_t* cmcnt;
  const float* own_lw;
  int* qhead;       // work queue head of the chunk-major kernel
  int* bad;         // set: the workspace was laid out for another pool capacity
  const unsigned long long* pool;  // the routing's counters and capacity
  const int* n_rm;  // tiles the routing left row-major
  float* plse;
  uint16_t* po;
};

struct DecodeAttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  int B, Hq, Hkv, g, Lmax;
  int d;  // the caller's head_dim: 64 or 128
  const int* seqlens;
  float scale_log2;
  int n_slots, n_splits;
  const int* counts;
  const int* lists;
  const float* bias;
  float* part;
};

// ---------------------------------------------------------------------------
// DashAttention prefill backward. Column-layout per-(row, chunk) arrays are
// [B, Hq, n_slots, N] (the rows of one chunk contiguous).
// ---------------------------------------------------------------------------
struct DashBwdLayout {
  int n_slots = 0, n_sum = 0;  // chunk slots; chunks whose summaries the routing read
  size_t off_wt = 0, off_dzt = 0, off_lse = 0, off_dd = 0, off_dqf = 0, off_dkf = 0, off_dsum = 0;
  size_t off_dks = 0, off_sbp = 0, off_dcs = 0, off_dcp = 0, total = 0;
};

inline DashBwdLayout dash_bwd_layout(int B, int Hq, int Hkv, int N, int Lmax, int d, bool causal) {
  DashBwdLayout L;
  L.n_slots = (N + kChunk - 1) / kChunk;
  L.n_sum = causal ? N / kChunk : L.n_slots;
  const size_t rows = (size_t)B * Hq * N;
  size_t o = 0;
  L.off_wt = o;   o += align256(rows * L.n_slots * sizeof(float));
  L.off_dzt = o;  o += align256(rows * L.n_slots * sizeof(float));
  L.off_lse = o;  o += align256(rows * sizeof(float));
  L.off_dd = o;   o += align256(rows * sizeof(float));
  L.off_dqf = o;  o += align256(rows * d * sizeof(float));
  L.off_dkf = o;  o += align256((size_t)B * Hkv * N * d * sizeof(float));
  L.off_dsum = o; o += align256((size_t)B * Hkv * L.n_slots * d * sizeof(float));
  L.off_dks = o;  o += align256((size_t)B * Hkv * Lmax * d * sizeof(float));
  L.off_sbp = o;  o += align256((size_t)B * Hkv * (L.n_sum > 0 ? L.n_sum : 1) * d * sizeof(float));
  L.off_dcs = o;  o += align256((size_t)Hkv * d * sizeof(float));
  L.off_dcp = o;  o += align256((size_t)B * Hkv * L.n_slots * d * sizeof(float));
  L.total = o;
  return L;
}

struct DashBwdArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* dO;
  const uint16_t* cls;
  const float* S;          // [B, Hkv, s_cap, d] summaries the forward routed against
  const float* tau;        // [B, Hq, N]
  const uint32_t* bits;    // [B, Hq, N, bits_words] attended chunks
  int bits_words;
  int B, Hq, Hkv, g, N, Lmax, s_cap, n_slots, n_sum;
  int d;             // head_dim (64 or 128): the width of every row above and below
  int causal, est;
  float alpha, beta;
  float uscale;      // (alpha - 1) * scaling_factor / sqrt(d): u per <q, s>
  float rt;          // scaling_factor / sqrt(d): z per <q, s>
  float sf;          // scaling_factor
  float scale_log2;  // log2(e) / sqrt(d)
  float inv_sqrt_d;
  float* WT;      // log2 weights, column layout (-inf: not attended)
  float* DZT;     // gradients of the routing scores z, column layout
  float* lse;     // [B, Hq, N] log2 of the row's softmax normaliser (exp2 domain)
  float* Dd;      // [B, Hq, N] sum_j P_ij dP_ij
  float* dQf;     // [B, Hq, N, d]
  float* dKf;     // [B, Hkv, N, d] attention (and own-chunk estimate) part of dK
  float* dSum;    // [B, Hkv, n_slots, d] gradients of the summaries
  float* dKs;     // [B, Hkv, Lmax, d] summary part of dK
  float* sb_part; // summary backward scratch
  float* dcls_s;  // [Hkv, d] summary part of dcls
  float* dcls_p;  // [B, Hkv, n_slots, d] own-chunk estimate part of dcls, per chunk
  void* dQ;
  void* dK;
  void* dV;
  float* dcls;
};

struct EntmaxAttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int B, H, N, d;
  const int* varlen;
  float alpha, beta, scale;  // scale = (alpha - 1) / sqrt(d)
  int n_iter, causal;
  float* tau;
  uint32_t* mask;
  int mask_words;
  int only_marked;  // general kernel: only row blocks a row of which has tau = NaN
};

struct EntmaxBwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const float* tau;
  const uint32_t* mask;  // or nullptr
  int mask_words;
  int B, H, N, d;
  const int* varlen;
  float alpha, beta, scale;  // scale = (alpha - 1) / sqrt(d)
  float inv_sqrt_d;
  int causal;
  void* dQ;
  void* dK;
  void* dV;
  float* coef;  // [B, H, N] row terms sum(g dP) / sum(g)
};

struct EntmaxRowsArgs {
  const void* X;      // forward: scores; backward: the forward's output Y
  const void* dY;     // backward only: the cotangent (nullptr: forward)
  void* Y;            // forward: probabilities; backward: dX
  long long rows;
  int n;
  float alpha, beta;  // beta = 1 / (alpha - 1)
  int n_iter;
  float* tau;  // or nullptr
  int n_cu;    // sizes the grid-stride grid
};

hipError_t launch_summarize(const SummarizeArgs& a, hipStream_t stream);
hipError_t launch_summarize_bwd(const SummarizeBwdArgs& a, hipStream_t stream);
hipError_t launch_route_prefill(const RouteArgs& a, hipStream_t stream);
hipError_t launch_route_decode(const RouteArgs& a, hipStream_t stream);
hipError_t launch_sparse_prefill(const PrefillAttnArgs& a, hipStream_t stream);  // plan, scatter, chunk-major, row-major + merge
hipError_t launch_sparse_decode(const DecodeAttnArgs& a, hipStream_t stream);
hipError_t launch_entmax_attn(const EntmaxAttnArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_entmax_rows(const EntmaxRowsArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_entmax_attn_bwd(const EntmaxBwdArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_dash_bwd(const DashBwdArgs& a, hipStream_t stream);

// Limits of the current kernels (checked by the host API).
constexpr int kPrefillMaxSlots = 2048;       // prefill: N <= 131072
constexpr int kRouteRegSlots = 512;          // general routing kernel: scores in registers (32 blocks of 16 chunks)
constexpr int kRouteCap = 128;               // routing candidates per row held in LDS
constexpr int kRouteDecodeMaxComplete = 4096; // 64 per lane
constexpr int kEntmaxMaxTiles = 1024;        // candidate-tile bitmask per wavefront
constexpr int kEntmaxCap = 16;               // candidate scores per lane in the single-pass kernel
constexpr int kEntmaxRowsMax = 32768;        // row-wise entmax: 32 entries per thread of 1024
constexpr int kDashBwdMaxSlots = 1024;       // DashAttention backward: chunk slots per row (N <= 65536)

}  // namespace dash
