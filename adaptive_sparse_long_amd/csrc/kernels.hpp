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
// Partial-result pool of the chunk-major kernel: kCmSlots slots per query row
// on average. Every attended chunk of a row (its routed past chunks and its
// own chunk) is attended by the chunk-major kernel into a slot of its own, and
// the merge kernel combines the row's partials. A tile whose rows find the pool
// exhausted has all its chunks attended by the row-major kernel instead.
constexpr int kCmSlots = 16;
// Chunk-major work item: up to kCmBlocks blocks of 32 (row, chunk) pairs of one
// (b, kv head, chunk).
constexpr int kCmBlocks = 12;
// The partial-result pool is split into kPools equal parts, each with its own
// allocation counter (workgroup id modulo kPools picks the part).
constexpr int kPools = 8;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Prefill work lists, per (b, query head) and 128-row tile, each an ascending
// list of chunk ids:
//   row-major list ("rm", tiles without pool slots): every attended chunk, with
//     one log2 weight per row of the tile (-inf: not attended by that row);
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
// Per tile: its first pool slot (tbase). Per row: its first slot (rslot) and
// number of partials (cmcnt); a row's slots follow its attended chunks in
// ascending order. pool: the slot allocation counter. Per slot: the log2 of
// the partial's sum of exp2 weights (its max included) in float32 and its
// output normalised by that sum in fp16, dims in natural order.
// ---------------------------------------------------------------------------
struct PrefillLayout {
  int n_tiles = 0;
  int n_slots = 0;        // chunk slots = ceil(N / 64)
  long long per_head = 0; // list slots per (b, head)
  int n_bhc = 0;          // B * Hkv * n_slots
  long long max_items = 0;
  size_t off_counts = 0, off_lists = 0, off_bias = 0;          // row-major list
  size_t off_ccounts = 0, off_clists = 0, off_ceo = 0, off_cbase = 0;  // chunk-major list
  size_t off_cmp = 0, off_cs = 0, off_nitems = 0, off_items = 0, off_recs = 0, off_trec = 0;  // chunk-major pairs
  size_t off_pool = 0, off_tbase = 0, off_rslot = 0, off_cmcnt = 0, off_plse = 0, off_po = 0;  // partials
  size_t off_fb = 0, off_fb_count = 0;  // tiles left to the general routing kernel
  long long pool_cap = 0;
  size_t off_split = 0, total = 0;
  size_t off_serr = 0;  // per chunk: bound on |hi-only score - full score| / |q|
};

__host__ __device__ inline long long prefill_tile_offset(int tile, int n_slots, bool causal) {
  return causal ? (long long)tile * (tile + 1) : (long long)tile * n_slots;
}
__host__ __device__ inline int prefill_tile_cap(int tile, int n_slots, bool causal) {
  return causal ? min(n_slots, 2 * tile + 2) : n_slots;
}

// off_split: the summaries split into bf16 high and low parts, [B, Hkv, n_slots, d] each.
inline PrefillLayout prefill_layout(int B, int Hq, int Hkv, int N, int d, bool causal) {
  PrefillLayout L;
  L.n_tiles = (N + kTileRows - 1) / kTileRows;
  L.n_slots = (N + kChunk - 1) / kChunk;
  const int t = L.n_tiles - 1;
  L.per_head = prefill_tile_offset(t, L.n_slots, causal) + prefill_tile_cap(t, L.n_slots, causal);
  const size_t heads = (size_t)B * Hq;
  const size_t entries = heads * (size_t)L.per_head * kTileRows;
  const size_t rows = heads * (size_t)N;
  const size_t pairs = rows * kCmSlots;
  L.pool_cap = (long long)pairs;
  L.n_bhc = B * Hkv * L.n_slots;
  L.max_items = (long long)((pairs + 32 * kCmBlocks - 1) / (32 * kCmBlocks)) + L.n_bhc;
  size_t o = 0;
  L.off_counts = o;  o += align256(heads * L.n_tiles * sizeof(int));
  L.off_lists = o;   o += align256(heads * (size_t)L.per_head * sizeof(int));
  L.off_bias = o;    o += align256(entries * sizeof(float));
  L.off_ccounts = o; o += align256(heads * L.n_tiles * sizeof(int));
  L.off_clists = o;  o += align256(heads * (size_t)L.per_head * sizeof(int));
  L.off_ceo = o;     o += align256(heads * (size_t)L.per_head * 2 * sizeof(int));
  L.off_cbase = o;   o += align256(heads * (size_t)L.per_head * sizeof(int));
  L.off_cmp = o;     o += align256((size_t)L.n_bhc * sizeof(int));
  L.off_cs = o;      o += align256((size_t)L.n_bhc * sizeof(int));
  L.off_nitems = o;  o += align256(sizeof(int));
  L.off_items = o;   o += align256((size_t)L.max_items * 2 * sizeof(int));
  L.off_recs = o;    o += align256(pairs * 4 * sizeof(int));
  L.off_trec = o;    o += align256(pairs * 4 * sizeof(int));
  L.off_pool = o;    o += align256(kPools * sizeof(unsigned long long));
  L.off_tbase = o;   o += align256(heads * L.n_tiles * sizeof(uint32_t));
  L.off_fb = o;      o += align256(heads * L.n_tiles * 2 * sizeof(int));
  L.off_fb_count = o; o += align256(2 * sizeof(int));  // queued tiles, row-major tiles
  L.off_rslot = o;   o += align256(rows * sizeof(uint32_t));
  L.off_cmcnt = o;   o += align256(rows * sizeof(uint16_t));
  L.off_plse = o;    o += align256(pairs * sizeof(float));
  L.off_po = o;      o += align256(pairs * (size_t)d * sizeof(uint16_t));
  L.off_split = o;   o += align256((size_t)2 * B * Hkv * L.n_slots * d * sizeof(uint16_t));
  L.off_serr = o;    o += align256((size_t)B * Hkv * L.n_slots * sizeof(float));
  L.total = o;
  return L;
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
  float* bias;
  int* ccounts;
  int* clists;
  int2* ceo;
  int4* trec;
  int* cbase;
  int* cmp;  // zeroed by the summary split, counted by the routing
  int n_bhc;
  unsigned long long* pool;  // kPools counters, zeroed by the summary split
  long long pool_cap;
  uint32_t* tbase;
  uint32_t* rslot;
  uint16_t* cmcnt;
  int2* fb_tiles;   // tiles the list-based kernel left: (tile, b * Hq + h)
  int* fb_count;     // their number, zeroed by the summary split
  int* n_rm;         // tiles without pool slots (row-major), zeroed by the summary split
  // summaries split into bf16 high / low parts (prefill), [B, Hkv, n_slots, d] each
  uint16_t* s_hi;
  uint16_t* s_lo;
  // per chunk: |s_lo| + 2^-14 |s| (u units), so that |q| times it bounds the
  // difference between a score from the high parts alone and the full one
  float* s_err;
  // decode scratch
  float* z;
};

struct PrefillAttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  int B, Hq, Hkv, g, N, Lmax, causal;
  float scale_log2;
  int n_tiles, n_slots;
  long long per_head;
  const int* counts;
  const int* lists;
  const float* bias;
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
  const int* seqlens;
  float scale_log2;
  int n_slots, n_splits;
  const int* counts;
  const int* lists;
  const float* bias;
  float* part;
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

// Limits of the current kernels (checked by the host API).
constexpr int kRoutePrefillMaxSlots = 512;   // 32 blocks of 16 chunks in registers
constexpr int kRouteCap = 128;               // routing candidates per row held in LDS
constexpr int kRouteListCap = 5120;          // LDS list words per tile: candidates, then 1024 for the chunk entries
constexpr int kRouteDecodeMaxComplete = 4096; // 64 per lane
constexpr int kEntmaxMaxTiles = 1024;        // candidate-tile bitmask per wavefront
constexpr int kEntmaxCap = 16;               // candidate scores per lane in the single-pass kernel
constexpr int kEntmaxRowsMax = 32768;        // row-wise entmax: 32 entries per thread of 1024

}  // namespace dash
