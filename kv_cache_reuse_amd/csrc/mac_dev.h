// Device-side definitions shared by the libmac kernels (gfx950).
//
// Contents: bf16 conversion, the 16-token KV tile permutation, the ring and
// workspace layouts, and the split-K plan that the attention and merge
// kernels derive identically from the match results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mac {

constexpr int kTile = 16;        // tokens per KV tile (= page size when paged)
constexpr int kSliceMin = 64;    // fewest keys a split-K slice is given (4 tiles)
constexpr int kMaxSlices = 1024; // most split-K slices per KV group
constexpr int kMaxGroup = 16;    // query heads per KV head: the MFMA N width
constexpr int kMergeCap = 2048;  // most (query head, slice) pairs one merge holds
// Wide groups (bf16 caches, more than kMaxGroup query heads per KV head) are
// matched in a launch of their own and attended in groups of at most
// kWideGroup heads, two matrix-core column tiles per key fragment.
constexpr int kWideGroup = 32;
constexpr int kMergeCapWide = 8192;

// Cache policy of the KV tile loads, the cache-policy operand of the buffer
// load instruction: kKeep, the default; kStream, non-temporal (the "nt"
// bit: lines are not kept for reuse), for keys a step streams once.
constexpr std::integral_constant<int, 0> kKeep{};
constexpr std::integral_constant<int, 2> kStream{};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Instantiate FN(T, D) for the (dtype, head_dim) pairs the library builds.
#define MAC_DISPATCH(dtype, d, FN)                                         \
  do {                                                                     \
    if ((dtype) == 1 && (d) == 128) { FN(uint16_t, 128); }                 \
    else if ((dtype) == 1 && (d) == 64) { FN(uint16_t, 64); }              \
    else if ((dtype) == 0 && (d) == 128) { FN(float, 128); }               \
    else { FN(float, 64); }                                                \
  } while (0)

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round to nearest, ties to even (IEEE 754 binary32 -> bfloat16); NaN stays
// a NaN.  gfx950 converts in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// 2^x with one v_exp_f32: results below the smallest normal flush to 0,
// 2^-inf = 0.  The attention and the merge only take it of x <= 0 or of
// differences of maxima.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazy rescaling threshold of the step kernels' online softmax, log2 units:
// a head's reference maximum moves only when a score passes it by more than
// this, so a weight exp2(s - m) stays below 2^8.
constexpr float kLazyRescale = 8.f;

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f(float x) { return x; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static float to_f(uint16_t x) { return bf16_to_f32(x); }
};

// ---------------------------------------------------------- KV tiles ----
// A tile holds 16 tokens x D elements of one (sequence, KV head).  Its bytes
// are split into 1 KiB blocks; lane l of a wave reads bytes [16 l, 16 l + 16)
// of block j with one 128-bit load.  Let E = 16 / sizeof(T) be the elements
// of one such 16-byte piece, lg = l / 16 and c = l % 16.
//
// Keys: lane (lg, c) of block j holds token c, dims [E (4 j + lg), +E): the
//   A operand (rows = tokens, k = dims) of the QK^T matrix-core product.
// Values: lane (lg, c) of block i holds tokens 4 lg .. 4 lg + 3 of dim c of
//   E/4 consecutive 16-dim column tiles (ct = (E/4) i + th): the A operand
//   (rows = dims, k = tokens) of the O^T = V^T P^T product, whose k index
//   (tokens 4 lg + r) matches the row order of the QK^T accumulator.
template <typename T>
__host__ __device__ __forceinline__ int k_tile_offset(int tok, int dim) {
  constexpr int E = 16 / sizeof(T);
  const int piece = dim / E, e = dim % E;
  const int j = piece / 4, lg = piece % 4;
  return j * (64 * E) + (lg * 16 + tok) * E + e;
}

template <typename T>
__host__ __device__ __forceinline__ int v_tile_offset(int tok, int dim) {
  constexpr int E = 16 / sizeof(T);
  constexpr int TP = E / 4;               // column tiles per 16-byte piece
  const int ct = dim / 16, c = dim % 16;
  const int i = ct / TP, th = ct % TP;
  const int lg = tok / 4, r = tok % 4;
  return i * (64 * E) + (lg * 16 + c) * E + th * 4 + r;
}

// Natural (row) layout, kv_layout = 1: element (token, dim) of a 16-token
// tile at token * D + dim, the caller's [..][tokens][d] rows as they are.
template <typename T>
__host__ __device__ __forceinline__ int kv_row_offset(int tok, int dim, int d) {
  return tok * d + dim;
}

struct KvGeom {
  int hkv, d;
  int ctx_stride;        // contiguous: token rows per (sequence, KV head)
                         // (tiles: 16 * ceil(max_context / 16); rows: max_context)
  int paged;             // 1: tile t of sequence b is page_table[b*mp + t]
  int max_pages;         // paged: page-table columns
  int n_pages;           // paged: pages in the pool
  int capacity;          // keys per sequence
  int natural;           // 1: rows in natural order (kv_layout 1), else tiles
};

// Element offsets of (token, dim) inside a tile, for either layout.
template <typename T>
__host__ __device__ __forceinline__ int k_elem_offset(const KvGeom& g, int tok, int dim) {
  return g.natural ? kv_row_offset<T>(tok, dim, g.d) : k_tile_offset<T>(tok, dim);
}
template <typename T>
__host__ __device__ __forceinline__ int v_elem_offset(const KvGeom& g, int tok, int dim) {
  return g.natural ? kv_row_offset<T>(tok, dim, g.d) : v_tile_offset<T>(tok, dim);
}

// Page of tile t of sequence b; -1 if the table entry is outside the pool.
__device__ __forceinline__ int64_t page_of(const KvGeom& g, const int32_t* pt, int b, int t) {
  const int32_t page = pt[int64_t(b) * g.max_pages + t];
  return (page >= 0 && page < g.n_pages) ? page : -1;
}

// Element offset of the start of tile t of (b, g) for reading.  A page-table
// entry outside the pool is clamped into it, so a corrupt table gives wrong
// values but never an out-of-bounds access.
__device__ __forceinline__ int64_t tile_base(const KvGeom& g, const int32_t* pt,
                                             int b, int kvh, int t) {
  const int64_t tile_elems = int64_t(kTile) * g.d;
  if (g.paged) {
    int64_t page = page_of(g, pt, b, t);
    if (page < 0) page = 0;
    return (page * g.hkv + kvh) * tile_elems;
  }
  return ((int64_t(b) * g.hkv + kvh) * g.ctx_stride + int64_t(t) * kTile) * g.d;
}

// Token rows of tile t that lie inside the cache: 16, except for the last
// tile of a contiguous natural-layout cache whose max_context is not a
// multiple of 16 (the rows after it belong to the next KV head).
__device__ __forceinline__ int tile_rows(const KvGeom& g, int t) {
  if (!g.natural || g.paged) return kTile;
  const int r = g.ctx_stride - t * kTile;
  return r < kTile ? (r > 0 ? r : 0) : kTile;
}

// Element offset of tile t of (b, g) for writing, or -1 when position
// t * 16 is not writable (past the capacity or an invalid page): writes there
// are dropped instead of landing outside the cache.
__device__ __forceinline__ int64_t tile_base_w(const KvGeom& g, const int32_t* pt,
                                               int b, int kvh, int t) {
  if (t < 0 || int64_t(t) * kTile >= g.capacity) return -1;
  const int64_t tile_elems = int64_t(kTile) * g.d;
  if (g.paged) {
    const int64_t page = page_of(g, pt, b, t);
    return page < 0 ? -1 : (page * g.hkv + kvh) * tile_elems;
  }
  return ((int64_t(b) * g.hkv + kvh) * g.ctx_stride + int64_t(t) * kTile) * g.d;
}

// --------------------------------------------------------------- ring ----
// Per (b, h): a push counter and W + 1 slots.  Slot of the k-th most recent
// entry (k = 0 newest) is (count - 1 - k) mod (W + 1); a push writes slot
// count mod (W + 1), which is never one of the W entries a step can match.
struct RingView {
  int32_t* count;   // [batch*Hq]
  void* q;          // [batch*Hq][W+1][D] dtype
  float* o;         // [batch*Hq][W+1][D]
  float* ml;        // [batch*Hq][W+1][2]  (m natural log base, l)
  int32_t* pn;      // [batch*Hq][W+1][2]  (prefix end p, context length n)
  int slots;        // W + 1
  int window;       // W
};

// ---------------------------------------------------------- workspace ----
// Match result of one query head for one step, recorded by the step kernel
// for the merge kernel.
struct HeadState {
  int hit;       // 1 on a hit
  int slot;      // ring slot of the matched entry
  int s;         // start of the fresh key range
  int cnt;       // ring pushes before this step
  int match_n;   // context length of the matched entry, -1 on a miss
  float dist;    // distance of the best candidate, +inf if none
  int n;         // keys of the sequence after this step's append
  int pad;
};

// Split-K plan of one KV group: fresh keys [lo, hi) split at mid = p_new
// into n_pre slices over [lo, mid) and n_post slices over [mid, hi).
// Interior boundaries fall on 16-token tile edges.  Slice order: the n_post
// slices come first (indices 0 .. n_post - 1): their keys do not depend on
// the match, so a workgroup can start loading them before it knows the match
// result; the n_pre slices follow.
struct Plan {
  int lo, mid, hi, n_pre, n_post;
};

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// first: slices per group in the first round of workgroups (max_slices when
// the launch fills the GPU in one round).  With a second round, the slices
// after p_new are capped at first - 2: every slice a hit needs (those and the
// first one before p_new) is then in the first round, and so is one slice a
// hit leaves empty (slice first - 1, which copies the reused states).
__host__ __device__ __forceinline__ Plan make_plan(int lo, int n, int band, int max_slices,
                                                   int first) {
  Plan p;
  p.hi = n;
  p.mid = n - band > 0 ? n - band : 0;
  p.lo = lo < p.mid ? lo : p.mid;
  const int lpre = p.mid - p.lo, lpost = p.hi - p.mid;
  int post_cap = max_slices / 2;
  if (first < max_slices && post_cap > first - 2) post_cap = first - 2;
  if (post_cap < 1) post_cap = 1;
  p.n_post = lpost > 0 ? min(ceil_div(lpost, kSliceMin), post_cap) : 0;
  const int pre_cap = max_slices - p.n_post;
  p.n_pre = lpre > 0 ? min(ceil_div(lpre, kSliceMin), pre_cap) : 0;
  return p;
}

// Part i of [a, e) split into n parts on tile edges: the range's tiles
// t0 .. t1 - 1 are dealt q = (t1 - t0) / n to each part and one more to the
// first (t1 - t0) mod n parts; the first part starts at a and the last ends at
// e.  One unsigned 32-bit division per call (the plan is computed before the
// tile loop can start, where each instruction adds to the latency).  Every
// part holds at least one tile when t1 - t0 >= n, which the slice counts of
// make_plan guarantee.
__host__ __device__ __forceinline__ void part_range(int a, int e, int n, int i, int* pa, int* pe) {
  const unsigned t0 = static_cast<unsigned>(a) / kTile;
  const unsigned nt = (static_cast<unsigned>(e) + kTile - 1) / kTile - t0;
  const unsigned q = nt / static_cast<unsigned>(n), r = nt - q * static_cast<unsigned>(n);
  auto bound = [&](int j) -> int {
    if (j <= 0) return a;
    if (j >= n) return e;
    const unsigned uj = static_cast<unsigned>(j);
    const int x = static_cast<int>((t0 + uj * q + (uj < r ? uj : r)) * kTile);
    return x > a ? x : a;
  };
  *pa = bound(i);
  *pe = bound(i + 1);
}

__host__ __device__ __forceinline__ bool slice_is_pre(const Plan& p, int i) { return i >= p.n_post; }

// Key range [*a, *e) of slice i of a plan (i < n_pre + n_post).
__host__ __device__ __forceinline__ void slice_range(const Plan& p, int i, int* a, int* e) {
  if (i < p.n_post) part_range(p.mid, p.hi, p.n_post, i, a, e);
  else part_range(p.lo, p.mid, p.n_pre, i - p.n_post, a, e);
}

// Workgroup id -> (group, slice) of the step launch, and the grid size.
// Ids run slice-major (group = id mod groups): the hardware deals ids
// round-robin to the 8 XCDs, so with 8 groups every slice of a group shares
// one XCD and its L2 holds the group's ring rows once.  Wide groups split
// into nchunk chunks read the same keys in every chunk: their ids run
// chunk-major, each chunk's run padded to a multiple of 8, so the chunks of
// a slice share an XCD and its L2 reads of the slice's tiles.  Padding ids
// return false, with slice = S (a slice no plan gives work) and a valid
// group.
//
// A narrow launch with a second round of workgroups (slices >= first, dealt
// to compute units as they come free) can take an order of the sequences,
// longest first: its second-round ids then run sequence by sequence in that
// order (slice-major within a sequence), so each XCD's queue holds its
// longest slices first and the units that finish short first-round slices
// take them (longest-processing-time-first list scheduling).  Any
// permutation gives the same bijection, so a stale order costs time, never
// results.
constexpr int kXcds = 8;
constexpr int kOrderMax = 16;   // sequences an order can hold (4 bits each)

__host__ __device__ __forceinline__ int step_grid(int groups, int nchunk, int S) {
  if (nchunk == 1) return groups * S;
  const int per = groups / nchunk * S;
  return nchunk * ((per + kXcds - 1) / kXcds * kXcds);
}

__host__ __device__ __forceinline__ bool step_coords(int id, int groups, int nchunk, int S,
                                                     int* grp, int* slice, int hkv = 1, int first = 0,
                                                     bool ordered = false, unsigned long long order = 0) {
  if (nchunk == 1) {
    const int r1 = groups * first;
    if (ordered && id >= r1) {
      const int per = hkv * (S - first), j = id - r1;
      const int rem = j % per, k = j / per;   // the sequence in nibble k
      *grp = static_cast<int>((order >> (4 * k)) & 15u) * hkv + rem % hkv;
      *slice = first + rem / hkv;
      return true;
    }
    *grp = id % groups;
    *slice = id / groups;
    return true;
  }
  const int nreal = groups / nchunk;
  const int per = nreal * S, run = (per + kXcds - 1) / kXcds * kXcds;
  const int c = id / run, j = id % run;
  *grp = (j % nreal) * nchunk + c;
  *slice = j < per ? j / nreal : S;
  return j < per;
}

// Partial states: o unnormalized, m in log2 units of the scaled score.
struct PartialView {
  float* o;    // [groups][S][G][D]
  float* ml;   // [groups][S][G][2]
  int S;
  int first;   // slices per group in the first round of workgroups (S: one round)
};

struct StepArgs {
  const void* q_pre;        // [batch][Hq][D] dtype
  const void* k_cache;
  const void* v_cache;
  const int32_t* page_table;
  int32_t* seq_lens;        // [batch] device lengths
  const double* inv_freq;   // [D/2] theta^(-2i/D), float64
  const void* k_new;        // fused append: [batch][Hkv][D] dtype, else null
  const void* v_new;
  float* out;               // [batch][Hq][D]
  int32_t* match_ctx_out;   // nullable
  float* dist_out;          // nullable
  HeadState* heads;         // [batch*Hq] match results of the step
  float* reuse_o;           // [batch*Hq][D] the matched entry's o (hit heads)
  float* reuse_ml;          // [batch*Hq][2] its (m, l)
  PartialView part;
  RingView ring;
  KvGeom geom;
  // A KV head with more than kMaxGroup query heads is split into nchunk
  // groups of `group` heads each ("virtual" KV heads; hkv counts them); KV
  // addressing uses the real head, virtual index / nchunk.
  int batch, hq, hkv, group, band, nchunk;
  float tau2;               // tau^2 rounded to fp32
  // sequences longest first, for the second round's ids (used when
  // 1 < batch <= kOrderMax): nibble k holds the sequence of rank k.  (This
  // keeps the argument block at 256 bytes; a larger block cost the hit
  // path time even when no workgroup read the extra bytes.)
  unsigned long long order;
  // (last, so that the fields the match reads first keep their offsets)
  // [groups] (ring count of the group's first head << 32 | plan start),
  // published by each group's slice-0 workgroup once its match is done
  unsigned long long* plan_pub;
};

}  // namespace mac
