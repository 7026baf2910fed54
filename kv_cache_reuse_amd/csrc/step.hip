// libmac decode step for gfx950 (MI355X): two launches per MAC-Attention step.
//
// Method: "MAC-Attention: a Match-Amend-Complete Scheme for Fast and
// Accurate Attention Computation", abstract: a match stage (pre-RoPE L2
// matching over a short window of recent queries), an amend stage (the reused
// attention is rectified by recomputing a band of keys at the match
// boundary), a complete stage (fresh attention over the KV tail fused with the
// rest through a numerically stable merge); on a hit the cost does not depend
// on the context length.
//
// Two launches per step, so that the only cross-workgroup hand-off goes
// through a kernel boundary (no device-wide fences or atomics):
//
//  step_kernel, one workgroup per (slice, KV group), over a fixed number of
//  slices S per group (the launch is the same for every step and can be
//  captured in a graph; ids slice-major, or chunk-major for wide groups
//  split into chunks); 8 waves (4 for wide groups of fp32 d128 tiles):
//   A. read the sequence length; for each of the group's G query heads rotate
//      the query (float64 angles) and match the pre-RoPE query against the
//      ring (two waves per head, each over half of its slots, or up to two
//      heads per wave for wide groups; 16 lanes per ring slot); derive the
//      group's split-K plan and this workgroup's slice of keys.  The slice-0
//      workgroup records every head's match result for the merge, and the
//      last workgroup copies the hit heads' matched ring states for it.
//   B. with a non-empty slice: split-K attention on the matrix cores, one
//      partial state (o, m, l) per head.  Each wave's first tile under the
//      plan a miss would give is loaded while the match runs, and kept when
//      the real plan gives the wave the same first tile (always on a miss,
//      and for the slices after p_new on a hit); for the first slice before
//      p_new one wave loads the tile a typical hit starts in instead.  With a
//      fused append, the workgroup whose slice holds the new token stores it
//      in the cache and patches it into the tile it loads.
//  merge_kernel, one workgroup per query head (one wave, or up to 16 for
//  more than 32 slices): log-sum-exp merge of the reused state and the
//  slices, the head's new ring entry and its output; with a fused append it
//  also publishes the new length.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "mac_dev.h"
#include "mac_launch.h"

namespace mac {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr double kLog2e = 1.4426950408889634074;
constexpr float kLn2 = 0.69314718055994530942f;
// ring slots per 16-lane group per round.  A wave that takes all of a head's
// slots covers 36 per round (a window of 32, 33 slots, in one round); two
// waves that split a head's slots (even / odd) cover 20 each, 40 together.
constexpr int kMatchSlotsWhole = 9;
constexpr int kMatchSlotsHalf = 5;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Raw buffer descriptor over `bytes` bytes at p: no stride, 32-bit data
// format (the word the gfx9 family takes for untyped buffer access).
// Offsets past `bytes` read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }
// Sum over each 16-lane row of the wave, result in every lane of the row:
// DPP row rotations (VALU, no LDS round trip) by 8, 4, 2, 1.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<1>(v));
  return v;
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Wave-wide max and sum, the same value in every lane: DPP within each row
// of 16 lanes, then the four rows' results read from lanes 0, 16, 32, 48 in
// a fixed order (no LDS round trip).
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Row stride of the query rows in LDS: four elements of padding, so that the
// 16 head columns of a fragment read fall in different banks.
__host__ __device__ constexpr int qstride(int d) { return d + 4; }

template <int D, int NE, int OC>
struct Shared {
  HeadState head[kMaxGroup];
  // rotated, scaled queries: bf16 hi/lo halves or fp32, rows of qstride(D)
  // elements
  __attribute__((aligned(16))) unsigned char q[kMaxGroup * qstride(D) * 4];
  // match: each half of a head's ring slots' best candidate (d2 bits, age,
  // p, n, pushes), combined after the match
  int half_best[2][kMaxGroup][5];
  // phase B epilogue: the streaming waves' states (OC head columns)
  float m[NE][kMaxGroup];
  float l[NE][kMaxGroup];
  float o[NE][OC][D + 1];
  // fused append: the new token's key and value
  __attribute__((aligned(16))) unsigned char patch[2 * D * 4];
  int leave;   // second round: the workgroup's slice is empty
};

// =========================================================== phase A ====
// A wave matches one query head h (index hi in the group) over the ring
// slots off, off + st, off + 2 st, ... (st = 2 splits a head's slots between
// two waves).  The loads do not depend on the sequence length, so they are
// issued first (match_load) and the length is read while they are in
// flight; match_best then picks the best ring entry.  16 lanes share one
// ring slot, each lane holding D/16 elements of the row; a round covers
// 4 KMS slots.
template <typename T, int D, int KMS>
struct MatchIn {
  static constexpr int EPL = D / 16;                       // elements per lane
  static constexpr int NW = EPL * (int)sizeof(T) / 4;      // dwords per lane
  uint32_t qw[NW];                          // this lane's piece of q_pre
  uint32_t rw[KMS][NW];                     // its piece of the round's ring rows
  int2 pnl;                                 // (p, n) of the round's slot `lane`
  double inv;                               // theta^(-2 lane / D)
  // rotate-half pair of this lane, widened to 32 bits: two 16-bit values
  // sharing a register would have to be packed, which waits for both loads
  uint32_t q1, q2;
  int cnt;                                  // ring pushes so far
};

__device__ __forceinline__ uint32_t bits_of(uint16_t x) { return x; }
__device__ __forceinline__ uint32_t bits_of(float x) { return __float_as_uint(x); }
template <typename T> __device__ __forceinline__ float from_bits(uint32_t w);
template <> __device__ __forceinline__ float from_bits<uint16_t>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float from_bits<float>(uint32_t w) { return __uint_as_float(w); }

// a lane's D/16 elements of one row as 2, 4 or 8 dwords, one vector load
// (rows start 16-byte aligned, so the lane's piece is aligned too)
template <typename T, int D>
__device__ __forceinline__ void load_row(const T* src, uint32_t (&w)[D / 16 * (int)sizeof(T) / 4]) {
  constexpr int NW = D / 16 * (int)sizeof(T) / 4;
  if constexpr (NW == 2) {
    const u2 v = *reinterpret_cast<const u2*>(src);
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (NW == 4) {
    const u4 v = *reinterpret_cast<const u4*>(src);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const u4 v0 = reinterpret_cast<const u4*>(src)[0];
    const u4 v1 = reinterpret_cast<const u4*>(src)[1];
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
  }
}

// Ring slots s0 + st (gi + 4u) + off (u < KMS) of head bh, and the (p, n) of
// slot s0 + st lane + off, one lane per slot.  Slot indices are clamped into
// the ring; slots past W + 1 are dropped by the candidate test.
template <typename T, int D, int KMS>
__device__ __forceinline__ void load_slots(const StepArgs& a, int bh, int lane, int s0, int st,
                                           int off, MatchIn<T, D, KMS>& mi) {
  const RingView& R = a.ring;
  const int gi = lane / 16, c = lane % 16;
  const T* rq = static_cast<const T*>(R.q) + (size_t)bh * R.slots * D;
  const int2* rpn = reinterpret_cast<const int2*>(R.pn) + (size_t)bh * R.slots;
  // (p, n) first: loads complete in order, and the candidate mask needs them
  const int sl = s0 + st * lane + off;
  mi.pnl = rpn[sl < R.slots ? sl : 0];
#pragma unroll
  for (int u = 0; u < KMS; ++u) {
    const int s = s0 + st * (gi + 4 * u) + off;
    const int sc = s < R.slots ? s : 0;
    load_row<T, D>(rq + (size_t)sc * D + c * MatchIn<T, D, KMS>::EPL, mi.rw[u]);
  }
}

template <typename T, int D, int KMS>
__device__ __forceinline__ void match_load(const StepArgs& a, int bh, int lane, int st, int off,
                                           MatchIn<T, D, KMS>& mi) {
  const T* q = static_cast<const T*>(a.q_pre) + (size_t)bh * D;
  const bool rot = lane < D / 2;
  mi.cnt = a.ring.count[bh];
  mi.inv = rot ? a.inv_freq[lane] : 0.0;
  mi.q1 = rot ? bits_of(q[lane]) : 0u;
  mi.q2 = rot ? bits_of(q[lane + D / 2]) : 0u;
  load_row<T, D>(q + (lane % 16) * MatchIn<T, D, KMS>::EPL, mi.qw);
  load_slots<T, D, KMS>(a, bh, lane, 0, st, off, mi);
}

// Rotate-half pairs (i, i + D/2) of head hi's query: float64 angle and
// rotation, result scaled by log2(e)/sqrt(D) so that the attention can use
// exp2; pairs i0 <= i < i1 are stored in LDS as bf16 hi/lo halves (or fp32).
// Every lane that loaded a pair computes it, so the loads are consumed.
template <typename T, int D, int KMS, class SH>
__device__ __forceinline__ void rope_q(SH& sh, int hi, int lane, int n, const MatchIn<T, D, KMS>& mi,
                                       int i0 = 0, int i1 = D / 2) {
  if (lane < D / 2) {
    const int i = lane;
    double sn, cs;
    sincos(static_cast<double>(n - 1) * mi.inv, &sn, &cs);
    const double x1 = from_bits<T>(mi.q1), x2 = from_bits<T>(mi.q2);
    const double sc = kLog2e / sqrt(static_cast<double>(D));
    const float r1 = static_cast<float>((x1 * cs - x2 * sn) * sc);
    const float r2 = static_cast<float>((x2 * cs + x1 * sn) * sc);
    if (i < i0 || i >= i1) return;
    if constexpr (sizeof(T) == 2) {
      uint16_t* qh = reinterpret_cast<uint16_t*>(sh.q) + hi * qstride(D);
      uint16_t* ql = reinterpret_cast<uint16_t*>(sh.q) + (kMaxGroup + hi) * qstride(D);
      const uint16_t h1 = f32_to_bf16(r1), h2 = f32_to_bf16(r2);
      qh[i] = h1;
      qh[i + D / 2] = h2;
      ql[i] = f32_to_bf16(r1 - bf16_to_f32(h1));
      ql[i + D / 2] = f32_to_bf16(r2 - bf16_to_f32(h2));
    } else {
      float* qs = reinterpret_cast<float*>(sh.q) + hi * qstride(D);
      qs[i] = r1;
      qs[i + D / 2] = r2;
    }
  }
}

// Best ring entry among this wave's slots: d2 = dist^2 (+inf if none),
// k = its age (-1 if none), (p, n) of the entry.
struct Best {
  float d2;
  int k, p, n;
};

// the better of two candidates: smaller distance, then the newer entry
__device__ __forceinline__ bool better_than(float d2, int k, float bd2, int bk) {
  return k >= 0 && (bk < 0 || d2 < bd2 || (d2 == bd2 && k < bk));
}

// Slot s holds the entry k = (cnt - 1 - s) mod (W + 1) steps old; it is a
// candidate iff k < min(cnt, W) and 0 <= p <= p_new.  Best candidate:
// smallest squared distance, then smallest k (the newest entry).  The
// candidate test is taken one lane per slot and shared as a ballot mask; the
// best entry's (p, n) come from the lane of its slot, so no load follows the
// argmin.  Every wave consumes its loads (a wave past the group's heads
// too): loads left unread make the compiler wait for every load in flight
// before their registers are reused.
template <typename T, int D, int KMS>
__device__ __forceinline__ Best match_best(const StepArgs& a, int bh, int lane, int p_new, int st,
                                           int off, MatchIn<T, D, KMS>& mi) {
  constexpr int EPL = MatchIn<T, D, KMS>::EPL;
  const int gi = lane / 16;
  const RingView& R = a.ring;
  auto elem = [&](const uint32_t (&w)[MatchIn<T, D, KMS>::NW], int e) -> float {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16)));
    else return __uint_as_float(w[e]);
  };
  const int cnt = mi.cnt;
  const int nvalid = cnt < R.window ? cnt : R.window;
  // slot s is (r - s) mod (W + 1) steps old, r = (cnt - 1) mod (W + 1)
  const int r = cnt > 0 ? (cnt - 1) % R.slots : R.slots - 1;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = elem(mi.qw, e);
  float best = __builtin_inff();
  int bestk = -1, bp = 0, bn = -1;
  auto age = [&](int s) { return s >= R.slots ? R.slots : (r >= s ? r - s : r - s + R.slots); };
  auto round = [&](int s0) {
    const int sl = s0 + st * lane + off;
    const int pl = mi.pnl.x;
    const bool cl = lane < 4 * KMS && age(sl) < nvalid && pl >= 0 && pl <= p_new;
    const uint64_t cmask = __ballot(cl);
    int bj = -1;   // this round's best slot (index within the round) in this lane
#pragma unroll
    for (int u = 0; u < KMS; ++u) {
      if (s0 + st * 4 * u + off >= R.slots) break;   // the rest of the round is padding
      const int j = gi + 4 * u;
      float d2 = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float df = qv[e] - elem(mi.rw[u], e);
        d2 = fmaf(df, df, d2);
      }
      d2 = row16_sum(d2);
      const int k = age(s0 + st * j + off);
      const bool cand = ((cmask >> j) & 1) != 0 && d2 == d2;
      const bool better = cand && (d2 < best || (d2 == best && k < bestk));
      best = better ? d2 : best;
      bestk = better ? k : bestk;
      bj = better ? j : bj;
    }
    const int px = __shfl(mi.pnl.x, bj >= 0 ? bj : 0, 64);
    const int py = __shfl(mi.pnl.y, bj >= 0 ? bj : 0, 64);
    bp = bj >= 0 ? px : bp;
    bn = bj >= 0 ? py : bn;
  };
  // the first round straight-line: a loop header here would merge the
  // pending-load state and wait for every load in flight, the first tile's
  // included
  // (the second round too; a loop takes the rest)
  const int round_step = st * 4 * KMS;
  round(0);
  if (round_step + off < R.slots) {
    load_slots<T, D, KMS>(a, bh, lane, round_step, st, off, mi);
    round(round_step);
  }
  for (int s0 = 2 * round_step; s0 + off < R.slots; s0 += round_step) {
    load_slots<T, D, KMS>(a, bh, lane, s0, st, off, mi);
    round(s0);
  }
#pragma unroll
  for (int xo = 16; xo <= 32; xo <<= 1) {
    const float ob = shfl_xor_f(best, xo);
    const int ok = shfl_xor_i(bestk, xo);
    const int op = shfl_xor_i(bp, xo);
    const int on = shfl_xor_i(bn, xo);
    if (better_than(ob, ok, best, bestk)) {
      best = ob;
      bestk = ok;
      bp = op;
      bn = on;
    }
  }
  return Best{best, bestk, bp, bn};
}

// The head's match record from its best entry.
__device__ __forceinline__ HeadState head_record(const StepArgs& a, const Best& bst, int cnt, int n) {
  const bool hit = bst.k >= 0 && bst.d2 < a.tau2;
  HeadState hs;
  hs.hit = hit ? 1 : 0;
  hs.slot = hit ? (cnt - 1 - bst.k) % a.ring.slots : -1;
  hs.s = hit ? bst.p : 0;
  hs.cnt = cnt;
  hs.match_n = hit ? bst.n : -1;
  hs.dist = bst.k >= 0 ? sqrtf(bst.d2) : __builtin_inff();
  hs.n = n;
  hs.pad = 0;
  return hs;
}

// ========================================================== the kernel ==
// Waves per workgroup: 8, except for wide groups of fp32 d128 tiles, whose
// registers do not fit two waves per SIMD (4 waves, up to four heads each).
template <typename T, int D, bool WIDE>
__host__ __device__ constexpr int step_waves() {
  return WIDE && sizeof(T) == 4 && D == 128 ? 4 : 8;
}

// Narrow groups (at most 4 query heads): 8 waves; wave w matches head
// w mod 4 over half of its ring slots (even slots for w < 4, odd for the
// others), and the halves are combined after the match.  WIDE: groups of
// more than 4 query heads, each wave matching up to two heads (four with 4
// waves) over all their slots; a separate instantiation so that the narrow
// case's code has no conditional loads (which make the compiler wait for
// every load in flight).  In both, four waves stream the tiles.
// R2: a narrow launch with a second round of workgroups (more slices per
// group than one round fills): the slice-0 workgroup publishes its plan
// start and second-round workgroups whose slice is empty leave early.  A
// separate instantiation, so that one-round launches carry none of it.
template <typename T, int D, bool PAGED, bool WIDE, bool R2 = false>
__global__ __launch_bounds__((64 * step_waves<T, D, WIDE>())) void step_kernel(StepArgs a) {
  constexpr int NWV = step_waves<T, D, WIDE>(); // waves per workgroup
  constexpr int NWB = 4;                        // waves that stream tiles
  constexpr int NTH = 64 * NWV;
  constexpr int KMS = WIDE ? kMatchSlotsWhole : kMatchSlotsHalf;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int E = 16 / (int)sizeof(T);
  constexpr int NL = D * (int)sizeof(T) / 64;   // 1 KiB blocks per tile, K and V each
  constexpr int NQ = BF ? 2 * NL : 4 * NL;      // QK MFMA steps per tile
  constexpr int NCT = D / 16;                   // 16-dim column tiles of O^T

  __shared__ Shared<D, NWB, WIDE ? kMaxGroup : 4> sh;
  // (padding ids of a chunked group get slice S: no plan gives it work, and
  // it writes nothing; no early return here, so that the compiler issues the
  // argument loads phase A needs together with the ones for this mapping)
  int grp, slice;
  step_coords(blockIdx.x, a.batch * a.hkv, a.nchunk, a.part.S, &grp, &slice, a.hkv, a.part.first,
              R2 && a.batch > 1 && a.batch <= kOrderMax, a.order);
  const int b = grp / a.hkv, kvh = grp % a.hkv;
  const int kvr = kvh / a.nchunk;          // the KV head whose cache is read
  const int G = a.group;
  // the wave index is the same in every lane of a wave; readfirstlane makes
  // that visible to the compiler, so per-wave loop bounds and branches are
  // scalar (vector control flow around loads makes it wait for all of them)
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const bool fused = a.k_new != nullptr;

  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  KvGeom geom = a.geom;
  geom.paged = PAGED ? 1 : 0;
  geom.d = D;   // a compile-time tile size in the address arithmetic
  // One tile's K and V through buffer loads: the tile's address goes into a
  // buffer descriptor in scalar registers, and each lane's byte offset
  // (16 lane + 1024 j) is the same for every tile, so no vector register is
  // rewritten per tile (a per-tile vector address can land on a register
  // that a load in flight still targets, and the compiler then waits for
  // every load).  The descriptor covers exactly the tile.
  const uint32_t loff = 16u * static_cast<uint32_t>(lane);
  auto load_tile = [&](int tt, u4 (&kk)[NL], u4 (&vv)[NL]) {
    const int64_t base = tile_base(geom, a.page_table, b, kvr, tt);
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc + base, kTile * D * (int)sizeof(T));
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + base, kTile * D * (int)sizeof(T));
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      kk[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rk, loff + 1024u * j, 0, 0));
      vv[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rv, loff + 1024u * j, 0, 0));
    }
  };

  // ---------------------------------------------------------------- A ----
  // the match loads of this wave's first head go out before the length
  // (waves past the group's heads load a valid head's rows and ignore them:
  // no branch, so the compiler need not wait for the loads at a join)
  const int hi0 = WIDE ? wave : wave % 4;      // the wave's (first) head
  const int half = WIDE ? 0 : wave / 4;        // narrow: which half of its slots
  const int st = WIDE ? 1 : 2;                 // slot stride
  const int bh0 = b * a.hq + kvh * G + (hi0 < G ? hi0 : 0);
  // groups wider than the waves: a second buffer takes the wave's next
  // head right behind the first, and later heads are loaded one match ahead
  MatchIn<T, D, KMS> mi[WIDE ? 2 : 1];
  match_load<T, D, KMS>(a, bh0, lane, st, half, mi[0]);
  if constexpr (WIDE) match_load<T, D, KMS>(a, wave + NWV < G ? bh0 + NWV : bh0, lane, st, half, mi[1]);
  const int n0 = a.seq_lens[b];
  const bool append = fused && n0 >= 0 && n0 < a.geom.capacity;
  const int n = append ? n0 + 1 : n0;
  const int p_new = n - a.band > 0 ? n - a.band : 0;
  // A second-round workgroup (two rounds per launch) whose slice this step's
  // plan leaves empty leaves before its tile loads and its match, when the
  // group's slice-0 workgroup has already published the plan start (tagged
  // with the ring count of the group's first head, so an earlier step's
  // value never matches).  Wave 0 decides for the whole workgroup.
  if (R2 && slice >= a.part.first) {
    // (a plain load: an atomic one would keep the compiler from reading the
    // page table through scalar loads in the tile loop; a stale value only
    // fails the tag check, and the workgroup then matches as usual)
    const unsigned long long pub = a.plan_pub[grp];
    const int cnt0 = a.ring.count[b * a.hq + kvh * G];
    // every lane decides (so every wave consumes the load); wave 0's
    // decision is the workgroup's
    int leave = 0;
    if (static_cast<unsigned>(pub >> 32) == static_cast<unsigned>(cnt0)) {
      const Plan pp = make_plan(static_cast<int>(static_cast<unsigned>(pub)), n, a.band, a.part.S,
                                a.part.first);
      leave = slice >= pp.n_pre + pp.n_post;
    }
    if (wave == 0 && lane == 0) sh.leave = leave;
    __syncthreads();
    if (sh.leave) return;
  }
  // The group's plan when any of its heads misses does not depend on the
  // match: this wave's first tile under it is loaded while the match runs
  // and kept if the real plan gives the wave the same first tile.
  const Plan ps = make_plan(0, n, a.band, a.part.S, a.part.first);
  int ska = 0, ske = 0;
  if (slice < ps.n_pre + ps.n_post) slice_range(ps, slice, &ska, &ske);
  const int st0 = ska / kTile, st1 = (ske + kTile - 1) / kTile;
  // (waves past the streaming ones load wave - NWB's tile: the same lines,
  // an L2 hit, and every wave issues the same loads)
  const int wb = wave % NWB;
  int tspec = st0 + wb < st1 ? st0 + wb : st1 - 1;
  if (tspec < 0) tspec = 0;
  // On a hit the first slice before p_new usually holds only key p_new - 1
  // (a match one step old starts its band one key earlier): wave 0 of that
  // workgroup loads the tile of that key instead.  On a miss it reloads.
  if (ps.n_pre > 0 && slice == ps.n_post && wave == 0) tspec = (p_new - 1) / kTile;
  u4 kA[NL], vA[NL];
  load_tile(tspec, kA, vA);
  // n_post does not depend on the match either: the workgroup of the last
  // slice after p_new, which holds the new token, stages it in LDS now
  // (held in registers through the match, written to LDS after it, so no
  // wait for these loads lands in front of the match)
  T* pk = reinterpret_cast<T*>(sh.patch);
  T* pv = pk + D;
  const bool early_patch = append && ps.n_post > 0 && slice == ps.n_post - 1;
  T pke = T(0), pve = T(0);
  if (early_patch && tid < D) {
    pke = static_cast<const T*>(a.k_new)[((size_t)b * a.geom.hkv + kvr) * D + tid];
    pve = static_cast<const T*>(a.v_new)[((size_t)b * a.geom.hkv + kvr) * D + tid];
  }
  if constexpr (WIDE) {
    // heads NWV r + wave, with the buffers chosen at compile time
    if (hi0 < G) rope_q<T, D, KMS>(sh, hi0, lane, n, mi[0]);
    {
      const Best bst = match_best<T, D, KMS>(a, bh0, lane, p_new, st, half, mi[0]);
      if (hi0 < G && lane == 0) sh.head[hi0] = head_record(a, bst, mi[0].cnt, n);
    }
    auto more = [&](auto rc) {
      constexpr int r = decltype(rc)::value;
      const int hi = wave + NWV * r;
      if (hi < G) {
        if (hi + NWV < G) match_load<T, D, KMS>(a, bh0 + NWV * (r + 1), lane, st, half, mi[(r + 1) & 1]);
        rope_q<T, D, KMS>(sh, hi, lane, n, mi[r & 1]);
        const Best bst = match_best<T, D, KMS>(a, bh0 + NWV * r, lane, p_new, st, half, mi[r & 1]);
        if (lane == 0) sh.head[hi] = head_record(a, bst, mi[r & 1].cnt, n);
      }
    };
    static_assert(kMaxGroup == 16 && (NWV == 8 || NWV == 4), "16 heads over the waves");
    more(std::integral_constant<int, 1>{});
    if constexpr (NWV == 4) {
      more(std::integral_constant<int, 2>{});
      more(std::integral_constant<int, 3>{});
    }
  } else {
    // both halves rotate the query, each storing half of the pairs: every
    // wave consumes the rotation's loads (loads some path leaves unread make
    // the compiler wait for every load in flight before their registers are
    // reused, at the tile loop's head)
    if (hi0 < G) rope_q<T, D, KMS>(sh, hi0, lane, n, mi[0], half * (D / 4), (half + 1) * (D / 4));
    const Best bst = match_best<T, D, KMS>(a, bh0, lane, p_new, st, half, mi[0]);
    if (hi0 < G && lane == 0) {
      int* hb = sh.half_best[half][hi0];
      hb[0] = __float_as_int(bst.d2);
      hb[1] = bst.k;
      hb[2] = bst.p;
      hb[3] = bst.n;
      hb[4] = mi[0].cnt;
    }
  }
  if (early_patch && tid < D) {
    pk[tid] = pke;
    pv[tid] = pve;
  }
  __syncthreads();
  if constexpr (!WIDE) {
    // the two halves of each head's slots -> the head's record
    if (wave == 0 && lane < G) {
      const int* e0 = sh.half_best[0][lane];
      const int* e1 = sh.half_best[1][lane];
      Best bst{__int_as_float(e0[0]), e0[1], e0[2], e0[3]};
      const float d1 = __int_as_float(e1[0]);
      if (better_than(d1, e1[1], bst.d2, bst.k)) bst = Best{d1, e1[1], e1[2], e1[3]};
      sh.head[lane] = head_record(a, bst, e0[4], n);
    }
    __syncthreads();
  }
  int lo = sh.head[0].s, smax = sh.head[0].s;
  for (int i = 1; i < G; ++i) {
    lo = min(lo, sh.head[i].s);
    smax = max(smax, sh.head[i].s);
  }
  const Plan p = make_plan(lo, n, a.band, a.part.S, a.part.first);
  const int nact = p.n_pre + p.n_post;

  // ---------------------------------------------------------------- B ----
  if (slice < nact) {
    int ka, ke;
    slice_range(p, slice, &ka, &ke);
    const int lg = lane / 16, col = lane % 16;
    const bool hv = col < G;
    const int s_col = hv ? sh.head[col].s : 0;

    // query fragments (B operand of S = K Q^T) from LDS; zero for padding heads
    v4s qh[BF ? NQ : 1], ql[BF ? NQ : 1];
    float qf[BF ? 1 : NQ];
    if constexpr (BF) {
      const uint16_t* qhs = reinterpret_cast<const uint16_t*>(sh.q) + col * qstride(D);
      const uint16_t* qls = reinterpret_cast<const uint16_t*>(sh.q) + (kMaxGroup + col) * qstride(D);
#pragma unroll
      for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int d0 = 8 * (4 * j + lg) + 4 * hh;
          v4s x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
          if (hv) {
            x = *reinterpret_cast<const v4s*>(qhs + d0);
            y = *reinterpret_cast<const v4s*>(qls + d0);
          }
          qh[2 * j + hh] = x;
          ql[2 * j + hh] = y;
        }
    } else {
      const float* qss = reinterpret_cast<const float*>(sh.q) + col * qstride(D);
#pragma unroll
      for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * j + e] = hv ? qss[4 * (4 * j + lg) + e] : 0.f;
    }

    // fused append: the slice holding the new token (the last post slice,
    // or the last pre slice when there are none) stores it and patches it
    // into the tile it loads
    const bool patcher = append && slice == (p.n_post > 0 ? p.n_post - 1 : nact - 1);
    const int tnew = (n - 1) / kTile, rnew = (n - 1) % kTile;
    // the new token's key and value are staged in LDS (not registers, which
    // would stay live through the whole tile loop); with slices after p_new
    // that happened during the match, else (B = 0) it happens here
    if (patcher && !early_patch) {
      const T* kn = static_cast<const T*>(a.k_new) + ((size_t)b * a.geom.hkv + kvr) * D;
      const T* vn = static_cast<const T*>(a.v_new) + ((size_t)b * a.geom.hkv + kvr) * D;
      for (int e = tid; e < D; e += NTH) {
        pk[e] = kn[e];
        pv[e] = vn[e];
      }
      __syncthreads();
    }

    v4f acc[NCT];
#pragma unroll
    for (int i = 0; i < NCT; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    float m = neg_inf();
    float lsum = 0.f;
    const int t0 = ka / kTile, t1 = (ke + kTile - 1) / kTile;

    auto process = [&](int tt, u4 (&kr)[NL], u4 (&vr)[NL]) {
      if (patcher && tt == tnew) {
        // lane (lg, c) holds K of token c and V of tokens 4 lg .. 4 lg + 3
        if (col == rnew) {
#pragma unroll
          for (int j = 0; j < NL; ++j) kr[j] = *reinterpret_cast<const u4*>(pk + E * (4 * j + lg));
        }
        if (lg == rnew / 4) {
#pragma unroll
          for (int i = 0; i < NL; ++i)
#pragma unroll
            for (int th = 0; th < E / 4; ++th) {
              const int e = th * 4 + rnew % 4;           // element in the 16 bytes
              uint32_t val, mask;
              int dw;
              if constexpr (BF) {
                const int shift = (e & 1) * 16;
                dw = e >> 1;
                val = static_cast<uint32_t>(pv[16 * ((E / 4) * i + th) + col]) << shift;
                mask = 0xffffu << shift;
              } else {
                dw = e;
                val = __float_as_uint(pv[16 * ((E / 4) * i + th) + col]);
                mask = 0xffffffffu;
              }
              vr[i].x = dw == 0 ? (vr[i].x & ~mask) | val : vr[i].x;
              vr[i].y = dw == 1 ? (vr[i].y & ~mask) | val : vr[i].y;
              vr[i].z = dw == 2 ? (vr[i].z & ~mask) | val : vr[i].z;
              vr[i].w = dw == 3 ? (vr[i].w & ~mask) | val : vr[i].w;
            }
        }
      }
      // ---- S = K Q^T: lane holds tokens 4 lg + r of head col
      v4f s = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const u2 k01 = kr[j].xy, k23 = kr[j].zw;
          const v4s ka0 = __builtin_bit_cast(v4s, k01);
          const v4s ka1 = __builtin_bit_cast(v4s, k23);
          s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka0, qh[2 * j], s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka0, ql[2 * j], s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka1, qh[2 * j + 1], s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka1, ql[2 * j + 1], s, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kr[j][e]), qf[4 * j + e], s, 0, 0, 0);
      }

      // ---- mask tokens outside [ka, ke) and, per head, before its start
      const int tok0 = tt * kTile;
      const bool full = tok0 >= ka && tok0 + kTile <= ke && tok0 >= smax;
      if (!full) {
        // tokens outside [ka, ke) may be unwritten slots past the end of the
        // sequence: zero their values too, so that 0 * (stale NaN/Inf) cannot
        // enter the PV product (lane's V fragment = its score tokens)
        uint32_t keep[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = tok0 + 4 * lg + r;
          const bool in = kk >= ka && kk < ke;
          keep[r] = in ? 0xffffffffu : 0u;
          if (!in || kk < s_col) s[r] = neg_inf();
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          if constexpr (BF) {
            const uint32_t m01 = (keep[0] & 0xffffu) | (keep[1] & 0xffff0000u);
            const uint32_t m23 = (keep[2] & 0xffffu) | (keep[3] & 0xffff0000u);
            vr[i].x &= m01;
            vr[i].y &= m23;
            vr[i].z &= m01;
            vr[i].w &= m23;
          } else {
            vr[i].x &= keep[0];
            vr[i].y &= keep[1];
            vr[i].z &= keep[2];
            vr[i].w &= keep[3];
          }
        }
      }

      // ---- online softmax, base 2
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float mnew = fmaxf(m, mx);
      if (mnew > m) {
        const float alpha = fast_exp2(m - mnew);
#pragma unroll
        for (int i = 0; i < NCT; ++i) acc[i] *= alpha;
        lsum *= alpha;
        m = mnew;
      }
      const float mref = m == neg_inf() ? 0.f : m;
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = fast_exp2(s[r] - mref);
        lsum += pr[r];
      }

      // ---- O^T += V^T P^T
      if constexpr (BF) {
        v4s ph, pl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t hb = f32_to_bf16(pr[r]);
          ph[r] = static_cast<short>(hb);
          pl[r] = static_cast<short>(f32_to_bf16(pr[r] - bf16_to_f32(hb)));
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          // materialize the halves first: a bit cast taken straight from a
          // swizzled lvalue (vr[i].zw) reads the vector's first 8 bytes
          const u2 v01 = vr[i].xy, v23 = vr[i].zw;
          const v4s va0 = __builtin_bit_cast(v4s, v01);
          const v4s va1 = __builtin_bit_cast(v4s, v23);
          acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va0, ph, acc[2 * i], 0, 0, 0);
          acc[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va0, pl, acc[2 * i], 0, 0, 0);
          acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va1, ph, acc[2 * i + 1], 0, 0, 0);
          acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va1, pl, acc[2 * i + 1], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vr[i][r]), pr[r], acc[i], 0, 0, 0);
      }
    };

    // Wave w < NWB takes tiles t0 + w, t0 + w + NWB, ...; the next tiles are
    // loaded
    // while the current one is processed (with 8 waves, two per SIMD, the
    // tile loop measured slower: waves past NWB only wait at the epilogue).
    // Prefetch loads are unconditional
    // (an index past the slice is clamped to its last tile, an in-bounds
    // cache hit): a load under a branch leaves the outstanding-load count
    // unknown at the join, and the compiler then waits for every load,
    // prefetches included, before the current tile's math.
    // nt tiles for this wave: t0 + wave, + NWB, ...; pairs in a loop with one
    // exit (a loop left in the middle makes the compiler wait for every
    // load in flight at its header) while the tile it prefetches is one the
    // wave processes, then the last one or two tiles with no prefetch (a
    // tile loaded and never used would still hold the wave until it
    // arrived)
    const int tlast = t1 - 1;
    const int tw = t0 + wave;
    const int nt = wave < NWB && tw < t1 ? (t1 - tw + NWB - 1) / NWB : 0;
    if (nt > 0) {
      u4 kB[NL], vB[NL];
      if (tw != tspec) load_tile(tw, kA, vA);
      int i = 0;
      for (; i + 2 < nt; i += 2) {
        const int t = tw + NWB * i;
        load_tile(t + NWB, kB, vB);
        process(t, kA, vA);
        load_tile(min(t + 2 * NWB, tlast), kA, vA);
        process(t + NWB, kB, vB);
      }
      if (i + 1 < nt) {
        const int t = tw + NWB * i;
        load_tile(t + NWB, kB, vB);
        process(t, kA, vA);
        process(t + NWB, kB, vB);
      } else {
        process(tw + NWB * i, kA, vA);
      }
    }
    // slice 0 publishes the plan start for the second round of workgroups.
    // The store comes after the tile loop in program order (a global store
    // ahead of the loop would keep the compiler from reading the page table
    // through scalar loads there), but a wave that streams no tiles reaches
    // it right after the plan.
    if (R2 && slice == 0 && wave == NWB && lane == 0)
      __hip_atomic_store(a.plan_pub + grp,
                         (static_cast<unsigned long long>(static_cast<unsigned>(sh.head[0].cnt)) << 32) |
                             static_cast<unsigned>(lo),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lsum += shfl_xor_f(lsum, 16);
    lsum += shfl_xor_f(lsum, 32);

    // The new token goes into the cache only now: stores count in the same
    // counter as loads, and one issued before the tile loop would be waited
    // for at its entry.  No other workgroup reads this slot in this step.
    // (with a split KV head, every chunk patches its own tile and the first
    // one writes the cache)
    if (patcher && wave == 0 && kvh % a.nchunk == 0) {
      const int64_t base = tile_base_w(geom, a.page_table, b, kvr, tnew);
      if (base >= 0) {
        T* kw = const_cast<T*>(kc);
        T* vw = const_cast<T*>(vc);
        for (int e = lane; e < D; e += 64) {
          kw[base + k_tile_offset<T>(rnew, e)] = pk[e];
          vw[base + v_tile_offset<T>(rnew, e)] = pv[e];
        }
      }
    }

    // ---- the NWB streaming waves' states -> the slice's partial state
    if (wave < NWB && lg == 0) {
      sh.m[wave][col] = m;
      sh.l[wave][col] = lsum;
    }
    if (wave < NWB && hv) {   // padding columns are never read
#pragma unroll
      for (int i = 0; i < NCT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sh.o[wave][col][16 * i + 4 * lg + r] = acc[i][r];
    }
    __syncthreads();
    const size_t pbase = ((size_t)grp * a.part.S + slice) * G;
    for (int idx = tid; idx < G * D; idx += NTH) {
      const int hh = idx / D, dim = idx % D;
      float Mx = sh.m[0][hh];
#pragma unroll
      for (int w = 1; w < NWB; ++w) Mx = fmaxf(Mx, sh.m[w][hh]);
      float o = 0.f, L = 0.f;
#pragma unroll
      for (int w = 0; w < NWB; ++w) {
        const float mw = sh.m[w][hh];
        const float sc = mw == neg_inf() ? 0.f : fast_exp2(mw - Mx);
        o += sc * sh.o[w][hh][dim];
        L += sc * sh.l[w][hh];
      }
      a.part.o[(pbase + hh) * D + dim] = o;
      if (dim == 0) {
        a.part.ml[(pbase + hh) * 2] = Mx;
        a.part.ml[(pbase + hh) * 2 + 1] = L;
      }
    }
  }


  // the match results, for the merge kernel and the optional outputs (last,
  // for the same reason as the token's store)
  if (slice == 0 && tid < G) {
    const int bh = b * a.hq + kvh * G + tid;
    a.heads[bh] = sh.head[tid];
    if (a.match_ctx_out) a.match_ctx_out[bh] = sh.head[tid].match_n;
    if (a.dist_out) a.dist_out[bh] = sh.head[tid].dist;
  }
  // the hit heads' matched ring states, copied to rows of their own so that
  // the merge kernel loads them in its first round instead of behind the
  // records.  The last workgroup of the first round does it: on a hit its
  // slice is empty, and when every head misses there is nothing to copy.
  if (slice == a.part.first - 1) {
    for (int idx = tid; idx < G * D; idx += NTH) {
      const int hh = idx / D, dim = idx % D;
      if (sh.head[hh].hit) {
        const int bh = b * a.hq + kvh * G + hh;
        const size_t re = (size_t)bh * a.ring.slots + sh.head[hh].slot;
        a.reuse_o[(size_t)bh * D + dim] = a.ring.o[re * D + dim];
        if (dim < 2) a.reuse_ml[(size_t)bh * 2 + dim] = a.ring.ml[re * 2 + dim];
      }
    }
  }
}

// ========================================================= merge kernel ==
// Merge of one query head (b, h) by `nw` waves: log-sum-exp merge of the
// reused state and the group's slices, the head's new ring entry and its
// output.  Wave w takes the contiguous slices [k0, k1) of the group's S
// (at most 64; lane j holds the (m, l) of slice k0 + j), and each lane owns
// D/64 output dims.  A wave folds its slices' o in slice order, with each
// side's (before and after p_new) weights taken relative to the wave's own
// maximum; wave 0 then rescales and adds the waves' sums in wave order, so
// results are bitwise reproducible, and with one wave the arithmetic is the
// plain ordered fold.  The loads go out in one round (two for more than 32
// slices per wave) and need nothing from the match records: the slices'
// (m, l) first (loads complete in order, and the reductions need these
// before any o), then the query the entry copies, the reused ring state as
// the step kernel copied it for a hit head, and the slices' o (slices the
// plan leaves unused hold stale values: read in bounds, never used).  The
// records come through scalar loads alongside.
constexpr int kMergeMaxWaves = 16;
constexpr int kMergeBatch = 32;   // slices whose o one wave loads per round

__host__ __device__ inline int merge_waves(int S) {
  const int w = (S + kMergeBatch - 1) / kMergeBatch;
  return w < kMergeMaxWaves ? w : kMergeMaxWaves;
}

template <int D>
struct MergeShared {
  float m[kMergeMaxWaves][2];           // per wave: max of the slices before / after p_new
  float l[kMergeMaxWaves][2];
  float o[kMergeMaxWaves][2][D];
};

template <typename T, int D, bool MW>
__device__ __forceinline__ void merge_head(const StepArgs& a, int bh, int grp, int kvh, int hi,
                                           int wave, int nw, int lane, MergeShared<MW ? D : 1>& xs) {
  constexpr int DL = D / 64;            // output dims per lane
  constexpr int kBatch = kMergeBatch;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.group, S = a.part.S;
  const RingView& R = a.ring;
  const size_t pbase = (size_t)grp * S * G + hi;        // slice k: pbase + k * G
  const int spw = (S + nw - 1) / nw;
  const int k0 = wave * spw;
  const int k1 = k0 + spw < S ? k0 + spw : S;           // empty when k0 >= S

  // ---- the loads
  const float2* pml = reinterpret_cast<const float2*>(a.part.ml);
  const int kl = k0 + lane < S ? k0 + lane : S - 1;
  const float2 ml0 = pml[pbase + (size_t)kl * G];
  const T* qsrc = static_cast<const T*>(a.q_pre) + (size_t)bh * D + DL * lane;
  T qv[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) qv[e] = qsrc[e];
  // the reused state (the ring stores natural-log m and normalized o), as
  // the step kernel copied it for a hit head; stale otherwise, and then
  // never selected
  const float2 rml = reinterpret_cast<const float2*>(a.reuse_ml)[bh];
  float ro[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) ro[e] = a.reuse_o[(size_t)bh * D + DL * lane + e];
  float ob[kBatch][DL];
  auto load_o = [&](int kb) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = kb + u < S ? kb + u : S - 1;
      const float* src = a.part.o + (pbase + (size_t)k * G) * D + DL * lane;
#pragma unroll
      for (int e = 0; e < DL; ++e) ob[u][e] = src[e];
    }
  };
  // wave 0 loads its slices' o in the first round: on a hit its slices are
  // the only live ones.  The other waves' slices are live only when the
  // plan is long (a miss); they load once the plan is known.
  if (wave == 0) load_o(k0);
  // the group's match records (uniform addresses: scalar loads) and the plan
  const HeadState* hsg = a.heads + (size_t)b * a.hq + (size_t)kvh * G;
  const HeadState hs = hsg[hi];
  int lo = hs.s;
  for (int i = 0; i < G; ++i) lo = min(lo, hsg[i].s);
  const int n = hs.n;
  const Plan p = make_plan(lo, n, a.band, S, a.part.first);
  const int npart = p.n_pre + p.n_post;
  const int ke = k1 < npart ? k1 : npart;               // this wave's live slices: [k0, ke)
  if (MW && wave != 0 && k0 < ke) load_o(k0);

  // ---- this wave's maxima of the slices before and after p_new, then
  // weights relative to them (slice k0 + j's weight in lane j)
  const bool live = k0 + lane < ke;
  const bool pre0 = slice_is_pre(p, k0 + lane);
  float mp = neg_inf(), mq = neg_inf();
  if (live) {
    if (pre0) mp = ml0.x;
    else mq = ml0.x;
  }
  float MA = wave_max(mp), MC = wave_max(mq);
  float lp = 0.f, lq = 0.f, w0 = 0.f;
  if (live) {
    w0 = ml0.x == neg_inf() ? 0.f : fast_exp2(ml0.x - (pre0 ? MA : MC));
    if (pre0) lp += w0 * ml0.y;
    else lq += w0 * ml0.y;
  }
  float LA = wave_sum(lp), LC = wave_sum(lq);

  // ---- o of both sides (unnormalized, relative to MA and MC), slice order;
  // weights read from the lane that holds them
  float oa[DL], oc[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) oa[e] = oc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    if (k0 + u < ke) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), u));
      if (slice_is_pre(p, k0 + u)) {
#pragma unroll
        for (int e = 0; e < DL; ++e) oa[e] += w * ob[u][e];
      } else {
#pragma unroll
        for (int e = 0; e < DL; ++e) oc[e] += w * ob[u][e];
      }
    }
  }
  // a wave's second round (more than 32 slices per wave)
  if (k0 + kBatch < ke) {
    load_o(k0 + kBatch);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (k0 + kBatch + u < ke) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), kBatch + u));
        if (slice_is_pre(p, k0 + kBatch + u)) {
#pragma unroll
          for (int e = 0; e < DL; ++e) oa[e] += w * ob[u][e];
        } else {
#pragma unroll
          for (int e = 0; e < DL; ++e) oc[e] += w * ob[u][e];
        }
      }
    }
  }

  // ---- the waves' sums, rescaled to the largest maximum and added in wave
  // order by wave 0
  if constexpr (MW) {
    if (lane == 0) {
      xs.m[wave][0] = MA;
      xs.m[wave][1] = MC;
      xs.l[wave][0] = LA;
      xs.l[wave][1] = LC;
    }
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      xs.o[wave][0][DL * lane + e] = oa[e];
      xs.o[wave][1][DL * lane + e] = oc[e];
    }
    __syncthreads();
    if (wave != 0) return;
    MA = xs.m[0][0];
    MC = xs.m[0][1];
    for (int w = 1; w < nw; ++w) {
      MA = fmaxf(MA, xs.m[w][0]);
      MC = fmaxf(MC, xs.m[w][1]);
    }
    LA = LC = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) oa[e] = oc[e] = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float ma = xs.m[w][0], mc = xs.m[w][1];
      const float sa = ma == neg_inf() ? 0.f : fast_exp2(ma - MA);
      const float sc = mc == neg_inf() ? 0.f : fast_exp2(mc - MC);
      LA += sa * xs.l[w][0];
      LC += sc * xs.l[w][1];
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        oa[e] += sa * xs.o[w][0][DL * lane + e];
        oc[e] += sc * xs.o[w][1][DL * lane + e];
      }
    }
  }

  // ---- prefix = merge(reused, A), base 2
  const float mr = (hs.hit && rml.x != neg_inf()) ? rml.x * static_cast<float>(kLog2e) : neg_inf();
  const float lr = hs.hit ? rml.y : 0.f;
  const float MP = fmaxf(mr, MA);
  const float sr = mr == neg_inf() ? 0.f : fast_exp2(mr - MP);
  const float sa = MA == neg_inf() ? 0.f : fast_exp2(MA - MP);
  const float LP = sr * lr + sa * LA;
  const float fr = sr * lr;
  float po[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) po[e] = hs.hit ? fr * ro[e] + sa * oa[e] : sa * oa[e];

  // ---- the head's new ring entry: (q_pre, prefix state, p_new, n)
  const size_t we = (size_t)bh * R.slots + hs.cnt % R.slots;
  T* qdst = static_cast<T*>(R.q) + we * D + DL * lane;
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    R.o[we * D + DL * lane + e] = LP == 0.f ? 0.f : po[e] / LP;
    qdst[e] = qv[e];
  }

  // ---- out = merge(prefix, C)
  const float M = fmaxf(MP, MC);
  const float sp = MP == neg_inf() ? 0.f : fast_exp2(MP - M);
  const float sc = MC == neg_inf() ? 0.f : fast_exp2(MC - M);
  const float den = sp * LP + sc * LC;
#pragma unroll
  for (int e = 0; e < DL; ++e)
    a.out[(size_t)bh * D + DL * lane + e] = den == 0.f ? 0.f : (sp * po[e] + sc * oc[e]) / den;
  if (lane == 0) {
    R.ml[we * 2] = LP == 0.f ? neg_inf() : MP * kLn2;
    R.ml[we * 2 + 1] = LP;
    R.pn[we * 2] = p.mid;
    R.pn[we * 2 + 1] = n;
    R.count[bh] = hs.cnt + 1;
    // fused append: publish the new length (no kernel of this step reads it
    // after the step kernel)
    if (a.k_new && h == 0) a.seq_lens[b] = n;
  }
}

// One workgroup of merge_waves(S) waves per query head, a launch after the
// step kernel: the group's match results come from the step kernel's records.
// MW: more than one wave (a separate instantiation, so the one-wave merge
// keeps a one-wave register budget and has no exchange).
template <typename T, int D, bool MW>
__global__ __launch_bounds__(MW ? 64 * kMergeMaxWaves : 64) void merge_kernel(StepArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.group, kvh = h / G, hi = h % G;
  const int grp = b * a.hkv + kvh;
  const int wave = MW ? __builtin_amdgcn_readfirstlane(threadIdx.x / 64) : 0;
  const int nw = MW ? blockDim.x / 64 : 1;
  __shared__ MergeShared<MW ? D : 1> xs;
  merge_head<T, D, MW>(a, bh, grp, kvh, hi, wave, nw, threadIdx.x % 64, xs);
}

hipError_t launch_step(const StepArgs& a, int dtype, int d, int paged, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0) (void)hipEventRecord(ev0, st);
  const int grid = step_grid(a.batch * a.hkv, a.nchunk, a.part.S);
  const bool wide = a.group > 4;
  const bool r2 = !wide && a.part.first < a.part.S;   // narrow, two rounds
#define L_STEP(T, D)                                                                              \
  if (paged && wide)                                                                                 \
    hipLaunchKernelGGL((step_kernel<T, D, true, true>), dim3(grid), dim3(64 * step_waves<T, D, true>()), 0, st, a); \
  else if (paged && r2)                                                                              \
    hipLaunchKernelGGL((step_kernel<T, D, true, false, true>), dim3(grid), dim3(64 * step_waves<T, D, false>()), 0, st, a); \
  else if (paged)                                                                                    \
    hipLaunchKernelGGL((step_kernel<T, D, true, false>), dim3(grid), dim3(64 * step_waves<T, D, false>()), 0, st, a); \
  else if (wide)                                                                                     \
    hipLaunchKernelGGL((step_kernel<T, D, false, true>), dim3(grid), dim3(64 * step_waves<T, D, true>()), 0, st, a); \
  else if (r2)                                                                                       \
    hipLaunchKernelGGL((step_kernel<T, D, false, false, true>), dim3(grid), dim3(64 * step_waves<T, D, false>()), 0, st, a); \
  else hipLaunchKernelGGL((step_kernel<T, D, false, false>), dim3(grid), dim3(64 * step_waves<T, D, false>()), 0, st, a)
  MAC_DISPATCH(dtype, d, L_STEP);
#undef L_STEP
  if (ev1) (void)hipEventRecord(ev1, st);
#define L_MERGE(T, D)                                                                              \
  if (merge_waves(a.part.S) > 1)                                                                   \
    hipLaunchKernelGGL((merge_kernel<T, D, true>), dim3(a.batch * a.hq), dim3(64 * merge_waves(a.part.S)), 0, st, a); \
  else hipLaunchKernelGGL((merge_kernel<T, D, false>), dim3(a.batch * a.hq), dim3(64), 0, st, a)
  MAC_DISPATCH(dtype, d, L_MERGE);
#undef L_MERGE
  return hipGetLastError();
}

}  // namespace mac
