// Device helpers shared by the libmac step kernels (gfx950): lane
// reductions, raw buffer descriptors, and the match of a pre-RoPE query
// against its ring (loads, rotation, best entry, match record).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mac_dev.h"
#include "rows_map.h"

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

// -------------------------------------------------- natural-layout tiles --
// A tile of the natural (row) layout loads like the library's tiles (1 KiB
// per wave load, every 128-byte line whole in one load); each streaming
// wave writes its K and V tile, as loaded, into LDS rows of its own and reads
// them back in the operand order of the library's tiles.  The lane maps are
// in rows_map.h.  LDS accesses of one wave complete in order, so the reads
// see the writes, and a later tile's writes follow this tile's reads.
template <int D>
struct KvRows {
  static constexpr int RS = D + kRowsPadBf16;
  __attribute__((aligned(16))) uint16_t v[16 * RS];
};

// (fp32 rows of D + 4: the reads of one element of 64 lanes fall in 64
// different banks)
template <int D>
struct KvRowsF {
  static constexpr int RS = D + kRowsPadF32;
  __attribute__((aligned(16))) float v[16 * RS];
};

// The NL loads of a tile, as loaded, into rows RS elements apart.
template <typename ET, int RS, int NL>
__device__ __forceinline__ void rows_store(ET* rows, int lane, const u4 (&x)[NL]) {
  constexpr int E = 16 / (int)sizeof(ET);
  constexpr int PR = 4 * NL;   // pieces per row: 16 rows of NL KiB / 16
#pragma unroll
  for (int j = 0; j < NL; ++j)
    *reinterpret_cast<u4*>(rows + rows_load_row(j, lane, PR) * RS + E * rows_load_piece(j, lane, PR)) = x[j];
}

// Key operand order.
template <typename ET, int RS, int NL>
__device__ __forceinline__ void rows_key_operand(const ET* rows, int lane, u4 (&kr)[NL]) {
  constexpr int E = 16 / (int)sizeof(ET);
#pragma unroll
  for (int j = 0; j < NL; ++j)
    kr[j] = *reinterpret_cast<const u4*>(rows + rows_key_row(lane) * RS + E * rows_key_piece(j, lane));
}

template <int D>
__device__ __forceinline__ void k_rows_to_operand(KvRows<D>& rows, int lane, u4 (&kr)[D / 32]) {
  rows_store<uint16_t, KvRows<D>::RS, D / 32>(rows.v, lane, kr);
  rows_key_operand<uint16_t, KvRows<D>::RS, D / 32>(rows.v, lane, kr);
}

template <int D>
__device__ __forceinline__ void k_rows_to_operand(KvRowsF<D>& rows, int lane, u4 (&kr)[D / 16]) {
  rows_store<float, KvRowsF<D>::RS, D / 16>(rows.v, lane, kr);
  rows_key_operand<float, KvRowsF<D>::RS, D / 16>(rows.v, lane, kr);
}

// fp32 values: vr[i] = tokens 4 lg .. 4 lg + 3 of dim 16 i + c.
template <int D>
__device__ __forceinline__ void v_rows_to_operand(KvRowsF<D>& rows, int lane, u4 (&vr)[D / 16]) {
  constexpr int NL = D / 16;
  constexpr int RS = KvRowsF<D>::RS;
  const int lg = lane / 16, c = lane % 16;
  rows_store<float, RS, NL>(rows.v, lane, vr);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int d = 16 * i + c;
    vr[i] = u4{__float_as_uint(rows.v[(4 * lg + 0) * RS + d]), __float_as_uint(rows.v[(4 * lg + 1) * RS + d]),
               __float_as_uint(rows.v[(4 * lg + 2) * RS + d]), __float_as_uint(rows.v[(4 * lg + 3) * RS + d])};
  }
}

// bf16 values, through the transposing LDS read: vr[i] holds tokens
// 4 lg .. 4 lg + 3 of dims 16 (2 i + th) + c for th = 0, 1 (element
// 4 th + r, two per dword).
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D>
__device__ __forceinline__ void v_rows_to_operand(KvRows<D>& rows, int lane, u4 (&vr)[D / 32]) {
  constexpr int NL = D / 32;
  constexpr int RS = KvRows<D>::RS;
  rows_store<uint16_t, RS, NL>(rows.v, lane, vr);
  const uint16_t* src = rows.v + tr16_row(lane) * RS + tr16_col(lane);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(src + 32 * i));
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(src + 32 * i + 16));
    const u2 w0 = __builtin_bit_cast(u2, x0), w1 = __builtin_bit_cast(u2, x1);
    vr[i] = u4{w0.x, w0.y, w1.x, w1.y};
  }
}

// Patch of a natural-layout tile as loaded: row r of K and V (one of
// D elements each, staged in LDS) replaces what the loads brought.
template <typename ET, int NL>
__device__ __forceinline__ void rows_patch(int lane, int r, const ET* pk, const ET* pv, u4 (&kr)[NL],
                                           u4 (&vr)[NL]) {
  constexpr int E = 16 / (int)sizeof(ET);
  constexpr int PR = 4 * NL;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    if (rows_load_row(j, lane, PR) == r) {
      kr[j] = *reinterpret_cast<const u4*>(pk + E * rows_load_piece(j, lane, PR));
      vr[j] = *reinterpret_cast<const u4*>(pv + E * rows_load_piece(j, lane, PR));
    }
  }
}

// Row stride of the query rows in LDS: four elements of padding, so that the
// 16 head columns of a fragment read fall in different banks.
__host__ __device__ constexpr int qstride(int d) { return d + 4; }

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
// Wave-wide minimum and maximum of an int, the same value in every lane
// (DPP within each row of 16 lanes, then the four rows' results).
template <int N>
__device__ __forceinline__ int row_ror_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x120 + N, 0xf, 0xf, false);
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, row_ror_i<8>(v));
  v = min(v, row_ror_i<4>(v));
  v = min(v, row_ror_i<2>(v));
  v = min(v, row_ror_i<1>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, row_ror_i<8>(v));
  v = max(v, row_ror_i<4>(v));
  v = max(v, row_ror_i<2>(v));
  v = max(v, row_ror_i<1>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

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

// The rotation of pair i at position pos: the angle pos * theta^(-2i/d) in
// float64 (pos reaches 1e5 and more, where a float32 angle errs by about
// 1e-2 rad), reduced to [-pi, pi] in float64 (Cody-Waite, 2 pi split into a
// 53-bit head and its tail), then sine and cosine in float32.
__device__ __forceinline__ void rope_sincos(int pos, double inv, float* sn, float* cs) {
  constexpr double kInv2Pi = 0.15915494309189533577;
  constexpr double k2PiHi = 6.28318530717958623200;    // nearest double to 2 pi
  constexpr double k2PiLo = 2.44929359829470635445e-16; // 2 pi - k2PiHi
  const double ang = static_cast<double>(pos) * inv;
  const double k = rint(ang * kInv2Pi);
  const double r = fma(-k, k2PiLo, fma(-k, k2PiHi, ang));
  sincosf(static_cast<float>(r), sn, cs);
}

// Rotate-half pairs (i, i + D/2) of head hi's query (angle as rope_sincos),
// result scaled by log2(e)/sqrt(D) so that the attention can use exp2; pairs
// i0 <= i < i1 are stored in LDS as bf16 hi/lo halves (or fp32).  Every lane
// that loaded a pair computes it, so the loads are consumed.
template <typename T, int D, int KMS, class SH>
__device__ __forceinline__ void rope_q(SH& sh, int hi, int lane, int n, const MatchIn<T, D, KMS>& mi,
                                       int i0 = 0, int i1 = D / 2) {
  if (lane < D / 2) {
    const int i = lane;
    float sn, cs;
    rope_sincos(n - 1, mi.inv, &sn, &cs);
    const float x1 = from_bits<T>(mi.q1), x2 = from_bits<T>(mi.q2);
    const float sc = static_cast<float>(kLog2e / sqrt(static_cast<double>(D)));
    const float r1 = fmaf(x1, cs, -x2 * sn) * sc;
    const float r2 = fmaf(x2, cs, x1 * sn) * sc;
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


}  // namespace mac
