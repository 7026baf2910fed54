// libmac decode step for wide query groups (more than 16 query heads per KV
// head, bf16 caches: MQA and large GQA groups) on gfx950 (MI355X).
//
// Method: "MAC-Attention: a Match-Amend-Complete Scheme for Fast and
// Accurate Attention Computation", abstract: the match stage (pre-RoPE L2
// matching over a short window of recent queries), the amend and complete
// stages (fresh attention over the band at the match boundary and the KV
// tail) and the numerically stable merge.  With many query heads on one KV
// head the match is as large as the keys a split-K slice streams, so here it
// runs once per query head, in a launch of its own, instead of in every
// workgroup of the group:
//
//  match_kernel, two waves per query head: rotates the query (float64
//  angles, scaled by log2(e)/sqrt(d)) into bf16 hi/lo rows of the
//  workspace, matches the pre-RoPE query against the ring and records the
//  head's result (for the attention, the merge and the optional outputs);
//  for a hit it copies the matched entry's state for the merge.
//
//  wide_step_kernel, one workgroup per (slice, group of up to 32 heads):
//  reads the group's records, derives the split-K plan and streams its
//  slice's KV tiles once for all heads of the group, two 16-head column
//  tiles of the matrix cores per key fragment; writes one partial state per
//  head.  With a fused append, the workgroup whose slice holds the new token
//  stores it in the cache and patches it into the tile it loads.
//
//  the merge launch (merge.hip) folds the partial states as for narrow groups.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mac_dev.h"
#include "mac_launch.h"
#include "match.h"

namespace mac {

// Rotated, scaled query rows of the wide path, after the reused-state rows
// of the workspace: per query head a bf16 hi row and a bf16 lo row of D.
__host__ __device__ inline uint16_t* wide_qrot(const StepArgs& a) {
  const size_t nbh = static_cast<size_t>(a.batch) * a.hq;
  uintptr_t p = reinterpret_cast<uintptr_t>(a.reuse_ml + 2 * nbh);
  p = (p + 15) & ~uintptr_t(15);
  return reinterpret_cast<uint16_t*>(p);
}

// ========================================================= match kernel ==
// Two waves per query head: wave w matches the head's ring slots w, w + 2,
// ... and rotates half of the query's pairs; both take the better of the two
// candidates (smaller distance, then the newer entry), wave 0 writes the
// head's record and, on a hit, the winning wave the matched entry's state.
template <int D>
__global__ __launch_bounds__(128) void match_kernel(StepArgs a) {
  using T = uint16_t;
  constexpr int KMS = kMatchSlotsHalf;
  const int bh = blockIdx.x;
  const int b = bh / a.hq;
  const int lane = threadIdx.x % 64;
  const int half = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  __shared__ int best[2][5];   // per wave: d2 bits, age, p, n, ring pushes
  MatchIn<T, D, KMS> mi;
  match_load<T, D, KMS>(a, bh, lane, 2, half, mi);
  const int n0 = a.seq_lens[b];
  const bool append = a.k_new != nullptr && n0 >= 0 && n0 < a.geom.capacity;
  const int n = append ? n0 + 1 : n0;
  const int p_new = n - a.band > 0 ? n - a.band : 0;
  // rotate-half pairs (i, i + D/2) at position n - 1, float64 angle and
  // rotation, scaled so that the attention can use exp2; hi and lo halves.
  // Both waves rotate every pair (so each consumes its loads) and store
  // half of them.
  if (lane < D / 2) {
    float sn, cs;
    rope_sincos(n - 1, mi.inv, &sn, &cs);
    const float x1 = from_bits<T>(mi.q1), x2 = from_bits<T>(mi.q2);
    const float sc = static_cast<float>(kLog2e / sqrt(static_cast<double>(D)));
    const float r1 = fmaf(x1, cs, -x2 * sn) * sc;
    const float r2 = fmaf(x2, cs, x1 * sn) * sc;
    if (lane / (D / 4) == half) {
      uint16_t* qh = wide_qrot(a) + static_cast<size_t>(bh) * 2 * D;
      uint16_t* ql = qh + D;
      const uint16_t h1 = f32_to_bf16(r1), h2 = f32_to_bf16(r2);
      qh[lane] = h1;
      qh[lane + D / 2] = h2;
      ql[lane] = f32_to_bf16(r1 - bf16_to_f32(h1));
      ql[lane + D / 2] = f32_to_bf16(r2 - bf16_to_f32(h2));
    }
  }
  const Best bst = match_best<T, D, KMS>(a, bh, lane, p_new, 2, half, mi);
  // A wave whose best candidate is under tau loads that entry's state now:
  // the load overlaps the exchange of the two waves' candidates, and on a
  // hit the winning wave writes the state from its registers.
  constexpr int EPL = D / 16;
  const RingView& R = a.ring;
  const bool own_hit = bst.k >= 0 && bst.d2 < a.tau2;
  const int own_slot = own_hit ? (mi.cnt - 1 - bst.k) % R.slots : 0;
  float ro[EPL];
  float2 rml = make_float2(0.f, 0.f);
  if (own_hit) {
    const size_t re = (size_t)bh * R.slots + own_slot;
    const float* src = R.o + re * D + EPL * (lane % 16);
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(src + e);
      ro[e] = x.x;
      ro[e + 1] = x.y;
      ro[e + 2] = x.z;
      ro[e + 3] = x.w;
    }
    rml = reinterpret_cast<const float2*>(R.ml)[re];
  }
  if (lane == 0) {
    best[half][0] = __float_as_int(bst.d2);
    best[half][1] = bst.k;
    best[half][2] = bst.p;
    best[half][3] = bst.n;
    best[half][4] = mi.cnt;
  }
  __syncthreads();
  // both waves take the same decision: the better candidate (two slots
  // never tie in both distance and age)
  Best b0{__int_as_float(best[0][0]), best[0][1], best[0][2], best[0][3]};
  int win = 0;
  const float d1 = __int_as_float(best[1][0]);
  if (better_than(d1, best[1][1], b0.d2, b0.k)) {
    b0 = Best{d1, best[1][1], best[1][2], best[1][3]};
    win = 1;
  }
  const HeadState hs = head_record(a, b0, best[0][4], n);
  if (half == 0 && lane == 0) {
    a.heads[bh] = hs;
    if (a.match_ctx_out) a.match_ctx_out[bh] = hs.match_n;
    if (a.dist_out) a.dist_out[bh] = hs.dist;
  }
  // on a hit the winner's own best is the matched entry, loaded above
  if (hs.hit && half == win) {
    if (lane < 16) {
      float* dst = a.reuse_o + (size_t)bh * D + EPL * lane;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(ro[e], ro[e + 1], ro[e + 2], ro[e + 3]);
    }
    if (lane == 0) {
      a.reuse_ml[(size_t)bh * 2] = rml.x;
      a.reuse_ml[(size_t)bh * 2 + 1] = rml.y;
    }
  }
}

// ==================================================== wide step kernel ==
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWideCols = 2;                   // 16-head column tiles per workgroup
constexpr int kWideHeads = 16 * kWideCols;     // query heads a workgroup attends for

template <int D, int NWB>
struct WideShared {
  float m[NWB][kWideHeads];
  float l[NWB][kWideHeads];
  float sc[NWB][kWideHeads];      // each wave's weight in its head's partial state
  // rows of D + 4 floats: 16-byte aligned, so a lane stores its four
  // accumulator values of a 16-dim column tile with one 128-bit write (the
  // 16 lanes of a pass then cover all 64 banks)
  __attribute__((aligned(16))) float o[NWB][kWideHeads][D + 4];
  // fused append: the new token's key and value
  __attribute__((aligned(16))) uint16_t patch[2 * D];
};

// NWB waves, all streaming tiles (wave w takes tiles t0 + w, t0 + w + NWB,
// ...).  With no match to do, the workgroup has no other waves: at one wave
// per SIMD each wave holds both column tiles' queries and accumulators and
// two KV tiles in flight in registers.
// NAT: caches in the natural (row) layout: tiles load like the library's
// tiles, and each K and V tile passes through the wave's LDS rows into
// operand order.
template <int D, bool PAGED, int NWB, bool NAT>
__global__ __launch_bounds__(64 * NWB) void wide_step_kernel(StepArgs a) {
  using T = uint16_t;
  constexpr int NTH = 64 * NWB;
  constexpr int E = 8;                          // bf16 per 16-byte piece
  constexpr int NL = D * 2 / 64;                // 1 KiB blocks per tile, K and V each
  constexpr int NCT = D / 16;                   // 16-dim column tiles of O^T
  constexpr int NC = kWideCols;

  __shared__ WideShared<D, NWB> sh;
  __shared__ KvRows<NAT ? D : 32> krows[NAT ? NWB : 1];
  __shared__ KvRows<NAT ? D : 32> vrows[NAT ? NWB : 1];
  int grp, slice;
  step_coords(blockIdx.x, a.batch * a.hkv, a.nchunk, a.part.S, &grp, &slice);
  const int b = grp / a.hkv, kvh = grp % a.hkv;
  const int kvr = kvh / a.nchunk;               // the KV head whose cache is read
  const int G = a.group;                        // heads of this group, <= kWideHeads
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const bool fused = a.k_new != nullptr;

  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  KvGeom geom = a.geom;
  geom.paged = PAGED ? 1 : 0;
  geom.natural = NAT ? 1 : 0;
  geom.d = D;
  // (a tile of either layout is 32 D contiguous bytes; a natural contiguous
  // cache's last tile may hold fewer than 16 rows, and the descriptor then
  // ends with them)
  const uint32_t loff = 16u * static_cast<uint32_t>(lane);
  constexpr uint32_t kBlockStep = 1024u;
  auto load_tile_p = [&](auto cpol, int tt, u4 (&kk)[NL], u4 (&vv)[NL]) {
    const int64_t base = tile_base(geom, a.page_table, b, kvr, tt);
    const int bytes = (NAT && !PAGED ? tile_rows(geom, tt) : kTile) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + base, bytes);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      kk[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rk, loff + kBlockStep * j, 0, decltype(cpol)::value));
      vv[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rv, loff + kBlockStep * j, 0, decltype(cpol)::value));
    }
  };
  auto load_tile = [&](int tt, u4 (&kk)[NL], u4 (&vv)[NL]) { load_tile_p(kKeep, tt, kk, vv); };

  // ---------------------------------------------------------------- A ----
  // The group's match records and rotated queries do not depend on the
  // length, so they go out first: loads complete in order, and waiting for
  // them then never waits for the tile issued after them.  Lane i < G reads
  // head i's start (one round trip for the group; a loop of scalar loads
  // would wait for each record in turn).
  const int lg = lane / 16, col = lane % 16;
  const HeadState* hsg = a.heads + (size_t)b * a.hq + (size_t)kvh * G;
  const int s_lane = hsg[lane < G ? lane : 0].s;
  // this lane's head in each column tile, its start and its query fragments
  // (B operand of S = K Q^T; zero for padding heads)
  bool hv[NC];
  int s_col[NC];
  u4 qh[NC][NL], ql[NC][NL];
  const uint16_t* qrot = wide_qrot(a) + ((size_t)b * a.hq + (size_t)kvh * G) * 2 * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int hh = 16 * c + col;
    hv[c] = hh < G;
    s_col[c] = hsg[hv[c] ? hh : 0].s;
    const uint16_t* qhs = qrot + (size_t)(hv[c] ? hh : 0) * 2 * D;
    const uint16_t* qls = qhs + D;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int d0 = 8 * (4 * j + lg);
      const u4 xh = *reinterpret_cast<const u4*>(qhs + d0);
      const u4 xl = *reinterpret_cast<const u4*>(qls + d0);
      const u4 zero = {0u, 0u, 0u, 0u};
      qh[c][j] = hv[c] ? xh : zero;
      ql[c][j] = hv[c] ? xl : zero;
    }
  }
  const int n0 = a.seq_lens[b];
  const bool append = fused && n0 >= 0 && n0 < a.geom.capacity;
  const int n = append ? n0 + 1 : n0;
  const int p_new = n - a.band > 0 ? n - a.band : 0;
  // the first tile under the plan a miss gives, loaded while the records
  // are read (kept when the real plan gives the wave the same first tile)
  const Plan ps = make_plan(0, n, a.band, a.part.S, a.part.first);
  int ska = 0, ske = 0;
  if (slice < ps.n_pre + ps.n_post) slice_range(ps, slice, &ska, &ske);
  const int st0 = ska / kTile, st1 = (ske + kTile - 1) / kTile;
  const int wb = wave % NWB;
  int tspec = st0 + wb < st1 ? st0 + wb : st1 - 1;
  if (tspec < 0) tspec = 0;
  if (ps.n_pre > 0 && slice == ps.n_post && wave == 0) tspec = (p_new - 1) / kTile;
  u4 kA[NL], vA[NL];
  load_tile(tspec, kA, vA);
  const bool early_patch = append && ps.n_post > 0 && slice == ps.n_post - 1;
  T pke = T(0), pve = T(0);
  if (early_patch && tid < D) {
    pke = static_cast<const T*>(a.k_new)[((size_t)b * a.geom.hkv + kvr) * D + tid];
    pve = static_cast<const T*>(a.v_new)[((size_t)b * a.geom.hkv + kvr) * D + tid];
  }
  const int lo = wave_min_i(s_lane), smax = wave_max_i(s_lane);
  T* pk = sh.patch;
  T* pv = pk + D;
  if (early_patch && tid < D) {
    pk[tid] = pke;
    pv[tid] = pve;
  }
  const Plan p = make_plan(lo, n, a.band, a.part.S, a.part.first);
  const int nact = p.n_pre + p.n_post;

  // ---------------------------------------------------------------- B ----
  if (slice < nact) {
    int ka, ke;
    slice_range(p, slice, &ka, &ke);
    const bool patcher = append && slice == (p.n_post > 0 ? p.n_post - 1 : nact - 1);
    const int tnew = (n - 1) / kTile, rnew = (n - 1) % kTile;
    if (patcher && !early_patch) {
      const T* kn = static_cast<const T*>(a.k_new) + ((size_t)b * a.geom.hkv + kvr) * D;
      const T* vn = static_cast<const T*>(a.v_new) + ((size_t)b * a.geom.hkv + kvr) * D;
      for (int e = tid; e < D; e += NTH) {
        pk[e] = kn[e];
        pv[e] = vn[e];
      }
    }
    // (the staged token's LDS stores, early or here, before any read of them)
    __syncthreads();

    v4f acc[NC][NCT];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < NCT; ++i) acc[c][i] = v4f{0.f, 0.f, 0.f, 0.f};
    float m[NC], lsum[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      m[c] = neg_inf();
      lsum[c] = 0.f;
    }
    const int t0 = ka / kTile, t1 = (ke + kTile - 1) / kTile;

    auto process = [&](int tt, u4 (&kr)[NL], u4 (&vr)[NL]) __attribute__((always_inline)) {
      if (patcher && tt == tnew) {
        // rows: the tile as loaded; tiles: lane (lg, c) holds K of token c
        // and V of tokens 4 lg .. 4 lg + 3
        if constexpr (NAT) rows_patch<T, NL>(lane, rnew, pk, pv, kr, vr);
        if (!NAT && col == rnew) {
#pragma unroll
          for (int j = 0; j < NL; ++j) kr[j] = *reinterpret_cast<const u4*>(pk + E * (4 * j + lg));
        }
        if (!NAT && lg == rnew / 4) {
#pragma unroll
          for (int i = 0; i < NL; ++i)
#pragma unroll
            for (int th = 0; th < E / 4; ++th) {
              const int e = th * 4 + rnew % 4;
              const int shift = (e & 1) * 16;
              const int dw = e >> 1;
              const uint32_t val = static_cast<uint32_t>(pv[16 * ((E / 4) * i + th) + col]) << shift;
              const uint32_t mask = 0xffffu << shift;
              vr[i].x = dw == 0 ? (vr[i].x & ~mask) | val : vr[i].x;
              vr[i].y = dw == 1 ? (vr[i].y & ~mask) | val : vr[i].y;
              vr[i].z = dw == 2 ? (vr[i].z & ~mask) | val : vr[i].z;
              vr[i].w = dw == 3 ? (vr[i].w & ~mask) | val : vr[i].w;
            }
        }
      }
      if constexpr (NAT) {
        k_rows_to_operand<D>(krows[wave], lane, kr);
        v_rows_to_operand<D>(vrows[wave], lane, vr);
      }
      // ---- S = K Q^T for both column tiles: lane holds tokens 4 lg + r.
      // One K = 32 product per 1 KiB block: a lane's 16-byte piece (8 dims
      // of its token) is its A operand as loaded, and the same 8 dims of
      // the query its B operand.  Even and odd blocks go to two
      // accumulators, so the dependent chains are half as long.
      v4f sa[NC], sb[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) sa[c] = sb[c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const v8bf ka = __builtin_bit_cast(v8bf, kr[j]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          v4f& acc_s = (j & 1) ? sb[c] : sa[c];
          acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, __builtin_bit_cast(v8bf, qh[c][j]), acc_s, 0, 0, 0);
          acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, __builtin_bit_cast(v8bf, ql[c][j]), acc_s, 0, 0, 0);
        }
      }
      v4f s[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) s[c] = sa[c] + sb[c];
      // ---- masks: tokens outside [ka, ke) (values zeroed too, so that a
      // stale NaN/Inf past the sequence cannot enter 0 * value) and, per
      // head, tokens before its start
      const int tok0 = tt * kTile;
      const bool full = tok0 >= ka && tok0 + kTile <= ke && tok0 >= smax;
      if (!full) {
        uint32_t keep[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = tok0 + 4 * lg + r;
          const bool in = kk >= ka && kk < ke;
          keep[r] = in ? 0xffffffffu : 0u;
#pragma unroll
          for (int c = 0; c < NC; ++c)
            if (!in || kk < s_col[c]) s[c][r] = neg_inf();
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const uint32_t m01 = (keep[0] & 0xffffu) | (keep[1] & 0xffff0000u);
          const uint32_t m23 = (keep[2] & 0xffffu) | (keep[3] & 0xffff0000u);
          vr[i].x &= m01;
          vr[i].y &= m23;
          vr[i].z &= m01;
          vr[i].w &= m23;
        }
      }
      // ---- online softmax per head, base 2; P split into bf16 hi/lo.
      // The reference maximum m moves only when a score passes it by more
      // than kLazyRescale: the weights exp2(s - m) then stay below
      // 2^kLazyRescale, (o, m, l) stays a consistent state, and most tiles
      // skip rescaling the accumulators (with 32 heads some head's maximum
      // grows on nearly every tile, and each rescale moves 64 accumulator
      // registers through the VALU).  Each lane tests its own four scores;
      // only on a ballot that one of the wave's scores passed (a branch the
      // whole wave takes or skips) does the wave form each head's tile
      // maximum across the four lane rows and rescale the heads whose
      // maximum passed.
      v4s ph[NC], pl[NC];
      bool up_any = false;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        up_any = up_any || fmaxf(fmaxf(s[c][0], s[c][1]), fmaxf(s[c][2], s[c][3])) > m[c] + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(up_any) != 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float mx = fmaxf(fmaxf(s[c][0], s[c][1]), fmaxf(s[c][2], s[c][3]));
          mx = fmaxf(mx, shfl_xor_f(mx, 16));
          mx = fmaxf(mx, shfl_xor_f(mx, 32));
          const bool up = mx > m[c] + kLazyRescale;   // the same in a head's four lanes
          const float alpha = up ? fast_exp2(m[c] - mx) : 1.f;
#pragma unroll
          for (int i = 0; i < NCT; ++i) acc[c][i] *= alpha;
          lsum[c] *= alpha;
          m[c] = up ? mx : m[c];
        }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float mref = m[c] == neg_inf() ? 0.f : m[c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = fast_exp2(s[c][r] - mref);
          lsum[c] += pr;
          const uint16_t hb = f32_to_bf16(pr);
          ph[c][r] = static_cast<short>(hb);
          pl[c][r] = static_cast<short>(f32_to_bf16(pr - bf16_to_f32(hb)));
        }
      }
      // ---- O^T += V^T P^T, the value fragments shared by both column tiles
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const u2 v01 = vr[i].xy, v23 = vr[i].zw;
        const v4s va0 = __builtin_bit_cast(v4s, v01);
        const v4s va1 = __builtin_bit_cast(v4s, v23);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          acc[c][2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va0, ph[c], acc[c][2 * i], 0, 0, 0);
          acc[c][2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va0, pl[c], acc[c][2 * i], 0, 0, 0);
          acc[c][2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va1, ph[c], acc[c][2 * i + 1], 0, 0, 0);
          acc[c][2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va1, pl[c], acc[c][2 * i + 1], 0, 0, 0);
        }
      }
    };

    // tiles t0 + wave, + NWB, ...: pairs in a loop with one exit while the
    // prefetched tile is one the wave processes, then the last one or two
    // with no prefetch; prefetch indices past the slice clamp to its last
    // tile (unconditional loads keep the compiler's waits precise)
    const int tlast = t1 - 1;
    const int tw = t0 + wave;
    const int nt = wave < NWB && tw < t1 ? (t1 - tw + NWB - 1) / NWB : 0;
    // slices before p_new stream with the non-temporal policy, the band and
    // the tail (read again by the next steps) with the default one; one
    // copy of the loop per policy (natural rows load whole lines too)
    auto stream = [&](auto cpol) __attribute__((always_inline)) {
      u4 kB[NL], vB[NL];
      if (tw != tspec) load_tile_p(cpol, tw, kA, vA);
      int i = 0;
      for (; i + 2 < nt; i += 2) {
        const int t = tw + NWB * i;
        load_tile_p(cpol, t + NWB, kB, vB);
        process(t, kA, vA);
        load_tile_p(cpol, min(t + 2 * NWB, tlast), kA, vA);
        process(t + NWB, kB, vB);
      }
      if (i + 1 < nt) {
        const int t = tw + NWB * i;
        load_tile_p(cpol, t + NWB, kB, vB);
        process(t, kA, vA);
        process(t + NWB, kB, vB);
      } else {
        process(tw + NWB * i, kA, vA);
      }
    };
    if (nt > 0) {
      if (slice_is_pre(p, slice)) stream(kStream);
      else stream(kKeep);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      lsum[c] += shfl_xor_f(lsum[c], 16);
      lsum[c] += shfl_xor_f(lsum[c], 32);
    }

    // the new token goes into the cache after the tile loop (a store before
    // it would be waited for at its entry); the first chunk writes it
    if (patcher && wave == 0 && kvh % a.nchunk == 0) {
      const int64_t base = tile_base_w(geom, a.page_table, b, kvr, tnew);
      if (base >= 0) {
        T* kw = const_cast<T*>(kc);
        T* vw = const_cast<T*>(vc);
        for (int e = lane; e < D; e += 64) {
          kw[base + k_elem_offset<T>(geom, rnew, e)] = pk[e];
          vw[base + v_elem_offset<T>(geom, rnew, e)] = pv[e];
        }
      }
    }

    // ---- the NWB streaming waves' states -> the slice's partial state
    if (wave < NWB) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int hh = 16 * c + col;
        if (lg == 0) {
          sh.m[wave][hh] = m[c];
          sh.l[wave][hh] = lsum[c];
        }
        if (hv[c]) {
#pragma unroll
          for (int i = 0; i < NCT; ++i)
            *reinterpret_cast<v4f*>(&sh.o[wave][hh][16 * i + 4 * lg]) = acc[c][i];
        }
      }
    }
    __syncthreads();
    // per head, once: the maximum over the waves, each wave's weight and the
    // partial sum (m, l); then o = sum_w weight_w o_w, rows of D dims
    const size_t pbase = ((size_t)grp * a.part.S + slice) * G;
    if (tid < G) {
      float Mx = sh.m[0][tid];
#pragma unroll
      for (int w = 1; w < NWB; ++w) Mx = fmaxf(Mx, sh.m[w][tid]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < NWB; ++w) {
        const float mw = sh.m[w][tid];
        const float sc = mw == neg_inf() ? 0.f : fast_exp2(mw - Mx);
        sh.sc[w][tid] = sc;
        L += sc * sh.l[w][tid];
      }
      a.part.ml[(pbase + tid) * 2] = Mx;
      a.part.ml[(pbase + tid) * 2 + 1] = L;
    }
    __syncthreads();
    // four dims per thread: 128-bit LDS reads of the waves' rows and one
    // 128-bit store of the sum
    constexpr int RPP = NTH / (D / 4);            // head rows per pass
#pragma unroll
    for (int h0 = 0; h0 < kWideHeads; h0 += RPP) {
      const int hh = h0 + tid / (D / 4), d4 = 4 * (tid % (D / 4));
      if (hh < G) {
        v4f o = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NWB; ++w) o += sh.sc[w][hh] * *reinterpret_cast<const v4f*>(&sh.o[w][hh][d4]);
        *reinterpret_cast<v4f*>(&a.part.o[(pbase + hh) * D + d4]) = o;
      }
    }
  }
}

hipError_t launch_match_wide(const StepArgs& a, int d, hipStream_t st) {
  if (d == 128) hipLaunchKernelGGL((match_kernel<128>), dim3(a.batch * a.hq), dim3(128), 0, st, a);
  else hipLaunchKernelGGL((match_kernel<64>), dim3(a.batch * a.hq), dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_step_wide(const StepArgs& a, int d, int paged, hipStream_t st, hipEvent_t ev0,
                            hipEvent_t ev1) {
  const int grid = step_grid(a.batch * a.hkv, a.nchunk, a.part.S);
  constexpr int NWB = 4;
#define L_WIDE(D, NAT)                                                                                 \
  if (paged) launch_attention(wide_step_kernel<D, true, NWB, NAT>, dim3(grid), dim3(64 * NWB), st, ev0, ev1, a); \
  else launch_attention(wide_step_kernel<D, false, NWB, NAT>, dim3(grid), dim3(64 * NWB), st, ev0, ev1, a)
  if (a.geom.natural) {
    if (d == 128) { L_WIDE(128, true); } else { L_WIDE(64, true); }
  } else {
    if (d == 128) { L_WIDE(128, false); } else { L_WIDE(64, false); }
  }
#undef L_WIDE
  return hipGetLastError();
}

}  // namespace mac
