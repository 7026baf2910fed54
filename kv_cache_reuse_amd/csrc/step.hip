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
// Two launches per step.  The partial states, the match records and the
// reused ring states pass from the step kernel to the merge kernel through a
// kernel boundary.  One hand-off stays inside the step kernel, and only in
// launches with more than one round of workgroups: the group's slice-0
// workgroup publishes its plan start (one 64-bit word, tagged with the ring
// count of the group's first head) with an agent-scope atomic store, and a
// later-round workgroup reads it with one plain 64-bit load; a word it reads
// too early or stale fails the tag check, and the workgroup then matches as
// usual.  The merge kernel clears the word after the step.
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
//  The merge launch follows (merge.hip): per query head, the log-sum-exp
//  merge of the reused state and the slices, the head's new ring entry and
//  its output; with a fused append it also publishes the new length.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "mac_dev.h"
#include "mac_launch.h"
#include "match.h"

namespace mac {

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
// NAT: caches in the natural (row) layout: tiles load like the library's
// tiles, and each K and V tile passes through the wave's LDS rows into
// operand order.
template <typename T, int D, bool PAGED, bool WIDE, bool R2 = false, bool NAT = false>
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
  // natural rows: each streaming wave's LDS rows for its key and value tiles
  using VR = std::conditional_t<BF, KvRows<NAT ? D : 32>, KvRowsF<NAT ? D : 32>>;
  __shared__ VR krows[NAT ? NWB : 1];
  __shared__ VR vrows[NAT ? NWB : 1];
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
  geom.natural = NAT ? 1 : 0;
  geom.d = D;   // a compile-time tile size in the address arithmetic
  // One tile's K and V through buffer loads: the tile's address goes into a
  // buffer descriptor in scalar registers, and each lane's byte offset
  // (16 lane + 1024 j) is the same for every tile, so no vector register is
  // rewritten per tile (a per-tile vector address can land on a register
  // that a load in flight still targets, and the compiler then waits for
  // every load).  The descriptor covers exactly the tile.
  // (a tile of either layout is 16 D sizeof(T) contiguous bytes; a natural
  // contiguous cache's last tile may hold fewer than 16 rows, and the
  // descriptor then ends with them)
  const uint32_t loff = 16u * static_cast<uint32_t>(lane);
  constexpr uint32_t kBlockStep = 1024u;
  // cpol: the loads' cache policy (kCachePolicyKeep or kCachePolicyStream),
  // a compile-time constant of the instruction
  auto load_tile_p = [&](auto cpol, int tt, u4 (&kk)[NL], u4 (&vv)[NL]) {
    const int64_t base = tile_base(geom, a.page_table, b, kvr, tt);
    const int bytes = (NAT && !PAGED ? tile_rows(geom, tt) : kTile) * D * (int)sizeof(T);
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
    // (the word is all ones from the previous step's merge until slice 0
    // publishes, so a read torn between the two values fails the tag check
    // or the range check of the start, which is at most p_new)
    int leave = 0;
    const unsigned lo_pub = static_cast<unsigned>(pub);
    if (static_cast<unsigned>(pub >> 32) == static_cast<unsigned>(cnt0) &&
        lo_pub <= static_cast<unsigned>(p_new)) {
      const Plan pp = make_plan(static_cast<int>(lo_pub), n, a.band, a.part.S, a.part.first);
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
      if constexpr (NAT) {
        k_rows_to_operand<D>(krows[wave], lane, kr);
        v_rows_to_operand<D>(vrows[wave], lane, vr);
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

      // ---- online softmax, base 2, with a lazy reference: each lane tests
      // its four scores against its head's reference m, and only when one of
      // the wave's scores passes it by more than kLazyRescale (one ballot, a
      // branch the whole wave takes or skips) does the wave form the heads'
      // tile maxima across the lane rows and rescale the heads whose maximum
      // passed.  Weights exp2(s - m) stay below 2^kLazyRescale.
      const float lmx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      if (__builtin_amdgcn_ballot_w64(lmx > m + kLazyRescale) != 0) {
        float mx = fmaxf(lmx, shfl_xor_f(lmx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const bool up = mx > m + kLazyRescale;   // the same in a head's four lanes
        const float alpha = up ? fast_exp2(m - mx) : 1.f;
#pragma unroll
        for (int i = 0; i < NCT; ++i) acc[i] *= alpha;
        lsum *= alpha;
        m = up ? mx : m;
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
    // The slices before p_new stream their keys once per step (on a miss,
    // nearly the whole cache), so their loads take the streaming policy and
    // leave the caches to what is read again: the slices after p_new hold
    // the band and the tail, which the next steps read again whether they
    // hit or miss.  (Each policy has its own copy of the loop, chosen
    // before it, so no load sits under a branch inside it; fp32 d128 at
    // two waves per SIMD has no registers for the second copy and streams
    // every slice with the non-temporal policy.  Natural rows load whole
    // lines too, so they take the same policies.)
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
    constexpr bool kTwoLoops = !(sizeof(T) == 4 && D == 128 && NWV > 4);
    if (nt > 0) {
      if constexpr (kTwoLoops) {
        if (slice_is_pre(p, slice)) stream(kStream);
        else stream(kKeep);
      } else {
        stream(kStream);
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
          kw[base + k_elem_offset<T>(geom, rnew, e)] = pk[e];
          vw[base + v_elem_offset<T>(geom, rnew, e)] = pv[e];
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

hipError_t launch_step(const StepArgs& a, int dtype, int d, int paged, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1) {
  if (a.group > kMaxGroup) {
    // wide groups (bf16 only): match launch, attention launch, merge
    hipError_t e = launch_match_wide(a, d, st);
    if (e != hipSuccess) return e;
    e = launch_step_wide(a, d, paged, st, ev0, ev1);
    if (e != hipSuccess) return e;
  } else {
  const int grid = step_grid(a.batch * a.hkv, a.nchunk, a.part.S);
  const bool wide = a.group > 4;
  // narrow, more than one round of workgroups: later rounds leave early on
  // hits.  (Wide groups measured slower with it: on the 70B shape, whose
  // groups rarely all hit, every later-round workgroup waits for the check
  // before its first tile load.)
  const bool r2 = !wide && a.part.first < a.part.S;
#define L_STEP_L(T, D, NAT)                                                                       \
  if (paged && wide)                                                                                 \
    launch_attention(step_kernel<T, D, true, true, false, NAT>, dim3(grid), dim3(64 * step_waves<T, D, true>()), st, ev0, ev1, a); \
  else if (paged && r2)                                                                              \
    launch_attention(step_kernel<T, D, true, false, true, NAT>, dim3(grid), dim3(64 * step_waves<T, D, false>()), st, ev0, ev1, a); \
  else if (paged)                                                                                    \
    launch_attention(step_kernel<T, D, true, false, false, NAT>, dim3(grid), dim3(64 * step_waves<T, D, false>()), st, ev0, ev1, a); \
  else if (wide)                                                                                     \
    launch_attention(step_kernel<T, D, false, true, false, NAT>, dim3(grid), dim3(64 * step_waves<T, D, true>()), st, ev0, ev1, a); \
  else if (r2)                                                                                       \
    launch_attention(step_kernel<T, D, false, false, true, NAT>, dim3(grid), dim3(64 * step_waves<T, D, false>()), st, ev0, ev1, a); \
  else launch_attention(step_kernel<T, D, false, false, false, NAT>, dim3(grid), dim3(64 * step_waves<T, D, false>()), st, ev0, ev1, a)
#define L_STEP(T, D) L_STEP_L(T, D, false)
    if (a.geom.natural) {
#define L_STEP_N(T, D) L_STEP_L(T, D, true)
      MAC_DISPATCH(dtype, d, L_STEP_N);
#undef L_STEP_N
    } else {
      MAC_DISPATCH(dtype, d, L_STEP);
    }
#undef L_STEP
#undef L_STEP_L
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_merge(a, dtype, d, st);
}

}  // namespace mac
