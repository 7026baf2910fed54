// libmac merge launch for gfx950 (MI355X): the last stage of a decode step.
//
// Method: "MAC-Attention: a Match-Amend-Complete Scheme for Fast and
// Accurate Attention Computation", abstract: the reused attention state of
// a matched query, the recomputed band at the match boundary and the fresh
// KV tail are fused by a numerically stable merge.  Per query head:
// prefix = merge(reused state on a hit, the slices before p_new) is the
// head's new ring entry, and out = merge(prefix, the slices after p_new).
// States are (o, m, l) with o unnormalized and m in log2 units of the scaled
// score inside a step; the ring stores natural-log m and normalized o.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mac_dev.h"
#include "mac_launch.h"
#include "match.h"

namespace mac {

// ========================================================= merge kernel ==
// Up to 32 slices per group (kMergeBatch): one wave per query head (b, h)
// does the log-sum-exp merge of the reused state and the group's slices,
// the head's new ring entry and its output.  Lane j holds the (m, l) of
// slice j and each lane owns D/64 output dims; the wave folds the slices'
// o in slice order, each side's (before and after p_new) weights taken
// relative to its maximum: the plain ordered fold, bitwise reproducible.
// The loads go out in one round and need nothing from the match records:
// the slices' (m, l) first (loads complete in order, and the reductions
// need these before any o), then the query the entry copies, the reused
// ring state as the step kernel copied it for a hit head, and the slices' o
// (slices the plan leaves unused hold stale values: read in bounds, never
// used).  The records come through scalar loads alongside.
constexpr int kMergeMaxWaves = 16;
constexpr int kMergeBatch = 32;   // slices the one-wave merge folds

// Waves of the merge launch per workgroup: 1 (merge_kernel) up to
// kMergeBatch slices, else one per 32 slices (merge_split_kernel).
__host__ __device__ inline int merge_waves(int S) {
  const int w = (S + kMergeBatch - 1) / kMergeBatch;
  return w < kMergeMaxWaves ? w : kMergeMaxWaves;
}

template <typename T, int D>
__device__ __forceinline__ void merge_head(const StepArgs& a, int bh, int grp, int kvh, int hi,
                                           int lane) {
  constexpr int DL = D / 64;            // output dims per lane
  constexpr int kBatch = kMergeBatch;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.group, S = a.part.S;
  const RingView& R = a.ring;
  const size_t pbase = (size_t)grp * S * G + hi;        // slice k: pbase + k * G
  const int k0 = 0;
  const int k1 = S;

  // ---- the loads
  // the group's fresh-range starts, lane i < G holding head i's: one vector
  // load, first (loads complete in order; a loop of scalar loads would wait
  // for each record in turn)
  const HeadState* hsg = a.heads + (size_t)b * a.hq + (size_t)kvh * G;
  const int s_lane = hsg[lane < G ? lane : 0].s;
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
  load_o(k0);
  // the head's own record (uniform address: scalar loads) and the plan
  const HeadState hs = hsg[hi];
  const int lo = wave_min_i(s_lane);
  const int n = hs.n;
  const Plan p = make_plan(lo, n, a.band, S, a.part.first);
  const int npart = p.n_pre + p.n_post;
  const int ke = k1 < npart ? k1 : npart;               // the live slices: [0, ke)

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
    // the group's published plan start is spent: clear it, so that every
    // step begins with no plan published and no later step (of this context
    // or of another one the workspace serves next) can take this one
    if (hi == 0 && a.part.first < a.part.S) a.plan_pub[grp] = ~0ull;
  }
}

// One one-wave workgroup per query head, a launch after the step kernel:
// the group's match results come from the step kernel's records.
template <typename T, int D>
__global__ __launch_bounds__(64) void merge_kernel(StepArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.group, kvh = h / G, hi = h % G;
  const int grp = b * a.hkv + kvh;
  merge_head<T, D>(a, bh, grp, kvh, hi, threadIdx.x % 64);
}

// ================================================ merge of many slices ==
// More than kMergeBatch slices per group (the wide path's 256, default launches of
// few KV groups, explicit slice counts): each head's dims are split over
// D / 32 workgroups of 32 dims, so that a compute unit reads a quarter (d =
// 128) of the head's partial states and every wave can load its slices' o
// in the first round, before the records give the plan (on a hit most of
// them are unused: read in bounds, never used).  Wave w takes the
// contiguous slices [k0, k1) (at most 2 PER); lane j holds the (m, l) of
// slice k0 + j; the two halves of the wave each fold every other slice of
// the wave's, in slice order, for dim 32 q + (lane mod 32), and the halves
// are added; wave 0 then rescales and adds the waves' sums in wave order.
// Results are bitwise reproducible.
constexpr int kMergeDims = 32;   // dims per merge workgroup

struct SplitShared {
  float m[kMergeMaxWaves][2];
  float l[kMergeMaxWaves][2];
  float o[kMergeMaxWaves][2][kMergeDims];
};

template <typename T, int D, int PER>
__global__ __launch_bounds__(64 * kMergeMaxWaves) void merge_split_kernel(StepArgs a) {
  constexpr int QP = D / kMergeDims;            // workgroups per query head
  const int bh = blockIdx.x / QP, q = blockIdx.x % QP;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.group, kvh = h / G, hi = h % G;
  const int grp = b * a.hkv + kvh;
  const int S = a.part.S;
  const int nw = blockDim.x / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int half = lane / 32;
  const int dim = q * kMergeDims + lane % 32;
  const RingView& R = a.ring;
  __shared__ SplitShared xs;

  const size_t pbase = (size_t)grp * S * G + hi;        // slice k: pbase + k * G
  const int spw = (S + nw - 1) / nw;                    // <= 2 PER
  const int k0 = wave * spw;
  const int k1 = k0 + spw < S ? k0 + spw : S;

  // ---- the loads, one round: the group's starts (lane i < G: head i's),
  // the slices' (m, l), the query the entry copies, the reused state as the
  // step (or match) kernel copied it, and the o of every slice of the wave
  const HeadState* hsg = a.heads + (size_t)b * a.hq + (size_t)kvh * G;
  const int s_lane = hsg[lane < G ? lane : 0].s;
  const int kl = k0 + lane < S ? k0 + lane : S - 1;
  const float2 ml0 = reinterpret_cast<const float2*>(a.part.ml)[pbase + (size_t)kl * G];
  const T qv = static_cast<const T*>(a.q_pre)[(size_t)bh * D + dim];
  const float2 rml = reinterpret_cast<const float2*>(a.reuse_ml)[bh];
  const float ro = a.reuse_o[(size_t)bh * D + dim];
  float ob[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = k0 + 2 * i + half < S ? k0 + 2 * i + half : S - 1;
    ob[i] = a.part.o[(pbase + (size_t)k * G) * D + dim];
  }
  const HeadState hs = hsg[hi];
  const int lo = wave_min_i(s_lane);
  const int n = hs.n;
  const Plan p = make_plan(lo, n, a.band, S, a.part.first);
  const int npart = p.n_pre + p.n_post;
  const int ke = k1 < npart ? k1 : npart;               // this wave's live slices: [k0, ke)

  // ---- the wave's maxima of the slices before and after p_new, weights
  // relative to them (slice k0 + j's in lane j) and the sums of l
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
    if (pre0) lp = w0 * ml0.y;
    else lq = w0 * ml0.y;
  }
  float LA = wave_sum(lp), LC = wave_sum(lq);

  // ---- o of both sides: each half of the wave folds slices k0 + 2 i + half
  // in order, then the halves are added
  float oa = 0.f, oc = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (k0 + 2 * i < ke) {
      const float we = lane_value(w0, 2 * i), wo = lane_value(w0, 2 * i + 1);
      const int k = k0 + 2 * i + half;
      if (k < ke) {
        const float w = half ? wo : we;
        if (slice_is_pre(p, k)) oa += w * ob[i];
        else oc += w * ob[i];
      }
    }
  }
  oa += shfl_xor_f(oa, 32);
  oc += shfl_xor_f(oc, 32);

  // ---- the waves' sums, rescaled to the largest maximum and added in wave
  // order by wave 0
  if (lane == 0) {
    xs.m[wave][0] = MA;
    xs.m[wave][1] = MC;
    xs.l[wave][0] = LA;
    xs.l[wave][1] = LC;
  }
  if (lane < kMergeDims) {
    xs.o[wave][0][lane] = oa;
    xs.o[wave][1][lane] = oc;
  }
  __syncthreads();
  if (wave != 0) return;
  const int c = lane % kMergeDims;
  MA = xs.m[0][0];
  MC = xs.m[0][1];
  for (int w = 1; w < nw; ++w) {
    MA = fmaxf(MA, xs.m[w][0]);
    MC = fmaxf(MC, xs.m[w][1]);
  }
  LA = LC = 0.f;
  oa = oc = 0.f;
  for (int w = 0; w < nw; ++w) {
    const float ma = xs.m[w][0], mc = xs.m[w][1];
    const float sa = ma == neg_inf() ? 0.f : fast_exp2(ma - MA);
    const float sc = mc == neg_inf() ? 0.f : fast_exp2(mc - MC);
    LA += sa * xs.l[w][0];
    LC += sc * xs.l[w][1];
    oa += sa * xs.o[w][0][c];
    oc += sc * xs.o[w][1][c];
  }

  // ---- prefix = merge(reused, A), base 2 (the ring stores natural-log m
  // and normalized o)
  const float mr = (hs.hit && rml.x != neg_inf()) ? rml.x * static_cast<float>(kLog2e) : neg_inf();
  const float lr = hs.hit ? rml.y : 0.f;
  const float MP = fmaxf(mr, MA);
  const float sr = mr == neg_inf() ? 0.f : fast_exp2(mr - MP);
  const float sa = MA == neg_inf() ? 0.f : fast_exp2(MA - MP);
  const float LP = sr * lr + sa * LA;
  const float po = hs.hit ? (sr * lr) * ro + sa * oa : sa * oa;

  // ---- the head's new ring entry (this workgroup's dims), and out
  const size_t we = (size_t)bh * R.slots + hs.cnt % R.slots;
  const float M = fmaxf(MP, MC);
  const float sp = MP == neg_inf() ? 0.f : fast_exp2(MP - M);
  const float sc = MC == neg_inf() ? 0.f : fast_exp2(MC - M);
  const float den = sp * LP + sc * LC;
  if (lane < kMergeDims) {
    R.o[we * D + dim] = LP == 0.f ? 0.f : po / LP;
    static_cast<T*>(R.q)[we * D + dim] = qv;
    a.out[(size_t)bh * D + dim] = den == 0.f ? 0.f : (sp * po + sc * oc) / den;
  }
  if (q == 0 && lane == 0) {
    R.ml[we * 2] = LP == 0.f ? neg_inf() : MP * kLn2;
    R.ml[we * 2 + 1] = LP;
    R.pn[we * 2] = p.mid;
    R.pn[we * 2 + 1] = n;
    R.count[bh] = hs.cnt + 1;
    if (a.k_new && h == 0) a.seq_lens[b] = n;
    if (hi == 0 && a.part.first < a.part.S) a.plan_pub[grp] = ~0ull;
  }
}

hipError_t launch_merge(const StepArgs& a, int dtype, int d, hipStream_t st) {
  const int S = a.part.S;
  const int nw = merge_waves(S);
  const int spw = (S + nw - 1) / nw;
#define L_MERGE(T, D)                                                                            \
  if (nw == 1)                                                                                   \
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(a.batch * a.hq), dim3(64), 0, st, a);          \
  else if (spw > 32)                                                                             \
    hipLaunchKernelGGL((merge_split_kernel<T, D, 32>), dim3(a.batch * a.hq * (D / kMergeDims)),  \
                       dim3(64 * nw), 0, st, a);                                                 \
  else                                                                                           \
    hipLaunchKernelGGL((merge_split_kernel<T, D, 16>), dim3(a.batch * a.hq * (D / kMergeDims)),  \
                       dim3(64 * nw), 0, st, a)
  MAC_DISPATCH(dtype, d, L_MERGE);
#undef L_MERGE
  return hipGetLastError();
}

}  // namespace mac
