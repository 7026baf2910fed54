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
//
// merge_kernel: each query head's dims are split over D / MD workgroups of
// MD dims, so that a compute unit reads a fraction of the head's partial
// states and every wave loads all of its slices' o in the first round,
// before the match records give the plan (slices the plan leaves unused
// hold stale values: read in bounds, never used).  A workgroup has one wave
// per 32 slices of the group (at most kMergeMaxWaves); wave w takes the
// contiguous slices [k0, k1).  Inside a wave, lane (part, c) handles dim
// MD q + c and the slices k0 + part, k0 + part + NP, ... (NP = 64 / MD
// parts): it takes their maxima, weights and sums in slice order, and the
// parts are combined by a fixed butterfly of shuffles, so every lane of a
// dim ends with the same sums.  Wave 0 then rescales and adds the waves'
// sums in wave order.  Results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mac_dev.h"
#include "mac_launch.h"
#include "match.h"
#include "merge_map.h"

namespace mac {

constexpr int kMergeMaxWaves = 16;
constexpr int kMergeSlicesPerWave = 32;  // slices per wave up to 512 slices per group
constexpr int kMergeDims = 16;           // dims per workgroup (MD)

// Waves per merge workgroup: one per 32 slices of the group, at most 16
// (then up to 64 slices per wave).
__host__ __device__ inline int merge_waves(int S) {
  const int w = (S + kMergeSlicesPerWave - 1) / kMergeSlicesPerWave;
  return w < kMergeMaxWaves ? w : kMergeMaxWaves;
}

template <int MD>
struct MergeShared {
  float m[kMergeMaxWaves][2];   // per wave: maxima of its slices before / after p_new
  float l[kMergeMaxWaves][2];
  float o[kMergeMaxWaves][2][MD];
};

// PER: slices per lane, ceil(slices per wave / NP).
template <typename T, int D, int MD, int PER>
__global__ __launch_bounds__(64 * kMergeMaxWaves) void merge_kernel(StepArgs a) {
  constexpr int QP = D / MD;                    // workgroups per query head
  constexpr int NP = 64 / MD;                   // parts of a wave
  // ids run group-major (merge_coords): with a multiple of 8 groups a
  // group's merge workgroups share the XCD its step workgroups ran on,
  // whose L2 holds the partial states they wrote
  const MergeCoords mc = merge_coords(blockIdx.x, a.batch, a.hkv, a.group, QP);
  const int grp = mc.grp, b = mc.b, h = mc.h, hi = mc.hi, q = mc.q;
  const int G = a.group;
  const int bh = b * a.hq + h;
  const int S = a.part.S;
  const int nw = blockDim.x / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int part = lane / MD, c = lane % MD;
  const int dim = q * MD + c;
  const RingView& R = a.ring;
  __shared__ MergeShared<MD> xs;

  const size_t pbase = (size_t)grp * S * G + hi;        // slice k: pbase + k * G
  const int spw = (S + nw - 1) / nw;                    // <= NP * PER
  const int k0 = wave * spw;
  const int k1 = k0 + spw < S ? k0 + spw : S;

  // ---- the loads, one round: the group's starts (lane i < G: head i's;
  // one vector load), this lane's slices' (m, l) and o, the query the entry
  // copies, and the reused state as the step (or match) kernel copied it
  const HeadState* hsg = a.heads + (size_t)b * a.hq + (size_t)(h - hi);
  const int s_lane = hsg[lane < G ? lane : 0].s;
  const float2* pml = reinterpret_cast<const float2*>(a.part.ml);
  float2 ml[PER];
  float ob[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = k0 + NP * i + part < S ? k0 + NP * i + part : S - 1;
    ml[i] = pml[pbase + (size_t)k * G];
    ob[i] = a.part.o[(pbase + (size_t)k * G) * D + dim];
  }
  const T qv = static_cast<const T*>(a.q_pre)[(size_t)bh * D + dim];
  const float2 rml = reinterpret_cast<const float2*>(a.reuse_ml)[bh];
  const float ro = a.reuse_o[(size_t)bh * D + dim];
  const HeadState hs = hsg[hi];
  const int lo = wave_min_i(s_lane);
  const int n = hs.n;
  const Plan p = make_plan(lo, n, a.band, S, a.part.first);
  const int npart = p.n_pre + p.n_post;
  const int ke = k1 < npart ? k1 : npart;               // this wave's live slices: [k0, ke)

  // ---- the wave's maxima of its live slices before and after p_new
  float MA = neg_inf(), MC = neg_inf();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = k0 + NP * i + part;
    if (k < ke) {
      if (slice_is_pre(p, k)) MA = fmaxf(MA, ml[i].x);
      else MC = fmaxf(MC, ml[i].x);
    }
  }
#pragma unroll
  for (int x = MD; x < 64; x *= 2) {
    MA = fmaxf(MA, shfl_xor_f(MA, x));
    MC = fmaxf(MC, shfl_xor_f(MC, x));
  }
  // ---- weights relative to them; sums of l and of o (unnormalized), each
  // part in slice order, then the parts by the butterfly
  float LA = 0.f, LC = 0.f, oa = 0.f, oc = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = k0 + NP * i + part;
    if (k < ke) {
      const bool pre = slice_is_pre(p, k);
      const float w = ml[i].x == neg_inf() ? 0.f : fast_exp2(ml[i].x - (pre ? MA : MC));
      if (pre) {
        LA += w * ml[i].y;
        oa += w * ob[i];
      } else {
        LC += w * ml[i].y;
        oc += w * ob[i];
      }
    }
  }
#pragma unroll
  for (int x = MD; x < 64; x *= 2) {
    LA += shfl_xor_f(LA, x);
    LC += shfl_xor_f(LC, x);
    oa += shfl_xor_f(oa, x);
    oc += shfl_xor_f(oc, x);
  }

  // ---- more than one wave: the waves' sums, rescaled to the largest
  // maximum and added in wave order by wave 0
  if (nw > 1) {
    if (lane == 0) {
      xs.m[wave][0] = MA;
      xs.m[wave][1] = MC;
      xs.l[wave][0] = LA;
      xs.l[wave][1] = LC;
    }
    if (lane < MD) {
      xs.o[wave][0][lane] = oa;
      xs.o[wave][1][lane] = oc;
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

  // ---- the head's new ring entry (this workgroup's dims of it) and out
  const size_t we = (size_t)bh * R.slots + hs.cnt % R.slots;
  const float M = fmaxf(MP, MC);
  const float sp = MP == neg_inf() ? 0.f : fast_exp2(MP - M);
  const float sc = MC == neg_inf() ? 0.f : fast_exp2(MC - M);
  const float den = sp * LP + sc * LC;
  if (lane < MD) {
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
    // fused append: publish the new length (no kernel of this step reads it
    // after the step kernel)
    if (a.k_new && h == 0) a.seq_lens[b] = n;
    // the group's published plan start is spent: clear it, so that every
    // step begins with no plan published and no later step (of this context
    // or of another one the workspace serves next) can take this one
    if (hi == 0 && a.part.first < a.part.S) a.plan_pub[grp] = ~0ull;
  }
}

hipError_t launch_merge(const StepArgs& a, int dtype, int d, hipStream_t st) {
  constexpr int NP = 64 / kMergeDims;
  const int S = a.part.S;
  const int nw = merge_waves(S);
  const int spw = (S + nw - 1) / nw;
  // up to 32 slices per wave, or up to 64 (more than 512 slices per group)
#define L_MERGE(T, D)                                                                            \
  if (spw > kMergeSlicesPerWave)                                                                 \
    hipLaunchKernelGGL((merge_kernel<T, D, kMergeDims, 64 / NP>),                                \
                       dim3(a.batch * a.hq * (D / kMergeDims)), dim3(64 * nw), 0, st, a);        \
  else                                                                                           \
    hipLaunchKernelGGL((merge_kernel<T, D, kMergeDims, kMergeSlicesPerWave / NP>),               \
                       dim3(a.batch * a.hq * (D / kMergeDims)), dim3(64 * nw), 0, st, a)
  MAC_DISPATCH(dtype, d, L_MERGE);
#undef L_MERGE
  return hipGetLastError();
}

}  // namespace mac
