// libmac kernels for gfx950 (MI355X): the MAC-Attention decode step.
//
// Method: "MAC-Attention: a Match-Amend-Complete Scheme for Fast and
// Accurate Attention Computation", abstract (match stage, amend stage,
// complete stage with a numerically stable merge; constant cost on a hit).
//
// One decode step is three launches on the caller's stream:
//   1. match_kernel   one wave per (sequence, query head): rotary embedding of
//                     q (float64 angles), L2 distances to the ring's last W
//                     pre-RoPE queries, argmin and threshold, the head's plan.
//   2. attn_partial   split-K attention: one workgroup per (slice, KV group)
//                     over a fixed grid; every workgroup derives its key range
//                     from the match results, so a hit reads only the band and
//                     the tail while a miss spreads [0, n) over all slices.
//                     QK^T and PV run on the matrix cores (16x16 tiles).
//   3. merge_kernel   per (sequence, query head): log-sum-exp merge of the
//                     reused state and the prefix slices (written back as the
//                     head's new ring entry), then of the tail slices (out).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mac_dev.h"
#include "mac_launch.h"

namespace mac {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr double kLog2e = 1.4426950408889634074;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ int ring_slot(int count, int k, int slots) {
  // slot of the k-th most recent entry; count - 1 - k >= 0 by construction
  return (count - 1 - k) % slots;
}

// Smallest fresh-range start over the query heads of one KV group.
__device__ __forceinline__ void group_starts(const StepArgs& a, int b, int kvh, int* lo, int* smax) {
  const HeadPlan* hp = a.plan + (size_t)b * a.hq + (size_t)kvh * a.group;
  int mn = hp[0].s, mx = hp[0].s;
  for (int i = 1; i < a.group; ++i) {
    mn = min(mn, hp[i].s);
    mx = max(mx, hp[i].s);
  }
  *lo = mn;
  *smax = mx;
}

// ===================================================================== 1 ==
// Match: one 64-lane wave per (b, h).
template <typename T, int D>
__global__ __launch_bounds__(64) void match_kernel(StepArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.hq, h = bh % a.hq;
  const int lane = threadIdx.x;
  int n = a.seq_lens[b];
  if (a.k_new) {
    // fused append: the first query head of each KV group stores the group's
    // new key and value at position n (skipped if the sequence is full, which
    // the host rules out except when a captured step is replayed too often)
    const int n0 = n;
    if (n0 >= 0 && n0 < a.geom.capacity) {
      n = n0 + 1;
      if (h % a.group == 0) {
        const int kvh = h / a.group;
        const int64_t base = tile_base_w(a.geom, a.page_table, b, kvh, n0 / kTile);
        if (base >= 0) {
          const size_t src = ((size_t)b * a.hkv + kvh) * D;
          T* kc = const_cast<T*>(static_cast<const T*>(a.k_cache));
          T* vc = const_cast<T*>(static_cast<const T*>(a.v_cache));
          for (int e = lane; e < D; e += 64) {
            kc[base + k_tile_offset<T>(n0 % kTile, e)] = static_cast<const T*>(a.k_new)[src + e];
            vc[base + v_tile_offset<T>(n0 % kTile, e)] = static_cast<const T*>(a.v_new)[src + e];
          }
        }
      }
    }
  }
  if (h == 0 && lane == 0) a.n_step[b] = n;
  const int pos = n - 1;
  const int p_new = n - a.band > 0 ? n - a.band : 0;
  const T* q = static_cast<const T*>(a.q_pre) + (size_t)bh * D;

  // Rotary embedding, rotate-half pairs (i, i + D/2), one pair per lane.
  // Angles and the rotation in float64 (frequencies from a float64 table);
  // the result is scaled by log2(e)/sqrt(D) so the attention kernel can use
  // exp2.
  if (lane < D / 2) {
    const int i = lane;
    const double inv = a.inv_freq[i];
    double sn, cs;
    sincos(static_cast<double>(pos) * inv, &sn, &cs);
    const double x1 = Elem<T>::to_f(q[i]);
    const double x2 = Elem<T>::to_f(q[i + D / 2]);
    const double c = kLog2e / sqrt(static_cast<double>(D));
    const float r1 = static_cast<float>((x1 * cs - x2 * sn) * c);
    const float r2 = static_cast<float>((x2 * cs + x1 * sn) * c);
    if constexpr (sizeof(T) == 2) {
      uint16_t* hi = static_cast<uint16_t*>(a.qfrag) + (size_t)bh * D;
      uint16_t* lo = static_cast<uint16_t*>(a.qfrag) + (size_t)a.batch * a.hq * D + (size_t)bh * D;
      const uint16_t h1 = f32_to_bf16(r1), h2 = f32_to_bf16(r2);
      hi[i] = h1;
      hi[i + D / 2] = h2;
      lo[i] = f32_to_bf16(r1 - bf16_to_f32(h1));
      lo[i + D / 2] = f32_to_bf16(r2 - bf16_to_f32(h2));
    } else {
      float* qs = static_cast<float*>(a.qfrag) + (size_t)bh * D;
      qs[i] = r1;
      qs[i + D / 2] = r2;
    }
  }

  // Match: lanes [16 g, 16 g + 16) handle ring entry k0 + g, each lane D/16
  // elements; the squared distance is reduced over the 16 lanes.
  constexpr int EPL = D / 16;
  const int gi = lane / 16, c = lane % 16;
  const RingView& R = a.ring;
  const int cnt = R.count[bh];
  const int nvalid = cnt < R.window ? cnt : R.window;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = Elem<T>::to_f(q[c * EPL + e]);

  // Entries are processed in batches of 4 x kBatch, all of a batch's loads
  // issued before any is used, so a window of up to 32 entries costs one
  // memory round trip.
  constexpr int kBatch = 8;
  float best = __builtin_inff();
  int bestk = -1;
  for (int k0 = 0; k0 < nvalid; k0 += 4 * kBatch) {
    T rv[kBatch][EPL];
    int pe[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = k0 + 4 * u + gi;
      const bool ok = k < nvalid;
      const int slot = ok ? ring_slot(cnt, k, R.slots) : 0;
      const T* rq = static_cast<const T*>(R.q) + ((size_t)bh * R.slots + slot) * D + c * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) rv[u][e] = ok ? rq[e] : T(0);
      pe[u] = ok ? R.pn[((size_t)bh * R.slots + slot) * 2] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = k0 + 4 * u + gi;
      float d2 = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float df = qv[e] - Elem<T>::to_f(rv[u][e]);
        d2 = fmaf(df, df, d2);
      }
      d2 += shfl_xor_f(d2, 1);
      d2 += shfl_xor_f(d2, 2);
      d2 += shfl_xor_f(d2, 4);
      d2 += shfl_xor_f(d2, 8);
      const bool cand = k < nvalid && pe[u] >= 0 && pe[u] <= p_new && d2 == d2;
      if (cand && d2 < best) {      // newer entries come first: ties keep the newer
        best = d2;
        bestk = k;
      }
    }
  }
  // combine the four lane groups: smallest distance, then newest entry
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const float ob = shfl_xor_f(best, off);
    const int ok = shfl_xor_i(bestk, off);
    if (ok >= 0 && (bestk < 0 || ob < best || (ob == best && ok < bestk))) {
      best = ob;
      bestk = ok;
    }
  }
  if (lane == 0) {
    const bool hit = bestk >= 0 && best < a.tau2;
    HeadPlan hp;
    hp.hit = hit ? 1 : 0;
    hp.slot = hit ? ring_slot(cnt, bestk, R.slots) : -1;
    hp.s = hit ? R.pn[((size_t)bh * R.slots + hp.slot) * 2] : 0;
    // claim this step's slot now: the match kernel is the only reader of the
    // counter within a step, and the merge kernel fills the slot later
    hp.wslot = cnt % R.slots;
    R.count[bh] = cnt + 1;
    a.plan[bh] = hp;
    if (a.match_ctx_out) a.match_ctx_out[bh] = hit ? R.pn[((size_t)bh * R.slots + hp.slot) * 2 + 1] : -1;
    if (a.dist_out) a.dist_out[bh] = bestk >= 0 ? sqrtf(best) : __builtin_inff();
  }
}

// ===================================================================== 2 ==
// Split-K partial attention over one slice of one KV group.
//
// Workgroup = 4 waves; wave w takes tiles t0 + w, t0 + w + 4, ... of the
// slice.  Per 16-token tile a wave computes S = K Q^T (16 tokens x 16 padded
// heads) and O^T += V^T P^T on the matrix cores.  Lane (lg, c) (lg = lane/16,
// c = lane%16) holds scores of tokens 4 lg .. 4 lg + 3 for head c, which is
// exactly the B operand layout of the PV product, so no data moves between
// lanes except the per-head running max (two xor shuffles per tile).
//
// bf16: q is split into hi + lo bf16 parts (and so is P), each product is
// two MFMAs, which keeps scores and weights at about 16 significant bits.
// fp32: the 16x16x4 fp32 MFMA, no split.
template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(256) void attn_partial_kernel(StepArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int NL = D * (int)sizeof(T) / 64;   // 1 KiB blocks per tile, K and V each
  constexpr int NQ = BF ? 2 * NL : 4 * NL;      // QK MFMA steps per tile
  constexpr int NCT = D / 16;                   // 16-dim column tiles of O^T

  const int n_groups = a.batch * a.hkv;
  const int grp = blockIdx.x % n_groups;
  const int slice = blockIdx.x / n_groups;
  const int b = grp / a.hkv, kvh = grp % a.hkv;
  const int G = a.group;
  const int n = a.n_step[b];
  int lo, smax;
  group_starts(a, b, kvh, &lo, &smax);
  const Plan p = make_plan(lo, n, a.band, a.part.S);
  if (slice >= p.n_pre + p.n_post) return;
  int ka, ke;
  slice_range(p, slice, &ka, &ke);

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lg = lane / 16, col = lane % 16;
  const bool hv = col < G;
  const int h = kvh * G + (hv ? col : 0);
  const int s_col = hv ? a.plan[(size_t)b * a.hq + h].s : 0;

  // query fragments (B operand of S = K Q^T), zero for padding heads
  const size_t qoff = ((size_t)b * a.hq + h) * D;
  v4s qh[BF ? NQ : 1], ql[BF ? NQ : 1];
  float qf[BF ? 1 : NQ];
  if constexpr (BF) {
    const uint16_t* qhi = static_cast<const uint16_t*>(a.qfrag) + qoff;
    const uint16_t* qlo = static_cast<const uint16_t*>(a.qfrag) + (size_t)a.batch * a.hq * D + qoff;
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int d0 = 8 * (4 * j + lg) + 4 * hh;
        v4s x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
        if (hv) {
          x = *reinterpret_cast<const v4s*>(qhi + d0);
          y = *reinterpret_cast<const v4s*>(qlo + d0);
        }
        qh[2 * j + hh] = x;
        ql[2 * j + hh] = y;
      }
  } else {
    const float* qs = static_cast<const float*>(a.qfrag) + qoff;
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * j + e] = hv ? qs[4 * (4 * j + lg) + e] : 0.f;
  }

  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  KvGeom geom = a.geom;
  geom.paged = PAGED ? 1 : 0;

  v4f acc[NCT];
#pragma unroll
  for (int i = 0; i < NCT; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf();
  float lsum = 0.f;

  const int t0 = ka / kTile, t1 = (ke + kTile - 1) / kTile;
  u4 kr[NL], vr[NL], kn[NL], vn[NL];
  int t = t0 + wave;
  if (t < t1) {
    const int64_t base = tile_base(geom, a.page_table, b, kvh, t);
    const u4* kp = reinterpret_cast<const u4*>(kc + base) + lane;
    const u4* vp = reinterpret_cast<const u4*>(vc + base) + lane;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      kr[j] = kp[64 * j];
      vr[j] = vp[64 * j];
    }
  }
  for (; t < t1; t += 4) {
    const int tn = t + 4;
    if (tn < t1) {
      const int64_t base = tile_base(geom, a.page_table, b, kvh, tn);
      const u4* kp = reinterpret_cast<const u4*>(kc + base) + lane;
      const u4* vp = reinterpret_cast<const u4*>(vc + base) + lane;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        kn[j] = kp[64 * j];
        vn[j] = vp[64 * j];
      }
    }

    // ---- S = K Q^T : lane holds tokens 4 lg + r of head col
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
    const int tok0 = t * kTile;
    const bool full = tok0 >= ka && tok0 + kTile <= ke && tok0 >= smax;
    if (!full) {
      // Tokens outside [ka, ke) may be unwritten slots past the end of the
      // sequence: besides masking their scores, zero their values so that
      // 0 * (stale NaN/Inf) cannot enter the PV product.  The lane's V
      // fragment holds exactly its score tokens 4 lg + r.
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

    // ---- online softmax (base 2; scores carry the log2(e)/sqrt(d) scale)
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mnew = fmaxf(m, mx);
    if (mnew > m) {
      const float alpha = exp2f(m - mnew);
#pragma unroll
      for (int i = 0; i < NCT; ++i) acc[i] *= alpha;
      lsum *= alpha;
      m = mnew;
    }
    const float mref = m == neg_inf() ? 0.f : m;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = exp2f(s[r] - mref);
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

#pragma unroll
    for (int j = 0; j < NL; ++j) {
      kr[j] = kn[j];
      vr[j] = vn[j];
    }
  }
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);

  // ---- combine the four waves through LDS, write the slice's partial
  __shared__ float sm_m[4][kMaxGroup];
  __shared__ float sm_l[4][kMaxGroup];
  __shared__ float sm_o[4][kMaxGroup][D + 1];
  if (lg == 0) {
    sm_m[wave][col] = m;
    sm_l[wave][col] = lsum;
  }
#pragma unroll
  for (int i = 0; i < NCT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wave][col][16 * i + 4 * lg + r] = acc[i][r];
  __syncthreads();

  const size_t pbase = ((size_t)grp * a.part.S + slice) * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int hh = idx / D, dim = idx % D;
    float M = sm_m[0][hh];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][hh]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w][hh];
      const float sc = mw == neg_inf() ? 0.f : exp2f(mw - M);
      o += sc * sm_o[w][hh][dim];
      L += sc * sm_l[w][hh];
    }
    a.part.o[(pbase + hh) * D + dim] = o;
    if (dim == 0) {
      a.part.ml[(pbase + hh) * 2] = M;
      a.part.ml[(pbase + hh) * 2 + 1] = L;
    }
  }
}

// ===================================================================== 3 ==
// Merge: workgroup (b, h, chunk) of 256 threads owns dims
// [32 chunk, 32 chunk + 32) of head (b, h).  Every workgroup loads the m and
// l of all the group's slices at once (one memory round trip), turns them
// into weights in LDS, then its 8 x 32 threads fold the slices' o vectors
// with independent loads.  All reductions run in a fixed order, so results
// are bitwise reproducible.
constexpr int kMergeDims = 32;

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, shfl_xor_f(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += shfl_xor_f(v, off);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(StepArgs a) {
  constexpr int NCH = D / kMergeDims;
  constexpr int NSUB = 256 / kMergeDims;
  const int bh = blockIdx.x / NCH, chunk = blockIdx.x % NCH;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.group;
  const int kvh = h / G, hl = h % G;
  const int n = a.n_step[b];
  int lo, smax;
  group_starts(a, b, kvh, &lo, &smax);
  const Plan p = make_plan(lo, n, a.band, a.part.S);
  const HeadPlan hp = a.plan[bh];
  const RingView& R = a.ring;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  // fused append: publish the new length once every reader of the old one
  // (the match kernel) has finished; no kernel of this step reads it again
  if (a.k_new && h == 0 && chunk == 0 && tid == 0) a.seq_lens[b] = n;
  const int npart = p.n_pre + p.n_post;
  // partial i of this head: index (pbase + i * G)
  const size_t pbase = (size_t)(b * a.hkv + kvh) * a.part.S * G + hl;

  __shared__ float sw[kMaxSlices];
  __shared__ float sl[kMaxSlices];
  __shared__ float red[4][4];
  __shared__ float sm_pre[NSUB][kMergeDims];
  __shared__ float sm_post[NSUB][kMergeDims];

  // reused state: ring stores natural-log m and normalized o
  float mr = neg_inf(), lr = 0.f;
  size_t re = 0;
  if (hp.hit) {
    re = (size_t)bh * R.slots + hp.slot;
    const float mn = R.ml[re * 2];
    lr = R.ml[re * 2 + 1];
    mr = mn == neg_inf() ? neg_inf() : mn * static_cast<float>(kLog2e);
  }

  // ---- m, l of every slice; maxima of the prefix and the tail slices
  float mp = neg_inf(), mq = neg_inf();
  for (int i = tid; i < npart; i += 256) {
    const size_t idx = pbase + (size_t)i * G;
    const float mi = a.part.ml[idx * 2];
    sw[i] = mi;
    sl[i] = a.part.ml[idx * 2 + 1];
    if (i < p.n_pre) mp = fmaxf(mp, mi);
    else mq = fmaxf(mq, mi);
  }
  mp = wave_max(mp);
  mq = wave_max(mq);
  if (lane == 0) {
    red[0][wave] = mp;
    red[1][wave] = mq;
  }
  __syncthreads();
  const float Mpre = fmaxf(fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3])), mr);
  const float Mpost = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  const float Mall = fmaxf(Mpre, Mpost);

  // ---- weights (prefix slices relative to Mpre, tail slices to Mall), l sums
  float lp = 0.f, lq = 0.f;
  for (int i = tid; i < npart; i += 256) {
    const float mi = sw[i];
    const bool pre = i < p.n_pre;
    const float w = mi == neg_inf() ? 0.f : exp2f(mi - (pre ? Mpre : Mall));
    sw[i] = w;
    if (pre) lp += w * sl[i];
    else lq += w * sl[i];
  }
  lp = wave_sum(lp);
  lq = wave_sum(lq);
  __syncthreads();
  if (lane == 0) {
    red[2][wave] = lp;
    red[3][wave] = lq;
  }
  __syncthreads();
  const float wr = (hp.hit && mr != neg_inf()) ? exp2f(mr - Mpre) : 0.f;
  const float Lpre = ((red[2][0] + red[2][1]) + (red[2][2] + red[2][3])) + wr * lr;
  const float Lpost = (red[3][0] + red[3][1]) + (red[3][2] + red[3][3]);

  // ---- o: thread (sub, dd) folds slices sub, sub + 8, ...
  const int sub = tid / kMergeDims, dd = tid % kMergeDims;
  const int dim = chunk * kMergeDims + dd;
  float op = 0.f, oq = 0.f;
  for (int i0 = sub; i0 < npart; i0 += 4 * NSUB) {
    float ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NSUB;
      ov[u] = i < npart ? a.part.o[(pbase + (size_t)i * G) * D + dim] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NSUB;
      if (i < npart) {
        if (i < p.n_pre) op += sw[i] * ov[u];
        else oq += sw[i] * ov[u];
      }
    }
  }
  if (sub == 0 && hp.hit) op += wr * lr * R.o[re * D + dim];
  sm_pre[sub][dd] = op;
  sm_post[sub][dd] = oq;
  __syncthreads();
  if (sub != 0) return;
  float po = 0.f, qo = 0.f;
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    po += sm_pre[s][dd];
    qo += sm_post[s][dd];
  }

  // ---- the head's new ring entry: (q_pre, prefix state, p_new, n)
  const size_t we = (size_t)bh * R.slots + hp.wslot;
  R.o[we * D + dim] = Lpre == 0.f ? 0.f : po / Lpre;
  static_cast<T*>(R.q)[we * D + dim] = static_cast<const T*>(a.q_pre)[(size_t)bh * D + dim];
  if (chunk == 0 && dd == 0) {
    R.ml[we * 2] = Lpre == 0.f ? neg_inf() : Mpre * kLn2;
    R.ml[we * 2 + 1] = Lpre;
    R.pn[we * 2] = p.mid;
    R.pn[we * 2 + 1] = n;
  }

  // ---- out = merge(prefix, tail slices)
  const float sc = Mpre == neg_inf() ? 0.f : exp2f(Mpre - Mall);
  const float num = po * sc + qo;
  const float den = Lpre * sc + Lpost;
  a.out[(size_t)bh * D + dim] = den == 0.f ? 0.f : num / den;
}

// ============================================================ KV layout ==
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kernel(T* kc, T* vc, const int32_t* pt, const T* kn,
                                                     const T* vn, int32_t* seq_lens, KvGeom geom) {
  const int b = blockIdx.x;
  const int n0 = seq_lens[b];
  // a full sequence (possible only if a captured step is replayed past the
  // capacity the host checked) is left unchanged
  if (n0 < 0 || n0 >= geom.capacity) return;
  const int t = n0 / kTile, r = n0 % kTile;
  for (int idx = threadIdx.x; idx < geom.hkv * D; idx += blockDim.x) {
    const int g = idx / D, dim = idx % D;
    const int64_t base = tile_base_w(geom, pt, b, g, t);
    if (base < 0) continue;
    const size_t src = ((size_t)b * geom.hkv + g) * D + dim;
    kc[base + k_tile_offset<T>(r, dim)] = kn[src];
    vc[base + v_tile_offset<T>(r, dim)] = vn[src];
  }
  __syncthreads();
  if (threadIdx.x == 0) seq_lens[b] = n0 + 1;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_kernel(T* kc, T* vc, const int32_t* pt, const T* ks,
                                                      const T* vs, const int32_t* seq_lens, int seq,
                                                      int count, KvGeom geom) {
  const int g = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)count * D) return;
  const int tok = static_cast<int>(idx / D), dim = static_cast<int>(idx % D);
  const int pos = seq_lens[seq] + tok;
  if (pos < 0 || pos >= geom.capacity) return;
  const int64_t base = tile_base_w(geom, pt, seq, g, pos / kTile);
  if (base < 0) return;
  const size_t src = ((size_t)g * count + tok) * D + dim;
  kc[base + k_tile_offset<T>(pos % kTile, dim)] = ks[src];
  vc[base + v_tile_offset<T>(pos % kTile, dim)] = vs[src];
}

template <typename T, int D>
__global__ __launch_bounds__(256) void read_kernel(const T* kc, const T* vc, const int32_t* pt, T* kd,
                                                   T* vd, int seq, int start, int count, KvGeom geom) {
  const int g = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)count * D) return;
  const int tok = static_cast<int>(idx / D), dim = static_cast<int>(idx % D);
  const int pos = start + tok;
  const int64_t base = tile_base(geom, pt, seq, g, pos / kTile);
  const size_t dst = ((size_t)g * count + tok) * D + dim;
  kd[dst] = kc[base + k_tile_offset<T>(pos % kTile, dim)];
  vd[dst] = vc[base + v_tile_offset<T>(pos % kTile, dim)];
}

__global__ void add_len_kernel(int32_t* seq_lens, int seq, int count, int capacity) {
  const int n = seq_lens[seq] + count;
  seq_lens[seq] = n < capacity ? n : capacity;
}

// Rotary frequencies theta^(-2i/d), i < d/2, in float64 (once, at init).
__global__ void inv_freq_kernel(double* out, int d, double theta) {
  const int i = threadIdx.x;
  if (i < d / 2) out[i] = pow(theta, -2.0 * i / d);
}

hipError_t launch_inv_freq(double* out, int d, double theta, hipStream_t st) {
  hipLaunchKernelGGL(inv_freq_kernel, dim3(1), dim3(64), 0, st, out, d, theta);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void push_kernel(RingView R, int hq, const T* q, const float* o,
                                                   const float* m, const float* l, const int32_t* pe,
                                                   const int32_t* ne, const uint8_t* mask) {
  const int bh = blockIdx.x;
  if (mask && !mask[bh]) return;
  const int cnt = R.count[bh];
  const size_t we = (size_t)bh * R.slots + cnt % R.slots;
  for (int dim = threadIdx.x; dim < D; dim += blockDim.x) {
    static_cast<T*>(R.q)[we * D + dim] = q[(size_t)bh * D + dim];
    R.o[we * D + dim] = o[(size_t)bh * D + dim];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    R.ml[we * 2] = m[bh];
    R.ml[we * 2 + 1] = l[bh];
    R.pn[we * 2] = pe[bh];
    R.pn[we * 2 + 1] = ne[bh];
    R.count[bh] = cnt + 1;
  }
}

// ============================================================ launchers ==
#define MAC_DISPATCH(dtype, d, FN)                                         \
  do {                                                                     \
    if ((dtype) == 1 && (d) == 128) { FN(uint16_t, 128); }                 \
    else if ((dtype) == 1 && (d) == 64) { FN(uint16_t, 64); }              \
    else if ((dtype) == 0 && (d) == 128) { FN(float, 128); }               \
    else { FN(float, 64); }                                                \
  } while (0)

hipError_t launch_step(const StepArgs& a, int dtype, int d, int paged, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1) {
#define L_MATCH(T, D) hipLaunchKernelGGL((match_kernel<T, D>), dim3(a.batch * a.hq), dim3(64), 0, st, a)
  MAC_DISPATCH(dtype, d, L_MATCH);
#undef L_MATCH
  if (ev0) (void)hipEventRecord(ev0, st);
  const int grid = a.batch * a.hkv * a.part.S;
#define L_ATTN(T, D)                                                                          \
  if (paged) hipLaunchKernelGGL((attn_partial_kernel<T, D, true>), dim3(grid), dim3(256), 0, st, a); \
  else hipLaunchKernelGGL((attn_partial_kernel<T, D, false>), dim3(grid), dim3(256), 0, st, a)
  MAC_DISPATCH(dtype, d, L_ATTN);
#undef L_ATTN
  if (ev1) (void)hipEventRecord(ev1, st);
#define L_MERGE(T, D) hipLaunchKernelGGL((merge_kernel<T, D>), dim3(a.batch * a.hq * (D / kMergeDims)), dim3(256), 0, st, a)
  MAC_DISPATCH(dtype, d, L_MERGE);
#undef L_MERGE
  return hipGetLastError();
}

hipError_t launch_append(void* kc, void* vc, const int32_t* pt, const void* kn, const void* vn,
                         int32_t* seq_lens, const KvGeom& geom, int batch, int dtype,
                         hipStream_t st) {
#define L_APP(T, D)                                                                      \
  hipLaunchKernelGGL((append_kernel<T, D>), dim3(batch), dim3(256), 0, st, (T*)kc, (T*)vc, pt, \
                     (const T*)kn, (const T*)vn, seq_lens, geom)
  MAC_DISPATCH(dtype, geom.d, L_APP);
#undef L_APP
  return hipGetLastError();
}

hipError_t launch_prefill(void* kc, void* vc, const int32_t* pt, const void* ks, const void* vs,
                          int32_t* seq_lens, int seq, int count, const KvGeom& geom, int dtype,
                          hipStream_t st) {
  const int64_t total = (int64_t)count * geom.d;
  const dim3 grid((unsigned)((total + 255) / 256), geom.hkv);
#define L_PRE(T, D)                                                                            \
  hipLaunchKernelGGL((prefill_kernel<T, D>), grid, dim3(256), 0, st, (T*)kc, (T*)vc, pt, (const T*)ks, \
                     (const T*)vs, seq_lens, seq, count, geom)
  MAC_DISPATCH(dtype, geom.d, L_PRE);
#undef L_PRE
  hipLaunchKernelGGL(add_len_kernel, dim3(1), dim3(1), 0, st, seq_lens, seq, count, geom.capacity);
  return hipGetLastError();
}

hipError_t launch_read(const void* kc, const void* vc, const int32_t* pt, void* kd, void* vd,
                       int seq, int start, int count, const KvGeom& geom, int dtype,
                       hipStream_t st) {
  const int64_t total = (int64_t)count * geom.d;
  const dim3 grid((unsigned)((total + 255) / 256), geom.hkv);
#define L_RD(T, D)                                                                               \
  hipLaunchKernelGGL((read_kernel<T, D>), grid, dim3(256), 0, st, (const T*)kc, (const T*)vc, pt, \
                     (T*)kd, (T*)vd, seq, start, count, geom)
  MAC_DISPATCH(dtype, geom.d, L_RD);
#undef L_RD
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_push(const RingView& R, int batch, int hq, int d, int dtype, const void* q,
                       const float* o, const float* m, const float* l, const int32_t* pe,
                       const int32_t* ne, const uint8_t* mask, hipStream_t st) {
#define L_PUSH(T, D)                                                                          \
  hipLaunchKernelGGL((push_kernel<T, D>), dim3(batch * hq), dim3(128), 0, st, R, hq, (const T*)q, o, \
                     m, l, pe, ne, mask)
  MAC_DISPATCH(dtype, d, L_PUSH);
#undef L_PUSH
  return hipGetLastError();
}

}  // namespace mac
