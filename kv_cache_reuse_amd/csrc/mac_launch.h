// Host-side launchers of the libmac kernels (internal C++ interface).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "mac_dev.h"

namespace mac {

// Launch of a step's attention kernel.  With timing events, they are bound
// to the kernel's own dispatch (recorded when it starts and when it ends), so
// the measured time holds the kernel alone, also when the host enqueues
// slower than the GPU runs.
template <typename K>
inline void launch_attention(K kernel, dim3 grid, dim3 block, hipStream_t st, hipEvent_t ev0,
                             hipEvent_t ev1, const StepArgs& a) {
  if (ev0) hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev0, ev1, 0, a);
  else hipLaunchKernelGGL(kernel, grid, block, 0, st, a);
}

// match -> split-K attention -> merge, on `st`.  If ev0/ev1 are non-null they
// time the split-K attention kernel (launch_attention).
hipError_t launch_step(const StepArgs& a, int dtype, int d, int paged, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1);

// The merge launch of a step (merge.hip): log-sum-exp merge of each query
// head's reused state and slices, its new ring entry and its output.
hipError_t launch_merge(const StepArgs& a, int dtype, int d, hipStream_t st);

// Wide groups (bf16, more than kMaxGroup heads per group): the match of
// every query head (records, rotated queries, reused states) and the split-K
// attention that reads them (wide.hip).
hipError_t launch_match_wide(const StepArgs& a, int d, hipStream_t st);
hipError_t launch_step_wide(const StepArgs& a, int d, int paged, hipStream_t st,
                            hipEvent_t ev0, hipEvent_t ev1);

hipError_t launch_append(void* kc, void* vc, const int32_t* pt, const void* kn, const void* vn,
                         int32_t* seq_lens, const KvGeom& geom, int batch, int dtype,
                         hipStream_t st);

hipError_t launch_prefill(void* kc, void* vc, const int32_t* pt, const void* ks, const void* vs,
                          int32_t* seq_lens, int seq, int count, const KvGeom& geom, int dtype,
                          hipStream_t st);

hipError_t launch_read(const void* kc, const void* vc, const int32_t* pt, void* kd, void* vd,
                       int seq, int start, int count, const KvGeom& geom, int dtype,
                       hipStream_t st);

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);

// mode 0: saved = lens; 1: lens = saved + offset; 2: lens = saved
hipError_t launch_seed_len(int32_t* lens, int32_t* saved, int batch, int mode, int offset,
                           hipStream_t st);

hipError_t launch_inv_freq(double* out, int d, double theta, hipStream_t st);

hipError_t launch_push(const RingView& R, int batch, int hq, int d, int dtype, const void* q,
                       const float* o, const float* m, const float* l, const int32_t* pe,
                       const int32_t* ne, const uint8_t* mask, hipStream_t st);

}  // namespace mac
