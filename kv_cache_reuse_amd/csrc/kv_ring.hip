// libmac kernels for gfx950 (MI355X): KV-cache tile writes and reads, ring
// pushes and small set-up fills.  The decode step itself is in step.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mac_dev.h"
#include "mac_launch.h"

namespace mac {

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
    kc[base + k_elem_offset<T>(geom, r, dim)] = kn[src];
    vc[base + v_elem_offset<T>(geom, r, dim)] = vn[src];
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
  kc[base + k_elem_offset<T>(geom, pos % kTile, dim)] = ks[src];
  vc[base + v_elem_offset<T>(geom, pos % kTile, dim)] = vs[src];
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
  kd[dst] = kc[base + k_elem_offset<T>(geom, pos % kTile, dim)];
  vd[dst] = vc[base + v_elem_offset<T>(geom, pos % kTile, dim)];
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

// Sequence lengths around ring seeding: mode 0 saves them, mode 1 sets each
// to its saved value plus `offset`, mode 2 restores them.
__global__ void seed_len_kernel(int32_t* lens, int32_t* saved, int batch, int mode, int offset) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  if (mode == 0) saved[b] = lens[b];
  else if (mode == 1) lens[b] = saved[b] + offset;
  else lens[b] = saved[b];
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

hipError_t launch_seed_len(int32_t* lens, int32_t* saved, int batch, int mode, int offset,
                           hipStream_t st) {
  hipLaunchKernelGGL(seed_len_kernel, dim3((batch + 255) / 256), dim3(256), 0, st, lens, saved,
                     batch, mode, offset);
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
