// Streaming-read probe (measurement only, not part of the decode path): the
// HBM read rate a plain, fully coalesced read kernel reaches on this device.
// The benchmark reports the decode step's bandwidth against it next to the
// published peak.  Built into its own library, libmac_bw.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Each workgroup streams its own contiguous chunk of the buffer, every thread
// keeping 8 16-byte loads in flight, and folds them with xor; the fold is
// stored only when it equals a value the caller passes (practically never),
// which keeps the loads alive.  NT: non-temporal loads (lines not kept for
// reuse), the policy the decode step streams its long key ranges with.
template <bool NT>
__device__ __forceinline__ u4 load16(const u4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u4* __restrict__ buf, size_t n16,
                                                   uint32_t* sink, uint32_t magic) {
  const size_t per = n16 / gridDim.x;
  const u4* p = buf + (size_t)blockIdx.x * per;
  const size_t end = blockIdx.x + 1 == gridDim.x ? n16 - (size_t)blockIdx.x * per : per;
  u4 acc = {0u, 0u, 0u, 0u};
  size_t i = threadIdx.x;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    u4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = load16<NT>(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < end; i += 256) acc ^= load16<NT>(p + i);
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == magic) sink[blockIdx.x] = x;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the device buffer `buf` with `blocks`
// workgroups of 256 threads on `stream`, with non-temporal loads if
// `nontemporal` is nonzero.  `sink` is a device array of `blocks` words,
// written only where a chunk's xor equals `magic`.  Returns the HIP error
// code.
extern "C" int mac_bw_read(const void* buf, size_t bytes, uint32_t* sink, uint32_t magic,
                           int blocks, int nontemporal, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u4* p = static_cast<const u4*>(buf);
  if (nontemporal) hipLaunchKernelGGL(read_kernel<true>, dim3(blocks), dim3(256), 0, st, p, bytes / 16, sink, magic);
  else hipLaunchKernelGGL(read_kernel<false>, dim3(blocks), dim3(256), 0, st, p, bytes / 16, sink, magic);
  return (int)hipGetLastError();
}
