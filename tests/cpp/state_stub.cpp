// Host test of libmac's error states: the C ABI (mac_api.hip) linked
// against stand-ins for its kernel launchers, which succeed until told to
// fail.  A device error reported by a launch must poison the context: the
// call returns MAC_ERR_DEVICE with the HIP code in the message, and every
// later call on that context returns MAC_ERR_STATE without launching
// anything.  No GPU is needed (nothing reaches the device).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "../../include/mac.h"
#include "../../kv_cache_reuse_amd/csrc/mac_launch.h"

static int launches = 0;          // launcher calls so far
static int fail_at = -1;          // the launcher call that fails (-1: none)
static hipError_t fail_code = hipErrorLaunchFailure;

static hipError_t outcome() {
  const int i = launches++;
  return i == fail_at ? fail_code : hipSuccess;
}

namespace mac {
hipError_t launch_step(const StepArgs&, int, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  return outcome();
}
hipError_t launch_append(void*, void*, const int32_t*, const void*, const void*, int32_t*,
                         const KvGeom&, int, int, hipStream_t) { return outcome(); }
hipError_t launch_prefill(void*, void*, const int32_t*, const void*, const void*, int32_t*, int,
                          int, const KvGeom&, int, hipStream_t) { return outcome(); }
hipError_t launch_read(const void*, const void*, const int32_t*, void*, void*, int, int, int,
                       const KvGeom&, int, hipStream_t) { return outcome(); }
hipError_t launch_fill_i32(int32_t*, int, int32_t, hipStream_t) { return outcome(); }
hipError_t launch_seed_len(int32_t*, int32_t*, int, int, int, hipStream_t) { return outcome(); }
hipError_t launch_inv_freq(double*, int, double, hipStream_t) { return outcome(); }
hipError_t launch_push(const RingView&, int, int, int, int, const void*, const float*,
                       const float*, const float*, const int32_t*, const int32_t*,
                       const uint8_t*, hipStream_t) { return outcome(); }
}  // namespace mac

static int fails = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::printf("FAIL line %d: %s (last error: %s)\n", __LINE__, #cond,         \
                  mac_last_error());                                              \
      ++fails;                                                                    \
    }                                                                             \
  } while (0)

int main() {
  mac_config c;
  std::memset(&c, 0, sizeof c);
  c.batch = 2;
  c.n_q_heads = 8;
  c.n_kv_heads = 2;
  c.head_dim = 128;
  c.dtype = MAC_DTYPE_BF16;
  c.max_context = 4096;
  c.window = 8;
  c.band = 64;
  c.tau = 4.0f;
  c.rope_theta = 5e5;
  // plausible, aligned, never dereferenced device addresses
  void* dev = reinterpret_cast<void*>(0x100000);
  void* ws = reinterpret_cast<void*>(0x200000);
  int32_t* lens = reinterpret_cast<int32_t*>(0x300000);
  const int32_t host[2] = {100, 200};
  const int32_t full[2] = {4096, 4096};

  // a device error while creating the context: no context, MAC_ERR_DEVICE
  mac_ctx* ctx = nullptr;
  launches = 0;
  fail_at = 0;
  EXPECT(mac_init(&c, dev, ws, lens, host, nullptr, &ctx) == MAC_ERR_DEVICE);
  EXPECT(ctx == nullptr);
  EXPECT(std::strstr(mac_last_error(), "HIP error") != nullptr);

  // a context that works until its append fails
  launches = 0;
  fail_at = -1;
  EXPECT(mac_init(&c, dev, ws, lens, host, nullptr, &ctx) == MAC_OK);
  EXPECT(ctx != nullptr);
  EXPECT(mac_append_kv(ctx, dev, dev, nullptr, dev, dev, nullptr) == MAC_OK);
  EXPECT(mac_decode_step(ctx, dev, dev, dev, nullptr, reinterpret_cast<float*>(dev), nullptr,
                         nullptr, nullptr) == MAC_OK);
  // argument errors come before any launch and do not poison the context
  EXPECT(mac_decode_step(ctx, nullptr, dev, dev, nullptr, reinterpret_cast<float*>(dev),
                         nullptr, nullptr, nullptr) == MAC_ERR_INVALID_ARG);
  const int before = launches;
  fail_at = launches;
  fail_code = hipErrorIllegalAddress;
  EXPECT(mac_append_kv(ctx, dev, dev, nullptr, dev, dev, nullptr) == MAC_ERR_DEVICE);
  EXPECT(std::strstr(mac_last_error(), "mac_append_kv") != nullptr);
  char code[32];
  std::snprintf(code, sizeof code, "HIP error %d", static_cast<int>(hipErrorIllegalAddress));
  EXPECT(std::strstr(mac_last_error(), code) != nullptr);
  EXPECT(launches == before + 1);
  fail_at = -1;
  // every call on the poisoned context is refused, and nothing is launched
  EXPECT(mac_append_kv(ctx, dev, dev, nullptr, dev, dev, nullptr) == MAC_ERR_STATE);
  EXPECT(mac_decode_step(ctx, dev, dev, dev, nullptr, reinterpret_cast<float*>(dev), nullptr,
                         nullptr, nullptr) == MAC_ERR_STATE);
  EXPECT(mac_decode_step_append(ctx, dev, dev, dev, dev, dev, nullptr,
                                reinterpret_cast<float*>(dev), nullptr, nullptr,
                                nullptr) == MAC_ERR_STATE);
  EXPECT(mac_prefill_kv(ctx, dev, dev, nullptr, 0, dev, dev, 16, nullptr) == MAC_ERR_STATE);
  EXPECT(mac_read_kv(ctx, dev, dev, nullptr, 0, 0, 16, dev, dev, nullptr) == MAC_ERR_STATE);
  EXPECT(mac_seed_ring(ctx, dev, 1, dev, dev, nullptr, nullptr) == MAC_ERR_STATE);
  EXPECT(mac_query_cache_push(ctx, dev, reinterpret_cast<float*>(dev),
                              reinterpret_cast<float*>(dev), reinterpret_cast<float*>(dev),
                              lens, lens, nullptr, nullptr) == MAC_ERR_STATE);
  EXPECT(mac_profile_enable(ctx, 1) == MAC_ERR_STATE);
  EXPECT(std::strstr(mac_last_error(), "earlier device error") != nullptr);
  EXPECT(launches == before + 1);
  EXPECT(mac_destroy(ctx) == MAC_OK);

  // a failed decode launch poisons too; another context is unaffected
  mac_ctx* other = nullptr;
  launches = 0;
  EXPECT(mac_init(&c, dev, ws, lens, host, nullptr, &ctx) == MAC_OK);
  EXPECT(mac_resume(&c, dev, ws, lens, host, nullptr, &other) == MAC_OK);
  fail_at = launches;
  EXPECT(mac_decode_step(ctx, dev, dev, dev, nullptr, reinterpret_cast<float*>(dev), nullptr,
                         nullptr, nullptr) == MAC_ERR_DEVICE);
  EXPECT(mac_decode_step(ctx, dev, dev, dev, nullptr, reinterpret_cast<float*>(dev), nullptr,
                         nullptr, nullptr) == MAC_ERR_STATE);
  EXPECT(mac_decode_step(other, dev, dev, dev, nullptr, reinterpret_cast<float*>(dev), nullptr,
                         nullptr, nullptr) == MAC_OK);
  EXPECT(mac_destroy(ctx) == MAC_OK);
  // capacity is checked on the host mirror before any launch
  EXPECT(mac_destroy(other) == MAC_OK);
  EXPECT(mac_init(&c, dev, ws, lens, full, nullptr, &ctx) == MAC_OK);
  const int n0 = launches;
  EXPECT(mac_append_kv(ctx, dev, dev, nullptr, dev, dev, nullptr) == MAC_ERR_CAPACITY);
  EXPECT(mac_decode_step_append(ctx, dev, dev, dev, dev, dev, nullptr,
                                reinterpret_cast<float*>(dev), nullptr, nullptr,
                                nullptr) == MAC_ERR_CAPACITY);
  EXPECT(launches == n0);
  EXPECT(mac_destroy(ctx) == MAC_OK);

  if (fails) return 1;
  std::printf("OK\n");
  return 0;
}
