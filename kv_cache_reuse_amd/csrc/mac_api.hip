// libmac C ABI: argument checks, buffer carving, host length mirror and
// launch orchestration.  The declarations and the contract are in
// include/mac.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/mac.h"
#include "mac_dev.h"
#include "mac_launch.h"

namespace {

thread_local std::string g_last_error;

mac_status fail(mac_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mac_status fail(mac_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mac_status ok() {
  g_last_error.clear();
  return MAC_OK;
}

// Split-K workgroups a miss step aims for: one workgroup per compute unit
// of a 256-CU part.
constexpr int kTargetWorkgroups = 256;
// Keys per slice of a full-length sequence that the default slice count
// aims for, by adding rounds of workgroups (at most kMaxRounds)
constexpr int64_t kSliceTarget = 4096;
constexpr int kMaxRounds = 4;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------ static scratch (noalloc) --
// mac_decode_step_append_noalloc keeps the scratch of a step in this array
// instead of the context's workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  Layout: kScratchPlanGroups plan words
// (all ones between steps), then the step scratch a workspace starts with
// (partial states, match records, reused ring states).
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kScratchPlanGroups = 4096;
constexpr size_t kScratchStepOffset = size_t(kScratchPlanGroups) * 8;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The array's device address on each device, resolved once per device (with
// that device current) by the first mac_init / mac_resume on it.  In host
// code `scratch` names a host-side stand-in: only these addresses are used.
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  bool resolved = false;
  hipError_t err = hipSuccess;
  char* ptr = nullptr;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

struct Layout {
  // ring: the entries, and the rotary table (per-context state kept beside
  // them, so that the workspace holds nothing from one step to the next)
  size_t r_count, r_q, r_o, r_ml, r_pn, r_invf, ring_bytes;
  // workspace
  size_t w_po, w_pml, w_heads, w_reuse, w_pub, w_out, w_save, ws_bytes;
  int slices;
  int first;            // slices per group in the first round of workgroups
  int64_t capacity;     // keys per sequence
  int ctx_stride;       // contiguous cache: token rows per (sequence, KV head)
};

int elem_size(int dtype) { return dtype == MAC_DTYPE_F32 ? 4 : 2; }

// Wide groups: bf16 caches with G > kMaxGroup query heads per KV head.  They
// are matched in a launch of their own and attended by workgroups of up to
// kWideGroup heads (two matrix-core column tiles); fp32 caches keep 16-head
// groups matched inside the attention workgroups.
bool wide_mode(const mac_config* c) {
  return c->dtype == MAC_DTYPE_BF16 && c->n_q_heads / c->n_kv_heads > mac::kMaxGroup;
}
// A KV head whose G query heads exceed one group is processed as nchunk
// groups of G / nchunk heads ("virtual" KV heads reading the same cache).
int chunk_cap(const mac_config* c) { return wide_mode(c) ? mac::kWideGroup : mac::kMaxGroup; }
int n_chunks(const mac_config* c) {
  const int G = c->n_q_heads / c->n_kv_heads;
  return (G + chunk_cap(c) - 1) / chunk_cap(c);
}
int chunk_heads(const mac_config* c) { return c->n_q_heads / c->n_kv_heads / n_chunks(c); }

mac_status check_config(const mac_config* c) {
  if (!c) return fail(MAC_ERR_INVALID_ARG, "config is NULL");
  if (c->batch < 1) return fail(MAC_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", c->batch);
  if (c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(MAC_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", c->n_q_heads,
                c->n_kv_heads);
  if (c->n_q_heads % c->n_kv_heads)
    return fail(MAC_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                c->n_q_heads, c->n_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(MAC_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->dtype != MAC_DTYPE_F32 && c->dtype != MAC_DTYPE_BF16)
    return fail(MAC_ERR_UNSUPPORTED, "dtype must be MAC_DTYPE_F32 or MAC_DTYPE_BF16 (got %d)", c->dtype);
  {
    const int G = c->n_q_heads / c->n_kv_heads;
    const int cap = chunk_cap(c);
    const int nc = (G + cap - 1) / cap;
    if (G % nc)
      return fail(MAC_ERR_UNSUPPORTED, "query heads per KV head (%d) above %d must split into "
                  "%d equal groups of at most %d", G, cap, nc, cap);
  }
  if (c->window < 0) return fail(MAC_ERR_INVALID_ARG, "window must be >= 0 (got %d)", c->window);
  if (c->band < 0) return fail(MAC_ERR_INVALID_ARG, "band must be >= 0 (got %d)", c->band);
  if (!(c->tau >= 0.f)) return fail(MAC_ERR_INVALID_ARG, "tau must be >= 0 (got %g)", (double)c->tau);
  if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta))
    return fail(MAC_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (c->max_slices != 0 && (c->max_slices < 2 || c->max_slices > mac::kMaxSlices))
    return fail(MAC_ERR_INVALID_ARG, "max_slices must be 0 (default) or in [2, %d] (got %d)",
                mac::kMaxSlices, c->max_slices);
  if (c->kv_layout != MAC_KV_TILES && c->kv_layout != MAC_KV_ROWS)
    return fail(MAC_ERR_INVALID_ARG, "kv_layout must be MAC_KV_TILES or MAC_KV_ROWS (got %d)",
                c->kv_layout);
  if (c->page_size == 0) {
    if (c->max_context < 1)
      return fail(MAC_ERR_INVALID_ARG, "max_context must be >= 1 (got %d)", c->max_context);
  } else if (c->page_size == mac::kTile) {
    if (c->max_pages_per_seq < 1 || c->n_pages < 1)
      return fail(MAC_ERR_INVALID_ARG, "paged cache needs max_pages_per_seq >= 1 and n_pages >= 1");
    if ((int64_t)c->max_pages_per_seq * mac::kTile > INT32_MAX)
      return fail(MAC_ERR_INVALID_ARG, "max_pages_per_seq too large");
  } else {
    return fail(MAC_ERR_UNSUPPORTED, "page_size must be 0 (contiguous) or 16 (got %d)", c->page_size);
  }
  return MAC_OK;
}

Layout layout(const mac_config* c) {
  Layout L{};
  const size_t bh = (size_t)c->batch * c->n_q_heads;
  const size_t slots = (size_t)c->window + 1;
  const size_t d = c->head_dim;
  const size_t es = elem_size(c->dtype);
  size_t off = 0;
  L.r_count = off; off = align256(off + bh * 4);
  L.r_q = off;     off = align256(off + bh * slots * d * es);
  L.r_o = off;     off = align256(off + bh * slots * d * 4);
  L.r_ml = off;    off = align256(off + bh * slots * 2 * 4);
  L.r_pn = off;    off = align256(off + bh * slots * 2 * 4);
  L.r_invf = off;  off = align256(off + (d / 2) * 8);
  L.ring_bytes = off;

  L.capacity = c->page_size ? (int64_t)c->max_pages_per_seq * mac::kTile : (int64_t)c->max_context;
  L.ctx_stride = c->page_size ? 0
                 : c->kv_layout == MAC_KV_ROWS ? c->max_context
                                               : mac::ceil_div(c->max_context, mac::kTile) * mac::kTile;
  const int groups = c->batch * c->n_kv_heads * n_chunks(c);   // matched groups
  int S = c->max_slices;
  L.first = 0;
  if (S == 0) {
    // enough slices to give every compute unit a workgroup, and further
    // rounds of as many when a full-length sequence's slices would otherwise
    // hold more than about 1.5 kSliceTarget keys: one round per kSliceTarget
    // keys a slice of the first round would hold, up to kMaxRounds.  With
    // one round, a batch step in which a few sequences miss waits for their
    // few workgroups to stream a quarter of a sequence each; the hardware
    // deals the later rounds to whichever units are free.  Each later round
    // costs a hit step about 1 us: its workgroups leave as soon as they read
    // the group's published plan start.
    const int base = mac::ceil_div(kTargetWorkgroups, groups);
    const int64_t per_round = (int64_t)base * kSliceTarget;
    int rounds = 1;
    if (L.capacity * 2 > per_round * 3) {
      const int64_t r = (L.capacity + per_round - 1) / per_round;
      rounds = r < kMaxRounds ? (int)r : kMaxRounds;
    }
    S = base * rounds;
    L.first = base;
    // never more slices than the longest context can fill
    const int cap = (int)((L.capacity + mac::kSliceMin - 1) / mac::kSliceMin) + 1;
    if (S > cap) S = cap;
    if (S > mac::kMaxSlices) S = mac::kMaxSlices;
    if (S < 2) S = 2;
  }
  const size_t G = chunk_heads(c);
  const size_t merge_cap = wide_mode(c) ? mac::kMergeCapWide : mac::kMergeCap;
  if (S * G > merge_cap) S = (int)(merge_cap / G);
  L.slices = S;
  if (L.first <= 0 || L.first > S) L.first = S;
  off = 0;
  L.w_po = off;      off = align256(off + (size_t)groups * S * G * d * 4);
  L.w_pml = off;     off = align256(off + (size_t)groups * S * G * 2 * 4);
  L.w_heads = off;   off = align256(off + bh * sizeof(mac::HeadState));
  // o rows, then (m, l) pairs, then (16-byte aligned) the wide path's
  // rotated query rows (bf16 hi and lo per head)
  L.w_reuse = off;   off = align256(off + bh * (d + 2) * 4 + 16 + bh * 2 * d * 2);
  L.w_out = off;   off = align256(off + bh * d * 4);          // ring seeding: discarded outputs
  L.w_save = off;  off = align256(off + (size_t)c->batch * 4); // ring seeding: saved lengths
  L.w_pub = off;   off = align256(off + (size_t)groups * 8);    // second round: published plans
  L.ws_bytes = off;
  return L;
}

}  // namespace

struct mac_ctx {
  mac_config cfg;
  Layout L;
  char* ring;
  char* ws;
  int32_t* seq_lens_dev;
  std::vector<int64_t> mirror;
  bool poisoned = false;
  bool profiling = false;
  char* scratch = nullptr;          // this device's static scratch, or null
  hipError_t scratch_err = hipSuccess;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
  size_t ev_used = 0;

  mac::RingView ring_view() const {
    mac::RingView R;
    R.count = reinterpret_cast<int32_t*>(ring + L.r_count);
    R.q = ring + L.r_q;
    R.o = reinterpret_cast<float*>(ring + L.r_o);
    R.ml = reinterpret_cast<float*>(ring + L.r_ml);
    R.pn = reinterpret_cast<int32_t*>(ring + L.r_pn);
    R.slots = cfg.window + 1;
    R.window = cfg.window;
    return R;
  }
  mac::KvGeom geom() const {
    mac::KvGeom g;
    g.hkv = cfg.n_kv_heads;
    g.d = cfg.head_dim;
    g.ctx_stride = L.ctx_stride;
    g.natural = cfg.kv_layout == MAC_KV_ROWS ? 1 : 0;
    g.paged = cfg.page_size ? 1 : 0;
    g.max_pages = cfg.max_pages_per_seq;
    g.n_pages = cfg.n_pages;
    g.capacity = (int)L.capacity;
    return g;
  }
};

namespace {

mac_status check_ctx(mac_ctx* ctx) {
  if (!ctx) return fail(MAC_ERR_INVALID_ARG, "context is NULL");
  if (ctx->poisoned) return fail(MAC_ERR_STATE, "context unusable after an earlier device error");
  return MAC_OK;
}

mac_status device_fail(mac_ctx* ctx, hipError_t e, const char* what) {
  if (ctx) ctx->poisoned = true;
  return fail(MAC_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

mac_status check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(MAC_ERR_INVALID_ARG, "%s is NULL", name) : MAC_OK;
  if (!aligned16(p)) return fail(MAC_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MAC_OK;
}

mac_status check_kv(mac_ctx* ctx, const void* k, const void* v, const int32_t* pt) {
  mac_status s;
  if ((s = check_ptr(k, "k_cache"))) return s;
  if ((s = check_ptr(v, "v_cache"))) return s;
  if (ctx->cfg.page_size) {
    if (!pt) return fail(MAC_ERR_INVALID_ARG, "page_table is required for a paged cache");
    if ((s = check_ptr(pt, "page_table"))) return s;
  } else if (pt) {
    return fail(MAC_ERR_INVALID_ARG, "page_table given for a contiguous cache");
  }
  return MAC_OK;
}

}  // namespace

extern "C" {

size_t mac_kv_cache_bytes(const mac_config* cfg) {
  if (check_config(cfg)) return 0;
  const size_t tile = (size_t)mac::kTile * cfg->head_dim * elem_size(cfg->dtype);
  if (cfg->page_size) return (size_t)cfg->n_pages * cfg->n_kv_heads * tile;
  const Layout L = layout(cfg);
  return (size_t)cfg->batch * cfg->n_kv_heads * L.ctx_stride * cfg->head_dim * elem_size(cfg->dtype);
}

size_t mac_ring_bytes(const mac_config* cfg) {
  if (check_config(cfg)) return 0;
  return layout(cfg).ring_bytes;
}

size_t mac_workspace_bytes(const mac_config* cfg) {
  if (check_config(cfg)) return 0;
  return layout(cfg).ws_bytes;
}

}  // extern "C"

namespace {

// The current device's static scratch: resolved on the first call for the
// device, its plan words set to all ones (synchronously, so that a context
// on another stream cannot step before that), and kept.  Returns the
// address, or null with *err set.
char* device_scratch(hipStream_t st, hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (!sl.resolved) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess)
      e = mac::launch_fill_i32(static_cast<int32_t*>(p), kScratchPlanGroups * 2, -1, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    sl.resolved = true;
    sl.err = e;
    sl.ptr = e == hipSuccess ? static_cast<char*>(p) : nullptr;
  }
  *err = sl.err;
  return sl.ptr;
}

// mac_init (keep_ring false: the ring is emptied) and mac_resume (keep_ring
// true: the ring's entries and counts are taken as they are).  Both write
// the rotary table into the ring and clear the workspace's plan words.
mac_status bind(const mac_config* cfg, void* ring, void* workspace, int32_t* seq_lens_dev,
                const int32_t* seq_lens_host, void* stream, mac_ctx** out, bool keep_ring) {
  mac_status s;
  if (!out) return fail(MAC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if ((s = check_config(cfg))) return s;
  if ((s = check_ptr(ring, "ring"))) return s;
  if ((s = check_ptr(workspace, "workspace", false))) return s;
  if ((s = check_ptr(seq_lens_dev, "seq_lens_dev"))) return s;
  if (!seq_lens_host) return fail(MAC_ERR_INVALID_ARG, "seq_lens_host is NULL");
  const Layout L = layout(cfg);
  for (int b = 0; b < cfg->batch; ++b)
    if (seq_lens_host[b] < 0 || seq_lens_host[b] > L.capacity)
      return fail(MAC_ERR_CAPACITY, "seq_lens_host[%d] = %d outside [0, %lld]", b, seq_lens_host[b],
                  (long long)L.capacity);
  mac_ctx* ctx = new (std::nothrow) mac_ctx;
  if (!ctx) return fail(MAC_ERR_INVALID_ARG, "out of host memory");
  ctx->cfg = *cfg;
  ctx->L = L;
  ctx->ring = static_cast<char*>(ring);
  ctx->ws = static_cast<char*>(workspace);
  ctx->seq_lens_dev = seq_lens_dev;
  ctx->mirror.assign(seq_lens_host, seq_lens_host + cfg->batch);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (!keep_ring)
    e = mac::launch_fill_i32(reinterpret_cast<int32_t*>(ctx->ring + L.r_count),
                             cfg->batch * cfg->n_q_heads, 0, st);
  if (e == hipSuccess && ctx->ws)   // no published plan yet (all ones never matches a ring count)
    e = mac::launch_fill_i32(reinterpret_cast<int32_t*>(ctx->ws + L.w_pub),
                             (int)((L.ws_bytes - L.w_pub) / 4), -1, st);
  if (e == hipSuccess)
    e = mac::launch_inv_freq(reinterpret_cast<double*>(ctx->ring + L.r_invf), cfg->head_dim,
                             cfg->rope_theta, st);
  if (e != hipSuccess) {
    delete ctx;
    return device_fail(nullptr, e, keep_ring ? "mac_resume: binding the buffers"
                                             : "mac_init: clearing the ring");
  }
  // the static scratch of mac_decode_step_append_noalloc; a failure here is
  // reported by that entry point (the workspace entry points do not need it)
  ctx->scratch = device_scratch(st, &ctx->scratch_err);
  *out = ctx;
  return ok();
}

}  // namespace

extern "C" {

mac_status mac_init(const mac_config* cfg, void* ring, void* workspace, int32_t* seq_lens_dev,
                    const int32_t* seq_lens_host, void* stream, mac_ctx** out) {
  return bind(cfg, ring, workspace, seq_lens_dev, seq_lens_host, stream, out, false);
}

mac_status mac_resume(const mac_config* cfg, void* ring, void* workspace, int32_t* seq_lens_dev,
                      const int32_t* seq_lens_host, void* stream, mac_ctx** out) {
  return bind(cfg, ring, workspace, seq_lens_dev, seq_lens_host, stream, out, true);
}

mac_status mac_append_kv(mac_ctx* ctx, void* k_cache, void* v_cache, const int32_t* page_table,
                         const void* k_new, const void* v_new, void* stream) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  if ((s = check_kv(ctx, k_cache, v_cache, page_table))) return s;
  if ((s = check_ptr(k_new, "k_new"))) return s;
  if ((s = check_ptr(v_new, "v_new"))) return s;
  for (int b = 0; b < ctx->cfg.batch; ++b)
    if (ctx->mirror[b] + 1 > ctx->L.capacity)
      return fail(MAC_ERR_CAPACITY, "sequence %d is full (%lld keys)", b, (long long)ctx->mirror[b]);
  hipError_t e = mac::launch_append(k_cache, v_cache, page_table, k_new, v_new, ctx->seq_lens_dev,
                                    ctx->geom(), ctx->cfg.batch, ctx->cfg.dtype,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(ctx, e, "mac_append_kv");
  for (auto& n : ctx->mirror) ++n;
  return ok();
}

mac_status mac_prefill_kv(mac_ctx* ctx, void* k_cache, void* v_cache, const int32_t* page_table,
                          int32_t seq, const void* k_src, const void* v_src, int32_t count,
                          void* stream) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  if ((s = check_kv(ctx, k_cache, v_cache, page_table))) return s;
  if (seq < 0 || seq >= ctx->cfg.batch)
    return fail(MAC_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, ctx->cfg.batch);
  if (count < 0) return fail(MAC_ERR_INVALID_ARG, "count must be >= 0 (got %d)", count);
  if (count == 0) return ok();
  if ((s = check_ptr(k_src, "k_src"))) return s;
  if ((s = check_ptr(v_src, "v_src"))) return s;
  if (ctx->mirror[seq] + count > ctx->L.capacity)
    return fail(MAC_ERR_CAPACITY, "sequence %d: %lld + %d keys exceed capacity %lld", seq,
                (long long)ctx->mirror[seq], count, (long long)ctx->L.capacity);
  hipError_t e = mac::launch_prefill(k_cache, v_cache, page_table, k_src, v_src, ctx->seq_lens_dev,
                                     seq, count, ctx->geom(), ctx->cfg.dtype,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(ctx, e, "mac_prefill_kv");
  ctx->mirror[seq] += count;
  return ok();
}

mac_status mac_read_kv(mac_ctx* ctx, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, int32_t seq, int32_t start, int32_t count,
                       void* k_dst, void* v_dst, void* stream) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  if ((s = check_kv(ctx, k_cache, v_cache, page_table))) return s;
  if (seq < 0 || seq >= ctx->cfg.batch)
    return fail(MAC_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, ctx->cfg.batch);
  if (start < 0 || count < 0 || (int64_t)start + count > ctx->mirror[seq])
    return fail(MAC_ERR_INVALID_ARG, "range [%d, %d + %d) outside the %lld stored keys", start, start,
                count, (long long)ctx->mirror[seq]);
  if (count == 0) return ok();
  if ((s = check_ptr(k_dst, "k_dst"))) return s;
  if ((s = check_ptr(v_dst, "v_dst"))) return s;
  hipError_t e = mac::launch_read(k_cache, v_cache, page_table, k_dst, v_dst, seq, start, count,
                                  ctx->geom(), ctx->cfg.dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(ctx, e, "mac_read_kv");
  return ok();
}

}  // extern "C"

namespace {

// Kernel arguments of one step; fused-append and optional outputs unset.
// The step's scratch (partial states, match records, reused states) is
// carved from `base` at the workspace's offsets, the plan words are `pub`.
mac::StepArgs step_args(mac_ctx* ctx, const void* q_pre, const void* k_cache, const void* v_cache,
                        const int32_t* page_table, float* out, char* base,
                        unsigned long long* pub) {
  const mac_config& c = ctx->cfg;
  const Layout& L = ctx->L;
  mac::StepArgs a;
  a.q_pre = q_pre;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.page_table = page_table;
  a.seq_lens = ctx->seq_lens_dev;
  a.inv_freq = reinterpret_cast<const double*>(ctx->ring + L.r_invf);
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.out = out;
  a.match_ctx_out = nullptr;
  a.dist_out = nullptr;
  a.heads = reinterpret_cast<mac::HeadState*>(base + L.w_heads);
  a.reuse_o = reinterpret_cast<float*>(base + L.w_reuse);
  a.plan_pub = pub;
  a.part.first = L.first;
  a.reuse_ml = a.reuse_o + (size_t)c.batch * c.n_q_heads * c.head_dim;
  a.part.o = reinterpret_cast<float*>(base + L.w_po);
  a.part.ml = reinterpret_cast<float*>(base + L.w_pml);
  a.part.S = L.slices;
  a.ring = ctx->ring_view();
  a.geom = ctx->geom();
  a.batch = c.batch;
  a.hq = c.n_q_heads;
  a.nchunk = n_chunks(&c);
  a.hkv = c.n_kv_heads * a.nchunk;
  a.group = chunk_heads(&c);
  a.band = c.band;
  a.tau2 = static_cast<float>((double)c.tau * (double)c.tau);
  // the second round's sequence order, longest first by the host mirror
  // (ties by index); the mirror is exact for calls made eagerly, and a
  // graph replays the order it captured, which stays right while every
  // sequence grows by one key per step
  a.order = 0;
  if (c.batch > 1 && c.batch <= mac::kOrderMax) {
    unsigned char ord[mac::kOrderMax];
    for (int b = 0; b < c.batch; ++b) ord[b] = static_cast<unsigned char>(b);
    std::stable_sort(ord, ord + c.batch,
                     [ctx](unsigned char x, unsigned char y) { return ctx->mirror[x] > ctx->mirror[y]; });
    for (int k = 0; k < c.batch; ++k) a.order |= static_cast<unsigned long long>(ord[k]) << (4 * k);
  }
  return a;
}

// Shared body of the decode entry points (k_new != null: fused append).
// noalloc: the step's scratch is the device's static array, not the
// workspace, and nothing is allocated (no timing events either).
mac_status decode_impl(mac_ctx* ctx, const void* q_pre, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, float* out, int32_t* match_ctx_out,
                       float* dist_out, const void* k_new, const void* v_new, void* stream,
                       bool noalloc = false) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  char* base;
  unsigned long long* pub;
  if (noalloc) {
    const int groups = ctx->cfg.batch * ctx->cfg.n_kv_heads * n_chunks(&ctx->cfg);
    const size_t need = kScratchStepOffset + ctx->L.w_out;
    if (groups > kScratchPlanGroups || need > kScratchBytes)
      return fail(MAC_ERR_CAPACITY, "mac_decode_step_append_noalloc: the step needs %zu bytes "
                  "of static scratch for %d KV groups; the library holds %zu bytes and %d groups "
                  "(use mac_decode_step_append with a workspace)", need, groups, kScratchBytes,
                  kScratchPlanGroups);
    if (!ctx->scratch)
      return fail(MAC_ERR_DEVICE, "mac_decode_step_append_noalloc: the static scratch of this "
                  "device is unavailable: HIP error %d (%s)", (int)ctx->scratch_err,
                  hipGetErrorString(ctx->scratch_err));
    base = ctx->scratch + kScratchStepOffset;
    pub = reinterpret_cast<unsigned long long*>(ctx->scratch);
  } else {
    if (!ctx->ws)
      return fail(MAC_ERR_INVALID_ARG, "this context was created without a workspace: use "
                  "mac_decode_step_append_noalloc");
    base = ctx->ws;
    pub = reinterpret_cast<unsigned long long*>(ctx->ws + ctx->L.w_pub);
  }
  if ((s = check_kv(ctx, k_cache, v_cache, page_table))) return s;
  if ((s = check_ptr(q_pre, "q_pre"))) return s;
  if ((s = check_ptr(out, "out"))) return s;
  if ((s = check_ptr(match_ctx_out, "match_ctx_out", false))) return s;
  if ((s = check_ptr(dist_out, "dist_out", false))) return s;
  const bool fused = k_new != nullptr || v_new != nullptr;
  if (fused) {
    if ((s = check_ptr(k_new, "k_new"))) return s;
    if ((s = check_ptr(v_new, "v_new"))) return s;
    for (int b = 0; b < ctx->cfg.batch; ++b)
      if (ctx->mirror[b] + 1 > ctx->L.capacity)
        return fail(MAC_ERR_CAPACITY, "sequence %d is full (%lld keys)", b, (long long)ctx->mirror[b]);
  } else {
    for (int b = 0; b < ctx->cfg.batch; ++b)
      if (ctx->mirror[b] < 1)
        return fail(MAC_ERR_INVALID_ARG, "sequence %d has no keys: append before decoding", b);
  }

  const mac_config& c = ctx->cfg;
  mac::StepArgs a = step_args(ctx, q_pre, k_cache, v_cache, page_table, out, base, pub);
  a.k_new = k_new;
  a.v_new = v_new;
  a.match_ctx_out = match_ctx_out;
  a.dist_out = dist_out;

  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (ctx->profiling && !noalloc && ctx->ev_used < 65536) {
    if (ctx->ev_used == ctx->events.size()) {
      // timing only (read after the stream has been synchronized): no
      // system-scope fence, whose cache write-back and invalidation would
      // otherwise fall inside the timed interval
      hipEvent_t x, y;
      hipError_t e = hipEventCreateWithFlags(&x, hipEventDisableSystemFence);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&y, hipEventDisableSystemFence);
      if (e != hipSuccess) return device_fail(ctx, e, "mac_decode_step: creating timing events");
      ctx->events.emplace_back(x, y);
    }
    e0 = ctx->events[ctx->ev_used].first;
    e1 = ctx->events[ctx->ev_used].second;
    ++ctx->ev_used;
  }
  hipError_t e = mac::launch_step(a, c.dtype, c.head_dim, c.page_size ? 1 : 0,
                                  static_cast<hipStream_t>(stream), e0, e1);
  if (e != hipSuccess) return device_fail(ctx, e, "mac_decode_step");
  if (fused)
    for (auto& n : ctx->mirror) ++n;
  return ok();
}

}  // namespace

extern "C" {

mac_status mac_decode_step(mac_ctx* ctx, const void* q_pre, const void* k_cache,
                           const void* v_cache, const int32_t* page_table, float* out,
                           int32_t* match_ctx_out, float* dist_out, void* stream) {
  return decode_impl(ctx, q_pre, k_cache, v_cache, page_table, out, match_ctx_out, dist_out,
                     nullptr, nullptr, stream);
}

mac_status mac_decode_step_append(mac_ctx* ctx, const void* q_pre, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* page_table, float* out, int32_t* match_ctx_out,
                                  float* dist_out, void* stream) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  if (!k_new || !v_new) return fail(MAC_ERR_INVALID_ARG, "k_new and v_new are required");
  return decode_impl(ctx, q_pre, k_cache, v_cache, page_table, out, match_ctx_out, dist_out,
                     k_new, v_new, stream);
}

mac_status mac_decode_step_append_noalloc(mac_ctx* ctx, const void* q_pre, const void* k_new,
                                          const void* v_new, void* k_cache, void* v_cache,
                                          const int32_t* page_table, float* out,
                                          int32_t* match_ctx_out, float* dist_out, void* stream) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  if (!k_new || !v_new) return fail(MAC_ERR_INVALID_ARG, "k_new and v_new are required");
  return decode_impl(ctx, q_pre, k_cache, v_cache, page_table, out, match_ctx_out, dist_out,
                     k_new, v_new, stream, true);
}

mac_status mac_seed_ring(mac_ctx* ctx, const void* q_hist, int n_hist, const void* k_cache,
                         const void* v_cache, const int32_t* page_table, void* stream) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  const mac_config& c = ctx->cfg;
  if (n_hist < 0 || n_hist > c.window)
    return fail(MAC_ERR_INVALID_ARG, "n_hist must be in [0, W = %d] (got %d)", c.window, n_hist);
  if (n_hist == 0) return ok();
  if (!ctx->ws) return fail(MAC_ERR_INVALID_ARG, "mac_seed_ring needs a context with a workspace");
  if ((s = check_kv(ctx, k_cache, v_cache, page_table))) return s;
  if ((s = check_ptr(q_hist, "q_hist"))) return s;
  for (int b = 0; b < c.batch; ++b)
    if (ctx->mirror[b] < n_hist)
      return fail(MAC_ERR_INVALID_ARG, "sequence %d holds %lld keys, fewer than the %d positions "
                  "to seed", b, (long long)ctx->mirror[b], n_hist);
  // Position N - n_hist + j of every sequence is replayed as a decode step
  // whose match cannot hit (tau^2 < 0): the step reads the sequence length
  // as that position + 1, attends over [0, position], and pushes the entry
  // a miss there would have pushed.  Outputs land in the workspace.
  const Layout& L = ctx->L;
  mac::StepArgs a = step_args(ctx, q_hist, k_cache, v_cache, page_table,
                              reinterpret_cast<float*>(ctx->ws + L.w_out), ctx->ws,
                              reinterpret_cast<unsigned long long*>(ctx->ws + L.w_pub));
  a.tau2 = -1.0f;
  int32_t* saved = reinterpret_cast<int32_t*>(ctx->ws + L.w_save);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t q_step = (size_t)c.batch * c.n_q_heads * c.head_dim * elem_size(c.dtype);
  hipError_t e = mac::launch_seed_len(ctx->seq_lens_dev, saved, c.batch, 0, 0, st);
  for (int j = 0; j < n_hist && e == hipSuccess; ++j) {
    e = mac::launch_seed_len(ctx->seq_lens_dev, saved, c.batch, 1, j + 1 - n_hist, st);
    if (e != hipSuccess) break;
    a.q_pre = static_cast<const char*>(q_hist) + j * q_step;
    e = mac::launch_step(a, c.dtype, c.head_dim, c.page_size ? 1 : 0, st, nullptr, nullptr);
  }
  if (e == hipSuccess) e = mac::launch_seed_len(ctx->seq_lens_dev, saved, c.batch, 2, 0, st);
  if (e != hipSuccess) return device_fail(ctx, e, "mac_seed_ring");
  return ok();
}

mac_status mac_query_cache_push(mac_ctx* ctx, const void* q_pre, const float* o, const float* m,
                                const float* l, const int32_t* prefix_end, const int32_t* ctx_len,
                                const uint8_t* mask, void* stream) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  if ((s = check_ptr(q_pre, "q_pre"))) return s;
  if ((s = check_ptr(o, "o"))) return s;
  if (!m || !l || !prefix_end || !ctx_len)
    return fail(MAC_ERR_INVALID_ARG, "m, l, prefix_end and ctx_len are required");
  hipError_t e = mac::launch_push(ctx->ring_view(), ctx->cfg.batch, ctx->cfg.n_q_heads,
                                  ctx->cfg.head_dim, ctx->cfg.dtype, q_pre, o, m, l, prefix_end,
                                  ctx_len, mask, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(ctx, e, "mac_query_cache_push");
  return ok();
}

mac_status mac_profile_enable(mac_ctx* ctx, int enable) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  ctx->profiling = enable != 0;
  return ok();
}

mac_status mac_profile_read(mac_ctx* ctx, double* ms_total, int64_t* launches) {
  mac_status s;
  if ((s = check_ctx(ctx))) return s;
  if (!ms_total || !launches) return fail(MAC_ERR_INVALID_ARG, "ms_total and launches are required");
  double tot = 0.0;
  for (size_t i = 0; i < ctx->ev_used; ++i) {
    hipError_t e = hipEventSynchronize(ctx->events[i].second);
    if (e != hipSuccess) return device_fail(ctx, e, "mac_profile_read");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, ctx->events[i].first, ctx->events[i].second);
    if (e != hipSuccess) return device_fail(ctx, e, "mac_profile_read");
    tot += ms;
  }
  *ms_total = tot;
  *launches = (int64_t)ctx->ev_used;
  ctx->ev_used = 0;
  return ok();
}

mac_status mac_destroy(mac_ctx* ctx) {
  if (!ctx) return ok();
  for (auto& p : ctx->events) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  delete ctx;
  return ok();
}

const char* mac_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
