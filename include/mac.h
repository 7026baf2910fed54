/*
 * libmac: the MAC-Attention decode step (match -> amend -> complete) for
 * AMD MI355X (gfx950).
 *
 * Method source: "MAC-Attention: a Match-Amend-Complete Scheme for Fast and
 * Accurate Attention Computation", abstract.  Per decode step and query head
 * the library
 *   - matches the current pre-RoPE query against the last W cached pre-RoPE
 *     queries of that head by L2 distance, with a strict threshold tau
 *     (abstract: the match stage);
 *   - on a hit reuses the matched entry's cached partial softmax state
 *     (o, m, l) over its prefix, recomputes the band of B keys at the match
 *     boundary (abstract: the amend stage) and attends fresh to the KV tail
 *     (abstract: the complete stage), fusing all partial states with a
 *     log-sum-exp merge (abstract: "numerically stable merge");
 *   - on a miss runs full split-K decode attention;
 *   - pushes the step's own entry (q_pre, prefix state, prefix end, context
 *     length) into the head's ring, hit or miss.
 *
 * Definitions the abstract leaves open, as this library fixes them:
 *   step order   mac_append_kv stores token n-1, then mac_decode_step attends
 *                with the query at position n-1 over keys [0, n).
 *   rotary       rotate-half pairing (i, i + d/2), angle pos * theta^(-2i/d)
 *                evaluated in double precision; the library rotates q itself,
 *                keys are stored already rotated.
 *   state        z = <rope(q), k>/sqrt(d); m = max z, l = sum e^(z-m),
 *                o = sum e^(z-m) v / l (natural base).  Empty: o=0, m=-inf, l=0.
 *   entry        the state of the entry's own query over [0, p) with
 *                p = max(0, n_entry - B).
 *   match        dist = ||q_pre - entry.q||_2 over entries with
 *                0 <= entry.p <= p_new; argmin with exact ties to the most
 *                recent entry; hit iff dist^2 < tau^2 evaluated in fp32.
 *                NaN distances are never chosen.
 *   ranges       p_new = max(0, n - B); s = hit ? entry.p : 0;
 *                prefix = merge(reused, state[s, p_new)), out = merge(prefix,
 *                state[p_new, n)).o; the pushed entry stores prefix.
 *
 * Conventions for every entry point:
 *   - Device pointers are plain HIP device addresses (e.g. from PyTorch
 *     tensors), 16-byte aligned.  Host pointers are marked "host".
 *   - Every call enqueues on `stream` (a hipStream_t; NULL = the default
 *     stream) and returns without synchronizing.  Stream order is the only
 *     ordering: call append, then decode, on the same stream.
 *   - The caller owns every device buffer.  The library never allocates
 *     device memory.  Ring and workspace are bound at mac_init and must stay
 *     allocated, and not be touched by the caller, until mac_destroy and
 *     every enqueued call using them has completed.
 *   - The ring holds all of a context's state between steps (its entries and
 *     the rotary table); it belongs to one context.  The workspace is scratch
 *     of a single call: nothing in it outlives the call, so contexts created
 *     with identical configs may share one workspace as long as their calls
 *     never overlap (e.g. the layers of a model stepped in order on one
 *     stream).  Calls that overlap on a shared workspace race.
 *   - Errors are returned as mac_status; mac_last_error() gives a message for
 *     the calling thread.  Argument checks happen before any HIP call, so a
 *     rejected call enqueues nothing.  A HIP error poisons the context: every
 *     later call on it returns MAC_ERR_STATE.  Data problems are not errors:
 *     NaN propagates to the affected head's output, and a NaN distance never
 *     matches.
 *   - Calls on one context are not thread-safe; use one context per thread
 *     or serialize.
 */
#ifndef LIBMAC_MAC_H
#define LIBMAC_MAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MAC_OK = 0,
  MAC_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or value   */
  MAC_ERR_UNSUPPORTED = 2,  /* valid but not built (head_dim, dtype, G)     */
  MAC_ERR_CAPACITY = 3,     /* a sequence would exceed its KV capacity      */
  MAC_ERR_DEVICE = 4,       /* a HIP call failed; the message has its code  */
  MAC_ERR_STATE = 5         /* context poisoned by an earlier device error  */
} mac_status;

typedef enum { MAC_DTYPE_F32 = 0, MAC_DTYPE_BF16 = 1 } mac_dtype;

/* Order of the elements inside the K and V caches (see the layout note below). */
typedef enum { MAC_KV_TILES = 0, MAC_KV_ROWS = 1 } mac_kv_layout;

/* Shape and method parameters.  All fields are read at mac_init only. */
typedef struct {
  int32_t batch;             /* sequences, >= 1                              */
  int32_t n_q_heads;         /* Hq, a multiple of n_kv_heads                 */
  int32_t n_kv_heads;        /* Hkv; G = Hq / Hkv <= C, or G splitting into  */
                             /* ceil(G/C) equal groups of at most C heads:   */
                             /* C = 32 for bf16 (MQA: 32, 64, ...), 16 fp32  */
  int32_t head_dim;          /* d: 64 or 128                                 */
  int32_t dtype;             /* mac_dtype of q, keys, values and ring q      */
  int32_t max_context;       /* contiguous cache: keys per sequence          */
  int32_t page_size;         /* 0 = contiguous cache, 16 = paged cache       */
  int32_t max_pages_per_seq; /* paged: columns of the page table             */
  int32_t n_pages;           /* paged: pages in the pool                     */
  int32_t window;            /* W >= 0: ring entries per (sequence, head)    */
  int32_t band;              /* B >= 0                                       */
  float tau;                 /* >= 0; hit iff dist < tau (fp32 dist^2 test)  */
  double rope_theta;         /* > 0                                          */
  int32_t max_slices;        /* split-K slices per KV group; 0 = default     */
  int32_t kv_layout;         /* mac_kv_layout                                */
} mac_config;

/*
 * Default slice count (max_slices = 0): base = ceil(256 / groups) slices per
 * KV group, one workgroup per compute unit, where groups = batch * Hkv *
 * ceil(G/C) (C as for n_kv_heads).  When a full-length sequence's base
 * slices would hold more than about 6K keys, the launch takes further rounds
 * of as many workgroups, one per 4096 keys a first-round slice would hold,
 * at most 4 rounds.  The hardware deals the later rounds to compute units as
 * they come free.  On a step where a group's heads all hit, its later-round
 * workgroups leave as soon as they read the group's plan, and for 2 to 16
 * sequences the later rounds visit the sequences longest first (by the
 * host's length mirror at the call); both apply to groups of at most 4 query
 * heads.  Wider groups run every later-round workgroup's match, except bf16
 * groups of more than 16 heads: matched in a launch of their own, their
 * later-round workgroups leave an empty slice once they have read the
 * group's match records.  The count is capped by ceil(capacity / 64) + 1, by
 * 1024 and by G' * slices <= 2048 (8192 for bf16 groups of more than 16
 * heads), G' the heads per group, and is at least 2.  An explicit
 * max_slices (capped by the G' * slices bound only) runs all its slices in
 * one round.  The slice count fixes mac_workspace_bytes.
 */

typedef struct mac_ctx mac_ctx;

/*
 * KV cache layouts (abstract: the method "composes with ... paged-KV
 * managers"; a cache is contiguous or paged, in 16-token pages).
 *
 * MAC_KV_ROWS, natural rows (either dtype): element (b, g, pos, i) of a
 *   contiguous cache is at ((b*Hkv + g)*max_context + pos)*d + i, the layout
 *   [batch][Hkv][max_context][d]; in a paged cache (page_size 16) position
 *   pos of sequence b is row pos % 16 of page page_table[b*max_pages_per_seq
 *   + pos/16], element ((page*Hkv + g)*16 + pos % 16)*d + i, the layout
 *   [n_pages][Hkv][16][d].  The caller may write tokens directly (a KV
 *   manager's own pool) or with mac_append_kv / mac_prefill_kv.
 * MAC_KV_TILES, library tiles (the default, both dtypes): the same 16-token
 *   tiles (contiguous: tile (b, g, t) starts at element ((b*Hkv + g)*T + t)
 *   *16*d with T = ceil(max_context/16); paged: as for rows), with the 16 x d
 *   elements inside a tile permuted so that each 64-lane wave load of 1 KiB
 *   lands directly in matrix-core operand order.  The permutation is private
 *   to the library: write tokens only with mac_append_kv or mac_prefill_kv,
 *   read them back with mac_read_kv.
 * Both layouts give bitwise identical results; the tile layout spares the
 * step kernels an LDS pass of each key and value tile.
 */
size_t mac_kv_cache_bytes(const mac_config* cfg);  /* bytes of ONE of K, V   */
size_t mac_ring_bytes(const mac_config* cfg);      /* opaque ring            */
size_t mac_workspace_bytes(const mac_config* cfg); /* opaque scratch         */

/*
 * Create a context (abstract: the match stage looks for similar queries in a
 * short local window of recent ones; the ring is that window, W entries per
 * sequence and query head, and it starts empty).
 *   ring          device, mac_ring_bytes(cfg): the window's entries and the
 *                 rotary table; emptied here.
 *   workspace     device, mac_workspace_bytes(cfg): scratch of one call
 *                 (see the conventions above for sharing it); may be NULL
 *                 for a context stepped only by
 *                 mac_decode_step_append_noalloc (the other decode entry
 *                 points and mac_seed_ring then return MAC_ERR_INVALID_ARG).
 *   seq_lens_dev  device int32[batch]: keys stored per sequence.  Device
 *                 truth, updated by the library's kernels.
 *   seq_lens_host host int32[batch]: the same lengths now; seeds the host
 *                 mirror used for capacity checks (no device sync needed).
 * The ring is emptied and the rotary table written on `stream`.  Returns
 * MAC_ERR_INVALID_ARG, MAC_ERR_UNSUPPORTED, MAC_ERR_CAPACITY (a length
 * beyond capacity) or MAC_ERR_DEVICE.
 */
mac_status mac_init(const mac_config* cfg, void* ring, void* workspace,
                    int32_t* seq_lens_dev, const int32_t* seq_lens_host,
                    void* stream, mac_ctx** out);

/*
 * Create a context that continues from a checkpoint.  A checkpoint of a
 * context is a byte copy, taken with no call of it in flight, of its ring,
 * its K and V caches, its page table (if paged) and seq_lens_dev, together
 * with the lengths on the host.  mac_resume binds such copies (or the
 * originals) under the same config: the ring's entries and push counts are
 * kept as they are, the rotary table is rewritten, and the steps that
 * follow give results bitwise identical to the steps the checkpointed
 * context would have run.  Arguments and errors as for mac_init; the
 * caller guarantees the ring was written by a context of the same config
 * (the library cannot check a ring's contents).
 */
mac_status mac_resume(const mac_config* cfg, void* ring, void* workspace,
                      int32_t* seq_lens_dev, const int32_t* seq_lens_host,
                      void* stream, mac_ctx** out);

/*
 * Append one token per sequence (abstract: "each token re-reads an
 * ever-growing KV cache"): k_new, v_new are device [batch][Hkv][d] in the
 * config dtype, already rotated.  Stored at position seq_lens_dev[b], which
 * is then incremented.  page_table: device int32
 * [batch][max_pages_per_seq] for a paged cache, NULL otherwise.  Returns
 * MAC_ERR_CAPACITY if any sequence is full (checked on the host mirror).
 */
mac_status mac_append_kv(mac_ctx* ctx, void* k_cache, void* v_cache,
                         const int32_t* page_table, const void* k_new,
                         const void* v_new, void* stream);

/*
 * Bulk append for one sequence: k_src, v_src are device [Hkv][count][d]
 * (natural layout, rotated keys), stored at positions
 * [seq_lens_dev[seq], +count); seq_lens_dev[seq] grows by count.
 */
mac_status mac_prefill_kv(mac_ctx* ctx, void* k_cache, void* v_cache,
                          const int32_t* page_table, int32_t seq,
                          const void* k_src, const void* v_src, int32_t count,
                          void* stream);

/*
 * Gather positions [start, start+count) of sequence seq back to natural
 * layout: k_dst, v_dst device [Hkv][count][d].  Caller guarantees the range
 * was written.  For checkpoints and tests.
 */
mac_status mac_read_kv(mac_ctx* ctx, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, int32_t seq, int32_t start,
                       int32_t count, void* k_dst, void* v_dst, void* stream);

/*
 * One MAC decode step for every sequence (abstract: match, amend, complete).
 *   q_pre          device [batch][Hq][d] config dtype: pre-RoPE queries of
 *                  the token at position seq_lens_dev[b]-1.
 *   k/v_cache      the caches written by mac_append_kv / mac_prefill_kv.
 *   page_table     device, paged caches only (else NULL).
 *   out            device fp32 [batch][Hq][d]: attention output.
 *   match_ctx_out  device int32 [batch][Hq] or NULL: context length of the
 *                  matched entry on a hit, -1 on a miss.
 *   dist_out       device fp32 [batch][Hq] or NULL: L2 distance to the best
 *                  candidate entry (hit or not); +inf if there is none.
 * Requires seq_lens >= 1 for every sequence (checked on the host mirror).
 */
mac_status mac_decode_step(mac_ctx* ctx, const void* q_pre,
                           const void* k_cache, const void* v_cache,
                           const int32_t* page_table, float* out,
                           int32_t* match_ctx_out, float* dist_out,
                           void* stream);

/*
 * mac_append_kv followed by mac_decode_step as one call (one launch fewer):
 * k_new, v_new are device [batch][Hkv][d] (rotated keys, config dtype); the
 * token is stored at position seq_lens_dev[b], then the query at that
 * position attends to keys [0, seq_lens_dev[b] + 1), and seq_lens_dev[b]
 * is incremented.  Results are bitwise identical to the two calls.  Returns
 * MAC_ERR_CAPACITY if any sequence is full (host mirror).
 * Graph capture: the kernels read the lengths and ring counts on the
 * device, so each replay of a captured call performs the next step (a
 * full sequence's append is dropped on the device); the host mirror, and
 * with it the capacity check, advances once, at capture.
 */
mac_status mac_decode_step_append(mac_ctx* ctx, const void* q_pre, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* page_table, float* out,
                                  int32_t* match_ctx_out, float* dist_out,
                                  void* stream);

/*
 * mac_decode_step_append for callers that cannot allocate device memory at
 * the call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): same arguments, results bitwise identical, and it
 * calls no allocating routine.  The step's scratch (partial states, match
 * records, reused ring states, published plan starts) lives in a static
 * device array of the library, 8 MiB per GPU, held until the process ends,
 * instead of the context's workspace; so a context used only through this
 * entry point may be created with workspace = NULL.  The array is found at
 * mac_init / mac_resume, once per device.  A config whose step needs more
 * (32 KiB of plan words plus the part of mac_workspace_bytes before the
 * ring-seeding scratch: for G = 4, d = 128 about 2 KiB per (KV group,
 * slice); at most 4096 KV groups) is refused with MAC_ERR_CAPACITY before
 * any device call.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other threads, other contexts)
 * race and must be serialized by the caller.  Kernel timing
 * (mac_profile_enable) does not apply to this entry point.
 */
mac_status mac_decode_step_append_noalloc(mac_ctx* ctx, const void* q_pre,
                                          const void* k_new, const void* v_new,
                                          void* k_cache, void* v_cache,
                                          const int32_t* page_table, float* out,
                                          int32_t* match_ctx_out,
                                          float* dist_out, void* stream);

/*
 * Push entries into the rings directly (abstract: the match stage's short
 * local window of recent queries; e.g. states computed at prefill so that
 * the first decode steps can match).  Device arrays indexed [b][h]:
 * q_pre [batch][Hq][d] dtype, o fp32 [batch][Hq][d] (normalized), m, l fp32
 * [batch][Hq] (natural log base), prefix_end, ctx_len int32 [batch][Hq].
 * mask uint8 [batch][Hq] or NULL (= push for every head).  The oldest entry
 * beyond W is evicted.  Entries with prefix_end outside [0, p_new] of a
 * later step are never matched by that step.
 */
mac_status mac_query_cache_push(mac_ctx* ctx, const void* q_pre,
                                const float* o, const float* m, const float* l,
                                const int32_t* prefix_end,
                                const int32_t* ctx_len, const uint8_t* mask,
                                void* stream);

/*
 * Seed the rings from a prefill (abstract: the match stage looks for
 * similar queries in a short window of recent ones; with the window read as
 * the last W decode steps, a fresh prefill leaves it empty and the first
 * decode steps cannot match).  q_hist is device [n_hist][batch][Hq][d],
 * config dtype: the pre-RoPE queries of the last n_hist positions of every
 * sequence (q_hist[j][b] belongs to position seq_lens[b] - n_hist + j).
 * Each position is replayed, oldest first, as a decode step that does not
 * match: its query attends to keys [0, position], and the entry it pushes is
 * the one a miss there would push (exact prefix state over
 * [0, max(0, position + 1 - B)), p, n = position + 1).  The step's outputs
 * are discarded (workspace); seq_lens_dev is unchanged afterwards.
 * 0 <= n_hist <= W and every sequence must hold at least n_hist keys
 * (MAC_ERR_INVALID_ARG otherwise, before any device call).  Costs n_hist
 * miss-path steps.
 */
mac_status mac_seed_ring(mac_ctx* ctx, const void* q_hist, int n_hist,
                         const void* k_cache, const void* v_cache,
                         const int32_t* page_table, void* stream);

/*
 * Kernel timing for measurement.  While enabled, each mac_decode_step
 * times its split-K attention kernel with a pair of HIP events on the step's
 * stream, bound to the kernel's dispatch (recorded as the kernel starts and
 * ends, so host enqueue time is not included; at most 65536 pairs are
 * kept).  mac_profile_read waits for
 * the recorded events, returns the summed milliseconds and the number of
 * launches timed, and clears the record.
 */
mac_status mac_profile_enable(mac_ctx* ctx, int enable);
mac_status mac_profile_read(mac_ctx* ctx, double* ms_total, int64_t* launches);

/* Release the host context (never frees caller memory). NULL is a no-op. */
mac_status mac_destroy(mac_ctx* ctx);

/* Last error message of the calling thread ("" if none). */
const char* mac_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMAC_MAC_H */
