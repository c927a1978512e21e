/*
 * fb.h -- C ABI of the FlashBlock attention-step library (libfb.so, gfx950).
 *
 * FlashBlock ("FlashBlock: Attention Caching for Efficient Long-Context Block
 * Diffusion", page "Résumé Technique : FlashBlock", §2 "Mécanisme Central")
 * splits the attention of a denoising step of block diffusion into
 *   - block-external attention A_out over the tokens outside the current
 *     block (the committed prefix KV cache), with its log-normaliser
 *     L_out = log Z_out, which are cached and may be reused by later steps;
 *   - block-internal attention A_in, L_in over the block's own tokens;
 *   - the log-space merge A_full = (e^{L_out-m} A_out + e^{L_in-m} A_in) /
 *     (e^{L_out-m} + e^{L_in-m}) with m = max(L_out, L_in).
 * A step reuses the cache when the number M of updated block tokens is below
 * a threshold tau, or, per head, when the head's similarity across steps
 * exceeds gamma (§2 "Stratégies de Réutilisation Adaptatives").
 *
 * Conventions shared by every entry point
 *   - Every call returns fb_status; FB_OK is 0.  No C++ exception crosses the
 *     ABI.  On an error, fb_last_error() holds a message for the calling
 *     thread until its next call into the library.
 *   - Argument, shape and state checks are synchronous and happen before any
 *     work is enqueued: a call that returns an error enqueued nothing and left
 *     the cache's state as it was.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream) and is asynchronous unless stated otherwise.  The caller keeps
 *     every buffer it passed alive and unmodified until that work finished.
 *     Faults inside kernels surface at the next synchronising call.
 *   - Tensor pointers are device pointers owned by the caller, contiguous and
 *     row-major (innermost dimension last), in the cache's dtype:
 *       q_blk, out        [B][Hq][Bs][D]
 *       k_blk, v_blk      [B][Hkv][Bs][D]
 *       k_prefix,v_prefix [B][Hkv][max_prefix][D]; rows 0..prefix_len-1 are
 *                         the committed prefix tokens J_out, the rest unused.
 *     Query head h reads key/value head h / (Hq/Hkv) (grouped-query heads).
 *   - Softmax: scores are softmax_scale * <q, k>; L values are natural-log
 *     sum-exp of the scaled scores.  Attention arithmetic is fp32 with bf16
 *     operands for FB_BF16 (products exact, fp32 accumulation) and fp32
 *     operands for FB_F32.  A_out and L_out are cached in fp32 for both dtypes;
 *     for FB_BF16 the normalised part of each prefix chunk is rounded to bf16
 *     once (relative 2^-9) on its way to the fp32 combine.
 *   - The library keeps no caller pointer after a call returns.  The cache is
 *     bound to the device that was current at fb_cache_alloc; calls switch to
 *     it and back.  One cache must not be used by two threads at once.
 */
#ifndef FB_H
#define FB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fb_status;
enum {
  FB_OK = 0,
  FB_E_ARG = 1,          /* null pointer, bad enum, bad number */
  FB_E_SHAPE = 2,        /* sizes inconsistent or beyond the cache's limits */
  FB_E_DTYPE = 3,        /* dtype not FB_F32 / FB_BF16 */
  FB_E_STATE = 4,        /* call not valid in the cache's current state */
  FB_E_NOMEM = 5,        /* device allocation failed */
  FB_E_HIP = 6,          /* HIP runtime error or no usable device */
  FB_E_UNSUPPORTED = 7   /* valid request this build does not implement */
};

enum { FB_F32 = 0, FB_BF16 = 1 };
/* ALWAYS: recompute every step.  TAU (page §2, threshold reuse) and GAMMA
 * (page §2, per-head selection): see fb_policy_args.  Two variants at the
 * edges of those rules: TAU_CUM counts the updated tokens summed since the
 * sequence's cache was computed, this step's included; GAMMA_GROUP decides
 * per (sequence, kv head) with one similarity over the group's query heads
 * (their A_out taken as one vector), so a decision matches the K/V stream it
 * saves. */
enum { FB_POLICY_ALWAYS = 0, FB_POLICY_TAU = 1, FB_POLICY_GAMMA = 2, FB_POLICY_TAU_CUM = 3,
       FB_POLICY_GAMMA_GROUP = 4 };
enum {
  FB_FIELD_A_OUT = 0,    /* float [B][Hq][Bs][D]  current cached A_out of every head */
  FB_FIELD_L_OUT = 1,    /* float [B][Hq][Bs]     current cached L_out */
  FB_FIELD_SIM = 2,      /* float [B][Hq]         last similarity per head (NaN: none yet) */
  FB_FIELD_REUSE = 3,    /* uint8 [B][Hq]         1 if the head reused at the last fb_step */
  FB_FIELD_VALID = 4,    /* uint8 [B][Hq]         1 if the head's cache holds a computed A_out */
  FB_FIELD_WAIT_ERR = 5  /* uint32 [1]            nonzero once a single-launch step's combine gave up
                            waiting for its attention items (a diagnostic: the wait is bounded,
                            and the flag stays set until the next fb_cache_reset) */
};

#define FB_MAX_BATCH 1024     /* sequences per cache */
#define FB_MAX_HEADS 256      /* query heads per sequence */

typedef struct {
  int32_t batch;          /* B  >= 1, <= FB_MAX_BATCH */
  int32_t n_q_heads;      /* Hq >= 1, <= FB_MAX_HEADS, a multiple of n_kv_heads */
  int32_t n_kv_heads;     /* Hkv >= 1 */
  int32_t head_dim;       /* D: 64 or 128 (others give FB_E_UNSUPPORTED) */
  int32_t block_size;     /* Bs >= 1: tokens of the current block */
  int32_t max_prefix;     /* >= 0: row capacity of the caller's prefix K/V buffers */
  int32_t dtype;          /* FB_F32 | FB_BF16: dtype of Q/K/V and of the output */
  float softmax_scale;    /* <= 0 selects 1/sqrt(head_dim) */
} fb_config;

/* Options of fb_cache_alloc_ex beyond fb_config (tuning and tests).  The
 * struct may grow: struct_size = sizeof(fb_cache_opts) as the caller was
 * built; fields past struct_size take their defaults (0). */
typedef struct {
  uint32_t struct_size;
  int32_t kv_splits;      /* 0: automatic; else prefix chunks per (b, kv head), 1..64 */
} fb_cache_opts;

typedef struct fb_cache fb_cache;   /* opaque; owns device memory (hipMalloc) */

/* Allocate the A_out/L_out cache for `cfg` on the current device: fp32
 * A_out [B][Hq][Bs][D] and L_out [B][Hq][Bs] (a recomputed head's value
 * replaces the old one in place; under GAMMA the similarity is taken as it is
 * replaced), per-head flags, scratch for split-prefix partial results sized
 * for max_prefix, and for sparse steps a total buffer of the A_out size and
 * the list of left-out prefix tiles.  The new cache is in the reset state.
 * The cache holds what page "Résumé Technique : FlashBlock", §2 "Mécanisme
 * Central", says FlashBlock keeps from one diffusion step to the next: the
 * block-external output A_out and its log-normaliser L_out = log Z_out.
 * *out is set only on FB_OK.  The caller frees it with fb_cache_free.
 * Errors: FB_E_ARG (null), FB_E_DTYPE, FB_E_SHAPE, FB_E_UNSUPPORTED,
 * FB_E_NOMEM, FB_E_HIP (no device). */
fb_status fb_cache_alloc(const fb_config* cfg, fb_cache** out);

/* fb_cache_alloc with options (opts NULL: the defaults).  Errors: those of
 * fb_cache_alloc, FB_E_ARG (struct_size below 4, kv_splits outside
 * [0, 64]). */
fb_status fb_cache_alloc_ex(const fb_config* cfg, const fb_cache_opts* opts, fb_cache** out);

/* Release the cache's device memory after waiting for its device to finish
 * all work.  NULL is a no-op. */
fb_status fb_cache_free(fb_cache* c);

/* Block boundary (page §1: the next block starts on a prefix that now also
 * holds the finished block's K/V, appended by the caller).  Marks every head's
 * cache empty, clears the similarities to NaN and the step counter to 0.
 * Enqueued on `stream`. */
fb_status fb_cache_reset(fb_cache* c, void* stream);

/* Block-external attention, page §2 "Mécanisme Central": for every head with
 * head_mask[b*Hq+h] != 0 (head_mask: device uint8 [B][Hq]; NULL = all heads)
 * compute A_out (softmax attention of the block queries over prefix rows
 * 0..prefix_len-1, no mask) and L_out, store them as the head's cached pair,
 * and mark the head valid.  prefix_len == 0 stores A_out = 0, L_out = -inf.
 * What it stores serves fb_internal_attn_merge; fb_step recomputes every head
 * at the first step of a block whatever the cache holds.
 * Errors: FB_E_ARG, FB_E_SHAPE (prefix_len < 0 or > max_prefix). */
fb_status fb_external_attn(fb_cache* c, const void* q_blk, const void* k_prefix,
                           const void* v_prefix, int32_t prefix_len,
                           const uint8_t* head_mask, void* stream);

/* Block-internal bidirectional attention of the block queries over all Bs
 * block keys (A_in, L_in; no mask), merged in log space with the head's cached
 * A_out/L_out (page §2, A_full equation), written to `out` in the cache's
 * dtype.  A head whose cache holds nothing merges with an empty external part,
 * so its output is A_in.  Errors: FB_E_ARG. */
fb_status fb_internal_attn_merge(fb_cache* c, const void* q_blk, const void* k_blk,
                                 const void* v_blk, void* out, void* stream);

typedef struct {
  int32_t policy;            /* FB_POLICY_* */
  int32_t tau;               /* TAU: reuse iff the cache holds a computed A_out and
                                n_updated[b] < tau (strict); TAU_CUM: iff the sum of
                                n_updated[b] since the last computation, this step's
                                included, is < tau */
  float gamma;               /* GAMMA: reuse iff the head holds a similarity and it
                                is > gamma (strict); GAMMA_GROUP: the same with the
                                group's similarity */
  const int32_t* n_updated;  /* host int32 [B]: tokens of the block updated since the
                                previous step (TAU, TAU_CUM; ignored otherwise) */
} fb_policy_args;

/* Options of fb_step_ex / fb_step_sparse.  The struct may grow: struct_size =
 * sizeof(fb_step_opts) as the caller was built; fields past struct_size take
 * their defaults (NULL). */
typedef struct {
  uint32_t struct_size;
  const int32_t* n_updated_dev;
                             /* device int32 [B], values >= 0 (not checked): the threshold
                                counts in device memory, read by the step's kernels when
                                they run; the decisions are then made on the device, per
                                head, from each head's own valid flag.  Under TAU/TAU_CUM
                                exactly one of fb_policy_args.n_updated and n_updated_dev
                                is set; a block keeps the same choice until its reset. */
} fb_step_opts;

/* One denoising step (page §2): decide per head whether to reuse the cached
 * A_out/L_out; recompute block-external attention for the other heads and
 * refresh their cache; under GAMMA measure each recomputed head's cosine
 * similarity between its new and previous A_out (flattened over Bs x D) and
 * decide its reuse at the next step; compute block-internal attention and the
 * merge into `out`.  The first step after a reset recomputes every head, and
 * under GAMMA so does the second (a similarity needs two computed A_out).
 * The first step after a reset recomputes every head even when
 * fb_external_attn filled the cache since the reset.
 * The whole step is asynchronous on `stream` (GAMMA decisions and TAU
 * decisions from device counts stay on the device).  Where some head
 * recomputes, the split attention over the prefix and the block-internal
 * attention run as one kernel launch and the split combine as a second.  With
 * FB_FIN=1 in the environment at fb_cache_alloc all three run as one launch
 * (profiling counts it as external attention) where the dtype is bf16, the
 * head dim 128 and the query rows of a kv head (query heads per kv head x
 * block size) at most 256, and the decisions are made on the host or are TAU
 * decisions from device counts after the block's first step: the same cache
 * and decisions, and the same outputs for recomputed heads; a kv head whose
 * query heads all reuse then takes its output from the block-internal
 * attention's merge, within one output rounding of the two launches'.
 * Errors: FB_E_ARG (null,
 * bad policy, tau < 0, n_updated null under TAU, a negative n_updated),
 * FB_E_SHAPE, FB_E_STATE (prefix_len, policy or the host/device choice
 * differs from the previous step of the same block).
 *
 * Graph capture: fb_step and fb_cache_reset enqueue kernel launches only (no
 * copy, memset, allocation or synchronisation) and, when no decision is made
 * on the host (ALWAYS, GAMMA, GAMMA_GROUP, or TAU/TAU_CUM with device counts
 * through fb_step_ex), nothing they enqueue depends on device values read by the
 * host, so they may be recorded by HIP stream capture with profiling off.  A
 * replay repeats the launches as recorded, host choices included (the step's
 * position in its block, prefix_len, pointers such as n_updated_dev), so a
 * graph holds whole blocks, each starting with fb_cache_reset; between replays
 * the caller may change the contents of the buffers, not their addresses.
 * With profiling on, fb_step and fb_cache_reset on a capturing stream return
 * FB_E_STATE. */
fb_status fb_step(fb_cache* c, const fb_policy_args* p, const void* q_blk, const void* k_blk,
                  const void* v_blk, const void* k_prefix, const void* v_prefix,
                  int32_t prefix_len, void* out, void* stream);

/* fb_step with options (opts NULL: fb_step itself): with opts->n_updated_dev
 * set, the threshold counts are read from device memory and the decisions
 * made on the device (fb_policy_args.n_updated must then be NULL).  Errors:
 * those of fb_step, FB_E_ARG (struct_size below 4, both counts set). */
fb_status fb_step_ex(fb_cache* c, const fb_policy_args* p, const fb_step_opts* opts, const void* q_blk,
                     const void* k_blk, const void* v_blk, const void* k_prefix, const void* v_prefix,
                     int32_t prefix_len, void* out, void* stream);

/* One denoising step over a sparse attention (page §2, compatibility with
 * sparse attention; §3, synergy with sparsity): a sparse selection keeps some
 * 64-key tiles of the prefix; the tiles it leaves out are treated as the
 * block-external set, whose part (A, L) is cached and reused under the
 * policy exactly as fb_step does for the whole prefix, while the kept tiles
 * are attended afresh for every head at every step.  The output is the
 * log-space merge of the cached part, the kept part and the block-internal
 * part.  With every head recomputing (ALWAYS) it is exact attention over the
 * prefix and the block, for every selection that keeps the rule above.
 *   sel_tiles  device int32 [B][Hkv][n_sel]: for each (sequence, kv head), the
 *              kept tiles (tile t = prefix rows 64t .. 64t+63, cut at
 *              prefix_len), shared by the query heads of the kv head.  The
 *              entries of a (sequence, kv head) must be distinct tiles in
 *              [0, ceil(prefix_len / 64)) (ascending by convention): the
 *              library does not read device data back to check, and for any
 *              other selection the results are unspecified (every access
 *              stays in bounds).  Read at the block's first step (which lists
 *              the tiles left out) and at every step (kept tiles): the
 *              selection must stay the same within a block.
 *   n_sel      0 <= n_sel <= ceil(prefix_len / 64), the same for every step of
 *              a block.
 *   opts       NULL, or as for fb_step_ex (device counts).
 * Launches: where some head recomputes, one attention launch over the
 * left-out tiles (recomputing heads), the kept tiles (every head) and the
 * block, and one combine, when both tile sets' split partials fit the
 * cache's partial buffer together (else an attention launch and a combine
 * for each set); where every head reuses (known on the host), one launch
 * over the kept tiles and the block and one combine.
 * Under GAMMA the similarity is that of the cached (left-out) part.  The
 * cache fields A_out/L_out hold the left-out keys' part.  Policies, counts,
 * graph capture and asynchrony are as for fb_step; a block is either dense
 * (fb_step) or sparse (fb_step_sparse) until its reset.  Errors: those of
 * fb_step, FB_E_ARG (sel_tiles null with n_sel > 0), FB_E_SHAPE (n_sel out of
 * range), FB_E_STATE (n_sel, or sparse vs dense, changed inside a block). */
fb_status fb_step_sparse(fb_cache* c, const fb_policy_args* p, const fb_step_opts* opts,
                         const void* q_blk, const void* k_blk, const void* v_blk,
                         const void* k_prefix, const void* v_prefix, int32_t prefix_len,
                         const int32_t* sel_tiles, int32_t n_sel, void* out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): one
 * denoising step that recomputes every head, as fb_step under
 * FB_POLICY_ALWAYS, without a cache.  Its split partials and per-head flags
 * use a library-owned static device array of FB_NOALLOC_SCRATCH_BYTES per GPU
 * (held until the process ends; its device address is looked up at the
 * first call on each device); nothing is allocated.
 *   cfg      as for fb_cache_alloc (max_prefix = the prefix buffers' rows)
 *   a_out    device float [B][Hq][Bs][D]: block-external output A_out
 *   l_out    device float [B][Hq][Bs]: its log-normaliser L_out
 *   out      device [B][Hq][Bs][D] in cfg's dtype: the merged output
 * Other tensors as for fb_step.  The prefix is cut into as many chunks as the
 * scratch holds (at most as many as fb_step would use).  Calls that overlap
 * on one GPU share its array and race.  Asynchronous on `stream`.
 * Errors: those of fb_cache_alloc's config checks, FB_E_ARG (null),
 * FB_E_SHAPE (prefix_len out of range, or a shape whose partials for a single
 * chunk exceed the scratch), FB_E_HIP. */
#define FB_NOALLOC_SCRATCH_BYTES (64u << 20)
fb_status fb_step_noalloc(const fb_config* cfg, const void* q_blk, const void* k_blk, const void* v_blk,
                          const void* k_prefix, const void* v_prefix, int32_t prefix_len, float* a_out,
                          float* l_out, void* out, void* stream);

/* Copy one field of the cache (layouts in the FB_FIELD_* list) to host
 * memory `host_dst` of exactly `bytes` bytes, after the work already on
 * `stream`.  Synchronising; meant for tests and debugging.
 * Errors: FB_E_ARG (null, unknown field, wrong byte count), FB_E_HIP. */
fb_status fb_cache_read(const fb_cache* c, int32_t field, void* host_dst, size_t bytes,
                        void* stream);

/* Device bytes the cache allocated, and the number of prefix chunks
 * (split-KV) its external attention uses at max_prefix. */
fb_status fb_cache_info(const fb_cache* c, size_t* device_bytes, int32_t* kv_splits);

/* Kernel timing.  While enabled, every kernel the cache launches is bracketed
 * by HIP events on its launch stream; fb_profile_read synchronises with them
 * and returns, per kernel kind, the number of launches and their summed
 * duration in milliseconds since enabling (and clears the record).  Kinds:
 * 0 external attention, 1 split combine, 2 internal attention + merge,
 * 3 similarity / decision, 4 reset, 5 sparse kept-tile attention, 6 sparse
 * total combine, 7 sparse left-out tile list.  At most FB_PROFILE_KINDS
 * kinds. */
#define FB_PROFILE_KINDS 8
typedef struct {
  int64_t launches[FB_PROFILE_KINDS];
  double ms[FB_PROFILE_KINDS];
} fb_profile_stats;
fb_status fb_profile_enable(fb_cache* c, int32_t enable);
fb_status fb_profile_read(fb_cache* c, fb_profile_stats* out);

/* Message of the calling thread's last error ("" after success). */
const char* fb_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FB_H */
