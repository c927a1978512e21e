// Parameter blocks and launchers shared by the host runtime (fb_runtime.cpp)
// and the gfx950 kernels (fb_attn_bf16.hip, fb_attn_f32.hip, fb_aux.hip).  Not
// part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fb.h"

namespace fbk {

constexpr int kThreads = 256;     // threads of the fp32 attention and auxiliary workgroups
constexpr int kKeyTile = 64;      // keys staged in LDS per iteration
constexpr int kMaxSplits = 64;

// Combine workgroups are one wave; a row takes D/4 lanes (one float4 each).
constexpr int kCombineThreads = 64;
constexpr int combine_rows(int head_dim) { return 4 * kCombineThreads / head_dim; }

// Which heads a launch works on.  A head (b, h) is selected when bit b of
// `seq_bits` is set and, if `flags` is not null, (flags[b*Hq+h] != 0) equals
// `flags_select`; or, if `m` is not null (threshold decided on the device),
// unless the head holds a computed A_out (valid) and m[b] (+ cum[b] when cum
// is not null) < tau.  m, cum and valid must not change during the launch.
struct HeadSel {
  int32_t every_seq;      // 1: every sequence's bit is set (the bits need not be read)
  uint32_t seq_bits[FB_MAX_BATCH / 32];
  const uint8_t* flags;
  int32_t flags_select;
  int32_t tau;
  const int32_t* m;       // [B] updated tokens of this step
  const int32_t* cum;     // [B] sums since the last computation (cumulative rule) or null
  const uint8_t* valid;   // [B][Hq]
};

// Split plan chosen on the device (per-head decisions made on the device,
// gamma): with n of the (sequence, kv head) groups holding a selected head,
// their work is cut into splits[n] key ranges each, so that fewer active
// groups get more, shorter ranges and the launch keeps the chip busy.
// groups = 0: off (the host's static plan applies).
constexpr int kDynMaxGroups = 64;
struct DynPlan {
  int32_t groups;                        // B*Hkv when on
  uint8_t splits[kDynMaxGroups + 1];     // splits[n], n = 1..groups
};

// Attention of packed query rows over one key range.  The G = Hq/Hkv query
// heads of kv head g are contiguous in [B][Hq][Bs][D], so the G*Bs rows of a
// (b, g) group form one contiguous [G*Bs][D] matrix ("packed rows").
struct AttnParams {
  const void* q;          // [B][Hq][Bs][D]
  const void* k;          // [B][Hkv][kv_cap][D]
  const void* v;
  int64_t kv_cap;         // rows per (b, kv head) in k/v
  int32_t n_keys;         // keys 0..n_keys-1 are attended (tile list: 64 per listed tile)
  // Tile list (partial mode) or null.  Key tile v of group (b, g) is then the
  // 64 prefix rows starting at 64 * tiles[(b*hkv + g)*tiles_stride + v]; rows
  // at or past n_phys, and whole entries outside [0, ceil(n_phys/64)), hold
  // no key.
  const int32_t* tiles;
  int32_t tiles_stride;
  int32_t n_phys;
  int32_t batch, hq, hkv, bs, rows;   // rows = (Hq/Hkv) * Bs
  int32_t grp;            // Hq / Hkv (query heads per kv head)
  int32_t waves;          // wave64 per workgroup
  int32_t ksplit;         // 1, or 2: two wave sets split every key tile (waves/ksplit own 32 rows each)
  int32_t row_tiles;      // ceil(rows / (32 * waves / ksplit))
  int32_t grid;           // workgroups; 0: batch * hkv * splits * row_tiles
  int32_t splits;         // key ranges per group
  int32_t keys_per_split; // multiple of kKeyTile; with a device plan, the longest range it may pick
  // The work-item decode divides grid indices by row_tiles, splits and hkv:
  // each as a multiply by ceil(2^32 / d) (div_magic, set at launch; 0 = an
  // ordinary division).
  uint64_t dv_row_tiles, dv_splits, dv_hkv;
  int32_t ring_keys;      // longest key range of any item of the launch (LDS ring sizing)
  float scale_log2;       // softmax scale * log2(e)
  HeadSel sel;
  DynPlan dyn;            // partial mode only
  // Fused step (partial mode): the first int_count work items (B*Hkv*row_tiles,
  // or 0) attend the block's own keys (kblk/vblk [B][Hkv][Bs][D], every head,
  // no tile list) and store their partial at split index int_split; the
  // external items follow.
  const void* kblk;
  const void* vblk;
  int32_t int_count;
  int32_t int_split;
  // partial epilogue: normalised A and natural-log L per split.  A is bf16
  // from the bf16 kernels (one rounding of a normalised value, 2^-9
  // relative, on its way to the combine), fp32 from the fp32 ones.
  float* part_o;          // [splits][B][Hq][Bs][D]
  float* part_l;          // [splits][B][Hq][Bs]
  int64_t part_o_stride, part_l_stride;
  // merge epilogue: the cached external part (or, sparse steps, the total)
  const float* slot_o;    // [B][Hq][Bs][D]
  const float* slot_l;    // [B][Hq][Bs]
  const uint8_t* valid;   // [B][Hq]
  void* out;              // [B][Hq][Bs][D]
  // [B][Hq] or null: 1 - selected(b, h) is recorded (merge: by the head's own
  // rows; partial: every head, by the first workgroup, for the launches after)
  uint8_t* reuse_rec;
  // A second key set (partial mode, tile lists on both sets): after the
  // first set's items (whose plan the fields above give) come seg2_items
  // items over list tiles2 (tiles2_stride entries per group, n_keys2 keys)
  // for every group: seg2_splits ranges of seg2_kps keys each, whose
  // partials go to split index seg2_base + range.
  const int32_t* tiles2;
  int32_t tiles2_stride, n_keys2, seg2_items, seg2_splits, seg2_kps, seg2_base;
  // partial launches: 1 records reuse (1) for every head without evaluating
  // sel (a step the host knows reuses everywhere, e.g. a sparse step's
  // kept-key launch, whose sel selects every head)
  int32_t rec_reuse_all;
};

struct CombineParams {
  const float* part_o;    // bf16 elements when part_bf16
  const float* part_l;
  int64_t part_o_stride, part_l_stride;   // in elements
  int32_t part_bf16;
  int32_t splits, batch, hq, hkv, bs, row_chunks;
  HeadSel sel;
  DynPlan dyn;            // the external launch's plan (split count from the same active groups)
  float* slot_o;          // [B][Hq][Bs][D] the cache, refreshed in place
  float* slot_l;          // [B][Hq][Bs]
  uint8_t* valid;
  // 1 (gamma): before a value is replaced, sum <A_new, A_old>, |A_new|^2,
  // |A_old|^2 over the workgroup's rows for the similarity (each lane reads
  // the old value it then overwrites)
  int32_t sim_terms;
  float* cos_part;        // [B*Hq][row_chunks][3]
  // Total mode (tot_o not null): the fold starts from the head's cached part
  // (when valid) and the result goes to tot_o [B][Hq][Bs][D] /
  // tot_l [B][Hq][Bs]; the cache and its flags are left as they are.
  float* tot_o;
  float* tot_l;
  // Output mode (out not null; every head): after the external part (the
  // fold of the splits for a selected head, else its cached part, or the
  // total mode's sum) fold in the block-internal partial at split index
  // int_split and store the step's output [B][Hq][Bs][D] in the working dtype
  // (out_bf16); the cache is written only for selected heads, the total
  // buffer not at all.
  void* out;
  int32_t out_bf16;
  int32_t int_split;
  // cumulative threshold decided on the device: cum[b] restarts at 0 when a
  // head of b was selected (recomputed), else grows by cum_m[b]
  int32_t* cum;
  const int32_t* cum_m;
  // 1: a recomputed head's valid flag is left as it is (a single-launch step
  // whose workgroups read the flags for their decisions while others fold)
  int32_t keep_valid;
  // Two key sets (two_sets = 1; tot_o null, out set): splits 0 .. splits-1
  // of a selected head are its first key set (they refresh the cache as
  // usual); then every head folds splits base2 .. base2+splits2-1 (the
  // second set) onto its cached part before the block-internal partial.
  int32_t two_sets, splits2, base2;
};

// Single-launch fused step: the split attention items, the block-internal
// items and the split combine share one grid.  Workgroups below n_attn take
// the attention items (by index, as in the two-launch form, XCD placement
// included); the others take combine work, waiting (bounded) until every
// attention workgroup of their group has arrived.  Each XCD dispatches its
// workgroups in increasing index order, so a waiting combine workgroup only
// ever waits for attention workgroups that are running or will be dispatched
// once the attention workgroups ahead of them, which never wait, finish: the
// wait needs no co-resident grid.  A group's last combine workgroup returns
// its counter to zero, so a launch can be captured and replayed.
struct FinParams {
  CombineParams cp;
  // counter i at ctr[i * kFinStride] (one 128-byte line each): 0 error flag
  // (a combine workgroup gave up waiting), 1 + group: arrivals of group
  // b*Hkv + g
  uint32_t* ctr;
  int32_t n_attn;         // attention workgroups: indexes 0 .. n_attn-1
  int32_t n_total;        // + combine workgroups
  int32_t chunks;         // combine workgroups per query head (256/D rows per wave)
  uint32_t need;          // arrivals that complete a group (its attention items)
  uint32_t done_all;      // need + the group's combine workgroups: the last one resets the counter
  // With a device plan (cp.dyn.groups > 0) the two counts above are taken in
  // the kernel from the active groups instead: a group then has
  // (dyn.splits[n] + 1) * row_tiles attention items if active, row_tiles (its
  // block-internal ones) if not, and the workgroups past the plan's items
  // belong to no group and do not arrive.
  int32_t row_tiles;
  // 1: a group with no selected head is finished by its block-internal items
  // alone (the merge launch's epilogue: the cached part folded in, the output
  // stored; AttnParams' merge fields are set); its split items and its
  // combine workgroups exit at once and nothing counts on its counter.
  int32_t merge_reused;
};
constexpr int kFinCounters = 1;   // counters before the per-group ones
constexpr int kFinStride = 32;    // uint32 per counter

// Tile list of the prefix keys a sparse selection leaves out.
struct ComplementParams {
  const int32_t* sel;     // [groups][n_sel]
  int32_t n_sel;
  int32_t tiles;          // prefix tiles: ceil(prefix_len / 64)
  int32_t* comp;          // [groups][stride]
  int32_t stride;         // >= tiles
  int32_t groups;
};

struct DecideParams {
  int32_t n_heads;        // B*Hq
  int32_t hq, row_chunks;
  int32_t group;          // 1: a similarity per head; G = Hq/Hkv: one per kv group (its heads' terms summed)
  const uint8_t* reuse_now;  // decisions applied at this step
  uint8_t* reuse_next;       // decisions for the next step
  uint8_t* valid;
  float* sim;
  const float* cos_part;
  float gamma;
};

struct ResetParams {
  int32_t n_heads;
  int32_t batch;
  int32_t* cum;           // [B] or null
  uint8_t* valid;
  uint8_t* reuse;         // [2][B*Hq]
  float* sim;
  uint32_t* fin_ctr;      // the single-launch step's counters (zeroed), or null
  int32_t fin_n;
};

enum AttnMode { kModePartial = 0, kModeMerge = 1 };

// Launchers (fb_aux.hip; launch_attn dispatches to the attention kernel files).
// Return the launch status.
hipError_t launch_attn(int dtype, int head_dim, int mode, const AttnParams& p, hipStream_t s);
// The single-launch fused step (bf16, head dim 128, one row tile per group,
// dense keys, host decisions); hipErrorNotSupported for other launches.
hipError_t launch_attn_fin(const AttnParams& p, const FinParams& f, hipStream_t s);
bool fin_supported(int dtype, int head_dim, const AttnParams& p);
hipError_t launch_combine(int head_dim, const CombineParams& p, hipStream_t s);
hipError_t launch_decide(const DecideParams& p, hipStream_t s);
hipError_t launch_reset(const ResetParams& p, hipStream_t s);
hipError_t launch_complement(const ComplementParams& p, hipStream_t s);

// Sets the calling thread's error message (fb_last_error) and returns code.
fb_status report(fb_status code, const char* msg);

// fb_step_noalloc's work on a given scratch buffer (fb_runtime.cpp).
fb_status noalloc_step(const fb_config* cfg, void* scratch, size_t scratch_bytes, int n_cu, const void* q_blk,
                       const void* k_blk, const void* v_blk, const void* k_prefix, const void* v_prefix,
                       int32_t prefix_len, float* a_out, float* l_out, void* out, void* stream);

// ceil(2^32 / d): then n / d = floor(n * m / 2^32) exactly for every n with
// n * d < 2^32 (the rounding up of m adds less than n / 2^32 < 1 / d).  0
// (an ordinary division) when some index below n_max breaks that bound.
inline uint64_t div_magic(int d, long long n_max) {
  if (d <= 0 || n_max < 0 || (unsigned long long)n_max * (unsigned long long)d >= (1ull << 32)) return 0;
  return ((1ull << 32) + (uint64_t)d - 1) / (uint64_t)d;
}

// The decode's divisors for a launch of `blocks` workgroups.
inline AttnParams with_div_magic(const AttnParams& p, int blocks) {
  AttnParams q = p;
  q.dv_row_tiles = div_magic(p.row_tiles, blocks);
  q.dv_splits = div_magic(p.splits, blocks);
  q.dv_hkv = div_magic(p.hkv, blocks);
  return q;
}

}  // namespace fbk
