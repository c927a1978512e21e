// Host runtime of libfb.so: argument checks, the A_out/L_out cache, the reuse
// policy state, split-KV planning and stream-ordered launches.  The C ABI and
// its contract are in include/fb.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "fb.h"
#include "fb_internal.h"

namespace {

thread_local std::string g_err;

fb_status fail(fb_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

fb_status ok() {
  g_err.clear();
  return FB_OK;
}

fb_status hip_fail(hipError_t e, const char* what) {
  return fail(FB_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Switches to the cache's device for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int now = -1;
    if (prev >= 0 && hipGetDevice(&now) == hipSuccess && now != prev) (void)hipSetDevice(prev);
  }
};

struct ProfRec {
  int kind;
  hipEvent_t start, stop;
};

// Split counts chosen so far, keyed by (keys, active groups, co-scheduled
// workgroups, their tiles); a fixed table (no allocation), the oldest entry
// replaced when full.
struct SplitMemo {
  static constexpr int kCap = 256;
  struct Entry {
    int32_t keys, groups, co_items, co_tiles, splits;
  } e[kCap];
  int n = 0, next = 0;
  int find(int keys, int groups, int co_items, int co_tiles) const {
    for (int i = 0; i < n; ++i)
      if (e[i].keys == keys && e[i].groups == groups && e[i].co_items == co_items && e[i].co_tiles == co_tiles)
        return e[i].splits;
    return -1;
  }
  void put(int keys, int groups, int co_items, int co_tiles, int splits) {
    e[next] = Entry{keys, groups, co_items, co_tiles, splits};
    next = (next + 1) % kCap;
    n = n < kCap ? n + 1 : kCap;
  }
  void clear() { n = next = 0; }
};

}  // namespace

struct fb_cache {
  fb_config cfg{};
  int kv_splits = 0;     // 0: automatic; else forced prefix chunks (fb_cache_opts)
  int device = 0;
  int group = 1;         // Hq / Hkv
  int rows = 0;          // packed rows per (b, kv head) = group * Bs
  int ext_waves = 4;     // waves per external-attention workgroup
  int ext_ksplit = 1;    // 2: two wave sets share the rows and split each key tile
  int row_tiles = 0;     // external-attention row tiles per group
  int int_waves = 4;     // waves per internal-attention workgroup
  int int_ksplit = 1;
  int row_chunks = 0;    // combine workgroups per head
  int splits_cap = 1;    // splits the scratch is sized for
  // device split plan for per-head decisions made on the device (gamma),
  // for the prefix length it was made for
  fbk::DynPlan dyn{};
  int32_t dyn_keys = -1;
  int dyn_grid = 0;      // workgroups of the largest item count over the plan
  int dyn_kps = 0;       // longest key range of the plan
  int dyn_co = 0;        // co-scheduled workgroups the plan was made for
  SplitMemo split_memo;   // split counts chosen so far
  int n_cu = 256;        // compute units of the device
  float scale = 0.0f;
  size_t bytes = 0;
  // device memory
  float* slot_o = nullptr;   // [B][Hq][Bs][D] cached A_out
  float* slot_l = nullptr;   // [B][Hq][Bs]    cached L_out
  uint8_t* valid = nullptr;  // [B][Hq]
  uint8_t* reuse = nullptr;  // [2][B][Hq], indexed by step parity
  float* sim = nullptr;      // [B][Hq]
  float* part_o = nullptr;   // [splits_cap + 1][B][Hq][Bs][D] (the last: a fused step's block-internal part)
  float* part_l = nullptr;   // [splits_cap + 1][B][Hq][Bs]
  float* cos_part = nullptr; // [B][Hq][row_chunks][3]
  int32_t* cum = nullptr;    // [B] cumulative rule decided on the device: updated tokens since b's last computation
  float* tot_o = nullptr;    // [B][Hq][Bs][D] sparse steps: cached part merged with the kept keys' part
  float* tot_l = nullptr;    // [B][Hq][Bs]
  int32_t* comp = nullptr;   // [B*Hkv][comp_stride] sparse steps: prefix tiles the selection leaves out
  // single-launch fused step: error flag and per-group arrival counters
  // (FinParams); null where the step keeps its two launches
  uint32_t* fin_ctr = nullptr;
  int fin_n = 0;
  // single-launch steps: FB_FIN=1 at allocation (measured no faster)
  bool fin_on = false;
  int64_t part_o_stride_override = 0;   // > 0: distance of the partials' slots in elements (caller scratch)
  int64_t part_l_stride_override = 0;
  int comp_stride = 1;       // ceil(max_prefix / 64), at least 1
  // host state
  int64_t steps = 0;         // fb_step calls since the last reset
  bool ext_since_reset = false;   // fb_external_attn filled the cache since the last reset
  int32_t block_prefix = -1; // prefix_len of the current block
  int32_t block_policy = -1;
  int32_t block_dev_m = -1;  // 1: the block's threshold decisions are made on the device
  int32_t block_n_sel = -1;  // sparse blocks: kept tiles per group; -1: a dense block
  std::vector<uint8_t> host_valid;   // [B]: every head of b holds a computed A_out (tau bookkeeping)
  std::vector<int64_t> cum_updated;  // [B]: TAU_CUM, updated tokens summed since b's last computation
  // profiling
  bool prof = false;
  std::vector<ProfRec> prof_recs;
  int64_t prof_launches[FB_PROFILE_KINDS] = {};
  double prof_ms[FB_PROFILE_KINDS] = {};
};

namespace {

int64_t elems_per_slot(const fb_config& c) {
  return (int64_t)c.batch * c.n_q_heads * c.block_size * c.head_dim;
}
int64_t rows_per_slot(const fb_config& c) { return (int64_t)c.batch * c.n_q_heads * c.block_size; }

fb_status check_config(const fb_config* cfg) {
  if (!cfg) return fail(FB_E_ARG, "config is null");
  if (cfg->dtype != FB_F32 && cfg->dtype != FB_BF16) return fail(FB_E_DTYPE, "dtype %d is not FB_F32 or FB_BF16", cfg->dtype);
  if (cfg->batch < 1 || cfg->batch > FB_MAX_BATCH) return fail(FB_E_SHAPE, "batch %d outside [1, %d]", cfg->batch, FB_MAX_BATCH);
  if (cfg->n_kv_heads < 1 || cfg->n_q_heads < 1 || cfg->n_q_heads > FB_MAX_HEADS)
    return fail(FB_E_SHAPE, "heads q=%d kv=%d invalid", cfg->n_q_heads, cfg->n_kv_heads);
  if (cfg->n_q_heads % cfg->n_kv_heads != 0)
    return fail(FB_E_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", cfg->n_q_heads, cfg->n_kv_heads);
  if (cfg->block_size < 1 || cfg->block_size > (1 << 20)) return fail(FB_E_SHAPE, "block_size %d invalid", cfg->block_size);
  if (cfg->max_prefix < 0) return fail(FB_E_SHAPE, "max_prefix %d is negative", cfg->max_prefix);
  if (!(cfg->softmax_scale == cfg->softmax_scale) || std::isinf(cfg->softmax_scale))
    return fail(FB_E_ARG, "softmax_scale is not finite");
  if (cfg->head_dim != 64 && cfg->head_dim != 128)
    return fail(FB_E_UNSUPPORTED, "head_dim %d: this build supports 64 and 128", cfg->head_dim);
  const int64_t rows = (int64_t)(cfg->n_q_heads / cfg->n_kv_heads) * cfg->block_size;
  if (rows > (1 << 24)) return fail(FB_E_SHAPE, "packed rows %lld too many", (long long)rows);
  return FB_OK;
}

// Time in tiles of a launch whose first co_items workgroups take co_tiles
// tiles each and whose ext_wgs others take `per`: every CU runs one workgroup
// at a time and takes the next one (in launch order) as it frees up.  The
// moments at which CUs free up are kept as (time, CUs) pairs in a fixed,
// time-ordered table (no allocation; a launch has few distinct moments).
long span_with_co_items(int n_cu, long co_items, long co_tiles, long ext_wgs, long per) {
  constexpr int kCap = 512;
  long t_at[kCap], n_at[kCap];
  int len = 1;
  t_at[0] = 0;
  n_at[0] = n_cu;
  auto add = [&](long t, long n) {   // insert keeping times ascending, merging equal times
    int i = 0;
    while (i < len && t_at[i] < t) ++i;
    if (i < len && t_at[i] == t) {
      n_at[i] += n;
      return;
    }
    if (len == kCap) {   // out of room: fold into the last moment (a longer span, never a shorter one)
      n_at[len - 1] += n;
      t_at[len - 1] = std::max(t_at[len - 1], t);
      return;
    }
    for (int j = len; j > i; --j) {
      t_at[j] = t_at[j - 1];
      n_at[j] = n_at[j - 1];
    }
    t_at[i] = t;
    n_at[i] = n;
    ++len;
  };
  long qi = co_items, qe = ext_wgs, end = 0;
  while (qi + qe > 0 && len > 0) {
    const long t = t_at[0];
    long n = n_at[0];
    for (int j = 1; j < len; ++j) {   // pop the earliest moment
      t_at[j - 1] = t_at[j];
      n_at[j - 1] = n_at[j];
    }
    --len;
    const long a = std::min(n, qi);
    if (a > 0) {
      add(t + co_tiles, a);
      qi -= a;
      n -= a;
      end = std::max(end, t + co_tiles);
    }
    const long b = std::min(n, qe);
    if (b > 0) {
      add(t + per, b);
      qe -= b;
      end = std::max(end, t + per);
    }
  }
  return end;
}

// Number of prefix chunks.  Each (group, row tile, chunk) is one workgroup
// and each CU runs one at a time, so the time goes as
// ceil(workgroups / CUs) x tiles per chunk (with a fused step's
// block-internal workgroups in the same launch: as span_with_co_items
// gives).  Take the smallest chunk count within 2 % of the best such time
// (more chunks mean more partial traffic), with at least two 64-key tiles
// per chunk and at most the scratch capacity.
int choose_splits(fb_cache* c, int n_keys, int active_groups, int co_items = 0, int co_tiles = 0) {
  const int tiles = (n_keys + fbk::kKeyTile - 1) / fbk::kKeyTile;
  if (tiles <= 1) return 1;
  int want;
  if (c->kv_splits > 0) {
    want = c->kv_splits;
  } else {
    const int hit = c->split_memo.find(n_keys, active_groups, co_items, co_tiles);
    if (hit >= 0) return hit;
    const int base = std::max(1, active_groups * c->row_tiles);
    const int smax = std::max(1, std::min({tiles / 2, c->splits_cap, fbk::kMaxSplits}));
    // makespan in tiles: rounds of workgroups x tiles per chunk, after
    // rounding the chunks to whole tiles
    auto span = [&](int sp) {
      const int per = (tiles + sp - 1) / sp, eff = (tiles + per - 1) / per;
      if (co_items > 0) return (double)span_with_co_items(c->n_cu, co_items, co_tiles, (long)base * eff, per);
      return (double)((base * eff + c->n_cu - 1) / c->n_cu) * per;
    };
    double best = 1e30;
    for (int sp = 1; sp <= smax; ++sp) best = std::min(best, span(sp));
    want = 1;
    while (want < smax && span(want) > 1.02 * best) ++want;
    want = std::max(1, std::min({want, tiles, c->splits_cap}));
    const int tiles_per = (tiles + want - 1) / want;
    const int sp = (tiles + tiles_per - 1) / tiles_per;   // no empty chunk
    c->split_memo.put(n_keys, active_groups, co_items, co_tiles, sp);
    return sp;
  }
  want = std::max(1, std::min({want, tiles, c->splits_cap}));
  const int tiles_per = (tiles + want - 1) / want;
  return (tiles + tiles_per - 1) / tiles_per;   // no empty chunk
}

// Two key sets in one launch (a sparse step's left-out tiles for the groups1
// groups that recompute, its kept tiles for every group): the first set's
// chunk count when both are cut into chunks of the same length, taken as in
// choose_splits (the fewest chunks within 2 % of the best makespan, the
// block-internal workgroups included), with both sets' chunks together at
// most the scratch capacity; 0 if no length fits.
int choose_splits2(fb_cache* c, int t1, int groups1, int t2, int co_items, int co_tiles) {
  const int hit = c->split_memo.find(t1, groups1, co_items, -1 - t2);   // (a key no one-set entry has)
  if (hit >= 0) return hit;
  const long g_all = (long)c->cfg.batch * c->cfg.n_kv_heads;
  auto span = [&](int s1, int* e1_out) -> double {
    const int per = (t1 + s1 - 1) / s1, e1 = (t1 + per - 1) / per, e2 = (t2 + per - 1) / per;
    *e1_out = e1;
    if (e1 + e2 > c->splits_cap) return -1.0;
    const long items = ((long)groups1 * e1 + g_all * e2) * c->row_tiles;
    if (co_items > 0) return (double)span_with_co_items(c->n_cu, co_items, co_tiles, items, per);
    return (double)((items + c->n_cu - 1) / c->n_cu) * per;
  };
  const int smax = std::max(1, std::min(t1, c->splits_cap));
  double best = 1e30;
  int e1;
  for (int s1 = 1; s1 <= smax; ++s1) {
    const double v = span(s1, &e1);
    if (v >= 0.0) best = std::min(best, v);
  }
  int pick = 0;
  if (best < 1e30)
    for (int s1 = 1; s1 <= smax; ++s1) {
      const double v = span(s1, &e1);
      if (v >= 0.0 && v <= 1.02 * best) {
        pick = e1;
        break;
      }
    }
  c->split_memo.put(t1, groups1, co_items, -1 - t2, pick);
  return pick;
}

// Profiling records HIP events, which stream capture would take into a graph.
fb_status check_not_capturing_profiled(const fb_cache* c, hipStream_t s) {
  if (!c->prof) return FB_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return hip_fail(e, "stream capture query");
  if (cs != hipStreamCaptureStatusNone) return fail(FB_E_STATE, "profiling is on while the stream is being captured");
  return FB_OK;
}

void prof_begin(fb_cache* c, hipStream_t s, ProfRec* r, int kind) {
  r->kind = -1;
  if (!c->prof) return;
  if (hipEventCreate(&r->start) != hipSuccess) return;
  if (hipEventCreate(&r->stop) != hipSuccess) {
    (void)hipEventDestroy(r->start);
    return;
  }
  r->kind = kind;
  (void)hipEventRecord(r->start, s);
}
void prof_end(fb_cache* c, hipStream_t s, ProfRec* r) {
  if (r->kind < 0) return;
  (void)hipEventRecord(r->stop, s);
  c->prof_recs.push_back(*r);
}

fbk::HeadSel all_heads(const fb_cache* c) {
  fbk::HeadSel h{};
  for (int b = 0; b < c->cfg.batch; ++b) h.seq_bits[b >> 5] |= 1u << (b & 31);
  h.every_seq = 1;
  h.flags = nullptr;
  h.flags_select = 1;
  return h;
}

// Device split plan for up to kDynMaxGroups groups: for n active groups, the
// split count the host would choose for n groups (makespan rule).  The
// scratch allows at most max(static choice, kDynSplitCap) splits.
constexpr int kDynSplitCap = 16;
constexpr int kShortItemKeys = 6 * fbk::kKeyTile;   // work items up to this many keys: the one-wave-per-SIMD shape
bool dyn_possible(const fb_cache* c) { return c->cfg.batch * c->cfg.n_kv_heads <= fbk::kDynMaxGroups; }
void plan_dyn(fb_cache* c, int n_keys, int co_items = 0, int co_tiles = 0) {
  if (c->dyn_keys == n_keys && c->dyn_co == co_items) return;
  const int groups = c->cfg.batch * c->cfg.n_kv_heads;
  const int tiles = (n_keys + fbk::kKeyTile - 1) / fbk::kKeyTile;
  c->dyn.groups = groups;
  c->dyn.splits[0] = 1;
  c->dyn_grid = 0;
  int min_splits = fbk::kMaxSplits;
  for (int n = 1; n <= groups; ++n) {
    const int sp = choose_splits(c, n_keys, n, co_items, co_tiles);
    c->dyn.splits[n] = (uint8_t)sp;
    c->dyn_grid = std::max(c->dyn_grid, n * c->row_tiles * sp);
    min_splits = std::min(min_splits, sp);
  }
  c->dyn_kps = std::max(1, (tiles + min_splits - 1) / min_splits) * fbk::kKeyTile;
  c->dyn_keys = n_keys;
  c->dyn_co = co_items;
}

fbk::AttnParams attn_common(const fb_cache* c, const void* q, int waves, int ksplit) {
  fbk::AttnParams p{};
  p.waves = waves;
  p.ksplit = ksplit;
  const int rows_per_wg = 32 * waves / ksplit;
  p.row_tiles = (c->rows + rows_per_wg - 1) / rows_per_wg;
  p.q = q;
  p.batch = c->cfg.batch;
  p.hq = c->cfg.n_q_heads;
  p.hkv = c->cfg.n_kv_heads;
  p.bs = c->cfg.block_size;
  p.rows = c->rows;
  p.grp = c->group;
  p.scale_log2 = c->scale * 1.4426950408889634f;
  p.int_count = 0;   // no block-internal items unless a fused step adds them
  return p;
}

// Prefix keys of an external launch: rows 0..n_keys-1, or (tiles not null)
// the listed 64-row tiles of each group, n_keys = 64 per listed tile.
struct KeySet {
  int32_t n_keys;
  const int32_t* tiles;
  int32_t stride;
  int32_t n_phys;
};
KeySet dense_keys(int32_t n) { return KeySet{n, nullptr, 0, n}; }

// Options of an external launch and its split combine.
struct ExtOpts {
  bool gamma = false;        // the combine sums similarity terms as it replaces cached values
  uint8_t* rec = nullptr;    // the attention launch records its per-head decisions there
  bool follow_rec = true;    // the combine selects by that record (decisions made on the device);
                             // false: by `sel` itself (host decisions: no flag load before its work)
  bool to_total = false;     // the combine adds the cached part (sparse steps' kept keys)
  // fused step: the attention launch also runs the block-internal items and
  // the combine writes the step's output (every head)
  const void* kblk = nullptr;
  const void* vblk = nullptr;
  void* out = nullptr;
  const int32_t* cum_m = nullptr;   // cumulative threshold decided on the device
  // threshold decided on the device at a step after the block's first: every
  // head's valid flag is already set, so the step may run as one launch
  // whose workgroups each evaluate the rule (see run_external)
  bool fin_dev = false;
  bool rec_reuse_all = false;   // the attention launch records reuse for every head (rec, not followed)
  // A second key set attended for every head in the same launch (sparse
  // steps: the kept tiles), folded by the same combine onto each head's
  // cached part before the block-internal part (fused steps only).  When its
  // splits do not fit the partial buffer next to the first set's, nothing is
  // launched and *set2_done is false.
  const KeySet* set2 = nullptr;
  bool* set2_done = nullptr;
};

// External attention over a key set for the heads `sel` selects, and the
// split combine into the cache (or, to_total, the total buffer).  A fused
// step appends the block-internal items to the same launch and has the
// combine merge them in and store the output, so one attention launch and
// one combine make the whole step.
fb_status run_external(fb_cache* c, const void* q, const void* kp, const void* vp, const KeySet& ks,
                       const fbk::HeadSel& sel, int active_groups, hipStream_t s, const ExtOpts& o) {
  const int32_t n = ks.n_keys;
  const bool fused = o.out != nullptr;
  fbk::AttnParams p = attn_common(c, q, c->ext_waves, c->ext_ksplit);
  p.k = kp;
  p.v = vp;
  p.kv_cap = c->cfg.max_prefix;
  p.n_keys = n;
  p.tiles = ks.tiles;
  p.tiles_stride = ks.stride;
  p.n_phys = ks.n_phys;
  // a fused step's block-internal workgroups share the launch (and the CUs)
  const int co_items = fused ? c->cfg.batch * c->cfg.n_kv_heads * p.row_tiles : 0;
  const int co_tiles = (c->cfg.block_size + fbk::kKeyTile - 1) / fbk::kKeyTile;
  p.splits = choose_splits(c, n, active_groups, co_items, co_tiles);
  const int tiles = (n + fbk::kKeyTile - 1) / fbk::kKeyTile;
  p.keys_per_split = std::max(1, (tiles + p.splits - 1) / p.splits) * fbk::kKeyTile;
  int ext_items = c->cfg.batch * c->cfg.n_kv_heads * p.splits * p.row_tiles;
  if ((sel.flags != nullptr || sel.m != nullptr) && dyn_possible(c) && n > 0) {
    plan_dyn(c, n, co_items, co_tiles);   // heads chosen on the device: the split count follows how many groups it selects
    p.dyn = c->dyn;
    ext_items = c->dyn_grid;
    p.keys_per_split = c->dyn_kps;   // the longest range the plan may pick (LDS sizing)
  } else if (sel.flags == nullptr && sel.m == nullptr && dyn_possible(c) && n > 0 &&
             active_groups < c->cfg.batch * c->cfg.n_kv_heads) {
    // some sequences chosen on the host: enumerate only their groups, so the
    // work spreads over every XCD instead of the slice of the grid they own
    plan_dyn(c, n, co_items, co_tiles);
    p.dyn = c->dyn;
    ext_items = active_groups * p.row_tiles * p.splits;   // p.splits == dyn.splits[active_groups]
  }
  const bool skip_ext = o.to_total && n == 0;   // nothing kept: the total is the cached part
  if (skip_ext) ext_items = 0;
  p.ring_keys = p.keys_per_split;
  int seg2_items = 0;
  if (o.set2 != nullptr) {
    // The second set for every group, a static plan.  Where the host knows
    // the first set's groups (static plan, or its own decisions), both sets
    // are cut into items of one length chosen together (choose_splits2);
    // with decisions made on the device, the second set's items take the
    // first set's longest range.  Either way in as many ranges as the partial
    // buffer has left after the first set's.
    const KeySet& k2 = *o.set2;
    const int G = c->cfg.batch * c->cfg.n_kv_heads;
    const int tiles2 = (k2.n_keys + fbk::kKeyTile - 1) / fbk::kKeyTile;
    const bool dev_dyn = p.dyn.groups > 0 && (sel.flags != nullptr || sel.m != nullptr);
    int base2 = p.splits, s2 = -1;
    if (!dev_dyn && n > 0 && tiles2 > 0 && c->kv_splits == 0) {
      const int A = p.dyn.groups > 0 ? active_groups : G;
      const int s1 = choose_splits2(c, tiles, A, tiles2, co_items, co_tiles);
      if (s1 > 0) {
        const int per = (tiles + s1 - 1) / s1;
        if (p.dyn.groups > 0) {
          p.dyn.splits[A] = (uint8_t)s1;   // the host's own decisions select A groups
          p.keys_per_split = std::max(p.keys_per_split, per * fbk::kKeyTile);   // LDS sizing: the longest range
        } else {
          p.splits = s1;
          p.keys_per_split = per * fbk::kKeyTile;
        }
        ext_items = A * p.row_tiles * s1;
        base2 = s1;
        s2 = (tiles2 + per - 1) / per;
      }
    }
    if (s2 < 0) {
      for (int g = 1; g <= p.dyn.groups; ++g) base2 = std::max(base2, (int)p.dyn.splits[g]);
      const int kps_tiles = std::max(1, p.keys_per_split / fbk::kKeyTile);
      s2 = std::min((tiles2 + kps_tiles - 1) / kps_tiles, c->splits_cap - base2);
    }
    if (!fused || (tiles2 > 0 && s2 < 1)) {
      if (o.set2_done) *o.set2_done = false;
      return FB_OK;
    }
    if (o.set2_done) *o.set2_done = true;
    p.tiles2 = k2.tiles;
    p.tiles2_stride = k2.stride;
    p.n_keys2 = k2.n_keys;
    p.seg2_splits = s2;
    p.seg2_kps = s2 > 0 ? std::max(1, (tiles2 + s2 - 1) / s2) * fbk::kKeyTile : fbk::kKeyTile;
    p.seg2_base = base2;
    seg2_items = G * s2 * p.row_tiles;
    p.seg2_items = seg2_items;
    p.ring_keys = std::max(p.ring_keys, p.keys_per_split);
    if (s2 > 0) p.ring_keys = std::max(p.ring_keys, p.seg2_kps);
  }
  p.grid = ext_items + seg2_items;
  if (fused) {
    p.kblk = o.kblk;
    p.vblk = o.vblk;
    p.int_count = c->cfg.batch * c->cfg.n_kv_heads * p.row_tiles;
    p.int_split = c->splits_cap;
    p.grid = ext_items + seg2_items + p.int_count;
    p.ring_keys = std::max(p.ring_keys, ((c->cfg.block_size + fbk::kKeyTile - 1) / fbk::kKeyTile) * fbk::kKeyTile);
  }
  // Short work items (few tiles each, as at dLLM prefix lengths) run one
  // wave per SIMD over whole tiles instead of two waves on the key halves:
  // a short loop cannot hide the key-half exchange and its barrier, a long
  // one gains from the second wave (measured crossover 6-8 tiles per item).
  // The rows per workgroup, hence the row tiles and the split plan, are the
  // same for both shapes.
  if (p.ksplit == 2 && p.ring_keys <= kShortItemKeys) {
    p.waves = 4;
    p.ksplit = 1;
  }
  p.sel = sel;
  p.reuse_rec = o.rec;
  p.rec_reuse_all = o.rec_reuse_all ? 1 : 0;
  p.part_o = c->part_o;
  p.part_l = c->part_l;
  p.part_o_stride = c->part_o_stride_override > 0 ? c->part_o_stride_override : elems_per_slot(c->cfg);
  p.part_l_stride = c->part_l_stride_override > 0 ? c->part_l_stride_override : rows_per_slot(c->cfg);
  fbk::CombineParams cp{};
  cp.part_o = c->part_o;
  cp.part_l = c->part_l;
  cp.part_o_stride = p.part_o_stride;
  cp.part_bf16 = c->cfg.dtype == FB_BF16 ? 1 : 0;   // the bf16 kernels hand partial A over in bf16
  cp.part_l_stride = p.part_l_stride;
  cp.splits = skip_ext ? 0 : p.splits;
  cp.batch = c->cfg.batch;
  cp.hq = c->cfg.n_q_heads;
  cp.hkv = c->cfg.n_kv_heads;
  cp.dyn = p.dyn;
  cp.bs = c->cfg.block_size;
  cp.row_chunks = c->row_chunks;
  cp.sel = sel;
  // A threshold step decided on the device after the block's first may run
  // as one launch (below, opt-in): every workgroup, the combine's included, evaluates
  // the rule from flags that no workgroup of the launch changes (the valid
  // flags are all set after the block's first step, and the combine leaves
  // them alone), so they all see the same decisions and the same plan.
  const bool fin_dev = o.fin_dev && c->fin_ctr != nullptr && c->fin_on && fused && !o.to_total &&
                       o.cum_m == nullptr && sel.flags == nullptr && sel.m != nullptr && ext_items > 0 &&
                       fbk::fin_supported(c->cfg.dtype, c->cfg.head_dim, p);
  if (o.rec != nullptr && o.follow_rec && !fin_dev) {
    cp.sel = all_heads(c);
    cp.sel.flags = o.rec;
    cp.sel.flags_select = 0;
  }
  cp.keep_valid = fin_dev ? 1 : 0;
  cp.slot_o = c->slot_o;
  cp.slot_l = c->slot_l;
  cp.valid = c->valid;
  cp.sim_terms = o.gamma ? 1 : 0;
  cp.cos_part = c->cos_part;
  if (o.to_total) {
    cp.tot_o = c->tot_o;
    cp.tot_l = c->tot_l;
  }
  if (o.set2 != nullptr) {
    cp.two_sets = 1;
    cp.splits2 = p.seg2_splits;
    cp.base2 = p.seg2_base;
  }
  if (fused) {
    cp.out = o.out;
    cp.out_bf16 = c->cfg.dtype == FB_BF16 ? 1 : 0;
    cp.int_split = c->splits_cap;
  }
  if (o.cum_m != nullptr) {
    cp.cum = c->cum;
    cp.cum_m = o.cum_m;
  }
  // One launch for the whole step (opt-in, FB_FIN=1): the split and
  // block-internal items and the combine share a grid (FinParams); a group
  // whose heads all reuse is finished by its block-internal items.  The same
  // caches and decisions, and the same outputs for recomputed heads, as the
  // two launches.  Measured no faster: dllm-8k 19.5 against 18.2 us per
  // recompute step (long and max within 1 %); with device decisions a step
  // in which every head reuses still takes 9.5-10 us, most of it the
  // block-internal workgroup's own chain of dependent steps (parameters,
  // loads, one key tile, the merge: 8.3 us, against 2.9 us for a workgroup
  // of the lone-wave merge launch), so the two launches stay the default.
  const bool fin = fin_dev || (c->fin_ctr != nullptr && c->fin_on && fused && !o.to_total &&
                                o.cum_m == nullptr && !(o.rec != nullptr && o.follow_rec) && ext_items > 0 &&
                                sel.flags == nullptr && sel.m == nullptr &&
                                fbk::fin_supported(c->cfg.dtype, c->cfg.head_dim, p));
  ProfRec r;
  hipError_t e = hipSuccess;
  if (fin) {
    fbk::FinParams f{};
    f.cp = cp;
    f.ctr = c->fin_ctr;
    f.n_attn = p.grid;
    f.chunks = (c->row_chunks + p.waves - 1) / p.waves;
    f.n_total = p.grid + c->cfg.batch * c->cfg.n_q_heads * f.chunks;
    const int grp = c->cfg.n_q_heads / c->cfg.n_kv_heads;
    f.need = (uint32_t)((p.splits + 1) * p.row_tiles);   // static plan; a device plan counts in the kernel
    f.done_all = f.need + (uint32_t)(grp * f.chunks);
    f.row_tiles = p.row_tiles;
    // groups that reuse are finished by their block-internal items
    f.merge_reused = 1;
    p.slot_o = c->slot_o;
    p.slot_l = c->slot_l;
    p.valid = c->valid;
    p.out = o.out;
    prof_begin(c, s, &r, 0);
    e = fbk::launch_attn_fin(p, f, s);
    prof_end(c, s, &r);
    if (e != hipSuccess) return hip_fail(e, "single-launch step");
    return FB_OK;
  }
  if (p.grid > 0) {
    prof_begin(c, s, &r, o.to_total ? 5 : 0);
    e = fbk::launch_attn(c->cfg.dtype, c->cfg.head_dim, fbk::kModePartial, p, s);
    prof_end(c, s, &r);
    if (e != hipSuccess) return hip_fail(e, "external attention launch");
  }

  prof_begin(c, s, &r, o.to_total ? 6 : 1);
  e = fbk::launch_combine(c->cfg.head_dim, cp, s);
  prof_end(c, s, &r);
  if (e != hipSuccess) return hip_fail(e, "split combine launch");
  return FB_OK;
}

// Block-internal attention merged with the cached external part, one launch:
// the step when no head recomputes (and fb_internal_attn_merge).
fb_status run_internal(fb_cache* c, const void* q, const void* kb, const void* vb, void* out,
                       const fbk::HeadSel& rec_sel, uint8_t* reuse_rec, hipStream_t s) {
  fbk::AttnParams p = attn_common(c, q, c->int_waves, c->int_ksplit);
  p.k = kb;
  p.v = vb;
  p.kv_cap = c->cfg.block_size;
  p.n_keys = c->cfg.block_size;
  p.splits = 1;
  p.keys_per_split = ((c->cfg.block_size + fbk::kKeyTile - 1) / fbk::kKeyTile) * fbk::kKeyTile;
  p.ring_keys = p.keys_per_split;
  p.sel = rec_sel;
  p.slot_o = c->slot_o;
  p.slot_l = c->slot_l;
  p.valid = c->valid;
  p.out = out;
  p.reuse_rec = reuse_rec;
  ProfRec r;
  prof_begin(c, s, &r, 2);
  hipError_t e = fbk::launch_attn(c->cfg.dtype, c->cfg.head_dim, fbk::kModeMerge, p, s);
  prof_end(c, s, &r);
  if (e != hipSuccess) return hip_fail(e, "internal attention launch");
  return FB_OK;
}

fb_status run_reset(fb_cache* c, hipStream_t s) {
  fbk::ResetParams rp{};
  rp.n_heads = c->cfg.batch * c->cfg.n_q_heads;
  rp.batch = c->cfg.batch;
  rp.cum = c->cum;
  rp.valid = c->valid;
  rp.reuse = c->reuse;
  rp.sim = c->sim;
  rp.fin_ctr = c->fin_ctr;
  rp.fin_n = c->fin_n;
  ProfRec r;
  prof_begin(c, s, &r, 4);
  hipError_t e = fbk::launch_reset(rp, s);
  prof_end(c, s, &r);
  if (e != hipSuccess) return hip_fail(e, "reset launch");
  c->steps = 0;
  c->ext_since_reset = false;
  c->block_prefix = -1;
  c->block_policy = -1;
  c->block_dev_m = -1;
  c->block_n_sel = -1;
  std::fill(c->host_valid.begin(), c->host_valid.end(), 0);
  std::fill(c->cum_updated.begin(), c->cum_updated.end(), 0);
  return FB_OK;
}

void free_all(fb_cache* c) {
  void* ptrs[] = {c->slot_o, c->slot_l,   c->valid, c->reuse, c->sim,   c->part_o,
                  c->part_l, c->cos_part, c->cum,   c->tot_o, c->tot_l, c->comp, c->fin_ctr};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  for (auto& r : c->prof_recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
}

}  // namespace

extern "C" {

const char* fb_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

// Launch shapes of a cache of this config (no device state).
void setup_shape(fb_cache* c, const fb_config* cfg) {
  c->cfg = *cfg;
  c->group = cfg->n_q_heads / cfg->n_kv_heads;
  c->rows = c->group * cfg->block_size;
  if (cfg->dtype == FB_BF16) {
    // up to 128 rows: 4 row waves + 4 waves on the other key half of each
    // tile; more rows: 8 row waves; 32 rows or fewer: a single wave
    if (c->rows <= 32) c->ext_waves = 1, c->ext_ksplit = 1;
    else if (c->rows <= 128) c->ext_waves = 8, c->ext_ksplit = 2;
    else c->ext_waves = 8, c->ext_ksplit = 1;
    // block-internal attention: one wave per 32 rows for small blocks, the
    // split-key 8-wave shape for frame-sized ones
    if (c->rows >= 512) c->int_waves = 8, c->int_ksplit = 2;
    else c->int_waves = 1, c->int_ksplit = 1;
  } else {
    c->ext_waves = c->int_waves = 4;   // the fp32 kernel has a fixed shape
  }
  const int ext_rows_per_wg = 32 * c->ext_waves / c->ext_ksplit;
  c->row_tiles = (c->rows + ext_rows_per_wg - 1) / ext_rows_per_wg;
  const int crows = fbk::combine_rows(cfg->head_dim);
  c->row_chunks = (cfg->block_size + crows - 1) / crows;
  c->scale = cfg->softmax_scale > 0.0f ? cfg->softmax_scale : 1.0f / std::sqrt((float)cfg->head_dim);
}

// Copies a caller's options struct that starts with its own size: the bytes
// the caller has (at most sizeof(T)); fields past them keep T's defaults.
template <typename T>
fb_status read_opts(const T* in, T* out, const char* what) {
  *out = T{};
  if (!in) return FB_OK;
  if (in->struct_size < sizeof(uint32_t)) return fail(FB_E_ARG, "%s.struct_size %u is too small", what, in->struct_size);
  std::memcpy(out, in, std::min<size_t>(in->struct_size, sizeof(T)));
  return FB_OK;
}

fb_status alloc_impl(const fb_config* cfg, int kv_splits, fb_cache** out) {
  if (!out) return fail(FB_E_ARG, "out is null");
  fb_status st = check_config(cfg);
  if (st != FB_OK) return st;
  if (kv_splits < 0 || kv_splits > fbk::kMaxSplits)
    return fail(FB_E_ARG, "kv_splits %d outside [0, %d]", kv_splits, fbk::kMaxSplits);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "no usable HIP device");
  int ndev = 0;
  e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev < 1) return fail(FB_E_HIP, "no usable HIP device");

  fb_cache* c = new (std::nothrow) fb_cache();
  if (!c) return fail(FB_E_NOMEM, "host allocation failed");
  setup_shape(c, cfg);
  c->kv_splits = kv_splits;
  c->device = dev;
  c->host_valid.assign(cfg->batch, 0);
  c->cum_updated.assign(cfg->batch, 0);
  {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
      c->n_cu = prop.multiProcessorCount;
  }
  c->splits_cap = fbk::kMaxSplits;
  {
    int cap = choose_splits(c, cfg->max_prefix, cfg->batch * cfg->n_kv_heads);
    if (dyn_possible(c))   // room for the device plan's shorter ranges when few groups are active
      for (int n = 1; n < cfg->batch * cfg->n_kv_heads; ++n)
        cap = std::max(cap, std::min(kDynSplitCap, choose_splits(c, cfg->max_prefix, n)));
    c->splits_cap = cap;
  }
  if (kv_splits > 0) c->splits_cap = std::max(c->splits_cap, std::min(kv_splits, fbk::kMaxSplits));
  c->split_memo.clear();   // those choices were made before the cap was known

  c->comp_stride = std::max(1, (cfg->max_prefix + fbk::kKeyTile - 1) / fbk::kKeyTile);
  c->fin_n = (fbk::kFinCounters + cfg->batch * cfg->n_kv_heads) * fbk::kFinStride;
  {
    const char* e_fin = std::getenv("FB_FIN");
    c->fin_on = e_fin != nullptr && e_fin[0] == '1';
  }
  const int64_t nh = (int64_t)cfg->batch * cfg->n_q_heads;
  const size_t so = elems_per_slot(*cfg) * sizeof(float), sl = rows_per_slot(*cfg) * sizeof(float);
  struct {
    void** p;
    size_t n;
  } plan[] = {
      {(void**)&c->slot_o, so},
      {(void**)&c->slot_l, sl},
      {(void**)&c->valid, (size_t)nh},
      {(void**)&c->reuse, (size_t)(2 * nh)},
      {(void**)&c->sim, (size_t)nh * sizeof(float)},
      {(void**)&c->part_o, (size_t)(c->splits_cap + 1) * so},   // + the block-internal partial of a fused step
      {(void**)&c->part_l, (size_t)(c->splits_cap + 1) * sl},
      {(void**)&c->cos_part, (size_t)nh * c->row_chunks * 3 * sizeof(float)},
      {(void**)&c->cum, (size_t)cfg->batch * sizeof(int32_t)},
      {(void**)&c->tot_o, so},
      {(void**)&c->tot_l, sl},
      {(void**)&c->comp, (size_t)cfg->batch * cfg->n_kv_heads * c->comp_stride * sizeof(int32_t)},
      {(void**)&c->fin_ctr, (size_t)c->fin_n * sizeof(uint32_t)},
  };
  for (auto& a : plan) {
    e = hipMalloc(a.p, std::max<size_t>(a.n, 256));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      free_all(c);
      delete c;
      return fail(FB_E_NOMEM, "device allocation of %zu bytes failed: %s", a.n, hipGetErrorString(e));
    }
    c->bytes += a.n;
  }
  st = run_reset(c, nullptr);
  if (st == FB_OK) {
    e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess) st = hip_fail(e, "cache initialisation");
  }
  if (st != FB_OK) {
    free_all(c);
    delete c;
    return st;
  }
  *out = c;
  return ok();
}

}  // namespace

extern "C" {

fb_status fb_cache_alloc(const fb_config* cfg, fb_cache** out) { return alloc_impl(cfg, 0, out); }

fb_status fb_cache_alloc_ex(const fb_config* cfg, const fb_cache_opts* opts, fb_cache** out) {
  fb_cache_opts o;
  if (fb_status st = read_opts(opts, &o, "fb_cache_opts"); st != FB_OK) return st;
  return alloc_impl(cfg, o.kv_splits, out);
}

fb_status fb_cache_free(fb_cache* c) {
  if (!c) return ok();
  DeviceGuard g(c->device);
  (void)hipDeviceSynchronize();
  free_all(c);
  delete c;
  return ok();
}

fb_status fb_cache_reset(fb_cache* c, void* stream) {
  if (!c) return fail(FB_E_ARG, "cache is null");
  DeviceGuard g(c->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "set device");
  if (fb_status pst = check_not_capturing_profiled(c, (hipStream_t)stream); pst != FB_OK) return pst;
  fb_status st = run_reset(c, (hipStream_t)stream);
  return st == FB_OK ? ok() : st;
}

fb_status fb_external_attn(fb_cache* c, const void* q_blk, const void* k_prefix, const void* v_prefix,
                           int32_t prefix_len, const uint8_t* head_mask, void* stream) {
  if (!c) return fail(FB_E_ARG, "cache is null");
  if (!q_blk) return fail(FB_E_ARG, "q_blk is null");
  if (prefix_len < 0 || prefix_len > c->cfg.max_prefix)
    return fail(FB_E_SHAPE, "prefix_len %d outside [0, max_prefix=%d]", prefix_len, c->cfg.max_prefix);
  if (prefix_len > 0 && (!k_prefix || !v_prefix)) return fail(FB_E_ARG, "k_prefix/v_prefix is null");
  DeviceGuard g(c->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "set device");
  fbk::HeadSel sel = all_heads(c);
  sel.flags = head_mask;
  sel.flags_select = 1;
  fb_status st = run_external(c, q_blk, k_prefix, v_prefix, dense_keys(prefix_len), sel,
                              c->cfg.batch * c->cfg.n_kv_heads, (hipStream_t)stream, ExtOpts{});
  if (st != FB_OK) return st;
  std::fill(c->host_valid.begin(), c->host_valid.end(), head_mask ? 0 : 1);
  c->ext_since_reset = true;
  return ok();
}

fb_status fb_internal_attn_merge(fb_cache* c, const void* q_blk, const void* k_blk, const void* v_blk,
                                 void* out, void* stream) {
  if (!c) return fail(FB_E_ARG, "cache is null");
  if (!q_blk || !k_blk || !v_blk || !out) return fail(FB_E_ARG, "a tensor pointer is null");
  DeviceGuard g(c->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "set device");
  fb_status st = run_internal(c, q_blk, k_blk, v_blk, out, all_heads(c), nullptr, (hipStream_t)stream);
  return st == FB_OK ? ok() : st;
}

}  // extern "C"

namespace {

// Sparse attention's kept prefix tiles for a step (null: a dense step).
struct SparseSel {
  const int32_t* sel;   // device int32 [B][Hkv][n_sel]
  int32_t n_sel;
};

// One denoising step, dense or over a sparse selection.  Dense: the cached
// external part covers prefix rows 0..prefix_len-1.  Sparse: it covers the
// prefix tiles the selection leaves out (their list is built at the block's
// first step), and the kept tiles are attended afresh for every head at every
// step and folded with it into the total buffer that the merge reads.
fb_status step_impl(fb_cache* c, const fb_policy_args* pa, const fb_step_opts* opts_in, const void* q_blk,
                    const void* k_blk, const void* v_blk, const void* k_prefix, const void* v_prefix,
                    int32_t prefix_len, const SparseSel* sp, void* out, void* stream) {
  if (!c) return fail(FB_E_ARG, "cache is null");
  if (!pa) return fail(FB_E_ARG, "policy args are null");
  fb_step_opts opts;
  if (fb_status ost = read_opts(opts_in, &opts, "fb_step_opts"); ost != FB_OK) return ost;
  const int32_t* const n_updated_dev = opts.n_updated_dev;
  if (!q_blk || !k_blk || !v_blk || !out) return fail(FB_E_ARG, "a tensor pointer is null");
  if (pa->policy != FB_POLICY_ALWAYS && pa->policy != FB_POLICY_TAU && pa->policy != FB_POLICY_GAMMA &&
      pa->policy != FB_POLICY_TAU_CUM && pa->policy != FB_POLICY_GAMMA_GROUP)
    return fail(FB_E_ARG, "unknown policy %d", pa->policy);
  const bool tau_like = pa->policy == FB_POLICY_TAU || pa->policy == FB_POLICY_TAU_CUM;
  const bool gamma_like = pa->policy == FB_POLICY_GAMMA || pa->policy == FB_POLICY_GAMMA_GROUP;
  if (prefix_len < 0 || prefix_len > c->cfg.max_prefix)
    return fail(FB_E_SHAPE, "prefix_len %d outside [0, max_prefix=%d]", prefix_len, c->cfg.max_prefix);
  if (prefix_len > 0 && (!k_prefix || !v_prefix)) return fail(FB_E_ARG, "k_prefix/v_prefix is null");
  if (c->steps > 0 && prefix_len != c->block_prefix)
    return fail(FB_E_STATE, "prefix_len %d differs from %d used earlier in this block (reset first)",
                prefix_len, c->block_prefix);
  if (c->steps > 0 && pa->policy != c->block_policy)
    return fail(FB_E_STATE, "policy changed inside a block (reset first)");
  const int32_t n_tiles = (prefix_len + fbk::kKeyTile - 1) / fbk::kKeyTile;
  if (sp) {
    if (sp->n_sel < 0 || sp->n_sel > n_tiles)
      return fail(FB_E_SHAPE, "n_sel %d outside [0, %d prefix tiles]", sp->n_sel, n_tiles);
    if (sp->n_sel > 0 && !sp->sel) return fail(FB_E_ARG, "sel is null");
  }
  const int32_t n_sel = sp ? sp->n_sel : -1;
  if (c->steps > 0 && n_sel != c->block_n_sel)
    return fail(FB_E_STATE, "the sparse selection (or its absence) changed inside a block (reset first)");
  const int B = c->cfg.batch;
  const bool dev_m = tau_like && n_updated_dev != nullptr;
  if (tau_like) {
    if (pa->tau < 0) return fail(FB_E_ARG, "tau %d is negative", pa->tau);
    if (!pa->n_updated && !n_updated_dev) return fail(FB_E_ARG, "n_updated is null under the tau policy");
    if (pa->n_updated && n_updated_dev) return fail(FB_E_ARG, "both n_updated and n_updated_dev are set");
    if (!dev_m)
      for (int b = 0; b < B; ++b)
        if (pa->n_updated[b] < 0) return fail(FB_E_ARG, "n_updated[%d] = %d is negative", b, pa->n_updated[b]);
  }
  if (c->steps > 0 && (dev_m ? 1 : 0) != c->block_dev_m)
    return fail(FB_E_STATE, "decisions moved between host and device inside a block (reset first)");
  if (gamma_like && !(pa->gamma == pa->gamma)) return fail(FB_E_ARG, "gamma is NaN");
  // sequences whose heads recompute the external part (TAU decides per sequence)
  fbk::HeadSel sel{};
  int active = 0;
  std::vector<uint8_t> reuse_seq(B, 0);
  for (int b = 0; b < B && !dev_m; ++b) {
    bool reuse = false;
    const bool has = c->steps > 0 && c->host_valid[b];   // the first step of a block recomputes
    if (pa->policy == FB_POLICY_TAU) reuse = has && pa->n_updated[b] < pa->tau;
    if (pa->policy == FB_POLICY_TAU_CUM) reuse = has && c->cum_updated[b] + pa->n_updated[b] < pa->tau;
    reuse_seq[b] = reuse ? 1 : 0;
    if (!reuse) {
      sel.seq_bits[b >> 5] |= 1u << (b & 31);
      ++active;
    }
  }
  sel.every_seq = active == B ? 1 : 0;
  DeviceGuard g(c->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "set device");
  hipStream_t s = (hipStream_t)stream;
  if (fb_status pst = check_not_capturing_profiled(c, s); pst != FB_OK) return pst;
  if (c->steps == 0 && c->ext_since_reset) {
    // fb_external_attn filled the cache after the reset: empty it again, so
    // that the device-side flags (valid, similarity) make this first step
    // recompute every head as the host's decisions above do
    if (fb_status rst = run_reset(c, s); rst != FB_OK) return rst;
  }
  const int64_t nh = (int64_t)B * c->cfg.n_q_heads;
  uint8_t* reuse_now = c->reuse + (c->steps & 1) * nh;
  uint8_t* reuse_next = c->reuse + ((c->steps + 1) & 1) * nh;
  // the cached external part: the whole prefix, or the tiles the selection leaves out
  KeySet cached = dense_keys(prefix_len);
  if (sp) {
    cached = KeySet{(n_tiles - n_sel) * fbk::kKeyTile, c->comp, c->comp_stride, prefix_len};
    if (c->steps == 0) {
      fbk::ComplementParams cpl{};
      cpl.sel = sp->sel;
      cpl.n_sel = n_sel;
      cpl.tiles = n_tiles;
      cpl.comp = c->comp;
      cpl.stride = c->comp_stride;
      cpl.groups = B * c->cfg.n_kv_heads;
      ProfRec r;
      prof_begin(c, s, &r, 7);
      hipError_t e = fbk::launch_complement(cpl, s);
      prof_end(c, s, &r);
      if (e != hipSuccess) return hip_fail(e, "complement launch");
    }
  }

  fb_status st = FB_OK;
  const int groups = B * c->cfg.n_kv_heads;
  const KeySet kept = sp ? KeySet{n_sel * fbk::kKeyTile, sp->sel, n_sel, prefix_len} : KeySet{};
  bool sparse_done = false;   // the kept set went with the left-out set's launch
  // The step's external part: which heads recompute, and how (see each branch).
  ExtOpts eo;
  eo.kblk = k_blk;
  eo.vblk = v_blk;
  eo.out = out;   // fused: one attention launch and one combine for the whole step
  fbk::HeadSel ext_sel = sel;
  int ext_active = active * c->cfg.n_kv_heads;
  if (gamma_like) {
    ext_sel = all_heads(c);
    ext_sel.flags = reuse_now;
    ext_sel.flags_select = 0;   // compute the heads not marked for reuse
    ext_active = groups;
    eo.gamma = true;
  } else if (dev_m) {
    // threshold decided in the attention launch from the counts in device
    // memory; it records the decisions, the combine follows them
    ext_sel = all_heads(c);
    ext_sel.m = n_updated_dev;
    ext_sel.tau = pa->tau;
    ext_sel.valid = c->valid;
    ext_sel.cum = pa->policy == FB_POLICY_TAU_CUM ? c->cum : nullptr;
    ext_active = groups;
    eo.rec = reuse_now;
    if (pa->policy == FB_POLICY_TAU_CUM) eo.cum_m = n_updated_dev;
    eo.fin_dev = c->steps > 0 && pa->policy == FB_POLICY_TAU;
  } else {
    ext_sel.flags = nullptr;
    ext_sel.flags_select = 1;
    eo.rec = reuse_now;   // the host's per-sequence decisions, recorded per head
    eo.follow_rec = false;
  }
  if (!sp) {
    if (!gamma_like && !dev_m && active == 0) {
      // every head reuses (known on the host): block-internal attention merged
      // with the cache, one launch
      st = run_internal(c, q_blk, k_blk, v_blk, out, ext_sel, reuse_now, s);
    } else {
      st = run_external(c, q_blk, k_prefix, v_prefix, cached, ext_sel, ext_active, s, eo);
    }
    if (st != FB_OK) return st;
  } else {
    // sparse: the left-out tiles' part into the cache (recomputing heads),
    // then the kept tiles for every head folded with it, the block-internal
    // part and the output
    ExtOpts ro;
    ro.gamma = eo.gamma;
    ro.rec = eo.rec;
    ro.follow_rec = eo.follow_rec;
    ro.cum_m = eo.cum_m;   // the sums follow the decisions this combine selects by
    if (gamma_like || dev_m || active > 0) {
      // one attention launch over both key sets and one combine (the left-out
      // part into the cache, then the kept part, the block-internal part and
      // the output), where the two sets' partials fit side by side
      ExtOpts fo = ro;
      fo.kblk = k_blk;
      fo.vblk = v_blk;
      fo.out = out;
      fo.set2 = &kept;
      fo.set2_done = &sparse_done;
      st = run_external(c, q_blk, k_prefix, v_prefix, cached, ext_sel, ext_active, s, fo);
      if (st != FB_OK) return st;
      if (!sparse_done) {
        st = run_external(c, q_blk, k_prefix, v_prefix, cached, ext_sel, ext_active, s, ro);
        if (st != FB_OK) return st;
      }
    }
    // otherwise nothing recomputes (known on the host): the kept launch below
    // records the decisions
  }
  if (gamma_like) {   // similarity and the next step's decisions
    fbk::DecideParams dp{};
    dp.n_heads = (int32_t)nh;
    dp.hq = c->cfg.n_q_heads;
    dp.row_chunks = c->row_chunks;
    dp.reuse_now = reuse_now;
    dp.reuse_next = reuse_next;
    dp.valid = c->valid;
    dp.sim = c->sim;
    dp.cos_part = c->cos_part;
    dp.gamma = pa->gamma;
    dp.group = pa->policy == FB_POLICY_GAMMA_GROUP ? c->group : 1;
    ProfRec r;
    prof_begin(c, s, &r, 3);
    hipError_t e = fbk::launch_decide(dp, s);
    prof_end(c, s, &r);
    if (e != hipSuccess) return hip_fail(e, "decision launch");
  }
  if (sp && !sparse_done) {
    ExtOpts ko;
    ko.to_total = true;
    ko.kblk = k_blk;
    ko.vblk = v_blk;
    ko.out = out;
    if (!(gamma_like || dev_m || active > 0)) {
      ko.rec = reuse_now;
      ko.follow_rec = false;
      ko.rec_reuse_all = true;
    }
    st = run_external(c, q_blk, k_prefix, v_prefix, kept, all_heads(c), groups, s, ko);
    if (st != FB_OK) return st;
  }
  if (!gamma_like && !dev_m) {
    std::fill(c->host_valid.begin(), c->host_valid.end(), 1);
    for (int b = 0; b < B; ++b)   // TAU_CUM: the sum restarts where a sequence recomputed
      c->cum_updated[b] = reuse_seq[b] ? c->cum_updated[b] + pa->n_updated[b] : 0;
  }
  if (c->steps == 0) {
    c->block_prefix = prefix_len;
    c->block_policy = pa->policy;
    c->block_dev_m = dev_m ? 1 : 0;
    c->block_n_sel = n_sel;
  }
  c->steps += 1;
  return ok();
}

}  // namespace

extern "C" {

fb_status fb_step(fb_cache* c, const fb_policy_args* pa, const void* q_blk, const void* k_blk,
                  const void* v_blk, const void* k_prefix, const void* v_prefix, int32_t prefix_len,
                  void* out, void* stream) {
  return step_impl(c, pa, nullptr, q_blk, k_blk, v_blk, k_prefix, v_prefix, prefix_len, nullptr, out, stream);
}

fb_status fb_step_ex(fb_cache* c, const fb_policy_args* pa, const fb_step_opts* opts, const void* q_blk,
                     const void* k_blk, const void* v_blk, const void* k_prefix, const void* v_prefix,
                     int32_t prefix_len, void* out, void* stream) {
  return step_impl(c, pa, opts, q_blk, k_blk, v_blk, k_prefix, v_prefix, prefix_len, nullptr, out, stream);
}

fb_status fb_step_sparse(fb_cache* c, const fb_policy_args* pa, const fb_step_opts* opts, const void* q_blk,
                         const void* k_blk, const void* v_blk, const void* k_prefix, const void* v_prefix,
                         int32_t prefix_len, const int32_t* sel_tiles, int32_t n_sel, void* out, void* stream) {
  const SparseSel sp{sel_tiles, n_sel};
  return step_impl(c, pa, opts, q_blk, k_blk, v_blk, k_prefix, v_prefix, prefix_len, &sp, out, stream);
}

fb_status fb_cache_read(const fb_cache* c, int32_t field, void* host_dst, size_t bytes, void* stream) {
  if (!c) return fail(FB_E_ARG, "cache is null");
  if (!host_dst) return fail(FB_E_ARG, "host_dst is null");
  const int64_t nh = (int64_t)c->cfg.batch * c->cfg.n_q_heads;
  const int64_t so = elems_per_slot(c->cfg), sl = rows_per_slot(c->cfg);
  size_t want;
  switch (field) {
    case FB_FIELD_A_OUT: want = so * sizeof(float); break;
    case FB_FIELD_L_OUT: want = sl * sizeof(float); break;
    case FB_FIELD_SIM: want = nh * sizeof(float); break;
    case FB_FIELD_REUSE:
    case FB_FIELD_VALID: want = nh; break;
    case FB_FIELD_WAIT_ERR: want = sizeof(uint32_t); break;
    default: return fail(FB_E_ARG, "unknown field %d", field);
  }
  if (bytes != want) return fail(FB_E_ARG, "field %d needs %zu bytes, got %zu", field, want, bytes);
  DeviceGuard g(c->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "set device");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronise");
  if (field == FB_FIELD_WAIT_ERR) {
    uint32_t v = 0;
    if (c->fin_ctr != nullptr) {
      e = hipMemcpy(&v, c->fin_ctr, sizeof v, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "copy");
    }
    std::memcpy(host_dst, &v, sizeof v);
    return ok();
  }
  const void* src = field == FB_FIELD_A_OUT   ? (const void*)c->slot_o
                    : field == FB_FIELD_L_OUT ? (const void*)c->slot_l
                    : field == FB_FIELD_SIM   ? (const void*)c->sim
                    : field == FB_FIELD_VALID ? (const void*)c->valid
                                              : (const void*)(c->reuse + ((c->steps + 1) & 1) * nh);
  e = hipMemcpy(host_dst, src, want, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "copy");
  return ok();
}

fb_status fb_cache_info(const fb_cache* c, size_t* device_bytes, int32_t* kv_splits) {
  if (!c) return fail(FB_E_ARG, "cache is null");
  if (device_bytes) *device_bytes = c->bytes;
  if (kv_splits) *kv_splits = c->splits_cap;
  return ok();
}

fb_status fb_profile_enable(fb_cache* c, int32_t enable) {
  if (!c) return fail(FB_E_ARG, "cache is null");
  c->prof = enable != 0;
  return ok();
}

fb_status fb_profile_read(fb_cache* c, fb_profile_stats* out) {
  if (!c || !out) return fail(FB_E_ARG, "null argument");
  DeviceGuard g(c->device);
  if (g.err != hipSuccess) return hip_fail(g.err, "set device");
  for (auto& r : c->prof_recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "event timing");
    c->prof_launches[r.kind] += 1;
    c->prof_ms[r.kind] += ms;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  c->prof_recs.clear();
  for (int k = 0; k < FB_PROFILE_KINDS; ++k) {
    out->launches[k] = c->prof_launches[k];
    out->ms[k] = c->prof_ms[k];
    c->prof_launches[k] = 0;
    c->prof_ms[k] = 0.0;
  }
  return ok();
}

}  // extern "C"

namespace fbk {

fb_status report(fb_status code, const char* msg) { return code == FB_OK ? ok() : fail(code, "%s", msg); }

// One always-recompute step on caller buffers, with its split partials and
// per-head flags in `scratch` (scratch_bytes): the path of fb_step under
// FB_POLICY_ALWAYS, whose cached A_out/L_out are the caller's a_out/l_out.
// The cache object lives on the stack and its tables are fixed arrays, so
// nothing is allocated, on the host or the device.
fb_status noalloc_step(const fb_config* cfg, void* scratch, size_t scratch_bytes, int n_cu, const void* q_blk,
                       const void* k_blk, const void* v_blk, const void* k_prefix, const void* v_prefix,
                       int32_t prefix_len, float* a_out, float* l_out, void* out, void* stream) {
  fb_status st = check_config(cfg);
  if (st != FB_OK) return st;
  if (!q_blk || !k_blk || !v_blk || !a_out || !l_out || !out) return fail(FB_E_ARG, "a tensor pointer is null");
  if (prefix_len < 0 || prefix_len > cfg->max_prefix)
    return fail(FB_E_SHAPE, "prefix_len %d outside [0, max_prefix=%d]", prefix_len, cfg->max_prefix);
  if (prefix_len > 0 && (!k_prefix || !v_prefix)) return fail(FB_E_ARG, "k_prefix/v_prefix is null");
  fb_cache c;
  setup_shape(&c, cfg);
  if (n_cu > 0) c.n_cu = n_cu;
  // scratch: valid and reuse flags [B*Hq] each, then the split partials, L
  // (fp32) and A (the working dtype), for as many splits as fit (the last
  // slot holds the block-internal part)
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t nh = (size_t)cfg->batch * cfg->n_q_heads;
  const size_t part_a = (size_t)elems_per_slot(*cfg) * (cfg->dtype == FB_BF16 ? 2 : 4);
  const size_t part_l = (size_t)rows_per_slot(*cfg) * sizeof(float);
  const size_t fixed = 2 * up(nh);
  const size_t per_slot = up(part_l) + up(part_a);
  if (scratch_bytes < fixed + 2 * per_slot)
    return fail(FB_E_SHAPE, "this shape needs %zu bytes of scratch with a single prefix chunk; the limit is %zu",
                fixed + 2 * per_slot, scratch_bytes);
  const int slots = (int)std::min<size_t>((scratch_bytes - fixed) / per_slot, fbk::kMaxSplits + 1);
  c.splits_cap = slots - 1;
  char* base = static_cast<char*>(scratch);
  c.valid = reinterpret_cast<uint8_t*>(base);
  c.reuse = reinterpret_cast<uint8_t*>(base + up(nh));
  c.part_l = reinterpret_cast<float*>(base + fixed);
  c.part_o = reinterpret_cast<float*>(base + fixed + (size_t)slots * up(part_l));
  c.slot_o = a_out;
  c.slot_l = l_out;
  // part_l's slots are up(part_l) apart; the strides run in elements
  c.part_l_stride_override = (int64_t)(up(part_l) / sizeof(float));
  c.part_o_stride_override = (int64_t)(up(part_a) / (cfg->dtype == FB_BF16 ? 2 : 4));
  fbk::HeadSel sel = all_heads(&c);
  ExtOpts eo;
  eo.kblk = k_blk;
  eo.vblk = v_blk;
  eo.out = out;
  eo.rec = c.reuse;
  eo.follow_rec = false;
  st = run_external(&c, q_blk, k_prefix, v_prefix, dense_keys(prefix_len), sel, cfg->batch * cfg->n_kv_heads,
                    (hipStream_t)stream, eo);
  return st == FB_OK ? ok() : st;
}

}  // namespace fbk
