// Device-side helpers shared by the gfx950 attention kernels.
//
// Page "Résumé Technique : FlashBlock", §2 "Mécanisme Central": attention of
// the current block's queries is split into a block-external part (A_out,
// L_out = log Z_out, over the committed prefix) and a block-internal part
// (A_in, L_in, over the block itself), recombined in log space with
// m = max(L_out, L_in).  The same log-space rule combines the partial results
// of the prefix chunks that different workgroups attend (split-KV).
//
// Both attention kernels compute S^T = K Q^T and O^T += V^T P^T with 32x32
// MFMAs.  In the transposed products lane l holds query row l % 32 in both
// outputs (S^T: keys 8(j/4) + 4(l/32) + j%4 of a 32-key half in register j;
// O^T: head-dim columns 32dt + 8(j/4) + 4(l/32) + j%4), so the online softmax
// and the rescale of O stay inside the lane pair (l, l^32).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fb_internal.h"

namespace fbk {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FB_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum of a value over the lane pair (l, l^32) that shares a query row.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Map the hardware index so that consecutive logical work items share an XCD.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7, x = w & 7, j = w >> 3;
  return x * q + min(x, r) + j;
}

// Touch every 64-byte line of a kernel's parameter block at once.  The
// prologue reads its parameters with scalar loads that are each waited for
// before a branch; without this they go to memory one round trip after
// another, with it they hit the scalar cache after a single one.
template <typename P>
__device__ __forceinline__ void prefetch_params(const P& p) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(&p);
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(P) / 4); i += 16) acc ^= a[i];
  asm volatile("" ::"s"(acc));
}

__device__ __forceinline__ bool head_selected(const HeadSel& s, int b, int bh) {
  if (!s.every_seq && !((s.seq_bits[b >> 5] >> (b & 31)) & 1u)) return false;
  if (s.m != nullptr) {   // threshold rule with the updated-token counts in device memory
    const int64_t upd = (int64_t)s.m[b] + (s.cum != nullptr ? s.cum[b] : 0);
    return !(s.valid[bh] != 0 && upd < s.tau);
  }
  if (s.flags == nullptr) return true;
  return (s.flags[bh] != 0) == (s.flags_select != 0);
}

// Whether any query head of group (b, g) is selected.
__device__ __forceinline__ bool group_selected(const HeadSel& s, int b, int g, int hq, int grp) {
  bool any = false;
  for (int i = 0; i < grp; ++i) any |= head_selected(s, b, b * hq + g * grp + i);
  return any;
}

// Partial launches whose heads are decided in the kernel: the first workgroup
// records 1 - selected for every head, which the launches after it select
// from (they may change what the decision reads).  Runs before any early exit.
__device__ __forceinline__ void record_decisions(const AttnParams& p) {
  if (p.reuse_rec == nullptr || blockIdx.x != 0) return;
  const int nh = p.batch * p.hq;
  for (int bh = threadIdx.x; bh < nh; bh += blockDim.x)
    p.reuse_rec[bh] = (p.rec_reuse_all || !head_selected(p.sel, bh / p.hq, bh)) ? 1 : 0;
}



// Groups (sequence, kv head) with at least one selected query head, as a bit
// mask over the group index b*Hkv + g (groups <= 64), computed by every wave
// from the head flags; and the number of splits the device plan gives them.
__device__ __forceinline__ uint64_t active_groups(const HeadSel& sel, int groups, int hq, int hkv) {
  const int lane = threadIdx.x & 63, grp = hq / hkv;
  bool act = false;
  if (lane < groups) {
    const int b = lane / hkv, g = lane % hkv;
    for (int i = 0; i < grp; ++i) act |= head_selected(sel, b, b * hq + g * grp + i);
  }
  return __builtin_amdgcn_ballot_w64(act);
}

// n / d for a grid index, with m from div_magic (0: an ordinary division).
__device__ __forceinline__ int div_index(int n, int d, uint64_t m) {
  if (m == 0) return n / d;
  return (int)(((uint64_t)(uint32_t)n * m) >> 32);
}

// Work item of an attention workgroup: (sequence, kv head, key split, row
// tile) and its key range.  Static plan: the grid enumerates every group,
// groups without a selected head exit.  Device plan: the grid enumerates the
// active groups only, with the split count chosen for their number.
struct AttnItem {
  int b, g, split, rt;
  int key_begin, key_end;
  bool ok;
  bool internal;   // a fused step's block-internal item
  bool seg2;       // an item of the launch's second key set
};
// bid: the item's index in the launch (the workgroup index, or the ticket of
// a single-launch fused step), nblocks: the launch's attention items.
// TWO_SETS = false: a kernel never launched with a second key set.
template <bool TWO_SETS = true>
__device__ __forceinline__ AttnItem attn_item(const AttnParams& p, bool partial, int bid, int nblocks) {
  AttnItem it;
  it.internal = false;
  it.seg2 = false;
  int kps = p.keys_per_split;
  const int int_count = partial ? p.int_count : 0;
  if (bid < int_count) {   // a fused step's block-internal item (they come first)
    const int w = xcd_remap(bid, int_count);
    const int w1 = div_index(w, p.row_tiles, p.dv_row_tiles);
    it.rt = w - w1 * p.row_tiles;
    it.b = div_index(w1, p.hkv, p.dv_hkv);
    it.g = w1 - it.b * p.hkv;
    it.split = p.int_split;
    it.key_begin = 0;
    it.key_end = p.bs;
    it.ok = true;
    it.internal = true;
    return it;
  }
  const int w0 = bid - int_count;   // index among the external items
  const int seg2_items = TWO_SETS && partial ? p.seg2_items : 0;
  const int n1 = nblocks - int_count - seg2_items;   // the first key set's items
  if (TWO_SETS && w0 >= n1) {   // the second key set: every group, a static plan
    int w = xcd_remap(w0 - n1, seg2_items);
    it.rt = w % p.row_tiles;
    w /= p.row_tiles;
    const int split = w % p.seg2_splits;
    w /= p.seg2_splits;
    it.b = w / p.hkv;
    it.g = w % p.hkv;
    it.key_begin = split * p.seg2_kps;
    it.key_end = min(p.n_keys2, it.key_begin + p.seg2_kps);
    it.split = p.seg2_base + split;
    it.ok = true;
    it.seg2 = true;
    return it;
  }
  if (partial && p.dyn.groups > 0) {
    const uint64_t mask = active_groups(p.sel, p.dyn.groups, p.hq, p.hkv);
    const int n = __builtin_popcountll(mask);
    const int splits = n > 0 ? p.dyn.splits[n] : 1;
    const int items = n * p.row_tiles * splits;
    it.ok = w0 < items;
    if (!it.ok) return it;
    int w = xcd_remap(w0, items);
    it.rt = w % p.row_tiles;
    w /= p.row_tiles;
    it.split = w % splits;
    int rank = w / splits;   // the rank-th active group
    uint64_t m = mask;
    for (; rank > 0; --rank) m &= m - 1;
    const int group = __builtin_ctzll(m);
    it.b = group / p.hkv;
    it.g = group % p.hkv;
    const int tiles = (p.n_keys + kKeyTile - 1) / kKeyTile;
    kps = ((tiles + splits - 1) / splits) * kKeyTile;
  } else {
    int w = xcd_remap(w0, n1);
    int q = div_index(w, p.row_tiles, p.dv_row_tiles);
    it.rt = w - q * p.row_tiles;
    w = q;
    if (partial) {
      q = div_index(w, p.splits, p.dv_splits);
      it.split = w - q * p.splits;
      w = q;
    } else {
      it.split = 0;   // merge launches run one key range per group
    }
    it.b = div_index(w, p.hkv, p.dv_hkv);
    it.g = w - it.b * p.hkv;
    it.ok = true;
    if (partial) {
      bool any;
      if (p.sel.m == nullptr && p.sel.flags == nullptr) {
        // decided per sequence (the host's threshold decisions): no head loop
        any = p.sel.every_seq || ((p.sel.seq_bits[it.b >> 5] >> (it.b & 31)) & 1u);
      } else {
        any = group_selected(p.sel, it.b, it.g, p.hq, p.grp);
      }
      it.ok = any;
    }
  }
  it.key_begin = it.split * kps;
  it.key_end = min(p.n_keys, it.key_begin + kps);
  return it;
}

template <bool TWO_SETS = true>
__device__ __forceinline__ AttnItem attn_item(const AttnParams& p, bool partial) {
  return attn_item<TWO_SETS>(p, partial, (int)blockIdx.x, (int)gridDim.x);
}

// Work item of a merge launch on a 3-D grid (x: row tile, y: kv head, z:
// sequence): one key range, the whole of the block's keys; no division.
__device__ __forceinline__ AttnItem grid_item(const AttnParams& p) {
  AttnItem it;
  it.internal = false;
  it.seg2 = false;
  it.rt = blockIdx.x;
  it.g = blockIdx.y;
  it.b = blockIdx.z;
  it.split = 0;
  it.key_begin = 0;
  it.key_end = p.n_keys;
  it.ok = true;
  return it;
}

// Key tiles of a work item.  Contiguous range: tile v starts at key
// key_begin + 64v and keys at or past key_end (the range's end) hold no key.
// Tile list: tile v starts at key 64 * list[v] (the item's part of its group's
// list); keys at or past n_phys hold no key, and an entry outside the
// prefix's tiles maps to a tile with none (its loads stay in bounds).
// MAYBE_LIST = false compiles the contiguous form only.
template <bool MAYBE_LIST>
struct TileMap {
  const int32_t* list;
  int key_begin;
  int lim;          // first key that holds no key
  int phys_tiles;
  __device__ __forceinline__ int key0(int v) const {
    if (!MAYBE_LIST || list == nullptr) return key_begin + v * kKeyTile;
    const int t = load_scalar(list + v);
    return (t >= 0 && t < phys_tiles) ? t * kKeyTile : lim;
  }
  // A wave-uniform list entry through the scalar data path: a vector load
  // here would make the compiler wait for every vector memory operation in
  // flight (the K/V ring's DMA loads included) before the entry is used.
  // The list is written by an earlier launch, so the scalar cache holds no
  // stale copy.
  __device__ __forceinline__ static int load_scalar(const int32_t* ptr) {
    const uint64_t a = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const auto cp = (const __attribute__((address_space(4))) int32_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return *cp;
  }
};
template <bool MAYBE_LIST>
__device__ __forceinline__ TileMap<MAYBE_LIST> tile_map(const AttnParams& p, const AttnItem& it) {
  TileMap<MAYBE_LIST> m;
  const int b = it.b, g = it.g, key_begin = it.key_begin, key_end = it.key_end;
  const int32_t* tiles = it.seg2 ? p.tiles2 : p.tiles;
  if (!MAYBE_LIST || tiles == nullptr || it.internal) {
    m.list = nullptr;
    m.key_begin = key_begin;
    m.lim = key_end;
    m.phys_tiles = 0;
  } else {
    m.list = tiles + ((int64_t)b * p.hkv + g) * (it.seg2 ? p.tiles2_stride : p.tiles_stride) + key_begin / kKeyTile;
    m.key_begin = 0;
    m.lim = p.n_phys;
    m.phys_tiles = (p.n_phys + kKeyTile - 1) / kKeyTile;
  }
  return m;
}

// Online-softmax update of NH 32-key halves of S^T (raw scores) whose first
// key is key0.  c = softmax scale * log2(e) > 0, so the max of the raw scores
// gives the max of the scaled ones and P = exp2(c*s - m) takes one FMA per
// score.  The running max m (log2 units) is only raised when a row's tile max
// exceeds it by more than kRescale; until then P <= 2^kRescale, and the O/sum
// rescale (rarely needed after the first tile) runs only when some row of the
// wave raised its max.  The result is the same: the final normalisation
// divides by the sum taken against the same m.  MASKED drops keys at or past
// key_end (a row may then have seen no key yet: m stays -inf, P = 0).
constexpr float kRescale = 8.0f;

template <int kDt, int NH, bool MASKED>
__device__ __forceinline__ void softmax_halves(f32x16 (&s)[NH], f32x16 (&o)[kDt], float& m, float& lsum,
                                               int key0, int key_end, int hl, float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (MASKED) {
        const int key = key0 + 32 * h + 8 * (j >> 2) + 4 * hl + (j & 3);
        s[h][j] = key < key_end ? s[h][j] : -INFINITY;
      }
      mx = fmaxf(mx, s[h][j]);
    }
  }
  mx = pair_max(mx) * c;
  const bool raise = mx > m + kRescale;
  if (__builtin_amdgcn_ballot_w64(raise) != 0) {
    const float m_new = raise ? mx : m;
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < kDt; ++i) o[i] *= alpha;
  }
  const float mref = MASKED ? (m > -INFINITY ? m : 0.0f) : m;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e = fast_exp2(fmaf(s[h][j], c, -mref));
      s[h][j] = e;
      lsum += e;
    }
  }
}

template <int kDt, int NH>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[NH], f32x16 (&o)[kDt], float& m, float& lsum,
                                             int key0, int key_end, int hl, float c) {
  if (key0 + 32 * NH <= key_end) softmax_halves<kDt, NH, false>(s, o, m, lsum, key0, key_end, hl, c);
  else softmax_halves<kDt, NH, true>(s, o, m, lsum, key0, key_end, hl, c);
}

// Epilogue of a partial (one key split): normalised A and natural-log L.
template <int D>
__device__ __forceinline__ void store_partial(const AttnParams& p, const f32x16 (&o)[D / 32], float m,
                                              float ltot, int split, int64_t grow, int hl) {
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  const float lse = ltot > 0.0f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  float* od = p.part_o + split * p.part_o_stride + grow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 v4 = {o[dt][4 * gq] * inv, o[dt][4 * gq + 1] * inv, o[dt][4 * gq + 2] * inv,
                        o[dt][4 * gq + 3] * inv};
      *reinterpret_cast<f32x4*>(od + 32 * dt + 8 * gq + 4 * hl) = v4;
    }
  }
  if (hl == 0) p.part_l[split * p.part_l_stride + grow] = lse;
}

// External part of one row for the merge: the head's cached A_out columns of
// this lane (16 float4 for D=128) and L_out; an empty part when the head holds
// nothing.  The flag and the data are independent loads (the cache is always
// allocated), so both can be in flight at once.  The flag is kept as the
// loaded byte and tested only at the merge: converting it at once makes the
// compiler wait for the load before anything else is issued.
template <int D>
struct ExtPart {
  f32x4 a[D / 8];
  float l;
  uint32_t valid;
  __device__ __forceinline__ void load_state(const AttnParams& p, int bh) { valid = p.valid[bh]; }
  __device__ __forceinline__ void load_data(const AttnParams& p, int64_t grow, int hl) {
    l = p.slot_l[grow];
    const float* ao = p.slot_o + grow * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) a[4 * dt + gq] = *reinterpret_cast<const f32x4*>(ao + 32 * dt + 8 * gq + 4 * hl);
    }
  }
  __device__ __forceinline__ void load(const AttnParams& p, int bh, int64_t grow, int hl) {
    load_state(p, bh);
    load_data(p, grow, hl);
  }
};

// Epilogue of the block-internal attention: log-space merge with the external
// part (page §2, A_full equation) and store in the output dtype.
template <typename T, int D>
__device__ __forceinline__ void merge_store(const AttnParams& p, const f32x16 (&o)[D / 32], float m, float ltot,
                                            const ExtPart<D>& ext, int64_t grow, int hl) {
  const float l_in = (m + log2f(ltot)) * kLn2;
  uint32_t valid = ext.valid;
  asm volatile("" : "+v"(valid));   // keeps the test (and its wait for the load) here
  const bool has = valid != 0;
  const float l_out = has ? ext.l : -INFINITY;
  const float mm = fmaxf(l_out, l_in);
  const float w_out = fast_exp2((l_out - mm) * kLog2e);
  const float w_in = fast_exp2((l_in - mm) * kLog2e);
  const float inv_den = 1.0f / (w_out + w_in);
  const float c_in = w_in / ltot * inv_den, c_out = w_out * inv_den;
  T* od = reinterpret_cast<T*>(p.out) + grow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = 32 * dt + 8 * gq + 4 * hl;
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a_out = has ? ext.a[4 * dt + gq][e] : 0.0f;   // an empty cache may hold anything
        r[e] = c_out * a_out + c_in * o[dt][4 * gq + e];
      }
      if constexpr (sizeof(T) == 2) {
        bf16x4 rb = {(bf16)r[0], (bf16)r[1], (bf16)r[2], (bf16)r[3]};
        *reinterpret_cast<bf16x4*>(od + d0) = rb;
      } else {
        *reinterpret_cast<f32x4*>(od + d0) = r;
      }
    }
  }
}

// Launchers of the attention kernel families: fp32, bf16 (32 rows per wave),
// and bf16 with 64 rows per wave (partial launches of 256-row groups, D=128).
hipError_t launch_attn_f32(int head_dim, int mode, const AttnParams& p, hipStream_t s);
hipError_t launch_attn_bf16(int head_dim, int mode, const AttnParams& p, hipStream_t s);
hipError_t launch_attn_r64(const AttnParams& p, hipStream_t s);

}  // namespace fbk
