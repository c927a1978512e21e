// Split combine shared by the combine kernel and the single-launch fused
// step (gfx950): the fold of the split partials of a wave's rows into the
// cache, the similarity terms and the step's output.
#pragma once

#include <type_traits>

#include "fb_device.h"

namespace fbk {

namespace {

// Split combine (page §2's log-space rule over the prefix chunks):
// A = sum_s e^{L_s - M} A_s / sum_s e^{L_s - M}, L = M + log sum, M = max_s L_s.
// One wave per workgroup, D/4 lanes (one float4 column each) per row.  The
// splits are folded in a fixed order, BATCH (8, 16 or 32, from the largest
// split count the launch can see) at a time with all their loads in flight,
// keeping a running max (an online form of the same sum).  Under
// gamma, before replacing each cached value it sums <A_new, A_old>, |A_new|^2
// and |A_old|^2 over its rows for the similarity.  In total mode (sparse attention: the
// splits are the kept keys) the fold starts from the head's cached part and
// the result goes to the total buffer.  With two key sets (a sparse step in
// which some head recomputes) a selected head's splits of the first set
// (the left-out keys) refresh its cache, and then every head folds the
// second set's splits (the kept keys) onto its cached part.
// One float4 column of a partial A: fp32, or bf16 widened.
template <bool PB>
__device__ __forceinline__ f32x4 load_part(const float* base, int64_t off) {
  if constexpr (PB) {
    const bf16x4 t = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(base) + off);
    return f32x4{(float)t[0], (float)t[1], (float)t[2], (float)t[3]};
  } else {
    return *reinterpret_cast<const f32x4*>(base + off);
  }
}
// The same column as loaded, widened later by widen_part: a load that is to
// stay in flight must not be converted at once (the conversion waits for it).
template <bool PB>
using PartRaw = std::conditional_t<PB, bf16x4, f32x4>;
// COH: a device-coherent relaxed atomic load (the partials of the same
// launch, single-launch step; bf16 partials only).
template <bool PB, bool COH = false>
__device__ __forceinline__ PartRaw<PB> load_part_raw(const float* base, int64_t off) {
  static_assert(PB || !COH, "coherent partial loads are 8-byte bf16 columns");
  if constexpr (COH) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(reinterpret_cast<const bf16*>(base) + off),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_bit_cast(bf16x4, v);
  } else if constexpr (PB) {
    return *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(base) + off);
  } else {
    return *reinterpret_cast<const f32x4*>(base + off);
  }
}
template <bool COH>
__device__ __forceinline__ float load_l(const float* a) {
  if constexpr (COH) return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *a;
}
template <bool PB>
__device__ __forceinline__ f32x4 widen_part(const PartRaw<PB>& t) {
  if constexpr (PB) return f32x4{(float)t[0], (float)t[1], (float)t[2], (float)t[3]};
  else return t;
}

// Reductions and broadcasts inside a group of W = 16 or 32 consecutive lanes
// (one combine row), on the vector ALUs: DPP rotations within a 16-lane row
// (each step adds the same pair of values in both lanes, so every lane of
// the group ends with the bitwise-same result) and, for 32 lanes, a swap of
// the two rows.  A shuffle through the LDS unit would wait out its latency
// at every step.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}
template <int W>
__device__ __forceinline__ float group_max(float x) {
  static_assert(W == 16 || W == 32, "a combine row is 16 or 32 lanes");
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  x = fmaxf(x, row_ror<1>(x));
  if constexpr (W == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 16 || W == 32, "a combine row is 16 or 32 lanes");
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  if constexpr (W == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}
// Sum over the whole wave (every lane gets the same value): the 32-lane
// groups, then the two halves swapped and added.
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<32>(x);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value of lane j (wave-uniform) of this lane's W-lane group: read from every
// group of the wave with v_readlane and the lane's own group selected.
template <int W>
__device__ __forceinline__ float group_bcast(float x, int j, int group) {
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
#pragma unroll
  for (int g = 1; g < 64 / W; ++g) {
    const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), g * W + j));
    v = group == g ? o : v;
  }
  return v;
}

// The fold of one wave (tid = lane 0..63): rows ch * kRows .. of head bh
// (sequence b).
template <int D, int BATCH, bool PB, bool COH = false>
__device__ __forceinline__ void combine_fold(const CombineParams& p, int ch, int bh, int b, int tid) {
  constexpr int kLpr = D / 4;
  constexpr int kRows = kCombineThreads / kLpr;
  const bool out_mode = p.out != nullptr;
  const bool sel = head_selected(p.sel, b, bh);
  const bool two = p.two_sets != 0;
  if (p.cum != nullptr && bh % p.hq == 0 && ch == 0 && tid == 0) {   // once per sequence
    bool any = false;
    for (int h = 0; h < p.hq; ++h) any |= head_selected(p.sel, b, b * p.hq + h);
    p.cum[b] = any ? 0 : p.cum[b] + p.cum_m[b];
  }
  if (!sel && !out_mode) return;
  int splits = sel ? p.splits : 0;
  if (sel && p.dyn.groups > 0) {   // the external launch's device plan
    const int n = __builtin_popcountll(active_groups(p.sel, p.dyn.groups, p.hq, p.hkv));
    splits = p.dyn.splits[n];
  }
  const bool sim_terms = sel && p.sim_terms && p.valid[bh] != 0;
  const bool tot = p.tot_o != nullptr;
  const int c4 = tid % kLpr;
  const int i = ch * kRows + tid / kLpr;
  float dot = 0.0f, nn = 0.0f, no = 0.0f;
  if (i < p.bs) {
    const int64_t grow = (int64_t)bh * p.bs + i;
    const float* lp = p.part_l + grow;
    const int64_t ao = grow * D + 4 * c4;   // element offset of this lane's column
    float mx = -INFINITY, wsum = 0.0f;
    f32x4 acc = {0, 0, 0, 0};
    // the cached part enters as one more term, normalised (weight 1 at its
    // max): in total mode, and for the output of a head that reuses it
    if ((two ? !sel : (tot || !sel)) && p.valid[bh] != 0) {
      const float l0 = p.slot_l[grow];
      if (l0 > -INFINITY) {
        mx = l0;
        wsum = 1.0f;
        acc = *reinterpret_cast<const f32x4*>(p.slot_o + grow * D + 4 * c4);
      }
    }
    // A fused step's block-internal part, loaded before the rounds so that
    // it arrives with them instead of one memory round trip after the fold.
    float l_in = -INFINITY;
    PartRaw<PB> a_in_raw{};
    if (out_mode) {
      l_in = load_l<COH>(lp + p.int_split * p.part_l_stride);
      a_in_raw = load_part_raw<PB, COH>(p.part_o, ao + p.int_split * p.part_o_stride);
    }
    // BATCH splits per round, all their loads in flight; past the last split
    // a round re-reads it and gives it no weight (L = -inf).  The round's L
    // values are spread over the row's lanes (lane c4 holds split s + c4, and
    // s + c4 + kLpr, ...): one load per kLpr splits instead of one per split
    // (a wave keeps at most 63 loads in flight), one exponential per split;
    // the row max and weight sum are taken across the row's lanes and each
    // weight is read from the lane that holds it (vector-ALU cross-lane
    // operations, see group_max).  Every lane still adds the
    // splits' A in split order.
    constexpr int kLl = (BATCH + kLpr - 1) / kLpr;   // L values per lane and round
    // the splits first .. first + count - 1, folded into (mx, wsum, acc)
    auto fold = [&](int first, int count) {
    for (int s = 0; s < count; s += BATCH) {
      float lv[kLl];
      PartRaw<PB> a[BATCH];   // widened where used: a conversion here would wait for its load
#pragma unroll
      for (int k = 0; k < kLl; ++k) {
        const int u = c4 + kLpr * k;
        const int si = first + min(s + u, count - 1);
        lv[k] = load_l<COH>(lp + si * p.part_l_stride);
        if (u >= BATCH || s + u >= count) lv[k] = -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int si = first + min(s + u, count - 1);
        a[u] = load_part_raw<PB, COH>(p.part_o, ao + si * p.part_o_stride);
      }
      // keep every load of the round ahead of the arithmetic: left to itself
      // the scheduler trades the in-flight loads for registers and waits on
      // a few at a time
      __builtin_amdgcn_sched_barrier(0);
      float cm = lv[0];
#pragma unroll
      for (int k = 1; k < kLl; ++k) cm = fmaxf(cm, lv[k]);
      cm = group_max<kLpr>(cm);
      const float nm = fmaxf(mx, cm);
      if (nm > -INFINITY) {
        const float sc = fast_exp2((mx - nm) * kLog2e);
        acc *= sc;
        wsum *= sc;
        float wv[kLl];
        float ws = 0.0f;
#pragma unroll
        for (int k = 0; k < kLl; ++k) {
          wv[k] = fast_exp2((lv[k] - nm) * kLog2e);
          ws += wv[k];
        }
        wsum += group_sum<kLpr>(ws);
        const int grp_w = (tid & 63) / kLpr;   // this lane's row within the wave
#pragma unroll
        for (int u = 0; u < BATCH; ++u) acc += group_bcast<kLpr>(wv[u / kLpr], u % kLpr, grp_w) * widen_part<PB>(a[u]);
        mx = nm;
      }
    }
    };
    fold(0, splits);
    if (sel && !(tot && out_mode)) {   // a recomputed head's new value: into the cache (total mode: the buffer)
      const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
      const f32x4 a_new = acc * inv;
      const float lse = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
      if (sim_terms) {
        const f32x4 a_old = *reinterpret_cast<const f32x4*>(p.slot_o + grow * D + 4 * c4);   // replaced below
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dot += a_new[e] * a_old[e];
          nn += a_new[e] * a_new[e];
          no += a_old[e] * a_old[e];
        }
      }
      float* od = (tot ? p.tot_o : p.slot_o) + grow * D;
      float* ld = (tot ? p.tot_l : p.slot_l) + grow;
      *reinterpret_cast<f32x4*>(od + 4 * c4) = a_new;
      if (c4 == 0) *ld = lse;
      if (two) {   // the total starts from the cached part just stored, as a read of it would
        const bool has = lse > -INFINITY;
        mx = has ? lse : -INFINITY;
        wsum = has ? 1.0f : 0.0f;
        acc = has ? a_new : f32x4{0, 0, 0, 0};
      }
    }
    if (two) fold(p.base2, p.splits2);   // the second key set (kept keys), every head
    if (out_mode) {   // the block-internal part (page §2 merge), then the step's output
      const f32x4 a_in = widen_part<PB>(a_in_raw);
      const float nm = fmaxf(mx, l_in);
      if (nm > -INFINITY) {
        const float sc = fast_exp2((mx - nm) * kLog2e);
        const float w = fast_exp2((l_in - nm) * kLog2e);
        acc = acc * sc + w * a_in;
        wsum = wsum * sc + w;
      }
      const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
      const f32x4 r = acc * inv;
      if (p.out_bf16) {
        const bf16x4 rb = {(bf16)r[0], (bf16)r[1], (bf16)r[2], (bf16)r[3]};
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(p.out) + grow * D + 4 * c4) = rb;
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + grow * D + 4 * c4) = r;
      }
    }
  }
  if (sim_terms) {
    dot = wave_sum(dot);
    nn = wave_sum(nn);
    no = wave_sum(no);
    if (tid == 0) {
      float* t = p.cos_part + ((int64_t)bh * p.row_chunks + ch) * 3;
      t[0] = dot;
      t[1] = nn;
      t[2] = no;
    }
  }
  if (sel && !p.sim_terms && !tot && !p.keep_valid && ch == 0 && tid == 0) p.valid[bh] = 1;
}

}  // namespace

}  // namespace fbk
