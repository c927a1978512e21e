// Split combine, gamma decision and reset kernels (gfx950), and the attention
// dispatcher.
#include <algorithm>
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
// the result goes to the total buffer.
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
template <bool PB>
__device__ __forceinline__ PartRaw<PB> load_part_raw(const float* base, int64_t off) {
  if constexpr (PB) return *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(base) + off);
  else return *reinterpret_cast<const f32x4*>(base + off);
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

template <int D, int BATCH, bool PB>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const CombineParams p) {
  constexpr int kLpr = D / 4;
  constexpr int kRows = kCombineThreads / kLpr;
  prefetch_params(p);
  const int tid = threadIdx.x;
  // 3-D grid (row chunk, query head, sequence): no division
  const int ch = blockIdx.x, b = blockIdx.z;
  const int bh = b * p.hq + blockIdx.y;
  const bool out_mode = p.out != nullptr;
  const bool sel = head_selected(p.sel, b, bh);
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
    if ((tot || !sel) && p.valid[bh] != 0) {
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
      l_in = lp[p.int_split * p.part_l_stride];
      a_in_raw = load_part_raw<PB>(p.part_o, ao + p.int_split * p.part_o_stride);
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
    for (int s = 0; s < splits; s += BATCH) {
      float lv[kLl];
      PartRaw<PB> a[BATCH];   // widened where used: a conversion here would wait for its load
#pragma unroll
      for (int k = 0; k < kLl; ++k) {
        const int u = c4 + kLpr * k;
        const int si = min(s + u, splits - 1);
        lv[k] = lp[si * p.part_l_stride];
        if (u >= BATCH || s + u >= splits) lv[k] = -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int si = min(s + u, splits - 1);
        a[u] = load_part_raw<PB>(p.part_o, ao + si * p.part_o_stride);
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
    }
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
  if (sel && !p.sim_terms && !tot && ch == 0 && tid == 0) p.valid[bh] = 1;
}

// Gamma decisions, one workgroup per head: similarity of a recomputed head
// (or of its kv group: the same terms summed over the group's heads) from the
// combine's partial terms (summed in a fixed order), the head's valid flag,
// and the reuse decision of the next step (strict sim > gamma; NaN, i.e. no
// similarity yet, never reuses).
__global__ __launch_bounds__(kThreads) void decide_kernel(const DecideParams p) {
  __shared__ float red[3][kThreads / 64];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const bool computed = p.reuse_now[bh] == 0;
  const bool had_value = p.valid[bh] != 0;
  __syncthreads();   // every thread has read the flags before thread 0 updates them
  if (computed && had_value) {   // workgroup-uniform
    float dot = 0.0f, nn = 0.0f, no = 0.0f;
    // the terms of the head, or of every head of its group (in head order,
    // so that the heads of a group obtain the same sum)
    const int h0 = bh - (bh % p.hq) % p.group;
    const int terms = p.group * p.row_chunks;
    for (int c = tid; c < terms; c += kThreads) {
      const float* t = p.cos_part + ((int64_t)h0 * p.row_chunks + c) * 3;
      dot += t[0];
      nn += t[1];
      no += t[2];
    }
    dot = wave_sum(dot);
    nn = wave_sum(nn);
    no = wave_sum(no);
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = dot;
      red[1][tid >> 6] = nn;
      red[2][tid >> 6] = no;
    }
    __syncthreads();
    if (tid == 0) {
      dot = red[0][0] + red[0][1] + red[0][2] + red[0][3];
      nn = red[1][0] + red[1][1] + red[1][2] + red[1][3];
      no = red[2][0] + red[2][1] + red[2][2] + red[2][3];
      float sim;
      if (nn == 0.0f || no == 0.0f) sim = (nn == 0.0f && no == 0.0f) ? 1.0f : 0.0f;
      else sim = fminf(1.0f, fmaxf(-1.0f, dot / (sqrtf(nn) * sqrtf(no))));
      p.sim[bh] = sim;
    }
  }
  if (tid == 0) {
    if (computed) p.valid[bh] = 1;
    const float s = p.sim[bh];
    p.reuse_next[bh] = (p.valid[bh] && s > p.gamma) ? 1 : 0;
  }
}

// Per-head decisions made on the host, recorded for a step that launches no
// attention over them: 1 - selected.
__global__ __launch_bounds__(kThreads) void record_kernel(const HeadSel sel, uint8_t* rec, int n_heads, int hq) {
  const int bh = blockIdx.x * kThreads + threadIdx.x;
  if (bh < n_heads) rec[bh] = head_selected(sel, bh / hq, bh) ? 0 : 1;
}

__global__ __launch_bounds__(kThreads) void reset_kernel(const ResetParams p) {
  const int bh = blockIdx.x * kThreads + threadIdx.x;
  if (bh >= p.n_heads) return;
  p.valid[bh] = 0;
  p.reuse[bh] = 0;
  p.reuse[p.n_heads + bh] = 0;
  p.sim[bh] = __builtin_nanf("");
  if (p.cum != nullptr && bh < p.batch) p.cum[bh] = 0;
}

// Tile list of the prefix keys a sparse selection leaves out, one workgroup
// per (sequence, kv head): the selected tiles are marked in an LDS bitmap,
// then the unmarked tiles of [0, tiles) are written in ascending order (a
// workgroup-wide prefix count per 256 tiles) and the list is padded with -1
// (no key) to `stride` entries.  Entries of sel outside [0, tiles) mark
// nothing.
__global__ __launch_bounds__(kThreads) void complement_kernel(const ComplementParams p) {
  extern __shared__ uint32_t bits[];
  __shared__ int wave_cnt[kThreads / 64];
  const int grp = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = (p.tiles + 31) / 32;
  for (int i = tid; i < words; i += kThreads) bits[i] = 0u;
  __syncthreads();
  const int32_t* sel = p.sel + (int64_t)grp * p.n_sel;
  for (int i = tid; i < p.n_sel; i += kThreads) {
    const int t = sel[i];
    if (t >= 0 && t < p.tiles) atomicOr(&bits[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  int32_t* out = p.comp + (int64_t)grp * p.stride;
  int base = 0;
  for (int t0 = 0; t0 < p.tiles; t0 += kThreads) {
    const int t = t0 + tid;
    const bool left = t < p.tiles && ((bits[t >> 5] >> (t & 31)) & 1u) == 0u;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(left);
    if (lane == 0) wave_cnt[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = base, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      off += w < wave ? wave_cnt[w] : 0;
      total += wave_cnt[w];
    }
    if (left) out[off + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = t;   // < tiles <= stride
    base += total;
    __syncthreads();   // wave_cnt is rewritten next round
  }
  for (int i = base + tid; i < p.stride; i += kThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_complement(const ComplementParams& p, hipStream_t s) {
  if (p.groups == 0) return hipSuccess;
  const size_t lds = (size_t)((p.tiles + 31) / 32) * 4;
  hipLaunchKernelGGL(complement_kernel, dim3(p.groups), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, int head_dim, int mode, const AttnParams& p, hipStream_t s) {
  return dtype == FB_BF16 ? launch_attn_bf16(head_dim, mode, p, s) : launch_attn_f32(head_dim, mode, p, s);
}

template <int D, bool PB>
hipError_t launch_combine_batch(int most, dim3 grid, const CombineParams& p, hipStream_t s);

hipError_t launch_combine(int head_dim, const CombineParams& p, hipStream_t s) {
  if (p.batch * p.hq * p.row_chunks == 0) return hipSuccess;
  if (p.hq > 65535 || p.batch > 65535) return hipErrorInvalidValue;   // grid y / z limits
  const dim3 blocks(p.row_chunks, p.hq, p.batch);   // launch order = (sequence, head, chunk)
  // one memory round trip per BATCH splits: the smallest batch that holds the
  // largest split count this launch can see (the device plan's too)
  int most = p.splits;
  for (int n = 1; n <= p.dyn.groups; ++n) most = std::max(most, (int)p.dyn.splits[n]);
  if (p.part_bf16) {
    if (head_dim == 64) return launch_combine_batch<64, true>(most, blocks, p, s);
    return launch_combine_batch<128, true>(most, blocks, p, s);
  }
  if (head_dim == 64) return launch_combine_batch<64, false>(most, blocks, p, s);
  return launch_combine_batch<128, false>(most, blocks, p, s);
}

template <int D, bool PB>
hipError_t launch_combine_batch(int most, dim3 blocks, const CombineParams& p, hipStream_t s) {
  if (most <= 8) hipLaunchKernelGGL((combine_kernel<D, 8, PB>), blocks, dim3(kCombineThreads), 0, s, p);
  else if (most <= 16) hipLaunchKernelGGL((combine_kernel<D, 16, PB>), blocks, dim3(kCombineThreads), 0, s, p);
  else hipLaunchKernelGGL((combine_kernel<D, 32, PB>), blocks, dim3(kCombineThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decide(const DecideParams& p, hipStream_t s) {
  hipLaunchKernelGGL(decide_kernel, dim3(p.n_heads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_record(const HeadSel& sel, uint8_t* rec, int n_heads, int hq, hipStream_t s) {
  hipLaunchKernelGGL(record_kernel, dim3((n_heads + kThreads - 1) / kThreads), dim3(kThreads), 0, s, sel, rec, n_heads,
                     hq);
  return hipGetLastError();
}

hipError_t launch_reset(const ResetParams& p, hipStream_t s) {
  hipLaunchKernelGGL(reset_kernel, dim3((p.n_heads + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fbk
