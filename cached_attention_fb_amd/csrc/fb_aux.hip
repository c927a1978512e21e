// Split combine, gamma decision and reset kernels (gfx950), and the attention
// dispatcher.
#include <algorithm>
#include <type_traits>

#include "fb_combine.h"
#include "fb_device.h"

namespace fbk {

namespace {

// 3-D grid (row chunk, query head, sequence): no division.
template <int D, int BATCH, bool PB>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const CombineParams p) {
  prefetch_params(p);
  combine_fold<D, BATCH, PB>(p, blockIdx.x, blockIdx.z * p.hq + blockIdx.y, blockIdx.z, threadIdx.x);
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

__global__ __launch_bounds__(kThreads) void reset_kernel(const ResetParams p) {
  const int bh = blockIdx.x * kThreads + threadIdx.x;
  if (p.fin_ctr != nullptr && bh < p.fin_n) p.fin_ctr[bh] = 0;
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
  if (p.two_sets) most = std::max(most, (int)p.splits2);
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

hipError_t launch_reset(const ResetParams& p, hipStream_t s) {
  const int n = std::max(p.n_heads, p.fin_ctr != nullptr ? p.fin_n : 0);
  hipLaunchKernelGGL(reset_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fbk
