// fp32 attention kernel (gfx950): 4 wave64 per workgroup, 32 packed query
// rows per wave, 64-key K/V tiles staged through registers into LDS (K with
// one padding float per row, V row-major), S^T = K Q^T and O^T += V^T P^T with
// v_mfma_f32_32x32x2_f32.  Products and sums stay in fp32 throughout.
#include "fb_device.h"

namespace fbk {

namespace {

constexpr int kF32Waves = 4;

template <int D>
struct F32Tile {
  static constexpr int kUnits = kKeyTile * D / 4 / kThreads;   // float4 per thread per tensor
  f32x4 kreg[kUnits];
  f32x4 vreg[kUnits];

  __device__ __forceinline__ void load(const float* kb, const float* vb, int tile0, int key_end, int tid) {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const int u = i * kThreads + tid, key = u / (D / 4), c = u % (D / 4);
      const int gk = tile0 + key;
      const bool ok = gk < key_end;
      kreg[i] = ok ? *reinterpret_cast<const f32x4*>(kb + (int64_t)gk * D + c * 4) : f32x4{0, 0, 0, 0};
      vreg[i] = ok ? *reinterpret_cast<const f32x4*>(vb + (int64_t)gk * D + c * 4) : f32x4{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(float* ks, float* vs, int tid) {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const int u = i * kThreads + tid, key = u / (D / 4), c = u % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) ks[key * (D + 1) + c * 4 + e] = kreg[i][e];
      *reinterpret_cast<f32x4*>(vs + key * D + c * 4) = vreg[i];
    }
  }
};

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(const AttnParams p) {
  constexpr int kDt = D / 32;
  __shared__ float sk[kKeyTile * (D + 1)];
  __shared__ float sv[kKeyTile * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane & 31, hl = lane >> 5;
  const AttnItem it = attn_item(p, MODE == kModePartial);
  if constexpr (MODE == kModePartial) record_decisions(p);
  if (!it.ok) return;   // workgroup-uniform: no selected head, or past the device plan's items
  const int b = it.b, g = it.g, grp = p.grp;
  const int key_begin = it.key_begin, key_end = it.key_end;
  const int row0 = it.rt * kF32Waves * 32 + wave * 32;
  const int row = row0 + rl;
  const bool row_ok = row < p.rows;
  const bool wave_live = row0 < p.rows;
  const int64_t grow = (int64_t)(b * p.hq + g * grp) * p.bs + row;

  const float* qg = reinterpret_cast<const float*>(p.q);
  const int64_t kv_cap = it.internal ? p.bs : p.kv_cap;
  const float* kb = reinterpret_cast<const float*>(it.internal ? p.kblk : p.k) + ((int64_t)b * p.hkv + g) * kv_cap * D;
  const float* vb = reinterpret_cast<const float*>(it.internal ? p.vblk : p.v) + ((int64_t)b * p.hkv + g) * kv_cap * D;

  // Q^T as the B operand: lane (row, hl) holds Q[row][2t + hl].
  float qf[D / 2];
#pragma unroll
  for (int t = 0; t < D / 2; ++t) qf[t] = row_ok ? qg[grow * D + 2 * t + hl] : 0.0f;

  f32x16 o[kDt];
#pragma unroll
  for (int i = 0; i < kDt; ++i) o[i] = f32x16{};
  float m = -INFINITY, lsum = 0.0f;

  const TileMap<true> tm = tile_map<true>(p, it);
  const int ntiles = key_end > key_begin ? (key_end - key_begin + kKeyTile - 1) / kKeyTile : 0;
  F32Tile<D> stage;
  if (ntiles > 0) stage.load(kb, vb, tm.key0(0), tm.lim, tid);
  for (int t_i = 0; t_i < ntiles; ++t_i) {
    const int tile0 = tm.key0(t_i);
    __syncthreads();
    stage.store(sk, sv, tid);
    __syncthreads();
    if (t_i + 1 < ntiles) stage.load(kb, vb, tm.key0(t_i + 1), tm.lim, tid);
    if (!wave_live) continue;
    f32x16 s[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      s[c] = f32x16{};
      const int key = 32 * c + rl;
#pragma unroll
      for (int t = 0; t < D / 2; ++t)
        s[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(sk[key * (D + 1) + 2 * t + hl], qf[t], s[c], 0, 0, 0);
    }
    softmax_tile<kDt, 2>(s, o, m, lsum, tile0, tm.lim, hl, p.scale_log2);
    // k-step u takes key 32c + 8(j/4) + 4hl + j%4 (c = u/16, j = u%16) from both operands
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int c = u >> 4, j = u & 15;
      const int key = 32 * c + 8 * (j >> 2) + 4 * hl + (j & 3);
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sv[key * D + 32 * dt + rl], s[c][j], o[dt], 0, 0, 0);
    }
  }

  const float ltot = pair_sum(lsum);
  if (!row_ok) return;
  if constexpr (MODE == kModePartial) {
    store_partial<D>(p, o, m, ltot, it.split, grow, hl);
  } else {
    const int bh = b * p.hq + g * grp + row / p.bs;
    ExtPart<D> ext;
    ext.load(p, bh, grow, hl);
    merge_store<float, D>(p, o, m, ltot, ext, grow, hl);
    // the decision record last, so that the merge's wait for the cached
    // part's loads does not also wait for this store
    if (p.reuse_rec != nullptr && hl == 0 && (row % p.bs) == 0) p.reuse_rec[bh] = head_selected(p.sel, b, bh) ? 0 : 1;
  }
}

template <int D>
hipError_t launch_d(int mode, const AttnParams& p, hipStream_t s) {
  const int blocks = p.grid > 0 ? p.grid : p.batch * p.hkv * p.splits * p.row_tiles;
  if (blocks == 0) return hipSuccess;
  const AttnParams q = with_div_magic(p, blocks);
  if (mode == kModePartial)
    hipLaunchKernelGGL((attn_f32_kernel<D, kModePartial>), dim3(blocks), dim3(kThreads), 0, s, q);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, kModeMerge>), dim3(blocks), dim3(kThreads), 0, s, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(int head_dim, int mode, const AttnParams& p, hipStream_t s) {
  return head_dim == 64 ? launch_d<64>(mode, p, s) : launch_d<128>(mode, p, s);
}

}  // namespace fbk
