// gfx950 (CDNA4) kernels of the FlashBlock attention step.
//
// Page "Résumé Technique : FlashBlock", §2 "Mécanisme Central": attention of
// the current block's queries is split into a block-external part (A_out,
// L_out = log Z_out, over the committed prefix) and a block-internal part
// (A_in, L_in, over the block itself), recombined in log space with
// m = max(L_out, L_in).  The same log-space rule combines the partial results
// of the prefix chunks that different workgroups attend (split-KV).
//
// attn_kernel: one workgroup = 4 wave64 = 128 packed query rows of one
// (sequence, kv head) group x one key range.  Each wave owns 32 rows.  Per
// 64-key tile, K and V are staged in LDS (K row-major with a 16-byte-chunk XOR
// swizzle, V transposed), then each wave computes S^T = K Q^T and
// O^T += V^T P^T with 32x32 MFMAs.  Working on the transposes puts one query
// row per lane pair (lanes l and l+32) in both products, so the online softmax
// max/sum and the rescale of O stay in the lane, up to one permlane32 swap.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fb_internal.h"

namespace fbk {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ bool head_selected(const HeadSel& s, int b, int bh) {
  if (!((s.seq_bits[b >> 5] >> (b & 31)) & 1u)) return false;
  if (s.flags == nullptr) return true;
  return (s.flags[bh] != 0) == (s.flags_select != 0);
}

// ---------------------------------------------------------------------------
// Operand staging
// ---------------------------------------------------------------------------

// bf16 K tile: Ks[key][D], 16-byte chunk c of row `key` stored at chunk
// c ^ (key % chunks_per_row), so that 32 lanes reading one chunk column of
// 32 rows spread over the banks.
// bf16 V tile, transposed: Vt[d][64], key k stored at position sigma(k) (bits 2
// and 3 of k swapped, which makes the 8 keys one MFMA k-step takes from a lane
// contiguous), 16-byte chunk c of row d stored at chunk c ^ (d % 8).
template <int D>
struct Bf16Tile {
  static constexpr int kCpr = D / 8;                    // 16-byte chunks per K row
  static constexpr int kKLoads = kKeyTile * kCpr / kThreads;   // per thread
  static constexpr int kVUnits = 16 * kCpr;             // (4 keys x 8 d) units per tile
  u32x4 kreg[kKLoads];
  u32x4 vreg[4];

  __device__ __forceinline__ void load(const bf16* kb, const bf16* vb, int tile0, int key_end, int tid) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int u = i * kThreads + tid, key = u / kCpr, c = u % kCpr;
      const int gk = tile0 + key;
      kreg[i] = gk < key_end ? *reinterpret_cast<const u32x4*>(kb + (int64_t)gk * D + c * 8) : u32x4{0, 0, 0, 0};
    }
    if (tid < kVUnits) {
      const int qd = tid % 16, dg = tid / 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gk = tile0 + 4 * qd + r;
        vreg[r] = gk < key_end ? *reinterpret_cast<const u32x4*>(vb + (int64_t)gk * D + dg * 8) : u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ __forceinline__ void store(bf16* ks, bf16* vt, int tid) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int u = i * kThreads + tid, key = u / kCpr, c = u % kCpr;
      *reinterpret_cast<u32x4*>(ks + key * D + ((c ^ (key & (kCpr - 1))) * 8)) = kreg[i];
    }
    if (tid < kVUnits) {
      const int qd = tid % 16, dg = tid / 16;
      const int qp = (qd & ~3) | ((qd & 1) << 1) | ((qd >> 1) & 1);   // sigma on key quads
      const int chunk = qp >> 1, within = (qp & 1) * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int drow = dg * 8 + e;
        // element e of each row: 16-bit lane (e & 1) of dword (e >> 1)
        const int w = e >> 1, sh = (e & 1) * 16;
        const uint32_t x0 = (vreg[0][w] >> sh) & 0xffffu, x1 = (vreg[1][w] >> sh) & 0xffffu;
        const uint32_t x2 = (vreg[2][w] >> sh) & 0xffffu, x3 = (vreg[3][w] >> sh) & 0xffffu;
        const u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
        *reinterpret_cast<u32x2*>(vt + drow * kKeyTile + ((chunk ^ (drow & 7)) * 8) + within) = pk;
      }
    }
  }
};

// fp32 tiles: K row-major with one padding float per row, V row-major.
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

template <typename T, int D>
struct Smem;
template <int D>
struct Smem<bf16, D> {
  bf16 k[kKeyTile * D];
  bf16 vt[D * kKeyTile];
};
template <int D>
struct Smem<float, D> {
  float k[kKeyTile * (D + 1)];
  float v[kKeyTile * D];
};

// ---------------------------------------------------------------------------
// Attention kernel
// ---------------------------------------------------------------------------
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_kernel(const AttnParams p) {
  constexpr bool kBf = std::is_same<T, bf16>::value;
  constexpr int kDt = D / 32;   // 32-wide d tiles of O^T
  __shared__ Smem<T, D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = lane & 31, hl = lane >> 5;
  int w = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = w % p.row_tiles;
  w /= p.row_tiles;
  const int split = w % p.splits;
  w /= p.splits;
  const int g = w % p.hkv, b = w / p.hkv;
  const int grp = p.hq / p.hkv;

  // Skip the whole group when none of its heads is selected (partial mode).
  if (MODE == kModePartial) {
    bool any = false;
    for (int i = 0; i < grp; ++i) any |= head_selected(p.sel, b, b * p.hq + g * grp + i);
    if (!any) return;
  }

  const int key_begin = split * p.keys_per_split;
  const int key_end = min(p.n_keys, key_begin + p.keys_per_split);
  const int row0 = rt * kRowTile + wave * 32;
  const int row = row0 + rl;
  const bool row_ok = row < p.rows;
  const bool wave_live = row0 < p.rows;
  const int64_t grow = (int64_t)(b * p.hq + g * grp) * p.bs + row;   // global row of this lane

  const T* qg = reinterpret_cast<const T*>(p.q);
  const T* kb = reinterpret_cast<const T*>(p.k) + ((int64_t)b * p.hkv + g) * p.kv_cap * D;
  const T* vb = reinterpret_cast<const T*>(p.v) + ((int64_t)b * p.hkv + g) * p.kv_cap * D;

  // Q^T as the B operand: lane (row, hl) holds Q[row][16t + 8hl .. +7] (bf16)
  // or Q[row][2t + hl] (fp32).
  using QFrag = typename std::conditional<kBf, bf16x8, float>::type;
  constexpr int kQf = kBf ? D / 16 : D / 2;
  QFrag qf[kQf];
#pragma unroll
  for (int t = 0; t < kQf; ++t) {
    if constexpr (kBf) {
      qf[t] = row_ok ? *reinterpret_cast<const bf16x8*>(qg + grow * D + 16 * t + 8 * hl) : bf16x8{};
    } else {
      qf[t] = row_ok ? qg[grow * D + 2 * t + hl] : 0.0f;
    }
  }

  f32x16 o[kDt];
#pragma unroll
  for (int i = 0; i < kDt; ++i) o[i] = f32x16{};
  float m = -INFINITY, lsum = 0.0f;

  typename std::conditional<kBf, Bf16Tile<D>, F32Tile<D>>::type stage;
  if (key_begin < key_end) stage.load(kb, vb, key_begin, key_end, tid);

  for (int tile0 = key_begin; tile0 < key_end; tile0 += kKeyTile) {
    __syncthreads();   // every wave finished reading the previous tile
    if constexpr (kBf) stage.store(sm.k, sm.vt, tid);
    else stage.store(sm.k, sm.v, tid);
    __syncthreads();
    if (tile0 + kKeyTile < key_end) stage.load(kb, vb, tile0 + kKeyTile, key_end, tid);
    if (!wave_live) continue;

    // S^T for keys tile0 + 32c + (0..31): lane (row, hl) reg j holds key 8(j/4) + 4hl + j%4.
    f32x16 s[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      s[c] = f32x16{};
      const int key = 32 * c + rl;
#pragma unroll
      for (int t = 0; t < kQf; ++t) {
        if constexpr (kBf) {
          constexpr int kCpr = D / 8;
          const int chunk = (2 * t + hl) ^ (key & (kCpr - 1));
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.k + key * D + chunk * 8);
          s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[c], 0, 0, 0);
        } else {
          const float a = sm.k[key * (D + 1) + 2 * t + hl];
          s[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[t], s[c], 0, 0, 0);
        }
      }
    }

    // Online softmax in the log2 domain.
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = tile0 + 32 * c + 8 * (j >> 2) + 4 * hl + (j & 3);
        const float x = key < key_end ? s[c][j] * p.scale_log2 : -INFINITY;
        s[c][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = pair_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < kDt; ++i) o[i] *= alpha;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = fast_exp2(s[c][j] - m);
        s[c][j] = e;
        lsum += e;
      }
    }

    // O^T += V^T P^T.
    if constexpr (kBf) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c = ks >> 1, kk = ks & 1;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (bf16)s[c][8 * kk + i];
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) {
          const int drow = 32 * dt + rl;
          const int chunk = (2 * ks + hl) ^ (drow & 7);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.vt + drow * kKeyTile + chunk * 8);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int c = u >> 4, j = u & 15;
        const int key = 32 * c + 8 * (j >> 2) + 4 * hl + (j & 3);
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) {
          const float a = sm.v[key * D + 32 * dt + rl];
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[c][j], o[dt], 0, 0, 0);
        }
      }
    }
  }

  const float ltot = pair_sum(lsum);
  if (!row_ok) return;

  if constexpr (MODE == kModePartial) {
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    const float lse = ltot > 0.0f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
    float* od = p.part_o + split * p.part_o_stride + grow * D;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v4 = {o[dt][4 * gq] * inv, o[dt][4 * gq + 1] * inv, o[dt][4 * gq + 2] * inv,
                          o[dt][4 * gq + 3] * inv};
        *reinterpret_cast<f32x4*>(od + 32 * dt + 8 * gq + 4 * hl) = v4;
      }
    }
    if (hl == 0) p.part_l[split * p.part_l_stride + grow] = lse;
  } else {
    const int head = g * grp + row / p.bs;
    const int bh = b * p.hq + head;
    if (p.reuse_rec != nullptr && hl == 0 && (row % p.bs) == 0)
      p.reuse_rec[bh] = head_selected(p.sel, b, bh) ? 0 : 1;
    const bool has_out = p.valid[bh] != 0;
    const int slot = p.cur[bh];
    const float l_out = has_out ? p.slot_l[slot * p.slot_l_stride + grow] : -INFINITY;
    const float l_in = (m + log2f(ltot)) * kLn2;
    const float mm = fmaxf(l_out, l_in);
    const float w_out = fast_exp2((l_out - mm) * kLog2e);
    const float w_in = fast_exp2((l_in - mm) * kLog2e);
    const float inv_den = 1.0f / (w_out + w_in);
    const float c_in = w_in / ltot * inv_den, c_out = w_out * inv_den;
    const float* ao = p.slot_o + slot * p.slot_o_stride + grow * D;
    T* od = reinterpret_cast<T*>(p.out) + grow * D;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * hl;
        f32x4 a4 = has_out ? *reinterpret_cast<const f32x4*>(ao + d0) : f32x4{0, 0, 0, 0};
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = c_out * a4[e] + c_in * o[dt][4 * gq + e];
        if constexpr (kBf) {
          bf16x4 rb = {(bf16)r[0], (bf16)r[1], (bf16)r[2], (bf16)r[3]};
          *reinterpret_cast<bf16x4*>(od + d0) = rb;
        } else {
          *reinterpret_cast<f32x4*>(od + d0) = r;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split combine: A = sum_s e^{L_s - M} A_s / sum_s e^{L_s - M}, L = M + log sum,
// M = max_s L_s, splits in a fixed order.  Under gamma it writes the other slot
// and sums <A_new, A_old>, |A_new|^2, |A_old|^2 over its rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const CombineParams p) {
  constexpr int kLpr = D / 4;              // threads per row (one float4 each)
  constexpr int kRpp = kThreads / kLpr;    // rows per pass
  __shared__ float red[3][kThreads / 64];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / p.row_chunks, ch = blockIdx.x % p.row_chunks;
  const int b = bh / p.hq;
  if (!head_selected(p.sel, b, bh)) return;
  const int src = p.cur[bh];
  const int dst = p.to_other_slot ? (src ^ 1) : src;
  const bool sim_terms = p.to_other_slot && p.valid[bh] != 0;
  const int c4 = tid % kLpr;
  float dot = 0.0f, nn = 0.0f, no = 0.0f;
  for (int pass = 0; pass < kCombineRows / kRpp; ++pass) {
    const int i = ch * kCombineRows + pass * kRpp + tid / kLpr;
    if (i >= p.bs) continue;
    const int64_t grow = (int64_t)bh * p.bs + i;
    float mx = -INFINITY;
    for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.part_l[s * p.part_l_stride + grow]);
    f32x4 acc = {0, 0, 0, 0};
    float wsum = 0.0f;
    if (mx > -INFINITY) {
      for (int s = 0; s < p.splits; ++s) {
        const float wgt = fast_exp2((p.part_l[s * p.part_l_stride + grow] - mx) * kLog2e);
        const f32x4 a = *reinterpret_cast<const f32x4*>(p.part_o + s * p.part_o_stride + grow * D + 4 * c4);
        wsum += wgt;
        acc += wgt * a;
      }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const f32x4 a_new = acc * inv;
    const float lse = wsum > 0.0f ? mx + logf(wsum) : -INFINITY;
    if (sim_terms) {
      const f32x4 a_old = *reinterpret_cast<const f32x4*>(p.slot_o + src * p.slot_o_stride + grow * D + 4 * c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += a_new[e] * a_old[e];
        nn += a_new[e] * a_new[e];
        no += a_old[e] * a_old[e];
      }
    }
    *reinterpret_cast<f32x4*>(p.slot_o + dst * p.slot_o_stride + grow * D + 4 * c4) = a_new;
    if (c4 == 0) p.slot_l[dst * p.slot_l_stride + grow] = lse;
  }
  if (sim_terms) {
    dot = wave_sum(dot);
    nn = wave_sum(nn);
    no = wave_sum(no);
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = dot;
      red[1][tid >> 6] = nn;
      red[2][tid >> 6] = no;
    }
    __syncthreads();
    if (tid < 3) {
      float t = 0.0f;
      for (int i = 0; i < kThreads / 64; ++i) t += red[tid][i];
      p.cos_part[((int64_t)bh * p.row_chunks + ch) * 3 + tid] = t;
    }
  }
  if (!p.to_other_slot && ch == 0 && tid == 0) p.valid[bh] = 1;
}

// ---------------------------------------------------------------------------
// Gamma decisions: similarity of every recomputed head, slot flip, and the
// reuse decision of the next step (strict sim > gamma; NaN never reuses).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void decide_kernel(const DecideParams p) {
  const int bh = blockIdx.x * kThreads + threadIdx.x;
  if (bh >= p.n_heads) return;
  if (p.reuse_now[bh] == 0) {
    if (p.valid[bh]) {
      float dot = 0.0f, nn = 0.0f, no = 0.0f;
      for (int c = 0; c < p.row_chunks; ++c) {
        const float* t = p.cos_part + ((int64_t)bh * p.row_chunks + c) * 3;
        dot += t[0];
        nn += t[1];
        no += t[2];
      }
      float sim;
      if (nn == 0.0f || no == 0.0f) sim = (nn == 0.0f && no == 0.0f) ? 1.0f : 0.0f;
      else sim = fminf(1.0f, fmaxf(-1.0f, dot / (sqrtf(nn) * sqrtf(no))));
      p.sim[bh] = sim;
    }
    p.cur[bh] ^= 1;
    p.valid[bh] = 1;
  }
  const float s = p.sim[bh];
  p.reuse_next[bh] = (p.valid[bh] && s > p.gamma) ? 1 : 0;
}

__global__ __launch_bounds__(kThreads) void reset_kernel(const ResetParams p) {
  const int bh = blockIdx.x * kThreads + threadIdx.x;
  if (bh >= p.n_heads) return;
  p.cur[bh] = 0;
  p.valid[bh] = 0;
  p.reuse[bh] = 0;
  p.reuse[p.n_heads + bh] = 0;
  p.sim[bh] = __builtin_nanf("");
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_attn_t(int mode, const AttnParams& p, hipStream_t s) {
  const int blocks = p.batch * p.hkv * p.splits * p.row_tiles;
  if (blocks == 0) return hipSuccess;
  if (mode == kModePartial) {
    hipLaunchKernelGGL((attn_kernel<T, D, kModePartial>), dim3(blocks), dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((attn_kernel<T, D, kModeMerge>), dim3(blocks), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, int head_dim, int mode, const AttnParams& p, hipStream_t s) {
  if (dtype == FB_BF16) {
    return head_dim == 64 ? launch_attn_t<bf16, 64>(mode, p, s) : launch_attn_t<bf16, 128>(mode, p, s);
  }
  return head_dim == 64 ? launch_attn_t<float, 64>(mode, p, s) : launch_attn_t<float, 128>(mode, p, s);
}

hipError_t launch_combine(int head_dim, const CombineParams& p, hipStream_t s) {
  const int blocks = p.batch * p.hq * p.row_chunks;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 64) hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decide(const DecideParams& p, hipStream_t s) {
  hipLaunchKernelGGL(decide_kernel, dim3((p.n_heads + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_reset(const ResetParams& p, hipStream_t s) {
  hipLaunchKernelGGL(reset_kernel, dim3((p.n_heads + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fbk
