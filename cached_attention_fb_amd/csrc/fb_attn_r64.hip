// bf16 attention of 256 packed query rows per workgroup with 64 rows per
// wave (gfx950, CDNA4): the partial (split-KV) launches over dense prefix
// keys of groups of more than 128 packed rows (grouped query heads x block
// tokens), head dim 128.
//
// Workgroup = 4 row waves x 2 key halves (8 wave64, two per SIMD).  Row wave
// rw owns rows 64rw .. 64rw+63 of the workgroup's 256 as two 32-row MFMA
// blocks; key half kh takes keys 32kh .. 32kh+31 of every 64-key tile.  Each
// K or V fragment a wave reads from LDS feeds two 32x32x16 MFMAs (its two row
// blocks), so a tile costs the CU 128 KB of LDS reads for its 8.4 MFLOP,
// half of what 32 rows per wave need; LDS read bandwidth (128 B per clock
// per CU) then sits at half the MFMA rate instead of level with it.  The two
// waves of a SIMD drift out of phase within a tile (the second queues behind
// the first's MFMAs), so one's softmax runs under the other's MFMAs.  The two
// key halves' (O, m, sum) are merged through LDS at the end.
//
// K/V tiles stream HBM -> LDS through the 4-stage DMA ring of fb_lds.h.
// Every register of the wave is architectural (MFMA results in VGPRs):
// O^T 128, Q^T 64, S^T 32, P 16 and the fragment offsets just fit 256.
#include <algorithm>
#include <atomic>

#include "fb_device.h"
#include "fb_lds.h"

namespace fbk {

namespace {

constexpr int kD = 128;
constexpr int kRowW = 4;                    // row waves
constexpr int kWaves = 2 * kRowW;           // x 2 key halves
constexpr int kRb = 2;                      // 32-row MFMA blocks per wave
constexpr int kRowsWg = kRowW * 32 * kRb;   // 256 packed rows per workgroup
constexpr int kKs = kD / 16;                // k-steps of S^T = K Q^T
constexpr int kDt = kD / 32;                // head-dim tiles of O^T
using Ring = Pipe<kD, kWaves>;

// Per-lane LDS addressing of the K fragments and the transposed V reads.  K
// chunk 2t + hl of key rl sits at chunk (2t + hl) ^ (rl % 16) of its row, i.e.
// at k_base + 32 (t ^ k_sw) with k_sw = (rl % 16) / 2; the V^T operand of
// head-dim tile dt at v_base + 64 (dt ^ v_sw).  Two registers each instead of
// a table per k-step: the table would not fit beside O, Q and S.
struct FragAddr {
  uint32_t k_base, k_sw, v_base, v_sw;
};

// The lane index recomputed from the execution mask (two instructions), so
// that values derived from it need not stay live across the loop.  The empty
// asm keeps the compiler from reusing an earlier copy.
__device__ __forceinline__ int lane_id() {
  int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}

// S^T of a 32-key half for one row block: s = K_half Q_rb^T.
__device__ __forceinline__ void qk_block(f32x16& s, const bf16x8 (&qf)[kKs], uint32_t k_half, const FragAddr& fa) {
  s = f32x16{};
#pragma unroll
  for (int t = 0; t < kKs; ++t) {
    const u32x4 kf = lds_b128(k_half + fa.k_base + ((t ^ fa.k_sw) << 5));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf), qf[t], s, 0, 0, 0);
  }
  // one fragment ahead, then one read per MFMA: two fragments live at most
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int t = 0; t < kKs; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// O^T += V^T P^T for a 32-key half: the V^T operand of k-step kl and head-dim
// tile dt (two transposed 8-byte reads) is read once and used by both blocks.
__device__ __forceinline__ void pv_half2(f32x16 (&o)[kRb][kDt], const bf16x8 (&pb)[kRb][2], uint32_t v_half,
                                         const FragAddr& fa) {
#pragma unroll
  for (int kl = 0; kl < 2; ++kl) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const uint32_t a = v_half + fa.v_base + ((dt ^ fa.v_sw) << 6) + 16 * kl * kD * 2;
      const u32x2 lo = lds_tr16(a), hi = lds_tr16(a + 8 * kD * 2);
      const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int rb = 0; rb < kRb; ++rb)
        o[rb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), pb[rb][kl], o[rb][dt], 0,
                                                            0, 0);
    }
  }
  // one operand (two reads) ahead, then two reads per MFMA pair
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i < 2 * kDt; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// P = exp2(c s - mref) of one S^T block, its contribution to the lane's row
// sum (two short chains), and the bf16 B operands of its two k-steps.
__device__ __forceinline__ void exp_block(const f32x16& s, float mref, float c, float& lsum, bf16x8 (&pb)[2]) {
  float part[2] = {0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float e = fast_exp2(fmaf(s[j], c, -mref));
    part[j & 1] += e;
    pb[j >> 3][j & 7] = (bf16)e;
  }
  lsum += part[0] + part[1];
}

// Epilogue of a partial through LDS (as the other bf16 kernel's): normalise
// one 32-row block, stage it row-major (16-byte chunk c of row r at
// c ^ (r % (D/4))) and store whole rows, D/4 lanes per row.
__device__ __forceinline__ void store_block(const AttnParams& p, const f32x16 (&o)[kDt], float m, float ltot, int split,
                                            int64_t grow0, int nrows, FB_LDS float* st, int lane) {
  constexpr int kC = kD / 4;
  constexpr int kRowsPerOp = 64 / kC;
  const int rl = lane & 31, hl = lane >> 5;
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  const float lse = ltot > 0.0f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int cc = 8 * dt + 2 * gq + hl;
      const f32x4 v4 = {o[dt][4 * gq] * inv, o[dt][4 * gq + 1] * inv, o[dt][4 * gq + 2] * inv, o[dt][4 * gq + 3] * inv};
      *reinterpret_cast<FB_LDS f32x4*>(st + rl * kD + ((cc ^ (rl & (kC - 1))) * 4)) = v4;
    }
  }
  if (hl == 0 && rl < nrows) __builtin_nontemporal_store(lse, p.part_l + split * p.part_l_stride + grow0 + rl);
  bf16* od = reinterpret_cast<bf16*>(p.part_o) + split * p.part_o_stride + grow0 * kD;
#pragma unroll
  for (int k = 0; k < 32 / kRowsPerOp; ++k) {
    const int r = k * kRowsPerOp + lane / kC, cc = lane % kC;
    const f32x4 v = *reinterpret_cast<const FB_LDS f32x4*>(st + r * kD + ((cc ^ (r & (kC - 1))) * 4));
    const bf16x4 vb = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    if (r < nrows) __builtin_nontemporal_store(vb, reinterpret_cast<bf16x4*>(od + (int64_t)r * kD + 4 * cc));
  }
}

// LDS of the end-of-loop exchange: per row wave, 64 lanes x (4 kDt O chunks
// of 16 bytes per block + one (m, sum) chunk per block).
constexpr int kXchChunks = kRb * (4 * kDt + 1);
constexpr int kXchBytes = kRowW * kXchChunks * 64 * 16;

template <int AUX>
__global__ __launch_bounds__(64 * kWaves) void attn_r64_kernel(const AttnParams p) {
  extern __shared__ char smem_raw[];
  FB_LDS char* lds = (FB_LDS char*)smem_raw;

  prefetch_params(p);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave % kRowW, kh = wave / kRowW;
  const int rl = lane & 31, hl = lane >> 5;
  const AttnItem it = attn_item<false>(p, true);   // dense keys only
  record_decisions(p);
  if (!it.ok) return;   // workgroup-uniform
  const int b = it.b, g = it.g, grp = p.grp;
  const int key_begin = it.key_begin, key_end = it.key_end;
  const int n = key_end > key_begin ? (key_end - key_begin + kKeyTile - 1) / kKeyTile : 0;
  const int row0 = it.rt * kRowsWg + rw * 32 * kRb;   // first row of the row wave
  const bool wave_live = row0 < p.rows;
  const int64_t grow0 = (int64_t)(b * p.hq + g * grp) * p.bs + row0;   // its global row index
  const bf16* qg = reinterpret_cast<const bf16*>(p.q);
  const int64_t kv_cap = it.internal ? p.bs : p.kv_cap;
  const bf16* kb = reinterpret_cast<const bf16*>(it.internal ? p.kblk : p.k) + ((int64_t)b * p.hkv + g) * kv_cap * kD;
  const bf16* vb = reinterpret_cast<const bf16*>(it.internal ? p.vblk : p.v) + ((int64_t)b * p.hkv + g) * kv_cap * kD;
  const int lim = key_end;
  const int ring = Ring::ring_stages(p.ring_keys);

  // Prologue: Q of the row waves' blocks (ring stages 2-3, or past a short
  // ring) and the first two tiles; Q into registers once tile 0 landed.
  FB_LDS char* q_lds = lds + Ring::q_offset(ring, 2 * kRowW) + rw * 32 * kRb * kD * 2;
  if (kh == 0 && wave_live) {
    const int left = p.rows - row0;
    issue_q<kD>(q_lds, qg + grow0 * kD, left, lane);
    // a second block with no valid row re-reads the first block's rows
    issue_q<kD>(q_lds + 32 * kD * 2, qg + (grow0 + (left > 32 ? 32 : 0)) * kD, left > 32 ? left - 32 : left, lane);
  }
  int issued;
  if (n >= 2) {
    issue_tile<kD, kWaves, AUX>(lds, kb, vb, key_begin, lim, wave, lane);
    issue_tile<kD, kWaves, AUX>(lds + Ring::kStageBytes, kb, vb, key_begin + kKeyTile, lim, wave, lane);
    issued = 2;
    wait_vmcnt<Ring::kLpt>();   // tile 0 (and Q) landed; tile 1 may be in flight
  } else if (n == 1) {
    issue_tile<kD, kWaves, AUX>(lds, kb, vb, key_begin, lim, wave, lane);
    issued = 1;
    wait_vmcnt<0>();
  } else {
    issued = 0;
    wait_vmcnt<0>();
  }
  lds_barrier();
  bf16x8 qf[kRb][kKs];
  {
    const uint32_t q0 = (uint32_t)(uintptr_t)q_lds;
#pragma unroll
    for (int rb = 0; rb < kRb; ++rb) {
#pragma unroll
      for (int t = 0; t < kKs; ++t)
        qf[rb][t] = __builtin_bit_cast(
            bf16x8, lds_b128(q0 + rb * 32 * kD * 2 + rl * kD * 2 + (((2 * t + hl) ^ (rl & (Ring::kCpr - 1))) * 16)));
    }
  }
  // Q sits in ring stages 2-3 when the ring is full: read by every wave before
  // the first refill writes there
  if (!Ring::q_past(2 * kRowW) && ring == Ring::kStages) lds_barrier();

  // Per-lane LDS addressing of this wave's key half.  K fragment t: key rl
  // of the half, chunk (2t + hl) ^ (rl % 16) = 2 (t ^ k_sw) + (hl ^ (rl % 2)).
  // Transposed V reads (as in the other bf16 kernel): in a 16-lane group tg,
  // lane 4j + q addresses 4 columns of key 4hl + j; head-dim tile dt sits at
  // chunk (4dt + 2(tg % 2) + q / 2) ^ (4 key % 16) = 4 (dt ^ v_sw) + 2(tg % 2) + q / 2.
  const uint32_t hoff = kh * 32 * kD * 2;
  // From the lane index, once per tile: a handful of integer operations
  // instead of four registers held across the loop.
  auto frag_addr = [&](int ln) {
    FragAddr fa;
    const int r = ln & 31, h = ln >> 5;
    fa.k_base = hoff + r * kD * 2 + ((h ^ (r & 1)) * 16);
    fa.k_sw = (r & (Ring::kCpr - 1)) >> 1;
    const int tg = ln >> 4, tj = (ln & 15) >> 2, tq = ln & 3;
    const int key = 4 * h + tj;
    fa.v_base = hoff + key * kD * 2 + (2 * (tg & 1) + (tq >> 1)) * 16 + (tq & 1) * 8;
    fa.v_sw = ((4 * key) & (Ring::kCpr - 4)) >> 2;
    return fa;
  };

  f32x16 o[kRb][kDt];
#pragma unroll
  for (int rb = 0; rb < kRb; ++rb) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) o[rb][dt] = f32x16{};
  }
  float m[kRb] = {-INFINITY, -INFINITY}, lsum[kRb] = {0.0f, 0.0f};
  const float c = p.scale_log2;
  const uint32_t lds_off = (uint32_t)(uintptr_t)lds;
  for (int t = 0; t < n; ++t) {
    if (t > 0) {
      wait_tile<Ring::kLpt, Ring::kStages>(issued - t - 1);   // tiles issued after t may stay in flight
      lds_barrier();   // every wave's share of tile t landed; all waves finished tile t-1
    }
    const int key0 = key_begin + t * kKeyTile + 32 * kh;   // first key of this wave's half
    const uint32_t ks_off = lds_off + (t % Ring::kStages) * Ring::kStageBytes;
    // the fragment addresses, computed per tile (hoisted out of the loop
    // they would take 12 registers more)
    const FragAddr fa = frag_addr(lane_id());
    // The two row blocks one after the other (S of one block, 16 registers,
    // live at a time; the K fragments are read once per block), then the PV
    // MFMAs of both blocks, which share each V^T operand.
    bf16x8 pb[kRb][2];
#pragma unroll
    for (int rb = 0; rb < kRb; ++rb) {
      f32x16 s;
      qk_block(s, qf[rb], ks_off, fa);
      if (key0 + 32 > lim) {   // the range's ragged last tile
        const int k_l = key0 + 4 * (lane_id() >> 5);   // recomputed: not kept live across the loop
#pragma unroll
        for (int j = 0; j < 16; ++j) s[j] = k_l + 8 * (j >> 2) + (j & 3) >= lim ? -INFINITY : s[j];
      }
      // Row max (log2 units); the running max is raised only when a row's max
      // grows by more than 2^kRescale (exact: P and the sum use the same m),
      // so after the first tile the O rescale rarely runs.  A half with no key
      // (the second half of a short last tile) leaves m at -inf until it has one.
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[j]);
      mx = pair_max(mx) * c;
      const bool raise = mx > m[rb] + kRescale;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? mx : m[rb];
        const float alpha = m[rb] > -INFINITY ? fast_exp2(m[rb] - m_new) : 0.0f;
        lsum[rb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) o[rb][dt] *= alpha;
        m[rb] = m_new;
      }
      exp_block(s, m[rb] > -INFINITY ? m[rb] : 0.0f, c, lsum[rb], pb[rb]);
    }
    pv_half2(o, pb, ks_off + Ring::kTensorBytes, fa);
    // refill the stage of tile t-1 (every wave passed the barrier above); the
    // lane index is recomputed here, so that the loads' per-lane offsets are
    // computed where they are used instead of held across the loop
    for (; issued < n && issued <= t + Ring::kStages - 1; ++issued) {
      issue_tile<kD, kWaves, AUX>(lds + (issued % Ring::kStages) * Ring::kStageBytes, kb, vb,
                                  key_begin + issued * kKeyTile, lim, wave, lane_id());
    }
  }

  // Merge the two key halves of each row: the second half's waves hand their
  // (O, m, lane sum) to the first through LDS (no DMA is in flight: the last
  // tile waited for vmcnt 0), chunk c of lane l at c*64 + l.
  const int ln = lane_id();   // recomputed: the lane index is not kept live across the loop
  FB_LDS f32x4* xch = (FB_LDS f32x4*)lds + rw * kXchChunks * 64 + ln;
  lds_barrier();
  if (kh == 1 && wave_live) {
#pragma unroll
    for (int rb = 0; rb < kRb; ++rb) {
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xch[(rb * (4 * kDt + 1) + 4 * dt + q) * 64] =
              f32x4{o[rb][dt][4 * q], o[rb][dt][4 * q + 1], o[rb][dt][4 * q + 2], o[rb][dt][4 * q + 3]};
      }
      xch[(rb * (4 * kDt + 1) + 4 * kDt) * 64] = f32x4{m[rb], lsum[rb], 0.0f, 0.0f};
    }
  }
  lds_barrier();
  if (kh == 1 || !wave_live) return;
#pragma unroll
  for (int rb = 0; rb < kRb; ++rb) {
    const f32x4 ml = xch[(rb * (4 * kDt + 1) + 4 * kDt) * 64];
    const float m2 = ml[0], l2 = ml[1];
    const float mt = fmaxf(m[rb], m2);
    const float a1 = m[rb] > -INFINITY ? fast_exp2(m[rb] - mt) : 0.0f;
    const float a2 = m2 > -INFINITY ? fast_exp2(m2 - mt) : 0.0f;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = xch[(rb * (4 * kDt + 1) + 4 * dt + q) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[rb][dt][4 * q + e] = a1 * o[rb][dt][4 * q + e] + a2 * v[e];
      }
    }
    lsum[rb] = a1 * lsum[rb] + a2 * l2;
    m[rb] = mt;
  }
  // Partial epilogue: each first-half wave stages its two blocks in its own
  // exchange region (34 KB, read into registers above; the 32 KB of staging
  // fit) and stores whole rows.
  static_assert(kRb * 32 * kD * 4 <= kXchChunks * 64 * 16, "staging fits the exchange region");
  FB_LDS float* st = (FB_LDS float*)lds + rw * kXchChunks * 64 * 4;
#pragma unroll
  for (int rb = 0; rb < kRb; ++rb) {
    const int nrows = min(32, p.rows - row0 - 32 * rb);
    if (nrows <= 0) break;
    store_block(p, o[rb], m[rb], pair_sum(lsum[rb]), it.split, grow0 + 32 * rb, nrows, st + rb * 32 * kD, ln);
  }
}

}  // namespace

hipError_t launch_attn_r64(const AttnParams& p, hipStream_t s) {
  const int blocks = p.grid > 0 ? p.grid : p.batch * p.hkv * p.splits * p.row_tiles;
  if (blocks == 0) return hipSuccess;
  constexpr int kQBytes = kRowsWg * kD * 2;
  constexpr int kMaxLds = std::max({Ring::kLdsBytes, Ring::q_offset(Ring::kStages, 2 * kRowW) + kQBytes, kXchBytes});
  static_assert(kMaxLds <= 160 * 1024, "fits the CU's LDS");
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (bit == 0 || (attr_done.load(std::memory_order_acquire) & bit) == 0) {
    for (const void* f : {(const void*)attn_r64_kernel<0>, (const void*)attn_r64_kernel<2>}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
      if (e != hipSuccess) return e;
    }
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  const int ring = Ring::ring_stages(p.ring_keys);
  const int lds = std::max({ring * Ring::kStageBytes, Ring::q_offset(ring, 2 * kRowW) + kQBytes, kXchBytes});
  const AttnParams q = with_div_magic(p, blocks);
  // each K/V tile read by one workgroup (one row tile per group): non-temporal loads
  if (p.row_tiles == 1) hipLaunchKernelGGL(attn_r64_kernel<2>, dim3(blocks), dim3(64 * kWaves), lds, s, q);
  else hipLaunchKernelGGL(attn_r64_kernel<0>, dim3(blocks), dim3(64 * kWaves), lds, s, q);
  return hipGetLastError();
}

}  // namespace fbk
