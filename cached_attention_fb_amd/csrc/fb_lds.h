// LDS staging helpers shared by the bf16 attention kernels (gfx950): the
// HBM -> LDS DMA loads of K/V tiles and Q rows, their waits, and the LDS
// fragment reads that feed the MFMAs.
//
// LDS layout of one ring stage: K tile [64][D] then V tile [64][D], bf16, both
// row-major in 16-byte chunks with an XOR swizzle chosen on the global side
// (each lane of a DMA load writes a fixed LDS slot, so the lane picks which
// global chunk to fetch):
//   K: chunk c of key k at c ^ (k % (D/8))       (16 rows, one chunk column: all banks)
//   V: chunk c of key k at c ^ (4(k % 4) % (D/8)) (4 rows x 64 B of a transposed read: all banks)
#pragma once

#include "fb_device.h"

namespace fbk {

// The K/V/Q DMA loads are issued from asm (see dma16), so the compiler does
// not know about them: every wait for them is written here, in asm, and is a
// compiler memory barrier, so that no LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that LDS accesses may not be moved across by the
// compiler (the builtin alone does not order memory operations).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte-per-lane DMA load HBM -> LDS (global_load_lds_dwordx4): lane i
// writes dst + 16 i.  Issued from asm so that the compiler, unaware of it,
// does not wait for every DMA load still in flight before each LDS read (it
// would with the builtin, draining the tile ring).  AUX 2 = non-temporal.
// The compiler does not look inside asm for hazards, so the asm supplies the
// wait states itself: the LDS address comes from M0, which the compiler sets
// just before with a scalar instruction, and an LDS DMA needs one wait state
// after a scalar write of M0.
template <int AUX>
__device__ __forceinline__ void dma16(FB_LDS char* dst, const void* src) {
  static_assert(AUX == 0 || AUX == 2, "cache policy: default or non-temporal");
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  if constexpr (AUX == 2)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The same load with a wave-uniform base address (SGPRs) and a per-lane 32-bit
// byte offset (the saddr form), so that a lane adds no 64-bit address.  The
// base must be the same in every lane (it is read from the first).  The base
// SGPRs may be written by a vector instruction (v_readfirstlane) right before,
// and a memory instruction may read such an SGPR only 5 wait states later:
// the asm waits them out (they also cover the M0 write).
template <int AUX>
__device__ __forceinline__ void dma16s(FB_LDS char* dst, const void* base_any, uint32_t voff) {
  static_assert(AUX == 0 || AUX == 2, "cache policy: default or non-temporal");
  const uint64_t a = (uint64_t)(uintptr_t)base_any;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const void* base = (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  const uint32_t m0 = (uint32_t)(uintptr_t)dst;
  if constexpr (AUX == 2)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

// Plain LDS reads at a byte address; the compiler waits for them where their
// values are first used.
__device__ __forceinline__ u32x4 lds_b128(uint32_t a) { return *(const FB_LDS u32x4*)(size_t)a; }
__device__ __forceinline__ u32x2 lds_tr16(uint32_t a) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FB_LDS s16x4*)(size_t)a));
}

// Transposed LDS reads (ds_read_b64_tr_b16) of the V^T operands of one 32-key
// half C (k-steps 2C and 2C+1, every head-dim tile, both 4-key sub-halves).
// base[dt] = the lane's offset for head-dim tile dt; k-step kl, sub-half hf
// sits (32C + 16kl + 8hf) rows further.  r[(kl*kDt + dt)*2 + hf].
template <int D, int C>
__device__ __forceinline__ void tr_read_half(u32x2 (&r)[D / 8], const uint32_t (&base)[D / 32]) {
  constexpr int kDt = D / 32;
#pragma unroll
  for (int kl = 0; kl < 2; ++kl) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) r[(kl * kDt + dt) * 2 + hf] = lds_tr16(base[dt] + (32 * C + 16 * kl + 8 * hf) * D * 2);
    }
  }
}

// Both 32-key halves' V^T operands (the whole-tile shapes): r0 = half 0,
// r1 = half 1, each in the layout of tr_read_half.
template <int D>
__device__ __forceinline__ void tr_read_both(u32x2 (&r0)[D / 8], u32x2 (&r1)[D / 8], const uint32_t (&base)[D / 32]) {
  tr_read_half<D, 0>(r0, base);
  tr_read_half<D, 1>(r1, base);
}

// Wait until at most `after` tiles' DMA loads (kLpt per tile and wave) are
// still in flight, i.e. this wave's share of the current tile has landed.
// When after*kLpt does not fit the 6-bit counter, wait for fewer (safe).
template <int kLpt, int kMaxAfter>
__device__ __forceinline__ void wait_tile(int after) {
  if constexpr (kMaxAfter >= 3 && 3 * kLpt <= 63) {
    if (after >= 3) { wait_vmcnt<3 * kLpt>(); return; }
  }
  if constexpr (kMaxAfter >= 2 && 2 * kLpt <= 63) {
    if (after >= 2) { wait_vmcnt<2 * kLpt>(); return; }
  }
  if constexpr (kLpt <= 63) {
    if (after >= 1) { wait_vmcnt<kLpt>(); return; }
  }
  wait_vmcnt<0>();
}

// K^T operand fragments of one 32-key half: 16-byte chunk 2t + hl of the
// lane's key row, t = 0..D/16-1 (ds_read_b128).  a[t] = row/chunk offset of
// the lane in the stage, OFF = the half's offset (32 rows per half).
template <int D, int OFF>
__device__ __forceinline__ void k_read_half(u32x4 (&r)[D / 16], const uint32_t (&a)[D / 16]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) r[t] = lds_b128(a[t] + OFF);
}

// Both halves' K^T operand fragments (r0 = keys 0-31 of the tile, r1 = keys
// 32-63), as k_read_half.
template <int D>
__device__ __forceinline__ void k_read_both(u32x4 (&r0)[D / 16], u32x4 (&r1)[D / 16], const uint32_t (&a)[D / 16]) {
  k_read_half<D, 0>(r0, a);
  k_read_half<D, 32 * D * 2>(r1, a);
}


// P = exp2(c*s - mref) of one S^T half, its contribution to the lane's row
// sum, and the bf16 B operands of its two k-steps (registers j = 8kl .. 8kl+7).
__device__ __forceinline__ void exp_half(f32x16& s, float mref, float c, float& lsum, bf16x8 (&pb)[2]) {
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // four short sum chains instead of one long one
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float e = fast_exp2(fmaf(s[j], c, -mref));
    part[j & 3] += e;
    pb[j >> 3][j & 7] = (bf16)e;
  }
  lsum += (part[0] + part[1]) + (part[2] + part[3]);
}

// O^T += V^T P^T for one 32-key half: k-step kl takes keys 16kl + 8(i/4) +
// 4hl + i%4 (i = 0..7) of the half from both operands.
template <int kDt>
__device__ __forceinline__ void pv_half(f32x16 (&o)[kDt], const u32x2 (&vr)[4 * kDt], const bf16x8 (&pb)[2]) {
#pragma unroll
  for (int kl = 0; kl < 2; ++kl) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const u32x2 lo = vr[(kl * kDt + dt) * 2], hi = vr[(kl * kDt + dt) * 2 + 1];
      const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), pb[kl], o[dt], 0, 0, 0);
    }
  }
}

template <int D, int WAVES>
struct Pipe {
  static constexpr int kCpr = D / 8;                             // 16-byte chunks per row
  static constexpr int kTensorBytes = kKeyTile * D * 2;          // one K or V tile
  static constexpr int kInstrPerTensor = kKeyTile * kCpr / 64;   // wave-wide 1 KB DMA loads
  static constexpr int kLpt = 2 * kInstrPerTensor / WAVES;       // DMA loads per wave per tile
  static constexpr int kStages = 4;                              // 4 x 32 KB ring (D = 128)
  static constexpr int kStageBytes = 2 * kTensorBytes;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static_assert(2 * kInstrPerTensor % WAVES == 0, "tile loads split evenly over the waves");
  // Ring stages a workgroup uses (never more than its key range has tiles).
  __host__ __device__ static int ring_stages(int keys_per_split) {
    const int t = (keys_per_split + kKeyTile - 1) / kKeyTile;
    return t < 1 ? 1 : (t < kStages ? t : kStages);
  }
  // Q staging (ROWW x 32 rows x D, read once before the first tile): past
  // the ring when a full ring and Q fit the CU's 160 KB (no barrier between
  // reading Q and refilling the ring), else, with a full ring, in stages 2-3
  // (first filled after Q has been read).
  __host__ __device__ static constexpr bool q_past(int rows_w) { return kLdsBytes + rows_w * 32 * D * 2 <= 160 * 1024; }
  __host__ __device__ static constexpr int q_offset(int ring, int rows_w) {
    return (ring == kStages && !q_past(rows_w)) ? 2 * kStageBytes : ring * kStageBytes;
  }
};

// AUX: cache policy of the DMA loads (2: non-temporal, for K/V that no other
// workgroup of the launch reads again).
//
// A whole tile (every key below key_end) takes the short form: instruction ii
// covers keys kKpi*ii + key_l (key_l = lane / (D/8)), so its base is uniform
// and the lane's offset depends on ii only through the K swizzle, whose
// ii-part is a multiple of kKpi while key_l < kKpi:
//   K chunk pc ^ ((kKpi*ii + key_l) % (D/8)) = (pc ^ key_l) ^ ((kKpi*ii) % (D/8)),
//   V chunk pc ^ ((4*key) % (D/8) & ~3) = pc ^ (4*key_l % (D/8)) (4*kKpi*ii is
//   a multiple of D/8).
// A ragged tile clamps every key to the last valid one.
template <int D, int WAVES, int AUX>
__device__ __forceinline__ void issue_tile(FB_LDS char* stage, const bf16* kb, const bf16* vb, int tile0,
                                           int key_end, int wave, int lane) {
  using P = Pipe<D, WAVES>;
  constexpr int kKpi = 64 / P::kCpr;   // keys per DMA instruction
  static_assert(P::kCpr % kKpi == 0 && P::kCpr <= 16, "the swizzles split into a uniform and a per-lane part");
  if (tile0 + kKeyTile <= key_end) {
    const int key_l = lane / P::kCpr, pc = lane % P::kCpr;
    const uint32_t row_b = key_l * D * 2;
    const uint32_t k_c = (pc ^ key_l) * 16;
    const uint32_t v_off = row_b + (pc ^ ((4 * key_l) & (P::kCpr - 4))) * 16;
    // A wave's instructions are consecutive: with several waves they lie in
    // one tensor (ii = ii0 + j), a lone wave issues all of them (ii = j % kIPT).
    constexpr int kIPT = P::kInstrPerTensor;
    static_assert(WAVES == 1 || kIPT % P::kLpt == 0, "a wave's loads stay in one tensor");
    const int idx0 = wave * P::kLpt;
    const int tensor_w = idx0 / kIPT, ii0 = idx0 % kIPT;
    const bf16* base0 = (tensor_w == 0 ? kb : vb) + (int64_t)(tile0 + kKpi * ii0) * D;
    FB_LDS char* dst0 = stage + tensor_w * P::kTensorBytes + ii0 * 1024;
#pragma unroll
    for (int j = 0; j < P::kLpt; ++j) {
      const int tensor = WAVES == 1 ? j / kIPT : tensor_w;
      const int ii = WAVES == 1 ? j % kIPT : ii0 + j;
      const bf16* base = WAVES == 1 ? (tensor == 0 ? kb : vb) + (int64_t)(tile0 + kKpi * ii) * D : base0 + j * kKpi * D;
      FB_LDS char* dst = WAVES == 1 ? stage + tensor * P::kTensorBytes + ii * 1024 : dst0 + j * 1024;
      const uint32_t voff = tensor == 0 ? row_b + (k_c ^ (((kKpi * ii) & (P::kCpr - 1)) * 16)) : v_off;
      dma16s<AUX>(dst, base, voff);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < P::kLpt; ++j) {
    const int idx = wave * P::kLpt + j;
    const int tensor = idx / P::kInstrPerTensor;   // 0: K, 1: V (wave-uniform)
    const int ii = idx % P::kInstrPerTensor;
    const int pos = ii * 64 + lane;                 // 16-byte slot inside the tile
    const int key = pos / P::kCpr, pc = pos % P::kCpr;
    const int swz = tensor == 0 ? (key & (P::kCpr - 1)) : ((4 * key) & (P::kCpr - 4));
    const int gk = max(0, min(tile0 + key, key_end - 1));   // rows past the end: any valid row (masked later)
    const bf16* src = (tensor == 0 ? kb : vb) + (int64_t)gk * D + (pc ^ swz) * 8;
    dma16<AUX>(stage + tensor * P::kTensorBytes + ii * 1024, src);
  }
}

// The wave's 32 query rows into LDS ([32][D], the K tile layout: 16-byte
// chunk c of row r at c ^ (r % (D/8))), so that they are read like a K half.
// Rows at or past rows_left repeat the last valid row.
// With all 32 rows valid, the short form of issue_tile's K (rows for keys).
template <int D>
__device__ __forceinline__ void issue_q(FB_LDS char* dst, const bf16* q_rows, int rows_left, int lane) {
  constexpr int kCpr = D / 8, kKpi = 64 / kCpr;
  if (rows_left >= 32) {
    const int key_l = lane / kCpr, pc = lane % kCpr;
    const uint32_t row_b = key_l * D * 2, k_c = (pc ^ key_l) * 16;
#pragma unroll
    for (int j = 0; j < 32 * kCpr / 64; ++j)
      dma16s<0>(dst + j * 1024, q_rows + (int64_t)(kKpi * j) * D, row_b + (k_c ^ (((kKpi * j) & (kCpr - 1)) * 16)));
    return;
  }
#pragma unroll
  for (int j = 0; j < 32 * kCpr / 64; ++j) {
    const int pos = j * 64 + lane, r = pos / kCpr, pc = pos % kCpr;
    const bf16* src = q_rows + (int64_t)min(r, rows_left - 1) * D + (pc ^ (r & (kCpr - 1))) * 8;
    dma16<0>(dst + j * 1024, src);
  }
}


}  // namespace fbk
