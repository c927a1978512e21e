// bf16 attention kernel for gfx950 (CDNA4).
//
// One workgroup = ROWW x KSPLIT wave64.  The ROWW row-waves own 32 packed
// query rows each of one (sequence, kv head) group; with KSPLIT = 2 a second
// set of ROWW waves takes the same rows and the other 32-key half of every
// tile, so two independent waves share each SIMD and one's softmax overlaps
// the other's MFMAs.  The two halves' (O, m, sum) are merged in LDS at the end.
//
// K/V 64-key tiles stream from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging) through a ring of kStages
// buffers, so kStages-1 tiles are in flight per workgroup.  Each wave computes
// S^T = K Q^T (K rows read with ds_read_b128) and O^T += V^T P^T, the V^T
// operand coming from row-major LDS through the transposing
// ds_read_b64_tr_b16.  The softmax runs in the log2 domain in fp32.
//
// LDS layout of one stage: K tile [64][D] then V tile [64][D], bf16, both
// row-major in 16-byte chunks with an XOR swizzle chosen on the global side
// (each lane of a DMA load writes a fixed LDS slot, so the lane picks which
// global chunk to fetch):
//   K: chunk c of key k at c ^ (k % (D/8))       (16 rows, one chunk column: all banks)
//   V: chunk c of key k at c ^ (4(k % 4) % (D/8)) (4 rows x 64 B of a transposed read: all banks)
#include <algorithm>
#include <atomic>
#include <cstdlib>

#include "fb_combine.h"
#include "fb_device.h"
#include "fb_lds.h"

namespace fbk {

namespace {

// Epilogue of a partial through LDS: normalise, write this wave's 32 rows to
// `st` (row-major, 16-byte chunk c of row r at c ^ (r % (D/4))), read them
// back as whole rows and store D/4 lanes per row.  nrows = valid rows.
// COH (the single-launch step): the partials are stored as device-coherent
// relaxed atomics (past the XCD's L2), for a combine in the same launch.
template <int D, bool COH>
__device__ __forceinline__ void store_partial_rows(const AttnParams& p, const f32x16 (&o)[D / 32], float m,
                                                   float ltot, int split, int64_t grow0, int nrows,
                                                   FB_LDS float* st, int lane) {
  constexpr int kC = D / 4;                 // 16-byte chunks per fp32 row
  constexpr int kRowsPerOp = 64 / kC;
  const int rl = lane & 31, hl = lane >> 5;
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  const float lse = ltot > 0.0f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int c = 8 * dt + 2 * gq + hl;
      const f32x4 v4 = {o[dt][4 * gq] * inv, o[dt][4 * gq + 1] * inv, o[dt][4 * gq + 2] * inv,
                        o[dt][4 * gq + 3] * inv};
      *reinterpret_cast<FB_LDS f32x4*>(st + rl * D + ((c ^ (rl & (kC - 1))) * 4)) = v4;
    }
  }
  // streaming stores: the partials leave this launch for the combine, and
  // kept out of L2 they need no write-back when the launch ends
  if (hl == 0 && rl < nrows) {
    float* dl = p.part_l + split * p.part_l_stride + grow0 + rl;
    if constexpr (COH) __hip_atomic_store(dl, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else __builtin_nontemporal_store(lse, dl);
  }
  bf16* od = reinterpret_cast<bf16*>(p.part_o) + split * p.part_o_stride + grow0 * D;
#pragma unroll
  for (int k = 0; k < 32 / kRowsPerOp; ++k) {
    const int r = k * kRowsPerOp + lane / kC, c = lane % kC;
    const f32x4 v = *reinterpret_cast<const FB_LDS f32x4*>(st + r * D + ((c ^ (r & (kC - 1))) * 4));
    const bf16x4 vb = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    if (r < nrows) {
      bf16x4* dst = reinterpret_cast<bf16x4*>(od + (int64_t)r * D + 4 * c);
      if constexpr (COH)
        __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), __builtin_bit_cast(uint64_t, vb), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        __builtin_nontemporal_store(vb, dst);
    }
  }
}

// LDS bytes of the end-of-loop exchange between the two key halves: per row
// wave, 4 D/32 + 1 chunks of 16 bytes per lane (O, then m and the sum).
template <int D, int ROWW>
constexpr int xch_bytes() { return ROWW * (4 * (D / 32) + 1) * 64 * 16; }

// AUX: cache policy of the K/V DMA loads (see issue_tile).  ONE: the launch
// gives every item at most one key tile (short blocks), so the loop body runs
// once at most and carries no refill.
// One work item of a workgroup (it.ok): the attention of its rows over its
// key range, and its epilogue.
template <int D, int ROWW, int KSPLIT, int MODE, bool PREFETCH_EXT, bool LIST, int AUX, bool ONE, bool COH = false>
__device__ __forceinline__ void attn_body(const AttnParams& p, const AttnItem& it) {
  constexpr int WAVES = ROWW * KSPLIT;
  constexpr int NH = 2 / KSPLIT;   // 32-key halves of a tile per wave
  using P = Pipe<D, WAVES>;
  constexpr int kDt = D / 32;
  constexpr int kAux = AUX;
  extern __shared__ char smem_raw[];
  FB_LDS char* lds = (FB_LDS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave % ROWW, kh = wave / ROWW;
  const int rl = lane & 31, hl = lane >> 5;
  const int b = it.b, g = it.g, grp = p.grp;
  const int key_begin = it.key_begin, key_end = it.key_end;
  const int ntiles_all = key_end > key_begin ? (key_end - key_begin + kKeyTile - 1) / kKeyTile : 0;
  const int ntiles = ONE ? min(ntiles_all, 1) : ntiles_all;
  const int row0 = it.rt * ROWW * 32 + rw * 32;
  const int row = row0 + rl;
  const bool row_ok = row < p.rows;
  const bool wave_live = row0 < p.rows;
  const int64_t grow = (int64_t)(b * p.hq + g * grp) * p.bs + row;
  const int bh = b * p.hq + g * grp + (row_ok ? row / p.bs : 0);

  const bf16* qg = reinterpret_cast<const bf16*>(p.q);
  // keys of the item: the prefix (or the merge launch's block), or a fused
  // step's block for its block-internal items
  const int64_t kv_cap = it.internal ? p.bs : p.kv_cap;
  const bf16* kb = reinterpret_cast<const bf16*>(it.internal ? p.kblk : p.k) + ((int64_t)b * p.hkv + g) * kv_cap * D;
  const bf16* vb = reinterpret_cast<const bf16*>(it.internal ? p.vblk : p.v) + ((int64_t)b * p.hkv + g) * kv_cap * D;
  const TileMap<LIST> tm = tile_map<LIST>(p, it);
  const int lim = tm.lim;

  // Prologue loads, none waiting on another: the merge's head flags, then Q
  // and the first two tiles (more would only queue behind them in the memory
  // system while the first is awaited), all three through the LDS DMA path.
  // Q goes through LDS rather than straight into registers because the
  // compiler, which counts its register loads but not the DMA loads, would
  // wait for Q with counts that drain the whole ring (except in the
  // lone-wave merge launch, see below).
  ExtPart<D> ext;
  const bool ext_lane = MODE == kModeMerge && row_ok && kh == 0;
  if (ext_lane) {
    ext.load_state(p, bh);
    if constexpr (PREFETCH_EXT) ext.load_data(p, grow, hl);   // in flight with Q and the tiles
  }
  // The lone-wave merge launch (blocks of fewer than 512 packed rows) loads Q
  // straight into registers, in flight with everything else: issued before
  // the tiles, those loads have landed once the first tile has.
  constexpr bool kQReg = MODE == kModeMerge && ROWW == 1 && PREFETCH_EXT;
  bf16x8 qf[D / 16];
  FB_LDS char* q_lds = lds + P::q_offset(P::ring_stages(p.ring_keys), ROWW) + rw * 32 * D * 2;
  if constexpr (kQReg) {
    const bf16* qrow = qg + (grow - rl + min(rl, p.rows - row0 - 1)) * D + 8 * hl;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = *reinterpret_cast<const bf16x8*>(qrow + 16 * t);
  } else {
    if (kh == 0 && wave_live) issue_q<D>(q_lds, qg + (grow - rl) * D, p.rows - row0, lane);
  }
  int issued;
  if (ntiles >= 2) {
    issue_tile<D, WAVES, kAux>(lds, kb, vb, tm.key0(0), lim, wave, lane);
    issue_tile<D, WAVES, kAux>(lds + P::kStageBytes, kb, vb, tm.key0(1), lim, wave, lane);
    issued = 2;
    wait_vmcnt<P::kLpt>();   // tile 0 (and everything issued before it) landed
  } else if (ntiles == 1) {
    issue_tile<D, WAVES, kAux>(lds, kb, vb, tm.key0(0), lim, wave, lane);
    issued = 1;
    wait_vmcnt<0>();
  } else {
    issued = 0;
    wait_vmcnt<0>();
  }
  if constexpr (kQReg) {
    // Q's register loads were issued before the tiles, so they have landed;
    // the compiler, which does not count the DMA loads, would otherwise wait
    // for them inside the loop with counts that drain the ring every tile.
#pragma unroll
    for (int t = 0; t < D / 16; ++t) asm volatile("" : "+v"(qf[t]));
  }
  lds_barrier();   // every wave's share of tile 0 (and Q) landed
  // Q^T as the B operand: lane (row, hl) holds Q[row][16t + 8hl .. +7].
  if constexpr (!kQReg) {
    uint32_t qa[D / 16];
    const uint32_t q0 = (uint32_t)(uintptr_t)q_lds;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qa[t] = q0 + rl * D * 2 + (((2 * t + hl) ^ (rl & (P::kCpr - 1))) * 16);
    u32x4 qr[D / 16];
    k_read_half<D, 0>(qr, qa);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = __builtin_bit_cast(bf16x8, qr[t]);
  }
  // When Q sits in ring stages 2-3, every wave must have read it before the
  // first refill writes there (past the ring it needs no barrier).
  if (!P::q_past(ROWW) && P::ring_stages(p.ring_keys) == P::kStages) lds_barrier();

  f32x16 o[kDt];
#pragma unroll
  for (int i = 0; i < kDt; ++i) o[i] = f32x16{};
  float m = -INFINITY, lsum = 0.0f;

  // Per-lane byte offsets of the transposed V reads inside a V tile.  In a
  // 16-lane group tg, lane 4j + q addresses 4 columns of key 4hl + j (plus
  // 16ks + 8hf); the instruction hands lane i the column 16(tg%2) + i of the
  // 4 keys, i.e. the A-operand layout of V^T for head-dim tile dt.
  uint32_t tr_off[kDt];
  {
    const int tg = lane >> 4, tj = (lane & 15) >> 2, tq = lane & 3;
    const int key = 4 * hl + tj;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      const int cl = 4 * dt + 2 * (tg & 1) + (tq >> 1);
      const int pc = cl ^ ((4 * key) & (P::kCpr - 4));
      tr_off[dt] = key * D * 2 + pc * 16 + (tq & 1) * 8;
    }
  }
  // Per-lane byte offsets of the K reads (key rl of a 32-key half, 16-byte
  // chunk 2t + hl); half c is 32c rows further.
  uint32_t k_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) k_off[t] = rl * D * 2 + (((2 * t + hl) ^ (rl & (P::kCpr - 1))) * 16);

  // Single-wave workgroups serve short blocks: a second key half that holds
  // no key is skipped (wave-uniform; compiled only there, where registers allow).
  constexpr bool kShortSkip = ROWW == 1 && NH == 2;
  const uint32_t lds_off = (uint32_t)(uintptr_t)lds;
  for (int t_i = 0; t_i < ntiles; ++t_i) {
    if (t_i > 0) {
      wait_tile<P::kLpt, P::kStages>(issued - t_i - 1);   // tiles issued after this one may stay in flight
      lds_barrier();   // every wave's share landed; all waves finished tile t_i-1
    }
    if (wave_live) {
      const int tile0 = tm.key0(t_i);
      const uint32_t ks_off = lds_off + (t_i % P::kStages) * P::kStageBytes;
      const uint32_t vs_off = ks_off + P::kTensorBytes;
      // S^T = K Q^T per 32-key half: the half's K fragments, then its MFMA
      // chain over the head dimension (LDS byte addresses of the fragments).
      uint32_t ka[D / 16];
#pragma unroll
      for (int t = 0; t < D / 16; ++t) ka[t] = ks_off + k_off[t];
      f32x16 s[NH];
      const int nh_live = (kShortSkip && tile0 + 32 >= lim) ? 1 : NH;
      uint32_t vbase[kDt];
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) vbase[dt] = vs_off + tr_off[dt];
      u32x2 vr[D / 8];
      u32x2 vr1[D / 8];
      if constexpr (NH == 2 && ROWW > 1) {
        // Whole tiles: the K fragments of both halves (in the order the two
        // interleaved S chains use them) and then both halves' V^T operands
        // are read while the S MFMAs run; the scheduler is told to issue a
        // few LDS reads after every MFMA, so the reads hide under the MFMAs
        // and the compiler waits for each fragment only where it is used.
        u32x4 kf0[D / 16], kf1[D / 16];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          kf0[t] = lds_b128(ka[t]);
          kf1[t] = lds_b128(ka[t] + 32 * D * 2);
        }
        tr_read_both<D>(vr, vr1, vbase);
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf0[t]), qf[t], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf1[t]), qf[t], s[1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // the first LDS reads
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // then up to three LDS reads
        }
      } else if constexpr (NH == 1) {
        // Key halves: this wave's half of K and of V^T read under its S
        // MFMAs, as above (the half's offset added, not branched on, so that
        // the reads and the MFMAs share one scheduling region).
        const uint32_t hoff = kh * (32 * D * 2);
        uint32_t kh_a[D / 16], kh_v[kDt];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) kh_a[t] = ka[t] + hoff;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) kh_v[dt] = vbase[dt] + hoff;
        u32x4 kf[D / 16];
        k_read_half<D, 0>(kf, kh_a);
        tr_read_half<D, 0>(vr, kh_v);
        s[0] = f32x16{};
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[t]), qf[t], s[0], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // the first LDS reads
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // then up to three LDS reads
        }
      } else {
        // The lone wave of short blocks: half 0's K and V^T read under its S
        // MFMAs (as above; half 1's V^T is read after its exponentials), and
        // a half 1 with no key is skipped.
        u32x4 kf[D / 16];
        k_read_half<D, 0>(kf, ka);
        tr_read_half<D, 0>(vr, vbase);
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[t]), qf[t], s[0], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // the first LDS reads
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // then up to three LDS reads
        }
        if (nh_live > 1) {
          u32x4 kf1[D / 16];
          k_read_half<D, 32 * D * 2>(kf1, ka);
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf1[t]), qf[t], s[1], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);   // all its K reads (one wait),
          __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);   // then its MFMAs
        }
      }
      // Ragged last tile: keys at or past the limit do not count.  In the
      // single-wave kernels (short blocks: often one tile, often half full) a
      // half with no key is filled whole and a full half left alone; the
      // multi-wave loops keep the plain form, whose code schedules better.
      const int key0 = tile0 + 32 * kh * NH;
      if (key0 + 32 * NH > lim) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          if constexpr (kShortSkip) {
            if (key0 + 32 * h + 32 <= lim || h >= nh_live) continue;   // full, or skipped below
            if (key0 + 32 * h >= lim) {
#pragma unroll
              for (int j = 0; j < 16; ++j) s[h][j] = -INFINITY;
              continue;
            }
          }
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (key0 + 32 * h + 8 * (j >> 2) + 4 * hl + (j & 3) >= lim) s[h][j] = -INFINITY;
        }
      }
      // Row max of this wave's keys (log2 units); the running max is raised
      // only when it grows by more than 2^kRescale (see softmax_halves), so
      // the O rescale below rarely runs after the first tile.
      {
        float mx = -INFINITY;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          if (kShortSkip && h >= nh_live) continue;   // a half with no key: never exponentiated
#pragma unroll
          for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[h][j]);
        }
        mx = pair_max(mx) * p.scale_log2;
        const bool raise = mx > m + kRescale;
        if (kShortSkip && t_i == 0) {
          m = raise ? mx : m;   // first tile: O and the sum are still zero, nothing to rescale
        } else if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float m_new = raise ? mx : m;
          const float alpha = fast_exp2(m - m_new);
          m = m_new;
          lsum *= alpha;
#pragma unroll
          for (int i = 0; i < kDt; ++i) o[i] *= alpha;
        }
      }
      const float mref = m > -INFINITY ? m : 0.0f;   // a row with no key yet (second half of a short block)
      bf16x8 pb0[2];
      exp_half(s[0], mref, p.scale_log2, lsum, pb0);
      if (kShortSkip && nh_live == 1) {
        pv_half<kDt>(o, vr, pb0);   // the second half holds no key (short block)
      } else if constexpr (NH == 2 && ROWW > 1) {
        // half 1's V^T was read with half 0's, under the S MFMAs; its
        // exponentials are interleaved with half 0's PV MFMAs
        bf16x8 pb1[2];
        pv_half<kDt>(o, vr, pb0);
        exp_half(s[NH - 1], mref, p.scale_log2, lsum, pb1);
#pragma unroll
        for (int i = 0; i < 2 * kDt; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // then VALU
        }
        pv_half<kDt>(o, vr1, pb1);
      } else if constexpr (NH == 2) {
        // half 1's exponentials are interleaved with half 0's PV MFMAs
        bf16x8 pb1[2];
        pv_half<kDt>(o, vr, pb0);
        exp_half(s[NH - 1], mref, p.scale_log2, lsum, pb1);
#pragma unroll
        for (int i = 0; i < 2 * kDt; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // then VALU
        }
        tr_read_half<D, 1>(vr, vbase);
        pv_half<kDt>(o, vr, pb1);
      } else {
        pv_half<kDt>(o, vr, pb0);
      }
    }
    // Refill after the compute, so that a stalled issue does not delay it:
    // the stage of tile t_i-1 is free (every wave passed the barrier above).
    if constexpr (!ONE) {
      for (; issued < ntiles && issued <= t_i + P::kStages - 1; ++issued)
        issue_tile<D, WAVES, kAux>(lds + (issued % P::kStages) * P::kStageBytes, kb, vb, tm.key0(issued), lim, wave,
                                   lane);
    }
  }

  if constexpr (KSPLIT == 2) {
    // Merge the two key halves of each row: the second wave set hands its
    // (O, m, lane sum) to the first through LDS, 16 bytes per lane and
    // instruction (chunk c of lane l at c*64 + l).  No DMA is in flight here
    // (the last tile waited for vmcnt 0), so the ring can be reused.
    constexpr int kChunks = 4 * kDt + 1;
    FB_LDS f32x4* xch = (FB_LDS f32x4*)lds + rw * kChunks * 64 + lane;
    lds_barrier();
    if (kh == 1 && wave_live) {
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xch[(4 * dt + q) * 64] = f32x4{o[dt][4 * q], o[dt][4 * q + 1], o[dt][4 * q + 2], o[dt][4 * q + 3]};
      }
      xch[(4 * kDt) * 64] = f32x4{m, lsum, 0.0f, 0.0f};
    }
    lds_barrier();
    if (kh == 1) return;
    if (wave_live) {
      const f32x4 ml = xch[(4 * kDt) * 64];
      const float m2 = ml[0], l2 = ml[1];
      const float mt = fmaxf(m, m2);
      const float a1 = m > -INFINITY ? fast_exp2(m - mt) : 0.0f;
      const float a2 = m2 > -INFINITY ? fast_exp2(m2 - mt) : 0.0f;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = xch[(4 * dt + q) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[dt][4 * q + e] = a1 * o[dt][4 * q + e] + a2 * v[e];
        }
      }
      lsum = a1 * lsum + a2 * l2;
      m = mt;
    }
  }

  if constexpr (MODE == kModePartial) {
    // Stage the wave's 32 normalised rows in its own LDS region (row-major,
    // 16-byte chunks XOR-swizzled by row) and store whole rows: each store
    // instruction then writes 1 KB of contiguous partials instead of 32
    // scattered 32-byte pieces.  Waves use disjoint regions, so after the
    // ring is released (barrier below, or the exchange above) no further
    // synchronisation is needed.
    if constexpr (KSPLIT == 1) lds_barrier();   // every wave finished reading the ring
    if (!wave_live) return;
    const float ltot = pair_sum(lsum);
    constexpr int kRegionFloats = KSPLIT == 2 ? (4 * kDt + 1) * 64 * 4 : 32 * D;
    store_partial_rows<D, COH>(p, o, m, ltot, it.split, grow - rl, min(32, p.rows - row0),
                          (FB_LDS float*)lds + rw * kRegionFloats, lane);
    return;
  }
  const float ltot = pair_sum(lsum);
  if (!row_ok) return;
  {
    if constexpr (!PREFETCH_EXT) ext.load_data(p, grow, hl);
    merge_store<bf16, D>(p, o, m, ltot, ext, grow, hl);
    // The decision record goes last: a store issued before the merge would
    // hold up its wait for the cached part's loads (one counter for both).
    if (p.reuse_rec != nullptr && hl == 0 && (row % p.bs) == 0) p.reuse_rec[bh] = head_selected(p.sel, b, bh) ? 0 : 1;
  }
}

template <int D, int ROWW, int KSPLIT, int MODE, bool PREFETCH_EXT, bool LIST, int AUX, bool ONE>
__global__ __launch_bounds__(64 * ROWW * KSPLIT) void attn_bf16_kernel(const AttnParams p) {
  prefetch_params(p);
  // ONE: a 3-D grid (row tile, kv head, sequence), one key range per group
  const AttnItem it = ONE ? grid_item(p) : attn_item(p, MODE == kModePartial);
  if constexpr (MODE == kModePartial) record_decisions(p);
  if (!it.ok) return;   // workgroup-uniform: no selected head, or past the device plan's items
  attn_body<D, ROWW, KSPLIT, MODE, PREFETCH_EXT, LIST, AUX, ONE>(p, it);
}

// Single-launch fused step (see FinParams).  A combine workgroup polls its
// group's counter every s_sleep 16 (about 0.5 us) and gives up after
// kFinSpin polls (about 0.3 s in all): it sets the error flag and folds what
// it finds.  One lane per workgroup touches a counter, each counter on a
// line of its own.
constexpr int kFinSpin = 1 << 19;

// An attention workgroup is done with its item: every wave waits until its
// partial stores (device-coherent) have completed, then the workgroup counts
// itself in its group.
__device__ __forceinline__ void fin_arrive(const FinParams& f, int group) {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(f.ctr + (kFinCounters + group) * kFinStride, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Combine item c = (query head, chunk): the workgroup waits for its group's
// attention items, each wave folds its rows (the combine kernel's fold, rows
// 256/D * (chunk * WAVES + wave) ..), and the workgroup counts itself out;
// the group's last combine workgroup returns the counter to zero.
template <int D, int WAVES, int BATCH>
__device__ __forceinline__ void fin_combine(const FinParams& f, int c) {
  const CombineParams& p = f.cp;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int bh = c / f.chunks, chunk = c - bh * f.chunks;
  const int b = bh / p.hq, h = bh - b * p.hq;
  const int gi = b * p.hkv + h / (p.hq / p.hkv);
  uint32_t* cnt = f.ctr + (kFinCounters + gi) * kFinStride;
  uint32_t need = f.need, done_all = f.done_all;
  if (p.dyn.groups > 0) {   // the device plan: what the attention workgroups derived, from the same flags
    const uint64_t mask = active_groups(p.sel, p.dyn.groups, p.hq, p.hkv);
    const bool act = (mask >> gi) & 1;
    if (f.merge_reused && !act) return;   // the block-internal items finished the group
    const int splits = act ? p.dyn.splits[__builtin_popcountll(mask)] : 0;
    need = (uint32_t)((splits + 1) * f.row_tiles);
    done_all = need + (uint32_t)((p.hq / p.hkv) * f.chunks);
  } else if (f.merge_reused && !group_selected(p.sel, b, h / (p.hq / p.hkv), p.hq, p.hq / p.hkv)) {
    return;
  }
  if (threadIdx.x == 0) {
    for (int i = 0;; ++i) {
      if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) break;
      if (i == kFinSpin) {
        __hip_atomic_fetch_or(f.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(16);
    }
  }
  __syncthreads();   // the partials are read (device-coherent loads) after the arrivals were seen
  const int ch = chunk * WAVES + wave;
  if (ch < p.row_chunks) combine_fold<D, BATCH, true, true>(p, ch, bh, b, lane);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t o = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (o + 1 == done_all) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int D, int ROWW, int KSPLIT, int AUX, int BATCH>
__global__ __launch_bounds__(64 * ROWW * KSPLIT) void attn_fin_kernel(const AttnParams p, const FinParams f) {
  prefetch_params(p);
  prefetch_params(f);
  if ((int)blockIdx.x < f.n_attn) {   // workgroup-uniform
    const AttnItem it = attn_item<false>(p, true, blockIdx.x, f.n_attn);   // dense keys only
    record_decisions(p);
    // A group with no selected head (block-internal items; static-plan split
    // items, which the device plan does not enumerate): its block-internal
    // items merge with the cache and store the output, as the merge launch
    // does; nothing waits for the group.
    if (f.merge_reused && (it.internal || p.dyn.groups == 0) &&
        !(it.internal ? group_selected(p.sel, it.b, it.g, p.hq, p.grp) : it.ok)) {
      if (it.internal) attn_body<D, ROWW, KSPLIT, kModeMerge, false, false, AUX, false>(p, it);
      return;
    }
    if (it.ok) attn_body<D, ROWW, KSPLIT, kModePartial, false, false, AUX, false, true>(p, it);
    // static plan: every item of a selected group counts (and, without
    // merge_reused, those of the other groups too); device plan: the items
    // past the active groups' belong to no group
    if (it.ok || p.dyn.groups == 0) fin_arrive(f, it.b * p.hkv + it.g);
  } else {
    fin_combine<D, ROWW * KSPLIT, BATCH>(f, blockIdx.x - f.n_attn);
  }
}

template <int D, int ROWW, int KSPLIT, int MODE, bool PF, bool LIST, int AUX, bool ONE = false>
hipError_t launch_one(const AttnParams& p, hipStream_t s) {
  using P = Pipe<D, ROWW * KSPLIT>;
  const int blocks = p.grid > 0 ? p.grid : p.batch * p.hkv * p.splits * p.row_tiles;
  if (blocks == 0) return hipSuccess;
  const dim3 grid = ONE ? dim3(p.row_tiles, p.hkv, p.batch) : dim3(blocks);
  constexpr int kStageOut = MODE == kModePartial ? ROWW * 32 * D * 4 : 0;   // partial staging (KSPLIT 1)
  constexpr int kQBytes = ROWW * 32 * D * 2;
  constexpr int kMaxLds = std::max({P::kLdsBytes, P::q_offset(P::kStages, ROWW) + kQBytes,
                                    (P::kStages - 1) * P::kStageBytes + kQBytes,
                                    KSPLIT == 2 ? xch_bytes<D, ROWW>() : 0, kStageOut});
  // The LDS limit is raised once per device (a bit per device id below 64;
  // others set it at every launch).  Two threads may both set it: harmless.
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (bit == 0 || (attr_done.load(std::memory_order_acquire) & bit) == 0) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_bf16_kernel<D, ROWW, KSPLIT, MODE, PF, LIST, AUX, ONE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  // a workgroup never uses more ring stages than its key range has tiles
  const int ring = P::ring_stages(p.ring_keys);
  int lds = std::max(ring * P::kStageBytes, P::q_offset(ring, ROWW) + kQBytes);
  if (KSPLIT == 2) lds = std::max(lds, xch_bytes<D, ROWW>());
  lds = std::max(lds, kStageOut);
  hipLaunchKernelGGL((attn_bf16_kernel<D, ROWW, KSPLIT, MODE, PF, LIST, AUX, ONE>), grid, dim3(64 * ROWW * KSPLIT),
                     lds, s, with_div_magic(p, blocks));
  return hipGetLastError();
}

template <int D, int ROWW, int KSPLIT, int BATCH>
hipError_t launch_fin(const AttnParams& p, const FinParams& f, hipStream_t s) {
  using P = Pipe<D, ROWW * KSPLIT>;
  constexpr int kStageOut = ROWW * 32 * D * 4;
  constexpr int kQBytes = ROWW * 32 * D * 2;
  constexpr int kMaxLds = std::max({P::kLdsBytes, P::q_offset(P::kStages, ROWW) + kQBytes,
                                    (P::kStages - 1) * P::kStageBytes + kQBytes,
                                    KSPLIT == 2 ? xch_bytes<D, ROWW>() : 0, kStageOut});
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (bit == 0 || (attr_done.load(std::memory_order_acquire) & bit) == 0) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_fin_kernel<D, ROWW, KSPLIT, 2, BATCH>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  const int ring = P::ring_stages(p.ring_keys);
  int lds = std::max(ring * P::kStageBytes, P::q_offset(ring, ROWW) + kQBytes);
  if (KSPLIT == 2) lds = std::max(lds, xch_bytes<D, ROWW>());
  lds = std::max(lds, kStageOut);
  hipLaunchKernelGGL((attn_fin_kernel<D, ROWW, KSPLIT, 2, BATCH>), dim3(f.n_total), dim3(64 * ROWW * KSPLIT), lds, s,
                     with_div_magic(p, f.n_attn), f);
  return hipGetLastError();
}

template <int D, int ROWW, int KSPLIT>
hipError_t launch_fin_batch(const AttnParams& p, const FinParams& f, hipStream_t s) {
  // the combine kernel's round size: the largest split count of the plan
  int most = f.cp.splits;
  for (int n = 1; n <= f.cp.dyn.groups; ++n) most = std::max(most, (int)f.cp.dyn.splits[n]);
  if (most <= 8) return launch_fin<D, ROWW, KSPLIT, 8>(p, f, s);
  if (most <= 16) return launch_fin<D, ROWW, KSPLIT, 16>(p, f, s);
  return launch_fin<D, ROWW, KSPLIT, 32>(p, f, s);
}

// Streaming K/V: in a partial launch with one row tile per group every K/V
// tile is read by exactly one workgroup, so its loads are marked
// non-temporal (AUX 2); with several row tiles (frame-sized blocks) each tile
// is re-read from L2 by every row tile and keeps the default policy.
template <int D, int MODE, bool PF_SMALL, bool LIST, int AUX>
hipError_t launch_aux(const AttnParams& p, hipStream_t s) {
  if (p.waves == 8 && p.ksplit == 1) return launch_one<D, 8, 1, MODE, false, LIST, AUX>(p, s);
  if (p.waves == 8 && p.ksplit == 2) return launch_one<D, 4, 2, MODE, false, LIST, AUX>(p, s);
  if (p.waves == 4 && p.ksplit == 1) return launch_one<D, 4, 1, MODE, false, LIST, AUX>(p, s);
  // block-internal attention of a block of at most one key tile
  if (MODE == kModeMerge && p.ring_keys <= kKeyTile) return launch_one<D, 1, 1, MODE, PF_SMALL, LIST, AUX, true>(p, s);
  return launch_one<D, 1, 1, MODE, PF_SMALL, LIST, AUX>(p, s);
}
template <int D, int MODE, bool PF_SMALL, bool LIST>
hipError_t launch_shape(const AttnParams& p, hipStream_t s) {
  if constexpr (MODE == kModePartial) {
    if (p.row_tiles == 1) return launch_aux<D, MODE, PF_SMALL, LIST, 2>(p, s);
  }
  return launch_aux<D, MODE, PF_SMALL, LIST, 0>(p, s);
}

// Tile lists occur in partial launches only (sparse steps).
template <int D, int MODE, bool PF_SMALL>
hipError_t launch_mode(const AttnParams& p, hipStream_t s) {
  if constexpr (MODE == kModePartial) {
    if (p.tiles != nullptr) return launch_shape<D, MODE, PF_SMALL, true>(p, s);
  }
  return launch_shape<D, MODE, PF_SMALL, false>(p, s);
}

}  // namespace

// The 64-row-per-wave kernel can take the partial launches of the
// 8-row-wave shape (groups of more than 128 packed rows; the same 256 rows
// per workgroup, so the same split plan) over dense prefix keys at head dim
// 128.  Off unless FB_ATTN_R64=1: measured slower than the 32-row kernel.
static bool r64_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("FB_ATTN_R64");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

hipError_t launch_attn_bf16(int head_dim, int mode, const AttnParams& p, hipStream_t s) {
  if (head_dim == 128 && mode == kModePartial && p.tiles == nullptr && p.waves == 8 && p.ksplit == 1 && r64_enabled())
    return launch_attn_r64(p, s);
  if (head_dim == 64)
    return mode == kModePartial ? launch_mode<64, kModePartial, false>(p, s) : launch_mode<64, kModeMerge, true>(p, s);
  return mode == kModePartial ? launch_mode<128, kModePartial, false>(p, s) : launch_mode<128, kModeMerge, true>(p, s);
}

bool fin_supported(int dtype, int head_dim, const AttnParams& p) {
  const bool shape = (p.waves == 8 && p.ksplit == 1) || (p.waves == 8 && p.ksplit == 2) ||
                     (p.waves == 4 && p.ksplit == 1);
  return dtype == FB_BF16 && head_dim == 128 && shape && p.row_tiles == 1 && p.tiles == nullptr &&
         p.int_count > 0;
}

hipError_t launch_attn_fin(const AttnParams& p, const FinParams& f, hipStream_t s) {
  if (!fin_supported(FB_BF16, 128, p) || f.row_tiles != p.row_tiles || f.cp.dyn.groups != p.dyn.groups)
    return hipErrorNotSupported;
  if (p.waves == 8 && p.ksplit == 1) return launch_fin_batch<128, 8, 1>(p, f, s);
  if (p.waves == 8 && p.ksplit == 2) return launch_fin_batch<128, 4, 2>(p, f, s);
  return launch_fin_batch<128, 4, 1>(p, f, s);
}

}  // namespace fbk
