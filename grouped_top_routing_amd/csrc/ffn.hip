// Expert SwiGLU MLPs of the Beam-1.0 MoE block as two bf16 grouped GEMMs on
// the gfx950 matrix cores.
//
// "Welcome Beam: a 501B open model you can own, customize, and scale", section
// "Mixture of Experts": each of the 256 experts is a SwiGLU MLP with
// intermediate size 2,560 (hidden 5,120); section "Residual Stream": the SwiGLU
// product is computed in FP32.
//
//   gate/up:  h[r, :] = bf16( SiLU(g) * u ),  g = A_r . Wg_e^T,  u = A_r . Wu_e^T
//             A_r = x[perm_src[r] / topk]   (row gather fused into the A load)
//   down:     y[r, :] = bf16( h_r . Wd_e^T )
//
// At every Beam batch size up to a few thousand tokens these GEMMs are bound
// by streaming the touched experts' weights from HBM (a 4096-token chunk puts
// ~128 rows on each expert: ~127 FLOP per weight byte, under the MI355X ridge
// of ~315), so the kernel is built around keeping HBM busy:
//
// * Weights and activations go global -> LDS with gfx950's direct loads
//   (global_load_lds_dwordx4: 64 lanes x 16 B into 1 KB of LDS, no VGPRs),
//   through rings of LDS slots: 64-row tiles stage 32 k of weights and rows
//   per slot; bf16 128..256-row tiles keep weights in 32-k slots and rows in
//   64-k slots (schedule in half_ring.h); fp8 128/192-row tiles run 64-k
//   stages.  Each wave waits on its own vmcnt and a workgroup barrier
//   publishes each step to the other waves.
// * One 1 KB weight "fragment" is exactly one MFMA operand (16 rows x 32 k,
//   bf16): lane l fetches row l%16, k chunk (l/16)*8, and later reads the
//   same 16 bytes back with a conflict-free ds_read_b128 at lane*16.  The
//   gathered A rows are staged the same way for 64-row tiles, and 64 k at a
//   time in whole 128-byte lines for larger tiles (layout below).  Every
//   operand is read in the v_mfma_f32_16x16x32_bf16 lane order, so A and B
//   lanes always carry matching k.
// * A work item is one (m-tile, n-tile) pair.  A device-built plan cuts each
//   expert's rows into balanced m-tiles of at most 16*MB rows, so at Beam's
//   prefill size an expert's rows fit one m-tile and its weights are fetched
//   once.  Each wave computes NCBW 16-column weight blocks (for gate/up:
//   NCBW/2 gate blocks and the matching up blocks, so the SwiGLU epilogue is
//   wave-local) for its share of the item's rows (see the work split below).
// * A persistent grid walks the items.  Workgroup b runs on XCD b % 8; items
//   are dealt so that the n-tiles of one m-tile land on one XCD in the same
//   round, sharing the gathered A rows through that XCD's L2 (at 256-row
//   tiles the gate/up GEMM deals blocks of 8 m-tiles x 4 n-tiles of one
//   expert instead, item_order.h, and aligns each XCD's rounds).  In the
//   128..256-row configurations a workgroup issues the first weight loads of
//   its next item before the current item's epilogue, so its weight stream
//   keeps running while the outputs are written.
// * Wave-level values (wave index, wait counts, weight row bases) are kept in
//   scalar registers: every weight load takes a 64-bit base in SGPRs and one
//   32-bit lane offset, and the run-time vmcnt waits branch on scalars.
#include <stdlib.h>

#include "common.h"
#include "half_ring.h"
#include "item_order.h"
#include "kernels.h"

namespace beam {

// Pipeline shape.  The defaults were chosen by timing on MI355X; the macros
// only exist so that other shapes can be built for comparison.
#ifndef BEAM_GEMM_S4
#define BEAM_GEMM_S4 4
#endif
#ifndef BEAM_GEMM_S8
#define BEAM_GEMM_S8 4
#endif
#ifndef BEAM_GEMM_S12
#define BEAM_GEMM_S12 3
#endif
#ifndef BEAM_GEMM_MAXMB
#define BEAM_GEMM_MAXMB 12
#endif
#ifndef BEAM_GEMM_MB16
#define BEAM_GEMM_MB16 1
#endif
#ifndef BEAM_GEMM_S16
#define BEAM_GEMM_S16 3
#endif
#ifndef BEAM_GEMM_DOWN_NT
#define BEAM_GEMM_DOWN_NT 0
#endif
// bf16 weights at 128..256-row tiles: weight ring of half-stage (32-k)
// slots, A ring of SA 64-k slots, and the weight sub-steps of the next item
// issued before the epilogue (0: the 64-k stage pipeline instead)
#ifndef BEAM_GEMM_HALF
#define BEAM_GEMM_HALF 1
#endif
#ifndef BEAM_HALF_SA8
#define BEAM_HALF_SA8 3
#endif
#ifndef BEAM_HALF_SB8
#define BEAM_HALF_SB8 7
#endif
#ifndef BEAM_HALF_SA12
#define BEAM_HALF_SA12 3
#endif
#ifndef BEAM_HALF_SB12
#define BEAM_HALF_SB12 5
#endif
#ifndef BEAM_HALF_SA16
#define BEAM_HALF_SA16 3
#endif
#ifndef BEAM_HALF_SB16
#define BEAM_HALF_SB16 4
#endif
#ifndef BEAM_HALF_KP
#define BEAM_HALF_KP 2
#endif
// refill lag (half_ring.h): 1 drops the per-sub-step wait for the wave's own
// LDS reads before the barrier, at one sub-step less look-ahead (skewed
// 16K-token batch at 256-row tiles: 11.52 -> 11.38 ms; prefill at 192-row
// tiles unchanged, so those keep lag 0 and the deeper look-ahead)
#ifndef BEAM_HALF_LAG8
#define BEAM_HALF_LAG8 0
#endif
#ifndef BEAM_HALF_LAG12
#define BEAM_HALF_LAG12 0
#endif
#ifndef BEAM_HALF_LAG16
#define BEAM_HALF_LAG16 1
#endif
// 256-row tiles (batches whose experts hold > 160 rows on average): the
// gate/up GEMM walks its items in expert blocks of 8 m-tiles x 4 n-tiles per
// XCD and round, and each XCD's workgroups start a round together, so a
// block's workgroups stream their shared weights and rows through L2 at the
// same time (skewed 16K-token batch: gate/up 7.39 -> 6.97 ms; unaligned
// blocks: 7.27 ms; blocks of 4 m-tiles x 8 n-tiles: 7.07 ms).  The down GEMM
// keeps the plain order (blocked: 3.85 -> 3.92 ms aligned, 3.79 unaligned).
// 0: plain order everywhere.
#ifndef BEAM_GEMM_BLOCKED
#define BEAM_GEMM_BLOCKED 1
#endif
// 16-byte epilogue stores (pairs of column blocks regrouped across lane
// rows); 0: 8-byte stores
#ifndef BEAM_EPI_WIDE
#define BEAM_EPI_WIDE 1
#endif
// cache policy bits of the epilogue's stores (0: default)
#ifndef BEAM_STORE_POLICY_GU
#define BEAM_STORE_POLICY_GU 0
#endif
#ifndef BEAM_STORE_POLICY_DOWN
#define BEAM_STORE_POLICY_DOWN 0
#endif
#ifndef BEAM_GEMM_BLOCKED_DOWN
#define BEAM_GEMM_BLOCKED_DOWN 0
#endif
#ifndef BEAM_SYNC_SPIN
#define BEAM_SYNC_SPIN 2048
#endif
#ifndef BEAM_GEMM_NW8
#define BEAM_GEMM_NW8 8
#endif
#ifndef BEAM_GEMM_NW12
#define BEAM_GEMM_NW12 8
#endif
#ifndef BEAM_GEMM_RG8
#define BEAM_GEMM_RG8 2
#endif
#ifndef BEAM_GEMM_RG12
#define BEAM_GEMM_RG12 2
#endif
constexpr int kBKS = 32;                // k per MFMA step (a 64-row tile's pipeline stage)
constexpr int kFrag = 1024;             // bytes of one 16 x 32 bf16 MFMA operand
constexpr int kFragElems = kFrag / 2;
// Output columns of one work item: every configuration covers 128 h columns
// (gate/up) or 256 y columns (down), so the host's item count is config-free.
constexpr int kColsGateUp = 128;
constexpr int kColsDown = 256;

// Everything one work item needs, resolved once per item.
struct ItemArgs {
  const uint16_t* A;
  const int32_t* gather;
  int topk;
  const uint16_t* W;       // this expert's weights (row-major or fragment-packed)
  uint16_t* C;
  int K, n_out, up_row0;
  int packed;              // 1: W is in fragment order (see pack_weights_kernel)
  int row0, nrows, ntile;
  // Optional expert LoRA, second factor: acc += t_r . Lb_e^T before the
  // epilogue, with t [rows, lora_r] (already scaled, permuted row order) and
  // this expert's Lb [n_total, lora_r], both bf16 row-major.  lora_t == null:
  // no adapter.
  const uint16_t* lora_t;
  const uint16_t* lora_b;
  int lora_r;
  // The persistent walk, for configurations that start the workgroup's next
  // item (q + grid, if below total) while this one finishes: item q is
  // (m-tile q / nt_n, n-tile q % nt_n), its expert plan_expert[m-tile], and
  // every item but a workgroup's first (q >= grid) finds its first weight
  // stages already issued.
  const uint16_t* W0;      // expert 0's weights
  int64_t w_expert_stride;
  const int32_t* plan_expert;
  // blocked item order (see item_of): each tile's expert's first m-tile and
  // m-tile count; null for the plain order
  const int32_t* plan_first;
  const int32_t* plan_count;
  int q, grid, total, nt_n;
  // checked builds: permuted rows and rows of A the indices must stay below
  int64_t n_rows, n_src;
  // fp8 weights: this expert's fp32 scale per weight row (W then holds the
  // E4M3FN codes in the fp8 fragment layout); null for bf16 weights
  const float* scale;
};

// Work split inside a workgroup: the kNW waves form RG row groups x CG = kNW /
// RG column groups.  Every item covers 16 weight-row blocks (kColsGateUp gate
// rows and as many up rows, or kColsDown down rows), so a wave owns NCBW = 16 / CG
// column blocks and RB of the item's NRB row blocks.  With RG = 2 each A
// fragment is read from LDS by half the waves and each B fragment by two,
// which cuts LDS read traffic per MFMA against RG = 1 (every wave reading
// every A fragment).
constexpr int kItemBlocks = 16;

// LDS ring layouts.  64-row tiles: S slots of [16 B fragments | MB A
// fragments] per 32-k stage, every A fragment a 16-row x 32-k MFMA operand
// (64 bytes of 16 rows).  128..256-row tiles stage A 64 k at a time so that
// every A load fetches whole 128-byte lines (the half-line loads cost ~10%
// at prefill): per 16-row block a stage's A holds 2 KB, rows 0-7 then rows
// 8-15, each row's 128 bytes with its 16-byte chunks XOR-swizzled by
// (row / 2) % 8 so that the MFMA operand reads (16 rows at one logical
// chunk) hit distinct LDS banks.  With bf16 weights: a ring of SB 16 KB
// weight slots, one per 32-k sub-step, then SA A slots (half_ring.h).  With
// fp8 weights: S 16 KB stage slots of codes (two sub-steps, one barrier),
// issued S - 1 stages ahead, then two A slots issued one stage ahead.
// Below, "paired" names this 128..256-row family (A staged two MFMA k-steps
// at a time).
template <int MB>
constexpr bool pair_a() { return MB >= 8; }
__device__ __forceinline__ int a_swizzle(int row) { return (row >> 1) & 7; }
// bf16 paired tiles with the half-stage weight ring: its slot counts (weight
// sub-steps SB, A stages SA) and the weight sub-steps issued ahead of an item
// (KP, at most SB - 1)
template <int MB, bool F8>
constexpr bool half_b() { return BEAM_GEMM_HALF && pair_a<MB>() && !F8; }
template <int MB>
constexpr int half_sa() { return MB <= 8 ? BEAM_HALF_SA8 : MB <= 12 ? BEAM_HALF_SA12 : BEAM_HALF_SA16; }
template <int MB>
constexpr int half_sb() { return MB <= 8 ? BEAM_HALF_SB8 : MB <= 12 ? BEAM_HALF_SB12 : BEAM_HALF_SB16; }
template <int MB>
constexpr int half_kp() { return BEAM_HALF_KP < half_sb<MB>() ? BEAM_HALF_KP : half_sb<MB>() - 1; }
template <int MB>
constexpr int half_lag() { return MB <= 8 ? BEAM_HALF_LAG8 : MB <= 12 ? BEAM_HALF_LAG12 : BEAM_HALF_LAG16; }
template <int MB, int S, bool F8 = false>
constexpr int ring_bytes() {
  if constexpr (half_b<MB, F8>())
    return (half_sb<MB>() * kItemBlocks + half_sa<MB>() * MB * 2) * kFrag;
  return pair_a<MB>() ? S * (F8 ? 1 : 2) * kItemBlocks * kFrag + 2 * MB * 2 * kFrag
                      : S * (kItemBlocks + MB) * kFrag;
}

// Source rows of this wave's A loads in the 128/192-row configurations: for
// each of its row blocks j (block wave + kNW j of the m-tile) and half hf,
// lane l reads tile row 16 (wave + kNW j) + 8 hf + l / 8 (rows past the tile
// repeat its last row), i.e. row gather[row0 + that] / topk of A (or row0 +
// that without a gather).  The gather indices are read with scalar loads of
// uniform addresses: those are counted in lgkmcnt, never in the vector memory
// counter that the direct-load ring is waited on with, so reading them does
// not drain loads in flight.
template <int AM, int kNW>
__device__ __forceinline__ void paired_a_rows(int (&rows)[AM][2], const int32_t* gather, int topk,
                                              int row0, int nrows, int wave, int lane,
                                              int64_t n_rows, int64_t n_src) {
  (void)n_rows;
  (void)n_src;
  const int sel = lane >> 3;
#pragma unroll
  for (int j = 0; j < AM; ++j) {
    const int blk = __builtin_amdgcn_readfirstlane((wave + kNW * j) * 16);
    if (gather) {
      const __attribute__((address_space(4))) int32_t* cg =
          (const __attribute__((address_space(4))) int32_t*)gather;
      int v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        v[k] = cg[BEAM_CLAMP(row0 + min(blk + k, nrows - 1), 0, n_rows - 1, kCheckGatherIndex)];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        int x = v[8 * hf];
#pragma unroll
        for (int k = 1; k < 8; ++k) x = sel == k ? v[8 * hf + k] : x;
        rows[j][hf] = BEAM_CLAMP(x / topk, 0, n_src - 1, kCheckTokenIndex);
      }
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        rows[j][hf] = BEAM_CLAMP(row0 + min(blk + 8 * hf + sel, nrows - 1), 0, n_src - 1,
                                 kCheckTokenIndex);
    }
  }
}

// Wait of the half-stage pipeline at distance d (D0, D0 + 2, .. DMAX) from
// the end of the k loop: the count of half_ring::tail_count for this wave's
// A load count (hi: the larger one); any other d drains.
template <int SA, int SB, int KP, int LAG, int NBL, int NA2H, int NA2L, int D, int DMAX>
__device__ __forceinline__ void wait_half_tail(int d, bool hi) {
  if constexpr (D > DMAX) {
    wait_vm<0>();
  } else {
    if (d == D) {
      if (hi) wait_vm<half_ring::tail_count(SA, SB, KP, LAG, NBL, NA2H, D)>();
      else wait_vm<half_ring::tail_count(SA, SB, KP, LAG, NBL, NA2L, D)>();
    } else {
      wait_half_tail<SA, SB, KP, LAG, NBL, NA2H, NA2L, D + 2, DMAX>(d, hi);
    }
  }
}

// One (m-tile, n-tile) item with exactly NRB live 16-row blocks, of which
// this wave computes RB blocks starting at block row_off.  MB sizes the LDS
// ring; fragments of blocks NRB..MB-1 are not loaded.
template <int NRB, int RB, int MB, int kNW, int RG, int S, bool SWIGLU, bool F8, bool NT>
__device__ __forceinline__ void gemm_item_rows(const ItemArgs& a, uint8_t* lds, int wave, int lane,
                                               int row_off) {
  constexpr int CG = kNW / RG;
  constexpr int NCBW = kItemBlocks / CG;        // column blocks this wave computes
  constexpr int NBL = NCBW / RG;                // ... and loads per stage (shared with its row peers)
  constexpr int D = S - 1;                      // stages in flight ahead of compute
  constexpr bool kPairA = pair_a<MB>();
  constexpr int AOFF = kItemBlocks * kFrag;     // unpaired slot = B fragments, then A fragments
  constexpr int SLOT = AOFF + MB * kFrag;       // unpaired slot
  constexpr int BSUB = kItemBlocks * kFrag;     // paired: one 32-k half of a weight stage
  constexpr int BSTAGE = F8 ? BSUB : 2 * BSUB;  // paired: one 64-k weight stage slot
  static_assert(!F8 || kPairA, "fp8 weights run the 64-k stage pipeline only");
  constexpr int APAIR = MB * 2 * kFrag;         // paired: one 64-k A slot
  // bf16 paired tiles: weight ring of HSB half-stage slots (BSUB each), A ring
  // of HSA slots
  constexpr bool kHalfB = half_b<MB, F8>();
  constexpr int HSA = half_sa<MB>(), HSB = half_sb<MB>(), HKP = half_kp<MB>(), HLAG = half_lag<MB>();
  constexpr int APOFF = kHalfB ? HSB * BSUB : S * BSTAGE;  // paired: A ring after the weight ring
  static_assert(!kPairA || S >= 3, "a weight stage is issued before the A stage waited with it");
  constexpr int HALF = SWIGLU ? NCBW / 2 : NCBW;
  constexpr int WCOLS = CG * HALF * 16;
  constexpr int RBX = RB > 0 ? RB : 1;
  // Paired: weight stages of the workgroup's next item issued while this
  // item's epilogue runs: S - 2 (the prologue issues stage S - 1 after the
  // first A stages).
  constexpr int kPre = kHalfB ? HKP : kPairA ? S - 2 : 0;
  // NT: weights are loaded with the non-temporal policy.  The launch picks
  // it where the kernel is a pure weight stream (see launch_grouped_gemm).
  constexpr bool kStreamWeights = NT;
  static_assert(CG * RG == kNW && NCBW * CG == kItemBlocks && NBL * RG == NCBW, "work split");
  // A fragments this wave loads: blocks wave, wave + kNW, ... below NRB
  constexpr int AMAX = (NRB + kNW - 1) / kNW;
  const int r = lane & 15, g = lane >> 4;
  const int cg = wave % CG, rg = wave / CG;
  const int nk = a.K / kBKS;
  // Waves own different numbers of A fragments when NRB % kNW != 0, so each
  // wave's loads per stage (and thus its vmcnt thresholds) are its own:
  // na in {AMAX - 1, AMAX}.  Both values are handled by separate waits.
  const int na = (NRB - wave + kNW - 1) / kNW;

  // A sources.  Unpaired: lane = (row r, k chunk g) of a 16 x 32 fragment.
  // Paired: per 16-row block two loads (hf = rows 0-7, rows 8-15); lane l
  // fetches row 8 hf + l / 8, the 16-byte chunk that the swizzle places at
  // position l % 8 of that row's 128 bytes.  Rows are kept as 32-bit indices
  // (the 192-row configuration has no registers to spare).
  constexpr int NHF = kPairA ? 2 : 1;
  int asrow[AMAX > 0 ? AMAX : 1][NHF];
  if constexpr (kPairA) {
    paired_a_rows<(AMAX > 0 ? AMAX : 1), kNW>(asrow, a.gather, a.topk, a.row0, a.nrows, wave, lane,
                                              a.n_rows, a.n_src);
  } else {
#pragma unroll
    for (int j = 0; j < AMAX; ++j) {
      int row = (wave + kNW * j) * 16 + r;
      row = row < a.nrows ? row : a.nrows - 1;  // rows past the tile repeat its last row
      asrow[j][0] = a.gather
          ? a.gather[BEAM_CLAMP(a.row0 + row, 0, a.n_rows - 1, kCheckGatherIndex)] / a.topk
          : a.row0 + row;
      asrow[j][0] = BEAM_CLAMP(asrow[j][0], 0, a.n_src - 1, kCheckTokenIndex);
    }
  }
  auto asrc = [&](int j, int hf, int k0) {
    const int rho = hf * 8 + (lane >> 3);
    return a.A + (size_t)asrow[j][hf] * a.K + k0 + 8 * (kPairA ? ((lane & 7) ^ a_swizzle(rho)) : g);
  };
  // the weight row (output column) of lane r in column block cb of group cg
  // of n-tile ntile
  auto weight_row_of = [&](int cb, int ntile) {
    if (SWIGLU) {
      const int j = cb % HALF;
      return ntile * WCOLS + cg * HALF * 16 + j * 16 + r + (cb >= HALF ? a.up_row0 : 0);
    }
    return ntile * WCOLS + cg * NCBW * 16 + cb * 16 + r;
  };
  auto weight_row = [&](int cb) { return weight_row_of(cb, a.ntile); };
  // Weight loads address a wave-uniform base (the lane-0 row of the column
  // block, in SGPRs) plus one per-lane byte offset shared by every stream:
  // row-major: row r, k chunk 8g; packed: fragment (wrow/16, stage) holds
  // this lane's 16 bytes at lane*16, and a row block's fragments follow each
  // other along k (bf16: one per 32 k; fp8: one per 64 k).
  auto bbase_of = [&](const uint16_t* W, int ntile, int t) -> const uint8_t* {
    // uniform; the block's 16 rows lie inside the expert's weight rows
    const int wrow0 = BEAM_CLAMP(weight_row_of(rg + RG * t, ntile) - r, 0,
                                 (SWIGLU ? a.up_row0 : 0) + a.n_out - 16, kCheckWeightOffset);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(W);
    if constexpr (F8) return w + (size_t)(wrow0 >> 4) * (nk >> 1) * kFrag;
    return a.packed ? w + (size_t)(wrow0 >> 4) * nk * kFrag : w + (size_t)wrow0 * a.K * 2;
  };
  const uint32_t boff = a.packed ? (uint32_t)lane * 16u : (uint32_t)(r * a.K + 8 * g) * 2u;
  const uint8_t* bsrc[NBL];
#pragma unroll
  for (int t = 0; t < NBL; ++t) bsrc[t] = bbase_of(a.W, a.ntile, t);
  const int bstep = a.packed ? kFrag : kBKS * 2;  // bf16: bytes per 32-k stage along a stream
  // fp8: the fp32 scales of this lane's four output columns (weight rows
  // 4g..4g+3 of each column block), applied to the accumulators after the k
  // loop
  f32x4_t wscale[F8 ? NCBW : 1];
  if constexpr (F8) {
#pragma unroll
    for (int cb = 0; cb < NCBW; ++cb)
      wscale[cb] = *reinterpret_cast<const f32x4_t*>(a.scale + weight_row(cb) - r + 4 * g);
  }
  // LDS byte offset of the ring (addrspace cast, not the flat address)
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);
  const uint32_t b_base = __builtin_amdgcn_readfirstlane(lds0 + (cg * NCBW + rg) * kFrag);
  const uint32_t a_base = __builtin_amdgcn_readfirstlane(
      kPairA ? lds0 + APOFF + wave * 2 * kFrag : lds0 + AOFF + wave * kFrag);
  // byte offset, inside a 64-k stage's 2 KB row block, of this lane's MFMA
  // operand (row r, logical chunk g) for the stage's first 32-k sub-step; the
  // second reads logical chunk 4 + g, the same address with bit 6 flipped
  const int aoff0 = (r >> 3) * kFrag + (r & 7) * 128 + ((g ^ a_swizzle(r)) << 4);

  f32x4_t acc[RBX][NCBW];
#pragma unroll
  for (int i = 0; i < RBX; ++i)
#pragma unroll
    for (int cb = 0; cb < NCBW; ++cb) acc[i][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 af[RBX];
  uint4 b0[NCBW], b1[NCBW];
  // MFMAs of one 32-k sub-step on the operands in registers, reading the
  // next sub-step's A fragments from LDS right after each row block's MFMAs
  // (one A register set).
  auto mfmas = [&](const uint4 (&cbf)[NCBW], bool more, auto next_a) {
    if constexpr (RB > 0) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
#pragma unroll
        for (int cb = 0; cb < NCBW; ++cb)
          acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(cbf[cb]), as_bf16x8(af[i]), acc[i][cb], 0, 0, 0);
        if (more) af[i] = next_a(i);
      }
    }
  };

  // paired: issue the weights of 64-k stage P into slot P % S
  auto issue_b64 = [&](const uint8_t* const (&src)[NBL], int P) {
    BEAM_CHECK(P >= 0 && P < (nk >> 1), kCheckWeightOffset);
    const uint32_t so = (uint32_t)((P % S) * BSTAGE);
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < NBL; ++t)
        lds_dma16_sv<kStreamWeights>(src[t] + (size_t)P * kFrag, boff,
                                     b_base + so + RG * t * kFrag);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < NBL; ++t)
          lds_dma16_sv<kStreamWeights>(src[t] + (size_t)(2 * P + h) * bstep, boff,
                                       b_base + so + h * BSUB + RG * t * kFrag);
    }
  };

  if constexpr (kHalfB) {
    // ---- bf16, 128..256-row tiles: 32-k weight slots, 64-k A slots ----
    // The schedule and its wait counts are those of half_ring.h: iteration kt
    // waits for sub-step kt + 1, passes the barrier, refills the slots of
    // sub-step j = kt - HLAG (A slot ((j - 1) / 2) % HSA for odd j, weight
    // slot j % HSB), then reads sub-step kt + 1's weights while sub-step kt's
    // MFMAs run.  A stages are issued 2 HSA - 2 - HLAG sub-steps ahead of
    // their use, weights HSB - 1 - HLAG.
    namespace hr = half_ring;
    const int nst = nk >> 1;  // K is a multiple of 128: nk >= 4
    // the two per-wave A load counts (na = AMAX or AMAX - 1 blocks)
    constexpr int NA2H = 2 * AMAX, NA2L = AMAX > 0 ? 2 * (AMAX - 1) : 0;
    using SH = hr::Steady<HSA, HSB, HKP, HLAG, NBL, NA2H>;
    using SL = hr::Steady<HSA, HSB, HKP, HLAG, NBL, NA2L>;
    constexpr int kS0 = SH::from > SL::from ? SH::from : SL::from;
    constexpr int kT = SH::tail > SL::tail ? SH::tail : SL::tail;
    static_assert(kS0 < 64 && kT < 64, "the schedule reaches a steady state");
    constexpr int kWOddH = SH::odd, kWOddL = SL::odd, kWEvenH = SH::even, kWEvenL = SL::even;
    constexpr int kMaxW = SH::max > SL::max ? SH::max : SL::max;
    static_assert(kMaxW < 64, "vmcnt holds 6 bits");
    static_assert(SH::ok && SL::ok, "steady counts are safe from sub-step 1 on");
    static_assert(HLAG == 0 || HLAG == 1, "refill lag");
    constexpr int kDeepMin = SH::deep > SL::deep ? SH::deep : SL::deep;
    // Waits of the loop (the rule stated in half_ring.h): a loop shorter than
    // kDeepMin sub-steps drains; otherwise the steady count of the parity of
    // s, or for the last sub-steps the count at distance d = nk - s from the
    // end.
    const bool deep = nk >= kDeepMin;

    auto issue_b = [&](const uint8_t* const (&src)[NBL], int st, uint32_t slot) {
      BEAM_CHECK(st >= 0 && st < nk, kCheckWeightOffset);
#pragma unroll
      for (int t = 0; t < NBL; ++t)
        lds_dma16_sv<kStreamWeights>(src[t] + (size_t)st * bstep, boff,
                                     b_base + slot * BSUB + RG * t * kFrag);
    };
    auto issue_a = [&](int P, uint32_t slot) {
      const int k0 = P * 2 * kBKS;
#pragma unroll
      for (int j = 0; j < AMAX; ++j)
        if (j < na) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            lds_dma16(asrc(j, hf, k0), a_base + slot * APAIR + kNW * j * 2 * kFrag + hf * kFrag);
        }
    };
    auto read_b = [&](uint32_t slot, uint4 (&bf)[NCBW]) {
      const uint8_t* sl = lds + slot * BSUB;
#pragma unroll
      for (int cb = 0; cb < NCBW; ++cb)
        bf[cb] = *reinterpret_cast<const uint4*>(sl + (cg * NCBW + cb) * kFrag + 16 * lane);
    };
    // sub-step operand of row block i from A slot `slot`: logical chunk g of
    // the stage's first 32 k (half 0), 4 + g of the second (bit 6 flipped)
    auto read_a = [&](uint32_t slot, int half, int i) {
      const uint8_t* pl = lds + APOFF + slot * APAIR + (aoff0 ^ (half << 6));
      return *reinterpret_cast<const uint4*>(pl + (row_off + i) * 2 * kFrag);
    };
    auto wait_dyn = [&](int s) {
      wait_vm_dyn<0, kMaxW>(hr::younger_fast(HSA, HSB, HKP, NBL, 2 * na, nk, s, hr::last_of(s, HLAG)));
    };
    // lag 0: this wave's reads of the operands of the sub-step whose slots
    // the coming barrier frees must have landed; lag 1 frees older slots
    auto wait_reads = [&]() {
      if constexpr (HLAG == 0) wait_lgkm0();
    };
    auto next_slot = [](uint32_t x, uint32_t n) { return x + 1 == n ? 0u : x + 1; };

    // Prologue: the front weight sub-steps (unless the previous item issued
    // them), then what model iterations first_iter .. -1 - HLAG would have
    // issued.
    if (a.q < a.grid) {
#pragma unroll
      for (int st = 0; st < HKP; ++st)
        if (st < nk) issue_b(bsrc, st, (uint32_t)st);
    }
#pragma unroll
    for (int j = hr::first_iter(HSA, HSB); j < -HLAG; ++j) {
      if (j % 2 != 0) {
        const int P = (j - 1) / 2 + HSA;
        if (P >= 0 && P < nst) issue_a(P, (uint32_t)P);
      }
      const int st = j + HSB;
      if (st >= HKP && st < nk) issue_b(bsrc, st, (uint32_t)st);
    }
    wait_dyn(0);
    stage_barrier();
    read_b(0u, b0);
    if constexpr (RB > 0) {
#pragma unroll
      for (int i = 0; i < RB; ++i) af[i] = read_a(0u, 0, i);
    }
    // bs: weight slot of sub-step kt; as: A slot of stage kt / 2
    uint32_t bs = 0, as = 0;
    // Sub-steps kt (even) and kt + 1 but the last two.  Away from both ends of
    // the loop the waits take the counts of a deep loop (immediates); near
    // them the counts are computed.
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
      const uint32_t bs1 = next_slot(bs, HSB), bs2 = next_slot(bs1, HSB);
      const uint32_t asn = next_slot(as, HSA);
      // sub-step kt: wait for kt + 1 (odd)
      if (!deep) wait_vm<0>();
      else if (kt + 1 + kT < nk) {
        if (na == AMAX) wait_vm<kWOddH>();
        else wait_vm<kWOddL>();
      } else {
        wait_half_tail<HSA, HSB, HKP, HLAG, NBL, NA2H, NA2L, 1, kT>(nk - kt - 1, na == AMAX);
      }
      wait_reads();
      stage_barrier();  // sub-step kt + 1 is visible; the slots of sub-step kt - HLAG are free
      if constexpr (HLAG == 0) {
        // model iteration kt (even): weights only
        if (kt + HSB < nk) issue_b(bsrc, kt + HSB, bs);
      } else {
        // model iteration kt - 1 (odd): A stage kt / 2 - 1 + HSA, then weights
        const uint32_t bsp = bs == 0 ? HSB - 1 : bs - 1, asp = as == 0 ? HSA - 1 : as - 1;
        const int P = (kt >> 1) - 1 + HSA;
        if (P < nst) issue_a(P, asp);
        if (kt - 1 + HSB < nk) issue_b(bsrc, kt - 1 + HSB, bsp);
      }
      read_b(bs1, b1);
      mfmas(b0, true, [&](int i) { return read_a(as, 1, i); });
      // sub-step kt + 1: wait for kt + 2 (even, a new A stage)
      if (!deep) wait_vm<0>();
      else if (kt + 2 + kT < nk) {
        if (na == AMAX) wait_vm<kWEvenH>();
        else wait_vm<kWEvenL>();
      } else {
        wait_half_tail<HSA, HSB, HKP, HLAG, NBL, NA2H, NA2L, 2, kT>(nk - kt - 2, na == AMAX);
      }
      wait_reads();
      stage_barrier();
      if constexpr (HLAG == 0) {
        // model iteration kt + 1 (odd): A stage kt / 2 + HSA, then weights
        const int P = (kt >> 1) + HSA;
        if (P < nst) issue_a(P, as);
        if (kt + 1 + HSB < nk) issue_b(bsrc, kt + 1 + HSB, bs1);
      } else {
        // model iteration kt (even): weights only
        if (kt + HSB < nk) issue_b(bsrc, kt + HSB, bs);
      }
      read_b(bs2, b0);
      mfmas(b1, true, [&](int i) { return read_a(asn, 0, i); });
      bs = bs2;
      as = asn;
    }
    // the last two sub-steps (kt = nk - 2): nothing left to issue
    if (!deep) wait_vm<0>();
    else wait_half_tail<HSA, HSB, HKP, HLAG, NBL, NA2H, NA2L, 1, 1>(1, na == AMAX);
    wait_reads();
    stage_barrier();
    read_b(next_slot(bs, HSB), b1);
    mfmas(b0, true, [&](int i) { return read_a(as, 1, i); });
    mfmas(b1, false, [&](int i) { return read_a(as, 1, i); });
    wait_lgkm0();
    stage_barrier();  // every wave is done with the ring

  } else if constexpr (kPairA) {
    // ---- 128/192-row tiles: 64-k stages ----
    // Stage P: weights of sub-steps 2P, 2P+1 in slot P % S (issued S - 1
    // stages ahead), A rows in slot P & 1 (issued one stage ahead).  Order of
    // issue: prologue B(0..S-2), A(0), A(1), B(S-1); then after the barrier
    // that publishes stage P + 1: A(P + 2), B(P + S).  So the only loads
    // younger than A(P + 1) when stage P + 1 is waited for are those of
    // B(P - 1 + S), and every B(P + 1) is older than A(P + 1).
    const int nst = nk >> 1;  // K is a multiple of 128: nst >= 2
    // weight loads of one stage per wave: bf16 two 1 KB fragments (32 k
    // each) per column block it loads, fp8 one (64 k)
    constexpr int kStageLoads = F8 ? NBL : 2 * NBL;
    auto issue_a64 = [&](int P) {
      const uint32_t po = (uint32_t)((P & 1) * APAIR);
      const int k0 = P * 2 * kBKS;
#pragma unroll
      for (int j = 0; j < AMAX; ++j)
        if (j < na) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            lds_dma16(asrc(j, hf, k0), a_base + po + kNW * j * 2 * kFrag + hf * kFrag);
        }
    };
    auto read_b64 = [&](int kt, uint4 (&bf)[NCBW]) {
      if constexpr (F8) {
        // the fragment's first 512 bytes hold every lane's 8 codes of the
        // first 32 k, the next 512 those of the second; widened to bf16
        const uint8_t* sl = lds + ((kt >> 1) % S) * BSTAGE + (kt & 1) * 512;
#pragma unroll
        for (int cb = 0; cb < NCBW; ++cb) {
          const uint2 c = *reinterpret_cast<const uint2*>(sl + (cg * NCBW + cb) * kFrag + 8 * lane);
          bf[cb] = make_uint4(fp8x2_to_bf16x2<false>(c.x), fp8x2_to_bf16x2<true>(c.x),
                              fp8x2_to_bf16x2<false>(c.y), fp8x2_to_bf16x2<true>(c.y));
        }
      } else {
        const uint8_t* sl = lds + ((kt >> 1) % S) * BSTAGE + (kt & 1) * BSUB;
#pragma unroll
        for (int cb = 0; cb < NCBW; ++cb)
          bf[cb] = *reinterpret_cast<const uint4*>(sl + (cg * NCBW + cb) * kFrag + 16 * lane);
      }
    };
    // sub-step kt's A operand of row block i: logical chunk g of the first
    // 32 k, 4 + g of the second (the same address with bit 6 flipped)
    auto read_a64 = [&](int kt, int i) {
      const uint8_t* pl = lds + APOFF + ((kt >> 1) & 1) * APAIR + (aoff0 ^ ((kt & 1) << 6));
      return *reinterpret_cast<const uint4*>(pl + (row_off + i) * 2 * kFrag);
    };

    // Prologue.  Every item except a workgroup's first finds its first kPre
    // weight stages issued by its predecessor.  Stages at or past nst do not
    // exist (K = 128 has two) and are never issued; leaving out such older
    // loads only lowers the counts the waits below have to reach.
    if (a.q < a.grid) {
#pragma unroll
      for (int P = 0; P < kPre; ++P)
        if (P < nst) issue_b64(bsrc, P);
    }
#pragma unroll
    for (int P = kPre; P < S - 1; ++P)
      if (P < nst) issue_b64(bsrc, P);
    issue_a64(0);
    issue_a64(1);
    if (S - 1 < nst) issue_b64(bsrc, S - 1);
    wait_vm_dyn<0, 15>(2 * na + (S - 1 < nst ? kStageLoads : 0));  // stage 0 landed
    stage_barrier();
    read_b64(0, b0);
    if constexpr (RB > 0) {
#pragma unroll
      for (int i = 0; i < RB; ++i) af[i] = read_a64(0, i);
    }
    for (int P = 0; P < nst; ++P) {
      const int kt = 2 * P;
      // sub-step 2P: the operands of 2P + 1 are in the same, published stage
      read_b64(kt + 1, b1);
      mfmas(b0, true, [&](int i) { return read_a64(kt + 1, i); });
      // sub-step 2P + 1: publish stage P + 1, refill stage P's slots
      const bool more = P + 1 < nst;
      if (more) {
        if (P - 1 + S < nst) wait_vm<kStageLoads>();  // stage P + 1 landed
        else wait_vm<0>();
        wait_lgkm0();     // this wave's reads of stage P have landed
        stage_barrier();  // stage P + 1 is visible; stage P's slots are free
        if (P + 2 < nst) issue_a64(P + 2);
        if (P + S < nst) issue_b64(bsrc, P + S);
        read_b64(kt + 2, b0);
      }
      mfmas(b1, more, [&](int i) { return read_a64(kt + 2, i); });
    }
    wait_lgkm0();
    stage_barrier();  // every wave is done with the ring
    if constexpr (F8 && RB > 0) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int cb = 0; cb < NCBW; ++cb) acc[i][cb] *= wscale[cb];
    }

  } else {
    // ---- 64-row tiles: 32-k stages, B and A of a stage in one slot ----
    auto issue = [&](int st) {
      BEAM_CHECK(st >= 0 && st < nk, kCheckWeightOffset);
      const uint32_t so = (uint32_t)((st % S) * SLOT);
#pragma unroll
      for (int t = 0; t < NBL; ++t)
        lds_dma16_sv<kStreamWeights>(bsrc[t] + (size_t)st * bstep, boff,
                                     b_base + so + RG * t * kFrag);
#pragma unroll
      for (int j = 0; j < AMAX; ++j)
        if (j < na) lds_dma16(asrc(j, 0, st * kBKS), a_base + so + kNW * j * kFrag);
    };
    // wait until stage `st` has landed, given that stages up to
    // min(st + D - 1, nk - 1) have been issued
    auto wait_for = [&](int st) {
      const int ahead = min(D - 1, nk - 1 - st);
      if (na == AMAX) wait_stage<D - 1, NBL + AMAX>(ahead);
      else wait_stage<D - 1, NBL + AMAX - 1>(ahead);
    };
    auto read_b = [&](int st, uint4 (&bf)[NCBW]) {
      const uint8_t* sl = lds + (st % S) * SLOT;
#pragma unroll
      for (int cb = 0; cb < NCBW; ++cb)
        bf[cb] = *reinterpret_cast<const uint4*>(sl + (cg * NCBW + cb) * kFrag + 16 * lane);
    };
    auto read_a = [&](int st, int i) {
      const uint8_t* sl = lds + (st % S) * SLOT;
      return *reinterpret_cast<const uint4*>(sl + AOFF + (row_off + i) * kFrag + 16 * lane);
    };
    // One K-stage.  The next stage's operands are read from LDS while this
    // stage's MFMAs run.  Slot reuse: stage kt + D refills the slot of stage
    // kt - 1, whose fragments every wave read (and waited for) before the
    // previous barrier.
    auto step = [&](int kt, const uint4 (&cbf)[NCBW], uint4 (&nb_)[NCBW]) {
      if (kt + D < nk) issue(kt + D);
      if (kt + 1 < nk) wait_for(kt + 1);
      wait_lgkm0();      // this wave's reads of stage kt have landed
      stage_barrier();   // stage kt + 1 is visible to every wave
      const bool more = kt + 1 < nk;
      if (more) read_b(kt + 1, nb_);
      mfmas(cbf, more, [&](int i) { return read_a(kt + 1, i); });
    };

#pragma unroll
    for (int st = 0; st < D; ++st)
      if (st < nk) issue(st);
    wait_for(0);
    stage_barrier();
    read_b(0, b0);
    if constexpr (RB > 0) {
#pragma unroll
      for (int i = 0; i < RB; ++i) af[i] = read_a(0, i);
    }
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, b0, b1);
      step(kt + 1, b1, b0);
    }
    if (kt < nk) step(kt, b0, b1);
    wait_lgkm0();
    stage_barrier();  // every wave is done with the ring before the next item refills it
  }

  // LoRA second factor: rank steps of 32 (ranks past lora_r contribute zeros),
  // operands loaded straight from global memory in the MFMA lane order.
  if constexpr (RB > 0 && !F8) {
    if (a.lora_t) {
      const int R = a.lora_r;
      for (int k0 = 0; k0 < R; k0 += 32) {
        const bool live = k0 + 8 * g < R;
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
        uint4 bl[NCBW];
#pragma unroll
        for (int cb = 0; cb < NCBW; ++cb)
          bl[cb] = live ? ld16(a.lora_b + (size_t)weight_row(cb) * R + k0 + 8 * g) : zero;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          int row = (row_off + i) * 16 + r;
          row = row < a.nrows ? row : a.nrows - 1;
          const uint4 al = live ? ld16(a.lora_t + (size_t)(a.row0 + row) * R + k0 + 8 * g) : zero;
#pragma unroll
          for (int cb = 0; cb < NCBW; ++cb)
            acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bl[cb]), as_bf16x8(al),
                                                                 acc[i][cb], 0, 0, 0);
        }
      }
    }
  }

  // Paired: start the next item's weight stream now (stage slots
  // 0..kPre-1), before this item's epilogue, which needs no LDS.
  if constexpr (kPairA) {
    const int qn = a.q + a.grid;
    if (kPre > 0 && qn < a.total) {
      int tn, ntn;
      item_of(qn, a.nt_n, a.plan_first, a.plan_count, tn, ntn);
      const uint16_t* nw = a.W0 + (size_t)a.plan_expert[tn] * a.w_expert_stride;
      const uint8_t* nsrc[NBL];
#pragma unroll
      for (int t = 0; t < NBL; ++t) nsrc[t] = bbase_of(nw, ntn, t);
      if constexpr (kHalfB) {
#pragma unroll
        for (int st = 0; st < kPre; ++st)
          if (st < nk) {  // the next item's weight sub-steps (same K) into slots 0..kPre-1
#pragma unroll
            for (int t = 0; t < NBL; ++t)
              lds_dma16_sv<kStreamWeights>(nsrc[t] + (size_t)st * bstep, boff,
                                           b_base + st * BSUB + RG * t * kFrag);
          }
      } else {
        const int nst = a.K / (2 * kBKS);  // the next item's k stages (same K)
#pragma unroll
        for (int P = 0; P < kPre; ++P)
          if (P < nst) issue_b64(nsrc, P);
      }
    }
  }

  // Epilogue straight from the accumulators.  The MFMAs take the weights as
  // their first operand, so each 16x16 accumulator block is the transposed
  // output tile: lane (r, g) holds output columns 4g..4g+3 of row r, which
  // leave as one 8-byte store (four bf16); the column blocks of one row are
  // written by neighbouring lanes and waves in the same few instructions and
  // merge into whole lines in L2.
  // The stores are range-checked buffer stores over this m-tile's output
  // rows: a lane whose row lies past the tile gets an offset outside the
  // range and its store is dropped (no branch around the stores), and the
  // four values are rounded to bf16 and packed in pairs by the hardware
  // conversion.
  if constexpr (RB > 0) {
    const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
        a.C + (size_t)a.row0 * a.n_out, 0, a.nrows * a.n_out * 2, kBufferRsrcWord3);
    // the lane's row and column, opaque to the optimiser so that the store
    // offsets are formed here rather than kept live (or spilled) across the
    // k loop
    int er = r, eg = g;
    asm volatile("" : "+v"(er), "+v"(eg));
    // the lane's four outputs of row block i, column block j, as bf16 pairs
    auto outputs = [&](int i, int j) {
      float o[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (SWIGLU) {
          const float gt = acc[i][j][v], up = acc[i][j + HALF][v];
          o[v] = silu_mul(gt, up);
        } else {
          o[v] = acc[i][j][v];
        }
      }
      return u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    };
    constexpr int kPolicy = SWIGLU ? BEAM_STORE_POLICY_GU : BEAM_STORE_POLICY_DOWN;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int row = (row_off + i) * 16 + er;
      if constexpr (BEAM_EPI_WIDE && HALF % 2 == 0) {
        // Column blocks j, j + 1 together: lane rows g = 2m and 2m + 1 (16
        // lanes each) hold columns 8m..8m+3 and 8m+4..8m+7 of both blocks;
        // v_permlane16_swap trades block j + 1's half of row 2m for block
        // j's half of row 2m + 1, so each lane then holds 8 consecutive
        // columns (row 2m of block j, row 2m + 1 of block j + 1) and writes
        // them with one 16-byte store: half the store instructions.
#pragma unroll
        for (int j = 0; j < HALF; j += 2) {
          const u32x2_t d0 = outputs(i, j), d1 = outputs(i, j + 1);
          const auto sx = __builtin_amdgcn_permlane16_swap(d0[0], d1[0], false, false);
          const auto sy = __builtin_amdgcn_permlane16_swap(d0[1], d1[1], false, false);
          const int col = a.ntile * WCOLS + cg * HALF * 16 + (j + (eg & 1)) * 16 + 4 * (eg & ~1);
          const uint32_t off = row < a.nrows ? (uint32_t)(row * a.n_out + col) * 2u : 0x80000000u;
          const u32x4_t d = {sx[0], sy[0], sx[1], sy[1]};
          __builtin_amdgcn_raw_buffer_store_b128(d, out, off, 0, kPolicy);
        }
      } else {
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
          const int col = a.ntile * WCOLS + cg * HALF * 16 + j * 16 + 4 * eg;
          const uint32_t off = row < a.nrows ? (uint32_t)(row * a.n_out + col) * 2u : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b64(outputs(i, j), out, off, 0, kPolicy);
        }
      }
    }
  }
}

// Item with NRB live row blocks: row group 0 takes the first ceil(NRB / RG)
// blocks, row group 1 the rest.
template <int NRB, int MB, int kNW, int RG, int S, bool SWIGLU, bool F8, bool NT>
__device__ __forceinline__ void gemm_item(const ItemArgs& a, uint8_t* lds, int wave, int lane) {
  if constexpr (RG == 1) {
    gemm_item_rows<NRB, NRB, MB, kNW, 1, S, SWIGLU, F8, NT>(a, lds, wave, lane, 0);
  } else {
    static_assert(RG == 2, "one or two row groups");
    constexpr int RB0 = (NRB + 1) / 2;
    if (wave < kNW / 2)
      gemm_item_rows<NRB, RB0, MB, kNW, 2, S, SWIGLU, F8, NT>(a, lds, wave, lane, 0);
    else
      gemm_item_rows<NRB, NRB - RB0, MB, kNW, 2, S, SWIGLU, F8, NT>(a, lds, wave, lane, RB0);
  }
}

template <int N, int MB, int kNW, int RG, int S, bool SWIGLU, bool F8, bool NT>
__device__ __forceinline__ void gemm_item_dispatch(int nrb, const ItemArgs& a, uint8_t* lds,
                                                   int wave, int lane) {
  if constexpr (N > MB) {
    return;
  } else {
    if (nrb == N) gemm_item<N, MB, kNW, RG, S, SWIGLU, F8, NT>(a, lds, wave, lane);
    else gemm_item_dispatch<N + 1, MB, kNW, RG, S, SWIGLU, F8, NT>(nrb, a, lds, wave, lane);
  }
}

template <int MB, int kNW, int RG, int S, bool SWIGLU, bool F8, bool NT>
__global__ __launch_bounds__(kNW * 64, 1) void stream_gemm_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather, int topk,
    const uint16_t* __restrict__ W, int64_t w_expert_stride, uint16_t* __restrict__ C,
    const int32_t* __restrict__ plan, int max_tiles, int K, int n_out, int up_row0, int packed,
    const uint16_t* __restrict__ lora_t, const uint16_t* __restrict__ lora_b,
    int64_t lora_b_stride, int lora_r, const float* __restrict__ scales, int64_t scale_stride,
    int64_t n_rows, int64_t n_src, int n_experts, int* sync) {
  (void)n_experts;
  constexpr int WCOLS = (SWIGLU ? kItemBlocks / 2 : kItemBlocks) * 16;
  static_assert(WCOLS == (SWIGLU ? kColsGateUp : kColsDown), "item width is fixed");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[ring_bytes<MB, S, F8>()];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = plan[0];
  const int* plan_expert = plan + 4;
  const int* plan_row0 = plan_expert + max_tiles;
  const int* plan_rows = plan_row0 + max_tiles;
  constexpr bool kBlocked = BEAM_GEMM_BLOCKED && MB == 16 && !F8 && (SWIGLU || BEAM_GEMM_BLOCKED_DOWN);
  const int* plan_first = kBlocked ? plan_rows + max_tiles : nullptr;
  const int* plan_count = kBlocked ? plan_rows + 2 * max_tiles : nullptr;
  // sync: this GEMM's round counters in the plan, one per (round, XCD),
  // zeroed by the plan kernel
  const int64_t sync_len = (int64_t)kPlanSyncPerTile * max_tiles;
  const int nt_n = n_out / WCOLS;
  const int total = ntiles * nt_n;
  const int grid = balanced_grid(total, gridDim.x), per_xcd = grid / 8;
  if ((int)blockIdx.x >= grid) return;  // whole workgroup: blockIdx is uniform
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;

  for (int round = 0;; round += grid) {
    const int q = round + xcd * per_xcd + slot;
    if (q >= total) break;
    if constexpr (kBlocked) {
      // Start the round with this XCD's other workgroups, so that the items
      // of a block stream their shared weights and rows through L2 together.
      // The wait is bounded: past BEAM_SYNC_SPIN polls the workgroup goes on
      // alone (results never depend on it).
      const int64_t idx = (int64_t)(round / grid) * 8 + xcd;
      if (idx < sync_len) {
        const int expected = min(per_xcd, total - (round + xcd * per_xcd));
        if (threadIdx.x == 0) {
          __hip_atomic_fetch_add(sync + idx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (int it = 0; it < BEAM_SYNC_SPIN; ++it) {
            if (__hip_atomic_load(sync + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= expected)
              break;
            __builtin_amdgcn_s_sleep(1);
          }
        }
        stage_barrier();
      }
    }
    int tile, ntile;
    item_of(q, nt_n, plan_first, plan_count, tile, ntile);
    const int e = BEAM_CLAMP(plan_expert[tile], 0, n_experts - 1, kCheckPlanRows);
    BEAM_CHECK(plan_rows[tile] >= 1 && plan_row0[tile] >= 0 &&
                   (int64_t)plan_row0[tile] + plan_rows[tile] <= n_rows,
               kCheckPlanRows);
    ItemArgs a{A, gather, topk, W + (size_t)e * w_expert_stride, C, K, n_out, up_row0, packed,
               plan_row0[tile], plan_rows[tile], ntile, lora_t,
               lora_t ? lora_b + (size_t)e * lora_b_stride : nullptr, lora_r, W,
               w_expert_stride, plan_expert, plan_first, plan_count, q, grid, total, nt_n,
               n_rows, n_src, F8 ? scales + (size_t)e * scale_stride : nullptr};
    const int nrb = (a.nrows + 15) >> 4;
    gemm_item_dispatch<1, MB, kNW, RG, S, SWIGLU, F8, NT>(nrb, a, lds, wave, lane);
  }
}

// One thread per expert: cut each expert's rows into ceil(n / bmax) balanced
// m-tiles (rows rounded up to 16, at most bmax).  plan[0] = tile count,
// plan[4 ..] = expert, row0, rows arrays of max_tiles entries each.
__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int bmax, int32_t* __restrict__ plan,
                                                        int max_tiles, int sync) {
  __shared__ int sc[256];
  const int e = threadIdx.x;
  int n = 0, nt = 0, per = 0;
  if (e < E) {
    n = offsets[e + 1] - offsets[e];
    nt = (n + bmax - 1) / bmax;
    if (nt > 0) per = min(bmax, (((n + nt - 1) / nt) + 15) & ~15);
  }
  sc[e] = nt;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int base = sc[e] - nt;
  int* pe = plan + 4;
  int* pr0 = pe + max_tiles;
  int* prn = pr0 + max_tiles;
  int* pfirst = prn + max_tiles;
  int* pcount = pfirst + max_tiles;
  for (int i = 0; i < nt; ++i) {
    const int idx = base + i;
    if (idx < max_tiles) {
      pe[idx] = e;
      pr0[idx] = offsets[e] + i * per;
      prn[idx] = min(per, n - i * per);
      pfirst[idx] = base;
      pcount[idx] = nt;
    }
  }
  if (sync) {
    int* ps = pcount + max_tiles;
    const int64_t len = plan_sync_ints(max_tiles);
    for (int64_t i = e; i < len; i += 256) ps[i] = 0;
  }
  if (e == 255) {
    BEAM_CHECK(sc[255] <= max_tiles, kCheckPlanCapacity);
    plan[0] = min(sc[255], max_tiles);
  }
}

// Fragment packing: expert e's [N, K] row-major matrix is rewritten as
// [N/16][K/32][64 lanes][8] -- the 1 KB MFMA operand of rows 16b..16b+15 and
// k 32s..32s+31, lane l holding row 16b + l%16, k 32s + 8(l/16) .. +7.  A row
// block's fragments are contiguous along k, so a weight stream reads whole
// kilobytes from consecutive addresses.  One thread moves 16 bytes.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ src,
                                                           uint16_t* __restrict__ dst, int N,
                                                           int K, int64_t chunks) {
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8-element chunk of dst
  if (d >= chunks) return;
  const int64_t per_expert = (int64_t)N * K / 8;
  const int64_t e = d / per_expert;
  const int64_t f = d - e * per_expert;
  const int lane = (int)(f & 63);
  const int64_t frag = f >> 6;
  const int nk = K / kBKS;
  const int64_t blk = frag / nk;
  const int st = (int)(frag - blk * nk);
  const int64_t row = blk * 16 + (lane & 15);
  const int64_t k = (int64_t)st * kBKS + (lane >> 4) * 8;
  st16(dst + d * 8, ld16(src + e * (int64_t)N * K + row * K + k));
}

// ---------------------------------------------------------------------------
// Launch configurations (MB, waves, row groups, S).  LDS per workgroup =
// S * (16 + MB) KB.  Small m-tiles use 4 waves and fit two workgroups per CU;
// large ones use 8 waves (two per SIMD) in one workgroup, as 2 row groups x 4
// column groups.
template <int MB, int NW, int RG, int S, bool SWIGLU, bool F8 = false, bool NT = (MB <= 8)>
static hipError_t launch_stream(const uint16_t* A, const int32_t* gather, int topk,
                                const uint16_t* W, int64_t wstride, uint16_t* C,
                                const int32_t* plan, int max_tiles, int K, int n_out, int up_row0,
                                int packed, const LoraArgs& lora, int64_t max_items,
                                hipStream_t stream, const GemmBounds& bounds,
                                const float* scales = nullptr, int64_t scale_stride = 0) {
  auto kern = stream_gemm_kernel<MB, NW, RG, S, SWIGLU, F8, NT>;
  static int per_cu = 0;  // resident workgroups per CU, fixed per build
  static int cus = 0;
  if (per_cu == 0) {
    int dev = 0, n = 0, occ = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, NW * 64, 0);
    if (err != hipSuccess) return err;
    cus = n;
    per_cu = occ > 0 ? occ : 1;
  }
  const int64_t grid = persistent_grid((int64_t)cus * per_cu, max_items);
  // the round counters of this GEMM: gate/up and down each have a region
  int* sync = const_cast<int32_t*>(plan) + 4 + 5 * (int64_t)max_tiles +
              (SWIGLU ? 0 : (int64_t)kPlanSyncPerTile * max_tiles);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), 0, stream, A, gather, topk, W,
                     wstride, C, plan, max_tiles, K, n_out, up_row0, packed, lora.t, lora.b,
                     lora.b_stride, lora.rank, scales, scale_stride, bounds.n_rows, bounds.n_src,
                     bounds.n_experts, sync);
  return hipGetLastError();
}

int64_t persistent_grid(int64_t resident, int64_t max_items) {
  int64_t grid = resident;
  const int64_t cap = (max_items + 7) / 8 * 8;
  if (cap < grid) grid = cap;
  if (const char* env = getenv("BEAM_MOE_MAX_GRID")) {
    const long long m = atoll(env);
    if (m > 0 && m < grid) grid = m;
  }
  grid = (grid + 7) / 8 * 8;
  return grid < 8 ? 8 : grid;
}

int ffn_rows_per_tile(int mb) { return 16 * mb; }

// m-tile height from the mean rows per expert: 64 rows while experts hold a
// few dozen rows (decode, mid batches), 192 once they hold ~100 or more, so
// an expert of a 4096-token chunk (95..165 rows) is a single m-tile.
int ffn_choose_mb(int64_t rows, int E) {
  const int64_t mean = rows / (E > 0 ? E : 1);
  if (mean <= 40) return 4;
  if (mean <= 80 || BEAM_GEMM_MAXMB == 8) return 8;
  if (BEAM_GEMM_MB16 && mean > 160) return 16;
  return BEAM_GEMM_MAXMB;
}

int ffn_out_cols_per_item(bool swiglu) { return swiglu ? kColsGateUp : kColsDown; }

// Up to 128-row tiles (batches of up to ~2.5K tokens) the kernel is a pure
// weight stream and always loads weights non-temporally (6.6 TB/s against
// 6.1 with the default policy at decode).  The 192-row gate/up GEMM does so
// while the mean expert holds at most 160 rows: nearly every expert is then
// a single m-tile whose weights are read once (4096-token chunk: 2.41 ->
// 2.34 ms).  With more rows per expert (the skewed 16K-token batch re-reads
// hot experts' weights for several m-tiles) the default policy keeps those
// re-reads in the caches (non-temporal: 7.6 -> 8.4 ms), and the 192-row down
// GEMM was 2-4 % slower with non-temporal loads in both cases.
bool ffn_stream_weights(int64_t rows, int E) { return rows / (E > 0 ? E : 1) <= 160; }

hipError_t launch_tile_plan(const int32_t* offsets, int E, int bmax, int32_t* plan, int max_tiles,
                            bool sync, hipStream_t stream) {
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, stream, offsets, E, bmax, plan,
                     max_tiles, sync ? 1 : 0);
  return hipGetLastError();
}

bool ffn_blocked_order(int mb) { return BEAM_GEMM_BLOCKED && BEAM_GEMM_MB16 && mb == 16; }

hipError_t launch_pack_weights(const uint16_t* src, uint16_t* dst, int E, int N, int K,
                               hipStream_t stream) {
  const int64_t chunks = (int64_t)E * N * K / 8;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst,
                     N, K, chunks);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int mb, bool swiglu, const uint16_t* A, const int32_t* gather,
                               int topk, const uint16_t* W, int64_t wstride, uint16_t* C,
                               const int32_t* plan, int max_tiles, int K, int n_out, int up_row0,
                               int packed, const LoraArgs& lora, int64_t max_items,
                               hipStream_t stream, bool stream_weights, const GemmBounds& bounds) {
#define BEAM_STREAM_ARGS                                                                    \
  A, gather, topk, W, wstride, C, plan, max_tiles, K, n_out, up_row0, packed, lora, max_items, \
      stream, bounds
#define BEAM_STREAM_CASE(MBV, NWV, RGV, SV)                                \
  case MBV:                                                                \
    return swiglu ? launch_stream<MBV, NWV, RGV, SV, true>(BEAM_STREAM_ARGS) \
                  : launch_stream<MBV, NWV, RGV, SV, false>(BEAM_STREAM_ARGS);
  switch (mb) {
    BEAM_STREAM_CASE(4, 4, 1, BEAM_GEMM_S4)
    BEAM_STREAM_CASE(8, BEAM_GEMM_NW8, BEAM_GEMM_RG8, BEAM_GEMM_S8)
#if BEAM_GEMM_MAXMB != 8
    case BEAM_GEMM_MAXMB:
      if (swiglu && stream_weights)
        return launch_stream<BEAM_GEMM_MAXMB, BEAM_GEMM_NW12, BEAM_GEMM_RG12, BEAM_GEMM_S12, true,
                             false, true>(BEAM_STREAM_ARGS);
#if BEAM_GEMM_DOWN_NT
      if (!swiglu && stream_weights)
        return launch_stream<BEAM_GEMM_MAXMB, BEAM_GEMM_NW12, BEAM_GEMM_RG12, BEAM_GEMM_S12, false,
                             false, true>(BEAM_STREAM_ARGS);
#endif
      return swiglu ? launch_stream<BEAM_GEMM_MAXMB, BEAM_GEMM_NW12, BEAM_GEMM_RG12,
                                    BEAM_GEMM_S12, true>(BEAM_STREAM_ARGS)
                    : launch_stream<BEAM_GEMM_MAXMB, BEAM_GEMM_NW12, BEAM_GEMM_RG12,
                                    BEAM_GEMM_S12, false>(BEAM_STREAM_ARGS);
#endif
#if BEAM_GEMM_MB16
    case 16:
      return swiglu ? launch_stream<16, 8, 2, BEAM_GEMM_S16, true, false, false>(BEAM_STREAM_ARGS)
                    : launch_stream<16, 8, 2, BEAM_GEMM_S16, false, false, false>(BEAM_STREAM_ARGS);
#endif
    default:
      return hipErrorInvalidValue;
  }
#undef BEAM_STREAM_CASE
#undef BEAM_STREAM_ARGS
}

BEAM_DEFINE_CHECK_READER(check_flags_ffn)

// FP8 (E4M3FN) weights through the same 64-k stage pipeline: a weight stage
// is one 1 KB fragment of 16 rows x 64 k per row block (16 KB per stage),
// widened to bf16 in registers, and the per-row scales multiply the fp32
// accumulators after the k loop.  128- and 192-row tiles.
#ifndef BEAM_FP8P_S8
#define BEAM_FP8P_S8 5
#endif
#ifndef BEAM_FP8P_S12
#define BEAM_FP8P_S12 5
#endif
hipError_t launch_grouped_gemm_fp8_paired(int mb, bool swiglu, const uint16_t* A,
                                          const int32_t* gather, int topk, const uint8_t* Q,
                                          const float* scales, int64_t qstride, int N, uint16_t* C,
                                          const int32_t* plan, int max_tiles, int K, int n_out,
                                          int up_row0, int64_t max_items, hipStream_t stream,
                                          const GemmBounds& bounds) {
  const uint16_t* W = reinterpret_cast<const uint16_t*>(Q);
  const int64_t wstride = qstride / 2;  // in 2-byte units: N * K codes per expert
  const LoraArgs none{};
#define BEAM_FP8P_CASE(MBV, SV)                                                                \
  case MBV:                                                                                     \
    return swiglu ? launch_stream<MBV, 8, 2, SV, true, true>(A, gather, topk, W, wstride, C,    \
                                                             plan, max_tiles, K, n_out,         \
                                                             up_row0, 1, none, max_items,       \
                                                             stream, bounds, scales, N)         \
                  : launch_stream<MBV, 8, 2, SV, false, true>(A, gather, topk, W, wstride, C,   \
                                                              plan, max_tiles, K, n_out,        \
                                                              up_row0, 1, none, max_items,      \
                                                              stream, bounds, scales, N);
  switch (mb) {
    BEAM_FP8P_CASE(8, BEAM_FP8P_S8)
    BEAM_FP8P_CASE(12, BEAM_FP8P_S12)
    default:
      return hipErrorInvalidValue;
  }
#undef BEAM_FP8P_CASE
}

}  // namespace beam
