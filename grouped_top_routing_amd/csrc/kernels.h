// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

constexpr int kChunk = 1024;  // (token, slot) pairs per permute workgroup

// Workgroups of a persistent grouped-GEMM launch: `resident` (one per
// resident slot on the device) capped by the item count, a multiple of 8
// (one per XCD), at least 8.  BEAM_MOE_MAX_GRID=<n> in the environment caps
// it further (results do not depend on the grid; tests use it to run many
// items per workgroup).
int64_t persistent_grid(int64_t resident, int64_t max_items);

int router_splits(int64_t T, int H);
hipError_t launch_router_logits(const uint16_t* x, const float* wr, float* part, int T, int H,
                                int splits, hipStream_t stream);
hipError_t launch_select(const float* part, int splits, const float* sel_bias, int32_t* ids,
                         float* w, int T, int G, int topk_groups, int topk, int renormalize,
                         hipStream_t stream);
hipError_t launch_replay(const float* part, int splits, const int32_t* ids, float* w, int T,
                         int E, int topk, int renormalize, hipStream_t stream);

hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int32_t* counts, int32_t* offsets,
                          int32_t* perm_src, int32_t* perm_dst, int32_t* chunk_hist,
                          hipStream_t stream);

int ffn_choose_mb(int64_t rows, int E);
int ffn_rows_per_tile(int mb);
int ffn_out_cols_per_item(bool swiglu);
// The plan (int32): [0] m-tile count, [4 ..] five arrays of max_tiles entries
// (expert, first row, rows, first m-tile of the tile's expert, m-tiles of the
// tile's expert), then the round counters of the blocked item order
// (plan_sync_ints(max_tiles) entries, zeroed by the plan kernel when `sync`).
constexpr int kPlanSyncPerTile = 32;  // counters per m-tile and GEMM
constexpr int64_t plan_sync_ints(int64_t max_tiles) { return 2 * kPlanSyncPerTile * max_tiles; }
constexpr int64_t plan_ints(int64_t max_tiles) { return 4 + 5 * max_tiles + plan_sync_ints(max_tiles); }
hipError_t launch_tile_plan(const int32_t* offsets, int E, int bmax, int32_t* plan, int max_tiles,
                            bool sync, hipStream_t stream);
// whether the bf16 grouped GEMMs at m-tile height 16 * mb walk their items
// in the blocked order (and need the plan's round counters zeroed)
bool ffn_blocked_order(int mb);
// Expert LoRA second factor for the bf16 expert GEMMs (t == nullptr: none).
struct LoraArgs {
  const uint16_t* t = nullptr;  // [rows, rank] bf16, scaled first factor
  const uint16_t* b = nullptr;  // [E, n_total, rank] bf16
  int64_t b_stride = 0;         // elements per expert of b
  int rank = 0;
};
// Sizes the checked build verifies indices against (unused otherwise):
// permuted rows (pairs), rows of A, experts.
struct GemmBounds {
  int64_t n_rows = 0;
  int64_t n_src = 0;
  int n_experts = 0;
};
hipError_t launch_grouped_gemm(int mb, bool swiglu, const uint16_t* A, const int32_t* gather,
                               int topk, const uint16_t* W, int64_t wstride, uint16_t* C,
                               const int32_t* plan, int max_tiles, int K, int n_out, int up_row0,
                               int packed, const LoraArgs& lora, int64_t max_items,
                               hipStream_t stream, bool stream_weights, const GemmBounds& bounds);
// whether the gate/up GEMM of a batch of `rows` (token, expert) pairs over E
// experts loads its weights non-temporally (only the 192-row tiles differ)
bool ffn_stream_weights(int64_t rows, int E);
hipError_t launch_lora_a(const uint16_t* X, const int32_t* gather, int topk, const uint16_t* La,
                         int K, int rank, float scale, uint16_t* t, const int32_t* plan,
                         int max_tiles, hipStream_t stream);
hipError_t launch_pack_weights(const uint16_t* src, uint16_t* dst, int E, int N, int K,
                               hipStream_t stream);

int ffn_fp8_choose_mb(int64_t rows, int E);
hipError_t launch_grouped_gemm_fp8(int mb, bool swiglu, const uint16_t* A, const int32_t* gather,
                                   int topk, const uint8_t* Q, const float* scales, int64_t qstride,
                                   int N, uint16_t* C, const int32_t* plan, int max_tiles, int K,
                                   int n_out, int up_row0, int64_t max_items, hipStream_t stream,
                                   const GemmBounds& bounds);
// 128/192-row tiles (mb 8 or 12) of the fp8 path, run by the bf16 kernel's
// 64-k stage pipeline (ffn.hip)
hipError_t launch_grouped_gemm_fp8_paired(int mb, bool swiglu, const uint16_t* A,
                                          const int32_t* gather, int topk, const uint8_t* Q,
                                          const float* scales, int64_t qstride, int N, uint16_t* C,
                                          const int32_t* plan, int max_tiles, int K, int n_out,
                                          int up_row0, int64_t max_items, hipStream_t stream,
                                          const GemmBounds& bounds);
hipError_t launch_quantize_fp8(const uint16_t* w, uint8_t* q, float* scales, int E, int N, int K,
                               hipStream_t stream);

// Checked builds: each translation unit's check-flag word, read and cleared
// (always 0 in the normal build).
uint32_t check_flags_permute();
uint32_t check_flags_ffn();
uint32_t check_flags_combine();

hipError_t launch_combine(const uint16_t* y, const int32_t* perm_dst, const float* w,
                          uint16_t* out, int T, int H, int topk, float scale, hipStream_t stream);

}  // namespace beam
