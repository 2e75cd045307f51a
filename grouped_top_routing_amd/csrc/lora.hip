// Expert LoRA, first factor: t = s * (A_r . La_e^T) for every permuted row.
//
// "Beam 1.0" miles recipes, section 5.5 "LoRA": an adapter of rank 16 and
// alpha 32 on every routed expert.  An adapted expert weight W [out, in]
// computes W a + s * Lb (La a) with La [rank, in], Lb [out, rank] and
// s = alpha / rank.  The second factor is applied inside the expert GEMMs'
// epilogue (ffn.hip); this kernel produces the rank-wide intermediate
// t [rows, rank] = bf16(s * fp32(a . La^T)) in the permuted row order.
//
// The grouped GEMM here is tall and thin (N = rank = 16..64, K = H or I), so
// it is bound by reading its input rows once: one workgroup per m-tile of the
// same plan the expert GEMMs use (tiles never straddle experts), each wave
// taking 16-row blocks of the tile.  Every k step is one
// v_mfma_f32_16x16x32_bf16 per 16 ranks, with both operands loaded straight
// from global memory in the MFMA's lane order (the input rows are gathered
// through perm_src for the gate/up adapter, exactly like the GEMM's A loads).
#include "common.h"
#include "kernels.h"

namespace beam {

namespace {

constexpr int kK = 32;  // k per MFMA

constexpr int kLoraWaves = 8;  // waves per workgroup, each on its own 16-row blocks

template <int RB>
__global__ __launch_bounds__(kLoraWaves * 64) void lora_a_kernel(const uint16_t* __restrict__ X,
                                                     const int32_t* __restrict__ gather, int topk,
                                                     const uint16_t* __restrict__ La, int K,
                                                     float scale, uint16_t* __restrict__ t,
                                                     const int32_t* __restrict__ plan,
                                                     int max_tiles) {
  constexpr int R = RB * 16;  // rank
  const int tile = blockIdx.x;
  if (tile >= plan[0]) return;
  const int* plan_expert = plan + 4;
  const int e = plan_expert[tile];
  const int row0 = plan_expert[max_tiles + tile];
  const int nrows = plan_expert[2 * max_tiles + tile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* La_e = La + (size_t)e * R * K;
  const int nblk = (nrows + 15) >> 4;
  for (int b = wave; b < nblk; b += kLoraWaves) {
    int row = b * 16 + r;
    row = row < nrows ? row : nrows - 1;
    const int src = gather ? gather[row0 + row] / topk : row0 + row;
    const uint16_t* ap = X + (size_t)src * K + 8 * g;
    const uint16_t* bp = La_e + (size_t)r * K + 8 * g;  // rank r of each 16-rank block
    f32x4_t acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // K is a multiple of 128 (hidden % 256 == 0, intermediate % 128 == 0):
    // 8 k-steps per group when K allows (all their loads issued before the
    // first MFMA), else 4
    auto group = [&](int k0, auto steps) {
      constexpr int U = decltype(steps)::value;
      uint4 av[U], bv[U][RB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        av[u] = ld16(ap + k0 + u * kK);
#pragma unroll
        for (int j = 0; j < RB; ++j) bv[u][j] = ld16(bp + (size_t)j * 16 * K + k0 + u * kK);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < RB; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(bv[u][j]),
                                                           acc[j], 0, 0, 0);
    };
    if (K % (8 * kK) == 0) {
      for (int k0 = 0; k0 < K; k0 += 8 * kK) group(k0, std::integral_constant<int, 8>{});
    } else {
      for (int k0 = 0; k0 < K; k0 += 4 * kK) group(k0, std::integral_constant<int, 4>{});
    }
    // lane holds rows 4g..4g+3 of rank column j*16 + r
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rr = b * 16 + 4 * g + v;
      if (rr < nrows) {
#pragma unroll
        for (int j = 0; j < RB; ++j)
          t[(size_t)(row0 + rr) * R + j * 16 + r] = (uint16_t)f32_to_bf16(scale * acc[j][v]);
      }
    }
  }
}

}  // namespace

hipError_t launch_lora_a(const uint16_t* X, const int32_t* gather, int topk, const uint16_t* La,
                         int K, int rank, float scale, uint16_t* t, const int32_t* plan,
                         int max_tiles, hipStream_t stream) {
  const dim3 grid((unsigned)max_tiles), block(kLoraWaves * 64);
  switch (rank) {
    case 16:
      hipLaunchKernelGGL(lora_a_kernel<1>, grid, block, 0, stream, X, gather, topk, La, K, scale,
                         t, plan, max_tiles);
      break;
    case 32:
      hipLaunchKernelGGL(lora_a_kernel<2>, grid, block, 0, stream, X, gather, topk, La, K, scale,
                         t, plan, max_tiles);
      break;
    case 48:
      hipLaunchKernelGGL(lora_a_kernel<3>, grid, block, 0, stream, X, gather, topk, La, K, scale,
                         t, plan, max_tiles);
      break;
    case 64:
      hipLaunchKernelGGL(lora_a_kernel<4>, grid, block, 0, stream, X, gather, topk, La, K, scale,
                         t, plan, max_tiles);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace beam
