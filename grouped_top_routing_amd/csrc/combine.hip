// Weighted un-permute of the Beam-1.0 MoE block on gfx950.
//
// "Welcome Beam: a 501B open model you can own, customize, and scale", section
// "Mixture of Experts": a token's output sums its chosen experts' outputs,
// each weighted by its score over the sum of the chosen scores, and multiplies
// the sum by 2.5; there is no shared expert.
//
// out[t, :] = bf16( scale * sum_j w[t, j] * y[perm_dst[t*topk + j], :] ), the
// sum taken in fp32 in slot order.  Workgroup (t, c) handles token t's c-th
// slice of columns (one slice for large batches; small batches split each
// row so that enough workgroups run); every thread owns 8 consecutive
// columns, so each of the token's rows is read with coalesced 16-byte loads
// and the output row is written the same way.
#include "common.h"
#include "kernels.h"

namespace beam {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ perm_dst,
                                                      const float* __restrict__ w,
                                                      uint16_t* __restrict__ out, int H, int topk,
                                                      float scale) {
  const int t = blockIdx.x;
  const int per = (H / 8 + gridDim.y - 1) / gridDim.y;  // 16-byte column groups per slice
  const int v0 = blockIdx.y * per, v1 = min(v0 + per, H / 8);
  int rows[8];
  float wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < topk ? perm_dst[(size_t)t * topk + j] : -1;
    if (rows[j] >= 0)
      rows[j] = BEAM_CLAMP(rows[j], 0, (int64_t)gridDim.x * topk - 1, kCheckCombineRow);
    wt[j] = j < topk ? w[(size_t)t * topk + j] : 0.f;
  }
  for (int v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
    // all of the token's row loads in flight before the sums (each y row is
    // read once: non-temporal)
    uint4 q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      q[j] = rows[j] >= 0 ? ld16_nt(y + (size_t)rows[j] * H + 8 * v) : make_uint4(0u, 0u, 0u, 0u);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] >= 0) {
        const uint32_t u[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * c] += wt[j] * bf16_to_f32(u[c] & 0xffffu);
          acc[2 * c + 1] += wt[j] * bf16_to_f32(u[c] >> 16);
        }
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c] = f32_to_bf16(scale * acc[2 * c]) | (f32_to_bf16(scale * acc[2 * c + 1]) << 16);
    st16(out + (size_t)t * H + 8 * v, make_uint4(o[0], o[1], o[2], o[3]));
  }
}

BEAM_DEFINE_CHECK_READER(check_flags_combine)

hipError_t launch_combine(const uint16_t* y, const int32_t* perm_dst, const float* w,
                          uint16_t* out, int T, int H, int topk, float scale, hipStream_t stream) {
  // slices of at least 128 column groups, enough of them for ~1024 workgroups
  const int groups = H / 8;
  int slices = (1024 + T - 1) / (T > 0 ? T : 1);
  const int max_slices = (groups + 127) / 128;
  if (slices > max_slices) slices = max_slices;
  if (slices < 1) slices = 1;
  // whole rows: 256 threads; row slices: 128
  const int threads = slices == 1 ? 256 : 128;
  hipLaunchKernelGGL(combine_kernel, dim3(T, slices), dim3(threads), 0, stream, y, perm_dst, w, out,
                     H, topk, scale);
  return hipGetLastError();
}

}  // namespace beam
