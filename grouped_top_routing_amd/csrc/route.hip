// Router of the Beam-1.0 MoE block on gfx950.
//
// "Welcome Beam: a 501B open model you can own, customize, and scale", section
// "Mixture of Experts": every expert gets a sigmoid score; the experts form 8
// groups of 32; the 4 groups with the largest sum of their two best scores are
// kept; the 8 best experts inside them are chosen; their outputs are later
// combined with normalized router weights.  The router runs in FP32 (same page,
// section "Residual Stream"; "Beam 1.0" miles recipes, section 1: router weights
// stay FP32).
//
// Two kernels:
//   router_logits_kernel  logits[T, 256] = x . W_r^T on the fp32 matrix cores
//                         (v_mfma_f32_16x16x4_f32): products and sums are true
//                         fp32, bf16 activations are widened exactly.
//   select_kernel<G>      one wavefront per token: sigmoid, group top-two sums
//                         by butterfly shuffles, group ranking, then topk
//                         rounds of a wavefront-wide arg-max; writes ids and
//                         combine weights.
#include "common.h"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// logits tile: 64 tokens x 64 experts per workgroup, 4 waves; wave w owns the
// 16 experts [16w, 16w + 16) of the tile and all 64 tokens (4 row blocks).
// K advances by 32 per step: lane (r = lane % 16, g = lane / 16) holds the 8
// consecutive k values [8g, 8g + 8) of its token rows and of its expert row;
// MFMA m (m = 0..7) consumes the m-th of them, so lane group g always supplies
// the same k to both operands.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, float* __restrict__ logits,
    int T, int H, int E) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int t0 = blockIdx.x * 64;
  const int e = blockIdx.y * 64 + wave * 16 + r;

  const float* wrow = wr + (size_t)e * H + 8 * g;
  const uint16_t* xrow[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    int t = t0 + rb * 16 + r;
    t = t < T ? t : T - 1;  // clamp: rows past T are computed but never stored
    xrow[rb] = x + (size_t)t * H + 8 * g;
  }

  f32x4_t acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < H; k0 += 32) {
    const float4 w0 = *reinterpret_cast<const float4*>(wrow + k0);
    const float4 w1 = *reinterpret_cast<const float4*>(wrow + k0 + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint4 xv[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) xv[rb] = ld16(xrow[rb] + k0);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const uint32_t xw[4] = {xv[rb].x, xv[rb].y, xv[rb].z, xv[rb].w};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t half = (m & 1) ? (xw[m >> 1] >> 16) : (xw[m >> 1] & 0xffffu);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf16_to_f32(half), wv[m], acc[rb], 0, 0, 0);
      }
    }
  }

  // D layout of a 16x16 MFMA: lane holds rows 4g..4g+3 of column r.
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + rb * 16 + 4 * g + i;
      if (t < T) logits[(size_t)t * E + e] = acc[rb][i];
    }
  }
}

// ---------------------------------------------------------------------------
// selection: one wave per token, lane l owns experts 4l..4l+3 (E = 256).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ float pick4(const float (&v)[4], int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

template <int G>
__global__ __launch_bounds__(256) void select_kernel(
    const float* __restrict__ logits, const float* __restrict__ sel_bias,
    int32_t* __restrict__ ids, float* __restrict__ wout, int T, int topk_groups, int topk,
    int renormalize) {
  constexpr int LPG = kWave / G;  // lanes per group (group = 4 * LPG experts)
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave

  const float4 lv = *reinterpret_cast<const float4*>(logits + (size_t)t * 256 + 4 * lane);
  const float lg[4] = {lv.x, lv.y, lv.z, lv.w};
  float s[4], sel[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = sigmoidf_(lg[i]);
    sel[i] = sel_bias ? s[i] + sel_bias[4 * lane + i] : s[i];
  }

  // top two of this lane's four (a repeated maximum counts twice)
  float m1 = fmaxf(sel[0], sel[1]), m2 = fminf(sel[0], sel[1]);
#pragma unroll
  for (int i = 2; i < 4; ++i) {
    const float v = sel[i];
    m2 = fmaxf(m2, fminf(m1, v));
    m1 = fmaxf(m1, v);
  }
  // merge top-two pairs across the lanes of a group
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    const float b1 = __shfl_xor(m1, off);
    const float b2 = __shfl_xor(m2, off);
    m2 = fmaxf(fminf(m1, b1), fmaxf(m2, b2));
    m1 = fmaxf(m1, b1);
  }
  const float gs = m1 + m2;
  const int my_group = lane / LPG;

  // rank of this lane's group among all groups by (score desc, index asc)
  int rank = 0;
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const float o = __shfl(gs, gg * LPG);
    rank += better(o, gg, gs, my_group) ? 1 : 0;
  }
  const bool keep = rank < topk_groups;

  float cand[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cand[i] = keep ? sel[i] : -INFINITY;

  int my_id = 0;
  float my_s = 0.f, ssum = 0.f;
  for (int j = 0; j < topk; ++j) {
    float bv = cand[0];
    int bi = 4 * lane;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (cand[i] > bv) { bv = cand[i]; bi = 4 * lane + i; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const int owner = bi >> 2, slot = bi & 3;
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i == slot) cand[i] = -INFINITY;
    }
    const float sw = __shfl(pick4(s, slot), owner);
    if (lane == j) { my_id = bi; my_s = sw; }
    ssum += sw;
  }
  if (lane < topk) {
    ids[(size_t)t * topk + lane] = my_id;
    wout[(size_t)t * topk + lane] = renormalize ? my_s / ssum : my_s;
  }
}

// Routing replay: scores of caller-given experts, weights only.
__global__ __launch_bounds__(256) void replay_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ ids, float* __restrict__ wout,
    int T, int E, int topk, int renormalize) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float my_s = 0.f;
  if (lane < topk) {
    int e = ids[(size_t)t * topk + lane];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    my_s = sigmoidf_(logits[(size_t)t * E + e]);
  }
  float ssum = 0.f;
  for (int j = 0; j < topk; ++j) ssum += __shfl(my_s, j);
  if (lane < topk) wout[(size_t)t * topk + lane] = renormalize ? my_s / ssum : my_s;
}

// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t* x, const float* wr, float* logits, int T, int H,
                                int E, hipStream_t stream) {
  dim3 grid((T + 63) / 64, E / 64);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, x, wr, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_select(const float* logits, const float* sel_bias, int32_t* ids, float* w,
                         int T, int G, int topk_groups, int topk, int renormalize,
                         hipStream_t stream) {
  dim3 grid((T + 3) / 4);
#define BEAM_SELECT_CASE(GV)                                                                   \
  case GV:                                                                                     \
    hipLaunchKernelGGL(select_kernel<GV>, grid, dim3(256), 0, stream, logits, sel_bias, ids, w, \
                       T, topk_groups, topk, renormalize);                                     \
    break;
  switch (G) {
    BEAM_SELECT_CASE(1)
    BEAM_SELECT_CASE(2)
    BEAM_SELECT_CASE(4)
    BEAM_SELECT_CASE(8)
    BEAM_SELECT_CASE(16)
    BEAM_SELECT_CASE(32)
    BEAM_SELECT_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef BEAM_SELECT_CASE
  return hipGetLastError();
}

hipError_t launch_replay(const float* logits, const int32_t* ids, float* w, int T, int E,
                         int topk, int renormalize, hipStream_t stream) {
  hipLaunchKernelGGL(replay_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, ids, w, T, E,
                     topk, renormalize);
  return hipGetLastError();
}

}  // namespace beam
