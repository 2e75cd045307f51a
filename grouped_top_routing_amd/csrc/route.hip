// Router of the Beam-1.0 MoE block on gfx950.
//
// "Welcome Beam: a 501B open model you can own, customize, and scale", section
// "Mixture of Experts": every expert gets a sigmoid score; the experts form 8
// groups of 32; the 4 groups with the largest sum of their two best scores are
// kept; the 8 best experts inside them are chosen; their outputs are later
// summed with weights proportional to their scores (summing to one).  The router runs in FP32 (same page,
// section "Residual Stream"; "Beam 1.0" miles recipes, section 1: router weights
// stay FP32).
//
// Two kernels:
//   router_logits_kernel  k-split partial logits x . W_r^T on the bf16 matrix
//                         cores with an exact three-way bf16 split of the fp32
//                         weights (fp32 products, fp32 accumulation).
//   select_kernel<G>      one wavefront per token: sums the partials, sigmoid,
//                         group top-two sums
//                         by butterfly shuffles, group ranking, then topk
//                         rounds of a wavefront-wide arg-max; writes ids and
//                         combine weights.
#include "common.h"
#include "kernels.h"

namespace beam {

// ---------------------------------------------------------------------------
// Logits on the bf16 matrix cores, fp32-exact.
//
// Every fp32 router weight w splits exactly into three bf16 values by
// truncation: hi = w with its low 16 bits cleared, mid likewise from w - hi,
// lo = w - hi - mid (at most 8 significant bits left, so it is a bf16 value).
// The activations are bf16, so each product x*hi, x*mid, x*lo is exact in the
// fp32 accumulator of v_mfma_f32_16x16x32_bf16, and logit = sum over k of
// x*hi + x*mid + x*lo is an fp32-accumulated dot product of the exact fp32
// weights -- at a third of the bf16 rate, ~5x the fp32 matrix rate.
//
// Tile: 128 tokens x 256 experts per workgroup, k split over blockIdx.y (the
// partial sums are added in split order by select_kernel, so results do not
// depend on the grid).  Wave w of 8 owns experts [32w, 32w + 32) and all 128
// tokens (two waves per SIMD).  x fragments (16 tokens x 32 k, MFMA lane
// order) stream into an LDS ring with direct loads shared by the 8 waves;
// each wave's weights go straight to registers (no other wave needs them),
// both kRD stages ahead.
// ---------------------------------------------------------------------------
constexpr int kRT = 128;              // tokens per workgroup
constexpr int kRB = kRT / 16;         // token row blocks
// Stages in flight (template parameter kRD): 5 from 4096 tokens up (skewed
// 16K-token batch: route 174 -> 146 us), 3 below (decode and 512 tokens are
// 1-2 us slower with 5; the results are the same bits either way).
constexpr int kRDSmall = 3, kRDLarge = 5;
constexpr int64_t kRDLargeFrom = 4096;
constexpr int kRW = 8;                // waves per workgroup
constexpr int kRC = 256 / kRW / 16;   // 16-expert column blocks per wave
constexpr int kRL = kRB / kRW + 2 * kRC;  // loads per wave per stage: x fragments + weight halves

__device__ __forceinline__ uint32_t hi16(uint32_t u) { return u & 0xffff0000u; }

// Three bf16x8 operands (hi, mid, lo) from 8 fp32 weights held in two uint4.
__device__ __forceinline__ void split3(const uint4& w0, const uint4& w1, bf16x8_t& ph,
                                       bf16x8_t& pm, bf16x8_t& pl) {
  const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = hi16(w[i]);
    const float r1 = __uint_as_float(w[i]) - __uint_as_float(h[i]);
    m[i] = hi16(__float_as_uint(r1));
    l[i] = __float_as_uint(r1 - __uint_as_float(m[i]));  // low 16 bits are zero
  }
  uint4 H, M, L;
  H.x = (h[0] >> 16) | h[1]; H.y = (h[2] >> 16) | h[3]; H.z = (h[4] >> 16) | h[5]; H.w = (h[6] >> 16) | h[7];
  M.x = (m[0] >> 16) | m[1]; M.y = (m[2] >> 16) | m[3]; M.z = (m[4] >> 16) | m[5]; M.w = (m[6] >> 16) | m[7];
  L.x = (l[0] >> 16) | l[1]; L.y = (l[2] >> 16) | l[3]; L.z = (l[4] >> 16) | l[5]; L.w = (l[6] >> 16) | l[7];
  ph = as_bf16x8(H);
  pm = as_bf16x8(M);
  pl = as_bf16x8(L);
}

template <int kRD>
__global__ __launch_bounds__(kRW * 64, 1) void router_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, float* __restrict__ part,
    int T, int H, int kchunk) {
  constexpr int kRS = kRD + 1;  // LDS ring slots
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kRS * kRB * 1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int t0 = tile * kRT;
  const int kbeg = split * kchunk;
  const int nk = kchunk / 32;

  // x fragments this wave loads: row blocks wave, wave + kRW, ...
  constexpr int XJ = kRB / kRW;
  const uint16_t* xsrc[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    int t = t0 + (wave + kRW * j) * 16 + r;
    t = t < T ? t : T - 1;  // rows past T repeat the last token (computed, never stored)
    xsrc[j] = x + (size_t)t * H + kbeg + 8 * g;
  }
  // weight rows of this lane: expert 16 * (kRC * wave + cb) + r, k chunk 8g
  const float* wsrc[kRC];
#pragma unroll
  for (int cb = 0; cb < kRC; ++cb)
    wsrc[cb] = wr + (size_t)(16 * (kRC * wave + cb) + r) * H + kbeg + 8 * g;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);

  uint4 wreg[kRD][kRC][2];
  auto issue = [&](int st, uint4 (&wr_)[kRC][2]) {
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((st % kRS) * kRB * 1024));
#pragma unroll
    for (int j = 0; j < XJ; ++j) lds_dma16(xsrc[j] + st * 32, sl + (wave + kRW * j) * 1024);
#pragma unroll
    for (int cb = 0; cb < kRC; ++cb) {
      wr_[cb][0] = ld16(wsrc[cb] + st * 32);
      wr_[cb][1] = ld16(wsrc[cb] + st * 32 + 4);
    }
  };

  f32x4_t acc[kRB][kRC];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int cb = 0; cb < kRC; ++cb) acc[i][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < kRD; ++st)
    if (st < nk) issue(st, wreg[st]);

  // one stage: consume register set `cur`, then refill it with stage kt + kRD
  auto step = [&](int kt, uint4 (&cur)[kRC][2]) {
    wait_stage<kRD - 1, kRL>(min(kRD - 1, nk - 1 - kt));
    stage_barrier();
    const uint8_t* sl = lds + (kt % kRS) * kRB * 1024;
    bf16x8_t bh[kRC], bm[kRC], bl[kRC];
#pragma unroll
    for (int cb = 0; cb < kRC; ++cb) split3(cur[cb][0], cur[cb][1], bh[cb], bm[cb], bl[cb]);
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(sl + i * 1024 + 16 * lane));
#pragma unroll
      for (int cb = 0; cb < kRC; ++cb) {
        acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[cb], acc[i][cb], 0, 0, 0);
        acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm[cb], acc[i][cb], 0, 0, 0);
        acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[cb], acc[i][cb], 0, 0, 0);
      }
    }
    wait_lgkm0();
    if (kt + kRD < nk) issue(kt + kRD, cur);
  };
  int kt = 0;
  for (; kt + kRD <= nk; kt += kRD) {
#pragma unroll
    for (int j = 0; j < kRD; ++j) step(kt + j, wreg[j]);
  }
#pragma unroll
  for (int j = 0; j < kRD; ++j)
    if (kt + j < nk) step(kt + j, wreg[j]);

  // D layout of a 16x16 MFMA: lane holds rows 4g..4g+3 of column r
  float* out = part + (size_t)split * T * 256;
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + i * 16 + 4 * g + v;
      if (t < T) {
#pragma unroll
        for (int cb = 0; cb < kRC; ++cb)
          out[(size_t)t * 256 + 16 * (kRC * wave + cb) + r] = acc[i][cb][v];
      }
    }
}

// k splits for the logits: about 256 workgroups in all, at most 32 splits
// (the selection kernel adds the partials), each split a whole number of
// 32-wide k steps.
int router_splits(int64_t T, int H) {
  const int64_t tiles = (T + kRT - 1) / kRT;
  const int steps = H / 32;
  int64_t want = (256 + tiles - 1) / (tiles > 0 ? tiles : 1);
  if (want > 32) want = 32;
  if (want > steps) want = steps;
  int best = 1;
  for (int s = 1; s <= want; ++s)
    if (steps % s == 0) best = s;
  return best;
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

// Sum of the k-split partial logits of token t, experts 4*lane .. 4*lane+3,
// added in split order.
__device__ __forceinline__ void gather_logits(const float* __restrict__ part, int splits, int T,
                                              int t, int lane, float (&lg)[4]) {
  float4 a = *reinterpret_cast<const float4*>(part + (size_t)t * 256 + 4 * lane);
#pragma unroll 8
  for (int s = 1; s < splits; ++s) {
    const float4 b = *reinterpret_cast<const float4*>(part + ((size_t)s * T + t) * 256 + 4 * lane);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  lg[0] = a.x; lg[1] = a.y; lg[2] = a.z; lg[3] = a.w;
}

template <int G>
__global__ __launch_bounds__(256) void select_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ sel_bias,
    int32_t* __restrict__ ids, float* __restrict__ wout, int T, int topk_groups, int topk,
    int renormalize) {
  constexpr int LPG = kWave / G;  // lanes per group (group = 4 * LPG experts)
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave

  float lg[4];
  gather_logits(part, splits, T, t, lane, lg);
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

// Routing replay: scores of caller-given experts, weights only.  An id
// outside [0, E) is dropped, as the permutation drops it: its weight is 0 and
// its slot takes no part in the normalising sum (a token whose ids are all
// dropped gets weights 0).
__global__ __launch_bounds__(256) void replay_kernel(
    const float* __restrict__ part, int splits, const int32_t* __restrict__ ids,
    float* __restrict__ wout, int T, int E, int topk, int renormalize) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float my_s = 0.f;
  if (lane < topk) {
    const int e = ids[(size_t)t * topk + lane];
    if (e >= 0 && e < E) {
      float lg = 0.f;
      for (int s = 0; s < splits; ++s) lg += part[((size_t)s * T + t) * E + e];
      my_s = sigmoidf_(lg);
    }
  }
  float ssum = 0.f;
  for (int j = 0; j < topk; ++j) ssum += __shfl(my_s, j);
  if (lane < topk)
    wout[(size_t)t * topk + lane] = renormalize ? (ssum > 0.f ? my_s / ssum : 0.f) : my_s;
}

// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t* x, const float* wr, float* part, int T, int H,
                                int splits, hipStream_t stream) {
  dim3 grid((T + kRT - 1) / kRT, splits);
  if (T >= kRDLargeFrom)
    hipLaunchKernelGGL(router_logits_kernel<kRDLarge>, grid, dim3(kRW * 64), 0, stream, x, wr,
                       part, T, H, H / splits);
  else
    hipLaunchKernelGGL(router_logits_kernel<kRDSmall>, grid, dim3(kRW * 64), 0, stream, x, wr,
                       part, T, H, H / splits);
  return hipGetLastError();
}

hipError_t launch_select(const float* part, int splits, const float* sel_bias, int32_t* ids,
                         float* w, int T, int G, int topk_groups, int topk, int renormalize,
                         hipStream_t stream) {
  dim3 grid((T + 3) / 4);
#define BEAM_SELECT_CASE(GV)                                                                   \
  case GV:                                                                                     \
    hipLaunchKernelGGL(select_kernel<GV>, grid, dim3(256), 0, stream, part, splits, sel_bias,  \
                       ids, w, T, topk_groups, topk, renormalize);                            \
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

hipError_t launch_replay(const float* part, int splits, const int32_t* ids, float* w, int T,
                         int E, int topk, int renormalize, hipStream_t stream) {
  hipLaunchKernelGGL(replay_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, part, splits, ids, w,
                     T, E, topk, renormalize);
  return hipGetLastError();
}

}  // namespace beam
