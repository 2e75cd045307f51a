// Expert SwiGLU MLPs with FP8 (E4M3FN) per-channel weights on gfx950.
//
// The vLLM recipe "Beam-1.0-501B-A23B" lists an FP8 variant with per-channel
// weights and an unquantized router.  Here each expert matrix row n (an
// output channel) carries one fp32 scale s_n and E4M3FN codes q_n,k with
// w_n,k ~ s_n * q_n,k.  Activations stay bf16: the GEMM streams half the
// bytes of the bf16 weights, widens the codes to bf16 in registers (exact:
// every E4M3FN value is a bf16 value) and applies s_n to the fp32 accumulator
// column in the epilogue: y_n = s_n * sum_k x_k q_n,k, which is the product
// with the dequantised weights up to fp32 rounding order.
//
// Packed layout (moe_quantize_fp8): each expert's [N, K] code matrix is
// stored as [N/16][K/64][2][64 lanes][8 bytes]; entry (b, s, h, l) holds row
// 16b + l%16 at k = 64s + 32h + 8(l/16) .. +7.  One 1 KB direct load
// therefore brings 16 rows x 64 k, and its two 512-byte halves are the
// operands of two consecutive 32-wide MFMA k-steps in the
// v_mfma_f32_16x16x32_bf16 lane order, each read with a linear 8-byte LDS
// read per lane.
//
// Batches of 128/192-row m-tiles run the bf16 kernel's 64-k stage pipeline
// (ffn.hip, launch_grouped_gemm_fp8_paired).  This file holds the quantiser
// and the 32-row configuration for decode-sized batches: a direct-to-LDS
// ring of 64-k stages with per-wave vmcnt waits, one barrier per stage,
// persistent XCD-dealt items and an LDS-staged epilogue, two workgroups per
// CU.
#include "common.h"
#include "kernels.h"

namespace beam {

namespace {

constexpr int kStageK = 64;   // k per stage (one fp8 fragment, two MFMA k-steps)
constexpr int kFragB = 1024;  // bytes of one direct load

// E4M3FN code of an fp32 value with |v| <= 448, round to nearest even.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {                      // below 2^-6: multiples of 2^-9
    code = (uint32_t)rintf(a * 512.0f);     // exact scaling, RNE (8 -> 2^-6)
  } else {
    uint32_t b = __float_as_uint(a);
    b = (b + 0x7ffffu + ((b >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, RNE
    code = b - (120u << 3);                       // rebias 127 -> 7
  }
  return sign | code;
}

}  // namespace

// One workgroup per (expert, 16-row block) of a [E, N, K] bf16 matrix:
// per-row absmax -> scale = absmax / 448 (1 for a zero row), codes of
// clamp(w / scale, +-448), written in the packed layout above.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ w,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scales, int N,
                                                           int K) {
  __shared__ float s_scale[16];
  const int blocks = N / 16;
  const int e = blockIdx.x / blocks, b = blockIdx.x - e * blocks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* W = w + ((size_t)e * N + (size_t)b * 16) * K;
  for (int rr = wave; rr < 16; rr += 4) {
    float m = 0.f;
    for (int k = lane * 8; k < K; k += 512) {
      const uint4 v = ld16(W + (size_t)rr * K + k);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        m = fmaxf(m, fmaxf(fabsf(bf16_to_f32(u[c] & 0xffffu)), fabsf(bf16_to_f32(u[c] >> 16))));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) {
      const float s = m > 0.f ? m / 448.0f : 1.0f;
      s_scale[rr] = s;
      scales[(size_t)e * N + b * 16 + rr] = s;
    }
  }
  __syncthreads();
  const int nks = K / kStageK;
  uint8_t* Q = q + ((size_t)e * N + (size_t)b * 16) * K;  // this block's packed bytes
  for (int c = threadIdx.x; c < nks * 64; c += 256) {
    const int st = c >> 6, l = c & 63, r = l & 15, g = l >> 4;
    const float s = s_scale[r];
    const uint16_t* row = W + (size_t)r * K + st * kStageK + 8 * g;
    const uint4 lo = ld16(row), hi = ld16(row + 32);
    const uint32_t u[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t pair = u[2 * i + h];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float v = bf16_to_f32(p ? pair >> 16 : pair & 0xffffu) / s;
          v = fminf(fmaxf(v, -448.0f), 448.0f);
          word |= e4m3_rne(v) << (8 * (2 * h + p));
        }
      }
      out[i] = word;
    }
    uint8_t* frag = Q + (size_t)st * kFragB + l * 8;
    *reinterpret_cast<uint2*>(frag) = make_uint2(out[0], out[1]);        // k 64st + 8g ..
    *reinterpret_cast<uint2*>(frag + 512) = make_uint2(out[2], out[3]);  // k 64st + 32 + 8g ..
  }
}

// ---------------------------------------------------------------------------
// The waves form RG row groups x NW / RG column groups over the item's 16
// weight-row blocks (as in ffn.hip): a wave computes RB of the NRB row blocks
// (from block row_off) for NCBW column blocks and loads NCBW / RG of those
// blocks' weight fragments.
constexpr int kItemBlocks = 16;

template <int NRB, int RB, int MB, int NW, int RG, int S, bool SWIGLU>
__device__ __forceinline__ void fp8_item_rows(const uint16_t* __restrict__ A,
                                              const int32_t* __restrict__ gather, int topk,
                                              const uint8_t* __restrict__ Qe,
                                              const float* __restrict__ Se,
                                              uint16_t* __restrict__ C, int K, int n_out,
                                              int up_row0, int row0, int nrows, int ntile,
                                              uint8_t* lds, int wave, int lane, int row_off) {
  constexpr int CG = NW / RG;
  constexpr int NCBW = kItemBlocks / CG;
  constexpr int NBL = NCBW / RG;
  constexpr int D = S - 1;
  constexpr int AOFF = kItemBlocks * kFragB;      // slot = B fragments, then A (2 per block)
  constexpr int SLOT = AOFF + 2 * MB * kFragB;
  constexpr int HALF = SWIGLU ? NCBW / 2 : NCBW;
  constexpr int WCOLS = CG * HALF * 16;
  constexpr int AMAX = (NRB + NW - 1) / NW;
  constexpr int RBX = RB > 0 ? RB : 1;
  static_assert(CG * RG == NW && NCBW * CG == kItemBlocks && NBL * RG == NCBW, "work split");
  const int r = lane & 15, g = lane >> 4;
  const int cg = wave % CG, rg = wave / CG;
  const int nk = K / kStageK;
  const int na = (NRB - wave + NW - 1) / NW;      // A row blocks this wave loads

  // A rows of a 64-k stage go to LDS as whole 128-byte lines: per 16-row
  // block, rows 0-7 then rows 8-15 (1 KB each), lane l fetching row
  // 8 hf + l / 8 and the 16-byte chunk that the swizzle places at position
  // l % 8 of the row (the bf16 GEMM's paired layout, ffn.hip).
  int asrow[AMAX > 0 ? AMAX : 1][2];
#pragma unroll
  for (int j = 0; j < AMAX; ++j) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      int row = (wave + NW * j) * 16 + hf * 8 + (lane >> 3);
      row = row < nrows ? row : nrows - 1;        // rows past the tile repeat its last row
      asrow[j][hf] = gather ? gather[row0 + row] / topk : row0 + row;
    }
  }
  auto asrc = [&](int j, int hf, int st) {
    const int rho = hf * 8 + (lane >> 3);
    return A + (size_t)asrow[j][hf] * K + st * kStageK + 8 * ((lane & 7) ^ ((rho >> 1) & 7));
  };
  // this lane's MFMA operand (row r, logical chunk g) inside a row block's
  // 2 KB; the second 32-k half (chunk 4 + g) flips bit 6
  const int aoff = (r >> 3) * kFragB + (r & 7) * 128 + ((g ^ ((r >> 1) & 7)) << 4);
  auto weight_row = [&](int cb) {
    if (SWIGLU) {
      const int j = cb % HALF;
      return ntile * WCOLS + cg * HALF * 16 + j * 16 + r + (cb >= HALF ? up_row0 : 0);
    }
    return ntile * WCOLS + cg * NCBW * 16 + cb * 16 + r;
  };
  const uint8_t* bsrc[NBL];
#pragma unroll
  for (int t = 0; t < NBL; ++t) {
    const int wrow = weight_row(rg + RG * t);
    bsrc[t] = Qe + (size_t)((wrow - r) >> 4) * nk * kFragB + lane * 16;
  }
  float scale[NCBW];
#pragma unroll
  for (int cb = 0; cb < NCBW; ++cb) scale[cb] = Se[weight_row(cb)];
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);
  const uint32_t b_base = lds0 + (cg * NCBW + rg) * kFragB;
  const uint32_t a_base = lds0 + AOFF + wave * 2 * kFragB;

  auto issue = [&](int st) {
    const uint32_t so = (uint32_t)((st % S) * SLOT);
#pragma unroll
    for (int t = 0; t < NBL; ++t) {
      if constexpr (MB <= 8)  // weight streams read once: non-temporal (as in ffn.hip)
        lds_dma16_nt(bsrc[t] + (size_t)st * kFragB, b_base + so + RG * t * kFragB);
      else
        lds_dma16(bsrc[t] + (size_t)st * kFragB, b_base + so + RG * t * kFragB);
    }
#pragma unroll
    for (int j = 0; j < AMAX; ++j)
      if (j < na) {
        const uint32_t ao = a_base + so + NW * j * 2 * kFragB;
        lds_dma16(asrc(j, 0, st), ao);
        lds_dma16(asrc(j, 1, st), ao + kFragB);
      }
  };

  f32x4_t acc[RBX][NCBW];
#pragma unroll
  for (int i = 0; i < RBX; ++i)
#pragma unroll
    for (int cb = 0; cb < NCBW; ++cb) acc[i][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < D; ++st)
    if (st < nk) issue(st);

  for (int kt = 0; kt < nk; ++kt) {
    const int ahead = min(D - 1, nk - 1 - kt);
    if (na == AMAX) wait_stage<D - 1, NBL + 2 * AMAX>(ahead);
    else wait_stage<D - 1, NBL + 2 * (AMAX > 0 ? AMAX - 1 : 0)>(ahead);
    stage_barrier();  // stage kt visible to all waves; slot (kt - 1) % S is free
    if (kt + D < nk) issue(kt + D);
    if constexpr (RB > 0) {
      const uint8_t* sl = lds + (kt % S) * SLOT;
      bf16x8_t blo[NCBW], bhi[NCBW];
#pragma unroll
      for (int cb = 0; cb < NCBW; ++cb) {
        const uint2 lo = *reinterpret_cast<const uint2*>(sl + (cg * NCBW + cb) * kFragB + 8 * lane);
        const uint2 hi =
            *reinterpret_cast<const uint2*>(sl + (cg * NCBW + cb) * kFragB + 512 + 8 * lane);
        const uint32_t w4[4] = {lo.x, lo.y, hi.x, hi.y};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[i], 1.0f, false));
          o[2 * i + 1] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[i], 1.0f, true));
        }
        blo[cb] = as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
        bhi[cb] = as_bf16x8(make_uint4(o[4], o[5], o[6], o[7]));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(
              sl + AOFF + 2 * (row_off + i) * kFragB + (aoff ^ (h << 6))));
#pragma unroll
          for (int cb = 0; cb < NCBW; ++cb)
            acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, h ? bhi[cb] : blo[cb],
                                                                 acc[i][cb], 0, 0, 0);
        }
      }
    }
  }
  wait_lgkm0();
  stage_barrier();  // every wave is done with the ring

  // epilogue through LDS, columns scaled by their channel scale (see ffn.hip)
  constexpr int TSTRIDE = WCOLS + 8;
  static_assert(16 * NRB * TSTRIDE * 2 <= S * SLOT, "epilogue tile fits the ring");
  uint16_t* tile = reinterpret_cast<uint16_t*>(lds);
  if constexpr (RB > 0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const int col = cg * HALF * 16 + j * 16 + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = (row_off + i) * 16 + 4 * g + v;
          float o;
          if (SWIGLU) {
            const float gt = acc[i][j][v] * scale[j], up = acc[i][j + HALF][v] * scale[j + HALF];
            o = silu_mul(gt, up);
          } else {
            o = acc[i][j][v] * scale[j];
          }
          const uint32_t bb = f32_to_bf16(o);
          const uint32_t nb = __shfl_xor(bb, 1);
          if ((r & 1) == 0)
            *reinterpret_cast<uint32_t*>(tile + row * TSTRIDE + col) = bb | (nb << 16);
        }
      }
    }
  }
  wait_lgkm0();
  stage_barrier();
  constexpr int CPR = WCOLS / 8;
  const int nchunks = nrows * CPR;
  uint16_t* out = C + (size_t)row0 * n_out + ntile * WCOLS;
  for (int c = wave * 64 + lane; c < nchunks; c += NW * 64) {
    const int row = c / CPR, cc = c - row * CPR;
    st16(out + (size_t)row * n_out + cc * 8,
         *reinterpret_cast<const uint4*>(tile + row * TSTRIDE + cc * 8));
  }
  wait_lgkm0();
  stage_barrier();
}

template <int NRB, int MB, int NW, int RG, int S, bool SWIGLU>
__device__ __forceinline__ void fp8_item(const uint16_t* A, const int32_t* gather, int topk,
                                         const uint8_t* Qe, const float* Se, uint16_t* C, int K,
                                         int n_out, int up_row0, int row0, int nrows, int ntile,
                                         uint8_t* lds, int wave, int lane) {
  static_assert(RG == 1, "the 32-row configuration has one row group");
  fp8_item_rows<NRB, NRB, MB, NW, 1, S, SWIGLU>(A, gather, topk, Qe, Se, C, K, n_out, up_row0, row0,
                                                nrows, ntile, lds, wave, lane, 0);
}

template <int N, int MB, int NW, int RG, int S, bool SWIGLU>
__device__ __forceinline__ void fp8_dispatch(int nrb, const uint16_t* A, const int32_t* gather,
                                             int topk, const uint8_t* Qe, const float* Se,
                                             uint16_t* C, int K, int n_out, int up_row0, int row0,
                                             int nrows, int ntile, uint8_t* lds, int wave,
                                             int lane) {
  if constexpr (N > MB) {
    return;
  } else {
    if (nrb == N)
      fp8_item<N, MB, NW, RG, S, SWIGLU>(A, gather, topk, Qe, Se, C, K, n_out, up_row0, row0,
                                         nrows, ntile, lds, wave, lane);
    else
      fp8_dispatch<N + 1, MB, NW, RG, S, SWIGLU>(nrb, A, gather, topk, Qe, Se, C, K, n_out,
                                                 up_row0, row0, nrows, ntile, lds, wave, lane);
  }
}

template <int MB, int NW, int RG, int S, bool SWIGLU>
__global__ __launch_bounds__(NW * 64, 1) void stream_gemm_fp8_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather, int topk,
    const uint8_t* __restrict__ Q, const float* __restrict__ scales, int64_t q_expert_stride,
    int N, uint16_t* __restrict__ C, const int32_t* __restrict__ plan, int max_tiles, int K,
    int n_out, int up_row0) {
  constexpr int SLOT = (kItemBlocks + 2 * MB) * kFragB;
  constexpr int WCOLS = (SWIGLU ? kItemBlocks / 2 : kItemBlocks) * 16;
  static_assert(WCOLS == (SWIGLU ? 128 : 256), "item width matches the bf16 kernels");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * SLOT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = plan[0];
  const int* plan_expert = plan + 4;
  const int* plan_row0 = plan_expert + max_tiles;
  const int* plan_rows = plan_row0 + max_tiles;
  const int nt_n = n_out / WCOLS;
  const int total = ntiles * nt_n;
  const int grid = balanced_grid(total, gridDim.x), per_xcd = grid / 8;
  if ((int)blockIdx.x >= grid) return;  // whole workgroup: blockIdx is uniform
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  for (int round = 0;; round += grid) {
    const int q = round + xcd * per_xcd + slot;
    if (q >= total) break;
    const int tile = q / nt_n;
    const int e = plan_expert[tile], row0 = plan_row0[tile], nrows = plan_rows[tile];
    fp8_dispatch<1, MB, NW, RG, S, SWIGLU>((nrows + 15) >> 4, A, gather, topk,
                                             Q + (size_t)e * q_expert_stride,
                                             scales + (size_t)e * N, C, K, n_out, up_row0, row0,
                                             nrows, q - tile * nt_n, lds, wave, lane);
  }
}

template <int MB, int NW, int RG, int S, bool SWIGLU>
static hipError_t launch_fp8(const uint16_t* A, const int32_t* gather, int topk, const uint8_t* Q,
                             const float* scales, int64_t qstride, int N, uint16_t* C,
                             const int32_t* plan, int max_tiles, int K, int n_out, int up_row0,
                             int64_t max_items, hipStream_t stream) {
  auto kern = stream_gemm_fp8_kernel<MB, NW, RG, S, SWIGLU>;
  static int per_cu = 0, cus = 0;
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
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), 0, stream, A, gather, topk, Q,
                     scales, qstride, N, C, plan, max_tiles, K, n_out, up_row0);
  return hipGetLastError();
}

// m-tile height of the fp8 path: 32 rows for decode-sized batches (the small
// activation ring lets two workgroups share a CU), else as the bf16 path.
int ffn_fp8_choose_mb(int64_t rows, int E) {
  const int64_t mean = rows / (E > 0 ? E : 1);
  if (mean <= 24) return 2;
  if (mean <= 80) return 8;
  return 12;
}


hipError_t launch_grouped_gemm_fp8(int mb, bool swiglu, const uint16_t* A, const int32_t* gather,
                                   int topk, const uint8_t* Q, const float* scales, int64_t qstride,
                                   int N, uint16_t* C, const int32_t* plan, int max_tiles, int K,
                                   int n_out, int up_row0, int64_t max_items, hipStream_t stream,
                                   const GemmBounds& bounds) {
#define BEAM_FP8_CASE(MBV, NWV, RGV, SV)                                                      \
  case MBV:                                                                                     \
    return swiglu ? launch_fp8<MBV, NWV, RGV, SV, true>(A, gather, topk, Q, scales, qstride,  \
                                                          N, C, plan, max_tiles, K, n_out,      \
                                                          up_row0, max_items, stream)           \
                  : launch_fp8<MBV, NWV, RGV, SV, false>(A, gather, topk, Q, scales, qstride, \
                                                           N, C, plan, max_tiles, K, n_out,     \
                                                           up_row0, max_items, stream);
  switch (mb) {
    BEAM_FP8_CASE(2, 4, 1, 4)
    case 8:
    case 12:
      return launch_grouped_gemm_fp8_paired(mb, swiglu, A, gather, topk, Q, scales, qstride, N, C,
                                            plan, max_tiles, K, n_out, up_row0, max_items, stream,
                                            bounds);
    default:
      return hipErrorInvalidValue;
  }
#undef BEAM_FP8_CASE
}

hipError_t launch_quantize_fp8(const uint16_t* w, uint8_t* q, float* scales, int E, int N, int K,
                               hipStream_t stream) {
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)(E * (N / 16))), dim3(256), 0, stream, w,
                     q, scales, N, K);
  return hipGetLastError();
}

}  // namespace beam
