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
// Work decomposition.  A device-built plan (tile_plan_kernel) cuts each
// expert's rows into m-tiles of at most 16*MB rows.  A work item is one
// (m-tile, n-tile) pair; a persistent grid walks the items.  Items are dealt
// so that a round of the grid gives consecutive items -- the n-tiles of one
// m-tile, then the next m-tile of the same expert -- to workgroups of the same
// XCD (workgroup b runs on XCD b % 8), so the gathered A rows and the expert's
// weight rows are shared through that XCD's L2.
//
// Inside an item: 4 waves; wave w owns NCB 16-column blocks of the weight
// (for gate/up: NCB/2 gate blocks and the matching NCB/2 up blocks, so the
// SwiGLU epilogue is wave-local).  Weights stream from HBM straight into
// registers (each weight element is used by exactly one wave), one K-step
// ahead.  The A tile (<= 16*MB rows x 64 k) is staged in LDS, double
// buffered, XOR-swizzled by row so the 16 rows a fragment read touches hit
// distinct banks.  MFMA: v_mfma_f32_16x16x32_bf16, fp32 accumulation.
//
// Operand k-mapping: within a K-step of 64, lane (r = lane%16, g = lane/16)
// holds k in [16g, 16g+16) of its A row and of its weight row; sub-step s
// (0, 1) feeds the MFMA the 8 values [16g + 8s, 16g + 8s + 8).  Both operands
// use the same mapping, so each MFMA sums matching k.
#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kBK = 64;  // K per pipeline step

// LDS byte offset of 16-byte chunk c (0..7) of A-tile row `row`.
__device__ __forceinline__ int a_lds_off(int row, int c) {
  return row * (kBK * 2) + ((c ^ (row & 7)) << 4);
}

template <int MB, int NCB, bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather, int topk,
    const uint16_t* __restrict__ W, int64_t w_expert_stride, uint16_t* __restrict__ C,
    const int32_t* __restrict__ plan, int max_tiles, int K, int n_out, int up_row0) {
  constexpr int ROWS = 16 * MB;
  constexpr int HALF = SWIGLU ? NCB / 2 : NCB;    // output column blocks per wave
  constexpr int WCOLS = 4 * HALF * 16;            // output columns per item
  constexpr int LOADERS = ROWS * 8;               // threads that stage A (16 B each)
  constexpr int APASS = (LOADERS + 255) / 256;    // staging passes per thread
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][ROWS * kBK * 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int ntiles = plan[0];
  const int* plan_expert = plan + 4;
  const int* plan_row0 = plan_expert + max_tiles;
  const int* plan_rows = plan_row0 + max_tiles;
  const int nt_n = n_out / WCOLS;
  const int total = ntiles * nt_n;
  const int grid = gridDim.x, per_xcd = grid / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int nk = K / kBK;

  for (int round = 0;; round += grid) {
    const int q = round + xcd * per_xcd + slot;
    if (q >= total) break;
    const int tile = q / nt_n, ntile = q - tile * nt_n;
    const int e = plan_expert[tile], row0 = plan_row0[tile], nrows = plan_rows[tile];
    const int nrb = (nrows + 15) >> 4;

    // --- A staging addresses (row gather happens here) ---
    const uint16_t* a_src[APASS];
    int a_off[APASS];
    bool a_ok[APASS];
#pragma unroll
    for (int p = 0; p < APASS; ++p) {
      const int li = p * 256 + tid;
      const int row = li >> 3, c = li & 7;
      a_ok[p] = li < LOADERS && row < nrows;
      a_off[p] = a_lds_off(row < ROWS ? row : 0, c);
      int src_row = 0;
      if (a_ok[p]) src_row = gather ? gather[row0 + row] / topk : row0 + row;
      a_src[p] = A + (size_t)src_row * K + c * 8;
    }

    // --- weight row pointers of this wave ---
    const uint16_t* wp[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      int wrow;
      if (SWIGLU) {
        const int j = cb % HALF;
        wrow = ntile * WCOLS + wave * HALF * 16 + j * 16 + r + (cb >= HALF ? up_row0 : 0);
      } else {
        wrow = ntile * WCOLS + wave * NCB * 16 + cb * 16 + r;
      }
      wp[cb] = W + (size_t)e * w_expert_stride + (size_t)wrow * K + 16 * g;
    }

    f32x4_t acc[MB][NCB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[i][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // --- prologue: stage K-step 0 ---
    uint4 areg[APASS];
    uint4 bcur[NCB][2], bnxt[NCB][2];
#pragma unroll
    for (int p = 0; p < APASS; ++p) areg[p] = a_ok[p] ? ld16(a_src[p]) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      bcur[cb][0] = ld16(wp[cb]);
      bcur[cb][1] = ld16(wp[cb] + 8);
    }
    __syncthreads();  // previous item's last LDS reads are done
#pragma unroll
    for (int p = 0; p < APASS; ++p)
      if (p * 256 + tid < LOADERS) *reinterpret_cast<uint4*>(&lds_a[0][a_off[p]]) = areg[p];
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        const int k1 = (kt + 1) * kBK;
#pragma unroll
        for (int p = 0; p < APASS; ++p)
          areg[p] = a_ok[p] ? ld16(a_src[p] + k1) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          bnxt[cb][0] = ld16(wp[cb] + k1);
          bnxt[cb][1] = ld16(wp[cb] + k1 + 8);
        }
      }
      const uint8_t* la = lds_a[cur];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          if (i < nrb) {
            const uint4 av = *reinterpret_cast<const uint4*>(la + a_lds_off(i * 16 + r, 2 * g + s));
            const bf16x8_t a8 = as_bf16x8(av);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(bcur[cb][s]),
                                                                   acc[i][cb], 0, 0, 0);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int p = 0; p < APASS; ++p)
          if (p * 256 + tid < LOADERS)
            *reinterpret_cast<uint4*>(&lds_a[cur ^ 1][a_off[p]]) = areg[p];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          bcur[cb][0] = bnxt[cb][0];
          bcur[cb][1] = bnxt[cb][1];
        }
      }
      __syncthreads();
    }

    // --- epilogue: lane holds rows 4g..4g+3 of column r of each 16x16 block ---
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i < nrb) {
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
          const int col = ntile * WCOLS + wave * HALF * 16 + j * 16 + r;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = i * 16 + 4 * g + v;
            if (row < nrows) {
              float o;
              if (SWIGLU) {
                const float gt = acc[i][j][v], up = acc[i][j + HALF][v];
                o = gt / (1.0f + expf(-gt)) * up;
              } else {
                o = acc[i][j][v];
              }
              C[(size_t)(row0 + row) * n_out + col] = (uint16_t)f32_to_bf16(o);
            }
          }
        }
      }
    }
  }
}

// One thread per expert: cut each expert's rows into ceil(n / bmax) balanced
// m-tiles (rows rounded up to 16, at most bmax).  plan[0] = tile count,
// plan[4 ..] = expert, row0, rows arrays of max_tiles entries each.
__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t* __restrict__ offsets,
                                                        int E, int bmax, int32_t* __restrict__ plan,
                                                        int max_tiles) {
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
  for (int i = 0; i < nt; ++i) {
    const int idx = base + i;
    if (idx < max_tiles) {
      pe[idx] = e;
      pr0[idx] = offsets[e] + i * per;
      prn[idx] = min(per, n - i * per);
    }
  }
  if (e == 255) plan[0] = min(sc[255], max_tiles);
}

template <int MB, int NCB, bool SWIGLU>
static hipError_t launch_gemm_t(const uint16_t* A, const int32_t* gather, int topk,
                                const uint16_t* W, int64_t wstride, uint16_t* C,
                                const int32_t* plan, int max_tiles, int K, int n_out, int up_row0,
                                int grid, hipStream_t stream) {
  hipLaunchKernelGGL((grouped_gemm_kernel<MB, NCB, SWIGLU>), dim3(grid), dim3(256), 0, stream, A,
                     gather, topk, W, wstride, C, plan, max_tiles, K, n_out, up_row0);
  return hipGetLastError();
}

int ffn_rows_per_tile(int mb) { return 16 * mb; }

// Picks the m-tile height from the mean rows per expert.
int ffn_choose_mb(int64_t rows, int E) {
  const int64_t mean = rows / (E > 0 ? E : 1);
  if (mean <= 8) return 1;
  if (mean <= 24) return 2;
  if (mean <= 48) return 4;
  return 8;
}

hipError_t launch_tile_plan(const int32_t* offsets, int E, int bmax, int32_t* plan, int max_tiles,
                            hipStream_t stream) {
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, stream, offsets, E, bmax, plan,
                     max_tiles);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int mb, bool swiglu, const uint16_t* A, const int32_t* gather,
                               int topk, const uint16_t* W, int64_t wstride, uint16_t* C,
                               const int32_t* plan, int max_tiles, int K, int n_out, int up_row0,
                               int grid, hipStream_t stream) {
  constexpr int NCB = 4;
#define BEAM_GEMM_CASE(MBV)                                                                     \
  case MBV:                                                                                     \
    return swiglu ? launch_gemm_t<MBV, NCB, true>(A, gather, topk, W, wstride, C, plan,         \
                                                  max_tiles, K, n_out, up_row0, grid, stream)   \
                  : launch_gemm_t<MBV, NCB, false>(A, gather, topk, W, wstride, C, plan,        \
                                                   max_tiles, K, n_out, up_row0, grid, stream);
  switch (mb) {
    BEAM_GEMM_CASE(1)
    BEAM_GEMM_CASE(2)
    BEAM_GEMM_CASE(4)
    BEAM_GEMM_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef BEAM_GEMM_CASE
}

int ffn_out_cols_per_item(bool swiglu) { return swiglu ? 4 * 2 * 16 : 4 * 4 * 16; }

}  // namespace beam
