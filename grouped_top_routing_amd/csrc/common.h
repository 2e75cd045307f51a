// Shared device helpers for the gfx950 kernels of the MoE block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// Fourth word of a raw (stride 0, untyped) buffer descriptor on gfx9-family
// GPUs: DATA_FORMAT = 32 bits (a zero format would make every access out of
// range).  Accesses at offsets at or past the descriptor's byte count are
// dropped by the hardware: stores do nothing, loads return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t v) {
  return __uint_as_float(v << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values rounded to bf16 (round-to-nearest-even, as f32_to_bf16
// for every non-NaN input) and packed, lo in the low half: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte global load / store.
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}
// 16-byte global load with the non-temporal cache policy (data read once).
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float sigmoidf_(float v) {
  return 1.0f / (1.0f + expf(-v));
}

// SwiGLU product SiLU(g) * u = g * sigmoid(g) * u in FP32, with the library
// expf and an IEEE divide (no approximate intrinsics)
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// ---------------------------------------------------------------------------
// Checked builds (BEAM_MOE_CHECKED=1, the debug library).  Kernels verify the
// indices they derive from their inputs before using them; a failing check
// sets its bit in the translation unit's flag word and clamps the index into
// range, so no access leaves its buffer and no load is skipped (the expert
// GEMMs' wait counts stay exact).  The host reads and clears the words with
// moe_debug_check_flags.  In the normal build the checks compile to nothing.
enum CheckBit : uint32_t {
  kCheckPermuteRow = 1u << 0,     // permutation row outside [0, pairs)
  kCheckPlanCapacity = 1u << 1,   // more m-tiles than the plan holds
  kCheckPlanRows = 1u << 2,       // m-tile rows outside [0, pairs) or bad expert
  kCheckGatherIndex = 1u << 3,    // gathered pair index outside [0, pairs)
  kCheckTokenIndex = 1u << 4,     // A row (token) outside the activations
  kCheckWeightOffset = 1u << 5,   // weight stage or row block outside the expert
  kCheckCombineRow = 1u << 6,     // combine row outside [0, pairs)
};
#ifndef BEAM_MOE_CHECKED
#define BEAM_MOE_CHECKED 0
#endif
#if BEAM_MOE_CHECKED
static __device__ uint32_t g_check_flags;  // one word per translation unit
// v if lo <= v <= hi; else records `bit` and returns v clamped into [lo, hi]
template <class T>
__device__ __forceinline__ T check_clamp(T v, int64_t lo, int64_t hi, uint32_t bit) {
  if ((int64_t)v < lo || (int64_t)v > hi) {
    atomicOr(&g_check_flags, bit);
    return (T)((int64_t)v < lo ? lo : hi);
  }
  return v;
}
__device__ __forceinline__ void check_that(bool ok, uint32_t bit) {
  if (!ok) atomicOr(&g_check_flags, bit);
}
#define BEAM_CLAMP(v, lo, hi, bit) (::beam::check_clamp((v), (lo), (hi), (bit)))
#define BEAM_CHECK(ok, bit) ::beam::check_that((ok), (bit))
// Host side: this translation unit's flag word, read and cleared (0 when the
// device call fails).
#define BEAM_DEFINE_CHECK_READER(fn)                                          \
  uint32_t fn() {                                                              \
    uint32_t v = 0, zero = 0;                                                  \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_flags), sizeof v) != hipSuccess) return 0; \
    (void)hipMemcpyToSymbol(HIP_SYMBOL(g_check_flags), &zero, sizeof zero);    \
    return v;                                                                  \
  }
#else
#define BEAM_CLAMP(v, lo, hi, bit) (v)
#define BEAM_CHECK(ok, bit) ((void)0)
#define BEAM_DEFINE_CHECK_READER(fn) \
  uint32_t fn() { return 0; }
#endif

// ---------------------------------------------------------------------------
// Direct global -> LDS streaming (used by the expert GEMMs and the router).
// s_waitcnt immediate (GFX9 encoding) that waits until at most n vector
// memory operations of this wave are outstanding; other counters untouched.
__host__ __device__ constexpr int vm_wait_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(N));
}

// Wait for all of this wave's LDS reads (lgkmcnt(0)); other counters untouched.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Compiler-level fence: no memory access moves across it (emits nothing).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding direct load).
__device__ __forceinline__ void stage_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// wait_vm with a run-time count (a branch tree down to the immediate forms);
// counts of 63 and more wait for at most 63.
template <int LO = 0, int HI = 63>
__device__ __forceinline__ void wait_vm_dyn(int n) {
  n = __builtin_amdgcn_readfirstlane(n);  // keep the tree on scalar branches
  if constexpr (LO == HI) {
    wait_vm<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vm_dyn<LO, MID>(n);
    else wait_vm_dyn<MID + 1, HI>(n);
  }
}

template <int AHEAD, int L>
__device__ __forceinline__ void wait_stage(int ahead) {
  // wait until only `ahead` later stages (L loads each) remain in flight
  if constexpr (AHEAD == 0) {
    wait_vm<0>();
  } else {
    if (ahead >= AHEAD) wait_vm<AHEAD * L>();
    else wait_stage<AHEAD - 1, L>(ahead);
  }
}

// Workgroups a persistent walk over `total` items uses out of a grid of
// `grid` (a multiple of 8, one per XCD): the fewest, again a multiple of 8,
// that still finish in the same number of rounds, so that the last round is
// as full as it can be (e.g. 2940 items on 512 workgroups: 496 do 6 rounds
// instead of 512 doing 5 or 6).  The others exit at once.
__device__ __forceinline__ int balanced_grid(int total, int grid) {
  if (total <= 0) return grid;
  const int rounds = (total + grid - 1) / grid;
  const int per = (total + rounds - 1) / rounds;
  const int eff = (per + 7) / 8 * 8;
  return eff < grid ? eff : grid;
}

// Two E4M3FN codes (bytes 0-1 of w, or bytes 2-3 for HI) widened to two bf16
// values in one 32-bit word, the lower code in the low half.  Exact: every
// E4M3FN value is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// One direct global -> LDS load: lane l's 16 bytes at `g` land at LDS byte
// address lds_addr + 16*l (lds_addr must be wave-uniform; it goes in M0).
// Issued from inline asm so the compiler's own wait-count pass does not see
// it: the pass would otherwise put a vmcnt(0) -- a full drain of the ring --
// before every later LDS read.  Completion is tracked by hand with
// wait_vm<>() (vector memory operations of a wave complete in order).  M0 is
// saved and restored, and s_nop covers the M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);  // free when already uniform
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_addr)
      : "memory");
}

// As lds_dma16, with the non-temporal cache policy: for data read once (the
// expert weight streams), so it does not displace reused lines in the caches.
__device__ __forceinline__ void lds_dma16_nt(const void* g, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_addr)
      : "memory");
}

// As lds_dma16 / lds_dma16_nt, addressing base + off with a wave-uniform
// 64-bit base in SGPRs and a 32-bit per-lane byte offset (one VGPR).
template <bool NT>
__device__ __forceinline__ void lds_dma16_sv(const void* base, uint32_t off, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(lds_addr), "s"(base)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(lds_addr), "s"(base)
        : "memory");
  }
}

}  // namespace beam
