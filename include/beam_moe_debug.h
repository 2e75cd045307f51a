/*
 * beam_moe_debug.h -- bounds checking in the debug build of the MoE-block
 * library (libbeam_moe_checked.so, compiled with BEAM_MOE_CHECKED=1; the
 * build step `python -m grouped_top_routing_amd.build` writes it beside
 * libbeam_moe.so).
 *
 * In the checked build every kernel verifies the indices it derives from its
 * inputs before using them: the permutation's destination rows, the m-tile
 * plan (tile count within its capacity, each tile's rows within the permuted
 * rows, a valid expert), the gathered pair indices and the activation rows
 * they name, the weight row blocks and k stages of each expert's stream, and
 * the rows the combine reads.  A failing check records its bit below and the
 * index is clamped into range, so the kernel stays inside its buffers (its
 * results are then meaningless, and the check says why).  Correct inputs
 * produce the same results as the normal build, bit for bit.
 */
#ifndef BEAM_MOE_DEBUG_H
#define BEAM_MOE_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_check_bit {
  MOE_CHECK_PERMUTE_ROW = 1u << 0,    /* permutation row outside [0, T*topk)            */
  MOE_CHECK_PLAN_CAPACITY = 1u << 1,  /* more m-tiles than the plan can hold            */
  MOE_CHECK_PLAN_ROWS = 1u << 2,      /* an m-tile's rows or expert out of range        */
  MOE_CHECK_GATHER_INDEX = 1u << 3,   /* a gathered pair index outside [0, T*topk)      */
  MOE_CHECK_TOKEN_INDEX = 1u << 4,    /* an activation row outside the activations      */
  MOE_CHECK_WEIGHT_OFFSET = 1u << 5,  /* a weight block or k stage outside the expert   */
  MOE_CHECK_COMBINE_ROW = 1u << 6     /* a combine row (perm_dst) outside [0, T*topk)   */
};

/*
 * Waits for the current device, then writes to *flags the OR of the check
 * bits recorded since the previous call (or the library load) and clears
 * them.  Returns MOE_OK in the checked build; MOE_ERR_UNSUPPORTED (with
 * *flags = 0) in the normal build, which has no checks; MOE_ERR_INVALID_ARG
 * for a NULL pointer; MOE_ERR_HIP if the device cannot be reached.
 */
int moe_debug_check_flags(uint32_t* flags);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_DEBUG_H */
