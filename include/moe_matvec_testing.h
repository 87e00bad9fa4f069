/*
 * moe_matvec_testing.h -- kernel-variant switches of libmoe_matvec, for
 * tests and measurements only.
 *
 * Several entry points of moe_matvec.h choose among kernels that compute the
 * same result (the same bits, except where a comment below says otherwise):
 * rows per wave, waves per workgroup, x from the caches or staged on chip,
 * the MoE top-k in a kernel of its own or inside the expert kernel, the
 * down projection in one kernel or by expert.  The choice is automatic
 * (value 0).  A test sets a switch to force one variant and compares it with
 * the automatic one; a measurement sets it to time a variant.  The switches
 * are process-wide (atomic, read at every launch); a caller that computes
 * results never sets them.  A forced variant that does not apply to a call
 * (a shape it does not cover, an on-chip memory limit) falls back to the
 * automatic choice.
 */
#ifndef MOE_MATVEC_TESTING_H
#define MOE_MATVEC_TESTING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mmv_path_switch {
  /* gemv_bf16, B = 1 with the per-wave kernel: rows per wave (1, 2 or 4) */
  MMV_PATH_BF16_ROWS = 0,
  /* gemv_bf16: waves per workgroup of the B = 1 per-wave kernel (1 or 4);
   * for B >= 2 with K % 512 != 0, waves per 16-row tile (4, 8 or 16: the
   * k-steps are grouped differently, so rows agree within rounding) */
  MMV_PATH_BF16_WAVES = 1,
  /* gemv_bf16, B = 1, K % 512 == 0: waves per workgroup of the kernel that
   * stages x on chip (2, 4, 5, 8, 10 or 16); -1 = the per-wave kernel */
  MMV_PATH_BF16_XL = 2,
  /* gemv_bf16, B >= 2, K % 512 == 0: matrix-core shape
   * 10000 * rows + 1000 * waves + 100 * chunks in flight + tile rows,
   * + 1000000 for the chunk loop: 1168216, 1328216, 1168316, 1088208 (same
   * bits) or 1164216 (4 waves: within rounding) */
  MMV_PATH_BF16_ML = 3,
  /* gemv_q4_0 whole-row kernel: rows per lane group (2, 4, 6 or 8) */
  MMV_PATH_Q4_RP = 4,
  /* gemv_q4_0: 1 = the grid-stride kernel for every K */
  MMV_PATH_Q4_GENERIC = 5,
  /* gemv_q4_0 grid-stride kernel: workgroups per compute unit */
  MMV_PATH_Q4_WG_PER_CU = 6,
  /* moe_layer_decode, B <= 8: 1 = top-k and row lists in a kernel of their
   * own; -1 = top-k inside every gate/up workgroup */
  MMV_PATH_MOE_TOPK = 7,
  /* moe_mul_mat_id / moe_layer_decode, B <= 8: 1 = the one-kernel down
   * projection; 2 = the down projection by expert plus a combine kernel */
  MMV_PATH_MOE_DOWN = 8,
  /* gemv_q4_0_f32 on the matrix cores: 0 = from B = 2, n > 0 = from B = n,
   * -1 = never (the fp32 kernels; rows agree within rounding) */
  MMV_PATH_Q4F32_MF = 9,
  /* gemv_q4_0 on the matrix cores (K <= 4096): 0 = from B = 3 for fp32 x,
   * from B = 5 for a Q8_1 buffer; n > 0 = from B = n; -1 = never (the dot4
   * kernels; rows agree within rounding) */
  MMV_PATH_Q4_MF = 10,
  MMV_PATH_COUNT = 11
};

/* Sets switch `which` to `value` (0 = automatic); returns the previous value,
 * or MMV_E_ARG (-9) for an unknown switch. */
int mmv_set_path(int which, int value);
/* Current value of switch `which` (0 for an unknown switch). */
int mmv_get_path(int which);

/* Timeline of the MoE kernels, for measurement.  Only a library built with
 * the timeline option (python -m moe_matvec_amd.build --timeline ->
 * libmoe_matvec_timeline.so) notes, per workgroup of the MoE kernels, the
 * chip's 100 MHz constant clock at fixed points of its work; the normal
 * library does nothing here and returns 0.  Copies the array of the last
 * launches ([7 kernel kinds: router, LDS router, top-k + row lists, gate/up,
 * down, down by expert, combine][4096 workgroups][8 points] uint64, 0 where
 * nothing was noted) to the device buffer dst when dst is not NULL, then
 * zeroes it when `clear` is nonzero; both ordered on `stream`.  Returns the
 * array's size in bytes. */
size_t mmv_timeline(void *dst, int clear, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MATVEC_TESTING_H */
