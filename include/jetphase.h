/*
 * jetphase.h -- phase timing of the block-scaled GEMM kernel (k_gemm_fp8), a
 * diagnostic build of the library: libjetfp8_phase.so exports everything
 * jetfp8.h declares plus the call below; libjetfp8.so does not contain it.
 *
 * While the device flag is non-zero, thread 0 of every workgroup b <
 * capacity of each k_gemm_fp8 launch writes record b, eight uint64:
 *   [0] wall counter at the workgroup's entry,
 *   [1] wall counter before its first DMA (after the tile/segment set-up),
 *   [2] wall counter after its K loop,
 *   [3] wall counter at its exit (the epilogue's stores issued),
 *   [4] HW_REG_HW_ID in the low and HW_REG_XCC_ID in the high 32 bits
 *       (which CU of which XCD ran it), [5] the launch's grid size in the
 *       low and its workgroup size (threads) in the high 32 bits,
 *   [6], [7] shader-clock counter before the first DMA and after the K loop.
 * The wall counter runs at a constant rate (hipDeviceAttributeWallClockRate
 * kHz); [6] and [7] count shader clocks, so ([7]-[6]) / ([2]-[1]) is the
 * clock the K loop ran at.  A later launch overwrites the records of the
 * workgroup numbers it shares with an earlier one (a GEMM call that runs
 * as two launches leaves records of both, told apart by [5]).
 */
#ifndef JETPHASE_H
#define JETPHASE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Device addresses of the current device's records (capacity * 8 uint64)
 * and of its int flag, both owned by the library (read and write them with
 * hipMemcpy); 0 on success, 1 for a null argument, 2 if the symbols are not
 * found on the current device. */
int jet_phase_buffers(void** records, void** flag, int* capacity);

#ifdef __cplusplus
}
#endif

#endif
