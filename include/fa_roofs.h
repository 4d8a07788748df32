/*
 * fa_roofs.h -- microbenchmarks of libfa.so that measure, on the GPU at hand,
 * the roofs the attention kernels are judged against: the dense bf16 MFMA
 * rate, the v_exp_f32 (transcendental) rate, the fp32 VALU FMA rate, how much
 * VALU work overlaps MFMA work on one SIMD, and device-memory bandwidth.
 *
 * Why: "Flash Attention Memory Optimization Explained" (lzwjava.github.io),
 * "Key Mechanisms", attributes the method's speed to cutting traffic to
 * high-bandwidth memory so the arithmetic units are kept busy; whether a
 * kernel is bound by the matrix units, by the exponentials of the softmax or
 * by memory is decided against these measured rates (and the published peaks).
 *
 * Every entry point only enqueues kernels on `stream` (a hipStream_t or NULL)
 * and returns; the caller times them (e.g. with events on the same stream).
 * Work per launch is fixed by the arguments, so rate = work / time:
 *   fa_roof_mfma:  grid_blocks * 4 waves * n_iter * 4 MFMA 32x32x16 bf16
 *                  (32768 FLOP each)
 *   fa_roof_valu:  grid_blocks * 4 waves * n_iter * 16 wave64 instructions
 *                  (v_exp_f32 when op = FA_ROOF_EXP, v_fma_f32 when
 *                  op = FA_ROOF_FMA)
 *   fa_roof_overlap: grid_blocks work-groups of 8 waves; waves 0-3 (one per
 *                  SIMD) run n_mfma * 4 MFMAs when mask bit 0 is set, waves
 *                  4-7 (sharing those SIMDs) run n_valu * 16 instructions of
 *                  kind `op` when mask bit 1 is set. Comparing the time with
 *                  both bits against each alone shows the overlap.
 *   fa_roof_copy:  reads and writes `bytes` bytes (16-byte vectors), each of
 *                  8192 work-groups streaming its own contiguous chunk.
 *   fa_roof_read:  reads `bytes` bytes (16-byte vectors, eight in flight per
 *                  thread, 8192 work-groups each streaming its own contiguous
 *                  chunk); sink needs 8192 elements (one per work-group).
 * sink: device float array of at least grid_blocks elements (written, holds
 * nothing useful; it keeps the arithmetic from being optimised away).
 * Returns 0 on success, 9 (FA_ERR_LAUNCH) if the runtime rejects a launch,
 * 2 for a non-positive size or count, 1 for a NULL pointer, 7 for a pointer
 * or size not a multiple of 16 bytes (copy, read).
 */
#ifndef FA_ROOFS_H_
#define FA_ROOFS_H_

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_ROOF_FMA = 0, FA_ROOF_EXP = 1 } fa_roof_op_t;

int fa_roof_mfma(int grid_blocks, int n_iter, float *sink, void *stream);
int fa_roof_valu(int grid_blocks, int n_iter, int op, float *sink, void *stream);
int fa_roof_overlap(int grid_blocks, int n_mfma, int n_valu, int op, int mask, float *sink,
                    void *stream);
int fa_roof_copy(const void *src, void *dst, long long bytes, void *stream);
int fa_roof_read(const void *src, long long bytes, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_ROOFS_H_ */
