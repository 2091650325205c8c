/* Rate probes of one MI355X, used only to measure the hot path against
 * peaks taken on the same GPU (libdsa_peak.so, separate from libdsa.so).
 *
 * None of these is a step of the method: they put a number next to the
 * published peaks (dense MFMA 2.5 PFLOP/s bf16, 5.0 PFLOP/s fp8; HBM
 * 8 TB/s) so that the kernels' fractions can be stated against both, and a
 * random row gather next to the sparse attention's.
 * All calls are asynchronous on the given HIP stream (NULL: the default
 * stream), take device pointers the caller owns, allocate nothing and return
 * 0 on success, 1 for an invalid argument, 2 for a launch error.
 */
#ifndef DSA_PEAK_H
#define DSA_PEAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Back-to-back dense MFMAs from registers: `blocks` workgroups of 256
 * threads, each wave `iters` rounds of four independent accumulations with
 * v_mfma_f32_32x32x16_bf16 (dtype 0, 32768 flop each) or
 * v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands (dtype 1, 131072 flop
 * each). out: blocks * 256 floats (the accumulators' sums, so the work is not
 * removed). *flop receives the flop count of the launch. */
int dsa_peak_mfma(int dtype, int blocks, int iters, float* out, double* flop, void* stream);

/* HBM copy: dst[i] = src[i] for `bytes` bytes (a multiple of 16, both
 * 16-byte aligned) with 16-byte nontemporal loads and stores, eight in
 * flight per thread, grid-stride over `blocks` workgroups of 256 threads.
 * Moves 2 * bytes. */
int dsa_peak_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

/* HBM read: every 16-byte word of src (bytes a multiple of 16) is read
 * (nontemporal, sixteen in flight per thread) and folded (xor) into
 * out[block] (blocks words), so the loads are kept. */
int dsa_peak_read(const void* src, size_t bytes, int blocks, uint32_t* out, void* stream);

/* Row gather: for i < n, the 256-byte row table[idx[i]] of a table of `rows`
 * rows (16-byte aligned) is read and folded (xor) into out[block] (blocks
 * words), sixteen lanes per row and sixteen rows in flight per lane group,
 * grid-stride over `blocks` workgroups of 256 threads. An index outside
 * [0, rows) reads the last row. Moves 256 * n bytes of rows plus 4 * n of
 * indices: the rate an index-driven gather of bf16 rows of 128 values (the
 * sparse attention's K and V rows) reaches from wherever the table sits. */
int dsa_peak_gather(const void* table, size_t rows, const int32_t* idx, size_t n, int blocks, uint32_t* out,
                    void* stream);

#ifdef __cplusplus
}
#endif
#endif
