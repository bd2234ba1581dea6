/*
 * libselscan_calib: copy kernels of known size, used only to calibrate the HBM
 * byte counters (rocprofv3 FETCH_SIZE / WRITE_SIZE) for the memory access
 * patterns of libselscan's kernels. Not part of the scan; nothing in
 * libselscan calls it.
 *
 * selscan_calib_copy copies `bytes` bytes from src to dst (device pointers,
 * caller-owned, 16-byte aligned, not overlapping) on `stream`:
 *   mode 0: ordinary 16-byte loads and stores, consecutive lanes on
 *           consecutive 16-byte vectors (a plain streaming copy);
 *   mode 1: the same with non-temporal loads and stores;
 *   mode 2: non-temporal, in the forward kernel's row pattern: the buffer is
 *           rows of 4096 bytes, four adjacent lanes take one row's 64-byte
 *           piece, a wave covers 16 rows, and each thread walks its row's
 *           64 pieces in order. bytes must be a multiple of 64 rows (256 KiB).
 * Returns 0, -1 (NULL pointer), -2 (bytes not a positive multiple of 16, or of
 * 256 KiB for mode 2), -7 (misaligned), -9 (mode) or -5 (launch failed).
 */
#ifndef SELSCAN_CALIB_H
#define SELSCAN_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int selscan_calib_copy(const void* src, void* dst, int64_t bytes, int32_t mode, void* stream);

/*
 * selscan_calib_scan_mix runs the forward kernel's inner loop alone (per lane
 * 4 states; per token and state: l*A, v_exp_f32, w*B with B a scalar
 * operand, the state FMA and the readout FMA; B/C by s_load_dwordx16 from a
 * hot 32 KiB buffer, (l, w) from LDS) for nsub 4-token sub-blocks in
 * `blocks` workgroups of 256 threads, with no HBM traffic and no barriers. Its
 * rate is the measured ceiling of that instruction mix: (lane, token, state)
 * updates = blocks * 256 * nsub * 4 * 4, at 6 VALU slots each.
 *   rec : >= 8192 floats of device memory (contents irrelevant, read only)
 *   out : blocks * 256 floats of device memory (written)
 * Returns 0, -1 (NULL), -2 (blocks < 1, or nsub not even and >= 2), -5.
 */
int selscan_calib_scan_mix(const float* rec, float* out, int32_t blocks, int32_t nsub, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_CALIB_H */
