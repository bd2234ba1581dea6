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

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_CALIB_H */
