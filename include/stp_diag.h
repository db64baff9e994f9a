/*
 * stp_diag.h -- measurement kernels beside the sparse-attention library
 * (libstp_diag.so, not part of libstp.so): the practical ceilings the decode's
 * rates are set against.  Status codes, errors and stream conventions as in
 * stp.h; stp_last_error() of libstp.so (which this library links) returns
 * the message of a failed call.
 */
#ifndef STP_DIAG_H_
#define STP_DIAG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Diagnostic: the bandwidth ceiling of the decode's row gather ("5.1.1 · 从
 * 索引到 Kernel" §2, eq. (8)-(9): decode time is set by the candidate rows'
 * bytes).  Reads every byte of the rows row_ids[t, lo:lo+len] of each query
 * token t, for `parts` contiguous ranges per token (lo, len as the decode's
 * splits: ranges of ceil(counts[t] / parts) entries), each range read by
 * `replicas` workgroups (as the decode reads a range once per group of 64
 * query heads), with the decode's placement of workgroups on XCDs.  Computes
 * nothing but an xor of the words read, one uint32 per workgroup in
 * checksum[stp_row_gather_blocks(T, parts, replicas)].
 *   rows       [num_rows, row_bytes] bytes (row_bytes a multiple of 16)
 *   row_ids    [T, cap] int32; -1 and ids outside [0, num_rows) read nothing
 *   counts     [T] or NULL (then cap)
 * Errors: sizes < 0 or parts / replicas < 1, ceil(cap / parts) > 4096,
 * row_bytes not a positive multiple of 16 -> STP_ERR_INVALID_ARG.
 */
int stp_row_gather(const void* rows, int64_t num_rows, int64_t row_bytes, const int32_t* row_ids,
                   const int32_t* counts, int32_t cap, int32_t T, int32_t parts, int32_t replicas,
                   uint32_t* checksum, hipStream_t stream);

/* Workgroups (= checksum words) of stp_row_gather; 0 for invalid sizes. */
int32_t stp_row_gather_blocks(int32_t T, int32_t parts, int32_t replicas);

/*
 * Diagnostic: what HBM delivers to a plain sequential read on this device
 * ("5.1.1 · 从索引到 Kernel" §6.1: rates against what the hardware sustains).
 * Reads bytes (a multiple of 16) from src with `blocks` workgroups of 256
 * threads, grid-stride over 16-byte units (unit u is read by thread u mod
 * (256 blocks) of the grid), and writes the xor of the 32-bit words each
 * workgroup read to checksum[blocks].  Errors: bytes not a multiple of 16,
 * blocks < 1, null pointers -> STP_ERR_INVALID_ARG.
 */
int stp_stream_read(const void* src, int64_t bytes, int32_t blocks, uint32_t* checksum,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STP_DIAG_H_ */
