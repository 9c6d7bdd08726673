/*
 * skinny_floors.h -- measurement helpers for the small-M GEMM benchmark.
 * Not part of the GEMM: these kernels give the floors a GEMM time is read
 * against, and the reference copy for scaling hardware byte counters.
 *
 * All pointers are DEVICE pointers; work is enqueued on `stream` and the
 * calls return at once.  Return 0 on success, else the hipError_t of the
 * launch.
 */
#ifndef SKINNY_FLOORS_H
#define SKINNY_FLOORS_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* An empty kernel of `grid` workgroups of `threads` threads: the launch and
 * dispatch floor for a kernel of that shape. */
int skinny_floor_empty(int grid, int threads, hipStream_t stream);

/* Reads `rows` rows of `row_bytes` bytes (row_bytes % 16 == 0, rows
 * contiguous from `buf`, 16-byte aligned), one workgroup of `threads`
 * threads per row, every 16-byte load issued before any is consumed
 * (row_bytes <= 16 * 8 * threads).  Writes nothing unless the data hash to a
 * fixed constant (then one word per workgroup to sink[rows]).  The floor for
 * streaming the same bytes the GEMM's weight stream reads. */
int skinny_floor_read(const void *buf, int rows, int row_bytes, int threads, unsigned *sink,
                      hipStream_t stream);

/* Reads `bytes` bytes (a multiple of 16, 16-byte aligned) from `buf` as one
 * flat array: ceil(bytes / 32768) workgroups of 256 threads, each reading
 * its 32 KB with every 16-byte load in flight at once.  Writes nothing
 * unless the data hash to a fixed constant (then one word per workgroup to
 * sink[ceil(bytes / 32768)]).  The read-stream floor for buffers whose rows
 * are too short for one workgroup each. */
int skinny_floor_read_flat(const void *buf, size_t bytes, unsigned *sink, hipStream_t stream);

/* The operand intake of the bf16 dot-product plan (cols columns per
 * workgroup, `threads` threads, `vecs` 16-byte vectors per thread per row;
 * the plan's cols, threads and depth) with no arithmetic: ceil(N / cols)
 * workgroups each load their cols rows of W[N, K] and all M rows of x[M, K]
 * with the dot kernel's load pattern, all in flight at once, and fold them
 * with xor.  Writes nothing unless the data hash to a fixed constant (then
 * one word per workgroup to sink[ceil(N / cols)]).  1 <= M <= 16, K % 8 == 0,
 * vecs * threads >= K / 8, x and W 16-byte aligned; an unbuilt (M, cols,
 * vecs) or too many threads for it returns hipErrorInvalidValue. */
int skinny_floor_intake(const void *x, const void *W, int M, int N, int K, int cols, int threads,
                        int vecs, unsigned *sink, hipStream_t stream);

/* Copies `bytes` (a multiple of 16, 16-byte aligned) from src to dst with
 * 16-byte loads and stores: the reference for hardware read/write byte
 * counters (it must read and write exactly `bytes`). */
int skinny_floor_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_FLOORS_H */
