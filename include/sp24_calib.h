/*
 * sp24_calib.h -- measurement aid exported by libsp24 (not a step of the
 * 2:4 method): a plain HBM stream used to measure, on the machine at hand,
 * the rate a bandwidth-bound kernel of the library could at best reach for
 * the same bytes and the same launch shape.  The benchmark reports each
 * bandwidth-bound kernel against both this measured floor and the published
 * HBM peak.
 */
#ifndef SP24_CALIB_H
#define SP24_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * sp24_calib_stream -- reads read_bytes from src in 16-byte pieces and
 * copies the first write_bytes of them to dst (write_bytes <= read_bytes)
 * with workgroups of `threads` threads (a multiple of 64, at most 1024):
 *   workgroups > 0: that many workgroups walk the pieces in a grid-stride
 *                   loop, four 16-byte loads in flight per thread;
 *   workgroups == 0: one pass, ceil(read_bytes / (128 * threads))
 *                   workgroups, each thread with eight 16-byte loads in
 *                   flight at a stride of the block size, then its stores
 *                   (the shape of the library's compress kernels).
 * The xor of everything read by workgroup w is xor-ed into sink[w], so no
 * load can be left out by the compiler.
 *
 *   src, dst  DEVICE pointers, 16-byte aligned; read_bytes and write_bytes
 *             multiples of 16.  dst may be NULL when write_bytes == 0.
 *   sink      DEVICE pointer to one uint32 per workgroup launched.
 * Errors: SP24_ERR_INVALID_VALUE (sizes, null pointers, workgroups < 0,
 * threads not a multiple of 64 in 64..1024), SP24_ERR_MISALIGNED,
 * SP24_ERR_LAUNCH.  Enqueues on `stream` only.
 */
int sp24_calib_stream(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes, uint32_t* sink,
                      int workgroups, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SP24_CALIB_H */
