/*
 * sp24_calib.h -- measurement aids exported by libsp24 (not steps of the
 * 2:4 method):
 *   - a plain HBM stream, to measure on the machine at hand the rate a
 *     bandwidth-bound kernel of the library could at best reach for the
 *     same bytes and the same launch shape;
 *   - the product's sparse matrix-core instruction stream with its operands
 *     held in registers, to measure the rate the matrix cores sustain on the
 *     workload's own operand values (their power draw depends on the data,
 *     and the clock on the power); optionally with the product's
 *     direct-to-LDS loads issued between the instructions, or with the
 *     32x32 instruction shape in place of 16x16.
 * The benchmark reports each kernel against both the measured figure and
 * the published peak.
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

/*
 * sp24_calib_mfma -- the instruction stream of sp24_gemm's large-tile main
 * loop with no memory traffic.  Each of `workgroups` workgroups runs 8 waves
 * (two per SIMD).  Wave v = 8 * workgroup + wave index loads, once, the
 * operands of one k-step of a 128 x 64 wave tile:
 *   8 A fragments:  bytes [8192 * (v % na), +8192) of a_vals, 16 per lane
 *                   per fragment (na = a_bytes / 8192);
 *   8 code words:   bytes [2048 * (v % nc), +2048) of codes, one 32-bit
 *                   word per lane per fragment (nc = code_bytes / 2048);
 *   4 B fragments:  bytes [8192 * (v % nb), +8192) of b, 32 per lane per
 *                   fragment (nb = b_bytes / 8192);
 * and then issues `rounds` times the 32 sparse instructions of one k-step of
 * the (a_type, b_type) pair (16x16x64 for 16-bit types, 16x16x128 for 8-bit)
 * into 32 accumulator tiles.  Dense-equivalent work per launch:
 *   workgroups * 8 * rounds * 32 * 2 * 16 * 16 * (64 or 128) flop.
 * Pass the product's own compressed A, its codes and B so the instructions
 * multiply the workload's values; any bytes are accepted (code words are
 * used as they are).  The xor of each wave's accumulator bits is xor-ed into
 * sink[workgroup].
 *
 *   a_vals, codes, b   DEVICE pointers, 16-byte aligned, with at least 8192,
 *                      2048 and 8192 bytes.
 *   sink               DEVICE pointer to `workgroups` uint32 values.
 * Errors: SP24_ERR_UNSUPPORTED (type pair), SP24_ERR_INVALID_VALUE (null
 * pointer, too few bytes, rounds or workgroups < 1), SP24_ERR_MISALIGNED,
 * SP24_ERR_LAUNCH.  Enqueues on `stream` only.
 */
int sp24_calib_mfma(const void* a_vals, uint64_t a_bytes, const uint32_t* codes, uint64_t code_bytes, const void* b,
                    uint64_t b_bytes, int a_type, int b_type, int rounds, int workgroups, uint32_t* sink, void* stream);

/*
 * sp24_calib_mfma_ex -- sp24_calib_mfma with two variations of the
 * instruction stream (sp24_calib_mfma is this call with shape 16 and no
 * load source):
 *   shape 16   the product's 16x16 instructions (32 per round);
 *   shape 32   the 32x32 sparse instructions of the same pair (32x32x32 for
 *              16-bit types, 32x32x64 for 8-bit), 16 per round over the
 *              same operand registers read as 32x32 fragments; the same
 *              work per round, so the dense-equivalent work per launch is
 *              the formula above for either shape;
 *   load_src   NULL, or a DEVICE buffer (16-byte aligned, at least 1024
 *              bytes): then every wave also issues, per round, the
 *              product's number of 1 KiB direct-to-LDS loads per wave and
 *              k-step (7 for 16-bit types, 8 for 8-bit), one after each
 *              of the first 7 or 8 of the round's 8 instruction groups, in
 *              the product's form (an LDS base and a per-lane offset set
 *              for each load), reading consecutive 1 KiB blocks of the
 *              largest power-of-two prefix of load_src (at most 1 GiB) into
 *              a 16 KiB LDS ring per wave; each round waits for the loads of
 *              the round before.  The loads change no result: the sinks
 *              equal those of the same call without them.
 * Errors: as sp24_calib_mfma, and SP24_ERR_INVALID_VALUE for a shape other
 * than 16 or 32 or a load source under 1024 bytes.  Enqueues on `stream`
 * only.
 */
int sp24_calib_mfma_ex(const void* a_vals, uint64_t a_bytes, const uint32_t* codes, uint64_t code_bytes,
                       const void* b, uint64_t b_bytes, int a_type, int b_type, int rounds, int workgroups, int shape,
                       const void* load_src, uint64_t load_src_bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SP24_CALIB_H */
