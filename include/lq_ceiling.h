/*
 * lq_ceiling.h — C ABI of liblq_ceiling: memory-system ceilings for liblq's
 * fake-quant kernels on MI355X (gfx950). Measurement tools, not part of the
 * method: they move the same bytes as a fake-quant call in the same layout,
 * with no quantization arithmetic, so that a call's time can be set against
 * what the memory system delivers for that exact traffic (the pages place
 * the cost of low-bit inference in memory traffic: m.youleyou.com/wenzhang/
 * 3165839 §1, decoding is memory bound).
 *
 * The kernels use liblq's lane-contiguous layout: a wave takes 1024
 * consecutive elements (a chunk); lane L reads elements 8L..8L+7 and
 * 512+8L..512+8L+7 with two 16-byte loads, waves stride over the chunks by the
 * grid, the next chunk's loads are issued before the current chunk's stores
 * (the same software pipeline), and every store is non-temporal. lqc_read
 * and lqc_write take only the loads, or only the stores, of that layout.
 *
 * All pointers are DEVICE pointers, 16-byte aligned, each given with the
 * byte size of its buffer; work is enqueued on `stream` (a hipStream_t, NULL
 * = default) and the call returns at once. threads: 256 or 1024 per
 * workgroup; workgroups: grid size (>= 1). The caller owns every buffer.
 * Returns 0, or a negative value before anything is launched: -1 a NULL
 * pointer, -3 a bad size (including a buffer smaller than what the call
 * reads or writes), -4 a misaligned pointer; -6 a failed launch.
 */
#ifndef LQ_CEILING_H
#define LQ_CEILING_H

#include <stddef.h>
#include <stdint.h>

#define LQC_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* Read n 16-bit elements from src and write them to dst (2n bytes each way:
 * src_bytes and dst_bytes at least 2n); n must be a multiple of 1024. */
LQC_API int lqc_copy(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int64_t n, int threads,
                     int workgroups, void* stream);

/* Read `bytes` bytes of src (src_bytes >= bytes; bytes a multiple of 2048:
 * a wave's 2 KB per pass in the layout above) and nothing else in practice: a
 * lane stores its xor of what it read to its wave's 4-byte word of sink only
 * if that equals one fixed value (sink_bytes >= 4 * workgroups * threads / 64),
 * which keeps the loads from being dropped. The read-only ceiling. */
LQC_API int lqc_read(const void* src, size_t src_bytes, int64_t bytes, void* sink, size_t sink_bytes, int threads,
                     int workgroups, void* stream);

/* Write `bytes` bytes of dst (dst_bytes >= bytes; bytes a multiple of 1024:
 * a wave's 1 KB per pass, 16 bytes per lane, non-temporal), values made from
 * the position. The write-only ceiling. */
LQC_API int lqc_write(void* dst, size_t dst_bytes, int64_t bytes, int threads, int workgroups, void* stream);

/* The traffic of one bf16 fake-quant call: read n bf16 elements of x
 * (x_bytes >= 2n); write n * code_bits / 8 bytes of codes (code_bits 4, 6 or
 * 8, each code taken from its element's bits; 6-bit codes are stored as
 * liblq's FP6 kernels store them, a dword and a short per 8 codes), n / block
 * one-byte scales (block 16 .. 256, one store per block by its first lane,
 * as liblq stores 8-bit scales), and n bf16 elements of y (a copy of x,
 * y_bytes >= 2n). n must be a multiple of 1024. */
LQC_API int lqc_pattern(const void* x, size_t x_bytes, int64_t n, void* codes, size_t codes_bytes, int code_bits,
                        void* scales, size_t scales_bytes, int block, void* y, size_t y_bytes, int threads,
                        int workgroups, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LQ_CEILING_H */
