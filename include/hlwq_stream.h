/*
 * hlwq_stream.h — C ABI of libhlwq_stream, the streaming-bandwidth probe that
 * bench.py uses as the practical HBM ceiling for a kernel's own traffic mix.
 *
 * Not part of the quantization path: the kernels here read and write bytes
 * with no arithmetic, in the access pattern of the HLWQ kernels (each wave
 * loads a run of `read_bytes` with 1 KB-contiguous direct-to-LDS loads and
 * stores a run of `write_bytes` with 1 KB-contiguous stores, both with the
 * streaming cache policy), so that a quantize or dequantize launch can be
 * compared with the fastest pure data movement of the same read:write mix on
 * the same device.
 *
 * Units: unit u (0 <= u < units) reads bytes [u * read_bytes, (u + 1) *
 * read_bytes) of `src` and writes bytes [u * write_bytes, (u + 1) *
 * write_bytes) of `dst`; what is written is unspecified (stale staging
 * data).  The waves of a persistent grid, `workgroups_per_cu` 4-wave
 * workgroups per compute unit, take units in turn.
 *
 * Variants (how a wave overlaps its loads and stores):
 *   0  load a unit, wait, store it; 16 KB of LDS per wave (read_bytes <= 16384)
 *   1  the same with 32 KB of LDS per wave (read_bytes <= 32768)
 *   2  double-buffered: the next unit's loads are issued before this unit is
 *      waited for and stored; 2 x 16 KB per wave (read_bytes <= 16384)
 *   3  double-buffered with 2 x 4 KB per wave (read_bytes <= 4096)
 * LDS per workgroup is 4 waves times the stage, so variant 0 allows up to 2
 * workgroups per CU, 1 and 2 one, 3 up to 4.
 *
 * Ownership and errors as in hlwq.h: the caller owns device buffers of at
 * least units * read_bytes (src) and units * write_bytes (dst) bytes, 16-byte
 * aligned; the call validates its arguments, enqueues one launch on
 * `hip_stream` and returns 0, or a negative status without enqueuing
 * anything: -1 NULL pointer, -2 sizes (not multiples of 16, too large for the
 * variant, zero write size), -3 unknown variant or workgroups_per_cu outside
 * 1..4, -5 launch error, -6 misaligned buffer.
 */
#ifndef HLWQ_STREAM_H
#define HLWQ_STREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int hlwq_stream_mix(const void* src, void* dst, uint32_t read_bytes, uint32_t write_bytes, uint32_t units,
                    int variant, int workgroups_per_cu, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* HLWQ_STREAM_H */
