/*
 * tv_probe.h -- measurement probes that the benchmark runs beside libtv (libtv_probe.so).
 *
 * None of the probes is part of the verify step. Two give the ceilings that the attention
 * kernel's bandwidth is set against on the machine it runs on:
 *   - the rate at which plain reads stream from HBM, contiguous or in the KV cache's
 *     pattern (one KV head's 256-byte rows every Hkv * 256 bytes);
 *   - the shader clock the chip runs at under a given load (it drops below the nominal
 *     2.4 GHz when power limits bind).
 * The third times MFMA and VALU instruction mixes in shader cycles: how far one wave, or
 * two sharing a SIMD, overlap matrix and vector work. The fourth runs MFMA streams with
 * LDS reads and VALU work beside them on every CU at once: the throughput that the
 * attention loop's instruction mix can reach with no dependencies between its parts.
 * Pointers are device pointers; `stream` is a hipStream_t passed as void*. The calls
 * only enqueue work. They return 0 on success, 1 for an invalid argument and 5 when the
 * HIP runtime refuses the launch.
 */
#ifndef TV_PROBE_H_
#define TV_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streams `rows` x `cols` blocks of `row_bytes` bytes from HBM: block (r, c) lies at
 * base + r * row_stride + c * row_bytes. Workgroup w (256 threads, each keeping eight
 * 16-byte loads in flight) reads rows [(w / cols) * rows_per_wg, + rows_per_wg) of column
 * w % cols; the grid has ceil(rows / rows_per_wg) * cols workgroups. Each workgroup writes
 * the XOR of what it read to sink[w] (uint32 [grid]), so no load is dead.
 * Limits: row_bytes a power of two in [16, 65536], row_stride >= row_bytes * cols and a
 * multiple of 16, base 16-byte aligned, rows_per_wg * row_bytes / 16 below 2^30.
 */
int tv_probe_stream_read(const void* base, int64_t rows, int row_bytes, int64_t row_stride, int cols,
                         int64_t rows_per_wg, uint32_t* sink, void* stream);

/*
 * One wave spins for `ticks` ticks of the constant-rate real-time counter and writes
 * out[0] = shader-clock cycles and out[1] = real-time ticks elapsed (uint64 [2]); their
 * ratio times the real-time rate is the shader clock over the spin. 1 <= ticks <= 1e8.
 */
int tv_probe_clock(uint64_t* out, uint64_t ticks, void* stream);

/*
 * One workgroup of `threads` (64, 256 or 512) threads runs `iters` iterations of an
 * instruction mix and each wave writes its shader-clock cycle count to cycles[wave]
 * (uint64 [threads / 64]). Every iteration issues eight v_mfma_f32_32x32x16_bf16 on four
 * independent accumulators and/or VALU work: mode 0 MFMAs only; 1 64 fp32 FMAs (eight
 * independent chains); 2 each MFMA followed by 8 FMAs; 3 each MFMA followed by 4 exp2 and
 * 4 FMAs; 4 64 exp2; 5 each MFMA followed by 2 exp2 and 6 FMAs. `in` (fp32, >= 128
 * values) seeds the operands; `out` (fp32 [threads]) receives a checksum so that no work
 * is dead. Returns 1 for an invalid argument.
 */
int tv_probe_coissue(int mode, int threads, int iters, const float* in, float* out, uint64_t* cycles,
                     void* stream);

/*
 * `workgroups` workgroups of `threads` (256 or 512: one or two waves per SIMD) threads
 * each run `iters` iterations of eight v_mfma_f32_32x32x16_bf16 on four independent
 * accumulators. lds_step 1: every MFMA's A operand is a fresh 16-byte-per-lane LDS read
 * (1 KB per wave and MFMA); 2: every second MFMA's (0.5 KB); 0: no LDS reads. 3-5 read
 * 1 KB per MFMA in the attention tiles' layout (256-byte rows, the K and V swizzles): 3
 * alternates K fragments (128-bit reads) with V^T fragments (two ds_read_b64_tr_b16 per
 * lane), the attention loop's mix; 4 reads only V^T fragments, 5 only K; 6 and 7 model 64
 * rows per wave (each fragment feeding two MFMAs): 6 reads K, -, V^T, - per four MFMAs
 * (0.5 KB per MFMA), 7 reads K, K, V^T, - (0.75 KB). valu 1: each
 * MFMA is followed by one exp2 and four FMAs on independent values; 0: none. Workgroup 0's
 * first wave writes clk[0] = shader-clock cycles and clk[1] = real-time ticks around its
 * loop (uint64 [2]). `in` (fp32, >= 1024 values) seeds the operands; `out` (fp32
 * [workgroups * threads]) receives a checksum per thread. 1 <= workgroups <= 65536.
 */
int tv_probe_mix(int lds_step, int valu, int threads, int workgroups, int iters, const float* in, float* out,
                 uint64_t* clk, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TV_PROBE_H_ */
