/*
 * i8h_probe — measurement probes beside the library (libi8h_probe.so; not
 * part of the product path): an HBM read-bandwidth probe, the ceiling the
 * HBM-bound kernels are measured against on the same GPU, an FP8
 * matrix-core precision probe, which runs gfx950's native E4M3 MFMA forms on
 * caller data so that their sums can be compared with exact ones, and a
 * matrix-core / vector-ALU overlap probe.
 */
#ifndef I8H_PROBE_H
#define I8H_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at device address `buf` once, with `blocks` workgroups
 * of 256 threads (16-byte non-temporal loads, 8 in flight per thread, grid
 * stride). Nothing is written unless the XOR of a thread's pieces equals
 * `key`; then that thread writes it to sink[thread index] (sink: device
 * array of blocks * 256 uint32_t, caller-owned). buf 16-B aligned, bytes a
 * positive multiple of 16, blocks > 0 (else -1, nothing launched). Returns 0,
 * or -3 when the HIP runtime refuses the launch. Enqueued on `stream`
 * (hipStream_t as void*). */
int i8h_read_probe(const void* buf, size_t bytes, int blocks, uint32_t key, uint32_t* sink, void* stream);

/* 32x32 MFMA with float32 accumulation on caller data, one wave per tile.
 * form 0: v_mfma_f32_32x32x64_f8f6f4 on E4M3FN bytes (64 deep, 32 values of
 * one byte per lane); form 1: v_mfma_f32_32x32x16_fp8_fp8 on E4M3FN bytes
 * (16 deep, 8 per lane); form 2: v_mfma_f32_32x32x16_bf16 on bf16 values
 * (16 deep, 8 of two bytes per lane). a, b: device arrays
 * [tiles][steps][64 lanes][values per lane]; lane l holds row l % 32 of A
 * (column l % 32 of B) for contraction half l / 32. c: device float32
 * [tiles][32][32], row-major, written as
 *   c[t][m][n] = sum over steps s, h < 2, i of
 *                a[t][s][m + 32h][i] * b[t][s][n + 32h][i],
 * summed by the instruction, steps accumulated in order in float32.
 * a and b aligned to the bytes per lane (32, 8, 16), c to 4; form 0..2;
 * tiles, steps > 0; else -1 and nothing
 * launched. Returns 0, or -3 when the HIP runtime refuses the launch.
 * Enqueued on `stream` (hipStream_t as void*). */
int i8h_fp8_mfma_probe(int form, const void* a, const void* b, float* c, int tiles, int steps, void* stream);

/* MFMA / VALU overlap: `blocks` workgroups of `threads` (256 or 512: one or
 * two waves a SIMD with one workgroup a CU) threads, each wave running
 * `iters` iterations of four independent v_mfma_f32_32x32x16_bf16
 * accumulation chains with `nvalu` (0, 2, 4, 6, 8, 12 or 16) independent
 * float FMAs after each MFMA, in that order. out: device float32 array of
 * blocks * threads values (one sum per thread, caller-owned, 4-B aligned).
 * The caller times the launch; launch time / (4 iters) is the time per MFMA
 * and wave. Invalid arguments: -1, nothing launched. Returns 0, or -3 when
 * the HIP runtime refuses the launch. Enqueued on `stream`. */
int i8h_overlap_probe(int nvalu, int threads, int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* I8H_PROBE_H */
