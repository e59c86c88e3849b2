/*
 * i8h_probe — HBM read-bandwidth probe for measuring the library's
 * HBM-bound kernels against what a plain read reaches on the same GPU
 * (libi8h_probe.so; not part of the product path).
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

#ifdef __cplusplus
}
#endif

#endif /* I8H_PROBE_H */
