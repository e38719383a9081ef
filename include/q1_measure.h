/*
 * q1_measure.h -- measurement aid of the packed Q1 library (libq1.so), not a
 * step of the decode path.  Status codes and conventions as in q1.h.
 */
#ifndef Q1_MEASURE_H
#define Q1_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "q1.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * q1_stream_read -- one pass that reads `bytes` bytes at `data` with 16-byte
 * non-temporal loads (the access of the packed kernels) and computes nothing
 * else.  Its duration is the ceiling a single launch reading that many bytes
 * can reach: the context for the HBM rooflines of the other calls.
 *   data   device memory, 16-byte aligned; bytes a multiple of 16, < 2^31
 *   sink   device uint32, written only if the data XOR to a fixed sentinel
 */
q1_status q1_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q1_MEASURE_H */
