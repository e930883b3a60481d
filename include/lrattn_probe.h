/*
 * lrattn_probe.h - plain kernels shipped beside lrattn for measurement: the
 * attainable read / copy bandwidth of the device, a copy of known size
 * against which hardware byte counters are calibrated, and a shader-clock
 * sample.  They compute nothing of the attention method.
 *
 * Same conventions as lrattn.h: device pointers, 16-byte aligned, caller-owned,
 * asynchronous on `stream`, negative lrattn_status on error, host-side
 * validation before any launch.
 */
#ifndef LRATTN_PROBE_H
#define LRATTN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "lrattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of fp32 values lrattn_probe_read writes to its sink. */
size_t lrattn_probe_sink_floats(void);

/*
 * Read `bytes` bytes (a multiple of 16) from `src` with 16-byte loads and
 * write one fp32 per workgroup to `sink` (lrattn_probe_sink_floats() values)
 * so the loads cannot be removed.  Bytes moved: `bytes` read, a few KB written.
 */
int lrattn_probe_read(const void* src, size_t bytes, float* sink, lrattn_stream stream);

/* Copy `bytes` bytes (a multiple of 16) from `src` to `dst` (no overlap). */
int lrattn_probe_copy(void* dst, const void* src, size_t bytes, lrattn_stream stream);

/*
 * Shader clock: one lane of one workgroup spins for about 5 us of the
 * 100 MHz real-time counter and writes out[0] = shader-clock cycles
 * (s_memtime) and out[1] = real-time ticks over that spin, so the clock in
 * GHz is out[0] / out[1] / 10.  Enqueued on `stream` between other launches,
 * it samples the clock they run at.  `out`: 2 uint64 of device memory,
 * 16-byte aligned.
 */
int lrattn_probe_clock(uint64_t* out, lrattn_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* LRATTN_PROBE_H */
