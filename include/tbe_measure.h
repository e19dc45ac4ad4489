/*
 * tbe_measure.h - measurement hooks of libtbe.so.  Not part of the TBE
 * computation: a program that only runs the forward and backward never needs
 * them.  The benchmark uses them to time one kernel on the stream it runs on
 * and to calibrate the hardware byte counters against a copy of known size.
 * They follow the conventions of tbe.h (status codes, tbe_last_error, device
 * pointers, stream order).
 */
#ifndef TBE_MEASURE_H_
#define TBE_MEASURE_H_

#include "tbe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Kernel timing for measurement.  tbe_profile_select(name) makes the library
 * record a pair of HIP events on the launch stream around every later launch
 * of the kernel called `name` (NULL stops recording);
 * tbe_profile_read waits for the recorded events and returns the number of
 * timed launches and their total milliseconds, then forgets them.
 */
tbe_status tbe_profile_select(const char* kernel_name);
tbe_status tbe_profile_read(int64_t* launches, double* total_ms);

/*
 * Measurement support: copies `bytes` (a multiple of 16, buffers 16-byte aligned)
 * from src to dst with one 16-byte load and store per lane, like the library's
 * kernels.  Its hardware byte counters, for a copy of known size, calibrate the
 * counters read for the other kernels.
 */
tbe_status tbe_calibration_copy(const void* src, void* dst, int64_t bytes, tbe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TBE_MEASURE_H_ */
