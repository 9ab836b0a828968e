/*
 * mla8 auxiliary calls: measurement and test aids exported by libmla8.so next
 * to the attention path (include/mla8.h) but not part of it.  Like every call
 * of the library they keep no state between calls and only enqueue work on
 * `stream`.  A decode loop needs none of them.
 */
#ifndef MLA8_AUX_H
#define MLA8_AUX_H

#include "mla8.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read-bandwidth reference, the line the decode's HBM rate is compared with.
 * Loads every 16-byte word of [p, p + bytes) once (coalesced, grid-stride) and
 * XOR-folds them: out (device memory, MLA8_STREAM_WORDS uint32, 16-byte
 * aligned) receives one fold per wave, every word written, so that the XOR of
 * all its words is the XOR of the buffer's 32-bit words and no load can be
 * dropped.  p: device pointer, 16-byte aligned; bytes a multiple of 16.
 * Errors: E_INVAL (NULL pointer, misalignment, bytes < 0 or not a multiple of
 * 16), E_HIP.
 */
#define MLA8_STREAM_WORDS 32768
MLA8_API int mla8_stream_read(const void* p, int64_t bytes, uint32_t* out, void* stream);

/*
 * Test aid: the device e4m3 encoder applied elementwise, codes[i] = enc(x[i])
 * for i < n, with no scaling, so that tests can compare it with the reference
 * on every f32 bit pattern, including finite |x| > 448 which the quantizer
 * never produces.  Errors: E_INVAL, E_HIP.
 */
MLA8_API int mla8_test_encode(const float* x, int64_t n, uint8_t* codes, void* stream);

/*
 * Test aid: the packed hardware e4m3 encoder that the e4m3 lo query term of
 * mla8_opts uses (v_cvt_pk_fp8_f32, round to nearest even onto OCP e4m3),
 * codes[i] = e4m3(x[i]) for i < n.  Exact for finite |x[i]| < 448, the only
 * inputs the decode gives it (|lo 2^j| < 256); it does not saturate, so other
 * inputs give codes that differ from mla8_test_encode.  n a multiple of 4, x
 * 16-byte aligned, codes 4-byte aligned.  Errors: E_INVAL, E_HIP.
 */
MLA8_API int mla8_test_encode_pk(const float* x, int64_t n, uint8_t* codes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA8_AUX_H */
