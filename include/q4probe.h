/* q4probe.h -- C ABI of libq4probe.so: memory-bandwidth probes that measure
 * the practical ceiling of the fused 4-bit AdamW step's byte mix on the
 * device they run on.  They compute nothing of the method; the benchmark
 * reports their rates beside the step's own.
 *
 * The byte mix is the one the packed step must move per element: the FP32
 * master read and written, the BF16 gradient read, the 4-bit codes of both
 * moments read and written and one FP32 scale per 128-element block and
 * moment read and written, 12.125 bytes per element ("Rounding in
 * Preconditioner Space", Table 2 recipes; AReno docs "4-bit AdamW", section
 * "State representation": 128-element blocks of 4-bit codes with one FP32
 * scale; the news article's storage paragraph: 1.0625 bytes of state per
 * parameter).
 *
 * Every pointer is device memory of the current HIP device, 16-byte
 * aligned, owned by the caller; `stream` is a hipStream_t (NULL: the null
 * stream).  Calls enqueue one kernel and return; they allocate nothing.
 * Return values: Q4PROBE_OK, Q4PROBE_ERR_ARG (nothing enqueued) or
 * Q4PROBE_ERR_HIP (the launch failed).
 */
#ifndef Q4PROBE_H
#define Q4PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4PROBE_OK 0
#define Q4PROBE_ERR_ARG 1
#define Q4PROBE_ERR_HIP 2

/* Bytes one q4probe_byte_mix call moves for n elements: 12.125 n. */
int64_t q4probe_byte_mix_bytes(int64_t n);

/* The step's byte mix over n elements (n a positive multiple of 512):
 * param (n floats) and the codes (n/2 bytes each) and scales (n/128 floats
 * each) are read and rewritten in place with trivial arithmetic; grad (n
 * BF16 bit patterns) is read.  Same lane layout, cache policy (masters and
 * gradients nontemporal) and work-group walk as the step kernel. */
int q4probe_byte_mix(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                     float* v_scales, int64_t n, void* stream);

/* The same byte mix and arithmetic as q4probe_byte_mix, its chunks taken
 * by one round of resident work-groups from a queue (a device word of this
 * library, zeroed before the launch; calls that overlap on one device race
 * on it): the fastest way found to move this byte mix. */
int q4probe_byte_mix_queue(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                           float* v_scales, int64_t n, void* stream);

/* Bytes one q4probe_byte_mix8 call moves for n elements: 14.125 n. */
int64_t q4probe_byte_mix8_bytes(int64_t n);

/* The byte mix of the 8-bit blockwise step (AReno docs "4-bit AdamW",
 * section "Requirements and errors", names the 8-bit blockwise AdamW; one
 * byte per code and 128-element blocks here): as
 * q4probe_byte_mix, with m_codes and v_codes holding n bytes each, read and
 * rewritten 8 bytes per lane (4 in each half of its block), and the
 * work-groups taking runs of 4 slabs as the 8-bit step does. */
int q4probe_byte_mix8(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                      float* v_scales, int64_t n, void* stream);

/* The 8-bit byte mix taken from the queue, as q4probe_byte_mix_queue (the
 * same device word: calls that overlap on one device race on it). */
int q4probe_byte_mix8_queue(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes,
                            float* m_scales, float* v_scales, int64_t n, void* stream);

/* dst <- src, `bytes` (a positive multiple of 16) read and written once. */
int q4probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/* x <- x * 0.999f (FP32) in place: `bytes` (a positive multiple of 16) read
 * and written back to the same addresses, the way the step rewrites its
 * state. */
int q4probe_update_in_place(float* x, size_t bytes, void* stream);

/* Words a q4probe_read sink must hold. */
int64_t q4probe_read_sink_words(void);

/* Reads `bytes` (a positive multiple of 16) of src once; each thread leaves
 * the XOR of what it read in `sink` (q4probe_read_sink_words() words). */
int q4probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* Q4PROBE_H */
