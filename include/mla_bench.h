/*
 * mla_bench.h - C ABI of libmla_bench.so: a measurement helper that sits beside libmla.so
 * and is no part of the decode path.
 *
 * mla_bench_stream_read gives the streaming-read rate of the device, the reference against
 * which the decode's cache-read rate is judged (the decode is bound by reading the latent
 * cache from HBM once per step).  It reads every 16-byte word of buf once: workgroup w
 * (256 threads) reads words [w * per, min((w + 1) * per, words)), per = ceil(words /
 * num_workgroups), four loads in flight per thread, plain loads (nontemporal = 0) or loads
 * with the non-temporal hint, and writes the XOR of each wavefront's words to
 * sink[4 * w + wavefront], so that no load is dead and the caller can check what was read.
 *
 * buf            device pointer, 16-byte aligned.      bytes  a multiple of 16, >= 16.
 * sink           device uint32 [4 * num_workgroups], 4-byte aligned, written, never read.
 * num_workgroups 1 .. 65535 (a few per compute unit fill the device: 2,048 on MI355X).
 * stream         hipStream_t as void* (NULL = null stream); asynchronous, allocates nothing.
 * Returns 0, or 1 (NULL pointer), 2 (size or count out of range), 3 (alignment), 6 (launch
 * failed), the MLA_ERR_* numbering of mla.h.
 */
#ifndef MLA_BENCH_H_
#define MLA_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MLA_BENCH_API __attribute__((visibility("default")))
#else
#define MLA_BENCH_API
#endif

MLA_BENCH_API int mla_bench_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int32_t num_workgroups,
                                        int32_t nontemporal, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_BENCH_H_ */
