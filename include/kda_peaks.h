/*
 * kda_peaks.h -- C ABI of libkda_peaks, the on-device reference measurements
 * that the benchmark reports beside libkda's rates: what a plain streaming copy
 * and a dense bf16 matrix-core loop reach on the GPU at hand, and the device's
 * own description of itself.  The operator never calls these; they exist so
 * that a measured rate can be set against both the vendor's published peak and
 * what the same device delivers to a kernel that does nothing else.
 *
 * Pointers are device pointers owned by the caller; every call validates its
 * arguments on the host before any HIP call and returns 0 on success, 1 for a
 * bad argument and 2 when HIP reports an error.  Work is enqueued on `stream`
 * (a hipStream_t passed as void*) and timed by the caller.
 */
#ifndef KDA_PEAKS_H_
#define KDA_PEAKS_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copies `bytes` bytes (a multiple of 16; src and dst 16-byte aligned and not
 * overlapping) with 16-byte loads and stores, four per thread in flight: every
 * byte is read once from src and written once to dst.  Timing it gives the
 * device's streaming rate, 2*bytes / time. */
int kda_peaks_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Runs `workgroups` workgroups of four wavefronts; each wavefront issues
 * `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 instructions
 * (16 x 16 x 32 multiply-adds = 16,384 flop each) and writes one float per lane
 * to sink ([workgroups * 256] floats) so that nothing is optimised away.
 * flop = workgroups * 4 * iters * 8 * 16384. */
int kda_peaks_mfma_bf16(float* sink, int workgroups, int iters, void* stream);

/* What the runtime reports for `device`. */
typedef struct kda_device_info {
    char name[256];            /* marketing name                                  */
    char arch[64];             /* gfx target, e.g. "gfx950:sramecc+:xnack-"       */
    int compute_units;         /* multiProcessorCount                             */
    int clock_khz;             /* peak shader clock                               */
    int memory_clock_khz;      /* peak memory clock                               */
    int memory_bus_bits;       /* memory bus width                                */
    int l2_bytes;              /* L2 cache of one die as reported                 */
    long long total_bytes;     /* device memory                                   */
    int lds_bytes_per_cu;      /* shared memory per compute unit                  */
    int warp_size;             /* wavefront width                                 */
} kda_device_info;

int kda_peaks_device(int device, kda_device_info* info);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PEAKS_H_ */
