/*
 * ikbo_probe.h -- ceiling probes for the roofline (libikbo_probe.so, gfx950). Not part of the
 * method: they measure what a kernel of this part reaches for bf16 dense MFMA, HBM streaming, the
 * transcendental unit and LDS reads, to report beside the published peaks.
 *
 * ikbo_probe_launch enqueues one probe on hip_stream (a hipStream_t; NULL = default stream) and
 * returns 0, or 1 for a bad argument and 5 for a failed launch. Work per launch:
 *   IKBO_PROBE_MFMA_BF16  blocks * 4 waves * iters * 4 * 32768 FLOP; writes blocks * 256 floats
 *                         to buf (bytes >= blocks * 1024)
 *   IKBO_PROBE_EXP2       blocks * 256 threads * iters * 8 exp2 evaluations; same output
 *   IKBO_PROBE_COPY       copies the first bytes / 2 of buf (rounded down to 16) onto the
 *                         second half: that many bytes read and written
 *   IKBO_PROBE_READ       reads buf except its last blocks * 1024 bytes, which receive one word
 *                         per thread
 *   IKBO_PROBE_LDS_B128   blocks * 4 waves * iters * 16 ds_read_b128 of 1 KiB per wave (32 KiB of
 *                         LDS per block); writes blocks * 256 words of 0 to buf
 *   IKBO_PROBE_LDS_TR16   blocks * 4 waves * iters * 16 ds_read_b64_tr_b16 of 512 B per wave, over
 *                         rows of 320 bytes; same output
 * buf: device memory, 16-byte aligned, owned by the caller. iters >= 0; 1 <= blocks < 2^31.
 */
#ifndef IKBO_PROBE_H
#define IKBO_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IKBO_PROBE_MFMA_BF16 0
#define IKBO_PROBE_EXP2 1
#define IKBO_PROBE_COPY 2
#define IKBO_PROBE_READ 3
#define IKBO_PROBE_LDS_B128 4
#define IKBO_PROBE_LDS_TR16 5

int ikbo_probe_launch(int32_t kind, void *buf, size_t bytes, int64_t iters, int64_t blocks, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif
