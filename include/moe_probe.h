/* Measurement helpers of libmoe.so -- not part of the MoE layer.
 *
 * They measure, on the device and in the run that times the layer, the
 * peaks its kernels can reach: a read stream (the decode GEMMs stream their
 * weights) and a dense MFMA loop (the prefill GEMMs).  bench.py reports the
 * layer's kernels against these as well as against the nominal peaks.
 * All return MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_HIP (launch failure);
 * launches are asynchronous on `stream`; time them with events. */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of buf (device memory, bytes a multiple of 16) once with
 * 16-byte non-temporal loads.  sink: device uint32 [moe_probe_read_blocks()],
 * one folded word per workgroup (written, values meaningless). */
int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, moe_stream_t stream);
int32_t moe_probe_read_blocks(void);

/* iters rounds of 8 independent MFMAs per wave, 4 workgroups of 4 waves per
 * CU: dtype 0 = v_mfma_f32_32x32x16_bf16, 1 = v_mfma_scale_f32_16x16x128_f8f6f4
 * (e4m3, unit scales).  sink: device float [moe_probe_mfma_blocks() * 256].
 * moe_probe_mfma_flops gives the FLOPs of one launch. */
int moe_probe_mfma(int32_t dtype, int32_t iters, float* sink, moe_stream_t stream);
int32_t moe_probe_mfma_blocks(void);
int64_t moe_probe_mfma_flops(int32_t dtype, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
