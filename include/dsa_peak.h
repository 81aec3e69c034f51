/*
 * dsa_peak.h -- measured peaks of the current HIP device (gfx950), for
 * reporting the indexer kernels' efficiency against what the device really
 * sustains next to its specification sheet.  Built as libdsa_peak.so, apart
 * from the indexer library; used by the benchmark only.
 *
 * The indexer's prefill is a dense fp8 contraction and its decode streams the
 * fp8 key cache from HBM ("IndexCache deep-dive report", abstract and
 * section 1.1: the indexer runs in FP8 and scores every earlier token;
 * "Multi-layer Indexer" abstract: at decode the indexer scan over the whole
 * cache is where the time goes), so the two yardsticks are the matrix-core
 * rate and the HBM read rate.
 *
 * Every function runs its kernel on `stream` (a hipStream_t, NULL = the
 * default stream), synchronizes it, and returns 0 on success or a HIP error
 * code.  Each is timed with HIP events on that stream over `iters` launches
 * after one untimed launch; the result is the mean rate over the timed ones.
 * Unlike the indexer library these calls synchronize, and the MFMA ones
 * allocate (and free) 16 bytes of device memory for the clock readings.
 */
#ifndef DSA_PEAK_H
#define DSA_PEAK_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense MFMA rate in TFLOP/s (2 flops per multiply-add): every wave of a
 * grid that fills the device issues only independent
 * v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 e4m3) or v_mfma_f32_32x32x16_bf16
 * instructions.  *clock_mhz (may be NULL) receives the shader clock the
 * kernel observed (shader-clock counter against the constant-rate clock). */
int dsa_peak_mfma_fp8(int iters, double* tflops, double* clock_mhz, void* stream);
int dsa_peak_mfma_bf16(int iters, double* tflops, double* clock_mhz, void* stream);

/* HBM read rate in GB/s: `bytes` (a multiple of 16, at least 1 MiB) of
 * device memory at `buf` (16-byte aligned) read once per launch with
 * coalesced 16-byte loads.  Choose `bytes` well above the 256 MB last-level
 * cache so the reads come from HBM. */
int dsa_peak_hbm_read(const void* buf, size_t bytes, int iters, double* gbps, void* stream);

/* HBM copy rate in GB/s counting read + written bytes (2 * bytes per launch). */
int dsa_peak_hbm_copy(const void* src, void* dst, size_t bytes, int iters, double* gbps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_PEAK_H */
