/*
 * streamkl_probe.h — measurement aid shipped with the attention-KL library (not part of the
 * method): the dense bf16 matrix-core rate this GPU sustains, and the shader clock it runs at
 * meanwhile, as the denominator the benchmark reports beside the published MI355X peak.
 */
#ifndef STREAMKL_PROBE_H
#define STREAMKL_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `nblocks` workgroups of 256 threads (four wavefronts) on hip_stream; every wavefront
 * issues 4 * iters v_mfma_f32_32x32x16_bf16 (32768 flops each) on register operands, with no
 * memory traffic in its loop.  Outputs (DEVICE buffers owned by the caller):
 *   sink    float [nblocks * 256]: one value per thread, written only so the work is kept;
 *   clocks  uint64 [2 * nblocks]: per workgroup, the shader-clock counter (s_memtime) and the
 *           constant-rate counter (s_memrealtime) elapsed across its loop.
 * wall_clock_khz (HOST) receives the rate of the constant-rate counter (hipDeviceAttributeWallClockRate),
 * so a workgroup's clock in kHz is clocks[2b] / clocks[2b + 1] * wall_clock_khz.  The caller times
 * the launch (e.g. with events) for the rate: nblocks * 4 * 4 * iters * 32768 flops.
 * Returns 0, 1 for a bad argument (nothing launched) or 3 when the launch fails.  Allocates nothing. */
int streamkl_probe_mfma(int nblocks, int iters, float* sink, unsigned long long* clocks, double* wall_clock_khz,
                        void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* STREAMKL_PROBE_H */
