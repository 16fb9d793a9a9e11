/*
 * libsqa_probe -- issue-rate probes for gfx950 (measurement aids, not part of
 * the attention path; built next to libsqa as libsqa_probe.so).
 *
 * They bound what the d = 64 forward kernel can reach with its instruction
 * mix: each kind runs a fixed per-iteration instruction stream from
 * registers only (no HBM traffic, no barriers) in 4-wave workgroups with the
 * forward's occupancy of two workgroups per compute unit. Time a launch with
 * HIP events and divide the work below by it.
 *
 *   kind 0  16 v_mfma_f32_32x32x16_bf16 per wave and iteration, nothing else
 *           (32768 FLOP each): the matrix pipe's rate under this load.
 *   kind 1  the forward's two-phase step: per iteration 16 MFMAs (as kind 0)
 *           interleaved with the softmax of 2 x 16 scores per lane (32
 *           v_fma_f32, 32 v_exp_f32, 16 v_cvt_pk_bf16_f32, 16
 *           v_dot2c_f32_bf16, running-sum update and range check).
 *   kind 2  kind 1 plus the forward's LDS fragment reads per iteration
 *           (4 ds_read_b128, 8 ds_read_b64_tr_b16) from a tile written once.
 *   kind 3  16 v_exp_f32 per lane and iteration (64 lanes per wave).
 *   kind 4  16 v_fma_f32 per lane and iteration.
 *
 *   workgroups  >= 1 (use 2 x the compute units to fill the chip)
 *   iters       >= 1 iterations per wave
 *   out         DEVICE float buffer of sqa_probe_threads(workgroups) floats,
 *               owned by the caller; receives meaningless checksums
 *   stream      hipStream_t as void*; the launch is asynchronous
 * Returns 0 (hipSuccess) or the HIP error code of the launch; invalid
 * arguments return hipErrorInvalidValue without launching.
 */
#ifndef SQA_PROBE_H_
#define SQA_PROBE_H_

#ifdef __cplusplus
extern "C" {
#endif

int sqa_probe_threads(int workgroups);
int sqa_probe_run(int kind, int workgroups, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SQA_PROBE_H_ */
