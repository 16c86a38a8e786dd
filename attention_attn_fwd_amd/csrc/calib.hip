// Calibration kernel for the hardware counters the benchmark reads
// (libattn_calib.so, loaded only by bench.py --workload mfma_cal; not part of
// the attention library).  Every wave issues exactly `iters` * 8
// v_mfma_f32_16x16x32_bf16 instructions (the prefill kernel's instruction)
// on four independent accumulators and nothing else in its loop, so
// SQ_INSTS_MFMA must read waves * iters * 8, SQ_VALU_MFMA_BUSY_CYCLES that
// times the instruction's cycles, and with two waves per SIMD the matrix
// units are busy for the whole dispatch: busy cycles over SIMDs x duration
// give the shader clock, against which GRBM_GUI_ACTIVE is scaled.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__global__ __launch_bounds__(512) void calib_mfma_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (tid + e));
    b[e] = (__bf16)(0.002f * (tid - e));
  }
  f32x4 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int g = 0; g < 8; ++g) c[g & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[g & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[(int64_t)blockIdx.x * blockDim.x + tid] = s;
}

}  // namespace

extern "C" {

// Launches `blocks` workgroups of 512 threads (8 waves); out holds
// blocks * 512 floats (device memory).  Returns a hipError_t as int.
int attn_calib_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream), out, iters);
  return (int)hipGetLastError();
}

// MFMA instructions one call issues.
int64_t attn_calib_mfma_count(int blocks, int iters) { return (int64_t)blocks * 8 * iters * 8; }

}  // extern "C"
