// Measurement probes (libfa_probe.so, declared in include/fa_probe.h): the
// rates the attention kernels of libfa.so are bounded by, taken on the device
// they run on.
//   * the dense fp16 MFMA rate: waves issuing back-to-back independent
//     v_mfma_f32_32x32x16_f16 on register operands (the ceiling of every
//     matrix product in the forward and backward);
//   * the v_exp_f32 rate: waves issuing independent base-2 exponentials, one
//     per score in the forward's online softmax and per recomputed
//     probability in the backward ("Triton FlashAttention": exp2 on
//     log2(e)-prescaled scores), the secondary ceiling beside the MFMAs.
// Each launch fills every SIMD with two waves and writes one float per
// thread to a caller-owned sink so that no work is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_probe.h"
#include "fa_common.h"

namespace fa {

namespace {

__global__ __launch_bounds__(256, 2) void probe_mfma_kernel(int iters, float* sink) {
  const int t = (int)threadIdx.x;
  h8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (half_t)(0.001f * (float)((t + e) & 15));
    b[e] = (half_t)(0.001f * (float)((t * 3 + e) & 15));
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = Mfma<half_t>::mma(a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  sink[(int64_t)blockIdx.x * blockDim.x + t] = s;
}

__global__ __launch_bounds__(256, 2) void probe_exp_kernel(int iters, float* sink) {
  const int t = (int)threadIdx.x;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.25f + 0.001f * (float)((t + j) & 63);
  // x -> 2^-x keeps every chain inside (0.5, 1): one v_exp_f32 (with its
  // negate modifier) per step, eight independent chains per lane.
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fast_exp2(-x[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  sink[(int64_t)blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

int probe_workgroups() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  return 2 * cus;  // 4 waves each: two waves per SIMD
}

hipError_t launch_probe(int kind, int iters, float* sink, hipStream_t s) {
  const int grid = probe_workgroups();
  void* args[] = {&iters, &sink};
  const void* k = kind == 0 ? reinterpret_cast<const void*>(&probe_mfma_kernel)
                            : reinterpret_cast<const void*>(&probe_exp_kernel);
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(256), args, 0, s);
}

}  // namespace fa

extern "C" {

int64_t fa_probe_threads(void) { return (int64_t)fa::probe_workgroups() * 256; }

int fa_probe(int kind, int iters, float* sink, void* stream) {
  if (kind < 0 || kind > 1 || iters < 1) return FA_ERR_SHAPE;
  if (!sink) return FA_ERR_NULL;
  return fa::launch_probe(kind, iters, sink, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
