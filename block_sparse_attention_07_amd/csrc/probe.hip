// bsa_mfma_probe: a measurement aid beside the attention path, not part of it.
// Every wave runs a loop of bf16 MFMAs (v_mfma_f32_32x32x16_bf16, the
// instruction the attention kernels use) on operands held in registers: four
// independent accumulator chains of four MFMAs each per iteration, no memory
// traffic, two workgroups of four waves per CU (the attention kernels'
// occupancy).  Its rate is the MFMA issue rate at the clock the chip holds under
// sustained MFMA load, which bounds any bf16 contraction on this GPU.
#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_CHAINS = 4;
constexpr int PROBE_DEPTH = 4;

__global__ __launch_bounds__(PROBE_THREADS, 2) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // Four operand sets of pseudo-random values in [-2, 2), used in rotation so that
  // consecutive MFMAs see different data: the datapath then switches (and draws
  // power) as it does on attention tiles, instead of repeating one product.
  bf16x8 a[4], b[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ha = (uint32_t)(lane * 8 + j) * 2654435761u + (uint32_t)m * 40503u;
      const uint32_t hb = (uint32_t)(lane * 8 + j) * 2246822519u + (uint32_t)m * 97007u + 12345u;
      a[m][j] = (__bf16)((float)((ha >> 16) & 0xffff) * (1.0f / 16384.0f) - 2.0f);
      b[m][j] = (__bf16)((float)((hb >> 16) & 0xffff) * (1.0f / 16384.0f) - 2.0f);
    }
  f32x16 acc[PROBE_CHAINS];
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < PROBE_DEPTH; ++r)
#pragma unroll
      for (int c = 0; c < PROBE_CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + c) & 3], b[(r + 2 * c + 1) & 3], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[(size_t)blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
}

}  // namespace
}  // namespace bsa

extern "C" int bsa_mfma_probe(int iterations, float* sink, long long sink_floats, double* flops_host,
                              hipStream_t stream) {
  using namespace bsa;
  if (iterations < 1 || iterations > 10000000)
    return fail(BSA_ERR_INVALID_ARG, "iterations must be in [1, 1e7] (got %d)", iterations);
  if (!sink || !aligned(sink, 4) || !flops_host)
    return fail(BSA_ERR_INVALID_ARG, "sink must be a 4-byte aligned device pointer and flops_host non-null");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  const long long wgs = 2LL * cus;
  if (sink_floats < wgs * PROBE_THREADS)
    return fail(BSA_ERR_INVALID_ARG, "sink holds %lld floats; the probe writes %lld", sink_floats,
                wgs * PROBE_THREADS);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)wgs), dim3(PROBE_THREADS), 0, stream, iterations, sink);
  BSA_CHECK_HIP(hipGetLastError());
  *flops_host = (double)wgs * (PROBE_THREADS / 64) * iterations * (PROBE_CHAINS * PROBE_DEPTH) * 32.0 * 32.0 * 16.0 * 2.0;
  return ok();
}
