// Resolution scaling of block maps (ScalingAttention section 4.3.1, Eq. 7).
//
// A map built at a base block count n_b is resized to n_t blocks by bilinear
// interpolation at (u / s, v / s), s = n_t / n_b, with a ceiling that keeps any
// overlap with an active region.  On a binary region map the ceiling of the
// interpolated value is 1 exactly when a base sample with positive weight is
// active, so the kernels evaluate that rule in integers: along each axis the
// sample is x0 = floor(u n_b / n_t) (clamped to n_b - 1) and the next sample
// enters with positive weight iff u n_b is not a multiple of n_t.
//   * mask_resize: packed region maps; one wave builds one target word (OR of
//     up to four base bits per lane, then a ballot).
//   * threshold_map_resize: float32 threshold maps; the conservative
//     counterpart of the ceiling is the minimum over the positive-weight
//     samples (NaN ignored), so thresholding and resizing commute.
#include <algorithm>
#include <cmath>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int NT = 256;

struct Axis {
  int a, b;   // samples (b == a when only one has positive weight)
};

__device__ __forceinline__ Axis axis_samples(int u, int nb, int nt) {
  const long long x = (long long)u * nb;
  int q = (int)(x / nt);
  const bool frac = (x % nt) != 0;
  q = min(q, nb - 1);
  return {q, frac ? min(q + 1, nb - 1) : q};
}

__device__ __forceinline__ bool bit_at(const uint64_t* row, int v) { return (row[v >> 6] >> (v & 63)) & 1ull; }

__global__ __launch_bounds__(NT) void mask_resize_kernel(const uint64_t* __restrict__ base, int nb, int nt,
                                                         int Wb, int Wt, long long words,
                                                         uint64_t* __restrict__ target) {
  const int lane = threadIdx.x & 63;
  const long long stride = (long long)gridDim.x * (NT / 64);
  for (long long wid = (long long)blockIdx.x * (NT / 64) + (threadIdx.x >> 6); wid < words; wid += stride) {
    const long long row = wid / Wt;              // h * nt + u
    const int w = (int)(wid - row * Wt);
    const int h = (int)(row / nt), u = (int)(row - (long long)h * nt);
    const int v = 64 * w + lane;
    bool on = false;
    if (v < nt) {
      const Axis x = axis_samples(u, nb, nt), y = axis_samples(v, nb, nt);
      const uint64_t* r0 = base + ((size_t)h * nb + x.a) * Wb;
      const uint64_t* r1 = base + ((size_t)h * nb + x.b) * Wb;
      on = bit_at(r0, y.a) || bit_at(r0, y.b) || bit_at(r1, y.a) || bit_at(r1, y.b);
    }
    const uint64_t bits = __ballot(on);
    if (lane == 0) target[wid] = bits;
  }
}

__global__ __launch_bounds__(NT) void threshold_resize_kernel(const float* __restrict__ base, int nb, int nt,
                                                              long long total, float* __restrict__ target) {
  const long long stride = (long long)gridDim.x * NT;
  for (long long i = (long long)blockIdx.x * NT + threadIdx.x; i < total; i += stride) {
    const long long row = i / nt;
    const int v = (int)(i - row * nt);
    const int h = (int)(row / nt), u = (int)(row - (long long)h * nt);
    const Axis x = axis_samples(u, nb, nt), y = axis_samples(v, nb, nt);
    const float* b = base + (size_t)h * nb * nb;
    const float m = fminf(fminf(b[(size_t)x.a * nb + y.a], b[(size_t)x.a * nb + y.b]),
                          fminf(b[(size_t)x.b * nb + y.a], b[(size_t)x.b * nb + y.b]));
    target[i] = m;
  }
}

int check_resize(const void* base, const void* target, int n_heads, int nb, int nt, size_t align) {
  if (!base || !target) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(base, align) || !aligned(target, align)) return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || nb < 1 || nt < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if ((long long)n_heads * nt > 0x7fffffffLL || (long long)n_heads * nb > 0x7fffffffLL)
    return fail(BSA_ERR_INVALID_ARG, "problem too large");
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" int mask_resize(const uint64_t* base_bits, int n_heads, int nb_base, int nb_target,
                           uint64_t* target_bits, hipStream_t stream) {
  using namespace bsa;
  int rc = check_resize(base_bits, target_bits, n_heads, nb_base, nb_target, 8);
  if (rc) return rc;
  const int Wb = n_words(nb_base), Wt = n_words(nb_target);
  const long long words = (long long)n_heads * nb_target * Wt;
  const long long blocks = std::min<long long>((words + NT / 64 - 1) / (NT / 64), 1 << 16);
  hipLaunchKernelGGL(mask_resize_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, base_bits, nb_base,
                     nb_target, Wb, Wt, words, target_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}

extern "C" int threshold_map_resize(const float* base, int n_heads, int nb_base, int nb_target,
                                    float* target, hipStream_t stream) {
  using namespace bsa;
  int rc = check_resize(base, target, n_heads, nb_base, nb_target, 4);
  if (rc) return rc;
  if (base == target) return fail(BSA_ERR_INVALID_ARG, "base and target must not alias");
  const long long total = (long long)n_heads * nb_target * nb_target;
  const long long blocks = std::min<long long>((total + NT - 1) / NT, 1 << 16);
  hipLaunchKernelGGL(threshold_resize_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, base, nb_base,
                     nb_target, total, target);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
