// Resolution scaling of block maps (ScalingAttention section 4.3.1, Eq. 7).
//
// A map built at a base block count n_b is resized to n_t blocks by bilinear
// interpolation at (u / s, v / s), s = n_t / n_b, with a ceiling that keeps any
// overlap with an active region.  On a binary region map the ceiling of the
// interpolated value is 1 exactly when a base sample with positive weight is
// active, so the kernels evaluate that rule in integers: along each axis the
// sample is x0 = floor(u n_b / n_t) (clamped to n_b - 1) and the next sample
// enters with positive weight iff u n_b is not a multiple of n_t.
//   * mask_resize: packed region maps; a wave owns one 64-column word of the
//     target for a run of rows: its column samples come from one division per
//     lane, its row samples advance by remainder arithmetic (or, with the
//     head's base map staged in LDS when it fits, come from one division per
//     lane and are broadcast with v_readlane), and each row's word is the
//     ballot of the OR of up to four base bits per lane.
//   * threshold_map_resize: float32 threshold maps; the conservative
//     counterpart of the ceiling is the minimum over the positive-weight
//     samples (NaN ignored), so thresholding and resizing commute.  A thread
//     owns one column for a run of rows, reads and writes coalesced.
#include <algorithm>
#include <cmath>

#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int NT = 256;

struct Axis {
  int a, b;   // samples (b == a when only one has positive weight)
};

// Samples of target index u: x0 = floor(u nb / nt) clamped to nb - 1, and
// x0 + 1 (clamped) when u nb is not a multiple of nt.
__device__ __forceinline__ Axis axis_samples(int u, int nb, int nt) {
  const unsigned long long x = (unsigned long long)u * (unsigned)nb;
  unsigned q, r;
  if (x < (1ull << 32)) {
    q = (unsigned)x / (unsigned)nt;
    r = (unsigned)x - q * (unsigned)nt;
  } else {
    q = (unsigned)(x / (unsigned)nt);
    r = (unsigned)(x % (unsigned)nt);
  }
  const int a = min((int)q, nb - 1);
  return {a, r != 0 ? min((int)q + 1, nb - 1) : a};
}

// Row samples walked incrementally: q = floor(u nb / nt), r = u nb mod nt.
struct RowWalk {
  int q, r;
  __device__ __forceinline__ void start(int u, int nb, int nt) {
    const unsigned long long x = (unsigned long long)u * (unsigned)nb;
    q = (int)(x / (unsigned)nt);
    r = (int)(x % (unsigned)nt);
  }
  __device__ __forceinline__ Axis samples(int nb) const {
    const int a = min(q, nb - 1);
    return {a, r != 0 ? min(q + 1, nb - 1) : a};
  }
  __device__ __forceinline__ void next(int nb, int nt) {
    r += nb;
    while (r >= nt) {
      r -= nt;
      ++q;
    }
  }
};

constexpr int ROWS_PER_WAVE = 64;   // one row's word per lane at the end

__global__ __launch_bounds__(NT) void mask_resize_kernel(const uint64_t* __restrict__ base, int nb, int nt,
                                                         int Wb, int Wt, int n_chunks, long long waves,
                                                         uint64_t* __restrict__ target) {
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  if (gw >= waves) return;
  const int chunk = (int)(gw % n_chunks);
  const long long hw = gw / n_chunks;
  const int w = (int)(hw % Wt);
  const int h = (int)(hw / Wt);
  const int v = 64 * w + lane;
  const bool vin = v < nt;
  const Axis y = axis_samples(vin ? v : 0, nb, nt);
  const int u0 = chunk * ROWS_PER_WAVE, u1 = min(nt, u0 + ROWS_PER_WAVE);
  RowWalk rw;
  rw.start(u0, nb, nt);
  const uint64_t* bh = base + (size_t)h * nb * Wb;
  uint64_t* th = target + (size_t)h * nt * Wt + w;
  // Eight rows at a time: their loads are issued together, so the loop waits
  // for one memory round trip per eight rows rather than per row.
  constexpr int UNROLL = 8;
  const int ya = y.a >> 6, yb = y.b >> 6, sa = y.a & 63, sb = y.b & 63;
  uint64_t mine = 0;
  for (int u = u0; u < u1; u += UNROLL) {
    uint64_t w0[UNROLL], w1[UNROLL], w2[UNROLL], w3[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const Axis x = rw.samples(nb);
      w0[k] = w1[k] = w2[k] = w3[k] = 0;
      if (vin && u + k < u1) {
        const uint64_t* r0 = bh + (size_t)x.a * Wb;
        const uint64_t* r1 = bh + (size_t)x.b * Wb;
        w0[k] = r0[ya];
        w1[k] = r0[yb];
        w2[k] = r1[ya];
        w3[k] = r1[yb];
      }
      rw.next(nb, nt);
    }
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) {
      const bool on = ((w0[k] >> sa) | (w1[k] >> sb) | (w2[k] >> sa) | (w3[k] >> sb)) & 1ull;
      const uint64_t bits = __ballot(on);
      if (lane == u + k - u0) mine = bits;    // lane j keeps row u0 + j
    }
  }
  if (u0 + lane < u1) th[(size_t)(u0 + lane) * Wt] = mine;
}

// The same rule with the head's whole base map staged in LDS (when it fits):
// a workgroup takes RS_ITEMS (word column, 64-row chunk) items of one head,
// lane k holds the row samples of target row u0 + k (taken with v_readlane),
// and every lookup is an LDS read.
constexpr int RS_ITEMS = 16;

__global__ __launch_bounds__(NT) void mask_resize_lds_kernel(const uint64_t* __restrict__ base, int nb, int nt,
                                                             int Wb, int Wt, int items,
                                                             uint64_t* __restrict__ target) {
  extern __shared__ uint64_t bm[];             // [nb][Wb], base map of head h
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const uint64_t* bh = base + (size_t)h * nb * Wb;
  for (int i = tid; i < nb * Wb; i += NT) bm[i] = bh[i];
  __syncthreads();
  for (int it = wave; it < RS_ITEMS; it += NT / 64) {
    const int item = blockIdx.x * RS_ITEMS + it;
    if (item >= items) break;                  // uniform per wave
    const int w = item % Wt, chunk = item / Wt;
    const int v = 64 * w + lane;
    const bool vin = v < nt;
    const Axis y = axis_samples(vin ? v : 0, nb, nt);
    const int u0 = chunk * ROWS_PER_WAVE, u1 = min(nt, u0 + ROWS_PER_WAVE);
    const Axis xs = axis_samples(min(u0 + lane, nt - 1), nb, nt);
    const int ya = y.a >> 6, yb = y.b >> 6, sa = y.a & 63, sb = y.b & 63;
    uint64_t mine = 0;
    for (int k = 0; k < u1 - u0; ++k) {
      const int xa = __builtin_amdgcn_readlane(xs.a, k), xb = __builtin_amdgcn_readlane(xs.b, k);
      const uint64_t* r0 = bm + xa * Wb;
      const uint64_t* r1 = bm + xb * Wb;
      const bool on = vin && ((((r0[ya] >> sa) | (r0[yb] >> sb) | (r1[ya] >> sa) | (r1[yb] >> sb)) & 1ull));
      const uint64_t bits = __ballot(on);
      if (lane == k) mine = bits;
    }
    if (u0 + lane < u1) target[((size_t)h * nt + u0 + lane) * Wt + w] = mine;
  }
}

constexpr int TR_ROWS = 32;   // target rows per workgroup of the threshold resize

// grid (ceil(nt / NT), ceil(nt / TR_ROWS), n_heads): thread = one column.
__global__ __launch_bounds__(NT) void threshold_resize_kernel(const float* __restrict__ base, int nb, int nt,
                                                              float* __restrict__ target) {
  const int v = blockIdx.x * NT + threadIdx.x;
  if (v >= nt) return;
  const int h = blockIdx.z;
  const Axis y = axis_samples(v, nb, nt);
  const int u0 = blockIdx.y * TR_ROWS, u1 = min(nt, u0 + TR_ROWS);
  RowWalk rw;
  rw.start(u0, nb, nt);
  const float* bh = base + (size_t)h * nb * nb;
  float* th = target + (size_t)h * nt * nt + v;
  for (int u = u0; u < u1; ++u) {
    const Axis x = rw.samples(nb);
    const float* r0 = bh + (size_t)x.a * nb;
    const float* r1 = bh + (size_t)x.b * nb;
    th[(size_t)u * nt] = fminf(fminf(r0[y.a], r0[y.b]), fminf(r1[y.a], r1[y.b]));
    rw.next(nb, nt);
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
  const int n_chunks = (nb_target + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
  int dev = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    lds_max = 0;
  const size_t map_bytes = (size_t)nb_base * Wb * sizeof(uint64_t);
  const long long items = (long long)Wt * n_chunks;
  if (map_bytes <= (size_t)lds_max && items <= 0x7fffffffLL && n_heads <= 65535) {
    const unsigned gx = (unsigned)((items + RS_ITEMS - 1) / RS_ITEMS);
    hipLaunchKernelGGL(mask_resize_lds_kernel, dim3(gx, (unsigned)n_heads), dim3(NT), map_bytes, stream, base_bits,
                       nb_base, nb_target, Wb, Wt, (int)items, target_bits);
    BSA_CHECK_HIP(hipGetLastError());
    return ok();
  }
  const long long waves = (long long)n_heads * Wt * n_chunks;
  const long long blocks = (waves + NT / 64 - 1) / (NT / 64);
  if (blocks > 0x7fffffffLL) return fail(BSA_ERR_INVALID_ARG, "problem too large");
  hipLaunchKernelGGL(mask_resize_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, base_bits, nb_base,
                     nb_target, Wb, Wt, n_chunks, waves, target_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}

extern "C" int threshold_map_resize(const float* base, int n_heads, int nb_base, int nb_target,
                                    float* target, hipStream_t stream) {
  using namespace bsa;
  int rc = check_resize(base, target, n_heads, nb_base, nb_target, 4);
  if (rc) return rc;
  if (base == target) return fail(BSA_ERR_INVALID_ARG, "base and target must not alias");
  if (n_heads > 65535 || (nb_target + TR_ROWS - 1) / TR_ROWS > 65535)
    return fail(BSA_ERR_INVALID_ARG, "problem too large");
  const dim3 grid((unsigned)((nb_target + NT - 1) / NT), (unsigned)((nb_target + TR_ROWS - 1) / TR_ROWS),
                  (unsigned)n_heads);
  hipLaunchKernelGGL(threshold_resize_kernel, grid, dim3(NT), 0, stream, base, nb_base, nb_target, target);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
