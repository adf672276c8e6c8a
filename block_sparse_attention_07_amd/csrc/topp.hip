// Hybrid top-p block selection with a top-k minimum ("Competition Domains Matter"
// abstract: online top-p over block proxy scores; SCOPE abstract: a fixed top-k
// minimum for over-concentrated rows; ScalingAttention Appendix A, Algorithm 1:
// sort, cumulative sum, cut where it reaches p).
//
// The kept set is an integer decision taken on floating-point sums, so it is
// pinned to one float32 procedure: every operation below is a single IEEE
// float32 operation rounded to nearest, never contracted (this file is built
// with -ffp-contract=off and the arithmetic sits under `fp contract(off)`), the
// sums run sequentially in sorted order, and the exponential is the library's
// own (Cody-Waite reduction with a two-part ln 2, degree-7 Taylor polynomial in
// Horner form, 2^n assembled from exponent bits, 0 below -87).
//
// One workgroup per score row: the row is staged in LDS, bitonic-sorted by
// (score descending, index ascending), the exponentials are summed and scanned
// by one lane in sorted order, and the chosen blocks are OR-ed into LDS words.
#include <cmath>

#include "bsa_internal.h"

#pragma clang fp contract(off)

namespace bsa {
namespace {

constexpr int NT = 256;
constexpr int MAX_N = 4096;

// float32 constants (bit patterns of the nearest float32 values):
// log2(e); 355/512 (n * 355/512 is exact for |n| < 2^15); ln 2 - 355/512; 1/k!.
__device__ __forceinline__ float f32_bits(uint32_t b) { return __uint_as_float(b); }

__device__ float exp_cw(float x) {
#pragma clang fp contract(off)
  if (!(x >= -87.0f)) return 0.0f;
  const float log2e = f32_bits(0x3fb8aa3bu);
  const float ln2_hi = f32_bits(0x3f318000u);
  const float ln2_lo = f32_bits(0xb95e8083u);
  const float t = x * log2e;
  const float n = floorf(t + 0.5f);
  const float hi = n * ln2_hi;
  const float r0 = x - hi;
  const float lo = n * ln2_lo;
  const float r = r0 - lo;
  float p = f32_bits(0x39500d01u);            // 1/7!
  p = p * r; p = p + f32_bits(0x3ab60b61u);   // 1/6!
  p = p * r; p = p + f32_bits(0x3c088889u);   // 1/5!
  p = p * r; p = p + f32_bits(0x3d2aaaabu);   // 1/4!
  p = p * r; p = p + f32_bits(0x3e2aaaabu);   // 1/3!
  p = p * r; p = p + 0.5f;                    // 1/2!
  p = p * r; p = p + 1.0f;                    // 1/1!
  p = p * r; p = p + 1.0f;                    // 1/0!
  const int ni = (int)n;
  const float two_n = __int_as_float((ni + 127) << 23);
  return p * two_n;
}

__device__ __forceinline__ bool before(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(NT) void topp_kernel(const float* __restrict__ scores, int nk, int W,
                                                  float p, int min_blocks,
                                                  uint64_t* __restrict__ mask) {
#pragma clang fp contract(off)
  __shared__ float key[MAX_N];
  __shared__ unsigned short idx[MAX_N];
  __shared__ float ex[MAX_N];
  __shared__ float red[NT];
  __shared__ unsigned long long words[MAX_N / 64];
  __shared__ int k_keep;

  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const float* s = scores + row * (size_t)nk;
  int npad = 1;
  while (npad < nk) npad <<= 1;

  float mx = -INFINITY;
  for (int j = tid; j < npad; j += NT) {
    if (j < nk) {
      const float v = s[j];
      key[j] = v;
      idx[j] = (unsigned short)j;
      mx = fmaxf(mx, v);
    } else {
      key[j] = -INFINITY;
      idx[j] = 0xffff;
    }
  }
  red[tid] = mx;
  for (int w = tid; w < MAX_N / 64; w += NT) words[w] = 0ull;
  __syncthreads();
  for (int st = NT / 2; st > 0; st >>= 1) {
    if (tid < st) red[tid] = fmaxf(red[tid], red[tid + st]);
    __syncthreads();
  }
  const float m = red[0];
  for (int j = tid; j < nk; j += NT) ex[j] = exp_cw(key[j] - m);
  __syncthreads();

  // bitonic sort of (key, idx) into "before" order
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < npad; i += NT) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const float ki = key[i], kj = key[j];
          const int ii = idx[i], ij = idx[j];
          const bool swap = up ? before(kj, ij, ki, ii) : before(ki, ii, kj, ij);
          if (swap) {
            key[i] = kj; key[j] = ki;
            idx[i] = (unsigned short)ij; idx[j] = (unsigned short)ii;
          }
        }
      }
      __syncthreads();
    }
  }

  // exponentials in sorted order (reuse key[])
  for (int r = tid; r < nk; r += NT) key[r] = ex[idx[r]];
  __syncthreads();
  if (tid == 0) {
    float z = 0.0f;
    for (int r = 0; r < nk; ++r) z = z + key[r];
    red[0] = z;
  }
  __syncthreads();
  const float z = red[0];
  for (int r = tid; r < nk; r += NT) key[r] = key[r] / z;
  __syncthreads();
  if (tid == 0) {
    float c = 0.0f;
    int kp = nk;
    for (int r = 0; r < nk; ++r) {
      c = c + key[r];
      if (c >= p) {
        kp = r + 1;
        break;
      }
    }
    const int floor_k = min_blocks < nk ? min_blocks : nk;
    k_keep = kp > floor_k ? kp : floor_k;
  }
  __syncthreads();
  const int kk = k_keep;
  for (int r = tid; r < kk; r += NT) {
    const int b = idx[r];
    atomicOr(&words[b >> 6], 1ull << (b & 63));
  }
  __syncthreads();
  uint64_t* out = mask + row * (size_t)W;
  for (int w = tid; w < W; w += NT) out[w] = words[w];
}

}  // namespace
}  // namespace bsa

extern "C" int mask_from_block_scores_topp(const float* scores, int n_heads, int n_q_blocks,
                                           int n_k_blocks, float p, int min_blocks,
                                           uint64_t* mask_bits, hipStream_t stream) {
  using namespace bsa;
  if (!scores || !mask_bits) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(scores, 4) || !aligned(mask_bits, 8))
    return fail(BSA_ERR_INVALID_ARG, "misaligned pointer argument");
  if (n_heads < 1 || n_q_blocks < 1 || n_k_blocks < 1)
    return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (n_k_blocks > MAX_N)
    return fail(BSA_ERR_UNSUPPORTED, "at most %d key blocks per row (got %d)", MAX_N, n_k_blocks);
  if (!(p > 0.0f && p <= 1.0f)) return fail(BSA_ERR_INVALID_ARG, "p must lie in (0, 1]");
  if (min_blocks < 0) return fail(BSA_ERR_INVALID_ARG, "min_blocks must be >= 0");
  const long long rows = (long long)n_heads * n_q_blocks;
  if (rows > 0x7fffffffLL) return fail(BSA_ERR_INVALID_ARG, "problem too large");
  hipLaunchKernelGGL(topp_kernel, dim3((unsigned)rows), dim3(NT), 0, stream, scores, n_k_blocks,
                     n_words(n_k_blocks), p, min_blocks, mask_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
