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
// One workgroup per score row: the row is held in registers (E values per lane),
// bitonic-sorted by (score descending, index ascending) mostly inside threads and
// waves, the exponentials are summed and scanned by one lane in sorted order,
// and the chosen blocks are OR-ed into LDS words.
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

// Bitonic sort of npad = E * NT (key, index) pairs into "before" order, with
// thread t holding positions E t .. E t + E - 1 in registers.  Partners closer
// than E positions are exchanged inside the thread, partners within the wave by
// lane shuffles, and only the few stages whose partner lies in another wave go
// through LDS (lk / li, with barriers).
template <int E>
__device__ void bitonic_sort(float (&k)[E], int (&ix)[E], float* lk, unsigned short* li, int tid) {
  constexpr int npad = E * NT;
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int f = e ^ stride;
          if (f > e) {
            const bool up = ((E * tid + e) & size) == 0;
            const bool sw = up ? before(k[f], ix[f], k[e], ix[e]) : before(k[e], ix[e], k[f], ix[f]);
            if (sw) {
              const float tk = k[e]; k[e] = k[f]; k[f] = tk;
              const int ti = ix[e]; ix[e] = ix[f]; ix[f] = ti;
            }
          }
        }
      } else {
        float pk[E];
        int pi[E];
        if (stride < E * 64) {
          const int ld = stride / E;                 // lane distance inside the wave
#pragma unroll
          for (int e = 0; e < E; ++e) {
            pk[e] = __shfl_xor(k[e], ld);
            pi[e] = __shfl_xor(ix[e], ld);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            lk[E * tid + e] = k[e];
            li[E * tid + e] = (unsigned short)ix[e];
          }
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) {
            pk[e] = lk[(E * tid + e) ^ stride];
            pi[e] = li[(E * tid + e) ^ stride];
          }
          __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int pos = E * tid + e;
          const bool lower = (pos & stride) == 0, up = (pos & size) == 0;
          const bool mine_first = before(k[e], ix[e], pk[e], pi[e]);
          const bool keep_mine = (lower == up) ? mine_first : !mine_first;
          if (!keep_mine) {
            k[e] = pk[e];
            ix[e] = pi[e];
          }
        }
      }
    }
  }
}

template <int E>
__global__ __launch_bounds__(NT) void topp_kernel(const float* __restrict__ scores, int nk, int W,
                                                  float p, int min_blocks,
                                                  uint64_t* __restrict__ mask) {
#pragma clang fp contract(off)
  constexpr int npad = E * NT;
  __shared__ __attribute__((aligned(16))) float key[npad];
  __shared__ unsigned short idx[npad];
  __shared__ float ex[npad];
  __shared__ float red[NT];
  __shared__ unsigned long long words[MAX_N / 64];
  __shared__ int k_keep;

  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const float* s = scores + row * (size_t)nk;

  float k[E];
  int ix[E];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = E * tid + e;
    if (j < nk) {
      k[e] = s[j];
      ix[e] = j;
      mx = fmaxf(mx, k[e]);
    } else {
      k[e] = -INFINITY;
      ix[e] = 0xffff;
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
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (E * tid + e < nk) ex[E * tid + e] = exp_cw(k[e] - m);

  bitonic_sort<E>(k, ix, key, idx, tid);
  __syncthreads();                       // ex[] complete, LDS exchange buffers free

  // exponentials in sorted order
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int r = E * tid + e;
    idx[r] = (unsigned short)ix[e];
    if (r < nk) key[r] = ex[ix[e]];
  }
  __syncthreads();
  // The two sums are sequential by definition; one lane runs each, reading four
  // values per LDS load so the loads run ahead of the dependent adds.
  const float4* key4 = reinterpret_cast<const float4*>(key);
  if (tid == 0) {
    float z = 0.0f;
    int r = 0;
#pragma unroll 4
    for (; r + 4 <= nk; r += 4) {
      const float4 v = key4[r >> 2];
      z = z + v.x; z = z + v.y; z = z + v.z; z = z + v.w;
    }
    for (; r < nk; ++r) z = z + key[r];
    red[0] = z;
  }
  __syncthreads();
  const float z = red[0];
  for (int r = tid; r < nk; r += NT) key[r] = key[r] / z;
  __syncthreads();
  if (tid == 0) {
    float c = 0.0f;
    int kp = nk;
    int r = 0;
    // kp keeps the first crossing; the loop stops at the end of the group of
    // four where it happens
    for (; r + 4 <= nk && kp == nk; r += 4) {
      const float4 v = key4[r >> 2];
      c = c + v.x; kp = (kp == nk && c >= p) ? r + 1 : kp;
      c = c + v.y; kp = (kp == nk && c >= p) ? r + 2 : kp;
      c = c + v.z; kp = (kp == nk && c >= p) ? r + 3 : kp;
      c = c + v.w; kp = (kp == nk && c >= p) ? r + 4 : kp;
    }
    for (; r < nk && kp == nk; ++r) {
      c = c + key[r];
      if (c >= p) kp = r + 1;
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
  const dim3 grid((unsigned)rows), block(NT);
  const int W = n_words(n_k_blocks);
  if (n_k_blocks <= NT)
    hipLaunchKernelGGL(topp_kernel<1>, grid, block, 0, stream, scores, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 2 * NT)
    hipLaunchKernelGGL(topp_kernel<2>, grid, block, 0, stream, scores, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 4 * NT)
    hipLaunchKernelGGL(topp_kernel<4>, grid, block, 0, stream, scores, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 8 * NT)
    hipLaunchKernelGGL(topp_kernel<8>, grid, block, 0, stream, scores, n_k_blocks, W, p, min_blocks, mask_bits);
  else
    hipLaunchKernelGGL(topp_kernel<16>, grid, block, 0, stream, scores, n_k_blocks, W, p, min_blocks, mask_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
