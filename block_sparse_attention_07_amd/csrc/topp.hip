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
// Horner form, 2^n assembled from exponent bits, 0 below -87).  Scores are read
// through one clamp, NaN to -FLT_MAX and +-inf to +-FLT_MAX, before anything
// else (the pages only consider finite scores; this makes the result defined,
// and the same for every row length, when some are not).
//
// Rows of up to 2048 blocks: one wave per row, the row held as 32-bit keys in
// registers and sorted inside the wave by a bitonic network in mirror form (no
// comparator needs a direction); rows of 1025 .. 1536 blocks sort their first
// 1024 blocks and the rest apart and merge the two (topp_wave2_kernel), which
// spares most of the padding to 2048.  The mask words are built by ballots from
// the keys in index order.  Longer rows: one workgroup per row (topp_kernel),
// sorted mostly inside threads and waves, the chosen blocks OR-ed into LDS
// words.  Either way the exponentials are summed and scanned by one lane in
// sorted order.
#include <cfloat>
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

// Non-finite scores: NaN reads as the lowest finite score and +-inf as the
// largest finite magnitudes (maxNum / minNum drop a NaN operand), so every
// kernel width sees a total order and the same sums.
__device__ __forceinline__ float clamp_score(float x) { return fminf(fmaxf(x, -FLT_MAX), FLT_MAX); }

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

// Number of leading values of v[0..n) whose running fp32 sum, added left to
// right, first reaches p (n if it never does).  The values are non-negative,
// so the running sum never decreases: a group of four whose last partial sum is
// below p holds no crossing, and only the group that reaches p is examined term
// by term.  The additions are the same, in the same order, as one sum per step.
__device__ __forceinline__ int first_crossing(const float* v, int n, float p) {
  const float4* v4 = reinterpret_cast<const float4*>(v);
  float c = 0.0f;
  int r = 0;
  for (; r + 4 <= n; r += 4) {
    const float4 x = v4[r >> 2];
    const float c1 = c + x.x;
    const float c2 = c1 + x.y;
    const float c3 = c2 + x.z;
    const float c4 = c3 + x.w;
    if (c4 >= p) return c1 >= p ? r + 1 : (c2 >= p ? r + 2 : (c3 >= p ? r + 3 : r + 4));
    c = c4;
  }
  for (; r < n; ++r) {
    c = c + v[r];
    if (c >= p) return r + 1;
  }
  return n;
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
      k[e] = clamp_score(s[j]);
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
    const int kp = first_crossing(key, nk, p);
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


// One wave per row.  Block j of the row is loaded by lane j % 64 as element
// j / 64, so the loads are coalesced and that copy of the keys is already laid
// out as the row's mask words (word w = the bits of element w over the lanes).
// A key is the score's bits mapped to an order-preserving unsigned 32-bit
// integer (after -0 -> +0, so equal scores stay equal); rows past the end hold
// key 0, which sorts after every real key.  The sort leaves equal scores in no
// particular order, which changes nothing in the sums: equal scores have equal
// exponentials, so the normaliser and the cumulative scan (run exactly as in
// topp_kernel) see the same sequence of values as in (score descending, index
// ascending) order.  The kept set is that order's first k blocks: every block
// whose key exceeds the k-th key, and the lowest-index blocks whose key equals
// it, as many as are still needed.  Each wave has its own LDS region for its
// row; the sequential sums of a workgroup's rows run side by side on lanes of
// one wave (topp_count), between workgroup barriers.  Waves past the last row
// work on row 0 and write nothing.
constexpr int TW_WAVES = 4;

__device__ __forceinline__ uint32_t ord_bits(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float ord_float(uint32_t o) {
  return __uint_as_float(o ^ ((o >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}

// Exchange with lane ^ D (D a power of two below 64), in registers:
//  * D = 1, 2: DPP quad permutation;
//  * D = 4, 8: DPP row shifts; lanes whose D bit is clear take the lane D above,
//    the others the lane D below, both inside the same 16-lane row;
//  * D = 16, 32: the permlane swaps, which exchange the two halves of every
//    32- or 64-lane group.  Called with the same value twice, one result holds
//    the lane's own value and the other its partner's.
template <int D>
__device__ __forceinline__ uint32_t xlane32(uint32_t v) {
  if constexpr (D == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  } else if constexpr (D == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  } else if constexpr (D == 4 || D == 8) {
    const uint32_t up = __builtin_amdgcn_mov_dpp(v, 0x100 + D, 0xF, 0xF, true);   // row_shl: lane + D
    const uint32_t dn = __builtin_amdgcn_mov_dpp(v, 0x110 + D, 0xF, 0xF, true);   // row_shr: lane - D
    return (threadIdx.x & D) ? dn : up;
  } else if constexpr (D == 16) {
    const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? sw[0] : sw[1];
  } else {
    static_assert(D == 32, "lane distance");
    const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? sw[0] : sw[1];
  }
}

// Value of lane ^ (2D - 1) (D a power of two below 64): the lane mirrored
// inside its group of 2D lanes.
template <int D>
__device__ __forceinline__ uint32_t xmirror32(uint32_t v) {
  if constexpr (D == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);          // quad_perm 1,0,3,2
  } else if constexpr (D == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x1B, 0xF, 0xF, true);          // quad_perm 3,2,1,0
  } else if constexpr (D == 4) {
    return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);         // row_half_mirror
  } else if constexpr (D == 8) {
    return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true);         // row_mirror
  } else if constexpr (D == 16) {
    return __builtin_amdgcn_mov_dpp(xlane32<16>(v), 0x140, 0xF, 0xF, true);
  } else {
    static_assert(D == 32, "lane distance");
    return __builtin_amdgcn_mov_dpp(xlane32<16>(xlane32<32>(v)), 0x140, 0xF, 0xF, true);
  }
}

// Bitonic merge network in mirror form (every comparator puts the larger key at
// the lower position, so no stage needs a direction): the first stage of the
// merge of size SIZE pairs position i of each SIZE-block with position
// SIZE - 1 - i, the following stages pair i with i + STRIDE.  Row element
// EW * lane + e is a[e] of lane `lane`.
template <int EW, int SIZE, int STRIDE, bool MIRROR>
__device__ __forceinline__ void merge_stage(uint32_t (&a)[EW], int lane) {
  if constexpr (SIZE <= EW && MIRROR) {
#pragma unroll
    for (int e = 0; e < EW; ++e)
      if ((e & (SIZE / 2)) == 0) {
        const int f = e ^ (SIZE - 1);
        const uint32_t x = a[e], y = a[f];
        a[e] = x > y ? x : y;
        a[f] = x > y ? y : x;
      }
  } else if constexpr (STRIDE < EW && !MIRROR) {
#pragma unroll
    for (int e = 0; e < EW; ++e)
      if ((e & STRIDE) == 0) {
        const int f = e | STRIDE;
        const uint32_t x = a[e], y = a[f];
        a[e] = x > y ? x : y;
        a[f] = x > y ? y : x;
      }
  } else {
    // across lanes: the partner lane is lane ^ (2D - 1) (mirror) or lane ^ D
    constexpr int D = MIRROR ? SIZE / (2 * EW) : STRIDE / EW;
    const bool lower = (lane & D) == 0;
    uint32_t y[EW];
#pragma unroll
    for (int e = 0; e < EW; ++e) y[e] = MIRROR ? xmirror32<D>(a[EW - 1 - e]) : xlane32<D>(a[e]);
#pragma unroll
    for (int e = 0; e < EW; ++e) {
      const bool take_mine = (a[e] > y[e]) == lower;
      a[e] = take_mine ? a[e] : y[e];
    }
  }
  if constexpr (MIRROR) {
    if constexpr (SIZE > 2) merge_stage<EW, SIZE, SIZE / 4, false>(a, lane);
  } else if constexpr (STRIDE > 1) {
    merge_stage<EW, SIZE, STRIDE / 2, false>(a, lane);
  }
}

// Sorts the 64 * EW keys of a wave in descending order.
template <int EW, int SIZE = 2>
__device__ __forceinline__ void wave_sort_desc(uint32_t (&a)[EW], int lane) {
  merge_stage<EW, SIZE, SIZE / 2, true>(a, lane);
  if constexpr (SIZE < 64 * EW) wave_sort_desc<EW, SIZE * 2>(a, lane);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0)
  asm volatile("" ::: "memory");
}

// buf[w] holds row w's keys in sorted order (as uint32) at positions 0 .. nk-1.
// Each wave turns its row into exponentials; lanes 0 .. TW_WAVES-1 of wave 0
// then run the sequential sums of all rows side by side.
template <int NS>
__device__ __forceinline__ int topp_count(float (*buf)[NS], float* zs, int* ks, int nk, float m, float p,
                                          int min_blocks, int lane, int wv) {
#pragma clang fp contract(off)
  float* b = buf[wv];
  const uint32_t* bu = reinterpret_cast<const uint32_t*>(b);
  for (int r = lane; r < nk; r += 64) b[r] = exp_cw(ord_float(bu[r]) - m);
  __syncthreads();
  if (wv == 0 && lane < TW_WAVES) {
    const float* bl = buf[lane];
    const float4* b4 = reinterpret_cast<const float4*>(bl);
    float z = 0.0f;
    int r = 0;
#pragma unroll 4
    for (; r + 4 <= nk; r += 4) {
      const float4 v = b4[r >> 2];
      z = z + v.x; z = z + v.y; z = z + v.z; z = z + v.w;
    }
    for (; r < nk; ++r) z = z + bl[r];
    zs[lane] = z;
  }
  __syncthreads();
  const float z = zs[wv];
  for (int r = lane; r < nk; r += 64) b[r] = b[r] / z;
  __syncthreads();
  if (wv == 0 && lane < TW_WAVES) {
    const int kp = first_crossing(buf[lane], nk, p);
    const int floor_k = min_blocks < nk ? min_blocks : nk;
    ks[lane] = kp > floor_k ? kp : floor_k;
  }
  __syncthreads();
  return ks[wv];
}

// Writes the row's W mask words (W <= NW).  o[w] is the key of block 64 w + lane,
// which word w holds in bit `lane`.  Kept: every block whose key exceeds kstar,
// and the `need` lowest-index blocks whose key equals it.
template <int NW>
__device__ __forceinline__ void emit_mask(const uint32_t (&o)[NW], int nk, int W, uint32_t kstar, int need,
                                          uint64_t* __restrict__ out, int lane) {
  const uint64_t below = (1ull << lane) - 1ull;
  int before = 0;                                     // tied blocks at lower indices
  uint64_t mine = 0;                                  // word `lane` of the row
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < W) {
      const bool real = 64 * w + lane < nk;
      const uint64_t gt = __ballot(real && o[w] > kstar);
      const uint64_t eq = __ballot(real && o[w] == kstar);
      const bool tk = ((eq >> lane) & 1ull) && before + __popcll(eq & below) < need;
      const uint64_t word = gt | __ballot(tk);
      before += __popcll(eq);
      if (lane == w) mine = word;
    }
  }
  if (lane < W) out[lane] = mine;
}

// Rows of at most 64 * EW blocks; the sort leaves sorted position EW l + e in
// element e of lane l.
template <int EW>
__global__ __launch_bounds__(64 * TW_WAVES) void topp_wave_kernel(const float* __restrict__ scores,
                                                                   int n_rows, int nk, int W, float p,
                                                                   int min_blocks,
                                                                   uint64_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) float buf[TW_WAVES][64 * EW];
  __shared__ float zs[TW_WAVES];
  __shared__ int ks[TW_WAVES];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * TW_WAVES + wv;
  const bool valid = row < n_rows;
  const float* s = scores + (valid ? row : 0ll) * (long long)nk;
  float* b = buf[wv];

  uint32_t a[EW], o[EW];                              // o: the keys in index order
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EW; ++e) {
    const int j = 64 * e + lane;
    o[e] = 0u;
    if (j < nk) {
      const float v = clamp_score(s[j]);
      mx = fmaxf(mx, v);
      o[e] = ord_bits(v);
    }
    a[e] = o[e];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));

  wave_sort_desc<EW>(a, lane);

  uint32_t* bu = reinterpret_cast<uint32_t*>(b);
#pragma unroll
  for (int e = 0; e < EW; ++e)
    if (EW * lane + e < nk) bu[EW * lane + e] = a[e];
  wave_lds_sync();
  const int kk = topp_count(buf, zs, ks, nk, mx, p, min_blocks, lane, wv);
  // the kk-th key of the sorted row, and how many keys exceed it
  const int pos = kk - 1;
  uint32_t cand = 0u;
#pragma unroll
  for (int e = 0; e < EW; ++e) cand = (e == pos % EW) ? a[e] : cand;
  const uint32_t kstar = __shfl(cand, pos / EW);
  int n_gt = 0;
#pragma unroll
  for (int e = 0; e < EW; ++e) n_gt += __popcll(__ballot(a[e] > kstar));
  if (valid) emit_mask<EW>(o, nk, W, kstar, kk - n_gt, mask + row * (long long)W, lane);
}

// Rows of 1025 .. 64 * (16 + EW2) blocks: blocks 0 .. 1023 (part A, 16 per lane)
// and the rest (part B, EW2 per lane) are sorted separately, part B is spread
// to 16 per lane through LDS (zero keys after its end), and one merge joins
// them: position i of A faces position 1023 - i of B (lane ^ 63, element
// 15 - e), A keeps the larger key and B the smaller, then each part is finished
// by its own half-cleaners.  Sorted position r is then element r % 16 of lane
// (r % 1024) / 16 of A for r < 1024 and of B otherwise.
// Six waves per SIMD (at most 80 registers, a few of them spilled) and a row
// buffer of only nk's bound (20 KB per workgroup at up to 1280 blocks) measure
// faster than five waves without spills: the sequential scans are latency.
template <int EW2>
__global__ __launch_bounds__(64 * TW_WAVES, 6) void topp_wave2_kernel(const float* __restrict__ scores,
                                                                    int n_rows, int nk, int W, float p,
                                                                    int min_blocks,
                                                                    uint64_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) float buf[TW_WAVES][EW2 == 4 ? 1280 : 1536];
  __shared__ float zs[TW_WAVES];
  __shared__ int ks[TW_WAVES];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * TW_WAVES + wv;
  const bool valid = row < n_rows;
  const float* s = scores + (valid ? row : 0ll) * (long long)nk;
  float* b = buf[wv];
  uint32_t* bu = reinterpret_cast<uint32_t*>(b);

  uint32_t a[16], c2[EW2];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float v = clamp_score(s[64 * e + lane]);    // blocks 0 .. 1023 all exist
    mx = fmaxf(mx, v);
    a[e] = ord_bits(v);
  }
#pragma unroll
  for (int e = 0; e < EW2; ++e) {
    const int j = 1024 + 64 * e + lane;
    c2[e] = 0u;
    if (j < nk) {
      const float v = clamp_score(s[j]);
      mx = fmaxf(mx, v);
      c2[e] = ord_bits(v);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));

  wave_sort_desc<16>(a, lane);
  wave_sort_desc<EW2>(c2, lane);
#pragma unroll
  for (int e = 0; e < EW2; ++e) bu[EW2 * lane + e] = c2[e];
  wave_lds_sync();
  uint32_t c[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) c[e] = 16 * lane + e < 64 * EW2 ? bu[16 * lane + e] : 0u;
  wave_lds_sync();
  // a[e] and c[15 - e] face each other's partner-lane copies
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t ya = xmirror32<32>(c[15 - e]);
    const uint32_t yc = xmirror32<32>(a[e]);
    a[e] = a[e] > ya ? a[e] : ya;
    c[15 - e] = c[15 - e] > yc ? yc : c[15 - e];
  }
  merge_stage<16, 2048, 512, false>(a, lane);
  merge_stage<16, 2048, 512, false>(c, lane);

#pragma unroll
  for (int e = 0; e < 16; ++e) {
    bu[16 * lane + e] = a[e];
    if (1024 + 16 * lane + e < nk) bu[1024 + 16 * lane + e] = c[e];
  }
  wave_lds_sync();
  const int kk = topp_count(buf, zs, ks, nk, mx, p, min_blocks, lane, wv);
  const int pos = kk - 1;
  uint32_t cand = 0u;
#pragma unroll
  for (int e = 0; e < 16; ++e) cand = (e == pos % 16) ? (pos < 1024 ? a[e] : c[e]) : cand;
  const uint32_t kstar = __shfl(cand, (pos % 1024) / 16);
  int n_gt = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) n_gt += __popcll(__ballot(a[e] > kstar)) + __popcll(__ballot(c[e] > kstar));
  // the keys again in index order (coalesced; keeping them through the sort
  // costs more registers than the two-part sort leaves)
  uint32_t o[16 + EW2];
#pragma unroll
  for (int w = 0; w < 16 + EW2; ++w) o[w] = 64 * w + lane < nk ? ord_bits(clamp_score(s[64 * w + lane])) : 0u;
  if (valid) emit_mask<16 + EW2>(o, nk, W, kstar, kk - n_gt, mask + row * (long long)W, lane);
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
  const dim3 wgrid((unsigned)((rows + TW_WAVES - 1) / TW_WAVES)), wblock(64 * TW_WAVES);
  if (n_k_blocks <= 64)
    hipLaunchKernelGGL(topp_wave_kernel<1>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 128)
    hipLaunchKernelGGL(topp_wave_kernel<2>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 256)
    hipLaunchKernelGGL(topp_wave_kernel<4>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 512)
    hipLaunchKernelGGL(topp_wave_kernel<8>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 1024)
    hipLaunchKernelGGL(topp_wave_kernel<16>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 1280)
    hipLaunchKernelGGL(topp_wave2_kernel<4>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 1536)
    hipLaunchKernelGGL(topp_wave2_kernel<8>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else if (n_k_blocks <= 2048)
    hipLaunchKernelGGL(topp_wave_kernel<32>, wgrid, wblock, 0, stream, scores, (int)rows, n_k_blocks, W, p, min_blocks, mask_bits);
  else
    hipLaunchKernelGGL(topp_kernel<16>, grid, block, 0, stream, scores, n_k_blocks, W, p, min_blocks, mask_bits);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}
