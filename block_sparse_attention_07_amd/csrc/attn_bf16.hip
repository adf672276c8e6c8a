// Block-sparse attention forward, bf16 inputs, bf16 MFMA, fp32 online softmax.
//
// ScalingAttention, section 4.3.2 (CRM kernel) and Appendix E (Algorithm 2): a
// FlashAttention forward whose dense key-block loop is replaced by a walk over
// the set bits of the query block's packed row mask; kept 64x64 tiles are
// computed densely, all other tiles are skipped without touching their K/V.
//
// gfx950 mapping (one workgroup of 4 waves per (head, query block)):
//  * wave w owns query rows 32*(w&1) .. +31 and key half 32*(w>>1) .. +31 of every
//    kept tile, so each wave keeps its own running max / sum and output
//    accumulator; the two key halves are merged once at the end.
//  * S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16 with K (A operand) from LDS and
//    Q^T (B operand) held in registers for the whole row.  The accumulator gives
//    lane l the logits of query row l%32 for 16 keys, so the row max and row sum
//    are lane-local plus one exchange with lane l^32.
//  * The same 16 probabilities, rounded to bf16, are exactly the B operand of
//    O^T += V^T P^T, provided the A operand (V^T) pairs each k-slot with the key
//    the accumulator register held: four consecutive keys at one head-dim
//    column per half operand.  V stays row-major in LDS and that operand is read
//    with ds_read_b64_tr_b16, the gfx950 LDS transpose load: in each group of 16
//    lanes, lanes 4r..4r+3 point at four 4-column pieces of key row base+r, and
//    every lane receives the four keys at its own column.
//  * K and V tiles are both fetched with the same contiguous pattern (each wave
//    instruction reads 1 KB of consecutive rows) and written to LDS with 16-byte
//    stores; no register shuffling of V is needed.
//  * Kept K/V tiles stream through a 2-stage LDS ring: the next tile's global
//    loads are issued before the current tile's math and written to the other
//    stage after it, with one barrier per tile.
//  * The row's kept-block list is decoded once per 2048 blocks by wave 0: one mask
//    word per lane, popcount, and a ballot-based exclusive prefix (one ballot per
//    bit of the count) give every lane its write offset into an LDS list.
//  * Softmax rescaling is lazy: the running max used for exponentials only moves
//    when a tile's max exceeds it by more than 8 (a factor 256), which keeps every
//    probability <= 256 and leaves the result exact up to rounding.
#include <cmath>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BLK = 64;
constexpr int NT = 256;
constexpr int LIST_CAP = 2048;
constexpr int CHUNK_WORDS = LIST_CAP / 64;
constexpr int PAD = 16;       // bf16 elements of padding per LDS tile row
constexpr float RESCALE_SLACK = 8.0f;
// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family GPUs:
// 32-bit data format, so the per-access range check against num_records applies.
constexpr int BUFFER_DWORD3 = 0x00020000;

template <int D>
struct __attribute__((aligned(16))) Tiles {
  u16 k[2][BLK][D + PAD];     // K tile, row-major
  u16 v[2][BLK][D + PAD];     // V tile, row-major
};

template <int D>
struct __attribute__((aligned(16))) Merge {
  float o[2][D / 2][64];      // [query-row half][accumulator register][lane]
  float m[2][32];
  float l[2][32];
};

template <int D>
union __attribute__((aligned(16))) Smem {
  Tiles<D> t;
  Merge<D> mg;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read: see the file comment for the lane mapping.
__device__ __forceinline__ s16x4 lds_read_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(p));
}

template <int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ order, int n_heads, int N,
    int nb, int W, float c, u16* __restrict__ O) {
  constexpr int CPR = D / 8;             // 16-byte chunks per token row
  constexpr int KCH = BLK * CPR / NT;    // 16-byte chunks per thread, for K and for V
  constexpr int NDB = D / 32;            // 32-wide output column blocks
  constexpr int NKS = D / 16;            // k-steps of the QK^T contraction

  __shared__ Smem<D> sm;
  __shared__ u16 list[LIST_CAP];
  __shared__ int nlist;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rh = wave & 1;
  const int kh = wave >> 1;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  int row_id = blockIdx.x;
  if (order) {
    row_id = order[blockIdx.x];
    if (row_id < 0 || row_id >= n_heads * nb) return;
  }
  const int h = row_id / nb;
  const int u = row_id - h * nb;
  const size_t head_off = (size_t)h * N * D;
  const u16* Qh = Q + head_off;
  const u16* Kh = K + head_off;
  const u16* Vh = V + head_off;
  const uint64_t* mrow = mask + ((size_t)h * nb + u) * W;

  // Q^T fragments (B operand): lane holds Q[row][16ks + 8g .. +7] of its query row.
  bf16x8 qf[NKS];
  {
    // Rows past the sequence end read the last real row (always in bounds) and
    // are zeroed by a select on the loaded value.
    const int qrow = BLK * u + 32 * rh + r32;
    const bool qvalid = qrow < N;
    const int qsrc = qvalid ? qrow : N - 1;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 x = *reinterpret_cast<const uint4*>(Qh + (size_t)qsrc * D + 16 * ks + 8 * g);
      if (!qvalid) x = make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  // Running max in the exp2 domain.  It starts at a large finite value instead
  // of -inf so a tile whose keys are all masked for this wave yields
  // exp2(-inf) = 0 everywhere without a special case.
  float m_run = -1.0e30f;
  float l_part = 0.f;

  // Register staging for the tiles in flight (vector values, so they stay in
  // VGPRs): chunk r of this thread in dwords 4r..4r+3.
  static_assert(KCH <= 4, "staging holds at most four 16-byte chunks per tensor");
  struct Stage {
    u32x16 k, v;
  };
  Stage st = {};

  // Tiles are read with raw buffer loads: one descriptor per head, a scalar
  // byte offset for the tile and per-thread byte offsets fixed for the whole
  // row (chunk tid + 256 r of the tile: every wave instruction covers 1 KB of
  // consecutive bytes).  The descriptor's range check returns zeros for rows
  // at or past the sequence end (the ragged last block), which are masked out
  // of the softmax.
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(Kh), 0, (int)head_bytes, BUFFER_DWORD3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(Vh), 0, (int)head_bytes, BUFFER_DWORD3);

  auto gload = [&](int kvb, int vvb) {
    const int ktile_off = kvb * BLK * D * 2;
    const int vtile_off = vvb * BLK * D * 2;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int off = (tid + NT * r) * 16;
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(krs, off, ktile_off, 0);
      const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, vtile_off, 0);
      st.k[4 * r] = x[0]; st.k[4 * r + 1] = x[1]; st.k[4 * r + 2] = x[2]; st.k[4 * r + 3] = x[3];
      st.v[4 * r] = y[0]; st.v[4 * r + 1] = y[1]; st.v[4 * r + 2] = y[2]; st.v[4 * r + 3] = y[3];
    }
  };

  auto sstore_k = [&](int kbuf) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ch = tid + NT * r;
      *reinterpret_cast<uint4*>(&sm.t.k[kbuf][ch / CPR][(ch % CPR) * 8]) =
          make_uint4(st.k[4 * r], st.k[4 * r + 1], st.k[4 * r + 2], st.k[4 * r + 3]);
    }
  };
  auto sstore_v = [&](int vbuf) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int ch = tid + NT * r;
      *reinterpret_cast<uint4*>(&sm.t.v[vbuf][ch / CPR][(ch % CPR) * 8]) =
          make_uint4(st.v[4 * r], st.v[4 * r + 1], st.v[4 * r + 2], st.v[4 * r + 3]);
    }
  };

  // Per-lane pieces of the V^T operand: key row 4*g + (lane%16)/4 (+8 for the
  // second half, +16 per k-step, +32*kh per key half) and column
  // 16*((lane%32)/16) + 4*(lane%4) (+32 per output column block).
  const int p0 = 32 * kh;         // first tile position of this wave's key half
  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane & 31) >> 4) + 4 * (lane & 3);

  // One pipeline step for this wave: online softmax of S (tile vb, already in
  // registers), the QK^T MFMAs of the next tile from K stage kbuf (returned),
  // and O^T += V^T P^T from V stage vbuf.  The next tile's MFMAs do not depend on
  // the softmax, so they are issued in the same straight-line block as the
  // exponentials and interleaved with them (one MFMA, then a few VALU ops).
  // s[i] is the logit of query row r32 for tile position p0 + 8*(i/4) + 4*g + i%4.
  auto step = [&](f32x16 s, int vb, int kbuf, int vbuf, bool may_be_ragged) {
    if (may_be_ragged) {
      const int hi = N - vb * BLK;   // tile positions >= hi lie past the sequence end
      if (hi < p0 + 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (p0 + 8 * (i >> 2) + 4 * g + (i & 3) >= hi) s[i] = -INFINITY;
      }
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(s[0], s[1]), __builtin_fmaxf(s[2], s[3]));
#pragma unroll
    for (int i = 4; i < 16; i += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[i], s[i + 1]));
    {
      // lanes l and l^32 hold the two 16-key halves of the same query row
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mt = mx * c;       // -inf when every key of this half is masked
    if (__any(mt > m_run + RESCALE_SLACK)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_run = mn;
    }
    // --- straight-line block: next tile's QK^T interleaved with this tile's exp2
    f32x16 sn;
#pragma unroll
    for (int i = 0; i < 16; ++i) sn[i] = 0.f;
    float p[16];
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.t.k[kbuf][p0 + r32][16 * ks + 8 * g]);
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sn, 0, 0, 0);
      if (2 * ks < 16) {
        const int i = 2 * ks;
        p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m_run));
        p[i + 1] = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -m_run));
        ls0 += p[i];
        ls1 += p[i + 1];
      }
    }
#pragma unroll
    for (int i = 2 * NKS; i < 16; i += 2) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m_run));
      p[i + 1] = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -m_run));
      ls0 += p[i];
      ls1 += p[i + 1];
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // the K operand read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU ops
    }
    l_part += ls0 + ls1;
    bf16x8 pb0, pb1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pb0[j] = (__bf16)p[j];
      pb1[j] = (__bf16)p[8 + j];
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int s0 = 0; s0 < 2; ++s0) {
        const u16* base = &sm.t.v[vbuf][p0 + 16 * s0 + tr_row][32 * db + tr_col];
        const s16x4 lo = lds_read_tr16(base);
        const s16x4 hi2 = lds_read_tr16(base + 8 * (D + PAD));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, s0 ? pb1 : pb0, o[db], 0, 0, 0);
      }
    }
    return sn;
  };

  // S^T of the first tile of a list (no softmax work to overlap with).
  auto qk = [&](int kbuf) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.t.k[kbuf][p0 + r32][16 * ks + 8 * g]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
    }
    return s;
  };

  const int tail_bits = nb & 63;
  const uint64_t lastmask = tail_bits ? ((1ull << tail_bits) - 1ull) : ~0ull;
  const uint64_t lanes_below = (1ull << lane) - 1ull;

  for (int w0 = 0; w0 < W; w0 += CHUNK_WORDS) {
    __syncthreads();   // every wave is done with the previous chunk's list
    if (wave == 0) {
      const int wi = w0 + lane;
      uint64_t word = 0;
      if (lane < CHUNK_WORDS && wi < W) {
        word = mrow[wi];
        if (wi == W - 1) word &= lastmask;
      }
      const int cnt = __popcll(word);
      int pre = 0, tot = 0;
#pragma unroll
      for (int b = 0; b < 7; ++b) {
        const uint64_t bal = __ballot((cnt >> b) & 1);
        pre += __popcll(bal & lanes_below) << b;
        tot += __popcll(bal) << b;
      }
      const int base = 64 * wi;
      while (word) {
        list[pre++] = (u16)(base + __ffsll((unsigned long long)word) - 1);
        word &= word - 1ull;
      }
      if (lane == 0) nlist = tot;
    }
    __syncthreads();
    const int n = nlist;
    if (n == 0) continue;
    // Software pipeline with K one tile ahead of V.  At the top of step t the K
    // stage (t+1)&1 holds K(t+1), the V stage t&1 holds V(t), and S(t) is in
    // registers.  Step t issues the loads of K(t+2) and V(t+1), runs the QK^T
    // MFMAs of tile t+1 next to the softmax of tile t (independent work the
    // scheduler can interleave), then PV of tile t, and stores K(t+2), V(t+1)
    // into the stages just freed.  Past the end of the list the last tile is
    // used again (loads stay unconditional; the extra S is discarded).
    auto tile = [&](int t) { return __builtin_amdgcn_readfirstlane(list[min(t, n - 1)]); };
    gload(tile(0), tile(0));
    sstore_k(0);
    sstore_v(0);
    __syncthreads();
    gload(tile(1), tile(1));
    f32x16 s_cur = qk(0);
    sstore_k(1);
    __syncthreads();
    // only the last block of the sequence can be ragged, and it is always the
    // last entry of an ascending list
    for (int t = 0; t < n; ++t) {
      gload(tile(t + 2), tile(t + 1));
      s_cur = step(s_cur, tile(t), (t + 1) & 1, t & 1, t == n - 1);
      sstore_k(t & 1);
      sstore_v((t + 1) & 1);
      __syncthreads();
    }
  }

  // Merge the two key halves of each query-row half and write the output.
  __syncthreads();
  const float l_row = l_part + __shfl_xor(l_part, 32);
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.mg.o[rh][16 * db + i][lane] = o[db][i];
    if (g == 0) {
      sm.mg.m[rh][r32] = m_run;
      sm.mg.l[rh][r32] = l_row;
    }
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = sm.mg.m[rh][r32];
    const float l1 = sm.mg.l[rh][r32];
    const float mm = fmaxf(m_run, m1);
    float a0 = 0.f, a1 = 0.f;
    if (mm != -INFINITY) {
      a0 = __builtin_amdgcn_exp2f(m_run - mm);
      a1 = __builtin_amdgcn_exp2f(m1 - mm);
    }
    const float L = l_row * a0 + l1 * a1;
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const int row = BLK * u + 32 * rh + r32;
    if (row < N) {
      u16* orow = O + head_off + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * q4 + r;
            y[r] = (__bf16)((o[db][i] * a0 + sm.mg.o[rh][16 * db + i][lane] * a1) * inv);
          }
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * q4 + 4 * g) = y;
        }
    }
  }
}

}  // namespace

int launch_attn_bf16(const void* q, const void* k, const void* v, const uint64_t* mask,
                     const int32_t* order, int n_heads, int seq_len, int head_dim, float scale,
                     void* out, hipStream_t stream) {
  const int nb = n_blocks(seq_len, 64);
  const int W = n_words(nb);
  if (nb > 65535) return fail(BSA_ERR_UNSUPPORTED, "at most 65535 key blocks per head (seq_len %d)", seq_len);
  const float c = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(n_heads * nb)), block(NT);
  const u16* Q = static_cast<const u16*>(q);
  const u16* K = static_cast<const u16*>(k);
  const u16* V = static_cast<const u16*>(v);
  u16* O = static_cast<u16*>(out);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, block, 0, stream, Q, K, V, mask, order,
                       n_heads, seq_len, nb, W, c, O);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, block, 0, stream, Q, K, V, mask, order,
                       n_heads, seq_len, nb, W, c, O);
  BSA_CHECK_HIP(hipGetLastError());
  return ok();
}

}  // namespace bsa

extern "C" int sparse_attn_fwd(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                               int n_heads, int seq_len, int head_dim, int block_q, int block_k,
                               float scale, void* out, hipStream_t stream) {
  using namespace bsa;
  int rc = check_attn_args(q, k, v, mask_bits, out, n_heads, seq_len, head_dim, block_q, block_k,
                           scale, 16);
  if (rc) return rc;
  const size_t rows = (size_t)n_heads * n_blocks(seq_len, 64);
  const size_t off_tiles = (rows * 4 + 255) & ~size_t(255);
  const size_t off_order = (off_tiles + (size_t)n_heads * 8 + 255) & ~size_t(255);
  char* ws = static_cast<char*>(scratch(off_order + rows * 4, stream));
  if (!ws) return BSA_ERR_HIP;
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  int64_t* tiles = reinterpret_cast<int64_t*>(ws + off_tiles);
  int32_t* order = reinterpret_cast<int32_t*>(ws + off_order);
  rc = launch_plan(mask_bits, n_heads, seq_len, counts, tiles, order, stream);
  if (rc) return rc;
  return launch_attn_bf16(q, k, v, mask_bits, order, n_heads, seq_len, head_dim, scale, out, stream);
}

extern "C" int sparse_attn_fwd_planned(const void* q, const void* k, const void* v,
                                       const uint64_t* mask_bits, const int32_t* work_order,
                                       int n_heads, int seq_len, int head_dim, int block_q,
                                       int block_k, float scale, void* out, hipStream_t stream) {
  using namespace bsa;
  int rc = check_attn_args(q, k, v, mask_bits, out, n_heads, seq_len, head_dim, block_q, block_k,
                           scale, 16);
  if (rc) return rc;
  if (!work_order || !aligned(work_order, 4))
    return fail(BSA_ERR_INVALID_ARG, "work_order must be a non-null 4-byte aligned pointer");
  return launch_attn_bf16(q, k, v, mask_bits, work_order, n_heads, seq_len, head_dim, scale, out,
                          stream);
}
