// Block-sparse attention forward, bf16 inputs, bf16 MFMA, fp32 online softmax.
//
// ScalingAttention, section 4.3.2 (CRM kernel) and Appendix E (Algorithm 2): a
// FlashAttention forward whose dense key-block loop is replaced by a walk over
// the set bits of the query block's packed row mask; kept 64x64 tiles are
// computed densely, all other tiles are skipped without touching their K/V.
//
// gfx950 mapping (one workgroup of 4 waves per (head, query block); two query
// blocks with identical mask rows share one workgroup, pair_body below):
//  * wave w owns query rows 32*(w&1) .. +31 and key half 32*(w>>1) .. +31 of every
//    kept tile, so each wave keeps its own running max / sum and output
//    accumulator; the two key halves are merged once at the end.
//  * S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16 with K (A operand) from LDS and
//    Q^T (B operand) held in registers for the whole row.  The accumulator gives
//    lane l the logits of query row l%32 for 16 keys, so the row max and row sum
//    are lane-local plus one exchange with lane l^32.
//  * The same 16 probabilities, rounded to bf16, are exactly the B operand of
//    O^T += V^T P^T, provided the A operand (V^T) pairs each k-slot with the key
//    the accumulator register held.  K rows are stored in a permuted key order
//    (key_of_row) that makes the keys of each group of 8 probability registers
//    consecutive, so the matching V^T operand is one 16-byte run of a row of
//    the transposed V tile.  Every MFMA operand is a single 16-byte LDS read.
//  * V is copied transposed ([head][d][key], rows zero-padded to whole blocks)
//    by a small kernel ahead of the attention kernel.  K and V^T tiles then both
//    travel global -> LDS by DMA (buffer_load ... lds), without VGPRs or VALU
//    work, into 2-stage rings with 16-byte chunks XOR-swizzled against LDS
//    bank conflicts.  The next tile's DMA is issued before the current tile's
//    math, with one barrier per tile.
//  * The row's kept-block list is decoded once per 2048 blocks by wave 0: one mask
//    word per lane, popcount, and a ballot-based exclusive prefix (one ballot per
//    bit of the count) give every lane its write offset into an LDS list.
//  * Single rows first walk their tiles with the running max that the row's
//    first tile sets, taking no max per tile: a NaN-safe test of each tile's
//    probability sum (<= 2^20) goes into a sticky flag.  Only if some wave of the
//    workgroup raised the flag does the workgroup walk the row again in the
//    max-tracking form, whose rescaling is lazy: the running max used for
//    exponentials moves when a tile's max exceeds it by more than 8 (a factor
//    256).  Either walk keeps every probability within a range where the result
//    is exact up to rounding.
//  * pair_body: wave w owns the 32 query rows 32*(w&1) .. +31 of query block
//    w>>1 and both key halves of every tile (no merge at the end).  Both kernels
//    run two workgroups per CU, one wave of each per SIMD, and raise wave
//    priority for their PV MFMAs so that one wave's MFMAs run while the other
//    wave on the SIMD works through its softmax.
//  * With a work order, single rows go out one device-full of workgroups per
//    launch so that rows of similar length start together and walk their tile
//    lists in step; within a launch the XCDs are split into groups that walk
//    different heads (see the row decode in single_row_body).  The pair
//    workgroups and the last few single-row slices (the lightest heads' rows)
//    share one launch (attn_mixed_kernel), so single rows fill the slots the
//    pairs' last, partial round leaves idle; a layer of at most 16 slices sends
//    all of them with the pairs.
#include <cmath>
#include <type_traits>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BLK = 64;
constexpr int NT = 256;
constexpr int LIST_CAP = 2048;
constexpr int CHUNK_WORDS = LIST_CAP / 64;
// Softmax rescaling is checked on each lane's row sum of a tile's 16 bf16
// probabilities, taken against the running max (exp2 domain): while it stays
// at or below 2^20 no probability exceeds 2^20, and O and l cannot overflow
// (2^20 times any key count and value scale here is far below the fp32 range).
// A larger, infinite or NaN sum sends the step to the rescale path.
constexpr float SUM_LIMIT = 1048576.0f;
// Single rows keep the running max: it moves only when a tile's max exceeds it
// by more than this (a factor 2^8 in probability).
constexpr float RESCALE_SLACK = 8.0f;
// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family GPUs:
// 32-bit data format, so the per-access range check against num_records applies.
constexpr int BUFFER_DWORD3 = 0x00020000;

// Rounds a tile-half's 16 probabilities to the bf16 B operands of the PV MFMAs
// and sums the rounded values (the weights PV uses) with two-way dot products
// against (1, 1).
__device__ __forceinline__ void to_bf16_sum(const float (&p)[16], bf16x8& pb0, bf16x8& pb1, float& ls) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pb0[j] = (__bf16)p[j];
    pb1[j] = (__bf16)p[8 + j];
  }
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb0[2 * j], pb0[2 * j + 1]}, one, ls0, false);
    ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb1[2 * j], pb1[2 * j + 1]}, one, ls1, false);
  }
  ls = ls0 + ls1;
}

// Key order inside a tile.  K row r holds key key_of_row(r): r with bits 2 and
// 3 exchanged.  The QK^T accumulator register i of lane l (query l % 32) then
// holds the logit of key 32 kh + 16 (i / 8) + 8 (l / 32) + i % 8, so the eight
// registers 8 s .. 8 s + 7 that form the bf16 B operand of PV MFMA s cover eight
// consecutive keys, and the matching A operand is one 16-byte run of a V^T row.
__device__ __forceinline__ int key_of_row(int r) {
  return (r & ~12) | ((r >> 1) & 4) | ((r << 1) & 8);
}

// LDS bank model behind the tile layouts (measured on gfx950 with the
// bank-conflict counter): a 16-byte read of a wave is served in four passes
// over 64 four-byte banks, each pass taking the lanes of one half-wave whose
// 4-lane quad index has a given bit parity.  Both tiles arrive by LDS DMA,
// which writes 1 KB runs, so rows are unpadded and 16-byte chunks are
// XOR-swizzled instead: chunk c of K row r sits at chunk c ^ k_swz(r), chunk c
// of V^T row d at chunk c ^ v_swz(d).  The rows one read pass touches then land
// on distinct bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 128)
    return r & 15;
  else
    return (r >> 1) & 7;
}
__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

// V transposed in HBM: vt[h][d][key], rows padded to nb * 64 keys with zeros, so
// a V tile is D runs of 128 bytes and travels by LDS DMA like K.  One workgroup
// per (head, key block); the tile goes through LDS with a row stride of D + 2
// elements, which keeps the column reads free of bank conflicts.
template <int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const u16* __restrict__ V, int N, int nb,
                                                          u16* __restrict__ VT) {
  constexpr int S = D + 2;
  __shared__ __attribute__((aligned(16))) u16 tile[BLK * S];
  const int t = blockIdx.x % nb, h = blockIdx.x / nb;
  const u16* src = V + ((size_t)h * N + (size_t)BLK * t) * D;
  for (int i = threadIdx.x; i < BLK * D / 8; i += 256) {
    const int r = i / (D / 8), c = i % (D / 8);
    uint4 x = make_uint4(0, 0, 0, 0);
    if (BLK * t + r < N) x = *reinterpret_cast<const uint4*>(src + (size_t)r * D + 8 * c);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[r * S + 8 * c]);
    dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
  }
  __syncthreads();
  const size_t npad = (size_t)nb * BLK;
  u16* dst = VT + (size_t)h * D * npad + (size_t)BLK * t;
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int d = i / 8, c = i % 8;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[(8 * c + 2 * j) * S + d] | ((uint32_t)tile[(8 * c + 2 * j + 1) * S + d] << 16);
    *reinterpret_cast<uint4*>(dst + (size_t)d * npad + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Single rows: one 64-query row per workgroup of 4 waves, two workgroups per CU.
template <int D>
__device__ __forceinline__ void single_row_body(
    int wg, const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ VT,
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ order, int stream_off,
    int groups, int n_heads, int N, int nb, int W, float c, u16* __restrict__ O,
    u16* __restrict__ kst0, u16* __restrict__ kst1, u16* __restrict__ vts0, u16* __restrict__ vts1, u16* __restrict__ list, int& nlist) {
  constexpr int CPR = D / 8;             // 16-byte chunks per token row
  constexpr int NDB = D / 32;            // 32-wide output column blocks
  constexpr int NKS = D / 16;            // k-steps of the QK^T contraction

  // LDS.  Every stage is a separate object so the compiler can tell the stage
  // being filled by DMA from the stages being read, and waits for a DMA only
  // where its own stage is read.  After the tile loop the V^T stages hold the
  // merge of the two key halves' accumulators and the list their running max
  // and sum.
  // (K stages: row r holds key_of_row(r); V^T stages: row d holds 64 keys)
  auto kstage = [&](int b) { return b ? kst1 : kst0; };
  auto vstage = [&](int b) { return b ? vts1 : vts0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rh = wave & 1;
  const int kh = (wave >> 1) & 1;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // Work entries: e in [0, H nb) is the single row e; pair entries (>= H nb,
  // run by pair_body) and empty slots (-1) are skipped.
  //
  // With a work order the rows go out in slices.  The workgroups of a launch
  // are handed to the 8 XCDs in turn (workgroup i to XCD i mod 8); the XCDs
  // form `groups` groups (XCD x in group x mod groups), and group g walks its
  // own stream of slots: the head segments of the heads ranked g, g + groups,
  // g + 2 groups, ... back to back.  A slice takes gridDim.x / groups
  // consecutive slots of every stream from stream_off on, so the K/V tiles of
  // a head are fetched into the L2s of 8 / groups XCDs instead of all eight.
  // With groups == 1 slot stream_off + blockIdx.x is taken (any grid size).
  const int total_rows = n_heads * nb;
  int row_id = wg;
  if (order) {
    const int i = wg, x = i & 7, g = x % groups;
    const int p = stream_off + x / groups + (8 / groups) * (i >> 3);
    const int r = g + groups * (p / nb);
    if (r >= n_heads) return;
    row_id = order[r * nb + p % nb];
    if (row_id < 0 || row_id >= total_rows) return;
  }
  const int h = row_id / nb;
  const int u = row_id - h * nb;
  const size_t head_off = (size_t)h * N * D;
  const u16* Qh = Q + head_off;
  const u16* Kh = K + head_off;
  const size_t npad = (size_t)nb * BLK;
  const u16* VTh = VT + (size_t)h * D * npad;
  const uint64_t* mrow = mask + ((size_t)h * nb + u) * W;

  // The first chunk's mask words are requested ahead of Q, so the two loads'
  // latencies overlap (wave 0 decodes the chunks; see run_row).
  uint64_t word0 = 0;
  if (wave == 0 && lane < CHUNK_WORDS && lane < W) word0 = mrow[lane];

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
  // Set by the fast form when a tile's probabilities may have left the exact
  // range (see run_row below).
  bool over = false;

  // Both tiles travel by LDS DMA (global -> LDS without VGPRs).  One wave
  // instruction writes 1 KB: KR consecutive K rows, or 8 consecutive V^T rows.
  // Lane l fills its row at chunk position l % (chunks per row), so it fetches
  // the chunk the swizzle stores there.  Each wave issues NI instructions per
  // tensor and tile.
  constexpr int KR = 1024 / (2 * D);                  // K rows per DMA instruction
  constexpr int NI = D / 32;                           // DMA instructions per wave and tensor
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int k_voff[NI], v_voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ii = wave_u * NI + i;
    const int r = ii * KR + lane / CPR;
    k_voff[i] = (key_of_row(r) * CPR + ((lane % CPR) ^ k_swz<D>(r))) * 16;
    const int d = 8 * ii + (lane >> 3);
    v_voff[i] = d * (int)npad * 2 + 16 * ((lane & 7) ^ v_swz(d));
  }
  // Byte offsets (within a K stage) of this lane's QK^T A operands: row
  // p0 + r32, logical chunk 2 ks + g.
  const int p0 = 32 * kh;         // first K row of this wave's key half
  int k_rd[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int r = p0 + r32;
    k_rd[ks] = r * D * 2 + 16 * ((2 * ks + g) ^ k_swz<D>(r));
  }

  // Buffer descriptors with per-lane byte offsets fixed for the whole row.  A K
  // descriptor starts at its tile and its num_records covers only the bytes from
  // there to the end of the head's K, so the per-lane range check (on the lane
  // offset alone; the scalar offset is 0) returns zeros for key rows past the
  // sequence end (the ragged last block, masked out by the softmax) and no read
  // leaves the tensor.  V^T rows are zero-padded to whole blocks, so every V^T
  // tile lies inside its head's descriptor.
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(VTh), 0, (int)(D * npad * 2), BUFFER_DWORD3);

  auto kdma = [&](int kvb, int kbuf) {
#ifdef __HIP_DEVICE_COMPILE__   // the host pass cannot form LDS address-space pointers
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(Kh + (size_t)kvb * BLK * D), 0, (N - kvb * BLK) * D * 2, BUFFER_DWORD3);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krs, (__attribute__((address_space(3))) void*)(kstage(kbuf) + (wave_u * NI + i) * KR * D), 16,
          k_voff[i], 0, 0, 0);
#endif
  };
  auto vdma = [&](int vvb, int vbuf) {
#ifdef __HIP_DEVICE_COMPILE__
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, (__attribute__((address_space(3))) void*)(vstage(vbuf) + (wave_u * NI + i) * 8 * BLK), 16,
          v_voff[i], vvb * BLK * 2, 0, 0);
#endif
  };

  // Keys past the sequence end (only in the ragged last block) get -inf.
  auto mask_ragged = [&](f32x16& s, int vb) {
    const int hi = N - vb * BLK;   // tile positions >= hi lie past the sequence end
    if (hi < BLK) {
      // key of register i = lane base + a constant; compare the base with a
      // scalar threshold per register
      const int kbase = 32 * kh + 8 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kbase >= hi - (16 * (i >> 3) + (i & 7))) s[i] = -INFINITY;
    }
  };
  // Max over this wave's 32 keys of the tile for the lane's query row.  IEEE
  // maximum (NaN-propagating) needs no input canonicalisation and maps to
  // three-input v_maximum3_f32, so the 16 lane-local values take 8 instructions;
  // lanes l and l^32 hold the two 16-key halves of the same query row.
  auto row_max = [&](const f32x16& s) {
    float mx = __builtin_elementwise_maximum(s[0], s[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, s[i]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };

  // One pipeline step for this wave: online softmax of S (tile vb, already in
  // registers), the QK^T MFMAs of the next tile from K stage kbuf (returned),
  // and O^T += V^T P^T from V stage vbuf.  The fast form (SAFE false) keeps the
  // running max the row's first tile set and only records whether a tile's
  // probabilities could have left the range the result is exact in; the safe
  // form checks each tile's max first and rescales lazily.  The next tile's
  // MFMAs do not depend on the softmax, so they are issued in the same
  // straight-line block as the exponentials and interleaved with them (one
  // MFMA, then a few VALU ops).
  // s[i] is the logit of query row r32 for the key held by K row
  // p0 + 8*(i/4) + 4*g + i%4, i.e. key 32kh + 16(i>>3) + 8g + (i&7).
  auto step = [&](f32x16 s, int vb, int kbuf, int vbuf, bool may_be_ragged, auto safe) {
    constexpr bool SAFE = decltype(safe)::value;
    if (may_be_ragged) mask_ragged(s, vb);
    if constexpr (SAFE) {
      const float mt = row_max(s) * c;   // -inf when every key of this half is masked
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
    }
    // --- straight-line block: next tile's QK^T interleaved with this tile's exp2
    f32x16 sn;
#pragma unroll
    for (int i = 0; i < 16; ++i) sn[i] = 0.f;
    float p[16];
    // MFMA operands in registers of their own: all K operands are read first,
    // the V operands between the QK^T MFMAs, so no MFMA waits on a read that
    // was issued just before it.
    bf16x8 ka[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      ka[ks] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kstage(kbuf)) + k_rd[ks]);
    bf16x8 va[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + r32;
#pragma unroll
      for (int s0 = 0; s0 < 2; ++s0) {
        const int chunk = (4 * kh + 2 * s0 + g) ^ v_swz(d);
        va[db][s0] = *reinterpret_cast<const bf16x8*>(vstage(vbuf) + d * BLK + 8 * chunk);
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], sn, 0, 0, 0);
      if (2 * ks < 16) {
        const int i = 2 * ks;
        p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m_run));
        p[i + 1] = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -m_run));
      }
    }
#pragma unroll
    for (int i = 2 * NKS; i < 16; i += 2) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m_run));
      p[i + 1] = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -m_run));
    }
    bf16x8 pb0, pb1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pb0[j] = (__bf16)p[j];
      pb1[j] = (__bf16)p[8 + j];
    }
    // Row sum of the bf16-rounded probabilities, the same weights the PV
    // product uses: four two-way dot products with (1, 1) per operand.
    {
      const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb0[2 * j], pb0[2 * j + 1]}, one, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb1[2 * j], pb1[2 * j + 1]}, one, ls1, false);
      }
      const float ls = ls0 + ls1;
      if constexpr (!SAFE) over = over || !(ls <= SUM_LIMIT);   // also catches inf and NaN
      l_part += ls;
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      if (ks < 2 * NDB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one V operand read
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU ops
    }
    // Two workgroups share each SIMD, one wave of each.  Raising the wave's
    // priority for its PV MFMAs lets them issue back to back while the other
    // wave runs its VALU-heavy softmax, instead of interleaving both waves'
    // MFMAs and stretching both steps.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s0 = 0; s0 < 2; ++s0)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][s0], s0 ? pb1 : pb0, o[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    return sn;
  };

  // S^T of the first tile of a list (no softmax work to overlap with).
  auto qk = [&](int kbuf) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kstage(kbuf)) + k_rd[ks]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
    }
    return s;
  };

  const int tail_bits = nb & 63;
  const uint64_t lastmask = tail_bits ? ((1ull << tail_bits) - 1ull) : ~0ull;
  const uint64_t lanes_below = (1ull << lane) - 1ull;

  // The row's tile walk.  The fast form runs first; if any lane of any wave
  // saw a tile whose bf16 probability sum exceeds SUM_LIMIT (or is not
  // finite), its output could have lost accuracy or overflowed, and the whole
  // workgroup walks the row again in the safe form, which tracks the max tile by
  // tile.  On inputs whose logits stay within 20 (exp2 domain) of the first
  // tile's max the safe form never runs.
  int first_w0 = -1;
  auto run_row = [&](auto safe) {
    constexpr bool SAFE = decltype(safe)::value;
    for (int w0 = 0; w0 < W; w0 += CHUNK_WORDS) {
      __syncthreads();   // every wave is done with the previous chunk's list
      if (wave == 0) {
        const int wi = w0 + lane;
        uint64_t word = 0;
        if (lane < CHUNK_WORDS && wi < W) {
          word = w0 == 0 ? word0 : mrow[wi];
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
      if (first_w0 < 0) first_w0 = w0;
      // Software pipeline with K one tile ahead of V.  At the top of step t the K
      // stage (t+1)&1 holds K(t+1), the V stage t&1 holds V(t) and S(t) is in
      // registers; the K stage t&1 and the V stage (t+1)&1 were last read in step
      // t-1.  Step t starts the DMA of K(t+2) and V(t+1) into those two stages,
      // runs the QK^T MFMAs of tile t+1 next to the softmax of tile t
      // (independent work the scheduler can interleave), then PV of tile t; the
      // barrier at its end (whose fence waits for the wave's DMA) publishes both
      // stages.  Past the end of the list the last tile is used again (loads stay
      // unconditional; the extra S is discarded).
      // Lane j of lv holds list entry t0 + j (clamped to the last entry), so a
      // step takes its tile indices with v_readlane instead of an LDS round trip
      // on its critical path; the window moves once every 60 steps or so.
      int t0 = 0;
      int lv = list[min(lane, n - 1)];
      auto tile = [&](int t) { return __builtin_amdgcn_readlane(lv, t - t0); };
      // only the last block of the sequence can be ragged, and it is always the
      // last entry of an ascending list.  The first two K tiles and the first V
      // tile go out together and land behind one barrier.
      kdma(tile(0), 0);
      vdma(tile(0), 0);
      kdma(tile(1), 1);
      __syncthreads();
      f32x16 s_cur = qk(0);
      if (!SAFE && w0 == first_w0) {
        // the fast form takes the running max from the row's first tile
        mask_ragged(s_cur, tile(0));
        m_run = fmaxf(row_max(s_cur) * c, -1.0e30f);
      }
      __syncthreads();
      // The loop is unrolled by two so each step's stage indices are constants and
      // every LDS address is a per-lane base plus an instruction offset.
      auto body = [&](int t, auto parity) {
        constexpr int P = decltype(parity)::value;   // t & 1
        kdma(tile(t + 2), P);
        vdma(tile(t + 1), P ^ 1);
        s_cur = step(s_cur, tile(t), P ^ 1, P, t == n - 1, safe);
        __syncthreads();
      };
      for (int t = 0; t < n; t += 2) {
        if (t + 3 - t0 > 63) {      // the two steps below read entries up to t + 3
          t0 = t;
          lv = list[min(t0 + lane, n - 1)];
        }
        body(t, std::integral_constant<int, 0>{});
        if (t + 1 < n) body(t + 1, std::integral_constant<int, 1>{});
      }
    }
  };
  run_row(std::false_type{});
  // Workgroup-wide vote on the fast form's flag (nlist is free here: every wave
  // is past its last read of it).
  __syncthreads();
  if (tid == 0) nlist = 0;
  __syncthreads();
  if (__any(over) && lane == 0) nlist = 1;
  __syncthreads();
  if (nlist) {
    m_run = -1.0e30f;
    l_part = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    run_row(std::true_type{});
  }

  // Merge the two key halves of each query-row half and write the output.
  // mo(j)[accumulator register][lane], j = rh, overlays a V^T stage (each
  // 128 * D bytes); mm / ml overlay the block list.
  static_assert(D * BLK * sizeof(u16) == (D / 2) * 64 * sizeof(float), "merge overlay size");
  static_assert(LIST_CAP * sizeof(u16) >= 2 * 2 * 32 * sizeof(float), "merge overlay size");
  auto mo = [&](int j) { return reinterpret_cast<float (*)[64]>(j ? vts1 : vts0); };
  const int mj = rh;
  auto mm = reinterpret_cast<float (*)[32]>(list);
  auto ml = reinterpret_cast<float (*)[32]>(list) + 2;
  __syncthreads();
  const float l_row = l_part + __shfl_xor(l_part, 32);
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) mo(mj)[16 * db + i][lane] = o[db][i];
    if (g == 0) {
      mm[mj][r32] = m_run;
      ml[mj][r32] = l_row;
    }
  }
  __syncthreads();
  if (kh == 0) {
    const float m1 = mm[mj][r32];
    const float l1 = ml[mj][r32];
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
            y[r] = (__bf16)((o[db][i] * a0 + mo(mj)[16 * db + i][lane] * a1) * inv);
          }
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * q4 + 4 * g) = y;
        }
    }
  }
}

// Pair rows (two query blocks with identical mask rows), four waves: wave w owns
// the 32 query rows 32 (w & 1) .. +31 of query block u + (w >> 1) against all 64
// keys of every tile (two QK^T accumulator chains, one per key half, and 16 PV
// MFMAs).  Both query blocks read the same K/V stages, so each tile is fetched
// once for 128 queries, and the workgroup is as small as a single-row one: two
// of them share a CU and each SIMD runs one wave of each, which are not in step.
template <int D>
__device__ __forceinline__ void pair_body(
    int wg, const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ VT,
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ order, int n_heads, int N,
    int nb, int W, float c, u16* __restrict__ O, u16* __restrict__ kst0, u16* __restrict__ kst1, u16* __restrict__ vts0, u16* __restrict__ vts1, u16* __restrict__ list, int& nlist) {
  constexpr int CPR = D / 8;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  auto kstage = [&](int b) { return b ? kst1 : kst0; };
  auto vstage = [&](int b) { return b ? vts1 : vts0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qb = wave >> 1;
  const int rh = wave & 1;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int total_rows = n_heads * nb;
  const int half = nb >> 1;
  const int e = order[(wg / half) * nb + (wg % half)];
  if (e < total_rows || e >= 2 * total_rows) return;
  const int row_id = e - total_rows;
  if ((row_id % nb) & 1 || (row_id % nb) + 1 >= nb) return;
  const int h = row_id / nb;
  const int u = row_id - h * nb;
  const size_t head_off = (size_t)h * N * D;
  const u16* Qh = Q + head_off;
  const u16* Kh = K + head_off;
  const size_t npad = (size_t)nb * BLK;
  const u16* VTh = VT + (size_t)h * D * npad;
  const uint64_t* mrow = mask + ((size_t)h * nb + u) * W;

  bf16x8 qf[NKS];
  {
    const int qrow = BLK * (u + qb) + 32 * rh + r32;
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
  float m_run = -1.0e30f;
  float l_part = 0.f;

  constexpr int KR = 1024 / (2 * D);
  constexpr int NI = D / 32;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // V^T copy offsets: instruction i fills V^T rows 8 (NI w + i) .. +7; at d = 128
  // instructions i and i + 2 differ only by 16 rows (the swizzle repeats), which
  // the scalar offset carries, so two registers hold all four lane offsets.
  constexpr int NVO = NI >= 4 ? 2 : NI;
  int k_voff[NI], v_voff[NVO];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ii = wave_u * NI + i;
    const int r = ii * KR + lane / CPR;
    k_voff[i] = (key_of_row(r) * CPR + ((lane % CPR) ^ k_swz<D>(r))) * 16;
    if (i < NVO) {
      const int d = 8 * ii + (lane >> 3);
      v_voff[i] = d * (int)npad * 2 + 16 * ((lane & 7) ^ v_swz(d));
    }
  }
  // K operand offsets of key half 0 (rows r32); half 1 is 32 rows further.
  int k_rd[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) k_rd[ks] = r32 * D * 2 + 16 * ((2 * ks + g) ^ k_swz<D>(r32));
  // K descriptors start at their tile (see attn_fwd_bf16_kernel).
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(VTh), 0, (int)(D * npad * 2), BUFFER_DWORD3);
  auto kdma = [&](int kvb, int kbuf) {
#ifdef __HIP_DEVICE_COMPILE__
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(Kh + (size_t)kvb * BLK * D), 0, (N - kvb * BLK) * D * 2, BUFFER_DWORD3);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krs, (__attribute__((address_space(3))) void*)(kstage(kbuf) + (wave_u * NI + i) * KR * D), 16,
          k_voff[i], 0, 0, 0);
#endif
  };
  auto vdma = [&](int vvb, int vbuf) {
#ifdef __HIP_DEVICE_COMPILE__
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, (__attribute__((address_space(3))) void*)(vstage(vbuf) + (wave_u * NI + i) * 8 * BLK), 16,
          v_voff[i % NVO], vvb * BLK * 2 + (i / NVO) * 32 * (int)npad, 0, 0);
#endif
  };
  auto kread = [&](int kbuf, int kh, int ks) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kstage(kbuf)) + k_rd[ks] +
                                            kh * 32 * D * 2);
  };
  auto qk = [&](int kbuf, int kh) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kbuf, kh, ks), qf[ks], s, 0, 0, 0);
    return s;
  };

  // One step on tile vb: softmax of S(vb) = (s0, s1) (key halves 0 and 1),
  // QK^T of the next tile from K stage kbuf (returned in s0n, s1n), PV from V^T
  // stage vbuf.  Register i of s_kh holds key 32 kh + 16 (i >> 3) + 8 g + (i & 7).
  auto step = [&](f32x16& s0, f32x16& s1, int vb, int kbuf, int vbuf, bool may_be_ragged) {
    if (may_be_ragged) {
      const int hi = N - vb * BLK;
      if (hi < BLK) {
        const int kbase = 8 * g;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (kbase >= hi - (16 * (i >> 3) + (i & 7))) s0[i] = -INFINITY;
          if (kbase >= hi - (32 + 16 * (i >> 3) + (i & 7))) s1[i] = -INFINITY;
        }
      }
    }
    // key half 0: next tile's QK^T interleaved with this tile's exp2, then half 1;
    // exponentials against the running max as it stands (see the single-row step)
    bf16x8 pb[2][2];
    float lh[2];
    f32x16 sn[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const f32x16& s = kh ? s1 : s0;
      bf16x8 ka[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) ka[ks] = kread(kbuf, kh, ks);
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[kh][i] = 0.f;
      float p[16];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sn[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], sn[kh], 0, 0, 0);
        if (2 * ks < 16) {
          p[2 * ks] = __builtin_amdgcn_exp2f(fmaf(s[2 * ks], c, -m_run));
          p[2 * ks + 1] = __builtin_amdgcn_exp2f(fmaf(s[2 * ks + 1], c, -m_run));
        }
      }
#pragma unroll
      for (int i = 2 * NKS; i < 16; i += 2) {
        p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m_run));
        p[i + 1] = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, -m_run));
      }
      to_bf16_sum(p, pb[kh][0], pb[kh][1], lh[kh]);
      __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
    if (__any(!(lh[0] <= SUM_LIMIT && lh[1] <= SUM_LIMIT))) {
      float mx = __builtin_elementwise_maximum(s0[0], s0[1]);
#pragma unroll
      for (int i = 2; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, s0[i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, s1[i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float mn = fmaxf(m_run, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_run = mn;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const f32x16& s = kh ? s1 : s0;
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -m_run));
        to_bf16_sum(p, pb[kh][0], pb[kh][1], lh[kh]);
      }
    }
    l_part += lh[0] + lh[1];
    // V^T operand of PV MFMA (k-slot j: keys 16 j .. 16 j + 15, column block db).
    // Key half 0's operands are read ahead of the raised-priority PV block, in
    // the registers the K operands held, so its first MFMAs do not each wait for
    // an LDS round trip; the wave has no registers left to read half 1's ahead too.
    auto vread = [&](int j, int db) {
      const int d = 32 * db + r32;
      const int chunk = (2 * j + g) ^ v_swz(d);
      return *reinterpret_cast<const bf16x8*>(vstage(vbuf) + d * BLK + 8 * chunk);
    };
    constexpr int PRE = 2 * NDB;
    bf16x8 vpre[PRE];
#pragma unroll
    for (int i = 0; i < PRE; ++i) vpre[i] = vread(i / NDB, i % NDB);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kh = j >> 1, s0i = j & 1;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int i = j * NDB + db;
        const bf16x8 a = i < PRE ? vpre[i < PRE ? i : 0] : vread(j, db);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kh][s0i], o[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    s0 = sn[0];
    s1 = sn[1];
  };

  const int tail_bits = nb & 63;
  const uint64_t lastmask = tail_bits ? ((1ull << tail_bits) - 1ull) : ~0ull;
  const uint64_t lanes_below = (1ull << lane) - 1ull;
  for (int w0 = 0; w0 < W; w0 += CHUNK_WORDS) {
    __syncthreads();
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
    int t0 = 0;
    int lv = list[min(lane, n - 1)];
    auto tile = [&](int t) { return __builtin_amdgcn_readlane(lv, t - t0); };
    kdma(tile(0), 0);
    vdma(tile(0), 0);
    kdma(tile(1), 1);
    __syncthreads();
    f32x16 s0 = qk(0, 0), s1 = qk(0, 1);
    __syncthreads();
    auto body = [&](int t, auto parity) {
      constexpr int P = decltype(parity)::value;
      kdma(tile(t + 2), P);
      vdma(tile(t + 1), P ^ 1);
      step(s0, s1, tile(t), P ^ 1, P, t == n - 1);
      __syncthreads();
    };
    for (int t = 0; t < n; t += 2) {
      if (t + 3 - t0 > 63) {
        t0 = t;
        lv = list[min(t0 + lane, n - 1)];
      }
      body(t, std::integral_constant<int, 0>{});
      if (t + 1 < n) body(t + 1, std::integral_constant<int, 1>{});
    }
  }

  // Each wave holds whole rows (both key halves): lanes l and l ^ 32 hold the two
  // key parities of each row's sum.
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
  const float l_row = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;
  const int row = BLK * (u + qb) + 32 * rh + (int)(__lane_id() & 31);
  if (row < N) {
    u16* orow = O + head_off + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = (__bf16)(o[db][4 * q4 + r] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * q4 + 4 * g) = y;
      }
  }
}


// The kernels: single rows, and one launch holding the pair workgroups
// followed by the last single-row slices (attn_mixed_kernel), so
// that single rows take the slots the pair launch's last, partial round leaves
// free.  Both declare the same LDS objects.
template <int D>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ VT,
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ order, int stream_off,
    int groups, int n_heads, int N, int nb, int W, float c, u16* __restrict__ O) {
  __shared__ __attribute__((aligned(16))) u16 kst0[BLK * D];
  __shared__ __attribute__((aligned(16))) u16 kst1[BLK * D];
  __shared__ __attribute__((aligned(16))) u16 vts0[D * BLK];
  __shared__ __attribute__((aligned(16))) u16 vts1[D * BLK];
  __shared__ __attribute__((aligned(16))) u16 list[LIST_CAP];
  __shared__ int nlist;
  single_row_body<D>(blockIdx.x, Q, K, VT, mask, order, stream_off, groups, n_heads, N, nb, W, c, O,
                     kst0, kst1, vts0, vts1, list, nlist);
}

// Workgroups [0, pair_wgs) are the pair launch (pair_wgs a multiple of 8; those
// past n_heads * (nb / 2) exit); the rest are single-row slices of slice_wgs
// workgroups each (a multiple of 8 when groups > 1), so every workgroup keeps
// its XCD (workgroup index mod 8) in the slice's layout.
template <int D>
__global__ __launch_bounds__(NT, 2) void attn_mixed_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ VT,
    const uint64_t* __restrict__ mask, const int32_t* __restrict__ order, int pair_wgs,
    int slice_wgs, int stream_off, int groups, int n_heads, int N, int nb, int W, float c,
    u16* __restrict__ O) {
  __shared__ __attribute__((aligned(16))) u16 kst0[BLK * D];
  __shared__ __attribute__((aligned(16))) u16 kst1[BLK * D];
  __shared__ __attribute__((aligned(16))) u16 vts0[D * BLK];
  __shared__ __attribute__((aligned(16))) u16 vts1[D * BLK];
  __shared__ __attribute__((aligned(16))) u16 list[LIST_CAP];
  __shared__ int nlist;
  const int b = blockIdx.x;
  if (b < pair_wgs) {
    if (b < n_heads * (nb / 2))
      pair_body<D>(b, Q, K, VT, mask, order, n_heads, N, nb, W, c, O, kst0, kst1, vts0, vts1, list, nlist);
    return;
  }
  const int j = b - pair_wgs;
  if (groups > 1)
    single_row_body<D>(j % slice_wgs, Q, K, VT, mask, order, stream_off + (j / slice_wgs) * (slice_wgs / groups),
                       groups, n_heads, N, nb, W, c, O, kst0, kst1, vts0, vts1, list, nlist);
  else
    single_row_body<D>(j, Q, K, VT, mask, order, stream_off, 1, n_heads, N, nb, W, c, O, kst0, kst1, vts0, vts1, list, nlist);
}

// Workgroups the device holds at once for this kernel (CUs x resident
// workgroups per CU), cached per device.
template <int D>
int generation_size() {
  constexpr int kMaxDev = 64;
  static int cache[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  if (cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_bf16_kernel<D>, NT, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 0;
  cache[dev] = cus * per_cu;
  return cache[dev];
}

template <int D>
int launch_generations(const u16* Q, const u16* K, const u16* V, const uint64_t* mask,
                       const int32_t* order, int n_heads, int seq_len, int nb, int W, float c,
                       u16* O, u16* VT, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_v_kernel<D>, dim3((unsigned)(n_heads * nb)), dim3(256), 0, stream, V,
                     seq_len, nb, VT);
  BSA_CHECK_HIP(hipGetLastError());
  // With a work order the rows are launched one device-full of workgroups at a
  // time.  Every workgroup of a slice starts together, so rows of similar
  // length from the same head (the planner groups them) walk their ascending
  // tile lists in step and find each other's K/V tiles in L2; a single launch
  // lets start times drift apart after the first wave of workgroups retires,
  // and the tiles in use then spread over the whole head.  Within a slice the
  // XCDs are split into groups that work on different heads (see the kernel's
  // row decode).  Without an order the grid goes out in one launch.
  // Pair entries (two query blocks with identical mask rows) go first, as
  // 128-query workgroups over the pair slots of every head segment.  They are
  // all the same length (a full head's pair row walks every tile), so their last
  // round is partial; the last MIX single-row slices ride in the same launch,
  // after the pair workgroups, and take those idle slots (a whole launch of
  // 4728 pairs at the Wan2.1-14B shape leaves about 1 ms of the layer idle).
  const int total = n_heads * nb;
  int gen = order ? generation_size<D>() : 0;
  if (gen <= 0) gen = total;
  // XCD groups for the single-row slices: 4 when the heads split evenly over
  // four streams, else 2 or 1; a slice must be a whole number of rounds of 8.
  int groups = 1;
  if (order && gen % 8 == 0) groups = n_heads % 4 == 0 ? 4 : (n_heads % 2 == 0 ? 2 : 1);
  const int per = gen / groups;                 // slots of each stream per slice
  const int len = (n_heads / groups) * nb;      // slots in each stream
  // Pair entries go first, in the same launch as the last MIX single-row slices
  // (see attn_mixed_kernel): those hold the lightest heads' rows, which are
  // short, and hold rows at all unless every row of those heads is paired (the
  // heads whose rows are all paired are the full ones, which rank first by total
  // work, so their empty single-row slots are the first slices).  The other
  // slices follow one launch each, heaviest first.  A layer of at most 16
  // slices sends them all with the pairs: its heads are small and its rows
  // short, so a launch boundary per slice costs more than the common start
  // gains (Wan2.1-1.3B 480p: 1.78 -> 1.74 ms).
  const int slices = groups == 1 ? (total + gen - 1) / gen : (len + per - 1) / per;
  const int MIX = slices <= 16 ? slices : 8;
  int last = slices;                            // slices [last, slices) ride with the pairs
  if (order && nb >= 2) {
    const int pair_wgs = (n_heads * (nb / 2) + 7) & ~7;
    last = slices > MIX ? slices - MIX : 0;
    const int off = groups == 1 ? last * gen : last * per;
    const int singles = groups == 1 ? total - off : (slices - last) * gen;
    hipLaunchKernelGGL((attn_mixed_kernel<D>), dim3((unsigned)(pair_wgs + singles)), dim3(NT), 0, stream, Q,
                       K, VT, mask, order, pair_wgs, gen, off, groups, n_heads, seq_len, nb, W, c, O);
    BSA_CHECK_HIP(hipGetLastError());
  }
  if (groups == 1) {
    for (int off = 0; off < last * gen && off < total; off += gen) {
      const int count = min(gen, total - off);
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<D>), dim3((unsigned)count), dim3(NT), 0, stream, Q, K, VT,
                         mask, order, off, 1, n_heads, seq_len, nb, W, c, O);
      BSA_CHECK_HIP(hipGetLastError());
    }
    return ok();
  }
  for (int off = 0; off < last * per && off < len; off += per) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D>), dim3((unsigned)gen), dim3(NT), 0, stream, Q, K, VT,
                       mask, order, off, groups, n_heads, seq_len, nb, W, c, O);
    BSA_CHECK_HIP(hipGetLastError());
  }
  return ok();
}

}  // namespace

size_t vt_bytes(int n_heads, int seq_len, int head_dim) {
  return (size_t)n_heads * head_dim * n_blocks(seq_len, 64) * 64 * 2;
}

int launch_attn_bf16(const void* q, const void* k, const void* v, const uint64_t* mask,
                     const int32_t* order, int n_heads, int seq_len, int head_dim, float scale,
                     void* out, void* vt, hipStream_t stream) {
  const int nb = n_blocks(seq_len, 64);
  const int W = n_words(nb);
  if (nb > 65535) return fail(BSA_ERR_UNSUPPORTED, "at most 65535 key blocks per head (seq_len %d)", seq_len);
  if ((size_t)head_dim * nb * 64 * 2 > 0x7fffffffull)
    return fail(BSA_ERR_UNSUPPORTED, "one head's transposed V must stay below 2 GiB (seq_len %d)", seq_len);
  const float c = scale * 1.4426950408889634f;
  const u16* Q = static_cast<const u16*>(q);
  const u16* K = static_cast<const u16*>(k);
  const u16* V = static_cast<const u16*>(v);
  u16* O = static_cast<u16*>(out);
  u16* VT = static_cast<u16*>(vt);
  if (head_dim == 128)
    return launch_generations<128>(Q, K, V, mask, order, n_heads, seq_len, nb, W, c, O, VT, stream);
  return launch_generations<64>(Q, K, V, mask, order, n_heads, seq_len, nb, W, c, O, VT, stream);
}

}  // namespace bsa

namespace bsa {
namespace {
// Workspace of the unplanned bf16 entry points: row counts, head totals and the
// work order of the planner, then the transposed V; every part 256-byte aligned.
struct AttnWorkspace {
  size_t off_tiles, off_order, off_vt, bytes;
};
AttnWorkspace attn_workspace(int n_heads, int seq_len, int head_dim) {
  const size_t rows = (size_t)n_heads * n_blocks(seq_len, 64);
  AttnWorkspace w;
  w.off_tiles = (rows * 4 + 255) & ~size_t(255);
  w.off_order = (w.off_tiles + (size_t)n_heads * 8 + 255) & ~size_t(255);
  w.off_vt = (w.off_order + rows * 4 + 255) & ~size_t(255);
  w.bytes = w.off_vt + vt_bytes(n_heads, seq_len, head_dim);
  return w;
}
}  // namespace

size_t attn_workspace_bytes(int n_heads, int seq_len, int head_dim) {
  return attn_workspace(n_heads, seq_len, head_dim).bytes;
}

int attn_bf16_with_workspace(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                             int n_heads, int seq_len, int head_dim, float scale, void* out, char* ws,
                             hipStream_t stream) {
  const AttnWorkspace w = attn_workspace(n_heads, seq_len, head_dim);
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  int64_t* tiles = reinterpret_cast<int64_t*>(ws + w.off_tiles);
  int32_t* order = reinterpret_cast<int32_t*>(ws + w.off_order);
  int rc = launch_plan(mask_bits, n_heads, seq_len, counts, tiles, order, stream);
  if (rc) return rc;
  return launch_attn_bf16(q, k, v, mask_bits, order, n_heads, seq_len, head_dim, scale, out,
                          ws + w.off_vt, stream);
}
}  // namespace bsa

extern "C" int sparse_attn_fwd(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                               int n_heads, int seq_len, int head_dim, int block_q, int block_k,
                               float scale, void* out, hipStream_t stream) {
  using namespace bsa;
  int rc = check_attn_args(q, k, v, mask_bits, out, n_heads, seq_len, head_dim, block_q, block_k,
                           scale, 16);
  if (rc) return rc;
  ScratchLease lease(attn_workspace(n_heads, seq_len, head_dim).bytes);
  char* ws = static_cast<char*>(lease.get());
  if (!ws) return BSA_ERR_HIP;
  return attn_bf16_with_workspace(q, k, v, mask_bits, n_heads, seq_len, head_dim, scale, out, ws, stream);
}

extern "C" size_t sparse_attn_workspace_bytes(int n_heads, int seq_len, int head_dim) {
  using namespace bsa;
  if (n_heads < 1 || seq_len < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  if ((long long)n_heads * n_blocks(seq_len, 64) > 0x7fffffffLL) return 0;
  return attn_workspace(n_heads, seq_len, head_dim).bytes;
}

extern "C" int sparse_attn_fwd_ws(const void* q, const void* k, const void* v,
                                  const uint64_t* mask_bits, int n_heads, int seq_len, int head_dim,
                                  int block_q, int block_k, float scale, void* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  using namespace bsa;
  int rc = check_attn_args(q, k, v, mask_bits, out, n_heads, seq_len, head_dim, block_q, block_k,
                           scale, 16);
  if (rc) return rc;
  if (!workspace || !aligned(workspace, 256))
    return fail(BSA_ERR_INVALID_ARG, "workspace must be a non-null 256-byte aligned device pointer");
  const size_t need = attn_workspace(n_heads, seq_len, head_dim).bytes;
  if (workspace_bytes < need)
    return fail(BSA_ERR_INVALID_ARG, "workspace holds %zu bytes, this call needs %zu", workspace_bytes,
                need);
  return attn_bf16_with_workspace(q, k, v, mask_bits, n_heads, seq_len, head_dim, scale, out,
                                  static_cast<char*>(workspace), stream);
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
  ScratchLease lease(vt_bytes(n_heads, seq_len, head_dim));
  void* vt = lease.get();
  if (!vt) return BSA_ERR_HIP;
  return launch_attn_bf16(q, k, v, mask_bits, work_order, n_heads, seq_len, head_dim, scale, out,
                          vt, stream);
}
