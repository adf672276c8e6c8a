/*
 * bsattn.h -- block-sparse video-DiT self-attention for AMD MI355X (gfx950).
 *
 * One operation and its mask producers, exported with a plain C ABI:
 *
 *   O = softmax(scale * Q K^T + M) V,   M = 0 on kept 64x64 blocks, -inf elsewhere,
 *
 * over the flattened (frame, height, width) tokens of one video-DiT attention
 * layer.  This is the bit-wise block-sparse FlashAttention kernel of
 * ScalingAttention (section 4.3.2, "CRM kernel"; Appendix E, Algorithm 2), the
 * same operation PSA runs under stripe masks (PSA page, Figure 3) and that online
 * top-p methods run under predicted block masks (SCOPE and "Competition Domains
 * Matter" abstracts).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers owned by the caller unless marked "host".  The
 *   library never frees or retains them.
 * - Tensors are dense and row-major:  q, k, v, out are [n_heads][seq_len][head_dim]
 *   (batch folded into n_heads).  bf16 entry points take raw bfloat16 storage.
 * - Mask rows (the packed row mask, "CRM" in ScalingAttention section 4.3.2) are
 *   uint64 [n_heads][nb][W] with nb = ceil(seq_len / 64) and W = ceil(nb / 64);
 *   bit b (least significant = 0) of word w marks key block 64*w + b as kept for
 *   that query block.  Bits at positions >= nb are ignored.
 * - seq_len is the real token count; keys at positions >= seq_len in the last
 *   block do not exist (they are excluded, never treated as zero keys).
 *   A query row whose mask row keeps no block produces an output of 0.
 * - Device pointers and `stream` must belong to the calling thread's current HIP
 *   device: launch sizes and the library's scratch memory are taken per current
 *   device.
 * - Every device entry point is stream-ordered and asynchronous: it validates its
 *   arguments on the host, enqueues kernels on `stream` and returns.  Faults of
 *   enqueued kernels surface at the caller's next synchronisation.
 * - Return value: BSA_OK (0) or an error code; a thread-local message describing
 *   the last error is available from bsa_last_error().  Argument errors are
 *   detected before any HIP call, so nothing is enqueued when one is returned.
 *   The library never aborts and never throws across this boundary.
 * - Alignment: q, k, v, out, scores and x/y must be 16-byte aligned; mask and
 *   index arrays 8- and 4-byte aligned respectively.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_OK 0
#define BSA_ERR_INVALID_ARG 1   /* null/misaligned pointer, bad size, non-finite scale ... */
#define BSA_ERR_UNSUPPORTED 2   /* valid but not implemented (block != 64, head_dim not 64/128) */
#define BSA_ERR_HIP 3           /* a HIP runtime call failed; message holds hipGetErrorString */

/* Message for the last error returned on this host thread ("" if none). */
const char* bsa_last_error(void);

/* Words per mask row, ceil(ceil(seq_len / block) / 64); -1 if seq_len < 1 or block < 1.
 * ScalingAttention section 4.3.2: one word load decodes as many blocks as the word
 * has bits (ScalingAttention's 32-bit words and 128-token blocks give 64 loads per row at
 * 256k tokens; this library's 64-bit words and 64-token blocks give 31 at 126,720). */
int bsa_mask_words(int seq_len, int block);

/*
 * sparse_attn_fwd -- block-sparse attention forward, bfloat16 in/out, fp32 softmax.
 * ScalingAttention section 4.3.2 and Appendix E (Algorithm 2): each (head, query
 * block) workgroup walks the set bits of its mask row and runs dense FlashAttention
 * tiles only on kept key blocks, with an online softmax (running max and sum).
 *
 *   q, k, v    bf16 [n_heads][seq_len][head_dim], read only.
 *   mask_bits  uint64 [n_heads][nb][W] as above, read only.
 *   n_heads    >= 1;  seq_len >= 1;  head_dim in {64, 128};
 *   block_q, block_k  must both be 64 (else BSA_ERR_UNSUPPORTED);
 *   scale      finite and > 0 (typically 1/sqrt(head_dim));
 *   out        bf16 [n_heads][seq_len][head_dim], written (round to nearest even).
 *
 * Work is ordered by a device-side planning pass (row popcounts; heads, then rows,
 * in decreasing kept-block count).  V is first copied transposed ([n_heads][head_dim]
 * [nb * 64], zero-padded) so its tiles stream like K's.  The plan and the transposed
 * V live in a library-owned per-device scratch buffer that grows on demand (the
 * first call at a larger size synchronises the device, then frees the old buffer,
 * so it must not run under stream capture).  Host threads may call concurrently:
 * each call holds the device's scratch lock until its launches are enqueued, so a
 * buffer is never freed under a call.  But the buffer's contents are shared:
 * calls whose kernels overlap on one device (different streams) race on them.
 * sparse_attn_fwd_ws below takes a caller workspace instead.
 */
int sparse_attn_fwd(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                    int n_heads, int seq_len, int head_dim, int block_q, int block_k,
                    float scale, void* out, hipStream_t stream);

/*
 * sparse_attn_workspace_bytes -- bytes of device workspace sparse_attn_fwd_ws needs
 * for this shape: the plan (int32 row counts and work order [n_heads * nb], int64
 * head totals [n_heads]) and the transposed V (bf16 [n_heads][head_dim][nb * 64]),
 * each part 256-byte aligned.  0 when the arguments are invalid (n_heads or
 * seq_len < 1, head_dim not 64 or 128, n_heads * nb >= 2^31).
 */
size_t sparse_attn_workspace_bytes(int n_heads, int seq_len, int head_dim);

/*
 * sparse_attn_fwd_ws -- sparse_attn_fwd with a caller-owned workspace in place of
 * the library's scratch buffer; it allocates, frees and synchronises nothing.
 *   workspace        device pointer, 256-byte aligned, at least
 *                    sparse_attn_workspace_bytes(n_heads, seq_len, head_dim) bytes;
 *                    its contents on entry do not matter and are not preserved.
 *   workspace_bytes  its size; a smaller size is BSA_ERR_INVALID_ARG.
 * Calls with distinct workspaces are independent of each other on any streams and
 * threads; two calls sharing a workspace must be ordered by the caller.  Other
 * arguments and behaviour as sparse_attn_fwd (bf16 only).
 */
int sparse_attn_fwd_ws(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                       int n_heads, int seq_len, int head_dim, int block_q, int block_k,
                       float scale, void* out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * sparse_attn_fwd_noalloc -- sparse_attn_fwd for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, same result bit for bit.  Its scratch memory (plan +
 * transposed V) is one fixed 256 MiB array in the library's code object, which every
 * device the library runs on holds until the process ends; the call itself allocates,
 * frees and synchronises nothing.  The heads go through in chunks whose scratch fits
 * the array (a multiple of 4 heads when at least 4 fit), one after another on `stream`.
 * A shape whose single head needs more than the array (about 1M tokens at
 * head_dim 128) is BSA_ERR_UNSUPPORTED, returned before any HIP call.  Every call on a
 * device shares that device's array and leaves its contents behind (each call rewrites
 * all it reads), so calls whose kernels overlap on one device race on it.
 */
int sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                            int n_heads, int seq_len, int head_dim, int block_q, int block_k,
                            float scale, void* out, hipStream_t stream);

/*
 * sparse_attn_fwd_f32 -- same operation and arguments with fp32 q, k, v, out and
 * fp32 arithmetic throughout (reference-precision path for small cases).
 */
int sparse_attn_fwd_f32(const float* q, const float* k, const float* v, const uint64_t* mask_bits,
                        int n_heads, int seq_len, int head_dim, int block_q, int block_k,
                        float scale, float* out, hipStream_t stream);

/*
 * sparse_attn_plan -- the tile scheduler on its own.  For static masks (computed
 * offline and reused across denoising steps, ScalingAttention section 4.1 and
 * Appendix A) the plan can be computed once and reused.
 *
 *   mask_bits   uint64 [n_heads][nb][W], read only.
 *   row_counts  int32 [n_heads * nb], written: kept blocks of each (head, query block) row.
 *   head_tiles  int64 [n_heads], written: kept blocks of each head.
 *   work_order  int32 [n_heads * nb], written: work entries, one segment of nb
 *               slots per head, heads in decreasing head_tiles (ties by head index).
 *               Entry values: h * nb + u is the single row u of head h;
 *               n_heads * nb + h * nb + u (u even) is the pair of rows u, u + 1, whose
 *               mask rows are identical, run by one 128-query workgroup that fetches
 *               each K/V tile once for both; -1 is an empty slot.  Within a segment:
 *               pairs, then singles, each in decreasing row_counts (ties by increasing
 *               u), then the -1 slots.  When nb > 8192 the segment lists the single
 *               rows in increasing u (no pairs).  Rows of equal length then run side by
 *               side, which keeps their tile walks in step and their K/V in L2.
 */
int sparse_attn_plan(const uint64_t* mask_bits, int n_heads, int seq_len, int block,
                     int32_t* row_counts, int64_t* head_tiles, int32_t* work_order,
                     hipStream_t stream);

/*
 * sparse_attn_fwd_planned -- sparse_attn_fwd with a caller-provided work order
 * (normally from sparse_attn_plan).  Single entries h * nb + u may appear anywhere;
 * pair entries (see sparse_attn_plan) are read only from the first nb / 2 slots of
 * each nb-slot segment, and the two rows of a pair must have identical mask rows.
 * Every row must be covered exactly once; other values are skipped.  A plain
 * permutation of [0, n_heads * nb) is a valid order.  The transposed copy of V uses the
 * library's per-device scratch buffer (see sparse_attn_fwd about overlapping calls).
 * After the transpose, the single entries go out in slices of one device-full of
 * workgroups each (compute units x resident workgroups per unit), so that the rows of each
 * slice start together.  The pair entries share one launch with the last eight slices
 * (pair workgroups first, the slices behind them: the lightest rows, which fill the
 * pairs' last round), or with every slice when there are at most 16; the other slices
 * follow as consecutive kernel launches.  The
 * XCDs are split into G groups (G = 4 when n_heads is a multiple of 4, else 2 when it
 * is even, else 1): group g walks the segments g, g + G, g + 2G, ... back to back, and
 * each launch takes the next device-full / G slots of every group's walk, so the K/V
 * tiles of a head are fetched by 8 / G of the 8 XCDs.  Within a segment the order given
 * is kept.
 */
int sparse_attn_fwd_planned(const void* q, const void* k, const void* v, const uint64_t* mask_bits,
                            const int32_t* work_order, int n_heads, int seq_len, int head_dim,
                            int block_q, int block_k, float scale, void* out, hipStream_t stream);

/*
 * sparse_attn_fwd_b128 -- sparse_attn_fwd with ScalingAttention's own mask format:
 * 128 x 128-token blocks, each row packed in 32-bit words (ScalingAttention section
 * 4.3.2: one uint32 load decodes 32 KV blocks; Appendix E, Algorithm 2 steps its
 * base by 32 per word).
 *
 *   q, k, v, out  as sparse_attn_fwd (bf16 [n_heads][seq_len][head_dim]).
 *   mask_words    uint32 [n_heads][nb128][W], nb128 = ceil(seq_len / 128),
 *                 W = ceil(nb128 / 32) (= bsa_mask_words(seq_len, 64)); bit b of
 *                 word w is key block 32 w + b; padding bits are ignored.  4-byte
 *                 aligned, read only.
 * Keys and queries of the last, possibly short, 128-block are its real tokens only.
 * The mask is expanded (mask_b128_to_b64) into the library's per-device scratch
 * buffer; the two 64-token halves of every 128-row then form a pair in the work
 * order, so each K/V tile is fetched once per 128 queries.  Scratch and error
 * behaviour as sparse_attn_fwd.  Rows pair only while ceil(seq_len / 64) <= 8192.
 */
int sparse_attn_fwd_b128(const void* q, const void* k, const void* v, const uint32_t* mask_words,
                         int n_heads, int seq_len, int head_dim, float scale, void* out,
                         hipStream_t stream);

/*
 * mask_b128_to_b64 -- the same mask rewritten over 64-token blocks: 64-block (u, v)
 * is kept iff 128-block (u / 2, v / 2) is.  Word w of a 32-bit row and word w of a
 * 64-bit row cover the same tokens, so the expansion is word for word.
 *   mask_words  uint32 [n_heads][ceil(seq_len/128)][W], read only (W as above).
 *   mask_bits   uint64 [n_heads][ceil(seq_len/64)][W], written in full (padding
 *               bits zero).
 */
int mask_b128_to_b64(const uint32_t* mask_words, int n_heads, int seq_len, uint64_t* mask_bits,
                     hipStream_t stream);

/*
 * mask_from_stripes -- expand per-head PSA stripe tuples into packed row masks.
 * PSA page, Figure 3 and Appendix Tables 7-9: per head either "full window" or a
 * temporal (width, offset, stride) and a spatial (width, offset, stride) stripe.
 * Reading used (the page names the parameters but prints no predicate): distances
 * are key minus query, in frames (temporal) and in 64-token spatial blocks of the
 * frame (spatial); x = dist - offset + width/2 (integer division); a stride of 0
 * means a single band, 0 <= x < width; otherwise the stride is the gap between
 * stripes and the band repeats with period width + stride, (x mod period) < width.
 * A pair is kept when full, or when both the temporal and spatial tests hold.
 * When frame_tokens is not a multiple of block, a block is placed by its first token.
 *
 *   params      int32 [n_heads][7] = {full, Tw, To, Ts, Sw, So, Ss}; widths >= 1,
 *               strides >= 0 (device memory).
 *   n_frames, frame_tokens  with n_frames * frame_tokens == seq_len.
 *   block       must be 64.
 *   mask_bits   uint64 [n_heads][nb][W], written in full (padding bits zero).
 * Widths/strides are not checked on the device; a width < 1 keeps nothing.
 */
int mask_from_stripes(const int32_t* params, int n_heads, int n_frames, int frame_tokens,
                      int seq_len, int block, uint64_t* mask_bits, hipStream_t stream);

/*
 * block_scores_meanpool -- block proxy scores for online mask prediction (SCOPE
 * abstract: masks predicted from block-level proxy scores; pooling as in
 * ScalingAttention Eq. 1).  qbar_u, kbar_v are fp32 means over the real tokens of
 * each 64-token block; scores[h][u][v] = scale * <qbar_u, kbar_v> in fp32.
 *
 *   q, k     bf16 [n_heads][seq_len][head_dim], head_dim in {64, 128}; block must be 64.
 *   scores   fp32 [n_heads][nb][nb], written.
 * Uses the library's per-device scratch buffer for the pooled means (see
 * sparse_attn_fwd about overlapping calls).
 */
int block_scores_meanpool(const void* q, const void* k, int n_heads, int seq_len, int head_dim,
                          int block, float scale, float* scores, hipStream_t stream);

/*
 * mask_from_block_scores_topp -- hybrid top-p selection with a top-k minimum
 * ("Competition Domains Matter" and SCOPE abstracts; cumulative-mass cut-off as in
 * ScalingAttention Appendix A, Algorithm 1).  Per row of n = n_k_blocks scores, in
 * float32 with every operation rounded to nearest and never fused:
 *   m = max s;  e_j = EXP(s_j - m)  (the library's Cody-Waite + degree-7 Taylor exp,
 *   0 below -87);  order = s descending, ties to the lower index;  Z = sequential sum
 *   of e in that order;  c accumulates e/Z in that order and the first position where
 *   c >= p gives k_p (k_p = n if never);  keep the first max(k_p, min(min_blocks, n))
 *   blocks of the order.
 *
 *   scores      fp32 [n_heads][n_q_blocks][n_k_blocks]; 1 <= n_k_blocks <= 4096.  Each
 *               score is first clamped: NaN becomes -FLT_MAX, +inf FLT_MAX and -inf
 *               -FLT_MAX (so a NaN block is kept only when the top-k minimum or p
 *               reaches the lowest scores, lower-index ties first).
 *   p           in (0, 1];  min_blocks >= 0.
 *   mask_bits   uint64 [n_heads][n_q_blocks][ceil(n_k_blocks/64)], written in full.
 */
int mask_from_block_scores_topp(const float* scores, int n_heads, int n_q_blocks, int n_k_blocks,
                                float p, int min_blocks, uint64_t* mask_bits, hipStream_t stream);

/*
 * mask_from_threshold_map -- static block masks from a threshold map
 * (ScalingAttention section 4.1.2, Eq. 2 and the comparison after it; Appendix A,
 * Algorithm 1, static block mask generation): mask = I(T <= p*) per head.
 *
 *   thresholds  fp32 [n_heads][n_q_blocks][n_k_blocks]: per block, the smallest
 *               sparsity level at which it is active (device memory, read only).
 *   p_head      fp32 [n_heads]: each head's level p* (device memory).
 *   mask_bits   uint64 [n_heads][n_q_blocks][ceil(n_k_blocks/64)], written in full
 *               (padding bits zero).
 * The comparison is float32 and inclusive (T == p* keeps the block); NaN entries
 * are not kept.
 */
int mask_from_threshold_map(const float* thresholds, const float* p_head, int n_heads,
                            int n_q_blocks, int n_k_blocks, uint64_t* mask_bits,
                            hipStream_t stream);

/*
 * mask_resize -- resolution scaling of packed region maps (ScalingAttention section
 * 4.3.1, Eq. 7: bilinear interpolation at (u / s, v / s), s = nb_target / nb_base,
 * then a ceiling, so any overlap with an active region is kept).  On a binary map
 * this is exact in integers: target block (u, v) is kept iff a base sample with
 * positive bilinear weight is kept (samples at integer coordinates, clamped at the
 * last one).
 *   base_bits    uint64 [n_heads][nb_base][ceil(nb_base/64)], read only.
 *   target_bits  uint64 [n_heads][nb_target][ceil(nb_target/64)], written in full.
 */
int mask_resize(const uint64_t* base_bits, int n_heads, int nb_base, int nb_target,
                uint64_t* target_bits, hipStream_t stream);

/*
 * threshold_map_resize -- the threshold-map counterpart of mask_resize: each target
 * entry is the minimum of the base entries with positive bilinear weight (NaN
 * ignored), so I(resized T <= p) equals mask_resize of I(T <= p) for every p (a
 * ceiling on thresholds would drop activity instead of keeping it).
 *   base    fp32 [n_heads][nb_base][nb_base], read only.
 *   target  fp32 [n_heads][nb_target][nb_target], written; must not alias base.
 */
int threshold_map_resize(const float* base, int n_heads, int nb_base, int nb_target, float* target,
                         hipStream_t stream);

/*
 * attn_fidelity -- Hellinger distance and Fidelity Score between dense and sparse
 * attention on sampled query rows (ScalingAttention section 4.2.1, Eqs. 3 and 4;
 * rows drawn by block-wise stratified sampling, section 4.2.3).  For row i of head
 * h, P = softmax(scale * q_i K^T) over every key and P~ = the softmax over the keys
 * of the blocks its mask row keeps; H = (1/sqrt 2) * ||sqrt P - sqrt P~||_2.
 * Computed through the equivalent form H = sqrt((1 - rho) / (1 + sqrt rho)), rho =
 * the dense mass on kept keys, with fp32 logits from the bf16 inputs.
 *
 *   q, k           bf16 [n_heads][seq_len][head_dim], head_dim in {64, 128}; block 64.
 *   mask_bits      uint64 [n_heads][nb][W] as for sparse_attn_fwd.
 *   rows           int32 [n_heads][n_rows]: token index of each sampled query row
 *                  (device memory); an index outside [0, seq_len) yields NaN.
 *   row_hellinger  fp32 [n_heads][n_rows], written; 1 for a row that keeps nothing.
 *   head_fidelity  fp32 [n_heads] or NULL: 1 - mean of the head's row distances.
 * Uses the library's per-device scratch buffer for per-chunk partial sums (see
 * sparse_attn_fwd about overlapping calls).
 */
int attn_fidelity(const void* q, const void* k, const uint64_t* mask_bits, const int32_t* rows,
                  int n_heads, int seq_len, int head_dim, int block, int n_rows, float scale,
                  float* row_hellinger, float* head_fidelity, hipStream_t stream);

/*
 * permute_tokens -- token reordering for Hilbert-ordered attention (DFSAttn
 * abstract: tokens reordered along a Hilbert curve before block-sparse attention;
 * SCOPE abstract: attention is then taken over the selected original keys/values,
 * so the output is scattered back).
 *   inverse = 0:  y[h][i][:] = x[h][perm[i]][:]      (gather into curve order)
 *   inverse = 1:  y[h][perm[i]][:] = x[h][i][:]      (scatter back)
 *   x, y        [n_heads][seq_len][head_dim] of elem_bytes each (2 or 4); x != y.
 *   perm        int32 [seq_len], a permutation of [0, seq_len); out-of-range
 *               entries are skipped (their rows of y are left untouched).
 *   head_dim * elem_bytes must be a multiple of 16.
 */
int permute_tokens(const void* x, const int32_t* perm, int n_heads, int seq_len, int head_dim,
                   int elem_bytes, int inverse, void* y, hipStream_t stream);

/*
 * hilbert3d_order -- host-only, synchronous.  The token reordering that DFSAttn
 * applies before block-sparse attention (DFSAttn abstract: tokens reordered along a
 * Hilbert curve so that tokens close in space and time share blocks).  The page names
 * the curve only; perm_host (int32 [T*H*W], host memory) receives the token ids
 * (t-major id t*H*W + y*W + x) in increasing 3D Hilbert index, using J. Skilling's
 * transpose construction ("Programming the Hilbert curve", 2004) on the smallest 2^b
 * cube holding the grid, axes ordered (t, y, x).
 * T, H, W >= 1 and T*H*W < 2^31.
 */
int hilbert3d_order(int T, int H, int W, int32_t* perm_host);

/*
 * bsa_mfma_probe -- a measurement aid beside the attention path, not part of it.
 * The roofline of the attention kernels is the bf16 MFMA rate; the data-sheet peak
 * assumes a clock the chip does not hold under sustained MFMA load, so this probe
 * measures the rate on the GPU itself: every wave of two 4-wave workgroups per CU
 * runs `iterations` rounds of 16 v_mfma_f32_32x32x16_bf16 (four independent
 * accumulator chains) on register operands, with no memory traffic.
 *   sink        fp32 device buffer of sink_floats >= 512 * (compute units) floats; each
 *               thread writes one sum there (keeps the work observable).
 *   flops_host  host pointer; receives the flops the launch performs (time the call
 *               with events on `stream` for the rate).
 *   iterations  in [1, 1e7].
 * Argument errors are returned before any device call, except the sink size, which
 * is checked against the device's compute-unit count.
 */
int bsa_mfma_probe(int iterations, float* sink, long long sink_floats, double* flops_host,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
