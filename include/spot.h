/*
 * spot.h — C ABI of libspot: the SpotAttention decode hot path on gfx950 (MI355X).
 *
 * Source of the method: "SpotAttention: Plug-In Block-Sparse Routing for Pretrained
 * Long-Context Transformers" (Ahmad and Yun, KAIST). Section, equation and table
 * numbers below are that paper's.
 *
 * One decode step of one attention layer is three calls on one stream:
 *   spot_select_score  -> a score for every past KV block      (§2.1, §2.3)
 *   spot_select_topp   -> the per-query block set S_q           (§2.3, Eq. 7-8)
 *   spot_sparse_attn   -> exact softmax attention over S_q      (§2.3)
 * plus a prefill variant (spot_prefill_select_score, spot_prefill_select_topp,
 * spot_prefill_attn) for one tile or a whole sequence of query tiles with a causal
 * mask (§2.1 tile scoring; §6 notes the selector runs in the prefill regime), and
 * spot_quantize_selector, which encodes new selector keys into a quantised cache.
 *
 * Conventions shared by every call:
 *  - Every pointer argument is DEVICE memory owned by the caller (allocated and freed
 *    by the caller; the library keeps no pointer after the call returns). The library
 *    allocates nothing and never synchronises the device. Its only global state is
 *    the per-GPU scratch array of spot_sparse_attn_noalloc (declared below), whose
 *    device address it looks up once per GPU.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream. Every
 *    call validates its arguments on the host, then enqueues its kernels on `stream`
 *    and returns; results are ready when the stream reaches that point.
 *  - Arrays are dense and row-major with the innermost index last, as written.
 *  - Return value: SPOT_OK, or
 *      SPOT_ERR_INVALID      bad argument (null or misaligned pointer, size <= 0, values
 *                            out of range); nothing is enqueued;
 *      SPOT_ERR_UNSUPPORTED  a valid combination the library has no kernel for; nothing
 *                            is enqueued;
 *      SPOT_ERR_DEVICE       the HIP runtime refused a launch. A fault inside a kernel
 *                            surfaces at the caller's next synchronisation instead.
 *  - Counts named n_sink, n_rec, K_min, K_max are counts of BLOCKS.
 *  - NaN or infinite scores and inputs are not supported.
 */
#ifndef SPOT_H
#define SPOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPOT_API __attribute__((visibility("default")))

enum spot_status {
  SPOT_OK = 0,
  SPOT_ERR_INVALID = -1,
  SPOT_ERR_UNSUPPORTED = -2,
  SPOT_ERR_DEVICE = -3
};

/* Element formats. The quantised ones (§5.3 and Appendix G, Table 9: the selector's
 * queries and key cache at INT8, INT4, FP8 and FP4) are selector-only. */
enum spot_dtype {
  SPOT_F32 = 0,           /* IEEE binary32 */
  SPOT_BF16 = 1,          /* bfloat16 */
  SPOT_INT4_G32 = 2,      /* 4-bit two's-complement codes, two per byte (even element in
                             the low nibble), one IEEE binary16 scale per 32 consecutive
                             elements of d_idx: value = code * scale. 4.5 bits/element. */
  SPOT_INT8 = 3,          /* 8-bit two's-complement codes with ONE fp32 scale for the
                             whole tensor: value = code * scale. 8 bits/element (the
                             paper's 0.500x of BF16 leaves no room for group scales). */
  SPOT_FP8_E4M3 = 4,      /* FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
                             bits, subnormals, no infinities) with ONE fp32 scale for the
                             whole tensor: value = fp8 * scale. 8 bits/element. */
  SPOT_FP4_E2M1_G32 = 5   /* FP4 E2M1 codes (values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), two
                             per byte (even element in the low nibble), one E8M0 byte per
                             32 elements of d_idx (scale 2^(byte - 127)): value = fp4 *
                             scale. 4.25 bits/element, the footprint §5.3 prints. */
};

/*
 * spot_select_score — selector block scores (§2.1 score formula, §2.3 block maximum).
 *
 *   scores[b][blk] = max_{j < kpb} sum_{h < H_idx} sel_w[b][h] * ReLU( sum_i
 *                    q[b][h][i] * k[b][blk][j][h][i] )
 *
 * where q and k are the decoded values of sel_q and sel_k. No 1/sqrt(d_idx) factor (the
 * paper's formula has none; temperature 1, Table 3). Each of sel_q and sel_k is in one
 * of the spot_dtype formats, with its scale array:
 *   SPOT_F32, SPOT_BF16        elements [..][d_idx]; scale pointer NULL;
 *   SPOT_INT8, SPOT_FP8_E4M3   codes [..][d_idx]; scale -> one fp32 (4-byte aligned);
 *   SPOT_INT4_G32              codes uint8 [..][d_idx/2]; scales fp16 [..][d_idx/32]
 *                              (2-byte aligned);
 *   SPOT_FP4_E2M1_G32          codes uint8 [..][d_idx/2]; scales E8M0 bytes [..][d_idx/32].
 *   sel_q        [B][H_idx][..] in q_dtype, with sel_q_scale; 16-byte aligned.
 *   sel_w        [B][H_idx] fp32 mixing weights (any sign); 4-byte aligned.
 *   sel_k        [B][nb][kpb][H_idx][..] in k_dtype, with sel_k_scale; 16-byte aligned.
 *   scores       out fp32 [B][nb]; 4-byte aligned.
 *   kpb          selector keys per block (1 = one pooled key per block; the paper's
 *                per-token form is kpb = block size).
 * Errors: SPOT_ERR_INVALID for an unknown format, a missing scale of a quantised format,
 * or a scale given for fp32/bf16.
 * Supported: d_idx in {32, 64, 128}; H_idx a power of two with H_idx*d_idx/c <= 64,
 * c = 8 (fp32/bf16 keys), 16 (INT8/FP8 keys) or 32 (INT4/FP4 keys).
 */
SPOT_API int spot_select_score(const void* sel_q, int q_dtype, const void* sel_q_scale,
                               const float* sel_w, const void* sel_k, const void* sel_k_scale,
                               int k_dtype, float* scores, int B, int nb, int kpb, int H_idx,
                               int d_idx, void* stream);

/*
 * spot_select_topp — dual top-p block selection (§2.3, Eq. 7 and Eq. 8).
 *
 * Per query row b of scores [B][nb]:
 *   R     = {0 .. n_sink-1} u {nb-n_rec .. nb-1}, clipped to [0, nb); r = |R|;
 *   B_res = the other blocks. p~ = softmax over B_res of the scores (Eq. 7);
 *   order B_res by score descending, ties by lower block index (-0.0 == +0.0);
 *   k_p   = length of the shortest prefix whose cumulative p~ mass is >= p
 *           (p >= 1: all of B_res; p <= 0: none);
 *   k     = min(max(k_p, K_min - r, 0), K_max - r, |B_res|)   (|S| in [K_min, K_max]);
 *   S     = R u (first k of the order), written in ascending block order.
 * If B_res is empty, S is every block.
 * Static top-K (Eq. 6: the K highest-scoring blocks, no reserved blocks) is the case
 * p <= 0, n_sink = n_rec = 0, K_min = K_max = K.
 *   scores   fp32 [B][nb]; 4-byte aligned.
 *   sel_idx  out int32 [B][K_max]: S ascending, then -1 up to K_max; 4-byte aligned.
 *   sel_cnt  out int32 [B]: |S|.
 *   sel_mass optional out fp32 [B]: p~ mass of the k chosen residual blocks (NULL to
 *            skip). 0 when k = 0 or B_res is empty.
 * Errors: SPOT_ERR_INVALID when p is not finite, n_sink/n_rec/K_min < 0, or
 * K_max < r (the reserved set would not fit). Supported: 1 <= nb <= 16384.
 * Each block's mass exp(s - max) is rounded to 2^-29 fixed point (relative error near
 * 1e-7) and masses are summed as integers, exactly, so the result does not depend on
 * thread scheduling.
 */
SPOT_API int spot_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                              float* sel_mass, int B, int nb, float p, int K_min, int K_max,
                              int n_sink, int n_rec, void* stream);

/*
 * spot_quantize_selector — encode selector keys into a quantised cache format: the
 * write side of §5.3 (the selector is trained in BF16 and its key cache quantised at
 * inference), e.g. to append the new token's selector key to the cache (point codes
 * and scales at its row).
 *
 * Rows are split into groups of 32 consecutive elements:
 *   SPOT_INT4_G32      scale = fp16(amax / 7) (fp32 quotient, rounded to nearest even);
 *                      code = clamp(rne(x / scale), -8, 7); all codes 0 when scale = 0.
 *   SPOT_FP4_E2M1_G32  scale = 2^e, e the smallest integer with amax <= 6 * 2^e, clamped
 *                      to [-127, 127] (-127 when amax = 0), stored as the byte e + 127;
 *                      code = the E2M1 value nearest to x / 2^e, ties to the even code.
 *   SPOT_INT8          code = clamp(rne(x / s), -127, 127) with the cache's fixed scale s.
 *   SPOT_FP8_E4M3      y = clamp(x / s, -448, 448); code = the E4M3 value nearest to y,
 *                      ties to the even code.
 * x / scale is a correctly rounded fp32 division; rne rounds to nearest, ties to even;
 * sign bits follow x (a negative value rounding to zero gives -0 in FP8 and FP4).
 *   src           [n_rows][row_len] in src_dtype (SPOT_F32 or SPOT_BF16); 16-byte aligned.
 *   row_len       a multiple of 32 (row_len = H_idx * d_idx for one selector key).
 *   codes         out [n_rows][row_len / 2] (4-bit formats) or [n_rows][row_len] bytes
 *                 (8-bit formats); 16-byte aligned.
 *   scales        out, group formats only: [n_rows][row_len / 32] fp16 (INT4, 2-byte
 *                 aligned) or E8M0 bytes (FP4); must be NULL for the 8-bit formats.
 *   tensor_scale  in, 8-bit formats only: the cache's one fp32 scale s (device, 4-byte
 *                 aligned); must be NULL for the group formats.
 * Errors: SPOT_ERR_INVALID for a bad pointer, size or format, or a scale argument that
 * does not match the format.
 */
SPOT_API int spot_quantize_selector(const void* src, int src_dtype, int n_rows, int row_len,
                                    int fmt, void* codes, void* scales,
                                    const float* tensor_scale, void* stream);

/*
 * spot_sparse_attn_workspace_bytes — size of the workspace spot_sparse_attn needs for
 * these arguments (the same values passed to it): the split-K partial results of the
 * split plan the call will use, B * Hq * nslot * (d + 2) fp32 values, nslot being the
 * partial-result slots of one (query, head). Returns 0 for a non-positive size, an
 * unknown kv_dtype or a shape spot_sparse_attn does not support.
 */
SPOT_API size_t spot_sparse_attn_workspace_bytes(int B, int Hq, int Hkv, int d, int K_max,
                                                 int block, int kv_dtype);

/*
 * spot_sparse_attn — decode attention over the selected blocks only (§2.3: the layer
 * attends only to keys in blocks of S_q; one S_q per query, shared by all heads).
 *
 * For query b and head hq (KV head g = hq / (Hq/Hkv)):
 *   out[b][hq] = sum_t softmax_t(sm_scale * q[b][hq] . K[b][g][t]) V[b][g][t]
 * over the tokens t < L whose block t / block is one of sel_idx[b][0 .. sel_cnt[b]-1].
 * Entries outside [0, ceil(L/block)) are ignored; entries must not repeat. A row with
 * no valid entry gets a zero output.
 *   q            [B][Hq][d]; K and V [B][Hkv][L][d]; out [B][Hq][d]; all of kv_dtype
 *                (SPOT_F32 or SPOT_BF16; bf16 output is rounded to nearest even);
 *                16-byte aligned.
 *   sel_idx      int32 [B][K_max], sel_cnt int32 [B] (as written by spot_select_topp).
 *   workspace    device scratch of at least spot_sparse_attn_workspace_bytes(B, Hq, Hkv,
 *                d, K_max, block, kv_dtype) bytes, 256-byte aligned; contents on entry
 *                do not matter. Calls that run at the same time must not share a
 *                workspace.
 * Split-K: each work-group reduces a run of selected blocks with an online softmax (for
 * bf16 at batch 2..64 the runs are cut from all queries' lists together, so rows with
 * very different counts stay balanced); a second kernel merges the runs of every
 * (b, head) in run order, so the result is deterministic.
 * Supported: d in {64, 128}; block in {16, 32, 64, 128} tokens (16 is the paper's page
 * size, Appendix A Table 3); Hq % Hkv == 0 with Hq/Hkv in {1, 2, 4, 8}.
 */
SPOT_API int spot_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                              int kv_dtype, const int32_t* sel_idx, const int32_t* sel_cnt,
                              int K_max, void* out, void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int d, int L, int block,
                              float sm_scale, void* stream);

/*
 * spot_sparse_attn_noalloc — for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments, checks and result as spot_sparse_attn, without the workspace. The partial
 * results go to a device array of SPOT_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on, from when its code is loaded there until the process ends; the
 * first call for a GPU looks up that GPU's copy. No call allocates memory.
 * Errors: as spot_sparse_attn; SPOT_ERR_UNSUPPORTED when the workspace these sizes need
 * (spot_sparse_attn_workspace_bytes) exceeds the array (at 32 query heads of 128 dims
 * and 256 selected blocks, batches up to 30); SPOT_ERR_DEVICE when the array's address
 * cannot be found. All calls on one GPU share its array and nothing in it has to start
 * at a given value: calls that can overlap on one GPU (other streams, other host
 * threads) race with each other, and the caller must order them.
 */
#define SPOT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
SPOT_API int spot_sparse_attn_noalloc(const void* q, const void* k_cache,
                                      const void* v_cache, int kv_dtype,
                                      const int32_t* sel_idx, const int32_t* sel_cnt,
                                      int K_max, void* out, int B, int Hq, int Hkv, int d,
                                      int L, int block, float sm_scale, void* stream);

/*
 * Prefill (§2.1 tile scoring; §6 names sparse prefill as the open direction). A batch
 * element holds T consecutive queries at positions q_pos0 .. q_pos0+T-1, cut into
 * tiles of Tq queries (the last one shorter): n_tiles = ceil(T / Tq). Tile t holds
 * queries t*Tq .. min((t+1)*Tq, T)-1 and sees the blocks whose first token is at or
 * before its last query's position: nb_t = ceil((q_pos0 + min((t+1)*Tq, T)) / block).
 * T == Tq is a single tile. Per-tile arrays are [B][n_tiles][..].
 */

/*
 * spot_prefill_select_score — tile block scores (§2.1: one score per query-block x
 * key-block tile; §2.3 block maximum). For tile t of batch element b and blk < nb_t:
 *   scores[b][t][blk] = max over the tile's queries i that see blk (blk*block <=
 *                       position of i) of max_{j<kpb} sum_h sel_w[b][i][h] *
 *                       ReLU(sel_q[b][i][h] . sel_k[b][blk][j][h])
 * Entries blk >= nb_t of a row are not written. Computed as one matrix product per
 * selector head on the MFMA units.
 *   sel_q   [B][T][H_idx][d_idx] (q_dtype), sel_w fp32 [B][T][H_idx];
 *   sel_k   [B][nb_cache][kpb][H_idx][..] in k_dtype with sel_k_scale, laid out as for
 *           spot_select_score (16-byte aligned): bf16, or the quantised cache formats
 *           SPOT_INT4_G32, SPOT_FP4_E2M1_G32, SPOT_INT8, SPOT_FP8_E4M3 (§5.3: the
 *           quantised selector's savings apply in prefill too);
 *   scores  out fp32 [B][n_tiles][nb_seq], nb_seq = ceil((q_pos0 + T) / block).
 * Errors: SPOT_ERR_INVALID when nb_seq > nb_cache, q_pos0 < 0 or q_pos0 + T > INT_MAX,
 * or as spot_select_score for the formats and scales.
 * Supported: d_idx in {32, 64, 128}; bf16 queries; keys in any format but fp32;
 * 1 <= Tq <= 128; B * n_tiles <= 65535.
 */
SPOT_API int spot_prefill_select_score(const void* sel_q, int q_dtype, const float* sel_w,
                                       const void* sel_k, const void* sel_k_scale,
                                       int k_dtype, float* scores, int B, int T, int Tq,
                                       int q_pos0, int nb_cache, int kpb, int H_idx,
                                       int d_idx, int block, void* stream);

/*
 * spot_prefill_select_topp — dual top-p per tile: row (b, t) of scores [B][n_tiles]
 * [nb_seq] is treated as spot_select_topp treats a row of nb_t blocks, so its recency
 * window is the n_rec blocks ending at the tile's diagonal (Table 3: recency "per
 * tile"), and its sink the first n_sink blocks.
 *   sel_idx  out int32 [B][n_tiles][K_max]; sel_cnt out [B][n_tiles]; sel_mass optional
 *            out [B][n_tiles].
 * Errors and ordering as spot_select_topp (K_max must hold the largest reserved set);
 * also SPOT_ERR_INVALID when q_pos0 + T > INT_MAX.
 * Supported: nb_seq <= 16384.
 */
SPOT_API int spot_prefill_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                                      float* sel_mass, int B, int T, int Tq, int q_pos0,
                                      int block, float p, int K_min, int K_max, int n_sink,
                                      int n_rec, void* stream);

/*
 * spot_prefill_attn — causal block-sparse attention for the tiles of a prefill.
 *
 * Query i of tile t (position q_pos0 + i) attends to the tokens s <= q_pos0 + i, s < L,
 * whose block is in sel_idx[b][t][0 .. sel_cnt[b][t]-1] (one set for the whole tile
 * and every head). Rows with no visible selected token get zeros.
 *   q    [B][Hq][T][d]; K, V [B][Hkv][L][d]; out [B][Hq][T][d]; kv_dtype SPOT_BF16;
 *        16-byte aligned. q_pos0 + T <= L (the queries' own tokens are in the cache).
 * Supported: d == 128, block == 64, 1 <= Tq <= 128, K_max <= 8192, Hq/Hkv in
 * {1, 2, 4, 8}, B * n_tiles <= 65535.
 */
SPOT_API int spot_prefill_attn(const void* q, const void* k_cache, const void* v_cache,
                               int kv_dtype, const int32_t* sel_idx, const int32_t* sel_cnt,
                               int K_max, void* out, int B, int Hq, int Hkv, int T, int Tq,
                               int q_pos0, int d, int L, int block, float sm_scale,
                               void* stream);

/* Human-readable name of a status code (static storage; never NULL). */
SPOT_API const char* spot_status_string(int status);

/* ABI version of this library (incremented on any incompatible change). */
SPOT_API int spot_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPOT_H */
