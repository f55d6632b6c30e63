/*
 * kvq.h -- rotated residual/product vector quantisation of a transformer KV
 * cache, and single-token decode attention that reads the codes directly.
 * C ABI of libkvq.so (gfx950 / AMD Instinct MI355X).
 *
 * The method (sources are the web pages these calls restate):
 *   - Rotation: every head vector is multiplied by the orthonormal Sylvester
 *     Walsh-Hadamard matrix H_D (natural order, entries +-1/sqrt(D)) to spread
 *     its energy before quantisation ("ZeroKV-Neo 4.0.0", Architecture, FWHT
 *     energy spreading; "VeloxQuant-MLX 0.5.1", VecInfer, Walsh-Hadamard
 *     rotation).
 *   - Encode: the rotated vector is split into G groups of dsub = D/G dims;
 *     each group runs S greedy residual stages, each picking the nearest entry
 *     (squared Euclidean distance, lowest index on exact ties) of that
 *     stage's C-entry codebook and subtracting it ("VQKV" summary,
 *     2. Methodology, Residual Simple Vector Quantization; "VeloxQuant-MLX
 *     0.5.1", VecInfer product VQ with one codebook per sub-vector).
 *   - Reconstruct: the sum over stages of the chosen entries, optionally
 *     unrotated by H_D ("VQKV" summary, RSimVQ reconstruction;
 *     "VeloxQuant-MLX 0.5.1", Architecture, decode then unrotate).
 *   - Decode attention: the query is rotated once (the inverse rotation is
 *     absorbed into the query, "VeloxQuant-MLX 0.5.1", VecInfer), scored
 *     against the codes through a per-query table LUT[s][g][c] = q_rot_g .
 *     C_sg[c] without materialising K ("Differential-KV" README, Decode &
 *     Prefill Innovations, query scoring in the compressed domain), and the
 *     coded part is merged with a dense fp16 window of the most recent
 *     tokens by an fp32 log-sum-exp combine (same README, Flash-Style LSE
 *     Combine; "VQKV" summary, 3. Inference Integration, local sliding
 *     window).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates device memory and keeps no state beyond a
 *     thread-local last-error value.  Scratch memory is passed in as a
 *     caller-owned workspace whose size the matching *_workspace_size call
 *     reports.
 *   - Every argument is validated before any HIP call.  On error nothing is
 *     launched, outputs are untouched and a status other than KVQ_OK is
 *     returned.
 *   - Calls are asynchronous: they enqueue kernels on `stream` and return.
 *     Results are valid once the caller synchronises that stream.
 *   - Tensors are dense, row-major, and every pointer must be 16-byte
 *     aligned.
 *   - Codes are one byte each (C <= 256); a vector's codes are stored
 *     stage-major: code(s, g) at byte s*G + g of its S*G-byte row.
 *   - Codebooks are float32 [S][G][C][dsub].
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef KVQ_API
#define KVQ_API __attribute__((visibility("default")))
#endif

/* Status codes, element types and level kinds are plain 32-bit integers with
 * named values (not enum types), so any value a caller passes is data that a
 * call checks and rejects, never an out-of-range enum. */
typedef int32_t kvq_status;
enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,        /* a required pointer is NULL                      */
  KVQ_ERR_SHAPE = 2,       /* sizes inconsistent or out of range              */
  KVQ_ERR_UNSUPPORTED = 3, /* valid request the library has no kernel for    */
  KVQ_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
  KVQ_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required         */
  KVQ_ERR_DTYPE = 6,       /* unknown element type                            */
  KVQ_ERR_HIP = 7          /* a HIP launch failed; see kvq_last_hip_error()   */
};

typedef int32_t kvq_dtype;
enum { KVQ_F32 = 0, KVQ_BF16 = 1, KVQ_F16 = 2 };

/* Quantiser shape.  head_dim D in {64, 128, 256}; n_groups G divides D;
 * dsub = D/G a power of two in [8, 128]; 1 <= n_stages S <= 8;
 * 1 <= n_codewords C <= 256. */
typedef struct {
  int32_t head_dim;
  int32_t n_groups;
  int32_t n_stages;
  int32_t n_codewords;
} kvq_vq_desc;

/* Decode attention shape.  One query token per (sequence, query head).
 * Query head h reads KV head h / (n_q_heads / n_kv_heads).  The cache of a
 * (sequence, KV head) holds n_code_tokens coded tokens followed by n_window
 * fp16 tokens on one position axis; either count may be 0, not both.
 * softmax_scale <= 0 selects 1/sqrt(head_dim).  code_stride / window_stride:
 * token rows allocated per (sequence, KV head) in the code / window buffers
 * (a cache grown in place by kvq_window_flush); 0 means dense (= the count). */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t n_code_tokens;
  int32_t n_window;
  kvq_vq_desc vq;          /* vq.head_dim is the attention head_dim */
  float softmax_scale;
  int32_t code_stride;     /* 0 or >= n_code_tokens */
  int32_t window_stride;   /* 0 or >= n_window */
} kvq_attn_desc;

/* Flags */
#define KVQ_INPUT_PRE_ROTATED 0x1u /* kvq_encode: x is already H_D x          */
#define KVQ_UNROTATE          0x2u /* kvq_decode_reconstruct: output H_D x_rot */
#define KVQ_ENCODE_GENERIC    0x4u /* kvq_encode: force the plain fp32 kernel  */
#define KVQ_CODEBOOKS_PACKED  0x8u /* kvq_encode: workspace already holds these
                                      codebooks packed (skip the packing pass) */

/* y = H_D x for n_rows rows of length dim (dim in {64, 128, 256}).
 * x: [n_rows][dim] of type xt; y: [n_rows][dim] float32.  H_D is symmetric
 * and orthonormal, so applying it twice returns the input.  x == y is
 * allowed when xt == KVQ_F32 (in place).  n_rows == 0 is a no-op. */
KVQ_API kvq_status kvq_rotate(const void* x, kvq_dtype xt, float* y, int64_t n_rows,
                      int32_t dim, hipStream_t stream);

/* Workspace bytes kvq_encode needs for n_books codebooks of shape *vq
 * (packed bf16 operand copies of the codebooks).  May be 0. */
KVQ_API kvq_status kvq_encode_workspace_size(const kvq_vq_desc* vq, int64_t n_books,
                                     size_t* bytes);

/* Encode rows [0, n_rows) of every sequence into codes.
 * x:         [n_books][n_seq][seq_stride][D] of type xt (original domain,
 *            or already rotated with KVQ_INPUT_PRE_ROTATED);
 * codebooks: [n_books][S][G][C][dsub] float32 -- book b codes the vectors of
 *            x[b];
 * codes:     [n_books][n_seq][n_rows][S][G] uint8 (output).
 * Requires n_rows <= seq_stride.  Any of n_books, n_seq, n_rows may be 0
 * (no-op).  On the MFMA path the codebooks are first packed into the
 * workspace (bf16 operand pieces and norms); the codebooks of a layer are
 * constants, so a caller may pack once and pass KVQ_CODEBOOKS_PACKED on later
 * calls with the same codebooks and the same workspace, which skips that
 * pass.  codebooks is still required (the generic kernel reads it and
 * ignores the flag).  Codes equal the float64 greedy search except where the best two
 * squared distances of a stage are within a relative 1e-4 of each other,
 * where either choice may be returned. */
KVQ_API kvq_status kvq_encode(const void* x, kvq_dtype xt, const kvq_vq_desc* vq,
                      int64_t n_books, int64_t n_seq, int64_t seq_stride,
                      int64_t n_rows, const float* codebooks, uint8_t* codes,
                      uint32_t flags, void* workspace, size_t ws_bytes,
                      hipStream_t stream);

/* out[b][n] = sum over stages s (ascending) of codebooks[b][s][g][z(s,g)]
 * placed at dims g*dsub.., accumulated in float64 and rounded once to
 * float32 (rotated domain); with KVQ_UNROTATE, H_D is applied afterwards.
 * codes: [n_books][n_per_book][S][G] uint8; out: [n_books][n_per_book][D]
 * float32.  Codes >= C are out of range: they read entry C-1 (no fault). */
KVQ_API kvq_status kvq_decode_reconstruct(const uint8_t* codes, const kvq_vq_desc* vq,
                                  int64_t n_books, int64_t n_per_book,
                                  const float* codebooks, float* out,
                                  uint32_t flags, hipStream_t stream);

/* Workspace bytes kvq_attend_decode needs for shape *a. */
KVQ_API kvq_status kvq_attend_workspace_size(const kvq_attn_desc* a, size_t* bytes);

/* Single-token decode attention.
 * q:       [B][Hq][D] float32, original domain;
 * k_codes, v_codes: [B][Hkv][code_stride][S][G] uint8, rows [0, Tc) read
 *          (Tc = n_code_tokens);
 * k_cb, v_cb: [S][G][C][dsub] float32 (one codebook set for K, one for V);
 * k_win, v_win: [B][Hkv][window_stride][D] IEEE fp16 bit patterns, rows
 *          [0, W) read (W = n_window; may be
 *          NULL when W == 0);
 * out:     [B][Hq][D] float32 = softmax(scale * K q) V over the Tc coded
 *          tokens (K, V = H_D reconstruction) followed by the W window tokens;
 * workspace: at least kvq_attend_workspace_size bytes.
 * Codes >= C read entry C-1 (no fault). */
KVQ_API kvq_status kvq_attend_decode(const kvq_attn_desc* a, const float* q,
                             const uint8_t* k_codes, const uint8_t* v_codes,
                             const float* k_cb, const float* v_cb,
                             const uint16_t* k_win, const uint16_t* v_win,
                             float* out, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* Bytes of the device array kvq_attend_decode_noalloc works in, per GPU. */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Decode attention for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, layouts, results and checks as kvq_attend_decode,
 * without a workspace: the call works in a device array the library holds,
 * KVQ_NOALLOC_SCRATCH_BYTES on each GPU it runs on, from the first call on
 * that GPU until the process ends; it calls no allocator.  A shape whose
 * kvq_attend_workspace_size exceeds that is KVQ_ERR_WORKSPACE (nothing
 * launched).  A stream of a device other than the current one is
 * KVQ_ERR_UNSUPPORTED.  Every call on one GPU uses the same array, which
 * keeps the last call's contents: calls that overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.  Each
 * call writes every byte of it that it reads, so it needs no clearing. */
KVQ_API kvq_status kvq_attend_decode_noalloc(const kvq_attn_desc* a, const float* q,
                             const uint8_t* k_codes, const uint8_t* v_codes,
                             const float* k_cb, const float* v_cb,
                             const uint16_t* k_win, const uint16_t* v_win,
                             float* out, hipStream_t stream);

/* Bytes one layer's compressed cache of shape *a holds ("VeloxQuant-MLX
 * 0.5.1", Quick start: the cache reports its memory use; its results count
 * compression as code bytes against fp16 K and V).  K and V together, over
 * the n_code_tokens coded and n_window window tokens of every (sequence, KV
 * head):
 *   code_bytes     = 2 * B * Hkv * n_code_tokens * S * G   (one byte per code)
 *   window_bytes   = 2 * B * Hkv * n_window * D * 2        (fp16 rows)
 *   codebook_bytes = 2 * S * G * C * dsub * 4              (float32 K and V sets)
 *   dense_bytes    = 2 * B * Hkv * (n_code_tokens + n_window) * D * 2
 *                    (the same tokens held as a dense fp16 cache).
 * Rows allocated beyond the counts (code_stride, window_stride) are not
 * counted.  Host arithmetic only: no HIP call.  Every output pointer is
 * required.  Shape checks are those of kvq_attend_workspace_size, except that
 * both counts may be 0; a total past 2^63 is KVQ_ERR_SHAPE. */
KVQ_API kvq_status kvq_cache_bytes(const kvq_attn_desc* a, uint64_t* code_bytes,
                                   uint64_t* window_bytes, uint64_t* codebook_bytes,
                                   uint64_t* dense_bytes);

/* ---------------------------------------------------------------------------
 * Streaming window ("VeloxQuant-MLX 0.5.1", Quick start: a cache grown one
 * token at a time by append; "ZeroKV-Neo 4.0.0", profiling output: periodic
 * flush_quantize; "VQKV" summary, 3. Inference Integration: a local window of
 * recent tokens kept uncompressed, older ones compressed).  The caller keeps
 * the counts (n_window, n_code); buffers have fixed capacities:
 *   k_win, v_win:     [B][Hkv][window_cap][D] fp16 bit patterns;
 *   k_codes, v_codes: [B][Hkv][code_cap][S][G] uint8.
 * kvq_attend_decode reads such a cache with code_stride = code_cap and
 * window_stride = window_cap.
 * ------------------------------------------------------------------------ */

/* Writes k_new / v_new ([B][Hkv][D] fp16) into row n_window of every
 * (sequence, KV head) window.  Requires 0 <= n_window < window_cap and
 * head_dim in {64, 128, 256}. */
KVQ_API kvq_status kvq_window_append(int32_t batch, int32_t n_kv_heads, int32_t head_dim,
                             int32_t window_cap, int32_t n_window,
                             const uint16_t* k_new, const uint16_t* v_new,
                             uint16_t* k_win, uint16_t* v_win, hipStream_t stream);

/* Workspace bytes kvq_window_flush needs (packed K and V codebooks; may be 0). */
KVQ_API kvq_status kvq_window_flush_workspace_size(const kvq_vq_desc* vq, size_t* bytes);

/* Flush: the oldest n_flush window tokens of every (sequence, KV head),
 * rows [0, n_flush), are encoded exactly as kvq_encode would (rotation, then
 * the greedy residual stages; K with k_cb, V with v_cb, each [S][G][C][dsub]
 * float32) and their codes written to rows [n_code, n_code + n_flush); the
 * remaining window rows [n_flush, n_window) then move to rows
 * [0, n_window - n_flush).  Requires 0 <= n_flush <= n_window <= window_cap
 * and n_code + n_flush <= code_cap; n_flush == 0 is a no-op.  The caller's
 * counts become n_window - n_flush and n_code + n_flush.  flags: 0 or
 * KVQ_CODEBOOKS_PACKED (the workspace still holds the K and V codebooks
 * packed by an earlier flush with the same codebooks). */
KVQ_API kvq_status kvq_window_flush(const kvq_vq_desc* vq, int32_t batch, int32_t n_kv_heads,
                            int32_t window_cap, int32_t n_window, int32_t n_flush,
                            uint16_t* k_win, uint16_t* v_win, int32_t code_cap,
                            int32_t n_code, uint8_t* k_codes, uint8_t* v_codes,
                            const float* k_cb, const float* v_cb, uint32_t flags,
                            void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Dual transform ("VeloxQuant-MLX 0.5.1", VecInfer section: per-channel smooth
 * scaling by lambda_i = sqrt(max |K_i|) ahead of the Walsh-Hadamard rotation,
 * its inverse absorbed into the query).  Keys are coded as H_D (k / lambda)
 * (channel-wise division); decode multiplies the query by lambda before
 * rotating it, so q . k is unchanged.  Values and the fp16 window keep the
 * plain path (the window holds the original keys and is scored with the
 * original query).
 *
 * Factors live in a float32 device array [n_books][n_scale][D]: the vectors of
 * sequence n of book b use row n % n_scale of book b.  For a cache laid out
 * [B][Hkv][T][D] (sequence n = b * Hkv + kv), n_scale = Hkv gives one row per
 * KV head shared by the batch, n_scale = B * Hkv one per (sequence, KV head)
 * and n_scale = 1 one per book.  Factors must be positive and finite; other
 * values give unspecified codes and outputs (no fault).
 * ------------------------------------------------------------------------ */
typedef struct {
  const float* factors;    /* [n_books][n_scale][D] float32, device, 16-byte aligned */
  int32_t n_scale;         /* >= 1 */
} kvq_smooth_desc;

/* Calibrates factors from the rows [0, n_rows) of every sequence of
 * x [n_books][n_seq][seq_stride][D] (type xt, original domain):
 * factors[b][j][i] = sqrt(max |x[b][n][t][i]|) over every sequence n with
 * n % n_scale == j and every row t < n_rows, rounded to float32; a channel
 * whose maximum is 0, or a row j no sequence maps to, gets 1.  A NaN in x
 * gives NaN factors in its channel.  factors: [n_books][n_scale][D] float32
 * (output; also the kernels' reduction target, so it may not overlap x).
 * Requires head_dim in {64, 128, 256}, n_scale >= 1, n_rows <= seq_stride;
 * n_books == 0 is a no-op; n_seq == 0 or n_rows == 0 writes ones. */
KVQ_API kvq_status kvq_smooth_calibrate(const void* x, kvq_dtype xt, int32_t head_dim,
                                int64_t n_books, int64_t n_seq, int64_t seq_stride,
                                int64_t n_rows, int32_t n_scale, float* factors,
                                hipStream_t stream);

/* kvq_encode of x / factors: each vector divided channel-wise by its
 * sequence's factor row before the rotation and the residual stages.  Same
 * arguments, layouts, workspace and flags as kvq_encode except that
 * KVQ_INPUT_PRE_ROTATED is refused (the division acts on the original
 * channels).  smooth->factors: [n_books][n_scale][D]. */
KVQ_API kvq_status kvq_encode_smooth(const void* x, kvq_dtype xt, const kvq_vq_desc* vq,
                             int64_t n_books, int64_t n_seq, int64_t seq_stride,
                             int64_t n_rows, const kvq_smooth_desc* smooth,
                             const float* codebooks, uint8_t* codes, uint32_t flags,
                             void* workspace, size_t ws_bytes, hipStream_t stream);

/* Original-domain reconstruction of codes made by kvq_encode_smooth:
 * out[b][n][t] = factors[b][n % n_scale] * (H_D sum of the chosen entries),
 * the unrotation first, then the channel-wise product.
 * codes: [n_books][n_seq][n_rows][S][G] uint8; out: [n_books][n_seq][n_rows][D]
 * float32.  Codes >= C read entry C-1 (no fault). */
KVQ_API kvq_status kvq_decode_reconstruct_smooth(const uint8_t* codes, const kvq_vq_desc* vq,
                                         int64_t n_books, int64_t n_seq, int64_t n_rows,
                                         const float* codebooks,
                                         const kvq_smooth_desc* smooth, float* out,
                                         hipStream_t stream);

/* kvq_attend_decode over a cache whose coded keys were smoothed: the table
 * of KV head kv of sequence b is built from H_D (factors[(b * Hkv + kv) %
 * n_scale] * q) (one book: factors [n_scale][D]).  Window keys are original;
 * everything else as kvq_attend_decode, same workspace size. */
KVQ_API kvq_status kvq_attend_decode_smooth(const kvq_attn_desc* a, const float* q,
                                    const uint8_t* k_codes, const uint8_t* v_codes,
                                    const float* k_cb, const float* v_cb,
                                    const kvq_smooth_desc* k_smooth,
                                    const uint16_t* k_win, const uint16_t* v_win,
                                    float* out, void* workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* kvq_window_flush whose flushed keys are coded as by kvq_encode_smooth, the
 * window of (sequence b, KV head kv) using factor row (b * Hkv + kv) %
 * n_scale (one book: factors [n_scale][D]); values as in kvq_window_flush. */
KVQ_API kvq_status kvq_window_flush_smooth(const kvq_vq_desc* vq, int32_t batch,
                                   int32_t n_kv_heads, int32_t window_cap, int32_t n_window,
                                   int32_t n_flush, uint16_t* k_win, uint16_t* v_win,
                                   int32_t code_cap, int32_t n_code, uint8_t* k_codes,
                                   uint8_t* v_codes, const float* k_cb, const float* v_cb,
                                   const kvq_smooth_desc* k_smooth, uint32_t flags,
                                   void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Codebook fitting ("VeloxQuant-MLX 0.5.1", VecInfer section: the product-VQ
 * codebooks are K-means codebooks trained before use, its allocator list
 * naming train_codebook; "VQKV" summary, 2. Methodology: trained residual
 * stage codebooks).  K-means (Lloyd) on a sample, stage by stage: on the
 * residuals the already fitted earlier stages leave, n_iter times {assign
 * every vector to its nearest entry of stage s, group g (as kvq_encode does);
 * move every entry to the mean of its vectors, an entry with no vector keeping
 * its value}; then one more assignment with the fitted entries, whose
 * subtraction gives the next stage's residuals.
 * ------------------------------------------------------------------------ */
#define KVQ_FIT_MAX_VECTORS (((int64_t)1) << 24)

/* Workspace bytes kvq_codebook_fit needs for n_vectors sample vectors
 * (4*D + S*G bytes per vector plus fixed parts).  n_vectors <= 2^24. */
KVQ_API kvq_status kvq_codebook_fit_workspace_size(const kvq_vq_desc* vq, int64_t n_vectors,
                                           size_t* bytes);

/* Fits codebooks [S][G][C][dsub] float32 IN PLACE (in: the starting entries,
 * out: the fitted ones) on the sample rows [0, n_rows) of every sequence of
 * x [n_seq][seq_stride][D] (type xt, original domain; rotated inside, and
 * divided by smoothing factors first when smooth is not NULL: one book,
 * factors [n_scale][D], sequence n using row n % n_scale, as
 * kvq_encode_smooth).  n_seq * n_rows <= 2^24 vectors; 0 <= n_iter <= 100000
 * (0: the entries are left as they are).  The entry means are sums of the
 * float32 residuals in 64-bit fixed point (F fraction bits with every term
 * below 2^(62 - ceil(log2 N)); a residual is taken exactly when it is a
 * multiple of 2^-F, else truncated toward zero), divided in float64 and
 * rounded once to float32; integer sums do not depend on the order, so
 * repeated calls give identical codebooks.  Assignments follow kvq_encode's
 * rule (near ties within a relative 1e-4 may go either way).  Non-finite
 * inputs give unspecified entries. */
KVQ_API kvq_status kvq_codebook_fit(const void* x, kvq_dtype xt, const kvq_vq_desc* vq,
                            int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                            const kvq_smooth_desc* smooth, int32_t n_iter,
                            float* codebooks, void* workspace, size_t ws_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Scalar residual variant ("VeloxQuant-MLX 0.5.1": Architecture, TurboQuantRVQ
 * pipeline -- rotate, stage-1 Gaussian Lloyd-Max scalar quantiser, residual,
 * stage-2 Laplacian Lloyd-Max, the indices only, decode by summing the two
 * levels and unrotating; throughput journey -- the index counted over decision
 * boundaries instead of an argmin; module table -- dsa.bit_pack sub-byte
 * index packing; the allocator's bit choices include 3 bits).  bits b in
 * 1..4: 2^b levels per stage.
 *
 * Codes: a vector's row is [stage-1 bytes][stage-2 bytes], D*b/8 bytes each;
 * each stage is one bit string, least significant bit first: bit t of element
 * i is bit i*b + t of the stage's bytes (for b in {1, 2, 4}: bits
 * [(i mod k)*b, (i mod k)*b + b) of byte i / k, k = 8/b; for b = 3 an element
 * may straddle two bytes).  Levels: float32 [n_books][2][2^b], each stage's
 * levels strictly increasing (stage 1 for the rotated element, stage 2 for
 * its residual); other orders give unspecified codes (no fault).  For b in
 * {1, 2, 4} a byte of stage s is also a code of the product codebook
 * kvq_scalar_product_codebook writes, so kvq_attend_decode reads scalar codes
 * with vq = {D, G = D*b/8, S = 2, C = 256}; 3-bit codes have no whole
 * elements per byte and are encoded and reconstructed only.
 * ------------------------------------------------------------------------ */
typedef int32_t kvq_levels_kind;
enum { KVQ_LEVELS_GAUSSIAN = 0, KVQ_LEVELS_LAPLACIAN = 1 };

/* Host call (no GPU): the 2^bits levels (ascending) of the Lloyd-Max
 * quantiser for the unit-variance Gaussian or Laplacian density, iterated to a
 * fixed point with the cell moments in closed form; *distortion (if not NULL)
 * receives its mean squared error.  bits in 1..4; levels: host [2^bits]. */
KVQ_API kvq_status kvq_lloyd_max(kvq_levels_kind kind, int32_t bits, double* levels,
                         double* distortion);

/* y = H_D x (unless KVQ_INPUT_PRE_ROTATED); per element z1 = number of
 * stage-1 thresholds (float32 midpoints of neighbouring levels) strictly below
 * y, r = y - levels1[z1], z2 likewise on r with the stage-2 levels; packed as
 * above.  x: [n_books][n_seq][seq_stride][D] of type xt, rows [0, n_rows);
 * levels: [n_books][2][2^b]; codes: [n_books][n_seq][n_rows][2][D*b/8].
 * Equals the nearest level per stage except where an element lies within
 * float32 rounding of a threshold. */
KVQ_API kvq_status kvq_scalar_encode(const void* x, kvq_dtype xt, int32_t head_dim, int32_t bits,
                             int64_t n_books, int64_t n_seq, int64_t seq_stride,
                             int64_t n_rows, const float* levels, uint8_t* codes,
                             uint32_t flags, hipStream_t stream);

/* out[b][n] = levels1[z1] + levels2[z2] per element (float32), then H_D with
 * KVQ_UNROTATE.  codes: [n_books][n_per_book][2][D*b/8]; out:
 * [n_books][n_per_book][D] float32. */
KVQ_API kvq_status kvq_scalar_decode_reconstruct(const uint8_t* codes, int32_t head_dim,
                                         int32_t bits, int64_t n_books, int64_t n_per_book,
                                         const float* levels, float* out, uint32_t flags,
                                         hipStream_t stream);

/* codebooks[s][g][c][j] = levels[s][(c >> j*b) & (2^b - 1)] for s < 2,
 * g < D*b/8, c < 256, j < 8/b (one book's levels [2][2^b]); b in {1, 2, 4}
 * (b = 3 is KVQ_ERR_SHAPE). */
KVQ_API kvq_status kvq_scalar_product_codebook(int32_t head_dim, int32_t bits,
                                       const float* levels, float* codebooks,
                                       hipStream_t stream);

/* Static description of a status code. */
KVQ_API const char* kvq_status_string(kvq_status status);

/* hipError_t value of the last KVQ_ERR_HIP on the calling thread (0 if none). */
KVQ_API int kvq_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
