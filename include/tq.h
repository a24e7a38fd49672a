/*
 * tq.h -- C ABI of the rotated-basis ternary projection library (libtq.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Activations are rotated by the signed blockwise
 * Walsh-Hadamard transform H(D.x)/sqrt(1024) and then multiplied by a ternary
 * weight matrix stored as row-split planes (base / high / fp16 scale) with one
 * scale per 128-weight group.  Sources (page title, section):
 *   [ninfer-skill]   "ninfer 三元制品：容器格式与几何" (ninfer ternary artifact:
 *                    container format and geometry): §1 alignment constants,
 *                    §2 ternary formats, §3 row-split geometry, §6 constants.
 *   [gguf-explainer] "GGUF 完整讲解": §4.3 2-bit code semantics.
 *   [ninfer-v3]      "artifact-container.md": §6.1 formats, §6.2 layouts,
 *                    §8 hadamard_signs, §11 error ownership.
 *   [tensorsharp]    "从 TensorSharp 视角解读 Ternary Bonsai 2 27B": §4.2
 *                    transform contract, §4.4 network flow, §5.1 rejection
 *                    policy.
 *
 * Conventions shared by every entry point:
 *  - All sizes are int64_t / uint64_t element or byte counts; leading
 *    dimensions (ld*) are in elements and must be >= the row width.
 *  - Pointers named host_* are host memory; all others are device memory
 *    allocated and owned by the caller.  The library allocates nothing, keeps
 *    no pointer after returning, and never frees caller memory.
 *  - Device entry points enqueue work on `stream` (a hipStream_t; NULL means
 *    the legacy null stream) and return immediately; the caller keeps every
 *    buffer alive until that work has completed.
 *  - Validation is synchronous and complete before anything is launched: on
 *    any status other than TQ_OK nothing was enqueued and tq_last_error()
 *    returns a message naming the offending argument ("reject rather than
 *    run wrong": [tensorsharp] §4.2, §5.1; [ninfer-v3] §11.3).
 *  - Kernels read the stored planes in place (no repacking at run time,
 *    [ninfer-v3] §7.3) and do not check codes: a PQ2_0 code 3 decodes as +2
 *    and an out-of-range PTQ1_0 byte decodes by the digit arithmetic;
 *    tq_unpack_rowsplit reports both.
 *  - Every output element is written by exactly one thread in a fixed
 *    order, so results are bitwise reproducible for a given build and shape.
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_ARG = 1,          /* null pointer, bad enum, bad leading dimension */
  TQ_ERR_FORMAT = 2,       /* unknown numeric format                        */
  TQ_ERR_GEOMETRY = 3,     /* payload size does not match the layout        */
  TQ_ERR_ALIGN = 4,        /* pointer alignment requirement not met         */
  TQ_ERR_SHAPE = 5,        /* n, k, rows, batch or count out of range       */
  TQ_ERR_UNSUPPORTED = 6,  /* valid request this library does not implement */
  TQ_ERR_DEVICE = 7,       /* the HIP runtime reported an error             */
  TQ_ERR_DATA = 8          /* host data outside the format's value set      */
} tq_status;

/* Ternary formats, numbered by their GGUF tensor type ids ([ninfer-skill]
 * §6: T_PQ2_0 = 142, T_PTQ1_0 = 143).
 *  PQ2_0_G128:  32 base bytes + 0 high bytes + 2 scale bytes per group of
 *               128 weights ([ninfer-skill] §2).  Weight j of a group is the
 *               2-bit code at base byte j/4, bits 2*(j%4), value code-1
 *               ([gguf-explainer] §4.3).
 *  PTQ1_0_G128: 24 base + 2 high + 2 scale bytes per group ([ninfer-skill]
 *               §2).  The pages do not give the trit order; this library's
 *               convention: u = trit+1; base byte b (0..23) holds trits
 *               5b..5b+4 as sum u_i*3^i; high byte h (0..1) holds trits
 *               120+4h..123+4h as sum u_i*3^i.                            */
typedef enum { TQ_PQ2_0_G128 = 142, TQ_PTQ1_0_G128 = 143 } tq_format;

/* Element types of activations and outputs. */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* The 16-field row-split geometry, in the field order of [ninfer-skill] §3.
 * k_pad = align_up(k,128); groups_per_row = k_pad/128; per-row plane bytes
 * are groups times the per-group bytes (2 for the scale); base_offset = 0;
 * high_offset = align_up(base_bytes,256); scale_offset = high_offset +
 * align_up(high_bytes,256); payload_bytes = scale_offset + scale_bytes.
 * Planes are row-major over (row, group); scales are little-endian binary16. */
typedef struct {
  uint64_t n, k, k_pad, groups_per_row, base_bytes_per_group,
      high_bytes_per_group, base_row_bytes, high_row_bytes, scale_row_bytes,
      base_offset, base_bytes, high_offset, high_bytes, scale_offset,
      scale_bytes, payload_bytes;
} tq_geometry;

/* Message for the last non-OK status returned on the calling thread
 * (thread-local; valid until the next call on that thread). */
const char *tq_last_error(void);

/* Library version string ("major.minor.patch"). */
const char *tq_version(void);

/* ----------------------------------------------------------- host ----- */

/* Fill *out with the geometry of an [n, k] matrix ([ninfer-skill] §3).
 * Errors: TQ_ERR_FORMAT for an unknown format, TQ_ERR_SHAPE unless n,k >= 1,
 * TQ_ERR_ARG for a null `out`. */
tq_status tq_geometry_get(int32_t format, int64_t n, int64_t k,
                          tq_geometry *out);

/* Host packer: encode host_trits (int8 row-major [n][k], values in
 * {-1,0,1}) and host_scale_bits (binary16 bit patterns, row-major
 * [n][groups_per_row]) into the row-split payload host_payload, which must
 * hold exactly payload_bytes = geometry.payload_bytes bytes.  Writes every
 * byte (inter-plane padding and trits past k up to k_pad are zero trits).
 * Errors: TQ_ERR_GEOMETRY when payload_bytes differs from the layout size
 * ("stores N bytes; layout requires M", [ninfer-skill] §1), TQ_ERR_DATA when
 * a trit lies outside {-1,0,1} (nothing is written then). */
tq_status tq_pack_rowsplit(int32_t format, int64_t n, int64_t k,
                           const int8_t *host_trits,
                           const uint16_t *host_scale_bits,
                           uint8_t *host_payload, uint64_t payload_bytes);

/* Host unpacker (inverse of tq_pack_rowsplit), by the same plane addressing
 * ([ninfer-skill] §3) and code rules ([gguf-explainer] §4.3 for PQ2_0: value
 * code-1; the radix-3 convention above for PTQ1_0): host_values int8 [n][k_pad]
 * receives code-1 for PQ2_0 (so -1..2) and the decoded digit-1 for PTQ1_0;
 * host_scale_bits [n][groups_per_row] receives the stored binary16 bits.
 * *host_bad_codes (may be NULL) receives the number of stored codes that are
 * not ternary (PQ2_0 code 3, PTQ1_0 base byte > 242 or high byte > 80);
 * the decode is still written.  Errors as for tq_pack_rowsplit. */
tq_status tq_unpack_rowsplit(int32_t format, int64_t n, int64_t k,
                             const uint8_t *host_payload,
                             uint64_t payload_bytes, int8_t *host_values,
                             uint16_t *host_scale_bits,
                             uint64_t *host_bad_codes);

/* .ninfer v2 container ([ninfer-skill] §1): bytes 0-7 the magic
 * "NINFER\0\2", bytes 8-15 the little-endian uint64 directory length
 * json_bytes, then the compact UTF-8 JSON directory; the payload starts at
 * align_up(16 + json_bytes, 4096) and object offsets are relative to it.
 * Validation (all of it, in directory order): root members exactly
 * {identity, objects}; identity exactly {model_id, weights_id}, both
 * non-empty strings; a tensor exactly {name, kind, shape, format, layout,
 * offset, bytes}, a resource exactly {name, kind, encoding, offset, bytes};
 * kind "tensor" or "resource"; resource encoding "raw-bytes-v1"; a tensor's
 * bytes equal to its encoded size ("tensor <name> stores N bytes; layout
 * requires M"); offset >= the end of the previous object, a multiple of the
 * alignment (256 for tensors, 1 for resources), and offset + bytes inside
 * the payload; unique names ("duplicate object name: <name>").
 * Readings where the page is silent: layouts are the four NInfer v3
 * layouts ([ninfer-v3] §6.2); encoded sizes are known for
 * row_split_k128_v1 with PQ2_0_G128 / PTQ1_0_G128 (the row-split geometry)
 * and for contiguous_le_v1 with bf16, fp32, int32 (elements times size,
 * rank 0 = one element); block_scale_k16_m128x4_v1 and row_scale_v1 give
 * TQ_ERR_UNSUPPORTED; other names TQ_ERR_FORMAT ("unknown numeric format:
 * <f>", "unknown layout: <l>"); "compact" means no whitespace outside JSON
 * strings; shape entries and bytes are positive integers, offsets
 * non-negative integers. */
typedef struct {
  int32_t kind;        /* 0 tensor, 1 resource */
  int32_t rank;        /* tensors: number of shape entries (0..16) */
  int64_t shape[16];
  uint64_t offset;     /* payload-relative byte offset */
  uint64_t bytes;
  char name[256];      /* NUL-terminated */
  char format[64];     /* tensors: the format; resources: the encoding */
  char layout[64];     /* tensors only */
} tq_container_object;

/* Validate host_file (file_bytes bytes of a whole container in host memory)
 * and return the payload's file offset and the number of directory objects
 * (either output may be NULL).  Errors: TQ_ERR_FORMAT with the message of
 * the first rule broken, TQ_ERR_UNSUPPORTED as above, TQ_ERR_ARG for a
 * NULL file with file_bytes > 0. */
tq_status tq_container_parse(const uint8_t *host_file, uint64_t file_bytes,
                             uint64_t *payload_offset, int64_t *count);

/* Directory entry `index` (in directory order) of a valid container. */
tq_status tq_container_object_at(const uint8_t *host_file, uint64_t file_bytes,
                                 int64_t index, tq_container_object *out);

/* --------------------------------------------------------- device ----- */

/* GGUF block stream -> row-split planes ([ninfer-skill] §3-§4).  blocks:
 * one block per (row, group) in row-major order over the [n, k_pad] groups,
 * block_bytes 34 for PQ2_0_G128 ([scale 2][base 32]) or 28 for PTQ1_0_G128
 * ([base 24][high 2][scale 2]); blocks_bytes must equal
 * n * groups_per_row * block_bytes and payload_bytes the layout size.  Every
 * payload byte is written (the padding between planes is zero).  The two
 * buffers must not overlap (TQ_ERR_ARG); payload 256-byte and blocks 8-byte
 * aligned (TQ_ERR_ALIGN).  Errors: TQ_ERR_GEOMETRY for a size mismatch. */
tq_status tq_blocks_to_planes(const uint8_t *blocks, uint64_t blocks_bytes,
                              int32_t format, int64_t n, int64_t k,
                              uint8_t *payload, uint64_t payload_bytes,
                              void *stream);

/* Row-split planes -> GGUF block stream: the exact inverse of
 * tq_blocks_to_planes on the plane bytes. */
tq_status tq_planes_to_blocks(const uint8_t *payload, uint64_t payload_bytes,
                              int32_t format, int64_t n, int64_t k,
                              uint8_t *blocks, uint64_t blocks_bytes,
                              void *stream);

/* 2-bit G64 block stream: the lossless expansion a runtime without the
 * ternary types uses ([tensorsharp] §4.1: blocks expanded, not requantised,
 * into the upstream 2-bit type, about +6% memory over PQ2_0 and +29% over
 * PTQ1_0).  Layout (a reading: [gguf-explainer] §4.3 gives the code rule,
 * [ninfer-v3] §6.1 the q2_g64_fp16 codec): row-major [n][k_pad/64] blocks
 * of 18 bytes, each [binary16 d, little-endian][16 code bytes]; weight j of
 * a block is code byte j/4, bits 2*(j%4), value (code-1)*d.  Blocks 2g and
 * 2g+1 of a row hold group g's 128 weights, both with its scale. */

/* *bytes = n * (k_pad/64) * 18.  Errors: TQ_ERR_SHAPE unless n, k >= 1,
 * TQ_ERR_ARG for a NULL `bytes`. */
tq_status tq_g64_bytes(int64_t n, int64_t k, uint64_t *bytes);

/* Row-split planes (either format, validated as for tq_gemv_rowsplit) ->
 * the G64 block stream `blocks` (exactly tq_g64_bytes bytes, 16-byte
 * aligned, not overlapping the payload).  Every decoded value is kept: a
 * PQ2_0 code 3 stays code 3 (+2) and a PTQ1_0 byte decodes by the digit
 * arithmetic.  Errors: TQ_ERR_GEOMETRY for either size, TQ_ERR_ALIGN,
 * TQ_ERR_ARG. */
tq_status tq_expand_g64(const uint8_t *payload, uint64_t payload_bytes, int32_t format,
                        int64_t n, int64_t k, uint8_t *blocks, uint64_t blocks_bytes,
                        void *stream);

/* Decode GEMV over the G64 block stream: y[n] = sum_j W[n][j] * xrot[j]
 * with W as above; xrot and y as for tq_gemv_rowsplit (x rounded to
 * binary16, fp32 accumulation).  Requirements: k % 1024 == 0 and
 * k <= 17408 (TQ_ERR_SHAPE), n < 2^30, blocks 16-byte aligned.  Covered:
 * batch 1; batch > 1 returns TQ_ERR_UNSUPPORTED with nothing enqueued. */
tq_status tq_gemv_g64(const uint8_t *blocks, uint64_t blocks_bytes, int64_t n, int64_t k,
                      const void *xrot, int32_t x_dtype, int64_t batch, int64_t ldx, float *y,
                      int64_t ldy, void *stream);

/* Signed blockwise Walsh-Hadamard transform of `rows` rows of width k
 * ([tensorsharp] §4.2; [ninfer-v3] §8 hadamard_signs):
 *   inverse == 0:  y_b = H (d_b . x_b) / 32     (projection inputs, head)
 *   inverse == 1:  y_b = d_b . (H x_b) / 32     (embedding rows)
 * for every 1024-element block b, with H the unnormalised Sylvester
 * Hadamard matrix (natural order, H[i][j] = (-1)^popcount(i&j)) and d the
 * bf16 sign table `signs_bf16` [k] (each entry +1 or -1; only the sign bit
 * is used).  x: x_dtype (F32, BF16 or F16) row-major with leading dimension
 * ldx; y: y_dtype (F32, BF16 or F16, rounded to nearest even from the fp32
 * result) with leading dimension ldy.  rows == 0 is a no-op.
 * Requirements: k % 1024 == 0 (TQ_ERR_SHAPE), x/y 16-byte aligned and
 * ldx, ldy multiples of 8 (TQ_ERR_ALIGN), ldx, ldy >= k (TQ_ERR_ARG);
 * x and y must not overlap unless they are the same buffer with the same
 * dtype and leading dimension (in-place). */
tq_status tq_hadamard_signed(const void *x, int32_t x_dtype, int64_t rows,
                             int64_t k, int64_t ldx,
                             const uint16_t *signs_bf16, int32_t inverse,
                             void *y, int32_t y_dtype, int64_t ldy,
                             void *stream);

/* The signed transform of a row held in the tiled head order, taken in the
 * grouped head order first ([ninfer-skill] §5 perm48 / perm_row; [tensorsharp]
 * §4.2: with grouped GatedDeltaNet metadata the input of the projection
 * after the GatedDeltaNet is reordered into the publisher's head order
 * before its transform):
 *   r[j] = x[src(j)],  src(h*head_dim + i) = ((h % tiles)*groups + h/tiles)*head_dim + i
 *   y_b = H (d_b . r_b) / 32  per 1024-element block b (as tq_hadamard_signed
 *   with inverse 0).
 * The model's value heads: tiles 3, groups 16, head_dim 128 (k = 6144; target
 * head g*3+t comes from source head t*16+g).  Reading: r[j] = x[src(j)], the
 * page's "source row" of row j.
 * Requirements: as tq_hadamard_signed; tiles, groups >= 1, head_dim a
 * multiple of 16 and tiles*groups*head_dim == k (TQ_ERR_SHAPE); x and y must
 * not overlap (TQ_ERR_ARG). */
tq_status tq_hadamard_signed_grouped(const void *x, int32_t x_dtype, int64_t rows, int64_t k,
                                     int64_t ldx, int32_t tiles, int32_t groups,
                                     int32_t head_dim, const uint16_t *signs_bf16, void *y,
                                     int32_t y_dtype, int64_t ldy, void *stream);

/* Decode GEMV ([ninfer-v3] §8: a projection multiplies the stored matrix by
 * the transformed input; [gguf-explainer] §4.3-§4.4: value (code-1)*d per
 * group, dot product with the activations):
 *   y[b][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * xrot[b][j]
 * for b < batch, n < N, over the row-split payload (`payload`, exactly
 * payload_bytes bytes, 256-byte aligned).  xrot: already-rotated
 * activations, x_dtype F32, BF16 or F16, row-major [batch][ldx]; the kernel
 * rounds them to binary16 and accumulates in fp32 (finite |xrot| <= 65504).
 * y: fp32 row-major [batch][ldy].
 * Requirements: k % 128 == 0, 1 <= batch <= 8, k <= 65536 (PQ2_0) or
 * k <= 32768 (PTQ1_0) (TQ_ERR_SHAPE); xrot 16-byte aligned, ldx a multiple
 * of 8 (TQ_ERR_ALIGN); ldx >= k, ldy >= n. */
tq_status tq_gemv_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                           int32_t format, int64_t n, int64_t k,
                           const void *xrot, int32_t x_dtype, int64_t batch,
                           int64_t ldx, float *y, int64_t ldy, void *stream);

/* Decode step in one launch: the signed transform of the projection input
 * ([tensorsharp] §4.2) fused with the decode GEMV,
 *   y[b][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * r[b][j],
 *   r_b = binary16( H (d_b . x_b) / 32 )  per 1024-element block b,
 * i.e. exactly tq_hadamard_signed (inverse 0, y_dtype F16) followed by
 * tq_gemv_rowsplit on its output, without the intermediate buffer or the
 * second launch.  x: unrotated activations, x_dtype F32, BF16 or F16,
 * row-major [batch][ldx]; signs_bf16 [k] as for tq_hadamard_signed; y: fp32
 * row-major [batch][ldy].
 * Requirements: k % 1024 == 0, 1 <= batch <= 8 (TQ_ERR_SHAPE); x, signs
 * 16-byte aligned, ldx a multiple of 8 (TQ_ERR_ALIGN); ldx >= k, ldy >= n
 * (TQ_ERR_ARG).  Covered: PQ2_0_G128 with batch 1 and k <= 11264; any other
 * valid request returns TQ_ERR_UNSUPPORTED with nothing enqueued. */
tq_status tq_rotated_gemv_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                                   int32_t format, int64_t n, int64_t k,
                                   const void *x, int32_t x_dtype, int64_t batch,
                                   int64_t ldx, const uint16_t *signs_bf16,
                                   float *y, int64_t ldy, void *stream);

/* Output head of a decode step in one launch ([tensorsharp] §4.4: after the
 * last layer, RMSNorm, the signed Hadamard transform and the low-bit output
 * head give the logits) with the greedy choice fused in (a GEMV that also
 * finds the argmax: [gguf-explainer] §4.5):
 *   r = x * g / sqrt(mean_j(x_j^2) + eps)        (RMSNorm; a reading: the
 *       pages name the step, not its formula; g = norm_bf16 [k], eps >= 0)
 *   xrot = binary16( H (d . r) / 32 )  per 1024-element block
 *   logits[n] = sum_g s[n][g] * sum_{j in g} t[n][j] * xrot[j]
 *   *token = the lowest index among the largest logits (-0 equals +0).
 * x: one hidden row, x_dtype F32, BF16 or F16, 16-byte aligned; the sum of
 * squares and the scale are fp32.  logits: fp32 [n], or NULL to skip them.
 * work: two uint64 words of device memory, 16-byte aligned, owned by the
 * caller, zero before the first call; every call leaves them zero again.
 * Calls that share a work buffer must not run concurrently.  token: one
 * device int32.  A NaN logit is never chosen (it orders below every number,
 * -inf included); if every logit is NaN the token is -1.
 * Requirements: k % 1024 == 0, n < 2^30 (TQ_ERR_SHAPE); alignment as above
 * (TQ_ERR_ALIGN).  Covered: PQ2_0_G128 with k <= 11264 (the decode GEMV's
 * batch-1 kernel); other valid requests return TQ_ERR_UNSUPPORTED with
 * nothing enqueued. */
tq_status tq_head_argmax(const uint8_t *payload, uint64_t payload_bytes, int32_t format,
                         int64_t n, int64_t k, const void *x, int32_t x_dtype,
                         const uint16_t *norm_bf16, float eps, const uint16_t *signs_bf16,
                         float *logits, uint64_t *work, int32_t *token, void *stream);

/* tq_head_argmax for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments, requirements and results, without the
 * `work` argument.  The two work words live in a device global of 16 bytes
 * per GPU inside the library, held until the process ends; no call
 * allocates or frees anything.  Every request the one-launch head covers
 * (n < 2^30, k <= 11264) fits those two words; other requests are rejected
 * as by tq_head_argmax (TQ_ERR_SHAPE / TQ_ERR_UNSUPPORTED).  Each call
 * leaves the words zero for the next.  All calls on one GPU share them:
 * calls that overlap on one GPU (on different streams, or from different
 * threads) race and must not be issued. */
tq_status tq_head_argmax_noalloc(const uint8_t *payload, uint64_t payload_bytes, int32_t format,
                                 int64_t n, int64_t k, const void *x, int32_t x_dtype,
                                 const uint16_t *norm_bf16, float eps, const uint16_t *signs_bf16,
                                 float *logits, int32_t *token, void *stream);

/* tq_rotated_gemv_rowsplit with the grouped head order: the signed
 * transform input is x gathered as for tq_hadamard_signed_grouped, i.e.
 * exactly tq_hadamard_signed_grouped (y_dtype F16) then tq_gemv_rowsplit, in
 * one launch.  Requirements and coverage as for both. */
tq_status tq_rotated_gemv_rowsplit_grouped(const uint8_t *payload, uint64_t payload_bytes,
                                           int32_t format, int64_t n, int64_t k, const void *x,
                                           int32_t x_dtype, int64_t batch, int64_t ldx,
                                           int32_t tiles, int32_t groups, int32_t head_dim,
                                           const uint16_t *signs_bf16, float *y, int64_t ldy,
                                           void *stream);

/* Prefill GEMM ([tensorsharp] §4.4: every low-bit projection of the
 * network, prefill included, takes the rotated input; [gguf-explainer] §4.3
 * code rule):
 *   Y[m][n] = sum_g s[n][g] * sum_{j in g} t[n][j] * X[m][j]
 * for m < M rows of rotated activations X (x_dtype TQ_F16 or TQ_BF16,
 * row-major [M][ldx], 16-byte aligned, ldx a multiple of 8) against a
 * PQ2_0_G128 or PTQ1_0_G128 payload, on the matrix cores.  Each weight is
 * decoded to the binary16 value t*s, which is exact (s is a binary16 and t
 * is -1, 0 or +1); X is used as binary16 (bf16 input is rounded to binary16,
 * finite |X| <= 65504); products accumulate in fp32.  Y: y_dtype TQ_F32 or
 * TQ_BF16, [M][ldy].  M == 0 is a no-op.
 * Requirements: k % 128 == 0 and k <= 2^20 (TQ_ERR_SHAPE); ldx < 2^22
 * (TQ_ERR_ARG: a tile of 256 rows of X is addressed with 32-bit byte
 * offsets); alignment as above. */
tq_status tq_gemm_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                           int32_t format, int64_t n, int64_t k, const void *x,
                           int32_t x_dtype, int64_t m, int64_t ldx, void *y,
                           int32_t y_dtype, int64_t ldy, void *stream);

/* Embedding rows with the inverse transform ([tensorsharp] §4.2, §4.4):
 * out[i] = per 1024-block d . (H r)/32 where r = dequantised row ids[i] of
 * the [n, k] payload.  ids: int32 device array [count]; out: fp32
 * [count][ldo].  An id outside [0, n) produces a zero row and, when
 * err_word is not NULL, stores 1 into *err_word (device int32, which the
 * caller zeroes beforehand); nothing outside the payload is read.
 * Requirements: k % 1024 == 0 (TQ_ERR_SHAPE), ldo >= k, count >= 0. */
tq_status tq_embed_rows_inverse(const uint8_t *payload, uint64_t payload_bytes,
                                int32_t format, int64_t n, int64_t k,
                                const int32_t *ids, int64_t count,
                                const uint16_t *signs_bf16, float *out,
                                int64_t ldo, int32_t *err_word, void *stream);

/* Decode hook (for bit-exact checks of the device unpack against the code
 * rules: [gguf-explainer] §4.3 for PQ2_0, the radix-3 convention above for
 * PTQ1_0; planes addressed as in [ninfer-skill] §3): for each of `count` row
 * indices in
 * `rows` (device int32, each in [0, n); others give zero output), write the
 * decoded values code-1 / digit-1 to values [count][k_pad] (int8) and the
 * stored scale bits to scale_bits [count][groups_per_row] (uint16). */
tq_status tq_decode_rowsplit(const uint8_t *payload, uint64_t payload_bytes,
                             int32_t format, int64_t n, int64_t k,
                             const int32_t *rows, int64_t count,
                             int8_t *values, uint16_t *scale_bits,
                             void *stream);

/* Measurement reference (not part of the projection): read `bytes` bytes of
 * device memory at `src` once, in 16-byte non-temporal loads from a one-shot
 * grid of 256-thread workgroups, each thread reading four 16-byte words of
 * its workgroup's contiguous span.  This is the access the decode GEMVs'
 * weight stream makes, without the decode, so its duration at a given size
 * is the read floor those kernels are compared with (decode is
 * bandwidth-bound: [gguf-explainer] §4.8).  The loaded words are folded
 * into one value that is stored to *sink (device uint32) only if it equals
 * a fixed constant; the caller owns sink and ignores its contents.
 * Requirements: bytes a positive multiple of 16 below 2^40 (TQ_ERR_SHAPE);
 * src 16-byte and sink 4-byte aligned (TQ_ERR_ALIGN); non-NULL (TQ_ERR_ARG). */
tq_status tq_stream_read(const void *src, uint64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
