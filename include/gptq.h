/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer quantizer.
 *
 * The method is the GPTQ layer-wise quantizer as described on the page
 * "GPTQ, with the code open" (modelfoundations.com/notes/gptq):
 *   - section "Measuring damage where it matters": H = 2 X X^T, one matrix
 *     shared by every output row;
 *   - section "Paper vs. code": H accumulated over calibration batches, inputs
 *     that never fire ("dead") zeroed, 1 % of the mean diagonal added as
 *     damping, full fp32 arithmetic, act-order, rulers per group of columns;
 *   - section "From one repair to a whole model": the upper Cholesky factor of
 *     the inverse of H drives every repair; columns are quantized in one fixed
 *     order for all rows, in blocks of 128 whose repairs are applied at once
 *     inside the block and deferred to one matrix product beyond it;
 *   - section "What quantization is, and why anyone bothers": the asymmetric
 *     min-max ruler, scale = (max - min)/(2^b - 1), the zero point rounded to
 *     a whole tick, w_hat = scale * (q - zero); and the use of the stored
 *     ticks at generation, dequantized inside a matrix-vector product.
 *
 * Conventions shared by every call:
 *   - Every pointer argument that names an array is a DEVICE pointer (memory
 *     allocated by the caller on the current HIP device) unless stated
 *     otherwise.  Output-size pointers of the *_workspace_size queries are
 *     HOST pointers.  The library allocates no memory of its own: scratch
 *     space is a caller-provided workspace sized by the matching query.
 *   - Matrices are row-major with an explicit leading dimension in ELEMENTS.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on that stream and never synchronise; results are valid once the
 *     stream has reached the call.
 *   - Every argument is validated on the host before anything is enqueued:
 *     a call that returns an error has enqueued nothing.  GPTQ_EHIP reports a
 *     failed kernel launch (gptq_last_error() carries HIP's message).
 *   - Buffers passed to one call must not overlap unless stated.
 *   - Calls are deterministic: the same inputs give bitwise-identical outputs
 *     (no floating-point atomics; every reduction has a fixed order).
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enumerations take int as their fixed underlying type, so every
 * int a caller passes (from C, or a foreign-function interface) is a value of
 * the type; the calls themselves reject values outside the lists.  In C an
 * enumeration is an int already. */
#ifdef __cplusplus
#define GPTQ_ENUM_BASE : int
#else
#define GPTQ_ENUM_BASE
#endif

typedef enum GPTQ_ENUM_BASE {
  GPTQ_OK = 0,
  GPTQ_EINVAL = 1,        /* null pointer, negative size, bad enum value      */
  GPTQ_EDTYPE = 2,        /* dtype not supported by this call                 */
  GPTQ_ESHAPE = 3,        /* inconsistent sizes / leading dimensions           */
  GPTQ_EALIGN = 4,        /* a pointer or leading dimension is misaligned      */
  GPTQ_EUNSUPPORTED = 5,  /* valid request outside what the library supports */
  GPTQ_EWORKSPACE = 6,    /* workspace missing or smaller than the query says */
  GPTQ_EHIP = 7           /* a HIP launch failed                               */
} gptq_status;

typedef enum GPTQ_ENUM_BASE { GPTQ_F32 = 0, GPTQ_BF16 = 1, GPTQ_F16 = 2 } gptq_dtype;

/* ------------------------------------------------------------------------
 * Hessian accumulation.  Page: "GPTQ, with the code open", section
 * "Measuring damage where it matters" (H = 2 X X^T) and the "Paper vs. code"
 * table (H built up over calibration batches).
 *
 *   H[i][j] += 2 * sum_t X[t][i] * X[t][j]      for 0 <= i <= j < d
 *
 * H      : d x d fp32, row-major, leading dimension d.  Only the upper
 *          triangle including the diagonal is defined on return; entries
 *          strictly below the diagonal are unspecified (they may be
 *          overwritten).  The caller zeroes H once before the first batch;
 *          repeated calls accumulate the raw sum (no running-mean rescale).
 * X      : n_tok x d calibration inputs, token-major (one row per token),
 *          row stride ldx >= d elements, dtype xt (GPTQ_BF16, GPTQ_F16 or
 *          GPTQ_F32).  Products are formed exactly and summed in fp32.
 *          X must be aligned to its element size (GPTQ_EALIGN otherwise);
 *          16-bit X that is 16-byte aligned with ldx % 8 == 0 takes the fast
 *          load path.  n_tok == 0 or d == 0 is a no-op.
 * ws     : workspace of at least gptq_hessian_workspace_size() bytes
 *          (may be NULL when that size is 0); 256-byte aligned.
 * ------------------------------------------------------------------------ */
gptq_status gptq_hessian_workspace_size(int64_t d, int64_t n_tok, gptq_dtype xt,
                                        size_t* bytes);
gptq_status gptq_hessian_accumulate(float* H, int64_t d, const void* X, gptq_dtype xt,
                                    int64_t n_tok, int64_t ldx, void* ws, size_t ws_bytes,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Preparation of H.  Page: "GPTQ, with the code open", "Paper vs. code"
 * (dead inputs, 1 % damping of the mean diagonal, act-order) and "From one
 * repair to a whole model" (the Cholesky factor of the inverse).
 *
 * In order, on the device:
 *   1. dead[j] = (H[j][j] == 0); such diagonals are set to 1;
 *   2. if act_order: perm = indices sorted by H[j][j] descending, ties by
 *      ascending index (a stable sort); else perm = identity.  H is
 *      permuted symmetrically into processing order;
 *   3. lambda = percdamp * mean(diag H); H[j][j] += lambda;
 *   4. H is replaced by U, the upper triangular matrix with positive
 *      diagonal and U^T U = H^{-1} (processing order).  The strictly lower
 *      triangle is set to 0.
 *
 * H_to_U : d x d fp32 row-major (ld d), upper triangle read, U written.
 * perm   : int32[d] out (processing position k -> original column perm[k]).
 *          May be NULL only when act_order == 0.
 * dead   : uint8[d] out, indexed by ORIGINAL column.
 * info   : int32 out (device): 0 on success; k > 0 if the damped matrix is not
 *          positive definite, k being the 1-based processing position of the
 *          first failing pivot found; -1 if a diagonal entry is NaN or Inf.
 *          U is undefined when info != 0.  The call itself cannot see info
 *          (it does not synchronise): read it after the stream reaches it.
 * ws     : workspace of at least gptq_prepare_workspace_size() bytes.
 * ------------------------------------------------------------------------ */
gptq_status gptq_prepare_workspace_size(int64_t d, int act_order, size_t* bytes);
gptq_status gptq_prepare(float* H_to_U, int64_t d, float percdamp, int act_order,
                         int32_t* perm, uint8_t* dead, int32_t* info, void* ws,
                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gptq_prepare without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same operation, arguments, kernels and
 * results (bit for bit) as gptq_prepare; the scratch it needs lives in a
 * static device array of the library, GPTQ_PREPARE_NOALLOC_SCRATCH_BYTES
 * bytes on each GPU the library runs on, held until the process ends.
 *
 * d      : 1 .. GPTQ_PREPARE_NOALLOC_MAX_D (4096); larger d returns
 *          GPTQ_EUNSUPPORTED (use gptq_prepare with a workspace).
 * The call allocates nothing (no hipMalloc, no library allocation).  Every
 * call on one GPU uses that GPU's one scratch array: calls that overlap in
 * time on one GPU (two streams, two host threads) race and must be ordered
 * by the caller.  The first call on each device looks up the array's device
 * address (hipGetSymbolAddress); GPTQ_EHIP if that fails.
 * ------------------------------------------------------------------------ */
#define GPTQ_PREPARE_NOALLOC_MAX_D 4096
#define GPTQ_PREPARE_NOALLOC_SCRATCH_BYTES (4096ull * 4096ull * 4ull + 4096ull * 4ull + 256ull)
gptq_status gptq_prepare_noalloc(float* H_to_U, int64_t d, float percdamp, int act_order,
                                 int32_t* perm, uint8_t* dead, int32_t* info, void* stream);

/* ------------------------------------------------------------------------
 * Quantize one layer.  Page: "GPTQ, with the code open", sections "What
 * quantization is" (ruler), "The repair rule" and "From one repair to a whole
 * model" (the column loop, the per-weight loss (w - q)^2 / (2 d^2), blocks of
 * `blocksize` columns with deferred repairs, rulers fitted before repairs),
 * and "Paper vs. code" (groupsize, act-order, dead inputs).
 *
 * W        : r x c weights (one output per row), row stride ldw >= c, dtype
 *            wt; read only.
 * U        : c x c from gptq_prepare (processing order).
 * perm     : int32[c] from gptq_prepare, or NULL for the identity order.
 * dead     : uint8[c] from gptq_prepare (original order), or NULL (none).
 * bits     : 2, 3, 4 or 8.
 * sym      : 0 -> asymmetric ruler (range stretched to include 0, zero =
 *            rne(-min / scale)); 1 -> symmetric ruler: range [-m, m] with
 *            m = max(|min|, |max|), scale = 2m / (2^bits - 1), zero = the
 *            middle tick 2^(bits-1).  The pages name a symmetric option
 *            ("Paper vs. code") without a formula; this is the plainest
 *            reading that keeps 0.0 exactly on a tick.  Other values:
 *            GPTQ_EINVAL.
 * groupsize: <= 0 -> one ruler per row, fitted on the original weights
 *            before dead inputs are zeroed; > 0 -> one ruler per run of
 *            `groupsize` columns in processing order, fitted when the loop
 *            reaches the run's first column on the current (repaired) values.
 *            The last run may be shorter than groupsize.  Requires
 *            groupsize % blocksize == 0 or blocksize % groupsize == 0.
 * blocksize: 1 .. 128 (columns whose repairs are applied immediately).
 * codes    : r x c uint8 out, ORIGINAL column order, values 0 .. 2^bits - 1.
 * scales   : r x n_groups fp32 out; zeros: r x n_groups int32 out, where
 *            n_groups = groupsize > 0 ? ceil(c / groupsize) : 1, in
 *            processing order of the runs.
 * g_idx    : int32[c] out: run index of each ORIGINAL column (0 when
 *            groupsize <= 0).
 * W_hat    : r x c fp32 out (nullable), ORIGINAL column order,
 *            scale * (code - zero).
 * row_loss : fp32[r] out (nullable): sum over the row of (w - q)^2 / (2 U_jj^2).
 * ws       : workspace of at least gptq_quantize_layer_workspace_size() bytes.
 * Ties round half to even; the code is clamp(rne(w / scale) + zero, 0, 2^b-1);
 * every decision (ruler and rounding) is taken in IEEE fp32.
 * ------------------------------------------------------------------------ */
gptq_status gptq_quantize_layer_workspace_size(int64_t r, int64_t c, int64_t blocksize,
                                               size_t* bytes);
gptq_status gptq_quantize_layer(const void* W, gptq_dtype wt, int64_t r, int64_t c,
                                int64_t ldw, const float* U, const int32_t* perm,
                                const uint8_t* dead, int bits, int sym, int64_t groupsize,
                                int64_t blocksize, uint8_t* codes, float* scales,
                                int32_t* zeros, int32_t* g_idx, float* W_hat,
                                float* row_loss, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Pack codes into 32-bit words.  The pages only state that each weight is
 * stored as the index of its tick ("What quantization is, and why anyone
 * bothers"); the word layout is this library's:
 *   bits == 4: 8 codes per word, code k of the word in bits 4k .. 4k+3;
 *   bits == 3: 32 codes per 3 words, code k in bits 3k .. 3k+2 of the
 *              little-endian 96-bit value (word 0 = bits 0..31), so codes 10
 *              and 21 straddle two words.
 * Packed along the input (column) axis, one output row at a time.
 * codes    : r x c uint8 (values must fit in `bits`; higher bits are ignored).
 * col_perm : int32[c] (nullable).  When given, packed column j holds the code
 *            of original column col_perm[j] (entries outside 0 .. c-1 are
 *            clamped).  Passing the act-order permutation of gptq_prepare
 *            stores the codes in the order the columns were quantized, where
 *            every group of columns is contiguous -- the layout
 *            gptq_dequant_gemv reads for act-order layers.
 * packed   : r x ld_words uint32 out; ld_words >= c * bits / 32.
 * Requires c % 8 == 0 (4-bit) or c % 32 == 0 (3-bit).
 * ------------------------------------------------------------------------ */
gptq_status gptq_pack(const uint8_t* codes, int64_t r, int64_t c, int bits,
                      const int32_t* col_perm, uint32_t* packed, int64_t ld_words,
                      void* stream);

/* ------------------------------------------------------------------------
 * Dequantize-on-the-fly matrix-vector product (batch 1) over packed codes.
 * Pages: "GPTQ, with the code open", section "What quantization is, and why
 * anyone bothers" (generation reads every weight once per token; the stored
 * tick index is turned back into scale * (tick - zero) while multiplying) and
 * "Post-training quantization", section "Weight-only and weight-and-
 * activation" (4- or 3-bit weights with 16-bit activations).
 *
 *   y[i] = sum_j scales[i, g(j)] * (q[i, j] - zeros[i, g(j)]) * x[src(j)]
 *
 * over the packed columns j = 0 .. c-1, where q[i, j] is packed column j of
 * row i (layout of gptq_pack), g(j) = j / groupsize (0 for one ruler per row)
 * and src(j) = col_perm[j] when col_perm is given, else j.  For an act-order
 * layer pack with col_perm = the act-order permutation and pass the same
 * col_perm here; scales / zeros are then used as gptq_quantize_layer wrote
 * them (group g covers quantization positions g*groupsize ..).
 *
 * packed    : r x ld_words uint32 (gptq_pack output); 4 bits: 16-byte aligned
 *             base and ld_words % 4 == 0.
 * bits      : 3 or 4.
 * scales    : r x ld_groups fp32; zeros: r x ld_groups int32.
 * groupsize : <= 0 or >= c: one ruler per row; else a multiple of 32, and
 *             ld_groups >= ceil(c / groupsize).
 * col_perm  : int32[c] or NULL (entries outside 0 .. c-1 are clamped).
 * x         : c activations, GPTQ_BF16 or GPTQ_F16 (GPTQ_F32 -> GPTQ_EDTYPE);
 *             16-byte aligned unless col_perm is given.
 * y         : fp32[r] out.
 * Requires c % 32 == 0 and c <= 49152 (GPTQ_EUNSUPPORTED beyond).  c == 0
 * writes y = 0.  Products are exact and sums are fp32: the result is within
 * about 64 * 2^-24 * sum_j scale * (q + zero) * |x_j| of the exact value.
 * ------------------------------------------------------------------------ */
gptq_status gptq_dequant_gemv(const uint32_t* packed, int64_t r, int64_t c, int bits,
                              int64_t ld_words, const float* scales, const int32_t* zeros,
                              int64_t ld_groups, int64_t groupsize, const int32_t* col_perm,
                              const void* x, gptq_dtype xt, float* y, void* stream);

/* ------------------------------------------------------------------------
 * Hadamard pre-rotation of rows.  Page: "Post-Training Quantization:
 * Calibration, GPTQ and Why Rotations Help", sections "Rotations: making
 * outliers disappear" and "Why do Hadamard rotations help quantization?"
 * (a Hadamard matrix scaled to a rotation spreads outliers; rotating a
 * layer's inputs and applying the inverse rotation to its weights leaves the
 * product unchanged).
 *
 *   out[i, :] = A[i, :] * blockdiag(H_b / sqrt(b), ..., H_b / sqrt(b))
 *
 * with H_b Sylvester's Hadamard matrix of order b (symmetric; the rotation is
 * its own inverse).  Rotate the calibration activations X (token-major, one
 * token per row) and the weights W (one output per row) with the same b: then
 * W_rot x_rot = W x for every input, and H of the rotated X is Q H Q^T.
 *
 * A    : rows x d, row stride lda, dtype at (f32 / bf16 / f16).
 * block: b, a power of two in 32 .. 8192 dividing d; <= 0 picks the largest
 *        power of two dividing d, capped at 8192 (a width that is not a power
 *        of two is rotated block-wise).
 * out  : rows x d, row stride ldo, dtype ot; fp32 arithmetic, rounded once
 *        (round-to-nearest-even) to ot.  out may be A itself (same dtype and
 *        stride); any other overlap is GPTQ_EINVAL.
 * ------------------------------------------------------------------------ */
gptq_status gptq_hadamard_rotate(const void* A, gptq_dtype at, int64_t rows, int64_t d,
                                 int64_t lda, int64_t block, void* out, gptq_dtype ot,
                                 int64_t ldo, void* stream);

/* ------------------------------------------------------------------------
 * Forward pass of a quantized linear layer over calibration tokens, for the
 * layer-by-layer pass.  Page: "What is GPTQ" (queryfeedz glossary), section
 * "How it works": layers are quantized in sequence, and each one is
 * calibrated on what the already-quantized layers before it produce.
 *
 *   act == 0:  Y[t, i] = round_yt( sum_k X[t, k] * round_xt(W_hat[i, k]) )
 *   act == 1:  Y[t, i] = round_yt( silu(G[t, i]) * round_xt(sum_k ...) ),
 *              silu(g) = g / (1 + exp(-g)): the gated MLP's silu(gate) * up.
 *
 * W_hat is the dequantized weight matrix gptq_quantize_layer writes (fp32,
 * original column order), rounded once (round-to-nearest-even) to the
 * activations' 16-bit type, the model's own precision: either inside this
 * call (wt = GPTQ_F32) or beforehand by gptq_round16 (wt = xt); the results
 * are the same bit for bit.  Products are exact in fp32, sums are fp32
 * (matrix cores), results are rounded once to yt.
 *
 * X     : n_tok x d, xt = GPTQ_BF16 or GPTQ_F16, row stride ldx (multiple of
 *         8), 16-byte aligned.
 * W_hat : r x d of type wt (GPTQ_F32, or xt), row stride ldw (a multiple of
 *         4 for fp32, of 8 for 16-bit), 16-byte aligned.  With 16-bit
 *         W_hat, ldx and ldw must be below 2^22 (GPTQ_EUNSUPPORTED).
 * G     : n_tok x r of type xt, row stride ldg (act == 1 only; may be NULL
 *         otherwise).
 * Y     : n_tok x r of type yt, row stride ldy.  Y may be G itself (same type
 *         and stride); any other overlap with X, W_hat or G is GPTQ_EINVAL.
 * Requires d a positive multiple of 64.
 * ------------------------------------------------------------------------ */
gptq_status gptq_linear_forward(const void* X, gptq_dtype xt, int64_t n_tok, int64_t d,
                                int64_t ldx, const void* W_hat, gptq_dtype wt, int64_t r,
                                int64_t ldw, int act, const void* G, int64_t ldg, void* Y,
                                gptq_dtype yt, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * Rounds fp32 values to a 16-bit type, element by element:
 *   dst[i, j] = round_dt(src[i, j]),  round-to-nearest-even; bf16 keeps NaN
 *   (quiet), fp16 overflows to infinity.
 * The rounding of the dequantized weights that the layer-by-layer forward
 * applies (same page and section as gptq_linear_forward), as a pass of its
 * own so that a layer's weights are rounded once rather than once per token
 * tile.
 *
 * src : rows x cols fp32, row stride lds, 4-byte aligned.
 * dst : rows x cols of type dt (GPTQ_BF16 or GPTQ_F16), row stride ldd,
 *       2-byte aligned; must not overlap src (GPTQ_EINVAL).
 * Stream-ordered and asynchronous; the caller owns both buffers.
 * ------------------------------------------------------------------------ */
gptq_status gptq_round16(const float* src, int64_t rows, int64_t cols, int64_t lds,
                         gptq_dtype dt, void* dst, int64_t ldd, void* stream);

/* SHA-256 (hex, static storage) of the sources this library was built from:
 * every file under csrc/ and this header, as the in-tree build hashes them.
 * The Python loader refuses a library whose id differs from the sources
 * beside it, so a stale build is never run. */
const char* gptq_build_id(void);

/* Human-readable name of a status code (static storage). */
const char* gptq_status_string(gptq_status s);
/* Detail of the last failure on the calling thread (thread-local storage). */
const char* gptq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_MI355X_H */
