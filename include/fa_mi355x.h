/*
 * fa_mi355x.h - C ABI of libfa_mi355x: exact IO-aware attention on MI355X
 * (gfx950, CDNA4).
 *
 * What is computed.  For every (sequence, query head h):
 *     S = scale * Q_h K_g^T,   P = softmax(S + mask),   O_h = P V_g,
 *     LSE_h[i] = ln sum_j exp(S_ij + mask_ij),
 * with g = h / (Hq / Hkv) the KV head shared by a contiguous group of query
 * heads (GQA; Hkv = 1 is MQA).  The result is the plain softmax attention,
 * computed tile by tile with the online-softmax recurrence so that no N x N
 * score or probability matrix ever reaches device memory.
 *   - S, P, O: llms.blog "FlashAttention: How IO-Aware Tiling and Online
 *     Softmax Solved Transformer Memory Bottlenecks", "Naive Attention
 *     Execution Profile"; tiling and the running (m, l, O) state: same page,
 *     "1. IO-Aware Tiling" and "2. Online Softmax Reduction".
 *   - logsumexp saved for a recomputing backward: tokrepo.com "Flash
 *     Attention - Fast Memory-Efficient Exact Attention", "Architecture
 *     Overview"; the backward that reloads Q, K, V tiles and recomputes the
 *     scores: llms.blog page, "3. Recomputation in the Backward Pass".
 *   - causal, sliding-window, variable-length and GQA/MQA: tokrepo.com page,
 *     "What Flash Attention Does" and "Key Features".
 *
 * Mask conventions (the pages fix none; these are this library's readings):
 *   - causal != 0: query i sees key j only if j <= i + (Nk - Nq)
 *     (bottom-right aligned; for Nq == Nk the usual lower triangle);
 *   - window > 0: query i sees key j only if (i + Nk - Nq) - j < window,
 *     i.e. at most `window` keys counting itself; window == 0: no window;
 *   - packed batches (cu_seqlens != NULL): a query sees only keys of its own
 *     sequence, and sequence positions start at 0 in each sequence;
 *   - a query that sees no key gets O = 0 and LSE = -inf.
 *
 * Layouts (all tensors dense and contiguous, head dimension innermost):
 *   dense  (cu_seqlens == NULL): Q, O [B, Nq, Hq, d];  K, V [B, Nk, Hkv, d];
 *                                LSE [B, Hq, Nq] fp32
 *   packed (cu_seqlens != NULL): Q, O [T, Hq, d];  K, V [T, Hkv, d];
 *                                LSE [Hq, T] fp32,  T = cu_seqlens[B]
 *     cu_seqlens: device int32[B + 1], nondecreasing prefix sums of the B
 *     sequence lengths, cu_seqlens[0] == 0; Q and K share it (self-attention),
 *     Nq == Nk must be >= every sequence length (it sizes the launch grid).
 *   dq, dk, dv have the layouts of q, k, v.
 *
 * Ownership and execution.  Every buffer is owned by the caller and lives in
 * device memory (HBM) unless stated otherwise.  The library never allocates,
 * frees or synchronises.  Its only global state is the static device scratch
 * of fa_decode_noalloc and that array's per-device address, looked up once:
 * calls are thread safe and only enqueue work on `stream` (a hipStream_t;
 * NULL = the null stream) before returning.  Inputs are read-only; outputs are fully
 * overwritten, never accumulated into.  Results are deterministic: the same
 * inputs give the same bits.
 *
 * Errors.  Each entry point returns an fa_status.  Argument checks happen on
 * the host before any HIP call, so a call that returns FA_ERR_INVALID_ARG or
 * FA_ERR_UNSUPPORTED has enqueued nothing.  FA_ERR_HIP reports a failed
 * launch (hipGetLastError).  Device-side errors cannot be detected: a
 * malformed cu_seqlens (decreasing, or sequences longer than Nq, or a total
 * larger than the buffers) is undefined behaviour.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size, bad scale */
  FA_ERR_UNSUPPORTED = 2,  /* valid request this library does not implement */
  FA_ERR_HIP = 3,          /* the HIP runtime rejected a launch */
  FA_ERR_TOO_LARGE = 4     /* needs more than the static scratch of
                              fa_decode_noalloc holds */
} fa_status;

/*
 * Forward, bf16 inputs and output, fp32 LSE.
 *   q, k, v : bf16 (raw bits, 2 bytes per element), layouts above
 *   o       : bf16 output, layout of q, rounded to nearest even
 *   lse     : fp32 output, natural-log logsumexp of the scaled, masked scores
 *   B       : batch size (dense) or number of sequences (packed), >= 1
 *   Hq, Hkv : query / KV heads, >= 1, Hq % Hkv == 0
 *   Nq, Nk  : query / key sequence lengths (packed: the longest sequence,
 *             and Nq == Nk), >= 1
 *   d       : head dimension, 64 or 128
 *   scale   : finite multiplier of Q K^T (usually 1/sqrt(d))
 *   causal  : 0 or 1
 *   window  : 0 = none, > 0 = keys visible per query counting itself
 *   cu_seqlens : NULL (dense) or device int32[B + 1] (packed)
 * Pointers q, k, v, o must be 16-byte aligned; lse 4-byte aligned.
 * Returns FA_ERR_INVALID_ARG for a null or misaligned pointer, a size < 1,
 * Hq % Hkv != 0, a non-finite scale, causal not in {0,1}, window < 0;
 * FA_ERR_UNSUPPORTED for d not in {64, 128}, packed with Nq != Nk, or
 * Hq * d * 128 >= 2^32 (64 token rows of one tensor must span less than
 * 4 GiB; tensors themselves may be larger).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d,
           float scale, int causal, int window,
           const int32_t* cu_seqlens, void* stream);

/*
 * Forward with IEEE fp16 q, k, v, o (same arguments, layouts and errors as
 * fa_fwd; tokrepo.com "Flash Attention - Fast Memory-Efficient Exact
 * Attention", "Self-Hosting & Configuration" names fp16 and bf16).  Scores,
 * softmax state and the output accumulator are fp32; P is rounded to fp16
 * (nearest even) for the P V product and O to fp16.
 */
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d,
               float scale, int causal, int window,
               const int32_t* cu_seqlens, void* stream);

/*
 * Forward with fp32 q, k, v, o (same arguments, layouts and errors as
 * fa_fwd, with 4 bytes per element).  Scores, softmax and the output
 * accumulator are computed in fp32 on the vector ALUs.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
               float scale, int causal, int window,
               const int32_t* cu_seqlens, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for T_q = B * Nq query rows and Hq
 * heads (for packed batches B * Nq bounds cu_seqlens[B], which the host
 * cannot read).  O(T_q * Hq), never quadratic in the sequence length.  d is
 * accepted for future layouts.  Returns 0 for a negative or zero argument.
 */
size_t fa_bwd_workspace_size(int T_q, int Hq, int d);

/*
 * Backward by recomputation (bf16 in, bf16 out).
 *   q, k, v, o, dout : bf16, layouts above; o is the output of fa_fwd for the
 *                      same q, k, v and arguments
 *   lse              : fp32, the LSE written by that fa_fwd call
 *   dq, dk, dv       : bf16 outputs, fully overwritten; for GQA, dk and dv
 *                      of a KV head sum over its query-head group
 *   workspace        : device buffer of at least
 *                      fa_bwd_workspace_size(B * Nq, Hq, d) bytes, 16-byte
 *                      aligned, used as scratch (contents undefined after the
 *                      call); it must not alias any other argument
 * The backward recomputes P = exp(S - LSE) tile by tile and forms
 * D_i = sum_c dO_ic O_ic, dS = P (dP - D); dQ = scale dS K, dK = scale dS^T Q,
 * dV = P^T dO, with no N x N buffer.
 * Errors as fa_fwd, plus FA_ERR_INVALID_ARG when the workspace is NULL or
 * smaller than required.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int B, int Hq, int Hkv, int Nq, int Nk, int d,
           float scale, int causal, int window,
           const int32_t* cu_seqlens, void* stream);

/*
 * Backward of fa_fwd_f16: q, k, v, o, dout, dq, dk, dv are IEEE fp16, with
 * the arguments, layouts, workspace and errors of fa_bwd (fa_fwd_f16 is the
 * forward whose o and lse it takes).  The products run on fp16 matrix cores
 * with fp32 accumulation; P and dS are rounded to fp16 (nearest even) as
 * their operands, and D = rowsum(dO * O) is formed in fp32 from the fp16 O.
 * Plain attention only (causal, window, GQA and packed batches as fa_bwd;
 * no bias or dropout variant).
 */
int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes,
               int B, int Hq, int Hkv, int Nq, int Nk, int d,
               float scale, int causal, int window,
               const int32_t* cu_seqlens, void* stream);

/*
 * Forward and backward with an additive bias (a custom attention mask:
 * tokrepo.com "Flash Attention - Fast Memory-Efficient Exact Attention",
 * "Key Features"):  S = scale * Q K^T + bias, then the causal and window
 * masks as in fa_fwd, then the same softmax, O and LSE.  A -inf entry hides
 * a key; a row whose every visible key is hidden gets O = 0, LSE = -inf.
 * The bias is a constant: fa_bwd_bias returns dQ, dK, dV only.  Dense
 * batches only (no cu_seqlens); other arguments, layouts and errors as
 * fa_fwd and fa_bwd.
 *   bias : fp32, caller-owned device memory; element (b, h, i, j) for batch
 *          entry b, query head h, query row i, key j is
 *          bias[b*bias_stride_b + h*bias_stride_h + i*bias_stride_q + j]
 *          and must be readable for every b < B, h < Hq, i < Nq, j < Nk.
 *          A stride of 0 broadcasts (e.g. one [Nq, Nk] bias for all heads,
 *          or a key-padding row with bias_stride_q = 0).
 *   bias_stride_* : element strides, >= 0
 * Returns FA_ERR_INVALID_ARG, in addition to fa_fwd's cases, for a NULL or
 * not 4-byte-aligned bias or a negative stride, and FA_ERR_UNSUPPORTED when
 * (31 * bias_stride_q + Nk) * 4 >= 2^32 (the kernels address 32 bias rows
 * of one head through one 32-bit byte range).  Entries must be finite or
 * -inf.
 */
int fa_fwd_bias(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int Nq, int Nk, int d,
                float scale, int causal, int window,
                const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                int64_t bias_stride_q, void* stream);
int fa_bwd_bias(const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes,
                int B, int Hq, int Hkv, int Nq, int Nk, int d,
                float scale, int causal, int window,
                const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                int64_t bias_stride_q, void* stream);

/*
 * Forward and backward with dropout on the attention probabilities
 * (inferensys.com glossary "FlashAttention", the paragraph on the single
 * fused kernel, lists dropout among the operations fused into one pass).
 * O = (P * Z / (1 - p)) V, where P is the softmax of fa_fwd and Z is a 0/1
 * keep-mask; LSE is that of the undropped P (as fa_fwd), so fa_bwd_dropout
 * rebuilds P from it and regenerates Z instead of storing it.  Gradients: dV = (P Z / (1 - p))^T dO,
 * dP = (dO V^T) Z / (1 - p), D_i = sum_c dO_ic O_ic, dS = P (dP - D).
 * The pages fix no random number generator; this library's mask is:
 *   element (b, h, i, j) -- batch entry or packed sequence b, query head h,
 *   query row i and key j counted from the start of the sequence -- reads
 *   Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
 *   As Easy as 1, 2, 3", SC 2011) at counter
 *   (2 floor(j / 16) + (floor(j / 4) mod 2), i, h, b) with key
 *   (seed mod 2^32, floor(seed / 2^32)); with s = 4 (floor(j / 8) mod 2) +
 *   (j mod 4), its 16-bit slot is half (s mod 2) (0 = low) of output word
 *   floor(s / 2).  The key is kept iff the slot >= T = floor(p * 2^16), p
 *   being dropout_p widened to double, and kept probabilities are scaled by
 *   2^16 / (2^16 - T), the inverse of the exact keep probability (the
 *   1 / (1 - p) of the formulas above).
 * The same seed and dropout_p must be passed to the forward and the
 * backward.  dropout_p = 0 gives exactly fa_fwd / fa_bwd.  Other arguments,
 * layouts and errors as fa_fwd and fa_bwd (dense or packed batches), plus
 * FA_ERR_INVALID_ARG for dropout_p outside [0, 1) or NaN.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   float scale, int causal, int window,
                   const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                   void* stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   float scale, int causal, int window,
                   const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                   void* stream);

/*
 * Split-KV attention for a few query rows per sequence over a long key/value
 * cache: single-token decode and short chunked prefill, where the cost is
 * streaming the cached keys and values (klaylearn.com glossary
 * "flash-attention", "Does FlashAttention speed up every LLM inference
 * path?").  Same result as fa_fwd on each sequence's first seqlens_k[b] keys:
 * the key range is split over work-groups, each runs the online softmax over
 * its range, and the partial results are merged exactly through their
 * logsumexps (LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s).
 *   q, o      : bf16 [B, Nq, Hq, d]
 *   k, v      : bf16 [B, Nk, Hkv, d], a cache of capacity Nk per sequence
 *   lse       : fp32 [B, Hq, Nq]
 *   seqlens_k : NULL (every sequence uses all Nk keys) or device int32[B],
 *               keys used by sequence b (clamped to [0, Nk]); query position
 *               i of sequence b sits at key position i + seqlens_k[b] - Nq
 *               for the causal and window masks (bottom-right alignment)
 *   num_splits: 1..1024 key-range splits; fa_decode_num_splits gives a
 *               default that fills the GPU
 *   workspace : device buffer of at least
 *               fa_decode_workspace_size(B, Hq, Nq, d, num_splits) bytes,
 *               16-byte aligned, scratch for the partial results; it must
 *               not alias any other argument
 * Other arguments, mask conventions and errors as fa_fwd (no packed
 * batches), plus FA_ERR_INVALID_ARG for num_splits out of range, a
 * misaligned seqlens_k, or a NULL or too small workspace.  Costs O(Nk) per
 * row; every K/V byte of a KV head is read once for its whole query group.
 */
size_t fa_decode_workspace_size(int B, int Hq, int Nq, int d, int num_splits);
int fa_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nk);
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int Nq, int Nk, int d,
              float scale, int causal, int window,
              const int32_t* seqlens_k, int num_splits,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library routine): the split partials live in a
 * static device array of FA_DECODE_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds from the library's load until the process ends.
 *   Arguments as fa_decode, without workspace and workspace_bytes;
 *   num_splits == 0 picks fa_decode_num_splits' count, lowered to
 *   fa_decode_noalloc_max_splits so that the partials fit.
 *   Returns FA_ERR_TOO_LARGE, before enqueueing anything, when the partials
 *   of the request (fa_decode_workspace_size bytes) exceed the array;
 *   FA_ERR_INVALID_ARG also when `stream` belongs to another device than the
 *   current one.  The results are bit for bit those of fa_decode with the
 *   same num_splits.
 *   The array is shared by every call on a GPU and keeps the last call's
 *   contents; nothing in it needs to start at zero (every partial a call
 *   reads, the same call writes first).  Calls that overlap on one GPU (two
 *   streams, or two host threads with work in flight at once) race on it
 *   and corrupt each other's results: serialise them.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
int fa_decode_noalloc_max_splits(int B, int Hq, int Nq, int d);
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      float scale, int causal, int window,
                      const int32_t* seqlens_k, int num_splits, void* stream);

/*
 * FP8 forward (llms.blog "FlashAttention: How IO-Aware Tiling and Online
 * Softmax Solved Transformer Memory Bottlenecks", "FlashAttention-3:
 * Asynchronous Execution on Hopper Architectures": 8-bit floating point with
 * block quantization and incoherent processing).  Dense batches only.
 *
 * Codes are OCP FP8 E4M3 bytes (bias 7, 3 mantissa bits, largest finite
 * 448, S.1111.111 NaN).  Every block of 64 consecutive tokens of one head
 * (all d columns) has one fp32 scale; the value of a code c of token n is
 * e4m3(c) * scale[b, h, n / 64].
 *
 * fa_quantize_fp8: block quantization of a bf16 tensor.
 *   x         : bf16 [B, N, H, d]
 *   signs     : NULL, or device fp32[d] of +1 / -1: each row is first rotated
 *               to x D H / sqrt(d) (D = diag(signs), H the Sylvester-
 *               Hadamard matrix, H[i][j] = (-1)^popcount(i & j)); pass the
 *               same signs for Q and K (the scores are unchanged, an outlier
 *               coordinate is spread over the row), none for V
 *   transpose : 0 -> x8 is [B, N, H, d] (the layout of Q and K);
 *               1 -> x8 is [B, H, d, ldn], ldn = N rounded up to 64, keys
 *               innermost, padding written as zeros (the layout V takes)
 *   scales    : fp32 output [B, H, ceil(N / 64)]
 * Per block, in fp32: amax = max |x| (after the rotation), scale = amax / 448,
 * code = RNE_e4m3(clamp(x * (448 / amax), -448, 448)); a block with
 * amax < 2^-119 gets scale 1 and zero codes.  NaN inputs give NaN codes.
 * x, x8 16-byte aligned, scales and signs 4-byte aligned.  Errors:
 * FA_ERR_INVALID_ARG (null or misaligned pointer, size < 1, transpose not 0
 * or 1), FA_ERR_UNSUPPORTED (d not 64 or 128).
 *
 * fa_fwd_fp8: attention of the quantized problem,
 *   S = scale * (sQ Q~)(sK K~)^T (+ causal / window masks),
 *   O = softmax(S) (sV V~) in bf16, LSE as fa_fwd.
 *   q8        : E4M3 [B, Nq, Hq, d];  k8 : E4M3 [B, Nk, Hkv, d]
 *   vt8       : E4M3 [B, Hkv, d, ldv], ldv = Nk rounded up to 64 (what
 *               fa_quantize_fp8 writes with transpose = 1); the padding keys
 *               must hold finite codes (zeros)
 *   q_scale   : fp32 [B, Hq, ceil(Nq / 64)];  k_scale, v_scale : fp32
 *               [B, Hkv, ceil(Nk / 64)]; positive and finite
 *   o         : bf16 [B, Nq, Hq, d];  lse : fp32 [B, Hq, Nq]
 * Both products run on the 8-bit matrix cores, so the probabilities are
 * rounded to E4M3 before they multiply V (relative error <= 2^-4 of each
 * term of O); the row normaliser and LSE use the unrounded values.  Other
 * arguments, masks and errors as fa_fwd (no packed batches), plus
 * FA_ERR_UNSUPPORTED when (d - 1) * ldv + 64 >= 2^32.
 */
int fa_quantize_fp8(const void* x, void* x8, float* scales, int B, int N, int H, int d,
                    int transpose, const float* signs, void* stream);
int fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* q_scale,
               const float* k_scale, const float* v_scale, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d,
               float scale, int causal, int window, void* stream);

/* Static, human-readable name of a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
