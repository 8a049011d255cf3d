/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact-attention library.
 *
 * The library computes exact scaled-dot-product attention
 *
 *     O = softmax(scale * Q K^T + mask) V
 *
 * without writing the N x N score or probability matrices to device memory:
 * K/V are streamed through on-chip tiles and per-row (m, l, O~) states are
 * merged with the online-softmax rescaling rule (page 1, "注意力为什么受限于
 * 显存带宽：用算术强度与分块把 FlashAttention 推导清楚", section 六; page 2,
 * "4. FlashAttention 深度剖析", 4.2.3-4.2.4 and the tiled forward of 4.3.2).
 * The backward pass recomputes the probabilities from the saved per-row
 * logsumexp, P_ij = exp(S_ij - L_i) (page 1 section 八; page 2 4.3.4).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout:    every tensor Q, K, V, O, dO, dQ, dK, dV is a contiguous
 *            [batch, heads, n, d] array (d fastest); LSE is a contiguous
 *            [batch, heads, n] float32 array. Queries and keys have the same
 *            length n (self-attention). The *_gqa entry points take K, V, dK
 *            and dV as [batch, heads_kv, n, d] instead (grouped K/V heads,
 *            below); the *_varlen entry points take packed batches (below).
 * Pointers:  device pointers (memory from hipMalloc or an allocator on top of
 *            it), at least 16-byte aligned. The caller owns every buffer;
 *            the library only borrows pointers until the work it enqueued on
 *            `stream` has finished. The library never allocates, frees or
 *            synchronises the host.
 * dtype:     FA_BF16 -- Q, K, V, O, dO, dQ, dK, dV are bfloat16; products on
 *            bf16 matrix cores with float32 accumulation; the probabilities
 *            are rounded to bf16 before the P V product; outputs rounded to
 *            nearest-even. FA_FP32 -- every tensor is float32 and every step
 *            computes in float32 (no bf16 rounding anywhere).
 * d:         64, 128 or 256 (bf16 and fp32).
 * Sizes:     1 <= n <= 2^22 (packed batches: max_seqlen, with total >=
 *            max_seqlen); one head's rows must occupy less than 2 GiB
 *            (rows x d x element size < 2^31 bytes); otherwise FA_E_SHAPE.
 * Masks:     causal != 0 hides key j from query i when j > i (the upper-right
 *            triangle). kv_len, when not NULL, is a device int32[batch]; key
 *            j of batch b is hidden from every query row when
 *            j >= kv_len[b]. Every query row is computed, padded or not.
 *            Hidden probabilities are exactly 0; a row with no visible key
 *            gets O = 0, LSE = -inf and zero gradients.
 * Scale:     softmax_scale is any finite float (0 gives uniform weights over
 *            the visible keys). The usual choice is 1/sqrt(d).
 * LSE:       LSE_i = ln sum_j exp(scale * q_i . k_j) over the visible keys,
 *            natural logarithm, float32 (page 2, 4.3.2: L = m + log l).
 * Streams:   `stream` is a hipStream_t (NULL = the null stream). All work is
 *            enqueued asynchronously on it; nothing is enqueued elsewhere.
 * Errors:    arguments are validated synchronously, before anything is
 *            enqueued; on a validation error nothing is written and a
 *            FA_E_* code is returned. A failed kernel launch returns
 *            FA_E_LAUNCH. Faults during execution surface at the caller's
 *            next synchronisation, as with any HIP kernel.
 * Grouped K/V heads (GQA, MQA): heads_kv divides heads, and query head h
 *            attends with K/V head h / (heads / heads_kv): consecutive runs
 *            of heads / heads_kv query heads share one K/V head. heads_kv =
 *            heads is ordinary multi-head attention, heads_kv = 1 multi-query
 *            attention. The gradient of a shared K/V head is the sum over the
 *            query heads that use it. (Grouped and multi-query attention as
 *            supported variants: page 1, section 九; page 4, "FlashAttention
 *            原理深入剖析（下篇）", section 六.)
 * Packed variable-length batches (*_varlen): num_seqs sequences stored
 *            back to back, head by head: Q, O, dO, dQ are [heads, total, d],
 *            K, V, dK, dV [heads_kv, total, d], LSE [heads, total] float32.
 *            cu_seqlens is a device int32[num_seqs + 1] of offsets:
 *            sequence s is rows cu_seqlens[s] .. cu_seqlens[s+1] - 1 of
 *            every head, and attends only to itself; causal positions count
 *            from its first row (a block-diagonal mask over the total rows).
 *            The offsets must start at 0, be non-decreasing, and no length
 *            may exceed max_seqlen. They are read on the device only (no
 *            host synchronisation); the kernels clamp them to [0, total] and
 *            each length to max_seqlen, so other values cannot cause an
 *            out-of-bounds access, and rows outside every sequence are left
 *            unwritten. (Variable-length batches without padding: page 2,
 *            "4. FlashAttention 深度剖析", 4.7.2 and 4.7.4.)
 * Windows and block-sparse masks (*_masked, *_varlen: the fa_mask
 *            argument, NULL for none): a window (window_left, window_right)
 *            hides key j from query i when j < i - window_left or
 *            j > i + window_right (a side of -1 is unbounded; positions
 *            count within each sequence). A block mask is a boolean matrix
 *            over FA_BLOCK x FA_BLOCK blocks (query block i / FA_BLOCK, key
 *            block j / FA_BLOCK) that hides every key of a block that is not
 *            set; it is passed as an index built once per mask by
 *            fa_block_index_build, and blocks that are not set are skipped
 *            entirely. All masks combine by AND; a query row left with no
 *            visible key gets O = 0, LSE = -inf and zero gradients. (The
 *            window_size argument of the flash-attn call: page 4,
 *            "FlashAttention 原理深入剖析（下篇）", section 六, and page 2,
 *            4.8.1; the block-level mask: page 3, "深入浅出 FlashAttention",
 *            第八部分.)
 * Threads:   entry points are reentrant; concurrent calls on different
 *            streams may share inputs but must not share outputs.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 6

typedef enum { FA_BF16 = 0, FA_FP32 = 1 } fa_dtype;

/* Side of a block of the block-sparse mask, in rows and in keys. */
#define FA_BLOCK 128

/*
 * Optional masks beyond causal and key padding (see the conventions above).
 * block_index: NULL, or a device array written by fa_block_index_build for
 * the same sequence length n (packed batches: max_seqlen); it must stay
 * unchanged while calls that use it are in flight.
 */
typedef struct {
  int64_t window_left;   /* -1: unbounded */
  int64_t window_right;  /* -1: unbounded */
  const int32_t* block_index;
} fa_mask;

typedef enum {
  FA_OK = 0,
  FA_E_NULLPTR = 1,     /* a required pointer is NULL                        */
  FA_E_SHAPE = 2,       /* bad batch, heads, heads_kv, n or total            */
  FA_E_UNSUPPORTED = 3, /* d not in {64,128,256}, unknown dtype, bad scale   */
  FA_E_WORKSPACE = 4,   /* workspace NULL or smaller than required           */
  FA_E_ALIAS = 5,       /* an output overlaps an input or another output     */
  FA_E_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch          */
  FA_E_ALIGN = 7,       /* a pointer is not 16-byte aligned                  */
  FA_E_SCRATCH = 8      /* fa_bwd_noalloc: the call needs more scratch than
                           FA_NOALLOC_SCRATCH_BYTES                          */
} fa_status;

/*
 * fa_fwd -- forward pass (page 2, 4.3.2: tiled forward with deferred
 * normalisation, storing L_i = m_i + log l_i).
 *
 *   q, k, v : inputs, [batch, heads, n, d] of `dtype`.
 *   kv_len  : device int32[batch] key lengths, each in [1, n], or NULL
 *             (no key padding). Values are trusted: the kernels clamp them
 *             to [0, n], so an out-of-range value cannot cause an
 *             out-of-bounds access.
 *   o       : output, [batch, heads, n, d] of `dtype`, overwritten.
 *   lse     : output, float32 [batch, heads, n], overwritten.
 *
 * o and lse must not overlap each other or any input.
 */
fa_status fa_fwd(int64_t batch, int64_t heads, int64_t n, int64_t d,
                 int causal, float softmax_scale, fa_dtype dtype,
                 const void* q, const void* k, const void* v,
                 const int32_t* kv_len,
                 void* o, float* lse,
                 void* stream);

/*
 * fa_fwd_gqa -- fa_fwd with grouped K/V heads: k and v are
 * [batch, heads_kv, n, d]; q, o and lse as for fa_fwd. heads_kv must be in
 * [1, heads] and divide heads (else FA_E_SHAPE). fa_fwd(...) is
 * fa_fwd_gqa(batch, heads, heads, ...).
 */
fa_status fa_fwd_gqa(int64_t batch, int64_t heads, int64_t heads_kv,
                     int64_t n, int64_t d,
                     int causal, float softmax_scale, fa_dtype dtype,
                     const void* q, const void* k, const void* v,
                     const int32_t* kv_len,
                     void* o, float* lse,
                     void* stream);

/*
 * fa_fwd_masked -- fa_fwd_gqa with the optional window and block-sparse
 * masks (mask may be NULL). Window sides below -1 return FA_E_SHAPE; a
 * block index for n > 1024 * FA_BLOCK returns FA_E_UNSUPPORTED; the index
 * must be 4-byte aligned and must not overlap an output.
 */
fa_status fa_fwd_masked(int64_t batch, int64_t heads, int64_t heads_kv,
                        int64_t n, int64_t d,
                        int causal, float softmax_scale, fa_dtype dtype,
                        const void* q, const void* k, const void* v,
                        const int32_t* kv_len, const fa_mask* mask,
                        void* o, float* lse,
                        void* stream);

/*
 * fa_fwd_varlen -- forward over a packed variable-length batch (layout and
 * offsets as described above). total >= max_seqlen >= 1; q, o: [heads,
 * total, d]; k, v: [heads_kv, total, d]; lse: float32 [heads, total]. No key
 * padding argument: each sequence's keys are exactly its rows. mask: as for
 * fa_fwd_masked (NULL for none), positions and blocks counted within each
 * sequence, the block index built for n = max_seqlen.
 */
fa_status fa_fwd_varlen(int64_t num_seqs, int64_t heads, int64_t heads_kv,
                        int64_t total, int64_t max_seqlen, int64_t d,
                        const int32_t* cu_seqlens,
                        int causal, float softmax_scale, fa_dtype dtype,
                        const void* q, const void* k, const void* v,
                        const fa_mask* mask,
                        void* o, float* lse,
                        void* stream);

/*
 * fa_bwd_workspace_bytes -- size of the scratch buffer fa_bwd needs: two
 * float32 vectors, D_i = sum_k dO_ik O_ik and L_i log2(e), each with the
 * rows of every (batch entry, head) padded to a multiple of 64, each rounded
 * up to 256 bytes. Returns 0 for invalid sizes. The size depends on the
 * query heads only, so it serves fa_bwd_gqa too; for fa_bwd_varlen pass
 * batch = num_seqs and n = max_seqlen.
 */
size_t fa_bwd_workspace_bytes(int64_t batch, int64_t heads, int64_t n,
                              int64_t d, fa_dtype dtype);

/*
 * fa_bwd -- backward pass: the gradients of f = sum(O * dO) with respect to
 * Q, K and V, recomputing P_ij = exp(scale q_i.k_j - L_i) tile by tile from
 * the saved LSE (page 1 section 八; page 2 4.3.4). With dS = P * (dP - D),
 * dP = dO V^T and D_i = sum_k dO_ik O_ik:
 *     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
 *
 *   q, k, v, o, d_o : inputs, [batch, heads, n, d] of `dtype`; o is the
 *                     forward output for the same arguments.
 *   lse             : input, float32 [batch, heads, n], from fa_fwd.
 *   kv_len          : as for fa_fwd (must match the forward call).
 *   dq, dk, dv      : outputs, [batch, heads, n, d] of `dtype`; overwritten,
 *                     not accumulated into.
 *   workspace       : device scratch of at least
 *                     fa_bwd_workspace_bytes(batch, heads, n, d, dtype)
 *                     bytes, 256-byte aligned; contents on entry are
 *                     ignored and undefined on exit.
 *
 * Outputs and the workspace must not overlap each other or any input.
 * bf16: dK and dV come from a key-outer kernel and dQ from a query-outer
 * kernel, each accumulated in registers and written once, so all three are
 * bitwise deterministic. fp32: dQ is accumulated into dq with float atomics,
 * so its last bits may differ from run to run.
 */
fa_status fa_bwd(int64_t batch, int64_t heads, int64_t n, int64_t d,
                 int causal, float softmax_scale, fa_dtype dtype,
                 const void* q, const void* k, const void* v,
                 const void* o, const void* d_o, const float* lse,
                 const int32_t* kv_len,
                 void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * fa_bwd_gqa -- fa_bwd with grouped K/V heads: k, v, dk and dv are
 * [batch, heads_kv, n, d]; every other tensor as for fa_bwd. dK and dV of a
 * K/V head are the sums of the gradients through each query head of its
 * group; they are accumulated in registers by the workgroup that owns the
 * key tile, in a fixed head order, and written once, so they stay bitwise
 * deterministic in bf16. heads_kv as for fa_fwd_gqa.
 */
fa_status fa_bwd_gqa(int64_t batch, int64_t heads, int64_t heads_kv,
                     int64_t n, int64_t d,
                     int causal, float softmax_scale, fa_dtype dtype,
                     const void* q, const void* k, const void* v,
                     const void* o, const void* d_o, const float* lse,
                     const int32_t* kv_len,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * fa_bwd_masked -- fa_bwd_gqa with the optional masks of fa_fwd_masked
 * (the same mask as the forward call).
 */
fa_status fa_bwd_masked(int64_t batch, int64_t heads, int64_t heads_kv,
                        int64_t n, int64_t d,
                        int causal, float softmax_scale, fa_dtype dtype,
                        const void* q, const void* k, const void* v,
                        const void* o, const void* d_o, const float* lse,
                        const int32_t* kv_len, const fa_mask* mask,
                        void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * fa_bwd_varlen -- backward over a packed variable-length batch: the
 * gradients of fa_bwd for each sequence on its own, with the layouts of
 * fa_fwd_varlen (dq like q; dk, dv like k, v) and the mask of the forward
 * call. workspace: at least
 * fa_bwd_workspace_bytes(num_seqs, heads, max_seqlen, d, dtype) bytes. Rows
 * outside every sequence are left unwritten.
 */
fa_status fa_bwd_varlen(int64_t num_seqs, int64_t heads, int64_t heads_kv,
                        int64_t total, int64_t max_seqlen, int64_t d,
                        const int32_t* cu_seqlens,
                        int causal, float softmax_scale, fa_dtype dtype,
                        const void* q, const void* k, const void* v,
                        const void* o, const void* d_o, const float* lse,
                        const fa_mask* mask,
                        void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd_gqa for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments and results as fa_bwd_gqa, without the
 * workspace: the library uses a static device array of
 * FA_NOALLOC_SCRATCH_BYTES bytes instead, one copy on each device it runs on,
 * held until the process ends. The call allocates and frees nothing.
 *
 * Limit: calls whose fa_bwd_workspace_bytes(batch, heads, n, d, dtype)
 * exceeds FA_NOALLOC_SCRATCH_BYTES (16 MiB: batch x heads x n up to about
 * 2^21 rows, e.g. 32 heads of 65536 or 128 heads of 16384) return
 * FA_E_SCRATCH before anything is enqueued; use fa_bwd_gqa for them.
 * Every call on one device shares that device's array, and the array keeps
 * whatever the last call left in it (each call writes every element it reads
 * before reading it, so leftovers are never used). Calls that overlap in time
 * on one device -- on different streams, or from different threads without
 * ordering -- race on the array and give undefined results; calls ordered on
 * one stream are safe. The array's device address is looked up on a device's
 * first call (a HIP runtime query made with the stream's device current);
 * make that first call outside graph capture. A failed lookup returns
 * FA_E_LAUNCH.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

fa_status fa_bwd_noalloc(int64_t batch, int64_t heads, int64_t heads_kv,
                         int64_t n, int64_t d,
                         int causal, float softmax_scale, fa_dtype dtype,
                         const void* q, const void* k, const void* v,
                         const void* o, const void* d_o, const float* lse,
                         const int32_t* kv_len,
                         void* dq, void* dk, void* dv,
                         void* stream);

/*
 * fa_block_index_bytes -- size of the block-sparse index for sequence
 * length n: 4 * (2 (nb + 1) + 2 nb^2) bytes with nb = ceil(n / FA_BLOCK).
 * Returns 0 unless 1 <= n and nb <= 1024.
 */
size_t fa_block_index_bytes(int64_t n);

/*
 * fa_block_index_build -- builds the index of a block mask for sequence
 * length n. block_mask: device uint8 [nb][nb] (row = query block, column =
 * key block; nonzero = visible). index: device int32 output of
 * fa_block_index_bytes(n) bytes, 4-byte aligned, not overlapping the mask:
 * for every query block the ascending list of its visible key blocks and
 * for every key block the ascending list of the query blocks that see it.
 * Enqueued on `stream` (one small kernel); reuse the index for every call
 * with that mask.
 */
fa_status fa_block_index_build(int64_t n, const uint8_t* block_mask,
                               int32_t* index, void* stream);

/*
 * fa_bwd_timed -- fa_bwd_gqa, additionally recording caller-owned HIP events on
 * `stream` between its kernels, for measurement harnesses that time each
 * kernel with events. events[0] is recorded at the start; bf16: events[1]
 * after the dQ kernel (which also forms D_i and L_i log2 e), i.e. before the
 * dK/dV kernel, and events[2] after it; fp32: events[1] after the D_i kernel,
 * before the single backward kernel, events[2] after it; events[3] at the
 * end (with events[2]). Any entry may
 * be NULL (not recorded); `events` itself may be NULL, which makes the call
 * identical to fa_bwd_gqa. The events must have been created on the device that
 * owns `stream` (hipEventCreate); the library records them and nothing else.
 * A failed hipEventRecord returns FA_E_LAUNCH.
 */
fa_status fa_bwd_timed(int64_t batch, int64_t heads, int64_t heads_kv,
                       int64_t n, int64_t d,
                       int causal, float softmax_scale, fa_dtype dtype,
                       const void* q, const void* k, const void* v,
                       const void* o, const void* d_o, const float* lse,
                       const int32_t* kv_len,
                       void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes,
                       void* stream, void* const events[4]);

/*
 * FP8 forward (page 2, "4. FlashAttention 深度剖析", 4.5.4: E4M3 operands in
 * the forward, one scale per block recorded when the block is encoded, FP32
 * accumulation, optional random Hadamard rotation of Q and K; exercise 3:
 * E4M3's largest magnitude is 448 and its smallest normal 2^-6).
 *
 * E4M3 here is the 1-4-3 format with exponent bias 7, subnormals, no
 * infinities and S.1111.111 as NaN. A tensor [batch, heads, n, d] is encoded
 * in blocks of FA_BLOCK rows of one head (np = n rounded up to a multiple of
 * FA_BLOCK, nb = np / FA_BLOCK blocks per head):
 *   codes  -- uint8, batch * heads * np * d bytes, in one of two layouts:
 *             FA_FP8_ROWS  [batch, heads, np, d] (Q and K),
 *             FA_FP8_VT    [batch, heads, nb, d, FA_BLOCK]: every block
 *                          transposed, channel-major (V);
 *             codes of rows n .. np - 1 are zero;
 *   scales -- float32 [batch, heads, nb]; block b stands for
 *             scales[b] * decode(codes of b).
 * The scale of a block is 2^e with e the smallest integer such that the
 * block's largest magnitude is at most 448 * 2^e (e = 0 for an all-zero
 * block), so x * 2^-e is exact and the only rounding is E4M3's own (to
 * nearest, ties to even). With a rotation the encoded block is x R with
 * R = diag(signs) H_d (H_d the Sylvester Hadamard matrix, entries +-1) and
 * the stored scale is 2^e / sqrt(d): scale * codes approximates x R / sqrt(d),
 * the page's x H. Rotating Q and K with the same signs leaves Q K^T
 * unchanged.
 */
#define FA_FP8_ROWS 0
#define FA_FP8_VT 1

/* Bytes of the codes and of the scales of a [batch, heads, n, d] tensor;
 * 0 for invalid sizes. */
size_t fa_fp8_codes_bytes(int64_t batch, int64_t heads, int64_t n, int64_t d);
size_t fa_fp8_scales_bytes(int64_t batch, int64_t heads, int64_t n);

/*
 * fa_fp8_quantize -- encodes the bf16 tensor x [batch, heads, n, d]
 * (d = 64, 128 or 256, else FA_E_UNSUPPORTED) into `codes` (layout FA_FP8_ROWS or
 * FA_FP8_VT, else FA_E_UNSUPPORTED) and `scales`, as described above.
 * signs: NULL (no rotation) or a device int8[d] of +1 / -1 entries (any
 * negative value counts as -1), 16-byte aligned; a rotation with the
 * FA_FP8_VT layout returns FA_E_UNSUPPORTED (V is not rotated). Outputs
 * must not overlap x, signs or each other. Sizes as for fa_fwd; x, codes
 * 16-byte aligned, scales 4-byte aligned. x must be finite; blocks whose
 * largest magnitude lies below 2^-100 or above 2^120 are outside the
 * supported range.
 */
fa_status fa_fp8_quantize(int64_t batch, int64_t heads, int64_t n, int64_t d,
                          int layout, const void* x, const int8_t* signs,
                          uint8_t* codes, float* scales, void* stream);

/*
 * fa_fwd_fp8 -- attention forward on encoded operands: q8 (FA_FP8_ROWS,
 * [batch, heads, np, d]), k8 (FA_FP8_ROWS, [batch, heads_kv, np, d]), v8
 * (FA_FP8_VT, [batch, heads_kv, nb, d, FA_BLOCK]) with their scales; d = 64,
 * 128 or 256 (else FA_E_UNSUPPORTED); grouped heads, causal, kv_len and softmax_scale
 * as for fa_fwd_gqa. Both products run on the E4M3 matrix cores with FP32
 * accumulation. With t_ij = softmax_scale * log2(e) * (sq q^_i . sk k^_j)
 * and the integer row frame f_i = ceil(max_j t_ij) over the visible keys,
 * the probabilities enter the P V product as P^_ij = E4M3(2^(t_ij - f_i + 8))
 * and
 *     O_i   = sum_j P^_ij sv v^_j / l_i,
 *     l_i   = sum_j P^_ij   (the sum of the ROUNDED probabilities, taken on
 *             the matrix cores with the same operands as the P V product),
 *     LSE_i = ln 2 * (f_i - 8 + log2 l_i)   (natural log of the row's sum
 *             of exp(scores), up to the rounding of the probabilities: each
 *             is within half an E4M3 step, 2^-4 relative, of its exact
 *             value, so LSE_i is within ln(1 + 2^-4) of the exact one),
 * up to the matrix cores' fp32 accumulation. The frame is an integer, so the
 * rounding of a probability does not depend on the order in which the key
 * tiles are visited. o: bf16 [batch, heads, n, d]; lse: float32 [batch,
 * heads, n]; hidden keys and empty rows as for fa_fwd. The V scales must be
 * powers of two (as fa_fp8_quantize writes them; only each entry's
 * exponent is used); Q and K scales are any positive floats. Code pointers
 * and o 16-byte aligned; scales, lse and kv_len 4-byte aligned; outputs
 * must not overlap any input or each other.
 */
fa_status fa_fwd_fp8(int64_t batch, int64_t heads, int64_t heads_kv,
                     int64_t n, int64_t d, int causal, float softmax_scale,
                     const uint8_t* q8, const float* q_scales,
                     const uint8_t* k8, const float* k_scales,
                     const uint8_t* v8, const float* v_scales,
                     const int32_t* kv_len,
                     void* o, float* lse, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_str(fa_status s);

/* FA_ABI_VERSION of the library that was loaded. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
