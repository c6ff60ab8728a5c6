/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * The library computes exact attention O = softmax(scale * Q K^T) V with the
 * tiled, IO-aware method: one fused forward kernel that never writes the N x N
 * score matrix to HBM and saves only O and one log-sum-exp per row, and a
 * backward that recomputes the probabilities block by block from that
 * statistic ("FlashAttention: Fast and Memory-Efficient Exact Attention with
 * IO-Awareness", reading notes (hackmd): §Background › Standard Attention
 * Implementation for S, P and O; §Algorithm › Tiling, Recomputation and Kernel
 * Fusion for the method; §Introduction › Block-sparse FlashAttention for the
 * block-sparse variant).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors.  Q, K, V, O, dO, dQ, dK, dV are [B, H, N, d] arrays of the
 *   descriptor's dtype whose last dimension is contiguous; element (b, h, n, i)
 *   lives at base + b*stride_b + h*stride_h + n*stride_n + i (strides in
 *   elements, shared by all of them). Queries and keys have the same length N.
 *   LSE is a contiguous float32 [B, H, N] array.
 * Pointers.  Every tensor, key_len, block_mask and workspace pointer is a
 *   DEVICE pointer owned by the caller; the library never allocates or frees
 *   device memory. Base pointers must be 16-byte aligned, and every stride times
 *   the bytes per element a multiple of 16. Outputs must not alias inputs.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream). Work is
 *   enqueued on it and the call returns without synchronising: inputs must stay
 *   alive, and outputs must not be read, until the stream reaches that point.
 * Masking.  Entry (i, j) of S is kept iff every active mask keeps it; masked
 *   entries are -inf before the softmax, so they get probability 0:
 *     causal != 0   keeps key j for query i iff j <= i;
 *     key_len       (device int32 [B], or NULL) keeps key j iff j < key_len[b]
 *                   (values are clamped to [0, N] on the device);
 *     block_mask    (block-sparse calls) keeps (i, j) iff
 *                   block_mask[(i / bs) * (N / bs) + j / bs] != 0.
 *   A query row with no kept key gets O = 0, LSE = -inf and no gradient.
 * Numbers.  All products accumulate in float32. bf16 outputs are rounded to
 *   nearest even. LSE[i] = m_i + ln(l_i), natural log, where m_i is the row
 *   max of the scaled, masked S and l_i the float32 row sum of exp(S - m_i)
 *   (reading notes, §Algorithm › Tiling: the running row sum). In the bf16
 *   forward the P V product takes the probabilities rounded to bf16, and O is
 *   normalised by the sum of exactly those rounded weights (so O stays a convex
 *   combination of V rows); LSE uses the unrounded sum.
 *   `scale` must be finite and >= 0. Inputs must be finite.
 * Errors.  Every call returns FA_OK (0) or a negative FA_ERR_* code. Argument
 *   checks run before anything is enqueued; a failed check enqueues nothing.
 *   FA_ERR_HIP reports a launch error from the HIP runtime.
 * Threads.  Calls are reentrant and thread-safe: they share no state and take
 *   no lock. (The optional kernel timer below keeps its state per calling
 *   thread.)
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_VERSION 104

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID = -1,     /* null pointer, bad shape, stride, alignment or scale */
  FA_ERR_UNSUPPORTED = -2, /* d not in {64, 128}, or dtype not built for this call */
  FA_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required */
  FA_ERR_HIP = -4,         /* the HIP runtime reported an error at launch */
  FA_ERR_SCRATCH = -5      /* fa_bwd_noalloc: more workspace than its static scratch holds */
};

enum fa_dtype { FA_BF16 = 0, FA_F32 = 1 };

typedef struct fa_desc {
  int32_t B, H, N, d; /* batch, heads, sequence length (1 .. 2^30), head dim (64 or 128);
                          FA_ERR_UNSUPPORTED when B H >= 2^31, B H N > 2^40 or N > 2^30 */
  int32_t dtype;      /* FA_BF16 or FA_F32 */
  int32_t reserved;   /* must be 0 */
  int64_t stride_b, stride_h, stride_n; /* element strides; the d stride is 1. stride_n
                          must be below 2^23 elements (FA_ERR_UNSUPPORTED otherwise: the
                          tile copies form a lane's offset within 256 rows in 32 bits) */
} fa_desc;

/* Forward: O = softmax(scale * Q K^T + mask) V and LSE (see above).
 * Reads Q, K, V (and key_len); writes O and LSE. bf16 and fp32.
 * Defines: S = QK^T, P = softmax(S), O = PV (reading notes, §Background ›
 * Standard Attention Implementation), computed tile by tile with the running
 * row max and row sum of §Algorithm › Tiling; only O, m and l leave the chip
 * (§Recomputation), stored here as LSE = m + ln l. */
int fa_fwd(const fa_desc* desc, const void* Q, const void* K, const void* V, float scale,
           int causal, const int32_t* key_len, void* O, float* LSE, void* stream);

/* Bytes of device workspace fa_bwd needs: two float32 values per row
 * (rowsum(dO o O) and the base-2 LSE), i.e. O(N) per head and never O(N^2)
 * (the linear extra memory of Theorem 1, anthology LIT-074 key takeaways). */
size_t fa_bwd_workspace_bytes(const fa_desc* desc);

/* Backward: the gradient of <dO, O> with respect to Q, K and V, given the O and
 * LSE that fa_fwd produced for the same Q, K, V, scale, causal and key_len.
 * Recomputes P = exp(scale * Q K^T - LSE) tile by tile (reading notes,
 * §Algorithm › Recomputation), then dV = P^T dO, dP = dO V^T,
 * dS = P o (dP - rowsum(dO o O)), dQ = scale dS K, dK = scale dS^T Q.
 * Keys that no query may see get dK = dV = 0. bf16 only (fp32:
 * FA_ERR_UNSUPPORTED). `workspace` must hold fa_bwd_workspace_bytes(desc)
 * bytes; its contents on entry are ignored. */
int fa_bwd(const fa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
           const void* dO, const float* LSE, float scale, int causal, const int32_t* key_len,
           void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace the block-sparse calls need for block_size `bs`:
 * none for the forward (each workgroup reads its own row of the block mask),
 * the fa_bwd workspace for the backward. Returns 0 for an invalid descriptor or
 * block size. */
size_t fa_blocksparse_workspace_bytes(const fa_desc* desc, int32_t block_size, int backward);

/* Block-sparse forward: fa_fwd restricted to the nonzero blocks of
 * `block_mask` (device uint8 [N/bs][N/bs], row = query block, shared over B
 * and H); zero blocks are never loaded or computed (reading notes,
 * §Introduction › Block-sparse FlashAttention). `causal` and `key_len` (as in
 * fa_fwd, may be 0 / NULL) combine with the block mask by AND: an entry is kept
 * iff its block is nonzero, and it is causal-allowed, and its key is below the
 * batch's key length. Blocks above the diagonal are then skipped when causal.
 * Requires bs to be a positive multiple of 128 that divides N (else
 * FA_ERR_INVALID) and N / bs <= 1024 (else FA_ERR_UNSUPPORTED). bf16 only. `workspace` is not used (it may be
 * NULL with workspace_bytes 0; the argument stays for a stable ABI). */
int fa_blocksparse_fwd(const fa_desc* desc, const void* Q, const void* K, const void* V,
                       float scale, int causal, const int32_t* key_len,
                       const uint8_t* block_mask, int32_t block_size, void* O, float* LSE,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Block-sparse backward: fa_bwd restricted to the kept blocks; needs the O and
 * LSE of fa_blocksparse_fwd with the same mask, causal flag and key lengths.
 * Same requirements on the mask; `workspace` must hold
 * fa_blocksparse_workspace_bytes(desc, bs, 1) bytes (= fa_bwd_workspace_bytes). */
int fa_blocksparse_bwd(const fa_desc* desc, const void* Q, const void* K, const void* V,
                       const void* O, const void* dO, const float* LSE, float scale, int causal,
                       const int32_t* key_len, const uint8_t* block_mask, int32_t block_size,
                       void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Forward with dropout on P (reading notes, §Algorithm › Tiling and Kernel
 * Fusion: the fused kernel applies dropout after the softmax): as fa_fwd, but
 * O = (P o Z) V / (1 - p) with keep bits Z drawn per (instance, query, key) from
 * Philox4x32-10 (Salmon et al., SC 2011): pair (i, j) of instance bh = b H + h
 * takes byte j mod 4 of word i mod 4 at counter (i div 4, j div 4, bh, offset)
 * with key (seed low word, seed high word), and is kept iff that byte is >=
 * p8 = round(256 dropout_p); the drop probability applied is p8 / 256. LSE is
 * that of the softmax before dropout. dropout_p must lie in [0, 1) (else
 * FA_ERR_INVALID); p8 = 0 is fa_fwd. bf16 only when p8 > 0 (else
 * FA_ERR_UNSUPPORTED). Dense, causal and key_len masks (block-sparse:
 * fa_blocksparse_fwd_dropout). */
int fa_fwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V, float scale,
                   int causal, const int32_t* key_len, float dropout_p, uint64_t seed,
                   uint32_t offset, void* O, float* LSE, void* stream);

/* Backward of fa_fwd_dropout: the keep bits are regenerated from the same
 * (seed, offset), which must match the forward's, as must scale, causal and
 * key_len. Same workspace as fa_bwd. */
int fa_bwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE, float scale, int causal, const int32_t* key_len,
                   float dropout_p, uint64_t seed, uint32_t offset, void* dQ, void* dK, void* dV,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Backward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): fa_bwd with its workspace (8 bytes per row of B H N) taken from a
 * static device array of 16 MiB that the library holds on each device it runs on
 * until the process ends. The caller still passes every input and output. Same
 * arguments, checks and results as fa_bwd (bit for bit); allocates nothing and
 * calls no allocating routine. Problems with B H N > 2^21 rows (the workspace
 * of fa_bwd_workspace_bytes above 16 MiB) return FA_ERR_SCRATCH before anything
 * is enqueued. All calls on one
 * device share that device's array: calls that overlap on one GPU (two streams,
 * or two threads, without ordering between them) race on it and must be
 * serialised by the caller. Nothing in the array needs to start at zero (each
 * call writes every entry it reads). The array's device address is looked up on
 * the first call on each device (hipGetSymbolAddress; FA_ERR_HIP if it fails). */
int fa_bwd_noalloc(const fa_desc* desc, const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE, float scale, int causal, const int32_t* key_len,
                   void* dQ, void* dK, void* dV, void* stream);

/* Block-sparse forward with dropout on P: fa_blocksparse_fwd (same mask,
 * causal and key_len semantics and requirements) with the dropout of
 * fa_fwd_dropout (same keep bits, scaling and LSE; reading notes, §Algorithm ›
 * Kernel Fusion: masking and dropout in the one fused kernel; §Experiments ›
 * 4.4 runs block-sparse attention with dropout). dropout_p in [0, 1) (else
 * FA_ERR_INVALID); bf16 only. */
int fa_blocksparse_fwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V,
                               float scale, int causal, const int32_t* key_len,
                               const uint8_t* block_mask, int32_t block_size, float dropout_p,
                               uint64_t seed, uint32_t offset, void* O, float* LSE, void* stream);

/* Backward of fa_blocksparse_fwd_dropout: needs the same mask, scale, causal,
 * key_len and (dropout_p, seed, offset). Workspace as fa_blocksparse_bwd. */
int fa_blocksparse_bwd_dropout(const fa_desc* desc, const void* Q, const void* K, const void* V,
                               const void* O, const void* dO, const float* LSE, float scale, int causal,
                               const int32_t* key_len, const uint8_t* block_mask, int32_t block_size,
                               float dropout_p, uint64_t seed, uint32_t offset, void* dQ, void* dK,
                               void* dV, void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* fa_status_string(int status);

/* FA_VERSION of the built library. */
int fa_version(void);

/* Optional kernel timer (instrumentation for benchmarks). While enabled on a
 * thread, every kernel the library launches from that thread is bracketed by two
 * HIP events on its stream. fa_timer_read synchronises on the calling thread's
 * recorded events and returns the summed duration (ms) and launch count of the
 * kernels whose name equals `kernel` since that thread's last reset. The state
 * is per thread: launches from other threads are neither recorded nor affected,
 * and a thread whose timer is off only reads one thread-local flag per launch.
 * Up to 8192 launches are recorded between resets; later ones are not timed.
 * fa_timer_enable returns FA_OK or FA_ERR_HIP (events could not be created). */
int fa_timer_enable(int enable);
void fa_timer_reset(void);
int fa_timer_read(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
