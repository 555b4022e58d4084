/*
 * flash_attn.h -- C ABI of the MI355X (gfx950) exact fused attention library.
 *
 * What is computed: exact attention O = softmax(scale * Q Kᵀ [+ causal mask]) V,
 * tiled with an online softmax so that the N x N score matrix never reaches
 * device memory, plus the recomputation backward and a split-KV decode over a
 * paged KV cache.  Sources of each operation:
 *
 *   - Forward: "Flash-Attention" concept page (awesome-system-papers), section
 *     "Core idea" (tiles of Q/K/V staged on chip; running max, running sum and
 *     running output; Q outer, K/V inner as in FlashAttention-2) and the
 *     tutorial "FlashAttention and efficient attention kernels" (plumephp),
 *     sections "Standard attention", "Online softmax", "Correction formula",
 *     "Forward" and the forward pseudocode skeleton.
 *   - Backward: the same tutorial, sections "Backward" and "Backward recompute
 *     flow" (S and P are rebuilt on chip from Q, K, V and the saved per-row
 *     statistics, combined with dO into dQ, dK, dV, and discarded block by
 *     block).
 *   - Decode: the tutorial's "Variant family" section (FlashDecoding splits the
 *     KV sequence, computes partial results in parallel and reduces them;
 *     PagedAttention reads KV stored in non-contiguous fixed-size blocks) and
 *     the related-work page (CuFlash-Attn), papers #5 (PagedAttention) and
 *     #6 (grouped-query attention: each group of query heads shares one K/V
 *     head).
 *   - Library shape: the related-work page's repository comparison and
 *     "zero dependency" positioning (a standalone dynamic library callable
 *     through ctypes, head_dim in {32, 64, 128}, full forward and backward).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Layouts (dense, row-major, element strides implied by the shapes):
 *     Q, O, dO, dQ : [B, Hq,  Nq, d]
 *     K, V, dK, dV : [B, Hkv, Nk, d]
 *     LSE          : [B, Hq,  Nq]  float32, natural-log logsumexp of each
 *                    scaled, masked score row (LSE = m + ln l).
 *   Query head h reads K/V head h / (Hq / Hkv) (contiguous groups); Hq must
 *   be a multiple of Hkv (Hkv == Hq: multi-head; Hkv == 1: multi-query).
 *   dtype is one of FA_F32, FA_F16, FA_BF16 and applies to every tensor
 *   except LSE, the workspaces and the integer decode metadata.  Products run
 *   on the matrix cores with float32 accumulation; the probabilities P (and
 *   dS in the backward) are rounded to dtype before their second product
 *   (round-to-nearest-even), except for FA_F32 which keeps float32 throughout.
 *   causal != 0 applies the bottom-right aligned mask: query row i sees key j
 *   iff j <= i + (Nk - Nq).  Rows that see no key (only when Nq > Nk) produce
 *   O = 0, LSE = -inf and zero gradients.
 *   scale is applied to Q Kᵀ before the mask and the softmax (1/sqrt(d) is
 *   customary; any finite value is accepted).
 *   Pointers are device pointers (hipMalloc'd or torch CUDA tensors) unless
 *   stated; all are owned by the caller.  The library allocates nothing,
 *   keeps no pointer after a call returns and holds no mutable global state.
 *   Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL means the default stream); results are valid after the caller
 *   synchronises that stream.
 *   Arguments are validated on the host before any HIP call; a failed
 *   validation returns its error code and leaves every buffer untouched.
 *   FA_ERR_LAUNCH reports a failure of the kernel launch itself.  No entry
 *   point throws or aborts.
 */
#ifndef FLASH_ATTN_MI355X_H
#define FLASH_ATTN_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_dtype { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 };

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL                                   */
  FA_ERR_SHAPE = 2,     /* a size is <= 0 (or < 0 where 0 is allowed), or too large     */
  FA_ERR_HEADDIM = 3,   /* d not in {32, 64, 128}                                       */
  FA_ERR_DTYPE = 4,     /* dtype not one of enum fa_dtype                               */
  FA_ERR_GQA = 5,       /* Hq is not a multiple of Hkv                                  */
  FA_ERR_BLOCKSIZE = 6, /* decode page size other than 16 tokens                        */
  FA_ERR_WORKSPACE = 7, /* workspace pointer NULL or smaller than the size query says   */
  FA_ERR_LAUNCH = 8,    /* a kernel launch failed (hipGetLastError after the launch)    */
  FA_ERR_SCALE = 9,     /* scale is not finite                                          */
  FA_ERR_ALIGN = 10,    /* a pointer is misaligned: dtype tensors and workspaces need   */
                        /* 16-byte alignment, LSE and int32 arrays 4-byte alignment     */
  FA_ERR_SCRATCH = 11   /* the allocation-free decode needs more than its fixed scratch */
};

/* Human-readable text of a status code (static storage, never NULL). */
const char* flash_attn_strerror(int code);

/*
 * Forward.  Inputs Q, K, V; outputs O (dtype) and LSE (float32, one value per
 * query row, needed by the backward).  Sizes: B, Hq, Hkv, Nq, Nk >= 1;
 * d in {32, 64, 128}; B*Hq*Nq*d and B*Hkv*Nk*d below 2^31 elements.
 * Errors (checked in this order): FA_ERR_NULL, FA_ERR_DTYPE, FA_ERR_SHAPE,
 * FA_ERR_HEADDIM, FA_ERR_GQA, FA_ERR_SHAPE (too large), FA_ERR_SCALE,
 * FA_ERR_ALIGN, then FA_ERR_LAUNCH.
 */
int flash_attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, void* stream);

/*
 * Bytes of device workspace flash_attn_bwd needs: two float32 values per query
 * row (the row term D_i = sum_c dO_ic * O_ic, stored negated, and
 * LSE_i * log2(e)).  Returns 0 for invalid sizes.
 */
size_t flash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int dtype);

/*
 * Backward.  Inputs Q, K, V, the forward's O and LSE, and the upstream
 * gradient dO; outputs dQ, dK, dV (dtype; fully overwritten, not
 * accumulated into).  dK and dV of a K/V head are summed over the query heads
 * of its group.  workspace must hold flash_attn_bwd_workspace_bytes(...)
 * bytes; its contents on entry are ignored.  Deterministic: identical inputs
 * give bitwise identical outputs.  Runs flash_attn_bwd_dq_rowterms, then
 * flash_attn_bwd_dkdv, on one stream.
 * Errors: as flash_attn_fwd, with FA_ERR_WORKSPACE checked before FA_ERR_ALIGN.
 */
int flash_attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* dQ, void* dK, void* dV,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward's phases, for callers that schedule them themselves:
 *   1. flash_attn_bwd_preprocess writes the per-row terms D_i and
 *      LSE_i*log2(e) into the workspace (reads O, dO, LSE);
 *   2. flash_attn_bwd_dkdv writes dK, dV and flash_attn_bwd_dq writes dQ;
 *      both read the workspace written by phase 1 and are independent of
 *      each other, so they may run concurrently on two streams once phase 1
 *      has completed.
 * flash_attn_bwd_dq_rowterms is phase 2's dQ computing the row terms of its
 * own rows (it reads O, dO and LSE as well) and writing them into the
 * workspace, in place of phase 1: flash_attn_bwd_dkdv may run after it has
 * completed.  flash_attn_bwd runs these two in that order; the row terms are
 * the same up to float32 rounding order, so its results can differ from the
 * three-phase order in the last bits.
 * Arguments mean what they mean for flash_attn_bwd; the workspace must hold
 * flash_attn_bwd_workspace_bytes(...) bytes.  Same error codes and order.
 */
int flash_attn_bwd_preprocess(const void* O, const void* dO, const float* LSE,
                              int B, int Hq, int Nq, int d, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream);
int flash_attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                        void* dK, void* dV,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                        int dtype, const void* workspace, size_t workspace_bytes, void* stream);
int flash_attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, void* dQ,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int dtype, const void* workspace, size_t workspace_bytes, void* stream);
int flash_attn_bwd_dq_rowterms(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                               const float* LSE, void* dQ,
                               int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                               int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed (variable-length) batches.  Sources: the related-work page
 * (CuFlash-Attn), repository comparison (variable-length support of the
 * reference implementation); the concept page "Flash-Attention", key
 * observation 4 (packing sequences of different lengths); the tutorial's
 * "Validation checklist" (variable-length sequences).  The pages fix no
 * layout.  Here a packed batch is the concatenation of each sequence's dense
 * [1, H, n_b, d] tensor:
 *   cu_seqlens_q [B + 1] int32 device array: 0 = cu[0] <= cu[1] <= ... <=
 *                cu[B] = total_q; sequence b has n_b = cu[b+1] - cu[b]
 *                queries (cu_seqlens_k likewise for keys; n_b may be 0).
 *   Q, O, dO, dQ [Hq  * total_q, d]: head h of sequence b is the contiguous
 *                [n_b, d] block starting at row Hq * cu_q[b] + h * n_b.
 *   K, V, dK, dV [Hkv * total_k, d]: likewise with Hkv and cu_seqlens_k.
 *   LSE          [Hq  * total_q] float32, the same row order as O.
 * Each sequence is attended on its own (its queries see only its keys), with
 * the causal mask aligned bottom-right within the sequence; a sequence with
 * queries but no keys gives O = 0 and LSE = -inf, one with keys but no
 * queries gives dK = dV = 0.  max_seqlen_q / max_seqlen_k bound every n_b
 * (the grids are sized by them) and may not exceed total_q / total_k.
 * Sizes: B, Hq, Hkv >= 1; total_q, total_k, max_seqlen_q, max_seqlen_k >= 0;
 * Hq*total_q*d and Hkv*total_k*d below 2^31 elements; max_seqlen * d below
 * 2^31 bytes (one sequence's slab of one head).
 * The cumulative arrays live on the device, so the host cannot check them:
 * a sequence whose entries break the ordering above or exceed the bounds is
 * skipped (its output rows are left unwritten) and no access leaves the
 * tensors.  Errors: as the dense calls, with the packed sizes.
 */
int flash_attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          const int* cu_seqlens_q, const int* cu_seqlens_k,
                          int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                          int d, float scale, int causal, int dtype, void* stream);

/* Bytes of device workspace flash_attn_bwd_varlen needs: two float32 values
 * per query row (Hq * total_q rows).  Returns 0 for invalid sizes (and for
 * total_q = 0, when no workspace is needed and NULL is accepted). */
size_t flash_attn_bwd_varlen_workspace_bytes(int B, int Hq, int Hkv, int total_q, int total_k,
                                             int max_seqlen_q, int max_seqlen_k, int d, int dtype);

/* Backward of flash_attn_fwd_varlen: dQ, dK, dV (fully overwritten) from Q,
 * K, V, O, LSE and dO, all in the packed layout above.  Deterministic, like
 * flash_attn_bwd, whose errors (and order) it shares. */
int flash_attn_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                          const float* LSE, void* dQ, void* dK, void* dV,
                          const int* cu_seqlens_q, const int* cu_seqlens_k,
                          int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                          int d, float scale, int causal, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Number of KV splits the decode uses for num_splits = 0 (automatic): about
 * four splits (one per wave) per compute unit of the current device (256 on
 * a whole MI355X; 256 is also assumed when the device query fails), with at
 * least 4 pages per split.  Its only HIP call is that device query, made
 * after the arguments are checked; invalid sizes return 0.
 */
int flash_attn_decode_num_splits(int B, int Hkv, int max_blocks_per_seq, int block_size);

/*
 * Bytes of device workspace flash_attn_decode_paged needs for the given
 * split count (0 = automatic, resolved as above on the current device, so
 * query it with the device current that the decode will run on): per
 * (sequence, query head, split) a record of d + 4 float32 values (the
 * partial output, its running max and sum, two pad words).  Besides the
 * split count itself, the automatic count needs Hkv, max_blocks_per_seq and
 * block_size, which is why they are arguments.  Returns 0 for invalid sizes
 * (num_splits outside [0, 65536] included).
 */
size_t flash_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_blocks_per_seq,
                                         int block_size, int num_splits);

/*
 * Split-KV decode of one new query token per sequence over a paged KV cache.
 *   Q        [B, Hq, d]                            (the token's queries)
 *   K_cache  [num_blocks, Hkv, block_size, d]      (pages; token t of sequence
 *   V_cache  [num_blocks, Hkv, block_size, d]       b is slot t % block_size of
 *                                                   page block_table[b][t / block_size])
 *   block_table [B, max_blocks_per_seq] int32 device array of page ids in
 *               [0, num_blocks); entries past a sequence's last page are
 *               never read.  An id outside [0, num_blocks) is read as a page
 *               of zeros (it cannot fault, but the result is meaningless).
 *   seq_lens    [B] int32 device array: tokens of sequence b (the tail of
 *               its last page is ignored).  Values outside [0,
 *               max_blocks_per_seq * block_size] are clamped to that range,
 *               so no length reads past the sequence's table row.  A length
 *               of 0 gives O = 0 and LSE = -inf.
 *   O   [B, Hq, d] dtype;  LSE [B, Hq] float32, or NULL if not wanted.
 * The query is the sequence's last position, so it sees every cached token
 * (no mask).  Each split runs an online softmax over its share of the pages;
 * a second kernel merges the splits' (max, sum, output) partials.
 * block_size must be 16.  dtype must be FA_F16 or FA_BF16 (the float32 KV
 * cache is not supported: FA_ERR_DTYPE).  0 <= num_splits <= 65536 (0 =
 * automatic); results depend on the split count only through float32
 * rounding order.  B * Hkv <= 65535 (the split kernel's grid) and
 * max_blocks_per_seq * block_size below 2^31, else FA_ERR_SHAPE.
 * Errors (in this order): FA_ERR_NULL, FA_ERR_DTYPE, FA_ERR_SHAPE,
 * FA_ERR_HEADDIM, FA_ERR_GQA, FA_ERR_BLOCKSIZE, FA_ERR_SHAPE (too large),
 * FA_ERR_SCALE, FA_ERR_WORKSPACE, FA_ERR_ALIGN, FA_ERR_LAUNCH.
 */
int flash_attn_decode_paged(const void* Q, const void* K_cache, const void* V_cache,
                            const int* block_table, const int* seq_lens, void* O, float* LSE,
                            int B, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
                            int num_blocks, float scale, int num_splits, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same inputs, outputs, semantics and
 * kernels as flash_attn_decode_paged, without the workspace arguments: the
 * split records live in a fixed scratch area of FLASH_ATTN_DECODE_SCRATCH_BYTES
 * bytes that the library holds on every GPU it runs on until the process
 * ends.  Its device address is resolved once per device, on the first call
 * with that device current; nothing is allocated or freed by any call.
 * Limit: flash_attn_decode_workspace_bytes(B, Hq, Hkv, d, max_blocks_per_seq,
 * block_size, num_splits) must not exceed FLASH_ATTN_DECODE_SCRATCH_BYTES,
 * else FA_ERR_SCRATCH (8 MiB holds, e.g., B = 8, Hq = 32, d = 128 with up to
 * 62 splits).  Every call on a GPU shares that GPU's scratch area: calls that
 * overlap on one GPU (on different streams, or from different threads without
 * ordering) race and give undefined results; calls ordered on one stream are
 * safe.  The scratch holds no state between calls (every record is rewritten
 * before it is read).
 * Errors (in this order): FA_ERR_NULL, FA_ERR_DTYPE, FA_ERR_SHAPE,
 * FA_ERR_HEADDIM, FA_ERR_GQA, FA_ERR_BLOCKSIZE, FA_ERR_SHAPE (too large),
 * FA_ERR_SCALE, FA_ERR_SCRATCH, FA_ERR_ALIGN, FA_ERR_LAUNCH (also when the
 * scratch address cannot be resolved).
 */
#define FLASH_ATTN_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
int flash_attn_decode_paged_noalloc(const void* Q, const void* K_cache, const void* V_cache,
                                    const int* block_table, const int* seq_lens, void* O, float* LSE,
                                    int B, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
                                    int num_blocks, float scale, int num_splits, int dtype, void* stream);

/*
 * Paged prefill: a chunk of Nq new queries per sequence attends to the
 * sequence's tokens in a paged KV cache.  Sources: the tutorial's "Variant
 * family" section (PagedAttention: K/V stored in non-contiguous fixed-size
 * blocks) and the concept page "Flash-Attention", key observation 4 (paged
 * KV fused with the tiled kernel).
 *   Q, O     [B, Hq, Nq, d] dtype: the chunk's queries are the last Nq
 *            positions of each sequence;
 *   LSE      [B, Hq, Nq] float32;
 *   K_cache, V_cache, block_table, seq_lens: as for flash_attn_decode_paged
 *            (seq_lens[b] counts every cached token of sequence b, the
 *            chunk's own included; values outside [0, max_blocks_per_seq *
 *            block_size] are clamped to that range).
 * causal != 0 applies the bottom-right mask: query i of the chunk sees cached
 * token j iff j <= i + seq_lens[b] - Nq, so rows with i < Nq - seq_lens[b]
 * see nothing (O = 0, LSE = -inf).  Without the mask every cached token is
 * seen.  The tiled forward runs unchanged except that each K/V tile is
 * staged page by page through the table.  dtype: FA_F32, FA_F16, FA_BF16;
 * block_size must be 16.  A table entry outside [0, num_blocks) reads as a
 * page of zeros.
 * Errors (in this order): FA_ERR_NULL, FA_ERR_DTYPE, FA_ERR_SHAPE,
 * FA_ERR_HEADDIM, FA_ERR_GQA, FA_ERR_BLOCKSIZE, FA_ERR_SHAPE (too large),
 * FA_ERR_SCALE, FA_ERR_ALIGN, FA_ERR_LAUNCH.
 */
int flash_attn_prefill_paged(const void* Q, const void* K_cache, const void* V_cache,
                             const int* block_table, const int* seq_lens, void* O, float* LSE,
                             int B, int Hq, int Hkv, int Nq, int d, int block_size, int max_blocks_per_seq,
                             int num_blocks, float scale, int causal, int dtype, void* stream);

/*
 * FP8 forward.  Sources: the concept page "Flash-Attention", key
 * observations (FlashAttention-3's FP8 path on Hopper) and the tutorial's
 * "Validation checklist" (FP8).  The pages give no encoding or scaling
 * recipe; here:
 *   Q [B, Hq, Nq, d], K, V [B, Hkv, Nk, d]: OCP FP8 E4M3 codes (one byte per
 *   element); the value of an element is its code times the tensor's float32
 *   descale (q_descale, k_descale, v_descale, all finite).
 *   O [B, Hq, Nq, d] bfloat16; LSE [B, Hq, Nq] float32 (natural log), as for
 *   flash_attn_fwd, of the decoded tensors.
 * Both products run on the FP8 matrix cores with float32 accumulation; the
 * probabilities are rounded to E4M3 (round to nearest even, after scaling
 * into (0, 256]) before the second product, while the softmax row sum is
 * taken in float32 from the unrounded values.  d must be 64 or 128 (else
 * FA_ERR_HEADDIM).  causal as for flash_attn_fwd.
 * workspace: flash_attn_fwd_fp8_workspace_bytes(...) bytes of device memory
 * (V is staged there transposed, 64 keys per tile); contents on entry are
 * ignored.  B * Hkv must not exceed 65535.
 * Errors (in this order): FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM,
 * FA_ERR_GQA, FA_ERR_SHAPE (too large), FA_ERR_SCALE, FA_ERR_WORKSPACE,
 * FA_ERR_ALIGN, FA_ERR_LAUNCH.
 */
size_t flash_attn_fwd_fp8_workspace_bytes(int B, int Hkv, int Nk, int d);
int flash_attn_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       float scale, float q_descale, float k_descale, float v_descale, int causal,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_MI355X_H */
