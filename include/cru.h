/*
 * cru.h -- C ABI of the context-parallel attention library (libcru.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes (sources are the pages this library follows):
 *
 *  - Softmax attention with its per-row log-sum-exp, non-causal and unmasked:
 *    O = softmax(Q K^T * scale) V per (batch, head).  diffusers "Attention
 *    backends" page, "Available backends" table: the default backend is
 *    PyTorch's scaled_dot_product_attention, whose default scale is
 *    1/sqrt(D).  diffusers "Parallelism" API page, ContextParallelConfig,
 *    convert_to_fp32: ring attention carries the output *and* the LSE, in
 *    fp32 by default.
 *  - The LSE merge that folds partial results over disjoint key chunks into
 *    the full result (the fold each ring step performs; same two pages).
 *  - One ring rank's share: its query rows against every K/V chunk, folded
 *    in ascending chunk order.  diffusers "Context parallelism" guide,
 *    "Ring Attention" section (K/V blocks visited one after another) and
 *    "Ring Anything Attention" section (chunks of unequal length).
 *  - The sequence<->head regrouping of Ulysses attention.  Same guide,
 *    "Ulysses Attention" section: the first all-to-all leaves each device
 *    with every token of a subset of heads, the second regroups by token;
 *    "Ulysses Anything Attention" section: head count and sequence length
 *    need not divide by the degree.
 *  - Unified attention on a 2-D mesh of ulysses_degree x ring_degree
 *    devices.  Same guide, "Unified Attention" section: an all-to-all
 *    regroups heads and tokens, ring attention runs on the result, and the
 *    reverse all-to-all restores the layout.
 *
 * Conventions shared by every entry point:
 *  - All data pointers are device memory on the current HIP device, owned by
 *    the caller.  The library never allocates, frees or synchronises; each
 *    call only enqueues kernels on `stream` and returns.
 *  - Tensors are described by cru_tensor: a [B, S, H, D] view with element
 *    strides for b, s and h; d is contiguous (stride 1).  Strides must be
 *    non-negative; the data pointer must be 16-byte aligned and the b/s/h
 *    strides multiples of 8 elements (bf16) or 4 elements (fp32), so rows can
 *    be moved 16 bytes at a time.
 *  - Input views may repeat elements: a stride of 0 (a broadcast, as torch's
 *    expand() gives) or rows that overlap (a sequence stride below D) read
 *    the same values the view describes.  Output views (and output LSEs)
 *    must give every element its own address: with the dims of size > 1
 *    sorted by stride, each stride must exceed the largest offset the
 *    smaller-stride dims reach; other output views fail with CRU_EINVAL.
 *    Outputs must not share memory with inputs (not checked).
 *  - The LSE is fp32 [B, H, S], natural log, described by cru_lse (s stride 1).
 *  - Head dims: D = 64 or 128.
 *  - Sizes: each of B, S, H, D at most 2^30 and B*S*H*D at most 2^48
 *    elements; one call's kernel work items (threads, 16-byte vectors) below
 *    2^31 (split larger calls); for the attention, s strides below 2^22
 *    elements; a view's largest element offset (the sum over its dims of
 *    (size - 1) * stride) below 2^60.  Larger requests fail with CRU_EINVAL.
 *  - All checks run on the host before anything is enqueued.  A failed check
 *    returns a non-zero cru_status, enqueues nothing and leaves a message for
 *    cru_last_error() (thread-local).  The checks follow the three classes of
 *    the diffusers "Attention backends" page, "Checks" section: device
 *    (CRU_EDEVICE), data type (CRU_EUNSUPPORTED) and shape (CRU_EINVAL), plus
 *    the divisibility rules of the "Context parallelism" guide's variant
 *    table (CRU_ENOTDIV).
 *  - CRU_EHIP reports a HIP error raised while enqueueing.
 *  - Calls that overlap on one stream are ordered by the stream; concurrent
 *    calls on different streams must not write the same memory.
 *  - Calls only enqueue kernels (no allocation, memset or synchronisation),
 *    so they may be captured into a HIP graph and replayed.
 */
#ifndef CRU_H
#define CRU_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CRU_ABI_VERSION 2
/* Most partial results one merge (or one ring share) may fold. */
#define CRU_MAX_PARTS 64

typedef enum {
  CRU_OK = 0,
  CRU_EINVAL = 1,        /* null pointer, bad shape or stride, size mismatch */
  CRU_ENOTDIV = 2,       /* a divisibility rule of the variant is broken */
  CRU_EUNSUPPORTED = 3,  /* dtype combination or head dim not implemented */
  CRU_EDEVICE = 4,       /* a pointer is not device memory of the current device */
  CRU_EWORKSPACE = 5,    /* workspace missing, misaligned or too small */
  CRU_EHIP = 6           /* the HIP runtime reported an error */
} cru_status;

typedef enum { CRU_F32 = 0, CRU_BF16 = 1 } cru_dtype;

/* A [B, S, H, D] tensor view.  Element (b, s, h, d) lives at
 * data + (b*sb + s*ss + h*sh + d) elements of `dtype`. */
typedef struct {
  void*   data;
  int32_t dtype;          /* cru_dtype */
  int32_t reserved;       /* must be 0 */
  int64_t B, S, H, D;
  int64_t sb, ss, sh;
} cru_tensor;

/* Per-row LSE, fp32 [B, H, S]: element (b, h, s) at data + b*sb + h*sh + s. */
typedef struct {
  float*  data;
  int64_t B, H, S;
  int64_t sb, sh;
} cru_lse;

/*
 * cru_attn_fwd_lse -- O = softmax(Q K^T * scale) V and LSE = log sum_j
 * exp(q.k_j * scale), per batch, head and query row; non-causal, no mask.
 *
 *   q    [B, Sq, H, D]     bf16 or fp32
 *   k, v [B, Skv, H, D]    same dtype as q
 *   o    [B, Sq, H, D]     bf16 or fp32 for bf16 inputs; fp32 for fp32 inputs
 *   lse  [B, H, Sq] fp32, or NULL when not wanted
 *   scale  > 0, or 0 for 1/sqrt(D)
 *
 * bf16 inputs run on bf16 matrix cores with fp32 accumulation; P is rounded
 * to bf16 (nearest even) before the P V product, O is divided by the sum of
 * those rounded values (the LSE is taken from the sum of the unrounded
 * ones), and O is rounded to nearest even when o is bf16.  fp32 inputs run
 * in fp32 throughout.  The bf16 path moves its running max lazily: a row's
 * unnormalised sums may reach about 2^33 before the max moves, so O's fp32
 * accumulator stays finite for max|V| below 2^90 (bf16 reaches 2^128).
 * Skv = 0 gives O = 0 and LSE = -inf; Sq = 0 enqueues nothing.
 * o must not overlap q, k or v.
 * Defined by: diffusers "Attention backends" page, "Available backends"
 * (scaled_dot_product_attention as the default backend); the LSE output:
 * "Parallelism" API page, ContextParallelConfig.convert_to_fp32.
 */
cru_status cru_attn_fwd_lse(const cru_tensor* q, const cru_tensor* k,
                            const cru_tensor* v, const cru_tensor* o,
                            const cru_lse* lse, float scale,
                            hipStream_t stream);

/*
 * cru_attn_merge_lse -- combine n partial results over disjoint key sets:
 *   LSE = M + log sum_c exp(LSE_c - M),  M = max_c LSE_c
 *   O   = sum_c exp(LSE_c - LSE) * O_c, summed in ascending c.
 * A part with LSE_c = -inf holds no keys and contributes nothing; rows where
 * every part is empty give O = 0, LSE = -inf.
 *
 *   o_parts    host array of n [B, S, H, D] views, all the same shape, strides
 *              and dtype: fp32, or bf16 (partials kept in the model dtype,
 *              ContextParallelConfig.convert_to_fp32 = False); the sums are
 *              fp32 either way
 *   lse_parts  host array of n fp32 [B, H, S] LSE views, all the same strides
 *   o          [B, S, H, D] bf16 or fp32
 *   lse        [B, H, S] fp32, or NULL
 *   1 <= n <= CRU_MAX_PARTS
 * Outputs must not overlap the inputs.
 * Defined by: diffusers "Parallelism" API page, ContextParallelConfig
 * (convert_to_fp32: each step's output and LSE) and the "Context
 * parallelism" guide, "Ring Attention" section (one K/V block after
 * another); the closed form is the identity exp(LSE_c - LSE) exp(s - LSE_c)
 * = exp(s - LSE).
 */
cru_status cru_attn_merge_lse(int n, const cru_tensor* o_parts,
                              const cru_lse* lse_parts, const cru_tensor* o,
                              const cru_lse* lse, hipStream_t stream);

/*
 * cru_ring_workspace_bytes -- bytes of device workspace cru_ring_emulate
 * needs for a query share shaped like q_share cut into n_chunks chunks
 * (n_chunks fp32 partial outputs and LSEs).  The same size serves both the
 * step-wise and the fused schedule, and bf16 partials (which use less).
 * The partials are the per-step output and LSE that ring attention carries
 * in fp32: diffusers "Parallelism" API page, ContextParallelConfig,
 * convert_to_fp32.  Host-only; bytes is written on success.
 */
cru_status cru_ring_workspace_bytes(const cru_tensor* q_share, int n_chunks,
                                    size_t* bytes);

/*
 * cru_ring_chunk_bounds -- the split of S sequence rows into n consecutive
 * chunks that cru_ring_emulate uses when chunk_sizes is NULL: chunk c is
 * rows [starts[c], starts[c+1]).  The first S mod n chunks get one extra row
 * (sizes differ by at most one).  With anything = 0, S must be divisible by
 * n (CRU_ENOTDIV otherwise), as plain ring attention requires.  Host-only;
 * starts is a host array of n + 1 entries.  Ring rank r's query share is
 * chunk r of the same split.
 * Defined by: diffusers "Context parallelism" guide, "Ring Anything
 * Attention" section (sequence lengths that do not divide by the degree).
 */
cru_status cru_ring_chunk_bounds(int64_t S, int n, int anything, int64_t* starts);

/*
 * cru_ring_emulate -- one ring rank's share on one device: the rank's query
 * rows q_share against every K/V chunk, each chunk's fp32 partial (output,
 * LSE) folded into o and lse in ascending chunk order.
 *
 *   q_share      [B, Sq, H, D] bf16 or fp32: the rank's query rows
 *   k, v         [B, Skv, H, D], q's dtype: all chunks, back to back (what every
 *                rank holds after the K/V all-gather)
 *   n_chunks     ring degree, 1..CRU_MAX_PARTS
 *   anything     0: Skv must split evenly (CRU_ENOTDIV otherwise);
 *                1: any Skv ("Ring Anything": chunks may differ in length)
 *   chunk_sizes  host array of n_chunks lengths summing to Skv, or NULL for
 *                the near-equal split (the first Skv mod n chunks get one
 *                extra row); with anything = 0 they must all be equal.  Each
 *                is checked against the rows left before it is added
 *                (CRU_EINVAL), so no sum can wrap around
 *   fused        0: one attention launch per chunk (the ring's step order);
 *                1: one launch over every (chunk, query tile, head)
 *   convert_to_fp32  1: fp32 partial outputs (ContextParallelConfig's
 *                default); 0: partial outputs in the model dtype, bf16
 *                (bf16 inputs only, CRU_EUNSUPPORTED otherwise).  The
 *                partial LSEs are fp32 either way ("Parallelism" API page,
 *                convert_to_fp32)
 *   o            [B, Sq, H, D] bf16 or fp32;  lse [B, H, Sq] fp32 or NULL
 *   scale        as for cru_attn_fwd_lse
 *   workspace    device memory of at least cru_ring_workspace_bytes(),
 *                256-byte aligned, not overlapping any argument
 * Empty chunks are allowed with anything = 1 and contribute nothing.
 * Defined by: diffusers "Context parallelism" guide, "Ring Attention" and
 * "Ring Anything Attention" sections; "Parallelism" API page,
 * ContextParallelConfig (ring_degree, rotate_method, convert_to_fp32).
 */
cru_status cru_ring_emulate(const cru_tensor* q_share, const cru_tensor* k,
                            const cru_tensor* v, int n_chunks, int anything,
                            const int64_t* chunk_sizes, int fused,
                            int convert_to_fp32, const cru_tensor* o,
                            const cru_lse* lse,
                            float scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * cru_ring_emulate_noalloc -- cru_ring_emulate without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The
 * partials go to a static device array of CRU_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends; nothing is
 * allocated or freed by the call.
 *
 *   arguments    as for cru_ring_emulate, without workspace/workspace_bytes
 *   limit        cru_ring_workspace_bytes(q_share, n_chunks) must not exceed
 *                CRU_NOALLOC_SCRATCH_BYTES (CRU_EWORKSPACE otherwise, before
 *                anything is enqueued): 64 MiB holds, for example, an 8-chunk
 *                share of 576 rows x 24 heads x 128 dims
 *   results      identical to cru_ring_emulate's with the same arguments
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's partials (the call writes every partial it reads, so nothing
 * needs clearing).  Calls that overlap in time on one GPU (different
 * streams, or threads without ordering) race on the array: order them on
 * one stream.
 */
#define CRU_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
cru_status cru_ring_emulate_noalloc(const cru_tensor* q_share, const cru_tensor* k,
                                    const cru_tensor* v, int n_chunks, int anything,
                                    const int64_t* chunk_sizes, int fused,
                                    int convert_to_fp32, const cru_tensor* o,
                                    const cru_lse* lse, float scale,
                                    hipStream_t stream);

/*
 * cru_ulysses_head_bounds -- the heads of each Ulysses group: group p holds
 * heads [starts[p], starts[p+1]).  The first H mod P groups get one head
 * more (sizes differ by at most one).  With anything = 0, H must be
 * divisible by P (CRU_ENOTDIV otherwise).  Host-only; starts is a host array
 * of P + 1 entries.
 * Defined by: diffusers "Context parallelism" guide, "Ulysses Anything
 * Attention" section (head counts that do not divide by the degree).
 */
cru_status cru_ulysses_head_bounds(int64_t H, int P, int anything, int64_t* starts);

/*
 * cru_ulysses_seq2head -- the first Ulysses all-to-all's net effect on one
 * device, for n tensors in one launch.  With Hp = H / P:
 *   y_t[p, b, s, j, d] = x_t[b, s, p*Hp + j, d],
 * i.e. [B, S, H, D] -> [P, B, S, Hp, D]; group p holds every token of heads
 * [p*Hp, (p+1)*Hp).  A bit-exact copy.
 *
 *   x         host array of n views, all the same shape and dtype (bf16 or
 *             fp32)
 *   y         host array of n device pointers to contiguous buffers of
 *             B*S*H*D elements of that dtype, 16-byte aligned, not
 *             overlapping any x
 *   1 <= n <= 8;  P >= 1
 *   anything  0: P must divide H and S (CRU_ENOTDIV otherwise: the sequence
 *                is sharded P ways before the exchange);
 *             1: any H and S ("Ulysses Anything").  Groups follow
 *                cru_ulysses_head_bounds and lie back to back: group p is a
 *                contiguous [B, S, Hp_p, D] block at element B*S*D*starts[p]
 *                (which is the [P, B, S, Hp, D] layout when P divides H).
 * Defined by: diffusers "Context parallelism" guide, "Ulysses Attention"
 * section (the first all-to-all) and "Ulysses Anything Attention" section.
 */
cru_status cru_ulysses_seq2head(int n, const cru_tensor* x, void* const* y,
                                int P, int anything, hipStream_t stream);

/*
 * cru_ulysses_head2seq -- the inverse regrouping (the second all-to-all):
 *   x_t[b, s, p*Hp + j, d] = y_t[p, b, s, j, d]   (and likewise for uneven
 *   groups).
 *
 *   y   host array of n device pointers to packed buffers laid out as
 *       cru_ulysses_seq2head writes them
 *   x   host array of n output views [B, S, H, D] (shape, dtype, strides)
 *   same rules as cru_ulysses_seq2head.
 * Defined by: the same sections (the second all-to-all regroups the results
 * by token).
 */
cru_status cru_ulysses_head2seq(int n, const void* const* y,
                                const cru_tensor* x, int P, int anything,
                                hipStream_t stream);

/*
 * cru_usp_workspace_bytes -- bytes of device workspace cru_usp_emulate needs
 * for q's shape and the two degrees (the same size serves bf16 and fp32
 * outputs).  Same divisibility rules as cru_usp_emulate.  It holds the
 * regrouped q, k, v of the Ulysses all-to-all (diffusers "Context
 * parallelism" guide, "Unified Attention" section) and one ring workspace of
 * fp32 partials (diffusers "Parallelism" API page, ContextParallelConfig,
 * convert_to_fp32).  Host-only; bytes is written on success.
 */
cru_status cru_usp_workspace_bytes(const cru_tensor* q, int ulysses_degree,
                                   int ring_degree, size_t* bytes);

/*
 * cru_usp_emulate -- Unified (USP) attention over a 2-D mesh of
 * ulysses_degree x ring_degree devices, every device's share computed on
 * this one, with the full output and LSE as the result:
 *   1. seq2head of q, k, v with P = ulysses_degree;
 *   2. for each head group u, the ring over ring_degree equal sequence
 *      chunks: every query row of the group against every chunk, the fp32
 *      partials folded in ascending chunk order (the rows of chunk r are
 *      ring rank r's share; fused and convert_to_fp32 as in
 *      cru_ring_emulate);
 *   3. the reverse all-to-all: each group's result is stored straight into
 *      its heads of o (head2seq fused into the fold's store).
 *
 *   q, k, v   [B, S, H, D] bf16 or fp32, one sequence (k and v have q's S)
 *   ulysses_degree >= 1 must divide H, and ulysses_degree * ring_degree
 *   must divide S (CRU_ENOTDIV otherwise: the sequence is sharded over the
 *   whole mesh; the Anything variants do not combine with Unified attention);
 *   1 <= ring_degree <= CRU_MAX_PARTS
 *   o         [B, S, H, D] bf16 or fp32;  lse [B, H, S] fp32 or NULL
 *   scale     as for cru_attn_fwd_lse
 *   workspace device memory of at least cru_usp_workspace_bytes(), 256-byte
 *             aligned, not overlapping any argument
 * Defined by: diffusers "Context parallelism" guide, "Unified Attention"
 * section.
 */
cru_status cru_usp_emulate(const cru_tensor* q, const cru_tensor* k,
                           const cru_tensor* v, int ulysses_degree,
                           int ring_degree, int fused, int convert_to_fp32,
                           const cru_tensor* o,
                           const cru_lse* lse, float scale, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Name of a status code (static storage). */
const char* cru_status_str(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* cru_last_error(void);
/* CRU_ABI_VERSION of the built library. */
int cru_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CRU_H */
