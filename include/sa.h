/*
 * sa.h -- causal streaming attention for MI355X (gfx950), head width 64.
 *
 * A C ABI over hand-written HIP kernels.  Every entry point takes plain
 * device pointers, sizes and a HIP stream (as void*, NULL = the default
 * stream), enqueues its kernels on that stream and returns without
 * synchronising.  The library never allocates, frees or copies memory of its
 * own: the caller owns every buffer, apart from the static device array
 * behind sa_backward_static (SA_STATIC_SCRATCH_BYTES per GPU, held by the
 * loaded code object until the process ends).  No exception crosses the boundary and
 * the process is never aborted; every failure is a returned status, checked
 * before anything is launched (except SA_ERR_DEVICE, reported by the launch).
 *
 * The method (StreamingAttentionSM86 page):
 *   forward  -- banner "Causal attention as a streaming normalised sum":
 *               softmax(Q K^T scale) V one 64-key tile at a time, with a
 *               running row maximum m, row sum l and weighted sum O; scores
 *               in base-2 units t = S c, c the binary32 nearest scale / ln 2;
 *               P rounded to binary16 before P V; every sum in binary32; the
 *               output O / l and the base-2 log-sum-exp L = m + log2 l.
 *   backward -- banners "The backward pass, deterministic and in two
 *               launches" and "The query pass split in two around the key
 *               pass": P = 2^(S c - L), dP = dO V^T, D = rowsum(dO * O),
 *               dS = P (dP - D), dQ = s dS K, dK = s dS^T Q, dV = P^T dO,
 *               in three launches (row terms, key pass storing dS, dQ pass
 *               reading it), deterministic and without atomics.
 *   lengths  -- variable-length gist page (self_attn_fwd): a query or key at
 *               or past its sequence's length is masked, a row with no
 *               admitted key has O = 0.
 *
 * Grouped query attention: query head h uses K/V head h / (heads/kv_heads)
 * (contiguous groups).  dK and dV^T are the gradients with respect to the K
 * and V^T inputs, so they are summed over each group's query heads.
 *
 * Layouts (row-major, element offsets; B = batch, H = heads, KV = kv_heads):
 *   Q   fp16 [B][H][T][64]        K   fp16 [B][KV][T][64]
 *   Vt  fp16 [B][KV][64][T]       (V transposed, as the pages take it;
 *                                  with shape->v_rows = 1 it is V itself,
 *                                  fp16 [B][KV][T][64], like K)
 *   O   fp16 [B][T][H*64]         (token-major, heads merged)
 *   L   fp32 [B][H][T]            (base-2 log-sum-exp; -inf on masked rows)
 *   dO  fp16 [B][H][T][64]        D   fp32 [B][H][T]
 *   dQ  fp32 [B][H][T][64]        dK  fp32 [B][KV][T][64]
 *   dVt fp32 [B][KV][64][T]       (shape->v_rows = 1: dV, fp32 [B][KV][T][64])
 *   dS  workspace, sa_backward_workspace_bytes() bytes, contents private.
 * Every pointer must be non-NULL and 16-byte aligned.
 *
 * Rows and keys at or past a sequence's length (padding) never influence a
 * valid output, whatever the padding holds.  Padded rows get O = 0,
 * L = -inf, D = 0 and dQ = 0; padded keys get dK = dV = 0.
 *
 * Results are bitwise reproducible for equal inputs, shape and block order.
 * Calls on one stream run in order; calls that share output or workspace
 * buffers on different streams race.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
    SA_OK = 0,
    SA_ERR_SHAPE = 1,      /* the shape fails admission (see sa_check_shape) */
    SA_ERR_NULL = 2,       /* a required pointer is NULL */
    SA_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned (seqlens: 4-byte) */
    SA_ERR_WORKSPACE = 4,  /* dS_bytes < sa_backward_workspace_bytes(shape) */
    SA_ERR_ARGUMENT = 5,   /* c or s not finite and positive */
    SA_ERR_DEVICE = 6,     /* a HIP launch failed (read, and so cleared, by hipGetLastError) */
    SA_ERR_TOO_LARGE = 7   /* sa_backward_static: one 128-row block's dS
                              (sa_backward_chunked_min_bytes) exceeds
                              SA_STATIC_SCRATCH_BYTES */
} sa_status;

/* Size of the library's static device scratch that sa_backward_static uses
 * as its dS workspace (held on every GPU the library runs on, for the life of
 * the process). */
#define SA_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * Problem shape.  Admission (the pages' admission predicate for the grouped
 * launch, StreamingAttentionSM86 page, forward program, without its 32-bit
 * offset clause since every offset here is 64-bit):
 *   batch >= 1;  T >= 64 and T % 64 == 0;  heads >= 1;  kv_heads >= 1;
 *   heads % kv_heads == 0;  heads <= 65535;  batch * heads <= 2^24;
 *   T <= 2^20;  causal, block_order and v_rows are each 0 or 1.
 */
typedef struct sa_shape {
    int batch;
    int T;                    /* padded sequence length */
    int heads;                /* query heads */
    int kv_heads;             /* key/value heads */
    int causal;               /* 1: key j admitted for query i only if j <= i */
    const int32_t* seqlens;   /* device int32[batch] sequence lengths, or NULL
                                 (every sequence has length T).  Values are
                                 clamped to [0, T] by the kernels. */
    int block_order;          /* 0: heavy-first (longest causal blocks first,
                                 the pages' order 1); 1: natural order.  The
                                 results are bitwise identical either way. */
    int v_rows;               /* 0: the V operand is V^T [B][KV][64][T] and
                                 its gradient dV^T (the pages' layouts);
                                 1: V [B][KV][T][64] and dV [B][KV][T][64],
                                 rows like K (StreamingAttentionSM86 page,
                                 the shared forward with V as rows: no
                                 transposed copy of V, the staged V tile is
                                 read transposed for P V).
                                 Every entry point takes either.  Results
                                 are bitwise identical either way. */
} sa_shape;

/* SA_OK if `shape` passes admission, else SA_ERR_SHAPE (SA_ERR_NULL if NULL).
 * Host-only: makes no HIP call. */
sa_status sa_check_shape(const sa_shape* shape);

/*
 * Forward, batch 1, causal, every sequence of length T (the pages' call).
 *   Q, K, Vt: inputs (layouts above).  O, L: outputs, fully overwritten.
 *   c: binary32 nearest scale / ln 2 (e.g. 0x3E38AA3B for scale 1/8).
 */
sa_status sa_forward(const void* Q, const void* K, const void* Vt, void* O, float* L, float c,
                     int T, int heads, int kv_heads, void* stream);

/* Forward for a general shape (batch, causal or not, sequence lengths). */
sa_status sa_forward_ex(const sa_shape* shape, const void* Q, const void* K, const void* Vt,
                        void* O, float* L, float c, void* stream);

/*
 * Bytes of dS workspace sa_backward needs: one fp16 64x64 tile per
 * (batch, query head, query tile, key tile) the dQ pass reads -- the lower
 * triangle including the diagonal when causal, the full square otherwise.
 * Returns 0 if the shape fails admission.
 */
size_t sa_backward_workspace_bytes(const sa_shape* shape);

/*
 * Backward, batch 1, causal, every sequence of length T.
 *   dO: fp16 output gradient.  O, L: this shape's sa_forward outputs.
 *   D: fp32 [H][T] row terms, written (an output the caller may ignore).
 *   dS, dS_bytes: workspace of at least sa_backward_workspace_bytes bytes.
 *   Q, K, Vt: the forward's inputs.  c: as sa_forward; s: the natural
 *   score scale (dQ and dK carry it, dV does not).
 *   dQ, dK, dVt: fp32 gradients, fully overwritten.
 * Launches, in stream order: row terms, key pass (dK, dV^T, dS), dQ pass.
 */
sa_status sa_backward(const void* dO, const void* O, const float* L, float* D,
                      void* dS, size_t dS_bytes,
                      const void* Q, const void* K, const void* Vt, float c, float s,
                      int T, int heads, int kv_heads,
                      float* dQ, float* dK, float* dVt, void* stream);

/* Backward for a general shape; arguments as sa_backward. */
sa_status sa_backward_ex(const sa_shape* shape, const void* dO, const void* O, const float* L,
                         float* D, void* dS, size_t dS_bytes,
                         const void* Q, const void* K, const void* Vt, float c, float s,
                         float* dQ, float* dK, float* dVt, void* stream);

/*
 * The split backward over a dS workspace smaller than the whole problem's
 * (StreamingAttentionSM86 page, banner "The query pass split in two around
 * the key pass": the key pass stores dS, the dQ pass reads it back; here the
 * query rows are taken in chunks so that one chunk's dS at a time occupies
 * the workspace, which a small enough workspace keeps in the chip's last-level
 * cache).  After the row terms, for each chunk of query rows from the last
 * rows to the first: the key pass over that chunk's rows (dK and dV summed
 * onto the earlier chunks' in that fixed order), then the dQ pass over the
 * chunk's rows.  Each chunk is as many 128-row blocks as fit in dS_bytes.
 *   Arguments: as sa_backward_ex.  dS_bytes may be anything from
 *   sa_backward_chunked_min_bytes(shape) (one 128-row block's dS) up; with
 *   dS_bytes >= sa_backward_workspace_bytes(shape) it is one chunk and the
 *   results are bitwise sa_backward_ex's.
 *   Results: deterministic for equal inputs, shape, block order and
 *   dS_bytes; dK and dV sum the chunks in a different order than the
 *   one-chunk backward, so they may differ from it in rounding.
 *   Errors: SA_ERR_WORKSPACE if dS_bytes < sa_backward_chunked_min_bytes;
 *   otherwise as sa_backward_ex.
 */
sa_status sa_backward_chunked(const sa_shape* shape, const void* dO, const void* O, const float* L,
                              float* D, void* dS, size_t dS_bytes,
                              const void* Q, const void* K, const void* Vt, float c, float s,
                              float* dQ, float* dK, float* dVt, void* stream);

/* The smallest dS_bytes sa_backward_chunked accepts (the largest single
 * 128-row block's dS); 0 if the shape fails admission. */
size_t sa_backward_chunked_min_bytes(const sa_shape* shape);

/*
 * The backward's three launches, one at a time, for measurement and tests.
 * sa_backward_ex is exactly these three calls in this order.
 *
 * Row terms (StreamingAttentionSM86 page, banner "The query pass split in
 * two around the key pass", the row terms): D = rowsum(dO * O), binary32,
 * 0 on padded rows.
 */
sa_status sa_row_terms(const sa_shape* shape, const void* dO, const void* O, float* D, void* stream);

/*
 * Key pass (same page, banner "The key launch"; it also stores the score
 * gradients, per the split query pass's banner): for every 64-key tile,
 * recompute S, P and dP for every later query, accumulate dK and dV over the
 * group's heads and store dS (fp16, the words the dK product uses) into the
 * workspace, exact zeros where masked.  dS may be NULL (dS_bytes is then
 * ignored): nothing is stored, as in the two-launch backward's key launch.
 */
sa_status sa_key_pass(const sa_shape* shape, const void* Q, const void* K, const void* Vt,
                      const void* dO, const float* L, const float* D, void* dS, size_t dS_bytes,
                      float c, float s, float* dK, float* dVt, void* stream);

/*
 * dQ pass (same page, split query pass, dQ from stored dS): for each query
 * tile, dQ = s * sum over key tiles up to the diagonal of dS K.
 * The workspace must hold a key pass's dS for the same shape.
 */
sa_status sa_dq_pass(const sa_shape* shape, const void* K, const void* dS, size_t dS_bytes, float s,
                     float* dQ, void* stream);

/*
 * The dQ pass with the rotated epilogue (StreamingAttentionSM86 page, the
 * query pass's "dQ = s (the sum), turned back by the inverse half-split
 * rotation" epilogue, dQ from stored dS): dQ is formed as by sa_dq_pass, and
 * each scaled pair (x1, x2) of columns c and c + 32 (c < 32) of row p of head
 * h becomes (x1 cos + x2 sin, x2 cos - x1 sin), with cos = cos_t[p][c] and
 * sin = sin_t[p][c], rounded to bfloat16 (nearest even) and stored at columns
 * 64 h + c and 64 h + c + 32 of row p of the token-major projection gradient.
 * This is the gradient with respect to the queries before the half-split
 * rotation, laid out as the Q slice of a fused QKV projection's gradient.
 *   cos_t, sin_t: fp32 [T][32], the rotation's tables (shared by the batch
 *                 and the heads), 16-byte aligned.
 *   dqkv:         bf16 [B][T][width]; columns 0 .. 64 heads - 1 of every row
 *                 are overwritten (zeros on padded rows), every other column
 *                 is left untouched.
 *   width:        row length of dqkv in elements: a multiple of 8 and at
 *                 least 64 heads (else SA_ERR_ARGUMENT).
 * dQ itself is not written.  The page's admission also asks for a power-of-
 * two sequence and 32-bit byte offsets; neither is needed here (64-bit
 * addressing, no shift-based indexing).
 */
sa_status sa_dq_pass_rotated(const sa_shape* shape, const void* K, const void* dS, size_t dS_bytes, float s,
                             const float* cos_t, const float* sin_t, void* dqkv, int width, void* stream);

/*
 * The split backward storing its gradients straight into a fused QKV
 * projection's gradient (StreamingAttentionSM86 page: the query launch's
 * "dQ = s (the sum) stored straight into a fused projection's gradient" and
 * the key launch's "dK = s (the sum) and dV stored straight into a fused
 * projection's gradient"): row terms, key pass and dQ pass as sa_backward_ex,
 * but dQ, dK and dV are written token-major, each in binary32 and rounded to
 * bfloat16 (nearest even), instead of into the [head] planes.
 *   dQ32, dQ16:  the Q slice: row p (of batch b) at (b T + p) width, query
 *                head h's 64 values at columns 64 h .. 64 h + 63 of it;
 *   dK32, dK16:  the K slice, K/V head kv at columns 64 kv + 0..63 (the
 *                group sum, scaled by s);
 *   dV32, dV16:  the V slice, the same columns, unscaled.
 * Each pointer names its slice's first column (the caller offsets it into
 * the shared [B][T][width] buffers); fp32 pointers and bf16 pointers are
 * 16-byte aligned.  width: row length in elements, a multiple of 8 and at
 * least 64 heads; the slices must fit in the rows.  Other columns are left
 * untouched; padded rows and keys get zeros.  D and dS as sa_backward_ex.
 */
sa_status sa_backward_projection(const sa_shape* shape, const void* dO, const void* O, const float* L, float* D,
                                 void* dS, size_t dS_bytes, const void* Q, const void* K, const void* Vt,
                                 float c, float s, float* dQ32, void* dQ16, float* dK32, void* dK16,
                                 float* dV32, void* dV16, int width, void* stream);

/*
 * The backward in two launches, with no dS workspace (StreamingAttentionSM86
 * page, banner "The backward pass, deterministic and in two launches (no
 * atomics)"): the query launch forms D and dQ, recomputing S, P and dP per
 * key tile; the key launch forms dK and dV the same way.  S, P and dP are
 * formed twice instead of once, and nothing of size T x T is stored.
 *
 * Query pass: D = rowsum(dO * O) for every row (written, 0 on padded rows),
 * and dQ = s * sum_j dS_ij K_j with dS = P (dP - D), P = 2^(S c - L),
 * dP = dO V^T, walking the key tiles up to the diagonal.
 *   dO, O, L: as sa_backward (O and L this shape's sa_forward outputs).
 *   Q, K, Vt: the forward's inputs.  c, s: as sa_backward.
 *   D, dQ: fp32 outputs, fully overwritten.
 */
sa_status sa_query_pass(const sa_shape* shape, const void* dO, const void* O, const float* L,
                        const void* Q, const void* K, const void* Vt, float c, float s,
                        float* D, float* dQ, void* stream);

/*
 * The two-launch backward: sa_query_pass, then the key pass without a dS
 * store (dK, dV^T).  Arguments as sa_backward_ex without the workspace;
 * results agree with it up to rounding (the score products are formed in
 * another operand orientation).
 */
sa_status sa_backward_two_pass(const sa_shape* shape, const void* dO, const void* O, const float* L,
                               float* D, const void* Q, const void* K, const void* Vt, float c, float s,
                               float* dQ, float* dK, float* dVt, void* stream);

/*
 * The two-launch backward storing into a fused QKV projection's gradient
 * (same page: the shared query pass's and the key launch's projection
 * epilogues): sa_query_pass writing D and dQ's slice, then the key pass
 * without a dS store writing dK's and dV's slices.  The slices, their
 * layout, width and alignment are as sa_backward_projection's; D as
 * sa_backward_two_pass.
 */
sa_status sa_backward_two_pass_projection(const sa_shape* shape, const void* dO, const void* O, const float* L,
                                          float* D, const void* Q, const void* K, const void* Vt, float c, float s,
                                          float* dQ32, void* dQ16, float* dK32, void* dK16, float* dV32, void* dV16,
                                          int width, void* stream);

/*
 * The split backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): sa_backward_chunked with the dS
 * workspace in a static device array of SA_STATIC_SCRATCH_BYTES that the
 * library holds on each GPU until the process ends.  The call itself
 * allocates nothing.
 *   Arguments: as sa_backward_ex without dS and dS_bytes.
 *   Limit: a shape whose sa_backward_chunked_min_bytes exceeds
 *          SA_STATIC_SCRATCH_BYTES returns SA_ERR_TOO_LARGE (checked before
 *          anything else touches the GPU): e.g. batch 1, 32 heads, causal,
 *          runs up to T = 8192 (T = 16384 needs 134 MB for one 128-row
 *          block).
 *   Results: sa_backward_chunked's with dS_bytes = SA_STATIC_SCRATCH_BYTES:
 *          bitwise sa_backward_ex's when the whole dS fits (e.g. batch 1,
 *          T = 1024, 8 heads: 8.9 MB), within rounding of it otherwise.
 *   Concurrency: every call on one GPU shares that GPU's array; calls that
 *          overlap on one GPU (other streams, other host threads) race.  Calls
 *          on one stream run in order and are safe.
 *   Errors: as sa_backward_ex; SA_ERR_DEVICE also if the array's device
 *          address cannot be looked up on the current device.
 */
sa_status sa_backward_static(const sa_shape* shape, const void* dO, const void* O, const float* L, float* D,
                             const void* Q, const void* K, const void* Vt, float c, float s,
                             float* dQ, float* dK, float* dVt, void* stream);

/* Static text for a status value ("unknown status" for anything else). */
const char* sa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
