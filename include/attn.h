/*
 * attn.h -- C ABI of the gfx950 (MI355X) attention library libattn.so.
 *
 * The library computes exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 * and its gradients.  The forward pass is one fused tiled kernel that keeps,
 * for every query row, a running maximum m and a running exponential sum l and
 * never writes the N x N score matrix S or probability matrix P to memory
 * ("digest_existing.txt", answer q02_flashattention, sections 1 and 2: S and
 * P need not be materialised; the merge rule m = max(m1, m2),
 * l = e^(m1-m) l1 + e^(m2-m) l2).  The backward pass regenerates P from the
 * inputs and the per-row log-sum-exp saved by the forward pass
 * ("GPU Programming and Kernel Optimization", item 58).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are device pointers to dense row-major arrays.  With H query heads,
 * Hk key/value heads, Nq query rows and Nk key rows per head (Hk = H and
 * Nq = Nk = N for the entry points that take one H and one N):
 *   q, o, dout, dq : bfloat16 (raw 16-bit patterns), [B, H, Nq, d]
 *   k, v, dk, dv   : bfloat16, [B, Hk, Nk, d]
 *   lse, delta     : float32, [B, H, Nq]
 * Grouped-query attention: H is a multiple of Hk and query head h uses K/V
 * head h / (H / Hk) (the kernel wiki's "FlashAttention v3 (Tri Dao et al.)"
 * page, sections "What it is" and "Runtime parameters": separate counts of
 * query heads and K/V heads); dk and dv of a K/V head sum over its query
 * heads.  Hk = 1 is multi-query attention.
 * lse is the natural log of sum_j exp(scale * <q_i, k_j>) over the keys j that
 * query i sees; delta is D_i = sum_c dout[i][c] * o[i][c].
 * Causal masking (causal = 1) hides key j from query i when j > i + (Nk - Nq),
 * i.e. the mask is aligned to the bottom-right corner of the Nq x Nk score
 * matrix ("GPU Programming and Kernel Optimization", item 59),
 * which is the plain j > i when Nq = Nk.  A query that sees no key at all
 * (causal with Nq > Nk, rows i < Nq - Nk, or Nk = 0) gets o = 0, lse = -inf,
 * and dq = 0; it adds nothing to dk and dv.
 * scale is the factor applied to the dot products (usually 1/sqrt(d)).
 *
 * Ownership: the caller owns every buffer.  The library neither allocates,
 * frees nor keeps any pointer after a call returns.  Outputs must not overlap
 * inputs or each other.
 *
 * Asynchrony: a successful call only enqueues kernels on `stream` (a
 * hipStream_t; NULL means the default stream) and returns; completion is
 * observed by the caller through the stream.  Calls on one stream run in order.
 *
 * Errors: every entry point checks its arguments on the host before any HIP
 * call.  On a nonzero status nothing was enqueued and no output was touched.
 * The library never aborts or prints.  An empty problem (B, H or N equal to 0)
 * is valid, enqueues nothing and returns ATTN_OK; more generally a pointer to a
 * buffer of zero bytes may be NULL.
 * Sizes: B, H, Hk, N (Nq, Nk) >= 0; d in {64, 128, 192, 256}; B*H*N*d < 2^62;
 * (N + 256)*d*2 < 2^32 for N = Nq and N = Nk.  Pointers must be 16-byte aligned
 * (the per-head scale arrays of attn_fwd_fp8: 4-byte aligned).
 */
#ifndef ATTN_H_
#define ATTN_H_

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULLPTR = 1,        /* a required pointer is NULL (non-empty problem) */
    ATTN_ERR_BAD_SHAPE = 2,      /* a size negative, H not a multiple of Hk, or a limit exceeded */
    ATTN_ERR_UNSUPPORTED_D = 3,  /* head dimension d is not 64, 128, 192 or 256 */
    ATTN_ERR_MISALIGNED = 4,     /* a pointer is not 16-byte aligned */
    ATTN_ERR_BAD_SCALE = 5,      /* scale is not finite or not > 0 */
    ATTN_ERR_BAD_ARG = 6,        /* causal is not 0 or 1, or num_splits is not in 1..256 */
    ATTN_ERR_ALIAS = 7,          /* an output overlaps an input or another output */
    ATTN_ERR_HIP = 8,            /* the HIP runtime reported an error at launch */
    ATTN_ERR_WORKSPACE = 9,      /* a workspace is smaller than the call needs */
    ATTN_ERR_SCRATCH = 10        /* the call needs more than the library's static scratch buffer */
};

/* Forward pass.  Reads q, k, v; writes o [B,H,N,d] (bf16, rounded to nearest
 * even) and lse [B,H,N] (fp32, natural log).  One kernel launch.
 * Defines: O = softmax(scale Q K^T) V ("digest_existing.txt", answer
 * q02_flashattention, section 1), computed blockwise with the running maximum
 * and sum of section 2 and the rescaling of "GPU Programming and Kernel
 * Optimization", item 58; lse is the log of that softmax's denominator. */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int B, int H, int N, int d, int causal, float scale, void *stream);

/* Forward pass with H query heads and Hk K/V heads, Nq query rows and Nk
 * key/value rows per head (see the conventions above for grouped heads, the
 * causal alignment and rows that see no key).  Defines: the same O and lse
 * as attn_fwd, with the bottom-right causal alignment of "GPU Programming and
 * Kernel Optimization", item 59, and the separate query and K/V head counts
 * of the "FlashAttention v3 (Tri Dao et al.)" page, "Runtime parameters".
 * attn_fwd(..., H, N, ...) is attn_fwd_qk(..., H, H, N, N, ...). */
int attn_fwd_qk(const void *q, const void *k, const void *v, void *o, float *lse,
                int B, int H, int Hk, int Nq, int Nk, int d, int causal, float scale, void *stream);

/* Split-key forward pass, for few query rows and many keys (decoding): the
 * key range is cut into num_splits pieces ("GPU Programming and Kernel
 * Optimization", item 59: small-query attention split across thread blocks
 * with a separate combining kernel).  One launch computes, for every query
 * block and piece, the piece's normalised output O_s (fp32) and its lse_s into
 * `workspace`; a second launch merges the pieces of each row with the merge
 * rule of the running maxima and sums: lse = log sum_s exp(lse_s),
 * O = sum_s exp(lse_s - lse) O_s.  Results equal attn_fwd_qk's up to rounding.
 * With at most 4 query rows per head and d = 64, 128 or 256 (decoding) the
 * pieces come from a kernel that reads each piece's keys and values once for
 * all query rows of a K/V head (in groups of up to 4 rows) and keeps P in fp32;
 * otherwise from the tiled forward kernel.
 * workspace: caller-owned device memory of at least
 * attn_fwd_splitkv_workspace_size(B, H, Nq, d, num_splits) bytes, 16-byte
 * aligned, not overlapping any input or output; its contents on entry do not
 * matter.  num_splits in 1..256 (attn_fwd_splitkv_default_splits suggests one);
 * pieces past the last key a row sees hold no key and drop out of the merge. */
int attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                     int B, int H, int Hk, int Nq, int Nk, int d, int causal, float scale,
                     int num_splits, void *workspace, long long workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): attn_fwd_splitkv with
 * its workspace taken from a static device buffer of ATTN_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing.  Same arguments, results (bitwise) and
 * errors as attn_fwd_splitkv without workspace and workspace_bytes, plus
 * ATTN_ERR_SCRATCH when attn_fwd_splitkv_workspace_size(B, H, Nq, d,
 * num_splits) exceeds the buffer (checked on the host, nothing enqueued).
 * Every call on a GPU uses that GPU's one buffer: calls that overlap in time
 * on one GPU (different streams or host threads) race and must be ordered by
 * the caller; calls on one stream are ordered.  The first call on a device
 * looks up the buffer's device address once (a host query, no allocation). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16LL << 20)
int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                             int B, int H, int Hk, int Nq, int Nk, int d, int causal, float scale,
                             int num_splits, void *stream);

/* Bytes of workspace attn_fwd_splitkv needs: num_splits * B * H * Nq * (d + 1) * 4
 * (one fp32 output row and one lse per piece and query row, the partial results
 * that "GPU Programming and Kernel Optimization", item 59, combines in a second
 * kernel); -1 for invalid arguments or a size of 2^62 bytes or more. */
long long attn_fwd_splitkv_workspace_size(int B, int H, int Nq, int d, int num_splits);

/* A number of pieces for attn_fwd_splitkv with Hk K/V heads under H query heads
 * (Hk divides H): enough workgroups to fill the GPU (about one 8-wave workgroup
 * per compute unit; with at most 4 query rows per head, where the pieces come
 * from 4-wave workgroups over groups of up to 4 query rows of a K/V head, about
 * 512 of them) while keeping at least two 64-key blocks per piece and at most
 * 128 pieces; 1 when splitting does not help or the arguments are invalid.  (A
 * launch heuristic: the pages say only that small-query attention is split
 * across thread blocks, "GPU Programming and Kernel Optimization", item 59, and
 * that too few blocks leave the GPU underused.) */
int attn_fwd_splitkv_default_splits_qk(int B, int H, int Hk, int Nq, int Nk, int d);

/* attn_fwd_splitkv_default_splits_qk with Hk = H. */
int attn_fwd_splitkv_default_splits(int B, int H, int Nq, int Nk, int d);

/* Forward pass on 8-bit inputs ("FlashAttention v3 (Tri Dao et al.)",
 * section "What it is": FP8 input types; the "CUTLASS WGMMA Atom Skeleton"
 * page, table "Atom Family Names Seen In CUTLASS": FP8 products take e4m3).
 * q [B,H,Nq,d], k and v [B,Hk,Nk,d] hold e4m3 codes (OCP form: bias 7, no
 * infinity, largest 448), one byte each, 16-byte aligned.  descale_q [B*H],
 * descale_k and descale_v [B*Hk] are fp32 device arrays (4-byte aligned) of
 * per-head scales: the real input of head (b, h) is descale[b*H + h] times the
 * code's value ("GPU Programming and Kernel Optimization", item 33: affine
 * quantisation with zero point 0).  The scales must be finite and > 0.
 * Computes the same O and lse as attn_fwd_qk on those real inputs: o is bf16
 * [B,H,Nq,d], lse fp32 [B,H,Nq] (natural log, with `scale` as there).  Both
 * products run on 8-bit operands with fp32 accumulation; the probabilities
 * are rounded to e4m3 before the product with V, which makes O less exact
 * than the 16-bit path (each probability carries up to 2^-4 relative
 * rounding).  d in {64, 128} (else ATTN_ERR_UNSUPPORTED_D); causal alignment,
 * grouped heads and empty rows as in the conventions above. */
int attn_fwd_fp8(const void *q, const void *k, const void *v,
                 const float *descale_q, const float *descale_k, const float *descale_v,
                 void *o, float *lse, int B, int H, int Hk, int Nq, int Nk, int d, int causal,
                 float scale, void *stream);

/* Backward pass: the gradients of attn_fwd's O with respect to q, k and v
 * given dout = dL/dO, regenerating P from q, k and the saved lse instead of
 * storing it ("GPU Programming and Kernel Optimization", item 58); the
 * derivative itself is the chain rule of the definition in
 * "digest_existing.txt", answer q02_flashattention, section 1 (the pages print
 * no backward formula).  Enqueues attn_bwd_dq_delta then attn_bwd_dkdv (two
 * kernel launches) on `stream`; the results are bitwise those of attn_bwd_preprocess,
 * attn_bwd_dkdv and attn_bwd_dq run in that order.  Reads q, k, v, o, dout and
 * the lse written by attn_fwd with the same q, k, v, causal and scale; writes
 * dq, dk, dv [B,H,N,d] (bf16) and delta [B,H,N] (fp32), a caller-owned
 * workspace that holds D on return. */
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
             const float *lse, void *dq, void *dk, void *dv, float *delta,
             int B, int H, int N, int d, int causal, float scale, void *stream);

/* Backward pass with H query heads and Hk K/V heads, Nq query rows and Nk
 * key/value rows per head (the gradients of attn_fwd_qk; the alignment of
 * "GPU Programming and Kernel Optimization", item 59, and the head counts of
 * the "FlashAttention v3 (Tri Dao et al.)" page, "Runtime parameters"); the
 * same kernels as attn_bwd (the dK/dV
 * kernel loops over the H / Hk query heads of each K/V head).  delta is
 * [B, H, Nq].  With Nq = 0 it writes dk = dv = 0; with Nk = 0 it writes dq = 0. */
int attn_bwd_qk(const void *q, const void *k, const void *v, const void *o, const void *dout,
                const float *lse, void *dq, void *dk, void *dv, float *delta,
                int B, int H, int Hk, int Nq, int Nk, int d, int causal, float scale, void *stream);

/* The backward steps below take one length N (Nq = Nk = N); they exist so
 * that each kernel can be enqueued and timed on its own. */

/* Backward step 1: delta[i] = sum_c dout[i][c] * o[i][c] (fp32 products and
 * sums of the bf16 inputs).  Memory-bound; one kernel launch.  D_i is the
 * softmax chain rule's sum_j P_ij dP_ij, which equals <dO_i, O_i> because
 * O_i = sum_j P_ij v_j (section 1 of the digest's q02 answer). */
int attn_bwd_preprocess(const void *o, const void *dout, float *delta,
                        int B, int H, int N, int d, void *stream);

/* Backward step 2 (P regenerated from the saved statistics, "GPU Programming
 * and Kernel Optimization", item 58): for every key block, loops over the
 * query blocks that see it, regenerates P = exp(scale * Q K^T - lse) and
 * accumulates
 * dv = P^T dout and dk = scale * dS^T q with dS = P * (dout V^T - delta).
 * Writes dk and dv; one kernel launch. */
int attn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout,
                  const float *lse, const float *delta, void *dk, void *dv,
                  int B, int H, int N, int d, int causal, float scale, void *stream);

/* Backward step 3 (as step 2, item 58): for every query block, loops over the
 * key blocks it sees, regenerates P and dS as above and accumulates
 * dq = scale * dS k.  Writes dq;
 * one kernel launch.  No atomics: results are bitwise reproducible. */
int attn_bwd_dq(const void *q, const void *k, const void *v, const void *dout,
                const float *lse, const float *delta, void *dq,
                int B, int H, int N, int d, int causal, float scale, void *stream);

/* Backward steps 1 and 3 together, in one kernel launch: writes delta
 * exactly as attn_bwd_preprocess does (bitwise) and dq exactly as attn_bwd_dq
 * does with that delta.  The dQ kernel forms D of its own rows from o and dout
 * before its loop, summing in the preprocess kernel's order.  attn_bwd_dkdv,
 * which needs every row's D, is enqueued after it.  Same arguments and errors
 * as attn_bwd_dq, plus o (an input) and delta (an output, no longer an
 * input). */
int attn_bwd_dq_delta(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, float *delta, void *dq,
                      int B, int H, int N, int d, int causal, float scale, void *stream);

/* Static, NUL-terminated description of a status code (never NULL).  Error
 * reporting of this library; not an operation of the pages. */
const char *attn_status_string(int status);

/* The hipError_t value behind the last ATTN_ERR_HIP returned on the calling
 * thread (0 if none).  Error reporting of this library, as above. */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
