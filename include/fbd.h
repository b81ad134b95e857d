/*
 * fbd.h -- exact causal multi-head softmax attention on MI355X (gfx950):
 * forward, backward (optionally with GProj), backward-over-backward and the
 * Hessian-vector product built from them; extended forms with shared keys
 * and values (grouped-query attention), a sliding window, document masks and
 * block-sparse masks; a forward on the E4M3 matrix cores.
 *
 * C ABI of libfbd.so.  No torch or C++ types cross this boundary: plain
 * integers, floats and pointers.
 *
 * Layout.  Q, K, V, O, dO and every gradient and cotangent are (B, H, N, d)
 * contiguous row-major arrays (d fastest) of the element type `dt` -- the
 * (batch, heads, seq, head_dim) operand order of the attention call on the
 * FlashAttention explainer page (marketmaker.cc, flash-attention-trading-models,
 * section "Integration is eight lines").  LSE and the workspaces are fp32
 * arrays.  In the extended forms (attn_*_ex) the key-side arrays have Hkv
 * heads instead of H.  Only d = 64 is supported; any N >= 1 is.
 *
 * Pointers.  Every array pointer is a DEVICE pointer owned by the caller,
 * 16-byte aligned (the int32 doc_start of the extended forms: 4-byte; the
 * uint8 block_mask: any).  No call allocates, frees, synchronises, or reads
 * device memory from the host.  Inputs are never written.  Outputs are fully
 * overwritten (never accumulated into) and must not overlap any input, any
 * other output or the workspace.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Each call only enqueues kernels on that stream and returns; it is
 * asynchronous with respect to the host.  Calls on one stream run in order, so
 * attn_bwd / attn_bob may be enqueued right after the attn_fwd whose O and LSE
 * they read.
 *
 * Errors.  Every argument check runs before anything is enqueued, so on any
 * status other than ATTN_OK from validation nothing has been written.  There is
 * no fallback path: an unsupported request returns an error instead of being
 * computed some other way (the explainer page, section "Integration is eight
 * lines", warns that a silent fallback only looks like a slow working model).
 * ATTN_EHIP reports a failed kernel launch; attn_last_hip_error() then
 * returns the hipError_t value (per calling thread).
 *
 * Causal mask.  causal = 1 keeps key j for query i iff j <= i (equal query
 * and key lengths, top-left aligned), and key blocks entirely in the future
 * of a query block are skipped, never loaded (explainer page, section
 * "Causal masking is where trading gets a discount").  causal = 0 is full
 * attention.
 */
#ifndef FBD_H
#define FBD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,       /* null pointer, size <= 0, non-finite or <= 0 scale, overlap */
  ATTN_EUNSUPPORTED = 2, /* d != 64, unknown dtype, sizes beyond the index limits */
  ATTN_EALIGN = 3,       /* a pointer that is not 16-byte aligned */
  ATTN_EWORKSPACE = 4,   /* workspace pointer null or smaller than required */
  ATTN_EHIP = 5          /* a kernel launch failed; see attn_last_hip_error() */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype;

/*
 * Forward pass.  Explainer page, sections "The Flash Attention algorithm" and
 * "The online softmax recurrence": queries are processed in row blocks, key
 * and value blocks are streamed through LDS, and a running row max m and row
 * sum l rescale the output accumulator; no N x N matrix is written.  The max
 * is subtracted before the scale is applied, so the largest weight of a row is
 * exactly 1 (GProj page, rit.work flashattention-bf16-gradient-gproj, section
 * "Why the error shows up at the end of training").
 *
 *   O   = softmax(scale * Q K^T + mask) V                 (B, H, N, d), dtype dt
 *   LSE = scale * m + ln l   (natural log, per row)       (B, H, N) fp32
 *
 * scale must be finite and > 0 (1/sqrt(d) is the usual value).
 */
attn_status attn_fwd(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d,
                     const void* Q, const void* K, const void* V,
                     int causal, float scale,
                     void* O, float* LSE, void* stream);

/* Workspace of attn_bwd in bytes: three fp32 arrays of B*H*N rows, in order
 * D = rowsum(dO o O), r (written only when gproj != 0) and -LSE*log2(e), all
 * written by the row pass for the column pass. */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N);

/*
 * Backward pass.  Explainer page, section "Backward pass: recompute instead of
 * store": P is recomputed tile by tile from Q, K and the saved LSE,
 *   P = exp(scale * S - LSE),  dP = dO V^T,  D = rowsum(dO o O),
 *   dS = P o (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO.
 * A row-block pass computes D and dQ; a column-block pass computes dK and dV.
 *
 * gproj != 0 applies GProj (GProj page, section "How a zero sum turns into a
 * false gradient"): dS is fed to the matrix cores in bf16, so its rows no
 * longer sum to zero; the residual r_i = sum_j R(dS_ij) of exactly those
 * bf16 values is removed in proportion to the probabilities:
 *   dQ = scale * (R(dS) K - r o (R(P) K)),
 *   dK = scale * (R(dS)^T Q - Q^T R(r o P)).
 * The dQ correction rides in the row pass; the dK correction needs r and is
 * applied in the column pass.  For fp32 inputs R is the identity.
 *
 * O and LSE must be the outputs of attn_fwd with the same causal and scale.
 * ws must hold attn_bwd_workspace_bytes(B, H, N) bytes (fp32, device).
 */
attn_status attn_bwd(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d,
                     const void* Q, const void* K, const void* V, const void* O,
                     const float* LSE, const void* dO,
                     int causal, float scale, int gproj,
                     void* dQ, void* dK, void* dV,
                     void* ws, size_t ws_bytes, void* stream);

/* Workspace of attn_bob in bytes: five fp32 arrays of B*H*N rows, in order
 * D, alpha, beta, -LSE*log2(e) and -kappa = -(alpha*D + beta), all written by the
 * row pass for the column pass. */
size_t attn_bob_workspace_bytes(int64_t B, int64_t H, int64_t N);

/*
 * Backward-over-backward: the vector-Jacobian product of the first backward
 * map (Q, K, V, dO) -> (dQ, dK, dV) with cotangents (g_dQ, g_dK, g_dV), i.e.
 * the gradient of <g_dQ, dQ> + <g_dK, dK> + <g_dV, dV> with respect to
 * (Q, K, V, dO).  FlashBoB page (rit.work, flashbob-second-order-attention),
 * sections "Why go backward through an already computed gradient" and "Two
 * scalar states replace quadratic tensors": a row-block pass streams key
 * blocks, reduces each row's global dependence to two fp32 states
 *   alpha_i = sum_j P_ij W_ij,
 *   beta_i  = sum_j P_ij (W_ij (dP_ij - D_i) - alpha_i dP_ij + U_ij),
 * with W = scale (g_dQ K^T + Q g_dK^T) and U = dO g_dV^T, and finishes g_Q and
 * g_dO; a column-block pass streams query blocks past resident key blocks,
 * reads the row states and finishes g_K and g_V.  Each output block is
 * written once and no N x N matrix reaches device memory.
 *
 * O and LSE must be the outputs of attn_fwd with the same causal and scale.
 * ws must hold attn_bob_workspace_bytes(B, H, N) bytes; after the call it
 * holds D, alpha and beta (then two derived row arrays).
 */
attn_status attn_bob(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d,
                     const void* Q, const void* K, const void* V, const void* O,
                     const float* LSE, const void* dO,
                     const void* g_dQ, const void* g_dK, const void* g_dV,
                     int causal, float scale,
                     void* g_Q, void* g_K, void* g_V, void* g_dO,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * attn_bob for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, arguments, kernels and errors as attn_bob with no
 * workspace argument.  The row states live in a library-owned device array
 * of ATTN_BOB_NOALLOC_MAX_ROWS * 5 floats (60 MiB), one copy per GPU the
 * library runs on, held until the process ends; its device address is looked
 * up once per device, on the first call there.  The call allocates and frees
 * nothing.  B * H * N above ATTN_BOB_NOALLOC_MAX_ROWS (12 heads at N = 262144)
 * returns ATTN_EWORKSPACE before anything is enqueued.  Every call on one GPU
 * uses that GPU's array, so calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller;
 * calls on one stream are ordered.  Nothing in the array needs clearing: the
 * row pass writes every state the column pass reads.  Multi-head only (the
 * extended forms take a workspace).
 */
#define ATTN_BOB_NOALLOC_MAX_ROWS 3145728
attn_status attn_bob_noalloc(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d,
                             const void* Q, const void* K, const void* V, const void* O,
                             const float* LSE, const void* dO,
                             const void* g_dQ, const void* g_dK, const void* g_dV,
                             int causal, float scale,
                             void* g_Q, void* g_K, void* g_V, void* g_dO, void* stream);

/*
 * The two passes of attn_bwd / attn_bob as separate calls, for callers that
 * schedule or time them on their own.  `passes` is 1 (row-block pass only),
 * 2 (column-block pass only) or 3 (both; identical to attn_bwd / attn_bob).
 * The column pass reads the row states the row pass left in `ws` (D and r,
 * or D, alpha and beta), so a pass-2 call must follow a pass-1 call with the
 * same arguments on the same stream.  The row pass writes dQ (g_Q, g_dO),
 * the column pass dK, dV (g_K, g_V); all output pointers are validated in
 * either case.  Other arguments and errors as for attn_bwd / attn_bob;
 * passes outside 1..3 is ATTN_EINVAL.
 */
attn_status attn_bwd_passes(int passes, attn_dtype dt, int64_t B, int64_t H, int64_t N,
                            int64_t d, const void* Q, const void* K, const void* V,
                            const void* O, const float* LSE, const void* dO,
                            int causal, float scale, int gproj,
                            void* dQ, void* dK, void* dV,
                            void* ws, size_t ws_bytes, void* stream);

attn_status attn_bob_passes(int passes, attn_dtype dt, int64_t B, int64_t H, int64_t N,
                            int64_t d, const void* Q, const void* K, const void* V,
                            const void* O, const float* LSE, const void* dO,
                            const void* g_dQ, const void* g_dK, const void* g_dV,
                            int causal, float scale,
                            void* g_Q, void* g_K, void* g_V, void* g_dO,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Extended forms: shared keys and values, a sliding window, document masks
 * and block-sparse masks.  The FlashBoB
 * page (rit.work, flashbob-second-order-attention), in its closing paragraph
 * on where the method applies, names shared keys and values and flexible
 * masks among the extensions after plain multi-head attention.
 *
 * Shared keys and values (grouped-query / multi-query attention): Hkv
 * key/value heads serve H query heads (1 <= Hkv <= H, H % Hkv == 0); query
 * head h of a batch uses key head h / (H / Hkv).  Query-side tensors (Q, O,
 * dO, dQ, g_dQ, g_Q, g_dO), LSE and the workspace have H heads; key-side
 * tensors (K, V, dK, dV, g_dK, g_dV, g_K, g_V) are (B, Hkv, N, d).  The
 * key-side gradients are sums over each group's query heads: the column
 * passes stream every query head of a group past the resident key block, so
 * each key-side block is still written once.  Hkv == H is multi-head
 * attention; Hkv == 1 is multi-query attention.
 *
 * Split column passes (grouped-query heads only): when a group's column
 * workgroups alone would be too few to fill the chip (under 1536 of them),
 * each group's query heads are divided into slices that separate workgroups
 * stream; each slice writes fp32 partial sums of its key-side results into
 * the workspace, and one more kernel adds the slices up, in a fixed order,
 * into dK, dV (g_K, g_V).  This happens only when ws_bytes is at least
 * attn_bwd_ex_workspace_bytes (attn_bob_ex_workspace_bytes); a workspace of
 * attn_bwd_workspace_bytes (attn_bob_workspace_bytes) runs the unsplit
 * column pass, whose results differ only in the fp32 summation order over a
 * group.  The partial sums sit after the row states at the next 256-byte
 * boundary; the row-state layout is unchanged.
 *
 * Sliding window (window > 0, causal only): key j is visible to query i iff
 * i - window < j <= i.  Tiles wholly outside the window are never loaded.
 * window == 0 is plain causal (or full, with causal == 0) attention.
 *
 * Document masks (doc_start != NULL, causal only): packed sequences of
 * several documents per batch row.  doc_start is a device (B, N) int32 array
 * (4-byte aligned, read-only) giving for each query position the position of
 * its document's first token: key j is visible to query i of batch b iff
 * doc_start[b][i] <= j <= i (and within the window, if any).  It must be
 * non-decreasing along i with doc_start[b][i] <= i; other contents give
 * unspecified values but stay within every buffer.  The kernels skip tiles
 * outside the documents: a key block's column pass finds the last query row
 * it reaches with a wave-parallel search of doc_start.
 *
 * Block-sparse masks (block_mask != NULL, causal or not): a device (B, nb,
 * nb) uint8 array, nb = ceil(N / 128), row-major (query block, then key
 * block), read-only, any alignment.  block_mask[b][qb][kb] == 0 hides keys
 * 128 kb .. 128 kb + 127 from queries 128 qb .. 128 qb + 127 of batch b (all
 * heads), on top of the other masks; such blocks are never loaded, so the
 * cost follows the kept blocks.  A query left with no visible key gets O = 0,
 * LSE = -infinity and zero gradients and BoB outputs (the oracle's
 * convention for an empty softmax row).
 *
 * gproj != 0 in attn_bob_ex carries GProj (GProj page, section "How a zero
 * sum turns into a false gradient") over to g_Q.  The row pass writes the
 * weights of K in g_Q as
 *   Sh = P o (W o (dP - D) + U) - alpha dS - kappa P,   kappa = alpha D + beta
 * (P o dP = dS + D P), three parts that sum to exactly zero over each row;
 * it sends them to the matrix cores as separate bf16 operands, x = P o (W o
 * (dP - D) + U), dS and P, and combines them after the sums over keys.  The
 * residual row sum r_Sh of those operands (taken over exactly the bf16
 * values) would carry a false multiple of the keys' mean into g_Q, large
 * where the keys share a large mean and rows are near one-hot (the GProj
 * page's large-key regime).  With gproj it is removed along R(P) K:
 *   g_Q = scale * (sum_j R(x) K + R(dS) B_K - alpha sum_j R(dS) K
 *                  - (kappa + r_Sh) sum_j R(P) K).
 * g_dO's weights of V, P o (W - alpha), also sum to zero over each row; the
 * pass forms g_dO = sum_j R(P o W) V + R(P) C - alpha O, and with gproj their
 * residual r_H = sum_j R(P o W) - alpha is removed along O:
 *   g_dO = sum_j R(P o W) V + R(P) C - (alpha + r_H) O.
 * It changes g_Q and g_dO only, costs four row sums per tile of the row pass,
 * and has no effect on fp32 operands (nothing is rounded there); exact
 * arithmetic gives r_Sh = r_H = 0.
 *
 * With Hkv == H, window == 0, no doc_start, no block_mask and gproj == 0 these
 * equal attn_fwd / attn_bwd / attn_bob.  Hkv outside the range above, window < 0 or
 * a doc_start or block_mask that overlaps an output is ATTN_EINVAL; a
 * misaligned doc_start is ATTN_EALIGN;
 * window > 0 or doc_start with causal == 0 is ATTN_EUNSUPPORTED; other
 * arguments and errors as for the multi-head entry points (workspace sizes
 * count the H query heads).  The backward and BoB must get the same causal,
 * window, doc_start and block_mask as the forward.
 */
/* Workspace bytes that let attn_bwd_ex / attn_bob_ex split their column
 * passes (see above): the multi-head size when no split applies (Hkv == H, or
 * enough key blocks), else that size rounded up to 256 bytes plus
 * 2 * nslices * B * Hkv * N * 64 floats.  0 for invalid sizes. */
size_t attn_bwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N);
size_t attn_bob_ex_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N);

attn_status attn_fwd_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V,
                        int causal, int64_t window, const int32_t* doc_start,
                        const uint8_t* block_mask, float scale,
                        void* O, float* LSE, void* stream);

attn_status attn_bwd_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V, const void* O,
                        const float* LSE, const void* dO,
                        int causal, int64_t window, const int32_t* doc_start,
                        const uint8_t* block_mask, float scale,
                        int gproj, void* dQ, void* dK, void* dV,
                        void* ws, size_t ws_bytes, void* stream);

attn_status attn_bob_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V, const void* O,
                        const float* LSE, const void* dO,
                        const void* g_dQ, const void* g_dK, const void* g_dV,
                        int causal, int64_t window, const int32_t* doc_start,
                        const uint8_t* block_mask, float scale, int gproj,
                        void* g_Q, void* g_K, void* g_V, void* g_dO,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Hessian-vector product of one attention layer, the product that
 * second-order training consumes (FlashBoB page, section "Why go backward
 * through an already computed gradient": Hessian-vector products for methods
 * such as Sophia need the backward pass differentiated once more).  For
 *   Phi(Q, K, V) = <dO, O(Q, K, V)>  with dO held fixed,
 * the gradient is (dQ, dK, dV) (attn_bwd), so the Hessian applied to
 * v = (v_Q, v_K, v_V) is the vector-Jacobian product of that gradient map
 * with cotangents v: attn_bob with (g_dQ, g_dK, g_dV) = (v_Q, v_K, v_V).
 * One call runs
 *   attn_fwd                 -> O, LSE
 *   attn_bwd (if dQ != NULL) -> dQ, dK, dV   (GProj when gproj != 0)
 *   attn_bob_ex              -> Hv_Q, Hv_K, Hv_V = H v, and Hv_dO = the
 *      derivative of <v, (dQ, dK, dV)> with respect to dO, the term a
 *      network-level product adds through dO's own dependence on the inputs.
 * dQ, dK and dV are all NULL (gradient not computed) or all set.  Every
 * output is overwritten.  With bf16 operands and the gradient requested, the
 * backward's row pass is not run on its own: the BoB row pass already sums
 * sum_j R(dS_ij) K_j and sum_j R(P_ij) K_j, which are exactly the backward
 * row pass's dQ terms; it writes dQ, then the backward's and BoB's column
 * passes run.  gproj != 0 also applies attn_bob_ex's projections of Hv_Q's
 * and Hv_dO's residual row sums (the same flag as attn_bob_ex's gproj).  dQ,
 * dK, dV come out as attn_bwd's, and H v as attn_bob_ex's with the same
 * gproj, bit for bit.
 * ws must hold attn_hvp_workspace_bytes(B, H, N) bytes (six fp32
 * values per row); afterwards it starts with the BoB row states as after
 * attn_bob (D, alpha, beta, -LSE log2(e), -kappa), followed by the GProj row
 * sums r when the gradient was computed.  Shapes, layouts, ownership and
 * errors as for attn_bob (the v_* are read-only inputs); a partial set of
 * gradient pointers is ATTN_EINVAL.
 */
size_t attn_hvp_workspace_bytes(int64_t B, int64_t H, int64_t N);

attn_status attn_hvp(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d,
                     const void* Q, const void* K, const void* V, const void* dO,
                     const void* v_Q, const void* v_K, const void* v_V,
                     int causal, float scale, int gproj,
                     void* O, float* LSE, void* dQ, void* dK, void* dV,
                     void* Hv_Q, void* Hv_K, void* Hv_V, void* Hv_dO,
                     void* ws, size_t ws_bytes, void* stream);

/* The Hessian-vector product over the extended forms: Hkv key/value heads, a
 * causal sliding window, document starts and a block-sparse mask, with the
 * meanings, shapes and errors of attn_fwd_ex / attn_bwd_ex / attn_bob_ex.
 * K, V, v_K, v_V, dK, dV, Hv_K and Hv_V are (B, Hkv, N, d).  The Hessian is
 * that of Phi = <dO, O> as a function of the shared K and V, so Hv_K and
 * Hv_V are sums over each group's query heads, as dK and dV are.  ws must
 * hold attn_hvp_workspace_bytes(B, H, N); with
 * attn_hvp_ex_workspace_bytes(B, H, Hkv, N) the grouped-query column passes
 * split (as in attn_bwd_ex).  attn_hvp is the Hkv == H case with no masks
 * beyond causal. */
size_t attn_hvp_ex_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N);

attn_status attn_hvp_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V, const void* dO,
                        const void* v_Q, const void* v_K, const void* v_V,
                        int causal, int64_t window, const int32_t* doc_start,
                        const uint8_t* block_mask, float scale, int gproj,
                        void* O, float* LSE, void* dQ, void* dK, void* dV,
                        void* Hv_Q, void* Hv_K, void* Hv_V, void* Hv_dO,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * FP8 forward with optional incoherent processing.
 *
 * The FlashAttention explainer page (marketmaker.cc,
 * flash-attention-trading-models), section "FA3: the Hopper mechanics",
 * item 3, describes FP8 attention.  Plain block quantisation is hurt by
 * outliers, so the vectors are first multiplied by a random orthogonal matrix
 * that spreads an outlier over all coordinates.  Here that matrix is
 * R = diag(s) H / 8: H is the 64 x 64 Sylvester Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)) and s_i = -1 where bit i of `signs` is
 * set.  Since (Q R)(K R)^T = Q K^T, only the rounding changes.
 *
 * Format: OCP E4M3 (4 exponent bits, bias 7, 3 mantissa bits, subnormals,
 * largest finite value 448), rounded to nearest with ties to even.
 * Scales are powers of two, 2^e with e = floor(log2 amax) - 7 (0 for an
 * all-zero block), so each block's largest magnitude maps into [128, 256).
 * Q and K (rotated when rotate != 0) get one exponent per 64 rows of a head;
 * V (never rotated) gets one per column of a head.  Inputs must be finite,
 * and the score scale 2^(eq + ek) of a query block and a key block must be
 * a normal fp32 number.
 *
 * Two calls.  attn_fp8_quantize reads Q (B, H, N, 64) and K, V (B, Hkv, N,
 * 64) of type dt and writes the codes and exponents into the workspace.
 * attn_fwd_fp8 reads only the workspace and writes O (B, H, N, 64) of type dt
 * and LSE (B, H, N) fp32, the same outputs as attn_fwd_ex (with its window,
 * doc_start and block_mask, same rules and errors), computed with both
 * products on the E4M3 matrix cores.  The probabilities are rounded to E4M3
 * as 256 P against the running row max; l sums the unrounded values.
 * The workspace is device memory of attn_fp8_workspace_bytes(B, H, Hkv, N)
 * bytes, 16-byte aligned.  Its parts start at the offsets that
 * attn_fp8_workspace_layout writes, in the order of attn_fp8_part; each part
 * is per head, heads in order:
 *   Q, K   N x 64 uint8 codes, row-major;
 *   VT     64 x NP uint8 codes (NP = N rounded up to 64): row d is column d
 *          of V.  Within each group of 64 keys, stored 4-byte word w holds
 *          keys 4s .. 4s+3 with s = 2 (w % 8) + w / 8.  Keys past N are zero;
 *   EQ, EK int32 exponent per 64-row block (ceil(N / 64) per head);
 *   EV     int32 exponent per column (64 per head);
 *   VMAX   scratch of the pre-pass.
 * Errors as elsewhere; ATTN_EWORKSPACE for a missing or short workspace.
 * ------------------------------------------------------------------------ */
typedef enum {
  ATTN_FP8_Q = 0, ATTN_FP8_K = 1, ATTN_FP8_VT = 2, ATTN_FP8_EQ = 3, ATTN_FP8_EK = 4,
  ATTN_FP8_EV = 5, ATTN_FP8_VMAX = 6, ATTN_FP8_NPARTS = 7
} attn_fp8_part;

/* Bytes of the FP8 workspace (0 for non-positive sizes). */
size_t attn_fp8_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N);

/* Byte offsets of the ATTN_FP8_NPARTS parts of the workspace, written to
 * offsets[0 .. ATTN_FP8_NPARTS-1] (host array). */
attn_status attn_fp8_workspace_layout(int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                      size_t* offsets);

attn_status attn_fp8_quantize(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                              int64_t d, const void* Q, const void* K, const void* V,
                              int rotate, uint64_t signs, void* ws, size_t ws_bytes,
                              void* stream);

attn_status attn_fwd_fp8(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                         const void* ws, size_t ws_bytes, int causal, int64_t window,
                         const int32_t* doc_start, const uint8_t* block_mask, float scale,
                         void* O, float* LSE, void* stream);

/* Text of a status code (static storage). */
const char* attn_status_str(attn_status s);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FBD_H */
