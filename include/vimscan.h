/*
 * vimscan.h -- C ABI of the MI355X (gfx950) selective-scan library
 * (libvimscan.so).
 *
 * The operation is the selective state space scan (S6) as described on
 * "Vision Mamba Guide: Efficient Bidirectional SSM & VMamba" (aifetchly
 * blog):
 *   - section "Discretization via Zero-Order Hold": A_bar = exp(delta A),
 *     B_bar ~= delta B, h_t = A_bar h_{t-1} + B_bar x_t, y_t = C h_t;
 *   - section "Continuous-Time State Space Equations": the D x skip term;
 *   - box "The Selective State Space (S6) Mechanism": delta_t = softplus(.)
 *     and B_t, C_t change with every token;
 *   - section "2. The Bidirectional Mamba Block": a forward pass over the
 *     tokens, a backward pass in reverse order, and the gated fusion
 *     (y_f + y_b) * silu(z);
 *   - section "VMamba: 2D Selective Scan (SS2D) and Cross-Scan Traversal":
 *     four scan orders of an H x W grid (row-major, its reverse,
 *     column-major, its reverse), merged by summation.
 * The PyTorch code on the same page fixes A as diagonal (one decay per
 * state), zero initial state, and B_t, C_t shared by every channel.
 *
 * Per direction k, channel d and batch b, with p = pi_k(t) the token visited
 * at scan step t:
 *     delta = softplus(delta_raw[b,d,p] + dt_bias[k,d])   (or without softplus)
 *     h[n]  = exp(delta * A[k,d,n]) * h[n] + delta * B_t[n] * u[b,d,p]
 *     y_k[b,d,p] = sum_n C_t[n] * h[n] + Dskip[k,d] * u[b,d,p]
 * and the result is y[b,d,p] = (sum_k y_k[b,d,p]) * silu(z[b,d,p]) (no gate
 * when z is NULL). State and arithmetic are fp32 whatever the input dtype.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer on the current HIP device,
 *     owned by the caller (for example PyTorch's caching allocator). The
 *     library allocates nothing and keeps no pointer after it returns.
 *   - Activations (u, delta, z, B, C, y) are contiguous, in the dtype given
 *     by `dtype`; A, Dskip and dt_bias are contiguous fp32.
 *   - Layout is channel-major: u, delta, z, y are [batch][dim][L].
 *   - The call is asynchronous: it validates on the host, enqueues the
 *     kernels on `stream` (a hipStream_t; NULL is the null stream) and
 *     returns. Faults during execution surface at the caller's next
 *     synchronisation.
 *   - Errors are returned as negative status codes, checked before any HIP
 *     call is made; nothing is enqueued on error. vs_strerror() names a code
 *     and vs_last_error() gives the calling thread's last detailed message.
 *   - y must not overlap any input or the workspace (VS_ERR_ALIAS).
 *   - Thread-safe and re-entrant; calls on different streams are
 *     independent, provided their y and workspace buffers are distinct.
 */
#ifndef VIMSCAN_H
#define VIMSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VS_ABI_VERSION 1

/* dtype of u, delta, z, B, C and y */
enum { VS_F32 = 0, VS_BF16 = 1 };

/* status codes */
enum {
    VS_OK = 0,
    VS_ERR_NULL = -1,        /* a required pointer is NULL */
    VS_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or too large */
    VS_ERR_DTYPE = -3,       /* unknown dtype */
    VS_ERR_ALIGN = -4,       /* a pointer is not aligned to its element size */
    VS_ERR_ALIAS = -5,       /* y overlaps an input or the workspace */
    VS_ERR_UNSUPPORTED = -6, /* valid but not supported by the library (e.g. dstate > 16) */
    VS_ERR_HIP = -7,         /* the HIP runtime reported an error (see vs_last_error) */
    VS_ERR_WORKSPACE = -8    /* workspace missing or smaller than vs_workspace_bytes() */
};

/* operation kinds for vs_workspace_bytes */
enum { VS_OP_VIM_BIDIR = 0, VS_OP_CROSS4 = 1, VS_OP_1D = 2, VS_OP_VIM_GRAD = 3,
       VS_OP_VIM_SAVED = 4, VS_OP_VIM_GRAD_SAVED = 5 };

/* The delta_softplus argument of the scan entry points is a flags word.
 * VS_FLAG_SOFTPLUS: delta = softplus(delta_raw + dt_bias), else delta_raw +
 * dt_bias. VS_FLAG_ZOH: B_bar = (exp(delta A) - 1) / A * B, the exact
 * zero-order hold of "Discretization via Zero-Order Hold (ZOH)" (delta B
 * at A = 0), instead of the delta * B the guide's code uses. Other bits
 * return VS_ERR_UNSUPPORTED; the gradient takes VS_FLAG_SOFTPLUS only. */
#define VS_FLAG_SOFTPLUS 1
#define VS_FLAG_ZOH 2

/* Largest supported state size (the pages use 16 by default and 8 in a test). */
#define VS_MAX_DSTATE 16

/* Bytes of device workspace an operation needs (VS_OP_VIM_GRAD: the
 * gradient's forward output, per-block states, partial sums and the
 * per-workgroup dB/dC block sums, about 52 bytes per element;
 * VS_OP_VIM_SAVED: the saved-state buffer of vim_scan_bidir_fwd_saved, the
 * first two of those, about 12 bytes per element; VS_OP_VIM_GRAD_SAVED: the
 * workspace of vim_scan_bidir_grad_saved, the rest). Otherwise, in units of E =
 * batch*dim*seqlen elements. Direction merge: fp32 buffers of E floats,
 * one for VS_OP_VIM_BIDIR and two for VS_OP_CROSS4 (one per pair of opposite
 * directions); an fp32 y serves as the first, so fp32 needs one fewer.
 * VS_OP_CROSS4 also holds column-major copies of u and delta (2 E elements
 * of the input dtype) when the grid is too large to stage on chip: grids of
 * up to 256 tokens (fp32) or 512 (bf16) are copied to LDS by the scan
 * itself and need no copies. VS_OP_1D needs none. Returns 0 for invalid
 * arguments and for batch*dim*seqlen of 2^30 or more, which every entry
 * point refuses (VS_ERR_UNSUPPORTED). */
size_t vs_workspace_bytes(int op, int64_t batch, int64_t dim, int64_t seqlen, int dtype);

/*
 * Vision Mamba bidirectional scan (forward over tokens 0..L-1 and backward
 * over L-1..0), fused with softplus discretisation, the D skip, the merge
 * and the SiLU gate.
 *   batch, dim     >= 1; dstate in 1..16; seqlen >= 1 (L, tokens)
 *   u, delta, z    [batch][dim][L]; delta is the raw value before dt_bias and
 *                  softplus; z may be NULL (no gate)
 *   B, C           [batch][dstate][L], shared by both directions (token order)
 *   A              [2][dim][dstate] fp32, direction 0 = forward, 1 = backward
 *   Dskip, dt_bias [2][dim] fp32, or NULL for zeros
 *   delta_softplus flags: VS_FLAG_SOFTPLUS (delta = softplus(delta_raw +
 *                  dt_bias), else no softplus) | VS_FLAG_ZOH (exact hold)
 *   y              [batch][dim][L], written completely
 *   workspace      at least vs_workspace_bytes(VS_OP_VIM_BIDIR, ...) bytes
 *                  (may be NULL when that is 0); contents on entry are
 *                  ignored, contents on return are unspecified
 */
int vim_scan_bidir(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                   const void* u, const void* delta, const void* z, const void* B,
                   const void* C, const float* A, const float* Dskip, const float* dt_bias,
                   int delta_softplus, void* y, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * vim_scan_bidir with the sequence cut into `chunks` pieces that run in
 * parallel: the carry combine of a chunked scan. The inferensys glossary
 * "Vision Mamba (Vim)" (item "Parallel Scan Algorithm") and the guide's
 * "Production Engineering" section ("1. Compiling Fused CUDA Kernels") name a
 * parallel associative scan for the recurrence; since
 * h_t = exp(delta_t A) h_{t-1} + delta_t B_t u_t is linear in h, a run of
 * steps acts on the incoming state as h -> P h + h_0 with
 * P = prod_t exp(delta_t A) = exp(A sum_t delta_t) and h_0 its end state
 * from zero, and these pairs compose associatively:
 * (P1, h1) then (P2, h2) = (P1 P2, P2 h1 + h2). Each chunk first computes
 * the pairs of the tokens before it (forward) and after it (backward),
 * combines them into the states the two directions carry into the chunk,
 * and then scans its own tokens from those states.
 *   chunks         0: the library's choice (what vim_scan_bidir does: chunks
 *                  only when batch and dim give under 2 waves per SIMD);
 *                  1: one chunk; k >= 2: k chunks of whole 32-token tiles
 *                  (at most one per tile). Only VS_FLAG_SOFTPLUS may be set.
 *   everything else as for vim_scan_bidir (same workspace). The result is
 *   the same function of the inputs for every chunk count, up to fp32
 *   rounding of the carried states.
 * Returns VS_ERR_UNSUPPORTED for chunks > 1 with VS_FLAG_ZOH, VS_ERR_SHAPE
 * for chunks < 0.
 */
int vim_scan_bidir_chunked(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                           const void* u, const void* delta, const void* z, const void* B,
                           const void* C, const float* A, const float* Dskip, const float* dt_bias,
                           int delta_softplus, int chunks, void* y, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Largest batch*dim*seqlen that vim_scan_bidir_noalloc takes for bf16
 * activations: its library-owned merge buffer holds this many fp32 values
 * (128 MiB per GPU). fp32 activations need no buffer (y holds the partial
 * sums) and take any size the other entry points take. */
#define VS_NOALLOC_MAX_ELEMS (1 << 25)

/*
 * vim_scan_bidir for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, layouts and result as vim_scan_bidir, without the
 * workspace: the fp32 merge buffer is a static device array of the library
 * (VS_NOALLOC_MAX_ELEMS floats), allocated when the library's code object is
 * loaded on a GPU and held until the process ends. The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine). Each GPU has
 * its own copy of the buffer, which every call on that GPU shares and which
 * keeps the last call's contents (the scan needs no cleared buffer: every
 * entry is written before it is read). Calls that overlap in time on one GPU
 * (other streams, other host threads) race on the buffer: serialise them.
 * Returns VS_ERR_UNSUPPORTED when the activations are bf16 and
 * batch*dim*seqlen exceeds VS_NOALLOC_MAX_ELEMS, checked before any HIP call.
 */
int vim_scan_bidir_noalloc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                           const void* u, const void* delta, const void* z, const void* B,
                           const void* C, const float* A, const float* Dskip, const float* dt_bias,
                           int delta_softplus, void* y, void* stream);

/*
 * vim_scan_bidir with per-direction inputs. In the guide's block code
 * (section "1. PyTorch Implementation of the Bidirectional Vision Mamba
 * Block") each branch has its own conv1d and its own SimpleSelectiveSSM,
 * whose projections give that branch its own u, delta, B and C.
 *   u, delta       [2][batch][dim][L]: copy 0 feeds the forward direction,
 *                  copy 1 the backward one; token order in both
 *   B, C           [batch][2][dstate][L]: direction k's rows, token order
 *                  (the backward direction reads token L-1-t at step t)
 *   z              [batch][dim][L] or NULL: one gate on the merged output
 *   everything else as for vim_scan_bidir (same workspace). A caller that
 *   holds the backward branch in its own (flipped) order flips it first.
 * Returns VS_ERR_UNSUPPORTED when 2*batch*dim*L reaches 2^30.
 */
int vim_scan_bidir_dirs(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                        const void* u, const void* delta, const void* z, const void* B,
                        const void* C, const float* A, const float* Dskip, const float* dt_bias,
                        int delta_softplus, void* y, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * vim_scan_bidir with the Vim block's front end fused into the token loads:
 * each branch's scan input is u_k = silu(conv_k(x)), a depthwise Conv1d with
 * kernel 3, padding 1 and bias, applied to x in the forward branch and to
 * the flipped sequence in the backward branch (section "1. PyTorch
 * Implementation of the Bidirectional Vision Mamba Block": conv_f, conv_b and
 * the "Forward Branch" / "Backward Branch (Reverse sequence)" steps). Each
 * direction's D skip uses its own u_k; u is never written to memory.
 *   x              [batch][dim][L] (input dtype), takes the place of u
 *   conv_w         [2][dim][3] fp32: taps of direction k (0 forward,
 *                  1 backward) for channel d; in each branch's own order,
 *                  out[q] = b + w[0] in[q-1] + w[1] in[q] + w[2] in[q+1],
 *                  in[-1] = in[L] = 0 (PyTorch's Conv1d)
 *   conv_b         [2][dim] fp32, or NULL for zeros
 *   everything else as for vim_scan_bidir (same workspace).
 * Returns VS_ERR_NULL when conv_w is NULL.
 */
int vim_scan_bidir_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                        const void* x, const float* conv_w, const float* conv_b,
                        const void* delta, const void* z, const void* B, const void* C,
                        const float* A, const float* Dskip, const float* dt_bias,
                        int delta_softplus, void* y, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Gradient of vim_scan_bidir (reverse mode) for an upstream gradient dy of
 * y: the derivative of the definition at the top of this file with respect
 * to every input, differentiated step by step (the adjoint of the state,
 * lam_t = dy_t silu(z_t) C_t + e_{t+1} lam_{t+1}, runs backwards over each
 * direction's steps over states recomputed from the forward pass). It is
 * the backward half of a training step on the guide's Vim block (section
 * "2. The Bidirectional Mamba Block"); the pages themselves stop at the
 * forward pass.
 *   inputs         as for vim_scan_bidir (same layouts, dtype and meaning)
 *   dy             [batch][dim][L], dtype: dL/dy
 *   du, ddelta     [batch][dim][L], dtype: dL/du, dL/d delta_raw
 *   dz             [batch][dim][L], dtype; required when z is given, not
 *                  used (may be NULL) otherwise
 *   dB, dC         [batch][dstate][L] fp32, summed over channels and both
 *                  directions
 *   dA             [2][dim][dstate] fp32; dD, ddt_bias [2][dim] fp32 (summed
 *                  over batch rows); returned even when Dskip / dt_bias are
 *                  NULL (the gradient at 0)
 *   workspace      at least vs_workspace_bytes(VS_OP_VIM_GRAD, ...) bytes
 * Every output is overwritten, and is the same bit for bit on every call:
 * each per-token output has one writer, and the sums over channels and
 * batch rows are taken in a fixed order (no atomics). No output may overlap an input, another output or the
 * workspace (VS_ERR_ALIAS). Sequences longer than 2^26 tokens return
 * VS_ERR_UNSUPPORTED.
 */
int vim_scan_bidir_grad(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                        const void* u, const void* delta, const void* z, const void* B,
                        const void* C, const float* A, const float* Dskip, const float* dt_bias,
                        int delta_softplus, const void* dy, void* du, void* ddelta, void* dz,
                        float* dB, float* dC, float* dA, float* dD, float* ddt_bias,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * A training step's two halves with the backward's forward pass done once:
 * vim_scan_bidir_fwd_saved computes y exactly as vim_scan_bidir does (the
 * guide's section "2. The Bidirectional Mamba Block") and also writes what
 * the gradient needs from the forward pass into `saved`: the merged ungated
 * output y_f + y_b (fp32) and every recurrence's state at the start of each
 * 16-token block. vim_scan_bidir_grad_saved is vim_scan_bidir_grad reading
 * those instead of recomputing them; for the same inputs its outputs are
 * the same bit for bit.
 * vim_scan_bidir_fwd_saved:
 *   arguments      as for vim_scan_bidir; delta_softplus takes
 *                  VS_FLAG_SOFTPLUS only (the gradient's delta B form)
 *   saved          at least vs_workspace_bytes(VS_OP_VIM_SAVED, ...) bytes,
 *                  4-byte aligned; written completely, in a layout private to
 *                  the library; it must not overlap an input or y
 * vim_scan_bidir_grad_saved:
 *   arguments      as for vim_scan_bidir_grad
 *   saved          the buffer of a vim_scan_bidir_fwd_saved call on the same
 *                  u, delta, B, C, A, Dskip, dt_bias and flag, and the same
 *                  sizes (read only; not checked: other contents give
 *                  meaningless gradients); it must not overlap an output or
 *                  the workspace
 *   workspace      at least vs_workspace_bytes(VS_OP_VIM_GRAD_SAVED, ...) bytes
 * Both refuse sequences longer than 2^26 tokens (VS_ERR_UNSUPPORTED) and
 * return VS_ERR_WORKSPACE for a missing or short buffer.
 */
int vim_scan_bidir_fwd_saved(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                             const void* u, const void* delta, const void* z, const void* B,
                             const void* C, const float* A, const float* Dskip, const float* dt_bias,
                             int delta_softplus, void* y, void* saved, size_t saved_bytes, void* stream);
int vim_scan_bidir_grad_saved(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                              const void* u, const void* delta, const void* z, const void* B,
                              const void* C, const float* A, const float* Dskip, const float* dt_bias,
                              int delta_softplus, const void* saved, size_t saved_bytes, const void* dy,
                              void* du, void* ddelta, void* dz, float* dB, float* dC, float* dA, float* dD,
                              float* ddt_bias, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The linear maps around the scan, on the matrix cores (bf16 operands, fp32
 * accumulation, bf16 results). The guide's block code (section "1. PyTorch
 * Implementation of the Bidirectional Vision Mamba Block") builds them from
 * nn.Linear (out = in W^T + b); in the channel-major layout of the scan,
 * out[b][m][t] = sum_k W[m][k] in[b][k][t]. dtype must be VS_BF16 (VS_F32
 * returns VS_ERR_UNSUPPORTED). Tensors stay below 2^31 elements. Outputs
 * must not overlap inputs (VS_ERR_ALIAS) unless stated.
 */

/* SimpleSelectiveSSM.x_proj (Linear(d_model, 2 dstate + 1), no bias): the
 * projection's rows 0..N-1 are B, rows N..2N-1 are C and row 2N is dt (the
 * code's proj[..., :N], proj[..., N:2N], proj[..., 2N:]).
 *   u     [batch][dim][L] bf16 (the scan's input)
 *   W     [2 dstate + 1][dim] bf16 (nn.Linear's weight)
 *   B, C  [batch][dstate][L] bf16, ready for vim_scan_bidir
 *   dt    [batch][L] fp32 */
int vim_x_proj(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
               const void* u, const void* W, void* B, void* C, float* dt, void* stream);

/* dt_proj (Linear(1, d_model)) without its bias, which is the scan's
 * dt_bias (added inside the softplus): delta_raw[b][d][t] = w[d] dt[b][t].
 *   dt    [batch][L] fp32; w [dim] fp32 (the weight's only column)
 *   delta [batch][dim][L] bf16; dim at most 65535 */
int vim_dt_proj(int64_t batch, int64_t dim, int64_t seqlen, int dtype, const float* dt,
                const float* w, void* delta, void* stream);

/* The block's out_proj (Linear(d_model, d_model) in the guide; any shape
 * here) plus the residual:
 *   out[b][m][t] = sum_k W[m][k] y[b][k][t] + bias[m] + residual[b][m][t]
 *   y        [batch][dim_in][L] bf16; W [dim_out][dim_in] bf16
 *   bias     [dim_out] fp32 or NULL; residual [batch][dim_out][L] bf16 or NULL
 *   out      [batch][dim_out][L] bf16; it may be the residual itself
 *            (in place), but no other overlap is allowed */
int vim_out_proj(int64_t batch, int64_t dim_in, int64_t dim_out, int64_t seqlen, int dtype,
                 const void* y, const void* W, const float* bias, const void* residual, void* out,
                 void* stream);

/*
 * VMamba four-direction cross-scan of an H x W grid (L = H*W tokens, stored
 * row-major: token p = i*W + j). Direction 0 visits p = t, 1 visits
 * p = L-1-t, 2 visits the columns top to bottom, left to right
 * (p = (t mod H)*W + t div H), 3 is the reverse of 2. The four outputs are
 * summed, then gated by silu(z) when z is not NULL.
 *   u, delta, z, y [batch][dim][H][W]
 *   B, C           [batch][4][dstate][L]: direction k's B_t, C_t stored in
 *                  its own scan order (entry t is used at scan step t)
 *   A              [4][dim][dstate]; Dskip, dt_bias [4][dim] or NULL
 *   delta_softplus as for vim_scan_bidir; delta_raw is shared by the four
 *                  directions (spatial order), dt_bias is per direction
 *   workspace      at least vs_workspace_bytes(VS_OP_CROSS4, ...) bytes;
 *                  contents on entry are ignored, on return unspecified
 */
int vmamba_cross_scan4(int64_t batch, int64_t dim, int64_t dstate, int64_t H, int64_t W,
                       int dtype, const void* u, const void* delta, const void* z,
                       const void* B, const void* C, const float* A, const float* Dskip,
                       const float* dt_bias, int delta_softplus, void* y, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * One direction (reverse = 0: tokens 0..L-1; 1: L-1..0) with the optional
 * gate, no merge. Same layouts as vim_scan_bidir with A [dim][dstate] and
 * Dskip, dt_bias [dim] (or NULL). Needs no workspace.
 */
int s6_scan_1d(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
               int reverse, const void* u, const void* delta, const void* z, const void* B,
               const void* C, const float* A, const float* Dskip, const float* dt_bias,
               int delta_softplus, void* y, void* stream);

/* Static name of a status code ("VS_OK", ...). Never NULL. */
const char* vs_strerror(int status);

/* The calling thread's last detailed error message ("" if none). The string
 * stays valid until the thread's next call into the library. */
const char* vs_last_error(void);

/* VS_ABI_VERSION of the library. */
int vs_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VIMSCAN_H */
