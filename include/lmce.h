/*
 * lmce.h -- fused LM-head + cross-entropy (NLL) loss for AMD MI355X (gfx950).
 *
 * The operation (TRL docs "Training Beyond 1M Tokens", section "The loss is
 * the first thing to break"): the last hidden state h (L x H) is multiplied
 * by the LM-head weight W (V x H) to give logits z = h W^T (L x V), and the
 * loss is the cross entropy of z against the target labels.  Section "The
 * massive logits matrix: chunk it" of the same page computes it a block of
 * rows at a time so that the L x V logits are never held whole; rows split
 * cleanly because each row's softmax runs over its own vocabulary only.
 *
 * This library goes further than row chunks: no array of logits is ever
 * allocated or written whole.  In the plain forward each fp32 logit tile
 * exists only in registers while a kernel folds it into a running per-row
 * log-sum-exp.  The group-scheduled passes (the backward, and the training
 * forward) turn each tile into bf16 probabilities or G in registers and hand
 * it to the other workgroups of their group through a fixed exchange ring in
 * the workspace (at most 128 MiB), where it lives for the one round that
 * consumes it: over a pass every logit crosses that ring once as 2 bytes,
 * L x V x 2 bytes in all, but never more than the ring at a time.
 *
 *   lse_i  = log sum_v exp(z_iv)                       every row i
 *   loss   = sum_{i : y_i != ignore_index} (lse_i - z_{i,y_i}) / N
 *   G_iv   = g / N * [y_i != ignore_index] * (softmax(z_i)_v - [v == y_i])
 *   dh     = G W        (L x H)
 *   dW     = G^T h      (V x H)
 *
 * N is the number of rows whose label is not ignore_index, g the upstream
 * gradient of the scalar loss.  N == 0 gives loss = NaN and zero gradients.
 *
 * Conventions for every entry point:
 *   - h and W are bf16, row-major and contiguous: h[i*H + k], W[v*H + k]
 *     (W has the nn.Linear weight layout).  labels are int64 [L], already
 *     shifted (labels[i] is the target of row i).  All outputs are fp32.
 *   - Every pointer is a DEVICE pointer owned by the caller.  h, W, dh_out
 *     and dW_out must be 16-byte aligned, labels 8-byte, workspace 256-byte,
 *     the fp32 scalars and lse 4-byte; otherwise LMCE_ERR_NULL.
 *     The library keeps no pointer after a call returns.
 *   - Every call only enqueues work on `stream` and returns; it never
 *     allocates device memory and never synchronises (except
 *     lmce_read_status, which is documented as synchronising).
 *   - The caller supplies a workspace of at least lmce_workspace_size()
 *     bytes.  Calls that share a workspace must be ordered on one stream.
 *   - The group-scheduled passes (lmce_fwd_train, lmce_bwd_train, lmce_bwd,
 *     lmce_bwd_dh, lmce_bwd_dW) launch one cooperative grid sized to the
 *     whole device; running two of them at once on one device (other
 *     streams or processes) is not supported.  Every group wait is bounded,
 *     so members that cannot all be resident end the call with LMCE_ERR_HIP
 *     from lmce_read_status rather than a hang.
 *   - Return value: LMCE_OK (0) or a negative lmce_status.  Argument errors
 *     are detected before anything is enqueued.
 *   - Limits: 1 <= L <= 2^21, 1 <= V <= 2^21, 128 <= H <= 16384 with
 *     H % 128 == 0, chunk_rows a multiple of 32 in [32, 1024].
 */
#ifndef LMCE_H
#define LMCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMCE_OK = 0,
  LMCE_ERR_NULL = -1,        /* a required pointer is NULL or misaligned */
  LMCE_ERR_SHAPE = -2,       /* L, H or V out of range */
  LMCE_ERR_UNSUPPORTED = -3, /* H % 128 != 0, chunk_rows not a multiple of 32 in [32, 1024], or the device cannot run the grid */
  LMCE_ERR_WORKSPACE = -4,   /* workspace_bytes smaller than lmce_workspace_size() */
  LMCE_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed */
  LMCE_ERR_LABEL = -6,       /* (asynchronous) a label is outside [0, V) and not ignore_index */
  LMCE_ERR_STATE = -7,       /* (asynchronous) lmce_bwd_train without a preceding lmce_fwd_train on the workspace */
  LMCE_ERR_SCRATCH = -8      /* lmce_fwd_noalloc: the shape needs more than its fixed area holds */
} lmce_status;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lmce_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char* lmce_strerror(int status);

/*
 * Bytes of device workspace that lmce_fwd / lmce_bwd and the training pair
 * need for this shape: per-row partials and orders (O(L) words), a fixed
 * exchange ring for the group passes (at most 128 MiB), where H % 256 == 0
 * and H >= 1024 a parking area for their accumulators (at most 64 MiB), and
 * the dW pass's partial slices (at most 64 MiB).  h and W are read in place,
 * never copied or transposed; the passes that skip unlabelled rows read h's
 * rows through their order, except where H < 1024 or H % 256 != 0 or
 * L * H * 2 > 2^31 bytes: there the workspace also holds a gathered bf16
 * copy of those rows (L * H * 2 bytes).  It never holds an L x V array.
 * Writes the size to *bytes.  Returns LMCE_OK or a shape error.
 */
int lmce_workspace_size(int64_t L, int64_t H, int64_t V, int64_t chunk_rows, size_t* bytes);

/*
 * Forward.  Page: TRL docs "Training Beyond 1M Tokens", sections "The loss is
 * the first thing to break" (the definition) and "The massive logits matrix:
 * chunk it" (row chunks of chunk_rows rows, 256 by default; the pieces are
 * summed).
 *
 *   h        bf16 [L, H]   hidden states
 *   W        bf16 [V, H]   LM-head weight
 *   labels   int64 [L]     target of each row, or ignore_index
 *   loss_out fp32 [1]      mean NLL over non-ignored rows (NaN if none, or if
 *                          a label was out of range)
 *   lse_out  fp32 [L]      log-sum-exp of every row's logits (ignored rows too)
 *
 * chunk_rows only shapes the schedule (rows whose vocabulary sweep is run as
 * one unit); results do not depend on it.
 * An out-of-range label is reported asynchronously: loss_out becomes NaN and
 * lmce_read_status() returns LMCE_ERR_LABEL.
 */
int lmce_fwd(const void* h, const void* W, const int64_t* labels,
             int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
             float* loss_out, float* lse_out,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * lmce_fwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments (minus the workspace), same kernels
 * and bitwise the same loss_out and lse_out as lmce_fwd.
 *
 * Instead of a workspace it uses a fixed area of device memory that the
 * library holds: 65 MiB per device, reserved on each device where the
 * library's kernels are loaded and held until the process ends.  That area
 * has room for shapes with L <= 2^20 rows (any V and H within the limits
 * above); larger L returns LMCE_ERR_SCRATCH before anything is enqueued.
 * The call allocates nothing and synchronises nothing.
 *
 * All calls on one device share its area: calls that may overlap in time on
 * one device (other streams, other threads) race and must be serialised by
 * the caller.  Each call clears the area's header first, so the previous
 * call's contents never reach the results.  A bad label makes loss_out NaN;
 * there is no workspace for lmce_read_status here.
 */
int lmce_fwd_noalloc(const void* h, const void* W, const int64_t* labels,
                     int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
                     float* loss_out, float* lse_out, void* stream);

/*
 * Backward.  Same page and sections; the gradient of the mean NLL is
 * G = g/N * valid * (softmax - onehot).  Each logit tile is recomputed from
 * h and W, turned into bf16 G' = valid * (softmax - onehot) and contracted
 * in the same round into
 *   dh_out fp32 [L, H] = g/N * G' W     (overwritten, not accumulated)
 *   dW_out fp32 [V, H] = g/N * G'^T h   (overwritten, not accumulated)
 * by the co-resident workgroups that own the 128- or 256-wide H slices of
 * the outputs; g/N multiplies the fp32 results, so that its own rounding
 * does not scale every term alike, and a G' tile lives only in the
 * workspace's exchange ring for the one round that consumes it.  The device must support cooperative launches
 * (otherwise LMCE_ERR_HIP or LMCE_ERR_UNSUPPORTED).
 *
 *   lse        fp32 [L]  the lse_out of lmce_fwd on the same inputs
 *   grad_loss  fp32 [1]  device scalar g, the upstream gradient of the loss
 * Other arguments as in lmce_fwd.  Ignored rows get exactly zero dh rows.
 */
int lmce_bwd(const void* h, const void* W, const int64_t* labels, const float* lse,
             int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
             const float* grad_loss, float* dh_out, float* dW_out,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of lmce_bwd, for callers that need only one gradient (a
 * frozen LM head needs dh alone; a frozen trunk needs dW alone).  Same
 * arguments and results as lmce_bwd for the gradient they produce; calling
 * both equals one lmce_bwd.
 */
int lmce_bwd_dh(const void* h, const void* W, const int64_t* labels, const float* lse,
                int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
                const float* grad_loss, float* dh_out,
                void* workspace, size_t workspace_bytes, void* stream);
int lmce_bwd_dW(const void* h, const void* W, const int64_t* labels, const float* lse,
                int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
                const float* grad_loss, float* dW_out,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training pair.  Same page and sections, same results as lmce_fwd followed
 * by lmce_bwd, with less work: the forward's single vocabulary sweep also
 * accumulates O_i = sum_v softmax(z_i)_v W_v with a running-maximum rescale
 * (the gradient of the mean NLL is dh_i = g/N * valid_i * (O_i - W_{y_i})),
 * and writes O (fp32 [L, H]) into the caller's dh_out.  lmce_bwd_train then
 * forms dh in place in that buffer without recomputing any logit, and runs
 * the dW pass.  Between the two calls the buffer holds O, not dh.
 *
 * lmce_fwd_train: arguments and outputs as lmce_fwd, plus dh_out (fp32
 *   [L, H], 16-byte aligned), which receives O.
 * lmce_bwd_train: arguments and outputs as lmce_bwd; dh_out must be the
 *   buffer the preceding lmce_fwd_train wrote O into, on the same inputs,
 *   workspace and stream, with no other lmce_fwd or lmce_fwd_train on the
 *   workspace in between; otherwise dh_out is NaN and lmce_read_status()
 *   returns LMCE_ERR_STATE.  Calls of lmce_bwd, lmce_bwd_dh or lmce_bwd_dW
 *   on the workspace in between, with any inputs, are allowed: they leave
 *   the training forward's state alone.
 */
int lmce_fwd_train(const void* h, const void* W, const int64_t* labels,
                   int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
                   float* loss_out, float* lse_out, float* dh_out,
                   void* workspace, size_t workspace_bytes, void* stream);
int lmce_bwd_train(const void* h, const void* W, const int64_t* labels, const float* lse,
                   int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
                   const float* grad_loss, float* dh_out, float* dW_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * The pages' own chunked formulation, as a comparison path (TRL docs
 * "Training Beyond 1M Tokens", section "The massive logits matrix: chunk
 * it": a few hundred rows at a time, 256 in TRL, each chunk's logits formed,
 * its loss taken and the pieces summed; the backward walks the chunks again,
 * each adding its share of dW).  Same definition and results (within
 * rounding) as lmce_fwd / lmce_bwd, but each chunk's logits ARE written to
 * the workspace as fp32 [chunk_rows][V] (148 MiB at 256 x 151936) and read
 * back, and dW is accumulated in memory once per chunk.
 *
 *   lmce_chunked_workspace_size: bytes for this shape: the chunk's logits,
 *     its bf16 G, dh partials of the chunk, per-row nll (O(L) floats); W and
 *     the chunk's rows of h are read in place.
 *   lmce_chunked_fwd: loss_out and lse_out as lmce_fwd.
 *   lmce_chunked_bwd: dh_out and dW_out as lmce_bwd (overwritten); it
 *     recomputes every chunk's logits and their lse, as autograd over a
 *     checkpointed chunk would, so it takes no lse argument.
 * chunk_rows is 1 .. 4096 (any value); H % 128 == 0; other limits, pointer
 * rules, status reporting (lmce_read_status on this workspace) as above.
 */
int lmce_chunked_workspace_size(int64_t L, int64_t H, int64_t V, int64_t chunk_rows, size_t* bytes);
int lmce_chunked_fwd(const void* h, const void* W, const int64_t* labels,
                     int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
                     float* loss_out, float* lse_out,
                     void* workspace, size_t workspace_bytes, void* stream);
int lmce_chunked_bwd(const void* h, const void* W, const int64_t* labels,
                     int64_t L, int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_rows,
                     const float* grad_loss, float* dh_out, float* dW_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sequence-tiled MLP block (TRL docs "Training Beyond 1M Tokens", section
 * "One GPU is not enough: split the sequence across many": the line
 * down_proj(act_fn(gate_proj(x)) * up_proj(x)) builds four tensors at the
 * full intermediate width; TRL PR #6845 lists MLP sequence tiling as the
 * lever that removes them).  act_fn = SiLU.  The rows are processed
 * chunk_rows at a time, so those four intermediates exist (in bf16) for one
 * chunk only:
 *   y   = (silu(x Wg^T) * (x Wu^T)) Wd^T
 *   dx, dWg, dWu, dWd: the gradients for an upstream dy of y.
 *
 *   x   bf16 [L, H]   Wg, Wu  bf16 [I, H] (gate_proj, up_proj weights)
 *   Wd  bf16 [H, I]   (down_proj weight)     dy  bf16 [L, H]
 *   y_out, dx_out fp32 [L, H]; dWg_out, dWu_out fp32 [I, H]; dWd_out fp32
 *   [H, I]; every output overwritten.
 * The backward recomputes each chunk's gate and up projections (the forward
 * keeps nothing of them) and takes no forward state: it may run on its own.
 * Limits: 128 <= H <= 16384 with H % 128 == 0, 64 <= I <= 65536 with
 * I % 64 == 0, 1 <= L <= 2^24, 1 <= chunk_rows <= 65536, and 4 I H and
 * 4 I ceil(c / 64) 64 at most 2^31 - 4096, c = min(chunk_rows, L)
 * (LMCE_ERR_UNSUPPORTED otherwise).  The workspace holds the packed gate/up
 * weights (2 I H bf16) and one chunk's intermediates (its gate/up values, p
 * and their gradients); lmce_mlp_workspace_size gives its size.  Pointer
 * rules as above; there is no asynchronous status.
 */
int lmce_mlp_workspace_size(int64_t L, int64_t H, int64_t I, int64_t chunk_rows, size_t* bytes);
int lmce_mlp_fwd(const void* x, const void* Wg, const void* Wu, const void* Wd,
                 int64_t L, int64_t H, int64_t I, int64_t chunk_rows, float* y_out,
                 void* workspace, size_t workspace_bytes, void* stream);
int lmce_mlp_bwd(const void* x, const void* Wg, const void* Wu, const void* Wd, const void* dy,
                 int64_t L, int64_t H, int64_t I, int64_t chunk_rows,
                 float* dx_out, float* dWg_out, float* dWu_out, float* dWd_out,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Synchronises `stream` and returns the asynchronous status recorded in the
 * workspace by every call on it since the previous lmce_read_status (the
 * flags of the calls accumulate; a later call never erases an earlier
 * call's error), then clears those flags:
 *   LMCE_ERR_LABEL  a label was outside [0, V) and not ignore_index;
 *   LMCE_ERR_HIP    the synchronisation failed, or a group-scheduled
 *                   workgroup gave up waiting for the other members of its
 *                   group (a bounded wait; that call's results are then
 *                   incomplete: its loss is NaN, and after such an
 *                   lmce_fwd_train the following lmce_bwd_train writes a NaN
 *                   dh);
 *   LMCE_ERR_STATE  an lmce_bwd_train found no complete training forward;
 *   LMCE_OK         none of these.
 * With several flags set, the first in this list is returned.  A workspace
 * on which no call has run reads LMCE_OK.  Not to be called while other
 * calls on the workspace are in flight on another stream.
 */
int lmce_read_status(void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LMCE_H */
