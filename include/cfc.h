/*
 * cfc.h -- C ABI of libcfc_amd: a batched CfC (closed-form continuous-time)
 * recurrent cell K-loop for AMD Instinct MI355X (gfx950).
 *
 * Three calls make one training step of the cell's parameter gradient:
 *
 *   cfc_forward   x [B,K,n_in], h0 [B,H]           -> h_seq [B,K,H]
 *   cfc_backward  x, h0, h_seq, y [B,H]            -> scratch [B,N] (+ loss [B])
 *   reduce_axis0  scratch [B,N]                    -> out [N]
 *
 * cfc_forward_backward does the first two in one call (one launch where the
 * shape allows it).  cfc_backward_window runs the backward over a window of
 * steps; cfc_forward_backward_ws and cfc_backward_window_ws take a caller
 * workspace that lets accumulate mode at widths above 128 run the fast
 * 16-row backward; reduce_axis0_split is the reducer for narrow rows over a
 * long leading axis.
 *
 * The structure -- one independent chain per batch row, a per-batch gradient
 * scratch in which each row has a single writer and no atomics, and a
 * separate column-sum reducer that overwrites its output -- follows the
 * "K-loop Parallelization Implementation Plan" (foxhunt, 2026-05-17):
 * Task 1 (the reduce_axis0 kernel), Task 2 (the block-per-batch forward),
 * Task 3 (the block-per-batch backward writing per-batch scratch) and
 * Task 5 (scratch zeroed once per step, K invocations accumulate, reducer
 * before the optimizer).
 *
 * The cell (per unit i, elementwise), one of two:
 *   CFC_CELL_GATED (w_tau plays the per-unit role of the pages' tau[n_hid]):
 *     a      = W_in x_k + W_rec h_k + b
 *     g      = sigmoid(-softplus(w_tau) * a * dt)
 *     h_k+1  = g * h_k + (1 - g) * tanh(a)
 *   CFC_CELL_TAU_DECAY, the cell the pages print ("K-loop Parallelization
 *   Implementation Plan", Task 2 forward and Task 3 backward kernels; w_tau
 *   holds tau):
 *     g      = exp(-dt / max(tau, 1e-6))           (a per-unit constant)
 *     h_k+1  = g * h_k + (1 - g) * tanh(a)
 *     with dL/dtau = 0 where tau <= 1e-6 (the pages' guard)
 * and the loss of row b is  L_b = 1/2 |h_K - y_b|^2.
 *
 * Conventions shared by every call
 *  - All tensors are float32, dense, row-major, in DEVICE memory owned by the
 *    caller.  The library allocates nothing, never synchronises the device or
 *    the stream and never copies to the host: every call only validates its
 *    arguments on the host and enqueues kernels on `stream` (0 = the null
 *    stream), so the calls may be captured into a HIP graph.
 *  - Internal arithmetic of the cell and of the reducer is float64; inputs and
 *    outputs are float32 (each output is the float32 rounding of a float64
 *    value).
 *  - Outputs must not overlap any input or each other (checked on the host
 *    from the byte ranges the dimensions imply).
 *  - Identical inputs give bitwise-identical outputs: fixed summation orders,
 *    no atomics.
 *  - Argument errors are reported BEFORE anything is enqueued.  A launch
 *    failure is reported from hipGetLastError() without synchronising;
 *    errors raised later by the device surface at the caller's next sync.
 *  - Offsets are 64-bit: a scratch of more than 2^32 bytes is supported.
 */
#ifndef CFC_AMD_H
#define CFC_AMD_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define CFC_OK 0
#define CFC_ERR_NULL 1        /* a required pointer is NULL                          */
#define CFC_ERR_DIM 2         /* a dimension is out of range, or a size overflows     */
#define CFC_ERR_DT 3          /* dt is not finite                                     */
#define CFC_ERR_UNSUPPORTED 4 /* valid but beyond what the compiled kernels support   */
#define CFC_ERR_OVERLAP 5     /* an output range overlaps an input or another output  */
#define CFC_ERR_HIP 6         /* the HIP runtime rejected a launch                    */

/* cfc_backward flags. */
#define CFC_OVERWRITE 0  /* scratch[b,:] = this call's gradient (no prior memset needed) */
#define CFC_ACCUMULATE 1 /* scratch[b,:] += this call's gradient (caller zeroes first)   */

/* Compiled limits: n_in and n_hid up to 256; the backward also needs
 * K * (12 * n_hid + 4 * n_in) + 40 * n_hid + 2048 bytes of LDS <= 160 KiB,
 * e.g. K <= 76 at n_in = n_hid = 128 and K <= 37 at n_in = n_hid = 256
 * (cfc_backward_window takes longer K in windows within that bound).
 * The forward has no limit on K. */
#define CFC_MAX_N_IN 256
#define CFC_MAX_N_HID 256

/* Cell types (cfc_params_t.cell). */
#define CFC_CELL_GATED 0
#define CFC_CELL_TAU_DECAY 1

/* The cell's parameters, all device pointers:
 *   w_in  [n_hid, n_in]  row-major     w_rec [n_hid, n_hid] row-major
 *   b     [n_hid]                      w_tau [n_hid] (tau for CFC_CELL_TAU_DECAY)
 * and the cell type (any other value: CFC_ERR_UNSUPPORTED). */
typedef struct cfc_params {
    const float *w_in;
    const float *w_rec;
    const float *b;
    const float *w_tau;
    int n_in;
    int n_hid;
    int cell;
} cfc_params_t;

/* Length N of one per-batch gradient row:  N = n_hid * (n_in + n_hid + 2).
 * Row layout: [ dL/dW_in (n_hid x n_in, row-major) | dL/dW_rec (n_hid x n_hid,
 * row-major) | dL/db (n_hid) | dL/dw_tau (n_hid) ] -- the pages' four scratch
 * tensors (grad_w_in, grad_w_rec, grad_b, grad_tau; Task 4) laid end to end so
 * one reducer launch covers them all.  For CFC_CELL_TAU_DECAY the last slot
 * holds dL/dtau.  Returns -1 if a dimension is < 1 or
 * the product overflows. */
long long cfc_scratch_row_len(int n_in, int n_hid);

/* Forward K-loop ("K-loop Parallelization Implementation Plan", Task 2; here
 * the whole K-loop runs in one launch instead of one launch per k).
 *   params   cell parameters (see cfc_params_t); n_in, n_hid in [1, 256]
 *   x        [B, K, n_in]  inputs, row b, step k at x + (b*K + k)*n_in
 *   h0       [B, n_hid]    initial state
 *   dt       step length (finite; 0 allowed)
 *   B, K     batch rows >= 1, timesteps >= 1
 *   h_seq    [B, K, n_hid] OUTPUT: h_1 ... h_K of every row (h0 not repeated)
 * Returns a CFC_* status. */
int cfc_forward(const cfc_params_t *params, const float *x, const float *h0, float dt,
                int B, int K, float *h_seq, hipStream_t stream);

/* Backward through time of L = sum_b L_b ("K-loop Parallelization
 * Implementation Plan", Task 3: block-per-batch backward writing per-batch
 * scratch, single writer per row, no atomics).
 *   params, x, h0, dt, B, K   as for cfc_forward
 *   h_seq    [B, K, n_hid] the forward's output for the same inputs
 *   y        [B, n_hid]    targets
 *   scratch  [B, N] OUTPUT, N = cfc_scratch_row_len(n_in, n_hid):
 *            row b = dL_b / d(W_in, W_rec, b, w_tau) in the row layout above.
 *            flags = CFC_OVERWRITE: each row is written once with this call's
 *            gradient (equivalent to the pages' memset + K accumulating calls).
 *            flags = CFC_ACCUMULATE: each row is read and this call's gradient,
 *            rounded to float32, is added to it in float32 (scratch += g).
 *            At n_in or n_hid above 128 this entry has no workspace, so
 *            accumulate mode runs the general one-row-per-workgroup backward:
 *            about 8x slower than the 16-row kernel that
 *            cfc_backward_window_ws / cfc_forward_backward_ws run with a
 *            workspace (36.9 against 4.5 ms per step at B = 8192, K = 8,
 *            256/256).  The Python binding passes such a workspace itself.
 *   loss     [B] OUTPUT or NULL: L_b per row
 *   grad_x   [B, K, n_in] OUTPUT or NULL: dL/dx_k = W_in^T dL/da_k for every
 *            step (overwritten whatever the flags)
 *   grad_h0  [B, n_hid] OUTPUT or NULL: dL/dh_0, the gradient carried past
 *            step 0 (overwritten whatever the flags)
 *            These two are the pages' per-step grad_x and grad_h_old outputs
 *            (Task 3 kernel signature: overwrite, grad_x nullable) over the
 *            whole K-loop: each step's grad_h_old is the next step's carry,
 *            so only step 0's leaves the loop.  Requesting them does not
 *            change the other outputs.
 * Returns a CFC_* status; CFC_ERR_UNSUPPORTED if the LDS bound above fails. */
int cfc_backward(const cfc_params_t *params, const float *x, const float *h0,
                 const float *h_seq, const float *y, float dt, int B, int K,
                 float *scratch, float *loss, float *grad_x, float *grad_h0, int flags,
                 hipStream_t stream);

/* The backward over a window of steps [k_begin, k_end) of a K-step forward,
 * with the state gradient carried in and out -- for K beyond the backward's
 * LDS bound (which then applies to k_end - k_begin), or to feed an upstream
 * gradient dL/dh_K.  It generalises the pages' per-step backward ("K-loop
 * Parallelization Implementation Plan", Task 3: grad_h_new in, grad_h_old
 * out, parameter gradients accumulated into the scratch across the K calls
 * of Task 5) from one step to a window of steps.
 *   params, x, h0, h_seq, dt, B, K   as for cfc_backward (the whole forward)
 *   0 <= k_begin < k_end <= K
 *   delta_in  [B, n_hid] or NULL: dL/dh_k_end, the gradient flowing into the
 *             window's last state.  NULL seeds it from the loss instead:
 *             h_K - y, which needs k_end == K and y.
 *   y         [B, n_hid], read only when delta_in is NULL (may be NULL otherwise)
 *   scratch   [B, N]: this window's parameter gradient, CFC_OVERWRITE or
 *             CFC_ACCUMULATE (flags); running the windows from the last to the
 *             first, the first call overwriting and the others accumulating,
 *             gives cfc_backward's scratch up to float32 rounding (each call
 *             rounds once)
 *   loss      [B] or NULL: L_b, only in the seeded window (must be NULL when
 *             delta_in is given)
 *   grad_x    [B, K, n_in] or NULL: dL/dx_k for the window's steps (the rest
 *             of the array is not touched)
 *   delta_out [B, n_hid] or NULL: dL/dh_k_begin -- the next window's
 *             delta_in, or dL/dh_0 for k_begin = 0.  It may be the same buffer
 *             as delta_in (every element is read before it is written).
 * Windows of at most 64 steps at n_in, n_hid <= 128 (20 at wider shapes, in
 * overwrite mode, or in accumulate mode through cfc_backward_window_ws) run
 * the specialised kernels.
 * Returns a CFC_* status: CFC_ERR_DIM for a bad window, a missing seed or a
 * loss without one; CFC_ERR_UNSUPPORTED if the window exceeds the LDS bound. */
int cfc_backward_window(const cfc_params_t *params, const float *x, const float *h0,
                        const float *h_seq, const float *y, const float *delta_in, float dt,
                        int B, int K, int k_begin, int k_end, float *scratch, float *loss,
                        float *grad_x, float *delta_out, int flags, hipStream_t stream);

/* Bytes of device workspace that cfc_backward_window_ws needs for a window of
 * Kw steps: 8 * B * Kw * n_hid (dL/da of every row-step, float64) where the
 * window runs the 16-row backward in accumulate mode (n_in or n_hid above
 * 128, Kw <= 20, flags = CFC_ACCUMULATE); 0 where no kernel uses one.  The
 * same size serves cfc_forward_backward_ws for B rows of K = Kw steps.
 * Returns -1 for a non-positive size, unknown flags or overflow. */
long long cfc_backward_workspace(int B, int Kw, int n_in, int n_hid, int flags);

/* Bytes of device workspace for cfc_forward_backward_ws to run at its best:
 * cfc_backward_workspace(B, K, n_in, n_hid, flags), plus 1 MiB at exactly
 * 256 x 256 with K <= 8 in accumulate mode, where the call then also keeps a
 * float64 copy of W_in and W_rec there (the forward and the reverse pass read
 * it instead of converting the float32 weights; same results, bitwise).  A
 * workspace of only cfc_backward_workspace bytes is still accepted there.
 * Returns -1 for a non-positive size, unknown flags or overflow. */
long long cfc_forward_backward_workspace(int B, int K, int n_in, int n_hid, int flags);

/* cfc_backward_window with a caller-owned device workspace.  The pages' form
 * of the backward adds each call's gradient into the scratch ("K-loop
 * Parallelization Implementation Plan", Task 5: scratch zeroed once, the K
 * calls accumulate); at widths above 128 the 16-row backward keeps dL/da of
 * the window's steps in its rows' scratch tails until the weight gradients are
 * formed, which accumulate mode cannot do, since the old values there are
 * still needed.  With a workspace it parks dL/da there instead, so
 * accumulating windows of at most 20 steps at these widths run the 16-row
 * kernel rather than the general one-row-per-workgroup backward.
 *   arguments 1-16  as for cfc_backward_window
 *   workspace        device memory, 8-byte aligned, or NULL (then the call is
 *                    cfc_backward_window); contents on entry are ignored and
 *                    on return unspecified; it must not overlap any other
 *                    argument while it is in use (CFC_ERR_OVERLAP)
 *   workspace_bytes  its size; below cfc_backward_workspace(B, k_end -
 *                    k_begin, n_in, n_hid, flags), or a misaligned workspace,
 *                    is CFC_ERR_DIM when the window would use it
 * Outputs are the same as cfc_backward_window's for the same arguments up to
 * the summation order of the kernel that runs (the 16-row kernel's overwrite
 * and accumulate modes compute the same float32 gradient, bitwise).  The
 * workspace is ignored where the window does not use it (overwrite mode, or
 * n_in, n_hid <= 128, or more than 20 steps at the wider shapes).  A window
 * over the whole sequence, seeded from y, at exactly 256 x 256 with K <= 8
 * (x, h0, h_seq and the scratch 16-byte aligned) runs as two launches: the
 * reverse pass, which leaves dL/da in the workspace and adds dL/dw_tau to the
 * scratch, then the weight gradients and db, added on the vector units. */
int cfc_backward_window_ws(const cfc_params_t *params, const float *x, const float *h0,
                           const float *h_seq, const float *y, const float *delta_in, float dt,
                           int B, int K, int k_begin, int k_end, float *scratch, float *loss,
                           float *grad_x, float *delta_out, int flags, void *workspace,
                           long long workspace_bytes, hipStream_t stream);

/* cfc_forward followed by cfc_backward on the same inputs, in one call
 * ("K-loop Parallelization Implementation Plan", Tasks 2 and 3 back to back):
 *   params, x, h0, dt, B, K   as for cfc_forward
 *   y, scratch, loss, grad_x, grad_h0, flags   as for cfc_backward
 *   h_seq    [B, K, n_hid] OUTPUT, as cfc_forward writes it
 * For n_in, n_hid <= 128 and K <= 64 this is ONE kernel per row that keeps the
 * forward's float64 pre-activations and the staged [x_k | h_k-1] on chip for
 * the reverse pass instead of recomputing them from the float32 h_seq.  The
 * reverse pass then uses the unrounded pre-activations (the separate backward
 * recomputes them from float32 h); every other input of the backward
 * (h_K - y, h_k-1 in the gradients) is the float32 value written to h_seq.
 * Wider shapes with K <= 20 in overwrite mode (N even, scratch 8-byte
 * aligned) run three launches on `stream`: a forward that also parks its
 * float64 pre-activations in the head of each scratch row, then a backward in
 * two stages (the reverse pass, then the weight gradients) that reads them back
 * instead of recomputing them.  At exactly 256 x 256 with B >= 4 and a
 * 16-byte-aligned scratch, a fourth, first launch copies the weights to
 * float64 into scratch rows 0..3 for the forward and the reverse pass.  The
 * scratch thus serves as the call's temporary storage; every element holds
 * its gradient when the call's work completes.  Other shapes run cfc_forward and cfc_backward
 * as two launches on `stream`.  In both cases the backward's limits are checked
 * first, so nothing is enqueued when either direction would be refused.
 * Returns a CFC_* status; the same argument rules as the two calls, and no
 * output (h_seq, scratch, loss, grad_x, grad_h0) may overlap another. */
int cfc_forward_backward(const cfc_params_t *params, const float *x, const float *h0,
                         const float *y, float dt, int B, int K, float *h_seq, float *scratch,
                         float *loss, float *grad_x, float *grad_h0, int flags,
                         hipStream_t stream);

/* cfc_forward_backward with a caller-owned device workspace, for accumulate
 * mode at widths above 128 (the pages' scratch += of "K-loop Parallelization
 * Implementation Plan", Task 5): with K <= 20 the backward then runs the
 * 16-row kernel, parking dL/da in the workspace, as cfc_backward_window_ws
 * does; otherwise the call is cfc_forward_backward and the workspace is
 * ignored.  At exactly 256 x 256 with K <= 8 (weights, x, h0, h_seq and the
 * scratch 16-byte aligned) it is three launches, as in overwrite mode: the
 * forward parks its float64 pre-activations in the workspace, the reverse
 * pass reads them back, leaves dL/da there and adds dL/dw_tau to the scratch,
 * and the last launch adds the weight gradients and db; with a 16-byte-aligned
 * workspace of cfc_forward_backward_workspace bytes a fourth, first launch
 * copies the weights to float64 there, as overwrite mode does in the scratch.  The gradient added is
 * then the one cfc_forward_backward writes in overwrite mode, bitwise (rounded
 * to float32, then added in float32); the other shapes add the gradient of
 * cfc_forward followed by cfc_backward.
 *   arguments 1-13   as for cfc_forward_backward
 *   workspace        device memory, 8-byte aligned, or NULL; contents on entry
 *                    ignored, on return unspecified
 *   workspace_bytes  at least cfc_backward_workspace(B, K, n_in, n_hid, flags)
 *                    where it is used (else CFC_ERR_DIM);
 *                    cfc_forward_backward_workspace(...) bytes let the
 *                    256 x 256 accumulate path keep its float64 weight copy
 *                    there too (the range checked for overlap is then that
 *                    size).  A workspace that overlaps another argument is
 *                    CFC_ERR_OVERLAP.  Both are checked before the forward is
 *                    enqueued. */
int cfc_forward_backward_ws(const cfc_params_t *params, const float *x, const float *h0,
                            const float *y, float dt, int B, int K, float *h_seq, float *scratch,
                            float *loss, float *grad_x, float *grad_h0, int flags,
                            void *workspace, long long workspace_bytes, hipStream_t stream);

/* Column sum ("K-loop Parallelization Implementation Plan", Task 1):
 *   out[j] = sum_{b < B} per_batch[b, j]   for j < N, OVERWRITING out.
 * Float64 accumulation in a fixed order (no atomics), one float32 rounding.
 *   per_batch [B, N] float32, B >= 0, N >= 0 (B = 0 writes zeros; N = 0 is a
 *             no-op that enqueues nothing)
 *   out       [N] OUTPUT
 * Returns a CFC_* status (CFC_ERR_DIM if B*N*4 overflows). */
int reduce_axis0(const float *per_batch, long long B, long long N, float *out,
                 hipStream_t stream);

/* Bytes of workspace reduce_axis0_split needs for a [B, N] input: 0 when it
 * runs the one-pass reduce_axis0 instead (N > 256, or too few rows to split),
 * -1 if B or N is negative or B*N*4 overflows. */
long long reduce_axis0_split_workspace(long long B, long long N);

/* Column sum for narrow rows over a long leading axis -- e.g. N = 3 columns
 * over B = 524288 rows, the pages' bias-gradient reduce ("Custom Kernel
 * Optimization Implementation Plan", Tasks 4-5: batch-parallel partial sums,
 * then a final reduce of the partials).  reduce_axis0 gives such a shape a
 * single workgroup; here up to 1024 workgroups each sum a chunk of rows into
 * float64 partials in `workspace`, and one more sums the partials, both in a
 * fixed order that depends only on (B, N).
 *   per_batch, B, N, out   as for reduce_axis0 (out is overwritten)
 *   workspace  device memory of at least reduce_axis0_split_workspace(B, N)
 *              bytes, 8-byte aligned, owned by the caller, not overlapping
 *              per_batch or out; its contents on entry are ignored and on
 *              return are unspecified.  May be NULL when that size is 0.
 * The result is the float32 rounding of a float64 sum, bitwise reproducible
 * for a given (B, N); its grouping differs from reduce_axis0's, so the two
 * may differ in the last float32 bit.
 * Returns a CFC_* status: CFC_ERR_DIM also when the workspace is too small
 * or misaligned. */
int reduce_axis0_split(const float *per_batch, long long B, long long N, float *out,
                       void *workspace, long long workspace_bytes, hipStream_t stream);

/* Maximum bytes of partials reduce_axis0_split ever needs (256 K float64
 * partials); reduce_axis0_split_noalloc keeps them in a static device array of
 * this size. */
#define CFC_SPLIT_STATIC_BYTES (2LL * 1024 * 1024)

/* reduce_axis0_split for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result (bitwise) as reduce_axis0_split, without the
 * workspace: the float64 partials go to a static device array of
 * CFC_SPLIT_STATIC_BYTES that the library holds on each GPU it runs on until
 * the process ends.  Nothing is allocated, freed or copied to the host; phase 1
 * writes every partial that phase 2 reads, so the array needs no clearing.
 *   - The first call on a device resolves the array's address on that device
 *     (hipGetSymbolAddress, with the device current); make that first call
 *     outside a graph capture.  A failure there is CFC_ERR_HIP.
 *   - Every call on one GPU uses the same array: calls that may overlap on one
 *     GPU (concurrent streams, several host threads) race and must be
 *     serialised by the caller, e.g. by issuing them on one stream.
 *   - A shape whose partials would exceed the array is CFC_ERR_UNSUPPORTED
 *     (the split plan never needs more, so this is a guard).
 * Returns a CFC_* status, as reduce_axis0_split. */
int reduce_axis0_split_noalloc(const float *per_batch, long long B, long long N, float *out,
                               hipStream_t stream);

/* Static text for a status code (never NULL). */
const char *cfc_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* CFC_AMD_H */
