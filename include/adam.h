/*
 * adam.h - C ABI of libadamw_mi355x.so, the fused multi-tensor Adam / AdamW
 * parameter update for AMD Instinct MI355X (gfx950).
 *
 * The update is the one defined by the apex patch "Enhance Distributed Fused
 * Adam (#1794)" (multi_tensor_distopt_adam_kernel.cu hunk,
 * DistAdamCapturableFunctor::local_step and operator()), with the step and
 * flag rules of apex distributed_fused_adam.py (step(), _local_step,
 * _local_step_with_param_remainders, _bf16_rem_to_fp32) and the empty-group
 * counter rule of TransformerEngine PR "Advance FusedAdam step counter for
 * empty param groups" (section "Fix").  For every element, with t the step
 * after its increment, s the grad scale, wd the weight decay:
 *
 *   x   = g*s            (AdamW, mode 1)   or  g*s + wd*p   (L2, mode 0)
 *   m'  = beta1*m + (1-beta1)*x
 *   v'  = beta2*v + (1-beta2)*x*x
 *   u   = (m'/bc1) / (sqrt(v'/bc2) + eps)        [+ wd*p in mode 1]
 *   p'  = p - lr*u
 *
 * with bc1 = 1-beta1^t, bc2 = 1-beta2^t when bias_correction is 1, else 1.
 * All arithmetic is IEEE binary32, rounded to nearest-even, in the order
 * written (no fused multiply-add), with correctly rounded division and
 * square root and fp32 denormals kept.  beta^t is computed from the float
 * beta in double by binary exponentiation and 1-beta^t is rounded once to
 * float.  The library therefore reproduces a scalar C evaluation of these
 * expressions bit for bit.
 *
 * The param and moment type T may be float, bf16 or fp16 (the functor takes
 * it from the param list; apex passes its optimizer-state dtype): for a
 * 16-bit T, p, m and v are widened to float (exactly), updated as above, and
 * stored rounded to T (nearest even); the param-out copy is the cast of the
 * new stored param.  Two more storage schemes around the same fp32 update:
 *   - remainders (apex _bf16_rem_to_fp32): bf16 params plus int16 low halves
 *     hold the fp32 master exactly;
 *   - scaled 16-bit state (apex distributed_fused_adam.py,
 *     _local_step_with_scaled_states and _apply_state_scale): p, m and v are
 *     stored as bf16 or fp16 values times a per-tensor fp32 scale each; the
 *     step unscales them to fp32, updates, and stores them again with new
 *     scales taken from each buffer's largest magnitude.
 *
 * Conventions for every call below:
 *   - Pointers marked "device" point to GPU memory on the device that was
 *     current when the handle was built; "host" pointers to CPU memory.
 *   - Calls return 0 (ADAM_OK) or a negative adam_status; they never throw
 *     and never abort.  Argument errors are found before anything is
 *     enqueued and before any counter changes.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs
 *     asynchronously; faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - bf16 buffers hold raw bfloat16 bit patterns (uint16_t); fp16 buffers
 *     hold IEEE binary16 bit patterns.  Casts from fp32 round to nearest
 *     even (fp16: overflow to infinity, subnormals kept); NaN stays NaN.
 */
#ifndef ADAMW_MI355X_ADAM_H
#define ADAMW_MI355X_ADAM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADAM_ABI_VERSION 6

typedef enum {
    ADAM_OK = 0,
    ADAM_EINVAL = -1, /* bad argument (null pointer, size, flag value, overlap) */
    ADAM_EDTYPE = -2, /* dtype combination the library does not implement     */
    ADAM_ENOMEM = -3, /* device or host allocation failed                     */
    ADAM_EHIP = -4,   /* a HIP runtime call or kernel launch failed           */
    ADAM_ETOOBIG = -5 /* adam_step_noalloc: the list needs more work-table
                         records than its static scratch holds (65536)       */
} adam_status;

typedef enum {
    ADAM_DT_NONE = 0, /* buffer absent (p_out only) */
    ADAM_DT_F32 = 1,
    ADAM_DT_BF16 = 2,
    ADAM_DT_F16 = 3
} adam_dtype;

/* One tensor of a group: five (six with remainders) flat, dense arrays of
 * `numel` elements each.  p, m, v (and rem) are read and updated in place;
 * g is only read; p_out is only written.  The layout is the apex tensor-list
 * order [p, m, v, g, p_out] (remainder mode: [p, rem, m, v, g, p_out]). */
typedef struct {
    void *p;          /* device: the handle's p dtype: float, bf16 or fp16 (bf16
                         bits in remainder mode)                                  */
    int16_t *rem;     /* device: int16 remainders (remainder mode), else NULL      */
    void *m;          /* device: first moment: float, or p's 16-bit type (16-bit
                         or scaled state)                                         */
    void *v;          /* device: second moment: as m                               */
    const void *g;    /* device: gradient: float, bf16 or fp16 bits                */
    void *p_out;      /* device: float, bf16 or fp16 copy of the new param, or NULL */
    float *scales;    /* device: scaled state only: float[3] = the scales of p, m,
                         v (stored value x scale = fp32 value), read and replaced
                         by each step; NULL otherwise                             */
    int64_t numel;    /* >= 0; a tensor with numel == 0 may have NULL pointers     */
} adam_tensor;

/* The dtypes shared by every tensor of one handle, and the work-table
 * granularity. */
typedef struct {
    adam_dtype p;            /* ADAM_DT_F32, ADAM_DT_BF16 or ADAM_DT_F16 (a
                                16-bit p means 16-bit m and v too); BF16 with
                                remainders; BF16 or F16 with scaled state      */
    adam_dtype g;            /* ADAM_DT_F32, ADAM_DT_BF16 or ADAM_DT_F16         */
    adam_dtype p_out;        /* ADAM_DT_NONE, ADAM_DT_F32, ADAM_DT_BF16 or
                                ADAM_DT_F16 (remainders: NONE or BF16; scaled
                                state: not F32)                                 */
    int32_t with_remainders; /* 1: p is bf16 and rem holds the low fp32 halves  */
    int64_t chunk_elems;     /* elements per work-table record: 0 = automatic
                                (the largest power of two <= 65536 that wastes
                                under 1% of workgroups on ragged tensor ends);
                                else a power of two from 1024 to 2^30.  Results
                                do not depend on it.                           */
    int32_t scaled_state;    /* 1: p, m, v are p's 16-bit type with per-tensor
                                scales (adam_tensor.scales); 0: no             */
    int32_t dispatch_tiles;  /* tiles (512 elements each) per kernel dispatch of
                                the streaming passes: 0 = the most one dispatch
                                can carry (2^25 - 512: a dispatch counts its
                                work-items in 32 bits); else a positive limit,
                                capped at that.  Longer lists are launched as
                                several dispatches over consecutive tiles.
                                One-pass scaled state runs one persistent
                                dispatch; a nonzero value caps its workgroups
                                at dispatch_tiles / 8.  Results do not depend
                                on it.                                         */
    int32_t scaled_passes;   /* scaled state: 0 or 2 = two passes, 1 = one pass
                                (see adam_step_scaled; ADAM_EINVAL if the list
                                does not allow it); must be 0 otherwise.
                                Results do not depend on it.                   */
    int32_t scaled_wait_us;  /* one-pass scaled state: how long a workgroup
                                waits for the rest of its tensor before it
                                leaves its stores to the follow-up pass:
                                0 = 200 us, > 0 = that many us, -1 = no wait
                                (every tile is stored by the follow-up
                                pass).  Results do not depend on it.          */
} adam_tl_desc;

/* Per-group hyperparameters (apex defaults: betas (0.9, 0.999), eps 1e-8,
 * weight decay 0, AdamW mode, bias correction on). */
typedef struct {
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    int32_t mode;            /* 0 = L2 (decay in the gradient), 1 = AdamW       */
    int32_t bias_correction; /* 1 = divide by 1-beta^t, 0 = do not              */
} adam_hparams;

/* What a handle (or a plan) contains. */
typedef struct {
    int64_t tensors;         /* tensors passed in                                 */
    int64_t nonempty;        /* tensors with numel > 0                            */
    int64_t chunks;          /* work-table records                                */
    int64_t elements;        /* sum of numel                                      */
    int64_t chunk_elems;     /* elements per record                               */
    int64_t vector_tensors;  /* tensors whose buffers all allow 4-element vectors */
    int64_t grid_blocks;     /* tiles: workgroups of the update kernel per step,
                                over all its dispatches                          */
    int32_t tile_elems;      /* elements per workgroup (one tile)                 */
    int32_t block_threads;   /* threads per workgroup of the update (the scaled-
                                state maxima pass runs one 64-lane wave per tile) */
    int32_t bytes_per_elem;  /* algorithmic HBM bytes per element (read + write)  */
    int32_t device;          /* HIP device of the handle (-1 from adam_tl_plan)   */
    int32_t two_buffer;      /* 1: built by adam_tl_build_two_buffer               */
    int32_t pieces;          /* scaled state: pieces of consecutive tensors the
                                step is pipelined in over the caller's stream
                                and a second stream of the handle (see
                                adam_step_scaled): for a list of two or more
                                tensors whose work table holds at least 8192
                                tiles (about 4M elements), up to 16 pieces of
                                about equal tiles, cut at tensor boundaries,
                                each of at least 1024 tiles (512K elements);
                                1 otherwise                                     */
    int32_t dispatch_tiles;  /* tiles per kernel dispatch (adam_tl_desc)         */
    int32_t dispatches;      /* dispatches of the update kernel per step (scaled
                                state: of each of its two passes, summed over
                                the pieces; one pass: of the one-pass kernel)  */
    int32_t scaled_passes;   /* scaled state: 1 (one pass) or 2; 0 otherwise    */
} adam_tl_stats;

typedef struct adam_tl adam_tl; /* opaque handle: device work table */

/* ABI version of the loaded library (ADAM_ABI_VERSION).  This library's own
 * (the pages' interface is a Python extension module). */
int adam_abi_version(void);

/* Static text for a status code (never NULL).  This library's own: the
 * pages' launcher reports errors through TORCH_CHECK and C10_CUDA_CHECK
 * (apex patch "Enhance Distributed Fused Adam (#1794)",
 * multi_tensor_fused_adam_capturable_cuda); here every call returns a code. */
const char *adam_status_string(int status);

/* Validates a tensor list and computes its work table on the host only (no
 * HIP call, no device allocation); fills *stats (device = -1).  The list is
 * the one the pages hand to multi_tensor_applier (apex
 * distributed_fused_adam.py, _local_step: list(zip(*group_buffers)) of
 * [param, exp_avg, exp_avg_sq, grad, param-sync] per bucket); the dtype sets
 * are those of the DISPATCH_FLOAT_HALF_AND_BFLOAT over T, GRAD_T and
 * PARAM_OUT_T in the patch's multi_tensor_fused_adam_capturable_cuda, plus
 * the remainder and scaled-state schemes of distributed_fused_adam.py
 * (_check_params_shard_dtypes, _local_step_with_param_remainders,
 * _local_step_with_scaled_states).
 * Errors: ADAM_EINVAL for a NULL desc/stats, count < 0, NULL `tensors` with
 * count > 0, numel < 0, a NULL required pointer in a non-empty tensor, a
 * pointer given where the dtype says none, a bad chunk_elems, dispatch_tiles < 0,
 * with_remainders or scaled_state not 0/1 or both 1, or two buffers that
 * overlap (gradients may overlap other gradients; no other pair may share a
 * byte; a tensor's scales are written too); ADAM_EDTYPE for an unsupported
 * dtype set.  Supported sets (g F32|BF16|F16 in each):
 *   - fp32 state: p F32 (m, v float), p_out NONE|F32|BF16|F16;
 *   - 16-bit state: p BF16|F16 (m, v the same type), p_out NONE|F32|BF16|F16;
 *   - remainders: p BF16, p_out NONE|BF16 (apex: bf16 params need fp32
 *     optimizer state for the remainder scheme; p_out is the new bf16);
 *   - scaled state: p BF16|F16 (m and v the same type), p_out NONE|BF16|F16
 *     (apex: the param-sync buffer is a 16-bit type). */
int adam_tl_plan(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                 adam_tl_stats *stats);

/* Builds a handle for one group.  The pages rebuild a chunk table at every
 * launch: multi_tensor_apply<5> in the patch's
 * multi_tensor_fused_adam_capturable_cuda fills TensorListMetadata, and the
 * functor's operator() finds its (tensor, chunk) through
 * tl.block_to_tensor[blockIdx.x] and tl.block_to_chunk[blockIdx.x] (apex
 * patch "Enhance Distributed Fused Adam (#1794)",
 * DistAdamCapturableFunctor::operator()).  This library computes the
 * equivalent table once per list, for the life of the handle: validates as
 * adam_tl_plan, then copies the work table (one 128-byte record per chunk, plus a 64-byte scalar block used
 * by the capturable steps, partial-sum scratch for adam_grad_sumsq, and for
 * scaled state 12 bytes of maxima per 512-element tile and 24 bytes of maxima
 * and reciprocal scales per tensor) to the current device,
 * using `stream`, and waits for that copy.  `tensors` (host array of `count`) is
 * not retained; the device buffers it names must stay allocated and in place
 * for the handle's life.  On success *out owns device memory; release it with
 * adam_tl_destroy.  A list whose elements sum to 0 gives a valid handle that
 * holds no device memory.  Errors: as adam_tl_plan; ADAM_ENOMEM; ADAM_EHIP. */
int adam_tl_build(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                  hipStream_t stream, adam_tl **out);

/* Two-buffer state.  The apex patch "Enhance Distributed Fused Adam
 * (#1794)" (DistAdamCapturableFunctor::operator()) reads and writes p, m and
 * v in place; the same values can go to a second set of buffers instead.  In
 * place, every written line is one the step has just read, and on MI355X
 * that read-modify-write of the same lines costs about 5% of the HBM rate.
 * Where p, m, v are the optimizer's own state (the fp32 master shards of
 * apex distributed_fused_adam.py, whose model sees only the param-sync copy
 * p_out), they may live in two buffer sets and alternate:
 *   - `alternates` (host array of `count`, parallel to `tensors`) gives each
 *     tensor's second set: p, m, v (and rem in remainder mode) with the same
 *     numel; g, p_out and scales must be NULL (they are not alternated).
 *     Each second-set pointer must lie a multiple of 128 bytes away from its
 *     first-set pointer, and no buffer of either set may overlap another.
 *   - The state lives in set (t & 1), t the group's step counter (host
 *     step_io, or the device d_step of the capturable calls): set 0 before
 *     the first step.  A step with counter t reads set ((t - 1) & 1) and
 *     writes set (t & 1); it leaves the set it read unchanged (it then holds
 *     the state before the step).  A noop step moves neither the counter
 *     nor the state.  Because the capturable calls take the set from the
 *     device counter, a recorded graph replays correctly.
 *   - The caller must not change the counter other than through the step
 *     calls, or must move the state to set (t & 1) itself.
 * Storage schemes: fp32 state, 16-bit state and remainders (the scaled
 * state's two passes stay in place: ADAM_EINVAL).  Everything else is as
 * adam_tl_plan / adam_tl_build; the step, norm and clip calls are the same
 * for both kinds of handle.  ADAM_EINVAL also for NULL `alternates` with
 * count > 0 or an entry that breaks the rules above. */
int adam_tl_plan_two_buffer(const adam_tensor *tensors, const adam_tensor *alternates, int64_t count,
                            const adam_tl_desc *desc, adam_tl_stats *stats);
int adam_tl_build_two_buffer(const adam_tensor *tensors, const adam_tensor *alternates, int64_t count,
                             const adam_tl_desc *desc, hipStream_t stream, adam_tl **out);

/* Frees a handle (NULL is allowed).  Work enqueued with it must be finished.
 * This library's own (the handle has no counterpart on the pages). */
void adam_tl_destroy(adam_tl *tl);

/* Copies a handle's statistics to *stats (host). ADAM_EINVAL on NULL.  This
 * library's own. */
int adam_tl_info(const adam_tl *tl, adam_tl_stats *stats);

/* Non-capturable step on a handle with fp32 or 16-bit state (no remainders,
 * no scales): apex distributed_fused_adam.py, _local_step with capturable
 * off (multi_tensor_fused_adam, the DistAdamFunctor whose name the patch's
 * hunk header shows; its body is not on the pages, and the update is read as
 * DistAdamCapturableFunctor::local_step with host scalars), after step()
 * advances the counter (self.state["step"] += 1).
 *   lr          host value.
 *   step_io     host int32 counter: incremented first (the first update uses
 *               t = 1), also when the handle has no elements.  ADAM_EINVAL if
 *               it is INT32_MAX or below 0 (the counter would not give t >= 1).
 *   grad_scale  host multiplier of the gradient, used when d_grad_scale is
 *               NULL; d_grad_scale (device float, nullable) is read on the
 *               device instead (apex passes its grad scale as a device
 *               tensor).
 * On ADAM_EHIP the counter is restored if nothing of the step had been
 * enqueued; if a later launch of the step failed, the counter keeps the new
 * value and the buffers may hold a partly applied step.  Errors: ADAM_EINVAL
 * (NULL tl/hp/step_io, mode not 0/1, bias_correction not 0/1, a remainder
 * or scaled-state handle). */
int adam_step(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io,
              float grad_scale, const float *d_grad_scale, hipStream_t stream);

/* Capturable step on a handle with fp32 or 16-bit state: apex patch
 * "Enhance Distributed Fused Adam (#1794)", DistAdamCapturableFunctor::
 * operator() (returns when *noop_gmem == 1; reads *lr, *step and
 * *grad_scale_ptr on the device) and distributed_fused_adam.py step() with
 * capturable on (the counter advances by (_dummy_overflow_buf != 1); the
 * functor sees the advanced counter).  Every per-step scalar lives in device
 * memory, nothing is allocated, nothing is read back,
 * and the host never waits, so the call can be recorded into a HIP graph and
 * replayed.
 *   d_lr          device float.
 *   d_step        device int32 counter; advanced by one on the device after
 *                 the update, unless *d_noop == 1 (int32 wrap-around).
 *   d_grad_scale  device float, nullable (NULL = 1.0).
 *   d_noop        device int32 flag, nullable (NULL = never skip).  When
 *                 *d_noop == 1 no buffer and not the counter is written; any
 *                 other value runs the step.
 * The call enqueues a one-lane prologue (resolves these scalars and advances
 * the counter) and then the update, which reads the resolved scalars from
 * the handle's scalar block; capturable steps of one handle must therefore
 * be ordered (one stream, or synchronised streams).
 * Errors: ADAM_EINVAL (NULL tl/hp/d_lr/d_step, bad mode/flag, a remainder
 * or scaled-state handle); ADAM_EHIP (if the prologue was enqueued before a
 * launch failed, the device counter advances and the buffers may hold a
 * partly applied step). */
int adam_step_capturable(const adam_tl *tl, const adam_hparams *hp, const float *d_lr,
                         int32_t *d_step, const float *d_grad_scale, const int32_t *d_noop,
                         hipStream_t stream);

/* Non-capturable step on a remainder handle (bf16 params + int16
 * remainders, fp32 m and v): apex distributed_fused_adam.py,
 * _local_step_with_param_remainders (multi_tensor_fused_adam_with_param_
 * remainders, whose functor the patch names but does not show) and
 * _bf16_rem_to_fp32.  Each element's fp32 master is rebuilt from its
 * bf16 bits and remainder as apex's _bf16_rem_to_fp32 defines, updated as
 * above, and stored back in the same encoding (remainder = low 16 bits of the
 * fp32 word; bf16 = high 16 bits, plus one when that remainder is negative
 * as an int16, mod 2^16: a round to nearest with ties away from zero).
 * p_out, if present, receives the new bf16 param bits.  Arguments and errors
 * as adam_step; ADAM_EINVAL for a handle that is not in remainder mode. */
int adam_step_remainders(const adam_tl *tl, const adam_hparams *hp, float lr,
                         int32_t *step_io, float grad_scale, const float *d_grad_scale,
                         hipStream_t stream);

/* Capturable step on a remainder handle: the arithmetic and encoding of
 * adam_step_remainders with the device scalars, noop flag and counter rules
 * of adam_step_capturable.  An extension of this library: apex
 * distributed_fused_adam.py's constructor refuses store_param_remainders
 * with capturable ("doesn't support CUDA graph yet"); nothing in the update
 * needs host scalars, so both are offered.  Errors as adam_step_capturable;
 * ADAM_EINVAL for a handle that is not in remainder mode. */
int adam_step_remainders_capturable(const adam_tl *tl, const adam_hparams *hp, const float *d_lr,
                                    int32_t *d_step, const float *d_grad_scale,
                                    const int32_t *d_noop, hipStream_t stream);

/* Non-capturable step on a scaled-state handle (apex distributed_fused_adam.py
 * _local_step_with_scaled_states, _apply_state_scale and
 * _check_params_shard_dtypes).  Per tensor, with S = scales[0..2] and T the
 * state type (bf16 or fp16):
 *   P = float(p) * S[0],  M = float(m) * S[1],  V = float(v) * S[2]
 *   (P, M, V) <- the fp32 update above, with lr, counter and grad scale as
 *                in adam_step
 *   p_out     = P cast to p_out's type (param-sync copy), if present
 *   for (X, x, k) in (P, p, 0), (M, m, 1), (V, v, 2):
 *     amax = max |X| over the tensor (NaN if any element is NaN)
 *     S[k] = amax / L,   L = half the largest finite T (bf16 ~1.69e38,
 *                        fp16 32752), a correctly rounded float division
 *     r    = S[k] > 0 ? 1/S[k] : 0   (correctly rounded)
 *     x    = T(X * r)                (float product, then round to nearest even)
 * Note: with bf16 state a tensor whose largest magnitude is below about 0.5
 * gets a subnormal scale whose reciprocal overflows, so its values store as
 * +-inf (0 becomes NaN) -- the pages' formula does this; fp16 state does not.
 * Empty tensors keep their scales.  Per piece of the list (adam_tl_stats.
 * pieces) the call enqueues four kernels: a pass that computes each tile's
 * maxima of the updated buffers, a fold of those maxima per tensor, a pass
 * that recomputes the update and stores it, a per-tensor kernel that writes
 * the new scales (each pass as adam_tl_stats.dispatch_tiles allows).  With
 * two or more pieces they alternate between `stream` and a second stream the
 * handle owns, so that one piece's store pass runs beside the next piece's
 * maxima pass: the call records an event on `stream` that the second stream
 * waits for, events between the pieces, and a last event on the second
 * stream that `stream` waits for, so all of the step is ordered after the
 * work enqueued on `stream` before the call and before the work enqueued
 * on it after.  Under stream capture the same calls record that fork and
 * join into the graph.  The events and the second stream belong to the
 * handle (the call uses them through the const handle): steps of one handle
 * must be ordered (one stream, or synchronised streams), and one handle
 * must not be captured into two graphs that run at the same time.
 * One pass (adam_tl_desc.scaled_passes = 1): a persistent kernel whose
 * workgroups each update a 4096-element tile exactly, publish its maxima,
 * and store it once the last workgroup of its tensor has published the
 * tensor's scales (each input is read once, where two passes read it
 * twice); a follow-up kernel stores any tile whose bounded wait ran out
 * (adam_tl_desc.scaled_wait_us), and a per-tensor kernel writes the new
 * scales.  Same results bit for bit.  It needs every tensor within 2M
 * elements and 4-element accesses.  On MI355X it takes 7-10% less time
 * than two passes.  It relies on its grid being resident: each workgroup
 * counts itself in when it starts, and while not all have (other kernels
 * holding compute units), a wait ends after 20 us and leaves the tile to
 * the follow-up kernel, so the step still finishes and stays exact.  Two
 * passes depend on nothing being resident and are the default.
 * Arguments and errors as adam_step; ADAM_EINVAL for a handle without
 * scaled state. */
int adam_step_scaled(const adam_tl *tl, const adam_hparams *hp, float lr, int32_t *step_io,
                     float grad_scale, const float *d_grad_scale, hipStream_t stream);

/* Capturable step on a scaled-state handle: the arithmetic, maxima and new
 * scales of adam_step_scaled with the device scalars, noop flag and counter
 * rules of adam_step_capturable (apex refuses scaled state with its
 * capturable option; the per-tensor fold runs on the device between the two
 * passes, so nothing needs the host).  A noop step (*d_noop == 1) writes no
 * buffer, no scale and not the counter.  Errors as adam_step_capturable;
 * ADAM_EINVAL for a handle without scaled state. */
int adam_step_scaled_capturable(const adam_tl *tl, const adam_hparams *hp, const float *d_lr,
                                int32_t *d_step, const float *d_grad_scale, const int32_t *d_noop,
                                hipStream_t stream);

/* For callers that cannot allocate device memory (harnesses that forbid
 * hipMalloc, loops that must not allocate): adam_step without a handle.  The
 * call validates and plans `tensors` (host array of `count`) as
 * adam_tl_build does, copies the work table into a static device array of
 * the library (65,536 records of 128 bytes, 8 MiB, held on every device the
 * library runs on until the process ends) with an asynchronous copy on
 * `stream`, waits on the host for that copy (and so for the work enqueued
 * on `stream` before it), and enqueues the update.  It calls no device
 * allocation routine.
 *   - Storage: fp32 or 16-bit state (desc as for adam_tl_build; remainders
 *     and scaled state: ADAM_EINVAL).  With chunk_elems 0 the chunk is the
 *     automatic one, doubled until the table fits; a list that needs more
 *     than 65,536 records at the largest chunk (2^30 elements), or at the
 *     chunk the caller fixed, is refused with ADAM_ETOOBIG before anything
 *     runs (in practice: more than 65,536 non-empty tensors).
 *   - lr, step_io, grad_scale, d_grad_scale, errors and the counter rules:
 *     as adam_step.  The results equal adam_step's on a handle of the same
 *     list, bit for bit.
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's table: calls that overlap on one device (two streams, two
 *     host threads) race; order them.  The call is not capturable (the host
 *     waits for the copy). */
int adam_step_noalloc(const adam_tensor *tensors, int64_t count, const adam_tl_desc *desc,
                      const adam_hparams *hp, float lr, int32_t *step_io, float grad_scale,
                      const float *d_grad_scale, hipStream_t stream);

/* Sum of squares of every gradient element of a handle (apex
 * distributed_fused_adam.py, grad_norm: multi_tensor_l2norm over the grad
 * shards, then the square summed and all-reduced): the local part of
 * the global gradient norm that apex's distributed_fused_adam.py computes in
 * grad_norm (per-bucket L2 norms of the gradient shards, squared and summed,
 * then all-reduced across ranks).  Each square of a float, bf16 or fp16 gradient is
 * exact in double; the sum is accumulated in double with a fixed order of
 * additions, so repeated calls give identical bits.
 *   d_sumsq     device double: *d_sumsq = (accumulate ? *d_sumsq : 0) + sum.
 *               Calls for several groups chain with accumulate = 1.
 *   accumulate  0 or 1.
 * Non-finite gradients make the sum inf or NaN.  No allocation, no host wait
 * (capturable).  Uses the handle's partial-sum scratch: calls on one handle
 * must be ordered, like capturable steps.  Errors: ADAM_EINVAL (NULL tl or
 * d_sumsq, accumulate not 0/1); ADAM_EHIP. */
int adam_grad_sumsq(const adam_tl *tl, double *d_sumsq, int32_t accumulate, hipStream_t stream);

/* The clip / found-inf step from a gradient sum of squares (apex
 * distributed_fused_adam.py: grad_norm scales the raw norm by the grad
 * scale; clip_grad_norm multiplies the grad scale by
 * min(1, max_norm / (norm + 1e-6)); step() takes found_inf = the norm is not
 * finite and, when capturable, copies it into the noop flag).  One device
 * lane computes, in float:
 *   norm      = float(sqrt(*d_sumsq)) * grad_scale   (grad_scale = *d_grad_scale, or 1 if NULL)
 *   found_inf = norm is inf or NaN
 *   *d_norm   = norm                                  (d_norm nullable)
 *   *d_noop   = found_inf ? 1 : 0                     (d_noop nullable; overwritten)
 *   if !found_inf and max_norm > 0:
 *     *d_grad_scale = grad_scale * min(1, max_norm / (norm + 1e-6))
 * With found_inf the grad scale is left as it is (the step will be skipped).
 * max_norm <= 0 disables clipping.  No allocation, no host wait (capturable).
 * Errors: ADAM_EINVAL (NULL d_sumsq, NaN max_norm, max_norm > 0 with a NULL
 * d_grad_scale); ADAM_EHIP. */
int adam_clip_grad_scale(const double *d_sumsq, float *d_grad_scale, float max_norm, float *d_norm,
                         int32_t *d_noop, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ADAMW_MI355X_ADAM_H */
