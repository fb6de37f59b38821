/*
 * mambamix.h -- C ABI of libmambamix, the data-parallel core of the Mamba
 * selective state-space mixer on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (per sequence s, token position p, channel c):
 *
 *   window   = [the K-1 previous raw inputs of channel c, x[p,c]]   (newest last)
 *   u        = SiLU(conv_b[c] + sum_k conv_w[c,k] * window[k])
 *   delta    = softplus(dt[p,c] + dt_bias[c])
 *   A[c,n]   = -exp(A_log[c,n])
 *   h[c,n]   = exp(delta * A[c,n]) * h[c,n] + delta * B[p,n] * u
 *   y[p,c]   = (sum_n C[p,n] * h[c,n] + D[c] * u) * SiLU(z[p,c])
 *
 * This is the one-token step of the Mamba mixer as the TensorRT Mamba
 * tensor-parallel builder spells it out (NVIDIA TensorRT-Model-Connect,
 * families/mamba/tp_builder.py, _add_mamba_tp_layer: the conv window is the
 * state's newest columns with x appended; softplus of the biased dt;
 * A_bar = exp(dt * A); the state update; the readout from the updated state
 * plus D * u; the SiLU(z) gate), applied token after token.  The input and
 * output projections, the normalisation and the all-reduces around it are not
 * part of this library.
 *
 * Packed variable-length sequences (PackMamba page, abstract): a prefill call
 * takes S sequences laid end to end in one token stream, delimited by
 * cu_seqlens; no state passes from one sequence to the next.  The state cache
 * (tensor-parallel SSM page, abstract and Fig. 2 component (1)): sequence s
 * starts from slot s of conv_state / ssm_state and leaves its final state
 * there, so a later prefill call (a further chunk) or a decode step continues
 * it.  A zeroed slot is a fresh sequence.
 *
 * Conventions shared by every entry point
 *  - All pointers are DEVICE pointers except where stated.  Arrays are
 *    row-major with the last index contiguous.
 *  - "io" arrays (x, z, dt, B, C, y) hold MM_IO_F32 (float) or MM_IO_BF16
 *    (bfloat16 bit patterns, 2 bytes) elements; parameters and states are
 *    always float32.  bf16 outputs are rounded to nearest even.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *    null stream).  The library allocates no memory and keeps no caller
 *    pointer; its one piece of global state is the per-device address of the
 *    fixed scratch behind mamba_mixer_prefill_noalloc.  Calls on different
 *    streams may run concurrently provided their output buffers (and, for
 *    mamba_mixer_prefill_noalloc, their device) do not overlap.
 *  - The caller owns every buffer.  The states are read as the initial state
 *    and overwritten in place with the final state.
 *  - Return value: MM_OK (0) or a negative MM_ERR_* code.  Argument errors are
 *    detected on the host before anything is enqueued, and nothing is written
 *    then.  MM_ERR_HIP reports a failed kernel launch.
 *  - Preconditions NOT checked (checking would need a device sync):
 *    cu_seqlens[0] == 0, cu_seqlens non-decreasing, cu_seqlens[S] == T.
 *    Violating them is undefined behaviour (the kernels may read and write outside
 *    the arrays).  mamba_mixer_check_cu_seqlens checks a host copy of the array.
 */
#ifndef MAMBAMIX_H
#define MAMBAMIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MM_OK               0
#define MM_ERR_NULL        -1  /* a required pointer is NULL                                  */
#define MM_ERR_DIM         -2  /* a negative size, T > INT32_MAX, S == 0 with T > 0, too few events,
                                  an array of more than MM_MAX_ROWS_X_D rows x channels        */
#define MM_ERR_UNSUPPORTED -3  /* K != 4, N outside 1..16, unknown io dtype or engine, d too large */
#define MM_ERR_ALIGN       -4  /* a pointer not aligned to its element size                    */
#define MM_ERR_WORKSPACE   -5  /* workspace smaller than the size query returns (or NULL)      */
#define MM_ERR_ALIAS       -6  /* y overlaps an input, or conv_state overlaps ssm_state         */
#define MM_ERR_HIP         -7  /* a kernel launch failed                                        */

/* io element types */
#define MM_IO_F32  0
#define MM_IO_BF16 1

/* limits of this build */
#define MM_MAX_N 16
#define MM_CONV_K 4
/* Largest rows x channels of any array (tokens x d, sequences x d, batch x d): 2^36, far more
 * than one GPU's memory holds, and small enough that every byte extent fits in 64 bits. */
#define MM_MAX_ROWS_X_D (1ull << 36)

/*
 * mamba_mixer_prefill -- run the mixer over S packed sequences.
 *
 *   x, z, dt      [T, d]      io     token inputs: SSM-path input (pre-conv), gate input,
 *                                    and the dt-projection output before dt_bias
 *   B, C          [T, N]      io     input and readout vectors, shared by all channels
 *   A_log         [d, N]      f32    A = -exp(A_log)
 *   D, dt_bias    [d]         f32
 *   conv_w        [d, K]      f32    conv_w[c, K-1] weights the current token
 *   conv_b        [d]         f32
 *   cu_seqlens    [S+1]       int32  sequence s is tokens cu_seqlens[s] .. cu_seqlens[s+1]-1
 *   conv_state    [S, d, K-1] f32    in/out: the K-1 newest raw inputs x, oldest first
 *   ssm_state     [S, d, N]   f32    in/out: the SSM state h
 *   y             [T, d]      io     out
 *   workspace     device scratch of at least mamba_mixer_prefill_workspace_bytes(S,T,d,N,K)
 *                 bytes, 256-byte aligned; its contents on entry do not matter.
 *
 * An empty sequence (cu_seqlens[s] == cu_seqlens[s+1]) leaves slot s unchanged.
 * A sequence shorter than K-1 tokens keeps the older entries of its conv state
 * (they shift towards the front).  T == 0 or d == 0 is a successful no-op.
 */
int mamba_mixer_prefill(const void* x, const void* z, const void* dt, const void* B, const void* C,
                        const float* A_log, const float* D, const float* dt_bias,
                        const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                        float* conv_state, float* ssm_state, void* y,
                        int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mamba_mixer_prefill needs for these sizes (0 is possible).  Host only. */
size_t mamba_mixer_prefill_workspace_bytes(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K);

/*
 * mamba_mixer_prefill_noalloc -- mamba_mixer_prefill for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid it): the same
 * computation, plan and kernels, with no workspace argument.  The carries of a chunked plan go
 * to a fixed scratch array in the library's device code, MM_NOALLOC_SCRATCH_BYTES per GPU, which
 * each GPU the library runs on holds until the process ends.  The call allocates and frees
 * nothing.
 *   Arguments, layouts and results: those of mamba_mixer_prefill.
 *   A plan whose workspace (mamba_mixer_prefill_workspace_bytes) exceeds
 *   MM_NOALLOC_SCRATCH_BYTES is MM_ERR_WORKSPACE, returned before anything is enqueued.
 *   The scratch is found for the current device (hipGetDevice) on the first call that needs it
 *   there; `stream` must belong to that device.  MM_ERR_HIP if it cannot be resolved.
 *   Every call on one GPU uses the same scratch, and nothing in it needs to start at any value:
 *   calls that may overlap on one GPU (concurrent streams, or threads) race on it and must be
 *   serialised by the caller; calls ordered on one stream are safe.
 */
#define MM_NOALLOC_SCRATCH_BYTES (32u << 20)
int mamba_mixer_prefill_noalloc(const void* x, const void* z, const void* dt, const void* B, const void* C,
                                const float* A_log, const float* D, const float* dt_bias,
                                const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                                float* conv_state, float* ssm_state, void* y,
                                int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                                void* stream);

/* Prefill engines (see mamba_mixer_prefill_ex). */
#define MM_ENGINE_AUTO 0  /* the library picks from S, T and d                                        */
#define MM_ENGINE_LANE 1  /* one lane per channel, all N state entries of it in registers             */
#define MM_ENGINE_ROW  2  /* one channel per 16-lane row, one state entry per lane (for few sequences) */
/* The row engine (also behind mamba_mixer_prefill_train and mamba_mixer_prefill_backward)
 * takes d <= MM_ROW_MAX_D: with a larger d an explicit MM_ENGINE_ROW, the training forward
 * and the backward return MM_ERR_UNSUPPORTED, and MM_ENGINE_AUTO uses the lane engine. */
#define MM_ROW_MAX_D 4194304

/*
 * mamba_mixer_prefill_chunked -- mamba_mixer_prefill with an explicit time-chunk
 * length.  Each sequence is cut into chunks of `chunk_len` tokens (the last one
 * shorter) that are processed in parallel and stitched with the associative
 * combine of the recurrence; chunk_len <= 0 picks the length mamba_mixer_prefill
 * uses.  The result does not depend on chunk_len beyond floating-point rounding.
 * The workspace size for a given chunk_len comes from
 * mamba_mixer_prefill_workspace_bytes_chunked.
 */
int mamba_mixer_prefill_chunked(const void* x, const void* z, const void* dt, const void* B, const void* C,
                                const float* A_log, const float* D, const float* dt_bias,
                                const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                                float* conv_state, float* ssm_state, void* y,
                                int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                                int64_t chunk_len, void* workspace, size_t workspace_bytes, void* stream);

size_t mamba_mixer_prefill_workspace_bytes_chunked(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                                                   int64_t chunk_len);

/*
 * mamba_mixer_prefill_ex -- the full-control prefill: explicit chunk length
 * (<= 0: automatic), explicit engine (MM_ENGINE_*), and optional per-kernel timing
 * for measurement tools.  When `events` is not NULL the call also records
 * events[i] (a hipEvent_t the caller created) on `stream` just before the i-th
 * kernel it enqueues and events[n] just after the last one, where n is the kernel
 * count mamba_mixer_prefill_plan reports; n_events < n + 1 with events != NULL is
 * MM_ERR_DIM.  The events are only recorded; the caller owns and destroys them.
 * An unknown engine is MM_ERR_UNSUPPORTED.  The workspace size comes from
 * mamba_mixer_prefill_plan with the same chunk_len and engine.
 */
int mamba_mixer_prefill_ex(const void* x, const void* z, const void* dt, const void* B, const void* C,
                           const float* A_log, const float* D, const float* dt_bias,
                           const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                           float* conv_state, float* ssm_state, void* y,
                           int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                           int64_t chunk_len, int32_t engine, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* events, int32_t n_events);

/*
 * mamba_mixer_prefill_plan -- what a prefill call with these sizes, chunk_len and
 * engine will do (host only; each output pointer may be NULL): the chunk length,
 * the engine, the workspace bytes it needs and the number of kernels it enqueues.
 * Returns MM_OK or the argument error the call itself would return.
 */
int mamba_mixer_prefill_plan(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int64_t chunk_len,
                             int32_t engine, int64_t* chunk_len_out, int32_t* engine_out, size_t* workspace_out,
                             int32_t* kernels_out);

/* Name of the i-th kernel such a call enqueues ("" if out of range).  Host only. */
const char* mamba_mixer_prefill_kernel_name(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int64_t chunk_len,
                                            int32_t engine, int32_t i);

/*
 * mamba_mixer_decode -- one token for each of Bs independent rows; row r uses
 * state slot r.  This is the TensorRT builder's single-token step with a batch
 * dimension (same arithmetic as a prefill of Bs one-token sequences).
 *
 *   x, z, dt      [Bs, d]       io
 *   B, C          [Bs, N]       io
 *   A_log [d, N], D [d], dt_bias [d], conv_w [d, K], conv_b [d]   f32
 *   conv_state    [Bs, d, K-1]  f32 in/out (drops its oldest entry, appends x)
 *   ssm_state     [Bs, d, N]    f32 in/out
 *   y             [Bs, d]       io  out
 * Bs == 0 or d == 0 is a successful no-op.
 */
int mamba_mixer_decode(const void* x, const void* z, const void* dt, const void* B, const void* C,
                       const float* A_log, const float* D, const float* dt_bias,
                       const float* conv_w, const float* conv_b,
                       float* conv_state, float* ssm_state, void* y,
                       int32_t Bs, int32_t d, int32_t N, int32_t K, int32_t io_dtype, void* stream);

/*
 * mamba_mixer_decode_replay -- one decode token for each of Bs rows with the state
 * kept as a checkpoint plus the inputs of the recent steps ("ReplaySSM: Cache SSM
 * Inputs, Not State", abstract: the state is represented as a checkpoint and a
 * buffer of recent inputs, and the checkpoint is updated only periodically, so most
 * steps read the state but do not write it).
 *
 * A window has W steps (1 <= W <= 4); this call is step k of it (0 <= k < W).
 *   x_ring, dt_ring [W, Bs, d]  io   raw x and dt of window steps 0..k; the caller writes
 *                                    step k's x and dt into slot k before the call
 *   B_ring          [W, Bs, N]  io   B of window steps 0..k, slot k likewise
 *   z [Bs, d], C [Bs, N]        io   gate input and readout vector of step k
 *   A_log [d, N], D [d], dt_bias [d], conv_w [d, K], conv_b [d]   f32
 *   conv_state [Bs, d, K-1], ssm_state [Bs, d, N]   f32  the checkpoint: the state before
 *                                    window step 0.  Read every call; overwritten with the
 *                                    state after step k when the call commits
 *   y [Bs, d]                   io   out: step k's output
 * The call commits when commit != 0 or k == W - 1; after a committing call the next
 * window starts at k = 0 (the ring slots are free again).  Step k's output and the
 * committed state equal, bit for bit, those of k + 1 mamba_mixer_decode calls from the
 * checkpoint (the same operations in the same order).
 * Limits: N == 16 (else MM_ERR_UNSUPPORTED); W outside 1..4 or k outside 0..W-1 is
 * MM_ERR_DIM; A_log, conv_w and ssm_state must be 16-byte aligned and B_ring, C aligned
 * to 4 elements (MM_ERR_ALIGN).  Bs == 0 or d == 0 is a successful no-op.
 */
int mamba_mixer_decode_replay(const void* x_ring, const void* dt_ring, const void* B_ring, const void* z,
                              const void* C, const float* A_log, const float* D, const float* dt_bias,
                              const float* conv_w, const float* conv_b, float* conv_state, float* ssm_state,
                              void* y, int32_t Bs, int32_t d, int32_t N, int32_t K, int32_t io_dtype, int32_t W,
                              int32_t k, int32_t commit, void* stream);

/*
 * mamba_mixer_decode_replay_dual -- mamba_mixer_decode_replay with the dual-precision
 * checkpoint of the ReplaySSM page (abstract: a low-precision checkpoint serves the output
 * computation on most steps, a higher-precision checkpoint the recurrent updates).  Beside the
 * fp32 checkpoint (conv_state, ssm_state) the caller keeps its bf16 copy:
 *   conv_lo   [Bs, d, 4]  bf16   conv_state rounded to nearest even; entry 3 is zero
 *   ssm_lo    [Bs, d, N]  bf16   ssm_state rounded to nearest even
 * A call that does not commit reads only the copy (40 bytes per (row, channel) instead of 76):
 * its output is that of the window step from the rounded checkpoint.  A committing call
 * (commit != 0 or k == W - 1) reads the fp32 checkpoint: its output and the state it commits
 * equal, bit for bit, those of the eager decode, and it rewrites both checkpoints.  Fill the
 * copy once with mamba_mixer_replay_checkpoint_lo (e.g. after the prefill that initialises the
 * state).  Everything else, the ring layouts and the limits are those of
 * mamba_mixer_decode_replay; io must be MM_IO_BF16 (else MM_ERR_UNSUPPORTED); ssm_lo must be
 * 16-byte and conv_lo 8-byte aligned (MM_ERR_ALIGN); the copies may not overlap any other
 * array (MM_ERR_ALIAS).
 */
int mamba_mixer_decode_replay_dual(const void* x_ring, const void* dt_ring, const void* B_ring, const void* z,
                                   const void* C, const float* A_log, const float* D, const float* dt_bias,
                                   const float* conv_w, const float* conv_b, float* conv_state, float* ssm_state,
                                   void* conv_lo, void* ssm_lo, void* y, int32_t Bs, int32_t d, int32_t N, int32_t K,
                                   int32_t io_dtype, int32_t W, int32_t k, int32_t commit, void* stream);

/* The bf16 copy (conv_lo [Bs, d, 4], ssm_lo [Bs, d, N], rounded to nearest even, conv entry 3
 * zero) of an fp32 replay checkpoint, for mamba_mixer_decode_replay_dual.  N must be 16;
 * alignment and overlap rules as there. */
int mamba_mixer_replay_checkpoint_lo(const float* conv_state, const float* ssm_state, void* conv_lo, void* ssm_lo,
                                     int32_t Bs, int32_t d, int32_t N, int32_t K, void* stream);

/*
 * mamba_mixer_decode_replay_multi -- several steps of a replay window in one call, for
 * speculative decoding (the ReplaySSM page, abstract: with the recent inputs kept,
 * rolling back a speculation is a buffer-pointer move, and outputs of draft tokens can be
 * checked without materialising intermediate states).
 *
 * Window steps 0..k1 are taken from the checkpoint; steps k0..k1 (0 <= k0 <= k1 < W <= 4)
 * write their outputs; no state is written unless 0 <= commit_step <= k1, in which case the
 * state after window step commit_step becomes the checkpoint (the accepted prefix of a
 * draft; the caller then starts the next window at slot 0, with the rejected drafts
 * dropped).  commit_step == -1 commits nothing.
 *   x_ring, dt_ring, z_ring, y_ring [W, Bs, d] io   (y_ring out, slots k0..k1 written)
 *   B_ring, C_ring                  [W, Bs, N] io
 * Everything else, the alignment rules and the limits are those of
 * mamba_mixer_decode_replay; the outputs and the committed state equal, bit for bit, those
 * of the corresponding single-step calls.  k0 > k1, k1 >= W or commit_step outside -1..k1
 * is MM_ERR_DIM.
 */
int mamba_mixer_decode_replay_multi(const void* x_ring, const void* dt_ring, const void* B_ring, const void* z_ring,
                                    const void* C_ring, const float* A_log, const float* D, const float* dt_bias,
                                    const float* conv_w, const float* conv_b, float* conv_state, float* ssm_state,
                                    void* y_ring, int32_t Bs, int32_t d, int32_t N, int32_t K, int32_t io_dtype,
                                    int32_t W, int32_t k0, int32_t k1, int32_t commit_step, void* stream);

/*
 * mamba_mixer_prefill_backward -- the gradients of a loss L with respect to every input of
 * a prefill call, its parameters and its initial states, given dy = dL/dy (L does not
 * depend on the final states).  This is the reverse mode of the step above, by the chain
 * rule, sequence by sequence: no gradient crosses a cu_seqlens boundary (PackMamba page,
 * abstract: packed sequences do not influence one another).  Training with packed
 * sequences needs it; the pages describe the forward step only, so the gradients follow
 * from that step alone.
 *
 * Inputs, with the layouts and dtypes of mamba_mixer_prefill (read only):
 *   x, z, dt [T, d], B, C [T, N] (io), A_log, D, dt_bias, conv_w, conv_b (f32),
 *   cu_seqlens [S+1], conv_state [S, d, K-1] and ssm_state [S, d, N]: the INITIAL states
 *   (those a forward call reads; the backward does not change them)
 *   dy            [T, d]      io     dL/dy
 *   ckpt          NULL, or the checkpoints mamba_mixer_prefill_train stored for these
 *                 inputs and initial states: the backward then skips its own forward pass
 *                 and does not read ssm_state (which may be NULL).
 * Outputs (all overwritten):
 *   dx, dz, ddt   [T, d]      io     ddt is dL/d(dt) (equal to the share of dt_bias)
 *   dB, dC        [T, N]      io     summed over channels
 *   dA_log        [d, N]      f32
 *   dD, ddt_bias, dconv_b [d] f32
 *   dconv_w       [d, K]      f32
 *   dconv_state   [S, d, K-1] f32    dL/d(initial conv state)
 *   dssm_state    [S, d, N]   f32    dL/d(initial SSM state)
 *   workspace     device scratch of at least mamba_mixer_prefill_backward_workspace_bytes
 *                 bytes (with has_ckpt = ckpt != NULL), 256-byte aligned: about
 *                 128 * T * N * d/16 bytes of per-16-channel partial sums of dB and dC, plus
 *                 mamba_mixer_checkpoint_bytes when ckpt is NULL
 *   events, n_events   optional, as in mamba_mixer_prefill_ex: events[i] is recorded before
 *                 the i-th kernel and events[n] after the last; n is the kernel count
 *                 mamba_mixer_prefill_backward_plan reports (4 without ckpt, 3 with it, 1
 *                 when S == 0).
 * The sums over channels, tokens and sequences are taken in a fixed order: the results do
 * not vary from run to run.  An empty sequence gets zero state gradients.  d == 0 is a
 * successful no-op; with T == 0 the parameter and state gradients are zeros.  Arrays of
 * zero bytes may be NULL.  Outputs overlapping an input or one another are MM_ERR_ALIAS.
 */
int mamba_mixer_prefill_backward(const void* x, const void* z, const void* dt, const void* B, const void* C,
                                 const float* A_log, const float* D, const float* dt_bias, const float* conv_w,
                                 const float* conv_b, const int32_t* cu_seqlens, const float* conv_state,
                                 const float* ssm_state, const void* dy, const float* ckpt, void* dx, void* dz,
                                 void* ddt, void* dB, void* dC, float* dA_log, float* dD, float* ddt_bias, float* dconv_w, float* dconv_b,
                                 float* dconv_state, float* dssm_state, int32_t S, int64_t T, int32_t d, int32_t N,
                                 int32_t K, int32_t io_dtype, void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events, int32_t n_events);
/* Workspace bytes and kernel count of mamba_mixer_prefill_backward for these sizes, with
 * (has_ckpt != 0) or without checkpoints (host only; either output pointer may be NULL).
 * Returns MM_OK or the size error the call would return. */
int mamba_mixer_prefill_backward_plan(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K, int32_t has_ckpt,
                                      size_t* workspace_out, int32_t* kernels_out);
size_t mamba_mixer_prefill_backward_workspace_bytes(int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                                                    int32_t has_ckpt);
/*
 * mamba_mixer_prefill_train -- the forward of a training step: mamba_mixer_prefill (row
 * engine, MM_ENGINE_ROW) that also stores the SSM state before every 16-token block, so
 * that mamba_mixer_prefill_backward need not run the forward again.
 *   ckpt   [ceil(T/16) + S, d, 16] f32, out, mamba_mixer_checkpoint_bytes(S, T, d) bytes,
 *          4-byte aligned: the 16-token blocks are aligned in the packed token stream; the
 *          state before the block starting at token tb of sequence s (entries n >= N zero)
 *          is row s + tb/16.  Rows of blocks no sequence has stay unwritten.
 * Everything else is mamba_mixer_prefill_ex with engine MM_ENGINE_ROW (the workspace size
 * comes from mamba_mixer_prefill_plan with that engine).  The states are overwritten with
 * the final states as usual: a caller that runs the backward keeps a copy of the initial
 * conv_state (the backward reads it; the initial SSM state is in the checkpoints).
 */
int mamba_mixer_prefill_train(const void* x, const void* z, const void* dt, const void* B, const void* C,
                              const float* A_log, const float* D, const float* dt_bias, const float* conv_w,
                              const float* conv_b, const int32_t* cu_seqlens, float* conv_state, float* ssm_state,
                              void* y, float* ckpt, int32_t S, int64_t T, int32_t d, int32_t N, int32_t K,
                              int32_t io_dtype, int64_t chunk_len, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events, int32_t n_events);
/* Bytes of the checkpoints of a prefill of S sequences and T tokens with d channels (0 for sizes
 * the calls reject). */
size_t mamba_mixer_checkpoint_bytes(int32_t S, int64_t T, int32_t d);
/*
 * mamba_mixer_project -- the input-dependent projections that produce the scan's dt, B and C
 * from x, in the layer order of the TensorRT Mamba tensor-parallel builder (builder page,
 * _add_mamba_tp_layer): the conv activation u = SiLU(conv(x)) (the same window, weights and
 * initial conv state as the mixer), then dt_in = u w_dt_in, B = u w_B, C = u w_C, and
 * dt = dt_in w_dt_out.  The outputs are exactly what mamba_mixer_prefill takes: dt before
 * dt_bias (the mixer adds it before its softplus, as the builder adds dt_proj_bias), B and C.
 * In a tensor-parallel layer the builder all-reduces dt_in, B and C between the two products;
 * on one GPU nothing is reduced.
 *
 *   x            [T, d]      bf16   raw SSM-path input (before the conv), 16-byte aligned
 *   conv_w [d, K], conv_b [d]  f32  16-byte aligned;  cu_seqlens [S+1]
 *   conv_state   [S, d, K-1] f32    the INITIAL conv state (read only); 4-byte aligned, and when
 *                                   16-byte aligned the kernel stages it with the x tiles (faster
 *                                   for tiles where sequences start)
 *   w_x          [d, R+2N]   bf16   input-major: columns 0..R-1 are w_dt_in, then w_B, then w_C
 *   w_dt         [R, d]      bf16   w_dt_out
 *   dt           [T, d]      bf16   out, 16-byte aligned
 *   B, C         [T, N]      bf16   out
 *   workspace    mamba_mixer_project_workspace_bytes(T, d, N, R) bytes, 256-byte aligned (the
 *                weights re-laid for the matrix cores, and dt_in between the two products;
 *                contents on entry do not matter)
 * Both products run on the matrix cores (bf16 MFMA, fp32 accumulation); the computed operands
 * u and dt_in enter as bf16 high + low parts, so the products have fp32-quality operands and
 * the outputs are rounded once, to bf16 (nearest even).
 * Limits: io MM_IO_BF16 only, d a multiple of 16 and at most MM_PROJECT_MAX_D, 1 <= R <= 256
 * (else MM_ERR_UNSUPPORTED).
 * T == 0 or d == 0 is a successful no-op.  Outputs overlapping an input or one another are
 * MM_ERR_ALIAS.  Three kernels are enqueued (weight re-layout; u x w_x, which writes B, C and
 * dt_in; dt_in x w_dt, which writes dt); events, n_events are optional as in
 * mamba_mixer_prefill_ex (n = 3: events[i] before kernel i, events[3] after the last).
 */
#define MM_PROJECT_MAX_D (1 << 22) /* channels of mamba_mixer_project (its per-row offsets are 32-bit) */
int mamba_mixer_project(const void* x, const float* conv_w, const float* conv_b, const int32_t* cu_seqlens,
                        const float* conv_state, const void* w_x, const void* w_dt, void* dt, void* B, void* C,
                        int32_t S, int64_t T, int32_t d, int32_t N, int32_t R, int32_t K, int32_t io_dtype,
                        void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                        int32_t n_events);
/* Workspace bytes of mamba_mixer_project for T tokens (0 for invalid sizes).  Host only. */
size_t mamba_mixer_project_workspace_bytes(int64_t T, int32_t d, int32_t N, int32_t R);
/* Static text for a status code (never NULL).  Host only. */
const char* mamba_mixer_status_string(int status);

/* Library version, e.g. "libmambamix 0.1 gfx950".  Host only. */
const char* mamba_mixer_version(void);

/* The cu_seqlens preconditions of every call that takes the array, checked on a HOST copy of
 * it (cu_seqlens_host [S+1]): cu[0] == 0, cu non-decreasing, cu[S] == T.  MM_OK, or MM_ERR_DIM
 * for a violation or negative S or T, MM_ERR_NULL for a NULL array.  For callers that want the
 * check (the calls themselves never read the array on the host).  Host only. */
int mamba_mixer_check_cu_seqlens(const int32_t* cu_seqlens_host, int32_t S, int64_t T);

#ifdef __cplusplus
}
#endif

#endif /* MAMBAMIX_H */
