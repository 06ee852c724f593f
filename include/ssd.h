/*
 * ssd.h -- C ABI of libssd.so, the MI355X (gfx950) SSD chunked-scan library.
 *
 * The operation is the selective state-space recurrence evaluated chunk-wise
 * ("Structured State Space Duality" concept page, sections "The recurrence as
 * one matrix" and "The chunked algorithm takes both"):
 *
 *     h_t = a_t * h_{t-1} + x_t B_t^T        (per head: state P x N)
 *     y_t = h_t C_t + D_h * x_t
 *
 * with a scalar decay per head and token, a_t = exp(dt_t * A_h), or -- for the
 * diagonal variant ("What the duality gives up" on the same page; "Diagonal
 * Equivalence in State Space Models", abstract) -- one decay per state
 * dimension, a_{t,n} = exp(dt_t * A_{h,n}).  h0 is the state before token 0; the
 * final state h_T is the state after the last token.  The sequence is split into
 * chunks of `chunk` tokens: a masked matmul on each diagonal block, and one state
 * step per chunk across blocks; the result does not depend on the chunk size
 * beyond floating-point rounding.
 *
 * Layouts (row-major, contiguous, no strides):
 *     x, y   [batch, seqlen, nheads, headdim]        dtype of the problem
 *     dt     [batch, seqlen, nheads]                 float32
 *     A      [nheads] (scalar) / [nheads, dstate]    float32
 *     B, C   [batch, seqlen, ngroups, dstate]        dtype of the problem
 *     D      [nheads]                                float32 (may be NULL = 0)
 *     h0, hT [batch, nheads, headdim, dstate]        float32 (h0 NULL = 0; hT NULL = not written)
 * Head h reads B/C group floor(h * ngroups / nheads) (contiguous blocks of heads).
 *
 * Precision: decay sums, exponentials and the carried state are float32; x, B, C (and
 * the masked scores and entering states fed to the matrix cores) are in the problem
 * dtype, and so is each chunk's state S_c where the split schedule stores it (rounded
 * once, then summed in float32); accumulation is float32; y is rounded once to the
 * problem dtype.
 * Accuracy is stated for A <= 0 (decays in (0, 1]); NaN inputs propagate.
 *
 * Ownership and ordering: every pointer is a device pointer owned by the caller.
 * The library allocates nothing and keeps no global mutable state; calls are
 * thread-safe.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising: inputs and the workspace
 * must stay alive until the stream has passed this work.  Outputs must not
 * overlap any input or the workspace.  Two calls that share a workspace must be
 * ordered on one stream.
 *
 * Errors: every entry point validates on the host, before any HIP call, and
 * returns an ssd_status; nothing is enqueued on failure.  SSD_ERR_HIP reports a
 * launch failure (hipGetLastError after enqueueing).
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_VERSION 100 /* 1.0.0 */

typedef enum {
    SSD_F32 = 0,  /* x, B, C, y are float32 */
    SSD_BF16 = 1  /* x, B, C, y are bfloat16 */
} ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* a dimension is negative/zero where it must not be, or nheads % ngroups != 0 */
    SSD_ERR_UNSUPPORTED = 3, /* chunk, headdim, dstate or dtype outside the supported set */
    SSD_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than ssd_workspace_bytes() */
    SSD_ERR_ALIGN = 5,       /* x/B/C/y/h0/hT not 16-byte aligned, dt/A/D not 4-byte, workspace not 256-byte */
    SSD_ERR_ALIAS = 6,       /* y or hT overlaps an input, the other output or the workspace */
    SSD_ERR_HIP = 7          /* a kernel launch failed */
} ssd_status;

/* Problem descriptor.  Supported: chunk in {64, 128, 256}; headdim in {16, 32, 64, 128};
 * dstate in {16, 32, 64, 128, 256}; any seqlen >= 0 (a ragged last chunk is allowed);
 * batch >= 0; nheads >= 1; ngroups >= 1 dividing nheads; launch-grid limits: batch and
 * batch * ngroups at most 65535, ceil(nheads / 16) + 28 * ngroups at most 65535, nheads
 * at most 2^20, batch * nheads * nchunks under 2^31 (else SSD_ERR_UNSUPPORTED). */
typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int32_t dtype;  /* ssd_dtype */
    int32_t flags;  /* 0 = the whole forward; see SSD_STAGE_* */
} ssd_problem;

/* Schedules.  The library runs one of two kernel sequences:
 *   fused  k_cumsum, k_cb, k_bt, then k_fused: one work-group per (batch, head) walks its
 *          chunks in order with the state held on chip (scalar decay, bf16, headdim 64,
 *          dstate 64 or 128);
 *   split  k_cumsum, k_cb (scalar decay), k_state, k_scan, k_out: every stage is a
 *          separate chunk-parallel launch and chunk states go through the workspace.
 *          k_scan is one sequential pass over chunks per state element; when
 *          batch * nheads * headdim * dstate / 4 is under 131072 and there are at least 8
 *          chunks, it runs instead as a parallel scan over 2 to 64 segments of at least 4
 *          chunks ("Semiseparable Matrix Transformations": state-space evaluation as a
 *          parallel scan): each segment from a zero state, a short pass over segments for
 *          the state entering each, and each segment again from that state.
 * flags = 0 runs fused where it exists and there are at least 512 (batch, head) chains
 * to fill the GPU (one work-group each), else split.  SSD_SCHEDULE_SPLIT asks for split
 * explicitly; SSD_SCHEDULE_FUSED asks for fused at any (batch, head) count and is
 * SSD_ERR_UNSUPPORTED where the fused kernel does not exist (other dtype, decay,
 * headdim or dstate).
 *
 * Diagnostics only (per-kernel timing and per-stage inspection): a nonzero stage mask
 * in the low byte of `flags` enqueues just those kernels; their inputs are read from the
 * workspace, which a previous full call on the same problem, inputs and workspace must
 * have filled.  The mask may name only kernels of the schedule that runs (the workspace
 * holds that schedule's regions only): cumsum, cb, bt and fused for the fused schedule;
 * cumsum, cb, state, scan and out for the split one.  Any other bit is
 * SSD_ERR_UNSUPPORTED. */
#define SSD_STAGE_CUMSUM 0x01 /* chunk-local cumulative sum of dt      -> ws cdt     */
#define SSD_STAGE_CB 0x02     /* C_c B_c^T per chunk (scalar decay)    -> ws cb      */
#define SSD_STAGE_STATE 0x04  /* chunk states S_c                      -> ws states  */
#define SSD_STAGE_SCAN 0x08   /* inter-chunk state scan                -> ws hin, hT */
#define SSD_STAGE_OUT 0x10    /* diagonal blocks + state output + D    -> y          */
#define SSD_STAGE_BT 0x20     /* per-chunk B with tokens contiguous    -> ws bt      */
#define SSD_STAGE_FUSED 0x40  /* fused per-(batch, head) scan          -> y, hT      */
#define SSD_STAGE_ALL 0x7f
#define SSD_SCHEDULE_SPLIT 0x100
#define SSD_SCHEDULE_FUSED 0x200

/* Bytes of device workspace that ssd_scan_fwd (diag = 0) or ssd_diag_scan_fwd
 * (diag = 1) needs for this problem; 0 if the problem is invalid or empty.  The size
 * follows the schedule the problem runs (the schedule flags in p->flags and the shape;
 * see the schedule notes): the fused schedule needs the per-chunk tables only, the
 * split schedule also the chunk states and entering states.  Pure host function. */
size_t ssd_workspace_bytes(const ssd_problem* p, int diag);

/* Where each intermediate lives inside the workspace (byte offsets, each 256-aligned;
 * a size of 0 means "absent"), for inspection after a call has completed:
 *   cdt  float32 [batch, nheads, nchunks, chunk]  chunk-local cumulative sum of dt
 *        (positions past seqlen repeat the chunk total)
 *   cb   dtype   [batch, nchunks, ngroups, chunk, chunk]  C_c B_c^T, blocks on and below
 *        the diagonal (scalar decay); for the diagonal decay, where its output tile does
 *        not fit LDS (see ssd_diag_scan_fwd), [batch, nheads, nchunks, chunk, chunk] each
 *        head's decay-weighted block sum_n C_in B_jn exp(A_n (cdt_i - cdt_j)), D on the
 *        diagonal, zero above it
 *   states dtype [batch, nheads, nchunks, headdim, dstate]  chunk states S_c
 *   hin  dtype   [batch, nheads, nchunks, headdim, dstate]  state entering chunk c
 *   bt   dtype   [batch, nchunks, ngroups, dstate, chunk]  B of each chunk by token, then
 *        [batch, nchunks, ngroups, chunk, dstate] C of each chunk (fused schedule)
 * The per-chunk tables (cb and bt: a chunk's rows of `chunk` columns) are stored in
 * matrix-core fragment order: entry (r, col) of a chunk's table sits at element
 *   ((r / 16) * (chunk / 32) + col / 32) * 512 + ((col % 32) / 8) * 128 + (r % 16) * 8 + col % 8
 * of that chunk's block, so that the 16 x 32 fragment a kernel loads is one contiguous
 * run.
 *   carry float32 [nseg, batch, nheads, headdim, dstate] then [batch, nheads, nseg]: the
 *        state entering each segment of chunks and each segment's summed cdt totals,
 *        when the split schedule's state scan runs as a parallel scan over segments
 *        (batch * nheads * headdim * dstate too small to fill the GPU; see the schedule
 *        notes); absent otherwise
 * Only the regions of the schedule that runs are present (the others have size 0): the
 * split schedule has cdt, cb, states and hin (and carry); the fused one cdt, cb and bt.
 * Returns an ssd_status.  Pure host function. */
typedef struct {
    size_t cdt_off, cdt_bytes;
    size_t cb_off, cb_bytes;
    size_t states_off, states_bytes;
    size_t hin_off, hin_bytes;
    size_t bt_off, bt_bytes;
    size_t carry_off, carry_bytes;
    size_t total_bytes;
} ssd_workspace_layout;
int ssd_get_workspace_layout(const ssd_problem* p, int diag, ssd_workspace_layout* out);

/* Stream capture: no entry point allocates, sets memory with a memset, synchronises the
 * host or reads device memory on the host, so every call can be captured into a HIP
 * graph on the caller's stream and replayed (with the same arguments and workspace). */

/* Scalar-decay SSD forward: A is [nheads].  Writes y (and hT if non-NULL).
 * `ws` must hold ssd_workspace_bytes(p, 0) bytes. */
int ssd_scan_fwd(const ssd_problem* p, const void* x, const float* dt, const float* A,
                 const void* B, const void* C, const float* D, const float* h0,
                 void* y, float* hT, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): ssd_scan_fwd with its workspace taken
 * from a scratch array the library keeps in each GPU's memory, SSD_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held from the first call on that GPU (the current device) until the
 * process ends.  The caller passes inputs and outputs only; arguments, schedule flags and
 * errors are as for ssd_scan_fwd, and a problem whose ssd_workspace_bytes(p, 0) exceeds
 * the scratch returns SSD_ERR_WORKSPACE before any HIP call (the 2.7B layer shape,
 * b8 T4096 H80 P64 N128 Q256 on the fused schedule, needs 44.0 MB).  The forward fully
 * writes every scratch region it reads, so no clearing is needed between calls.  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from threads without ordering) race on it and must be ordered
 * on one stream.  The stream must belong to the current device.  Nothing is allocated
 * and nothing is freed. */
#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)
int ssd_scan_fwd_noalloc(const ssd_problem* p, const void* x, const float* dt, const float* A,
                         const void* B, const void* C, const float* D, const float* h0,
                         void* y, float* hT, void* stream);

/* Diagonal-decay SSD forward: A is [nheads, dstate].  Same conventions;
 * `ws` must hold ssd_workspace_bytes(p, 1) bytes.  Every supported (chunk, headdim,
 * dstate, dtype) runs.  The output kernel keeps a chunk's x rows and its rescaled C and B
 * rows in LDS where (chunk * (headdim + 8) + 2 * chunk * (dstate + 8)) elements plus
 * (2 * chunk + dstate) floats fit the 160 KiB of one CU; otherwise (bfloat16 at chunk 256
 * with dstate 128 or more, for example) a table kernel first forms each (batch, head,
 * chunk)'s decay-weighted query-key block in the workspace's cb region,
 * batch * nheads * nchunks * chunk^2 elements, and the output kernel reads it. */
int ssd_diag_scan_fwd(const ssd_problem* p, const void* x, const float* dt, const float* A,
                      const void* B, const void* C, const float* D, const float* h0,
                      void* y, float* hT, void* ws, size_t ws_bytes, void* stream);

/* Packed variable-length sequences.  The batch holds `batch` sequences of different
 * lengths back to back on one token axis of `seqlen` tokens: sequence s is tokens
 * [cu_seqlens[s], cu_seqlens[s+1]).  Each sequence is a separate map with its own state
 * ("Structured State Space Duality" concept page, section "The chunked algorithm takes
 * both": the state passes from chunk to chunk within a sequence), so the result for
 * sequence s equals ssd_scan_fwd on that sequence alone, up to rounding.  Chunks restart
 * at each sequence's first token.
 *
 *   x, y            [seqlen, nheads, headdim]   (the batch dimension is the packing)
 *   dt              [seqlen, nheads] float32
 *   B, C            [seqlen, ngroups, dstate]
 *   A, D            [nheads] float32 (scalar decay; D may be NULL)
 *   h0, hT          [batch, nheads, headdim, dstate] float32, one state per sequence
 *                   (h0 NULL = zero; hT NULL = not written)
 *   cu_seqlens      device int32 [batch + 1], nondecreasing from 0 to seqlen.  The
 *                   library reads only clamped copies (each offset is clamped into
 *                   [previous offset, seqlen]), so any values are memory-safe; offsets
 *                   outside that contract give unspecified y and hT.  Empty sequences
 *                   are allowed (their hT is their h0).
 *
 * Runs on the fused schedule: dtype SSD_BF16, headdim 64, dstate 64 or 128, scalar
 * decay; any other problem, SSD_SCHEDULE_SPLIT, or a packed axis whose per-tensor spans
 * reach 2 GiB returns SSD_ERR_UNSUPPORTED before any HIP call.  `ws` must hold
 * ssd_varlen_workspace_bytes(p) bytes (0 for an empty problem); alignment and aliasing
 * rules as for ssd_scan_fwd, and cu_seqlens must not overlap the workspace or outputs.
 * Stage flags work as for ssd_scan_fwd (the row map is built with the cumsum stage). */
size_t ssd_varlen_workspace_bytes(const ssd_problem* p);
int ssd_scan_fwd_varlen(const ssd_problem* p, const int32_t* cu_seqlens, const void* x,
                        const float* dt, const float* A, const void* B, const void* C,
                        const float* D, const float* h0, void* y, float* hT, void* ws,
                        size_t ws_bytes, void* stream);

/* The recurrence itself, token by token, on a state the caller holds (the linear form of
 * the same map: "Structured State Space Duality" concept page, section "The recurrence as
 * one matrix"; section "When it breaks" on serving with this form).  For t = 0 .. seqlen-1:
 *
 *     h <- a_t h + x_t B_t^T,    y_t = h C_t + D_h x_t,
 *
 * with a_t = exp(dt_t A_h) (ssd_step) or exp(dt_t A_{h,n}) per state dimension
 * (ssd_diag_step).  A decode step is seqlen = 1; longer sequences run the tokens in
 * order (results agree with ssd_scan_fwd on the same tokens up to rounding, not
 * bitwise).
 *
 *   x, y, dt, A, B, C, D   as for ssd_scan_fwd (same layouts and dtypes; D may be NULL);
 *   h                      [batch, nheads, headdim, dstate] float32, read and overwritten
 *                          in place: the state before the first token on entry, the
 *                          state after the last on return.
 * `chunk` is ignored; `flags` must be 0.  No workspace.  headdim in {16,32,64,128},
 * dstate in {16,32,64,128,256}.  batch = 0 or seqlen = 0 leaves h untouched.
 * Errors as for ssd_scan_fwd: NULL pointers, h not 16-byte aligned, B/C not aligned to
 * 4 elements, y or h overlapping an input or each other, unsupported sizes -- all
 * reported before any HIP call. */
int ssd_step(const ssd_problem* p, const void* x, const float* dt, const float* A,
             const void* B, const void* C, const float* D, float* h, void* y, void* stream);
int ssd_diag_step(const ssd_problem* p, const void* x, const float* dt, const float* A,
                  const void* B, const void* C, const float* D, float* h, void* y,
                  void* stream);

/* Backward pass of ssd_scan_fwd (scalar decay): the gradients of a loss L with respect to
 * every input, given dy = dL/dy and dhT = dL/dhT.  The pages define the forward map only
 * ("Structured State Space Duality" concept page, sections "The recurrence as one matrix"
 * and "The chunked algorithm takes both"); these are its derivatives.  With
 * g_t = dL/dh_t = dy_t C_t^T + a_{t+1} g_{t+1} (and dhT after the last token):
 *
 *     dx_t  = g_t B_t + D_h dy_t            dB_t = sum over the group's heads of g_t^T x_t
 *     dC_t  = sum over heads of h_t^T dy_t  dh0  = a_0 g_0
 *     ddt_t = A_h sum_{u >= t} [dy_u . (y_u - D_h x_u) - x_u . (dx_u - D_h dy_u)] + A_h <dhT, hT>
 *     dA_h  = sum_{b,t} dt_t ddt_t / A_h (formed without the division)
 *     dD_h  = sum_{b,t} dy_t . x_t
 *
 * computed chunk-wise like the forward: the adjoint g is the same recurrence run backward in
 * time, carried across chunks by a reverse scan; the forward states entering each chunk are
 * rebuilt from the inputs (nothing from a previous forward call is reused).
 *
 *   inputs   x, dt, A [nheads], B, C, D, h0: as for ssd_scan_fwd (D, h0 may be NULL = 0);
 *            dy [batch, seqlen, nheads, headdim] in the problem dtype;
 *            dhT [batch, nheads, headdim, dstate] float32 (NULL = 0)
 *   outputs  dx [batch, seqlen, nheads, headdim] problem dtype; ddt [batch, seqlen, nheads]
 *            float32; dA [nheads] float32; dB, dC [batch, seqlen, ngroups, dstate] problem
 *            dtype; dD [nheads] float32 (NULL = not written); dh0 [batch, nheads, headdim,
 *            dstate] float32 (NULL = not written).  Every output is overwritten, not
 *            accumulated into; dD and dh0 are the gradients for D and h0 whether or not D
 *            and h0 were given.
 * Precision as for the forward: decay sums, exponentials, states and every accumulation in
 * float32; matrix-core operands in the problem dtype; each output rounded once.
 * `ws` must hold ssd_bwd_workspace_bytes(p) bytes (0 for an empty problem, where dA = dD = 0
 * and dh0 = dhT).  flags must be 0.  Same support set as ssd_scan_fwd (chunk, headdim,
 * dstate, dtype) except float32 with headdim 128 at chunk 256, whose per-head LDS tiles
 * do not fit one CU: SSD_ERR_UNSUPPORTED.  Alignment as for ssd_scan_fwd
 * (dy, dx, dB, dC 16 bytes; ddt, dA, dD 4; dhT, dh0 16); no output may overlap an input,
 * the workspace or another output (SSD_ERR_ALIAS).  Errors are reported before any HIP
 * call. */
size_t ssd_bwd_workspace_bytes(const ssd_problem* p);
int ssd_scan_bwd(const ssd_problem* p, const void* x, const float* dt, const float* A,
                 const void* B, const void* C, const float* D, const float* h0, const void* dy,
                 const float* dhT, void* dx, float* ddt, float* dA, void* dB, void* dC, float* dD,
                 float* dh0, void* ws, size_t ws_bytes, void* stream);

/* Backward pass of ssd_diag_scan_fwd (a_{t,n} = exp(dt_t A_{h,n}), A [nheads, dstate]):
 * the same gradients as ssd_scan_bwd with the decay taken per state dimension
 * ("Structured State Space Duality" concept page, the diagonal generalisation of the
 * scalar decay):
 *
 *     dx_t  = sum_n g_t[:, n] B_{t,n} + D_h dy_t      dB_{t,n} = sum over heads of x_t . g_t[:, n]
 *     dC_{t,n} = sum over heads of dy_t . h_t[:, n]   dh0 = (a_{0,n} g_0[:, n])_n
 *     ddt_t = sum_n A_{h,n} dl_{t,n},   dA_{h,n} = sum_{b,t} dt_t dl_{t,n},
 *     dl_{t,n} = sum_{u >= t} [C_{u,n} dy_u . h_u[:, n] - B_{u,n} x_u . g_u[:, n]] + <dhT, hT>_n
 *
 * with h_t the state after token t and g_t = dy_t C_t^T + a_{t+1} g_{t+1} its gradient.
 * Across chunks it runs the forward's chunk states and scan and the same scan backward for
 * the adjoint; within a chunk every (batch, head) walks its tokens forward and backward
 * from the chunk's boundary states, all in float32.  Arguments, layouts, outputs and
 * alignment as for ssd_scan_bwd, except A and dA, which are [nheads, dstate] float32.
 * `ws` must hold ssd_diag_bwd_workspace_bytes(p) bytes (0 for an empty problem, where
 * dA = dD = 0 and dh0 = dhT).  flags must be 0.  Every chunk, headdim, dstate and dtype
 * of ssd_scan_fwd's support set; errors as for ssd_scan_bwd, reported before any HIP
 * call. */
size_t ssd_diag_bwd_workspace_bytes(const ssd_problem* p);
int ssd_diag_scan_bwd(const ssd_problem* p, const void* x, const float* dt, const float* A,
                      const void* B, const void* C, const float* D, const float* h0, const void* dy,
                      const float* dhT, void* dx, float* ddt, float* dA, void* dB, void* dC, float* dD,
                      float* dh0, void* ws, size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* ssd_status_string(int status);

/* SSD_VERSION of the built library. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
