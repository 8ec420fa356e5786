/*
 * mamba2_ssd.h - C ABI of the MI355X (gfx950) chunked Mamba-2 SSD forward pass.
 *
 * The method (pages: devotd.net news item on the Mamba-2 CUDA Tile
 * forward-pass kernels, sections 1-2; disconfirmai.com "Jane Street ML
 * Engineers Map Mamba-2 Recurrent State Computation to Tensor Cores with
 * cuTile", abstract and body) evaluates the recurrence
 *
 *     h_t = exp(dt_t * A) * h_{t-1} + dt_t * x_t (outer) B_t      state [P, N]
 *     y_t = h_t . C_t + D * x_t
 *
 * chunk by chunk: an in-chunk log-space cumulative sum of dt*A
 * (chunk_cumsum), per-chunk B X^T contractions and the decayed jump that
 * carries the state across chunks in order (fwd_pass_state, exposed here as
 * chunk_state + state_passing), and the fused output stage (compute_out,
 * exposed as chunk_scan): carried-state term C.h, the causally masked,
 * decay-weighted C B^T interaction times X, and the D skip.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Sizes: B = batch, L = seqlen, H = nheads, P = headdim, N = dstate,
 *        G = ngroups (H % G == 0; head h reads B/C group h / (H/G)),
 *        Q = chunk_size, nc = ceil(L / Q).
 * Layouts (contiguous, row-major, innermost last):
 *        x, y          [B, L, H, P]
 *        dt            [B, L, H]
 *        A, D          [H]                 float32
 *        B, C          [B, L, G, N]
 *        init/final    [B, H, P, N]        float32
 *        dA_cs, dt_T   [B, H, nc, Q]       float32 (time contiguous)
 *        states        [B, nc, H, P, N]    float32
 * dtype: MAMBA2_DTYPE_F32  - every tensor is float32;
 *        MAMBA2_DTYPE_BF16 - x, dt, B, C and y are bfloat16; A, D, the
 *                            cumsum outputs, states and the initial/final
 *                            state are float32.
 * Positions past L inside the last chunk are treated as zero input (dt = 0,
 * x = 0), following the zero-padded tile loads of the pages' chunk_cumsum
 * figure; y is written only for t < L.
 * Memory: every pointer is device memory owned by the caller.  The library
 * never allocates or frees and keeps no pointer after a call returns.  Every
 * pointer must be 16-byte aligned (MAMBA2_ERR_ALIGN otherwise).
 * Streams: `stream` is a hipStream_t (NULL = default stream).  Every call
 * only enqueues work on that stream; there is no device synchronisation
 * inside.  Stages given the same stream run in call order.
 * Errors: every int-returning call returns a mamba2_status.  Arguments are
 * checked on the host before anything is enqueued; on a failed check nothing
 * is launched and no output is touched.  MAMBA2_ERR_HIP reports a launch
 * failure, with the HIP error text in mamba2_last_error().  No C++ exception
 * crosses this interface.  Calls are thread-safe: the library keeps no
 * mutable global state except the calling thread's last-error message.
 * Preconditions that are not checked (checking would cost a pass over the
 * data): A <= 0, dt >= 0 and every input finite - the decay regime the
 * method describes (decay rate times time interval).
 * Supported sizes: Q in {16, 32, 64, 128, 256} for float32 and
 * {64, 128, 256} for bfloat16; bfloat16 also needs P and N multiples of 16
 * with P <= 128 and N <= 512 (the MFMA tile is 16 wide; larger states do not
 * fit one workgroup's registers and LDS).  The fastest kernels (shared B/C
 * operands across the heads of a group, spans of chunks) cover bfloat16
 * with P = 64 and N in {64, 128, 256, 512}; other supported sizes run
 * per-head kernels.  Other sizes give MAMBA2_ERR_UNSUPPORTED.
 */
#ifndef MAMBA2_SSD_H_
#define MAMBA2_SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MAMBA2_OK = 0,
  MAMBA2_ERR_NULL = 1,        /* a required pointer is NULL */
  MAMBA2_ERR_SHAPE = 2,       /* non-positive size, H % G != 0, overflow */
  MAMBA2_ERR_DTYPE = 3,       /* unknown dtype code */
  MAMBA2_ERR_UNSUPPORTED = 4, /* valid but not implemented size */
  MAMBA2_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
  MAMBA2_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  MAMBA2_ERR_HIP = 7          /* a HIP launch failed */
} mamba2_status;

typedef enum { MAMBA2_DTYPE_F32 = 0, MAMBA2_DTYPE_BF16 = 1 } mamba2_dtype;

typedef struct {
  int64_t batch;      /* B  >= 1 */
  int64_t seqlen;     /* L  >= 1 */
  int64_t nheads;     /* H  >= 1 */
  int64_t headdim;    /* P  >= 1 */
  int64_t dstate;     /* N  >= 1 */
  int64_t ngroups;    /* G  >= 1, divides H */
  int64_t chunk_size; /* Q */
  int32_t dtype;      /* mamba2_dtype */
  int32_t reserved;   /* must be 0 */
} mamba2_dims;

/* Checks `dims` alone (host only, touches no device).  Returns MAMBA2_OK when
 * every entry point supports these sizes. */
int mamba2_validate(const mamba2_dims* dims);

/*
 * chunk_cumsum (devotd.net page, section 2 and its code figure): for every
 * batch b, head h and chunk c, the inclusive cumulative sum of A[h]*dt along
 * the chunk's time steps, multiplied by log2(e) so consumers use base-2
 * exponentials:
 *     dA_cs[b,h,c,i] = log2(e) * sum_{j<=i} A[h] * dt[b, c*Q+j, h]
 *     dt_T[b,h,c,i]  = dt[b, c*Q+i, h]        (0 past L)
 * Inputs dt (dtype of dims), A (float32).  Outputs float32 [B,H,nc,Q],
 * fully overwritten.  The sum is evaluated as a tree (wavefront scan).
 */
int mamba2_chunk_cumsum(const mamba2_dims* dims, const void* dt, const float* A,
                        float* dA_cs, float* dt_T, void* stream);

/*
 * chunk_state (first half of fwd_pass_state; disconfirmai.com page, body:
 * the jump formula's B X^T product with rows pre-scaled by exponentials): the
 * state each chunk reaches from a zero start,
 *     states[b,c,h,p,n] = sum_{j in chunk} 2^(cs[Q-1] - cs[j]) * dt_j
 *                                          * x[b,cQ+j,h,p] * B[b,cQ+j,g,n]
 * with cs = dA_cs[b,h,c,:], dt_j = dt_T[b,h,c,j].  Inputs x, B (dtype of
 * dims), dA_cs and dt_T from mamba2_chunk_cumsum.  Output states float32
 * [B,nc,H,P,N], fully overwritten.
 */
int mamba2_chunk_state(const mamba2_dims* dims, const void* x, const void* B,
                       const float* dA_cs, const float* dt_T, float* states,
                       void* stream);

/*
 * state_passing (second half of fwd_pass_state; devotd.net page, section 2:
 * the state at each chunk start and after the last chunk, chunks in order,
 * independent parts of the state in parallel).  In place over `states`:
 *     run = init_state (zeros if NULL)
 *     for c in 0..nc-1:  S = states[b,c,h];  states[b,c,h] = run;
 *                        run = 2^(dA_cs[b,h,c,Q-1]) * run + S
 *     final_state = run                   (not written if NULL)
 * On entry states holds chunk_state's per-chunk states; on return it holds
 * the state at the start of every chunk.  All float32.
 */
int mamba2_state_passing(const mamba2_dims* dims, float* states, const float* dA_cs,
                         const float* init_state, float* final_state, void* stream);

/*
 * chunk_scan = compute_out (devotd.net page, section 2; disconfirmai.com
 * page, abstract): outputs of every chunk from its start state, fused so the
 * Q x Q interaction matrix never reaches memory.  For token i of chunk c,
 * head h, group g:
 *     y[i,p] = 2^cs[i] * sum_n C[i,n] h[p,n]
 *            + sum_{j<=i} (sum_n C[i,n] B[j,n]) 2^(cs[i]-cs[j]) dt_j x[j,p]
 *            + D[h] x[i,p]
 * with h = states[b,c,h] (chunk-start states from mamba2_state_passing),
 * cs = dA_cs[b,h,c,:], dt = dt_T[b,h,c,:].  D may be NULL (no skip term).
 * Output y (dtype of dims) [B,L,H,P]; rows t >= L are not written.
 */
int mamba2_chunk_scan(const mamba2_dims* dims, const void* x, const void* B,
                      const void* C, const float* dA_cs, const float* dt_T,
                      const float* states, const float* D, void* y, void* stream);

/* Bytes of device workspace mamba2_ssd_forward needs for `dims` (0 if the
 * dims are invalid).  Host only. */
size_t mamba2_ssd_workspace_bytes(const mamba2_dims* dims);

/*
 * The whole forward pass: chunk_cumsum -> fwd_pass_state -> chunk_scan on
 * `stream`, intermediates in the caller's workspace (at least
 * mamba2_ssd_workspace_bytes(dims) bytes, 256-byte aligned; contents on
 * return are unspecified).  init_state and D may be NULL; final_state may
 * be NULL (not written).  Outputs y [B,L,H,P] (dtype of dims) and
 * final_state [B,H,P,N] float32.  fwd_pass_state runs as chunk_state ->
 * state_passing, or, for bfloat16 with headdim 64, dstate 64/128/256/512
 * and enough (batch, head, span) work to fill the device, over spans of 8
 * (or 4) chunks (devotd.net news item, section 2: the same jump across
 * chunks, taken span by span): the state after each span from a zero start,
 * the jump across spans, then each span replayed from its start state.  At
 * dstate 256 and 512 the replay writes bfloat16 chunk-start states for
 * chunk_scan; at dstate 64 and 128, with an even number of heads per group,
 * one kernel replays each span and forms its outputs in the same pass, so
 * the chunk-start states stay on chip.  At dstate 512 the output stage runs
 * over two halves of the state columns and the first hands its partial y to
 * the second in bfloat16 (one more rounding of that partial).  All forms
 * give the same result up to rounding.
 */
int mamba2_ssd_forward(const mamba2_dims* dims, const void* x, const void* dt,
                       const float* A, const void* B, const void* C, const float* D,
                       const float* init_state, void* y, float* final_state,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * mamba2_ssd_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, with the workspace taken from a static
 * device array of MAMBA2_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends.  The caller passes inputs and
 * outputs only; the call allocates and frees nothing.  Sizes whose
 * mamba2_ssd_workspace_bytes exceed the array are rejected with
 * MAMBA2_ERR_WORKSPACE before any launch.  The array's address on the
 * current device is looked up once per device (hipGetSymbolAddress) and
 * kept; the current device must be the one the pointers and the stream
 * belong to.  Every call on one GPU shares that GPU's array and it keeps the
 * last call's contents (no part needs clearing: each piece is written
 * before it is read within a call), so calls that overlap on one GPU - on
 * different streams, or from different threads - race and give wrong
 * results: order them on one stream or otherwise.  Other rules as for
 * mamba2_ssd_forward.
 */
#define MAMBA2_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

int mamba2_ssd_forward_noalloc(const mamba2_dims* dims, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* init_state, void* y, float* final_state,
                               void* stream);

/*
 * Same as mamba2_ssd_forward, then waits for the work to finish and writes
 * the device time of each stage in milliseconds to stage_ms[0..3]
 * (chunk_cumsum, chunk_state, state_passing, chunk_scan; on the span path
 * the second and third are the span-end kernel and the jump across spans
 * plus the replay), measured with HIP events recorded on `stream` between
 * the launches.  For measurement only:
 * it creates and destroys five events and blocks the calling thread.
 */
int mamba2_ssd_forward_profile(const mamba2_dims* dims, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* init_state, void* y, float* final_state,
                               void* workspace, size_t workspace_bytes, void* stream,
                               float* stage_ms);

/*
 * fwd_pass_state as one kernel, the pages' own second kernel (devotd.net news
 * item, section 2: the state at every chunk start and after the last chunk,
 * chunk order kept while independent parts of the state run in parallel;
 * disconfirmai.com, body: the jump formula with exponentially pre-scaled rows
 * of X): per state tile, walks the chunks in order with the running state in
 * float32 MFMA accumulators, so the per-chunk states never reach memory.
 * Inputs: x, B, dA_cs, dt_T (from mamba2_chunk_cumsum), init_state (NULL =
 * zeros).  Outputs: w_T [B,H,nc,Q] float32, the contraction weights
 * 2^(cs[Q-1] - cs[j]) * dt_j (written first, then read by the kernel);
 * chunk_start_states [B,nc,H,P,N] bfloat16 (round to nearest even);
 * final_state [B,H,P,N] float32.  Supported: bfloat16 with headdim 64,
 * dstate 64, 128 or 256 and chunk_size 64, 128 or 256 (UNSUPPORTED
 * otherwise).  The default forward (chunk_state + state_passing) is faster on
 * this chip; this path is the one-kernel form for callers that want it.
 */
int mamba2_fwd_pass_state(const mamba2_dims* dims, const void* x, const void* B,
                          const float* dA_cs, const float* dt_T, const float* init_state,
                          float* w_T, void* chunk_start_states, float* final_state,
                          void* stream);

/*
 * The whole forward through the one-kernel fwd_pass_state: chunk_cumsum ->
 * weights -> fwd_pass_state -> chunk_scan.  Same arguments, results (up to
 * rounding order) and workspace as mamba2_ssd_forward (at least
 * mamba2_ssd_workspace_bytes(dims)); final_state is required.  Sizes as for
 * mamba2_fwd_pass_state.
 */
int mamba2_ssd_forward_fused(const mamba2_dims* dims, const void* x, const void* dt,
                             const float* A, const void* B, const void* C, const float* D,
                             const float* init_state, void* y, float* final_state,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Recurrent single-token step: the constant-memory inference mode of the same
 * recurrence (pages: devotd.net news item, section 1 - a fixed-size hidden
 * state updated as tokens are processed; disconfirmai.com, abstract - the
 * recurrent state).  For one new token of every (batch, head), in place:
 *     state[b,h] = exp(dt[b,h] * A[h]) * state[b,h] + dt[b,h] * x[b,h] (outer) B[b,g]
 *     y[b,h]     = state[b,h] . C[b,g] + D[h] * x[b,h]          (g = h / (H/G))
 * i.e. one token of the forward pass, reading the state after the update.
 * dims: seqlen must be 1 (MAMBA2_ERR_SHAPE otherwise); chunk_size is not
 *       used but must be a supported value, as for every dims.
 * Layouts: x, y [B, H, P] (the forward's [B, L, H, P] with L = 1);
 *          dt [B, H]; B, C [B, G, N]; A, D [H] float32 (D may be NULL);
 *          state [B, H, P, N] float32, read and overwritten.
 * dtype as for the forward: bfloat16 makes x, dt, B, C and y bfloat16.
 * Every pointer 16-byte aligned, as everywhere (a per-token view sliced out
 * of a [B, L, ...] tensor usually is not: copy it).
 * Bound by HBM on the state (read once, written once).
 */
int mamba2_decode_step(const mamba2_dims* dims, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, float* state, void* y,
                       void* stream);

/*
 * Backward pass: gradients of a scalar loss through mamba2_ssd_forward.  The
 * pages publish no backward pass (disconfirmai.com, lead paragraph: the
 * forward speedups rest on one that is not yet published); this is the exact
 * derivative of the forward's chunked form (devotd.net news item, section 2),
 * for the loss whose gradients with respect to y and final_state are dy and
 * dfinal:
 *     dx, ddt, dB, dC   same layouts and dtype as x, dt, B, C
 *     dA [H], dD [H]    float32 (dD written only when D is non-NULL; it is
 *                       required then)
 *     dinit [B,H,P,N]   float32, may be NULL (not written); it is the
 *                       gradient with respect to init_state (whether or not
 *                       init_state is NULL, which means a zero start)
 * Inputs are the forward's (x, dt, A, B, C, D, init_state; D and init_state
 * may be NULL), dy [B,L,H,P] (dtype of dims) and dfinal [B,H,P,N] float32
 * (NULL = zero).  The forward quantities the gradients need are recomputed
 * inside (nothing from an earlier forward call is read).
 * Supported: every size the forward accepts.  bfloat16 with headdim 64 and
 * dstate 64, 128 or 256 with chunk_size 64, 128 or 256, or dstate 512 with
 * chunk_size 256, runs MFMA kernels; every other size (float32, other head
 * sizes, dstate 512 with shorter chunks and the other multiples of 16) runs
 * a generic path of float32 vector-ALU kernels without MFMA: exact to
 * float32 rounding, and much slower.  Workspace: at least
 * mamba2_ssd_backward_workspace_bytes(dims), 256-byte aligned, contents on
 * return unspecified.  Pointer, stream and error rules as for the forward.
 */
size_t mamba2_ssd_backward_workspace_bytes(const mamba2_dims* dims);

int mamba2_ssd_backward(const mamba2_dims* dims, const void* x, const void* dt, const float* A,
                        const void* B, const void* C, const float* D, const float* init_state,
                        const void* dy, const float* dfinal, void* dx, void* ddt, float* dA,
                        void* dB, void* dC, float* dD, float* dinit, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Same as mamba2_ssd_backward, then waits and writes the device time of each
 * of its eight stages in milliseconds to stage_ms[0..7]: chunk_cumsum,
 * chunk_state, state_passing (the recomputed forward states), adjoint
 * chunk_state, reverse state_passing, dB/dC kernel, dx kernel (at dstate 512
 * with the kernel forming dx's state term before it), dA/dD sums.
 * On the generic path stage 0 holds the whole pass and the others read 0.
 * For measurement only (creates events, blocks).
 */
int mamba2_ssd_backward_profile(const mamba2_dims* dims, const void* x, const void* dt,
                                const float* A, const void* B, const void* C, const float* D,
                                const float* init_state, const void* dy, const float* dfinal,
                                void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD,
                                float* dinit, void* workspace, size_t workspace_bytes,
                                void* stream, float* stage_ms);

/* Static description of a status code. */
const char* mamba2_status_string(int status);

/* Detail of the calling thread's most recent failure ("" if none). */
const char* mamba2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA2_SSD_H_ */
