/*
 * prnn.h - persistent basic-RNN forward recurrence for AMD Instinct MI355X (gfx950).
 *
 * The operation (a basic RNN layer; "persistent-rnn", section "Important
 * Constraints": basic RNN layers only):
 *
 *     H[t][b][i] = max(0, X[t][b][i] + sum_j W[i][j] * H[t-1][b][j]),   H[-1] = h0
 *
 * for t = 0 .. T-1, b = 0 .. B-1, i = 0 .. N-1.  X already holds the input
 * projection (and bias) of every timestep, computed before the recurrence
 * ("Optimizing Performance of Recurrent Neural Networks on GPUs", Abstract:
 * the single-layer stage takes the input-side product out of the sequential
 * loop).  The activation is ReLU.
 *
 * The recurrence runs as ONE persistent kernel per call: every workgroup loads
 * its rows of W once into registers and keeps them there for all T steps, so W
 * is never re-read from memory inside the time loop ("persistent-rnn", "What
 * This Project Does": weights cached in the register files instead of being
 * reloaded every step).  Workgroups exchange h_{t-1} once per step through a
 * small ring buffer whose words carry their own step tag, so no separate
 * barrier pass and no reset pass are needed between steps ("Sparse Persistent
 * RNNs: Squeezing Large Recurrent Networks On-Chip", table "Measured effects
 * reported in the paper": Lamport timestamps row).  W may be dense, or sparse
 * with the same number K of nonzeros in every row (same table: load-balanced
 * pruning row).
 *
 * Around the recurrence: prnn_project computes X for a whole sequence on the
 * matrix cores; prnn_forward_layer_* run a whole layer (projection, then the
 * recurrence); prnn_forward_stack_dense runs a stack of layers with the
 * layers at the same time on separate XCDs (same page, entire-network stage).
 *
 * API style follows a cuDNN-like library ("persistent-rnn", "Who Would Use
 * This"): an opaque handle, a status code from every call, caller-owned device
 * buffers, and asynchronous execution on a caller-provided stream.
 *
 * Conventions shared by every call below
 * --------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller.  The library
 *    reads the inputs, writes only the outputs each call names (H; X for
 *    prnn_project; the workspace Xbuf of layer and stack calls), and keeps no
 *    pointer after the work it enqueued has finished.  Buffers must stay
 *    valid until then.
 *  - All arrays are dense, row-major, with the last index fastest:
 *      W   [N][N]   W[i*N + j] = weight from input neuron j to output neuron i
 *      col [N][K]   int16 column indices of row i's nonzeros, each in [0, N)
 *      val [N][K]   values belonging to col
 *      X   [T][B][N] fp32 pre-activations
 *      h0  [B][N]   fp32 initial state, or NULL for zeros
 *      H   [T][B][N] fp32 output: H[t] is the state after consuming X[t]
 *    X, h0 and H need 4-byte alignment; W, col and val need the alignment of
    their element type (fp16 2 bytes, fp32 4, int16 2).  A dense W that is
    16-byte aligned is loaded with vector loads, any other W element by
    element (the result is the same).
 *  - Calls are asynchronous: a SUCCESS return means the work was enqueued on
 *    `stream` (NULL = the default stream).  An error found while a kernel
 *    runs (a step that never completes within the watchdog limit, or a value
 *    outside the fp16 range where a path needs it) is sticky: the failing
 *    kernel marks a host-visible copy of the handle's status (pinned host
 *    memory), and the next call on the handle that enqueues work (forward,
 *    layer, stack, projection or floor), prnn_synchronize() or prnn_destroy(),
 *    whichever comes first, returns PRNN_STATUS_EXECUTION_FAILED without
 *    waiting for the GPU; that call enqueues nothing.  The failure is
 *    reported once; the handle is then usable again (its exchange ring is
 *    reset before the next launch).  Calls enqueued after the failing one but
 *    before the failure reached the host (made while it was still running)
 *    return SUCCESS and do nothing: their kernels see the failure at entry and
 *    leave H as it was.  A call that enqueues several launches (layer and
 *    stack calls) and fails after the first leaves its outputs undefined.
 *  - One forward call may be in flight per handle at a time (the handle owns
 *    the exchange ring).  Use one handle per concurrently used stream.  A
 *    handle is not thread-safe.  Every call must be made with the handle's
 *    device current.
 *  - No C++ exception crosses this interface.
 */
#ifndef PRNN_H_
#define PRNN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct prnnContext* prnnHandle_t;

typedef enum {
  PRNN_STATUS_SUCCESS = 0,
  PRNN_STATUS_BAD_PARAM = 1,        /* invalid argument; nothing was enqueued            */
  PRNN_STATUS_NOT_SUPPORTED = 2,    /* valid, but outside what fits on chip / this GPU   */
  PRNN_STATUS_ALLOC_FAILED = 3,     /* device or pinned allocation failed                */
  PRNN_STATUS_EXECUTION_FAILED = 4, /* an earlier launch failed on the GPU (sticky, below) */
  PRNN_STATUS_INTERNAL_ERROR = 5,   /* a HIP runtime call failed                         */
  PRNN_STATUS_MAX_ENUM = 0x7FFFFFFF  /* not a value: keeps every int in the type's range */
} prnnStatus_t;

typedef enum {
  PRNN_DATA_FLOAT = 0, /* fp32 */
  PRNN_DATA_HALF = 1,  /* fp16 (IEEE binary16); products and sums are taken in fp32 */
  PRNN_DATA_MAX_ENUM = 0x7FFFFFFF  /* not a value: keeps every int in the type's range */
} prnnDataType_t;

/* How workgroups exchange h_{t-1} each step.
 *  DIRECT: every workgroup reads the whole of h_{t-1} from a device-coherent
 *          ring that every producer writes.
 *  RELAY:  each workgroup first copies one slice of h_{t-1} from that ring
 *          into a copy of the ring kept per XCD (in that XCD's L2), and then
 *          reads all of h_{t-1} from its XCD's copy: h crosses between XCDs
 *          once per XCD instead of once per workgroup.  Needs a grid that is
 *          a multiple of 8 workgroups dealt round-robin over the 8 XCDs.
 *  AUTO:   RELAY for grids of 192 or more workgroups when possible, else
 *          DIRECT (the default). */
typedef enum {
  PRNN_EXCHANGE_AUTO = 0,
  PRNN_EXCHANGE_DIRECT = 1,
  PRNN_EXCHANGE_RELAY = 2,
  PRNN_EXCHANGE_MAX_ENUM = 0x7FFFFFFF  /* not a value: keeps every int in the type's range */
} prnnExchange_t;

/* How the recurrence is laid out on the GPU.
 *  SPREAD: up to one workgroup per compute unit over the whole GPU; each
 *          workgroup owns some rows of W and runs one wave per batch row
 *          (all batch rows share the workgroup's resident rows).  h_{t-1}
 *          crosses between XCDs every step (see prnnExchange_t).
 *  TEAM:   each of the 8 XCDs runs one batch row's whole recurrence with up
 *          to 32 workgroups of 8 waves (12 or 16 for sparse fp16 layers that
 *          would hold more than 8 rows per wave); a wave owns a few rows of W.  h_{t-1}
 *          is exchanged inside the XCD's L2 only.  With B < 8 the remaining
 *          XCDs compute nothing; they only mark their exchange memory as
 *          written for the call's last steps.  Holds W once per XCD: for
 *          dense fp16 W up to N = 2560, fp32 W up to N = 1792.
 *          Larger dense fp16 layers ("persistent-rnn", "Important
 *          Constraints": the layer size is bounded by what stays on chip)
 *          split each batch row over 2 XCDs (N <= 3584, B <= 4) or 4 XCDs
 *          (N <= 5120, B <= 2), each holding a part of the rows; the parts
 *          exchange their rows of h_{t-1} through device-coherent memory
 *          every step.  EXACT math only (SPLIT and HALF: NOT_SUPPORTED), no
 *          phase tracing (NOT_SUPPORTED while tracing is on).  Heavy sparse
 *          fp16 layers split the same way over 2 XCDs (see
 *          prnn_set_xcds_per_row).
 *  AUTO:   TEAM when an instance fits, else SPREAD (the default). */
typedef enum {
  PRNN_LAYOUT_AUTO = 0,
  PRNN_LAYOUT_SPREAD = 1,
  PRNN_LAYOUT_TEAM = 2,
  PRNN_LAYOUT_MAX_ENUM = 0x7FFFFFFF  /* not a value: keeps every int in the type's range */
} prnnLayout_t;

/* How the dense fp16 recurrence forms W h_{t-1}.
 * EXACT: fp32 h times the exactly widened fp16 weights, fp32 sums (VALU).
 * SPLIT: h enters as two fp16 values, hi = fp16(h) and lo = fp16(h - hi), and
 *   the matrix cores form W hi + W lo with exact products and fp32 sums: the
 *   product sees h to about 2^-22 of |h| (fp32 h carries 2^-24).  Needs
 *   |h| < 65504; a larger value makes the call report EXECUTION_FAILED.
 *   TEAM layout, fp16 W, N <= 2048 only (else NOT_SUPPORTED).
 * HALF: h_{t-1} is rounded to fp16 (to nearest, ties to even) before the
 *   product, and each instruction adds two fp16 x fp16 products (exact in
 *   fp32) to the fp32 sums: half the multiply-adds of EXACT.  The product sees
 *   h to 2^-11 of |h|, the relative precision the fp16 weights themselves
 *   carry; X, h0, H, the sums, the ReLU and the exchanged state stay fp32.
 *   Needs every h (and h0) to round to a finite fp16 (|h| < 65520); a larger
 *   value makes the call report EXECUTION_FAILED.  TEAM layout, fp16 W,
 *   N <= 2560 only (else NOT_SUPPORTED).  Blocked and fused stacks use EXACT;
 *   a layer-by-layer stack follows this setting.
 * AUTO: EXACT.  fp32 weights and sparse layers always use EXACT. */
typedef enum {
  PRNN_MATH_AUTO = 0,
  PRNN_MATH_EXACT = 1,
  PRNN_MATH_SPLIT = 2,
  PRNN_MATH_HALF = 3,
  PRNN_MATH_MAX_ENUM = 0x7FFFFFFF  /* not a value: keeps every int in the type's range */
} prnnMath_t;

/* Launch plan of the last forward call on a handle (for tests and reports). */
typedef struct {
  int layout;        /* PRNN_LAYOUT_SPREAD or PRNN_LAYOUT_TEAM                 */
  int grid;          /* workgroups launched                                    */
  int waves_per_wg;  /* SPREAD: min(B, 4), one wave per batch row; TEAM: 8,
                        or 12 / 16 for sparse fp16 layers (and the floor)
                        that would hold more than 8 rows per wave at 8      */
  int rows_per_wave; /* largest number of W rows one wave keeps resident       */
  int rmax;          /* compiled row capacity of the kernel instance           */
  int chunks;        /* dense: 256-column chunk capacity; sparse: 64-pair slots */
  int lds_bytes;     /* dynamic LDS per workgroup                              */
  int relay_slice;   /* SPREAD: words of h each workgroup relays (0: DIRECT)   */
  uint64_t first_step; /* ring step counter of the call's first timestep       */
  int math;          /* PRNN_MATH_EXACT, PRNN_MATH_HALF or PRNN_MATH_SPLIT
                        (SPLIT: rows_per_wave and rmax count rows per
                        workgroup)                                            */
  int xcds_per_row;  /* TEAM: XCDs serving one batch row (1; 2 or 4 for dense
                        fp16 layers beyond one XCD's registers); SPREAD: 0   */
} prnnPlanInfo_t;

/* HIP graphs: forward, layer, stack and floor calls may be captured (stream
 * capture).  A captured call resets the handle's exchange state inside the
 * captured sequence (a fill kernel, no memset) and counts its steps from 0,
 * so every replay starts afresh; after the first capture every call on the
 * handle does so (one extra small kernel per call).  Nothing is allocated
 * while capturing: a call whose exchange buffer would have to grow returns
 * NOT_SUPPORTED, so run one call of the largest shape before capturing.  As
 * for any call, one graph replay or call at a time per handle. */

/* Environment: PRNN_LOG set to anything but "" or "0" when a handle is
 * created makes that handle print one line to stderr per launch (its plan:
 * layout, grid, waves per workgroup, rows per wave, kernel instance, LDS,
 * math) and one per failed run when it is reported.  Otherwise the
 * library prints nothing. */

/* Creates a handle bound to the current HIP device.
 * Returns NOT_SUPPORTED if the device is not gfx950, ALLOC_FAILED if the small
 * internal buffers (the device status word and its 64-byte pinned host
 * mirror) cannot be allocated, BAD_PARAM if handle is NULL. */
prnnStatus_t prnn_create(prnnHandle_t* handle);

/* Waits for all work the handle enqueued, frees its buffers and the handle.
 * NULL is accepted (SUCCESS).  Returns EXECUTION_FAILED if a run on this handle
 * failed and that was not yet reported, else SUCCESS. */
prnnStatus_t prnn_destroy(prnnHandle_t handle);

/* Dense W.  w_type selects fp32 or fp16 W; X, h0, H are fp32.
 * BAD_PARAM: NULL handle/W/X/H (h0 may be NULL), N < 1, B not in [1, 8],
 *            T < 0, bad w_type, misaligned pointer, X and H overlapping.
 * NOT_SUPPORTED: W does not fit in the register files of the grid, or the
 *            cooperative grid cannot be resident.
 * T == 0 enqueues nothing and returns SUCCESS. */
prnnStatus_t prnn_forward_dense(prnnHandle_t handle, int N, int B, int T,
                                prnnDataType_t w_type, const void* W,
                                const float* X, const float* h0, float* H,
                                hipStream_t stream);

/* Row-balanced sparse W: row i has exactly K nonzeros, at columns col[i][k]
 * with values val[i][k].  Columns within a row must be distinct (a repeated
 * column is summed, like the dense equivalent with the values added).
 * BAD_PARAM: as for dense, plus K not in [1, N]; N > 32767 (int16 columns).
 * NOT_SUPPORTED: the nonzeros or the staged h do not fit on chip.
 * Column indices outside [0, N) are not checked on the device; they read
 * zeros (buffer bounds checking), never memory outside the staging area. */
prnnStatus_t prnn_forward_sparse(prnnHandle_t handle, int N, int B, int T, int K,
                                 const int16_t* col, prnnDataType_t val_type, const void* val,
                                 const float* X, const float* h0, float* H,
                                 hipStream_t stream);

/* Sparse W whose rows hold different numbers of nonzeros ("Sparse Persistent
 * RNNs: Squeezing Large Recurrent Networks On-Chip", table "Measured effects
 * reported in the paper", load-balanced pruning row: unbalanced pruning).
 * col and val are [N][K] as for prnn_forward_sparse, K the width of the
 * longest row; row i is its first row_len[i] pairs (row_len: int32 [N],
 * device memory, 4-byte aligned, read by the call on `stream`; lengths below
 * 0 count as 0 and above K as K).  Pairs past a row's length are never used,
 * whatever they hold.  Columns as for prnn_forward_sparse.  The rows are dealt
 * to the waves by length, so a step costs the pairs that are there rather than
 * N times the longest row.  TEAM layout, fp16 values, K <= 1024 (else
 * NOT_SUPPORTED); a small ordering kernel runs before the recurrence (the
 * handle keeps an [N] int32 buffer for it, grown outside stream capture).
 * Where one XCD's waves cannot hold the rows (the longest row's slots of 64
 * pairs times the rows per wave, e.g. rows of 1010 pairs at N = 2304), or
 * with prnn_set_xcds_per_row(2), each batch row runs on two XCDs (B <= 4),
 * each ordering and dealing the rows of its part; NOT_SUPPORTED when neither
 * form holds the rows.  Such rows, each slot run for the rows that have it,
 * can cost more than the row-balanced call on the same arrays padded with
 * zero values: the rows of a wave's slots run as short batches of gathers in
 * sequence.
 * BAD_PARAM: as for prnn_forward_sparse, plus a NULL or misaligned row_len. */
prnnStatus_t prnn_forward_sparse_rows(prnnHandle_t handle, int N, int B, int T, int K,
                                      const int16_t* col, prnnDataType_t val_type, const void* val,
                                      const int32_t* row_len, const float* X, const float* h0, float* H,
                                      hipStream_t stream);

/* Input projection of a layer ("Optimizing Performance of Recurrent Neural
 * Networks on GPUs", Abstract, single-layer stage: the input-side product of
 * every timestep is independent of the state, so a whole sequence's is one
 * matrix product computed before the recurrence):
 *
 *   X[m][n] = bias[n] + sum_i U[n][i] * x[m][i],   0 <= m < M, 0 <= n < N,
 *
 * with x [M][I] row-major (M = T * B rows for a sequence [T][B][I]), U [N][I]
 * row-major (row n feeds output neuron n, like W), bias [N] or NULL (zeros)
 * and X [M][N] fp32 (the pre-activations the forward calls take).  All are
 * device pointers owned by the caller; only X is written.
 * u_type: PRNN_DATA_HALF (PRNN_DATA_FLOAT returns NOT_SUPPORTED).
 * x_type: PRNN_DATA_FLOAT or PRNN_DATA_HALF.  Runs on the matrix cores with
 * fp32 accumulation.  An fp32 x enters as fp16 hi (x with the low 13 bits
 * of its significand cleared) plus lo = fp16(x - hi), whose products with the
 * fp16 U are exact: x is seen to about 2^-22 of |x|.  |x| >= 2^16 (infinities
 * included) does not fit the split; X is then not valid and the failure is
 * reported as EXECUTION_FAILED (sticky, see the conventions above).  A NaN in
 * x gives NaN in the X rows that use it.
 * BAD_PARAM: NULL handle, x, U or X (when M > 0); M < 0, N < 1, I < 1;
 * unknown types; x, U, bias or X not aligned to their element size; X
 * overlapping x, U or bias.  NOT_SUPPORTED: fp32 U; x or U over 4 GiB.
 * M == 0 enqueues nothing and returns SUCCESS.  Asynchronous on `stream`. */
prnnStatus_t prnn_project(prnnHandle_t handle, int M, int N, int I,
                          prnnDataType_t x_type, const void* x,
                          prnnDataType_t u_type, const void* U, const float* bias,
                          float* X, hipStream_t stream);

/* One whole layer: prnn_project of the input sequence x [T][B][I] into the
 * caller's workspace Xbuf [T][B][N] (fp32), then the dense recurrence over it
 * (prnn_forward_dense with X = Xbuf), both on `stream`.  Every argument is
 * checked, and the recurrence planned, before anything is enqueued; the
 * errors are those of the two calls, plus BAD_PARAM when Xbuf overlaps h0 or
 * W.  T == 0 enqueues nothing and returns SUCCESS. */
prnnStatus_t prnn_forward_layer_dense(prnnHandle_t handle, int N, int I, int B, int T,
                                      prnnDataType_t x_type, const void* x,
                                      prnnDataType_t u_type, const void* U, const float* bias,
                                      prnnDataType_t w_type, const void* W,
                                      const float* h0, float* Xbuf, float* H,
                                      hipStream_t stream);

/* The same with a row-balanced sparse recurrent matrix (as in
 * prnn_forward_sparse); BAD_PARAM also when Xbuf overlaps col or val. */
prnnStatus_t prnn_forward_layer_sparse(prnnHandle_t handle, int N, int I, int B, int T, int K,
                                       prnnDataType_t x_type, const void* x,
                                       prnnDataType_t u_type, const void* U, const float* bias,
                                       const int16_t* col, prnnDataType_t val_type, const void* val,
                                       const float* h0, float* Xbuf, float* H,
                                       hipStream_t stream);

/* A stack of L dense fp16 layers of width N as one wavefront ("Optimizing
 * Performance of Recurrent Neural Networks on GPUs", Abstract, entire-network
 * stage):
 *
 *   H[0][t]   = max(0, bias[0] + U[0] x[t] + W[0] H[0][t-1])
 *   H[l][t]   = max(0, bias[l] + U[l] H[l-1][t] + W[l] H[l][t-1]),  l >= 1
 *   H[l][-1]  = h0[l] (zeros if h0 or h0[l] is NULL)
 *
 * Layer l + 1's step t needs only layer l's step t and its own step t - 1,
 * so the layers run at the same time on separate XCDs (layer l, batch row b
 * on XCD l B + b; hence L B <= 8), keeping their weights in registers
 * widened to fp32 (prnnStackMode_t: in blocks of steps, layer l + 1 one block
 * behind layer l, each launch computing its blocks' input products itself
 * before the recurrence; or fused per step).  Where the weights do not fit
 * (N > 1792) the layers run one after another (prnn_forward_layer_dense
 * each, with layer l's output as layer l + 1's input).  x [T][B][I] (fp32 or
 * fp16); U[0] [N][I], U[l >= 1] [N][N], W[l] [N][N], all fp16, 16-byte
 * aligned; bias[l] [N] or NULL; Xbuf [T][B][N] fp32 workspace (written by
 * the fused mode and the layer-by-layer mode with layer 0's, or each layer's,
 * input product; the blocked mode does not use it); H[l] [T][B][N] fp32
 * outputs.  U, bias, W, h0 and H are host arrays of L device pointers (bias
 * and h0 may be NULL arrays).  All device buffers are the caller's.  H[0] ..
 * H[L-1] (blocked) or H[0] .. H[L-2] (fused) also carry intermediate values
 * (the layer's projected input, or a not-yet-written marker) before the
 * results overwrite them.  Not traced.
 * BAD_PARAM: NULL handle/arrays/pointers, L < 1, N < 1, I < 1, B outside
 * [1, 8], T < 0, unknown x_type, misalignment, any output overlapping any
 * input, the workspace or another output, the workspace overlapping an
 * input.  NOT_SUPPORTED: L B > 8 or L > 8, sizes over 4 GiB, and what
 * prnn_project or (one layer after another) prnn_forward_dense does not
 * support.  EXECUTION_FAILED (sticky, at the next call; see the conventions):
 * a bounded wait expired, or x exceeded the fp16 range of its split.
 * T == 0 enqueues nothing and returns SUCCESS. */
/* How prnn_forward_stack_dense runs the layers (see there).
 * BLOCKED: blocks of about 64 steps, layer l one block behind layer l - 1;
 *   a launch starts with its blocks' input products (each workgroup its own
 *   rows, on the matrix cores) and then runs the recurrence.
 * FUSED: one launch; each layer l >= 1 forms U_l H_{l-1}[t] itself at every
 *   step (N <= 1280).
 * LAYERS: one layer after another (prnn_forward_layer_dense each).
 * AUTO: BLOCKED where an instance fits (N <= 1792), else LAYERS. */
typedef enum {
  PRNN_STACK_AUTO = 0,
  PRNN_STACK_BLOCKED = 1,
  PRNN_STACK_FUSED = 2,
  PRNN_STACK_LAYERS = 3,
  PRNN_STACK_MAX_ENUM = 0x7FFFFFFF  /* not a value: keeps every int in the type's range */
} prnnStackMode_t;

/* Stack mode for later calls (default AUTO).  A forced mode the shape
 * cannot use makes stack calls return NOT_SUPPORTED.  BAD_PARAM for an
 * unknown mode. */
prnnStatus_t prnn_set_stack_mode(prnnHandle_t handle, prnnStackMode_t mode);

prnnStatus_t prnn_forward_stack_dense(prnnHandle_t handle, int L, int N, int I, int B, int T,
                                      prnnDataType_t x_type, const void* x,
                                      const void* const* U, const float* const* bias,
                                      const void* const* W, const float* const* h0,
                                      float* Xbuf, float* const* H, hipStream_t stream);

/* A stack of L row-balanced sparse layers of width N (the entire-network
 * stage of "Optimizing Performance of Recurrent Neural Networks on GPUs",
 * Abstract, over the sparse layers of "Sparse Persistent RNNs: Squeezing
 * Large Recurrent Networks On-Chip"):
 *
 *   H[0]     = layer(x,        U[0], bias[0], col[0], val[0], h0[0])
 *   H[l]     = layer(H[l - 1], U[l], bias[l], col[l], val[l], h0[l]),  l >= 1
 *
 * where layer() is prnn_forward_layer_sparse (projection into Xbuf, then the
 * recurrence).  The layers run one after another (no wavefront).  x
 * [T][B][I] (fp32 or fp16); U[0] [N][I], U[l >= 1] [N][N] fp16; col[l] int16
 * [N][K] and val[l] [N][K] (val_type fp16 or fp32) as for
 * prnn_forward_sparse; bias[l] [N] or NULL; h0[l] [B][N] or NULL; Xbuf
 * [T][B][N] fp32 workspace; H[l] [T][B][N] fp32 outputs.  U, bias, col, val,
 * h0 and H are host arrays of L device pointers (bias and h0 may be NULL
 * arrays).  All device buffers are the caller's.
 * BAD_PARAM: NULL handle/arrays/pointers, L < 1, N < 1, I < 1, B outside
 * [1, 8], T < 0, K outside [1, N], N > 32767, unknown x_type or val_type,
 * misalignment, any output overlapping any input, the workspace or another
 * output, the workspace overlapping an input; nothing is enqueued then.
 * NOT_SUPPORTED: what prnn_forward_layer_sparse does not support.
 * EXECUTION_FAILED as for the other calls.  T == 0 enqueues nothing. */
prnnStatus_t prnn_forward_stack_sparse(prnnHandle_t handle, int L, int N, int I, int B, int T, int K,
                                       prnnDataType_t x_type, const void* x,
                                       const void* const* U, const float* const* bias,
                                       const int16_t* const* col, prnnDataType_t val_type,
                                       const void* const* val, const float* const* h0,
                                       float* Xbuf, float* const* H, hipStream_t stream);

/* The exchange and step protocol of a dense call with the same N, B and T and
 * the same grid, without weights or arithmetic: the per-step floor that
 * synchronisation alone costs.  Writes H (values are step numbers, not a
 * recurrence).  Same errors as prnn_forward_dense. */
prnnStatus_t prnn_sync_floor(prnnHandle_t handle, int N, int B, int T, float* H,
                             hipStream_t stream);

/* Waits for `stream`, then reports whether any run on the handle failed
 * (EXECUTION_FAILED: a wait hit the watchdog, or a value left the fp16 range
 * of a path that needs it) and that failure has not been reported yet. */
prnnStatus_t prnn_synchronize(prnnHandle_t handle, hipStream_t stream);
/* (After a reported failure the handle is usable again: its exchange ring is
 * reset before the next forward call.) */

/* Number of workgroups for later calls (0 = automatic: up to one per compute
 * unit).  In the TEAM layout it must be a multiple of 8 (8 XCDs x workgroups
 * per XCD).  BAD_PARAM if negative. */
prnnStatus_t prnn_set_grid(prnnHandle_t handle, int workgroups);

/* Waves per workgroup of the TEAM layout for later calls: 0 (default) =
 * automatic (for sparse fp16 layers that would hold more than 8 rows per
 * wave at 8 waves: 12, or first 16 above 16 rows, where an instance of that
 * count fits, else 8; the floor picks 12 or 16 by the same row counts; 8
 * otherwise), 8, 12 or 16.  12 and 16 are
 * offered to sparse fp16 layers and to prnn_sync_floor only; a forced count
 * that the call cannot use makes it return NOT_SUPPORTED (or fall back to the
 * SPREAD layout under LAYOUT_AUTO).  BAD_PARAM for any other value. */
prnnStatus_t prnn_set_team_waves(prnnHandle_t handle, int waves);

/* XCDs per batch row of dense fp16 layers in the TEAM layout, for later
 * calls: 0 = automatic (the default: one XCD per batch row where the team
 * instances hold the layer, else the fewest XCDs of a split that holds it),
 * 1, 2 or 4 (2: B <= 4, 4: B <= 2; see prnnLayout_t).  A forced width that
 * the call cannot use makes it return NOT_SUPPORTED (or fall back to the
 * SPREAD layout under LAYOUT_AUTO).  Row-balanced sparse fp16 layers take 1
 * or 2 (B <= 4; 4: NOT_SUPPORTED); automatically 2 where one XCD's waves
 * would each hold more than 60 slots of 64 pairs (e.g. 5 % at N = 5760) or
 * where no one-XCD instance holds the rows, else 1.  prnn_sync_floor runs a forced width (with the wave count of
 * prnn_set_team_waves, 8 or 12), else the width of the dense fp16 layer of
 * the same N and B.  Sparse rows of unequal length take 1 or 2 as well
 * (automatically 2 only where one XCD cannot hold the rows).  fp32 W and
 * fp32 values always use one XCD per batch row.  BAD_PARAM for any other
 * value. */
prnnStatus_t prnn_set_xcds_per_row(prnnHandle_t handle, int xcds);

/* Exchange mode for later calls (default AUTO).  A forced RELAY that the
 * plan cannot use makes forward calls return NOT_SUPPORTED.  BAD_PARAM for an
 * unknown mode. */
prnnStatus_t prnn_set_exchange(prnnHandle_t handle, prnnExchange_t mode);

/* Layout for later calls (default AUTO).  A forced layout that the shape
 * cannot use makes forward calls return NOT_SUPPORTED.  BAD_PARAM for an
 * unknown layout.  The exchange mode applies to the SPREAD layout only. */
prnnStatus_t prnn_set_layout(prnnHandle_t handle, prnnLayout_t layout);

/* Math of the dense fp16 path for later calls (default AUTO; see
 * prnnMath_t).  BAD_PARAM for an unknown mode. */
prnnStatus_t prnn_set_math(prnnHandle_t handle, prnnMath_t mode);

/* Upper bound, in microseconds, on one wait for h_{t-1} (default 200000).
 * A wait that exceeds it stops the run and reports EXECUTION_FAILED. */
prnnStatus_t prnn_set_watchdog_us(prnnHandle_t handle, uint32_t microseconds);

/* How the persistent kernels are dispatched.  Every workgroup of such a
 * kernel waits for the others' rows of h_{t-1}, so all of them must be
 * resident at once.
 *  - COOPERATIVE: hipLaunchCooperativeKernel; the runtime checks that the
 *    grid fits the device and guarantees that it runs whole.
 *  - PLAIN: hipLaunchKernel.  The library checks that the grid fits the
 *    device with nothing else on it (occupancy of the kernel at its LDS size
 *    times the compute units; NOT_SUPPORTED otherwise) and that workgroups
 *    are dealt to the XCDs as the layouts assume.  Kernels of other streams
 *    or processes that hold compute units while such a launch starts can
 *    keep some of its workgroups waiting: the resident ones then stop when
 *    the watchdog expires and the call reports EXECUTION_FAILED (nothing
 *    hangs).  A stream's own kernels never overlap (streams are in order).
 * The kernels and results are the same either way; a plain launch starts
 * 10-20 us sooner after the kernel before it.  The default is PLAIN where
 * plain launches deal workgroups to the XCDs as the layouts assume (checked
 * when the handle is created), else COOPERATIVE.  Choosing a kind whose
 * placement check failed leaves the layouts that need it unavailable
 * (NOT_SUPPORTED from the calls that would use them).  BAD_PARAM for an
 * unknown kind. */
typedef enum {
  PRNN_LAUNCH_COOPERATIVE = 0,
  PRNN_LAUNCH_PLAIN = 1,
  PRNN_LAUNCH_MAX_ENUM = 0x7FFFFFFF  /* not a value: keeps every int in the type's range */
} prnnLaunch_t;
prnnStatus_t prnn_set_launch(prnnHandle_t handle, prnnLaunch_t kind);

/* Copies the plan of the last successful forward call into *info. */
prnnStatus_t prnn_get_last_plan(prnnHandle_t handle, prnnPlanInfo_t* info);

/* Phase tracing (TEAM layout only).  With enable != 0, later forward and
 * floor calls run trace instances of the team kernels: each wave of each
 * workgroup that serves a batch row records, per call, the shader-clock
 * cycles it spent in staging h_{t-1} (polling the exchange and writing LDS),
 * waiting at the workgroup barrier, reading LDS and multiplying, reducing
 * across lanes, and in the epilogue (x, ReLU, stores), then the whole time
 * loop in cycles and in ticks of the 100 MHz constant clock, and the number
 * of steps (8 uint64 words per wave, in that order).  Tracing slows each step
 * a little (each mark reads the clock).  The first enable allocates the
 * handle-owned trace buffer (ALLOC_FAILED if that fails).  While tracing is
 * on, shapes without a trace instance and the SPREAD layout return
 * NOT_SUPPORTED.  enable = 0 returns to the untraced kernels. */
prnnStatus_t prnn_set_trace(prnnHandle_t handle, int enable);

/* Copies the trace of the last traced call into `out` (host memory,
 * `capacity` uint64 words), after synchronizing `stream`.  Record w (words
 * [8 w, 8 w + 8)) belongs to wave w % V of workgroup w / V, V = the
 * plan's waves_per_wg; records of workgroups that serve no batch row of
 * their own are zero.  *records receives the number of records
 * (grid * waves_per_wg).  BAD_PARAM if no traced call
 * was made, or if out is NULL or capacity < 8 * records (then *records is
 * still set, so out = NULL, capacity = 0 asks for the size). */
prnnStatus_t prnn_get_trace(prnnHandle_t handle, uint64_t* out, size_t capacity, int* records,
                            hipStream_t stream);

/* TEST ONLY: in the next forward call, workgroup `wg` (TEAM layout: the
 * workgroups of rank `wg` within every XCD) does not publish its rows at
 * timestep `step`, so the consumers' bounded waits expire and the
 * run reports EXECUTION_FAILED (every kernel still exits normally).
 * wg < 0 disables. */
prnnStatus_t prnn_debug_skip_publish(prnnHandle_t handle, int wg, int step);

/* TEST ONLY: from the next call on, until span is set to 0, every wave of the
 * recurrent kernels (single layer and stack, every layout) sleeps before it
 * publishes its rows of each timestep, for n < span periods of about 64
 * shader clocks, n drawn per (workgroup, wave, timestep) from a hash of
 * `seed`.  Rows then reach their consumers in a different order and at
 * different times; the results must be bitwise those of span = 0.  span in
 * [0, PRNN_DEBUG_JITTER_MAX], else BAD_PARAM.  Delays longer than the
 * watchdog (prnn_set_watchdog_us) make the run report EXECUTION_FAILED. */
#define PRNN_DEBUG_JITTER_MAX 1024
prnnStatus_t prnn_debug_jitter(prnnHandle_t handle, uint32_t seed, int span);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * The operation, argument meanings, layouts, ownership and argument errors of
 * prnn_forward_dense with its default options (TEAM layout, EXACT math, the
 * automatic XCDs per batch row), but no handle: the exchange ring lives in a
 * fixed array in the library's device memory (32 * PRNN_NOALLOC_MAX_N words +
 * 256 bytes, about 320 KiB: the team ring and, for dense fp16 layers split
 * over several XCDs per batch row, their shared ring), one copy per device,
 * held until the process ends.  No call allocates anything.
 *  - N > PRNN_NOALLOC_MAX_N returns NOT_SUPPORTED (the array's capacity), as
 *    do shapes the TEAM layout cannot take (fp32 W beyond N = 1792).
 *  - status: NULL, or one caller-owned device word (4-byte aligned).  The call
 *    first sets it to 0 on `stream`; a run that fails (a wait for h_{t-1}
 *    expired) sets it nonzero and leaves H undefined.  Read it once the
 *    stream's work has finished.  With NULL, failures are not reported (every
 *    kernel still exits).
 *  - Every call resets the array on `stream` (two or three small fill
 *    kernels, no memset, so calls can be captured into a graph) and counts
 *    its steps from 0.
 *  - Every call on a device shares that device's array and leaves it as its
 *    run left it: calls that overlap in time on one device (on different
 *    streams, or graph replays running at once) race and give wrong results.
 *    Run one at a time per device.
 *  - The first call on a device looks up the array's address and checks how
 *    workgroups are placed on the XCDs (a small kernel and a synchronous
 *    copy); it cannot be made while `stream` is being captured and then
 *    returns NOT_SUPPORTED: make one call outside capture first.
 *  - Call with the device current.  T == 0 returns SUCCESS and enqueues
 *    nothing. */
#define PRNN_NOALLOC_MAX_N 2560
prnnStatus_t prnn_forward_dense_noalloc(int N, int B, int T, prnnDataType_t w_type, const void* W,
                                        const float* X, const float* h0, float* H, uint32_t* status,
                                        hipStream_t stream);

/* Static description of a status code; never NULL, never allocates. */
const char* prnn_status_string(prnnStatus_t status);

#ifdef __cplusplus
}
#endif

#endif /* PRNN_H_ */
