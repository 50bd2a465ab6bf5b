/*
 * recurrent_nn_amd.h -- C-ABI of the MI355X (gfx950) implementation of the
 * ONNX recurrent operators RNN, GRU and LSTM.
 *
 * What is computed is defined on the onemodel page "Recurrent operators: RNN,
 * GRU, LSTM":
 *   - gate packing (LSTM i,o,f,c; GRU z,r,h; B = [W biases, R biases];
 *     P = [i, o, f] peepholes) ..................... section "Support"
 *   - XW = X . W^T over all steps, the per-step H . R^T, the gate arithmetic
 *     in its written order ........................ section "Computation"
 *   - activations, their parameters and cursors ... section "Activations"
 *   - sequence_lens, input_forget, layout 1, omitted inputs, zero-size,
 *     hidden_size .................................. section "Choices the
 *                                                     specification leaves open"
 *   - every NaN written as 0x7FC00000 ............. section "Exact mode"
 *   - fused multiply-add only inside the products . section "Fast mode"
 *   - scratch limit, Unsupported at plan time ..... section "Limits"
 * The input/output tables (shapes for layout 0 and 1, float32 T, int32
 * sequence_lens) are those of the WebGPU "ai.onnx.RNN" package README,
 * sections "Inputs", "Outputs", "Attributes", "Type constraints".
 *
 * This library runs the "fast mode" order: the two products (projection and
 * recurrent product) accumulate in the matrix cores' order with a fixed
 * tiling, so results are deterministic run to run; every other operation is
 * the written IEEE binary32 operation, unfused, in the written order.
 *
 * Conventions for every entry point
 *   - Tensors are dense row-major float32 in ONNX shapes for the attribute
 *     `layout` (layout 0: X [seq, batch, input], initial states and Y_h/Y_c
 *     [dirs, batch, hidden], Y [seq, dirs, batch, hidden]; layout 1: X
 *     [batch, seq, input], states [batch, dirs, hidden], Y [batch, seq, dirs,
 *     hidden]).  W is [dirs, G*hidden, input], R [dirs, G*hidden, hidden],
 *     B [dirs, 2*G*hidden], P [dirs, 3*hidden]; G = 1 (RNN), 3 (GRU), 4 (LSTM).
 *   - Every tensor pointer given to rnn_run is a DEVICE pointer on the current
 *     HIP device, except sequence_lens, which is a HOST int32 array (so that the
 *     range check is synchronous).  Device pointers must be 16-byte aligned.
 *   - The caller owns every tensor and the workspace; the plan owns host
 *     memory only.  rnn_run is stream-ordered and asynchronous: keep the
 *     tensors and the workspace alive until the stream has passed the work.
 *   - A plan with one workspace serves one stream at a time; concurrent runs
 *     need distinct workspaces.
 *   - Every check happens before anything is enqueued: a non-OK status leaves
 *     every output untouched.  rnn_last_error() then describes the failure.
 */
#ifndef RECURRENT_NN_AMD_H
#define RECURRENT_NN_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rnn_status {
    RNN_OK = 0,
    RNN_ERR_INVALID_INPUT = 1,   /* bad attribute, shape, pointer or sequence length */
    RNN_ERR_UNSUPPORTED = 2,     /* valid, but beyond this library (scratch limit)   */
    RNN_ERR_DEVICE = 3,          /* a HIP call failed, or a device-side check fired  */
    RNN_ERR_OUT_OF_MEMORY = 4    /* host allocation failed                           */
} rnn_status;

typedef enum rnn_op { RNN_OP_RNN = 0, RNN_OP_GRU = 1, RNN_OP_LSTM = 2 } rnn_op;

/* Element type of the projection's operands.  BF16 rounds X and W to
 * bfloat16 (round to nearest even) and accumulates in float32; XW, the
 * recurrence, the states and the gate arithmetic stay float32. */
typedef enum rnn_proj_dtype { RNN_PROJ_F32 = 0, RNN_PROJ_BF16 = 1 } rnn_proj_dtype;

/* How the step loop is run.  AUTO picks PERSISTENT when every workgroup can be
 * resident at once, else PER_STEP. */
typedef enum rnn_kernel_path {
    RNN_PATH_AUTO = 0,
    RNN_PATH_PERSISTENT = 1,     /* one cooperative launch, device-wide step barrier */
    RNN_PATH_PER_STEP = 2        /* one launch per step (two for GRU lbr = 0)        */
} rnn_kernel_path;

/* Operator attributes (onemodel "Computation"/"Activations"; WebGPU README
 * "Attributes").  Zero-initialise and set what is needed. */
typedef struct rnn_attrs {
    int32_t op;                        /* rnn_op                                          */
    const char *direction;             /* "forward" | "reverse" | "bidirectional"; NULL = forward */
    int64_t hidden_size;               /* 0 = absent; else must equal R's last dimension  */
    int32_t layout;                    /* 0 or 1                                          */
    int32_t n_activations;             /* 0 = defaults (LSTM Sigmoid,Tanh,Tanh; GRU       */
    const char *const *activations;    /*   Sigmoid,Tanh; RNN Tanh); names case-insensitive;
                                          one set, or forward then reverse set            */
    int32_t n_alpha;                   /* activation_alpha, consumed in activation order  */
    const float *activation_alpha;
    int32_t n_beta;                    /* activation_beta, its own cursor                 */
    const float *activation_beta;
    int32_t has_clip;                  /* clamp pre-activations to [-clip, clip] only when */
    float clip;                        /*   has_clip && clip > 0; a NaN passes through    */
    int32_t input_forget;              /* LSTM only: forget gate = 1 - input gate         */
    int32_t linear_before_reset;       /* GRU only                                        */
    int32_t proj_dtype;                /* rnn_proj_dtype                                  */
    int32_t constant_weights;          /* W, R, B, P do not change between runs of this
                                          plan with this workspace: pack them once       */
    int32_t kernel_path;               /* rnn_kernel_path                                 */
    int32_t units_per_block;           /* 0 = automatic; hidden units per workgroup       */
    int32_t batch_tile;                /* 0 = automatic; batch rows per workgroup (16/32/64) */
    int32_t waves_per_block;           /* 0 = automatic; 4 or 8 waves split the step product */
    int32_t barrier_spin_limit;        /* 0 = default; polls before a step barrier gives up,
                                          raising the error rnn_workspace_check reports   */
    int32_t batch_halves;              /* 0 = automatic; 1 = each step over the whole batch
                                          tile; 2 = each step as two half-tile sub-steps, so
                                          that one half's H exchange overlaps the other
                                          half's product (needs R resident in registers, an
                                          RNN, LSTM or GRU with linear_before_reset = 1, and
                                          a batch tile of 32 or 64; else InvalidInput).
                                          Results are identical either way.              */
    int32_t time_chunk;                /* 0 = all steps at once; else steps per chunk: the
                                          projections and the H history are held for one
                                          chunk at a time and the states carry over between
                                          chunks, so the scratch limit applies to the chunk
                                          length instead of seq_length.  Results are
                                          identical either way.                          */
    int32_t exact;                     /* 1 = exact mode (onemodel "Exact mode"): every
                                          product value is one binary32 accumulator over
                                          k in increasing order from +0, each multiply and
                                          add rounded on its own (no matrix cores), and
                                          the transcendental activations follow one fixed
                                          binary64 method; results do not depend on the
                                          tiling and match that definition bit for bit.
                                          0 = fast mode (matrix-core products).           */
    int32_t fuse_projection;           /* 0 or 1 = the input projection as its own launch
                                          into a buffer of the workspace (the faster form
                                          where both apply); 2 = the projection inside the
                                          step loop, each workgroup computing the values of
                                          its own gate columns and rows one step ahead from
                                          its slice of W held in LDS, so that the workspace
                                          holds no projections (needs the two-half schedule
                                          in fast mode, an F32 projection, input_size a
                                          multiple of 256 and the slice within LDS; else
                                          InvalidInput).  Results are identical either way. */
} rnn_attrs;

/* Dimensions: hidden is R's last dimension, num_directions W's first. */
typedef struct rnn_dims {
    int64_t seq_length;
    int64_t batch_size;
    int64_t input_size;
    int64_t hidden;
    int64_t num_directions;
} rnn_dims;

typedef struct rnn_plan rnn_plan;

/*
 * rnn_plan_create -- validate attributes and dimensions, resolve the
 * activations (f, g, h per direction with alpha/beta cursors), choose the
 * tiling and lay out the workspace.  Host only: touches no device.
 *   attrs, dims: read during the call only.  *out receives a new plan.
 *   Errors, each with the passage that defines the rule (sections of the
 *   onemodel page "Recurrent operators: RNN, GRU, LSTM" unless stated):
 *   RNN_ERR_INVALID_INPUT for
 *     - an activation name outside the supported list, or a list that is
 *       neither one set nor (bidirectional) a forward and a reverse set
 *       .................................................. "Activations";
 *     - hidden 0, or a hidden_size attribute that differs from R's last
 *       dimension ....... "Choices the specification leaves open", hidden_size;
 *     - input_forget on a non-LSTM, linear_before_reset on a non-GRU (the
 *       attributes exist for those operators only) ......... "Computation";
 *     - layout other than 0 or 1 ..... "Choices ...", layout = 1; WebGPU README
 *       "Attributes";
 *     - an unknown op or direction, num_directions not matching direction
 *       (W's first dimension is the direction count) ..... WebGPU README
 *       "Inputs" and "Attributes";
 *     - negative sizes, time_chunk, barrier_spin_limit or tiling overrides
 *       outside their ranges (this library's own attributes);
 *   RNN_ERR_UNSUPPORTED when, per direction, L*batch*G*hidden + 4*batch*hidden
 *   (+ G*hidden*(input+hidden) unless constant_weights) reaches 2^30 floats,
 *   with L = seq_length, or the chunk length when time_chunk is set
 *   ............................................................... "Limits".
 */
rnn_status rnn_plan_create(const rnn_attrs *attrs, const rnn_dims *dims, rnn_plan **out);

/* Bytes of device workspace rnn_run needs for this plan (0 for zero-size). */
rnn_status rnn_plan_workspace_size(const rnn_plan *plan, size_t *bytes);

/*
 * rnn_run -- enqueue one operator invocation on `hip_stream` (a hipStream_t;
 * NULL = the null stream).  X, W, R are required; B, initial_h, initial_c, P
 * may be NULL (bias additions skipped, zero states, no peepholes);
 * sequence_lens may be NULL (every row runs seq steps) and is a HOST array of
 * batch_size int32 values in [0, seq].  Y, Y_h, Y_c may each be NULL (output
 * not wanted); Y_c, initial_c and P must be NULL unless the op is LSTM.
 * Y is written in full: positions t >= sequence_lens[b] hold +0.0; Y_h / Y_c
 * hold the state after each row's last valid step and 0 for a row of length
 * 0; with seq = 0 or batch = 0 they hold the initial states (or zeros).
 *   workspace: device memory of at least rnn_plan_workspace_size() bytes,
 *   256-byte aligned, owned by the caller, used by this run until the stream
 *   passes it.  With constant_weights the packed weights stay in it between
 *   runs: reuse the same workspace and weight pointers.
 *   Errors (nothing is enqueued): RNN_ERR_INVALID_INPUT for
 *     - a sequence length outside [0, seq] ..... "Choices the specification
 *       leaves open", sequence_lens (the run-time InvalidInput it names);
 *     - Y_c, initial_c or P given to a non-LSTM plan (LSTM-only tensors)
 *       ...................................... "Support"; WebGPU README "Inputs";
 *     - NULL X, W or R (required inputs) ........... WebGPU README "Inputs";
 *     - misaligned pointers or a workspace missing, too small or misaligned
 *       (this library's own conventions, above);
 *   RNN_ERR_DEVICE when a HIP call fails (the run may then be partial).
 */
rnn_status rnn_run(rnn_plan *plan, void *hip_stream, void *workspace, size_t workspace_bytes,
                   const float *X, const float *W, const float *R, const float *B,
                   const int32_t *sequence_lens, const float *initial_h,
                   const float *initial_c, const float *P,
                   float *Y, float *Y_h, float *Y_c);

/*
 * rnn_cell_run -- one step of the operator in the single-cell convention of
 * the OpenVINO page "RNNCell-3" (sections "Inputs" and "Outputs"; its formula
 * Ht = f(Xt Wi^T + Ht-1 Ri^T + Wbi + Rbi) in the description): the same
 * operator as rnn_run at seq_length 1, except that the bias is ONE vector,
 * the sum of the W and R biases, and only the new state is produced.
 *   plan: created with dims.seq_length = 1 and dims.num_directions = 1 (any
 *   op; the cell page itself defines the RNN cell, and the same convention is
 *   applied to GRU and LSTM gates).
 *   X [batch, input]; H [batch, hidden] (NULL = zeros); C [batch, hidden]
 *   (LSTM only, NULL = zeros); W [G*hidden, input]; R [G*hidden, hidden];
 *   B_sum [G*hidden] summed biases in the operator's gate order (NULL = no
 *   bias); P [3*hidden] (LSTM peepholes, NULL = none) -- all DEVICE pointers.
 *   H_out [batch, hidden] (required), C_out [batch, hidden] (LSTM only,
 *   nullable): the state after the step.  NaN is written as 0x7FC00000.
 *   The summed bias enters as ((X Wi^T + H Ri^T) + B_sum); internally it is
 *   the ONNX B with Wb = B_sum and Rb = +0, which is exact.  It is staged in
 *   the workspace, so the same workspace rules as rnn_run apply.
 *   Errors (nothing is enqueued): those of rnn_run, plus InvalidInput when
 *   the plan is not single-step and single-direction, when H_out is NULL, or
 *   when B_sum is given for GRU with linear_before_reset = 1 (its recurrent
 *   candidate bias is multiplied by the reset gate, so a sum cannot carry it:
 *   use rnn_run with the full B there).
 */
rnn_status rnn_cell_run(rnn_plan *plan, void *hip_stream, void *workspace, size_t workspace_bytes,
                        const float *X, const float *H, const float *C, const float *W,
                        const float *R, const float *B_sum, const float *P, float *H_out,
                        float *C_out);

/*
 * rnn_run_noalloc -- rnn_run for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace, the same launches and
 * results, and no allocating call at all.  Its scratch is a device array of
 * RNN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; sequence_lens reach the device as kernel arguments.
 *   Limits (RNN_ERR_UNSUPPORTED, nothing enqueued, no device call made): a plan
 *   whose rnn_plan_workspace_size() exceeds RNN_NOALLOC_SCRATCH_BYTES, or
 *   sequence_lens with more than RNN_NOALLOC_MAX_LENS_BATCH batch rows.
 *   Sharing: every call on one GPU uses that GPU's one scratch array, and each
 *   call leaves it holding its own state; calls that overlap in time on the
 *   same GPU (another stream, another thread, another plan) race and give
 *   undefined results.  Serialise them.  With constant_weights the packed
 *   weights are reused only while no other plan has run here in between.
 *   Stage timing (rnn_plan_enable_timing) records nothing on this path, and a
 *   barrier time-out is not reported (rnn_workspace_check needs a workspace).
 *   Other errors: those of rnn_run.
 */
#define RNN_NOALLOC_SCRATCH_BYTES (64u << 20)
#define RNN_NOALLOC_MAX_LENS_BATCH 256
rnn_status rnn_run_noalloc(rnn_plan *plan, void *hip_stream, const float *X, const float *W,
                           const float *R, const float *B, const int32_t *sequence_lens,
                           const float *initial_h, const float *initial_c, const float *P,
                           float *Y, float *Y_h, float *Y_c);

/*
 * rnn_workspace_check -- wait for `hip_stream`, then read the device-side
 * error word that the last run on this workspace left (a step barrier that
 * timed out).  RNN_OK when clean, RNN_ERR_DEVICE otherwise.  For tests of
 * this path, a plan created while the environment variable
 * RNN_AMD_TEST_WITHHOLD_FLAGS is set to a non-zero value never stores its
 * step flags, so every wait between steps runs out barrier_spin_limit (results
 * are then undefined, and the kernel still finishes).
 */
rnn_status rnn_workspace_check(const rnn_plan *plan, void *hip_stream, const void *workspace);

/*
 * rnn_plan_enable_timing -- when enabled, rnn_run records HIP events around
 * each stage on its stream; rnn_plan_last_timings then waits for them and
 * writes up to n durations in milliseconds of the last run, in the order
 * pack, projection, recurrence, other (init and final writes).
 */
rnn_status rnn_plan_enable_timing(rnn_plan *plan, int32_t enable);
rnn_status rnn_plan_last_timings(rnn_plan *plan, float *ms, int32_t n);

/* A short human-readable description of the tiling and kernel path. */
rnn_status rnn_plan_describe(const rnn_plan *plan, char *buf, size_t len);

/* Release a plan (host memory only).  NULL is a no-op. */
void rnn_plan_destroy(rnn_plan *plan);

/* Thread-local text describing the last non-OK status on this thread. */
const char *rnn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RECURRENT_NN_AMD_H */
