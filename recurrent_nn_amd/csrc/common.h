// common.h -- internal definitions shared by the host code and the kernels of
// the MI355X ONNX RNN/GRU/LSTM library: the plan, the workspace layout and the
// parameter blocks passed to the kernels.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/recurrent_nn_amd.h"

namespace rnnamd {

// Activation kinds (onemodel "Activations": the supported list).
enum ActKind : int32_t {
    ACT_SIGMOID = 0, ACT_TANH, ACT_RELU, ACT_AFFINE, ACT_LEAKYRELU,
    ACT_THRESHOLDEDRELU, ACT_SCALEDTANH, ACT_HARDSIGMOID, ACT_ELU,
    ACT_SOFTSIGN, ACT_SOFTPLUS, ACT_KIND_COUNT
};

struct ActSpec {
    int32_t kind;
    float alpha;
    float beta;
};

// Stage indices for the optional event timing.
enum Stage { STAGE_PACK = 0, STAGE_PROJ = 1, STAGE_REC = 2, STAGE_OTHER = 3, STAGE_COUNT = 4 };

constexpr int kThreads = 256;          // threads of the auxiliary kernels' workgroups
constexpr int kMaxPairs = 8;           // (row, unit) pairs per thread in the epilogue
constexpr int kMaxWorkgroups = 256;    // one workgroup per CU on MI355X
constexpr uint32_t kDefaultSpinLimit = 1u << 26;   // ~seconds of polling: a step takes microseconds

// Workspace layout: byte offsets from the workspace base, each 256-aligned.
struct Layout {
    size_t wp = 0;      // packed W: rows in block-column order, [D*G*H][I] f32 or bf16
    size_t rp = 0;      // packed R: [D][NUB][NT*16][Hp] f32, zero-padded
    size_t xb = 0;      // bf16 projection: the chunk's X rows by step, rounded, [D][C*Bt][I]
    size_t xw = 0;      // projections: [D][C][Bt][G*H] f32 by step, block-column order
    size_t hbuf = 0;    // H history: plane j mod (C+1) = H before step j, [C+1][D][Btp][Hp] f32
    size_t sbuf = 0;    // GRU lbr=0: r (.) H_prev of step j in plane j mod C, [C][D][Btp][Hp]
    size_t cbuf = 0;    // LSTM cell state between launches [D][Bt][H]
    size_t zbuf = 0;    // GRU lbr=0 update gate between launches [D][Bt][H]
    size_t rowmap = 0;  // int32 [C * Bt]: the projection's rows of a time chunk
    size_t lens = 0;    // int32 [3][Bt]: lengths by position, the batch row at each
                        // position, the position of each rank (rows by decreasing length)
    size_t bar = 0;     // uint32 step flags [D*NBB][2][NUB], then int32 error word
    size_t cellb = 0;   // rnn_cell_run: summed biases expanded to [D][Wb = sum, Rb = 0]
    size_t stamps = 0;  // instrumented build only: cycle stamps [kStampSlots][kStampEvents]
    size_t total = 0;
};

// Cycle stamps of the instrumented build (-DRNN_STAMPS): one workgroup's
// wave 0 records the shader clock at fixed points of each step (phase or
// half-step) into the workspace; the normal build records nothing.
constexpr int kStampSlots = 1024;
constexpr int kStampEvents = 8;

}  // namespace rnnamd

struct rnn_plan {
    // operator
    int32_t op = 0;           // rnn_op
    int32_t G = 1;            // gates
    int32_t D = 1;            // directions
    int32_t reverse_only = 0;
    int32_t layout = 0;
    int32_t clip_on = 0;
    float clip = 0.0f;
    int32_t input_forget = 0;
    int32_t lbr = 0;
    int32_t proj_bf16 = 0;
    int32_t constant_weights = 0;
    int32_t kernel_path = 0;
    uint32_t spin_limit = 0;  // polls before a step barrier gives up
    int32_t withhold_flags = 0;   // test fault injection: step flags are never stored
    int32_t proj_rows = 0;    // projection rows with sequence_lens: 0 auto, 1 list, 2 tiles
    int32_t stamp_wg = 0;     // instrumented build: the workgroup whose steps are stamped
    int64_t S = 0, Bt = 0, I = 0, H = 0;
    int64_t C = 0;            // steps per chunk (time_chunk; S when not chunked)
    rnnamd::ActSpec act[2][3] = {};

    // tiling of the recurrence
    int32_t U = 1;            // hidden units per workgroup (last block may be ragged)
    int32_t NUB = 1;          // unit blocks per direction
    int32_t BT = 16;          // batch rows per workgroup (16, 32, 64 or 128)
    int32_t NBB = 1;          // batch blocks
    int32_t MT = 1;           // 16-row MFMA tiles per workgroup (BT / 16)
    int32_t NTA = 1;          // 16-column tiles of phase 0
    int32_t NTB = 0;          // 16-column tiles of phase 1 (GRU lbr=0 candidate)
    int32_t NT = 1;           // NTA + NTB
    int32_t phases = 1;       // 2 for GRU lbr=0
    int64_t Hp = 64;          // hidden padded to a multiple of 16 * NW (K of the step product)
    int32_t NW = 4;           // waves per workgroup (4 or 8); they split k
    int32_t KB = 1;           // 16-wide k blocks per wave (Hp / (16 * NW))
    int32_t resident = 0;     // R slice held in registers across steps
    int32_t halves = 1;       // 2: each step as two half-batch sub-steps (rec_pipe_kernel)
    int32_t fused = 0;        // 1: the projection computed inside the step loop (rec_fused_kernel)
    int32_t exact = 0;        // exact mode: k-ordered unfused products, exact activations
    int64_t Btp = 16;         // NBB * BT
    int32_t n_wg = 1;         // D * NBB * NUB

    rnnamd::Layout ws;

    // constant-weights cache: what the workspace holds packed
    int32_t packed_valid = 0;
    const void *packed_ws = nullptr;
    const void *packed_W = nullptr, *packed_R = nullptr;

    // device-dependent decisions, made on the first run
    int32_t dev_ready = 0;
    int32_t can_persist = 0;
    int32_t device = -1;

    // timing
    // pinned host staging of sequence_lens, their order and sorting room,
    // [5][Bt] (the first three copied to the device asynchronously; the
    // event guards its reuse by the next run)
    int32_t *lens_host = nullptr;
    void *lens_event = nullptr;
    int32_t lens_pending = 0;

    int32_t timing = 0;
    void *events[2 * rnnamd::STAGE_COUNT] = {};
    int32_t events_recorded = 0;
};

namespace rnnamd {

void set_error(const std::string &msg);
// step flags in the workspace: one per (direction, batch block, half, unit block)
inline int64_t n_flags(const rnn_plan &p) { return (int64_t)p.D * p.NBB * 2 * p.NUB; }
int64_t round_up(int64_t x, int64_t m);
void block_columns(const rnn_plan &p, int64_t ub, int32_t *u0, int32_t *uc);

// ---------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files).  Each returns a hipError_t
// value as int (0 = success) and enqueues on `stream`.
// ---------------------------------------------------------------------------

struct PackArgs {
    const float *W, *R;
    void *Wp;           // f32 or bf16
    float *Rp;
    int64_t D, G, H, I, Hp;
    int32_t U, NUB, NTA, NTB, phases, bf16;
};
int launch_pack(const PackArgs &a, void *stream);


struct InitArgs {
    const float *h0, *c0;       // nullable, layout-dependent
    float *hbuf, *sbuf, *cbuf;  // sbuf/cbuf nullable
    int32_t *lens_dev;
    const int32_t *order;       // [Bt] batch row held at each position, or NULL (identity)
    int32_t fill_lens;          // >= 0: every row gets this length (sequence_lens absent)
    uint32_t *bar;
    int64_t n_bar;
    int64_t D, Bt, Btp, H, Hp;
    int32_t layout;
};
int launch_init(const InitArgs &a, void *stream);

// Sequence lengths handed to the device as kernel arguments (no staging
// buffer, no copy): the lengths by position, the batch row at each position
// and the position of each rank, for at most kInlineRows rows.
constexpr int kInlineRows = 256;
struct InlineLens {
    int32_t n;
    int32_t lens[kInlineRows];
    int32_t order[kInlineRows];
    int32_t rank_pos[kInlineRows];
};
// dst[0, n) = lens, dst[n, 2n) = order, dst[2n, 3n) = rank_pos
int launch_lens_inline(const InlineLens &l, int32_t *dst, void *stream);

struct ProjArgs {
    const void *X;          // f32 X in the operator's layout
    uint16_t *Xb;           // bf16 projection: [D][steps * Bt][K] staging of the gathered rows
    const void *Wp;         // f32 or bf16 packed W, [D][GH][I]
    float *XW;              // [D][steps][Bt][GH], row (j - j_base, b) of direction d
    int64_t K;              // I
    int64_t S, Bt, GH, D;
    int64_t steps;          // steps held by XW (the chunk length)
    int64_t j_base;         // first step of the chunk
    const int32_t *lens;    // [Bt] lengths by position, on the device
    const int32_t *order;   // [Bt] batch row at each position, or NULL (identity)
    // [Bt] position of the row of rank r (ranks by decreasing length), or
    // NULL (identity): the product walks its rows by rank, so that rows the
    // step loop never reads fill whole tiles, and stores each at its position
    const int32_t *rank_pos;
    // The rows computed.  With rowmap (sequence_lens given): m_rows rows, row
    // m' being dense row rowmap[m'] = (j - j_base) * Bt + r, the rows the step
    // loop reads, step by step (built by launch_proj_rows).  Without it:
    // m_rows = steps * Bt dense rows.
    const int32_t *rowmap;
    int64_t m_rows;
    int32_t reverse_only;   // direction 0 runs in reverse
    int32_t layout;         // 0: X [S][Bt][I]; 1: X [Bt][S][I]
    int32_t bf16;
    int32_t exact;          // exact mode: one accumulator per output, k in order, VALU
};
int launch_projection(const ProjArgs &a, void *stream);
// rowmap[0, m_rows) of the chunk, from the lengths by position and the
// positions by rank (one workgroup)
int launch_proj_rows(const ProjArgs &a, int32_t *rowmap, void *stream);

struct RecArgs {
    // sizes
    int32_t S, Bt, H, D, G, op;
    int32_t Hp, KB, NW, U, NUB, BT, NBB, MT, NTA, NTB, NT, phases;
    int32_t Btp;
    int32_t halves;         // 1, or 2 half-batch sub-steps per step (rec_pipe_kernel)
    int32_t fused;          // 1: the projection inside the two-half step loop (rec_fused_kernel)
    int32_t I;              // input size (the fused projection's k)
    int32_t exact;          // exact mode (rec_exact_kernel)
    int32_t reverse_only, layout, clip_on, input_forget, lbr;
    float clip;
    ActSpec act[2][3];
    // buffers
    const float *Rp, *XW, *B, *P;
    // fused projection: X in the operator's layout, W packed [D][GH][I] (fp32)
    const float *X, *Wp;
    // Position s holds batch row order[s] (identity when order is NULL) and
    // lens[s] is its length; each block of BT positions holds its rows in
    // order of decreasing length, so that the rows still active at a step
    // come first.  The H history, cell state and XW rows use positions; only
    // the outputs Y, Y_h, Y_c use batch rows.
    const int32_t *lens, *order;
    float *hbuf, *sbuf, *cbuf, *zbuf;
    float *Y, *Yh, *Yc;
    uint32_t *bar;
    int32_t *err;
    uint32_t spin_limit;
    int32_t withhold_flags;  // test fault injection: never store the step flags
    // launch range in phase units (step j, phase p) -> q = j * phases + p
    int32_t q_begin, q_end;
    // instrumented build: stamps[slot][event] of workgroup stamp_wg
    uint64_t *stamps;
    int32_t stamp_wg;
    // time chunk of xw_steps steps starting at j_base: XW row = j - j_base;
    // the H history is a ring of xw_steps + 1 planes (plane j mod (steps+1)),
    // r (.) H_prev a ring of xw_steps planes, so one chunk's last plane is the
    // next chunk's first and every plane is fresh within a launch
    int32_t j_base, xw_steps;
};
// persistent: one cooperative launch covering every phase; else one phase.
int launch_recurrence(const RecArgs &a, int resident, int persistent, void *stream);
int recurrence_can_persist(const RecArgs &a, int resident, int device, int *ok);
bool recurrence_supported(int nw, int mt, int nt, int nta, int phases, int kb, int bt, int u,
                          int resident, int halves);
// whether rec_fused_kernel takes a two-half tiling with this input size
bool recurrence_fused_supported(int bt, int nt, int u, int64_t I);

struct FinalArgs {
    const float *h0, *c0;
    float *Yh, *Yc;
    int64_t n;              // D * Bt * H
};
int launch_zero_size_states(const FinalArgs &a, void *stream);
// dst[d][0, GH) = B_sum[d][...], dst[d][GH, 2 GH) = +0 for d < D
int launch_cell_bias(const float *B_sum, float *dst, int64_t D, int64_t GH, void *stream);

}  // namespace rnnamd
