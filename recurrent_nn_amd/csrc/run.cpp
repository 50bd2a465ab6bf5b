// run.cpp -- rnn_run: host-side checks (every one before anything is
// enqueued), then the stream-ordered launch sequence
//   pack W and R (unless constant and already packed)  -> init states
//   -> projection XW = X . W^T over all steps -> step loop -> (final states
//   are written by the step loop itself)
// for the ONNX recurrent operators.  The sequence_lens range check is the
// onemodel page's run-time InvalidInput ("Choices the specification leaves
// open"); seq = 0 or batch = 0 runs nothing but the initial-state copy.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "common.h"

using namespace rnnamd;

namespace {

rnn_status hip_fail(hipError_t e, const char *where)
{
    set_error(std::string(where) + ": " + hipGetErrorString(e));
    return RNN_ERR_DEVICE;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Timer {
    rnn_plan *p;
    hipStream_t s;
    bool on;
    void begin(int stage)
    {
        if (on)
            (void)hipEventRecord((hipEvent_t)p->events[2 * stage], s);
    }
    void end(int stage)
    {
        if (on)
            (void)hipEventRecord((hipEvent_t)p->events[2 * stage + 1], s);
    }
};

RecArgs rec_args(const rnn_plan &p, unsigned char *ws, const float *B, const float *P, float *Y,
                 float *Yh, float *Yc)
{
    RecArgs r{};
    r.S = (int32_t)p.S;
    r.Bt = (int32_t)p.Bt;
    r.H = (int32_t)p.H;
    r.D = p.D;
    r.G = p.G;
    r.op = p.op;
    r.Hp = (int32_t)p.Hp;
    r.KB = p.KB;
    r.NW = p.NW;
    r.U = p.U;
    r.NUB = p.NUB;
    r.BT = p.BT;
    r.NBB = p.NBB;
    r.MT = p.MT;
    r.NTA = p.NTA;
    r.NTB = p.NTB;
    r.NT = p.NT;
    r.phases = p.phases;
    r.Btp = (int32_t)p.Btp;
    r.halves = p.halves;
    r.fused = p.fused;
    r.I = (int32_t)p.I;
    r.exact = p.exact;
    r.reverse_only = p.reverse_only;
    r.layout = p.layout;
    r.clip_on = p.clip_on;
    r.clip = p.clip;
    r.input_forget = p.input_forget;
    r.lbr = p.lbr;
    std::memcpy(r.act, p.act, sizeof(r.act));
    r.Rp = (const float *)(ws + p.ws.rp);
    r.Wp = (const float *)(ws + p.ws.wp);
    r.XW = (const float *)(ws + p.ws.xw);
    r.B = B;
    r.P = P;
    r.lens = (const int32_t *)(ws + p.ws.lens);
    r.hbuf = (float *)(ws + p.ws.hbuf);
    r.sbuf = p.phases == 2 ? (float *)(ws + p.ws.sbuf) : nullptr;
    r.cbuf = p.op == RNN_OP_LSTM ? (float *)(ws + p.ws.cbuf) : nullptr;
    r.zbuf = p.phases == 2 ? (float *)(ws + p.ws.zbuf) : nullptr;
    r.Y = Y;
    r.Yh = Yh;
    r.Yc = Yc;
    r.bar = (uint32_t *)(ws + p.ws.bar);
    r.err = (int32_t *)(ws + p.ws.bar) + n_flags(p);
    r.spin_limit = p.spin_limit;
    r.withhold_flags = p.withhold_flags;
    r.q_begin = 0;
    r.q_end = (int32_t)(p.S * p.phases);
    r.stamps = p.ws.stamps ? (uint64_t *)(ws + p.ws.stamps) : nullptr;
    r.stamp_wg = p.stamp_wg;
    r.j_base = 0;
    r.xw_steps = (int32_t)p.C;
    return r;
}

rnn_status device_setup(rnn_plan *p, unsigned char *ws)
{
    if (p->dev_ready)
        return RNN_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    p->device = dev;
    RecArgs r = rec_args(*p, ws, nullptr, nullptr, nullptr, nullptr, nullptr);
    int ok = 0;
    int rc = recurrence_can_persist(r, p->resident, dev, &ok);
    if (rc != 0)
        return hip_fail((hipError_t)rc, "recurrence occupancy query");
    p->can_persist = ok;
    if (p->kernel_path == RNN_PATH_PERSISTENT && !ok) {
        set_error("persistent path requested but the workgroups cannot all be resident");
        return RNN_ERR_UNSUPPORTED;
    }
    p->dev_ready = 1;
    return RNN_OK;
}

// The timing events of the stages (created once, when timing is enabled).
rnn_status ensure_events(rnn_plan *p)
{
    for (int i = 0; i < 2 * STAGE_COUNT; ++i)
        if (!p->events[i]) {
            hipEvent_t ev;
            hipError_t e = hipEventCreate(&ev);
            if (e != hipSuccess)
                return hip_fail(e, "hipEventCreate");
            p->events[i] = ev;
        }
    return RNN_OK;
}

// The batch rows by decreasing length (ties by lower row) -- their ranks --
// dealt over the batch blocks of BT positions (the last block may hold
// fewer) in proportion to each block's capacity: slot k of a block of cap
// rows falls at the fraction (k + 1/2) / cap of the deal, slots are taken in
// that order (lower block first on ties) and rank r fills the r-th slot.
// With equal blocks this is round robin.  Every block then holds a run of
// decreasing lengths (its active rows come first) and a like share of every
// length, which matters because the step loop waits for its slowest block
// at every step.  order[i] is the batch row at position i, byPos[i] its
// length, rank_pos[r] the position of the row of rank r; tmp holds 2 Bt
// values.  Nothing is allocated.
void order_rows(const int32_t *lens, int64_t Bt, int64_t BT, int32_t *byPos, int32_t *order,
                int32_t *rank_pos, int32_t *tmp)
{
    int32_t *rank = tmp, *slot = tmp + Bt;
    for (int64_t b = 0; b < Bt; ++b)
        rank[b] = (int32_t)b;
    std::sort(rank, rank + Bt, [lens](int32_t x, int32_t y) {
        return lens[x] != lens[y] ? lens[x] > lens[y] : x < y;
    });
    for (int64_t i = 0; i < Bt; ++i)
        slot[i] = (int32_t)i;          // position i = block i / BT, slot i % BT
    auto cap = [Bt, BT](int64_t blk) { return std::min<int64_t>(BT, Bt - blk * BT); };
    std::sort(slot, slot + Bt, [&](int32_t x, int32_t y) {
        const int64_t bx = x / BT, by = y / BT;
        const int64_t fx = (2 * (x - bx * BT) + 1) * cap(by), fy = (2 * (y - by * BT) + 1) * cap(bx);
        return fx != fy ? fx < fy : bx < by;
    });
    for (int64_t r = 0; r < Bt; ++r) {
        const int32_t pos = slot[r];
        order[pos] = rank[r];
        byPos[pos] = lens[rank[r]];
        rank_pos[r] = pos;
    }
}


// Every argument check of a run; nothing is enqueued.
rnn_status run_checks(const rnn_plan *p, const void *workspace, size_t workspace_bytes,
                      const float *X, const float *W, const float *R, const float *B,
                      const int32_t *sequence_lens, const float *initial_h,
                      const float *initial_c, const float *P, const float *Y, const float *Y_h,
                      const float *Y_c, bool check_workspace = true)
{
    const bool zero = p->S == 0 || p->Bt == 0;
    if (p->op != RNN_OP_LSTM && (initial_c || P || Y_c)) {
        set_error("rnn_run: initial_c, P and Y_c are LSTM-only");
        return RNN_ERR_INVALID_INPUT;
    }
    if (!zero && (!X || !W || !R)) {
        set_error("rnn_run: X, W and R are required");
        return RNN_ERR_INVALID_INPUT;
    }
    const void *ptrs[] = {X, W, R, B, initial_h, initial_c, P, Y, Y_h, Y_c};
    for (const void *q : ptrs)
        if (q && !aligned(q, 4)) {
            set_error("rnn_run: tensors must be 4-byte aligned");
            return RNN_ERR_INVALID_INPUT;
        }
    if (X && !aligned(X, 16)) {
        set_error("rnn_run: X must be 16-byte aligned");
        return RNN_ERR_INVALID_INPUT;
    }
    if (sequence_lens)
        for (int64_t b = 0; b < p->Bt; ++b)
            if (sequence_lens[b] < 0 || sequence_lens[b] > p->S) {
                set_error("rnn_run: sequence_lens[" + std::to_string(b) + "] = " +
                          std::to_string(sequence_lens[b]) + " is outside [0, seq]");
                return RNN_ERR_INVALID_INPUT;
            }

    if (check_workspace && !zero &&
        (!workspace || workspace_bytes < p->ws.total || !aligned(workspace, 256))) {
        set_error("rnn_run: workspace missing, smaller than rnn_plan_workspace_size() or not "
                  "256-byte aligned");
        return RNN_ERR_INVALID_INPUT;
    }
    return RNN_OK;
}

// The launch sequence of a checked run.
// noalloc: the allocation-free form (rnn_run_noalloc): no stage timing, and
// the sequence lengths reach the device as kernel arguments instead of
// through the plan's pinned staging buffer.
rnn_status run_enqueue(rnn_plan *p, hipStream_t s, void *workspace, const float *X,
                       const float *W, const float *R, const float *B,
                       const int32_t *sequence_lens, const float *initial_h,
                       const float *initial_c, const float *P, float *Y, float *Y_h, float *Y_c,
                       bool noalloc = false)
{
    if (p->S == 0 || p->Bt == 0) {
        FinalArgs f{initial_h, initial_c, Y_h, Y_c, (int64_t)p->D * p->Bt * p->H};
        int rc = launch_zero_size_states(f, s);
        return rc ? hip_fail((hipError_t)rc, "zero-size state copy") : RNN_OK;
    }
    unsigned char *ws = (unsigned char *)workspace;
    rnn_status st = device_setup(p, ws);
    if (st != RNN_OK)
        return st;
    const bool persistent = p->kernel_path == RNN_PATH_PERSISTENT ||
                            (p->kernel_path == RNN_PATH_AUTO && p->can_persist);
    const bool timed = p->timing && !noalloc;
    if (timed) {
        st = ensure_events(p);
        if (st != RNN_OK)
            return st;
    }
    Timer tm{p, s, timed};
    p->events_recorded = timed;
    hipError_t e;

    // 1. pack W (block-column row order, optional bf16) and R (padded tiles)
    tm.begin(STAGE_PACK);
    const bool reuse = p->constant_weights && p->packed_valid && p->packed_ws == workspace &&
                       p->packed_W == W && p->packed_R == R;
    if (!reuse) {
        PackArgs pa{};
        pa.W = W;
        pa.R = R;
        pa.Wp = ws + p->ws.wp;
        pa.Rp = (float *)(ws + p->ws.rp);
        pa.D = p->D;
        pa.G = p->G;
        pa.H = p->H;
        pa.I = p->I;
        pa.Hp = p->Hp;
        pa.U = p->U;
        pa.NUB = p->NUB;
        pa.NTA = p->NTA;
        pa.NTB = p->NTB;
        pa.phases = p->phases;
        pa.bf16 = p->proj_bf16;
        int rc = launch_pack(pa, s);
        if (rc)
            return hip_fail((hipError_t)rc, "weight pack");
        p->packed_valid = p->constant_weights;
        p->packed_ws = workspace;
        p->packed_W = W;
        p->packed_R = R;
    }
    tm.end(STAGE_PACK);

    // 2. states, exchange buffers, barrier counters, lengths
    tm.begin(STAGE_OTHER);
    int32_t *lens_dev = (int32_t *)(ws + p->ws.lens);
    const int32_t *order_dev = nullptr;
    if (sequence_lens && noalloc) {
        // the lengths by position and the row order as kernel arguments
        InlineLens il;
        il.n = (int32_t)p->Bt;
        int32_t tmp[2 * kInlineRows];
        order_rows(sequence_lens, p->Bt, p->BT, il.lens, il.order, il.rank_pos, tmp);
        int rc = launch_lens_inline(il, lens_dev, s);
        if (rc)
            return hip_fail((hipError_t)rc, "sequence_lens (kernel arguments)");
        order_dev = lens_dev + p->Bt;
    } else if (sequence_lens) {
        // the lengths by position and the row order, staged in pinned memory
        // owned by the plan and copied on the stream
        if (!p->lens_host) {
            e = hipHostMalloc((void **)&p->lens_host, (size_t)p->Bt * 5 * sizeof(int32_t),
                              hipHostMallocDefault);
            if (e != hipSuccess)
                return hip_fail(e, "hipHostMalloc (sequence_lens staging)");
            hipEvent_t ev;
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
            if (e != hipSuccess)
                return hip_fail(e, "hipEventCreate");
            p->lens_event = ev;
        }
        if (p->lens_pending) {
            e = hipEventSynchronize((hipEvent_t)p->lens_event);   // the last run's copy is done
            if (e != hipSuccess)
                return hip_fail(e, "hipEventSynchronize (sequence_lens staging)");
            p->lens_pending = 0;
        }
        // lengths by position, the order, the positions by rank, then 2 Bt
        // values of sorting room (not copied)
        int32_t *hs = p->lens_host;
        order_rows(sequence_lens, p->Bt, p->BT, hs, hs + p->Bt, hs + 2 * p->Bt, hs + 3 * p->Bt);
        e = hipMemcpyAsync(lens_dev, hs, (size_t)p->Bt * 3 * sizeof(int32_t),
                           hipMemcpyHostToDevice, s);
        if (e != hipSuccess)
            return hip_fail(e, "sequence_lens copy");
        e = hipEventRecord((hipEvent_t)p->lens_event, s);
        if (e != hipSuccess)
            return hip_fail(e, "hipEventRecord (sequence_lens staging)");
        p->lens_pending = 1;
        order_dev = lens_dev + p->Bt;
    }
    InitArgs ia{};
    ia.h0 = initial_h;
    ia.c0 = p->op == RNN_OP_LSTM ? initial_c : nullptr;
    ia.hbuf = (float *)(ws + p->ws.hbuf);
    ia.sbuf = p->phases == 2 ? (float *)(ws + p->ws.sbuf) : nullptr;
    ia.cbuf = p->op == RNN_OP_LSTM ? (float *)(ws + p->ws.cbuf) : nullptr;
    ia.lens_dev = lens_dev;
    ia.order = order_dev;
    ia.fill_lens = sequence_lens ? -1 : (int32_t)p->S;
    ia.bar = (uint32_t *)(ws + p->ws.bar);
    ia.n_bar = n_flags(*p);
    ia.D = p->D;
    ia.Bt = p->Bt;
    ia.Btp = p->Btp;
    ia.H = p->H;
    ia.Hp = p->Hp;
    ia.layout = p->layout;
    int rc = launch_init(ia, s);
    if (rc)
        return hip_fail((hipError_t)rc, "state init");
    tm.end(STAGE_OTHER);

    // 3-4. per time chunk: the projection of the chunk's steps (both
    // directions in one launch), then its step loop
    const int64_t nchunks = (p->S + p->C - 1) / p->C;
    RecArgs ra = rec_args(*p, ws, B, P, Y, Y_h, Y_c);
    ra.order = order_dev;
    ra.X = X;
    for (int64_t ck = 0; ck < nchunks; ++ck) {
        const int64_t j0 = ck * p->C, j1 = std::min<int64_t>(p->S, j0 + p->C);
        if (ck == 0)
            tm.begin(STAGE_PROJ);
        // (a fused plan: the step loop computes the projections itself)
        if (!p->fused) {
            ProjArgs pr{};
            pr.X = X;
            pr.Xb = (uint16_t *)(ws + p->ws.xb);
            pr.Wp = ws + p->ws.wp;
            pr.XW = (float *)(ws + p->ws.xw);
            pr.K = p->I;
            pr.S = p->S;
            pr.Bt = p->Bt;
            pr.GH = (int64_t)p->G * p->H;
            pr.D = p->D;
            pr.steps = p->C;
            pr.j_base = j0;
            pr.lens = lens_dev;
            pr.order = order_dev;
            pr.rank_pos = order_dev ? order_dev + p->Bt : nullptr;
            // With sequence_lens and a product of many tiles, only the rows the
            // step loop reads in this chunk, listed on the device (for a small
            // product the extra launch costs more than the rows it saves, and
            // whole tiles with no row read are skipped anyway).
            pr.m_rows = p->C * p->Bt;
            const int64_t dense_tiles = p->D * ((p->C * p->Bt + 127) / 128) * ((pr.GH + 127) / 128);
            const bool row_list = sequence_lens && (p->proj_rows == 1 ||
                                                    (p->proj_rows == 0 && dense_tiles >= 2048));
            if (row_list) {
                pr.m_rows = 0;
                for (int64_t b = 0; b < p->Bt; ++b)
                    pr.m_rows += std::min<int64_t>(p->C, std::max<int64_t>(0, sequence_lens[b] - j0));
                int32_t *rowmap = (int32_t *)(ws + p->ws.rowmap);
                pr.rowmap = rowmap;
                rc = launch_proj_rows(pr, rowmap, s);
                if (rc)
                    return hip_fail((hipError_t)rc, "projection rows");
            }
            pr.reverse_only = p->reverse_only;
            pr.layout = p->layout;
            pr.bf16 = p->proj_bf16;
            pr.exact = p->exact;
            rc = launch_projection(pr, s);
            if (rc)
                return hip_fail((hipError_t)rc, "projection");
        }
        if (ck == 0) {
            tm.end(STAGE_PROJ);
            tm.begin(STAGE_REC);
        }
        ra.j_base = (int32_t)j0;
        if (persistent) {
            ra.q_begin = (int32_t)(j0 * p->phases);
            ra.q_end = (int32_t)(j1 * p->phases);
            rc = launch_recurrence(ra, p->resident, 1, s);
            if (rc)
                return hip_fail((hipError_t)rc, "recurrence (persistent)");
        } else {
            for (int64_t q = j0 * p->phases; q < j1 * p->phases; ++q) {
                ra.q_begin = (int32_t)q;
                ra.q_end = (int32_t)(q + 1);
                rc = launch_recurrence(ra, p->resident, 0, s);
                if (rc)
                    return hip_fail((hipError_t)rc, "recurrence (per step)");
            }
        }
    }
    tm.end(STAGE_REC);
    return RNN_OK;
}

}  // namespace

extern "C" rnn_status rnn_run(rnn_plan *p, void *hip_stream, void *workspace, size_t workspace_bytes,
                              const float *X, const float *W, const float *R, const float *B,
                              const int32_t *sequence_lens, const float *initial_h,
                              const float *initial_c, const float *P, float *Y, float *Y_h,
                              float *Y_c)
{
    set_error("");
    if (!p) {
        set_error("rnn_run: NULL plan");
        return RNN_ERR_INVALID_INPUT;
    }
    rnn_status st = run_checks(p, workspace, workspace_bytes, X, W, R, B, sequence_lens, initial_h,
                               initial_c, P, Y, Y_h, Y_c);
    if (st != RNN_OK)
        return st;
    return run_enqueue(p, (hipStream_t)hip_stream, workspace, X, W, R, B, sequence_lens, initial_h,
                       initial_c, P, Y, Y_h, Y_c);
}

extern "C" rnn_status rnn_cell_run(rnn_plan *p, void *hip_stream, void *workspace,
                                   size_t workspace_bytes, const float *X, const float *H,
                                   const float *C, const float *W, const float *R,
                                   const float *B_sum, const float *P, float *H_out, float *C_out)
{
    set_error("");
    if (!p) {
        set_error("rnn_cell_run: NULL plan");
        return RNN_ERR_INVALID_INPUT;
    }
    if (p->S != 1 || p->D != 1) {
        set_error("rnn_cell_run: the plan must have seq_length 1 and one direction");
        return RNN_ERR_INVALID_INPUT;
    }
    if (!H_out && p->Bt > 0) {
        set_error("rnn_cell_run: H_out is required");
        return RNN_ERR_INVALID_INPUT;
    }
    if (B_sum && p->op == RNN_OP_GRU && p->lbr) {
        set_error("rnn_cell_run: a summed bias cannot express GRU with linear_before_reset = 1 "
                  "(its recurrent candidate bias is scaled by the reset gate)");
        return RNN_ERR_INVALID_INPUT;
    }
    if (B_sum && !aligned(B_sum, 4)) {
        set_error("rnn_run: tensors must be 4-byte aligned");
        return RNN_ERR_INVALID_INPUT;
    }
    // the expanded bias lives in the workspace; checked as rnn_run checks it
    const float *B = nullptr;
    if (B_sum && p->Bt > 0 && workspace)
        B = (const float *)((unsigned char *)workspace + p->ws.cellb);
    rnn_status st = run_checks(p, workspace, workspace_bytes, X, W, R, B, nullptr, H, C, P,
                               nullptr, H_out, C_out);
    if (st != RNN_OK)
        return st;
    hipStream_t s = (hipStream_t)hip_stream;
    if (B) {
        int rc = launch_cell_bias(B_sum, (float *)B, p->D, (int64_t)p->G * p->H, s);
        if (rc)
            return hip_fail((hipError_t)rc, "summed-bias expansion");
    }
    return run_enqueue(p, s, workspace, X, W, R, B, nullptr, H, C, P, nullptr, H_out, C_out);
}

// ---------------------------------------------------------------------------
// rnn_run_noalloc: rnn_run without a caller workspace and without any
// allocation.  Its scratch is one file-scope device array per GPU, of
// RNN_NOALLOC_SCRATCH_BYTES; every call on a GPU shares that GPU's array (a
// second call overlapping the first on the same GPU races with it).
// ---------------------------------------------------------------------------
namespace {

static_assert(RNN_NOALLOC_MAX_LENS_BATCH == kInlineRows, "inline lengths limit");

static __device__ __align__(256) unsigned char scratch[RNN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` on each GPU

// The address of this GPU's copy of `scratch`, looked up once per device with
// that device current.  In host code the array's own name is only a host-side
// stand-in, so every use goes through the address kept here.
rnn_status scratch_of_current_device(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("rnn_run_noalloc: device index beyond the library's table");
        return RNN_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress (scratch)");
        if (!ptr || !aligned(ptr, 256)) {
            set_error("rnn_run_noalloc: scratch address is not 256-byte aligned");
            return RNN_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return RNN_OK;
}

}  // namespace

extern "C" rnn_status rnn_run_noalloc(rnn_plan *p, void *hip_stream, const float *X,
                                      const float *W, const float *R, const float *B,
                                      const int32_t *sequence_lens, const float *initial_h,
                                      const float *initial_c, const float *P, float *Y,
                                      float *Y_h, float *Y_c)
{
    set_error("");
    if (!p) {
        set_error("rnn_run_noalloc: NULL plan");
        return RNN_ERR_INVALID_INPUT;
    }
    const bool zero = p->S == 0 || p->Bt == 0;
    // the limits first: refused before any device call
    if (!zero && p->ws.total > (size_t)RNN_NOALLOC_SCRATCH_BYTES) {
        set_error("rnn_run_noalloc: this plan needs " + std::to_string(p->ws.total) +
                  " bytes of scratch, more than the " +
                  std::to_string((size_t)RNN_NOALLOC_SCRATCH_BYTES) +
                  " the allocation-free entry point holds; use rnn_run with a workspace");
        return RNN_ERR_UNSUPPORTED;
    }
    if (!zero && sequence_lens && p->Bt > RNN_NOALLOC_MAX_LENS_BATCH) {
        set_error("rnn_run_noalloc: sequence_lens with more than " +
                  std::to_string(RNN_NOALLOC_MAX_LENS_BATCH) +
                  " batch rows; use rnn_run with a workspace");
        return RNN_ERR_UNSUPPORTED;
    }
    void *ws = nullptr;
    rnn_status st = run_checks(p, nullptr, 0, X, W, R, B, sequence_lens, initial_h, initial_c, P,
                               Y, Y_h, Y_c, /*check_workspace=*/false);
    if (st != RNN_OK)
        return st;
    if (!zero) {
        st = scratch_of_current_device(&ws);
        if (st != RNN_OK)
            return st;
    }
    return run_enqueue(p, (hipStream_t)hip_stream, ws, X, W, R, B, sequence_lens, initial_h,
                       initial_c, P, Y, Y_h, Y_c, /*noalloc=*/true);
}

extern "C" rnn_status rnn_workspace_check(const rnn_plan *p, void *hip_stream, const void *workspace)
{
    if (!p || !workspace) {
        set_error("rnn_workspace_check: NULL argument");
        return RNN_ERR_INVALID_INPUT;
    }
    if (p->S == 0 || p->Bt == 0)
        return RNN_OK;
    hipError_t e = hipStreamSynchronize((hipStream_t)hip_stream);
    if (e != hipSuccess)
        return hip_fail(e, "hipStreamSynchronize");
    int32_t err = 0;
    const unsigned char *ws = (const unsigned char *)workspace;
    e = hipMemcpy(&err, ws + p->ws.bar + (size_t)n_flags(*p) * 4, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return hip_fail(e, "error word read");
    if (err) {
        set_error("a step barrier timed out on the device");
        return RNN_ERR_DEVICE;
    }
    return RNN_OK;
}

extern "C" rnn_status rnn_plan_enable_timing(rnn_plan *p, int32_t enable)
{
    if (!p) {
        set_error("rnn_plan_enable_timing: NULL plan");
        return RNN_ERR_INVALID_INPUT;
    }
    p->timing = enable ? 1 : 0;
    if (p->timing && p->dev_ready) {
        for (int i = 0; i < 2 * STAGE_COUNT; ++i)
            if (!p->events[i]) {
                hipEvent_t ev;
                hipError_t e = hipEventCreate(&ev);
                if (e != hipSuccess)
                    return hip_fail(e, "hipEventCreate");
                p->events[i] = ev;
            }
    }
    return RNN_OK;
}

extern "C" rnn_status rnn_plan_last_timings(rnn_plan *p, float *ms, int32_t n)
{
    if (!p || !ms) {
        set_error("rnn_plan_last_timings: NULL argument");
        return RNN_ERR_INVALID_INPUT;
    }
    if (!p->events_recorded) {
        set_error("rnn_plan_last_timings: no timed run");
        return RNN_ERR_INVALID_INPUT;
    }
    for (int i = 0; i < n && i < STAGE_COUNT; ++i) {
        hipError_t e = hipEventSynchronize((hipEvent_t)p->events[2 * i + 1]);
        if (e != hipSuccess)
            return hip_fail(e, "hipEventSynchronize");
        float v = 0.0f;
        e = hipEventElapsedTime(&v, (hipEvent_t)p->events[2 * i], (hipEvent_t)p->events[2 * i + 1]);
        if (e != hipSuccess)
            return hip_fail(e, "hipEventElapsedTime");
        ms[i] = v;
    }
    return RNN_OK;
}

extern "C" void rnn_plan_destroy(rnn_plan *p)
{
    if (!p)
        return;
    for (int i = 0; i < 2 * STAGE_COUNT; ++i)
        if (p->events[i])
            (void)hipEventDestroy((hipEvent_t)p->events[i]);
    if (p->lens_event) {
        (void)hipEventSynchronize((hipEvent_t)p->lens_event);
        (void)hipEventDestroy((hipEvent_t)p->lens_event);
    }
    if (p->lens_host)
        (void)hipHostFree(p->lens_host);
    delete p;
}
