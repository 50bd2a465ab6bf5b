// plan.cpp -- host-side plan creation for the ONNX recurrent operators:
// attribute parsing (activation names, defaults and alpha/beta cursors of the
// onemodel page's "Activations" section), the checks of its "Choices the
// specification leaves open" and "Limits" sections, the recurrence tiling and
// the workspace layout.  Pure C++: no device call happens here, so every
// plan-time error can be produced on a machine without a GPU.
#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "common.h"

namespace rnnamd {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Units [u0, u0 + uc) of unit block ub.
void block_columns(const rnn_plan &p, int64_t ub, int32_t *u0, int32_t *uc)
{
    int64_t s = ub * p.U;
    *u0 = (int32_t)s;
    *uc = (int32_t)std::min<int64_t>(p.U, p.H - s);
}

namespace {

struct NameKind {
    const char *name;
    int32_t kind;
};
const NameKind kNames[] = {
    {"sigmoid", ACT_SIGMOID},       {"tanh", ACT_TANH},
    {"relu", ACT_RELU},             {"affine", ACT_AFFINE},
    {"leakyrelu", ACT_LEAKYRELU},   {"thresholdedrelu", ACT_THRESHOLDEDRELU},
    {"scaledtanh", ACT_SCALEDTANH}, {"hardsigmoid", ACT_HARDSIGMOID},
    {"elu", ACT_ELU},               {"softsign", ACT_SOFTSIGN},
    {"softplus", ACT_SOFTPLUS},
};

int32_t kind_of(const char *name)
{
    if (!name)
        return -1;
    std::string low;
    for (const char *c = name; *c; ++c)
        low.push_back((char)std::tolower((unsigned char)*c));
    for (const auto &nk : kNames)
        if (low == nk.name)
            return nk.kind;
    return -1;
}

bool uses_alpha(int32_t k)
{
    return k == ACT_AFFINE || k == ACT_SCALEDTANH || k == ACT_HARDSIGMOID ||
           k == ACT_LEAKYRELU || k == ACT_THRESHOLDEDRELU || k == ACT_ELU;
}
bool uses_beta(int32_t k) { return k == ACT_AFFINE || k == ACT_SCALEDTANH || k == ACT_HARDSIGMOID; }

float alpha_default(int32_t k)
{
    switch (k) {
    case ACT_LEAKYRELU: return 0.01f;
    case ACT_HARDSIGMOID: return 0.2f;
    case ACT_THRESHOLDEDRELU:
    case ACT_ELU:
    case ACT_AFFINE:
    case ACT_SCALEDTANH: return 1.0f;
    default: return 0.0f;
    }
}
float beta_default(int32_t k) { return k == ACT_HARDSIGMOID ? 0.5f : 0.0f; }

rnn_status resolve_activations(const rnn_attrs &a, rnn_plan &p)
{
    const int na = p.op == RNN_OP_LSTM ? 3 : p.op == RNN_OP_GRU ? 2 : 1;
    static const int32_t defaults[3][3] = {{ACT_TANH, 0, 0},
                                           {ACT_SIGMOID, ACT_TANH, 0},
                                           {ACT_SIGMOID, ACT_TANH, ACT_TANH}};
    if (a.n_activations == 0 || a.activations == nullptr) {
        for (int d = 0; d < p.D; ++d)
            for (int j = 0; j < na; ++j) {
                int32_t k = defaults[p.op][j];
                p.act[d][j] = {k, alpha_default(k), beta_default(k)};
            }
        return RNN_OK;
    }
    if (!(a.n_activations == na || (p.D == 2 && a.n_activations == 2 * na))) {
        set_error("activations: expected " + std::to_string(na) + " names per direction set, got " +
                  std::to_string(a.n_activations));
        return RNN_ERR_INVALID_INPUT;
    }
    ActSpec list[6];
    int ca = 0, cb = 0;
    for (int i = 0; i < a.n_activations; ++i) {
        int32_t k = kind_of(a.activations[i]);
        if (k < 0) {
            set_error(std::string("activations: unknown name '") +
                      (a.activations[i] ? a.activations[i] : "(null)") + "'");
            return RNN_ERR_INVALID_INPUT;
        }
        ActSpec s{k, alpha_default(k), beta_default(k)};
        // separate cursors for alpha and beta, walked in activation order
        if (uses_alpha(k) && ca < a.n_alpha && a.activation_alpha)
            s.alpha = a.activation_alpha[ca++];
        if (uses_beta(k) && cb < a.n_beta && a.activation_beta)
            s.beta = a.activation_beta[cb++];
        list[i] = s;
    }
    for (int d = 0; d < p.D; ++d)
        for (int j = 0; j < na; ++j)
            p.act[d][j] = (a.n_activations == na) ? list[j] : list[d * na + j];
    return RNN_OK;
}

// Column tiles of one unit block for a unit count uc.
void tiles_for(const rnn_plan &p, int uc, int *nta, int *ntb)
{
    if (p.op == RNN_OP_GRU && !p.lbr) {
        *nta = (2 * uc + 15) / 16;
        *ntb = (uc + 15) / 16;
    } else {
        *nta = (p.G * uc + 15) / 16;
        *ntb = 0;
    }
}

// The recurrence kernel is compiled for these shapes only (recurrence.hip).
// R in registers: 2 or 4 row tiles, 1 or 2 column tiles, 8 or 16 k blocks of
// 16 per wave, at most 2 (row, unit) pairs per thread.
bool resident_ok(int nw, int nt, int nta, int phases, int kb, int mt, int pairs)
{
    const bool tiles = phases == 1 ? nt <= 2 : (nt == 2 && nta == 1 && mt == 2);
    // R slice per wave: nt * kb * 4 registers; 4 waves run one wave per SIMD
    // (512 registers), 8 waves two (256 registers each)
    const bool kbs = nw == 4 ? (kb == 8 || kb == 16) : (kb == 4 || kb == 8);
    return (mt == 2 || mt == 4) && tiles && kbs && pairs <= 2;
}

// R streamed every step (4 waves): 1, 2, 3, 4 or 6 column tiles for one
// phase; for two (GRU lbr=0) 1+1, 2+1 or 4+2; at most 8 pairs.  A batch tile
// of 128 rows (mt 8) holds at most 3 column tiles (more spill registers).
bool streamed_ok(int nw, int nt, int nta, int phases, int pairs, int mt)
{
    if (nw != 4 || (mt == 8 && nt > 3))
        return false;
    const bool tiles = phases == 1 ? (nt == 1 || nt == 2 || nt == 3 || nt == 4 || nt == 6)
                                   : ((nt == 2 && nta == 1) || (nt == 3 && nta == 2) ||
                                      (nt == 6 && nta == 4));
    return tiles && pairs <= kMaxPairs;
}

// Choose the batch tile and the units per workgroup: at most kMaxWorkgroups
// workgroups, the least matrix-core work per wave per step, then the larger
// batch tile (rows are held in order of decreasing length, so a tile that
// holds more of them keeps its workgroups busy while the shortest rows end,
// instead of leaving a whole block of workgroups idle), then the fewest
// workgroups.
rnn_status choose_tiling(const rnn_attrs &a, rnn_plan &p)
{
    if (a.batch_tile) {
        if (a.batch_tile != 16 && a.batch_tile != 32 && a.batch_tile != 64 &&
            a.batch_tile != 128) {
            set_error("batch_tile must be 0, 16, 32, 64 or 128");
            return RNN_ERR_INVALID_INPUT;
        }
        if (a.batch_tile == 128 && p.exact) {
            set_error("batch_tile = 128 is a fast-mode tiling (R streamed)");
            return RNN_ERR_INVALID_INPUT;
        }
        p.BT = a.batch_tile;
    } else {
        p.BT = p.Bt <= 16 ? 16 : p.Bt <= 32 ? 32 : 64;
    }
    // a tile of 128 rows is tried beside the automatic one for larger
    // batches (fast mode, R streamed)
    const int bt_alt = (!a.batch_tile && !p.exact && p.Bt > 64) ? 128 : 0;
    p.phases = (p.op == RNN_OP_GRU && !p.lbr) ? 2 : 1;
    if (a.waves_per_block != 0 && a.waves_per_block != 4 && a.waves_per_block != 8) {
        set_error("waves_per_block must be 0, 4 or 8");
        return RNN_ERR_INVALID_INPUT;
    }
    auto set_waves = [&](int nw) {
        p.NW = nw;
        p.Hp = round_up(std::max<int64_t>(p.H, 1), 16 * nw);
        p.KB = (int32_t)(p.Hp / (16 * nw));
    };
    set_waves(a.waves_per_block ? a.waves_per_block : 4);

    auto set_tile = [&](int bt) {
        p.BT = bt;
        p.MT = bt / 16;
        p.NBB = (int32_t)std::max<int64_t>(1, (p.Bt + bt - 1) / bt);
        p.Btp = (int64_t)p.NBB * bt;
    };
    set_tile(p.BT);
    bool cap_wg = true;   // first look for tilings whose workgroups fit at once
    auto evaluate = [&](int u, int *nta, int *ntb, bool *res, long *cost) -> bool {
        int nub = (int)((p.H + u - 1) / u);
        long wg = (long)p.D * p.NBB * nub;
        if (cap_wg && wg > kMaxWorkgroups && !a.units_per_block)
            return false;
        const int nthr = 64 * p.NW;
        if ((long)p.BT * u > (long)nthr * kMaxPairs)
            return false;
        tiles_for(p, u, nta, ntb);
        int nt = *nta + *ntb;
        int pairs = (p.BT * u + nthr - 1) / nthr;
        *res = resident_ok(p.NW, nt, *nta, p.phases, p.KB, p.MT, pairs);
        if (!*res && !streamed_ok(p.NW, nt, *nta, p.phases, pairs, p.MT))
            return false;
        long lds = ((long)p.NW * nt * 16 * (p.BT + 4) + 3L * p.BT * u + 2L * p.BT + 11L * u) * 4;
        if (lds > 160 * 1024)
            return false;
        *cost = (long)p.MT * nt * p.KB * 16 + (*res ? 0 : (long)p.MT * nt * p.KB * 4);
        return true;
    };

    int best_u = -1, bnta = 0, bntb = 0, bbt = p.BT;
    bool bres = false;
    long bcost = 0;
    if (a.units_per_block) {
        int u = a.units_per_block;
        if (u < 1 || u > p.H) {
            set_error("units_per_block out of range");
            return RNN_ERR_INVALID_INPUT;
        }
        long c;
        bool r;
        if (!evaluate(u, &bnta, &bntb, &r, &c)) {
            set_error("units_per_block gives an unsupported tiling");
            return RNN_ERR_INVALID_INPUT;
        }
        best_u = u;
        bres = r;
    } else {
        const int tiles[2] = {p.BT, bt_alt};
        for (int pass = 0; pass < 2 && best_u < 0; ++pass) {
            cap_wg = pass == 0;   // second pass: more workgroups, run one step per launch
            for (int ti = 0; ti < 2; ++ti) {
                if (!tiles[ti])
                    continue;
                set_tile(tiles[ti]);
                for (int u = 1; u <= std::min<int64_t>(p.H, 128); ++u) {
                    int nta, ntb;
                    bool r;
                    long c;
                    if (!evaluate(u, &nta, &ntb, &r, &c))
                        continue;
                    // (a 128-row tile runs the streamed kernel only)
                    if (p.BT == 128 && r)
                        continue;
                    const bool better = best_u < 0 || c < bcost ||
                                        (c == bcost && (p.BT > bbt || (p.BT == bbt && u > best_u)));
                    if (better) {
                        best_u = u;
                        bcost = c;
                        bnta = nta;
                        bntb = ntb;
                        bres = r;
                        bbt = p.BT;
                    }
                }
            }
        }
        set_tile(bbt);
        if (best_u < 0) {
            set_error("no recurrence tiling fits this shape");
            return RNN_ERR_UNSUPPORTED;
        }
    }
    p.U = best_u;
    p.NUB = (int32_t)((p.H + p.U - 1) / p.U);
    p.NTA = bnta;
    p.NTB = bntb;
    p.NT = bnta + bntb;
    p.resident = bres ? 1 : 0;
    p.n_wg = p.D * p.NBB * p.NUB;

    // Two half-batch sub-steps per step (rec_pipe_kernel): R resident, four
    // waves, one phase per step, at most two pairs per thread and half.
    const bool halves_ok = p.resident && p.NW == 4 && p.phases == 1 && (p.MT == 2 || p.MT == 4) &&
                           p.NT <= 2 && (p.KB == 8 || p.KB == 16) &&
                           (long)(p.BT / 2) * p.U <= 2L * 256;
    if (a.batch_halves < 0 || a.batch_halves > 2) {
        set_error("batch_halves must be 0, 1 or 2");
        return RNN_ERR_INVALID_INPUT;
    }
    if (a.batch_halves == 2 && !halves_ok) {
        set_error("batch_halves = 2 needs R resident, a single-phase operator and a batch tile of 32 or 64");
        return RNN_ERR_INVALID_INPUT;
    }
    p.halves = (halves_ok && a.batch_halves != 1) ? 2 : 1;
    if (p.exact) {
        p.halves = 1;                              // the exact kernel has one form
        if (a.batch_halves == 2) {
            set_error("batch_halves = 2 is a fast-mode schedule; exact mode has one form");
            return RNN_ERR_INVALID_INPUT;
        }
        if (p.NT * 16 > 128) {
            set_error("exact mode supports at most 128 gate columns per workgroup");
            return RNN_ERR_UNSUPPORTED;
        }
    }

    // The projection inside the two-half step loop (rec_fused_kernel), on
    // request only: fast mode, an fp32 projection, I in whole 256-input
    // ranges and the workgroup's slice of W within LDS.  It needs no XW
    // buffer (bidirectional LSTM, hidden 1024, batch 64, 512 steps: 0.34
    // instead of 1.41 GB of workspace) but measured slower than the separate
    // projection launch (10.2 against 9.0 ms there).
    const bool fused_ok = p.halves == 2 && !p.exact && !p.proj_bf16 &&
                          recurrence_fused_supported(p.BT, p.NT, p.U, p.I);
    if (a.fuse_projection < 0 || a.fuse_projection > 2) {
        set_error("fuse_projection must be 0, 1 or 2");
        return RNN_ERR_INVALID_INPUT;
    }
    if (a.fuse_projection == 2 && !fused_ok) {
        set_error("fuse_projection = 2 needs the two-half schedule in fast mode, an fp32 projection, "
                  "input_size a multiple of 256 and the workgroup's W slice within LDS");
        return RNN_ERR_INVALID_INPUT;
    }
    p.fused = (fused_ok && a.fuse_projection == 2) ? 1 : 0;
    return RNN_OK;
}

void make_layout(rnn_plan &p)
{
    Layout &L = p.ws;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (size_t)round_up((int64_t)bytes, 256);
        return o;
    };
    const size_t GH = (size_t)p.G * p.H;
    const size_t wsz = p.proj_bf16 ? 2 : 4;
    L.wp = take((size_t)p.D * GH * p.I * wsz);
    L.rp = take((size_t)p.D * p.NUB * p.NT * 16 * p.Hp * 4);
    L.xb = take(p.proj_bf16 ? (size_t)p.D * p.C * p.Bt * p.I * 2 : 0);
    L.xw = take(p.fused ? 0 : (size_t)p.D * p.C * p.Bt * GH * 4);   // (fused: no XW)
    L.hbuf = take((size_t)(p.C + 1) * p.D * p.Btp * p.Hp * 4);
    L.sbuf = take(p.phases == 2 ? (size_t)p.C * p.D * p.Btp * p.Hp * 4 : 0);
    L.cbuf = take(p.op == RNN_OP_LSTM ? (size_t)p.D * p.Bt * p.H * 4 : 0);
    L.zbuf = take(p.phases == 2 ? (size_t)p.D * p.Bt * p.H * 4 : 0);
    L.rowmap = take(p.fused ? 0 : (size_t)p.C * std::max<int64_t>(p.Bt, 1) * 4);
    L.lens = take((size_t)std::max<int64_t>(p.Bt, 1) * 3 * 4);   // lengths by position, order, positions by rank
    L.bar = take((size_t)(n_flags(p) + 1) * 4);
    L.cellb = take((size_t)p.D * 2 * GH * 4);
#ifdef RNN_STAMPS
    L.stamps = take((size_t)kStampSlots * kStampEvents * 8);
#endif
    L.total = off;
}

}  // namespace
}  // namespace rnnamd

using namespace rnnamd;

extern "C" const char *rnn_last_error(void) { return g_last_error.c_str(); }

extern "C" rnn_status rnn_plan_create(const rnn_attrs *attrs, const rnn_dims *dims, rnn_plan **out)
{
    set_error("");
    if (!attrs || !dims || !out) {
        set_error("rnn_plan_create: NULL argument");
        return RNN_ERR_INVALID_INPUT;
    }
    *out = nullptr;
    const rnn_attrs &a = *attrs;
    rnn_plan *p = new (std::nothrow) rnn_plan();
    if (!p) {
        set_error("rnn_plan_create: out of host memory");
        return RNN_ERR_OUT_OF_MEMORY;
    }
    auto fail = [&](rnn_status s, const std::string &m) {
        if (!m.empty())
            set_error(m);
        delete p;
        return s;
    };
    if (a.op != RNN_OP_RNN && a.op != RNN_OP_GRU && a.op != RNN_OP_LSTM)
        return fail(RNN_ERR_INVALID_INPUT, "unknown op");
    p->op = a.op;
    p->G = a.op == RNN_OP_LSTM ? 4 : a.op == RNN_OP_GRU ? 3 : 1;
    int want_d = 1;
    if (a.direction == nullptr || std::strcmp(a.direction, "forward") == 0) {
        want_d = 1;
    } else if (std::strcmp(a.direction, "reverse") == 0) {
        want_d = 1;
        p->reverse_only = 1;
    } else if (std::strcmp(a.direction, "bidirectional") == 0) {
        want_d = 2;
    } else {
        return fail(RNN_ERR_INVALID_INPUT, "direction must be forward, reverse or bidirectional");
    }
    if (dims->num_directions != want_d)
        return fail(RNN_ERR_INVALID_INPUT, "num_directions does not match direction");
    p->D = want_d;
    if (a.layout != 0 && a.layout != 1)
        return fail(RNN_ERR_INVALID_INPUT, "layout must be 0 or 1");
    p->layout = a.layout;
    if (dims->seq_length < 0 || dims->batch_size < 0 || dims->input_size < 0 || dims->hidden < 0)
        return fail(RNN_ERR_INVALID_INPUT, "negative dimension");
    if (dims->hidden == 0)
        return fail(RNN_ERR_INVALID_INPUT, "hidden size is zero");
    if (a.hidden_size != 0 && a.hidden_size != dims->hidden)
        return fail(RNN_ERR_INVALID_INPUT, "hidden_size does not match R's last dimension");
    if (a.op != RNN_OP_LSTM && a.input_forget)
        return fail(RNN_ERR_INVALID_INPUT, "input_forget is an LSTM attribute");
    if (a.op != RNN_OP_GRU && a.linear_before_reset)
        return fail(RNN_ERR_INVALID_INPUT, "linear_before_reset is a GRU attribute");
    if (a.proj_dtype != RNN_PROJ_F32 && a.proj_dtype != RNN_PROJ_BF16)
        return fail(RNN_ERR_INVALID_INPUT, "proj_dtype must be F32 or BF16");
    if (a.kernel_path < RNN_PATH_AUTO || a.kernel_path > RNN_PATH_PER_STEP)
        return fail(RNN_ERR_INVALID_INPUT, "unknown kernel_path");
    p->S = dims->seq_length;
    p->Bt = dims->batch_size;
    p->I = dims->input_size;
    p->H = dims->hidden;
    p->clip_on = (a.has_clip && a.clip > 0.0f) ? 1 : 0;   // only when given and positive
    p->clip = a.clip;
    p->input_forget = a.input_forget ? 1 : 0;
    p->lbr = a.linear_before_reset ? 1 : 0;
    p->proj_bf16 = a.proj_dtype == RNN_PROJ_BF16;
    p->constant_weights = a.constant_weights ? 1 : 0;
    p->kernel_path = a.kernel_path;
    if (a.time_chunk < 0)
        return fail(RNN_ERR_INVALID_INPUT, "time_chunk must be >= 0");
    if (a.exact != 0 && a.exact != 1)
        return fail(RNN_ERR_INVALID_INPUT, "exact must be 0 or 1");
    p->exact = a.exact;
    p->C = (a.time_chunk > 0 && a.time_chunk < p->S) ? a.time_chunk : p->S;
    if (a.barrier_spin_limit < 0)
        return fail(RNN_ERR_INVALID_INPUT, "barrier_spin_limit must be >= 0");
    p->spin_limit = a.barrier_spin_limit ? (uint32_t)a.barrier_spin_limit : kDefaultSpinLimit;
    // Fault injection for tests of the barrier time-out: with this set, the
    // step loops never store their flags, so every wait between steps runs
    // out its (bounded) spin limit and the kernel then finishes normally.
    {
        const char *e = std::getenv("RNN_AMD_TEST_WITHHOLD_FLAGS");
        p->withhold_flags = (e && *e && *e != '0') ? 1 : 0;
    }
    // Which rows the projection computes with sequence_lens (test switch):
    // "list" always the list of rows read, "tiles" always whole tiles (those
    // with no row read skipped); unset, the list when the product is large.
    {
        const char *e = std::getenv("RNN_AMD_TEST_PROJ_ROWS");
        p->proj_rows = !e ? 0 : std::strcmp(e, "list") == 0 ? 1 : std::strcmp(e, "tiles") == 0 ? 2 : 0;
    }
#ifdef RNN_STAMPS
    {
        const char *e = std::getenv("RNN_AMD_STAMP_WG");
        p->stamp_wg = e ? std::atoi(e) : 0;
    }
#endif

    rnn_status st = resolve_activations(a, *p);
    if (st != RNN_OK)
        return fail(st, "");

    // Limits: per direction, seq*batch*G*H + 4*batch*H (+ transposed weights
    // when not constant) floats must stay below 2^30.  With time chunks the
    // projections held at once are those of one chunk: seq becomes the chunk
    // length (the limit the chunked form lifts).
    double need = (double)p->C * (double)p->Bt * p->G * (double)p->H + 4.0 * (double)p->Bt * p->H;
    if (!p->constant_weights)
        need += (double)p->G * p->H * ((double)p->I + (double)p->H);
    if (!(need < 1073741824.0))
        return fail(RNN_ERR_UNSUPPORTED, "per-direction scratch reaches 2^30 floats");
    if (p->H > 65536 || p->I > (int64_t)1 << 30 || p->S > INT32_MAX || p->Bt > INT32_MAX)
        return fail(RNN_ERR_UNSUPPORTED, "dimension beyond this library's index range");

    if (p->S > 0 && p->Bt > 0) {
        st = choose_tiling(a, *p);
        if (st != RNN_OK)
            return fail(st, "");
        make_layout(*p);
    }
    *out = p;
    return RNN_OK;
}

extern "C" rnn_status rnn_plan_workspace_size(const rnn_plan *plan, size_t *bytes)
{
    if (!plan || !bytes) {
        set_error("rnn_plan_workspace_size: NULL argument");
        return RNN_ERR_INVALID_INPUT;
    }
    *bytes = (plan->S > 0 && plan->Bt > 0) ? plan->ws.total : 0;
    return RNN_OK;
}

extern "C" rnn_status rnn_plan_describe(const rnn_plan *p, char *buf, size_t len)
{
    if (!p || !buf || len == 0) {
        set_error("rnn_plan_describe: NULL argument");
        return RNN_ERR_INVALID_INPUT;
    }
    std::snprintf(buf, len,
                  "op=%d G=%d D=%d S=%lld C=%lld Bt=%lld I=%lld H=%lld U=%d NUB=%d BT=%d NBB=%d "
                  "MT=%d NTA=%d NTB=%d phases=%d Hp=%lld waves=%d KB=%d resident=%d halves=%d "
                  "fused=%d exact=%d workgroups=%d path=%d persist=%d ws=%zu stamps=%zu",
                  p->op, p->G, p->D, (long long)p->S, (long long)p->C, (long long)p->Bt,
                  (long long)p->I,
                  (long long)p->H, p->U, p->NUB, p->BT, p->NBB, p->MT, p->NTA, p->NTB, p->phases,
                  (long long)p->Hp, p->NW, p->KB, p->resident, p->halves, p->fused, p->exact, p->n_wg,
                  p->kernel_path,
                  p->can_persist, p->ws.total, p->ws.stamps);
    return RNN_OK;
}
