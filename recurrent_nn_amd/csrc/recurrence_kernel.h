// recurrence_kernel.h -- the step loop of the ONNX recurrent operators: the
// recurrent product Rec = H . R^T for the whole batch, then the gate
// arithmetic per row in the written order (onemodel "Recurrent operators",
// section "Computation", steps 2 and 3 and the pre-activation / LSTM / GRU /
// RNN paragraphs), sequence_lens masking and reverse traversal ("Choices the
// specification leaves open"), and the Y / Y_h / Y_c writers for both layouts
// with NaN written as 0x7FC00000 ("Exact mode").
//
// Work split.  A workgroup owns (direction d, batch block bb of BT rows, unit
// block ub of U hidden units) and computes every gate column of its units, so
// the gate arithmetic of a unit never leaves the workgroup.  Its NW (4 or 8)
// waves split the reduction index k of the product (Hp / NW each) and compute
// the whole [BT x 16*NT] tile over their k range with v_mfma_f32_16x16x4_f32;
// the partial tiles meet in LDS and are summed in a fixed order (w = 0, 1,
// ...), so the result does not depend on the grid size.  With `RES` the wave's
// slice of R stays in registers for the whole sequence; otherwise it is
// re-read (from L2 / the memory-side cache) every step.
//
// Steps.  The persistent form runs every step in one cooperative launch.  H
// is exchanged through a history buffer in device memory: step j reads plane
// j and writes plane j + 1 with agent-coherent (write-through) stores, so no
// cache ever holds a stale copy of a plane and no whole-cache writeback or
// invalidate is needed between steps.  Steps are separated by a barrier
// among the workgroups of one (d, bb) group built on one flag per workgroup
// (no contended counter).  GRU with linear_before_reset = 0 has two phases
// per step: z and r first (their product over H), then the candidate's
// product over r (.) H_prev, with a barrier in between.  The per-step form
// runs one phase per launch, the kernel boundary being the barrier.
//
// Activation sets known per launch (the defaults, HardSigmoid/Tanh) are
// compiled into their own kernels; any other set goes through a run-time
// switch.
//
// Epilogue.  This file is compiled with -ffp-contract=off: every written
// addition and multiplication is its own IEEE operation, in the written order
// (the page allows fused multiply-adds only inside the products).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "activations.h"
#include "common.h"

namespace rnnamd {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cycle stamps (instrumented build only, -DRNN_STAMPS): thread 0 of workgroup
// a.stamp_wg stores the shader clock for event e of slot `slot` (a phase or a
// half-step of the launch).  Compiled out otherwise.
#ifdef RNN_STAMPS
#define RNN_STAMP(slot, e)                                                                        \
    do {                                                                                         \
        if ((int)blockIdx.x == a.stamp_wg && threadIdx.x == 0 && (slot) >= 0 &&                  \
            (slot) < kStampSlots)                                                                \
            a.stamps[(size_t)(slot) * kStampEvents + (e)] = __builtin_amdgcn_s_memtime();        \
    } while (0)
#else
#define RNN_STAMP(slot, e) do { } while (0)
#endif

// Agent-coherent store (write-through to the device coherence point, no
// dirty line left in this XCD's L2): how H and r (.) H_prev are published.
__device__ __forceinline__ void store_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until flags[0 .. n) all reach `target` (one wave; every lane reads a
// share of the flags).  More than spin_limit polls raises the error word and
// stops waiting.
__device__ __forceinline__ void wave_wait_flags(const uint32_t *flags, int n, uint32_t target,
                                                int32_t *err, uint32_t spin_limit, bool &dead)
{
    const int lane = threadIdx.x & 63;
    uint32_t polls = 0;
    for (;;) {
        bool ok = true;
        for (int i = lane; i < n; i += 64)
            ok = ok && __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target;
        if (__all(ok))
            break;
        __builtin_amdgcn_s_sleep(1);
        if (++polls > spin_limit) {
            if (lane == 0)
                __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            dead = true;
            break;
        }
    }
    asm volatile("" ::: "memory");   // no later load is moved above the wait
}

// First and last H column of the 64-column (256-byte) spans that hold the
// columns [k0, k1) of a plane row (rows start 256-byte aligned: Hp is a
// multiple of 64).
__device__ __forceinline__ int kline_lo(int k0) { return k0 & ~63; }
__device__ __forceinline__ int kline_hi(int k1, int Hp) { return min(Hp, (k1 + 63) & ~63) - 1; }

// Step hand-over among the NUB workgroups of one (direction, batch block)
// group when the waves split k: the workgroup publishes "phase q done" in its
// own flag once every wave's coherent stores have completed (the barrier
// also ends this phase's reads of the partial tiles), then each wave waits
// only for the flags of the unit blocks [lo, lo + n) that write the cache
// lines its own k range reads.
__device__ __forceinline__ void group_publish_wait(uint32_t *flags, int me, uint32_t target, int lo,
                                                   int n, int32_t *err, uint32_t spin_limit,
                                                   bool withhold, bool &dead)
{
    wait_stores();                 // this wave's coherent stores have completed
    __syncthreads();
    if (threadIdx.x == 0 && !withhold)
        __hip_atomic_store(flags + me, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!dead)
        wave_wait_flags(flags + lo, n, target, err, spin_limit, dead);
}

// Step barrier among the NUB workgroups of one (direction, batch block)
// group: each workgroup publishes "phase q done" in its own flag after its
// coherent stores have completed, then one wave polls the group's flags.
// No whole-cache writeback or invalidate is needed: every step writes a
// fresh plane of the H history that no cache has seen before.  A wait longer
// than spin_limit polls raises the error word and stops waiting.  `withhold`
// (test fault injection) skips the flag store.
__device__ __forceinline__ void group_barrier(uint32_t *flags, int nub, int me, uint32_t target,
                                              int32_t *err, uint32_t spin_limit, bool withhold,
                                              bool &dead)
{
    wait_stores();                 // this wave's coherent stores have completed
    __syncthreads();
    if (threadIdx.x == 0 && !withhold)
        __hip_atomic_store(flags + me, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < 64 && !dead) {
        uint32_t n = 0;
        for (;;) {
            bool ok = true;
            for (int i = threadIdx.x; i < nub; i += 64)
                ok = ok && __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target;
            if (__all(ok))
                break;
            __builtin_amdgcn_s_sleep(1);
            if (++n > spin_limit) {
                if (threadIdx.x == 0)
                    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                dead = true;
                break;
            }
        }
    }
    __syncthreads();
}

// The step product over one wave's k range, R in registers: acc[mt][nt] for
// the compile-time tile range [T0, T1), with A tiles prefetched PD k blocks
// ahead; `mid` runs right after the last A prefetch is issued (used to issue
// the loads the epilogue needs, after every load the product waits on).
template <int MT, int NT, int KBR, int T0, int T1, int PD, typename Mid>
__device__ __forceinline__ void product_res(f4 (&acc)[MT][NT], const float *asrc, int Hp,
                                            const f4 (&rr)[NT][KBR], Mid mid)
{
    // 16-k blocks; lane (r, q) supplies k = 16*kb + 4q + s of row r
    constexpr int D_ = PD < KBR ? PD : KBR;
    f4 ring[D_ + 1][MT];
#pragma unroll
    for (int p = 0; p < D_; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            ring[p][mt] = *(const f4 *)(asrc + (size_t)mt * 16 * Hp + p * 16);
    if constexpr (D_ >= KBR)
        mid();
#pragma unroll
    for (int kb = 0; kb < KBR; ++kb) {
        if (kb + D_ < KBR) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                ring[(kb + D_) % (D_ + 1)][mt] =
                    *(const f4 *)(asrc + (size_t)mt * 16 * Hp + (kb + D_) * 16);
            if (kb + D_ == KBR - 1)
                mid();
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int nt = T0; nt < T1; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        ring[kb % (D_ + 1)][mt][s], rr[nt][kb][s], acc[mt][nt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep the independent accumulators together
        }
    }
}

// The same with R streamed from memory every step (runtime KB).  Two
// register sets alternate: block kb + 1 is loaded while block kb is
// multiplied.  The loop body has no branch and no register copies, so the
// compiler's wait before a block's MFMAs covers that block's loads only (a
// copy of the prefetched block at the end of each iteration made it wait
// for the loads just issued, every block).
// f(std::integral_constant<int, M>) with M = min(max(n, 0), N): the number
// of row tiles, known at compile time, whose MFMAs a product issues.
template <int N, typename F>
__device__ __forceinline__ void with_row_tiles(int n, F f)
{
    if constexpr (N == 0) {
        f(std::integral_constant<int, 0>{});
    } else {
        if (n >= N)
            f(std::integral_constant<int, N>{});
        else
            with_row_tiles<N - 1>(n, f);
    }
}

// mt_act: row tiles that hold a row still active at this step (rows are held
// in order of decreasing length, so they form a prefix).  The whole k loop --
// A loads and MFMAs -- is specialised on that count (dispatched once per
// step, a uniform branch), so inactive tiles cost neither loads nor matrix
// cycles; their sums are never read.
template <int MT, int NT, int T0, int T1, typename Mid>
__device__ __forceinline__ void product_stream(f4 (&acc)[MT][NT], const float *asrc,
                                               const float *rfrag, int Hp, int KB, int mt_act,
                                               Mid mid)
{
    with_row_tiles<MT>(mt_act, [&](auto mta) {
        constexpr int MTA = decltype(mta)::value;
        f4 a0[MTA > 0 ? MTA : 1], b0[NT], a1[MTA > 0 ? MTA : 1], b1[NT];
        auto load = [&](auto &av, f4 (&bv)[NT], int kb) {
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt)
                av[mt] = *(const f4 *)(asrc + (size_t)mt * 16 * Hp + kb * 16);
#pragma unroll
            for (int nt = T0; nt < T1; ++nt)
                bv[nt] = *(const f4 *)(rfrag + (size_t)nt * 16 * Hp + kb * 16);
        };
        auto mma = [&](const auto &av, const f4 (&bv)[NT]) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int nt = T0; nt < T1; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MTA; ++mt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mt][s], bv[nt][s],
                                                                           acc[mt][nt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);   // keep the independent accumulators together
            }
        };
        if constexpr (MTA == 0) {
            mid();                                   // no active row: only the XW prefetch
        } else {
            // (per-tile pointers advanced once per two blocks; the blocks'
            // offsets from them are constants)
            const float *ap[MTA > 0 ? MTA : 1], *bp[NT];
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt)
                ap[mt] = asrc + (size_t)mt * 16 * Hp;
#pragma unroll
            for (int nt = T0; nt < T1; ++nt)
                bp[nt] = rfrag + (size_t)nt * 16 * Hp;
            auto load_at = [&](auto &av, f4 (&bv)[NT], int off) {
#pragma unroll
                for (int mt = 0; mt < MTA; ++mt)
                    av[mt] = *(const f4 *)(ap[mt] + off);
#pragma unroll
                for (int nt = T0; nt < T1; ++nt)
                    bv[nt] = *(const f4 *)(bp[nt] + off);
            };
            load_at(a0, b0, 0);
            int kb = 0;
            for (; kb + 2 < KB; kb += 2) {
                load_at(a1, b1, 16);
                mma(a0, b0);
                load_at(a0, b0, 32);
                mma(a1, b1);
#pragma unroll
                for (int mt = 0; mt < MTA; ++mt)
                    ap[mt] += 32;
#pragma unroll
                for (int nt = T0; nt < T1; ++nt)
                    bp[nt] += 32;
            }
            if (KB - kb == 2) {                      // two blocks left
                load(a1, b1, kb + 1);
                mid();
                mma(a0, b0);
                mma(a1, b1);
            } else {                                 // one block left
                mid();
                mma(a0, b0);
            }
        }
    });
}

// Gate arithmetic of one (row, unit) pair for the single-phase operators (RNN,
// GRU with linear_before_reset = 1, LSTM), in the written order.  xv[g] is the
// pair's XW value of gate g, rec(g) its recurrent product, cst(e) the pair's
// per-unit constants (e = g: Wb of gate g, 4 + g: Rb of gate g, 8, 9, 10: Pi,
// Po, Pf), hp the previous h and c the LSTM cell state (updated in place).
// Returns the new h.
template <typename F, typename Gf, typename Hf, typename Rec, typename Cst>
__device__ __forceinline__ float gates_one_phase(int op, const float *xv, Rec rec, Cst cst,
                                                 bool peep, bool clip_on, float clip,
                                                 bool input_forget, float hp, float &c, F f, Gf g,
                                                 Hf h)
{
    if (op == RNN_OP_RNN) {
        float pre = xv[0] + rec(0);
        pre = pre + cst(0);
        pre = pre + cst(4);
        pre = clip_pre(pre, clip_on, clip);
        return f(pre);
    }
    if (op == RNN_OP_GRU) {                                 // linear_before_reset = 1
        float pz = xv[0] + rec(0);
        float pr = xv[1] + rec(1);
        pz = pz + cst(0);
        pz = pz + cst(4);
        pr = pr + cst(1);
        pr = pr + cst(5);
        pz = clip_pre(pz, clip_on, clip);
        pr = clip_pre(pr, clip_on, clip);
        const float z = f(pz);
        const float r = f(pr);
        float rh = rec(2);
        rh = rh + cst(6);
        const float gated = r * rh;
        float ph = xv[2] + gated;
        ph = ph + cst(2);
        ph = clip_pre(ph, clip_on, clip);
        const float ht = g(ph);
        const float omz = 1.0f - z;
        const float a1 = omz * ht;
        const float a2 = z * hp;
        return a1 + a2;
    }
    // LSTM: i, o, f, c
    float pre[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float v = xv[k] + rec(k);
        v = v + cst(k);
        v = v + cst(4 + k);
        pre[k] = v;
    }
    const float cp = c;
    if (peep) {
        const float pi_ = cst(8) * cp;
        const float pf_ = cst(10) * cp;
        pre[0] = pre[0] + pi_;
        pre[2] = pre[2] + pf_;
    }
    const float ci = clip_pre(pre[0], clip_on, clip);
    const float cf = clip_pre(pre[2], clip_on, clip);
    const float cc = clip_pre(pre[3], clip_on, clip);
    const float ig = f(ci);
    const float fg = input_forget ? 1.0f - ig : f(cf);
    const float ct = g(cc);
    const float k1 = fg * cp;
    const float k2 = ig * ct;
    c = k1 + k2;
    float po = pre[1];
    if (peep) {
        const float pov = cst(9) * c;
        po = po + pov;
    }
    po = clip_pre(po, clip_on, clip);
    const float og = f(po);
    const float hc = h(c);
    return og * hc;
}

// GRU with linear_before_reset = 0, in the written order.  First phase: the
// update and reset gates from their XW values and recurrent products;
// returns z and stores r in *r.  Second phase: the candidate from its XW
// value and the product over r (.) H_prev, then the new h.
template <typename F>
__device__ __forceinline__ float gru0_gates(float xz, float xr, float rz, float rr, const float *cu,
                                            int U, int u, bool clip_on, float clip, F f, float *r)
{
    float pz = xz + rz;
    float pr = xr + rr;
    pz = pz + cu[u];
    pz = pz + cu[4 * U + u];
    pr = pr + cu[U + u];
    pr = pr + cu[5 * U + u];
    pz = clip_pre(pz, clip_on, clip);
    pr = clip_pre(pr, clip_on, clip);
    *r = f(pr);
    return f(pz);
}

template <typename Gf>
__device__ __forceinline__ float gru0_candidate(float xh, float rh, const float *cu, int U, int u,
                                                bool clip_on, float clip, float z, float hp, Gf g)
{
    float ph = xh + rh;
    ph = ph + cu[2 * U + u];
    ph = ph + cu[6 * U + u];
    ph = clip_pre(ph, clip_on, clip);
    const float ht = g(ph);
    const float omz = 1.0f - z;
    const float a1 = omz * ht;
    const float a2 = z * hp;
    return a1 + a2;
}

// LDS bytes of one workgroup: the waves' partial tiles (column-major, bt + 4
// rows per column), then the per-pair states (h, c, z) and the per-row
// lengths.
__host__ __device__ inline size_t rec_lds_bytes(int nw, int bt, int nt, int u)
{
    return ((size_t)nw * nt * 16 * (bt + 4) + 3 * (size_t)bt * u + 2 * bt + 11 * (size_t)u) * 4;
}

// Depth (in 16-k blocks) of the A-operand prefetch of the register-resident
// product; deeper rings measured no faster and cost registers.
constexpr int kPrefetch = 1;

template <int MT, int NT, int KBR, int P, int TA, int ACT, int NW>
__global__ void __launch_bounds__(64 * NW, 1) rec_kernel(RecArgs a)
{
    constexpr int kThreads = 64 * NW;            // NW waves split the k range
    constexpr int kWaves = NW;
    constexpr bool RES = KBR > 0;
    constexpr int BT = MT * 16;
    constexpr int NTC = NT * 16;
    constexpr int LDC = BT + 4;                  // column stride of the partial tiles (floats)
    constexpr int PH = TA > 0 ? 2 : 1;           // phases per step (2: GRU, linear_before_reset 0)
    extern __shared__ float smem[];
    // partial tiles [kWaves][NTC][LDC], column-major: a lane's four rows of a
    // column are contiguous (one 16-byte store per tile), and the gate
    // arithmetic's reads of 16 units x 4 rows fall in distinct banks
    float *red = smem;
    float *hst = red + kWaves * NTC * LDC;       // [BT * U] h of each (row, unit) pair
    float *cst = hst + BT * a.U;                 // [BT * U] LSTM cell state
    float *zst = cst + BT * a.U;                 // [BT * U] GRU update gate between phases
    int *lst = (int *)(zst + BT * a.U);          // [BT] sequence length of each row
    int *ost = lst + BT;                         // [BT] batch row held at each position
    float *cst_u = (float *)(ost + BT);          // [11][U] Wb, Rb per gate, then Pi, Po, Pf

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    // Workgroups of one XCD (blockIdx % 8) take consecutive logical ids, so a
    // (direction, batch block) group shares as few L2s as possible.
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const int lg = (nwg % 8 == 0) ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
    const int ub = lg % a.NUB;
    const int bb = (lg / a.NUB) % a.NBB;
    const int d = lg / (a.NUB * a.NBB);
    const int u0 = ub * a.U;
    const int uc = min(a.U, a.H - u0);
    const int row0 = bb * BT;
    const int rows = min(BT, a.Bt - row0);
    const int KB = RES ? KBR : a.KB;
    const int Hp = a.Hp;
    const bool rev = a.reverse_only || d == 1;
    // ACT fixes the operator too: 1 LSTM, 2 and 4 GRU, 3 RNN; 0 reads it at run time
    const int op = ACT == 1 ? (int)RNN_OP_LSTM
                 : (ACT == 2 || ACT == 4) ? (int)RNN_OP_GRU
                 : ACT == 3 ? (int)RNN_OP_RNN : a.op;
    const int G = ACT == 1 ? 4 : (ACT == 2 || ACT == 4) ? 3 : ACT == 3 ? 1 : a.G;   // gates
    const int GH = G * a.H;
    const size_t plane = (size_t)a.D * a.Btp * Hp;           // one plane of the H history
    const size_t drow = ((size_t)d * a.Btp + row0) * Hp;     // this group's rows
    const int grp = d * a.NBB + bb;
    const ActSpec fa = a.act[d][0], ga = a.act[d][1], ha = a.act[d][2];

    const float *Wb = a.B ? a.B + (size_t)d * 2 * GH : nullptr;
    const float *Rb = a.B ? Wb + GH : nullptr;
    const float *Pd = a.P ? a.P + (size_t)d * 3 * a.H : nullptr;
    const size_t xwd = (size_t)d * a.xw_steps * a.Bt * GH + (size_t)ub * G * a.U;
    const int npairs = rows * uc;

    // The unit blocks whose H columns this wave's k range reads (the columns
    // [H, Hp) are written by the last unit block), widened to whole 64-column
    // (256-byte) spans: a load brings in its whole cache line, and a line
    // that also holds columns of a unit block not yet waited for would stay
    // stale in this CU's and XCD's caches for the waves that read them next.
    const int wub_lo = min(kline_lo(w * KB * 16) / a.U, a.NUB - 1);
    const int wub_hi = min(a.NUB - 1, kline_hi((w + 1) * KB * 16, Hp) / a.U);

    // R fragments: lane (lr, lq) of wave w holds R[col nt*16 + lr][k] for
    // k = w*KB*16 + kb*16 + 4*lq + s, s = 0..3.
    const float *rfrag = a.Rp + ((size_t)(d * a.NUB + ub) * NTC + lr) * Hp + w * KB * 16 + 4 * lq;
    f4 rr[NT][RES ? KBR : 1];
    if constexpr (RES) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int kb = 0; kb < KBR; ++kb)
                rr[nt][kb] = *(const f4 *)(rfrag + (size_t)nt * 16 * Hp + kb * 16);
    }

    // states at the start of this launch
    {
        const int j0 = a.q_begin / PH;
        for (int pi = tid; pi < npairs; pi += kThreads) {
            const int rl = pi / uc, u = pi - rl * uc;
            const int s = row0 + rl;                      // position
            hst[pi] = a.hbuf[(size_t)(j0 % (a.xw_steps + 1)) * plane + drow + (size_t)rl * Hp + u0 + u];
            cst[pi] = op == RNN_OP_LSTM ? a.cbuf[((size_t)d * a.Bt + s) * a.H + u0 + u] : 0.0f;
            zst[pi] = (PH == 2 && (a.q_begin % 2) == 1)
                          ? a.zbuf[((size_t)d * a.Bt + s) * a.H + u0 + u]
                          : 0.0f;
        }
        for (int rl = tid; rl < rows; rl += kThreads) {
            lst[rl] = a.lens[row0 + rl];
            ost[rl] = a.order ? a.order[row0 + rl] : row0 + rl;
        }
        // Wb, Rb (zeros when B is absent: adding +0 to a pre-activation is the
        // identity here, since xw + rec is never -0 -- both sums start at +0),
        // then the peepholes Pi, Po, Pf
        for (int e = tid; e < 11 * uc; e += kThreads) {
            const int k = e / uc, u = e - k * uc;
            float v = 0.0f;
            if (k < 4 && k < G && Wb)
                v = Wb[k * a.H + u0 + u];
            else if (k >= 4 && k < 8 && k - 4 < G && Rb)
                v = Rb[(k - 4) * a.H + u0 + u];
            else if (k >= 8 && Pd)
                v = Pd[(k - 8) * a.H + u0 + u];
            cst_u[k * a.U + u] = v;
        }
        __syncthreads();
    }

    // XW of pair pi for phase qq (zeros for an absent pair or a row no longer
    // active).  XW is stored by step: row (jj - j_base, position) already
    // holds the projection of the time index this step reads (reverse
    // included).
    auto fetch_xw_q = [&](int qq, int pi, float *xv) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
            xv[g] = 0.0f;
        const int jj = qq / PH, pp = qq - jj * PH;
        const int rl = pi / uc, u = pi - rl * uc;
        if (pi >= npairs || jj >= lst[rl])
            return;
        const float *src = a.XW + xwd + ((size_t)(jj - a.j_base) * a.Bt + row0 + rl) * GH + u;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            if (g < G && (PH == 1 || (pp == 1) == (g == 2)))
                xv[g] = src[g * uc];
    };
    // Each phase's XW values are loaded during the previous phase's product
    // (issued after its last H load, so that no product wait is held up by
    // them), the first phase's before the loop.
    float xw_next[P][4];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (a.q_begin < a.q_end)
            fetch_xw_q(a.q_begin, tid + kThreads * i, xw_next[i]);
        else
            for (int g = 0; g < 4; ++g)
                xw_next[i][g] = 0.0f;
    }
    bool dead = false;
    for (int q = a.q_begin; q < a.q_end; ++q) {
        RNN_STAMP(q - a.q_begin, 0);
        const int j = q / PH;
        const int ph = q - j * PH;
        const int t0 = ph == 0 ? 0 : a.NTA;              // this phase's column tiles
        const int t1 = ph == 0 ? a.NTA : a.NTA + a.NTB;
        const bool last_phase = ph == PH - 1;

        float xw[P][4];
#pragma unroll
        for (int i = 0; i < P; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                xw[i][g] = xw_next[i][g];
        auto prefetch_xw = [&]() {
            if (q + 1 < a.q_end) {
#pragma unroll
                for (int i = 0; i < P; ++i)
                    fetch_xw_q(q + 1, tid + kThreads * i, xw_next[i]);
            }
        };

        // ---- the product over this wave's k range --------------------------
        const float *asrc = (ph == 0 ? a.hbuf + (size_t)(j % (a.xw_steps + 1)) * plane
                                     : a.sbuf + (size_t)(j % a.xw_steps) * plane) + drow +
                            (size_t)lr * Hp + w * KB * 16 + 4 * lq;
        // row tiles that hold a row still active at step j (the rows are held
        // in order of decreasing length); the streamed product skips the
        // MFMAs of the rest, whose sums are never read.  (The register-
        // resident products issue every tile: their copies per tile count
        // measured slower where all rows are active.)
        int mt_act = MT;
        if constexpr (!RES) {
            int na = 0;                          // active rows: a prefix of the block
#pragma unroll
            for (int r0 = 0; r0 < BT; r0 += 64)
                na += __popcll(__ballot(r0 + lane < rows && lst[r0 + lane] > j));
            mt_act = (na + 15) / 16;
        }
        f4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
        // phase tiles: [0, NT) for one phase, [0, TA) then [TA, NT) for two
        constexpr int TA0 = TA > 0 ? TA : NT;
        if constexpr (RES) {
            if (ph == 0)
                product_res<MT, NT, KBR, 0, TA0, kPrefetch>(acc, asrc, Hp, rr, prefetch_xw);
            else if constexpr (TA > 0)
                product_res<MT, NT, KBR, TA, NT, kPrefetch>(acc, asrc, Hp, rr, prefetch_xw);
        } else {
            if (ph == 0)
                product_stream<MT, NT, 0, TA0>(acc, asrc, rfrag, Hp, KB, mt_act, prefetch_xw);
            else if constexpr (TA > 0)
                product_stream<MT, NT, TA, NT>(acc, asrc, rfrag, Hp, KB, mt_act, prefetch_xw);
        }
        RNN_STAMP(q - a.q_begin, 1);
        // ---- partial tiles -> LDS, summed in wave order ----------------------
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (nt < t0 || nt >= t1)
                    continue;          // (uniform: the other phase's tiles)
                *(f4 *)(red + (w * NTC + nt * 16 + lr) * LDC + mt * 16 + 4 * lq) = acc[mt][nt];
            }
        __syncthreads();
        RNN_STAMP(q - a.q_begin, 2);
        auto rec_at = [&](int rl, int col) {
            const float *p = red + col * LDC + rl;
            float v = p[0];
#pragma unroll
            for (int w2 = 1; w2 < NW; ++w2)
                v = v + p[w2 * NTC * LDC];            // fixed wave order
            return v;
        };

        // ---- gate arithmetic of one (row, unit) pair, in the written order --
        float *hnext = a.hbuf + (size_t)((j + 1) % (a.xw_steps + 1)) * plane + drow;
        float *snext = a.sbuf ? a.sbuf + (size_t)(j % a.xw_steps) * plane + drow : nullptr;
        auto do_pair = [&](int pi, const float *xv, auto F, auto Gf, auto Hf) {
            const int rl = pi / uc, u = pi - rl * uc;
            const int b = ost[rl];                         // batch row (outputs)
            const int gu = u0 + u;                         // hidden unit
            const int len = lst[rl];
            const bool active = j < len;
            const float hp = hst[pi];
            float hn = hp, cn = cst[pi];
            if (active) {
                if (op != RNN_OP_GRU || PH == 1) {    // (compile-time for LSTM, RNN)
                    hn = gates_one_phase(
                        op, xv, [&](int g) { return rec_at(rl, g * uc + u); },
                        [&](int e) { return cst_u[e * a.U + u]; }, Pd != nullptr, a.clip_on, a.clip, a.input_forget != 0, hp, cn, F, Gf, Hf);
                } else if (ph == 0) {                       // GRU lbr = 0: z and r
                    float r;
                    zst[pi] = gru0_gates(xv[0], xv[1], rec_at(rl, u), rec_at(rl, uc + u), cst_u,
                                         a.U, u, a.clip_on, a.clip, F, &r);
                    store_coherent(snext + (size_t)rl * Hp + gu, r * hp);   // r (.) H_prev
                } else {                                    // GRU lbr = 0: candidate
                    hn = gru0_candidate(xv[2], rec_at(rl, a.NTA * 16 + u), cst_u, a.U, u,
                                        a.clip_on, a.clip, zst[pi], hp, Gf);
                }
            } else if (PH == 2 && ph == 0) {
                store_coherent(snext + (size_t)rl * Hp + gu, 0.0f);
            }
            if (last_phase) {
                store_coherent(hnext + (size_t)rl * Hp + gu, hn);   // carried when inactive
                hst[pi] = hn;
                cst[pi] = cn;
                if (a.Y) {
                    const int t = active ? (rev ? len - 1 - j : j) : j;
                    const size_t yo = a.layout == 0
                                          ? (((size_t)t * a.D + d) * a.Bt + b) * a.H + gu
                                          : (((size_t)b * a.S + t) * a.D + d) * a.H + gu;
                    a.Y[yo] = active ? canon_nan(hn) : 0.0f;
                }
            }
        };

        // One-phase gates of N pairs (N = 1 or 2) of this thread: every LDS
        // value they read (the waves' partial sums of their gate columns, the
        // constants of their units, their states and rows) is loaded first,
        // the gates are computed for every pair and kept only while its row is
        // active, and the stores come last -- no branch separates the loads
        // from their use, and the pairs' chains interleave.
        auto gates_n = [&](auto NC, const int *pis, const float (*xv)[4], auto F, auto Gf,
                           auto Hf) {
            constexpr int N = decltype(NC)::value;
            int rl[N], u[N], len[N];
            float hp[N], cp[N], part[N][4][kWaves], cv[N][11];
#pragma unroll
            for (int n = 0; n < N; ++n) {
                rl[n] = pis[n] / uc;
                u[n] = pis[n] - rl[n] * uc;
                len[n] = lst[rl[n]];
                hp[n] = hst[pis[n]];
                cp[n] = cst[pis[n]];
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int w2 = 0; w2 < kWaves; ++w2)
                        part[n][g][w2] = g < G ? red[(w2 * NTC + g * uc + u[n]) * LDC + rl[n]] : 0.0f;
#pragma unroll
                for (int e = 0; e < 11; ++e) {
                    const bool need = op == RNN_OP_RNN   ? (e == 0 || e == 4)
                                      : op == RNN_OP_GRU ? (e < 8 && e % 4 < 3)
                                                         : (e < 8 || Pd != nullptr);
                    cv[n][e] = need ? cst_u[e * a.U + u[n]] : 0.0f;
                }
            }
            float hn[N], cn[N];
#pragma unroll
            for (int n = 0; n < N; ++n) {
                float cx = cp[n];
                const float hx = gates_one_phase(
                    op, xv[n],
                    [&](int g) {
                        float v = part[n][g][0];
#pragma unroll
                        for (int w2 = 1; w2 < kWaves; ++w2)
                            v = v + part[n][g][w2];               // fixed wave order
                        return v;
                    },
                    [&](int e) { return cv[n][e]; }, Pd != nullptr, a.clip_on, a.clip,
                    a.input_forget != 0, hp[n], cx, F, Gf, Hf);
                const bool active = j < len[n];
                hn[n] = active ? hx : hp[n];                      // carried when inactive
                cn[n] = active ? cx : cp[n];
            }
#pragma unroll
            for (int n = 0; n < N; ++n) {
                store_coherent(hnext + (size_t)rl[n] * Hp + u0 + u[n], hn[n]);
                hst[pis[n]] = hn[n];
                cst[pis[n]] = cn[n];
            }
            if (a.Y) {
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const bool active = j < len[n];
                    const int b = ost[rl[n]];                     // batch row (outputs)
                    const int t = active ? (rev ? len[n] - 1 - j : j) : j;
                    const size_t yo = a.layout == 0
                                          ? (((size_t)t * a.D + d) * a.Bt + b) * a.H + u0 + u[n]
                                          : (((size_t)b * a.S + t) * a.D + d) * a.H + u0 + u[n];
                    a.Y[yo] = active ? canon_nan(hn[n]) : 0.0f;
                }
            }
        };

        // Pairs tid + kThreads i.  Up to 2 pairs: one at a time, unrolled.  Up
        // to 8 pairs, one phase: four at a time (two when the count is not a
        // multiple of four) where every thread has all of them (a uniform
        // test; four measured 1% faster than two at 8 pairs per thread), in a
        // loop that is not unrolled -- unrolled, the LDS
        // addresses of every pair are hoisted out of the step loop and spill
        // -- with the pairs' XW values moved down the array instead of
        // indexed at run time.  Up to 8 pairs, two phases (GRU,
        // linear_before_reset 0): one at a time, likewise.
        auto run_pairs = [&](auto F, auto Gf, auto Hf) {
            if constexpr (P <= 2) {
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const int pi = tid + kThreads * i;
                    if (pi < npairs)
                        do_pair(pi, xw[i], F, Gf, Hf);
                }
            } else if constexpr (PH == 1) {
                static_assert(P % 2 == 0, "pairs are taken two at a time");
                constexpr int NB = P % 4 == 0 ? 4 : 2;
#pragma unroll 1
                for (int i = 0; i < P; i += NB) {
                    const int pi0 = tid + kThreads * i;
                    if (npairs >= kThreads * (i + NB)) {
                        int pis[NB];
#pragma unroll
                        for (int n = 0; n < NB; ++n)
                            pis[n] = pi0 + kThreads * n;
                        gates_n(std::integral_constant<int, NB>{}, pis, xw, F, Gf, Hf);
                    } else {
#pragma unroll
                        for (int n = 0; n < NB; ++n) {
                            const int pin = pi0 + kThreads * n;
                            if (pin < npairs)
                                gates_n(std::integral_constant<int, 1>{}, &pin, xw + n, F, Gf, Hf);
                        }
                    }
                    if (npairs <= kThreads * (i + NB))
                        break;
#pragma unroll
                    for (int k = 0; k + NB < P; ++k)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            xw[k][g] = xw[k + NB][g];
                }
            } else {
#pragma unroll 1
                for (int i = 0; i < P; ++i) {
                    const int pi = tid + kThreads * i;
                    if (pi >= npairs)
                        break;
                    do_pair(pi, xw[0], F, Gf, Hf);
#pragma unroll
                    for (int k = 0; k + 1 < P; ++k)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            xw[k][g] = xw[k + 1][g];
                }
            }
        };
        // ACT (compile time): 1 LSTM Sigmoid/Tanh/Tanh, 2 GRU HardSigmoid/Tanh,
        // 3 RNN Tanh, 4 GRU Sigmoid/Tanh, 0 any set through the run-time switch
        if constexpr (ACT == 1 || ACT == 4)
            run_pairs(ActSigmoid{}, ActTanh{}, ActTanh{});
        else if constexpr (ACT == 2)
            run_pairs(ActHardSigmoid{fa.alpha, fa.beta}, ActTanh{}, ActTanh{});
        else if constexpr (ACT == 3)
            run_pairs(ActTanh{}, ActTanh{}, ActTanh{});
        else
            run_pairs(ActAny{fa}, ActAny{ga}, ActAny{ha});
        // The last unit block also writes the padding columns [H, Hp) of the
        // plane it published, as zeros (they meet zero rows of R).
        if (u0 + uc == a.H && Hp > a.H && (last_phase || PH == 2)) {
            float *pl = last_phase ? hnext : snext;
            const int padw = Hp - a.H;
            for (int e = tid; e < rows * padw; e += kThreads)
                store_coherent(pl + (size_t)(e / padw) * Hp + a.H + e % padw, 0.0f);
        }
        RNN_STAMP(q - a.q_begin, 3);
        if (q + 1 < a.q_end)
            group_publish_wait(a.bar + (size_t)grp * 2 * a.NUB, ub, (uint32_t)(q + 1), wub_lo,
                               wub_hi - wub_lo + 1, a.err, a.spin_limit, a.withhold_flags != 0,
                               dead);
        else
            __syncthreads();
        RNN_STAMP(q - a.q_begin, 4);
    }

    // ---- end of this launch: keep or publish the states ---------------------
    const bool done = a.q_end == a.S * PH;
    for (int pi = tid; pi < npairs; pi += kThreads) {
        const int rl = pi / uc, u = pi - rl * uc;
        const int s = row0 + rl;
        const int b = ost[rl];                            // batch row (outputs)
        const size_t so = ((size_t)d * a.Bt + s) * a.H + u0 + u;
        if (op == RNN_OP_LSTM)
            a.cbuf[so] = cst[pi];
        if (PH == 2)
            a.zbuf[so] = zst[pi];
        if (done) {
            const size_t yo = a.layout == 0 ? ((size_t)d * a.Bt + b) * a.H + u0 + u
                                            : ((size_t)b * a.D + d) * a.H + u0 + u;
            const bool none = lst[rl] == 0;
            if (a.Yh)
                a.Yh[yo] = none ? 0.0f : canon_nan(hst[pi]);
            if (a.Yc)
                a.Yc[yo] = none ? 0.0f : canon_nan(cst[pi]);
        }
    }
}

typedef void (*rec_fn)(RecArgs);

}  // namespace rnnamd
