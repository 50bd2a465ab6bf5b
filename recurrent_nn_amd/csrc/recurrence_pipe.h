// recurrence_pipe.h -- the step loop (same operator semantics as
// recurrence_kernel.h: onemodel "Recurrent operators", section "Computation",
// the pre-activation / LSTM / GRU / RNN paragraphs, "Choices the
// specification leaves open" for masking and reverse traversal, "Exact mode"
// for NaN canonicalisation) software-pipelined over two half-batch sub-steps.
//
// The workgroup's BT rows are processed as two halves of BT/2 rows, one after
// the other, every step: product, reduction and gate arithmetic of half 0,
// then of half 1.  Each half has flags of its own, so the exchange of one
// half's new H (store completion, flag store, the other workgroups' polls)
// proceeds while the workgroup computes the other half's product, instead of
// stalling every wave between steps:
//   - a half's flag is published from inside the NEXT product (the other
//     half's), at an early fixed k block: each wave waits there for its own H
//     stores to complete and the last wave of the four to arrive stores the
//     flag;
//   - before a half's product, each wave waits only for the flags of the
//     workgroups that produce its own k range of H.
// The waves split k and sum their partial tiles exactly as the four-wave
// kernel does (same fragments, same MFMA order per output, same wave order),
// so the results are bit-identical to it.  Single-phase operators (RNN, LSTM,
// GRU with linear_before_reset = 1) with R resident in registers.
#pragma once

#include "recurrence_kernel.h"

namespace rnnamd {

// The register-resident product (as product_res) with A tiles prefetched PD
// k blocks ahead.  The first PD blocks are loaded by prime_ring beforehand
// (so that their latency overlaps other work); `mid` runs right after the
// last A prefetch, `hook` at the top of k block KH, before that block's
// prefetch is issued, `late` at the top of k block KP (after every A
// prefetch when KP >= KBR - PD) and `check` at the top of k block KC (none
// for KC < 0).
template <int MT, int KBR, int PD>
__device__ __forceinline__ void prime_ring(f4 (&ring)[(PD < KBR ? PD : KBR) + 1][MT],
                                           const float *asrc, int Hp)
{
    constexpr int D_ = PD < KBR ? PD : KBR;
#pragma unroll
    for (int p = 0; p < D_; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            ring[p][mt] = *(const f4 *)(asrc + (size_t)mt * 16 * Hp + p * 16);
}

template <int MT, int NT, int KBR, int PD, int KH, int KP, int KC, typename Mid, typename Hook,
          typename Late, typename Check>
__device__ __forceinline__ void product_res_hooked(f4 (&acc)[MT][NT],
                                                   f4 (&ring)[(PD < KBR ? PD : KBR) + 1][MT],
                                                   const float *asrc, int Hp,
                                                   const f4 (&rr)[NT][KBR], Mid mid, Hook hook,
                                                   Late late, Check check)
{
    constexpr int D_ = PD < KBR ? PD : KBR;
    if constexpr (D_ >= KBR)
        mid();
#pragma unroll
    for (int kb = 0; kb < KBR; ++kb) {
        if (kb == KH)
            hook();
        if (kb == KP)
            late();
        if (kb == KC)
            check();
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
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        ring[kb % (D_ + 1)][mt][s], rr[nt][kb][s], acc[mt][nt], 0, 0, 0);
            // keep the MT x NT independent accumulators of one k sub-block
            // together: left alone, the scheduler groups them by row tile,
            // leaving two dependent chains that stall the matrix pipe
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// LDS bytes: partial tiles of both halves (column-major, BT/2 + 4 rows per
// column), h and c per pair, lengths, the per-unit constants, two publish
// counters.
__host__ __device__ inline size_t rec_pipe_lds_bytes(int bt, int nt, int u)
{
    return ((size_t)8 * nt * 16 * (bt / 2 + 4) + 2 * (size_t)bt * u + bt + 11 * (size_t)u + 2) * 4;
}

// Depth of the A prefetch for the half-height products (fewer MFMAs per k
// block than the full tile, so more blocks in flight; 3 measured best).
constexpr int kPipePrefetch = 3;

template <int MTH, int NT, int KBR, int ACT, int P>
__global__ void __launch_bounds__(256, 1) rec_pipe_kernel(RecArgs a)
{
    constexpr int BTH = MTH * 16;                // rows per half
    constexpr int BT = 2 * BTH;
    constexpr int NTC = NT * 16;
    constexpr int LDC = BTH + 4;                 // partial tiles: column stride (floats)
    // gates per pair (compile-time unless the activation set is generic)
    constexpr int GC = ACT == 1 ? 4 : (ACT == 2 || ACT == 4) ? 3 : ACT == 3 ? 1 : 4;
    // P: pairs per thread and half, at most (1 or 2)
    // k block where the other half is published: early (its H stores, issued
    // just before this product, have had two blocks to complete), so that the
    // flag is out well before the other workgroups poll for it (publishing
    // at block 2 of 16 measured 2% faster than at block 8, at 0 slower)
    constexpr int KH = KBR >= 4 ? 2 : KBR / 2;
    // k block where the next product's flags are polled: after the publish,
    // and one block after the last A prefetch is issued (the later it goes,
    // the more flags are already set: with the value compared right after
    // the load, at block 14 of 16 the step loop of a bidirectional LSTM of
    // hidden size 1024, batch 64, took 9.76 us per step against 10.05 at
    // block 13, and a hidden-1024 GRU 8.96 against 9.17; block 15 was the
    // same as 14)
    constexpr int KPF = KBR - (kPipePrefetch < KBR ? kPipePrefetch : KBR);
    constexpr int KP0 = KPF + 1 > KH + 1 ? KPF + 1 : KH + 1;
    constexpr int KP = KP0 < KBR ? KP0 : KBR - 1;
    static_assert(KP > KH && KP < KBR, "the poll falls inside the product, after the publish");
    // Poll the next product's flags inside this product and load its first k
    // blocks before this half's gate arithmetic only when the product is long
    // enough (>= 128 MFMAs per wave) to hide the poll's memory round trip;
    // short products wait for their flags right before they start.
    constexpr bool EARLY = 4 * MTH * NT * KBR >= 128;
    extern __shared__ float smem[];
    float *red = smem;                           // [2 halves][4 waves][NTC][LDC] partial tiles
    float *hst = red + 8 * NTC * LDC;            // [BT * U] h of each (row, unit) pair
    float *cst = hst + BT * a.U;                 // [BT * U] LSTM cell state
    int *lst = (int *)(cst + BT * a.U);          // [BT] sequence length of each row
    float *cst_u = (float *)(lst + BT);          // [11][U] Wb, Rb per gate, then Pi, Po, Pf
    uint32_t *ctr = (uint32_t *)(cst_u + 11 * a.U);   // [2] arrivals at each half's publish

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    // same workgroup -> (d, batch block, unit block) map as the four-wave kernel
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
    const int Hp = a.Hp;
    const bool rev = a.reverse_only || d == 1;
    const int GH = a.G * a.H;
    const int op = ACT == 1 ? (int)RNN_OP_LSTM
                 : (ACT == 2 || ACT == 4) ? (int)RNN_OP_GRU
                 : ACT == 3 ? (int)RNN_OP_RNN : a.op;
    const size_t plane = (size_t)a.D * a.Btp * Hp;
    const size_t drow = ((size_t)d * a.Btp + row0) * Hp;
    const int grp = d * a.NBB + bb;
    uint32_t *flags0 = a.bar + (size_t)grp * 2 * a.NUB;     // [2 halves][NUB]
    const ActSpec fa = a.act[d][0], ga = a.act[d][1], ha = a.act[d][2];

    const float *Wb = a.B ? a.B + (size_t)d * 2 * GH : nullptr;
    const float *Rb = a.B ? Wb + GH : nullptr;
    const float *Pd = a.P ? a.P + (size_t)d * 3 * a.H : nullptr;
    const size_t xwd = (size_t)d * a.xw_steps * a.Bt * GH + (size_t)ub * a.G * a.U;
    const int npairs = rows * uc;

    // The unit blocks whose H columns this wave's k range reads (the columns
    // [H, Hp) are written by the last unit block), widened to whole cache
    // lines as in the four-wave kernel (a no-op here: KBR * 16 >= 128).
    const int k0 = w * KBR * 16;
    const int wub_lo = min(kline_lo(k0) / a.U, a.NUB - 1);
    const int wub_hi = min(a.NUB - 1, kline_hi(k0 + KBR * 16, Hp) / a.U);

    // R fragments, as in the four-wave kernel
    const float *rfrag = a.Rp + ((size_t)(d * a.NUB + ub) * NTC + lr) * Hp + k0 + 4 * lq;
    f4 rr[NT][KBR];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int kb = 0; kb < KBR; ++kb)
            rr[nt][kb] = *(const f4 *)(rfrag + (size_t)nt * 16 * Hp + kb * 16);

    // states at the start of this launch, constants, counters
    {
        const int j0 = a.q_begin;
        for (int pi = tid; pi < npairs; pi += 256) {
            const int rl = pi / uc, u = pi - rl * uc;
            hst[pi] = a.hbuf[(size_t)(j0 % (a.xw_steps + 1)) * plane + drow + (size_t)rl * Hp + u0 + u];
            cst[pi] = op == RNN_OP_LSTM ? a.cbuf[((size_t)d * a.Bt + row0 + rl) * a.H + u0 + u] : 0.0f;
        }
        for (int rl = tid; rl < rows; rl += 256)
            lst[rl] = a.lens[row0 + rl];
        // zeros when B is absent (adding +0 is the identity here: xw + rec is
        // never -0, both sums starting at +0)
        for (int e = tid; e < 11 * uc; e += 256) {
            const int k = e / uc, u = e - k * uc;
            float v = 0.0f;
            if (k < 4 && k < a.G && Wb)
                v = Wb[k * a.H + u0 + u];
            else if (k >= 4 && k < 8 && k - 4 < a.G && Rb)
                v = Rb[(k - 4) * a.H + u0 + u];
            else if (k >= 8 && Pd)
                v = Pd[(k - 8) * a.H + u0 + u];
            cst_u[k * a.U + u] = v;
        }
        if (tid < 2)
            ctr[tid] = 0u;
        __syncthreads();
    }

    // this thread's pairs of half h: (local row, unit) = (h * BTH + i / uc,
    // i % uc) for i = tid + 256 * k, decoded once as (row << 16) | unit, or
    // -1 where the half has fewer pairs
    auto hpairs_of = [&](int h) { return max(0, min(BTH, rows - h * BTH)) * uc; };
    int pk[2][P];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int i = tid + 256 * k;
            pk[h][k] = i < hpairs_of(h) ? ((h * BTH + i / uc) << 16) | (i % uc) : -1;
        }
    // A thread keeps its pairs for the whole launch: their h, c, length,
    // per-unit constants and output offsets live in registers.
    const int G = ACT == 0 ? a.G : GC;
    const size_t xstep = (size_t)a.Bt * GH;      // XW: one step
    const size_t ystep = a.layout == 0 ? (size_t)a.D * a.Bt * a.H : (size_t)a.D * a.H;
    float hreg[2][P], creg[2][P], kc[2][P][11];
    int lreg[2][P];
    uint32_t hoff[2][P];                         // offset of the pair in an H plane (from drow)
    // XW element offsets fit 32 bits: the scratch limit keeps each
    // direction's projections under 2^30 floats
    // (xbo: byte offset inside one step's rows of this direction, under 2^32)
    uint32_t xoff[2][P], xbo[2][P];
    const float *XWd = a.XW + (size_t)d * a.xw_steps * a.Bt * GH;
    size_t yoff[2][P];                           // offset of the pair's Y at step 0
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int rl = pk[h][k] < 0 ? 0 : pk[h][k] >> 16, u = pk[h][k] < 0 ? 0 : pk[h][k] & 0xffff;
            const int pi = rl * uc + u;
            const int s = row0 + rl, gu = u0 + u;
            const int b = a.order ? a.order[s] : s;       // batch row (outputs)
            hreg[h][k] = hst[pi];
            creg[h][k] = cst[pi];
            lreg[h][k] = pk[h][k] < 0 ? 0 : lst[rl];
#pragma unroll
            for (int e = 0; e < 11; ++e)
                kc[h][k][e] = cst_u[e * a.U + u];
            hoff[h][k] = (uint32_t)(rl * Hp + gu);
            xoff[h][k] = (uint32_t)(xwd + (size_t)(row0 + rl) * GH + u);
            xbo[h][k] = 4u * (uint32_t)((size_t)ub * a.G * a.U + (size_t)(row0 + rl) * GH + u);
            yoff[h][k] = a.layout == 0 ? ((size_t)d * a.Bt + b) * a.H + gu
                                       : ((size_t)b * a.S * a.D + d) * a.H + gu;
        }
    auto fetch_xw_q = [&](int qq, int h, int k, float *xv) {
        xv[0] = xv[1] = xv[2] = xv[3] = 0.0f;
        if (qq >= lreg[h][k])
            return;
        // XW is stored by step (reverse included)
        const float *src = a.XW + xoff[h][k] + (size_t)(qq - a.j_base) * xstep;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            if (g < G)
                xv[g] = src[g * uc];
    };
    float xw_next[2][P][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < P; ++k) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                xw_next[h][k][g] = 0.0f;
            if (pk[h][k] >= 0 && a.q_begin < a.q_end)
                fetch_xw_q(a.q_begin, h, k, xw_next[h][k]);
        }

    bool dead = false;
    // a publish left for the next product: half, flag value, generation
    int pend_h = -1;
    uint32_t pend_v = 0, pend_gen = 0;
    uint32_t gens[2] = {0u, 0u};
    auto publish = [&]() {
        if (pend_h >= 0) {
            wait_stores();                       // this wave's H stores have completed
            if (lane == 0) {
                const uint32_t old = __hip_atomic_fetch_add(ctr + pend_h, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_WORKGROUP);
                if (old == 4u * pend_gen + 3u && !a.withhold_flags)   // the last of the four waves
                    __hip_atomic_store(flags0 + (size_t)pend_h * a.NUB + ub, pend_v,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            pend_h = -1;
        }
    };

    // A operand of half h from H history plane `pl`: this wave's k range of
    // its rows.  Planes form a ring of xw_steps + 1: step j reads plane
    // j mod ring and writes the next one.
    const int ring_n = a.xw_steps + 1;
    auto a_src = [&](int pl, int h) {
        return a.hbuf + (size_t)pl * plane + drow + (size_t)(h * BTH + lr) * Hp + k0 + 4 * lq;
    };
    int pj = a.q_begin % ring_n;                 // plane of step q
    auto next_plane = [&](int pl) { return pl + 1 == ring_n ? 0 : pl + 1; };
    constexpr int RING = (kPipePrefetch < KBR ? kPipePrefetch : KBR) + 1;
    f4 ring[RING][MTH];
    if (a.q_begin < a.q_end)
        prime_ring<MTH, KBR, kPipePrefetch>(ring, a_src(pj, 0), Hp);
    bool primed = true;                          // the next product's first blocks are loaded

    for (int q = a.q_begin; q < a.q_end; ++q) {
        const int j = q;                         // one phase per step
        const int pj1 = next_plane(pj);
        float *hnext = a.hbuf + (size_t)pj1 * plane + drow;   // (+ hoff: the pair)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int slot = 2 * (q - a.q_begin) + h;    // (instrumented build)
            (void)slot;
            RNN_STAMP(slot, 0);
            const int hrow0 = h * BTH;
            const int hpairs = hpairs_of(h);
            // the next product: half 1 of this step, or half 0 of the next
            const int nq = h == 0 ? q : q + 1, nh = 1 - h;
            const bool has_next = nq < a.q_end;
            if (!primed) {                       // its flags were not all set earlier
                if (!dead)
                    wave_wait_flags(flags0 + (size_t)h * a.NUB + wub_lo, wub_hi - wub_lo + 1,
                                    (uint32_t)q, a.err, a.spin_limit, dead);
                prime_ring<MTH, KBR, kPipePrefetch>(ring, a_src(pj, h), Hp);
            }
            RNN_STAMP(slot, 1);
            float xw[P][4];
#pragma unroll
            for (int k = 0; k < P; ++k)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    xw[k][g] = xw_next[h][k][g];
            // The next step's XW row of each pair, issued inside the product
            // right after the publish, so that neither the publish's wait for
            // the H stores nor the flag poll's wait near the end of the
            // product holds these memory reads (memory operations retire in
            // issue order).  Issued at the last A prefetch instead, the poll's
            // wait covered their latency: 10.2 against 10.05 us per step for
            // the bidirectional LSTM of hidden size 1024, batch 64.  The row
            // is loaded whether or not the pair is still active there (an
            // inactive pair's gate results are discarded), by every lane (a
            // lane without a pair reads the rows' first element) and at every
            // step (the last one reloads its own row), with the gate's uniform
            // base plus the pair's 32-bit byte offset as the address: no
            // branch and little vector arithmetic inside the product.
            auto prefetch_xw = [&]() {
                const int qn = q + 1 < a.q_end ? q + 1 : q;
                const char *base = (const char *)(XWd + (size_t)(qn - a.j_base) * xstep);
#pragma unroll
                for (int k = 0; k < P; ++k)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        if (g < G)
                            xw_next[h][k][g] =
                                *(const float *)(base + (size_t)g * uc * 4 + xbo[h][k]);
            };

            // ---- product over this wave's k range, this half's rows ---------
            // (its first k blocks were loaded by prime_ring)
            f4 acc[MTH][NT];
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
            // The next product's flags (a step after the launch's first) are
            // read once near the end of this product, after its last A
            // prefetch, so that the loads return during its last MFMAs (one
            // flag per lane; more than 64 flags: always wait later).
            const uint32_t *nflags = flags0 + (size_t)nh * a.NUB + wub_lo;
            const int nfl = wub_hi - wub_lo + 1;
            const bool need_wait = has_next && nq > a.q_begin && !dead;
            // The load is issued by every lane (lanes past the last flag
            // read the first one again) and its value compared one k block
            // later, so that a block of MFMAs runs under its round trip
            // (9.79 -> 9.53 us per step for the bidirectional LSTM of hidden
            // size 1024; compared right after the load, or only after the
            // product's partial-tile barrier, it was slower).
            uint32_t fv = 0u;
            bool fset = false;
            auto poll_next = [&]() {
                if (EARLY)
                    fv = __hip_atomic_load(nflags + (lane < nfl ? lane : 0), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            };
            auto check_next = [&]() {
                if (EARLY)
                    fset = __all(lane >= nfl || fv >= (uint32_t)nq);
            };
            constexpr int KC = KP + 1 < KBR ? KP + 1 : -1;
            product_res_hooked<MTH, NT, KBR, kPipePrefetch, KH, KP, KC>(
                acc, ring, a_src(pj, h), Hp, rr, []() {},
                [&]() {
                    const bool had = pend_h >= 0;
                    publish();
                    prefetch_xw();
                    if (had)
                        RNN_STAMP(slot - 1, 5);   // the previous half's flag is out
                },
                poll_next, check_next);
            if constexpr (KC < 0)
                check_next();
            RNN_STAMP(slot, 2);
            // partial tiles, column-major: a lane's four rows of a column are
            // contiguous (one 16-byte store per tile)
            float *redh = red + h * 4 * NTC * LDC;
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    *(f4 *)(redh + (w * NTC + nt * 16 + lr) * LDC + mt * 16 + 4 * lq) = acc[mt][nt];
            __syncthreads();
            RNN_STAMP(slot, 3);
            // if they were all set, load the next product's first k blocks now,
            // so that their latency overlaps this half's gate arithmetic;
            // otherwise wait for them only before that product
            primed = !need_wait || (EARLY && nfl <= 64 && fset);
            asm volatile("" ::: "memory");
            if (has_next && primed)
                prime_ring<MTH, KBR, kPipePrefetch>(ring, a_src(h == 0 ? pj : pj1, nh), Hp);

            // ---- gate arithmetic of this thread's pairs of half h -------------
            // (computed for every pair and kept only while the row is active,
            // so that no branch separates the loads from their use)
            auto run_pairs = [&](auto F, auto Gf, auto Hf) {
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    if (pk[h][k] < 0)
                        continue;
                    const int rl = pk[h][k] >> 16, u = pk[h][k] & 0xffff;
                    const int rh = rl - hrow0;
                    // the four waves' partial sums of each gate column, all
                    // loaded before the first is used
                    float part[4][4];
                    const float *rp = redh + u * LDC + rh;
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int w2 = 0; w2 < 4; ++w2)
                            part[g][w2] = g < G ? rp[(w2 * NTC + g * uc) * LDC] : 0.0f;
                    const int len = lreg[h][k];
                    const bool active = j < len;
                    const float hp = hreg[h][k], cp = creg[h][k];
                    float cx = cp;
                    const float hx = gates_one_phase(
                        op, xw[k],
                        [&](int g) {
                            float v = part[g][0];
#pragma unroll
                            for (int w2 = 1; w2 < 4; ++w2)
                                v = v + part[g][w2];    // fixed wave order
                            return v;
                        },
                        [&](int e) { return kc[h][k][e]; }, Pd != nullptr, a.clip_on, a.clip,
                        a.input_forget != 0, hp, cx, F, Gf, Hf);
                    const float hn = active ? hx : hp;   // carried when inactive
                    hreg[h][k] = hn;
                    creg[h][k] = active ? cx : cp;
                    store_coherent(hnext + hoff[h][k], hn);
                    if (a.Y) {
                        const int t = active ? (rev ? len - 1 - j : j) : j;
                        a.Y[yoff[h][k] + (size_t)t * ystep] = active ? canon_nan(hn) : 0.0f;
                    }
                }
            };
            if constexpr (ACT == 1 || ACT == 4)
                run_pairs(ActSigmoid{}, ActTanh{}, ActTanh{});
            else if constexpr (ACT == 2)
                run_pairs(ActHardSigmoid{fa.alpha, fa.beta}, ActTanh{}, ActTanh{});
            else if constexpr (ACT == 3)
                run_pairs(ActTanh{}, ActTanh{}, ActTanh{});
            else
                run_pairs(ActAny{fa}, ActAny{ga}, ActAny{ha});
            RNN_STAMP(slot, 4);
            // the last unit block also zeroes this half's padding columns [H, Hp)
            if (u0 + uc == a.H && Hp > a.H) {
                const int padw = Hp - a.H;
                const int hr = hpairs / uc;
                for (int e = tid; e < hr * padw; e += 256)
                    store_coherent(hnext + (size_t)(hrow0 + e / padw) * Hp + a.H + e % padw, 0.0f);
            }
            // published from inside the next product (there is one whenever a
            // later step exists: half 1 of this step, or half 0 of the next)
            if (q + 1 < a.q_end) {
                pend_h = h;
                pend_v = (uint32_t)(q + 1);
                pend_gen = gens[h]++;
            }
        }
        pj = pj1;
    }

    // ---- end of this launch: keep or publish the states ----------------------
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < P; ++k)
            if (pk[h][k] >= 0) {
                const int pi = (pk[h][k] >> 16) * uc + (pk[h][k] & 0xffff);
                hst[pi] = hreg[h][k];
                cst[pi] = creg[h][k];
            }
    __syncthreads();                             // (the loop below maps pairs to threads anew)
    const bool done = a.q_end == a.S;
    for (int pi = tid; pi < npairs; pi += 256) {
        const int rl = pi / uc, u = pi - rl * uc;
        const int s = row0 + rl;
        const int b = a.order ? a.order[s] : s;           // batch row (outputs)
        if (op == RNN_OP_LSTM)
            a.cbuf[((size_t)d * a.Bt + s) * a.H + u0 + u] = cst[pi];
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

}  // namespace rnnamd
