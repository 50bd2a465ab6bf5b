// recurrence_fused.h -- the two-half step loop of recurrence_pipe.h with the
// input projection computed inside it (onemodel "Recurrent operators",
// section "Computation": step 1's product X . W^T, restricted to the rows of
// one step, then step 2 and the gate arithmetic as in the step loop;
// "Choices the specification leaves open" for which X row a step of a
// reversed or shortened row reads).
//
// A workgroup needs the projections of its own gate columns for its own
// batch rows only.  It keeps that slice of W (its 16 * NT gate columns over
// all I inputs) in LDS for the whole launch and, during step q, computes the
// projections that step q + 1 reads, in two k halves: one after each
// half-step's gate arithmetic and H stores.  That matrix work runs while the
// half's H stores are acknowledged and its flag reaches the other
// workgroups, so the next recurrent product finds its flags set and issues
// its loads behind no pending store; the separate projection launch and its
// XW buffer in device memory are not needed.
//
// Each projection value is one accumulator per output over k in 16-wide
// blocks in increasing order, each block as four v_mfma_f32_16x16x4_f32 with
// lane (r, q) supplying k = 4q .. 4q + 3 of the block: the chain of the
// projection kernel (proj_gemm.hip).  The values, and with them every
// output, are bit-identical to the unfused kernels.
#pragma once

#include "recurrence_pipe.h"

namespace rnnamd {

// Depth of the X fragment prefetch of the fused projection, in k blocks: 8
// blocks of matrix work (about 2k cycles at two tiles per wave) cover the
// acknowledgement of the H stores issued just before the projection starts.
constexpr int kFusedXRing = 8;

// LDS bytes: the W slice [NTC][I], the partial tiles of one half, the step's
// projections [NTC][BT + 4], lengths, per-unit constants, two publish
// counters.  The states at the start and the end of a launch pass through
// the partial-tile area.
__host__ __device__ inline size_t rec_fused_lds_bytes(int bt, int nt, int u, int64_t I)
{
    const size_t ntc = (size_t)nt * 16;
    return (ntc * (size_t)I + 4 * ntc * (size_t)(bt / 2 + 4) + ntc * (size_t)(bt + 4) + (size_t)bt +
            11 * (size_t)u + 2) * 4;
}

// Shapes the fused kernel takes: I in whole 256-input ranges (each half-step
// then covers a whole number of prefetch rounds) and the workgroup's LDS
// within the 160 KiB of a CU.
__host__ __device__ inline bool rec_fused_shape_ok(int bt, int nt, int u, int64_t I)
{
    return I >= 256 && I % 256 == 0 && rec_fused_lds_bytes(bt, nt, u, I) <= 160 * 1024;
}

template <int MTH, int NT, int KBR, int ACT, int P>
__global__ void __launch_bounds__(256, 1) rec_fused_kernel(RecArgs a)
{
    constexpr int BTH = MTH * 16;                // rows per half
    constexpr int BT = 2 * BTH;
    constexpr int NTC = NT * 16;
    constexpr int LDC = BTH + 4;                 // partial tiles: column stride (floats)
    constexpr int LDX = BT + 4;                  // projections: column stride (floats)
    constexpr int GC = ACT == 1 ? 4 : (ACT == 2 || ACT == 4) ? 3 : ACT == 3 ? 1 : 4;
    // publish / poll positions of the recurrent product, as in the two-half
    // kernel (the publish there only when the projection's k half is too
    // short to hold it)
    constexpr int KH = KBR >= 4 ? 2 : KBR / 2;
    // (the poll one block after the last A prefetch: 20.4 against 20.2 us
    // per step at block 13 and 14 of 16)
    constexpr int KPF = KBR - (kPipePrefetch < KBR ? kPipePrefetch : KBR);
    constexpr int KP0 = KPF + 1 > KH + 1 ? KPF + 1 : KH + 1;
    constexpr int KP = KP0 < KBR ? KP0 : KBR - 1;
    static_assert(KP > KH && KP < KBR, "the poll falls inside the product, after the publish");
    constexpr bool EARLY = 4 * MTH * NT * KBR >= 128;
    constexpr int XR = kFusedXRing;
    // Projection tiles: BT / 16 row tiles x NT column tiles.  With four row
    // tiles each wave takes one row tile and every column tile (its X
    // fragment serves NT accumulators); with two, one tile per wave (waves 2
    // and 3 idle when NT = 1).
    constexpr int XNT = MTH == 2 ? NT : 1;

    const int I = (int)a.I;
    const int KXH = I / 32;                      // 16-wide k blocks per half-step
    // the flag of a half goes out from inside the projection when its k half
    // has room for it after the first prefetch round (I >= 512)
    const bool pub_in_x = KXH >= 2 * XR;

    extern __shared__ float smem[];
    float *wl = smem;                            // [NTC][I] W slice, 16-byte chunks XOR-swizzled
    float *red = wl + (size_t)NTC * I;           // [4 waves][NTC][LDC] partial tiles of a half
    float *xs = red + 4 * NTC * LDC;             // [NTC][LDX] projections of the current step
    int *lst = (int *)(xs + NTC * LDX);          // [BT] sequence length of each row
    float *cst_u = (float *)(lst + BT);          // [11][U] Wb, Rb per gate, then Pi, Po, Pf
    uint32_t *ctr = (uint32_t *)(cst_u + 11 * a.U);   // [2] arrivals at each half's publish
    float *hst = red;                            // [BT * U] states (launch start and end)
    float *cst = red + BT * a.U;                 // [BT * U]

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    // same workgroup -> (d, batch block, unit block) map as the other kernels
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
    const int npairs = rows * uc;

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

    // W slice: row n = gate column n of this unit block (packed W row
    // ub * G * U + n, zero past the block's G * uc columns); 16-byte chunk c
    // of row n at chunk c ^ (n mod 8), so that the 8 lanes of a fragment read
    // that share a chunk index hit distinct banks.
    {
        const float *Wd = a.Wp + ((size_t)d * GH + (size_t)ub * a.G * a.U) * I;
        const int cpr = I / 4;                   // chunks per row
        const int gcols = a.G * uc;
        for (int e = tid; e < NTC * cpr; e += 256) {
            const int n = e / cpr, c = e - n * cpr;
            const f4 v = n < gcols ? *(const f4 *)(Wd + (size_t)n * I + 4 * c) : f4{0.f, 0.f, 0.f, 0.f};
            *(f4 *)(wl + (size_t)n * I + 4 * (c ^ (n & 7))) = v;
        }
    }
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

    auto hpairs_of = [&](int h) { return max(0, min(BTH, rows - h * BTH)) * uc; };
    int pk[2][P];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int i = tid + 256 * k;
            pk[h][k] = i < hpairs_of(h) ? ((h * BTH + i / uc) << 16) | (i % uc) : -1;
        }
    const int G = ACT == 0 ? a.G : GC;
    const size_t ystep = a.layout == 0 ? (size_t)a.D * a.Bt * a.H : (size_t)a.D * a.H;
    float hreg[2][P], creg[2][P], kc[2][P][11];
    int lreg[2][P];
    uint32_t hoff[2][P];
    size_t yoff[2][P];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int rl = pk[h][k] < 0 ? 0 : pk[h][k] >> 16, u = pk[h][k] < 0 ? 0 : pk[h][k] & 0xffff;
            const int pi = rl * uc + u;
            const int s = row0 + rl, gu = u0 + u;
            const int b = a.order ? a.order[s] : s;
            hreg[h][k] = hst[pi];
            creg[h][k] = cst[pi];
            lreg[h][k] = pk[h][k] < 0 ? 0 : lst[rl];
#pragma unroll
            for (int e = 0; e < 11; ++e)
                kc[h][k][e] = cst_u[e * a.U + u];
            hoff[h][k] = (uint32_t)(rl * Hp + gu);
            yoff[h][k] = a.layout == 0 ? ((size_t)d * a.Bt + b) * a.H + gu
                                       : ((size_t)b * a.S * a.D + d) * a.H + gu;
        }
    __syncthreads();                             // (the states' area becomes the partial tiles)

    // ---- the projection ------------------------------------------------------
    const int xrt = MTH == 2 ? w : (w & 1);     // this wave's row tile
    const int xnt0 = (MTH == 1 && NT == 2) ? (w >> 1) : 0;
    const bool xon = MTH == 2 || NT == 2 || w < 2;
    // this lane's row of the row tile (clamped into the block), its length
    // and batch row; step qn of it reads X at time qn forward, len - 1 - qn
    // in reverse (a step past its length reads time 0; its values are never
    // used)
    const int xrl = min(xrt * 16 + lr, rows - 1);
    const int xlen = a.lens[row0 + xrl];
    const int xb = a.order ? a.order[row0 + xrl] : row0 + xrl;
    auto x_src = [&](int qn) {
        const int t = qn < xlen ? (rev ? xlen - 1 - qn : qn) : 0;
        const size_t xi = a.layout == 0 ? (size_t)t * a.Bt + xb : (size_t)xb * a.S + t;
        return a.X + xi * I + 4 * lq;
    };
    f4 xa[XR];                                   // X fragments in flight
    f4 xacc[XNT];
#pragma unroll
    for (int nt = 0; nt < XNT; ++nt)
        xacc[nt] = f4{0.f, 0.f, 0.f, 0.f};
    // W fragment of column tile nt, k block kb: row n = tile column lr,
    // chunk 4 kb + lq, swizzled by n mod 8 = lr mod 8.  For kb = 2 p + e the
    // chunk is 8 p + ((4 e + lq) ^ (lr mod 8)): its byte address is the
    // lane's base for parity e plus 128 p, a constant inside a round.
    const char *wbase[XNT][2];
#pragma unroll
    for (int nt = 0; nt < XNT; ++nt)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            wbase[nt][e] = (const char *)(wl + (size_t)((xnt0 + nt) * 16 + lr) * I) +
                           16 * ((4 * e + lq) ^ (lr & 7));
    auto w_frag = [&](int nt, int kb) {
        return *(const f4 *)(wbase[nt][kb & 1] + 128 * (kb >> 1));
    };
    // the first XR k blocks of the half starting at block kb0
    auto x_prime = [&](const float *src, int kb0) {
        if (xon) {
#pragma unroll
            for (int i = 0; i < XR; ++i)
                xa[i] = *(const f4 *)(src + (size_t)(kb0 + i) * 16);
        }
    };
    // k blocks [kb0, kb0 + KXH) of the step's projections (primed by
    // x_prime), in rounds of XR blocks; at_pub() runs at the top of block
    // XR + 1 (when pub_in_x), at_prime() at the top of block KXH - 6.  Every
    // address inside a round is a per-round base plus a constant, and the
    // last round (no loads) is its own copy, so that no vector instruction
    // sits between the MFMAs of a round (on this part a vector instruction
    // waits for the matrix pipe to drain).
    auto x_slice = [&](const float *src, int kb0, auto at_pub, auto at_prime) {
        // W fragments double-buffered by block parity (XR is even, so every
        // round starts on buffer 0 and nothing rotates between rounds); each
        // X fragment is reloaded only after its MFMAs, into its own
        // registers
        f4 wb[2][XNT];
        if (xon) {
#pragma unroll
            for (int nt = 0; nt < XNT; ++nt)
                wb[0][nt] = w_frag(nt, kb0);
        }
        auto round = [&](int g, auto more_c) {
            constexpr bool MORE = decltype(more_c)::value;   // a later round follows
            const bool pub = g == XR;
            // this round's bases: W blocks kb0 + g .. (128 bytes per block
            // pair), X blocks kb0 + g + XR .. (64 bytes per block)
            const int wo = 64 * (kb0 + g);
            const float *xr = src + (size_t)(kb0 + g + XR) * 16;
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                if (i == 1 && pub)
                    at_pub();
                if (i == 2 && !MORE)
                    at_prime();
                if (xon) {
                    // (the W fragment after the last block of the step reads
                    // the next row or the partial tiles: in LDS, not used)
#pragma unroll
                    for (int nt = 0; nt < XNT; ++nt)
                        wb[(i + 1) & 1][nt] =
                            *(const f4 *)(wbase[nt][(i + 1) & 1] + wo + 128 * ((i + 1) >> 1));
                    // (the next block's W reads go out before this block's
                    // MFMAs: left alone, the scheduler sinks them to their use)
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int nt = 0; nt < XNT; ++nt)
                            xacc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[i][s], wb[i & 1][nt][s],
                                                                            xacc[nt], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (MORE)
                        xa[i] = *(const f4 *)(xr + 16 * i);
                }
            }
        };
        int g = 0;
        for (; g + XR < KXH; g += XR)
            round(g, std::true_type{});
        round(g, std::false_type{});
    };
    // the step's projections into xs (lane: rows 4 lq .. 4 lq + 3, column lr
    // of each tile), then cleared for the next step
    auto x_store = [&]() {
        if (xon) {
#pragma unroll
            for (int nt = 0; nt < XNT; ++nt) {
                *(f4 *)(xs + ((xnt0 + nt) * 16 + lr) * LDX + xrt * 16 + 4 * lq) = xacc[nt];
                xacc[nt] = f4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto no_hook = []() {};

    // the projections of the launch's first step
    if (a.q_begin < a.q_end) {
        const float *src = x_src(a.q_begin);
        x_prime(src, 0);
        x_slice(src, 0, no_hook, no_hook);
        x_prime(src, KXH);
        x_slice(src, KXH, no_hook, no_hook);
        x_store();
    }
    __syncthreads();

    bool dead = false;
    // a publish left pending: half, flag value, generation
    int pend_h = -1;
    uint32_t pend_v = 0, pend_gen = 0;
    uint32_t gens[2] = {0u, 0u};
    // each wave counts itself in once its own H stores have completed; the
    // last of the four stores the flag
    auto arrive = [&]() {
        if (lane == 0) {
            const uint32_t old = __hip_atomic_fetch_add(ctr + pend_h, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_WORKGROUP);
            if (old == 4u * pend_gen + 3u && !a.withhold_flags)
                __hip_atomic_store(flags0 + (size_t)pend_h * a.NUB + ub, pend_v, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        pend_h = -1;
    };
    // from the next recurrent product (a short projection half): wait for
    // every store
    auto publish_full = [&]() {
        if (pend_h >= 0) {
            wait_stores();
            arrive();
        }
    };
    // from inside the projection, at block XR + 1: vector memory operations
    // complete in issue order and at most XR loads (of blocks XR + 1 .. 2 XR)
    // were issued after block XR's, so once at most XR - 1 are outstanding
    // block XR's load has returned and the H stores issued before the
    // projection's first load have completed.  A wave with no projection
    // tile has only its stores outstanding.
    auto publish_x = [&]() {
        if (pend_h >= 0) {
            if (xon)
                asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
            else
                wait_stores();
            arrive();
        }
    };
    static_assert(XR == 8, "publish_x waits for vmcnt(XR - 1)");

    const int ring_n = a.xw_steps + 1;
    auto a_src = [&](int pl, int h) {
        return a.hbuf + (size_t)pl * plane + drow + (size_t)(h * BTH + lr) * Hp + k0 + 4 * lq;
    };
    int pj = a.q_begin % ring_n;
    auto next_plane = [&](int pl) { return pl + 1 == ring_n ? 0 : pl + 1; };
    constexpr int RING = (kPipePrefetch < KBR ? kPipePrefetch : KBR) + 1;
    f4 ring[RING][MTH];
    if (a.q_begin < a.q_end)
        prime_ring<MTH, KBR, kPipePrefetch>(ring, a_src(pj, 0), Hp);
    bool primed = true;

    for (int q = a.q_begin; q < a.q_end; ++q) {
        const int j = q;
        const int pj1 = next_plane(pj);
        float *hnext = a.hbuf + (size_t)pj1 * plane + drow;
        // the projections of step q + 1 are computed during this step
        const bool xnext = q + 1 < a.q_end;
        const float *xsrc = x_src(xnext ? q + 1 : q);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int slot = 2 * (q - a.q_begin) + h;
            (void)slot;
            RNN_STAMP(slot, 0);
            const int hrow0 = h * BTH;
            const int hpairs = hpairs_of(h);
            const int nq = h == 0 ? q : q + 1, nh = 1 - h;
            const bool has_next = nq < a.q_end;
            if (!primed) {
                if (!dead)
                    wave_wait_flags(flags0 + (size_t)h * a.NUB + wub_lo, wub_hi - wub_lo + 1,
                                    (uint32_t)q, a.err, a.spin_limit, dead);
                prime_ring<MTH, KBR, kPipePrefetch>(ring, a_src(pj, h), Hp);
            }
            RNN_STAMP(slot, 1);

            // ---- recurrent product of this half ------------------------------
            f4 acc[MTH][NT];
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
            const uint32_t *nflags = flags0 + (size_t)nh * a.NUB + wub_lo;
            const int nfl = wub_hi - wub_lo + 1;
            const bool need_wait = has_next && nq > a.q_begin && !dead;
            // (loaded by every lane as in the two-half kernel, and compared
            // only after the product: 20.26 -> 19.85 us per step; one k
            // block after the load, 19.91)
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
            constexpr int KC = -1;
            // after the product's last A load: the first X blocks of this
            // half's share of the next step's projections
            auto mid = [&]() {
                if (xnext)
                    x_prime(xsrc, h * KXH);
            };
            product_res_hooked<MTH, NT, KBR, kPipePrefetch, KH, KP, KC>(
                acc, ring, a_src(pj, h), Hp, rr, mid, [&]() { publish_full(); }, poll_next,
                check_next);
            if constexpr (KC < 0)
                check_next();
            RNN_STAMP(slot, 2);
#pragma unroll
            for (int mt = 0; mt < MTH; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    *(f4 *)(red + (w * NTC + nt * 16 + lr) * LDC + mt * 16 + 4 * lq) = acc[mt][nt];
            __syncthreads();
            RNN_STAMP(slot, 3);
            primed = !need_wait || (EARLY && nfl <= 64 && fset);

            // ---- gate arithmetic of this thread's pairs of half h -----------
            auto run_pairs = [&](auto F, auto Gf, auto Hf) {
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    if (pk[h][k] < 0)
                        continue;
                    const int rl = pk[h][k] >> 16, u = pk[h][k] & 0xffff;
                    const int rh = rl - hrow0;
                    float part[4][4], xv[4];
                    const float *rp = red + u * LDC + rh;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
#pragma unroll
                        for (int w2 = 0; w2 < 4; ++w2)
                            part[g][w2] = g < G ? rp[(w2 * NTC + g * uc) * LDC] : 0.0f;
                        xv[g] = g < G ? xs[(g * uc + u) * LDX + rl] : 0.0f;
                    }
                    const int len = lreg[h][k];
                    const bool active = j < len;
                    const float hp = hreg[h][k], cp = creg[h][k];
                    float cx = cp;
                    const float hx = gates_one_phase(
                        op, xv,
                        [&](int g) {
                            float v = part[g][0];
#pragma unroll
                            for (int w2 = 1; w2 < 4; ++w2)
                                v = v + part[g][w2];    // fixed wave order
                            return v;
                        },
                        [&](int e) { return kc[h][k][e]; }, Pd != nullptr, a.clip_on, a.clip,
                        a.input_forget != 0, hp, cx, F, Gf, Hf);
                    const float hn = active ? hx : hp;
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
            if (u0 + uc == a.H && Hp > a.H) {
                const int padw = Hp - a.H;
                const int hr = hpairs / uc;
                for (int e = tid; e < hr * padw; e += 256)
                    store_coherent(hnext + (size_t)(hrow0 + e / padw) * Hp + a.H + e % padw, 0.0f);
            }
            RNN_STAMP(slot, 4);
            if (q + 1 < a.q_end) {
                pend_h = h;
                pend_v = (uint32_t)(q + 1);
                pend_gen = gens[h]++;
            }

            // ---- this half's share of the next step's projections ------------
            // (the half's flag goes out inside it; the next product's first
            // k blocks are loaded near its end)
            auto rprime = [&]() {
                if (has_next && primed)
                    prime_ring<MTH, KBR, kPipePrefetch>(ring, a_src(h == 0 ? pj : pj1, nh), Hp);
            };
            if (xnext) {
                x_slice(
                    xsrc, h * KXH,
                    [&]() {
                        if (pub_in_x) {
                            publish_x();
                            RNN_STAMP(slot, 5);
                        }
                    },
                    rprime);
            } else {
                rprime();
            }
            RNN_STAMP(slot, 6);
            __syncthreads();                     // every wave is done with red and xs
            if (h == 1 && xnext)
                x_store();
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
    __syncthreads();
    const bool done = a.q_end == a.S;
    for (int pi = tid; pi < npairs; pi += 256) {
        const int rl = pi / uc, u = pi - rl * uc;
        const int s = row0 + rl;
        const int b = a.order ? a.order[s] : s;
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
