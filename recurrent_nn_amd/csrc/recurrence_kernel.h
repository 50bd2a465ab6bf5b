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
// the gate arithmetic of a unit never leaves the workgroup.  Its 4 waves split
// the reduction index k of the product (Hp / 4 each) and compute the whole
// [BT x 16*NT] tile over their k range with v_mfma_f32_16x16x4_f32; the four
// partial tiles meet in LDS and are summed in a fixed order (w = 0, 1, 2, 3),
// so the result does not depend on the grid size.  With `RES` the wave's
// slice of R stays in registers for the whole sequence; otherwise it is
// re-read (from L2 / the memory-side cache) every step.
//
// Steps.  The persistent form runs every step in one cooperative launch and
// separates steps with a barrier among the workgroups of one (d, bb) group:
// a monotonic counter with an agent-scope release before the arrival and an
// acquire after the wait.  H is exchanged through a ping-pong buffer in
// device memory.  GRU with linear_before_reset = 0 has two phases per step:
// z and r first (their product over H), then the candidate's product over
// r (.) H_prev, with a barrier in between.  The per-step form runs one phase
// per launch, the kernel boundary being the barrier.
//
// Epilogue.  This file is compiled with -ffp-contract=off: every written
// addition and multiplication is its own IEEE operation, in the written order
// ("No step fuses a multiply with an add").
#pragma once

#include <hip/hip_runtime.h>

#include "activations.h"
#include "common.h"

namespace rnnamd {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Barrier among the NUB workgroups of one (direction, batch block) group.
// Returns false (and raises the error word) if the wait exceeded spin_limit.
__device__ __forceinline__ void group_barrier(uint32_t *ctr, uint32_t target, int32_t *err,
                                              uint32_t spin_limit, bool &dead)
{
    wait_stores();                 // this wave's stores have reached L2
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");        // write L2 back
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!dead) {
            uint32_t n = 0;
            while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                __builtin_amdgcn_s_sleep(1);
                if (++n > spin_limit) {
                    __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    dead = true;
                    break;
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");        // drop stale lines
    }
    __syncthreads();
}

// LDS bytes of one workgroup: the four partial tiles, then the per-pair
// states (h, c, z) and the per-row lengths.
__host__ __device__ inline size_t rec_lds_bytes(int bt, int nt, int u)
{
    return ((size_t)kWaves * bt * (nt * 16 + 4) + 3 * (size_t)bt * u + bt) * 4;
}

template <int MT, int NT, int KBR, int P>
__global__ void __launch_bounds__(kThreads, 1) rec_kernel(RecArgs a)
{
    constexpr bool RES = KBR > 0;
    constexpr int BT = MT * 16;
    constexpr int NTC = NT * 16;
    constexpr int LDR = NTC + 4;                 // LDS row stride of the partial tiles
    constexpr bool kPrefetchXW = P <= 2;         // XW loads issued before the product
    extern __shared__ float smem[];
    float *red = smem;                           // [kWaves][BT][LDR] partial tiles
    float *hst = red + kWaves * BT * LDR;        // [BT * U] h of each (row, unit) pair
    float *cst = hst + BT * a.U;                 // [BT * U] LSTM cell state
    float *zst = cst + BT * a.U;                 // [BT * U] GRU update gate between phases
    int *lst = (int *)(zst + BT * a.U);          // [BT] sequence length of each row

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
    const int GH = a.G * a.H;
    const int op = a.op;
    const size_t plane = (size_t)a.D * a.Btp * Hp;           // one hbuf plane
    const size_t drow = ((size_t)d * a.Btp + row0) * Hp;     // this group's rows
    const int grp = d * a.NBB + bb;
    const ActSpec fa = a.act[d][0], ga = a.act[d][1], ha = a.act[d][2];
    const float *Wb = a.B ? a.B + (size_t)d * 2 * GH : nullptr;
    const float *Rb = a.B ? Wb + GH : nullptr;
    const float *Pd = a.P ? a.P + (size_t)d * 3 * a.H : nullptr;
    const size_t xwd = (size_t)d * a.S * a.Bt * GH + (size_t)ub * a.G * a.U;
    const int npairs = rows * uc;

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
        const int j0 = a.q_begin / a.phases;
        for (int pi = tid; pi < npairs; pi += kThreads) {
            const int rl = pi / uc, u = pi - rl * uc;
            const int b = row0 + rl;
            hst[pi] = a.hbuf[(size_t)(j0 & 1) * plane + drow + (size_t)rl * Hp + u0 + u];
            cst[pi] = op == RNN_OP_LSTM ? a.cbuf[((size_t)d * a.Bt + b) * a.H + u0 + u] : 0.0f;
            zst[pi] = (a.phases == 2 && (a.q_begin % 2) == 1)
                          ? a.zbuf[((size_t)d * a.Bt + b) * a.H + u0 + u]
                          : 0.0f;
        }
        for (int rl = tid; rl < rows; rl += kThreads)
            lst[rl] = a.lens[row0 + rl];
        __syncthreads();
    }

    bool dead = false;
    const uint32_t nub = (uint32_t)a.NUB;
    for (int q = a.q_begin; q < a.q_end; ++q) {
        const int j = q / a.phases;
        const int ph = q - j * a.phases;
        const int t0 = ph == 0 ? 0 : a.NTA;              // this phase's column tiles
        const int t1 = ph == 0 ? a.NTA : a.NTA + a.NTB;
        const bool last_phase = ph == a.phases - 1;

        // XW of pair pi at this step, gates of this phase (0 for inactive rows)
        auto fetch_xw = [&](int pi, float *xv) {
            xv[0] = xv[1] = xv[2] = xv[3] = 0.0f;
            const int rl = pi / uc, u = pi - rl * uc;
            const int len = lst[rl];
            if (j >= len)
                return;
            const int t = rev ? len - 1 - j : j;
            const float *src = a.XW + xwd + ((size_t)t * a.Bt + row0 + rl) * GH + u;
            if (a.phases == 2 && ph == 1) {
                xv[2] = src[2 * uc];
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    if (g < a.G && !(a.phases == 2 && g == 2))
                        xv[g] = src[g * uc];
            }
        };
        float xw[kPrefetchXW ? P : 1][4];
        if constexpr (kPrefetchXW) {
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const int pi = tid + kThreads * i;
                if (pi < npairs)
                    fetch_xw(pi, xw[i]);
            }
        }

        // ---- the product over this wave's k range --------------------------
        const float *asrc = (ph == 0 ? a.hbuf + (size_t)(j & 1) * plane : a.sbuf) + drow +
                            (size_t)lr * Hp + w * KB * 16 + 4 * lq;
        f4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};

        f4 av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            av[mt] = *(const f4 *)(asrc + (size_t)mt * 16 * Hp);
        if constexpr (RES) {
#pragma unroll
            for (int kb = 0; kb < KBR; ++kb) {
                f4 an[MT];
                if (kb + 1 < KBR) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        an[mt] = *(const f4 *)(asrc + (size_t)mt * 16 * Hp + (kb + 1) * 16);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        if (nt < t0 || nt >= t1)
                            continue;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                av[mt][s], rr[nt][kb][s], acc[mt][nt], 0, 0, 0);
                    }
                if (kb + 1 < KBR) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        av[mt] = an[mt];
                }
            }
        } else {
            f4 bv[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                bv[nt] = (nt >= t0 && nt < t1) ? *(const f4 *)(rfrag + (size_t)nt * 16 * Hp)
                                               : f4{0.f, 0.f, 0.f, 0.f};
            for (int kb = 0; kb < KB; ++kb) {
                f4 an[MT], bn[NT];
                if (kb + 1 < KB) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        an[mt] = *(const f4 *)(asrc + (size_t)mt * 16 * Hp + (kb + 1) * 16);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        bn[nt] = (nt >= t0 && nt < t1)
                                     ? *(const f4 *)(rfrag + (size_t)nt * 16 * Hp + (kb + 1) * 16)
                                     : f4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        if (nt < t0 || nt >= t1)
                            continue;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                av[mt][s], bv[nt][s], acc[mt][nt], 0, 0, 0);
                    }
                if (kb + 1 < KB) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        av[mt] = an[mt];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        bv[nt] = bn[nt];
                }
            }
        }

        // ---- partial tiles -> LDS, summed in wave order ----------------------
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (nt < t0 || nt >= t1)
                    continue;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[(w * BT + mt * 16 + 4 * lq + r) * LDR + nt * 16 + lr] = acc[mt][nt][r];
            }
        __syncthreads();
        auto rec_at = [&](int rl, int col) {
            const float *p = red + rl * LDR + col;
            float s0 = p[0];
            float s1 = p[BT * LDR];
            float s2 = p[2 * BT * LDR];
            float s3 = p[3 * BT * LDR];
            float v = s0 + s1;
            v = v + s2;
            v = v + s3;
            return v;
        };

        // ---- gate arithmetic of one (row, unit) pair, in the written order --
        float *hnext = a.hbuf + (size_t)((j + 1) & 1) * plane + drow;
        auto do_pair = [&](int pi, const float *xv) {
            const int rl = pi / uc, u = pi - rl * uc;
            const int b = row0 + rl;
            const int gu = u0 + u;                         // hidden unit
            const int len = lst[rl];
            const bool active = j < len;
            const float hp = hst[pi];
            float hn = hp, cn = cst[pi];
            if (active) {
                if (op == RNN_OP_RNN) {
                    float pre = xv[0] + rec_at(rl, u);
                    if (Wb) {
                        pre = pre + Wb[gu];
                        pre = pre + Rb[gu];
                    }
                    pre = clip_pre(pre, a.clip_on, a.clip);
                    hn = act_apply(fa.kind, fa.alpha, fa.beta, pre);
                } else if (op == RNN_OP_GRU) {
                    if (a.phases == 1) {                    // linear_before_reset = 1
                        float pz = xv[0] + rec_at(rl, u);
                        float pr = xv[1] + rec_at(rl, uc + u);
                        if (Wb) {
                            pz = pz + Wb[gu];
                            pz = pz + Rb[gu];
                            pr = pr + Wb[a.H + gu];
                            pr = pr + Rb[a.H + gu];
                        }
                        pz = clip_pre(pz, a.clip_on, a.clip);
                        pr = clip_pre(pr, a.clip_on, a.clip);
                        const float z = act_apply(fa.kind, fa.alpha, fa.beta, pz);
                        const float r = act_apply(fa.kind, fa.alpha, fa.beta, pr);
                        float rh = rec_at(rl, 2 * uc + u);
                        if (Wb)
                            rh = rh + Rb[2 * a.H + gu];
                        const float gated = r * rh;
                        float ph_ = xv[2] + gated;
                        if (Wb)
                            ph_ = ph_ + Wb[2 * a.H + gu];
                        ph_ = clip_pre(ph_, a.clip_on, a.clip);
                        const float ht = act_apply(ga.kind, ga.alpha, ga.beta, ph_);
                        const float omz = 1.0f - z;
                        const float a1 = omz * ht;
                        const float a2 = z * hp;
                        hn = a1 + a2;
                    } else if (ph == 0) {                   // lbr = 0: z and r
                        float pz = xv[0] + rec_at(rl, u);
                        float pr = xv[1] + rec_at(rl, uc + u);
                        if (Wb) {
                            pz = pz + Wb[gu];
                            pz = pz + Rb[gu];
                            pr = pr + Wb[a.H + gu];
                            pr = pr + Rb[a.H + gu];
                        }
                        pz = clip_pre(pz, a.clip_on, a.clip);
                        pr = clip_pre(pr, a.clip_on, a.clip);
                        zst[pi] = act_apply(fa.kind, fa.alpha, fa.beta, pz);
                        const float r = act_apply(fa.kind, fa.alpha, fa.beta, pr);
                        a.sbuf[drow + (size_t)rl * Hp + gu] = r * hp;   // r (.) H_prev
                    } else {                                // lbr = 0: candidate
                        float ph_ = xv[2] + rec_at(rl, a.NTA * 16 + u);
                        if (Wb) {
                            ph_ = ph_ + Wb[2 * a.H + gu];
                            ph_ = ph_ + Rb[2 * a.H + gu];
                        }
                        ph_ = clip_pre(ph_, a.clip_on, a.clip);
                        const float ht = act_apply(ga.kind, ga.alpha, ga.beta, ph_);
                        const float z = zst[pi];
                        const float omz = 1.0f - z;
                        const float a1 = omz * ht;
                        const float a2 = z * hp;
                        hn = a1 + a2;
                    }
                } else {                                    // LSTM: i, o, f, c
                    float pre[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float v = xv[g] + rec_at(rl, g * uc + u);
                        if (Wb) {
                            v = v + Wb[g * a.H + gu];
                            v = v + Rb[g * a.H + gu];
                        }
                        pre[g] = v;
                    }
                    const float cp = cn;
                    if (Pd) {
                        const float pi_ = Pd[gu] * cp;
                        const float pf_ = Pd[2 * a.H + gu] * cp;
                        pre[0] = pre[0] + pi_;
                        pre[2] = pre[2] + pf_;
                    }
                    const float ci = clip_pre(pre[0], a.clip_on, a.clip);
                    const float cf = clip_pre(pre[2], a.clip_on, a.clip);
                    const float cc = clip_pre(pre[3], a.clip_on, a.clip);
                    const float ig = act_apply(fa.kind, fa.alpha, fa.beta, ci);
                    const float fg =
                        a.input_forget ? 1.0f - ig : act_apply(fa.kind, fa.alpha, fa.beta, cf);
                    const float ct = act_apply(ga.kind, ga.alpha, ga.beta, cc);
                    const float k1 = fg * cp;
                    const float k2 = ig * ct;
                    cn = k1 + k2;
                    float po = pre[1];
                    if (Pd) {
                        const float pov = Pd[a.H + gu] * cn;
                        po = po + pov;
                    }
                    po = clip_pre(po, a.clip_on, a.clip);
                    const float og = act_apply(fa.kind, fa.alpha, fa.beta, po);
                    const float hc = act_apply(ha.kind, ha.alpha, ha.beta, cn);
                    hn = og * hc;
                }
            } else if (a.phases == 2 && ph == 0) {
                a.sbuf[drow + (size_t)rl * Hp + gu] = 0.0f;
            }
            if (last_phase) {
                hnext[(size_t)rl * Hp + gu] = hn;           // carried unchanged when inactive
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

        if constexpr (kPrefetchXW) {
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const int pi = tid + kThreads * i;
                if (pi < npairs)
                    do_pair(pi, xw[i]);
            }
        } else {
#pragma unroll 1
            for (int pi = tid; pi < npairs; pi += kThreads) {
                float xv[4];
                fetch_xw(pi, xv);
                do_pair(pi, xv);
            }
        }

        if (q + 1 < a.q_end)
            group_barrier(a.bar + grp, nub * (uint32_t)(q + 1), a.err, a.spin_limit, dead);
        else
            __syncthreads();
    }

    // ---- end of this launch: keep or publish the states ---------------------
    const bool done = a.q_end == a.S * a.phases;
    for (int pi = tid; pi < npairs; pi += kThreads) {
        const int rl = pi / uc, u = pi - rl * uc;
        const int b = row0 + rl;
        const size_t so = ((size_t)d * a.Bt + b) * a.H + u0 + u;
        if (op == RNN_OP_LSTM)
            a.cbuf[so] = cst[pi];
        if (a.phases == 2)
            a.zbuf[so] = zst[pi];
        if (done) {
            const size_t yo = a.layout == 0 ? so : ((size_t)b * a.D + d) * a.H + u0 + u;
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
