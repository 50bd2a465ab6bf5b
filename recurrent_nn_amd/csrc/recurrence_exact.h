// recurrence_exact.h -- the step loop in exact mode (onemodel "Recurrent
// operators", section "Exact mode": the same bits on every machine; the
// operator itself as in section "Computation" and the pre-activation / LSTM /
// GRU / RNN paragraphs, masking and reverse traversal as in "Choices the
// specification leaves open").
//
// Same work split, H history ring, flags and writers as the fast kernels
// (recurrence_kernel.h); what differs is the product and the activations:
//   - every recurrent product Rec[row][col] is ONE accumulator that starts
//     at +0 and adds the binary32 products H[row][k] * R[col][k] for
//     k = 0, 1, ..., H-1 in order, each multiply and add rounded on its own
//     (plain VALU arithmetic; no matrix cores, no split of k), so the value
//     does not depend on the tiling or the grid;
//   - the activations are the exact-mode ones (exact_math.h).
// Each phase stages k-chunks of the block's H rows and R rows in LDS (the
// next chunk is loaded into registers while the current one is consumed);
// thread t owns columns c and c + NTC/2 of the block, c = t % (NTC/2), and
// rows t / (NTC/2) + rpp * i, i < NACC, all in registers, and reads four
// consecutive k of its H rows and R rows per LDS access.  Summing the padding columns [H, Hp) (zeros in H and
// in the packed R) adds +0 to a sum that started at +0, which leaves it
// unchanged: such a sum is never -0.
#pragma once

#include "exact_math.h"
#include "recurrence_kernel.h"

namespace rnnamd {

constexpr int kExactKT = 64;         // k values per staged chunk (Hp, a multiple of 64, is a multiple)
constexpr int kExactKTP = kExactKT + 4;   // LDS row stride (floats)
// Threads per workgroup: sixteen waves, four per SIMD, so that one wave's LDS
// and dependency waits are covered by the others' arithmetic.
constexpr int kExactThreads = 1024;

// LDS bytes: H chunk [BT][KTP], R chunk [NTC][KTP], the sums [BT][NTC],
// then h, c, z per pair, lengths, per-unit constants.
__host__ __device__ inline size_t rec_exact_lds_bytes(int bt, int nt, int u)
{
    const size_t ntc = (size_t)nt * 16;
    return (bt * (size_t)kExactKTP + ntc * kExactKTP + (size_t)bt * ntc +
            3 * (size_t)bt * u + bt + 11 * (size_t)u) * 4;
}

// Rows per thread for a block of bt rows and ntc columns (two columns per
// thread, kExactThreads threads): the rows per pass rpp = kExactThreads /
// (ntc / 2), and ceil(bt / rpp) rounded up to a power of two (at most 4 for
// the blocks exact mode takes: bt <= 64, ntc <= 128).
__host__ __device__ inline int rec_exact_nacc(int bt, int ntc)
{
    const int rpp = kExactThreads / (ntc / 2);
    const int need = (bt + rpp - 1) / rpp;
    int n = 1;
    while (n < need)
        n *= 2;
    return n;
}

template <int NACC>
__global__ void __launch_bounds__(kExactThreads, 1) rec_exact_kernel(RecArgs a)
{
    constexpr int KT = kExactKT, KTP = kExactKTP;
    const int BT = a.BT;
    const int NTC = a.NT * 16;
    extern __shared__ __attribute__((aligned(16))) float smem[];
    float *hs = smem;                            // [BT][KTP]  H rows, one k chunk
    float *rs = hs + BT * KTP;                   // [NTC][KTP] R rows, one k chunk
    float *red = rs + NTC * KTP;                 // [BT][NTC]   the products of this phase
    float *hst = red + BT * NTC;                 // [BT * U]
    float *cst = hst + BT * a.U;
    float *zst = cst + BT * a.U;
    int *lst = (int *)(zst + BT * a.U);          // [BT]
    float *cst_u = (float *)(lst + BT);          // [11][U]

    const int tid = threadIdx.x;
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
    const int op = a.op;
    const size_t plane = (size_t)a.D * a.Btp * Hp;
    const size_t drow = ((size_t)d * a.Btp + row0) * Hp;
    const int grp = d * a.NBB + bb;
    const int ring_n = a.xw_steps + 1;
    const ActSpec fa = a.act[d][0], ga = a.act[d][1], ha = a.act[d][2];
    const ActExact F{fa}, Gf{ga}, Hf{ha};

    const float *Wb = a.B ? a.B + (size_t)d * 2 * GH : nullptr;
    const float *Rb = a.B ? Wb + GH : nullptr;
    const float *Pd = a.P ? a.P + (size_t)d * 3 * a.H : nullptr;
    const size_t xwd = (size_t)d * a.xw_steps * a.Bt * GH + (size_t)ub * a.G * a.U;
    const int npairs = rows * uc;
    // packed R rows of this block: [NTC][Hp]
    const float *rblk = a.Rp + (size_t)(d * a.NUB + ub) * NTC * Hp;

    // states at the start of this launch
    {
        const int j0 = a.q_begin / a.phases;
        for (int pi = tid; pi < npairs; pi += kExactThreads) {
            const int rl = pi / uc, u = pi - rl * uc;
            const int s = row0 + rl;                      // position
            hst[pi] = a.hbuf[(size_t)(j0 % ring_n) * plane + drow + (size_t)rl * Hp + u0 + u];
            cst[pi] = op == RNN_OP_LSTM ? a.cbuf[((size_t)d * a.Bt + s) * a.H + u0 + u] : 0.0f;
            zst[pi] = (a.phases == 2 && (a.q_begin % 2) == 1)
                          ? a.zbuf[((size_t)d * a.Bt + s) * a.H + u0 + u]
                          : 0.0f;
        }
        for (int rl = tid; rl < rows; rl += kExactThreads)
            lst[rl] = a.lens[row0 + rl];
        for (int e = tid; e < 11 * uc; e += kExactThreads) {
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
        __syncthreads();
    }

    // thread -> (columns c, c + NC2; rows r0 + rpp * i)
    const int NC2 = NTC / 2;
    const int rpp = kExactThreads / NC2;         // rows per pass (NTC <= 128)
    const int c = tid % NC2;
    const int r0 = tid / NC2;
    const bool worker = r0 < rpp;
    // staging: H chunk = BT rows x KT/4 float4, R chunk = ncol rows x KT/4
    constexpr int Q = KT / 4;                    // float4 per row and chunk
    constexpr int SH = (64 * Q + kExactThreads - 1) / kExactThreads;    // H float4 per thread (BT <= 64)
    constexpr int SR = (128 * Q + kExactThreads - 1) / kExactThreads;   // R float4 per thread (ncol <= 128)
    const int nchunks = Hp / KT;

    bool dead = false;
    for (int q = a.q_begin; q < a.q_end; ++q) {
        const int j = q / a.phases;
        const int ph = q - j * a.phases;
        const bool last_phase = ph == a.phases - 1;
        // this phase's columns of the block: phase 0 tiles [0, NTA), phase 1 [NTA, NT)
        const int cb = ph == 0 ? 0 : a.NTA * 16;
        const int ncol = (ph == 0 ? a.NTA : a.NTB) * 16;
        const float *asrc = (ph == 0 ? a.hbuf + (size_t)(j % ring_n) * plane
                                     : a.sbuf + (size_t)(j % a.xw_steps) * plane) + drow;
        const float *rsrc = rblk + (size_t)cb * Hp;

        // ---- the product, one accumulator per output, k increasing --------
        f4 hreg[SH], rreg[SR];
        auto gload = [&](int kc) {
            const int k0 = kc * KT;
#pragma unroll
            for (int i = 0; i < SH; ++i) {
                const int e = tid + kExactThreads * i, rl = e / Q, kq = e - rl * Q;
                if (rl < BT)
                    hreg[i] = *(const f4 *)(asrc + (size_t)rl * Hp + k0 + 4 * kq);
            }
#pragma unroll
            for (int i = 0; i < SR; ++i) {
                const int e = tid + kExactThreads * i, cl = e / Q, kq = e - cl * Q;
                if (cl < ncol)
                    rreg[i] = *(const f4 *)(rsrc + (size_t)cl * Hp + k0 + 4 * kq);
            }
        };
        auto sstore = [&]() {
#pragma unroll
            for (int i = 0; i < SH; ++i) {
                const int e = tid + kExactThreads * i, rl = e / Q, kq = e - rl * Q;
                if (rl < BT)
                    *(f4 *)(hs + rl * KTP + 4 * kq) = hreg[i];
            }
#pragma unroll
            for (int i = 0; i < SR; ++i) {
                const int e = tid + kExactThreads * i, cl = e / Q, kq = e - cl * Q;
                if (cl < ncol)
                    *(f4 *)(rs + cl * KTP + 4 * kq) = rreg[i];
            }
        };
        float acc[NACC], acc2[NACC];
#pragma unroll
        for (int i = 0; i < NACC; ++i)
            acc[i] = acc2[i] = 0.0f;
        // rows past the block's BT read row BT - 1; their sums are never stored
        int hrow[NACC];
#pragma unroll
        for (int i = 0; i < NACC; ++i)
            hrow[i] = min(r0 + rpp * i, BT - 1) * KTP;
        const bool computes = worker && c < ncol;
        gload(0);
        for (int kc = 0; kc < nchunks; ++kc) {
            __syncthreads();                     // the previous chunk is consumed
            sstore();
            __syncthreads();
            if (kc + 1 < nchunks)
                gload(kc + 1);
            if (computes) {
                // (the whole chunk unrolled: its LDS reads issue ahead of the
                // arithmetic that waits for them; 7% faster than two at a time)
#pragma unroll
                for (int kk = 0; kk < KT; kk += 4) {
                    const f4 rv = *(const f4 *)(rs + c * KTP + kk);
                    const f4 rv2 = *(const f4 *)(rs + (c + NC2) * KTP + kk);
#pragma unroll
                    for (int i = 0; i < NACC; ++i) {
                        const f4 hv = *(const f4 *)(hs + hrow[i] + kk);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            acc[i] = __fadd_rn(acc[i], __fmul_rn(hv[e], rv[e]));
                            acc2[i] = __fadd_rn(acc2[i], __fmul_rn(hv[e], rv2[e]));
                        }
                    }
                }
            }
        }
        if (computes) {
#pragma unroll
            for (int i = 0; i < NACC; ++i) {
                const int rl = r0 + rpp * i;
                if (rl < rows) {
                    red[rl * NTC + cb + c] = acc[i];
                    if (c + NC2 < ncol)
                        red[rl * NTC + cb + c + NC2] = acc2[i];
                }
            }
        }
        __syncthreads();

        // ---- gate arithmetic of each (row, unit) pair, in the written order
        float *hnext = a.hbuf + (size_t)((j + 1) % ring_n) * plane + drow;
        float *snext = a.sbuf ? a.sbuf + (size_t)(j % a.xw_steps) * plane + drow : nullptr;
        for (int pi = tid; pi < npairs; pi += kExactThreads) {
            const int rl = pi / uc, u = pi - rl * uc;
            const int s = row0 + rl;                      // position (XW row)
            const int b = a.order ? a.order[s] : s;       // batch row (outputs)
            const int gu = u0 + u;
            const int len = lst[rl];
            const bool active = j < len;
            const float hp = hst[pi];
            float hn = hp, cn = cst[pi];
            float xv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (active) {
                const float *src = a.XW + xwd + ((size_t)(j - a.j_base) * a.Bt + s) * GH + u;
                for (int g = 0; g < a.G; ++g)
                    xv[g] = src[g * uc];
            }
            const float *rr = red + rl * NTC;
            if (active) {
                if (a.phases == 1) {
                    hn = gates_one_phase(
                        op, xv, [&](int g) { return rr[g * uc + u]; },
                        [&](int e) { return cst_u[e * a.U + u]; }, Pd != nullptr,
                        a.clip_on, a.clip, a.input_forget != 0, hp, cn, F, Gf, Hf);
                } else if (ph == 0) {                   // GRU lbr = 0: z and r
                    float r;
                    zst[pi] = gru0_gates(xv[0], xv[1], rr[u], rr[uc + u], cst_u, a.U, u,
                                         a.clip_on, a.clip, F, &r);
                    store_coherent(snext + (size_t)rl * Hp + gu, r * hp);   // r (.) H_prev
                } else {                                // GRU lbr = 0: candidate
                    hn = gru0_candidate(xv[2], rr[a.NTA * 16 + u], cst_u, a.U, u, a.clip_on,
                                        a.clip, zst[pi], hp, Gf);
                }
            } else if (a.phases == 2 && ph == 0) {
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
        }
        // the last unit block also zeroes the padding columns [H, Hp)
        if (u0 + uc == a.H && Hp > a.H && (last_phase || a.phases == 2)) {
            float *pl = last_phase ? hnext : snext;
            const int padw = Hp - a.H;
            for (int e = tid; e < rows * padw; e += kExactThreads)
                store_coherent(pl + (size_t)(e / padw) * Hp + a.H + e % padw, 0.0f);
        }
        if (q + 1 < a.q_end)
            group_barrier(a.bar + (size_t)grp * 2 * a.NUB, a.NUB, ub, (uint32_t)(q + 1), a.err,
                          a.spin_limit, a.withhold_flags != 0, dead);
        else
            __syncthreads();
    }

    // ---- end of this launch: keep or publish the states ---------------------
    const bool done = a.q_end == a.S * a.phases;
    for (int pi = tid; pi < npairs; pi += kExactThreads) {
        const int rl = pi / uc, u = pi - rl * uc;
        const int s = row0 + rl;
        const int b = a.order ? a.order[s] : s;           // batch row (outputs)
        const size_t so = ((size_t)d * a.Bt + s) * a.H + u0 + u;
        if (op == RNN_OP_LSTM)
            a.cbuf[so] = cst[pi];
        if (a.phases == 2)
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

}  // namespace rnnamd
