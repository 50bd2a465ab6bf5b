// recurrence.hip -- selection and launch of the step-loop kernels
// (recurrence_kernel.h, recurrence_pipe.h, recurrence_fused.h,
// recurrence_exact.h): the compiled
// shapes (tables in recurrence_inst.hip, one per kernel family and activation
// set), the occupancy check of the persistent (cooperative) form, and the
// launches.
#include <hip/hip_runtime.h>

#include "recurrence_exact.h"
#include "recurrence_fused.h"

namespace rnnamd {

#define RNN_DECL(A)                                                                               \
    rec_fn rec_get_resident_a##A(int nw, int mt, int nt, int kb, int ta);                         \
    rec_fn rec_get_streamed2_a##A(int mt, int nt, int ta);                                        \
    rec_fn rec_get_streamed8_a##A(int mt, int nt, int ta);                                        \
    rec_fn rec_get_pipe_a##A(int mth, int nt, int kb, int p);                                      \
    rec_fn rec_get_fused_a##A(int mth, int nt, int kb, int p);
RNN_DECL(0)
RNN_DECL(1)
RNN_DECL(2)
RNN_DECL(3)
RNN_DECL(4)
#undef RNN_DECL

// Operator and activation set compiled into the kernel: 1 LSTM with
// Sigmoid/Tanh/Tanh, 2 GRU with HardSigmoid/Tanh, 3 RNN with Tanh, 4 GRU with
// Sigmoid/Tanh, 0 anything else (run-time switch).
static int act_set(const RecArgs &a)
{
    bool same = true;                      // both directions use the same kinds
    for (int d = 1; d < a.D; ++d)
        for (int k = 0; k < 3; ++k)
            same = same && a.act[d][k].kind == a.act[0][k].kind;
    if (!same)
        return 0;
    const int f = a.act[0][0].kind, g = a.act[0][1].kind, h = a.act[0][2].kind;
    if (a.op == RNN_OP_LSTM && f == ACT_SIGMOID && g == ACT_TANH && h == ACT_TANH)
        return 1;
    if (a.op == RNN_OP_GRU && f == ACT_SIGMOID && g == ACT_TANH)
        return 4;
    if (a.op == RNN_OP_GRU && f == ACT_HARDSIGMOID && g == ACT_TANH)
        return 2;
    if (a.op == RNN_OP_RNN && f == ACT_TANH)
        return 3;
    return 0;
}

static rec_fn get_resident(int act, int nw, int mt, int nt, int kb, int ta)
{
    switch (act) {
    case 1: return rec_get_resident_a1(nw, mt, nt, kb, ta);
    case 2: return rec_get_resident_a2(nw, mt, nt, kb, ta);
    case 3: return rec_get_resident_a3(nw, mt, nt, kb, ta);
    case 4: return rec_get_resident_a4(nw, mt, nt, kb, ta);
    default: return rec_get_resident_a0(nw, mt, nt, kb, ta);
    }
}

static rec_fn get_streamed(int act, int p, int mt, int nt, int ta)
{
    switch (act) {
    case 1: return p == 2 ? rec_get_streamed2_a1(mt, nt, ta) : rec_get_streamed8_a1(mt, nt, ta);
    case 2: return p == 2 ? rec_get_streamed2_a2(mt, nt, ta) : rec_get_streamed8_a2(mt, nt, ta);
    case 3: return p == 2 ? rec_get_streamed2_a3(mt, nt, ta) : rec_get_streamed8_a3(mt, nt, ta);
    case 4: return p == 2 ? rec_get_streamed2_a4(mt, nt, ta) : rec_get_streamed8_a4(mt, nt, ta);
    default: return p == 2 ? rec_get_streamed2_a0(mt, nt, ta) : rec_get_streamed8_a0(mt, nt, ta);
    }
}

static rec_fn get_pipe(int act, int mth, int nt, int kb, int p)
{
    switch (act) {
    case 1: return rec_get_pipe_a1(mth, nt, kb, p);
    case 2: return rec_get_pipe_a2(mth, nt, kb, p);
    case 3: return rec_get_pipe_a3(mth, nt, kb, p);
    case 4: return rec_get_pipe_a4(mth, nt, kb, p);
    default: return rec_get_pipe_a0(mth, nt, kb, p);
    }
}

static rec_fn get_fused(int act, int mth, int nt, int kb, int p)
{
    switch (act) {
    case 1: return rec_get_fused_a1(mth, nt, kb, p);
    case 2: return rec_get_fused_a2(mth, nt, kb, p);
    case 3: return rec_get_fused_a3(mth, nt, kb, p);
    case 4: return rec_get_fused_a4(mth, nt, kb, p);
    default: return rec_get_fused_a0(mth, nt, kb, p);
    }
}

static rec_fn pick(const RecArgs &a, int resident)
{
    if (a.exact) {  // exact mode: up to 128 columns and 64 rows per block
        if (a.NT * 16 > 128 || a.BT > 64 || a.Hp % kExactKT != 0)
            return nullptr;
        switch (rec_exact_nacc(a.BT, a.NT * 16)) {
        case 1: return rec_exact_kernel<1>;
        case 2: return rec_exact_kernel<2>;
        case 4: return rec_exact_kernel<4>;
        default: return nullptr;
        }
    }
    if (a.halves == 2) {
        // two half-batch sub-steps per step: R in registers, four waves, one
        // phase, at most two pairs per thread and half
        const bool ok = resident && a.NW == 4 && a.phases == 1 && a.MT % 2 == 0 &&
                        (a.BT / 2) * a.U <= 2 * 256;
        if (!ok)
            return nullptr;
        const int np = ((a.BT / 2) * a.U + 255) / 256;
        if (a.fused)   // ... with the projection inside
            return rec_fused_shape_ok(a.BT, a.NT, a.U, a.I) ? get_fused(act_set(a), a.MT / 2, a.NT, a.KB, np)
                                                             : nullptr;
        return get_pipe(act_set(a), a.MT / 2, a.NT, a.KB, np);
    }
    const int nthr = 64 * a.NW;
    const int np = (a.BT * a.U + nthr - 1) / nthr;
    const int ta = a.phases == 2 ? a.NTA : 0;
    const int act = act_set(a);
    if (resident)
        return np <= 2 ? get_resident(act, a.NW, a.MT, a.NT, a.KB, ta) : nullptr;
    if (a.NW != 4)
        return nullptr;
    if (np <= 2)
        return get_streamed(act, 2, a.MT, a.NT, ta);
    if (np <= kMaxPairs)
        return get_streamed(act, 8, a.MT, a.NT, ta);
    return nullptr;
}

bool recurrence_supported(int nw, int mt, int nt, int nta, int phases, int kb, int bt, int u,
                          int resident, int halves)
{
    RecArgs a{};
    a.halves = halves;
    a.NW = nw;
    a.MT = mt;
    a.NT = nt;
    a.NTA = nta;
    a.phases = phases;
    a.KB = kb;
    a.BT = bt;
    a.U = u;
    return pick(a, resident) != nullptr;
}

bool recurrence_fused_supported(int bt, int nt, int u, int64_t I)
{
    return rec_fused_shape_ok(bt, nt, u, I);
}

static size_t rec_shmem(const RecArgs &a)
{
    if (a.exact)
        return rec_exact_lds_bytes(a.BT, a.NT, a.U);
    if (a.halves == 2 && a.fused)
        return rec_fused_lds_bytes(a.BT, a.NT, a.U, a.I);
    return a.halves == 2 ? rec_pipe_lds_bytes(a.BT, a.NT, a.U) : rec_lds_bytes(a.NW, a.BT, a.NT, a.U);
}

static int rec_threads(const RecArgs &a) { return a.exact ? kExactThreads : 64 * a.NW; }

int recurrence_can_persist(const RecArgs &a, int resident, int device, int *ok)
{
    *ok = 0;
    rec_fn f = pick(a, resident);
    if (!f)
        return (int)hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)rec_shmem(a));
    if (e != hipSuccess)
        return (int)e;
    int per_cu = 0, cus = 0, coop = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)f, rec_threads(a),
                                                     rec_shmem(a));
    if (e != hipSuccess)
        return (int)e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess)
        return (int)e;
    e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device);
    if (e != hipSuccess)
        return (int)e;
    const int n_wg = a.D * a.NBB * a.NUB;
    *ok = (coop && per_cu * cus >= n_wg) ? 1 : 0;
    return 0;
}

int launch_recurrence(const RecArgs &a, int resident, int persistent, void *stream)
{
    rec_fn f = pick(a, resident);
    if (!f)
        return (int)hipErrorInvalidValue;
    const size_t shmem = rec_shmem(a);
    hipError_t e = hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)shmem);
    if (e != hipSuccess)
        return (int)e;
    const int n_wg = a.D * a.NBB * a.NUB;
    if (persistent) {
        RecArgs arg = a;
        void *params[] = {&arg};
        e = hipLaunchCooperativeKernel((const void *)f, dim3(n_wg), dim3(rec_threads(a)), params,
                                       (unsigned)shmem, (hipStream_t)stream);
        return (int)e;
    }
    hipLaunchKernelGGL(f, dim3(n_wg), dim3(rec_threads(a)), shmem, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

}  // namespace rnnamd

