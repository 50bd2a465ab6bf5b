// recurrence.hip -- selection and launch of the step-loop kernels
// (recurrence_kernel.h): the compiled shapes, the occupancy check of the
// persistent (cooperative) form, and the launches.
#include <hip/hip_runtime.h>

#include "recurrence_kernel.h"

namespace rnnamd {

rec_fn rec_get_resident(int mt, int nt, int kb);
rec_fn rec_get_streamed2(int mt, int nt);
rec_fn rec_get_streamed8(int mt, int nt);

static rec_fn pick(const RecArgs &a, int resident)
{
    const int np = (a.BT * a.U + kThreads - 1) / kThreads;
    if (resident)
        return np <= 2 ? rec_get_resident(a.MT, a.NT, a.KB) : nullptr;
    if (np <= 2)
        return rec_get_streamed2(a.MT, a.NT);
    if (np <= kMaxPairs)
        return rec_get_streamed8(a.MT, a.NT);
    return nullptr;
}

bool recurrence_supported(int mt, int nt, int kb, int bt, int u, int resident)
{
    RecArgs a{};
    a.MT = mt;
    a.NT = nt;
    a.KB = kb;
    a.BT = bt;
    a.U = u;
    return pick(a, resident) != nullptr;
}

static size_t rec_shmem(const RecArgs &a) { return rec_lds_bytes(a.BT, a.NT, a.U); }

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
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)f, kThreads,
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
        e = hipLaunchCooperativeKernel((const void *)f, dim3(n_wg), dim3(kThreads), params,
                                       (unsigned)shmem, (hipStream_t)stream);
        return (int)e;
    }
    hipLaunchKernelGGL(f, dim3(n_wg), dim3(kThreads), shmem, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

}  // namespace rnnamd
