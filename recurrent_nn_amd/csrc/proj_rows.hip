// proj_rows.hip -- the list of rows the input projection computes when
// sequence_lens is given (onemodel "Recurrent operators", sections
// "Computation", step 1, and "Choices the specification leaves open":
// a row's steps at or past its length are never read, so their projections
// are not computed).  Rows are ranked by decreasing length (rank r sits at
// position rank_pos[r]), so at step j the rows read are the ranks below the
// number of rows still active; the list holds them step by step as dense
// row numbers (j - j_base) * Bt + r, which the projection kernels
// (proj_gemm.hip) walk instead of every row.
#include <hip/hip_runtime.h>

#include "common.h"

namespace rnnamd {

// The rows the step loop reads in the chunk, step by step: step jl reads the
// ranks r < na(j) (na(j) = rows with length > j; lengths by rank do not
// increase), listed as jl * Bt + r.  One workgroup: the lengths by rank are
// staged in LDS (up to kRowsLds rows; more are read from memory), then 1024
// steps at a time: the counts by binary search, their exclusive scan, and the
// rows, each of the 16 waves writing one step's rows at a time.
constexpr int kRowsLds = 8192;
__global__ void __launch_bounds__(1024) proj_rows_kernel(ProjArgs a, int32_t *rowmap)
{
    __shared__ int32_t cnt[1024], off[1024], lrank[kRowsLds];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool staged = a.Bt <= kRowsLds;
    if (staged)
        for (int r = tid; r < a.Bt; r += 1024)
            lrank[r] = a.lens[a.rank_pos[r]];
    __syncthreads();
    int64_t base = 0;
    for (int64_t s0 = 0; s0 < a.steps; s0 += 1024) {
        const int64_t jl = s0 + tid;
        int32_t na = 0;
        if (jl < a.steps) {
            const int64_t j = a.j_base + jl;
            int lo = 0, hi = (int)a.Bt;                 // first rank whose length <= j
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                const int32_t len = staged ? lrank[mid] : a.lens[a.rank_pos[mid]];
                if (len > j)
                    lo = mid + 1;
                else
                    hi = mid;
            }
            na = lo;
        }
        cnt[tid] = na;
        off[tid] = na;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {            // inclusive scan of the counts
            const int32_t v = tid >= o ? off[tid - o] : 0;
            __syncthreads();
            off[tid] += v;
            __syncthreads();
        }
        const int nsteps = (int)(a.steps - s0 < 1024 ? a.steps - s0 : 1024);
        for (int k = w; k < nsteps; k += 16) {
            const int64_t o = base + off[k] - cnt[k];
            const int32_t first = (int32_t)((s0 + k) * a.Bt);
            for (int r = lane; r < cnt[k]; r += 64)
                rowmap[o + r] = first + r;
        }
        base += off[nsteps - 1];
        __syncthreads();                                 // before cnt and off are reused
    }
}

int launch_proj_rows(const ProjArgs &a, int32_t *rowmap, void *stream)
{
    if (a.steps <= 0 || a.Bt <= 0)
        return 0;
    hipLaunchKernelGGL(proj_rows_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, a, rowmap);
    return (int)hipGetLastError();
}

}  // namespace rnnamd
