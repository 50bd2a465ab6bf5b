// proj_gemm.hip -- the input projection XW = X . W^T over all time steps
// (onemodel "Recurrent operators", section "Computation", step 1: one matrix
// product of shape [seq*batch, G*H] per direction).  W arrives packed (rows
// in block-column order, see pack.hip), so XW comes out in the order the
// recurrence reads it.
//
// Rows.  Position i holds batch row order[i]; XW is stored by STEP: row
// (j - j_base, i) of direction d holds the projection of the X row that step
// j of the row at position i reads -- time j forward, len_b - 1 - j in
// reverse ("Choices the specification leaves open": sequence_lens and
// reverse traversal) -- for the steps of one time chunk.  Dense row
// m = (j - j_base) * Bt + r is step j of the row of rank r (decreasing
// length; rank r sits at position rank_pos[r]), stored at the row's
// position.  With sequence_lens the product computes only the rows the step
// loop reads (j < len_b): at step j those are the ranks below the number of
// rows still active, and rowmap lists them step by step (built on the device
// per chunk), so the rows computed are one dense list with no holes.  Both
// directions are one launch (the direction is part of the tile index).
//
// Tiling: 128x128 output tile per 256-thread workgroup, 4 waves of 64x64, K
// staged through LDS in 128-byte row slices (32 fp32 or 64 bf16 values): the
// next slice is loaded into registers while the current one is consumed and
// replaces it between two barriers, so one LDS buffer (40 KiB) suffices and
// three workgroups share a CU (measured faster than two double-buffered).  fp32 uses v_mfma_f32_16x16x4_f32, bf16 uses the gfx950
// v_mfma_f32_16x16x32_bf16; for bf16, the chunk's X rows are first gathered
// and rounded to bfloat16 (nearest even) once by gather_bf16_kernel.  Accumulation is in the
// matrix cores' order with a fixed tiling (deterministic, "fast mode").
//
// Each lane feeds the matrix core 16 contiguous bytes of one row per 16x16
// tile and k block: lane (r = l % 16, q = l / 16) supplies k = 4q..4q+3 (fp32)
// or 8q..8q+7 (bf16) of the block; for fp32 the four components go to four
// consecutive MFMAs, i.e. the k order inside a block is permuted, which only
// changes the (already unspecified) summation order.
#include <hip/hip_runtime.h>

#include "common.h"

namespace rnnamd {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 128;              // bytes of k per row per stage
constexpr int LDSROW = ROWB + 32;      // padded LDS row stride (bytes): no bank conflicts
constexpr int TILEB = BM * LDSROW;     // bytes of one operand tile in LDS

__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (u >> 16) | 0x0040u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// 4 fp32 values of row `row` at k .. k+3, zero for row < 0 or row >= rows
// and outside [0, K).
__device__ __forceinline__ f4 load4(const float *__restrict__ p, int64_t row, int64_t k,
                                    int64_t rows, int64_t K, bool vec_ok)
{
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < 0 || row >= rows)
        return v;
    const float *q = p + row * K + k;
    if (vec_ok && k + 3 < K)
        return *(const f4 *)q;
    if (k + 0 < K) v[0] = q[0];
    if (k + 1 < K) v[1] = q[1];
    if (k + 2 < K) v[2] = q[2];
    if (k + 3 < K) v[3] = q[3];
    return v;
}

// 8 bf16 values (16 bytes) of row `row` at k .. k+7 of a bf16 matrix.
__device__ __forceinline__ u4 load8h(const uint16_t *__restrict__ p, int64_t row, int64_t k,
                                     int64_t rows, int64_t K, bool vec_ok)
{
    u4 v = {0u, 0u, 0u, 0u};
    if (row >= rows)
        return v;
    const uint16_t *q = p + row * K + k;
    if (vec_ok && k + 7 < K)
        return *(const u4 *)q;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        h[e] = (k + e < K) ? q[e] : 0u;
    v[0] = h[0] | (h[1] << 16);
    v[1] = h[2] | (h[3] << 16);
    v[2] = h[4] | (h[5] << 16);
    v[3] = h[6] | (h[7] << 16);
    return v;
}

// Buffer resource over `bytes` bytes at p (raw, 32-bit offsets; a load at
// an offset at or past `bytes` returns zeros).  Word 3 is the gfx9 default
// (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// Offset that no buffer here reaches (buffers of the fast path are smaller
// than 2 GiB, and a stage adds at most K * 4 < 2 GiB bytes).
constexpr uint32_t kOffNone = 0x80000000u;

__device__ __forceinline__ u4 pack8(f4 a, f4 b)
{
    u4 v;
    v[0] = bf16_bits(a[0]) | (bf16_bits(a[1]) << 16);
    v[1] = bf16_bits(a[2]) | (bf16_bits(a[3]) << 16);
    v[2] = bf16_bits(b[0]) | (bf16_bits(b[1]) << 16);
    v[3] = bf16_bits(b[2]) | (bf16_bits(b[3]) << 16);
    return v;
}

// Logical row m = (j - j_base) * Bt + r of the product is step j of the row
// of rank r.  Its XW row (step j - j_base, the row's position):
__device__ __forceinline__ int64_t proj_outrow(const ProjArgs &a, int64_t m)
{
    const uint32_t jl = (uint32_t)m / (uint32_t)a.Bt, r = (uint32_t)m - jl * (uint32_t)a.Bt;
    return (int64_t)jl * a.Bt + (a.rank_pos ? a.rank_pos[r] : r);
}

// The X row that logical row m of direction d reads; -1 when the step loop
// never reads it (j >= len) or m is past the chunk.
__device__ __forceinline__ int64_t proj_xrow(const ProjArgs &a, int64_t d, int64_t m)
{
    if (m >= a.steps * a.Bt)
        return -1;
    const uint32_t jl = (uint32_t)m / (uint32_t)a.Bt, r = (uint32_t)m - jl * (uint32_t)a.Bt;
    const int64_t i = a.rank_pos ? a.rank_pos[r] : r;   // position of rank r
    const int64_t b = a.order ? a.order[i] : i;          // position i holds batch row b
    const int64_t j = a.j_base + jl, len = a.lens[i];
    if (j >= len)
        return -1;
    const int64_t t = (a.reverse_only || d == 1) ? len - 1 - j : j;
    return a.layout == 0 ? t * a.Bt + b : b * a.S + t;
}

// Dense row of computed row mc.
__device__ __forceinline__ int64_t proj_dense(const ProjArgs &a, int64_t mc)
{
    return a.rowmap ? (int64_t)a.rowmap[mc] : mc;
}

// bf16 projection: the chunk's computed X rows in order, rounded to
// bfloat16 (nearest even) once, zeros for rows never read; the product then
// reads bf16 rows directly instead of converting in every N tile.
__global__ void gather_bf16_kernel(ProjArgs a)
{
    const int64_t Mc = a.m_rows;
    const float *X = (const float *)a.X;
    const bool vec = a.K % 8 == 0;
    for (int64_t row = blockIdx.x; row < a.D * Mc; row += gridDim.x) {
        const int64_t d = row / Mc, m = row - d * Mc;
        const int64_t xr = proj_xrow(a, d, proj_dense(a, m));
        uint16_t *dst = a.Xb + row * a.K;
        const float *src = xr >= 0 ? X + xr * a.K : nullptr;
        if (vec) {
            for (int64_t k = threadIdx.x * 8; k < a.K; k += blockDim.x * 8) {
                f4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
                if (src) {
                    x0 = *(const f4 *)(src + k);
                    x1 = *(const f4 *)(src + k + 4);
                }
                *(u4 *)(dst + k) = pack8(x0, x1);
            }
        } else {
            for (int64_t k = threadIdx.x; k < a.K; k += blockDim.x)
                dst[k] = src ? (uint16_t)bf16_bits(src[k]) : (uint16_t)0;
        }
    }
}

// Tile order: workgroups on one XCD (blockIdx % 8) take a contiguous range
// of tiles, walked in bands of GM tile-rows so that neighbours share panels.
__device__ __forceinline__ void tile_of(int64_t wg, int64_t nwg, int64_t tiles_m, int64_t tiles_n,
                                        int64_t *tm, int64_t *tn)
{
    int64_t t = wg;
    if (nwg % 8 == 0)
        t = (wg % 8) * (nwg / 8) + wg / 8;
    constexpr int64_t GM = 8;
    const int64_t band = GM * tiles_n;
    const int64_t g = t / band;
    const int64_t first = g * GM;
    const int64_t gm = (tiles_m - first) < GM ? (tiles_m - first) : GM;
    const int64_t r = t - g * band;
    *tm = first + r % gm;
    *tn = r / gm;
}

template <bool BF16>
__global__ void __launch_bounds__(256, 3) proj_gemm_kernel(ProjArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];   // [A,B][TILEB]
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int wm = w >> 1, wn = w & 1;

    const int64_t Md = a.steps * a.Bt;                 // XW rows per direction
    const int64_t Mc = a.m_rows;                       // rows computed per direction
    const int64_t tiles_m = (Mc + BM - 1) / BM, tiles_n = (a.GH + BN - 1) / BN;
    int64_t tmg, tn;
    tile_of(blockIdx.x, gridDim.x, a.D * tiles_m, tiles_n, &tmg, &tn);
    const int64_t d = tmg / tiles_m, tm = tmg - d * tiles_m;
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t xrows = a.S * a.Bt;

    // k values per stage: 32 (fp32) or 64 (bf16)
    constexpr int KS = BF16 ? 64 : 32;
    const int64_t nk = (a.K + KS - 1) / KS;
    const bool a_vec = BF16 ? (a.K % 4 == 0) : (a.K % 4 == 0);
    const bool b_vec = BF16 ? (a.K % 8 == 0) : (a.K % 4 == 0);
    // Stages whose k range lies inside K are loaded with buffer loads from
    // row offsets computed once (rows that do not exist read as zeros); the
    // partial last stage, and operands of 2 GiB or more, take the checked
    // loads.
    constexpr int ESZ = BF16 ? 2 : 4;
    const int64_t a_bytes = BF16 ? a.D * Mc * a.K * 2 : a.S * a.Bt * a.K * 4;
    const int64_t b_bytes = a.GH * a.K * ESZ;
    const bool fast = (BF16 ? a.K % 8 == 0 : a.K % 4 == 0) && a_bytes < (int64_t)kOffNone &&
                      b_bytes < (int64_t)kOffNone;
    const int64_t nk_fast = fast ? a.K / KS : 0;

    // staging: thread -> (row = tid / 8 + 32 i, chunk = tid % 8 of 16 bytes)
    const int srow = tid >> 3, sch = tid & 7;
    int64_t xr[4];
    int any = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + srow + 32 * i;
        xr[i] = m < Mc ? proj_xrow(a, d, proj_dense(a, m)) : -1;
        any |= xr[i] >= 0;
    }
    if (!__syncthreads_or(any))
        return;                                      // no row of this tile is ever read
    const char *Wd = (const char *)a.Wp + (size_t)d * a.GH * a.K * (BF16 ? 2 : 4);
    __amdgpu_buffer_rsrc_t rsa = buffer_of(BF16 ? (const void *)a.Xb : a.X, (uint32_t)(fast ? a_bytes : 0));
    __amdgpu_buffer_rsrc_t rsb = buffer_of(Wd, (uint32_t)(fast ? b_bytes : 0));
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = srow + 32 * i;
        const int64_t ar = BF16 ? (m0 + row < Mc ? d * Mc + m0 + row : -1) : xr[i];
        aoff[i] = ar >= 0 ? (uint32_t)(ar * a.K * ESZ) + sch * 16 : kOffNone;
        boff[i] = n0 + row < a.GH ? (uint32_t)((n0 + row) * a.K * ESZ) + sch * 16 : kOffNone;
    }
    u4 ra[4], rb[4];
    auto gload_fast = [&](uint32_t kt, u4 (&ra)[4], u4 (&rb)[4]) {
        const uint32_t kb = kt * (KS * ESZ);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rsa, aoff[i] + kb, 0, 0));
            rb[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rsb, boff[i] + kb, 0, 0));
        }
    };
    auto gload = [&](int64_t kt, u4 (&ra)[4], u4 (&rb)[4]) {
        const int64_t kbase = kt * KS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = srow + 32 * i;
            if constexpr (BF16) {
                const int64_t k = kbase + sch * 8;
                ra[i] = load8h(a.Xb + (size_t)d * Mc * a.K, m0 + row, k, Mc, a.K, b_vec);
                rb[i] = load8h((const uint16_t *)Wd, n0 + row, k, a.GH, a.K, b_vec);
            } else {
                const int64_t k = kbase + sch * 4;
                f4 x = load4((const float *)a.X, xr[i], k, xrows, a.K, a_vec);
                f4 y = load4((const float *)Wd, n0 + row, k, a.GH, a.K, b_vec);
                ra[i] = __builtin_bit_cast(u4, x);
                rb[i] = __builtin_bit_cast(u4, y);
            }
        }
    };
    auto sstore = [&](int buf, const u4 (&ra)[4], const u4 (&rb)[4]) {
        unsigned char *A = lds + buf * 2 * TILEB;
        unsigned char *B = A + TILEB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = srow + 32 * i;
            *(u4 *)(A + row * LDSROW + sch * 16) = ra[i];
            *(u4 *)(B + row * LDSROW + sch * 16) = rb[i];
        }
    };

    f4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    auto stage = [&](int buf) {
        const unsigned char *A = lds + buf * 2 * TILEB;
        const unsigned char *B = A + TILEB;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {            // two 64-byte k blocks per stage
            u4 av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = *(const u4 *)(A + (wm * 64 + i * 16 + lr) * LDSROW + kb * 64 + lq * 16);
                bv[i] = *(const u4 *)(B + (wn * 64 + i * 16 + lr) * LDSROW + kb * 64 + lq * 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (BF16) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf8, av[i]), __builtin_bit_cast(bf8, bv[j]),
                            acc[i][j], 0, 0, 0);
                    } else {
                        const f4 x = __builtin_bit_cast(f4, av[i]);
                        const f4 y = __builtin_bit_cast(f4, bv[j]);
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], y[s], acc[i][j],
                                                                             0, 0, 0);
                    }
                }
        }
    };
    // one LDS buffer: the next stage waits in registers while this one is
    // consumed, then replaces it between two barriers
    // (whole stages first, then the checked ones)
    const int nkf = (int)nk_fast;
    if (nkf > 0)
        gload_fast(0, ra, rb);
    else
        gload(0, ra, rb);
    sstore(0, ra, rb);
    __syncthreads();
    for (int kt = 0; kt + 1 < nkf; ++kt) {
        gload_fast(kt + 1, ra, rb);
        // left to itself the scheduler sinks these loads to just before
        // their LDS stores, exposing their whole latency
        __builtin_amdgcn_sched_barrier(0);
        stage(0);
        __syncthreads();
        sstore(0, ra, rb);
        __syncthreads();
    }
    for (int64_t kt = nkf > 0 ? nkf - 1 : 0; kt < nk; ++kt) {
        if (kt + 1 < nk)
            gload(kt + 1, ra, rb);
        stage(0);
        __syncthreads();
        if (kt + 1 < nk) {
            sstore(0, ra, rb);
            __syncthreads();
        }
    }

    // store: lane holds rows 4*lq + r, column lr of each 16x16 tile;
    // logical row m goes to XW's row for its step and position
    float *XWd = a.XW + (size_t)d * Md * a.GH;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + wm * 64 + i * 16 + lq * 4 + r;
            if (m >= Mc)
                continue;
            const size_t ro = (size_t)proj_outrow(a, proj_dense(a, m)) * a.GH;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + wn * 64 + j * 16 + lr;
                if (n < a.GH)
                    XWd[ro + n] = acc[i][j][r];
            }
        }
}

// Exact mode (onemodel "Recurrent operators", section "Exact mode"): each
// XW value is one accumulator that starts at +0 and adds the binary32
// products X[m][k] * W[n][k] for k = 0, 1, ..., K-1 in order, every multiply
// and add rounded on its own (for bf16 the operands are the rounded bf16
// values, whose products are exact in binary32).  VALU only; the value does
// not depend on the tiling.  64x64 tile per 256-thread workgroup, each
// thread 4x4 outputs (rows 4 ty .. 4 ty + 3, columns 4 tx .. 4 tx + 3, so
// that a k step reads each operand with one 16-byte LDS load); k staged
// through LDS in chunks of 32, k-major, the next chunk loaded into registers
// while the current one is consumed.  Same rows, tile skip and XW order as
// the fast form.
template <bool BF16>
__global__ void __launch_bounds__(256) proj_exact_kernel(ProjArgs a)
{
    constexpr int TM = 64, TN = 64, KC = 32, LDT = TM + 4;
    __shared__ __attribute__((aligned(16))) float As[KC][LDT], Bs[KC][LDT];
    __shared__ int64_t xrow_s[TM];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t Md = a.steps * a.Bt;                 // XW rows per direction
    const int64_t Mc = a.m_rows;                       // rows computed per direction
    const int64_t tiles_m = (Mc + TM - 1) / TM, tiles_n = (a.GH + TN - 1) / TN;
    const int64_t tmg = blockIdx.x / tiles_n, tn = blockIdx.x - tmg * tiles_n;
    const int64_t d = tmg / tiles_m, tm = tmg - d * tiles_m;
    const int64_t m0 = tm * TM, n0 = tn * TN;
    int any = 0;
    if (tid < TM) {
        xrow_s[tid] = m0 + tid < Mc ? proj_xrow(a, d, proj_dense(a, m0 + tid)) : -1;
        any = xrow_s[tid] >= 0;
    }
    if (!__syncthreads_or(any))
        return;                                      // no row of this tile is ever read
    const float *X = (const float *)a.X;
    const uint16_t *Xb = BF16 ? a.Xb + (size_t)d * Mc * a.K : nullptr;
    const char *Wd = (const char *)a.Wp + (size_t)d * a.GH * a.K * (BF16 ? 2 : 4);
    auto bf = [](uint32_t h) { return __uint_as_float(h << 16); };

    // staging: thread -> (row r = tid / 8 + 32 i, 4 k at 4 (tid % 8)), i < 2
    const int sr = tid >> 3, sk = (tid & 7) * 4;
    auto row_a = [&](int r) -> int64_t {        // source row of A, or -1
        if (BF16)
            return m0 + r < Mc ? m0 + r : -1;
        return xrow_s[r];
    };
    auto row_b = [&](int r) -> int64_t { return n0 + r < a.GH ? n0 + r : -1; };
    // four consecutive k of a row (zeros past K or for a missing row)
    auto load4k = [&](bool is_b, int64_t row, int64_t k) -> f4 {
        f4 v = {0.f, 0.f, 0.f, 0.f};
        if (row < 0)
            return v;
        if (BF16) {
            const uint16_t *src = is_b ? (const uint16_t *)Wd : Xb;
            const uint16_t *q = src + (size_t)row * a.K + k;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < a.K)
                    v[e] = bf(q[e]);
        } else {
            const float *src = is_b ? (const float *)Wd : X;
            const float *q = src + (size_t)row * a.K + k;
            if (a.K % 4 == 0 && k + 3 < a.K)
                return *(const f4 *)q;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < a.K)
                    v[e] = q[e];
        }
        return v;
    };
    int64_t ra_[2], rb_[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        ra_[i] = row_a(sr + 32 * i);
        rb_[i] = row_b(sr + 32 * i);
    }
    f4 ga[2], gb[2];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            ga[i] = load4k(false, ra_[i], k0 + sk);
            gb[i] = load4k(true, rb_[i], k0 + sk);
        }
    };
    // k-major tiles with the row index XOR-swizzled by 4 x ((k / 4) mod 8):
    // the staging stores (eight k groups of a row per eight lanes) spread
    // over all banks, and each thread's four consecutive rows stay one
    // aligned 16-byte word for the reads
    auto sw = [](int k) { return 4 * ((k >> 2) & 7); };
    auto sstore = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                As[sk + e][(sr + 32 * i) ^ sw(sk + e)] = ga[i][e];
                Bs[sk + e][(sr + 32 * i) ^ sw(sk + e)] = gb[i][e];
            }
    };

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = 0.0f;
    gload(0);
    for (int64_t k0 = 0; k0 < a.K; k0 += KC) {
        const int kn = (int)(a.K - k0 < KC ? a.K - k0 : KC);
        __syncthreads();                         // the previous chunk is consumed
        sstore();
        __syncthreads();
        if (k0 + KC < a.K)
            gload(k0 + KC);
        for (int kk = 0; kk < kn; ++kk) {
            const f4 av = *(const f4 *)&As[kk][(4 * ty) ^ sw(kk)];
            const f4 bv = *(const f4 *)&Bs[kk][(4 * tx) ^ sw(kk)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __fadd_rn(acc[i][j], __fmul_rn(av[i], bv[j]));
        }
    }
    float *XWd = a.XW + (size_t)d * Md * a.GH;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * ty + i;
        if (m >= Mc)
            continue;
        const size_t ro = (size_t)proj_outrow(a, proj_dense(a, m)) * a.GH;   // step, position
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + 4 * tx + j;
            if (n < a.GH)
                XWd[ro + n] = acc[i][j];
        }
    }
}

int launch_projection(const ProjArgs &a, void *stream)
{
    if (a.steps <= 0 || a.Bt <= 0 || a.GH <= 0 || a.m_rows <= 0)
        return 0;
    if (a.exact) {
        if (a.bf16) {
            int64_t blocks = a.D * a.m_rows;
            if (blocks > 65536)
                blocks = 65536;
            hipLaunchKernelGGL(gather_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0,
                               (hipStream_t)stream, a);
        }
        const int64_t et = a.D * ((a.m_rows + 63) / 64) * ((a.GH + 63) / 64);
        if (a.bf16)
            hipLaunchKernelGGL(proj_exact_kernel<true>, dim3((unsigned)et), dim3(256), 0,
                               (hipStream_t)stream, a);
        else
            hipLaunchKernelGGL(proj_exact_kernel<false>, dim3((unsigned)et), dim3(256), 0,
                               (hipStream_t)stream, a);
        return (int)hipGetLastError();
    }
    const int64_t tiles = a.D * ((a.m_rows + BM - 1) / BM) * ((a.GH + BN - 1) / BN);
    const size_t shmem = 2 * TILEB;               // one buffer of A and B
    const void *fn = a.bf16 ? (const void *)proj_gemm_kernel<true> : (const void *)proj_gemm_kernel<false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess)
        return (int)e;
    if (a.bf16) {
        int64_t blocks = a.D * a.m_rows;
        if (blocks > 65536)
            blocks = 65536;
        hipLaunchKernelGGL(gather_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, a);
        hipLaunchKernelGGL(proj_gemm_kernel<true>, dim3((unsigned)tiles), dim3(256), shmem,
                           (hipStream_t)stream, a);
    }
    else
        hipLaunchKernelGGL(proj_gemm_kernel<false>, dim3((unsigned)tiles), dim3(256), shmem,
                           (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

}  // namespace rnnamd
