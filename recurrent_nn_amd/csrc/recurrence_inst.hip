// recurrence_inst.hip -- the instantiation tables of the step-loop kernels
// (recurrence_kernel.h, recurrence_pipe.h, recurrence_fused.h).  This one
// source is compiled once per (kernel family RNN_FAMILY, activation set
// RNN_ACT), so that the tables build in parallel; the build passes both as
// -D definitions.
//
//   RNN_ACT: activation set compiled into the kernels -- 1 LSTM with
//            Sigmoid/Tanh/Tanh, 2 GRU with HardSigmoid/Tanh, 3 RNN with Tanh,
//            4 GRU with Sigmoid/Tanh, 0 any operator and set (run-time switch)
//   RNN_FAMILY: 0 R resident in registers, 1 R streamed with up to 2 (row,
//            unit) pairs per thread, 2 R streamed with up to 8 pairs, 3 two
//            half-batch sub-steps per step (R resident), 4 the same with the
//            input projection inside the step loop
#include "recurrence_fused.h"

#if !defined(RNN_ACT) || !defined(RNN_FAMILY)
#error "compile with -DRNN_ACT=<0..4> -DRNN_FAMILY=<0..4>"
#endif

#define RNN_CAT2(a, b) a##b
#define RNN_CAT(a, b) RNN_CAT2(a, b)

namespace rnnamd {

#if RNN_FAMILY == 0
// R in registers.  nw waves split k: kb 16-k blocks per wave (8 or 16 with 4
// waves, 4 or 8 with 8 waves).  ta = 0: one phase over all NT tiles; ta > 0:
// GRU lbr=0, tiles [0, ta) then [ta, NT).
rec_fn RNN_CAT(rec_get_resident_a, RNN_ACT)(int nw, int mt, int nt, int kb, int ta)
{
#define RNN_RES(MT_, NT_, TA_)                                                                    \
    if (mt == MT_ && nt == NT_ && ta == TA_) {                                                   \
        if (nw == 4 && kb == 8)                                                                  \
            return rec_kernel<MT_, NT_, 8, 2, TA_, RNN_ACT, 4>;                                  \
        if (nw == 4 && kb == 16)                                                                 \
            return rec_kernel<MT_, NT_, 16, 2, TA_, RNN_ACT, 4>;                                 \
        if (nw == 8 && kb == 4)                                                                  \
            return rec_kernel<MT_, NT_, 4, 2, TA_, RNN_ACT, 8>;                                  \
        if (nw == 8 && kb == 8)                                                                  \
            return rec_kernel<MT_, NT_, 8, 2, TA_, RNN_ACT, 8>;                                  \
    }
    RNN_RES(2, 1, 0)
    RNN_RES(2, 2, 0)
    RNN_RES(2, 2, 1)
    RNN_RES(4, 1, 0)
    RNN_RES(4, 2, 0)
#undef RNN_RES
    return nullptr;
}

#elif RNN_FAMILY == 1 || RNN_FAMILY == 2
// R streamed every step (4 waves), up to P_ (row, unit) pairs per thread;
// mt 16-row tiles (a batch tile of 16 to 128 rows); ta as for the resident
// family.
#if RNN_FAMILY == 1
#define P_ 2
#define RNN_NAME rec_get_streamed2_a
#else
#define P_ 8
#define RNN_NAME rec_get_streamed8_a
#endif
rec_fn RNN_CAT(RNN_NAME, RNN_ACT)(int mt, int nt, int ta)
{
#define RNN_STR(MT_)                                                                              \
    if (mt == MT_) {                                                                             \
        if (ta == 0) {                                                                           \
            switch (nt) {                                                                        \
            case 1: return rec_kernel<MT_, 1, 0, P_, 0, RNN_ACT, 4>;                             \
            case 2: return rec_kernel<MT_, 2, 0, P_, 0, RNN_ACT, 4>;                             \
            case 3: return rec_kernel<MT_, 3, 0, P_, 0, RNN_ACT, 4>;                             \
            case 4: return rec_kernel<MT_, 4, 0, P_, 0, RNN_ACT, 4>;                             \
            case 6: return rec_kernel<MT_, 6, 0, P_, 0, RNN_ACT, 4>;                             \
            default: return nullptr;                                                             \
            }                                                                                    \
        }                                                                                        \
        if (nt == 2 && ta == 1) return rec_kernel<MT_, 2, 0, P_, 1, RNN_ACT, 4>;                 \
        if (nt == 3 && ta == 2) return rec_kernel<MT_, 3, 0, P_, 2, RNN_ACT, 4>;                 \
        if (nt == 6 && ta == 4) return rec_kernel<MT_, 6, 0, P_, 4, RNN_ACT, 4>;                 \
        return nullptr;                                                                          \
    }
    RNN_STR(1)
    RNN_STR(2)
    RNN_STR(4)
#undef RNN_STR
    // 128-row tiles: at most 3 column tiles (wider ones spill registers)
    if (mt == 8) {
        if (ta == 0) {
            switch (nt) {
            case 1: return rec_kernel<8, 1, 0, P_, 0, RNN_ACT, 4>;
            case 2: return rec_kernel<8, 2, 0, P_, 0, RNN_ACT, 4>;
            case 3: return rec_kernel<8, 3, 0, P_, 0, RNN_ACT, 4>;
            default: return nullptr;
            }
        }
        if (nt == 2 && ta == 1) return rec_kernel<8, 2, 0, P_, 1, RNN_ACT, 4>;
        if (nt == 3 && ta == 2) return rec_kernel<8, 3, 0, P_, 2, RNN_ACT, 4>;
        return nullptr;
    }
    return nullptr;
}
#undef P_
#undef RNN_NAME

#elif RNN_FAMILY == 3 || RNN_FAMILY == 4
// Two half-batch sub-steps: mth 16-row tiles per half (BT = 32 * mth), nt
// 16-column tiles, kb 16-k blocks per wave (R slice of nt * kb * 4 registers
// per lane), p pairs per thread and half: 1 (R resident allows at most two
// pairs per thread over the whole tile, so one per half).
#if RNN_FAMILY == 3
#define RNN_KERNEL rec_pipe_kernel
#define RNN_NAME rec_get_pipe_a
#else
#define RNN_KERNEL rec_fused_kernel
#define RNN_NAME rec_get_fused_a
#endif
rec_fn RNN_CAT(RNN_NAME, RNN_ACT)(int mth, int nt, int kb, int p)
{
#define RNN_P2(MTH_, NT_, KB_)                                                                    \
    if (mth == MTH_ && nt == NT_ && kb == KB_ && p == 1)                                         \
        return RNN_KERNEL<MTH_, NT_, KB_, RNN_ACT, 1>;
    RNN_P2(1, 1, 8)
    RNN_P2(1, 1, 16)
    RNN_P2(1, 2, 8)
    RNN_P2(1, 2, 16)
    RNN_P2(2, 1, 8)
    RNN_P2(2, 1, 16)
    RNN_P2(2, 2, 8)
    RNN_P2(2, 2, 16)
#undef RNN_P2
    return nullptr;
}
#undef RNN_KERNEL
#undef RNN_NAME
#endif

}  // namespace rnnamd
