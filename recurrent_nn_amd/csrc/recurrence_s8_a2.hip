// recurrence_s8_a2.hip -- instantiations of the step-loop kernel (recurrence_kernel.h),
// one translation unit per activation set so that they compile in parallel.
#include "recurrence_kernel.h"

namespace rnnamd {

// R streamed every step (4 waves), up to 8 (row, unit) pairs per thread.
rec_fn rec_get_streamed8_a2(int mt, int nt, int ta)
{
#define RNN_STR(MT_)                                                                              \
    if (mt == MT_) {                                                                             \
        if (ta == 0) {                                                                           \
            switch (nt) {                                                                        \
            case 1: return rec_kernel<MT_, 1, 0, 8, 0, 2, 4>;                                 \
            case 2: return rec_kernel<MT_, 2, 0, 8, 0, 2, 4>;                                 \
            case 4: return rec_kernel<MT_, 4, 0, 8, 0, 2, 4>;                                 \
            case 6: return rec_kernel<MT_, 6, 0, 8, 0, 2, 4>;                                 \
            default: return nullptr;                                                             \
            }                                                                                    \
        }                                                                                        \
        if (nt == 2 && ta == 1) return rec_kernel<MT_, 2, 0, 8, 1, 2, 4>;                     \
        if (nt == 3 && ta == 2) return rec_kernel<MT_, 3, 0, 8, 2, 2, 4>;                     \
        if (nt == 6 && ta == 4) return rec_kernel<MT_, 6, 0, 8, 4, 2, 4>;                     \
        return nullptr;                                                                          \
    }
    RNN_STR(1)
    RNN_STR(2)
    RNN_STR(4)
#undef RNN_STR
    return nullptr;
}

}  // namespace rnnamd
