// recurrence_res_a0.hip -- instantiations of the step-loop kernel (recurrence_kernel.h),
// one translation unit per activation set so that they compile in parallel.
#include "recurrence_kernel.h"

namespace rnnamd {

// R in registers; ta = 0: one phase over all NT tiles, ta > 0: GRU lbr=0
// (tiles [0, ta) then [ta, NT)).
rec_fn rec_get_resident_a0(int mt, int nt, int kb, int ta)
{
#define RNN_RES(MT_, NT_, TA_)                                                                    \
    if (mt == MT_ && nt == NT_ && ta == TA_) {                                                   \
        if (kb == 8)                                                                             \
            return rec_kernel<MT_, NT_, 8, 2, TA_, 0>;                                          \
        if (kb == 16)                                                                            \
            return rec_kernel<MT_, NT_, 16, 2, TA_, 0>;                                         \
    }
    RNN_RES(2, 1, 0)
    RNN_RES(2, 2, 0)
    RNN_RES(2, 2, 1)
    RNN_RES(4, 1, 0)
    RNN_RES(4, 2, 0)
#undef RNN_RES
    return nullptr;
}

}  // namespace rnnamd
