// recurrence_res_a2.hip -- instantiations of the step-loop kernel (recurrence_kernel.h),
// one translation unit per activation set so that they compile in parallel.
#include "recurrence_kernel.h"

namespace rnnamd {

// R in registers.  nw waves split k: kb 16-k blocks per wave (8 or 16 with 4
// waves, 4 or 8 with 8 waves).  ta = 0: one phase over all NT tiles; ta > 0:
// GRU lbr=0, tiles [0, ta) then [ta, NT).
rec_fn rec_get_resident_a2(int nw, int mt, int nt, int kb, int ta)
{
#define RNN_RES(MT_, NT_, TA_)                                                                    \
    if (mt == MT_ && nt == NT_ && ta == TA_) {                                                   \
        if (nw == 4 && kb == 8)                                                                  \
            return rec_kernel<MT_, NT_, 8, 2, TA_, 2, 4>;                                       \
        if (nw == 4 && kb == 16)                                                                 \
            return rec_kernel<MT_, NT_, 16, 2, TA_, 2, 4>;                                      \
        if (nw == 8 && kb == 4)                                                                  \
            return rec_kernel<MT_, NT_, 4, 2, TA_, 2, 8>;                                       \
        if (nw == 8 && kb == 8)                                                                  \
            return rec_kernel<MT_, NT_, 8, 2, TA_, 2, 8>;                                       \
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
