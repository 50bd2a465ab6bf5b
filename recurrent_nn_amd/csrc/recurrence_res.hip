// recurrence_res.hip -- recurrence kernels that keep the R slice in registers.
// (separate translation unit so that the instantiations compile in parallel)
#include "recurrence_kernel.h"

namespace rnnamd {

rec_fn rec_get_resident(int mt, int nt, int kb)
{
#define RNN_RES(MT_, NT_)                                                                         \
    if (mt == MT_ && nt == NT_) {                                                                \
        if (kb == 8)                                                                             \
            return rec_kernel<MT_, NT_, 8, 2>;                                                   \
        if (kb == 16)                                                                            \
            return rec_kernel<MT_, NT_, 16, 2>;                                                  \
    }
    RNN_RES(2, 1)
    RNN_RES(2, 2)
    RNN_RES(4, 1)
    RNN_RES(4, 2)
#undef RNN_RES
    return nullptr;
}

}  // namespace rnnamd
