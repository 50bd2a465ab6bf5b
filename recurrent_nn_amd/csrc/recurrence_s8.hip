// recurrence_s8.hip -- recurrence kernels that stream R every step, up to 8 pairs per thread.
// (separate translation unit so that the instantiations compile in parallel)
#include "recurrence_kernel.h"

namespace rnnamd {

rec_fn rec_get_streamed8(int mt, int nt)
{
#define RNN_STR(MT_)                                                                              \
    if (mt == MT_) {                                                                             \
        switch (nt) {                                                                            \
        case 1: return rec_kernel<MT_, 1, 0, 8>;                                                \
        case 2: return rec_kernel<MT_, 2, 0, 8>;                                                \
        case 4: return rec_kernel<MT_, 4, 0, 8>;                                                \
        case 6: return rec_kernel<MT_, 6, 0, 8>;                                                \
        default: return nullptr;                                                                 \
        }                                                                                        \
    }
    RNN_STR(1)
    RNN_STR(2)
    RNN_STR(4)
#undef RNN_STR
    return nullptr;
}

}  // namespace rnnamd
