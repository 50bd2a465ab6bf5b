// recurrence_p2_a2.hip -- instantiations of the step loop with two half-batch
// sub-steps per step (recurrence_pipe.h), one translation unit per activation
// set so that they compile in parallel.
#include "recurrence_pipe.h"

namespace rnnamd {

// mth 16-row tiles per half (BT = 32 * mth), nt 16-column tiles, kb 16-k
// blocks per wave (R slice of nt * kb * 4 registers per lane), p pairs per
// thread and half (1 or 2).
rec_fn rec_get_pipe_a2(int mth, int nt, int kb, int p)
{
#define RNN_P2(MTH_, NT_, KB_)                                                                    \
    if (mth == MTH_ && nt == NT_ && kb == KB_)                                                   \
        return p == 1 ? rec_pipe_kernel<MTH_, NT_, KB_, 2, 1> : rec_pipe_kernel<MTH_, NT_, KB_, 2, 2>;
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

}  // namespace rnnamd
