// K2 + K3: the top-k Markov walk (vLLM PR #49969, Purpose). Placeholder until the kernels land.
#include "internal.hpp"

namespace dspark {

int launch_topk_walk(const TopkLaunch& a, hipStream_t stream) {
    (void)a;
    (void)stream;
    return DSPARK_ERR_UNSUPPORTED;
}

}  // namespace dspark
