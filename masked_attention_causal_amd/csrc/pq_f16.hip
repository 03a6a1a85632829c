// PQ-path task kernels for f16 I/O (see pq_impl.h).
#include "pq_impl.h"

namespace tfl {

hipError_t launch_pq_f16(int d, int dh, const PqArgs& a, hipStream_t s) {
    return pq_launch_mode<f16>(d, dh, a, s);
}

}  // namespace tfl
