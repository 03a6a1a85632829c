// PQ-path task kernels for f32 I/O (see pq_impl.h).
#include "pq_impl.h"

namespace tfl {

hipError_t launch_pq_f32(int d, int dh, const PqArgs& a, hipStream_t s) {
    return pq_launch_mode<float>(d, dh, a, s);
}

}  // namespace tfl
