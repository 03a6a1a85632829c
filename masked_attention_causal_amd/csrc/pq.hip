// Dispatch of the PQ path (task list of 64-row tiles) by I/O dtype, and its shape set.
#include "kernels.h"

namespace tfl {

hipError_t launch_pq_f32(int d, int dh, const PqArgs& a, hipStream_t s);
hipError_t launch_pq_f16(int d, int dh, const PqArgs& a, hipStream_t s);
hipError_t launch_pq_bf16(int d, int dh, const PqArgs& a, hipStream_t s);

bool pq_supported(Mode m, int d, int dh, int f, int n_layers) {
    (void)m;
    if (d != 64 && d != 128 && d != 256) return false;
    if (dh != 32 && dh != 64) return false;
    return f % 128 == 0 && f >= 128 && n_layers >= 1 && n_layers <= SEQ_MAX_LAYERS;
}

hipError_t launch_pq(Mode m, int d, int dh, const PqArgs& a, hipStream_t s) {
    switch (m) {
        case MODE_F32: return launch_pq_f32(d, dh, a, s);
        case MODE_F16: return launch_pq_f16(d, dh, a, s);
        case MODE_BF16: return launch_pq_bf16(d, dh, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tfl
