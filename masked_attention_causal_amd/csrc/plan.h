// Frozen per-shape plans: the dispatcher's choice of path, the workspace
// layout and the launch sequence.  Host-only; no device call is made while
// a plan is built.
#pragma once
#include <string>

#include "kernels.h"
#include "tfl.h"

namespace tfl {

struct Plan {
    int path;       // tfl_path actually used
    int seq_kind;   // SEQ path: 0 MFMA kernel (two sequences per workgroup), 1 small-shape kernel
    bool row_fused; // TILED path: one fused row kernel per layer after attention
    char name[64];
    Mode mode;
    int n_layers, d, H, dh, f, B, L, Lp;
    long T;         // B * L token rows
    float eps;
    size_t op;      // operand element size (4 in F32 mode, 2 otherwise)
    // workspace offsets in bytes (TILED); off_W: fp16 weight planes of the
    // GEMMs (BF16 and F32 modes), n_wconv layers of them
    size_t off_Xr, off_X1, off_Z, off_A, off_Q, off_K, off_Vt, off_O, off_G, off_W, off_S;
    int n_wconv;
    // PQ path: key tiles per split, (tile, split) pairs per (sequence, head),
    // tasks, and workspace offsets
    int pq_ks, pq_ctot, pq_tasks, pq_fs;
    size_t off_pX, off_pX1, off_pFP, off_Qh, off_Kh, off_Ql, off_Kl, off_pVt, off_Op, off_ML, off_pW, off_pS;
    size_t ws_bytes;
};

// HIP-event timing of one stage's launches (see tfl_timer_arm).
struct StageTimer {
    int stage = 0;
    int cap = 0;
    int n = 0;
    hipEvent_t* start = nullptr;
    hipEvent_t* stop = nullptr;
};

size_t dtype_size(int dtype);

// Device counters the attention kernels add their visited tiles to in the
// audit build (set through tfl_audit_attach); null in the product build.
extern unsigned long long* audit_counters;

// The dispatcher's rule for a valid configuration (tfl_path, never AUTO).
int choose_path(const tfl_config& cfg);

tfl_status make_plan(const tfl_config& cfg, Plan* p, std::string* why);

hipError_t run_plan(const Plan& p, const tfl_layer* layers, const void* x, const int32_t* lens, void* y,
                    char* ws, hipStream_t s, StageTimer* timer);

}  // namespace tfl
