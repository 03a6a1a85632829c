// C ABI of tfl: argument checks, the frozen per-shape plan, the workspace
// layout and the launch sequence.  Declarations and contracts: include/tfl.h.
#include "tfl.h"
#include "tfl_audit.h"

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "plan.h"

struct tfl_handle {
    tfl_config cfg;
    std::vector<tfl_layer> layers;
    tfl::Plan plan;
    tfl::StageTimer timer;
};

namespace {

thread_local std::string g_err;

tfl_status fail(tfl_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

tfl_status hip_fail(hipError_t e, const char* what) {
    return fail(TFL_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Workspace of tfl_forward_noalloc: one static array in device memory, which
// every GPU the library runs on holds (at its own address) until the process
// ends.  Host code never passes the array's name to a kernel or copy (on the
// host it is a stand-in, not a device address): the address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t STATIC_WS_MAX = (size_t)TFL_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[STATIC_WS_MAX];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

tfl_status static_workspace(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "tfl_forward_noalloc: hipGetDevice");
    if (dev < 0 || dev >= MAX_DEVICES) return fail(TFL_E_UNSUPPORTED, "tfl_forward_noalloc: device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "tfl_forward_noalloc: hipGetSymbolAddress of the static workspace");
        if (!p || !aligned(p, 256)) return fail(TFL_E_INTERNAL, "tfl_forward_noalloc: static workspace address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TFL_OK;
}

// Device word of the TFL_CHECK=1 magnitude check (one per GPU, its address
// taken with that device current).
static __device__ unsigned check_amax_word;
void* g_amax_ptr[MAX_DEVICES];

// TFL_CHECK=1: the inputs the kernels round to fp16 operands must be finite
// and below 65504 in magnitude (x and the GEMM weights with bf16 I/O on every
// path and with fp32 I/O on the PQ and layer-wise paths); x must be finite on
// every path.  One reduction launch per array, then a synchronising copy.
tfl_status check_magnitudes(const tfl_handle* h, const void* x, hipStream_t s) {
    const tfl::Plan& P = h->plan;
    const int dt = h->cfg.dtype;
    const bool f16_operands = dt == TFL_BF16 || (dt == TFL_F32 && !(P.path == TFL_PATH_SEQ && P.seq_kind == 1));
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return hip_fail(e, "tfl_forward: TFL_CHECK hipGetDevice");
    if (!g_amax_ptr[dev]) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_amax_word));
        if (e != hipSuccess) return hip_fail(e, "tfl_forward: TFL_CHECK hipGetSymbolAddress");
        g_amax_ptr[dev] = p;
    }
    unsigned* word = (unsigned*)g_amax_ptr[dev];
    const size_t esz = tfl::dtype_size(dt);
    auto amax = [&](const void* a, long n, unsigned* bits) -> hipError_t {
        hipError_t r = hipMemsetAsync(word, 0, sizeof(unsigned), s);
        if (r == hipSuccess) r = tfl::launch_amax((int)esz, dt == TFL_BF16, a, n, word, s);
        if (r == hipSuccess) r = hipMemcpyAsync(bits, word, sizeof(unsigned), hipMemcpyDeviceToHost, s);
        if (r == hipSuccess) r = hipStreamSynchronize(s);
        return r;
    };
    const float limit = 65504.f;
    unsigned bits = 0;
    if ((e = amax(x, (long)P.T * P.d, &bits)) != hipSuccess) return hip_fail(e, "tfl_forward: TFL_CHECK of x");
    float v;
    std::memcpy(&v, &bits, 4);
    if (!(v <= 3.4028235e38f)) return fail(TFL_E_INVALID, "tfl_forward: x holds a non-finite value");
    if (f16_operands && !(v < limit))
        return fail(TFL_E_INVALID, "tfl_forward: |x| reaches " + std::to_string(v) +
                                       "; the fp16 operands of this path need |x| < 65504");
    if (!f16_operands) return TFL_OK;
    const long dd = (long)P.d * P.d, df = (long)P.d * P.f;
    for (int l = 0; l < P.n_layers; l++) {
        const tfl_layer& w = h->layers[l];
        const void* m[4] = {w.w_qkv, w.w_o, w.w_1, w.w_2};
        const long n[4] = {3 * dd, dd, df, df};
        for (int k = 0; k < 4; k++) {
            if ((e = amax(m[k], n[k], &bits)) != hipSuccess) return hip_fail(e, "tfl_forward: TFL_CHECK of the weights");
            std::memcpy(&v, &bits, 4);
            if (!(v < limit))
                return fail(TFL_E_INVALID, "tfl_forward: layer " + std::to_string(l) + " weight matrix " +
                                               std::to_string(k) + " reaches |w| = " + std::to_string(v) +
                                               "; the fp16 operands of this path need |w| < 65504");
        }
    }
    return TFL_OK;
}

}  // namespace

extern "C" {

tfl_status tfl_create(const tfl_config* cfg, const tfl_layer* layers, tfl_handle** out) {
    if (!cfg || !layers || !out) return fail(TFL_E_INVALID, "tfl_create: null argument");
    *out = nullptr;
    std::string why;
    tfl::Plan plan;
    const tfl_status st = tfl::make_plan(*cfg, &plan, &why);
    if (st != TFL_OK) return fail(st, "tfl_create: " + why);
    for (int l = 0; l < cfg->n_layers; l++) {
        const tfl_layer& w = layers[l];
        const void* mats[4] = {w.w_qkv, w.w_o, w.w_1, w.w_2};
        const void* vecs[8] = {w.b_qkv, w.b_o, w.ln1_g, w.ln1_b, w.b_1, w.b_2, w.ln2_g, w.ln2_b};
        for (const void* m : mats)
            if (!m || !aligned(m, 16))
                return fail(TFL_E_INVALID, "tfl_create: layer " + std::to_string(l) +
                                               ": weight matrix pointer null or not 16-byte aligned");
        for (const void* v : vecs)
            if (!v || !aligned(v, 16))
                return fail(TFL_E_INVALID, "tfl_create: layer " + std::to_string(l) +
                                               ": bias/LayerNorm pointer null or not 16-byte aligned");
    }
    tfl_handle* h = new (std::nothrow) tfl_handle;
    if (!h) return fail(TFL_E_INTERNAL, "tfl_create: out of host memory");
    h->cfg = *cfg;
    h->layers.assign(layers, layers + cfg->n_layers);
    h->plan = plan;
    *out = h;
    return TFL_OK;
}

tfl_status tfl_workspace_bytes(const tfl_handle* h, size_t* bytes) {
    if (!h || !bytes) return fail(TFL_E_INVALID, "tfl_workspace_bytes: null argument");
    *bytes = h->plan.ws_bytes;
    return TFL_OK;
}

// tfl_forward with the host-side length check of TFL_CHECK=1 allowed or not
// (that check copies the lengths into host memory).
static tfl_status forward_impl(tfl_handle* h, const void* x, const int32_t* valid_len, void* y, void* workspace,
                               size_t workspace_bytes, void* hip_stream, bool allow_check) {
    if (!h) return fail(TFL_E_INVALID, "tfl_forward: null handle");
    if (!x || !y || !valid_len) return fail(TFL_E_INVALID, "tfl_forward: null x, y or valid_len");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(valid_len, 4))
        return fail(TFL_E_INVALID, "tfl_forward: x and y must be 16-byte aligned, valid_len 4-byte aligned");
    const tfl::Plan& P = h->plan;
    if (workspace_bytes < P.ws_bytes)
        return fail(TFL_E_WORKSPACE, "tfl_forward: workspace of " + std::to_string(workspace_bytes) +
                                         " bytes, plan needs " + std::to_string(P.ws_bytes));
    if (P.ws_bytes > 0 && (!workspace || !aligned(workspace, 256)))
        return fail(TFL_E_INVALID, "tfl_forward: workspace null or not 256-byte aligned");
    const size_t io_bytes = (size_t)P.T * P.d * tfl::dtype_size(h->cfg.dtype);
    if (overlap(x, io_bytes, y, io_bytes)) return fail(TFL_E_INVALID, "tfl_forward: y overlaps x");
    if (P.ws_bytes > 0 && overlap(y, io_bytes, workspace, P.ws_bytes))
        return fail(TFL_E_INVALID, "tfl_forward: y overlaps the workspace");
    if (P.ws_bytes > 0 && overlap(x, io_bytes, workspace, P.ws_bytes))
        return fail(TFL_E_INVALID, "tfl_forward: x overlaps the workspace");
    hipStream_t s = (hipStream_t)hip_stream;

    const char* chk = allow_check ? std::getenv("TFL_CHECK") : nullptr;
    const bool check = chk && chk[0] == '1';
    if (check) {
        std::vector<int32_t> lens(P.B);
        hipError_t e = hipMemcpyAsync(lens.data(), valid_len, sizeof(int32_t) * P.B, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "tfl_forward: TFL_CHECK copy of valid_len");
        for (int b = 0; b < P.B; b++)
            if (lens[b] < 1 || lens[b] > P.L)
                return fail(TFL_E_INVALID, "tfl_forward: valid_len[" + std::to_string(b) + "] = " +
                                               std::to_string(lens[b]) + " outside [1, seq_len]");
        const tfl_status st = check_magnitudes(h, x, s);
        if (st != TFL_OK) return st;
    }
    tfl::StageTimer* tm = h->timer.stage ? &h->timer : nullptr;
    const hipError_t e = tfl::run_plan(P, h->layers.data(), x, valid_len, y, (char*)workspace, s, tm);
    if (e != hipSuccess) return hip_fail(e, "tfl_forward: kernel launch");
    return TFL_OK;
}

tfl_status tfl_forward(tfl_handle* h, const void* x, const int32_t* valid_len, void* y, void* workspace,
                       size_t workspace_bytes, void* hip_stream) {
    return forward_impl(h, x, valid_len, y, workspace, workspace_bytes, hip_stream, true);
}

tfl_status tfl_forward_noalloc(tfl_handle* h, const void* x, const int32_t* valid_len, void* y, void* hip_stream) {
    if (!h) return fail(TFL_E_INVALID, "tfl_forward_noalloc: null handle");
    const size_t need = h->plan.ws_bytes;
    if (need > STATIC_WS_MAX)
        return fail(TFL_E_WORKSPACE, "tfl_forward_noalloc: the plan " + std::string(h->plan.name) + " needs " +
                                         std::to_string(need) + " bytes of workspace; the static workspace holds " +
                                         std::to_string(STATIC_WS_MAX) + " (use tfl_forward with a workspace)");
    void* ws = nullptr;
    if (need > 0) {
        const tfl_status st = static_workspace(&ws);
        if (st != TFL_OK) return st;
    }
    return forward_impl(h, x, valid_len, y, ws, need, hip_stream, false);
}

static void timer_release(tfl::StageTimer& t) {
    for (int i = 0; i < t.cap; i++) {
        if (t.start) (void)hipEventDestroy(t.start[i]);
        if (t.stop) (void)hipEventDestroy(t.stop[i]);
    }
    delete[] t.start;
    delete[] t.stop;
    t = tfl::StageTimer{};
}

tfl_status tfl_timer_arm(tfl_handle* h, int32_t stage, int32_t max_launches) {
    if (!h) return fail(TFL_E_INVALID, "tfl_timer_arm: null handle");
    if (stage < TFL_STAGE_PREP || stage > TFL_STAGE_ROW || max_launches < 1 || max_launches > 1 << 20)
        return fail(TFL_E_INVALID, "tfl_timer_arm: bad stage or launch count");
    timer_release(h->timer);
    tfl::StageTimer t;
    t.start = new (std::nothrow) hipEvent_t[max_launches]();
    t.stop = new (std::nothrow) hipEvent_t[max_launches]();
    if (!t.start || !t.stop) {
        delete[] t.start;
        delete[] t.stop;
        return fail(TFL_E_INTERNAL, "tfl_timer_arm: out of host memory");
    }
    for (int i = 0; i < max_launches; i++) {
        hipError_t e = hipEventCreate(&t.start[i]);
        if (e == hipSuccess) e = hipEventCreate(&t.stop[i]);
        if (e != hipSuccess) {
            t.cap = i + 1;
            timer_release(t);
            return hip_fail(e, "tfl_timer_arm: hipEventCreate");
        }
    }
    t.cap = max_launches;
    t.stage = stage;
    h->timer = t;
    return TFL_OK;
}

tfl_status tfl_timer_read(tfl_handle* h, float* total_ms, int32_t* launches) {
    if (!h || !total_ms || !launches) return fail(TFL_E_INVALID, "tfl_timer_read: null argument");
    tfl::StageTimer& t = h->timer;
    float sum = 0.f;
    for (int i = 0; i < t.n; i++) {
        hipError_t e = hipEventSynchronize(t.stop[i]);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start[i], t.stop[i]);
        if (e != hipSuccess) {
            timer_release(t);
            return hip_fail(e, "tfl_timer_read");
        }
        sum += ms;
    }
    *total_ms = sum;
    *launches = t.n;
    timer_release(t);
    return TFL_OK;
}

tfl_status tfl_destroy(tfl_handle* h) {
    if (h) timer_release(h->timer);
    delete h;
    return TFL_OK;
}

const char* tfl_plan_name(const tfl_handle* h) { return h ? h->plan.name : "(null handle)"; }

int32_t tfl_plan_path(const tfl_handle* h) { return h ? h->plan.path : -1; }

const char* tfl_last_error(void) { return g_err.c_str(); }

#if TFL_AUDIT
// Test build only (include/tfl_audit.h).
tfl_status tfl_audit_attach(void* counters) {
    if (counters && !aligned(counters, 8)) return fail(TFL_E_INVALID, "tfl_audit_attach: counters not 8-byte aligned");
    tfl::audit_counters = (unsigned long long*)counters;
    return TFL_OK;
}
#endif

}  // extern "C"
