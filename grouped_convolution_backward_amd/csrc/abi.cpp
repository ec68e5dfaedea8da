// extern "C" entry points declared in include/wgrad.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <string>

#include "wgrad_internal.hpp"

struct wgrad_plan_s {
    wgrad::Plan plan;
};

namespace {

thread_local std::string g_last_error;

int set_error(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// hip_device >= 0: size the plan for that device, which must be gfx950;
// -1 keeps the MI355X model (256 CUs, 8 XCDs) without touching HIP.
int device_model(int hip_device, wgrad::DeviceModel& dev) {
    if (hip_device < 0) return WGRAD_OK;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, hip_device);
    if (e != hipSuccess)
        return set_error(WGRAD_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return set_error(WGRAD_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName +
                                                    ", kernels are built for gfx950 only");
    dev.num_cus = prop.multiProcessorCount;
    return WGRAD_OK;
}

}  // namespace

extern "C" {

int wgrad_plan(const wgrad_problem* problem, const wgrad_overrides* overrides, int hip_device,
               wgrad_plan_t** out) {
    g_last_error.clear();
    if (!problem || !out) return set_error(WGRAD_ERR_INVALID_ARG, "problem and out must not be NULL");
    *out = nullptr;
    wgrad::DeviceModel dev{256, 8};   // MI355X: 256 CUs in 8 XCDs
    if (int rc = device_model(hip_device, dev)) return rc;
    std::string msg;
    wgrad_plan_s* p = new (std::nothrow) wgrad_plan_s();
    if (!p) return set_error(WGRAD_ERR_INVALID_ARG, "out of host memory");
    int rc = wgrad::build_plan(*problem, overrides, dev, p->plan, &msg);
    if (rc != WGRAD_OK) {
        delete p;
        return set_error(rc, msg);
    }
    *out = p;
    return WGRAD_OK;
}

int wgrad_dgrad_plan(const wgrad_problem* problem, const wgrad_overrides* overrides, int hip_device,
                     wgrad_plan_t** out) {
    g_last_error.clear();
    if (!problem || !out) return set_error(WGRAD_ERR_INVALID_ARG, "problem and out must not be NULL");
    *out = nullptr;
    wgrad::DeviceModel dev{256, 8};
    if (int rc = device_model(hip_device, dev)) return rc;
    std::string msg;
    wgrad_plan_s* p = new (std::nothrow) wgrad_plan_s();
    if (!p) return set_error(WGRAD_ERR_INVALID_ARG, "out of host memory");
    int rc = wgrad::build_dgrad_plan(*problem, overrides, dev, p->plan, &msg);
    if (rc != WGRAD_OK) {
        delete p;
        return set_error(rc, msg);
    }
    *out = p;
    return WGRAD_OK;
}

int wgrad_dgrad_run(const wgrad_plan_t* plan, const void* dy, const void* w, void* dx, void* stream) {
    g_last_error.clear();
    if (!plan) return set_error(WGRAD_ERR_INVALID_ARG, "plan is NULL");
    const wgrad::Plan& P = plan->plan;
    if (P.op != wgrad::OP_DGRAD) return set_error(WGRAD_ERR_INVALID_ARG, "not a backward-data plan");
    const int64_t grid = P.dg_ring >= 0 ? P.dgr.total_wg : P.dg_dwt ? P.dgdwt.total_wg
                                                    : P.dg_dw ? P.dgdw.total_wg : P.dg.total_wg;
    if (grid == 0) return WGRAD_OK;   // N = 0: dX is empty
    if (!dx || !dy || !w) return set_error(WGRAD_ERR_INVALID_ARG, "dy, w and dx must not be NULL");
    if (!aligned16(dy) || !aligned16(w) || !aligned16(dx))
        return set_error(WGRAD_ERR_INVALID_ARG, "dy, w and dx must be 16-byte aligned");
    int e;
    if (P.dg_ring >= 0) {
        wgrad::DgradRingArgs a = P.dgr;
        a.dy = static_cast<const uint16_t*>(dy);
        a.w = static_cast<const uint16_t*>(w);
        a.dx = dx;
        e = wgrad::launch_dgrad_ring(P, a, stream);
    } else if (P.dg_dwt) {
        wgrad::DgradDwTileArgs a = P.dgdwt;
        a.dy = static_cast<const uint16_t*>(dy);
        a.w = static_cast<const uint16_t*>(w);
        a.dx = dx;
        e = wgrad::launch_dgrad_dwtile(P, a, stream);
    } else if (P.dg_dw) {
        wgrad::DgradDwArgs a = P.dgdw;
        a.dy = static_cast<const uint16_t*>(dy);
        a.w = static_cast<const uint16_t*>(w);
        a.dx = dx;
        e = wgrad::launch_dgrad_dw(P, a, stream);
    } else {
        wgrad::DgradArgs a = P.dg;
        a.dy = static_cast<const uint16_t*>(dy);
        a.w = static_cast<const uint16_t*>(w);
        a.dx = dx;
        e = wgrad::launch_dgrad(P, a, stream);
    }
    if (e != hipSuccess)
        return set_error(WGRAD_ERR_HIP, std::string("dgrad kernel launch: ") + hipGetErrorString((hipError_t)e));
    return WGRAD_OK;
}

size_t wgrad_workspace_bytes(const wgrad_plan_t* plan) {
    return plan ? static_cast<size_t>(plan->plan.info.workspace_bytes) : 0;
}

}  // extern "C"

namespace {

// Checks of a backward-weight run's plan and tensor pointers.
int check_run_args(const wgrad_plan_t* plan, const void* x, const void* dy, const void* dw) {
    if (!plan) return set_error(WGRAD_ERR_INVALID_ARG, "plan is NULL");
    const wgrad::Plan& P = plan->plan;
    if (P.op != wgrad::OP_WGRAD) return set_error(WGRAD_ERR_INVALID_ARG, "not a backward-weight plan");
    const bool empty_in = P.info.gemm_k == 0;
    if (!dw) return set_error(WGRAD_ERR_INVALID_ARG, "dw is NULL");
    if (!empty_in && (!x || !dy)) return set_error(WGRAD_ERR_INVALID_ARG, "x and dy must not be NULL");
    if ((x && !aligned16(x)) || (dy && !aligned16(dy)) || !aligned16(dw))
        return set_error(WGRAD_ERR_INVALID_ARG, "x, dy and dw must be 16-byte aligned");
    return WGRAD_OK;
}

int run_stages(const wgrad_plan_t* plan, int first, int last, const void* x, const void* dy, void* dw,
               void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (int rc = check_run_args(plan, x, dy, dw)) return rc;
    const wgrad::Plan& P = plan->plan;
    const size_t need = static_cast<size_t>(P.info.workspace_bytes);
    if (need) {
        if (!ws) return set_error(WGRAD_ERR_INVALID_ARG, "workspace is NULL but the plan needs " + std::to_string(need) + " bytes");
        if (ws_bytes < need)
            return set_error(WGRAD_ERR_INVALID_ARG, "workspace of " + std::to_string(ws_bytes) +
                                                        " bytes is smaller than the " + std::to_string(need) + " needed");
        if (!aligned16(ws)) return set_error(WGRAD_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    int e = hipSuccess;
    if (first <= 1) {
        void* main_out = P.info.split_k > 1 ? ws : dw;
        if (P.variant == WGRAD_VARIANT_ROWSLAB && P.ring_inst >= 0) {
            wgrad::RingArgs a = P.ring;
            a.x = static_cast<const uint16_t*>(x);
            a.dy = static_cast<const uint16_t*>(dy);
            a.out = main_out;
            e = wgrad::launch_ring(P, a, stream);
        } else if (P.variant == WGRAD_VARIANT_ROWSLAB) {
            wgrad::RowSlabArgs a = P.rs;
            a.x = static_cast<const uint16_t*>(x);
            a.dy = static_cast<const uint16_t*>(dy);
            a.out = main_out;
            e = wgrad::launch_rowslab(P, a, stream);
        } else if (P.variant == WGRAD_VARIANT_DEPTHWISE && P.dwt_cb) {
            wgrad::DwTileArgs a = P.dwt;
            a.x = static_cast<const uint16_t*>(x);
            a.dy = static_cast<const uint16_t*>(dy);
            a.out = main_out;
            e = wgrad::launch_dwtile(P, a, stream);
        } else if (P.variant == WGRAD_VARIANT_DEPTHWISE && P.dw3_ty) {
            wgrad::Dw3Args a = P.dw3;
            a.x = static_cast<const uint16_t*>(x);
            a.dy = static_cast<const uint16_t*>(dy);
            a.out = main_out;
            e = wgrad::launch_depthwise3(P, a, stream);
        } else if (P.variant == WGRAD_VARIANT_DEPTHWISE && P.dw2_ty) {
            wgrad::Dw2Args a = P.dw2;
            a.x = static_cast<const uint16_t*>(x);
            a.dy = static_cast<const uint16_t*>(dy);
            a.out = main_out;
            e = wgrad::launch_depthwise2(P, a, stream);
        } else if (P.variant == WGRAD_VARIANT_DEPTHWISE) {
            wgrad::DwArgs a = P.dwk;
            a.x = static_cast<const uint16_t*>(x);
            a.dy = static_cast<const uint16_t*>(dy);
            a.out = main_out;
            e = wgrad::launch_depthwise(P, a, stream);
        } else {
            wgrad::MfmaArgs a = P.mfma;
            a.x = static_cast<const uint16_t*>(x);
            a.dy = static_cast<const uint16_t*>(dy);
            a.out = main_out;
            e = wgrad::launch_mfma(P, a, stream);
        }
        if (e != hipSuccess)
            return set_error(WGRAD_ERR_HIP, std::string("main kernel launch: ") + hipGetErrorString((hipError_t)e));
    }
    if (last >= 2 && P.info.split_k > 1) {
        wgrad::ReduceArgs r = P.red;
        r.ws = static_cast<const float*>(ws);
        r.dw = dw;
        e = wgrad::launch_reduce(r, P.info.grid_reduce, stream);
        if (e != hipSuccess)
            return set_error(WGRAD_ERR_HIP, std::string("reduce kernel launch: ") + hipGetErrorString((hipError_t)e));
    }
    return WGRAD_OK;
}

}  // namespace

extern "C" {

int wgrad_run(const wgrad_plan_t* plan, const void* x, const void* dy, void* dw, void* ws, size_t ws_bytes,
              void* stream) {
    return run_stages(plan, 1, 2, x, dy, dw, ws, ws_bytes, stream);
}

int wgrad_run_stage(const wgrad_plan_t* plan, int stage, const void* x, const void* dy, void* dw, void* ws,
                    size_t ws_bytes, void* stream) {
    if (stage != 1 && stage != 2) return set_error(WGRAD_ERR_INVALID_ARG, "stage must be 1 or 2");
    return run_stages(plan, stage, stage, x, dy, dw, ws, ws_bytes, stream);
}

int wgrad_run_noalloc(const wgrad_plan_t* plan, const void* x, const void* dy, void* dw, void* stream) {
    g_last_error.clear();
    if (int rc = check_run_args(plan, x, dy, dw)) return rc;
    const size_t need = static_cast<size_t>(plan->plan.info.workspace_bytes);
    if (need > static_cast<size_t>(WGRAD_NOALLOC_SCRATCH_BYTES))
        return set_error(WGRAD_ERR_INVALID_ARG,
                         "the plan's split-K workspace of " + std::to_string(need) +
                             " bytes exceeds the library scratch of " +
                             std::to_string(static_cast<size_t>(WGRAD_NOALLOC_SCRATCH_BYTES)) +
                             " bytes; use wgrad_run with a caller workspace or a plan with a smaller split_k");
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need) {
        const int e = wgrad::scratch_workspace(stream, &ws, &ws_bytes);
        if (e != hipSuccess)
            return set_error(WGRAD_ERR_HIP, std::string("library scratch on this device: ") +
                                                hipGetErrorString((hipError_t)e));
    }
    return run_stages(plan, 1, 2, x, dy, dw, ws, ws_bytes, stream);
}

int wgrad_plan_query(const wgrad_plan_t* plan, wgrad_plan_info* info) {
    g_last_error.clear();
    if (!plan || !info) return set_error(WGRAD_ERR_INVALID_ARG, "plan and info must not be NULL");
    *info = plan->plan.info;
    return WGRAD_OK;
}

const char* wgrad_plan_describe(const wgrad_plan_t* plan) {
    return plan ? plan->plan.name.c_str() : "";
}

void wgrad_plan_destroy(wgrad_plan_t* plan) { delete plan; }

const char* wgrad_last_error(void) { return g_last_error.c_str(); }

const char* wgrad_version(void) { return "0.2.0"; }

int wgrad_probe_transpose_read(void* out, void* stream) {
    g_last_error.clear();
    if (!out) return set_error(WGRAD_ERR_INVALID_ARG, "out must not be NULL");
    if (!aligned16(out)) return set_error(WGRAD_ERR_INVALID_ARG, "out must be 16-byte aligned");
    const int e = wgrad::launch_tr_probe(static_cast<uint16_t*>(out), stream);
    if (e != hipSuccess)
        return set_error(WGRAD_ERR_HIP, std::string("probe kernel launch: ") + hipGetErrorString((hipError_t)e));
    return WGRAD_OK;
}

}  // extern "C"
