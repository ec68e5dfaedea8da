// Drives the host planner and C ABI (plan.cpp, abi.cpp, with the launcher
// stubs of hip_stubs.cpp) from a list of problems on stdin, for the
// sanitizer build. One line per case:
//
//   <op> ndim in_dtype out_dtype G N C K in_len[3] filt_len[3] stride[3]
//        dilation[3] pad_lo[3] pad_hi[3] split_k group_merge variant tile
//
// op 0 plans backward weight, op 1 backward data. For each case it prints
//
//   status|name|variant|tile|split_k|group_merge|grid_main|grid_reduce|workspace_bytes
//
// and, for a plan that was made, exercises the run entry points with NULL,
// misaligned and valid-looking pointers (the stub launchers never touch them)
// and checks the status each must return. Exit status 1 on a failed check.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "wgrad.h"

int stub_launch_count();

namespace {

int fails = 0;

void expect(bool ok, const char* what, long line) {
    if (!ok) {
        std::fprintf(stderr, "case %ld: %s\n", line, what);
        ++fails;
    }
}

}  // namespace

int main() {
    long line = 0;
    long long v[30];
    // distinct 256-byte-aligned addresses that are never dereferenced
    void* const fake_x = reinterpret_cast<void*>(uintptr_t{0x100000});
    void* const fake_dy = reinterpret_cast<void*>(uintptr_t{0x200000});
    void* const fake_dw = reinterpret_cast<void*>(uintptr_t{0x300000});
    void* const fake_ws = reinterpret_cast<void*>(uintptr_t{0x400000});
    void* const odd = reinterpret_cast<void*>(uintptr_t{0x500008});
    while (true) {
        int n = 0;
        for (; n < 30; ++n)
            if (std::scanf("%lld", &v[n]) != 1) break;
        if (n == 0) break;
        if (n != 30) {
            std::fprintf(stderr, "malformed input line %ld\n", line);
            return 2;
        }
        ++line;
        const int op = (int)v[0];
        wgrad_problem p;
        std::memset(&p, 0, sizeof p);
        p.ndim = (int32_t)v[1];
        p.in_dtype = (int32_t)v[2];
        p.out_dtype = (int32_t)v[3];
        p.G = v[4]; p.N = v[5]; p.C = v[6]; p.K = v[7];
        for (int i = 0; i < 3; ++i) {
            p.in_len[i] = v[8 + i];
            p.filt_len[i] = v[11 + i];
            p.stride[i] = v[14 + i];
            p.dilation[i] = v[17 + i];
            p.pad_lo[i] = v[20 + i];
            p.pad_hi[i] = v[23 + i];
        }
        wgrad_overrides o;
        o.split_k = (int32_t)v[26];
        o.group_merge = (int32_t)v[27];
        o.variant = (int32_t)v[28];
        o.tile = (int32_t)v[29];
        wgrad_plan_t* plan = nullptr;
        const int st = op == 0 ? wgrad_plan(&p, &o, -1, &plan) : wgrad_dgrad_plan(&p, &o, -1, &plan);
        if (st != WGRAD_OK) {
            expect(plan == nullptr, "failed plan left *out set", line);
            expect(std::strlen(wgrad_last_error()) > 0, "failed plan without a reason", line);
            std::printf("%d|||||||||\n", st);
            continue;
        }
        wgrad_plan_info info;
        expect(wgrad_plan_query(plan, &info) == WGRAD_OK, "query", line);
        expect(wgrad_plan_query(plan, nullptr) == WGRAD_ERR_INVALID_ARG, "query NULL info", line);
        const size_t ws = wgrad_workspace_bytes(plan);
        expect((int64_t)ws == info.workspace_bytes, "workspace bytes differ from the plan info", line);
        const char* name = wgrad_plan_describe(plan);
        std::printf("%d|%s|%d|%d|%d|%d|%lld|%lld|%lld\n", st, name, info.variant, info.tile, info.split_k,
                    info.group_merge, (long long)info.grid_main, (long long)info.grid_reduce,
                    (long long)info.workspace_bytes);
        const bool empty = info.gemm_k == 0;
        const int before = stub_launch_count();
        if (op == 0) {
            expect(wgrad_dgrad_run(plan, fake_dy, fake_x, fake_dw, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "dgrad run accepted a wgrad plan", line);
            expect(wgrad_run(plan, fake_x, fake_dy, nullptr, fake_ws, ws, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "NULL dw accepted", line);
            if (!empty)
                expect(wgrad_run(plan, nullptr, fake_dy, fake_dw, fake_ws, ws, nullptr) == WGRAD_ERR_INVALID_ARG,
                       "NULL x accepted", line);
            expect(wgrad_run(plan, fake_x, fake_dy, odd, fake_ws, ws, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "misaligned dw accepted", line);
            if (ws) {
                expect(wgrad_run(plan, fake_x, fake_dy, fake_dw, fake_ws, ws - 1, nullptr) == WGRAD_ERR_INVALID_ARG,
                       "short workspace accepted", line);
                expect(wgrad_run(plan, fake_x, fake_dy, fake_dw, nullptr, ws, nullptr) == WGRAD_ERR_INVALID_ARG,
                       "NULL workspace accepted", line);
            }
            expect(wgrad_run_stage(plan, 3, fake_x, fake_dy, fake_dw, fake_ws, ws, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "stage 3 accepted", line);
            expect(stub_launch_count() == before, "a rejected call launched a kernel", line);
            expect(wgrad_run(plan, fake_x, fake_dy, fake_dw, fake_ws, ws, nullptr) == WGRAD_ERR_HIP,
                   "launch failure not reported", line);
            expect(std::strlen(wgrad_last_error()) > 0, "launch failure without a reason", line);
            expect(stub_launch_count() == before + 1, "run did not stop at the failed launch", line);
            expect(wgrad_run_stage(plan, 2, fake_x, fake_dy, fake_dw, fake_ws, ws, nullptr) ==
                       (info.split_k > 1 ? WGRAD_ERR_HIP : WGRAD_OK),
                   "stage 2", line);
            // the library-scratch variant: a workspace beyond the scratch is
            // rejected before any device call; otherwise the stubbed device
            // lookup (or launch) fails
            const int before_na = stub_launch_count();
            const int na = wgrad_run_noalloc(plan, fake_x, fake_dy, fake_dw, nullptr);
            if (ws > WGRAD_NOALLOC_SCRATCH_BYTES) {
                expect(na == WGRAD_ERR_INVALID_ARG, "oversized workspace accepted by the no-allocation run", line);
                expect(stub_launch_count() == before_na, "oversized no-allocation run launched", line);
            } else {
                expect(na == WGRAD_ERR_HIP, "no-allocation run without a device", line);
            }
            expect(wgrad_run_noalloc(plan, fake_x, fake_dy, nullptr, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "no-allocation run accepted a NULL dw", line);
            expect(wgrad_run_noalloc(plan, fake_x, fake_dy, odd, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "no-allocation run accepted a misaligned dw", line);
            expect(stub_launch_count() == before_na + (ws > WGRAD_NOALLOC_SCRATCH_BYTES || ws ? 0 : 1),
                   "a rejected no-allocation run launched", line);
        } else {
            expect(wgrad_run(plan, fake_x, fake_dy, fake_dw, fake_ws, ws, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "wgrad run accepted a dgrad plan", line);
            expect(wgrad_run_noalloc(plan, fake_x, fake_dy, fake_dw, nullptr) == WGRAD_ERR_INVALID_ARG,
                   "no-allocation run accepted a dgrad plan", line);
            if (info.grid_main > 0) {   // an empty dX (N = 0) needs no pointers
                expect(wgrad_dgrad_run(plan, fake_dy, fake_x, nullptr, nullptr) == WGRAD_ERR_INVALID_ARG,
                       "NULL dx accepted", line);
                expect(wgrad_dgrad_run(plan, fake_dy, odd, fake_dw, nullptr) == WGRAD_ERR_INVALID_ARG,
                       "misaligned w accepted", line);
            }
            expect(stub_launch_count() == before, "a rejected call launched a kernel", line);
            const int rs = wgrad_dgrad_run(plan, fake_dy, fake_x, fake_dw, nullptr);
            expect(rs == (info.grid_main == 0 ? WGRAD_OK : WGRAD_ERR_HIP), "dgrad launch status", line);
        }
        wgrad_plan_destroy(plan);
    }
    wgrad_plan_destroy(nullptr);
    expect(std::strlen(wgrad_version()) > 0, "version", 0);
    std::fflush(stdout);
    return fails ? 1 : 0;
}
