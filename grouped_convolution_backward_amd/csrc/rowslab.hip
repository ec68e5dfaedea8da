// Row-slab MFMA kernel for grouped convolution backward-weight on gfx950.
//
// The implicit GEMM of the Composable Kernel wgrad page (A = dY rows, B = X
// gathered per filter tap, reduction over r = (n*Ho + ho)*Wo + wo), tiled so
// that X is staged once per output row instead of once per tap:
//
// * A workgroup owns one filter row y of one (group block, M block, C block)
//   tile and every filter column x of that row: its output tile is
//   MB x (X*CB), and for one output row it needs exactly one input row.
// * The reduction runs over slabs of PR output rows x SW output columns. A
//   slab's dY rows are staged K-outer ([position][channel]) and its input
//   rows as a pixel tile ([row][column][channel]); tap x of position k is
//   pixel (k / SW, (k % SW)*stride + x*dilation) of that tile, so the three
//   (or five) taps of the row are shifted reads of one tile.
// * MFMA operands come from the CDNA4 transposed LDS read
//   ds_read_b64_tr_b16 (rocm-libraries PR 11602): each lane supplies the
//   address of its own reduction row, which here is a per-lane pixel offset,
//   so the halo tile needs no per-tap copy and nothing is transposed on store.
// * Each of the four waves holds the whole workgroup tile in registers and
//   takes every fourth slab of the workgroup's split; a wave only touches its
//   own LDS region, so the slab loop has no workgroup barrier. The next
//   slab's global loads are issued before the current slab's MFMAs and wait
//   in registers (the single-buffer "basic" schedule of PR 11602).
// * At the end the four wave tiles are added in LDS in a fixed order and the
//   workgroup writes one partial (S > 1: fp32 workspace slice) or dW itself.
//   With merged groups only diagonal group pairs are stored (PR 12359).
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;


__device__ __forceinline__ void store4(void* out, int mode, int64_t e, const f32x4& v) {
    if (mode == OUT_BF16) {
        u32x2 p;
        p[0] = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        p[1] = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + e) = p;
    } else if (mode == OUT_FP16) {
        u32x2 p;
        p[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[1]) << 16);
        p[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[3]) << 16);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + e) = p;
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + e) = v;
    }
}

template <int MB, int CB, int XF, int NKS, int NXR, int NXC, int PA, int PX, bool ASWZ, bool F16>
__global__ __launch_bounds__(256, 1) void rowslab_kernel(const RowSlabArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    static_assert(PA >= MB && PX >= CB && PA % 8 == 0 && PX % 8 == 0, "LDS pitches");
    static_assert(!ASWZ || MB == 64, "the dY swizzle is defined for 64-wide rows");
    constexpr int FM = MB / 32, FC = CB / 32, FN = XF * FC;
    constexpr int AV = MB / 8, XV = CB / 8;        // 16-byte vectors per position / pixel
    constexpr int KS = 16 * NKS;                   // positions per slab (padded)
    constexpr int APL = 64 / AV;                   // positions per dY load instruction
    constexpr int NA = KS / APL;
    constexpr int PPL = 64 / XV;                   // pixels per X load instruction
    constexpr int XWP = NXC * PPL;                 // pixels per X tile row in LDS
    constexpr int WAVE_LDS = KS * PA + NXR * XWP * PX;
    constexpr int RP = CB + 4;                     // row pitch of the reduction tile (floats)
    constexpr int TILE = MB * RP;
    static_assert(KS % APL == 0, "slab positions");

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint16_t* sA = smem + wave * WAVE_LDS;
    uint16_t* sX = sA + KS * PA;

    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    int t = L % a.tiles;
    const int z = L / a.tiles;
    const int y = t % a.Y;
    t /= a.Y;
    const int cbk = t % a.cblocks;
    t /= a.cblocks;
    const int mbk = t % a.mblocks;
    const int gb = t / a.mblocks;
    const int m0 = mbk * MB, c0 = cbk * CB;
    const int s_begin = z * a.spw;
    const int s_end = min(a.nslabs, s_begin + a.spw);
    const int hoff = y * a.dh - a.ph;
    const int kreal = a.PR * a.SW;

    // dY: the slab's positions are one contiguous run of r (whole rows, or a
    // segment of one row), so load i of a lane reads position lane/AV + i*APL
    const int a_cv = lane % AV;
    const bool a_ok = m0 + a_cv * 8 < a.Mm;
    const __amdgpu_buffer_rsrc_t dy_rs = buf_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t x_rs = buf_rsrc(a.x, a.x_bytes);
    const uint32_t a_lane = (uint32_t)(((lane / AV) * a.Ktot + gb * a.gkpg + m0 + a_cv * 8) * 2);
    const uint32_t a_step = (uint32_t)(APL * a.Ktot * 2);
    // X: load (q, cc) of a lane reads pixel column cc*PPL + lane/XV of tile row q
    const int x_cv = lane % XV;
    const int x_col = lane / XV;
    const int x_chan = gb * a.gcpg + c0 + x_cv * 8;

    u32x4 ra[NA], rx[NXR][NXC];
    // per-slab load geometry, computed once; the loads themselves are issued
    // in NKS parts, one part per k-step of the previous slab's MFMA stream
    struct SlabGeo {
        uint32_t abase;
        int kvalid, wbase;
        int pix0[NXR];
        bool row_ok[NXR];
    };
    // valid == false gives a geometry whose loads are all out of range (they
    // return zeros without touching memory), so the load stream needs no branch
    auto slab_geo = [&](int slab, bool valid) {
        SlabGeo gq;
        const int sr = slab / a.nseg;
        const int row0 = sr * a.PR, wo0 = (slab - sr * a.nseg) * a.SW;
        const int r0 = row0 * a.Wo + wo0;
        gq.kvalid = valid ? min(kreal, a.SW == a.Wo ? a.NHo * a.Wo - r0 : a.Wo - wo0) : 0;
        gq.abase = a_lane + (uint32_t)(r0 * a.Ktot * 2);
        gq.wbase = wo0 * a.sw - a.pw;
#pragma unroll
        for (int q = 0; q < NXR; ++q) {
            const int row = row0 + q;
            const int n = (int)magic_div((uint32_t)row, a.mHo);
            const int hi = (row - n * a.Ho) * a.sh + hoff;
            gq.row_ok[q] = valid && q < a.PR && row < a.NHo && (unsigned)hi < (unsigned)a.Hi;
            gq.pix0[q] = (n * a.Hi + hi) * a.Wi + gq.wbase + x_col;
        }
        return gq;
    };
    constexpr int NL = NA + NXR * NXC;                 // loads per slab
    auto gload_part = [&](const SlabGeo& gq, int part, int nparts) {
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            if (l * nparts / NL != part) continue;
            if (l < NA) {
                const int k = lane / AV + l * APL;
                ra[l] = buf_load16(dy_rs, (a_ok && k < gq.kvalid) ? gq.abase + l * a_step : kBufOob);
            } else {
                const int q = (l - NA) / NXC, cc = (l - NA) % NXC;
                const int col = cc * PPL + x_col;
                const bool ok = gq.row_ok[q] && col < a.XW && (unsigned)(gq.wbase + col) < (unsigned)a.Wi;
                rx[q][cc] = buf_load16(x_rs, ok ? (uint32_t)(((gq.pix0[q] + cc * PPL) * a.Ctot + x_chan) * 2) : kBufOob);
            }
        }
    };
    // every slot of the wave's tiles is written (out-of-range slots hold zeros);
    // dY chunk a_cv of position k goes to slot a_cv ^ 4*((k >> 1) & 1), and bit 1
    // of k = lane/AV + i*APL is bit 1 of lane/AV for every i
    const int a_slot = ASWZ ? (a_cv ^ (4 * (((lane / AV) >> 1) & 1))) : a_cv;
    uint16_t* sA_lane = sA + (lane / AV) * PA + a_slot * 8;
    uint16_t* sX_lane = sX + x_col * PX + x_cv * 8;
    auto sstore = [&]() {
#pragma unroll
        for (int i = 0; i < NA; ++i) *reinterpret_cast<u32x4*>(sA_lane + i * APL * PA) = ra[i];
#pragma unroll
        for (int q = 0; q < NXR; ++q)
#pragma unroll
            for (int cc = 0; cc < NXC; ++cc)
                *reinterpret_cast<u32x4*>(sX_lane + (q * XWP + cc * PPL) * PX) = rx[q][cc];
    };

    // issue the first slab's loads before the lane tables are built, so that
    // their latency covers the setup arithmetic
    int s = s_begin + wave;
    if (s < s_end) {
        const SlabGeo g0 = slab_geo(s, true);
#pragma unroll
        for (int p = 0; p < NKS; ++p) gload_part(g0, p, NKS);
    }

    // lane geometry of the transposed reads: rows frow (+4), columns fcol..fcol+3
    const int g16 = lane >> 4;
    const int frow = (g16 >> 1) * 8 + ((lane & 15) >> 2);
    const int fcol = (g16 & 1) * 16 + (lane & 3) * 4;
    // pixel (as an LDS element offset) of each reduction row this lane
    // addresses; rows past the slab's positions point at pixel 0 (their dY is 0)
    int xoff[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = ks * 16 + frow + 4 * h;
            const int q = (int)magic_div((uint32_t)k, a.mSW);
            xoff[ks][h] = k < kreal ? (q * XWP + (k - q * a.SW) * a.sw) * PX : 0;
        }

    // the lane's reduction rows share bit 1 (bit 3 of the lane id), so its swizzle
    // swaps the two 32-column fragments of a 64-wide row
    const int a_sw = ASWZ ? ((lane >> 3) & 1) : 0;
    const uint16_t* aread = sA + frow * PA + fcol;
    const uint16_t* bread = sX + fcol;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{0};

    i16x8 af[2][FM], bf[2][FN];
    auto read_frags = [&](int ks, i16x8* fa, i16x8* fb) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = tr_frag(aread + ks * 16 * PA + (i ^ a_sw) * 32, PA);
#pragma unroll
        for (int x = 0; x < XF; ++x)
#pragma unroll
            for (int fc = 0; fc < FC; ++fc) {
                const uint16_t* b = bread + x * PX + fc * 32;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + xoff[ks][0]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + xoff[ks][1]));
                fb[x * FC + fc] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
    };
    for (; s < s_end; s += 4) {
        sstore();
        const bool more = s + 4 < s_end;
        const SlabGeo gn = slab_geo(more ? s + 4 : s, more);
        read_frags(0, af[0], bf[0]);
        // each k-step: the MFMAs of this step interleaved with the fragment
        // reads of the next step and one part of the next slab's global loads,
        // so that LDS latency, VMEM issue and address arithmetic overlap the
        // matrix pipe
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int cur = ks & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < NKS) read_frags(ks + 1, af[cur ^ 1], bf[cur ^ 1]);
            gload_part(gn, ks, NKS);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) mfma_step32<F16>(af[cur][i], bf[cur][j], acc[i][j]);
#pragma unroll
            for (int m = 0; m < FM * FN; ++m) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, 6, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the next iteration's stores must follow this slab's reads
        asm volatile("" ::: "memory");
    }

    // ---- sum the four wave tiles in LDS (fixed order) and store, one tap at a time
    lds_barrier();
    float* red = reinterpret_cast<float*>(smem);
    const int mbase = gb * a.gkpg;
    const int64_t zoff = a.out_mode == OUT_WORKSPACE ? (int64_t)z * a.slice_elems : 0;
#pragma unroll
    for (int x = 0; x < XF; ++x) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int fc = 0; fc < FC; ++fc)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = i * 32 + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
                    const int col = fc * 32 + (lane & 31);
                    red[wave * TILE + row * RP + col] = acc[i][x * FC + fc][v];
                }
        lds_barrier();
        // thread t sums the float4 at row t/(CB/4) + u*(256/(CB/4)), columns
        // (t % (CB/4))*4 .. +3 of this tap's tile, for u = 0, 1, ...
        constexpr int TPR = CB / 4;                 // threads per tile row
        constexpr int RPI = 256 / TPR;              // rows per pass
        const int col = (threadIdx.x % TPR) * 4;
        const int cg = c0 + col;                    // channel inside the merged run
        const int gj = cg / a.cpg;                  // group of this column
        const int glo = gj * a.kpg, ghi = glo + a.kpg;   // its rows (the diagonal block)
        const int64_t e0 = (int64_t)mbase * a.row_len + (y * XF + x) * a.cpg + (cg - gj * a.cpg);
#pragma unroll
        for (int u = 0; u < MB / RPI; ++u) {
            const int row = threadIdx.x / TPR + u * RPI;
            const int o = row * RP + col;
            const f32x4 sum = ((*reinterpret_cast<const f32x4*>(red + o) +
                                *reinterpret_cast<const f32x4*>(red + TILE + o)) +
                               *reinterpret_cast<const f32x4*>(red + 2 * TILE + o)) +
                              *reinterpret_cast<const f32x4*>(red + 3 * TILE + o);
            const int mg = m0 + row;
            if (mg < a.Mm && mg >= glo && mg < ghi) store4(a.out, a.out_mode, zoff + e0 + (int64_t)mg * a.row_len, sum);
        }
        lds_barrier();
    }
}

template <int I, bool F16>
int launch_rs(const Plan& plan, const RowSlabArgs& a, hipStream_t s) {
    constexpr RsInstance r = kRsInstances[I];
    auto k = rowslab_kernel<r.mb, r.cb, r.xf, r.nks, r.nxr, r.nxc, r.pa, r.px, (bool)r.aswz, F16>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, plan.lds_bytes);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(k, dim3(a.total_wg), dim3(256), plan.lds_bytes, s, a);
    return (int)hipGetLastError();
}

template <bool F16>
int launch_rs_t(const Plan& plan, const RowSlabArgs& a, hipStream_t s) {
    static_assert(kNumRsInstances == 5, "dispatch table");
    switch (plan.rs_inst) {
        case 0: return launch_rs<0, F16>(plan, a, s);
        case 1: return launch_rs<1, F16>(plan, a, s);
        case 2: return launch_rs<2, F16>(plan, a, s);
        case 3: return launch_rs<3, F16>(plan, a, s);
        case 4: return launch_rs<4, F16>(plan, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_rowslab(const Plan& plan, const RowSlabArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_rs_t<true>(plan, a, s) : launch_rs_t<false>(plan, a, s);
}

}  // namespace wgrad
