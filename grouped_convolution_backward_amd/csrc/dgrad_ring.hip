// Row-ring backward data (dgrad) of the grouped convolution on gfx950: 2D,
// 3x3 filter, unit stride and dilation.
//
// Per group block the input gradient is the GEMM over (filter tap, output
// channel) of the dgrad kernel in dgrad.hip:
//
//   dX[(n, hi, wi)][c] = sum_{y, x, k} dY[n, hi + ph - y, wi + pw - x][k] * W[k][y][x][c].
//
// Here a workgroup owns one group block and one block of cbd dX channels for
// a split of input rows, and every operand enters it once:
//
// * The block's weights (9 taps x Gm*K/G rows x cbd channels, zero where a
//   row's group differs from a column's) are loaded into LDS once, K-outer
//   like the dgrad kernel's B tile, and read with ds_read_b64_tr_b16
//   (rocm-libraries PR 11602's transposed read for backward data).
// * Input rows are walked four at a time (one per MFMA wave). Input row hi
//   reads dY rows hi + ph - y, y = 0..2, so four consecutive rows read six
//   dY rows and the next four share two of them: dY rows live in an LDS ring
//   and each step stages only the four it adds. Rows are numbered with two
//   padding rows after each image (virtual row v = n*(Hi + 2) + hi), which
//   makes the dY row of every (v, y) the row v + ph - y of the same
//   numbering: the padding rows absorb the image boundaries (they are
//   computed and not stored), so the ring needs no special case there.
// * A dY row is staged [pixel][channel]: tap x of position wi is the pixel
//   wi + 2 - x of the row tile, so the three taps of a row are shifted plain
//   16-byte reads of one slot (the operand already runs along the reduction
//   axis). 16-byte chunks are XOR-swizzled by pixel so that 16 consecutive
//   pixels fall on all banks.
// * Accumulators hold dX^T blocks (weights are the first MFMA operand): a
//   lane holds four consecutive channels of one position, stored as one
//   vector per channel quad.
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;

template <int CBD, int MT, int CH, bool F16>
__global__ __launch_bounds__(384, 1) void dgrad_ring_kernel(const DgradRingArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    constexpr int GK = 8 * CH;                     // merged output channels per group block
    constexpr int KST = GK / 16;                   // 16-channel MFMA k-steps per tap
    constexpr int NT = CBD / 32;                   // 32-channel N tiles
    constexpr int PXL = 64 / CH;                   // pixels one 1 KB dY load fills
    constexpr int WEL = 9 * GK * CBD;              // weight tile elements
    constexpr int NWL = WEL / 512;                 // 1 KB weight loads
    constexpr int RS = kDgRingSlots;
    constexpr int NXLMAX = (32 * MT + 2 + PXL - 1) / PXL;
    constexpr int PPB = 16 / CH;                   // pixels per 256-byte bank row (swizzle period)
    static_assert(WEL % 512 == 0 && GK % 16 == 0, "tile geometry");
    static_assert(6 * NXLMAX <= 63, "vmcnt range of a fresh six-row window");
    uint16_t* const sW = smem;
    uint16_t* const ring = smem + WEL;
    const int slot_el = a.qp * GK;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0..3 rows, 4 weights, 5 dY
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    const int tt = L % a.tiles, z = L / a.tiles;
    const int cbk = tt % a.cblocks, gb = tt / a.cblocks;
    const int c0 = cbk * CBD;
    const int vb = z * a.vpw;
    const int ve = min(a.NV, vb + a.vpw);
    const int nsteps = (ve - vb + 3) / 4;

    // the pixel-dependent chunk swizzle of the dY ring
    auto swz = [&](int q) { return (q / PPB) & (CH - 1); };

    if (wave == 4) {
        // weights: row r = tap*GK + k' (k' = gi*kpg + k), channels c' of the
        // block; 64-channel rows XOR-swizzle chunks by bit 1 of the row, as
        // the row-slab kernel's dY tile
        const u32x4 w_desc = buf_desc(a.w, a.w_bytes);
        constexpr int WCH = CBD / 8, WR = 64 / WCH;
        const int jr = lane / WCH;
#pragma unroll 4
        for (int l = 0; l < NWL; ++l) {
            const int row = l * WR + jr;
            const int tap = row / GK, kk = row - tap * GK;
            const int chunk = (lane % WCH) ^ (CBD == 64 ? 4 * ((row >> 1) & 1) : 0);
            const int cc = c0 + chunk * 8;
            const int gi = (int)magic_div((uint32_t)kk, a.mkpg), gj = (int)magic_div((uint32_t)cc, a.mcpg);
            const int k = kk - gi * a.kpg, c = cc - gj * a.cpg;
            const uint32_t off = (uint32_t)(((((gb * a.Gm + gi) * a.kpg + k) * 9 + tap) * a.cpg + c) * 2);
            dma_load16(w_desc, lds_addr(sW + l * 512), gi == gj ? off : kBufOob);
            if ((l & 31) == 31) __builtin_amdgcn_s_waitcnt(kWaitVm<16>);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
        __builtin_amdgcn_s_barrier();
        for (int s = 0; s < nsteps; ++s) __builtin_amdgcn_s_barrier();
        return;
    }
    if (wave == 5) {
        // dY rows: lane t of a load fills pixel t / CH, chunk slot t % CH with
        // source chunk slot ^ swz(pixel); per-lane byte offsets within a dY row
        const u32x4 dy_desc = buf_desc(a.dy, a.dy_bytes);
        const int jq = lane / CH, sl = lane % CH;
        uint32_t off[NXLMAX];
#pragma unroll
        for (int l = 0; l < NXLMAX; ++l) {
            const int q = l * PXL + jq;
            const int wo = q - 2 + a.pw;
            const int chunk = sl ^ swz(q);
            off[l] = (unsigned)wo < (unsigned)a.Wo ? (uint32_t)((wo * a.Ktot + gb * a.gkpg + chunk * 8) * 2) : kBufOob;
        }
        const uint32_t row_bytes = (uint32_t)(a.Wo * a.Ktot * 2);
        // virtual dY row u (of image u / VR, row u % VR; rows past Ho and
        // negative u are zeros) into ring slot (u + 2) % RS
        auto stage = [&](int u) {
            bool ok = u >= 0;
            uint32_t rb = 0;
            if (ok) {
                const int n = (int)magic_div((uint32_t)u, a.mVR);
                const int ho = u - n * a.VR;
                ok = n < a.N && ho < a.Ho;
                rb = (uint32_t)(n * a.Ho + ho) * row_bytes;
            }
            uint16_t* dst = ring + ((u + 2) % RS) * slot_el;
#pragma unroll
            for (int l = 0; l < NXLMAX; ++l)
                if (l < a.nxl) dma_load16(dy_desc, lds_addr(dst + l * 512), ok ? rb + off[l] : kBufOob);
        };
        // step s covers virtual rows v0 = vb + 4s .. v0 + 3, whose dY rows are
        // v0 + ph - 2 .. v0 + ph + 3; each later step adds its last four
        if (nsteps > 0)
            for (int j = -2; j < 4; ++j) stage(vb + a.ph + j);
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
        __builtin_amdgcn_s_barrier();
        for (int s = 0; s < nsteps; ++s) {
            if (s + 1 < nsteps)
                for (int j = 0; j < 4; ++j) stage(vb + 4 * (s + 1) + a.ph + j);
            __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
            __builtin_amdgcn_s_barrier();
        }
        return;
    }

    // ---- MFMA waves: wave w computes virtual row vb + 4s + w of each step
    const int g16 = lane >> 4;
    const int frow = (g16 >> 1) * 8 + ((lane & 15) >> 2);
    const int fcol = (g16 & 1) * 16 + (lane & 3) * 4;
    const int w_sw = CBD == 64 ? ((lane >> 3) & 1) : 0;
    const int kg = lane >> 5;                      // 8-channel group of the lane's k values
    // per M tile and tap x: element offset of the lane's dY pixel in a slot
    // (positions past Wi read pixel 2 - x, their results are not stored) and
    // its chunk swizzle
    int qoff[MT][3], qsw[MT][3];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int pos = i * 32 + (lane & 31);
        const int pb = pos < a.Wi ? pos : 0;
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int q = pb + 2 - x;
            qoff[i][x] = q * GK;
            qsw[i][x] = swz(q);
        }
    }

    __builtin_amdgcn_s_barrier();
    for (int s = 0; s < nsteps; ++s) {
        const int v = vb + 4 * s + wave;
        const uint16_t* sY[3];
#pragma unroll
        for (int y = 0; y < 3; ++y) sY[y] = ring + ((v + a.ph - y + 2) % RS) * slot_el;

        f32x16 acc[MT][NT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{0};
        // k-steps t = (y*3 + x)*KST + ks, operands read one k-step ahead
        constexpr int T = 9 * KST;
        i16x8 fw[2][NT], fy[2][MT];
        auto read_t = [&](int t, int b) {
            const int tap = t / KST, ks = t % KST, y = tap / 3, x = tap % 3;
            const uint16_t* wr = sW + (tap * GK + ks * 16 + frow) * CBD;
#pragma unroll
            for (int j = 0; j < NT; ++j) fw[b][j] = tr_frag(wr + (j ^ w_sw) * 32 + fcol, CBD);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int chunk = (ks * 2 + kg) ^ qsw[i][x];
                fy[b][i] = *reinterpret_cast<const i16x8*>(sY[y] + qoff[i][x] + chunk * 8);
            }
        };
        read_t(0, 0);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int cur = t & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < T) read_t(t + 1, cur ^ 1);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) mfma_step32<F16>(fw[cur][j], fy[cur][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- store the row. Lane l holds channels j*32 + 8*vq + 4*kg .. +3 of
        // position i*32 + l%32; one lane swap per register pair gives the
        // lower half-wave whole 8-channel groups 2p and the upper half-wave
        // groups 2p + 1, so each lane stores 16 contiguous bytes (bf16/fp16)
        const int n = (int)magic_div((uint32_t)v, a.mVR);
        const int hi = v - n * a.VR;
        if (v < ve && hi < a.Hi) {
            const int64_t rowe = ((int64_t)(n * a.Hi + hi) * a.Wi) * a.Ctot + gb * a.gcpg + c0 + 8 * kg;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int pos = i * 32 + (lane & 31);
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                    for (int pq = 0; pq < 2; ++pq) {
                        const f32x16& c = acc[i][j];
                        float lo[4], hi4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[8 * pq + e]),
                                                                             __float_as_uint(c[8 * pq + 4 + e]), false, false);
                            lo[e] = __uint_as_float(sw[0]);
                            hi4[e] = __uint_as_float(sw[1]);
                        }
                        if (pos >= a.Wi) continue;
                        const int64_t e0 = rowe + (int64_t)pos * a.Ctot + j * 32 + 16 * pq;
                        if (a.out_mode == OUT_FP32) {
                            float* o = static_cast<float*>(a.dx) + e0;
                            *reinterpret_cast<f32x4*>(o) = f32x4{lo[0], lo[1], lo[2], lo[3]};
                            *reinterpret_cast<f32x4*>(o + 4) = f32x4{hi4[0], hi4[1], hi4[2], hi4[3]};
                        } else {
                            u32x4 p;
                            if (a.out_mode == OUT_BF16) {
                                // one v_cvt_pk_bf16_f32 per pair
#pragma unroll
                                for (int h = 0; h < 2; ++h) {
                                    p[h] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo[2 * h], (__bf16)lo[2 * h + 1]});
                                    p[2 + h] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)hi4[2 * h], (__bf16)hi4[2 * h + 1]});
                                }
                            } else {
#pragma unroll
                                for (int h = 0; h < 2; ++h) {
                                    p[h] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo[2 * h]) |
                                           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo[2 * h + 1]) << 16);
                                    p[2 + h] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi4[2 * h]) |
                                               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi4[2 * h + 1]) << 16);
                                }
                            }
                            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.dx) + e0) = p;
                        }
                    }
            }
        }
        // the step's rows are consumed and the next step's dY rows have landed
        lds_barrier();
    }
}

template <int I, bool F16>
int launch_dgr_i(const Plan& plan, const DgradRingArgs& a, hipStream_t s) {
    constexpr DgradRingInstance r = kDgRingInstances[I];
    auto k = dgrad_ring_kernel<r.cbd, r.mt, r.ch, F16>;
    const int lds = dg_ring_lds_bytes(r, a.qp);
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(k, dim3(a.total_wg), dim3(384), lds, s, a);
    return (int)hipGetLastError();
}

template <bool F16>
int launch_dgr_t(const Plan& plan, const DgradRingArgs& a, hipStream_t s) {
    static_assert(kNumDgRingInstances == 8, "dispatch table");
    switch (plan.dg_ring) {
        case 0: return launch_dgr_i<0, F16>(plan, a, s);
        case 1: return launch_dgr_i<1, F16>(plan, a, s);
        case 2: return launch_dgr_i<2, F16>(plan, a, s);
        case 3: return launch_dgr_i<3, F16>(plan, a, s);
        case 4: return launch_dgr_i<4, F16>(plan, a, s);
        case 5: return launch_dgr_i<5, F16>(plan, a, s);
        case 6: return launch_dgr_i<6, F16>(plan, a, s);
        case 7: return launch_dgr_i<7, F16>(plan, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_dgrad_ring(const Plan& plan, const DgradRingArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_dgr_t<true>(plan, a, s) : launch_dgr_t<false>(plan, a, s);
}

}  // namespace wgrad
