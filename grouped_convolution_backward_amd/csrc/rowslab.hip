// Row-slab MFMA kernel for grouped convolution backward-weight on gfx950.
//
// The implicit GEMM of the Composable Kernel wgrad page (A = dY rows, B = X
// gathered per filter tap, reduction over r = (n*Ho + ho)*Wo + wo), tiled so
// that X is staged once per output row instead of once per tap:
//
// * A workgroup owns one filter row (z, y) of one (group block, M block,
//   C block) tile and every filter column x of that row: its output tile is
//   MB x (X*CB), and for one output row (n, do, ho) it needs exactly one
//   input row (n, di, hi). 2D is the depth-1 case, 1D also height 1.
// * The reduction runs over slabs of PR output rows x SW output columns. A
//   slab's dY rows are staged K-outer ([position][channel]) and its input
//   rows as a pixel tile ([row][pixel][channel]); tap x of position k is a
//   fixed pixel shift of k's own pixel, so the three (or five) taps of the
//   row are shifted reads of one tile. For stride 2 the tile holds the even
//   input columns, then the odd ones, so every tap still reads consecutive
//   pixels.
// * MFMA operands come from the CDNA4 transposed LDS read
//   ds_read_b64_tr_b16 (rocm-libraries PR 11602): each lane supplies the
//   address of its own reduction row, which here is a per-lane pixel offset,
//   so the tile needs no per-tap copy and nothing is transposed on store.
// * Tiles go from HBM to LDS with buffer loads that write LDS directly (16
//   bytes per lane, lane-major), so no registers stage them and no LDS store
//   instructions compete with the fragment reads.
//   16-byte chunks are XOR-swizzled by bit 1 of the row (64-channel rows), so
//   the four rows a 16-lane group reads land on all banks; the loads apply
//   the swizzle by choosing which source chunk each lane fetches.
// * The slabs are dealt to the S splits in turn (split z takes z, z + S,
//   z + 2S, ..., or the same for groups of four consecutive slabs on 3D
//   filters): at any moment the splits read neighbouring slabs, which
//   measured faster per step than one contiguous range per split.
// * The workgroup runs four slab streams; stream p takes every fourth slab of
//   the workgroup's split into its own nb LDS buffers. A stream's MFMA waves
//   (two, each holding 32 of 64 channels, or one for 32-channel blocks) hold
//   the workgroup tile in registers and never touch vector memory: one
//   producer wave per stream issues all of its loads and waits for them, so
//   a stalled load issue never holds up an MFMA. One workgroup barrier per
//   slab hands slab i + 1 to the MFMA waves and slab i's buffer back to the
//   producer, which refills it nb - 1 slabs ahead.
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
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(out) + e));
    }
}

// s_waitcnt that leaves at most later * PER of this wave's vector-memory
// loads outstanding, for later in 0..MAXL (immediate operands need a branch)
template <int MAXL, int PER>
__device__ __forceinline__ void vm_wait_slabs(int later) {
    if (MAXL >= 2 && later >= 2) __builtin_amdgcn_s_waitcnt(kWaitVm<(MAXL >= 2 ? 2 * PER : 0)>);
    else if (MAXL >= 1 && later >= 1) __builtin_amdgcn_s_waitcnt(kWaitVm<PER>);
    else __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
}

template <int MB, int CB, int XF, int NKS, int NXR, int XWP, int STRIDE, int NB, int GS, int WPS, bool F16>
__global__ __launch_bounds__(256 * (WPS + 1), 1) void rowslab_kernel(const RowSlabArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    constexpr int NT = 256 * WPS;                  // consumer threads (the MFMA waves)
    constexpr int FM = MB / 32, FC = CB / 32;
    constexpr int FCW = FC / WPS, FNW = XF * FCW;  // 32-channel blocks and B fragments per wave
    constexpr int KS = 16 * NKS;                   // positions per slab (padded)
    constexpr int ACH = MB / 8, XCH = CB / 8;      // 16-byte chunks per position / pixel
    constexpr int RA = 64 / ACH, RX = 64 / XCH;    // rows one 1 KB load fills
    constexpr int NA = KS / RA, NXI = NXR * XWP / RX;
    constexpr int NL = NA + NXI;                   // loads per slab
    constexpr int ABUF = KS * MB;                  // elements of the dY tile
    constexpr int BUF = ABUF + NXR * XWP * CB;     // elements of one slab buffer
    constexpr int HALF = XWP / 2;                  // stride 2: odd input columns start here
    constexpr int RP = CB + 4;                     // row pitch of the reduction tile (floats)
    constexpr int TILE = MB * RP;
    static_assert(KS % RA == 0 && XWP % RX == 0 && (STRIDE == 1 || HALF % RX == 0), "slab geometry");
    static_assert((NB - 1) * NL <= 63, "vmcnt range");
    static_assert(NB >= 2 && NB <= 4, "slab buffers");
    static_assert(MB == 64 || MB == 32, "M block");
    static_assert(FC % WPS == 0 && (WPS == 1 || CB == 64), "channel split between the waves of a slab");
    static_assert(NKS % 2 == 0, "fragment double buffer restarts at 0 each slab");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool producer = wave >= 4 * WPS;         // one load-issuing wave per stream
    const int pair = wave & 3;                     // slab stream of this wave
    const int half = producer ? 0 : wave >> 2;     // its part of the channel block (WPS = 2)
    uint16_t* wbuf = smem + pair * NB * BUF;

    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    int t = L % a.tiles;
    const int z = L / a.tiles;
    const int y = t % a.Y;                         // filter row (z, y) = z*Yf + y
    t /= a.Y;
    const int cbk = t % a.cblocks;
    t /= a.cblocks;
    const int mbk = t % a.mblocks;
    const int gb = t / a.mblocks;
    const int m0 = mbk * MB, c0 = cbk * CB;
    // slabs of this split, interleaved with the other splits in groups of GS
    // consecutive slabs: groups z, z + S, z + 2S, ... (at any moment the
    // splits read neighbouring slabs)
    static_assert(GS == 1 || GS == 2 || GS == 4, "slab group");
    constexpr int GPR = 4 / GS;                    // groups per round of the four streams
    const int ngroups = (a.nslabs + GS - 1) / GS;
    const int mygroups = z < ngroups ? (ngroups - z + a.S - 1) / a.S : 0;
    const int fz = y / a.Yf, fy = y - fz * a.Yf;
    const int doff = fz * a.dd - a.pd, hoff = fy * a.dh - a.ph;
    const int kreal = a.PR * a.SW;
    const u32x4 dy_desc = buf_desc(a.dy, a.dy_bytes);
    const u32x4 x_desc = buf_desc(a.x, a.x_bytes);

    // lane roles in the loads: lane -> (row ja of the 1 KB block, LDS slot);
    // the slot holds source chunk slot ^ swizzle(row), and bit 1 of the row is
    // bit 1 of ja for every block (a block starts on a multiple of 8 rows)
    const int ja = lane / ACH;
    const int a_chunk = (lane % ACH) ^ (MB == 64 ? 4 * ((ja >> 1) & 1) : 0);
    const bool a_ok = m0 + a_chunk * 8 < a.Mm;
    const uint32_t a_lane = (uint32_t)((ja * a.Ktot + gb * a.gkpg + m0 + a_chunk * 8) * 2);
    const uint32_t a_step = (uint32_t)(RA * a.Ktot * 2);
    const int jx = lane / XCH;
    const int x_chunk = (lane % XCH) ^ (CB == 64 ? 4 * ((jx >> 1) & 1) : 0);
    const int x_chan = gb * a.gcpg + c0 + x_chunk * 8;

    // per-slab load geometry; issue_part then issues this wave's share
    // (loads l with l % WPS == half) of loads [l0, l1) of the slab into buffer
    // bsel. Out-of-range lanes write zeros, so padding needs no branch.
    struct SlabGeo {
        uint32_t abase;
        int kvalid, wbase;
        int pixrow[NXR];
        bool rowok[NXR];
    };
    auto slab_geo = [&](int slab) {
        SlabGeo gq;
        const int sr = (int)magic_div((uint32_t)slab, a.mSeg);
        const int row0 = sr * a.PR, wo0 = (slab - sr * a.nseg) * a.SW;
        const int r0 = row0 * a.Wo + wo0;
        gq.kvalid = min(kreal, a.SW == a.Wo ? a.NHo * a.Wo - r0 : a.Wo - wo0);
        gq.abase = a_lane + (uint32_t)(r0 * a.Ktot * 2);
        gq.wbase = wo0 * a.sw - a.pw;
#pragma unroll
        for (int q = 0; q < NXR; ++q) {
            // output row = (n*Do + do)*Ho + ho
            const int row = row0 + q;
            const int b = (int)magic_div((uint32_t)row, a.mHo);
            const int n = (int)magic_div((uint32_t)b, a.mDo);
            const int di = (b - n * a.Do) * a.sd + doff;
            const int hi = (row - b * a.Ho) * a.sh + hoff;
            gq.rowok[q] = q < a.PR && row < a.NHo && (unsigned)di < (unsigned)a.Di && (unsigned)hi < (unsigned)a.Hi;
            gq.pixrow[q] = ((n * a.Di + di) * a.Hi + hi) * a.Wi;
        }
        return gq;
    };
    auto issue_part = [&](const SlabGeo& gq, int bsel, int l0, int l1) {
        uint16_t* sA = wbuf + bsel * BUF;
        uint16_t* sX = sA + ABUF;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            if (l < l0 || l >= l1) continue;           // l0, l1 are compile-time at every call
            if (l < NA) {
                const bool ok = a_ok && l * RA + ja < gq.kvalid;
                dma_load16(dy_desc, lds_addr(sA + l * RA * MB), ok ? gq.abase + l * a_step : kBufOob);
            } else {
                const int i = l - NA;
                const int q = (i * RX) / XWP;
                const int pj = (i * RX) % XWP + jx;
                const int off = STRIDE == 1 ? pj : (pj < HALF ? 2 * pj : 2 * (pj - HALF) + 1);
                const int col = gq.wbase + off;
                const bool ok = gq.rowok[q] && off < a.XW && (unsigned)col < (unsigned)a.Wi;
                dma_load16(x_desc, lds_addr(sX + i * RX * CB),
                           ok ? (uint32_t)(((gq.pixrow[q] + col) * a.Ctot + x_chan) * 2) : kBufOob);
            }
        }
    };
    // loads of one slab this wave issues (compile-time per half)
    constexpr int NLW0 = (NL + WPS - 1) / WPS, NLW1 = NL / WPS;

    // this stream's slabs: slab pair % GS of the split's groups
    // pair / GS + GPR*i, i < cnt (the last group of all may be short). Every
    // wave of the workgroup passes the same cnt_max + 1 barriers.
    const int q = pair / GS, rr = pair % GS;
    int cnt = mygroups > q ? (mygroups - q + GPR - 1) / GPR : 0;
    if (GS > 1 && cnt > 0 && GS * (z + (q + (cnt - 1) * GPR) * a.S) + rr >= a.nslabs) --cnt;
    const int cnt_max = (mygroups + GPR - 1) / GPR;
    auto slab_of = [&](int i) { return GS * (z + (q + i * GPR) * a.S) + rr; };
    if (producer) {
        // issue slabs 0 .. NB-2, then before barrier i+1 issue slab i+NB-1
        // (into the buffer slab i-1 left) and wait for slab i+1
#pragma unroll
        for (int i = 0; i < NB - 1; ++i)
            if (i < cnt) issue_part(slab_geo(slab_of(i)), i, 0, NL);
        if (cnt > 0) vm_wait_slabs<NB - 2, NL>(min(cnt - 1, NB - 2));
        __builtin_amdgcn_s_barrier();
        for (int i = 0; i < cnt_max; ++i) {
            if (i + NB - 1 < cnt) issue_part(slab_geo(slab_of(i + NB - 1)), (i + NB - 1) % NB, 0, NL);
            if (i + 1 < cnt) vm_wait_slabs<NB - 2, NL>(min(cnt - 2 - i, NB - 2));
            __builtin_amdgcn_s_barrier();
        }
        // the epilogue's barriers
        lds_barrier();
#pragma unroll
        for (int x = 0; x < XF; ++x) {
            lds_barrier();
            lds_barrier();
        }
        return;
    }

    // lane geometry of the transposed reads: rows frow (+4), columns fcol..fcol+3
    const int g16 = lane >> 4;
    const int frow = (g16 >> 1) * 8 + ((lane & 15) >> 2);
    const int fcol = (g16 & 1) * 16 + (lane & 3) * 4;
    // LDS element offset (inside a buffer's X tile) of the pixel each
    // reduction row of this lane reads for tap x, swizzle included, for the
    // wave's first 32-channel block (for 64-channel rows the other block is
    // the same address with bit 5 flipped); rows past the slab's positions
    // read pixel 0, whose products are zero because their dY rows are zero
    constexpr int XOFF_N = CB == 64 ? XF : 1;
    int xaddr[NKS][2][XOFF_N];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = ks * 16 + frow + 4 * h;
            const int q = (int)magic_div((uint32_t)k, a.mSW);
            const int col = k - q * a.SW;
            const int base = k < kreal ? q * XWP + col : 0;
#pragma unroll
            for (int x = 0; x < XOFF_N; ++x) {
                const int j = base + (STRIDE == 1 ? x : (x & 1) * HALF + (x >> 1));
                xaddr[ks][h][x] = CB == 64 ? (j * CB + (((j >> 1) & 1) << 5) + fcol) ^ ((half * FCW) << 5)
                                           : j * CB + fcol;
            }
        }

    // the lane's reduction rows share bit 1 (bit 3 of the lane id), so the dY
    // swizzle swaps the two 32-column fragments of a 64-wide row
    const int a_sw = MB == 64 ? ((lane >> 3) & 1) : 0;

    // X fragments are the MFMA's first operand and dY fragments its second,
    // so acc[i][j] holds the transposed 32x32 block: each lane's registers
    // 4q..4q+3 are four consecutive dW columns of one dW row, which the
    // epilogue stores to LDS as one 16-byte write.
    f32x16 acc[FM][FNW];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FNW; ++j) acc[i][j] = f32x16{0};

    i16x8 af[2][FM], bf[2][FNW];
    auto read_frags = [&](const uint16_t* sA, int ks, i16x8* fa, i16x8* fb) {
        const uint16_t* sX = sA + ABUF;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = tr_frag(sA + (ks * 16 + frow) * MB + (i ^ a_sw) * 32 + fcol, MB);
#pragma unroll
        for (int x = 0; x < XF; ++x)
#pragma unroll
            for (int fc = 0; fc < FCW; ++fc) {
                int o0, o1;
                if constexpr (CB == 64) {
                    o0 = xaddr[ks][0][x] ^ (fc << 5);
                    o1 = xaddr[ks][1][x] ^ (fc << 5);
                } else {
                    const int dx = (STRIDE == 1 ? x : (x & 1) * HALF + (x >> 1)) * CB + fc * 32;
                    o0 = xaddr[ks][0][0] + dx;
                    o1 = xaddr[ks][1][0] + dx;
                }
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sX + o0));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sX + o1));
                fb[x * FCW + fc] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
    };
    __builtin_amdgcn_s_barrier();
    for (int i = 0; i < cnt_max; ++i) {
        if (i < cnt) {
            const uint16_t* sA = wbuf + (i % NB) * BUF;
            read_frags(sA, 0, af[0], bf[0]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int cur = ks & 1;
                __builtin_amdgcn_sched_barrier(0);
                if (ks + 1 < NKS) read_frags(sA, ks + 1, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
                for (int j = 0; j < FNW; ++j)
#pragma unroll
                    for (int i2 = 0; i2 < FM; ++i2) mfma_step32<F16>(bf[cur][j], af[cur][i2], acc[i2][j]);
#pragma unroll
                for (int m = 0; m < FM * FNW; ++m) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // slab i is consumed (its buffer may be refilled) and slab i + 1 has landed
        lds_barrier();
    }

    // ---- sum the four stream tiles in LDS (fixed order) and store, as many
    // taps per pass as the slab buffers hold (two on the 3-tap 64x64 shapes:
    // one barrier pair less than a tap at a time)
    constexpr int TPP0 = (4 * NB * BUF * 2) / (4 * TILE * 4);
    constexpr int TPP = TPP0 < 1 ? 1 : TPP0 > XF ? XF : TPP0;   // taps per pass
    static_assert(TPP == 1 || TPP * 4 * TILE * 4 <= 4 * NB * BUF * 2, "pass tiles fit the slab buffers");
    lds_barrier();
    float* red = reinterpret_cast<float*>(smem);
    const int mbase = gb * a.gkpg;
    // this workgroup's workspace slice (partials only)
    const __amdgpu_buffer_rsrc_t ws = buf_rsrc(static_cast<float*>(a.out) + (int64_t)z * a.slice_elems,
                                               4u * (uint32_t)a.slice_elems);
    // thread t sums the float4 at row t/(CB/4) + u*(NT/(CB/4)), columns
    // (t % (CB/4))*4 .. +3 of a tap's tile, for u = 0, 1, ...
    constexpr int TPR = CB / 4;                     // threads per tile row
    constexpr int RPI = NT / TPR;                   // rows per pass
    static_assert(MB % RPI == 0, "reduction passes");
    static_assert(NT % TPR == 0, "consumer threads cover whole rows");
    const int col = (threadIdx.x % TPR) * 4;
    const int cg = c0 + col;
    const int gj = cg / a.cpg;                      // group of this column
    const int glo = gj * a.kpg, ghi = glo + a.kpg;  // its rows (the diagonal block)
#pragma unroll
    for (int x0 = 0; x0 < XF; x0 += TPP) {
#pragma unroll
        for (int tp = 0; tp < TPP; ++tp) {
            const int x = x0 + tp;
            if (x >= XF) break;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int fc = 0; fc < FCW; ++fc)
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        const int row = i * 32 + (lane & 31);
                        const int cc = (half * FCW + fc) * 32 + 8 * vq + 4 * (lane / 32);
                        const f32x16& c = acc[i][x * FCW + fc];
                        *reinterpret_cast<f32x4*>(red + (tp * 4 + pair) * TILE + row * RP + cc) =
                            f32x4{c[4 * vq], c[4 * vq + 1], c[4 * vq + 2], c[4 * vq + 3]};
                    }
        }
        lds_barrier();
#pragma unroll
        for (int tp = 0; tp < TPP; ++tp) {
            const int x = x0 + tp;
            if (x >= XF) break;
            const float* rt = red + tp * 4 * TILE;
            const int64_t e0 = (int64_t)mbase * a.row_len + (y * XF + x) * a.cpg + (cg - gj * a.cpg);
#pragma unroll
            for (int u = 0; u < MB / RPI; ++u) {
                const int row = threadIdx.x / TPR + u * RPI;
                const int o = row * RP + col;
                const f32x4 sum = ((*reinterpret_cast<const f32x4*>(rt + o) +
                                    *reinterpret_cast<const f32x4*>(rt + TILE + o)) +
                                   *reinterpret_cast<const f32x4*>(rt + 2 * TILE + o)) +
                                  *reinterpret_cast<const f32x4*>(rt + 3 * TILE + o);
                const int mg = m0 + row;
                if (mg < a.Mm && mg >= glo && mg < ghi) {
                    if (a.out_mode == OUT_WORKSPACE) store_partial4(ws, e0 + (int64_t)mg * a.row_len, sum);
                    else store4(a.out, a.out_mode, e0 + (int64_t)mg * a.row_len, sum);
                }
            }
        }
        // the next pass overwrites the tiles
        if (x0 + TPP < XF) lds_barrier();
    }
}

template <int I, bool F16>
int launch_rs(const Plan& plan, const RowSlabArgs& a, hipStream_t s) {
    constexpr RsInstance r = kRsInstances[I];
    constexpr int wps = rs_waves_per_slab(r);
    auto k = rowslab_kernel<r.mb, r.cb, r.xf, r.nks, r.nxr, r.xwp, r.stride, r.nb, r.gs, wps, F16>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, plan.lds_bytes);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(k, dim3(a.total_wg), dim3(256 * (wps + 1)), plan.lds_bytes, s, a);
    return (int)hipGetLastError();
}

template <bool F16>
int launch_rs_t(const Plan& plan, const RowSlabArgs& a, hipStream_t s) {
    static_assert(kNumRsInstances == 9, "dispatch table");
    switch (plan.rs_inst) {
        case 0: return launch_rs<0, F16>(plan, a, s);
        case 1: return launch_rs<1, F16>(plan, a, s);
        case 2: return launch_rs<2, F16>(plan, a, s);
        case 3: return launch_rs<3, F16>(plan, a, s);
        case 4: return launch_rs<4, F16>(plan, a, s);
        case 5: return launch_rs<5, F16>(plan, a, s);
        case 6: return launch_rs<6, F16>(plan, a, s);
        case 7: return launch_rs<7, F16>(plan, a, s);
        case 8: return launch_rs<8, F16>(plan, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_rowslab(const Plan& plan, const RowSlabArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_rs_t<true>(plan, a, s) : launch_rs_t<false>(plan, a, s);
}

}  // namespace wgrad
