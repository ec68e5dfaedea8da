// Filter-row ring MFMA kernel for grouped convolution backward-weight on
// gfx950 (2D, 3x3 filter, dilation 1).
//
// The implicit GEMM of the Composable Kernel wgrad page (A = dY rows, B = X
// gathered per filter tap, reduction over r = (n*Ho + ho)*Wo + wo), tiled so
// that every input row and every dY row enters a workgroup once:
//
// * A workgroup owns one (group block, M block, 32-channel C block) tile and
//   all nine taps: its output tile is MB x (3*3*32). Wave y (0..2) holds the
//   MB x (3*32) block of filter row y in registers; two more waves issue the
//   loads, one the dY rows and one the input rows, each counting only its
//   own outstanding loads, so more rows can be in flight.
// * The reduction runs over whole output rows (n, ho) of the workgroup's
//   split, one at a time. Output row ho reads input rows ho*sh - ph + y for
//   y = 0..2, so consecutive output rows of one image share 3 - sh of them.
//   Input rows live in an LDS ring of 3*nb slots: each output row stages its
//   dY row and only the input rows the previous output row did not already
//   stage (all three at an image start or at the start of the split), and
//   wave y reads the slot of its own window row. Within the row, tap x of
//   position k is the pixel k + x (w-stride 1), or for w-stride 2 a pixel of
//   the even or odd half of the row tile, so the three taps are shifted
//   transposed reads of one slot, as in the row-slab kernel.
// * Output rows are handed over rps at a time (one workgroup barrier per
//   step), and loads run nb - 1 steps ahead. An output row issues its dY
//   loads and one group of loads per newly staged input row, so the count
//   varies; the waits assume the smallest count (one new row), which waits at
//   least for every load of the step about to be computed. A last step past
//   the split's end is padded with zero rows (zero dY, zero new input rows),
//   which add nothing.
// * w-stride 1: a lane's operand for tap x is its tap-0 operand moved x
//   positions along the reduction: the eight positions a lane holds continue
//   in the lane 32 above it (and, for the upper half, in the next k-step), so
//   taps 1 and 2 are built in registers from the tap-0 fragment with one
//   cross-half lane swap (v_permlane32_swap) and 16-bit funnel shifts,
//   instead of two more LDS reads each. Past a row's last k-step the missing
//   positions are zero: they meet only reduction rows past the row's end,
//   whose dY is zero.
// * MFMA operands come from ds_read_b64_tr_b16 (rocm-libraries PR 11602).
//   X fragments are the first operand, so each lane's accumulators are four
//   consecutive dW columns of one dW row. The three waves' tiles are
//   disjoint (no cross-wave reduction); they are gathered in LDS and stored
//   as whole 32-channel runs of one tap (rows of a tile are a dW row apart,
//   so stores straight from registers would write 32-byte pieces of 32
//   scattered lines per instruction). Merged groups (PR 12359) store only
//   their diagonal blocks.
// * Compared with one filter row per workgroup, per-workgroup traffic into
//   LDS drops about threefold for the same work.
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;

// s_waitcnt that leaves at most min(later, MAXL) * PER of this wave's
// vector-memory loads outstanding (immediate operands need a branch)
template <int MAXL, int PER>
__device__ __forceinline__ void vm_wait_rows(int later) {
    if constexpr (MAXL > 0) {
        if (later >= MAXL) {
            __builtin_amdgcn_s_waitcnt(kWaitVm<MAXL * PER>);
            return;
        }
        vm_wait_rows<MAXL - 1, PER>(later);
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    }
}

template <int MB, int NKS, int XWP, int STRIDE, int NB, int RPS, bool F16>
__global__ __launch_bounds__(320, 1) void ring_kernel(const RingArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    constexpr int CB = kRingCB;
    constexpr int FM = MB / 32;
    constexpr int KS = 16 * NKS;                   // positions per output row (padded)
    constexpr int ACH = MB / 8, XCH = CB / 8;      // 16-byte chunks per position / pixel
    constexpr int RA = 64 / ACH, RX = 64 / XCH;    // rows one 1 KB load fills
    constexpr int NA = KS / RA, NXL = XWP / RX;
    // loads per output row: NA dY loads (one producer), NXL per newly staged
    // input row (the other): one row, or three at a fresh window
    constexpr int ABUF = KS * MB;                  // elements of one dY buffer
    constexpr int XROW = XWP * CB;                 // elements of one ring slot
    constexpr int NBR = NB * RPS;                  // dY buffers (one per output row)
    constexpr int RS = 3 * NBR;                    // ring slots
    constexpr int HALF = XWP / 2;                  // w-stride 2: odd input columns start here
    static_assert(KS % RA == 0 && XWP % RX == 0 && (STRIDE == 1 || HALF % RX == 0), "row geometry");
    static_assert((NB - 1) * RPS * NA <= 63 && (NB - 1) * RPS * 3 * NXL <= 63, "vmcnt range");
    static_assert(NB >= 2, "dY buffers");
    static_assert(NKS % 2 == 0, "fragment double buffer restarts at 0 each row");
    static_assert(MB == 32 || MB == 64, "M block");
    uint16_t* const sA0 = smem;                    // NBR dY buffers
    uint16_t* const ring = smem + NBR * ABUF;      // RS slots

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0..2 filter row, 3 and 4 loads

    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    int t = L % a.tiles;
    const int z = L / a.tiles;
    const int cbk = t % a.cblocks;
    t /= a.cblocks;
    const int mbk = t % a.mblocks;
    const int gb = t / a.mblocks;
    const int m0 = mbk * MB, c0 = cbk * CB;
    const int r_begin = z * a.rpw;
    const int cnt = max(0, min(a.NHo, r_begin + a.rpw) - r_begin);
    const int nsteps = (cnt + RPS - 1) / RPS;
    const int n0 = (int)magic_div((uint32_t)r_begin, a.mHo);

    // output row j of the split: image n, row ho, and the ring position of
    // its window's first row (it advances by sh within an image and by 3,
    // a fresh window, at each image start)
    auto row_of = [&](int j, int& n, int& ho) {
        const int r = r_begin + j;
        n = (int)magic_div((uint32_t)r, a.mHo);
        ho = r - n * a.Ho;
        return j * a.sh + (n - n0) * (3 - a.sh);
    };

    if (wave >= 3) {
        const bool dy_part = wave == 3;            // wave 3 loads dY rows, wave 4 input rows
        const u32x4 dy_desc = buf_desc(a.dy, a.dy_bytes);
        const u32x4 x_desc = buf_desc(a.x, a.x_bytes);
        // lane roles, as in the row-slab kernel: dY chunks of 64-channel rows
        // are XOR-swizzled by bit 1 of the position; 32-channel pixels are not
        const int ja = lane / ACH;
        const int a_chunk = (lane % ACH) ^ (MB == 64 ? 4 * ((ja >> 1) & 1) : 0);
        const bool a_ok = m0 + a_chunk * 8 < a.Mm;
        const uint32_t a_lane = (uint32_t)((ja * a.Ktot + gb * a.gkpg + m0 + a_chunk * 8) * 2);
        const uint32_t a_step = (uint32_t)(RA * a.Ktot * 2);
        const int jx = lane / XCH;
        const int x_chan = gb * a.gcpg + c0 + (lane % XCH) * 8;
        // the per-lane part of every load is the same for all rows: dY byte
        // offsets within a row (or out of range past Wo), and input-row byte
        // offsets of this lane's pixels (or out of range outside the row)
        uint32_t a_off[NA], x_off[NXL];
#pragma unroll
        for (int l = 0; l < NA; ++l)
            a_off[l] = a_ok && l * RA + ja < a.Wo ? a_lane + l * a_step : kBufOob;
#pragma unroll
        for (int l = 0; l < NXL; ++l) {
            const int pj = l * RX + jx;
            const int off = STRIDE == 1 ? pj : (pj < HALF ? 2 * pj : 2 * (pj - HALF) + 1);
            const int col = off - a.pw;
            x_off[l] = off < a.XW && (unsigned)col < (unsigned)a.Wi ? (uint32_t)((col * a.Ctot + x_chan) * 2) : kBufOob;
        }
        const uint32_t a_row = (uint32_t)(a.Wo * a.Ktot * 2), x_row = (uint32_t)(a.Wi * a.Ctot * 2);
        // an out-of-range lane offset stays out of range (>= 2^31) after a row
        // base below 2 GiB is added, so the row's own check is one select
        auto issue_row = [&](int j) {
            int n, ho;
            const int base = row_of(j, n, ho);
            const bool real = j < cnt;                 // else a zero row padding the last step
            if (dy_part) {
                uint16_t* sA = sA0 + (j % NBR) * ABUF;
                const uint32_t rb = (uint32_t)(r_begin + j) * a_row;
#pragma unroll
                for (int l = 0; l < NA; ++l)
                    dma_load16(dy_desc, lds_addr(sA + l * RA * MB), real ? rb + a_off[l] : kBufOob);
                return;
            }
            // the window rows the previous output row did not stage (all three
            // at a window start); rows outside the image are staged as zeros
            const int w0 = (j == 0 || ho == 0) ? 0 : 3 - a.sh;
            for (int w = w0; w < 3; ++w) {
                const int hi = ho * a.sh - a.ph + w;
                const bool rok = real && (unsigned)hi < (unsigned)a.Hi;
                uint16_t* dst = ring + ((base + w) % RS) * XROW;
                const uint32_t rb = (uint32_t)(n * a.Hi + hi) * x_row;
#pragma unroll
                for (int l = 0; l < NXL; ++l)
                    dma_load16(x_desc, lds_addr(dst + l * RX * CB), rok ? rb + x_off[l] : kBufOob);
            }
        };
        auto issue_step = [&](int st) {
#pragma unroll
            for (int q = 0; q < RPS; ++q) issue_row(st * RPS + q);
        };
        // issue steps 0 .. NB-2, then before barrier s+1 issue step s+NB-1
        // (into the dY buffers step s-1 left) and wait for step s+1
#pragma unroll
        for (int st = 0; st < NB - 1; ++st)
            if (st < nsteps) issue_step(st);
        // each producer waits for its own loads of the step: dY rows are NA
        // loads each, input rows at least NXL (one new row)
        auto wait_step = [&](int later) {
            if (dy_part) vm_wait_rows<NB - 2, RPS * NA>(later);
            else vm_wait_rows<NB - 2, RPS * NXL>(later);
        };
        if (nsteps > 0) wait_step(min(nsteps - 1, NB - 2));
        __builtin_amdgcn_s_barrier();
        for (int st = 0; st < nsteps; ++st) {
            if (st + NB - 1 < nsteps) issue_step(st + NB - 1);
            if (st + 1 < nsteps) wait_step(min(nsteps - 2 - st, NB - 2));
            __builtin_amdgcn_s_barrier();
        }
        return;
    }

    const int y = wave;
    // lane geometry of the transposed reads: rows frow (+4), columns fcol..fcol+3
    const int g16 = lane >> 4;
    const int frow = (g16 >> 1) * 8 + ((lane & 15) >> 2);
    const int fcol = (g16 & 1) * 16 + (lane & 3) * 4;
    // element offset inside a ring slot of the pixel each reduction row of
    // this lane reads for tap 0. w-stride 1: every row reads its own pixel
    // (the row tile is KS pixels wide, so all are in the slot; pixels past the
    // input row are zeros), which the register shifts rely on. w-stride 2:
    // rows past Wo read pixel 0 (their dY is zero).
    static_assert(STRIDE != 1 || XWP == KS, "w-stride 1 row tiles are one pixel per position");
    int xaddr[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = ks * 16 + frow + 4 * h;
            xaddr[ks][h] = (STRIDE == 1 || k < a.Wo ? k : 0) * CB + fcol;
        }
    const int a_sw = MB == 64 ? ((lane >> 3) & 1) : 0;

    f32x16 acc[FM][3];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int x = 0; x < 3; ++x) acc[i][x] = f32x16{0};

    i16x8 af[2][FM], bf[2][3];
    auto read_frags = [&](const uint16_t* sA, const uint16_t* sX, int ks, i16x8* fa, i16x8* fb) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = tr_frag(sA + (ks * 16 + frow) * MB + (i ^ a_sw) * 32 + fcol, MB);
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int dx = (STRIDE == 1 ? x : (x & 1) * HALF + (x >> 1)) * CB;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sX + xaddr[ks][0] + dx));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sX + xaddr[ks][1] + dx));
            fb[x] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    __builtin_amdgcn_s_barrier();
    for (int st = 0; st < nsteps; ++st) {
        // the step's rows: dY buffer and this wave's window row slot
        const uint16_t* sA[RPS];
        const uint16_t* sX[RPS];
#pragma unroll
        for (int q = 0; q < RPS; ++q) {
            int n, ho;
            const int j = st * RPS + q;
            sA[q] = sA0 + (j % NBR) * ABUF;
            sX[q] = ring + ((row_of(j, n, ho) + y) % RS) * XROW;
        }
        // RPS*NKS k-steps, fragments read one k-step ahead across row ends
        constexpr int T = RPS * NKS;
        if constexpr (STRIDE == 1) {
            // tap 0 of k-step t, then taps 1 and 2 of k-step t - 1, whose
            // shifted operand needs k-step t's tap-0 fragment (same row) or
            // zeros (t - 1 ends a row); fragments are read two k-steps ahead,
            // so those of t - 1 .. t + 2 are live
            i16x8 fa[4][FM], fx[4];
            auto read_t = [&](int tt, int sl) {
                const int q = tt / NKS, ks = tt % NKS;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[sl][i] = tr_frag(sA[q] + (ks * 16 + frow) * MB + (i ^ a_sw) * 32 + fcol, MB);
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sX[q] + xaddr[ks][0]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sX[q] + xaddr[ks][1]));
                fx[sl] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            auto shifted_taps = [&](int sl, int nsl) {
                const u32x4 w = __builtin_bit_cast(u32x4, fx[sl]);
                const uint32_t nw0 = nsl >= 0 ? __builtin_bit_cast(u32x4, fx[nsl])[0] : 0u;
                // lanes 0..31 continue in lane + 32, lanes 32..63 in the next k-step's lane - 32
                const auto sw = __builtin_amdgcn_permlane32_swap(w[0], nw0, false, false);
                const uint32_t ext = lane < 32 ? sw[1] : sw[0];
                const u32x4 s1 = {__builtin_amdgcn_alignbit(w[1], w[0], 16), __builtin_amdgcn_alignbit(w[2], w[1], 16),
                                  __builtin_amdgcn_alignbit(w[3], w[2], 16), __builtin_amdgcn_alignbit(ext, w[3], 16)};
                const u32x4 s2 = {w[1], w[2], w[3], ext};
#pragma unroll
                for (int i2 = 0; i2 < FM; ++i2) {
                    mfma_step32<F16>(__builtin_bit_cast(i16x8, s1), fa[sl][i2], acc[i2][1]);
                    mfma_step32<F16>(__builtin_bit_cast(i16x8, s2), fa[sl][i2], acc[i2][2]);
                }
            };
            read_t(0, 0);
            if (T > 1) read_t(1, 1);
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
                const int c = tt % 4;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i2 = 0; i2 < FM; ++i2) mfma_step32<F16>(fx[c], fa[c][i2], acc[i2][0]);
                if (tt > 0) shifted_taps((tt - 1) % 4, tt % NKS ? c : -1);
                // issued after this k-step's operands are in registers, so the
                // waits for k-step t never cover the reads of t + 1 and t + 2
                if (tt + 2 < T) read_t(tt + 2, (tt + 2) % 4);
                __builtin_amdgcn_sched_barrier(0);
            }
            shifted_taps((T - 1) % 4, -1);
        } else {
        read_frags(sA[0], sX[0], 0, af[0], bf[0]);
#pragma unroll
        for (int k = 0; k < T; ++k) {
            const int cur = k & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (k + 1 < T) read_frags(sA[(k + 1) / NKS], sX[(k + 1) / NKS], (k + 1) % NKS, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
            for (int x = 0; x < 3; ++x)
#pragma unroll
                for (int i2 = 0; i2 < FM; ++i2) mfma_step32<F16>(bf[cur][x], af[cur][i2], acc[i2][x]);
#pragma unroll
            for (int m = 0; m < FM * 3; ++m) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        }
        // step st is consumed (its dY buffers may be refilled) and step st + 1 has landed
        lds_barrier();
    }

    // ---- the three waves' blocks meet in LDS as one fp32 tile [m][tap][c]
    // (the staging buffers are free: every wave is past the last step), and
    // are stored from there as whole 128-byte runs of 32 channels of one tap,
    // so each store instruction writes eight full lines
    float* const red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int x = 0; x < 3; ++x)
#pragma unroll
            for (int vq = 0; vq < 4; ++vq) {
                const f32x16& c = acc[i][x];
                *reinterpret_cast<f32x4*>(red + (i * 32 + (lane & 31)) * kRingTilePitch + (y * 3 + x) * CB + 8 * vq +
                                          4 * (lane >> 5)) = f32x4{c[4 * vq], c[4 * vq + 1], c[4 * vq + 2], c[4 * vq + 3]};
            }
    // the load waves have ended; this barrier joins the three MFMA waves
    lds_barrier();
    // element it = row * RUNS + run of the tile (run = tap * CB/4 + chunk, a
    // 4-channel chunk) goes to thread it % 192, so eight consecutive lanes
    // store one tap's 32 channels (a whole 128-byte line) of one row. A
    // thread's runs repeat every PER passes; with merged groups only the
    // diagonal blocks are stored. Offsets are relative to the slice start.
    constexpr int NTH = 3 * 64, RUNS = 9 * (CB / 4), PER = 3, ITER = MB * RUNS / NTH;
    constexpr int RSTEP = PER * NTH / RUNS;        // tile rows advanced every PER passes
    static_assert((MB * RUNS) % NTH == 0 && ITER % PER == 0 && (PER * NTH) % RUNS == 0, "store passes");
    const int tid = threadIdx.x;
    int lrow[PER], lcol[PER], glo[PER];
    int64_t goff[PER];
#pragma unroll
    for (int ph = 0; ph < PER; ++ph) {
        const int it = tid + ph * NTH;
        const int run = it % RUNS, tap = run / (CB / 4), c4 = (run % (CB / 4)) * 4;
        const int cg = c0 + c4;
        const int gj = (int)magic_div((uint32_t)cg, a.mCpg);   // group of these channels (cpg % 4 == 0)
        lrow[ph] = it / RUNS;
        lcol[ph] = tap * CB + c4;
        glo[ph] = gj * a.kpg;
        goff[ph] = tap * a.cpg + (cg - gj * a.cpg);
    }
    const int64_t tile0 = (int64_t)(gb * a.gkpg) * a.row_len;   // within dW or a workspace slice
    auto store_all = [&](auto put) {
#pragma unroll
        for (int u = 0; u < ITER / PER; ++u)
#pragma unroll
            for (int ph = 0; ph < PER; ++ph) {
                const int row = lrow[ph] + u * RSTEP;
                const int mg = m0 + row;
                if (mg < a.Mm && mg >= glo[ph] && mg < glo[ph] + a.kpg)
                    put(mg * a.row_len + goff[ph],
                        *reinterpret_cast<const f32x4*>(red + row * kRingTilePitch + lcol[ph]));
            }
    };
    // one loop per output type, so that no store carries the type switch
    if (a.out_mode == OUT_WORKSPACE) {
        const __amdgpu_buffer_rsrc_t ws = buf_rsrc(static_cast<float*>(a.out) + (int64_t)z * a.slice_elems,
                                                   4u * (uint32_t)a.slice_elems);
        store_all([&](int e, const f32x4& v) { store_partial4(ws, tile0 + e, v); });
    } else if (a.out_mode == OUT_FP32) {
        float* o = static_cast<float*>(a.out) + tile0;
        store_all([&](int e, const f32x4& v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o + e)); });
    } else if (a.out_mode == OUT_BF16) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + tile0;
        store_all([&](int e, const f32x4& v) {
            u32x2 p;
            p[0] = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            p[1] = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            *reinterpret_cast<u32x2*>(o + e) = p;
        });
    } else {
        uint16_t* o = static_cast<uint16_t*>(a.out) + tile0;
        store_all([&](int e, const f32x4& v) {
            u32x2 p;
            p[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[0]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[1]) << 16);
            p[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[3]) << 16);
            *reinterpret_cast<u32x2*>(o + e) = p;
        });
    }
}

template <int I, bool F16>
int launch_ring_i(const Plan& plan, const RingArgs& a, hipStream_t s) {
    constexpr RingInstance r = kRingInstances[I];
    auto k = ring_kernel<r.mb, r.nks, r.xwp, r.stride, r.nb, r.rps, F16>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, plan.lds_bytes);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(k, dim3(a.total_wg), dim3(320), plan.lds_bytes, s, a);
    return (int)hipGetLastError();
}

template <bool F16>
int launch_ring_t(const Plan& plan, const RingArgs& a, hipStream_t s) {
    static_assert(kNumRingInstances == 6, "dispatch table");
    switch (plan.ring_inst) {
        case 0: return launch_ring_i<0, F16>(plan, a, s);
        case 1: return launch_ring_i<1, F16>(plan, a, s);
        case 2: return launch_ring_i<2, F16>(plan, a, s);
        case 3: return launch_ring_i<3, F16>(plan, a, s);
        case 4: return launch_ring_i<4, F16>(plan, a, s);
        case 5: return launch_ring_i<5, F16>(plan, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_ring(const Plan& plan, const RingArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_ring_t<true>(plan, a, s) : launch_ring_t<false>(plan, a, s);
}

}  // namespace wgrad
