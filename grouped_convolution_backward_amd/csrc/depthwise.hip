// Depthwise (C/G = K/G = 1) backward-weight kernel for gfx950.
//
// With one channel per group the per-group GEMM of the Composable Kernel wgrad
// page degenerates to 1 x (Y*X) x (N*Ho*Wo): no matrix to speak of, and the
// work is bound by streaming X and dY once from HBM. The group-merging idea of
// rocm-libraries PR 12359 (fold Gm adjacent groups into one workgroup so that
// a load covers Gm consecutive channels) is taken to the vector width here:
// each lane owns 8 adjacent channels (one 16-byte load per pixel) and only the
// diagonal group pairs are ever formed.
//
// A lane processes "units": 4 consecutive output positions of one output row.
// For a filter of width 3 (w-stride and w-dilation 1) the unit needs a
// 6-column window of each of the Y input rows; positions are taken in pairs,
// and v_perm_b32 packs (dY[w], dY[w+1]) and (X[w+x], X[w+x+1]) of one channel
// into one register so that a single v_dot2c_f32_{bf16,f16} adds both
// products to the fp32 accumulator of that (channel, tap).
//
// All loads are raw buffer loads whose out-of-range offsets return zeros, so
// padding, row ends and the tail need no branches. At the end each workgroup
// sums its lanes (shuffles across the wave, then LDS across the 4 waves, in a
// fixed order) and writes one partial (S > 1) or dW itself.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;

constexpr int kUnit = 4;            // output positions per unit
constexpr int kWin = kUnit + 2;     // input columns per unit for a width-3 filter

template <int TY>
struct UnitRegs {
    u32x4 d[kUnit];          // dY of the unit's 4 positions
    u32x4 x[TY][kWin];       // X window: TY rows x 6 columns
};

template <int TY, bool F16>
__global__ __launch_bounds__(256, 1) void dw2_kernel(const Dw2Args a) {
    constexpr int T = TY * 3;
    const int tid = threadIdx.x;
    const int cl = a.cl, ul = 256 / cl;
    const int cv = tid % cl, ulane = tid / cl;
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    const int cb = L / a.S, z = L - (L / a.S) * a.S;     // adjacent splits of one channel block share an XCD
    const int c0 = (cb * cl + cv) * 8;
    const __amdgpu_buffer_rsrc_t x_rs = buf_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t dy_rs = buf_rsrc(a.dy, a.dy_bytes);
    const int u_end = min(a.units, (z + 1) * a.upw);

    // issue the 4 + 6*TY loads of the lane's k-th unit (out-of-range units and
    // pixels load zeros)
    auto load_unit = [&](int k, UnitRegs<TY>& r) {
        const int u = z * a.upw + k * ul + ulane;
        const bool valid = u < u_end;
        const int row = (int)magic_div((uint32_t)u, a.mSeg);
        const int wo0 = (u - row * a.nseg) * kUnit;
        const int n = (int)magic_div((uint32_t)row, a.mHo);
        const int ho = row - n * a.Ho;
#pragma unroll
        for (int p = 0; p < kUnit; ++p) {
            const bool ok = valid && wo0 + p < a.Wo;
            r.d[p] = buf_load16(dy_rs, ok ? (uint32_t)(((row * a.Wo + wo0 + p) * a.C + c0) * 2) : kBufOob);
        }
#pragma unroll
        for (int y = 0; y < TY; ++y) {
            const int hi = ho * a.sh - a.ph + y * a.dh;
            const bool rok = valid && (unsigned)hi < (unsigned)a.Hi;
            const int pix = (n * a.Hi + hi) * a.Wi + wo0 - a.pw;
#pragma unroll
            for (int j = 0; j < kWin; ++j) {
                const bool ok = rok && (unsigned)(wo0 - a.pw + j) < (unsigned)a.Wi;
                r.x[y][j] = buf_load16(x_rs, ok ? (uint32_t)(((pix + j) * a.C + c0) * 2) : kBufOob);
            }
        }
    };

    float acc[T][8];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[t][k] = 0.f;

    auto compute_unit = [&](const UnitRegs<TY>& r) {
#pragma unroll
        for (int q = 0; q < kUnit / 2; ++q)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t dlo = pair_lo(r.d[2 * q][w], r.d[2 * q + 1][w]);
                const uint32_t dhi = pair_hi(r.d[2 * q][w], r.d[2 * q + 1][w]);
#pragma unroll
                for (int y = 0; y < TY; ++y)
#pragma unroll
                    for (int x = 0; x < 3; ++x) {
                        const uint32_t a0 = r.x[y][2 * q + x][w], a1 = r.x[y][2 * q + x + 1][w];
                        acc[y * 3 + x][2 * w] = dot2<F16>(dlo, pair_lo(a0, a1), acc[y * 3 + x][2 * w]);
                        acc[y * 3 + x][2 * w + 1] = dot2<F16>(dhi, pair_hi(a0, a1), acc[y * 3 + x][2 * w + 1]);
                    }
            }
    };

    // two register sets: the next unit's loads are in flight while the
    // current unit is computed
    UnitRegs<TY> ra, rb;
    load_unit(0, ra);
    for (int k = 0; k < a.upt; k += 2) {
        load_unit(k + 1, rb);
        compute_unit(ra);
        if (k + 2 < a.upt) load_unit(k + 2, ra);
        if (k + 1 < a.upt) compute_unit(rb);
    }

    // lanes with the same channel lane are cl apart within a wave
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float v = acc[t][k];
            for (int off = cl; off < 64; off <<= 1) v += __shfl_xor(v, off);
            acc[t][k] = v;
        }
    __shared__ float part[4][64][T * 8];
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < cl) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int k = 0; k < 8; ++k) part[wave][lane][t * 8 + k] = acc[t][k];
    }
    __syncthreads();
    const int64_t zoff = a.out_mode == OUT_WORKSPACE ? (int64_t)z * a.slice_elems : 0;
    for (int o = tid; o < cl * T * 8; o += 256) {
        const int v = o / (T * 8), w = o - v * (T * 8);
        const int t = w / 8, k = w - t * 8;
        const float sum = ((part[0][v][w] + part[1][v][w]) + part[2][v][w]) + part[3][v][w];
        const int c = (cb * cl + v) * 8 + k;
        store_out(a.out, a.out_mode, zoff + (int64_t)c * T + t, sum);
    }
}

template <bool F16>
int launch_t(int ty, const Dw2Args& a, hipStream_t s) {
    dim3 grid(a.total_wg), block(256);
    switch (ty) {
        case 1: hipLaunchKernelGGL((dw2_kernel<1, F16>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((dw2_kernel<3, F16>), grid, block, 0, s, a); break;
        case 5: hipLaunchKernelGGL((dw2_kernel<5, F16>), grid, block, 0, s, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}


// Strip variant (3x3 filter, stride 1 and dilation 1 on both axes).
//
// Work items: a 4-wide column strip of one image, cut into nch chunks of
// consecutive output rows; a worker (a wave, or a 64/cl-th of one when a
// channel block is narrower than the wave) takes items grid-stride. Within an
// item it walks the chunk's rows one output row ("step") at a time and keeps
// the three input rows of the step in a register ring, already packed into
// the (column j, column j+1) pairs the dot products read, so a step loads and
// packs one new input row (6 pixels) and its dY row (4 pixels). Steps are
// loaded kAhead ahead into three rotating buffers; the loop is unrolled by
// three so that the ring and buffer rotation is static.
//
// HBM reuse: items are numbered strip-major, chunk-minor, and chunk c walks
// down when c is even and up when c is odd. All chunk rows are aligned across
// strips, so neighbouring strips read their two shared input columns at the
// same moment, and the two chunks on either side of a chunk boundary reach
// the boundary's halo rows at the same moment (both at their start, or both
// at their end). Each shared line then comes from HBM once and from L2 for
// the second reader, instead of twice.
//
// A lane owns kDw3Channels adjacent channels (one 8- or 16-byte load per
// pixel); kDw3Waves waves per workgroup, one workgroup per CU.
constexpr int kAhead = 2;           // steps loaded ahead of the one computed (1 or 2)
constexpr int kW3 = kDw3Words;      // 32-bit words (channel pairs) per lane

typedef typename VecT<2 * kW3>::T PxVec;   // one lane's channels of one pixel
template <int W = kW3>
__device__ __forceinline__ typename VecT<2 * W>::T load_px(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (W == 4) return buf_load16(r, off);
    else return buf_load8(r, off);
}
struct StepBuf {
    PxVec d[kUnit];      // dY of the step's 4 positions
    PxVec xn[kWin];      // the input row that enters the ring at this step
};
struct RowPairs {
    uint32_t lo[kW3][kWin - 1], hi[kW3][kWin - 1];   // [word][column j]: (col j, col j+1)
};

__device__ __forceinline__ void pack_row(const PxVec* raw, RowPairs& r) {
#pragma unroll
    for (int w = 0; w < kW3; ++w)
#pragma unroll
        for (int j = 0; j < kWin - 1; ++j) {
            r.lo[w][j] = pair_lo(raw[j][w], raw[j + 1][w]);
            r.hi[w][j] = pair_hi(raw[j][w], raw[j + 1][w]);
        }
}

// ring slot of window row y (0 = top) at step i of an item: walking down the
// new row is y = 2 and takes the slot row 0 left; walking up it is y = 0 and
// takes the slot row 2 left
template <bool UP>
constexpr int ring_slot(int y, int i) { return UP ? (y + 2 * i) % 3 : (y + i) % 3; }

template <bool F16>
__global__ __launch_bounds__(64 * kDw3Waves, 1) void dw3_kernel(const Dw3Args a) {
    constexpr int T = 9, CH = 2 * kW3;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cl = a.cl;
    const int cv = lane % cl;
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    // channel blocks are the fastest index: the blocks of one split read the
    // two (or more) halves of the same pixels at the same time on one XCD, so
    // each pixel's full channel run is fetched from HBM together
    const int cb = L % a.cblocks, z = L / a.cblocks;
    const int c0 = (cb * cl + cv) * CH;
    const __amdgpu_buffer_rsrc_t x_rs = buf_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t dy_rs = buf_rsrc(a.dy, a.dy_bytes);
    const int sub = lane / cl, nsub = 64 / cl;
    // Item order. When every XCD holds whole splits (the same number for each
    // channel block), XCD x takes items [x*items/8, (x+1)*items/8): the
    // strips there are mostly neighbours of each other, so the input columns
    // two strips share come from HBM once and from this XCD's L2 after (with
    // one range per XCD the neighbours on two XCDs are 7 pairs, against one
    // pair in four strips when items go round-robin over the XCDs). Within an
    // XCD, and otherwise over the whole grid, worker (wave, sub, z) takes
    // items rank, rank + workers, ... with rank = (wave, sub) * (splits) + z:
    // consecutive items go to the same wave slot of consecutive workgroups,
    // and idle workers spread evenly.
    const int xq = a.total_wg >> 3;
    const bool xmajor = (a.total_wg & 7) == 0 && xq % a.cblocks == 0;
    const int zpx = xmajor ? xq / a.cblocks : a.S;  // splits per XCD (or all of them)
    const int zx = z / zpx, zl = z - zx * zpx;
    const int wid = (wave * nsub + sub) * zpx + zl;
    const int nworkers = kDw3Waves * nsub * zpx;
    const int it_begin = xmajor ? (int)((int64_t)a.items * zx / 8) : 0;
    const int it_end = xmajor ? (int)((int64_t)a.items * (zx + 1) / 8) : a.items;

    float acc[T][CH];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < CH; ++k) acc[t][k] = 0.f;

    // input row hi of image n, columns wo0 - pw .. wo0 - pw + 5 (zeros outside)
    auto x_row = [&](int n, int hi, int wo0, PxVec* r) {
        const bool rok = (unsigned)hi < (unsigned)a.Hi;
        const int pix = (n * a.Hi + hi) * a.Wi + wo0 - a.pw;
#pragma unroll
        for (int j = 0; j < kWin; ++j) {
            const bool ok = rok && (unsigned)(wo0 - a.pw + j) < (unsigned)a.Wi;
            r[j] = load_px(x_rs, ok ? (uint32_t)(((pix + j) * a.C + c0) * 2) : kBufOob);
        }
    };

    auto run_item = [&](int n, int wo0, int r0, int r1, auto up_tag) {
        constexpr bool UP = decltype(up_tag)::value;
        const int nsteps = r1 - r0;
        // output row of step i, and the input row that enters the ring there
        auto ho_of = [&](int i) { return UP ? r1 - 1 - i : r0 + i; };
        auto load_step = [&](int i, StepBuf& b) {
            const bool valid = i < nsteps;
            const int ho = ho_of(i);
#pragma unroll
            for (int p = 0; p < kUnit; ++p) {
                const bool ok = valid && wo0 + p < a.Wo;
                b.d[p] = load_px(dy_rs, ok ? (uint32_t)((((n * a.Ho + ho) * a.Wo + wo0 + p) * a.C + c0) * 2)
                                           : kBufOob);
            }
            x_row(n, valid ? ho - a.ph + (UP ? 0 : 2) : -1, wo0, b.xn);
        };
        RowPairs ring[3];
        StepBuf buf[3];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) load_step(i, buf[i]);
        {
            // the two rows of the first window that do not enter at step 0
            const int ho = ho_of(0);
            PxVec raw[kWin];
            x_row(n, ho - a.ph + 1, wo0, raw);
            pack_row(raw, ring[ring_slot<UP>(1, 0)]);
            x_row(n, ho - a.ph + (UP ? 2 : 0), wo0, raw);
            pack_row(raw, ring[ring_slot<UP>(UP ? 2 : 0, 0)]);
        }
        auto sub_step = [&](int i, auto rot) {
            constexpr int R = decltype(rot)::value;     // i % 3
            if (i >= nsteps) return;
            load_step(i + kAhead, buf[(R + kAhead) % 3]);
            const StepBuf& b = buf[R];
            pack_row(b.xn, ring[ring_slot<UP>(UP ? 0 : 2, R)]);
#pragma unroll
            for (int q = 0; q < kUnit / 2; ++q)
#pragma unroll
                for (int w = 0; w < kW3; ++w) {
                    const uint32_t dlo = pair_lo(b.d[2 * q][w], b.d[2 * q + 1][w]);
                    const uint32_t dhi = pair_hi(b.d[2 * q][w], b.d[2 * q + 1][w]);
#pragma unroll
                    for (int y = 0; y < 3; ++y)
#pragma unroll
                        for (int x = 0; x < 3; ++x) {
                            const RowPairs& rp = ring[ring_slot<UP>(y, R)];
                            acc[y * 3 + x][2 * w] = dot2<F16>(dlo, rp.lo[w][2 * q + x], acc[y * 3 + x][2 * w]);
                            acc[y * 3 + x][2 * w + 1] =
                                dot2<F16>(dhi, rp.hi[w][2 * q + x], acc[y * 3 + x][2 * w + 1]);
                        }
                }
        };
        for (int i = 0; i < nsteps; i += 3) {
            sub_step(i, std::integral_constant<int, 0>{});
            sub_step(i + 1, std::integral_constant<int, 1>{});
            sub_step(i + 2, std::integral_constant<int, 2>{});
        }
    };

    for (int it = it_begin + wid; it < it_end; it += nworkers) {
        const int strip = it / a.nch, c = it - strip * a.nch;
        const int n = strip / a.nseg;
        const int wo0 = (strip - n * a.nseg) * kUnit;
        const int r0 = (int)((int64_t)c * a.Ho / a.nch), r1 = (int)((int64_t)(c + 1) * a.Ho / a.nch);
        if (c & 1)
            run_item(n, wo0, r0, r1, std::true_type{});
        else
            run_item(n, wo0, r0, r1, std::false_type{});
    }

    // lanes of one channel lane are cl apart within the wave; then the waves
    // are summed through LDS, both in a fixed order
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            float v = acc[t][k];
            for (int off = cl; off < 64; off <<= 1) v += __shfl_xor(v, off);
            acc[t][k] = v;
        }
    __shared__ float part[kDw3Waves][64][T * CH];
    if (lane < cl) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int k = 0; k < CH; ++k) part[wave][lane][t * CH + k] = acc[t][k];
    }
    __syncthreads();
    // thread o writes element o of the block's contiguous dW run (channel
    // c = o / 9, tap t = o % 9), so the stores are coalesced
    const int64_t zoff = a.out_mode == OUT_WORKSPACE ? (int64_t)z * a.slice_elems : 0;
    const int64_t base = zoff + (int64_t)cb * cl * CH * T;
    for (int o = tid; o < cl * T * CH; o += 64 * kDw3Waves) {
        const int cloc = o / T, t = o - cloc * T;
        const int v = cloc / CH, k = cloc - v * CH;
        const int w = t * CH + k;
        float sum = part[0][v][w];
#pragma unroll
        for (int q = 1; q < kDw3Waves; ++q) sum += part[q][v][w];
        store_out(a.out, a.out_mode, base + o, sum);
    }
}

template <bool F16>
int launch_t3(int ty, const Dw3Args& a, hipStream_t s) {
    dim3 grid(a.total_wg), block(64 * kDw3Waves);
    if (ty != 3) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL((dw3_kernel<F16>), grid, block, 0, s, a);
    return (int)hipGetLastError();
}

}  // namespace

int launch_depthwise3(const Plan& plan, const Dw3Args& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_t3<true>(plan.dw3_ty, a, s) : launch_t3<false>(plan.dw3_ty, a, s);
}

int launch_depthwise2(const Plan& plan, const Dw2Args& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_t<true>(plan.dw2_ty, a, s) : launch_t<false>(plan.dw2_ty, a, s);
}

}  // namespace wgrad
