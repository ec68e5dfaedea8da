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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// (lo half of a, lo half of b) and (hi half of a, hi half of b)
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

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


// Strip variant (3x3 filter, stride 1 and dilation 1 on both axes). A lane
// owns 4 adjacent channels (one 8-byte load per pixel), so that two waves fit
// on a SIMD. A worker (a wave, or a 64/cl-th of one when a channel block is
// narrower than the wave) owns a contiguous range of row steps; a step is one
// output row of a 4-wide column strip, and consecutive steps walk down the
// strip. The three input rows a step needs are kept in a register ring,
// already packed into the (column j, column j+1) pairs the dot products read,
// so a step loads and packs one new input row (6 pixels) and its dY row (4
// pixels). Compared with independent 4-position units this cuts the L1-to-L2
// request volume per output position by about 2.2x and the packing work by
// 3x. Steps are loaded kAhead ahead into three rotating buffers; the loop is
// unrolled by three so that the ring and buffer rotation is static. Only the
// first step of a worker and the first step of each new strip reload the two
// older ring rows.
#ifndef DW3_AHEAD
#define DW3_AHEAD 2
#endif
constexpr int kAhead = DW3_AHEAD;   // steps loaded ahead of the one computed (1 or 2)
constexpr int kW3 = 2;              // 32-bit words (channel pairs) per lane

struct StepBuf {
    u32x2 d[kUnit];      // dY of the step's 4 positions
    u32x2 xn[kWin];      // newest input row of the step
};
struct RowPairs {
    uint32_t lo[kW3][kWin - 1], hi[kW3][kWin - 1];   // [word][column j]: (col j, col j+1)
};

__device__ __forceinline__ void pack_row(const u32x2* raw, RowPairs& r) {
#pragma unroll
    for (int w = 0; w < kW3; ++w)
#pragma unroll
        for (int j = 0; j < kWin - 1; ++j) {
            r.lo[w][j] = pair_lo(raw[j][w], raw[j + 1][w]);
            r.hi[w][j] = pair_hi(raw[j][w], raw[j + 1][w]);
        }
}

template <bool F16>
__global__ __launch_bounds__(256, 2) void dw3_kernel(const Dw3Args a) {
    constexpr int TY = 3, T = 9, CH = 2 * kW3;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cl = a.cl;
    const int cv = lane % cl;
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    const int cb = L / a.S, z = L - (L / a.S) * a.S;
    const int c0 = (cb * cl + cv) * CH;
    const __amdgpu_buffer_rsrc_t x_rs = buf_rsrc(a.x, a.x_bytes);
    const __amdgpu_buffer_rsrc_t dy_rs = buf_rsrc(a.dy, a.dy_bytes);
    const int sub = lane / cl, nsub = 64 / cl;
    const int wid = (z * 4 + wave) * nsub + sub;
    const int nworkers = a.waves * nsub;
    const int st0 = (int)((int64_t)wid * a.steps / nworkers);
    const int st1 = (int)((int64_t)(wid + 1) * a.steps / nworkers);

    float acc[T][CH];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < CH; ++k) acc[t][k] = 0.f;

    // input row hi of image n, columns wo0 - pw .. wo0 - pw + 5 (zeros outside)
    auto x_row = [&](int n, int hi, int wo0, u32x2* r) {
        const bool rok = (unsigned)hi < (unsigned)a.Hi;
        const int pix = (n * a.Hi + hi) * a.Wi + wo0 - a.pw;
#pragma unroll
        for (int j = 0; j < kWin; ++j) {
            const bool ok = rok && (unsigned)(wo0 - a.pw + j) < (unsigned)a.Wi;
            r[j] = buf_load8(x_rs, ok ? (uint32_t)(((pix + j) * a.C + c0) * 2) : kBufOob);
        }
    };
    // a step cursor: image, strip start column, output row
    struct Cur {
        int n, wo0, ho;
    };
    auto decode = [&](int st) {
        const int strip = st / a.Ho;
        Cur c;
        c.ho = st - strip * a.Ho;
        c.n = strip / a.nseg;
        c.wo0 = (strip - c.n * a.nseg) * kUnit;
        return c;
    };
    auto advance = [&](Cur& c) {
        if (++c.ho == a.Ho) {
            c.ho = 0;
            c.wo0 += kUnit;
            if (c.wo0 == a.nseg * kUnit) {
                c.wo0 = 0;
                ++c.n;
            }
        }
    };
    // loads of one step (all zeros when the step is outside the worker's range)
    auto load_step = [&](const Cur& c, bool valid, StepBuf& b) {
#pragma unroll
        for (int p = 0; p < kUnit; ++p) {
            const bool ok = valid && c.wo0 + p < a.Wo;
            b.d[p] = buf_load8(dy_rs, ok ? (uint32_t)((((c.n * a.Ho + c.ho) * a.Wo + c.wo0 + p) * a.C + c0) * 2)
                                         : kBufOob);
        }
        x_row(c.n, valid ? c.ho - a.ph + TY - 1 : -1, c.wo0, b.xn);
    };

    RowPairs ring[3];
    StepBuf buf[3];
    Cur cc = decode(st0 < st1 ? st0 : 0);   // compute cursor
    Cur pc = cc;                            // prefetch cursor
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
        load_step(pc, st0 + i < st1, buf[i]);
        advance(pc);
    }

    // step st with rotation R: ring slot (R + y) % 3 holds input row y of the step
    auto sub_step = [&](int st, auto rot) {
        constexpr int R = decltype(rot)::value;
        if (st >= st1) return;
        if (st == st0 || cc.ho == 0) {
            u32x2 raw[kWin];
            x_row(cc.n, cc.ho - a.ph, cc.wo0, raw);
            pack_row(raw, ring[R % 3]);
            x_row(cc.n, cc.ho - a.ph + 1, cc.wo0, raw);
            pack_row(raw, ring[(R + 1) % 3]);
        }
        load_step(pc, st + kAhead < st1, buf[(R + kAhead) % 3]);
        advance(pc);
        const StepBuf& b = buf[R % 3];
        pack_row(b.xn, ring[(R + 2) % 3]);
#pragma unroll
        for (int q = 0; q < kUnit / 2; ++q)
#pragma unroll
            for (int w = 0; w < kW3; ++w) {
                const uint32_t dlo = pair_lo(b.d[2 * q][w], b.d[2 * q + 1][w]);
                const uint32_t dhi = pair_hi(b.d[2 * q][w], b.d[2 * q + 1][w]);
#pragma unroll
                for (int y = 0; y < TY; ++y)
#pragma unroll
                    for (int x = 0; x < 3; ++x) {
                        const RowPairs& rp = ring[(R + y) % 3];
                        acc[y * 3 + x][2 * w] = dot2<F16>(dlo, rp.lo[w][2 * q + x], acc[y * 3 + x][2 * w]);
                        acc[y * 3 + x][2 * w + 1] = dot2<F16>(dhi, rp.hi[w][2 * q + x], acc[y * 3 + x][2 * w + 1]);
                    }
            }
        advance(cc);
    };
    for (int st = st0; st < st1; st += 3) {
        sub_step(st, std::integral_constant<int, 0>{});
        sub_step(st + 1, std::integral_constant<int, 1>{});
        sub_step(st + 2, std::integral_constant<int, 2>{});
    }

    // lanes of one channel lane are cl apart within the wave; then the 4
    // waves are summed through LDS, both in a fixed order
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            float v = acc[t][k];
            for (int off = cl; off < 64; off <<= 1) v += __shfl_xor(v, off);
            acc[t][k] = v;
        }
    __shared__ float part[4][64][T * CH];
    if (lane < cl) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int k = 0; k < CH; ++k) part[wave][lane][t * CH + k] = acc[t][k];
    }
    __syncthreads();
    const int64_t zoff = a.out_mode == OUT_WORKSPACE ? (int64_t)z * a.slice_elems : 0;
    for (int o = tid; o < cl * T * CH; o += 256) {
        const int v = o / (T * CH), w = o - v * (T * CH);
        const int t = w / CH, k = w - t * CH;
        const float sum = ((part[0][v][w] + part[1][v][w]) + part[2][v][w]) + part[3][v][w];
        const int c = (cb * cl + v) * CH + k;
        store_out(a.out, a.out_mode, zoff + (int64_t)c * T + t, sum);
    }
}

template <bool F16>
int launch_t3(int ty, const Dw3Args& a, hipStream_t s) {
    dim3 grid(a.total_wg), block(256);
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
