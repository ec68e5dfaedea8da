// HIP kernels for grouped convolution backward-weight on gfx950 (MI355X).
//
// 1. mfma_kernel: batched-over-groups implicit GEMM
//      C[m][j] = sum_r A[m][r] * B[j][r]
//    with A = dY (m = output channel of the group), B = X gathered at the
//    filter tap of column j (j = tap*cpg + c), r = (n*Ho + ho)*Wo + wo, as in
//    the Composable Kernel wgrad kernel page (operator(): one tile of one
//    group's dW over one K slice per workgroup). Tiles are staged in LDS in
//    global order (reduction axis outer, "K-outer"), written with full-width
//    vector stores straight from the coalesced global loads, and the MFMA
//    operands are fetched with the CDNA4 transposed read ds_read_b64_tr_b16
//    (rocm-libraries PR 11602, "K-outer LDS tile"), so nothing is transposed
//    on the way into LDS. Optional group merging folds Gm adjacent groups into
//    one tile and stores only the diagonal group pairs (PR 12359). With S > 1
//    each slice writes fp32 partials to a workspace (deterministic two-stage
//    split-K; no atomics).
// 2. reduce_kernel: dW = round(sum_z ws[z]) in a fixed order.
// 3. dw_kernel: depthwise (C/G = K/G = 1) direct kernel; one lane owns 8
//    adjacent channels (8 merged groups, one 16-byte load per pixel).
#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;

template <int BM, int BN, int BK, int WM, int WN, int ATOM, int V, bool F16>
__global__ __launch_bounds__(256) void mfma_kernel(const MfmaArgs a) {
    typedef typename VecT<V>::T VT;
    constexpr int PA = BM + kLdsPad, PB = BN + kLdsPad;
    constexpr int AK = ATOM == 32 ? 16 : 32;       // reduction depth of one MFMA
    constexpr int WTM = BM / WM, WTN = BN / WN;    // wave tile
    constexpr int FM = WTM / ATOM, FN = WTN / ATOM;
    constexpr int AVR = BM / V, BVR = BN / V;      // vectors per tile row
    constexpr int A_RPP = 256 / AVR, B_RPP = 256 / BVR;   // rows per load pass
    constexpr int A_PASSES = (BK + A_RPP - 1) / A_RPP;
    constexpr int B_PASSES = (BK + B_RPP - 1) / B_RPP;
    static_assert(WM * WN == 4, "4 waves per workgroup");
    static_assert(FM >= 1 && FN >= 1 && WTM % ATOM == 0 && WTN % ATOM == 0, "wave tile");
    static_assert(BK % AK == 0 && 256 % AVR == 0 && 256 % BVR == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t sA[BK * PA];
    __shared__ __attribute__((aligned(16))) uint16_t sB[BK * PB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    const int tiles_mn = a.tiles_m * a.tiles_n;
    const int tile = L % tiles_mn;
    const int rest = L / tiles_mn;
    const int gb = rest % a.gblocks;
    const int z = rest / a.gblocks;
    const int m0 = (tile / a.tiles_n) * BM;
    const int n0 = (tile % a.tiles_n) * BN;
    const int r_begin = z * a.kslice;
    const int r_end = min(a.R, r_begin + a.kslice);
    const int niter = r_end > r_begin ? (r_end - r_begin + BK - 1) / BK : 0;

    // operand bases of the (merged) group block
    const uint16_t* dyp = a.dy + gb * a.gkpg;
    const uint16_t* xp = a.x + gb * a.gcpg;

    // A (dY) loads: thread owns column a_col of the tile, rows a_row0 + p*A_RPP
    const int a_col = (tid % AVR) * V;
    const int a_row0 = tid / AVR;
    const bool a_col_ok = m0 + a_col < a.Mm;
    const uint16_t* a_src = dyp + m0 + a_col;
    // B (X) loads: column jb is one filter tap and one channel run
    const int b_col = (tid % BVR) * V;
    const int b_row0 = tid / BVR;
    const int jb = n0 + b_col;
    const bool b_col_ok = jb < a.Nm;
    const int tap = jb / a.gcpg;
    const int cc = jb - tap * a.gcpg;
    const int tzy = tap / a.Xf, tx = tap - tzy * a.Xf;   // tap = (z*Y + y)*X + x
    const int tz = tzy / a.Yf, ty = tzy - tz * a.Yf;
    const int doff = tz * a.dd - a.pd, hoff = ty * a.dh - a.ph, woff = tx * a.dw - a.pw;
    const uint16_t* b_src = xp + cc;

    VT ra[A_PASSES], rb[B_PASSES];

    auto gload = [&](int r0) {
#pragma unroll
        for (int p = 0; p < A_PASSES; ++p) {
            const int row = a_row0 + p * A_RPP;
            const int r = r0 + row;
            VT v = 0;
            if ((A_PASSES * A_RPP <= BK || row < BK) && a_col_ok && r < r_end)
                v = *reinterpret_cast<const VT*>(a_src + r * a.Ktot);
            ra[p] = v;
        }
#pragma unroll
        for (int p = 0; p < B_PASSES; ++p) {
            const int row = b_row0 + p * B_RPP;
            const int r = r0 + row;
            VT v = 0;
            if ((B_PASSES * B_RPP <= BK || row < BK) && b_col_ok && r < r_end) {
                // r = ((n*Do + do)*Ho + ho)*Wo + wo
                const uint32_t q1 = magic_div((uint32_t)r, a.mWo);
                const int wo = r - (int)q1 * a.Wo;
                const uint32_t q2 = magic_div(q1, a.mHo);
                const int ho = (int)q1 - (int)q2 * a.Ho;
                const uint32_t n = magic_div(q2, a.mDo);
                const int od = (int)q2 - (int)n * a.Do;
                const int di = od * a.sd + doff;
                const int hi = ho * a.sh + hoff;
                const int wi = wo * a.sw + woff;
                if ((unsigned)di < (unsigned)a.Di && (unsigned)hi < (unsigned)a.Hi && (unsigned)wi < (unsigned)a.Wi)
                    v = *reinterpret_cast<const VT*>(b_src + ((((int)n * a.Di + di) * a.Hi + hi) * a.Wi + wi) * a.Ctot);
            }
            rb[p] = v;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int p = 0; p < A_PASSES; ++p) {
            const int row = a_row0 + p * A_RPP;
            if (A_PASSES * A_RPP <= BK || row < BK)
                *reinterpret_cast<VT*>(sA + row * PA + a_col) = ra[p];
        }
#pragma unroll
        for (int p = 0; p < B_PASSES; ++p) {
            const int row = b_row0 + p * B_RPP;
            if (B_PASSES * B_RPP <= BK || row < BK)
                *reinterpret_cast<VT*>(sB + row * PB + b_col) = rb[p];
        }
    };

    // wave tile and the lane's fragment offsets inside it
    const int wm0 = (wave % WM) * WTM, wn0 = (wave / WM) * WTN;
    const int g16 = lane >> 4;
    const int frag_row = (ATOM == 32 ? (g16 >> 1) * 8 : g16 * 8) + ((lane & 15) >> 2);
    const int frag_col = (ATOM == 32 ? (g16 & 1) * 16 : 0) + (lane & 3) * 4;

    typedef typename std::conditional<ATOM == 32, f32x16, f32x4>::type AccT;
    AccT acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = AccT{0};

    if (niter > 0) {
        gload(r_begin);
        sstore();
        __syncthreads();
    }
    for (int it = 0; it < niter; ++it) {
        const bool more = it + 1 < niter;
        if (more) gload(r_begin + (it + 1) * BK);   // next tile waits in registers
#pragma unroll
        for (int ks = 0; ks < BK / AK; ++ks) {
            i16x8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = tr_frag(sA + (ks * AK + frag_row) * PA + wm0 + i * ATOM + frag_col, PA);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = tr_frag(sB + (ks * AK + frag_row) * PB + wn0 + j * ATOM + frag_col, PB);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (ATOM == 32)
                        mfma_step32<F16>(af[i], bf[j], acc[i][j]);
                    else
                        mfma_step16<F16>(af[i], bf[j], acc[i][j]);
                }
        }
        if (more) {
            __syncthreads();
            sstore();
            __syncthreads();
        }
    }

    // ---- epilogue: element (m, j) of the merged tile is dW[g0 + gi, k, tap, c]
    // with m = gi*kpg + k and j = tap*Gm*cpg + gj*cpg + c; only gi == gj is real.
    void* out = a.out;
    const int64_t zoff = a.out_mode == OUT_WORKSPACE ? (int64_t)z * a.slice_elems : 0;
    const int mbase = gb * a.gkpg;   // first dW row of this group block
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = wn0 + j * ATOM + (ATOM == 32 ? (lane & 31) : (lane & 15));
        const int jg = n0 + col;
        if (jg >= a.Nm) continue;
        const int t2 = jg / a.gcpg;
        const int rem = jg - t2 * a.gcpg;
        const int gj = rem / a.cpg;
        const int c = rem - gj * a.cpg;
        const int col_off = t2 * a.cpg + c;
        const int mlo = gj * a.kpg, mhi = mlo + a.kpg;   // rows of the diagonal block
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int v = 0; v < (ATOM == 32 ? 16 : 4); ++v) {
                const int row = ATOM == 32 ? wm0 + i * 32 + 8 * (v / 4) + 4 * (lane / 32) + (v % 4)
                                           : wm0 + i * 16 + 4 * (lane / 16) + v;
                const int mg = m0 + row;
                if (mg < mlo || mg >= mhi || mg >= a.Mm) continue;
                const int64_t e = (int64_t)(mbase + mg) * a.row_len + col_off;
                store_out(out, a.out_mode, zoff + e, acc[i][j][v]);
            }
        }
    }
}

// dW[e] = round(sum_z ws[z][e]) in fp32, in one fixed order: z-lane l of a
// workgroup sums slices l, l+ZL, l+2ZL, ... (in groups of four into four
// running sums, the rest into the first, the four added in a fixed order),
// then the ZL lane sums are combined by a fixed binary tree. The order
// depends only on (S, ZL), so a plan always produces the same bits. Splitting the slices over ZL lanes
// keeps the grid wide when dW is small and S is large.
__global__ __launch_bounds__(256) void reduce_kernel(const ReduceArgs a) {
    __shared__ f32x4 part[256];
    const int zl = a.zl;
    const int eg = 256 / zl;                 // element vectors per workgroup
    const int t = threadIdx.x;
    const int lane_e = t % eg, lane_z = t / eg;
    const int v = blockIdx.x * eg + lane_e;   // element vector index
    const int nvec = a.vec4 ? a.elems / 4 : a.elems;
    // four independent running sums (slices z, z+zl, z+2zl, z+3zl of each
    // group of four) keep four loads in flight; they are added in a fixed order
    f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, p2 = p0, p3 = p0;
    if (v < nvec) {
        const int64_t stride = (int64_t)zl * a.elems;
        if (a.vec4) {
            const float* w = a.ws + (int64_t)lane_z * a.elems + 4 * v;
            int z = lane_z;
            for (; z + 3 * zl < a.S; z += 4 * zl, w += 4 * stride) {
                p0 += *reinterpret_cast<const f32x4*>(w);
                p1 += *reinterpret_cast<const f32x4*>(w + stride);
                p2 += *reinterpret_cast<const f32x4*>(w + 2 * stride);
                p3 += *reinterpret_cast<const f32x4*>(w + 3 * stride);
            }
            for (; z < a.S; z += zl, w += stride) p0 += *reinterpret_cast<const f32x4*>(w);
        } else {
            for (int z = lane_z; z < a.S; z += zl) p0[0] += a.ws[(int64_t)z * a.elems + v];
        }
    }
    const f32x4 acc = (p0 + p1) + (p2 + p3);
    part[t] = acc;
    // the zl slice lanes of an element are combined by a binary tree in LDS
    // (lane z takes lane z + h, h = zl/2, zl/4, ..., 1): a fixed order, and
    // log2(zl) steps instead of a zl-long chain in one thread
    for (int h = zl >> 1; h >= 1; h >>= 1) {
        __syncthreads();
        if (lane_z < h) part[t] += part[t + h * eg];
    }
    __syncthreads();
    if (lane_z == 0 && v < nvec) {
        const f32x4 s = part[lane_e];
        if (a.vec4) {
#pragma unroll
            for (int k = 0; k < 4; ++k) store_out(a.dw, a.out_mode, 4 * v + k, s[k]);
        } else {
            store_out(a.dw, a.out_mode, v, s[0]);
        }
    }
}

template <bool F16>
__device__ __forceinline__ void widen8(const u32x4& v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t w = v[k];
        if constexpr (F16) {
            f[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
            f[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
        } else {
            f[2 * k] = __uint_as_float(w << 16);
            f[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
        }
    }
}

// Depthwise: thread (cv, pl) owns channels c0..c0+7 and a contiguous run of
// reduction positions; partial sums over the workgroup's position lanes are
// combined with lane shuffles and LDS before the store.
template <int TY, int TX, bool F16>
__global__ __launch_bounds__(256) void dw_kernel(const DwArgs a) {
    constexpr int T = TY * TX;
    const int tid = threadIdx.x;
    const int cl = a.cl;
    const int npl = 256 / cl;
    const int cv = tid % cl, pl = tid / cl;
    const int L = blockIdx.x;
    const int cb = L % a.cblocks, z = L / a.cblocks;
    const int c0 = (cb * cl + cv) * 8;
    const int r_begin = z * a.kslice;
    const int r_end = min(a.R, r_begin + a.kslice);
    const int len = max(0, r_end - r_begin);
    const int per = (len + npl - 1) / npl;
    const int ra = r_begin + pl * per;
    const int rb = min(r_end, ra + per);

    float acc[T][8];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[t][k] = 0.f;

    if (ra < rb) {
        const uint32_t q1 = magic_div((uint32_t)ra, a.mWo);
        int wo = ra - (int)q1 * a.Wo;
        int n = (int)magic_div(q1, a.mHo);
        int ho = (int)q1 - n * a.Ho;
        for (int r = ra; r < rb; ++r) {
            float d[8];
            widen8<F16>(*reinterpret_cast<const u32x4*>(a.dy + (int64_t)r * a.C + c0), d);
#pragma unroll
            for (int y = 0; y < TY; ++y) {
                const int hi = ho * a.sh - a.ph + y * a.dh;
                if ((unsigned)hi >= (unsigned)a.Hi) continue;
#pragma unroll
                for (int x = 0; x < TX; ++x) {
                    const int wi = wo * a.sw - a.pw + x * a.dw;
                    if ((unsigned)wi >= (unsigned)a.Wi) continue;
                    float xv[8];
                    widen8<F16>(*reinterpret_cast<const u32x4*>(a.x + ((int64_t)(n * a.Hi + hi) * a.Wi + wi) * a.C + c0), xv);
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc[y * TX + x][k] += d[k] * xv[k];
                }
            }
            if (++wo == a.Wo) {
                wo = 0;
                if (++ho == a.Ho) { ho = 0; ++n; }
            }
        }
    }
    // reduce over the position lanes of each wave (lanes cl apart)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float v = acc[t][k];
            for (int off = cl; off < 64; off <<= 1) v += __shfl_xor(v, off);
            acc[t][k] = v;
        }
    __shared__ float part[4][8][T * 8];   // [wave][cv][tap*8 + channel]
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
        const float s = part[0][v][w] + part[1][v][w] + part[2][v][w] + part[3][v][w];
        const int c = (cb * cl + v) * 8 + k;
        store_out(a.out, a.out_mode, zoff + (int64_t)c * T + t, s);
    }
}

// ---------------------------------------------------------------- dispatch

template <int BM, int BN, int BK, int WM, int WN, int ATOM, bool F16>
int launch_tile_v(int V, const MfmaArgs& a, hipStream_t s) {
    dim3 grid(a.total_wg), block(256);
    switch (V) {
        case 8: hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, ATOM, 8, F16>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, ATOM, 4, F16>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, ATOM, 2, F16>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, ATOM, 1, F16>), grid, block, 0, s, a); break;
    }
    return (int)hipGetLastError();
}

template <bool F16>
int launch_tile(int tile, int V, const MfmaArgs& a, hipStream_t s) {
    switch (tile) {
        case 1: return launch_tile_v<64, 64, 32, 2, 2, 32, F16>(V, a, s);
        case 2: return launch_tile_v<64, 128, 32, 2, 2, 32, F16>(V, a, s);
        case 3: return launch_tile_v<128, 128, 32, 2, 2, 32, F16>(V, a, s);
        case 4: return launch_tile_v<32, 128, 32, 1, 4, 32, F16>(V, a, s);
        case 5: return launch_tile_v<16, 128, 32, 1, 4, 16, F16>(V, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

template <bool F16>
int launch_dw_t(int ty, int tx, const DwArgs& a, hipStream_t s) {
    dim3 grid(a.total_wg), block(256);
    if (ty == 3 && tx == 3) hipLaunchKernelGGL((dw_kernel<3, 3, F16>), grid, block, 0, s, a);
    else if (ty == 1 && tx == 3) hipLaunchKernelGGL((dw_kernel<1, 3, F16>), grid, block, 0, s, a);
    else if (ty == 1 && tx == 5) hipLaunchKernelGGL((dw_kernel<1, 5, F16>), grid, block, 0, s, a);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace

int launch_mfma(const Plan& plan, const MfmaArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_tile<true>(plan.info.tile, plan.info.vector_width, a, s)
                       : launch_tile<false>(plan.info.tile, plan.info.vector_width, a, s);
}

int launch_depthwise(const Plan& plan, const DwArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_dw_t<true>(plan.dw_tile_y, plan.dw_tile_x, a, s)
                       : launch_dw_t<false>(plan.dw_tile_y, plan.dw_tile_x, a, s);
}

int launch_reduce(const ReduceArgs& a, int64_t grid, void* stream) {
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

}  // namespace wgrad
