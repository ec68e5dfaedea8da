// Depthwise (C/G = K/G = 1) backward-weight kernel for gfx950, tile form:
// 3x3 filters with unit stride and dilation on both axes.
//
// The depthwise case of the Composable Kernel wgrad page has no matrix to
// speak of: per channel, dW[y][x] = sum over (n, ho, wo) of dY * X at the
// tap's offset, bound by streaming X and dY once from HBM. rocm-libraries PR
// 12359 widens its loads by merging adjacent groups; here a lane owns 8
// adjacent channels (one 16-byte load per pixel) and a wave-load covers 64
// lanes, so every load is 1 KB of whole channel runs (whole pixels when a
// workgroup takes 512 channels).
//
// Work: output tiles of th rows x TW columns x CB channels (TW = 14 for 512
// channels, 28 for 256). A workgroup has kDwtCompute + 1 waves:
// * the last wave streams the tile's th + 2 input rows, TW + 2 pixels each,
//   into a ring of kDwtRing LDS rows with direct buffer-to-LDS loads (one
//   1 KB instruction per pixel or pixel pair; padding and the image edge load
//   zeros), keeping three rows in flight and waiting for each with an exact
//   vector-memory count;
// * compute wave w owns output columns 2w and 2w + 1 (of every 64 / (CB / 8)
//   lane group); it walks the tile's rows, loads its two dY pixels kDwtAhead
//   rows ahead into registers, reads the new input row's four pixels it needs
//   from LDS once and keeps the three rows of the window packed in registers,
//   so each (channel, tap) accumulator takes both columns' products in one
//   v_dot2.
// One workgroup barrier per output row hands the ring over. The input halo of
// a tile is one row above and below and one column each side: 1.31x the input
// in load requests on 14 x 14 tiles, all of which hit L2 except the first
// reader's, since the tiles of one image are numbered together and sit on
// one XCD.
//
// A workgroup takes tiles z, z + S, ... of its channel block; at the end its
// compute waves' accumulators are summed through LDS in a fixed order and
// stored as one split-K partial (S > 1) or as dW.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;

constexpr int kDwtAhead = 2;           // dY rows loaded ahead of the row computed (3 and 5 measured slower)
constexpr int kDwtRot = 3;             // step unroll: the window ring (3) and the dY buffers rotate statically
static_assert(kDwtAhead >= 1 && kDwtAhead < kDwtRot && kDwtRot % 3 == 0, "dY buffers");

// wait until at most `later` rows of PER loads each are outstanding
template <int MAXL, int PER>
__device__ __forceinline__ void wait_rows(int later) {
    if constexpr (MAXL > 0) {
        if (later >= MAXL) {
            __builtin_amdgcn_s_waitcnt(kWaitVm<MAXL * PER>);
            return;
        }
        wait_rows<MAXL - 1, PER>(later);
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    }
}

template <int CB>
struct DwtGeom {
    static constexpr int LP = CB / 8;                 // lanes per pixel
    static constexpr int PW = 64 / LP;                // pixels per wave-load
    static constexpr int TW = dwt_tile_w(CB);         // output columns per tile
    static constexpr int ROWB = dwt_row_bytes(CB);    // ring row bytes
    static constexpr int INS = ROWB / 1024;           // 1 KB loads per ring row
    static_assert(TW == 2 * kDwtCompute * PW, "two columns per lane");
    static_assert(ROWB % 1024 == 0 && ROWB >= (TW + 2) * CB * 2, "ring row of whole loads");
    static_assert((kDwtRing - 3) * INS <= 63, "outstanding loads of the streaming wave");
    static_assert(kDwtRing >= 4, "ring holds the window and one row in flight");
    static_assert(dwt_lds_bytes(CB) <= 160 * 1024, "LDS");
};

// the three window rows packed as (column j, column j + 1) pairs of one
// channel, for the three column offsets of the filter
struct WinRow {
    uint32_t lo[4][3], hi[4][3];
};

__device__ __forceinline__ void pack_win(const u32x4* px, WinRow& r) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            r.lo[w][j] = pair_lo(px[j][w], px[j + 1][w]);
            r.hi[w][j] = pair_hi(px[j][w], px[j + 1][w]);
        }
}

// The streaming wave's part of one tile: rows r = 0 .. rows + 1 of the
// source (row ys + r of image n, pixels xs .. xs + TW + 1, channels cbase ..
// cbase + CB - 1 of C; zeros outside H x W) into ring slot r % kDwtRing, with
// the workgroup barriers of the compute waves' steps: one before the first
// step (rows 0..2 landed) and one after each step s (row s + 3 landed).
template <int CB>
__device__ __forceinline__ void stream_tile(const u32x4& desc, uint32_t lds0, int lane, int n, int ys, int xs, int H,
                                            int W, int C, int cbase, int rows) {
    using G = DwtGeom<CB>;
    const int R = rows + 2;
    auto issue = [&](int r) {
        const int yy = ys + r;
        const bool rok = (unsigned)yy < (unsigned)H;
        const uint32_t slot = lds0 + (uint32_t)((r % kDwtRing) * G::ROWB);
#pragma unroll
        for (int i = 0; i < G::INS; ++i) {
            const int b = i * 1024 + lane * 16;
            const int j = b / (CB * 2), cbyte = b - j * (CB * 2);
            const int xx = xs + j;
            const bool ok = rok && j < G::TW + 2 && (unsigned)xx < (unsigned)W;
            const uint32_t off = ok ? (uint32_t)((((n * H + yy) * W + xx) * C + cbase) * 2 + cbyte) : kBufOob;
            dma_load16(desc, slot + (uint32_t)(i * 1024), off);
        }
    };
    // prologue: the first rows, at most three in flight; rows 0..2 must have
    // landed before the first barrier
    const int pro = min(kDwtRing, R);
    for (int r = 0; r < pro; ++r) {
        if (r >= 3) wait_rows<2, G::INS>(2);
        issue(r);
    }
    wait_rows<3, G::INS>(pro - 3);
    __builtin_amdgcn_s_barrier();
    int last = pro - 1;
    for (int s = 0; s < rows; ++s) {
        // compute step s reads row s + 2; row s - 1 was read at step s - 3
        // or earlier, so its slot takes row s - 1 + kDwtRing
        if (s >= 1 && s - 1 + kDwtRing < R) {
            last = s - 1 + kDwtRing;
            issue(last);
        }
        if (s + 1 < rows) wait_rows<3, G::INS>(last - (s + 3));
        __builtin_amdgcn_s_barrier();
    }
}

template <int CB, bool F16>
__global__ __launch_bounds__(64 * (kDwtCompute + 1), 1) void dwtile_kernel(const DwTileArgs a) {
    using G = DwtGeom<CB>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    // channel block slowest: the tiles of one block are numbered together, so
    // an XCD holds whole images of one block (their halo rows and columns
    // come from its L2). Measured on the 512-channel 56x56 shape, this beats
    // taking both blocks of a tile on one XCD by 0.4 us: with the blocks
    // fastest the workgroups of block 0 finished 0.8 us after those of
    // block 1 (in either block order, so it is the placement, not the
    // address half).
    const int cb = L / a.S, z = L - (L / a.S) * a.S;
    const uint32_t lds0 = lds_addr(smem);

    auto tile_of = [&](int t, int& n, int& y0, int& x0, int& rows) {
        const int tx = t % a.tiles_x;
        const int r = t / a.tiles_x;
        const int ty = r % a.tiles_y;
        n = r / a.tiles_y;
        y0 = ty * a.th;
        x0 = tx * G::TW;
        rows = min(a.th, a.Ho - y0);
    };

    if (wave == kDwtCompute) {
        // ---- the streaming wave
        const u32x4 desc = buf_desc(a.x, a.x_bytes);
        for (int t = z; t < a.tiles; t += a.S) {
            int n, y0, x0, rows;
            tile_of(t, n, y0, x0, rows);
            // input row r of the tile is image row y0 - ph + r
            stream_tile<CB>(desc, lds0, lane, n, y0 - a.ph, x0 - a.pw, a.Hi, a.Wi, a.C, cb * CB, rows);
        }
        // every load has landed (the last row was waited for before the last
        // step); the epilogue's barrier
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
        lds_barrier();
    } else {
        // ---- compute waves
        const int pw_ = lane / G::LP, ch = lane % G::LP;
        const int colA = (wave * G::PW + pw_) * 2;         // first of the lane's two output columns
        const __amdgpu_buffer_rsrc_t dy_rs = buf_rsrc(a.dy, a.dy_bytes);
        const uint32_t cbase = (uint32_t)(cb * CB + ch * 8) * 2;
        float acc[9][8];
#pragma unroll
        for (int t = 0; t < 9; ++t)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[t][k] = 0.f;

        for (int t = z; t < a.tiles; t += a.S) {
            int n, y0, x0, rows;
            tile_of(t, n, y0, x0, rows);
            auto load_dy = [&](int s, u32x4* d) {
                const int ho = y0 + s;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int wo = x0 + colA + q;
                    const bool ok = s < rows && wo < a.Wo;
                    d[q] = buf_load16(dy_rs, ok ? (uint32_t)((n * a.Ho + ho) * a.Wo + wo) * (uint32_t)(a.C * 2) + cbase
                                                : kBufOob);
                }
            };
            auto read_row = [&](int r, WinRow& w) {
                const uint8_t* p = smem + (r % kDwtRing) * G::ROWB + colA * CB * 2 + ch * 16;
                u32x4 px[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) px[j] = *reinterpret_cast<const u32x4*>(p + j * CB * 2);
                pack_win(px, w);
            };
            u32x4 dbuf[kDwtRot][2];
#pragma unroll
            for (int s = 0; s < kDwtAhead; ++s) load_dy(s, dbuf[s]);
            WinRow win[3];
            lds_barrier();
            read_row(0, win[0]);
            read_row(1, win[1]);
            // step s: output row y0 + s with window rows s, s + 1, s + 2 in
            // win[s % 3], win[(s + 1) % 3], win[(s + 2) % 3] and its dY in
            // dbuf[s % kDwtRot]; unrolled by kDwtRot so that both rotate
            // statically
            auto step = [&](int s, auto rot) {
                constexpr int U = decltype(rot)::value;   // s % kDwtRot
                if (s >= rows) return;
                load_dy(s + kDwtAhead, dbuf[(U + kDwtAhead) % kDwtRot]);
                read_row(s + 2, win[(U + 2) % 3]);
                const u32x4* d = dbuf[U];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t dlo = pair_lo(d[0][w], d[1][w]);
                    const uint32_t dhi = pair_hi(d[0][w], d[1][w]);
#pragma unroll
                    for (int ky = 0; ky < 3; ++ky)
#pragma unroll
                        for (int kx = 0; kx < 3; ++kx) {
                            const WinRow& r = win[(U + ky) % 3];
                            acc[ky * 3 + kx][2 * w] = dot2<F16>(dlo, r.lo[w][kx], acc[ky * 3 + kx][2 * w]);
                            acc[ky * 3 + kx][2 * w + 1] = dot2<F16>(dhi, r.hi[w][kx], acc[ky * 3 + kx][2 * w + 1]);
                        }
                }
                lds_barrier();
            };
            for (int s = 0; s < rows; s += kDwtRot) {
                step(s, std::integral_constant<int, 0>{});
                step(s + 1, std::integral_constant<int, 1>{});
                step(s + 2, std::integral_constant<int, 2>{});
            }
        }
        // The ring is free (every wave passed the last row's barrier): park
        // the accumulators there in dW order. Lanes q*32 + chunk (q = 0, 1)
        // hold channels chunk*8 .. chunk*8+7 of the block for two different
        // columns, i.e. the 72 dW elements from chunk*72 on, channel-major
        // like dW, as v[k*9 + t] = acc[t][k]. One v_permlane32_swap per pair
        // (v[m], v[m + 36]) and an add leave lane chunk with the two columns'
        // sum of v[m] and lane 32 + chunk with that of v[m + 36], so the wave
        // writes part[w][chunk*72 + 36*q + m] and element o of the block is
        // part[w][o] for every compute wave w.
        static_assert(G::PW == 2, "two pixel slots per wave");
        float* part = reinterpret_cast<float*>(smem) + wave * (CB * 9) + ch * 72 + 36 * pw_;
#pragma unroll
        for (int e = 0; e < 36; e += 4) {
            f32x4 v;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i = e + m, j = e + m + 36;
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i % 9][i / 9]),
                                                                __float_as_uint(acc[j % 9][j / 9]), false, false);
                v[m] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            }
            *reinterpret_cast<f32x4*>(part + e) = v;
        }
        lds_barrier();
    }
    // ---- sum the compute waves' accumulators in a fixed order and store
    // four consecutive dW elements per thread (the block's run of CB*9
    // elements is contiguous in dW and in the workspace slice)
    const float* part = reinterpret_cast<const float*>(smem);
    const int64_t base = (int64_t)cb * CB * 9;
    // this workgroup's workspace slice (partials only)
    const __amdgpu_buffer_rsrc_t ws = buf_rsrc(static_cast<float*>(a.out) + (int64_t)z * a.slice_elems,
                                               4u * (uint32_t)a.slice_elems);
    for (int o = threadIdx.x * 4; o < CB * 9; o += 4 * 64 * (kDwtCompute + 1)) {
        f32x4 sum = *reinterpret_cast<const f32x4*>(part + o);
#pragma unroll
        for (int w = 1; w < kDwtCompute; ++w) sum += *reinterpret_cast<const f32x4*>(part + w * (CB * 9) + o);
        if (a.out_mode == OUT_WORKSPACE) {
            store_partial4(ws, (int64_t)cb * CB * 9 + o, sum);
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) store_out(a.out, a.out_mode, base + o + m, sum[m]);
        }
    }
}

// ---- backward data: with unit stride and dilation, dX of a depthwise 3x3
// layer is dY correlated with the flipped filter,
//   dX[y][x] = sum over ky, kx of dY[y + ph - ky][x + pw - kx] * w[ky][kx],
// so a dX tile needs the dY rows y0 + ph - 2 .. y0 + th - 1 + ph and
// columns x0 + pw - 2 .. x0 + TW - 1 + pw: ring row r is dY row
// y0 + ph - 2 + r and output row s reads ring rows s .. s + 2, the same
// window walk as the weight gradient above. A lane's two output columns c,
// c + 1 read window pixels c .. c + 3; with the pixels packed as (j, j + 1)
// pairs, column c + q takes taps (kx = 1, kx = 0) from pair q + 1 and tap
// kx = 2 from the low half of pair q, i.e. two v_dot2 per filter row against
// the weight pairs (w[ky][1], w[ky][0]) and (w[ky][2], 0). No reduction over
// workgroups: each lane stores its dX pixels as it goes.
template <int CB, bool F16>
__global__ __launch_bounds__(64 * (kDwtCompute + 1), 1) void dgrad_dwtile_kernel(const DgradDwTileArgs a) {
    using G = DwtGeom<CB>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wg = xcd_logical_id(blockIdx.x, a.total_wg);
    const uint32_t lds0 = lds_addr(smem);
    const int T = a.tiles * a.cblocks;
    // tile t of all blocks: block t / tiles (slowest, so consecutive
    // workgroups on one XCD share an image's halo rows), then image, tile row,
    // tile column
    auto tile_of = [&](int t, int& cb, int& n, int& y0, int& x0, int& rows) {
        cb = t / a.tiles;
        const int u = t - cb * a.tiles;
        const int tx = u % a.tiles_x;
        const int r = u / a.tiles_x;
        const int ty = r % a.tiles_y;
        n = r / a.tiles_y;
        y0 = ty * a.th;
        x0 = tx * G::TW;
        rows = min(a.th, a.Hi - y0);
    };
    if (wave == kDwtCompute) {
        const u32x4 desc = buf_desc(a.dy, a.dy_bytes);
        for (int t = wg; t < T; t += a.total_wg) {
            int cb, n, y0, x0, rows;
            tile_of(t, cb, n, y0, x0, rows);
            stream_tile<CB>(desc, lds0, lane, n, y0 + a.ph - 2, x0 + a.pw - 2, a.Ho, a.Wo, a.C, cb * CB, rows);
        }
        return;
    }
    const int pw_ = lane / G::LP, ch = lane % G::LP;
    const int colA = (wave * G::PW + pw_) * 2;
    for (int t = wg; t < T; t += a.total_wg) {
        int cb, n, y0, x0, rows;
        tile_of(t, cb, n, y0, x0, rows);
        const int c0 = cb * CB + ch * 8;                 // the lane's first channel
        // weight pairs of the lane's 8 channels (GKYXC with one channel per
        // group: channel c's taps are elements 9c .. 9c + 8)
        uint32_t wv[36];
        {
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(a.w + (int64_t)c0 * 9);
#pragma unroll
            for (int i = 0; i < 36; ++i) wv[i] = wp[i];
        }
        auto w16 = [&](int e) -> uint32_t { return (e & 1) ? wv[e >> 1] >> 16 : wv[e >> 1] & 0xffffu; };
        uint32_t wa[8][3], wb[8][3];
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int ky = 0; ky < 3; ++ky) {
                wa[k][ky] = w16(9 * k + 3 * ky + 1) | (w16(9 * k + 3 * ky) << 16);
                wb[k][ky] = w16(9 * k + 3 * ky + 2);
            }
        auto read_row = [&](int r, WinRow& w) {
            const uint8_t* p = smem + (r % kDwtRing) * G::ROWB + colA * CB * 2 + ch * 16;
            u32x4 px[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) px[j] = *reinterpret_cast<const u32x4*>(p + j * CB * 2);
            pack_win(px, w);
        };
        WinRow win[3];
        lds_barrier();
        read_row(0, win[0]);
        read_row(1, win[1]);
        auto step = [&](int s, auto rot) {
            constexpr int U = decltype(rot)::value;   // s % 3
            if (s >= rows) return;
            read_row(s + 2, win[(U + 2) % 3]);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float o[8];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float lo = 0.f, hi = 0.f;
                    // ring row s + 2 - ky; the row read at this step last, so
                    // that its LDS reads are in flight while the other two
                    // rows are used
#pragma unroll
                    for (int ky = 2; ky >= 0; --ky) {
                        const WinRow& r = win[(U + 2 - ky) % 3];
                        lo = dot2<F16>(r.lo[w][q + 1], wa[2 * w][ky], lo);
                        lo = dot2<F16>(r.lo[w][q], wb[2 * w][ky], lo);
                        hi = dot2<F16>(r.hi[w][q + 1], wa[2 * w + 1][ky], hi);
                        hi = dot2<F16>(r.hi[w][q], wb[2 * w + 1][ky], hi);
                    }
                    o[2 * w] = lo;
                    o[2 * w + 1] = hi;
                }
                const int xo = x0 + colA + q;
                if (xo < a.Wi) {
                    const int64_t e = ((int64_t)(n * a.Hi + y0 + s) * a.Wi + xo) * a.C + c0;
                    // streaming stores: dX is not read again here (on the
                    // 512-channel 56x56 shape they cut the kernel from 27.0
                    // to 24.2 us against plain stores)
                    if (a.out_mode == OUT_FP32) {
                        float* d = static_cast<float*>(a.dx) + e;
                        __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(d));
                        __builtin_nontemporal_store(f32x4{o[4], o[5], o[6], o[7]}, reinterpret_cast<f32x4*>(d + 4));
                    } else {
                        // round to nearest even in hardware (v_cvt_pk_bf16_f32,
                        // v_cvt_f16_f32)
                        u32x4 v;
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            if (a.out_mode == OUT_BF16)
                                v[m] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)o[2 * m], (__bf16)o[2 * m + 1]});
                            else
                                v[m] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)o[2 * m], (_Float16)o[2 * m + 1]});
                        }
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.dx) + e));
                    }
                }
            }
            lds_barrier();
        };
        for (int s = 0; s < rows; s += 3) {
            step(s, std::integral_constant<int, 0>{});
            step(s + 1, std::integral_constant<int, 1>{});
            step(s + 2, std::integral_constant<int, 2>{});
        }
    }
}

template <int CB, bool F16>
int launch_cb(const DwTileArgs& a, hipStream_t s) {
    auto k = dwtile_kernel<CB, F16>;
    constexpr int lds = dwt_lds_bytes(CB);
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(k, dim3(a.total_wg), dim3(64 * (kDwtCompute + 1)), lds, s, a);
    return (int)hipGetLastError();
}

template <bool F16>
int launch_t(int cb, const DwTileArgs& a, hipStream_t s) {
    return cb == 256 ? launch_cb<256, F16>(a, s) : (int)hipErrorInvalidValue;
}

}  // namespace

template <int CB, bool F16>
int launch_dg(const DgradDwTileArgs& a, hipStream_t s) {
    auto k = dgrad_dwtile_kernel<CB, F16>;
    constexpr int lds = kDwtRing * dwt_row_bytes(CB);
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(k, dim3(a.total_wg), dim3(64 * (kDwtCompute + 1)), lds, s, a);
    return (int)hipGetLastError();
}

int launch_dgrad_dwtile(const Plan& plan, const DgradDwTileArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan.dg_dwt != 256) return (int)hipErrorInvalidValue;
    return plan.in_f16 ? launch_dg<256, true>(a, s) : launch_dg<256, false>(a, s);
}

int launch_dwtile(const Plan& plan, const DwTileArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_t<true>(plan.dwt_cb, a, s) : launch_t<false>(plan.dwt_cb, a, s);
}

}  // namespace wgrad
