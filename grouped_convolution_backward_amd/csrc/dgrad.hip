// Backward data (dgrad) of the grouped convolution on gfx950.
//
// Per group the input gradient is a GEMM over the (filter tap, output
// channel) pairs:
//
//   dX[m][c] = sum_{t, k} A[m][(t, k)] * B[(t, k)][c],
//   A[m][(t, k)] = dY at the output position whose tap t reads position m
//                  (zero when that position does not exist),
//   B[(t, k)][c] = W[k][t][c]    (GK[Z]YXC),
//
// with m = (n, di, hi, wi) the input positions. The reduction runs one tap at
// a time in chunks of BK output channels. As in the dgrad part of
// rocm-libraries PR 11602 (transpose load for bwd weight and bwd data), only
// the B tile is staged K-outer ([k][c], straight from the weight's
// channel-contiguous rows) and read with the CDNA4 transposed LDS read
// ds_read_b64_tr_b16; the A tile stays M-outer ([m][k], each row one
// contiguous run of dY channels), which is already the MFMA operand layout,
// so a plain 16-byte LDS read serves it.
// Every dX element is written once: no workspace and no split of the
// reduction, so the result is deterministic. Small groups are merged Gm at a
// time into one block-diagonal GEMM (the group merging that rocm-libraries
// PR 12359 applies to backward weight): the A tile is then a contiguous run
// of Gm*K/G dY channels and the B tile holds zeros where a row's group
// differs from a column's. Strided problems are split into stride phases
// (see DgradArgs), so every workgroup walks only taps that reach its
// positions. Depthwise shapes (C/G = K/G = 1) have their own channel-vector
// kernels at the end of this file.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"

namespace wgrad {
namespace {

using namespace dev;

// V 16-bit elements (V = 8, 4, 2, 1) from a raw buffer; an out-of-range
// offset returns zeros without touching memory
template <int V> struct BufVec;
template <> struct BufVec<8> {
    static __device__ __forceinline__ u32x4 load(__amdgpu_buffer_rsrc_t r, uint32_t o) { return buf_load16(r, o); }
};
template <> struct BufVec<4> {
    static __device__ __forceinline__ u32x2 load(__amdgpu_buffer_rsrc_t r, uint32_t o) { return buf_load8(r, o); }
};
template <> struct BufVec<2> {
    static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
    }
};
template <> struct BufVec<1> {
    static __device__ __forceinline__ uint16_t load(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, 0);
    }
};

__device__ __forceinline__ void widen8(const u32x4& v, float* f, bool f16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = v[i];
        if (f16) {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
        } else {
            f[2 * i] = __uint_as_float(u << 16);
            f[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
        }
    }
}

// Streaming (nontemporal) stores: dX is not read again by the kernel; on
// the strided and 3D shapes they cut the flat kernel by 1.6-2.3 us against
// plain stores (the row-ring kernel measured no difference).
__device__ __forceinline__ void store8(void* out, int mode, int64_t e, const float* v) {
    if (mode == OUT_FP32) {
        float* o = static_cast<float*>(out) + e;
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(o));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(o + 4));
        return;
    }
    u32x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo, hi;
        if (mode == OUT_FP16) {
            lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
            hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
            p[i] = lo | (hi << 16);
        } else {
            p[i] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2 * i], (__bf16)v[2 * i + 1]});   // one v_cvt_pk_bf16_f32
        }
    }
    __builtin_nontemporal_store(p, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + e));
}

template <int BM, int BN, int BK, int WM, int WN, int V, bool PH, bool F16>
__global__ __launch_bounds__(256) void dgrad_kernel(const DgradArgs a) {
    typedef typename VecT<V>::T VT;
    // BK output channels per reduction chunk. A rows are BK elements (64
    // bytes) with their 16-byte chunks XOR-swizzled by bits 2-3 of the row
    // (a_off): the 16 rows a 16-lane group reads at one chunk, and the 4
    // rows x 4 chunks a 16-lane group stores, each cover all 64 banks once.
    // (Rows padded to 80 bytes instead, the stores of 4 rows wrapped onto the
    // same banks: with the B stores below, a quarter of the LDS-active cycles
    // of the strided c3 launch were bank conflicts. Removing them took 0.2 us
    // off the 3D shape and the pointwise one and left c3 where it was: the
    // conflicts were mostly off the critical path.)
    constexpr int PA = BK;
    static_assert(BK == 32, "A swizzle: four 16-byte chunks per row");
    constexpr int PB = BN + kLdsPad;               // B row pitch for the transposed reads
    constexpr int WTM = BM / WM, WTN = BN / WN;    // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int AV = BK / V;                     // vectors per A row
    constexpr int A_LOADS = BM * AV / 256;         // A vectors per thread
    constexpr int BVR = BN / V;                    // vectors per B row
    constexpr int B_LOADS = (BK * BVR + 255) / 256;
    static_assert(WM * WN == 4 && FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert((BM * AV) % 256 == 0, "A loads");
    static_assert(A_LOADS + B_LOADS <= 63, "vmcnt range");

    // two LDS stages: chunk c is computed from stage c % 2 while chunk c + 1
    // is stored into the other one; the epilogue reuses the space (sized as
    // with 80-byte A rows, so that its passes stay as wide)
    constexpr int LDS_ELEMS = 2 * BM * (BK + 8) + 2 * BK * PB;
    auto a_off = [](int row, int e) { return row * PA + ((((e >> 3) ^ (row >> 2)) & 3) << 3) + (e & 7); };
    // B stores: with 64-channel rows of 16-byte vectors a 16-lane group
    // stores two rows, and on the 192-byte B pitch rows one apart share banks
    // while rows two apart do not, so each group takes rows r and r + 2 (a
    // permutation of the chunk's rows)
    auto b_row_of = [](int idx) {
        if constexpr (BN == 64 && V == 8) {
            static_assert(PB == 96 && BK * BN / V == 256, "B store order: one vector per thread, 192-byte rows");
            const int g = idx >> 4;
            return ((g >> 1) << 2) + (g & 1) + (((idx >> 3) & 1) << 1);
        } else {
            return idx / (BN / V);
        }
    };
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
    uint16_t* const sA[2] = {lds, lds + BM * PA};
    uint16_t* const sB[2] = {lds + 2 * BM * PA, lds + 2 * BM * PA + BK * PB};

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    // phase fastest: the phases of one tile read the same dY rows (PH: the
    // problem has a stride above 1; without, one phase and every tap). The
    // phases differ in work (1, 2, 2 and 4 taps at stride 2 with a 3x3
    // filter), and when the whole grid is resident the workgroups that share
    // a CU are the ones whose logical ids differ by the CUs of one XCD; so the
    // phase order within each group of tiles is rotated by one per CU round
    // (ph_rot groups), which gives each CU different phases. Unrotated, every
    // CU held workgroups of a single phase and the 4-tap CUs ran 2.4x longer
    // than the 1-tap ones (strided c3: kernel 26.6 us, its CUs ending between
    // 11 and 26.6 us).
    int r = L;
    const int phase = PH ? (r % a.phases + (r / a.phases / a.ph_rot) % a.phases) % a.phases : 0;
    if (PH) r /= a.phases;
    const int mt = r % a.tiles_m;
    r /= a.tiles_m;
    const int nt = r % a.tiles_n;
    const int gb = r / a.tiles_n;   // block of Gm merged groups
    const int m0 = mt * BM, c0 = nt * BN;
    const int ph_w = PH ? phase % a.sw : 0, ph_dh = PH ? phase / a.sw : 0;
    const int ph_h = PH ? ph_dh % a.sh : 0, ph_d = PH ? ph_dh / a.sh : 0;

    // this phase's taps per axis (host tables): first tap, count, and the
    // output offset od = i_d + o0 of the first one
    const int z0 = PH ? a.t0[0][ph_d] : 0, y0 = PH ? a.t0[1][ph_h] : 0, x0 = PH ? a.t0[2][ph_w] : 0;
    const int nz = PH ? a.nt[0][ph_d] : a.Zf, ny = PH ? a.nt[1][ph_h] : a.Yf, nx = PH ? a.nt[2][ph_w] : a.Xf;
    const int od0 = PH ? a.o0[0][ph_d] : a.pd, oh0 = PH ? a.o0[1][ph_h] : a.ph, ow0 = PH ? a.o0[2][ph_w] : a.pw;
    const int nchunks = nz * ny * nx * a.kchunks;

    // A rows this thread loads: phase-grid position m -> (n, i_d, i_h, i_w),
    // input (n, ph_d + i_d*sd, ph_h + i_h*sh, ph_w + i_w*sw)
    const int a_kv = (tid % AV) * V;
    int a_qd[A_LOADS], a_qh[A_LOADS], a_qw[A_LOADS];
    bool a_in[A_LOADS];
    // dY offset of output (n, i_d, i_h, i_w); a tap adds a constant. Unsigned
    // arithmetic: only the sum for a valid tap is a true offset.
    uint32_t a_base[A_LOADS];
    const int dy_g = gb * a.gkpg;   // element offsets of the group block
    const int w_g = gb * a.gkpg * a.taps * a.cpg;
#pragma unroll
    for (int p = 0; p < A_LOADS; ++p) {
        const int row = tid / AV + p * (256 / AV);
        const int m = m0 + row;
        const uint32_t mm = m < a.M ? (uint32_t)m : 0u;
        const uint32_t q1 = magic_div(mm, a.mqw);
        const uint32_t q2 = magic_div(q1, a.mqh);
        const uint32_t q3 = magic_div(q2, a.mqd);
        a_qw[p] = (int)(mm - q1 * (uint32_t)a.qw);
        a_qh[p] = (int)(q1 - q2 * (uint32_t)a.qh);
        a_qd[p] = (int)(q2 - q3 * (uint32_t)a.qd);
        const int n = (int)q3;
        const int di = ph_d + a_qd[p] * a.sd, hi = ph_h + a_qh[p] * a.sh, wi = ph_w + a_qw[p] * a.sw;
        a_in[p] = m < a.M && di < a.Di && hi < a.Hi && wi < a.Wi;
        a_base[p] = (uint32_t)dy_g +
                    (((uint32_t)(n * a.Do + a_qd[p]) * a.Ho + a_qh[p]) * a.Wo + a_qw[p]) * (uint32_t)a.Ktot + a_kv;
    }
    const __amdgpu_buffer_rsrc_t dy_rs = buf_rsrc(a.dy, a.dy_bytes);
    const __amdgpu_buffer_rsrc_t w_rs = buf_rsrc(a.w, a.w_bytes);
    // B rows and columns this thread loads; merged groups: row k carries
    // weights only for the columns of its own group, [wlo, wlo + kpg)
    int b_base[B_LOADS], b_row[B_LOADS], b_lo[B_LOADS];
    bool b_ok[B_LOADS];
#pragma unroll
    for (int p = 0; p < B_LOADS; ++p) {
        const int idx = tid + p * 256;
        const int row = b_row_of(idx), cv = (idx % BVR) * V;
        const int c = c0 + cv;
        const int gc = (int)magic_div((uint32_t)c, a.mcpg);
        b_row[p] = row;
        b_lo[p] = gc * a.kpg;
        b_ok[p] = row < BK && c < a.gcpg;
        b_base[p] = w_g + row * a.taps * a.cpg + c - gc * a.cpg;
    }

    // the chunk the next gload fetches: k-chunk kc of the phase's tap
    // (iz, iy, ix), advanced one chunk per call. Uniform across the
    // workgroup and kept incrementally (the scalar unit is shared by every
    // wave of the CU): a new k-chunk adds to k0 and kw, a new tap adjusts the
    // output offsets (od, oh, ow), the dY tap offset and the weight tap offset.
    int cur = 0, cur_kc = 0, cur_iy = 0, cur_ix = 0;   // the depth tap is the outermost: no counter
    int k0 = 0, kw = 0;                                     // k0 * taps * cpg
    int od = od0, oh = oh0, ow = ow0;
    uint32_t tapoff = ((uint32_t)(od0 * a.Ho + oh0) * a.Wo + ow0) * (uint32_t)a.Ktot;
    int wt = ((z0 * a.Yf + y0) * a.Xf + x0) * a.cpg;       // weight offset of the tap
    const uint32_t ost_w = (uint32_t)(a.xdo * a.Ktot), ost_h = (uint32_t)(a.ydo * a.Wo * a.Ktot),
                   ost_d = (uint32_t)(a.zdo * a.Ho * a.Wo * a.Ktot);
    const int wst_x = a.xstep * a.cpg, wst_y = a.ystep * a.Xf * a.cpg, wst_z = a.zstep * a.Yf * a.Xf * a.cpg;
    const int w_kstride = a.taps * a.cpg;
    auto advance = [&]() {
        ++cur;
        k0 += BK;
        kw += BK * w_kstride;
        if (++cur_kc < a.kchunks) return;
        cur_kc = 0;
        k0 = 0;
        kw = 0;
        if (++cur_ix < nx) {
            ow -= a.xdo;
            tapoff -= ost_w;
            wt += wst_x;
            return;
        }
        cur_ix = 0;
        ow = ow0;
        tapoff += (uint32_t)(nx - 1) * ost_w;
        wt -= (nx - 1) * wst_x;
        if (++cur_iy < ny) {
            oh -= a.ydo;
            tapoff -= ost_h;
            wt += wst_y;
            return;
        }
        cur_iy = 0;
        oh = oh0;
        tapoff += (uint32_t)(ny - 1) * ost_h;
        wt -= (ny - 1) * wst_y;
        od -= a.zdo;
        tapoff -= ost_d;
        wt += wst_z;
    };

    // two register sets: chunk c + 2 is loaded into the set chunk c came in.
    // Every load is issued (a masked element reads at an out-of-range
    // offset, which returns zeros), chunks past the last included, so each
    // chunk issues the same number of loads and the waits stay exact.
    VT ra[2][A_LOADS], rb[2][B_LOADS];
    auto gload = [&](VT* ra, VT* rb) {
        const bool live = cur < nchunks;
        const uint32_t toff = tapoff + k0;
        const bool kok = live && k0 + a_kv < a.gkpg;
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p) {
            const bool ok = kok && a_in[p] && (unsigned)(a_qd[p] + od) < (unsigned)a.Do &&
                            (unsigned)(a_qh[p] + oh) < (unsigned)a.Ho && (unsigned)(a_qw[p] + ow) < (unsigned)a.Wo;
            ra[p] = BufVec<V>::load(dy_rs, ok ? (a_base[p] + toff) * 2u : kBufOob);
        }
        const int wofs = kw + wt;
#pragma unroll
        for (int p = 0; p < B_LOADS; ++p) {
            const int k = k0 + b_row[p];
            const bool ok = live && b_ok[p] && (unsigned)(k - b_lo[p]) < (unsigned)a.kpg;
            rb[p] = BufVec<V>::load(w_rs, ok ? (uint32_t)(b_base[p] + wofs) * 2u : kBufOob);
        }
        advance();
    };
    auto sstore = [&](const VT* ra, const VT* rb, uint16_t* sa, uint16_t* sb) {
#pragma unroll
        for (int p = 0; p < A_LOADS; ++p) {
            const int row = tid / AV + p * (256 / AV);
            *reinterpret_cast<VT*>(sa + a_off(row, a_kv)) = ra[p];
        }
#pragma unroll
        for (int p = 0; p < B_LOADS; ++p) {
            const int idx = tid + p * 256;
            const int row = b_row_of(idx), cv = (idx % BVR) * V;
            if (row < BK) *reinterpret_cast<VT*>(sb + row * PB + cv) = rb[p];
        }
    };

    const int wm0 = (wave % WM) * WTM, wn0 = (wave / WM) * WTN;
    const int g16 = lane >> 4;
    const int frag_row = (g16 >> 1) * 8 + ((lane & 15) >> 2);   // transposed-read row
    const int frag_col = (g16 & 1) * 16 + (lane & 3) * 4;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{0};

    // Chunk c: its loads were issued two chunks earlier; compute it from LDS
    // stage c % 2, then store chunk c + 1 (loaded one chunk earlier) into the
    // other stage. One barrier per chunk: every thread has finished computing
    // from a stage before any thread stores into it again. The chunk count is
    // padded to even with an all-zero chunk, so the loop body has no branch.
    auto step = [&](int c, auto stage_tag) {
        constexpr int P = decltype(stage_tag)::value;
        gload(ra[P], rb[P]);   // chunk c + 2
        const uint16_t* sa = sA[P];
        const uint16_t* sb = sB[P];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            i16x8 af[FM], bf[FN];
            // A operand: row lane%32 of the wave's block, k = 8*(lane/32) .. +7
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const i16x8*>(sa + a_off(wm0 + i * 32 + (lane & 31), ks * 16 + 8 * (lane >> 5)));
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = tr_frag(sb + (ks * 16 + frag_row) * PB + wn0 + j * 32 + frag_col, PB);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) mfma_step32<F16>(af[i], bf[j], acc[i][j]);
        }
        // the loads of chunk c + 2 (issued above) may stay in flight
        __builtin_amdgcn_s_waitcnt(kWaitVm<A_LOADS + B_LOADS>);
        sstore(ra[1 - P], rb[1 - P], sA[1 - P], sB[1 - P]);
        __syncthreads();
    };
    gload(ra[0], rb[0]);
    gload(ra[1], rb[1]);
    __builtin_amdgcn_s_waitcnt(kWaitVm<A_LOADS + B_LOADS>);
    sstore(ra[0], rb[0], sA[0], sB[0]);
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        step(c + 1, std::integral_constant<int, 1>{});
    }

    // ---- epilogue: element (row, c) of the tile is dX[xpos(row)][gb*gcpg + c]
    // input position of tile row `row` (-1: none); one phase: the rows are
    // consecutive positions
    auto xpos = [&](int row) {
        const int m = m0 + row;
        if (!PH) return m < a.M ? m : -1;
        const uint32_t mm = m < a.M ? (uint32_t)m : 0u;
        const uint32_t q1 = magic_div(mm, a.mqw);
        const uint32_t q2 = magic_div(q1, a.mqh);
        const uint32_t q3 = magic_div(q2, a.mqd);
        const int wi = ph_w + (int)(mm - q1 * (uint32_t)a.qw) * a.sw;
        const int hi = ph_h + (int)(q1 - q2 * (uint32_t)a.qh) * a.sh;
        const int di = ph_d + (int)(q2 - q3 * (uint32_t)a.qd) * a.sd;
        const bool in = m < a.M && di < a.Di && hi < a.Hi && wi < a.Wi;
        return in ? (((int)q3 * a.Di + di) * a.Hi + hi) * a.Wi + wi : -1;
    };
    if constexpr (V == 8) {
        // 8-channel runs are whole and aligned: stage the tile in LDS as fp32
        // [m][c], EPC columns at a time, and write 16-byte (32-byte for
        // fp32) vectors of consecutive channels
        constexpr int EPC0 = (LDS_ELEMS * 2 / (BM * 4)) / 32 * 32;
        constexpr int EPC = EPC0 < BN ? EPC0 : BN;
        static_assert(EPC >= 32 && BN % EPC == 0, "epilogue passes");
        float* const stage = reinterpret_cast<float*>(lds);
#pragma unroll
        for (int pc = 0; pc < BN; pc += EPC) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = wn0 + j * 32;
                if (col < pc || col >= pc + EPC) continue;   // uniform per wave
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = wm0 + i * 32 + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
                        stage[row * EPC + col - pc + (lane & 31)] = acc[i][j][v];
                    }
            }
            __syncthreads();
            for (int e = tid; e < BM * EPC / 8; e += 256) {
                const int row = e / (EPC / 8), cg = (e - row * (EPC / 8)) * 8;
                const int pos = xpos(row), c = c0 + pc + cg;
                if (pos >= 0 && c < a.gcpg) {
                    const f32x4 lo = *reinterpret_cast<const f32x4*>(stage + row * EPC + cg);
                    const f32x4 hi = *reinterpret_cast<const f32x4*>(stage + row * EPC + cg + 4);
                    const float v8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    store8(a.dx, a.out_mode, (int64_t)pos * a.Ctot + gb * a.gcpg + c, v8);
                }
            }
            __syncthreads();
        }
    } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int c = c0 + wn0 + j * 32 + (lane & 31);
            if (c >= a.gcpg) continue;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int pos = xpos(wm0 + i * 32 + 8 * (v / 4) + 4 * (lane / 32) + (v % 4));
                    if (pos >= 0) store_out(a.dx, a.out_mode, (int64_t)pos * a.Ctot + gb * a.gcpg + c, acc[i][j][v]);
                }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool PH, bool F16>
int launch_v(const Plan& plan, const DgradArgs& a, hipStream_t s) {
    // 32-channel chunks: 64 measured slower on every shape here (half the
    // workgroups per CU for the doubled LDS stages)
    constexpr int BK = 32;
    if (plan.dg_bk != BK) return (int)hipErrorInvalidValue;
    dim3 grid(a.total_wg), block(256);
    switch (plan.dg_v) {
        case 8: hipLaunchKernelGGL((dgrad_kernel<BM, BN, BK, WM, WN, 8, PH, F16>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((dgrad_kernel<BM, BN, BK, WM, WN, 4, PH, F16>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((dgrad_kernel<BM, BN, BK, WM, WN, 2, PH, F16>), grid, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL((dgrad_kernel<BM, BN, BK, WM, WN, 1, PH, F16>), grid, block, 0, s, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool F16>
int launch_p(const Plan& plan, const DgradArgs& a, hipStream_t s) {
    return a.phases > 1 ? launch_v<BM, BN, WM, WN, true, F16>(plan, a, s) : launch_v<BM, BN, WM, WN, false, F16>(plan, a, s);
}

template <bool F16>
int launch_t(const Plan& plan, const DgradArgs& a, hipStream_t s) {
    switch (plan.dg_bn) {
        case 32: return launch_p<128, 32, 4, 1, F16>(plan, a, s);
        case 64: return launch_p<128, 64, 2, 2, F16>(plan, a, s);
        case 128: return launch_p<128, 128, 2, 2, F16>(plan, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Depthwise backward data (C/G = K/G = 1): no contraction over channels, so
// no MFMA. dX[n,d,h,w,c] = sum over taps of dY at the output position the tap
// maps back to, times W[c][tap]: a stencil per channel. A lane owns 8
// channels (one 16-byte dY load per tap and position) of a strip of
// kDgDwStrip input positions along w; lanes of a wave run along the channels
// first, so each dY load instruction of a wave reads whole contiguous pixels.
// The workgroup's weights sit in LDS as fp32 [tap][channel], read back as two
// 16-byte reads per tap. Accumulation in fp32 in tap order (z, y, x).
template <bool F16>
__global__ __launch_bounds__(256) void dgrad_dw_kernel(const DgradDwArgs a) {
    extern __shared__ __attribute__((aligned(16))) float wlds[];   // [taps][cb]
    const int tid = threadIdx.x;
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    const int sg = L % a.sgroups, cbk = L / a.sgroups;
    const int c_base = cbk * a.cb;
    // stage the block's weights, transposed to [tap][channel]
    for (int e = tid; e < a.cb * a.taps; e += 256) {
        const int cl = e / a.taps, t = e - cl * a.taps;
        const uint16_t u = a.w[(int64_t)(c_base + cl) * a.taps + t];
        wlds[t * a.cb + cl] = F16 ? (float)__builtin_bit_cast(_Float16, u) : __uint_as_float((uint32_t)u << 16);
    }
    __syncthreads();
    const int cvl = tid % a.cbv, sl = tid / a.cbv;
    const int s = sg * a.spw + sl;
    if (sl >= a.spw || s >= a.strips) return;   // no barrier follows
    int r = s / a.nstrip;
    const int w0 = (s - r * a.nstrip) * kDgDwStrip;
    const int h = r % a.Hi;
    r /= a.Hi;
    const int d = r % a.Di;
    const int n = r / a.Di;
    const int c = c_base + cvl * 8;
    auto out_coord = [](int i, int pad, int tdil, int len, MagicU32 ms, int stride) {
        const int num = i + pad - tdil;
        if (num < 0) return -1;
        const int q = (int)magic_div((uint32_t)num, ms);
        if (q * stride != num || q >= len) return -1;
        return q;
    };
    float acc[kDgDwStrip][8];
#pragma unroll
    for (int j = 0; j < kDgDwStrip; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
    for (int z = 0; z < a.Zf; ++z) {
        const int od = out_coord(d, a.pd, z * a.dd, a.Do, a.msd, a.sd);
        if (od < 0) continue;
        for (int y = 0; y < a.Yf; ++y) {
            const int oh = out_coord(h, a.ph, y * a.dh, a.Ho, a.msh, a.sh);
            if (oh < 0) continue;
            const int row = (n * a.Do + od) * a.Ho + oh;
            const int tbase = (z * a.Yf + y) * a.Xf;
            for (int x = 0; x < a.Xf; ++x) {
                const float* wp = wlds + (tbase + x) * a.cb + cvl * 8;
                const f32x4 wa = *reinterpret_cast<const f32x4*>(wp);
                const f32x4 wb = *reinterpret_cast<const f32x4*>(wp + 4);
                const float wv[8] = {wa[0], wa[1], wa[2], wa[3], wb[0], wb[1], wb[2], wb[3]};
#pragma unroll
                for (int j = 0; j < kDgDwStrip; ++j) {
                    const int ow = w0 + j < a.Wi ? out_coord(w0 + j, a.pw, x * a.dw, a.Wo, a.msw, a.sw) : -1;
                    if (ow < 0) continue;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(a.dy + (int64_t)(row * a.Wo + ow) * a.C + c);
                    float f[8];
                    widen8(v, f, F16);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[j][i] = __builtin_fmaf(f[i], wv[i], acc[j][i]);
                }
            }
        }
    }
    const int64_t pix = (((int64_t)n * a.Di + d) * a.Hi + h) * a.Wi;
#pragma unroll
    for (int j = 0; j < kDgDwStrip; ++j)
        if (w0 + j < a.Wi) store8(a.dx, a.out_mode, (pix + w0 + j) * a.C + c, acc[j]);
}

// Row-walking form (3x3 filter, unit stride and dilation). A lane group
// (the lanes of one channel block, kDgRingCh channels per lane) owns one
// 4-wide strip of one row chunk and walks its rows downward: input row h
// needs dY rows h + ph - y, y = 0..2, each over the 6 columns
// w0 + pw - 2 .. w0 + pw + 3, so every step loads one new dY row segment (two
// steps ahead) into a 5-slot register ring and computes 4 positions x 9 taps
// from registers. The block's weights sit in LDS as fp32 [tap][channel].
// Chunks are numbered strip-fastest with aligned row ranges, so neighbouring
// strips read their shared columns at the same time (one HBM fetch, one L2
// hit); odd chunks walk upward, so neighbouring chunks meet at their shared
// halo rows at the same time too.
__device__ __forceinline__ void widen4(const u32x2& v, float* f, bool f16) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t u = v[i];
        if (f16) {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
        } else {
            f[2 * i] = __uint_as_float(u << 16);
            f[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ void store4v(void* out, int mode, int64_t e, const float* v) {
    if (mode == OUT_FP32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + e) = f32x4{v[0], v[1], v[2], v[3]};
        return;
    }
    u32x2 p;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t lo, hi;
        if (mode == OUT_FP16) {
            lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
            hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
            p[i] = lo | (hi << 16);
        } else {
            p[i] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2 * i], (__bf16)v[2 * i + 1]});   // one v_cvt_pk_bf16_f32
        }
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + e) = p;
}

template <bool F16>
__global__ __launch_bounds__(256) void dgrad_dw_ring_kernel(const DgradDwArgs a) {
    constexpr int S = kDgDwStrip, XF = 3, COLS = S + XF - 1, SLOTS = 5, CH = kDgRingCh;
    __shared__ __attribute__((aligned(16))) float wlds[9 * kDgRingMaxCb];   // [tap][channel of the block]
    const int tid = threadIdx.x;
    const int L = xcd_logical_id(blockIdx.x, a.total_wg);
    const int sg = L % a.sgroups, cbk = L / a.sgroups;
    // the block's weights, transposed to [tap][channel]
    for (int e = tid; e < a.cb * 9; e += 256) {
        const int cl = e / 9, t = e - cl * 9;
        const uint16_t u = a.w[(int64_t)(cbk * a.cb + cl) * 9 + t];
        wlds[t * a.cb + cl] = F16 ? (float)__builtin_bit_cast(_Float16, u) : __uint_as_float((uint32_t)u << 16);
    }
    __syncthreads();
    const int cvl = tid % a.cbv, sl = tid / a.cbv;
    const int it = sg * a.spw + sl;
    if (it >= a.items) return;   // no barrier follows
    const int strip = it % a.nstrip;
    int r = it / a.nstrip;
    const int chunk = r % a.nch;
    const int n = r / a.nch;
    const int r0 = (int)((int64_t)chunk * a.Hi / a.nch), r1 = (int)((int64_t)(chunk + 1) * a.Hi / a.nch);
    const int w0 = strip * S;
    const int c = cbk * a.cb + cvl * CH;
    const float* wl = wlds + cvl * CH;

    const __amdgpu_buffer_rsrc_t dy_rs = buf_rsrc(a.dy, a.dy_bytes);
    // column validity and byte offsets within a row, fixed for the lane
    bool col_ok[COLS];
#pragma unroll
    for (int jj = 0; jj < COLS; ++jj) col_ok[jj] = (unsigned)(w0 + a.pw - (XF - 1) + jj) < (unsigned)a.Wo;
    const uint32_t col0 = (uint32_t)(((w0 + a.pw - (XF - 1)) * a.C + c) * 2), colstep = (uint32_t)(a.C * 2);
    const uint32_t rowbytes = (uint32_t)(a.Wo * a.C * 2);
    // dY row `oh` (zeros outside), columns w0 + pw - 2 + jj
    auto load_row = [&](int oh, u32x2* dst) {
        const bool rok = (unsigned)oh < (unsigned)a.Ho;
        const uint32_t base = (uint32_t)(n * a.Ho + oh) * rowbytes + col0;
#pragma unroll
        for (int jj = 0; jj < COLS; ++jj) dst[jj] = buf_load8(dy_rs, rok && col_ok[jj] ? base + jj * colstep : kBufOob);
    };
    // The walk runs down the chunk's input rows (even chunks) or up (odd
    // chunks), so the two chunks on either side of a chunk boundary read the
    // halo dY rows they share at the same moment (both at their start, or
    // both at their end) and the second reader finds them in L2. dY rows are
    // numbered along the walk: row(k) = r0 + ph - 2 + k going down,
    // r1 - 1 + ph - k going up. Step i computes input row r0 + i (down) or
    // r1 - 1 - i (up) from rows k = i, i + 1, i + 2: filter row y takes
    // k = i + 2 - y going down, k = i + y going up. Row k lives in register
    // slot (k + 3) % 5; four rows are loaded before the first step and one
    // per step, two steps ahead.
    const int nsteps = r1 - r0;
    const int64_t pix0 = ((int64_t)n * a.Hi) * a.Wi;
    auto walk = [&](auto up_tag) {
        constexpr bool UP = decltype(up_tag)::value;
        auto row_k = [&](int k) { return UP ? r1 - 1 + a.ph - k : r0 + a.ph - 2 + k; };
        u32x2 ring[SLOTS][COLS];
#pragma unroll
        for (int k = 0; k < 4; ++k) load_row(row_k(k), ring[(k + 3) % SLOTS]);
        auto step = [&](int i, auto rot) {
            constexpr int R = decltype(rot)::value;   // i % 5
            // the prefetch is issued on every step, past the chunk's end too
            // (rows outside dY read as zeros), so no branch sits between a
            // load and its use and the waits stay exact
            load_row(row_k(i + 4), ring[(R + 2) % SLOTS]);
            if (i >= nsteps) return;
            float acc[S][CH];
#pragma unroll
            for (int j = 0; j < S; ++j)
#pragma unroll
                for (int k = 0; k < CH; ++k) acc[j][k] = 0.f;
#pragma unroll
            for (int y = 0; y < 3; ++y) {
                const u32x2* row = ring[UP ? (R + y + 3) % SLOTS : (R - y + SLOTS) % SLOTS];
                float f[COLS][CH];
#pragma unroll
                for (int jj = 0; jj < COLS; ++jj) widen4(row[jj], f[jj], F16);
#pragma unroll
                for (int x = 0; x < XF; ++x) {
                    const f32x4 wv = *reinterpret_cast<const f32x4*>(wl + (y * 3 + x) * a.cb);
#pragma unroll
                    for (int j = 0; j < S; ++j)
#pragma unroll
                        for (int k = 0; k < CH; ++k) acc[j][k] = __builtin_fmaf(f[j + XF - 1 - x][k], wv[k], acc[j][k]);
                }
            }
            const int64_t pix = pix0 + (int64_t)(UP ? r1 - 1 - i : r0 + i) * a.Wi;
#pragma unroll
            for (int j = 0; j < S; ++j)
                if (w0 + j < a.Wi) store4v(a.dx, a.out_mode, (pix + w0 + j) * a.C + c, acc[j]);
        };
        for (int i = 0; i < nsteps; i += SLOTS) {
            step(i, std::integral_constant<int, 0>{});
            step(i + 1, std::integral_constant<int, 1>{});
            step(i + 2, std::integral_constant<int, 2>{});
            step(i + 3, std::integral_constant<int, 3>{});
            step(i + 4, std::integral_constant<int, 4>{});
        }
    };
    if (chunk & 1)
        walk(std::true_type{});
    else
        walk(std::false_type{});
}

}  // namespace

int launch_dgrad_dw(const Plan& plan, const DgradDwArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.form == 2) {
        if (plan.in_f16)
            hipLaunchKernelGGL(dgrad_dw_ring_kernel<true>, dim3(a.total_wg), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(dgrad_dw_ring_kernel<false>, dim3(a.total_wg), dim3(256), 0, s, a);
        return (int)hipGetLastError();
    }
    const size_t lds = (size_t)a.taps * a.cb * 4;
    if (plan.in_f16)
        hipLaunchKernelGGL(dgrad_dw_kernel<true>, dim3(a.total_wg), dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL(dgrad_dw_kernel<false>, dim3(a.total_wg), dim3(256), lds, s, a);
    return (int)hipGetLastError();
}

int launch_dgrad(const Plan& plan, const DgradArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return plan.in_f16 ? launch_t<true>(plan, a, s) : launch_t<false>(plan, a, s);
}

}  // namespace wgrad
