// Internal types shared by the host planner (plan.cpp), the C ABI (abi.cpp)
// and the HIP kernels (kernels.hip). Not part of the public interface.
#pragma once

#include <cstdint>
#include <string>

#include "../../include/wgrad.h"
#include "dgrad_internal.hpp"
#include "magic.hpp"

namespace wgrad {

enum OutMode : int32_t { OUT_BF16 = 0, OUT_FP16 = 1, OUT_FP32 = 2, OUT_WORKSPACE = 3 };

// Kernel arguments of the MFMA implicit-GEMM kernel. Every element offset
// fits in 31 bits (checked by the planner).
struct MfmaArgs {
    const uint16_t* x;
    const uint16_t* dy;
    void* out;              // dW (out_mode < 3) or the fp32 workspace
    int32_t Ktot, Ctot;     // channels per pixel of dY and X
    int32_t kpg, cpg, Gm;   // per-group K, C and merge degree
    int32_t gkpg, gcpg;     // Gm*kpg (merged M), Gm*cpg (merged channel run)
    int32_t Hi, Wi, Ho, Wo; // 1D: Hi = Ho = 1
    int32_t Xf, Yf;         // filter width and height
    int32_t Di, Do;         // input and output depth (2D, 1D: 1)
    int32_t sd, dd, pd;     // depth stride, dilation, left pad
    int32_t sh, sw, dh, dw, ph, pw;
    int32_t R;              // N*Ho*Wo
    int32_t Mm, Nm;         // merged GEMM sizes: Gm*kpg, Z*Y*X*Gm*cpg
    int32_t row_len;        // Z*Y*X*cpg: length of one dW row
    int32_t tiles_m, tiles_n, gblocks, S;
    int32_t kslice;         // reduction elements per split, a multiple of the tile K
    int32_t total_wg;
    int32_t out_mode;
    int32_t slice_elems;    // K*Z*Y*X*cpg: elements of one workspace slice
    MagicU32 mWo, mHo, mDo;
};

// Row-slab kernel instances, shared by the planner and the kernels. Each
// fixes the tile (M block mb, C block cb, filter width xf) and the slab
// geometry at compile time: nks 16-position MFMA steps per slab and an X tile
// of nxr rows x xwp pixels, for one w-stride. Fixed shapes keep the slab loop
// free of runtime guards, so accumulators never need merging copies.
// LDS: each slab stream owns nb slab buffers of 16*nks*mb + nxr*xwp*cb
// elements, filled by 1 KB direct-to-LDS loads (8 rows of 64 channels or 16
// rows of 32); slabs are loaded nb - 1 ahead of the one computed.
constexpr int kRsLdsMax = 160 * 1024;
// gs: the slabs are dealt to the splits in turn, in groups of gs consecutive
// slabs (1, or 4 = one per slab stream)
struct RsInstance {
    int mb, cb, xf, nks, nxr, xwp, stride, nb, gs;
};
constexpr RsInstance kRsInstances[] = {
    {64, 64, 3, 2, 1, 40, 1, 4, 1},    // 32-position row segments
    {64, 64, 3, 2, 1, 64, 2, 3, 1},    // one row up to 31 wide, stride 2
    {32, 32, 3, 4, 2, 32, 1, 4, 1},    // two rows up to 30 wide
    {32, 32, 3, 4, 1, 80, 1, 4, 1},    // one row (or segment) up to 64 wide
    {32, 32, 5, 4, 1, 80, 1, 4, 1},    // width-5 filter: 64-position segments, 4 buffers (faster than
                                       // 128-position ones with 2: more slabs in flight per CU)
    {64, 64, 1, 2, 1, 32, 1, 4, 1},    // pointwise (width-1 filter): 32-position row segments
    {64, 64, 1, 2, 1, 64, 2, 3, 1},    // pointwise, stride 2: 32-position segments
    {32, 32, 1, 4, 1, 64, 1, 4, 1},    // pointwise, 32-channel blocks
    {64, 64, 3, 2, 1, 40, 1, 4, 4},    // as the first, slabs dealt four at a time (3D filters)
};
constexpr int kNumRsInstances = sizeof(kRsInstances) / sizeof(kRsInstances[0]);
// MFMA waves per slab stream: two for 64-channel blocks (each holds 32
// channels); every stream also has one load-issuing producer wave
constexpr int rs_waves_per_slab(const RsInstance& r) { return r.cb == 64 ? 2 : 1; }
inline int rs_buffer_elems(const RsInstance& r) { return 16 * r.nks * r.mb + r.nxr * r.xwp * r.cb; }
inline int rs_lds_bytes(const RsInstance& r) {
    const int slabs = 4 * r.nb * rs_buffer_elems(r) * 2;         // 4 streams, 16-bit elements
    const int reduce = 4 * r.mb * (r.cb + 4) * 4;                // fp32 stream tiles of the epilogue
    return slabs > reduce ? slabs : reduce;
}

// Row-slab MFMA kernel: a workgroup owns one filter row y of one
// (group block, M block, C block) tile and all X taps of that row; the
// reduction runs over slabs of PR output rows x SW output columns.
struct RowSlabArgs {
    const uint16_t* x;
    const uint16_t* dy;
    void* out;
    int32_t Ktot, Ctot, kpg, cpg, gkpg, gcpg;
    int32_t Hi, Wi, Ho, Wo;
    int32_t Y, Yf;          // filter rows (z, y) = Z*Y, and the filter height Y
    int32_t Di, Do, sd, dd, pd;   // depth (2D, 1D: Di = Do = 1, pd = 0)
    int32_t sh, sw, dh, dw, ph, pw;
    int32_t NHo;            // N*Do*Ho output rows
    int32_t Mm;             // merged M = Gm*kpg
    int32_t row_len;        // Z*Y*X*cpg
    int32_t mblocks, cblocks, tiles;
    int32_t PR, SW;         // slab rows and columns (PR*SW <= the instance's positions)
    int32_t XW;             // X tile columns: (SW-1)*sw + (X-1)*dw + 1
    int32_t nseg, nslabs;   // column segments per row block, slabs in total
    int32_t spw;            // slabs per split the split count was sized for (split z takes slabs z + m*S)
    int32_t S, total_wg, out_mode, slice_elems;
    uint32_t x_bytes, dy_bytes;   // buffer sizes for the bounds-checked loads
    MagicU32 mSW, mXW, mHo, mDo, mSeg;   // mSeg: division by nseg
};

// Filter-row ring kernel (2D, 3x3 filter, dilation 1, h-stride 1 or 2): a
// workgroup owns one (group block, M block, 32-channel C block) tile and all
// three filter rows, one MFMA wave per filter row; it walks consecutive
// output rows of its split, staging each dY row once and each input row once
// into an LDS ring that the three waves read at their own row offset.
// Instances fix the M block, the positions per row (16*nks >= Wo), the X row
// width in pixels and the w-stride; nb dY buffers, loaded nb - 1 rows ahead.
struct RingInstance {
    int mb, nks, xwp, stride, nb, rps;
};
constexpr RingInstance kRingInstances[] = {
    {32, 2, 32, 1, 3, 4},    // rows up to 30 wide
    {64, 2, 32, 1, 3, 4},
    {32, 4, 64, 1, 4, 1},    // rows up to 62 wide
    {64, 4, 64, 1, 4, 1},
    {32, 2, 64, 2, 4, 1},    // w-stride 2, rows up to 31 wide
    {64, 2, 64, 2, 4, 1},
};
constexpr int kNumRingInstances = sizeof(kRingInstances) / sizeof(kRingInstances[0]);
constexpr int kRingCB = 32;                       // channels per C block
constexpr int ring_slots(const RingInstance& r) { return 3 * r.nb * r.rps; }
// the epilogue's fp32 tile: mb rows of 9 taps x 32 channels, pitch padded
// by 4 floats so that 16 consecutive rows start on distinct bank quads
constexpr int kRingTilePitch = 9 * kRingCB + 4;
inline int ring_lds_bytes(const RingInstance& r) {
    const int stage = 2 * (r.nb * r.rps * 16 * r.nks * r.mb + ring_slots(r) * r.xwp * kRingCB);
    const int tile = 4 * r.mb * kRingTilePitch;
    return stage > tile ? stage : tile;
}

struct RingArgs {
    const uint16_t* x;
    const uint16_t* dy;
    void* out;
    int32_t Ktot, Ctot, kpg, cpg, gkpg, gcpg;
    int32_t Hi, Wi, Ho, Wo;
    int32_t sh, ph, pw;      // h-stride and left pads (dilations 1, 3x3 filter)
    int32_t NHo;             // N*Ho output rows
    int32_t Mm;              // merged M = Gm*kpg
    int32_t row_len;         // 9*cpg: length of one dW row
    int32_t mblocks, cblocks, tiles;
    int32_t XW;              // input columns one output row reads: (Wo-1)*sw + 3
    int32_t rpw;             // output rows per workgroup (one split)
    int32_t S, total_wg, out_mode, slice_elems;
    uint32_t x_bytes, dy_bytes;
    MagicU32 mHo, mCpg;
};

// Depthwise (C/G = K/G = 1) channel-vector kernel.
struct DwArgs {
    const uint16_t* x;
    const uint16_t* dy;
    void* out;
    int32_t C;                   // = G = K
    int32_t Hi, Wi, Ho, Wo;
    int32_t Y, Xf, sh, sw, dh, dw, ph, pw;
    int32_t R;                   // N*Ho*Wo
    int32_t cl;                  // channel lanes per workgroup (each lane: 8 channels)
    int32_t cblocks;             // C / (8*cl)
    int32_t S, kslice;           // reduction splits and elements per split
    int32_t total_wg;
    int32_t out_mode;
    int32_t slice_elems;         // C*Y*X
    MagicU32 mWo, mHo;
};

// Depthwise windowed kernel (C/G = K/G = 1, filter width 3, w-stride and
// w-dilation 1): one lane owns 8 channels of one 4-wide output segment
// ("unit") at a time and keeps the 6-column X window of each filter row.
struct Dw2Args {
    const uint16_t* x;
    const uint16_t* dy;
    void* out;
    int32_t C, Hi, Wi, Ho, Wo, Y, sh, dh, ph, pw;
    int32_t NHo;           // N*Ho output rows
    int32_t nseg;          // 4-wide segments per output row
    int32_t units;         // NHo*nseg
    int32_t cl;            // channel lanes per workgroup (8 channels each)
    int32_t cblocks;       // C / (8*cl)
    int32_t upt;           // units per thread
    int32_t upw;           // units per workgroup = upt * (256/cl)
    int32_t S, total_wg, out_mode, slice_elems;
    uint32_t x_bytes, dy_bytes;
    MagicU32 mHo, mSeg;
};

// Depthwise strip kernel (3x3 filter, stride and dilation 1 on both axes):
// work items are row chunks of 4-wide column strips; a worker walks a chunk
// keeping the filter's input rows in registers, so each output row loads one
// new input row and one dY row.
// strip kernel shape: 32-bit words (channel pairs) each lane loads per pixel,
// waves per workgroup, and the most lanes that share one pixel's channels
// (fewer lanes per pixel let one wave cover several strips)
// (measured on the 512-channel 56x56 depthwise shape: 8-byte lanes with two
// waves per SIMD beat 16-byte lanes with one, and three waves per SIMD with a
// shallower prefetch)
constexpr int kDw3Words = 2, kDw3Waves = 8, kDw3MaxLanes = 64;
constexpr int kDw3Channels = 2 * kDw3Words;   // channels per lane

struct Dw3Args {
    const uint16_t* x;
    const uint16_t* dy;
    void* out;
    int32_t C, Hi, Wi, Ho, Wo, ph, pw;
    int32_t nseg;          // 4-wide strips per image row
    int32_t nch;           // row chunks per strip
    int32_t items;         // N * nseg * nch items per channel block (strip-major)
    int32_t cl, cblocks;   // lanes per pixel (kDw3Channels channels each) and channel blocks
    int32_t S, total_wg, out_mode, slice_elems;   // S: workgroups (slices) per channel block
    uint32_t x_bytes, dy_bytes;
};

// Depthwise tile kernel (3x3 filter, stride and dilation 1 on both axes):
// a workgroup takes output tiles of th rows x dwt_tile_w(cb) columns x cb
// channels; one wave streams the tile's input rows into an LDS ring with
// direct-to-LDS loads and seven waves compute, each on two adjacent output
// columns, with dY loaded into registers.
constexpr int kDwtCompute = 7;   // compute waves (one more wave loads)
constexpr int kDwtRing = 6;      // input rows in the LDS ring
// output columns per tile: each compute wave takes two columns of each of the
// 64 / (cb / 8) pixels one wave-load covers
constexpr int dwt_tile_w(int cb) { return 2 * kDwtCompute * (512 / cb); }
// bytes of one ring row: tile_w + 2 pixels, rounded up to whole 1 KB loads
constexpr int dwt_row_bytes(int cb) {
    return (dwt_tile_w(cb) + 2 + 1024 / (cb * 2) - 1) / (1024 / (cb * 2)) * (1024 / (cb * 2)) * cb * 2;
}
// the ring, or in the epilogue one cb-channel x 9-tap fp32 block per compute wave
constexpr int dwt_lds_bytes(int cb) {
    return kDwtRing * dwt_row_bytes(cb) > kDwtCompute * cb * 9 * 4 ? kDwtRing * dwt_row_bytes(cb)
                                                                  : kDwtCompute * cb * 9 * 4;
}
struct DwTileArgs {
    const uint16_t* x;
    const uint16_t* dy;
    void* out;
    int32_t C, Hi, Wi, Ho, Wo, ph, pw;
    int32_t th;                    // output rows per tile
    int32_t tiles_x, tiles_y;      // tiles per image row / column
    int32_t tiles;                 // N * tiles_y * tiles_x
    int32_t cblocks;               // C / cb
    int32_t S, total_wg, out_mode, slice_elems;   // S: workgroups per channel block
    uint32_t x_bytes, dy_bytes;
};

struct ReduceArgs {
    const float* ws;
    void* dw;
    int32_t elems;    // elements per slice
    int32_t S;
    int32_t out_mode; // OUT_BF16 / OUT_FP16 / OUT_FP32
    int32_t zl;       // slice lanes per workgroup (power of two, <= 64)
    int32_t vec4;     // 1: elements handled 4 at a time (elems % 4 == 0)
};

// MFMA tile table (id -> shape). Ids are stable: tests and overrides use them.
struct TileShape {
    int id, bm, bn, bk, wm, wn, atom;
};
constexpr TileShape kTiles[] = {
    {1, 64, 64, 32, 2, 2, 32},
    {2, 64, 128, 32, 2, 2, 32},
    {3, 128, 128, 32, 2, 2, 32},
    {4, 32, 128, 32, 1, 4, 32},
    {5, 16, 128, 32, 1, 4, 16},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
const TileShape* find_tile(int id);

struct DeviceModel {
    int num_cus;
    int num_xcds;
};

enum PlanOp : int { OP_WGRAD = 0, OP_DGRAD = 1 };

struct Plan {
    int op;              // PlanOp
    wgrad_problem prob;
    wgrad_plan_info info;
    int variant;
    int in_f16;          // 1 if inputs are fp16
    MfmaArgs mfma;       // pointers filled at run time
    DwArgs dwk;
    Dw2Args dw2;
    int dw2_ty;                  // filter height of the windowed depthwise instance (0 = not used)
    Dw3Args dw3;
    int dw3_ty;                  // filter height of the strip depthwise instance (0 = not used)
    DwTileArgs dwt;
    int dwt_cb;                  // channels per workgroup of the tile depthwise kernel (0 = not used)
    RowSlabArgs rs;
    int rs_inst;                 // index into kRsInstances
    RingArgs ring;
    int ring_inst;               // index into kRingInstances, or -1 (row-slab variant: per-filter-row form)
    int lds_bytes;               // dynamic LDS of the main kernel
    ReduceArgs red;
    int dw_tile_y, dw_tile_x;   // depthwise kernel filter instance
    DgradArgs dg;
    int dg_bn, dg_v, dg_bk;      // dgrad tile width, load vector width, channels per reduction chunk
    DgradDwArgs dgdw;
    int dg_dw;                   // 1: the depthwise dgrad kernel
    DgradDwTileArgs dgdwt;
    int dg_dwt;                  // channels per workgroup of the depthwise dgrad tile kernel (0 = not used)
    DgradRingArgs dgr;
    int dg_ring;                 // index into kDgRingInstances, or -1
    std::string name;
};

// Host planning (no HIP calls). Returns a wgrad_status and sets *msg on error.
int build_plan(const wgrad_problem& p, const wgrad_overrides* ov, const DeviceModel& dev,
               Plan& out, std::string* msg);
int build_dgrad_plan(const wgrad_problem& p, const wgrad_overrides* ov, const DeviceModel& dev,
                     Plan& out, std::string* msg);

// Kernel launchers (kernels.hip). Return a hipError_t value (0 = success).
int launch_mfma(const Plan& plan, const MfmaArgs& a, void* stream);
int launch_depthwise(const Plan& plan, const DwArgs& a, void* stream);
int launch_rowslab(const Plan& plan, const RowSlabArgs& a, void* stream);
int launch_ring(const Plan& plan, const RingArgs& a, void* stream);          // ring.hip
int launch_depthwise2(const Plan& plan, const Dw2Args& a, void* stream);
int launch_depthwise3(const Plan& plan, const Dw3Args& a, void* stream);
int launch_dwtile(const Plan& plan, const DwTileArgs& a, void* stream);   // dwtile.hip
int launch_reduce(const ReduceArgs& a, int64_t grid, void* stream);
int launch_dgrad(const Plan& plan, const DgradArgs& a, void* stream);   // dgrad.hip
int launch_dgrad_dw(const Plan& plan, const DgradDwArgs& a, void* stream);
int launch_dgrad_dwtile(const Plan& plan, const DgradDwTileArgs& a, void* stream);   // dwtile.hip
int launch_dgrad_ring(const Plan& plan, const DgradRingArgs& a, void* stream);   // dgrad_ring.hip
// Device address and size of the library's split-K scratch array on the
// stream's GPU (noalloc.hip); resolved once per device. Returns a hipError_t
// value (0 = success).
int scratch_workspace(void* stream, void** ptr, size_t* bytes);
// One wave's transposed-LDS-read fragment, 64 lanes x 8 values, into out
// (probe.hip). Returns a hipError_t value.
int launch_tr_probe(uint16_t* out, void* stream);

}  // namespace wgrad
