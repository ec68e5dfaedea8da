// Kernel-argument blocks of the backward-data (dgrad) kernels (dgrad.hip),
// kept apart from the backward-weight ones. Not part of the public interface.
#pragma once

#include <cstdint>

#include "magic.hpp"

namespace wgrad {

// Backward data: flat MFMA implicit GEMM over input positions, one block of
// Gm adjacent groups per grid slice, reduction over (tap, output channel) in
// chunks of 32 channels of one tap. Merged groups form one block-diagonal
// GEMM: their dY and dX channel runs are contiguous, and weight entries that
// pair different groups are zero.
//
// Stride phases: input positions are split by (di mod sd, hi mod sh,
// wi mod sw). Within a phase, tap z either reaches an output position for
// every input of the phase, at od = i_d + (ph_d + pd - z*dd) / sd with
// di = ph_d + i_d*sd, or for none of them. A workgroup covers positions of
// one phase and walks only that phase's taps: the valid z form the
// progression z0, z0 + zstep, ... with zstep = sd / gcd(sd, dd).
constexpr int kDgMaxStride = 16;   // per-axis stride limit of the phase tables
struct DgradArgs {
    const uint16_t* dy;
    const uint16_t* w;
    void* dx;
    int32_t Ktot, Ctot, kpg, cpg;
    int32_t Gm, gkpg, gcpg;        // merge degree, Gm*kpg, Gm*cpg
    int32_t Di, Hi, Wi, Do, Ho, Wo;
    int32_t Zf, Yf, Xf, taps;      // filter depth, height, width and Z*Y*X
    int32_t sd, sh, sw, dd, dh, dw, pd, ph, pw;
    int32_t zstep, ystep, xstep;   // s / gcd(s, dilation) per axis: taps between valid taps
    int32_t zdo, ydo, xdo;         // dilation / gcd(s, dilation): output step between valid taps
    // per axis (d, h, w) and phase residue r < stride: first valid tap, number
    // of valid taps and the output offset (r + pad - t0*dil) / stride of the first
    int16_t t0[3][kDgMaxStride], nt[3][kDgMaxStride], o0[3][kDgMaxStride];
    int32_t qd, qh, qw;            // phase grid: ceil(Di / sd), ceil(Hi / sh), ceil(Wi / sw)
    int32_t phases;                // sd * sh * sw
    int32_t ph_rot;                // phase groups per CU round (rotation of the phase order, see the kernel)
    int32_t M;                     // N * qd * qh * qw positions per phase
    int32_t kchunks;               // ceil(gkpg / 32)
    uint32_t dy_bytes, w_bytes;    // buffer sizes for the bounds-checked loads
    int32_t tiles_m, tiles_n, total_wg, out_mode;
    MagicU32 mqw, mqh, mqd, mkpg, mcpg;
};
// Depthwise backward data (C/G = K/G = 1, C % 8 == 0): a lane owns 8
// channels of a 4-wide strip of one input row; a workgroup covers a channel
// block of cb channels (weights staged in LDS as fp32 [tap][channel]) and
// 256 / (cb / 8) strips.
constexpr int kDgDwStrip = 4;
// row-walking form: channels per lane and the widest channel block (64 lanes)
constexpr int kDgRingCh = 4, kDgRingMaxCb = 64 * kDgRingCh;
constexpr int kDgDwLdsMax = 64 * 1024;
struct DgradDwArgs {
    const uint16_t* dy;
    const uint16_t* w;
    void* dx;
    int32_t C, Di, Hi, Wi, Do, Ho, Wo;
    int32_t Zf, Yf, Xf, taps;
    int32_t sd, sh, sw, dd, dh, dw, pd, ph, pw;
    int32_t cb, cbv, spw;          // channels per block, channel vectors per block (cb/8), strips per workgroup
    int32_t nstrip, strips;        // strips per input row, N*Di*Hi*nstrip
    int32_t cblocks, sgroups, total_wg, out_mode;
    MagicU32 msd, msh, msw;
    // row-walking form (3x3, unit stride and dilation, 2D/1D): strips are cut
    // into nch chunks of rows; items = N * nch * nstrip per channel block
    int32_t form;                  // 1: per-tap loads, 2: row walk
    int32_t nch, items;
    uint32_t dy_bytes;
};
// Depthwise backward data, tile form (2D, 3x3 filter, unit stride and
// dilation, C a multiple of 256): dX tiles of th rows x dwt_tile_w(cb)
// columns x cb channels (cb = 256); one wave streams the tile's dY
// rows (halo included) into an LDS ring, seven compute waves write dX rows
// from registers.
struct DgradDwTileArgs {
    const uint16_t* dy;
    const uint16_t* w;
    void* dx;
    int32_t C, Hi, Wi, Ho, Wo, ph, pw;
    int32_t th;                    // dX rows per tile
    int32_t tiles_x, tiles_y;      // tiles per dX row / column
    int32_t tiles;                 // N * tiles_y * tiles_x, per channel block
    int32_t cblocks;               // C / cb
    int32_t total_wg, out_mode;    // workgroups (each takes tiles wg, wg + total_wg, ... of all blocks)
    uint32_t dy_bytes;
};
// Row-ring backward data (2D, 3x3 filter, unit stride and dilation): a
// workgroup owns one group block and one block of cbd dX channels, keeps that
// block's weights in LDS for the whole launch, and walks its split of input
// rows four at a time, one row per MFMA wave. Input rows are numbered
// "virtually", Hi + 2 per image (the last two are padding rows that are
// computed but not stored), so that dY row u = v + ph - y of virtual input
// row v is the same for every image and a window of dY rows can be kept in
// an LDS ring across the rows of a step and from one step to the next.
struct DgradRingInstance {
    int cbd, mt, ch;     // dX channels per block, 32-position M tiles per row, 8-channel dY chunks per pixel
};
constexpr DgradRingInstance kDgRingInstances[] = {
    {32, 1, 4}, {32, 2, 4}, {64, 1, 4}, {64, 2, 4},
    {32, 1, 8}, {32, 2, 8}, {64, 1, 8}, {64, 2, 8},
};
constexpr int kNumDgRingInstances = sizeof(kDgRingInstances) / sizeof(kDgRingInstances[0]);
constexpr int kDgRingSlots = 10;         // a step's 6-row dY window plus the next step's 4 rows
constexpr int kDgRingLdsMax = 160 * 1024;
struct DgradRingArgs {
    const uint16_t* dy;
    const uint16_t* w;
    void* dx;
    int32_t Ktot, Ctot, kpg, cpg, Gm, gkpg, gcpg;
    int32_t Hi, Wi, Ho, Wo, ph, pw;
    int32_t N, VR, NV;             // virtual rows per image (Hi + 2) and in all (N * VR)
    int32_t cblocks, tiles;        // dX channel blocks per group block; group blocks * cblocks
    int32_t vpw;                   // virtual rows per workgroup (a multiple of 4)
    int32_t qp, nxl;               // pixels per ring slot (>= Wi + 2) and 1 KB loads per dY row
    int32_t total_wg, out_mode;
    uint32_t dy_bytes, w_bytes;
    MagicU32 mVR, mkpg, mcpg;
};
inline int dg_ring_lds_bytes(const DgradRingInstance& r, int qp) {
    return 2 * (9 * 8 * r.ch * r.cbd + kDgRingSlots * qp * 8 * r.ch);
}

// dgrad tiles: id -> (BM, BN); 4 waves each
struct DgradTile {
    int id, bm, bn;
};
constexpr DgradTile kDgradTiles[] = {{1, 128, 32}, {2, 128, 64}, {3, 128, 128}};

}  // namespace wgrad
