// Host planner: validation, output size, kernel family, tile, split-K degree
// S, group-merge degree Gm and the kernel-argument blocks. Pure C++ (no HIP
// calls), so it runs and is tested on machines without a GPU.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "wgrad_internal.hpp"

namespace wgrad {

const TileShape* find_tile(int id) {
    for (const auto& t : kTiles)
        if (t.id == id) return &t;
    return nullptr;
}

namespace {

constexpr int64_t kMax31 = (int64_t{1} << 31) - 1;

// a*b for non-negative a and b, saturated at INT64_MAX instead of wrapping
inline int64_t smul(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

int fail(std::string* msg, int code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
int fail(std::string* msg, int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (msg) *msg = buf;
    return code;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int64_t gcd64(int64_t a, int64_t b) { while (b) { int64_t t = a % b; a = b; b = t; } return a; }

// Geometry with 1D folded into 2D (h axis of size 1).
// Spatial geometry along (d, h, w); axes a problem does not have are 1 long
// (stride and dilation 1, no pad).
struct Geo {
    int64_t Hi, Wi, Y, X, sh, sw, dh, dw, ph, pw, Ho, Wo;
    int64_t Di, Z, sd, dd, pd, Do;
};

// elements of X and dY (the problem has passed check_problem, so both fit in
// 31 bits and these products in int64)
inline int64_t in_elems(const wgrad_problem& p, const Geo& g) { return p.N * g.Di * g.Hi * g.Wi * p.C; }
inline int64_t dy_elems(const wgrad_problem& p, const Geo& g) { return p.N * g.Do * g.Ho * g.Wo * p.K; }

// Split-K degree in the manner of a groups-aware occupancy target: enough
// workgroups for `target` per CU across the whole grid, clamped to the number
// of K tiles and a workspace budget, and only then snapped so that the grid is
// a multiple of the XCD count (clamping after the snap would undo it).
int64_t choose_split(int64_t base_grid, int64_t k_tiles, int64_t slice_bytes, int64_t input_bytes,
                     const DeviceModel& dev, int64_t target_per_cu) {
    int64_t want = ceil_div(target_per_cu * dev.num_cus, std::max<int64_t>(1, base_grid));
    // the workspace round trip (write + read of S fp32 slices) should not
    // exceed the unavoidable input traffic
    int64_t ws_cap = std::max<int64_t>(1, (input_bytes / 2) / std::max<int64_t>(1, slice_bytes));
    int64_t cap = std::max<int64_t>(1, std::min<int64_t>({k_tiles, ws_cap, 65535}));
    int64_t s = std::max<int64_t>(1, std::min(want, cap));
    if (s > 1) {
        int64_t step = dev.num_xcds / gcd64(base_grid, dev.num_xcds);
        int64_t up = ceil_div(s, step) * step;
        int64_t down = (s / step) * step;
        if (up <= cap) s = up;
        else if (down >= 1) s = down;
    }
    return s;
}


// Row-slab plan: filter width 3 or 5, channel runs of 32 or 64 after merging,
// 16-byte vectors everywhere. Returns false (with a reason) when the shape
// does not fit the kernel.
bool plan_rowslab(const wgrad_problem& p, const Geo& g, const wgrad_overrides& o, const DeviceModel& dev,
                  int out_final, Plan& out, std::string* why) {
    const int64_t cpg = p.C / p.G, kpg = p.K / p.G;
    auto no = [&](const char* m) { if (why) *why = m; return false; };
    if (g.X != 1 && g.X != 3 && g.X != 5) return no("row-slab needs a filter width of 1, 3 or 5");
    if (g.dw != 1) return no("row-slab needs a filter dilation of 1 along w");
    if (2 * in_elems(p, g) >= (int64_t{1} << 31) || 2 * dy_elems(p, g) >= (int64_t{1} << 31))
        return no("row-slab needs X and dY below 2 GiB");
    int64_t Gm = o.group_merge;
    if (!Gm) {
        Gm = 1;
        while (Gm * cpg < 32 && Gm * 2 <= 8 && p.G % (Gm * 2) == 0) Gm *= 2;
    }
    if (!is_pow2(Gm) || p.G % Gm) return no("group_merge must be a power of two dividing G");
    const int64_t gkpg = Gm * kpg, gcpg = Gm * cpg;
    if (cpg % 4 || gkpg % 8 || p.K % 8 || p.C % 8) return no("row-slab needs 16-byte channel vectors");
    // tile: 64 x 64 channel blocks when the merged runs allow it, else 32 x 32
    int mb, cb;
    if ((g.X == 3 || g.X == 1) && gcpg % 64 == 0 && gkpg > 32) { mb = 64; cb = 64; }
    else if (gcpg % 32 == 0) { mb = 32; cb = 32; }
    else return no("row-slab needs a merged channel run that is a multiple of 32");
    const int64_t NHo = p.N * g.Do * g.Ho;       // output rows (n, do, ho)
    auto xw_of = [&](int64_t sw) { return (sw - 1) * g.sw + (g.X - 1) * g.dw + 1; };
    // slab: PR output rows x SW output columns whose positions are one
    // contiguous run of r (whole output rows, or a segment of one row). Pick
    // the instance and slab with the largest useful fraction PR*SW/KS.
    int inst = -1;
    int64_t PR = 0, SW = 0;
    double best = 0.0;
    for (int i = 0; i < kNumRsInstances; ++i) {
        const RsInstance& r = kRsInstances[i];
        if (r.mb != mb || r.cb != cb || r.xf != g.X) continue;
        if (r.gs != 1 && g.Z == 1) continue;             // slab groups: 3D filters only
        if (r.stride != (g.sw == 2 ? 2 : 1)) continue;   // stride 2 splits the tile into even / odd columns
        if (rs_lds_bytes(r) > kRsLdsMax) continue;
        const int64_t ks = 16 * r.nks;
        // input columns the tile holds: xwp (stride 1), xwp/2 of each parity (stride 2)
        auto fits = [&](int64_t sw) {
            const int64_t xw = xw_of(sw);
            return r.stride == 1 ? xw <= r.xwp : (xw + 1) / 2 <= r.xwp / 2;
        };
        int64_t sw = std::min<int64_t>(g.Wo, ks);
        while (sw > 1 && !fits(sw)) --sw;
        if (!fits(sw)) continue;
        int64_t pr = sw == g.Wo ? std::min<int64_t>({ks / sw, (int64_t)r.nxr, std::max<int64_t>(1, NHo)}) : 1;
        // useful fraction of the slab slots over whole rows: a row cut into
        // segments of sw fills ceil(Wo / sw) slabs
        const double eff = double(pr * g.Wo) / double(ceil_div(g.Wo, sw) * ks);
        // equal slabs: 3D filters take the instance that deals slabs in
        // groups (measured faster there, slower on 2D shapes)
        const bool tie = inst >= 0 && eff > best - 1e-9 && eff < best + 1e-9;
        if (eff > best + 1e-9 || (tie && r.gs > kRsInstances[inst].gs)) { best = eff; inst = i; PR = pr; SW = sw; }
    }
    if (inst < 0) return no("row-slab: no kernel instance fits this slab geometry");
    const RsInstance& ri = kRsInstances[inst];
    const int64_t XW = xw_of(SW);
    const int64_t nseg = ceil_div(g.Wo, SW);
    const int64_t nslabs = ceil_div(NHo, PR) * nseg;
    const int64_t mblocks = ceil_div(gkpg, mb), cblocks = gcpg / cb, gblocks = p.G / Gm;
    const int64_t tiles = gblocks * mblocks * cblocks * g.Z * g.Y;   // one filter row (z, y) per tile
    int64_t spw, S;
    if (nslabs == 0) {
        spw = 0; S = 1;
    } else if (o.split_k) {
        spw = ceil_div(nslabs, std::min<int64_t>(o.split_k, nslabs));
        S = ceil_div(nslabs, spw);
    } else {
        // one workgroup per CU (the kernel's LDS allows no more): as many
        // splits as fit beside the tiles, each sized to a multiple of four
        // slabs (the kernel's four slab streams), then as few splits as those
        // slab counts need, which keeps the workspace small. The kernel
        // deals the slabs out interleaved (split z takes z, z + S, ...), so
        // splits differ by at most one slab.
        const int64_t smax = std::max<int64_t>(1, (int64_t)dev.num_cus / tiles);
        spw = 4 * ceil_div(ceil_div(nslabs, smax), 4);
        S = ceil_div(nslabs, spw);
    }
    if (tiles * S > kMax31 || S > 65535) return no("row-slab grid too large");
    const int64_t ndw = p.K * g.Z * g.Y * g.X * cpg;
    if (S > 1 && 4 * ndw >= (int64_t{1} << 31)) return no("row-slab partials need a dW below 2 GiB of fp32");
    RowSlabArgs& a = out.rs;
    a = RowSlabArgs{};
    a.Ktot = (int32_t)p.K; a.Ctot = (int32_t)p.C; a.kpg = (int32_t)kpg; a.cpg = (int32_t)cpg;
    a.gkpg = (int32_t)gkpg; a.gcpg = (int32_t)gcpg;
    a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
    a.Y = (int32_t)(g.Z * g.Y); a.Yf = (int32_t)g.Y;
    a.Di = (int32_t)g.Di; a.Do = (int32_t)g.Do; a.sd = (int32_t)g.sd; a.dd = (int32_t)g.dd; a.pd = (int32_t)g.pd;
    a.sh = (int32_t)g.sh; a.sw = (int32_t)g.sw; a.dh = (int32_t)g.dh; a.dw = (int32_t)g.dw;
    a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
    a.NHo = (int32_t)NHo; a.Mm = (int32_t)gkpg; a.row_len = (int32_t)(g.Z * g.Y * g.X * cpg);
    a.mblocks = (int32_t)mblocks; a.cblocks = (int32_t)cblocks; a.tiles = (int32_t)tiles;
    a.PR = (int32_t)PR; a.SW = (int32_t)SW; a.XW = (int32_t)XW;
    a.nseg = (int32_t)nseg; a.nslabs = (int32_t)nslabs; a.spw = (int32_t)spw;
    a.S = (int32_t)S; a.total_wg = (int32_t)(tiles * S);
    a.out_mode = S == 1 ? out_final : OUT_WORKSPACE;
    a.slice_elems = (int32_t)ndw;
    a.x_bytes = (uint32_t)(2 * p.N * g.Di * g.Hi * g.Wi * p.C);
    a.dy_bytes = (uint32_t)(2 * NHo * g.Wo * p.K);
    a.mSW = make_magic((uint32_t)SW); a.mXW = make_magic((uint32_t)XW); a.mHo = make_magic((uint32_t)g.Ho);
    a.mSeg = make_magic((uint32_t)nseg);
    a.mDo = make_magic((uint32_t)g.Do);
    out.rs_inst = inst;
    out.lds_bytes = rs_lds_bytes(ri);
    wgrad_plan_info& info = out.info;
    info.tile = 0;
    info.tile_m = mb; info.tile_n = (int32_t)(g.X * cb); info.tile_k = 16 * ri.nks;
    info.split_k = (int32_t)S;
    info.group_merge = (int32_t)Gm;
    info.vector_width = 8;
    info.grid_main = a.total_wg;
    info.workspace_bytes = S > 1 ? S * ndw * 4 : 0;
    return true;
}

// Filter-row ring plan: 2D, 3x3 filter, dilation 1, h-stride 1..3, w-stride
// 1 or 2, whole output rows up to 64 positions, merged channel runs that are
// a multiple of 32. Returns false (with a reason) when the shape does not fit.
bool plan_ring(const wgrad_problem& p, const Geo& g, const wgrad_overrides& o, const DeviceModel& dev,
               int out_final, Plan& out, std::string* why) {
    const int64_t cpg = p.C / p.G, kpg = p.K / p.G;
    auto no = [&](const char* m) { if (why) *why = m; return false; };
    if (p.ndim != 2) return no("filter-row ring form needs a 2D problem");
    if (g.Y != 3 || g.X != 3 || g.dh != 1 || g.dw != 1) return no("filter-row ring form needs a 3x3 filter with dilation 1");
    if (g.sh > 3 || g.sw > 2) return no("filter-row ring form needs an h-stride of at most 3 and a w-stride of 1 or 2");
    if (2 * in_elems(p, g) >= (int64_t{1} << 31) || 2 * dy_elems(p, g) >= (int64_t{1} << 31))
        return no("filter-row ring form needs X and dY below 2 GiB");
    int64_t Gm = o.group_merge;
    if (!Gm) {
        Gm = 1;
        while (Gm * cpg < 32 && Gm * 2 <= 8 && p.G % (Gm * 2) == 0) Gm *= 2;
    }
    if (!is_pow2(Gm) || p.G % Gm) return no("group_merge must be a power of two dividing G");
    const int64_t gkpg = Gm * kpg, gcpg = Gm * cpg;
    if (cpg % 4 || gkpg % 8 || p.K % 8 || p.C % 8) return no("filter-row ring form needs 16-byte channel vectors");
    if (gcpg % kRingCB) return no("filter-row ring form needs a merged channel run that is a multiple of 32");
    const int mb = gkpg > 32 ? 64 : 32;
    const int stride = (int)g.sw;
    // the smallest row tile that holds a whole output row and its input columns
    int inst = -1;
    for (int i = 0; i < kNumRingInstances; ++i) {
        const RingInstance& r = kRingInstances[i];
        if (r.mb != mb || r.stride != stride) continue;
        if (16 * r.nks < g.Wo) continue;
        if (stride == 1 ? g.Wo + 2 > r.xwp : g.Wo + 1 > r.xwp / 2) continue;
        if (ring_lds_bytes(r) > kRsLdsMax) continue;
        if (inst < 0 || 16 * r.nks < 16 * kRingInstances[inst].nks) inst = i;
    }
    if (inst < 0) return no("filter-row ring form: no instance holds a whole output row");
    const RingInstance& ri = kRingInstances[inst];
    const int64_t NHo = p.N * g.Ho;
    const int64_t mblocks = ceil_div(gkpg, mb), cblocks = gcpg / kRingCB, gblocks = p.G / Gm;
    const int64_t tiles = gblocks * mblocks * cblocks;
    int64_t S;
    if (NHo == 0) S = 1;
    else if (o.split_k) S = std::min<int64_t>(o.split_k, NHo);
    else S = std::max<int64_t>(1, std::min<int64_t>(NHo, (int64_t)dev.num_cus / std::max<int64_t>(1, tiles)));
    const int64_t rpw = NHo ? ceil_div(NHo, S) : 0;
    if (NHo) S = ceil_div(NHo, rpw);
    if (tiles * S > kMax31 || S > 65535) return no("filter-row ring grid too large");
    const int64_t ndw = p.K * 9 * cpg;
    if (S > 1 && 4 * ndw >= (int64_t{1} << 31)) return no("filter-row ring partials need a dW below 2 GiB of fp32");
    RingArgs& a = out.ring;
    a = RingArgs{};
    a.Ktot = (int32_t)p.K; a.Ctot = (int32_t)p.C; a.kpg = (int32_t)kpg; a.cpg = (int32_t)cpg;
    a.gkpg = (int32_t)gkpg; a.gcpg = (int32_t)gcpg;
    a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
    a.sh = (int32_t)g.sh; a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
    a.NHo = (int32_t)NHo; a.Mm = (int32_t)gkpg; a.row_len = (int32_t)(9 * cpg);
    a.mblocks = (int32_t)mblocks; a.cblocks = (int32_t)cblocks; a.tiles = (int32_t)tiles;
    a.XW = (int32_t)((g.Wo - 1) * g.sw + 3);
    a.rpw = (int32_t)rpw;
    a.S = (int32_t)S; a.total_wg = (int32_t)(tiles * S);
    a.out_mode = S == 1 ? out_final : OUT_WORKSPACE;
    a.slice_elems = (int32_t)ndw;
    a.x_bytes = (uint32_t)(2 * p.N * g.Hi * g.Wi * p.C);
    a.dy_bytes = (uint32_t)(2 * NHo * g.Wo * p.K);
    a.mHo = make_magic((uint32_t)g.Ho); a.mCpg = make_magic((uint32_t)cpg);
    out.ring_inst = inst;
    out.lds_bytes = ring_lds_bytes(ri);
    wgrad_plan_info& info = out.info;
    info.tile = 2;
    info.tile_m = mb; info.tile_n = 9 * kRingCB; info.tile_k = 16 * ri.nks;
    info.split_k = (int32_t)S;
    info.group_merge = (int32_t)Gm;
    info.vector_width = 8;
    info.grid_main = a.total_wg;
    info.workspace_bytes = S > 1 ? S * ndw * 4 : 0;
    return true;
}

// Auto choice between the two row-slab forms: the ring form stages each
// row once per workgroup instead of once per filter row, but its workgroup
// partial spans all nine taps, so it pays off where the stored partial is
// small (merged groups store only their diagonal blocks).
bool ring_preferred(const wgrad_problem& p, const Geo& g) {
    (void)g;
    const int64_t cpg = p.C / p.G;
    return cpg < 32 && p.G > 1;
}

// Validation and spatial geometry shared by both directions.
int check_problem(const wgrad_problem& p, Geo& g, std::string* msg) {
    const int E = WGRAD_ERR_INVALID_ARG;
    if (p.ndim < 1 || p.ndim > 3) return fail(msg, E, "ndim must be 1, 2 or 3 (got %d)", p.ndim);
    if (p.reserved != 0) return fail(msg, E, "reserved field must be 0");
    if (p.in_dtype != WGRAD_BF16 && p.in_dtype != WGRAD_FP16)
        return fail(msg, E, "in_dtype must be BF16 or FP16");
    if (p.out_dtype != p.in_dtype && p.out_dtype != WGRAD_FP32)
        return fail(msg, E, "out_dtype must equal in_dtype or be FP32");
    if (p.G < 1 || p.C < 1 || p.K < 1 || p.N < 0)
        return fail(msg, E, "need G, C, K >= 1 and N >= 0");
    if (p.C % p.G || p.K % p.G)
        return fail(msg, E, "C (%lld) and K (%lld) must be multiples of G (%lld)", (long long)p.C,
                    (long long)p.K, (long long)p.G);
    // every field is bounded before any product of fields is formed, and the
    // products below saturate, so no int64 arithmetic here can wrap
    if (p.G > kMax31 || p.C > kMax31 || p.K > kMax31 || p.N > kMax31)
        return fail(msg, E, "G, N, C and K must fit in 31 bits");
    for (int i = 0; i < p.ndim; ++i) {
        if (p.in_len[i] < 1 || p.filt_len[i] < 1 || p.stride[i] < 1 || p.dilation[i] < 1)
            return fail(msg, E, "lengths, strides and dilations must be >= 1 (axis %d)", i);
        if (p.pad_lo[i] < 0 || p.pad_hi[i] < 0) return fail(msg, E, "pads must be >= 0 (axis %d)", i);
        if (p.in_len[i] > kMax31 || p.filt_len[i] > kMax31 || p.stride[i] > kMax31 || p.dilation[i] > kMax31 ||
            p.pad_lo[i] > kMax31 || p.pad_hi[i] > kMax31)
            return fail(msg, E, "lengths, strides, dilations and pads must fit in 31 bits (axis %d)", i);
    }
    // axes outermost first; the problem's ndim axes are the last ones of (d, h, w)
    int64_t len[3], fl[3], st[3], dl[3], pl[3], ol[3];
    const int lead = 3 - p.ndim;
    for (int ax = 0; ax < 3; ++ax) {
        if (ax < lead) {
            len[ax] = fl[ax] = st[ax] = dl[ax] = 1;
            pl[ax] = 0;
            ol[ax] = 1;
            continue;
        }
        const int i = ax - lead;
        len[ax] = p.in_len[i]; fl[ax] = p.filt_len[i]; st[ax] = p.stride[i];
        dl[ax] = p.dilation[i]; pl[ax] = p.pad_lo[i];
        const int64_t span = p.in_len[i] + p.pad_lo[i] + p.pad_hi[i] - p.dilation[i] * (p.filt_len[i] - 1) - 1;
        if (span < 0) return fail(msg, E, "empty output: the dilated filter exceeds the padded input");
        ol[ax] = span / p.stride[i] + 1;
    }
    g = Geo{};
    g.Di = len[0]; g.Hi = len[1]; g.Wi = len[2];
    g.Z = fl[0];   g.Y = fl[1];   g.X = fl[2];
    g.sd = st[0];  g.sh = st[1];  g.sw = st[2];
    g.dd = dl[0];  g.dh = dl[1];  g.dw = dl[2];
    g.pd = pl[0];  g.ph = pl[1];  g.pw = pl[2];
    g.Do = ol[0];  g.Ho = ol[1];  g.Wo = ol[2];
    const int64_t cpg = p.C / p.G;
    const int64_t R = smul(smul(smul(p.N, g.Do), g.Ho), g.Wo);
    const int64_t nx = smul(smul(smul(smul(p.N, g.Di), g.Hi), g.Wi), p.C);
    const int64_t ndy = smul(R, p.K);
    const int64_t ndw = smul(smul(smul(smul(p.K, g.Z), g.Y), g.X), cpg);
    if (nx > kMax31 || ndy > kMax31 || ndw > kMax31 || R > kMax31)
        return fail(msg, E, "tensor element offsets must fit in 31 bits");
    // index arithmetic on the padded input also stays in 31 bits (every
    // factor is below 2^31 here, so these products fit in int64)
    if ((g.Do * g.sd + g.Z * g.dd) > kMax31 || (g.Ho * g.sh + g.Y * g.dh) > kMax31 ||
        (g.Wo * g.sw + g.X * g.dw) > kMax31)
        return fail(msg, E, "spatial index range must fit in 31 bits");
    return WGRAD_OK;
}

}  // namespace

int build_plan(const wgrad_problem& p, const wgrad_overrides* ov, const DeviceModel& dev, Plan& out,
               std::string* msg) {
    const int E = WGRAD_ERR_INVALID_ARG, U = WGRAD_ERR_UNSUPPORTED;
    Geo g;
    if (int rc = check_problem(p, g, msg)) return rc;
    const int64_t cpg = p.C / p.G, kpg = p.K / p.G;
    const int64_t R = p.N * g.Do * g.Ho * g.Wo;
    const int64_t nx = p.N * g.Di * g.Hi * g.Wi * p.C;
    const int64_t ndy = R * p.K;
    const int64_t ndw = p.K * g.Z * g.Y * g.X * cpg;

    wgrad_overrides o{};
    if (ov) o = *ov;
    if (o.split_k < 0 || o.group_merge < 0 || o.variant < 0 || o.tile < 0)
        return fail(msg, E, "overrides must be >= 0");

    out = Plan{};
    out.prob = p;
    out.in_f16 = p.in_dtype == WGRAD_FP16;
    out.ring_inst = -1;
    out.dg_ring = -1;
    wgrad_plan_info& info = out.info;
    {
        const int64_t all[3] = {g.Do, g.Ho, g.Wo};
        for (int i = 0; i < 3; ++i) info.out_len[i] = i < p.ndim ? all[3 - p.ndim + i] : 0;
    }
    info.gemm_m = kpg;
    info.gemm_n = cpg * g.Z * g.Y * g.X;
    info.gemm_k = R;
    info.num_cus = dev.num_cus;
    const int out_final = p.out_dtype == WGRAD_BF16 ? OUT_BF16 : p.out_dtype == WGRAD_FP16 ? OUT_FP16 : OUT_FP32;
    const int64_t in_bytes = 2 * (nx + ndy);
    const char* dname = out.in_f16 ? "fp16" : "bf16";

    // ---- kernel family
    const bool dw_shape = cpg == 1 && kpg == 1 && p.C % 8 == 0 && p.ndim <= 2;
    // windowed depthwise kernel: width-3 filter, w-stride and w-dilation 1, height 1, 3 or 5
    const bool dw2_ok = g.X == 3 && g.sw == 1 && g.dw == 1 && (g.Y == 1 || g.Y == 3 || g.Y == 5) &&
                        2 * nx < (int64_t{1} << 31) && 2 * ndy < (int64_t{1} << 31);
    const bool dw_filter = dw2_ok || (g.Y == 3 && g.X == 3) || (g.Y == 1 && (g.X == 3 || g.X == 5));
    int variant = o.variant;
    if (variant == WGRAD_VARIANT_DGRAD) return fail(msg, U, "the DGRAD variant belongs to backward-data plans");
    if (variant < WGRAD_VARIANT_AUTO || variant > WGRAD_VARIANT_ROWSLAB)
        return fail(msg, E, "unknown variant %d", variant);
    std::string rs_why;
    // row-slab forms: the filter-row ring (tile 2) where it applies and is
    // preferred, else one filter row per workgroup (tile 1)
    auto plan_rs_forms = [&](int form, std::string* why) {
        if (form != 1 && ring_preferred(p, g) && plan_ring(p, g, o, dev, out_final, out, nullptr)) return true;
        if (form == 2) return plan_ring(p, g, o, dev, out_final, out, why);
        out.ring_inst = -1;
        return plan_rowslab(p, g, o, dev, out_final, out, why);
    };
    if (variant == WGRAD_VARIANT_AUTO) {
        if (dw_shape && dw_filter && !o.group_merge && !o.tile) variant = WGRAD_VARIANT_DEPTHWISE;
        else if (!o.tile && plan_rs_forms(0, &rs_why)) variant = WGRAD_VARIANT_ROWSLAB;
        else variant = WGRAD_VARIANT_MFMA;
    }
    if (variant == WGRAD_VARIANT_DEPTHWISE && !(dw_shape && dw_filter))
        return fail(msg, U, "depthwise variant needs a 1D or 2D problem with C/G = K/G = 1, C %% 8 == 0 and a 3x3, 1x3 or 1x5 filter");
    out.variant = variant;
    info.variant = variant;

    char name[256];
    if (variant == WGRAD_VARIANT_ROWSLAB) {
        if (o.tile > 2)
            return fail(msg, U, "row-slab variant: tile is 0 (auto), 1 (one filter row per workgroup) or 2 (filter-row ring)");
        if (!plan_rs_forms(o.tile, &rs_why)) return fail(msg, U, "%s", rs_why.c_str());
        if (out.ring_inst >= 0) {
            const RingArgs& a = out.ring;
            const RingInstance& ri = kRingInstances[out.ring_inst];
            snprintf(name, sizeof name, "wgrad_ring_%s_m%dc%dx3x3_k%d_w%d_s%dx%d_kouter_spk%d_gm%d", dname, ri.mb, kRingCB,
                     16 * ri.nks, ri.xwp, (int)g.sh, (int)g.sw, a.S, info.group_merge);
        } else {
            const RowSlabArgs& a = out.rs;
            const RsInstance& ri = kRsInstances[out.rs_inst];
            snprintf(name, sizeof name, "wgrad_rowslab_%s_m%dc%dx%d_k%d_slab%dx%d%s_kouter_spk%d_gm%d", dname, ri.mb,
                     ri.cb, ri.xf, 16 * ri.nks, a.PR, a.SW, ri.gs == 4 ? "_sg4" : ri.gs == 2 ? "_sg2" : "", a.S, info.group_merge);
        }
    } else if (variant == WGRAD_VARIANT_DEPTHWISE) {
        if (o.group_merge > 1) return fail(msg, U, "group_merge applies to the MFMA variant only");
        DwArgs& a = out.dwk;
        a = DwArgs{};
        a.C = (int32_t)p.C;
        a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
        a.Y = (int32_t)g.Y; a.Xf = (int32_t)g.X;
        a.sh = (int32_t)g.sh; a.sw = (int32_t)g.sw; a.dh = (int32_t)g.dh; a.dw = (int32_t)g.dw;
        a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
        a.R = (int32_t)R;
        int64_t vecs = p.C / 8;
        int cl = 8;
        while (vecs % cl) cl >>= 1;
        a.cl = cl;
        a.cblocks = (int32_t)(vecs / cl);
        const int pl = 256 / cl;
        int64_t S;
        const int64_t slice_bytes = ndw * 4;
        if (o.split_k) {
            S = o.split_k;
        } else {
            int64_t max_s = std::max<int64_t>(1, ceil_div(R, pl));   // at least one position per lane
            S = choose_split(a.cblocks, max_s, slice_bytes, in_bytes, dev, 4);
        }
        if (R == 0) S = 1;
        int64_t kslice = std::max<int64_t>(1, ceil_div(R, S));
        if (R > 0) S = ceil_div(R, kslice);
        // kernel form: strip (3x3, unit stride and dilation), windowed (width 3), or generic
        const bool dw3_ok = dw2_ok && g.Y == 3 && g.sh == 1 && g.dh == 1;
        // tile kernel: 256 channels a workgroup, two pixels' 512-byte runs per
        // 1 KB load (on the 512-channel 56x56 shape whole-pixel 512-channel
        // workgroups stream 1 % faster but write twice the partials, and the
        // step is 3 % slower)
        const int dwt_cb = p.C % 256 == 0 ? 256 : 0;
        const bool dwt_ok = dw3_ok && dwt_cb != 0;
        int form = o.tile ? o.tile : dwt_ok ? 4 : dw3_ok ? 3 : dw2_ok ? 2 : 1;
        if (form < 1 || form > 4) return fail(msg, U, "depthwise kernel form %d is not 1, 2, 3 or 4", form);
        if (form == 4 && !dwt_ok)
            return fail(msg, U, "tile depthwise kernel needs a 3x3 filter with unit stride and dilation and C a multiple of 256");
        if (form == 3 && !dw3_ok) return fail(msg, U, "strip depthwise kernel needs a 3x3 filter with unit stride and dilation");
        if (form == 2 && !dw2_ok) return fail(msg, U, "windowed depthwise kernel needs filter width 3, w-stride 1, w-dilation 1 and height 1, 3 or 5");
        if (form == 1 && !((g.Y == 3 && g.X == 3) || (g.Y == 1 && (g.X == 3 || g.X == 5))))
            return fail(msg, U, "generic depthwise kernel needs a 3x3, 1x3 or 1x5 filter");
        // channel lanes of the windowed and strip kernels: a wave covers up to
        // 64 x 8 = 512 channels of one pixel, so each load reads one contiguous run
        int cl2 = 64;
        while ((p.C / 8) % cl2) cl2 >>= 1;
        if (form == 4) {
            DwTileArgs& b = out.dwt;
            b = DwTileArgs{};
            b.C = (int32_t)p.C; b.Hi = (int32_t)g.Hi; b.Wi = (int32_t)g.Wi; b.Ho = (int32_t)g.Ho; b.Wo = (int32_t)g.Wo;
            b.ph = (int32_t)g.ph; b.pw = (int32_t)g.pw;
            const int64_t tw = dwt_tile_w(dwt_cb);
            b.tiles_x = (int32_t)ceil_div(g.Wo, tw);
            b.cblocks = (int32_t)(p.C / dwt_cb);
            // workgroups per channel block: one per CU unless overridden
            const int64_t slots = std::max<int64_t>(1, (int64_t)dev.num_cus / b.cblocks);
            // rows per tile: fewest passes x (rows + 2 halo rows + about 3 rows'
            // worth of pipeline start and end per tile)
            int64_t best_th = 1, best_cost = INT64_MAX;
            for (int64_t th = 1; th <= g.Ho; ++th) {
                const int64_t tiles = p.N * ceil_div(g.Ho, th) * b.tiles_x;
                const int64_t passes = ceil_div(std::max<int64_t>(tiles, 1), o.split_k ? o.split_k : slots);
                const int64_t cost = passes * (th + 5);
                if (cost < best_cost) { best_cost = cost; best_th = th; }
            }
            b.th = (int32_t)best_th;
            b.tiles_y = (int32_t)ceil_div(g.Ho, best_th);
            const int64_t tiles = p.N * b.tiles_y * b.tiles_x;
            if (tiles > kMax31) return fail(msg, U, "too many depthwise tiles");
            b.tiles = (int32_t)tiles;
            int64_t St = o.split_k ? o.split_k : slots;
            St = std::max<int64_t>(1, std::min<int64_t>(St, tiles));
            if (St > 65535 || St * b.cblocks > kMax31) return fail(msg, U, "split_k too large");
            b.S = (int32_t)St;
            b.total_wg = (int32_t)(St * b.cblocks);
            b.out_mode = St == 1 ? out_final : OUT_WORKSPACE;
            b.slice_elems = (int32_t)ndw;
            b.x_bytes = (uint32_t)(2 * nx);
            b.dy_bytes = (uint32_t)(2 * ndy);
            out.dwt_cb = dwt_cb;
            out.lds_bytes = dwt_lds_bytes(dwt_cb);
            S = St;
            cl = dwt_cb / 8;
        } else if (form == 3) {
            Dw3Args& b = out.dw3;
            b = Dw3Args{};
            b.C = (int32_t)p.C; b.Hi = (int32_t)g.Hi; b.Wi = (int32_t)g.Wi; b.Ho = (int32_t)g.Ho; b.Wo = (int32_t)g.Wo;
            b.ph = (int32_t)g.ph; b.pw = (int32_t)g.pw;
            b.nseg = (int32_t)ceil_div(g.Wo, 4);
            // lanes of kDw3Channels channels; one workgroup per CU, a split is
            // one workgroup's share of a channel block
            if (p.C % kDw3Channels) return fail(msg, U, "strip depthwise kernel needs C to be a multiple of %d", kDw3Channels);
            int cl3 = kDw3MaxLanes;
            while ((p.C / kDw3Channels) % cl3) cl3 >>= 1;
            b.cl = cl3;
            b.cblocks = (int32_t)(p.C / kDw3Channels / cl3);
            const int64_t nsub = 64 / cl3;
            const int64_t strips = p.N * b.nseg;
            int64_t S3 = o.split_k ? o.split_k : std::max<int64_t>(1, (int64_t)dev.num_cus / b.cblocks);
            // never more workgroups than strips need at one chunk per strip
            S3 = std::max<int64_t>(1, std::min<int64_t>(S3, ceil_div(std::max<int64_t>(strips * g.Ho, 1), kDw3Waves * nsub)));
            if (S3 > 65535 || S3 * b.cblocks > kMax31) return fail(msg, U, "split_k too large");
            // chunks per strip: fewest passes x rows per chunk, counting the
            // two ring rows loaded at each item's start as one more row
            const int64_t workers = kDw3Waves * nsub * S3;
            int64_t best_nch = 1, best_cost = INT64_MAX;
            for (int64_t nch = 1; nch <= std::max<int64_t>(1, g.Ho); ++nch) {
                const int64_t passes = ceil_div(std::max<int64_t>(strips * nch, 1), workers);
                const int64_t cost = passes * (ceil_div(g.Ho, nch) + 1);
                if (cost < best_cost) { best_cost = cost; best_nch = nch; }
            }
            if (strips * best_nch > kMax31) return fail(msg, U, "too many strip chunks");
            b.nch = (int32_t)best_nch;
            b.items = (int32_t)(strips * best_nch);
            b.S = (int32_t)S3;
            b.total_wg = (int32_t)(S3 * b.cblocks);
            b.out_mode = S3 == 1 ? out_final : OUT_WORKSPACE;
            b.slice_elems = (int32_t)ndw;
            b.x_bytes = (uint32_t)(2 * nx);
            b.dy_bytes = (uint32_t)(2 * ndy);
            out.dw3_ty = 3;
            S = S3;
            cl = cl3 * kDw3Channels / 8;   // reported in 8-channel units like the other forms
        } else if (form == 2) {
            // windowed kernel: units of 4 output positions; splits hold whole units
            Dw2Args& b = out.dw2;
            b = Dw2Args{};
            b.C = (int32_t)p.C; b.Hi = (int32_t)g.Hi; b.Wi = (int32_t)g.Wi; b.Ho = (int32_t)g.Ho; b.Wo = (int32_t)g.Wo;
            b.Y = (int32_t)g.Y; b.sh = (int32_t)g.sh; b.dh = (int32_t)g.dh; b.ph = (int32_t)g.ph; b.pw = (int32_t)g.pw;
            b.NHo = (int32_t)(p.N * g.Ho);
            b.nseg = (int32_t)ceil_div(g.Wo, 4);
            const int64_t units = (int64_t)b.NHo * b.nseg;
            b.units = (int32_t)units;
            b.cl = cl2;
            b.cblocks = (int32_t)(p.C / 8 / cl2);
            const int64_t ul = 256 / cl2;
            // one workgroup per CU (the kernel double-buffers a lane's loads in
            // registers and runs one wave per SIMD); a split's units are spread
            // over the workgroup's lanes, a lane takes every ul-th unit
            int64_t S2 = o.split_k ? o.split_k : std::max<int64_t>(1, (int64_t)dev.num_cus / b.cblocks);
            S2 = std::max<int64_t>(1, std::min<int64_t>(S2, std::max<int64_t>(1, ceil_div(units, ul))));
            const int64_t upw = std::max<int64_t>(1, ceil_div(units, S2));
            const int64_t upt = ceil_div(upw, ul);
            S2 = units > 0 ? ceil_div(units, upw) : 1;
            if (S2 > 65535 || S2 * b.cblocks > kMax31) return fail(msg, U, "split_k too large");
            b.upt = (int32_t)upt;
            b.upw = (int32_t)upw;
            b.S = (int32_t)S2;
            b.total_wg = (int32_t)(S2 * b.cblocks);
            b.out_mode = S2 == 1 ? out_final : OUT_WORKSPACE;
            b.slice_elems = (int32_t)ndw;
            b.x_bytes = (uint32_t)(2 * nx);
            b.dy_bytes = (uint32_t)(2 * ndy);
            b.mHo = make_magic((uint32_t)g.Ho);
            b.mSeg = make_magic((uint32_t)b.nseg);
            out.dw2_ty = (int)g.Y;
            S = S2;
            cl = cl2;
        }
        if (S > 65535) return fail(msg, U, "split_k too large");
        a.S = (int32_t)S;
        a.kslice = (int32_t)kslice;
        a.total_wg = (int32_t)(a.cblocks * S);
        a.out_mode = S == 1 ? out_final : OUT_WORKSPACE;
        a.slice_elems = (int32_t)ndw;
        a.mWo = make_magic((uint32_t)g.Wo);
        a.mHo = make_magic((uint32_t)g.Ho);
        out.dw_tile_y = (int)g.Y;
        out.dw_tile_x = (int)g.X;
        info.split_k = (int32_t)S;
        info.group_merge = 8 * cl;   // channels (groups) one workgroup covers
        info.vector_width = 8;
        info.grid_main = out.dwt_cb ? out.dwt.total_wg : out.dw3_ty ? out.dw3.total_wg
                                                       : out.dw2_ty ? out.dw2.total_wg : a.total_wg;
        info.tile = out.dwt_cb ? 4 : out.dw3_ty ? 3 : out.dw2_ty ? 2 : 1;
        info.workspace_bytes = S > 1 ? S * ndw * 4 : 0;
        if (out.dwt_cb)
            snprintf(name, sizeof name, "wgrad_dwtile_%s_3x3_t%dx%d_spk%lld_gm%d", dname, out.dwt.th,
                     dwt_tile_w(out.dwt_cb), (long long)S, 8 * cl);
        else
            snprintf(name, sizeof name, "wgrad_dw%s_%s_%lldx%lld_cl%d_spk%lld_gm%d",
                     out.dw3_ty ? "strip" : out.dw2_ty ? "win" : "", dname,
                     (long long)g.Y, (long long)g.X, cl, (long long)S, 8 * cl);
    } else {
        // ---- group merge degree
        int64_t Gm = o.group_merge;
        if (Gm) {
            if (!is_pow2(Gm) || p.G % Gm)
                return fail(msg, U, "group_merge %lld must be a power of two dividing G = %lld", (long long)Gm,
                            (long long)p.G);
        } else {
            // fill the 16-row MFMA edge with adjacent groups, at most 8 of them
            Gm = 1;
            while (Gm * 2 <= 8 && Gm * kpg < 16 && p.G % (Gm * 2) == 0) Gm *= 2;
        }
        const int64_t Mm = Gm * kpg, Nm = Gm * cpg * g.Z * g.Y * g.X;
        if (Mm > kMax31 || Nm > kMax31) return fail(msg, E, "merged GEMM too large");
        // ---- load vector width: a vector stays inside one channel run and
        // every run starts on a multiple of it
        int V = 8;
        while (V > 1 && ((Gm * kpg) % V || (Gm * cpg) % V || p.K % V || p.C % V)) V >>= 1;
        // ---- tile
        int tile_id = o.tile;
        if (!tile_id) tile_id = Mm <= 16 ? 5 : Mm <= 32 ? 4 : Mm <= 64 ? 2 : 3;
        const TileShape* t = find_tile(tile_id);
        if (!t) return fail(msg, U, "unknown tile id %d", tile_id);
        const int64_t tiles_m = ceil_div(Mm, t->bm), tiles_n = ceil_div(Nm, t->bn);
        const int64_t gblocks = p.G / Gm;
        const int64_t base = tiles_m * tiles_n * gblocks;
        const int64_t k_tiles = std::max<int64_t>(1, ceil_div(R, t->bk));
        int64_t S = o.split_k ? o.split_k : choose_split(base, k_tiles, ndw * 4, in_bytes, dev, 2);
        if (R == 0) S = 1;
        // slices hold whole K tiles, so S slices may round to fewer non-empty
        // ones; when choosing automatically, step down to a degree whose
        // effective count keeps the grid a multiple of the XCD count
        auto slice_len = [&](int64_t s) { return std::max<int64_t>(1, ceil_div(ceil_div(R, s), t->bk)) * t->bk; };
        auto effective = [&](int64_t s) { return R > 0 ? ceil_div(R, slice_len(s)) : int64_t{1}; };
        if (!o.split_k && S > 1) {
            const int64_t step = dev.num_xcds / gcd64(base, dev.num_xcds);
            for (int64_t s = S; s >= 2; --s) {
                const int64_t e = effective(s);
                if (e % step == 0) { S = s; break; }
                if (s < S / 2) break;   // do not give up more than half the parallelism
            }
        }
        int64_t kslice = slice_len(S);
        S = effective(S);
        if (S > 65535 || base * S > kMax31) return fail(msg, U, "grid too large");
        MfmaArgs& a = out.mfma;
        a = MfmaArgs{};
        a.Ktot = (int32_t)p.K; a.Ctot = (int32_t)p.C;
        a.kpg = (int32_t)kpg; a.cpg = (int32_t)cpg; a.Gm = (int32_t)Gm;
        a.gkpg = (int32_t)(Gm * kpg); a.gcpg = (int32_t)(Gm * cpg);
        a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
        a.Xf = (int32_t)g.X; a.Yf = (int32_t)g.Y;
        a.Di = (int32_t)g.Di; a.Do = (int32_t)g.Do; a.sd = (int32_t)g.sd; a.dd = (int32_t)g.dd; a.pd = (int32_t)g.pd;
        a.sh = (int32_t)g.sh; a.sw = (int32_t)g.sw; a.dh = (int32_t)g.dh; a.dw = (int32_t)g.dw;
        a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
        a.R = (int32_t)R;
        a.Mm = (int32_t)Mm; a.Nm = (int32_t)Nm;
        a.row_len = (int32_t)(g.Z * g.Y * g.X * cpg);
        a.tiles_m = (int32_t)tiles_m; a.tiles_n = (int32_t)tiles_n; a.gblocks = (int32_t)gblocks;
        a.S = (int32_t)S;
        a.kslice = (int32_t)kslice;
        a.total_wg = (int32_t)(base * S);
        a.out_mode = S == 1 ? out_final : OUT_WORKSPACE;
        a.slice_elems = (int32_t)ndw;
        a.mWo = make_magic((uint32_t)g.Wo);
        a.mHo = make_magic((uint32_t)g.Ho);
        a.mDo = make_magic((uint32_t)g.Do);
        info.tile = tile_id;
        info.tile_m = t->bm; info.tile_n = t->bn; info.tile_k = t->bk;
        info.split_k = (int32_t)S;
        info.group_merge = (int32_t)Gm;
        info.vector_width = V;
        info.grid_main = a.total_wg;
        info.workspace_bytes = S > 1 ? S * ndw * 4 : 0;
        snprintf(name, sizeof name, "wgrad_mfma_%s_t%d_%dx%dx%d_a%d_v%d_kouter_spk%lld_gm%lld", dname, tile_id,
                 t->bm, t->bn, t->bk, t->atom, V, (long long)S, (long long)Gm);
    }
    out.name = name;
    // ---- reduce / convert pass
    // slice lanes: the fewest that still give a few workgroups per CU
    const int vec4 = ndw % 4 == 0;
    const int64_t nvec = vec4 ? ndw / 4 : ndw;
    int zl = 1;
    while (zl < 64 && zl * 2 <= info.split_k && ceil_div(nvec, 256 / zl) < 2 * dev.num_cus) zl *= 2;
    out.red = ReduceArgs{nullptr, nullptr, (int32_t)ndw, info.split_k, out_final, zl, vec4};
    if (info.split_k > 1) info.grid_reduce = ceil_div(nvec, 256 / zl);
    return WGRAD_OK;
}

// Row-ring backward data (tile 6): 2D, 3x3 filter, unit stride and
// dilation, h-pads with pad_lo <= 2 and Ho <= Hi (so the two padding rows
// after each image read only zero dY rows), rows up to 64 wide, merged runs
// of 32 or 64 dY channels and a multiple of 32 dX channels, weight chunks
// inside one group. Returns false with a reason when the shape does not fit.
bool plan_dgrad_ring(const wgrad_problem& p, const Geo& g, int64_t Gm, const DeviceModel& dev, Plan& out,
                     std::string* why) {
    const int64_t cpg = p.C / p.G, kpg = p.K / p.G;
    auto no = [&](const char* m) { if (why) *why = m; return false; };
    if (p.ndim != 2 || g.Y != 3 || g.X != 3 || g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1)
        return no("row-ring dgrad needs a 2D 3x3 filter with unit stride and dilation");
    if (g.ph > 2 || g.Ho > g.Hi) return no("row-ring dgrad needs pad_lo <= 2 and pad_lo + pad_hi <= 2 along h");
    if (g.Wi > 64) return no("row-ring dgrad needs input rows of at most 64 positions");
    const int64_t gkpg = Gm * kpg, gcpg = Gm * cpg;
    if (cpg % 8 || p.K % 8 || p.C % 8) return no("row-ring dgrad needs 16-byte channel vectors inside one group");
    if (gkpg != 32 && gkpg != 64) return no("row-ring dgrad needs 32 or 64 merged output channels per group block");
    if (gcpg % 32) return no("row-ring dgrad needs a merged input-channel run that is a multiple of 32");
    const int64_t ndy = p.N * g.Ho * g.Wo * p.K, nw = p.K * 9 * cpg, ndx = p.N * g.Hi * g.Wi * p.C;
    if (2 * ndy >= (int64_t{1} << 31) || 2 * nw >= (int64_t{1} << 31) || 4 * ndx >= (int64_t{1} << 31))
        return no("row-ring dgrad needs dY, W and dX below 2 GiB");
    const int ch = (int)(gkpg / 8), mt = g.Wi <= 32 ? 1 : 2;
    const int pxl = 64 / ch;
    const int64_t qp = ceil_div(g.Wi + 2, pxl) * pxl;
    // 64 dX channels per block when the run allows it and the LDS holds it
    int inst = -1;
    for (int cbd : {64, 32}) {
        if (gcpg % cbd) continue;
        for (int i = 0; i < kNumDgRingInstances; ++i) {
            const DgradRingInstance& r = kDgRingInstances[i];
            if (r.cbd == cbd && r.mt == mt && r.ch == ch && dg_ring_lds_bytes(r, (int)qp) <= kDgRingLdsMax) inst = i;
        }
        if (inst >= 0) break;
    }
    if (inst < 0) return no("row-ring dgrad: no instance fits the LDS");
    const DgradRingInstance& ri = kDgRingInstances[inst];
    const int64_t VR = g.Hi + 2, NV = p.N * VR;
    const int64_t cblocks = gcpg / ri.cbd, tiles = (p.G / Gm) * cblocks;
    // four rows per step; as many splits as leave one workgroup per CU
    const int64_t s0 = std::max<int64_t>(1, (int64_t)dev.num_cus / tiles);
    const int64_t vpw = 4 * ceil_div(ceil_div(NV, s0), 4);
    const int64_t S = ceil_div(NV, vpw);
    if (tiles * S > kMax31) return no("row-ring dgrad grid too large");
    DgradRingArgs& a = out.dgr;
    a = DgradRingArgs{};
    a.Ktot = (int32_t)p.K; a.Ctot = (int32_t)p.C; a.kpg = (int32_t)kpg; a.cpg = (int32_t)cpg;
    a.Gm = (int32_t)Gm; a.gkpg = (int32_t)gkpg; a.gcpg = (int32_t)gcpg;
    a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
    a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
    a.N = (int32_t)p.N; a.VR = (int32_t)VR; a.NV = (int32_t)NV;
    a.cblocks = (int32_t)cblocks; a.tiles = (int32_t)tiles;
    a.vpw = (int32_t)vpw;
    a.qp = (int32_t)qp; a.nxl = (int32_t)(qp / pxl);
    a.total_wg = (int32_t)(tiles * S);
    a.out_mode = p.out_dtype == WGRAD_BF16 ? OUT_BF16 : p.out_dtype == WGRAD_FP16 ? OUT_FP16 : OUT_FP32;
    a.dy_bytes = (uint32_t)(2 * ndy); a.w_bytes = (uint32_t)(2 * nw);
    a.mVR = make_magic((uint32_t)VR); a.mkpg = make_magic((uint32_t)kpg); a.mcpg = make_magic((uint32_t)cpg);
    out.dg_ring = inst;
    return true;
}

int build_dgrad_plan(const wgrad_problem& p, const wgrad_overrides* ov, const DeviceModel& dev, Plan& out,
                     std::string* msg) {
    const int U = WGRAD_ERR_UNSUPPORTED;
    Geo g;
    if (int rc = check_problem(p, g, msg)) return rc;
    wgrad_overrides o{};
    if (ov) o = *ov;
    if (o.split_k < 0 || o.group_merge < 0 || o.variant < 0 || o.tile < 0)
        return fail(msg, WGRAD_ERR_INVALID_ARG, "overrides must be >= 0");
    if (o.split_k > 1) return fail(msg, U, "backward data does not split its reduction");
    if (o.group_merge && (!is_pow2(o.group_merge) || p.G % o.group_merge))
        return fail(msg, U, "group_merge %d must be a power of two dividing G = %lld", o.group_merge, (long long)p.G);
    if (o.variant != WGRAD_VARIANT_AUTO && o.variant != WGRAD_VARIANT_DGRAD)
        return fail(msg, U, "backward data plans use the DGRAD variant only");
    const int64_t cpg = p.C / p.G, kpg = p.K / p.G;
    const int64_t taps = g.Z * g.Y * g.X;
    const int64_t M = p.N * g.Di * g.Hi * g.Wi;
    // depthwise direct kernel (tile id 4): channel block cb = the largest
    // power of two <= 512 dividing C whose fp32 weights fit the LDS budget
    int dw_cb = 0;
    if (cpg == 1 && kpg == 1 && p.C % 8 == 0)
        for (int cb = 512; cb >= 8 && !dw_cb; cb >>= 1)
            if (p.C % cb == 0 && taps * cb * 4 <= kDgDwLdsMax) dw_cb = cb;
    // row-walking form: 3x3 in 2D, unit stride and dilation
    const bool ring_ok = dw_cb && g.Di == 1 && g.Z == 1 && g.Y == 3 && g.X == 3 && g.sh == 1 && g.sw == 1 &&
                         g.dh == 1 && g.dw == 1 && 2 * p.N * g.Ho * g.Wo * p.C < (int64_t{1} << 31);
    // tile form (tile id 7): whole 256-channel runs of the dY rows streamed
    // into an LDS ring; automatic where it applies
    const bool dwt_ok = ring_ok && p.C % 256 == 0;
    if (o.tile == 7 && (!dwt_ok || o.group_merge > 1))
        return fail(msg, U, "the depthwise dgrad tile kernel needs C/G = K/G = 1, C a multiple of 256 and a 2D 3x3 "
                            "filter with unit stride and dilation");
    if (dwt_ok && (o.tile == 7 || (o.tile == 0 && o.group_merge <= 1))) {
        out = Plan{};
        out.dg_ring = -1;
        out.op = OP_DGRAD;
        out.prob = p;
        out.in_f16 = p.in_dtype == WGRAD_FP16;
        out.variant = WGRAD_VARIANT_DGRAD;
        // 256-channel blocks (512-channel ones, whole pixels per load, measured
        // the same on the 512-channel 56x56 shape)
        const int cb = 256;
        out.dg_dwt = cb;
        DgradDwTileArgs& a = out.dgdwt;
        a = DgradDwTileArgs{};
        a.C = (int32_t)p.C;
        a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
        a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
        const int64_t tw = dwt_tile_w(cb);
        a.tiles_x = (int32_t)ceil_div(g.Wi, tw);
        a.cblocks = (int32_t)(p.C / cb);
        // dX rows per tile: fewest passes of one workgroup per CU x (rows +
        // 2 halo rows + about 3 rows' worth of pipeline start and end)
        int64_t best_th = 1, best_cost = INT64_MAX;
        for (int64_t th = 1; th <= g.Hi; ++th) {
            const int64_t tiles = p.N * ceil_div(g.Hi, th) * a.tiles_x * a.cblocks;
            const int64_t cost = ceil_div(std::max<int64_t>(tiles, 1), (int64_t)dev.num_cus) * (th + 5);
            if (cost < best_cost) { best_cost = cost; best_th = th; }
        }
        a.th = (int32_t)best_th;
        a.tiles_y = (int32_t)ceil_div(g.Hi, best_th);
        const int64_t tiles = p.N * a.tiles_y * a.tiles_x;
        if (tiles * a.cblocks > kMax31) return fail(msg, U, "grid too large");
        a.tiles = (int32_t)tiles;
        a.total_wg = (int32_t)std::min<int64_t>(tiles * a.cblocks, dev.num_cus);
        a.out_mode = p.out_dtype == WGRAD_BF16 ? OUT_BF16 : p.out_dtype == WGRAD_FP16 ? OUT_FP16 : OUT_FP32;
        a.dy_bytes = (uint32_t)(2 * p.N * g.Ho * g.Wo * p.C);
        wgrad_plan_info& info = out.info;
        {
            const int64_t all[3] = {g.Do, g.Ho, g.Wo};
            for (int i = 0; i < 3; ++i) info.out_len[i] = i < p.ndim ? all[3 - p.ndim + i] : 0;
        }
        info.gemm_m = M; info.gemm_n = 1; info.gemm_k = taps;
        info.variant = WGRAD_VARIANT_DGRAD;
        info.tile = 7;
        info.tile_m = (int32_t)(best_th * tw); info.tile_n = cb; info.tile_k = (int32_t)taps;
        info.split_k = 1; info.group_merge = 1; info.vector_width = 8;
        info.grid_main = a.total_wg;
        info.num_cus = dev.num_cus;
        char name[160];
        snprintf(name, sizeof name, "dgrad_dwtile_%s_t%dx%d", out.in_f16 ? "fp16" : "bf16", a.th, (int)tw);
        out.name = name;
        return WGRAD_OK;
    }
    const bool dw_tile = o.tile == 4 || o.tile == 5;
    if (dw_tile && o.group_merge > 1) return fail(msg, U, "the depthwise dgrad kernel does not merge groups");
    if (dw_tile && !dw_cb)
        return fail(msg, U, "the depthwise dgrad kernel needs C/G = K/G = 1, C %% 8 == 0 and at most %d taps",
                    kDgDwLdsMax / 32);
    if (dw_cb && (dw_tile || (o.tile == 0 && o.group_merge <= 1))) {
        out = Plan{};
        out.dg_ring = -1;
        out.op = OP_DGRAD;
        out.prob = p;
        out.in_f16 = p.in_dtype == WGRAD_FP16;
        out.variant = WGRAD_VARIANT_DGRAD;
        out.dg_dw = 1;
        DgradDwArgs& a = out.dgdw;
        a = DgradDwArgs{};
        a.C = (int32_t)p.C;
        a.Di = (int32_t)g.Di; a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi;
        a.Do = (int32_t)g.Do; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
        a.Zf = (int32_t)g.Z; a.Yf = (int32_t)g.Y; a.Xf = (int32_t)g.X; a.taps = (int32_t)taps;
        a.sd = (int32_t)g.sd; a.sh = (int32_t)g.sh; a.sw = (int32_t)g.sw;
        a.dd = (int32_t)g.dd; a.dh = (int32_t)g.dh; a.dw = (int32_t)g.dw;
        a.pd = (int32_t)g.pd; a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
        a.form = ring_ok && o.tile != 5 ? 2 : 1;
        // channel block: 8 channels per lane (per-tap form) or kDgRingCh
        // (row walk), at most 64 lanes
        int cb = dw_cb;
        if (a.form == 2) {
            cb = kDgRingMaxCb;
            while (p.C % cb) cb >>= 1;
        }
        const int lane_ch = a.form == 2 ? kDgRingCh : 8;
        a.cb = cb; a.cbv = cb / lane_ch; a.spw = 256 / a.cbv;
        a.nstrip = (int32_t)ceil_div(g.Wi, kDgDwStrip);
        const int64_t strips = p.N * g.Di * g.Hi * a.nstrip;
        const int64_t cblocks = p.C / cb;
        if (strips > kMax31) return fail(msg, U, "grid too large");
        a.strips = (int32_t)strips;
        int64_t sgroups;
        if (a.form == 2) {
            // row chunks per strip: about eight waves per CU (two per SIMD at
            // the kernel's register use) in as few passes as possible, each
            // chunk paying two extra rows to fill its window
            const int64_t per_chunk = p.N * a.nstrip;
            int64_t best = 1, best_cost = INT64_MAX;
            for (int64_t nch = 1; nch <= g.Hi; ++nch) {
                const int64_t waves = cblocks * ceil_div(per_chunk * nch * a.cbv, 64);
                const int64_t cost = ceil_div(waves, 8 * (int64_t)dev.num_cus) * (ceil_div(g.Hi, nch) + 2);
                if (cost <= best_cost) { best_cost = cost; best = nch; }
            }
            a.nch = (int32_t)best;
            const int64_t items = per_chunk * best;
            if (items > kMax31) return fail(msg, U, "grid too large");
            a.items = (int32_t)items;
            sgroups = ceil_div(items, a.spw);
        } else {
            sgroups = ceil_div(strips, a.spw);
        }
        if (cblocks * sgroups > kMax31) return fail(msg, U, "grid too large");
        a.cblocks = (int32_t)cblocks; a.sgroups = (int32_t)sgroups; a.total_wg = (int32_t)(cblocks * sgroups);
        a.dy_bytes = (uint32_t)(2 * p.N * g.Do * g.Ho * g.Wo * p.C);
        a.out_mode = p.out_dtype == WGRAD_BF16 ? OUT_BF16 : p.out_dtype == WGRAD_FP16 ? OUT_FP16 : OUT_FP32;
        a.msd = make_magic((uint32_t)g.sd); a.msh = make_magic((uint32_t)g.sh); a.msw = make_magic((uint32_t)g.sw);
        wgrad_plan_info& info = out.info;
        {
            const int64_t all[3] = {g.Do, g.Ho, g.Wo};
            for (int i = 0; i < 3; ++i) info.out_len[i] = i < p.ndim ? all[3 - p.ndim + i] : 0;
        }
        info.gemm_m = M; info.gemm_n = 1; info.gemm_k = taps;
        info.variant = WGRAD_VARIANT_DGRAD;
        info.tile = a.form == 2 ? 4 : 5;
        info.tile_m = kDgDwStrip * a.spw; info.tile_n = cb; info.tile_k = (int32_t)taps;
        info.split_k = 1; info.group_merge = 1; info.vector_width = lane_ch;
        info.grid_main = a.total_wg;
        info.num_cus = dev.num_cus;
        char name[160];
        if (a.form == 2)
            snprintf(name, sizeof name, "dgrad_dwring_%s_cb%d_s%d_ch%d", out.in_f16 ? "fp16" : "bf16", cb, kDgDwStrip, a.nch);
        else
            snprintf(name, sizeof name, "dgrad_dw_%s_cb%d_s%d", out.in_f16 ? "fp16" : "bf16", cb, kDgDwStrip);
        out.name = name;
        return WGRAD_OK;
    }
    // merge adjacent groups until both merged runs fill the 32-wide MFMA
    // edges (at most 8: the block-diagonal GEMM does Gm times the useful work)
    int64_t Gm = o.group_merge;
    if (!Gm) {
        Gm = 1;
        while (Gm * 2 <= 8 && p.G % (Gm * 2) == 0 && (Gm * cpg < 32 || Gm * kpg < 32)) Gm *= 2;
    }
    const int64_t gkpg = Gm * kpg, gcpg = Gm * cpg;
    // row-ring form (tile 6), automatic where it applies
    if (o.tile == 6 || o.tile == 0) {
        Plan rp{};
        std::string why;
        if (p.N > 0 && plan_dgrad_ring(p, g, Gm, dev, rp, &why)) {
            out = Plan{};
            out.op = OP_DGRAD;
            out.prob = p;
            out.in_f16 = p.in_dtype == WGRAD_FP16;
            out.variant = WGRAD_VARIANT_DGRAD;
            out.dg_ring = rp.dg_ring;
            out.dgr = rp.dgr;
            const DgradRingInstance& ri = kDgRingInstances[out.dg_ring];
            wgrad_plan_info& info = out.info;
            {
                const int64_t all[3] = {g.Do, g.Ho, g.Wo};
                for (int i = 0; i < 3; ++i) info.out_len[i] = i < p.ndim ? all[3 - p.ndim + i] : 0;
            }
            info.gemm_m = M; info.gemm_n = cpg; info.gemm_k = kpg * taps;
            info.variant = WGRAD_VARIANT_DGRAD;
            info.tile = 6;
            info.tile_m = 32 * ri.mt; info.tile_n = ri.cbd; info.tile_k = 16;
            info.split_k = 1; info.group_merge = (int32_t)Gm; info.vector_width = 8;
            info.grid_main = out.dgr.total_wg;
            info.num_cus = dev.num_cus;
            char name[160];
            snprintf(name, sizeof name, "dgrad_ring_%s_m%dx32_n%d_k%d_v%d_gm%lld", out.in_f16 ? "fp16" : "bf16", ri.mt,
                     ri.cbd, 8 * ri.ch, out.dgr.vpw, (long long)Gm);
            out.name = name;
            return WGRAD_OK;
        }
        if (o.tile == 6) return fail(msg, U, "%s", p.N > 0 ? why.c_str() : "row-ring dgrad needs N > 0");
    }
    int V = 8;
    while (V > 1 && (kpg % V || cpg % V || p.K % V || p.C % V)) V >>= 1;
    int tile_id = o.tile;
    if (!tile_id) {
        const int64_t tm = ceil_div(M, 128);
        tile_id = gcpg <= 32 ? 1 : gcpg <= 64 ? 2 : (tm * ceil_div(gcpg, 128) * (p.G / Gm) >= 2 * dev.num_cus ? 3 : 2);
    }
    const DgradTile* t = nullptr;
    for (const auto& d : kDgradTiles)
        if (d.id == tile_id) t = &d;
    if (!t) return fail(msg, U, "unknown dgrad tile id %d", tile_id);
    // stride phases: one grid slice per (di mod sd, hi mod sh, wi mod sw),
    // each over the phase grid of ceil(Di/sd) x ceil(Hi/sh) x ceil(Wi/sw)
    if (g.sd > kDgMaxStride || g.sh > kDgMaxStride || g.sw > kDgMaxStride)
        return fail(msg, U, "the dgrad kernel supports strides up to %d", kDgMaxStride);
    // the phase tables hold 16-bit tap indices and output offsets
    if (g.Z > 32767 || g.Y > 32767 || g.X > 32767 || g.pd > 32767 || g.ph > 32767 || g.pw > 32767 ||
        g.dd * g.Z > 32767 || g.dh * g.Y > 32767 || g.dw * g.X > 32767)
        return fail(msg, U, "filter, pad or dilation too large for the dgrad kernel");
    const int64_t qd = ceil_div(g.Di, g.sd), qh = ceil_div(g.Hi, g.sh), qw = ceil_div(g.Wi, g.sw);
    const int64_t phases = g.sd * g.sh * g.sw;
    const int64_t Mq = p.N * qd * qh * qw;
    const int64_t tiles_m = ceil_div(Mq, t->bm), tiles_n = ceil_div(gcpg, t->bn);
    const int64_t total = phases * tiles_m * tiles_n * (p.G / Gm);
    const int64_t ndy = p.N * g.Do * g.Ho * g.Wo * p.K, nw = p.K * taps * cpg;
    if (2 * ndy >= (int64_t{1} << 31) || 2 * nw >= (int64_t{1} << 31))
        return fail(msg, U, "the dgrad kernel needs dY and W below 2 GiB each");
    if (total > kMax31 || Mq > kMax31) return fail(msg, U, "grid too large");
    out = Plan{};
    out.dg_ring = -1;
    out.op = OP_DGRAD;
    out.prob = p;
    out.in_f16 = p.in_dtype == WGRAD_FP16;
    out.variant = WGRAD_VARIANT_DGRAD;
    DgradArgs& a = out.dg;
    a = DgradArgs{};
    a.Ktot = (int32_t)p.K; a.Ctot = (int32_t)p.C; a.kpg = (int32_t)kpg; a.cpg = (int32_t)cpg;
    a.Gm = (int32_t)Gm; a.gkpg = (int32_t)gkpg; a.gcpg = (int32_t)gcpg;
    a.Di = (int32_t)g.Di; a.Hi = (int32_t)g.Hi; a.Wi = (int32_t)g.Wi;
    a.Do = (int32_t)g.Do; a.Ho = (int32_t)g.Ho; a.Wo = (int32_t)g.Wo;
    a.Zf = (int32_t)g.Z; a.Yf = (int32_t)g.Y; a.Xf = (int32_t)g.X; a.taps = (int32_t)taps;
    a.sd = (int32_t)g.sd; a.sh = (int32_t)g.sh; a.sw = (int32_t)g.sw;
    a.dd = (int32_t)g.dd; a.dh = (int32_t)g.dh; a.dw = (int32_t)g.dw;
    a.pd = (int32_t)g.pd; a.ph = (int32_t)g.ph; a.pw = (int32_t)g.pw;
    a.zstep = (int32_t)(g.sd / gcd64(g.sd, g.dd)); a.zdo = (int32_t)(g.dd / gcd64(g.sd, g.dd));
    a.ystep = (int32_t)(g.sh / gcd64(g.sh, g.dh)); a.ydo = (int32_t)(g.dh / gcd64(g.sh, g.dh));
    a.xstep = (int32_t)(g.sw / gcd64(g.sw, g.dw)); a.xdo = (int32_t)(g.dw / gcd64(g.sw, g.dw));
    {
        // per axis and residue r: the taps t with (r + pad - t*dil) divisible
        // by the stride form t0, t0 + step, ... below the filter length
        const int64_t fl[3] = {g.Z, g.Y, g.X}, st[3] = {g.sd, g.sh, g.sw}, dl[3] = {g.dd, g.dh, g.dw},
                      pl[3] = {g.pd, g.ph, g.pw};
        for (int ax = 0; ax < 3; ++ax) {
            const int64_t step = st[ax] / gcd64(st[ax], dl[ax]);
            for (int64_t r = 0; r < st[ax]; ++r) {
                int64_t t0 = 0;
                while (t0 < step && t0 < fl[ax] && (r + pl[ax] - t0 * dl[ax]) % st[ax] != 0) ++t0;
                const bool any = t0 < step && t0 < fl[ax];
                a.t0[ax][r] = (int16_t)(any ? t0 : 0);
                a.nt[ax][r] = (int16_t)(any ? (fl[ax] - 1 - t0) / step + 1 : 0);
                a.o0[ax][r] = (int16_t)(any ? (r + pl[ax] - t0 * dl[ax]) / st[ax] : 0);
            }
        }
    }
    a.qd = (int32_t)qd; a.qh = (int32_t)qh; a.qw = (int32_t)qw;
    a.phases = (int32_t)phases;
    a.ph_rot = (int32_t)std::max<int64_t>(1, dev.num_cus / 8 / phases);
    a.M = (int32_t)Mq;
    const int bk = 32;   // channels per reduction chunk (the kernel's BK)
    a.kchunks = (int32_t)ceil_div(gkpg, bk);
    a.dy_bytes = (uint32_t)(2 * ndy);
    a.w_bytes = (uint32_t)(2 * nw);
    a.tiles_m = (int32_t)tiles_m; a.tiles_n = (int32_t)tiles_n; a.total_wg = (int32_t)total;
    a.out_mode = p.out_dtype == WGRAD_BF16 ? OUT_BF16 : p.out_dtype == WGRAD_FP16 ? OUT_FP16 : OUT_FP32;
    a.mqw = make_magic((uint32_t)qw); a.mqh = make_magic((uint32_t)qh); a.mqd = make_magic((uint32_t)qd);
    a.mkpg = make_magic((uint32_t)kpg); a.mcpg = make_magic((uint32_t)cpg);
    out.dg_bn = t->bn;
    out.dg_bk = bk;
    out.dg_v = V;
    wgrad_plan_info& info = out.info;
    {
        const int64_t all[3] = {g.Do, g.Ho, g.Wo};
        for (int i = 0; i < 3; ++i) info.out_len[i] = i < p.ndim ? all[3 - p.ndim + i] : 0;
    }
    info.gemm_m = M;
    info.gemm_n = cpg;
    info.gemm_k = kpg * taps;
    info.variant = WGRAD_VARIANT_DGRAD;
    info.tile = tile_id;
    info.tile_m = t->bm; info.tile_n = t->bn; info.tile_k = bk;
    info.split_k = 1;
    info.group_merge = (int32_t)Gm;
    info.vector_width = V;
    info.grid_main = total;
    info.grid_reduce = 0;
    info.workspace_bytes = 0;
    info.num_cus = dev.num_cus;
    char name[160];
    snprintf(name, sizeof name, "dgrad_mfma_%s_t%d_%dx%dx%d_v%d_kouterB_gm%lld", out.in_f16 ? "fp16" : "bf16", tile_id,
             t->bm, t->bn, bk, V, (long long)Gm);
    out.name = name;
    return WGRAD_OK;
}

}  // namespace wgrad
