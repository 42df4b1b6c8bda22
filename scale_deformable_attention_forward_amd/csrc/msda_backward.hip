// Backward of multi-scale deformable attention for gfx950 (float32 or
// bfloat16 storage, float32 arithmetic).
//
// For every (b, q, h) and sample (l, p), with G = grad_output[b, q, h*C_h:(h+1)*C_h]
// and S the bilinear sample ("MS Deformable Attention Backward Kernel API
// Reference", Returns and Notes):
//   grad_A[b,q,h,l,p]      = <G, S>
//   grad_loc[b,q,h,l,p,x]  = A * <G, dS/dx> * dx/du_x    (same for y)
//   grad_value[corner]    += A * w_corner * G             (every in-range corner)
//
// Fast path (C_h % 4 == 0, C_h <= 64, channel rows aligned to 4 elements):
//  1. backward_fast_kernel, one unit = one (b, h, q) owned by C_h/4 lanes with
//     4 channels per lane. Per chunk of up to SC samples the workgroup stages,
//     one thread per (unit, sample), the corner pixel index, in-range mask,
//     fractional offsets, coordinate slopes (0 where border padding clamped)
//     and the attention weight in LDS. The unit's lanes re-gather the four
//     corners, form S, dS/dx and dS/dy, reduce the three dot products with
//     DPP, and grad_A / grad_loc leave through LDS as coalesced stores. When
//     grad_value is wanted, the staging also writes each sample's anchor
//     corner (x0, y0) and a record of its anchor, fractions and weight to the
//     workspace.
//  2. grad_value by destination instead of by source, so no float atomics and
//     no order-dependent sums (global float atomics run at about one 128-byte
//     line per request and LDS float atomics are an order of magnitude slower
//     than LDS integer atomics on this part). Each level is cut into bands of
//     rows x cols pixels; band_count / band_scan / band_fill bucket the
//     samples into one list per (b, h, band); tile_scatter_kernel takes one
//     band (and, for dense coarse levels, one chunk of its list), sorts the
//     entries by anchor corner in LDS, and each lane group adds A * w * G of
//     the entries of its block of anchor bins to the four pixels each reaches,
//     in registers, then trades the pixels of its block's rim with the
//     neighbouring groups. A band of one chunk is stored directly; the chunks
//     of a split band write
//     float32 partial tiles to the workspace and band_reduce_kernel adds them
//     in chunk order. grad_value is therefore bitwise reproducible.
// Generic path (any C_h / alignment): backward_generic_kernel, one channel per
// lane, grad_value through float atomics issued one channel per lane (into
// grad_value for float32, into a float32 workspace then converted for
// bfloat16); its grad_value may differ in the last bits from run to run.
#include <algorithm>

#include "msda_device.h"

namespace msda {

struct BwdRecord {
    float fx, fy;   // fractional offsets inside the cell
    float kx, ky;   // d(pixel)/d(location) per axis, 0 where border clamped
    int32_t off;    // element offset of corner (x0, y0) within the (b, h) slab of value
    int32_t rowp;   // element distance between pixel rows of the level
    int32_t mask;   // bit k: corner k = 2*dy + dx lies inside the level
    float a;        // attention weight
};
static_assert(sizeof(BwdRecord) == 2 * sizeof(float4), "records must tile two float4 slots");

// grad_value is overwritten: cleared by plain store kernels.
__global__ __launch_bounds__(kBlock) void zero4_kernel(float4* __restrict__ p, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(kBlock) void zero1_kernel(float* __restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

__global__ __launch_bounds__(kBlock) void zero_u16_kernel(uint16_t* __restrict__ p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// bfloat16 grad_value of the generic path from its float32 accumulator:
// dst = RNE(acc (+ dst when accumulating)).
__global__ __launch_bounds__(kBlock) void acc_to_bf16_kernel(const float* __restrict__ acc,
                                                             uint16_t* __restrict__ dst, int64_t n,
                                                             int accumulate)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float v = acc[i] + (accumulate ? bf16_to_f32(dst[i]) : 0.f);
        dst[i] = f32_to_bf16_rne(v);
    }
}

// Sum over aligned groups of LPU lanes; every lane of a group gets the total
// (pairwise butterfly, so all lanes add in the same order and agree bitwise).
template <int LPU>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (LPU >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));  // xor 1
    if constexpr (LPU >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));  // xor 2
    if constexpr (LPU >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false)); // mirror 8
    if constexpr (LPU >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, false)); // mirror 16
    if constexpr (LPU >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (LPU >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Unit u -> (b, h, q) with q fastest.
struct UnitIdx {
    int b, h, q;
};
__device__ __forceinline__ UnitIdx unit_index(const Geometry& g, int u)
{
    UnitIdx r;
    const int t = fdiv(u, g.nq_div);
    r.q = u - t * g.Nq;
    r.b = fdiv(t, g.nh_div);
    r.h = t - r.b * g.Nh;
    return r;
}

__device__ __forceinline__ int value_slab_offset(const Geometry& g, int b, int h)
{
    return g.bnlc ? (b * g.Nh + h) * g.L * g.Ch : b * g.L * g.Nh * g.Ch + h * g.Ch;
}

// Read the normalised (x, y) of sample si of unit (b, q, h).
__device__ __forceinline__ void read_loc(const Geometry& g, const float* __restrict__ loc, int b, int q, int h,
                                         int si, float& ux, float& uy)
{
    const int S = g.S;
    if (g.b2q) {
        const int plane = g.Nq * g.Nh * S;
        const int j = b * 2 * plane + (q * g.Nh + h) * S + si;
        ux = loc[j];
        uy = loc[j + plane];
    } else {
        const int idx = ((b * g.Nq + q) * g.Nh + h) * S + si;
        if (g.loc_pair_aligned) {
            const float2 xy = *reinterpret_cast<const float2*>(loc + 2 * idx);
            ux = xy.x;
            uy = xy.y;
        } else {
            ux = loc[2 * idx];
            uy = loc[2 * idx + 1];
        }
    }
}

// Coordinate map, padding and corners of one sample of level (H, W, start).
// (x0, y0) receives the anchor corner in level pixels.
__device__ __forceinline__ BwdRecord make_record(const Geometry& g, float ux, float uy, float a, int H, int W,
                                                 int start, int& x0, int& y0)
{
    BwdRecord r;
    float x = pixel_coord(ux, W, g.align_corners);
    float y = pixel_coord(uy, H, g.align_corners);
    float kx = g.align_corners ? (float)(W - 1) : (float)W;
    float ky = g.align_corners ? (float)(H - 1) : (float)H;
    if (g.border) {
        if (!(x >= 0.f)) { x = 0.f; kx = 0.f; }  // also NaN
        else if (x > (float)(W - 1)) { x = (float)(W - 1); kx = 0.f; }
        if (!(y >= 0.f)) { y = 0.f; ky = 0.f; }
        else if (y > (float)(H - 1)) { y = (float)(H - 1); ky = 0.f; }
    } else {
        // anything past [-1, W] reads nothing; keeps the int conversion safe
        x = fminf(fmaxf(x, -2.f), (float)(W + 1));
        y = fminf(fmaxf(y, -2.f), (float)(H + 1));
    }
    const float x0f = floorf(x), y0f = floorf(y);
    x0 = (int)x0f;
    y0 = (int)y0f;
    const bool ix0 = x0 >= 0 && x0 < W, ix1 = x0 >= -1 && x0 + 1 < W;
    const bool iy0 = y0 >= 0 && y0 < H, iy1 = y0 >= -1 && y0 + 1 < H;
    r.fx = x - x0f;
    r.fy = y - y0f;
    r.kx = kx;
    r.ky = ky;
    const uint32_t pstride = (uint32_t)(g.bnlc ? g.Ch : g.Nh * g.Ch);  // element distance between neighbouring pixels
    r.off = (int32_t)((uint32_t)(start + y0 * W + x0) * pstride);  // may wrap for corners outside the level (masked)
    r.rowp = (int32_t)((uint32_t)W * pstride);
    r.mask = (ix0 && iy0 ? 1 : 0) | (ix1 && iy0 ? 2 : 0) | (ix0 && iy1 ? 4 : 0) | (ix1 && iy1 ? 8 : 0);
    r.a = a;
    return r;
}

// Per-sample data for the destination-tiled grad_value pass, laid out
// [b * N_h + h][l][q][p]: the anchor corner packed (x0 + 2) | (y0 + 2) << 16
// (x0, y0 >= -2 after the clamp above) on its own for the bucketing kernels,
// and (anchor bits, fx, fy, A) as one 16-byte record for the tile kernel,
// stored non-temporal: it is read about once, by the tile kernel, and would
// otherwise take cache room from the inputs.
struct AnchorWs {
    uint32_t* anchor;
    float4* rec;
};

// Stage one record per (unit, sample) of the chunk [s0, s0 + sc).
__device__ __forceinline__ void stage_records(const Geometry& g, const float* __restrict__ loc,
                                              const float* __restrict__ attn, BwdRecord* s_rec, int row,
                                              int u0, int upb, int s0, int sc, const FastDiv& scd,
                                              const int4* s_lv)
{
    for (int i = threadIdx.x; i < upb * sc; i += blockDim.x) {
        const int gi = fdiv(i, scd);
        const int s = i - gi * sc;
        const int uu = u0 + gi;
        BwdRecord r = {0.f, 0.f, 0.f, 0.f, 0, 1, 0, 0.f};
        if (uu < g.units) {
            const UnitIdx ui = unit_index(g, uu);
            const int si = s0 + s;
            const int l = fdiv(si, g.np_div);
            const int4 lvl = s_lv[l];
            const int H = lvl.x, W = lvl.y, start = lvl.z;
            float ux, uy;
            read_loc(g, loc, ui.b, ui.q, ui.h, si, ux, uy);
            const float a = attn[((ui.b * g.Nq + ui.q) * g.Nh + ui.h) * g.S + si];
            int x0, y0;
            r = make_record(g, ux, uy, a, H, W, start, x0, y0);
        }
        s_rec[gi * row + s] = r;
    }
}

// Record of the fast path: fractions, the coordinate slopes times the
// attention weight, and the four corners' element offsets in value
// (no_corner<T, BUF>() for a corner outside the level).
struct BwdFastRecord {
    float fx, fy;
    float akx, aky;  // A * d(pixel)/d(location), 0 where border clamped
    int4 o;          // corners (x0,y0), (x0+1,y0), (x0,y0+1), (x0+1,y0+1)
};
static_assert(sizeof(BwdFastRecord) == 2 * sizeof(float4), "records must tile two float4 slots");

// Stage one fast-path record per (unit, sample) of the chunk [s0, s0 + sc),
// and (with ws) the per-sample anchor of the grad_value pass.
template <typename T, bool BUF>
__device__ __forceinline__ void stage_fast_records(const Geometry& g, const float* __restrict__ loc,
                                                   const float* __restrict__ attn, BwdFastRecord* s_rec, int row,
                                                   int u0, int upb, int s0, int sc, const FastDiv& scd,
                                                   const int4* s_lv, AnchorWs ws)
{
    const int32_t nc = no_corner<T, BUF>();
    const int pstride = g.bnlc ? g.Ch : g.Nh * g.Ch;
    for (int i = threadIdx.x; i < upb * sc; i += blockDim.x) {
        const int gi = fdiv(i, scd);
        const int s = i - gi * sc;
        const int uu = u0 + gi;
        BwdFastRecord f = {0.f, 0.f, 0.f, 0.f, make_int4(nc, nc, nc, nc)};
        if (uu < g.units) {
            const UnitIdx ui = unit_index(g, uu);
            const int si = s0 + s;
            const int l = fdiv(si, g.np_div);
            const int4 lvl = s_lv[l];
            const int H = lvl.x, W = lvl.y, start = lvl.z;
            float ux, uy;
            read_loc(g, loc, ui.b, ui.q, ui.h, si, ux, uy);
            const float a = attn[((ui.b * g.Nq + ui.q) * g.Nh + ui.h) * g.S + si];
            int x0, y0;
            const BwdRecord r = make_record(g, ux, uy, a, H, W, start, x0, y0);
            const int o00 = value_slab_offset(g, ui.b, ui.h) + r.off;
            f.fx = r.fx;
            f.fy = r.fy;
            f.akx = a * r.kx;
            f.aky = a * r.ky;
            f.o.x = (r.mask & 1) ? o00 : nc;
            f.o.y = (r.mask & 2) ? o00 + pstride : nc;
            f.o.z = (r.mask & 4) ? o00 + r.rowp : nc;
            f.o.w = (r.mask & 8) ? o00 + r.rowp + pstride : nc;
            if (ws.anchor) {
                const int k = (((ui.b * g.Nh + ui.h) * g.Nl + l) * g.Nq + ui.q) * g.Np + (si - l * g.Np);
                // a sample that border padding clamped onto a level's edge
                // (fraction 0, slope 0) reaches only pixel column x0, which
                // anchor x0 - 1 with fraction 1 reaches with the same weight:
                // every other such sample takes that anchor, so the edge's
                // pile-up is split over two bins (in x and in y, so a
                // corner's over four); the grad_value terms are unchanged
                int ax = x0, ay = y0;
                float sfx = r.fx, sfy = r.fy;
                if (r.kx == 0.f && sfx == 0.f && x0 >= 0 && (k & 1)) { ax = x0 - 1; sfx = 1.f; }
                if (r.ky == 0.f && sfy == 0.f && y0 >= 0 && (k & 2)) { ay = y0 - 1; sfy = 1.f; }
                const uint32_t an = (uint32_t)(ax + 2) | ((uint32_t)(ay + 2) << 16);
                ws.anchor[k] = an;
                nt_store4(reinterpret_cast<float*>(ws.rec + k), __uint_as_float(an), sfx, sfy, a);
            }
        }
        s_rec[gi * row + s] = f;
    }
}

// Write grad_A and grad_loc of the chunk from LDS with coalesced stores.
__device__ __forceinline__ void store_results(const Geometry& g, const float4* s_res, int row, int u0, int upb,
                                              int s0, int sc, const FastDiv& scd, float* __restrict__ grad_loc,
                                              float* __restrict__ grad_attn)
{
    for (int i = threadIdx.x; i < upb * sc; i += blockDim.x) {
        const int gi = fdiv(i, scd);
        const int s = i - gi * sc;
        const int uu = u0 + gi;
        if (uu >= g.units) continue;
        const UnitIdx ui = unit_index(g, uu);
        const int si = s0 + s;
        const int idx = ((ui.b * g.Nq + ui.q) * g.Nh + ui.h) * g.S + si;
        const float4 res = s_res[gi * row + s];
        if (grad_attn) nt_store(grad_attn + idx, res.x);
        if (grad_loc) {
            if (g.b2q) {
                const int plane = g.Nq * g.Nh * g.S;
                const int j = ui.b * 2 * plane + (ui.q * g.Nh + ui.h) * g.S + si;
                nt_store(grad_loc + j, res.y);
                nt_store(grad_loc + j + plane, res.z);
            } else if (g.loc_pair_aligned) {
                nt_store2(grad_loc + 2 * idx, res.y, res.z);
            } else {
                nt_store(grad_loc + 2 * idx, res.y);
                nt_store(grad_loc + 2 * idx + 1, res.z);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Fast path, kernel 1: C_h <= VEC * LPU <= 64, C_h % VEC == 0, channel rows
// aligned to VEC elements. LPU lanes per unit, VEC channels per lane (4; 8
// for bfloat16 rows of whole 16-byte groups: one 16-byte load per corner).
template <typename T, int LPU, bool BUF, int VEC>
__global__ __launch_bounds__(kBlock) void backward_fast_kernel(Geometry g, int sc_max, ChunkDiv cdiv,
                                                               int64_t value_bytes,
                                                               const T* __restrict__ grad_out,
                                                               const T* __restrict__ value,
                                                               const float* __restrict__ loc,
                                                               const float* __restrict__ attn,
                                                               float* __restrict__ grad_loc,
                                                               float* __restrict__ grad_attn, AnchorWs ws)
{
    constexpr int upb = kBlock / LPU;  // units per workgroup

    extern __shared__ float4 smem[];
    const int row = sc_max + 1;
    BwdFastRecord* s_rec = reinterpret_cast<BwdFastRecord*>(smem);
    float4* s_res = smem + 2 * upb * row;
    __shared__ int4 s_lv[kMaxLevels];
    fill_level_table(g.lv, s_lv);

    const int tid = threadIdx.x;
    const int u0 = xcd_logical_block(blockIdx.x, gridDim.x) * upb;
    const bool want_dots = grad_loc != nullptr || grad_attn != nullptr;
    const __amdgpu_buffer_rsrc_t vr = value_rsrc(value, BUF ? value_bytes : 0);

    const int grp = tid / LPU, lig = tid % LPU;
    const int u = u0 + grp;
    const bool unit_ok = u < g.units;
    const UnitIdx ui = unit_index(g, unit_ok ? u : 0);
    const int c0 = lig * VEC;
    const bool lane_ok = unit_ok && c0 < g.Ch;
    float G[VEC] = {};
    if (lane_ok && want_dots)
        VecIO<T, VEC>::load(grad_out + ((ui.b * g.Nq + ui.q) * g.Nh + ui.h) * g.Ch + c0, G);

    for (int s0 = 0; s0 < g.S; s0 += sc_max) {
        const int sc = min(sc_max, g.S - s0);
        if (s0 > 0) __syncthreads();
        const FastDiv& scd = cdiv.of(sc, sc_max);
        stage_fast_records<T, BUF>(g, loc, attn, s_rec, row, u0, upb, s0, sc, scd, s_lv, ws);
        if (!want_dots) continue;
        __syncthreads();
        if (unit_ok) {
            for (int s = 0; s < sc; ++s) {
                const BwdFastRecord r = s_rec[grp * row + s];
                const int ok[4] = {r.o.x, r.o.y, r.o.z, r.o.w};
                float v[4][VEC];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (BUF) {
                        BufIO<T, VEC>::load(vr, (uint32_t)(ok[k] + c0) * (uint32_t)sizeof(T), v[k]);
                    } else {
#pragma unroll
                        for (int i = 0; i < VEC; ++i) v[k][i] = 0.f;
                        // no_corner<T, false>() is -1
                        if (lane_ok && ok[k] >= 0) VecIO<T, VEC>::load(value + ok[k] + c0, v[k]);
                    }
                }
                if (BUF && !lane_ok) {
                    // channels past C_h: read as zero (G is zero there too)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
#pragma unroll
                        for (int i = 0; i < VEC; ++i) v[k][i] = 0.f;
                }
                // the three dot products are linear in the four corner rows: form this
                // lane's <G, v_k> for each corner k, then combine them
                float d[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    d[k] = G[0] * v[k][0];
#pragma unroll
                    for (int i = 1; i < VEC; ++i) d[k] = __builtin_fmaf(G[i], v[k][i], d[k]);
                }
                // interpolate along x first: r0 and r1 are the dots of the
                // two corner rows' x-interpolations, so <G, S> = r0 + fy (r1 - r0),
                // <G, dS/dy> = r1 - r0 and <G, dS/dx> = e0 + fy (e1 - e0) with
                // e0, e1 the rows' x-differences
                const float e0 = d[1] - d[0], e1 = d[3] - d[2];
                const float r0 = __builtin_fmaf(r.fx, e0, d[0]), r1 = __builtin_fmaf(r.fx, e1, d[2]);
                float py = r1 - r0;
                float pa = __builtin_fmaf(r.fy, py, r0);
                float px = __builtin_fmaf(r.fy, e1 - e0, e0);
                pa = group_sum<LPU>(pa);
                px = group_sum<LPU>(px);
                py = group_sum<LPU>(py);
                if (lig == 0) s_res[grp * row + s] = make_float4(pa, r.akx * px, r.aky * py, 0.f);
            }
        }
        __syncthreads();
        store_results(g, s_res, row, u0, upb, s0, sc, scd, grad_loc, grad_attn);
    }
}

// ---------------------------------------------------------------------------
// Fast path, grad_value by destination.
//
// Workspace views: the per-(slab, band, run) counts and offsets, the band
// lists (`cap` entries reserved per slab; an entry is the sample index
// k = q * N_p + p within its (slab, level)). Run w of a band holds that
// band's samples among k in [w * kBandChunk, (w + 1) * kBandChunk).
struct BandWs {
    int* cnt;            // [slabs][bands][nwg]
    int* off;            // [slabs][bands * nwg + 1], exclusive prefix of cnt per slab
    uint32_t* k;         // list entries: sample indices k
    const float4* rec;   // AnchorWs::rec
};

struct LevelTiles {
    int H, W, start, R, CW, nbr, nbc, nch, band0, job0, pjob0, part;
    FastDiv rd, cd;  // by R, by CW
};

// Tile geometry of level l, which is the same for the whole workgroup: read
// through pointers into the kernel arguments, as scalar loads at l's offset.
// (Indexing the arrays by value, the compiler kept every level's entries in
// scalar registers and spilled hundreds of them in the tile kernels.)
__device__ __forceinline__ LevelTiles level_tiles(const Geometry& g, const TilePlan& tp, int l)
{
    const Geometry* gp = &g;
    const TilePlan* pp = &tp;
    l = __builtin_amdgcn_readfirstlane(l);
    LevelTiles t;
    t.H = gp->lv.H[l];
    t.W = gp->lv.W[l];
    t.start = gp->lv.start[l];
    t.R = pp->rows[l];
    t.CW = pp->cols[l];
    t.nbr = pp->row_bands[l];
    t.nbc = pp->col_bands[l];
    t.nch = pp->chunks[l];
    t.band0 = pp->band_begin[l];
    t.job0 = pp->job_begin[l];
    t.pjob0 = pp->pjob_begin[l];
    t.part = pp->part_off[l];
    t.rd = pp->rows_div[l];
    t.cd = pp->cols_div[l];
    return t;
}

// Level-local bands touched by the in-level corners of the 2x2 block anchored
// at (x0, y0); returns how many (0..4).
__device__ __forceinline__ int sample_bands(const LevelTiles& t, int x0, int y0, int (&out)[4])
{
    int rb[2], cb[2], nr = 0, nc = 0;
    if (y0 >= 0 && y0 < t.H) rb[nr++] = fdiv(y0, t.rd);
    if (y0 + 1 >= 0 && y0 + 1 < t.H) {
        const int r = fdiv(y0 + 1, t.rd);
        if (nr == 0 || rb[0] != r) rb[nr++] = r;
    }
    if (x0 >= 0 && x0 < t.W) cb[nc++] = fdiv(x0, t.cd);
    if (x0 + 1 >= 0 && x0 + 1 < t.W) {
        const int c = fdiv(x0 + 1, t.cd);
        if (nc == 0 || cb[0] != c) cb[nc++] = c;
    }
    int n = 0;
    for (int i = 0; i < nr; ++i)
        for (int j = 0; j < nc; ++j) out[n++] = rb[i] * t.nbc + cb[j];
    return n;
}

__device__ __forceinline__ void unpack_anchor(uint32_t a, int& x0, int& y0)
{
    x0 = (int)(a & 0xffffu) - 2;
    y0 = (int)(a >> 16) - 2;
}

// The anchors of this thread's samples k0 + tid + i * kBandBlock of one run,
// all loads issued before any is used (0xffffffff past the run's end).
constexpr int kRunPerThread = kBandChunk / kBandBlock;
__device__ __forceinline__ void load_run_anchors(const uint32_t* __restrict__ an, int k0, int k1,
                                                 uint32_t (&a)[kRunPerThread])
{
#pragma unroll
    for (int i = 0; i < kRunPerThread; ++i) {
        const int k = k0 + (int)threadIdx.x + i * kBandBlock;
        a[i] = k < k1 ? an[k] : 0xffffffffu;
    }
}

// Bucketing 1/3: per-(slab, band, run) sample counts. Grid (run, level,
// slab); every workgroup writes the counts of all bands of its level, so the
// array needs no clearing.
__global__ __launch_bounds__(kBandBlock) void band_count_kernel(Geometry g, TilePlan tp,
                                                                const uint32_t* __restrict__ anchor,
                                                                int* __restrict__ cnt)
{
    __shared__ int hist[kMaxBandsPerLevel];
    const int wg = blockIdx.x, l = blockIdx.y, slab = blockIdx.z;
    const LevelTiles t = level_tiles(g, tp, l);
    const int nb = t.nbr * t.nbc;
    const int nsamp = g.Nq * g.Np;
    const int k0 = wg * kBandChunk, k1 = min(nsamp, k0 + kBandChunk);
    for (int i = threadIdx.x; i < nb; i += kBandBlock) hist[i] = 0;
    __syncthreads();
    uint32_t a[kRunPerThread];
    load_run_anchors(anchor + (size_t)(slab * g.Nl + l) * nsamp, k0, k1, a);
#pragma unroll
    for (int i = 0; i < kRunPerThread; ++i) {
        if (a[i] == 0xffffffffu) continue;
        int x0, y0, bands[4];
        unpack_anchor(a[i], x0, y0);
        const int n = sample_bands(t, x0, y0, bands);
        for (int j = 0; j < n; ++j) atomicAdd(&hist[bands[j]], 1);
    }
    __syncthreads();
    int* c = cnt + ((size_t)slab * tp.bands + t.band0) * tp.nwg + wg;
    for (int i = threadIdx.x; i < nb; i += kBandBlock) c[(size_t)i * tp.nwg] = hist[i];
}

// Bucketing 2/3: exclusive prefix of the (band, run) counts of each slab.
// Each thread scans kScanItems consecutive counts, so one block-wide scan of
// the threads' totals covers kBlock * kScanItems counts.
constexpr int kScanItems = 16;
__global__ __launch_bounds__(kBlock) void band_scan_kernel(TilePlan tp, const int* __restrict__ cnt,
                                                           int* __restrict__ off)
{
    __shared__ int s_wave[kBlock / kWave];
    const int slab = blockIdx.x, n = tp.bands * tp.nwg;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int* c = cnt + (size_t)slab * n;
    int* o = off + (size_t)slab * (n + 1);
    int carry = 0;
    for (int base = 0; base < n; base += kBlock * kScanItems) {
        const int i0 = base + tid * kScanItems;
        int v[kScanItems];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            v[j] = i0 + j < n ? c[i0 + j] : 0;
            sum += v[j];
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int u = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += u;
        }
        if (lane == kWave - 1) s_wave[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < kBlock / kWave; ++w) {
            before += w < wave ? s_wave[w] : 0;
            total += s_wave[w];
        }
        int run = carry + before + incl - sum;
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            if (i0 + j < n) o[i0 + j] = run;
            run += v[j];
        }
        carry += total;
        __syncthreads();
    }
    if (tid == 0) o[n] = carry;
}

// Bucketing 3/3: fill the band lists. Grid as band_count_kernel. Each
// workgroup writes its run of every band at the offset the scan gave it: an
// LDS counter per band hands out the places in the run (so the order inside
// a run is arbitrary; the tile pass orders what it sums). An entry is the
// sample index k.
// Dynamic LDS: 2 * max_bands ints.
__global__ __launch_bounds__(kBandBlock) void band_fill_kernel(Geometry g, TilePlan tp, BandWs w,
                                                               const uint32_t* __restrict__ anchor, int max_bands)
{
    extern __shared__ int dyn[];
    int* placed = dyn;               // entries of each band placed so far
    int* start = placed + max_bands;  // where this run starts in each band's list
    const int tid = threadIdx.x;
    const int wg = blockIdx.x, l = blockIdx.y, slab = blockIdx.z;
    const LevelTiles t = level_tiles(g, tp, l);
    const int nb = t.nbr * t.nbc;
    const int nsamp = g.Nq * g.Np;
    const int k0 = wg * kBandChunk, k1 = min(nsamp, k0 + kBandChunk);
    const int* run_off = w.off + (size_t)slab * (tp.bands * tp.nwg + 1) + (size_t)t.band0 * tp.nwg + wg;
    for (int i = tid; i < nb; i += kBandBlock) {
        placed[i] = 0;
        start[i] = run_off[(size_t)i * tp.nwg];
    }
    const size_t sbase = (size_t)(slab * g.Nl + l) * nsamp;
    uint32_t a[kRunPerThread];
    load_run_anchors(anchor + sbase, k0, k1, a);
    __syncthreads();
    uint32_t* list = w.k + (size_t)slab * tp.cap;
#pragma unroll
    for (int i = 0; i < kRunPerThread; ++i) {
        if (a[i] == 0xffffffffu) continue;
        const uint32_t k = (uint32_t)(k0 + tid + i * kBandBlock);
        int x0, y0, bands[4];
        unpack_anchor(a[i], x0, y0);
        const int n = sample_bands(t, x0, y0, bands);
        for (int j = 0; j < n; ++j) list[start[bands[j]] + atomicAdd(&placed[bands[j]], 1)] = k;
    }
}

// Bucketing in one kernel when every (slab, level) is a single run (N_q *
// N_p <= kBandChunk: decoder-sized query sets), in place of the three above.
// One workgroup per (level, slab): it counts the list entries of the slab's
// earlier levels (every sample once per band its corners touch) for where
// its level's lists start, counts its own samples per band, turns the counts
// into the bands' list offsets (the same exclusive prefix over the slab's
// bands that band_scan_kernel writes) and fills its lists. Grid (level,
// slab). Dynamic LDS: 2 * max_bands ints.
constexpr int kBucketItems = kMaxBandsPerLevel / kBandBlock;  // bands scanned per thread
__global__ __launch_bounds__(kBandBlock) void band_bucket_kernel(Geometry g, TilePlan tp, BandWs w,
                                                                 const uint32_t* __restrict__ anchor, int max_bands)
{
    extern __shared__ int dyn[];
    int* cnt = dyn;                 // per band of the level: its entries, then the places handed out
    int* start = cnt + max_bands;   // where each band's list starts
    __shared__ int s_wave[kBandBlock / kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int l = blockIdx.x, slab = blockIdx.y;
    const int nsamp = g.Nq * g.Np;
    int* off = w.off + (size_t)slab * (tp.bands + 1);  // one run per band
    uint32_t* list = w.k + (size_t)slab * tp.cap;
    const LevelTiles t = level_tiles(g, tp, l);
    const int nb = t.nbr * t.nbc;
    uint32_t a[kRunPerThread];
    load_run_anchors(anchor + (size_t)(slab * g.Nl + l) * nsamp, 0, nsamp, a);
    for (int i = tid; i < nb; i += kBandBlock) cnt[i] = 0;
    // entries of the earlier levels
    int earlier = 0;
    for (int le = 0; le < l; ++le) {
        const LevelTiles te = level_tiles(g, tp, le);
        uint32_t ae[kRunPerThread];
        load_run_anchors(anchor + (size_t)(slab * g.Nl + le) * nsamp, 0, nsamp, ae);
#pragma unroll
        for (int i = 0; i < kRunPerThread; ++i) {
            if (ae[i] == 0xffffffffu) continue;
            int x0, y0, bands[4];
            unpack_anchor(ae[i], x0, y0);
            earlier += sample_bands(te, x0, y0, bands);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRunPerThread; ++i) {
        if (a[i] == 0xffffffffu) continue;
        int x0, y0, bands[4];
        unpack_anchor(a[i], x0, y0);
        const int n = sample_bands(t, x0, y0, bands);
        for (int j = 0; j < n; ++j) atomicAdd(&cnt[bands[j]], 1);
    }
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) earlier += __shfl_xor(earlier, d, kWave);
    if (lane == 0) s_wave[wave] = earlier;
    __syncthreads();
    int carry = 0;
    for (int ww = 0; ww < kBandBlock / kWave; ++ww) carry += s_wave[ww];
    __syncthreads();  // s_wave is reused below
    // exclusive prefix of the level's counts, kBucketItems consecutive bands
    // per thread; the counters restart at zero for the placement
    const int i0 = tid * kBucketItems;
    int v[kBucketItems];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kBucketItems; ++j) {
        v[j] = i0 + j < nb ? cnt[i0 + j] : 0;
        sum += v[j];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += u;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int ww = 0; ww < kBandBlock / kWave; ++ww) {
        before += ww < wave ? s_wave[ww] : 0;
        total += s_wave[ww];
    }
    int run = carry + before + incl - sum;
#pragma unroll
    for (int j = 0; j < kBucketItems; ++j) {
        if (i0 + j < nb) {
            start[i0 + j] = run;
            off[t.band0 + i0 + j] = run;
            cnt[i0 + j] = 0;
        }
        run += v[j];
    }
    if (l == g.Nl - 1 && tid == 0) off[tp.bands] = carry + total;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRunPerThread; ++i) {
        if (a[i] == 0xffffffffu) continue;
        const uint32_t k = (uint32_t)(tid + i * kBandBlock);
        int x0, y0, bands[4];
        unpack_anchor(a[i], x0, y0);
        const int n = sample_bands(t, x0, y0, bands);
        for (int j = 0; j < n; ++j) list[start[bands[j]] + atomicAdd(&cnt[bands[j]], 1)] = k;
    }
}
static_assert(kMaxBandsPerLevel % kBandBlock == 0, "whole scan items per thread");

// Band of level-local index `band`: rows [r0, r0 + th), columns [c0, c0 + tw).
struct BandRect {
    int r0, c0, th, tw;
};
__device__ __forceinline__ BandRect band_rect(const LevelTiles& t, int band)
{
    const int kr = band / t.nbc, kc = band - kr * t.nbc;
    BandRect r;
    r.r0 = kr * t.R;
    r.c0 = kc * t.CW;
    r.th = min(t.H, r.r0 + t.R) - r.r0;
    r.tw = min(t.W, r.c0 + t.CW) - r.c0;
    return r;
}

// Final grad_value store of 4 channels: dst = v (+ dst when accumulating).
template <typename T>
__device__ __forceinline__ void store_grad4(T* dst, float4 a, int accumulate)
{
    float v[4] = {a.x, a.y, a.z, a.w};
    if (accumulate) {
        float o[4];
        VecIO<T, 4>::load(dst, o);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += o[i];
    }
    VecIO<T, 4>::store(dst, v);
}

// Tile kernel. LPU lanes per lane group (4 channels per lane). A job takes
// one band (or one chunk of a split band's list). Entries are staged in LDS
// a pass at a time (whole runs, at most kTileEntries entries) in (anchor
// bin, k) order. An entry anchored at (x0, y0) reaches the pixels
// (x0..x0+1, y0..y0+1). Two ways of walking the bins, chosen per level:
//  - halo mode (levels with at least as many samples as pixels): the band's
//    anchor bins (anchor rows r0-1..r1-1, columns c0-1..c1-1) are dealt out
//    to the kTileBlock / LPU groups in blocks of kRectRows x kRectCols bins; a
//    group's block reaches (kRectRows + 1) x (kRectCols + 1) pixels: its own
//    kRectRows x kRectCols and a halo row above and column to the left, which
//    belong to the neighbouring groups. Every entry's grad_output row is
//    thus loaded once and applied to all four corners; after the passes the
//    groups hand their halos to their neighbours through LDS, which add
//    them in a fixed order;
//  - pixel mode (levels with fewer samples than pixels; tile_pixel_kernel):
//    bands are as large as the bin table allows and every group owns blocks of kRectRows x
//    kPixCols pixels, one block per round, walking the (kRectRows + 1) x
//    (kPixCols + 1) bins around it and keeping only the corners that fall in
//    its block. An entry's row is loaded by every group it reaches (up to
//    four), but there is no halo exchange, and a band of one pass is staged
//    once for all its rounds, so the per-job work shrinks for sparse levels.
// Byte offset past the end of every grad_output buffer the tile kernel reads
// (buffer spans stay below 2^31 bytes): such a load returns zeros.
constexpr uint32_t kNoRowBytes = 1u << 31;

// Bins of up to this many entries in a pass are ranked by the lane that
// holds the entry; larger ones by the whole wave.
constexpr int kLaneRankKeys = 128;

// Number of keys in bkey[b0, b1) (one bin's sample indices, unique within a
// band list) smaller than key: the entry's place in its bin in k order.
// Every lane of the wave calls it (valid: the lane has an entry; bkey is
// 16-byte aligned with at least four readable slots past the last bin). A
// lane scans a bin of up to kLaneRankKeys keys itself, eight keys per two
// LDS reads. Where many samples share an anchor bin (border padding clamps
// every sample past a level's edge onto the edge pixels: edge bins then hold
// several times, and corner bins tens of times, the entries of the others)
// the lanes holding such entries set the pace of their waves, so the wave
// ranks the entries of bins beyond that size together, one after the other,
// 64 keys per step.
__device__ __forceinline__ int rank_in_bin(const uint32_t* bkey, bool valid, uint32_t key, int b0, int b1)
{
    int rank = 0;
    const bool big = valid && b1 - b0 > kLaneRankKeys;
    if (valid && !big) {
        for (int j = b0 & ~3; j < b1; j += 8) {
            const uint4 v = *reinterpret_cast<const uint4*>(bkey + j);
            const uint4 v2 = *reinterpret_cast<const uint4*>(bkey + j + 4);
            rank += (j >= b0 && v.x < key) ? 1 : 0;
            rank += (j + 1 >= b0 && j + 1 < b1 && v.y < key) ? 1 : 0;
            rank += (j + 2 >= b0 && j + 2 < b1 && v.z < key) ? 1 : 0;
            rank += (j + 3 < b1 && v.w < key) ? 1 : 0;
            rank += (j + 4 < b1 && v2.x < key) ? 1 : 0;
            rank += (j + 5 < b1 && v2.y < key) ? 1 : 0;
            rank += (j + 6 < b1 && v2.z < key) ? 1 : 0;
            rank += (j + 7 < b1 && v2.w < key) ? 1 : 0;
        }
    }
    uint64_t todo = __ballot(big);
    const int lane = (int)(threadIdx.x % kWave);
    while (todo) {
        const int src = __ffsll((unsigned long long)todo) - 1;
        todo &= todo - 1;
        const uint32_t ks = (uint32_t)__builtin_amdgcn_readlane((int)key, src);
        const int s0 = __builtin_amdgcn_readlane(b0, src), s1 = __builtin_amdgcn_readlane(b1, src);
        int r = 0;
        for (int j = s0; j < s1; j += kWave) {
            const int idx = j + lane;
            r += __popcll(__ballot(idx < s1 && bkey[min(idx, s1 - 1)] < ks));
        }
        if (lane == src) rank = r;
    }
    return rank;
}

// LDS of one tile workgroup.
struct TileLds {
    // entries in (bin, k) order: the corner weights A (1-fy)(1-fx), A (1-fy) fx,
    // A fy (1-fx), A fy fx and the element offset q * N_h * C_h of the
    // grad_output row; the three slots after a pass's last entry hold zeros
    float4 w[kTileEntries + 3];
    uint32_t row[kTileEntries + 3];
    uint32_t bkey[kTileEntries];     // sample indices k in binned order
    int bstart[kTileBins + 1];       // bin boundaries in w / row
    int cursor[kTileBins];
    int wave[kTileBlock / kWave];
};

// The pass that starts at run wr of a job: its end run wn (the pass ends
// before the first run that would overflow kTileEntries entries), its first
// list offset p0 and entry count m. Run ends never decrease, so the lanes
// test 64 runs per load instead of walking them one dependent load at a time.
__device__ __forceinline__ void find_pass(const int* run_off, int wr, int w_hi, int& wn, int& p0, int& m)
{
    p0 = run_off[wr];
    wn = wr + 1;
    while (wn < w_hi) {
        const int w = wn + (int)(threadIdx.x % kWave);
        const uint64_t fits = __ballot(w < w_hi && run_off[w + 1] - p0 <= kTileEntries);
        if (~fits == 0) {
            wn += kWave;
            continue;
        }
        wn += __ffsll((unsigned long long)~fits) - 1;
        break;
    }
    m = run_off[wn] - p0;
}

// Stage one pass (m_cnt list entries from offset p0) of a band whose anchor
// bins are rows r0-1.., columns c0-1.. (nbw bins a row, nbins in all): count
// the entries per bin, scan, place the sample indices in their bins, rank
// each entry among its bin by k (keys are unique within a band list) and
// write its corner weights and grad_output row offset to its place.
// Every thread takes part; ends with a barrier.
__device__ __forceinline__ void stage_pass(TileLds& s, const Geometry& g, const uint32_t* __restrict__ list,
                                           const float4* __restrict__ srec, int p0, int m_cnt, int r0, int c0,
                                           int nbw, int nbins, int gq)
{
    constexpr int kWaves = kTileBlock / kWave;
    const int tid = threadIdx.x;
    for (int i = tid; i < nbins; i += kTileBlock) s.cursor[i] = 0;
    __syncthreads();
    // (each thread keeps its entries' sample indices, bins and records in
    // registers until it writes them to LDS in their sorted place)
    constexpr int kStage = kTileEntries / kTileBlock;
    uint32_t kk[kStage];
    int bn[kStage];
    float rfx[kStage], rfy[kStage], ra[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
        const int i = tid + u * kTileBlock;
        kk[u] = i < m_cnt ? __builtin_nontemporal_load(list + p0 + i) : 0u;  // read once
    }
    // each entry's record (anchor corner, fractions, attention weight) as
    // the backward kernel wrote it (read about once)
    f32x4_t rc[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
        rc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (tid + u * kTileBlock < m_cnt)
            rc[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(srec + kk[u]));
    }
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
        const int i = tid + u * kTileBlock;
        if (i >= m_cnt) continue;
        int x0, y0;
        unpack_anchor(__float_as_uint(rc[u].x), x0, y0);
        rfx[u] = rc[u].y;
        rfy[u] = rc[u].z;
        ra[u] = rc[u].w;
        bn[u] = (y0 - r0 + 1) * nbw + (x0 - c0 + 1);
        atomicAdd(&s.cursor[bn[u]], 1);
    }
    __syncthreads();
    // exclusive scan of the bin counts into the bin starts and the placement
    // cursors: each thread adds up to kBinsPerThread consecutive counts, one
    // block-wide scan of those sums
    {
        constexpr int kBinsPerThread = (kTileBins + kTileBlock - 1) / kTileBlock;
        const int per = (nbins + kTileBlock - 1) / kTileBlock;
        const int i0 = tid * per;
        int v[kBinsPerThread];
        int sum = 0;
#pragma unroll
        for (int j = 0; j < kBinsPerThread; ++j) {
            v[j] = j < per && i0 + j < nbins ? s.cursor[i0 + j] : 0;
            sum += v[j];
        }
        const int lane = tid % kWave, wave = tid / kWave;
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int u = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += u;
        }
        if (lane == kWave - 1) s.wave[wave] = incl;
        __syncthreads();
        int run = incl - sum;
        for (int ww = 0; ww < wave; ++ww) run += s.wave[ww];
#pragma unroll
        for (int j = 0; j < kBinsPerThread; ++j) {
            if (j < per && i0 + j < nbins) {
                s.bstart[i0 + j] = run;
                s.cursor[i0 + j] = run;
            }
            run += v[j];
        }
        if (tid == kTileBlock - 1) {
            int tot = 0;
            for (int ww = 0; ww < kWaves; ++ww) tot += s.wave[ww];
            s.bstart[nbins] = tot;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kStage; ++u)
        if (tid + u * kTileBlock < m_cnt) s.bkey[atomicAdd(&s.cursor[bn[u]], 1)] = kk[u];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
        const int i = tid + u * kTileBlock;
        if (i >= m_cnt) continue;
        const uint32_t key = kk[u];
        const int b0 = s.bstart[bn[u]], b1 = s.bstart[bn[u] + 1];
        // (pixel-mode levels hold fewer samples than pixels, so their bins
        // stay small and a plain scan is the cheapest rank; rank_in_bin's
        // aligned layout measured 2% slower here)
        int rank = 0;
        for (int j = b0; j < b1; ++j) rank += s.bkey[j] < key ? 1 : 0;
        const int q = fdiv((int)key, g.np_div);
        const float fx = rfx[u], fy = rfy[u], A = ra[u];
        const float a0 = A * (1.f - fy), a1 = A * fy;
        s.w[b0 + rank] = make_float4(a0 * (1.f - fx), a0 * fx, a1 * (1.f - fx), a1 * fx);
        s.row[b0 + rank] = (uint32_t)(q * gq);
    }
    if (tid < 3) {
        s.w[m_cnt + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
        s.row[m_cnt + tid] = 0u;
    }
    __syncthreads();
}

// Pixel mode: terms of four entries of window bin (bi, bj) for a lane
// group's block of WR x WC pixels; the bin is anchored at block pixel
// (bi - 1, bj - 1), so corner (dx, dy) of an entry lands on block pixel
// (bi - 1 + dy, bj - 1 + dx), and corners outside the block are dropped. The
// four entries' terms are summed before they join the pixel's total, which
// keeps float32 rounding chains short.
template <int WR, int WC>
__device__ __forceinline__ void add_bin_terms(float4 (&acc)[WR][WC], int bi, int bj, const float4 (&wv)[4],
                                              const float (&gv)[4][4])
{
#pragma unroll
    for (int dy = 0; dy < 2; ++dy) {
        const int pr = bi - 1 + dy;
        if (pr < 0 || pr >= WR) continue;
#pragma unroll
        for (int dx = 0; dx < 2; ++dx) {
            const int pc = bj - 1 + dx;
            if (pc < 0 || pc >= WC) continue;
            float4 ts;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 w4 = wv[u];
                const float wc = dy ? (dx ? w4.w : w4.z) : (dx ? w4.y : w4.x);
                if (u == 0) {
                    ts = make_float4(wc * gv[u][0], wc * gv[u][1], wc * gv[u][2], wc * gv[u][3]);
                } else {
                    ts.x = __builtin_fmaf(wc, gv[u][0], ts.x);
                    ts.y = __builtin_fmaf(wc, gv[u][1], ts.y);
                    ts.z = __builtin_fmaf(wc, gv[u][2], ts.z);
                    ts.w = __builtin_fmaf(wc, gv[u][3], ts.w);
                }
            }
            acc[pr][pc].x += ts.x;
            acc[pr][pc].y += ts.y;
            acc[pr][pc].z += ts.z;
            acc[pr][pc].w += ts.w;
        }
    }
}

// Pixel mode: walk the (WR + 1) x (WC + 1) bins around the block whose first
// pixel is (py0, px0) (bins past the band's th x tw pixels are empty), four
// entries at a time: their grad_output rows are loaded (slots past a bin's
// end load no row: the buffer returns zeros past its end, so whatever weights
// they read add nothing) and their terms added to the block.
template <typename T, int WR, int WC>
__device__ __forceinline__ void walk_bins(const TileLds& s, __amdgpu_buffer_rsrc_t gr, int ch, int py0, int px0,
                                          int th, int tw, int nbw, float4 (&acc)[WR][WC])
{
#pragma unroll
    for (int bi = 0; bi <= WR; ++bi) {
#pragma unroll
        for (int bj = 0; bj <= WC; ++bj) {
            const int by = py0 + bi, bx = px0 + bj;
            int e0 = 0, e1 = 0;
            if (by <= th && bx <= tw) {
                e0 = s.bstart[by * nbw + bx];
                e1 = s.bstart[by * nbw + bx + 1];
            }
            for (int e = e0; e < e1; e += 4) {
                float4 wv[4];
                float gv[4][4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    wv[u] = s.w[e + u];
                    const uint32_t row = s.row[e + u];
                    BufIO<T, 4>::load(gr, e + u < e1 ? (row + ch) * (uint32_t)sizeof(T) : kNoRowBytes, gv[u]);
                }
                add_bin_terms<WR, WC>(acc, bi, bj, wv, gv);
            }
        }
    }
}

// Halo-mode tile kernel. It keeps its own copy of the staging (the same
// results as stage_pass; its bin scan goes 512 bins at a time): built from
// that function it took 1-2% longer (more scalar registers spilled).
template <typename T, int LPU>
__global__ __launch_bounds__(kTileBlock) __attribute__((amdgpu_waves_per_eu(4))) void tile_scatter_kernel(
    Geometry g, TilePlan tp, BandWs w, const T* __restrict__ grad_out, T* __restrict__ grad_value,
    float* __restrict__ partial, int accumulate)
{
    constexpr int RH = kRectRows, RW = kRectCols;
    constexpr int E = kTileEntries;
    constexpr int kWaves = kTileBlock / kWave;
    // entries in (bin, k) order: the corner weights A (1-fy)(1-fx), A (1-fy) fx,
    // A fy (1-fx), A fy fx and the element offset q * N_h * C_h of the
    // grad_output row; the three slots after a pass's last entry hold zeros
    __shared__ float4 s_w[E + 3];
    __shared__ uint32_t s_row[E + 3];
    __shared__ __align__(16) uint32_t s_bkey[E + 4];  // sample indices k in binned order (+ read slack)
    __shared__ int s_bstart[kTileBins + 1];  // bin boundaries in s_w / s_row
    __shared__ int s_cursor[kTileBins];
    __shared__ int s_wave[kWaves];

    const int tid = threadIdx.x;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int slab = lb / tp.jobs;
    // jobs run in reverse plan order: the coarse levels' jobs (dense bands,
    // several passes each) start first, so the kernel does not end waiting
    // on one of them
    const int job = tp.jobs - 1 - (lb - slab * tp.jobs);
    const int b = slab / g.Nh, h = slab - b * g.Nh;

    int l = 0;
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k)
        if (job >= tp.job_begin[k] && job < tp.job_begin[k + 1]) l = k;
    const LevelTiles t = level_tiles(g, tp, l);
    const int local = job - t.job0;
    const int band = local / t.nch, chunk = local - band * t.nch;
    const BandRect br = band_rect(t, band);
    const int r0 = br.r0, c0 = br.c0, tw = br.tw, th = br.th;
    const int nbw = tw + 1;                  // anchor bins cover rows r0-1..r1-1, cols c0-1..c1-1
    const int nbins = (th + 1) * nbw;
    // this chunk's runs [w_lo, w_hi) of the band's list; run_off[w] is where run w starts
    const int* run_off = w.off + (size_t)slab * (tp.bands * tp.nwg + 1) + (size_t)(t.band0 + band) * tp.nwg;
    const int w_lo = (int)((int64_t)tp.nwg * chunk / t.nch), w_hi = (int)((int64_t)tp.nwg * (chunk + 1) / t.nch);
    const size_t lbase = (size_t)slab * tp.cap;
    const float4* srec = w.rec + (size_t)(slab * g.Nl + l) * (g.Nq * g.Np);  // records of this (slab, level)
    const T* grow0 = grad_out + (b * g.Nq * g.Nh + h) * g.Ch;  // + q * N_h * C_h
    const int gq = g.Nh * g.Ch;
    // rows of this slab: q * gq elements past grow0, as byte offsets of a buffer over the slab's span
    const __amdgpu_buffer_rsrc_t gr = value_rsrc(grow0, (int64_t)g.Nq * gq * (int64_t)sizeof(T));

    const int grp = tid / LPU, lig = tid % LPU;
    const int ch = lig * 4;
    const int gnx = (tw + RW) / RW, gny = (th + RH) / RH;  // group blocks cover the (th+1) x (tw+1) bins
    const int gy = grp / gnx, gx = grp - gy * gnx;
    const int by0 = gy * RH, bx0 = gx * RW;  // the group's first bin (bin row 0 is anchor row r0 - 1)
    const bool grp_ok = ch < g.Ch && gy < gny;

    // acc[a][c] is band-local pixel (by0 - 1 + a, bx0 - 1 + c): rows and
    // columns 1.. are the group's own, row 0 and column 0 its halo
    float4 acc[RH + 1][RW + 1];
#pragma unroll
    for (int i = 0; i <= RH; ++i)
#pragma unroll
        for (int j = 0; j <= RW; ++j) acc[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);

    // A pass stages whole runs (at most E entries; one run never exceeds
    // kBandChunk <= E), so which entries share a pass does not depend on the
    // order inside runs; inside a pass every bin is summed in k order. The
    // sums are therefore the same on every call.
    for (int wr = w_lo; wr < w_hi;) {
        const int p0 = run_off[wr];
        // the pass ends before the first run that would overflow E entries;
        // run ends never decrease, so the lanes test 64 runs per load instead
        // of walking them one dependent load at a time
        int wn = wr + 1;
        while (wn < w_hi) {
            const int w = wn + tid % kWave;
            const uint64_t fits = __ballot(w < w_hi && run_off[w + 1] - p0 <= E);
            if (~fits == 0) {
                wn += kWave;
                continue;
            }
            wn += __ffsll((unsigned long long)~fits) - 1;
            break;
        }
        const int m_cnt = run_off[wn] - p0;
        wr = wn;
        // stage a pass of list entries and count them per anchor bin; the
        // entries' loads are issued before the bin counts are cleared, so
        // their latency covers the clearing and its barrier
        // (each thread keeps its entries' sample indices, bins and records in
        // registers until it writes them to LDS in their sorted place)
        constexpr int kStage = kTileEntries / kTileBlock;
        uint32_t kk[kStage];
        int bn[kStage];
        float rfx[kStage], rfy[kStage], ra[kStage];
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            const int i = tid + u * kTileBlock;
            kk[u] = i < m_cnt ? __builtin_nontemporal_load(w.k + lbase + p0 + i) : 0u;  // read once
        }
        // each entry's record (anchor corner, fractions, attention weight) as
        // the backward kernel wrote it (read about once)
        f32x4_t rc[kStage];
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            rc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (tid + u * kTileBlock < m_cnt)
                rc[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(srec + kk[u]));
        }
        for (int i = tid; i < nbins; i += kTileBlock) s_cursor[i] = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            const int i = tid + u * kTileBlock;
            if (i >= m_cnt) continue;
            int x0, y0;
            unpack_anchor(__float_as_uint(rc[u].x), x0, y0);
            rfx[u] = rc[u].y;
            rfy[u] = rc[u].z;
            ra[u] = rc[u].w;
            bn[u] = (y0 - r0 + 1) * nbw + (x0 - c0 + 1);
            atomicAdd(&s_cursor[bn[u]], 1);
        }
        __syncthreads();
        // exclusive scan of the bin counts into the bin starts and the
        // placement cursors
        for (int base = 0; base < nbins; base += kTileBlock) {
            const int i = base + tid;
            const int v = i < nbins ? s_cursor[i] : 0;
            int incl = v;
            const int lane = tid % kWave, wave = tid / kWave;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int u = __shfl_up(incl, d, kWave);
                if (lane >= d) incl += u;
            }
            if (lane == kWave - 1) s_wave[wave] = incl;
            __syncthreads();
            int before = base == 0 ? 0 : s_bstart[base];
            for (int ww = 0; ww < wave; ++ww) before += s_wave[ww];
            if (i < nbins) {
                s_bstart[i] = before + incl - v;
                s_cursor[i] = before + incl - v;  // (only this thread read s_cursor[i])
            }
            if (tid == kTileBlock - 1) {
                int tot = base == 0 ? 0 : s_bstart[base];
                for (int ww = 0; ww < kWaves; ++ww) tot += s_wave[ww];
                s_bstart[min(base + kTileBlock, nbins)] = tot;
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < kStage; ++u)
            if (tid + u * kTileBlock < m_cnt) s_bkey[atomicAdd(&s_cursor[bn[u]], 1)] = kk[u];
        __syncthreads();
        // rank every entry among its bin by k (keys are unique within a band
        // list) and write it to its place in (bin, k) order
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            const bool valid = tid + u * kTileBlock < m_cnt;
            const uint32_t key = kk[u];
            const int bin = valid ? bn[u] : 0;
            const int b0 = s_bstart[bin], b1 = s_bstart[bin + 1];
            const int rank = rank_in_bin(s_bkey, valid, key, b0, b1);
            if (!valid) continue;
            const int q = fdiv((int)key, g.np_div);
            const float fx = rfx[u], fy = rfy[u], A = ra[u];
            const float a0 = A * (1.f - fy), a1 = A * fy;
            s_w[b0 + rank] = make_float4(a0 * (1.f - fx), a0 * fx, a1 * (1.f - fx), a1 * fx);
            s_row[b0 + rank] = (uint32_t)(q * gq);
        }
        if (tid < 3) {
            s_w[m_cnt + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
            s_row[m_cnt + tid] = 0u;
        }
        __syncthreads();
        // every group walks its block of bins
        if (grp_ok) {
            // terms of four entries of the group's bin (bi, bj): corner (dx, dy)
            // of such an entry is acc[bi + dy][bj + dx]; the four terms are
            // summed before they join the pixel's total, which keeps float32
            // rounding chains short
            auto add_terms = [&](int bi, int bj, const float4 (&wv)[4], const float (&gv)[4][4]) {
#pragma unroll
                for (int dy = 0; dy < 2; ++dy) {
                    const int pr = bi + dy;
#pragma unroll
                    for (int dx = 0; dx < 2; ++dx) {
                        const int pc = bj + dx;
                        float4 ts;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float4 w4 = wv[u];
                            const float wc = dy ? (dx ? w4.w : w4.z) : (dx ? w4.y : w4.x);
                            if (u == 0) {
                                ts = make_float4(wc * gv[u][0], wc * gv[u][1], wc * gv[u][2], wc * gv[u][3]);
                            } else {
                                ts.x = __builtin_fmaf(wc, gv[u][0], ts.x);
                                ts.y = __builtin_fmaf(wc, gv[u][1], ts.y);
                                ts.z = __builtin_fmaf(wc, gv[u][2], ts.z);
                                ts.w = __builtin_fmaf(wc, gv[u][3], ts.w);
                            }
                        }
                        acc[pr][pc].x += ts.x;
                        acc[pr][pc].y += ts.y;
                        acc[pr][pc].z += ts.z;
                        acc[pr][pc].w += ts.w;
                    }
                }
            };
            // entry range [b0, b1) of the group's bin (bi, bj); empty where there is no such bin
            auto bin_range = [&](int bi, int bj, int& b0, int& b1) {
                const int by = by0 + bi, bx = bx0 + bj;
                b0 = b1 = 0;
                if (by > th || bx > tw) return;
                const int bin = by * nbw + bx;
                b0 = s_bstart[bin];
                b1 = s_bstart[bin + 1];
            };
#pragma unroll
            for (int bi = 0; bi < RH; ++bi) {
#pragma unroll
                for (int bj = 0; bj < RW; ++bj) {
                    int e0, e1;
                    bin_range(bi, bj, e0, e1);
                    for (int e = e0; e < e1; e += 4) {
                        float4 wv[4];
                        float gv[4][4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            // slots past the bin's end load no row (the buffer
                            // returns zeros past its end), so whatever
                            // weights they read add nothing
                            wv[u] = s_w[e + u];
                            const uint32_t row = s_row[e + u];
                            BufIO<T, 4>::load(gr, e + u < e1 ? (row + ch) * (uint32_t)sizeof(T) : kNoRowBytes, gv[u]);
                        }
                        add_terms(bi, bj, wv, gv);
                    }
                }
            }
        }
        __syncthreads();
    }

    // halo exchange through LDS (s_w is free now): the halo row goes to the
    // group above, the halo column to the group on the left and the corner to
    // the group above-left; a pixel adds its own sum, then the values from
    // below, from the right and from below-right, in that order
    // (a job without entries has nothing to trade)
    static_assert(RW * kTileBlock <= E + 3 && (RH + 1) * kTileBlock <= E + 3, "halo exchange fits s_w");
    float4* s_x = s_w;
    if (run_off[w_hi] > run_off[w_lo]) {
        if (grp_ok) {
#pragma unroll
            for (int c = 1; c <= RW; ++c) s_x[(c - 1) * kTileBlock + tid] = acc[0][c];
        }
        __syncthreads();
        if (grp_ok && gy + 1 < gny) {
#pragma unroll
            for (int c = 1; c <= RW; ++c) {
                const float4 v = s_x[(c - 1) * kTileBlock + tid + gnx * LPU];
                acc[RH][c].x += v.x;
                acc[RH][c].y += v.y;
                acc[RH][c].z += v.z;
                acc[RH][c].w += v.w;
            }
        }
        __syncthreads();
        if (grp_ok) {
#pragma unroll
            for (int r = 1; r <= RH; ++r) s_x[(r - 1) * kTileBlock + tid] = acc[r][0];
            s_x[RH * kTileBlock + tid] = acc[0][0];
        }
        __syncthreads();
        if (grp_ok && gx + 1 < gnx) {
#pragma unroll
            for (int r = 1; r <= RH; ++r) {
                const float4 v = s_x[(r - 1) * kTileBlock + tid + LPU];
                acc[r][RW].x += v.x;
                acc[r][RW].y += v.y;
                acc[r][RW].z += v.z;
                acc[r][RW].w += v.w;
            }
            if (gy + 1 < gny) {
                const float4 v = s_x[RH * kTileBlock + tid + (gnx + 1) * LPU];
                acc[RH][RW].x += v.x;
                acc[RH][RW].y += v.y;
                acc[RH][RW].z += v.z;
                acc[RH][RW].w += v.w;
            }
        }
    }
    if (!grp_ok) return;

    // own pixels: band-local (by0 - 1 + i, bx0 - 1 + j) for i, j >= 1
    if (t.nch == 1) {
        // the band's only job: store the final values
        const int pstride = g.bnlc ? g.Ch : g.Nh * g.Ch;
        T* out = grad_value + value_slab_offset(g, b, h) + t.start * pstride;
#pragma unroll
        for (int i = 1; i <= RH; ++i)
#pragma unroll
            for (int j = 1; j <= RW; ++j) {
                const int py = by0 - 1 + i, px = bx0 - 1 + j;
                if (py < th && px < tw)
                    store_grad4(out + ((r0 + py) * t.W + c0 + px) * pstride + ch, acc[i][j], accumulate);
            }
        return;
    }
    // one chunk of a split band: its partial tile, pixel-major (band-local
    // row-major pixel index), C_h floats per pixel (stored non-temporal too:
    // the reduction reads it back once, and in L2 it would only displace the
    // rows the other tile jobs re-read)
    float* slot = partial + (size_t)slab * tp.part_per_slab + t.part +
                  (size_t)(band * t.nch + chunk) * (t.R * t.CW) * g.Ch;
#pragma unroll
    for (int i = 1; i <= RH; ++i)
#pragma unroll
        for (int j = 1; j <= RW; ++j) {
            const int py = by0 - 1 + i, px = bx0 - 1 + j;
            if (py < th && px < tw)
                nt_store4(slot + (py * tw + px) * g.Ch + ch, acc[i][j].x, acc[i][j].y, acc[i][j].z, acc[i][j].w);
        }
}

// Pixel-mode tile kernel (levels with fewer samples than pixels): one
// workgroup per band; the lane groups take the band's kRectRows x kPixCols
// pixel blocks in rounds, each walking the bins around its block.
template <typename T, int LPU>
__global__ __launch_bounds__(kTileBlock) __attribute__((amdgpu_waves_per_eu(4))) void tile_pixel_kernel(
    Geometry g, TilePlan tp, BandWs w, const T* __restrict__ grad_out, T* __restrict__ grad_value, int accumulate)
{
    constexpr int RH = kRectRows;
    __shared__ TileLds s;

    const int tid = threadIdx.x;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int slab = lb / tp.pjobs;
    const int job = tp.pjobs - 1 - (lb - slab * tp.pjobs);  // coarser levels first, as in halo mode
    const int b = slab / g.Nh, h = slab - b * g.Nh;

    int l = 0;
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k)
        if (job >= tp.pjob_begin[k] && job < tp.pjob_begin[k + 1]) l = k;
    const LevelTiles t = level_tiles(g, tp, l);
    const int band = job - t.pjob0;  // pixel-mode bands are not split
    const BandRect br = band_rect(t, band);
    const int r0 = br.r0, c0 = br.c0, tw = br.tw, th = br.th;
    const int nbw = tw + 1;  // anchor bins cover rows r0-1..r1-1, cols c0-1..c1-1
    const int nbins = (th + 1) * nbw;
    // the band's runs [0, nwg); run_off[w] is where run w starts
    const int* run_off = w.off + (size_t)slab * (tp.bands * tp.nwg + 1) + (size_t)(t.band0 + band) * tp.nwg;
    const int w_lo = 0, w_hi = tp.nwg;
    const uint32_t* list = w.k + (size_t)slab * tp.cap;
    const float4* srec = w.rec + (size_t)(slab * g.Nl + l) * (g.Nq * g.Np);  // records of this (slab, level)
    const T* grow0 = grad_out + (b * g.Nq * g.Nh + h) * g.Ch;  // + q * N_h * C_h
    const int gq = g.Nh * g.Ch;
    const __amdgpu_buffer_rsrc_t gr = value_rsrc(grow0, (int64_t)g.Nq * gq * (int64_t)sizeof(T));
    const int pstride = g.bnlc ? g.Ch : g.Nh * g.Ch;
    T* out = grad_value + value_slab_offset(g, b, h) + t.start * pstride;  // + pixel * pstride
    const int grp = tid / LPU, lig = tid % LPU;
    const int ch = lig * 4;

    constexpr int PC = kPixCols;
    constexpr int kGroups = kTileBlock / LPU;
    const int pbw = (tw + PC - 1) / PC, nblk = ((th + RH - 1) / RH) * pbw;
    int wn, p0, m_cnt;
    find_pass(run_off, w_lo, w_hi, wn, p0, m_cnt);
    const bool single = wn >= w_hi;  // one pass: staged once for every round
    if (single) stage_pass(s, g, list, srec, p0, m_cnt, r0, c0, nbw, nbins, gq);
    for (int rb = 0; rb < nblk; rb += kGroups) {
        const int blk = rb + grp;
        const bool own = blk < nblk && ch < g.Ch;
        const int pby = own ? blk / pbw : 0, pbx = own ? blk - (blk / pbw) * pbw : 0;
        const int py0 = pby * RH, px0 = pbx * PC;  // the block's first pixel, band-local
        float4 acc[RH][PC];
#pragma unroll
        for (int i = 0; i < RH; ++i)
#pragma unroll
            for (int j = 0; j < PC; ++j) acc[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int wr = w_lo; wr < w_hi;) {
            if (!single) {
                find_pass(run_off, wr, w_hi, wn, p0, m_cnt);
                stage_pass(s, g, list, srec, p0, m_cnt, r0, c0, nbw, nbins, gq);
            }
            // bins py0..py0+RH, px0..px0+PC reach the block (bin (by, bx)
            // is anchored at band-local pixel (by - 1, bx - 1))
            if (own) walk_bins<T, RH, PC>(s, gr, ch, py0, px0, th, tw, nbw, acc);
            if (!single) __syncthreads();  // the next pass is staged over this one
            wr = wn;
        }
        if (own) {
#pragma unroll
            for (int i = 0; i < RH; ++i)
#pragma unroll
                for (int j = 0; j < PC; ++j) {
                    const int py = py0 + i, px = px0 + j;
                    if (py < th && px < tw)
                        store_grad4(out + ((r0 + py) * t.W + c0 + px) * pstride + ch, acc[i][j], accumulate);
                }
        }
    }
}

// Adds the partial tiles of split bands in chunk order and stores grad_value.
// Grid: (reduction piece, slab); a piece is up to kReduceF4 float4s of one band.
template <typename T>
__global__ __launch_bounds__(kBlock) void band_reduce_kernel(Geometry g, TilePlan tp,
                                                             const float* __restrict__ partial,
                                                             T* __restrict__ grad_value, int accumulate)
{
    const int piece = blockIdx.x, slab = blockIdx.y;
    const int b = slab / g.Nh, h = slab - b * g.Nh;
    int l = 0;
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k)
        if (piece >= tp.rpiece_begin[k] && piece < tp.rpiece_begin[k + 1]) l = k;
    const LevelTiles t = level_tiles(g, tp, l);
    int ppb = 1;
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k)
        if (k == l) ppb = tp.rpieces_per_band[k];
    const int local = piece - tp.rpiece_begin[l];
    const int band = local / ppb, sub = local - band * ppb;
    const BandRect br = band_rect(t, band);
    const int n4 = br.th * br.tw * g.Ch / 4;
    const int i0 = sub * kReduceF4, i1 = min(n4, i0 + kReduceF4);
    const size_t tile = (size_t)t.R * t.CW * g.Ch;
    const float* slot0 = partial + (size_t)slab * tp.part_per_slab + t.part + (size_t)band * t.nch * tile;
    const int pstride = g.bnlc ? g.Ch : g.Nh * g.Ch;
    T* out = grad_value + value_slab_offset(g, b, h) + t.start * pstride;
    for (int i = i0 + (int)threadIdx.x; i < i1; i += kBlock) {
        const float4* part = reinterpret_cast<const float4*>(slot0) + i;
        const size_t step = tile / 4;  // float4s between consecutive chunks' tiles
        float4 s = part[0];
        int c = 1;
        // eight chunks' loads in flight at a time; the sum still runs in chunk order
        for (; c + 8 <= t.nch; c += 8) {
            float4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = part[(size_t)(c + j) * step];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                s.x += v[j].x;
                s.y += v[j].y;
                s.z += v[j].z;
                s.w += v[j].w;
            }
        }
        for (; c < t.nch; ++c) {
            const float4 v = part[(size_t)c * step];
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        const int e = 4 * i;
        const int p = e / g.Ch, ch = e - p * g.Ch;
        const int py = p / br.tw, px = p - py * br.tw;
        store_grad4(out + ((br.r0 + py) * t.W + br.c0 + px) * pstride + ch, s, accumulate);
    }
}

// ---------------------------------------------------------------------------
// Generic path: any C_h, any alignment. One channel per lane (LPU lanes per
// unit, channels beyond LPU in a loop); grad_value via float atomics into
// `gacc` (grad_value itself for float32, a float32 workspace for bfloat16).
template <typename T, int LPU>
__global__ __launch_bounds__(kBlock) void backward_generic_kernel(Geometry g, int sc_max, ChunkDiv cdiv,
                                                                  const T* __restrict__ grad_out,
                                                                  const T* __restrict__ value,
                                                                  const float* __restrict__ loc,
                                                                  const float* __restrict__ attn,
                                                                  float* __restrict__ gacc,
                                                                  float* __restrict__ grad_loc,
                                                                  float* __restrict__ grad_attn)
{
    constexpr int upb = kBlock / LPU;
    extern __shared__ float4 smem[];
    const int row = sc_max + 1;
    BwdRecord* s_rec = reinterpret_cast<BwdRecord*>(smem);
    float4* s_res = smem + 2 * upb * row;
    __shared__ int4 s_lv[kMaxLevels];
    fill_level_table(g.lv, s_lv);

    const int tid = threadIdx.x;
    const int u0 = xcd_logical_block(blockIdx.x, gridDim.x) * upb;
    const bool want_dots = grad_loc != nullptr || grad_attn != nullptr;

    const int grp = tid / LPU, lig = tid % LPU;
    const int u = u0 + grp;
    const bool unit_ok = u < g.units;
    const UnitIdx ui = unit_index(g, unit_ok ? u : 0);
    const int pstride = g.bnlc ? g.Ch : g.Nh * g.Ch;
    const int slab_off = value_slab_offset(g, ui.b, ui.h);
    const T* vslab = value + slab_off;
    float* gslab = gacc ? gacc + slab_off : nullptr;
    const T* grow = grad_out + ((ui.b * g.Nq + ui.q) * g.Nh + ui.h) * g.Ch;

    for (int s0 = 0; s0 < g.S; s0 += sc_max) {
        const int sc = min(sc_max, g.S - s0);
        if (s0 > 0) __syncthreads();
        const FastDiv& scd = cdiv.of(sc, sc_max);
        stage_records(g, loc, attn, s_rec, row, u0, upb, s0, sc, scd, s_lv);
        __syncthreads();
        if (unit_ok) {
            for (int s = 0; s < sc; ++s) {
                const BwdRecord r = s_rec[grp * row + s];
                const float gxw = 1.f - r.fx, gyw = 1.f - r.fy;
                const float w00 = gxw * gyw, w01 = r.fx * gyw, w10 = gxw * r.fy, w11 = r.fx * r.fy;
                const int o00 = r.off;
                const int o01 = o00 + pstride;
                const int o10 = o00 + r.rowp;
                const int o11 = o10 + pstride;
                float pa = 0.f, px = 0.f, py = 0.f;
                for (int c = lig; c < g.Ch; c += LPU) {
                    const float Gc = load_f32(grow + c);
                    if (want_dots) {
                        const float v00 = (r.mask & 1) ? load_f32(vslab + o00 + c) : 0.f;
                        const float v01 = (r.mask & 2) ? load_f32(vslab + o01 + c) : 0.f;
                        const float v10 = (r.mask & 4) ? load_f32(vslab + o10 + c) : 0.f;
                        const float v11 = (r.mask & 8) ? load_f32(vslab + o11 + c) : 0.f;
                        const float smp = w00 * v00 + w01 * v01 + w10 * v10 + w11 * v11;
                        const float dx = gyw * (v01 - v00) + r.fy * (v11 - v10);
                        const float dy = gxw * (v10 - v00) + r.fx * (v11 - v01);
                        pa = __builtin_fmaf(Gc, smp, pa);
                        px = __builtin_fmaf(Gc, dx, px);
                        py = __builtin_fmaf(Gc, dy, py);
                    }
                    if (gslab) {
                        const float ag = r.a * Gc;
                        if (r.mask & 1) unsafeAtomicAdd(gslab + o00 + c, ag * w00);
                        if (r.mask & 2) unsafeAtomicAdd(gslab + o01 + c, ag * w01);
                        if (r.mask & 4) unsafeAtomicAdd(gslab + o10 + c, ag * w10);
                        if (r.mask & 8) unsafeAtomicAdd(gslab + o11 + c, ag * w11);
                    }
                }
                if (want_dots) {
                    pa = group_sum<LPU>(pa);
                    px = group_sum<LPU>(px);
                    py = group_sum<LPU>(py);
                    if (lig == 0) s_res[grp * row + s] = make_float4(pa, r.a * px * r.kx, r.a * py * r.ky, 0.f);
                }
            }
        }
        if (!want_dots) continue;
        __syncthreads();
        store_results(g, s_res, row, u0, upb, s0, sc, scd, grad_loc, grad_attn);
    }
}

// ---------------------------------------------------------------------------
// host launchers

static unsigned grid_for(int64_t n)
{
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + kBlock - 1) / kBlock, 8192));
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t n4 = ((uintptr_t)p % 16 == 0) ? n / 4 : 0;
    const int64_t rest = n - 4 * n4;
    if (n4 > 0)
        hipLaunchKernelGGL(zero4_kernel, dim3(grid_for(n4)), dim3(kBlock), 0, stream, reinterpret_cast<float4*>(p), n4);
    if (rest > 0) hipLaunchKernelGGL(zero1_kernel, dim3(grid_for(rest)), dim3(kBlock), 0, stream, p + 4 * n4, rest);
    return hipGetLastError();
}

// Clear n elements of grad_value in its storage type (4 or 2 bytes).
hipError_t launch_zero_elems(void* p, int64_t n, int elem, hipStream_t stream)
{
    if (elem == 4) return launch_zero(static_cast<float*>(p), n, stream);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_u16_kernel, dim3(grid_for(n)), dim3(kBlock), 0, stream, static_cast<uint16_t*>(p), n);
    return hipGetLastError();
}

static int samples_per_chunk(int S, int upb)
{
    const size_t per = sizeof(BwdRecord) + sizeof(float4);  // staged record + result slot
    int sc = S < 16 ? S : 16;
    while (sc > 1 && (size_t)upb * (sc + 1) * per > kLdsBudget) --sc;
    return sc;
}

template <typename T, int LPU, int VEC>
static hipError_t launch_fast_t(const Geometry& g, const void* grad_out, const void* value, const float* loc,
                                const float* attn, float* grad_loc, float* grad_attn, AnchorWs ws,
                                hipStream_t stream)
{
    constexpr int upb = kBlock / LPU;
    const int sc = samples_per_chunk(g.S, upb);
    const size_t lds = (size_t)upb * (sc + 1) * (sizeof(BwdFastRecord) + sizeof(float4));
    const int64_t value_bytes = (int64_t)g.B * g.L * g.Nh * g.Ch * (int64_t)sizeof(T);
    const ChunkDiv cdiv = make_chunkdiv(g.S, sc);
    if (buffer_loads_ok(value_bytes))
        hipLaunchKernelGGL((backward_fast_kernel<T, LPU, true, VEC>), dim3(g.blocks), dim3(kBlock), lds, stream, g, sc,
                           cdiv, value_bytes, static_cast<const T*>(grad_out), static_cast<const T*>(value), loc,
                           attn, grad_loc, grad_attn, ws);
    else
        hipLaunchKernelGGL((backward_fast_kernel<T, LPU, false, VEC>), dim3(g.blocks), dim3(kBlock), lds, stream, g, sc,
                           cdiv, value_bytes, static_cast<const T*>(grad_out), static_cast<const T*>(value), loc,
                           attn, grad_loc, grad_attn, ws);
    return hipGetLastError();
}

template <typename T, int LPU>
static void launch_tile_kernel(const Geometry& g, const TilePlan& tp, BandWs w, const void* grad_out,
                               void* grad_value, float* partial, int accumulate, hipStream_t stream)
{
    // the host sends this path only problems whose grad_output rows of one
    // batch span fewer than 2^31 - 2^20 bytes (tile_rows_fit), so the walk's
    // buffer loads reach every row
    const int64_t blocks = (int64_t)tp.jobs * g.B * g.Nh;
    if (blocks > 0)
        hipLaunchKernelGGL((tile_scatter_kernel<T, LPU>), dim3((unsigned)blocks), dim3(kTileBlock), 0, stream,
                           g, tp, w, static_cast<const T*>(grad_out), static_cast<T*>(grad_value), partial,
                           accumulate);
    const int64_t pblocks = (int64_t)tp.pjobs * g.B * g.Nh;
    if (pblocks > 0)
        hipLaunchKernelGGL((tile_pixel_kernel<T, LPU>), dim3((unsigned)pblocks), dim3(kTileBlock), 0, stream, g, tp,
                           w, static_cast<const T*>(grad_out), static_cast<T*>(grad_value), accumulate);
}

template <typename T, int LPU>
static hipError_t launch_tiles_t(const Geometry& g, const TilePlan& tp, BandWs w, const void* grad_out,
                                 void* grad_value, float* partial, int accumulate, hipStream_t stream)
{
    launch_tile_kernel<T, LPU>(g, tp, w, grad_out, grad_value, partial, accumulate, stream);
    if (tp.rpieces > 0)
        hipLaunchKernelGGL((band_reduce_kernel<T>), dim3((unsigned)tp.rpieces, (unsigned)(g.B * g.Nh)), dim3(kBlock),
                           0, stream, g, tp, partial, static_cast<T*>(grad_value), accumulate);
    return hipGetLastError();
}

template <typename T, int LPU>
static hipError_t launch_generic_t(const Geometry& g, const void* grad_out, const void* value, const float* loc,
                                   const float* attn, float* gacc, float* grad_loc, float* grad_attn,
                                   hipStream_t stream)
{
    constexpr int upb = kBlock / LPU;
    const int sc = samples_per_chunk(g.S, upb);
    const size_t lds = (size_t)upb * (sc + 1) * (sizeof(BwdRecord) + sizeof(float4));
    hipLaunchKernelGGL((backward_generic_kernel<T, LPU>), dim3(g.blocks), dim3(kBlock), lds, stream, g, sc,
                       make_chunkdiv(g.S, sc),
                       static_cast<const T*>(grad_out), static_cast<const T*>(value), loc, attn, gacc, grad_loc,
                       grad_attn);
    return hipGetLastError();
}

// Workspace of the fast path with grad_value: per-sample anchors and records
// (20 bytes per sample), per-(band, run) counts and offsets, the band lists
// (4 bytes per reserved entry) and the float32 partial tiles of split bands.
// Every piece starts 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t fast_workspace_layout(const Geometry& g, const TilePlan& tp, void* base, AnchorWs* aws, BandWs* bws,
                             float** partial)
{
    const size_t ns = (size_t)g.B * g.Nh * g.Nq * g.S;
    const size_t slabs = (size_t)g.B * g.Nh;
    const size_t nb = (size_t)tp.bands;
    const size_t cap = (size_t)tp.cap * slabs;
    size_t at = 0;
    char* p = static_cast<char*>(base);
    auto take = [&](size_t bytes) {
        char* r = p ? p + at : nullptr;
        at = align256(at + bytes);
        return r;
    };
    AnchorWs a;
    a.anchor = reinterpret_cast<uint32_t*>(take(ns * 4));
    a.rec = reinterpret_cast<float4*>(take(ns * 16));
    BandWs w;
    const size_t runs = nb * (size_t)tp.nwg;
    w.cnt = reinterpret_cast<int*>(take(slabs * runs * 4));
    w.off = reinterpret_cast<int*>(take(slabs * (runs + 1) * 4));
    w.k = reinterpret_cast<uint32_t*>(take(cap * 4));
    w.rec = a.rec;
    float* part = reinterpret_cast<float*>(take(slabs * (size_t)tp.part_per_slab * 4));
    if (aws) *aws = a;
    if (bws) *bws = w;
    if (partial) *partial = part;
    return at;
}

template <typename T, int VEC>
static hipError_t launch_fast_typed(const Geometry& g, int lpu, const void* grad_out, const void* value,
                                    const float* loc, const float* attn, float* grad_loc, float* grad_attn,
                                    AnchorWs ws, hipStream_t stream)
{
    switch (lpu) {
    case 1: return launch_fast_t<T, 1, VEC>(g, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
    case 2: return launch_fast_t<T, 2, VEC>(g, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
    case 4: return launch_fast_t<T, 4, VEC>(g, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
    case 8: return launch_fast_t<T, 8, VEC>(g, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
    case 16:
        if constexpr (VEC == 4)
            return launch_fast_t<T, 16, VEC>(g, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
        else
            return hipErrorInvalidValue;  // 8 lanes cover the 64 channels at most
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_tiles_typed(const Geometry& g, const TilePlan& tp, int lpu, BandWs w, const void* grad_out,
                                     void* grad_value, float* partial, int accumulate, hipStream_t stream)
{
    switch (lpu) {
    case 1: return launch_tiles_t<T, 1>(g, tp, w, grad_out, grad_value, partial, accumulate, stream);
    case 2: return launch_tiles_t<T, 2>(g, tp, w, grad_out, grad_value, partial, accumulate, stream);
    case 4: return launch_tiles_t<T, 4>(g, tp, w, grad_out, grad_value, partial, accumulate, stream);
    case 8: return launch_tiles_t<T, 8>(g, tp, w, grad_out, grad_value, partial, accumulate, stream);
    case 16: return launch_tiles_t<T, 16>(g, tp, w, grad_out, grad_value, partial, accumulate, stream);
    default: return hipErrorInvalidValue;
    }
}

// Fast path. Every grad_value element is written by exactly one store (no
// clearing needed); with `accumulate` the store adds the element's old value.
hipError_t launch_backward_fast(const Geometry& g, const TilePlan& tp, int lpu, int glpu, int gvec, int bf16,
                                int accumulate, const void* grad_out, const void* value, const float* loc,
                                const float* attn, void* grad_value, float* grad_loc, float* grad_attn,
                                void* workspace, hipStream_t stream)
{
    AnchorWs ws = {nullptr, nullptr};
    BandWs bw = {};
    float* partial = nullptr;
    if (grad_value) fast_workspace_layout(g, tp, workspace, &ws, &bw, &partial);
    // the gather: glpu lanes of gvec channels per unit (g.blocks counts its workgroups)
    hipError_t e = hipErrorInvalidValue;
    if (!bf16 && gvec == 4)
        e = launch_fast_typed<float, 4>(g, glpu, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
    else if (bf16 && gvec == 8)
        e = launch_fast_typed<uint16_t, 8>(g, glpu, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
    else if (bf16 && gvec == 4)
        e = launch_fast_typed<uint16_t, 4>(g, glpu, grad_out, value, loc, attn, grad_loc, grad_attn, ws, stream);
    if (e != hipSuccess || !grad_value) return e;
    const int slabs = g.B * g.Nh;
    // bucket the samples by band, one run per (band, bucketing workgroup)
    int max_bands = 1;
    for (int l = 0; l < g.Nl; ++l) max_bands = std::max(max_bands, tp.row_bands[l] * tp.col_bands[l]);
    const size_t band_lds = (size_t)2 * max_bands * sizeof(int);
    if (tp.nwg == 1) {
        hipLaunchKernelGGL(band_bucket_kernel, dim3(g.Nl, slabs), dim3(kBandBlock), band_lds, stream, g, tp, bw,
                           ws.anchor, max_bands);
    } else {
        const dim3 bgrid(tp.nwg, g.Nl, slabs);
        hipLaunchKernelGGL(band_count_kernel, bgrid, dim3(kBandBlock), 0, stream, g, tp, ws.anchor, bw.cnt);
        hipLaunchKernelGGL(band_scan_kernel, dim3(slabs), dim3(kBlock), 0, stream, tp, bw.cnt, bw.off);
        hipLaunchKernelGGL(band_fill_kernel, bgrid, dim3(kBandBlock), band_lds, stream, g, tp, bw, ws.anchor,
                           max_bands);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return bf16 ? launch_tiles_typed<uint16_t>(g, tp, lpu, bw, grad_out, grad_value, partial, accumulate, stream)
                : launch_tiles_typed<float>(g, tp, lpu, bw, grad_out, grad_value, partial, accumulate, stream);
}

template <typename T>
static hipError_t launch_generic_typed(const Geometry& g, int lpu, const void* grad_out, const void* value,
                                       const float* loc, const float* attn, float* gacc, float* grad_loc,
                                       float* grad_attn, hipStream_t stream)
{
    switch (lpu) {
    case 1: return launch_generic_t<T, 1>(g, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    case 2: return launch_generic_t<T, 2>(g, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    case 4: return launch_generic_t<T, 4>(g, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    case 8: return launch_generic_t<T, 8>(g, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    case 16: return launch_generic_t<T, 16>(g, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    case 32: return launch_generic_t<T, 32>(g, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    case 64: return launch_generic_t<T, 64>(g, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    default: return hipErrorInvalidValue;
    }
}

// Generic path. float32: atomics straight into grad_value (cleared first
// unless accumulating). bfloat16: atomics into the float32 workspace
// (value-sized, cleared here), then one RNE conversion into grad_value.
hipError_t launch_backward_generic(const Geometry& g, int lpu, int bf16, int accumulate, const void* grad_out,
                                   const void* value, const float* loc, const float* attn, void* grad_value,
                                   float* grad_loc, float* grad_attn, void* workspace, hipStream_t stream)
{
    const int64_t nv = (int64_t)g.B * g.L * g.Nh * g.Ch;
    float* gacc = nullptr;
    hipError_t e = hipSuccess;
    if (grad_value) {
        gacc = bf16 ? static_cast<float*>(workspace) : static_cast<float*>(grad_value);
        if (bf16 || !accumulate) e = launch_zero(gacc, nv, stream);
        if (e != hipSuccess) return e;
    }
    e = bf16 ? launch_generic_typed<uint16_t>(g, lpu, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream)
             : launch_generic_typed<float>(g, lpu, grad_out, value, loc, attn, gacc, grad_loc, grad_attn, stream);
    if (e != hipSuccess || !grad_value || !bf16) return e;
    hipLaunchKernelGGL(acc_to_bf16_kernel, dim3(grid_for(nv)), dim3(kBlock), 0, stream, gacc,
                       static_cast<uint16_t*>(grad_value), nv, accumulate);
    return hipGetLastError();
}

}  // namespace msda
