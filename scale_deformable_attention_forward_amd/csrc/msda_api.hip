// C ABI of the library: host-side validation and kernel dispatch.
//
// Every check below runs before the first HIP call, so a non-OK status means
// nothing was enqueued. The entry points and their argument order follow the
// signatures on "MS Deformable Attention Kernel API Reference" (API
// Reference) and "MS Deformable Attention Backward Kernel API Reference"
// (API Reference); the Trainium-only tuning knobs of the backward page
// (gather/scatter indirection caps, replicated scatter buffers, dumps) have
// no counterpart here.
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/msda.h"
#include "msda_device.h"
#include "msda_producer.h"

namespace msda {
hipError_t launch_forward(const Geometry& g, int bf16, int vec, int64_t value_bytes, const void* value,
                          const float* loc, const float* attn, void* out, hipStream_t stream);
hipError_t launch_zero_elems(void* p, int64_t n, int elem, hipStream_t stream);
hipError_t launch_backward_fast(const Geometry& g, const TilePlan& tp, int lpu, int glpu, int gvec, int bf16,
                                int accumulate, const void* grad_out, const void* value, const float* loc,
                                const float* attn, void* grad_value, float* grad_loc, float* grad_attn,
                                void* workspace, hipStream_t stream);
hipError_t launch_backward_generic(const Geometry& g, int lpu, int bf16, int accumulate, const void* grad_out,
                                   const void* value, const float* loc, const float* attn, void* grad_value,
                                   float* grad_loc, float* grad_attn, void* workspace, hipStream_t stream);
struct AnchorWs;
struct BandWs;
size_t fast_workspace_layout(const Geometry& g, const TilePlan& tp, void* base, AnchorWs* aws, BandWs* bws,
                             float** partial);
}  // namespace msda

namespace {

using msda::Geometry;
using msda::TilePlan;

constexpr int64_t kIndexLimit = (int64_t)1 << 31;  // kernels index with 32-bit offsets
constexpr int64_t kForwardMinWaves = 8192;           // about 8 waves per SIMD of the 1,024 (256 CUs x 4)

struct Sizes {
    int64_t value_elems, loc_elems, attn_elems, out_elems;
    size_t value_bytes, out_bytes;
    int elem;  // bytes per value element
};

// Products that stay exact in int64 for any in-range problem or flag overflow.
bool mul_ok(int64_t a, int64_t b, int64_t* r)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *r = a * b;
    return true;
}

msda_status check_problem(const msda_problem* p, Geometry* g, Sizes* z)
{
    if (!p) return MSDA_ERR_INVALID_ARGUMENT;
    if (p->B < 0 || p->N_q < 0 || p->N_h < 1 || p->C_h < 1 || p->N_l < 1 || p->N_p < 1 || p->L < 1)
        return MSDA_ERR_INVALID_ARGUMENT;
    if (p->value_layout != MSDA_VALUE_BLNC && p->value_layout != MSDA_VALUE_BNLC) return MSDA_ERR_INVALID_ARGUMENT;
    if (p->sampling_locations_layout != MSDA_LOC_BQHLP2 && p->sampling_locations_layout != MSDA_LOC_B2QHLP)
        return MSDA_ERR_INVALID_ARGUMENT;
    if (p->align_corners != 0 && p->align_corners != 1) return MSDA_ERR_INVALID_ARGUMENT;
    if (p->padding_mode != MSDA_PAD_ZEROS && p->padding_mode != MSDA_PAD_BORDER) return MSDA_ERR_INVALID_ARGUMENT;
    if (p->value_dtype != MSDA_F32 && p->value_dtype != MSDA_BF16) return MSDA_ERR_INVALID_ARGUMENT;
    if (p->N_l > MSDA_MAX_LEVELS) return MSDA_ERR_UNSUPPORTED;
    if (!p->spatial_shapes || !p->level_start_index) return MSDA_ERR_INVALID_ARGUMENT;

    // level table: H, W >= 1, starts are the exclusive prefix sums, L = sum H*W
    int64_t total = 0;
    for (int64_t l = 0; l < p->N_l; ++l) {
        const int64_t H = p->spatial_shapes[2 * l], W = p->spatial_shapes[2 * l + 1];
        if (H < 1 || W < 1) return MSDA_ERR_INVALID_LEVELS;
        if (p->level_start_index[l] != total) return MSDA_ERR_INVALID_LEVELS;
        int64_t hw;
        if (!mul_ok(H, W, &hw) || hw >= kIndexLimit || total + hw >= kIndexLimit) return MSDA_ERR_UNSUPPORTED;
        total += hw;
        // the float32 coordinate map needs pixel coordinates well inside 2^24
        if (H + 2 >= ((int64_t)1 << 24) || W + 2 >= ((int64_t)1 << 24)) return MSDA_ERR_UNSUPPORTED;
    }
    if (total != p->L) return MSDA_ERR_INVALID_LEVELS;

    int64_t S, t;
    if (!mul_ok(p->N_l, p->N_p, &S)) return MSDA_ERR_UNSUPPORTED;
    z->elem = p->value_dtype == MSDA_BF16 ? 2 : 4;
    if (!mul_ok(p->B, p->L, &t) || !mul_ok(t, p->N_h, &t) || !mul_ok(t, p->C_h, &z->value_elems))
        return MSDA_ERR_UNSUPPORTED;
    if (!mul_ok(p->B, p->N_q, &t) || !mul_ok(t, p->N_h, &t) || !mul_ok(t, S, &z->attn_elems))
        return MSDA_ERR_UNSUPPORTED;
    if (!mul_ok(z->attn_elems, 2, &z->loc_elems)) return MSDA_ERR_UNSUPPORTED;
    if (!mul_ok(p->B, p->N_q, &t) || !mul_ok(t, p->N_h, &t) || !mul_ok(t, p->C_h, &z->out_elems))
        return MSDA_ERR_UNSUPPORTED;
    if (z->value_elems >= kIndexLimit || z->loc_elems >= kIndexLimit || z->out_elems >= kIndexLimit)
        return MSDA_ERR_UNSUPPORTED;
    z->value_bytes = (size_t)z->value_elems * z->elem;
    z->out_bytes = (size_t)z->out_elems * z->elem;

    g->B = (int32_t)p->B;
    g->L = (int32_t)p->L;
    g->Nq = (int32_t)p->N_q;
    g->Nh = (int32_t)p->N_h;
    g->Ch = (int32_t)p->C_h;
    g->Nl = (int32_t)p->N_l;
    g->Np = (int32_t)p->N_p;
    g->S = (int32_t)S;
    g->bnlc = p->value_layout == MSDA_VALUE_BNLC;
    g->b2q = p->sampling_locations_layout == MSDA_LOC_B2QHLP;
    g->align_corners = p->align_corners;
    g->border = p->padding_mode == MSDA_PAD_BORDER;
    g->loc_pair_aligned = 0;
    for (int l = 0; l < msda::kMaxLevels; ++l) {
        const bool in = l < p->N_l;
        g->lv.H[l] = in ? (int32_t)p->spatial_shapes[2 * l] : 1;
        g->lv.W[l] = in ? (int32_t)p->spatial_shapes[2 * l + 1] : 1;
        g->lv.start[l] = in ? (int32_t)p->level_start_index[l] : 0;
    }
    g->nq_div = msda::make_fastdiv((uint32_t)g->Nq);
    g->nh_div = msda::make_fastdiv((uint32_t)g->Nh);
    g->np_div = msda::make_fastdiv((uint32_t)g->Np);
    g->ch_div = msda::make_fastdiv(1);
    return MSDA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int ilog2(int v)
{
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Widest per-lane vector (in elements) that the channel count and every
// pointer stepping by it allow: 16-byte loads where possible.
int pick_vec(int64_t C_h, int elem, std::initializer_list<const void*> ptrs)
{
    for (int vec = 16 / elem; vec > 1; vec /= 2) {
        if (C_h % vec) continue;
        bool ok = true;
        for (const void* p : ptrs) ok = ok && (!p || aligned(p, (size_t)vec * elem));
        if (ok) return vec;
    }
    return 1;
}

// Lanes per destination pixel / per unit on the fast backward path: C_h / 4
// rounded up to a power of two (4 channels per lane).
int fast_lanes(int64_t C_h) { return 1 << ilog2((int)((C_h + 3) / 4)); }

// The fast backward path needs C_h % 4 == 0, C_h <= 64 (4 channels per lane,
// at most 16 lanes per pixel), pixel coordinates that pack in 16 bits, at
// most 65535 (b, h) slabs (a grid dimension of the bucketing kernels), and
// grad_output rows of one batch spanning fewer than 2^31 - 2^20 bytes (the
// tile pass reads them through a buffer resource with 32-bit byte offsets).
bool fast_backward_shape(const msda_problem& p)
{
    if (p.C_h % 4 != 0 || p.C_h > 64) return false;
    if (p.B * p.N_h > 65535) return false;
    const int64_t elem = p.value_dtype == MSDA_BF16 ? 2 : 4;
    if (!msda::buffer_loads_ok(p.N_q * p.N_h * p.C_h * elem)) return false;
    for (int64_t l = 0; l < p.N_l; ++l)
        if (p.spatial_shapes[2 * l] > 60000 || p.spatial_shapes[2 * l + 1] > 60000) return false;
    return true;
}

// Cut every level into bands (destination tiles) of rows x cols pixels.
// Levels with fewer samples per slab than pixels take pixel mode: bands of
// at most kTileBins anchor bins expected to hold about three quarters of
// one LDS pass of entries, fewest bands first, walked by lane groups that
// own pixel blocks; so do levels small enough for one such band. Every
// other level takes halo mode: the
// (rows + 1) x (cols + 1) anchor bins of a band are dealt out to ny x nx lane
// groups in blocks of kRectRows x kRectCols bins (ny * nx <= the groups of
// one tile workgroup), so rows = ny * kRectRows - 1 and cols = nx *
// kRectCols - 1 (or the level's size), with at most kTileBins anchor bins;
// of those shapes the one with the fewest tiles is taken (then the fewest
// column bands: a sample is listed once per band its 2x2 corner block
// touches). The choices depend on the shapes only. At most
// kMaxBandsPerLevel bands per level. A
// band whose list is expected to hold more than three LDS passes of entries
// (coarse levels, where many samples land on each pixel) is split into
// chunks of its list of about three passes, one workgroup each (smaller
// chunks add partial tiles and reduction work, larger ones make the tile
// pass wait on its longest jobs); each chunk writes a float32 partial
// tile and the reduction pass adds a band's partial tiles in chunk order.
// Returns false if a level cannot be tiled that way.
bool plan_tiles(const msda_problem& p, int lpu, TilePlan* tp)
{
    constexpr int64_t RH = msda::kRectRows, RW = msda::kRectCols;
    const int64_t groups = msda::kTileBlock / lpu;
    const int64_t nsamp = p.N_q * p.N_p;
    const int64_t nwg = std::max<int64_t>(1, (nsamp + msda::kBandChunk - 1) / msda::kBandChunk);
    if (nwg >= 65536) return false;  // grid x of the bucketing kernels stays small
    int64_t jobs = 0, pjobs = 0, bands = 0, cap = 0, part = 0, pieces = 0;
    for (int64_t l = 0; l < msda::kMaxLevels; ++l) {
        tp->job_begin[l] = (int32_t)jobs;
        tp->pjob_begin[l] = (int32_t)pjobs;
        tp->band_begin[l] = (int32_t)bands;
        tp->part_off[l] = (int32_t)part;
        tp->rpiece_begin[l] = (int32_t)pieces;
        tp->rpieces_per_band[l] = 1;
        tp->rows_div[l] = msda::make_fastdiv(1);
        tp->cols_div[l] = msda::make_fastdiv(1);
        if (l >= p.N_l) {
            tp->rows[l] = tp->row_bands[l] = tp->cols[l] = tp->col_bands[l] = tp->chunks[l] = 1;
            continue;
        }
        const int64_t H = p.spatial_shapes[2 * l], W = p.spatial_shapes[2 * l + 1];
        int64_t rows = 0, cols = 0, rb = 0, cb = 0;
        bool pixel = false;
        if (nsamp > 0 && nsamp < H * W) {
            // pixel mode: bands of at most kTileBins anchor bins holding about
            // three quarters of a pass of entries if locations spread evenly
            // (so one pass is the rule), fewest bands, then fewest column
            // bands. Only the smallest band height giving each row-band
            // count can win (a taller band only narrows the columns), so
            // the heights tried are the distinct values of ceil(H / k).
            const int64_t r_max = std::min<int64_t>(H, msda::kTileBins / 2 - 1);
            for (int64_t k = 1; k <= H;) {
                const int64_t r = (H + k - 1) / k;  // the smallest height with ceil(H / r) row bands
                if (r <= r_max) {
                    const int64_t c_bins = msda::kTileBins / (r + 1) - 1;
                    const int64_t c_fill = 3 * msda::kTileEntries / 4 * (H + 1) * (W + 1) / (nsamp * (r + 1)) - 1;
                    const int64_t c = std::min<int64_t>(W, std::min(c_bins, c_fill));
                    const int64_t nrb = (H + r - 1) / r, ncb = c >= 1 ? (W + c - 1) / c : 0;
                    if (c >= 1 && (rows == 0 || nrb * ncb < rb * cb || (nrb * ncb == rb * cb && ncb < cb))) {
                        rows = r;
                        cols = c;
                        rb = nrb;
                        cb = ncb;
                    }
                }
                if (r == 1) break;
                k = (H + r - 2) / (r - 1);  // the first k with a smaller height
            }
            pixel = rows > 0;
        } else if (nsamp > 0 && (H + 1) * (W + 1) <= msda::kTileBins && nsamp <= 3 * msda::kTileEntries / 4) {
            // a small level that one pixel-mode band covers with about one pass
            rows = H;
            cols = W;
            rb = cb = 1;
            pixel = true;
        }
        // halo mode: a band of r x c pixels has (r + 1) x (c + 1) anchor bins,
        // dealt out to ny x nx lane groups in blocks of RH x RW bins
        const int64_t nx_max = pixel ? 0 : std::min<int64_t>(groups, W / RW + 1);
        for (int64_t nx = 1; nx <= nx_max; ++nx) {
            const int64_t ny = std::min<int64_t>(groups / nx, H / RH + 1);
            const int64_t r = std::min<int64_t>(H, ny * RH - 1), c = std::min<int64_t>(W, nx * RW - 1);
            if (r < 1 || c < 1 || (r + 1) * (c + 1) > msda::kTileBins) continue;
            const int64_t nrb = (H + r - 1) / r, ncb = (W + c - 1) / c;
            if (rows == 0 || nrb * ncb < rb * cb || (nrb * ncb == rb * cb && ncb < cb)) {
                rows = r;
                cols = c;
                rb = nrb;
                cb = ncb;
            }
        }
        if (rows == 0) return false;
        if (rb * cb > msda::kMaxBandsPerLevel) return false;
        // list entries of one band if locations spread evenly
        const int64_t expect = nsamp * (rows + 1) / (H + 1) * (cols + 1) / (W + 1) + 1;
        int64_t chunks = (expect + 3 * msda::kTileEntries - 1) / (3 * msda::kTileEntries);
        chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, std::min<int64_t>(nwg, 1024)));  // >= 1 run each
        if (pixel) chunks = 1;  // pixel-mode bands are not split
        tp->rows[l] = (int32_t)rows;
        tp->rows_div[l] = msda::make_fastdiv((uint32_t)rows);
        tp->cols_div[l] = msda::make_fastdiv((uint32_t)cols);
        tp->row_bands[l] = (int32_t)rb;
        tp->cols[l] = (int32_t)cols;
        tp->col_bands[l] = (int32_t)cb;
        tp->chunks[l] = (int32_t)chunks;
        (pixel ? pjobs : jobs) += rb * cb * chunks;
        bands += rb * cb;
        cap += nsamp * (cb > 1 ? 4 : 2);  // a sample touches at most 2 row bands x 2 column bands
        if (chunks > 1) {
            const int64_t tile = rows * cols * p.C_h;  // floats of one partial tile
            part += rb * cb * chunks * tile;
            const int64_t ppb = (tile / 4 + msda::kReduceF4 - 1) / msda::kReduceF4;
            tp->rpieces_per_band[l] = (int32_t)ppb;
            pieces += rb * cb * ppb;
        }
        if (part >= kIndexLimit || pieces >= kIndexLimit) return false;
    }
    tp->job_begin[msda::kMaxLevels] = (int32_t)jobs;
    tp->pjob_begin[msda::kMaxLevels] = (int32_t)pjobs;
    tp->rpiece_begin[msda::kMaxLevels] = (int32_t)pieces;
    tp->jobs = (int32_t)jobs;
    tp->pjobs = (int32_t)pjobs;
    tp->bands = (int32_t)bands;
    tp->rpieces = (int32_t)pieces;
    tp->nwg = (int32_t)nwg;
    tp->cap = cap;
    tp->part_per_slab = part;
    return jobs < kIndexLimit && pjobs < kIndexLimit && cap < kIndexLimit && bands * nwg + 1 < kIndexLimit &&
           (int64_t)p.B * p.N_h * (bands * nwg + 1) < kIndexLimit;
}

// Fast-path workspace bytes for `p` (0 if the tiled pass cannot take it).
size_t fast_workspace_bytes(const msda_problem& p, const Geometry& g)
{
    TilePlan tp = {};
    if (!plan_tiles(p, fast_lanes(p.C_h), &tp)) return 0;
    return msda::fast_workspace_layout(g, tp, nullptr, nullptr, nullptr, nullptr);
}

// Generic-path workspace bytes: a float32 accumulator of value's shape for
// bfloat16 grad_value, nothing for float32.
size_t generic_workspace_bytes(const msda_problem& p, const Sizes& z)
{
    return p.value_dtype == MSDA_BF16 ? (size_t)z.value_elems * 4 : 0;
}

// Outputs [o] must not overlap any input or each other (NULL entries skipped).
struct Span {
    const void* p;
    size_t n;
};
bool spans_disjoint(std::initializer_list<Span> outs, std::initializer_list<Span> ins)
{
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlap(o->p, o->n, i.p, i.n)) return false;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(o->p, o->n, o2->p, o2->n)) return false;
    }
    return true;
}

// Producer geometry and the byte sizes of its tensors.
struct ProducerSizes {
    size_t query, ref, w_off, b_off, w_att, b_att;
};

msda_status check_producer(const msda_problem* p, int64_t D, bool fused, Geometry* g, Sizes* z,
                           msda::ProducerGeom* pg, ProducerSizes* ps)
{
    const msda_status st = check_problem(p, g, z);
    if (st != MSDA_OK) return st;
    if (D < 1) return MSDA_ERR_INVALID_ARGUMENT;
    const int64_t S = (int64_t)g->S;
    if (S > (fused ? msda::kPFusedMaxSamples : msda::kPMaxSamples)) return MSDA_ERR_UNSUPPORTED;
    int64_t M, qe, we;
    if (!mul_ok(p->B, p->N_q, &M) || !mul_ok(M, D, &qe) || qe >= kIndexLimit) return MSDA_ERR_UNSUPPORTED;
    if (!mul_ok(p->N_h * 3 * S, D + 1, &we) || we >= kIndexLimit) return MSDA_ERR_UNSUPPORTED;
    if (M * p->N_l * 2 >= kIndexLimit) return MSDA_ERR_UNSUPPORTED;
    ps->query = (size_t)qe * z->elem;
    ps->ref = (size_t)M * p->N_l * 2 * 4;
    ps->w_off = (size_t)p->N_h * S * 2 * D * z->elem;
    ps->b_off = (size_t)p->N_h * S * 2 * 4;
    ps->w_att = (size_t)p->N_h * S * D * z->elem;
    ps->b_att = (size_t)p->N_h * S * 4;
    pg->M = (int32_t)M;
    pg->D = (int32_t)D;
    pg->S = (int32_t)S;
    pg->Nh = g->Nh;
    pg->Nl = g->Nl;
    pg->Np = g->Np;
    pg->Nq = g->Nq;
    const int64_t ct = (3 * S + 15) / 16;
    pg->ct = ct <= 3 ? 3 : ct <= 6 ? 6 : 12;  // the instantiated column-tile counts
    pg->tpr = std::max(4, 1 << ilog2((int)S));
    pg->b2q = g->b2q;
    pg->loc_pair_aligned = 0;
    pg->vec = 1;
    // weight gradients: about 1024 workgroups of (row chunk, head, 64 columns)
    const int64_t per_chunk = p->N_h * ((D + 63) / 64);
    const int64_t target = std::max<int64_t>(1, 1024 / std::max<int64_t>(1, per_chunk));
    int64_t rows = (std::max<int64_t>(M, 1) + target - 1) / target;
    rows = std::max<int64_t>(32, (rows + 31) / 32 * 32);
    pg->mrows = (int32_t)std::min<int64_t>(rows, kIndexLimit / 2);
    pg->mchunks = (int32_t)std::max<int64_t>(1, (M + pg->mrows - 1) / pg->mrows);
    return MSDA_OK;
}

// 4-element row loads for the projection operands when D and the pointers allow.
int producer_vec(int64_t D, int elem, std::initializer_list<const void*> ptrs)
{
    if (D % 4) return 1;
    for (const void* q : ptrs)
        if (q && !aligned(q, 4 * (size_t)elem)) return 1;
    return 4;
}

msda::ProducerArgsRaw producer_args(const void* query, const float* ref, const void* w_off, const float* b_off,
                                    const void* w_att, const float* b_att)
{
    return msda::ProducerArgsRaw{query, ref, w_off, b_off, w_att, b_att};
}

// msda_backward's validation and dispatch. With need_out, nothing is launched:
// every check except the workspace's runs, and *need_out receives the bytes
// of workspace the call would use.
msda_status backward_call(const msda_problem* problem, const void* grad_output, const void* value,
                          const float* sampling_locations, const float* attention_weights, void* grad_value,
                          float* grad_sampling_locations, float* grad_attention_weights, unsigned int flags,
                          void* workspace, size_t workspace_bytes, hipStream_t stream, size_t* need_out)
{
    if (need_out) *need_out = 0;
    Geometry g;
    Sizes z;
    const msda_status st = check_problem(problem, &g, &z);
    if (st != MSDA_OK) return st;
    if (flags & ~(unsigned int)MSDA_BACKWARD_ACCUMULATE_GRAD_VALUE) return MSDA_ERR_INVALID_ARGUMENT;
    const int accumulate = (flags & MSDA_BACKWARD_ACCUMULATE_GRAD_VALUE) ? 1 : 0;
    if (!grad_value && !grad_sampling_locations && !grad_attention_weights) return MSDA_ERR_NOTHING_TO_COMPUTE;
    const bool empty = z.out_elems == 0;
    const bool bf16 = problem->value_dtype == MSDA_BF16;
    if (!empty && (!grad_output || !value || !sampling_locations || !attention_weights))
        return MSDA_ERR_INVALID_ARGUMENT;
    const void* ins[4] = {grad_output, value, sampling_locations, attention_weights};
    const size_t in_align[4] = {(size_t)z.elem, (size_t)z.elem, 4, 4};
    for (int i = 0; i < 4; ++i)
        if (ins[i] && !aligned(ins[i], in_align[i])) return MSDA_ERR_INVALID_ARGUMENT;
    const void* outs[3] = {grad_value, grad_sampling_locations, grad_attention_weights};
    const size_t out_align[3] = {(size_t)z.elem, 4, 4};
    for (int o = 0; o < 3; ++o)
        if (outs[o] && !aligned(outs[o], out_align[o])) return MSDA_ERR_INVALID_ARGUMENT;
    const size_t loc_bytes = (size_t)z.loc_elems * 4, attn_bytes = (size_t)z.attn_elems * 4;
    const size_t in_bytes[4] = {z.out_bytes, z.value_bytes, loc_bytes, attn_bytes};
    const size_t out_bytes[3] = {z.value_bytes, loc_bytes, attn_bytes};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 4; ++i)
            if (overlap(outs[o], out_bytes[o], ins[i], in_bytes[i])) return MSDA_ERR_INVALID_ARGUMENT;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (overlap(outs[o], out_bytes[o], outs[o2], out_bytes[o2])) return MSDA_ERR_INVALID_ARGUMENT;
    }

    // Fast path: 4 channels per lane (one 16-byte float32 or 8-byte bfloat16
    // load; see gvec below for the bfloat16 gather) and the destination-tiled
    // grad_value pass; otherwise one channel per lane and atomics.
    const int64_t C_h = problem->C_h;
    const size_t row_align = 4 * (size_t)z.elem;
    TilePlan tp = {};
    const bool fast = fast_backward_shape(*problem) && plan_tiles(*problem, fast_lanes(C_h), &tp) &&
                      aligned(value, row_align) && aligned(grad_output, row_align) &&
                      (!grad_value || aligned(grad_value, row_align));
    if (grad_value && !empty) {
        const size_t need = fast ? msda::fast_workspace_layout(g, tp, nullptr, nullptr, nullptr, nullptr)
                                 : generic_workspace_bytes(*problem, z);
        if (need_out) *need_out = need;
        if (need > 0 && !need_out) {
            if (!workspace || workspace_bytes < need) return MSDA_ERR_WORKSPACE_TOO_SMALL;
            if (!aligned(workspace, 16)) return MSDA_ERR_INVALID_ARGUMENT;
            for (int i = 0; i < 4; ++i)
                if (overlap(workspace, need, ins[i], in_bytes[i])) return MSDA_ERR_INVALID_ARGUMENT;
            for (int o = 0; o < 3; ++o)
                if (overlap(workspace, need, outs[o], out_bytes[o])) return MSDA_ERR_INVALID_ARGUMENT;
        }
    }
    const int lpu = fast ? fast_lanes(C_h) : 1 << ilog2((int)std::min<int64_t>(64, C_h));
    // the fast path's gather of grad_A and grad_loc: glpu lanes of gvec
    // channels per unit; bfloat16 rows of whole 16-byte groups take 8 channels
    // a lane (one 16-byte load per corner), everything else 4 as the tiles do
    const int gvec = fast && bf16 && C_h % 8 == 0 && aligned(value, 16) && aligned(grad_output, 16) ? 8 : 4;
    const int glpu = gvec == 8 ? std::max(1, lpu / 2) : lpu;
    const int64_t units = (int64_t)g.B * g.Nh * g.Nq;
    const int64_t upb = msda::kBlock / glpu;
    g.lpu_log2 = ilog2(glpu);
    g.chunks = 1;
    g.units = (int32_t)units;
    g.blocks = (int32_t)((units + upb - 1) / upb);
    g.loc_pair_aligned = aligned(sampling_locations, 8) && (!grad_sampling_locations || aligned(grad_sampling_locations, 8));
    if (fast && grad_value && !empty && (int64_t)(tp.jobs + tp.pjobs) * g.B * g.Nh >= kIndexLimit) return MSDA_ERR_UNSUPPORTED;
    if (need_out) return MSDA_OK;

    hipError_t e = hipSuccess;
    if (empty) {
        // no query reaches grad_value: it is all zeros (or left as is)
        if (grad_value && !accumulate) e = msda::launch_zero_elems(grad_value, z.value_elems, z.elem, stream);
        return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
    }
    if (fast) {
        e = msda::launch_backward_fast(g, tp, lpu, glpu, gvec, bf16, accumulate, grad_output, value,
                                       sampling_locations, attention_weights, grad_value, grad_sampling_locations,
                                       grad_attention_weights, workspace, stream);
    } else {
        e = msda::launch_backward_generic(g, lpu, bf16, accumulate, grad_output, value, sampling_locations,
                                          attention_weights, grad_value, grad_sampling_locations,
                                          grad_attention_weights, workspace, stream);
    }
    return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
}

// Static scratch of msda_backward_noalloc: the workspace msda_backward would
// take, as a device array of the library. Each GPU holds its own copy (at its
// own address) from the module's load until the process ends. Host code never
// uses the array's name as an address: it takes each device's address from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)MSDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's scratch address; `stream` (if not NULL) must belong to the
// current device.
msda_status scratch_for_current_device(hipStream_t stream, void** ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MSDA_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = 0;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MSDA_ERR_HIP;
        if ((int)sdev != dev) return MSDA_ERR_INVALID_ARGUMENT;
    }
    if (dev < 0 || dev >= kMaxDevices) return MSDA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSDA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MSDA_OK;
}

}  // namespace

extern "C" {

msda_status msda_forward(const msda_problem* problem, const void* value, const float* sampling_locations,
                         const float* attention_weights, void* output, hipStream_t stream)
{
    Geometry g;
    Sizes z;
    const msda_status st = check_problem(problem, &g, &z);
    if (st != MSDA_OK) return st;
    if (z.out_elems == 0) return MSDA_OK;  // B == 0 or N_q == 0
    if (!value || !sampling_locations || !attention_weights || !output) return MSDA_ERR_INVALID_ARGUMENT;
    if (!aligned(value, z.elem) || !aligned(output, z.elem) || !aligned(sampling_locations, 4) ||
        !aligned(attention_weights, 4))
        return MSDA_ERR_INVALID_ARGUMENT;
    const size_t loc_bytes = (size_t)z.loc_elems * 4, attn_bytes = (size_t)z.attn_elems * 4;
    if (overlap(output, z.out_bytes, value, z.value_bytes) || overlap(output, z.out_bytes, sampling_locations, loc_bytes) ||
        overlap(output, z.out_bytes, attention_weights, attn_bytes))
        return MSDA_ERR_INVALID_ARGUMENT;

    // Widest vector the alignment allows; for small problems narrower ones,
    // which spread a unit's channels over more lanes (each channel's
    // multiply-add chain, and so every output bit, stays the same), until
    // the grid has kForwardMinWaves waves to cover the gathers' latency.
    int vec = pick_vec(problem->C_h, z.elem, {value, output});
    auto lanes_for = [&](int v) { return 1 << ilog2((int)std::min<int64_t>(64, (problem->C_h + v - 1) / v)); };
    auto chunks_for = [&](int v) { return (problem->C_h + (int64_t)lanes_for(v) * v - 1) / ((int64_t)lanes_for(v) * v); };
    auto waves_for = [&](int v) { return (int64_t)g.B * g.Nh * g.Nq * chunks_for(v) * lanes_for(v) / msda::kWave; };
    while (vec > 1 && waves_for(vec) < kForwardMinWaves) vec /= 2;
    g.lpu_log2 = ilog2(lanes_for(vec));
    g.chunks = (int32_t)chunks_for(vec);
    g.ch_div = msda::make_fastdiv((uint32_t)g.chunks);
    const int64_t units = (int64_t)g.B * g.Nh * g.Nq * g.chunks;
    const int64_t upb = msda::kBlock >> g.lpu_log2;
    if (units >= kIndexLimit) return MSDA_ERR_UNSUPPORTED;
    g.units = (int32_t)units;
    g.blocks = (int32_t)((units + upb - 1) / upb);
    g.loc_pair_aligned = aligned(sampling_locations, 8);
    const hipError_t e = msda::launch_forward(g, problem->value_dtype == MSDA_BF16, vec, (int64_t)z.value_bytes,
                                              value, sampling_locations, attention_weights, output, stream);
    return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
}

msda_status msda_backward_workspace_size(const msda_problem* problem, size_t* bytes)
{
    if (!bytes) return MSDA_ERR_INVALID_ARGUMENT;
    Geometry g;
    Sizes z;
    const msda_status st = check_problem(problem, &g, &z);
    if (st != MSDA_OK) return st;
    // The path is chosen per call (it also depends on pointer alignment), so
    // the size covers whichever of the two a call may take.
    const size_t fast = fast_backward_shape(*problem) ? fast_workspace_bytes(*problem, g) : 0;
    *bytes = std::max(fast, generic_workspace_bytes(*problem, z));
    return MSDA_OK;
}

msda_status msda_backward(const msda_problem* problem, const void* grad_output, const void* value,
                          const float* sampling_locations, const float* attention_weights, void* grad_value,
                          float* grad_sampling_locations, float* grad_attention_weights, unsigned int flags,
                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return backward_call(problem, grad_output, value, sampling_locations, attention_weights, grad_value,
                         grad_sampling_locations, grad_attention_weights, flags, workspace, workspace_bytes, stream,
                         nullptr);
}

msda_status msda_backward_noalloc(const msda_problem* problem, const void* grad_output, const void* value,
                                  const float* sampling_locations, const float* attention_weights, void* grad_value,
                                  float* grad_sampling_locations, float* grad_attention_weights, unsigned int flags,
                                  hipStream_t stream)
{
    // every check first, without a HIP call; then this device's scratch
    size_t need = 0;
    msda_status st = backward_call(problem, grad_output, value, sampling_locations, attention_weights, grad_value,
                                   grad_sampling_locations, grad_attention_weights, flags, nullptr, 0, stream, &need);
    if (st != MSDA_OK) return st;
    if (need > kNoAllocScratchBytes) return MSDA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_for_current_device(stream, &ws);
        if (st != MSDA_OK) return st;
    }
    return backward_call(problem, grad_output, value, sampling_locations, attention_weights, grad_value,
                         grad_sampling_locations, grad_attention_weights, flags, ws, ws ? kNoAllocScratchBytes : 0,
                         stream, nullptr);
}

msda_status msda_producer_forward(const msda_problem* problem, int64_t D, const void* query,
                                  const float* reference_points, const void* offset_weight, const float* offset_bias,
                                  const void* attention_weight, const float* attention_bias,
                                  float* sampling_locations, float* attention_weights, hipStream_t stream)
{
    Geometry g;
    Sizes z;
    msda::ProducerGeom pg;
    ProducerSizes ps;
    const msda_status st = check_producer(problem, D, false, &g, &z, &pg, &ps);
    if (st != MSDA_OK) return st;
    if (pg.M == 0) return MSDA_OK;
    if (!query || !reference_points || !offset_weight || !attention_weight || !sampling_locations ||
        !attention_weights)
        return MSDA_ERR_INVALID_ARGUMENT;
    if (!aligned(query, z.elem) || !aligned(offset_weight, z.elem) || !aligned(attention_weight, z.elem) ||
        !aligned(reference_points, 4) || !aligned(offset_bias, 4) || !aligned(attention_bias, 4) ||
        !aligned(sampling_locations, 4) || !aligned(attention_weights, 4))
        return MSDA_ERR_INVALID_ARGUMENT;
    const size_t loc_bytes = (size_t)z.loc_elems * 4, attn_bytes = (size_t)z.attn_elems * 4;
    if (!spans_disjoint({{sampling_locations, loc_bytes}, {attention_weights, attn_bytes}},
                        {{query, ps.query}, {reference_points, ps.ref}, {offset_weight, ps.w_off},
                         {offset_bias, ps.b_off}, {attention_weight, ps.w_att}, {attention_bias, ps.b_att}}))
        return MSDA_ERR_INVALID_ARGUMENT;
    pg.vec = producer_vec(D, z.elem, {query, offset_weight, attention_weight});
    pg.loc_pair_aligned = aligned(sampling_locations, 8);
    const hipError_t e = msda::launch_producer_forward(
        g, pg, problem->value_dtype == MSDA_BF16,
        producer_args(query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias),
        sampling_locations, attention_weights, stream);
    return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
}

msda_status msda_fused_forward(const msda_problem* problem, int64_t D, const void* query,
                               const float* reference_points, const void* offset_weight, const float* offset_bias,
                               const void* attention_weight, const float* attention_bias, const void* value,
                               void* output, float* sampling_locations, float* attention_weights, hipStream_t stream)
{
    Geometry g;
    Sizes z;
    msda::ProducerGeom pg;
    ProducerSizes ps;
    const msda_status st = check_producer(problem, D, true, &g, &z, &pg, &ps);
    if (st != MSDA_OK) return st;
    if (pg.M == 0) return MSDA_OK;
    if (!query || !reference_points || !offset_weight || !attention_weight || !value || !output)
        return MSDA_ERR_INVALID_ARGUMENT;
    if (!aligned(query, z.elem) || !aligned(offset_weight, z.elem) || !aligned(attention_weight, z.elem) ||
        !aligned(value, z.elem) || !aligned(output, z.elem) || !aligned(reference_points, 4) ||
        !aligned(offset_bias, 4) || !aligned(attention_bias, 4) || !aligned(sampling_locations, 4) ||
        !aligned(attention_weights, 4))
        return MSDA_ERR_INVALID_ARGUMENT;
    const size_t loc_bytes = (size_t)z.loc_elems * 4, attn_bytes = (size_t)z.attn_elems * 4;
    if (!spans_disjoint({{output, z.out_bytes}, {sampling_locations, loc_bytes}, {attention_weights, attn_bytes}},
                        {{query, ps.query}, {reference_points, ps.ref}, {offset_weight, ps.w_off},
                         {offset_bias, ps.b_off}, {attention_weight, ps.w_att}, {attention_bias, ps.b_att},
                         {value, z.value_bytes}}))
        return MSDA_ERR_INVALID_ARGUMENT;
    if ((int64_t)g.B * g.Nh * ((g.Nq + 63) / 64) >= kIndexLimit) return MSDA_ERR_UNSUPPORTED;
    // the sampler's lane layout, as in msda_forward
    const int vec = pick_vec(problem->C_h, z.elem, {value, output});
    const int lanes = (int)std::min<int64_t>(64, (problem->C_h + vec - 1) / vec);
    g.lpu_log2 = ilog2(lanes);
    const int64_t per_chunk = ((int64_t)1 << g.lpu_log2) * vec;
    g.chunks = (int32_t)((problem->C_h + per_chunk - 1) / per_chunk);
    g.ch_div = msda::make_fastdiv((uint32_t)g.chunks);
    g.units = 0;
    g.blocks = 0;
    pg.vec = producer_vec(D, z.elem, {query, offset_weight, attention_weight});
    pg.loc_pair_aligned = sampling_locations && aligned(sampling_locations, 8);
    const hipError_t e = msda::launch_fused_forward(
        g, pg, problem->value_dtype == MSDA_BF16, vec,
        producer_args(query, reference_points, offset_weight, offset_bias, attention_weight, attention_bias),
        (int64_t)z.value_bytes, value, output, sampling_locations, attention_weights, stream);
    return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
}

msda_status msda_producer_backward_workspace_size(const msda_problem* problem, int64_t D, size_t* bytes)
{
    if (!bytes) return MSDA_ERR_INVALID_ARGUMENT;
    Geometry g;
    Sizes z;
    msda::ProducerGeom pg;
    ProducerSizes ps;
    const msda_status st = check_producer(problem, D, false, &g, &z, &pg, &ps);
    if (st != MSDA_OK) return st;
    *bytes = pg.M == 0 ? 0 : msda::producer_bwd_workspace_floats(pg) * sizeof(float);
    return MSDA_OK;
}

msda_status msda_producer_backward(const msda_problem* problem, int64_t D, const void* query,
                                   const void* offset_weight, const void* attention_weight,
                                   const float* attention_weights, const float* grad_sampling_locations,
                                   const float* grad_attention_weights, void* grad_query,
                                   float* grad_reference_points, float* grad_offset_weight, float* grad_offset_bias,
                                   float* grad_attention_weight, float* grad_attention_bias, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream)
{
    Geometry g;
    Sizes z;
    msda::ProducerGeom pg;
    ProducerSizes ps;
    const msda_status st = check_producer(problem, D, false, &g, &z, &pg, &ps);
    if (st != MSDA_OK) return st;
    const bool want_w = grad_offset_weight || grad_offset_bias || grad_attention_weight || grad_attention_bias;
    if (!grad_query && !grad_reference_points && !want_w) return MSDA_ERR_NOTHING_TO_COMPUTE;
    const size_t loc_bytes = (size_t)z.loc_elems * 4, attn_bytes = (size_t)z.attn_elems * 4;
    const std::initializer_list<Span> outs = {{grad_query, ps.query}, {grad_reference_points, ps.ref},
                                              {grad_offset_weight, ps.w_off / z.elem * 4},
                                              {grad_offset_bias, ps.b_off},
                                              {grad_attention_weight, ps.w_att / z.elem * 4},
                                              {grad_attention_bias, ps.b_att}};
    for (const Span& o : outs)
        if (o.p && !aligned(o.p, o.p == grad_query ? (size_t)z.elem : 4)) return MSDA_ERR_INVALID_ARGUMENT;
    if (pg.M == 0) {
        // no rows: the weight and bias gradients are sums over nothing
        hipError_t e = hipSuccess;
        for (const Span& o : {outs.begin()[2], outs.begin()[3], outs.begin()[4], outs.begin()[5]})
            if (o.p && e == hipSuccess) e = msda::launch_zero_elems(const_cast<void*>(o.p), (int64_t)(o.n / 4), 4, stream);
        return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
    }
    if (!query || !offset_weight || !attention_weight || !attention_weights) return MSDA_ERR_INVALID_ARGUMENT;
    if (!aligned(query, z.elem) || !aligned(offset_weight, z.elem) || !aligned(attention_weight, z.elem) ||
        !aligned(attention_weights, 4) || !aligned(grad_sampling_locations, 4) || !aligned(grad_attention_weights, 4))
        return MSDA_ERR_INVALID_ARGUMENT;
    const std::initializer_list<Span> ins = {{query, ps.query}, {offset_weight, ps.w_off},
                                             {attention_weight, ps.w_att}, {attention_weights, attn_bytes},
                                             {grad_sampling_locations, loc_bytes},
                                             {grad_attention_weights, attn_bytes}};
    if (!spans_disjoint(outs, ins)) return MSDA_ERR_INVALID_ARGUMENT;
    const size_t need = msda::producer_bwd_workspace_floats(pg) * sizeof(float);
    if (want_w) {
        if (!workspace || workspace_bytes < need) return MSDA_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 16)) return MSDA_ERR_INVALID_ARGUMENT;
        for (const Span& s : ins)
            if (overlap(workspace, need, s.p, s.n)) return MSDA_ERR_INVALID_ARGUMENT;
        for (const Span& s : outs)
            if (overlap(workspace, need, s.p, s.n)) return MSDA_ERR_INVALID_ARGUMENT;
    }
    pg.vec = producer_vec(D, z.elem, {query, offset_weight, attention_weight});
    const msda::ProducerGradIn in{attention_weights, grad_attention_weights, grad_sampling_locations};
    const msda::ProducerGradOut out{grad_query, grad_reference_points, grad_offset_weight, grad_offset_bias,
                                    grad_attention_weight, grad_attention_bias};
    const hipError_t e = msda::launch_producer_backward(
        g, pg, problem->value_dtype == MSDA_BF16,
        producer_args(query, nullptr, offset_weight, nullptr, attention_weight, nullptr), in, out,
        want_w ? workspace : nullptr, stream);
    return e == hipSuccess ? MSDA_OK : MSDA_ERR_HIP;
}

const char* msda_status_string(msda_status status)
{
    switch (status) {
    case MSDA_OK: return "MSDA_OK";
    case MSDA_ERR_INVALID_ARGUMENT: return "MSDA_ERR_INVALID_ARGUMENT: bad pointer, alignment, overlap, size or enum";
    case MSDA_ERR_INVALID_LEVELS:
        return "MSDA_ERR_INVALID_LEVELS: spatial_shapes / level_start_index inconsistent with L";
    case MSDA_ERR_NOTHING_TO_COMPUTE: return "MSDA_ERR_NOTHING_TO_COMPUTE: all gradient outputs are NULL";
    case MSDA_ERR_UNSUPPORTED: return "MSDA_ERR_UNSUPPORTED: size, level count or dtype not supported";
    case MSDA_ERR_WORKSPACE_TOO_SMALL: return "MSDA_ERR_WORKSPACE_TOO_SMALL";
    case MSDA_ERR_HIP: return "MSDA_ERR_HIP: a kernel launch failed";
    }
    return "unknown msda_status";
}

int msda_abi_version(void) { return MSDA_ABI_VERSION; }

}  // extern "C"
