// Producer of the sampler's inputs for gfx950: sampling locations and
// attention weights from per-query features, its fusion with the forward
// sampler, and its backward.
//
// "MS Deformable Attention Kernel API Reference" (Background) samples the
// value pyramid at learned sampling locations with attention weights. They
// are produced, per query row m = (b, q) with feature vector x_m (D floats),
// by a linear projection followed by the usual normalisations:
//   off[m, h, l, p, xy] = x_m . W_off[(h, l, p, xy), :] + b_off[(h, l, p, xy)]   (pixels of level l)
//   z[m, h, l, p]       = x_m . W_att[(h, l, p), :]     + b_att[(h, l, p)]
//   loc[m, h, l, p, x]  = ref[m, l, x] + off[m, h, l, p, x] / W_l   (y: ref[m, l, y] + off / H_l)
//   A[m, h, :, :]       = softmax of z[m, h, :, :] over its N_l * N_p entries
//
// The projection is a dense contraction, so it runs on the matrix cores:
// v_mfma_f32_16x16x4f32 tiles (float32 operands staged in LDS; bfloat16
// inputs are widened exactly when staged). A workgroup (4 waves) owns 64 query
// rows and the 3S projection columns of one head (S = N_l * N_p: 2S offsets
// then S logits), so the softmax and the normalisation run in the epilogue on
// the tile it just produced. Wave w computes rows 16w..16w+15 against every
// 16-column tile of the head; K (= D) is staged 32 at a time.
//
// fused_forward_kernel continues from that epilogue straight into the
// sampler: the epilogue writes the sampler's gather records (the forward
// kernel's per-sample records) into LDS and the workgroup gathers its 64
// queries of one (b, h) slab, so the locations and weights never travel
// through HBM unless the caller asks for them (for the backward).
//
// Backward, with G_off / G_z the loss gradients with respect to off and z:
//   G_off[m, h, l, p, x] = dL/dloc[m, h, l, p, x] / W_l    (y: / H_l)
//   G_z[m, h, s]         = A[m, h, s] * (dL/dA[m, h, s] - sum_s' A[m, h, s'] dL/dA[m, h, s'])
//   dL/dx_m   = G_off[m] . W_off + G_z[m] . W_att           (producer_bwd_rows_kernel, MFMA)
//   dL/dref[m, l, xy] = sum over (h, p) of dL/dloc[m, h, l, p, xy]   (same kernel)
//   dL/dW     = G^T . X, dL/db = column sums of G            (producer_bwd_weights_kernel over
//               chunks of rows, then producer_bwd_reduce_kernel adds the chunks in order)
// Every sum has a fixed order, so all results are bitwise reproducible.
#include <math.h>

#include "msda_device.h"
#include "msda_producer.h"

namespace msda {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPRows = 64;              // query rows per workgroup: 4 waves x 16
constexpr int kPKc = 32;                // K elements staged per step
constexpr int kPStride = kPKc + 4;      // LDS row stride (floats) of staged K-major tiles
constexpr int kPDBlock = 256;           // grad_query columns per workgroup (16 tiles of 16)
constexpr int kPWStride = kPDBlock + 16;
constexpr int kPWCols = 64;             // weight-gradient columns per workgroup (one tile per wave)
constexpr int kPBStride = kPWCols + 16;
static_assert(kPRows == 4 * 16 && kBlock == 4 * kWave, "one 16-row MFMA tile per wave");

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Stage columns [k0, k0 + KC) of `nrows` rows of a row-major operand into
// dst (row stride `dst_stride` floats) as float32. row_ptr(r) gives the start
// of row r, or nullptr for a zero row; columns at or past `ncols` are zero.
// vec == 4: the row starts are aligned for 4-element loads and ncols % 4 == 0.
template <int KC, typename TQ, typename RowFn>
__device__ __forceinline__ void stage_rows(float* dst, int dst_stride, int nrows, int k0, int ncols, int vec,
                                           RowFn row_ptr)
{
    if (vec == 4) {
        constexpr int per_row = KC / 4;
        for (int e = threadIdx.x; e < nrows * per_row; e += kBlock) {
            const int r = e / per_row, c = (e - r * per_row) * 4;
            const TQ* p = row_ptr(r);
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (p && k0 + c < ncols) VecIO<TQ, 4>::load(p + k0 + c, v);
            *reinterpret_cast<float4*>(dst + r * dst_stride + c) = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
        for (int e = threadIdx.x; e < nrows * KC; e += kBlock) {
            const int r = e / KC, c = e - r * KC;
            const TQ* p = row_ptr(r);
            dst[r * dst_stride + c] = (p && k0 + c < ncols) ? load_f32(p + k0 + c) : 0.f;
        }
    }
}

// Row j of head h's projection matrix: the 2S offset rows, then the S logit rows.
template <typename TQ>
__device__ __forceinline__ const TQ* head_weight_row(const ProducerGeom& pg, const ProducerArgs<TQ>& a, int h, int j)
{
    const int S = pg.S;
    if (j < 2 * S) return a.w_off + (size_t)(h * 2 * S + j) * pg.D;
    if (j < 3 * S) return a.w_att + (size_t)(h * S + j - 2 * S) * pg.D;
    return nullptr;
}

// acc[t] = rows 16w..16w+15 (w = this wave) of the 64-row query tile starting
// at row m0 (rows at or past `rows_valid` read as zero) times column tile t of
// head h, summed over the D features in steps of kPKc. s_x holds kPRows and
// s_w holds 16 * ct rows of kPStride floats.
template <typename TQ>
__device__ __forceinline__ void head_projection(const ProducerGeom& pg, const ProducerArgs<TQ>& a, int m0,
                                                int rows_valid, int h, float* s_x, float* s_w,
                                                f32x4 (&acc)[kPMaxColTiles])
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int t = 0; t < kPMaxColTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < pg.D; k0 += kPKc) {
        __syncthreads();  // the previous step's tiles are consumed
        stage_rows<kPKc, TQ>(s_x, kPStride, kPRows, k0, pg.D, pg.vec, [&](int r) -> const TQ* {
            return r < rows_valid ? a.query + (size_t)(m0 + r) * pg.D : nullptr;
        });
        stage_rows<kPKc, TQ>(s_w, kPStride, 16 * pg.ct, k0, pg.D, pg.vec,
                             [&](int j) -> const TQ* { return head_weight_row(pg, a, h, j); });
        __syncthreads();
        const float* xa = s_x + (16 * wave + (lane & 15)) * kPStride + (lane >> 4);
        const float* wb = s_w + (lane & 15) * kPStride + (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < kPKc; kk += 4) {
            const float av = xa[kk];
#pragma unroll
            for (int t = 0; t < kPMaxColTiles; ++t)
                if (t < pg.ct) acc[t] = mfma_16x16x4(av, wb[t * 16 * kPStride + kk], acc[t]);
        }
    }
}

// Write the projection tile into s_o (kPRows rows of `ost` floats): MFMA
// output element v of lane l is row 4 * (l / 16) + v, column l % 16 of its tile.
__device__ __forceinline__ void store_projection(const ProducerGeom& pg, const f32x4 (&acc)[kPMaxColTiles], float* s_o,
                                                 int ost)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float* o = s_o + (16 * wave + 4 * (lane >> 4)) * ost + (lane & 15);
#pragma unroll
    for (int t = 0; t < kPMaxColTiles; ++t)
        if (t < pg.ct)
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v * ost + 16 * t] = acc[t][v];
}

// Epilogue of one head over the 64-row tile in s_o: for row r and sample j,
// emit(r, j, l, ux, uy, A) with the normalised location and the attention
// weight (softmax over the head's S logits). tpr lanes per row (tpr >= S, a
// power of two, 4..64), lane j < S holds sample j; rows at or past rows_valid
// are not emitted. ref_rows points at the reference points of row m0.
template <typename Emit>
__device__ __forceinline__ void head_outputs(const Geometry& g, const ProducerGeom& pg, const float* s_o, int ost,
                                             const float* b_off, const float* b_att, const float* ref_rows,
                                             int rows_valid, int h, Emit emit)
{
    const int S = pg.S, tpr = pg.tpr;
    const int rpp = kBlock / tpr;
    const int j = threadIdx.x & (tpr - 1);
    const bool jok = j < S;
    for (int r0 = 0; r0 < kPRows; r0 += rpp) {
        const int r = r0 + (int)threadIdx.x / tpr;
        const float* o = s_o + r * ost;
        const float z = jok ? o[2 * S + j] + (b_att ? b_att[h * S + j] : 0.f) : -INFINITY;
        float mx = z;
        for (int d = tpr >> 1; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
        const float e = jok ? expf(z - mx) : 0.f;
        float sum = e;
        for (int d = tpr >> 1; d > 0; d >>= 1) sum += __shfl_xor(sum, d, kWave);
        if (jok && r < rows_valid) {
            const int l = j / pg.Np;
            int H, W, start;
            level_of(g.lv, l, H, W, start);
            const float ox = o[2 * j] + (b_off ? b_off[h * 2 * S + 2 * j] : 0.f);
            const float oy = o[2 * j + 1] + (b_off ? b_off[h * 2 * S + 2 * j + 1] : 0.f);
            const float* rp = ref_rows + (r * pg.Nl + l) * 2;
            emit(r, j, l, rp[0] + ox / (float)W, rp[1] + oy / (float)H, e / sum);
        }
    }
}

// Store one sample's location (in the requested layout) and weight.
__device__ __forceinline__ void store_sample(const ProducerGeom& pg, int m, int h, int j, float ux, float uy, float A,
                                             float* loc, float* attn)
{
    const int idx = (m * pg.Nh + h) * pg.S + j;
    if (attn) attn[idx] = A;
    if (!loc) return;
    if (pg.b2q) {
        const int b = m / pg.Nq, q = m - b * pg.Nq;
        const int plane = pg.Nq * pg.Nh * pg.S;
        const int i = b * 2 * plane + (q * pg.Nh + h) * pg.S + j;
        loc[i] = ux;
        loc[i + plane] = uy;
    } else if (pg.loc_pair_aligned) {
        *reinterpret_cast<float2*>(loc + 2 * idx) = make_float2(ux, uy);
    } else {
        loc[2 * idx] = ux;
        loc[2 * idx + 1] = uy;
    }
}

// Row tile and head of a producer workgroup: heads fastest, so the N_h
// workgroups of one row tile run back to back on one XCD and share its L2.
__device__ __forceinline__ void producer_tile(const ProducerGeom& pg, int& m0, int& h)
{
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    h = lb % pg.Nh;
    m0 = (lb / pg.Nh) * kPRows;
}

// Dynamic LDS floats of the projection phase: the staged K tiles, later the
// output tile (aliased).
__host__ __device__ inline int projection_lds_floats(int ct)
{
    const int stage = (kPRows + 16 * ct) * kPStride;
    const int out = kPRows * (16 * ct + 4);
    return stage > out ? stage : out;
}

template <typename TQ>
__global__ __launch_bounds__(kBlock) void producer_forward_kernel(Geometry g, ProducerGeom pg, ProducerArgs<TQ> a,
                                                                  float* __restrict__ loc, float* __restrict__ attn)
{
    extern __shared__ float4 smem4[];
    float* s_x = reinterpret_cast<float*>(smem4);
    float* s_w = s_x + kPRows * kPStride;
    float* s_o = s_x;  // aliases the staging tiles once the K loop is done
    const int ost = 16 * pg.ct + 4;
    int m0, h;
    producer_tile(pg, m0, h);
    const int rows_valid = min(kPRows, pg.M - m0);
    f32x4 acc[kPMaxColTiles];
    head_projection(pg, a, m0, rows_valid, h, s_x, s_w, acc);
    __syncthreads();  // every wave is done reading the staged tiles
    store_projection(pg, acc, s_o, ost);
    __syncthreads();
    head_outputs(g, pg, s_o, ost, a.b_off, a.b_att, a.ref + (size_t)m0 * pg.Nl * 2, rows_valid, h,
                 [&](int r, int j, int, float ux, float uy, float A) {
                     store_sample(pg, m0 + r, h, j, ux, uy, A, loc, attn);
                 });
}

// Producer and forward sampler in one kernel. Workgroup = (b, h, 64
// consecutive queries); workgroups of one (b, h) slab are consecutive and
// each XCD sweeps a contiguous range of them (as in the sampler). Dynamic
// LDS: the projection phase, then the gather records of the 64 queries
// (float4 weights and FwdRecordPix, rows of S + 1 against bank conflicts).
template <typename T, int VEC>
__global__ __launch_bounds__(kBlock) void fused_forward_kernel(Geometry g, ProducerGeom pg, ProducerArgs<T> a,
                                                               const T* __restrict__ value, T* __restrict__ out,
                                                               float* __restrict__ loc, float* __restrict__ attn)
{
    extern __shared__ float4 smem4[];
    const int row = pg.S + 1;
    float4* s_rw = smem4;
    FwdRecordPix* s_rp = reinterpret_cast<FwdRecordPix*>(s_rw + kPRows * row);
    float* s_x = reinterpret_cast<float*>(s_rp + kPRows * row);
    float* s_w = s_x + kPRows * kPStride;
    float* s_o = s_x;
    const int ost = 16 * pg.ct + 4;

    const int qtiles = (g.Nq + kPRows - 1) / kPRows;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int slab = lb / qtiles;
    const int q0 = (lb - slab * qtiles) * kPRows;
    const int b = slab / g.Nh, h = slab - b * g.Nh;
    const int m0 = b * g.Nq + q0;
    const int rows_valid = min(kPRows, g.Nq - q0);

    f32x4 acc[kPMaxColTiles];
    head_projection(pg, a, m0, rows_valid, h, s_x, s_w, acc);
    __syncthreads();
    store_projection(pg, acc, s_o, ost);
    __syncthreads();
    head_outputs(g, pg, s_o, ost, a.b_off, a.b_att, a.ref + (size_t)m0 * pg.Nl * 2, rows_valid, h,
                 [&](int r, int j, int l, float ux, float uy, float A) {
                     if (loc || attn) store_sample(pg, m0 + r, h, j, ux, uy, A, loc, attn);
                     int H, W, start;
                     level_of(g.lv, l, H, W, start);
                     float4 w;
                     FwdRecordPix rp;
                     sampler_record(g, ux, uy, A, H, W, start, w, rp);
                     s_rw[r * row + j] = w;
                     s_rp[r * row + j] = rp;
                 });
    __syncthreads();

    // gather: the sampler's lane layout (VEC channels per lane, 2^lpu_log2 lanes per unit)
    const int lpu_log2 = g.lpu_log2;
    const int upb = kBlock >> lpu_log2;
    const int grp = threadIdx.x >> lpu_log2, lig = threadIdx.x & ((1 << lpu_log2) - 1);
    const int pstride = g.bnlc ? g.Ch : g.Nh * g.Ch;
    const T* slab_v = value + (g.bnlc ? (b * g.Nh + h) * g.L * g.Ch : b * g.L * g.Nh * g.Ch + h * g.Ch);
    for (int u = grp; u < rows_valid * g.chunks; u += upb) {
        const int r = u / g.chunks, chunk = u - r * g.chunks;
        const int c0 = ((chunk << lpu_log2) + lig) * VEC;
        if (c0 >= g.Ch) continue;
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = 0.f;
        gather_samples<T, VEC>(slab_v + c0, pstride, s_rw + r * row, s_rp + r * row, pg.S, o);
        VecIO<T, VEC>::store(out + ((size_t)(m0 + r) * g.Nh + h) * g.Ch + c0, o);
    }
}

// ---------------------------------------------------------------------------
// Backward.

// Loss gradients at the head's projection outputs for row m, sample j (lane j
// of a group of tpr lanes; every lane of the group must call it): the offset
// gradients gx, gy, the logit gradient gz, and the raw location gradients
// (rawx, rawy). Rows that are not valid give zeros.
__device__ __forceinline__ void head_grads(const Geometry& g, const ProducerGeom& pg, const ProducerGradIn& in,
                                           int m, bool row_ok, int h, int j, float& gx, float& gy, float& gz,
                                           float& rawx, float& rawy)
{
    const int S = pg.S;
    const bool ok = row_ok && j < S;
    const int idx = (m * pg.Nh + h) * S + j;
    const float A = ok ? in.attn[idx] : 0.f;
    const float gA = ok && in.grad_attn ? in.grad_attn[idx] : 0.f;
    float dot = A * gA;
    for (int d = pg.tpr >> 1; d > 0; d >>= 1) dot += __shfl_xor(dot, d, kWave);
    gz = A * (gA - dot);
    rawx = rawy = 0.f;
    if (ok && in.grad_loc) {
        if (pg.b2q) {
            const int b = m / pg.Nq, q = m - b * pg.Nq;
            const int plane = pg.Nq * pg.Nh * S;
            const int i = b * 2 * plane + (q * pg.Nh + h) * S + j;
            rawx = in.grad_loc[i];
            rawy = in.grad_loc[i + plane];
        } else {
            rawx = in.grad_loc[2 * idx];
            rawy = in.grad_loc[2 * idx + 1];
        }
    }
    int H = 1, W = 1, start;
    if (ok) level_of(g.lv, j / pg.Np, H, W, start);
    gx = rawx / (float)W;
    gy = rawy / (float)H;
}

// grad_query (MFMA: G tile x W) and grad_reference_points. Grid: row tiles x
// column blocks of kPDBlock. Dynamic LDS: the head's gradient tile s_g
// (kPRows x gst), a 16-row slice of W (16 x kPWStride), and the location
// gradient sums s_ref (kPRows x 2S).
template <typename TQ>
__global__ __launch_bounds__(kBlock) void producer_bwd_rows_kernel(Geometry g, ProducerGeom pg, ProducerArgs<TQ> a,
                                                                   ProducerGradIn in, TQ* __restrict__ grad_query,
                                                                   float* __restrict__ grad_ref)
{
    extern __shared__ float4 smem4[];
    const int gst = 16 * pg.ct + 4;
    float* s_g = reinterpret_cast<float*>(smem4);
    float* s_wk = s_g + kPRows * gst;
    float* s_ref = s_wk + 16 * kPWStride;
    const int S = pg.S;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nmt = (pg.M + kPRows - 1) / kPRows;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int db = lb / nmt, m0 = (lb - db * nmt) * kPRows;
    const int d0 = db * kPDBlock;
    const int rows_valid = min(kPRows, pg.M - m0);
    const int dtiles = min(16, (min(kPDBlock, pg.D - d0) + 15) / 16);
    const bool do_ref = grad_ref && db == 0;

    for (int i = tid; i < kPRows * gst; i += kBlock) s_g[i] = 0.f;  // padding columns stay zero
    f32x4 acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int tpr = pg.tpr, rpp = kBlock / tpr, j = tid & (tpr - 1);
    for (int h = 0; h < pg.Nh; ++h) {
        __syncthreads();  // s_g is free
        for (int r0 = 0; r0 < kPRows; r0 += rpp) {
            const int r = r0 + tid / tpr;
            float gx, gy, gz, rx, ry;
            head_grads(g, pg, in, m0 + r, r < rows_valid, h, j, gx, gy, gz, rx, ry);
            if (j < S) {
                s_g[r * gst + 2 * j] = gx;
                s_g[r * gst + 2 * j + 1] = gy;
                s_g[r * gst + 2 * S + j] = gz;
                if (do_ref) {
                    // this thread owns (r, j) for every head: sums over h in order
                    float* sr = s_ref + r * 2 * S + 2 * j;
                    sr[0] = h == 0 ? rx : sr[0] + rx;
                    sr[1] = h == 0 ? ry : sr[1] + ry;
                }
            }
        }
        if (!grad_query) continue;
        for (int kc = 0; kc < pg.ct; ++kc) {
            __syncthreads();  // s_g written / previous W slice consumed
            stage_rows<kPDBlock, TQ>(s_wk, kPWStride, 16, d0, pg.D, pg.vec, [&](int i) -> const TQ* {
                return head_weight_row(pg, a, h, kc * 16 + i);
            });
            __syncthreads();
            const float* ga = s_g + (16 * wave + (lane & 15)) * gst + kc * 16 + (lane >> 4);
            const float* wb = s_wk + (lane >> 4) * kPWStride + (lane & 15);
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4) {
                const float av = ga[kk];
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    if (t < dtiles) acc[t] = mfma_16x16x4(av, wb[kk * kPWStride + 16 * t], acc[t]);
            }
        }
    }
    if (grad_query) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int d = d0 + 16 * t + (lane & 15);
            if (t >= dtiles || d >= pg.D) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * wave + 4 * (lane >> 4) + v;
                if (m < pg.M) store_f32(grad_query + (size_t)m * pg.D + d, acc[t][v]);
            }
        }
    }
    if (do_ref) {
        __syncthreads();
        const int per_row = pg.Nl * 2;
        for (int e = tid; e < rows_valid * per_row; e += kBlock) {
            const int r = e / per_row, lx = e - r * per_row;
            const int l = lx >> 1, xy = lx & 1;
            const float* sr = s_ref + r * 2 * S + 2 * l * pg.Np + xy;
            float s = 0.f;
            for (int p = 0; p < pg.Np; ++p) s += sr[2 * p];
            grad_ref[(size_t)(m0 + r) * per_row + lx] = s;
        }
    }
}

// Partial weight and bias gradients of one chunk of rows: for head h and
// columns [d0, d0 + kPWCols) of the features, part_w[chunk][h][n][d] =
// sum over the chunk's rows m of G[m, h, n] * x_m[d] (n over the head's 3S
// projection outputs), part_b[chunk][h][n] = sum of G[m, h, n]. Grid:
// (chunk, head, column block) with column blocks fastest. Dynamic LDS: G^T
// (16 * ct rows x kPStride) and the query rows (kPKc x kPBStride).
template <typename TQ>
__global__ __launch_bounds__(kBlock) void producer_bwd_weights_kernel(Geometry g, ProducerGeom pg, ProducerArgs<TQ> a,
                                                                      ProducerGradIn in, float* __restrict__ part_w,
                                                                      float* __restrict__ part_b)
{
    extern __shared__ float4 smem4[];
    float* s_a = reinterpret_cast<float*>(smem4);
    float* s_b = s_a + 16 * pg.ct * kPStride;
    const int S = pg.S, cols = 3 * S;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int ndb = (pg.D + kPWCols - 1) / kPWCols;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int db = lb % ndb;
    const int h = (lb / ndb) % pg.Nh;
    const int mc = lb / (ndb * pg.Nh);
    const int d0 = db * kPWCols;
    const int mbeg = mc * pg.mrows, mend = min(pg.M, mbeg + pg.mrows);

    for (int i = tid; i < 16 * pg.ct * kPStride; i += kBlock) s_a[i] = 0.f;  // padding rows stay zero
    f32x4 acc[kPMaxColTiles];
#pragma unroll
    for (int t = 0; t < kPMaxColTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bsum = 0.f;
    const int tpr = pg.tpr, rpp = kBlock / tpr, j = tid & (tpr - 1);
    for (int mm0 = mbeg; mm0 < mend; mm0 += kPKc) {
        __syncthreads();  // previous step consumed
        for (int r0 = 0; r0 < kPKc; r0 += rpp) {
            // with rpp > kPKc the groups past the step's rows still join the shuffles
            const int r = r0 + tid / tpr;
            const bool in_step = r < kPKc;
            float gx, gy, gz, rx, ry;
            head_grads(g, pg, in, mm0 + r, in_step && mm0 + r < mend, h, j, gx, gy, gz, rx, ry);
            if (in_step && j < S) {
                s_a[(2 * j) * kPStride + r] = gx;
                s_a[(2 * j + 1) * kPStride + r] = gy;
                s_a[(2 * S + j) * kPStride + r] = gz;
            }
        }
        stage_rows<kPWCols, TQ>(s_b, kPBStride, kPKc, d0, pg.D, pg.vec, [&](int r) -> const TQ* {
            return mm0 + r < mend ? a.query + (size_t)(mm0 + r) * pg.D : nullptr;
        });
        __syncthreads();
        const float* ab = s_a + (lane & 15) * kPStride + (lane >> 4);
        const float* xb = s_b + (lane >> 4) * kPBStride + 16 * wave + (lane & 15);
#pragma unroll
        for (int kk = 0; kk < kPKc; kk += 4) {
            const float bv = xb[kk * kPBStride];
#pragma unroll
            for (int t = 0; t < kPMaxColTiles; ++t)
                if (t < pg.ct) acc[t] = mfma_16x16x4(ab[t * 16 * kPStride + kk], bv, acc[t]);
        }
        if (db == 0 && tid < cols) {
            const float* ar = s_a + tid * kPStride;
            for (int r = 0; r < kPKc; ++r) bsum += ar[r];
        }
    }
    const size_t base = ((size_t)mc * pg.Nh + h) * cols;
    const int d = d0 + 16 * wave + (lane & 15);
#pragma unroll
    for (int t = 0; t < kPMaxColTiles; ++t) {
        if (t >= pg.ct) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int n = 16 * t + 4 * (lane >> 4) + v;
            if (n < cols && d < pg.D) part_w[(base + n) * pg.D + d] = acc[t][v];
        }
    }
    if (db == 0 && tid < cols) part_b[base + tid] = bsum;
}

// Sum the row chunks' partial gradients in chunk order and scatter them into
// grad_offset_weight / grad_attention_weight and the two bias gradients.
__global__ __launch_bounds__(kBlock) void producer_bwd_reduce_kernel(ProducerGeom pg, const float* __restrict__ part_w,
                                                                     const float* __restrict__ part_b,
                                                                     float* __restrict__ gw_off, float* __restrict__ gb_off,
                                                                     float* __restrict__ gw_att, float* __restrict__ gb_att)
{
    const int S = pg.S, cols = 3 * S;
    const int nw = pg.Nh * cols * pg.D, nb = pg.Nh * cols;
    const int e = blockIdx.x * kBlock + threadIdx.x;
    if (e < nw) {
        if (!gw_off && !gw_att) return;
        float s = 0.f;
        for (int c = 0; c < pg.mchunks; ++c) s += part_w[(size_t)c * nw + e];
        const int hn = e / pg.D, d = e - hn * pg.D;
        const int h = hn / cols, n = hn - h * cols;
        if (n < 2 * S) {
            if (gw_off) gw_off[(size_t)(h * 2 * S + n) * pg.D + d] = s;
        } else if (gw_att) {
            gw_att[(size_t)(h * S + n - 2 * S) * pg.D + d] = s;
        }
    } else if (e < nw + nb) {
        if (!gb_off && !gb_att) return;
        const int i = e - nw;
        float s = 0.f;
        for (int c = 0; c < pg.mchunks; ++c) s += part_b[(size_t)c * nb + i];
        const int h = i / cols, n = i - h * cols;
        if (n < 2 * S) {
            if (gb_off) gb_off[h * 2 * S + n] = s;
        } else if (gb_att) {
            gb_att[h * S + n - 2 * S] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Host launchers.

size_t producer_forward_lds(const ProducerGeom& pg) { return (size_t)projection_lds_floats(pg.ct) * sizeof(float); }

size_t fused_forward_lds(const ProducerGeom& pg)
{
    return (size_t)kPRows * (pg.S + 1) * (sizeof(float4) + sizeof(FwdRecordPix)) + producer_forward_lds(pg);
}

size_t producer_bwd_rows_lds(const ProducerGeom& pg)
{
    return ((size_t)kPRows * (16 * pg.ct + 4) + 16 * kPWStride + (size_t)kPRows * 2 * pg.S) * sizeof(float);
}

size_t producer_bwd_weights_lds(const ProducerGeom& pg)
{
    return ((size_t)16 * pg.ct * kPStride + (size_t)kPKc * kPBStride) * sizeof(float);
}

size_t producer_bwd_workspace_floats(const ProducerGeom& pg)
{
    return (size_t)pg.mchunks * pg.Nh * 3 * pg.S * ((size_t)pg.D + 1);
}

int producer_row_tiles(int M) { return (M + kPRows - 1) / kPRows; }
int producer_grad_query_blocks(int D) { return (D + kPDBlock - 1) / kPDBlock; }
int producer_weight_col_blocks(int D) { return (D + kPWCols - 1) / kPWCols; }

template <typename TQ>
static ProducerArgs<TQ> typed(const ProducerArgsRaw& r)
{
    return ProducerArgs<TQ>{static_cast<const TQ*>(r.query), r.ref, static_cast<const TQ*>(r.w_off), r.b_off,
                            static_cast<const TQ*>(r.w_att), r.b_att};
}

hipError_t launch_producer_forward(const Geometry& g, const ProducerGeom& pg, int bf16, const ProducerArgsRaw& a,
                                   float* loc, float* attn, hipStream_t stream)
{
    const dim3 grid(producer_row_tiles(pg.M) * pg.Nh);
    const size_t lds = producer_forward_lds(pg);
    if (bf16)
        hipLaunchKernelGGL(producer_forward_kernel<uint16_t>, grid, dim3(kBlock), lds, stream, g, pg,
                           typed<uint16_t>(a), loc, attn);
    else
        hipLaunchKernelGGL(producer_forward_kernel<float>, grid, dim3(kBlock), lds, stream, g, pg, typed<float>(a),
                           loc, attn);
    return hipGetLastError();
}

template <typename T, int VEC>
static hipError_t launch_fused_t(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& a, const void* value,
                                 void* out, float* loc, float* attn, hipStream_t stream)
{
    const int qtiles = (g.Nq + kPRows - 1) / kPRows;
    const dim3 grid(g.B * g.Nh * qtiles);
    hipLaunchKernelGGL((fused_forward_kernel<T, VEC>), grid, dim3(kBlock), fused_forward_lds(pg), stream, g, pg,
                       typed<T>(a), static_cast<const T*>(value), static_cast<T*>(out), loc, attn);
    return hipGetLastError();
}

hipError_t launch_fused_forward(const Geometry& g, const ProducerGeom& pg, int bf16, int vec, const ProducerArgsRaw& a,
                                const void* value, void* out, float* loc, float* attn, hipStream_t stream)
{
    if (bf16) {
        switch (vec) {
        case 8: return launch_fused_t<uint16_t, 8>(g, pg, a, value, out, loc, attn, stream);
        case 4: return launch_fused_t<uint16_t, 4>(g, pg, a, value, out, loc, attn, stream);
        case 2: return launch_fused_t<uint16_t, 2>(g, pg, a, value, out, loc, attn, stream);
        default: return launch_fused_t<uint16_t, 1>(g, pg, a, value, out, loc, attn, stream);
        }
    }
    switch (vec) {
    case 4: return launch_fused_t<float, 4>(g, pg, a, value, out, loc, attn, stream);
    case 2: return launch_fused_t<float, 2>(g, pg, a, value, out, loc, attn, stream);
    default: return launch_fused_t<float, 1>(g, pg, a, value, out, loc, attn, stream);
    }
}

template <typename TQ>
static hipError_t launch_producer_backward_t(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& ar,
                                             const ProducerGradIn& in, const ProducerGradOut& o, float* part,
                                             hipStream_t stream)
{
    const ProducerArgs<TQ> a = typed<TQ>(ar);
    if (o.grad_query || o.grad_ref) {
        const dim3 grid(producer_row_tiles(pg.M) * producer_grad_query_blocks(pg.D));
        hipLaunchKernelGGL(producer_bwd_rows_kernel<TQ>, grid, dim3(kBlock), producer_bwd_rows_lds(pg), stream, g, pg,
                           a, in, static_cast<TQ*>(o.grad_query), o.grad_ref);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (o.grad_w_off || o.grad_b_off || o.grad_w_att || o.grad_b_att) {
        float* part_w = part;
        float* part_b = part + (size_t)pg.mchunks * pg.Nh * 3 * pg.S * pg.D;
        const dim3 grid(pg.mchunks * pg.Nh * producer_weight_col_blocks(pg.D));
        hipLaunchKernelGGL(producer_bwd_weights_kernel<TQ>, grid, dim3(kBlock), producer_bwd_weights_lds(pg), stream,
                           g, pg, a, in, part_w, part_b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int n = pg.Nh * 3 * pg.S * (pg.D + 1);
        hipLaunchKernelGGL(producer_bwd_reduce_kernel, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, stream, pg,
                           part_w, part_b, o.grad_w_off, o.grad_b_off, o.grad_w_att, o.grad_b_att);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_producer_backward(const Geometry& g, const ProducerGeom& pg, int bf16, const ProducerArgsRaw& a,
                                    const ProducerGradIn& in, const ProducerGradOut& o, void* workspace,
                                    hipStream_t stream)
{
    float* part = static_cast<float*>(workspace);
    return bf16 ? launch_producer_backward_t<uint16_t>(g, pg, a, in, o, part, stream)
                : launch_producer_backward_t<float>(g, pg, a, in, o, part, stream);
}

}  // namespace msda
