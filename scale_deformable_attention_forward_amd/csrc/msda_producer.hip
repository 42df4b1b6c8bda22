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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kPRows = 64;              // query rows per workgroup: 4 waves x 16
constexpr int kPKc = 32;                // K elements staged per step
constexpr int kPStride = kPKc + 4;      // LDS row stride (floats) of staged K-major tiles
constexpr int kPDBlock = 256;           // grad_query columns per workgroup (16 tiles of 16)
constexpr int kPWStride = kPDBlock + 16;
constexpr int kPWCols = 64;             // weight-gradient columns per workgroup (one tile per wave)
constexpr int kPBStride = kPWCols + 16;
constexpr int kPMStep = 32;             // rows per step of the weight-gradient pass
constexpr int kPMStride = kPMStep + 4;  // LDS row stride (floats) of its transposed gradient tile
static_assert(kPRows == 4 * 16 && kBlock == 4 * kWave, "one 16-row MFMA tile per wave");

__device__ __forceinline__ f32x4 mfma_16x16x4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bfloat16 operands, float32 accumulation: lane l supplies row l % 16 of A
// and column l % 16 of B at k = 8 * (l / 16) .. + 7 (the products are exact
// in float32); the output layout is mfma_16x16x4's (checked with an
// in-bounds probe).
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
constexpr int kPHStride = kPKc + 8;  // LDS row stride (bfloat16 elements) of staged bfloat16 tiles

// Per-(row, sample) loops run tpr lanes per row and kBlock / tpr rows per
// pass; a tile of kPRows rows takes at most this many passes (tpr <= 16, 32,
// 64 for 3, 6, 12 column tiles).
template <int CTM>
constexpr int max_passes()
{
    return 4 * CTM / 3;
}

// Four consecutive elements of an operand row, as loaded from memory.
template <typename TQ> struct Quad;
template <> struct Quad<float> {
    float4 v;
};
template <> struct Quad<uint16_t> {
    uint2 v;
};

__device__ __forceinline__ float4 to_float4(const Quad<float>& q) { return q.v; }
__device__ __forceinline__ float4 to_float4(const Quad<uint16_t>& q)
{
    return make_float4(__uint_as_float(q.v.x << 16), __uint_as_float(q.v.x & 0xffff0000u),
                       __uint_as_float(q.v.y << 16), __uint_as_float(q.v.y & 0xffff0000u));
}

// Elements c..c+3 of `row` (nullptr: a zero row); columns at or past ncols
// read 0. vec == 4: one vector load (row + c aligned, ncols % 4 == 0).
__device__ __forceinline__ Quad<float> load_quad(const float* row, int c, int ncols, int vec)
{
    Quad<float> q{make_float4(0.f, 0.f, 0.f, 0.f)};
    if (!row || c >= ncols) return q;
    if (vec == 4) {
        q.v = *reinterpret_cast<const float4*>(row + c);
    } else {
        q.v.x = row[c];
        if (c + 1 < ncols) q.v.y = row[c + 1];
        if (c + 2 < ncols) q.v.z = row[c + 2];
        if (c + 3 < ncols) q.v.w = row[c + 3];
    }
    return q;
}

__device__ __forceinline__ Quad<uint16_t> load_quad(const uint16_t* row, int c, int ncols, int vec)
{
    Quad<uint16_t> q{make_uint2(0u, 0u)};
    if (!row || c >= ncols) return q;
    if (vec == 4) {
        q.v = *reinterpret_cast<const uint2*>(row + c);
    } else {
        uint32_t e[4] = {row[c], 0u, 0u, 0u};
        if (c + 1 < ncols) e[1] = row[c + 1];
        if (c + 2 < ncols) e[2] = row[c + 2];
        if (c + 3 < ncols) e[3] = row[c + 3];
        q.v = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
    }
    return q;
}

// A tile of rows x (4 * PR) columns of a row-major operand held in
// registers: quad i of a thread is element e = threadIdx.x + i * kBlock of the
// tile, row e / PR, columns 4 * (e % PR) .. + 3. load() issues every load
// before any is used, so a tile costs one memory round trip; store() writes
// it to LDS as float32.
template <typename TQ, int NQ, int PR>
struct TileRegs {
    Quad<TQ> q[NQ];

    // row_ptr(r): start of row r or nullptr (zero row); columns k0.. of the rows
    template <typename RowFn>
    __device__ __forceinline__ void load(int nrows, int k0, int ncols, int vec, RowFn row_ptr)
    {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = threadIdx.x + i * kBlock;
            const int r = e / PR, c = k0 + (e - r * PR) * 4;
            q[i] = load_quad(r < nrows ? row_ptr(r) : nullptr, c, ncols, vec);
        }
    }

    __device__ __forceinline__ void store(float* dst, int stride, int nrows) const
    {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = threadIdx.x + i * kBlock;
            const int r = e / PR, c = (e - r * PR) * 4;
            if (r < nrows) *reinterpret_cast<float4*>(dst + r * stride + c) = to_float4(q[i]);
        }
    }

    // bfloat16 operands kept as they are (stride in elements)
    __device__ __forceinline__ void store_raw(uint16_t* dst, int stride, int nrows) const
    {
        static_assert(sizeof(Quad<TQ>) == 8, "raw stores are for bfloat16 tiles");
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = threadIdx.x + i * kBlock;
            const int r = e / PR, c = (e - r * PR) * 4;
            if (r < nrows) *reinterpret_cast<uint2*>(dst + r * stride + c) = q[i].v;
        }
    }
};

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
// head h, summed over the D features kPKc at a time. The next step's operands
// are loaded into registers while the matrix cores work on the current one.
// s_x holds kPRows and s_w 16 * ct rows of kPStride floats.
template <typename TQ, int CTM>
__device__ __forceinline__ void head_projection(const ProducerGeom& pg, const ProducerArgs<TQ>& a, int m0,
                                                int rows_valid, int h, float* s_x, float* s_w, f32x4 (&acc)[CTM])
{
    constexpr int PR = kPKc / 4;
    constexpr int XQ = kPRows * PR / kBlock;
    constexpr int WQ = (16 * CTM * PR + kBlock - 1) / kBlock;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    constexpr int wrows = 16 * CTM;
    auto xrow = [&](int r) -> const TQ* { return r < rows_valid ? a.query + (size_t)(m0 + r) * pg.D : nullptr; };
    auto wrow = [&](int j) -> const TQ* { return head_weight_row(pg, a, h, j); };
    TileRegs<TQ, XQ, PR> xr;
    TileRegs<TQ, WQ, PR> wr;
    xr.load(kPRows, 0, pg.D, pg.vec, xrow);
    wr.load(wrows, 0, pg.D, pg.vec, wrow);
#pragma unroll
    for (int t = 0; t < CTM; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(TQ) == 2) {
        // bfloat16 inputs: staged as they are, one 16x16x32 bfloat16 MFMA per
        // column tile and step (a lane's 8 A and 8 B elements are one 16-byte
        // LDS read each)
        uint16_t* hx = reinterpret_cast<uint16_t*>(s_x);
        uint16_t* hw = reinterpret_cast<uint16_t*>(s_w);
        const bf16x8* xa = reinterpret_cast<const bf16x8*>(hx + (16 * wave + (lane & 15)) * kPHStride + 8 * (lane >> 4));
        const uint16_t* wb = hw + (lane & 15) * kPHStride + 8 * (lane >> 4);
        for (int k0 = 0; k0 < pg.D; k0 += kPKc) {
            __syncthreads();  // the previous step's tiles are consumed
            xr.store_raw(hx, kPHStride, kPRows);
            wr.store_raw(hw, kPHStride, wrows);
            __syncthreads();
            if (k0 + kPKc < pg.D) {
                xr.load(kPRows, k0 + kPKc, pg.D, pg.vec, xrow);
                wr.load(wrows, k0 + kPKc, pg.D, pg.vec, wrow);
            }
            const bf16x8 av = *xa;
#pragma unroll
            for (int t = 0; t < CTM; ++t)
                acc[t] = mfma_16x16x32_bf16(av, *reinterpret_cast<const bf16x8*>(wb + t * 16 * kPHStride), acc[t]);
        }
        return;
    }
    const float* xa = s_x + (16 * wave + (lane & 15)) * kPStride + (lane >> 4);
    const float* wb = s_w + (lane & 15) * kPStride + (lane >> 4);
    for (int k0 = 0; k0 < pg.D; k0 += kPKc) {
        __syncthreads();  // the previous step's tiles are consumed
        xr.store(s_x, kPStride, kPRows);
        wr.store(s_w, kPStride, wrows);
        __syncthreads();
        if (k0 + kPKc < pg.D) {
            xr.load(kPRows, k0 + kPKc, pg.D, pg.vec, xrow);
            wr.load(wrows, k0 + kPKc, pg.D, pg.vec, wrow);
        }
#pragma unroll
        for (int kk = 0; kk < kPKc; kk += 4) {
            const float av = xa[kk];
#pragma unroll
            for (int t = 0; t < CTM; ++t) acc[t] = mfma_16x16x4(av, wb[t * 16 * kPStride + kk], acc[t]);
        }
    }
}

// Write the projection tile into s_o (kPRows rows of `ost` floats): MFMA
// output element v of lane l is row 4 * (l / 16) + v, column l % 16 of its tile.
template <int CTM>
__device__ __forceinline__ void store_projection(const ProducerGeom& pg, const f32x4 (&acc)[CTM], float* s_o, int ost)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float* o = s_o + (16 * wave + 4 * (lane >> 4)) * ost + (lane & 15);
#pragma unroll
    for (int t = 0; t < CTM; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v * ost + 16 * t] = acc[t][v];
}

// Epilogue of one head over the 64-row tile in s_o: for row r and sample j,
// emit(r, j, l, ux, uy, A) with the normalised location and the attention
// weight (softmax over the head's S logits). tpr lanes per row (tpr >= S, a
// power of two, 4..64), lane j < S holds sample j; rows at or past rows_valid
// are not emitted. ref_rows points at the reference points of row m0.
// Two phases: HeadOut::load copies the thread's projection outputs (and its
// biases and reference points) into registers, so the caller may reuse the
// LDS of s_o after a barrier; HeadOut::finish computes and emits.
template <int CTM>
struct HeadOut {
    static constexpr int PMAX = max_passes<CTM>();
    float ox[PMAX], oy[PMAX], oz[PMAX], rx[PMAX], ry[PMAX];
    int l, W, H;

    __device__ __forceinline__ void load(const Geometry& g, const ProducerGeom& pg, const float* s_o, int ost,
                                         const float* b_off, const float* b_att, const float* ref_rows,
                                         int rows_valid, int h)
    {
        const int S = pg.S, tpr = pg.tpr;
        const int rpp = kBlock / tpr, passes = kPRows / rpp;
        const int j = threadIdx.x & (tpr - 1), r_in = (int)threadIdx.x / tpr;
        const bool jok = j < S;
        l = jok ? j / pg.Np : 0;
        int start;
        level_of(g.lv, l, H, W, start);
        const float bx = jok && b_off ? b_off[h * 2 * S + 2 * j] : 0.f;
        const float by = jok && b_off ? b_off[h * 2 * S + 2 * j + 1] : 0.f;
        const float bz = jok && b_att ? b_att[h * S + j] : 0.f;
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
            const int r = p * rpp + r_in;
            const bool ok = p < passes && jok && r < rows_valid;
            rx[p] = ok ? ref_rows[(r * pg.Nl + l) * 2] : 0.f;
            ry[p] = ok ? ref_rows[(r * pg.Nl + l) * 2 + 1] : 0.f;
            const float* o = s_o + min(r, kPRows - 1) * ost;
            ox[p] = p < passes && jok ? o[2 * j] + bx : 0.f;
            oy[p] = p < passes && jok ? o[2 * j + 1] + by : 0.f;
            oz[p] = p < passes && jok ? o[2 * S + j] + bz : -INFINITY;
        }
    }

    template <typename Emit>
    __device__ __forceinline__ void finish(const ProducerGeom& pg, int rows_valid, Emit emit) const
    {
        const int S = pg.S, tpr = pg.tpr;
        const int rpp = kBlock / tpr, passes = kPRows / rpp;
        const int j = threadIdx.x & (tpr - 1), r_in = (int)threadIdx.x / tpr;
        const bool jok = j < S;
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
            if (p < passes) {  // uniform
                const int r = p * rpp + r_in;
                float mx = oz[p];
                for (int d = tpr >> 1; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, kWave));
                const float e = jok ? expf(oz[p] - mx) : 0.f;
                float sum = e;
                for (int d = tpr >> 1; d > 0; d >>= 1) sum += __shfl_xor(sum, d, kWave);
                if (jok && r < rows_valid)
                    emit(r, j, l, rx[p] + ox[p] / (float)W, ry[p] + oy[p] / (float)H, e / sum);
            }
        }
    }
};

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

// Dynamic LDS floats of the projection phase: the staged K tiles, later the
// output tile (aliased).
__host__ __device__ inline int projection_lds_floats(int ct)
{
    const int stage = (kPRows + 16 * ct) * kPStride;
    const int out = kPRows * (16 * ct + 4);
    return stage > out ? stage : out;
}

// Grid: row tiles x heads with heads fastest, so the N_h workgroups of one row
// tile run back to back on one XCD and share its L2.
template <typename TQ, int CTM>
__global__ __launch_bounds__(kBlock) void producer_forward_kernel(Geometry g, ProducerGeom pg, ProducerArgs<TQ> a,
                                                                  float* __restrict__ loc, float* __restrict__ attn)
{
    extern __shared__ float4 smem4[];
    float* s_x = reinterpret_cast<float*>(smem4);
    float* s_w = s_x + kPRows * kPStride;
    float* s_o = s_x;  // aliases the staging tiles once the K loop is done
    constexpr int ost = 16 * CTM + 4;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int h = lb % pg.Nh, m0 = (lb / pg.Nh) * kPRows;
    const int rows_valid = min(kPRows, pg.M - m0);
    f32x4 acc[CTM];
    head_projection<TQ, CTM>(pg, a, m0, rows_valid, h, s_x, s_w, acc);
    __syncthreads();  // every wave is done reading the staged tiles
    store_projection<CTM>(pg, acc, s_o, ost);
    __syncthreads();
    HeadOut<CTM> ho;
    ho.load(g, pg, s_o, ost, a.b_off, a.b_att, a.ref + (size_t)m0 * pg.Nl * 2, rows_valid, h);
    ho.finish(pg, rows_valid, [&](int r, int j, int, float ux, float uy, float A) {
        store_sample(pg, m0 + r, h, j, ux, uy, A, loc, attn);
    });
}

// Producer and forward sampler in one kernel. Workgroup = (b, h, 64
// consecutive queries); workgroups of one (b, h) slab are consecutive and
// each XCD sweeps a contiguous range of them (as in the sampler). Dynamic
// LDS: the projection phase, then (over the same bytes, once the epilogue
// holds its inputs in registers) the gather records of the 64 queries
// (FwdRecord, rows of S + 1 against bank conflicts).
template <typename T, int VEC, int CTM, bool BUF>
__global__ __launch_bounds__(kBlock) void fused_forward_kernel(Geometry g, ProducerGeom pg, ProducerArgs<T> a,
                                                               int64_t value_bytes, const T* __restrict__ value,
                                                               T* __restrict__ out, float* __restrict__ loc,
                                                               float* __restrict__ attn)
{
    extern __shared__ float4 smem4[];
    const int row = pg.S + 1;
    FwdRecord* s_rec = reinterpret_cast<FwdRecord*>(smem4);
    float* s_x = reinterpret_cast<float*>(smem4);
    float* s_w = s_x + kPRows * kPStride;
    float* s_o = s_x;
    constexpr int ost = 16 * CTM + 4;

    const int qtiles = (g.Nq + kPRows - 1) / kPRows;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int slab = lb / qtiles;
    const int q0 = (lb - slab * qtiles) * kPRows;
    const int b = slab / g.Nh, h = slab - b * g.Nh;
    const int m0 = b * g.Nq + q0;
    const int rows_valid = min(kPRows, g.Nq - q0);

    f32x4 acc[CTM];
    head_projection<T, CTM>(pg, a, m0, rows_valid, h, s_x, s_w, acc);
    __syncthreads();
    store_projection<CTM>(pg, acc, s_o, ost);
    __syncthreads();
    HeadOut<CTM> ho;
    ho.load(g, pg, s_o, ost, a.b_off, a.b_att, a.ref + (size_t)m0 * pg.Nl * 2, rows_valid, h);
    __syncthreads();  // s_o is in registers: the records take its place
    const int slab_off = g.bnlc ? (b * g.Nh + h) * g.L * g.Ch : b * g.L * g.Nh * g.Ch + h * g.Ch;
    ho.finish(pg, rows_valid, [&](int r, int j, int l, float ux, float uy, float A) {
        if (loc || attn) store_sample(pg, m0 + r, h, j, ux, uy, A, loc, attn);
        int H, W, start;
        level_of(g.lv, l, H, W, start);
        sampler_record<T, BUF>(g, ux, uy, A, H, W, start, slab_off, s_rec[r * row + j]);
    });
    __syncthreads();

    // gather: the sampler's lane layout (VEC channels per lane, 2^lpu_log2 lanes per unit)
    const int lpu_log2 = g.lpu_log2;
    const int upb = kBlock >> lpu_log2;
    const int grp = threadIdx.x >> lpu_log2, lig = threadIdx.x & ((1 << lpu_log2) - 1);
    const __amdgpu_buffer_rsrc_t vr = value_rsrc(value, BUF ? value_bytes : 0);
    for (int u = grp; u < rows_valid * g.chunks; u += upb) {
        const int r = u / g.chunks, chunk = u - r * g.chunks;
        const int c0 = ((chunk << lpu_log2) + lig) * VEC;
        if (c0 >= g.Ch) continue;
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = 0.f;
        gather_samples<T, VEC, BUF>(value, vr, c0, s_rec + r * row, pg.S, o);
        VecIO<T, VEC>::store(out + ((size_t)(m0 + r) * g.Nh + h) * g.Ch + c0, o);
    }
}

// ---------------------------------------------------------------------------
// Backward.

// What one (row, sample) lane reads for the gradient at the head's
// projection outputs: A, dL/dA and dL/dloc (x, y). Invalid lanes read zeros.
struct GradIn {
    float A, gA, lx, ly;
};

__device__ __forceinline__ GradIn load_grad_in(const ProducerGeom& pg, const ProducerGradIn& in, int m, bool ok, int h,
                                               int j)
{
    GradIn r = {0.f, 0.f, 0.f, 0.f};
    if (!ok) return r;
    const int S = pg.S;
    const int idx = (m * pg.Nh + h) * S + j;
    r.A = in.attn[idx];
    if (in.grad_attn) r.gA = in.grad_attn[idx];
    if (in.grad_loc) {
        if (pg.b2q) {
            const int b = m / pg.Nq, q = m - b * pg.Nq;
            const int plane = pg.Nq * pg.Nh * S;
            const int i = b * 2 * plane + (q * pg.Nh + h) * S + j;
            r.lx = in.grad_loc[i];
            r.ly = in.grad_loc[i + plane];
        } else {
            r.lx = in.grad_loc[2 * idx];
            r.ly = in.grad_loc[2 * idx + 1];
        }
    }
    return r;
}

// Gradients at the projection outputs from what load_grad_in read: offsets
// gx = dL/dloc_x / W, gy = dL/dloc_y / H, logit gz = A (dL/dA - sum over the
// head's samples of A dL/dA). Every lane of the tpr-lane group must call it
// (the sum is a butterfly over the group). inv_w, inv_h: the lane's level size.
__device__ __forceinline__ void finish_grads(const GradIn& r, int tpr, float W, float H, float& gx, float& gy, float& gz)
{
    float dot = r.A * r.gA;
    for (int d = tpr >> 1; d > 0; d >>= 1) dot += __shfl_xor(dot, d, kWave);
    gz = r.A * (r.gA - dot);
    gx = r.lx / W;
    gy = r.ly / H;
}

// grad_query (MFMA: gradient tile x W) and grad_reference_points. Grid: row
// tiles x column blocks of kPDBlock. Dynamic LDS: the head's gradient tile s_g
// (kPRows x gst), a 16-row slice of W (16 x kPWStride), and the location
// gradient sums s_ref (kPRows x 2S). The next head's inputs and the next W
// slice are loaded while the matrix cores work on the current ones.
template <typename TQ, int CTM>
__global__ __launch_bounds__(kBlock) void producer_bwd_rows_kernel(Geometry g, ProducerGeom pg, ProducerArgs<TQ> a,
                                                                   ProducerGradIn in, TQ* __restrict__ grad_query,
                                                                   float* __restrict__ grad_ref)
{
    constexpr int PMAX = max_passes<CTM>();
    constexpr int PR = kPDBlock / 4;
    constexpr int WQ = 16 * PR / kBlock;
    extern __shared__ float4 smem4[];
    constexpr int gst = 16 * CTM + 4;
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
    const bool do_ref = grad_ref && db == 0;
    const int tpr = pg.tpr, rpp = kBlock / tpr, passes = kPRows / rpp;
    const int j = tid & (tpr - 1), r_in = tid / tpr;
    const bool jok = j < S;
    int H = 1, W = 1, start;
    if (jok) level_of(g.lv, j / pg.Np, H, W, start);

    for (int i = tid; i < kPRows * gst; i += kBlock) s_g[i] = 0.f;  // padding columns stay zero
    f32x4 acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    GradIn gin[PMAX];
    auto load_head = [&](int h) {
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
            const int r = p * rpp + r_in;
            gin[p] = load_grad_in(pg, in, m0 + r, p < passes && jok && r < rows_valid, h, j);
        }
    };
    TileRegs<TQ, WQ, PR> wr;
    auto load_slice = [&](int h, int kc) {
        wr.load(16, d0, pg.D, pg.vec, [&](int i) -> const TQ* { return head_weight_row(pg, a, h, kc * 16 + i); });
    };
    load_head(0);
    if (grad_query) load_slice(0, 0);
    const float* ga = s_g + (16 * wave + (lane & 15)) * gst + (lane >> 4);
    const float* wb = s_wk + (lane >> 4) * kPWStride + (lane & 15);

    for (int h = 0; h < pg.Nh; ++h) {
        __syncthreads();  // the previous head's gradient tile is consumed
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
            if (p >= passes) continue;  // uniform
            const int r = p * rpp + r_in;
            float gx, gy, gz;
            finish_grads(gin[p], tpr, (float)W, (float)H, gx, gy, gz);
            if (jok) {
                s_g[r * gst + 2 * j] = gx;
                s_g[r * gst + 2 * j + 1] = gy;
                s_g[r * gst + 2 * S + j] = gz;
                if (do_ref) {
                    // this thread owns (r, j) for every head: sums over h in order
                    float* sr = s_ref + r * 2 * S + 2 * j;
                    sr[0] = h == 0 ? gin[p].lx : sr[0] + gin[p].lx;
                    sr[1] = h == 0 ? gin[p].ly : sr[1] + gin[p].ly;
                }
            }
        }
        if (h + 1 < pg.Nh) load_head(h + 1);
        if (!grad_query) continue;
        for (int kc = 0; kc < CTM; ++kc) {
            __syncthreads();  // the gradient tile is written / the previous W slice consumed
            wr.store(s_wk, kPWStride, 16);
            __syncthreads();
            if (kc + 1 < CTM) load_slice(h, kc + 1);
            else if (h + 1 < pg.Nh) load_slice(h + 1, 0);
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4) {
                const float av = ga[kc * 16 + kk];
#pragma unroll
                for (int t = 0; t < 16; ++t) acc[t] = mfma_16x16x4(av, wb[kk * kPWStride + 16 * t], acc[t]);
            }
        }
    }
    if (grad_query) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int d = d0 + 16 * t + (lane & 15);
            if (d >= pg.D) continue;
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
// (16 * ct rows x kPMStride) and the query rows (kPMStep x kPBStride). The next
// step's inputs are loaded while the matrix cores work on the current ones.
template <typename TQ, int CTM>
__global__ __launch_bounds__(kBlock) void producer_bwd_weights_kernel(Geometry g, ProducerGeom pg, ProducerArgs<TQ> a,
                                                                      ProducerGradIn in, float* __restrict__ part_w,
                                                                      float* __restrict__ part_b)
{
    constexpr int PMAX = max_passes<CTM>() / 2 > 0 ? max_passes<CTM>() / 2 : 1;  // passes over kPMStep rows
    constexpr int PR = kPWCols / 4;
    constexpr int XQ = kPMStep * PR / kBlock;
    extern __shared__ float4 smem4[];
    float* s_a = reinterpret_cast<float*>(smem4);
    float* s_b = s_a + 16 * CTM * kPMStride;
    const int S = pg.S, cols = 3 * S;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int ndb = (pg.D + kPWCols - 1) / kPWCols;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int db = lb % ndb;
    const int h = (lb / ndb) % pg.Nh;
    const int mc = lb / (ndb * pg.Nh);
    const int d0 = db * kPWCols;
    const int mbeg = mc * pg.mrows, mend = min(pg.M, mbeg + pg.mrows);
    const int tpr = pg.tpr, rpp = kBlock / tpr;
    const int passes = rpp >= kPMStep ? 1 : kPMStep / rpp;
    const int j = tid & (tpr - 1), r_in = tid / tpr;
    const bool jok = j < S;
    int H = 1, W = 1, start;
    if (jok) level_of(g.lv, j / pg.Np, H, W, start);

    for (int i = tid; i < 16 * CTM * kPMStride; i += kBlock) s_a[i] = 0.f;  // padding rows stay zero
    f32x4 acc[CTM];
#pragma unroll
    for (int t = 0; t < CTM; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bsum = 0.f;

    GradIn gin[PMAX];
    TileRegs<TQ, XQ, PR> xr;
    auto load_step = [&](int mm0) {
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
            const int r = p * rpp + r_in;
            gin[p] = load_grad_in(pg, in, mm0 + r, p < passes && jok && r < kPMStep && mm0 + r < mend, h, j);
        }
        xr.load(kPMStep, d0, pg.D, pg.vec,
                [&](int r) -> const TQ* { return mm0 + r < mend ? a.query + (size_t)(mm0 + r) * pg.D : nullptr; });
    };
    load_step(mbeg);
    const float* ab = s_a + (lane & 15) * kPMStride + (lane >> 4);
    const float* xb = s_b + (lane >> 4) * kPBStride + 16 * wave + (lane & 15);
    for (int mm0 = mbeg; mm0 < mend; mm0 += kPMStep) {
        __syncthreads();  // previous step consumed
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
            if (p >= passes) continue;  // uniform
            const int r = p * rpp + r_in;
            float gx, gy, gz;
            finish_grads(gin[p], tpr, (float)W, (float)H, gx, gy, gz);
            if (jok && r < kPMStep) {
                s_a[(2 * j) * kPMStride + r] = gx;
                s_a[(2 * j + 1) * kPMStride + r] = gy;
                s_a[(2 * S + j) * kPMStride + r] = gz;
            }
        }
        xr.store(s_b, kPBStride, kPMStep);
        __syncthreads();
        if (mm0 + kPMStep < mend) load_step(mm0 + kPMStep);
#pragma unroll
        for (int kk = 0; kk < kPMStep; kk += 4) {
            const float bv = xb[kk * kPBStride];
#pragma unroll
            for (int t = 0; t < CTM; ++t) acc[t] = mfma_16x16x4(ab[t * 16 * kPMStride + kk], bv, acc[t]);
        }
        if (db == 0 && tid < cols) {
            const float* ar = s_a + tid * kPMStride;
            for (int r = 0; r < kPMStep; ++r) bsum += ar[r];
        }
    }
    const size_t base = ((size_t)mc * pg.Nh + h) * cols;
    const int d = d0 + 16 * wave + (lane & 15);
#pragma unroll
    for (int t = 0; t < CTM; ++t) {
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
    const size_t records = (size_t)kPRows * (pg.S + 1) * sizeof(FwdRecord);
    return records > producer_forward_lds(pg) ? records : producer_forward_lds(pg);
}

size_t producer_bwd_rows_lds(const ProducerGeom& pg)
{
    return ((size_t)kPRows * (16 * pg.ct + 4) + 16 * kPWStride + (size_t)kPRows * 2 * pg.S) * sizeof(float);
}

size_t producer_bwd_weights_lds(const ProducerGeom& pg)
{
    return ((size_t)16 * pg.ct * kPMStride + (size_t)kPMStep * kPBStride) * sizeof(float);
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

template <typename TQ, int CTM>
static void launch_producer_forward_c(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& a, float* loc,
                                      float* attn, hipStream_t stream)
{
    hipLaunchKernelGGL((producer_forward_kernel<TQ, CTM>), dim3(producer_row_tiles(pg.M) * pg.Nh), dim3(kBlock),
                       producer_forward_lds(pg), stream, g, pg, typed<TQ>(a), loc, attn);
}

template <typename TQ>
static void launch_producer_forward_t(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& a, float* loc,
                                      float* attn, hipStream_t stream)
{
    switch (pg.ct) {
    case 3: launch_producer_forward_c<TQ, 3>(g, pg, a, loc, attn, stream); break;
    case 6: launch_producer_forward_c<TQ, 6>(g, pg, a, loc, attn, stream); break;
    default: launch_producer_forward_c<TQ, 12>(g, pg, a, loc, attn, stream); break;
    }
}

hipError_t launch_producer_forward(const Geometry& g, const ProducerGeom& pg, int bf16, const ProducerArgsRaw& a,
                                   float* loc, float* attn, hipStream_t stream)
{
    if (bf16) launch_producer_forward_t<uint16_t>(g, pg, a, loc, attn, stream);
    else launch_producer_forward_t<float>(g, pg, a, loc, attn, stream);
    return hipGetLastError();
}

template <typename T, int VEC, int CTM>
static void launch_fused_c(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& a, int64_t value_bytes,
                           const void* value, void* out, float* loc, float* attn, hipStream_t stream)
{
    const int qtiles = (g.Nq + kPRows - 1) / kPRows;
    const dim3 grid(g.B * g.Nh * qtiles);
    const size_t lds = fused_forward_lds(pg);
    if (buffer_loads_ok(value_bytes))
        hipLaunchKernelGGL((fused_forward_kernel<T, VEC, CTM, true>), grid, dim3(kBlock), lds, stream, g, pg,
                           typed<T>(a), value_bytes, static_cast<const T*>(value), static_cast<T*>(out), loc, attn);
    else
        hipLaunchKernelGGL((fused_forward_kernel<T, VEC, CTM, false>), grid, dim3(kBlock), lds, stream, g, pg,
                           typed<T>(a), value_bytes, static_cast<const T*>(value), static_cast<T*>(out), loc, attn);
}

template <typename T, int VEC>
static void launch_fused_t(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& a, int64_t value_bytes,
                           const void* value, void* out, float* loc, float* attn, hipStream_t stream)
{
    if (pg.ct == 3) launch_fused_c<T, VEC, 3>(g, pg, a, value_bytes, value, out, loc, attn, stream);
    else launch_fused_c<T, VEC, 6>(g, pg, a, value_bytes, value, out, loc, attn, stream);
}

hipError_t launch_fused_forward(const Geometry& g, const ProducerGeom& pg, int bf16, int vec, const ProducerArgsRaw& a,
                                int64_t value_bytes, const void* value, void* out, float* loc, float* attn,
                                hipStream_t stream)
{
    if (bf16) {
        switch (vec) {
        case 8: launch_fused_t<uint16_t, 8>(g, pg, a, value_bytes, value, out, loc, attn, stream); break;
        case 4: launch_fused_t<uint16_t, 4>(g, pg, a, value_bytes, value, out, loc, attn, stream); break;
        case 2: launch_fused_t<uint16_t, 2>(g, pg, a, value_bytes, value, out, loc, attn, stream); break;
        default: launch_fused_t<uint16_t, 1>(g, pg, a, value_bytes, value, out, loc, attn, stream); break;
        }
    } else {
        switch (vec) {
        case 4: launch_fused_t<float, 4>(g, pg, a, value_bytes, value, out, loc, attn, stream); break;
        case 2: launch_fused_t<float, 2>(g, pg, a, value_bytes, value, out, loc, attn, stream); break;
        default: launch_fused_t<float, 1>(g, pg, a, value_bytes, value, out, loc, attn, stream); break;
        }
    }
    return hipGetLastError();
}

template <typename TQ, int CTM>
static hipError_t launch_producer_backward_c(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& ar,
                                             const ProducerGradIn& in, const ProducerGradOut& o, float* part,
                                             hipStream_t stream)
{
    const ProducerArgs<TQ> a = typed<TQ>(ar);
    if (o.grad_query || o.grad_ref) {
        const dim3 grid(producer_row_tiles(pg.M) * producer_grad_query_blocks(pg.D));
        hipLaunchKernelGGL((producer_bwd_rows_kernel<TQ, CTM>), grid, dim3(kBlock), producer_bwd_rows_lds(pg), stream,
                           g, pg, a, in, static_cast<TQ*>(o.grad_query), o.grad_ref);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (o.grad_w_off || o.grad_b_off || o.grad_w_att || o.grad_b_att) {
        float* part_w = part;
        float* part_b = part + (size_t)pg.mchunks * pg.Nh * 3 * pg.S * pg.D;
        const dim3 grid(pg.mchunks * pg.Nh * producer_weight_col_blocks(pg.D));
        hipLaunchKernelGGL((producer_bwd_weights_kernel<TQ, CTM>), grid, dim3(kBlock), producer_bwd_weights_lds(pg),
                           stream, g, pg, a, in, part_w, part_b);
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

template <typename TQ>
static hipError_t launch_producer_backward_t(const Geometry& g, const ProducerGeom& pg, const ProducerArgsRaw& a,
                                             const ProducerGradIn& in, const ProducerGradOut& o, float* part,
                                             hipStream_t stream)
{
    switch (pg.ct) {
    case 3: return launch_producer_backward_c<TQ, 3>(g, pg, a, in, o, part, stream);
    case 6: return launch_producer_backward_c<TQ, 6>(g, pg, a, in, o, part, stream);
    default: return launch_producer_backward_c<TQ, 12>(g, pg, a, in, o, part, stream);
    }
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
