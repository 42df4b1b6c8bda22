// Backward of multi-scale deformable attention for gfx950 (float32).
//
// For every (b, q, h) and sample (l, p), with G = grad_output[b, q, h*C_h:(h+1)*C_h]
// and S the bilinear sample ("MS Deformable Attention Backward Kernel API
// Reference", Returns and Notes):
//   grad_A[b,q,h,l,p]      = <G, S>
//   grad_loc[b,q,h,l,p,x]  = A * <G, dS/dx> * dx/du_x    (same for y)
//   grad_value[corner]    += A * w_corner * G             (every in-range corner)
//
// Decomposition: one unit = one (b, h, q), owned by LPU lanes of a wave64
// with VEC consecutive channels per lane (more channels loop in chunks of
// LPU*VEC). Units are numbered (b, h, q) with q fastest; workgroups are
// renumbered per XCD as in the forward, so each XCD's L2 serves one (b, h)
// slab for both the re-gather and the grad_value atomics.
// Per chunk of up to SC samples the workgroup stages, one thread per
// (unit, sample): the corner pixel index, the in-range mask, the fractional
// offsets and the two coordinate slopes (0 where border padding clamped).
// The lanes then re-gather the four corners, form S, dS/dx and dS/dy per
// channel, reduce the three dot products over the unit's lanes with
// cross-lane shuffles, and add A * w * G into grad_value with float32
// atomics (global_atomic_add_f32, no return). grad_A and grad_loc go through
// LDS and leave the workgroup as coalesced stores.
#include <algorithm>

#include "msda_device.h"

namespace msda {

struct BwdRecord {
    float fx, fy;   // fractional offsets inside the cell
    float kx, ky;   // d(pixel)/d(location) per axis, 0 where border clamped
    int32_t pix;    // flat pixel index (along L) of corner (x0, y0)
    int32_t W;      // level row length in pixels
    int32_t mask;   // bit k: corner k = 2*dy + dx lies inside the level
    float a;        // attention weight
};

// grad_value is overwritten: cleared by a plain store kernel (a memset node
// would misbehave inside a captured graph).
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

template <int LPU>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int m = LPU / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, LPU);
    return v;
}

template <int VEC, int LPU>
__global__ __launch_bounds__(kBlock) void backward_kernel(Geometry g, int sc_max,
                                                          const float* __restrict__ grad_out,
                                                          const float* __restrict__ value,
                                                          const float* __restrict__ loc,
                                                          const float* __restrict__ attn,
                                                          float* __restrict__ grad_value,
                                                          float* __restrict__ grad_loc,
                                                          float* __restrict__ grad_attn)
{
    constexpr int upb = kBlock / LPU;
    extern __shared__ float4 smem[];
    const int row = sc_max + 1;
    BwdRecord* s_rec = reinterpret_cast<BwdRecord*>(smem);
    float4* s_res = smem + (upb * row * sizeof(BwdRecord)) / sizeof(float4);  // (gA, gx, gy, -)

    const int tid = threadIdx.x;
    const int u0 = xcd_logical_block(blockIdx.x, gridDim.x) * upb;
    const int S = g.S;
    const int plane = g.Nq * g.Nh * S;

    const int grp = tid / LPU;
    const int lig = tid % LPU;
    const int u = u0 + grp;
    const bool unit_ok = u < g.units;
    const int uc = unit_ok ? u : 0;  // tail lanes: keep every address in range
    const int q = uc % g.Nq;
    const int bh = uc / g.Nq;
    const int h = bh % g.Nh, b = bh / g.Nh;
    const int c0 = lig * VEC;
    const int cstep = LPU * VEC;
    const int pstride = g.bnlc ? g.Ch : g.Nh * g.Ch;
    const int slab_off = g.bnlc ? (b * g.Nh + h) * g.L * g.Ch : b * g.L * g.Nh * g.Ch + h * g.Ch;
    const float* vslab = value + slab_off;
    float* gslab = grad_value ? grad_value + slab_off : nullptr;
    const float* grow = grad_out + ((b * g.Nq + q) * g.Nh + h) * g.Ch;
    const bool want_dots = grad_loc != nullptr || grad_attn != nullptr;

    // grad_output of the first channel chunk stays in registers
    float G0[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) G0[i] = 0.f;
    if (unit_ok && c0 < g.Ch) VecIO<float, VEC>::load(grow + c0, G0);

    for (int s0 = 0; s0 < S; s0 += sc_max) {
        const int sc = min(sc_max, S - s0);
        if (s0 > 0) __syncthreads();
        // ---- stage one record per (unit, sample) ----
        for (int i = tid; i < upb * sc; i += kBlock) {
            const int gi = i / sc;
            const int s = i - gi * sc;
            const int uu = u0 + gi;
            BwdRecord r = {0.f, 0.f, 0.f, 0.f, 0, 1, 0, 0.f};
            if (uu < g.units) {
                const int qq = uu % g.Nq;
                const int t = uu / g.Nq;
                const int hh = t % g.Nh, bb = t / g.Nh;
                const int si = s0 + s;
                const int l = si / g.Np;
                int H, W, start;
                level_of(g.lv, l, H, W, start);
                const int idx = ((bb * g.Nq + qq) * g.Nh + hh) * S + si;
                float ux, uy;
                if (g.b2q) {
                    const int j = bb * 2 * plane + (qq * g.Nh + hh) * S + si;
                    ux = loc[j];
                    uy = loc[j + plane];
                } else if (g.loc_pair_aligned) {
                    const float2 xy = *reinterpret_cast<const float2*>(loc + 2 * idx);
                    ux = xy.x; uy = xy.y;
                } else {
                    ux = loc[2 * idx];
                    uy = loc[2 * idx + 1];
                }
                float x = pixel_coord(ux, W, g.align_corners);
                float y = pixel_coord(uy, H, g.align_corners);
                float kx = g.align_corners ? (float)(W - 1) : (float)W;
                float ky = g.align_corners ? (float)(H - 1) : (float)H;
                if (g.border) {
                    if (!(x >= 0.f)) { x = 0.f; kx = 0.f; }                        // also NaN
                    else if (x > (float)(W - 1)) { x = (float)(W - 1); kx = 0.f; }
                    if (!(y >= 0.f)) { y = 0.f; ky = 0.f; }
                    else if (y > (float)(H - 1)) { y = (float)(H - 1); ky = 0.f; }
                } else {
                    x = fminf(fmaxf(x, -2.f), (float)(W + 1));
                    y = fminf(fmaxf(y, -2.f), (float)(H + 1));
                }
                const float x0f = floorf(x), y0f = floorf(y);
                const int x0 = (int)x0f, y0 = (int)y0f;
                const bool ix0 = x0 >= 0 && x0 < W, ix1 = x0 >= -1 && x0 + 1 < W;
                const bool iy0 = y0 >= 0 && y0 < H, iy1 = y0 >= -1 && y0 + 1 < H;
                r.fx = x - x0f;
                r.fy = y - y0f;
                r.kx = kx;
                r.ky = ky;
                r.pix = start + y0 * W + x0;
                r.W = W;
                r.mask = (ix0 && iy0 ? 1 : 0) | (ix1 && iy0 ? 2 : 0) | (ix0 && iy1 ? 4 : 0) | (ix1 && iy1 ? 8 : 0);
                r.a = attn[idx];
            }
            s_rec[gi * row + s] = r;
        }
        __syncthreads();
        // ---- re-gather, three reductions, scatter ----
        if (unit_ok) {
            const BwdRecord* rr = s_rec + grp * row;
            for (int s = 0; s < sc; ++s) {
                const BwdRecord r = rr[s];
                const float gxw = 1.f - r.fx, gyw = 1.f - r.fy;
                const float w00 = gxw * gyw, w01 = r.fx * gyw, w10 = gxw * r.fy, w11 = r.fx * r.fy;
                const int o00 = r.pix * pstride;
                const int o01 = o00 + pstride;
                const int o10 = o00 + r.W * pstride;
                const int o11 = o10 + pstride;
                float pa = 0.f, px = 0.f, py = 0.f;
                for (int c = c0; c < g.Ch; c += cstep) {
                    if (!want_dots && !gslab) break;
                    float G[VEC], v00[VEC], v01[VEC], v10[VEC], v11[VEC];
                    if (c == c0) {
#pragma unroll
                        for (int i = 0; i < VEC; ++i) G[i] = G0[i];
                    } else {
                        VecIO<float, VEC>::load(grow + c, G);
                    }
#pragma unroll
                    for (int i = 0; i < VEC; ++i) { v00[i] = 0.f; v01[i] = 0.f; v10[i] = 0.f; v11[i] = 0.f; }
                    if (r.mask & 1) VecIO<float, VEC>::load(vslab + o00 + c, v00);
                    if (r.mask & 2) VecIO<float, VEC>::load(vslab + o01 + c, v01);
                    if (r.mask & 4) VecIO<float, VEC>::load(vslab + o10 + c, v10);
                    if (r.mask & 8) VecIO<float, VEC>::load(vslab + o11 + c, v11);
                    if (want_dots) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        const float smp = w00 * v00[i] + w01 * v01[i] + w10 * v10[i] + w11 * v11[i];
                        const float dx = gyw * (v01[i] - v00[i]) + r.fy * (v11[i] - v10[i]);
                        const float dy = gxw * (v10[i] - v00[i]) + r.fx * (v11[i] - v01[i]);
                        pa = __builtin_fmaf(G[i], smp, pa);
                        px = __builtin_fmaf(G[i], dx, px);
                        py = __builtin_fmaf(G[i], dy, py);
                    }
                    }
                    if (gslab) {
#pragma unroll
                        for (int i = 0; i < VEC; ++i) {
                            const float ag = r.a * G[i];
                            if (r.mask & 1) unsafeAtomicAdd(gslab + o00 + c + i, ag * w00);
                            if (r.mask & 2) unsafeAtomicAdd(gslab + o01 + c + i, ag * w01);
                            if (r.mask & 4) unsafeAtomicAdd(gslab + o10 + c + i, ag * w10);
                            if (r.mask & 8) unsafeAtomicAdd(gslab + o11 + c + i, ag * w11);
                        }
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
        // ---- coalesced stores of grad_A and grad_loc for this chunk ----
        for (int i = tid; i < upb * sc; i += kBlock) {
            const int gi = i / sc;
            const int s = i - gi * sc;
            const int uu = u0 + gi;
            if (uu >= g.units) continue;
            const int qq = uu % g.Nq;
            const int t = uu / g.Nq;
            const int hh = t % g.Nh, bb = t / g.Nh;
            const int si = s0 + s;
            const int idx = ((bb * g.Nq + qq) * g.Nh + hh) * S + si;
            const float4 res = s_res[gi * row + s];
            if (grad_attn) grad_attn[idx] = res.x;
            if (grad_loc) {
                if (g.b2q) {
                    const int j = bb * 2 * plane + (qq * g.Nh + hh) * S + si;
                    grad_loc[j] = res.y;
                    grad_loc[j + plane] = res.z;
                } else if (g.loc_pair_aligned) {
                    *reinterpret_cast<float2*>(grad_loc + 2 * idx) = make_float2(res.y, res.z);
                } else {
                    grad_loc[2 * idx] = res.y;
                    grad_loc[2 * idx + 1] = res.z;
                }
            }
        }
    }
}

template <int VEC, int LPU>
static hipError_t launch_backward_t(const Geometry& g, const float* grad_out, const float* value,
                                    const float* loc, const float* attn, float* grad_value,
                                    float* grad_loc, float* grad_attn, hipStream_t stream)
{
    constexpr int upb = kBlock / LPU;
    static_assert(sizeof(BwdRecord) % sizeof(float4) == 0, "records must tile float4 slots");
    const size_t per = sizeof(BwdRecord) + sizeof(float4);  // staged record + result slot
    int sc = g.S < 16 ? g.S : 16;
    while (sc > 1 && (size_t)upb * (sc + 1) * per > kLdsBudget) --sc;
    const size_t lds = (size_t)upb * (sc + 1) * per;
    hipLaunchKernelGGL((backward_kernel<VEC, LPU>), dim3(g.blocks), dim3(kBlock), lds, stream, g, sc,
                       grad_out, value, loc, attn, grad_value, grad_loc, grad_attn);
    return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t n4 = ((uintptr_t)p % 16 == 0) ? n / 4 : 0;
    const int64_t rest = n - 4 * n4;
    if (n4 > 0) {
        const int64_t blocks = std::min<int64_t>((n4 + kBlock - 1) / kBlock, 8192);
        hipLaunchKernelGGL(zero4_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                           reinterpret_cast<float4*>(p), n4);
    }
    if (rest > 0) {
        const int64_t blocks = std::min<int64_t>((rest + kBlock - 1) / kBlock, 8192);
        hipLaunchKernelGGL(zero1_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream, p + 4 * n4, rest);
    }
    return hipGetLastError();
}

hipError_t launch_backward(const Geometry& g, int vec, int lpu, const float* grad_out, const float* value,
                           const float* loc, const float* attn, float* grad_value, float* grad_loc,
                           float* grad_attn, hipStream_t stream)
{
#define MSDA_BWD_CASE(V, P)                                                                       \
    if (vec == V && lpu == P)                                                                     \
        return launch_backward_t<V, P>(g, grad_out, value, loc, attn, grad_value, grad_loc, grad_attn, stream);
    MSDA_BWD_CASE(1, 1) MSDA_BWD_CASE(1, 2) MSDA_BWD_CASE(1, 4) MSDA_BWD_CASE(1, 8)
    MSDA_BWD_CASE(1, 16) MSDA_BWD_CASE(1, 32) MSDA_BWD_CASE(1, 64)
    MSDA_BWD_CASE(2, 1) MSDA_BWD_CASE(2, 2) MSDA_BWD_CASE(2, 4) MSDA_BWD_CASE(2, 8)
    MSDA_BWD_CASE(2, 16) MSDA_BWD_CASE(2, 32) MSDA_BWD_CASE(2, 64)
    MSDA_BWD_CASE(4, 1) MSDA_BWD_CASE(4, 2) MSDA_BWD_CASE(4, 4) MSDA_BWD_CASE(4, 8)
    MSDA_BWD_CASE(4, 16) MSDA_BWD_CASE(4, 32) MSDA_BWD_CASE(4, 64)
#undef MSDA_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace msda
