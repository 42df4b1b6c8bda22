// Forward sampler of multi-scale deformable attention for gfx950.
//
// Computes, for every (b, q, h) ("MS Deformable Attention Kernel API
// Reference", Background and Returns):
//   out[b, q, h*C_h + c] = sum_{l,p} A[b,q,h,l,p] * bilinear(level l of value[b,:,h,:], loc[b,q,h,l,p])[c]
//
// Work decomposition (one "unit" = one (b, h, q, channel chunk)):
//  - a unit is owned by a group of LPU = 2^lpu_log2 lanes of one wave64;
//    each lane holds VEC consecutive channels, so one corner fetch of a unit
//    is a single contiguous C_h-run of value (128 B for 32 float32 channels)
//    and a wave instruction fetches 64/LPU corners;
//  - units are numbered (b, h, q) with q fastest and a workgroup takes
//    256/LPU consecutive units, so a workgroup works inside one (b, h) slab
//    of value; workgroup ids are renumbered so that each XCD sweeps one
//    contiguous range of slabs (its L2 then holds the slab it gathers from);
//  - per chunk of up to SC samples, the workgroup first stages every sample
//    of its units in LDS, one thread per (unit, sample): the coordinate map,
//    padding, floor, the four bilinear weights premultiplied by the attention
//    weight (0 for a corner outside the level) and the four corners' element
//    offsets in value (a "no corner" mark where the weight is 0);
//  - then each lane walks the staged samples and loads the corners, as
//    range-checked buffer loads (a no-corner offset lies past the end of the
//    buffer and returns zeros without a memory access, so there is no branch)
//    or, for value tensors of 2^31 bytes and more, as plain loads of the
//    nonzero-weight corners only; accumulation is float32 in registers.
#include "msda_device.h"

namespace msda {

template <typename T, int VEC, bool BUF>
__global__ __launch_bounds__(kBlock) void forward_kernel(Geometry g, int sc_max, ChunkDiv cdiv, int64_t value_bytes,
                                                         const T* __restrict__ value,
                                                         const float* __restrict__ loc,
                                                         const float* __restrict__ attn,
                                                         T* __restrict__ out)
{
    extern __shared__ float4 smem[];
    const int lpu_log2 = g.lpu_log2;
    const int upb = kBlock >> lpu_log2;
    const int row = sc_max + 1;  // padded LDS row (one row per unit) against bank conflicts
    FwdRecord* s_rec = reinterpret_cast<FwdRecord*>(smem);
    __shared__ int4 s_lv[kMaxLevels];
    fill_level_table(g.lv, s_lv);

    const int tid = threadIdx.x;
    const int u0 = xcd_logical_block(blockIdx.x, gridDim.x) * upb;
    const int S = g.S;
    const int plane = g.Nq * g.Nh * S;  // distance between the x and y planes (B2QHLP)
    const __amdgpu_buffer_rsrc_t vr = value_rsrc(value, BUF ? value_bytes : 0);

    // The unit this lane works on.
    const int grp = tid >> lpu_log2;
    const int lig = tid & ((1 << lpu_log2) - 1);
    const int u = u0 + grp;
    int b = 0, h = 0, q = 0, chunk = 0;
    {
        int t = fdiv(u, g.ch_div);
        chunk = u - t * g.chunks;
        const int t2 = fdiv(t, g.nq_div);
        q = t - t2 * g.Nq;
        b = fdiv(t2, g.nh_div);
        h = t2 - b * g.Nh;
    }
    const int c0 = ((chunk << lpu_log2) + lig) * VEC;
    const bool active = (u < g.units) && (c0 < g.Ch);
    if (u >= g.units) { b = 0; h = 0; q = 0; }  // tail lanes: keep every address in range

    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;

    for (int s0 = 0; s0 < S; s0 += sc_max) {
        const int sc = min(sc_max, S - s0);
        if (s0 > 0) __syncthreads();
        // ---- stage: one thread per (unit, sample) of this chunk ----
        const FastDiv& scd = cdiv.of(sc, sc_max);
        for (int i = tid; i < upb * sc; i += kBlock) {
            const int gi = fdiv(i, scd);
            const int s = i - gi * sc;
            const int uu = u0 + gi;
            FwdRecord rec = {make_float4(0.f, 0.f, 0.f, 0.f),
                             make_int4(no_corner<T, BUF>(), no_corner<T, BUF>(), no_corner<T, BUF>(),
                                       no_corner<T, BUF>())};
            if (uu < g.units) {
                const int t = fdiv(uu, g.ch_div);
                const int t2 = fdiv(t, g.nq_div);
                const int qq = t - t2 * g.Nq;
                const int bb = fdiv(t2, g.nh_div), hh = t2 - bb * g.Nh;
                const int si = s0 + s;
                const int4 lvl = s_lv[fdiv(si, g.np_div)];
                const int H = lvl.x, W = lvl.y, start = lvl.z;
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
                const int slab_off = g.bnlc ? (bb * g.Nh + hh) * g.L * g.Ch : bb * g.L * g.Nh * g.Ch + hh * g.Ch;
                sampler_record<T, BUF>(g, ux, uy, attn[idx], H, W, start, slab_off, rec);
            }
            s_rec[gi * row + s] = rec;
        }
        __syncthreads();
        // ---- gather: VEC channels per lane ----
        if (active) gather_samples<T, VEC, BUF>(value, vr, c0, s_rec + grp * row, sc, acc);
    }
    if (active) VecIO<T, VEC>::store(out + ((b * g.Nq + q) * g.Nh + h) * g.Ch + c0, acc);
}

// Host launcher: grid/LDS sizing for one instantiation.
template <typename T, int VEC>
static hipError_t launch_forward_t(const Geometry& g, int64_t value_bytes, const void* value, const float* loc,
                                   const float* attn, void* out, hipStream_t stream)
{
    const int upb = kBlock >> g.lpu_log2;
    const size_t rec = sizeof(FwdRecord);
    int sc = g.S < 16 ? g.S : 16;
    while (sc > 1 && (size_t)upb * (sc + 1) * rec > kLdsBudget) --sc;
    const size_t lds = (size_t)upb * (sc + 1) * rec;
    const ChunkDiv cdiv = make_chunkdiv(g.S, sc);
    if (buffer_loads_ok(value_bytes))
        hipLaunchKernelGGL((forward_kernel<T, VEC, true>), dim3(g.blocks), dim3(kBlock), lds, stream, g, sc, cdiv,
                           value_bytes, static_cast<const T*>(value), loc, attn, static_cast<T*>(out));
    else
        hipLaunchKernelGGL((forward_kernel<T, VEC, false>), dim3(g.blocks), dim3(kBlock), lds, stream, g, sc, cdiv,
                           value_bytes, static_cast<const T*>(value), loc, attn, static_cast<T*>(out));
    return hipGetLastError();
}

hipError_t launch_forward(const Geometry& g, int bf16, int vec, int64_t value_bytes, const void* value,
                          const float* loc, const float* attn, void* out, hipStream_t stream)
{
    if (bf16) {
        switch (vec) {
        case 8: return launch_forward_t<uint16_t, 8>(g, value_bytes, value, loc, attn, out, stream);
        case 4: return launch_forward_t<uint16_t, 4>(g, value_bytes, value, loc, attn, out, stream);
        case 2: return launch_forward_t<uint16_t, 2>(g, value_bytes, value, loc, attn, out, stream);
        default: return launch_forward_t<uint16_t, 1>(g, value_bytes, value, loc, attn, out, stream);
        }
    }
    switch (vec) {
    case 4: return launch_forward_t<float, 4>(g, value_bytes, value, loc, attn, out, stream);
    case 2: return launch_forward_t<float, 2>(g, value_bytes, value, loc, attn, out, stream);
    default: return launch_forward_t<float, 1>(g, value_bytes, value, loc, attn, out, stream);
    }
}

}  // namespace msda
