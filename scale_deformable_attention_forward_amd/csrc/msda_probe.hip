// Read-bandwidth probes of the memory levels that serve the sampler's
// gathers, for the benchmark's roofline (built into libmsda_probe.so, which
// only the benchmark loads; the sampling library does not use it).
//
// Every probe reads float32 data with 16-byte buffer loads, the load form the
// gathers use, sums what it reads and stores one float per thread so the
// loads stay live. The caller times a launch and divides the bytes the probe
// reports by the time.
//
//  mode 0, vector L1: every workgroup reads two 8 KiB windows in turn (16
//          KiB in all, within the 32 KiB vector L1 of a CU), one contiguous
//          KiB per wave instruction; the window changes every iteration so
//          no load is loop-invariant;
//  mode 1, L2 stream: the workgroups of each XCD (block i runs on XCD i % 8)
//          sweep that XCD's own span of `span` bytes, each from its own
//          starting offset; a span of a few MiB stays in the XCD's 4 MiB L2
//          and is far larger than the vector L1, so loads miss L1 and hit L2;
//  mode 2, L2 gather: as mode 1, but every group of 8 lanes reads one
//          128-byte row at a pseudo-random row of the span, four rows in
//          flight per lane: the access shape of the float32 gathers;
//  mode 3, HBM stream: all workgroups sweep one span of `span` bytes (a
//          span far larger than L2 and the 256 MiB last-level cache), each
//          from its own starting offset.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kProbeBlock = 256;
constexpr int kXcds = 8;
constexpr int kWindow = 8 * 1024;  // bytes of one vector-L1 window (mode 0)

__device__ __forceinline__ float sum4(const __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]) + __uint_as_float(t[2]) + __uint_as_float(t[3]);
}

__global__ __launch_bounds__(kProbeBlock) void read_probe_kernel(const float* __restrict__ buf, int64_t span,
                                                                 int mode, int iters, float* __restrict__ sink)
{
    const int tid = threadIdx.x;
    const int blk = blockIdx.x;
    float acc = 0.f;
    if (mode == 0) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(buf), (short)0, (int)span, 0x00020000);
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
            const uint32_t base = (uint32_t)((it & 1) * kWindow);
#pragma unroll
            for (int k = 0; k < kWindow / (16 * kProbeBlock); ++k)
                acc += sum4(r, base + (uint32_t)((k * kProbeBlock + tid) * 16));
        }
    } else if (mode == 1 || mode == 2) {
        const int xcd = blk % kXcds;
        const float* xbase = buf + (size_t)xcd * (size_t)(span / 4);
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(xbase), (short)0, (int)span, 0x00020000);
        if (mode == 1) {
            const uint32_t chunk = 16 * kProbeBlock;  // bytes per workgroup step
            const uint32_t nchunks = (uint32_t)(span / chunk);
            uint32_t c = (uint32_t)(blk / kXcds) * 97u % nchunks;
            for (int it = 0; it < iters; ++it) {
#pragma unroll 4
                for (int k = 0; k < 4; ++k) {
                    acc += sum4(r, c * chunk + (uint32_t)tid * 16);
                    c = c + 1 == nchunks ? 0 : c + 1;
                }
            }
        } else {
            const uint32_t rows = (uint32_t)(span / 128);
            uint32_t h = (uint32_t)(blk * kProbeBlock + tid) / 8u * 2654435761u + 12345u;
            const uint32_t lane_off = (uint32_t)(tid % 8) * 16;
            for (int it = 0; it < iters; ++it) {
                uint32_t row[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    h = h * 1664525u + 1013904223u;
                    row[k] = (h >> 8) % rows;
                }
                float v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = sum4(r, row[k] * 128u + lane_off);
                acc += (v[0] + v[1]) + (v[2] + v[3]);
            }
        }
    } else {
        const int64_t chunk = 16 * kProbeBlock;
        const int64_t nchunks = span / chunk;
        int64_t c = (int64_t)blk * 131 % nchunks;
        for (int it = 0; it < iters; ++it) {
#pragma unroll 4
            for (int k = 0; k < 4; ++k) {
                const float4 t = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(buf) + c * chunk +
                                                                 (int64_t)tid * 16);
                acc += (t.x + t.y) + (t.z + t.w);
                c = c + 1 == nchunks ? 0 : c + 1;
            }
        }
    }
    sink[(size_t)blk * kProbeBlock + tid] = acc;
}

}  // namespace

extern "C" {

// Bytes one launch of `mode` reads with `blocks` workgroups and `iters`
// iterations (negative: bad arguments).
int64_t msda_probe_bytes(int mode, int blocks, int iters)
{
    if (blocks < 1 || iters < 1) return -1;
    const int64_t per_wg_iter = mode == 0 ? kWindow : mode == 1 ? 4 * 16 * kProbeBlock
                              : mode == 2 ? 4 * 16 * kProbeBlock : mode == 3 ? 4 * 16 * kProbeBlock : -1;
    if (per_wg_iter < 0) return -1;
    return per_wg_iter * blocks * (int64_t)iters;
}

// Launch one probe. buf: device buffer of at least 16 KiB (mode 0), 8 * span
// bytes (modes 1-2) or span bytes (mode 3); sink: blocks * 256 floats.
// Returns 0, or 1 for bad arguments (nothing launched), or 2 if the launch
// failed.
int msda_probe_read(const void* buf, int64_t buf_bytes, int64_t span, int mode, int blocks, int iters,
                    float* sink, hipStream_t stream)
{
    if (!buf || !sink || blocks < 1 || iters < 1 || mode < 0 || mode > 3) return 1;
    if ((uintptr_t)buf % 16) return 1;
    if (mode == 0 && buf_bytes < (int64_t)2 * kWindow) return 1;
    if (mode == 0) span = (int64_t)2 * kWindow;
    if ((mode == 1 || mode == 2) &&
        (span < 16 * kProbeBlock || span % (16 * kProbeBlock) || span >= ((int64_t)1 << 31) || kXcds * span > buf_bytes))
        return 1;
    if (mode == 3 && (span < 16 * kProbeBlock || span % (16 * kProbeBlock) || span > buf_bytes)) return 1;
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kProbeBlock), 0, stream,
                       static_cast<const float*>(buf), span, mode, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
