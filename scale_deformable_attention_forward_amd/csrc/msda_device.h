// Internal to the gfx950 library: kernel parameter blocks and small device
// helpers shared by the forward and backward kernels. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

constexpr int kMaxLevels = 16;
constexpr int kBlock = 256;      // 4 wave64s per workgroup
constexpr int kWave = 64;
constexpr int kNumXcd = 8;       // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr size_t kLdsBudget = 64 * 1024;  // dynamic LDS per workgroup kept within 64 KiB

// Level table of the flattened pyramid ("MS Deformable Attention Kernel API
// Reference", Parameters: spatial_shapes, level_start_index).
struct Levels {
    int32_t H[kMaxLevels];
    int32_t W[kMaxLevels];
    int32_t start[kMaxLevels];
};

// Division by a divisor fixed for a launch, as a multiply-high, an add and a
// shift (the round-up method of division by invariant integers: with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, every n < 2^31
// has n / d = (mulhi(n, m) + n) >> l). Built on the host, used by kernels in
// place of a runtime integer division.
struct FastDiv {
    uint32_t d, m, l;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d)
{
    if (d < 1) d = 1;
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    const uint64_t m = ((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d) + 1;
    return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ int fdiv(int n, const FastDiv& f)
{
    return (int)((__umulhi((uint32_t)n, f.m) + (uint32_t)n) >> f.l);
}

// Divisions by the samples per staged chunk: a launch stages chunks of
// sc_max samples and at most one shorter last chunk.
struct ChunkDiv {
    FastDiv full, tail;
    __device__ __forceinline__ const FastDiv& of(int sc, int sc_max) const { return sc == sc_max ? full : tail; }
};

__host__ inline ChunkDiv make_chunkdiv(int S, int sc_max)
{
    const int rest = S % sc_max;
    return ChunkDiv{make_fastdiv((uint32_t)sc_max), make_fastdiv((uint32_t)(rest ? rest : sc_max))};
}

// Everything a kernel needs to address one problem. Sizes are validated on
// the host (every element count below 2^31 except where noted).
struct Geometry {
    int32_t B, L, Nq, Nh, Ch, Nl, Np, S;  // S = Nl * Np samples per (b, q, h)
    int32_t bnlc;          // value layout is (B, N_h, L, C_h)
    int32_t b2q;           // sampling-location layout is (B, 2, N_q, N_h, N_l, N_p)
    int32_t align_corners;
    int32_t border;
    int32_t loc_pair_aligned;  // BQHLP2 (x, y) pairs may be read/written as one float2
    int32_t lpu_log2;      // lanes per unit = 1 << lpu_log2
    int32_t chunks;        // channel chunks per (b, q, h)
    int32_t units;         // B * N_h * N_q * chunks
    int32_t blocks;        // grid size
    Levels lv;
    FastDiv nq_div, nh_div, np_div, ch_div;  // by N_q, N_h, N_p, chunks
};

// Destination-tiled grad_value pass (backward). Every level is cut into
// bands (tiles) of `rows` x `cols` pixels. Samples are bucketed by the bands
// their 2x2 corner block touches into one list per (b, h, band), made of one
// run per bucketing workgroup (kBandChunk consecutive samples) in workgroup
// order. A tile job is (band, chunk), a chunk being a range of runs. A band
// of one chunk is stored by its job; the jobs of a band split into several
// chunks write float32 partial tiles, which a reduction pass adds in chunk
// order.
constexpr int kTileBlock = 512;          // threads per tile workgroup
constexpr int kRectRows = 2;             // halo mode: a lane group owns kRectRows x kRectCols anchor bins
constexpr int kRectCols = 2;
constexpr int kTileEntries = 2048;       // list entries staged in LDS per pass
constexpr int kTileBins = 1536;          // anchor bins per tile: (rows + 1) * (cols + 1)
constexpr int kPixCols = 4;              // pixel mode: a lane group's block is kRectRows x kPixCols pixels
constexpr int kBandBlock = 512;          // threads of the bucketing kernels
constexpr int kBandChunk = 2048;         // samples per bucketing workgroup
constexpr int kMaxBandsPerLevel = 4096;  // bands of one level (LDS histogram size)
constexpr int kReduceF4 = 256;           // float4s of a band one reduction workgroup adds up
static_assert(kBandChunk <= kTileEntries, "one run (<= kBandChunk entries) must fit one LDS pass");
static_assert(kBandChunk % kBandBlock == 0 && kTileEntries % kTileBlock == 0, "whole per-thread batches");

struct TilePlan {
    int32_t jobs;                        // halo-mode tile jobs per (b, h) slab
    int32_t pjobs;                       // pixel-mode tile jobs (bands) per (b, h) slab
    int32_t bands;                       // bands per slab
    int32_t rpieces;                     // reduction pieces per slab (0: no band is split)
    int32_t nwg;                         // bucketing workgroups (runs) per (slab, level)
    int64_t cap;                         // list entries reserved per slab
    int64_t part_per_slab;               // floats of partial tiles per slab
    int32_t rows[kMaxLevels];
    int32_t row_bands[kMaxLevels];
    int32_t cols[kMaxLevels];
    int32_t col_bands[kMaxLevels];
    int32_t chunks[kMaxLevels];
    int32_t band_begin[kMaxLevels];      // first band of level l within the slab
    int32_t job_begin[kMaxLevels + 1];   // first halo-mode job of level l (none for pixel-mode levels)
    int32_t pjob_begin[kMaxLevels + 1];  // first pixel-mode job of level l (none for halo-mode levels)
    int32_t part_off[kMaxLevels];        // first partial-tile float of level l within the slab
    int32_t rpieces_per_band[kMaxLevels];
    int32_t rpiece_begin[kMaxLevels + 1];
    FastDiv rows_div[kMaxLevels];        // by rows[l]
    FastDiv cols_div[kMaxLevels];        // by cols[l]
};

// Workgroups are dealt to the XCDs round-robin (block i runs on XCD i % 8).
// Renumber them so that each XCD receives one contiguous range of logical
// blocks: consecutive logical blocks share a (b, h) slab of value, so each
// XCD's L2 holds the slab it is working on.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblk)
{
    const int q = nblk / kNumXcd, r = nblk % kNumXcd;
    const int xcd = bid % kNumXcd, slot = bid / kNumXcd;
    return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Level row of the table by a (possibly divergent) index, with static
// indexing only so the table stays in kernel-argument memory.
__device__ __forceinline__ void level_of(const Levels& lv, int l, int& H, int& W, int& start)
{
    H = 1; W = 1; start = 0;
#pragma unroll
    for (int k = 0; k < kMaxLevels; ++k) {
        if (k == l) { H = lv.H[k]; W = lv.W[k]; start = lv.start[k]; }
    }
}

// The level table in LDS, one int4 (H, W, start, 0) per level, so per-thread
// lookups by a divergent level index are one LDS read. Every thread of the
// workgroup must call fill_level_table; it ends with a barrier.
__device__ __forceinline__ void fill_level_table(const Levels& lv, int4* s_lv)
{
    if (threadIdx.x < kMaxLevels) {
        int H, W, start;
        level_of(lv, threadIdx.x, H, W, start);
        s_lv[threadIdx.x] = make_int4(H, W, start, 0);
    }
    __syncthreads();
}

// Normalised -> pixel coordinate along an axis of `size` pixels, in float32:
// align_corners maps [0,1] to [0, size-1], otherwise to [-0.5, size-0.5]
// ("MS Deformable Attention Kernel API Reference", Parameters: align_corners).
__device__ __forceinline__ float pixel_coord(float u, int size, int align)
{
    return align ? u * (float)(size - 1) : __builtin_fmaf(u, (float)size, -0.5f);
}

// bfloat16 helpers (storage only; arithmetic is float32).
__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One element of storage type T as float32, and back (bfloat16: RNE).
__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_f32(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_f32(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// Non-temporal stores, for final outputs and for workspace data that is read
// back about once: their lines are not kept in L2 (nor in the last-level
// cache), which stay with the tensors the gathers re-read (measured: forward
// 121 -> 113 us, and the backward's kernels faster too, at the encoder
// shape).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void nt_store(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void nt_store(uint16_t* p, uint16_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void nt_store(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void nt_store2(float* p, float a, float b)
{
    f32x2_t t;
    t.x = a;
    t.y = b;
    __builtin_nontemporal_store(t, reinterpret_cast<f32x2_t*>(p));
}
__device__ __forceinline__ void nt_store4(float* p, float a, float b, float c, float d)
{
    f32x4_t t;
    t.x = a;
    t.y = b;
    t.z = c;
    t.w = d;
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void nt_store2u(uint32_t* p, uint32_t a, uint32_t b)
{
    u32x2_t t;
    t.x = a;
    t.y = b;
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void nt_store4u(uint32_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4_t t;
    t.x = a;
    t.y = b;
    t.z = c;
    t.w = d;
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

// Load VEC consecutive elements of storage type T as float32; store VEC
// float32 values as T (non-temporal: only final outputs are stored this
// way).
template <typename T, int VEC> struct VecIO;

template <int VEC> struct VecIO<float, VEC> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[VEC])
    {
        if constexpr (VEC == 4) {
            const float4 t = *reinterpret_cast<const float4*>(p);
            v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
        } else if constexpr (VEC == 2) {
            const float2 t = *reinterpret_cast<const float2*>(p);
            v[0] = t.x; v[1] = t.y;
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) v[i] = p[i];
        }
    }
    static __device__ __forceinline__ void store(float* p, const float (&v)[VEC])
    {
        if constexpr (VEC == 4) {
            nt_store4(p, v[0], v[1], v[2], v[3]);
        } else if constexpr (VEC == 2) {
            nt_store2(p, v[0], v[1]);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) nt_store(p + i, v[i]);
        }
    }
};

template <int VEC> struct VecIO<uint16_t, VEC> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[VEC])
    {
        if constexpr (VEC == 8) {
            const uint4 t = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        } else if constexpr (VEC == 4) {
            const uint2 t = *reinterpret_cast<const uint2*>(p);
            v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
            v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
        } else if constexpr (VEC == 2) {
            const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
            v[0] = __uint_as_float(t << 16); v[1] = __uint_as_float(t & 0xffff0000u);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) v[i] = bf16_to_f32(p[i]);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[VEC])
    {
        if constexpr (VEC % 2 == 0) {
            uint32_t w[VEC / 2];
#pragma unroll
            for (int i = 0; i < VEC / 2; ++i)
                w[i] = (uint32_t)f32_to_bf16_rne(v[2 * i]) | ((uint32_t)f32_to_bf16_rne(v[2 * i + 1]) << 16);
            if constexpr (VEC == 8) {
                nt_store4u(reinterpret_cast<uint32_t*>(p), w[0], w[1], w[2], w[3]);
            } else if constexpr (VEC == 4) {
                nt_store2u(reinterpret_cast<uint32_t*>(p), w[0], w[1]);
            } else {
                nt_store(reinterpret_cast<uint32_t*>(p), w[0]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) nt_store(p + i, f32_to_bf16_rne(v[i]));
        }
    }
};

// ---------------------------------------------------------------------------
// Buffer loads. A raw buffer resource over `value` (base, byte size) makes the
// hardware range-check every load: an offset at or past the size returns
// zeros without touching memory. The gathers use it for corners that must
// read nothing (outside the level, or zero weight), with no branch and no
// zero fill. Used when value is smaller than 2^31 - 2^20 bytes (offsets are
// 32-bit byte offsets); larger tensors take the pointer path.
constexpr int kBufferWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format, no swizzle

__device__ __forceinline__ __amdgpu_buffer_rsrc_t value_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// Element offset that marks "no corner". With buffer loads it is 2^31 bytes
// past the base, beyond every byte offset a buffer load may legitimately use,
// so the load returns zeros. On the plain-pointer path (value tensors of
// 2^31 - 2^20 bytes or more, where 2^31 / sizeof(T) is a valid element) it is
// -1, below every valid offset; that path tests for it and skips the load.
template <typename T, bool BUF>
__host__ __device__ constexpr int32_t no_corner()
{
    return BUF ? (int32_t)((1u << 31) / sizeof(T)) : -1;
}

// Whether a value tensor of `bytes` bytes takes the buffer-load path.
__host__ __device__ inline bool buffer_loads_ok(int64_t bytes) { return bytes <= ((int64_t)1 << 31) - ((int64_t)1 << 20); }

// Load VEC elements of T at byte offset `off` of the buffer as float32.
template <typename T, int VEC> struct BufIO;

template <int VEC> struct BufIO<float, VEC> {
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[VEC])
    {
        if constexpr (VEC == 4) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
            v[0] = __uint_as_float(t[0]); v[1] = __uint_as_float(t[1]);
            v[2] = __uint_as_float(t[2]); v[3] = __uint_as_float(t[3]);
        } else if constexpr (VEC == 2) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            v[0] = __uint_as_float(t[0]); v[1] = __uint_as_float(t[1]);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0));
        }
    }
};

template <int VEC> struct BufIO<uint16_t, VEC> {
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[VEC])
    {
        if constexpr (VEC == 8) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(t[i] << 16);
                v[2 * i + 1] = __uint_as_float(t[i] & 0xffff0000u);
            }
        } else if constexpr (VEC == 4) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            v[0] = __uint_as_float(t[0] << 16); v[1] = __uint_as_float(t[0] & 0xffff0000u);
            v[2] = __uint_as_float(t[1] << 16); v[3] = __uint_as_float(t[1] & 0xffff0000u);
        } else if constexpr (VEC == 2) {
            const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
            v[0] = __uint_as_float(t << 16); v[1] = __uint_as_float(t & 0xffff0000u);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                v[i] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * i, 0, 0) << 16);
        }
    }
};

// ---------------------------------------------------------------------------
// Forward sampling of one unit, shared by the sampler and the fused
// producer + sampler kernels.

// Gather record of one sample: the four corner weights (x0,y0), (x0+1,y0),
// (x0,y0+1), (x0+1,y0+1) premultiplied by the attention weight (0 for a
// corner outside the level), and the element offsets in value of those
// corners' first channel of the sample's (b, h); no_corner<T, BUF>() where
// the weight is 0.
struct FwdRecord {
    float4 w;
    int4 o;
};

// Coordinate map, padding and bilinear corners of one sample at normalised
// (ux, uy) of level (H, W, start) with attention weight a, for the (b, h)
// slab starting at element slab_off of value.
template <typename T, bool BUF>
__device__ __forceinline__ void sampler_record(const Geometry& g, float ux, float uy, float a, int H, int W,
                                               int start, int slab_off, FwdRecord& rec)
{
    float x = pixel_coord(ux, W, g.align_corners);
    float y = pixel_coord(uy, H, g.align_corners);
    if (g.border) {
        // clamp into the level before taking corners (NaN lands on 0)
        x = fminf(fmaxf(x, 0.f), (float)(W - 1));
        y = fminf(fmaxf(y, 0.f), (float)(H - 1));
    } else {
        // anything past [-1, W] reads nothing; keeps the int conversion safe
        x = fminf(fmaxf(x, -2.f), (float)(W + 1));
        y = fminf(fmaxf(y, -2.f), (float)(H + 1));
    }
    const float x0f = floorf(x), y0f = floorf(y);
    const float fx = x - x0f, fy = y - y0f;
    const int x0 = (int)x0f, y0 = (int)y0f;
    // corner column / row inside the level
    const bool ix0 = x0 >= 0 && x0 < W, ix1 = x0 >= -1 && x0 + 1 < W;
    const bool iy0 = y0 >= 0 && y0 < H, iy1 = y0 >= -1 && y0 + 1 < H;
    const float gx = 1.f - fx, gy = 1.f - fy;
    float4 w;
    w.x = (ix0 && iy0) ? a * (gx * gy) : 0.f;
    w.y = (ix1 && iy0) ? a * (fx * gy) : 0.f;
    w.z = (ix0 && iy1) ? a * (gx * fy) : 0.f;
    w.w = (ix1 && iy1) ? a * (fx * fy) : 0.f;
    // unsigned arithmetic: offsets of corners outside the level may wrap; they are replaced below
    const uint32_t pstride = (uint32_t)(g.bnlc ? g.Ch : g.Nh * g.Ch);
    const uint32_t o00 = (uint32_t)slab_off + (uint32_t)(start + y0 * W + x0) * pstride;
    const uint32_t orow = (uint32_t)W * pstride;
    const int32_t nc = no_corner<T, BUF>();
    rec.w = w;
    rec.o.x = w.x != 0.f ? (int32_t)o00 : nc;
    rec.o.y = w.y != 0.f ? (int32_t)(o00 + pstride) : nc;
    rec.o.z = w.z != 0.f ? (int32_t)(o00 + orow) : nc;
    rec.o.w = w.w != 0.f ? (int32_t)(o00 + orow + pstride) : nc;
}

// Accumulate sc staged samples of one unit into acc: VEC channels per lane
// starting at channel c0. BUF: every corner is a buffer load (a no-corner
// offset returns zeros, so the multiply-add is a no-op); otherwise only the
// corners with nonzero weight are loaded through `value`.
template <typename T, int VEC, bool BUF>
__device__ __forceinline__ void gather_samples(const T* value, __amdgpu_buffer_rsrc_t vr, int c0, const FwdRecord* rec,
                                               int sc, float (&acc)[VEC])
{
#pragma unroll 4
    for (int s = 0; s < sc; ++s) {
        const FwdRecord r = rec[s];
        const float wk[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
        const int ok[4] = {r.o.x, r.o.y, r.o.z, r.o.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float v[VEC];
            if constexpr (BUF) {
                BufIO<T, VEC>::load(vr, (uint32_t)(ok[k] + c0) * (uint32_t)sizeof(T), v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] = __builtin_fmaf(wk[k], v[i], acc[i]);
            } else if (wk[k] != 0.f) {
                VecIO<T, VEC>::load(value + ok[k] + c0, v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] = __builtin_fmaf(wk[k], v[i], acc[i]);
            }
        }
    }
}

}  // namespace msda
