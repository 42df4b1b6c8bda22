// Internal to the gfx950 library: parameter blocks of the producer kernels
// (sampling locations and attention weights from query features). Not part
// of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda_device.h"

namespace msda {

constexpr int kPMaxColTiles = 12;   // 16-column MFMA tiles per head: 3 * N_l * N_p <= 192
constexpr int kPMaxSamples = 64;    // N_l * N_p of the producer
constexpr int kPFusedMaxSamples = 32;  // N_l * N_p of the fused producer + sampler

struct ProducerGeom {
    int32_t M;                // B * N_q query rows
    int32_t D;                // features per query
    int32_t S;                // N_l * N_p
    int32_t Nh, Nl, Np, Nq;
    int32_t ct;               // MFMA column tiles per head: 3, 6 or 12, the first >= 3 * S / 16
                              // (tiles past the head's 3S columns compute zeros)
    int32_t tpr;              // lanes per (row, head) in the epilogues: power of two >= max(S, 4), <= 64
    int32_t b2q;              // locations in (B, 2, N_q, N_h, N_l, N_p)
    int32_t loc_pair_aligned; // BQHLP2 (x, y) pairs may be stored as one float2
    int32_t vec;              // 4: query / weight rows are read 4 elements at a time; else 1
    int32_t mchunks;          // row chunks of the weight-gradient pass
    int32_t mrows;            // rows per chunk (a multiple of 32)
};

template <typename TQ>
struct ProducerArgs {
    const TQ* query;      // (M, D)
    const float* ref;     // (M, N_l, 2) reference points (x, y), normalised
    const TQ* w_off;      // (N_h * S * 2, D), rows ordered (h, l, p, xy)
    const float* b_off;   // (N_h * S * 2) or nullptr
    const TQ* w_att;      // (N_h * S, D), rows ordered (h, l, p)
    const float* b_att;   // (N_h * S) or nullptr
};

struct ProducerArgsRaw {
    const void* query;
    const float* ref;
    const void* w_off;
    const float* b_off;
    const void* w_att;
    const float* b_att;
};

struct ProducerGradIn {
    const float* attn;        // forward's attention weights (M, N_h, S)
    const float* grad_attn;   // (M, N_h, S) or nullptr (zero)
    const float* grad_loc;    // sampling-location layout, or nullptr (zero)
};

struct ProducerGradOut {
    void* grad_query;         // (M, D), query dtype, or nullptr
    float* grad_ref;          // (M, N_l, 2) or nullptr
    float* grad_w_off;        // (N_h * S * 2, D) or nullptr
    float* grad_b_off;        // (N_h * S * 2) or nullptr
    float* grad_w_att;        // (N_h * S, D) or nullptr
    float* grad_b_att;        // (N_h * S) or nullptr
};

size_t producer_forward_lds(const ProducerGeom& pg);
size_t fused_forward_lds(const ProducerGeom& pg);
size_t producer_bwd_rows_lds(const ProducerGeom& pg);
size_t producer_bwd_weights_lds(const ProducerGeom& pg);
size_t producer_bwd_workspace_floats(const ProducerGeom& pg);
int producer_row_tiles(int M);
int producer_grad_query_blocks(int D);
int producer_weight_col_blocks(int D);

hipError_t launch_producer_forward(const Geometry& g, const ProducerGeom& pg, int bf16, const ProducerArgsRaw& a,
                                   float* loc, float* attn, hipStream_t stream);
hipError_t launch_fused_forward(const Geometry& g, const ProducerGeom& pg, int bf16, int vec, const ProducerArgsRaw& a,
                                int64_t value_bytes, const void* value, void* out, float* loc, float* attn,
                                hipStream_t stream);
hipError_t launch_producer_backward(const Geometry& g, const ProducerGeom& pg, int bf16, const ProducerArgsRaw& a,
                                    const ProducerGradIn& in, const ProducerGradOut& o, void* workspace,
                                    hipStream_t stream);

}  // namespace msda
