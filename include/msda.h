/*
 * msda.h - C ABI of the gfx950 (MI355X) multi-scale deformable attention library.
 *
 * Operations, each a call below:
 *   msda_forward   - "MS Deformable Attention Kernel API Reference"
 *                    (Background; Parameters; Returns).
 *   msda_backward  - "MS Deformable Attention Backward Kernel API Reference"
 *                    (Background; Parameters: grad_output and the
 *                    compute_grad_* flags; Returns; Notes).
 *   msda_producer_forward, msda_fused_forward, msda_producer_backward -
 *                    the step that feeds the sampler: "MS Deformable
 *                    Attention Kernel API Reference" (Background) samples at
 *                    learned sampling locations with attention weights; these
 *                    calls produce them from per-query features (a linear
 *                    projection, the per-level normalisation and the softmax
 *                    written out below), alone or fused with the sampler.
 *
 * Notation follows the pages: B batch, N_q queries, N_h heads, C_h channels
 * per head, N_l pyramid levels, N_p sampling points per (query, head, level),
 * L = sum over levels of H_l * W_l.
 *
 * Conventions shared by every call:
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays in the
 *    stated layout. The caller owns every buffer; the library allocates
 *    nothing and keeps no state between calls; calls are reentrant (except
 *    msda_backward_noalloc, whose static scratch is shared by the calls on
 *    one GPU).
 *  - Work is enqueued on `stream` (NULL = the null stream) and the call
 *    returns before it finishes. Outputs must not overlap inputs.
 *  - Every check happens on the host before the first HIP call, so an error
 *    status means nothing was enqueued. No call aborts or throws.
 *  - value, output, grad_output and grad_value share problem->value_dtype;
 *    sampling locations, attention weights and their gradients are float32;
 *    all accumulation is float32.
 *  - Pointers need the natural alignment of their element type.
 */
#ifndef MSDA_H
#define MSDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSDA_ABI_VERSION 3
#define MSDA_MAX_LEVELS 16

typedef enum msda_status {
    MSDA_OK = 0,
    MSDA_ERR_INVALID_ARGUMENT = 1,  /* NULL/misaligned/overlapping pointer, bad size or enum */
    MSDA_ERR_INVALID_LEVELS = 2,    /* H or W < 1, L != sum H*W, starts not the prefix sums */
    MSDA_ERR_NOTHING_TO_COMPUTE = 3,/* backward with all three gradient outputs NULL */
    MSDA_ERR_UNSUPPORTED = 4,       /* N_l > MSDA_MAX_LEVELS or a size past the index range */
    MSDA_ERR_WORKSPACE_TOO_SMALL = 5,
    MSDA_ERR_HIP = 6                /* a HIP launch reported an error */
} msda_status;

/* value layouts ("MS Deformable Attention Kernel API Reference", Parameters: value) */
typedef enum msda_value_layout {
    MSDA_VALUE_BLNC = 0,  /* (B, L, N_h, C_h) */
    MSDA_VALUE_BNLC = 1   /* (B, N_h, L, C_h) */
} msda_value_layout;

/* sampling_locations layouts (same page, Parameters: sampling_locations);
   the size-2 axis holds (x, y): x along W, y along H. */
typedef enum msda_loc_layout {
    MSDA_LOC_BQHLP2 = 0,  /* (B, N_q, N_h, N_l, N_p, 2) */
    MSDA_LOC_B2QHLP = 1   /* (B, 2, N_q, N_h, N_l, N_p) */
} msda_loc_layout;

/* padding_mode (same page, Parameters; backward page, Notes) */
typedef enum msda_padding {
    MSDA_PAD_ZEROS = 0,   /* a corner outside the level reads 0 */
    MSDA_PAD_BORDER = 1   /* the pixel coordinate is clamped into the level first */
} msda_padding;

typedef enum msda_dtype {
    MSDA_F32 = 0,
    MSDA_BF16 = 1         /* bfloat16 storage, float32 arithmetic, RNE stores */
} msda_dtype;

/*
 * Problem description (host memory, read during the call only).
 * spatial_shapes: N_l x 2 int64 (H_l, W_l) ("... Kernel API Reference",
 *   Parameters: spatial_shapes). level_start_index: N_l int64, the start of
 *   each level in the flattened L axis (Parameters: level_start_index); it
 *   must be the exclusive prefix sum of H_l * W_l. Inside level l, pixel
 *   (row i, column j) is element level_start_index[l] + i * W_l + j of L.
 * align_corners != 0 maps a normalised coordinate u in [0, 1] to u * (W - 1);
 *   0 maps it to u * W - 0.5, formed in float32 as fmaf(u, W, -0.5f)
 *   (Parameters: align_corners; the page states the map for H, it is applied
 *   to W the same way).
 */
typedef struct msda_problem {
    int64_t B, L, N_q, N_h, C_h, N_l, N_p;
    const int64_t* spatial_shapes;
    const int64_t* level_start_index;
    int32_t value_layout;               /* msda_value_layout */
    int32_t sampling_locations_layout;  /* msda_loc_layout */
    int32_t align_corners;              /* 0 or 1 */
    int32_t padding_mode;               /* msda_padding */
    int32_t value_dtype;                /* msda_dtype */
} msda_problem;

/*
 * Forward sampler ("MS Deformable Attention Kernel API Reference",
 * Background and Returns):
 *   output[b, q, h*C_h + c] = sum_{l,p} attention_weights[b,q,h,l,p] * S_{l,p}[c]
 * where S is the bilinear interpolation of level l of value[b, :, h, :] at
 * sampling location [b,q,h,l,p] after the coordinate map and padding above.
 *
 *   value               (B, L, N_h, C_h) or (B, N_h, L, C_h), value_dtype
 *   sampling_locations  (B, N_q, N_h, N_l, N_p, 2) or (B, 2, N_q, N_h, N_l, N_p), float32
 *   attention_weights   (B, N_q, N_h, N_l, N_p), float32, used as given
 *   output              (B, N_q, N_h * C_h), value_dtype, fully overwritten
 *
 * B == 0 or N_q == 0 is a valid empty problem (nothing is enqueued).
 */
msda_status msda_forward(const msda_problem* problem, const void* value,
                         const float* sampling_locations, const float* attention_weights,
                         void* output, hipStream_t stream);

/*
 * Bytes of device workspace msda_backward needs for `problem` (0 when none).
 * The backward takes one of two paths per call:
 *  - destination-tiled (C_h % 4 == 0, C_h <= 64, value / grad_output /
 *    grad_value aligned to 4 elements, B * N_h <= 65535): for
 *    S = B*N_q*N_h*N_l*N_p samples, 20 bytes per sample (anchor corner,
 *    fractions, attention weight), per-(batch, head, pixel band, run of
 *    samples) counts and offsets, band lists of 4-byte sample indices with
 *    room for 2 entries per sample (4 on levels wider than one band), and
 *    float32 partial tiles for the bands of coarse levels that are split over
 *    several workgroups; about 236 MB for 2 x 22223 queries, 8 heads,
 *    4 levels, 4 points, 32 channels;
 *  - generic (any other shape or alignment): a float32 array of value's
 *    element count for bfloat16, nothing for float32.
 * The size returned covers both. The contents are scratch and need no
 * initialisation.
 */
msda_status msda_backward_workspace_size(const msda_problem* problem, size_t* bytes);

/* flags of msda_backward */
#define MSDA_BACKWARD_ACCUMULATE_GRAD_VALUE 1u  /* grad_value += result instead of = result */

/*
 * Backward ("MS Deformable Attention Backward Kernel API Reference",
 * Returns and Notes). With G = grad_output[b, q, h*C_h : (h+1)*C_h]:
 *   grad_attention_weights[b,q,h,l,p] = <G, S_{l,p}>
 *   grad_sampling_locations[..., x]   = A * <G, dS/dx> * dx/du_x   (same for y)
 *   grad_value[b, corner, h, :]       = sum over every (q, l, p) whose in-range
 *                                       corner it is of A * w_corner * G
 * dx/du is W (align_corners off) or W - 1 (on), and 0 where border padding
 * clamped the coordinate. The interpolant's derivative is that of the
 * four-corner form (a right derivative at integer coordinates).
 *
 *   grad_output               (B, N_q, N_h * C_h), value_dtype
 *   value, sampling_locations, attention_weights: as msda_forward
 *   grad_value                same shape and layout as value, value_dtype, or NULL
 *   grad_sampling_locations   same shape and layout as sampling_locations, float32, or NULL
 *   grad_attention_weights    (B, N_q, N_h, N_l, N_p), float32, or NULL
 *   flags                     0 or MSDA_BACKWARD_ACCUMULATE_GRAD_VALUE (other
 *                             bits: MSDA_ERR_INVALID_ARGUMENT)
 *   workspace, workspace_bytes: device memory, 16-byte aligned, at least
 *                             msda_backward_workspace_size bytes, not
 *                             overlapping any tensor (may be NULL/0 when
 *                             grad_value is NULL); else
 *                             MSDA_ERR_WORKSPACE_TOO_SMALL
 *
 * A NULL gradient pointer skips that gradient (the compute_grad_* flags of the
 * page); all three NULL returns MSDA_ERR_NOTHING_TO_COMPUTE ("at least one
 * must be True"). grad_sampling_locations and grad_attention_weights are
 * fully overwritten. grad_value is overwritten, or with
 * MSDA_BACKWARD_ACCUMULATE_GRAD_VALUE the result is added to what it holds
 * (for bfloat16: one rounding of old + new); elements no sample reaches are
 * written 0 (left as they are when accumulating). Sums are float32; a
 * bfloat16 grad_value is rounded to nearest even once, at the end.
 * Determinism: grad_A and grad_loc are bitwise reproducible; so is grad_value
 * on the destination-tiled path (every element is the sum of its
 * contributions in a fixed order); on the generic path grad_value is summed
 * with float32 atomics and its last bits may differ from run to run.
 */
msda_status msda_backward(const msda_problem* problem, const void* grad_output, const void* value,
                          const float* sampling_locations, const float* attention_weights,
                          void* grad_value, float* grad_sampling_locations,
                          float* grad_attention_weights, unsigned int flags, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Bytes of the static device scratch msda_backward_noalloc uses in place of a workspace. */
#define MSDA_NOALLOC_SCRATCH_BYTES (256u << 20)

/*
 * msda_backward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The workspace msda_backward would take is
 * a static device array of MSDA_NOALLOC_SCRATCH_BYTES (256 MiB) inside the
 * library; each GPU the call runs on holds its own copy from the first call
 * on it until the process ends, and the call allocates nothing. A problem
 * whose workspace (msda_backward_workspace_size) is larger returns
 * MSDA_ERR_WORKSPACE_TOO_SMALL with nothing enqueued; the encoder-sized
 * backward (2 x 22223 queries, 8 heads, 4 levels x 4 points, 32 channels)
 * fits. `stream` must belong to the current device (else
 * MSDA_ERR_INVALID_ARGUMENT). All calls on one GPU share its array: calls
 * that overlap in time on one GPU (different streams, or threads) race and
 * must be serialised by the caller. Arguments, results, determinism and the
 * other errors are those of msda_backward.
 */
msda_status msda_backward_noalloc(const msda_problem* problem, const void* grad_output, const void* value,
                                  const float* sampling_locations, const float* attention_weights,
                                  void* grad_value, float* grad_sampling_locations,
                                  float* grad_attention_weights, unsigned int flags, hipStream_t stream);

/*
 * Producer of the sampler's inputs. For query row m = (b, q) with features
 * x_m = query[b, q, :] (D elements) and S = N_l * N_p:
 *   off[m, h, l, p, c] = x_m . offset_weight[((h*N_l + l)*N_p + p)*2 + c, :]
 *                        + offset_bias[same row]            (c = 0: x, 1: y; pixels)
 *   z[m, h, l, p]      = x_m . attention_weight[(h*N_l + l)*N_p + p, :]
 *                        + attention_bias[same row]
 *   sampling_locations[b, q, h, l, p, x] = reference_points[b, q, l, x] + off[m, h, l, p, x] / W_l
 *   sampling_locations[b, q, h, l, p, y] = reference_points[b, q, l, y] + off[m, h, l, p, y] / H_l
 *   attention_weights[b, q, h, :, :]     = softmax over the S logits z[m, h, :, :]
 * (the pages leave how the locations and weights are learned open; this is
 * the plain reading: offsets in pixels of their level, normalised by the
 * level's size, around per-level reference points).
 *
 *   query               (B, N_q, D), value_dtype, row-major
 *   reference_points    (B, N_q, N_l, 2), float32, normalised (x, y)
 *   offset_weight       (N_h * N_l * N_p * 2, D), value_dtype (out_features, in_features)
 *   offset_bias         (N_h * N_l * N_p * 2), float32, or NULL (zero)
 *   attention_weight    (N_h * N_l * N_p, D), value_dtype
 *   attention_bias      (N_h * N_l * N_p), float32, or NULL (zero)
 * problem->L, C_h and value_layout describe the value tensor of the sampler
 * (msda_fused_forward); the producer alone only needs them to be valid.
 * Supported: 1 <= D, N_l * N_p <= 64 (<= 32 for msda_fused_forward),
 * M * D < 2^31 (M = B * N_q); otherwise MSDA_ERR_UNSUPPORTED. Products are
 * float32 on the matrix cores (bfloat16 inputs widened exactly); the softmax
 * and the normalisation are float32.
 */
msda_status msda_producer_forward(const msda_problem* problem, int64_t D, const void* query,
                                  const float* reference_points, const void* offset_weight,
                                  const float* offset_bias, const void* attention_weight,
                                  const float* attention_bias, float* sampling_locations,
                                  float* attention_weights, hipStream_t stream);

/*
 * msda_producer_forward followed by msda_forward in one kernel: output as
 * msda_forward computes it from the locations and weights msda_producer_forward
 * computes (the same float32 values, so the result is bitwise that of the two
 * calls). sampling_locations and attention_weights are outputs here and may
 * each be NULL (not stored; a backward needs them). value and output as in
 * msda_forward.
 */
msda_status msda_fused_forward(const msda_problem* problem, int64_t D, const void* query,
                               const float* reference_points, const void* offset_weight,
                               const float* offset_bias, const void* attention_weight,
                               const float* attention_bias, const void* value, void* output,
                               float* sampling_locations, float* attention_weights, hipStream_t stream);

/* Bytes of device workspace msda_producer_backward needs (float32 partial
   weight gradients of row chunks; 0 when no weight or bias gradient is
   possible). */
msda_status msda_producer_backward_workspace_size(const msda_problem* problem, int64_t D, size_t* bytes);

/*
 * Backward of msda_producer_forward. Inputs: query, offset_weight and
 * attention_weight as in the forward; attention_weights = the forward's
 * output; grad_sampling_locations (sampling-location layout) and
 * grad_attention_weights (B, N_q, N_h, N_l, N_p), float32, each NULL for a
 * zero gradient. With G_off = grad_loc / (W_l or H_l) and
 * G_z = A * (grad_A - sum over the head's S entries of A * grad_A):
 *   grad_query[m, :]          = G_off[m] . offset_weight + G_z[m] . attention_weight   (value_dtype)
 *   grad_reference_points[m, l, c] = sum over (h, p) of grad_sampling_locations[m, h, l, p, c]
 *   grad_offset_weight        = G_off^T . X,  grad_offset_bias    = column sums of G_off
 *   grad_attention_weight     = G_z^T . X,    grad_attention_bias = column sums of G_z
 * (weight and bias gradients float32). Every output may be NULL (skipped);
 * all six NULL returns MSDA_ERR_NOTHING_TO_COMPUTE. Outputs are overwritten.
 * Every sum has a fixed order: results are bitwise reproducible. workspace:
 * 16-byte aligned device memory of msda_producer_backward_workspace_size bytes
 * (may be NULL when no weight or bias gradient is asked for).
 */
msda_status msda_producer_backward(const msda_problem* problem, int64_t D, const void* query,
                                   const void* offset_weight, const void* attention_weight,
                                   const float* attention_weights, const float* grad_sampling_locations,
                                   const float* grad_attention_weights, void* grad_query,
                                   float* grad_reference_points, float* grad_offset_weight,
                                   float* grad_offset_bias, float* grad_attention_weight,
                                   float* grad_attention_bias, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* msda_status_string(msda_status status);

/* MSDA_ABI_VERSION of the built library. */
int msda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H */
