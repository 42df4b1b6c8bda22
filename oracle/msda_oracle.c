/*
 * CPU oracle for multi-scale deformable attention (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only code allowed to load this
 * library. It shares no source, header, table or helper with the HIP
 * library, and the HIP library never calls it.
 *
 * What it computes (the plain definition, evaluated directly in fp64):
 *
 *  - "MS Deformable Attention Kernel API Reference", Background: values are
 *    sampled from every pyramid level at the sampling locations with bilinear
 *    interpolation; Parameters (value, spatial_shapes, level_start_index,
 *    sampling_locations, attention_weights) give the layouts; Returns gives
 *    the output shape (B, N_q, N_h * C_h).
 *  - Same page, Parameters "align_corners": align_corners=True maps [0,1] to
 *    [0, H-1], False maps it to [-0.5, H-0.5]. The same map is applied along
 *    W (reading; the page states it for H only).
 *  - Same page, Parameters "padding_mode" and the backward page's Notes:
 *    "zeros" reads 0 outside the map, "border" clamps to the edge.
 *  - "MS Deformable Attention Backward Kernel API Reference", Returns and
 *    Notes: gradients w.r.t. value (same layout as value), sampling_locations
 *    (same layout as the input) and attention_weights, from the derivatives
 *    of the bilinear interpolation.
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes):
 *  - the size-2 axis of sampling_locations is (x, y): x runs along W, y
 *    along H;
 *  - inside level l, pixel (row i, column j) sits at flat index
 *    level_start_index[l] + i * W_l + j;
 *  - attention weights are used exactly as given (no renormalisation);
 *  - coordinate rounding: with coord_fp32 != 0 the pixel coordinate is
 *    formed in binary32, as fmaf(loc, (float)W, -0.5f) (align_corners off)
 *    or loc * (float)(W - 1) (align_corners on); everything after that is
 *    binary64. With coord_fp32 == 0 the map is evaluated in binary64.
 *  - "border" clamps the pixel coordinate into [0, W-1] x [0, H-1] before the
 *    corners are taken; a clamped coordinate has zero derivative.
 *  - the derivative of the interpolant is the one of the floor-based
 *    four-corner form (a right derivative at integer coordinates).
 *
 * Value, weights and locations are passed as binary64 arrays; callers upcast
 * binary32 or bfloat16 inputs exactly.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

enum { ORACLE_BLNC = 0, ORACLE_BNLC = 1 };
enum { ORACLE_BQHLP2 = 0, ORACLE_B2QHLP = 1 };
enum { ORACLE_ZEROS = 0, ORACLE_BORDER = 1 };

typedef struct {
    int64_t B, L, Nq, Nh, Ch, Nl, Np;
    const int64_t *shapes; /* Nl x 2: (H_l, W_l) */
    const int64_t *starts; /* Nl */
    int value_layout, loc_layout, align_corners, padding, coord_fp32;
} prob_t;

/* Flat index of value[b, pix, h, c] in the caller's layout
   ("MS Deformable Attention Kernel API Reference", Parameters: value). */
static int64_t value_index(const prob_t *P, int64_t b, int64_t pix, int64_t h, int64_t c)
{
    if (P->value_layout == ORACLE_BLNC)
        return ((b * P->L + pix) * P->Nh + h) * P->Ch + c;
    return ((b * P->Nh + h) * P->L + pix) * P->Ch + c;
}

/* Flat index of coordinate k (0 = x, 1 = y) of sampling location
   [b, q, h, l, p] ("... Kernel API Reference", Parameters: sampling_locations). */
static int64_t loc_index(const prob_t *P, int64_t b, int64_t q, int64_t h, int64_t l, int64_t p, int k)
{
    if (P->loc_layout == ORACLE_BQHLP2)
        return ((((b * P->Nq + q) * P->Nh + h) * P->Nl + l) * P->Np + p) * 2 + k;
    return ((((b * 2 + k) * P->Nq + q) * P->Nh + h) * P->Nl + l) * P->Np + p;
}

/* Flat index of attention_weights[b, q, h, l, p]. */
static int64_t attn_index(const prob_t *P, int64_t b, int64_t q, int64_t h, int64_t l, int64_t p)
{
    return (((b * P->Nq + q) * P->Nh + h) * P->Nl + l) * P->Np + p;
}

/* Normalised location -> pixel coordinate along an axis of `size` pixels.
   *slope receives d(pixel)/d(location); it is 0 where border padding clamps. */
static double pixel_coord(const prob_t *P, double loc, int64_t size, double *slope)
{
    double x;
    if (P->coord_fp32) {
        float lf = (float)loc;
        float xf = P->align_corners ? lf * (float)(size - 1) : fmaf(lf, (float)size, -0.5f);
        x = (double)xf;
    } else {
        x = P->align_corners ? loc * (double)(size - 1) : loc * (double)size - 0.5;
    }
    *slope = P->align_corners ? (double)(size - 1) : (double)size;
    if (P->padding == ORACLE_BORDER) {
        if (x < 0.0) { x = 0.0; *slope = 0.0; }
        else if (x > (double)(size - 1)) { x = (double)(size - 1); *slope = 0.0; }
    }
    return x;
}

/* The four bilinear corners of one sample. Corner k = 2*dy + dx sits at
   column x0 + dx, row y0 + dy. */
typedef struct {
    int64_t pix[4];   /* flat pixel index along L, valid only where inb[k] */
    int inb[4];       /* corner lies inside the level */
    double w[4];      /* bilinear weight */
    double dwdx[4];   /* d w / d x (pixel units) */
    double dwdy[4];   /* d w / d y */
    double sx, sy;    /* d x / d loc_x, d y / d loc_y */
} corners_t;

static void make_corners(const prob_t *P, int64_t l, double lx, double ly, corners_t *K)
{
    int64_t H = P->shapes[2 * l], W = P->shapes[2 * l + 1], start = P->starts[l];
    double x = pixel_coord(P, lx, W, &K->sx);
    double y = pixel_coord(P, ly, H, &K->sy);
    /* Far outside (or not a number): no corner can be inside the level. */
    if (!(fabs(x) < 1e9) || !(fabs(y) < 1e9)) {
        for (int k = 0; k < 4; ++k) {
            K->inb[k] = 0; K->pix[k] = 0; K->w[k] = 0.0; K->dwdx[k] = 0.0; K->dwdy[k] = 0.0;
        }
        return;
    }
    double x0f = floor(x), y0f = floor(y);
    double fx = x - x0f, fy = y - y0f;
    int64_t x0 = (int64_t)x0f, y0 = (int64_t)y0f;
    for (int dy = 0; dy < 2; ++dy) {
        for (int dx = 0; dx < 2; ++dx) {
            int k = 2 * dy + dx;
            int64_t xi = x0 + dx, yi = y0 + dy;
            double wx = dx ? fx : 1.0 - fx;
            double wy = dy ? fy : 1.0 - fy;
            K->inb[k] = (xi >= 0 && xi < W && yi >= 0 && yi < H);
            K->pix[k] = start + yi * W + xi;
            K->w[k] = wx * wy;
            K->dwdx[k] = (dx ? 1.0 : -1.0) * wy;
            K->dwdy[k] = (dy ? 1.0 : -1.0) * wx;
        }
    }
}

static int check(const prob_t *P)
{
    if (P->B < 0 || P->Nq < 0 || P->Nh < 1 || P->Ch < 1 || P->Nl < 1 || P->Np < 1 || P->L < 1)
        return 1;
    int64_t total = 0;
    for (int64_t l = 0; l < P->Nl; ++l) {
        if (P->shapes[2 * l] < 1 || P->shapes[2 * l + 1] < 1) return 2;
        if (P->starts[l] != total) return 2;
        total += P->shapes[2 * l] * P->shapes[2 * l + 1];
    }
    return total == P->L ? 0 : 2;
}

/*
 * Forward: out[b, q, h*C_h + c] = sum_{l,p} A[b,q,h,l,p] * S_{l,p}[c], where
 * S is the bilinear sample of level l at the mapped location
 * ("MS Deformable Attention Kernel API Reference", Background and Returns).
 * Returns 0 on success, 1 for bad sizes, 2 for an inconsistent level table.
 */
int oracle_forward(int64_t B, int64_t L, int64_t Nq, int64_t Nh, int64_t Ch, int64_t Nl, int64_t Np,
                   const int64_t *spatial_shapes, const int64_t *level_start_index,
                   int value_layout, int loc_layout, int align_corners, int padding, int coord_fp32,
                   const double *value, const double *loc, const double *attn, double *out)
{
    prob_t P = {B, L, Nq, Nh, Ch, Nl, Np, spatial_shapes, level_start_index,
                value_layout, loc_layout, align_corners, padding, coord_fp32};
    int rc = check(&P);
    if (rc) return rc;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t q = 0; q < Nq; ++q) {
            for (int64_t h = 0; h < Nh; ++h) {
                double *o = out + (b * Nq + q) * Nh * Ch + h * Ch;
                for (int64_t c = 0; c < Ch; ++c) o[c] = 0.0;
                for (int64_t l = 0; l < Nl; ++l) {
                    for (int64_t p = 0; p < Np; ++p) {
                        corners_t K;
                        make_corners(&P, l, loc[loc_index(&P, b, q, h, l, p, 0)],
                                     loc[loc_index(&P, b, q, h, l, p, 1)], &K);
                        double a = attn[attn_index(&P, b, q, h, l, p)];
                        for (int k = 0; k < 4; ++k) {
                            if (!K.inb[k]) continue;
                            for (int64_t c = 0; c < Ch; ++c)
                                o[c] += a * K.w[k] * value[value_index(&P, b, K.pix[k], h, c)];
                        }
                    }
                }
            }
        }
    }
    return 0;
}

/*
 * Backward ("MS Deformable Attention Backward Kernel API Reference",
 * Returns and Notes). With G = grad_output[b, q, h*C_h : (h+1)*C_h]:
 *   grad_attention_weights[b,q,h,l,p] = <G, S_{l,p}>
 *   grad_sampling_locations (x)      = A * <G, dS/dx> * dx/dloc_x   (same for y)
 *   grad_value[corner]              += A * w_corner * G             (every in-range corner)
 * Any of the three output pointers may be NULL (that gradient is skipped).
 * grad_value is overwritten (zeroed, then accumulated). Work is split over
 * (b, h) slabs, so every element of every output has exactly one writer and
 * the accumulation order is the fixed loop order (q, l, p, corner).
 */
int oracle_backward(int64_t B, int64_t L, int64_t Nq, int64_t Nh, int64_t Ch, int64_t Nl, int64_t Np,
                    const int64_t *spatial_shapes, const int64_t *level_start_index,
                    int value_layout, int loc_layout, int align_corners, int padding, int coord_fp32,
                    const double *grad_out, const double *value, const double *loc, const double *attn,
                    double *grad_value, double *grad_loc, double *grad_attn)
{
    prob_t P = {B, L, Nq, Nh, Ch, Nl, Np, spatial_shapes, level_start_index,
                value_layout, loc_layout, align_corners, padding, coord_fp32};
    int rc = check(&P);
    if (rc) return rc;
    if (grad_value) {
        int64_t n = B * L * Nh * Ch;
        for (int64_t i = 0; i < n; ++i) grad_value[i] = 0.0;
    }
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < Nh; ++h) {
            for (int64_t q = 0; q < Nq; ++q) {
                const double *g = grad_out + (b * Nq + q) * Nh * Ch + h * Ch;
                for (int64_t l = 0; l < Nl; ++l) {
                    for (int64_t p = 0; p < Np; ++p) {
                        corners_t K;
                        int64_t ix = loc_index(&P, b, q, h, l, p, 0);
                        int64_t iy = loc_index(&P, b, q, h, l, p, 1);
                        make_corners(&P, l, loc[ix], loc[iy], &K);
                        double a = attn[attn_index(&P, b, q, h, l, p)];
                        double gs = 0.0, gdx = 0.0, gdy = 0.0;
                        for (int k = 0; k < 4; ++k) {
                            if (!K.inb[k]) continue;
                            for (int64_t c = 0; c < Ch; ++c) {
                                double v = value[value_index(&P, b, K.pix[k], h, c)];
                                gs += g[c] * K.w[k] * v;
                                gdx += g[c] * K.dwdx[k] * v;
                                gdy += g[c] * K.dwdy[k] * v;
                            }
                            if (grad_value) {
                                for (int64_t c = 0; c < Ch; ++c)
                                    grad_value[value_index(&P, b, K.pix[k], h, c)] += a * K.w[k] * g[c];
                            }
                        }
                        if (grad_attn) grad_attn[attn_index(&P, b, q, h, l, p)] = gs;
                        if (grad_loc) {
                            grad_loc[ix] = a * gdx * K.sx;
                            grad_loc[iy] = a * gdy * K.sy;
                        }
                    }
                }
            }
        }
    }
    return 0;
}

/* Threads an OpenMP region of this library uses (for reporting only). */
int oracle_max_threads(void) { return omp_get_max_threads(); }

/* Threads later oracle calls use (timing only; results do not depend on it). */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
