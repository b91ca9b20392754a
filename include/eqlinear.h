/*
 * eqlinear.h -- C ABI of libeqlinear.so, the MI355X (gfx950) equivariant
 * linear layers.
 *
 * Layers
 *  - C_N layer ("Flash EQ-Linear", gist.science summary, Core Insight and
 *    Algorithmic Approach):
 *        y[t][o][g] = sum_{i < C_in} sum_{h < N} w[o][i][(g-h) mod N] * x[t][i][h]
 *    computed as a real DFT along the group axis, one channel-mixing product per
 *    kept frequency (floor(N/2)+1 bins; the DC and, for even N, Nyquist bins are
 *    real products, every other bin is a complex product done as a real 2x2
 *    block product), and an inverse DFT, in one fused kernel.
 *  - D8 Fourier-domain layer ("Quick ViTs", papernotes, key design 2): four
 *    square (C/8) blocks for the 1-D irreps A1, A2, B1, B2 and one (C/4) block
 *    shared by both coordinates of the 2-D irrep E.
 *  - The expanded-dense comparator ("Flash EQ-Linear", Problem Statement):
 *    the weights replicated into the full group-circulant matrix and a dense
 *    product.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them.  Base pointers must be 16-byte aligned.
 *  - Element type is the plan dtype: EQL_F32 = IEEE fp32, EQL_BF16 = bfloat16,
 *    EQL_F16 = IEEE binary16 (accumulation is always fp32).  fp16 ("Flash
 *    EQ-Linear", Implementation: FP32 and FP16 kernels; "Quick ViTs", key
 *    findings, Table 2 in fp16) is taken by the C_N plans' weight spectrum,
 *    forward (every tile; with fused bias/GELU), adjoint spectrum, input and
 *    weight gradients and expanded-dense comparator, and by the D8 and
 *    dihedral plans' layer, passes and comparator.  fp16 holds values up to
 *    65504: inputs, outputs and (in the matrix-core transform kernel and the
 *    weight gradient's transformed x and dy) the Fourier-domain intermediates
 *    must stay within that range.
 *  - Layouts are row-major with the last index contiguous:
 *      x [T][C_in][N], y [T][C_out][N], w [C_out][C_in][N]           (C_N)
 *      x [T][C_in], y [T][C_out] with features [A1|A2|B1|B2|E0|E1]  (D8)
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls that take a stream are asynchronous on it; they do no host
 *    synchronisation, no allocation and use no workspace.
 *  - Every call returns an eqlinear_status; nothing is thrown across the ABI and
 *    there is no global error state.  Argument checks happen before any HIP
 *    call, so they can be exercised without a GPU.  A kernel launch failure is
 *    EQL_ERR_HIP; faults inside an asynchronous kernel surface on the stream.
 *  - A plan is immutable after creation and may be used from several host
 *    threads and streams at once.  Using a destroyed plan is undefined.
 */
#ifndef EQLINEAR_H
#define EQLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EQL_OK = 0,
    EQL_ERR_INVALID = 1,     /* bad argument: NULL, size, alignment, aliasing, kind */
    EQL_ERR_UNSUPPORTED = 2, /* valid request outside what the library implements */
    EQL_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
    EQL_ERR_NOMEM = 4        /* host allocation failed */
} eqlinear_status;

typedef enum { EQL_F32 = 0, EQL_BF16 = 1, EQL_F16 = 2 } eqlinear_dtype;

typedef enum { EQL_KIND_CN = 0, EQL_KIND_D8 = 1 } eqlinear_kind;

typedef struct eqlinear_plan_s* eqlinear_plan_t;

/* Plan metadata.  Counts follow "Flash EQ-Linear", Algorithmic Approach
 * (kept half spectrum) and Specialization for p4 (six real products at N=4),
 * and "Quick ViTs", key design 2 (D8 parameter and multiply counts). */
typedef struct {
    int32_t kind;               /* eqlinear_kind */
    int32_t dtype;              /* eqlinear_dtype */
    int32_t N;                  /* group order (8 for D8) */
    int32_t C_in, C_out;        /* C_N: channels per group element; D8: full widths */
    int32_t bins;               /* C_N: floor(N/2)+1 kept frequencies; D8: 5 irrep blocks */
    int32_t planes;             /* C_N: real frequency planes (= N) */
    int32_t has_nyquist;        /* C_N: 1 when N is even */
    int64_t params;             /* learnable parameters */
    int64_t w_hat_elems;        /* elements of w_hat (C_N) or of the packed blocks (D8) */
    int64_t real_gemms;         /* C_N: real T x C_in x C_out products (2N-2 even, 2N-1 odd) */
    int64_t macs_per_token;     /* multiply-adds per token of the layer's products */
    int64_t dense_macs_per_token; /* same for the expanded dense matrix */
} eqlinear_info;

/* Human-readable name of a status code (static storage, never NULL). */
const char* eqlinear_status_string(eqlinear_status s);

/* Create a C_N plan.  1 <= N <= 16, C_in >= 1, C_out >= 1, dt in {EQL_F32,
 * EQL_BF16, EQL_F16}; otherwise EQL_ERR_INVALID and *out is left NULL.  Host
 * metadata only: needs no GPU.  Release with eqlinear_plan_destroy. */
eqlinear_status eqlinear_plan(eqlinear_plan_t* out, int N, int C_in, int C_out,
                              eqlinear_dtype dt);

/* Create a D8 plan ("Quick ViTs", key design 2).  C_in and C_out are full
 * widths, multiples of 8 (C/8 channels per 1-D irrep, C/4 copies of E); dt in
 * {EQL_F32, EQL_BF16, EQL_F16}.  Same as
 * eqlinear_dihedral_plan(out, 4, C_in, C_out, dt). */
eqlinear_status eqlinear_d8_plan(eqlinear_plan_t* out, int C_in, int C_out,
                                 eqlinear_dtype dt);

/* Create a plan for the dihedral group D_n of the regular n-gon (order 2n,
 * 2 <= n <= 12; n = 4 is D8): the extension to other shapes that "Flash
 * EQ-Linear" (Dutch summary, closing paragraph) names, in the Fourier-domain
 * form of "Quick ViTs" key design 2.  D_n has 1-D irreps A1, A2 (and B1, B2 for
 * even n) and 2-D irreps E_k (k = 1 .. n/2 - 1 for even n, .. (n-1)/2 for odd
 * n; r turns by 2 pi k / n, s = diag(1, -1)).  C_in, C_out multiples of 2n;
 * m = C/2n.  Layout per token: the 1-D irreps' slabs of m, then for each E_k
 * a coordinate-0 and a coordinate-1 slab of 2m copies.  Weights packed
 * [W per 1-D irrep (m_out x m_in) | W per E_k (2m_out x 2m_in)], each [out][in];
 * a block of E_k acts on both of its coordinates.  Every eqlinear_d8_* call
 * and the comparator take these plans (kind EQL_KIND_D8, info.N = 2n,
 * info.bins = number of irrep blocks); dt as for eqlinear_d8_plan. */
eqlinear_status eqlinear_dihedral_plan(eqlinear_plan_t* out, int n, int C_in, int C_out,
                                       eqlinear_dtype dt);

/* Free a plan.  NULL -> EQL_ERR_INVALID. */
eqlinear_status eqlinear_plan_destroy(eqlinear_plan_t plan);

/* Fill *out with the plan's metadata. */
eqlinear_status eqlinear_plan_info(eqlinear_plan_t plan, eqlinear_info* out);

/* Number of elements of w_hat for a C_N plan (N*C_out*C_in), or of the packed
 * D8 blocks (C_in*C_out/8); 0 for a NULL plan. */
size_t eqlinear_w_hat_elems(eqlinear_plan_t plan);

/* Weight spectrum, computed once per weight ("Flash EQ-Linear", Algorithmic
 * Approach: DFT along the group axis, non-redundant half kept; Implementation:
 * a plug-and-play replacement for layers with trained weights).
 *   w     [C_out][C_in][N]   plan dtype, device
 *   w_hat [N][C_out][C_in]   plan dtype, device: N real planes of
 *         What[k] = sum_m w[m] exp(-2 pi i m k / N), unnormalised:
 *         plane 0 = Re What[0]; planes 2k-1, 2k = Re, Im What[k] (1 <= k < N/2);
 *         plane N-1 = Re What[N/2] when N is even.
 * Computed in fp64 and rounded once to the plan dtype.  Runs on the null
 * stream and returns after it completes (synchronous); the caller must have
 * finished writing w.  C_N plans only (EQL_ERR_INVALID for D8). */
eqlinear_status eqlinear_weight_fft(eqlinear_plan_t plan, const void* w, void* w_hat);

/* C_N forward, fused: per token tile, forward real DFT of x along the group
 * axis, the per-frequency channel products against w_hat (fp32 accumulation),
 * and the inverse DFT, writing y once ("Flash EQ-Linear", Algorithmic Approach
 * and Implementation: fused dataflow with no intermediate global writes).
 *   x     [T][C_in][N]  device, plan dtype
 *   w_hat [N][C_out][C_in] device, as written by eqlinear_weight_fft
 *   y     [T][C_out][N] device, plan dtype; must not overlap x or w_hat
 *   T >= 0 tokens (T == 0: returns EQL_OK, launches nothing)
 * 16-bit plans (bf16, fp16) round the frequency-domain inputs to the plan
 * dtype before the matrix cores and round y once from fp32; for 2 <= N <= 8
 * the transforms run on the matrix cores too, with coefficients in the plan
 * dtype, and the frequency-domain outputs are rounded to it before the inverse
 * transform (see eqlinear_forward_tiled for which kernel takes which shape). */
eqlinear_status eqlinear_forward(eqlinear_plan_t plan, const void* x, const void* w_hat,
                                 void* y, int64_t T, void* stream);

/* eqlinear_forward with a fixed tile configuration instead of the automatic
 * choice, for tuning and tests.  A workgroup covers 16*W tokens and 16*B output
 * channels (B is capped so that 4*N*B <= 192 accumulators per lane and the LDS
 * tiles fit):
 *   tile 0: W=4 B=6   1: W=4 B=5   2: W=4 B=4   3: W=4 B=3   4: W=4 B=2
 *   tile 5: W=1 B=2   6: W=1 B=1   -1: automatic (same as eqlinear_forward).
 * Tiles 7..13 are the shapes of tiles 0..6 on the kernel that runs the group
 * DFT and its inverse as block-diagonal matrix-core products (bf16 and fp16
 * plans with 2 <= N <= 8; other plans run tile - 7).  It rounds the transform
 * coefficients and the Fourier-domain outputs to the plan dtype, so its
 * results differ from the other tiles by that rounding; the automatic choice
 * uses it where it applies.  Tiles 14 and 15 (fp32 plans with N <= 10, C_in a multiple of
 * 4; other plans and shapes run tile 13) cover 16 tokens and 32 output channels (16
 * when C_out <= 16) with the input channels of every step split over 2 or 4
 * waves per output block, whose partial spectra are summed in a fixed order;
 * complex bins use three real products instead of four (Gauss's method), so
 * their results differ from the other tiles by fp32 rounding.  The automatic
 * choice uses tile 14 for fp32 layers too small for one wave per SIMD.  Shapes
 * with C_in not a multiple of 16 bytes of channels use a generic kernel with
 * fewer shapes.  Tile 16 (bf16 and fp16 plans with 2 <= N <= 8 and C_in, C_out
 * multiples of 8; otherwise the automatic choice among the others) is the
 * persistent kernel: one workgroup per CU and output slice of 48 channels, x
 * streamed into registers ahead of use, w_hat held in LDS; its transforms run
 * on the matrix cores like tiles 7..13, with 1/N folded into the forward
 * coefficients (and N into the inverse ones) so that no 16-bit intermediate
 * exceeds the range of x and y.  The automatic choice does not use it (it
 * measured slower than tiles 7..13 on MI355X).  Tile 17 (bf16 and fp16 plans
 * with 2 <= N <= 8; otherwise the automatic choice) is the kernel of tiles
 * 7..13 with 8 waves over 128 tokens x 48 output channels (64 for N = 7):
 * each weight chunk serves twice the tokens of the 4-wave tiles.  The
 * automatic choice takes it for layers of 81..96 output channels when the
 * token batch gives at least 192 tiles of 64 tokens, and for N = 7 layers of
 * more than 96 output channels whose tiles number at least 256.  Other tile
 * values -> EQL_ERR_INVALID. */
eqlinear_status eqlinear_forward_tiled(eqlinear_plan_t plan, const void* x, const void* w_hat,
                                       void* y, int64_t T, void* stream, int tile);

/* Activations that eqlinear_forward_bias_act can apply. */
typedef enum {
    EQL_ACT_NONE = 0, /* y = layer(x) + bias                                   */
    EQL_ACT_GELU = 1  /* y = GELU(layer(x) + bias), GELU(v) = v * Phi(v) =
                         v/2 * (1 + erf(v / sqrt 2)), the exact (erf) form     */
} eqlinear_act;

/* C_N forward with the layer's neighbours fused into the store: a per-channel
 * bias and an optional GELU ("Quick ViTs", key design 2: an MLP keeps its
 * pointwise nonlinearity, applied to the regular-representation (group-axis)
 * values, which a group element only permutes, so the block stays equivariant).
 *   y[t][o][g] = act(sum_{i,m} w[o][i][m] x[t][i][(g-m) mod N] + bias[o])
 * bias is constant along the group axis, as an equivariant bias must be.
 *   bias  [C_out] device, plan dtype, aligned to its element size, must not
 *         overlap y; NULL means no bias
 *   act   EQL_ACT_NONE or EQL_ACT_GELU (others -> EQL_ERR_INVALID)
 *   tile  as for eqlinear_forward_tiled (-1: automatic)
 * The bias add and the activation run in fp32 on the fp32 layer output
 * before its one rounding to the plan dtype; everything else (arguments,
 * layouts, precision, T == 0, asynchrony) is as for eqlinear_forward.
 * With bias == NULL and act == EQL_ACT_NONE it equals eqlinear_forward_tiled. */
eqlinear_status eqlinear_forward_bias_act(eqlinear_plan_t plan, const void* x, const void* w_hat,
                                          const void* bias, int act, void* y, int64_t T, void* stream,
                                          int tile);

/* D8 layer's pointwise neighbours in the regular representation ("Quick ViTs",
 * key design 2: GELU does not commute with a general representation, so the
 * features go back to the regular representation, where the group only
 * permutes coordinates, GELU acts there, and they return to the Fourier
 * domain; the page fuses this round trip into one kernel).
 *   y_in, y_out [T][C_out] D8 Fourier layout (as eqlinear_d8_forward writes),
 *         plan dtype, 16-byte aligned; y_out == y_in (in place) or apart
 *   bias  [C_out/8] plan dtype, one value per regular channel (constant over
 *         the 8 group elements, as an equivariant bias must be), aligned to
 *         its element size, not overlapping y_out; NULL means no bias
 *   act   EQL_ACT_NONE or EQL_ACT_GELU (others -> EQL_ERR_INVALID)
 * Per token and regular channel j (m = C_out/8): its 8 Fourier features
 * (A1, A2, B1, B2 at j; E copies 2j and 2j+1 -- the columns of its E
 * coefficient matrix -- in the coordinate-0 and coordinate-1 slabs) go to its
 * values at the 8 group elements by the group's orthonormal Fourier matrix
 * F^T, become act(f + bias[j]) in fp32, and return through F; one rounding to
 * the plan dtype.  Element q = a + 4b is r^a s^b with the layer's generators
 * (E(r) = [[0,-1],[1,0]], E(s) = diag(1,-1)).  With no bias and no activation
 * the pass is the identity up to that rounding.  Dihedral plans of other orders
 * (eqlinear_dihedral_plan) take the same pass with their own Fourier matrix:
 * 2n values per channel, rows sqrt(1/2n) times the 1-D irreps and sqrt(2/2n)
 * times the entries (k, c) of E_k, element q = a + n b; bias [C_out/2n].  C_N
 * plans -> EQL_ERR_INVALID; T == 0: EQL_OK, nothing launched.  Asynchronous on
 * stream; no allocation. */
eqlinear_status eqlinear_d8_bias_act(eqlinear_plan_t plan, const void* y_in, const void* bias, int act,
                                     void* y_out, int64_t T, void* stream);

/* The two halves of that round trip alone, for D8 layers between regular-
 * representation features: eqlinear_d8_to_fourier takes x_reg [T][C_in/8][8]
 * (regular channel j's values at the 8 group elements) to the Fourier layout
 * x_four [T][C_in] that eqlinear_d8_forward consumes; eqlinear_d8_to_regular
 * takes the layer's output y_four [T][C_out] to y_reg [T][C_out/8][8].  Same
 * transform, layouts and rules as eqlinear_d8_bias_act (fp32 arithmetic, one
 * rounding), except that input and output must not overlap. */
eqlinear_status eqlinear_d8_to_fourier(eqlinear_plan_t plan, const void* x_reg, void* x_four, int64_t T,
                                       void* stream);
eqlinear_status eqlinear_d8_to_regular(eqlinear_plan_t plan, const void* y_four, void* y_reg, int64_t T,
                                       void* stream);

/* The dihedral layer between regular-representation features, in one launch
 * ("Quick ViTs", key design 2: the MLP keeps its features in the regular
 * representation, where the group only permutes each channel's values and
 * GELU acts pointwise; the linear map is block-diagonal in the group-Fourier
 * basis; the page fuses the transforms and GELU around the products):
 *   y_reg = act( to_regular( layer( to_fourier(x_reg) ) ) + b )
 * i.e. eqlinear_d8_to_fourier, eqlinear_d8_forward, and the regular half of
 * eqlinear_d8_bias_act, with no Fourier-domain tensor in memory.
 *   x_reg [T][C_in/G][G], y_reg [T][C_out/G][G] (G = the plan's group order;
 *     regular channel j's values at the G group elements, as for
 *     eqlinear_d8_to_fourier);
 *   wb    the packed blocks, as for eqlinear_d8_forward;
 *   bias  NULL or C_out/G values, one per output regular channel (constant
 *         over the group elements, so the block stays equivariant);
 *   act   EQL_ACT_NONE or EQL_ACT_GELU (the erf form).
 * The group-Fourier transform and its inverse run in fp32; the Fourier
 * features of x are rounded once to the plan dtype for the matrix-core
 * products (fp32 accumulation); y is rounded once.  Device pointers, plan
 * dtype, 16-byte aligned (bias: element-aligned); y_reg must not overlap
 * x_reg, wb or bias.  Asynchronous on stream; no allocation; T == 0: EQL_OK.
 * EQL_ERR_UNSUPPORTED for fp32 plans and for C_in/G or C_out/G not a multiple
 * of 8 (use the three separate calls); EQL_ERR_INVALID for C_N plans. */
eqlinear_status eqlinear_d8_regular_forward(eqlinear_plan_t plan, const void* x_reg, const void* wb,
                                            const void* bias, int act, void* y_reg, int64_t T, void* stream);

/* Backward pass ("Flash EQ-Linear", Implementation: the kernels cover forward
 * and backward; Experimental Results, Operator Level, backward pass).  The
 * pages give no formulas; these are the derivatives of the layer
 * y[t][o][g] = sum_{i,m} w[o][i][m] x[t][i][(g-m) mod N] for an upstream
 * gradient dy = dL/dy [T][C_out][N]:
 *   dx[t][i][h] = sum_{o,g} w[o][i][(g-h) mod N] dy[t][o][g]
 *   dw[o][i][m] = sum_{t,g} dy[t][o][g] x[t][i][(g-m) mod N]
 *
 * eqlinear_w_hat_adjoint: the spectrum of the adjoint layer, once per weight:
 *   w_hat_adj[p][i][o] = w_hat[p][o][i] on real planes, -w_hat[p][o][i] on
 *   imaginary planes (planes 2k, 1 <= k < N/2) -- conj(What[k])^T, the w_hat
 *   of the layer with C_in and C_out exchanged and the group axis reversed.
 *   Both device buffers hold N*C_in*C_out plan-dtype elements, 16-byte
 *   aligned, not overlapping.  Asynchronous on stream; no allocation.
 *   C_N plans only (EQL_ERR_INVALID otherwise). */
eqlinear_status eqlinear_w_hat_adjoint(eqlinear_plan_t plan, const void* w_hat, void* w_hat_adj,
                                       void* stream);

/* Input gradient: dx [T][C_in][N] from dy [T][C_out][N] and w_hat_adj (as
 * written by eqlinear_w_hat_adjoint), computed by the forward kernels on the
 * exchanged-channel layer (same precision contract as eqlinear_forward).
 * Device pointers, plan dtype, 16-byte aligned; dx must not overlap dy or
 * w_hat_adj.  T == 0: EQL_OK, nothing launched.  Asynchronous on stream. */
eqlinear_status eqlinear_backward_data(eqlinear_plan_t plan, const void* dy, const void* w_hat_adj,
                                       void* dx, int64_t T, void* stream);

/* Bytes of device workspace that eqlinear_backward_weight needs for T tokens
 * (0 for T <= 0 or a non-C_N plan). */
size_t eqlinear_backward_weight_workspace(eqlinear_plan_t plan, int64_t T);

/* Weight gradient: dw [C_out][C_in][N] in fp32 (overwritten, for either plan
 * dtype) from x [T][C_in][N] and dy [T][C_out][N] in the plan dtype.  Computed
 * in the frequency domain: real DFT of every record of x and dy along the
 * group axis (fp32, stored in the plan dtype in the workspace), per kept bin
 * the products C_k = sum_t DY[t][o][k] conj(X[t][i][k]) on the matrix cores
 * with fp32 accumulation over token ranges, the ranges' partials summed in a
 * fixed order (results are deterministic), then the inverse real DFT.
 * workspace: device, 256-byte aligned, at least
 * eqlinear_backward_weight_workspace(plan, T) bytes, owned by the caller and
 * not overlapping x, dy or dw; its contents are scratch.  x, dy, dw 16-byte
 * aligned.  T == 0 writes zeros to dw.  Asynchronous on stream; no allocation.
 * EQL_ERR_INVALID for a D8 plan, bad pointers, overlap or a short workspace;
 * EQL_ERR_UNSUPPORTED when the transformed x or dy held in
 * the workspace would reach 2 GiB (N C T S bytes each, S the element size; for
 * N = 7, C = 160, bf16 that is about 958 000 tokens): split the tokens into
 * parts and add the parts' gradients. */
eqlinear_status eqlinear_backward_weight(eqlinear_plan_t plan, const void* x, const void* dy, float* dw,
                                         int64_t T, void* workspace, size_t workspace_bytes, void* stream);

/* Largest workspace eqlinear_backward_weight_noalloc can serve: the size of
 * its library-held scratch array on each GPU. */
#define EQL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Weight gradient without allocation and without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Computes exactly what
 * eqlinear_backward_weight computes (same kernels, same fixed summation order,
 * so the same bits), with the workspace taken from a device array of
 * EQL_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  It calls no hipMalloc/hipFree.
 *   x, dy, dw, T: as for eqlinear_backward_weight.
 *   stream: a stream of the current device (NULL: the null stream); the
 *   current device's array is used.
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (nothing in it needs to start at zero).  Calls that overlap
 * on one GPU (several streams, or host threads) race on it: serialise them.
 * EQL_ERR_UNSUPPORTED, before any launch, when the shape's workspace
 * (eqlinear_backward_weight_workspace) exceeds EQL_NOALLOC_SCRATCH_BYTES (use
 * eqlinear_backward_weight, or split the tokens and add the gradients);
 * EQL_ERR_INVALID as for eqlinear_backward_weight, or for a stream of another
 * device.  Asynchronous on stream.  T == 0 writes zeros to dw. */
eqlinear_status eqlinear_backward_weight_noalloc(eqlinear_plan_t plan, const void* x, const void* dy, float* dw,
                                                 int64_t T, void* stream);

/* D8 forward: y_rho = W_rho x_rho for rho in A1, A2, B1, B2 and
 * y_Ec = W_E x_Ec for both E coordinates c ("Quick ViTs", key design 2).
 *   x  [T][C_in], y [T][C_out], features laid out [A1|A2|B1|B2|E0|E1] with
 *      widths (m, m, m, m, 2m, 2m), m = C/8
 *   wb packed [W_A1 | W_A2 | W_B1 | W_B2 | W_E], each row-major [out][in]:
 *      1-D blocks (C_out/8 x C_in/8), W_E (C_out/4 x C_in/4) */
eqlinear_status eqlinear_d8_forward(eqlinear_plan_t plan, const void* x, const void* wb,
                                    void* y, int64_t T, void* stream);

/* Comparator: expand weights into the dense matrix a replicate-and-multiply
 * implementation would use ("Flash EQ-Linear", Problem Statement).
 *   C_N: W_dense [N*C_out][N*C_in] with W_dense[o*N+g][i*N+h] = w[o][i][(g-h) mod N]
 *        from w [C_out][C_in][N]
 *   D8:  W_dense [C_out][C_in], block-diagonal, from the packed blocks
 * Asynchronous on stream.  Plan dtype. */
eqlinear_status eqlinear_expand_dense(eqlinear_plan_t plan, const void* w, void* w_dense,
                                      void* stream);

/* Comparator: plain dense product y[t] = W_dense x[t] (F.linear without bias)
 * on the matrix cores, x [T][K], W_dense [M][K], y [T][M] with K, M the full
 * input and output widths of the plan. */
eqlinear_status eqlinear_dense_forward(eqlinear_plan_t plan, const void* x,
                                       const void* w_dense, void* y, int64_t T, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EQLINEAR_H */
