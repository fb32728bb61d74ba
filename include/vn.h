/*
 * vn.h -- C ABI of the virtual-noise evolution-strategies linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one documented on the EvoX API page
 * "evox.triton_kernels.kernels.virtual_noise": a population of individuals
 * i = 0..pop-1 each sees the weights perturbed by its own noise matrix N_i,
 * which is never stored but regenerated from (seed_i, flat element index):
 *
 *   forward   Y[i] = X[i] (W + sigma N_i)^T + (b + sigma nb_i)       (module intro, model equation)
 *   gradient  grad_W[j,k] = sum_i f_i N_i[j,k] / (pop sigma)        (module intro, gradient equation)
 *             grad_b[j]   = sum_i f_i nb_i[j]  / (pop sigma)        (API entry virtual_bias_gradient)
 *
 * Noise (page sections "RNG: fast centered-uniform approximation" and
 * "Noise indexing scheme", API entries _splitmix64_step and _cpu_normal_noise):
 *   s    = seed_i as a 64-bit two's-complement pattern (int32 seeds sign-extended)
 *   z    = s + (idx + 1) * 0x9E3779B97F4A7C15                      (mod 2^64)
 *   z    = (z ^ (z >> 30)) * 0x9E3779B97F4A7C15;  z = (z ^ (z >> 27)) * 0x9E3779B97F4A7C15;
 *   r    = low 32 bits of (z ^ (z >> 31))
 *   N    = (r >> 8) * 2^-24 - 0.5                                 in [-0.5, 0.5), exact in fp32
 *   idx  = offset + j*in + k for weight (j,k); offset + out*in + j for the bias in the forward.
 * How the seed and the index form the state, the finalizer multipliers and
 * the r -> N mapping are readings of the page (it leaves them open); they are
 * fixed here and used identically by every entry point.
 *
 * Conventions for every entry point below:
 *  - All pointers except those of vn_compute_offsets are DEVICE pointers owned
 *    by the caller.  The library keeps no state between calls and allocates
 *    no memory: the entry points that use scratch space (vn_reduce_metric, and
 *    vn_perturbed_linear for large batches) take it from the caller; the one
 *    exception, vn_reduce_metric_noalloc, uses a fixed device array described
 *    at its declaration.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *    VN_OK means "validated and enqueued"; outputs are valid once the stream
 *    reaches the launch.  Arguments are validated before any HIP call and a
 *    failure is returned as a vn_status with nothing enqueued; the library
 *    never aborts.  A zero extent (pop, batch, out, n ...) returns VN_OK
 *    without a launch.
 *  - Arrays are dense and row-major.  Floating point inputs are fp32 unless a
 *    vn_dtype argument says otherwise; outputs are fp32.
 *  - Results are deterministic: the same inputs give bit-identical outputs on
 *    every call (no atomics; all reductions run in a fixed order that depends
 *    only on the sizes).
 *  - Calls that write overlapping outputs on the same device must be ordered
 *    by the caller (same stream or events).
 */
#ifndef VN_H_
#define VN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VN_ABI_VERSION 3

typedef enum vn_status {
  VN_OK = 0,
  VN_ERR_NULL = 1,      /* a required pointer is NULL while its extent is > 0            */
  VN_ERR_SHAPE = 2,     /* negative size, or x_pop_stride not in {0, batch*in}           */
  VN_ERR_VALUE = 3,     /* sigma not finite, sigma == 0 in a gradient, pop_size <= 0 in
                           a gradient, offset < 0, unknown activation or math mode      */
  VN_ERR_DTYPE = 4,     /* unknown vn_dtype / vn_index_dtype                             */
  VN_ERR_OVERFLOW = 5,  /* offset + out*in + out, a size product or a prefix sum
                           exceeds INT64_MAX, or a grid dimension limit is exceeded      */
  VN_ERR_HIP = 6,       /* the HIP runtime reported an error at launch                   */
  VN_ERR_ALIGN = 7      /* a pointer is not aligned to its element size                  */
} vn_status;

typedef enum vn_dtype {
  VN_F32 = 0,           /* IEEE binary32                                                 */
  VN_BF16 = 1           /* bfloat16 (upper half of a binary32)                           */
} vn_dtype;

typedef enum vn_index_dtype {
  VN_I64 = 0,           /* int64 seeds                                                   */
  VN_I32 = 1            /* int32 seeds, sign-extended to 64 bits                         */
} vn_index_dtype;

typedef enum vn_activation {
  VN_ACT_NONE = 0,      /* Y as defined above                                            */
  VN_ACT_RELU = 1       /* max(Y, 0) applied in the same kernel (for chaining layers)    */
} vn_activation;

typedef enum vn_math {
  VN_MATH_DEFAULT = 0,  /* bf16 operands: one bf16 matrix-core product per element pair.
                           fp32 operands: each operand split into bf16 hi + lo, products
                           hi*hi + hi*lo + lo*hi on the bf16 matrix cores (relative error
                           about 2^-16 per product), fp32 accumulation                    */
  VN_MATH_F32 = 1       /* fp32 operands only: fp32 matrix-core products, fp32 accumulation.
                           Slower on gfx950, where fp32 MFMAs do not overlap the hash    */
} vn_math;

/* Human-readable name of a status code (static string, never NULL). */
const char* vn_status_string(int status);

/* VN_ABI_VERSION of the built library. */
int vn_abi_version(void);

/* Text of the last HIP error seen by this thread ("" if none); static storage. */
const char* vn_last_hip_error(void);

/*
 * compute_offsets (API entry compute_offsets): starting flat noise offset of
 * each parameter block = element count of all blocks before it.
 *   dims      HOST, concatenated shape dims of all blocks (sum(ndims) entries)
 *   ndims     HOST, rank of each block (n_blocks entries); rank 0 = scalar = 1 element
 *   n_blocks  >= 0
 *   offsets_out HOST, n_blocks entries (written only on VN_OK)
 *   total_out HOST or NULL: total element count
 * Errors: VN_ERR_NULL, VN_ERR_SHAPE (negative dim or rank), VN_ERR_OVERFLOW.
 * Example from the page: shapes [(256,784),(256,),(10,256),(10,)] give
 * offsets [0, 200704, 200960, 203520].
 */
int vn_compute_offsets(const int64_t* dims, const int32_t* ndims, int32_t n_blocks,
                       int64_t* offsets_out, int64_t* total_out);

/*
 * Perturbed linear forward (API entry virtual_perturbed_linear):
 *   y[i,b,j] = sum_k x_i[b,k] (w[j,k] + sigma N_i[j,k]) + (bias[j] + sigma nb_i[j])
 * for i < pop, b < batch, j < out, with N_i[j,k] at index offset + j*in + k and
 * nb_i[j] at offset + out*in + j.
 *   x             (batch, in) rows of individual i start at x + i*x_pop_stride
 *                 elements; x_pop_stride is batch*in (per-individual inputs,
 *                 shape (pop,batch,in)) or 0 (one (batch,in) input shared by all)
 *   w             (out, in), same dtype as x (VN_F32 or VN_BF16)
 *   bias          (out,) fp32, or NULL for no bias term and no bias noise
 *   seeds         (pop,) int64 or int32 (seed_dtype)
 *   sigma         perturbation scale (finite; 0 gives the plain linear layer)
 *   offset        flat noise offset of this weight block (>= 0)
 *   activation    VN_ACT_NONE or VN_ACT_RELU
 *   math          vn_math (VN_MATH_F32 requires dtype VN_F32)
 *   y             (pop, batch, out) fp32 output
 *   workspace     DEVICE scratch of workspace_bytes (16-byte aligned), or NULL
 *                 with workspace_bytes 0.  When it holds at least
 *                 vn_perturbed_linear_workspace_size bytes for these sizes (bf16
 *                 operands, many rows per individual, at least 256 outputs;
 *                 16-byte aligned x and w), the perturbed weights of groups of individuals are formed
 *                 there once and multiplied on the matrix cores; otherwise the
 *                 noise is generated inside the product.  Both give the same
 *                 bits.  The library only reads what it wrote there during the
 *                 call; calls sharing a workspace must be ordered by the caller.
 * W + sigma*N is always formed in fp32 (one fma).  The bf16 variant rounds it
 * to bf16 (nearest even) before the product; the fp32 variant keeps it to
 * about 16 significant bits (VN_MATH_DEFAULT) or to fp32 (VN_MATH_F32).
 * Errors also: VN_ERR_SHAPE for workspace_bytes < 0, VN_ERR_ALIGN for a
 * workspace not 16-byte aligned.
 */
int vn_perturbed_linear(const void* x, int64_t x_pop_stride, const void* w, int32_t dtype,
                        const float* bias, const void* seeds, int32_t seed_dtype,
                        int64_t pop, int64_t batch, int64_t in, int64_t out,
                        float sigma, int64_t offset, int32_t activation, int32_t math,
                        float* y, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Device workspace, in bytes, with which vn_perturbed_linear takes its
 * materialized-weights path for these sizes; 0 when the sizes do not take it
 * (fp32 operands, fewer than 2048 rows per individual, fewer than 256 outputs,
 * in not a multiple of 64 in [128, 2^22)).  At most 256 MiB, or one individual's out*in bf16 values
 * when that is larger.  Errors: VN_ERR_NULL (bytes_out), VN_ERR_DTYPE,
 * VN_ERR_SHAPE (negative size), VN_ERR_VALUE (math), VN_ERR_OVERFLOW.
 */
int vn_perturbed_linear_workspace_size(int32_t dtype, int64_t pop, int64_t batch, int64_t in, int64_t out,
                                       int32_t math, int64_t* bytes_out);

/*
 * A chain of perturbed layers in one call: the model equation applied
 * layer after layer as an MLP evaluates it (API entry virtual_perturbed_linear
 * per layer, the parameter blocks chained as in compute_offsets):
 *   h_0 = x_i,   h_{l+1} = act(h_l (W_l + sigma N_i^(l))^T + (b_l + sigma nb_i^(l)))
 *   y[i] = h_{n_layers}   (act is applied between layers, not after the last)
 * Layer l's weight noise is at offsets[l] + j*in_l + k and its bias noise at
 * offsets[l] + out_l*in_l + j: each layer is vn_perturbed_linear with that
 * offset, and the call equals n_layers such calls with fp32 activations
 * passed between them, except that the intermediate activations never leave
 * the GPU's on-chip memory and the chain is one launch.
 *   n_layers   1..8
 *   dims       HOST, n_layers + 1 widths (in_0, out_0 = in_1, ...): in_0 >= 1,
 *              every output width 1..256
 *   weights    HOST array of n_layers DEVICE pointers: (dims[l+1], dims[l]) in `dtype`
 *   biases     HOST array of n_layers DEVICE pointers to fp32 (dims[l+1],) or NULL
 *              entries (no bias term and no bias noise); NULL = no biases at all
 *   offsets    HOST, n_layers weight-block noise offsets (>= 0)
 *   x          (batch, dims[0]) rows of individual i at x + i*x_pop_stride
 *              elements (x_pop_stride = batch*dims[0], or 0 for a shared input)
 *   batch      0..64
 *   activation VN_ACT_NONE or VN_ACT_RELU, between layers
 *   y          (pop, batch, dims[n_layers]) fp32
 * Precision as vn_perturbed_linear's default math for more than 4 rows (fp32
 * operands as three bf16 products); for VN_BF16 the
 * intermediate activations are rounded to bf16 (nearest even), as a caller
 * feeding the next bf16 layer would.  Errors: VN_ERR_SHAPE for an output
 * width outside 1..256, in_0 < 1, batch > 64 or n_layers outside 1..8;
 * VN_ERR_OVERFLOW when batch*in_0 or a layer's last noise index overflows
 * int64; VN_ERR_VALUE also for
 * 0 < |sigma| < 2^-100 (take such layers through vn_perturbed_linear).
 */
int vn_perturbed_mlp(const void* x, int64_t x_pop_stride, int32_t dtype, int32_t n_layers,
                     const int64_t* dims, const void* const* weights, const float* const* biases,
                     const int64_t* offsets, const void* seeds, int32_t seed_dtype, int64_t pop,
                     int64_t batch, float sigma, int32_t activation, float* y, void* stream);


/*
 * Weight gradient (API entry virtual_weight_gradient):
 *   grad_w[j,k] = sum_i fitness[i] N_i[j,k] / (pop_size sigma),  N_i at offset + j*in + k
 *   fitness  (pop_size,) fp32;  seeds (pop_size,) int64 or int32
 *   grad_w   (out, in) fp32 output
 * pop_size must be > 0 and equal the length of fitness and seeds; sigma must
 * be finite and non-zero.  1/(pop_size sigma) is formed in double and rounded
 * to fp32 once.
 */
int vn_weight_gradient(const float* fitness, const void* seeds, int32_t seed_dtype,
                       int64_t pop_size, int64_t out, int64_t in, float sigma, int64_t offset,
                       float* grad_w, void* stream);

/*
 * Bias gradient (API entry virtual_bias_gradient):
 *   grad_b[j] = sum_i fitness[i] nb_i[j] / (pop_size sigma),  nb_i at offset + j
 * where `offset` already points at the bias region (weight offset + out*in),
 * as the page asks of callers.  Same rules as vn_weight_gradient.
 */
int vn_bias_gradient(const float* fitness, const void* seeds, int32_t seed_dtype,
                     int64_t pop_size, int64_t out, float sigma, int64_t offset,
                     float* grad_b, void* stream);

/*
 * Flat gradient over any span of the parameter vector (the estimator of the
 * gradient equation applied to n consecutive flat elements starting at offset):
 *   grad[t] = sum_i fitness[i] noise_i[offset + t] / (pop_size sigma),  t < n
 * vn_weight_gradient and vn_bias_gradient are this with n = out*in and n = out.
 */
int vn_flat_gradient(const float* fitness, const void* seeds, int32_t seed_dtype,
                     int64_t pop_size, int64_t n, float sigma, int64_t offset,
                     float* grad, void* stream);

/*
 * Device workspace, in bytes, that vn_reduce_metric needs for (pop, n_params):
 * 0 from 512 individuals on or below 131072 parameters, otherwise
 * pop * segments * 4 with pop * segments < 1536 (at most 6 KiB).
 *   bytes_out  HOST
 * Errors: VN_ERR_NULL (bytes_out), VN_ERR_SHAPE (negative size).
 */
int vn_reduce_metric_workspace_size(int64_t pop, int64_t n_params, int64_t* bytes_out);

/*
 * Mean-absolute reduction metric (API entry virtual_reduce_metric):
 *   out[i] = (1/n_params) sum_k | center[k] + sigma noise_i[offset + k] |
 *   center     (n_params,) fp32;  out (pop,) fp32;  n_params > 0 when pop > 0.
 *   workspace  DEVICE scratch of workspace_bytes >= vn_reduce_metric_workspace_size
 *              (may be NULL when that size is 0); 4-byte aligned.  A population
 *              below 512 splits each individual's sum into segments whose partial
 *              sums go there; its contents on entry do not matter, and calls that
 *              share a workspace must be ordered by the caller.
 * Every sum has a fixed order for each (pop, n_params), so repeated calls are
 * bit-identical.  Errors: VN_ERR_NULL for a missing workspace, VN_ERR_SHAPE for
 * one smaller than needed.
 */
int vn_reduce_metric(const float* center, const void* seeds, int32_t seed_dtype, int64_t pop,
                     int64_t n_params, float sigma, int64_t offset, float* out,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * vn_reduce_metric without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under stream capture into
 * a graph, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, result and summation order as vn_reduce_metric.  Its partial sums
 * live in a fixed array of 8 KiB in each GPU's memory, held from the first
 * call on that GPU until the process ends; every (pop, n_params) needs at most
 * 6 KiB of it (VN_ERR_OVERFLOW would report a larger need).  All calls on one
 * GPU share that array: calls that may overlap on one GPU (different streams,
 * other threads) race and must be ordered by the caller.  VN_ERR_HIP if the
 * array's address cannot be obtained.
 */
int vn_reduce_metric_noalloc(const float* center, const void* seeds, int32_t seed_dtype, int64_t pop,
                             int64_t n_params, float sigma, int64_t offset, float* out, void* stream);

/*
 * Noise readout (API entry _cpu_normal_noise, here on the GPU with the same
 * device hash as every kernel above; for verification):
 *   r_out[i,t] = low 32 bits of the hash of (seed_i, offset + t)       (pop, n) uint32
 *   n_out[i,t] = (r >> 8) * 2^-24 - 0.5                                  (pop, n) fp32
 */
int vn_noise_u32(const void* seeds, int32_t seed_dtype, int64_t pop, int64_t n, int64_t offset,
                 uint32_t* r_out, void* stream);
int vn_noise_f32(const void* seeds, int32_t seed_dtype, int64_t pop, int64_t n, int64_t offset,
                 float* n_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VN_H_ */
