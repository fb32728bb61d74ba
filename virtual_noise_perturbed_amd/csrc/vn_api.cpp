// C ABI of the virtual-noise ES linear layer: argument validation and launch
// selection.  Every check runs before any HIP call; the kernels themselves are
// in vn_kernels.hip.  Declarations and the contract are in include/vn.h.

#include "vn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>

#include "vn_launch.hpp"

namespace {

constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();

thread_local char g_last_hip_error[256] = "";

bool mul_ok(int64_t a, int64_t b, int64_t* r) {  // a, b >= 0
  if (a != 0 && b > kI64Max / a) return false;
  *r = a * b;
  return true;
}
bool add_ok(int64_t a, int64_t b, int64_t* r) {  // a, b >= 0
  if (b > kI64Max - a) return false;
  *r = a + b;
  return true;
}

int seed_kind(int32_t seed_dtype, bool* is_i32) {
  if (seed_dtype == VN_I64) { *is_i32 = false; return VN_OK; }
  if (seed_dtype == VN_I32) { *is_i32 = true; return VN_OK; }
  return VN_ERR_DTYPE;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return VN_OK;
  std::strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  return VN_ERR_HIP;
}

// Shared checks of the gradient-style entry points over n flat elements.
int check_gradient(const float* fitness, const void* seeds, int32_t seed_dtype, int64_t pop_size, int64_t n,
                   float sigma, int64_t offset, const void* out, bool* i32, float* scale) {
  int st = seed_kind(seed_dtype, i32);
  if (st != VN_OK) return st;
  if (n < 0) return VN_ERR_SHAPE;
  if (pop_size <= 0) return VN_ERR_VALUE;
  if (!std::isfinite(sigma) || sigma == 0.0f) return VN_ERR_VALUE;
  if (offset < 0) return VN_ERR_VALUE;
  int64_t last;
  if (!add_ok(offset, n, &last)) return VN_ERR_OVERFLOW;
  if (fitness == nullptr || seeds == nullptr) return VN_ERR_NULL;
  if (n > 0 && out == nullptr) return VN_ERR_NULL;
  if (!aligned(fitness, 4) || !aligned(seeds, *i32 ? 4 : 8) || !aligned(out, 4)) return VN_ERR_ALIGN;
  const double s = 1.0 / (static_cast<double>(pop_size) * static_cast<double>(sigma));
  *scale = static_cast<float>(s);
  if (!std::isfinite(*scale)) return VN_ERR_VALUE;
  return VN_OK;
}

}  // namespace

extern "C" {

const char* vn_status_string(int status) {
  switch (status) {
    case VN_OK: return "ok";
    case VN_ERR_NULL: return "null pointer";
    case VN_ERR_SHAPE: return "invalid shape";
    case VN_ERR_VALUE: return "invalid value";
    case VN_ERR_DTYPE: return "invalid dtype";
    case VN_ERR_OVERFLOW: return "index or size overflow";
    case VN_ERR_HIP: return "HIP runtime error";
    case VN_ERR_ALIGN: return "misaligned pointer";
    default: return "unknown status";
  }
}

int vn_abi_version(void) { return VN_ABI_VERSION; }

const char* vn_last_hip_error(void) { return g_last_hip_error; }

int vn_compute_offsets(const int64_t* dims, const int32_t* ndims, int32_t n_blocks, int64_t* offsets_out,
                       int64_t* total_out) {
  if (n_blocks < 0) return VN_ERR_SHAPE;
  if (n_blocks > 0 && (ndims == nullptr || offsets_out == nullptr)) return VN_ERR_NULL;
  // Validate everything before writing any output.
  int64_t running = 0, pos = 0;
  for (int32_t b = 0; b < n_blocks; ++b) {
    if (ndims[b] < 0) return VN_ERR_SHAPE;
    if (ndims[b] > 0 && dims == nullptr) return VN_ERR_NULL;
    int64_t count = 1;
    for (int32_t d = 0; d < ndims[b]; ++d) {
      const int64_t v = dims[pos + d];
      if (v < 0) return VN_ERR_SHAPE;
      if (!mul_ok(count, v, &count)) return VN_ERR_OVERFLOW;
    }
    pos += ndims[b];
    if (!add_ok(running, count, &running)) return VN_ERR_OVERFLOW;
  }
  running = 0;
  pos = 0;
  for (int32_t b = 0; b < n_blocks; ++b) {
    offsets_out[b] = running;
    int64_t count = 1;
    for (int32_t d = 0; d < ndims[b]; ++d) count *= dims[pos + d];
    pos += ndims[b];
    running += count;
  }
  if (total_out != nullptr) *total_out = running;
  return VN_OK;
}

int vn_perturbed_linear_workspace_size(int32_t dtype, int64_t pop, int64_t batch, int64_t in, int64_t out,
                                       int32_t math, int64_t* bytes_out) {
  if (bytes_out == nullptr) return VN_ERR_NULL;
  if (dtype != VN_F32 && dtype != VN_BF16) return VN_ERR_DTYPE;
  if (pop < 0 || batch < 0 || in < 0 || out < 0) return VN_ERR_SHAPE;
  if (math != VN_MATH_DEFAULT && math != VN_MATH_F32) return VN_ERR_VALUE;
  int64_t oi;
  if (!mul_ok(out, in, &oi) || !mul_ok(oi, 2, &oi)) return VN_ERR_OVERFLOW;
  *bytes_out = 0;
  if (dtype == VN_BF16 && math == VN_MATH_DEFAULT && pop > 0 && vn::materialized_forward_applies(batch, in, out))
    *bytes_out = vn::materialized_workspace_bytes(pop, batch, in, out);
  return VN_OK;
}

int vn_perturbed_linear(const void* x, int64_t x_pop_stride, const void* w, int32_t dtype, const float* bias,
                        const void* seeds, int32_t seed_dtype, int64_t pop, int64_t batch, int64_t in, int64_t out,
                        float sigma, int64_t offset, int32_t activation, int32_t math, float* y, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  bool i32 = false;
  if (dtype != VN_F32 && dtype != VN_BF16) return VN_ERR_DTYPE;
  int st = seed_kind(seed_dtype, &i32);
  if (st != VN_OK) return st;
  if (pop < 0 || batch < 0 || in < 0 || out < 0) return VN_ERR_SHAPE;
  int64_t per_x;
  if (!mul_ok(batch, in, &per_x)) return VN_ERR_OVERFLOW;
  if (x_pop_stride != 0 && x_pop_stride != per_x) return VN_ERR_SHAPE;
  if (!std::isfinite(sigma)) return VN_ERR_VALUE;
  if (offset < 0) return VN_ERR_VALUE;
  if (activation != VN_ACT_NONE && activation != VN_ACT_RELU) return VN_ERR_VALUE;
  if (math != VN_MATH_DEFAULT && math != VN_MATH_F32) return VN_ERR_VALUE;
  if (math == VN_MATH_F32 && dtype != VN_F32) return VN_ERR_VALUE;
  // Largest noise index used: offset + out*in + out - 1 (bias); all in int64.
  int64_t oi, last, ysize, xsize;
  if (!mul_ok(out, in, &oi) || !add_ok(oi, out, &last) || !add_ok(offset, last, &last)) return VN_ERR_OVERFLOW;
  if (!mul_ok(pop, batch, &ysize) || !mul_ok(ysize, out, &ysize)) return VN_ERR_OVERFLOW;
  if (!mul_ok(pop, x_pop_stride, &xsize)) return VN_ERR_OVERFLOW;
  if (pop == 0 || batch == 0 || out == 0) return VN_OK;
  // The kernels take row tiles of up to 256 (fp32) on grid.y.
  if ((batch + 255) / 256 > 65535) return VN_ERR_OVERFLOW;
  if (y == nullptr || seeds == nullptr || (w == nullptr && in > 0) || (x == nullptr && in > 0)) return VN_ERR_NULL;
  const size_t esz = dtype == VN_F32 ? 4 : 2;
  if (!aligned(x, esz) || !aligned(w, esz) || !aligned(y, 4) || !aligned(bias, 4) ||
      !aligned(seeds, i32 ? 4 : 8))
    return VN_ERR_ALIGN;
  if (workspace_bytes < 0) return VN_ERR_SHAPE;
  if (!aligned(workspace, 16)) return VN_ERR_ALIGN;

  vn::FwdParams p;
  p.x = x;
  p.x_pop_stride = x_pop_stride;
  p.w = w;
  p.bias = bias;
  p.seeds = seeds;
  p.seeds_i32 = i32;
  p.pop = pop;
  p.batch = batch;
  p.in = in;
  p.out = out;
  p.sigma = sigma;
  p.sigma_q = sigma * 0x1p-24f;
  p.offset = offset;
  p.relu = activation == VN_ACT_RELU;
  p.y = y;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The fast kernels scale the integer noise by sigma * 2^-24, exact unless it
  // falls below the normal range; such a sigma takes the kernels that form
  // sigma * N in floating point.
  const bool tiny_sigma = sigma != 0.0f && std::fabs(sigma) < 0x1p-100f;
  if (dtype == VN_BF16) {
    if (tiny_sigma) return hip_status(vn::launch_forward_bf16_exact(p, s));
    // Many rows per individual: perturbed weights formed once in the caller's
    // workspace, then a matrix-core product (the same bits as the fused path).
    if (workspace != nullptr && vn::materialized_forward_applies(batch, in, out) &&
        workspace_bytes >= vn::materialized_workspace_bytes(pop, batch, in, out) && aligned(x, 16) && aligned(w, 16) &&
        x_pop_stride % 8 == 0)
      return hip_status(vn::launch_forward_bf16_materialized(p, workspace, s));
    return hip_status(vn::launch_forward_bf16(p, s));
  }
  return hip_status(math == VN_MATH_F32 || tiny_sigma ? vn::launch_forward_f32_exact(p, s)
                                                       : vn::launch_forward_f32(p, s));
}

int vn_flat_gradient(const float* fitness, const void* seeds, int32_t seed_dtype, int64_t pop_size, int64_t n,
                     float sigma, int64_t offset, float* grad, void* stream) {
  bool i32 = false;
  float scale = 0.0f;
  int st = check_gradient(fitness, seeds, seed_dtype, pop_size, n, sigma, offset, grad, &i32, &scale);
  if (st != VN_OK) return st;
  if (n == 0) return VN_OK;
  vn::GradParams p;
  p.fitness = fitness;
  p.seeds = seeds;
  p.seeds_i32 = i32;
  p.pop = pop_size;
  p.n = n;
  p.offset = offset;
  p.scale = scale;
  p.out = grad;
  return hip_status(vn::launch_gradient(p, static_cast<hipStream_t>(stream)));
}

int vn_perturbed_mlp(const void* x, int64_t x_pop_stride, int32_t dtype, int32_t n_layers, const int64_t* dims,
                     const void* const* weights, const float* const* biases, const int64_t* offsets,
                     const void* seeds, int32_t seed_dtype, int64_t pop, int64_t batch, float sigma,
                     int32_t activation, float* y, void* stream) {
  bool i32 = false;
  if (dtype != VN_F32 && dtype != VN_BF16) return VN_ERR_DTYPE;
  int st = seed_kind(seed_dtype, &i32);
  if (st != VN_OK) return st;
  if (n_layers < 1 || n_layers > vn::kChainMaxLayers) return VN_ERR_SHAPE;
  if (dims == nullptr || weights == nullptr || offsets == nullptr) return VN_ERR_NULL;
  if (pop < 0 || batch < 0 || batch > vn::kChainMaxBatch) return VN_ERR_SHAPE;
  for (int l = 0; l <= n_layers; ++l)
    if (dims[l] < 1 || (l > 0 && dims[l] > vn::kChainMaxWidth)) return VN_ERR_SHAPE;
  int64_t per_x;
  if (!mul_ok(batch, dims[0], &per_x)) return VN_ERR_OVERFLOW;
  if (x_pop_stride != 0 && x_pop_stride != per_x) return VN_ERR_SHAPE;
  if (!std::isfinite(sigma)) return VN_ERR_VALUE;
  if (sigma != 0.0f && std::fabs(sigma) < 0x1p-100f) return VN_ERR_VALUE;
  if (activation != VN_ACT_NONE && activation != VN_ACT_RELU) return VN_ERR_VALUE;
  for (int l = 0; l < n_layers; ++l) {
    // largest noise index of the layer: offset + out*in + out - 1
    if (offsets[l] < 0) return VN_ERR_VALUE;
    int64_t oi, last;
    if (!mul_ok(dims[l + 1], dims[l], &oi) || !add_ok(oi, dims[l + 1], &oi) || !add_ok(offsets[l], oi, &last))
      return VN_ERR_OVERFLOW;
  }
  int64_t ysize, xsize;
  if (!mul_ok(pop, batch, &ysize) || !mul_ok(ysize, dims[n_layers], &ysize)) return VN_ERR_OVERFLOW;
  if (!mul_ok(pop, x_pop_stride, &xsize)) return VN_ERR_OVERFLOW;
  if (pop == 0 || batch == 0) return VN_OK;
  if (pop > vn::kMaxGridX) return VN_ERR_OVERFLOW;
  if (x == nullptr || y == nullptr || seeds == nullptr) return VN_ERR_NULL;
  const size_t esz = dtype == VN_F32 ? 4 : 2;
  if (!aligned(x, esz) || !aligned(y, 4) || !aligned(seeds, i32 ? 4 : 8)) return VN_ERR_ALIGN;

  vn::ChainParams p;
  p.x = x;
  p.x_pop_stride = x_pop_stride;
  p.n_layers = n_layers;
  p.wvec = 0;
  for (int l = 0; l <= n_layers; ++l) p.dims[l] = dims[l];
  for (int l = 0; l < n_layers; ++l) {
    if (weights[l] == nullptr) return VN_ERR_NULL;
    if (!aligned(weights[l], esz)) return VN_ERR_ALIGN;
    const float* b = biases != nullptr ? biases[l] : nullptr;
    if (!aligned(b, 4)) return VN_ERR_ALIGN;
    p.w[l] = weights[l];
    p.bias[l] = b;
    p.offset[l] = offsets[l];
    if (aligned(weights[l], 16) && dims[l] % static_cast<int64_t>(16 / esz) == 0) p.wvec |= 1u << l;
  }
  p.relu = activation == VN_ACT_RELU;
  // the first layer's X chunks in 16-byte loads
  const int64_t per = static_cast<int64_t>(16 / esz);
  p.xvec = aligned(x, 16) && dims[0] % per == 0 && x_pop_stride % per == 0;
  p.seeds = seeds;
  p.seeds_i32 = i32;
  p.pop = pop;
  p.batch = batch;
  p.sigma = sigma;
  p.sigma_q = sigma * 0x1p-24f;
  p.y = y;
  return hip_status(vn::launch_chain(p, dtype == VN_BF16, static_cast<hipStream_t>(stream)));
}

int vn_weight_gradient(const float* fitness, const void* seeds, int32_t seed_dtype, int64_t pop_size, int64_t out,
                       int64_t in, float sigma, int64_t offset, float* grad_w, void* stream) {
  if (out < 0 || in < 0) return VN_ERR_SHAPE;
  int64_t n;
  if (!mul_ok(out, in, &n)) return VN_ERR_OVERFLOW;
  return vn_flat_gradient(fitness, seeds, seed_dtype, pop_size, n, sigma, offset, grad_w, stream);
}

int vn_bias_gradient(const float* fitness, const void* seeds, int32_t seed_dtype, int64_t pop_size, int64_t out,
                     float sigma, int64_t offset, float* grad_b, void* stream) {
  if (out < 0) return VN_ERR_SHAPE;
  return vn_flat_gradient(fitness, seeds, seed_dtype, pop_size, out, sigma, offset, grad_b, stream);
}

int vn_reduce_metric_workspace_size(int64_t pop, int64_t n_params, int64_t* bytes_out) {
  if (bytes_out == nullptr) return VN_ERR_NULL;
  if (pop < 0 || n_params < 0) return VN_ERR_SHAPE;
  *bytes_out = pop == 0 || n_params == 0 ? 0 : vn::reduce_metric_workspace_floats(pop, n_params) * 4;
  return VN_OK;
}

int vn_reduce_metric(const float* center, const void* seeds, int32_t seed_dtype, int64_t pop, int64_t n_params,
                     float sigma, int64_t offset, float* out, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  bool i32 = false;
  int st = seed_kind(seed_dtype, &i32);
  if (st != VN_OK) return st;
  if (pop < 0 || n_params < 0 || workspace_bytes < 0) return VN_ERR_SHAPE;
  if (!std::isfinite(sigma) || offset < 0) return VN_ERR_VALUE;
  int64_t last;
  if (!add_ok(offset, n_params, &last)) return VN_ERR_OVERFLOW;
  if (pop == 0) return VN_OK;
  if (n_params == 0) return VN_ERR_SHAPE;  // the mean of nothing is undefined
  if (center == nullptr || seeds == nullptr || out == nullptr) return VN_ERR_NULL;
  if (!aligned(center, 4) || !aligned(out, 4) || !aligned(seeds, i32 ? 4 : 8) || !aligned(workspace, 4))
    return VN_ERR_ALIGN;
  // A population too small to fill the GPU with one workgroup per individual
  // splits each individual into segments whose partial sums go to the
  // caller's workspace (vn_reduce_metric_workspace_size); there is one
  // summation order for each (pop, n_params).
  const int64_t need = vn::reduce_metric_workspace_floats(pop, n_params) * 4;
  if (need > 0 && workspace == nullptr) return VN_ERR_NULL;
  if (workspace_bytes < need) return VN_ERR_SHAPE;
  return hip_status(vn::launch_reduce_metric(center, seeds, i32, pop, n_params, sigma, offset, out,
                                             need > 0 ? static_cast<float*>(workspace) : nullptr,
                                             static_cast<hipStream_t>(stream)));
}

int vn_reduce_metric_noalloc(const float* center, const void* seeds, int32_t seed_dtype, int64_t pop,
                             int64_t n_params, float sigma, int64_t offset, float* out, void* stream) {
  bool i32 = false;
  int st = seed_kind(seed_dtype, &i32);
  if (st != VN_OK) return st;
  if (pop < 0 || n_params < 0) return VN_ERR_SHAPE;
  if (!std::isfinite(sigma) || offset < 0) return VN_ERR_VALUE;
  int64_t last;
  if (!add_ok(offset, n_params, &last)) return VN_ERR_OVERFLOW;
  if (pop == 0) return VN_OK;
  if (n_params == 0) return VN_ERR_SHAPE;
  if (center == nullptr || seeds == nullptr || out == nullptr) return VN_ERR_NULL;
  if (!aligned(center, 4) || !aligned(out, 4) || !aligned(seeds, i32 ? 4 : 8)) return VN_ERR_ALIGN;
  const int64_t need = vn::reduce_metric_workspace_floats(pop, n_params);
  if (need > vn::kMetricScratchFloats) return VN_ERR_OVERFLOW;   // beyond the fixed scratch array
  float* work = nullptr;
  if (need > 0) {
    const hipError_t e = vn::metric_scratch_address(&work);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(vn::launch_reduce_metric(center, seeds, i32, pop, n_params, sigma, offset, out, work,
                                             static_cast<hipStream_t>(stream)));
}

static int noise_common(const void* seeds, int32_t seed_dtype, int64_t pop, int64_t n, int64_t offset,
                        uint32_t* r_out, float* n_out, void* out_ptr, void* stream) {
  bool i32 = false;
  int st = seed_kind(seed_dtype, &i32);
  if (st != VN_OK) return st;
  if (pop < 0 || n < 0) return VN_ERR_SHAPE;
  if (offset < 0) return VN_ERR_VALUE;
  int64_t last, total;
  if (!add_ok(offset, n, &last) || !mul_ok(pop, n, &total)) return VN_ERR_OVERFLOW;
  if (total == 0) return VN_OK;
  if (seeds == nullptr || out_ptr == nullptr) return VN_ERR_NULL;
  if (!aligned(out_ptr, 4) || !aligned(seeds, i32 ? 4 : 8)) return VN_ERR_ALIGN;
  return hip_status(vn::launch_noise(seeds, i32, pop, n, offset, r_out, n_out, static_cast<hipStream_t>(stream)));
}

int vn_noise_u32(const void* seeds, int32_t seed_dtype, int64_t pop, int64_t n, int64_t offset, uint32_t* r_out,
                 void* stream) {
  return noise_common(seeds, seed_dtype, pop, n, offset, r_out, nullptr, r_out, stream);
}

int vn_noise_f32(const void* seeds, int32_t seed_dtype, int64_t pop, int64_t n, int64_t offset, float* n_out,
                 void* stream) {
  return noise_common(seeds, seed_dtype, pop, n, offset, nullptr, n_out, n_out, stream);
}

}  // extern "C"
