// Internal launch interface between the C ABI (vn_api.cpp) and the kernels
// (vn_kernels.hip).  Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vn {

struct FwdParams {
  const void* x;
  int64_t x_pop_stride;  // elements between individuals' inputs (0 = shared)
  const void* w;
  const float* bias;     // may be null
  const void* seeds;
  bool seeds_i32;
  int64_t pop, batch, in, out;
  float sigma;
  float sigma_q;         // sigma * 2^-24 (exact): multiplier of the integer noise (r >> 8) - 2^23
  int64_t offset;
  bool relu;
  float* y;
};

struct GradParams {
  const float* fitness;
  const void* seeds;
  bool seeds_i32;
  int64_t pop;
  int64_t n;        // elements
  int64_t offset;   // absolute flat index of element 0
  float scale;      // 1 / (pop * sigma), rounded once from double
  float* out;
};

// A chain of layers evaluated in one launch (vn_perturbed_mlp).
constexpr int kChainMaxLayers = 8;
constexpr int kChainMaxWidth = 256;   // every layer's out (the first layer's in is free)
constexpr int kChainMaxBatch = 64;
struct ChainParams {
  const void* x;                      // (batch, dims[0]) per individual
  int64_t x_pop_stride;
  int32_t n_layers;
  int64_t dims[kChainMaxLayers + 1];
  const void* w[kChainMaxLayers];     // (dims[l+1], dims[l])
  const float* bias[kChainMaxLayers]; // may be null
  int64_t offset[kChainMaxLayers];    // weight-block noise offset of each layer
  bool relu;                          // ReLU between layers (not after the last)
  uint32_t wvec;                      // bit l: w[l] takes 16-byte loads
  bool xvec;                          // x rows take 16-byte loads (aligned, dims[0] and stride whole vectors)
  const void* seeds;
  bool seeds_i32;
  int64_t pop, batch;
  float sigma, sigma_q;
  float* y;                           // (pop, batch, dims[n_layers])
};

// Each returns hipSuccess or the launch error.
hipError_t launch_forward_f32(const FwdParams& p, hipStream_t stream);        // split-bf16 matrix cores
hipError_t launch_forward_f32_exact(const FwdParams& p, hipStream_t stream);  // fp32 matrix cores
hipError_t launch_forward_bf16(const FwdParams& p, hipStream_t stream);
// bf16 operands with the noise formed in floating point (sigma * N): for a
// sigma too small for sigma * 2^-24 to be a normal float.
hipError_t launch_forward_bf16_exact(const FwdParams& p, hipStream_t stream);
hipError_t launch_chain(const ChainParams& p, bool bf16, hipStream_t stream);
hipError_t launch_gradient(const GradParams& p, hipStream_t stream);
hipError_t launch_noise(const void* seeds, bool seeds_i32, int64_t pop, int64_t n, int64_t offset,
                        uint32_t* r_out, float* n_out, hipStream_t stream);
// Floats of workspace the reduce metric uses for (pop, n); 0 = none needed.
int64_t reduce_metric_workspace_floats(int64_t pop, int64_t n);
// workspace: reduce_metric_workspace_floats(pop, n) floats (null when that
// is 0).
hipError_t launch_reduce_metric(const float* center, const void* seeds, bool seeds_i32, int64_t pop,
                                int64_t n, float sigma, int64_t offset, float* out, float* workspace,
                                hipStream_t stream);

// Floats in each GPU's allocation-free reduce-metric scratch array: more than
// the most any (pop, n) needs (pop * segments < 1536, see metric_segments).
constexpr int64_t kMetricScratchFloats = 2048;
// Device address of the current GPU's scratch array (looked up once per device).
hipError_t metric_scratch_address(float** ptr);

// Largest grid.x the launchers use (they loop inside the kernel beyond it).
constexpr int64_t kMaxGridX = 0x7FFFFFFF;

// Large-batch bf16 forward through materialized perturbed weights (vn_gemm.hip).
constexpr int64_t kMaterializeMinBatch = 2048;          // rows per individual from which it is used
constexpr int64_t kMaterializeBytes = int64_t{1} << 28; // workspace budget: individuals per group
constexpr int64_t kMatmulGrid = 256;                    // persistent workgroups (one per CU)
struct MatParams {
  const __bf16* x;
  int64_t x_pop_stride;
  const __bf16* wp;       // perturbed weights of the group, (group, out, in)
  int64_t wp_stride;      // out * in
  const float* bias;      // may be null
  const void* seeds;
  bool seeds_i32;
  float sigma;
  int64_t offset;
  bool relu;
  float* y;
  int64_t i0;             // first individual of the group
  int64_t total_tiles;    // group size * tiles_m * tiles_n
  int64_t m, n, k;        // batch, out, in
  int32_t tiles_m, tiles_n;
};
// Shapes the materialized path takes: batch >= kMaterializeMinBatch,
// 256 <= out < 2^26, in a multiple of 64 in [128, 2^22), and fewer than 2^31
// tiles per individual.
bool materialized_forward_applies(int64_t batch, int64_t in, int64_t out);
// Individuals per group and the workspace bytes the path needs.
int64_t materialized_group(int64_t pop, int64_t batch, int64_t in, int64_t out);
int64_t materialized_workspace_bytes(int64_t pop, int64_t batch, int64_t in, int64_t out);
// x, w 16-byte aligned, x_pop_stride a multiple of 8, workspace 16-byte
// aligned with materialized_workspace_bytes.
hipError_t launch_forward_bf16_materialized(const FwdParams& p, void* workspace, hipStream_t stream);

}  // namespace vn
