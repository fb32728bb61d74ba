// Device-side noise generator shared by every kernel of the library.
//
// Follows the EvoX API page "evox.triton_kernels.kernels.virtual_noise":
// section "RNG: fast centered-uniform approximation" (noise = u - 0.5 with u
// uniform in [0,1) from the low 32 bits of a splitmix64 hash), API entry
// _splitmix64_step (two xor-shift / multiply-by-GAMMA rounds and a final
// xor-shift, all mod 2^64) and section "Noise indexing scheme".
//
// Fixed readings (the page leaves them open):
//   state    z0 = seed + (idx + 1) * GAMMA mod 2^64   (idx-th output of the
//            splitmix64 sequence seeded with `seed`; consecutive indices step
//            the state by +GAMMA, which the kernels exploit)
//   mapping  N = (r >> 8) * 2^-24 - 0.5, exact in fp32 and strictly < 0.5
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vn {

// API data entry _SPLITMIX64_GAMMA = 11400714819323198485.
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

// (idx + 1) * GAMMA for a compile-time step count.
__host__ __device__ constexpr uint64_t gamma_times(uint64_t t) { return t * kGamma; }

// 64-bit state -> low 32 bits of the finalizer output.
__device__ __forceinline__ uint32_t mix_lo32(uint64_t z) {
  z = (z ^ (z >> 30)) * kGamma;
  z = (z ^ (z >> 27)) * kGamma;
  return static_cast<uint32_t>(z ^ (z >> 31));
}

// Initial state of element `idx` (absolute flat index) for seed `s`.
__device__ __forceinline__ uint64_t state_of(uint64_t s, uint64_t idx) {
  return s + (idx + 1ull) * kGamma;
}

// r -> centered uniform noise in [-0.5, 0.5); every step is exact in fp32.
__device__ __forceinline__ float noise_of_bits(uint32_t r) {
  return __builtin_fmaf(static_cast<float>(r >> 8), 0x1p-24f, -0.5f);
}

__device__ __forceinline__ float noise_of_state(uint64_t z) { return noise_of_bits(mix_lo32(z)); }

// Seed i as a 64-bit two's-complement pattern (int32 seeds sign-extended).
__device__ __forceinline__ uint64_t load_seed(const void* seeds, bool seeds_i32, int64_t i) {
  return seeds_i32 ? static_cast<uint64_t>(static_cast<int64_t>(static_cast<const int32_t*>(seeds)[i]))
                   : static_cast<uint64_t>(static_cast<const int64_t*>(seeds)[i]);
}

}  // namespace vn
