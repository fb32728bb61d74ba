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
constexpr uint32_t kGammaLo = static_cast<uint32_t>(kGamma);
constexpr uint32_t kGammaHi = static_cast<uint32_t>(kGamma >> 32);

// (idx + 1) * GAMMA for a compile-time step count.
__host__ __device__ constexpr uint64_t gamma_times(uint64_t t) { return t * kGamma; }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// t * GAMMA mod 2^64 on 32-bit words.  The two cross products only matter
// mod 2^32, so the second one takes the first as the addend of a 32x32->64
// multiply-add (whose high word is left arbitrary), and their sum enters the
// low product as the high word of its addend: three multiplies and a move,
// where the plain 64-bit product costs two multiply-lows, a multiply-add and
// a three-way add.
__device__ __forceinline__ uint64_t mul_gamma(uint64_t t) {
  const uint32_t lo = static_cast<uint32_t>(t), hi = static_cast<uint32_t>(t >> 32);
  u32x2 c;
  c.x = lo * kGammaHi;
  c.y = __builtin_nondeterministic_value(c.x);
  const uint32_t cross = static_cast<uint32_t>(static_cast<uint64_t>(hi) * kGammaLo + __builtin_bit_cast(uint64_t, c));
  return static_cast<uint64_t>(lo) * kGammaLo + (static_cast<uint64_t>(cross) << 32);
}

// The finalizer in its steps, so that a kernel can run the steps of several
// elements in lockstep and place other work between them:
//   round 1 = mul_gamma(xorshift(z, 30)), round 2 = mul_gamma(xorshift(z, 27)),
//   then keep_words() and, on the 64-bit result, final_centered().
__device__ __forceinline__ uint64_t xorshift(uint64_t z, int s) { return z ^ (z >> s); }

// Use the product's words as computed: without this the compiler recomputes
// the low word of the last product with a separate multiply.
__device__ __forceinline__ uint64_t keep_words(uint64_t z) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm("" : "+v"(z));
#endif
  return z;
}

// Finalizer rounds on the state, up to the last product (still 64-bit).
__device__ __forceinline__ uint64_t mix_rounds(uint64_t z) {
  z = mul_gamma(xorshift(z, 30));
  z = mul_gamma(xorshift(z, 27));
  return keep_words(z);
}

// 64-bit state -> low 32 bits of the finalizer output.
__device__ __forceinline__ uint32_t mix_lo32(uint64_t z) {
  z = mix_rounds(z);
  return static_cast<uint32_t>(z ^ (z >> 31));
}

// Last step on the output z of mix_rounds: (r >> 8) - 2^23 as a signed
// integer, r = low word of z ^ (z >> 31): the noise times 2^24, exact in fp32.
// Flipping bit 31 of r turns the unsigned shift into an arithmetic one on the
// centred value; the flip rides on the final xor as a three-way xor (one
// bitop3, at the xor's rate).
__device__ __forceinline__ int32_t final_centered(uint64_t z) {
  const uint32_t lo = static_cast<uint32_t>(z), hi = static_cast<uint32_t>(z >> 32);
  const uint32_t sh = __builtin_amdgcn_alignbit(hi, lo, 31);   // low word of z >> 31
  uint32_t r;
#if defined(__HIP_DEVICE_COMPILE__)
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(lo), "v"(sh), "s"(0x80000000u));
#else
  r = lo ^ sh ^ 0x80000000u;
#endif
  return static_cast<int32_t>(r) >> 8;
}

// 64-bit state -> the noise times 2^24 as a signed integer (see final_centered).
__device__ __forceinline__ int32_t centered_q(uint64_t z) { return final_centered(mix_rounds(z)); }

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
