// Calibration probe for the ALU roofline of the noise hash on gfx950.
//
// Measures (1) the issue rate of every vector instruction the hash sequence
// uses, as lane-operations per second and as a fraction of the full 32-bit
// rate (64 lane-ops per CU per clock), (2) the throughput of the hash
// sequence of vn_device.hpp itself, in hashes per second, and (3) that of
// whole noise elements as the kernels consume them (state step, hash, N * 2^24
// as fp32, one fma into an accumulator).
//
// Each probe kernel runs 16 independent dependency chains per lane (so
// latency never limits issue) at 8 waves per SIMD; the only memory accesses
// are one store per thread of a checksum, into a buffer sized to the grid,
// and two clock readings by thread 0 of block 0.  Those readings (the shader
// clock counter against the constant 100 MHz reference counter, over block
// 0's lifetime) give the shader clock the probe ran at, so every rate is also
// reported per clock cycle.  Prints one JSON object per line.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "vn_device.hpp"

#define CHECK(x)                                                                       \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(1);                                                                    \
    }                                                                                  \
  } while (0)

constexpr int kThreads = 256;
constexpr int kChains = 16;

// Shader-clock and reference-clock counters at the start and end of block 0.
#define CLOCK_BEGIN                                                                     \
  uint64_t clk_t0 = 0, clk_r0 = 0;                                                      \
  if (blockIdx.x == 0 && threadIdx.x == 0) {                                            \
    clk_t0 = __builtin_amdgcn_s_memtime();                                              \
    clk_r0 = __builtin_amdgcn_s_memrealtime();                                          \
  }
#define CLOCK_END                                                                       \
  if (blockIdx.x == 0 && threadIdx.x == 0) {                                            \
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime(); \
    clk[0] = t1 - clk_t0;                                                               \
    clk[1] = r1 - clk_r0;                                                               \
  }

// 32-bit ops: a = op(a, b[, b2]) on 16 chains.
#define PROBE32(NAME, ASM)                                                              \
  __global__ __launch_bounds__(kThreads) void NAME(uint32_t* out, uint64_t* clk, int iters, uint32_t seed) { \
    CLOCK_BEGIN                                                                         \
    uint32_t a[kChains];                                                                \
    const uint32_t b = seed * 2654435761u + threadIdx.x;                                \
    const uint32_t b2 = seed ^ (threadIdx.x * 40503u);                                  \
    _Pragma("unroll") for (int c = 0; c < kChains; ++c) a[c] = threadIdx.x + c * 977u + seed; \
    for (int it = 0; it < iters; ++it) {                                                \
      _Pragma("unroll") for (int c = 0; c < kChains; ++c) asm volatile(ASM : "+v"(a[c]) : "v"(b), "v"(b2)); \
    }                                                                                   \
    uint32_t r = 0;                                                                     \
    _Pragma("unroll") for (int c = 0; c < kChains; ++c) r ^= a[c];                      \
    CLOCK_END                                                                           \
    out[blockIdx.x * kThreads + threadIdx.x] = r;                                       \
  }

// 64-bit ops on 16 chains of register pairs (%1: 64-bit operand, %2, %3: 32-bit operands).
#define PROBE64(NAME, ASM)                                                              \
  __global__ __launch_bounds__(kThreads) void NAME(uint32_t* out, uint64_t* clk, int iters, uint32_t seed) { \
    CLOCK_BEGIN                                                                         \
    uint64_t a[kChains];                                                                \
    const uint64_t b = (static_cast<uint64_t>(seed) << 32) | threadIdx.x;               \
    const uint32_t b1 = seed * 2654435761u + threadIdx.x, b2 = seed ^ 0x9E3779B9u;      \
    _Pragma("unroll") for (int c = 0; c < kChains; ++c) a[c] = threadIdx.x + c * 977ull + seed; \
    for (int it = 0; it < iters; ++it) {                                                \
      _Pragma("unroll") for (int c = 0; c < kChains; ++c)                               \
        asm volatile(ASM : "+v"(a[c]) : "v"(b), "v"(b1), "v"(b2) : "vcc");             \
    }                                                                                   \
    uint64_t r = 0;                                                                     \
    _Pragma("unroll") for (int c = 0; c < kChains; ++c) r ^= a[c];                      \
    CLOCK_END                                                                           \
    out[blockIdx.x * kThreads + threadIdx.x] = static_cast<uint32_t>(r ^ (r >> 32));    \
  }

PROBE32(p_xor, "v_xor_b32 %0, %0, %1")
PROBE32(p_add_u32, "v_add_u32 %0, %0, %1")
PROBE32(p_mul_lo, "v_mul_lo_u32 %0, %0, %1")
PROBE32(p_mul_hi, "v_mul_hi_u32 %0, %0, %1")
PROBE32(p_mul_u24, "v_mul_u32_u24 %0, %0, %1")
PROBE32(p_alignbit, "v_alignbit_b32 %0, %0, %1, 30")
PROBE32(p_add3, "v_add3_u32 %0, %0, %1, %0")
PROBE32(p_lshr, "v_lshrrev_b32 %0, 8, %0")
PROBE32(p_cvt, "v_cvt_f32_u32 %0, %0")
PROBE32(p_fma, "v_fma_f32 %0, %0, %1, %0")
PROBE32(p_fmac, "v_fmac_f32 %0, %1, %2")
PROBE32(p_mov, "v_mov_b32 %0, %1")
PROBE32(p_xad, "v_xad_u32 %0, %0, %1, %0")
PROBE32(p_bitop3, "v_bitop3_b32 %0, %0, %1, %0 bitop3:0x96")
PROBE32(p_ashr, "v_ashrrev_i32 %0, 8, %0")
PROBE32(p_cvt_i32, "v_cvt_f32_i32 %0, %0")
PROBE32(p_cvt_ubyte, "v_cvt_f32_ubyte2 %0, %0")
PROBE32(p_perm, "v_perm_b32 %0, %0, %1, %1")
PROBE32(p_cvt_pk_bf16, "v_cvt_pk_bf16_f32 %0, %0, %1")
PROBE32(p_sub_f32, "v_sub_f32 %0, %0, %1")
PROBE32(p_and, "v_and_b32 %0, %0, %1")
PROBE64(p_mad64, "v_mad_u64_u32 %0, vcc, %2, %3, %0")
PROBE64(p_shr64, "v_lshrrev_b64 %0, 30, %0")
PROBE64(p_add64, "v_lshl_add_u64 %0, %0, 0, %1")

// The shipped hash: Weyl-stepped states, low 32 bits of the finalizer.
__global__ __launch_bounds__(kThreads) void p_hash(uint32_t* out, uint64_t* clk, int iters, uint32_t seed) {
  CLOCK_BEGIN
  constexpr int S = 8;
  uint64_t z[S];
  const uint64_t g = blockIdx.x * kThreads + threadIdx.x;
#pragma unroll
  for (int c = 0; c < S; ++c) z[c] = vn::state_of(seed, g * 64 + c);
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < S; ++c) {
      acc ^= vn::mix_lo32(z[c]);
      z[c] += vn::gamma_times(S);
    }
  }
  CLOCK_END
  out[g] = acc;
}

// The same hash written as plain 64-bit C (z * GAMMA), for comparison with
// the library's word-level form.
__global__ __launch_bounds__(kThreads) void p_hash_plain(uint32_t* out, uint64_t* clk, int iters, uint32_t seed) {
  CLOCK_BEGIN
  constexpr int S = 8;
  uint64_t z[S];
  const uint64_t g = blockIdx.x * kThreads + threadIdx.x;
#pragma unroll
  for (int c = 0; c < S; ++c) z[c] = vn::state_of(seed, g * 64 + c);
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < S; ++c) {
      uint64_t t = z[c];
      t = (t ^ (t >> 30)) * vn::kGamma;
      t = (t ^ (t >> 27)) * vn::kGamma;
      acc ^= static_cast<uint32_t>(t ^ (t >> 31));
      z[c] += vn::gamma_times(S);
    }
  }
  CLOCK_END
  out[g] = acc;
}

// Noise elements as every kernel consumes them: Weyl-stepped states, N * 2^24
// as fp32 (centered_q and the conversion), each folded into an fp32
// accumulator by one fma (eight independent accumulators per lane).
template <int S>
__global__ __launch_bounds__(kThreads) void p_noise(uint32_t* out, uint64_t* clk, int iters, uint32_t seed) {
  CLOCK_BEGIN
  uint64_t z[S];
  float acc[S];
  const uint64_t g = blockIdx.x * kThreads + threadIdx.x;
  const float f = 1.0f + static_cast<float>(seed) * 1e-3f;
#pragma unroll
  for (int c = 0; c < S; ++c) {
    z[c] = vn::state_of(seed, g * 64 + c);
    acc[c] = 0.0f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < S; ++c) {
      acc[c] = __builtin_fmaf(f, static_cast<float>(vn::centered_q(z[c])), acc[c]);
      z[c] += vn::gamma_times(S);
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int c = 0; c < S; ++c) t += acc[c];
  CLOCK_END
  out[g] = __builtin_bit_cast(uint32_t, t);
}

// MFMA / VALU co-execution: per loop slot, one MFMA (or none) and NV integer
// multiplies on 8 independent chains; 2 waves per SIMD.  If a shape's MFMAs
// run beside the VALU, slot cycles (launch time at the measured shader clock)
// stay near the VALU-only figure.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int SHAPE, int NV>
__global__ __launch_bounds__(kThreads) void p_coexec(uint32_t* out, uint64_t* clk, int iters, uint32_t seed) {
  CLOCK_BEGIN
  f32x16 A0 = {}, A1 = {};
  f32x4 B0 = {}, B1 = {};
  const float a = threadIdx.x * 1e-3f, b = 1.0001f;
  bf16x8 ab, bb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ab[e] = static_cast<__bf16>(threadIdx.x * 1e-3f + e);
    bb[e] = static_cast<__bf16>(1.0f + e * 1e-2f);
  }
  uint32_t v[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) v[c] = threadIdx.x + c + seed;
  const uint32_t m = 0x9E3779B9u;
  for (int it = 0; it < iters; ++it) {
#define VN_PROBE_MFMA(ACC32, ACC16)                                                                              \
    if (SHAPE == 1) asm volatile("v_mfma_f32_32x32x2_f32 %0, %1, %2, %0" : "+v"(ACC32) : "v"(a), "v"(b));       \
    if (SHAPE == 2) asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+v"(ACC16) : "v"(a), "v"(b));       \
    if (SHAPE == 3) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(ACC32) : "v"(ab), "v"(bb));   \
    if (SHAPE == 4) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(ACC16) : "v"(ab), "v"(bb));
    VN_PROBE_MFMA(A0, B0)
#pragma unroll
    for (int r = 0; r < NV / 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) asm volatile("v_mul_lo_u32 %0, %0, %1" : "+v"(v[c]) : "v"(m));
    VN_PROBE_MFMA(A1, B1)
#pragma unroll
    for (int r = 0; r < NV / 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) asm volatile("v_mul_lo_u32 %0, %0, %1" : "+v"(v[c]) : "v"(m));
#undef VN_PROBE_MFMA
  }
  float sacc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc += A0[i] + A1[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) sacc += B0[i] + B1[i];
  uint32_t x = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) x ^= v[c];
  CLOCK_END
  out[blockIdx.x * kThreads + threadIdx.x] = x ^ __builtin_bit_cast(uint32_t, sacc);
}

struct CoProbe {
  const char* name;
  void (*fn)(uint32_t*, uint64_t*, int, uint32_t);
  int nv;
};

struct Probe {
  const char* name;
  void (*fn)(uint32_t*, uint64_t*, int, uint32_t);
  int per_iter;   // instructions (or hashes) per lane per iteration
  const char* what;
};

int main(int argc, char** argv) {
  int dev = 0;
  CHECK(hipSetDevice(dev));
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, dev));
  int clock_khz = 0;
  CHECK(hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeClockRate, dev));
  const int cus = prop.multiProcessorCount;
  const int blocks = cus * 8;  // 8 blocks of 4 waves per CU = 8 waves per SIMD
  const int iters = argc > 1 ? std::atoi(argv[1]) : 2048;
  std::printf("{\"device\": \"%s\", \"gcn_arch\": \"%s\", \"cus\": %d, \"clock_mhz\": %.0f, \"blocks\": %d, "
              "\"threads\": %d, \"iters\": %d}\n",
              prop.name, prop.gcnArchName, cus, clock_khz / 1e3, blocks, kThreads, iters);
  uint32_t* out = nullptr;
  CHECK(hipMalloc(&out, sizeof(uint32_t) * blocks * kThreads));
  uint64_t* clk = nullptr;
  CHECK(hipMalloc(&clk, sizeof(uint64_t) * 2));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const Probe probes[] = {
      {"v_xor_b32", p_xor, kChains, "32-bit"},
      {"v_add_u32", p_add_u32, kChains, "32-bit"},
      {"v_mul_lo_u32", p_mul_lo, kChains, "32-bit"},
      {"v_mul_hi_u32", p_mul_hi, kChains, "32-bit"},
      {"v_mul_u32_u24", p_mul_u24, kChains, "32-bit"},
      {"v_alignbit_b32", p_alignbit, kChains, "32-bit"},
      {"v_add3_u32", p_add3, kChains, "32-bit"},
      {"v_lshrrev_b32", p_lshr, kChains, "32-bit"},
      {"v_cvt_f32_u32", p_cvt, kChains, "32-bit"},
      {"v_fma_f32", p_fma, kChains, "32-bit"},
      {"v_fmac_f32", p_fmac, kChains, "32-bit"},
      {"v_mov_b32", p_mov, kChains, "32-bit"},
      {"v_xad_u32", p_xad, kChains, "32-bit"},
      {"v_bitop3_b32", p_bitop3, kChains, "32-bit"},
      {"v_ashrrev_i32", p_ashr, kChains, "32-bit"},
      {"v_cvt_f32_i32", p_cvt_i32, kChains, "32-bit"},
      {"v_cvt_f32_ubyte2", p_cvt_ubyte, kChains, "32-bit"},
      {"v_perm_b32", p_perm, kChains, "32-bit"},
      {"v_cvt_pk_bf16_f32", p_cvt_pk_bf16, kChains, "32-bit"},
      {"v_sub_f32", p_sub_f32, kChains, "32-bit"},
      {"v_and_b32", p_and, kChains, "32-bit"},
      {"v_mad_u64_u32", p_mad64, kChains, "64-bit"},
      {"v_lshrrev_b64", p_shr64, kChains, "64-bit"},
      {"v_lshl_add_u64", p_add64, kChains, "64-bit"},
      {"hash", p_hash, 8, "hash"},
      {"hash_plain", p_hash_plain, 8, "hash"},
      {"noise_fma", p_noise<8>, 8, "hash"},
  };
  const double peak_lane_ops = static_cast<double>(cus) * 64.0 * clock_khz * 1e3;
  for (const Probe& pr : probes) {
    // warm-up, then the best of 3 timed launches
    pr.fn<<<blocks, kThreads>>>(out, clk, iters / 8, 1u);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    float best = 1e30f;
    double ghz = 0.0;   // shader clock of the best launch
    for (int rep = 0; rep < 3; ++rep) {
      CHECK(hipEventRecord(e0));
      pr.fn<<<blocks, kThreads>>>(out, clk, iters, 2u + rep);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      uint64_t c[2];
      CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
      if (ms < best) {
        best = ms;
        ghz = c[1] > 0 ? static_cast<double>(c[0]) / (static_cast<double>(c[1]) / 100e6) / 1e9 : 0.0;
      }
    }
    const double ops = static_cast<double>(blocks) * kThreads * iters * pr.per_iter;
    const double rate = ops / (best * 1e-3);
    const double per_clk = static_cast<double>(cus) * 64.0 * ghz * 1e9;   // full-rate lane-ops at that clock
    if (std::strcmp(pr.what, "hash") == 0) {
      std::printf("{\"probe\": \"%s\", \"ms\": %.4f, \"hashes_per_s\": %.4e, \"lane_cycles_per_hash\": %.2f, "
                  "\"shader_ghz\": %.3f, \"lane_cycles_per_hash_at_that_clock\": %.2f}\n",
                  pr.name, best, rate, peak_lane_ops / rate, ghz, per_clk / rate);
    } else {
      std::printf("{\"probe\": \"%s\", \"ms\": %.4f, \"lane_ops_per_s\": %.4e, \"rate_vs_full\": %.3f, "
                  "\"shader_ghz\": %.3f, \"rate_per_clock\": %.3f}\n",
                  pr.name, best, rate, rate / peak_lane_ops, ghz, rate / per_clk);
    }
    std::fflush(stdout);
  }
  // co-execution: 2 waves per SIMD, cycles per slot = SIMD cycles / (slots per wave * waves per SIMD)
  // The noise sequence at lower occupancy (waves per SIMD) and fewer
  // independent chains per lane, as the kernels run it: the per-element cost
  // in lane-cycles at the launch's clock.
  {
    struct NoiseCfg {
      int chains, waves;
      void (*fn)(uint32_t*, uint64_t*, int, uint32_t);
    };
    const NoiseCfg nc[] = {{1, 2, p_noise<1>}, {4, 2, p_noise<4>}, {1, 4, p_noise<1>}, {4, 4, p_noise<4>},
                           {1, 8, p_noise<1>}, {4, 8, p_noise<4>}};
    for (const NoiseCfg& c : nc) {
      const int nb = cus * c.waves;               // blocks of 4 waves: c.waves waves per SIMD
      const int it = iters * 64 / (c.chains * c.waves);   // the same work per SIMD in every configuration
      c.fn<<<nb, kThreads>>>(out, clk, it / 8, 1u);
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
      CHECK(hipEventRecord(e0));
      c.fn<<<nb, kThreads>>>(out, clk, it, 2u);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      uint64_t cc[2];
      CHECK(hipMemcpy(cc, clk, sizeof(cc), hipMemcpyDeviceToHost));
      const double ghz = cc[1] > 0 ? static_cast<double>(cc[0]) / (static_cast<double>(cc[1]) / 100e6) / 1e9 : 0.0;
      const double elems = static_cast<double>(nb) * kThreads * it * c.chains;
      const double rate = elems / (ms * 1e-3);
      std::printf("{\"noise_fma_occupancy\": {\"chains\": %d, \"waves_per_simd\": %d}, \"ms\": %.4f, "
                  "\"shader_ghz\": %.3f, \"lane_cycles_per_elem_at_that_clock\": %.2f}\n",
                  c.chains, c.waves, ms, ghz, static_cast<double>(cus) * 64.0 * ghz * 1e9 / rate);
      std::fflush(stdout);
    }
  }
  const CoProbe co[] = {
      {"none", p_coexec<0, 16>, 16},           {"v_mfma_f32_32x32x2_f32", p_coexec<1, 0>, 0},
      {"v_mfma_f32_32x32x2_f32", p_coexec<1, 16>, 16}, {"v_mfma_f32_16x16x4_f32", p_coexec<2, 0>, 0},
      {"v_mfma_f32_16x16x4_f32", p_coexec<2, 16>, 16}, {"v_mfma_f32_32x32x16_bf16", p_coexec<3, 0>, 0},
      {"v_mfma_f32_32x32x16_bf16", p_coexec<3, 16>, 16}, {"v_mfma_f32_16x16x32_bf16", p_coexec<4, 0>, 0},
      {"v_mfma_f32_16x16x32_bf16", p_coexec<4, 16>, 16},
  };
  const int co_blocks = cus * 2;   // 2 blocks of 4 waves per CU = 2 waves per SIMD
  const int co_iters = 10000;
  for (const CoProbe& pr : co) {
    pr.fn<<<co_blocks, kThreads>>>(out, clk, co_iters / 8, 1u);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    float best = 1e30f;
    double ghz = 0.0;   // shader clock of the best launch
    for (int rep = 0; rep < 3; ++rep) {
      CHECK(hipEventRecord(e0));
      pr.fn<<<co_blocks, kThreads>>>(out, clk, co_iters, 2u + rep);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      uint64_t c[2];
      CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
      if (ms < best) {
        best = ms;
        ghz = c[1] > 0 ? static_cast<double>(c[0]) / (static_cast<double>(c[1]) / 100e6) / 1e9 : 0.0;
      }
    }
    // launch time at the measured clock, over the slots one SIMD issues
    const double simd_cycles = best * 1e-3 * ghz * 1e9;
    const double slots_per_simd = 2.0 * co_iters * 2.0;  // 2 slots per iteration, 2 waves per SIMD
    std::printf("{\"coexec\": \"%s\", \"v_mul_lo_u32_per_slot\": %d, \"ms\": %.4f, \"shader_ghz\": %.3f, "
                "\"simd_cycles_per_slot\": %.2f}\n",
                pr.name, pr.nv, best, ghz, simd_cycles / slots_per_simd);
    std::fflush(stdout);
  }
  CHECK(hipFree(clk));
  CHECK(hipFree(out));
  return 0;
}
