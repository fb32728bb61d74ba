// Forward for large batches with bf16 operands (gfx950), in two steps per
// group of individuals:
//   1. perturb_kernel forms the perturbed weights bf16(W + sigma N_i) of the
//      group once, in a caller workspace (one fp32 fma per element, nearest-even
//      to bf16: the rounding every bf16 forward kernel of the library applies);
//   2. matmul_kernel, a persistent MFMA kernel, multiplies every individual's
//      X rows by them: Y[i] = X[i] Wp_i^T + (b + sigma nb_i).
// Method: EvoX API page "evox.triton_kernels.kernels.virtual_noise", module
// introduction (model equation) and API entry virtual_perturbed_linear; the
// noise is the generator of vn_device.hpp.
//
// Why two steps: the fused large-batch kernel generates each noise element
// once per 512 rows, so the hash (about 20 vector instructions per element)
// still costs more than the matrix cores' share.  Formed once per individual,
// the perturbed weights cost a fixed 2 bytes per element of workspace traffic
// each way, and for thousands of rows per individual the product is bound by
// the matrix cores.  Every output accumulates the same MFMA sequence as in the
// fused kernels (v_mfma_f32_32x32x16_bf16, ascending k in steps of 16, one
// fp32 accumulator), so the two paths give the same bits.
//
// matmul_kernel: one workgroup of 4 waves per CU walks 256 x 256 output tiles
// t = blockIdx.x, + gridDim.x, ...; each wave owns a 128 x 128 quarter (16
// accumulator blocks of 32 x 32, all 256 accumulator registers).  k advances in
// stages of 64 through two LDS slots (A: 256 rows x 64 k of X, B: 256 rows x
// 64 k of Wp, 64 KB per slot), filled by direct global->LDS loads issued two
// stages ahead; the last two stages of a tile load the first two of the next
// tile, so consecutive tiles overlap.  A stage's 64 loads per workgroup are
// spread one per two MFMAs over two k-steps (the X half in the k-step that
// frees the slot, the Wp half in the next), and the MFMA fragments of the
// next k-step are read one per MFMA, so that neither the address unit's queue
// nor the LDS sees a burst.  The loads are issued through inline asm and every
// wait on them is explicit (vmcnt before the barrier that publishes a stage);
// the compiler neither tracks nor waits on them.  A ragged last row or column
// tile is moved back to end at the last row or column (batch and out are at
// least 256 here), so every load reads 256 valid rows and the per-lane load
// offsets are the same for every tile; the outputs that the previous tile
// owns are recomputed and not stored.
#include <stdint.h>

#include <utility>

#include "vn_device.hpp"
#include "vn_launch.hpp"

namespace vn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ float lo_bf16(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// dst[il][e] = bf16(fma(sigma_q, q_i(offset + e), w[e])) for e < n, n % 8 == 0,
// individual i = i0 + blockIdx.y; q_i is the noise times 2^24 (an integer),
// sigma_q = sigma * 2^-24.  Runs of 8 consecutive elements per thread.
__global__ __launch_bounds__(256) void perturb_kernel(const __bf16* __restrict__ w, const void* seeds, bool seeds_i32,
                                                      int64_t i0, int64_t n, int64_t offset, float sigma_q,
                                                      __bf16* __restrict__ dst) {
  const int64_t il = blockIdx.y;
  const uint64_t s = load_seed(seeds, seeds_i32, i0 + il);
  __bf16* __restrict__ d = dst + il * n;
  const int64_t runs = n / 8;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; r < runs;
       r += static_cast<int64_t>(gridDim.x) * 256) {
    const uint4 wv = *reinterpret_cast<const uint4*>(w + r * 8);
    uint32_t wr[4], o[4];
    __builtin_memcpy(wr, &wv, 16);
    const uint64_t z = state_of(s, static_cast<uint64_t>(offset + r * 8));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = __builtin_fmaf(sigma_q, static_cast<float>(centered_q(z + gamma_times(2 * e))), lo_bf16(wr[e]));
      const float b =
          __builtin_fmaf(sigma_q, static_cast<float>(centered_q(z + gamma_times(2 * e + 1))), hi_bf16(wr[e]));
      o[e] = pack2_bf16(a, b);
    }
    uint4 ov;
    __builtin_memcpy(&ov, o, 16);
    *reinterpret_cast<uint4*>(d + r * 8) = ov;
  }
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int UNITS = BM * 8;   // 16-byte units per operand per stage (256 rows x 64 k bf16)

// LDS layout of a stage: unit (16 B) of (row r, k-segment s of 8) is
// r*8 + (s ^ swz(r)); the swizzle keeps the MFMA fragment reads (32 rows at
// one segment) free of bank conflicts for 8 or 16 lanes per LDS cycle.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 16 bytes at sbase + voff (a wave-uniform 64-bit base, a 32-bit per-lane
// offset) -> LDS byte address base + IMM + 16 * lane (base wave-uniform).
// M0 takes the LDS address; one wait state separates its write from the load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int IMM>
__device__ __forceinline__ void lds_load16(uint32_t voff, const void* sbase, uint32_t base) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(base), "n"(IMM)
               : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// An accumulator value out of its AGPR, at this point of the program.
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One tile's operand sources.  The tile owns output rows [m0, m0 + 256) and
// columns [n0, n0 + 256) (cut at batch and out); it computes rows from me and
// columns from ne, which differ from m0 and n0 only for a ragged last tile.
struct Tile {
  const char* a;   // X rows of the tile (byte address of row me, k 0)
  const char* b;   // Wp rows of the tile (row ne)
  int64_t i, m0, n0, me, ne;
};

__global__ __launch_bounds__(256, 1) void matmul_kernel(MatParams g) {
  __shared__ uint4 smem[4 * UNITS];   // slot 0: A, B; slot 1: A, B
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::: "a0");   // accumulators in AGPRs
#endif
  const int64_t K = g.k;
  const int64_t nk = K / BK;
  const uint32_t K2 = static_cast<uint32_t>(K * 2);
  const uint32_t tiles_m = g.tiles_m, tiles_n = g.tiles_n, per_ind = tiles_m * tiles_n;

  // Tile t: individual t / per_ind.  Within an individual, tiles whose index
  // is congruent mod 8 run on one XCD (the grid is a multiple of 8); each XCD
  // takes a contiguous range of the tile order below, which walks groups of 4
  // row tiles column by column, so an XCD's tiles share X and Wp rows in L2.
  auto setup = [&](uint32_t t, Tile& r) {
    const uint32_t il = __builtin_amdgcn_readfirstlane(t / per_ind);
    const uint32_t rest = t - il * per_ind;
    const uint32_t q = (per_ind % 8 == 0) ? (rest % 8) * (per_ind / 8) + rest / 8 : rest;
    const uint32_t first = q / (4 * tiles_n) * 4;
    const uint32_t gsz = (tiles_m - first) < 4 ? (tiles_m - first) : 4;
    const uint32_t r2 = q - first * tiles_n;
    r.i = g.i0 + il;
    r.m0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(first + r2 % gsz)) * BM;
    r.n0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(r2 / gsz)) * BN;
    r.me = r.m0 + BM <= g.m ? r.m0 : g.m - BM;
    r.ne = r.n0 + BN <= g.n ? r.n0 : g.n - BN;
    r.a = reinterpret_cast<const char*>(g.x + r.i * g.x_pop_stride + r.me * K);
    r.b = reinterpret_cast<const char*>(g.wp + il * g.wp_stride + r.ne * K);
  };

  // Load u of a stage (u < 8: A, else B) fills unit (u % 8) * 256 + tid of its
  // operand: row (u % 8) * 32 + tid / 8, k-segment (tid % 8) ^ swz(row), at a
  // per-lane offset voff[u % 8] from the operand's row 0 at the stage's k.
  const int lrow = tid >> 3;
  const uint32_t lseg16 = static_cast<uint32_t>(((tid & 7) ^ swz(lrow)) * 16);
  const uint32_t wave_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem)) + wave * 64 * 16;
  uint32_t voff[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) voff[u] = static_cast<uint32_t>(lrow + 32 * u) * K2 + lseg16;
  auto load_u = [&](const char* abase, const char* bbase, int slot, int64_t k0, auto uc) {
    constexpr int u = decltype(uc)::value;
    const uint32_t kb = static_cast<uint32_t>(k0 * 2);
    const uint32_t sa = __builtin_amdgcn_readfirstlane(wave_lds + slot * (2 * UNITS * 16));
    if constexpr (u < 8)
      lds_load16<u * 256 * 16>(voff[u], abase + kb, sa);
    else
      lds_load16<UNITS * 16 + (u - 8) * 256 * 16>(voff[u - 8], bbase + kb, sa);
  };
  auto load_stage = [&](const Tile& r, int slot, int64_t k0) {
    static_for<16>([&](auto uc) { load_u(r.a, r.b, slot, k0, uc); });
  };

  // MFMA fragments: lane l reads row (or column) l % 32 of a 32-block at
  // k-segment 2t + l / 32 of k-step t.
  const int l32 = lane & 31, lh = lane >> 5;
  const int swl = swz(l32);
  const int arow_u = (wm * 128 + l32) * 8;
  const int bcol_u = UNITS + (wn * 128 + l32) * 8;
  bf16x8 fa[2][4], fb[2][4];
  auto read_one = [&](int slot, int t, int buf, int q) {
    const int seg = (2 * t + lh) ^ swl;
    if (q < 4)
      fa[buf][q] = __builtin_bit_cast(bf16x8, smem[slot * 2 * UNITS + arow_u + seg + q * 256]);
    else
      fb[buf][q - 4] = __builtin_bit_cast(bf16x8, smem[slot * 2 * UNITS + bcol_u + seg + (q - 4) * 256]);
  };
  f32x16 acc[4][4];
  auto mfma1 = [&](int m, int buf) {
    const int a = m >> 2, b = m & 3;
    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][a], fb[buf][b], acc[a][b], 0, 0, 0);
  };

  const uint32_t total = g.total_tiles;
  Tile cur, nxt;
  setup(blockIdx.x, cur);
  uint32_t tnext = blockIdx.x + gridDim.x;
  bool has_next = tnext < total;
  if (has_next) setup(tnext, nxt);
  else nxt = cur;
  const int64_t klast = (nk - 1) * BK;

  // The Wp half of a stage's loads, deferred to the next k-step 0: Wp rows
  // at pb, row limit pbl, k offset pkn, into slot pslot (stage 1's here).
  const char* pb = cur.b;
  int64_t pkn = BK;
  int pslot = 1;
  load_stage(cur, 0, 0);
  static_for<8>([&](auto uc) { load_u(cur.a, cur.b, 1, BK, uc); });
  wait_vm<8>();
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; ++q) read_one(0, 0, 0, q);
  int par = 0;   // slot of the current tile's stage 0
  while (true) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};
    for (int64_t c = 0; c < nk; ++c) {
      const int slot = (par + static_cast<int>(c)) & 1;
      // k-step 0: the fragments of k-step 1 and the deferred Wp loads between
      // the MFMAs; k-steps 1 and 2: the fragments of the next k-step.
      {
        static_for<16>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          mfma1(m, 0);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (m < 8) read_one(slot, 1, 1, m);
          if constexpr (m % 2 == 0) load_u(pb, pb, pslot, pkn, std::integral_constant<int, 8 + m / 2>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      static_for<2>([&](auto tc) {
        constexpr int tt = decltype(tc)::value + 1;
        static_for<16>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          mfma1(m, tt & 1);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (m < 8) read_one(slot, tt + 1, (tt + 1) & 1, m);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
      // k-step 3: wait for stage c+1 and the barrier that publishes it and
      // frees this slot (every wave holds this k-step's fragments); then the X
      // loads of stage c+2 (this tile's, else the next tile's stage c+2-nk,
      // else an unused in-bounds reload) and the fragments of stage c+1's
      // k-step 0 go between the MFMAs, and stage c+2's Wp loads wait for the
      // next k-step 0.
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<0>();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      const bool own = c + 2 < nk;
      const bool nx = !own && has_next;
      const char* sa_ = nx ? nxt.a : cur.a;
      const char* sb_ = nx ? nxt.b : cur.b;
      const int64_t kn = own ? (c + 2) * BK : (nx ? (c + 2 - nk) * BK : klast);
      static_for<16>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        mfma1(m, 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (m % 2 == 0) load_u(sa_, sb_, slot, kn, std::integral_constant<int, m / 2>{});
        if constexpr (m >= 1 && m <= 8) read_one(slot ^ 1, 0, 0, m - 1);
        __builtin_amdgcn_sched_barrier(0);
      });
      pb = sb_;
      pkn = kn;
      pslot = slot;
    }

    // Epilogue: bias b_j + sigma nb_i[j] with nb at offset + out*in + j.
    // Lane l holds column l % 32 of each 32-block and rows
    // 8 * (v / 4) + 4 * (l / 32) + v % 4 for v < 16.  Each accumulator is
    // copied out of its AGPR right before its store, so that no block's copies
    // are held at once.  (Without a bias the epilogue issues no loads: a load
    // here would wait for the next tile's stage loads too.)  The activation
    // and the ownership checks of a ragged tile are resolved per tile, so a
    // full tile's stores carry no per-element branches.
    {
      float bj[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (g.bias != nullptr) {
        const uint64_t s = load_seed(g.seeds, g.seeds_i32, cur.i);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t j = cur.ne + wn * 128 + b * 32 + l32;
          if (j < g.n) {
            const float nz = noise_of_state(state_of(s, static_cast<uint64_t>(g.offset + g.n * K + j)));
            bj[b] = __builtin_fmaf(g.sigma, nz, g.bias[j]);
          }
        }
      }
      const bool full = cur.me == cur.m0 && cur.ne == cur.n0;
      // the row pitch, opaque here so that the row steps below are formed per
      // tile rather than held in scalar registers through the k loop
      int64_t pitch = g.n;
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" : "+s"(pitch));
#endif
      // A lane's 16 values of a block lie in rows 0-3, 8-11, 16-19, 24-27 of
      // its 4-row offset: one row step within a group of four, five between.
      const int64_t step1 = pitch * 4, step5 = pitch * 20;
      auto store_tile = [&](auto checked, auto relu) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t j = cur.ne + wn * 128 + b * 32 + l32;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int64_t row0 = cur.me + wm * 128 + a * 32 + 4 * lh;
            char* yp = reinterpret_cast<char*>(g.y + (cur.i * g.m + row0) * pitch + j);
            // ragged tile: this lane stores row0 + ro when ro >= skip (the rows
            // before m0, or all 32 when the column belongs to the previous tile)
            const int skip = j < cur.n0 ? 32 : static_cast<int>(cur.m0 - row0 > 0 ? cur.m0 - row0 : 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float val = agpr_read(acc[a][b][v]) + bj[b];
              if constexpr (decltype(relu)::value) val = val > 0.0f ? val : 0.0f;
              if (!decltype(checked)::value || 8 * (v >> 2) + (v & 3) >= skip) *reinterpret_cast<float*>(yp) = val;
              yp += (v & 3) == 3 ? step5 : step1;
            }
          }
        }
      };
      if (full) {
        if (g.relu) store_tile(std::false_type{}, std::true_type{});
        else store_tile(std::false_type{}, std::false_type{});
      } else {
        if (g.relu) store_tile(std::true_type{}, std::true_type{});
        else store_tile(std::true_type{}, std::false_type{});
      }
    }
    if (!has_next) break;
    cur = nxt;
    par = (par + static_cast<int>(nk)) & 1;
    tnext += gridDim.x;
    has_next = tnext < total;
    if (has_next) setup(tnext, nxt);
  }
  // Drain the last (unused) loads before the workgroup's LDS is released.
  wait_vm<0>();
}

}  // namespace

static_assert(kMaterializeMinBatch >= BM, "a ragged last row tile is moved back by up to BM - 1 rows");

bool materialized_forward_applies(int64_t batch, int64_t in, int64_t out) {
  if (batch < kMaterializeMinBatch || in < 2 * BK || in % BK != 0 || in >= (int64_t{1} << 22) || out < BN ||
      out >= (int64_t{1} << 26))
    return false;
  const int64_t tm = (batch + BM - 1) / BM, tn = (out + BN - 1) / BN;
  return tm < (int64_t{1} << 31) / tn;
}

// Individuals per group: as many as kMaterializeBytes of perturbed weights
// hold (at least one), at most 65535 (grid.y of perturb_kernel) and fewer
// than 2^31 tiles in all (matmul_kernel counts them in 32 bits).
int64_t materialized_group(int64_t pop, int64_t batch, int64_t in, int64_t out) {
  const int64_t per = out * in * 2;
  const int64_t tiles = ((batch + BM - 1) / BM) * ((out + BN - 1) / BN);
  int64_t gsz = kMaterializeBytes / per;
  if (gsz > 65535) gsz = 65535;
  if (gsz > ((int64_t{1} << 31) - 1) / tiles) gsz = ((int64_t{1} << 31) - 1) / tiles;
  if (gsz < 1) gsz = 1;
  return gsz < pop ? gsz : pop;
}

int64_t materialized_workspace_bytes(int64_t pop, int64_t batch, int64_t in, int64_t out) {
  return materialized_group(pop, batch, in, out) * out * in * 2;
}

hipError_t launch_forward_bf16_materialized(const FwdParams& p, void* workspace, hipStream_t stream) {
  const int64_t gsz = materialized_group(p.pop, p.batch, p.in, p.out);
  const int64_t n = p.out * p.in;
  MatParams g;
  g.x = static_cast<const __bf16*>(p.x);
  g.x_pop_stride = p.x_pop_stride;
  g.wp = static_cast<const __bf16*>(workspace);
  g.wp_stride = n;
  g.bias = p.bias;
  g.seeds = p.seeds;
  g.seeds_i32 = p.seeds_i32;
  g.sigma = p.sigma;
  g.offset = p.offset;
  g.relu = p.relu;
  g.y = p.y;
  g.m = p.batch;
  g.n = p.out;
  g.k = p.in;
  g.tiles_m = static_cast<int32_t>((p.batch + BM - 1) / BM);
  g.tiles_n = static_cast<int32_t>((p.out + BN - 1) / BN);
  const int64_t runs = n / 8;
  const unsigned pblocks = static_cast<unsigned>((runs + 255) / 256 < 4096 ? (runs + 255) / 256 : 4096);
  for (int64_t i0 = 0; i0 < p.pop; i0 += gsz) {
    const int64_t gi = (p.pop - i0) < gsz ? (p.pop - i0) : gsz;
    perturb_kernel<<<dim3(pblocks, static_cast<unsigned>(gi)), 256, 0, stream>>>(
        static_cast<const __bf16*>(p.w), p.seeds, p.seeds_i32, i0, n, p.offset, p.sigma_q,
        static_cast<__bf16*>(workspace));
    g.i0 = i0;
    g.total_tiles = static_cast<int32_t>(gi * g.tiles_m * g.tiles_n);
    const unsigned grid = static_cast<unsigned>(g.total_tiles < kMatmulGrid ? g.total_tiles : kMatmulGrid);
    matmul_kernel<<<grid, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

}  // namespace vn
