// HIP kernels of the virtual-noise ES linear layer for gfx950 (MI355X).
//
// Method: EvoX API page "evox.triton_kernels.kernels.virtual_noise" -- module
// introduction (model and gradient equations), section "Noise indexing
// scheme", API entries virtual_perturbed_linear, virtual_weight_gradient,
// virtual_bias_gradient and virtual_reduce_metric.  The noise generator itself
// lives in vn_device.hpp.
//
// Design notes (gfx950):
//  * The hash (two 64-bit multiplies per element, built from 32-bit integer
//    multiplies) is the dominant cost of every entry point, so each noise
//    element is generated exactly once per (individual, element) and every
//    kernel is organised around keeping the vector ALUs busy with it.
//  * Forward (forward_mm_kernel, up to 256 rows): one workgroup (4 or 8 waves)
//    per (individual, column tile).  Each wave owns NB column blocks and ALL
//    rows of its individual's batch, so the noise it generates for a weight
//    element is reused by every batch row through the matrix cores.  The
//    perturbed weights W + sigma*N are generated directly in the MFMA
//    B-operand layout in VGPRs and never touch LDS or HBM.  The sum over k is
//    order-free, so each lane is given a contiguous run of k for its column:
//    consecutive noise indices differ by +GAMMA in the state (one 64-bit add
//    per element) and the W loads are 16-byte vectors.  The X rows of a
//    k-chunk are staged once per workgroup in LDS and read by every wave.
//  * Forward, larger batches (forward_rows_kernel): the waves split 512 rows
//    and share one LDS tile of W + sigma*N per k-chunk, so the noise is
//    generated once per 512 rows.
//  * Forward, 1-4 fp32 rows (forward_vec_kernel): products on the vector ALUs
//    in fp32; groups of 16 lanes split k and own columns in turn.
//  * Forward, fp32 matrix cores (forward_kernel): the same ownership with X
//    read straight from memory in the A layout; exact fp32 products.
//  * Layer chain (forward_chain_kernel): every layer of an MLP in one launch,
//    one workgroup per individual, activations kept in LDS.
//  * Gradients: element-major (lanes own consecutive elements, the population is
//    walked with wave-uniform scalar loads of seed and fitness, split over the
//    4 or 16 waves of a workgroup and reduced through LDS in a fixed order) for
//    large blocks;
//    population-major (lanes own individuals, one wave per element, fixed
//    butterfly reduction) for small blocks such as biases.
//  * Reduce metric (metric_kernel): one workgroup per (individual, segment),
//    runs of four centre values per thread, fixed-order sums; noise readout
//    (noise_kernel) for verification.
//  * No atomics anywhere: every output is a fixed-order reduction, so repeated
//    calls are bit-identical.
//  * Workgroup ids are remapped with the XCDs in mind (the hardware deals
//    workgroups round-robin over 8 XCDs, each with its own L2): the
//    workgroups an XCD runs together share X rows and W tiles (xcd_remap,
//    blocked_order).

#include <mutex>
#include <type_traits>

#include "vn_device.hpp"
#include "vn_launch.hpp"

namespace vn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kXcds = 8;

// Bijection on [0, n): hardware block b runs on XCD b % 8; give each XCD a
// contiguous range of logical ids.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t n) {
  const int64_t per = n / kXcds, rem = n % kXcds;
  const int64_t x = b % kXcds, local = b / kXcds;
  return (x < rem) ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

// (individual, column tile) of workgroup b when every individual has its own
// X and several column tiles.  Each XCD takes a contiguous range of the
// logical order (xcd_remap), which walks groups of IG individuals x all tiles,
// within a group blocks of TG tiles, individual fastest inside a block, with
// TG = min(n_tiles, 8) and IG = 64 / TG: a block of 64 consecutive workgroups
// of an XCD (one round of its 32 CUs at two workgroups per CU, two rounds at
// one) shares IG individuals' X rows and TG tiles of W in its L2.  On the
// 4096 -> 4096 bf16 projection (pop 128, batch 256, 16 tiles) reads beyond L2
// fell from 2.42 GB to 1.61 GB per launch against an order that ran each
// individual's tiles back to back on one XCD, in the same time.  A bijection
// on [0, pop * n_tiles) (the last group and block may be smaller).
__device__ __forceinline__ void blocked_order(int64_t b, int64_t n, int64_t pop, int64_t n_tiles, int64_t& i,
                                              int64_t& tile) {
  const int64_t TG = n_tiles < 8 ? n_tiles : 8;
  const int64_t IG = 64 / TG;
  const int64_t L = xcd_remap(b, n);
  const int64_t ig = L / (IG * n_tiles);
  const int64_t igs = (pop - ig * IG) < IG ? (pop - ig * IG) : IG;   // individuals in this group
  const int64_t rem = L - ig * IG * n_tiles;
  const int64_t tg = rem / (igs * TG);
  const int64_t w = rem - tg * igs * TG;
  i = ig * IG + w % igs;
  tile = tg * TG + w / igs;
}

// ---------------------------------------------------------------------------
// MFMA shapes.  For every shape below the A operand of lane l holds row
// (l % DIM) and the B operand holds column (l % DIM), both at the same k-slots
// selected by (l / DIM); the kernels rely only on that symmetry and on the
// output layout given by row_base() and row_off().
template <typename DT, int DIM> struct Mfma;

// Output element v of lane l sits at column l % DIM and row
// row_base(l) + row_off(v).
struct Out32 {
  static constexpr int NACC = 16;
  static __device__ __forceinline__ int row_base(int lane) { return 4 * (lane >> 5); }
  static constexpr int row_off(int v) { return 8 * (v >> 2) + (v & 3); }
};
struct Out16 {
  static constexpr int NACC = 4;
  static __device__ __forceinline__ int row_base(int lane) { return 4 * (lane >> 4); }
  static constexpr int row_off(int v) { return v; }
};
template <> struct Mfma<float, 32> : Out32 {   // v_mfma_f32_32x32x2_f32
  static constexpr int KPL = 1, H = 2;
  using Acc = f32x16;
};
template <> struct Mfma<float, 16> : Out16 {   // v_mfma_f32_16x16x4_f32
  static constexpr int KPL = 1, H = 4;
  using Acc = f32x4;
};
template <> struct Mfma<__bf16, 32> : Out32 {  // v_mfma_f32_32x32x16_bf16
  static constexpr int KPL = 8, H = 2;
  using Acc = f32x16;
};
template <> struct Mfma<__bf16, 16> : Out16 {  // v_mfma_f32_16x16x32_bf16
  static constexpr int KPL = 8, H = 4;
  using Acc = f32x4;
};

// Epilogue of the matrix-core forward kernels: y[r][j[nb]] = act(acc + bj[nb])
// for a lane's output rows r = rstart + mb * DIMR + MF::row_off(v) (rstart
// counted from y's row 0; with !FULL, only rows with mb * DIMR + row_off(v) <
// rleft) and its columns j[nb] < out.  The activation and the row check are
// compile-time, so a full tile's stores carry no per-element branches, and
// the address steps from one row to the next instead of being recomputed.
template <typename MF, int DIMR, bool FULL, bool RELU, int MB, int NB, typename Acc>
__device__ __forceinline__ void store_rows(float* __restrict__ y, int64_t rstart, int64_t rleft, int64_t out,
                                           const int64_t (&j)[NB], const float (&bj)[NB], const Acc (&acc)[MB][NB]) {
  const int64_t step = out * static_cast<int64_t>(sizeof(float));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (j[nb] >= out) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      char* yp = reinterpret_cast<char*>(y + (rstart + mb * DIMR) * out + j[nb]);
      const int64_t lim = rleft - mb * DIMR;
#pragma unroll
      for (int v = 0; v < MF::NACC; ++v) {
        float val = acc[mb][nb][v] + bj[nb];
        if constexpr (RELU) val = val > 0.0f ? val : 0.0f;
        if (FULL || MF::row_off(v) < lim) *reinterpret_cast<float*>(yp) = val;
        if (v + 1 < MF::NACC) yp += (MF::row_off(v + 1) - MF::row_off(v)) * step;
      }
    }
  }
}
template <typename MF, int DIMR, int MB, int NB, typename Acc>
__device__ __forceinline__ void store_outputs(bool full, bool relu, float* __restrict__ y, int64_t rstart,
                                              int64_t rleft, int64_t out, const int64_t (&j)[NB],
                                              const float (&bj)[NB], const Acc (&acc)[MB][NB]) {
  if (full) {
    if (relu) store_rows<MF, DIMR, true, true>(y, rstart, rleft, out, j, bj, acc);
    else store_rows<MF, DIMR, true, false>(y, rstart, rleft, out, j, bj, acc);
  } else {
    if (relu) store_rows<MF, DIMR, false, true>(y, rstart, rleft, out, j, bj, acc);
    else store_rows<MF, DIMR, false, false>(y, rstart, rleft, out, j, bj, acc);
  }
}

template <int DIM>
__device__ __forceinline__ typename Mfma<float, DIM>::Acc mfma_f32(float a, float b, typename Mfma<float, DIM>::Acc c) {
  if constexpr (DIM == 32) return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
template <int DIM>
__device__ __forceinline__ typename Mfma<__bf16, DIM>::Acc mfma_bf16(bf16x8 a, bf16x8 b, typename Mfma<__bf16, DIM>::Acc c) {
  if constexpr (DIM == 32) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }

template <typename DT> __device__ __forceinline__ DT zero_of() { return static_cast<DT>(0.0f); }

// R contiguous elements at p.  VEC: p is 16-byte aligned (checked on the host).
template <typename DT, int R, bool VEC>
__device__ __forceinline__ void load_run(DT (&dst)[R], const DT* p) {
  if constexpr (VEC) {
    constexpr int PER = 16 / sizeof(DT);
    static_assert(R % PER == 0, "run must be whole 16-byte vectors");
#pragma unroll
    for (int q = 0; q < R / PER; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + q * PER);
      __builtin_memcpy(&dst[q * PER], &v, 16);
    }
  } else {
#pragma unroll
    for (int t = 0; t < R; ++t) dst[t] = p[t];
  }
}

// First `valid` elements at p, zeros after (valid may be <= 0 or >= R).
template <typename DT, int R>
__device__ __forceinline__ void load_run_guarded(DT (&dst)[R], const DT* p, int valid) {
#pragma unroll
  for (int t = 0; t < R; ++t) dst[t] = (t < valid) ? p[t] : zero_of<DT>();
}

// ---------------------------------------------------------------------------
// Forward: Y[i] = X[i] (W + sigma N_i)^T + (b + sigma nb_i)
//
// DT   operand type (float or __bf16)
// DIM  MFMA block edge (32 or 16)
// MB   row blocks per wave (the wave covers MB*DIM batch rows)
// NB   column blocks per wave (the workgroup covers 4*NB*DIM columns)
// T    MFMAs per k-chunk; each lane holds a run of R = T*KPL contiguous k
template <typename DT, int DIM, int MB, int NB, int T, int WAVES, bool VEC>
__global__ __launch_bounds__(256, WAVES) void forward_kernel(FwdParams p, int64_t n_tiles) {
  using MF = Mfma<DT, DIM>;
  using Acc = typename MF::Acc;
  constexpr int R = T * MF::KPL;
  constexpr int KC = MF::H * R;
  constexpr int NT = 4 * NB * DIM;
  constexpr uint64_t kChunkStep = gamma_times(KC);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane % DIM;   // row (A) / column (B) inside a block
  const int lh = lane / DIM;   // k-slot group

  const int64_t in = p.in, out = p.out, batch = p.batch;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * (MB * DIM);
  const int64_t nfull = in / KC;
  const int rem = static_cast<int>(in - nfull * KC);

  {
    const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t i = L / n_tiles;
    const int64_t tile = L - i * n_tiles;

    const uint64_t s = load_seed(p.seeds, p.seeds_i32, i);
    const DT* __restrict__ xi = static_cast<const DT*>(p.x) + i * p.x_pop_stride;
    const DT* __restrict__ w = static_cast<const DT*>(p.w);

    const int64_t jbase = tile * NT + wave * (NB * DIM);
    const DT* wrow[NB];
    uint64_t z[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int64_t j = jbase + nb * DIM + ln;
      j = j < out ? j : out - 1;   // columns past `out` only feed discarded outputs
      wrow[nb] = w + j * in + lh * R;
      z[nb] = state_of(s, static_cast<uint64_t>(p.offset + j * in + lh * R));
    }
    const DT* xrow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int64_t b = m0 + mb * DIM + ln;
      b = b < batch ? b : batch - 1;  // rows past `batch` only feed discarded outputs
      xrow[mb] = xi + b * in + lh * R;
    }

    Acc acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Acc{};

    // One k-chunk: for each column block, generate the lane's run of perturbed
    // weights and feed it straight to the matrix cores (one block at a time
    // keeps the live noise state small).
    auto chunk = [&](const DT (&wv)[NB][R], const DT (&xv)[MB][R], int valid) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float wp[R];
#pragma unroll
        for (int t = 0; t < R; ++t) {
          const float nz = noise_of_state(z[nb] + gamma_times(t));
          const float v = __builtin_fmaf(p.sigma, nz, to_f32(wv[nb][t]));
          wp[t] = (t < valid) ? v : 0.0f;
        }
        z[nb] += kChunkStep;
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          if constexpr (sizeof(DT) == 4) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = mfma_f32<DIM>(xv[mb][tt], wp[tt], acc[mb][nb]);
          } else {
            bf16x8 bq;
#pragma unroll
            for (int e = 0; e < 8; ++e) bq[e] = static_cast<__bf16>(wp[tt * 8 + e]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              bf16x8 a;
#pragma unroll
              for (int e = 0; e < 8; ++e) a[e] = xv[mb][tt * 8 + e];
              acc[mb][nb] = mfma_bf16<DIM>(a, bq, acc[mb][nb]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    for (int64_t c = 0; c < nfull; ++c) {
      DT wv[NB][R], xv[MB][R];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) load_run<DT, R, VEC>(wv[nb], wrow[nb] + c * KC);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) load_run<DT, R, VEC>(xv[mb], xrow[mb] + c * KC);
      chunk(wv, xv, R);
    }
    if (rem > 0) {
      const int valid = rem - lh * R;
      DT wv[NB][R], xv[MB][R];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) load_run_guarded<DT, R>(wv[nb], wrow[nb] + nfull * KC, valid);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) load_run_guarded<DT, R>(xv[mb], xrow[mb] + nfull * KC, valid);
      chunk(wv, xv, valid);
    }

    // Epilogue: bias b_j + sigma nb_i[j] with nb at offset + out*in + j.
    const int rb = MF::row_base(lane);
    int64_t jj[NB];
    float bj[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      jj[nb] = jbase + nb * DIM + ln;
      bj[nb] = 0.0f;
      if (p.bias != nullptr && jj[nb] < out) {
        const float nz = noise_of_state(state_of(s, static_cast<uint64_t>(p.offset + out * in + jj[nb])));
        bj[nb] = __builtin_fmaf(p.sigma, nz, p.bias[jj[nb]]);
      }
    }
    store_outputs<MF, DIM>(m0 + MB * DIM <= batch, p.relu, p.y, i * batch + m0 + rb, batch - (m0 + rb), out, jj, bj,
                              acc);
  }
}

// ---------------------------------------------------------------------------
// Forward on the bf16 matrix cores with X staged through LDS.
//
// On gfx950 the fp32 MFMAs occupy the SIMD like VALU work (they do not run
// beside the integer hash), while bf16 MFMAs largely do.  This kernel
// therefore multiplies on v_mfma_f32_{32x32x16,16x16x32}_bf16 with fp32
// accumulation:
//   bf16 operands: A = X, B = bf16(W + sigma N) (one product);
//   fp32 operands (SPLIT): every operand v is split into hi = bf16(v) and
//     lo = bf16(v - hi) and the product is hi_x*hi_w + hi_x*lo_w + lo_x*hi_w,
//     which leaves a relative error of about 2^-16 per product (the dropped
//     lo*lo term and the split residuals); the sum is accumulated in fp32.
// The X rows of a k-chunk are loaded once per workgroup (not once per wave),
// split if needed, and kept in a double-buffered LDS tile that all the waves
// read; one barrier per chunk.  The noise side is as in forward_kernel:
// each lane generates its column's run of R = 16 consecutive k in registers.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> one dword of two bf16 (nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}
// The two bf16 halves of a packed dword back to fp32 (exact).
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

template <typename IN_T, bool SPLIT, int DIM, int MB, int NB, int R, int WAVES, int WPG, bool VEC>
__global__ __launch_bounds__(64 * WPG, WAVES) void forward_mm_kernel(FwdParams p, int64_t n_tiles) {
  using MF = Mfma<__bf16, DIM>;
  using Acc = typename MF::Acc;
  constexpr int H = MF::H;            // k-slot groups per MFMA
  static_assert(R % 8 == 0, "R: k per lane per chunk, whole MFMA k-slots");
  constexpr int T = R / 8;            // MFMAs per (row block, column block) per chunk
  constexpr int KC = H * R;           // k per chunk
  constexpr int ROWS = MB * DIM;
  constexpr int NT = WPG * NB * DIM;
  constexpr int NTHR = 64 * WPG;
  constexpr int STRIDE = KC + 8;      // LDS row pitch in bf16 (16-byte pad against bank conflicts)
  constexpr int PLANES = SPLIT ? 2 : 1;
  constexpr int PLANE = ROWS * STRIDE;
  constexpr int BUF = PLANES * PLANE;
  // A segment is SEGK consecutive k of one X row: 8, or 4 for fp32 when the
  // tile has fewer eight-wide segments than threads (so no thread repeats one).
  constexpr int SEGK = (sizeof(IN_T) == 4 && ROWS * KC / 8 < NTHR) ? 4 : 8;
  constexpr int SEG_LOADS = SEGK * static_cast<int>(sizeof(IN_T)) / 16;   // 16-byte loads per segment
  constexpr int SEG_PER_ROW = KC / SEGK;
  constexpr int NSEG = ROWS * SEG_PER_ROW;
  constexpr int SEG_PER_THREAD = (NSEG + NTHR - 1) / NTHR;
  constexpr uint64_t kChunkStep = gamma_times(KC);
  static_assert(!SPLIT || sizeof(IN_T) == 4, "split is for fp32 operands");

  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane % DIM;
  const int lh = lane / DIM;

  const int64_t in = p.in, out = p.out, batch = p.batch;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * ROWS;
  const int64_t nfull = VEC ? in / KC : 0;            // chunks taken on the unguarded path
  const int64_t nchunks = (in + KC - 1) / KC;

  int64_t i, tile;
  if (p.x_pop_stride != 0 && n_tiles > 1) {
    blocked_order(blockIdx.x, gridDim.x, p.pop, n_tiles, i, tile);
  } else {
    const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
    i = L / n_tiles;
    tile = L - i * n_tiles;
  }
  const uint64_t s = load_seed(p.seeds, p.seeds_i32, i);
  const IN_T* __restrict__ xi = static_cast<const IN_T*>(p.x) + i * p.x_pop_stride;
  const IN_T* __restrict__ w = static_cast<const IN_T*>(p.w);

  // ---- B side: this lane's columns, their W rows and noise states.  Columns
  // past `out` read the last column: they only feed discarded outputs.
  const int64_t jbase = tile * NT + wave * (NB * DIM);
  const IN_T* wrow[NB];
  uint64_t z[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int64_t j = jbase + nb * DIM + ln;
    j = j < out ? j : out - 1;
    wrow[nb] = w + j * in + lh * R;
    z[nb] = state_of(s, static_cast<uint64_t>(p.offset + j * in + lh * R));
  }

  // ---- A side: this thread's segments of the X tile.  Segment q covers row
  // q / SEG_PER_ROW and k = (q % SEG_PER_ROW) * SEGK .. + SEGK of the chunk.
  // Rows past `batch` read the last row: they only feed discarded outputs.
  const IN_T* xsrc[SEG_PER_THREAD];
  int xdst[SEG_PER_THREAD];
#pragma unroll
  for (int u = 0; u < SEG_PER_THREAD; ++u) {
    // Threads past the last segment (when the tile has fewer than 256 per
    // pass) repeat one: same source, same LDS slot, same bytes -- this keeps
    // the pipelined loop free of branches.
    const int q = (tid + u * NTHR) % NSEG;
    const int row = q / SEG_PER_ROW;
    const int kk = (q % SEG_PER_ROW) * SEGK;
    int64_t b = m0 + row;
    b = b < batch ? b : batch - 1;
    xsrc[u] = xi + b * in + kk;
    xdst[u] = row * STRIDE + kk;
  }
  IN_T xs[SEG_PER_THREAD][SEGK];
  auto load_x = [&](int64_t c, bool guarded) {
    const int64_t k0 = c * KC;
#pragma unroll
    for (int u = 0; u < SEG_PER_THREAD; ++u) {
      const IN_T* src = xsrc[u] + k0;
      if (!guarded) {
#pragma unroll
        for (int h = 0; h < SEG_LOADS; ++h) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + h * (16 / sizeof(IN_T)));
          __builtin_memcpy(&xs[u][h * (16 / sizeof(IN_T))], &v, 16);
        }
      } else {
        const int64_t kmax = in - (k0 + (xdst[u] % STRIDE));   // valid k left in this segment
        // (xdst % STRIDE is the segment's k offset within the chunk)
#pragma unroll
        for (int e = 0; e < SEGK; ++e) xs[u][e] = (e < kmax) ? src[e] : static_cast<IN_T>(0.0f);
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int u = 0; u < SEG_PER_THREAD; ++u) {
      if constexpr (sizeof(IN_T) == 2) {
        uint4 v;
        __builtin_memcpy(&v, &xs[u][0], 16);   // bf16 operands go to LDS as they are
        *reinterpret_cast<uint4*>(&lds[buf * BUF + xdst[u]]) = v;
      } else {
        using Packed = std::conditional_t<SEGK == 8, uint4, uint2>;   // SEGK bf16 values
        uint32_t hw[SEGK / 2], lw[SEGK / 2];
#pragma unroll
        for (int e = 0; e < SEGK / 2; ++e) {
          const float a = to_f32(xs[u][2 * e]), b = to_f32(xs[u][2 * e + 1]);
          hw[e] = pack_bf16x2(a, b);
          if constexpr (SPLIT) lw[e] = pack_bf16x2(a - bf16_lo_to_f32(hw[e]), b - bf16_hi_to_f32(hw[e]));
        }
        Packed hi, lo;
        __builtin_memcpy(&hi, hw, sizeof(Packed));
        *reinterpret_cast<Packed*>(&lds[buf * BUF + xdst[u]]) = hi;
        if constexpr (SPLIT) {
          __builtin_memcpy(&lo, lw, sizeof(Packed));
          *reinterpret_cast<Packed*>(&lds[buf * BUF + PLANE + xdst[u]]) = lo;
        }
      }
    }
  };

  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Acc{};

  // Software pipeline over k-chunks: iteration c generates the noise and the
  // packed B fragments of chunk c+1 on the VALU while the matrix cores work on
  // chunk c, whose B fragments were made in the previous iteration and whose X
  // tile sits in LDS buffer c & 1.  The X rows of chunk c+1 reach the other
  // buffer at the start of iteration c, those of chunk c+2 are loaded into
  // registers meanwhile; one barrier per iteration.
  IN_T wv[NB][R];                           // W runs of the chunk being prepared
  uint32_t bh[NB][R / 2], bl[NB][R / 2];    // packed B fragments of the chunk being multiplied

  auto load_w = [&](int64_t c, bool guarded) {
    if (!guarded) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) load_run<IN_T, R, true>(wv[nb], wrow[nb] + c * KC);
    } else {
      const int64_t left = in - c * KC;
      const int valid = left >= KC ? R : static_cast<int>(left) - lh * R;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) load_run_guarded<IN_T, R>(wv[nb], wrow[nb] + c * KC, valid);
    }
  };
  // Noise of chunk c (the lane's runs; consecutive k step the state by +GAMMA),
  // as the integers N * 2^24 (exact in fp32); sigma_q = sigma * 2^-24 scales
  // them back inside the fma of make_b.
  auto make_noise = [&](float (&nz)[NB][R]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint64_t zt = z[nb];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        nz[nb][t] = static_cast<float>(centered_q(zt));
        zt += kGamma;
      }
      z[nb] += kChunkStep;
    }
  };
  // W + sigma N of chunk c -> packed bf16 B fragments (hi, and lo when split).
  auto make_b = [&](const float (&nz)[NB][R], int64_t c, bool guarded) {
    int valid = R;
    if (guarded) {
      const int64_t left = in - c * KC;
      valid = left >= KC ? R : static_cast<int>(left) - lh * R;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int e = 0; e < R / 2; ++e) {
        float a = __builtin_fmaf(p.sigma_q, nz[nb][2 * e], to_f32(wv[nb][2 * e]));
        float b = __builtin_fmaf(p.sigma_q, nz[nb][2 * e + 1], to_f32(wv[nb][2 * e + 1]));
        if (guarded) {
          a = (2 * e < valid) ? a : 0.0f;
          b = (2 * e + 1 < valid) ? b : 0.0f;
        }
        bh[nb][e] = pack_bf16x2(a, b);
        if constexpr (SPLIT) bl[nb][e] = pack_bf16x2(a - bf16_lo_to_f32(bh[nb][e]), b - bf16_hi_to_f32(bh[nb][e]));
      }
    }
  };
  // Matrix cores on chunk c: A fragments from LDS buffer `buf`, B from bh/bl.
  auto multiply = [&](int buf) {
    const __bf16* abase = &lds[buf * BUF + ln * STRIDE + lh * R];
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(abase + mb * DIM * STRIDE + t * 8);
        bf16x8 alo;
        if constexpr (SPLIT) alo = *reinterpret_cast<const bf16x8*>(abase + PLANE + mb * DIM * STRIDE + t * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 bfh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bh[nb][t * 4]));
          if constexpr (SPLIT) {
            const bf16x8 bfl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bl[nb][t * 4]));
            acc[mb][nb] = mfma_bf16<DIM>(alo, bfh, acc[mb][nb]);
            acc[mb][nb] = mfma_bf16<DIM>(ahi, bfl, acc[mb][nb]);
          }
          acc[mb][nb] = mfma_bf16<DIM>(ahi, bfh, acc[mb][nb]);
        }
      }
    }
  };

  // Steady-state chunk: the noise of chunk c+1 and the MFMAs of chunk c,
  // interleaved by hand.  Each MFMA is fenced between scheduling barriers
  // with its share of the noise work in front of it, so consecutive MFMAs on
  // one accumulator sit a few hundred VALU cycles apart: the wave never waits
  // on the previous MFMA and the matrix cores run under the hash.  The A
  // fragments of the next (k-step, row block) are read from LDS while the
  // current one's MFMAs issue.
  auto noise_and_multiply = [&](int buf, float (&nz)[NB][R]) {
    constexpr int G = T * MB;                     // (k-step, row block) groups
    constexpr int PER_G = NB * (SPLIT ? 3 : 1);   // MFMAs per group
    constexpr int NM = G * PER_G;
    constexpr int NE = NB * R;                    // noise elements per lane
    const __bf16* abase = &lds[buf * BUF + ln * STRIDE + lh * R];
    bf16x8 ah[2], al[2];
    auto read_a = [&](int g) {
      const int t = g / MB, mb = g % MB;
      ah[g & 1] = *reinterpret_cast<const bf16x8*>(abase + mb * DIM * STRIDE + t * 8);
      if constexpr (SPLIT) al[g & 1] = *reinterpret_cast<const bf16x8*>(abase + PLANE + mb * DIM * STRIDE + t * 8);
    };
    read_a(0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int g = m / PER_G, w = m % PER_G;
      const int nb = w / (SPLIT ? 3 : 1), term = w % (SPLIT ? 3 : 1);
      const int t = g / MB, mb = g % MB;
      if (w == 0 && g + 1 < G) read_a(g + 1);
#pragma unroll
      for (int e = m * NE / NM; e < (m + 1) * NE / NM; ++e)
        nz[e / R][e % R] = static_cast<float>(centered_q(z[e / R] + gamma_times(e % R)));
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 bfh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bh[nb][t * 4]));
      if constexpr (SPLIT) {
        const bf16x8 bfl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bl[nb][t * 4]));
        if (term == 0) acc[mb][nb] = mfma_bf16<DIM>(al[g & 1], bfh, acc[mb][nb]);
        if (term == 1) acc[mb][nb] = mfma_bf16<DIM>(ah[g & 1], bfl, acc[mb][nb]);
        if (term == 2) acc[mb][nb] = mfma_bf16<DIM>(ah[g & 1], bfh, acc[mb][nb]);
      } else {
        acc[mb][nb] = mfma_bf16<DIM>(ah[g & 1], bfh, acc[mb][nb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) z[nb] += kChunkStep;
  };

  // A wave whose columns all lie past `out` (narrow layers) only helps stage
  // X and joins the barriers: no noise, no matrix work.
  const bool live = jbase < out;
#if defined(__HIP_DEVICE_COMPILE__)
  // 256 rows of bf16 operands: keep the 128 accumulator registers in the
  // accumulation register file (an accumulation-register clobber lets the
  // compiler choose that form of the matrix instructions), which leaves the
  // vector registers to the hash (1% faster on the 4096-wide layer).
  if constexpr (!SPLIT && MB == 8 && VEC) asm volatile("" ::: "a0");
#endif

  if (nchunks > 0) {
    load_x(0, nfull == 0);
    store_x(0);
    if (live) {
      load_w(0, nfull == 0);
      float nz[NB][R];
      make_noise(nz);
      make_b(nz, 0, nfull == 0);
    }
    if (nchunks > 1) load_x(1, nfull <= 1);
  }
  __syncthreads();
  // Steady state: chunks c+1 and c+2 are whole, nothing is guarded.
  int64_t c = 0;
  for (; c + 2 < nfull; ++c) {
    store_x(static_cast<int>((c + 1) & 1));
    load_x(c + 2, false);
    if (live) {
      load_w(c + 1, false);
      float nz[NB][R];
      noise_and_multiply(static_cast<int>(c & 1), nz);
      make_b(nz, c + 1, false);
    }
    __syncthreads();
  }
  // The last chunks: same steps with guards.
  for (; c < nchunks; ++c) {
    const bool next = c + 1 < nchunks;
    if (next) {
      store_x(static_cast<int>((c + 1) & 1));
      if (live) load_w(c + 1, c + 1 >= nfull);
      if (c + 2 < nchunks) load_x(c + 2, c + 2 >= nfull);
    }
    float nz[NB][R];
    if (next && live) make_noise(nz);
    if (live) multiply(static_cast<int>(c & 1));
    if (next && live) make_b(nz, c + 1, c + 1 >= nfull);
    __syncthreads();
  }

  // Epilogue: bias b_j + sigma nb_i[j] with nb at offset + out*in + j.
  const int rb = MF::row_base(lane);
  int64_t jj[NB];
  float bj[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    jj[nb] = jbase + nb * DIM + ln;
    bj[nb] = 0.0f;
    if (p.bias != nullptr && jj[nb] < out) {
      const float nz = noise_of_state(state_of(s, static_cast<uint64_t>(p.offset + out * in + jj[nb])));
      bj[nb] = __builtin_fmaf(p.sigma, nz, p.bias[jj[nb]]);
    }
  }
  store_outputs<MF, DIM>(m0 + MB * DIM <= batch, p.relu, p.y, i * batch + m0 + rb, batch - (m0 + rb), out, jj, bj,
                            acc);
}

// WAVES: waves per SIMD the register allocation must allow; WPG: waves per
// workgroup (each owns NB column blocks; all share the X tile).
template <typename IN_T, bool SPLIT, int DIM, int MB, int NB, int R, int WAVES, int WPG = 4>
static hipError_t launch_mm_cfg(const FwdParams& p, hipStream_t stream) {
  constexpr int NT = WPG * NB * DIM;
  constexpr int ROWS = MB * DIM;
  const int64_t n_tiles = (p.out + NT - 1) / NT;
  const int64_t total = p.pop * n_tiles;
  const int64_t m_tiles = (p.batch + ROWS - 1) / ROWS;
  if (total > kMaxGridX || m_tiles > 65535) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(total), static_cast<unsigned>(m_tiles));
  // 16-byte loads need 16-byte aligned bases, rows and individual strides.
  const int64_t per = 16 / static_cast<int64_t>(sizeof(IN_T));
  const bool vec = (reinterpret_cast<uintptr_t>(p.x) % 16 == 0) && (reinterpret_cast<uintptr_t>(p.w) % 16 == 0) &&
                   (p.in % per == 0) && (p.x_pop_stride % per == 0);
  if (vec)
    forward_mm_kernel<IN_T, SPLIT, DIM, MB, NB, R, WAVES, WPG, true><<<grid, 64 * WPG, 0, stream>>>(p, n_tiles);
  else
    forward_mm_kernel<IN_T, SPLIT, DIM, MB, NB, R, WAVES, WPG, false><<<grid, 64 * WPG, 0, stream>>>(p, n_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Forward for large batches.  The 8 waves of a workgroup split 512 batch rows
// (two 32-row blocks each) and share one 128-column tile of perturbed weights:
// per k-chunk of KC the workgroup generates the tile once -- thread t hashes
// the run of KC/4 consecutive k of column t / 4 -- and packs it to bf16 (hi and
// lo planes for fp32 operands) into a double-buffered LDS tile; every wave
// multiplies its own X rows, read straight from memory in the A layout,
// against the whole tile.  Each noise element is generated once per 512 rows,
// so past a few hundred rows the hash no longer binds: the tile takes
// (1/128 + 1/512) bytes of X and W per flop from L2, and the rate at which a
// compute unit can fetch them (its L1 keeps about 60 requests in flight)
// holds the matrix cores near a third of their peak.
template <typename IN_T, bool SPLIT, int KC, bool VEC>
__global__ __launch_bounds__(512, 1) void forward_rows_kernel(FwdParams p, int64_t n_tiles) {
  using MF = Mfma<__bf16, 32>;
  using Acc = typename MF::Acc;
  constexpr int WAVES = 8;
  constexpr int MBW = 2;                  // 32-row blocks per wave
  constexpr int NB = 4;                   // 32-column blocks: the whole tile
  constexpr int T = KC / 16;              // MFMA k-steps per chunk
  constexpr int NT = NB * 32;
  constexpr int ROWS_W = MBW * 32;
  constexpr int ROWS = WAVES * ROWS_W;
  constexpr int RB = NT * KC / (64 * WAVES);   // k per thread in the B tile
  constexpr int GPC = KC / RB;                 // threads per tile column
  constexpr int STRIDE = KC + 8;               // LDS column pitch in bf16 (16-byte pad)
  constexpr int PLANES = SPLIT ? 2 : 1;
  constexpr int PLANE = NT * STRIDE;
  constexpr int BUF = PLANES * PLANE;
  constexpr uint64_t kChunkStep = gamma_times(KC);
  static_assert(GPC == 4 && (RB == 4 || RB % 8 == 0), "tile generation mapping");

  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lh = lane >> 5;

  const int64_t in = p.in, out = p.out, batch = p.batch;
  const int64_t nfull = VEC ? in / KC : 0;     // chunks taken on the unguarded path
  const int64_t nchunks = (in + KC - 1) / KC;

  // Work order.  With a shared X the individuals of one column tile are
  // neighbours (they run together on one XCD and share its L2 copy of the W
  // tile and the X rows); otherwise the column tiles of one individual are
  // (they share that individual's X rows).
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  int64_t i, tile;
  if (p.x_pop_stride == 0) {
    tile = L / p.pop;
    i = L - tile * p.pop;
  } else {
    i = L / n_tiles;
    tile = L - i * n_tiles;
  }
  const uint64_t s = load_seed(p.seeds, p.seeds_i32, i);
  const IN_T* __restrict__ xi = static_cast<const IN_T*>(p.x) + i * p.x_pop_stride;
  const IN_T* __restrict__ w = static_cast<const IN_T*>(p.w);
  const int64_t j0 = tile * NT;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * ROWS + wave * ROWS_W;
  // A wave whose rows all lie past the batch only helps build the tiles.
  const bool live = m0 < batch;

  // ---- tile generation: this thread's column and run of RB k.  Columns past
  // `out` read the last column: they only feed discarded outputs.
  const int gcol = tid / GPC;
  const int gk = (tid % GPC) * RB;
  int64_t gj = j0 + gcol;
  gj = gj < out ? gj : out - 1;
  const IN_T* wsrc = w + gj * in + gk;
  uint64_t z = state_of(s, static_cast<uint64_t>(p.offset + gj * in + gk));
  const int gdst = gcol * STRIDE + gk;

  // ---- A side: row ln of each of the wave's row blocks, k-group lh.  Rows
  // past the batch read the last row: they only feed discarded outputs.
  const IN_T* xrow[MBW];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    int64_t r = m0 + mb * 32 + ln;
    r = r < batch ? r : batch - 1;
    xrow[mb] = xi + r * in + lh * 8;
  }

  IN_T wv[RB];                    // W run of the chunk being generated
  IN_T xr[MBW][T][8];                     // X of the chunk being loaded
  uint32_t ah[MBW][T][4], al[MBW][T][4];  // packed A fragments of the chunk being multiplied

  auto load_w = [&](int64_t c, bool guarded) {
    const int64_t k0 = c * KC;
    if (!guarded) {
      if constexpr (RB * sizeof(IN_T) >= 16) {
        load_run<IN_T, RB, true>(wv, wsrc + k0);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(wsrc + k0);
        __builtin_memcpy(wv, &v, 8);
      }
    } else {
      load_run_guarded<IN_T, RB>(wv, wsrc + k0, static_cast<int>(in - k0 - gk));
    }
  };
  auto load_x = [&](int64_t c, bool guarded) {
    const int64_t k0 = c * KC;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if (!guarded)
          load_run<IN_T, 8, true>(xr[mb][t], xrow[mb] + k0 + t * 16);
        else
          load_run_guarded<IN_T, 8>(xr[mb][t], xrow[mb] + k0 + t * 16, static_cast<int>(in - k0 - t * 16 - lh * 8));
      }
  };
  // The thread's run of W + sigma N -> LDS buffer `buf` (hi, and lo when split).
  auto store_tile = [&](int buf, const float (&v)[RB]) {
    uint32_t hw[RB / 2], lw[RB / 2];
#pragma unroll
    for (int e = 0; e < RB / 2; ++e) {
      hw[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      if constexpr (SPLIT) lw[e] = pack_bf16x2(v[2 * e] - bf16_lo_to_f32(hw[e]), v[2 * e + 1] - bf16_hi_to_f32(hw[e]));
    }
    using Packed = std::conditional_t<RB >= 8, uint4, uint2>;
    constexpr int NPK = RB / 2 * 4 / static_cast<int>(sizeof(Packed));
#pragma unroll
    for (int q = 0; q < NPK; ++q) {
      Packed h2;
      __builtin_memcpy(&h2, &hw[q * sizeof(Packed) / 4], sizeof(Packed));
      *reinterpret_cast<Packed*>(&lds[buf * BUF + gdst + q * sizeof(Packed) / 2]) = h2;
      if constexpr (SPLIT) {
        Packed l2;
        __builtin_memcpy(&l2, &lw[q * sizeof(Packed) / 4], sizeof(Packed));
        *reinterpret_cast<Packed*>(&lds[buf * BUF + PLANE + gdst + q * sizeof(Packed) / 2]) = l2;
      }
    }
  };
  auto make_tile = [&](int buf) {
    float v[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t)
      v[t] = __builtin_fmaf(p.sigma_q, static_cast<float>(centered_q(z + gamma_times(t))), to_f32(wv[t]));
    z += kChunkStep;
    store_tile(buf, v);
  };
  // X of the loaded chunk -> packed A fragments (hi, and lo when split);
  // bf16 operands are the fragments as loaded.
  auto make_a = [&]() {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        if constexpr (sizeof(IN_T) == 2) {
          __builtin_memcpy(ah[mb][t], xr[mb][t], 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = to_f32(xr[mb][t][2 * e]), b = to_f32(xr[mb][t][2 * e + 1]);
            ah[mb][t][e] = pack_bf16x2(a, b);
            if constexpr (SPLIT)
              al[mb][t][e] = pack_bf16x2(a - bf16_lo_to_f32(ah[mb][t][e]), b - bf16_hi_to_f32(ah[mb][t][e]));
          }
        }
      }
  };

  Acc acc[MBW][NB];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Acc{};

  auto multiply = [&](int buf) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const __bf16* bsrc = &lds[buf * BUF + (nb * 32 + ln) * STRIDE + t * 16 + lh * 8];
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(bsrc);
        bf16x8 bl;
        if constexpr (SPLIT) bl = *reinterpret_cast<const bf16x8*>(bsrc + PLANE);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
          const bf16x8 a_h = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ah[mb][t]));
          if constexpr (SPLIT) {
            const bf16x8 a_l = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(al[mb][t]));
            acc[mb][nb] = mfma_bf16<32>(a_l, bh, acc[mb][nb]);
            acc[mb][nb] = mfma_bf16<32>(a_h, bl, acc[mb][nb]);
          }
          acc[mb][nb] = mfma_bf16<32>(a_h, bh, acc[mb][nb]);
        }
      }
  };

  // bf16 operands: the B fragments of a chunk are read right after the barrier
  // that publishes its tile (their latency hides behind the hash), and the
  // tile of the next chunk is built with the MFMAs of this one placed among
  // its steps.  The hash of the thread's RB elements advances in five
  // lockstep steps (RB independent chains each); each step shares its
  // scheduling region with a fifth of the MFMAs, which the scheduler spreads
  // one per ten vector instructions, so that the matrix cores run while the
  // wave keeps issuing the hash.  (fp32 operands double the B fragments and
  // would spill; they keep the plain order.)
  bf16x8 bfh[T][NB];
  auto read_b = [&](int buf) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bfh[t][nb] = *reinterpret_cast<const bf16x8*>(&lds[buf * BUF + (nb * 32 + ln) * STRIDE + t * 16 + lh * 8]);
  };
  auto tile_and_multiply = [&](int tbuf) {
    constexpr int NM = T * NB * MBW;
    constexpr int NST = 5;
    uint64_t zz[RB];
    float v[RB];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int e = 0; e < RB; ++e) {
        if (st == 0) zz[e] = xorshift(z + gamma_times(e), 30);
        if (st == 1) zz[e] = mul_gamma(zz[e]);
        if (st == 2) zz[e] = xorshift(zz[e], 27);
        if (st == 3) zz[e] = keep_words(mul_gamma(zz[e]));
        if (st == 4) v[e] = __builtin_fmaf(p.sigma_q, static_cast<float>(final_centered(zz[e])), to_f32(wv[e]));
      }
#pragma unroll
      for (int m = st * NM / NST; m < (st + 1) * NM / NST; ++m) {
        const int mb = m % MBW, nb = (m / MBW) % NB, t = m / (MBW * NB);
        const bf16x8 a_h = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ah[mb][t]));
        acc[mb][nb] = mfma_bf16<32>(a_h, bfh[t][nb], acc[mb][nb]);
      }
#pragma unroll
      for (int m = st * NM / NST; m < (st + 1) * NM / NST; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    z += kChunkStep;
    store_tile(tbuf, v);
  };

  // Software pipeline: iteration c loads X of chunk c+1, builds the tile of
  // chunk c+1 in the other LDS buffer from the W run loaded one iteration
  // earlier and loads the W run of chunk c+2, while the matrix cores work on
  // chunk c; then it packs the X of chunk c+1 into the A fragments.  One
  // barrier per iteration.  (Loading W in the same iteration as its tile left
  // every tile build waiting on a global load.)  bf16 operands take the
  // interleaved step above in the steady state.
  if (nchunks > 0) {
    load_w(0, nfull == 0);
    load_x(0, nfull == 0);
    make_tile(0);
    make_a();
    if (nchunks > 1) load_w(1, nfull <= 1);
  }
  __syncthreads();
  int64_t c = 0;
  for (; c + 2 < nfull; ++c) {
    if constexpr (!SPLIT) {
      // (a wave whose rows all lie past the batch multiplies clamped rows here
      // and discards the result: keeping the MFMAs unconditional keeps them in
      // the hash's scheduling regions)
      read_b(static_cast<int>(c & 1));
      load_x(c + 1, false);
      tile_and_multiply(static_cast<int>((c + 1) & 1));
      load_w(c + 2, false);
    } else {
      load_x(c + 1, false);
      make_tile(static_cast<int>((c + 1) & 1));
      load_w(c + 2, false);
      if (live) multiply(static_cast<int>(c & 1));
    }
    make_a();
    __syncthreads();
  }
  for (; c < nchunks; ++c) {
    const bool next = c + 1 < nchunks;
    if (next) {
      load_x(c + 1, c + 1 >= nfull);
      make_tile(static_cast<int>((c + 1) & 1));
      if (c + 2 < nchunks) load_w(c + 2, c + 2 >= nfull);
    }
    if (live) multiply(static_cast<int>(c & 1));
    if (next) make_a();
    __syncthreads();
  }

  // Epilogue: bias b_j + sigma nb_i[j] with nb at offset + out*in + j.
  if (!live) return;
  const int rb = MF::row_base(lane);
  int64_t jj[NB];
  float bj[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    jj[nb] = j0 + nb * 32 + ln;
    bj[nb] = 0.0f;
    if (p.bias != nullptr && jj[nb] < out) {
      const float nz = noise_of_state(state_of(s, static_cast<uint64_t>(p.offset + out * in + jj[nb])));
      bj[nb] = __builtin_fmaf(p.sigma, nz, p.bias[jj[nb]]);
    }
  }
  store_outputs<MF, 32>(m0 + MBW * 32 <= batch, p.relu, p.y, i * batch + m0 + rb, batch - (m0 + rb), out, jj, bj,
                            acc);
}

template <typename IN_T, bool SPLIT>
static hipError_t launch_rows(const FwdParams& p, hipStream_t stream) {
  constexpr int NT = 128, ROWS = 512;
  const int64_t n_tiles = (p.out + NT - 1) / NT;
  const int64_t total = p.pop * n_tiles;
  const int64_t m_tiles = (p.batch + ROWS - 1) / ROWS;
  if (total > kMaxGridX || m_tiles > 65535) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(total), static_cast<unsigned>(m_tiles));
  // 16-byte loads need 16-byte aligned bases, rows and individual strides.
  const int64_t per = 16 / static_cast<int64_t>(sizeof(IN_T));
  const bool vec = (reinterpret_cast<uintptr_t>(p.x) % 16 == 0) && (reinterpret_cast<uintptr_t>(p.w) % 16 == 0) &&
                   (p.in % per == 0) && (p.x_pop_stride % per == 0);
  if (vec)
    forward_rows_kernel<IN_T, SPLIT, 32, true><<<grid, 512, 0, stream>>>(p, n_tiles);
  else
    forward_rows_kernel<IN_T, SPLIT, 32, false><<<grid, 512, 0, stream>>>(p, n_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Forward for one or two fp32 rows per individual, on the vector ALUs.  With
// so few rows the matrix cores would idle and the bf16 split would cost more
// than the products; here every lane multiplies in fp32 directly.  A group of
// 16 lanes owns NCW columns in turn; lane g of the group takes the run of RL
// consecutive k at g*RL of every chunk of 16*RL, keeps its X values for the
// chunk in registers (reused by all NCW columns) and accumulates
// x * (W + sigma N) per column; the 16 partial sums of a column are combined
// by a fixed butterfly at the end.
template <int B, int NCW, int RL, bool VEC>
__global__ __launch_bounds__(256, 4) void forward_vec_kernel(FwdParams p, int64_t n_tiles) {
  constexpr int KC = 16 * RL;                 // k per chunk
  constexpr int NT = 16 * NCW;                // columns per workgroup (4 waves x 4 groups)
  constexpr uint64_t kChunkStep = gamma_times(KC);
  static_assert(RL % 4 == 0, "whole 16-byte loads");
  const int tid = threadIdx.x;
  const int grp = tid >> 4;                   // 16 groups per workgroup
  const int g = tid & 15;

  const int64_t in = p.in, out = p.out, batch = p.batch;
  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t i = L / n_tiles;
  const int64_t tile = L - i * n_tiles;
  const uint64_t s = load_seed(p.seeds, p.seeds_i32, i);
  const float* __restrict__ xi = static_cast<const float*>(p.x) + i * p.x_pop_stride;
  const float* __restrict__ w = static_cast<const float*>(p.w);

  // this group's columns: tile*NT + grp + 16*c, c < NCW (clamped past `out`)
  const float* wrow[NCW];
  uint64_t z[NCW];
#pragma unroll
  for (int c = 0; c < NCW; ++c) {
    int64_t j = tile * NT + grp + 16 * c;
    j = j < out ? j : out - 1;
    wrow[c] = w + j * in + g * RL;
    z[c] = state_of(s, static_cast<uint64_t>(p.offset + j * in + g * RL));
  }
  float acc[NCW][B];
#pragma unroll
  for (int c = 0; c < NCW; ++c)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[c][b] = 0.0f;

  const int64_t nchunks = (in + KC - 1) / KC;
  const int64_t nfull = VEC ? in / KC : 0;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t k0 = ch * KC + g * RL;
    const bool whole = ch < nfull;
    const int valid = whole ? RL : static_cast<int>(in - k0);
    float xv[B][RL];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int64_t bb = b < batch ? b : batch - 1;   // rows past the batch only feed discarded outputs
      const float* xs = xi + bb * in + k0;
      if (whole)
        load_run<float, RL, true>(xv[b], xs);
      else
        load_run_guarded<float, RL>(xv[b], xs, valid);
    }
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      float wv[RL];
      if (whole)
        load_run<float, RL, true>(wv, wrow[c] + ch * KC);
      else
        load_run_guarded<float, RL>(wv, wrow[c] + ch * KC, valid);
#pragma unroll
      for (int t = 0; t < RL; ++t) {
        const float wp = __builtin_fmaf(p.sigma_q, static_cast<float>(centered_q(z[c] + gamma_times(t))), wv[t]);
#pragma unroll
        for (int b = 0; b < B; ++b) acc[c][b] = __builtin_fmaf(xv[b][t], wp, acc[c][b]);
      }
      z[c] += kChunkStep;
    }
  }

  // Combine the 16 partial sums of each column (fixed butterfly), epilogue.
#pragma unroll
  for (int c = 0; c < NCW; ++c) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = acc[c][b];
#pragma unroll
      for (int d = 8; d >= 1; d >>= 1) v += __shfl_xor(v, d, 16);
      acc[c][b] = v;
    }
    const int64_t j = tile * NT + grp + 16 * c;
    if (g != 0 || j >= out) continue;
    float bj = 0.0f;
    if (p.bias != nullptr) {
      const float nz = noise_of_state(state_of(s, static_cast<uint64_t>(p.offset + out * in + j)));
      bj = __builtin_fmaf(p.sigma, nz, p.bias[j]);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (b >= batch) break;
      float val = acc[c][b] + bj;
      if (p.relu) val = val > 0.0f ? val : 0.0f;
      p.y[(i * batch + b) * out + j] = val;
    }
  }
}

template <int B>
static hipError_t launch_vec(const FwdParams& p, hipStream_t stream) {
  constexpr int NCW = B >= 4 ? 2 : 4, RL = 8;   // columns per lane group, k per lane per chunk
  constexpr int NT = 16 * NCW;
  const int64_t n_tiles = (p.out + NT - 1) / NT;
  const int64_t total = p.pop * n_tiles;
  if (total > kMaxGridX) return hipErrorInvalidConfiguration;
  const bool vec = (reinterpret_cast<uintptr_t>(p.x) % 16 == 0) && (reinterpret_cast<uintptr_t>(p.w) % 16 == 0) &&
                   (p.in % 4 == 0) && (p.x_pop_stride % 4 == 0);
  if (vec)
    forward_vec_kernel<B, NCW, RL, true><<<static_cast<unsigned>(total), 256, 0, stream>>>(p, n_tiles);
  else
    forward_vec_kernel<B, NCW, RL, false><<<static_cast<unsigned>(total), 256, 0, stream>>>(p, n_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// A chain of layers in one launch: every output width <= 256, batch <= 64,
// any input width.  One 8-wave workgroup per individual.  The first layer
// streams X through a double-buffered LDS tile as forward_mm_kernel does
// (8 waves x 32 columns, one barrier per k-chunk); its output and every
// later activation stay in LDS (bf16 hi/lo planes for fp32 operands), so the
// later layers need no barrier inside their k loops and no activation ever
// reaches HBM.  In the resident layers the 32-column blocks of the output are
// spread over the waves: with 5..8 blocks one wave per block, with fewer
// several waves share a block and split its k-chunks (chunk c to wave
// c mod wpb), their partial sums added through LDS in wave order.  A wave
// hashes its columns' noise in registers exactly as forward_mm_kernel does.
// After each layer the waves write the next activation (bias, ReLU, split)
// over the old one; the last layer writes Y.
template <typename IN_T, bool SPLIT>
__global__ __launch_bounds__(512, 4) void forward_chain_kernel(ChainParams p) {
  using MF = Mfma<__bf16, 32>;
  using Acc = typename MF::Acc;
  constexpr int WAVES = 8, NTHR = 64 * WAVES;
  constexpr int MB = 2;                        // 64 rows
  constexpr int R = SPLIT ? 8 : 16;            // k per lane per chunk (fp32 operands: hi and lo runs, half as long)
  constexpr int T = R / 8;
  constexpr int KC = MF::H * R;                // 32
  constexpr int ROWS = MB * 32;
  constexpr int ASTRIDE = kChainMaxWidth + 8;  // resident rows: LDS pitch in bf16 (16-byte pad)
  constexpr int PLANES = SPLIT ? 2 : 1;
  constexpr int PLANE = ROWS * ASTRIDE;
  constexpr int SSTRIDE = KC + 8;              // streamed X chunks: LDS pitch
  constexpr int SPLANE = ROWS * SSTRIDE;
  constexpr int SBUF = PLANES * SPLANE;        // one staging buffer (two, inside `act`)
  constexpr int SEGK = (sizeof(IN_T) == 4 && ROWS * KC / 8 < NTHR) ? 4 : 8;
  constexpr int SEG_PER_ROW = KC / SEGK;
  constexpr int NSEG = ROWS * SEG_PER_ROW;
  constexpr int PART = MB * MF::NACC * 64;     // floats of one wave's partial sums
  // all partial sums of a layer whose blocks are shared must fit the activation buffer
  constexpr int kMaxLive = (PLANES * PLANE * 2) / (PART * 4) >= WAVES ? WAVES : (PLANES * PLANE * 2) / (PART * 4);
  static_assert(kMaxLive >= 1, "room for one wave's partial sums");
  static_assert(ROWS == kChainMaxBatch, "one row tile holds the batch");
  static_assert(2 * SBUF <= PLANES * PLANE, "the staging buffers fit the activation buffer");
  static_assert(NSEG <= NTHR, "one X segment per thread");

  __shared__ __attribute__((aligned(16))) __bf16 act[PLANES * PLANE];
  float* const part = reinterpret_cast<float*>(act);   // reused for partial sums after a layer's k loop

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lh = lane >> 5;
  // (wave-uniform values pinned to scalar registers: the k loops need every VGPR)
  const int64_t i = __builtin_amdgcn_readfirstlane(static_cast<int>(xcd_remap(blockIdx.x, gridDim.x)));
  const int64_t batch = p.batch;
  const uint64_t s0 = load_seed(p.seeds, p.seeds_i32, i);
  const uint64_t s = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(s0 >> 32))) << 32) |
                     __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(s0));

  auto put = [&](int r, int k, float v) {      // v -> act[r][k] (hi, lo)
    const __bf16 h = static_cast<__bf16>(v);
    act[r * ASTRIDE + k] = h;
    if constexpr (SPLIT) act[PLANE + r * ASTRIDE + k] = static_cast<__bf16>(v - static_cast<float>(h));
  };

  for (int l = 0; l < p.n_layers; ++l) {
    const int64_t in = p.dims[l], out = p.dims[l + 1];
    const bool last = l + 1 == p.n_layers;
    const bool streamed = l == 0;
    const int nblk = static_cast<int>((out + 31) / 32);
    int wpb = 1;                               // waves per column block (a power of two); 1 when streamed
    if (!streamed)
      while (wpb * 2 * nblk <= kMaxLive) wpb *= 2;
    const int blk = wave / wpb, q = wave % wpb;
    const bool live = blk < nblk;
    const int64_t jbase = static_cast<int64_t>(blk) * 32;
    Acc acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = Acc{};

    int64_t jc = jbase + ln;
    jc = jc < out ? jc : out - 1;              // columns past `out` feed only discarded outputs
    const IN_T* __restrict__ wrow = static_cast<const IN_T*>(p.w[l]) + jc * in + lh * R;
    uint64_t z = state_of(s, static_cast<uint64_t>(p.offset[l] + jc * in + q * KC + lh * R));
    const uint64_t zstep = gamma_times(KC) * static_cast<uint64_t>(wpb);
    const bool wvec = (p.wvec >> l) & 1u;
    const int64_t nch = (in + KC - 1) / KC;
    const int64_t nfull = wvec ? in / KC : 0;  // chunks whose lane runs all lie inside `in`
    IN_T wv[R];
    uint32_t bh[R / 2], bl[R / 2];
    auto load_w = [&](int64_t c, bool guarded) {
      if (!guarded) {
        load_run<IN_T, R, true>(wv, wrow + c * KC);
      } else {
        const int64_t left = in - c * KC - lh * R;
        load_run_guarded<IN_T, R>(wv, wrow + c * KC, left >= R ? R : static_cast<int>(left));
      }
    };
    // noise of the lane's run of chunk c (as N * 2^24) folded into W + sigma N
    auto make_b = [&](int64_t c, bool guarded) {
      int valid = R;
      if (guarded) {
        const int64_t left = in - c * KC - lh * R;
        valid = left >= R ? R : static_cast<int>(left);
      }
      float v[R];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const float w1 = __builtin_fmaf(p.sigma_q, static_cast<float>(centered_q(z + gamma_times(t))), to_f32(wv[t]));
        v[t] = (!guarded || t < valid) ? w1 : 0.0f;
      }
      z += zstep;
#pragma unroll
      for (int e = 0; e < R / 2; ++e) {
        bh[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        if constexpr (SPLIT) bl[e] = pack_bf16x2(v[2 * e] - bf16_lo_to_f32(bh[e]), v[2 * e + 1] - bf16_hi_to_f32(bh[e]));
      }
    };
    // MFMAs of one chunk: A fragments from `abase` (row pitch `pitch`, planes
    // `plane` apart), B from bh/bl.
    auto multiply = [&](const __bf16* abase, int pitch, int plane) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bf16x8 bfh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bh[t * 4]));
        bf16x8 bfl;
        if constexpr (SPLIT) bfl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&bl[t * 4]));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(abase + mb * 32 * pitch + t * 8);
          if constexpr (SPLIT) {
            const bf16x8 alo = *reinterpret_cast<const bf16x8*>(abase + plane + mb * 32 * pitch + t * 8);
            acc[mb] = mfma_bf16<32>(alo, bfh, acc[mb]);
            acc[mb] = mfma_bf16<32>(ahi, bfl, acc[mb]);
          }
          acc[mb] = mfma_bf16<32>(ahi, bfh, acc[mb]);
        }
      }
    };

    if (streamed) {
      // ---- first layer: X chunks staged through two buffers inside `act`.
      // Thread t stages segment t (threads past the last repeat one: same
      // source, same slot, same bytes).  Rows past the batch read the last row.
      const int qs = tid % NSEG;
      const int srow = qs / SEG_PER_ROW, skk = (qs % SEG_PER_ROW) * SEGK;
      const IN_T* __restrict__ xsrc = static_cast<const IN_T*>(p.x) + i * p.x_pop_stride +
                                      (srow < batch ? srow : batch - 1) * in + skk;
      const int sdst = srow * SSTRIDE + skk;
      const int64_t xfull = p.xvec ? in / KC : 0;   // chunks staged with 16-byte loads
      IN_T xs[SEGK];
      auto load_x = [&](int64_t c) {
        if (c < xfull) {
#pragma unroll
          for (int h = 0; h < SEGK * static_cast<int>(sizeof(IN_T)) / 16; ++h) {
            const uint4 v = *reinterpret_cast<const uint4*>(xsrc + c * KC + h * (16 / sizeof(IN_T)));
            __builtin_memcpy(&xs[h * (16 / sizeof(IN_T))], &v, 16);
          }
        } else {
          const int64_t kmax = in - c * KC - skk;
#pragma unroll
          for (int e = 0; e < SEGK; ++e) xs[e] = (e < kmax) ? xsrc[c * KC + e] : static_cast<IN_T>(0.0f);
        }
      };
      auto store_x = [&](int buf) {
        using Packed = std::conditional_t<SEGK == 8, uint4, uint2>;
        uint32_t hw[SEGK / 2], lw[SEGK / 2];
#pragma unroll
        for (int e = 0; e < SEGK / 2; ++e) {
          const float a = to_f32(xs[2 * e]), b = to_f32(xs[2 * e + 1]);
          hw[e] = pack_bf16x2(a, b);
          if constexpr (SPLIT) lw[e] = pack_bf16x2(a - bf16_lo_to_f32(hw[e]), b - bf16_hi_to_f32(hw[e]));
        }
        Packed hi, lo;
        __builtin_memcpy(&hi, hw, sizeof(Packed));
        *reinterpret_cast<Packed*>(&act[buf * SBUF + sdst]) = hi;
        if constexpr (SPLIT) {
          __builtin_memcpy(&lo, lw, sizeof(Packed));
          *reinterpret_cast<Packed*>(&act[buf * SBUF + SPLANE + sdst]) = lo;
        }
      };
      auto mult_chunk = [&](int buf) { multiply(&act[buf * SBUF + ln * SSTRIDE + lh * R], SSTRIDE, SPLANE); };
      // iteration c: stage chunk c+1, load chunk c+2, prepare B of chunk c+1
      // while chunk c multiplies; one barrier per chunk.
      if (nch > 0) {
        load_x(0);
        store_x(0);
        if (live) {
          load_w(0, 0 >= nfull);
          make_b(0, 0 >= nfull);
        }
        if (nch > 1) load_x(1);
      }
      __syncthreads();
      for (int64_t c = 0; c < nch; ++c) {
        const bool next = c + 1 < nch;
        if (next) {
          store_x(static_cast<int>((c + 1) & 1));
          if (c + 2 < nch) load_x(c + 2);
        }
        if (live) {
          if (next) load_w(c + 1, c + 1 >= nfull);
          mult_chunk(static_cast<int>(c & 1));
          if (next) make_b(c + 1, c + 1 >= nfull);
        }
        __syncthreads();
      }
    } else if (live) {
      // ---- resident layers: this wave's chunks q, q + wpb, ...; the W run
      // and noise of the next one are prepared while the current one
      // multiplies (no barrier inside).
      auto mult_res = [&](int64_t c) { multiply(&act[ln * ASTRIDE + c * KC + lh * R], ASTRIDE, PLANE); };
      int64_t c = q;
      if (c < nch) {
        load_w(c, c >= nfull);
        make_b(c, c >= nfull);
      }
      for (; c + wpb < nfull; c += wpb) {
        load_w(c + wpb, false);
        mult_res(c);
        make_b(c + wpb, false);
      }
      for (; c < nch; c += wpb) {
        const bool next = c + wpb < nch;
        if (next) load_w(c + wpb, c + wpb >= nfull);
        mult_res(c);
        if (next) make_b(c + wpb, c + wpb >= nfull);
      }
    }
    __syncthreads();                           // every wave is done reading the activations

    if (wpb > 1) {
      // partial sums of the waves sharing a block, added in wave order
      if (live) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < MF::NACC; ++v) part[((wave * MB + mb) * MF::NACC + v) * 64 + lane] = acc[mb][v];
      }
      __syncthreads();
      if (live) {
        // value e = mb * NACC + v of the block belongs to its wave e % wpb,
        // which adds the block's partial sums in wave order (the waves share
        // the additions and the stores below)
        const int w0 = wave - q;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < MF::NACC; ++v) {
            if ((mb * MF::NACC + v) % wpb != q) continue;
            float t = part[((w0 * MB + mb) * MF::NACC + v) * 64 + lane];
            for (int u = 1; u < wpb; ++u) t += part[(((w0 + u) * MB + mb) * MF::NACC + v) * 64 + lane];
            acc[mb][v] = t;
          }
      }
      __syncthreads();                         // partial sums consumed
    }

    if (live) {
      const int64_t j = jbase + ln;
      float bj = 0.0f;
      if (p.bias[l] != nullptr && j < out) {
        const float nz = noise_of_state(state_of(s, static_cast<uint64_t>(p.offset[l] + out * in + j)));
        bj = __builtin_fmaf(p.sigma, nz, p.bias[l][j]);
      }
      int rb = MF::row_base(lane);
#if defined(__HIP_DEVICE_COMPILE__)
      // keep the row addresses inside the layer loop (hoisted, they are spilled)
      asm volatile("" : "+v"(rb));
#endif
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int v = 0; v < MF::NACC; ++v) {
          if ((mb * MF::NACC + v) % wpb != q) continue;   // another wave of the block stores it
          const int row = mb * 32 + rb + MF::row_off(v);
          float val = acc[mb][v] + bj;
          if (last) {
            if (row < batch && j < out) p.y[(i * batch + row) * out + j] = val;
          } else {
            if (p.relu) val = val > 0.0f ? val : 0.0f;
            put(row, static_cast<int>(j), j < out ? val : 0.0f);   // dead columns are the next layer's zero k tail
          }
        }
      }
    }
    __syncthreads();                           // the next activations are in place
  }
}

hipError_t launch_chain(const ChainParams& p, bool bf16, hipStream_t stream) {
  if (p.pop > kMaxGridX) return hipErrorInvalidConfiguration;
  const unsigned grid = static_cast<unsigned>(p.pop);
  if (bf16)
    forward_chain_kernel<__bf16, false><<<grid, 512, 0, stream>>>(p);
  else
    forward_chain_kernel<float, true><<<grid, 512, 0, stream>>>(p);
  return hipGetLastError();
}

template <typename IN_T, bool SPLIT>
static hipError_t launch_mm_dtype(const FwdParams& p, hipStream_t stream) {
  // <DIM, MB row blocks, NB column blocks per wave, R k per lane per chunk,
  //  waves per SIMD>, chosen by measurement on MI355X.
  if (p.batch <= 16) return launch_mm_cfg<IN_T, SPLIT, 16, 1, 1, 16, 4>(p, stream);
  // Narrow outputs: 16-wide column blocks waste the least noise work on
  // columns past `out` (whole waves past it are skipped in the kernel).
  if (p.out <= 16 && p.batch <= 64) return launch_mm_cfg<IN_T, SPLIT, 16, 4, 1, 16, 2>(p, stream);
  // 17..32 rows: 8-wave workgroups (256 columns) stage each X tile once for
  // twice the columns -- the same time on the MLP hidden layer, 37% fewer
  // bytes fetched (161 MB against 257 MB per launch) -- unless the layer is
  // narrow.
  if (p.batch <= 32)
    return p.out > 128 ? launch_mm_cfg<IN_T, SPLIT, 32, 1, 1, 16, 4, 8>(p, stream)
                       : launch_mm_cfg<IN_T, SPLIT, 32, 1, 1, 16, 4>(p, stream);
  // 33..64 rows: 8-wave workgroups (256 columns) share each staged X tile
  // over twice the columns, unless the layer is narrow.
  if (p.batch <= 64 && p.out <= 128) return launch_mm_cfg<IN_T, SPLIT, 32, 2, 1, 16, 4>(p, stream);
  if (p.batch <= 64) return launch_mm_cfg<IN_T, SPLIT, 32, 2, 1, 16, 4, 8>(p, stream);
  if (p.batch <= 128) return launch_mm_cfg<IN_T, SPLIT, 32, 4, 1, 16, 2>(p, stream);
  // 129..256 rows: 8-wave workgroups, each staged X tile serving 256 columns
  // (3% faster on the 4096-wide bf16 layer at 256 rows than 4 waves).
  if (p.batch <= 256) return launch_mm_cfg<IN_T, SPLIT, 32, 8, 1, 16, 2, 8>(p, stream);
  // Larger batches: 512 rows per workgroup sharing one generated weight tile
  // (more rows take further row tiles on grid.y).
  return launch_rows<IN_T, SPLIT>(p, stream);
}

// WAVES: waves per SIMD the register allocation must allow.
template <typename DT, int DIM, int MB, int NB, int T, int WAVES>
static hipError_t launch_fwd_cfg(const FwdParams& p, hipStream_t stream) {
  constexpr int NT = 4 * NB * DIM;
  constexpr int ROWS = MB * DIM;
  constexpr int R = T * Mfma<DT, DIM>::KPL;
  const int64_t n_tiles = (p.out + NT - 1) / NT;
  const int64_t total = p.pop * n_tiles;
  const int64_t m_tiles = (p.batch + ROWS - 1) / ROWS;
  if (total > kMaxGridX || m_tiles > 65535) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(total), static_cast<unsigned>(m_tiles));
  // 16-byte vector loads need every lane's run start to be 16-byte aligned:
  // base pointers aligned, row length and pop stride multiples of 16 bytes.
  const int64_t per = 16 / static_cast<int64_t>(sizeof(DT));
  const bool vec = (reinterpret_cast<uintptr_t>(p.x) % 16 == 0) && (reinterpret_cast<uintptr_t>(p.w) % 16 == 0) &&
                   (p.in % per == 0) && (p.x_pop_stride % per == 0) && (R % per == 0);
  if (vec)
    forward_kernel<DT, DIM, MB, NB, T, WAVES, true><<<grid, 256, 0, stream>>>(p, n_tiles);
  else
    forward_kernel<DT, DIM, MB, NB, T, WAVES, false><<<grid, 256, 0, stream>>>(p, n_tiles);
  return hipGetLastError();
}

// Tile choice by batch size.  Each wave holds all rows of its individual in
// MB row blocks, so every noise element is generated once per individual.
template <typename DT, int T16, int T32, int TBIG>
static hipError_t launch_fwd_dtype(const FwdParams& p, hipStream_t stream) {
  if (p.batch <= 16) return launch_fwd_cfg<DT, 16, 1, 2, T16, 2>(p, stream);
  if (p.batch <= 32) return launch_fwd_cfg<DT, 32, 1, 2, T32, 2>(p, stream);
  if (p.batch <= 64) return launch_fwd_cfg<DT, 32, 2, 2, T32, 2>(p, stream);
  if (p.batch <= 128) return launch_fwd_cfg<DT, 32, 4, 1, TBIG, 2>(p, stream);
  // 256 rows per workgroup; larger batches take several row tiles (grid.y),
  // each regenerating the same noise.
  return launch_fwd_cfg<DT, 32, 8, 1, TBIG, 2>(p, stream);
}

hipError_t launch_forward_f32(const FwdParams& p, hipStream_t stream) {
  switch (p.batch) {
    case 1: return launch_vec<1>(p, stream);
    case 2: return launch_vec<2>(p, stream);
    case 3: return launch_vec<3>(p, stream);
    case 4: return launch_vec<4>(p, stream);
    default: break;
  }
  return launch_mm_dtype<float, true>(p, stream);
}
hipError_t launch_forward_f32_exact(const FwdParams& p, hipStream_t stream) {
  return launch_fwd_dtype<float, 4, 8, 4>(p, stream);
}
hipError_t launch_forward_bf16(const FwdParams& p, hipStream_t stream) {
  return launch_mm_dtype<__bf16, false>(p, stream);
}
hipError_t launch_forward_bf16_exact(const FwdParams& p, hipStream_t stream) {
  return launch_fwd_cfg<__bf16, 32, 8, 1, 1, 2>(p, stream);
}

// ---------------------------------------------------------------------------
// Gradient, element-major: grad[t] = scale * sum_i f_i noise_i[offset + t].
// A workgroup owns 64*E consecutive elements, lane l of every wave the E at
// l*E; its S waves split the population into S contiguous parts.  Each wave
// walks its part in groups of four individuals, whose seeds and fitness values
// (wave-uniform, scalar loads) are fetched one group ahead.  The S partial sums
// of an element are added in wave order.  The sums run over the integers
// N * 2^24 and take the 2^-24 at the end: a power-of-two factor, so every
// rounding is the one of the sum over N.
template <int E, bool SEEDS_I32, int S>
__global__ __launch_bounds__(64 * S) void grad_elem_kernel(GradParams p, int64_t n_blocks) {
  static_assert(S >= E, "the final sums take one thread per element");
  __shared__ float red[S][64 * E];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t q = p.pop / S, r = p.pop % S;
  const int64_t i_begin = wave * q + (wave < r ? wave : r);
  const int64_t i_end = i_begin + q + (wave < r ? 1 : 0);
  // Nothing the kernel writes aliases the inputs: lets the compiler use scalar loads.
  const float* __restrict__ fitness = p.fitness;
  const int64_t* __restrict__ seeds64 = static_cast<const int64_t*>(p.seeds);
  const int32_t* __restrict__ seeds32 = static_cast<const int32_t*>(p.seeds);
  float* __restrict__ out = p.out;
  auto seed = [&](int64_t i) -> uint64_t {
    return SEEDS_I32 ? static_cast<uint64_t>(static_cast<int64_t>(seeds32[i])) : static_cast<uint64_t>(seeds64[i]);
  };

  for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
    const int64_t e0 = blk * (64 * E) + lane * E;
    uint64_t c[E];
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int64_t t = e0 + e;
      t = t < p.n ? t : p.n - 1;
      c[e] = state_of(0, static_cast<uint64_t>(p.offset + t));
      acc[e] = 0.0f;
    }
    int64_t i = i_begin;
    uint64_t sn[4];
    float fn[4];
    if (i + 4 <= i_end) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sn[u] = seed(i + u);
        fn[u] = fitness[i + u];
      }
    }
    for (; i + 4 <= i_end; i += 4) {
      uint64_t sc[4];
      float fc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sc[u] = sn[u];
        fc[u] = fn[u];
      }
      if (i + 8 <= i_end) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sn[u] = seed(i + 4 + u);
          fn[u] = fitness[i + 4 + u];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(fc[u], static_cast<float>(centered_q(sc[u] + c[e])), acc[e]);
    }
    for (; i < i_end; ++i) {
      const uint64_t s = seed(i);
      const float f = fitness[i];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(f, static_cast<float>(centered_q(s + c[e])), acc[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) red[wave][lane * E + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < 64 * E) {
      const int k = threadIdx.x;
      float v = red[0][k];
#pragma unroll
      for (int w = 1; w < S; ++w) v += red[w][k];
      const int64_t t = blk * (64 * E) + k;
      if (t < p.n) out[t] = (v * 0x1p-24f) * p.scale;
    }
    __syncthreads();
  }
}

// Waves per workgroup.  Workgroups are handed out in rounds of (CUs x
// workgroups a CU holds, 8 of 4 waves here); a last, partly filled round leaves
// most of the chip idle for one workgroup's duration.  With 16 waves a
// workgroup takes a quarter as long as with 4 for the same work, which shortens
// that round, but each wave then pays its setup and the final sums over a
// quarter of the noise.  Measured: 16 waves gain 7% when a wave's part is 1024
// noise values per lane in 2052 workgroups (population 4096, 512x256 layer),
// and lose 2-8% when it would be 64-256 values; so 16 only for few workgroups
// (under four rounds) and when a 4-wave part is at least 1024 values.
inline int grad_elem_waves(int64_t n_blocks, int64_t pop, int e) {
  return (n_blocks < 8192 && pop * e >= 4096) ? 16 : 4;
}

template <int E, int S>
static void launch_grad_elem_s(const GradParams& p, int64_t n_blocks, hipStream_t stream) {
  const int64_t g = n_blocks < kMaxGridX ? n_blocks : kMaxGridX;
  if (p.seeds_i32)
    grad_elem_kernel<E, true, S><<<static_cast<unsigned>(g), 64 * S, 0, stream>>>(p, n_blocks);
  else
    grad_elem_kernel<E, false, S><<<static_cast<unsigned>(g), 64 * S, 0, stream>>>(p, n_blocks);
}

template <int E>
static void launch_grad_elem(const GradParams& p, hipStream_t stream) {
  const int64_t n_blocks = (p.n + 64 * E - 1) / (64 * E);
  if (grad_elem_waves(n_blocks, p.pop, E) == 16)
    launch_grad_elem_s<E, 16>(p, n_blocks, stream);
  else
    launch_grad_elem_s<E, 4>(p, n_blocks, stream);
}

// Gradient, population-major: one wave per element, lanes own individuals.
__global__ __launch_bounds__(256) void grad_pop_kernel(GradParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t t = wave_id; t < p.n; t += n_waves) {
    const uint64_t c = state_of(0, static_cast<uint64_t>(p.offset + t));
    float acc = 0.0f;
    for (int64_t i = lane; i < p.pop; i += 64)
      acc = __builtin_fmaf(p.fitness[i], static_cast<float>(centered_q(load_seed(p.seeds, p.seeds_i32, i) + c)), acc);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) p.out[t] = (acc * 0x1p-24f) * p.scale;
  }
}

hipError_t launch_gradient(const GradParams& p, hipStream_t stream) {
  if (p.n <= 16384) {
    const int64_t waves = p.n;
    int64_t blocks = (waves + 3) / 4;
    blocks = blocks < 65536 ? blocks : 65536;
    grad_pop_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(p);
  } else if (p.n < (int64_t(1) << 20)) {
    launch_grad_elem<1>(p, stream);
  } else {
    launch_grad_elem<4>(p, stream);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Noise readout: r[i, t] and/or N[i, t] for indices offset + t.
__global__ __launch_bounds__(256) void noise_kernel(const void* seeds, bool seeds_i32, int64_t pop, int64_t n,
                                                    int64_t offset, uint32_t* r_out, float* n_out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = blockIdx.y; i < pop; i += gridDim.y) {
    const uint64_t s = load_seed(seeds, seeds_i32, i);
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < n; t += stride) {
      const uint32_t r = mix_lo32(state_of(s, static_cast<uint64_t>(offset + t)));
      if (r_out) r_out[i * n + t] = r;
      if (n_out) n_out[i * n + t] = noise_of_bits(r);
    }
  }
}

hipError_t launch_noise(const void* seeds, bool seeds_i32, int64_t pop, int64_t n, int64_t offset,
                        uint32_t* r_out, float* n_out, hipStream_t stream) {
  int64_t gx = (n + 255) / 256;
  gx = gx < 4096 ? gx : 4096;
  const int64_t gy = pop < 65535 ? pop : 65535;
  noise_kernel<<<dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), 256, 0, stream>>>(
      seeds, seeds_i32, pop, n, offset, r_out, n_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reduce metric: out[i] = mean_k |center[k] + sigma noise_i[offset + k]|.
// A 1024-thread workgroup (16 waves) reduces one segment of one individual:
// thread t takes the runs of four consecutive k starting at 4 (t + 1024 m)
// within the segment; its sum, the wave butterfly and the sum over the 16
// waves all have a fixed order.  With one segment per individual the
// workgroup writes the mean; otherwise it writes a partial sum and
// metric_finish adds an individual's partials in segment order.
constexpr int kMetricThreads = 1024;

// The same with the noise formed as N itself (for |sigma| < 2^-100).
__global__ __launch_bounds__(256) void metric_kernel_small_sigma(const float* center, const void* seeds,
                                                                 bool seeds_i32, int64_t pop, int64_t n, float sigma,
                                                                 int64_t offset, float* out) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  for (int64_t i = blockIdx.x; i < pop; i += gridDim.x) {
    const uint64_t s = load_seed(seeds, seeds_i32, i);
    uint64_t z = state_of(s, static_cast<uint64_t>(offset + tid));
    float acc = 0.0f;
    for (int64_t k = tid; k < n; k += 256) {
      acc += __builtin_fabsf(__builtin_fmaf(sigma, noise_of_state(z), center[k]));
      z += gamma_times(256);
    }
    red[tid] = acc;
    __syncthreads();
#pragma unroll
    for (int h = 128; h >= 1; h >>= 1) {
      if (tid < h) red[tid] += red[tid + h];
      __syncthreads();
    }
    if (tid == 0) out[i] = red[0] / static_cast<float>(n);
    __syncthreads();
  }
}

struct MetricParams {
  const float* center;
  const void* seeds;
  bool seeds_i32;
  bool vec;           // center 16-byte aligned: runs of four as one load
  int64_t pop, n, offset;
  int64_t seg_len;    // elements per segment, a multiple of 4
  int64_t n_seg;      // segments per individual
  float sigma_q;      // sigma * 2^-24
  float* out;         // (pop,) means when n_seg == 1, else (pop, n_seg) partial sums
};

__global__ __launch_bounds__(kMetricThreads) void metric_kernel(MetricParams p) {
  __shared__ float red[kMetricThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr uint64_t kStep = gamma_times(4 * kMetricThreads);
  const int64_t units = p.pop * p.n_seg;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t i = u / p.n_seg, seg = u - i * p.n_seg;
    const int64_t k0 = seg * p.seg_len;
    const int64_t k1 = k0 + p.seg_len < p.n ? k0 + p.seg_len : p.n;
    const int64_t nvec = p.vec ? (k1 - k0) / 4 : 0;          // whole runs of four
    const uint64_t s = load_seed(p.seeds, p.seeds_i32, i);
    float acc = 0.0f;
    uint64_t z = state_of(s, static_cast<uint64_t>(p.offset + k0 + 4 * tid));
    for (int64_t v = tid; v < nvec; v += kMetricThreads) {
      const float4 c = reinterpret_cast<const float4*>(p.center + k0)[v];
      acc += __builtin_fabsf(__builtin_fmaf(p.sigma_q, static_cast<float>(centered_q(z)), c.x));
      acc += __builtin_fabsf(__builtin_fmaf(p.sigma_q, static_cast<float>(centered_q(z + gamma_times(1))), c.y));
      acc += __builtin_fabsf(__builtin_fmaf(p.sigma_q, static_cast<float>(centered_q(z + gamma_times(2))), c.z));
      acc += __builtin_fabsf(__builtin_fmaf(p.sigma_q, static_cast<float>(centered_q(z + gamma_times(3))), c.w));
      z += kStep;
    }
    for (int64_t k = k0 + 4 * nvec + tid; k < k1; k += kMetricThreads)
      acc += __builtin_fabsf(__builtin_fmaf(
          p.sigma_q, static_cast<float>(centered_q(state_of(s, static_cast<uint64_t>(p.offset + k)))), p.center[k]));
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < kMetricThreads / 64; ++w) t += red[w];
      p.out[u] = p.n_seg == 1 ? t / static_cast<float>(p.n) : t;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void metric_finish(const float* partial, int64_t pop, int64_t n_seg, int64_t n,
                                                     float* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= pop) return;
  float t = 0.0f;
  for (int64_t g = 0; g < n_seg; ++g) t += partial[i * n_seg + g];
  out[i] = t / static_cast<float>(n);
}

// Segments per individual.  A CU holds two of these 16-wave workgroups (8
// waves per SIMD), 512 on the chip.  From one such round of individuals on,
// one segment each is fastest (no finishing launch: 6% on 512 individuals of
// 269K parameters).  Smaller populations split into segments of at least 64K
// elements, aiming at two whole rounds (1024 workgroups; 1-3% faster than 1.5).
static int64_t metric_segments(int64_t pop, int64_t n) {
  constexpr int64_t kOneRound = 512, kTargetGroups = 1024, kMinSeg = 65536;
  if (pop >= kOneRound) return 1;
  int64_t seg = (kTargetGroups + pop - 1) / pop;
  const int64_t by_len = n / kMinSeg;
  if (seg > by_len) seg = by_len;
  return seg < 1 ? 1 : seg;
}

int64_t reduce_metric_workspace_floats(int64_t pop, int64_t n) {
  const int64_t seg = metric_segments(pop, n);
  return seg > 1 ? pop * seg : 0;
}

// Partial sums of the allocation-free reduce metric: one array per GPU,
// alive until the process ends.  Every call on a GPU uses that GPU's copy
// (calls that overlap on one GPU race); each call writes every slot it
// reads before reading it, so nothing needs clearing between calls.
static __device__ __align__(256) float scratch[kMetricScratchFloats];

hipError_t metric_scratch_address(float** ptr) {
  // The address of a device's copy, looked up once per device with that
  // device current (host code must not use the array's name itself).
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(a);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_reduce_metric(const float* center, const void* seeds, bool seeds_i32, int64_t pop, int64_t n,
                                float sigma, int64_t offset, float* out, float* workspace, hipStream_t stream) {
  // sigma * 2^-24 scales the integer noise (r >> 8) - 2^23; below 2^-100 it
  // would be subnormal, so such a sigma takes the kernel that forms sigma * N.
  if (sigma != 0.0f && __builtin_fabsf(sigma) < 0x1p-100f) {
    const int64_t g = pop < 65536 ? pop : 65536;
    metric_kernel_small_sigma<<<static_cast<unsigned>(g), 256, 0, stream>>>(center, seeds, seeds_i32, pop, n, sigma,
                                                                            offset, out);
    return hipGetLastError();
  }
  MetricParams p;
  p.center = center;
  p.seeds = seeds;
  p.seeds_i32 = seeds_i32;
  p.vec = reinterpret_cast<uintptr_t>(center) % 16 == 0;
  p.pop = pop;
  p.n = n;
  p.offset = offset;
  p.n_seg = metric_segments(pop, n);
  p.seg_len = p.n_seg == 1 ? n : ((n + p.n_seg - 1) / p.n_seg + 3) / 4 * 4;
  p.n_seg = (n + p.seg_len - 1) / p.seg_len;    // the last segment is never empty
  p.sigma_q = sigma * 0x1p-24f;
  p.out = p.n_seg == 1 ? out : workspace;
  const int64_t units = pop * p.n_seg;
  const int64_t g = units < 65536 ? units : 65536;
  metric_kernel<<<static_cast<unsigned>(g), kMetricThreads, 0, stream>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_seg == 1) return e;
  metric_finish<<<static_cast<unsigned>((pop + 255) / 256), 256, 0, stream>>>(workspace, pop, p.n_seg, n, out);
  return hipGetLastError();
}

}  // namespace vn
