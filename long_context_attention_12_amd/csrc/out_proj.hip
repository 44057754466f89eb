// out_proj.hip — grouped output projection after core attention.
//
// [Qiaomu] 预训练策略 (model configurations) and [cdjax] §1.1: the n_h heads
// form g groups of n_h/g heads; each group's head outputs (n_h/g * c values
// per row) project to d_g channels, the g results concatenate, and a second
// projection maps the g * d_g channels to the model width (Flash: 64 heads of
// 512 in 8 groups of 1024, model width 4096; Pro: 128 heads in 16 groups,
// width 7168). [kwkr] §3.4: this keeps the output projection small when
// heads are many.
//
// Both stages are products C = A B^T with B in the layout of a linear layer's
// weight ([N, K], row n = output channel n), bf16 operands, fp32 sums, bf16
// results (the intermediate stays bf16 as the operand of the second stage).
// At decode the rows are few (16 - 64) and the weights are many (128 MB for
// Flash): the kernel is a weight stream. A workgroup owns 16 output columns;
// its eight waves take an eighth of K each, load their weight rows with
// 16-byte loads straight into MFMA operands (a batch of 4 - 8 steps in flight
// behind the one being summed), and keep every row of the block in up to four
// 16-row MFMA tiles, so each weight byte is read once per 64 rows. The eight
// partial tiles are summed through LDS in a fixed order (deterministic).
#include "lca_device.h"
#include "lca_internal.h"
#include "../../include/lca.h"

namespace lca {
namespace {

constexpr int kProjWaves = 8;                      // waves per workgroup, one eighth of K each
constexpr int kProjThreads = 64 * kProjWaves;

// Batch of U K-steps (32 each) of one wave: B fragments of its 16 columns and
// A fragments of its MT row tiles, 16 bytes per lane per fragment.
template <int MT, int U>
struct ProjBatch {
  bf16x8 b[U];
  bf16x8 a[MT][U];
};

template <int MT, int U>
__device__ __forceinline__ void proj_load(ProjBatch<MT, U>& x, const uint16_t* bp, const uint16_t* const (&ap)[MT],
                                          int ks) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    x.b[u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(bp + ks + 32 * u));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      x.a[mt][u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ap[mt] + ks + 32 * u));
  }
}

template <int MT, int U>
__device__ __forceinline__ void proj_mfma(const ProjBatch<MT, U>& x, f32x4 (&acc)[MT]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.a[mt][u], x.b[u], acc[mt], 0, 0, 0);
}

// C[m, n] = sum_k A[m, k] B[n, k] for the rows [m0, m0 + 16 MT) and columns
// [n0, n0 + 16) of group blockIdx.y. Wave w sums K in [w K/8, (w + 1) K/8) in
// batches of U steps, the next batch's loads in flight while the current one
// feeds the MFMAs; the eight partial tiles add in a fixed order.
template <int MT>
__global__ __launch_bounds__(kProjThreads) void proj_nt_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                               int64_t a_group, const uint16_t* __restrict__ Bw,
                                                               int64_t b_group, uint16_t* __restrict__ C,
                                                               int64_t ldc, int64_t c_group, int M, int K) {
  constexpr int U = MT <= 2 ? 4 : 2;              // two batches of U steps in flight (registers for 2+ workgroups per CU)
  __shared__ float red[kProjWaves][MT * 256];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int gi = blockIdx.y;
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.z * 16 * MT;
  const int kq = K / kProjWaves, k0 = wid * kq;
  const int kk = 8 * (lane >> 4);                  // the lane's 8 K values in each step of 32
  // lane l: column n0 + l % 16 of B, rows m0 + 16 mt + l % 16 of A (rows past M
  // read row M - 1, and their results are dropped)
  const uint16_t* bp = Bw + gi * b_group + static_cast<int64_t>(n0 + (lane & 15)) * K + k0 + kk;
  const uint16_t* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = m0 + 16 * mt + (lane & 15);
    if (r > M - 1) r = M - 1;
    ap[mt] = A + gi * a_group + static_cast<int64_t>(r) * lda + k0 + kk;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nb = kq / (32 * U);                    // whole batches
  ProjBatch<MT, U> x0, x1;
  if (nb > 0) proj_load<MT, U>(x0, bp, ap, 0);
  for (int j = 0; j < nb; j += 2) {
    if (j + 1 < nb) proj_load<MT, U>(x1, bp, ap, (j + 1) * 32 * U);
    proj_mfma<MT, U>(x0, acc);
    if (j + 2 < nb) proj_load<MT, U>(x0, bp, ap, (j + 2) * 32 * U);
    if (j + 1 < nb) proj_mfma<MT, U>(x1, acc);
  }
  for (int ks = nb * 32 * U; ks < kq; ks += 32) {
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(bp + ks));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ap[mt] + ks));
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[mt], 0, 0, 0);
    }
  }
  // lane l holds C rows 4 (l / 16) + i, column l % 16 of each tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wid][mt * 256 + lane * 4 + i] = acc[mt][i];
  __syncthreads();
  uint16_t* c = C + gi * c_group;
  for (int e = threadIdx.x; e < MT * 256; e += kProjThreads) {
    const int mt = e >> 8, el = e & 255;
    const int row = 4 * ((el >> 2) >> 4) + (el & 3), col = (el >> 2) & 15;
    float v = red[0][e];
#pragma unroll
    for (int w = 1; w < kProjWaves; ++w) v += red[w][e];
    const int m = m0 + 16 * mt + row;
    if (m < M) c[static_cast<int64_t>(m) * ldc + n0 + col] = f32_to_bf16(v);
  }
}

template <int MT>
void launch_proj(LaunchScope& sc, const uint16_t* A, int64_t lda, int64_t a_group, const uint16_t* Bw,
                 int64_t b_group, uint16_t* C, int64_t ldc, int64_t c_group, int M, int N, int K, int groups) {
  const dim3 grid(N / 16, groups, (M + 16 * MT - 1) / (16 * MT));
  sc.launch(proj_nt_kernel<MT>, grid, dim3(kProjThreads), 0, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, K);
}

void launch_proj_any(LaunchScope& sc, const uint16_t* A, int64_t lda, int64_t a_group, const uint16_t* Bw,
                     int64_t b_group, uint16_t* C, int64_t ldc, int64_t c_group, int M, int N, int K, int groups) {
  // rows per workgroup: as few 16-row tiles as cover M, up to four (64 rows)
  if (M <= 16) launch_proj<1>(sc, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, N, K, groups);
  else if (M <= 32) launch_proj<2>(sc, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, N, K, groups);
  else launch_proj<4>(sc, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, N, K, groups);
}

}  // namespace

hipError_t launch_grouped_out_proj(hipStream_t s, const OutProjArgs& p) {
  const int64_t kg = static_cast<int64_t>(p.n_h / p.g) * p.c;          // K of a group
  const int64_t mid_w = static_cast<int64_t>(p.g) * p.d_g;
  const uint16_t* o = static_cast<const uint16_t*>(p.o);
  uint16_t* mid = static_cast<uint16_t*>(p.mid);
  {
    LaunchScope scope(s, "out_proj_groups");
    launch_proj_any(scope, o, static_cast<int64_t>(p.n_h) * p.c, kg, static_cast<const uint16_t*>(p.w_g),
                    static_cast<int64_t>(p.d_g) * kg, mid, mid_w, p.d_g, p.T, p.d_g, static_cast<int>(kg), p.g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope scope(s, "out_proj_merge");
    launch_proj_any(scope, mid, mid_w, 0, static_cast<const uint16_t*>(p.w_o), 0, static_cast<uint16_t*>(p.out),
                    p.d_model, 0, p.T, p.d_model, static_cast<int>(mid_w), 1);
    return hipGetLastError();
  }
}

}  // namespace lca
