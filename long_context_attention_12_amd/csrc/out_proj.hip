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
// Flash): the kernel is a weight stream. A workgroup owns 16, 32 or 64 output
// columns (one to four 16-column MFMA tiles); its eight waves take an eighth of K each, load their weight rows with
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

// Batch of U K-steps (32 each) of one wave: B fragments of its NT column
// tiles and A fragments of its MT row tiles, 16 bytes per lane per fragment.
template <int MT, int NT, int U>
struct ProjBatch {
  bf16x8 b[NT][U];
  bf16x8 a[MT][U];
};

template <int MT, int NT, int U>
__device__ __forceinline__ void proj_load(ProjBatch<MT, NT, U>& x, const uint16_t* const (&bp)[NT],
                                          const uint16_t* const (&ap)[MT], int ks) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      x.b[nt][u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(bp[nt] + ks + 32 * u));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      x.a[mt][u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ap[mt] + ks + 32 * u));
  }
}

template <int MT, int NT, int U>
__device__ __forceinline__ void proj_mfma(const ProjBatch<MT, NT, U>& x, f32x4 (&acc)[MT][NT]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.a[mt][u], x.b[nt][u], acc[mt][nt], 0, 0, 0);
}

// C[m, n] = sum_k A[m, k] B[n, k] for the rows [m0, m0 + 16 MT) and columns
// [n0, n0 + 16 NT) of group blockIdx.y. Wave w sums K in [w K/8, (w + 1) K/8)
// in batches of U steps, the next batch's loads in flight while the current
// one feeds the MFMAs; the eight partial tiles add in a fixed order. Every
// A fragment a wave loads feeds NT column tiles, so the rows' activations are
// read from the L2 once per 16 NT columns. Each column's sum is the same MFMA
// chain whatever NT is, so its bits do not depend on NT.
template <int MT, int NT>
__global__ __launch_bounds__(kProjThreads) void proj_nt_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                               int64_t a_group, const uint16_t* __restrict__ Bw,
                                                               int64_t b_group, uint16_t* __restrict__ C,
                                                               int64_t ldc, int64_t c_group, int M, int K) {
  // two batches of U steps in flight (registers for 2+ workgroups per CU)
  constexpr int U = MT + NT <= 3 ? 4 : 2;
  __shared__ float red[kProjWaves][MT * NT * 256];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int gi = blockIdx.y;
  const int n0 = blockIdx.x * 16 * NT;
  const int m0 = blockIdx.z * 16 * MT;
  const int kq = K / kProjWaves, k0 = wid * kq;
  const int kk = 8 * (lane >> 4);                  // the lane's 8 K values in each step of 32
  // lane l: columns n0 + 16 nt + l % 16 of B, rows m0 + 16 mt + l % 16 of A
  // (rows past M read row M - 1, and their results are dropped)
  const uint16_t* bp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    bp[nt] = Bw + gi * b_group + static_cast<int64_t>(n0 + 16 * nt + (lane & 15)) * K + k0 + kk;
  const uint16_t* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = m0 + 16 * mt + (lane & 15);
    if (r > M - 1) r = M - 1;
    ap[mt] = A + gi * a_group + static_cast<int64_t>(r) * lda + k0 + kk;
  }
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nb = kq / (32 * U);                    // whole batches
  ProjBatch<MT, NT, U> x0, x1;
  if (nb > 0) proj_load<MT, NT, U>(x0, bp, ap, 0);
  for (int j = 0; j < nb; j += 2) {
    if (j + 1 < nb) proj_load<MT, NT, U>(x1, bp, ap, (j + 1) * 32 * U);
    proj_mfma<MT, NT, U>(x0, acc);
    if (j + 2 < nb) proj_load<MT, NT, U>(x0, bp, ap, (j + 2) * 32 * U);
    if (j + 1 < nb) proj_mfma<MT, NT, U>(x1, acc);
  }
  for (int ks = nb * 32 * U; ks < kq; ks += 32) {
    bf16x8 b1[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) b1[nt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(bp[nt] + ks));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ap[mt] + ks));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1[nt], acc[mt][nt], 0, 0, 0);
    }
  }
  // lane l holds C rows 4 (l / 16) + i, column l % 16 of each tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wid][(mt * NT + nt) * 256 + lane * 4 + i] = acc[mt][nt][i];
  __syncthreads();
  uint16_t* c = C + gi * c_group;
  for (int e = threadIdx.x; e < MT * NT * 256; e += kProjThreads) {
    const int tile = e >> 8, el = e & 255;
    const int mt = tile / NT, nt = tile % NT;
    const int row = 4 * ((el >> 2) >> 4) + (el & 3), col = (el >> 2) & 15;
    float v = red[0][e];
#pragma unroll
    for (int w = 1; w < kProjWaves; ++w) v += red[w][e];
    const int m = m0 + 16 * mt + row;
    if (m < M) c[static_cast<int64_t>(m) * ldc + n0 + 16 * nt + col] = f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// Many rows (prefill): a 256 x 128 block of C per workgroup, each of its four
// waves a 128 x 64 quarter (8 x 4 MFMA tiles), operand tiles of 32 K values
// copied HBM -> LDS by the load units into a ring of three stages. Every
// fragment read from LDS feeds four (A) or eight (B) MFMAs: 12 KB of LDS reads
// per wave per 32 MFMAs, under the LDS rate at one workgroup per CU.
// The sum over K keeps the arithmetic of proj_nt_kernel: K in eight slices,
// each an MFMA chain in K order from zero, the slices added in order. So a
// row's result does not depend on which kernel, or how many rows, computed it.
// LDS rows are 64 bytes (4 slots of 16 B); slot c of row r sits at physical
// slot c ^ ((r >> 2) & 3), which spreads a fragment read (16 rows, one slot)
// over all 64 banks.
// ---------------------------------------------------------------------------
constexpr int kGemmBM = 256, kGemmBN = 128, kGemmBK = 32, kGemmStages = 4;
constexpr int kGemmThreads = 256;

__global__ __launch_bounds__(kGemmThreads) void gemm_nt_tiled_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t a_group, const uint16_t* __restrict__ Bw, int64_t b_group,
    uint16_t* __restrict__ C, int64_t ldc, int64_t c_group, int M, int K, int nb, int mb, int groups) {
  constexpr int AT = kGemmBM * kGemmBK, BT = kGemmBN * kGemmBK;   // elements per stage
  __shared__ __attribute__((aligned(1024))) uint16_t Ls[kGemmStages][AT + BT];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  // XCD-aware order: the hardware hands consecutive blocks to the 8 XCDs in
  // turn; block L is the (L / 8)-th of XCD L % 8, and an XCD's blocks take the
  // nb column blocks of one (group, row block) pair back to back, so the
  // pair's A rows come from HBM once and then from that XCD's L2. Pairs are
  // padded to a multiple of 8.
  const int xcd = static_cast<int>(blockIdx.x) & 7, jx = static_cast<int>(blockIdx.x) >> 3;
  const int pair = (jx / nb) * 8 + xcd;
  if (pair >= groups * mb) return;
  const int gi = pair / mb;
  const int n0 = (jx % nb) * kGemmBN, m0 = (pair % mb) * kGemmBM;
  const int wm = wid >> 1, wn = wid & 1;           // wave quarter: rows 128 wm, columns 64 wn
  const uint16_t* Ag = A + gi * a_group;
  const uint16_t* Bg = Bw + gi * b_group;
  // copies: instruction j of a stage fills LDS bytes [1 KB j, 1 KB j + 1 KB) =
  // 16 rows; lane l -> row 16 j' + l / 4 of its operand, physical slot l % 4
  const int crow = lane >> 2, cslot = lane & 3;
  auto issue = [&](int kt, int st) {
    const int k0 = kt * kGemmBK;
    const uint32_t base = lds_address(&Ls[st][0]);
#pragma unroll
    for (int q = 0; q < 6; ++q) {                  // 24 copies per stage, 6 per wave
      const int j = wid * 6 + q;                   // 0..15: A rows 16 j ..; 16..23: B rows 16 (j - 16) ..
      const bool isA = j < 16;
      const int row = (isA ? 16 * j : 16 * (j - 16)) + crow;
      const int ls = cslot ^ ((row >> 2) & 3);     // logical slot stored at this physical slot
      const uint16_t* src;
      if (isA) {
        int r = m0 + row;
        if (r > M - 1) r = M - 1;                  // rows past M: any valid row, results dropped
        src = Ag + static_cast<int64_t>(r) * lda + k0 + 8 * ls;
      } else {
        src = Bg + static_cast<int64_t>(n0 + row) * K + k0 + 8 * ls;
      }
      lds_copy16(src, base + 1024u * static_cast<uint32_t>(j));
    }
  };
  const int nk = K / kGemmBK, per_slice = nk / 8;  // stages per K slice (K % 256 == 0)
  f32x4 acc[8][4], tot[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = tot[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Stages: three copies in flight ahead of the one being summed; the
  // fragments of stage kt + 1 are read from LDS while stage kt's MFMAs run.
#pragma unroll
  for (int s0 = 0; s0 < kGemmStages - 1; ++s0)
    if (s0 < nk) issue(s0, s0);
  // fragment byte offsets in a stage: A tile rows 128 wm + 16 mt + r16, B rows 64 wn + 16 nt + r16
  const int ra = 128 * wm + r16, rb = 64 * wn + r16;
  struct Frags {
    bf16x8 a[8], b[4];
  };
  auto read_frags = [&](int kt, Frags& f) {
    const char* st = reinterpret_cast<const char*>(&Ls[kt % kGemmStages][0]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int r = ra + 16 * mt;
      f.a[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(st + r * 64 + 16 * (g ^ ((r >> 2) & 3))));
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int r = rb + 16 * nt;
      f.b[nt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(st + 2 * AT + r * 64 + 16 * (g ^ ((r >> 2) & 3))));
    }
  };
  // Stage s landed for every wave: this wave's 6 copies of it are done (the
  // stage after it, the only later one issued yet, may stay in flight), then
  // a bare barrier (a fence would drain that stage too). Every wave is then
  // also past the MFMAs of stage s - 2, whose slot the next copies overwrite.
  auto land = [&](int st) {
    if (st + 1 < nk) wait_vmcnt<6>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  auto step = [&](int kt, const Frags& cur, Frags& nxt) {
    if (kt + 1 < nk) {
      land(kt + 1);
      if (kt + 3 < nk) issue(kt + 3, (kt + 3) % kGemmStages);
      read_frags(kt + 1, nxt);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[mt], cur.b[nt], acc[mt][nt], 0, 0, 0);
    if ((kt + 1) % per_slice == 0) {               // a K slice ends: add it, restart the chain
      const bool first = kt + 1 == per_slice;      // the first slice is taken as it is (as red[0])
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          tot[mt][nt] = first ? acc[mt][nt] : tot[mt][nt] + acc[mt][nt];
          acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
  };
  Frags f0, f1;
  if (nk > 0) {
    if (nk > 2) wait_vmcnt<12>();
    else if (nk > 1) wait_vmcnt<6>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    read_frags(0, f0);
  }
  for (int kt = 0; kt < nk; kt += 2) {             // two steps per pass: the fragment sets swap roles
    step(kt, f0, f1);
    if (kt + 1 < nk) step(kt + 1, f1, f0);
  }
  // lane (g, r16) holds C rows 4 g + i, column r16 of each tile
  uint16_t* Cg = C + gi * c_group;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 128 * wm + 16 * mt + 4 * g + i;
      if (m < M) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          Cg[static_cast<int64_t>(m) * ldc + n0 + 64 * wn + 16 * nt + r16] = f32_to_bf16(tot[mt][nt][i]);
      }
    }
}

template <int MT, int NT>
void launch_proj_nt(LaunchScope& sc, const uint16_t* A, int64_t lda, int64_t a_group, const uint16_t* Bw,
                    int64_t b_group, uint16_t* C, int64_t ldc, int64_t c_group, int M, int N, int K, int groups) {
  const dim3 grid(N / (16 * NT), groups, (M + 16 * MT - 1) / (16 * MT));
  sc.launch(proj_nt_kernel<MT, NT>, grid, dim3(kProjThreads), 0, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, K);
}

// Column tiles per workgroup: the most (up to four) that still leave the
// launch at least kProjMinWG workgroups. More columns per workgroup read the
// activations from the L2 fewer times (Pro decode, 64 rows: the first stage
// 74 -> 36 us with four tiles, the second 144 -> 91 us with two); fewer than
// about 200 workgroups leave CUs idle (Flash second stage at 16 rows: 17 us with
// one tile and 256 workgroups, 24 us with two and 128).
constexpr int64_t kProjMinWG = 200;

template <int MT>
void launch_proj(LaunchScope& sc, const uint16_t* A, int64_t lda, int64_t a_group, const uint16_t* Bw,
                 int64_t b_group, uint16_t* C, int64_t ldc, int64_t c_group, int M, int N, int K, int groups) {
  const int64_t rb = (M + 16 * MT - 1) / (16 * MT);
  auto fits = [&](int nt) { return N % (16 * nt) == 0 && static_cast<int64_t>(N / (16 * nt)) * groups * rb >= kProjMinWG; };
  const int nt = fits(4) ? 4 : fits(2) ? 2 : 1;
  if (nt == 4) launch_proj_nt<MT, 4>(sc, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, N, K, groups);
  else if (nt == 2) launch_proj_nt<MT, 2>(sc, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, N, K, groups);
  else launch_proj_nt<MT, 1>(sc, A, lda, a_group, Bw, b_group, C, ldc, c_group, M, N, K, groups);
}

void launch_proj_any(LaunchScope& sc, const uint16_t* A, int64_t lda, int64_t a_group, const uint16_t* Bw,
                     int64_t b_group, uint16_t* C, int64_t ldc, int64_t c_group, int M, int N, int K, int groups) {
  // many rows: the tiled kernel (same arithmetic)
  if (M >= kGemmBM && N % kGemmBN == 0 && K % (8 * kGemmBK) == 0) {
    const int nb = N / kGemmBN, mb = (M + kGemmBM - 1) / kGemmBM;
    const int64_t pairs = (static_cast<int64_t>(groups) * mb + 7) / 8 * 8;
    sc.launch(gemm_nt_tiled_kernel, dim3(static_cast<uint32_t>(pairs * nb)), dim3(kGemmThreads), 0, A, lda, a_group,
              Bw, b_group, C, ldc, c_group, M, K, nb, mb, groups);
    return;
  }
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
