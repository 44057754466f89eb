// index_topk.hip — Lightning Indexer scores of every visible compressed entry
// and top-k selection.
//
// [Qiaomu] 混合注意力机制: cheap indexer queries score every compressed block and
// only the top-k are kept; [kwkr] §3.1: CSA runs DeepSeek Sparse Attention on
// the compressed entries, whose indexer score is s_j = sum_h w_h relu(q_h.k_j);
// [Qiaomu] FP4量化感知训练 and [kwkr] §4.4: scores rounded to BF16 before top-k.
//
// Scoring streams the indexer keys once from HBM (the bulk of a CSA decode
// step's bytes). bf16 keys go through v_mfma_f32_16x16x32_bf16 with the 16
// M-rows holding (16 / H_I) queries x H_I heads, so each lane's 4 accumulator
// registers carry the H_I head dots of one (query, key) pair when H_I = 4 and
// the ReLU-weighted head sum needs no cross-lane traffic. Scores go to the
// workspace (float32, 4 B per entry: small next to the 256 B key row).
//
// Selection is an MSB-first radix select per query in one 1024-thread
// workgroup (LDS histograms of 12/10/10-bit digits, 12/4 bits for bf16
// scores). Up to 32768 scores stay in registers (32 consecutive scores per
// thread, fetched once as coalesced 1 KB rows and passed through LDS into each
// thread's run); longer lists are processed in rounds of 32768. Short lists
// first bound the k-th score by thread (or run-of-8) maxima and take only the
// candidates above the bound through the digits. An order-preserving
// compaction follows: output indices come out in increasing order and ties at
// the threshold go to the lowest indices, so the result is deterministic.
#include <type_traits>

#include "lca_device.h"
#include "lca_internal.h"
#include "../../include/lca.h"

namespace lca {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kKeysPerWave = 32;   // 2 MFMA key groups, all loads issued together (many short waves stream best)
constexpr int kKeysPerWG = 4 * kKeysPerWave;

// An MFMA reads its operands only from lanes enabled in EXEC. Its result here
// feeds lane-conditional stores, and the compiler may otherwise sink the MFMA
// into that divergent branch; the empty asm makes the accumulator live at a
// point every lane reaches, so the MFMA runs with the full wave.
__device__ __forceinline__ void pin_uniform(f32x4& acc) { asm volatile("" : "+v"(acc)); }

// ReLU as the median of (x, 0, FLT_MAX), and the maximum of two values as the
// median of (a, b, FLT_MAX): one instruction each, equal to fmaxf for every
// argument below +inf (+inf becomes FLT_MAX). fmaxf itself, on a value read
// from an accumulator or a DPP move, first quiets it with an extra max.
__device__ __forceinline__ float relu1(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.40282347e38f); }
__device__ __forceinline__ float max1(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, 3.40282347e38f); }

// Rank of this lane's set bit among the set bits of its 16-lane row in the
// wave mask (bit: this lane's own bit), and the row's count of set bits, from
// the wave prefix count (mbcnt) and two row broadcasts.
__device__ __forceinline__ uint32_t row_rank(uint64_t mask, bool bit, uint32_t* row_count) {
  const uint32_t pm = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
  const uint32_t first = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(pm), 0x150, 0xf, 0xf, false));          // row_newbcast:0
  const uint32_t last = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(pm + bit), 0x15F, 0xf, 0xf, false));    // row_newbcast:15
  *row_count = last - first;
  return pm - first;
}

// The weighted head terms of one accumulator quad (rows 4g .. 4g + 3):
// p01 = fma(w1, relu(a1), w0 relu(a0)), p23 = fma(w3, relu(a3), w2 relu(a2)).
// Every scoring kernel forms its head sums from these in this order, written
// out so that the compiler's contraction choices cannot differ between them.
__device__ __forceinline__ void head_pairs(const f32x4& acc, const float (&wv)[4], float& p01, float& p23) {
  p01 = __builtin_fmaf(wv[1], relu1(acc[1]), wv[0] * relu1(acc[0]));
  p23 = __builtin_fmaf(wv[3], relu1(acc[3]), wv[2] * relu1(acc[2]));
}

// Order-preserving key: larger score -> larger unsigned key; -0 folds into +0.
// Key 0 never comes from a real number (it would be a NaN pattern), so it
// marks "no element" below.
__device__ __forceinline__ uint32_t score_key(float v, bool key16) {
  if (v == 0.f) v = 0.f;
  const uint32_t u = __float_as_uint(v);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key16 ? (k >> 16) : k;
}

// Scores of key j from one 16 x 16 MFMA tile: accumulator row 4g + i is the
// dot of (query tq0 + (4g+i) / HI, head (4g+i) % HI) with key j. ReLU, the
// head weights and the head sum are folded here, in the same order for every
// operand type: ((p0 + p1) + (p2 + p3)), then across lane groups for HI >= 8.
// Each stored score also enters gm[slot], the running maximum of the query
// slot the lane owns (see emit_group_max), for the top-k's group bound.
template <int HI>
__device__ __forceinline__ void emit_scores(const f32x4& acc, const float (&wv)[4], const int64_t (&nvq)[4], int g,
                                            int tq0, int t_off, int t_end, int64_t j, float* srow, int64_t ld,
                                            bool round_bf16, float (&gm)[4]) {
  if constexpr (HI == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qt = tq0 + 4 * g + i;
      const float pi = wv[i] * relu1(acc[i]);
      const float v = round_bf16 ? bf16_round(pi) : pi;
      if (qt < t_end && j < nvq[i]) {
        srow[(qt - t_off) * ld + j] = v;
        gm[i] = fmaxf(gm[i], v);
      }
    }
  } else if constexpr (HI == 2) {
    float pr[2];
    head_pairs(acc, wv, pr[0], pr[1]);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int qt = tq0 + 2 * g + p;
      const float sc = pr[p];
      const float v = round_bf16 ? bf16_round(sc) : sc;
      if (qt < t_end && j < nvq[2 * p]) {
        srow[(qt - t_off) * ld + j] = v;
        gm[p] = fmaxf(gm[p], v);
      }
    }
  } else {
    float p01, p23;
    head_pairs(acc, wv, p01, p23);
    float sc = p01 + p23;
    if constexpr (HI >= 8) sc += __shfl_xor(sc, 16, 64);
    if constexpr (HI >= 16) sc += __shfl_xor(sc, 32, 64);
    const int qt = tq0 + (4 * g) / HI;
    const bool writer = (g % (HI / 4 > 0 ? HI / 4 : 1)) == 0;
    const float v = round_bf16 ? bf16_round(sc) : sc;
    if (writer && qt < t_end && j < nvq[0]) {
      srow[(qt - t_off) * ld + j] = v;
      gm[0] = fmaxf(gm[0], v);
    }
  }
}

// Group maxima for the top-k (one float per query and group of kGroup = 16
// keys, the 16 key lanes r16 of one MFMA tile): the largest stored score of
// the group's visible keys. Reduces the lane's gm slots over those 16 lanes;
// lane r16 == 0 writes the slots of queries that see the group's first key.
constexpr int kGroup = 16;
template <int HI>
__device__ __forceinline__ void emit_group_max(float (&gm)[4], int g, int r16, int tq0, int t_off, int t_end,
                                               const int64_t (&nvq)[4], int64_t grp, float* gmrow, int64_t ldg) {
  constexpr int NS = HI == 1 ? 4 : (HI == 2 ? 2 : 1);
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    float v = gm[sl];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int qt = HI == 1 ? tq0 + 4 * g + sl : (HI == 2 ? tq0 + 2 * g + sl : tq0 + (4 * g) / HI);
    const int64_t nv = HI == 1 ? nvq[sl] : (HI == 2 ? nvq[2 * sl] : nvq[0]);
    const bool writer = HI <= 4 || (g % (HI / 4 > 0 ? HI / 4 : 1)) == 0;
    if (r16 == 0 && writer && qt < t_end && grp * kGroup < nv) gmrow[(qt - t_off) * ldg + grp] = v;
    gm[sl] = -INFINITY;
  }
}

// Side outputs of the scoring kernels for the chunked top-k: group maxima
// [B, Tc, ldg] (gmax == nullptr: not produced). The tiled kernel's candidate
// pass instead compares every score with its row's bound (bound[2 r]) and
// writes, per row and key range, the candidates above it (key, index) at
// slots [0, per) and the indices of those equal to it at [per, 2 per), each
// in index order, with (above << 16) | equal in cnt[r, range].
struct SelAux {
  float* gmax;
  int64_t ldg;
  const uint32_t* bound;
  uint32_t* ckey;
  int32_t* cidx;
  uint32_t* cnt;
  int nchs;
  int64_t capc;
  const uint32_t* lim;     // per row: keys at or past it hold no candidate (bound kernel)
};
constexpr int kTiledScores = 0;     // tiled kernel: store every score (and group maxima if asked)
constexpr int kTiledMaxima = 1;     // group maxima only
constexpr int kTiledCands = 2;      // candidates against the row bound only

// As emit_scores, but into the wave's LDS staging block (row = query of the
// wave, column = key of the tile) instead of the score rows: the block is then
// written out as 256-byte row segments (see index_score_tiled_kernel). HI >= 2.
constexpr int kStageStride = 80;     // floats per staged query row (64 keys + bank shift)
template <int HI>
__device__ __forceinline__ void stage_scores(const f32x4& acc, const float (&wv)[4], int g, int q0, int col,
                                             float* stage, bool round_bf16) {
  float pr[2];
  head_pairs(acc, wv, pr[0], pr[1]);
  if constexpr (HI == 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float sc = pr[p];
      stage[(q0 + 2 * g + p) * kStageStride + col] = round_bf16 ? bf16_round(sc) : sc;
    }
  } else {
    float sc = pr[0] + pr[1];
    if constexpr (HI >= 8) sc += __shfl_xor(sc, 16, 64);
    if constexpr (HI >= 16) sc += __shfl_xor(sc, 32, 64);
    const bool writer = (g % (HI / 4 > 0 ? HI / 4 : 1)) == 0;
    if (writer) stage[(q0 + (4 * g) / HI) * kStageStride + col] = round_bf16 ? bf16_round(sc) : sc;
  }
}

// ---------------------------------------------------------------------------
// bf16 scoring with MFMA 16x16x32 (A = 16 indexer query-head rows, B = 16 keys)
// ---------------------------------------------------------------------------
template <int HI, int DI>
__global__ __launch_bounds__(kScoreThreads) void index_score_bf16_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const uint16_t* __restrict__ kI,
    float* __restrict__ scores, int64_t ld, int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0,
    const int64_t* __restrict__ q_pos, int m, bool round_bf16, SelAux aux) {
  constexpr int QPB = 16 / HI;       // queries per M tile
  constexpr int KS = DI / 32;        // K steps
  constexpr int UNR = kKeysPerWave / 16;
  static_assert(kGroup == 16, "a group is the 16 keys of one MFMA tile");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int b = blockIdx.z;
  q_pos0 = seq_pos(q_pos, q_pos0, b);                // this sequence's position
  const int tq0 = t_off + blockIdx.y * QPB;          // first query of this M tile
  const int t_end = min(Tq, t_off + Tc);             // queries of this chunk only
  const int tq_last = min(tq0 + QPB, t_end) - 1;
  int64_t nv_max = n_visible(q_pos0 + tq_last, m);
  if (nv_max > N_cap) nv_max = N_cap;
  const int64_t key0 = static_cast<int64_t>(blockIdx.x) * kKeysPerWG + wid * kKeysPerWave;
  if (key0 >= nv_max) return;

  // keys first: every load of this wave is in flight before anything waits
  const uint16_t* kb = kI + static_cast<int64_t>(b) * N_cap * DI;
  uint4 kv[UNR][KS];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    int64_t j = key0 + 16 * u + r16;
    if (j >= nv_max) j = nv_max - 1;               // stay in bounds; result discarded
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[u][s] = *reinterpret_cast<const uint4*>(kb + j * DI + 32 * s + 8 * g);
  }
  // A operand: row r16 -> (query tq0 + r16 / HI, head r16 % HI); K chunk 8g..8g+7
  bf16x8 aq[KS];
  {
    const int qt = tq0 + r16 / HI, h = r16 % HI;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qt < t_end) v = *reinterpret_cast<const uint4*>(qI + ((static_cast<int64_t>(b) * Tq + qt) * HI + h) * DI + 32 * s + 8 * g);
      aq[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // per-accumulator-row weights: row 4g+i -> (query (4g+i)/HI, head (4g+i)%HI)
  float wv[4];
  int64_t nvq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i, qt = tq0 + row / HI, h = row % HI;
    wv[i] = qt < t_end ? w[(static_cast<int64_t>(b) * Tq + qt) * HI + h] : 0.f;
    nvq[i] = qt < t_end ? n_visible(q_pos0 + qt, m) : 0;
  }
  float gm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[s], __builtin_bit_cast(bf16x8, kv[u][s]), acc, 0, 0, 0);
    pin_uniform(acc);
    emit_scores<HI>(acc, wv, nvq, g, tq0, t_off, t_end, key0 + 16 * u + r16,
                    scores + static_cast<int64_t>(b) * Tc * ld, ld, round_bf16, gm);
    if (aux.gmax)
      emit_group_max<HI>(gm, g, r16, tq0, t_off, t_end, nvq, (key0 + 16 * u) / kGroup,
                         aux.gmax + static_cast<int64_t>(b) * Tc * aux.ldg, aux.ldg);
  }
}

// ---------------------------------------------------------------------------
// 32 or 64 indexer heads in bf16: one query's heads fill MT = HI / 16 MFMA M
// tiles, and each wave scores 32 keys of one query (grid y = query). Per tile
// the head sum is folded as for 16 heads (head pairs, then across the lane
// groups), and the tiles' sums add in tile order.
// ---------------------------------------------------------------------------
template <int MT, int DI>
__global__ __launch_bounds__(kScoreThreads) void index_score_bf16_wide_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const uint16_t* __restrict__ kI,
    float* __restrict__ scores, int64_t ld, int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0,
    const int64_t* __restrict__ q_pos, int m, bool round_bf16, SelAux aux) {
  constexpr int HI = 16 * MT;
  constexpr int KS = DI / 32;
  constexpr int UNR = kKeysPerWave / 16;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int b = blockIdx.z;
  q_pos0 = seq_pos(q_pos, q_pos0, b);
  const int qt = t_off + blockIdx.y;                 // this workgroup's query
  if (qt >= min(Tq, t_off + Tc)) return;
  int64_t nv = n_visible(q_pos0 + qt, m);
  if (nv > N_cap) nv = N_cap;
  const int64_t key0 = static_cast<int64_t>(blockIdx.x) * kKeysPerWG + wid * kKeysPerWave;
  if (key0 >= nv) return;

  const uint16_t* kb = kI + static_cast<int64_t>(b) * N_cap * DI;
  uint4 kv[UNR][KS];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    int64_t j = key0 + 16 * u + r16;
    if (j >= nv) j = nv - 1;                        // stay in bounds; result discarded
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[u][s] = *reinterpret_cast<const uint4*>(kb + j * DI + 32 * s + 8 * g);
  }
  // A operand of tile mt: row r16 -> head 16 mt + r16; K chunk 8g .. 8g + 7
  const int64_t qrow = (static_cast<int64_t>(b) * Tq + qt) * HI;
  bf16x8 aq[MT][KS];
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      aq[mt][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qI + (qrow + 16 * mt + r16) * DI + 32 * s + 8 * g));
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = w[qrow + 16 * mt + 4 * g + i];   // accumulator row 4g + i
  }
  float* srow = scores + (static_cast<int64_t>(b) * Tc + (qt - t_off)) * ld;
  float* gmrow = aux.gmax ? aux.gmax + (static_cast<int64_t>(b) * Tc + (qt - t_off)) * aux.ldg : nullptr;
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    float sc = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[mt][s], __builtin_bit_cast(bf16x8, kv[u][s]), acc, 0, 0, 0);
      pin_uniform(acc);
      float p01, p23;
      head_pairs(acc, wv[mt], p01, p23);
      float t = p01 + p23;
      t += __shfl_xor(t, 16, 64);
      t += __shfl_xor(t, 32, 64);
      sc = mt == 0 ? t : sc + t;
    }
    const int64_t j = key0 + 16 * u + r16;
    const float v = round_bf16 ? bf16_round(sc) : sc;
    if (g == 0 && j < nv) srow[j] = v;
    if (gmrow) {
      // the group's largest visible score (lanes r16 of one row of 16)
      float x = j < nv ? v : -INFINITY;
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false)));
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false)));
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));
      const int64_t grp = (key0 + 16 * u) / kGroup;
      if (lane == 0 && grp * kGroup < nv) gmrow[grp] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Many queries per call (prefill): the decode kernel above would re-read every
// key once per 16-row query tile. Here a workgroup holds 256 / H_I queries in
// registers (4 waves x 4 M tiles of 16 query-head rows, d_I = 128) and walks a
// range of keys in 64-key tiles. Each tile is copied HBM -> LDS by the load
// units (double-buffered, 16 KB), with the 16-byte slots of each 256-byte key
// row XOR-swizzled by (key & 15), so the B-fragment reads (16 keys at one
// column) hit distinct banks; every tile then feeds 64 MFMAs per wave.
// ---------------------------------------------------------------------------
constexpr int kTileKeys = 64;
constexpr int kTiledMinQueries = 64;

// The scores one lane holds after an M tile's MFMAs (the values stage_scores
// stages, in the same arithmetic order): HI = 2, queries 2 g and 2 g + 1 of
// the tile; HI >= 4, query 4 g / HI, valid in the lanes that hold the head
// sum. Returns the number of slots filled.
template <int HI>
__device__ __forceinline__ int acc_scores(const f32x4& acc, const float (&wv)[4], int g, bool round_bf16,
                                          float (&v)[2]) {
  float pr[2];
  head_pairs(acc, wv, pr[0], pr[1]);
  if constexpr (HI == 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) v[p] = round_bf16 ? bf16_round(pr[p]) : pr[p];
    return 2;
  } else {
    float sc = pr[0] + pr[1];
    if constexpr (HI >= 8) sc += __shfl_xor(sc, 16, 64);
    if constexpr (HI >= 16) sc += __shfl_xor(sc, 32, 64);
    v[0] = round_bf16 ? bf16_round(sc) : sc;
    v[1] = v[0];
    (void)g;
    return 1;
  }
}

// R16: scores rounded to bf16 (a template parameter, so that no per-block
// branch splits a tile's straight-line code).
template <int HI, int MODE, bool R16>
__global__ __launch_bounds__(kScoreThreads) void index_score_tiled_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const uint16_t* __restrict__ kI,
    float* __restrict__ scores, int64_t ld, int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0,
    const int64_t* __restrict__ q_pos, int m, int64_t keys_per_wg, SelAux aux, int kc, int nq, int nbatch, int ss) {
  constexpr bool round_bf16 = R16;
  constexpr int DI = 128, KS = DI / 32, MB = 4, NB = kTileKeys / 16, QPB = 16 / HI;
  constexpr int QPW = MB * QPB, QPWG = 4 * QPW;
  constexpr int ROWB = DI * 2;                       // bytes per key row
  constexpr bool kStaged = HI >= 2;                  // HI = 1: 64 queries per wave, stored directly
  static_assert(kStaged || MODE == kTiledScores, "maxima and candidates come from the staged tile");
  constexpr int RPL = kStaged ? QPW / 4 : 1;         // staged rows a lane writes out per tile
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[2][kTileKeys * DI];
  __shared__ __attribute__((aligned(16))) float St[4][kStaged ? QPW * kStageStride : 4];
  __shared__ int64_t nv_tab[QPWG];                   // visible entries of the workgroup's queries
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  // XCD-aware block order: the hardware hands consecutive blocks to the 8
  // XCDs in turn. Block L runs on XCD L % 8 as that XCD's (L / 8)-th block;
  // those take the nq query tiles of one (sequence, key range) pair back to
  // back, so the range's keys are read from HBM once into that XCD's L2 and
  // the other query tiles hit there. Pairs are padded to a multiple of 8.
  const int xcd = static_cast<int>(blockIdx.x) & 7, jx = static_cast<int>(blockIdx.x) >> 3;
  const int krb = (jx / nq) * 8 + xcd;
  if (krb >= kc * nbatch) return;
  const int b = krb / kc, kr = krb - b * kc, qtile = jx % nq;
  q_pos0 = seq_pos(q_pos, q_pos0, b);                // this sequence's position
  const int t_end = min(Tq, t_off + Tc);
  const int tw0 = t_off + qtile * QPWG;
  if (tw0 >= t_end) return;
  // one division per query (not one per lane and slot)
  for (int i = threadIdx.x; i < QPWG; i += kScoreThreads) {
    int64_t nv = tw0 + i < t_end ? n_visible(q_pos0 + tw0 + i, m) : 0;
    nv_tab[i] = nv < N_cap ? nv : N_cap;
  }
  __syncthreads();
  auto nv_of = [&](int qt) { return qt < t_end ? nv_tab[qt - tw0] : int64_t(0); };   // clamped to N_cap
  const int64_t nv_max = nv_of(min(tw0 + QPWG, t_end) - 1);
  const int64_t k_begin = static_cast<int64_t>(kr) * keys_per_wg;
  if (k_begin >= nv_max) return;
  const int64_t k_end = min(k_begin + keys_per_wg, nv_max);
  const int ntiles = static_cast<int>((k_end - k_begin + kTileKeys - 1) / kTileKeys);

  // tile tt -> LDS buffer: 16 copies of 1 KB (4 key rows each), 4 per wave;
  // lane l fills key 4c + l/16 at physical slot l % 16 from logical slot
  // (l % 16) ^ (key & 15); keys past k_end repeat the last key (not scored)
  const char* kb = reinterpret_cast<const char*>(kI) + static_cast<int64_t>(b) * N_cap * ROWB;
  auto issue = [&](int tt, int buf) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int c = wid * 4 + cc;
      const int kl = 4 * c + (lane >> 4);
      int64_t key = k_begin + static_cast<int64_t>(tt) * kTileKeys + kl;
      if (key >= k_end) key = k_end - 1;
      const char* src = kb + key * ROWB + 16 * ((lane & 15) ^ (kl & 15));
      lds_copy16(src, lds_address(&Ks[buf][0]) + c * 1024);
    }
  };
  issue(0, 0);

  // queries of this wave: M tile mb covers queries tq0 + r16 / HI (heads r16 % HI)
  bf16x8 aq[MB][KS];
  float wv[MB][4];
  int64_t nvq[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int tq0 = tw0 + wid * QPW + mb * QPB;
    const int qt = tq0 + r16 / HI, h = r16 % HI;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qt < t_end) v = *reinterpret_cast<const uint4*>(qI + ((static_cast<int64_t>(b) * Tq + qt) * HI + h) * DI + 32 * s + 8 * g);
      aq[mb][s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g + i, q2 = tq0 + row / HI, h2 = row % HI;
      wv[mb][i] = q2 < t_end ? w[(static_cast<int64_t>(b) * Tq + q2) * HI + h2] : 0.f;
      const int64_t nv = nv_of(q2);
      nvq[mb][i] = nv < k_end ? nv : k_end;        // this workgroup scores keys < k_end only
    }
  }
  float* srow = scores + static_cast<int64_t>(b) * Tc * ld;
  const int slot_r = r16;                          // key & 15 of the keys this lane reads
  // the staged rows this lane writes out (row i * 4 + lane / 16 of the wave): visible count
  int64_t nv_l[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) nv_l[i] = nv_of(tw0 + wid * QPW + i * 4 + (lane >> 4));
  // maxima and candidate passes: the (M tile, slot) queries of this lane's
  // accumulators (acc_scores), their visible count past k_begin, row index,
  // whether the lane holds them; for maxima the running maximum and the row's
  // first group slot of this lane, for candidates the bound (as a key, and as
  // a float below which no candidate lies) and the running counts
  int nvl_l[2 * MB];
  int64_t rix_l[2 * MB];
  bool writer_l[2 * MB];
  uint32_t lo_c[2 * MB], run_a[2 * MB], run_e[2 * MB];
  float gm_l[2 * MB], lof_l[2 * MB], lofg_l[2 * MB];
  int limt_l[2 * MB];                                // candidate pass: first tile past the row's index limit
  int64_t gslot_l[2 * MB], cb_l[2 * MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int ci = mb * 2 + sl;
      const int ql = HI == 2 ? 2 * g + sl : (4 * g) / HI;          // query of the M tile
      const int qt = tw0 + wid * QPW + mb * QPB + ql;
      const bool holds = (HI == 2 || sl == 0) && (HI <= 4 || (g % (HI / 4 > 0 ? HI / 4 : 1)) == 0);
      int64_t nv = nv_of(qt);
      if (nv > k_end) nv = k_end;
      nvl_l[ci] = static_cast<int>(nv > k_begin ? nv - k_begin : 0);
      rix_l[ci] = static_cast<int64_t>(b) * Tc + qt - t_off;
      writer_l[ci] = holds && qt < t_end;
      gm_l[ci] = -INFINITY;
      // maxima of every ss-th tile only (sampled pass): tile u ss of the row
      // keeps slots 4 u .. 4 u + 3 (k_begin is a multiple of 64 ss)
      gslot_l[ci] = rix_l[ci] * aux.ldg + k_begin / (kGroup * ss) + (r16 >> 2);
      cb_l[ci] = (rix_l[ci] * aux.nchs + kr) * aux.capc;
      lo_c[ci] = 0;
      lof_l[ci] = INFINITY;
      lofg_l[ci] = INFINITY;
      limt_l[ci] = 0x7fffffff;
      run_a[ci] = run_e[ci] = 0;
    }
  }
  if constexpr (MODE == kTiledCands) {
    // all loads first (clamped rows of non-writers are read and ignored)
    uint32_t lo_raw[2 * MB], lim_raw[2 * MB];
#pragma unroll
    for (int ci = 0; ci < 2 * MB; ++ci) {
      const int64_t rr = writer_l[ci] ? rix_l[ci] : int64_t(0);
      lo_raw[ci] = aux.bound[2 * rr];
      lim_raw[ci] = aux.lim[rr];
    }
#pragma unroll
    for (int ci = 0; ci < 2 * MB; ++ci) {
      if (!writer_l[ci]) continue;
      lo_c[ci] = lo_raw[ci];
      // tiles from limt on start at or past the index limit: no ties with
      // lo there, only scores above it
      const int64_t lrel = static_cast<int64_t>(lim_raw[ci]) - k_begin;
      limt_l[ci] = lrel <= 0 ? 0 : static_cast<int>((lrel + kTileKeys - 1) / kTileKeys);
      // key(x) >= lo implies x >= lof: lof is the bound's own float when
      // that is a normal number, and -FLT_MIN for a bound among the
      // subnormals and zeros (a superset either way, whether or not the
      // comparison flushes subnormals); lofg the same for lo + 1
      auto key_floor = [&](uint32_t key) {
        const uint32_t k32 = round_bf16 ? key << 16 : key;
        if (k32 >= 0x80800000u) return __uint_as_float(k32 & 0x7fffffffu);        // >= +FLT_MIN
        if (k32 >= 0x7f7fffffu) return -1.17549435e-38f;                         // >= key(-FLT_MIN)
        if (k32 > 0x007fffffu) return __uint_as_float(~k32);                      // <= -FLT_MIN
        return -INFINITY;                                                         // key(-inf) and below (no number)
      };
      // (a key above that of +0 is a positive number, whose own float is a
      // superset filter in either subnormal mode: it keeps the exact zeros,
      // a crowd of ties when every head weight is negative, out of the
      // exact comparisons)
      const uint32_t kmax = round_bf16 ? 0xffffu : 0xffffffffu;
      lof_l[ci] = key_floor(lo_raw[ci]);
      const uint32_t g32 = round_bf16 ? (lo_raw[ci] + 1u) << 16 : lo_raw[ci] + 1u;
      lofg_l[ci] = lo_raw[ci] >= kmax         ? INFINITY
                   : g32 >= 0x80000001u      ? __uint_as_float(g32 & 0x7fffffffu)
                                             : key_floor(lo_raw[ci] + 1u);
    }
  }
  // the smallest visible count past k_begin among this wave's queries (its
  // first query): tiles below it need no visibility masks
  int nvl_w = 0;
  {
    const int qw0 = tw0 + wid * QPW;
    int64_t nv = nv_of(qw0);
    if (nv > k_end) nv = k_end;
    nvl_w = __builtin_amdgcn_readfirstlane(static_cast<int>(nv > k_begin ? nv - k_begin : 0));
  }

  // One tile of the maxima or candidate pass; FULL: every key of the tile is
  // visible to every query of the wave (no per-key masks).
  auto sel_tile = [&](int tt, int it, const char* xb, auto full_c) __attribute__((always_inline)) {
    constexpr bool full = decltype(full_c)::value;
    constexpr int NSL = HI == 2 ? 2 : 1;             // query slots per lane (acc_scores)
    float vs[NB][2 * MB];                            // candidate pass: the tile's scores
    uint64_t mk[NB][2 * MB];                         // and which may be candidates
    float lof_t[2 * MB];                             // the float filter: key >= lo, or key > lo past the limit
#pragma unroll
    for (int ci = 0; ci < 2 * MB; ++ci) lof_t[ci] = tt >= limt_l[ci] ? lofg_l[ci] : lof_l[ci];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 acc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint4 kv = *reinterpret_cast<const uint4*>(xb + (nb * 16 + r16) * ROWB + 16 * ((4 * s + g) ^ slot_r));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[mb][s], __builtin_bit_cast(bf16x8, kv), acc[mb], 0, 0, 0);
      }
      // lanes 16 gr .. 16 gr + 15 hold one query's scores of these 16 keys
      const int jl = tt * kTileKeys + nb * 16 + r16;                 // key - k_begin
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        pin_uniform(acc[mb]);
        float v[2];
        acc_scores<HI>(acc[mb], wv[mb], g, round_bf16, v);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          const int ci = mb * 2 + sl;
          const bool vis = full || jl < nvl_l[ci];
          if constexpr (MODE == kTiledMaxima) {
            gm_l[ci] = fmaxf(gm_l[ci], vis ? v[sl] : -INFINITY);     // over the tile's 4 key slabs
          } else {
            vs[nb][ci] = v[sl];
            mk[nb][ci] = __ballot(v[sl] >= lof_t[ci] && vis);
          }
        }
      }
    }
    if constexpr (MODE == kTiledMaxima) {
      // Lane r16 now holds the maximum of keys r16 + 16 s (s < 4) of the
      // tile; a quad of lanes (r16 = 4c .. 4c + 3) then covers the group of
      // keys 4c + i + 16 s. Group c of tile tt takes slot
      // gs = (k_begin + 64 tt) / 16 + c: a partition of the row into groups
      // of 16 keys. The bound reads the slots with key 16 gs visible; the
      // group's first key, 16 gs - 12 c, is then visible too, and the slot
      // is written.
#pragma unroll
      for (int ci = 0; ci < 2 * MB; ++ci) {
        if (ci % 2 >= NSL) continue;
        float x = gm_l[ci];
        x = max1(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));
        x = max1(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));
        const int c = r16 >> 2;
        if ((r16 & 3) == 0 && writer_l[ci] && tt * kTileKeys + 4 * c < nvl_l[ci]) aux.gmax[gslot_l[ci] + 4 * it] = x;
        gm_l[ci] = -INFINITY;
      }
    } else {
      // Candidates are rare: only the blocks with scores at or above the
      // float filter (a superset of those at or above the bound) take the
      // exact key comparisons. Each query's candidates go to its lists in key
      // order (slab by slab, lane by lane).
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int jl = tt * kTileKeys + nb * 16 + r16;
#pragma unroll
        for (int ci = 0; ci < 2 * MB; ++ci) {
          if (ci % 2 >= NSL) continue;
          if (mk[nb][ci] == 0) continue;                             // uniform
          const bool maybe = (mk[nb][ci] >> lane) & 1u;
          const uint32_t kk = score_key(vs[nb][ci], round_bf16);
          const bool is_a = maybe && writer_l[ci] && kk > lo_c[ci];
          const bool is_e = maybe && writer_l[ci] && kk == lo_c[ci] && tt < limt_l[ci];
          const uint64_t ba = __ballot(is_a), be = __ballot(is_e);
          if (ba != 0) {
            uint32_t na;
            const uint32_t pa = run_a[ci] + row_rank(ba, is_a, &na);
            if (is_a) {
              aux.ckey[cb_l[ci] + pa] = kk;
              aux.cidx[cb_l[ci] + pa] = static_cast<int32_t>(k_begin + jl);
            }
            run_a[ci] += na;
          }
          if (be != 0) {
            uint32_t ne;
            const uint32_t pe = run_e[ci] + row_rank(be, is_e, &ne);
            if (is_e) aux.cidx[cb_l[ci] + aux.capc / 2 + pe] = static_cast<int32_t>(k_begin + jl);
            run_e[ci] += ne;
          }
        }
      }
    }
  };

  // the maxima pass takes every ss-th tile (tile 0 of the range is one)
  const int tstep = MODE == kTiledMaxima ? ss : 1;
  for (int tt = 0, it = 0; tt < ntiles; tt += tstep, ++it) {
    // tile tt has landed (every wave waited for its own copies) and every wave
    // is done with the buffer that the next tile overwrites
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (tt + tstep < ntiles) issue(tt + tstep, (it + 1) & 1);
    const char* xb = reinterpret_cast<const char*>(&Ks[it & 1][0]);
    if constexpr (MODE != kTiledScores) {
      if ((tt + 1) * kTileKeys <= nvl_w)                               // uniform
        sel_tile(tt, it, xb, std::true_type{});
      else
        sel_tile(tt, it, xb, std::false_type{});
      continue;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 acc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint4 kv = *reinterpret_cast<const uint4*>(xb + (nb * 16 + r16) * ROWB + 16 * ((4 * s + g) ^ slot_r));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[mb][s], __builtin_bit_cast(bf16x8, kv), acc[mb], 0, 0, 0);
      }
      const int64_t j = k_begin + static_cast<int64_t>(tt) * kTileKeys + nb * 16 + r16;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        pin_uniform(acc[mb]);
        if constexpr (kStaged) {
          stage_scores<HI>(acc[mb], wv[mb], g, mb * QPB, nb * 16 + r16, St[wid], round_bf16);
        } else {
          float gm_unused[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // no group maxima at HI = 1
          emit_scores<HI>(acc[mb], wv[mb], nvq[mb], g, tw0 + wid * QPW + mb * QPB, t_off, t_end, j, srow, ld,
                          round_bf16, gm_unused);
        }
      }
    }
    if constexpr (kStaged && MODE == kTiledScores) {
      // The wave's QPW x 64 tile of scores leaves as 16-byte stores, 16 lanes
      // per 256-byte row segment. Every key of the tile is written: cells past
      // a query's visible count lie inside its row (the stride is a multiple of
      // 64, tiles start at multiples of 64 within this workgroup's key range)
      // and the top-k never reads them. Queries past the chunk are skipped.
      wait_lgkmcnt0();                              // the wave's staging writes have landed
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const int64_t jt0 = k_begin + static_cast<int64_t>(tt) * kTileKeys;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int u = i * 64 + lane, row = u >> 4, c4 = u & 15;
        const int qt = tw0 + wid * QPW + row;
        const int64_t rix = static_cast<int64_t>(b) * Tc + qt - t_off;
        const float4 v = *reinterpret_cast<const float4*>(&St[wid][row * kStageStride + 4 * c4]);
        const int64_t j0 = jt0 + 4 * c4;
        if (qt < t_end) *reinterpret_cast<float4*>(srow + static_cast<int64_t>(qt - t_off) * ld + j0) = v;
        if (aux.gmax) {
          // group maxima: the 4 lanes of a row's 16-key quarter hold its 16
          // cells; cells past the query's visible count do not count
          const int64_t nv = nv_l[i];
          float mx = -INFINITY;
          mx = j0 < nv ? fmaxf(mx, v.x) : mx;
          mx = j0 + 1 < nv ? fmaxf(mx, v.y) : mx;
          mx = j0 + 2 < nv ? fmaxf(mx, v.z) : mx;
          mx = j0 + 3 < nv ? fmaxf(mx, v.w) : mx;
#pragma unroll
          for (int o = 1; o < 4; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
          const int64_t grp = jt0 / kGroup + (c4 >> 2);
          if ((c4 & 3) == 0 && qt < t_end && grp * kGroup < nv) aux.gmax[rix * aux.ldg + grp] = mx;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // reads done before the next tile's staging
    }
  }
  if constexpr (MODE == kTiledCands) {
#pragma unroll
    for (int ci = 0; ci < 2 * MB; ++ci)
      if (r16 == 0 && writer_l[ci]) aux.cnt[rix_l[ci] * aux.nchs + kr] = (run_a[ci] << 16) | run_e[ci];
  }
}

// ---------------------------------------------------------------------------
// MXFP4 scoring (d_I = 128) with the scaled MFMA 16x16x128 (f8f6f4, e2m1
// operands): lane l holds row / key l % 16 and the 32-element block l / 16 of
// it (16 packed bytes, low nibble first) together with that block's E8M0
// scale, so one MFMA forms the whole 128-channel dot of 16 query-head rows with
// 16 keys, each block scaled by 2^(e_q - 127) * 2^(e_k - 127). Products of
// e2m1 values and power-of-two scales are exact; the MFMA accumulates in fp32.
// A key costs 64 + 4 bytes; a wave keeps 256 keys (17 KiB) in flight.
// ---------------------------------------------------------------------------
constexpr int kFp4KeysPerWave = 256;
constexpr int kFp4KeysPerWG = 4 * kFp4KeysPerWave;

template <int HI>
__global__ __launch_bounds__(kScoreThreads) void index_score_fp4_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale, float* __restrict__ scores, int64_t ld,
    int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0, const int64_t* __restrict__ q_pos, int m,
    bool round_bf16, SelAux aux) {
  constexpr int QPB = 16 / HI;
  constexpr int UNR = kFp4KeysPerWave / 16;
  constexpr int ROW = 64;                          // packed bytes per 128-channel row
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int b = blockIdx.z;
  q_pos0 = seq_pos(q_pos, q_pos0, b);                // this sequence's position
  const int tq0 = t_off + blockIdx.y * QPB;
  const int t_end = min(Tq, t_off + Tc);
  const int tq_last = min(tq0 + QPB, t_end) - 1;
  int64_t nv_max = n_visible(q_pos0 + tq_last, m);
  if (nv_max > N_cap) nv_max = N_cap;
  const int64_t key0 = static_cast<int64_t>(blockIdx.x) * kFp4KeysPerWG + wid * kFp4KeysPerWave;
  if (key0 >= nv_max) return;

  const uint8_t* kb = kI + static_cast<int64_t>(b) * N_cap * ROW;
  const uint32_t* ksb = reinterpret_cast<const uint32_t*>(kI_scale) + static_cast<int64_t>(b) * N_cap;
  uint4 kc[UNR];
  uint32_t ks[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    int64_t j = key0 + 16 * u + r16;
    if (j >= nv_max) j = nv_max - 1;               // stay in bounds; result discarded
    kc[u] = *reinterpret_cast<const uint4*>(kb + j * ROW + 16 * g);
    ks[u] = ksb[j];                                 // the key's four block scales
  }
  uint4 qa = make_uint4(0, 0, 0, 0);
  int qs = 0;
  {
    const int qt = tq0 + r16 / HI, h = r16 % HI;
    if (qt < t_end) {
      const int64_t qrow = (static_cast<int64_t>(b) * Tq + qt) * HI + h;
      qa = *reinterpret_cast<const uint4*>(qI + qrow * ROW + 16 * g);
      qs = qI_scale[qrow * 4 + g];
    }
  }
  float wv[4];
  int64_t nvq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i, qt = tq0 + row / HI, h = row % HI;
    wv[i] = qt < t_end ? w[(static_cast<int64_t>(b) * Tq + qt) * HI + h] : 0.f;
    nvq[i] = qt < t_end ? n_visible(q_pos0 + qt, m) : 0;
  }
  const i32x8 A = {static_cast<int>(qa.x), static_cast<int>(qa.y), static_cast<int>(qa.z), static_cast<int>(qa.w),
                   0, 0, 0, 0};
  float gm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const i32x8 Bk = {static_cast<int>(kc[u].x), static_cast<int>(kc[u].y), static_cast<int>(kc[u].z),
                      static_cast<int>(kc[u].w), 0, 0, 0, 0};
    const int sb = static_cast<int>((ks[u] >> (8 * g)) & 0xffu);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bk, acc, 4, 4, 0, qs, 0, sb);
    pin_uniform(acc);
    emit_scores<HI>(acc, wv, nvq, g, tq0, t_off, t_end, key0 + 16 * u + r16,
                    scores + static_cast<int64_t>(b) * Tc * ld, ld, round_bf16, gm);
    if (aux.gmax)
      emit_group_max<HI>(gm, g, r16, tq0, t_off, t_end, nvq, (key0 + 16 * u) / kGroup,
                         aux.gmax + static_cast<int64_t>(b) * Tc * aux.ldg, aux.ldg);
  }
}

// 32 or 64 heads in MXFP4: as index_score_bf16_wide_kernel (one query per
// grid row, its heads over MT M tiles, tile sums added in order), one scaled
// MFMA per tile and key group.
template <int MT>
__global__ __launch_bounds__(kScoreThreads) void index_score_fp4_wide_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale, float* __restrict__ scores, int64_t ld,
    int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0, const int64_t* __restrict__ q_pos, int m,
    bool round_bf16, SelAux aux) {
  constexpr int HI = 16 * MT;
  constexpr int UNR = kFp4KeysPerWave / 16;
  constexpr int ROW = 64;                          // packed bytes per 128-channel row
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int b = blockIdx.z;
  q_pos0 = seq_pos(q_pos, q_pos0, b);
  const int qt = t_off + blockIdx.y;
  if (qt >= min(Tq, t_off + Tc)) return;
  int64_t nv = n_visible(q_pos0 + qt, m);
  if (nv > N_cap) nv = N_cap;
  const int64_t key0 = static_cast<int64_t>(blockIdx.x) * kFp4KeysPerWG + wid * kFp4KeysPerWave;
  if (key0 >= nv) return;

  const uint8_t* kb = kI + static_cast<int64_t>(b) * N_cap * ROW;
  const uint32_t* ksb = reinterpret_cast<const uint32_t*>(kI_scale) + static_cast<int64_t>(b) * N_cap;
  uint4 kc[UNR];
  uint32_t ks[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    int64_t j = key0 + 16 * u + r16;
    if (j >= nv) j = nv - 1;                        // stay in bounds; result discarded
    kc[u] = *reinterpret_cast<const uint4*>(kb + j * ROW + 16 * g);
    ks[u] = ksb[j];
  }
  const int64_t qrow = (static_cast<int64_t>(b) * Tq + qt) * HI;
  i32x8 A[MT];
  int qs[MT];
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t r = qrow + 16 * mt + r16;         // tile row r16: head 16 mt + r16
    const uint4 qa = *reinterpret_cast<const uint4*>(qI + r * ROW + 16 * g);
    A[mt] = i32x8{static_cast<int>(qa.x), static_cast<int>(qa.y), static_cast<int>(qa.z), static_cast<int>(qa.w),
                  0, 0, 0, 0};
    qs[mt] = qI_scale[r * 4 + g];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = w[qrow + 16 * mt + 4 * g + i];
  }
  float* srow = scores + (static_cast<int64_t>(b) * Tc + (qt - t_off)) * ld;
  float* gmrow = aux.gmax ? aux.gmax + (static_cast<int64_t>(b) * Tc + (qt - t_off)) * aux.ldg : nullptr;
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const i32x8 Bk = {static_cast<int>(kc[u].x), static_cast<int>(kc[u].y), static_cast<int>(kc[u].z),
                      static_cast<int>(kc[u].w), 0, 0, 0, 0};
    const int sb = static_cast<int>((ks[u] >> (8 * g)) & 0xffu);
    float sc = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[mt], Bk, acc, 4, 4, 0, qs[mt], 0, sb);
      pin_uniform(acc);
      float p01, p23;
      head_pairs(acc, wv[mt], p01, p23);
      float t = p01 + p23;
      t += __shfl_xor(t, 16, 64);
      t += __shfl_xor(t, 32, 64);
      sc = mt == 0 ? t : sc + t;
    }
    const int64_t j = key0 + 16 * u + r16;
    const float v = round_bf16 ? bf16_round(sc) : sc;
    if (g == 0 && j < nv) srow[j] = v;
    if (gmrow) {
      float x = j < nv ? v : -INFINITY;
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false)));
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false)));
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));
      x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));
      const int64_t grp = (key0 + 16 * u) / kGroup;
      if (lane == 0 && grp * kGroup < nv) gmrow[grp] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// float32 scoring on the vector ALUs (small fp32 layers)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScoreThreads) void index_score_f32_kernel(
    const float* __restrict__ qI, const float* __restrict__ w, const float* __restrict__ kI,
    float* __restrict__ scores, int64_t ld, int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0,
    const int64_t* __restrict__ q_pos, int m, int HI, int DI, bool round_bf16, SelAux aux) {
  extern __shared__ float qs[];                 // [HI * DI + HI]
  const int b = blockIdx.z, tl = blockIdx.y, t = t_off + tl;
  q_pos0 = seq_pos(q_pos, q_pos0, b);           // this sequence's position
  int64_t nv = n_visible(q_pos0 + t, m);
  if (nv > N_cap) nv = N_cap;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kScoreThreads + threadIdx.x;
  if (static_cast<int64_t>(blockIdx.x) * kScoreThreads >= nv) return;
  for (int i = threadIdx.x; i < HI * DI; i += kScoreThreads)
    qs[i] = qI[(static_cast<int64_t>(b) * Tq + t) * HI * DI + i];
  for (int i = threadIdx.x; i < HI; i += kScoreThreads)
    qs[HI * DI + i] = w[(static_cast<int64_t>(b) * Tq + t) * HI + i];
  __syncthreads();
  float sc = -INFINITY;
  if (j < nv) {
    const float* kr = kI + (static_cast<int64_t>(b) * N_cap + j) * DI;
    sc = 0.f;
    for (int h = 0; h < HI; ++h) {
      float dot = 0.f;
      for (int d = 0; d < DI; ++d) dot = fmaf(qs[h * DI + d], kr[d], dot);
      sc += qs[HI * DI + h] * fmaxf(dot, 0.f);
    }
    if (round_bf16) sc = bf16_round(sc);
    scores[(static_cast<int64_t>(b) * Tc + tl) * ld + j] = sc;
  }
  if (aux.gmax) {                               // kGroup consecutive threads: one group
    float mx = sc;
#pragma unroll
    for (int o = 1; o < kGroup; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((threadIdx.x & (kGroup - 1)) == 0 && j < nv) aux.gmax[(static_cast<int64_t>(b) * Tc + tl) * aux.ldg + j / kGroup] = mx;
  }
}

// ---------------------------------------------------------------------------
// Radix select + ordered compaction
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelItems = 32;                   // scores per thread per round
constexpr int kRound = kSelThreads * kSelItems; // scores per round (registers)
constexpr int kMaxBins = 4096;


// Inclusive scan over the 64 lanes of a wave in registers (DPP): shifts of
// 1, 2, 4, 8 lanes inside each 16-lane row, then the row totals carried across
// rows with the row_bcast:15 / row_bcast:31 moves of the gfx9 family.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  int v = static_cast<int>(x);
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return static_cast<uint32_t>(v);
}

// Block-wide exclusive scan of one value per thread (1024 threads, 16 waves).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
  const uint4* w4 = reinterpret_cast<const uint4*>(wsum);
#pragma unroll
  for (int i = 0; i < kSelThreads / 256; ++i) {
    const uint4 q = w4[i];
    const uint32_t e[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      before += 4 * i + c < wid ? e[c] : 0u;
      all += e[c];
    }
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Thread `tid` of round r owns the contiguous indices r*kRound + tid*kSelItems + j.
__device__ __forceinline__ void load_round(const float* __restrict__ s, int64_t n, int64_t base,
                                           bool key16, uint32_t (&key)[kSelItems]) {
  const int64_t i0 = base + static_cast<int64_t>(threadIdx.x) * kSelItems;
  if (i0 + kSelItems <= n) {
    float4 v[kSelItems / 4];
#pragma unroll
    for (int q = 0; q < kSelItems / 4; ++q) v[q] = *reinterpret_cast<const float4*>(s + i0 + 4 * q);
#pragma unroll
    for (int q = 0; q < kSelItems / 4; ++q) {
      key[4 * q + 0] = score_key(v[q].x, key16);
      key[4 * q + 1] = score_key(v[q].y, key16);
      key[4 * q + 2] = score_key(v[q].z, key16);
      key[4 * q + 3] = score_key(v[q].w, key16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) key[j] = i0 + j < n ? score_key(s[i0 + j], key16) : 0u;
  }
}

// One register round in the thread-contiguous layout of load_round, fetched
// coalesced: wave w reads its kSelItems * 64 scores as 1 KB rows (lane l: 16
// bytes at 256 q + 4 l), parks them in its own 8 KB of LDS, and each lane
// reads back its kSelItems consecutive scores. Read straight from memory,
// each load instruction of load_round spreads over 64 cache lines. The 16-byte
// slot f of a wave's block sits at f ^ ((f >> 4) & 15), which keeps both the
// row-wise writes and the lane-contiguous reads free of bank conflicts. stage:
// kRound floats; the caller syncs the block before reusing it.
__device__ __forceinline__ void load_round_staged(const float* __restrict__ s, int64_t n, bool key16,
                                                  uint32_t (&key)[kSelItems], float4* stage) {
  constexpr int NQ = kSelItems / 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t i0 = static_cast<int64_t>(w) * (64 * kSelItems) + 4 * lane;
  const float pad = __uint_as_float(0xffffffffu);  // key 0: "no element"
  float4 v[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t i = i0 + 256 * q;
    if (i + 4 <= n) {
      v[q] = *reinterpret_cast<const float4*>(s + i);
    } else {
      v[q].x = i + 0 < n ? s[i + 0] : pad;
      v[q].y = i + 1 < n ? s[i + 1] : pad;
      v[q].z = i + 2 < n ? s[i + 2] : pad;
      v[q].w = pad;
    }
  }
  float4* st = stage + (64 * kSelItems / 4) * w;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int f = 64 * q + lane;
    st[f ^ ((f >> 4) & 15)] = v[q];
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int f = NQ * lane + q;
    const float4 u = st[f ^ ((f >> 4) & 15)];
    key[4 * q + 0] = score_key(u.x, key16);
    key[4 * q + 1] = score_key(u.y, key16);
    key[4 * q + 2] = score_key(u.z, key16);
    key[4 * q + 3] = score_key(u.w, key16);
  }
}

// Histogram of one digit is in hist[0, nb); find the digit whose bin holds the
// krem-th largest element (bins scanned in descending digit order) and that
// element's rank inside the bin. Four bins per thread; on return the result
// is visible to the whole block.
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nb, uint32_t krem, uint32_t* wsum,
                                           uint32_t* sh_digit, uint32_t* sh_krem) {
  const int tid = threadIdx.x;
  uint32_t c[4], tsum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int d = nb - 1 - (4 * tid + q);
    c[q] = d >= 0 ? hist[d] : 0u;
    tsum += c[q];
  }
  uint32_t total;
  const uint32_t before = block_excl_scan(tsum, wsum, &total);
  if (before < krem && before + tsum >= krem) {
    uint32_t cum = before;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cum < krem && cum + c[q] >= krem) {
        *sh_digit = static_cast<uint32_t>(nb - 1 - (4 * tid + q));
        *sh_krem = krem - cum;
      }
      cum += c[q];
    }
  }
  __syncthreads();
}

// Row of one query: where its scores are, how many are visible, where its
// k indices (and optionally scores) go.
struct SelRow {
  const float* s;
  int64_t n;
  int32_t* io;
  float* so;
};

__device__ __forceinline__ SelRow sel_row(const float* scores, int64_t ld, int64_t N_cap, int Tq, int t_off, int Tc,
                                          int64_t q_pos0, const int64_t* q_pos, int m, int k, int32_t* idx_out,
                                          float* score_out) {
  const int b = blockIdx.y, tl = blockIdx.x, t = t_off + tl;
  int64_t n = n_visible(seq_pos(q_pos, q_pos0, b) + t, m);
  if (n > N_cap) n = N_cap;
  SelRow r;
  r.s = scores + (static_cast<int64_t>(b) * Tc + tl) * ld;
  r.n = n;
  r.io = idx_out + (static_cast<int64_t>(b) * Tq + t) * k;
  r.so = score_out ? score_out + (static_cast<int64_t>(b) * Tq + t) * k : nullptr;
  return r;
}

// Fewer visible entries than k: all of them, then -1 padding.
__device__ __forceinline__ void select_all(const SelRow& r, int k) {
  for (int i = threadIdx.x; i < k; i += kSelThreads) {
    r.io[i] = i < r.n ? i : -1;
    if (r.so) r.so[i] = i < r.n ? r.s[i] : -INFINITY;
  }
}

// Radix select by full passes over the scores: one per digit, then one that
// writes the output. A list that fits one register round is read only once.
__device__ __forceinline__ void select_by_passes(const SelRow& row, int k, bool key16, uint32_t* hist, uint32_t* wsum,
                                                 uint32_t* sh_digit_p, uint32_t* sh_krem_p) {
  uint32_t& sh_digit = *sh_digit_p;
  uint32_t& sh_krem = *sh_krem_p;
  const int tid = threadIdx.x;
  const float* s = row.s;
  const int64_t n = row.n;
  int32_t* io = row.io;
  float* so = row.so;
  const int rounds = static_cast<int>((n + kRound - 1) / kRound);
  uint32_t key[kSelItems];
  if (rounds == 1) load_round(s, n, 0, key16, key);     // kept in registers for every pass

  // MSB-first digits: 32-bit keys 12/10/10, 16-bit keys 12/4
  const int nd = key16 ? 2 : 3;
  uint32_t prefix = 0, pmask = 0;
  uint32_t krem = static_cast<uint32_t>(k);
  int shift = key16 ? 16 : 32;
  for (int p = 0; p < nd; ++p) {
    const int wd = key16 ? (p == 0 ? 12 : 4) : (p == 0 ? 12 : 10);
    shift -= wd;
    const int nb = 1 << wd;
    for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
      if (rounds > 1) load_round(s, n, static_cast<int64_t>(r) * kRound, key16, key);
#pragma unroll
      for (int j = 0; j < kSelItems; ++j)
        if (key[j] != 0u && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_digit(hist, nb, krem, wsum, &sh_digit, &sh_krem);
    prefix |= sh_digit << shift;
    pmask |= static_cast<uint32_t>(nb - 1) << shift;
    krem = sh_krem;
    __syncthreads();
  }
  const uint32_t thr = prefix;       // key of the k-th largest score

  // ordered compaction, round by round: positions follow increasing index
  uint32_t run_gt = 0, run_eq = 0;
  for (int r = 0; r < rounds; ++r) {
    const int64_t base = static_cast<int64_t>(r) * kRound;
    if (rounds > 1) load_round(s, n, base, key16, key);
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
      gtm |= static_cast<uint32_t>(key[j] > thr) << j;
      eqm |= static_cast<uint32_t>(key[j] == thr) << j;
    }
    const uint32_t gt = __builtin_popcount(gtm), eq = __builtin_popcount(eqm);
    uint32_t tot;
    const uint32_t pre = block_excl_scan((gt << 16) | eq, wsum, &tot);  // both < 2^16 per round
    const uint32_t gt_pre = run_gt + (pre >> 16), eq_pre = run_eq + (pre & 0xffffu);
    uint32_t pos = gt_pre + min(eq_pre, krem);
    // ties at the threshold: the first (krem - eq_pre) of them in index order
    uint32_t take = gtm;
    for (uint32_t c = eq_pre; eqm && c < krem; ++c) {
      take |= eqm & (~eqm + 1u);
      eqm &= eqm - 1;
    }
    const int64_t i0 = base + static_cast<int64_t>(tid) * kSelItems;
    while (take) {
      const int j = __builtin_ctz(take);
      take &= take - 1;
      io[pos] = static_cast<int32_t>(i0 + j);
      if (so) so[pos] = s[i0 + j];
      ++pos;
    }
    run_gt += tot >> 16;
    run_eq += tot & 0xffffu;
  }
}

// Short lists whose threads hold at least 2k scores' worth of maxima: each
// thread's largest key is a score of the list, so the lower edge `lo` of the
// top-digit bin holding the k-th largest of those maxima has at least k scores
// at or above it, and the k-th largest score is at or above `lo`. Lists too
// short for 2k thread maxima (ragged batches) take four maxima per thread, one
// per run of 8 scores (fine): the same bound over smaller disjoint groups. Only the
// scores from `lo` up (a few percent of a list, typically) are candidates:
// they go to LDS in increasing index order, and their digits are taken on the
// offset key - lo over [lo, max key] (12 bits at a time, from the top), which
// spreads them over the bins where the raw key's top digit would stack them
// into one or two (a float's sign and exponent). Same threshold, same ties in
// index order, same output as the full passes. Returns false, having written
// nothing, when the candidates exceed kCandCap.
constexpr int kCandCap = 4096;
constexpr int kCandPer = kCandCap / kSelThreads;
constexpr int kFewMax = 64;        // boundary-bin candidates one wave ranks directly

__device__ __forceinline__ bool select_filtered(const SelRow& row, int k, bool key16,
                                                const uint32_t (&key)[kSelItems], uint32_t* hist, uint32_t* wsum,
                                                uint32_t* ckey, int32_t* cidx, uint32_t* sh_digit_p,
                                                uint32_t* sh_krem_p, uint32_t* sh_hi_p, bool fine) {
  uint32_t& sh_digit = *sh_digit_p;
  uint32_t& sh_krem = *sh_krem_p;
  const int tid = threadIdx.x;
  const int top = key16 ? 4 : 20;                  // shift of the key's top 12-bit digit
  __shared__ uint32_t sh_nfew, few[kFewMax];       // a boundary bin's few candidates (any order)
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < kSelItems; ++j) mx = max(mx, key[j]);
  uint32_t wmx = mx;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wmx = max(wmx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(wmx), o, kWave)));
  for (int i = tid; i < kMaxBins; i += kSelThreads) hist[i] = 0;
  if (tid == 0) {
    *sh_hi_p = 0;
    sh_nfew = 0;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {                    // fine: the maxima of the runs of 8; else mx alone
    uint32_t mq = 0;
#pragma unroll
    for (int j = 8 * c; j < 8 * c + 8; ++j) mq = max(mq, key[j]);
    const uint32_t v = fine ? mq : (c == 0 ? mx : 0u);
    if (v != 0u) atomicAdd(&hist[v >> top], 1u);
  }
  if ((tid & 63) == 0) atomicMax(sh_hi_p, wmx);
  __syncthreads();
  find_digit(hist, kMaxBins, static_cast<uint32_t>(k), wsum, &sh_digit, &sh_krem);
  const uint32_t lo = sh_digit << top, hi = *sh_hi_p;
  uint32_t cm = 0;
#pragma unroll
  for (int j = 0; j < kSelItems; ++j) cm |= static_cast<uint32_t>(key[j] >= lo && key[j] != 0u) << j;
  uint32_t tot;
  const uint32_t pre = block_excl_scan(__builtin_popcount(cm), wsum, &tot);
  if (tot > static_cast<uint32_t>(kCandCap)) return false;
  {
    uint32_t pos = pre;
    const int32_t i0 = tid * kSelItems;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j)
      if ((cm >> j) & 1u) {
        ckey[pos] = key[j];
        cidx[pos] = i0 + j;
        ++pos;
      }
  }
  __syncthreads();
  // candidate c = kCandPer * tid + q: contiguous per thread, so one scan orders them
  uint32_t ck[kCandPer];
  {
    const uint4 v = reinterpret_cast<const uint4*>(ckey)[tid];
    const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < kCandPer; ++q) ck[q] = static_cast<uint32_t>(kCandPer * tid + q) < tot ? e[q] : 0u;
  }
  // digits of key - base over [base, base + width), 12 bits at a time
  uint32_t base = lo, krem = static_cast<uint32_t>(k);
  uint64_t width = static_cast<uint64_t>(hi) - lo + 1;
  while (width > 1) {
    const int bl = 64 - __builtin_clzll(width - 1);
    const int sh = bl > 12 ? bl - 12 : 0;
    const int nb = static_cast<int>((width - 1) >> sh) + 1;
    for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCandPer; ++q) {
      const uint32_t off = ck[q] - base;
      if (ck[q] != 0u && static_cast<uint64_t>(off) < width) atomicAdd(&hist[off >> sh], 1u);
    }
    __syncthreads();
    find_digit(hist, nb, krem, wsum, &sh_digit, &sh_krem);
    base += sh_digit << sh;
    krem = sh_krem;
    width = uint64_t(1) << sh;
    const uint32_t nbin = hist[sh_digit];           // candidates in [base, base + width)
    __syncthreads();                                 // read by all before a next pass clears it
    if (width > 1 && nbin <= static_cast<uint32_t>(kFewMax)) {
      // A boundary bin of at most 64 candidates (the usual case after one
      // digit: the k-th largest sits a few key steps above its neighbours):
      // one wave ranks them by comparison instead of more block-wide passes.
      // Key v is the threshold when (#keys > v) < krem <= (#keys >= v);
      // krem becomes krem - (#keys > v), as the remaining digits would give.
#pragma unroll
      for (int q = 0; q < kCandPer; ++q) {
        const uint32_t off = ck[q] - base;
        if (ck[q] != 0u && static_cast<uint64_t>(off) < width) few[atomicAdd(&sh_nfew, 1u)] = ck[q];
      }
      __syncthreads();
      if (tid < 64) {
        const uint32_t mine = tid < static_cast<int>(nbin) ? few[tid] : 0u;
        uint32_t gt = 0, ge = 0;
        for (uint32_t j = 0; j < nbin; ++j) {
          const uint32_t o = few[j];
          gt += o > mine;
          ge += o >= mine;
        }
        if (tid < static_cast<int>(nbin) && gt < krem && krem <= ge) {
          sh_digit = mine;                           // equal keys write equal values
          sh_krem = krem - gt;
        }
      }
      __syncthreads();
      base = sh_digit;
      krem = sh_krem;
      break;
    }
  }
  const uint32_t thr = base;       // key of the k-th largest score

  uint32_t gtm = 0, eqm = 0;
#pragma unroll
  for (int q = 0; q < kCandPer; ++q) {
    gtm |= static_cast<uint32_t>(ck[q] > thr) << q;
    eqm |= static_cast<uint32_t>(ck[q] == thr) << q;
  }
  uint32_t tot2;
  const uint32_t pre2 = block_excl_scan((__builtin_popcount(gtm) << 16) | __builtin_popcount(eqm), wsum, &tot2);
  const uint32_t gt_pre = pre2 >> 16, eq_pre = pre2 & 0xffffu;
  uint32_t pos = gt_pre + min(eq_pre, krem);
  uint32_t take = gtm;
  for (uint32_t c = eq_pre; eqm && c < krem; ++c) {
    take |= eqm & (~eqm + 1u);
    eqm &= eqm - 1;
  }
  while (take) {
    const int q = __builtin_ctz(take);
    take &= take - 1;
    const int32_t ix = cidx[kCandPer * tid + q];
    row.io[pos] = ix;
    if (row.so) row.so[pos] = row.s[ix];
    ++pos;
  }
  return true;
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t N_cap, int Tq, int t_off, int Tc,
    int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int k, bool key16, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out) {
  // the staging area of the coalesced load, then the histogram and candidates
  __shared__ __attribute__((aligned(16))) uint32_t pool[kRound];
  static_assert(kMaxBins + 2 * kCandCap <= kRound, "LDS pool");
  uint32_t* hist = pool;
  uint32_t* ckey = pool + kMaxBins;
  int32_t* cidx = reinterpret_cast<int32_t*>(pool + kMaxBins + kCandCap);
  __shared__ __attribute__((aligned(16))) uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t sh_digit, sh_krem, sh_hi;
  const SelRow row = sel_row(scores, ld, N_cap, Tq, t_off, Tc, q_pos0, q_pos, m, k, idx_out, score_out);
  if (row.n <= k) {
    select_all(row, k);
    return;
  }
  // threads holding a score: (n + kSelItems - 1) / kSelItems, one round (n <= kRound here);
  // below 2k of them, runs of 8 scores: (n + 7) / 8
  if ((row.n + 7) / 8 >= 2 * static_cast<int64_t>(k)) {
    const bool fine = (row.n + kSelItems - 1) / kSelItems < 2 * static_cast<int64_t>(k);
    uint32_t key[kSelItems];
    load_round_staged(row.s, row.n, key16, key, reinterpret_cast<float4*>(pool));
    __syncthreads();                 // every wave has read its staged scores back
    if (select_filtered(row, k, key16, key, hist, wsum, ckey, cidx, &sh_digit, &sh_krem, &sh_hi, fine)) return;
    __syncthreads();                 // candidate and histogram memory are reused below
  }
  select_by_passes(row, k, key16, hist, wsum, &sh_digit, &sh_krem);
}

// Number of entries of the increasing array a[0, n) that are < x.
__device__ __forceinline__ int count_below(const int32_t* a, int n, int32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

constexpr int kMaxK = 4096;        // largest k the library accepts
constexpr int kLongCap = 8192;     // boundary-bin candidates held in LDS

// Lists longer than one register round, in two reads of the scores instead of
// one per digit plus one for the output. Read 1 builds the first (12-bit)
// digit's histogram, which fixes the boundary bin b* and how many of its
// entries are taken. Read 2 puts the indices above b* and the (key, index)
// pairs inside b* into LDS, both in increasing index order (block scans). The
// remaining digits are resolved on the candidates alone, and the two sorted
// lists are merged into the output: the same set and order as the pass-based
// select. Candidates past kLongCap (a bin crowded by ties, e.g. the exact
// zeros of a query whose head weights are all negative) keep only their index,
// in the row's spill buffer (ld entries), and their key is read again from the
// scores.
// One round's raw scores for this thread, fetched a round ahead of their use
// so that the next round's loads are in flight while this round's histogram
// atomics run (read 1 of the long select; read 2 keeps one round, since its
// block scan and ordered writes need the registers). Past the list end the
// cells hold the bit pattern 0xffffffff, whose key is 0 ("no element").
template <int NI = kSelItems>
struct RoundRaw {
  float4 v[NI / 4];
};

template <int NI>
__device__ __forceinline__ void fetch_round(const float* __restrict__ s, int64_t n, int64_t base, RoundRaw<NI>& r) {
  const int64_t i0 = base + static_cast<int64_t>(threadIdx.x) * NI;
  if (i0 + NI <= n) {
#pragma unroll
    for (int q = 0; q < NI / 4; ++q) r.v[q] = *reinterpret_cast<const float4*>(s + i0 + 4 * q);
  } else {
    const float pad = __uint_as_float(0xffffffffu);
#pragma unroll
    for (int q = 0; q < NI / 4; ++q) {
      const int64_t j = i0 + 4 * q;
      r.v[q] = make_float4(j < n ? s[j] : pad, j + 1 < n ? s[j + 1] : pad, j + 2 < n ? s[j + 2] : pad,
                           j + 3 < n ? s[j + 3] : pad);
    }
  }
}

// Key of cell j (a compile-time index once unrolled) of a fetched round.
template <int NI>
__device__ __forceinline__ uint32_t raw_key(const RoundRaw<NI>& r, int j, bool key16) {
  const float4 q = r.v[j >> 2];
  const float v = (j & 3) == 0 ? q.x : (j & 3) == 1 ? q.y : (j & 3) == 2 ? q.z : q.w;
  return score_key(v, key16);
}

__global__ __launch_bounds__(kSelThreads) void topk_select_long_kernel(
    const float* __restrict__ scores, int64_t ld, int32_t* __restrict__ spill, int64_t N_cap, int Tq, int t_off,
    int Tc, int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int k, bool key16,
    int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  __shared__ uint32_t hist[kMaxBins];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t sh_digit, sh_krem, sh_cmin, sh_cmax;
  __shared__ int32_t a_idx[kMaxK];        // above b*, increasing index
  __shared__ int32_t w_idx[kMaxK];        // winners inside b*, increasing index
  __shared__ uint32_t c_key[kLongCap];    // candidates inside b*, increasing index
  __shared__ int32_t c_idx[kLongCap];
  const int tid = threadIdx.x;
  const SelRow row = sel_row(scores, ld, N_cap, Tq, t_off, Tc, q_pos0, q_pos, m, k, idx_out, score_out);
  if (row.n <= k) {
    select_all(row, k);
    return;
  }
  const float* s = row.s;
  const int64_t n = row.n;
  int32_t* sp = spill + (static_cast<int64_t>(blockIdx.y) * Tc + blockIdx.x) * ld;   // candidate kLongCap + i at sp[i]
  const int rounds = static_cast<int>((n + kRound - 1) / kRound);
  const int sh0 = (key16 ? 16 : 32) - 12;

  // read 1: first digit
  for (int i = tid; i < kMaxBins; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  RoundRaw<> nxt;
  fetch_round(s, n, 0, nxt);
  for (int r = 0; r < rounds; ++r) {
    const RoundRaw<> cur = nxt;
    if (r + 1 < rounds) fetch_round(s, n, static_cast<int64_t>(r + 1) * kRound, nxt);
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
      const uint32_t kj = raw_key(cur, j, key16);
      if (kj != 0u) atomicAdd(&hist[kj >> sh0], 1u);
    }
  }
  __syncthreads();
  if (tid == 0) {
    sh_cmin = 0xffffffffu;
    sh_cmax = 0u;
  }
  find_digit(hist, kMaxBins, static_cast<uint32_t>(k), wsum, &sh_digit, &sh_krem);
  const uint32_t bstar = sh_digit, krem1 = sh_krem;
  uint32_t cmin = 0xffffffffu, cmax = 0u;     // candidate key range, this thread

  // read 2: entries above b* and candidates inside it, in index order; half
  // rounds (16 scores per thread) so that the next one's loads fit in
  // registers beside this one's during the block scan and ordered writes
  constexpr int kHalf = kSelItems / 2, kHalfRound = kSelThreads * kHalf;
  const int rounds2 = static_cast<int>((n + kHalfRound - 1) / kHalfRound);
  uint32_t run_a = 0, run_c = 0;
  RoundRaw<kHalf> nxt2;
  fetch_round(s, n, 0, nxt2);
  for (int r = 0; r < rounds2; ++r) {
    const int64_t base = static_cast<int64_t>(r) * kHalfRound;
    const RoundRaw<kHalf> cur = nxt2;
    if (r + 1 < rounds2) fetch_round(s, n, base + kHalfRound, nxt2);
    uint32_t key[kHalf];
#pragma unroll
    for (int j = 0; j < kHalf; ++j) key[j] = raw_key(cur, j, key16);
    uint32_t am = 0, cm = 0;
#pragma unroll
    for (int j = 0; j < kHalf; ++j) {
      const uint32_t d = key[j] >> sh0;
      am |= static_cast<uint32_t>(key[j] != 0u && d > bstar) << j;
      cm |= static_cast<uint32_t>(key[j] != 0u && d == bstar) << j;
    }
    uint32_t tot;   // both counts < 2^16 per round
    const uint32_t pre = block_excl_scan((static_cast<uint32_t>(__builtin_popcount(am)) << 16) |
                                         static_cast<uint32_t>(__builtin_popcount(cm)), wsum, &tot);
    uint32_t pa = run_a + (pre >> 16), pc = run_c + (pre & 0xffffu);
    const int32_t i0 = static_cast<int32_t>(base) + tid * kHalf;
#pragma unroll
    for (int j = 0; j < kHalf; ++j) {
      if ((am >> j) & 1u) a_idx[pa++] = i0 + j;
      if ((cm >> j) & 1u) {
        const uint32_t kj = key[j];
        cmin = min(cmin, kj);
        cmax = max(cmax, kj);
        if (pc < static_cast<uint32_t>(kLongCap)) {
          c_key[pc] = kj;
          c_idx[pc] = i0 + j;
        } else {
          sp[pc - kLongCap] = i0 + j;
        }
        ++pc;
      }
    }
    run_a += tot >> 16;
    run_c += tot & 0xffffu;
  }
  if (cmin <= cmax) {
    atomicMin(&sh_cmin, cmin);
    atomicMax(&sh_cmax, cmax);
  }
  __syncthreads();
  const int nc = static_cast<int>(run_c);
  const int n_w = static_cast<int>(krem1), n_a = k - n_w;
  if (sh_cmin == sh_cmax) {
    // one key fills the boundary bin (exact ties, e.g. zeros): the winners
    // are its first krem1 entries in index order, all held in LDS
    for (int i = tid; i < n_w; i += kSelThreads) w_idx[i] = c_idx[i];
    __syncthreads();
  } else {
    // candidate i: from LDS, or from the spill buffer with its key read again
    auto cand_idx = [&](int i) { return i < kLongCap ? c_idx[i] : sp[i - kLongCap]; };
    auto cand_key = [&](int i) { return i < kLongCap ? c_key[i] : score_key(s[sp[i - kLongCap]], key16); };

    // remaining digits on the candidates
    uint32_t prefix = bstar << sh0, pmask = 0xfffu << sh0, krem = krem1;
    int shift = sh0;
    while (shift > 0) {
      const int wd = shift >= 10 ? 10 : shift;
      shift -= wd;
      const int nb = 1 << wd;
      for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += kSelThreads) {
        const uint32_t kk = cand_key(i);
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      find_digit(hist, nb, krem, wsum, &sh_digit, &sh_krem);
      prefix |= sh_digit << shift;
      pmask |= static_cast<uint32_t>(nb - 1) << shift;
      krem = sh_krem;
      __syncthreads();
    }
    const uint32_t thr = prefix;

    // winners inside b* in index order: above thr, then the first krem equal to it
    uint32_t run_gt = 0, run_eq = 0;
    for (int c0 = 0; c0 < nc; c0 += kSelThreads) {
      const int i = c0 + tid;
      const uint32_t kk = i < nc ? cand_key(i) : 0u;
      const uint32_t gt = i < nc && kk > thr, eq = i < nc && kk == thr;
      uint32_t tot;
      const uint32_t pre = block_excl_scan((gt << 16) | eq, wsum, &tot);
      const uint32_t eq_rank = run_eq + (pre & 0xffffu);
      if (gt || (eq && eq_rank < krem)) w_idx[run_gt + (pre >> 16) + min(eq_rank, krem)] = cand_idx(i);
      run_gt += tot >> 16;
      run_eq += tot & 0xffffu;
    }
    __syncthreads();
  }

  // merge the two increasing lists
  for (int i = tid; i < n_a; i += kSelThreads) {
    const int32_t x = a_idx[i];
    const int pos = i + count_below(w_idx, n_w, x);
    row.io[pos] = x;
    if (row.so) row.so[pos] = s[x];
  }
  for (int i = tid; i < n_w; i += kSelThreads) {
    const int32_t x = w_idx[i];
    const int pos = i + count_below(a_idx, n_a, x);
    row.io[pos] = x;
    if (row.so) row.so[pos] = s[x];
  }
}

// ---------------------------------------------------------------------------
// Chunked select bounded by group maxima.
//
// A select held by one 1024-thread workgroup per query spends its time on
// vector ALU work (four waves per SIMD) and on barrier-separated phases, so a
// long list is cut into chunks of kFiltChunk scores, one 256-thread workgroup
// each (topk_chunk_kernel), and a second kernel (topk_final_kernel, one
// workgroup per query) resolves the selection from their candidates; the
// kernel boundary makes the candidates visible to it. The scoring kernel left
// the maximum of every group of kGroup keys. From them follows a lower bound
// lo on the k-th largest score: wave w of a chunk workgroup takes the groups g
// with g % 4 == w and finds t_w, the r-th largest of their maxima (r =
// ceil(k / 4), a bitwise search on ballots over the top 16 key bits; the lower
// edge of that 16-bit bin is still a bound); each maximum is a distinct score,
// so at least k scores are >= lo = min_w t_w. (A wave with fewer than r groups
// bounds nothing: lo falls to the smallest key.) Lists with too many groups
// take lo from topk_bound_kernel. A chunk writes its scores above lo, then its
// scores equal to lo, each list in index order, and both counts. If at least
// k candidates lie above lo, the k-th largest is among them and radix passes
// on their keys find it; otherwise it is lo itself, and the winners are every
// candidate above lo plus the first (k - above) ties in index order (a crowd
// of equal scores, e.g. the exact zeros of a query whose head weights are all
// negative, costs nothing). The output is the same set in the same order as
// the full passes. A chunk with more candidates than its slots, or a row with
// more than the final workgroup holds, falls back to full passes over the row.
// ---------------------------------------------------------------------------
constexpr int kFiltThreads = 256;
constexpr int kFiltItems = 16;
constexpr int kFiltChunk = kFiltThreads * kFiltItems;   // scores per chunk workgroup
constexpr int kRunMax = 32;                              // candidates per thread of the final workgroup
constexpr int kStageKeys = kMaxBins;                     // candidate keys the final workgroup stages in LDS
constexpr int kMaxChunks = 1024;                         // chunks whose counts fit LDS
constexpr int kInlineItems = 8;                          // group maxima per lane, bound inside the chunk kernel
constexpr int kBoundItems = 32;                          // group maxima per lane, bound kernel
constexpr uint32_t kOverflow = 0xffffffffu;

struct FiltWs {
  float* gmax;            // [rows, ldg] group maxima
  int64_t ldg;
  uint32_t* bound;        // [rows, 2] lo, hi keys (bound kernel output)
  uint32_t* ckey;         // [rows, nchs, capc] candidate keys: above lo, then equal to lo
  int32_t* cidx;          // [rows, nchs, capc] their indices
  uint32_t* cnt;          // [rows, nchs] (above << 16) | equal, kOverflow past capc
  int nchs;               // chunk stride per row
  int capc;               // candidate slots per chunk
  uint32_t* lim;          // [rows] candidate index limit (bound kernel output)
};

// Exclusive scan over NT threads (NT / 64 waves), one value per thread.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_t(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t e = wsum[w];
    before += w < wid ? e : 0u;
    all += e;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// As find_digit, for NT threads (nb <= kMaxBins).
template <int NT>
__device__ __forceinline__ void find_digit_t(const uint32_t* hist, int nb, uint32_t krem, uint32_t* wsum,
                                             uint32_t* sh_digit, uint32_t* sh_krem) {
  constexpr int BPT = kMaxBins / NT;
  const int tid = threadIdx.x;
  uint32_t c[BPT], tsum = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int d = nb - 1 - (BPT * tid + q);
    c[q] = d >= 0 ? hist[d] : 0u;
    tsum += c[q];
  }
  uint32_t total;
  const uint32_t before = block_excl_scan_t<NT>(tsum, wsum, &total);
  if (before < krem && before + tsum >= krem) {
    uint32_t cum = before;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (cum < krem && cum + c[q] >= krem) {
        *sh_digit = static_cast<uint32_t>(nb - 1 - (BPT * tid + q));
        *sh_krem = krem - cum;
      }
      cum += c[q];
    }
  }
  __syncthreads();
}

// Lower bound lo and upper bound hi (keys) of a row's k-th largest score from
// its ng group maxima (see above); the result is the same in every workgroup
// and thread. BI: maxima per lane kept in registers; with more groups than
// 4 * 64 * BI, each item takes the maximum of gs consecutive groups (a coarser
// but still valid bound).
template <int BI>
__device__ __forceinline__ void group_bound(const float* __restrict__ gm, int64_t ng, int k, bool key16,
                                            uint32_t* wv, uint32_t* lo_out, uint32_t* hi_out) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int64_t kPer = 4 * kWave * BI;
  const int64_t gs = (ng + kPer - 1) / kPer;             // groups per item
  const int64_t ns = (ng + gs - 1) / gs;                 // items in the row
  // item i of this lane: groups [sg * gs, sg * gs + gs), sg = 4 (64 i + lane) + wid;
  // the loads of one pass over d are independent and go out together
  float fm[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) fm[i] = -INFINITY;
  for (int64_t d = 0; d < gs; ++d) {
    // every load of the pass is issued unconditionally (out-of-row items read
    // group 0) before any is used
    float x[BI];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int64_t sg = 4 * (static_cast<int64_t>(kWave) * i + lane) + wid;
      const int64_t gg = sg * gs + d;
      x[i] = gm[sg < ns && gg < ng ? gg : 0];
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int64_t sg = 4 * (static_cast<int64_t>(kWave) * i + lane) + wid;
      if (sg < ns && sg * gs + d < ng) fm[i] = fmaxf(fm[i], x[i]);
    }
  }
  uint32_t kv[BI], mx = 0;
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int64_t sg = 4 * (static_cast<int64_t>(kWave) * i + lane) + wid;
    kv[i] = sg < ns ? score_key(fm[i], key16) : 0u;
    mx = max(mx, kv[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), o, kWave)));
  // the search runs on the keys' top 16 bits: the lower edge of the 16-bit
  // bin of the r-th largest is at or below it, so still a bound
  const int ksh = key16 ? 0 : 16;
  const uint32_t r = static_cast<uint32_t>((k + 3) / 4);
  const int64_t have = ns > wid ? (ns - wid + 3) / 4 : 0;    // items of this wave
  uint32_t t = 0;
  if (have >= r) {
    uint32_t k16[BI];
#pragma unroll
    for (int i = 0; i < BI; ++i) k16[i] = kv[i] >> ksh;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = t | (1u << bit);
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < BI; ++i) cnt += static_cast<uint32_t>(__popcll(__ballot(k16[i] >= c)));
      if (cnt >= r) t = c;
    }
    t <<= ksh;
  }
  if (lane == 0) {
    wv[wid] = t;
    wv[4 + wid] = mx;
  }
  __syncthreads();
  uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    lo = min(lo, wv[w]);
    hi = max(hi, wv[4 + w]);
  }
  *lo_out = lo > 0u ? lo : 1u;                           // key 0 is "no element"
  *hi_out = hi;
  __syncthreads();
}

// group_bound for rows of at most 256 * 4 * NV maxima (the bound kernel's
// common case): thread i loads maxima 4 (i + 256 j) .. + 3 as one 16-byte
// load for j < NV (all loads issued before any is used), and each load's two
// pairs are its items (the maximum of 2 groups): 2 NV items per lane, the
// waves' items a partition of the row. Then as group_bound: each wave the
// ceil(k / 4)-th largest of its items on the keys' top 16 bits, lo the
// smallest of the four.
// SINGLE: every group its own item (4 NV items per lane), for the sampled
// maxima, which are few and spread over the row; the loads are dealt to the
// waves in turn (load f to wave f % 4), so that each wave holds a quarter of
// a short row and bounds it.
template <int NV, bool SINGLE = false>
__device__ __forceinline__ void group_bound_v4(const float* __restrict__ gm, int64_t ng, int k, bool key16,
                                               uint32_t* wv, uint32_t* lo_out, uint32_t* hi_out) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int IPL = SINGLE ? 4 : 2;              // items per load
  const int fl = SINGLE ? 4 * lane + wid : tid;     // this thread's load within a round of 256
  float4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t f = fl + static_cast<int64_t>(kFiltThreads) * j;
    v[j] = 4 * f < ng ? *reinterpret_cast<const float4*>(gm + 4 * f) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  uint32_t kv[IPL * NV], mx = 0, have = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t g0 = 4 * (fl + static_cast<int64_t>(kFiltThreads) * j);
    if constexpr (SINGLE) {
      const float x[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kv[4 * j + i] = g0 + i < ng ? score_key(x[i], key16) : 0u;
        mx = max(mx, kv[4 * j + i]);
        have += static_cast<uint32_t>(__popcll(__ballot(g0 + i < ng)));
      }
    } else {
      // an item counts the groups of its pair that exist (a row's last pair may hold one)
      const float a0 = g0 < ng ? v[j].x : -INFINITY, a1 = g0 + 1 < ng ? v[j].y : -INFINITY;
      const float b0 = g0 + 2 < ng ? v[j].z : -INFINITY, b1 = g0 + 3 < ng ? v[j].w : -INFINITY;
      kv[2 * j] = g0 < ng ? score_key(fmaxf(a0, a1), key16) : 0u;
      kv[2 * j + 1] = g0 + 2 < ng ? score_key(fmaxf(b0, b1), key16) : 0u;
      mx = max(mx, max(kv[2 * j], kv[2 * j + 1]));
      have += static_cast<uint32_t>(__popcll(__ballot(g0 < ng))) + static_cast<uint32_t>(__popcll(__ballot(g0 + 2 < ng)));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), o, kWave)));
  const int ksh = key16 ? 0 : 16;
  const uint32_t r = static_cast<uint32_t>((k + 3) / 4);
  uint32_t t = 0;
  if (have >= r) {
    uint32_t k16[IPL * NV];
#pragma unroll
    for (int i = 0; i < IPL * NV; ++i) k16[i] = kv[i] >> ksh;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = t | (1u << bit);
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < IPL * NV; ++i) cnt += static_cast<uint32_t>(__popcll(__ballot(k16[i] >= c)));
      if (cnt >= r) t = c;
    }
    t <<= ksh;
  }
  if (lane == 0) {
    wv[wid] = t;
    wv[4 + wid] = mx;
  }
  __syncthreads();
  uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    lo = min(lo, wv[w]);
    hi = max(hi, wv[4 + w]);
  }
  *lo_out = lo > 0u ? lo : 1u;                           // key 0 is "no element"
  *hi_out = hi;
  __syncthreads();
}

// Row (b, tl) of a chunked call: scores, visible count, outputs.
struct FiltRow {
  const float* s;
  int64_t n;
  int64_t r;               // row index b * Tc + tl
  int32_t* io;
  float* so;
};

__device__ __forceinline__ FiltRow filt_row(const float* scores, int64_t ld, int64_t N_cap, int Tq, int t_off, int Tc,
                                            int64_t q_pos0, const int64_t* q_pos, int m, int k, int32_t* idx_out,
                                            float* score_out) {
  const int b = blockIdx.z, tl = blockIdx.y, t = t_off + tl;
  int64_t n = n_visible(seq_pos(q_pos, q_pos0, b) + t, m);
  if (n > N_cap) n = N_cap;
  FiltRow f;
  f.r = static_cast<int64_t>(b) * Tc + tl;
  f.s = scores + f.r * ld;
  f.n = n;
  f.io = idx_out + (static_cast<int64_t>(b) * Tq + t) * k;
  f.so = score_out ? score_out + (static_cast<int64_t>(b) * Tq + t) * k : nullptr;
  return f;
}

// Radix select by full passes over a row in global memory, NT threads: one
// pass per digit, then the ordered output. The fallback of the chunked select.
template <int NT>
__device__ void select_passes_t(const FiltRow& row, int k, bool key16, uint32_t* hist, uint32_t* wsum,
                                uint32_t* sh_digit, uint32_t* sh_krem) {
  constexpr int IT = 16;                                 // scores per thread per round
  constexpr int RND = NT * IT;
  const int tid = threadIdx.x;
  const int64_t n = row.n;
  const int64_t rounds = (n + RND - 1) / RND;
  auto load = [&](int64_t base, uint32_t (&key)[IT]) {
    const int64_t i0 = base + static_cast<int64_t>(tid) * IT;
#pragma unroll
    for (int j = 0; j < IT; ++j) key[j] = i0 + j < n ? score_key(row.s[i0 + j], key16) : 0u;
  };
  const int nd = key16 ? 2 : 3;
  uint32_t prefix = 0, pmask = 0, krem = static_cast<uint32_t>(k);
  int shift = key16 ? 16 : 32;
  for (int p = 0; p < nd; ++p) {
    const int wd = key16 ? (p == 0 ? 12 : 4) : (p == 0 ? 12 : 10);
    shift -= wd;
    const int nb = 1 << wd;
    for (int i = tid; i < nb; i += NT) hist[i] = 0;
    __syncthreads();
    for (int64_t rr = 0; rr < rounds; ++rr) {
      uint32_t key[IT];
      load(rr * RND, key);
#pragma unroll
      for (int j = 0; j < IT; ++j)
        if (key[j] != 0u && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_digit_t<NT>(hist, nb, krem, wsum, sh_digit, sh_krem);
    prefix |= *sh_digit << shift;
    pmask |= static_cast<uint32_t>(nb - 1) << shift;
    krem = *sh_krem;
    __syncthreads();
  }
  const uint32_t thr = prefix;
  uint32_t run_gt = 0, run_eq = 0;
  for (int64_t rr = 0; rr < rounds; ++rr) {
    uint32_t key[IT];
    load(rr * RND, key);
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      gtm |= static_cast<uint32_t>(key[j] > thr) << j;
      eqm |= static_cast<uint32_t>(key[j] == thr) << j;
    }
    uint32_t tg, te;
    const uint32_t pg = block_excl_scan_t<NT>(__builtin_popcount(gtm), wsum, &tg);
    const uint32_t pe = block_excl_scan_t<NT>(__builtin_popcount(eqm), wsum, &te);
    const uint32_t eq_pre = run_eq + pe;
    uint32_t pos = run_gt + pg + min(eq_pre, krem);
    uint32_t take = gtm;
    for (uint32_t c = eq_pre; eqm && c < krem; ++c) {
      take |= eqm & (~eqm + 1u);
      eqm &= eqm - 1;
    }
    const int64_t i0 = rr * RND + static_cast<int64_t>(tid) * IT;
    while (take) {
      const int j = __builtin_ctz(take);
      take &= take - 1;
      row.io[pos] = static_cast<int32_t>(i0 + j);
      if (row.so) row.so[pos] = row.s[i0 + j];
      ++pos;
    }
    run_gt += tg;
    run_eq += te;
  }
}

// One workgroup per row: the group bound, for rows whose maxima are too many
// to take inside every chunk workgroup.
// Also the row's candidate index limit: when the bound equals the row's
// largest key (every key at or above it ties at it, as in a row whose head
// weights are all negative, with its many exact zeros), the k selected are
// the first k ties in index order, and they lie in the groups up to the k-th
// group (in index order) whose maximum reaches the bound: at least k ties sit
// there. Keys past that group are no candidates. Otherwise the limit is the
// visible count.
// ss > 1: the row holds the maxima of every ss-th 64-key tile only (the
// sampled maxima pass), tile u ss at slots 4 u .. 4 u + 3; each is still the
// largest of distinct scores, so the bound holds, only less tight. The index
// limit then ends at the tile of the k-th sampled group at or above lo: when
// hi == lo, each such group holds a tie, so the first k ties lie before it
// (scores above lo may lie anywhere: the candidate pass keeps those past it).
__global__ __launch_bounds__(kFiltThreads) void topk_bound_kernel(
    FiltWs fw, int64_t N_cap, int Tc, int64_t q_pos0, const int64_t* __restrict__ q_pos, int t_off, int m, int k,
    bool key16, int ss) {
  __shared__ uint32_t wv[8];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[kFiltThreads / 64];
  __shared__ uint32_t sh_lim;
  const int b = blockIdx.z, tl = blockIdx.y;
  int64_t n = n_visible(seq_pos(q_pos, q_pos0, b) + t_off + tl, m);
  if (n > N_cap) n = N_cap;
  if (n <= k) return;
  const int64_t r = static_cast<int64_t>(b) * Tc + tl;
  uint32_t lo, hi;
  // groups held: with sampling, the slots whose first key (tile base + 4 c)
  // is visible
  const int64_t tspan = int64_t(kTileKeys) * ss;
  const int64_t ulast = (n - 1) / tspan, rem = n - ulast * tspan;
  const int64_t ng = ss == 1 ? (n + kGroup - 1) / kGroup : 4 * ulast + (rem >= 13 ? 4 : (rem + 3) / 4);
  const float* gm = fw.gmax + r * fw.ldg;
  // 16-byte loads of 4 groups for rows up to 4 * 256 * 17 groups (lists of
  // 278528 entries: the 1M-token prefill's rows are just past 262144)
  if (ss > 1 && ng <= 4 * kFiltThreads * 4)
    group_bound_v4<4, true>(gm, ng, k, key16, wv, &lo, &hi);
  else if (ss > 1 && ng <= 4 * kFiltThreads * 8)
    group_bound_v4<8, true>(gm, ng, k, key16, wv, &lo, &hi);
  else if (ng <= 4 * kFiltThreads * 16)
    group_bound_v4<16>(gm, ng, k, key16, wv, &lo, &hi);
  else if (ng <= 4 * kFiltThreads * 17)
    group_bound_v4<17>(gm, ng, k, key16, wv, &lo, &hi);
  else
    group_bound<kBoundItems>(gm, ng, k, key16, wv, &lo, &hi);
  if (threadIdx.x == 0) sh_lim = static_cast<uint32_t>(n);
  if (hi == lo) {                                   // uniform across the block
    const int tid = threadIdx.x;
    uint32_t need = static_cast<uint32_t>(k);
    for (int64_t g0 = 0; g0 < ng; g0 += 4 * kFiltThreads) {
      const int64_t gi = g0 + 4 * tid;             // 4 consecutive groups per thread
      const float4 v = gi < ng ? *reinterpret_cast<const float4*>(gm + gi) : make_float4(0.f, 0.f, 0.f, 0.f);
      const uint32_t c0 = gi < ng && score_key(v.x, key16) >= lo;
      const uint32_t c1 = gi + 1 < ng && score_key(v.y, key16) >= lo;
      const uint32_t c2 = gi + 2 < ng && score_key(v.z, key16) >= lo;
      const uint32_t c3 = gi + 3 < ng && score_key(v.w, key16) >= lo;
      const uint32_t c = c0 + c1 + c2 + c3;
      uint32_t tot;
      const uint32_t pre = block_excl_scan_t<kFiltThreads>(c, wsum, &tot);
      if (pre < need && pre + c >= need) {          // the need-th such group is one of this thread's
        const uint32_t q = need - pre;              // 1..4
        const int j = c0 >= q ? 0 : (c0 + c1 >= q ? 1 : (c0 + c1 + c2 >= q ? 2 : 3));
        const int64_t lim = ((gi + j) / 4 * ss + 1) * kTileKeys;   // the end of its tile
        sh_lim = static_cast<uint32_t>(lim < n ? lim : n);
      }
      if (tot >= need) break;                       // uniform
      need -= tot;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    fw.bound[2 * r] = lo;
    fw.bound[2 * r + 1] = hi;
    fw.lim[r] = sh_lim;
  }
}

// Chunk c of row (b, tl): the bound, then this chunk's candidates.
template <int BI>
__global__ __launch_bounds__(kFiltThreads) void topk_chunk_kernel(
    const float* __restrict__ scores, int64_t ld, FiltWs fw, int64_t N_cap, int Tq, int t_off, int Tc,
    int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int k, bool key16) {
  __shared__ __attribute__((aligned(16))) uint32_t wsum[kFiltThreads / 64];
  __shared__ uint32_t wv[8];
  const int tid = threadIdx.x;
  const FiltRow row = filt_row(scores, ld, N_cap, Tq, t_off, Tc, q_pos0, q_pos, m, k, nullptr, nullptr);
  const int c = blockIdx.x;
  if (row.n <= k || c >= (row.n + kFiltChunk - 1) / kFiltChunk) return;
  // this chunk's scores first: their loads are in flight during the bound
  const int64_t i0 = static_cast<int64_t>(c) * kFiltChunk + static_cast<int64_t>(tid) * kFiltItems;
  uint32_t key[kFiltItems];
  if (i0 + kFiltItems <= row.n) {
    float4 v[kFiltItems / 4];
#pragma unroll
    for (int q = 0; q < kFiltItems / 4; ++q) v[q] = *reinterpret_cast<const float4*>(row.s + i0 + 4 * q);
#pragma unroll
    for (int q = 0; q < kFiltItems / 4; ++q) {
      key[4 * q] = score_key(v[q].x, key16);
      key[4 * q + 1] = score_key(v[q].y, key16);
      key[4 * q + 2] = score_key(v[q].z, key16);
      key[4 * q + 3] = score_key(v[q].w, key16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kFiltItems; ++j) key[j] = i0 + j < row.n ? score_key(row.s[i0 + j], key16) : 0u;
  }
  uint32_t lo, hi;
  if constexpr (BI > 0) {
    group_bound<BI>(fw.gmax + row.r * fw.ldg, (row.n + kGroup - 1) / kGroup, k, key16, wv, &lo, &hi);
  } else {
    lo = fw.bound[2 * row.r];
    hi = fw.bound[2 * row.r + 1];
  }
  uint32_t am = 0, em = 0;
#pragma unroll
  for (int j = 0; j < kFiltItems; ++j) {
    am |= static_cast<uint32_t>(key[j] > lo) << j;
    em |= static_cast<uint32_t>(key[j] == lo) << j;
  }
  uint32_t tot;   // both counts < 2^16
  const uint32_t pre = block_excl_scan_t<kFiltThreads>((static_cast<uint32_t>(__builtin_popcount(am)) << 16) |
                                                           static_cast<uint32_t>(__builtin_popcount(em)), wsum, &tot);
  const uint32_t A = tot >> 16, E = tot & 0xffffu;
  const bool fits = A + E <= static_cast<uint32_t>(fw.capc);
  if (fits) {
    const int64_t cb = (row.r * fw.nchs + c) * fw.capc;
    uint32_t pa = pre >> 16, pe = A + (pre & 0xffffu);
#pragma unroll
    for (int j = 0; j < kFiltItems; ++j) {
      if ((am >> j) & 1u) {
        fw.ckey[cb + pa] = key[j];
        fw.cidx[cb + pa] = static_cast<int32_t>(i0 + j);
        ++pa;
      }
      if ((em >> j) & 1u) {
        fw.ckey[cb + pe] = key[j];
        fw.cidx[cb + pe] = static_cast<int32_t>(i0 + j);
        ++pe;
      }
    }
  }
  if (tid == 0) fw.cnt[row.r * fw.nchs + c] = fits ? tot : kOverflow;
  if (BI > 0 && c == 0 && tid == 0) {               // the final kernel reads the bound here
    fw.bound[2 * row.r] = lo;
    fw.bound[2 * row.r + 1] = hi;
  }
}

// Map of candidate position p of a row (chunks concatenated in order) to its
// chunk: pre[c] = candidates before chunk c (pre[nch] = all).
__device__ __forceinline__ int chunk_of(const uint32_t* pre, int nch, uint32_t p) {
  int lo = 0, hi = nch;                                  // pre[lo] <= p < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Exclusive prefix over the 64 lanes of a wave (DPP scan), and the wave total.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
  const uint32_t incl = wave_incl_scan(v);
  *total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
  return incl - v;
}

// In one wave: the digit (bins in hist[0, nb), nb <= 256) whose bin holds the
// krem-th largest element and that element's rank inside the bin.
__device__ __forceinline__ void wave_find_digit(const uint32_t* hist, int nb, uint32_t krem, uint32_t* digit,
                                                uint32_t* krem_out) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4], tsum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int d = nb - 1 - (4 * lane + q);
    c[q] = d >= 0 ? hist[d] : 0u;
    tsum += c[q];
  }
  uint32_t total;
  const uint32_t before = wave_excl_scan(tsum, &total);
  uint32_t dg = 0, kr = 0;
  const bool mine = before < krem && before + tsum >= krem;
  if (mine) {
    uint32_t cum = before;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cum < krem && cum + c[q] >= krem) {
        dg = static_cast<uint32_t>(nb - 1 - (4 * lane + q));
        kr = krem - cum;
      }
      cum += c[q];
    }
  }
  const uint64_t bal = __ballot(mine);
  const int src = bal ? __builtin_ctzll(bal) : 0;
  *digit = static_cast<uint32_t>(__shfl(static_cast<int>(dg), src, kWave));
  *krem_out = static_cast<uint32_t>(__shfl(static_cast<int>(kr), src, kWave));
}

// The k-th largest of n keys staged in LDS (keys > base are counted; krem
// counts from the top), taken by one wave with a private 256-bin histogram:
// 8-bit digits of key - base over [base, base + width). Every wave may run it
// on the same keys and reaches the same result. Returns thr; *krem_out = how
// many keys equal to thr are taken.
__device__ __forceinline__ uint32_t wave_kth(const uint32_t* keys, int n, uint32_t base, uint64_t width,
                                             uint32_t krem, uint32_t* hist, uint32_t* krem_out) {
  const int lane = threadIdx.x & 63;
  while (width > 1) {
    const int bl = 64 - __builtin_clzll(width - 1);
    const int sh = bl > 8 ? bl - 8 : 0;
    const int nb = static_cast<int>((width - 1) >> sh) + 1;
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < n; i += kWave) {
      const uint32_t kk = keys[i];
      const uint32_t off = kk - base;
      if (kk >= base && static_cast<uint64_t>(off) < width) atomicAdd(&hist[off >> sh], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t dg;
    wave_find_digit(hist, nb, krem, &dg, &krem);
    base += dg << sh;
    width = uint64_t(1) << sh;
    __builtin_amdgcn_wave_barrier();
  }
  *krem_out = krem;
  return base;
}

// The score a selection key stands for (score_key inverted; with 16-bit keys
// the score was rounded to bf16, so its low 16 bits are zero). -0 comes back
// as +0, which compares equal.
__device__ __forceinline__ float key_score(uint32_t k, bool key16) {
  uint32_t u;
  if (key16) u = (k & 0x8000u) ? (k & 0x7fffu) << 16 : (~k & 0xffffu) << 16;
  else u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// One workgroup per row: the selection from the chunks' candidates. chunk:
// scores per chunk (the row has ceil(n / chunk) chunks); e_off: where a
// chunk's equal list starts in its slots (0: right after its above list);
// have_scores: the row's scores are in memory (the full passes can run).
__global__ __launch_bounds__(kFiltThreads) void topk_final_kernel(
    const float* __restrict__ scores, int64_t ld, FiltWs fw, int64_t N_cap, int Tq, int t_off, int Tc,
    int64_t q_pos0, const int64_t* __restrict__ q_pos, int m, int k, bool key16, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, int64_t chunk, int64_t e_off, bool have_scores) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kMaxBins];   // staged keys / histograms
  __shared__ uint32_t preA[kMaxChunks + 1], preE[kMaxChunks + 1];
  __shared__ __attribute__((aligned(16))) uint32_t whist[kFiltThreads / 64][256];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[kFiltThreads / 64];
  __shared__ uint32_t wmx[kFiltThreads / 64];
  __shared__ uint32_t sh_digit, sh_krem, sh_fallback;
  const int tid = threadIdx.x;
  const int wid = tid >> 6;
  // the largest candidate key over the block (hi of the bound kernel is the
  // largest of the maxima it read, which a sampled maxima pass leaves below
  // the row's largest score)
  auto block_max = [&](uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, kWave)));
    if ((tid & 63) == 0) wmx[wid] = x;
    __syncthreads();
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < kFiltThreads / 64; ++w) y = max(y, wmx[w]);
    return y;
  };
  const FiltRow row = filt_row(scores, ld, N_cap, Tq, t_off, Tc, q_pos0, q_pos, m, k, idx_out, score_out);
  if (row.n <= k) {                                      // every visible entry, then -1
    // (rows without stored scores are never this short: the host sends only
    // rows longer than k down that path)
    for (int i = tid; i < k; i += kFiltThreads) {
      row.io[i] = i < row.n ? i : -1;
      if (row.so) row.so[i] = i < row.n && have_scores ? row.s[i] : -INFINITY;
    }
    return;
  }
  const int nch = static_cast<int>((row.n + chunk - 1) / chunk);
  if (nch > kMaxChunks) {                                // (the host keeps the candidate passes within this)
    if (have_scores) select_passes_t<kFiltThreads>(row, k, key16, hist, wsum, &sh_digit, &sh_krem);
    return;
  }
  const uint32_t lo = fw.bound[2 * row.r];
  // per-chunk counts -> exclusive prefixes preA / preE over the chunks
  constexpr int CPT = kMaxChunks / kFiltThreads;
  uint32_t ca[CPT], ce[CPT], sa = 0, se = 0;
  bool ovf = false;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int ch = CPT * tid + q;
    const uint32_t v = ch < nch ? fw.cnt[row.r * fw.nchs + ch] : 0u;
    ovf |= v == kOverflow;
    ca[q] = v == kOverflow ? 0u : v >> 16;
    ce[q] = v == kOverflow ? 0u : v & 0xffffu;
    sa += ca[q];
    se += ce[q];
  }
  if (tid == 0) sh_fallback = 0;
  __syncthreads();
  if (ovf) sh_fallback = 1;
  uint32_t G, E;
  uint32_t ra = block_excl_scan_t<kFiltThreads>(sa, wsum, &G);
  uint32_t re = block_excl_scan_t<kFiltThreads>(se, wsum, &E);
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int ch = CPT * tid + q;
    if (ch <= nch) {
      preA[ch] = ra;
      preE[ch] = re;
    }
    ra += ca[q];
    re += ce[q];
  }
  const bool above = G >= static_cast<uint32_t>(k);      // the k-th largest lies above lo
  __syncthreads();
  if (sh_fallback && have_scores) {                      // a chunk ran out of slots
    select_passes_t<kFiltThreads>(row, k, key16, hist, wsum, &sh_digit, &sh_krem);
    return;
  }
  const int64_t rbase = row.r * fw.nchs;
  const uint32_t* ckr = fw.ckey + rbase * fw.capc;
  const int32_t* cir = fw.cidx + rbase * fw.capc;
  if (above && G <= static_cast<uint32_t>(kFiltThreads * kRunMax)) {
    // the candidates above lo, concatenated over the chunks: this thread's run [p0, p1)
    const uint32_t per = (G + kFiltThreads - 1) / kFiltThreads;
    const uint32_t p0 = min(G, per * tid), p1 = min(G, p0 + per);
    uint32_t rk[kRunMax];
    int32_t rc[kRunMax];
    {
      int ch = p0 < p1 ? chunk_of(preA, nch, p0) : 0;
#pragma unroll
      for (int q = 0; q < kRunMax; ++q) {
        const uint32_t p = p0 + q;
        rc[q] = -1;
        if (p < p1) {
          while (p >= preA[ch + 1]) ++ch;
          rc[q] = static_cast<int32_t>(ch * fw.capc + (p - preA[ch]));
        }
      }
#pragma unroll
      for (int q = 0; q < kRunMax; ++q) rk[q] = rc[q] >= 0 ? ckr[rc[q]] : 0u;
    }
    uint32_t mx = 0;
#pragma unroll
    for (int q = 0; q < kRunMax; ++q) mx = rc[q] >= 0 ? max(mx, rk[q]) : mx;
    const uint32_t hi = block_max(mx);
    uint32_t thr, krem;
    if (G <= static_cast<uint32_t>(kStageKeys)) {
      // stage the keys; every wave finds the k-th largest on its own (no barriers)
#pragma unroll
      for (int q = 0; q < kRunMax; ++q)
        if (rc[q] >= 0) hist[p0 + q] = rk[q];
      __syncthreads();
      thr = wave_kth(hist, static_cast<int>(G), lo + 1u, static_cast<uint64_t>(hi) - lo, static_cast<uint32_t>(k),
                     whist[wid], &krem);
    } else {
      uint32_t base = lo + 1u;
      krem = static_cast<uint32_t>(k);
      uint64_t width = static_cast<uint64_t>(hi) - lo;
      while (width > 1) {
        const int bl = 64 - __builtin_clzll(width - 1);
        const int sh = bl > 12 ? bl - 12 : 0;
        const int nb = static_cast<int>((width - 1) >> sh) + 1;
        for (int i = tid; i < nb; i += kFiltThreads) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kRunMax; ++q) {
          const uint32_t off = rk[q] - base;
          if (rc[q] >= 0 && rk[q] >= base && static_cast<uint64_t>(off) < width) atomicAdd(&hist[off >> sh], 1u);
        }
        __syncthreads();
        find_digit_t<kFiltThreads>(hist, nb, krem, wsum, &sh_digit, &sh_krem);
        base += sh_digit << sh;
        krem = sh_krem;
        width = uint64_t(1) << sh;
      }
      thr = base;
    }
    // ordered output: above thr, then the first krem equal to it, in index order
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int q = 0; q < kRunMax; ++q) {
      gt += rc[q] >= 0 && rk[q] > thr;
      eq += rc[q] >= 0 && rk[q] == thr;
    }
    uint32_t tg, te;
    const uint32_t pg = block_excl_scan_t<kFiltThreads>(gt, wsum, &tg);
    const uint32_t pe = block_excl_scan_t<kFiltThreads>(eq, wsum, &te);
    uint32_t pos = pg + min(pe, krem), eq_rank = pe;
#pragma unroll
    for (int q = 0; q < kRunMax; ++q) {
      if (rc[q] < 0) continue;
      bool take = rk[q] > thr;
      if (rk[q] == thr) take = eq_rank++ < krem;
      if (take && pos < static_cast<uint32_t>(k)) {       // (never past k; the bound keeps a bad row in its row)
        row.io[pos] = cir[rc[q]];
        if (row.so) row.so[pos] = key_score(rk[q], key16);
        ++pos;
      }
    }
    return;
  }
  if (above) {
    // more candidates than the threads hold: streamed from their chunk lists,
    // radix passes over all of them, then the output chunk by chunk
    uint32_t mx = 0;
    for (int ch = 0; ch < nch; ++ch)
      for (uint32_t i = tid; i < preA[ch + 1] - preA[ch]; i += kFiltThreads)
        mx = max(mx, ckr[static_cast<int64_t>(ch) * fw.capc + i]);
    const uint32_t hi = block_max(mx);
    uint32_t base = lo + 1u, krem = static_cast<uint32_t>(k);
    uint64_t width = static_cast<uint64_t>(hi) - lo;
    while (width > 1) {
      const int bl = 64 - __builtin_clzll(width - 1);
      const int sh = bl > 12 ? bl - 12 : 0;
      const int nb = static_cast<int>((width - 1) >> sh) + 1;
      for (int i = tid; i < nb; i += kFiltThreads) hist[i] = 0;
      __syncthreads();
      for (int ch = 0; ch < nch; ++ch)
        for (uint32_t i = tid; i < preA[ch + 1] - preA[ch]; i += kFiltThreads) {
          const uint32_t kk = ckr[static_cast<int64_t>(ch) * fw.capc + i];
          const uint32_t off = kk - base;
          if (kk >= base && static_cast<uint64_t>(off) < width) atomicAdd(&hist[off >> sh], 1u);
        }
      __syncthreads();
      find_digit_t<kFiltThreads>(hist, nb, krem, wsum, &sh_digit, &sh_krem);
      base += sh_digit << sh;
      krem = sh_krem;
      width = uint64_t(1) << sh;
    }
    const uint32_t thr = base;
    uint32_t run_gt = 0, run_eq = 0;
    for (int ch = 0; ch < nch; ++ch) {
      const uint32_t cn = preA[ch + 1] - preA[ch];
      for (uint32_t s0 = 0; s0 < cn; s0 += kFiltThreads) {
        const uint32_t i = s0 + tid;
        const int64_t ci = static_cast<int64_t>(ch) * fw.capc + i;
        const uint32_t kk = i < cn ? ckr[ci] : 0u;
        const uint32_t gt = i < cn && kk > thr, eq = i < cn && kk == thr;
        uint32_t tg, te;
        const uint32_t pg = block_excl_scan_t<kFiltThreads>(gt, wsum, &tg);
        const uint32_t pe = block_excl_scan_t<kFiltThreads>(eq, wsum, &te);
        const uint32_t eq_rank = run_eq + pe;
        const uint32_t pos = run_gt + pg + min(eq_rank, krem);
        if ((gt || (eq && eq_rank < krem)) && pos < static_cast<uint32_t>(k)) {
          row.io[pos] = cir[ci];
          if (row.so) row.so[pos] = key_score(kk, key16);
        }
        run_gt += tg;
        run_eq += te;
      }
    }
    return;
  }
  // The k-th largest is lo: every candidate above lo wins, and the first
  // krem = k - G ties at lo in index order. Chunk ch contributes its A
  // candidates and its first take = clamp(krem - ties before it, 0, E) ties;
  // inside a chunk both lists are in index order, so an entry's position is
  // the chunk's offset plus its rank in its own list plus the entries of the
  // other list below it (a binary search).
  const uint32_t krem = static_cast<uint32_t>(k) - G;
  const float lo_score = key_score(lo, key16);
  for (int ch = wid; ch < nch; ch += kFiltThreads / 64) {
    const uint32_t a_n = preA[ch + 1] - preA[ch];
    const uint32_t eb = preE[ch], e_n = preE[ch + 1] - eb;
    const uint32_t t_n = eb >= krem ? 0u : min(e_n, krem - eb);
    if (a_n + t_n == 0) continue;
    const uint32_t off = preA[ch] + min(eb, krem);       // winners before this chunk
    const int32_t* ii = cir + static_cast<int64_t>(ch) * fw.capc;
    const uint32_t* kk = ckr + static_cast<int64_t>(ch) * fw.capc;
    const int32_t* ties = ii + (e_off ? e_off : static_cast<int64_t>(a_n));
    for (uint32_t i = tid & 63; i < a_n + t_n; i += kWave) {
      const bool is_a = i < a_n;
      const uint32_t r = is_a ? i : i - a_n;
      const int32_t x = is_a ? ii[r] : ties[r];
      const int32_t* other = is_a ? ties : ii;            // entries of the other list below x
      uint32_t lo_i = 0, hi_i = is_a ? t_n : a_n;
      while (lo_i < hi_i) {
        const uint32_t mid = (lo_i + hi_i) >> 1;
        if (other[mid] < x) lo_i = mid + 1;
        else hi_i = mid;
      }
      const uint32_t pos = off + r + lo_i;
      if (pos >= static_cast<uint32_t>(k)) continue;
      row.io[pos] = x;
      if (row.so) row.so[pos] = is_a ? key_score(kk[r], key16) : lo_score;
    }
  }
}

template <int MT>
void launch_score_bf16_wide(LaunchScope& ls, const IndexArgs& a, float* sc, int64_t ld, int t_off, int Tc,
                            dim3 grid, SelAux aux) {
  const bool rb = (a.flags & LCA_SCORE_BF16) != 0;
  const uint16_t* q = static_cast<const uint16_t*>(a.qI);
  const uint16_t* k = static_cast<const uint16_t*>(a.kI);
  switch (a.d_I) {
    case 64: ls.launch(index_score_bf16_wide_kernel<MT, 64>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
    case 128: ls.launch(index_score_bf16_wide_kernel<MT, 128>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
    case 256: ls.launch(index_score_bf16_wide_kernel<MT, 256>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
    default: ls.launch(index_score_bf16_wide_kernel<MT, 32>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
  }
}

template <int HI>
void launch_score_bf16_hi(LaunchScope& ls, const IndexArgs& a, float* sc, int64_t ld, int t_off, int Tc,
                          dim3 grid, SelAux aux) {
  const bool rb = (a.flags & LCA_SCORE_BF16) != 0;
  const uint16_t* q = static_cast<const uint16_t*>(a.qI);
  const uint16_t* k = static_cast<const uint16_t*>(a.kI);
  switch (a.d_I) {
    case 64: ls.launch(index_score_bf16_kernel<HI, 64>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
    case 128: ls.launch(index_score_bf16_kernel<HI, 128>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
    case 256: ls.launch(index_score_bf16_kernel<HI, 256>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
    default: ls.launch(index_score_bf16_kernel<HI, 32>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb, aux); break;
  }
}

// row stride of the score buffer: 64-element aligned for vector loads
int64_t score_ld(const IndexArgs& a) { return (a.N_cap + 63) / 64 * 64; }

// Bytes per query row of the workspace beyond the scores: group maxima,
// candidates of the chunked select (slots per chunk capc), counts, bound, counter.
// candidate slots per chunk: the whole chunk for lists of up to 4 register
// rounds (no overflow), an eighth of it for longer ones
int filt_capc(int64_t ld) { return ld <= 4 * int64_t(kRound) ? kFiltChunk : kFiltChunk / 8; }
int64_t filt_nchs(int64_t ld) { return (ld + kFiltChunk - 1) / kFiltChunk; }
int64_t filt_row_bytes(int64_t ld) {
  return ld / kGroup * 4 + filt_nchs(ld) * (filt_capc(ld) * int64_t(8) + 4) + 8;
}

// Whether a chunk may take topk_select_long_kernel (which needs a spill row
// per query): a list longer than one round whose group bound would be too
// weak for k (the chunked select's condition, taken at the shortest such
// list), or tiled scoring without group maxima.
bool long_old_possible(const IndexArgs& a) {
  if (a.N_cap <= kRound) return false;
  const int64_t ng = (kRound + 1 + kGroup - 1) / kGroup;
  return ng / 4 < 2 * ((a.k + 3) / 4) || (a.dt == LCA_BF16 && a.d_I == 128 && a.H_I == 1);
}

// The prefill path that stores no scores: tiled scoring writes only the group
// maxima, topk_bound_kernel takes each row's bound from them, tiled scoring
// runs again and writes only each row's candidates against its bound (per key
// range of a workgroup, with room for the whole range, so nothing overflows),
// and topk_final_kernel selects. Writing and reading every score costs more
// than the second pass of MFMA scoring. For calls of many queries (the tiled
// kernel, bf16 keys of 128 channels, H_I >= 2, its staged tile), one position
// for the batch, long lists, and every row longer than k (so every output
// score comes from a candidate's key).
bool cand_mode(const IndexArgs& a) {
  if (!(a.dt == LCA_BF16 && a.d_I == 128 && a.H_I >= 2 && a.H_I <= 16 && a.Tq >= kTiledMinQueries && !a.q_pos))
    return false;
  int64_t nv0 = n_visible(a.q_pos0, a.m), nv1 = n_visible(a.q_pos0 + a.Tq - 1, a.m);
  if (nv0 > a.N_cap) nv0 = a.N_cap;
  if (nv1 > a.N_cap) nv1 = a.N_cap;
  return nv0 > a.k && nv1 > kRound;
}

// key ranges of the tiled kernel: about 2048 workgroups over (keys, queries);
// in candidate mode at most kMaxChunks ranges (the final kernel's count
// table) of at most 32768 keys (the counts pack in 16 bits)
void tiled_ranges(const IndexArgs& a, int64_t nv_max, int tcn, bool cands, int64_t* kc_out, int64_t* per_out,
                  int ss = 1) {
  const int qpwg = 4 * 4 * (16 / a.H_I);
  const int64_t n_qt = (tcn + qpwg - 1) / qpwg;
  int64_t kc = (2048 + n_qt * a.B - 1) / (n_qt * a.B);
  const int64_t kc_max = (nv_max + 255) / 256;
  if (kc > kc_max) kc = kc_max;
  if (cands) {
    if (kc < (nv_max + 32767) / 32768) kc = (nv_max + 32767) / 32768;
    if (kc > kMaxChunks) kc = kMaxChunks;
  }
  if (kc < 1) kc = 1;
  int64_t per = (nv_max + kc - 1) / kc;
  const int64_t span = int64_t(kTileKeys) * ss;     // whole sampling periods per range
  per = (per + span - 1) / span * span;
  *kc_out = (nv_max + per - 1) / per;
  *per_out = per;
}

// The maxima pass of candidate mode scores every ss-th tile of 64 keys. The
// bound from those maxima is looser (about ss times the candidates, whose
// exact comparisons and stores the candidate pass pays), so ss grows only
// while the shortest row of the chunk keeps at least kSampleGroups k sampled
// groups, and to 2 at most (1M-token prefill, per step: 4.80 ms at 1, 4.53 at
// 2, 4.70 at 4).
constexpr int kMaxSample = 2;
constexpr int kSampleGroups = 3;
int maxima_sample(const IndexArgs& a, int64_t nv_min) {
  int ss = 1;
  while (ss < kMaxSample && nv_min / (int64_t(kTileKeys) * 2 * ss) * 4 >= int64_t(kSampleGroups) * a.k) ss *= 2;
  return ss;
}

// candidate slots per row in candidate mode: 2 per key of every range
// (kc * per <= nv + 64 kc and per >= 256, so under 2.5 ld)
int64_t cand_slots(int64_t ld) { return (ld * 5 + 1) / 2 + 2 * kTileKeys; }

// queries per chunk so that the score buffer and the select's side arrays stay
// under a fixed budget (in candidate mode: the candidate slots, in whole tiles
// of queries)
int query_chunk(const IndexArgs& a) {
  const int64_t ld = score_ld(a);
  const bool cm = cand_mode(a);
  const int64_t per_q = cm ? static_cast<int64_t>(a.B) * (ld / kGroup * 4 + 8 + kMaxChunks * 4 + cand_slots(ld) * 8)
                           : static_cast<int64_t>(a.B) * (ld * (long_old_possible(a) ? 8 : 4) + filt_row_bytes(ld));
  const int64_t budget = cm ? int64_t(4) << 30 : int64_t(640) << 20;
  int64_t tc = per_q > 0 ? budget / per_q : a.Tq;
  if (tc < 1) tc = 1;
  if (tc > a.Tq) tc = a.Tq;
  const int gran = cm ? kTiledMinQueries : 16;
  if (tc < a.Tq && tc >= gran) tc -= tc % gran;      // whole query tiles per chunk
  return static_cast<int>(tc);
}

// Workspace regions (each 256-byte aligned) for a chunk of Tc queries.
struct IndexWs {
  float* sc;
  int32_t* spill;
  FiltWs fw;
  size_t bytes;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

IndexWs index_ws(const IndexArgs& a, void* base) {
  const int Tc = query_chunk(a);
  const bool cm = cand_mode(a);
  const int64_t ld = score_ld(a), rows = static_cast<int64_t>(a.B) * Tc;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) { char* q = p ? p + off : nullptr; off += align256(n); return q; };
  IndexWs w;
  w.sc = reinterpret_cast<float*>(take(cm ? 0 : rows * ld * 4));
  w.spill = reinterpret_cast<int32_t*>(take(!cm && long_old_possible(a) ? rows * ld * 4 : 0));
  w.fw.ldg = ld / kGroup;
  w.fw.nchs = cm ? kMaxChunks : static_cast<int>(filt_nchs(ld));
  w.fw.capc = filt_capc(ld);
  const int64_t slots = cm ? cand_slots(ld) : w.fw.nchs * int64_t(w.fw.capc);   // per row
  w.fw.gmax = reinterpret_cast<float*>(take(rows * w.fw.ldg * 4));
  w.fw.ckey = reinterpret_cast<uint32_t*>(take(rows * slots * 4));
  w.fw.cidx = reinterpret_cast<int32_t*>(take(rows * slots * 4));
  w.fw.cnt = reinterpret_cast<uint32_t*>(take(rows * w.fw.nchs * 4));
  w.fw.bound = reinterpret_cast<uint32_t*>(take(rows * 8));
  w.fw.lim = reinterpret_cast<uint32_t*>(take(rows * 4));
  w.bytes = off + 256;
  return w;
}

}  // namespace

size_t index_topk_workspace(const IndexArgs& a) { return index_ws(a, nullptr).bytes; }

template <int MODE>
void launch_tiled(LaunchScope& scope, const IndexArgs& a, int64_t kc, int tcn, float* sc, int64_t ld, int t_off,
                  int Tc, int64_t per, bool key16, SelAux aux, int ss = 1) {
  const uint16_t* q = static_cast<const uint16_t*>(a.qI);
  const uint16_t* k = static_cast<const uint16_t*>(a.kI);
  const int qpwg = 4 * 4 * (16 / a.H_I);
  const int nq = (tcn + qpwg - 1) / qpwg;
  const int64_t pairs = (kc * a.B + 7) / 8 * 8;        // (sequence, key range) pairs, padded
  const dim3 grid(static_cast<uint32_t>(pairs * nq));
  const int kci = static_cast<int>(kc);
#define LCA_TILED(H)                                                                                         \
  (key16 ? scope.launch(index_score_tiled_kernel<H, MODE, true>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, \
                        a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, per, aux, kci, nq, a.B, ss)             \
         : scope.launch(index_score_tiled_kernel<H, MODE, false>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, \
                        a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, per, aux, kci, nq, a.B, ss))
  switch (a.H_I) {
    case 1:
      if constexpr (MODE == kTiledScores) LCA_TILED(1);
      break;
    case 2: LCA_TILED(2); break;
    case 4: LCA_TILED(4); break;
    case 8: LCA_TILED(8); break;
    default: LCA_TILED(16); break;
  }
#undef LCA_TILED
}

// The select of one chunk of queries whose longest list is nv_max: the
// chunked select serves lists longer than one register round (one workgroup
// per query is quicker below that: each extra kernel in the chain costs its
// own latency); it needs the group maxima (every scoring path but the tiled
// one at H_I = 1 writes them) and enough groups per wave share for a bound
// well above the smallest score.
bool use_chunked(const IndexArgs& a, int64_t nv_max, bool tiled) {
  const int64_t ng_max = (nv_max + kGroup - 1) / kGroup;
  return nv_max > kRound && !(tiled && a.H_I == 1) && nv_max > a.k && ng_max / 4 >= 2 * ((a.k + 3) / 4);
}

hipError_t launch_index_topk(hipStream_t s, const IndexArgs& a, void* ws, size_t) {
  const IndexWs w = index_ws(a, ws);
  float* sc = w.sc;
  const int Tc = query_chunk(a);
  const int64_t ld = score_ld(a);
  const bool key16 = (a.flags & LCA_SCORE_BF16) != 0;
  // before anything is enqueued: every chunk that takes the long select has its spill rows
  for (int t_off = 0; t_off < a.Tq; t_off += Tc) {
    const int tcn = min(Tc, a.Tq - t_off);
    int64_t nv_max = n_visible(a.q_pos0 + t_off + tcn - 1, a.m);
    if (nv_max > a.N_cap) nv_max = a.N_cap;
    const bool tiled = a.dt == LCA_BF16 && a.d_I == 128 && a.H_I <= 16 && tcn >= kTiledMinQueries;
    if (nv_max > kRound && nv_max > a.k && !use_chunked(a, nv_max, tiled) && !long_old_possible(a))
      return hipErrorInvalidValue;
  }
  const bool cm = cand_mode(a);
  for (int t_off = 0; t_off < a.Tq; t_off += Tc) {
    const int tcn = min(Tc, a.Tq - t_off);
    int64_t nv_max = n_visible(a.q_pos0 + t_off + tcn - 1, a.m);
    if (nv_max > a.N_cap) nv_max = a.N_cap;
    if (cm) {
      // no scores stored: maxima (of every ss-th tile), bound, candidates, final
      int64_t nv_min = n_visible(a.q_pos0 + t_off, a.m);
      if (nv_min > a.N_cap) nv_min = a.N_cap;
      const int ss = maxima_sample(a, nv_min);
      int64_t kc, per;
      tiled_ranges(a, nv_max, tcn, true, &kc, &per, ss);
      FiltWs fw = w.fw;
      fw.nchs = static_cast<int>(kc);
      fw.capc = static_cast<int>(2 * per);
      SelAux aux{fw.gmax, fw.ldg, fw.bound, fw.ckey, fw.cidx, fw.cnt, fw.nchs, fw.capc, fw.lim};
      {
        LaunchScope scope(s, "index_score");
        launch_tiled<kTiledMaxima>(scope, a, kc, tcn, nullptr, ld, t_off, Tc, per, key16, aux, ss);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      {
        LaunchScope scope(s, "topk_select");
        scope.launch(topk_bound_kernel, dim3(1, tcn, a.B), dim3(kFiltThreads), 0, fw, a.N_cap, Tc, a.q_pos0,
                     a.q_pos, t_off, a.m, a.k, key16, ss);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      {
        LaunchScope scope(s, "index_score");
        launch_tiled<kTiledCands>(scope, a, kc, tcn, nullptr, ld, t_off, Tc, per, key16, aux);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      {
        LaunchScope scope(s, "topk_select");
        scope.launch(topk_final_kernel, dim3(1, tcn, a.B), dim3(kFiltThreads), 0, static_cast<const float*>(nullptr),
                     ld, fw, a.N_cap, a.Tq, t_off, Tc, a.q_pos0, a.q_pos, a.m, a.k, key16, a.idx_out, a.score_out,
                     per, per, false);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      continue;
    }
    const bool tiled = a.dt == LCA_BF16 && a.d_I == 128 && a.H_I <= 16 && tcn >= kTiledMinQueries;
    const int64_t ng_max = (nv_max + kGroup - 1) / kGroup;
    const bool filt = use_chunked(a, nv_max, tiled);
    SelAux aux{filt ? w.fw.gmax : nullptr, w.fw.ldg, nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr};
    if (nv_max > 0) {
      LaunchScope scope(s, "index_score");
      if (a.dt == LCA_F32) {
        dim3 grid((nv_max + kScoreThreads - 1) / kScoreThreads, tcn, a.B);
        scope.launch(index_score_f32_kernel, grid, dim3(kScoreThreads),
                     static_cast<uint32_t>((a.H_I * a.d_I + a.H_I) * sizeof(float)),
                           static_cast<const float*>(a.qI), a.w, static_cast<const float*>(a.kI), sc, ld,
                           a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, a.H_I, a.d_I, key16, aux);
      } else if (a.dt == LCA_MXFP4 && a.H_I > 16) {
        dim3 grid((nv_max + kFp4KeysPerWG - 1) / kFp4KeysPerWG, tcn, a.B);
        const uint8_t* q = static_cast<const uint8_t*>(a.qI);
        const uint8_t* qs = static_cast<const uint8_t*>(a.qI_scale);
        const uint8_t* k = static_cast<const uint8_t*>(a.kI);
        const uint8_t* ks = static_cast<const uint8_t*>(a.kI_scale);
        if (a.H_I == 32)
          scope.launch(index_score_fp4_wide_kernel<2>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16, aux);
        else
          scope.launch(index_score_fp4_wide_kernel<4>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16, aux);
      } else if (a.dt == LCA_MXFP4) {
        const int QPB = 16 / a.H_I;
        dim3 grid((nv_max + kFp4KeysPerWG - 1) / kFp4KeysPerWG, (tcn + QPB - 1) / QPB, a.B);
        const uint8_t* q = static_cast<const uint8_t*>(a.qI);
        const uint8_t* qs = static_cast<const uint8_t*>(a.qI_scale);
        const uint8_t* k = static_cast<const uint8_t*>(a.kI);
        const uint8_t* ks = static_cast<const uint8_t*>(a.kI_scale);
        switch (a.H_I) {
          case 1: scope.launch(index_score_fp4_kernel<1>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16, aux); break;
          case 2: scope.launch(index_score_fp4_kernel<2>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16, aux); break;
          case 4: scope.launch(index_score_fp4_kernel<4>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16, aux); break;
          case 8: scope.launch(index_score_fp4_kernel<8>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16, aux); break;
          default: scope.launch(index_score_fp4_kernel<16>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16, aux); break;
        }
      } else if (tiled) {
        // many queries: key tiles through LDS, ~2048 workgroups over (keys, queries)
        int64_t kc, per;
        tiled_ranges(a, nv_max, tcn, false, &kc, &per);
        launch_tiled<kTiledScores>(scope, a, kc, tcn, sc, ld, t_off, Tc, per, key16, aux);
      } else if (a.H_I > 16) {
        // 32 or 64 heads: one query per grid row
        dim3 grid((nv_max + kKeysPerWG - 1) / kKeysPerWG, tcn, a.B);
        if (a.H_I == 32) launch_score_bf16_wide<2>(scope, a, sc, ld, t_off, Tc, grid, aux);
        else launch_score_bf16_wide<4>(scope, a, sc, ld, t_off, Tc, grid, aux);
      } else {
        const int QPB = 16 / a.H_I;
        dim3 grid((nv_max + kKeysPerWG - 1) / kKeysPerWG, (tcn + QPB - 1) / QPB, a.B);
        switch (a.H_I) {
          case 1: launch_score_bf16_hi<1>(scope, a, sc, ld, t_off, Tc, grid, aux); break;
          case 2: launch_score_bf16_hi<2>(scope, a, sc, ld, t_off, Tc, grid, aux); break;
          case 4: launch_score_bf16_hi<4>(scope, a, sc, ld, t_off, Tc, grid, aux); break;
          case 8: launch_score_bf16_hi<8>(scope, a, sc, ld, t_off, Tc, grid, aux); break;
          default: launch_score_bf16_hi<16>(scope, a, sc, ld, t_off, Tc, grid, aux); break;
        }
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      LaunchScope scope(s, "topk_select");
      if (filt) {
        const dim3 grid(static_cast<uint32_t>((nv_max + kFiltChunk - 1) / kFiltChunk), tcn, a.B);
        const float* scs = sc;
        if (ng_max <= int64_t(4 * kWave) * kInlineItems) {
          scope.launch(topk_chunk_kernel<kInlineItems>, grid, dim3(kFiltThreads), 0, scs, ld, w.fw, a.N_cap, a.Tq,
                       t_off, Tc, a.q_pos0, a.q_pos, a.m, a.k, key16);
        } else {
          scope.launch(topk_bound_kernel, dim3(1, tcn, a.B), dim3(kFiltThreads), 0, w.fw, a.N_cap, Tc, a.q_pos0,
                       a.q_pos, t_off, a.m, a.k, key16, 1);
          scope.launch(topk_chunk_kernel<0>, grid, dim3(kFiltThreads), 0, scs, ld, w.fw, a.N_cap, a.Tq, t_off, Tc,
                       a.q_pos0, a.q_pos, a.m, a.k, key16);
        }
        scope.launch(topk_final_kernel, dim3(1, tcn, a.B), dim3(kFiltThreads), 0, scs, ld, w.fw, a.N_cap, a.Tq,
                     t_off, Tc, a.q_pos0, a.q_pos, a.m, a.k, key16, a.idx_out, a.score_out,
                     static_cast<int64_t>(kFiltChunk), static_cast<int64_t>(0), true);
      } else if (nv_max > kRound) {
        // every row's list is at most nv_max long (and nv_max > kRound implies N_cap > kRound)
        scope.launch(topk_select_long_kernel, dim3(tcn, a.B), dim3(kSelThreads), 0, static_cast<const float*>(sc), ld,
                     w.spill, a.N_cap, a.Tq, t_off, Tc, a.q_pos0, a.q_pos, a.m, a.k, key16, a.idx_out, a.score_out);
      } else {
        scope.launch(topk_select_kernel, dim3(tcn, a.B), dim3(kSelThreads), 0, static_cast<const float*>(sc), ld,
                     a.N_cap, a.Tq, t_off, Tc, a.q_pos0, a.q_pos, a.m, a.k, key16, a.idx_out, a.score_out);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace lca
