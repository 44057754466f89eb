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
// scores). Up to 32768 scores stay in registers (32 per thread, loaded once,
// all loads in flight together); longer lists are processed in rounds of
// 32768. An order-preserving compaction follows: output indices come out in
// increasing order and ties at the threshold go to the lowest indices, so the
// result is deterministic.
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

// Scores of key j from one 16 x 16 MFMA tile: accumulator row 4g + i is the
// dot of (query tq0 + (4g+i) / HI, head (4g+i) % HI) with key j. ReLU, the
// head weights and the head sum are folded here, in the same order for every
// operand type: ((p0 + p1) + (p2 + p3)), then across lane groups for HI >= 8.
template <int HI>
__device__ __forceinline__ void emit_scores(const f32x4& acc, const float (&wv)[4], const int64_t (&nvq)[4], int g,
                                            int tq0, int t_off, int t_end, int64_t j, float* srow, int64_t ld,
                                            bool round_bf16) {
  float part[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) part[i] = wv[i] * fmaxf(acc[i], 0.f);
  if constexpr (HI == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qt = tq0 + 4 * g + i;
      if (qt < t_end && j < nvq[i]) srow[(qt - t_off) * ld + j] = round_bf16 ? bf16_round(part[i]) : part[i];
    }
  } else if constexpr (HI == 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int qt = tq0 + 2 * g + p;
      const float sc = part[2 * p] + part[2 * p + 1];
      if (qt < t_end && j < nvq[2 * p]) srow[(qt - t_off) * ld + j] = round_bf16 ? bf16_round(sc) : sc;
    }
  } else {
    float sc = (part[0] + part[1]) + (part[2] + part[3]);
    if constexpr (HI >= 8) sc += __shfl_xor(sc, 16, 64);
    if constexpr (HI >= 16) sc += __shfl_xor(sc, 32, 64);
    const int qt = tq0 + (4 * g) / HI;
    const bool writer = (g % (HI / 4 > 0 ? HI / 4 : 1)) == 0;
    if (writer && qt < t_end && j < nvq[0]) srow[(qt - t_off) * ld + j] = round_bf16 ? bf16_round(sc) : sc;
  }
}

// As emit_scores, but into the wave's LDS staging block (row = query of the
// wave, column = key of the tile) instead of the score rows: the block is then
// written out as 256-byte row segments (see index_score_tiled_kernel). HI >= 2.
constexpr int kStageStride = 80;     // floats per staged query row (64 keys + bank shift)
template <int HI>
__device__ __forceinline__ void stage_scores(const f32x4& acc, const float (&wv)[4], int g, int q0, int col,
                                             float* stage, bool round_bf16) {
  float part[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) part[i] = wv[i] * fmaxf(acc[i], 0.f);
  if constexpr (HI == 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float sc = part[2 * p] + part[2 * p + 1];
      stage[(q0 + 2 * g + p) * kStageStride + col] = round_bf16 ? bf16_round(sc) : sc;
    }
  } else {
    float sc = (part[0] + part[1]) + (part[2] + part[3]);
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
    const int64_t* __restrict__ q_pos, int m, bool round_bf16) {
  constexpr int QPB = 16 / HI;       // queries per M tile
  constexpr int KS = DI / 32;        // K steps
  constexpr int UNR = kKeysPerWave / 16;
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
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[s], __builtin_bit_cast(bf16x8, kv[u][s]), acc, 0, 0, 0);
    pin_uniform(acc);
    emit_scores<HI>(acc, wv, nvq, g, tq0, t_off, t_end, key0 + 16 * u + r16,
                    scores + static_cast<int64_t>(b) * Tc * ld, ld, round_bf16);
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

template <int HI>
__global__ __launch_bounds__(kScoreThreads) void index_score_tiled_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const uint16_t* __restrict__ kI,
    float* __restrict__ scores, int64_t ld, int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0,
    const int64_t* __restrict__ q_pos, int m, int64_t keys_per_wg, bool round_bf16) {
  constexpr int DI = 128, KS = DI / 32, MB = 4, NB = kTileKeys / 16, QPB = 16 / HI;
  constexpr int QPW = MB * QPB, QPWG = 4 * QPW;
  constexpr int ROWB = DI * 2;                       // bytes per key row
  constexpr bool kStaged = HI >= 2;                  // HI = 1: 64 queries per wave, stored directly
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[2][kTileKeys * DI];
  __shared__ __attribute__((aligned(16))) float St[4][kStaged ? QPW * kStageStride : 4];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int b = blockIdx.z;
  q_pos0 = seq_pos(q_pos, q_pos0, b);                // this sequence's position
  const int t_end = min(Tq, t_off + Tc);
  const int tw0 = t_off + static_cast<int>(blockIdx.y) * QPWG;
  if (tw0 >= t_end) return;
  int64_t nv_max = n_visible(q_pos0 + min(tw0 + QPWG, t_end) - 1, m);
  if (nv_max > N_cap) nv_max = N_cap;
  const int64_t k_begin = static_cast<int64_t>(blockIdx.x) * keys_per_wg;
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
      int64_t nv = q2 < t_end ? n_visible(q_pos0 + q2, m) : 0;
      nvq[mb][i] = nv < k_end ? nv : k_end;        // this workgroup scores keys < k_end only
    }
  }
  float* srow = scores + static_cast<int64_t>(b) * Tc * ld;
  const int slot_r = r16;                          // key & 15 of the keys this lane reads

  for (int tt = 0; tt < ntiles; ++tt) {
    // tile tt has landed (every wave waited for its own copies) and every wave
    // is done with the buffer that tile tt + 1 overwrites
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (tt + 1 < ntiles) issue(tt + 1, (tt + 1) & 1);
    const char* xb = reinterpret_cast<const char*>(&Ks[tt & 1][0]);
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
        if constexpr (kStaged)
          stage_scores<HI>(acc[mb], wv[mb], g, mb * QPB, nb * 16 + r16, St[wid], round_bf16);
        else
          emit_scores<HI>(acc[mb], wv[mb], nvq[mb], g, tw0 + wid * QPW + mb * QPB, t_off, t_end, j, srow, ld,
                          round_bf16);
      }
    }
    if constexpr (kStaged) {
      // The wave's QPW x 64 tile of scores leaves as 16-byte stores, 16 lanes
      // per 256-byte row segment. Every key of the tile is written: cells past
      // a query's visible count lie inside its row (the stride is a multiple of
      // 64, tiles start at multiples of 64 within this workgroup's key range)
      // and the top-k never reads them. Queries past the chunk are skipped.
      wait_lgkmcnt0();                              // the wave's staging writes have landed
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const int64_t jt0 = k_begin + static_cast<int64_t>(tt) * kTileKeys;
#pragma unroll
      for (int i = 0; i < QPW / 4; ++i) {
        const int u = i * 64 + lane, row = u >> 4, c4 = u & 15;
        const int qt = tw0 + wid * QPW + row;
        const float4 v = *reinterpret_cast<const float4*>(&St[wid][row * kStageStride + 4 * c4]);
        if (qt < t_end) *reinterpret_cast<float4*>(srow + static_cast<int64_t>(qt - t_off) * ld + jt0 + 4 * c4) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // reads done before the next tile's staging
    }
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
    bool round_bf16) {
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
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const i32x8 Bk = {static_cast<int>(kc[u].x), static_cast<int>(kc[u].y), static_cast<int>(kc[u].z),
                      static_cast<int>(kc[u].w), 0, 0, 0, 0};
    const int sb = static_cast<int>((ks[u] >> (8 * g)) & 0xffu);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bk, acc, 4, 4, 0, qs, 0, sb);
    pin_uniform(acc);
    emit_scores<HI>(acc, wv, nvq, g, tq0, t_off, t_end, key0 + 16 * u + r16,
                    scores + static_cast<int64_t>(b) * Tc * ld, ld, round_bf16);
  }
}

// ---------------------------------------------------------------------------
// float32 scoring on the vector ALUs (small fp32 layers)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScoreThreads) void index_score_f32_kernel(
    const float* __restrict__ qI, const float* __restrict__ w, const float* __restrict__ kI,
    float* __restrict__ scores, int64_t ld, int Tq, int t_off, int Tc, int64_t N_cap, int64_t q_pos0,
    const int64_t* __restrict__ q_pos, int m, int HI, int DI, bool round_bf16) {
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
  if (j >= nv) return;
  const float* kr = kI + (static_cast<int64_t>(b) * N_cap + j) * DI;
  float sc = 0.f;
  for (int h = 0; h < HI; ++h) {
    float dot = 0.f;
    for (int d = 0; d < DI; ++d) dot = fmaf(qs[h * DI + d], kr[d], dot);
    sc += qs[HI * DI + h] * fmaxf(dot, 0.f);
  }
  if (round_bf16) sc = bf16_round(sc);
  scores[(static_cast<int64_t>(b) * Tc + tl) * ld + j] = sc;
}

// ---------------------------------------------------------------------------
// Radix select + ordered compaction
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelItems = 32;                   // scores per thread per round
constexpr int kRound = kSelThreads * kSelItems; // scores per round (registers)
constexpr int kMaxBins = 4096;

// Order-preserving key: larger score -> larger unsigned key; -0 folds into +0.
// Key 0 never comes from a real number (it would be a NaN pattern), so it
// marks "no element" below.
__device__ __forceinline__ uint32_t score_key(float v, bool key16) {
  if (v == 0.f) v = 0.f;
  const uint32_t u = __float_as_uint(v);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key16 ? (k >> 16) : k;
}

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
// at or above it, and the k-th largest score is at or above `lo`. Only the
// scores from `lo` up (a few percent of a list, typically) are candidates:
// they go to LDS in increasing index order, and their digits are taken on the
// offset key - lo over [lo, max key] (12 bits at a time, from the top), which
// spreads them over the bins where the raw key's top digit would stack them
// into one or two (a float's sign and exponent). Same threshold, same ties in
// index order, same output as the full passes. Returns false, having written
// nothing, when the candidates exceed kCandCap.
constexpr int kCandCap = 4096;
constexpr int kCandPer = kCandCap / kSelThreads;

__device__ __forceinline__ bool select_filtered(const SelRow& row, int k, bool key16,
                                                const uint32_t (&key)[kSelItems], uint32_t* hist, uint32_t* wsum,
                                                uint32_t* ckey, int32_t* cidx, uint32_t* sh_digit_p,
                                                uint32_t* sh_krem_p, uint32_t* sh_hi_p) {
  uint32_t& sh_digit = *sh_digit_p;
  uint32_t& sh_krem = *sh_krem_p;
  const int tid = threadIdx.x;
  const int top = key16 ? 4 : 20;                  // shift of the key's top 12-bit digit
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < kSelItems; ++j) mx = max(mx, key[j]);
  uint32_t wmx = mx;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wmx = max(wmx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(wmx), o, kWave)));
  for (int i = tid; i < kMaxBins; i += kSelThreads) hist[i] = 0;
  if (tid == 0) *sh_hi_p = 0;
  __syncthreads();
  if (mx != 0u) atomicAdd(&hist[mx >> top], 1u);
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
  __shared__ uint32_t hist[kMaxBins];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[kSelThreads / 64];
  __shared__ __attribute__((aligned(16))) uint32_t ckey[kCandCap];
  __shared__ int32_t cidx[kCandCap];
  __shared__ uint32_t sh_digit, sh_krem, sh_hi;
  const SelRow row = sel_row(scores, ld, N_cap, Tq, t_off, Tc, q_pos0, q_pos, m, k, idx_out, score_out);
  if (row.n <= k) {
    select_all(row, k);
    return;
  }
  // threads holding a score: (n + kSelItems - 1) / kSelItems, one round (n <= kRound here)
  if ((row.n + kSelItems - 1) / kSelItems >= 2 * static_cast<int64_t>(k)) {
    uint32_t key[kSelItems];
    load_round(row.s, row.n, 0, key16, key);
    if (select_filtered(row, k, key16, key, hist, wsum, ckey, cidx, &sh_digit, &sh_krem, &sh_hi)) return;
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

template <int HI>
void launch_score_bf16_hi(LaunchScope& ls, const IndexArgs& a, float* sc, int64_t ld, int t_off, int Tc,
                          dim3 grid) {
  const bool rb = (a.flags & LCA_SCORE_BF16) != 0;
  const uint16_t* q = static_cast<const uint16_t*>(a.qI);
  const uint16_t* k = static_cast<const uint16_t*>(a.kI);
  switch (a.d_I) {
    case 64: ls.launch(index_score_bf16_kernel<HI, 64>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb); break;
    case 128: ls.launch(index_score_bf16_kernel<HI, 128>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb); break;
    case 256: ls.launch(index_score_bf16_kernel<HI, 256>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb); break;
    default: ls.launch(index_score_bf16_kernel<HI, 32>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, rb); break;
  }
}

// row stride of the score buffer: 64-element aligned for vector loads
int64_t score_ld(const IndexArgs& a) { return (a.N_cap + 63) / 64 * 64; }

// queries per chunk so that the score buffer stays under a fixed budget
int query_chunk(const IndexArgs& a) {
  const int64_t per_q = static_cast<int64_t>(a.B) * score_ld(a) * 4;
  const int64_t budget = int64_t(512) << 20;
  int64_t tc = per_q > 0 ? budget / per_q : a.Tq;
  if (tc < 1) tc = 1;
  if (tc > a.Tq) tc = a.Tq;
  if (tc < a.Tq && tc >= 16) tc -= tc % 16;          // whole M tiles per chunk
  return static_cast<int>(tc);
}

}  // namespace

// Workspace: the chunk's scores [B, Tc, ld] (float32); for lists longer than
// one register round, then the select's spill buffer [B, Tc, ld] (int32).
bool long_lists(const IndexArgs& a) { return a.N_cap > kRound; }

size_t index_topk_workspace(const IndexArgs& a) {
  const size_t cells = static_cast<size_t>(a.B) * query_chunk(a) * score_ld(a);
  return cells * (sizeof(float) + (long_lists(a) ? sizeof(int32_t) : 0)) + 256;
}

hipError_t launch_index_topk(hipStream_t s, const IndexArgs& a, void* ws, size_t) {
  float* sc = static_cast<float*>(ws);
  const int Tc = query_chunk(a);
  const int64_t ld = score_ld(a);
  int32_t* spill = reinterpret_cast<int32_t*>(sc + static_cast<int64_t>(a.B) * Tc * ld);
  const bool key16 = (a.flags & LCA_SCORE_BF16) != 0;
  for (int t_off = 0; t_off < a.Tq; t_off += Tc) {
    const int tcn = min(Tc, a.Tq - t_off);
    int64_t nv_max = n_visible(a.q_pos0 + t_off + tcn - 1, a.m);
    if (nv_max > a.N_cap) nv_max = a.N_cap;
    if (nv_max > 0) {
      LaunchScope scope(s, "index_score");
      if (a.dt == LCA_F32) {
        dim3 grid((nv_max + kScoreThreads - 1) / kScoreThreads, tcn, a.B);
        scope.launch(index_score_f32_kernel, grid, dim3(kScoreThreads),
                     static_cast<uint32_t>((a.H_I * a.d_I + a.H_I) * sizeof(float)),
                           static_cast<const float*>(a.qI), a.w, static_cast<const float*>(a.kI), sc, ld,
                           a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, a.H_I, a.d_I, key16);
      } else if (a.dt == LCA_MXFP4) {
        const int QPB = 16 / a.H_I;
        dim3 grid((nv_max + kFp4KeysPerWG - 1) / kFp4KeysPerWG, (tcn + QPB - 1) / QPB, a.B);
        const uint8_t* q = static_cast<const uint8_t*>(a.qI);
        const uint8_t* qs = static_cast<const uint8_t*>(a.qI_scale);
        const uint8_t* k = static_cast<const uint8_t*>(a.kI);
        const uint8_t* ks = static_cast<const uint8_t*>(a.kI_scale);
        switch (a.H_I) {
          case 1: scope.launch(index_score_fp4_kernel<1>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16); break;
          case 2: scope.launch(index_score_fp4_kernel<2>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16); break;
          case 4: scope.launch(index_score_fp4_kernel<4>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16); break;
          case 8: scope.launch(index_score_fp4_kernel<8>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16); break;
          default: scope.launch(index_score_fp4_kernel<16>, grid, dim3(kScoreThreads), 0, q, qs, a.w, k, ks, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, key16); break;
        }
      } else if (a.d_I == 128 && tcn >= kTiledMinQueries) {
        // many queries: key tiles through LDS, ~2048 workgroups over (keys, queries)
        const int qpwg = 4 * 4 * (16 / a.H_I);
        const int64_t n_qt = (tcn + qpwg - 1) / qpwg;
        int64_t kc = (2048 + n_qt * a.B - 1) / (n_qt * a.B);
        const int64_t kc_max = (nv_max + 255) / 256;
        if (kc > kc_max) kc = kc_max;
        if (kc < 1) kc = 1;
        int64_t per = (nv_max + kc - 1) / kc;
        per = (per + kTileKeys - 1) / kTileKeys * kTileKeys;
        kc = (nv_max + per - 1) / per;
        dim3 grid(static_cast<uint32_t>(kc), static_cast<uint32_t>(n_qt), a.B);
        const uint16_t* q = static_cast<const uint16_t*>(a.qI);
        const uint16_t* k = static_cast<const uint16_t*>(a.kI);
        switch (a.H_I) {
          case 1: scope.launch(index_score_tiled_kernel<1>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, per, key16); break;
          case 2: scope.launch(index_score_tiled_kernel<2>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, per, key16); break;
          case 4: scope.launch(index_score_tiled_kernel<4>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, per, key16); break;
          case 8: scope.launch(index_score_tiled_kernel<8>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, per, key16); break;
          default: scope.launch(index_score_tiled_kernel<16>, grid, dim3(kScoreThreads), 0, q, a.w, k, sc, ld, a.Tq, t_off, Tc, a.N_cap, a.q_pos0, a.q_pos, a.m, per, key16); break;
        }
      } else {
        const int QPB = 16 / a.H_I;
        dim3 grid((nv_max + kKeysPerWG - 1) / kKeysPerWG, (tcn + QPB - 1) / QPB, a.B);
        switch (a.H_I) {
          case 1: launch_score_bf16_hi<1>(scope, a, sc, ld, t_off, Tc, grid); break;
          case 2: launch_score_bf16_hi<2>(scope, a, sc, ld, t_off, Tc, grid); break;
          case 4: launch_score_bf16_hi<4>(scope, a, sc, ld, t_off, Tc, grid); break;
          case 8: launch_score_bf16_hi<8>(scope, a, sc, ld, t_off, Tc, grid); break;
          default: launch_score_bf16_hi<16>(scope, a, sc, ld, t_off, Tc, grid); break;
        }
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      LaunchScope scope(s, "topk_select");
      // every row's list is at most nv_max long (and nv_max > kRound implies N_cap > kRound)
      if (nv_max > kRound)
        scope.launch(topk_select_long_kernel, dim3(tcn, a.B), dim3(kSelThreads), 0, static_cast<const float*>(sc), ld,
                     spill, a.N_cap, a.Tq, t_off, Tc, a.q_pos0, a.q_pos, a.m, a.k, key16, a.idx_out, a.score_out);
      else
        scope.launch(topk_select_kernel, dim3(tcn, a.B), dim3(kSelThreads), 0, static_cast<const float*>(sc), ld,
                     a.N_cap, a.Tq, t_off, Tc, a.q_pos0, a.q_pos, a.m, a.k, key16, a.idx_out, a.score_out);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace lca
