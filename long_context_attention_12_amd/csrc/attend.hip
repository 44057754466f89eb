// attend.hip — core multi-query attention of CSA (selected entries) and HCA
// (all visible entries), each with the raw sliding window and the sink logit.
//
// [PACMAN] §3.1 / §3.2: CSA attends the top-k compressed entries, HCA every
// heavily compressed entry, both plus a recent uncompressed window; [kwkr]
// §3.3: the 128 window rows join the core computation, and a learnable sink
// term enters the softmax denominator; [cdjax] §1.1: multi-query form (a KV
// row is key and value for every head), RoPE at the negative query position
// on the output.
//
// Decomposition: one workgroup per (sequence, query, row split, head group of
// up to 64 heads). All heads of a group share each staged KV row, which is
// read from HBM once per split. Rows of a split are staged 32 at a time into
// an LDS tile. S^T = X Q^T reads the tile row-wise (rows as MFMA M); O^T =
// X^T P^T reads it transposed with gfx950's ds_read_b64_tr_b16 (rows as MFMA
// K). Each wave owns 16 heads: its 16 x D query block stays in registers as
// the B operand, its 16 x D output block in accumulators, and the
// probabilities produced by the S^T accumulators feed the PV MFMA's B operand
// with no data movement. Three kernels stage tiles:
//   attend_dma_kernel        bf16 rows, D = 512: HBM -> LDS copies by the
//                            load units into a 4-tile ring (XOR-swizzled);
//   attend_mixed_dma_kernel  fp8 + bf16 rows, D = 512: raw rows by DMA, then
//                            an exact fp8 -> bf16 conversion pass in LDS;
//   attend_mfma_kernel       bf16 rows, D <= 256: staged through registers
//                            into a double-buffered padded tile.
// The softmax keeps a fixed reference max per head (no rescaling of the
// accumulators); see kHeadroom. Each split writes (max, sum, o) partials (o
// in bf16 at D = 512) and the combine kernel merges splits in a fixed order, adds the sink once,
// divides and applies the inverse RoPE; a query whose rows form a single
// split gets its output from the attention kernel itself. Split sizes depend
// only on per-sequence shapes, so results are independent of the batch size.
#include "lca_device.h"
#include "lca_internal.h"
#include "../../include/lca.h"

namespace lca {
namespace {

constexpr int kTileRows = 32;
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));   // 16-byte streaming stores

struct SplitPlan {
  int S, RS, n_hg, HG;
  int SPW;                     // splits per workgroup: 1, or S (one workgroup per query and head group)
  int xcd;                     // 1: one-dimensional grid, each sequence's workgroups on one XCD
  int qmaj;                    // 1: each XCD takes a contiguous range of the units (queries)
};

struct RowSpan {
  int64_t n_ent, win_lo, nrows;
};

__device__ __forceinline__ RowSpan row_span(const AttendArgs& a, int b, int t) {
  const int64_t p = seq_pos(a.q_pos, a.q_pos0, b) + t;
  RowSpan r;
  if (a.sparse) {
    r.n_ent = a.k;
  } else {
    int64_t nv = n_visible(p, a.m);
    r.n_ent = nv < a.N_cap ? nv : a.N_cap;
  }
  r.win_lo = p - a.W + 1 > 0 ? p - a.W + 1 : 0;
  r.nrows = r.n_ent + (p - r.win_lo + 1);
  return r;
}

// Source of virtual row v of query t: returns the row index in kv (kind 0),
// in win (kind 1), or -1 when the row is absent (padding, out of range).
__device__ __forceinline__ int64_t row_source(const AttendArgs& a, int b, int t, const RowSpan& rs,
                                              int64_t v, int* kind) {
  *kind = 0;
  if (v < rs.n_ent) {
    if (a.sparse) {
      const int32_t e = a.idx[(static_cast<int64_t>(b) * a.Tq + t) * a.k + v];
      return (e >= 0 && e < a.N_cap) ? static_cast<int64_t>(e) : -1;
    }
    return v;
  }
  if (v < rs.nrows) {
    *kind = 1;
    const int64_t pos = rs.win_lo + (v - rs.n_ent);
    if (a.flags & LCA_WIN_RING) return pos % (a.W - 1 + a.Tq);    // ring: position p in row p mod rows
    return pos - (seq_pos(a.q_pos, a.q_pos0, b) - (a.W - 1));
  }
  return -1;
}

// ---------------------------------------------------------------------------
// bf16 / mixed-storage MFMA kernel
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kMaxSplitRows = 2048;
constexpr int kAttThreads = 256;

// Row table entry: >= 0 entry row of kv; <= -2 window row (-2 - r); -1 absent.
__device__ __forceinline__ int32_t encode_row(const AttendArgs& a, int b, int t, const RowSpan& rs,
                                              int64_t v) {
  int kind;
  const int64_t src = row_source(a, b, t, rs, v, &kind);
  if (src < 0) return -1;
  return kind == 0 ? static_cast<int32_t>(src) : static_cast<int32_t>(-2 - src);
}

// One 32-row tile for one wave (16 heads), in two parts.
// tile_softmax: S^T = X Q^T and the online-softmax update; returns the PV
// operand P^T (bf16). tile_pv: O^T += X^T P^T.
// rows[v] == -1 marks an absent row; the row table is padded with -1 to a
// whole number of tiles.
//
// Fixed reference max: each head takes the max logit of its first non-empty
// tile as m_run and keeps it. Later probabilities p = exp(l - m_run) exceed 1
// when later logits are larger, which float32 accumulators and the bf16 P
// operand (float32 exponent range) absorb as long as l - m_run <= kHeadroom:
// p <= e^60 ~ 1e26 and sums stay below ~1e30. The 16 x D output accumulators
// are therefore never rescaled in the loop. If a logit ever exceeds the
// reference by more than kHeadroom, the split is flagged (its partial max is
// written as NaN) and the combine kernel recomputes that split exactly.
constexpr float kHeadroom = 60.f;

// LDS tile layouts. Padded: row r at r * (D + 8) elements. Swizzled (D = 512):
// row r at r * 512 elements with its 16-byte slots permuted, logical slot c
// stored at physical slot c ^ swz(r), swz(r) = (2r + (r >> 3)) & 15. Both
// layouts keep the row-wise 16-byte reads of S^T = X Q^T and the transposed
// 8-byte reads of X^T P^T free of LDS bank conflicts.
__device__ __forceinline__ int slot_swizzle(int r) { return (2 * r + ((r >> 3) & 1)) & 15; }

template <int D, bool SWZ>
__device__ __forceinline__ int tile_offset(int r, int col) {
  if constexpr (!SWZ) {
    return r * (D + 8) + col;
  } else {
    return r * D + ((((col >> 3) ^ slot_swizzle(r)) << 3) | (col & 7));
  }
}

// Online-softmax update of one 32-row tile from the S^T accumulators (lane:
// head r16, rows 16h2 + 4g + i), with a fixed reference max (see above).
__device__ __forceinline__ void softmax_update(const f32x4 (&sacc)[2], int v0, const int32_t* rows,
                                               float scale, int g, float& m_run, float& z_run, bool& flag,
                                               bf16x8& pf) {
  const int4 rv0 = *reinterpret_cast<const int4*>(rows + v0 + 4 * g);
  const int4 rv1 = *reinterpret_cast<const int4*>(rows + v0 + 16 + 4 * g);
  const int rr[8] = {rv0.x, rv0.y, rv0.z, rv0.w, rv1.x, rv1.y, rv1.z, rv1.w};
  float lg[8];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float l = rr[i] != -1 ? sacc[i >> 2][i & 3] * scale : -INFINITY;
    lg[i] = l;
    mx = fmaxf(mx, l);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (m_run == -INFINITY) m_run = mx;              // first non-empty tile sets the reference
  flag = flag || (mx > m_run + kHeadroom);
  float psum = 0.f;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = lg[i] == -INFINITY ? 0.f : __expf(fminf(lg[i] - m_run, kHeadroom));
    psum += p[i];
  }
  psum += __shfl_xor(psum, 16, 64);
  psum += __shfl_xor(psum, 32, 64);
  z_run += psum;
  uint4 pw;
  pw.x = pack_bf16x2(p[0], p[1]);
  pw.y = pack_bf16x2(p[2], p[3]);
  pw.z = pack_bf16x2(p[4], p[5]);
  pw.w = pack_bf16x2(p[6], p[7]);
  pf = __builtin_bit_cast(bf16x8, pw);
}

template <int D, bool SWZ = false>
__device__ __forceinline__ void tile_softmax(const uint16_t* X, int v0, const int32_t* rows,
                                             const bf16x8 (&qf)[D / 32], float scale, int g, int r16,
                                             float& m_run, float& z_run, bool& flag, bf16x8& pf) {
  constexpr int KS = D / 32;
  // S^T (32 rows x 16 heads) in two 16-row halves; lane: head r16, rows 16h2 + 4g + i
  f32x4 sacc[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = h2 * 16 + r16;
    constexpr int XB = KS < 8 ? KS : 8;            // K-step fragments read ahead of MFMAs
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < KS; s0 += XB) {
      uint4 xa[XB];
#pragma unroll
      for (int e = 0; e < XB; ++e)
        xa[e] = *reinterpret_cast<const uint4*>(X + tile_offset<D, SWZ>(row, 32 * (s0 + e) + 8 * g));
#pragma unroll
      for (int e = 0; e < XB; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[e]), qf[s0 + e], acc, 0, 0, 0);
    }
    sacc[h2] = acc;
  }
  softmax_update(sacc, v0, rows, scale, g, m_run, z_run, flag, pf);
}

template <int D, bool SWZ = false>
__device__ __forceinline__ void tile_pv(const uint16_t* X, const bf16x8& pf, int g, int r16,
                                        f32x4 (&acc_o)[D / 16]) {
  constexpr int DT = D / 16;
  // O^T += X^T P^T. A operand = rows {4g..4g+3, 16+4g..16+4g+3} of channel 16dt + r16,
  // read transposed from the row-major tile (ds_read_b64_tr_b16: lane L of a
  // 16-lane group supplies row 4g + L/4, channels 16dt + 4(L%4) .. +3)
  const int row0 = 4 * g + (r16 >> 2), row1 = row0 + 16, c0 = 4 * (r16 & 3);
  constexpr int PB = DT < 8 ? DT : 8;              // transposed reads batched ahead of MFMAs
#pragma unroll
  for (int d8 = 0; d8 < DT; d8 += PB) {
    bf16x8 af[PB];
#pragma unroll
    for (int e = 0; e < PB; ++e) {
      const int dt = d8 + e;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + tile_offset<D, SWZ>(row0, 16 * dt + c0)));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(X + tile_offset<D, SWZ>(row1, 16 * dt + c0)));
      const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
      af[e] = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
    }
#pragma unroll
    for (int e = 0; e < PB; ++e)
      acc_o[d8 + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[e], pf, acc_o[d8 + e], 0, 0, 0);
  }
}

// Swizzled tile (D = 512) with all LDS addresses precomputed per lane: every
// read in the tile loop is `lane base + immediate offset`.
//   S^T reads: lane (r16, g), row 16h2 + r16, K step s = 4j + k:
//     byte = row*1024 + 256j + 64(k ^ w2) + 16(g ^ w1),  w = swz(r16) = 4w2 + w1
//   X^T reads: lane (g, L), row0 = 4g + L/4 (+16 for the second half),
//     channel tile dt = 8j + k: byte = row0*1024 + 256j + 32(k ^ a) + 16(h ^ c) + 8(L & 1)
//     with swz(row0) = 2a + c and h = (L & 3) >> 1.
struct SwzOffsets {
  uint32_t qk[4];   // byte offsets of K-step groups k = 0..3 (row r16)
  uint32_t pv[8];   // byte offsets of channel tiles k = 0..7 (row0)
};

__device__ __forceinline__ SwzOffsets swz_offsets(int g, int r16) {
  SwzOffsets o;
  const int w = slot_swizzle(r16), w2 = w >> 2, w1 = w & 3;
#pragma unroll
  for (int k = 0; k < 4; ++k) o.qk[k] = r16 * 1024 + 64 * (k ^ w2) + 16 * (g ^ w1);
  const int row0 = 4 * g + (r16 >> 2);
  const int sw = slot_swizzle(row0), aa = sw >> 1, cc = sw & 1, hh = (r16 & 3) >> 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) o.pv[k] = row0 * 1024 + 32 * (k ^ aa) + 16 * (hh ^ cc) + 8 * (r16 & 1);
  return o;
}

// Reductions across lanes l and l ^ 16, l and l ^ 32 with the gfx950 lane
// swaps (VALU only: no LDS operation that would queue behind LDS reads in
// flight). Each swap returns the pair {x[l], x[l ^ 16 or 32]} in a fixed
// order, so both lanes of a pair compute the same value.
__device__ __forceinline__ float pair_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online-softmax update as softmax_update, with the row table entries already
// in registers and the reductions done by lane swaps.
__device__ __forceinline__ void softmax_update_regs(const f32x4 (&sacc)[2], const int4 (&rv)[2], float scale,
                                                    float& m_run, float& z_run, bool& flag, bf16x8& pf) {
  const int rr[8] = {rv[0].x, rv[0].y, rv[0].z, rv[0].w, rv[1].x, rv[1].y, rv[1].z, rv[1].w};
  float lg[8];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float l = rr[i] != -1 ? sacc[i >> 2][i & 3] * scale : -INFINITY;
    lg[i] = l;
    mx = fmaxf(mx, l);
  }
  mx = pair_max32(pair_max16(mx));
  if (m_run == -INFINITY) m_run = mx;              // first non-empty tile sets the reference
  flag = flag || (mx > m_run + kHeadroom);
  float psum = 0.f;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = lg[i] == -INFINITY ? 0.f : __expf(fminf(lg[i] - m_run, kHeadroom));
    psum += p[i];
  }
  z_run += pair_sum32(pair_sum16(psum));
  uint4 pw;
  pw.x = pack_bf16x2(p[0], p[1]);
  pw.y = pack_bf16x2(p[2], p[3]);
  pw.z = pack_bf16x2(p[4], p[5]);
  pw.w = pack_bf16x2(p[6], p[7]);
  pf = __builtin_bit_cast(bf16x8, pw);
}

// Stages of one 32-row tile for one wave (16 heads) on the swizzled D = 512
// layout. qk_load: the row-table entries and the 32 S^T fragments (fragment
// f = 16 h2 + s: rows 16 h2 .. 16 h2 + 15, K step s). qk_mfma: S^T = X Q^T,
// two independent accumulation chains (the row halves). pv_load: the 32 X^T
// fragments (channel tile dt). pv_mfma: O^T += X^T P^T.
__device__ __forceinline__ void qk_load(const uint16_t* X, const SwzOffsets& so, const int32_t* rows, int v0, int g,
                                        bf16x8 (&xf)[32], int4 (&rv)[2]) {
  const char* xb = reinterpret_cast<const char*>(X);
  rv[0] = *reinterpret_cast<const int4*>(rows + v0 + 4 * g);
  rv[1] = *reinterpret_cast<const int4*>(rows + v0 + 16 + 4 * g);
#pragma unroll
  for (int f = 0; f < 32; ++f) {
    const int h2 = f >> 4, st = f & 15;
    xf[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xb + so.qk[st & 3] + h2 * 16384 + 256 * (st >> 2)));
  }
}

__device__ __forceinline__ void qk_mfma(const bf16x8 (&xf)[32], const bf16x8 (&qf)[16], f32x4 (&sacc)[2]) {
  sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 16; ++st)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      sacc[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[16 * h2 + st], qf[st], sacc[h2], 0, 0, 0);
}

template <int DT0 = 0, int NDT = 32>
__device__ __forceinline__ void pv_load(const uint16_t* X, const SwzOffsets& so, bf16x8 (&vf)[NDT]) {
  const char* xb = reinterpret_cast<const char*>(X);
#pragma unroll
  for (int i = 0; i < NDT; ++i) {
    const int dt = DT0 + i;
    const int j = dt >> 3, k = dt & 7;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(xb + so.pv[k] + 256 * j));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(xb + so.pv[k] + 256 * j + 16384));
    const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
    vf[i] = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
  }
}

template <int DT0 = 0, int NDT = 32>
__device__ __forceinline__ void pv_mfma(const bf16x8 (&vf)[NDT], const bf16x8& pf, f32x4 (&acc_o)[32]) {
#pragma unroll
  for (int i = 0; i < NDT; ++i)
    acc_o[DT0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[i], pf, acc_o[DT0 + i], 0, 0, 0);
}

// Steady state of the tile pipeline: S^T of the next tile and the output
// update of the current one. With one wave per SIMD nothing else hides a wait,
// so the wave itself overlaps the units:
//   1. LDS reads: the next tile's S^T fragments, then the first half of this
//      tile's X^T fragments;
//   2. the next tile's S^T MFMAs interleaved with this tile's softmax on the
//      VALU (the matrix core runs one MFMA while the wave issues several VALU
//      instructions);
//   3. one wait for all LDS reads (long landed by then; the LDS counter is
//      in-order, so a later partial wait would also wait for younger reads),
//      the second half's reads into the registers the S^T fragments freed,
//      and the 32 PV MFMAs.
// The sched_barrier fences keep each group in its place; the group barriers
// ask for the MFMA / VALU interleave.
__device__ __forceinline__ void tile_pipe_step(const uint16_t* Xc, const uint16_t* Xn, const SwzOffsets& so,
                                               const int32_t* rows, int v0n, int g, const bf16x8 (&qf)[16],
                                               float scale, f32x4 (&sacc)[2], int4 (&rv)[2], float& m_run,
                                               float& z_run, bool& flag, f32x4 (&acc_o)[32]) {
  f32x4 sn[2];
  int4 rvn[2];
  bf16x8 va[16], pf;
  {
    bf16x8 xf[32];
    qk_load(Xn, so, rows, v0n, g, xf, rvn);
    pv_load<0, 16>(Xc, so, va);
    __builtin_amdgcn_sched_barrier(0);
    qk_mfma(xf, qf, sn);
    softmax_update_regs(sacc, rv, scale, m_run, z_run, flag, pf);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then up to four VALU
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_lgkmcnt0();
  bf16x8 vb[16];
  pv_load<16, 16>(Xc, so, vb);
  pv_mfma<0, 16>(va, pf, acc_o);
  pv_mfma<16, 16>(vb, pf, acc_o);
  sacc[0] = sn[0];
  sacc[1] = sn[1];
  rv[0] = rvn[0];
  rv[1] = rvn[1];
}

// One tile for a wave serving 32 heads (two 16-head tiles): every X fragment
// read from LDS feeds two MFMAs, halving LDS reads per FLOP (the LDS is the
// limit of the 16-head form: its reads of a 32-row tile take longer than its
// MFMAs). Fragments stream four ahead of the MFMAs that consume them; the
// group barriers fix that order (left alone, the compiler pairs each read with
// its MFMA and waits on every read). S^T fragments go in the order
// (K step s, row half h2) so that four accumulation chains alternate.
__device__ __forceinline__ void tile_step_32(const uint16_t* X, const SwzOffsets& so, int v0, const int32_t* rows,
                                             const bf16x8 (&qf)[2][16], float scale, int g, float (&m_run)[2],
                                             float (&z_run)[2], bool (&flag)[2], f32x4 (&acc_o)[2][32]) {
  const char* xb = reinterpret_cast<const char*>(X);
  int4 rv[2];
  rv[0] = *reinterpret_cast<const int4*>(rows + v0 + 4 * g);
  rv[1] = *reinterpret_cast<const int4*>(rows + v0 + 16 + 4 * g);
  f32x4 sacc[2][2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) sacc[ht][0] = sacc[ht][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  __builtin_amdgcn_sched_barrier(0);
  {
    bf16x8 xf[32];
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const int st = f >> 1, h2 = f & 1;
      xf[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xb + so.qk[st & 3] + h2 * 16384 + 256 * (st >> 2)));
    }
#pragma unroll
    for (int f = 0; f < 32; ++f)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        sacc[ht][f & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[f], qf[ht][f >> 1], sacc[ht][f & 1], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);     // rows entries + first four fragments
#pragma unroll
    for (int i = 0; i < 28; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one fragment read ...
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // ... and the two MFMAs of a landed one
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 pf[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) softmax_update_regs(sacc[ht], rv, scale, m_run[ht], z_run[ht], flag[ht], pf[ht]);
  __builtin_amdgcn_sched_barrier(0);
  {
    bf16x8 vf[32];
    pv_load(X, so, vf);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        acc_o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf[ht], acc_o[ht][dt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);     // first four fragments (two reads each)
#pragma unroll
    for (int i = 0; i < 28; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Work items of one sequence: u = t * S + split over its Tq queries and S
// splits, times n_hg head groups. Consecutive workgroup ids land on
// consecutive XCDs (id % 8), so with two head groups the ids i and i + 8 (same
// XCD, shared L2) take the two groups of one work item u and fetch its rows
// once; successive u spread over all XCDs.
__host__ __device__ __forceinline__ int64_t work_blocks(const SplitPlan& sp, int Tq) {
  const int64_t U = static_cast<int64_t>(Tq) * (sp.S / sp.SPW);
  return sp.n_hg == 2 ? (U + 7) / 8 * 16 : U * sp.n_hg;
}

__device__ __forceinline__ bool work_item(const SplitPlan& sp, int Tq, int i, int& split, int& hg, int& t) {
  int64_t u;
  if (sp.n_hg == 2) {
    hg = (i >> 3) & 1;
    u = (static_cast<int64_t>(i >> 4) << 3) | (i & 7);
  } else {
    hg = i % sp.n_hg;
    u = i / sp.n_hg;
  }
  const int per_q = sp.S / sp.SPW;                // workgroups per query and head group
  if (u >= static_cast<int64_t>(Tq) * per_q) return false;
  t = static_cast<int>(u / per_q);
  split = static_cast<int>(u % per_q) * sp.SPW;    // first split of this workgroup
  return true;
}

// Units per XCD when each XCD takes a contiguous range (sp.qmaj): whole
// groups of 16, so the two head groups of a unit (8 apart) stay together.
__host__ __device__ __forceinline__ int64_t qmaj_per(const SplitPlan& sp, int Tq) {
  return (work_blocks(sp, Tq) + 127) / 128 * 16;
}

// Workgroup -> (split, head group, query, sequence). With sp.qmaj (calls of
// many queries, one sequence) XCD c takes the c-th eighth of the units, so
// neighbouring queries, whose window rows and many of whose selected rows
// coincide, gather through the same L2. With sp.xcd the grid is
// one-dimensional: the dispatcher hands workgroup i to XCD i % 8, and every
// workgroup of sequence b gets i % 8 == b % 8, so all of b's workgroups share
// one L2 (and the top-k workgroup of b at decode, which wrote b's selected
// indices, ran there too). Otherwise the grid is (units, 1, B).
__device__ __forceinline__ bool work_item_b(const SplitPlan& sp, int Tq, int& split, int& hg, int& t, int& b) {
  int64_t x;
  if (sp.xcd) {
    const int64_t i = blockIdx.x, slot = i >> 3, W = work_blocks(sp, Tq);
    b = static_cast<int>((i & 7) + 8 * (slot / W));
    x = slot % W;
  } else if (sp.qmaj) {
    const int64_t i = blockIdx.x;
    x = (i & 7) * qmaj_per(sp, Tq) + (i >> 3);
    b = blockIdx.z;
    if (x >= work_blocks(sp, Tq)) return false;
  } else {
    x = blockIdx.x;
    b = blockIdx.z;
  }
  return work_item(sp, Tq, static_cast<int>(x), split, hg, t);
}

// A query's only split is its whole row set: the head's output is final here.
// Accumulators are relative to the fixed reference m_run; with M = max(sink,
// m_run), out = o e^(m_run - M) / (z e^(m_run - M) + e^(sink - M)), then the
// RoPE channels are turned back by -p. Lane (g, r16) holds channels
// 16 dt + 4g .. +3 of head r16. The (max) slot is set to +inf (done), or NaN
// when the logits outgrew the headroom (an exact recompute follows).
// Angles of the inverse RoPE at query t: rope_tab[i] = (cos, sin) of pair i
// at position -(q_pos0 + t), filled once per workgroup.
__device__ __forceinline__ void fill_rope_table(const AttendArgs& a, int b, int t, float2* rope_tab) {
  const int R = ((a.flags & LCA_INV_ROPE) && a.rope_dims > 0) ? a.rope_dims : 0;
  for (int i = threadIdx.x; i < R / 2; i += blockDim.x) {
    float sn, cs;
    rope_sincos(-static_cast<double>(seq_pos(a.q_pos, a.q_pos0, b) + t), i, a.rope_r, &sn, &cs);
    rope_tab[i] = make_float2(cs, sn);
  }
}

// Merge of a query's split results, in one fixed order and arithmetic that
// every path shares (the combine kernel over partials in memory, an attention
// kernel over its own registers), so the bits never depend on where a split
// ran. The state starts at the sink (M = sink, Z = e^0 = 1, U = 0); split
// (m_s, z_s, o_s), its sums relative to its own reference m_s, folds in as
//   a = e^(M - m_s), c = 1, M = m_s   when m_s > M,   else   a = 1, c = e^(m_s - M)
//   Z = fma(Z, a, z_s c),   U = fma(U, a, o_s c)  (each channel);
// an empty split (m_s = -inf) changes nothing. The output is U * (1 / Z),
// lse = M + log Z. Scaling by exactly 1 keeps the fused form equal to the
// two-case form, bit for bit.
struct SplitFold {
  float M, Z;
};
__device__ __forceinline__ SplitFold fold_start(float sink) { return SplitFold{sink, 1.0f}; }
__device__ __forceinline__ void fold_coeffs(SplitFold& f, float ms, float zs, float& ca, float& cc) {
  if (ms == -INFINITY) {
    ca = 1.0f;
    cc = 0.0f;
    return;
  }
  if (ms > f.M) {
    ca = __expf(f.M - ms);
    cc = 1.0f;
    f.M = ms;
  } else {
    ca = 1.0f;
    cc = __expf(ms - f.M);
  }
  f.Z = fmaf(f.Z, ca, zs * cc);
}
// Inverse-RoPE turn of one channel pair by (cos, sin), in a fixed form.
__device__ __forceinline__ void rope_turn(float& x, float& y, float2 cs) {
  const float nx = fmaf(x, cs.x, -(y * cs.y));
  const float ny = fmaf(x, cs.y, y * cs.x);
  x = nx;
  y = ny;
}

// Lane (g, r16) holds channels 16 dt + 4 g .. +3 of its head in U; writes the
// head's output row (U / Z, inverse RoPE, q's dtype) and its lse.
// Ufn(dt, i) gives the folded value of the lane's channel 16 dt + 4 g + i.
template <int D, typename UFn>
__device__ __forceinline__ void store_folded(const AttendArgs& a, int b, int t, int head, int g, UFn Ufn,
                                             const SplitFold& f, const float2* rope_tab) {
  constexpr int DT = D / 16;
  const float inv = 1.0f / f.Z;
  const int64_t row = (static_cast<int64_t>(b) * a.Tq + t) * a.H + head;
  uint16_t* op = static_cast<uint16_t*>(a.out) + row * D;
  const int R = ((a.flags & LCA_INV_ROPE) && a.rope_dims > 0) ? a.rope_dims : 0;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    float v[4] = {Ufn(dt, 0) * inv, Ufn(dt, 1) * inv, Ufn(dt, 2) * inv, Ufn(dt, 3) * inv};
    const int c0 = 16 * dt + 4 * g;
    if (c0 >= D - R) {
#pragma unroll
      for (int p = 0; p < 2; ++p) rope_turn(v[2 * p], v[2 * p + 1], rope_tab[(c0 + 2 * p - (D - R)) / 2]);
    }
    uint2 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(op + c0) = w;
  }
  if (g == 0 && a.lse_out) a.lse_out[row] = f.M + logf(f.Z);
}

// The query's only split, merged with the sink and written (fold of one split).
// A split whose logits outgrew the headroom is left to the fixup kernel (max
// slot NaN); otherwise the slot is set to +inf (done).
template <int D>
__device__ __forceinline__ void write_output(const AttendArgs& a, int b, int t, int head, int g,
                                             const f32x4 (&acc_o)[D / 16], float m_run, float z_run, bool flag,
                                             const float2* rope_tab, float* ml) {
  if (flag) {
    if (g == 0) ml[0] = __builtin_nanf("");
    return;
  }
  SplitFold f = fold_start(a.sink[head]);
  float ca, cc;
  fold_coeffs(f, m_run, z_run, ca, cc);
  store_folded<D>(a, b, t, head, g, [&](int dt, int i) { return fmaf(0.0f, ca, acc_o[dt][i] * cc); }, f, rope_tab);
  if (g == 0) ml[0] = INFINITY;
}

template <int D>
__global__ __launch_bounds__(kAttThreads) void attend_mfma_kernel(AttendArgs a, SplitPlan sp,
                                                                  float* __restrict__ part_o,
                                                                  float* __restrict__ part_ml) {
  constexpr int XS = D + 8;                       // LDS row stride (bf16)
  constexpr int KS = D / 32;                      // K steps of S^T
  constexpr int DT = D / 16;                      // 16-channel output tiles
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int CPT = kTileRows * CPR / kAttThreads;   // chunks per thread per tile
  constexpr int RB = 2 * D;                       // bytes per stored row
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kTileRows * XS];
  __shared__ int32_t rows[kMaxSplitRows];
  __shared__ float2 rope_tab[D / 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform in a scalar register
  const int g = lane >> 4, r16 = lane & 15;
  int split, hg, t;
  int b;
  if (!work_item_b(sp, a.Tq, split, hg, t, b)) return;
  const bool active = wid * 16 < sp.HG;
  const int head = hg * sp.HG + wid * 16 + r16;
  const RowSpan rs = row_span(a, b, t);
  if (sp.S == 1) fill_rope_table(a, b, t, rope_tab);   // read after the tile loop's barriers
  const int64_t r_begin = static_cast<int64_t>(split) * sp.RS;
  int64_t r_end = r_begin + sp.RS;
  if (r_end > rs.nrows) r_end = rs.nrows;
  const int nr = r_end > r_begin ? static_cast<int>(r_end - r_begin) : 0;

  // prologue: the row table's index loads and the query loads go out together
  int32_t myrows[kMaxSplitRows / kAttThreads];
#pragma unroll
  for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) {
    const int v = tid + kAttThreads * q;
    myrows[q] = v < nr ? encode_row(a, b, t, rs, r_begin + v) : -1;
  }
  // (a wave past the block's heads computes on zero queries and writes nothing;
  // a branch around the MFMAs would make the compiler copy the accumulators)
  bf16x8 qf[KS];
  if (active) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g));
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
  }
#pragma unroll
  for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) rows[tid + kAttThreads * q] = myrows[q];
  f32x4 acc_o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, z_run = 0.f;
  bool flag = false;
  const float scale = a.scale;
  const int64_t win_rows = a.W - 1 + a.Tq;
  __syncthreads();

  // staging: each thread moves CPT 16-byte chunks of a tile. Base pointers are
  // chosen per lane from values held in registers, so the selection never
  // turns into a per-lane load of a kernel argument.
  const uint8_t* kv_base = static_cast<const uint8_t*>(a.kv);
  const uint8_t* win_base = static_cast<const uint8_t*>(a.win);
  const int64_t kv_off = static_cast<int64_t>(b) * a.N_cap;
  const int64_t win_off = static_cast<int64_t>(b) * win_rows;
  uint4 pre[CPT];
  auto issue = [&](int tile) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + kAttThreads * c;
      const int r = chunk / CPR, d0 = (chunk % CPR) * 8;
      const int v = tile * kTileRows + r;
      const int32_t src = v < nr ? rows[v] : -1;
      const bool is_kv = src >= 0;
      const int64_t ridx = is_kv ? kv_off + src : win_off + (-2 - src);
      const uint8_t* base = (is_kv ? kv_base : win_base) + ridx * RB;
      pre[c] = src != -1 ? *reinterpret_cast<const uint4*>(base + 2 * d0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + kAttThreads * c;
      const int r = chunk / CPR, d0 = (chunk % CPR) * 8;
      *reinterpret_cast<uint4*>(&Xs[buf][r * XS + d0]) = pre[c];
    }
  };

  const int ntiles = (nr + kTileRows - 1) / kTileRows;
  if (ntiles > 0) {
    issue(0);
    commit(0);
  }
  // nothing may be in flight when the loop starts: the loop body then needs
  // no wait on the query fragments, and the next tile's loads overlap compute
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) issue(it + 1);
    {
      const uint16_t* X = Xs[buf];
      bf16x8 pf;
      tile_softmax<D>(X, it * kTileRows, rows, qf, scale, g, r16, m_run, z_run, flag, pf);
      tile_pv<D>(X, pf, g, r16, acc_o);
    }
    if (it + 1 < ntiles) commit(buf ^ 1);
    __syncthreads();
  }

  if (active) {
    const int64_t part_idx = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * sp.S + split;
    if (sp.S == 1) {
      write_output<D>(a, b, t, head, g, acc_o, m_run, z_run, flag, rope_tab, part_ml + 2 * part_idx);
    } else {
      float* po = part_o + part_idx * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) = make_float4(acc_o[dt][0], acc_o[dt][1], acc_o[dt][2], acc_o[dt][3]);
      if (g == 0) {
        part_ml[2 * part_idx] = flag ? __builtin_nanf("") : m_run;   // NaN: recompute in combine
        part_ml[2 * part_idx + 1] = z_run;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 rows of 512 channels: tiles are copied HBM -> LDS by the load units
// themselves (global_load_lds_dwordx4: one 1 KB row per wave instruction, no
// registers involved) into a ring of four LDS tiles. Each step works on two
// landed tiles (S^T of the next, the output update of the current) while up
// to two more are in flight.
// ---------------------------------------------------------------------------
constexpr int kRing = 4;

// NHT 16-head tiles per wave: NHT = 1 serves 64 heads per workgroup, NHT = 2
// serves 128 (half the LDS reads and tile copies per head; the per-head state
// fills the unified register file of this one-wave-per-SIMD kernel).
template <int NHT>
__global__ __launch_bounds__(kAttThreads) void attend_dma_kernel(AttendArgs a, SplitPlan sp,
                                                                 float* __restrict__ part_o,
                                                                 float* __restrict__ part_ml) {
  constexpr int D = 512, KS = D / 32, DT = D / 16;
  constexpr int RPW = kTileRows / 4;               // rows per wave per tile
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kRing][kTileRows * D];
  __shared__ int32_t rows[kMaxSplitRows];
  __shared__ float2 rope_tab[D / 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform in a scalar register
  const int g = lane >> 4, r16 = lane & 15;
  int split, hg, t;
  int b;
  if (!work_item_b(sp, a.Tq, split, hg, t, b)) return;
  const bool active = wid * 16 * NHT < sp.HG;
  const int head0 = hg * sp.HG + wid * 16 * NHT + r16;   // + 16 ht for head tile ht
  const RowSpan rs = row_span(a, b, t);
  if (sp.S == 1) fill_rope_table(a, b, t, rope_tab);   // read after the tile loop's barriers
  const int64_t r_begin = static_cast<int64_t>(split) * sp.RS;
  int64_t r_end = r_begin + sp.RS;
  if (r_end > rs.nrows) r_end = rs.nrows;
  const int nr = r_end > r_begin ? static_cast<int>(r_end - r_begin) : 0;

  // query fragments first: their loads are in flight with the row table's
  // (a wave past the block's heads computes on zero queries and writes nothing)
  bf16x8 qf[NHT][KS];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    if (active) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head0 + 16 * ht) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qf[ht][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g));
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[ht][s] = bf16x8{};
    }
  }
  // row table (its index loads all in flight together)
  int32_t myrows[kMaxSplitRows / kAttThreads];
#pragma unroll
  for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) {
    const int v = tid + kAttThreads * q;
    myrows[q] = v < nr ? encode_row(a, b, t, rs, r_begin + v) : -1;
  }
#pragma unroll
  for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) rows[tid + kAttThreads * q] = myrows[q];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int64_t win_rows = a.W - 1 + a.Tq;
  const uint16_t* kvp = static_cast<const uint16_t*>(a.kv) + static_cast<int64_t>(b) * a.N_cap * D;
  const uint16_t* winp = static_cast<const uint16_t*>(a.win) + static_cast<int64_t>(b) * win_rows * D;
  // Wave w copies rows [RPW*w, RPW*w + RPW) of a tile, one 1 KB row per
  // instruction. Lane l fetches logical 16-byte slot l ^ swz(r), which lands at
  // physical slot l: the tile is stored swizzled. Lanes 0..RPW-1 resolve the
  // rows' addresses, which reach the copies through readlane. Absent rows copy
  // window row 0 (any valid memory) and are masked out of the softmax.
  auto issue = [&](int tile, uint16_t* dst) {
    const int v0 = tile * kTileRows + wid * RPW;
    uint64_t my = 0;
    if (lane < RPW) {
      const int v = v0 + lane;
      const int32_t sr = v < nr ? rows[v] : -1;
      const uint16_t* rowp = sr >= 0 ? kvp + static_cast<int64_t>(sr) * D
                                     : winp + (sr == -1 ? 0 : static_cast<int64_t>(-2 - sr) * D);
      my = reinterpret_cast<uint64_t>(rowp);
    }
    const uint32_t lds0 = lds_address(dst + wid * RPW * D);
    const uint32_t lo = static_cast<uint32_t>(my), hi = static_cast<uint32_t>(my >> 32);
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const uint64_t rb = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), rr))) << 32) |
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), rr));
      const uint32_t src_off = 16u * static_cast<uint32_t>((lane & 48) | ((lane & 15) ^ slot_swizzle(wid * RPW + rr)));
      lds_copy16(reinterpret_cast<const void*>(rb + src_off), lds0 + rr * D * 2);
    }
  };
  const int ntiles = (nr + kTileRows - 1) / kTileRows;
  // Ring: tiles 0..2 are issued up front. Step `it` waits for tile it + 1
  // (tile it + 2 may stay in flight) and, after that barrier, refills the slot
  // of tile it - 1 (consumed by every wave in step it - 1) with tile it + 3.
  auto wait_next = [&](int tt) {
    if (tt + 1 < ntiles) wait_vmcnt<RPW>();
    else wait_vmcnt<0>();
    // A bare barrier: the wave's own copies are complete (waited above) and
    // every LDS read of the freed slot fed an MFMA already, so no fence is
    // needed; a fence would also drain the later copies that must stay in flight.
    __builtin_amdgcn_s_barrier();
  };
#pragma unroll
  for (int t0 = 0; t0 < kRing - 1; ++t0)
    if (t0 < ntiles) issue(t0, Xs[t0]);
  f32x4 acc_o[NHT][DT];
  float m_run[NHT], z_run[NHT];
  bool flag[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
    for (int i = 0; i < DT; ++i) acc_o[ht][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[ht] = -INFINITY;
    z_run[ht] = 0.f;
    flag[ht] = false;
  }
  const SwzOffsets so = swz_offsets(g, r16);

  if constexpr (NHT == 1) {
    if (ntiles > 0) {
      // tile 0 landed (tiles 1, 2 may still be in flight); query fragments too
      if (ntiles > 2) wait_vmcnt<2 * RPW>();
      else if (ntiles > 1) wait_vmcnt<RPW>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      f32x4 sacc[2];
      int4 rv[2];
      {
        bf16x8 xf[32];
        qk_load(Xs[0], so, rows, 0, g, xf, rv);
        qk_mfma(xf, qf[0], sacc);
      }
      for (int it = 0; it + 1 < ntiles; ++it) {
        wait_next(it + 1);
        if (it + kRing - 1 < ntiles) issue(it + kRing - 1, Xs[(it + kRing - 1) % kRing]);
        tile_pipe_step(Xs[it % kRing], Xs[(it + 1) % kRing], so, rows, (it + 1) * kTileRows, g, qf[0], a.scale, sacc,
                       rv, m_run[0], z_run[0], flag[0], acc_o[0]);
      }
      // last tile: output update only
      bf16x8 vf[32], pf;
      pv_load(Xs[(ntiles - 1) % kRing], so, vf);
      softmax_update_regs(sacc, rv, a.scale, m_run[0], z_run[0], flag[0], pf);
      pv_mfma(vf, pf, acc_o[0]);
    }
  } else {
    // Ring step: consume tile it, then wait for tile it + 1 and refill the
    // slot of tile it with tile it + 4 (three tiles in flight meanwhile).
    auto wait_tile = [&](int tt) {
      const int later = min(ntiles - 1, tt + kRing - 2) - tt;
      if (later >= 2) wait_vmcnt<2 * RPW>();
      else if (later == 1) wait_vmcnt<RPW>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();                 // bare: see wait_next
    };
    if (ntiles > 0) {
      wait_tile(0);
      __builtin_amdgcn_s_waitcnt(0);                // query fragments too
    }
    for (int it = 0; it < ntiles; ++it) {
      if (it + kRing - 1 < ntiles) issue(it + kRing - 1, Xs[(it + kRing - 1) % kRing]);
      tile_step_32(Xs[it % kRing], so, it * kTileRows, rows, qf, a.scale, g, m_run, z_run, flag, acc_o);
      if (it + 1 < ntiles) wait_tile(it + 1);
    }
  }

  if constexpr (NHT == 1) {
    // Partials in bf16 (the fold rounds every split's output to bf16 wherever
    // it runs, so both placements fold the same values), through LDS: the
    // wave's 16 x D block goes to its own ring slot (8-byte slots
    // XOR-swizzled by head), then out one head row at a time, 1 KB per store
    // instruction, streamed past the cache (the combine kernel reads it once).
    if (sp.S > 1) {
      __syncthreads();                               // every wave is done with the ring
      if (active) {
        uint8_t* wl = reinterpret_cast<uint8_t*>(Xs[wid]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<uint2*>(wl + r16 * (2 * D) + 8 * ((4 * dt + g) ^ (r16 << 2))) =
              make_uint2(pack_bf16x2(acc_o[0][dt][0], acc_o[0][dt][1]), pack_bf16x2(acc_o[0][dt][2], acc_o[0][dt][3]));
        const int64_t pi0 = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + (head0 - r16)) * sp.S + split;
        uint16_t* pob = reinterpret_cast<uint16_t*>(part_o);
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) {
          const uint4 v = *reinterpret_cast<const uint4*>(wl + hh * (2 * D) + 8 * ((2 * lane) ^ (hh << 2)));
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v),
                                      reinterpret_cast<u32x4_nt*>(pob + (pi0 + static_cast<int64_t>(hh) * sp.S) * D + 8 * lane));
        }
        if (g == 0) {
          const int64_t part_idx = pi0 + static_cast<int64_t>(r16) * sp.S;
          part_ml[2 * part_idx] = flag[0] ? __builtin_nanf("") : m_run[0];   // NaN: recompute in combine
          part_ml[2 * part_idx + 1] = z_run[0];
        }
      }
      return;
    }
  }
  if (active) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int head = head0 + 16 * ht;
      const int64_t part_idx = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * sp.S + split;
      if (sp.S == 1) {
        write_output<D>(a, b, t, head, g, acc_o[ht], m_run[ht], z_run[ht], flag[ht], rope_tab, part_ml + 2 * part_idx);
      } else {
        // bf16 partial (32-byte pieces per head: plain stores, which the L2 merges into lines)
        uint16_t* pob = reinterpret_cast<uint16_t*>(part_o) + part_idx * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<uint2*>(pob + 16 * dt + 4 * g) =
              make_uint2(pack_bf16x2(acc_o[ht][dt][0], acc_o[ht][dt][1]), pack_bf16x2(acc_o[ht][dt][2], acc_o[ht][dt][3]));
        if (g == 0) {
          part_ml[2 * part_idx] = flag[ht] ? __builtin_nanf("") : m_run[ht];   // NaN: recompute in combine
          part_ml[2 * part_idx + 1] = z_run[ht];
        }
      }
    }
  }
}

__device__ void recompute_split(const AttendArgs& a, int RS, int b, int t, int h, int s, float* red,
                                float* lc, float& m_out, float& z_out, float2& o_out);

// One workgroup per (query, 64-head group) walks all S splits of the query in
// order (the placement for batches that fill the chip by themselves): no
// partials, no combine. Each split runs its tiles with the same MFMA and
// softmax steps as attend_dma_kernel<1>, so its (max, sum, o) has the same
// bits as that kernel's partial; it then folds into registers by SplitFold,
// the combine's order and arithmetic. A split whose logits outgrew the
// headroom is recomputed exactly here by the combine's own routine. So the
// output has the same bits as the split kernel + combine.
// Splits are only arithmetic boundaries here: the row table covers as many
// whole splits as it holds, and the tile ring streams across split ends
// (where the split's result folds in and its accumulators restart). The
// exact recompute has LDS of its own, so tiles stay in flight meanwhile.
// (The pipelined loop of the split kernel holds the next tile's fragments in
// the registers that the folded output takes here.)
__global__ __launch_bounds__(kAttThreads) void attend_dma_fold_kernel(AttendArgs a, SplitPlan sp) {
  constexpr int D = 512, KS = D / 32, DT = D / 16;
  constexpr int RPW = kTileRows / 4;               // rows per wave per tile
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kRing][kTileRows * D];
  __shared__ int32_t rows[kMaxSplitRows];
  __shared__ float2 rope_tab[D / 2];
  __shared__ float rc_lc[kMaxSplitRows];            // exact recompute: logits of one split
  __shared__ float rc_o[D + 8];                     // its output row, then (m, z); + partial sums
  __shared__ uint32_t flag_bits[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform in a scalar register
  const int g = lane >> 4, r16 = lane & 15;
  int split0, hg, t;
  int b;
  if (!work_item_b(sp, a.Tq, split0, hg, t, b)) return;
  const bool active = wid * 16 < sp.HG;
  const int head = hg * sp.HG + wid * 16 + r16;
  const RowSpan rs = row_span(a, b, t);
  fill_rope_table(a, b, t, rope_tab);              // read after the tile loop's barriers
  const int64_t win_rows = a.W - 1 + a.Tq;
  const uint16_t* kvp = static_cast<const uint16_t*>(a.kv) + static_cast<int64_t>(b) * a.N_cap * D;
  const uint16_t* winp = static_cast<const uint16_t*>(a.win) + static_cast<int64_t>(b) * win_rows * D;
  const SwzOffsets so = swz_offsets(g, r16);
  const int tps = sp.RS / kTileRows;               // tiles per split
  const int spc = kMaxSplitRows / sp.RS;           // splits per row table

  bf16x8 qf[KS];
  if (active) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g));
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
  }
  f32x4 U[DT];                                     // folded output, relative to fold.M
#pragma unroll
  for (int i = 0; i < DT; ++i) U[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  SplitFold fold = fold_start(active ? a.sink[head] : 0.f);

  for (int c0 = split0; c0 < split0 + sp.SPW; c0 += spc) {
    const int c1 = min(c0 + spc, split0 + sp.SPW);  // splits [c0, c1) in this row table
    __syncthreads();                               // the last table's reads of rows[] and the ring are done
    const int64_t r_begin = static_cast<int64_t>(c0) * sp.RS;
    int64_t r_end = static_cast<int64_t>(c1) * sp.RS;
    if (r_end > rs.nrows) r_end = rs.nrows;
    const int nr = r_end > r_begin ? static_cast<int>(r_end - r_begin) : 0;
    int32_t myrows[kMaxSplitRows / kAttThreads];
#pragma unroll
    for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) {
      const int v = tid + kAttThreads * q;
      myrows[q] = v < nr ? encode_row(a, b, t, rs, r_begin + v) : -1;
    }
#pragma unroll
    for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) rows[tid + kAttThreads * q] = myrows[q];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // tile copies as in attend_dma_kernel (swizzled 1 KB rows, absent rows
    // copy window row 0 and are masked out of the softmax)
    auto issue = [&](int tile, uint16_t* dst) {
      const int v0 = tile * kTileRows + wid * RPW;
      uint64_t my = 0;
      if (lane < RPW) {
        const int v = v0 + lane;
        const int32_t sr = v < nr ? rows[v] : -1;
        const uint16_t* rowp = sr >= 0 ? kvp + static_cast<int64_t>(sr) * D
                                       : winp + (sr == -1 ? 0 : static_cast<int64_t>(-2 - sr) * D);
        my = reinterpret_cast<uint64_t>(rowp);
      }
      const uint32_t lds0 = lds_address(dst + wid * RPW * D);
      const uint32_t lo = static_cast<uint32_t>(my), hi = static_cast<uint32_t>(my >> 32);
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const uint64_t rb = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), rr))) << 32) |
                            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), rr));
        const uint32_t src_off = 16u * static_cast<uint32_t>((lane & 48) | ((lane & 15) ^ slot_swizzle(wid * RPW + rr)));
        lds_copy16(reinterpret_cast<const void*>(rb + src_off), lds0 + rr * D * 2);
      }
    };
    const int ntiles = (nr + kTileRows - 1) / kTileRows;
#pragma unroll
    for (int t0 = 0; t0 < kRing - 1; ++t0)
      if (t0 < ntiles) issue(t0, Xs[t0]);
    f32x4 acc_o[DT];
    float m_run = -INFINITY, z_run = 0.f;
    bool flag = false;
#pragma unroll
    for (int i = 0; i < DT; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Every split of [c0, c1) ends on a tile boundary (RS is a multiple of the
    // tile); splits past the query's rows have no tiles and fold as empty.
    const int nsplit = c1 - c0;
    for (int sl = 0, it = 0; sl < nsplit; ++sl) {
      const int it_end = min(ntiles, (sl + 1) * tps);
      for (; it < it_end; ++it) {
        // tile it: wait for it (tiles it + 1, it + 2 may stay in flight),
        // refill the slot of tile it - 1 with tile it + 3, then S^T, softmax,
        // output update
        const int later = min(ntiles - 1, it + kRing - 2) - it;
        if (later >= 2) wait_vmcnt<2 * RPW>();
        else if (later == 1) wait_vmcnt<RPW>();
        else wait_vmcnt<0>();
        if (it == 0) __builtin_amdgcn_s_waitcnt(0);  // query fragments too
        __builtin_amdgcn_s_barrier();               // bare: the freed slot's reads fed MFMAs already
        if (it + kRing - 1 < ntiles) issue(it + kRing - 1, Xs[(it + kRing - 1) % kRing]);
        const uint16_t* X = Xs[it % kRing];
        const char* xb = reinterpret_cast<const char*>(X);
        const int v0 = it * kTileRows;
        int4 rv[2];
        rv[0] = *reinterpret_cast<const int4*>(rows + v0 + 4 * g);
        rv[1] = *reinterpret_cast<const int4*>(rows + v0 + 16 + 4 * g);
        // S^T = X Q^T as qk_load + qk_mfma do it (K steps in order, row halves
        // inner), with the fragments loaded half the K steps at a time
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int qtr = 0; qtr < 4; ++qtr) {
          bf16x8 xf[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int st = 4 * qtr + (j >> 1), h2 = j & 1;
            xf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xb + so.qk[st & 3] + h2 * 16384 + 256 * (st >> 2)));
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int st = 4 * qtr + (j >> 1), h2 = j & 1;
            sacc[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[j], qf[st], sacc[h2], 0, 0, 0);
          }
        }
        bf16x8 pf;
        softmax_update_regs(sacc, rv, a.scale, m_run, z_run, flag, pf);
        // output update in four channel quarters (same MFMAs, fewer live fragments)
        {
          bf16x8 v0f[8];
          pv_load<0, 8>(X, so, v0f);
          pv_mfma<0, 8>(v0f, pf, acc_o);
        }
        {
          bf16x8 v1f[8];
          pv_load<8, 8>(X, so, v1f);
          pv_mfma<8, 8>(v1f, pf, acc_o);
        }
        {
          bf16x8 v2f[8];
          pv_load<16, 8>(X, so, v2f);
          pv_mfma<16, 8>(v2f, pf, acc_o);
        }
        {
          bf16x8 v3f[8];
          pv_load<24, 8>(X, so, v3f);
          pv_mfma<24, 8>(v3f, pf, acc_o);
        }
      }

      // split c0 + sl ends: flagged heads are recomputed exactly by the whole
      // workgroup (the owning lanes take the result), then the split folds in
      const int split = c0 + sl;
      if (tid < 2) flag_bits[tid] = 0u;
      __syncthreads();
      if (active && g == 0 && flag) atomicOr(&flag_bits[wid >> 1], 1u << (16 * (wid & 1) + r16));
      __syncthreads();
      const uint64_t todo = static_cast<uint64_t>(flag_bits[0]) | (static_cast<uint64_t>(flag_bits[1]) << 32);
      if (todo) {
        for (int hh = 0; hh < sp.HG; ++hh) {
          if (!((todo >> hh) & 1u)) continue;       // uniform across the block
          float mx, zx;
          float2 ox;
          recompute_split(a, sp.RS, b, t, hg * sp.HG + hh, split, rc_o + D + 2, rc_lc, mx, zx, ox);
          if (2 * tid < D) {
            rc_o[2 * tid] = ox.x;
            rc_o[2 * tid + 1] = ox.y;
          }
          __syncthreads();
          if (tid == 0) {
            rc_o[D] = mx;
            rc_o[D + 1] = zx;
          }
          __syncthreads();
          if (wid == hh / 16 && r16 == hh % 16) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc_o[dt][i] = rc_o[16 * dt + 4 * g + i];
            m_run = rc_o[D];
            z_run = rc_o[D + 1];
          }
          __syncthreads();                          // rc_o free for the next head
        }
      }
      float ca, cc;
      fold_coeffs(fold, m_run, z_run, ca, cc);
      // a split's output folds as bf16, as the split kernel stores it, unless
      // it was recomputed (the exact path keeps fp32 in both placements)
      if (!((todo >> (wid * 16 + r16)) & 1u)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const uint32_t w = pack_bf16x2(acc_o[dt][i], acc_o[dt][i + 1]);
            acc_o[dt][i] = bf16_to_f32(static_cast<uint16_t>(w & 0xffffu));
            acc_o[dt][i + 1] = bf16_to_f32(static_cast<uint16_t>(w >> 16));
          }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          U[dt][i] = fmaf(U[dt][i], ca, acc_o[dt][i] * cc);
          // keep the folded output in accumulation registers across the next
          // split's tiles (the vector registers hold their fragments)
          asm volatile("" : "+a"(U[dt][i]));
          acc_o[dt][i] = 0.f;
        }
      m_run = -INFINITY;
      z_run = 0.f;
      flag = false;
    }
  }
  if (active) store_folded<D>(a, b, t, head, g, [&](int dt, int i) { return U[dt][i]; }, fold, rope_tab);
}

// ---------------------------------------------------------------------------
// Mixed rows (448 x e4m3fn bytes + 64 x bf16, one fp32 scale per row), D = 512.
// Raw 576-byte rows go HBM -> LDS by DMA into a ring of four raw tiles (with
// the 32 row scales copied beside each), a conversion pass turns each tile's
// fp8 bytes into bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 at scale 1: every
// e4m3fn value is a bf16 value), and the swizzled bf16 tile feeds the same
// MFMA code as bf16 rows. The row scale s multiplies only the fp8 channels, so
// the logit is s * (fp8-part dot) + (bf16-part dot) from two accumulators, and
// the P operand is p * s for output channels 0..447 and p for 448..511.
// ---------------------------------------------------------------------------
constexpr int kMixRow = 576;                     // stored bytes per row
constexpr int kRawRing = 4;
constexpr int kRawTile = kTileRows * kMixRow;    // 18432 bytes = 18 copies of 1 KB
constexpr int kRawSlot = kRawTile + 256;         // + 64 floats: row scales (32 used)

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Raw tile -> bf16 tile (row r's logical 16-byte slot c at physical slot
// c ^ swz(r)). Work unit: one 16-byte raw chunk; 28 fp8 chunks and 8 bf16
// chunks per row.
__device__ __forceinline__ void convert_mixed_tile(const uint8_t* raw, uint16_t* X) {
  char* xb = reinterpret_cast<char*>(X);
  for (int u = threadIdx.x; u < kTileRows * 36; u += kAttThreads) {
    const int r = u / 36, k = u - 36 * r;
    const int sw = slot_swizzle(r);
    const uint4 v = *reinterpret_cast<const uint4*>(raw + r * kMixRow + 16 * k);
    char* row = xb + r * 1024;
    if (k < 28) {
      uint4 lo, hi;
      lo.x = fp8x2_to_bf16x2<false>(v.x);
      lo.y = fp8x2_to_bf16x2<true>(v.x);
      lo.z = fp8x2_to_bf16x2<false>(v.y);
      lo.w = fp8x2_to_bf16x2<true>(v.y);
      hi.x = fp8x2_to_bf16x2<false>(v.z);
      hi.y = fp8x2_to_bf16x2<true>(v.z);
      hi.z = fp8x2_to_bf16x2<false>(v.w);
      hi.w = fp8x2_to_bf16x2<true>(v.w);
      *reinterpret_cast<uint4*>(row + 16 * ((2 * k) ^ sw)) = lo;
      *reinterpret_cast<uint4*>(row + 16 * ((2 * k + 1) ^ sw)) = hi;
    } else {
      *reinterpret_cast<uint4*>(row + 16 * ((56 + k - 28) ^ sw)) = v;
    }
  }
}

__device__ __forceinline__ void softmax_update_mixed(const f32x4 (&sa)[2], const f32x4 (&sb)[2], int v0,
                                                     const int32_t* rows, const float* rsc, float scale, int g,
                                                     float& m_run, float& z_run, bool& flag, bf16x8& pa,
                                                     bf16x8& pb) {
  const int4 rv0 = *reinterpret_cast<const int4*>(rows + v0 + 4 * g);
  const int4 rv1 = *reinterpret_cast<const int4*>(rows + v0 + 16 + 4 * g);
  const float4 s0 = *reinterpret_cast<const float4*>(rsc + 4 * g);
  const float4 s1 = *reinterpret_cast<const float4*>(rsc + 16 + 4 * g);
  const int rr[8] = {rv0.x, rv0.y, rv0.z, rv0.w, rv1.x, rv1.y, rv1.z, rv1.w};
  const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float lg[8];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float l = rr[i] != -1 ? (sa[i >> 2][i & 3] * sc[i] + sb[i >> 2][i & 3]) * scale : -INFINITY;
    lg[i] = l;
    mx = fmaxf(mx, l);
  }
  mx = pair_max32(pair_max16(mx));
  if (m_run == -INFINITY) m_run = mx;
  flag = flag || (mx > m_run + kHeadroom);
  float psum = 0.f;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = lg[i] == -INFINITY ? 0.f : __expf(fminf(lg[i] - m_run, kHeadroom));
    psum += p[i];
  }
  z_run += pair_sum32(pair_sum16(psum));
  uint4 wa, wb;
  wa.x = pack_bf16x2(p[0] * sc[0], p[1] * sc[1]);
  wa.y = pack_bf16x2(p[2] * sc[2], p[3] * sc[3]);
  wa.z = pack_bf16x2(p[4] * sc[4], p[5] * sc[5]);
  wa.w = pack_bf16x2(p[6] * sc[6], p[7] * sc[7]);
  wb.x = pack_bf16x2(p[0], p[1]);
  wb.y = pack_bf16x2(p[2], p[3]);
  wb.z = pack_bf16x2(p[4], p[5]);
  wb.w = pack_bf16x2(p[6], p[7]);
  pa = __builtin_bit_cast(bf16x8, wa);
  pb = __builtin_bit_cast(bf16x8, wb);
}

__device__ __forceinline__ void tile_softmax_mixed(const uint16_t* X, const SwzOffsets& so, int v0,
                                                   const int32_t* rows, const float* rsc, const bf16x8 (&qf)[16],
                                                   float scale, int g, float& m_run, float& z_run, bool& flag,
                                                   bf16x8& pa, bf16x8& pb) {
  const char* xb = reinterpret_cast<const char*>(X);
  f32x4 sa[2], sb[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    f32x4 acc_a = {0.f, 0.f, 0.f, 0.f}, acc_b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j0 = 0; j0 < 4; j0 += 2) {
      uint4 xa[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + (e >> 2), k = e & 3;
        xa[e] = *reinterpret_cast<const uint4*>(xb + so.qk[k] + h2 * 16384 + 256 * j);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ks = 4 * (j0 + (e >> 2)) + (e & 3);          // K step: channels 32 ks .. 32 ks + 31
        if (ks < 14) acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[e]), qf[ks], acc_a, 0, 0, 0);
        else acc_b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[e]), qf[ks], acc_b, 0, 0, 0);
      }
    }
    sa[h2] = acc_a;
    sb[h2] = acc_b;
  }
  softmax_update_mixed(sa, sb, v0, rows, rsc, scale, g, m_run, z_run, flag, pa, pb);
}

__device__ __forceinline__ void tile_pv_mixed(const uint16_t* X, const SwzOffsets& so, const bf16x8& pa,
                                              const bf16x8& pb, f32x4 (&acc_o)[32]) {
  const char* xb = reinterpret_cast<const char*>(X);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x8 af[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(xb + so.pv[k] + 256 * j));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(xb + so.pv[k] + 256 * j + 16384));
      const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
      af[k] = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)                    // channel tile 8j + k: fp8 part below 28
      acc_o[8 * j + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[k], 8 * j + k < 28 ? pa : pb, acc_o[8 * j + k], 0, 0, 0);
  }
}

// One mixed tile for a wave serving 32 heads (two 16-head tiles): as
// tile_step_32, with S^T split into the fp8-channel accumulator (K steps
// 0..13, scaled by the row scale in the softmax) and the bf16-channel one,
// and P scaled by the row scale on the fp8 channel tiles.
__device__ __forceinline__ void tile_step_mixed_32(const uint16_t* X, const SwzOffsets& so, int v0,
                                                   const int32_t* rows, const float* rsc,
                                                   const bf16x8 (&qf)[2][16], float scale, int g,
                                                   float (&m_run)[2], float (&z_run)[2], bool (&flag)[2],
                                                   f32x4 (&acc_o)[2][32]) {
  const char* xb = reinterpret_cast<const char*>(X);
  f32x4 sa[2][2], sb[2][2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) sa[ht][0] = sa[ht][1] = sb[ht][0] = sb[ht][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  __builtin_amdgcn_sched_barrier(0);
  {
    bf16x8 xf[32];
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const int st = f >> 1, h2 = f & 1;
      xf[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xb + so.qk[st & 3] + h2 * 16384 + 256 * (st >> 2)));
    }
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const int st = f >> 1, h2 = f & 1;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        if (st < 14) sa[ht][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[f], qf[ht][st], sa[ht][h2], 0, 0, 0);
        else sb[ht][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[f], qf[ht][st], sb[ht][h2], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // first four fragments
#pragma unroll
    for (int i = 0; i < 28; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one fragment read ...
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // ... and the two MFMAs of a landed one
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 pa[2], pb[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
    softmax_update_mixed(sa[ht], sb[ht], v0, rows, rsc, scale, g, m_run[ht], z_run[ht], flag[ht], pa[ht], pb[ht]);
  __builtin_amdgcn_sched_barrier(0);
  {
    bf16x8 vf[32];
    pv_load(X, so, vf);
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)                 // channel tile dt: fp8 part below 28
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        acc_o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], dt < 28 ? pa[ht] : pb[ht], acc_o[ht][dt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);     // first four fragments (two reads each)
#pragma unroll
    for (int i = 0; i < 28; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// NHT 16-head tiles per wave, as attend_dma_kernel.
template <int NHT>
__global__ __launch_bounds__(kAttThreads) void attend_mixed_dma_kernel(AttendArgs a, SplitPlan sp,
                                                                       float* __restrict__ part_o,
                                                                       float* __restrict__ part_ml) {
  constexpr int D = 512, KS = D / 32, DT = D / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t Raw[kRawRing][kRawSlot];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kTileRows * D];
  __shared__ __attribute__((aligned(16))) int32_t rows[kMaxSplitRows];
  __shared__ float2 rope_tab[D / 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  int split, hg, t;
  int b;
  if (!work_item_b(sp, a.Tq, split, hg, t, b)) return;
  const bool active = wid * 16 * NHT < sp.HG;
  const int head0 = hg * sp.HG + wid * 16 * NHT + r16;   // + 16 ht for head tile ht
  const RowSpan rs = row_span(a, b, t);
  if (sp.S == 1) fill_rope_table(a, b, t, rope_tab);
  const int64_t r_begin = static_cast<int64_t>(split) * sp.RS;
  int64_t r_end = r_begin + sp.RS;
  if (r_end > rs.nrows) r_end = rs.nrows;
  const int nr = r_end > r_begin ? static_cast<int>(r_end - r_begin) : 0;

  int32_t myrows[kMaxSplitRows / kAttThreads];
#pragma unroll
  for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) {
    const int v = tid + kAttThreads * q;
    myrows[q] = v < nr ? encode_row(a, b, t, rs, r_begin + v) : -1;
  }
#pragma unroll
  for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) rows[tid + kAttThreads * q] = myrows[q];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int64_t win_rows = a.W - 1 + a.Tq;
  const uint8_t* kvb = static_cast<const uint8_t*>(a.kv) + static_cast<int64_t>(b) * a.N_cap * kMixRow;
  const uint8_t* winb = static_cast<const uint8_t*>(a.win) + static_cast<int64_t>(b) * win_rows * kMixRow;
  const float* kvs = a.kv_scale + static_cast<int64_t>(b) * a.N_cap;
  const float* wins = a.win_scale + static_cast<int64_t>(b) * win_rows;
  // Tile copies: 18 of 1 KB (lane l of copy c fetches tile byte 1024 c + 16 l)
  // and the 32 row scales (4 bytes per lane, twice so that every wave issues
  // exactly five copies per tile). Absent rows copy window row 0.
  auto issue = [&](int tile, int slot) {
    const int v0 = tile * kTileRows;
    uint8_t* base = &Raw[slot][0];
#pragma unroll
    for (int cc = 0; cc < 5; ++cc) {
      const int c = wid * 5 + cc;
      if (c < 18) {
        const int q = c * 1024 + 16 * lane;
        const int r = q / kMixRow, off = q - r * kMixRow;
        const int v = v0 + r;
        const int32_t sr = v < nr ? rows[v] : -1;
        const uint8_t* rowp = sr >= 0 ? kvb + static_cast<int64_t>(sr) * kMixRow
                                      : winb + (sr == -1 ? 0 : static_cast<int64_t>(-2 - sr) * kMixRow);
        lds_copy16(rowp + off, lds_address(base) + c * 1024);
      } else {
        const int v = v0 + (lane < kTileRows ? lane : 0);
        const int32_t sr = v < nr ? rows[v] : -1;
        const float* sp_ = sr >= 0 ? kvs + sr : wins + (sr == -1 ? 0 : -2 - sr);
        lds_copy4(sp_, lds_address(base + kRawTile));
      }
    }
  };
  const int ntiles = (nr + kTileRows - 1) / kTileRows;
#pragma unroll
  for (int t0 = 0; t0 < 3; ++t0)
    if (t0 < ntiles) issue(t0, t0);
  bf16x8 qf[NHT][KS];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    if (active) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head0 + 16 * ht) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qf[ht][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g));
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[ht][s] = bf16x8{};
    }
  }
  f32x4 acc_o[NHT][DT];
  float m_run[NHT], z_run[NHT];
  bool flag[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
    for (int i = 0; i < DT; ++i) acc_o[ht][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[ht] = -INFINITY;
    z_run[ht] = 0.f;
    flag[ht] = false;
  }
  const SwzOffsets so = swz_offsets(g, r16);
  __builtin_amdgcn_s_waitcnt(0);                   // tiles 0..2 and the query fragments
  __builtin_amdgcn_s_barrier();
  if (0 < ntiles) convert_mixed_tile(&Raw[0][0], Xs[0]);

  // Step it: (raw tile it+1 landed, everyone past tile it-1) -> refill the raw
  // slot of tile it-1 with tile it+3 -> convert tile it+1 -> consume tile it.
  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) {
      if (it + 2 < ntiles) wait_vmcnt<5>();        // tile it+2's copies may stay in flight
      else wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (it + 3 < ntiles) issue(it + 3, (it + 3) % kRawRing);
    if (it + 1 < ntiles) convert_mixed_tile(&Raw[(it + 1) % kRawRing][0], Xs[(it + 1) & 1]);
    const float* rsc = reinterpret_cast<const float*>(&Raw[it % kRawRing][kRawTile]);
    if constexpr (NHT == 1) {
      bf16x8 pa, pb;
      tile_softmax_mixed(Xs[it & 1], so, it * kTileRows, rows, rsc, qf[0], a.scale, g, m_run[0], z_run[0], flag[0],
                         pa, pb);
      tile_pv_mixed(Xs[it & 1], so, pa, pb, acc_o[0]);
    } else {
      tile_step_mixed_32(Xs[it & 1], so, it * kTileRows, rows, rsc, qf, a.scale, g, m_run, z_run, flag, acc_o);
    }
  }

  if (active) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int head = head0 + 16 * ht;
      const int64_t part_idx = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * sp.S + split;
      if (sp.S == 1) {
        write_output<D>(a, b, t, head, g, acc_o[ht], m_run[ht], z_run[ht], flag[ht], rope_tab, part_ml + 2 * part_idx);
      } else {
        // bf16 partial (32-byte pieces per head: plain stores, which the L2 merges into lines)
        uint16_t* pob = reinterpret_cast<uint16_t*>(part_o) + part_idx * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<uint2*>(pob + 16 * dt + 4 * g) =
              make_uint2(pack_bf16x2(acc_o[ht][dt][0], acc_o[ht][dt][1]), pack_bf16x2(acc_o[ht][dt][2], acc_o[ht][dt][3]));
        if (g == 0) {
          part_ml[2 * part_idx] = flag[ht] ? __builtin_nanf("") : m_run[ht];   // NaN: recompute in combine
          part_ml[2 * part_idx + 1] = z_run[ht];
        }
      }
    }
  }
}

// One workgroup per (query, 64-head group) over all S splits of the query,
// for mixed rows: attend_dma_fold_kernel's placement with
// attend_mixed_dma_kernel's tiles (raw ring, conversion pass, per-head MFMA
// chains and softmax of the 64-head mixed kernel, which are those of the
// 128-head one too). Each split's (max, sum, o) therefore has the bits of the
// split kernels' partial, and it folds by SplitFold as the combine does.
__global__ __launch_bounds__(kAttThreads) void attend_mixed_fold_kernel(AttendArgs a, SplitPlan sp) {
  constexpr int D = 512, KS = D / 32, DT = D / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t Raw[kRawRing][kRawSlot];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kTileRows * D];
  __shared__ __attribute__((aligned(16))) int32_t rows[kMaxSplitRows];
  __shared__ float2 rope_tab[D / 2];
  __shared__ float rc_lc[kMaxSplitRows];            // exact recompute: logits of one split
  __shared__ float rc_o[D + 8];                     // its output row, then (m, z); + partial sums
  __shared__ uint32_t flag_bits[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  int split0, hg, t;
  int b;
  if (!work_item_b(sp, a.Tq, split0, hg, t, b)) return;
  const bool active = wid * 16 < sp.HG;
  const int head = hg * sp.HG + wid * 16 + r16;
  const RowSpan rs = row_span(a, b, t);
  fill_rope_table(a, b, t, rope_tab);              // read after the tile loop's barriers
  const int64_t win_rows = a.W - 1 + a.Tq;
  const uint8_t* kvb = static_cast<const uint8_t*>(a.kv) + static_cast<int64_t>(b) * a.N_cap * kMixRow;
  const uint8_t* winb = static_cast<const uint8_t*>(a.win) + static_cast<int64_t>(b) * win_rows * kMixRow;
  const float* kvs = a.kv_scale + static_cast<int64_t>(b) * a.N_cap;
  const float* wins = a.win_scale + static_cast<int64_t>(b) * win_rows;
  const SwzOffsets so = swz_offsets(g, r16);
  const int tps = sp.RS / kTileRows;               // tiles per split
  const int spc = kMaxSplitRows / sp.RS;           // splits per row table

  bf16x8 qf[KS];
  if (active) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g));
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
  }
  f32x4 U[DT];                                     // folded output, relative to fold.M
#pragma unroll
  for (int i = 0; i < DT; ++i) U[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  SplitFold fold = fold_start(active ? a.sink[head] : 0.f);

  for (int c0 = split0; c0 < split0 + sp.SPW; c0 += spc) {
    const int c1 = min(c0 + spc, split0 + sp.SPW);  // splits [c0, c1) in this row table
    __syncthreads();                               // the last table's reads of rows[] and the rings are done
    const int64_t r_begin = static_cast<int64_t>(c0) * sp.RS;
    int64_t r_end = static_cast<int64_t>(c1) * sp.RS;
    if (r_end > rs.nrows) r_end = rs.nrows;
    const int nr = r_end > r_begin ? static_cast<int>(r_end - r_begin) : 0;
    int32_t myrows[kMaxSplitRows / kAttThreads];
#pragma unroll
    for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) {
      const int v = tid + kAttThreads * q;
      myrows[q] = v < nr ? encode_row(a, b, t, rs, r_begin + v) : -1;
    }
#pragma unroll
    for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) rows[tid + kAttThreads * q] = myrows[q];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // tile copies as in attend_mixed_dma_kernel: 18 of 1 KB and the row
    // scales, five per wave; absent rows copy window row 0
    auto issue = [&](int tile, int slot) {
      const int v0 = tile * kTileRows;
      uint8_t* base = &Raw[slot][0];
#pragma unroll
      for (int cc = 0; cc < 5; ++cc) {
        const int c = wid * 5 + cc;
        if (c < 18) {
          const int q = c * 1024 + 16 * lane;
          const int r = q / kMixRow, off = q - r * kMixRow;
          const int v = v0 + r;
          const int32_t sr = v < nr ? rows[v] : -1;
          const uint8_t* rowp = sr >= 0 ? kvb + static_cast<int64_t>(sr) * kMixRow
                                        : winb + (sr == -1 ? 0 : static_cast<int64_t>(-2 - sr) * kMixRow);
          lds_copy16(rowp + off, lds_address(base) + c * 1024);
        } else {
          const int v = v0 + (lane < kTileRows ? lane : 0);
          const int32_t sr = v < nr ? rows[v] : -1;
          const float* sp_ = sr >= 0 ? kvs + sr : wins + (sr == -1 ? 0 : -2 - sr);
          lds_copy4(sp_, lds_address(base + kRawTile));
        }
      }
    };
    const int ntiles = (nr + kTileRows - 1) / kTileRows;
#pragma unroll
    for (int t0 = 0; t0 < 3; ++t0)
      if (t0 < ntiles) issue(t0, t0);
    f32x4 acc_o[DT];
    float m_run = -INFINITY, z_run = 0.f;
    bool flag = false;
#pragma unroll
    for (int i = 0; i < DT; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_waitcnt(0);                 // tiles 0..2 (and the query fragments)
    __builtin_amdgcn_s_barrier();
    if (0 < ntiles) convert_mixed_tile(&Raw[0][0], Xs[0]);
    // Every split of [c0, c1) ends on a tile boundary (RS is a multiple of the
    // tile); splits past the query's rows have no tiles and fold as empty.
    const int nsplit = c1 - c0;
    for (int sl = 0, it = 0; sl < nsplit; ++sl) {
      const int it_end = min(ntiles, (sl + 1) * tps);
      for (; it < it_end; ++it) {
        // as attend_mixed_dma_kernel: raw tile it+1 landed and everyone is
        // past tile it-1 -> refill its raw slot with tile it+3, convert tile
        // it+1, consume tile it
        if (it + 1 < ntiles) {
          if (it + 2 < ntiles) wait_vmcnt<5>();    // tile it+2's copies may stay in flight
          else wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();
        if (it + 3 < ntiles) issue(it + 3, (it + 3) % kRawRing);
        if (it + 1 < ntiles) convert_mixed_tile(&Raw[(it + 1) % kRawRing][0], Xs[(it + 1) & 1]);
        const float* rsc = reinterpret_cast<const float*>(&Raw[it % kRawRing][kRawTile]);
        bf16x8 pa, pb;
        tile_softmax_mixed(Xs[it & 1], so, it * kTileRows, rows, rsc, qf, a.scale, g, m_run, z_run, flag, pa, pb);
        tile_pv_mixed(Xs[it & 1], so, pa, pb, acc_o);
      }

      // split c0 + sl ends: flagged heads are recomputed exactly by the whole
      // workgroup (the owning lanes take the result), then the split folds in
      const int split = c0 + sl;
      if (tid < 2) flag_bits[tid] = 0u;
      __syncthreads();
      if (active && g == 0 && flag) atomicOr(&flag_bits[wid >> 1], 1u << (16 * (wid & 1) + r16));
      __syncthreads();
      const uint64_t todo = static_cast<uint64_t>(flag_bits[0]) | (static_cast<uint64_t>(flag_bits[1]) << 32);
      if (todo) {
        for (int hh = 0; hh < sp.HG; ++hh) {
          if (!((todo >> hh) & 1u)) continue;       // uniform across the block
          float mx, zx;
          float2 ox;
          recompute_split(a, sp.RS, b, t, hg * sp.HG + hh, split, rc_o + D + 2, rc_lc, mx, zx, ox);
          if (2 * tid < D) {
            rc_o[2 * tid] = ox.x;
            rc_o[2 * tid + 1] = ox.y;
          }
          __syncthreads();
          if (tid == 0) {
            rc_o[D] = mx;
            rc_o[D + 1] = zx;
          }
          __syncthreads();
          if (wid == hh / 16 && r16 == hh % 16) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc_o[dt][i] = rc_o[16 * dt + 4 * g + i];
            m_run = rc_o[D];
            z_run = rc_o[D + 1];
          }
          __syncthreads();                          // rc_o free for the next head
        }
      }
      float ca, cc;
      fold_coeffs(fold, m_run, z_run, ca, cc);
      // a split's output folds as bf16, as the split kernels store it, unless
      // it was recomputed (the exact path keeps fp32 in both placements)
      if (!((todo >> (wid * 16 + r16)) & 1u)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const uint32_t w = pack_bf16x2(acc_o[dt][i], acc_o[dt][i + 1]);
            acc_o[dt][i] = bf16_to_f32(static_cast<uint16_t>(w & 0xffffu));
            acc_o[dt][i + 1] = bf16_to_f32(static_cast<uint16_t>(w >> 16));
          }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          U[dt][i] = fmaf(U[dt][i], ca, acc_o[dt][i] * cc);
          asm volatile("" : "+a"(U[dt][i]));
          acc_o[dt][i] = 0.f;
        }
      m_run = -INFINITY;
      z_run = 0.f;
      flag = false;
    }
  }
  if (active) store_folded<D>(a, b, t, head, g, [&](int dt, int i) { return U[dt][i]; }, fold, rope_tab);
}

// ---------------------------------------------------------------------------
// float32 kernel on the vector ALUs
// ---------------------------------------------------------------------------
constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads) void attend_f32_kernel(AttendArgs a, SplitPlan sp,
                                                                 float* __restrict__ part_o,
                                                                 float* __restrict__ part_ml) {
  extern __shared__ float sm[];
  const int D = a.D, HG = sp.HG;
  float* X = sm;                                 // [32][D]
  float* Q = X + kTileRows * D;                  // [HG][D]
  float* P = Q + HG * D;                         // [32][HG]
  float* AL = P + kTileRows * HG;                // [HG] alpha of the current tile
  float* MZ = AL + HG;                           // [HG][2] running max / sum
  __shared__ int64_t src_row[kTileRows];
  __shared__ int src_kind[kTileRows];
  const int tid = threadIdx.x;
  const int split = blockIdx.x / sp.n_hg, hg = blockIdx.x % sp.n_hg;
  const int t = blockIdx.y, b = blockIdx.z;
  const int h0 = hg * HG;
  const int nh = min(HG, a.H - h0);
  const RowSpan rs = row_span(a, b, t);
  const int64_t r_begin = static_cast<int64_t>(split) * sp.RS;
  int64_t r_end = r_begin + sp.RS;
  if (r_end > rs.nrows) r_end = rs.nrows;

  const float* qp = static_cast<const float*>(a.q) + ((static_cast<int64_t>(b) * a.Tq + t) * a.H + h0) * D;
  for (int i = tid; i < nh * D; i += kF32Threads) Q[i] = qp[i];
  for (int h = tid; h < HG; h += kF32Threads) { MZ[2 * h] = -INFINITY; MZ[2 * h + 1] = 0.f; }
  constexpr int kMaxOut = 16;
  float acc[kMaxOut];
#pragma unroll
  for (int i = 0; i < kMaxOut; ++i) acc[i] = 0.f;
  __syncthreads();

  for (int64_t t0 = r_begin; t0 < r_end; t0 += kTileRows) {
    if (tid < kTileRows) {
      int kind;
      const int64_t v = t0 + tid;
      src_row[tid] = v < r_end ? row_source(a, b, t, rs, v, &kind) : -1;
      src_kind[tid] = v < r_end ? kind : 0;
    }
    __syncthreads();
    for (int i = tid; i < kTileRows * D; i += kF32Threads) {
      const int r = i / D, d = i % D;
      const int64_t sr = src_row[r];
      float x = 0.f;
      if (sr >= 0)
        x = src_kind[r] == 0 ? static_cast<const float*>(a.kv)[(static_cast<int64_t>(b) * a.N_cap + sr) * D + d]
                             : static_cast<const float*>(a.win)[(static_cast<int64_t>(b) * (a.W - 1 + a.Tq) + sr) * D + d];
      X[i] = x;
    }
    __syncthreads();
    for (int pr = tid; pr < kTileRows * nh; pr += kF32Threads) {
      const int r = pr / nh, h = pr % nh;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(Q[h * D + d], X[r * D + d], dot);
      P[r * HG + h] = src_row[r] >= 0 ? dot * a.scale : -INFINITY;
    }
    __syncthreads();
    for (int h = tid; h < nh; h += kF32Threads) {
      float mx = -INFINITY;
      for (int r = 0; r < kTileRows; ++r) mx = fmaxf(mx, P[r * HG + h]);
      const float m_old = MZ[2 * h];
      const float m_new = fmaxf(m_old, mx);
      float alpha = 1.f, s = 0.f;
      if (m_new != -INFINITY) {
        alpha = m_old == -INFINITY ? 0.f : expf(m_old - m_new);
        for (int r = 0; r < kTileRows; ++r) {
          const float l = P[r * HG + h];
          const float pv = l == -INFINITY ? 0.f : expf(l - m_new);
          P[r * HG + h] = pv;
          s += pv;
        }
      } else {
        for (int r = 0; r < kTileRows; ++r) P[r * HG + h] = 0.f;
      }
      MZ[2 * h] = m_new;
      MZ[2 * h + 1] = MZ[2 * h + 1] * alpha + s;
      AL[h] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxOut; ++i) {
      const int o = tid + i * kF32Threads;
      if (o < nh * D) {
        const int h = o / D, d = o % D;
        float v = acc[i] * AL[h];
        for (int r = 0; r < kTileRows; ++r) v = fmaf(P[r * HG + h], X[r * D + d], v);
        acc[i] = v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kMaxOut; ++i) {
    const int o = tid + i * kF32Threads;
    if (o < nh * D) {
      const int h = o / D, d = o % D;
      const int64_t pi = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + h0 + h) * sp.S + split;
      part_o[pi * D + d] = acc[i];
    }
  }
  for (int h = tid; h < nh; h += kF32Threads) {
    const int64_t pi = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + h0 + h) * sp.S + split;
    part_ml[2 * pi] = MZ[2 * h];
    part_ml[2 * pi + 1] = MZ[2 * h + 1];
  }
}

// ---------------------------------------------------------------------------
// combine: merge split partials, add the sink, normalise, inverse RoPE.
// One workgroup per (sequence, query, head); thread c owns channel pair
// (2c, 2c+1). Split maxima/sums and the partial rows are loaded together, so
// the kernel makes a single round trip to memory.
// ---------------------------------------------------------------------------
constexpr int kCombBatch = 16;      // splits per register batch
constexpr int kCombMaxRows = 2048;  // logits cached by the exact recompute

// Channel pair (2c, 2c+1) of one stored row, as float.
__device__ __forceinline__ float2 load_pair(const AttendArgs& a, int b, int64_t src, int kind, int c) {
  const int D = a.D;
  const int64_t ridx = kind == 0 ? static_cast<int64_t>(b) * a.N_cap + src
                                 : static_cast<int64_t>(b) * (a.W - 1 + a.Tq) + src;
  const void* base = kind == 0 ? a.kv : a.win;
  if (a.dt_kv == LCA_F32) return reinterpret_cast<const float2*>(static_cast<const float*>(base) + ridx * D)[c];
  if (a.dt_kv == LCA_BF16) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + ridx * D)[c];
    return make_float2(bf16_to_f32(static_cast<uint16_t>(w & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(w >> 16)));
  }
  const int NQ = D - a.rope_dims;                  // mixed row: fp8 body, bf16 RoPE tail
  const uint8_t* row = static_cast<const uint8_t*>(base) + ridx * (D + a.rope_dims);
  if (2 * c < NQ) {
    const float sc = (kind == 0 ? a.kv_scale : a.win_scale)[ridx];
    return make_float2(e4m3fn_to_f32(row[2 * c]) * sc, e4m3fn_to_f32(row[2 * c + 1]) * sc);
  }
  const uint32_t w = *reinterpret_cast<const uint32_t*>(row + NQ + 2 * (2 * c - NQ));
  return make_float2(bf16_to_f32(static_cast<uint16_t>(w & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(w >> 16)));
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}

// Exact float32 recompute of one split's (max, sum, o pair) for head h: the
// slow path for splits whose logits outgrew the attention kernel's headroom.
__device__ void recompute_split(const AttendArgs& a, int RS, int b, int t, int h, int s, float* red,
                                float* lc, float& m_out, float& z_out, float2& o_out) {
  const int c = threadIdx.x;
  const bool own = 2 * c < a.D;
  const RowSpan rs = row_span(a, b, t);
  const int64_t r0 = static_cast<int64_t>(s) * RS;
  int64_t r1 = r0 + RS;
  if (r1 > rs.nrows) r1 = rs.nrows;
  float2 qv = make_float2(0.f, 0.f);
  if (own) {
    const int64_t qrow = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + h) * a.D;
    if (a.dt_q == LCA_F32) {
      qv = reinterpret_cast<const float2*>(static_cast<const float*>(a.q) + qrow)[c];
    } else {
      const uint32_t w = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + qrow)[c];
      qv = make_float2(bf16_to_f32(static_cast<uint16_t>(w & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(w >> 16)));
    }
  }
  float M = -INFINITY;
  for (int64_t v = r0; v < r1; ++v) {
    int kind;
    const int64_t src = row_source(a, b, t, rs, v, &kind);
    float part = 0.f;
    if (src >= 0 && own) {
      const float2 x = load_pair(a, b, src, kind, c);
      part = qv.x * x.x + qv.y * x.y;
    }
    // src depends only on (b, t, v): every thread takes the same branch
    const float l = src >= 0 ? block_sum(part, red) * a.scale : -INFINITY;
    if (c == 0) lc[v - r0] = l;
    M = fmaxf(M, l);
  }
  __syncthreads();
  float z = 0.f;
  float2 o = make_float2(0.f, 0.f);
  for (int64_t v = r0; v < r1; ++v) {
    const float l = lc[v - r0];
    if (l == -INFINITY) continue;
    const float p = expf(l - M);
    z += p;
    if (own) {
      int kind;
      const int64_t src = row_source(a, b, t, rs, v, &kind);
      const float2 x = load_pair(a, b, src, kind, c);
      o.x = fmaf(p, x.x, o.x);
      o.y = fmaf(p, x.y, o.y);
    }
  }
  m_out = M;
  z_out = z;
  o_out = o;
}

// Merge the S split partials of (b, t, h): the sink enters the denominator
// once, the result is normalised, its RoPE channels turned back by -p, and
// written to out (and lse). Every thread of the block calls it (it holds block
// barriers); thread c < D/2 owns channel pair (2c, 2c+1). sml holds 2S floats,
// red one float per wave, lc kCombMaxRows floats, all in LDS.
// Channel pair (2c, 2c+1) of split s's partial: fp32, or bf16 (pb16).
__device__ __forceinline__ float2 part_pair(const float* po, bool pb16, int64_t s, int D, int c) {
  if (pb16) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(po) + s * D)[c];
    return make_float2(bf16_to_f32(static_cast<uint16_t>(w & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(w >> 16)));
  }
  return *reinterpret_cast<const float2*>(po + s * D + 2 * c);
}

__device__ void combine_row(const AttendArgs& a, int S, int RS, int b, int t, int h,
                            const float* __restrict__ part_o, const float* __restrict__ part_ml,
                            float* sml, float* red, float* lc, bool pb16 = false) {
  const int c = threadIdx.x;
  const int D = a.D;
  const bool own = 2 * c < D;
  const int64_t row = (static_cast<int64_t>(b) * a.Tq + t) * a.H + h;
  const float* ml = part_ml + row * S * 2;
  const float* po = pb16 ? reinterpret_cast<const float*>(reinterpret_cast<const uint16_t*>(part_o) + row * S * D)
                        : part_o + row * S * D;
  for (int i = c; i < 2 * S; i += blockDim.x) sml[i] = ml[i];
  float2 ov[kCombBatch];
#pragma unroll
  for (int j = 0; j < kCombBatch; ++j)
    ov[j] = (j < S && own) ? part_pair(po, pb16, j, D, c) : make_float2(0.f, 0.f);
  const float sink = a.sink[h];
  __syncthreads();
  // splits flagged by the attention kernel (NaN max) are recomputed exactly
  bool any_flag = false;
  for (int s = 0; s < S; ++s) any_flag = any_flag || (sml[2 * s] != sml[2 * s]);
  if (any_flag) {
    for (int s = 0; s < S; ++s) {
      if (sml[2 * s] == sml[2 * s]) continue;      // uniform across the block
      float m, z;
      float2 o;
      recompute_split(a, RS, b, t, h, s, red, lc, m, z, o);
      __syncthreads();
      if (c == 0) { sml[2 * s] = m; sml[2 * s + 1] = z; }
#pragma unroll
      for (int j = 0; j < kCombBatch; ++j)
        if (j == s) ov[j] = o;                     // splits past the batch: recomputed below
      __syncthreads();
    }
  }
  SplitFold f = fold_start(sink);
  float u = 0.f, v = 0.f;
#pragma unroll
  for (int j = 0; j < kCombBatch; ++j) {
    if (j < S) {
      float ca, cc;
      fold_coeffs(f, sml[2 * j], sml[2 * j + 1], ca, cc);
      u = fmaf(u, ca, ov[j].x * cc);
      v = fmaf(v, ca, ov[j].y * cc);
    }
  }
  for (int s = kCombBatch; s < S; ++s) {
    float2 o = own ? part_pair(po, pb16, s, D, c) : make_float2(0.f, 0.f);
    float ms = sml[2 * s], zs = sml[2 * s + 1];
    if (any_flag && ml[2 * s] != ml[2 * s]) {       // flagged split beyond the batch: recompute again
      recompute_split(a, RS, b, t, h, s, red, lc, ms, zs, o);
    }
    float ca, cc;
    fold_coeffs(f, ms, zs, ca, cc);
    u = fmaf(u, ca, o.x * cc);
    v = fmaf(v, ca, o.y * cc);
  }
  if (own) {
    const float inv = 1.0f / f.Z;
    u *= inv;
    v *= inv;
    if (c == 0 && a.lse_out) a.lse_out[row] = f.M + logf(f.Z);
    const int R = ((a.flags & LCA_INV_ROPE) && a.rope_dims > 0) ? a.rope_dims : 0;
    const int d0 = 2 * c;
    if (d0 >= D - R) {
      float sn, cs;
      rope_sincos(-static_cast<double>(seq_pos(a.q_pos, a.q_pos0, b) + t), (d0 - (D - R)) / 2, a.rope_r, &sn, &cs);
      rope_turn(u, v, make_float2(cs, sn));
    }
    if (a.dt_q == LCA_F32) {
      float* o = static_cast<float*>(a.out) + row * D;
      o[d0] = u;
      o[d0 + 1] = v;
    } else {
      reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + row * D)[c] = pack_bf16x2(u, v);
    }
  }
  __syncthreads();                                 // sml / lc free for the next row
}

// Four heads per workgroup, one wave per head: lane l owns channels
// 8l .. 8l + 7 and loads them from every split's partial (two float4 in fp32,
// one 16-byte load in bf16), up to 16 splits in flight per batch. A workgroup whose heads hold a flagged split (max
// NaN) merges them with combine_row instead, which recomputes that split.
template <bool PB16>
__global__ __launch_bounds__(256) void combine4_kernel(AttendArgs a, int S, int RS,
                                                       const float* __restrict__ part_o,
                                                       const float* __restrict__ part_ml) {
  constexpr int NB = 16;                            // splits per batch of partial loads
  __shared__ float sml[2 * 256];
  __shared__ float red[4];
  __shared__ float lc[kCombMaxRows];
  __shared__ float2 rope_tab[256];
  __shared__ float2 wml[4][256];                    // each wave's split (max, sum) pairs
  __shared__ uint32_t any_nan;
  const int t = blockIdx.y, b = blockIdx.z, wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int D = a.D, h0 = blockIdx.x * 4, h = h0 + wid;
  const int64_t row = (static_cast<int64_t>(b) * a.Tq + t) * a.H + h;
  const bool live = h < a.H;
  const bool own = live && 8 * lane < D;
  const float* ml = part_ml + row * S * 2;
  const float* po = part_o + row * S * D + 8 * lane;
  const uint16_t* pob = reinterpret_cast<const uint16_t*>(part_o) + row * S * D + 8 * lane;
  // the first batch of partial rows and the wave's (max, sum) pairs are in
  // flight before anything waits
  float4 v[PB16 ? 1 : NB][2];
  uint4 vb[PB16 ? NB : 1];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool ok = own && s0 + j < S;
      if constexpr (PB16) {
        vb[j] = ok ? *reinterpret_cast<const uint4*>(pob + static_cast<int64_t>(s0 + j) * D) : make_uint4(0, 0, 0, 0);
      } else {
        v[j][0] = ok ? *reinterpret_cast<const float4*>(po + static_cast<int64_t>(s0 + j) * D) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[j][1] = ok ? *reinterpret_cast<const float4*>(po + static_cast<int64_t>(s0 + j) * D + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  load_batch(0);
  float2 mz[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    mz[q] = live && i < S ? *reinterpret_cast<const float2*>(ml + 2 * i) : make_float2(0.f, 0.f);
  }
  if (threadIdx.x == 0) any_nan = 0u;
  fill_rope_table(a, b, t, rope_tab);
  __syncthreads();
  bool nan_here = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = lane + 64 * q;
    if (live && i < S) {
      wml[wid][i] = mz[q];
      if (mz[q].x != mz[q].x) nan_here = true;
    }
  }
  if (nan_here) any_nan = 1u;
  __syncthreads();
  if (any_nan) {                                    // rare: exact path, head by head
    for (int hh = h0; hh < min(h0 + 4, a.H); ++hh)
      combine_row(a, S, RS, b, t, hh, part_o, part_ml, sml, red, lc, PB16);
    return;
  }
  if (!live) return;
  SplitFold f = fold_start(a.sink[h]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += NB) {
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (s0 + j < S) {
        float ca, cc;
        const float2 p = wml[wid][s0 + j];
        fold_coeffs(f, p.x, p.y, ca, cc);
        float o[8];
        if constexpr (PB16) {
          const uint32_t w4[4] = {vb[j].x, vb[j].y, vb[j].z, vb[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[2 * q] = bf16_to_f32(static_cast<uint16_t>(w4[q] & 0xffffu));
            o[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(w4[q] >> 16));
          }
        } else {
          o[0] = v[j][0].x; o[1] = v[j][0].y; o[2] = v[j][0].z; o[3] = v[j][0].w;
          o[4] = v[j][1].x; o[5] = v[j][1].y; o[6] = v[j][1].z; o[7] = v[j][1].w;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(acc[q], ca, o[q] * cc);
      }
    }
  }
  if (lane == 0 && a.lse_out) a.lse_out[row] = f.M + logf(f.Z);
  if (!own) return;
  const float inv = 1.f / f.Z;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] *= inv;
  const int R = ((a.flags & LCA_INV_ROPE) && a.rope_dims > 0) ? a.rope_dims : 0;
  const int c0 = 8 * lane;
  if (c0 >= D - R) {
#pragma unroll
    for (int p = 0; p < 4; ++p) rope_turn(acc[2 * p], acc[2 * p + 1], rope_tab[(c0 + 2 * p - (D - R)) / 2]);
  }
  if (a.dt_q == LCA_F32) {
    float* o = static_cast<float*>(a.out) + row * D + c0;
    *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    uint4 w;
    w.x = pack_bf16x2(acc[0], acc[1]);
    w.y = pack_bf16x2(acc[2], acc[3]);
    w.z = pack_bf16x2(acc[4], acc[5]);
    w.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + row * D + c0) = w;
  }
}

// One split per query: the attention kernel wrote every head's output itself
// and left (max) = +inf, except for heads whose logits outgrew the in-kernel
// headroom (max = NaN). One workgroup per (b, t) recomputes those exactly.
__global__ __launch_bounds__(256) void fixup_kernel(AttendArgs a, int RS, const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml) {
  __shared__ float sml[2 * 256];
  __shared__ float red[4];
  __shared__ float lc[kCombMaxRows];
  __shared__ uint32_t todo[8];                       // one bit per head (H <= 256)
  const int t = blockIdx.x, b = blockIdx.y;
  const int64_t row0 = (static_cast<int64_t>(b) * a.Tq + t) * a.H;
  if (threadIdx.x < 8) todo[threadIdx.x] = 0u;
  __syncthreads();
  for (int h = threadIdx.x; h < a.H; h += blockDim.x) {
    const float m0 = part_ml[2 * (row0 + h)];
    if (m0 != m0) atomicOr(&todo[h >> 5], 1u << (h & 31));
  }
  __syncthreads();
  for (int h = 0; h < a.H; ++h)
    if ((todo[h >> 5] >> (h & 31)) & 1u)             // uniform across the block
      combine_row(a, 1, RS, b, t, h, part_o, part_ml, sml, red, lc);
}

// bf16 or mixed rows of 512 channels with a multiple of 128 heads: 32 heads per wave
// 128 heads per workgroup (each row read once for all heads) for KV_MIXED rows
// and for calls of 16+ queries; bf16 decode calls take 64-head groups
// instead: the rows are read once per group, but each query needs about half
// the splits, hence half the partials (HCA decode B = 8 at 1048576: combine
// 12.0 -> 7.9 us at the same attention time).
bool heads_128(const AttendArgs& a) {
  return a.D == 512 && a.dt_q == LCA_BF16 && (a.dt_kv == LCA_KV_MIXED || (a.dt_kv == LCA_BF16 && a.Tq >= 16)) &&
         a.H % 128 == 0;
}

SplitPlan make_plan(const AttendArgs& a) {
  SplitPlan sp;
  const bool f32 = a.dt_kv == LCA_F32;
  if (f32) {
    int hg = 4096 / a.D;
    if (hg > a.H) hg = a.H;
    sp.HG = hg;
    sp.n_hg = (a.H + hg - 1) / hg;
  } else if (heads_128(a)) {
    sp.HG = 128;
    sp.n_hg = a.H / 128;
  } else {
    sp.HG = a.H < 64 ? a.H : 64;
    sp.n_hg = a.H / sp.HG;
  }
  // rows seen by the last query of the call (the most of any query)
  const int64_t p = a.q_pos0 + a.Tq - 1;
  int64_t n_ent;
  if (a.sparse) {
    n_ent = a.k;
  } else {
    n_ent = n_visible(p, a.m);
    if (n_ent > a.N_cap) n_ent = a.N_cap;
  }
  const int64_t win = p + 1 < a.W ? p + 1 : a.W;
  const int64_t nrows = n_ent + win;
  // Split size: each split writes a D-channel partial (bf16 at D = 512, fp32
  // otherwise) plus (max, sum) per head, so short splits move more partial
  // bytes than rows. With two head
  // groups (128 heads) a sequence gets 16 splits (32 workgroups), so a batch of
  // 8 fills the 256 CUs in one round; with one head group, splits of 64 rows.
  int64_t RS;
  if (sp.HG == 128 && !f32) {
    // 128 heads per workgroup: as many workgroups per query as two 64-head
    // groups with 16 splits would give (32), at least 256 rows each; mixed
    // rows at least 512 (their tiles carry a conversion pass, and a split's
    // partial weighs as much as 1.8 of their 576-byte rows)
    RS = (nrows * a.Tq + 31) / 32;
    const int64_t rs_min = a.dt_kv == LCA_KV_MIXED ? 512 : 256;
    if (RS < rs_min) RS = rs_min;
  } else if (sp.n_hg >= 2) {
    RS = (nrows * a.Tq + 15) / 16;
    if (RS < 256) RS = 256;
  } else {
    const int64_t work = nrows * a.Tq;
    RS = (work + 319) / 320;
    if (RS < 64) RS = 64;
  }
  if (RS > nrows) RS = nrows;
  RS = (RS + kTileRows - 1) / kTileRows * kTileRows;
  if (RS > kMaxSplitRows) RS = kMaxSplitRows;
  if (RS < kTileRows) RS = kTileRows;
  int64_t S = (nrows + RS - 1) / RS;
  if (S < 1) S = 1;
  if (S > 256) {                      // combine keeps split weights in LDS
    S = 256;
    RS = ((nrows + S - 1) / S + kTileRows - 1) / kTileRows * kTileRows;
  }
  sp.S = static_cast<int>(S);
  sp.RS = static_cast<int>(RS);
  sp.SPW = 1;
  sp.xcd = 0;
  sp.qmaj = 0;
  return sp;
}

template <int D>
void launch_mfma_d(LaunchScope& sc, const AttendArgs& a, const SplitPlan& sp, float* po, float* pml) {
  const int64_t W = work_blocks(sp, a.Tq);
  const dim3 grid = sp.xcd    ? dim3(static_cast<uint32_t>(W * a.B), 1, 1)
                    : sp.qmaj ? dim3(static_cast<uint32_t>(8 * qmaj_per(sp, a.Tq)), 1, a.B)
                              : dim3(static_cast<uint32_t>(W), 1, a.B);
  const dim3 block(kAttThreads);
  if constexpr (D == 512) {                        // KV_MIXED rows exist only at D = 512
    if (a.dt_kv == LCA_KV_MIXED && sp.SPW > 1)
      sc.launch(attend_mixed_fold_kernel, grid, block, 0, a, sp);
    else if (a.dt_kv == LCA_KV_MIXED && sp.HG == 128)
      sc.launch(attend_mixed_dma_kernel<2>, grid, block, 0, a, sp, po, pml);
    else if (a.dt_kv == LCA_KV_MIXED)
      sc.launch(attend_mixed_dma_kernel<1>, grid, block, 0, a, sp, po, pml);
    else if (sp.HG == 128)
      sc.launch(attend_dma_kernel<2>, grid, block, 0, a, sp, po, pml);
    else if (sp.SPW > 1)
      sc.launch(attend_dma_fold_kernel, grid, block, 0, a, sp);
    else
      sc.launch(attend_dma_kernel<1>, grid, block, 0, a, sp, po, pml);
  } else {
    sc.launch(attend_mfma_kernel<D>, grid, block, 0, a, sp, po, pml);
  }
}

}  // namespace

size_t attend_workspace(const AttendArgs& a) {
  const SplitPlan sp = make_plan(a);
  const size_t rows = static_cast<size_t>(a.B) * a.Tq * a.H * sp.S;
  return rows * (a.D + 2) * sizeof(float) + 256;
}

// Placement of a query's splits. The split kernel (one workgroup per split,
// partials, combine) spreads a query over many CUs; one workgroup per query
// and head group (all splits in turn, folded in registers) moves no partials,
// which at decode shapes weigh several times the rows themselves. Both give
// the same bits (SplitFold), so the choice may follow the batch size. The
// model: rounds of the chip (one workgroup per CU) times the bytes a workgroup
// moves per round; rows only for one workgroup per query, rows plus the
// split's partial (written, then read by the combine) for the split kernel.
// LCA_SPLITS_ONE_WG / LCA_SPLITS_MANY_WG force a placement.
constexpr int64_t kCUs = 256;

// attend_dma_fold_kernel (bf16 rows) and attend_mixed_fold_kernel (mixed
// rows): 512 channels, 64 heads per workgroup.
// A 128-head plan (attend_dma_kernel<2>) folds there too, as two 64-head
// groups over the same splits: per head that kernel runs the same MFMA chains
// and softmax as the 64-head one, so the splits' results, and the fold of
// them, keep their bits.
bool folds_in_kernel(const AttendArgs& a, const SplitPlan& sp) {
  return a.D == 512 && (a.dt_kv == LCA_BF16 || a.dt_kv == LCA_KV_MIXED) && (sp.HG != 128 || a.H % 64 == 0);
}

void place_splits(const AttendArgs& a, SplitPlan& sp) {
  if (!folds_in_kernel(a, sp) || sp.S == 1) return;
  const int fold_hg = sp.HG == 128 ? 64 : sp.HG;                          // head group of the fold kernel
  const int64_t q_items = static_cast<int64_t>(a.B) * a.Tq;
  const double rows = static_cast<double>(sp.RS) * (a.dt_kv == LCA_KV_MIXED ? kMixRow + 4 : a.D * 2);   // one split's rows
  const double part = 2.0 * sp.HG * (a.D * 2 + 8);                         // its bf16 partial + (max, sum), out and back
  const int64_t one_items = q_items * (a.H / fold_hg), split_items = q_items * sp.n_hg * sp.S;
  const double t_one = static_cast<double>((one_items + kCUs - 1) / kCUs) * sp.S * rows;
  const double t_split = static_cast<double>((split_items + kCUs - 1) / kCUs) * (rows + part);
  bool one = t_one <= t_split;
  if (a.flags & LCA_SPLITS_ONE_WG) one = true;
  if (a.flags & LCA_SPLITS_MANY_WG) one = false;
  if (one) {
    sp.SPW = sp.S;
    sp.HG = fold_hg;
    sp.n_hg = a.H / fold_hg;
  }
}

hipError_t launch_attend(hipStream_t s, const AttendArgs& a_in, void* ws, size_t) {
  AttendArgs a = a_in;
  a.rope_r = rope_ratio(a.rope_base, a.rope_dims);
  SplitPlan sp = make_plan(a);
  place_splits(a, sp);
  // 128-head workgroups in batches that fill every XCD: each sequence's
  // workgroups on one XCD, so its 128 query rows (128 KB) are fetched into one
  // L2 for all of its splits (mixed pair B = 64: hca_attend 354 -> 316 us; the
  // 64-head decode shapes measured slower this way)
  sp.xcd = a.B >= 8 && a.B % 8 == 0 && a.dt_kv != LCA_F32 && sp.HG == 128;
  sp.qmaj = !sp.xcd && a.B == 1 && a.Tq >= 64 && a.dt_kv != LCA_F32;
  if (work_blocks(sp, a.Tq) * a.B > 2147483647LL) return hipErrorInvalidConfiguration;
  const size_t rows = static_cast<size_t>(a.B) * a.Tq * a.H * sp.S;
  float* po = static_cast<float*>(ws);
  float* pml = po + rows * a.D;
  {
    LaunchScope scope(s, a.sparse ? "csa_attend" : "hca_attend");
    if (a.dt_kv == LCA_F32) {
      const size_t smem = (static_cast<size_t>(kTileRows) * a.D + static_cast<size_t>(sp.HG) * a.D +
                           kTileRows * sp.HG + 3 * sp.HG) * sizeof(float);
      scope.launch(attend_f32_kernel, dim3(sp.S * sp.n_hg, a.Tq, a.B), dim3(kF32Threads),
                   static_cast<uint32_t>(smem), a, sp, po, pml);
    } else {
      switch (a.D) {
        case 64: launch_mfma_d<64>(scope, a, sp, po, pml); break;
        case 128: launch_mfma_d<128>(scope, a, sp, po, pml); break;
        case 256: launch_mfma_d<256>(scope, a, sp, po, pml); break;
        default: launch_mfma_d<512>(scope, a, sp, po, pml); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // one workgroup per query folded its splits itself: nothing left to merge
  if (sp.SPW > 1) return hipSuccess;
  {
    LaunchScope scope(s, a.sparse ? "csa_combine" : "hca_combine");
    const dim3 cb(a.D / 2 > 64 ? a.D / 2 : 64);
    if (sp.S == 1 && a.dt_kv != LCA_F32)
      scope.launch(fixup_kernel, dim3(a.Tq, a.B), cb, 0, a, sp.RS, static_cast<const float*>(po),
                   static_cast<const float*>(pml));
    else if (a.D == 512 && a.dt_kv != LCA_F32)       // attend_dma_kernel, attend_mixed_dma_kernel: bf16 partials
      scope.launch(combine4_kernel<true>, dim3((a.H + 3) / 4, a.Tq, a.B), dim3(256), 0, a, sp.S, sp.RS,
                   static_cast<const float*>(po), static_cast<const float*>(pml));
    else
      scope.launch(combine4_kernel<false>, dim3((a.H + 3) / 4, a.Tq, a.B), dim3(256), 0, a, sp.S, sp.RS,
                   static_cast<const float*>(po), static_cast<const float*>(pml));
    return hipGetLastError();
  }
}

// ===========================================================================
// Backward of the core attention (training).
//
// [Qiaomu] 批不变 kernel and [kwkr] §4.3: the attention backward gives each
// SM its own accumulation buffer and sums the buffers in a fixed order, so
// the gradients are deterministic. Here, per query and head (P = softmax
// weights recomputed from the forward lse, do = the output gradient turned
// back by +p, D = do . o = dout . out):
//   dl_j = P_j (do . x_j - D),  dq = scale sum_j dl_j x_j,
//   dx_j = sum_h (P_hj do_h + scale dl_hj q_h),  dsink_h = -P_sink D.
// Four kernels:
//   bwd_prep_kernel   D, the turned gradient (row and [D, H] layouts), q in
//                     [D, H] layout, the sink's parts;
//   bwd_query_kernel  per (query, 64 heads): S and dP by MFMA from one set of
//                     row fragments, P and dl stored (bf16, [row][head]), dq;
//   bwd_kv_kernel     per slot (a fixed range of consecutive queries, walked
//                     in order): each row's gradient (an MFMA over the heads)
//                     added into the slot's own buffer (zeroed first);
//   bwd_reduce_kernel every entry and window row summed over the slots in
//                     slot order; bwd_sink_kernel: dsink over the queries
//                     (strided partial sums, then a fixed tree).
// ===========================================================================
namespace {

constexpr int kBwdSlotQueries = 16;                // queries per accumulation slot (at least)

struct BwdPlan {
  int64_t nr;                                      // row slots per query in the P / dl arrays
  int Ps, C;                                       // slots per sequence, queries per slot
  int wrows;                                       // window rows a slot can touch: C + W - 1
  size_t off_dor, off_dT, off_qT, off_Dv, off_dsp, off_P, off_dL, off_sE, off_sW, total;
};

BwdPlan make_bwd_plan(const AttendArgs& a) {
  BwdPlan bp{};
  const int64_t pl = a.q_pos0 + a.Tq - 1;          // the last query's position (the most rows)
  int64_t n_ent = a.k;
  if (!a.sparse) {
    n_ent = n_visible(pl, a.m);
    if (n_ent > a.N_cap) n_ent = a.N_cap;
  }
  const int64_t win = pl + 1 < a.W ? pl + 1 : a.W;
  bp.nr = (n_ent + win + kTileRows - 1) / kTileRows * kTileRows;
  // slots: one per 16 queries, at most 256 per sequence, and slot buffers within ~4 GB
  int64_t ps = (a.Tq + kBwdSlotQueries - 1) / kBwdSlotQueries;
  const double slot_bytes = static_cast<double>(a.N_cap) * a.D * 4.0 * a.B;
  int64_t cap = static_cast<int64_t>(4.0e9 / (slot_bytes > 1.0 ? slot_bytes : 1.0));
  if (cap < 1) cap = 1;
  if (ps > cap) ps = cap;
  if (ps > 256) ps = 256;
  bp.C = static_cast<int>((a.Tq + ps - 1) / ps);
  bp.Ps = (a.Tq + bp.C - 1) / bp.C;
  bp.wrows = bp.C + a.W - 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o += (bytes + 255) / 256 * 256;
    return r;
  };
  const size_t BT = static_cast<size_t>(a.B) * a.Tq;
  bp.off_dor = take(BT * a.H * a.D * 2);
  bp.off_dT = take(BT * a.H * a.D * 2);
  bp.off_qT = take(BT * a.H * a.D * 2);
  bp.off_Dv = take(BT * a.H * 4);
  bp.off_dsp = take(BT * a.H * 4);
  bp.off_P = take(BT * bp.nr * a.H * 2);
  bp.off_dL = take(BT * bp.nr * a.H * 2);
  bp.off_sE = take(static_cast<size_t>(a.B) * bp.Ps * a.N_cap * a.D * 4);
  bp.off_sW = take(static_cast<size_t>(a.B) * bp.Ps * bp.wrows * a.D * 4);
  bp.total = o;
  return bp;
}

// One workgroup per (query, sequence): D and the sink's part per head, the
// output gradient turned back by +p (the adjoint of the forward's turn by
// -p), and [D, H] copies of it and of q (the operands of the head sums).
// Requires D = 512 (eight channels per lane), H <= 128.
__device__ __forceinline__ float bwd_turn(float x, float y, bool odd, float2 cs) {
  return odd ? fmaf(x, cs.y, y * cs.x) : fmaf(x, cs.x, -(y * cs.y));
}

__global__ __launch_bounds__(256) void bwd_prep_kernel(AttendBwdArgs p, BwdPlan bp, uint8_t* ws) {
  constexpr int D = 512;
  const AttendArgs& a = p.a;
  const int t = blockIdx.x, b = blockIdx.y;
  const int H = a.H;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row0 = (static_cast<int64_t>(b) * a.Tq + t) * H;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* out = static_cast<const uint16_t*>(p.out);
  const uint16_t* dout = static_cast<const uint16_t*>(p.dout);
  uint16_t* dor = reinterpret_cast<uint16_t*>(ws + bp.off_dor);
  uint16_t* dT = reinterpret_cast<uint16_t*>(ws + bp.off_dT);
  uint16_t* qT = reinterpret_cast<uint16_t*>(ws + bp.off_qT);
  float* Dv = reinterpret_cast<float*>(ws + bp.off_Dv);
  float* dsp = reinterpret_cast<float*>(ws + bp.off_dsp);
  const int R = ((a.flags & LCA_INV_ROPE) && a.rope_dims > 0) ? a.rope_dims : 0;
  __shared__ float2 rt[256];                       // (cos, sin) of pair i at +p
  __shared__ uint16_t slab[2][128 * 64];           // 64 channels of every head (H <= 128)
  const int64_t pos = seq_pos(a.q_pos, a.q_pos0, b) + t;
  for (int i = threadIdx.x; i < R / 2; i += 256) {
    float sn, cs;
    rope_sincos(static_cast<double>(pos), i, a.rope_r, &sn, &cs);
    rt[i] = make_float2(cs, sn);
  }
  __syncthreads();
  // row layout: lane l owns channels 8 l .. 8 l + 7 of one head per wave
  for (int h = wid; h < H; h += 4) {
    const int64_t r = (row0 + h) * D + 8 * lane;
    const uint4 dw = *reinterpret_cast<const uint4*>(dout + r);
    const uint4 ow = *reinterpret_cast<const uint4*>(out + r);
    const uint32_t dv[4] = {dw.x, dw.y, dw.z, dw.w}, ov[4] = {ow.x, ow.y, ow.z, ow.w};
    float acc = 0.f;
    uint32_t tw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = bf16_to_f32(static_cast<uint16_t>(dv[j] & 0xffffu));
      const float y = bf16_to_f32(static_cast<uint16_t>(dv[j] >> 16));
      acc = fmaf(x, bf16_to_f32(static_cast<uint16_t>(ov[j] & 0xffffu)), acc);
      acc = fmaf(y, bf16_to_f32(static_cast<uint16_t>(ov[j] >> 16)), acc);
      const int c = 8 * lane + 2 * j;
      float u = x, v = y;
      if (c >= D - R) {
        const float2 cs = rt[(c - (D - R)) >> 1];
        u = bwd_turn(x, y, false, cs);
        v = bwd_turn(x, y, true, cs);
      }
      tw[j] = static_cast<uint32_t>(f32_to_bf16(u)) | (static_cast<uint32_t>(f32_to_bf16(v)) << 16);
    }
    *reinterpret_cast<uint4*>(dor + r) = make_uint4(tw[0], tw[1], tw[2], tw[3]);
    acc = wave_sum(acc);
    if (lane == 0) {
      Dv[row0 + h] = acc;
      dsp[row0 + h] = -expf(a.sink[h] - p.lse[row0 + h]) * acc;
    }
  }
  // [D, H] layouts through LDS, 64 channels at a time
  for (int c0 = 0; c0 < D; c0 += 64) {
    for (int e = threadIdx.x; e < H * 8; e += 256) {  // 8 channels per thread: coalesced loads
      const int h = e >> 3, c8 = 8 * (e & 7);
      *reinterpret_cast<uint4*>(&slab[0][h * 64 + c8]) = *reinterpret_cast<const uint4*>(q + (row0 + h) * D + c0 + c8);
      *reinterpret_cast<uint4*>(&slab[1][h * 64 + c8]) = *reinterpret_cast<const uint4*>(dout + (row0 + h) * D + c0 + c8);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < H * 64; e += 256) {
      const int c = e / H, h = e % H;
      const int64_t o = ((static_cast<int64_t>(b) * a.Tq + t) * D + c0 + c) * H + h;
      qT[o] = slab[0][h * 64 + c];
      float x = bf16_to_f32(slab[1][h * 64 + (c & ~1)]), y = bf16_to_f32(slab[1][h * 64 + (c | 1)]);
      float v = (c & 1) ? y : x;
      if (c0 + c >= D - R) v = bwd_turn(x, y, (c & 1) != 0, rt[(c0 + c - (D - R)) >> 1]);
      dT[o] = f32_to_bf16(v);
    }
    __syncthreads();
  }
}

// One workgroup per (64-head group, query, sequence), 16 heads per wave, rows
// in 32-row tiles (swizzled LDS, two-tile ring). S^T and dP^T share the row
// fragments; P = exp(l - lse) (the forward's lse), dl = P (dP - D); P and
// scale * dl go to memory as bf16 ([row][head] per query); dq^T += X^T dl^T.
__global__ __launch_bounds__(kAttThreads) void bwd_query_kernel(AttendBwdArgs p, BwdPlan bp, uint8_t* ws) {
  constexpr int D = 512, KS = D / 32, DT = D / 16, RPW = kTileRows / 4;
  const AttendArgs& a = p.a;
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][kTileRows * D];
  __shared__ int32_t rows[kMaxSplitRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int hg = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int head = hg * 64 + wid * 16 + r16;
  const int64_t qrow = (static_cast<int64_t>(b) * a.Tq + t) * a.H + head;
  const RowSpan rs = row_span(a, b, t);
  const int64_t win_rows = a.W - 1 + a.Tq;
  const uint16_t* kvp = static_cast<const uint16_t*>(a.kv) + static_cast<int64_t>(b) * a.N_cap * D;
  const uint16_t* winp = static_cast<const uint16_t*>(a.win) + static_cast<int64_t>(b) * win_rows * D;
  const SwzOffsets so = swz_offsets(g, r16);
  const float lse = p.lse[qrow];
  const float Dv = reinterpret_cast<const float*>(ws + bp.off_Dv)[qrow];
  const int64_t pl0 = (static_cast<int64_t>(b) * a.Tq + t) * bp.nr * a.H;
  uint16_t* Pw = reinterpret_cast<uint16_t*>(ws + bp.off_P) + pl0;
  uint16_t* Lw = reinterpret_cast<uint16_t*>(ws + bp.off_dL) + pl0;
  bf16x8 qf[KS], df[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow * D;
    const uint16_t* dp = reinterpret_cast<const uint16_t*>(ws + bp.off_dor) + qrow * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g));
      df[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(dp + 32 * s + 8 * g));
    }
  }
  f32x4 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t c0 = 0; c0 < rs.nrows; c0 += kMaxSplitRows) {
    const int nr = static_cast<int>(rs.nrows - c0 < kMaxSplitRows ? rs.nrows - c0 : kMaxSplitRows);
    __syncthreads();                               // the last chunk's reads of rows[] and the ring are done
    int32_t myrows[kMaxSplitRows / kAttThreads];
#pragma unroll
    for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) {
      const int v = tid + kAttThreads * q;
      myrows[q] = v < nr ? encode_row(a, b, t, rs, c0 + v) : -1;
    }
#pragma unroll
    for (int q = 0; q < kMaxSplitRows / kAttThreads; ++q) rows[tid + kAttThreads * q] = myrows[q];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto issue = [&](int tile, uint16_t* dst) {
      const int v0 = tile * kTileRows + wid * RPW;
      uint64_t my = 0;
      if (lane < RPW) {
        const int v = v0 + lane;
        const int32_t sr = v < nr ? rows[v] : -1;
        const uint16_t* rowp = sr >= 0 ? kvp + static_cast<int64_t>(sr) * D
                                       : winp + (sr == -1 ? 0 : static_cast<int64_t>(-2 - sr) * D);
        my = reinterpret_cast<uint64_t>(rowp);
      }
      const uint32_t lds0 = lds_address(dst + wid * RPW * D);
      const uint32_t lo = static_cast<uint32_t>(my), hi = static_cast<uint32_t>(my >> 32);
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        const uint64_t rb = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), rr))) << 32) |
                            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), rr));
        const uint32_t src_off = 16u * static_cast<uint32_t>((lane & 48) | ((lane & 15) ^ slot_swizzle(wid * RPW + rr)));
        lds_copy16(reinterpret_cast<const void*>(rb + src_off), lds0 + rr * D * 2);
      }
    };
    const int ntiles = (nr + kTileRows - 1) / kTileRows;
    issue(0, Xs[0]);
    for (int it = 0; it < ntiles; ++it) {
      if (it + 1 < ntiles) {
        issue(it + 1, Xs[(it + 1) & 1]);
        wait_vmcnt<RPW>();                         // tile it landed; tile it + 1 may stay in flight
      } else {
        wait_vmcnt<0>();
      }
      if (it == 0) __builtin_amdgcn_s_waitcnt(0);   // query and gradient fragments too
      __builtin_amdgcn_s_barrier();
      const uint16_t* X = Xs[it & 1];
      f32x4 sacc[2], dacc[2];
      int4 rv[2];
      {
        bf16x8 xf[32];
        qk_load(X, so, rows, it * kTileRows, g, xf, rv);
        qk_mfma(xf, qf, sacc);
        qk_mfma(xf, df, dacc);
      }
      // lane (g, r16): head r16, rows 4g + i (i < 4) and 16 + 4g + (i - 4)
      const int rr[8] = {rv[0].x, rv[0].y, rv[0].z, rv[0].w, rv[1].x, rv[1].y, rv[1].z, rv[1].w};
      float L[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float P = rr[i] != -1 ? expf(sacc[i >> 2][i & 3] * a.scale - lse) : 0.f;
        L[i] = P * (dacc[i >> 2][i & 3] - Dv);
        const int64_t v = c0 + it * kTileRows + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
        Pw[v * a.H + head] = f32_to_bf16(P);
        Lw[v * a.H + head] = f32_to_bf16(a.scale * L[i]);   // the row sums take scale * dl
      }
      uint4 lw;
      lw.x = pack_bf16x2(L[0], L[1]);
      lw.y = pack_bf16x2(L[2], L[3]);
      lw.z = pack_bf16x2(L[4], L[5]);
      lw.w = pack_bf16x2(L[6], L[7]);
      const bf16x8 lf = __builtin_bit_cast(bf16x8, lw);
      {
        bf16x8 vf[32];
        pv_load(X, so, vf);
        pv_mfma(vf, lf, acc);
      }
      __syncthreads();                             // every wave is done with this slot before its refill
    }
  }
  float* dq = p.dq + qrow * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<float4*>(dq + 16 * dt + 4 * g) =
        make_float4(acc[dt][0] * a.scale, acc[dt][1] * a.scale, acc[dt][2] * a.scale, acc[dt][3] * a.scale);
}

// One workgroup per (slot, sequence): queries [s C, s C + C) in order; wave w
// owns channels [128 w, 128 w + 128). A query's row sources go to LDS first;
// then each 32-row tile's gradients, P^T dO + (scale dl)^T Q summed over the
// heads (MFMA, K = heads, one accumulation chain), are added into the slot's
// buffer rows (entry or window row). With 64 heads the query's dO and Q
// operands stay in registers across its tiles. A query's rows are distinct,
// so its tiles never touch one row twice; consecutive queries are ordered by
// a barrier (the workgroup's waves share one CU and its cache, so plain loads
// and stores suffice).
template <int KSH>
__device__ __forceinline__ void bwd_kv_load_b(const uint16_t* dTq, const uint16_t* qTq, int H, int cb, int lane,
                                              int ks0, bf16x8 (&bD)[8][KSH], bf16x8 (&bQ)[8][KSH]) {
  const int kk = 8 * (lane >> 4);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int64_t col = cb + 16 * nt + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KSH; ++ks) {
      bD[nt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(dTq + col * H + 32 * (ks0 + ks) + kk));
      bQ[nt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qTq + col * H + 32 * (ks0 + ks) + kk));
    }
  }
}

template <int KSH>
__global__ __launch_bounds__(256) void bwd_kv_kernel(AttendBwdArgs p, BwdPlan bp, uint8_t* ws) {
  constexpr int D = 512;
  constexpr int KR = KSH <= 2 ? KSH : 2;          // head steps held in registers at a time
  const AttendArgs& a = p.a;
  const int s = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = threadIdx.x >> 6;
  const int t0 = s * bp.C;
  const int t1 = t0 + bp.C < a.Tq ? t0 + bp.C : a.Tq;
  const int64_t slot = static_cast<int64_t>(b) * bp.Ps + s;
  float* sE = reinterpret_cast<float*>(ws + bp.off_sE) + slot * a.N_cap * D;
  float* sW = reinterpret_cast<float*>(ws + bp.off_sW) + slot * bp.wrows * D;
  __shared__ int32_t src[kMaxSplitRows];
  const int H = a.H;
  const int cb = 128 * wid;
  const int kk = 8 * (lane >> 4);
  for (int t = t0; t < t1; ++t) {
    const RowSpan rs = row_span(a, b, t);
    const int64_t bt = static_cast<int64_t>(b) * a.Tq + t;
    const uint16_t* Pq = reinterpret_cast<const uint16_t*>(ws + bp.off_P) + bt * bp.nr * H;
    const uint16_t* Lq = reinterpret_cast<const uint16_t*>(ws + bp.off_dL) + bt * bp.nr * H;
    const uint16_t* dTq = reinterpret_cast<const uint16_t*>(ws + bp.off_dT) + bt * D * H;
    const uint16_t* qTq = reinterpret_cast<const uint16_t*>(ws + bp.off_qT) + bt * D * H;
    bf16x8 bD[8][KR], bQ[8][KR];
    if constexpr (KSH == KR) bwd_kv_load_b<KR>(dTq, qTq, H, cb, lane, 0, bD, bQ);
    for (int64_t c0 = 0; c0 < rs.nrows; c0 += kMaxSplitRows) {
      const int nr = static_cast<int>(rs.nrows - c0 < kMaxSplitRows ? rs.nrows - c0 : kMaxSplitRows);
      __syncthreads();                             // the last query's (or chunk's) src[] and row updates done
      for (int v = tid; v < (nr + kTileRows - 1) / kTileRows * kTileRows; v += 256)
        src[v] = v < nr ? encode_row(a, b, t, rs, c0 + v) : -1;
      __syncthreads();
      for (int v0 = 0; v0 < nr; v0 += kTileRows) {
        f32x4 c[2][8];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) c[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // lane l holds rows 16 mt + 4 (l / 16) + i, channel cb + 16 nt + l % 16.
        // A tile's rows are distinct entries (or window rows) of one query, so
        // the slot values of all eight of the lane's rows are loaded before
        // any is written back: one memory round trip per tile, not one per row.
        // When every head step's operands fit in registers, those loads go out
        // first and the slot loads right after them (loads complete in issue
        // order), so both round trips overlap and the MFMAs wait only for the
        // operands.
        float* dst[2][4];
        float old[2][4][8];
        auto slot_ptrs = [&]() {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int32_t e = src[v0 + 16 * mt + 4 * (lane >> 4) + i];
              dst[mt][i] = e == -1 ? nullptr
                           : (e >= 0 ? sE + static_cast<int64_t>(e) * D : sW + static_cast<int64_t>(-2 - e - t0) * D) +
                                 cb + (lane & 15);
            }
        };
        auto slot_loads = [&]() {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int nt = 0; nt < 8; ++nt) old[mt][i][nt] = dst[mt][i] ? dst[mt][i][16 * nt] : 0.f;
        };
        slot_ptrs();
#pragma unroll
        for (int k0 = 0; k0 < KSH; k0 += KR) {
          if constexpr (KSH != KR) bwd_kv_load_b<KR>(dTq, qTq, H, cb, lane, k0, bD, bQ);
          bf16x8 aP[KR][2], aL[KR][2];
#pragma unroll
          for (int ks = 0; ks < KR; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
              const int64_t row = c0 + v0 + 16 * mt + (lane & 15);
              aP[ks][mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Pq + row * H + 32 * (k0 + ks) + kk));
              aL[ks][mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Lq + row * H + 32 * (k0 + ks) + kk));
            }
          if constexpr (KSH == KR) slot_loads();
#pragma unroll
          for (int ks = 0; ks < KR; ++ks)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
              for (int mt = 0; mt < 2; ++mt) {
                c[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aP[ks][mt], bD[nt][ks], c[mt][nt], 0, 0, 0);
                c[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aL[ks][mt], bQ[nt][ks], c[mt][nt], 0, 0, 0);
              }
        }
        if constexpr (KSH != KR) slot_loads();
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (dst[mt][i]) {
#pragma unroll
              for (int nt = 0; nt < 8; ++nt) dst[mt][i][16 * nt] = old[mt][i][nt] + c[mt][nt][i];
            }
      }
    }
  }
}

// Entries slot s can touch: those visible to its last query (a causal bound;
// a slot's other rows stay zero).
__host__ __device__ __forceinline__ int64_t bwd_slot_entries(const AttendArgs& a, const BwdPlan& bp, int s) {
  const int t_last = (s + 1) * bp.C < a.Tq ? (s + 1) * bp.C - 1 : a.Tq - 1;
  const int64_t nv = n_visible(a.q_pos0 + t_last, a.m);
  return nv < a.N_cap ? nv : a.N_cap;
}

// Sum over the slots in slot order: one workgroup per block of 8 rows (entry
// rows, then window rows) of a sequence, 16 channels per thread (16 KB of
// each slot read as one block). Slots that cannot touch a row are skipped
// (their rows hold zeros).
constexpr int kRedRows = 8;

__global__ __launch_bounds__(256) void bwd_reduce_kernel(AttendBwdArgs p, BwdPlan bp, uint8_t* ws) {
  constexpr int D = 512;
  const AttendArgs& a = p.a;
  const int b = blockIdx.y;
  const int64_t nEb = (a.N_cap + kRedRows - 1) / kRedRows;
  const float* sE = reinterpret_cast<const float*>(ws + bp.off_sE);
  const float* sW = reinterpret_cast<const float*>(ws + bp.off_sW);
  const int e0 = threadIdx.x * 16;                 // element of the 8 x 512 block
  const int rl = e0 / D, c = e0 % D;               // its row in the block and first channel
  float4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](const float* src) {
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const float4*>(src + 4 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j].x += v[j].x;
      acc[j].y += v[j].y;
      acc[j].z += v[j].z;
      acc[j].w += v[j].w;
    }
  };
  if (blockIdx.x < nEb) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kRedRows + rl;
    if (row < a.N_cap) {
      int s = 0;                                     // slots before s cannot see this entry (their bound grows with s)
      while (s < bp.Ps && bwd_slot_entries(a, bp, s) <= row) ++s;
      const float* base = sE + ((static_cast<int64_t>(b) * bp.Ps) * a.N_cap + row) * D + c;
      const int64_t stride = a.N_cap * D;            // one slot to the next
      for (; s + 8 <= bp.Ps; s += 8) {               // eight slots of loads in flight, added in slot order
        float4 v[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) v[u][j] = *reinterpret_cast<const float4*>(base + (s + u) * stride + 4 * j);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[j].x += v[u][j].x;
            acc[j].y += v[u][j].y;
            acc[j].z += v[u][j].z;
            acc[j].w += v[u][j].w;
          }
      }
      for (; s < bp.Ps; ++s) add(base + s * stride);
      float* dst = p.dkv + (static_cast<int64_t>(b) * a.N_cap + row) * D + c;
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<float4*>(dst + 4 * j) = acc[j];
    }
  } else {
    const int r = static_cast<int>((blockIdx.x - nEb) * kRedRows + rl);   // window row r
    if (r < a.W - 1 + a.Tq) {
      const int tlo = r - (a.W - 1) > 0 ? r - (a.W - 1) : 0;            // read by queries r - W + 1 .. r
      const int thi = r < a.Tq - 1 ? r : a.Tq - 1;
      for (int s = tlo / bp.C; s <= thi / bp.C && tlo <= thi; ++s) {
        const int loc = r - s * bp.C;
        if (loc < 0 || loc >= bp.wrows) continue;
        add(sW + ((static_cast<int64_t>(b) * bp.Ps + s) * bp.wrows + loc) * D + c);
      }
      float* dst = p.dwin + (static_cast<int64_t>(b) * (a.W - 1 + a.Tq) + r) * D + c;
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<float4*>(dst + 4 * j) = acc[j];
    }
  }
}

// Zero the rows each slot can touch: its visible entries and its window rows.
__global__ __launch_bounds__(256) void bwd_zero_slots_kernel(AttendBwdArgs p, BwdPlan bp, uint8_t* ws) {
  constexpr int D = 512;
  const AttendArgs& a = p.a;
  const int s = blockIdx.y, b = blockIdx.z;
  const int64_t slot = static_cast<int64_t>(b) * bp.Ps + s;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  float4* e = reinterpret_cast<float4*>(reinterpret_cast<float*>(ws + bp.off_sE) + slot * a.N_cap * D);
  const int64_t ne4 = bwd_slot_entries(a, bp, s) * D / 4;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < ne4; i += static_cast<int64_t>(gridDim.x) * 256) e[i] = z;
  float4* w = reinterpret_cast<float4*>(reinterpret_cast<float*>(ws + bp.off_sW) + slot * bp.wrows * D);
  const int64_t nw4 = static_cast<int64_t>(bp.wrows) * D / 4;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < nw4; i += static_cast<int64_t>(gridDim.x) * 256) w[i] = z;
}

// dsink[h]: one workgroup per head; thread i sums queries i, i + 256, ... in
// order, then the 256 partial sums add in a fixed tree (deterministic).
__global__ __launch_bounds__(256) void bwd_sink_kernel(AttendBwdArgs p, BwdPlan bp, uint8_t* ws) {
  const AttendArgs& a = p.a;
  const float* dsp = reinterpret_cast<const float*>(ws + bp.off_dsp);
  __shared__ float part[256];
  const int h = blockIdx.x;
  float acc = 0.f;
  for (int64_t bt = threadIdx.x; bt < static_cast<int64_t>(a.B) * a.Tq; bt += 256) acc += dsp[bt * a.H + h];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.dsink[h] = part[0];
}

}  // namespace

size_t attend_backward_workspace(const AttendArgs& a) { return make_bwd_plan(a).total + 256; }

hipError_t launch_attend_backward(hipStream_t s, const AttendBwdArgs& p_in, void* ws, size_t) {
  AttendBwdArgs p = p_in;
  p.a.rope_r = rope_ratio(p.a.rope_base, p.a.rope_dims);
  const AttendArgs& a = p.a;
  const BwdPlan bp = make_bwd_plan(a);
  uint8_t* w = static_cast<uint8_t*>(ws);
  {
    LaunchScope scope(s, "attend_bwd_prep");
    scope.launch(bwd_prep_kernel, dim3(a.Tq, a.B), dim3(256), 0, p, bp, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope scope(s, "attend_bwd_query");
    scope.launch(bwd_query_kernel, dim3(a.H / 64, a.Tq, a.B), dim3(kAttThreads), 0, p, bp, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope scope(s, "attend_bwd_kv");
    // the rows each slot can touch start at zero
    scope.launch(bwd_zero_slots_kernel, dim3(8, bp.Ps, a.B), dim3(256), 0, p, bp, w);
    if (a.H == 64) scope.launch(bwd_kv_kernel<2>, dim3(bp.Ps, a.B), dim3(256), 0, p, bp, w);
    else scope.launch(bwd_kv_kernel<4>, dim3(bp.Ps, a.B), dim3(256), 0, p, bp, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope scope(s, "attend_bwd_reduce");
    const int64_t blocks = (a.N_cap + kRedRows - 1) / kRedRows + (a.W - 1 + a.Tq + kRedRows - 1) / kRedRows;
    scope.launch(bwd_reduce_kernel, dim3(static_cast<uint32_t>(blocks), a.B), dim3(256), 0, p, bp, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope scope(s, "attend_bwd_sink");
    scope.launch(bwd_sink_kernel, dim3(a.H), dim3(256), 0, p, bp, w);
    return hipGetLastError();
  }
}

}  // namespace lca
