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
// LDS, both row-major (for S^T = X Q^T, rows as MFMA M) and transposed (for
// O^T = X^T P^T, rows as MFMA K). Each wave owns 16 heads: its 16 x D query
// block stays in registers as the B operand, its 16 x D output block in
// accumulators, and the probabilities produced by the S^T accumulators feed
// the PV MFMA's B operand with no data movement. Online softmax runs per
// head in float32. Each split writes (max, sum, o) partials; the combine
// kernel merges splits in a fixed order, adds the sink once, divides and
// applies the inverse RoPE. Split sizes depend only on per-sequence shapes,
// so results are independent of the batch size.
#include "lca_device.h"
#include "lca_internal.h"
#include "../../include/lca.h"

namespace lca {
namespace {

constexpr int kTileRows = 32;

struct SplitPlan {
  int S, RS, n_hg, HG;
};

struct RowSpan {
  int64_t n_ent, win_lo, nrows;
};

__device__ __forceinline__ RowSpan row_span(const AttendArgs& a, int t) {
  const int64_t p = a.q_pos0 + t;
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
    return pos - (a.q_pos0 - (a.W - 1));
  }
  return -1;
}

// ---------------------------------------------------------------------------
// bf16 / mixed-storage MFMA kernel
// ---------------------------------------------------------------------------
template <int D, bool MIXED>
__global__ __launch_bounds__(256) void attend_mfma_kernel(AttendArgs a, SplitPlan sp,
                                                          float* __restrict__ part_o,
                                                          float* __restrict__ part_ml) {
  constexpr int XS = D + 8;              // row stride of X (bf16 elements)
  constexpr int TS = kTileRows + 8;      // row stride of X^T
  constexpr int KS = D / 32;             // K steps of S^T
  constexpr int DT = D / 16;             // 16-channel output tiles
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kTileRows * XS];
  __shared__ __attribute__((aligned(16))) uint16_t XTs[D * TS];
  __shared__ int64_t src_row[kTileRows];
  __shared__ int src_kind[kTileRows];

  const int nthreads = blockDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  // head group and split: consecutive workgroup ids of the same split land on
  // the same XCD when there are two head groups (ids i and i + 8 share one).
  int split, hg;
  {
    const int i = blockIdx.x;
    if (sp.n_hg == 2) {
      hg = (i >> 3) & 1;
      split = ((i >> 4) << 3) | (i & 7);
    } else {
      hg = i % sp.n_hg;
      split = i / sp.n_hg;
    }
  }
  const int t = blockIdx.y, b = blockIdx.z;
  const int head = hg * sp.HG + wid * 16 + r16;
  const RowSpan rs = row_span(a, t);
  const int64_t r_begin = static_cast<int64_t>(split) * sp.RS;
  int64_t r_end = r_begin + sp.RS;
  if (r_end > rs.nrows) r_end = rs.nrows;
  const int64_t part_idx = ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * sp.S + split;
  if (split >= sp.S) return;

  // Q fragments (B operand of S^T): head, channels 32s + 8g .. +7
  bf16x8 qf[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((static_cast<int64_t>(b) * a.Tq + t) * a.H + head) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * g));
  }
  f32x4 acc_o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, z_run = 0.f;
  const float scale = a.scale;

  for (int64_t t0 = r_begin; t0 < r_end; t0 += kTileRows) {
    if (tid < kTileRows) {
      int kind;
      const int64_t v = t0 + tid;
      src_row[tid] = v < r_end ? row_source(a, b, t, rs, v, &kind) : -1;
      src_kind[tid] = v < r_end ? kind : 0;
    }
    __syncthreads();
    // stage 32 rows: chunks of 8 channels
    for (int c = tid; c < kTileRows * (D / 8); c += nthreads) {
      const int r = c / (D / 8), d0 = (c % (D / 8)) * 8;
      const int64_t sr = src_row[r];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (sr >= 0) {
        const int kind = src_kind[r];
        if constexpr (!MIXED) {
          const uint16_t* base = kind == 0 ? static_cast<const uint16_t*>(a.kv) + (static_cast<int64_t>(b) * a.N_cap + sr) * D
                                           : static_cast<const uint16_t*>(a.win) + (static_cast<int64_t>(b) * (a.W - 1 + a.Tq) + sr) * D;
          v = *reinterpret_cast<const uint4*>(base + d0);
        } else {
          constexpr int R = 64, NQ = D - R, RB = NQ + 2 * R;
          const int64_t ridx = kind == 0 ? static_cast<int64_t>(b) * a.N_cap + sr
                                         : static_cast<int64_t>(b) * (a.W - 1 + a.Tq) + sr;
          const uint8_t* base = static_cast<const uint8_t*>(kind == 0 ? a.kv : a.win) + ridx * RB;
          if (d0 < NQ) {
            const float s = (kind == 0 ? a.kv_scale : a.win_scale)[ridx];
            const uint2 raw = *reinterpret_cast<const uint2*>(base + d0);
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t word = q < 2 ? raw.x : raw.y;
              const uint32_t b0 = (word >> (16 * (q & 1))) & 0xffu;
              const uint32_t b1 = (word >> (16 * (q & 1) + 8)) & 0xffu;
              w[q] = pack_bf16x2(e4m3fn_to_f32(b0) * s, e4m3fn_to_f32(b1) * s);
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
          } else {
            v = *reinterpret_cast<const uint4*>(base + NQ + 2 * (d0 - NQ));
          }
        }
      }
      *reinterpret_cast<uint4*>(&Xs[r * XS + d0]) = v;
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) XTs[(d0 + i) * TS + r] = static_cast<uint16_t>(wv[i >> 1] >> (16 * (i & 1)));
    }
    __syncthreads();

    // S^T (32 rows x 16 heads) in two 16-row halves
    f32x4 sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* xr = &Xs[(h2 * 16 + r16) * XS + 8 * g];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xr + 32 * s)), qf[s], acc, 0, 0, 0);
      sacc[h2] = acc;
    }
    // lane holds head r16, rows h2*16 + 4g + i
    float lg[8];
    float mx = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = h2 * 16 + 4 * g + i;
        const float l = src_row[r] >= 0 ? sacc[h2][i] * scale : -INFINITY;
        lg[h2 * 4 + i] = l;
        mx = fmaxf(mx, l);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    float alpha, psum = 0.f;
    float p[8];
    if (m_new == -INFINITY) {
      alpha = 1.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = 0.f;
    } else {
      alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = lg[i] == -INFINITY ? 0.f : __expf(lg[i] - m_new);
        psum += p[i];
      }
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    z_run = z_run * alpha + psum;
    m_run = m_new;
    uint4 pw;
    pw.x = pack_bf16x2(p[0], p[1]);
    pw.y = pack_bf16x2(p[2], p[3]);
    pw.z = pack_bf16x2(p[4], p[5]);
    pw.w = pack_bf16x2(p[6], p[7]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    // O^T += X^T P^T: A rows = channels 16dt + r16, K = rows {4g..4g+3, 16+4g..16+4g+3}
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* xt = &XTs[(16 * dt + r16) * TS + 4 * g];
      const uint2 lo = *reinterpret_cast<const uint2*>(xt);
      const uint2 hi = *reinterpret_cast<const uint2*>(xt + 16);
      const bf16x8 af = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      f32x4 o = acc_o[dt];
      o[0] *= alpha; o[1] *= alpha; o[2] *= alpha; o[3] *= alpha;
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf, o, 0, 0, 0);
    }
    __syncthreads();
  }

  // partials: o[head][16dt + 4g + i]
  float* po = part_o + part_idx * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) = make_float4(acc_o[dt][0], acc_o[dt][1], acc_o[dt][2], acc_o[dt][3]);
  if (g == 0) {
    part_ml[2 * part_idx] = m_run;
    part_ml[2 * part_idx + 1] = z_run;
  }
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
  const RowSpan rs = row_span(a, t);
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
// combine: merge split partials, add the sink, normalise, inverse RoPE
// ---------------------------------------------------------------------------
constexpr int kCombThreads = 128;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(AttendArgs a, int S,
                                                               const float* __restrict__ part_o,
                                                               const float* __restrict__ part_ml) {
  __shared__ float wsplit[256];
  __shared__ float sh_inv;
  __shared__ float rope_cs[2 * 256];
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int D = a.D;
  const int64_t row = (static_cast<int64_t>(b) * a.Tq + t) * a.H + h;
  const float* ml = part_ml + row * S * 2;
  const float sink = a.sink[h];
  if (tid == 0) {
    float M = sink;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
    float Z = expf(sink - M);
    for (int s = 0; s < S; ++s) {
      const float ms = ml[2 * s];
      const float w = ms == -INFINITY ? 0.f : expf(ms - M);
      wsplit[s] = w;
      Z += ml[2 * s + 1] * w;
    }
    sh_inv = 1.0f / Z;
    if (a.lse_out) a.lse_out[row] = M + logf(Z);
  }
  const bool rot = (a.flags & LCA_INV_ROPE) && a.rope_dims > 0;
  if (rot) {
    const double pos = -static_cast<double>(a.q_pos0 + t);
    for (int i = tid; i < a.rope_dims / 2; i += kCombThreads) {
      float sn, cs;
      rope_sincos(pos, i, a.rope_dims, static_cast<double>(a.rope_base), &sn, &cs);
      rope_cs[2 * i] = cs;
      rope_cs[2 * i + 1] = sn;
    }
  }
  __syncthreads();
  const float inv = sh_inv;
  const float* po = part_o + row * S * D;
  const int R = rot ? a.rope_dims : 0;
  // each thread owns channel pairs (2c, 2c+1)
  for (int c = tid; c < D / 2; c += kCombThreads) {
    float u = 0.f, v = 0.f;
    for (int s = 0; s < S; ++s) {
      const float w = wsplit[s];
      u = fmaf(w, po[s * D + 2 * c], u);
      v = fmaf(w, po[s * D + 2 * c + 1], v);
    }
    u *= inv;
    v *= inv;
    const int d0 = 2 * c;
    if (d0 >= D - R) {
      const int i = (d0 - (D - R)) / 2;
      const float cs = rope_cs[2 * i], sn = rope_cs[2 * i + 1];
      const float nu = u * cs - v * sn, nv = u * sn + v * cs;
      u = nu;
      v = nv;
    }
    if (a.dt_q == LCA_F32) {
      float* o = static_cast<float*>(a.out) + row * D;
      o[d0] = u;
      o[d0 + 1] = v;
    } else {
      uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + row * D);
      o[c] = pack_bf16x2(u, v);
    }
  }
}

SplitPlan make_plan(const AttendArgs& a) {
  SplitPlan sp;
  const bool f32 = a.dt_kv == LCA_F32;
  if (f32) {
    int hg = 4096 / a.D;
    if (hg > a.H) hg = a.H;
    sp.HG = hg;
    sp.n_hg = (a.H + hg - 1) / hg;
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
  const int64_t min_rows = nrows > 4096 ? 256 : 64;
  int64_t S = (1024 + static_cast<int64_t>(a.Tq) * sp.n_hg - 1) / (static_cast<int64_t>(a.Tq) * sp.n_hg);
  int64_t smax = (nrows + min_rows - 1) / min_rows;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  int64_t RS = (nrows + S - 1) / S;
  RS = (RS + kTileRows - 1) / kTileRows * kTileRows;
  S = (nrows + RS - 1) / RS;
  if (S < 1) S = 1;
  if (S > 256) {                      // combine keeps split weights in LDS
    S = 256;
    RS = ((nrows + S - 1) / S + kTileRows - 1) / kTileRows * kTileRows;
  }
  sp.S = static_cast<int>(S);
  sp.RS = static_cast<int>(RS);
  return sp;
}

template <int D>
void launch_mfma_d(hipStream_t s, const AttendArgs& a, const SplitPlan& sp, float* po, float* pml) {
  int nblk = sp.S * sp.n_hg;
  if (sp.n_hg == 2) nblk = ((sp.S + 7) / 8) * 16;     // XCD-paired id layout
  dim3 grid(nblk, a.Tq, a.B), block(64 * (sp.HG / 16));
  if (a.dt_kv == LCA_KV_MIXED)
    hipLaunchKernelGGL((attend_mfma_kernel<D, true>), grid, block, 0, s, a, sp, po, pml);
  else
    hipLaunchKernelGGL((attend_mfma_kernel<D, false>), grid, block, 0, s, a, sp, po, pml);
}

}  // namespace

size_t attend_workspace(const AttendArgs& a) {
  const SplitPlan sp = make_plan(a);
  const size_t rows = static_cast<size_t>(a.B) * a.Tq * a.H * sp.S;
  return rows * (a.D + 2) * sizeof(float) + 256;
}

hipError_t launch_attend(hipStream_t s, const AttendArgs& a, void* ws, size_t) {
  const SplitPlan sp = make_plan(a);
  const size_t rows = static_cast<size_t>(a.B) * a.Tq * a.H * sp.S;
  float* po = static_cast<float*>(ws);
  float* pml = po + rows * a.D;
  {
    LaunchScope scope(s, a.sparse ? "csa_attend" : "hca_attend");
    if (a.dt_kv == LCA_F32) {
      const size_t smem = (static_cast<size_t>(kTileRows) * a.D + static_cast<size_t>(sp.HG) * a.D +
                           kTileRows * sp.HG + 3 * sp.HG) * sizeof(float);
      hipLaunchKernelGGL(attend_f32_kernel, dim3(sp.S * sp.n_hg, a.Tq, a.B), dim3(kF32Threads), smem, s,
                         a, sp, po, pml);
    } else {
      switch (a.D) {
        case 64: launch_mfma_d<64>(s, a, sp, po, pml); break;
        case 128: launch_mfma_d<128>(s, a, sp, po, pml); break;
        case 256: launch_mfma_d<256>(s, a, sp, po, pml); break;
        default: launch_mfma_d<512>(s, a, sp, po, pml); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope scope(s, "attend_combine");
    hipLaunchKernelGGL(combine_kernel, dim3(a.H, a.Tq, a.B), dim3(kCombThreads), 0, s, a, sp.S, po, pml);
    return hipGetLastError();
  }
}

}  // namespace lca
