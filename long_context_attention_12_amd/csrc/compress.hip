// compress.hip — token compressor (CSA m = 4 with overlapping blocks over two
// KV streams; HCA m' = 128 over one stream) and quantise-on-write of rows.
//
// [kwkr] §3.1: two independent KV sequences merge with softmax-normalised gate
// weights and adjacent blocks overlap; [Qiaomu] 混合注意力机制: entries are
// normalised and carry partial RoPE; [cdjax] §1.1: RoPE channels in BF16, the
// rest in FP8; [kwkr] §3.4: FP4 indexer operands.
//
// The compressor is O(T*D) elementwise work: one workgroup per output entry,
// channels spread over the 256 threads (coalesced row reads), the entry kept
// in LDS for the row-wise epilogue (RMSNorm, RoPE, quantisation).
#include "lca_device.h"
#include "lca_internal.h"
#include "../../include/lca.h"

namespace lca {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxD = 1024;

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

template <typename T> __device__ __forceinline__ float load_elem(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<float>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load_elem<uint16_t>(const void* p, int64_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Write the LDS row e[0..D) in the output format. All threads participate.
__device__ void emit_row(const float* e, int D, int dt_out, int rope_dims, void* out,
                         int64_t row, void* out_scale, float* red, int* blk_exp) {
  const int tid = threadIdx.x;
  if (dt_out == LCA_F32) {
    float* o = static_cast<float*>(out) + row * D;
    for (int c = tid; c < D; c += kThreads) o[c] = e[c];
  } else if (dt_out == LCA_BF16) {
    uint16_t* o = static_cast<uint16_t*>(out) + row * D;
    for (int c = tid; c < D; c += kThreads) o[c] = f32_to_bf16(e[c]);
  } else if (dt_out == LCA_KV_MIXED) {
    const int nq = D - rope_dims;
    const int64_t row_bytes = nq + 2 * rope_dims;
    uint8_t* o = static_cast<uint8_t*>(out) + row * row_bytes;
    float amax = 0.f;
    for (int c = tid; c < nq; c += kThreads) amax = fmaxf(amax, fabsf(e[c]));
    amax = block_reduce(amax, red, true);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;     // IEEE float32 division
    for (int c = tid; c < nq; c += kThreads) o[c] = f32_to_e4m3fn(e[c] / s);
    uint16_t* tail = reinterpret_cast<uint16_t*>(o + nq);
    for (int c = tid; c < rope_dims; c += kThreads) tail[c] = f32_to_bf16(e[nq + c]);
    if (tid == 0) static_cast<float*>(out_scale)[row] = s;
  } else {  // LCA_MXFP4
    const int nb = D / 32;
    if (tid < nb) {
      float amax = 0.f;
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(e[tid * 32 + i]));
      int code = 0, E = 0;
      if (amax > 0.f) { E = mx_scale_exp(amax); code = E + 127; }
      blk_exp[tid] = amax > 0.f ? E : 1000;                 // 1000: all-zero block
      static_cast<uint8_t*>(out_scale)[row * nb + tid] = static_cast<uint8_t>(code);
    }
    __syncthreads();
    uint8_t* o = static_cast<uint8_t*>(out) + row * (D / 2);
    for (int p = tid; p < D / 2; p += kThreads) {
      const int E = blk_exp[(2 * p) / 32];
      uint32_t lo = 0, hi = 0;
      if (E != 1000) {
        lo = f32_to_e2m1(ldexpf(e[2 * p], -E));
        hi = f32_to_e2m1(ldexpf(e[2 * p + 1], -E));
      }
      o[p] = static_cast<uint8_t>(lo | (hi << 4));
    }
  }
}

// One entry from its nl rows: a softmax over the rows' gate logits, the
// weighted sum of the rows per channel (rows taken in order), then the
// epilogue (RMSNorm; RoPE at entry_pos; conversion to dt_out) into row
// out_row of a.out. logit(i) and row(i) give the gate logit and the row of the
// entry's i-th row. The one-shot and the token-at-a-time compressors both go
// through here, so an entry has the same bits whichever of them made it.
template <typename Tin, typename LogitF, typename RowF>
__device__ void merge_and_emit(const CompressArgs& a, int nl, LogitF logit, RowF row, int64_t entry_pos,
                               int64_t out_row, float* wts, float* e, float* red, int* blk_exp) {
  const int tid = threadIdx.x, D = a.D;
  float lmax = -INFINITY;
  for (int i = tid; i < nl; i += kThreads) {
    const float z = logit(i);
    wts[i] = z;
    lmax = fmaxf(lmax, z);
  }
  lmax = block_reduce(lmax, red, true);
  float lsum = 0.f;
  for (int i = tid; i < nl; i += kThreads) {
    const float w = expf(wts[i] - lmax);
    wts[i] = w;
    lsum += w;
  }
  lsum = block_reduce(lsum, red, false);      // also orders the wts[] writes
  const float inv = 1.0f / lsum;

  // rows are summed in order; their loads go out 8 at a time ahead of the
  // sums, so one memory latency covers 8 rows instead of one
  for (int c = tid; c < D; c += kThreads) {
    float acc = 0.f;
    int i = 0;
    for (; i + 8 <= nl; i += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = load_elem<Tin>(row(i + u), c);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(wts[i + u], x[u], acc);
    }
    for (; i < nl; ++i) acc = fmaf(wts[i], load_elem<Tin>(row(i), c), acc);
    e[c] = acc * inv;
  }
  __syncthreads();

  if (a.flags & LCA_NORM) {
    float ss = 0.f;
    for (int c = tid; c < D; c += kThreads) ss += e[c] * e[c];
    ss = block_reduce(ss, red, false);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(D) + a.eps);
    for (int c = tid; c < D; c += kThreads) e[c] = e[c] * r * a.norm_w[c];
    __syncthreads();
  }
  if (a.flags & LCA_ROPE) {
    const int R = a.rope_dims;
    for (int i = tid; i < R / 2; i += kThreads) {
      float s, cs;
      rope_sincos(static_cast<double>(entry_pos), i, a.rope_r, &s, &cs);
      const int c0 = D - R + 2 * i;
      const float u = e[c0], v = e[c0 + 1];
      e[c0] = u * cs - v * s;
      e[c0 + 1] = u * s + v * cs;
    }
    __syncthreads();
  }
  emit_row(e, D, a.dt_out, a.rope_dims, a.out, out_row, a.out_scale, red, blk_exp);
}

template <typename Tin>
__device__ __forceinline__ const Tin* row_ptr(const void* base, int64_t row, int D) {
  return static_cast<const Tin*>(base) + row * D;
}

// One workgroup per output entry j of sequence b (a whole chunk of T tokens).
template <typename Tin>
__global__ __launch_bounds__(kThreads) void compress_kernel(CompressArgs a) {
  __shared__ float wts[256];
  __shared__ float e[kMaxD];
  __shared__ float red[kThreads / 64];
  __shared__ int blk_exp[kMaxD / 32];
  const int j = blockIdx.x, b = blockIdx.y;
  const int m = a.m, D = a.D, T = a.T;
  const bool has_a = a.overlap && (j > 0 || a.prev_ca != nullptr);
  const int na = has_a ? m : 0, nl = na + m;
  const int64_t tok_a = static_cast<int64_t>(b) * T + static_cast<int64_t>(j - 1) * m;   // block j-1
  const int64_t tok_b = static_cast<int64_t>(b) * T + static_cast<int64_t>(j) * m;       // block j
  // rows entering entry j: stream a block j-1 (or prev_*), then stream b block j
  auto logit = [&](int i) -> float {
    if (i < na) return j > 0 ? a.za[tok_a + i] : a.prev_za[b * m + i];
    return a.zb[tok_b + (i - na)];
  };
  auto row = [&](int i) -> const Tin* {
    if (i < na) return j > 0 ? row_ptr<Tin>(a.ca, tok_a + i, D) : row_ptr<Tin>(a.prev_ca, static_cast<int64_t>(b) * m + i, D);
    return row_ptr<Tin>(a.cb, tok_b + (i - na), D);
  };
  merge_and_emit<Tin>(a, nl, logit, row, a.pos0 + static_cast<int64_t>(j) * m,
                      static_cast<int64_t>(b) * a.out_rows + j, wts, e, red, blk_exp);
}

// Token-at-a-time compressor: sequence b appends the token at position p.
// The caller-owned state keeps what a later entry still needs: stream a's
// rows of the last two blocks (a ring of 2m rows; block n in half n mod 2) and
// stream b's rows of the current block (m rows), each with its gate logit.
// When the token closes its block j, entry j is merged and written to out row
// b * out_rows + j. The token's own rows are read from the inputs, never back
// from the state, so no workgroup reads what it wrote.
template <typename Tin>
__device__ void compress_append(const CompressArgs& a, void* state, int b, int64_t p, float* wts, float* e,
                                float* red, int* blk_exp) {
  const int tid = threadIdx.x;
  const int m = a.m, D = a.D;
  const int R = a.overlap ? 3 * m : m;                    // state rows per sequence
  const int slot = static_cast<int>(p % m);
  const int64_t j = p / m;
  Tin* st = static_cast<Tin*>(state) + static_cast<int64_t>(b) * R * D;
  float* sz = reinterpret_cast<float*>(static_cast<uint8_t*>(state) + compress_state_logit_offset(a)) +
              static_cast<int64_t>(b) * R;
  const int b0 = a.overlap ? 2 * m : 0;                   // first stream-b row
  const int ra = static_cast<int>(j & 1) * m + slot;      // this token's stream-a row
  const Tin* cb_new = static_cast<const Tin*>(a.cb) + static_cast<int64_t>(b) * D;
  const Tin* ca_new = a.overlap ? static_cast<const Tin*>(a.ca) + static_cast<int64_t>(b) * D : nullptr;
  for (int c = tid; c < D; c += kThreads) {
    st[(b0 + slot) * D + c] = cb_new[c];
    if (a.overlap) st[ra * D + c] = ca_new[c];
  }
  if (tid == 0) {
    sz[b0 + slot] = a.zb[b];
    if (a.overlap) sz[ra] = a.za[b];
  }
  if (slot != m - 1) return;
  // the token closes block j: entry j from stream a of block j-1, stream b of block j
  const int na = (a.overlap && j > 0) ? m : 0, nl = na + m;
  const int ha = static_cast<int>((j - 1) & 1) * m;       // ring half of block j-1
  auto logit = [&](int i) -> float {
    if (i < na) return sz[ha + i];
    return i - na == m - 1 ? a.zb[b] : sz[b0 + (i - na)];
  };
  auto row = [&](int i) -> const Tin* {
    if (i < na) return st + static_cast<int64_t>(ha + i) * D;
    return i - na == m - 1 ? cb_new : st + static_cast<int64_t>(b0 + (i - na)) * D;
  };
  merge_and_emit<Tin>(a, nl, logit, row, j * m, static_cast<int64_t>(b) * a.out_rows + j, wts, e, red,
                      blk_exp);
}

// Sliding-window ring: sequence b stores the raw row of its token at position
// p (a.cb, [B, D]) in ring row p mod a.out_rows of a.out, converted to a.dt_out.
template <typename Tin>
__device__ void window_append(const CompressArgs& a, int b, int64_t p, float* e, float* red, int* blk_exp) {
  const Tin* x = static_cast<const Tin*>(a.cb) + static_cast<int64_t>(b) * a.D;
  for (int c = threadIdx.x; c < a.D; c += kThreads) e[c] = load_elem<Tin>(x, c);
  __syncthreads();
  emit_row(e, a.D, a.dt_out, a.rope_dims, a.out, static_cast<int64_t>(b) * a.out_rows + p % a.out_rows,
           a.out_scale, red, blk_exp);
}

// All append jobs of a decode step in one launch: workgroup (b, i) runs job i
// for sequence b, at position pos[b] (nothing when outside [0, pos_max]).
__global__ __launch_bounds__(kThreads) void decode_append_kernel(AppendJobs jobs, int64_t pos_max,
                                                                 const int64_t* __restrict__ pos) {
  __shared__ float wts[256];
  __shared__ float e[kMaxD];
  __shared__ float red[kThreads / 64];
  __shared__ int blk_exp[kMaxD / 32];
  const int b = blockIdx.x;
  const int64_t p = pos[b];
  if (p < 0 || p > pos_max) return;
  const AppendJob& job = jobs.j[blockIdx.y];
  if (job.window) {
    if (job.a.dt_in == LCA_F32) window_append<float>(job.a, b, p, e, red, blk_exp);
    else window_append<uint16_t>(job.a, b, p, e, red, blk_exp);
  } else {
    if (job.a.dt_in == LCA_F32) compress_append<float>(job.a, job.state, b, p, wts, e, red, blk_exp);
    else compress_append<uint16_t>(job.a, job.state, b, p, wts, e, red, blk_exp);
  }
}

__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(int dt_out, int D, int rope_dims,
                                                                 const float* __restrict__ src,
                                                                 void* out, void* out_scale) {
  __shared__ float e[kMaxD];
  __shared__ float red[kThreads / 64];
  __shared__ int blk_exp[kMaxD / 32];
  const int64_t row = blockIdx.x + static_cast<int64_t>(blockIdx.y) * gridDim.x;
  for (int c = threadIdx.x; c < D; c += kThreads) e[c] = src[row * D + c];
  __syncthreads();
  emit_row(e, D, dt_out, rope_dims, out, row, out_scale, red, blk_exp);
}

// ---------------------------------------------------------------------------
// Backward of the compressor ([kwkr] §4.3: the attention block's backward is
// the training workload). One workgroup per entry j of sequence b, the
// forward's merge recomputed in the same order, then the chain rule: the
// RoPE adjoint turns the entry's gradient back by the same angle; RMSNorm
// y = e r g (r = 1 / sqrt(mean(e^2) + eps)) gives de = g dy r - e (sum g dy e)
// r^3 / D and the gain's gradient dy e r (one row per entry in the
// workspace, summed over entries in a fixed order by the next kernel); the
// gated merge e = sum_i w_i x_i gives dx_i = w_i de and
// dl_i = w_i (x_i . de - e . de). Every stream-a row feeds the next block's
// entry only and every stream-b row its own, so the row gradients are written
// once, without atomics; rows that no entry reads (stream a of the last block,
// a trailing partial block) are written as zeros by the last workgroup.
// ---------------------------------------------------------------------------
struct CompressBwdArgs {
  CompressArgs a;                      // the forward's arguments (out and out_scale unused)
  const float* dout;                   // [B, T/m, D]
  float *dca, *dza, *dcb, *dzb;        // [B, T, D], [B, T]
  float *dprev_ca, *dprev_za;          // [B, m, D], [B, m] (with prev_ca)
  float* dg_rows;                      // [B * T/m, D] workspace (with LCA_NORM)
};

template <typename Tin>
__global__ __launch_bounds__(kThreads) void compress_bwd_kernel(CompressBwdArgs p) {
  const CompressArgs& a = p.a;
  __shared__ float wts[256];
  __shared__ float e[kMaxD];
  __shared__ float de[kMaxD];
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int j = blockIdx.x, b = blockIdx.y;
  const int m = a.m, D = a.D, T = a.T;
  const int n_out = T / m;
  const int64_t tok0 = static_cast<int64_t>(b) * T;
  // rows no entry reads: stream a of the last block and the tokens of a
  // trailing partial block (every token when there is no whole block)
  if (j == (n_out > 0 ? n_out - 1 : 0)) {
    const int64_t za0 = n_out > 0 ? static_cast<int64_t>(n_out - 1) * m : 0;
    const int64_t zb0 = static_cast<int64_t>(n_out) * m;
    if (a.overlap) {
      for (int64_t i = za0 * D + tid; i < static_cast<int64_t>(T) * D; i += kThreads) p.dca[tok0 * D + i] = 0.f;
      for (int64_t t = za0 + tid; t < T; t += kThreads) p.dza[tok0 + t] = 0.f;
    }
    for (int64_t i = zb0 * D + tid; i < static_cast<int64_t>(T) * D; i += kThreads) p.dcb[tok0 * D + i] = 0.f;
    for (int64_t t = zb0 + tid; t < T; t += kThreads) p.dzb[tok0 + t] = 0.f;
    if (n_out == 0) {
      if (a.overlap && a.prev_ca) {
        for (int i = tid; i < m * D; i += kThreads) p.dprev_ca[static_cast<int64_t>(b) * m * D + i] = 0.f;
        for (int i = tid; i < m; i += kThreads) p.dprev_za[static_cast<int64_t>(b) * m + i] = 0.f;
      }
      return;
    }
  }
  const bool has_a = a.overlap && (j > 0 || a.prev_ca != nullptr);
  const int na = has_a ? m : 0, nl = na + m;
  const int64_t tok_a = tok0 + static_cast<int64_t>(j - 1) * m;   // block j-1
  const int64_t tok_b = tok0 + static_cast<int64_t>(j) * m;       // block j
  auto logit = [&](int i) -> float {
    if (i < na) return j > 0 ? a.za[tok_a + i] : a.prev_za[b * m + i];
    return a.zb[tok_b + (i - na)];
  };
  auto row = [&](int i) -> const Tin* {
    if (i < na) return j > 0 ? row_ptr<Tin>(a.ca, tok_a + i, D) : row_ptr<Tin>(a.prev_ca, static_cast<int64_t>(b) * m + i, D);
    return row_ptr<Tin>(a.cb, tok_b + (i - na), D);
  };
  // where row i's gradients go
  auto drow = [&](int i) -> float* {
    if (i < na) return j > 0 ? p.dca + (tok_a + i) * D : p.dprev_ca + (static_cast<int64_t>(b) * m + i) * D;
    return p.dcb + (tok_b + (i - na)) * D;
  };
  auto dlog = [&](int i) -> float* {
    if (i < na) return j > 0 ? p.dza + tok_a + i : p.dprev_za + static_cast<int64_t>(b) * m + i;
    return p.dzb + tok_b + (i - na);
  };

  // the forward's gate weights and merge
  float lmax = -INFINITY;
  for (int i = tid; i < nl; i += kThreads) {
    const float z = logit(i);
    wts[i] = z;
    lmax = fmaxf(lmax, z);
  }
  lmax = block_reduce(lmax, red, true);
  float lsum = 0.f;
  for (int i = tid; i < nl; i += kThreads) {
    const float w = expf(wts[i] - lmax);
    wts[i] = w;
    lsum += w;
  }
  lsum = block_reduce(lsum, red, false);
  const float inv = 1.0f / lsum;
  for (int i = tid; i < nl; i += kThreads) wts[i] *= inv;
  for (int c = tid; c < D; c += kThreads) {
    float acc = 0.f;
    for (int i = 0; i < nl; ++i) acc = fmaf(wts[i], load_elem<Tin>(row(i), c), acc);
    e[c] = acc;
  }
  // the entry's gradient, turned back through the RoPE
  const float* dy = p.dout + (static_cast<int64_t>(b) * n_out + j) * D;
  for (int c = tid; c < D; c += kThreads) de[c] = dy[c];
  __syncthreads();
  if (a.flags & LCA_ROPE) {
    const int R = a.rope_dims;
    for (int i = tid; i < R / 2; i += kThreads) {
      float sn, cs;
      rope_sincos(static_cast<double>(a.pos0 + static_cast<int64_t>(j) * m), i, a.rope_r, &sn, &cs);
      const int c0 = D - R + 2 * i;
      const float u = de[c0], v = de[c0 + 1];
      de[c0] = u * cs + v * sn;
      de[c0 + 1] = v * cs - u * sn;
    }
    __syncthreads();
  }
  if (a.flags & LCA_NORM) {
    float ss = 0.f, sg = 0.f;
    for (int c = tid; c < D; c += kThreads) {
      ss += e[c] * e[c];
      sg += a.norm_w[c] * de[c] * e[c];
    }
    ss = block_reduce(ss, red, false);
    sg = block_reduce(sg, red, false);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(D) + a.eps);
    const float k3 = sg * r * r * r / static_cast<float>(D);
    float* dg = p.dg_rows + (static_cast<int64_t>(b) * n_out + j) * D;
    for (int c = tid; c < D; c += kThreads) {
      dg[c] = de[c] * e[c] * r;
      de[c] = a.norm_w[c] * de[c] * r - e[c] * k3;
    }
    __syncthreads();
  }
  // the gated merge: e . de once, then row i's dot with de (one wave per row)
  float ed = 0.f;
  for (int c = tid; c < D; c += kThreads) ed += e[c] * de[c];
  ed = block_reduce(ed, red, false);
  for (int i = wid; i < nl; i += kThreads / 64) {
    const Tin* x = row(i);
    float* dx = drow(i);
    const float wi = wts[i];
    float dot = 0.f;
    for (int c = lane; c < D; c += 64) {
      dot = fmaf(load_elem<Tin>(x, c), de[c], dot);
      dx[c] = wi * de[c];
    }
    dot = wave_sum(dot);
    if (lane == 0) *dlog(i) = wi * (dot - ed);
  }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

// dnorm_w[c] = the sum over every entry's row of the workspace, in row order.
__global__ __launch_bounds__(kThreads) void compress_bwd_gain_kernel(const float* __restrict__ dg_rows, int64_t rows,
                                                                     int D, float* __restrict__ dnorm_w) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= D) return;
  float acc = 0.f;
  int64_t r = 0;
  for (; r + 8 <= rows; r += 8) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = dg_rows[(r + u) * D + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += x[u];
  }
  for (; r < rows; ++r) acc += dg_rows[r * D + c];
  dnorm_w[c] = acc;
}

}  // namespace

hipError_t launch_compress(hipStream_t s, const CompressArgs& a_in) {
  CompressArgs a = a_in;
  a.rope_r = rope_ratio(a.rope_base, a.rope_dims);
  const int n_out = a.T / a.m;
  if (n_out == 0) return hipSuccess;
  LaunchScope scope(s, "compress");
  dim3 grid(n_out, a.B);
  if (a.dt_in == LCA_F32)
    scope.launch(compress_kernel<float>, grid, dim3(kThreads), 0, a);
  else
    scope.launch(compress_kernel<uint16_t>, grid, dim3(kThreads), 0, a);
  return hipGetLastError();
}

hipError_t launch_append(hipStream_t s, const AppendJobs& jobs_in, int B, int64_t pos_max, const int64_t* pos,
                         const char* name) {
  AppendJobs jobs = jobs_in;
  for (int i = 0; i < jobs.n; ++i) jobs.j[i].a.rope_r = rope_ratio(jobs.j[i].a.rope_base, jobs.j[i].a.rope_dims);
  LaunchScope scope(s, name);
  scope.launch(decode_append_kernel, dim3(B, jobs.n), dim3(kThreads), 0, jobs, pos_max, pos);
  return hipGetLastError();
}

size_t compress_backward_workspace(int B, int T, int D, int m, uint32_t flags) {
  return (flags & LCA_NORM) ? static_cast<size_t>(B) * (T / m) * D * sizeof(float) + 256 : 256;
}

hipError_t launch_compress_backward(hipStream_t s, const CompressArgs& a_in, const float* dout, float* dca,
                                    float* dza, float* dcb, float* dzb, float* dprev_ca, float* dprev_za,
                                    float* dnorm_w, void* ws) {
  CompressBwdArgs p{a_in, dout, dca, dza, dcb, dzb, dprev_ca, dprev_za, static_cast<float*>(ws)};
  p.a.rope_r = rope_ratio(p.a.rope_base, p.a.rope_dims);
  const int n_out = p.a.T / p.a.m;
  {
    LaunchScope scope(s, "compress_bwd");
    const dim3 grid(n_out > 0 ? n_out : 1, p.a.B);
    if (p.a.dt_in == LCA_F32)
      scope.launch(compress_bwd_kernel<float>, grid, dim3(kThreads), 0, p);
    else
      scope.launch(compress_bwd_kernel<uint16_t>, grid, dim3(kThreads), 0, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if ((p.a.flags & LCA_NORM) && dnorm_w) {
    LaunchScope scope(s, "compress_bwd_gain");
    const int64_t rows = static_cast<int64_t>(p.a.B) * n_out;
    if (rows == 0) {
      scope.launch(fill_zero_kernel, dim3((p.a.D + kThreads - 1) / kThreads), dim3(kThreads), 0, dnorm_w,
                   static_cast<int64_t>(p.a.D));
    } else {
      scope.launch(compress_bwd_gain_kernel, dim3((p.a.D + kThreads - 1) / kThreads), dim3(kThreads), 0,
                   static_cast<const float*>(p.dg_rows), rows, p.a.D, dnorm_w);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_quantize_rows(hipStream_t s, int dt_out, int64_t n_rows, int D, int rope_dims,
                                const float* src, void* out, void* out_scale) {
  if (n_rows == 0) return hipSuccess;
  LaunchScope scope(s, "quantize_rows");
  // split the row count over x (<= 65535 * 1024) and y so any count fits
  const int64_t gx = n_rows < 65536 ? n_rows : 65536;
  int64_t off = 0;
  while (off < n_rows) {
    const int64_t left = n_rows - off;
    const int64_t gy = left / gx;
    if (gy > 0) {
      const int64_t gyc = gy < 65535 ? gy : 65535;
      scope.launch(quantize_rows_kernel, dim3(gx, gyc), dim3(kThreads), 0, dt_out, D,
                         rope_dims, src + off * D,
                         dt_out == LCA_KV_MIXED ? static_cast<void*>(static_cast<uint8_t*>(out) + off * (D + rope_dims))
                                                : static_cast<void*>(static_cast<uint8_t*>(out) + off * (D / 2)),
                         dt_out == LCA_KV_MIXED ? static_cast<void*>(static_cast<float*>(out_scale) + off)
                                                : static_cast<void*>(static_cast<uint8_t*>(out_scale) + off * (D / 32)));
      off += gx * gyc;
    } else {
      scope.launch(quantize_rows_kernel, dim3(left, 1), dim3(kThreads), 0, dt_out, D,
                         rope_dims, src + off * D,
                         dt_out == LCA_KV_MIXED ? static_cast<void*>(static_cast<uint8_t*>(out) + off * (D + rope_dims))
                                                : static_cast<void*>(static_cast<uint8_t*>(out) + off * (D / 2)),
                         dt_out == LCA_KV_MIXED ? static_cast<void*>(static_cast<float*>(out_scale) + off)
                                                : static_cast<void*>(static_cast<uint8_t*>(out_scale) + off * (D / 32)));
      off = n_rows;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace lca
