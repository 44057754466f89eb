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

template <typename Tin>
__global__ __launch_bounds__(kThreads) void compress_kernel(CompressArgs a) {
  __shared__ float wts[256];
  __shared__ float e[kMaxD];
  __shared__ float red[kThreads / 64];
  __shared__ int blk_exp[kMaxD / 32];
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int m = a.m, D = a.D, T = a.T;
  const bool has_a = a.overlap && (j > 0 || a.prev_ca != nullptr);
  const int na = has_a ? m : 0, nl = na + m;

  // gate logits of the rows entering entry j: stream a block j-1, stream b block j
  float lmax = -INFINITY;
  for (int i = tid; i < nl; i += kThreads) {
    float z;
    if (i < na) z = j > 0 ? a.za[static_cast<int64_t>(b) * T + (j - 1) * m + i] : a.prev_za[b * m + i];
    else z = a.zb[static_cast<int64_t>(b) * T + j * m + (i - na)];
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

  for (int c = tid; c < D; c += kThreads) {
    float acc = 0.f;
    for (int i = 0; i < nl; ++i) {
      float x;
      if (i < na) {
        x = j > 0 ? load_elem<Tin>(a.ca, (static_cast<int64_t>(b) * T + (j - 1) * m + i) * D + c)
                  : load_elem<Tin>(a.prev_ca, (static_cast<int64_t>(b) * m + i) * D + c);
      } else {
        x = load_elem<Tin>(a.cb, (static_cast<int64_t>(b) * T + j * m + (i - na)) * D + c);
      }
      acc = fmaf(wts[i], x, acc);
    }
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
      rope_sincos(static_cast<double>(a.pos0 + static_cast<int64_t>(j) * m), i, R,
                  static_cast<double>(a.rope_base), &s, &cs);
      const int c0 = D - R + 2 * i;
      const float u = e[c0], v = e[c0 + 1];
      e[c0] = u * cs - v * s;
      e[c0 + 1] = u * s + v * cs;
    }
    __syncthreads();
  }
  emit_row(e, D, a.dt_out, a.rope_dims, a.out, static_cast<int64_t>(b) * a.out_rows + j,
           a.out_scale, red, blk_exp);
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

}  // namespace

hipError_t launch_compress(hipStream_t s, const CompressArgs& a) {
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
