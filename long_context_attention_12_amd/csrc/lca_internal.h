// lca_internal.h — launchers shared between the validated C ABI (lca_api.cpp)
// and the kernel translation units. Arguments reaching these functions have
// already been validated; they only compute grids and enqueue kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace lca {

// Kernel-launch bracket used by the optional timing mode (lca_profile_*).
// Launches one named step's kernels on `stream`. While kernel timing is on
// (lca_profile_enable), the launches go through hipExtLaunchKernel with a
// start event on the first kernel and a stop event on each, so the recorded
// time runs from the first kernel's start to the last kernel's end and holds
// no launch or event overhead.
struct LaunchScope {
  LaunchScope(hipStream_t s, const char* name);
  ~LaunchScope();
  template <typename F, typename... Args>
  void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, Args... args) {
    if (active) {
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, launched ? nullptr : ev_start, ev_stop, 0, args...);
      launched = true;
    } else {
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
    }
  }
  hipStream_t stream;
  const char* name;
  bool active;
  bool launched;
  hipEvent_t ev_start, ev_stop;
};

struct CompressArgs {
  int dt_in, dt_out, B, T, D, m, overlap;
  int64_t pos0;
  const void *ca, *cb, *prev_ca;
  const float *za, *zb, *prev_za;
  uint32_t flags;
  const float* norm_w;
  float eps, rope_base;
  int rope_dims;
  void* out;
  void* out_scale;
  int64_t out_rows;
  double rope_r;             // base^(-2/R), set by the launchers
};
hipError_t launch_compress(hipStream_t s, const CompressArgs& a);
size_t compress_backward_workspace(int B, int T, int D, int m, uint32_t flags);
hipError_t launch_compress_backward(hipStream_t s, const CompressArgs& a, const float* dout, float* dca,
                                    float* dza, float* dcb, float* dzb, float* dprev_ca, float* dprev_za,
                                    float* dnorm_w, void* ws);

// Token-at-a-time compressor state, per sequence: R = 3m rows with overlap (a
// ring of 2m stream-a rows, then m stream-b rows), R = m without; rows in the
// input type, then R fp32 gate logits per sequence from a 256-byte aligned offset.
__host__ __device__ inline size_t compress_state_rows_bytes(int dt_in, int B, int D, int m, int overlap) {
  const size_t esz = dt_in == 0 /* LCA_F32 */ ? 4 : 2;
  const size_t R = static_cast<size_t>(overlap ? 3 * m : m);
  return (static_cast<size_t>(B) * R * D * esz + 255) & ~static_cast<size_t>(255);
}
__host__ __device__ inline size_t compress_state_logit_offset(const CompressArgs& a) {
  return compress_state_rows_bytes(a.dt_in, a.B, a.D, a.m, a.overlap);
}
__host__ __device__ inline size_t compress_state_bytes(int dt_in, int B, int D, int m, int overlap) {
  return compress_state_rows_bytes(dt_in, B, D, m, overlap) + static_cast<size_t>(B) * (overlap ? 3 * m : m) * 4;
}
// One append of a decode step: a compressor (args + state) or, with window
// set, a window-ring store (a.cb = the raw rows, a.out = the ring, a.out_rows
// = ring rows, a.out_scale = its scales).
struct AppendJob {
  CompressArgs a;
  void* state;
  int window;
};
constexpr int kMaxAppendJobs = 4;
struct AppendJobs {
  AppendJob j[kMaxAppendJobs];
  int n;
};
hipError_t launch_append(hipStream_t s, const AppendJobs& jobs, int B, int64_t pos_max, const int64_t* pos,
                         const char* name);
hipError_t launch_quantize_rows(hipStream_t s, int dt_out, int64_t n_rows, int D, int rope_dims,
                                const float* src, void* out, void* out_scale);

struct IndexArgs {
  int dt, B, Tq, H_I, d_I, m, k;
  int64_t N_cap, q_pos0;
  const void *qI, *qI_scale, *kI, *kI_scale;
  const float* w;
  uint32_t flags;
  int32_t* idx_out;
  float* score_out;
  const int64_t* q_pos;      // per-sequence positions (ragged batch) or null: all at q_pos0
};
size_t index_topk_workspace(const IndexArgs& a);
hipError_t launch_index_topk(hipStream_t s, const IndexArgs& a, void* ws, size_t ws_bytes);

struct AttendArgs {
  int dt_q, dt_kv, B, Tq, H, D, m, k, W;
  bool sparse;               // true: CSA rows from idx; false: HCA all visible rows
  int64_t N_cap, q_pos0;
  const void *q, *kv, *win;
  const float *kv_scale, *win_scale, *sink;
  const int32_t* idx;
  float scale;
  uint32_t flags;
  float rope_base;
  int rope_dims;
  void* out;
  float* lse_out;
  const int64_t* q_pos;      // per-sequence positions (ragged batch) or null: all at q_pos0
  double rope_r;             // base^(-2/R), set by the launchers
};
size_t attend_workspace(const AttendArgs& a);

// Position of sequence b's first query: q_pos[b] clamped to [0, bound] for a
// ragged batch (the bound, q_pos0, sizes every grid, plan and buffer, so a
// clamped position keeps every access inside them), else the bound itself.
__device__ __forceinline__ int64_t seq_pos(const int64_t* q_pos, int64_t bound, int b) {
  if (!q_pos) return bound;
  const int64_t p = q_pos[b];
  return p < 0 ? 0 : (p > bound ? bound : p);
}
hipError_t launch_attend(hipStream_t s, const AttendArgs& a, void* ws, size_t ws_bytes);

// Backward of the core attention: the forward call's arguments plus what the
// backward reads (forward output and lse, the output's gradient) and writes.
struct AttendBwdArgs {
  AttendArgs a;
  const void* out;       // forward output [B, Tq, H, D]
  const float* lse;      // forward lse [B, Tq, H]
  const void* dout;      // gradient of out [B, Tq, H, D]
  float *dq, *dkv, *dwin, *dsink;
};
size_t attend_backward_workspace(const AttendArgs& a);
hipError_t launch_attend_backward(hipStream_t s, const AttendBwdArgs& p, void* ws, size_t ws_bytes);

struct OutProjArgs {
  int T, n_h, c, g, d_g, d_model;
  const void *o, *w_g, *w_o;
  void *mid, *out;
};
hipError_t launch_grouped_out_proj(hipStream_t s, const OutProjArgs& p);

}  // namespace lca
