// lca_api.cpp — the C ABI: argument validation (all of it before any launch,
// so an error leaves nothing enqueued or written), workspace sizing, dispatch
// to the kernel launchers, error reporting and the optional kernel timing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/lca.h"
#include "lca_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LCA_OK;
  return fail(LCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- kernel timing ---------------------------------------------------------
struct ProfRec {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

}  // namespace

namespace lca {

LaunchScope::LaunchScope(hipStream_t s, const char* n)
    : stream(s), name(n), active(false), launched(false), ev_start(nullptr), ev_stop(nullptr) {
  if (!g_prof_on) return;
  if (hipEventCreate(&ev_start) != hipSuccess) return;
  if (hipEventCreate(&ev_stop) != hipSuccess) { (void)hipEventDestroy(ev_start); return; }
  active = true;
}

LaunchScope::~LaunchScope() {
  if (!active) return;
  if (!launched) {                       // nothing ran: nothing to time
    (void)hipEventDestroy(ev_start);
    (void)hipEventDestroy(ev_stop);
    return;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back(ProfRec{name, ev_start, ev_stop});
}

}  // namespace lca

extern "C" {

const char* lca_status_str(int s) {
  switch (s) {
    case LCA_OK: return "ok";
    case LCA_ERR_ARG: return "invalid argument";
    case LCA_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case LCA_ERR_ALIGN: return "misaligned pointer";
    case LCA_ERR_WORKSPACE: return "workspace missing or too small";
    case LCA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* lca_last_error(void) { return g_err; }

int lca_version(void) { return 1 * 10000 + 0 * 100 + 0; }

int lca_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return LCA_OK;
}

int lca_profile_collect(lca_kernel_stat* out, int max_entries) {
  if (!out && max_entries > 0) return fail(LCA_ERR_ARG, "lca_profile_collect: out is NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<lca_kernel_stat> acc;
  int status = LCA_OK;
  for (auto& r : g_prof) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) status = hip_status(e, "lca_profile_collect");
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    bool found = false;
    for (auto& a : acc) {
      if (std::strncmp(a.name, r.name.c_str(), sizeof(a.name)) == 0) {
        a.launches += 1;
        a.total_ms += ms;
        found = true;
        break;
      }
    }
    if (!found) {
      lca_kernel_stat st;
      std::memset(&st, 0, sizeof(st));
      std::strncpy(st.name, r.name.c_str(), sizeof(st.name) - 1);
      st.launches = 1;
      st.total_ms = ms;
      acc.push_back(st);
    }
  }
  g_prof.clear();
  if (status != LCA_OK) return status;
  int n = 0;
  for (auto& a : acc) {
    if (n >= max_entries) break;
    out[n++] = a;
  }
  return n;
}

// ---------------------------------------------------------------------------
int csa_compress(void* stream, int dt_in, int dt_out, int B, int T, int D, int m, int overlap,
                 int64_t pos0, const void* ca, const float* za, const void* cb, const float* zb,
                 const void* prev_ca, const float* prev_za, uint32_t flags, const float* norm_w,
                 float eps, float rope_base, int rope_dims, void* out, void* out_scale,
                 int64_t out_rows) {
  if (B < 1 || T < 0 || m < 1 || D < 32 || D > 1024 || D % 32 != 0)
    return fail(LCA_ERR_ARG, "csa_compress: need B>=1, T>=0, m>=1, 32<=D<=1024, D%%32==0 (B=%d T=%d m=%d D=%d)", B, T, m, D);
  if (overlap != 0 && overlap != 1) return fail(LCA_ERR_ARG, "csa_compress: overlap must be 0 or 1");
  if (overlap == 1 ? 2 * m > 256 : m > 256) return fail(LCA_ERR_UNSUPPORTED, "csa_compress: too many rows per entry (m=%d)", m);
  if (pos0 < 0 || pos0 % m != 0) return fail(LCA_ERR_ARG, "csa_compress: pos0 must be >= 0 and a multiple of m");
  if (dt_in != LCA_F32 && dt_in != LCA_BF16) return fail(LCA_ERR_UNSUPPORTED, "csa_compress: dt_in must be F32 or BF16");
  if (dt_out < LCA_F32 || dt_out > LCA_MXFP4) return fail(LCA_ERR_UNSUPPORTED, "csa_compress: unknown dt_out %d", dt_out);
  if (flags & ~(LCA_NORM | LCA_ROPE)) return fail(LCA_ERR_ARG, "csa_compress: only LCA_NORM and LCA_ROPE apply");
  if (!cb || !zb || !out) return fail(LCA_ERR_ARG, "csa_compress: cb, zb and out are required");
  if (overlap) {
    if (!ca || !za) return fail(LCA_ERR_ARG, "csa_compress: overlap needs ca and za");
    if ((prev_ca == nullptr) != (prev_za == nullptr)) return fail(LCA_ERR_ARG, "csa_compress: prev_ca and prev_za go together");
  } else if (ca || za || prev_ca || prev_za) {
    return fail(LCA_ERR_ARG, "csa_compress: stream a and prev_* must be NULL without overlap");
  }
  if ((flags & LCA_NORM) && !norm_w) return fail(LCA_ERR_ARG, "csa_compress: LCA_NORM needs norm_w");
  if ((flags & LCA_NORM) && !(eps >= 0.f)) return fail(LCA_ERR_ARG, "csa_compress: eps must be >= 0");
  if (rope_dims < 0 || rope_dims > D || rope_dims % 2 != 0) return fail(LCA_ERR_ARG, "csa_compress: rope_dims must be even and in [0, D]");
  if ((flags & LCA_ROPE) && (rope_dims == 0 || !(rope_base > 0.f))) return fail(LCA_ERR_ARG, "csa_compress: LCA_ROPE needs rope_dims > 0 and rope_base > 0");
  if ((dt_out == LCA_KV_MIXED || dt_out == LCA_MXFP4) && !out_scale) return fail(LCA_ERR_ARG, "csa_compress: out_scale required for quantised output");
  if (!aligned16(ca) || !aligned16(cb) || !aligned16(prev_ca) || !aligned16(out))
    return fail(LCA_ERR_ALIGN, "csa_compress: row buffers must be 16-byte aligned");
  if (!aligned4(za) || !aligned4(zb) || !aligned4(prev_za) || !aligned4(norm_w) || !aligned4(out_scale))
    return fail(LCA_ERR_ALIGN, "csa_compress: float arrays must be 4-byte aligned");
  const int64_t n_out = T / m;
  if (out_rows == 0) out_rows = n_out;
  if (out_rows < n_out) return fail(LCA_ERR_ARG, "csa_compress: out_rows (%lld) < T/m (%lld)", (long long)out_rows, (long long)n_out);
  if (n_out > 2147483647LL) return fail(LCA_ERR_UNSUPPORTED, "csa_compress: too many entries");
  lca::CompressArgs a{dt_in, dt_out, B, T, D, m, overlap, pos0, ca, cb, prev_ca, za, zb, prev_za,
                      flags, norm_w, eps, rope_base, rope_dims, out, out_scale, out_rows};
  return hip_status(lca::launch_compress(static_cast<hipStream_t>(stream), a), "csa_compress");
}

size_t csa_compress_backward_workspace(int B, int T, int D, int m, uint32_t flags) {
  if (B < 1 || T < 0 || m < 1 || D < 1) return 0;
  return lca::compress_backward_workspace(B, T, D, m, flags);
}

int csa_compress_backward(void* stream, int dt_in, int B, int T, int D, int m, int overlap, int64_t pos0,
                          const void* ca, const float* za, const void* cb, const float* zb,
                          const void* prev_ca, const float* prev_za, uint32_t flags, const float* norm_w,
                          float eps, float rope_base, int rope_dims, const float* dout, float* dca, float* dza,
                          float* dcb, float* dzb, float* dprev_ca, float* dprev_za, float* dnorm_w, void* ws,
                          size_t ws_bytes) {
  const char* fn = "csa_compress_backward";
  if (B < 1 || T < 0 || m < 1 || D < 32 || D > 1024 || D % 32 != 0)
    return fail(LCA_ERR_ARG, "%s: need B>=1, T>=0, m>=1, 32<=D<=1024, D%%32==0 (B=%d T=%d m=%d D=%d)", fn, B, T, m, D);
  if (overlap != 0 && overlap != 1) return fail(LCA_ERR_ARG, "%s: overlap must be 0 or 1", fn);
  if (overlap == 1 ? 2 * m > 256 : m > 256) return fail(LCA_ERR_UNSUPPORTED, "%s: too many rows per entry (m=%d)", fn, m);
  if (pos0 < 0 || pos0 % m != 0) return fail(LCA_ERR_ARG, "%s: pos0 must be >= 0 and a multiple of m", fn);
  if (dt_in != LCA_F32 && dt_in != LCA_BF16) return fail(LCA_ERR_UNSUPPORTED, "%s: dt_in must be F32 or BF16", fn);
  if (flags & ~(LCA_NORM | LCA_ROPE)) return fail(LCA_ERR_ARG, "%s: only LCA_NORM and LCA_ROPE apply", fn);
  if (!cb || !zb || !dcb || !dzb || (T / m > 0 && !dout))
    return fail(LCA_ERR_ARG, "%s: cb, zb, dcb, dzb (and dout when T >= m) are required", fn);
  if (overlap) {
    if (!ca || !za || !dca || !dza) return fail(LCA_ERR_ARG, "%s: overlap needs ca, za, dca and dza", fn);
    if ((prev_ca == nullptr) != (prev_za == nullptr)) return fail(LCA_ERR_ARG, "%s: prev_ca and prev_za go together", fn);
    if (prev_ca && (!dprev_ca || !dprev_za)) return fail(LCA_ERR_ARG, "%s: prev_ca needs dprev_ca and dprev_za", fn);
    if (!prev_ca && (dprev_ca || dprev_za)) return fail(LCA_ERR_ARG, "%s: dprev_* without prev_ca", fn);
  } else if (ca || za || prev_ca || prev_za || dca || dza || dprev_ca || dprev_za) {
    return fail(LCA_ERR_ARG, "%s: stream a, prev_* and their gradients must be NULL without overlap", fn);
  }
  if ((flags & LCA_NORM) && (!norm_w || !dnorm_w)) return fail(LCA_ERR_ARG, "%s: LCA_NORM needs norm_w and dnorm_w", fn);
  if (!(flags & LCA_NORM) && dnorm_w) return fail(LCA_ERR_ARG, "%s: dnorm_w without LCA_NORM", fn);
  if ((flags & LCA_NORM) && !(eps >= 0.f)) return fail(LCA_ERR_ARG, "%s: eps must be >= 0", fn);
  if (rope_dims < 0 || rope_dims > D || rope_dims % 2 != 0) return fail(LCA_ERR_ARG, "%s: rope_dims must be even and in [0, D]", fn);
  if ((flags & LCA_ROPE) && (rope_dims == 0 || !(rope_base > 0.f))) return fail(LCA_ERR_ARG, "%s: LCA_ROPE needs rope_dims > 0 and rope_base > 0", fn);
  if (!aligned16(ca) || !aligned16(cb) || !aligned16(prev_ca) || !aligned16(dout) || !aligned16(dca) ||
      !aligned16(dcb) || !aligned16(dprev_ca))
    return fail(LCA_ERR_ALIGN, "%s: row buffers must be 16-byte aligned", fn);
  if (!aligned4(za) || !aligned4(zb) || !aligned4(prev_za) || !aligned4(norm_w) || !aligned4(dza) || !aligned4(dzb) ||
      !aligned4(dprev_za) || !aligned4(dnorm_w))
    return fail(LCA_ERR_ALIGN, "%s: float arrays must be 4-byte aligned", fn);
  if (T / m > 2147483647LL) return fail(LCA_ERR_UNSUPPORTED, "%s: too many entries", fn);
  const size_t need = lca::compress_backward_workspace(B, T, D, m, flags);
  if ((flags & LCA_NORM) && (!ws || ws_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  if (!aligned16(ws)) return fail(LCA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  lca::CompressArgs a{dt_in, LCA_F32, B, T, D, m, overlap, pos0, ca, cb, prev_ca, za, zb, prev_za,
                      flags, norm_w, eps, rope_base, rope_dims, nullptr, nullptr, T / m};
  return hip_status(lca::launch_compress_backward(static_cast<hipStream_t>(stream), a, dout, dca, dza, dcb, dzb,
                                                  dprev_ca, dprev_za, dnorm_w, ws), fn);
}

// ---------------------------------------------------------------------------
// Decode-time state: token-at-a-time compressor and the sliding-window ring.
static int check_positions(const int64_t* pos, int64_t pos_max, const char* fn) {
  if (!pos) return fail(LCA_ERR_ARG, "%s: pos is required", fn);
  if (reinterpret_cast<uintptr_t>(pos) % 8 != 0) return fail(LCA_ERR_ALIGN, "%s: pos must be 8-byte aligned", fn);
  if (pos_max < 0) return fail(LCA_ERR_ARG, "%s: pos_max must be >= 0", fn);
  return LCA_OK;
}

size_t csa_compress_state_bytes(int dt_in, int B, int D, int m, int overlap) {
  if (B < 1 || D < 1 || m < 1 || (dt_in != LCA_F32 && dt_in != LCA_BF16)) return 0;
  return lca::compress_state_bytes(dt_in, B, D, m, overlap ? 1 : 0);
}

// Validates one append job and fills its launch form.
static int check_compress_job(const char* fn, int B, int64_t pos_max, const lca_append_job& j, lca::AppendJob* job) {
  const int D = j.D, m = j.m;
  if (m < 1 || D < 32 || D > 1024 || D % 32 != 0)
    return fail(LCA_ERR_ARG, "%s: need m>=1, 32<=D<=1024, D%%32==0 (m=%d D=%d)", fn, m, D);
  if (j.overlap != 0 && j.overlap != 1) return fail(LCA_ERR_ARG, "%s: overlap must be 0 or 1", fn);
  if (j.overlap == 1 ? 2 * m > 256 : m > 256) return fail(LCA_ERR_UNSUPPORTED, "%s: too many rows per entry (m=%d)", fn, m);
  if (j.dt_in != LCA_F32 && j.dt_in != LCA_BF16) return fail(LCA_ERR_UNSUPPORTED, "%s: dt_in must be F32 or BF16", fn);
  if (j.dt_out < LCA_F32 || j.dt_out > LCA_MXFP4) return fail(LCA_ERR_UNSUPPORTED, "%s: unknown dt_out %d", fn, j.dt_out);
  if (j.flags & ~(LCA_NORM | LCA_ROPE)) return fail(LCA_ERR_ARG, "%s: only LCA_NORM and LCA_ROPE apply", fn);
  if (!j.cb || !j.zb || !j.out || !j.state) return fail(LCA_ERR_ARG, "%s: cb, zb, state and out are required", fn);
  if (j.overlap && (!j.ca || !j.za)) return fail(LCA_ERR_ARG, "%s: overlap needs ca and za", fn);
  if (!j.overlap && (j.ca || j.za)) return fail(LCA_ERR_ARG, "%s: stream a must be NULL without overlap", fn);
  if ((j.flags & LCA_NORM) && !j.norm_w) return fail(LCA_ERR_ARG, "%s: LCA_NORM needs norm_w", fn);
  if ((j.flags & LCA_NORM) && !(j.eps >= 0.f)) return fail(LCA_ERR_ARG, "%s: eps must be >= 0", fn);
  if (j.rope_dims < 0 || j.rope_dims > D || j.rope_dims % 2 != 0) return fail(LCA_ERR_ARG, "%s: rope_dims must be even and in [0, D]", fn);
  if ((j.flags & LCA_ROPE) && (j.rope_dims == 0 || !(j.rope_base > 0.f))) return fail(LCA_ERR_ARG, "%s: LCA_ROPE needs rope_dims > 0 and rope_base > 0", fn);
  if ((j.dt_out == LCA_KV_MIXED || j.dt_out == LCA_MXFP4) && !j.out_scale) return fail(LCA_ERR_ARG, "%s: out_scale required for quantised output", fn);
  if (!aligned16(j.ca) || !aligned16(j.cb) || !aligned16(j.out) || !aligned16(j.state))
    return fail(LCA_ERR_ALIGN, "%s: row buffers and state must be 16-byte aligned", fn);
  if (!aligned4(j.za) || !aligned4(j.zb) || !aligned4(j.norm_w) || !aligned4(j.out_scale))
    return fail(LCA_ERR_ALIGN, "%s: float arrays must be 4-byte aligned", fn);
  const size_t need = lca::compress_state_bytes(j.dt_in, B, D, m, j.overlap);
  if (j.state_bytes < need) return fail(LCA_ERR_WORKSPACE, "%s: state %zu < %zu bytes", fn, j.state_bytes, need);
  if (j.out_rows < (pos_max + 1) / m)
    return fail(LCA_ERR_ARG, "%s: out_rows (%lld) < (pos_max + 1) / m (%lld)", fn, (long long)j.out_rows, (long long)((pos_max + 1) / m));
  job->a = lca::CompressArgs{j.dt_in, j.dt_out, B, 1, D, m, j.overlap, 0, j.ca, j.cb, nullptr, j.za, j.zb, nullptr,
                             j.flags, j.norm_w, j.eps, j.rope_base, j.rope_dims, j.out, j.out_scale, j.out_rows};
  job->state = j.state;
  job->window = 0;
  return LCA_OK;
}

static int check_window_job(const char* fn, int B, const lca_append_job& j, lca::AppendJob* job) {
  const int D = j.D;
  if (j.out_rows < 1 || D < 32 || D > 1024 || D % 32 != 0)
    return fail(LCA_ERR_ARG, "%s: need ring_rows>=1, 32<=D<=1024, D%%32==0", fn);
  if (j.dt_in != LCA_F32 && j.dt_in != LCA_BF16) return fail(LCA_ERR_UNSUPPORTED, "%s: dt_in must be F32 or BF16", fn);
  if (j.dt_out != LCA_F32 && j.dt_out != LCA_BF16 && j.dt_out != LCA_KV_MIXED)
    return fail(LCA_ERR_UNSUPPORTED, "%s: dt_out must be F32, BF16 or KV_MIXED", fn);
  if (j.dt_out == LCA_KV_MIXED && (j.rope_dims < 0 || j.rope_dims > D || j.rope_dims % 2 != 0))
    return fail(LCA_ERR_ARG, "%s: rope_dims must be even and in [0, D]", fn);
  if (!j.cb || !j.out) return fail(LCA_ERR_ARG, "%s: src and win are required", fn);
  if (j.dt_out == LCA_KV_MIXED && !j.out_scale) return fail(LCA_ERR_ARG, "%s: KV_MIXED needs win_scale", fn);
  if (!aligned16(j.cb) || !aligned16(j.out)) return fail(LCA_ERR_ALIGN, "%s: src and win must be 16-byte aligned", fn);
  if (!aligned4(j.out_scale)) return fail(LCA_ERR_ALIGN, "%s: win_scale must be 4-byte aligned", fn);
  job->a = lca::CompressArgs{j.dt_in, j.dt_out, B, 1, D, 1, 0, 0, nullptr, j.cb, nullptr, nullptr, nullptr, nullptr,
                             0u, nullptr, 0.f, 0.f, j.dt_out == LCA_KV_MIXED ? j.rope_dims : 0, j.out, j.out_scale,
                             j.out_rows};
  job->state = nullptr;
  job->window = 1;
  return LCA_OK;
}

int lca_decode_append(void* stream, int B, int64_t pos_max, const int64_t* pos, const lca_append_job* jobs,
                      int n_jobs) {
  const char* fn = "lca_decode_append";
  if (B < 1) return fail(LCA_ERR_ARG, "%s: need B >= 1", fn);
  if (n_jobs < 1 || n_jobs > LCA_MAX_APPEND_JOBS || !jobs)
    return fail(LCA_ERR_ARG, "%s: need 1 to %d jobs", fn, LCA_MAX_APPEND_JOBS);
  int st = check_positions(pos, pos_max, fn);
  if (st != LCA_OK) return st;
  lca::AppendJobs js{};
  js.n = n_jobs;
  for (int i = 0; i < n_jobs; ++i) {
    if (jobs[i].kind == LCA_APPEND_COMPRESS) st = check_compress_job(fn, B, pos_max, jobs[i], &js.j[i]);
    else if (jobs[i].kind == LCA_APPEND_WINDOW) st = check_window_job(fn, B, jobs[i], &js.j[i]);
    else st = fail(LCA_ERR_ARG, "%s: job %d has unknown kind %d", fn, i, jobs[i].kind);
    if (st != LCA_OK) return st;
  }
  return hip_status(lca::launch_append(static_cast<hipStream_t>(stream), js, B, pos_max, pos, "decode_append"), fn);
}

int csa_compress_append(void* stream, int dt_in, int dt_out, int B, int D, int m, int overlap, int64_t pos_max,
                        const int64_t* pos, const void* ca, const float* za, const void* cb, const float* zb,
                        void* state, size_t state_bytes, uint32_t flags, const float* norm_w, float eps,
                        float rope_base, int rope_dims, void* out, void* out_scale, int64_t out_rows) {
  const char* fn = "csa_compress_append";
  if (B < 1) return fail(LCA_ERR_ARG, "%s: need B >= 1", fn);
  int st = check_positions(pos, pos_max, fn);
  if (st != LCA_OK) return st;
  lca_append_job j{};
  j.kind = LCA_APPEND_COMPRESS; j.dt_in = dt_in; j.dt_out = dt_out; j.D = D; j.m = m; j.overlap = overlap;
  j.flags = flags; j.rope_dims = rope_dims; j.eps = eps; j.rope_base = rope_base; j.ca = ca; j.za = za;
  j.cb = cb; j.zb = zb; j.norm_w = norm_w; j.state = state; j.state_bytes = state_bytes; j.out = out;
  j.out_scale = out_scale; j.out_rows = out_rows;
  lca::AppendJobs js{};
  js.n = 1;
  st = check_compress_job(fn, B, pos_max, j, &js.j[0]);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_append(static_cast<hipStream_t>(stream), js, B, pos_max, pos, "compress_append"), fn);
}

int lca_window_append(void* stream, int dt_in, int dt_out, int B, int D, int rope_dims, int ring_rows,
                      int64_t pos_max, const int64_t* pos, const void* src, void* win, float* win_scale) {
  const char* fn = "lca_window_append";
  if (B < 1) return fail(LCA_ERR_ARG, "%s: need B >= 1", fn);
  int st = check_positions(pos, pos_max, fn);
  if (st != LCA_OK) return st;
  lca_append_job j{};
  j.kind = LCA_APPEND_WINDOW; j.dt_in = dt_in; j.dt_out = dt_out; j.D = D; j.rope_dims = rope_dims;
  j.cb = src; j.out = win; j.out_scale = win_scale; j.out_rows = ring_rows;
  lca::AppendJobs js{};
  js.n = 1;
  st = check_window_job(fn, B, j, &js.j[0]);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_append(static_cast<hipStream_t>(stream), js, B, pos_max, pos, "window_append"), fn);
}

int lca_grouped_out_proj(void* stream, int T, int n_h, int c, int g, int d_g, int d_model, const void* o,
                         const void* w_g, const void* w_o, void* mid, void* out) {
  const char* fn = "lca_grouped_out_proj";
  if (T < 1 || n_h < 1 || c < 1 || g < 1 || d_g < 1 || d_model < 1)
    return fail(LCA_ERR_ARG, "%s: need T, n_h, c, g, d_g, d_model >= 1", fn);
  if (n_h % g != 0) return fail(LCA_ERR_ARG, "%s: n_h (%d) must be a multiple of g (%d)", fn, n_h, g);
  const int64_t kg = static_cast<int64_t>(n_h / g) * c, mid_w = static_cast<int64_t>(g) * d_g;
  if (kg % 256 != 0 || mid_w % 256 != 0)
    return fail(LCA_ERR_UNSUPPORTED, "%s: (n_h/g)*c (%lld) and g*d_g (%lld) must be multiples of 256", fn,
                (long long)kg, (long long)mid_w);
  if (d_g % 16 != 0 || d_model % 16 != 0) return fail(LCA_ERR_UNSUPPORTED, "%s: d_g and d_model must be multiples of 16", fn);
  if (kg > (1 << 30) || mid_w > (1 << 30) || d_model > (1 << 30) || g > 65535)
    return fail(LCA_ERR_UNSUPPORTED, "%s: dimensions too large", fn);
  if ((static_cast<int64_t>(T) + 15) / 16 > 65535LL * 4) return fail(LCA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  if (!o || !w_g || !w_o || !mid || !out) return fail(LCA_ERR_ARG, "%s: o, w_g, w_o, mid and out are required", fn);
  if (!aligned16(o) || !aligned16(w_g) || !aligned16(w_o) || !aligned16(mid) || !aligned16(out))
    return fail(LCA_ERR_ALIGN, "%s: buffers must be 16-byte aligned", fn);
  lca::OutProjArgs p{T, n_h, c, g, d_g, d_model, o, w_g, w_o, mid, out};
  return hip_status(lca::launch_grouped_out_proj(static_cast<hipStream_t>(stream), p), fn);
}

int lca_quantize_rows(void* stream, int dt_out, int64_t n_rows, int D, int rope_dims,
                      const float* src, void* out, void* out_scale) {
  if (n_rows < 0 || D < 32 || D > 1024 || D % 32 != 0)
    return fail(LCA_ERR_ARG, "lca_quantize_rows: need n_rows>=0, 32<=D<=1024, D%%32==0");
  if (dt_out != LCA_KV_MIXED && dt_out != LCA_MXFP4) return fail(LCA_ERR_UNSUPPORTED, "lca_quantize_rows: dt_out must be KV_MIXED or MXFP4");
  if (dt_out == LCA_KV_MIXED && (rope_dims < 0 || rope_dims > D || rope_dims % 2))
    return fail(LCA_ERR_ARG, "lca_quantize_rows: rope_dims must be even and in [0, D]");
  if (!src || !out || !out_scale) return fail(LCA_ERR_ARG, "lca_quantize_rows: src, out and out_scale are required");
  if (!aligned16(src) || !aligned16(out) || !aligned4(out_scale)) return fail(LCA_ERR_ALIGN, "lca_quantize_rows: misaligned buffer");
  return hip_status(lca::launch_quantize_rows(static_cast<hipStream_t>(stream), dt_out, n_rows, D,
                                              dt_out == LCA_KV_MIXED ? rope_dims : 0, src, out, out_scale),
                    "lca_quantize_rows");
}

// ---------------------------------------------------------------------------
static int check_index(const lca::IndexArgs& a) {
  if (a.B < 1 || a.Tq < 1 || a.H_I < 1 || a.d_I < 32 || a.N_cap < 0 || a.m < 1 || a.q_pos0 < 0)
    return fail(LCA_ERR_ARG, "csa_index_topk: need B,Tq,H_I>=1, d_I>=32, N_cap>=0, m>=1, q_pos0>=0");
  if (a.k < 1 || a.k > 4096) return fail(LCA_ERR_UNSUPPORTED, "csa_index_topk: k must be in [1, 4096] (k=%d)", a.k);
  if (a.d_I % 32 != 0 || a.d_I > 256) return fail(LCA_ERR_UNSUPPORTED, "csa_index_topk: d_I must be a multiple of 32, <= 256");
  if (a.dt == LCA_F32) {
    if (a.H_I > 64) return fail(LCA_ERR_UNSUPPORTED, "csa_index_topk: F32 supports H_I <= 64");
  } else if (a.dt == LCA_BF16 || a.dt == LCA_MXFP4) {
    const bool pow2 = a.H_I == 1 || a.H_I == 2 || a.H_I == 4 || a.H_I == 8 || a.H_I == 16;
    if (!(pow2 || a.H_I == 32 || a.H_I == 64))
      return fail(LCA_ERR_UNSUPPORTED, "csa_index_topk: H_I must be 1, 2, 4, 8, 16, 32 or 64 (H_I=%d)", a.H_I);
    if (a.dt == LCA_MXFP4) {
      if (a.d_I != 128) return fail(LCA_ERR_UNSUPPORTED, "csa_index_topk: MXFP4 needs d_I == 128");
      if (!a.qI_scale || !a.kI_scale) return fail(LCA_ERR_ARG, "csa_index_topk: MXFP4 needs qI_scale and kI_scale");
    }
  } else {
    return fail(LCA_ERR_UNSUPPORTED, "csa_index_topk: dt must be F32, BF16 or MXFP4");
  }
  if (a.flags & ~LCA_SCORE_BF16) return fail(LCA_ERR_ARG, "csa_index_topk: only LCA_SCORE_BF16 applies");
  const int64_t nv_last = (a.q_pos0 + a.Tq) / a.m;
  if (a.N_cap < nv_last) return fail(LCA_ERR_ARG, "csa_index_topk: N_cap (%lld) < visible entries of the last query (%lld)", (long long)a.N_cap, (long long)nv_last);
  if (a.N_cap > 2147483647LL) return fail(LCA_ERR_UNSUPPORTED, "csa_index_topk: N_cap must fit int32 indices");
  if (!a.qI || !a.w || !a.kI || !a.idx_out) return fail(LCA_ERR_ARG, "csa_index_topk: qI, w, kI and idx_out are required");
  if (!aligned16(a.qI) || !aligned16(a.kI) || !aligned4(a.w) || !aligned4(a.idx_out) || !aligned4(a.score_out) ||
      (a.dt == LCA_MXFP4 && !aligned4(a.kI_scale)))
    return fail(LCA_ERR_ALIGN, "csa_index_topk: misaligned buffer");
  return LCA_OK;
}

size_t csa_index_topk_workspace(int dt, int B, int Tq, int H_I, int d_I, int64_t N_cap, int m, int k,
                                int64_t q_pos0, uint32_t flags) {
  lca::IndexArgs a{dt, B, Tq, H_I, d_I, m, k, N_cap, q_pos0, nullptr, nullptr, nullptr, nullptr, nullptr, flags, nullptr, nullptr};
  if (B < 1 || Tq < 1 || N_cap < 0) return 0;
  return lca::index_topk_workspace(a);
}

int csa_index_topk(void* stream, int dt, int B, int Tq, int H_I, int d_I, int64_t N_cap, int m, int k,
                   int64_t q_pos0, const void* qI, const void* qI_scale, const float* w, const void* kI,
                   const void* kI_scale, uint32_t flags, int32_t* idx_out, float* score_out, void* ws,
                   size_t ws_bytes) {
  lca::IndexArgs a{dt, B, Tq, H_I, d_I, m, k, N_cap, q_pos0, qI, qI_scale, kI, kI_scale, w, flags, idx_out, score_out};
  int st = check_index(a);
  if (st != LCA_OK) return st;
  const size_t need = lca::index_topk_workspace(a);
  if (!ws || ws_bytes < need) return fail(LCA_ERR_WORKSPACE, "csa_index_topk: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(ws)) return fail(LCA_ERR_ALIGN, "csa_index_topk: workspace must be 16-byte aligned");
  return hip_status(lca::launch_index_topk(static_cast<hipStream_t>(stream), a, ws, ws_bytes), "csa_index_topk");
}

// ---------------------------------------------------------------------------
static int check_attend(const lca::AttendArgs& a, const char* fn) {
  if (a.B < 1 || a.Tq < 1 || a.H < 1 || a.N_cap < 0 || a.m < 1 || a.q_pos0 < 0)
    return fail(LCA_ERR_ARG, "%s: need B,Tq,H>=1, N_cap>=0, m>=1, q_pos0>=0", fn);
  if (a.W < 1 || a.W > 4096) return fail(LCA_ERR_ARG, "%s: W must be in [1, 4096]", fn);
  if (a.D < 32 || a.D % 32 != 0 || a.D > 512) return fail(LCA_ERR_UNSUPPORTED, "%s: D must be a multiple of 32 and <= 512", fn);
  if (a.sparse && (a.k < 1 || a.k > 4096)) return fail(LCA_ERR_UNSUPPORTED, "%s: k must be in [1, 4096]", fn);
  if (a.dt_kv == LCA_F32) {
    if (a.dt_q != LCA_F32) return fail(LCA_ERR_UNSUPPORTED, "%s: F32 kv needs F32 q", fn);
    if (a.D > 256) return fail(LCA_ERR_UNSUPPORTED, "%s: F32 path supports D <= 256", fn);
  } else if (a.dt_kv == LCA_BF16 || a.dt_kv == LCA_KV_MIXED) {
    if (a.dt_q != LCA_BF16) return fail(LCA_ERR_UNSUPPORTED, "%s: BF16/MIXED kv needs BF16 q", fn);
    if (!(a.D == 64 || a.D == 128 || a.D == 256 || a.D == 512)) return fail(LCA_ERR_UNSUPPORTED, "%s: MFMA path needs D in {64,128,256,512}", fn);
    if (a.H % 16 != 0 || (a.H > 64 && a.H % 64 != 0)) return fail(LCA_ERR_UNSUPPORTED, "%s: H must be 16, 32, 48, 64 or a multiple of 64", fn);
    if (a.H / 64 > 2 && a.H > 128) return fail(LCA_ERR_UNSUPPORTED, "%s: H <= 128", fn);
    if (a.dt_kv == LCA_KV_MIXED && (a.D != 512 || a.rope_dims != 64))
      return fail(LCA_ERR_UNSUPPORTED, "%s: KV_MIXED rows need D == 512 and rope_dims == 64", fn);
    if (a.dt_kv == LCA_KV_MIXED && (!a.kv_scale || !a.win_scale)) return fail(LCA_ERR_ARG, "%s: KV_MIXED needs kv_scale and win_scale", fn);
  } else {
    return fail(LCA_ERR_UNSUPPORTED, "%s: dt_kv must be F32, BF16 or KV_MIXED", fn);
  }
  if (a.flags & ~(LCA_INV_ROPE | LCA_WIN_RING | LCA_SPLITS_ONE_WG | LCA_SPLITS_MANY_WG))
    return fail(LCA_ERR_ARG, "%s: only LCA_INV_ROPE, LCA_WIN_RING and LCA_SPLITS_* apply", fn);
  if ((a.flags & LCA_SPLITS_ONE_WG) && (a.flags & LCA_SPLITS_MANY_WG))
    return fail(LCA_ERR_ARG, "%s: LCA_SPLITS_ONE_WG and LCA_SPLITS_MANY_WG exclude each other", fn);
  if (a.rope_dims < 0 || a.rope_dims > a.D || a.rope_dims % 2) return fail(LCA_ERR_ARG, "%s: rope_dims must be even and in [0, D]", fn);
  if ((a.flags & LCA_INV_ROPE) && (a.rope_dims == 0 || !(a.rope_base > 0.f))) return fail(LCA_ERR_ARG, "%s: LCA_INV_ROPE needs rope_dims > 0 and rope_base > 0", fn);
  if (!(a.scale == a.scale)) return fail(LCA_ERR_ARG, "%s: scale is NaN", fn);
  if (!a.q || !a.kv || !a.win || !a.sink || !a.out || (a.sparse && !a.idx)) return fail(LCA_ERR_ARG, "%s: missing required pointer", fn);
  if (!a.sparse) {
    const int64_t nv_last = (a.q_pos0 + a.Tq) / a.m;
    if (a.N_cap < nv_last) return fail(LCA_ERR_ARG, "%s: N_cap (%lld) < visible entries of the last query (%lld)", fn, (long long)a.N_cap, (long long)nv_last);
    // a query's rows are cut into at most 256 splits of at most 2048 rows
    if (nv_last + a.W > 256LL * 2048)
      return fail(LCA_ERR_UNSUPPORTED, "%s: %lld visible entries + W exceed the 524288 rows one query can attend", fn,
                  (long long)nv_last);
  }
  if (!aligned16(a.q) || !aligned16(a.kv) || !aligned16(a.win) || !aligned16(a.out) || !aligned4(a.idx) ||
      !aligned4(a.sink) || !aligned4(a.lse_out) || !aligned4(a.kv_scale) || !aligned4(a.win_scale))
    return fail(LCA_ERR_ALIGN, "%s: misaligned buffer", fn);
  return LCA_OK;
}

static int run_attend(void* stream, const lca::AttendArgs& a, void* ws, size_t ws_bytes, const char* fn) {
  int st = check_attend(a, fn);
  if (st != LCA_OK) return st;
  const size_t need = lca::attend_workspace(a);
  if (!ws || ws_bytes < need) return fail(LCA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (!aligned16(ws)) return fail(LCA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return hip_status(lca::launch_attend(static_cast<hipStream_t>(stream), a, ws, ws_bytes), fn);
}

size_t csa_attend_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int k,
                            int W, int64_t q_pos0) {
  if (B < 1 || Tq < 1 || H < 1 || D < 1 || m < 1 || W < 1) return 0;
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = k; a.W = W;
  a.sparse = true; a.N_cap = N_cap; a.q_pos0 = q_pos0;
  return lca::attend_workspace(a);
}

int csa_attend(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int k,
               int W, int64_t q_pos0, const void* q, const void* kv, const float* kv_scale,
               const int32_t* idx, const void* win, const float* win_scale, const float* sink,
               float scale, uint32_t flags, float rope_base, int rope_dims, void* out, float* lse_out,
               void* ws, size_t ws_bytes) {
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = k; a.W = W;
  a.sparse = true; a.N_cap = N_cap; a.q_pos0 = q_pos0; a.q = q; a.kv = kv; a.win = win;
  a.kv_scale = kv_scale; a.win_scale = win_scale; a.sink = sink; a.idx = idx; a.scale = scale;
  a.flags = flags; a.rope_base = rope_base; a.rope_dims = rope_dims; a.out = out; a.lse_out = lse_out;
  return run_attend(stream, a, ws, ws_bytes, "csa_attend");
}

size_t hca_attend_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int W,
                            int64_t q_pos0) {
  if (B < 1 || Tq < 1 || H < 1 || D < 1 || m < 1 || W < 1) return 0;
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = 0; a.W = W;
  a.sparse = false; a.N_cap = N_cap; a.q_pos0 = q_pos0;
  return lca::attend_workspace(a);
}

int hca_attend(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int W,
               int64_t q_pos0, const void* q, const void* kv, const float* kv_scale, const void* win,
               const float* win_scale, const float* sink, float scale, uint32_t flags, float rope_base,
               int rope_dims, void* out, float* lse_out, void* ws, size_t ws_bytes) {
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = 0; a.W = W;
  a.sparse = false; a.N_cap = N_cap; a.q_pos0 = q_pos0; a.q = q; a.kv = kv; a.win = win;
  a.kv_scale = kv_scale; a.win_scale = win_scale; a.sink = sink; a.idx = nullptr; a.scale = scale;
  a.flags = flags; a.rope_base = rope_base; a.rope_dims = rope_dims; a.out = out; a.lse_out = lse_out;
  return run_attend(stream, a, ws, ws_bytes, "hca_attend");
}

// ---------------------------------------------------------------------------
// csa_attend_noalloc: csa_attend with its split partials in a static device
// array instead of a caller workspace, for callers that cannot allocate.
// `scratch` is a host-side stand-in in host code: kernels get the device
// address that hipGetSymbolAddress returns for the current device (each GPU
// holds its own copy of the array, at its own address), never the name.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out, const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(LCA_ERR_UNSUPPORTED, "%s: device %d is beyond the %d this library tracks", fn, dev, kMaxScratchDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {                                   // once per device, with that device current
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, fn);
      if (!p) return fail(LCA_ERR_HIP, "%s: no device address for the static scratch array", fn);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LCA_OK;
}
}  // namespace

int csa_attend_noalloc(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int k,
                       int W, int64_t q_pos0, const void* q, const void* kv, const float* kv_scale,
                       const int32_t* idx, const void* win, const float* win_scale, const float* sink,
                       float scale, uint32_t flags, float rope_base, int rope_dims, void* out, float* lse_out) {
  const char* fn = "csa_attend_noalloc";
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = k; a.W = W;
  a.sparse = true; a.N_cap = N_cap; a.q_pos0 = q_pos0; a.q = q; a.kv = kv; a.win = win;
  a.kv_scale = kv_scale; a.win_scale = win_scale; a.sink = sink; a.idx = idx; a.scale = scale;
  a.flags = flags; a.rope_base = rope_base; a.rope_dims = rope_dims; a.out = out; a.lse_out = lse_out;
  int st = check_attend(a, fn);
  if (st != LCA_OK) return st;
  const size_t need = lca::attend_workspace(a);
  if (need > kScratchBytes)
    return fail(LCA_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch; the static array holds %zu "
                "(use csa_attend with a workspace)", fn, need, kScratchBytes);
  void* ws = nullptr;
  st = scratch_address(&ws, fn);
  if (st != LCA_OK) return st;
  return hip_status(lca::launch_attend(static_cast<hipStream_t>(stream), a, ws, kScratchBytes), fn);
}

// ---------------------------------------------------------------------------
// Backward of the core attention.
static int run_attend_bwd(void* stream, lca::AttendArgs& a, const void* out, const float* lse, const void* dout,
                          float* dq, float* dkv, float* dwin, float* dsink, void* ws, size_t ws_bytes,
                          const char* fn) {
  a.out = const_cast<void*>(out);                  // the forward's checks cover out
  int st = check_attend(a, fn);
  if (st != LCA_OK) return st;
  if (a.dt_q != LCA_BF16 || a.dt_kv != LCA_BF16 || a.D != 512 || a.H % 64 != 0 || a.H > 128)
    return fail(LCA_ERR_UNSUPPORTED, "%s: the backward takes bf16 q and rows, D = 512, H = 64 or 128", fn);
  if (a.flags & ~LCA_INV_ROPE) return fail(LCA_ERR_ARG, "%s: only LCA_INV_ROPE applies", fn);
  if (a.Tq > 65535) return fail(LCA_ERR_UNSUPPORTED, "%s: Tq must be <= 65535", fn);
  if (!lse || !dout || !dq || !dkv || !dwin || !dsink)
    return fail(LCA_ERR_ARG, "%s: lse, dout, dq, dkv, dwin and dsink are required", fn);
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dkv) || !aligned16(dwin) || !aligned4(lse) || !aligned4(dsink))
    return fail(LCA_ERR_ALIGN, "%s: misaligned buffer", fn);
  const size_t need = lca::attend_backward_workspace(a);
  if (!ws || ws_bytes < need) return fail(LCA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (!aligned16(ws)) return fail(LCA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  lca::AttendBwdArgs p{a, out, lse, dout, dq, dkv, dwin, dsink};
  return hip_status(lca::launch_attend_backward(static_cast<hipStream_t>(stream), p, ws, ws_bytes), fn);
}

size_t csa_attend_backward_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int k,
                                     int W, int64_t q_pos0) {
  if (B < 1 || Tq < 1 || H < 1 || D < 1 || m < 1 || W < 1 || N_cap < 0) return 0;
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = k; a.W = W;
  a.sparse = true; a.N_cap = N_cap; a.q_pos0 = q_pos0;
  return lca::attend_backward_workspace(a);
}

size_t hca_attend_backward_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int W,
                                     int64_t q_pos0) {
  if (B < 1 || Tq < 1 || H < 1 || D < 1 || m < 1 || W < 1 || N_cap < 0) return 0;
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = 0; a.W = W;
  a.sparse = false; a.N_cap = N_cap; a.q_pos0 = q_pos0;
  return lca::attend_backward_workspace(a);
}

int csa_attend_backward(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int k,
                        int W, int64_t q_pos0, const void* q, const void* kv, const int32_t* idx, const void* win,
                        const float* sink, float scale, uint32_t flags, float rope_base, int rope_dims,
                        const void* out, const float* lse, const void* dout, float* dq, float* dkv, float* dwin,
                        float* dsink, void* ws, size_t ws_bytes) {
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = k; a.W = W;
  a.sparse = true; a.N_cap = N_cap; a.q_pos0 = q_pos0; a.q = q; a.kv = kv; a.win = win; a.sink = sink;
  a.idx = idx; a.scale = scale; a.flags = flags; a.rope_base = rope_base; a.rope_dims = rope_dims;
  return run_attend_bwd(stream, a, out, lse, dout, dq, dkv, dwin, dsink, ws, ws_bytes, "csa_attend_backward");
}

int hca_attend_backward(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int W,
                        int64_t q_pos0, const void* q, const void* kv, const void* win, const float* sink,
                        float scale, uint32_t flags, float rope_base, int rope_dims, const void* out,
                        const float* lse, const void* dout, float* dq, float* dkv, float* dwin, float* dsink,
                        void* ws, size_t ws_bytes) {
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = 0; a.W = W;
  a.sparse = false; a.N_cap = N_cap; a.q_pos0 = q_pos0; a.q = q; a.kv = kv; a.win = win; a.sink = sink;
  a.idx = nullptr; a.scale = scale; a.flags = flags; a.rope_base = rope_base; a.rope_dims = rope_dims;
  return run_attend_bwd(stream, a, out, lse, dout, dq, dkv, dwin, dsink, ws, ws_bytes, "hca_attend_backward");
}

// ---------------------------------------------------------------------------
// Ragged batches: sequence b's queries sit at q_pos[b] + t (device array),
// with q_pos0 the bound that sizes workspaces, plans and validation.
static int check_q_pos(const int64_t* q_pos, const char* fn) {
  if (!q_pos) return fail(LCA_ERR_ARG, "%s: q_pos is required", fn);
  if (reinterpret_cast<uintptr_t>(q_pos) % 8 != 0) return fail(LCA_ERR_ALIGN, "%s: q_pos must be 8-byte aligned", fn);
  return LCA_OK;
}

int csa_index_topk_ragged(void* stream, int dt, int B, int Tq, int H_I, int d_I, int64_t N_cap, int m, int k,
                          int64_t q_pos_max, const int64_t* q_pos, const void* qI, const void* qI_scale,
                          const float* w, const void* kI, const void* kI_scale, uint32_t flags, int32_t* idx_out,
                          float* score_out, void* ws, size_t ws_bytes) {
  int st = check_q_pos(q_pos, "csa_index_topk_ragged");
  if (st != LCA_OK) return st;
  lca::IndexArgs a{dt, B, Tq, H_I, d_I, m, k, N_cap, q_pos_max, qI, qI_scale, kI, kI_scale, w, flags, idx_out,
                   score_out, q_pos};
  st = check_index(a);
  if (st != LCA_OK) return st;
  const size_t need = lca::index_topk_workspace(a);
  if (!ws || ws_bytes < need) return fail(LCA_ERR_WORKSPACE, "csa_index_topk_ragged: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(ws)) return fail(LCA_ERR_ALIGN, "csa_index_topk_ragged: workspace must be 16-byte aligned");
  return hip_status(lca::launch_index_topk(static_cast<hipStream_t>(stream), a, ws, ws_bytes), "csa_index_topk_ragged");
}

int csa_attend_ragged(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int k,
                      int W, int64_t q_pos_max, const int64_t* q_pos, const void* q, const void* kv,
                      const float* kv_scale, const int32_t* idx, const void* win, const float* win_scale,
                      const float* sink, float scale, uint32_t flags, float rope_base, int rope_dims, void* out,
                      float* lse_out, void* ws, size_t ws_bytes) {
  int st = check_q_pos(q_pos, "csa_attend_ragged");
  if (st != LCA_OK) return st;
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = k; a.W = W;
  a.sparse = true; a.N_cap = N_cap; a.q_pos0 = q_pos_max; a.q = q; a.kv = kv; a.win = win;
  a.kv_scale = kv_scale; a.win_scale = win_scale; a.sink = sink; a.idx = idx; a.scale = scale;
  a.flags = flags; a.rope_base = rope_base; a.rope_dims = rope_dims; a.out = out; a.lse_out = lse_out;
  a.q_pos = q_pos;
  return run_attend(stream, a, ws, ws_bytes, "csa_attend_ragged");
}

int hca_attend_ragged(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap, int m, int W,
                      int64_t q_pos_max, const int64_t* q_pos, const void* q, const void* kv, const float* kv_scale,
                      const void* win, const float* win_scale, const float* sink, float scale, uint32_t flags,
                      float rope_base, int rope_dims, void* out, float* lse_out, void* ws, size_t ws_bytes) {
  int st = check_q_pos(q_pos, "hca_attend_ragged");
  if (st != LCA_OK) return st;
  lca::AttendArgs a{};
  a.dt_q = dt_q; a.dt_kv = dt_kv; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.m = m; a.k = 0; a.W = W;
  a.sparse = false; a.N_cap = N_cap; a.q_pos0 = q_pos_max; a.q = q; a.kv = kv; a.win = win;
  a.kv_scale = kv_scale; a.win_scale = win_scale; a.sink = sink; a.idx = nullptr; a.scale = scale;
  a.flags = flags; a.rope_base = rope_base; a.rope_dims = rope_dims; a.out = out; a.lse_out = lse_out;
  a.q_pos = q_pos;
  return run_attend(stream, a, ws, ws_bytes, "hca_attend_ragged");
}

}  // extern "C"
