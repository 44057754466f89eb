/*
 * lca.h — C ABI of the MI355X (gfx950) hybrid compressed attention library.
 *
 * The library implements the attention hot path described on the source pages
 * (DeepSeek-V4 hybrid attention): the CSA path (token compressor with m = 4,
 * Lightning Indexer scores, top-k selection, multi-query attention over the
 * selected compressed entries plus a 128-token raw sliding window and a
 * learnable sink logit) and the HCA path (m' = 128 compression and dense
 * multi-query attention over all compressed entries plus the same window and
 * sink). Page short names in citations:
 *   [PACMAN] "DeepSeek-V4 technical report share" (THU PACMAN group, 10100.com)
 *   [Qiaomu] "DeepSeek-V4论文解析" (乔木博客 mirror)
 *   [cdjax]  "未来科技" DeepSeek-V4 essay (cdjax.com)
 *   [kwkr]   kwkr.cn DeepSeek-V4 report walk-through
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are device pointers to contiguous, row-major memory with the
 *   batch index outermost. The caller owns every buffer; the library never
 *   allocates, frees or synchronises. Scratch memory comes from a caller
 *   workspace sized by the matching *_workspace() call.
 * - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *   Kernels are enqueued asynchronously on it; execution errors surface at
 *   the caller's next synchronisation.
 * - Every argument is validated on the host before anything is launched, so
 *   a non-zero status means nothing was enqueued and nothing was written.
 *   The text of the last error of the calling thread is in lca_last_error().
 * - Query t of a call sits at absolute position q_pos0 + t (the same for all
 *   sequences of the batch). Compressed entry j covers tokens [j*m, (j+1)*m)
 *   and is visible to a query at position p iff j < (p + 1) / m.
 * - A window buffer `win` has W - 1 + Tq rows per sequence; row r holds the
 *   raw KV of position q_pos0 - (W - 1) + r. Rows at negative positions are
 *   never read. A query at p attends positions [max(0, p - W + 1), p].
 * - Results are bitwise deterministic run to run, and the result of sequence
 *   b does not depend on B or on the other sequences (work splits depend only
 *   on per-sequence shapes).
 * - Device pointers must be 16-byte aligned; float32 side arrays 4-byte.
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define LCA_OK               0
#define LCA_ERR_ARG         (-1) /* null pointer, bad dimension or position */
#define LCA_ERR_UNSUPPORTED (-2) /* dtype / shape combination not built     */
#define LCA_ERR_ALIGN       (-3) /* pointer not 16-byte aligned             */
#define LCA_ERR_WORKSPACE   (-4) /* workspace null or too small             */
#define LCA_ERR_HIP         (-5) /* kernel launch failed (see last_error)   */

/* ---- element formats --------------------------------------------------- */
#define LCA_F32       0 /* float32                                             */
#define LCA_BF16      1 /* bfloat16 stored as uint16                            */
#define LCA_KV_MIXED  2 /* KV row: (D - R) e4m3fn bytes, then R bf16 values;
                           plus one float32 scale per row in a side array.
                           [cdjax] §1.1: RoPE channels BF16, the rest FP8.      */
#define LCA_MXFP4     3 /* e2m1 codes packed two per byte (element 2i in the
                           low nibble), one e8m0 scale byte per 32 elements in
                           a side array. [Qiaomu] FP4量化感知训练, [kwkr] §3.4:
                           the indexer QK path runs in FP4.                     */

/* ---- flags ------------------------------------------------------------- */
#define LCA_NORM        1u /* compress: RMSNorm of each entry (gain norm_w)    */
#define LCA_ROPE        2u /* compress: RoPE of the last rope_dims channels at
                              the block start position pos0 + j*m             */
#define LCA_INV_ROPE    4u /* attend: rotate the output's last rope_dims
                              channels by the negative query position         */
#define LCA_SCORE_BF16  8u /* index_topk: round scores to bf16 before top-k    */
#define LCA_SPLITS_ONE_WG  32u /* attend: run all of a query's splits in one
                              workgroup (no partials, no combine) where a kernel
                              for it exists (bf16 rows, D = 512: fewer than
                              64 heads, or a multiple of 64, 128-head plans as
                              two 64-head groups); by default a cost model picks
                              it from the batch size ([Qiaomu] 批不变 kernel,
                              [kwkr] §4.3: a throughput and a latency kernel
                              with one accumulation order). Same bits either
                              way: a placement choice only                    */
#define LCA_SPLITS_MANY_WG 64u /* attend: one workgroup per split + combine     */
#define LCA_WIN_RING   16u /* attend: win is a ring of W-1+Tq rows per sequence,
                              position p in row p mod (W-1+Tq) (lca_window_append
                              fills it); without it, row r is position
                              q_pos - (W-1) + r                                */

/* ---------------------------------------------------------------------------
 * csa_compress — gated softmax-weighted token compressor (CSA and HCA).
 *
 * [kwkr] §3.1: two independent KV sequences are merged with softmax-normalised
 * gate weights, and adjacent compressed blocks overlap. [Qiaomu] 混合注意力机制:
 * every 4 tokens fold into one entry (CSA); HCA folds every 128 ([PACMAN] §3.2).
 *
 * With overlap = 1, entry j = sum over the 2m rows {stream a, block j-1} and
 * {stream b, block j} of softmax(their gate logits) * row. For j = 0 the
 * block j-1 rows are prev_ca / prev_za (the last m tokens of stream a before
 * this call) or, when prev_ca is NULL, absent. With overlap = 0 only stream b
 * is used (ca, za, prev_* must be NULL). The trailing T % m tokens emit nothing.
 * Then, per flags: RMSNorm (norm_w [D], eps), RoPE at position pos0 + j*m
 * (interleaved channel pairs of the last rope_dims channels, frequency
 * rope_base^(-2i/rope_dims)), then conversion to dt_out.
 *
 *   ca, cb    [B, T, D]   dt_in (LCA_F32 or LCA_BF16)
 *   za, zb    [B, T]      float32 gate logits
 *   prev_ca   [B, m, D]   dt_in, prev_za [B, m] float32 (both NULL or both set)
 *   out       [B, out_rows, ...] entry j of sequence b at row b*out_rows + j:
 *               LCA_F32 / LCA_BF16: D values;
 *               LCA_KV_MIXED: D - rope_dims + 2*rope_dims bytes,
 *                             out_scale float32 [B, out_rows];
 *               LCA_MXFP4: D/2 bytes, out_scale uint8 [B, out_rows, D/32].
 *   out_rows  row stride per sequence (>= T/m), lets entries land inside a
 *             larger cache; 0 means T/m.
 * Requirements: B >= 1, T >= 0, m >= 1, D % 32 == 0, D <= 1024,
 *   pos0 % m == 0, rope_dims even and <= D (0 with no LCA_ROPE unless
 *   dt_out is LCA_KV_MIXED, where it sets the bf16 channel count).
 * ------------------------------------------------------------------------- */
int csa_compress(void* stream, int dt_in, int dt_out, int B, int T, int D, int m,
                 int overlap, int64_t pos0,
                 const void* ca, const float* za, const void* cb, const float* zb,
                 const void* prev_ca, const float* prev_za,
                 uint32_t flags, const float* norm_w, float eps,
                 float rope_base, int rope_dims,
                 void* out, void* out_scale, int64_t out_rows);

/* ---------------------------------------------------------------------------
 * csa_compress_backward — gradients of csa_compress's entries (before the
 * conversion to dt_out) with respect to its inputs. [kwkr] §4.3 names the
 * attention block's backward as the training workload; this is the
 * compressor's part, by the chain rule through the RoPE (its adjoint turns
 * the gradient back by the same angle), the RMSNorm and the gated merge.
 *
 *   forward arguments as csa_compress (dt_in, B, T, D, m, overlap, pos0, ca,
 *             za, cb, zb, prev_ca, prev_za, flags, norm_w, eps, rope_base,
 *             rope_dims); no dt_out, out or out_scale
 *   dout      [B, T/m, D] float32: gradient of the entries
 *   dcb [B, T, D], dzb [B, T] float32, written in full (rows that no entry
 *             reads get 0)
 *   dca [B, T, D], dza [B, T] float32: required with overlap, else NULL
 *   dprev_ca [B, m, D], dprev_za [B, m] float32: required with prev_ca, else NULL
 *   dnorm_w [D] float32: required with LCA_NORM (summed over every entry of
 *             every sequence, in a fixed order), else NULL
 *   ws        workspace of csa_compress_backward_workspace() bytes (B*(T/m)*D
 *             floats with LCA_NORM); NULL allowed without LCA_NORM.
 * Deterministic: every row gradient is written once; dnorm_w sums per-entry
 * rows in order. Requirements as csa_compress; buffers 16-byte aligned.
 * ------------------------------------------------------------------------- */
size_t csa_compress_backward_workspace(int B, int T, int D, int m, uint32_t flags);
int csa_compress_backward(void* stream, int dt_in, int B, int T, int D, int m, int overlap, int64_t pos0,
                          const void* ca, const float* za, const void* cb, const float* zb,
                          const void* prev_ca, const float* prev_za,
                          uint32_t flags, const float* norm_w, float eps, float rope_base, int rope_dims,
                          const float* dout, float* dca, float* dza, float* dcb, float* dzb,
                          float* dprev_ca, float* dprev_za, float* dnorm_w, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * Decode-time state: csa_compress_append, lca_window_append.
 *
 * [kwkr] §4.4: the KV cache of a request splits into a state cache (what stays
 * a fixed size: the uncompressed tail of the compressor and the sliding
 * window) and a classical KV cache (the compressed entries, growing by one
 * entry every m tokens). These calls keep both while decoding one token per
 * sequence per call, each sequence at its own position (a ragged batch).
 *
 * csa_compress_append: sequence b appends its token at position pos[b]
 * (int64, device memory, 8-byte aligned; a sequence whose position lies
 * outside [0, pos_max] is left untouched this call). Positions must advance
 * one token at a time from 0 for the state to hold the right rows. The token's
 * rows are ca / cb [B, D] (dt_in) and its gate logits za / zb [B] (float32);
 * stream a is NULL without overlap. When the token closes block j (pos % m ==
 * m - 1), entry j is formed exactly as csa_compress forms it — same rows, same
 * softmax, same epilogue (RoPE at position j*m), so the same bits as a one-shot
 * csa_compress of the whole sequence with pos0 = 0 — and written to out row
 * b * out_rows + j (formats as csa_compress; out_rows >= (pos_max + 1) / m).
 * state: caller-owned device buffer of csa_compress_state_bytes() bytes,
 * 16-byte aligned, one region per sequence, no initialisation needed. Layout
 * (rows in dt_in): per sequence R rows of D values, R = 3m with overlap (stream
 * a of block n in rows (n mod 2)*m + i, stream b of the current block in rows
 * 2m + i), R = m without (stream b); after all rows, from the next 256-byte
 * boundary, float32 gate logits [B, R] indexed alike. Copying the buffer
 * takes a checkpoint of the state and copying it back restores it (the pages'
 * Full / Periodic / Zero SWA caching policies are such copies, made by the
 * caller). Calls on one state buffer must not overlap in time.
 * Returns 0 from csa_compress_state_bytes for invalid arguments.
 *
 * lca_window_append: sequence b stores its token's raw KV row src [B, D]
 * (dt_in F32 or BF16) into ring row pos[b] mod ring_rows of win [B,
 * ring_rows, ...] in dt_out (F32, BF16, or KV_MIXED with win_scale [B,
 * ring_rows] and rope_dims bf16 channels, converted as lca_quantize_rows).
 * Attention reads the ring with LCA_WIN_RING and ring_rows = W - 1 + Tq.
 * ------------------------------------------------------------------------- */
/* lca_decode_append: every append of one decode step in one launch — up to
 * LCA_MAX_APPEND_JOBS jobs, each a compressor append (as csa_compress_append)
 * or a window-ring store (as lca_window_append), over the same positions.
 * Results equal those of the separate calls, bit for bit. Each job is checked
 * as its separate call checks it; on any error nothing is launched. The jobs
 * array is read on the host during the call. */
#define LCA_APPEND_COMPRESS 0
#define LCA_APPEND_WINDOW   1
#define LCA_MAX_APPEND_JOBS 4
typedef struct lca_append_job {
  int kind;                 /* LCA_APPEND_COMPRESS or LCA_APPEND_WINDOW                  */
  int dt_in, dt_out, D;
  int m, overlap;           /* compressor: ratio and overlap                             */
  uint32_t flags;           /* compressor: LCA_NORM | LCA_ROPE                           */
  int rope_dims;            /* compressor: RoPE / bf16 channels; window: KV_MIXED bf16   */
  float eps, rope_base;     /* compressor                                                */
  const void* ca;           /* compressor, overlap: stream a row [B, D]                  */
  const float* za;          /*                      and its gate logit [B]               */
  const void* cb;           /* compressor: stream b row [B, D]; window: the raw row      */
  const float* zb;          /* compressor: stream b gate logit [B]; window: NULL          */
  const float* norm_w;      /* compressor with LCA_NORM                                  */
  void* state;              /* compressor: its state buffer                              */
  size_t state_bytes;
  void* out;                /* compressor: entry cache; window: the ring                 */
  void* out_scale;          /* scales of a quantised cache or ring                       */
  int64_t out_rows;         /* compressor: rows per sequence; window: ring rows          */
} lca_append_job;
int lca_decode_append(void* stream, int B, int64_t pos_max, const int64_t* pos,
                      const lca_append_job* jobs, int n_jobs);

size_t csa_compress_state_bytes(int dt_in, int B, int D, int m, int overlap);
int csa_compress_append(void* stream, int dt_in, int dt_out, int B, int D, int m, int overlap,
                        int64_t pos_max, const int64_t* pos,
                        const void* ca, const float* za, const void* cb, const float* zb,
                        void* state, size_t state_bytes,
                        uint32_t flags, const float* norm_w, float eps,
                        float rope_base, int rope_dims,
                        void* out, void* out_scale, int64_t out_rows);
int lca_window_append(void* stream, int dt_in, int dt_out, int B, int D, int rope_dims, int ring_rows,
                      int64_t pos_max, const int64_t* pos, const void* src, void* win,
                      float* win_scale);

/* ---------------------------------------------------------------------------
 * lca_quantize_rows — quantise-on-write of float32 rows to a storage format.
 *
 * LCA_KV_MIXED ([cdjax] §1.1): per row s = amax/448 over the first D - R
 * channels (float32 division; s = 1 if amax = 0); byte c = e4m3fn(x_c / s),
 * round to nearest even, saturating at 448; the last R channels are bf16
 * (round to nearest even). out [n_rows, D - R + 2R] bytes, out_scale float32
 * [n_rows].
 * LCA_MXFP4 ([kwkr] §3.4, OCP MX v1.0): per block of 32 channels, E8M0 scale
 * X = 2^(floor(log2 amax) - 2) (byte 0 and zero codes if amax = 0); element
 * code e2m1(x / X), round to nearest even, saturating at 6. out [n_rows, D/2],
 * out_scale uint8 [n_rows, D/32].
 * Requirements: n_rows >= 0, D % 32 == 0, D <= 1024; MIXED: 0 <= R <= D, R even.
 * ------------------------------------------------------------------------- */
int lca_quantize_rows(void* stream, int dt_out, int64_t n_rows, int D, int rope_dims,
                      const float* src, void* out, void* out_scale);

/* ---------------------------------------------------------------------------
 * csa_index_topk — Lightning Indexer scores of every visible entry + top-k.
 *
 * [Qiaomu] 混合注意力机制: cheap indexer queries score every compressed block and
 * the top-k most relevant are kept; [PACMAN] §3.1: k = 512 (Flash) / 1024
 * (Pro). Score (the pages print no formula; [kwkr] §3.1 says CSA runs
 * DeepSeek Sparse Attention on the entries): s_j = sum_h w_h * relu(qI_h . kI_j)
 * over the H_I indexer heads, for j < n_vis = (q_pos0 + t + 1) / m, accumulated
 * in float32. With LCA_SCORE_BF16 each score is rounded to bf16 first
 * ([Qiaomu] FP4量化感知训练: BF16 scores make top-k twice as fast).
 * Selection: the min(k, n_vis) largest scores, ties to the lower index.
 *
 *   dt        LCA_F32, LCA_BF16 (qI and kI in that type) or LCA_MXFP4
 *             (qI and kI packed e2m1, scales in qI_scale / kI_scale)
 *   qI        [B, Tq, H_I, d_I]       qI_scale [B, Tq, H_I, d_I/32] (MXFP4)
 *   w         [B, Tq, H_I] float32
 *   kI        [B, N_cap, d_I]         kI_scale [B, N_cap, d_I/32]  (MXFP4)
 *   idx_out   [B, Tq, k] int32: the selected entries in increasing index
 *             order, then -1 padding
 *   score_out [B, Tq, k] float32 or NULL: the score of each idx_out entry
 *             (-inf for padding)
 * Requirements: N_cap >= n_vis of the last query; 1 <= k <= 4096;
 *   d_I % 32 == 0 and d_I <= 256; H_I in {1, 2, 4, 8, 16, 32, 64} for LCA_BF16
 *   and LCA_MXFP4 (the pages' indexer has 64 heads, [Qiaomu] 训练配置; any
 *   H_I <= 64 for LCA_F32); MXFP4 needs d_I == 128.
 * ------------------------------------------------------------------------- */
size_t csa_index_topk_workspace(int dt, int B, int Tq, int H_I, int d_I, int64_t N_cap,
                                int m, int k, int64_t q_pos0, uint32_t flags);
int csa_index_topk(void* stream, int dt, int B, int Tq, int H_I, int d_I, int64_t N_cap,
                   int m, int k, int64_t q_pos0,
                   const void* qI, const void* qI_scale, const float* w,
                   const void* kI, const void* kI_scale, uint32_t flags,
                   int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * csa_attend — CSA core attention over selected entries + window + sink.
 *
 * [PACMAN] §3.1: only the top-k compressed entries are attended, plus a recent
 * uncompressed window; [kwkr] §3.3: the 128 window rows join the core
 * computation together with the sink (a learnable term in the softmax
 * denominator); [cdjax] §1.1: multi-query form (one KV row serves as key and
 * value for every head) and RoPE at the negative query position on the output.
 *
 * For query t (position p) and head h, over rows X = {kv[idx[t, i]] : idx >= 0}
 * followed by the window rows of positions [max(0, p-W+1), p]:
 *   l_x = scale * q_h . x,  M = max(sink_h, max l),
 *   Z = exp(sink_h - M) + sum exp(l_x - M),  out = sum exp(l_x - M) x / Z,
 *   lse = M + log Z; with LCA_INV_ROPE the last rope_dims channels of out are
 *   rotated by -p.
 *
 *   dt_q      LCA_F32 or LCA_BF16 (q and out)
 *   dt_kv     LCA_F32 (with dt_q = LCA_F32), LCA_BF16 or LCA_KV_MIXED
 *   q         [B, Tq, H, D]            out [B, Tq, H, D] dt_q
 *   kv        [B, N_cap, D] (MIXED: row of D - rope_dims + 2*rope_dims bytes,
 *             kv_scale float32 [B, N_cap])
 *   idx       [B, Tq, k] int32; entries < 0 or >= N_cap are skipped
 *   win       [B, W - 1 + Tq, D] same format as kv (win_scale [B, W-1+Tq])
 *   sink      [H] float32
 *   lse_out   [B, Tq, H] float32 or NULL
 * Requirements: D % 32 == 0, D <= 512; H % 16 == 0 unless dt_kv == LCA_F32;
 *   1 <= W <= 4096; 1 <= k <= 4096; q_pos0 >= 0.
 * ------------------------------------------------------------------------- */
size_t csa_attend_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                            int m, int k, int W, int64_t q_pos0);
int csa_attend(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
               int m, int k, int W, int64_t q_pos0,
               const void* q, const void* kv, const float* kv_scale, const int32_t* idx,
               const void* win, const float* win_scale, const float* sink, float scale,
               uint32_t flags, float rope_base, int rope_dims,
               void* out, float* lse_out, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * csa_attend_noalloc — csa_attend for callers that cannot allocate.
 *
 * For code that may not call hipMalloc or take a workspace: work under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * arguments, layouts, requirements, results and errors are those of
 * csa_attend (same kernels, same bits) without ws / ws_bytes: the split
 * partials go to a static device array of 64 MiB (LCA_NOALLOC_SCRATCH_BYTES)
 * inside the library, one per GPU, held until the process ends. A call whose
 * csa_attend_workspace() exceeds that size returns LCA_ERR_WORKSPACE and
 * enqueues nothing (at the CSA decode shape, H = 64, D = 512, k = 512 at
 * 131072 tokens, up to 51 sequences fit). The call allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, two threads) race on it and must be serialised by
 * the caller. Nothing in the array needs to start at zero; each call writes
 * every partial it reads.
 * ------------------------------------------------------------------------- */
#define LCA_NOALLOC_SCRATCH_BYTES (64u << 20)
int csa_attend_noalloc(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                       int m, int k, int W, int64_t q_pos0,
                       const void* q, const void* kv, const float* kv_scale, const int32_t* idx,
                       const void* win, const float* win_scale, const float* sink, float scale,
                       uint32_t flags, float rope_base, int rope_dims,
                       void* out, float* lse_out);

/* ---------------------------------------------------------------------------
 * hca_attend — HCA dense attention over every visible entry + window + sink.
 *
 * [PACMAN] §3.2 and [kwkr] §3.2: no sparse selection; dense multi-query
 * attention over all heavily compressed entries (m' = 128), with the same
 * sliding window and sink as CSA. Identical to csa_attend with the selected
 * set replaced by all entries j < (p + 1) / m. Arguments as for csa_attend.
 * ------------------------------------------------------------------------- */
size_t hca_attend_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                            int m, int W, int64_t q_pos0);
int hca_attend(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
               int m, int W, int64_t q_pos0,
               const void* q, const void* kv, const float* kv_scale,
               const void* win, const float* win_scale, const float* sink, float scale,
               uint32_t flags, float rope_base, int rope_dims,
               void* out, float* lse_out, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * Ragged batches: *_ragged — the same three calls with a position per sequence.
 *
 * [kwkr] §4.4: serving keeps a KV cache per request (state cache and classical
 * KV cache), so the sequences of one decode batch sit at different positions.
 * The pages leave the batching interface open; here sequence b's query t sits
 * at position q_pos[b] + t, and everything that depends on a position follows
 * it: visible entries n_vis = (q_pos[b] + t + 1) / m, the window rows (row r of
 * win[b] is position q_pos[b] - (W - 1) + r) and the inverse RoPE angle.
 *
 *   q_pos      int64 [B] in device memory, 8-byte aligned; each in
 *              [0, q_pos_max]. A value outside is clamped into that range
 *              (the kernels read it on the device; the host cannot check it).
 *   q_pos_max  the bound: it takes the place of q_pos0 in the requirements
 *              (N_cap >= visible entries at q_pos_max + Tq - 1) and in the
 *              workspace queries (call *_workspace with q_pos0 = q_pos_max).
 * Every other argument, layout and requirement is that of the uniform call.
 * Results for sequence b depend only on its own inputs, q_pos[b], q_pos_max and
 * the query shape: with a fixed bound (say the cache capacity) they are bitwise
 * independent of the batch, and equal to those of a uniform call with
 * q_pos0 = q_pos[b] whenever that call has the same split plan.
 * Returns LCA_ERR_ARG if q_pos is NULL, LCA_ERR_ALIGN if it is misaligned.
 * ------------------------------------------------------------------------- */
int csa_index_topk_ragged(void* stream, int dt, int B, int Tq, int H_I, int d_I, int64_t N_cap,
                          int m, int k, int64_t q_pos_max, const int64_t* q_pos,
                          const void* qI, const void* qI_scale, const float* w,
                          const void* kI, const void* kI_scale, uint32_t flags,
                          int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes);
int csa_attend_ragged(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                      int m, int k, int W, int64_t q_pos_max, const int64_t* q_pos,
                      const void* q, const void* kv, const float* kv_scale, const int32_t* idx,
                      const void* win, const float* win_scale, const float* sink, float scale,
                      uint32_t flags, float rope_base, int rope_dims,
                      void* out, float* lse_out, void* ws, size_t ws_bytes);
int hca_attend_ragged(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                      int m, int W, int64_t q_pos_max, const int64_t* q_pos,
                      const void* q, const void* kv, const float* kv_scale,
                      const void* win, const float* win_scale, const float* sink, float scale,
                      uint32_t flags, float rope_base, int rope_dims,
                      void* out, float* lse_out, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * csa_attend_backward / hca_attend_backward — gradients of the core attention.
 *
 * [Qiaomu] 批不变 kernel, [kwkr] §4.3: the attention backward accumulates per
 * SM into buffers of its own and sums them in a fixed order (deterministic).
 * Given the forward call's arguments, its output and lse, and dout (the
 * gradient of out), per query and head (P = softmax weights from lse, do =
 * dout turned back by +p when LCA_INV_ROPE was set, D = dout . out):
 *   dl_j = P_j (do . x_j - D),  dq = scale sum_j dl_j x_j,
 *   dx_j = sum_h (P_hj do_h + scale dl_hj q_h) into the entry or window row j
 *   was read from,  dsink_h = -sum over queries of P_sink D.
 * Every query is assigned to one of a fixed set of slots (ranges of 16 or
 * more consecutive queries); a slot walks its queries in order and adds the
 * rows' gradients into its own buffer; the buffers are then summed in slot
 * order. The result depends only on the arguments (run to run identical).
 *   q, kv, idx, win, sink, scale, flags, rope_*: as in the forward call
 *   out  [B, Tq, H, D] bf16, lse [B, Tq, H] fp32: the forward's results
 *   dout [B, Tq, H, D] bf16
 *   dq   [B, Tq, H, D] fp32;  dkv [B, N_cap, D] fp32 (rows no query read: 0);
 *   dwin [B, W-1+Tq, D] fp32 (rows at negative positions: 0);  dsink [H] fp32
 * Requirements: bf16 q and rows, D = 512, H = 64 or 128, Tq <= 65535,
 * window in the linear layout (no LCA_WIN_RING), one position for the batch;
 * a query's entry indices distinct and visible to it (index < (p + 1) / m),
 * as csa_index_topk gives them (other indices are not accumulated). Workspace
 * from *_backward_workspace (it holds per-slot buffers of N_cap x D fp32).
 * ------------------------------------------------------------------------- */
size_t csa_attend_backward_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                                     int m, int k, int W, int64_t q_pos0);
size_t hca_attend_backward_workspace(int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                                     int m, int W, int64_t q_pos0);
int csa_attend_backward(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                        int m, int k, int W, int64_t q_pos0, const void* q, const void* kv,
                        const int32_t* idx, const void* win, const float* sink, float scale,
                        uint32_t flags, float rope_base, int rope_dims, const void* out,
                        const float* lse, const void* dout, float* dq, float* dkv, float* dwin,
                        float* dsink, void* ws, size_t ws_bytes);
int hca_attend_backward(void* stream, int dt_q, int dt_kv, int B, int Tq, int H, int D, int64_t N_cap,
                        int m, int W, int64_t q_pos0, const void* q, const void* kv,
                        const void* win, const float* sink, float scale, uint32_t flags,
                        float rope_base, int rope_dims, const void* out, const float* lse,
                        const void* dout, float* dq, float* dkv, float* dwin, float* dsink,
                        void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * lca_grouped_out_proj — grouped output projection after core attention.
 *
 * [Qiaomu] 预训练策略 (model configurations), [cdjax] §1.1, [kwkr] §3.4: the
 * n_h heads form g groups of n_h/g consecutive heads; group gi's outputs
 * (n_h/g * c values per row) project to d_g channels, the g results
 * concatenate, and one more projection maps g*d_g channels to d_model
 * (Flash: n_h = 64, c = 512, g = 8, d_g = 1024, d_model = 4096; Pro: 128
 * heads, g = 16, d_model = 7168).
 *   o    [T, n_h, c] bf16        attention output rows (T = batch x queries)
 *   w_g  [g, d_g, (n_h/g)*c] bf16  row j of group gi = intermediate channel j
 *   w_o  [d_model, g*d_g] bf16   row n = output channel n
 *   mid  [T, g*d_g] bf16         the concatenated intermediate (written; the
 *                                second product reads it)
 *   out  [T, d_model] bf16
 * Sums are fp32; mid and out are rounded to bf16 (round to nearest even).
 * The sum over K runs in eight fixed parts added in a fixed order:
 * deterministic, and each row independent of T.
 * Requirements: n_h % g == 0; (n_h/g)*c and g*d_g multiples of 256; d_g and
 * d_model multiples of 16; buffers 16-byte aligned (device memory, caller-owned).
 * ------------------------------------------------------------------------- */
int lca_grouped_out_proj(void* stream, int T, int n_h, int c, int g, int d_g, int d_model,
                         const void* o, const void* w_g, const void* w_o, void* mid, void* out);

/* ---- diagnostics ------------------------------------------------------- */
const char* lca_status_str(int status);
const char* lca_last_error(void); /* thread-local text of the last failure */
int lca_version(void);            /* major*10000 + minor*100 + patch       */

/* ---------------------------------------------------------------------------
 * Kernel timing (diagnostic; not for production paths). When enabled, every
 * kernel the library enqueues is bracketed by a pair of HIP events recorded
 * on the caller's stream. lca_profile_collect waits for those events, sums
 * the durations per kernel name into `out` (at most max_entries, returns the
 * count written, or a negative status) and clears the record. This is the
 * one piece of process-global state; do not enable it while several threads
 * call the library.
 * ------------------------------------------------------------------------- */
typedef struct {
  char name[64];
  int64_t launches;
  double total_ms;
} lca_kernel_stat;
int lca_profile_enable(int on);
int lca_profile_collect(lca_kernel_stat* out, int max_entries);

#ifdef __cplusplus
}
#endif
#endif /* LCA_H */
