// C ABI of libdspark: argument validation, then the launch.
//
// Every host-checkable precondition is tested before the first HIP call, so
// an invalid call enqueues nothing and leaves the HIP state untouched.
#include <mutex>

#include "../../include/dspark.h"
#include "dspark_internal.h"

namespace dspark {

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] > 0) return cached[dev];
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    cached[dev] = cus;
  }
  return cus;
}

}  // namespace dspark

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Where the round's split lm_head workspace starts: past the Markov loop's,
// on a 256-byte boundary.
size_t round_split_offset(size_t markov_bytes) { return (markov_bytes + 255) / 256 * 256; }

dspark_status gemv_checks(const uint16_t* W, int N, int K, const float* X, int M, const float* Y) {
  if (!W || !X || !Y) return DSPARK_ERR_NULL;
  if (N < 1 || K < 8 || (K % 8) != 0 || M < 1 || !dspark::gemv_shape_fits(N, K, M)) return DSPARK_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 4)) return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

dspark_status gemv_q8_checks(const int8_t* Wq, const uint16_t* Wd, int N, int K, const float* X, int M,
                            const float* Y) {
  if (!Wq || !Wd || !X || !Y) return DSPARK_ERR_NULL;
  if (N < 1 || K < 32 || (K % 32) != 0 || M < 1 || !dspark::gemv_q8_shape_fits(N, K, M)) return DSPARK_ERR_SHAPE;
  if (!aligned(Wq, 16) || !aligned(Wd, 2) || !aligned(X, 16) || !aligned(Y, 4)) return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

dspark_status from_hip(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP; }

// A Q8_0 scale row stride: at least the K / 32 scales of a row, at most one
// 128-byte line (64 scales) of padding beyond them.
dspark_status q8_ldd_check(int ldd, int K) {
  return ldd >= K / 32 && ldd <= K / 32 + 64 ? DSPARK_OK : DSPARK_ERR_SHAPE;
}

}  // namespace

extern "C" {

const char* dspark_status_string(dspark_status status) {
  switch (status) {
    case DSPARK_OK: return "DSPARK_OK";
    case DSPARK_ERR_NULL: return "DSPARK_ERR_NULL: a required pointer is NULL";
    case DSPARK_ERR_SHAPE: return "DSPARK_ERR_SHAPE: a size is out of range or inconsistent";
    case DSPARK_ERR_ALIGN: return "DSPARK_ERR_ALIGN: a pointer lacks the required alignment";
    case DSPARK_ERR_WORKSPACE: return "DSPARK_ERR_WORKSPACE: workspace missing or too small";
    case DSPARK_ERR_HIP: return "DSPARK_ERR_HIP: the HIP runtime refused a call or launch";
    default: return "DSPARK_ERR_UNKNOWN";
  }
}

dspark_status dspark_proj_smallm(const uint16_t* W, int N, int K, const float* X, int M, float* Y,
                                 void* stream) {
  const dspark_status st = gemv_checks(W, N, K, X, M, Y);
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_gemv(W, N, K, X, M, Y, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_lm_head(const uint16_t* W_lm, int V, int d, const float* H, int rows, float* logits,
                             void* stream) {
  const dspark_status st = gemv_checks(W_lm, V, d, H, rows, logits);
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_gemv(W_lm, V, d, H, rows, logits, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_proj_smallm_q8(const int8_t* Wq, const uint16_t* Wd, int N, int K, const float* X, int M,
                                    float* Y, void* stream) {
  const dspark_status st = gemv_q8_checks(Wq, Wd, N, K, X, M, Y);
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_gemv_q8(Wq, Wd, N, K, X, M, Y, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_lm_head_sched(const uint16_t* W_lm, int V, int d, const float* H, int rows, float* logits,
                                  uint32_t* counter, void* stream) {
  const dspark_status st = gemv_checks(W_lm, V, d, H, rows, logits);
  if (st != DSPARK_OK) return st;
  if (!counter) return DSPARK_ERR_NULL;
  if (!aligned(counter, 4)) return DSPARK_ERR_ALIGN;
  return from_hip(dspark::launch_gemv_sched(W_lm, V, d, H, rows, logits, counter, static_cast<hipStream_t>(stream)));
}

size_t dspark_lm_head_split_workspace_bytes(int V, int d, int rows) {
  if (V < 1 || d < 1 || rows < 1) return 0;
  return dspark::gemv_split_workspace_bytes(V, d, rows);
}

dspark_status dspark_lm_head_split(const uint16_t* W_lm, int V, int d, const float* H, int rows, float* logits,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  const dspark_status st = gemv_checks(W_lm, V, d, H, rows, logits);
  if (st != DSPARK_OK) return st;
  const size_t need = dspark::gemv_split_workspace_bytes(V, d, rows);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (need == 0) return from_hip(dspark::launch_gemv(W_lm, V, d, H, rows, logits, s));
  if (!workspace || workspace_bytes < need) return DSPARK_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return DSPARK_ERR_ALIGN;
  return from_hip(dspark::launch_gemv_split(W_lm, V, d, H, rows, logits, workspace, s));
}

dspark_status dspark_lm_head_q8(const int8_t* Wq, const uint16_t* Wd, int V, int d, const float* H, int rows,
                                float* logits, void* stream) {
  const dspark_status st = gemv_q8_checks(Wq, Wd, V, d, H, rows, logits);
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_gemv_q8(Wq, Wd, V, d, H, rows, logits, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_lm_head_q8_ld(const int8_t* Wq, const uint16_t* Wd, int ldd, int V, int d, const float* H,
                                   int rows, float* logits, void* stream) {
  dspark_status st = gemv_q8_checks(Wq, Wd, V, d, H, rows, logits);
  if (st == DSPARK_OK) st = q8_ldd_check(ldd, d);
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_gemv_q8(Wq, Wd, V, d, H, rows, logits, static_cast<hipStream_t>(stream), ldd));
}

size_t dspark_markov_workspace_bytes(int num_reqs, int k, int V) {
  return dspark::markov_workspace_bytes(num_reqs, k, V);
}

uint32_t dspark_markov_set_spin_limit(uint32_t polls) { return dspark::markov_set_spin_limit(polls); }

dspark_status dspark_stream_read_sched(const void* buf, size_t bytes, int groups, int threads, uint32_t* counter,
                                       uint32_t* sink, void* stream) {
  if ((bytes > 0 && !buf) || !sink || !counter) return DSPARK_ERR_NULL;
  if (groups < 1 || groups > 65536 || (threads != 256 && threads != 512 && threads != 1024) || (bytes % 16) != 0 ||
      bytes / (16u * 16384u) >= (1u << 30))
    return DSPARK_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4) || !aligned(counter, 4)) return DSPARK_ERR_ALIGN;
  return from_hip(dspark::launch_stream_read_sched(buf, bytes, groups, threads, counter, sink,
                                                   static_cast<hipStream_t>(stream)));
}

dspark_status dspark_stream_read(const void* buf, size_t bytes, int groups, int threads, uint32_t* sink,
                                 void* stream) {
  if ((bytes > 0 && !buf) || !sink) return DSPARK_ERR_NULL;
  if (groups < 1 || groups > 65536 || (threads != 256 && threads != 512 && threads != 1024) || (bytes % 16) != 0)
    return DSPARK_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return DSPARK_ERR_ALIGN;
  return from_hip(dspark::launch_stream_read(buf, bytes, groups, threads, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

dspark_status markov_checks(const float* base, int num_reqs, int B, int V, const uint16_t* w1, const uint16_t* w2,
                            int r, const int64_t* d2t, const int64_t* prev0, int k, const int64_t* ids_out,
                            const void* workspace, size_t workspace_bytes) {
  if (!base || !w1 || !w2 || !prev0 || !ids_out) return DSPARK_ERR_NULL;
  if (num_reqs < 1 || num_reqs > 16 || B < 1 || V < 1 || k < 1 || k > B || k > 32 || r < 8 || r > 1024 || (r % 8) != 0)
    return DSPARK_ERR_SHAPE;
  if (!aligned(base, 4) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(prev0, 8) ||
      !aligned(ids_out, 8) || (d2t && !aligned(d2t, 8)))
    return DSPARK_ERR_ALIGN;
  const size_t need = dspark::markov_workspace_bytes(num_reqs, k, V);
  if (!workspace || workspace_bytes < need) return DSPARK_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

dspark_status markov_q8_checks(const float* base, int num_reqs, int B, int V, const int8_t* w1q, const uint16_t* w1d,
                               const int8_t* w2q, const uint16_t* w2d, int r, const int64_t* d2t,
                               const int64_t* prev0, int k, const int64_t* ids_out, const void* workspace,
                               size_t workspace_bytes) {
  if (!base || !w1q || !w1d || !w2q || !w2d || !prev0 || !ids_out) return DSPARK_ERR_NULL;
  if (num_reqs < 1 || num_reqs > 16 || B < 1 || V < 1 || k < 1 || k > B || k > 32 || r < 32 || r > 256 || (r % 32) != 0)
    return DSPARK_ERR_SHAPE;
  if (!aligned(base, 4) || !aligned(w1q, 16) || !aligned(w2q, 16) || !aligned(w1d, 2) || !aligned(w2d, 2) ||
      !aligned(prev0, 8) || !aligned(ids_out, 8) || (d2t && !aligned(d2t, 8)))
    return DSPARK_ERR_ALIGN;
  const size_t need = dspark::markov_workspace_bytes(num_reqs, k, V);
  if (!workspace || workspace_bytes < need) return DSPARK_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

dspark_status probe_checks(const float* x, int M, int D, const uint16_t* w, const float* logit_out,
                           const int32_t* pass_out) {
  if (!x || !w || !logit_out) return DSPARK_ERR_NULL;
  if (M < 1 || D < 8 || (D % 8) != 0) return DSPARK_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(logit_out, 4) || (pass_out && !aligned(pass_out, 4)))
    return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

}  // namespace

extern "C" {

dspark_status dspark_markov_sample(const float* base, int num_reqs, int B, int V, const uint16_t* w1,
                                   const uint16_t* w2, int r, const int64_t* d2t, const int64_t* prev0, int k,
                                   int64_t* ids_out, void* workspace, size_t workspace_bytes, void* stream) {
  const dspark_status st =
      markov_checks(base, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, workspace, workspace_bytes);
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_markov(base, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, workspace,
                                        nullptr, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_markov_sample_noalloc(const float* base, int num_reqs, int B, int V, const uint16_t* w1,
                                           const uint16_t* w2, int r, const int64_t* d2t, const int64_t* prev0,
                                           int k, int64_t* ids_out, void* stream) {
  const size_t have = dspark::markov_scratch_bytes();
  // (a non-null stand-in: the static workspace is looked up below, after every check)
  dspark_status st = markov_checks(base, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, ids_out, have);
  if (st != DSPARK_OK) return st;
  void* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dspark::markov_scratch(&ws, s) != hipSuccess) return DSPARK_ERR_HIP;
  return from_hip(dspark::launch_markov(base, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, ws, nullptr, s));
}

dspark_status dspark_conf_probe(const float* x, int M, int D, const uint16_t* w, float bias, float threshold,
                                float* logit_out, int32_t* pass_out, void* stream) {
  const dspark_status st = probe_checks(x, M, D, w, logit_out, pass_out);
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_probe(x, M, D, w, bias, threshold, logit_out, pass_out,
                                       static_cast<hipStream_t>(stream)));
}

dspark_status dspark_markov_sample_probe(const float* base, int num_reqs, int B, int V, const uint16_t* w1,
                                         const uint16_t* w2, int r, const int64_t* d2t, const int64_t* prev0, int k,
                                         int64_t* ids_out, void* workspace, size_t workspace_bytes,
                                         const float* probe_x, int probe_M, int probe_D, const uint16_t* probe_w,
                                         float probe_bias, float probe_threshold, float* logit_out,
                                         int32_t* pass_out, void* stream) {
  dspark_status st =
      markov_checks(base, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, workspace, workspace_bytes);
  if (st == DSPARK_OK) st = probe_checks(probe_x, probe_M, probe_D, probe_w, logit_out, pass_out);
  if (st != DSPARK_OK) return st;
  const dspark::ProbeArgs pa{probe_x, probe_M, probe_D, probe_w, probe_bias, probe_threshold, logit_out, pass_out};
  return from_hip(dspark::launch_markov(base, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, workspace, &pa,
                                        static_cast<hipStream_t>(stream)));
}

size_t dspark_draft_round_workspace_bytes(int num_reqs, int B, int k, int V, int d) {
  if (num_reqs < 1 || num_reqs > 16 || B < 1 || B > (1 << 20) || d < 1) return 0;
  const size_t mk = dspark::markov_workspace_bytes(num_reqs, k, V);
  if (mk == 0) return 0;
  return round_split_offset(mk) + dspark::gemv_split_workspace_bytes(V, d, num_reqs * B);
}

dspark_status dspark_draft_round(const uint16_t* W_lm, int V, int d, const float* H, int num_reqs, int B,
                                 const uint16_t* w1, const uint16_t* w2, int r, const int64_t* d2t,
                                 const int64_t* prev0, int k, const uint16_t* probe_w, float probe_bias,
                                 float probe_threshold, float* base_out, int64_t* ids_out, float* logit_out,
                                 int32_t* pass_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_reqs < 1 || num_reqs > 16 || B < 1 || B > (1 << 20)) return DSPARK_ERR_SHAPE;
  const int rows = num_reqs * B;
  dspark_status st = gemv_checks(W_lm, V, d, H, rows, base_out);
  if (st == DSPARK_OK)
    st = markov_checks(base_out, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, workspace, workspace_bytes);
  if (st == DSPARK_OK && probe_w) st = probe_checks(H, rows, d, probe_w, logit_out, pass_out);
  if (st != DSPARK_OK) return st;
  const size_t split = dspark::gemv_split_workspace_bytes(V, d, rows);
  const size_t split_at = round_split_offset(dspark::markov_workspace_bytes(num_reqs, k, V));
  if (split > 0 && workspace_bytes < split_at + split) return DSPARK_ERR_WORKSPACE;
  if (split > 0 && !aligned(workspace, 256)) return DSPARK_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      split > 0 ? dspark::launch_gemv_split(W_lm, V, d, H, rows, base_out, static_cast<unsigned char*>(workspace) + split_at,
                                            s, nullptr, dspark::markov_lm_counter(workspace))
                : dspark::launch_gemv_sched(W_lm, V, d, H, rows, base_out, dspark::markov_lm_counter(workspace), s);
  if (e != hipSuccess) return DSPARK_ERR_HIP;
  const dspark::ProbeArgs pa{H, rows, d, probe_w, probe_bias, probe_threshold, logit_out, pass_out};
  uint32_t* ticks = split > 0 ? reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(workspace) + split_at) : nullptr;
  return from_hip(dspark::launch_markov(base_out, num_reqs, B, V, w1, w2, r, d2t, prev0, k, ids_out, workspace,
                                        probe_w ? &pa : nullptr, s, ticks, split > 0 ? dspark::gemv_split_tick_words(V) : 0));
}

dspark_status dspark_markov_sample_q8(const float* base, int num_reqs, int B, int V, const int8_t* w1q,
                                      const uint16_t* w1d, const int8_t* w2q, const uint16_t* w2d, int r,
                                      const int64_t* d2t, const int64_t* prev0, int k, int64_t* ids_out,
                                      void* workspace, size_t workspace_bytes, const float* probe_x, int probe_M,
                                      int probe_D, const uint16_t* probe_w, float probe_bias, float probe_threshold,
                                      float* logit_out, int32_t* pass_out, void* stream) {
  dspark_status st = markov_q8_checks(base, num_reqs, B, V, w1q, w1d, w2q, w2d, r, d2t, prev0, k, ids_out, workspace,
                                      workspace_bytes);
  if (st == DSPARK_OK && probe_x) st = probe_checks(probe_x, probe_M, probe_D, probe_w, logit_out, pass_out);
  if (st != DSPARK_OK) return st;
  const dspark::ProbeArgs pa{probe_x, probe_M, probe_D, probe_w, probe_bias, probe_threshold, logit_out, pass_out};
  return from_hip(dspark::launch_markov_q8(base, num_reqs, B, V, w1q, w1d, w2q, w2d, r, d2t, prev0, k, ids_out,
                                           workspace, probe_x ? &pa : nullptr, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_draft_round_q8(const int8_t* Wq_lm, const uint16_t* Wd_lm, int V, int d, const float* H,
                                    int num_reqs, int B, const int8_t* w1q, const uint16_t* w1d, const int8_t* w2q,
                                    const uint16_t* w2d, int r, const int64_t* d2t, const int64_t* prev0, int k,
                                    const uint16_t* probe_w, float probe_bias, float probe_threshold, float* base_out,
                                    int64_t* ids_out, float* logit_out, int32_t* pass_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return dspark_draft_round_q8_ld(Wq_lm, Wd_lm, d / 32, V, d, H, num_reqs, B, w1q, w1d, w2q, w2d, r, d2t, prev0, k,
                                  probe_w, probe_bias, probe_threshold, base_out, ids_out, logit_out, pass_out,
                                  workspace, workspace_bytes, stream);
}

dspark_status dspark_draft_round_q8_ld(const int8_t* Wq_lm, const uint16_t* Wd_lm, int ldd_lm, int V, int d,
                                       const float* H, int num_reqs, int B, const int8_t* w1q, const uint16_t* w1d,
                                       const int8_t* w2q, const uint16_t* w2d, int r, const int64_t* d2t,
                                       const int64_t* prev0, int k, const uint16_t* probe_w, float probe_bias,
                                       float probe_threshold, float* base_out, int64_t* ids_out, float* logit_out,
                                       int32_t* pass_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_reqs < 1 || num_reqs > 16 || B < 1 || B > (1 << 20)) return DSPARK_ERR_SHAPE;
  const int rows = num_reqs * B;
  dspark_status st = gemv_q8_checks(Wq_lm, Wd_lm, V, d, H, rows, base_out);
  if (st == DSPARK_OK) st = q8_ldd_check(ldd_lm, d);
  if (st == DSPARK_OK)
    st = markov_q8_checks(base_out, num_reqs, B, V, w1q, w1d, w2q, w2d, r, d2t, prev0, k, ids_out, workspace,
                          workspace_bytes);
  if (st == DSPARK_OK && probe_w) st = probe_checks(H, rows, d, probe_w, logit_out, pass_out);
  if (st != DSPARK_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dspark::launch_gemv_q8(Wq_lm, Wd_lm, V, d, H, rows, base_out, s, ldd_lm) != hipSuccess) return DSPARK_ERR_HIP;
  const dspark::ProbeArgs pa{H, rows, d, probe_w, probe_bias, probe_threshold, logit_out, pass_out};
  return from_hip(dspark::launch_markov_q8(base_out, num_reqs, B, V, w1q, w1d, w2q, w2d, r, d2t, prev0, k, ids_out,
                                           workspace, probe_w ? &pa : nullptr, s));
}

dspark_status dspark_rmsnorm(const float* x, int M, int D, const uint16_t* gamma, float eps, float* y,
                             void* stream) {
  if (!x || !gamma || !y) return DSPARK_ERR_NULL;
  if (M < 1 || D < 1 || !(eps >= 0.f)) return DSPARK_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(gamma, 2) || !aligned(y, 4)) return DSPARK_ERR_ALIGN;
  return from_hip(dspark::launch_rmsnorm(x, M, D, gamma, eps, y, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_silu_gate(const float* gu, int M, int F, float* a, void* stream) {
  if (!gu || !a) return DSPARK_ERR_NULL;
  if (M < 1 || F < 1) return DSPARK_ERR_SHAPE;
  if (!aligned(gu, 4) || !aligned(a, 4)) return DSPARK_ERR_ALIGN;
  return from_hip(dspark::launch_silu_gate(gu, M, F, a, static_cast<hipStream_t>(stream)));
}

dspark_status dspark_proj_smallm_add(const uint16_t* W, int N, int K, const float* X, int M, const float* residual,
                                     float* Y, void* stream) {
  dspark_status st = gemv_checks(W, N, K, X, M, Y);
  if (st == DSPARK_OK && !residual) st = DSPARK_ERR_NULL;
  if (st == DSPARK_OK && !aligned(residual, 4)) st = DSPARK_ERR_ALIGN;
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_gemv(W, N, K, X, M, Y, static_cast<hipStream_t>(stream), residual));
}

int dspark_proj_smallm_norm_fits(int N, int K, int M) {
  return N >= 2 && K >= 8 && (K % 8) == 0 && M >= 1 && dspark::gemv_norm_fits(N, K, M) ? 1 : 0;
}

dspark_status dspark_proj_smallm_norm(const uint16_t* W, int N, int K, const float* X, int M, const uint16_t* gamma,
                                      float eps, float* Y, void* stream) {
  dspark_status st = gemv_checks(W, N, K, X, M, Y);
  if (st == DSPARK_OK && !gamma) st = DSPARK_ERR_NULL;
  if (st == DSPARK_OK && (!(eps >= 0.f) || !dspark_proj_smallm_norm_fits(N, K, M))) st = DSPARK_ERR_SHAPE;
  if (st == DSPARK_OK && !aligned(gamma, 16)) st = DSPARK_ERR_ALIGN;
  if (st != DSPARK_OK) return st;
  return from_hip(dspark::launch_gemv_norm(W, N, K, X, M, gamma, eps, Y, static_cast<hipStream_t>(stream)));
}

size_t dspark_attention_workspace_bytes(int num_reqs, int B, int H, int Dh, int Lmax) {
  if (!dspark::attention_shape_fits(num_reqs, B, H, Dh, Lmax)) return 0;
  return dspark::attention_workspace_bytes(num_reqs, B, H, Dh, Lmax);
}

dspark_status dspark_attention_ragged(const float* q, const float* k, const float* v, int ld, int R, int B, int H,
                                      int Dh, const uint16_t* k_ctx, const uint16_t* v_ctx, int Lmax,
                                      const int32_t* ctx_len, int block_causal, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !ctx_len || !out || (Lmax > 0 && (!k_ctx || !v_ctx))) return DSPARK_ERR_NULL;
  if (!dspark::attention_shape_fits(R, B, H, Dh, Lmax) || ld < H * Dh || (ld % 4) != 0) return DSPARK_ERR_SHAPE;
  if (!workspace || workspace_bytes < dspark::attention_workspace_bytes(R, B, H, Dh, Lmax)) return DSPARK_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4) || !aligned(ctx_len, 4) ||
      !aligned(workspace, 16) || (k_ctx && !aligned(k_ctx, 16)) || (v_ctx && !aligned(v_ctx, 16)))
    return DSPARK_ERR_ALIGN;
  return from_hip(dspark::launch_attention(q, k, v, ld, R, B, H, Dh, k_ctx, v_ctx, Lmax, ctx_len, block_causal ? 1 : 0,
                                           out, static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

// The draft block's intermediate buffers, carved out of the caller's
// workspace at 256-byte boundaries.
struct BlockLayout {
  size_t x, qkv, attn, h2, gu, act, attn_ws, total;
};

static BlockLayout block_layout(int R, int B, int H, int Dh, int d, int F, int Lmax) {
  const size_t M = static_cast<size_t>(R) * B, HD = static_cast<size_t>(H) * Dh;
  auto up = [](size_t n) { return (n + 255) & ~static_cast<size_t>(255); };
  BlockLayout l{};
  size_t off = 0;
  l.x = off; off += up(M * d * 4);
  l.qkv = off; off += up(M * 3 * HD * 4);
  l.attn = off; off += up(M * HD * 4);
  l.h2 = off; off += up(M * d * 4);
  l.gu = off; off += up(M * 2 * static_cast<size_t>(F) * 4);
  l.act = off; off += up(M * static_cast<size_t>(F) * 4);
  l.attn_ws = off; off += up(dspark::attention_workspace_bytes(R, B, H, Dh, Lmax));
  l.total = off;
  return l;
}

static bool block_shape_fits(int R, int B, int H, int Dh, int d, int F, int Lmax) {
  if (R < 1 || d < 8 || (d % 8) != 0 || F < 8 || (F % 8) != 0) return false;
  if (!dspark::attention_shape_fits(R, B, H, Dh, Lmax)) return false;
  const long long M = static_cast<long long>(R) * B, HD = static_cast<long long>(H) * Dh;
  if (M > (1 << 20) || 3 * HD > (1LL << 30) || 2LL * F > (1LL << 30)) return false;
  return dspark::gemv_shape_fits(static_cast<int>(3 * HD), d, static_cast<int>(M)) &&
         dspark::gemv_shape_fits(d, static_cast<int>(HD), static_cast<int>(M)) &&
         dspark::gemv_shape_fits(2 * F, d, static_cast<int>(M)) && dspark::gemv_shape_fits(d, F, static_cast<int>(M));
}

size_t dspark_draft_block_workspace_bytes(int num_reqs, int B, int H, int Dh, int d, int F, int Lmax) {
  if (!block_shape_fits(num_reqs, B, H, Dh, d, F, Lmax)) return 0;
  return block_layout(num_reqs, B, H, Dh, d, F, Lmax).total;
}

dspark_status dspark_draft_block(const uint16_t* w_qkv, const uint16_t* w_o, const uint16_t* w_gate_up,
                                 const uint16_t* w_down, const uint16_t* ln1, const uint16_t* ln2, int d, int F,
                                 int H, int Dh, int num_reqs, int B, const float* h_in, float* h_out,
                                 const uint16_t* k_ctx, const uint16_t* v_ctx, int Lmax, const int32_t* ctx_len,
                                 float eps, int block_causal, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!w_qkv || !w_o || !w_gate_up || !w_down || !ln1 || !ln2 || !h_in || !h_out || !ctx_len ||
      (Lmax > 0 && (!k_ctx || !v_ctx)))
    return DSPARK_ERR_NULL;
  if (!block_shape_fits(num_reqs, B, H, Dh, d, F, Lmax) || !(eps >= 0.f)) return DSPARK_ERR_SHAPE;
  const BlockLayout l = block_layout(num_reqs, B, H, Dh, d, F, Lmax);
  if (!workspace || workspace_bytes < l.total) return DSPARK_ERR_WORKSPACE;
  if (!aligned(w_qkv, 16) || !aligned(w_o, 16) || !aligned(w_gate_up, 16) || !aligned(w_down, 16) ||
      !aligned(ln1, 2) || !aligned(ln2, 2) || !aligned(h_in, 16) || !aligned(h_out, 16) || !aligned(ctx_len, 4) ||
      !aligned(workspace, 256) || (k_ctx && !aligned(k_ctx, 16)) || (v_ctx && !aligned(v_ctx, 16)))
    return DSPARK_ERR_ALIGN;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned char* base = static_cast<unsigned char*>(workspace);
  float* x = reinterpret_cast<float*>(base + l.x);
  float* qkv = reinterpret_cast<float*>(base + l.qkv);
  float* attn = reinterpret_cast<float*>(base + l.attn);
  float* h2 = reinterpret_cast<float*>(base + l.h2);
  float* gu = reinterpret_cast<float*>(base + l.gu);
  float* act = reinterpret_cast<float*>(base + l.act);
  float* aws = reinterpret_cast<float*>(base + l.attn_ws);
  const int M = num_reqs * B, HD = H * Dh;
  // Each norm runs inside the projection it feeds where that projection's
  // shape allows (dspark_proj_smallm_norm), else as its own launch.
  const bool fuse1 = dspark_proj_smallm_norm_fits(3 * HD, d, M) && aligned(ln1, 16);
  const bool fuse2 = dspark_proj_smallm_norm_fits(2 * F, d, M) && aligned(ln2, 16);
  hipError_t e = hipSuccess;
  if (fuse1) {
    e = dspark::launch_gemv_norm(w_qkv, 3 * HD, d, h_in, M, ln1, eps, qkv, st);
  } else {
    e = dspark::launch_rmsnorm(h_in, M, d, ln1, eps, x, st);
    if (e == hipSuccess) e = dspark::launch_gemv(w_qkv, 3 * HD, d, x, M, qkv, st);
  }
  if (e == hipSuccess)
    e = dspark::launch_attention(qkv, qkv + HD, qkv + 2 * HD, 3 * HD, num_reqs, B, H, Dh, k_ctx, v_ctx, Lmax, ctx_len,
                                 block_causal ? 1 : 0, attn, aws, st);
  if (e == hipSuccess) e = dspark::launch_gemv(w_o, d, HD, attn, M, h2, st, h_in);
  if (e == hipSuccess) {
    if (fuse2) {
      e = dspark::launch_gemv_gated_norm(w_gate_up, F, d, h2, M, ln2, eps, act, st);
    } else {
      e = dspark::launch_rmsnorm(h2, M, d, ln2, eps, x, st);
      if (e == hipSuccess) e = dspark::launch_gemv_gated(w_gate_up, F, d, x, M, act, gu, st);
    }
  }
  if (e == hipSuccess) e = dspark::launch_gemv(w_down, d, F, act, M, h_out, st, h2);
  return from_hip(e);
}

}  // extern "C"
