// csa_api.hip -- the C ABI of libcsa.so (declared in include/csa.h):
// argument validation, the gfx950 check, workspace carving and the order of
// the stage launches.  No device memory is allocated here.
#include <atomic>
#include <cstring>

#include "../../include/csa.h"
#include "csa_internal.hpp"

namespace {

using namespace csa;

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Workspace layout for (max rows per session, sessions):
//   [scores: sessions x rows_cap fp32][attention partials: sessions x kAttnPartFloats]
struct Layout {
  size_t rows_cap;  // floats per session in the score area
  size_t part_off;
  size_t total;
};

Layout make_layout(int64_t max_rows, int n_sessions) {
  Layout L;
  L.rows_cap = align_up((size_t)max_rows * sizeof(float)) / sizeof(float);
  L.part_off = align_up((size_t)n_sessions * L.rows_cap * sizeof(float));
  L.total = L.part_off + align_up((size_t)n_sessions * kAttnPartFloats * sizeof(float));
  return L;
}

std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CSA_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return CSA_EUNSUPPORTED;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return CSA_EDEVICE;
    st = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? CSA_OK : CSA_EUNSUPPORTED;
}

int status_of(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_EDEVICE; }

bool rows_ok(int64_t n) { return n >= 0 && n <= CSA_MAX_ROWS; }
bool heads_ok(int h) { return h >= 1 && h <= CSA_MAX_HEADS; }

int check_ws(const void *ws, size_t ws_bytes, int64_t max_rows, int n_sessions, Layout *L) {
  *L = make_layout(max_rows, n_sessions);
  if (ws == nullptr || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < L->total) return CSA_EWORKSPACE;
  return CSA_OK;
}

}  // namespace

extern "C" {

uint32_t csa_abi_version(void) { return CSA_ABI_VERSION; }

const char *csa_strerror(int status) {
  switch (status) {
    case CSA_OK: return "success";
    case CSA_EINVAL: return "invalid argument";
    case CSA_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case CSA_EDEVICE: return "HIP runtime error";
    case CSA_EUNSUPPORTED: return "device is not gfx950";
    default: return "unknown status";
  }
}

size_t csa_workspace_bytes(int64_t max_rows_per_session, int n_sessions) {
  if (!rows_ok(max_rows_per_session) || n_sessions < 1 || n_sessions > CSA_MAX_SESSIONS) return 0;
  return make_layout(max_rows_per_session, n_sessions).total;
}

int csa_dequant_idx(const uint8_t *idx_rows, int64_t n_rows, float *out, void *hip_stream) {
  if (!rows_ok(n_rows) || (n_rows > 0 && (!idx_rows || !out))) return CSA_EINVAL;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  return status_of(launch_dequant_idx(idx_rows, n_rows, out, (hipStream_t)hip_stream));
}

int csa_dequant_kv(const uint8_t *kv_rows, int64_t n_rows, float *out, void *hip_stream) {
  if (!rows_ok(n_rows) || (n_rows > 0 && (!kv_rows || !out))) return CSA_EINVAL;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  return status_of(launch_dequant_kv(kv_rows, n_rows, out, (hipStream_t)hip_stream));
}

int csa_score(const uint8_t *idx_rows, int64_t n_rows, const float *q_idx, const float *w_idx,
              int n_idx_heads, float *scores, void *hip_stream) {
  if (!rows_ok(n_rows) || !heads_ok(n_idx_heads) || !q_idx || !w_idx) return CSA_EINVAL;
  if (n_rows > 0 && (!idx_rows || !scores)) return CSA_EINVAL;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  ScoreSession s{idx_rows, q_idx, w_idx, scores, n_rows};
  return status_of(launch_score(&s, 1, n_idx_heads, n_rows, (hipStream_t)hip_stream));
}

int csa_topk(const float *scores, int64_t n_rows, int k, int32_t *sel_idx, float *sel_score,
             void *ws, size_t ws_bytes, void *hip_stream) {
  if (!rows_ok(n_rows) || k < 1 || k > CSA_TOPK || !sel_idx) return CSA_EINVAL;
  if (n_rows > 0 && !scores) return CSA_EINVAL;
  Layout L;
  int rc = check_ws(ws, ws_bytes, n_rows, 1, &L);
  if (rc != CSA_OK) return rc;
  rc = check_device();
  if (rc != CSA_OK) return rc;
  SelectSession s{scores, sel_idx, sel_score, n_rows};
  return status_of(launch_select(&s, 1, k, (hipStream_t)hip_stream));
}

int csa_sparse_attn(const uint8_t *kv_rows, int64_t n_rows, const int32_t *sel_idx, int n_sel,
                    const float *q_attn, int n_heads, float softmax_scale, float *out, float *lse,
                    void *ws, size_t ws_bytes, void *hip_stream) {
  if (!rows_ok(n_rows) || n_sel < 0 || n_sel > CSA_TOPK || !heads_ok(n_heads) || !q_attn || !out)
    return CSA_EINVAL;
  if ((n_sel > 0 && !sel_idx) || (n_rows > 0 && !kv_rows)) return CSA_EINVAL;
  Layout L;
  int rc = check_ws(ws, ws_bytes, 0, 1, &L);
  if (rc != CSA_OK) return rc;
  rc = check_device();
  if (rc != CSA_OK) return rc;
  AttnSession s{kv_rows, sel_idx, q_attn, out, lse, n_rows, n_sel};
  float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + L.part_off);
  return status_of(launch_attention(&s, 1, n_heads, softmax_scale, part, (hipStream_t)hip_stream));
}

int csa_decode_step(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                    float softmax_scale, void *ws, size_t ws_bytes, void *hip_stream) {
  if (!sessions || n_sessions < 1 || n_sessions > CSA_MAX_SESSIONS || !heads_ok(n_idx_heads) ||
      !heads_ok(n_heads))
    return CSA_EINVAL;
  int64_t max_rows = 0;
  for (int i = 0; i < n_sessions; ++i) {
    const csa_session &s = sessions[i];
    if (!rows_ok(s.n_rows) || !s.q_idx || !s.w_idx || !s.q_attn || !s.sel_idx || !s.out) return CSA_EINVAL;
    if (s.n_rows > 0 && (!s.idx_rows || !s.kv_rows)) return CSA_EINVAL;
    if (s.n_rows > max_rows) max_rows = s.n_rows;
  }
  Layout L;
  int rc = check_ws(ws, ws_bytes, max_rows, n_sessions, &L);
  if (rc != CSA_OK) return rc;
  rc = check_device();
  if (rc != CSA_OK) return rc;
  hipStream_t st = (hipStream_t)hip_stream;
  float *score_base = reinterpret_cast<float *>(ws);
  float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + L.part_off);

  ScoreSession sc[CSA_MAX_SESSIONS];
  SelectSession se[CSA_MAX_SESSIONS];
  AttnSession at[CSA_MAX_SESSIONS];
  for (int i = 0; i < n_sessions; ++i) {
    const csa_session &s = sessions[i];
    float *scores = score_base + (size_t)i * L.rows_cap;
    const int32_t n_sel = (int32_t)(s.n_rows < CSA_TOPK ? s.n_rows : CSA_TOPK);
    sc[i] = ScoreSession{s.idx_rows, s.q_idx, s.w_idx, scores, s.n_rows};
    se[i] = SelectSession{scores, s.sel_idx, s.sel_score, s.n_rows};
    at[i] = AttnSession{s.kv_rows, s.sel_idx, s.q_attn, s.out, s.lse, s.n_rows, n_sel};
  }
  hipError_t e = launch_score(sc, n_sessions, n_idx_heads, max_rows, st);
  if (e == hipSuccess) e = launch_select(se, n_sessions, CSA_TOPK, st);
  if (e == hipSuccess) e = launch_attention(at, n_sessions, n_heads, softmax_scale, part, st);
  return status_of(e);
}

}  // extern "C"
