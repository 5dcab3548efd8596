// csa_api.hip -- the C ABI of libcsa.so (declared in include/csa.h):
// argument validation, the gfx950 check, workspace carving and the order of
// the stage launches.  No device memory is allocated here.
#include <atomic>
#include <cstring>

#include "../../include/csa.h"
#include "csa_attn.hpp"
#include "csa_internal.hpp"
#include "csa_score.hpp"

namespace {

using namespace csa;

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Workspace layout for (max rows per session, sessions); sized for the
// smallest tile so that it grows monotonically with max_rows:
//   [attention query split][head keys][head lower-bound keys][tile next keys]
//   [items][item counts][attention partials][attention (m, l)]
//   [quantized indexer query, fp32]
// The items hold the exact keys of the rows that can reach the top-k: the
// head slots plus, for the rare tiles whose other rows may also reach it,
// every row of those tiles (at most every row of the session).
struct Layout {
  int64_t tiles_cap;  // tiles per session at the smallest tile size
  int64_t heads_cap;  // head slots per session
  int64_t items_cap;  // items per session
  size_t attn_q_off, hkey_off, hlow_off, hnext_off, items_off, count_off, part_off, ml_off, qhat_off, total;
};

Layout make_layout(int64_t max_rows, int n_sessions) {
  Layout L;
  L.tiles_cap = (max_rows + kMinTileRows - 1) / kMinTileRows;
  L.heads_cap = L.tiles_cap * kMaxTileHeads;
  L.items_cap = L.heads_cap + ((max_rows + 63) & ~(int64_t)63);
  const size_t ns = (size_t)n_sessions;
  L.attn_q_off = 0;
  L.hkey_off = L.attn_q_off + align_up(ns * kAttnQBytes);
  L.hlow_off = L.hkey_off + align_up(ns * (size_t)L.heads_cap * sizeof(uint64_t));
  L.hnext_off = L.hlow_off + align_up(ns * (size_t)L.heads_cap * sizeof(uint64_t));
  L.items_off = L.hnext_off + align_up(ns * (size_t)(L.tiles_cap > 0 ? L.tiles_cap : 1) * sizeof(uint64_t));
  L.count_off = L.items_off + align_up(ns * (size_t)(L.items_cap > 0 ? L.items_cap : 1) * sizeof(uint64_t));
  L.part_off = L.count_off + align_up(ns * sizeof(uint32_t));
  L.ml_off = L.part_off + align_up(ns * kAttnPartFloats * sizeof(float));
  L.qhat_off = L.ml_off + align_up(ns * kAttnMlFloats * sizeof(float));
  L.total = L.qhat_off + align_up(ns * (size_t)CSA_MAX_HEADS * 128 * sizeof(float));
  return L;
}

// Tile rows: as large as possible (fewer heads to merge) while the launch
// keeps at least ~512 workgroups (two per compute unit).  More, smaller
// tiles pay the per-tile start (query split, first loads) and heads twice
// per slot, which costs more than they win back by balancing.
int choose_tile_rows(int64_t total_rows) {
  int T = kMinTileRows;
  while (T < kMaxTileRows && total_rows / (2 * (int64_t)T) >= 512) T *= 2;
  return T;
}

// Largest selection grid that also runs the attention (about one
// workgroup per compute unit).
constexpr int kFusedAttnMaxWorkgroups = 256;

// log2 of the row groups per session of the attention when it runs as its
// own launch: about 512 workgroups (4 head groups each) over all sessions.
int separate_groups_lg(int n_sessions) {
  int lg = kAttnGroupsLg;
  while (lg > 0 && n_sessions * (kAttnHeadGroups << lg) > 512) --lg;
  return lg;
}

// Workgroups per session of the selection kernel: about one per compute
// unit in total.
int choose_slices(int n_sessions) {
  int s = 256 / n_sessions;
  return s < 4 ? 4 : (s > 32 ? 32 : s);
}

std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// Workspace of csa_decode_step_noalloc: one array per device, held from the
// module's load until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies get the device
// address that hipGetSymbolAddress returns for the current device, kept in
// g_scratch_ptr (each device holds its own copy at its own address).
__device__ __align__(256) uint8_t scratch[CSA_SCRATCH_BYTES];
std::atomic<void *> g_scratch_ptr[kMaxDevices];

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

// Device address of this device's `scratch`, looked up once per device (with
// that device current); null on a HIP error.
void *scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

bool rows_ok(int64_t n) { return n >= 0 && n <= CSA_MAX_ROWS; }
bool format_ok(int f) { return f == CSA_QUERY_FP32 || f == CSA_QUERY_MXFP4; }
bool heads_ok(int h) { return h >= 1 && h <= CSA_MAX_HEADS; }
// The scorer streams indexer rows with 16-byte loads.
bool idx_aligned(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_ws(const void *ws, size_t ws_bytes, int64_t max_rows, int n_sessions, Layout *L) {
  *L = make_layout(max_rows, n_sessions);
  if (ws == nullptr || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < L->total) return CSA_EWORKSPACE;
  return CSA_OK;
}

template <class T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

void fill_job(TileJob &job, const Layout &L, void *ws, int n_sessions) {
  job.n_sessions = n_sessions;
  job.hkey = at<uint64_t>(ws, L.hkey_off);
  job.hlow = at<uint64_t>(ws, L.hlow_off);
  job.hnext = at<uint64_t>(ws, L.hnext_off);
  job.heads_stride = L.heads_cap;
  job.tiles_stride = L.tiles_cap;
  job.bnd_up = job.bnd_lo = nullptr;
  job.query_format = kQueryFp32;
  job.qhat = nullptr;
  int64_t total = 0;
  for (int i = 0; i < n_sessions; ++i) total += job.n_rows[i];
  job.tile_rows = choose_tile_rows(total);
  for (int i = 0; i < n_sessions; ++i)
    job.hd[i] = heads_per_tile((job.n_rows[i] + job.tile_rows - 1) / job.tile_rows);
}

// Workgroups per session of the exact rescoring: about one per compute
// unit in total.
int refine_blocks(int n_sessions) {
  const int b = 256 / n_sessions;
  return b < 2 ? 2 : b;
}

// The exact rescoring that follows a tile launch.
void fill_refine(RefineJob &rj, const TileJob &job, const Layout &L, void *ws, int k) {
  rj.mode = job.mode == TileJob::kArray ? RefineJob::kArray : RefineJob::kDecode;
  rj.n_sessions = job.n_sessions;
  rj.n_idx_heads = job.n_idx_heads;
  rj.tile_rows = job.tile_rows;
  rj.k = k;
  rj.blocks = refine_blocks(job.n_sessions);
  rj.attn_q = nullptr;
  rj.n_attn_heads = 0;
  for (int i = 0; i < job.n_sessions; ++i) {
    rj.q_attn[i] = nullptr;
    rj.idx_rows[i] = job.idx_rows[i];
    rj.q[i] = job.q[i];
    rj.w[i] = job.w[i];
    rj.scores[i] = const_cast<float *>(job.scores_in[i]);
    rj.n_rows[i] = job.n_rows[i];
    rj.hd[i] = job.hd[i];
  }
  rj.hkey = job.hkey;
  rj.hlow = job.hlow;
  rj.hnext = job.hnext;
  rj.items = at<uint64_t>(ws, L.items_off);
  rj.count = at<uint32_t>(ws, L.count_off);
  rj.heads_stride = L.heads_cap;
  rj.tiles_stride = L.tiles_cap;
  rj.items_stride = L.items_cap;
}

// The selection that follows the rescoring.
void fill_select(SelectJob &sj, const TileJob &job, const RefineJob &rj, int k) {
  sj.n_sessions = job.n_sessions;
  sj.k = k;
  sj.slices = choose_slices(job.n_sessions);
  sj.array_scores = job.mode == TileJob::kArray;
  for (int i = 0; i < job.n_sessions; ++i) {
    sj.scores[i] = job.scores_in[i];
    sj.n_rows[i] = job.n_rows[i];
    sj.kv_rows[i] = nullptr;
  }
  sj.items = rj.items;
  sj.count = rj.count;
  sj.items_stride = rj.items_stride;
  sj.attn_q = nullptr;
  sj.attn_part = nullptr;
  sj.attn_ml = nullptr;
  sj.n_heads = 0;
  sj.softmax_scale = 0.0f;
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
              int n_idx_heads, float *scores, void *ws, size_t ws_bytes, void *hip_stream) {
  if (!rows_ok(n_rows) || !heads_ok(n_idx_heads) || !q_idx || !w_idx || !idx_aligned(q_idx)) return CSA_EINVAL;
  if (n_rows > 0 && (!idx_rows || !scores || !idx_aligned(idx_rows))) return CSA_EINVAL;
  Layout L;
  int rc = check_ws(ws, ws_bytes, n_rows, 1, &L);
  if (rc != CSA_OK) return rc;
  rc = check_device();
  if (rc != CSA_OK) return rc;
  if (n_rows == 0) return CSA_OK;
  RefineJob rj{};
  rj.mode = RefineJob::kAll;
  rj.n_sessions = 1;
  rj.n_idx_heads = n_idx_heads;
  rj.tile_rows = kMinTileRows;
  rj.k = CSA_TOPK;
  rj.blocks = 1024;  // four workgroups per compute unit: the fp64 arithmetic bounds it
  rj.idx_rows[0] = idx_rows;
  rj.q[0] = q_idx;
  rj.w[0] = w_idx;
  rj.scores[0] = scores;
  rj.n_rows[0] = n_rows;
  rj.hd[0] = kMinTileHeads;
  return status_of(launch_refine(rj, (hipStream_t)hip_stream));
}

int csa_score_bounds(const uint8_t *idx_rows, int64_t n_rows, const float *q_idx, const float *w_idx,
                     int n_idx_heads, int query_format, float *upper, float *lower, void *ws, size_t ws_bytes,
                     void *hip_stream) {
  if (!rows_ok(n_rows) || !heads_ok(n_idx_heads) || !q_idx || !w_idx || !idx_aligned(q_idx) ||
      !format_ok(query_format))
    return CSA_EINVAL;
  if (n_rows > 0 && (!idx_rows || !upper || !lower || !idx_aligned(idx_rows))) return CSA_EINVAL;
  Layout L;
  int rc = check_ws(ws, ws_bytes, n_rows, 1, &L);
  if (rc != CSA_OK) return rc;
  rc = check_device();
  if (rc != CSA_OK) return rc;
  TileJob job;
  job.mode = TileJob::kBounds;
  job.n_idx_heads = n_idx_heads;
  job.idx_rows[0] = idx_rows;
  job.scores_in[0] = nullptr;
  job.n_rows[0] = n_rows;
  job.q[0] = q_idx;
  job.w[0] = w_idx;
  fill_job(job, L, ws, 1);
  job.bnd_up = upper;
  job.bnd_lo = lower;
  job.query_format = query_format == CSA_QUERY_MXFP4 ? kQueryMxfp4 : kQueryFp32;
  if (n_rows == 0) return CSA_OK;
  return status_of(launch_tiles(job, (hipStream_t)hip_stream));
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
  hipStream_t st = (hipStream_t)hip_stream;
  TileJob job;
  job.mode = TileJob::kArray;
  job.n_idx_heads = 1;
  job.idx_rows[0] = nullptr;
  job.scores_in[0] = scores;
  job.n_rows[0] = n_rows;
  job.q[0] = job.w[0] = nullptr;
  fill_job(job, L, ws, 1);
  RefineJob rj;
  fill_refine(rj, job, L, ws, k);
  SelectJob sj;
  fill_select(sj, job, rj, k);
  sj.sel_idx[0] = sel_idx;
  sj.sel_score[0] = sel_score;
  hipError_t e = launch_tiles(job, st);
  if (e == hipSuccess && n_rows > 0) e = launch_refine(rj, st);
  if (e == hipSuccess) e = launch_select(sj, st);
  return status_of(e);
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
  hipStream_t st = (hipStream_t)hip_stream;
  uint4 *aq = at<uint4>(ws, L.attn_q_off);
  float *part = at<float>(ws, L.part_off), *ml = at<float>(ws, L.ml_off);
  hipError_t e = launch_attn_q_split(&q_attn, 1, n_heads, aq, st);
  if (e == hipSuccess) e = launch_attn_rows(&s, 1, n_heads, softmax_scale, aq, part, ml, kAttnGroupsLg, st);
  if (e == hipSuccess) e = launch_attn_combine(&s, 1, n_heads, part, ml, kAttnGroupsLg, st);
  return status_of(e);
}

int csa_score_topk_multi(const uint8_t *idx_rows, int64_t n_rows, const float *q_idx, const float *w_idx,
                         int n_tokens, int n_idx_heads, int k, int32_t *sel_idx, float *sel_score, void *ws,
                         size_t ws_bytes, void *hip_stream) {
  if (!rows_ok(n_rows) || n_tokens < 1 || n_tokens > CSA_MAX_SESSIONS || !heads_ok(n_idx_heads) || k < 1 ||
      k > CSA_TOPK || !q_idx || !w_idx || !sel_idx || !idx_aligned(q_idx))
    return CSA_EINVAL;
  if (n_rows > 0 && (!idx_rows || !idx_aligned(idx_rows))) return CSA_EINVAL;
  Layout L;
  int rc = check_ws(ws, ws_bytes, n_rows, n_tokens, &L);
  if (rc != CSA_OK) return rc;
  rc = check_device();
  if (rc != CSA_OK) return rc;
  hipStream_t st = (hipStream_t)hip_stream;
  // each token is a session over the same rows (the score kernel runs their
  // tiles side by side), selecting without attention
  TileJob job;
  job.mode = TileJob::kFilter;
  job.n_idx_heads = n_idx_heads;
  for (int t = 0; t < n_tokens; ++t) {
    job.idx_rows[t] = idx_rows;
    job.scores_in[t] = nullptr;
    job.n_rows[t] = n_rows;
    job.q[t] = q_idx + (size_t)t * n_idx_heads * CSA_IDX_DIM;
    job.w[t] = w_idx + (size_t)t * n_idx_heads;
  }
  fill_job(job, L, ws, n_tokens);
  RefineJob rj;
  fill_refine(rj, job, L, ws, k);
  const bool exact_all = n_rows <= (int64_t)2 * rj.blocks * kRefineWaves;
  if (exact_all) rj.mode = RefineJob::kKeysAll;
  SelectJob sj;
  fill_select(sj, job, rj, k);
  for (int t = 0; t < n_tokens; ++t) {
    sj.sel_idx[t] = sel_idx + (size_t)t * k;
    sj.sel_score[t] = sel_score ? sel_score + (size_t)t * k : nullptr;
  }
  hipError_t e = hipSuccess;
  if (!exact_all) e = launch_tiles(job, st);
  if (e == hipSuccess && n_rows > 0) e = launch_refine(rj, st);
  if (e == hipSuccess) e = launch_select(sj, st);
  return status_of(e);
}

int csa_pack_rows(const float *kv_vals, const float *idx_vals, int64_t n_rows, uint8_t *kv_rows, uint8_t *idx_rows,
                  void *hip_stream) {
  if (!rows_ok(n_rows) || (!kv_vals && !idx_vals)) return CSA_EINVAL;
  if (kv_vals && (!kv_rows || ((uintptr_t)kv_vals & 3u) != 0)) return CSA_EINVAL;
  if (idx_vals && (!idx_rows || ((uintptr_t)idx_vals & 7u) != 0)) return CSA_EINVAL;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  return status_of(launch_pack(kv_vals, idx_vals, n_rows, kv_rows, idx_rows, (hipStream_t)hip_stream));
}

int csa_lse_merge(const float *out_a, const float *lse_a, const float *out_b, const float *lse_b, int n_heads,
                  float *out, float *lse, void *hip_stream) {
  if (!heads_ok(n_heads) || !out_a || !lse_a || !out_b || !lse_b || !out || !lse) return CSA_EINVAL;
  if (lse == lse_a || lse == lse_b) return CSA_EINVAL;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  return status_of(launch_lse_merge(out_a, lse_a, out_b, lse_b, n_heads, out, lse, (hipStream_t)hip_stream));
}

// Workspace of csa_dense_attn: [attention query split][group partials][group (m, l)].
struct DenseLayout {
  size_t q_off, part_off, ml_off, total;
};
DenseLayout make_dense_layout(int64_t n_rows) {
  int per = 0, groups = 0;
  dense_grouping(n_rows, &per, &groups);
  DenseLayout L;
  L.q_off = 0;
  L.part_off = align_up(kAttnQBytes);
  L.ml_off = L.part_off + align_up((size_t)groups * CSA_MAX_HEADS * kKvDim * sizeof(float));
  L.total = L.ml_off + align_up((size_t)(groups > 0 ? groups : 1) * CSA_MAX_HEADS * 2 * sizeof(float));
  return L;
}

size_t csa_dense_workspace_bytes(int64_t n_rows) {
  if (n_rows < 0 || n_rows > CSA_DENSE_MAX_ROWS) return 0;
  return make_dense_layout(n_rows).total;
}

int csa_dense_attn(const uint8_t *kv_rows, int64_t n_rows, const float *q_attn, int n_heads, float softmax_scale,
                   float *out, float *lse, void *ws, size_t ws_bytes, void *hip_stream) {
  if (n_rows < 0 || n_rows > CSA_DENSE_MAX_ROWS || !heads_ok(n_heads) || !q_attn || !out) return CSA_EINVAL;
  if (n_rows > 0 && !kv_rows) return CSA_EINVAL;
  const DenseLayout L = make_dense_layout(n_rows);
  if (ws == nullptr || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < L.total) return CSA_EWORKSPACE;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  hipStream_t st = (hipStream_t)hip_stream;
  uint4 *aq = at<uint4>(ws, L.q_off);
  hipError_t e = launch_attn_q_split(&q_attn, 1, n_heads, aq, st);
  if (e == hipSuccess)
    e = launch_dense_attn(kv_rows, n_rows, aq, n_heads, softmax_scale, at<float>(ws, L.part_off), at<float>(ws, L.ml_off),
                          out, lse, st);
  return status_of(e);
}

static int decode_step_impl(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                            float softmax_scale, int query_format, void *ws, size_t ws_bytes, void *hip_stream,
                            void *const *events) {
  if (!sessions || n_sessions < 1 || n_sessions > CSA_MAX_SESSIONS || !heads_ok(n_idx_heads) ||
      !heads_ok(n_heads) || !format_ok(query_format))
    return CSA_EINVAL;
  int64_t max_rows = 0;
  for (int i = 0; i < n_sessions; ++i) {
    const csa_session &s = sessions[i];
    if (!rows_ok(s.n_rows) || !s.q_idx || !s.w_idx || !s.q_attn || !s.sel_idx || !s.out) return CSA_EINVAL;
    if (!idx_aligned(s.q_idx)) return CSA_EINVAL;
    if (s.n_rows > 0 && (!s.idx_rows || !s.kv_rows || !idx_aligned(s.idx_rows))) return CSA_EINVAL;
    if (s.n_rows > max_rows) max_rows = s.n_rows;
  }
  Layout L;
  int rc = check_ws(ws, ws_bytes, max_rows, n_sessions, &L);
  if (rc != CSA_OK) return rc;
  rc = check_device();
  if (rc != CSA_OK) return rc;
  hipStream_t st = (hipStream_t)hip_stream;

  TileJob job;
  job.mode = TileJob::kFilter;
  job.n_idx_heads = n_idx_heads;
  int32_t *sel[CSA_MAX_SESSIONS];
  float *sel_score[CSA_MAX_SESSIONS];
  AttnSession at_s[CSA_MAX_SESSIONS];
  for (int i = 0; i < n_sessions; ++i) {
    const csa_session &s = sessions[i];
    job.idx_rows[i] = s.idx_rows;
    job.scores_in[i] = nullptr;
    job.n_rows[i] = s.n_rows;
    job.q[i] = s.q_idx;
    job.w[i] = s.w_idx;
    sel[i] = s.sel_idx;
    sel_score[i] = s.sel_score;
    const int32_t n_sel = (int32_t)(s.n_rows < CSA_TOPK ? s.n_rows : CSA_TOPK);
    at_s[i] = AttnSession{s.kv_rows, s.sel_idx, s.q_attn, s.out, s.lse, s.n_rows, n_sel};
  }
  fill_job(job, L, ws, n_sessions);
  uint4 *aq = at<uint4>(ws, L.attn_q_off);
  float *part = at<float>(ws, L.part_off), *ml = at<float>(ws, L.ml_off);
  RefineJob rj;
  fill_refine(rj, job, L, ws, CSA_TOPK);
  if (query_format == CSA_QUERY_MXFP4) {
    // the score kernel quantizes the query and keeps it (fp32) for the
    // exact rescoring, which then scores with the quantized query
    job.query_format = kQueryMxfp4;
    job.qhat = at<float>(ws, L.qhat_off);
    for (int i = 0; i < n_sessions; ++i) rj.q[i] = job.qhat + (size_t)i * CSA_MAX_HEADS * 128;
  }
  // Short histories (at most two rows per rescoring wave in every session):
  // every row is scored exactly by the rescoring kernel and the score kernel
  // is skipped; the selection then takes the top-k of all rows' exact keys.
  // (The fp32 query only: the MXFP4 query is quantized by the score kernel.)
  bool exact_all = query_format == CSA_QUERY_FP32;
  for (int i = 0; i < n_sessions; ++i)
    exact_all = exact_all && sessions[i].n_rows <= (int64_t)2 * rj.blocks * kRefineWaves;
  if (exact_all) rj.mode = RefineJob::kKeysAll;
  rj.attn_q = aq;  // the attention query is split by the rescoring's workgroups
  rj.n_attn_heads = n_heads;
  for (int i = 0; i < n_sessions; ++i) rj.q_attn[i] = sessions[i].q_attn;
  SelectJob sj;
  fill_select(sj, job, rj, CSA_TOPK);
  // One session's selection workgroups also run its attention (one
  // workgroup per row group and head group).  With many sessions that grid
  // would take several rounds of the chip, so the selection runs alone and
  // the attention follows as its own launch (same partials, same bits).
  const bool fused_attn = n_sessions * kAttnSlices <= kFusedAttnMaxWorkgroups;
  // separate attention: the sessions supply the parallelism, so fewer row
  // groups (longer groups, smaller partials) per session
  const int groups_lg = fused_attn ? kAttnGroupsLg : separate_groups_lg(n_sessions);
  if (fused_attn) {
    sj.slices = kAttnSlices;
    sj.attn_q = aq;
    sj.attn_part = part;
    sj.attn_ml = ml;
    sj.n_heads = n_heads;
    sj.softmax_scale = softmax_scale;
  }
  for (int i = 0; i < n_sessions; ++i) {
    sj.sel_idx[i] = sel[i];
    sj.sel_score[i] = sel_score[i];
    sj.kv_rows[i] = sessions[i].kv_rows;
  }
  bool any_rows = false;
  for (int i = 0; i < n_sessions; ++i) any_rows = any_rows || sessions[i].n_rows > 0;
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord((hipEvent_t)events[i], st) : hipSuccess;
  };
  // the score kernel records stage 0's events at its own start and end
  hipError_t e = hipSuccess;
  if (exact_all) {
    e = mark(0);
    if (e == hipSuccess) e = mark(1);
  } else {
    e = launch_tiles(job, st, events ? (hipEvent_t)events[0] : nullptr, events ? (hipEvent_t)events[1] : nullptr);
  }
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess && any_rows) e = launch_refine(rj, st);
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess) e = mark(4);
  if (e == hipSuccess) e = launch_select(sj, st);
  if (e == hipSuccess && !fused_attn)
    e = launch_attn_rows(at_s, n_sessions, n_heads, softmax_scale, aq, part, ml, groups_lg, st);
  if (e == hipSuccess) e = mark(5);
  if (e == hipSuccess) e = mark(6);
  if (e == hipSuccess) e = launch_attn_combine(at_s, n_sessions, n_heads, part, ml, groups_lg, st);
  if (e == hipSuccess) e = mark(7);
  return status_of(e);
}

int csa_decode_step(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                    float softmax_scale, void *ws, size_t ws_bytes, void *hip_stream) {
  return decode_step_impl(sessions, n_sessions, n_idx_heads, n_heads, softmax_scale, CSA_QUERY_FP32, ws, ws_bytes,
                          hip_stream, nullptr);
}

int csa_decode_step_ex(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                       float softmax_scale, int query_format, void *ws, size_t ws_bytes, void *hip_stream,
                       void *const *events) {
  if (events)
    for (int i = 0; i < 2 * CSA_STAGES; ++i)
      if (!events[i]) return CSA_EINVAL;
  return decode_step_impl(sessions, n_sessions, n_idx_heads, n_heads, softmax_scale, query_format, ws, ws_bytes,
                          hip_stream, events);
}

int csa_quantize_query(const float *q_idx, int n_idx_heads, uint8_t *q_rows, void *hip_stream) {
  if (!heads_ok(n_idx_heads) || !q_idx || !q_rows || !idx_aligned(q_idx) || ((uintptr_t)q_rows & 3u) != 0)
    return CSA_EINVAL;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  return status_of(launch_quantize_query(q_idx, n_idx_heads, q_rows, (hipStream_t)hip_stream));
}

int csa_decode_step_noalloc(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                            float softmax_scale, void *hip_stream) {
  // the sizes are checked before the device is touched: a step whose
  // workspace exceeds the static array is rejected with nothing enqueued
  if (!sessions || n_sessions < 1 || n_sessions > CSA_MAX_SESSIONS) return CSA_EINVAL;
  int64_t max_rows = 0;
  for (int i = 0; i < n_sessions; ++i) {
    if (!rows_ok(sessions[i].n_rows)) return CSA_EINVAL;
    if (sessions[i].n_rows > max_rows) max_rows = sessions[i].n_rows;
  }
  if (make_layout(max_rows, n_sessions).total > (size_t)CSA_SCRATCH_BYTES) return CSA_EWORKSPACE;
  int rc = check_device();
  if (rc != CSA_OK) return rc;
  void *ws = scratch_ptr();
  if (ws == nullptr) return CSA_EDEVICE;
  return decode_step_impl(sessions, n_sessions, n_idx_heads, n_heads, softmax_scale, CSA_QUERY_FP32, ws,
                          CSA_SCRATCH_BYTES, hip_stream, nullptr);
}

int csa_decode_step_timed(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                          float softmax_scale, void *ws, size_t ws_bytes, void *hip_stream,
                          void *const *events) {
  if (!events) return CSA_EINVAL;
  for (int i = 0; i < 2 * CSA_STAGES; ++i)
    if (!events[i]) return CSA_EINVAL;
  return decode_step_impl(sessions, n_sessions, n_idx_heads, n_heads, softmax_scale, CSA_QUERY_FP32, ws, ws_bytes,
                          hip_stream, events);
}

}  // extern "C"
