// C ABI of the SparsePR call: argument validation, workspace carve-up, launch order.
// Declarations, layouts and error behaviour are documented in include/sparsepr.h.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "../../include/sparsepr.h"
#include "launch.h"
#include "plan_state.h"
#include "common.h"

namespace spr {
void launch_fill_i32(int* p, long long n, int v, hipStream_t s);
}

using spr::Bufs;
using spr::Dims;

constexpr int kTimingRing = 64;

struct sparsepr_plan_s {
  sparsepr_config cfg;
  Dims D;
  size_t ws_bytes;
  void* ws;
  int planned;  // 1 after sparsepr_plan / sparsepr_plan_from_labels on the bound workspace
  int timing;   // stage events enabled
  // ring of kTimingRing (begin, end) event pairs per stage; count = calls recorded since
  // the last sparsepr_stage_times (the ring keeps the most recent kTimingRing of them)
  hipEvent_t ev[SPARSEPR_NUM_STAGES][kTimingRing][2];
  int count[SPARSEPR_NUM_STAGES];
};

namespace {
// Stage timing guard: records the begin / end events of a stage when timing is on.
struct StageTimer {
  sparsepr_plan_s* p;
  int st;
  hipStream_t s;
  StageTimer(sparsepr_plan_s* p_, int st_, hipStream_t s_) : p(p_), st(st_), s(s_) {
    if (p->timing) (void)hipEventRecord(p->ev[st][p->count[st] % kTimingRing][0], s);
  }
  ~StageTimer() {
    if (p->timing) {
      (void)hipEventRecord(p->ev[st][p->count[st] % kTimingRing][1], s);
      ++p->count[st];
    }
  }
};
}  // namespace

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += sizeof(T) * (count ? count : 1);
    return p;
  }
};

Bufs carve(const Dims& D, void* base, size_t* total) {
  Carver c{(char*)base};
  Bufs B;
  const size_t BH = D.BH, N = D.N, d = D.d, C = D.C;
  const size_t esz = D.dtype == 1 ? 2 : 4;
  B.sampled = c.take<int>(BH * D.S);
  B.qs = c.take<float>(BH * D.S * d);
  B.metric = c.take<float>(BH * d * d);
  B.metric_h = c.take<spr::bf16>(BH * d * d);
  B.metric_l = c.take<spr::bf16>(BH * d * d);
  B.cent = c.take<float>(BH * C * d);
  B.cent_t = c.take<float>(BH * C * d);
  B.cnorm = c.take<float>(BH * C);
  B.cent_h = c.take<spr::bf16>(BH * C * d);
  B.cent_l = c.take<spr::bf16>(BH * C * d);
  B.cent_b = c.take<spr::bf16>(BH * C * 16);
  B.alpha = c.take<float>(BH * N);
  B.rowconst = c.take<float>(BH * N);
  B.rank = c.take<int>(BH * N);
  B.tab = c.take<int>(BH * C * D.nblk);
  B.lperm = c.take<int>(BH * N);
  B.ipart = c.take<double>(BH * D.nblk);
  B.init_k = c.take<int>(BH * D.Ck);
  B.init_q = c.take<int>(BH * D.Cq);
  B.lab = c.take<int>(BH * N);
  B.gstart = c.take<int>(BH * (C + 1));
  B.gcount = c.take<int>(BH * C);
  B.kst = c.take<spr::KmState>(BH);
  B.qst = c.take<spr::KmState>(BH);
  B.klab = c.take<int>(BH * N);
  B.kperm = c.take<int>(BH * N);
  B.koff = c.take<int>(BH * (D.Ck + 1));
  B.kcent = c.take<float>(BH * D.Ck * d);
  B.kcent_h = c.take<spr::bf16>(BH * D.Ck * d);
  B.kcent_l = c.take<spr::bf16>(BH * D.Ck * d);
  B.qcent = c.take<float>(BH * D.Cq * d);
  B.qlab = c.take<int>(BH * N);
  B.qperm = c.take<int>(BH * N);
  B.qoff = c.take<int>(BH * (D.Cq + 1));
  B.u = c.take<long long>(BH * D.Cq * D.Ck);
  B.sorted_b = c.take<int>(BH * D.Cq * D.Ck);
  B.cum = c.take<long long>(BH * D.Cq * D.Ck);
  B.ccost = c.take<long long>(BH * D.Cq * D.Ck);
  B.jsel = c.take<int>(BH * D.Cq);
  B.row_ptr = c.take<int>(BH * (D.Cq + 1));
  B.cols = c.take<int>(BH * D.Cq * D.Ck);
  B.runs = c.take<int2>(BH * D.Cq * D.Ck);
  B.nruns = c.take<int>(BH * D.Cq);
  B.rinfo = c.take<spr::RouteInfo>(BH);
  B.pcount = c.take<int>(BH * D.Cq);
  B.poff = c.take<int>(BH * (D.Cq + 1));
  B.pw_group = c.take<float>(BH * D.Cq);
  B.probes = c.take<int>(BH * D.M);
  B.pweights = c.take<float>(BH * D.M);
  B.pslot = c.take<int>(BH * N);
  B.kp = c.take<char>(BH * D.Npad * d * esz);
  B.vpt = c.take<char>(BH * D.Npad * d * esz);
  B.tiles = c.take<int2>(BH * D.max_tiles);
  B.ntiles = c.take<int>(BH);
  B.atiles = c.take<int2>(BH * D.max_tiles);  // max_atiles <= max_tiles for either tile height
  B.antiles = c.take<int>(BH);
  B.ptiles = c.take<int4>(BH * D.max_tiles);
  B.nptiles = c.take<int>(BH);
  B.gtiles = c.take<int>(BH * D.Cq);
  B.katt_rank = c.take<int>(BH * D.Ck);
  B.katt_start = c.take<int>(BH * (D.Ck + 1));
  B.kperm_att = c.take<int>(BH * N);
  B.tstart = c.take<int>(BH * (D.Cq + 1));
  B.mass_part = c.take<float>(BH * D.max_tiles * D.Ck);
  B.pp_o = c.take<float>(BH * D.M * D.pch * d);
  B.pp_ml = c.take<float2>(BH * D.M * D.pch);
  B.gram = c.take<double>(BH * (d + 1) * (2 * d + 1));
  B.rcov = c.take<float>(BH * d * d);
  B.rproj = c.take<float>(BH * d * d);
  B.theta_h = c.take<spr::bf16>(BH * d * d);
  B.theta_l = c.take<spr::bf16>(BH * d * d);
  B.status = c.take<int>(BH);
  if (total) *total = align_up(c.off, 256);
  return B;
}

sparsepr_status check_ws(sparsepr_plan_t p, void* ws, size_t bytes) {
  if (!ws) return SPARSEPR_ERR_WORKSPACE;
  if (bytes < p->ws_bytes) return SPARSEPR_ERR_WORKSPACE;
  if (((uintptr_t)ws) % 256 != 0) return SPARSEPR_ERR_WORKSPACE;
  return SPARSEPR_OK;
}

sparsepr_status hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPARSEPR_OK : SPARSEPR_ERR_HIP;
}

bool finite_d(double x) { return x == x && x < 1e300 && x > -1e300; }

}  // namespace

extern "C" {

const char* sparsepr_status_string(sparsepr_status s) {
  switch (s) {
    case SPARSEPR_OK: return "ok";
    case SPARSEPR_ERR_INVALID_ARG: return "invalid argument";
    case SPARSEPR_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPARSEPR_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SPARSEPR_ERR_HIP: return "HIP runtime error";
    case SPARSEPR_ERR_NUMERICAL: return "ridge system not positive definite";
    case SPARSEPR_ERR_STATE: return "call out of order";
    case SPARSEPR_ERR_TOO_LARGE: return "plan needs more device state than the static workspace holds";
  }
  return "unknown status";
}

sparsepr_status sparsepr_plan_create(const sparsepr_config* cfg, sparsepr_plan_t* out) {
  if (!cfg || !out) return SPARSEPR_ERR_INVALID_ARG;
  *out = nullptr;
  const sparsepr_config& c = *cfg;
  if (c.head_dim != 64 && c.head_dim != 128) return SPARSEPR_ERR_UNSUPPORTED;
  if (c.dtype != SPARSEPR_F32 && c.dtype != SPARSEPR_BF16) return SPARSEPR_ERR_UNSUPPORTED;
  if (c.batch < 1 || c.heads < 1 || c.seq_len < 1) return SPARSEPR_ERR_INVALID_ARG;
  if ((long long)c.batch * c.heads > 65535 || c.seq_len > (1 << 24)) return SPARSEPR_ERR_UNSUPPORTED;
  const int N = c.seq_len;
  if (c.n_sampled < 1 || c.n_sampled > N) return SPARSEPR_ERR_INVALID_ARG;
  if (c.n_key_groups < 1 || c.n_query_groups < 1) return SPARSEPR_ERR_INVALID_ARG;
  if (c.n_key_groups > N || c.n_query_groups > N) return SPARSEPR_ERR_INVALID_ARG;
  if (c.n_key_groups > spr::kMaxGroups || c.n_query_groups > spr::kMaxGroups) return SPARSEPR_ERR_UNSUPPORTED;
  if (c.n_probes < 0 || c.n_probes > N) return SPARSEPR_ERR_INVALID_ARG;
  if (!finite_d(c.density) || !(c.density > 0.0)) return SPARSEPR_ERR_INVALID_ARG;
  if (c.kmeans_max_iter < 1 || c.kmeans_max_iter > 10000) return SPARSEPR_ERR_INVALID_ARG;
  if (!finite_d(c.kmeans_tol) || c.kmeans_tol < 0.f) return SPARSEPR_ERR_INVALID_ARG;
  if (!finite_d(c.ridge_lambda) || c.ridge_lambda < 0.f) return SPARSEPR_ERR_INVALID_ARG;
  if (!finite_d(c.softmax_scale) || c.softmax_scale < 0.f) return SPARSEPR_ERR_INVALID_ARG;
  if (c.assign_precision != 0 && c.assign_precision != 1) return SPARSEPR_ERR_INVALID_ARG;
  if (c.warm_iters < 0 || c.warm_iters > 10000) return SPARSEPR_ERR_INVALID_ARG;
  if (c.partition < 0 || c.partition > 2) return SPARSEPR_ERR_INVALID_ARG;
  if (c.correction < 0 || c.correction > 2) return SPARSEPR_ERR_INVALID_ARG;
  if (c.probe_selector < 0 || c.probe_selector > 2) return SPARSEPR_ERR_INVALID_ARG;
  if (c.key_rank < 0) return SPARSEPR_ERR_INVALID_ARG;
  if (c.attn_tile_rows != 0 && c.attn_tile_rows != 128 && c.attn_tile_rows != 256) return SPARSEPR_ERR_INVALID_ARG;
  if (c.output_rank < 0) return SPARSEPR_ERR_INVALID_ARG;

  sparsepr_plan_s* p = new (std::nothrow) sparsepr_plan_s();
  if (!p) return SPARSEPR_ERR_INVALID_ARG;
  p->cfg = c;
  Dims& D = p->D;
  D.BH = c.batch * c.heads;
  D.N = N;
  D.d = c.head_dim;
  D.S = c.n_sampled;
  D.Ck = c.n_key_groups;
  D.Cq = c.n_query_groups;
  D.M = c.n_probes;
  D.C = D.Ck > D.Cq ? D.Ck : D.Cq;
  D.nblk = (N + spr::kKmRows - 1) / spr::kKmRows;
  D.Npad = (N + 63) / 64 * 64 + 64;
  D.qt = spr::kAttnQT;
  D.max_tiles = (N + spr::kAttnQT - 1) / spr::kAttnQT + D.Cq;
  // Attention tiles of 256 rows (8 waves: each staged key tile feeds twice the queries) when
  // the call has enough of them to fill the GPU several times over (at least 1,024 full tiles,
  // four per CU); small calls take 128-row tiles (4 waves, two workgroups per CU), whose
  // shorter tail keeps every CU busy to the end.
  if (c.attn_tile_rows == 128 || c.attn_tile_rows == 256) D.attn_w = c.attn_tile_rows / 32;
  else D.attn_w = (long long)D.BH * N >= 1024ll * 256 ? 8 : 4;
  D.max_atiles = (N + 32 * D.attn_w - 1) / (32 * D.attn_w) + D.Cq;
  {
    // split the probe rows' keys so that about 1024 workgroups share the probe attention
    // (probe tiles have the attention tiles' height), rounded up, when that at most doubles
    // the split, to whole rounds of the workgroups the CUs hold at once (one per CU for
    // 256-row tiles, two for 128-row ones), so that the last round is not a partial one
    const int ptiles = (D.M + 32 * D.attn_w - 1) / (32 * D.attn_w);
    const long long items = (long long)D.BH * ptiles;
    long long want = ptiles > 0 ? (1024 + items - 1) / items : 1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
      cus = 256;  // (no device: the MI355X's count)
    const long long slots = (long long)cus * (D.attn_w == 8 ? 1 : 2);
    for (long long c = want; ptiles > 0 && c <= 2 * want; ++c)
      if ((items * c) % slots == 0) {
        want = c;
        break;
      }
    const int maxch = (N + 511) / 512;
    int pch = (int)(want < 1 ? 1 : (want > maxch ? maxch : want));
    if (pch < 1) pch = 1;
    D.pkc = ((N + pch - 1) / pch + spr::kKeyTile - 1) / spr::kKeyTile * spr::kKeyTile;
    D.pch = (N + D.pkc - 1) / D.pkc;
  }
  D.dtype = c.dtype;
  D.scale = c.softmax_scale > 0.f ? c.softmax_scale : (float)(1.0 / sqrt((double)c.head_dim));
  D.log2_scale = (float)((double)D.scale * 1.4426950408889634);
  D.density = c.density;
  D.budget = (long long)floor(c.density * (double)((long long)N * N)) - (long long)D.M * N;
  D.max_iter = c.kmeans_max_iter;
  D.warm_iter = c.warm_iters > 0 ? c.warm_iters : 2;
  D.tol = c.kmeans_tol;
  D.lambda = c.ridge_lambda;
  D.pen_bias = c.penalize_bias ? 1 : 0;
  D.assign_lo = c.assign_precision ? 1 : 0;
  D.partition = c.partition;
  D.correction = c.correction;
  D.probe_sel = c.probe_selector;
  D.key_rank = c.key_rank;
  D.output_rank = c.output_rank < c.head_dim ? c.output_rank : 0;  // rank >= d keeps the whole span
  D.seed = c.seed;
  carve(D, nullptr, &p->ws_bytes);
  p->ws = nullptr;
  p->planned = 0;
  p->timing = 0;
  *out = p;
  return SPARSEPR_OK;
}

static void destroy_events(sparsepr_plan_t p, int upto) {
  hipEvent_t* e = &p->ev[0][0][0];
  for (int i = 0; i < upto; ++i) (void)hipEventDestroy(e[i]);
}

void sparsepr_plan_destroy(sparsepr_plan_t plan) {
  if (!plan) return;
  if (plan->timing) destroy_events(plan, SPARSEPR_NUM_STAGES * kTimingRing * 2);
  delete plan;
}

sparsepr_status sparsepr_set_stage_timing(sparsepr_plan_t p, int32_t enable) {
  if (!p) return SPARSEPR_ERR_INVALID_ARG;
  if (enable && !p->timing) {
    hipEvent_t* e = &p->ev[0][0][0];
    const int n = SPARSEPR_NUM_STAGES * kTimingRing * 2;
    for (int i = 0; i < n; ++i) {
      if (hipEventCreate(&e[i]) != hipSuccess) {
        destroy_events(p, i);
        return SPARSEPR_ERR_HIP;
      }
    }
    for (int i = 0; i < SPARSEPR_NUM_STAGES; ++i) p->count[i] = 0;
    p->timing = 1;
  } else if (!enable && p->timing) {
    destroy_events(p, SPARSEPR_NUM_STAGES * kTimingRing * 2);
    p->timing = 0;
  }
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_stage_times(sparsepr_plan_t p, float* ms, int32_t n) {
  if (!p || !ms || n < 1 || n > SPARSEPR_NUM_STAGES) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->timing) return SPARSEPR_ERR_STATE;
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.f;
    const int c = p->count[i] < kTimingRing ? p->count[i] : kTimingRing;
    double tot = 0.0;
    for (int j = 0; j < c; ++j) {
      float t = 0.f;
      if (hipEventSynchronize(p->ev[i][j][1]) != hipSuccess) return SPARSEPR_ERR_HIP;
      if (hipEventElapsedTime(&t, p->ev[i][j][0], p->ev[i][j][1]) != hipSuccess) return SPARSEPR_ERR_HIP;
      tot += t;
    }
    ms[i] = c ? (float)(tot / c) : 0.f;
  }
  for (int i = 0; i < SPARSEPR_NUM_STAGES; ++i) p->count[i] = 0;
  return SPARSEPR_OK;
}

size_t sparsepr_workspace_bytes(sparsepr_plan_t plan) { return plan ? plan->ws_bytes : 0; }

static sparsepr_status begin_plan(sparsepr_plan_t p, void* ws, size_t bytes, Bufs* B, hipStream_t s) {
  sparsepr_status st = check_ws(p, ws, bytes);
  if (st != SPARSEPR_OK) return st;
  p->ws = ws;
  p->planned = 0;
  *B = carve(p->D, ws, nullptr);
  spr::launch_fill_i32(B->status, p->D.BH, 0, s);
  return SPARSEPR_OK;
}

sparsepr_status sparsepr_plan(sparsepr_plan_t p, const void* q, const void* k, void* ws, size_t bytes,
                              void* stream) {
  if (!p || !q || !k) return SPARSEPR_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  Bufs B;
  sparsepr_status st = begin_plan(p, ws, bytes, &B, s);
  if (st != SPARSEPR_OK) return st;
  {
    StageTimer t(p, SPARSEPR_STAGE_PLAN, s);
    spr::launch_plan(q, k, p->D, B, s);
    spr::launch_route_probes(p->D, B, s);
  }
  st = hip_status();
  if (st == SPARSEPR_OK) p->planned = 1;
  return st;
}

sparsepr_status sparsepr_plan_warm(sparsepr_plan_t p, const void* q, const void* k, void* ws, size_t bytes,
                                   void* stream) {
  if (!p || !q || !k) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->planned || p->ws != ws) return SPARSEPR_ERR_STATE;
  hipStream_t s = (hipStream_t)stream;
  Bufs B;
  sparsepr_status st = begin_plan(p, ws, bytes, &B, s);
  if (st != SPARSEPR_OK) return st;
  {
    StageTimer t(p, SPARSEPR_STAGE_PLAN, s);
    spr::launch_plan_warm(q, k, p->D, B, s);
    spr::launch_route_probes(p->D, B, s);
  }
  st = hip_status();
  if (st == SPARSEPR_OK) p->planned = 1;
  return st;
}

sparsepr_status sparsepr_plan_from_labels(sparsepr_plan_t p, const void* q, const void* k, const int32_t* key_labels,
                                          const int32_t* query_labels, const int64_t* group_mass, void* ws,
                                          size_t bytes, void* stream) {
  if (!p || !q || !k || !key_labels || !query_labels) return SPARSEPR_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  Bufs B;
  sparsepr_status st = begin_plan(p, ws, bytes, &B, s);
  if (st != SPARSEPR_OK) return st;
  {
    StageTimer t(p, SPARSEPR_STAGE_PLAN, s);
    spr::launch_plan_from_labels(q, k, key_labels, query_labels, (const long long*)group_mass, p->D, B, s);
    spr::launch_route_probes(p->D, B, s);
  }
  st = hip_status();
  if (st == SPARSEPR_OK) p->planned = 1;
  return st;
}

sparsepr_status sparsepr_plan_set_probes(sparsepr_plan_t p, const int32_t* probes, const float* weights, void* ws,
                                        size_t bytes, void* stream) {
  if (!p || !probes) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->planned || p->ws != ws) return SPARSEPR_ERR_STATE;
  sparsepr_status st = check_ws(p, ws, bytes);
  if (st != SPARSEPR_OK) return st;
  const Dims& D = p->D;
  if (D.M == 0) return SPARSEPR_OK;
  hipStream_t s = (hipStream_t)stream;
  // host-side validation: every head's M rows in [0, N) and distinct
  const size_t n = (size_t)D.BH * D.M;
  int32_t* h = (int32_t*)malloc(n * sizeof(int32_t));
  unsigned char* seen = (unsigned char*)malloc((size_t)D.N);
  if (!h || !seen) {
    free(h);
    free(seen);
    return SPARSEPR_ERR_INVALID_ARG;
  }
  bool ok = hipMemcpyAsync(h, probes, n * sizeof(int32_t), hipMemcpyDeviceToHost, s) == hipSuccess &&
            hipStreamSynchronize(s) == hipSuccess;
  if (!ok) {
    free(h);
    free(seen);
    return SPARSEPR_ERR_HIP;
  }
  for (int bh = 0; bh < D.BH && ok; ++bh) {
    memset(seen, 0, (size_t)D.N);
    for (int r = 0; r < D.M && ok; ++r) {
      const int32_t t = h[(size_t)bh * D.M + r];
      ok = t >= 0 && t < D.N && !seen[t];
      if (ok) seen[t] = 1;
    }
  }
  free(h);
  free(seen);
  if (!ok) return SPARSEPR_ERR_INVALID_ARG;
  Bufs B = carve(D, ws, nullptr);
  {
    StageTimer t(p, SPARSEPR_STAGE_PLAN, s);
    spr::launch_set_probes(D, B, probes, weights, s);
  }
  return hip_status();
}

sparsepr_status sparsepr_attend(sparsepr_plan_t p, const void* q, const void* k, const void* v, void* o_sparse,
                                float* o_probe_sparse, float* o_probe_dense, void* stream) {
  if (!p || !q || !k || !v || !o_sparse) return SPARSEPR_ERR_INVALID_ARG;
  if (p->D.M > 0 && (!o_probe_dense || !o_probe_sparse)) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->planned) return SPARSEPR_ERR_STATE;
  hipStream_t s = (hipStream_t)stream;
  Bufs B = carve(p->D, p->ws, nullptr);
  {
    StageTimer t(p, SPARSEPR_STAGE_PERMUTE, s);
    spr::launch_permute_kv(k, v, p->D, B, p->D.dtype == 1 && p->D.attn_w == 8 ? B.kperm_att : B.kperm, s);
  }
  {
    StageTimer t(p, SPARSEPR_STAGE_SPARSE, s);
    spr::launch_attend_sparse(q, p->D, B, o_sparse, o_probe_sparse, s);
  }
  {
    StageTimer t(p, SPARSEPR_STAGE_PROBES, s);
    spr::launch_attend_probes(q, p->D, B, o_probe_dense, s);
  }
  return hip_status();
}

sparsepr_status sparsepr_fit_residual(sparsepr_plan_t p, const float* o_probe_sparse, const float* o_probe_dense,
                                      const float* probe_weights, float* coeffs, void* stream) {
  if (!p || !coeffs) return SPARSEPR_ERR_INVALID_ARG;
  if (p->D.M > 0 && (!o_probe_dense || !o_probe_sparse)) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->planned) return SPARSEPR_ERR_STATE;
  hipStream_t s = (hipStream_t)stream;
  Bufs B = carve(p->D, p->ws, nullptr);
  StageTimer t(p, SPARSEPR_STAGE_FIT, s);
  spr::launch_fit(p->D, B, o_probe_sparse, o_probe_dense, probe_weights, coeffs, s);
  return hip_status();
}

sparsepr_status sparsepr_apply(sparsepr_plan_t p, const void* o_sparse, const float* o_probe_dense,
                               const float* coeffs, void* out, void* stream) {
  if (!p || !o_sparse || !coeffs || !out) return SPARSEPR_ERR_INVALID_ARG;
  if (p->D.M > 0 && !o_probe_dense) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->planned) return SPARSEPR_ERR_STATE;
  hipStream_t s = (hipStream_t)stream;
  Bufs B = carve(p->D, p->ws, nullptr);
  StageTimer t(p, SPARSEPR_STAGE_APPLY, s);
  spr::launch_apply(p->D, B, o_sparse, o_probe_dense, coeffs, out, s);
  return hip_status();
}

sparsepr_status sparsepr_dense_attention(sparsepr_plan_t p, const void* q, const void* k, const void* v, void* out,
                                         void* ws, size_t bytes, void* stream) {
  if (!p || !q || !k || !v || !out) return SPARSEPR_ERR_INVALID_ARG;
  sparsepr_status st = check_ws(p, ws, bytes);
  if (st != SPARSEPR_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  p->ws = ws;
  p->planned = 0;  // the identity partition replaces any plan in this workspace
  Bufs B = carve(p->D, ws, nullptr);
  // one query group of N rows: full 256-row attention tiles
  Dims Dd = p->D;
  Dd.attn_w = 8;
  Dd.max_atiles = (Dd.N + 255) / 256 + Dd.Cq;
  spr::launch_identity_plan(Dd, B, s);
  spr::launch_permute_kv(k, v, Dd, B, B.kperm, s);
  spr::launch_attend_sparse(q, Dd, B, out, nullptr, s, true);
  return hip_status();
}

sparsepr_status sparsepr_plan_info(sparsepr_plan_t p, sparsepr_head_info* info, int32_t n_heads, void* stream) {
  if (!p || !info || n_heads < 1 || n_heads > p->D.BH) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->planned) return SPARSEPR_ERR_STATE;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return SPARSEPR_ERR_HIP;
  Bufs B = carve(p->D, p->ws, nullptr);
  const int n = n_heads;
  spr::KmState* ks = (spr::KmState*)malloc(sizeof(spr::KmState) * n * 2);
  spr::RouteInfo* ri = (spr::RouteInfo*)malloc(sizeof(spr::RouteInfo) * n);
  int* stv = (int*)malloc(sizeof(int) * n);
  sparsepr_status st = SPARSEPR_OK;
  if (!ks || !ri || !stv) st = SPARSEPR_ERR_INVALID_ARG;
  if (st == SPARSEPR_OK &&
      (hipMemcpy(ks, B.kst, sizeof(spr::KmState) * n, hipMemcpyDeviceToHost) != hipSuccess ||
       hipMemcpy(ks + n, B.qst, sizeof(spr::KmState) * n, hipMemcpyDeviceToHost) != hipSuccess ||
       hipMemcpy(ri, B.rinfo, sizeof(spr::RouteInfo) * n, hipMemcpyDeviceToHost) != hipSuccess ||
       hipMemcpy(stv, B.status, sizeof(int) * n, hipMemcpyDeviceToHost) != hipSuccess))
    st = SPARSEPR_ERR_HIP;
  if (st == SPARSEPR_OK) {
    for (int i = 0; i < n; ++i) {
      info[i].key_groups = ks[i].c_final;
      info[i].query_groups = ks[n + i].c_final;
      info[i].key_iters = ks[i].iters;
      info[i].query_iters = ks[n + i].iters;
      info[i].executed_pairs = ri[i].pairs;
      info[i].budget = ri[i].budget;
      info[i].tau = ri[i].tau;
      info[i].budget_exceeded = ri[i].exceeded;
      info[i].status = stv[i];
    }
  }
  free(ks);
  free(ri);
  free(stv);
  return st;
}

static bool export_region(sparsepr_plan_t p, int which, const Bufs& B, const void** src, size_t* bytes) {
  const Dims& D = p->D;
  const size_t BH = D.BH;
  switch (which) {
    case SPARSEPR_EXPORT_SAMPLED: *src = B.sampled; *bytes = BH * D.S * 4; return true;
    case SPARSEPR_EXPORT_KEY_LABELS: *src = B.klab; *bytes = BH * D.N * 4; return true;
    case SPARSEPR_EXPORT_QUERY_LABELS: *src = B.qlab; *bytes = BH * D.N * 4; return true;
    case SPARSEPR_EXPORT_KEY_PERM: *src = B.kperm; *bytes = BH * D.N * 4; return true;
    case SPARSEPR_EXPORT_QUERY_PERM: *src = B.qperm; *bytes = BH * D.N * 4; return true;
    case SPARSEPR_EXPORT_KEY_OFFSETS: *src = B.koff; *bytes = BH * (D.Ck + 1) * 4; return true;
    case SPARSEPR_EXPORT_QUERY_OFFSETS: *src = B.qoff; *bytes = BH * (D.Cq + 1) * 4; return true;
    case SPARSEPR_EXPORT_ROUTE_ROWPTR: *src = B.row_ptr; *bytes = BH * (D.Cq + 1) * 4; return true;
    case SPARSEPR_EXPORT_ROUTE_COLS: *src = B.cols; *bytes = BH * D.Cq * D.Ck * 4; return true;
    case SPARSEPR_EXPORT_PROBES: *src = B.probes; *bytes = BH * D.M * 4; return true;
    case SPARSEPR_EXPORT_PROBE_WEIGHTS: *src = B.pweights; *bytes = BH * D.M * 4; return true;
    case SPARSEPR_EXPORT_GROUP_MASS: *src = B.u; *bytes = BH * D.Cq * D.Ck * 8; return true;
    case SPARSEPR_EXPORT_KEY_CENTROIDS: *src = B.kcent; *bytes = BH * D.Ck * D.d * 4; return true;
    case SPARSEPR_EXPORT_KEY_SEEDS: *src = B.init_k; *bytes = BH * D.Ck * 4; return true;
    case SPARSEPR_EXPORT_QUERY_SEEDS: *src = B.init_q; *bytes = BH * D.Cq * 4; return true;
  }
  return false;
}

size_t sparsepr_export_bytes(sparsepr_plan_t p, int32_t which) {
  if (!p) return 0;
  Bufs B = carve(p->D, nullptr, nullptr);
  const void* src;
  size_t bytes;
  return export_region(p, which, B, &src, &bytes) ? bytes : 0;
}

sparsepr_status sparsepr_plan_export(sparsepr_plan_t p, int32_t which, void* dst, size_t dst_bytes, void* stream) {
  if (!p || !dst) return SPARSEPR_ERR_INVALID_ARG;
  if (!p->planned) return SPARSEPR_ERR_STATE;
  Bufs B = carve(p->D, p->ws, nullptr);
  const void* src;
  size_t bytes;
  if (!export_region(p, which, B, &src, &bytes)) return SPARSEPR_ERR_INVALID_ARG;
  if (dst_bytes < bytes) return SPARSEPR_ERR_INVALID_ARG;
  if (bytes == 0) return SPARSEPR_OK;
  if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream) != hipSuccess)
    return SPARSEPR_ERR_HIP;
  return SPARSEPR_OK;
}

}  // extern "C"
