// Planning kernels of the SparsePR call: Response-Coupled Partitioning, group masses,
// budgeted routing, stratified probes and the group-contiguous K/V layout.
//
// Sources: paper "Partition the Support, Reconstruct the Residual" -- abstract (key
// groups from sampled-query key responses, query groups from responses to key-group
// centroids, routing under an executed-pair density budget, stratified probe rows);
// Table C.1 (Lloyd limits: 25 iterations, tolerance 1e-4); Table D.1 (per-query RMS
// normalisation of the query responses); project website, Method section, stages 01-03.
//
// Lloyd runs in metric form. Key responses are R_K = s K Q_S^T and every centroid is a
// mean of such rows, so |R_K,j - c_b|^2 = (k_j - m_b) G (k_j - m_b)^T with G = s^2 Q_S^T Q_S
// and m_b the key-space mean. Query features F_i = (s / RMS_i) q_i C_k^T likewise give
// |F_i - g_a|^2 = (x_i - z_a) G_k (x_i - z_a)^T with x_i = alpha_i q_i, alpha_i = s / RMS_i,
// G_k = C_k^T C_k. The assignment therefore needs score_b = m_b G m_b - 2 x.(G m_b) over
// d-wide rows instead of S- or C_k-wide ones; the labels are those of Lloyd on the
// response rows themselves.
#include <type_traits>

#include "common.h"
#include "plan_state.h"
#include "launch.h"

namespace spr {

// =====================================================================================
// Block scans
// =====================================================================================
template <int BT>
__device__ int block_excl_scan_bool(bool f, int* total, int* ws /* LDS [BT/64] */) {
  const uint64_t b = __ballot(f);
  const int w = threadIdx.x / kWave;
  const int r = __popcll(b & lanemask_lt());
  if (lane_id() == 0) ws[w] = __popcll(b);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < BT / kWave; ++i) {
    const int c = ws[i];
    base += (i < w) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + r;
}

template <int BT, typename V>
__device__ V block_excl_scan(V v, V* total, V* ws /* LDS [BT/64] */) {
  const int w = threadIdx.x / kWave;
  V inc = v;
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    V t = __shfl_up(inc, o, kWave);
    if (l >= o) inc += t;
  }
  if (l == kWave - 1) ws[w] = inc;
  __syncthreads();
  V base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < BT / kWave; ++i) {
    V c = ws[i];
    base += (i < w) ? c : (V)0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

template <int BT, typename V>
__device__ V block_sum(V v, V* ws) {
  V t;
  (void)block_excl_scan<BT, V>(v, &t, ws);
  return t;
}

// The centroid side of the Lloyd assignment's bias product for cn = m_b G m_b (see
// k_km_assign_bf16): k-slots [cn_hi, cn_hi, cn_lo, 1, 1] and zeros (16 slots, 32 bytes), so
// that its product with the row side [1/alpha hi, lo, hi, rc/alpha hi, lo] is
// cn / alpha + rc / alpha. A dead centroid (cn = +inf) takes [+inf, 0, ...]: its value is
// +inf, with no inf x 0 term.
__device__ inline void store_bias_operand(bf16* dst, float cn) {
  const bf16 hi = (bf16)cn;
  const bool fin = cn < INFINITY;
  bf16x8 v = bf16x8{};
  v[0] = hi;
  if (fin) {
    v[1] = hi;
    v[2] = (bf16)(cn - (float)hi);
    v[3] = (bf16)1.f;
    v[4] = (bf16)1.f;
  }
  reinterpret_cast<bf16x8*>(dst)[0] = v;
  reinterpret_cast<bf16x8*>(dst)[1] = bf16x8{};
}

// =====================================================================================
// Selection of the m candidates with the smallest (hash, id), output in ascending id
// order. Candidates are cand(0..n-1), ascending. Radix select over the 64-bit hash
// finds the m-th smallest value T exactly; ties at T are broken by id.
// =====================================================================================
template <int BT, typename Cand>
__device__ void select_smallest(int n, int m, Cand cand, uint64_t base, int* out) {
  __shared__ int hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_k, s_alleq;
  __shared__ int ws[BT / kWave];
  __shared__ uint64_t ch[BT];
  __shared__ int ci[BT];
  const int tid = threadIdx.x;
  if (m <= 0) return;
  if (m >= n) {
    for (int i = tid; i < n; i += BT) out[i] = cand(i);
    return;
  }
  if (n <= BT) {
    // direct ranks: candidate i is chosen iff fewer than m candidates precede it in (hash, id)
    const bool valid = tid < n;
    const int id = valid ? cand(tid) : 0;
    const uint64_t h = valid ? splitmix64(base ^ (uint64_t)(uint32_t)id) : 0ull;
    if (valid) {
      ch[tid] = h;
      ci[tid] = id;
    }
    __syncthreads();
    int rank = 0;
    if (valid)
      for (int j = 0; j < n; ++j) rank += (ch[j] < h) || (ch[j] == h && ci[j] < id);
    int tot;
    const bool sel = valid && rank < m;
    const int pos = block_excl_scan_bool<BT>(sel, &tot, ws);
    if (sel) out[pos] = id;
    return;
  }
  // Three passes: a 4096-bin histogram of the hash's top 12 bits finds the bin T holding
  // the m-th smallest; the candidates of bin T (about n / 4096) are gathered in LDS and
  // ranked exactly; the last pass outputs every candidate below the m-th. A bin T larger
  // than the gather buffer (not expected for uniform hashes) falls back to the radix passes.
  if constexpr (BT >= 256) {
    constexpr int NB2 = 4096, BPT = NB2 / BT;
    __shared__ int hist2[NB2];
    __shared__ int s_bin, s_below, s_cnt, s_tid;
    __shared__ uint64_t s_th;
    for (int i = tid; i < NB2; i += BT) hist2[i] = 0;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    for (int i = tid; i < n; i += BT) {
      const uint64_t h = splitmix64(base ^ (uint64_t)(uint32_t)cand(i));
      atomicAdd(&hist2[(int)(h >> 52)], 1);
    }
    __syncthreads();
    int loc[BPT], sum = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      loc[q] = hist2[tid * BPT + q];
      sum += loc[q];
    }
    int tot2;
    const int exc = block_excl_scan<BT, int>(sum, &tot2, ws);
    if (exc < m && exc + sum >= m) {
      int cacc = exc;
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (cacc < m && cacc + loc[q] >= m) {
          s_bin = tid * BPT + q;
          s_below = cacc;
        }
        cacc += loc[q];
      }
    }
    __syncthreads();
    const int T = s_bin, kk = m - s_below;
    for (int i = tid; i < n; i += BT) {
      const int id = cand(i);
      const uint64_t h = splitmix64(base ^ (uint64_t)(uint32_t)id);
      if ((int)(h >> 52) == T) {
        const int p = atomicAdd(&s_cnt, 1);
        if (p < BT) {
          ch[p] = h;
          ci[p] = id;
        }
      }
    }
    __syncthreads();
    const int cnt = s_cnt;
    if (cnt <= BT) {
      if (tid < cnt) {
        const uint64_t h = ch[tid];
        const int id = ci[tid];
        int rank = 0;
        for (int j = 0; j < cnt; ++j) rank += (ch[j] < h) || (ch[j] == h && ci[j] < id);
        if (rank == kk - 1) {
          s_th = h;
          s_tid = id;
        }
      }
      __syncthreads();
      const uint64_t hT = s_th;
      const int idT = s_tid;
      int run_sel = 0;
      for (int c0 = 0; c0 < n; c0 += BT) {
        const int i = c0 + tid;
        const bool valid = i < n;
        const int id = valid ? cand(i) : 0;
        const uint64_t h = valid ? splitmix64(base ^ (uint64_t)(uint32_t)id) : 0ull;
        const int bin = (int)(h >> 52);
        const bool sel = valid && (bin < T || (bin == T && (h < hT || (h == hT && id <= idT))));
        int sel_tot;
        const int pos = block_excl_scan_bool<BT>(sel, &sel_tot, ws) + run_sel;
        if (sel) out[pos] = id;
        run_sel += sel_tot;
      }
      return;
    }
  }
  uint64_t prefix = 0;
  int k = m;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int i = tid; i < 256; i += BT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += BT) {
      const uint64_t h = splitmix64(base ^ (uint64_t)(uint32_t)cand(i));
      if ((h & hi_mask) == prefix) atomicAdd(&hist[(h >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < kWave) {
      // the lane whose 4 bins hold the k-th candidate picks the digit
      const int c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2], c3 = hist[4 * tid + 3];
      const int loc = c0 + c1 + c2 + c3;
      const int inc = wave_incl_scan(loc), exc = inc - loc;
      if (exc < k && inc >= k) {
        int c = exc, dg, cnt;
        if (c + c0 >= k) { dg = 4 * tid; cnt = c0; }
        else if ((c += c0) + c1 >= k) { dg = 4 * tid + 1; cnt = c1; }
        else if ((c += c1) + c2 >= k) { dg = 4 * tid + 2; cnt = c2; }
        else { c += c2; dg = 4 * tid + 3; cnt = c3; }
        s_prefix = prefix | ((uint64_t)dg << shift);
        s_k = k - c;
        s_alleq = (k - c) == cnt;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    k = s_k;
    __syncthreads();
  }
  // prefix = T, the m-th smallest hash; take every h < T and the first k ids with h == T
  const bool alleq = s_alleq;
  int run_sel = 0, run_eq = 0;
  for (int c0 = 0; c0 < n; c0 += BT) {
    const int i = c0 + tid;
    const bool valid = i < n;
    const int id = valid ? cand(i) : 0;
    const uint64_t h = valid ? splitmix64(base ^ (uint64_t)(uint32_t)id) : 0ull;
    int sel_tot;
    bool sel;
    if (alleq) {
      sel = valid && h <= prefix;
    } else {
      int eq_tot;
      const bool eq = valid && h == prefix;
      const int eq_rank = block_excl_scan_bool<BT>(eq, &eq_tot, ws) + run_eq;
      sel = (valid && h < prefix) || (eq && eq_rank < k);
      run_eq += eq_tot;
    }
    const int pos = block_excl_scan_bool<BT>(sel, &sel_tot, ws) + run_sel;
    if (sel) out[pos] = id;
    run_sel += sel_tot;
  }
}

// The three whole-sequence selections of a plan in one launch: blockIdx.y = 0 sampled
// queries (stream 1), 1 key-group seeds (stream 2), 2 query-group seeds (stream 3).
__global__ __launch_bounds__(1024) void k_select_all(Dims D, Bufs B) {
  const int bh = blockIdx.x, which = blockIdx.y;
  const int m = which == 0 ? D.S : (which == 1 ? D.Ck : D.Cq);
  int* out = which == 0 ? B.sampled + (size_t)bh * D.S
                        : (which == 1 ? B.init_k + (size_t)bh * D.Ck : B.init_q + (size_t)bh * D.Cq);
  const uint64_t base = head_hash_base(D.seed, (uint64_t)(which + 1), (uint64_t)bh);
  select_smallest<1024>(D.N, m, [](int i) { return i; }, base, out);
}

// Probe rows of query group a: m_a members with the smallest (hash, token id).
__global__ __launch_bounds__(256) void k_select_probes(Dims D, Bufs B) {
  const int a = blockIdx.x, bh = blockIdx.y;
  if (a >= B.qst[bh].c_final) return;
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const int n = qo[a + 1] - qo[a];
  const int m = B.pcount[(size_t)bh * D.Cq + a];
  const int o0 = B.poff[(size_t)bh * (D.Cq + 1) + a];
  const int* members = B.qperm + (size_t)bh * D.N + qo[a];
  const uint64_t base = head_hash_base(D.seed, kStreamProbes, (uint64_t)bh);
  int* out = B.probes + (size_t)bh * D.M + o0;
  select_smallest<256>(n, m, [members](int i) { return members[i]; }, base, out);
  __syncthreads();
  const float w = B.pw_group[(size_t)bh * D.Cq + a];
  for (int r = threadIdx.x; r < m; r += 256) {
    B.pweights[(size_t)bh * D.M + o0 + r] = w;
    B.pslot[(size_t)bh * D.N + out[r]] = o0 + r;
  }
}

// Probe rows of the comparison selectors (paper Table 4): random = the M tokens with the
// smallest probe hash; uniform = tokens floor((2p + 1) N / 2M), evenly spaced in token
// (raster) order. Ascending token id, unit weights.
__global__ __launch_bounds__(1024) void k_select_probes_plain(Dims D, Bufs B) {
  const int bh = blockIdx.x;
  int* out = B.probes + (size_t)bh * D.M;
  if (D.probe_sel == 1) {
    const uint64_t base = head_hash_base(D.seed, kStreamProbes, (uint64_t)bh);
    select_smallest<1024>(D.N, D.M, [](int i) { return i; }, base, out);
  } else {
    for (int r = threadIdx.x; r < D.M; r += 1024) out[r] = (int)(((2ll * r + 1) * D.N) / (2ll * D.M));
  }
  __syncthreads();
  for (int r = threadIdx.x; r < D.M; r += 1024) {
    B.pweights[(size_t)bh * D.M + r] = 1.f;
    B.pslot[(size_t)bh * D.N + out[r]] = r;
  }
}

// Probe rows given by the caller (validated on the host: in range and distinct per head):
// weights given or 1, slots rebuilt.
__global__ __launch_bounds__(256) void k_set_probes(Dims D, Bufs B, const int* probes, const float* weights) {
  const int bh = blockIdx.x;
  int* slot = B.pslot + (size_t)bh * D.N;
  for (int i = threadIdx.x; i < D.N; i += 256) slot[i] = -1;
  __syncthreads();
  for (int r = threadIdx.x; r < D.M; r += 256) {
    const size_t o = (size_t)bh * D.M + r;
    const int t = probes[o];
    B.probes[o] = t;
    B.pweights[o] = weights ? weights[o] : 1.f;
    slot[t] = r;
  }
}

void launch_set_probes(const Dims& D, const Bufs& B, const int* probes, const float* weights, hipStream_t s) {
  hipLaunchKernelGGL(k_set_probes, dim3(D.BH), dim3(256), 0, s, D, B, probes, weights);
}

// Identity Lloyd metric: semantic partitions cluster the raw vectors (paper Table 2).
template <int DD>
__global__ void k_identity_metric(Dims D, Bufs B) {
  const int bh = blockIdx.y;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < DD * DD; e += gridDim.x * blockDim.x) {
    const float v = (e / DD == e % DD) ? 1.f : 0.f;
    const size_t o = (size_t)bh * DD * DD + e;
    B.metric[o] = v;
    B.metric_h[o] = (bf16)v;
    B.metric_l[o] = (bf16)0.f;
  }
}

// =====================================================================================
// Small dense helpers
// =====================================================================================
template <typename T>
__global__ void k_gather_rows(const T* x, const int* idx, int N, int S, int d, float* out) {
  const int t = blockIdx.x, bh = blockIdx.y;
  const int row = idx[(size_t)bh * S + t];
  const T* src = x + ((size_t)bh * N + row) * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) out[((size_t)bh * S + t) * d + i] = to_f32(src[i]);
}

// G = scale2 * sum_r rows_r^T rows_r over the first count rows (count from KmState when
// given). Block (gi, bh) owns G rows [RG*gi, RG*gi + RG): one entry per thread.
template <int DD>
__global__ __launch_bounds__(256) void k_gram(const float* rows, int R, const KmState* cnt_state, float scale2,
                                              float* G, bf16* Gh, bf16* Gl) {
  constexpr int RG = 256 / DD;
  constexpr int CH = 32;
  __shared__ float sh[CH][DD];
  const int gi = blockIdx.x, bh = blockIdx.y;
  const int n = cnt_state ? cnt_state[bh].c_final : R;
  const float* src = rows + (size_t)bh * R * DD;
  const int i = gi * RG + threadIdx.x / DD, j = threadIdx.x % DD;
  float acc = 0.f;
  for (int r0 = 0; r0 < n; r0 += CH) {
    __syncthreads();
    for (int e = threadIdx.x; e < CH * DD / 4; e += 256) {
      const int r = e / (DD / 4), c4 = (e % (DD / 4)) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r0 + r < n) v = *reinterpret_cast<const float4*>(src + (size_t)(r0 + r) * DD + c4);
      *reinterpret_cast<float4*>(&sh[r][c4]) = v;
    }
    __syncthreads();
    const int rmax = min(CH, n - r0);
    for (int r = 0; r < rmax; ++r) acc = fmaf(sh[r][i], sh[r][j], acc);
  }
  const float g = scale2 * acc;
  const size_t o = (size_t)bh * DD * DD + (size_t)i * DD + j;
  G[o] = g;
  const bf16 gh = (bf16)g;
  Gh[o] = gh;
  Gl[o] = (bf16)(g - (float)gh);
}

// =====================================================================================
// SIMT tile engine: 128 rows (staged transposed in LDS) against 64-column tiles of a
// row-major float matrix Y[cols][DD]; thread (ty, tx) owns rows 8ty..8ty+7 and columns
// 4tx..4tx+3 of the tile.
// =====================================================================================
constexpr int kRB = kKmRows;
constexpr int kKC = 32;

template <typename T, int DD>
__device__ inline void stage_rows(const T* x, int N, int r0, const float* alpha, float (*Xs)[kRB + 4]) {
  // Xs[k][r] = alpha_r * x[r0 + r][k] (zero beyond N)
  for (int i = threadIdx.x; i < kRB * DD; i += 256) {
    const int r = i / DD, k = i % DD;
    const int row = r0 + r;
    float v = 0.f;
    if (row < N) {
      v = to_f32(x[(size_t)row * DD + k]);
      if (alpha) v *= alpha[row];
    }
    Xs[k][r] = v;
  }
}

template <int DD>
__device__ inline void tile_dot(float (*Xs)[kRB + 4], const float* Y, int col0, int ncols, float (*Ys)[64 + 4],
                                float acc[8][4]) {
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int k0 = 0; k0 < DD; k0 += kKC) {
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * kKC; i += 256) {
      const int c = i / kKC, k = i % kKC;
      Ys[k][c] = (col0 + c < ncols) ? Y[(size_t)(col0 + c) * DD + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kKC; ++k) {
      const float4 a0 = *reinterpret_cast<const float4*>(&Xs[k0 + k][ty * 8]);
      const float4 a1 = *reinterpret_cast<const float4*>(&Xs[k0 + k][ty * 8 + 4]);
      const float4 b = *reinterpret_cast<const float4*>(&Ys[k][tx * 4]);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
  }
}

// Row constants of Lloyd's inertia. Keys: rowconst_j = k_j G k_j. Queries (alpha_out set):
// qf_j = q_j G_k q_j, alpha_j = sqrt(C_k' / qf_j) (0 if qf_j <= 0), rowconst_j = |F_j|^2 = C_k'.
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_rowquad(const T* x, Dims D, const float* G, float* rowconst,
                                                 float* alpha_out, const KmState* kst_for_c) {
  __shared__ float Xs[DD][kRB + 4];
  __shared__ float Ys[kKC][64 + 4];
  __shared__ float red[kRB][17];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int r0 = blk * kRB;
  const T* xb = x + (size_t)bh * D.N * DD;
  const float* Gb = G + (size_t)bh * DD * DD;
  stage_rows<T, DD>(xb, D.N, r0, nullptr, Xs);
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  float part[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int c0 = 0; c0 < DD; c0 += 64) {
    float acc[8][4];
    tile_dot<DD>(Xs, Gb, c0, DD, Ys, acc);
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) part[r] = fmaf(acc[r][c], Xs[c0 + tx * 4 + c][ty * 8 + r], part[r]);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) red[ty * 8 + r][tx] = part[r];
  __syncthreads();
  if (threadIdx.x < kRB) {
    const int row = r0 + threadIdx.x;
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += red[threadIdx.x][i];
    if (row < D.N) {
      if (alpha_out) {
        const float cf = (float)kst_for_c[bh].c_final;
        const float a = s > 0.f ? sqrtf(cf / s) : 0.f;
        alpha_out[(size_t)bh * D.N + row] = a;
        rowconst[(size_t)bh * D.N + row] = s > 0.f ? cf : 0.f;
      } else {
        rowconst[(size_t)bh * D.N + row] = s;
      }
    }
  }
}

// =====================================================================================
// Lloyd iteration kernels (one run per head, all heads at once)
// =====================================================================================
// m_b = alpha x_{init_b}; G m_b and m_b G m_b; item b = 0 also resets the run state.
// Block of 256 threads; the first DD carry one coordinate each.
template <typename T, int DD>
__device__ void km_init_item(const T* x, const Dims& D, const Bufs& B, int C, const int* init, KmState* st, int b,
                             int bh) {
  __shared__ float m[DD];
  __shared__ float red[4];
  const int i = threadIdx.x;
  const int row = init[(size_t)bh * C + b];
  float v = 0.f;
  if (i < DD) {
    const float a = B.alpha ? B.alpha[(size_t)bh * D.N + row] : 1.f;
    v = a * to_f32(x[((size_t)bh * D.N + row) * DD + i]);
    m[i] = v;
  }
  __syncthreads();
  float p = 0.f;
  if (i < DD) {
    const float* G = B.metric + (size_t)bh * DD * DD;
    float t = 0.f;
    for (int k = 0; k < DD; ++k) t = fmaf(G[(size_t)k * DD + i], m[k], t);
    const size_t o = ((size_t)bh * D.C + b) * DD + i;
    B.cent[o] = v;
    B.cent_t[o] = t;
    const bf16 th = (bf16)(-2.f * t);  // the assignment's operand: -2 G m_b, hi / lo
    B.cent_h[o] = th;
    B.cent_l[o] = (bf16)(-2.f * t - (float)th);
    p = v * t;
  }
  p = wave_sum(p);
  if (lane_id() == 0) red[i / kWave] = p;
  __syncthreads();
  if (i == 0) {
    float sum = 0.f;
    for (int w = 0; w < DD / kWave; ++w) sum += red[w];
    B.cnorm[(size_t)bh * D.C + b] = sum;
    store_bias_operand(B.cent_b + ((size_t)bh * D.C + b) * 16, sum);
    B.gcount[(size_t)bh * D.C + b] = 0;  // no update has moved the centroid yet
    if (b == 0) {
      st[bh].done_iter = 0x7fffffff;
      st[bh].iters = 0;
      st[bh].c_final = C;
      st[bh].inertia[0] = st[bh].inertia[1] = 0.0;
    }
  }
  __syncthreads();
}

template <typename T, int DD>
__global__ __launch_bounds__(256) void k_km_init(const T* x, Dims D, Bufs B, int C, const int* init, KmState* st) {
  km_init_item<T, DD>(x, D, B, C, init, st, blockIdx.x, blockIdx.y);
}

// Scatter offsets, split in two launches. Per (group b, head): one wave turns the block
// counts tab[b][blk] into exclusive prefixes over the blocks and writes the group size.
__global__ __launch_bounds__(64) void k_km_scan_groups(Dims D, Bufs B, int C, KmState* st, int t) {
  const int b = blockIdx.x, bh = blockIdx.y;
  if (st[bh].done_iter < t) return;
  const int l = lane_id();
  int* tab = B.tab + ((size_t)bh * D.C + b) * D.nblk;
  int run = 0;
  for (int i0 = 0; i0 < D.nblk; i0 += kWave) {
    const int i = i0 + l;
    const int c = i < D.nblk ? (tab[i] & 255) : 0;  // the count (an update's lists also pack a start)
    const int inc = wave_incl_scan(c);
    if (i < D.nblk) tab[i] = run + inc - c;
    run += __shfl(inc, kWave - 1, kWave);
  }
  if (l == 0) B.gcount[(size_t)bh * D.C + b] = run;
}

// Per head: the inertia of assignment t, the stopping rule, and the group starts. With
// t = 0 (offsets of the final assignment of a Lloyd run, whose updates kept the books) only
// the group starts. Thread i owns groups [4i, 4i + 4).
__global__ __launch_bounds__(256) void k_km_scan_head(Dims D, Bufs B, int C, KmState* st, int t) {
  constexpr int LPT = kMaxGroups / 256;
  __shared__ long long wsl[4];
  const int bh = blockIdx.x;
  if (st[bh].done_iter < t) return;
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  long long loc[LPT], run = 0;
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int b = tid * LPT + j;
    loc[j] = run;
    run += b < C ? B.gcount[(size_t)bh * D.C + b] : 0;
  }
  long long tot;
  const long long base = block_excl_scan<256, long long>(run, &tot, wsl);
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int b = tid * LPT + j;
    if (b < C) B.gstart[(size_t)bh * (D.C + 1) + b] = (int)(base + loc[j]);
  }
  if (tid == 0) B.gstart[(size_t)bh * (D.C + 1) + C] = (int)tot;
  // t = 0: offsets of the final assignment only (the Lloyd updates kept the books)
  if (w == 0 && t > 0) {
    double sum = 0.0;
    for (int i = l; i < D.nblk; i += kWave) sum += B.ipart[(size_t)bh * D.nblk + i];
    sum = wave_sum(sum);
    if (l == 0) {
      const double prev = st[bh].inertia[(t - 1) & 1];
      int done = st[bh].done_iter;
      if (t > 1 && prev - sum <= (double)D.tol * prev) done = t;
      if (t >= D.max_iter) done = t;
      st[bh].done_iter = done;
      st[bh].inertia[t & 1] = sum;
      st[bh].iters = t;
    }
  }
}

__device__ inline void km_scatter_item(const Dims& D, const Bufs& B, KmState* st, int t, int* perm, int blk, int bh) {
  if (st[bh].done_iter < t) return;
  const int row = blk * kKmRows + threadIdx.x;
  if (threadIdx.x >= kKmRows || row >= D.N) return;
  const int lab = B.lab[(size_t)bh * D.N + row];
  const int pos = B.gstart[(size_t)bh * (D.C + 1) + lab] + B.tab[((size_t)bh * D.C + lab) * D.nblk + blk] +
                  B.rank[(size_t)bh * D.N + row];
  perm[(size_t)bh * D.N + pos] = row;
}

// The sort block's lists for the Lloyd update, 256 threads: per group its count and the
// start of the group in the block's group-ordered row list (tab, packed: count | start << 8,
// both at most kKmRows), and that list (lperm), which keeps rows of one group in index order.
// count(g) gives the block's count of group g; starts (LDS, kMaxGroups) receives the starts.
// Thread i owns groups 4i .. 4i + 3.
template <typename CountFn>
__device__ inline void km_block_lists(CountFn count, int* starts, int* ws, int C, const Dims& D, const Bufs& B, int bh,
                                      int sb, bool valid, int lab, int rank, int row) {
  int hc[4], run = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = 4 * threadIdx.x + q;
    hc[q] = g < C ? count(g) : 0;
    run += hc[q];
  }
  int tot;
  int s = block_excl_scan<256, int>(run, &tot, ws);
  static_assert(kKmRows < 256, "count and start take 8 bits each");
  int* tab = B.tab + (size_t)bh * D.C * D.nblk;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = 4 * threadIdx.x + q;
    if (g < C) {
      tab[(size_t)g * D.nblk + sb] = hc[q] | (s << 8);
      starts[g] = s;
    }
    s += hc[q];
  }
  __syncthreads();
  if (valid) B.lperm[(size_t)bh * D.N + (size_t)sb * kKmRows + starts[lab] + rank] = row;
}

// Assignment of iteration t: nearest centroid (ties to the lower id) of 128 rows, the
// block's inertia partial, and the stable in-block rank / histogram for the scatter.
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_km_assign(const T* x, Dims D, Bufs B, int C, KmState* st, int t) {
  __shared__ float Xs[DD][kRB + 4];
  __shared__ float Ys[kKC][64 + 4];
  __shared__ float bs[kRB][17];
  __shared__ int bi[kRB][17];
  __shared__ double dred[kRB];
  __shared__ int hist[kMaxGroups];
  const int blk = blockIdx.x, bh = blockIdx.y;
  if (st[bh].done_iter < t) return;
  const int r0 = blk * kRB;
  const T* xb = x + (size_t)bh * D.N * DD;
  const float* alpha = B.alpha ? B.alpha + (size_t)bh * D.N : nullptr;
  stage_rows<T, DD>(xb, D.N, r0, alpha, Xs);
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  const float* Ct = B.cent_t + (size_t)bh * D.C * DD;
  const float* cn = B.cnorm + (size_t)bh * D.C;
  float best[8];
  int bidx[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) { best[r] = INFINITY; bidx[r] = 0x7fffffff; }
  for (int c0 = 0; c0 < C; c0 += 64) {
    float acc[8][4];
    tile_dot<DD>(Xs, Ct, c0, C, Ys, acc);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = c0 + tx * 4 + c;
      if (col < C) {
        const float cnv = cn[col];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float sc = fmaf(-2.f, acc[r][c], cnv);
          if (sc < best[r] || (sc == best[r] && col < bidx[r])) { best[r] = sc; bidx[r] = col; }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) { bs[ty * 8 + r][tx] = best[r]; bi[ty * 8 + r][tx] = bidx[r]; }
  for (int i = threadIdx.x; i < C; i += 256) hist[i] = 0;
  __syncthreads();
  const int lr = threadIdx.x;  // local row for threads < 128
  const int row = r0 + lr;
  const bool valid = lr < kRB && row < D.N;
  int lab = 0;
  if (lr < kRB) {
    float b0 = INFINITY;
    int i0 = 0x7fffffff;
    for (int i = 0; i < 16; ++i) {
      const float s = bs[lr][i];
      const int j = bi[lr][i];
      if (s < b0 || (s == b0 && j < i0)) { b0 = s; i0 = j; }
    }
    lab = valid ? i0 : 0;
    dred[lr] = valid ? (double)B.rowconst[(size_t)bh * D.N + row] + (double)b0 : 0.0;
    if (valid) B.lab[(size_t)bh * D.N + row] = lab;
  }
  __syncthreads();
  // fixed-order tree reduction of the inertia partial
  for (int s = kRB / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) dred[threadIdx.x] += dred[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) B.ipart[(size_t)bh * D.nblk + blk] = dred[0];
  // stable rank: waves 0 and 1 hold rows 0..63 and 64..127 in order
  const int w = threadIdx.x / kWave;
  uint64_t mask = 0;
  if (w < 2) mask = wave_match(lab, valid, 10);
  const int rin = __popcll(mask & lanemask_lt());
  const bool leader = valid && rin == 0;
  if (w == 0 && leader) hist[lab] = __popcll(mask);
  __syncthreads();
  int rank = rin;
  if (w == 1 && valid) rank += hist[lab];
  __syncthreads();
  if (w == 1 && leader) hist[lab] += __popcll(mask);
  if (valid) B.rank[(size_t)bh * D.N + row] = rank;
  __syncthreads();
  __shared__ int scan_ws[4];
  km_block_lists([&](int g) { return hist[g]; }, hist, scan_ws, C, D, B, bh, blk, valid, lab, rank, row);
}


__global__ __launch_bounds__(kKmRows) void k_km_scatter(Dims D, Bufs B, KmState* st, int t, int* perm) {
  km_scatter_item(D, B, st, t, perm, blockIdx.x, blockIdx.y);
}

// Mean of the rows alpha_j x_j of a group, listed by `members` (group order). 256 threads:
// each 16-byte load covers EV elements, a row takes LPR lanes, RS rows are in flight per
// pass. Row r always lands in slot r % RS and the slots are summed in a fixed order, so the
// result does not depend on scheduling.
template <typename T, int DD>
__device__ void group_mean(const T* xb, const float* alpha, const int* members, int n, float* m_out,
                           float* sh /* [256 / (DD / (16 / sizeof(T)))][DD] */) {
  constexpr int EV = 16 / sizeof(T);
  constexpr int LPR = DD / EV;
  constexpr int RS = 256 / LPR;
  const int slot = threadIdx.x / LPR, c0 = (threadIdx.x % LPR) * EV;
  float acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;
  auto add_row = [&](const uint4& raw, float a) {
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] = fmaf(a, to_f32(v[e]), acc[e]);
  };
  int r = slot;
  for (; r + 7 * RS < n; r += 8 * RS) {
    int rows[8];
    uint4 raw[8];
    float al[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) rows[u] = members[r + u * RS];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      raw[u] = *reinterpret_cast<const uint4*>(xb + (size_t)rows[u] * DD + c0);
      al[u] = alpha ? alpha[rows[u]] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) add_row(raw[u], al[u]);
  }
  for (; r < n; r += RS) {
    const int row = members[r];
    add_row(*reinterpret_cast<const uint4*>(xb + (size_t)row * DD + c0), alpha ? alpha[row] : 1.f);
  }
#pragma unroll
  for (int e = 0; e < EV; ++e) sh[slot * DD + c0 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < DD) {
    float tot = 0.f;
    for (int q = 0; q < RS; ++q) tot += sh[q * DD + threadIdx.x];
    m_out[threadIdx.x] = tot / (float)n;
  }
  __syncthreads();
}

constexpr int kUpdWin = 1024;   // sort blocks per window of the update's member listing
constexpr int kUpdChunk = 1024; // members listed in LDS at a time

// Update of iteration t for group b (one block per group and head, 256 threads).
// First the stopping rule of the head: every block of the head evaluates it identically
// (the inertia of assignment t is the fixed-order sum of the sort blocks' partials, set
// against the inertia of assignment t - 1); block 0 records it. Unless the head stops at t,
// the new centroid m_b is the mean of the group's rows alpha_j x_j; with TERMS the block
// then forms G m_b and m_b G m_b itself, without it marks the group with t for
// k_km_metric_terms, which forms them next (same arithmetic). The members are read in stable group order (sort blocks in order, each
// block's rows of group b from its lists: count and start in tab, rows in lperm), listed
// in LDS a chunk at a time; member r of a chunk sits in slot r % RS and the slots are
// summed in a fixed order, so the result does not depend on scheduling.
template <typename T, int DD, bool TERMS>
__global__ __launch_bounds__(256) void k_km_update(const T* x, Dims D, Bufs B, KmState* st, int t) {
  constexpr int EV = 16 / sizeof(T);
  constexpr int LPR = DD / EV;
  constexpr int RS = 256 / LPR;
  __shared__ float sh[RS * DD];
  __shared__ float m[TERMS ? DD : 1];
  __shared__ float red[4];
  __shared__ int wpre[kUpdWin], wbeg[kUpdWin], mlist[kUpdChunk], ws[4];
  __shared__ int go;
  const int b = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  // Independent loads first, so that their latencies overlap: the head's state, the first
  // window of the group's per-block counts and (wave 0) the inertia partials, read 8 at a
  // time per lane and summed in the fixed order; the state is tested once they are all in
  // flight. (The terms under the metric G are formed by k_km_metric_terms, for 32 groups
  // per read of G.)
  const int done_iter = st[bh].done_iter;
  const double prev = st[bh].inertia[(t - 1) & 1];  // (this launch writes the other slot)
  const int* tab = B.tab + ((size_t)bh * D.C + b) * D.nblk;
  // (clamped, unconditional loads, masked afterwards: no branch between them)
  int tv0[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) tv0[q] = tab[min(4 * tid + q, D.nblk - 1)];
  const double* ip = B.ipart + (size_t)bh * D.nblk;
  double pv0[8];
  if (tid < kWave) {  // (only wave 0 sums them: the other waves would re-read the same bytes)
#pragma unroll
    for (int u = 0; u < 8; ++u) pv0[u] = ip[min(lane_id() + u * kWave, D.nblk - 1)];
  }
  asm volatile("" ::: "memory");  // (keeps the loads above ahead of the test)
  if (done_iter < t) return;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (4 * tid + q >= D.nblk) tv0[q] = 0;
  if (tid < kWave) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (lane_id() + u * kWave >= D.nblk) pv0[u] = 0.0;
    double sum = 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += pv0[u];
    for (int i0 = tid + 8 * kWave; i0 < D.nblk; i0 += 8 * kWave) {
      double pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = i0 + u * kWave < D.nblk ? ip[i0 + u * kWave] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += pv[u];
    }
    sum = wave_sum(sum);
    if (tid == 0) {
      const bool done = (t > 1 && prev - sum <= (double)D.tol * prev) || t >= D.max_iter;
      if (b == 0) {
        st[bh].inertia[t & 1] = sum;
        st[bh].iters = t;
        if (done) st[bh].done_iter = t;
      }
      go = !done;
    }
  }
  __syncthreads();
  if (!go) return;
  const T* xb = x + (size_t)bh * D.N * DD;
  const float* alpha = B.alpha ? B.alpha + (size_t)bh * D.N : nullptr;
  const int* lp = B.lperm + (size_t)bh * D.N;
  const int slot = tid / LPR, c0 = (tid % LPR) * EV;
  float acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;
  auto add_row = [&](const uint4& raw, float a) {
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] = fmaf(a, to_f32(v[e]), acc[e]);
  };
  int n = 0;
  // windows of 1024 sort blocks (thread i takes blocks 4i .. 4i + 3)
  for (int j0 = 0; j0 < D.nblk; j0 += kUpdWin) {
    int cq[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + 4 * tid + q;
      const int v = j0 == 0 ? tv0[q] : (j < D.nblk ? tab[j] : 0);
      cq[q] = v & 255;
      wbeg[4 * tid + q] = j * kKmRows + (v >> 8);
      run += cq[q];
    }
    int mw;
    int pre = block_excl_scan<256, int>(run, &mw, ws);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wpre[4 * tid + q] = pre;
      pre += cq[q];
    }
    __syncthreads();
    // members of the window, kUpdChunk at a time: listed in LDS (the last block whose prefix
    // is <= p holds member p), then gathered
    for (int p0 = 0; p0 < mw; p0 += kUpdChunk) {
      const int nc = min(kUpdChunk, mw - p0);
      for (int p = tid; p < nc; p += 256) {
        int k = 0;
#pragma unroll
        for (int step = kUpdWin / 2; step > 0; step >>= 1)
          if (wpre[k + step] <= p0 + p) k += step;
        mlist[p] = lp[wbeg[k] + (p0 + p - wpre[k])];
      }
      __syncthreads();
      int r = slot;
      for (; r + 7 * RS < nc; r += 8 * RS) {
        uint4 raw[8];
        float al[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = mlist[r + u * RS];
          raw[u] = *reinterpret_cast<const uint4*>(xb + (size_t)row * DD + c0);
          al[u] = alpha ? alpha[row] : 1.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) add_row(raw[u], al[u]);
      }
      for (; r < nc; r += RS) {
        const int row = mlist[r];
        add_row(*reinterpret_cast<const uint4*>(xb + (size_t)row * DD + c0), alpha ? alpha[row] : 1.f);
      }
      __syncthreads();
    }
    n += mw;
  }
  if (n == 0) return;  // an empty group keeps its centroid
#pragma unroll
  for (int e = 0; e < EV; ++e) sh[slot * DD + c0 + e] = acc[e];
  __syncthreads();
  if constexpr (!TERMS) {
    if (tid < DD) {
      float tot = 0.f;
      for (int q = 0; q < RS; ++q) tot += sh[q * DD + tid];
      B.cent[((size_t)bh * D.C + b) * DD + tid] = tot / (float)n;
    }
    // the mark k_km_metric_terms looks for (the group sizes are written here only after the run)
    if (tid == 0) B.gcount[(size_t)bh * D.C + b] = t;
  } else {
    // small launches: the terms here, in the order k_km_metric_terms reproduces
    constexpr int KH = 256 / DD;
    const int i = tid % DD, part = tid / DD;
    if (tid < DD) {
      float tot = 0.f;
      for (int q = 0; q < RS; ++q) tot += sh[q * DD + tid];
      m[tid] = tot / (float)n;
    }
    __syncthreads();
    float p = 0.f;
    const float* G = B.metric + (size_t)bh * DD * DD;
    float gv[DD / KH];
#pragma unroll
    for (int kk = 0; kk < DD / KH; ++kk) gv[kk] = G[(size_t)(part + kk * KH) * DD + i];
    float tt = 0.f;
#pragma unroll
    for (int kk = 0; kk < DD / KH; ++kk) tt = fmaf(gv[kk], m[part + kk * KH], tt);
    sh[tid] = tt;
    __syncthreads();
    if (tid < DD) {
      float tot = 0.f;
      for (int q = 0; q < KH; ++q) tot += sh[q * DD + i];
      const size_t o = ((size_t)bh * D.C + b) * DD + i;
      B.cent[o] = m[i];
      B.cent_t[o] = tot;
      const bf16 th = (bf16)(-2.f * tot);  // the assignment's operand: -2 G m_b, hi / lo
      B.cent_h[o] = th;
      B.cent_l[o] = (bf16)(-2.f * tot - (float)th);
      p = m[i] * tot;
    }
    p = wave_sum(p);
    if (lane_id() == 0) red[tid / kWave] = p;
    __syncthreads();
    if (tid == 0) {
      float sum = 0.f;
      for (int w = 0; w < DD / kWave; ++w) sum += red[w];
      B.cnorm[(size_t)bh * D.C + b] = sum;
      store_bias_operand(B.cent_b + ((size_t)bh * D.C + b) * 16, sum);
    }
  }
}

// The metric terms of the centroids that iteration t's update moved (marked with t): G m_b,
// -2 G m_b as the assignment's bf16 hi / lo operands, m_b G m_b and its bias operand. One
// workgroup per 32 groups of a head reads G once (the update's workgroups read it once per
// group). Each entry of G m_b is formed in the order the update uses on small launches:
// KH = 256 / DD partial chains over k = q + KH kk (kk ascending), added q = 0, 1, ... to 0;
// m_b G m_b sums m_i (G m_b)_i over 64-lane halves by the same butterfly, the halves in
// order. Threads take 4 groups x DD / 32 dims, so every G row read from LDS feeds 4 groups.
template <int DD>
__global__ __launch_bounds__(256) void k_km_metric_terms(Dims D, Bufs B, int C, const KmState* st, int t) {
  constexpr int GB = 32, KH = 256 / DD, DPT = DD / 32;
  constexpr int GH = DD / 2;  // rows of G staged at a time (two halves: three workgroups fit a CU)
  __shared__ __attribute__((aligned(16))) float Gs[GH * DD];  // half of G, then G m_b of the groups
  __shared__ __attribute__((aligned(16))) float mT[DD][GB];   // m_b, transposed
  __shared__ int mark[GB];
  const int bh = blockIdx.y, g0 = blockIdx.x * GB, tid = threadIdx.x;
  if (st[bh].done_iter < t) return;  // the head stopped before iteration t: no update ran
  if (tid < GB) mark[tid] = g0 + tid < C && B.gcount[(size_t)bh * D.C + g0 + tid] == t;
  const int any = __syncthreads_or(tid < GB && mark[tid]);
  if (!any) return;
  const float* G = B.metric + (size_t)bh * DD * DD;
  for (int e = tid; e < GB * DD; e += 256) {
    const int gl = e / DD, k = e % DD;
    mT[k][gl] = mark[gl] ? B.cent[((size_t)bh * D.C + g0 + gl) * DD + k] : 0.f;
  }
  const int gq = tid / 32, dq = tid % 32;  // groups 4 gq .. 4 gq + 3, dims DPT dq .. DPT dq + DPT - 1
  float acc[KH][4][DPT];
#pragma unroll
  for (int q = 0; q < KH; ++q)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < DPT; ++j) acc[q][g][j] = 0.f;
  // rows k of G in two halves; each chain still takes its k in ascending order
  for (int hf = 0; hf < 2; ++hf) {
    if (hf) __syncthreads();  // the first half's reads are done
    for (int e = tid; e < GH * DD / 4; e += 256)
      reinterpret_cast<float4*>(Gs)[e] = reinterpret_cast<const float4*>(G + (size_t)hf * GH * DD)[e];
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < GH / KH; ++kk) {
#pragma unroll
      for (int q = 0; q < KH; ++q) {
        const int kl = q + KH * kk, k = hf * GH + kl;
        float gv[DPT];
        if constexpr (DPT == 4) {
          const float4 v = *reinterpret_cast<const float4*>(&Gs[kl * DD + 4 * dq]);
          gv[0] = v.x; gv[1] = v.y; gv[2] = v.z; gv[3] = v.w;
        } else {
          const float2 v = *reinterpret_cast<const float2*>(&Gs[kl * DD + 2 * dq]);
          gv[0] = v.x; gv[1] = v.y;
        }
        const float4 mv4 = *reinterpret_cast<const float4*>(&mT[k][4 * gq]);
        const float mv[4] = {mv4.x, mv4.y, mv4.z, mv4.w};
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int j = 0; j < DPT; ++j) acc[q][g][j] = fmaf(gv[j], mv[g], acc[q][g][j]);
      }
    }
  }
  __syncthreads();  // every read of G is done: Gs takes G m_b, [group][dim]
  float* tT = Gs;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
      float tot = 0.f;
#pragma unroll
      for (int q = 0; q < KH; ++q) tot += acc[q][g][j];
      tT[(4 * gq + g) * DD + DPT * dq + j] = tot;
    }
  __syncthreads();
  // operands, and m_b G m_b: wave w takes groups w, w + 4, ...
  const int w = tid / kWave, l = lane_id();
  for (int gl = w; gl < GB; gl += 4) {
    if (!mark[gl]) continue;  // (uniform over the wave)
    const size_t ob = ((size_t)bh * D.C + g0 + gl) * DD;
    float sum = 0.f;
#pragma unroll
    for (int hh = 0; hh < DD / kWave; ++hh) {
      const int i = hh * kWave + l;
      const float tot = tT[gl * DD + i];
      B.cent_t[ob + i] = tot;
      const bf16 th = (bf16)(-2.f * tot);
      B.cent_h[ob + i] = th;
      B.cent_l[ob + i] = (bf16)(-2.f * tot - (float)th);
      sum += wave_sum(mT[i][gl] * tot);
    }
    if (l == 0) {
      B.cnorm[(size_t)bh * D.C + g0 + gl] = sum;
      store_bias_operand(B.cent_b + ((size_t)bh * D.C + g0 + gl) * 16, sum);
    }
  }
}

// Warm start (paper Table C.1: a first k-means of up to 25 iterations, 2 for subsequent
// calls). Centroid b starts from the d-dimensional representative reps[b] of the previous
// plan (key groups: mean key; query groups: mean of alpha q), which is what the metric form
// needs: G m_b and m_b G m_b under the current metric. Only the prev[bh].c_final groups the
// previous plan realised are live; the other slots score +inf, never win an assignment and
// are dropped again at compaction.
template <int DD>
__global__ __launch_bounds__(256) void k_km_warm_init(Dims D, Bufs B, const float* reps, int rep_groups,
                                                       const KmState* prev) {
  __shared__ float m[DD];
  __shared__ float red[4];
  const int b = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  const bool live = b < prev[bh].c_final;
  if (i < DD) m[i] = live ? reps[((size_t)bh * rep_groups + b) * DD + i] : 0.f;
  __syncthreads();
  float p = 0.f;
  if (i < DD) {
    const float* G = B.metric + (size_t)bh * DD * DD;
    float t = 0.f;
    for (int k = 0; k < DD; ++k) t = fmaf(G[(size_t)k * DD + i], m[k], t);
    const size_t o = ((size_t)bh * D.C + b) * DD + i;
    B.cent[o] = m[i];
    B.cent_t[o] = t;
    const bf16 th = (bf16)(-2.f * t);  // the assignment's operand: -2 G m_b, hi / lo
    B.cent_h[o] = th;
    B.cent_l[o] = (bf16)(-2.f * t - (float)th);
    p = m[i] * t;
  }
  p = wave_sum(p);
  if (lane_id() == 0) red[i / kWave] = p;
  __syncthreads();
  if (i == 0) {
    float sum = 0.f;
    for (int w = 0; w < DD / kWave; ++w) sum += red[w];
    B.cnorm[(size_t)bh * D.C + b] = live ? sum : INFINITY;
    store_bias_operand(B.cent_b + ((size_t)bh * D.C + b) * 16, live ? sum : INFINITY);
    B.gcount[(size_t)bh * D.C + b] = 0;  // no update has moved the centroid yet
  }
}

// Drop empty groups: compacted labels, offsets and the realised group count.
__global__ __launch_bounds__(1024) void k_km_compact(Dims D, Bufs B, int C, KmState* st, int* lab_out,
                                                     int* off_out, int off_stride) {
  __shared__ int ws[16];
  __shared__ int newid[kMaxGroups];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int cnt = tid < C ? B.gcount[(size_t)bh * D.C + tid] : 0;
  int tot;
  const int id = block_excl_scan<1024, int>(cnt > 0 ? 1 : 0, &tot, ws);
  if (tid < C) {
    newid[tid] = id;
    if (cnt > 0) off_out[(size_t)bh * off_stride + id] = B.gstart[(size_t)bh * (D.C + 1) + tid];
  }
  if (tid == 0) {
    off_out[(size_t)bh * off_stride + tot] = D.N;
    st[bh].c_final = tot;
  }
  __syncthreads();
  for (int j = tid; j < D.N; j += 1024)
    lab_out[(size_t)bh * D.N + j] = newid[B.lab[(size_t)bh * D.N + j]];
}

// Key-space centroid of each compacted key group (raw keys, group order).
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_key_centroids(const T* k, Dims D, Bufs B) {
  __shared__ float sh[2048];
  __shared__ float m[DD];
  const int b = blockIdx.x, bh = blockIdx.y;
  if (b >= B.kst[bh].c_final) return;
  const int* off = B.koff + (size_t)bh * (D.Ck + 1);
  const int s0 = off[b], n = off[b + 1] - off[b];
  group_mean<T, DD>(k + (size_t)bh * D.N * DD, nullptr, B.kperm + (size_t)bh * D.N + s0, n, m, sh);
  if (threadIdx.x < DD) {
    const size_t o = ((size_t)bh * D.Ck + b) * DD + threadIdx.x;
    const float v = m[threadIdx.x];
    B.kcent[o] = v;
    const bf16 vh = (bf16)v;
    B.kcent_h[o] = vh;
    B.kcent_l[o] = (bf16)(v - (float)vh);
  }
}

// Query-group representative: mean of alpha_i q_i over the compacted group (the query
// features are F_i = alpha_i q_i C_k^T, so a group's feature mean is this times C_k^T).
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_query_reps(const T* q, Dims D, Bufs B) {
  __shared__ float sh[2048];
  __shared__ float m[DD];
  const int a = blockIdx.x, bh = blockIdx.y;
  if (a >= B.qst[bh].c_final) return;
  const int* off = B.qoff + (size_t)bh * (D.Cq + 1);
  const int s0 = off[a], n = off[a + 1] - off[a];
  group_mean<T, DD>(q + (size_t)bh * D.N * DD, B.alpha ? B.alpha + (size_t)bh * D.N : nullptr,
                    B.qperm + (size_t)bh * D.N + s0, n, m, sh);
  if (threadIdx.x < DD) B.qcent[((size_t)bh * D.Cq + a) * DD + threadIdx.x] = m[threadIdx.x];
}

// =====================================================================================
// bf16 inputs: the same products on the matrix cores. A small float matrix Y (centroids,
// metric, key centroids) is split as Y = hi + lo with hi, lo bf16, so hi.x + lo.x carries
// ~16 significant bits of Y against the exact bf16 row x. Products are taken transposed,
// acc = Y_block x^T with v_mfma_f32_32x32x16_bf16, so lane l owns row (l % 32) and holds
// 16 of the 32 Y rows: Y row 8(v/4) + 4(l/32) + (v%4) in acc[v].
// =====================================================================================
template <int DD>
__device__ inline void load_row_operand(const bf16* xrow, bf16x8* xr) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int c = 0; c < DD / 16; ++c) xr[c] = *reinterpret_cast<const bf16x8*>(xrow + 16 * c + 8 * h);
}

// Y rows [r0, r0 + R) (float, row stride DD) -> Yh / Yl (bf16, row stride DD + 8); zero past nrows.
template <int DD, int R>
__device__ inline void stage_hilo(const float* Y, int r0, int nrows, bf16* Yh, bf16* Yl) {
  constexpr int KS = DD + 8;
  for (int e = threadIdx.x; e < R * DD / 4; e += blockDim.x) {
    const int r = e / (DD / 4), c4 = (e % (DD / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + r < nrows) v = *reinterpret_cast<const float4*>(Y + (size_t)(r0 + r) * DD + c4);
    const float f[4] = {v.x, v.y, v.z, v.w};
    bf16x4 hv, lv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16 hb = (bf16)f[q];
      hv[q] = hb;
      lv[q] = (bf16)(f[q] - (float)hb);
    }
    *reinterpret_cast<bf16x4*>(&Yh[r * KS + c4]) = hv;
    *reinterpret_cast<bf16x4*>(&Yl[r * KS + c4]) = lv;
  }
}

// Rows [r0, r0 + R) of a bf16 hi/lo pair (row stride DD) -> Yh / Yl (row stride DD + 8); zero past nrows.
template <int DD, int R>
__device__ inline void copy_hilo(const bf16* Sh, const bf16* Sl, int r0, int nrows, bf16* Yh, bf16* Yl) {
  constexpr int KS = DD + 8;
  for (int e = threadIdx.x; e < R * DD / 8; e += blockDim.x) {
    const int r = e / (DD / 8), c8 = (e % (DD / 8)) * 8;
    bf16x8 hv, lv;
    if (r0 + r < nrows) {
      hv = *reinterpret_cast<const bf16x8*>(Sh + (size_t)(r0 + r) * DD + c8);
      lv = *reinterpret_cast<const bf16x8*>(Sl + (size_t)(r0 + r) * DD + c8);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) { hv[q] = (bf16)0.f; lv[q] = (bf16)0.f; }
    }
    *reinterpret_cast<bf16x8*>(&Yh[r * KS + c8]) = hv;
    *reinterpret_cast<bf16x8*>(&Yl[r * KS + c8]) = lv;
  }
}

template <int DD>
__device__ inline f32x16 mfma_rows(const bf16* Yh, const bf16* Yl, int y0, const bf16x8* xr) {
  constexpr int KS = DD + 8;
  const int l32 = lane_id() & 31, h = lane_id() >> 5;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int c = 0; c < DD / 16; ++c) {
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Yh[(y0 + l32) * KS + 16 * c + 8 * h]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xr[c], acc, 0, 0, 0);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Yl[(y0 + l32) * KS + 16 * c + 8 * h]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xr[c], acc, 0, 0, 0);
  }
  return acc;
}

__device__ inline int acc_row(int v) { return 8 * (v >> 2) + 4 * (lane_id() >> 5) + (v & 3); }

// The same products with the operands swapped: lane l holds row y0 + l % 32 of Y against
// the rows acc_row(v) of the wave's x operand.
template <int DD>
__device__ inline f32x16 mfma_cols(const bf16* Yh, const bf16* Yl, int y0, const bf16x8* xr) {
  constexpr int KS = DD + 8;
  const int l32 = lane_id() & 31, h = lane_id() >> 5;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
  for (int c = 0; c < DD / 16; ++c) {
    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Yh[(y0 + l32) * KS + 16 * c + 8 * h]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xr[c], bh, acc, 0, 0, 0);
    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Yl[(y0 + l32) * KS + 16 * c + 8 * h]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xr[c], bl, acc, 0, 0, 0);
  }
  return acc;
}

// Assignment of iteration t for 128*RS rows: each of the 4 waves owns RS sets of 32 rows, so
// every centroid operand read from LDS feeds RS products. Centroid operands (-2 G m_b in
// bf16, plus its bf16 remainder when LO, and the bias operands) are double-buffered in LDS 64
// centroids at a time: the next chunk's global loads are issued before the current chunk's
// products. The plan runs RS = 1 (four waves per SIMD), and RS = 2 (half the LDS operand
// reads per product) with the remainder operand.
template <int DD, int RS, bool LO>
__global__ __launch_bounds__(256, RS == 1 ? 4 : 2) void k_km_assign_bf16(const bf16* x, Dims D, Bufs B, int C,
                                                                           KmState* st, int t) {
  constexpr int CB = 64, KS = DD + 8;
  constexpr int NL = CB * DD / 8 / 256;  // 16-byte loads per thread per chunk and operand
  constexpr int NO = LO ? 2 : 1;
  // the centroid operands; after the last chunk the same bytes hold the per-wave label counts
  constexpr size_t YB = sizeof(bf16) * 2 * NO * CB * KS, CNB = sizeof(int) * RS * 4 * kMaxGroups;
  __shared__ __attribute__((aligned(16))) char smem[YB > CNB ? YB : CNB];
  auto Y = reinterpret_cast<bf16(*)[NO][CB * KS]>(smem);
  auto cnt = reinterpret_cast<int(*)[4][kMaxGroups]>(smem);
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][CB * 16];  // bias operands of the chunk
  __shared__ double wpart[RS][4];
  const int sb0 = blockIdx.x * RS, bh = blockIdx.y;  // first 128-row sort block
  if (st[bh].done_iter < t) return;
  const int tid = threadIdx.x, w = tid / kWave, l32 = lane_id() & 31, h = lane_id() >> 5;
  const int r0 = sb0 * kKmRows;
  bf16x8 xr[RS][DD / 16];
  // Every product is the squared distance divided by the row's scale alpha (> 0), whose
  // argmin is the nearest centroid: d / alpha = x . (-2 G m_b) + m_b G m_b / alpha + rc / alpha
  // (rc = alpha^2 x G x, the row constant). The first term is the main products (the
  // centroid operand holds -2 G m_b); the other two come from one more product per 32
  // centroids, of k-slots [cn_hi, cn_hi, cn_lo, 1, 1] (centroid side) and [ia_hi, ia_lo,
  // ia_hi, rca_hi, rca_lo] (row side, ia = 1 / alpha, rca = rc / alpha, bf16 hi / lo pairs),
  // so no vector op touches a product. The value is >= 0 up to rounding, so its float bits
  // order like integers; the low 10 bits are replaced by the centroid index (the part shared
  // by both lane halves), and one integer min per pair of candidates keeps the nearest, the
  // lower index among distances equal in the kept bits. A row with alpha = 0 (its features
  // are 0) takes a zero operand and scale 1: its value is m_b G m_b.
  float sca[RS];  // alpha (1 for a zero row), to turn the kept value back into a distance
  int bkey[RS];
  bf16x8 brow[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int row = r0 + 128 * rs + 32 * w + l32;
    const bool valid = row < D.N;
    load_row_operand<DD>(x + ((size_t)bh * D.N + (valid ? row : D.N - 1)) * DD, xr[rs]);
    const float al = B.alpha ? B.alpha[(size_t)bh * D.N + (valid ? row : 0)] : 1.f;
    const float rc = B.rowconst[(size_t)bh * D.N + (valid ? row : 0)];
    const bool zero = !(al > 0.f);
    if (__builtin_amdgcn_ballot_w64(zero)) {  // (rare; no register copies on the common path)
#pragma unroll
      for (int c = 0; c < DD / 16; ++c) xr[rs][c] = zero ? bf16x8{} : xr[rs][c];
    }
    // 1 / alpha to within an ulp: its bf16 hi / lo pair below carries about 16 bits of it
    const float ia = zero ? 1.f : __builtin_amdgcn_rcpf(al), rca = zero ? 0.f : rc * ia;
    sca[rs] = zero ? 1.f : al;
    const bf16 iah = (bf16)ia, rch = (bf16)rca;
    const bf16 ial = (bf16)(ia - (float)iah), rcl = (bf16)(rca - (float)rch);
    brow[rs] = bf16x8{};
    if (h == 0) {
      brow[rs][0] = iah;
      brow[rs][1] = ial;
      brow[rs][2] = iah;
      brow[rs][3] = rch;
      brow[rs][4] = rcl;
    }
    bkey[rs] = 0x7fffffff;
  }
  const bf16* Cop[2] = {B.cent_h + (size_t)bh * D.C * DD, B.cent_l + (size_t)bh * D.C * DD};
  const bf16* Cb = B.cent_b + (size_t)bh * D.C * 16;
  bf16x8 pre[NO][NL], pb;
  // Centroids past the last one (the tail of the last chunk) re-read the last centroid's
  // operand, so every load is unconditional; their bias operand is [+inf, 0, ...], which makes
  // their value +inf, and they never win.
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int e = tid + 256 * i, r = e / (DD / 8), c8 = (e % (DD / 8)) * 8;
        pre[o][i] = *reinterpret_cast<const bf16x8*>(Cop[o] + (size_t)min(c0 + r, C - 1) * DD + c8);
      }
    // threads 0 .. 2 CB - 1: half tid % 2 of the bias operand of centroid c0 + tid / 2
    pb = *reinterpret_cast<const bf16x8*>(Cb + (size_t)min(c0 + (tid & (2 * CB - 1)) / 2, C - 1) * 16 + 8 * (tid & 1));
    if (c0 + (tid & (2 * CB - 1)) / 2 >= C) {
      pb = bf16x8{};
      if ((tid & 1) == 0) pb[0] = (bf16)INFINITY;
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int e = tid + 256 * i, r = e / (DD / 8), c8 = (e % (DD / 8)) * 8;
        *reinterpret_cast<bf16x8*>(&Y[buf][o][r * KS + c8]) = pre[o][i];
      }
    if (tid < 2 * CB) *reinterpret_cast<bf16x8*>(&Bs[buf][8 * tid]) = pb;
  };
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  int cur = 0;
  for (int c0 = 0; c0 < C; c0 += CB) {
    const bool more = c0 + CB < C;
    if (more) load_chunk(c0 + CB);
#pragma unroll
    for (int yb = 0; yb < CB; yb += 32) {
      // the centroid side of the bias product (k-slots 8 h .. 8 h + 7 of the 16)
      const bf16x8 bcen = *reinterpret_cast<const bf16x8*>(&Bs[cur][(yb + l32) * 16 + 8 * h]);
      f32x16 acc[RS];
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        const f32x16 z = {};
        acc[rs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bcen, brow[rs], z, 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < DD / 16; ++c) {
#pragma unroll
        for (int o = 0; o < NO; ++o) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Y[cur][o][(yb + l32) * KS + 16 * c + 8 * h]);
#pragma unroll
          for (int rs = 0; rs < RS; ++rs)
            acc[rs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, xr[rs][c], acc[rs], 0, 0, 0);
        }
      }
      // Candidate key = value bits with the low 10 replaced by c0 + yb + 8 (v / 4) + v % 4
      // (the index without the lane-half offset 4 h, which the merge of the halves restores).
      // (a bit-field insert per candidate: the mask is kept in a register)
      int im = 1023;
      asm volatile("" : "+v"(im));
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int i0 = c0 + yb + 8 * (v >> 2) + (v & 3), i1 = i0 + 1;
          const int k0 = (__float_as_int(acc[rs][v]) & ~im) | (i0 & im);
          const int k1 = (__float_as_int(acc[rs][v + 1]) & ~im) | (i1 & im);
          bkey[rs] = min(min(bkey[rs], k0), k1);
        }
    }
    if (more) store_chunk(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }
  // Tail, one barrier: labels; the inertia partial of each sort block (wave sums, then the
  // four waves in order); the stable in-block rank = rank among the wave's rows with the same
  // label + the counts of that label in the earlier waves; the block's label histogram.
  uint32_t mk[RS];  // lanes 0 .. 31 hold the rows
  int lab[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    // merge the halves: the smaller key wins; on equal keys the lower index, half 0
    const int ok = __shfl_xor(bkey[rs], 32, kWave), myk = bkey[rs];
    const int wk = min(ok, myk);
    const int wh = ok < myk ? (h ^ 1) : (ok == myk ? 0 : h);
    const int bidx = (wk & 1023) + 4 * wh;
    const float bestd = sca[rs] * __int_as_float(wk & ~1023);  // the squared distance
    const int row = r0 + 128 * rs + 32 * w + l32;
    const bool valid = h == 0 && row < D.N;
    lab[rs] = valid ? bidx : 0;
    if (valid) B.lab[(size_t)bh * D.N + row] = bidx;
    double v = valid ? (double)bestd : 0.0;
    v = wave_sum(v);
    if (lane_id() == 0) wpart[rs][w] = v;
    mk[rs] = wave_match_lo(lab[rs], valid, 10);
    // this wave's counts (zeroed, then one leader per label writes; one wave, in order)
    int* cw = cnt[rs][w];
    for (int i = lane_id(); i < C; i += kWave) cw[i] = 0;
    if (valid && __popc(mk[rs] & (uint32_t)lanemask_lt()) == 0) cw[lab[rs]] = __popc(mk[rs]);
  }
  __syncthreads();
  int rk[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int sb = sb0 + rs;
    const int row = r0 + 128 * rs + 32 * w + l32;
    rk[rs] = __popc(mk[rs] & (uint32_t)lanemask_lt());
    for (int w2 = 0; w2 < w; ++w2) rk[rs] += cnt[rs][w2][lab[rs]];
    if (h == 0 && row < D.N) B.rank[(size_t)bh * D.N + row] = rk[rs];
    if (tid == 0 && sb < D.nblk)
      B.ipart[(size_t)bh * D.nblk + sb] = ((wpart[rs][0] + wpart[rs][1]) + wpart[rs][2]) + wpart[rs][3];
  }
  // the lists for the update; the block's starts overwrite the first wave's counts once every
  // count of that row set has been read (the scan's barriers)
  __shared__ int scan_ws[4];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int sb = sb0 + rs;
    if (sb >= D.nblk) break;
    const int row = r0 + 128 * rs + 32 * w + l32;
    km_block_lists([&](int g) { return cnt[rs][0][g] + cnt[rs][1][g] + cnt[rs][2][g] + cnt[rs][3][g]; }, cnt[rs][0],
                   scan_ws, C, D, B, bh, sb, h == 0 && row < D.N, lab[rs], rk[rs], row);
  }
}

// Row constants (see k_rowquad) on the matrix cores: (G x)_i for 32 dims at a time, dotted
// with x in the lane that owns the row. G (bf16 hi / lo) is staged in LDS once per
// workgroup, which then takes the 128-row blocks blockIdx.x, + gridDim.x, ... of its head;
// the next block's rows are loaded while the current block's products run. Lane l32
// supplies G row 32 ib + pi(l32) (bits 2 and 3 of the index swapped), so the 16 dims whose
// (G x) a lane half receives are the ones its own share of the row operand holds (G is
// symmetric, but any row order works: only the pairing of (G x)_i with x_i matters).
template <int DD>
__global__ __launch_bounds__(256, 2) void k_rowquad_bf16(const bf16* x, Dims D, const bf16* Gsh, const bf16* Gsl,
                                                         float* rowconst, float* alpha_out,
                                                         const KmState* kst_for_c) {
  constexpr int KS = DD + 8;
  __shared__ __attribute__((aligned(16))) bf16 Gh[DD * KS];
  __shared__ __attribute__((aligned(16))) bf16 Gl[DD * KS];
  const int bh = blockIdx.y;
  const int w = threadIdx.x / kWave, l32 = lane_id() & 31, h = lane_id() >> 5;
  const bf16* xb = x + (size_t)bh * D.N * DD;
  auto row_of = [&](int blk) { return min(blk * kKmRows + 32 * w + l32, D.N - 1); };
  bf16x8 xr[DD / 16], xn[DD / 16];
  load_row_operand<DD>(xb + (size_t)row_of(blockIdx.x) * DD, xr);
  copy_hilo<DD, DD>(Gsh + (size_t)bh * DD * DD, Gsl + (size_t)bh * DD * DD, 0, DD, Gh, Gl);
  __syncthreads();
  const float cf = alpha_out ? (float)kst_for_c[bh].c_final : 0.f;
  const int prow = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);  // pi(l32)
  for (int blk = blockIdx.x; blk < D.nblk; blk += gridDim.x) {
    const int row = blk * kKmRows + 32 * w + l32;
    // the next block's rows (past the last block the current rows again: no branch)
    const int nx = blk + gridDim.x;
    load_row_operand<DD>(xb + (size_t)row_of(nx < D.nblk ? nx : blk) * DD, xn);
    // (the G operand reads are the same every block: a zero offset the compiler cannot see
    // through keeps them from being hoisted into registers)
    int z = 0;
    asm volatile("" : "+v"(z));
    float part = 0.f;
#pragma unroll
    for (int ib = 0; ib < DD / 32; ++ib) {
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int c = 0; c < DD / 16; ++c) {
        const int o = (32 * ib + prow) * KS + 16 * c + 8 * h + z;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(&Gh[o]), xr[c], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(&Gl[o]), xr[c], acc, 0, 0, 0);
      }
      // acc[4 g + r] = (G x)_i, i = 32 ib + pi(8 g + 4 h + r) = 32 ib + 16 (g >> 1) + 8 h + 4 (g & 1) + r:
      // element 4 (g & 1) + r of the lane's operand chunk 2 ib + (g >> 1)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) part = fmaf(acc[4 * g + r], (float)xr[2 * ib + (g >> 1)][4 * (g & 1) + r], part);
    }
    part += __shfl_xor(part, 32, kWave);
    if (h == 0 && row < D.N) {
      const size_t o = (size_t)bh * D.N + row;
      if (alpha_out) {
        alpha_out[o] = part > 0.f ? sqrtf(cf / part) : 0.f;
        rowconst[o] = part > 0.f ? cf : 0.f;
      } else {
        rowconst[o] = part;
      }
    }
#pragma unroll
    for (int c = 0; c < DD / 16; ++c) xr[c] = xn[c];
  }
}

// Group masses over attention tiles (128 rows of one query group, four waves each; TPB
// consecutive tiles per workgroup, so that each staged centroid chunk serves 128 TPB rows):
// pass 1 finds each row's softmax max and sum over the key groups, pass 2 adds the
// normalised masses into per-tile column sums (rows reduced inside the wave, the tile's
// waves in a fixed order).
template <int DD, int TPB>
__global__ __launch_bounds__(256 * TPB) void k_group_mass_bf16(const bf16* q, Dims D, Bufs B) {
  constexpr int CB = 64, KS = DD + 8, NT = 256 * TPB;
  __shared__ __attribute__((aligned(16))) bf16 Yh[CB * KS];
  __shared__ __attribute__((aligned(16))) bf16 Yl[CB * KS];
  __shared__ float lg[kMaxGroups];
  __shared__ float colw[TPB][4][CB];
  __shared__ float rowm[TPB][128], rowinv[TPB][128];
  const int bh = blockIdx.y, nt = B.ntiles[bh];
  if (blockIdx.x * TPB >= nt) return;  // (uniform over the workgroup)
  const int tid = threadIdx.x, w = tid / kWave, l32 = lane_id() & 31;
  const int k = w >> 2, wl = w & 3;  // this wave's tile in the workgroup, and its wave there
  const int t = blockIdx.x * TPB + k;
  const bool tile_ok = t < nt;
  const int2 tl = B.tiles[(size_t)bh * D.max_tiles + (tile_ok ? t : blockIdx.x * TPB)];
  const int a = tl.x, pos0 = tl.y;
  const int rows = tile_ok ? min(D.qt, B.qoff[(size_t)bh * (D.Cq + 1) + a + 1] - pos0) : 0;
  const int lrow = 32 * wl + l32;
  const bool valid = lrow < rows;
  const int tok = B.qperm[(size_t)bh * D.N + pos0 + (valid ? lrow : 0)];
  bf16x8 xr[DD / 16];
  load_row_operand<DD>(q + ((size_t)bh * D.N + tok) * DD, xr);
  const int Ck = B.kst[bh].c_final;
  const int* ko = B.koff + (size_t)bh * (D.Ck + 1);
  // log2 of the group sizes; -inf past the last group, so that a padded centroid (zero
  // operand) scores -inf with no test (every read below stays inside the array: C_k <=
  // kMaxGroups, a multiple of the 64-centroid chunk)
  for (int b = tid; b < kMaxGroups; b += NT) lg[b] = b < Ck ? log2f((float)(ko[b + 1] - ko[b])) : -INFINITY;
  const bf16* Kh = B.kcent_h + (size_t)bh * D.Ck * DD;
  const bf16* Kl = B.kcent_l + (size_t)bh * D.Ck * DD;
  const float sc2 = D.scale * 1.4426950408889634f;  // logits in the log2 domain
  // a wave past its tile's last row (or in a workgroup's missing last tile) only helps stage
  // the centroids: its products, which no row would use, are skipped
  const bool live = 32 * wl < rows;
  float m = -INFINITY, ssum = 0.f;
  for (int c0 = 0; c0 < Ck; c0 += CB) {  // pass 1
    __syncthreads();
    copy_hilo<DD, CB>(Kh, Kl, c0, Ck, Yh, Yl);
    __syncthreads();
    if (!live) continue;
#pragma unroll
    for (int yb = 0; yb < CB; yb += 32) {
      const f32x16 acc = mfma_rows<DD>(Yh, Yl, yb, xr);
      float z[16], mx = m;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        z[v] = fmaf(sc2, acc[v], lg[c0 + yb + acc_row(v)]);
        mx = fmaxf(mx, z[v]);
      }
      // a lane half whose 16 centroids are all past the last group (C_k' <= 4) has no
      // score yet: shift by 0 instead of -inf, so its terms are exp2(-inf) = 0, not NaN
      const float sh = mx == -INFINITY ? 0.f : mx;
      float add = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) add += __builtin_amdgcn_exp2f(z[v] - sh);
      ssum = ssum * __builtin_amdgcn_exp2f(m - sh) + add;
      m = mx;
    }
  }
  {
    const float mo = __shfl_xor(m, 32, kWave), so = __shfl_xor(ssum, 32, kWave);
    const float mm = fmaxf(m, mo);  // finite on a live wave: lane half 0 holds centroid 0
    ssum = ssum * __builtin_amdgcn_exp2f(m - mm) + so * __builtin_amdgcn_exp2f(mo - mm);
    m = mm;
  }
  const float inv = valid ? 1.f / ssum : 0.f;  // (a dead wave's rows are never read below)
  // pass 2 with the operands swapped, so that a lane holds one centroid against 16 rows and
  // the column sums are in-lane: the rows' max and 1 / sum come from LDS
  if (lane_id() < 32) {
    rowm[k][lrow] = m;
    rowinv[k][lrow] = inv;
  }
  float* part = B.mass_part + ((size_t)bh * D.max_tiles + t) * D.Ck;
  const int ttid = tid & 255;  // thread index within the tile's four waves
  for (int c0 = 0; c0 < Ck; c0 += CB) {  // pass 2
    __syncthreads();
    copy_hilo<DD, CB>(Kh, Kl, c0, Ck, Yh, Yl);
    __syncthreads();
#pragma unroll
    for (int yb = 0; yb < CB; yb += 32) {
      if (!live) {
        if (lane_id() < 32) colw[k][wl][yb + l32] = 0.f;
        continue;
      }
      const f32x16 acc = mfma_cols<DD>(Yh, Yl, yb, xr);
      // (a column past the last group has lg = -inf: its terms are exp2(-inf) = 0)
      const float lgc = lg[c0 + yb + l32];
      float cs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * wl + acc_row(v);
        cs += __builtin_amdgcn_exp2f(fmaf(sc2, acc[v], lgc) - rowm[k][r]) * rowinv[k][r];
      }
      cs += xor32(cs);
      if (lane_id() < 32) colw[k][wl][yb + l32] = cs;
    }
    __syncthreads();
    if (tile_ok && ttid < CB && c0 + ttid < Ck)
      part[c0 + ttid] = ((colw[k][0][ttid] + colw[k][1][ttid]) + colw[k][2][ttid]) + colw[k][3][ttid];
  }
}

// u[a][b] = rint(2^32 * mean over the group's rows of the masses), tiles summed in order.
__global__ __launch_bounds__(256) void k_group_mass_final(Dims D, Bufs B) {
  const int a = blockIdx.x, bh = blockIdx.y;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  if (a >= Cq) return;
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const int n = qo[a + 1] - qo[a];
  const int t0 = B.tstart[(size_t)bh * (D.Cq + 1) + a], t1 = B.tstart[(size_t)bh * (D.Cq + 1) + a + 1];
  const float* part = B.mass_part + (size_t)bh * D.max_tiles * D.Ck;
  long long* u = B.u + ((size_t)bh * D.Cq + a) * D.Ck;
  for (int b = threadIdx.x; b < Ck; b += 256) {
    double sum = 0.0;
    for (int t = t0; t < t1; ++t) sum += (double)part[(size_t)t * D.Ck + b];
    u[b] = (long long)rint(sum / (double)n * 4294967296.0);
  }
}

// =====================================================================================
// Labels given by the caller: copy into the working label buffer and histogram them
// through the same scan / scatter as a converged Lloyd run.
// =====================================================================================
__global__ __launch_bounds__(kKmRows) void k_labels_given(const int* labels, Dims D, Bufs B, KmState* st) {
  __shared__ int hist[kMaxGroups];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int C = st[bh].c_final;  // requested count (set by the host-side reset)
  for (int i = threadIdx.x; i < C; i += kKmRows) hist[i] = 0;
  __syncthreads();
  const int row = blk * kKmRows + threadIdx.x;
  const bool valid = row < D.N;
  int lab = valid ? labels[(size_t)bh * D.N + row] : 0;
  lab = min(max(lab, 0), C - 1);
  if (valid) B.lab[(size_t)bh * D.N + row] = lab;
  const int w = threadIdx.x / kWave;
  const uint64_t mask = wave_match(lab, valid, 10);
  const int rin = __popcll(mask & lanemask_lt());
  const bool leader = valid && rin == 0;
  if (w == 0 && leader) hist[lab] = __popcll(mask);
  __syncthreads();
  int rank = rin;
  if (w == 1 && valid) rank += hist[lab];
  __syncthreads();
  if (w == 1 && leader) hist[lab] += __popcll(mask);
  if (valid) B.rank[(size_t)bh * D.N + row] = rank;
  if (threadIdx.x == 0) B.ipart[(size_t)bh * D.nblk + blk] = 0.0;
  __syncthreads();
  int* tab = B.tab + (size_t)bh * D.C * D.nblk;
  for (int i = threadIdx.x; i < C; i += kKmRows) tab[(size_t)i * D.nblk + blk] = hist[i];
}

__global__ void k_state_reset(KmState* st, int BH, int C, int done) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh < BH) {
    st[bh].done_iter = done;
    st[bh].iters = 0;
    st[bh].c_final = C;
    st[bh].inertia[0] = st[bh].inertia[1] = 0.0;
  }
}

// =====================================================================================
// Group masses (a reading: softmax over key groups of the centroid logit plus the log
// group size, averaged over the members of each query group, rounded to u = rint(P 2^32)).
// One block per (query group, head); 16 rows at a time; logits staged in LDS.
// =====================================================================================
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_group_mass(const T* q, Dims D, Bufs B) {
  constexpr int RB = 16;
  __shared__ float Xs[DD][RB];
  __shared__ float Ls[RB][kMaxGroups];
  __shared__ double colw[4][kMaxGroups / 4];  // scratch for the final 4-wave sum
  const int a = blockIdx.x, bh = blockIdx.y;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  if (a >= Cq) return;
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const int s0 = qo[a], n = qo[a + 1] - qo[a];
  const int* members = B.qperm + (size_t)bh * D.N + s0;
  const T* qb = q + (size_t)bh * D.N * DD;
  const float* Ckm = B.kcent + (size_t)bh * D.Ck * DD;
  const int* ko = B.koff + (size_t)bh * (D.Ck + 1);
  const int w = threadIdx.x / kWave, l = lane_id();
  constexpr int PL = kMaxGroups / kWave;  // columns per lane (max)
  double colsum[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) colsum[i] = 0.0;
  const int ty = threadIdx.x / 64, tx = threadIdx.x % 64;  // rows 4ty..4ty+3, column tx of a 64-tile
  for (int r0 = 0; r0 < n; r0 += RB) {
    __syncthreads();
    for (int i = threadIdx.x; i < RB * DD; i += 256) {
      const int r = i / DD, kk = i % DD;
      Xs[kk][r] = (r0 + r < n) ? to_f32(qb[(size_t)members[r0 + r] * DD + kk]) : 0.f;
    }
    __syncthreads();
    for (int c0 = 0; c0 < Ck; c0 += 64) {
      const int col = c0 + tx;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      if (col < Ck) {
        const float* cr = Ckm + (size_t)col * DD;
        for (int kk = 0; kk < DD; ++kk) {
          const float cv = cr[kk];
          const float4 xv = *reinterpret_cast<const float4*>(&Xs[kk][ty * 4]);
          acc[0] = fmaf(xv.x, cv, acc[0]);
          acc[1] = fmaf(xv.y, cv, acc[1]);
          acc[2] = fmaf(xv.z, cv, acc[2]);
          acc[3] = fmaf(xv.w, cv, acc[3]);
        }
        const float lg = logf((float)(ko[col + 1] - ko[col]));
#pragma unroll
        for (int r = 0; r < 4; ++r) Ls[ty * 4 + r][col] = fmaf(D.scale, acc[r], lg);
      }
    }
    __syncthreads();
    // softmax per row (wave w handles rows w, w+4, ...), accumulated per lane column
    for (int r = w; r < RB && r0 + r < n; r += 4) {
      float mx = -INFINITY;
      for (int c = l; c < Ck; c += kWave) mx = fmaxf(mx, Ls[r][c]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      float sm = 0.f;
      for (int c = l; c < Ck; c += kWave) sm += expf(Ls[r][c] - mx);
      sm = wave_sum(sm);
      const float inv = 1.f / sm;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int c = l + kWave * i;
        if (c < Ck) colsum[i] += (double)(expf(Ls[r][c] - mx) * inv);
      }
    }
  }
  // combine the 4 waves in fixed order, one quarter of the columns at a time
  long long* u = B.u + ((size_t)bh * D.Cq + a) * D.Ck;
  for (int qtr = 0; qtr < 4; ++qtr) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int c = l + kWave * i;
      if (c >= qtr * (kMaxGroups / 4) && c < (qtr + 1) * (kMaxGroups / 4)) colw[w][c - qtr * (kMaxGroups / 4)] = colsum[i];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < kMaxGroups / 4; c += 256) {
      const int col = c + qtr * (kMaxGroups / 4);
      if (col < Ck) {
        const double P = (((colw[0][c] + colw[1][c]) + colw[2][c]) + colw[3][c]) / (double)n;
        u[col] = (long long)rint(P * 4294967296.0);
      }
    }
  }
}

// =====================================================================================
// Routing (a reading of group-level routing under the executed-pair budget): each query
// group ranks key groups by (-u, b); one global integer threshold tau on the prefix mass
// picks the shortest reaching prefix (at least one group) per row; tau* is the largest
// tau whose total pair cost fits floor(rho N^2) - M N.
// =====================================================================================
__global__ __launch_bounds__(256) void k_route_sort(Dims D, Bufs B) {
  __shared__ unsigned long long key[kMaxGroups];
  __shared__ long long ws[4];
  const int a = blockIdx.x, bh = blockIdx.y;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  if (a >= Cq) return;
  const int tid = threadIdx.x;
  const long long* u = B.u + ((size_t)bh * D.Cq + a) * D.Ck;
  // order by (-u, b): the keys (distinct: the group id is in the low bits) sorted ascending by
  // a bitonic network over the next power of two at or above C_k (padding keys sort last)
  int n = 1;
  while (n < Ck) n <<= 1;
  for (int i = tid; i < n; i += 256)
    key[i] = i < Ck ? ((((1ull << 34) - 1ull - (unsigned long long)u[i]) << 10) | (unsigned)i) : ~0ull;
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long x = key[i], y = key[l];
          if ((x > y) == ((i & k) == 0)) {
            key[i] = y;
            key[l] = x;
          }
        }
      }
    }
  __syncthreads();
  // thread t takes sorted positions 4t .. 4t + 3: group, mass and key count, then the prefix
  // sums of mass and cost in that order
  const int* ko = B.koff + (size_t)bh * (D.Ck + 1);
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const long long nq = qo[a + 1] - qo[a];
  int bq[4];
  long long mq[4], kq[4], sm = 0, sk = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = 4 * tid + q;
    const bool v = p < Ck;
    bq[q] = v ? (int)(key[p] & 1023ull) : 0;
    mq[q] = v ? u[bq[q]] : 0;
    kq[q] = v ? (long long)(ko[bq[q] + 1] - ko[bq[q]]) : 0;
    sm += mq[q];
    sk += kq[q];
  }
  long long t1, t2;
  long long cm = block_excl_scan<256, long long>(sm, &t1, ws);
  long long cn = block_excl_scan<256, long long>(sk, &t2, ws);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = 4 * tid + q;
    cm += mq[q];
    cn += kq[q];
    if (p < Ck) {
      const size_t o = ((size_t)bh * D.Cq + a) * D.Ck + p;
      B.sorted_b[o] = bq[q];
      B.cum[o] = cm;
      B.ccost[o] = nq * cn;
    }
  }
}

// First index in [lo, hi] whose prefix mass reaches tau (hi = Ck: none); the caller knows the
// answer lies in [lo, hi] (the index is monotone in tau).
__device__ inline int route_first(const long long* cum, long long tau, int lo, int hi) {
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] >= tau) hi = mid; else lo = mid + 1;
  }
  return lo;
}

__global__ __launch_bounds__(1024) void k_route_tau(Dims D, Bufs B) {
  __shared__ long long ws[16];
  __shared__ int wsi[16];
  const int bh = blockIdx.x, a = threadIdx.x;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  const size_t ro = ((size_t)bh * D.Cq + a) * D.Ck;
  const long long* cum = B.cum + ro;
  const long long* cc = B.ccost + ro;
  // cost(tau) = sum over rows of the pair cost of the shortest prefix reaching tau (at least
  // one group). Bisection on tau; each row keeps the index range its answer is known to lie
  // in (the answers at the current lo and hi), so its search shrinks with the interval.
  auto take = [&](int f) { return min(max(f + 1, 1), Ck); };
  auto cost_of = [&](int f) -> long long {
    const long long c = a < Cq ? cc[take(f) - 1] : 0;
    return block_sum<1024, long long>(c, ws);
  };
  const long long budget = D.budget;
  long long hi = (1ll << 32) + Ck, tau;
  int flo = 0, fhi = a < Cq ? route_first(cum, hi, 0, Ck) : 0;  // cum >= 0: f(0) = 0
  int exceeded = 0, fsel;
  if (cost_of(flo) > budget) {
    tau = 0;
    exceeded = 1;
    fsel = flo;
  } else if (cost_of(fhi) <= budget) {
    tau = hi;
    fsel = fhi;
  } else {
    long long lo = 0;
    while (hi - lo > 1) {
      const long long mid = (lo + hi) >> 1;
      const int fm = a < Cq ? route_first(cum, mid, flo, fhi) : 0;
      if (cost_of(fm) <= budget) {
        lo = mid;
        flo = fm;
      } else {
        hi = mid;
        fhi = fm;
      }
    }
    tau = lo;
    fsel = flo;
  }
  const int j = a < Cq ? take(fsel) : 0;
  const long long pc = a < Cq ? cc[j - 1] : 0;
  const long long pairs = block_sum<1024, long long>(pc, ws);
  int tot;
  const int rp = block_excl_scan<1024, int>(j, &tot, wsi);
  if (a < Cq) {
    B.jsel[(size_t)bh * D.Cq + a] = j;
    B.row_ptr[(size_t)bh * (D.Cq + 1) + a] = rp;
  }
  if (a == 0) {
    B.row_ptr[(size_t)bh * (D.Cq + 1) + Cq] = tot;
    B.rinfo[bh].tau = tau;
    B.rinfo[bh].budget = budget;
    B.rinfo[bh].pairs = pairs + (long long)D.M * D.N;
    B.rinfo[bh].exceeded = exceeded;
  }
}

// Selected key groups of one query group, in ascending key-group order.
__global__ __launch_bounds__(256) void k_route_emit(Dims D, Bufs B) {
  __shared__ int flag[kMaxGroups];
  __shared__ int ws[4];
  const int a = blockIdx.x, bh = blockIdx.y;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  if (a >= Cq) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < kMaxGroups; i += 256) flag[i] = 0;
  __syncthreads();
  const int j = B.jsel[(size_t)bh * D.Cq + a];
  for (int i = tid; i < j; i += 256) flag[B.sorted_b[((size_t)bh * D.Cq + a) * D.Ck + i]] = 1;
  __syncthreads();
  // thread t takes key groups 4t .. 4t + 3: selected, and first / last of a run of
  // consecutive selected groups (whose keys are contiguous after the permutation)
  bool f[4], st[4], en[4];
  int ns = 0, nst = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = 4 * tid + q;
    f[q] = g < Ck && flag[g];
    st[q] = f[q] && (g == 0 || !flag[g - 1]);
    en[q] = f[q] && (g + 1 == Ck || !flag[g + 1]);
    ns += f[q] ? 1 : 0;
    nst += st[q] ? 1 : 0;
  }
  int tot, nr;
  int pos = block_excl_scan<256, int>(ns, &tot, ws);
  int rs = block_excl_scan<256, int>(nst, &nr, ws);
  const int rp = B.row_ptr[(size_t)bh * (D.Cq + 1) + a];
  const int* ko = B.koff + (size_t)bh * (D.Ck + 1);
  int2* runs = B.runs + (size_t)bh * D.Cq * D.Ck + rp;
  int* cols = B.cols + (size_t)bh * D.Cq * D.Ck + rp;
  // key runs [koff[first], koff[last + 1])
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = 4 * tid + q;
    if (f[q]) cols[pos++] = g;
    if (st[q]) runs[rs].x = ko[g];
    if (en[q]) runs[rs + (st[q] ? 1 : 0) - 1].y = ko[g + 1];
    rs += st[q] ? 1 : 0;
  }
  if (tid == 0) B.nruns[(size_t)bh * D.Cq + a] = nr;
  // the attention kernel's key tiles over these runs (each run from its start rounded down to
  // 8 keys), for the pairing of its work items
  __syncthreads();
  int t = 0;
  for (int r = tid; r < nr; r += 256) {
    const int2 rv = runs[r];
    t += (rv.y - (rv.x & ~7) + kKeyTile - 1) / kKeyTile;
  }
  const int tt = block_sum<256, int>(t, ws);
  if (tid == 0) B.gtiles[(size_t)bh * D.Cq + a] = tt;
}

// The bf16 attention's key order (per head): key groups ranked by the number of query groups
// that select them, most first, ties to the lower index; the start of each rank's keys.
__global__ __launch_bounds__(1024) void k_key_order(Dims D, Bufs B) {
  __shared__ int cnt[kMaxGroups];
  __shared__ int sz[kMaxGroups];
  __shared__ int ws[16];
  const int bh = blockIdx.x, b = threadIdx.x;
  const int Ck = B.kst[bh].c_final, Cq = B.qst[bh].c_final;
  cnt[b] = 0;
  sz[b] = 0;
  __syncthreads();
  const int* rp = B.row_ptr + (size_t)bh * (D.Cq + 1);
  const int* cols = B.cols + (size_t)bh * D.Cq * D.Ck;
  const int tot = rp[Cq];
  for (int e = b; e < tot; e += 1024) atomicAdd(&cnt[cols[e]], 1);
  __syncthreads();
  const int* ko = B.koff + (size_t)bh * (D.Ck + 1);
  if (b < Ck) {
    const int cb = cnt[b];
    int rank = 0;
    for (int x = 0; x < Ck; ++x) {
      const int cx = cnt[x];
      rank += (cx > cb || (cx == cb && x < b)) ? 1 : 0;
    }
    B.katt_rank[(size_t)bh * D.Ck + b] = rank;
    sz[rank] = ko[b + 1] - ko[b];
  }
  __syncthreads();
  int total;
  const int st = block_excl_scan<1024, int>(b < Ck ? sz[b] : 0, &total, ws);
  int* ks = B.katt_start + (size_t)bh * (D.Ck + 1);
  if (b < Ck) ks[b] = st;
  if (b == 0) ks[Ck] = total;
}

// Key runs of one query group in the attention order (maximal stretches of consecutive
// ranks among its selected key groups), and their key tiles.
__global__ __launch_bounds__(256) void k_att_runs(Dims D, Bufs B) {
  __shared__ int flag[kMaxGroups];
  __shared__ int ws[4];
  const int a = blockIdx.x, bh = blockIdx.y;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  if (a >= Cq) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < kMaxGroups; i += 256) flag[i] = 0;
  __syncthreads();
  const int* rpa = B.row_ptr + (size_t)bh * (D.Cq + 1);
  const int rp = rpa[a], j = rpa[a + 1] - rp;
  const int* rank = B.katt_rank + (size_t)bh * D.Ck;
  for (int i = tid; i < j; i += 256) flag[rank[B.cols[(size_t)bh * D.Cq * D.Ck + rp + i]]] = 1;
  __syncthreads();
  // thread t takes positions 4t .. 4t + 3 of the order
  bool st[4], en[4];
  int nst = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * tid + q;
    const bool f = r < Ck && flag[r];
    st[q] = f && (r == 0 || !flag[r - 1]);
    en[q] = f && (r + 1 == Ck || !flag[r + 1]);
    nst += st[q] ? 1 : 0;
  }
  int nr;
  int rs = block_excl_scan<256, int>(nst, &nr, ws);
  const int* ks = B.katt_start + (size_t)bh * (D.Ck + 1);
  int2* runs = B.runs + (size_t)bh * D.Cq * D.Ck + rp;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * tid + q;
    if (st[q]) runs[rs].x = ks[r];
    if (en[q]) runs[rs + (st[q] ? 1 : 0) - 1].y = ks[r + 1];
    rs += st[q] ? 1 : 0;
  }
  if (tid == 0) B.nruns[(size_t)bh * D.Cq + a] = nr;
  __syncthreads();
  int t = 0;
  for (int r = tid; r < nr; r += 256) {
    const int2 rv = runs[r];
    t += (rv.y - (rv.x & ~7) + kKeyTile - 1) / kKeyTile;
  }
  const int tt = block_sum<256, int>(t, ws);
  if (tid == 0) B.gtiles[(size_t)bh * D.Cq + a] = tt;
}

// Key rows in the attention order: group b's rows (plan order) moved to its rank's start.
__global__ __launch_bounds__(256) void k_att_perm(Dims D, Bufs B) {
  const int b = blockIdx.x, bh = blockIdx.y;
  if (b >= B.kst[bh].c_final) return;
  const int* ko = B.koff + (size_t)bh * (D.Ck + 1);
  const int lo = ko[b], n = ko[b + 1] - lo;
  const int dst = B.katt_start[(size_t)bh * (D.Ck + 1) + B.katt_rank[(size_t)bh * D.Ck + b]];
  for (int i = threadIdx.x; i < n; i += 256)
    B.kperm_att[(size_t)bh * D.N + dst + i] = B.kperm[(size_t)bh * D.N + lo + i];
}

// Work items of the 8-wave attention kernel, per head (one thread per query group). A group's
// rows go in chunks of 256; a full chunk is one item on all 8 waves. The last chunk, of
// w = ceil(r / 32) < 8 waves, runs on its own: all waves on its keys when w >= 5 (T_g steps,
// 8 - w waves idle), the two wave halves on half the keys each when w <= 4 (T_g / 2 steps).
// A last chunk of w <= 3 waves and one of 8 - w waves (buckets in group order, rank for rank)
// instead share one item, each on its own waves and key stream (max(T_g, T_h) steps), unless
// the small chunk has more than twice the other's key tiles (then apart is no slower).
__global__ __launch_bounds__(1024) void k_pair_tiles(Dims D, Bufs B) {
  __shared__ int slot[8][kMaxGroups];  // bucket w: rank -> group
  __shared__ int taken[kMaxGroups];    // the group's last chunk shares an item it does not own
  __shared__ int ws[16];
  const int bh = blockIdx.x, g = threadIdx.x;
  const int Cq = B.qst[bh].c_final;
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const int* gt = B.gtiles + (size_t)bh * D.Cq;
  auto last_chunk = [&](int x, int& pos, int& w) {  // first row and waves of group x's last chunk
    const int n = qo[x + 1] - qo[x], c = (n + 255) / 256;
    pos = qo[x] + 256 * (c - 1);
    w = (n - 256 * (c - 1) + 31) / 32;
    return c;
  };
  int pos = 0, w = 8, c = 0;
  if (g < Cq) c = last_chunk(g, pos, w);  // (groups are non-empty)
  const bool rem = c > 0 && w < 8;
  __shared__ int cnt[8];  // chunks per bucket
  int rank = 0;
  for (int b = 1; b < 8; ++b) {
    int tot;
    const int rk = block_excl_scan<1024, int>(rem && w == b ? 1 : 0, &tot, ws);
    if (rem && w == b) rank = rk;
    if (g == 0) cnt[b] = tot;
  }
  taken[g] = 0;
  if (rem) slot[w][rank] = g;
  __syncthreads();
  int partner = -1;
  if (rem && w <= 3 && rank < cnt[8 - w]) {
    partner = slot[8 - w][rank];
    if (gt[g] > 2 * gt[partner]) partner = -1;
    else taken[partner] = 1;
  }
  __syncthreads();
  const bool own = rem && !taken[g];  // the last chunk's item is written by this group
  const int items = (c > 0 ? c - 1 : 0) + (c > 0 && w == 8 ? 1 : 0) + (own ? 1 : 0);
  int tot;
  int o = block_excl_scan<1024, int>(items, &tot, ws);
  int4* pt = B.ptiles + (size_t)bh * D.max_atiles;
  if (g == 0) B.nptiles[bh] = tot;
  for (int k = 0; k < c - 1 + (w == 8 ? 1 : 0); ++k) pt[o++] = make_int4(g, qo[g] + 256 * k, -1, 0);
  if (own) {
    if (partner >= 0) {
      int ph, wh;
      last_chunk(partner, ph, wh);
      pt[o] = make_int4(partner, ph, g, pos);  // stream 0: the larger chunk
    } else {
      pt[o] = make_int4(g, pos, w <= 4 ? -2 : -1, 0);
    }
  }
}

// =====================================================================================
// Probe allocation (paper Table 4: query-group stratified probes). m_a is the largest-
// remainder split of M over groups in proportion to n_q[a] (ties to the lower group);
// weights w = (n_q[a] / m_a) * M / sum_{m_a > 0} n_q[a].
// =====================================================================================
__global__ __launch_bounds__(1024) void k_probe_alloc(Dims D, Bufs B) {
  __shared__ long long rem[kMaxGroups];
  __shared__ int ws[16];
  __shared__ long long wsl[16];
  const int bh = blockIdx.x, a = threadIdx.x;
  const int Cq = B.qst[bh].c_final;
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const long long n = a < Cq ? (long long)(qo[a + 1] - qo[a]) : 0;
  const long long prod = (long long)D.M * n;
  const int base = (int)(prod / D.N);
  rem[a] = a < Cq ? prod % D.N : -1;
  int tot;
  (void)block_excl_scan<1024, int>(base, &tot, ws);
  const int left = D.M - tot;
  int rank = 0;
  if (a < Cq) {
    const long long r = rem[a];
    for (int b = 0; b < Cq; ++b) {
      const long long rb = rem[b];
      rank += (rb > r) || (rb == r && b < a);
    }
  }
  const int m = a < Cq ? base + (rank < left ? 1 : 0) : 0;
  int mtot;
  const int off = block_excl_scan<1024, int>(m, &mtot, ws);
  long long cov;
  (void)block_excl_scan<1024, long long>(m > 0 ? n : 0ll, &cov, wsl);
  if (a < Cq) {
    B.pcount[(size_t)bh * D.Cq + a] = m;
    B.poff[(size_t)bh * (D.Cq + 1) + a] = off;
    B.pw_group[(size_t)bh * D.Cq + a] = m > 0 ? (float)(((double)n / (double)m) * ((double)D.M / (double)cov)) : 0.f;
  }
  if (a == 0) B.poff[(size_t)bh * (D.Cq + 1) + Cq] = mtot;
}

__global__ void k_fill_i32(int* p, long long n, int v) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

// =====================================================================================
// Tiles of consecutive positions of one query group: 128 rows for the group masses
// (tiles / ntiles / tstart) and 32 * attn_w rows for the block-sparse attention (atiles /
// antiles).
// =====================================================================================
__global__ __launch_bounds__(1024) void k_build_tiles(Dims D, Bufs B) {
  __shared__ int ws[16];
  __shared__ int tstart[kMaxGroups + 1], astart[kMaxGroups + 1];
  const int bh = blockIdx.x, a = threadIdx.x;
  const int Cq = B.qst[bh].c_final;
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const int aqt = 32 * D.attn_w;
  const int n = a < Cq ? qo[a + 1] - qo[a] : 0;
  int tot, atot;
  const int s = block_excl_scan<1024, int>(ceil_div(n, D.qt), &tot, ws);
  tstart[a] = s;
  if (a < Cq) B.tstart[(size_t)bh * (D.Cq + 1) + a] = s;
  if (a == 0) B.tstart[(size_t)bh * (D.Cq + 1) + Cq] = tot;
  if (a == 0) {
    tstart[kMaxGroups] = tot;
    B.ntiles[bh] = tot;
  }
  __syncthreads();
  astart[a] = block_excl_scan<1024, int>(ceil_div(n, aqt), &atot, ws);
  if (a == 0) B.antiles[bh] = atot;
  __syncthreads();
  const int w = threadIdx.x / kWave, l = lane_id();
  int2* tiles = B.tiles + (size_t)bh * D.max_tiles;
  int2* atiles = B.atiles + (size_t)bh * D.max_atiles;
  for (int g = w; g < Cq; g += 16) {
    const int rows = qo[g + 1] - qo[g];
    const int nt = ceil_div(rows, D.qt), na = ceil_div(rows, aqt);
    for (int t = l; t < nt; t += kWave) tiles[tstart[g] + t] = make_int2(g, qo[g] + t * D.qt);
    for (int t = l; t < na; t += kWave) atiles[astart[g] + t] = make_int2(g, qo[g] + t * aqt);
  }
}

// =====================================================================================
// Group-contiguous K and transposed V: Kp[pos] = K[perm[pos]], VpT[i][pos] = V[perm[pos]][i];
// positions N..Npad-1 are zero.
// =====================================================================================
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_permute_kv(const T* k, const T* v, const int* perm, int N, int Npad,
                                                    T* kp, T* vpt) {
  constexpr int EV = 16 / sizeof(T);  // elements per 16-byte access
  __shared__ T vs[64][DD + EV];
  const int p0 = blockIdx.x * 64, bh = blockIdx.y;
  const int* pb = perm + (size_t)bh * N;
  const T* kb = k + (size_t)bh * N * DD;
  const T* vb = v + (size_t)bh * N * DD;
  T* kpb = kp + (size_t)bh * Npad * DD;
  T* vtb = vpt + (size_t)bh * DD * Npad;
  // rows: 64 positions x DD/EV chunks of 16 bytes
  for (int e = threadIdx.x; e < 64 * DD / EV; e += 256) {
    const int r = e / (DD / EV), c = (e % (DD / EV)) * EV;
    const int pos = p0 + r;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (pos < N) {
      const int src = pb[pos];
      kv = *reinterpret_cast<const uint4*>(kb + (size_t)src * DD + c);
      vv = *reinterpret_cast<const uint4*>(vb + (size_t)src * DD + c);
    }
    if (pos < Npad) *reinterpret_cast<uint4*>(kpb + (size_t)pos * DD + c) = kv;
    const T* vt = reinterpret_cast<const T*>(&vv);
#pragma unroll
    for (int q = 0; q < EV; ++q) vs[r][c + q] = vt[q];
  }
  __syncthreads();
  // transposed: DD rows x 64 positions, EV consecutive positions per 16-byte store
  for (int e = threadIdx.x; e < DD * 64 / EV; e += 256) {
    const int c = e / (64 / EV), r = (e % (64 / EV)) * EV;
    if (p0 + r < Npad) {
      uint4 out;
      T* ot = reinterpret_cast<T*>(&out);
#pragma unroll
      for (int q = 0; q < EV; ++q) ot[q] = vs[r + q][c];
      *reinterpret_cast<uint4*>(vtb + (size_t)c * Npad + p0 + r) = out;
    }
  }
}

// Identity partition for the dense reference call: one query group and one key group.
__global__ void k_identity_plan(Dims D, Bufs B) {
  const int bh = blockIdx.y;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < D.N; j += gridDim.x * blockDim.x) {
    B.qperm[(size_t)bh * D.N + j] = j;
    B.kperm[(size_t)bh * D.N + j] = j;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    B.qoff[(size_t)bh * (D.Cq + 1)] = 0;
    B.qoff[(size_t)bh * (D.Cq + 1) + 1] = D.N;
    B.koff[(size_t)bh * (D.Ck + 1)] = 0;
    B.koff[(size_t)bh * (D.Ck + 1) + 1] = D.N;
    B.row_ptr[(size_t)bh * (D.Cq + 1)] = 0;
    B.row_ptr[(size_t)bh * (D.Cq + 1) + 1] = 1;
    B.cols[(size_t)bh * D.Cq * D.Ck] = 0;
    B.runs[(size_t)bh * D.Cq * D.Ck] = make_int2(0, D.N);
    B.nruns[(size_t)bh * D.Cq] = 1;
    B.gtiles[(size_t)bh * D.Cq] = (D.N + kKeyTile - 1) / kKeyTile;
    B.qst[bh].c_final = 1;
    B.kst[bh].c_final = 1;
  }
}

// =====================================================================================
// Launchers
// =====================================================================================
#define SPR_DISPATCH(dtype, d, FN, ...)                                   \
  do {                                                                    \
    if ((dtype) == 1 && (d) == 128) FN<bf16, 128>(__VA_ARGS__);           \
    else if ((dtype) == 1 && (d) == 64) FN<bf16, 64>(__VA_ARGS__);        \
    else if ((dtype) == 0 && (d) == 128) FN<float, 128>(__VA_ARGS__);     \
    else FN<float, 64>(__VA_ARGS__);                                      \
  } while (0)

// Lloyd iterations from the centroids already in B.cent / cent_t / cnorm (state in st).
template <typename T, int DD>
static void lloyd_iterations(const T* x, const Dims& D, const Bufs& B, int C, KmState* st, int* perm,
                             hipStream_t s) {
  // The metric terms (G m_b, m_b G m_b, the operands) in their own launch, one read of G per 32
  // groups, when the update has at least 16 workgroups per CU to feed; on smaller launches the
  // extra launch's latency costs more than the update's reads of G (same arithmetic either way).
  const bool split_terms = (long long)C * D.BH >= 16 * 256;
  for (int t = 1; t <= D.max_iter; ++t) {
    if constexpr (std::is_same<T, bf16>::value)
      if (D.assign_lo)
        hipLaunchKernelGGL((k_km_assign_bf16<DD, 2, true>), dim3((D.nblk + 1) / 2, D.BH), dim3(256), 0, s, x, D, B, C,
                           st, t);
      else
        hipLaunchKernelGGL((k_km_assign_bf16<DD, 1, false>), dim3(D.nblk, D.BH), dim3(256), 0, s, x, D, B, C, st, t);
    else
      hipLaunchKernelGGL((k_km_assign<T, DD>), dim3(D.nblk, D.BH), dim3(256), 0, s, x, D, B, C, st, t);
    if (split_terms) {
      hipLaunchKernelGGL((k_km_update<T, DD, false>), dim3(C, D.BH), dim3(256), 0, s, x, D, B, st, t);
      hipLaunchKernelGGL((k_km_metric_terms<DD>), dim3((C + 31) / 32, D.BH), dim3(256), 0, s, D, B, C, st, t);
    } else {
      hipLaunchKernelGGL((k_km_update<T, DD, true>), dim3(C, D.BH), dim3(256), 0, s, x, D, B, st, t);
    }
  }
  // group starts and the permutation of the final assignment
  hipLaunchKernelGGL(k_km_scan_groups, dim3(C, D.BH), dim3(64), 0, s, D, B, C, st, 0);
  hipLaunchKernelGGL(k_km_scan_head, dim3(D.BH), dim3(256), 0, s, D, B, C, st, 0);
  hipLaunchKernelGGL(k_km_scatter, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, D, B, st, 0, perm);
}

template <typename T, int DD>
static void run_lloyd(const void* xv, const Dims& D, const Bufs& B, int C, const int* init, KmState* st, int* perm,
                      hipStream_t s) {
  const T* x = (const T*)xv;
  hipLaunchKernelGGL((k_km_init<T, DD>), dim3(C, D.BH), dim3(256), 0, s, x, D, B, C, init, st);
  lloyd_iterations<T, DD>(x, D, B, C, st, perm, s);
}

template <typename T, int DD>
static void rowquad(const T* x, const Dims& D, const Bufs& B, const float* G, float* rowconst, float* alpha_out,
                    const KmState* kst, hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value) {
    // about 2048 workgroups (eight per CU over the launch), each staging G once
    const int per = std::max(1, D.nblk * D.BH / 2048);
    hipLaunchKernelGGL((k_rowquad_bf16<DD>), dim3((D.nblk + per - 1) / per, D.BH), dim3(256), 0, s, x, D,
                       B.metric_h, B.metric_l, rowconst, alpha_out, kst);
  } else {
    hipLaunchKernelGGL((k_rowquad<T, DD>), dim3(D.nblk, D.BH), dim3(256), 0, s, x, D, G, rowconst, alpha_out, kst);
  }
}

template <typename T, int DD>
static void group_mass(const T* q, const Dims& D, const Bufs& B, hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value) {
    constexpr int TPB = kMassTiles;
    hipLaunchKernelGGL((k_group_mass_bf16<DD, TPB>), dim3((D.max_tiles + TPB - 1) / TPB, D.BH), dim3(256 * TPB), 0, s,
                       q, D, B);
    hipLaunchKernelGGL(k_group_mass_final, dim3(D.Cq, D.BH), dim3(256), 0, s, D, B);
  } else {
    hipLaunchKernelGGL((k_group_mass<T, DD>), dim3(D.Cq, D.BH), dim3(256), 0, s, q, D, B);
  }
}

// Leading eigen-directions of a symmetric d x d matrix per head, by cyclic two-sided Jacobi
// in LDS (float), round-robin pairings so that the n/2 rotations of a round act on disjoint
// index pairs and are applied together, 2 x 2 block by 2 x 2 block; sweeps until the
// off-diagonal mass is below 1e-14 of the total (at most 15). The `rank` largest diagonal
// entries (ties to the lower index) select the eigenvectors u_i, and the output is either the
// truncated matrix sum_i lambda_i u_i u_i^T (with its bf16 hi / lo split when out_h is given)
// or, with PROJ, the orthogonal projector sum_i u_i u_i^T.
// Uses: the key response rank (paper Table C.1, r_K: the key metric G = s^2 Q_S^T Q_S
// truncated to its r_K largest eigenvalues, the metric of the key responses projected on the
// sampled queries' r_K leading response directions), and the output truncation of the
// residual fit (the probe residuals' leading directions).
template <int DD, bool PROJ>
__global__ __launch_bounds__(1024) void k_top_rank(const float* in, float* out, bf16* out_h, bf16* out_l, int keep) {
  constexpr int n = DD, H2 = DD / 2, LD = DD + 1;
  __shared__ float A[DD * LD], V[DD * LD];
  __shared__ float cs_c[H2], cs_s[H2];
  __shared__ int pp[H2], qq[H2];
  __shared__ float red[2][16];
  __shared__ int sel[DD];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* G = in + (size_t)bh * DD * DD;
  for (int e = tid; e < n * n; e += 1024) {
    const int i = e / n, j = e % n;
    A[i * LD + j] = G[e];
    V[i * LD + j] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 15; ++sweep) {
    // off-diagonal and total mass, summed in a fixed order
    float off = 0.f, tot = 0.f;
    for (int e = tid; e < n * n; e += 1024) {
      const float v = A[(e / n) * LD + e % n];
      tot += v * v;
      if (e / n != e % n) off += v * v;
    }
    off = wave_sum(off);
    tot = wave_sum(tot);
    if (lane_id() == 0) {
      red[0][tid / kWave] = off;
      red[1][tid / kWave] = tot;
    }
    __syncthreads();
    float o = 0.f, t = 0.f;
    for (int w = 0; w < 16; ++w) {
      o += red[0][w];
      t += red[1][w];
    }
    __syncthreads();
    if (!(o > 1e-14f * t)) break;
    for (int rnd = 0; rnd < n - 1; ++rnd) {
      if (tid < H2) {
        auto player = [&](int pos) { return pos == 0 ? 0 : ((pos - 1 + rnd) % (n - 1)) + 1; };
        const int a = player(tid), b = player(n - 1 - tid);
        const int p = min(a, b), q = max(a, b);
        const float apq = A[p * LD + q];
        float c = 1.f, sn = 0.f;
        if (apq != 0.f) {
          const float tau = (A[q * LD + q] - A[p * LD + p]) / (2.f * apq);
          const float tt = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + tt * tt);
          sn = tt * c;
        }
        cs_c[tid] = c;
        cs_s[tid] = sn;
        pp[tid] = p;
        qq[tid] = q;
      }
      __syncthreads();
      // A <- J^T A J, block (i, j) = rows (p_i, q_i) x columns (p_j, q_j)
      for (int e = tid; e < H2 * H2; e += 1024) {
        const int i = e / H2, j = e % H2;
        const int pi = pp[i], qi = qq[i], pj = pp[j], qj = qq[j];
        const float ci = cs_c[i], si = cs_s[i], cj = cs_c[j], sj = cs_s[j];
        const float m00 = A[pi * LD + pj], m01 = A[pi * LD + qj], m10 = A[qi * LD + pj], m11 = A[qi * LD + qj];
        const float t00 = m00 * cj - m01 * sj, t01 = m00 * sj + m01 * cj;
        const float t10 = m10 * cj - m11 * sj, t11 = m10 * sj + m11 * cj;
        A[pi * LD + pj] = ci * t00 - si * t10;
        A[pi * LD + qj] = ci * t01 - si * t11;
        A[qi * LD + pj] = si * t00 + ci * t10;
        A[qi * LD + qj] = si * t01 + ci * t11;
      }
      // V <- V J
      for (int e = tid; e < n * H2; e += 1024) {
        const int r = e / H2, j = e % H2;
        const int pj = pp[j], qj = qq[j];
        const float cj = cs_c[j], sj = cs_s[j];
        const float vp = V[r * LD + pj], vq = V[r * LD + qj];
        V[r * LD + pj] = vp * cj - vq * sj;
        V[r * LD + qj] = vp * sj + vq * cj;
      }
      __syncthreads();
    }
  }
  // the r_K largest eigenvalues (ties to the lower index)
  if (tid < n) {
    const float li = A[tid * LD + tid];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const float lj = A[j * LD + j];
      rank += (lj > li) || (lj == li && j < tid);
    }
    sel[tid] = rank < keep;
  }
  __syncthreads();
  for (int e = tid; e < n * n; e += 1024) {
    const int a = e / n, b = e % n;
    float g = 0.f;
    for (int i = 0; i < n; ++i)
      if (sel[i]) g = fmaf(PROJ ? V[a * LD + i] : A[i * LD + i] * V[a * LD + i], V[b * LD + i], g);
    const size_t o = (size_t)bh * DD * DD + e;
    out[o] = g;
    if (out_h) {
      const bf16 gh = (bf16)g;
      out_h[o] = gh;
      out_l[o] = (bf16)(g - (float)gh);
    }
  }
}

// Lloyd metric of the key side: s^2 Q_S^T Q_S (responses to the sampled queries), or the
// identity for the semantic partition.
template <int DD>
static void key_metric(const Dims& D, const Bufs& B, hipStream_t s) {
  if (D.partition == 1) {
    hipLaunchKernelGGL((k_identity_metric<DD>), dim3(DD * DD / 256, D.BH), dim3(256), 0, s, D, B);
    return;
  }
  hipLaunchKernelGGL((k_gram<DD>), dim3(DD * DD / 256, D.BH), dim3(256), 0, s, B.qs, D.S, (const KmState*)nullptr,
                     D.scale * D.scale, B.metric, B.metric_h, B.metric_l);
  // rank reduction only below the rank of Q_S (at most min(d, S))
  if (D.key_rank > 0 && D.key_rank < DD && D.key_rank < D.S)
    hipLaunchKernelGGL((k_top_rank<DD, false>), dim3(D.BH), dim3(1024), 0, s, (const float*)B.metric, B.metric,
                       B.metric_h, B.metric_l, D.key_rank);
}

// Metric, row constants and row scales of the query side: responses to the key centroids,
// RMS-normalised (G_k = C_k^T C_k, alpha = s / RMS), or raw queries (identity, alpha = 1).
// Returns the buffers the query Lloyd runs with.
template <typename T, int DD>
static Bufs query_side(const T* q, const Dims& D, const Bufs& B, hipStream_t s) {
  Bufs Bq = B;
  if (D.partition == 0) {
    hipLaunchKernelGGL((k_gram<DD>), dim3(DD * DD / 256, D.BH), dim3(256), 0, s, B.kcent, D.Ck, (const KmState*)B.kst,
                       1.f, B.metric, B.metric_h, B.metric_l);
    rowquad<T, DD>(q, D, B, B.metric, B.rowconst, B.alpha, (const KmState*)B.kst, s);
  } else {
    hipLaunchKernelGGL((k_identity_metric<DD>), dim3(DD * DD / 256, D.BH), dim3(256), 0, s, D, B);
    rowquad<T, DD>(q, D, B, B.metric, B.rowconst, (float*)nullptr, (const KmState*)nullptr, s);
    Bq.alpha = nullptr;
  }
  return Bq;
}

template <typename T, int DD>
static void plan_impl(const void* qv, const void* kv, const Dims& D, const Bufs& B, hipStream_t s) {
  const T* q = (const T*)qv;
  const T* k = (const T*)kv;
  // 01: sampled queries and their key-response metric
  hipLaunchKernelGGL(k_select_all, dim3(D.BH, 3), dim3(1024), 0, s, D, B);
  hipLaunchKernelGGL((k_gather_rows<T>), dim3(D.S, D.BH), dim3(DD), 0, s, q, B.sampled, D.N, D.S, DD, B.qs);
  key_metric<DD>(D, B, s);
  // 02a: paired K/V groups by Lloyd on the key responses
  Bufs Bk = B;
  Bk.alpha = nullptr;
  rowquad<T, DD>(k, D, B, B.metric, B.rowconst, (float*)nullptr, (const KmState*)nullptr, s);
  run_lloyd<T, DD>(k, D, Bk, D.Ck, B.init_k, B.kst, B.kperm, s);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Ck, B.kst, B.klab, B.koff, D.Ck + 1);
  hipLaunchKernelGGL((k_key_centroids<T, DD>), dim3(D.Ck, D.BH), dim3(256), 0, s, k, D, B);
  // 02b: query-response coordinates (RMS-normalised) and query groups
  const Bufs Bq = query_side<T, DD>(q, D, B, s);
  run_lloyd<T, DD>(q, D, Bq, D.Cq, B.init_q, B.qst, B.qperm, s);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Cq, B.qst, B.qlab, B.qoff, D.Cq + 1);
  hipLaunchKernelGGL((k_query_reps<T, DD>), dim3(D.Cq, D.BH), dim3(256), 0, s, q, D, Bq);
  hipLaunchKernelGGL(k_build_tiles, dim3(D.BH), dim3(1024), 0, s, D, B);
  // 03: group masses
  group_mass<T, DD>(q, D, B, s);
}

// Warm-started plan: both k-means start from the previous plan's groups (k_km_warm_init)
// and run at most D.warm_iter iterations.
template <typename T, int DD>
static void plan_warm_impl(const void* qv, const void* kv, const Dims& D0, const Bufs& B, hipStream_t s) {
  const T* q = (const T*)qv;
  const T* k = (const T*)kv;
  Dims D = D0;
  D.max_iter = D0.warm_iter;
  hipLaunchKernelGGL(k_select_all, dim3(D.BH, 3), dim3(1024), 0, s, D, B);
  hipLaunchKernelGGL((k_gather_rows<T>), dim3(D.S, D.BH), dim3(DD), 0, s, q, B.sampled, D.N, D.S, DD, B.qs);
  key_metric<DD>(D, B, s);
  // key groups from the previous key centroids
  Bufs Bk = B;
  Bk.alpha = nullptr;
  rowquad<T, DD>(k, D, B, B.metric, B.rowconst, (float*)nullptr, (const KmState*)nullptr, s);
  hipLaunchKernelGGL((k_km_warm_init<DD>), dim3(D.Ck, D.BH), dim3(256), 0, s, D, Bk, B.kcent, D.Ck, B.kst);
  hipLaunchKernelGGL(k_state_reset, dim3((D.BH + 63) / 64), dim3(64), 0, s, B.kst, D.BH, D.Ck, 0x7fffffff);
  lloyd_iterations<T, DD>(k, D, Bk, D.Ck, B.kst, B.kperm, s);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Ck, B.kst, B.klab, B.koff, D.Ck + 1);
  hipLaunchKernelGGL((k_key_centroids<T, DD>), dim3(D.Ck, D.BH), dim3(256), 0, s, k, D, B);
  // query groups from the previous query representatives
  const Bufs Bq = query_side<T, DD>(q, D, B, s);
  hipLaunchKernelGGL((k_km_warm_init<DD>), dim3(D.Cq, D.BH), dim3(256), 0, s, D, Bq, B.qcent, D.Cq, B.qst);
  hipLaunchKernelGGL(k_state_reset, dim3((D.BH + 63) / 64), dim3(64), 0, s, B.qst, D.BH, D.Cq, 0x7fffffff);
  lloyd_iterations<T, DD>(q, D, Bq, D.Cq, B.qst, B.qperm, s);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Cq, B.qst, B.qlab, B.qoff, D.Cq + 1);
  hipLaunchKernelGGL((k_query_reps<T, DD>), dim3(D.Cq, D.BH), dim3(256), 0, s, q, D, Bq);
  hipLaunchKernelGGL(k_build_tiles, dim3(D.BH), dim3(1024), 0, s, D, B);
  group_mass<T, DD>(q, D, B, s);
}

template <typename T, int DD>
static void plan_labels_impl(const void* qv, const void* kv, const int* klab, const int* qlab,
                             const long long* mass, const Dims& D, const Bufs& B, hipStream_t s) {
  const T* q = (const T*)qv;
  const T* k = (const T*)kv;
  // key side
  hipLaunchKernelGGL(k_state_reset, dim3((D.BH + 63) / 64), dim3(64), 0, s, B.kst, D.BH, D.Ck, 1);
  hipLaunchKernelGGL(k_labels_given, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, klab, D, B, B.kst);
  hipLaunchKernelGGL(k_km_scan_groups, dim3(D.Ck, D.BH), dim3(64), 0, s, D, B, D.Ck, B.kst, 1);
  hipLaunchKernelGGL(k_km_scan_head, dim3(D.BH), dim3(256), 0, s, D, B, D.Ck, B.kst, 1);
  hipLaunchKernelGGL(k_km_scatter, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, D, B, B.kst, 1, B.kperm);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Ck, B.kst, B.klab, B.koff, D.Ck + 1);
  hipLaunchKernelGGL((k_key_centroids<T, DD>), dim3(D.Ck, D.BH), dim3(256), 0, s, k, D, B);
  // query side
  hipLaunchKernelGGL(k_state_reset, dim3((D.BH + 63) / 64), dim3(64), 0, s, B.qst, D.BH, D.Cq, 1);
  hipLaunchKernelGGL(k_labels_given, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, qlab, D, B, B.qst);
  hipLaunchKernelGGL(k_km_scan_groups, dim3(D.Cq, D.BH), dim3(64), 0, s, D, B, D.Cq, B.qst, 1);
  hipLaunchKernelGGL(k_km_scan_head, dim3(D.BH), dim3(256), 0, s, D, B, D.Cq, B.qst, 1);
  hipLaunchKernelGGL(k_km_scatter, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, D, B, B.qst, 1, B.qperm);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Cq, B.qst, B.qlab, B.qoff, D.Cq + 1);
  // query scales (as the planner computes them) for the warm-start representatives
  const Bufs Bq = query_side<T, DD>(q, D, B, s);
  hipLaunchKernelGGL((k_query_reps<T, DD>), dim3(D.Cq, D.BH), dim3(256), 0, s, q, D, Bq);
  hipLaunchKernelGGL(k_build_tiles, dim3(D.BH), dim3(1024), 0, s, D, B);
  if (mass) {
    (void)hipMemcpyAsync(B.u, mass, sizeof(long long) * (size_t)D.BH * D.Cq * D.Ck, hipMemcpyDeviceToDevice, s);
  } else {
    group_mass<T, DD>(q, D, B, s);
  }
}

void launch_plan(const void* q, const void* k, const Dims& D, const Bufs& B, hipStream_t s) {
  SPR_DISPATCH(D.dtype, D.d, plan_impl, q, k, D, B, s);
}

void launch_plan_warm(const void* q, const void* k, const Dims& D, const Bufs& B, hipStream_t s) {
  SPR_DISPATCH(D.dtype, D.d, plan_warm_impl, q, k, D, B, s);
}

void launch_plan_from_labels(const void* q, const void* k, const int* klab, const int* qlab,
                             const long long* mass, const Dims& D, const Bufs& B, hipStream_t s) {
  SPR_DISPATCH(D.dtype, D.d, plan_labels_impl, q, k, klab, qlab, mass, D, B, s);
}

// Steps shared by both planners: routing, probes, attention tiles.
void launch_route_probes(const Dims& D, const Bufs& B, hipStream_t s) {
  hipLaunchKernelGGL(k_route_sort, dim3(D.Cq, D.BH), dim3(256), 0, s, D, B);
  hipLaunchKernelGGL(k_route_tau, dim3(D.BH), dim3(1024), 0, s, D, B);
  hipLaunchKernelGGL(k_route_emit, dim3(D.Cq, D.BH), dim3(256), 0, s, D, B);
  if (D.dtype == 1 && D.attn_w == 8) {
    // the 8-wave attention's key order and its runs (on small calls, whose 4-wave tiles are
    // short, the three launches cost more than the shorter runs save; the fp32 kernel reads
    // the route itself)
    hipLaunchKernelGGL(k_key_order, dim3(D.BH), dim3(1024), 0, s, D, B);
    hipLaunchKernelGGL(k_att_runs, dim3(D.Cq, D.BH), dim3(256), 0, s, D, B);
    hipLaunchKernelGGL(k_att_perm, dim3(D.Ck, D.BH), dim3(256), 0, s, D, B);
  }
  hipLaunchKernelGGL(k_fill_i32, dim3(256), dim3(256), 0, s, B.pslot, (long long)D.BH * D.N, -1);
  if (D.M > 0 && D.probe_sel == 0) {
    hipLaunchKernelGGL(k_probe_alloc, dim3(D.BH), dim3(1024), 0, s, D, B);
    hipLaunchKernelGGL(k_select_probes, dim3(D.Cq, D.BH), dim3(256), 0, s, D, B);
  } else if (D.M > 0) {
    hipLaunchKernelGGL(k_select_probes_plain, dim3(D.BH), dim3(1024), 0, s, D, B);
  }
}

template <typename T, int DD>
static void permute_impl(const void* k, const void* v, const Dims& D, const Bufs& B, const int* perm, hipStream_t s) {
  hipLaunchKernelGGL((k_permute_kv<T, DD>), dim3(D.Npad / 64, D.BH), dim3(256), 0, s, (const T*)k, (const T*)v,
                     perm, D.N, D.Npad, (T*)B.kp, (T*)B.vpt);
}

void launch_permute_kv(const void* k, const void* v, const Dims& D, const Bufs& B, const int* perm, hipStream_t s) {
  SPR_DISPATCH(D.dtype, D.d, permute_impl, k, v, D, B, perm, s);
}

void launch_residual_projector(const Dims& D, const Bufs& B, hipStream_t s) {
  bf16* none = nullptr;
  if (D.d == 128)
    hipLaunchKernelGGL((k_top_rank<128, true>), dim3(D.BH), dim3(1024), 0, s, (const float*)B.rcov, B.rproj, none, none,
                       D.output_rank);
  else
    hipLaunchKernelGGL((k_top_rank<64, true>), dim3(D.BH), dim3(1024), 0, s, (const float*)B.rcov, B.rproj, none, none,
                       D.output_rank);
}

void launch_fill_i32(int* p, long long n, int v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_i32, dim3(64), dim3(256), 0, s, p, n, v);
}

void launch_pair_tiles(const Dims& D, const Bufs& B, hipStream_t s) {
  hipLaunchKernelGGL(k_pair_tiles, dim3(D.BH), dim3(1024), 0, s, D, B);
}

void launch_identity_plan(const Dims& D, const Bufs& B, hipStream_t s) {
  hipLaunchKernelGGL(k_identity_plan, dim3(64, D.BH), dim3(256), 0, s, D, B);
  hipLaunchKernelGGL(k_build_tiles, dim3(D.BH), dim3(1024), 0, s, D, B);
}

}  // namespace spr
