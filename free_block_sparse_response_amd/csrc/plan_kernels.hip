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

// =====================================================================================
// Selection of the m candidates with the smallest (hash, id), output in ascending id
// order. Candidates are cand(0..n-1), ascending. Radix select over the 64-bit hash
// finds the m-th smallest value T exactly; ties at T are broken by id.
// =====================================================================================
template <int BT, typename Cand>
__device__ void select_smallest(int n, int m, Cand cand, uint64_t base, int* out) {
  __shared__ int hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_k;
  __shared__ int ws[BT / kWave];
  const int tid = threadIdx.x;
  if (m <= 0) return;
  if (m >= n) {
    for (int i = tid; i < n; i += BT) out[i] = cand(i);
    return;
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
    if (tid == 0) {
      int c = 0, dg = 0;
      for (dg = 0; dg < 255; ++dg) {
        if (c + hist[dg] >= k) break;
        c += hist[dg];
      }
      s_prefix = prefix | ((uint64_t)dg << shift);
      s_k = k - c;
    }
    __syncthreads();
    prefix = s_prefix;
    k = s_k;
    __syncthreads();
  }
  int run_sel = 0, run_eq = 0;
  for (int c0 = 0; c0 < n; c0 += BT) {
    const int i = c0 + tid;
    const bool valid = i < n;
    const int id = valid ? cand(i) : 0;
    const uint64_t h = valid ? splitmix64(base ^ (uint64_t)(uint32_t)id) : 0ull;
    const bool lt = valid && h < prefix;
    const bool eq = valid && h == prefix;
    int eq_tot, sel_tot;
    const int eq_rank = block_excl_scan_bool<BT>(eq, &eq_tot, ws) + run_eq;
    const bool sel = lt || (eq && eq_rank < k);
    const int pos = block_excl_scan_bool<BT>(sel, &sel_tot, ws) + run_sel;
    if (sel) out[pos] = id;
    run_eq += eq_tot;
    run_sel += sel_tot;
  }
}

__global__ __launch_bounds__(1024) void k_select_all(int N, int m, uint64_t seed, uint64_t stream,
                                                     int* out, int out_stride) {
  const int bh = blockIdx.x;
  const uint64_t base = head_hash_base(seed, stream, (uint64_t)bh);
  select_smallest<1024>(N, m, [](int i) { return i; }, base, out + (size_t)bh * out_stride);
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

// G = scale2 * sum_r rows_r^T rows_r over the first count rows (count from KmState when given).
template <int DD>
__global__ __launch_bounds__(256) void k_gram(const float* rows, int R, const KmState* cnt_state, float scale2,
                                              float* G) {
  constexpr int E = DD * DD / 256;
  constexpr int CH = 32;
  __shared__ float sh[CH][DD];
  const int bh = blockIdx.x;
  const int n = cnt_state ? cnt_state[bh].c_final : R;
  const float* src = rows + (size_t)bh * R * DD;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int r0 = 0; r0 < n; r0 += CH) {
    __syncthreads();
    for (int i = threadIdx.x; i < CH * DD; i += 256) {
      const int r = i / DD, c = i % DD;
      sh[r][c] = (r0 + r < n) ? src[(size_t)(r0 + r) * DD + c] : 0.f;
    }
    __syncthreads();
    const int rmax = min(CH, n - r0);
    for (int r = 0; r < rmax; ++r) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int idx = threadIdx.x + 256 * e;
        acc[e] += sh[r][idx / DD] * sh[r][idx % DD];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) G[(size_t)bh * DD * DD + threadIdx.x + 256 * e] = scale2 * acc[e];
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
// m_b = alpha x_{init_b}; also resets the run state.
template <typename T, int DD>
__global__ __launch_bounds__(DD) void k_km_init(const T* x, Dims D, Bufs B, int C, KmState* st) {
  const int b = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  __shared__ float m[DD];
  __shared__ float red[DD / kWave];
  const int row = B.init_idx[(size_t)bh * D.C + b];
  float a = B.alpha ? B.alpha[(size_t)bh * D.N + row] : 1.f;
  const float v = a * to_f32(x[((size_t)bh * D.N + row) * DD + i]);
  m[i] = v;
  __syncthreads();
  const float* G = B.metric + (size_t)bh * DD * DD;
  float t = 0.f;
  for (int k = 0; k < DD; ++k) t = fmaf(G[(size_t)k * DD + i], m[k], t);
  const size_t o = ((size_t)bh * D.C + b) * DD + i;
  B.cent[o] = v;
  B.cent_t[o] = t;
  float p = wave_sum(v * t);
  if (lane_id() == 0) red[i / kWave] = p;
  __syncthreads();
  if (i == 0) {
    float s = 0.f;
    for (int w = 0; w < DD / kWave; ++w) s += red[w];
    B.cnorm[(size_t)bh * D.C + b] = s;
    if (b == 0) {
      st[bh].done_iter = 0x7fffffff;
      st[bh].iters = 0;
      st[bh].c_final = C;
      st[bh].prev = 0.0;
    }
  }
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
  int* tab = B.tab + (size_t)bh * D.C * D.nblk;
  for (int i = threadIdx.x; i < C; i += 256) tab[(size_t)i * D.nblk + blk] = hist[i];
}

// Per head: inertia, the stopping rule, group sizes and starts, per-(group, block)
// scatter offsets.
__global__ __launch_bounds__(1024) void k_km_scan(Dims D, Bufs B, int C, KmState* st, int t) {
  __shared__ long long wsl[16];
  __shared__ int gs[kMaxGroups];
  const int bh = blockIdx.x;
  if (st[bh].done_iter < t) return;
  const int w = threadIdx.x / kWave, l = lane_id();
  int* tab = B.tab + (size_t)bh * D.C * D.nblk;
  if (w == 0) {
    double s = 0.0;
    for (int i = l; i < D.nblk; i += kWave) s += B.ipart[(size_t)bh * D.nblk + i];
    s = wave_sum(s);
    if (l == 0) {
      const double prev = st[bh].prev;
      int done = st[bh].done_iter;
      if (t > 1 && prev - s <= (double)D.tol * prev) done = t;
      if (t >= D.max_iter) done = t;
      st[bh].done_iter = done;
      st[bh].prev = s;
      st[bh].iters = t;
    }
  }
  for (int b = w; b < C; b += 16) {
    int s = 0;
    for (int i = l; i < D.nblk; i += kWave) s += tab[(size_t)b * D.nblk + i];
    s = wave_sum_i(s);
    if (l == 0) gs[b] = s;
  }
  __syncthreads();
  long long tot;
  const long long cnt = threadIdx.x < C ? gs[threadIdx.x] : 0;
  const long long start = block_excl_scan<1024, long long>(cnt, &tot, wsl);
  if (threadIdx.x < C) {
    B.gcount[(size_t)bh * D.C + threadIdx.x] = (int)cnt;
    B.gstart[(size_t)bh * (D.C + 1) + threadIdx.x] = (int)start;
  }
  if (threadIdx.x == 0) B.gstart[(size_t)bh * (D.C + 1) + C] = (int)tot;
  __syncthreads();
  if (threadIdx.x < C) gs[threadIdx.x] = (int)start;
  __syncthreads();
  for (int b = w; b < C; b += 16) {
    int run = gs[b];
    for (int i0 = 0; i0 < D.nblk; i0 += kWave) {
      const int i = i0 + l;
      const int c = i < D.nblk ? tab[(size_t)b * D.nblk + i] : 0;
      const int inc = wave_incl_scan(c);
      if (i < D.nblk) tab[(size_t)b * D.nblk + i] = run + inc - c;
      run += __shfl(inc, kWave - 1, kWave);
    }
  }
}

__global__ __launch_bounds__(kKmRows) void k_km_scatter(Dims D, Bufs B, KmState* st, int t, int* perm) {
  const int blk = blockIdx.x, bh = blockIdx.y;
  if (st[bh].done_iter < t) return;
  const int row = blk * kKmRows + threadIdx.x;
  if (row >= D.N) return;
  const int lab = B.lab[(size_t)bh * D.N + row];
  const int pos = B.tab[((size_t)bh * D.C + lab) * D.nblk + blk] + B.rank[(size_t)bh * D.N + row];
  perm[(size_t)bh * D.N + pos] = row;
}

// Mean of the rows alpha_j x_j of group b, summed in group order; optionally G m_b and m_b G m_b.
template <typename T, int DD>
__device__ void group_mean(const T* xb, const float* alpha, const int* members, int n, float* m_out,
                           float* sh /* [256] */) {
  constexpr int RL = 256 / DD;  // row lanes
  const int c = threadIdx.x % DD, rl = threadIdx.x / DD;
  float s = 0.f;
  for (int r = rl; r < n; r += RL) {
    const int row = members[r];
    float v = to_f32(xb[(size_t)row * DD + c]);
    if (alpha) v *= alpha[row];
    s += v;
  }
  sh[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < DD) {
    float tot = 0.f;
    for (int q = 0; q < RL; ++q) tot += sh[q * DD + threadIdx.x];
    m_out[threadIdx.x] = tot / (float)n;
  }
  __syncthreads();
}

template <typename T, int DD>
__global__ __launch_bounds__(256) void k_km_update(const T* x, Dims D, Bufs B, KmState* st, int t, const int* perm) {
  __shared__ float sh[256];
  __shared__ float m[DD];
  __shared__ float red[4];
  const int b = blockIdx.x, bh = blockIdx.y;
  if (st[bh].done_iter <= t) return;
  const int n = B.gcount[(size_t)bh * D.C + b];
  if (n == 0) return;  // empty cluster keeps its centroid
  const int s0 = B.gstart[(size_t)bh * (D.C + 1) + b];
  const T* xb = x + (size_t)bh * D.N * DD;
  const float* alpha = B.alpha ? B.alpha + (size_t)bh * D.N : nullptr;
  group_mean<T, DD>(xb, alpha, perm + (size_t)bh * D.N + s0, n, m, sh);
  const float* G = B.metric + (size_t)bh * DD * DD;
  float p = 0.f;
  if (threadIdx.x < DD) {
    const int i = threadIdx.x;
    float tt = 0.f;
    for (int k = 0; k < DD; ++k) tt = fmaf(G[(size_t)k * DD + i], m[k], tt);
    const size_t o = ((size_t)bh * D.C + b) * DD + i;
    B.cent[o] = m[i];
    B.cent_t[o] = tt;
    p = m[i] * tt;
  }
  p = wave_sum(p);
  if (lane_id() == 0) red[threadIdx.x / kWave] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int w = 0; w < DD / kWave; ++w) s += red[w];
    B.cnorm[(size_t)bh * D.C + b] = s;
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
  __shared__ float sh[256];
  __shared__ float m[DD];
  const int b = blockIdx.x, bh = blockIdx.y;
  if (b >= B.kst[bh].c_final) return;
  const int* off = B.koff + (size_t)bh * (D.Ck + 1);
  const int s0 = off[b], n = off[b + 1] - off[b];
  group_mean<T, DD>(k + (size_t)bh * D.N * DD, nullptr, B.kperm + (size_t)bh * D.N + s0, n, m, sh);
  if (threadIdx.x < DD) B.kcent[((size_t)bh * D.Ck + b) * DD + threadIdx.x] = m[threadIdx.x];
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
    st[bh].prev = 0.0;
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
__global__ __launch_bounds__(1024) void k_route_sort(Dims D, Bufs B) {
  __shared__ unsigned long long key[kMaxGroups];
  __shared__ long long ws[16];
  const int a = blockIdx.x, bh = blockIdx.y;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  if (a >= Cq) return;
  const int tid = threadIdx.x;
  const long long* u = B.u + ((size_t)bh * D.Cq + a) * D.Ck;
  key[tid] = tid < Ck ? ((((1ull << 34) - 1ull - (unsigned long long)u[tid]) << 10) | (unsigned)tid) : ~0ull;
  __syncthreads();
  for (int size = 2; size <= kMaxGroups; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int p = tid ^ stride;
      if (p > tid) {
        const bool up = (tid & size) == 0;
        const unsigned long long x = key[tid], y = key[p];
        if ((x > y) == up) { key[tid] = y; key[p] = x; }
      }
      __syncthreads();
    }
  }
  const int* ko = B.koff + (size_t)bh * (D.Ck + 1);
  const int b = (int)(key[tid] & 1023ull);
  const long long mass = tid < Ck ? u[b] : 0;
  const long long nk = tid < Ck ? (long long)(ko[b + 1] - ko[b]) : 0;
  long long t1, t2;
  const long long cm = block_excl_scan<1024, long long>(mass, &t1, ws) + mass;
  const long long cn = block_excl_scan<1024, long long>(nk, &t2, ws) + nk;
  if (tid < Ck) {
    const size_t o = ((size_t)bh * D.Cq + a) * D.Ck + tid;
    const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
    B.sorted_b[o] = b;
    B.cum[o] = cm;
    B.ccost[o] = (long long)(qo[a + 1] - qo[a]) * cn;
  }
}

__device__ inline int route_take(const long long* cum, int Ck, long long tau) {
  int lo = 0, hi = Ck;  // first index with cum >= tau
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] >= tau) hi = mid; else lo = mid + 1;
  }
  return min(max(lo + 1, 1), Ck);
}

__global__ __launch_bounds__(1024) void k_route_tau(Dims D, Bufs B) {
  __shared__ long long ws[16];
  __shared__ int wsi[16];
  const int bh = blockIdx.x, a = threadIdx.x;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  const size_t ro = ((size_t)bh * D.Cq + a) * D.Ck;
  const long long* cum = B.cum + ro;
  const long long* cc = B.ccost + ro;
  auto cost = [&](long long tau) -> long long {
    const long long c = a < Cq ? cc[route_take(cum, Ck, tau) - 1] : 0;
    return block_sum<1024, long long>(c, ws);
  };
  const long long budget = D.budget;
  long long hi = (1ll << 32) + Ck, tau;
  int exceeded = 0;
  if (cost(0) > budget) {
    tau = 0;
    exceeded = 1;
  } else if (cost(hi) <= budget) {
    tau = hi;
  } else {
    long long lo = 0;
    while (hi - lo > 1) {
      const long long mid = (lo + hi) >> 1;
      if (cost(mid) <= budget) lo = mid; else hi = mid;
    }
    tau = lo;
  }
  const int j = a < Cq ? route_take(cum, Ck, tau) : 0;
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
__global__ __launch_bounds__(1024) void k_route_emit(Dims D, Bufs B) {
  __shared__ int flag[kMaxGroups];
  __shared__ int ws[16];
  const int a = blockIdx.x, bh = blockIdx.y;
  const int Cq = B.qst[bh].c_final, Ck = B.kst[bh].c_final;
  if (a >= Cq) return;
  const int tid = threadIdx.x;
  flag[tid] = 0;
  __syncthreads();
  const int j = B.jsel[(size_t)bh * D.Cq + a];
  if (tid < j) flag[B.sorted_b[((size_t)bh * D.Cq + a) * D.Ck + tid]] = 1;
  __syncthreads();
  int tot;
  const bool f = tid < Ck && flag[tid];
  const int pos = block_excl_scan_bool<1024>(f, &tot, ws);
  if (f) B.cols[(size_t)bh * D.Cq * D.Ck + B.row_ptr[(size_t)bh * (D.Cq + 1) + a] + pos] = tid;
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
// Attention tiles: kAttnQT consecutive positions of one query group.
// =====================================================================================
__global__ __launch_bounds__(1024) void k_build_tiles(Dims D, Bufs B) {
  __shared__ int ws[16];
  __shared__ int tstart[kMaxGroups + 1];
  const int bh = blockIdx.x, a = threadIdx.x;
  const int Cq = B.qst[bh].c_final;
  const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
  const int nt = a < Cq ? ceil_div(qo[a + 1] - qo[a], D.qt) : 0;
  int tot;
  const int s = block_excl_scan<1024, int>(nt, &tot, ws);
  tstart[a] = s;
  if (a == 0) {
    tstart[kMaxGroups] = tot;
    B.ntiles[bh] = tot;
  }
  __syncthreads();
  const int w = threadIdx.x / kWave, l = lane_id();
  int2* tiles = B.tiles + (size_t)bh * D.max_tiles;
  for (int g = w; g < Cq; g += 16) {
    const int n = ceil_div(qo[g + 1] - qo[g], D.qt);
    for (int t = l; t < n; t += kWave) tiles[tstart[g] + t] = make_int2(g, qo[g] + t * D.qt);
  }
}

// =====================================================================================
// Group-contiguous K and transposed V: Kp[pos] = K[perm[pos]], VpT[i][pos] = V[perm[pos]][i];
// positions N..Npad-1 are zero.
// =====================================================================================
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_permute_kv(const T* k, const T* v, const int* perm, int N, int Npad,
                                                    T* kp, T* vpt) {
  __shared__ T vs[64][DD + 2];
  const int p0 = blockIdx.x * 64, bh = blockIdx.y;
  const int* pb = perm + (size_t)bh * N;
  const T* kb = k + (size_t)bh * N * DD;
  const T* vb = v + (size_t)bh * N * DD;
  T* kpb = kp + (size_t)bh * Npad * DD;
  T* vtb = vpt + (size_t)bh * DD * Npad;
  for (int i = threadIdx.x; i < 64 * DD; i += 256) {
    const int r = i / DD, c = i % DD;
    const int pos = p0 + r;
    T kv = from_f32<T>(0.f), vv = from_f32<T>(0.f);
    if (pos < N) {
      const int src = pb[pos];
      kv = kb[(size_t)src * DD + c];
      vv = vb[(size_t)src * DD + c];
    }
    if (pos < Npad) kpb[(size_t)pos * DD + c] = kv;
    vs[r][c] = vv;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * DD; i += 256) {
    const int c = i / 64, r = i % 64;
    if (p0 + r < Npad) vtb[(size_t)c * Npad + p0 + r] = vs[r][c];
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

template <typename T, int DD>
static void run_lloyd(const void* xv, const Dims& D, const Bufs& B, int C, KmState* st, int* perm,
                      hipStream_t s) {
  const T* x = (const T*)xv;
  hipLaunchKernelGGL((k_km_init<T, DD>), dim3(C, D.BH), dim3(DD), 0, s, x, D, B, C, st);
  for (int t = 1; t <= D.max_iter; ++t) {
    hipLaunchKernelGGL((k_km_assign<T, DD>), dim3(D.nblk, D.BH), dim3(256), 0, s, x, D, B, C, st, t);
    hipLaunchKernelGGL(k_km_scan, dim3(D.BH), dim3(1024), 0, s, D, B, C, st, t);
    hipLaunchKernelGGL(k_km_scatter, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, D, B, st, t, perm);
    if (t < D.max_iter)
      hipLaunchKernelGGL((k_km_update<T, DD>), dim3(C, D.BH), dim3(256), 0, s, x, D, B, st, t, perm);
  }
}

template <typename T, int DD>
static void plan_impl(const void* qv, const void* kv, const Dims& D, const Bufs& B, hipStream_t s) {
  const T* q = (const T*)qv;
  const T* k = (const T*)kv;
  // 01: sampled queries and their key-response metric
  hipLaunchKernelGGL(k_select_all, dim3(D.BH), dim3(1024), 0, s, D.N, D.S, D.seed, (uint64_t)kStreamSampled,
                     B.sampled, D.S);
  hipLaunchKernelGGL((k_gather_rows<T>), dim3(D.S, D.BH), dim3(DD), 0, s, q, B.sampled, D.N, D.S, DD, B.qs);
  hipLaunchKernelGGL((k_gram<DD>), dim3(D.BH), dim3(256), 0, s, B.qs, D.S, (const KmState*)nullptr,
                     D.scale * D.scale, B.metric);
  // 02a: paired K/V groups by Lloyd on the key responses
  Bufs Bk = B;
  Bk.alpha = nullptr;
  hipLaunchKernelGGL((k_rowquad<T, DD>), dim3(D.nblk, D.BH), dim3(256), 0, s, k, D, B.metric, B.rowconst,
                     (float*)nullptr, (const KmState*)nullptr);
  hipLaunchKernelGGL(k_select_all, dim3(D.BH), dim3(1024), 0, s, D.N, D.Ck, D.seed, (uint64_t)kStreamKeyInit,
                     B.init_idx, D.C);
  run_lloyd<T, DD>(k, D, Bk, D.Ck, B.kst, B.kperm, s);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Ck, B.kst, B.klab, B.koff, D.Ck + 1);
  hipLaunchKernelGGL((k_key_centroids<T, DD>), dim3(D.Ck, D.BH), dim3(256), 0, s, k, D, B);
  // 02b: query-response coordinates (RMS-normalised) and query groups
  hipLaunchKernelGGL((k_gram<DD>), dim3(D.BH), dim3(256), 0, s, B.kcent, D.Ck, (const KmState*)B.kst, 1.f,
                     B.metric);
  hipLaunchKernelGGL((k_rowquad<T, DD>), dim3(D.nblk, D.BH), dim3(256), 0, s, q, D, B.metric, B.rowconst, B.alpha,
                     (const KmState*)B.kst);
  hipLaunchKernelGGL(k_select_all, dim3(D.BH), dim3(1024), 0, s, D.N, D.Cq, D.seed, (uint64_t)kStreamQueryInit,
                     B.init_idx, D.C);
  run_lloyd<T, DD>(q, D, B, D.Cq, B.qst, B.qperm, s);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Cq, B.qst, B.qlab, B.qoff, D.Cq + 1);
  // 03: group masses
  hipLaunchKernelGGL((k_group_mass<T, DD>), dim3(D.Cq, D.BH), dim3(256), 0, s, q, D, B);
}

template <typename T, int DD>
static void plan_labels_impl(const void* qv, const void* kv, const int* klab, const int* qlab,
                             const long long* mass, const Dims& D, const Bufs& B, hipStream_t s) {
  const T* q = (const T*)qv;
  const T* k = (const T*)kv;
  // key side
  hipLaunchKernelGGL(k_state_reset, dim3((D.BH + 63) / 64), dim3(64), 0, s, B.kst, D.BH, D.Ck, 1);
  hipLaunchKernelGGL(k_labels_given, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, klab, D, B, B.kst);
  hipLaunchKernelGGL(k_km_scan, dim3(D.BH), dim3(1024), 0, s, D, B, D.Ck, B.kst, 1);
  hipLaunchKernelGGL(k_km_scatter, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, D, B, B.kst, 1, B.kperm);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Ck, B.kst, B.klab, B.koff, D.Ck + 1);
  hipLaunchKernelGGL((k_key_centroids<T, DD>), dim3(D.Ck, D.BH), dim3(256), 0, s, k, D, B);
  // query side
  hipLaunchKernelGGL(k_state_reset, dim3((D.BH + 63) / 64), dim3(64), 0, s, B.qst, D.BH, D.Cq, 1);
  hipLaunchKernelGGL(k_labels_given, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, qlab, D, B, B.qst);
  hipLaunchKernelGGL(k_km_scan, dim3(D.BH), dim3(1024), 0, s, D, B, D.Cq, B.qst, 1);
  hipLaunchKernelGGL(k_km_scatter, dim3(D.nblk, D.BH), dim3(kKmRows), 0, s, D, B, B.qst, 1, B.qperm);
  hipLaunchKernelGGL(k_km_compact, dim3(D.BH), dim3(1024), 0, s, D, B, D.Cq, B.qst, B.qlab, B.qoff, D.Cq + 1);
  if (mass) {
    (void)hipMemcpyAsync(B.u, mass, sizeof(long long) * (size_t)D.BH * D.Cq * D.Ck, hipMemcpyDeviceToDevice, s);
  } else {
    hipLaunchKernelGGL((k_group_mass<T, DD>), dim3(D.Cq, D.BH), dim3(256), 0, s, q, D, B);
  }
}

void launch_plan(const void* q, const void* k, const Dims& D, const Bufs& B, hipStream_t s) {
  SPR_DISPATCH(D.dtype, D.d, plan_impl, q, k, D, B, s);
}

void launch_plan_from_labels(const void* q, const void* k, const int* klab, const int* qlab,
                             const long long* mass, const Dims& D, const Bufs& B, hipStream_t s) {
  SPR_DISPATCH(D.dtype, D.d, plan_labels_impl, q, k, klab, qlab, mass, D, B, s);
}

// Steps shared by both planners: routing, probes, attention tiles.
void launch_route_probes(const Dims& D, const Bufs& B, hipStream_t s) {
  hipLaunchKernelGGL(k_route_sort, dim3(D.Cq, D.BH), dim3(1024), 0, s, D, B);
  hipLaunchKernelGGL(k_route_tau, dim3(D.BH), dim3(1024), 0, s, D, B);
  hipLaunchKernelGGL(k_route_emit, dim3(D.Cq, D.BH), dim3(1024), 0, s, D, B);
  hipLaunchKernelGGL(k_fill_i32, dim3(256), dim3(256), 0, s, B.pslot, (long long)D.BH * D.N, -1);
  if (D.M > 0) {
    hipLaunchKernelGGL(k_probe_alloc, dim3(D.BH), dim3(1024), 0, s, D, B);
    hipLaunchKernelGGL(k_select_probes, dim3(D.Cq, D.BH), dim3(256), 0, s, D, B);
  }
  hipLaunchKernelGGL(k_build_tiles, dim3(D.BH), dim3(1024), 0, s, D, B);
}

template <typename T, int DD>
static void permute_impl(const void* k, const void* v, const Dims& D, const Bufs& B, hipStream_t s) {
  hipLaunchKernelGGL((k_permute_kv<T, DD>), dim3(D.Npad / 64, D.BH), dim3(256), 0, s, (const T*)k, (const T*)v,
                     B.kperm, D.N, D.Npad, (T*)B.kp, (T*)B.vpt);
}

void launch_permute_kv(const void* k, const void* v, const Dims& D, const Bufs& B, hipStream_t s) {
  SPR_DISPATCH(D.dtype, D.d, permute_impl, k, v, D, B, s);
}

void launch_fill_i32(int* p, long long n, int v, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_i32, dim3(64), dim3(256), 0, s, p, n, v);
}

void launch_identity_plan(const Dims& D, const Bufs& B, hipStream_t s) {
  hipLaunchKernelGGL(k_identity_plan, dim3(64, D.BH), dim3(256), 0, s, D, B);
  hipLaunchKernelGGL(k_build_tiles, dim3(D.BH), dim3(1024), 0, s, D, B);
}

}  // namespace spr
