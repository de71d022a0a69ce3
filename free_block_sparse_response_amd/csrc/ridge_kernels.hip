// Probe-Fitted Residual Reconstruction (paper "Partition the Support, Reconstruct the
// Residual", abstract; project website, PFRR panel): a weighted ridge fit of the affine map
// from a probe row's sparse output to its residual r = O_dense - O_sparse, then the
// predicted residual added to every unprobed row.
//
// Normal equations per head, in float64:
//   (Z^T W Z + Lambda) Theta = Z^T W R,  Z = [O_sp(probes), 1],  Lambda = diag(lambda 1_d, 0),
// built as one bordered matrix [A | B] (A (d+1)x(d+1), B (d+1)xd), then solved by a
// Cholesky factorisation held packed in LDS. A pivot at or below 1e-12 x max diag(A)
// marks the head numerically singular.
#include <type_traits>

#include "common.h"
#include "plan_state.h"
#include "launch.h"

namespace spr {

constexpr double kPivotRtol = 1e-12;

// [A | B] in 32x32 tiles; column j < d+1 of the left factor is Z, column j >= d+1 is R.
template <int DD>
__global__ __launch_bounds__(256) void k_ridge_gram(Dims D, Bufs B, const float* o_psp, const float* o_dn,
                                                    const float* weights) {
  constexpr int n = DD + 1;
  constexpr int W = n + DD;
  constexpr int PC = 32;  // probes per chunk
  __shared__ double Zi[PC][33];
  __shared__ double Zj[PC][33];
  __shared__ double wv[PC];
  const int bi = blockIdx.x, bj = blockIdx.y, bh = blockIdx.z;
  const int i0 = bi * 32, j0 = bj * 32;
  if (i0 >= n || j0 >= W) return;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 8 row groups of 4
  double acc[4] = {0, 0, 0, 0};
  const float* wp = weights ? weights + (size_t)bh * D.M : B.pweights + (size_t)bh * D.M;
  const float* zs = o_psp + (size_t)bh * D.M * DD;
  const float* zd = o_dn + (size_t)bh * D.M * DD;
  auto zval = [&](int p, int col) -> double {
    if (col < DD) return (double)zs[(size_t)p * DD + col];
    if (col == DD) return 1.0;
    const int c = col - n;
    return (double)zd[(size_t)p * DD + c] - (double)zs[(size_t)p * DD + c];
  };
  for (int p0 = 0; p0 < D.M; p0 += PC) {
    __syncthreads();
    for (int e = threadIdx.x; e < PC * 32; e += 256) {
      const int p = e / 32, c = e % 32;
      const bool pv = p0 + p < D.M;
      Zi[p][c] = (pv && i0 + c < n) ? zval(p0 + p, i0 + c) : 0.0;
      Zj[p][c] = (pv && j0 + c < W) ? zval(p0 + p, j0 + c) : 0.0;
    }
    if (threadIdx.x < PC) wv[threadIdx.x] = p0 + threadIdx.x < D.M ? (double)wp[p0 + threadIdx.x] : 0.0;
    __syncthreads();
    for (int p = 0; p < PC; ++p) {
      const double zj = wv[p] * Zj[p][tx];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fma(Zi[p][ty * 4 + r], zj, acc[r]);
    }
  }
  double* G = B.gram + (size_t)bh * n * W;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + ty * 4 + r, j = j0 + tx;
    if (i < n && j < W) {
      double v = acc[r];
      if (i == j && (i < DD || D.pen_bias)) v += (double)D.lambda;
      G[(size_t)i * W + j] = v;
    }
  }
}

// One block of 512 threads per (head, 32 right-hand-side columns); each block redoes the
// elimination of A. A = L1 Dg L1^T (unit lower L1, pivots Dg) by Gaussian elimination
// without pivoting -- the Cholesky factorisation up to the scaling sqrt(Dg), stable for
// symmetric positive definite A -- with the same row operations on the right-hand side,
// Z = L1^-1 B, then L1^T X = Dg^-1 Z.
//
// The system lives in registers: thread (ty, tx) of a 16 x 32 grid holds A(i, k) for
// i = ty + 16 r, k = tx + 32 q and B(i, c0 + tx). Elimination goes by panels of 3 columns:
// the panel's owners publish its columns and right-hand-side rows in LDS (double-buffered,
// so one barrier per panel), every thread factors the 3 x 3 diagonal block itself
// (identical arithmetic everywhere, so a failed pivot stops all threads together), forms
// the multipliers of its own rows and applies the rank-3 update to its elements. The back
// substitution runs panel by panel from the last, publishing panel rows of L1 and of the
// right-hand side the same way. A pivot at or below 1e-12 x max diag(A) (the squared
// Cholesky diagonal) fails the head.
template <int DD>
__global__ __launch_bounds__(512) void k_ridge_solve(Dims D, Bufs B, float* coeffs) {
  constexpr int n = DD + 1;
  constexpr int W = n + DD;
  constexpr int CB = 32;  // right-hand-side columns per block
  constexpr int TY = 16, TX = 32;
  constexpr int RT = (n + TY - 1) / TY;  // rows per thread
  constexpr int QT = (n + TX - 1) / TX;  // matrix columns per thread
  constexpr int NP = RT * TY > QT * TX ? RT * TY : QT * TX;  // padded index range
  constexpr int P = 3;                   // panel width (n = 129 = 43 panels)
  __shared__ double cb[2][P][NP];        // panel columns / panel rows of L1
  __shared__ double rb[2][P][CB];        // panel rows of the right-hand side
  __shared__ double piv[NP];
  __shared__ double s_floor;
  const int bh = blockIdx.y, c0 = blockIdx.x * CB;
  const int tid = threadIdx.x, ty = tid / TX, tx = tid % TX;
  float* Th = coeffs + (size_t)bh * n * DD;
  const bool col_ok = c0 + tx < DD;
  if (D.M == 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int i = ty + TY * r;
      if (i < n && col_ok) Th[(size_t)i * DD + c0 + tx] = 0.f;
    }
    return;
  }
  const double* G = B.gram + (size_t)bh * n * W;
  double a[RT][QT], b[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int i = ty + TY * r;
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      const int k = tx + TX * q;
      a[r][q] = (i < n && k < n) ? G[(size_t)i * W + k] : 0.0;
    }
    b[r] = (i < n && col_ok) ? G[(size_t)i * W + n + c0 + tx] : 0.0;
  }
  // entries never published stay zero (indices beyond n)
  for (int e = tid; e < 2 * P * NP; e += 512) (&cb[0][0][0])[e] = 0.0;
  for (int e = tid; e < 2 * P * CB; e += 512) (&rb[0][0][0])[e] = 0.0;
  if (tid < 64) {
    double mx = 0.0;
    for (int i = tid; i < n; i += 64) mx = fmax(mx, G[(size_t)i * W + i]);
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
    if (tid == 0) s_floor = kPivotRtol * mx;
  }
  __syncthreads();
  const double floor_ = s_floor;
  bool fail = false;
  int buf = 0;
  for (int j0 = 0; j0 < n; j0 += P, buf ^= 1) {
    const int pw = min(P, n - j0);
    // owners publish the panel columns (rows >= j0) and the panel rows of the right-hand side.
    // Here and below, a block of TY rows or TX columns that lies wholly before j0 is skipped:
    // its entries are final (block-uniform branches).
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      if (TX * q + TX <= j0) continue;
      const int pc = tx + TX * q - j0;
      if (pc >= 0 && pc < pw) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          if (TY * r + TY <= j0) continue;
          const int i = ty + TY * r;
          if (i >= j0 && i < n) cb[buf][pc][i] = a[r][q];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (TY * r + TY <= j0) continue;
      const int pr = ty + TY * r - j0;
      if (pr >= 0 && pr < pw) rb[buf][pr][tx] = b[r];
    }
    __syncthreads();
    // the diagonal block, factored by every thread alike: Lb unit lower, db pivots; entries
    // beyond the panel width are zero (their reciprocal pivots too)
    double Lb[P][P], db[P], rd[P];
#pragma unroll
    for (int p1 = 0; p1 < P; ++p1) {
      const bool in1 = p1 < pw;
#pragma unroll
      for (int p2 = 0; p2 < p1; ++p2) {
        double v = cb[buf][p2][j0 + p1];
#pragma unroll
        for (int m = 0; m < p2; ++m) v -= Lb[p1][m] * Lb[p2][m] * db[m];
        Lb[p1][p2] = in1 ? v * rd[p2] : 0.0;
      }
      double d = cb[buf][p1][j0 + p1];
#pragma unroll
      for (int m = 0; m < p1; ++m) d -= Lb[p1][m] * Lb[p1][m] * db[m];
      db[p1] = in1 ? d : 1.0;
      rd[p1] = in1 ? 1.0 / d : 0.0;
      fail |= in1 && !(d > floor_);
    }
    if (fail) break;
    if (tid == 0) {
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (p < pw) piv[j0 + p] = db[p];
    }
    // the panel entries of my columns, solved (y Lb^T = c); zero unless a trailing column
    double yq[QT][P];
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      if (TX * q + TX <= j0) continue;  // (yq of such a block is never read)
      const int k = tx + TX * q;
      const bool tk = k >= j0 + pw && k < n;
      double y[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        double v = cb[buf][p][k];
#pragma unroll
        for (int m = 0; m < p; ++m) v -= y[m] * Lb[p][m];
        y[p] = v;
        yq[q][p] = (tk && p < pw) ? v : 0.0;
      }
    }
    // right-hand side of the panel: z = Lb^-1 b_J
    double z[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      double v = rb[buf][p][tx];
#pragma unroll
      for (int m = 0; m < p; ++m) v -= Lb[p][m] * z[m];
      z[p] = p < pw ? v : 0.0;
    }
    // row by row: the multipliers of my row (below the diagonal of a panel column they are
    // L1's entries, for the panel's own rows too), the rank-pw update of a trailing row and
    // its right-hand side; the panel rows of the right-hand side take z
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (TY * r + TY <= j0) continue;
      const int i = ty + TY * r;
      const bool tr = i >= j0 + pw && i < n;
      double lf[P], li[P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        double v = cb[buf][p][i];
#pragma unroll
        for (int m = 0; m < p; ++m) v -= lf[m] * db[m] * Lb[p][m];
        lf[p] = v * rd[p];
        li[p] = tr ? lf[p] : 0.0;
      }
#pragma unroll
      for (int q = 0; q < QT; ++q) {
        if (TX * q + TX <= j0) continue;
        double v = a[r][q];
#pragma unroll
        for (int p = 0; p < P; ++p) v -= li[p] * yq[q][p];
        const int k = tx + TX * q, pc = k - j0;
        if (pc >= 0 && pc < pw && i > k && i < n) {
          double m = lf[0];
#pragma unroll
          for (int u = 1; u < P; ++u) m = pc == u ? lf[u] : m;
          v = m;
        }
        a[r][q] = v;
      }
      double v = b[r];
#pragma unroll
      for (int p = 0; p < P; ++p) v -= li[p] * z[p];
      const int pr = i - j0;
      if (pr >= 0 && pr < pw) {
        double m = z[0];
#pragma unroll
        for (int u = 1; u < P; ++u) m = pr == u ? z[u] : m;
        v = m;
      }
      b[r] = v;
    }
  }
  if (fail) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int i = ty + TY * r;
      if (i < n && col_ok) Th[(size_t)i * DD + c0 + tx] = 0.f;
    }
    if (tid == 0) B.status[bh] = 5;  // SPARSEPR_ERR_NUMERICAL
    return;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int i = ty + TY * r;
    if (i < n) b[r] /= piv[i];
  }
  // ---- L1^T X = Dg^-1 Z, panels from the last
  for (int j0 = ((n - 1) / P) * P; j0 >= 0; j0 -= P, buf ^= 1) {
    const int pw = min(P, n - j0);
    // owners publish the panel rows: right-hand side, and L1 left of the diagonal
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (TY * r + TY <= j0 || TY * r >= j0 + pw) continue;
      const int i = ty + TY * r;
      const int pr = i - j0;
      if (pr >= 0 && pr < pw) {
        rb[buf][pr][tx] = b[r];
#pragma unroll
        for (int q = 0; q < QT; ++q) {
          const int k = tx + TX * q;
          if (k < i) cb[buf][pr][k] = a[r][q];
        }
      }
    }
    __syncthreads();
    // Lb^T x = z inside the panel, for my column
    double x[P];
#pragma unroll
    for (int p = P - 1; p >= 0; --p) {
      double v = rb[buf][p][tx];
#pragma unroll
      for (int m = p + 1; m < P; ++m) v -= cb[buf][m][j0 + p] * x[m];
      x[p] = p < pw ? v : 0.0;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (TY * r >= j0 + pw) continue;  // rows wholly after the panel are final
      const int i = ty + TY * r;
      double v = b[r];
      if (i < j0) {
#pragma unroll
        for (int p = 0; p < P; ++p) v -= cb[buf][p][i] * x[p];
      }
      const int pr = i - j0;
      if (pr >= 0 && pr < pw) {
        double m = x[0];
#pragma unroll
        for (int u = 1; u < P; ++u) m = pr == u ? x[u] : m;
        v = m;
      }
      b[r] = v;
    }
  }
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int i = ty + TY * r;
    if (i < n && col_ok) Th[(size_t)i * DD + c0 + tx] = (float)b[r];
  }
}

// out_i = o_i + [o_i, 1] Theta (unprobed rows); probe rows take their exact dense output.
// 64 rows per block; thread (ty, tx) owns rows 4ty..4ty+3 and columns tx*CT .. +CT-1.
template <typename T, int DD>
__global__ __launch_bounds__(256) void k_apply(Dims D, Bufs B, const T* o_sp, const float* o_dn, const float* coeffs,
                                               T* out) {
  constexpr int CT = DD / 16;
  __shared__ float Th[DD + 1][DD];
  __shared__ float Os[DD][64 + 4];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int r0 = blk * 64;
  const float* cf = coeffs + (size_t)bh * (DD + 1) * DD;
  for (int e = threadIdx.x; e < (DD + 1) * DD; e += 256) Th[e / DD][e % DD] = cf[e];
  for (int e = threadIdx.x; e < 64 * DD; e += 256) {
    const int r = e / DD, c = e % DD;
    const int row = r0 + r;
    Os[c][r] = row < D.N ? to_f32(o_sp[((size_t)bh * D.N + row) * DD + c]) : 0.f;
  }
  __syncthreads();
  const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
  float acc[4][CT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[r][c] = Th[DD][tx * CT + c];
  for (int k = 0; k < DD; ++k) {
    const float4 a = *reinterpret_cast<const float4*>(&Os[k][ty * 4]);
    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const float b = Th[k][tx * CT + c];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r][c] = fmaf(av[r], b, acc[r][c]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = r0 + ty * 4 + r;
    if (row >= D.N) continue;
    const int slot = D.M > 0 ? B.pslot[(size_t)bh * D.N + row] : -1;
    T* orow = out + ((size_t)bh * D.N + row) * DD;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int col = tx * CT + c;
      const float v = slot >= 0 ? o_dn[((size_t)bh * D.M + slot) * DD + col] : Os[col][ty * 4 + r] + acc[r][c];
      orow[col] = from_f32<T>(v);
    }
  }
}

// Theta^T split as bf16 hi + lo (row j = output dim, column k = input dim), once per head.
template <int DD>
__global__ __launch_bounds__(256) void k_theta_split(Dims D, Bufs B, const float* coeffs) {
  const int j0 = blockIdx.x * (256 / DD), bh = blockIdx.y;
  const int j = j0 + threadIdx.x / DD, k = threadIdx.x % DD;  // one Theta^T entry per thread
  const float v = coeffs[(size_t)bh * (DD + 1) * DD + (size_t)k * DD + j];
  const bf16 hb = (bf16)v;
  const size_t o = (size_t)bh * DD * DD + (size_t)j * DD + k;
  B.theta_h[o] = hb;
  B.theta_l[o] = (bf16)(v - (float)hb);
}

// bf16 apply on the matrix cores: Theta^T (hi + lo bf16, copied into LDS) times the exact
// bf16 row of o (transposed product: lane l owns row l % 32 of a 32-row set and 16 output
// dims per 32-dim block); each wave owns RS row sets so every operand read feeds RS
// products. The epilogue adds o and the bias; probe rows take o_dense.
template <int DD, int RS>
__global__ __launch_bounds__(256) void k_apply_bf16(Dims D, Bufs B, const bf16* o_sp, const float* o_dn,
                                                    const float* coeffs, bf16* out) {
  constexpr int KS = DD + 8;
  __shared__ __attribute__((aligned(16))) bf16 Th[DD * KS];
  __shared__ __attribute__((aligned(16))) bf16 Tl[DD * KS];
  __shared__ float bias[DD];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid / kWave, l32 = lane_id() & 31, h = lane_id() >> 5;
  const bf16* sh = B.theta_h + (size_t)bh * DD * DD;
  const bf16* sl = B.theta_l + (size_t)bh * DD * DD;
  for (int e = tid; e < DD * DD / 8; e += 256) {
    const int r = e / (DD / 8), c8 = (e % (DD / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&Th[r * KS + c8]) = *reinterpret_cast<const bf16x8*>(sh + (size_t)r * DD + c8);
    *reinterpret_cast<bf16x8*>(&Tl[r * KS + c8]) = *reinterpret_cast<const bf16x8*>(sl + (size_t)r * DD + c8);
  }
  if (tid < DD) bias[tid] = coeffs[(size_t)bh * (DD + 1) * DD + (size_t)DD * DD + tid];
  int row[RS], slot[RS];
  bf16x8 xr[RS][DD / 16];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    row[rs] = blk * 128 * RS + 128 * rs + 32 * w + l32;
    const bool valid = row[rs] < D.N;
    const bf16* orow = o_sp + ((size_t)bh * D.N + (valid ? row[rs] : D.N - 1)) * DD;
#pragma unroll
    for (int c = 0; c < DD / 16; ++c) xr[rs][c] = *reinterpret_cast<const bf16x8*>(orow + 16 * c + 8 * h);
    slot[rs] = (valid && D.M > 0) ? B.pslot[(size_t)bh * D.N + row[rs]] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int jb = 0; jb < DD; jb += 32) {
    f32x16 acc[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rs][v] = 0.f;
#pragma unroll
    for (int c = 0; c < DD / 16; ++c) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Th[(jb + l32) * KS + 16 * c + 8 * h]);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Tl[(jb + l32) * KS + 16 * c + 8 * h]);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        acc[rs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xr[rs][c], acc[rs], 0, 0, 0);
        acc[rs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xr[rs][c], acc[rs], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      // o's own entries for the output layout (dims jb + 8 g + 4 h + r) come from the operand
      // registers: the 16 dims of chunk c sit 8 per lane half, and swapping dwords 0, 1 of
      // the upper half with dwords 2, 3 of the lower one gives each lane its two runs of 4
      uint32_t xo[2][4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bf16x8 xc = xr[rs][jb / 16 + q];
        uint32_t dw[4];
        __builtin_memcpy(dw, &xc, 16);
        const auto s02 = __builtin_amdgcn_permlane32_swap(dw[0], dw[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(dw[1], dw[3], false, false);
        xo[q][0] = s02[0];
        xo[q][1] = s13[0];
        xo[q][2] = s02[1];
        xo[q][3] = s13[1];
      }
      if (row[rs] >= D.N) continue;
      bf16* dst = out + ((size_t)bh * D.N + row[rs]) * DD;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = jb + 8 * g + 4 * h;
        bf16x4 ov;
        if (slot[rs] >= 0) {
          const float4 dv = *reinterpret_cast<const float4*>(o_dn + ((size_t)bh * D.M + slot[rs]) * DD + j);
          ov[0] = (bf16)dv.x; ov[1] = (bf16)dv.y; ov[2] = (bf16)dv.z; ov[3] = (bf16)dv.w;
        } else {
          bf16x4 xv;
          const uint32_t pr[2] = {xo[g >> 1][2 * (g & 1)], xo[g >> 1][2 * (g & 1) + 1]};
          __builtin_memcpy(&xv, pr, 8);
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = (bf16)((float)xv[r] + acc[rs][4 * g + r] + bias[j + r]);
        }
        *reinterpret_cast<bf16x4*>(dst + j) = ov;
      }
    }
  }
}

// Output truncation of the fit: C = R^T W R (d x d) of the probe residuals R = o_dense -
// o_sparse, in 32 x 32 tiles, float64 sums over the probes in order.
template <int DD>
__global__ __launch_bounds__(256) void k_resid_cov(Dims D, Bufs B, const float* o_psp, const float* o_dn,
                                                   const float* weights) {
  constexpr int PC = 32;  // probes per chunk
  __shared__ double Ri[PC][33];
  __shared__ double Rj[PC][33];
  __shared__ double wv[PC];
  const int i0 = blockIdx.x * 32, j0 = blockIdx.y * 32, bh = blockIdx.z;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 8 row groups of 4
  double acc[4] = {0, 0, 0, 0};
  const float* wp = weights ? weights + (size_t)bh * D.M : B.pweights + (size_t)bh * D.M;
  const float* zs = o_psp + (size_t)bh * D.M * DD;
  const float* zd = o_dn + (size_t)bh * D.M * DD;
  for (int p0 = 0; p0 < D.M; p0 += PC) {
    __syncthreads();
    for (int e = threadIdx.x; e < PC * 32; e += 256) {
      const int p = e / 32, c = e % 32;
      const bool pv = p0 + p < D.M;
      const size_t o = (size_t)(p0 + p) * DD;
      Ri[p][c] = pv ? (double)zd[o + i0 + c] - (double)zs[o + i0 + c] : 0.0;
      Rj[p][c] = pv ? (double)zd[o + j0 + c] - (double)zs[o + j0 + c] : 0.0;
    }
    if (threadIdx.x < PC) wv[threadIdx.x] = p0 + threadIdx.x < D.M ? (double)wp[p0 + threadIdx.x] : 0.0;
    __syncthreads();
    for (int p = 0; p < PC; ++p) {
      const double rj = wv[p] * Rj[p][tx];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fma(Ri[p][ty * 4 + r], rj, acc[r]);
    }
  }
  float* C = B.rcov + (size_t)bh * DD * DD;
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(size_t)(i0 + ty * 4 + r) * DD + j0 + tx] = (float)acc[r];
}

// Theta <- Theta P in place (rows of [(d+1) x d] Theta times the d x d projector): the
// predicted residual [o, 1] Theta lands in the probe residuals' leading directions.
template <int DD>
__global__ __launch_bounds__(256) void k_theta_project(Dims D, Bufs B, float* coeffs) {
  constexpr int RB = 8;  // rows of Theta per block
  __shared__ float P[DD * DD];
  __shared__ float T[RB][DD];
  const int r0 = blockIdx.x * RB, bh = blockIdx.y;
  const float* Pg = B.rproj + (size_t)bh * DD * DD;
  float* Th = coeffs + (size_t)bh * (DD + 1) * DD;
  for (int e = threadIdx.x; e < DD * DD; e += 256) P[e] = Pg[e];
  for (int e = threadIdx.x; e < RB * DD; e += 256) {
    const int r = r0 + e / DD;
    T[e / DD][e % DD] = r <= DD ? Th[(size_t)r * DD + e % DD] : 0.f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < RB * DD; e += 256) {
    const int rr = e / DD, j = e % DD, r = r0 + rr;
    if (r > DD) continue;
    float acc = 0.f;
    for (int k = 0; k < DD; ++k) acc = fmaf(T[rr][k], P[k * DD + j], acc);
    Th[(size_t)r * DD + j] = acc;
  }
}

// Correction families other than the ridge (paper Table 4 "Mean-only"; repair disabled in
// the Table 2 partition rows): Theta = 0 except the bias row, which is the weighted mean
// probe residual (mean-only) or zero (none). Probes summed in order; fp64 accumulation.
template <int DD>
__global__ __launch_bounds__(DD) void k_fit_mean(Dims D, Bufs B, const float* o_psp, const float* o_dn,
                                                 const float* weights, float* coeffs) {
  const int bh = blockIdx.x, i = threadIdx.x;
  float* th = coeffs + (size_t)bh * (DD + 1) * DD;
  for (int r = 0; r < DD; ++r) th[(size_t)r * DD + i] = 0.f;
  double num = 0.0, den = 0.0;
  if (D.correction == 1) {
    const float* wp = weights ? weights + (size_t)bh * D.M : B.pweights + (size_t)bh * D.M;
    for (int p = 0; p < D.M; ++p) {
      const size_t o = ((size_t)bh * D.M + p) * DD + i;
      num += (double)wp[p] * ((double)o_dn[o] - (double)o_psp[o]);
      den += (double)wp[p];
    }
  }
  th[(size_t)DD * DD + i] = den > 0.0 ? (float)(num / den) : 0.f;
}

template <int DD>
static void fit_impl(const Dims& D, const Bufs& B, const float* o_psp, const float* o_dn, const float* w, float* coeffs,
                     hipStream_t s) {
  constexpr int n = DD + 1;
  if (D.correction != 0) {
    hipLaunchKernelGGL((k_fit_mean<DD>), dim3(D.BH), dim3(DD), 0, s, D, B, o_psp, o_dn, w, coeffs);
    return;
  }
  if (D.M > 0) {
    dim3 g((n + 31) / 32, (n + DD + 31) / 32, D.BH);
    hipLaunchKernelGGL((k_ridge_gram<DD>), g, dim3(256), 0, s, D, B, o_psp, o_dn, w);
  }
  hipLaunchKernelGGL((k_ridge_solve<DD>), dim3((DD + 31) / 32, D.BH), dim3(512), 0, s, D, B, coeffs);
  if (D.output_rank > 0 && D.M > 0) {
    hipLaunchKernelGGL((k_resid_cov<DD>), dim3(DD / 32, DD / 32, D.BH), dim3(256), 0, s, D, B, o_psp, o_dn, w);
    launch_residual_projector(D, B, s);
    hipLaunchKernelGGL((k_theta_project<DD>), dim3((DD + 1 + 7) / 8, D.BH), dim3(256), 0, s, D, B, coeffs);
  }
}

template <typename T, int DD>
static void apply_impl(const Dims& D, const Bufs& B, const void* o_sp, const float* o_dn, const float* coeffs, void* out,
                       hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value) {
    constexpr int RS = 2;
    hipLaunchKernelGGL((k_theta_split<DD>), dim3(DD * DD / 256, D.BH), dim3(256), 0, s, D, B, coeffs);
    hipLaunchKernelGGL((k_apply_bf16<DD, RS>), dim3((D.N + 128 * RS - 1) / (128 * RS), D.BH), dim3(256), 0, s, D, B,
                       (const bf16*)o_sp, o_dn, coeffs, (bf16*)out);
  }
  else
    hipLaunchKernelGGL((k_apply<T, DD>), dim3((D.N + 63) / 64, D.BH), dim3(256), 0, s, D, B, (const T*)o_sp, o_dn,
                       coeffs, (T*)out);
}

#define SPR_DISPATCH2(dtype, d, FN, ...)                                  \
  do {                                                                    \
    if ((dtype) == 1 && (d) == 128) FN<bf16, 128>(__VA_ARGS__);           \
    else if ((dtype) == 1 && (d) == 64) FN<bf16, 64>(__VA_ARGS__);        \
    else if ((dtype) == 0 && (d) == 128) FN<float, 128>(__VA_ARGS__);     \
    else FN<float, 64>(__VA_ARGS__);                                      \
  } while (0)

void launch_fit(const Dims& D, const Bufs& B, const float* o_psp, const float* o_dn, const float* w, float* coeffs,
                hipStream_t s) {
  if (D.d == 128) fit_impl<128>(D, B, o_psp, o_dn, w, coeffs, s);
  else fit_impl<64>(D, B, o_psp, o_dn, w, coeffs, s);
}

void launch_apply(const Dims& D, const Bufs& B, const void* o_sp, const float* o_dn, const float* coeffs, void* out,
                  hipStream_t s) {
  SPR_DISPATCH2(D.dtype, D.d, apply_impl, D, B, o_sp, o_dn, coeffs, out, s);
}

}  // namespace spr
