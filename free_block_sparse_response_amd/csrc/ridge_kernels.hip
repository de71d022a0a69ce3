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

// One block per (head, 64 right-hand-side columns): packed Cholesky of A in LDS (redone
// per column block), then forward and back substitution of the block's columns.
template <int DD>
__global__ __launch_bounds__(1024) void k_ridge_solve(Dims D, Bufs B, float* coeffs) {
  constexpr int n = DD + 1;
  constexpr int W = n + DD;
  constexpr int NP = n * (n + 1) / 2;
  constexpr int CB = 64;
  __shared__ double Lp[NP];
  __shared__ double Bs[n][CB];
  __shared__ double s_floor;
  __shared__ int s_fail;
  const int cb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int c0 = cb * CB;
  float* Th = coeffs + (size_t)bh * n * DD;
  if (D.M == 0) {
    for (int e = tid; e < n * CB; e += 1024) {
      const int i = e / CB, c = e % CB;
      if (c0 + c < DD) Th[(size_t)i * DD + c0 + c] = 0.f;
    }
    return;
  }
  const double* G = B.gram + (size_t)bh * n * W;
  auto pk = [](int i, int k) { return i * (i + 1) / 2 + k; };
  for (int e = tid; e < n * n; e += 1024) {
    const int i = e / n, k = e % n;
    if (k <= i) Lp[pk(i, k)] = G[(size_t)i * W + k];
  }
  for (int e = tid; e < n * CB; e += 1024) {
    const int i = e / CB, c = e % CB;
    Bs[i][c] = (c0 + c < DD) ? G[(size_t)i * W + n + c0 + c] : 0.0;
  }
  if (tid == 0) {
    double mx = 0.0;
    for (int i = 0; i < n; ++i) mx = fmax(mx, G[(size_t)i * W + i]);
    s_floor = kPivotRtol * mx;
    s_fail = 0;
  }
  __syncthreads();
  for (int j = 0; j < n; ++j) {
    if (tid == 0) {
      const double piv = Lp[pk(j, j)];
      if (!(piv > s_floor)) s_fail = 1;
      else Lp[pk(j, j)] = sqrt(piv);
    }
    __syncthreads();
    if (s_fail) break;
    const double djj = Lp[pk(j, j)];
    for (int i = j + 1 + tid; i < n; i += 1024) Lp[pk(i, j)] /= djj;
    __syncthreads();
    const int m = n - j - 1;
    for (int e = tid; e < m * m; e += 1024) {
      const int ii = e / m, kk = e % m;
      if (kk <= ii) {
        const int i = j + 1 + ii, k = j + 1 + kk;
        Lp[pk(i, k)] -= Lp[pk(i, j)] * Lp[pk(k, j)];
      }
    }
    __syncthreads();
  }
  if (s_fail) {
    for (int e = tid; e < n * CB; e += 1024) {
      const int i = e / CB, c = e % CB;
      if (c0 + c < DD) Th[(size_t)i * DD + c0 + c] = 0.f;
    }
    if (tid == 0) B.status[bh] = 5;  // SPARSEPR_ERR_NUMERICAL
    return;
  }
  // L Y = B
  for (int i = 0; i < n; ++i) {
    if (tid < CB) Bs[i][tid] /= Lp[pk(i, i)];
    __syncthreads();
    for (int e = tid; e < (n - i - 1) * CB; e += 1024) {
      const int k = i + 1 + e / CB, c = e % CB;
      Bs[k][c] -= Lp[pk(k, i)] * Bs[i][c];
    }
    __syncthreads();
  }
  // L^T X = Y
  for (int i = n - 1; i >= 0; --i) {
    if (tid < CB) Bs[i][tid] /= Lp[pk(i, i)];
    __syncthreads();
    for (int e = tid; e < i * CB; e += 1024) {
      const int k = e / CB, c = e % CB;
      Bs[k][c] -= Lp[pk(i, k)] * Bs[i][c];
    }
    __syncthreads();
  }
  for (int e = tid; e < n * CB; e += 1024) {
    const int i = e / CB, c = e % CB;
    if (c0 + c < DD) Th[(size_t)i * DD + c0 + c] = (float)Bs[i][c];
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

template <int DD>
static void fit_impl(const Dims& D, const Bufs& B, const float* o_psp, const float* o_dn, const float* w, float* coeffs,
                     hipStream_t s) {
  constexpr int n = DD + 1;
  if (D.M > 0) {
    dim3 g((n + 31) / 32, (n + DD + 31) / 32, D.BH);
    hipLaunchKernelGGL((k_ridge_gram<DD>), g, dim3(256), 0, s, D, B, o_psp, o_dn, w);
  }
  hipLaunchKernelGGL((k_ridge_solve<DD>), dim3((DD + 63) / 64, D.BH), dim3(1024), 0, s, D, B, coeffs);
}

template <typename T, int DD>
static void apply_impl(const Dims& D, const Bufs& B, const void* o_sp, const float* o_dn, const float* coeffs, void* out,
                       hipStream_t s) {
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
