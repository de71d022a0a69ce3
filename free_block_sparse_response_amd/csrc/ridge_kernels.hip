// Probe-Fitted Residual Reconstruction (paper "Partition the Support, Reconstruct the
// Residual", abstract; project website, PFRR panel): a weighted ridge fit of the affine map
// from a probe row's sparse output to its residual r = O_dense - O_sparse, then the
// predicted residual added to every unprobed row.
//
// Normal equations per head, in float64:
//   (Z^T W Z + Lambda) Theta = Z^T W R,  Z = [O_sp(probes), 1],  Lambda = diag(lambda 1_d, 0),
// built as one bordered matrix [A | B] (A (d+1)x(d+1), B (d+1)xd), then solved by a blocked
// LDL^T factorisation (the Cholesky factorisation up to the scaling of its columns) held in
// LDS. A pivot at or below 1e-12 x max diag(A) marks the head numerically singular.
#include <type_traits>

#include "common.h"
#include "plan_state.h"
#include "launch.h"

namespace spr {

constexpr double kPivotRtol = 1e-12;

// Offset of element (r, c) of a row-major tile of 16 double columns whose 16-byte chunks are
// XOR-swizzled by the row's group of four rows: rows 4 apart (the rows of neighbouring 4 x 4
// blocks) fall on different LDS banks.
__device__ constexpr int swz(int r, int c) { return 16 * r + ((((c >> 1) ^ ((r >> 2) & 7)) << 1) | (c & 1)); }

// Makes the LDS writes of a wave visible to the same wave's later reads (no block barrier).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// [A | B] of one head. The products of the probe sparse outputs' columns with the columns of
// [O_sp | R] (R = O_dense - O_sp, the residual) form a d x 2d matrix, computed in 64 x 64
// tiles (thread (ty, tx) of a 16 x 16 grid owns the 4 x 4 block at rows 4 ty, columns 4 tx):
// the lower tiles of A (mirrored into the upper) and every tile of B. The weighted column
// sums, which are the bias row of [A | B] and the bias column of A, come with them: wave 0
// of each diagonal tile of A and of each first-row tile of B sums its 64 columns, and the
// first tile adds the weight total (the bias pivot). Probes go 32 at a time through LDS (the
// column operand pre-multiplied by the weight); the next 32 are loaded into registers while
// the current ones are multiplied. Probes are summed in order, so the result does not depend
// on scheduling.
template <int DD>
__global__ __launch_bounds__(256) void k_ridge_gram(Dims D, Bufs B, const float* o_psp, const float* o_dn,
                                                    const float* weights) {
  constexpr int n = DD + 1;
  constexpr int W = n + DD;
  constexpr int TI = DD / 64;               // row tiles (rows of A's z part)
  constexpr int NA = TI * (TI + 1) / 2;     // lower tiles of A
  constexpr int PC = 32;                    // probes per chunk
  constexpr int NJ = 2;                     // 16-byte loads per thread and operand per chunk
  __shared__ __attribute__((aligned(16))) double Zi[PC][64];
  __shared__ __attribute__((aligned(16))) double Zj[PC][64];
  const int bh = blockIdx.y, tix = blockIdx.x, tid = threadIdx.x;
  // tile -> (ti, tj): the lower tiles of A first, then B's
  int ti, tj;
  if (tix < NA) {
    ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= tix) ++ti;
    tj = tix - ti * (ti + 1) / 2;
  } else {
    ti = (tix - NA) / TI;
    tj = TI + (tix - NA) % TI;
  }
  const bool bpart = tj >= TI;
  const bool sums = bpart ? ti == 0 : ti == tj;  // this tile's wave 0 sums its columns
  const int ty = tid / 16, tx = tid % 16;
  const float* wp = (weights ? weights : B.pweights) + (size_t)bh * D.M;
  const float* zs = o_psp + (size_t)bh * D.M * DD;
  const float* zd = o_dn + (size_t)bh * D.M * DD;
  const int ci = 64 * ti, cj = 64 * (bpart ? tj - TI : tj);
  // staging: thread e covers probe p = e / 16 of the chunk, columns 4 (e % 16) .. + 3, for
  // e = tid and tid + 256
  float4 ri[NJ], rs[NJ], rd[NJ];
  float rw[NJ];
  auto load = [&](int p0) {
#pragma unroll
    for (int u = 0; u < NJ; ++u) {
      const int e = tid + 256 * u, p = p0 + e / 16, c = 4 * (e % 16);
      const bool pv = p < D.M;
      const size_t o = (size_t)(pv ? p : 0) * DD;
      ri[u] = pv ? *reinterpret_cast<const float4*>(zs + o + ci + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      rs[u] = pv ? *reinterpret_cast<const float4*>(zs + o + cj + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      if (bpart) rd[u] = pv ? *reinterpret_cast<const float4*>(zd + o + cj + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      rw[u] = pv ? wp[p] : 0.f;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < NJ; ++u) {
      const int e = tid + 256 * u, p = e / 16, c = 4 * (e % 16);
      const double wv = (double)rw[u];
      double2* di = reinterpret_cast<double2*>(&Zi[p][c]);
      di[0] = make_double2((double)ri[u].x, (double)ri[u].y);
      di[1] = make_double2((double)ri[u].z, (double)ri[u].w);
      double v[4] = {(double)rs[u].x, (double)rs[u].y, (double)rs[u].z, (double)rs[u].w};
      if (bpart) {
        v[0] = (double)rd[u].x - v[0];
        v[1] = (double)rd[u].y - v[1];
        v[2] = (double)rd[u].z - v[2];
        v[3] = (double)rd[u].w - v[3];
      }
      double2* dj = reinterpret_cast<double2*>(&Zj[p][c]);
      dj[0] = make_double2(wv * v[0], wv * v[1]);
      dj[1] = make_double2(wv * v[2], wv * v[3]);
    }
  };
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  double csum = 0.0, wsum = 0.0;  // wave 0: column tid's weighted sum; thread 0: weight total
  if (D.M > 0) load(0);
  for (int p0 = 0; p0 < D.M; p0 += PC) {
    __syncthreads();  // (the previous chunk's reads are done)
    store();
    __syncthreads();
    if (p0 + PC < D.M) load(p0 + PC);
#pragma unroll 4
    for (int p = 0; p < PC; ++p) {
      const double2 a0 = *reinterpret_cast<const double2*>(&Zi[p][4 * ty]);
      const double2 a1 = *reinterpret_cast<const double2*>(&Zi[p][4 * ty + 2]);
      const double2 b0 = *reinterpret_cast<const double2*>(&Zj[p][4 * tx]);
      const double2 b1 = *reinterpret_cast<const double2*>(&Zj[p][4 * tx + 2]);
      const double av[4] = {a0.x, a0.y, a1.x, a1.y}, bv[4] = {b0.x, b0.y, b1.x, b1.y};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(av[u], bv[v], acc[u][v]);
    }
    if (sums && tid < 64) {
      for (int p = 0; p < PC; ++p) csum += Zj[p][tid];
      if (tix == 0 && tid == 0)
        for (int p = 0; p < PC && p0 + p < D.M; ++p) wsum += (double)wp[p0 + p];
    }
  }
  double* G = B.gram + (size_t)bh * n * W;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ci + 4 * ty + u, c = cj + 4 * tx + v;
      if (bpart) {
        G[(size_t)i * W + n + c] = acc[u][v];
      } else {
        const double x = acc[u][v] + (i == c ? (double)D.lambda : 0.0);
        G[(size_t)i * W + c] = x;
        if (ti != tj) G[(size_t)c * W + i] = x;
      }
    }
  if (sums && tid < 64) {
    const int c = cj + tid;
    if (bpart) {
      G[(size_t)DD * W + n + c] = csum;
    } else {
      G[(size_t)DD * W + c] = csum;
      G[(size_t)c * W + DD] = csum;
    }
  }
  if (tix == 0 && tid == 0) G[(size_t)DD * W + DD] = wsum + (D.pen_bias ? (double)D.lambda : 0.0);
}

// The ridge solve of one head for 32 of its right-hand-side columns (one block of 256 threads
// per head and 32 columns; the blocks of a head factor A alike). The system is padded to
// NP = 16 NB rows with unit pivots (zero right-hand side), A's lower 16 x 16 blocks and the
// right-hand side sit in LDS, and A = L D L^T (L unit lower) by blocks of 16 columns:
//   * panel k: each of waves 0 .. 2 takes the diagonal block's 16 rows (lanes 0 .. 15, the
//     same in every wave) and 48 of the rows below (lanes 16 .. 63); wave 3 takes the
//     diagonal rows and the 32 right-hand-side columns (lanes 16 .. 47). Row lanes hold 16
//     panel entries, column lanes 16 right-hand-side entries. Column by column, the diagonal
//     lanes publish their current entry of the pivot column in the wave's own LDS slots;
//     every lane reads the pivot and the column, the rows below the pivot turn their entry
//     into the multiplier and update the rest of their panel entries, and the right-hand
//     side takes the forward substitution step. No block barrier inside a panel.
//   * the trailing update, by all threads in 4 x 4 blocks: A_ij -= L_ik (D_k L_jk^T) on the
//     lower blocks, B_i -= L_ik Z_k on the right-hand side.
// Then X = L^-T D^-1 Z by blocks from the last: a 16-step substitution with the diagonal
// block (one lane per column), and the rows above updated by all threads.
template <int DD>
__global__ __launch_bounds__(256) void k_ridge_solve(Dims D, Bufs B, float* coeffs) {
  constexpr int n = DD + 1;
  constexpr int W = n + DD;
  constexpr int NB = (n + 15) / 16;          // 16-row blocks of the padded system
  constexpr int NP = 16 * NB;
  constexpr int NLB = NB * (NB + 1) / 2;     // lower blocks
  constexpr int CB = 32;                     // right-hand-side columns per block
  constexpr int NBR = NP - 16;               // rows below the first diagonal block
  static_assert(NBR <= 144, "three waves of 48 rows below the diagonal block");
  __shared__ __attribute__((aligned(16))) double Ab[NLB * 256];  // block (bi, bj): swz(r, c)
  __shared__ __attribute__((aligned(16))) double Bs[NP * CB];
  __shared__ __attribute__((aligned(16))) double Wp[NBR * 16];   // D_k L_ik^T rows of the panel, swz
  __shared__ double xc[4][16];                                    // per-wave pivot column
  __shared__ double rdv[NP];                                      // reciprocal pivots
  __shared__ double s_floor;
  auto blk = [](int bi, int bj) { return (bi * (bi + 1) / 2 + bj) * 256; };
  const int bh = blockIdx.y, c0 = blockIdx.x * CB;
  const int tid = threadIdx.x, l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  float* Th = coeffs + (size_t)bh * n * DD;
  if (D.M == 0) {
    for (int e = tid; e < n * CB; e += 256) {
      const int i = e / CB, c = e % CB;
      if (c0 + c < DD) Th[(size_t)i * DD + c0 + c] = 0.f;
    }
    return;
  }
  const double* G = B.gram + (size_t)bh * n * W;
  // thread t loads element (t / 16, t % 16) of every lower block and rows t / 32 + 8 j of the
  // right-hand side, all loads issued before the first store (fully unrolled: block b's
  // coordinates are compile-time constants)
  {
    const int r = tid / 16, c = tid % 16;
    double va[NLB];
#pragma unroll
    for (int bi = 0, b = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj <= bi; ++bj, ++b) {
        const int i = 16 * bi + r, k = 16 * bj + c;
        const double g = G[(size_t)min(i, n - 1) * W + min(k, n - 1)];  // (clamped: no branch)
        va[b] = (i < n && k < n) ? g : (i == k ? 1.0 : 0.0);
      }
    constexpr int NBL = NP * CB / 256;
    double vb[NBL];
    const int rb = tid / CB, cb = tid % CB;
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      const int i = rb + (256 / CB) * j;
      const double g = G[(size_t)min(i, n - 1) * W + n + min(c0 + cb, DD - 1)];
      vb[j] = (i < n && c0 + cb < DD) ? g : 0.0;
    }
#pragma unroll
    for (int b = 0; b < NLB; ++b) Ab[256 * b + swz(r, c)] = va[b];
#pragma unroll
    for (int j = 0; j < NBL; ++j) Bs[256 * j + tid] = vb[j];
  }
  if (tid < kWave) {
    double mx = 0.0;
    for (int i = tid; i < n; i += kWave) mx = fmax(mx, G[(size_t)i * W + i]);
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, kWave));
    if (tid == 0) s_floor = kPivotRtol * mx;
  }
  __syncthreads();
  const double floor_ = s_floor;
  bool fail = false;
  for (int k = 0; k < NB; ++k) {
    const int j0 = 16 * k, nbr = NP - j0 - 16;
    const int b = 48 * w + l - 16;  // row below the diagonal block (waves 0 .. 2)
    const bool diag = l < 16;
    const bool below = w < 3 && l >= 16 && b < nbr;
    const bool rhs = w == 3 && l >= 16 && l < 16 + CB;
    const int ib = j0 + 16 + b;
    const int rrow = diag ? l : ib % 16, rsw = (rrow >> 2) & 7;  // row in its block, its swizzle
    double* rowp = diag ? &Ab[blk(k, k) + 16 * l] : (below ? &Ab[blk(ib / 16, k) + 16 * rrow] : nullptr);
    double a[16];
    if (diag || below) {
#pragma unroll
      for (int c = 0; c < 16; c += 2) {
        const double2 v = *reinterpret_cast<const double2*>(rowp + 2 * ((c >> 1) ^ rsw));
        a[c] = v.x;
        a[c + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] = rhs ? Bs[(j0 + r) * CB + l - 16] : 0.0;
    }
    double dk[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      wave_lds_sync();  // (the previous column's reads are done)
      if (diag) xc[w][l] = a[p];
      wave_lds_sync();
      const double d = xc[w][p];
      double wc[16];
#pragma unroll
      for (int c = p + 1; c < 16; ++c) wc[c] = xc[w][c];
      fail |= j0 + p < n && !(d > floor_);
      // 1 / d: the hardware reciprocal and two Newton steps (the pivot is > 0 here or the
      // head fails)
      double rd = __builtin_amdgcn_rcp(d);
      rd = fma(rd, fma(-d, rd, 1.0), rd);
      rd = fma(rd, fma(-d, rd, 1.0), rd);
      dk[p] = d;
      if (tid == 0) rdv[j0 + p] = rd;
      // one update for every lane: a row lane subtracts its multiplier times the pivot
      // column's entries W[x] (x > p), a column lane subtracts L[x][p] z_p (the same product);
      // other entries it touches are never read. A row lane then keeps its multiplier in
      // place of its pivot-column entry; the pivot row keeps the pivot, a column lane z_p.
      const double lv = a[p] * rd;
#pragma unroll
      for (int x = p + 1; x < 16; ++x) a[x] = fma(-lv, wc[x], a[x]);
      a[p] = (rhs || l == p) ? a[p] : lv;
    }
    if (fail) break;  // (every thread of the block takes the same pivots)
    if ((diag && w == 0) || below) {
#pragma unroll
      for (int c = 0; c < 16; c += 2)
        *reinterpret_cast<double2*>(rowp + 2 * ((c >> 1) ^ rsw)) = make_double2(a[c], a[c + 1]);
    }
    if (below) {
#pragma unroll
      for (int c = 0; c < 16; c += 2)
        *reinterpret_cast<double2*>(&Wp[swz(b, c)]) = make_double2(a[c] * dk[c], a[c + 1] * dk[c + 1]);
    }
    if (rhs) {
#pragma unroll
      for (int r = 0; r < 16; ++r) Bs[(j0 + r) * CB + l - 16] = a[r];
    }
    __syncthreads();
    // trailing update: lower blocks of A, then the right-hand side rows below the panel
    const int m = NB - 1 - k;
    const int nA = 16 * (m * (m + 1) / 2), nR = 32 * m;
    for (int it = tid; it < nA + nR; it += 256) {
      double acc[4][4];
      const double* Lr;
      if (it < nA) {
        const int pr = it / 16, sub = it % 16;
        int bi = 0;
        while ((bi + 1) * (bi + 2) / 2 <= pr) ++bi;
        const int bj = pr - bi * (bi + 1) / 2, rr = sub / 4, cc = sub % 4;
        const int wb = 16 * bj + 4 * cc, wsw = (wb >> 2) & 7;  // first W row, its swizzle
        Lr = &Ab[blk(k + 1 + bi, k) + 64 * rr];  // rows 4 rr .. 4 rr + 3 (swizzle rr)
        const double* Wr = &Wp[16 * wb];
        double* At = &Ab[blk(k + 1 + bi, k + 1 + bj)];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = At[swz(4 * rr + u, 4 * cc + v)];
#pragma unroll
        for (int p = 0; p < 16; p += 2) {
          double2 lv[4], wv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) lv[u] = *reinterpret_cast<const double2*>(Lr + 16 * u + 2 * ((p >> 1) ^ rr));
#pragma unroll
          for (int v = 0; v < 4; ++v) wv[v] = *reinterpret_cast<const double2*>(Wr + 16 * v + 2 * ((p >> 1) ^ wsw));
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              acc[u][v] = fma(-lv[u].x, wv[v].x, acc[u][v]);
              acc[u][v] = fma(-lv[u].y, wv[v].y, acc[u][v]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) At[swz(4 * rr + u, 4 * cc + v)] = acc[u][v];
      } else {
        const int t = it - nA, bi = t / 32, sub = t % 32, rr = sub / 8, cc = sub % 8;
        Lr = &Ab[blk(k + 1 + bi, k) + 64 * rr];
        double* dst = &Bs[(16 * (k + 1 + bi) + 4 * rr) * CB + 4 * cc];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = dst[u * CB + v];
#pragma unroll
        for (int p = 0; p < 16; p += 2) {
          double2 lv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) lv[u] = *reinterpret_cast<const double2*>(Lr + 16 * u + 2 * ((p >> 1) ^ rr));
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const double* zr = &Bs[(j0 + p + q) * CB + 4 * cc];
            const double2 z0 = *reinterpret_cast<const double2*>(zr), z1 = *reinterpret_cast<const double2*>(zr + 2);
            const double zv[4] = {z0.x, z0.y, z1.x, z1.y};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const double lu = q ? lv[u].y : lv[u].x;
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[u][v] = fma(-lu, zv[v], acc[u][v]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) dst[u * CB + v] = acc[u][v];
      }
    }
    __syncthreads();
  }
  if (!fail) {
    // y = D^-1 z, then L^T x = y by blocks from the last
    for (int e = tid; e < NP * CB; e += 256) Bs[e] *= rdv[e / CB];
    __syncthreads();
    for (int k = NB - 1; k >= 0; --k) {
      const int j0 = 16 * k;
      if (w == 0 && l < CB) {
        double y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = Bs[(j0 + r) * CB + l];
        const double* Lk = &Ab[blk(k, k)];
#pragma unroll
        for (int r = 15; r > 0; --r)
#pragma unroll
          for (int q = 0; q < r; ++q) y[q] = fma(-Lk[swz(r, q)], y[r], y[q]);
#pragma unroll
        for (int r = 0; r < 16; ++r) Bs[(j0 + r) * CB + l] = y[r];
      }
      __syncthreads();
      for (int it = tid; it < 32 * k; it += 256) {
        const int j = it / 32, sub = it % 32, rr = sub / 8, cc = sub % 8;
        const double* Lb = &Ab[blk(k, j)];  // columns 4 rr .. 4 rr + 3 of block (k, j), by rows p
        double* dst = &Bs[(16 * j + 4 * rr) * CB + 4 * cc];
        double acc[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = dst[u * CB + v];
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          const double2 l0 = *reinterpret_cast<const double2*>(Lb + swz(p, 4 * rr));
          const double2 l1 = *reinterpret_cast<const double2*>(Lb + swz(p, 4 * rr + 2));
          const double* xr = &Bs[(j0 + p) * CB + 4 * cc];
          const double2 x0 = *reinterpret_cast<const double2*>(xr), x1 = *reinterpret_cast<const double2*>(xr + 2);
          const double lu[4] = {l0.x, l0.y, l1.x, l1.y}, xv[4] = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = fma(-lu[u], xv[v], acc[u][v]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) dst[u * CB + v] = acc[u][v];
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < n * CB; e += 256) {
    const int i = e / CB, c = e % CB;
    if (c0 + c < DD) Th[(size_t)i * DD + c0 + c] = fail ? 0.f : (float)Bs[i * CB + c];
  }
  if (fail && tid == 0) B.status[bh] = 5;  // SPARSEPR_ERR_NUMERICAL
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
// products. The epilogue adds o and the bias (probe rows take o_dense) and writes the rows
// into LDS, where the operands were, so that they leave as whole contiguous rows: a store
// of 8-byte pieces scattered over 32 rows costs the L2 one request per piece.
template <int DD, int RS>
__global__ __launch_bounds__(256) void k_apply_bf16(Dims D, Bufs B, const bf16* o_sp, const float* o_dn,
                                                    const float* coeffs, bf16* out) {
  constexpr int KS = DD + 8;  // row stride (elements) of the operands and of the staged output
  constexpr int NT = DD * DD / 8 / 256;  // 16-byte chunks per thread and operand
  constexpr int TSZ = 2 * DD * KS > 4 * RS * 32 * KS ? 2 * DD * KS : 4 * RS * 32 * KS;
  __shared__ __attribute__((aligned(16))) bf16 Tsm[TSZ];  // the operands, then the output rows
  __shared__ float bias[DD];
  bf16* Th = Tsm;
  bf16* Tl = Tsm + DD * KS;
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid / kWave, l32 = lane_id() & 31, h = lane_id() >> 5;
  const bf16* sh = B.theta_h + (size_t)bh * DD * DD;
  const bf16* sl = B.theta_l + (size_t)bh * DD * DD;
  // every load in flight together: Theta^T (hi / lo), the bias, the rows of o; the LDS
  // stores wait for the Theta loads only
  bf16x8 th[NT], tl[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int e = tid + 256 * i, r = e / (DD / 8), c8 = (e % (DD / 8)) * 8;
    th[i] = *reinterpret_cast<const bf16x8*>(sh + (size_t)r * DD + c8);
    tl[i] = *reinterpret_cast<const bf16x8*>(sl + (size_t)r * DD + c8);
  }
  const float bv = tid < DD ? coeffs[(size_t)bh * (DD + 1) * DD + (size_t)DD * DD + tid] : 0.f;
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
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int e = tid + 256 * i, r = e / (DD / 8), c8 = (e % (DD / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&Th[r * KS + c8]) = th[i];
    *reinterpret_cast<bf16x8*>(&Tl[r * KS + c8]) = tl[i];
  }
  if (tid < DD) bias[tid] = bv;
  __syncthreads();
  // the output values, bf16 pairs in the accumulator's layout, until the operands are free
  uint32_t pk[RS][DD / 32][8];
#pragma unroll
  for (int jb = 0; jb < DD / 32; ++jb) {
    f32x16 acc[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rs][v] = 0.f;
#pragma unroll
    for (int c = 0; c < DD / 16; ++c) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Th[(32 * jb + l32) * KS + 16 * c + 8 * h]);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Tl[(32 * jb + l32) * KS + 16 * c + 8 * h]);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        acc[rs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xr[rs][c], acc[rs], 0, 0, 0);
        acc[rs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xr[rs][c], acc[rs], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      // o's own entries for the output layout (dims 32 jb + 8 g + 4 h + r) come from the
      // operand registers: the 16 dims of chunk c sit 8 per lane half, and swapping dwords
      // 0, 1 of the upper half with dwords 2, 3 of the lower one gives each lane its two runs
      uint32_t xo[2][4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bf16x8 xc = xr[rs][2 * jb + q];
        uint32_t dw[4];
        __builtin_memcpy(dw, &xc, 16);
        const auto s02 = __builtin_amdgcn_permlane32_swap(dw[0], dw[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(dw[1], dw[3], false, false);
        xo[q][0] = s02[0];
        xo[q][1] = s13[0];
        xo[q][2] = s02[1];
        xo[q][3] = s13[1];
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = 32 * jb + 8 * g + 4 * h;
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
        __builtin_memcpy(&pk[rs][jb][2 * g], &ov, 8);
      }
    }
  }
  __syncthreads();  // every operand read is done: the region takes the output rows
  bf16* stg = Tsm + (size_t)w * RS * 32 * KS;  // this wave's rows, RS sets of 32
#pragma unroll
  for (int rs = 0; rs < RS; ++rs)
#pragma unroll
    for (int jb = 0; jb < DD / 32; ++jb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        __builtin_memcpy(stg + (rs * 32 + l32) * KS + 32 * jb + 8 * g + 4 * h, &pk[rs][jb][2 * g], 8);
  __syncthreads();
  // whole rows out: DD / 8 lanes per row, 64 / (DD / 8) rows per store
  constexpr int LPR = DD / 8, RPI = kWave / LPR;
  const int lr = lane_id() / LPR, lc = (lane_id() % LPR) * 8;
#pragma unroll
  for (int rs = 0; rs < RS; ++rs)
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + lr;
      const int grow = blk * 128 * RS + 128 * rs + 32 * w + r;
      if (grow < D.N)
        *reinterpret_cast<bf16x8*>(out + ((size_t)bh * D.N + grow) * DD + lc) =
            *reinterpret_cast<const bf16x8*>(stg + (rs * 32 + r) * KS + lc);
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
  if (D.correction != 0) {
    hipLaunchKernelGGL((k_fit_mean<DD>), dim3(D.BH), dim3(DD), 0, s, D, B, o_psp, o_dn, w, coeffs);
    return;
  }
  if (D.M > 0) {
    constexpr int TI = DD / 64;
    hipLaunchKernelGGL((k_ridge_gram<DD>), dim3(TI * (TI + 1) / 2 + TI * TI, D.BH), dim3(256), 0, s, D, B, o_psp,
                       o_dn, w);
  }
  hipLaunchKernelGGL((k_ridge_solve<DD>), dim3((DD + 31) / 32, D.BH), dim3(256), 0, s, D, B, coeffs);
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
