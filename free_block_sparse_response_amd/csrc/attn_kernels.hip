// Block-sparse softmax attention over the selected (query group, key group) cells, and
// the exact attention of the probe rows (paper "Partition the Support, Reconstruct the
// Residual", abstract; project website, Method section, stage 03 and the PFRR panel).
//
// Query rows of one query group are taken 128 at a time (one tile); the keys are the
// union of the selected key groups, which the permutation made contiguous per group, so
// consecutive selected groups merge into one key run. Softmax is renormalised over the
// retained keys only (online softmax across 64-key tiles).
//
// bf16 path, per workgroup of 4 waves (32 query rows each):
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16: A = K tile rows from LDS, B = Q^T kept in
//                 registers; each lane then holds the scores of ONE query (lane % 32) for 32
//                 keys, so the row max / sum are in-lane plus one cross-half exchange.
//   O^T = V^T P^T with the same MFMA: B = P^T is the score registers converted to bf16 in
//                 place (no shuffles); A = V^T comes from the transposed V layout that the
//                 permutation pass writes, read as two 8-byte LDS loads per operand.
// K rows are 16 B-padded in LDS and V^T rows 16 B-padded so both operand reads are
// bank-conflict free; exp2 with the log2(e) factor folded into the score scale.
#include "common.h"
#include "plan_state.h"
#include "launch.h"

namespace spr {

// Remaps the linear block id so that each of the 8 XCDs (which receive blocks round-robin)
// walks a contiguous range of tiles: tiles of one query group share key runs in that XCD's L2.
__device__ inline int xcd_remap(int bid, int nblocks) {
  const int per = (nblocks + 7) / 8;
  const int xcd = bid % 8, slot = bid / 8;
  const int full = nblocks - (per - 1) * 8;  // XCDs that own `per` tiles (the rest own per-1)
  const int base = xcd < full ? xcd * per : full * per + (xcd - full) * (per - 1);
  return base + slot;
}

// Walks the key runs of a query group: consecutive selected key groups merge into one run.
struct RunIter {
  const int* cols;
  const int* koff;
  int c, cend;
  __device__ bool next(int& lo, int& hi) {
    if (c >= cend) return false;
    int b = cols[c];
    lo = koff[b];
    int e = b;
    ++c;
    while (c < cend && cols[c] == e + 1) { ++e; ++c; }
    hi = koff[e + 1];
    return true;
  }
};

// Sequence of 64-key tiles over the key runs of one work item. A run [lo, hi) starts its
// first tile at lo rounded down to 8 keys (16-byte aligned rows of the transposed V); keys
// outside [lo, hi) are masked.
struct TileSeq {
  RunIter it;
  int lo, hi, k0;
  bool single, used;
  __device__ bool first(int mode_lo, int mode_hi) {
    if (single) {
      lo = mode_lo;
      hi = mode_hi;
      used = true;
      k0 = lo & ~7;
      return lo < hi;
    }
    if (!it.next(lo, hi)) return false;
    k0 = lo & ~7;
    return true;
  }
  __device__ bool next() {
    k0 += kKeyTile;
    if (k0 < hi) return true;
    if (single) return false;
    if (!it.next(lo, hi)) return false;
    k0 = lo & ~7;
    return true;
  }
};

// -------------------------------------------------------------------------------------
// bf16 MFMA kernel. MODE 0: block-sparse tiles from the tile table, bf16 output in token
// order (plus float rows for probes). MODE 1: probe rows (128 per block) over one chunk of
// all keys, partial outputs for the chunk combine. MODE 2: the same code as MODE 0 under its
// own symbol, used by the dense reference call so that traces keep the two apart.
// K and V^T tiles are double-buffered in LDS: the global loads of tile j+1 are issued
// before the products of tile j and land in the other buffer afterwards, one barrier per
// tile. The accumulator is rescaled only when a query's running max grows by more than
// 2^8 (the stale max keeps every exponent <= 2^8, exact enough in fp32 and bf16).
// -------------------------------------------------------------------------------------
template <int DD, int MODE>
__global__ __launch_bounds__(256, 2) void k_bsfa_bf16(const bf16* __restrict__ q, Dims D, Bufs B, void* out,
                                                        float* psp) {
  constexpr int KS = DD + 8;          // K row stride in LDS (elements)
  constexpr int VS = kKeyTile + 8;    // V^T row stride in LDS (elements)
  constexpr int NC = DD / 16;         // k-chunks of the QK^T product
  constexpr int ND = DD / 32;         // 32-wide d blocks of the output
  constexpr int KL = (kKeyTile * DD / 8) / 256;  // 16-byte loads per thread per tile (K and V each)
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][kKeyTile * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][DD * VS];

  const int nb = gridDim.x;
  const int bid = xcd_remap(blockIdx.x, nb);
  int bh, rows, a = 0, pos0 = 0;
  if (MODE != 1) {
    bh = bid / D.max_tiles;
    const int t = bid % D.max_tiles;
    if (t >= B.ntiles[bh]) return;
    const int2 tl = B.tiles[(size_t)bh * D.max_tiles + t];
    a = tl.x;
    pos0 = tl.y;
    const int end = B.qoff[(size_t)bh * (D.Cq + 1) + a + 1];
    rows = min(D.qt, end - pos0);
  } else {
    // probe rows: (head, 128-row tile, key chunk)
    const int per = ((D.M + kAttnQT - 1) / kAttnQT) * D.pch;
    bh = bid / per;
    const int rem = bid % per;
    pos0 = (rem / D.pch) * kAttnQT;
    a = rem % D.pch;  // key chunk
    rows = min(kAttnQT, D.M - pos0);
  }
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id(), h = l >> 5, l32 = l & 31;

  // ---- Q^T operand in registers: query (32w + l32), d-slots 16c + 8h .. +7
  const int qr = 32 * w + l32;
  const bool qvalid = qr < rows;
  const bool wave_active = 32 * w < rows;  // a wave past the tile's last row only stages K / V
  int tok;
  if (MODE != 1) tok = B.qperm[(size_t)bh * D.N + pos0 + (qvalid ? qr : 0)];
  else tok = B.probes[(size_t)bh * D.M + pos0 + (qvalid ? qr : 0)];
  const bf16* qrow = q + ((size_t)bh * D.N + tok) * DD;
  bf16x8 qreg[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qreg[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * h);

  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  float m_run = -INFINITY, l_half = 0.f;
  const float c2 = D.log2_scale;

  const bf16* kpb = (const bf16*)B.kp + (size_t)bh * D.Npad * DD;
  const bf16* vtb = (const bf16*)B.vpt + (size_t)bh * DD * D.Npad;
  TileSeq ts;
  ts.single = MODE == 1;
  ts.used = false;
  if (MODE != 1) {
    ts.it.cols = B.cols + (size_t)bh * D.Cq * D.Ck;
    ts.it.koff = B.koff + (size_t)bh * (D.Ck + 1);
    const int* rp = B.row_ptr + (size_t)bh * (D.Cq + 1);
    ts.it.c = rp[a];
    ts.it.cend = rp[a + 1];
  }
  const int clo = MODE == 1 ? a * D.pkc : 0;
  bool have = ts.first(clo, MODE == 1 ? min(D.N, clo + D.pkc) : 0);

  // thread's share of a tile: K rows r = c / (DD/8), 16-byte column c8; V^T rows / columns
  bf16x8 kreg[KL], vreg[KL];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int c = tid + 256 * i;
      const int r = c / (DD / 8), c8 = c % (DD / 8);
      kreg[i] = *reinterpret_cast<const bf16x8*>(kpb + (size_t)(k0 + r) * DD + c8 * 8);
      const int rv = c / (kKeyTile / 8), cv = c % (kKeyTile / 8);
      vreg[i] = *reinterpret_cast<const bf16x8*>(vtb + (size_t)rv * D.Npad + k0 + cv * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int c = tid + 256 * i;
      const int r = c / (DD / 8), c8 = c % (DD / 8);
      *reinterpret_cast<bf16x8*>(&Ks[buf][r * KS + c8 * 8]) = kreg[i];
      const int rv = c / (kKeyTile / 8), cv = c % (kKeyTile / 8);
      *reinterpret_cast<bf16x8*>(&Vs[buf][rv * VS + cv * 8]) = vreg[i];
    }
  };
  int cur = 0;
  if (have) {
    load_tile(ts.k0);
    store_tile(0);
  }
  __syncthreads();
  while (have) {
    const int k0 = ts.k0, lo = ts.lo, hi = ts.hi;
    const bool more = ts.next();
    if (more) load_tile(ts.k0);
    if (wave_active) {
    // ---- S^T = K Q^T for two 32-key blocks
    const bf16* Kc = Ks[cur];
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Kc[(kb * 32 + l32) * KS + 16 * c + 8 * h]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[c], s[kb], 0, 0, 0);
      }
    }
    // ---- online softmax (scores of query l32; key = k0 + 32kb + 8(v/4) + 4h + v%4)
    if (k0 < lo || k0 + kKeyTile > hi) {
      const int vlo = lo - k0, vhi = hi - k0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
          if (kk < vlo || kk >= vhi) s[kb][v] = -INFINITY;
        }
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[kb][v]);
    mt = fmaxf(mt, xor32(mt)) * c2;
    if (mt > m_run + 8.f) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
      m_run = mt;
      l_half *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][v], c2, -m_run));
        s[kb][v] = p;
        ps += p;
      }
    l_half += ps;
    // ---- O^T += V^T P^T over four 16-key chunks
    const bf16* Vc = Vs[cur];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int kb = cc >> 1, sub = cc & 1;
      bf16x8 pb;
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[t] = (bf16)s[kb][8 * sub + t];
      const int key0 = 32 * kb + 16 * sub + 4 * h;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16* vr = &Vc[(32 * db + l32) * VS + key0];
        const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vr);
        const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vr + 8);
        bf16x8 av;
        av[0] = v0[0]; av[1] = v0[1]; av[2] = v0[2]; av[3] = v0[3];
        av[4] = v1[0]; av[5] = v1[1]; av[6] = v1[2]; av[7] = v1[3];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, o[db], 0, 0, 0);
      }
    }
    }  // wave_active
    if (more) store_tile(cur ^ 1);
    __syncthreads();
    cur ^= 1;
    have = more;
  }
  // ---- normalise and store query l32's row: d = 32db + 8g + 4h + r
  const float lsum = l_half + xor32(l_half);
  const float inv = 1.f / lsum;
  if (!qvalid) return;
  if (MODE != 1) {
    bf16* orow = (bf16*)out + ((size_t)bh * D.N + tok) * DD;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = (bf16)(o[db][4 * g + r] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * h) = ov;
      }
    // probe rows also keep their sparse output in float for the ridge fit
    const int slot = (psp && D.M > 0) ? B.pslot[(size_t)bh * D.N + tok] : -1;
    if (slot >= 0) {
      float* prow = psp + ((size_t)bh * D.M + slot) * DD;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 ov;
          ov.x = o[db][4 * g + 0] * inv;
          ov.y = o[db][4 * g + 1] * inv;
          ov.z = o[db][4 * g + 2] * inv;
          ov.w = o[db][4 * g + 3] * inv;
          *reinterpret_cast<float4*>(prow + 32 * db + 8 * g + 4 * h) = ov;
        }
    }
  } else {
    // partial of key chunk `a`: unnormalised output and (max, sum) in the log2 domain
    const size_t pr = ((size_t)bh * D.M + pos0 + qr) * D.pch + a;
    float* orow = B.pp_o + pr * DD;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 ov;
        ov.x = o[db][4 * g + 0];
        ov.y = o[db][4 * g + 1];
        ov.z = o[db][4 * g + 2];
        ov.w = o[db][4 * g + 3];
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * g + 4 * h) = ov;
      }
    if (h == 0) B.pp_ml[pr] = make_float2(m_run, lsum);
  }
}

// Exact probe output from the key-chunk partials, chunks combined in order.
template <int DD>
__global__ __launch_bounds__(DD) void k_probe_combine(Dims D, Bufs B, float* o_pdn) {
  const int p = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  const size_t r = (size_t)bh * D.M + p;
  const float2* ml = B.pp_ml + r * D.pch;
  float mx = -INFINITY;
  for (int c = 0; c < D.pch; ++c) mx = fmaxf(mx, ml[c].x);
  float S = 0.f, acc = 0.f;
  const float* po = B.pp_o + r * D.pch * DD;
  for (int c = 0; c < D.pch; ++c) {
    const float sc = exp2f(ml[c].x - mx);
    S = fmaf(ml[c].y, sc, S);
    acc = fmaf(po[(size_t)c * DD + i], sc, acc);
  }
  o_pdn[r * DD + i] = acc / S;
}

// -------------------------------------------------------------------------------------
// fp32 kernel (SIMT): one query row per thread, 128 rows per block; same tiles and runs.
// -------------------------------------------------------------------------------------
template <int DD, int MODE>
__global__ __launch_bounds__(128) void k_bsfa_f32(const float* __restrict__ q, Dims D, Bufs B, void* out,
                                                  float* psp) {
  __shared__ float Ks[kKeyTile][DD];
  __shared__ float Vs[DD][kKeyTile];
  const int nb = gridDim.x;
  const int bid = xcd_remap(blockIdx.x, nb);
  int bh, rows, a = 0, pos0 = 0;
  if (MODE == 0) {
    bh = bid / D.max_tiles;
    const int t = bid % D.max_tiles;
    if (t >= B.ntiles[bh]) return;
    const int2 tl = B.tiles[(size_t)bh * D.max_tiles + t];
    a = tl.x;
    pos0 = tl.y;
    rows = min(D.qt, B.qoff[(size_t)bh * (D.Cq + 1) + a + 1] - pos0);
  } else {
    const int per = (D.M + kAttnQT - 1) / kAttnQT;
    bh = bid / per;
    pos0 = (bid % per) * kAttnQT;
    rows = min(kAttnQT, D.M - pos0);
  }
  const int tid = threadIdx.x;
  const bool qvalid = tid < rows;
  int tok;
  if (MODE == 0) tok = B.qperm[(size_t)bh * D.N + pos0 + (qvalid ? tid : 0)];
  else tok = B.probes[(size_t)bh * D.M + pos0 + (qvalid ? tid : 0)];
  float qv[DD], ov[DD];
  const float* qrow = q + ((size_t)bh * D.N + tok) * DD;
#pragma unroll
  for (int i = 0; i < DD; ++i) { qv[i] = qrow[i] * D.log2_scale; ov[i] = 0.f; }
  float m_run = -INFINITY, lsum = 0.f;
  const float* kpb = (const float*)B.kp + (size_t)bh * D.Npad * DD;
  const float* vtb = (const float*)B.vpt + (size_t)bh * DD * D.Npad;
  RunIter it;
  if (MODE == 0) {
    it.cols = B.cols + (size_t)bh * D.Cq * D.Ck;
    it.koff = B.koff + (size_t)bh * (D.Ck + 1);
    const int* rp = B.row_ptr + (size_t)bh * (D.Cq + 1);
    it.c = rp[a];
    it.cend = rp[a + 1];
  }
  int lo, hi;
  bool first = true;
  while (true) {
    if (MODE == 0) {
      if (!it.next(lo, hi)) break;
    } else {
      if (!first) break;
      lo = 0;
      hi = D.N;
    }
    first = false;
    for (int k0 = lo & ~7; k0 < hi; k0 += kKeyTile) {
      __syncthreads();
      for (int i = tid; i < kKeyTile * DD; i += 128) {
        const int r = i / DD, c = i % DD;
        Ks[r][c] = kpb[(size_t)(k0 + r) * DD + c];
      }
      for (int i = tid; i < kKeyTile * DD; i += 128) {
        const int r = i / kKeyTile, c = i % kKeyTile;
        Vs[r][c] = vtb[(size_t)r * D.Npad + k0 + c];
      }
      __syncthreads();
      const int klo = max(lo - k0, 0), khi = min(hi - k0, kKeyTile);
      float sc[kKeyTile];
      float mt = -INFINITY;
      for (int j = 0; j < kKeyTile; ++j) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < DD; ++i) x = fmaf(qv[i], Ks[j][i], x);
        x = (j >= klo && j < khi) ? x : -INFINITY;
        sc[j] = x;
        mt = fmaxf(mt, x);
      }
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DD; ++i) ov[i] *= alpha;
      for (int j = 0; j < kKeyTile; ++j) {
        const float p = exp2f(sc[j] - m_new);
        lsum += p;
#pragma unroll
        for (int i = 0; i < DD; ++i) ov[i] = fmaf(p, Vs[i][j], ov[i]);
      }
    }
  }
  if (!qvalid) return;
  const float inv = 1.f / lsum;
  float* orow = MODE == 0 ? (float*)out + ((size_t)bh * D.N + tok) * DD : (float*)out + ((size_t)bh * D.M + pos0 + tid) * DD;
#pragma unroll
  for (int i = 0; i < DD; ++i) orow[i] = ov[i] * inv;
  if (MODE == 0 && psp && D.M > 0) {
    const int slot = B.pslot[(size_t)bh * D.N + tok];
    if (slot >= 0) {
      float* prow = psp + ((size_t)bh * D.M + slot) * DD;
#pragma unroll
      for (int i = 0; i < DD; ++i) prow[i] = ov[i] * inv;
    }
  }
}

void launch_attend_sparse(const void* q, const Dims& D, const Bufs& B, void* o_sparse, float* o_psp, hipStream_t s,
                          bool dense) {
  const int nb = D.BH * D.max_tiles;
  if (D.dtype == 1) {
    if (D.d == 128) {
      if (dense)
        hipLaunchKernelGGL((k_bsfa_bf16<128, 2>), dim3(nb), dim3(256), 0, s, (const bf16*)q, D, B, o_sparse, o_psp);
      else
        hipLaunchKernelGGL((k_bsfa_bf16<128, 0>), dim3(nb), dim3(256), 0, s, (const bf16*)q, D, B, o_sparse, o_psp);
    } else {
      if (dense)
        hipLaunchKernelGGL((k_bsfa_bf16<64, 2>), dim3(nb), dim3(256), 0, s, (const bf16*)q, D, B, o_sparse, o_psp);
      else
        hipLaunchKernelGGL((k_bsfa_bf16<64, 0>), dim3(nb), dim3(256), 0, s, (const bf16*)q, D, B, o_sparse, o_psp);
    }
  } else {
    if (D.d == 128)
      hipLaunchKernelGGL((k_bsfa_f32<128, 0>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, o_sparse, o_psp);
    else
      hipLaunchKernelGGL((k_bsfa_f32<64, 0>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, o_sparse, o_psp);
  }
}

void launch_attend_probes(const void* q, const Dims& D, const Bufs& B, float* o_pdn, hipStream_t s) {
  if (D.M == 0 || !o_pdn) return;
  const int nb = D.BH * ((D.M + kAttnQT - 1) / kAttnQT);
  float* none = nullptr;
  if (D.dtype == 1) {
    const int nbk = nb * D.pch;
    if (D.d == 128) {
      hipLaunchKernelGGL((k_bsfa_bf16<128, 1>), dim3(nbk), dim3(256), 0, s, (const bf16*)q, D, B, (void*)o_pdn, none);
      hipLaunchKernelGGL((k_probe_combine<128>), dim3(D.M, D.BH), dim3(128), 0, s, D, B, o_pdn);
    } else {
      hipLaunchKernelGGL((k_bsfa_bf16<64, 1>), dim3(nbk), dim3(256), 0, s, (const bf16*)q, D, B, (void*)o_pdn, none);
      hipLaunchKernelGGL((k_probe_combine<64>), dim3(D.M, D.BH), dim3(64), 0, s, D, B, o_pdn);
    }
  } else {
    if (D.d == 128)
      hipLaunchKernelGGL((k_bsfa_f32<128, 1>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, (void*)o_pdn, none);
    else
      hipLaunchKernelGGL((k_bsfa_f32<64, 1>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, (void*)o_pdn, none);
  }
}

}  // namespace spr
