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

// Walks the 64-key tiles of one work item over its key runs (the plan lists each query
// group's runs). The runs are held one per lane, 64 at a time, and read out with v_readlane,
// so stepping from tile to tile touches no memory. A run [lo, hi) starts its first tile at lo
// rounded down to 8 keys (16-byte aligned rows of the transposed V); keys outside [lo, hi)
// are masked.
struct TileWalk {
  const int2* runs;
  int nr, r;      // runs of the item, current run
  int rlo, rhi;   // this lane's run of the current batch of 64
  int lo, hi, k0;
  __device__ void load_batch(int base) {
    const int i = base + lane_id();
    const int2 v = i < nr ? runs[i] : make_int2(0, 0);
    rlo = v.x;
    rhi = v.y;
  }
  __device__ void set_run() {
    if (r > 0 && (r & 63) == 0) load_batch(r);
    lo = __builtin_amdgcn_readlane(rlo, r & 63);
    hi = __builtin_amdgcn_readlane(rhi, r & 63);
    k0 = lo & ~7;
  }
  __device__ bool first() {
    r = 0;
    if (nr <= 0) return false;
    load_batch(0);
    set_run();
    return true;
  }
  __device__ bool first_single(int a, int b) {  // one run [a, b), no run list
    r = 0;
    nr = a < b ? 1 : 0;
    rlo = a;
    rhi = b;
    lo = a;
    hi = b;
    k0 = a & ~7;
    return nr > 0;
  }
  __device__ bool next() {
    k0 += kKeyTile;
    if (k0 < hi) return true;
    if (++r >= nr) return false;
    set_run();
    return true;
  }
};

// -------------------------------------------------------------------------------------
// bf16 MFMA kernel. MODE 0: block-sparse tiles from the tile table, bf16 output in token
// order (plus float rows for probes). MODE 1: probe rows (128 per block) over one chunk of
// all keys, partial outputs for the chunk combine. MODE 2: the same code as MODE 0 under its
// own symbol, used by the dense reference call so that traces keep the two apart.
//
// Tiles move HBM -> LDS with direct-to-LDS loads (global_load_lds_dwordx4: lane i of a wave
// lands 16 bytes at base + 16 i), so no registers stage them. Rows carry an XOR swizzle of
// their 16-byte chunks so that the operand reads are bank-conflict free without padding.
//
// Pipeline per 64-key tile j (one barrier per tile):
//   barrier: K(j+1) and V(j) have landed; everyone is done with K(j) and V(j-1)
//   issue loads K(j+2) -> K buffer of j, V(j+1) -> V buffer of j-1
//   S(j+1) = K(j+1) Q^T  (MFMA)   interleaved with   softmax of S(j) (VALU)
//   O += V(j) P(j)       (MFMA)
// The K rows of a 32-key block are read in the order pi (bits 2 and 3 of the row swapped),
// which makes the eight scores a lane holds for one 16-key chunk eight consecutive keys, so
// the V^T operand is a single 16-byte read per MFMA.
// The accumulator is rescaled only when a query's running max grows by more than 2^8 (the
// stale max keeps every exponent <= 2^8, exact enough in fp32 and bf16).
// -------------------------------------------------------------------------------------
__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int DD, int MODE>
__global__ __launch_bounds__(256, 2) void k_bsfa_bf16(const bf16* __restrict__ q, Dims D, Bufs B, void* out,
                                                        float* psp) {
  constexpr int KT = kKeyTile;          // keys per tile
  constexpr int KRB = DD * 2;           // K row bytes (256 or 128)
  constexpr int KW = KRB / 16;          // 16-byte slots per K row
  constexpr int KR = 64 / KW;           // K rows per wave-wide direct load
  constexpr int KI = KT * KRB / 4096;   // direct loads per wave per K tile (4 waves, 1 KB each)
  constexpr int VI = DD * KT * 2 / 4096;  // and per V^T tile (rows of 128 bytes)
  constexpr int NC = DD / 16;           // k-chunks of the QK^T product
  constexpr int ND = DD / 32;           // 32-wide d blocks of the output
  static_assert(KT == 64 && (DD == 64 || DD == 128), "tile shape");
  __shared__ __attribute__((aligned(1024))) bf16 Kb0[KT * DD], Kb1[KT * DD], Vb0[DD * KT], Vb1[DD * KT];

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
  const int tid = threadIdx.x, l = lane_id(), h = l >> 5, l32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);

  // ---- Q^T operand in registers: query (32w + l32), d-slots 16c + 8h .. +7
  const int qr = 32 * w + l32;
  const bool qvalid = qr < rows;
  const bool wave_active = 32 * w < rows;  // a wave past the tile's last row only loads K / V
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

  // Tile layout in LDS, no padding: 16-byte slot s of row r holds chunk s ^ swz(r), with
  // swz(r) = r & 15 for 16-slot rows and (r >> 1) & 7 for 8-slot rows, so the 16 rows one
  // operand read touches fall on 16 distinct bank groups. Wave-wide direct load g fills
  // rows [64g / slots, ...) contiguously; the chunk a lane fetches depends on its lane and
  // wave only, so its source is one lane offset plus a per-load scalar.
  auto swz = [](int r, int slots) { return slots == 16 ? (r & 15) : ((r >> 1) & 7); };
  unsigned klane, vlane;
  {
    const int r = KR * w + l / KW;  // row within the wave's first load (load g = 4 i + w)
    klane = (unsigned)(r * KRB + 16 * ((l % KW) ^ swz(r, KW)));
    const int rv = 8 * w + l / 8;
    vlane = (unsigned)(rv * 2 * D.Npad + 16 * ((l % 8) ^ swz(rv, 8)));
  }
  auto issue_k = [&](bf16* dst, int k0) {
    const char* src = (const char*)(kpb + (size_t)k0 * DD);
#pragma unroll
    for (int i = 0; i < KI; ++i)
      __builtin_amdgcn_global_load_lds(src + (size_t)i * 4 * KR * KRB + klane, dst + (4 * i + w) * 512, 16, 0, 0);
  };
  auto issue_v = [&](bf16* dst, int k0) {
    const char* src = (const char*)(vtb + k0);
#pragma unroll
    for (int i = 0; i < VI; ++i)
      __builtin_amdgcn_global_load_lds(src + (size_t)i * 32 * 2 * D.Npad + vlane, dst + (4 * i + w) * 512, 16, 0, 0);
  };

  // operand reads. K: row 32 kb + pi(l32), chunk 2c + h -> byte (kaddr ^ 32c) + kb * 32 rows;
  // V^T: row 32 db + l32, chunk 2cc + h -> byte (vaddr ^ 32cc) + db * 32 rows.
  const int prow = swap_bits23(l32);
  const unsigned kaddr = (unsigned)(prow * KRB + 16 * (h ^ swz(prow, KW)));
  const unsigned vaddr = (unsigned)(l32 * 128 + 16 * (h ^ swz(l32, 8)));
  auto qk = [&](const bf16* Kc, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>((const char*)Kc + kb * 32 * KRB + (kaddr ^ (32u * c)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[c], s[kb], 0, 0, 0);
      }
  };
  // keys outside [lo, hi) of an edge tile get score -inf
  auto mask = [&](f32x16 (&s)[2], int k0, int lo, int hi) {
    const int vlo = lo - k0, vhi = hi - k0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = 32 * kb + 16 * (v >> 3) + 8 * h + (v & 7);  // key of score v (pi order)
        if (kk < vlo || kk >= vhi) s[kb][v] = -INFINITY;
      }
  };
  // exponentials of one tile against the running max, raised lazily: mu is the max this tile
  // uses (the tile max when it exceeds the running one by more than 2^8, else the running
  // max). Returns the P^T operands (chunk cc = 2 kb + sub) and the tile's share of the row sum.
  auto expo = [&](f32x16 (&s)[2], bf16x8 (&pb)[4], float& ps, float& mu) {
    float mx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, b = 8 * (t & 1);
      mx[t] = fmaxf(fmaxf(fmaxf(s[kb][b], s[kb][b + 1]), fmaxf(s[kb][b + 2], s[kb][b + 3])),
                    fmaxf(fmaxf(s[kb][b + 4], s[kb][b + 5]), fmaxf(s[kb][b + 6], s[kb][b + 7])));
    }
    float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    mt = fmaxf(mt, xor32(mt)) * c2;
    mu = mt > m_run + 8.f ? mt : m_run;
    float pt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, b = 8 * (t & 1);
      float e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) e[u] = __builtin_amdgcn_exp2f(fmaf(s[kb][b + u], c2, -mu));
      pt[t] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
#pragma unroll
      for (int u = 0; u < 8; ++u) pb[t][u] = (bf16)e[u];
    }
    ps = (pt[0] + pt[1]) + (pt[2] + pt[3]);
  };
  // moves the accumulator to the new max when any lane of the wave raised it
  auto rescale = [&](float mu, float ps) {
    if (__builtin_amdgcn_ballot_w64(mu != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
      m_run = mu;
      l_half *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    }
    l_half += ps;
  };
  auto pv = [&](const bf16* Vc, const bf16x8 (&pb)[4]) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>((const char*)Vc + db * 32 * 128 + (vaddr ^ (32u * cc)));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[cc], o[db], 0, 0, 0);
      }
  };

  TileWalk ts;
  bool hasc;
  if (MODE != 1) {
    ts.runs = B.runs + (size_t)bh * D.Cq * D.Ck + B.row_ptr[(size_t)bh * (D.Cq + 1) + a];
    ts.nr = B.nruns[(size_t)bh * D.Cq + a];
    hasc = ts.first();
  } else {
    const int clo = a * D.pkc;
    hasc = ts.first_single(clo, min(D.N, clo + D.pkc));
  }
  // tile descriptors: current (j), next (j+1), after next (j+2)
  int k0c = 0, loc = 0, hic = 0, k0n = 0, lon = 0, hin = 0;
  f32x16 sa[2], sb[2];
  if (hasc) {
    k0c = ts.k0; loc = ts.lo; hic = ts.hi;
    issue_k(Kb0, k0c);
    issue_v(Vb0, k0c);
  }
  bool hasn = hasc && ts.next();
  if (hasn) {
    k0n = ts.k0; lon = ts.lo; hin = ts.hi;
    issue_k(Kb1, k0n);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (hasc && wave_active) qk(Kb0, sa);

  // one tile: Kn = K buffer of tile j+1, Kc = K buffer of tile j (refilled with j+2),
  // Vc = V buffer of tile j, Vn = V buffer of tile j+1
  auto step = [&](f32x16 (&scur)[2], f32x16 (&snext)[2], bf16* Kc, const bf16* Kn, const bf16* Vc, bf16* Vn) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads have landed
    __syncthreads();
    bool hasnn = false;
    int k0nn = 0, lonn = 0, hinn = 0;
    if (hasn) {
      hasnn = ts.next();
      if (hasnn) {
        k0nn = ts.k0; lonn = ts.lo; hinn = ts.hi;
        issue_k(Kc, k0nn);
      }
      issue_v(Vn, k0n);
    }
    if (wave_active) {
      if (k0c < loc || k0c + KT > hic) mask(scur, k0c, loc, hic);
      bf16x8 pb[4];
      float ps, mu;
      if (hasn) {
        // S(j+1) on the matrix cores while the vector units exponentiate S(j)
        qk(Kn, snext);
        expo(scur, pb, ps, mu);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 2 * NC; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i + 2 < 2 * NC) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 128 / (2 * NC), 0);
        }
      } else {
        expo(scur, pb, ps, mu);
      }
      rescale(mu, ps);
      pv(Vc, pb);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 4 * ND; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + 2 < 4 * ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    hasc = hasn;
    k0c = k0n; loc = lon; hic = hin;
    hasn = hasnn;
    k0n = k0nn; lon = lonn; hin = hinn;
  };
  while (hasc) {
    step(sa, sb, Kb0, Kb1, Vb0, Vb1);
    if (!hasc) break;
    step(sb, sa, Kb1, Kb0, Vb1, Vb0);
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
