// Block-sparse softmax attention over the selected (query group, key group) cells, and
// the exact attention of the probe rows (paper "Partition the Support, Reconstruct the
// Residual", abstract; project website, Method section, stage 03 and the PFRR panel).
//
// Query rows of one query group are taken 128 at a time (one tile); the keys are the
// union of the selected key groups, which the permutation made contiguous per group, so
// consecutive selected groups merge into one key run. Softmax is renormalised over the
// retained keys only (online softmax across key tiles).
//
// bf16 path, per workgroup of 4 waves (32 query rows each):
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16: A = K tile rows from LDS, B = Q^T kept in
//                 registers; each lane then holds the scores of ONE query (lane % 32) for 16
//                 keys, so the row max / sum are in-lane plus one cross-half exchange.
//   O^T = V^T P^T with the same MFMA: B = P^T is the score registers converted to bf16 in
//                 place (no shuffles); A = V^T comes from the transposed V layout that the
//                 permutation pass writes, one 16-byte LDS read per operand.
// exp2 with the log2(e) factor folded into the score scale.
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

// Walks the KT-key tiles of one work item over its key runs (the plan lists each query
// group's runs). The runs are copied to LDS when the work item starts, so stepping from run
// to run reads LDS only and never waits on the global loads in flight. A run [lo, hi)
// starts its first tile at lo rounded down to 8 keys (16-byte aligned rows of the
// transposed V); keys outside [lo, hi) are masked.
template <int KT>
struct TileWalk {
  const int2* runs;  // the item's runs, in LDS
  int nr, r;         // runs of the item, current run
  int lo, hi, k0;
  __device__ void set_run() {
    const int2 v = runs[r];  // one address for the whole wave
    lo = __builtin_amdgcn_readfirstlane(v.x);
    hi = __builtin_amdgcn_readfirstlane(v.y);
    k0 = lo & ~7;
  }
  __device__ bool first() {
    r = 0;
    if (nr <= 0) return false;
    set_run();
    return true;
  }
  __device__ bool first_single(int a, int b) {  // one run [a, b), no run list
    r = 0;
    nr = a < b ? 1 : 0;
    lo = a;
    hi = b;
    k0 = a & ~7;
    return nr > 0;
  }
  __device__ bool next() {
    k0 += KT;
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
// Tiles of 32 keys move HBM -> registers -> LDS, two steps ahead: a step issues the global
// loads of K(j+2) and V(j+1) and stores K(j+1) and V(j), loaded a step earlier, at its end
// (direct-to-LDS loads were tried: while they are in flight the operand reads of every wave
// on the CU stall). Rows carry an XOR swizzle of their 16-byte chunks so that the operand
// reads are bank-conflict free without padding.
//
// Step j (one barrier): S(j) = K(j) Q^T on the matrix cores; then O += V(j-1) P(j-1), each
// MFMA followed by a slice of the softmax that turns S(j) into P(j) (P is double-buffered in
// registers). The K rows of a 32-key block are read in the order pi (bits 2 and 3 of the row
// swapped), which makes the eight scores a lane holds for one 16-key chunk eight consecutive
// keys, so the V^T operand is a single 16-byte read per MFMA.
// The reference max is lazy: a tile is exponentiated against the running max, and only a
// tile whose numerators could exceed 2^16 is redone against its exact max (then the
// accumulator is rescaled before the next PV product).
// -------------------------------------------------------------------------------------
__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int DD, int MODE>
__global__ __launch_bounds__(256, 2) void k_bsfa_bf16(const bf16* __restrict__ q, Dims D, Bufs B, void* out,
                                                        float* psp) {
  constexpr int KT = 32;                // keys per tile
  constexpr int KRB = DD * 2;           // K row bytes (256 or 128)
  constexpr int KW = KRB / 16;          // 16-byte slots per K row (16 or 8)
  constexpr int KR = 64 / KW;           // K rows per wave-wide 1 KB load
  constexpr int KI = KT * KRB / 4096;   // 1 KB loads per wave per K tile (4 waves)
  constexpr int VI = DD * KT * 2 / 4096;  // and per V^T tile (rows of 64 bytes)
  constexpr int NC = DD / 16;           // k-chunks of the QK^T product
  constexpr int ND = DD / 32;           // 32-wide d blocks of the output
  static_assert((DD == 64 || DD == 128) && KI >= 1 && VI >= 1, "tile shape");
  __shared__ __attribute__((aligned(1024))) bf16 Kb0[KT * DD], Kb1[KT * DD], Vb0[DD * KT], Vb1[DD * KT];
  __shared__ int2 runs_s[kMaxGroups];

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

  // Tile layout in LDS, no padding: 16-byte slot s of row r holds chunk s ^ swz(r), with
  // swz(r) = r & 15 for 16-slot K rows, (r >> 1) & 7 for 8-slot K rows and (r >> 2) & 3 for
  // the 4-slot V^T rows, so the 16 rows one operand read touches fall on distinct bank groups.
  // Each wave stages whole 1 KB row blocks; the chunk a lane fetches depends on its lane and
  // wave only, so its source is one lane offset plus a per-load scalar.
  auto kswz = [](int r) { return KW == 16 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return (r >> 2) & 3; };
  unsigned klane, vlane;
  {
    const int r = KR * w + l / KW;  // row of this lane in the wave's first load (load g = 4 i + w)
    klane = (unsigned)(r * KRB + 16 * ((l % KW) ^ kswz(r)));
    const int rv = 16 * w + l / 4;
    vlane = (unsigned)(rv * 2 * D.Npad + 16 * ((l % 4) ^ vswz(rv)));
  }
  // Tile staging through registers, two steps deep: the global loads issued in one step are
  // stored to LDS at the end of the next, so a load has about two steps to arrive. Every step
  // issues the same loads (past the last tile they re-read the current one, unused), so the
  // count of loads in flight is the same on every path and the wait before a store covers
  // only the loads of the step before.
  struct Stage {
    bf16x8 k[KI], v[VI];
  };
  auto load_k = [&](Stage& st, int k0) {
    const char* src = (const char*)(kpb + (size_t)k0 * DD);
#pragma unroll
    for (int i = 0; i < KI; ++i) st.k[i] = *reinterpret_cast<const bf16x8*>(src + i * 4 * KR * KRB + klane);
  };
  auto load_v = [&](Stage& st, int k0) {
    const char* src = (const char*)(vtb + k0);
#pragma unroll
    for (int i = 0; i < VI; ++i) st.v[i] = *reinterpret_cast<const bf16x8*>(src + (size_t)i * 128 * D.Npad + vlane);
  };
  auto store_k = [&](const Stage& st, bf16* dst) {
#pragma unroll
    for (int i = 0; i < KI; ++i) *reinterpret_cast<bf16x8*>(dst + (4 * i + w) * 512 + 8 * l) = st.k[i];
  };
  auto store_v = [&](const Stage& st, bf16* dst) {
#pragma unroll
    for (int i = 0; i < VI; ++i) *reinterpret_cast<bf16x8*>(dst + (4 * i + w) * 512 + 8 * l) = st.v[i];
  };

  // operand reads. K: row pi(l32), chunk 2c + h -> byte kaddr ^ 32c;
  // V^T: row 32 db + l32, chunk 2cc + h -> byte (vaddr ^ 32cc) + db * 32 rows.
  const int prow = swap_bits23(l32);
  const unsigned kaddr = (unsigned)(prow * KRB + 16 * (h ^ kswz(prow)));
  const unsigned vaddr = (unsigned)(l32 * 64 + 16 * (h ^ vswz(l32)));
  // The per-chunk addresses are formed where they are used (one v_xor each): an empty asm
  // makes the base opaque so that the compiler does not keep all of them live across the loop.
  auto kread = [&](const bf16* Kc, unsigned kb, int c) {
    return *reinterpret_cast<const bf16x8*>((const char*)Kc + (kb ^ (32u * c)));
  };
  auto vread = [&](const bf16* Vc, unsigned vb, int i) {  // i = cc * ND + db
    const int cc = i / ND, db = i % ND;
    return *reinterpret_cast<const bf16x8*>((const char*)Vc + db * 32 * 64 + (vb ^ (32u * cc)));
  };
  // S^T = K Q^T of one tile; K operands read two k-chunks ahead
  auto qk = [&](const bf16* Kc, f32x16& s) {
    unsigned kb = kaddr;
    asm volatile("" : "+v"(kb));
    bf16x8 ka[NC];
    ka[0] = kread(Kc, kb, 0);
    ka[1] = kread(Kc, kb, 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c == 0) {
        const f32x16 z = {};
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qreg[0], z, 0, 0, 0);
      } else {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qreg[c], s, 0, 0, 0);
      }
      if (c + 2 < NC) ka[c + 2] = kread(Kc, kb, c + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // keys outside [lo, hi) of an edge tile get score -inf; score v is key
  // 16 (v >> 3) + 8 h + (v & 7) of the tile (pi order)
  auto mask = [&](f32x16& s, int k0, int lo, int hi) {
    const int vlo = lo - k0 - 8 * h, vhi = hi - k0 - 8 * h;
    if (lo > k0) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (16 * (v >> 3) + (v & 7) < vlo) s[v] = -INFINITY;
    }
    if (hi < k0 + KT) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (16 * (v >> 3) + (v & 7) >= vhi) s[v] = -INFINITY;
    }
  };
  auto max16 = [&](const f32x16& s) {  // max of the 16 scores (v_max3 tree)
    const float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float c = fmaxf(fmaxf(s[6], s[7]), s[8]), e = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float f = fmaxf(fmaxf(s[12], s[13]), s[14]);
    return fmaxf(fmaxf(fmaxf(a, b), s[15]), fmaxf(fmaxf(c, e), f));
  };
  // moves the accumulator and row sum to max mu when any lane of the wave raised its max
  auto rescale = [&](float mu) {
    if (__builtin_amdgcn_ballot_w64(mu != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mu);
      m_run = mu;
      l_half *= alpha;
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    }
  };
  // Softmax numerators of one tile against the reference max mu, in pairs of scores: scale
  // and shift, exponentiate, pack to bf16 and add the packed pair to the row sum (one
  // v_dot2 with (1, 1), so the sum is of the same rounded values that enter PV). Pair g
  // goes through a three-slice pipeline (shift in slice g, exp in g+1, pack in g+2); slices
  // 0-7 each follow one MFMA of the previous tile's PV product, 8 and 9 close the pipeline.
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
  auto soft_slice = [&](const f32x16& s, int i, float mu, float& ps, float (&xe)[16], bf16x8 (&pn)[2]) {
    const int gp = i - 2, ge = i - 1, gf = i;
    if (gp >= 0 && gp < 8) {
      bf16x2 pr;
      pr[0] = (bf16)xe[2 * gp];
      pr[1] = (bf16)xe[2 * gp + 1];
      pn[gp >> 2][2 * (gp & 3)] = pr[0];
      pn[gp >> 2][2 * (gp & 3) + 1] = pr[1];
      ps = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps, false);
    }
    if (ge >= 0 && ge < 8) {
      xe[2 * ge] = __builtin_amdgcn_exp2f(xe[2 * ge]);
      xe[2 * ge + 1] = __builtin_amdgcn_exp2f(xe[2 * ge + 1]);
    }
    if (gf < 8) {
      xe[2 * gf] = fmaf(s[2 * gf], c2, -mu);
      xe[2 * gf + 1] = fmaf(s[2 * gf + 1], c2, -mu);
    }
  };
  // The reference max is kept lazily: numerators are formed against the running max, and
  // only when a lane's partial row sum of the tile exceeds 2^16 (so some numerator may be
  // large, or infinite) is the tile redone against its exact max; the first tile of a work
  // item, with no max yet, always is. Every numerator kept is therefore <= 2^16: far from
  // overflow in fp32, and bf16 keeps its relative precision at any magnitude.
  auto soft_exact = [&](const f32x16& s, float& mu, float& ps, bf16x8 (&pn)[2]) {
    const float mt = max16(s);
    mu = fmaxf(mu, fmaxf(mt, xor32(mt)) * c2);
    ps = 0.f;
    float xe[16];
#pragma unroll
    for (int i = 0; i < 10; ++i) soft_slice(s, i, mu, ps, xe, pn);
  };
  auto check = [&](const f32x16& s, float& mu, float& ps, bf16x8 (&pn)[2]) {
    if (__builtin_amdgcn_ballot_w64(!(ps <= 65536.f))) soft_exact(s, mu, ps, pn);
  };
  // O^T += V^T P^T of the previous tile (V operands two MFMAs ahead) interleaved with the
  // softmax numerators of the current tile
  auto pv_soft = [&](const bf16* Vp, const bf16x8 (&pp)[2], const f32x16& s, float& mu, float& ps,
                     bf16x8 (&pn)[2]) {
    constexpr int NI = 2 * ND;
    unsigned vb = vaddr;
    asm volatile("" : "+v"(vb));
    bf16x8 va[NI];
    va[0] = vread(Vp, vb, 0);
    va[1] = vread(Vp, vb, 1);
    float xe[16];
    ps = 0.f;
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      if (i < NI) {
        const int cc = i / ND, db = i % ND;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pp[cc], o[db], 0, 0, 0);
        if (i + 2 < NI) va[i + 2] = vread(Vp, vb, i + 2);
      }
      soft_slice(s, i, mu, ps, xe, pn);
      __builtin_amdgcn_sched_barrier(0);
    }
    check(s, mu, ps, pn);
  };
  auto pv = [&](const bf16* Vp, const bf16x8 (&pp)[2]) {
    constexpr int NI = 2 * ND;
    unsigned vb = vaddr;
    asm volatile("" : "+v"(vb));
    bf16x8 va[NI];
    va[0] = vread(Vp, vb, 0);
    va[1] = vread(Vp, vb, 1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int cc = i / ND, db = i % ND;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pp[cc], o[db], 0, 0, 0);
      if (i + 2 < NI) va[i + 2] = vread(Vp, vb, i + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  TileWalk<KT> ts;
  bool has;  // the next tile exists
  if (MODE != 1) {
    const int2* rg = B.runs + (size_t)bh * D.Cq * D.Ck + B.row_ptr[(size_t)bh * (D.Cq + 1) + a];
    const int nr = __builtin_amdgcn_readfirstlane(B.nruns[(size_t)bh * D.Cq + a]);  // <= C_k <= kMaxGroups
    for (int i = tid; i < nr; i += 256) runs_s[i] = rg[i];
    __syncthreads();
    ts.runs = runs_s;
    ts.nr = nr;
    has = ts.first();
  } else {
    const int clo = a * D.pkc;
    has = ts.first_single(clo, min(D.N, clo + D.pkc));
  }
  // Tile j: K(j) sits in K buffer j%2 and V(j) in V buffer j%2. Step j (j >= 1) loads K(j+1)
  // and V(j) into registers, forms S(j), runs O += V(j-1) P(j-1) while it turns S(j) into
  // P(j), and stores the loaded tiles at its end. P is double-buffered in registers (pa, pb
  // by parity); the max and row sum of P(j) are applied (rescale, sum) at the start of step
  // j+1, after P(j-1) has entered O. Tile 0 is handled before the loop and the last PV after
  // it, so every step runs the same code and O never changes registers.
  bf16x8 pp[2];  // P^T operands of the pending tile
  float mu = -INFINITY, ps = 0.f;
  if (has) {
    // tile descriptors: j (current), j+1, j+2
    int k0c = ts.k0, loc = ts.lo, hic = ts.hi;
    bool has1 = ts.next();
    int k01 = ts.k0, lo1 = ts.lo, hi1 = ts.hi;
    bool has2 = has1 && ts.next();
    int k02 = ts.k0;
    Stage sa, sb;  // sa: K(j+1), V(j) (stored at the end of step j); sb: K(j+2), V(j+1)
    load_k(sa, k0c);
    store_k(sa, Kb0);
    load_k(sa, has1 ? k01 : k0c);
    load_v(sa, k0c);
    // Step j: K(j) is in K buffer j%2, V(j-1) in V buffer (j-1)%2. Load K(j+2) and V(j+1);
    // S(j) = K(j) Q^T; O += V(j-1) P(j-1) while S(j) turns into P(j); store K(j+1) and V(j).
    // Step 0 has no PV; one loop body serves both parities, so O keeps its registers.
    __syncthreads();
    load_k(sb, has2 ? k02 : k0c);
    load_v(sb, has1 ? k01 : k0c);
    if (wave_active) {
      f32x16 s;
      qk(Kb0, s);
      if (loc > k0c || hic < k0c + KT) mask(s, k0c, loc, hic);
      soft_exact(s, mu, ps, pp);
    }
    if (has1) store_k(sa, Kb1);
    store_v(sa, Vb0);
    int par = 0;  // parity of the last tile
    // step of tile j; `cur` holds K(j+1), V(j) (loaded a step ago), `nxt` receives K(j+2), V(j+1)
    auto step = [&](Stage& cur, Stage& nxt) {
      k0c = k01; loc = lo1; hic = hi1;
      has1 = has2;
      k01 = k02; lo1 = ts.lo; hi1 = ts.hi;
      has2 = has2 && ts.next();
      k02 = ts.k0;
      par ^= 1;
      const bf16* Kc = par ? Kb1 : Kb0;
      bf16* Kn = par ? Kb0 : Kb1;
      const bf16* Vp = par ? Vb0 : Vb1;
      bf16* Vc = par ? Vb1 : Vb0;
      __syncthreads();
      load_k(nxt, has2 ? k02 : k0c);
      load_v(nxt, has1 ? k01 : k0c);
      if (wave_active) {
        rescale(mu);
        l_half += ps;
        f32x16 s;
        qk(Kc, s);
        if (loc > k0c || hic < k0c + KT) mask(s, k0c, loc, hic);
        bf16x8 pn[2];
        pv_soft(Vp, pp, s, mu, ps, pn);
        pp[0] = pn[0];
        pp[1] = pn[1];
      }
      if (has1) store_k(cur, Kn);
      store_v(cur, Vc);
    };
    // whole pairs of steps (stages swap roles twice), then at most one more step
    while (has1 && has2) {
      step(sb, sa);
      step(sa, sb);
    }
    if (has1) step(sb, sa);
    // O += V(T-1) P(T-1), V(T-1) in V buffer par
    __syncthreads();
    if (wave_active) {
      rescale(mu);
      l_half += ps;
      pv(par ? Vb1 : Vb0, pp);
    }
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
