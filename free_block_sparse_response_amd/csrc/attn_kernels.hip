// Block-sparse softmax attention over the selected (query group, key group) cells, and
// the exact attention of the probe rows (paper "Partition the Support, Reconstruct the
// Residual", abstract; project website, Method section, stage 03 and the PFRR panel).
//
// Query rows of one query group are taken 128 or 256 at a time (a tile of 4 or 8 waves,
// 32 rows each; the 8-wave kernel also runs two chunks of rows on separate key streams, see
// below); the keys are the union of the selected key groups, which the permutation made
// contiguous per group, so consecutive selected groups merge into one key run. Softmax is
// renormalised over the retained keys only (online softmax across key tiles).
//
// bf16 path, per wave of 32 query rows:
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16: A = K tile rows from LDS, B = Q^T kept in
//                 registers; each lane then holds the scores of ONE query (lane % 32) for 16
//                 keys, so the row max / sum are in-lane plus one cross-half exchange.
//   O^T = V^T P^T with the same MFMA: B = P^T is the score registers converted to bf16 in
//                 place (no shuffles); A = V^T comes from the transposed V layout that the
//                 permutation pass writes, one 16-byte LDS read per operand.
// exp2 with the log2(e) factor folded into the score scale.
#include <type_traits>

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

// Walks the key runs of a query group: consecutive selected key groups merge into one run
// (the fp32 kernel reads the route directly).
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
  // Tiles of one run (its first starts at lo rounded down to 8 keys).
  __device__ static int run_tiles(int2 v) { return (v.y - (v.x & ~7) + KT - 1) / KT; }
  // Tiles of the whole item; the wave's lanes share the runs (wave-uniform result).
  __device__ int count() const {
    int c = 0;
    for (int i = lane_id(); i < nr; i += kWave) c += run_tiles(runs[i]);
    return __builtin_amdgcn_readfirstlane(wave_sum_i(c));
  }
  // Positions the walk on tile t (0-based over the item's runs, t below count()): the lanes
  // scan 64 runs at a time for the first run whose tiles reach past t.
  __device__ void seek(int t) {
    int base = 0;  // tiles of the runs before this chunk
    for (int i0 = 0; i0 < nr; i0 += kWave) {
      const int i = i0 + lane_id();
      const int c = i < nr ? run_tiles(runs[i]) : 0;
      const int incl = wave_incl_scan(c);
      const uint64_t hit = __ballot(i < nr && base + incl > t);
      if (hit) {
        const int j = __builtin_amdgcn_readfirstlane(__builtin_ffsll((long long)hit) - 1);
        const int before = __builtin_amdgcn_readfirstlane(base + __shfl(incl - c, j, kWave));
        r = i0 + j;
        set_run();
        k0 += (t - before) * KT;
        return;
      }
      base += __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));
    }
  }
};

// -------------------------------------------------------------------------------------
// bf16 MFMA kernel, W waves of 32 query rows per workgroup (a tile of up to 32 W rows of one
// query group), KT keys per step (a multiple of 32). MODE 0: block-sparse work items from the
// attention tile table (4 waves) or the paired item table (8 waves), bf16 output in token
// order (plus float rows for probes). MODE 1:
// probe rows (32 W per block) over one chunk of all keys, partial outputs for the chunk
// combine. MODE 2: the same code as MODE 0 under its own symbol, used by the dense
// reference call so that traces keep the two apart.
//
// Tiles of KT keys move HBM -> registers -> LDS, STG steps ahead: a step issues the global
// loads of K(j+STG) and V(j+STG-1) and stores, at its end, the K and V tiles it loaded STG-1
// steps earlier (direct-to-LDS loads were tried: while they are in flight the operand reads
// of every wave on the CU stall). Rows carry an XOR swizzle of their 16-byte chunks so that
// the operand reads are bank-conflict free without padding (16 lanes of a 128-bit read
// cover the 64 banks).
//
// Step j (one barrier): S(j) = K(j) Q^T on the matrix cores, one 32-key sub-block per
// accumulator, the sub-blocks' product chains interleaved; then O += V(j-1) P(j-1), each
// MFMA followed by a slice of the softmax that turns S(j) into P(j) (P is double-buffered in
// registers). The K rows of a 32-key block are read in the order pi (bits 2 and 3 of the
// row swapped), which makes the eight scores a lane holds for one 16-key chunk eight
// consecutive keys, so the V^T operand is a single 16-byte read per MFMA. Operand reads run
// PF products ahead.
// The reference max is lazy: a tile is exponentiated against the running max, and only a
// tile whose numerators could exceed 2^16 is redone against its exact max (then the
// accumulator is rescaled before the next PV product).
// -------------------------------------------------------------------------------------
__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int DD, int MODE, int W, int KT, int STG>
__global__ __launch_bounds__(64 * W, W == 4 ? 2 : 1) void k_bsfa_bf16(const bf16* __restrict__ q, Dims D, Bufs B,
                                                                       void* out, float* psp) {
  constexpr int KRB = DD * 2;                // K row bytes (256 or 128)
  constexpr int KW = KRB / 16;               // 16-byte slots per K row (16 or 8)
  constexpr int KR = 64 / KW;                // K rows per wave-wide 1 KB load
  constexpr int VRB = KT * 2;                // V^T row bytes (keys of one dim)
  constexpr int VW = VRB / 16;               // 16-byte slots per V^T row
  constexpr int VR = 1024 / VRB;             // V^T rows per wave-wide 1 KB load
  constexpr int NC = DD / 16;                // k-chunks of the QK^T product
  constexpr int ND = DD / 32;                // 32-wide d blocks of the output
  constexpr int SB = KT / 32;                // 32-key sub-blocks per tile
  constexpr int NCC = KT / 16;               // 16-key chunks of P per tile
  constexpr int NPV = NCC * ND;              // PV products per step
  constexpr int NPAIR = 8 * SB;              // score pairs per lane per step
  constexpr int PF = 4;                      // operand reads ahead of their product
  constexpr int QT = 32 * W;                 // query rows per tile
  constexpr int KTB = KT * DD;               // elements of one K or V^T tile
  // 8-wave block-sparse work items (the attention item table) run one chunk of up to 256
  // rows on all waves, or two key streams, each with its own staging buffers and staged by
  // one wave half: a chunk of at most 128 rows split (waves w and w + 4 hold the same 32 rows
  // and walk half of the chunk's key tiles each; the two partial softmax states are merged
  // through LDS at the end), or a pair of chunks of two query groups (waves 0 .. w_0 - 1 on
  // the first, the rest on the second, each on its own group's keys)
  constexpr bool CAN_SPLIT = MODE == 0 && W == 8;
  constexpr int NS = CAN_SPLIT ? 2 : 1;      // key streams
  static_assert((DD == 64 || DD == 128) && (KT == 32 || KT == 64), "tile shape");
  static_assert(STG == 1 || STG == 2, "staging depth");
  __shared__ __attribute__((aligned(1024))) bf16 smem[NS * 4 * KTB];  // per stream: K[2], V^T[2]
  __shared__ int2 runs_s[NS][kMaxGroups];

  const int nb = gridDim.x;
  const int bid = xcd_remap(blockIdx.x, nb);
  int bh, rows, a = 0, pos0 = 0;
  int kind = -1, a1 = 0, pos1 = 0, rows1 = 0;  // the second chunk of a pair (kind >= 0)
  if (MODE != 1) {
    bh = bid / D.max_atiles;
    const int t = bid % D.max_atiles;
    const int* qo = B.qoff + (size_t)bh * (D.Cq + 1);
    if constexpr (CAN_SPLIT) {
      if (t >= B.nptiles[bh]) return;
      const int4 pt = B.ptiles[(size_t)bh * D.max_atiles + t];
      a = pt.x;
      pos0 = pt.y;
      kind = pt.z;
      if (kind >= 0) {
        a1 = pt.z;
        pos1 = pt.w;
        rows1 = min(QT, qo[a1 + 1] - pos1);
      }
    } else {
      if (t >= B.antiles[bh]) return;
      const int2 tl = B.atiles[(size_t)bh * D.max_atiles + t];
      a = tl.x;
      pos0 = tl.y;
    }
    rows = min(QT, qo[a + 1] - pos0);
  } else {
    // probe rows: (head, QT-row tile, key chunk)
    const int per = ((D.M + QT - 1) / QT) * D.pch;
    bh = bid / per;
    const int rem = bid % per;
    pos0 = (rem / D.pch) * QT;
    a = rem % D.pch;  // key chunk
    rows = min(QT, D.M - pos0);
  }
  const int tid = threadIdx.x, l = lane_id(), h = l >> 5, l32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const float c2 = D.log2_scale;
  const bf16* kpb = (const bf16*)B.kp + (size_t)bh * D.Npad * DD;
  const bf16* vtb = (const bf16*)B.vpt + (size_t)bh * DD * D.Npad;
  int nr = 0, nr1 = 0;
  if (MODE != 1) {
    const int* rp = B.row_ptr + (size_t)bh * (D.Cq + 1);
    const int2* rg = B.runs + (size_t)bh * D.Cq * D.Ck + rp[a];
    nr = __builtin_amdgcn_readfirstlane(B.nruns[(size_t)bh * D.Cq + a]);  // <= C_k <= kMaxGroups
    for (int i = tid; i < nr; i += 64 * W) runs_s[0][i] = rg[i];
    if (CAN_SPLIT && kind >= 0) {
      const int2* rg1 = B.runs + (size_t)bh * D.Cq * D.Ck + rp[a1];
      nr1 = __builtin_amdgcn_readfirstlane(B.nruns[(size_t)bh * D.Cq + a1]);
      for (int i = tid; i < nr1; i += 64 * W) runs_s[NS - 1][i] = rg1[i];
    }
    __syncthreads();
  }

  // BM 0: one chunk on all waves; 1: one chunk, its keys split between the wave halves;
  // 2: a pair of chunks
  auto body = [&](auto mode_tag) {
    constexpr int BM = decltype(mode_tag)::value;
    constexpr bool TWO = BM != 0;              // two key streams
    constexpr int WL = TWO ? W / 2 : W;        // loader waves per key stream
    constexpr int STGX = TWO ? 1 : STG;        // two streams stage one step ahead
    constexpr int KI = KT * KRB / (1024 * WL); // 1 KB loads per wave per K tile
    constexpr int VI = DD * VRB / (1024 * WL); // 1 KB loads per wave per V^T tile
    static_assert(KI >= 1 && VI >= 1, "loads per wave");
    const int ls = TWO ? w / WL : 0;           // the stream this wave stages
    const int lw = TWO ? w % WL : w;           // its loader index there
    const int wa = BM == 2 ? (rows + 31) / 32 : WL;    // waves on the first chunk of a pair
    const int cs = BM == 2 ? (w < wa ? 0 : 1) : ls;    // the stream this wave computes
    const int sw = BM == 2 ? (cs ? w - wa : w) : lw;   // its row slice there
    const int crows = BM == 2 && cs ? rows1 : rows;    // rows and first position of its chunk
    const int cpos = BM == 2 && cs ? pos1 : pos0;
    auto Kb = [&](int st, int p) { return smem + (4 * st + p) * KTB; };
    auto Vb = [&](int st, int p) { return smem + (4 * st + 2 + p) * KTB; };

    // ---- Q^T operand in registers: query (32 sw + l32), d-slots 16c + 8h .. +7
    const int qr = 32 * sw + l32;
    const bool qvalid = qr < crows;
    const bool wave_active = 32 * sw < crows;  // a wave past its chunk's last row only stages K / V
    int tok;
    if (MODE != 1) tok = B.qperm[(size_t)bh * D.N + cpos + (qvalid ? qr : 0)];
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

    // Tile layout in LDS, no padding: 16-byte slot s of row r holds chunk s ^ swz(r), with
    // swz(r) = r & 15 for 16-slot rows and (r >> 1) & 7 for 8-slot rows (K rows of d = 64,
    // V^T rows of 64 keys), (r >> 2) & 3 for the 4-slot V^T rows of 32 keys, so the 16 rows
    // one 16-lane group of an operand read touches fall on distinct banks. Each wave stages
    // whole 1 KB row blocks; the chunk a lane fetches depends on its lane and loader index
    // only, so its source is one lane offset plus a per-load scalar.
    auto kswz = [](int r) { return KW == 16 ? (r & 15) : ((r >> 1) & 7); };
    auto vswz = [](int r) { return VW == 4 ? ((r >> 2) & 3) : (VW == 8 ? ((r >> 1) & 7) : (r & 15)); };
    unsigned klane, vlane;
    {
      const int r = KR * lw + l / KW;  // row of this lane in the wave's first load (load g = WL i + lw)
      klane = (unsigned)(r * KRB + 16 * ((l % KW) ^ kswz(r)));
      const int rv = VR * lw + l / VW;
      vlane = (unsigned)(rv * 2 * D.Npad + 16 * ((l % VW) ^ vswz(rv)));
    }
    // Every step issues the same loads (past the last tile they re-read the current one,
    // unused), so the count of loads in flight is the same on every path and the wait before
    // a store covers only the loads issued STGX - 1 steps before.
    struct Stage {
      bf16x8 k[KI], v[VI];
    };
    auto load_k = [&](Stage& st, int k0) {
      const char* src = (const char*)(kpb + (size_t)k0 * DD);
#pragma unroll
      for (int i = 0; i < KI; ++i) st.k[i] = *reinterpret_cast<const bf16x8*>(src + i * WL * KR * KRB + klane);
    };
    auto load_v = [&](Stage& st, int k0) {
      const char* src = (const char*)(vtb + k0);
#pragma unroll
      for (int i = 0; i < VI; ++i)
        st.v[i] = *reinterpret_cast<const bf16x8*>(src + (size_t)i * WL * VR * 2 * D.Npad + vlane);
    };
    auto store_k = [&](const Stage& st, bf16* dst) {
#pragma unroll
      for (int i = 0; i < KI; ++i) *reinterpret_cast<bf16x8*>(dst + (WL * i + lw) * 512 + 8 * l) = st.k[i];
    };
    auto store_v = [&](const Stage& st, bf16* dst) {
#pragma unroll
      for (int i = 0; i < VI; ++i) *reinterpret_cast<bf16x8*>(dst + (WL * i + lw) * 512 + 8 * l) = st.v[i];
    };

    // operand reads. K: row 32 sb + pi(l32), chunk 2c + h -> byte sb * 32 rows + (kaddr ^ 32c);
    // V^T: row 32 db + l32, chunk 2cc + h -> byte (vaddr ^ 32cc) + db * 32 rows.
    const int prow = swap_bits23(l32);
    const unsigned kaddr = (unsigned)(prow * KRB + 16 * (h ^ kswz(prow)));
    const unsigned vaddr = (unsigned)(l32 * VRB + 16 * (h ^ vswz(l32)));
    auto kread = [&](const bf16* Kc, unsigned kb, int i) {  // i = sb * NC + c
      const int sb = i / NC, c = i % NC;
      return *reinterpret_cast<const bf16x8*>((const char*)Kc + sb * 32 * KRB + (kb ^ (32u * c)));
    };
    auto vread = [&](const bf16* Vc, unsigned vb, int i) {  // i = cc * ND + db
      const int cc = i / ND, db = i % ND;
      return *reinterpret_cast<const bf16x8*>((const char*)Vc + db * 32 * VRB + (vb ^ (32u * cc)));
    };
    // S^T = K Q^T of one tile: product j is chunk j / SB of sub-block j % SB, so consecutive
    // products feed different accumulators. The per-chunk addresses are formed where they
    // are used (one v_xor each): an empty asm makes the base opaque so that the compiler does
    // not keep all of them live across the loop.
    auto qk = [&](const bf16* Kc, f32x16 (&s)[SB]) {
      unsigned kb = kaddr;
      asm volatile("" : "+v"(kb));
      constexpr int NI = NC * SB;
      auto idx = [](int j) { return (j % SB) * NC + j / SB; };
      bf16x8 ka[NI];
#pragma unroll
      for (int j = 0; j < PF; ++j) ka[j] = kread(Kc, kb, idx(j));
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int sb = j % SB, c = j / SB;
        if (c == 0) {
          const f32x16 z = {};
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], qreg[0], z, 0, 0, 0);
        } else {
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[j], qreg[c], s[sb], 0, 0, 0);
        }
        if (j + PF < NI) ka[j + PF] = kread(Kc, kb, idx(j + PF));
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // keys outside [lo, hi) of an edge tile get score -inf; score v of sub-block sb is key
    // 32 sb + 16 (v >> 3) + 8 h + (v & 7) of the tile (pi order)
    auto mask = [&](f32x16 (&s)[SB], int k0, int lo, int hi) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int vlo = lo - k0 - 32 * sb - 8 * h, vhi = hi - k0 - 32 * sb - 8 * h;
        if (lo > k0 + 32 * sb) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (16 * (v >> 3) + (v & 7) < vlo) s[sb][v] = -INFINITY;
        }
        if (hi < k0 + 32 * sb + 32) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (16 * (v >> 3) + (v & 7) >= vhi) s[sb][v] = -INFINITY;
        }
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
    // Softmax numerators of one tile against the reference max mu, in pairs of scores:
    // scale and shift, exponentiate, pack to bf16 and add the packed pair to the row sum (one
    // v_dot2 with (1, 1), so the sum is of the same rounded values that enter PV). Pair g
    // (scores 2g, 2g + 1 of sub-block g / 8) goes through a three-slice pipeline (shift in
    // slice g, exp in g+1, pack in g+2) and lands in P chunk g / 4; the slices follow the
    // MFMAs of the previous tile's PV product, the last two close the pipeline.
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
    auto soft_slice = [&](const f32x16 (&s)[SB], int i, float mu, float& ps, float (&xe)[2 * NPAIR],
                          bf16x8 (&pn)[NCC]) {
      const int gp = i - 2, ge = i - 1, gf = i;
      if (gp >= 0 && gp < NPAIR) {
        bf16x2 pr;
        pr[0] = (bf16)xe[2 * gp];
        pr[1] = (bf16)xe[2 * gp + 1];
        pn[gp >> 2][2 * (gp & 3)] = pr[0];
        pn[gp >> 2][2 * (gp & 3) + 1] = pr[1];
        ps = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps, false);
      }
      if (ge >= 0 && ge < NPAIR) {
        xe[2 * ge] = __builtin_amdgcn_exp2f(xe[2 * ge]);
        xe[2 * ge + 1] = __builtin_amdgcn_exp2f(xe[2 * ge + 1]);
      }
      if (gf < NPAIR) {
        const int sb = gf / 8, v = 2 * (gf % 8);
        xe[2 * gf] = fmaf(s[sb][v], c2, -mu);
        xe[2 * gf + 1] = fmaf(s[sb][v + 1], c2, -mu);
      }
    };
    // The reference max is kept lazily: numerators are formed against the running max, and
    // only when a lane's partial row sum of the tile exceeds 2^16 (so some numerator may be
    // large, or infinite) is the tile redone against its exact max; the first tile of a work
    // item, with no max yet, always is. Every numerator kept is therefore <= 2^16: far from
    // overflow in fp32, and bf16 keeps its relative precision at any magnitude.
    auto soft_exact = [&](const f32x16 (&s)[SB], float& mu, float& ps, bf16x8 (&pn)[NCC]) {
      float mt = max16(s[0]);
#pragma unroll
      for (int sb = 1; sb < SB; ++sb) mt = fmaxf(mt, max16(s[sb]));
      mu = fmaxf(mu, fmaxf(mt, xor32(mt)) * c2);
      ps = 0.f;
      float xe[2 * NPAIR];
#pragma unroll
      for (int i = 0; i < NPAIR + 2; ++i) soft_slice(s, i, mu, ps, xe, pn);
    };
    auto check = [&](const f32x16 (&s)[SB], float& mu, float& ps, bf16x8 (&pn)[NCC]) {
      if (__builtin_amdgcn_ballot_w64(!(ps <= 65536.f))) soft_exact(s, mu, ps, pn);
    };
    // O^T += V^T P^T of the previous tile interleaved with the softmax numerators of the
    // current tile
    auto pv_soft = [&](const bf16* Vp, const bf16x8 (&pp)[NCC], const f32x16 (&s)[SB], float& mu, float& ps,
                       bf16x8 (&pn)[NCC]) {
      unsigned vb = vaddr;
      asm volatile("" : "+v"(vb));
      bf16x8 va[NPV];
#pragma unroll
      for (int j = 0; j < PF; ++j) va[j] = vread(Vp, vb, j);
      float xe[2 * NPAIR];
      ps = 0.f;
      constexpr int NSL = NPV > NPAIR + 2 ? NPV : NPAIR + 2;
#pragma unroll
      for (int i = 0; i < NSL; ++i) {
        if (i < NPV) {
          const int cc = i / ND, db = i % ND;
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pp[cc], o[db], 0, 0, 0);
          if (i + PF < NPV) va[i + PF] = vread(Vp, vb, i + PF);
        }
        if (i < NPAIR + 2) soft_slice(s, i, mu, ps, xe, pn);
        __builtin_amdgcn_sched_barrier(0);
      }
      check(s, mu, ps, pn);
    };
    auto pv = [&](const bf16* Vp, const bf16x8 (&pp)[NCC]) {
      unsigned vb = vaddr;
      asm volatile("" : "+v"(vb));
      bf16x8 va[NPV];
#pragma unroll
      for (int j = 0; j < PF; ++j) va[j] = vread(Vp, vb, j);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int cc = i / ND, db = i % ND;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pp[cc], o[db], 0, 0, 0);
        if (i + PF < NPV) va[i + PF] = vread(Vp, vb, i + PF);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Tile j: K(j) sits in K buffer j%2 and V(j) in V buffer j%2. Step j (j >= 1) loads
    // K(j+STGX) and V(j+STGX-1) into registers, forms S(j), runs O += V(j-1) P(j-1) while it
    // turns S(j) into P(j), and stores at its end K(j+1) and V(j), loaded STGX-1 steps earlier.
    // P is double-buffered in registers; the max and row sum of P(j) are applied (rescale,
    // sum) at the start of step j+1, after P(j-1) has entered O. Tile 0 is handled before the
    // loop and the last PV after it, so every step runs the same code and O never changes
    // registers. Tile descriptors (k0, lo, hi) run STGX steps ahead of the compute.
    bf16x8 pp[NCC];  // P^T operands of the pending tile
    float mu = -INFINITY, ps = 0.f;
    auto compute_first = [&](const bf16* Kc, int k0, int lo, int hi) {
      if (wave_active) {
        f32x16 s[SB];
        qk(Kc, s);
        if (lo > k0 || hi < k0 + KT) mask(s, k0, lo, hi);
        soft_exact(s, mu, ps, pp);
      }
    };
    auto compute_step = [&](const bf16* Kc, const bf16* Vp, int k0, int lo, int hi) {
      if (wave_active) {
        rescale(mu);
        l_half += ps;
        f32x16 s[SB];
        qk(Kc, s);
        if (lo > k0 || hi < k0 + KT) mask(s, k0, lo, hi);
        bf16x8 pn[NCC];
        pv_soft(Vp, pp, s, mu, ps, pn);
#pragma unroll
        for (int c = 0; c < NCC; ++c) pp[c] = pn[c];
      }
    };
    auto last_pv = [&](const bf16* Vp) {  // O += V(T-1) P(T-1)
      if (wave_active) {
        rescale(mu);
        l_half += ps;
        pv(Vp, pp);
      }
    };

    if constexpr (TWO) {
      // Both key streams step together (the barriers are shared), each wave tracking both:
      // it stages the tiles of stream ls and computes on those of stream cs. A stream runs
      // T_s tiles; after its last it only re-reads that tile's keys, unused. Split: stream 0
      // takes the first half of the chunk's tiles (rounded up), stream 1 the rest.
      struct Walk {
        TileWalk<KT> ts;
        int T, k0, lo, hi, k1, lo1, hi1, par;
        bool has1;
        __device__ void start(int skip) {  // first tile (after skipping `skip`), and the next
          ts.first();
          if (skip > 0 && T > 0) ts.seek(skip);
          k0 = T > 0 ? ts.k0 : 0;  // (a stream with no tile stages key 0, unused)
          lo = T > 0 ? ts.lo : 0;
          hi = T > 0 ? ts.hi : 0;
          has1 = T > 1 && ts.next();
          k1 = ts.k0;
          lo1 = ts.lo;
          hi1 = ts.hi;
          par = 0;
        }
        __device__ void step(int j) {  // tile j becomes current (while j < T)
          if (j < T) {
            k0 = k1;
            lo = lo1;
            hi = hi1;
            has1 = j + 1 < T && ts.next();
            k1 = ts.k0;
            lo1 = ts.lo;
            hi1 = ts.hi;
            par ^= 1;
          }
        }
      };
      Walk w0, w1;
      w0.ts.runs = runs_s[0];
      w0.ts.nr = nr;
      w1.ts.runs = runs_s[BM == 2 ? NS - 1 : 0];
      w1.ts.nr = BM == 2 ? nr1 : nr;
      int nsteps;
      if (BM == 1) {
        w0.ts.first();
        const int T = w0.ts.count();  // >= 1: every query group keeps a key group
        nsteps = (T + 1) / 2;
        w0.T = nsteps;
        w1.T = T - nsteps;
        w0.start(0);
        w1.start(nsteps);
      } else {
        w0.ts.first();
        w0.T = w0.ts.count();
        w1.ts.first();
        w1.T = w1.ts.count();
        nsteps = max(w0.T, w1.T);
        w0.start(0);
        w1.start(0);
      }
      // (per-wave selections between the two streams' scalars)
      auto L_k0 = [&]() { return ls ? w1.k0 : w0.k0; };
      auto L_next = [&]() { return ls ? (w1.has1 ? w1.k1 : w1.k0) : (w0.has1 ? w0.k1 : w0.k0); };
      auto L_has1 = [&]() { return ls ? w1.has1 : w0.has1; };
      auto L_par = [&]() { return ls ? w1.par : w0.par; };
      auto C_T = [&]() { return cs ? w1.T : w0.T; };
      Stage sa;  // K(j+1), V(j): loaded at the start of step j, stored at its end
      load_k(sa, L_k0());
      store_k(sa, Kb(ls, 0));
      __syncthreads();
      load_k(sa, L_next());
      load_v(sa, L_k0());
      if (C_T() > 0) compute_first(Kb(cs, 0), cs ? w1.k0 : w0.k0, cs ? w1.lo : w0.lo, cs ? w1.hi : w0.hi);
      if (L_has1()) store_k(sa, Kb(ls, 1));
      store_v(sa, Vb(ls, 0));
      for (int j = 1; j < nsteps; ++j) {
        w0.step(j);
        w1.step(j);
        __syncthreads();
        load_k(sa, L_next());
        load_v(sa, L_k0());
        if (j < C_T()) {
          const int cp = cs ? w1.par : w0.par;
          compute_step(Kb(cs, cp), Vb(cs, cp ^ 1), cs ? w1.k0 : w0.k0, cs ? w1.lo : w0.lo, cs ? w1.hi : w0.hi);
        }
        if (L_has1()) store_k(sa, Kb(ls, L_par() ^ 1));
        if (j < (ls ? w1.T : w0.T)) store_v(sa, Vb(ls, L_par()));
      }
      __syncthreads();
      if (C_T() > 0) last_pv(Vb(cs, cs ? w1.par : w0.par));
    } else {
      TileWalk<KT> ts;
      bool has;  // the first tile exists
      if (MODE != 1) {
        ts.runs = runs_s[0];
        ts.nr = nr;
        has = ts.first();
      } else {
        const int clo = a * D.pkc;
        has = ts.first_single(clo, min(D.N, clo + D.pkc));
      }
      int par = 0;  // parity of the current tile
      int k0c = ts.k0, loc = ts.lo, hic = ts.hi;
      if (has) {
        int k01 = 0, lo1 = 0, hi1 = 0, k02 = 0;
        bool has1 = ts.next();
        k01 = ts.k0; lo1 = ts.lo; hi1 = ts.hi;
        bool has2 = STGX == 2 && has1 && ts.next();  // STGX 2 only: the tile after next
        k02 = STGX == 2 ? ts.k0 : 0;
        if (STGX == 2) {
          Stage sa, sb;  // sa: K(j+1), V(j) (stored at the end of step j); sb: K(j+2), V(j+1)
          load_k(sa, k0c);
          store_k(sa, Kb(0, 0));
          load_k(sa, has1 ? k01 : k0c);
          load_v(sa, k0c);
          __syncthreads();
          load_k(sb, has2 ? k02 : k0c);
          load_v(sb, has1 ? k01 : k0c);
          compute_first(Kb(0, 0), k0c, loc, hic);
          if (has1) store_k(sa, Kb(0, 1));
          store_v(sa, Vb(0, 0));
          // step of tile j; `cur` holds K(j+1), V(j) (loaded a step ago), `nxt` receives K(j+2), V(j+1)
          auto step = [&](Stage& cur, Stage& nxt) {
            k0c = k01; loc = lo1; hic = hi1;
            has1 = has2;
            k01 = k02; lo1 = ts.lo; hi1 = ts.hi;
            has2 = has2 && ts.next();
            k02 = ts.k0;
            par ^= 1;
            __syncthreads();
            load_k(nxt, has2 ? k02 : k0c);
            load_v(nxt, has1 ? k01 : k0c);
            compute_step(Kb(0, par), Vb(0, par ^ 1), k0c, loc, hic);
            if (has1) store_k(cur, Kb(0, par ^ 1));
            store_v(cur, Vb(0, par));
          };
          // whole pairs of steps (stages swap roles twice), then at most one more step
          while (has1 && has2) {
            step(sb, sa);
            step(sa, sb);
          }
          if (has1) step(sb, sa);
        } else {
          Stage sa;  // K(j+1), V(j): loaded at the start of step j, stored at its end
          load_k(sa, k0c);
          store_k(sa, Kb(0, 0));
          __syncthreads();
          load_k(sa, has1 ? k01 : k0c);
          load_v(sa, k0c);
          compute_first(Kb(0, 0), k0c, loc, hic);
          if (has1) store_k(sa, Kb(0, 1));
          store_v(sa, Vb(0, 0));
          while (has1) {
            k0c = k01; loc = lo1; hic = hi1;
            has1 = ts.next();
            k01 = ts.k0; lo1 = ts.lo; hi1 = ts.hi;
            par ^= 1;
            __syncthreads();
            load_k(sa, has1 ? k01 : k0c);
            load_v(sa, k0c);
            compute_step(Kb(0, par), Vb(0, par ^ 1), k0c, loc, hic);
            if (has1) store_k(sa, Kb(0, par ^ 1));
            store_v(sa, Vb(0, par));
          }
        }
        // O += V(T-1) P(T-1), V(T-1) in V buffer par
        __syncthreads();
        last_pv(Vb(0, par));
      }
    }

    if constexpr (BM == 1) {
      // stream 1 hands its softmax state (running max, half row sum, unnormalised output)
      // to stream 0 through LDS (the staging buffers are free), lane for lane
      constexpr int NV = 16 * ND + 2;
      float* xs = reinterpret_cast<float*>(smem) + (size_t)sw * NV * kWave + l;
      __syncthreads();  // every wave is past its last operand read
      if (cs == 1) {
#pragma unroll
        for (int i = 0; i < ND; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) xs[(16 * i + v) * kWave] = o[i][v];
        xs[(16 * ND) * kWave] = m_run;
        xs[(16 * ND + 1) * kWave] = l_half;
      }
      __syncthreads();
      if (cs == 1) return;
      const float m1 = xs[(16 * ND) * kWave], l1 = xs[(16 * ND + 1) * kWave];
      const float mm = fmaxf(m_run, m1);  // finite: stream 0 has at least one tile
      const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] = o[i][v] * a0 + xs[(16 * i + v) * kWave] * a1;
      l_half = l_half * a0 + l1 * a1;
      m_run = mm;
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
  };
  if constexpr (CAN_SPLIT) {
    if (kind >= 0) body(std::integral_constant<int, 2>{});
    else if (kind == -2) body(std::integral_constant<int, 1>{});
    else body(std::integral_constant<int, 0>{});
  } else {
    body(std::integral_constant<int, 0>{});
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

template <int DD, int MODE>
static void launch_bsfa(const Dims& D, const Bufs& B, const bf16* q, void* out, float* psp, int nb, hipStream_t s) {
  // 64 keys per step; 8-wave tiles stage two steps ahead, 4-wave tiles (two workgroups per
  // CU, half the registers each) one step ahead
  if (D.attn_w == 8)
    hipLaunchKernelGGL((k_bsfa_bf16<DD, MODE, 8, 64, 2>), dim3(nb), dim3(512), 0, s, q, D, B, out, psp);
  else
    hipLaunchKernelGGL((k_bsfa_bf16<DD, MODE, 4, 64, 1>), dim3(nb), dim3(256), 0, s, q, D, B, out, psp);
}

void launch_attend_sparse(const void* q, const Dims& D, const Bufs& B, void* o_sparse, float* o_psp, hipStream_t s,
                          bool dense) {
  if (D.dtype == 1) {
    const int nb = D.BH * D.max_atiles;
    const bf16* qb = (const bf16*)q;
    if (!dense && D.attn_w == 8) launch_pair_tiles(D, B, s);
    if (D.d == 128) {
      if (dense) launch_bsfa<128, 2>(D, B, qb, o_sparse, o_psp, nb, s);
      else launch_bsfa<128, 0>(D, B, qb, o_sparse, o_psp, nb, s);
    } else {
      if (dense) launch_bsfa<64, 2>(D, B, qb, o_sparse, o_psp, nb, s);
      else launch_bsfa<64, 0>(D, B, qb, o_sparse, o_psp, nb, s);
    }
  } else {
    const int nb = D.BH * D.max_tiles;
    if (D.d == 128)
      hipLaunchKernelGGL((k_bsfa_f32<128, 0>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, o_sparse, o_psp);
    else
      hipLaunchKernelGGL((k_bsfa_f32<64, 0>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, o_sparse, o_psp);
  }
}

void launch_attend_probes(const void* q, const Dims& D, const Bufs& B, float* o_pdn, hipStream_t s) {
  if (D.M == 0 || !o_pdn) return;
  float* none = nullptr;
  if (D.dtype == 1) {
    // probe rows in tiles of the attention tiles' height, each over one key chunk
    const int nbk = D.BH * ((D.M + 32 * D.attn_w - 1) / (32 * D.attn_w)) * D.pch;
    const Dims& Dp = D;
    if (D.d == 128) {
      launch_bsfa<128, 1>(Dp, B, (const bf16*)q, (void*)o_pdn, none, nbk, s);
      hipLaunchKernelGGL((k_probe_combine<128>), dim3(D.M, D.BH), dim3(128), 0, s, D, B, o_pdn);
    } else {
      launch_bsfa<64, 1>(Dp, B, (const bf16*)q, (void*)o_pdn, none, nbk, s);
      hipLaunchKernelGGL((k_probe_combine<64>), dim3(D.M, D.BH), dim3(64), 0, s, D, B, o_pdn);
    }
  } else {
    const int nb = D.BH * ((D.M + kAttnQT - 1) / kAttnQT);
    if (D.d == 128)
      hipLaunchKernelGGL((k_bsfa_f32<128, 1>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, (void*)o_pdn, none);
    else
      hipLaunchKernelGGL((k_bsfa_f32<64, 1>), dim3(nb), dim3(128), 0, s, (const float*)q, D, B, (void*)o_pdn, none);
  }
}

}  // namespace spr
