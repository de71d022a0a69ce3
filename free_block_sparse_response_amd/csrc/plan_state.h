// Device-side plan state of one SparsePR call: sizes and the workspace carve-up.
// Every buffer is per flat head bh (B*H heads) and lives in the caller's workspace.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace spr {

// Lloyd bookkeeping of one head (one k-means run).
struct KmState {
  int done_iter;   // iteration whose assignment is final (INT_MAX while running)
  int iters;       // assignments run
  int c_final;     // groups left after dropping empty ones
  int pad;
  double inertia[2];  // inertia of assignment t in slot t & 1 (the previous one in the other)
};

// Routing facts of one head.
struct RouteInfo {
  long long tau;
  long long budget;
  long long pairs;     // executed pairs including probe rows
  int exceeded;
  int pad;
};

struct Dims {
  int BH, N, d, S, Ck, Cq, M;
  int C;          // max(Ck, Cq): k-means scratch width
  int nblk;       // Lloyd row blocks per head (kKmRows rows each)
  int Npad;       // padded key count of the permuted K / transposed V
  int qt;         // query rows per attention tile
  int max_tiles;  // 128-row tiles per head (group masses), upper bound
  int attn_w;     // waves (32 query rows each) per block-sparse attention tile: 4 or 8
  int max_atiles; // attention tiles of 32 * attn_w rows per head, upper bound
  int pch;        // key chunks of the probe attention (split over keys)
  int pkc;        // keys per probe chunk (multiple of the key tile)
  int dtype;      // 0 f32, 1 bf16
  float scale;
  float log2_scale;  // scale * log2(e)
  double density;
  long long budget;
  int max_iter;
  int warm_iter;  // iteration limit of a warm-started plan
  float tol;
  float lambda;
  int pen_bias;
  int assign_lo;  // Lloyd assignment with the bf16 remainder of the centroid operand
  int partition;  // 0 response-coupled, 1 semantic (raw K and Q), 2 key responses + raw Q
  int correction; // 0 weighted ridge, 1 mean-only, 2 none
  int probe_sel;  // 0 query-group stratified, 1 random, 2 uniform in token order
  int key_rank;   // key response rank r_K (0: full)
  int output_rank;  // residual fit truncated to this many probe-residual directions (0: none)
  uint64_t seed;
};

struct Bufs {
  int* sampled;      // [BH][S]
  float* qs;         // [BH][S][d] gathered sampled queries
  float* metric;     // [BH][d][d] Lloyd metric G
  bf16* metric_h;    // [BH][d][d] G rounded to bf16
  bf16* metric_l;    // [BH][d][d] G minus its bf16 rounding
  float* cent;       // [BH][C][d] Lloyd centroids (row space of X = alpha x)
  float* cent_t;     // [BH][C][d] G m_b
  float* cnorm;      // [BH][C]    m_b G m_b
  bf16* cent_h;      // [BH][C][d] -2 G m_b rounded to bf16 (the assignment's operand)
  bf16* cent_l;      // [BH][C][d] -2 G m_b minus its bf16 rounding, in bf16
  bf16* cent_b;      // [BH][C][16] centroid side of the assignment's bias product (m_b G m_b)
  float* alpha;      // [BH][N]    row scales of the query features
  float* rowconst;   // [BH][N]    alpha^2 x G x
  int* rank;         // [BH][N]    stable rank inside a Lloyd row block
  int* tab;          // [BH][C][nblk] count of group b in sort block j (low 8 bits) and its start in
                     //   the block's group-ordered rows (bits 8+); turned into scatter offsets
  int* lperm;        // [BH][N]    rows of each sort block, ordered by group (stable)
  double* ipart;     // [BH][nblk] inertia partial sums
  int* init_k;       // [BH][Ck] key-group seed rows
  int* init_q;       // [BH][Cq] query-group seed rows
  int* lab;          // [BH][N]    working labels
  int* gstart;       // [BH][C+1]  working group starts
  int* gcount;       // [BH][C]
  KmState* kst;      // [BH] key run
  KmState* qst;      // [BH] query run
  int* klab;         // [BH][N]
  int* kperm;        // [BH][N]
  int* koff;         // [BH][Ck+1]
  float* kcent;      // [BH][Ck][d] key-space centroids of the compacted groups
  bf16* kcent_h;     // [BH][Ck][d] key centroids rounded to bf16
  bf16* kcent_l;     // [BH][Ck][d] key centroids minus their bf16 rounding
  float* qcent;      // [BH][Cq][d] query-group means of alpha q (warm-start representatives)
  int* qlab;         // [BH][N]
  int* qperm;        // [BH][N]
  int* qoff;         // [BH][Cq+1]
  long long* u;      // [BH][Cq][Ck] integer group masses
  int* sorted_b;     // [BH][Cq][Ck]
  long long* cum;    // [BH][Cq][Ck] prefix masses in sorted order
  long long* ccost;  // [BH][Cq][Ck] prefix pair costs in sorted order
  int* jsel;         // [BH][Cq]
  int* row_ptr;      // [BH][Cq+1]
  int* cols;         // [BH][Cq*Ck]
  int2* runs;        // [BH][Cq*Ck] key runs [lo, hi) of merged consecutive selected groups (CSR as cols)
  int* nruns;        // [BH][Cq]
  RouteInfo* rinfo;  // [BH]
  int* pcount;       // [BH][Cq]
  int* poff;         // [BH][Cq+1]
  float* pw_group;   // [BH][Cq]
  int* probes;       // [BH][M]
  float* pweights;   // [BH][M]
  int* pslot;        // [BH][N] probe slot of a token or -1
  void* kp;          // [BH][Npad][d] keys in key-group order
  void* vpt;         // [BH][d][Npad] values in key-group order, transposed
  int2* tiles;       // [BH][max_tiles] (query group, first position), 128-row tiles
  int* ntiles;       // [BH]
  int2* atiles;      // [BH][max_atiles] (query group, first position), attention tiles
  int* antiles;      // [BH]
  int4* ptiles;      // [BH][max_atiles] 8-wave attention items: (group, first position) of stream 0,
                     // then (group, first position) of stream 1, or (-1, 0): one chunk on all
                     // waves, or (-2, 0): one chunk whose keys the two wave halves split
  int* nptiles;      // [BH]
  int* gtiles;       // [BH][Cq] key tiles (kKeyTile keys each) over a query group's key runs
  // 8-wave (bf16) attention layout of the keys: key groups by how many query groups select
  // them (most first, ties by index), so that groups selected together sit together and the
  // runs are fewer and longer; the plan's own key order (kperm, koff) is unchanged
  int* katt_rank;    // [BH][Ck]   position of key group b in that order
  int* katt_start;   // [BH][Ck+1] first key of the group at each position
  int* kperm_att;    // [BH][N]    key rows in that order (the permuted K and V follow it)
  int* tstart;       // [BH][Cq+1] first tile of each query group
  float* mass_part;  // [BH][max_tiles][Ck] per-tile column sums of the group masses
  float* pp_o;       // [BH][M][pch][d] probe attention partial outputs (unnormalised)
  float2* pp_ml;     // [BH][M][pch] probe attention partial (max, sum), log2 domain
  double* gram;      // [BH][d+1][2d+1]  [A | B] of the ridge normal equations
  float* rcov;       // [BH][d][d] weighted second moment R^T W R of the probe residuals
  float* rproj;      // [BH][d][d] projector on its output_rank leading eigenvectors
  bf16* theta_h;     // [BH][d][d] Theta^T (output dim major) rounded to bf16, for the apply
  bf16* theta_l;     // [BH][d][d] Theta^T minus its bf16 rounding
  int* status;       // [BH]
};

constexpr int kKmRows = 128;   // rows per Lloyd assignment block
constexpr int kAttnQT = 128;   // query rows per attention tile (4 waves x 32)
constexpr int kKeyTile = 64;   // keys per attention tile
constexpr int kMassTiles = 2;  // attention tiles per group-mass workgroup (one staged centroid chunk each)

}  // namespace spr
