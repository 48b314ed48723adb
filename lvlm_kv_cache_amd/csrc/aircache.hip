// AirCache visual KV-cache compression pass for MI355X (gfx950).
//
// Kernels (one HIP stream, launched in this order):
//   plan:     elite_select_kernel  -> cross_score_kernel -> finalize_kernel -> topk_select_kernel
//   compress: kv_gather_kernel
//
// Method: paper-notes page "AirCache: Activating Inter-Modal Relevancy KV Cache
// Compression for Efficient Large Vision-Language Model Inference" (ICCV 2025),
// sections "Elite Observation Window", "Layer-wise KV Cache Budget Allocation"
// and the training-free procedure. The readings taken where the page is silent
// are listed in include/aircache.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <type_traits>

#include "aircache.h"
#include "device_common.h"

namespace aircache {

// ----------------------------------------------------------------------------
// Launch-time description of the problem (passed by value to every kernel).
// ----------------------------------------------------------------------------
struct Shape {
  int L, B, Hq, Hkv, G, D, Nv, Nt, S;
  int cap;     // elite tokens per (layer, sample) the workspace holds
  int rcap16;  // G * cap rounded up to 16: row capacity of one (l, b, g) unit
  int T;       // visual keys per scoring tile
  int ntiles;  // scoring tiles per (l, b, g)
  float alpha;
  float scale2;  // log2(e) / sqrt(D): logits are kept in the base-2 domain
  double ratio;
  int budget_mode;  // AIRCACHE_BUDGET_*
  int window;       // 0: the elite window; k > 0: the last k text tokens (k <= N_t); -k: the last k visual tokens
  int nsel;         // selections per (layer, sample): 1, or H_kv (one per KV head)
  int per_head;     // one selection per KV head (I_v^g written to plan.iv_head)
  int lb0;          // first (layer * B + sample) of a one-layer launch (prefill), else 0
  int nstat;        // (max, sum) pairs per row in the scoring statistics: ntiles, +1 on the prefill path
  int qrows, qoff;  // rows per query head in the query buffers and the first text row among them
};

struct PlanPtrs {
  int32_t *elite, *n_elite;
  float *iv;
  double *s_t, *s_k, *bx;
  int32_t *budget;
  int64_t *out_off;
  int32_t *kept, *status;
  float *iv_head;  // [L][B][H_kv][N_v] I_v per KV head when nsel == H_kv
};

struct Ws {
  unsigned *epoch;    // [1]   call counter of the workspace (chunked path records carry it)
  unsigned *cnt_unit; // [L*B*Hkv] finished row tiles per (l, b, g)
  unsigned *cnt_lb;   // [L*B] finished scoring tiles (tiled path) or KV heads (rows path) per (l, b)
  unsigned *cnt_b;    // [B]   finished layers per sample
  unsigned *cnt_all;  // [1]   finished samples
  float2 *stats;      // [units][rcap16][ntiles] (tile max, tile sum) per row, base 2
  float *e;           // [units][Nv][row stride] exp2(logit - tile max) of visual keys
  float *part;        // [units][rt_grid][Nv] column sums of one row tile (row-complete path)
  unsigned *cnt_chunk; // [L*B][chunk_stride] finished row groups per chunk (chunked path), or NULL
  int chunk_stride;
  unsigned *cnt_elite; // [L*B] finished KV heads of the elite stage (reset by the last one)
  float *pbar_part;    // [L*B*Hkv][N_t] KV-head parts of pbar
};

struct LayerTable {
  const void *p[AIRCACHE_MAX_LAYERS];
};
struct LayerTableOut {
  void *p[AIRCACHE_MAX_LAYERS];
};

// ----------------------------------------------------------------------------
// Step 2a: elite cross-modal logits ("Elite Observation Window", the A_vtk
// equation). One workgroup per (layer, sample, KV head, column tile of up to
// 64*KTW visual keys). Rows are the G * N_tk elite queries of the KV head's
// query heads; columns are the tile's visual keys plus every ntiles-th elite
// text key (so each elite text key enters the softmax denominator once).
// MFMA gives S^T (keys x rows); per row the tile max m and sum z of
// exp2(S - m) are written to the workspace, and so is exp2(S - m) for every
// visual key. finalize_kernel merges the tiles' (m, z) into the exact
// row-softmax normaliser.
// ----------------------------------------------------------------------------
template <typename Tag, int D, int KTW>
__global__ __launch_bounds__(256) void cross_score_kernel(Shape sh, LayerTable qt, LayerTable kt, PlanPtrs plan,
                                                          Ws ws) {
  using E = typename Tag::store_t;
  extern __shared__ int el[];  // elite list of this (l, b)
  __shared__ float red_m[4][16], red_z[4][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int t = blockIdx.x % sh.ntiles;
  const int u = blockIdx.x / sh.ntiles;  // ((l * B + b) * Hkv + g)
  const int g = u % sh.Hkv, lb = u / sh.Hkv, l = lb / sh.B, b = lb % sh.B;
  int ntk = plan.n_elite[lb];
  if (ntk > sh.cap) ntk = sh.cap;
  if (ntk < 0) ntk = 0;
  const int R = sh.G * ntk;
  const int RP = (R + 15) & ~15;
  for (int i = tid; i < ntk; i += 256) el[i] = plan.elite[(size_t)lb * sh.Nt + i];
  __syncthreads();

  const E *q = static_cast<const E *>(qt.p[l]);
  const E *kb = static_cast<const E *>(kt.p[l]) + (size_t)(b * sh.Hkv + g) * sh.S * D;
  const int c0 = t * sh.T;
  const int nvis = min(sh.T, sh.Nv - c0);
  // elite text columns of this tile (none for the visual window: its rows
  // normalise over the visual keys only)
  const int nx = (t < ntk && sh.window >= 0) ? (ntk - t + sh.ntiles - 1) / sh.ntiles : 0;

  // This wave's visual key fragments stay in registers for every row tile.
  Frag<Tag> kf[KTW][D / 32];
#pragma unroll
  for (int i = 0; i < KTW; ++i) {
    const int key = (wave + 4 * i) * 16 + n;
    if (key < nvis) {
      const E *krow = kb + (size_t)(c0 + key) * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) kf[i][c].load(krow + c * 32 + grp * 8);
    } else {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) kf[i][c].zero();
    }
  }

  float *e_out = ws.e + (size_t)u * sh.Nv * sh.rcap16;
  float2 *st_out = ws.stats + (size_t)u * sh.rcap16 * sh.nstat;
  for (int rt = 0; rt * 16 < R; ++rt) {
    const int r = rt * 16 + n;
    Frag<Tag> qf[D / 32];
    if (r < R) {
      const int hl = r / ntk, e = r - hl * ntk;
      const E *qrow = q + ((size_t)(b * sh.Hq + g * sh.G + hl) * sh.qrows + (sh.window < 0 ? 0 : sh.qoff) + el[e]) * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qf[c].load(qrow + c * 32 + grp * 8);
    } else {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qf[c].zero();
    }
    // Elite text keys of this tile: online (max, sum) per lane.
    float mx = -INFINITY, zx = 0.f;
    for (int xt = wave; xt * 16 < nx; xt += 4) {
      const int slot = xt * 16 + n;
      Frag<Tag> kx[D / 32];
      if (slot < nx) {
        const E *krow = kb + (size_t)(sh.Nv + el[t + slot * sh.ntiles]) * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kx[c].load(krow + c * 32 + grp * 8);
      } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kx[c].zero();
      }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) mfma_slice(acc, kx[c], qf[c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (xt * 16 + grp * 4 + i < nx) {
          const float v = acc[i] * sh.scale2;
          const float mn = fmaxf(mx, v);
          zx = zx * exp2f(mx - mn) + exp2f(v - mn);
          mx = mn;
        }
      }
    }
    // Visual keys.
    f32x4_t acc[KTW];
    float mv = -INFINITY;
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
      acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) mfma_slice(acc[i], kf[i][c], qf[c]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] *= sh.scale2;
        if ((wave + 4 * i) * 16 + grp * 4 + j < nvis) mv = fmaxf(mv, acc[i][j]);
      }
    }
    float m = fmaxf(mv, mx);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane < 16) red_m[wave][lane] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red_m[0][n], red_m[1][n]), fmaxf(red_m[2][n], red_m[3][n]));
    float zs = (mx > -INFINITY) ? zx * exp2f(mx - m) : 0.f;
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = (wave + 4 * i) * 16 + grp * 4 + j < nvis;
        const float ev = ok ? exp2f(acc[i][j] - m) : 0.f;
        acc[i][j] = ev;
        zs += ev;
      }
    }
    zs += __shfl_xor(zs, 16);
    zs += __shfl_xor(zs, 32);
    if (lane < 16) red_z[wave][lane] = zs;
    __syncthreads();
    zs = red_z[0][n] + red_z[1][n] + red_z[2][n] + red_z[3][n];
    if (r < R && wave == 0 && grp == 0) st_out[(size_t)r * sh.nstat + t] = make_float2(m, zs);
    // rows R .. RP-1 of the last row tile are written as zeros, so that readers
    // can sum whole 16-row groups without masking
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = (wave + 4 * i) * 16 + grp * 4 + j;
        if (key < nvis) e_out[(size_t)(c0 + key) * RP + r] = (r < R) ? acc[i][j] : 0.f;
      }
    }
    __syncthreads();  // red_m / red_z are reused by the next row tile
  }
}

// Budget of every layer of one sample ("Layer-wise KV Cache Budget
// Allocation", the r_hat equation with the cross-layer normalisation reading
// documented in aircache.h). The three sums over layers run in ascending layer
// order on one thread; each layer's value is then formed independently. Plain
// double arithmetic with no fused multiply-add, so the same statistics give
// the same integers anywhere.
struct BudgetSums {
  double st_sum, mshift, u_sum;
};
__device__ __forceinline__ BudgetSums budget_sums(int L, const double *st, const double *sk) {
#pragma clang fp contract(off)
  BudgetSums r{0.0, 0.0, 0.0};
  for (int l = 0; l < L; ++l) r.st_sum += st[l];
  for (int l = 0; l < L; ++l)
    if (sk[l] < r.mshift) r.mshift = sk[l];
  for (int l = 0; l < L; ++l) r.u_sum += sk[l] - r.mshift;
  return r;
}
__device__ __forceinline__ void layer_budget(const Shape &sh, const BudgetSums &r, int l, double st, double sk,
                                             double *x_out, int *b_out) {
#pragma clang fp contract(off)
  const double rr = sh.ratio * (double)sh.Nv;
  const double stn = st * (double)sh.L / r.st_sum;
  const double skn = (r.u_sum > 0.0) ? (sk - r.mshift) * (double)sh.L / r.u_sum : 1.0;
  // the method's rule, or one of its allocation ablation's variants
  const int mode = sh.budget_mode;
  const double x = mode == AIRCACHE_BUDGET_UNIFORM    ? rr
                   : mode == AIRCACHE_BUDGET_STRENGTH ? stn * rr
                   : mode == AIRCACHE_BUDGET_SKEWNESS ? skn * rr
                   : mode == AIRCACHE_BUDGET_PYRAMID  ? rr * (double)(2 * (sh.L - l)) / (double)(sh.L + 1)
                                                      : 0.5 * (stn + skn) * rr;
  double f = floor(x);
  if (!(f > 0.0)) f = 0.0;
  if (f > (double)sh.Nv) f = (double)sh.Nv;
  *x_out = x;
  *b_out = (int)f;
}

// The last workgroup to finish a (layer, sample) runs this with the layer's
// I_v in LDS: strength and skewness ("Layer-wise KV Cache Budget Allocation",
// the s_t and s_k equations) in double precision, then, if it is the last
// layer of its sample to finish, that sample's budgets, and if it is the last
// sample, the compacted layout's offsets. Elections use relaxed device-scope
// counters; published values are written with agent-coherent stores whose
// completion is awaited before the counter moves, and read back with
// agent-coherent loads.
template <int NT>
__device__ void finish_layer_sample(const Shape &sh, const PlanPtrs &plan, const Ws &ws, int lb, const float *ivc) {
  constexpr int NW = NT / 64;
  __shared__ double redd[NW];
  __shared__ double lst[AIRCACHE_MAX_LAYERS], lsk[AIRCACHE_MAX_LAYERS];
  __shared__ BudgetSums sums;
  __shared__ int flag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Nv = sh.Nv, b = lb % sh.B;
  auto block_sum = [&](double v) {
    v = wave_sum_d(v);
    if (lane == 0) redd[wave] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < NW; ++w) t += redd[w];
    __syncthreads();
    return t;
  };
  double s = 0.0;
  for (int c = tid; c < Nv; c += NT) s += (double)ivc[c];
  s = block_sum(s);
  const double mu = s / (double)Nv;
  double v2 = 0.0;
  for (int c = tid; c < Nv; c += NT) {
    const double d = (double)ivc[c] - mu;
    v2 += d * d;
  }
  v2 = block_sum(v2);
  const double sigma = sqrt(v2 / (double)(Nv - 1));
  double k3 = 0.0;
  if (sigma > 0.0) {
    for (int c = tid; c < Nv; c += NT) {
      const double d = ((double)ivc[c] - mu) / sigma;
      k3 += d * d * d;
    }
  }
  k3 = block_sum(k3);
  if (tid == 0) {
    const double skew = (sigma > 0.0) ? k3 * ((double)Nv / ((double)(Nv - 1) * (double)(Nv - 2))) : 0.0;
    store_coherent(&plan.s_t[lb], s);
    store_coherent(&plan.s_k[lb], skew);
    wait_all_memory();
    flag = (counter_add(&ws.cnt_b[b], 1u) == (unsigned)sh.L - 1);
  }
  __syncthreads();
  if (!flag) return;

  // Last layer of sample b: budgets of all its layers.
  const int L = sh.L, B = sh.B;
  {
    const auto rst = coherent_rsrc(plan.s_t, (unsigned)(L * B * sizeof(double)));
    const auto rsk = coherent_rsrc(plan.s_k, (unsigned)(L * B * sizeof(double)));
    for (int l = tid; l < L; l += NT) {
      lst[l] = load_sc1_d(rst, (unsigned)((l * B + b) * sizeof(double)));
      lsk[l] = load_sc1_d(rsk, (unsigned)((l * B + b) * sizeof(double)));
    }
  }
  __syncthreads();
  if (tid == 0) sums = budget_sums(L, lst, lsk);
  __syncthreads();
  for (int l = tid; l < L; l += NT) {
    double x;
    int bud;
    layer_budget(sh, sums, l, lst[l], lsk[l], &x, &bud);
    if (plan.bx) store_coherent(&plan.bx[l * B + b], x);
    store_coherent(&plan.budget[l * B + b], (int32_t)bud);
  }
  wait_all_memory();
  __syncthreads();
  if (tid == 0) flag = (counter_add(ws.cnt_all, 1u) == (unsigned)B - 1);
  __syncthreads();
  if (!flag) return;

  // Last sample: element offsets of every sample's segment in each layer.
  const auto rbud = coherent_rsrc(plan.budget, (unsigned)(L * B * sizeof(int32_t)));
  for (int l = tid; l < L; l += NT) {
    int64_t off = 0;
    for (int bb = 0; bb < B; ++bb) {
      plan.out_off[(size_t)l * (B + 1) + bb] = off;
      off += (int64_t)sh.Hkv * (load_sc1_i(rbud, (unsigned)((l * B + bb) * sizeof(int32_t))) + sh.Nt) * sh.D;
    }
    plan.out_off[(size_t)l * (B + 1) + B] = off;
  }
}

// ----------------------------------------------------------------------------
// Step 2b + 3 + 4: I_v, layer statistics and budgets. One workgroup per
// (layer, sample, column tile). Row normalisers: M = max of the tile maxima,
// Z = sum of z_t * exp2(m_t - M) over tiles in ascending order; column c gets
// sum over KV heads and rows of e * exp2(m_t - M) / Z, divided by H_q * N_tk
// (the I_v equation). The last tile of a (layer, sample) computes s_t and s_k
// (strength and skewness equations) from the full I_v; the last layer of a
// sample computes that sample's budgets; the last sample writes the compacted
// layout's offsets. Finisher election is a relaxed device-scope counter; the
// data it publishes is written with agent-coherent stores whose completion is
// awaited before the counter moves, and read back with agent-coherent loads.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void finalize_kernel(Shape sh, PlanPtrs plan, Ws ws) {
  extern __shared__ float wl[];  // weights [Hkv][rcap16], then I_v cache [Nv] for the finisher
  __shared__ int flag;
  const int tid = threadIdx.x;
  const int t = blockIdx.x % sh.ntiles;
  const int lb = sh.lb0 + blockIdx.x / sh.ntiles, b = lb % sh.B;
  const int lbw = lb - sh.lb0;  // index of (layer, sample) in the scoring workspace
  int ntk = plan.n_elite[lb];
  if (ntk > sh.cap) ntk = sh.cap;
  if (ntk < 0) ntk = 0;
  const int R = sh.G * ntk;
  const int RP = (R + 15) & ~15;
  for (int idx = tid; idx < sh.Hkv * RP; idx += 256) {
    const int g = idx / RP, r = idx - g * RP;
    float wv = 0.f;
    if (r < R) {
      const float2 *st = ws.stats + ((size_t)(lbw * sh.Hkv + g) * sh.rcap16 + r) * sh.nstat;
      // online merge of the tiles' (max, sum) in ascending tile order, eight loads at a time
      float M = -INFINITY, Z = 0.f;
      for (int t0 = 0; t0 < sh.nstat; t0 += 8) {
        float2 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (t0 + j < sh.nstat) ? st[t0 + j] : make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (v[j].x == -INFINITY) continue;
          const float mn = fmaxf(M, v[j].x);
          Z = Z * exp2f(M - mn) + v[j].y * exp2f(v[j].x - mn);
          M = mn;
        }
      }
      wv = exp2f(st[t].x - M) / Z;
    }
    wl[g * RP + r] = wv;
  }
  __syncthreads();
  const float inv_rows = (ntk > 0) ? 1.f / (float)(sh.Hq * ntk) : 0.f;
  const int c0 = t * sh.T, c1 = min(sh.Nv, c0 + sh.T);
  // one selection per KV head: I_v^g over the G query heads of KV head g
  const float inv_grp = (ntk > 0) ? 1.f / (float)(sh.G * ntk) : 0.f;
  for (int c = c0 + tid; c < c1; c += 256) {
    float acc = 0.f;
    for (int g = 0; g < sh.Hkv; ++g) {
      const f32x4_t *e4 =
          reinterpret_cast<const f32x4_t *>(ws.e + (size_t)(lbw * sh.Hkv + g) * sh.Nv * sh.rcap16 + (size_t)c * RP);
      const f32x4_t *w4 = reinterpret_cast<const f32x4_t *>(wl + g * RP);
      float ag = 0.f;
      for (int r0 = 0; r0 < RP / 4; r0 += 4) {  // RP is a multiple of 16
        f32x4_t ev[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ev[j] = e4[r0 + j];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4_t wv = w4[r0 + j];
          ag += ev[j].x * wv.x;
          ag += ev[j].y * wv.y;
          ag += ev[j].z * wv.z;
          ag += ev[j].w * wv.w;
        }
      }
      if (sh.per_head) plan.iv_head[((size_t)lb * sh.Hkv + g) * sh.Nv + c] = ag * inv_grp;
      acc += ag;
    }
    store_coherent(&plan.iv[(size_t)lb * sh.Nv + c], acc * inv_rows);
  }
  wait_all_memory();
  __syncthreads();
  if (tid == 0) flag = (counter_add(&ws.cnt_lb[lb], 1u) == (unsigned)sh.ntiles - 1);
  __syncthreads();
  if (!flag) return;

  float *ivc = wl + sh.Hkv * sh.rcap16;
  const auto riv = coherent_rsrc(plan.iv + (size_t)lb * sh.Nv, (unsigned)(sh.Nv * sizeof(float)));
  for (int c = tid; c < sh.Nv; c += 256) ivc[c] = load_sc1_f(riv, (unsigned)(c * sizeof(float)));
  __syncthreads();
  finish_layer_sample<256>(sh, plan, ws, lb, ivc);
}

// ----------------------------------------------------------------------------
// Steps 2 + 3 + 4 in one launch when a whole row of logits fits in registers
// (N_v <= 8 waves x 16 x KT). A persistent grid of one 8-wave workgroup per
// CU walks the work items (layer-sample, KV head, group of RT row tiles of 16
// elite-query rows) in order; the item count of each (layer, sample) follows
// from its elite count. Per item: the elite queries are the MFMA A operand
// and 16 keys at a time the B operand (each key tile read from LDS once for
// the item's RT row tiles, so K is streamed once per RT tiles); wave w owns visual key tiles w, w + 8, ..., which
// stream through a per-wave LDS ring by DMA and whose logits stay in
// registers; the few elite text keys enter the row max and row sum through an
// online update. Exact row max and sum come from DPP row reductions, then a
// fixed-order sum over the waves. Each wave writes the column sums of
// exp2(S - M) / Z over the item's rows for its key tiles as this item's partial
// I_v; the last item of a (layer, sample) adds the partials in a fixed order
// and runs the statistics and budget finisher.
// ----------------------------------------------------------------------------
constexpr int kRowsThreads = 512;
constexpr int kRowsWaves = kRowsThreads / 64;

// LDS ring depth: up to 4 tiles per wave within 128 KB of LDS.
template <typename Tag, int D> constexpr int rows_ring() {
  return (131072 / (kRowsWaves * 16 * D * Tag::kBytes)) < 4 ? (131072 / (kRowsWaves * 16 * D * Tag::kBytes)) : 4;
}

// Row tiles per item of the rows kernel: 4, 2 or 1, as many as keep one
// lane's query fragments and logits of the item (per row tile: D / 32
// fragments and KT f32x4) within what the kernel has left without spilling
// (found by compiling: 128 registers for four tiles, 112 for two).
template <typename Tag, int D, int KT> constexpr int rows_rt() {
  constexpr int per = (D / 32) * (Tag::kBytes == 4 ? 8 : 4) + 4 * KT;
  return 4 * per <= 128 ? 4 : 2 * per <= 112 ? 2 : 1;
}

template <typename Tag, int D, int KT>
__global__ __launch_bounds__(kRowsThreads) void cross_score_rows_kernel(Shape sh, LayerTable qt, LayerTable kt,
                                                                        PlanPtrs plan, Ws ws, int rt_max) {
  using E = typename Tag::store_t;
  constexpr int NW = kRowsWaves;
  constexpr int RT = rows_rt<Tag, D, KT>();
  constexpr int kTileBytes = 16 * D * Tag::kBytes;  // one 16-key tile
  constexpr int kDma = kTileBytes / 1024;           // 16-byte DMA loads per lane per tile
  constexpr int kRing = rows_ring<Tag, D>();        // tiles in flight per wave
  static_assert(KT >= kRing, "ring deeper than the tile count");
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];  // ring[NW][kRing][tile] | el[cap]
  __shared__ float red[NW][16 * RT];
  __shared__ float rowv[16 * RT];
  __shared__ int flag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int Nv = sh.Nv, LB = sh.L * sh.B;
  unsigned char *ring = dyn + (size_t)wave * kRing * kTileBytes;
  int *el = reinterpret_cast<int *>(dyn + (size_t)NW * kRing * kTileBytes);
  auto elite_count = [&](int x) {
    int t = plan.n_elite[x];
    return t < 0 ? 0 : (t > sh.cap ? sh.cap : t);
  };
  // items of a (layer, sample): KV heads x groups of RT row tiles
  auto item_count = [&](int x) { return sh.Hkv * ((((sh.G * elite_count(x) + 15) >> 4) + RT - 1) / RT); };
  int lb = 0, base = 0, cnt = item_count(0);
  // Pass p covers items [p * grid, (p + 1) * grid); XCD x (blocks x, x + 8, ...
  // under round-robin dispatch) takes a contiguous eighth of each pass, so the
  // row tiles of one (l, b, g), which share K, run together under one L2.
  const int per_xcd = gridDim.x >> 3;
  const int pos = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  for (int item = pos;; item += gridDim.x) {
    while (lb < LB && item >= base + cnt) {
      base += cnt;
      if (++lb < LB) cnt = item_count(lb);
    }
    if (lb >= LB) break;
    const int ngrp = cnt / sh.Hkv;  // row-tile groups of a KV head
    const int local = item - base, g = local / ngrp, rg = local - g * ngrp;
    const int l = lb / sh.B, b = lb % sh.B;
    const int ntk = elite_count(lb);
    const int R = sh.G * ntk;
    __syncthreads();  // the previous item is done with el[] and the ring
    for (int i = tid; i < ntk; i += kRowsThreads) el[i] = plan.elite[(size_t)lb * sh.Nt + i];
    __syncthreads();

    const E *q = static_cast<const E *>(qt.p[l]);
    const E *kb = static_cast<const E *>(kt.p[l]) + (size_t)(b * sh.Hkv + g) * sh.S * D;
    const int nvt = (Nv + 15) >> 4;
    const int nxt = (ntk + 15) >> 4;
    Frag<Tag> qf[RT][D / 32];
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const int r = (rg * RT + j) * 16 + n;
      if (r < R) {
        const int hl = r / ntk, e = r - hl * ntk;
        const E *qrow = q + ((size_t)(b * sh.Hq + g * sh.G + hl) * sh.Nt + el[e]) * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[j][c].load(qrow + c * 32 + grp * 8);
      } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[j][c].zero();
      }
    }
    // Visual key tiles through the LDS ring. Loads are issued for every slot
    // (an empty slot rereads the last visual row and is ignored) so the count
    // of loads in flight is static.
    // Tile sequence of a wave: t = 0 is its elite text tile (text tile w for
    // wave w; an empty one for waves beyond the elite window), t = 1 .. KT its
    // visual tiles w, w + NW, .... Tiles stream through a per-wave LDS ring by
    // DMA; loads are issued for every slot (an empty slot rereads a valid row
    // and is ignored) so the count of loads in flight is static.
    f32x4_t S[RT][KT];
    float mx[RT][4], zx[RT][4];
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mx[j][i] = -INFINITY;
        zx[j][i] = 0.f;
      }
    auto stage = [&](int t) {
      int row;
      if (t == 0) {
        const int e = wave * 16 + n;
        row = (wave < nxt && e < ntk) ? Nv + el[e] : Nv - 1;
      } else {
        row = (wave + NW * (t - 1)) * 16 + n;
        row = row < Nv ? row : Nv - 1;
      }
      // keep the address computation inside its iteration instead of letting
      // all of a wave's tile addresses be precomputed (and spilled)
      asm volatile("" : "+v"(row));
      const unsigned char *src = reinterpret_cast<const unsigned char *>(kb + (size_t)row * D);
      unsigned char *slot = ring + (t % kRing) * kTileBytes;
      if (t >= kRing) wait_lds_reads();  // the slot's previous tile has been read
#pragma unroll
      for (int j = 0; j < kDma; ++j) load_lds16(src + 16 * grp + 64 * j, slot + 1024 * j);
    };
#pragma unroll
    for (int t = 0; t < kRing; ++t) stage(t);
#pragma unroll
    for (int t = 0; t <= KT; ++t) {
      // tile t has landed once only the loads of the tiles staged after it remain
      wait_tiles<kDma>(min(kRing - 1, KT - t));
      f32x4_t acc[RT];
#pragma unroll
      for (int j = 0; j < RT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const unsigned char *slot = ring + (t % kRing) * kTileBytes;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        Frag<Tag> kf;
        LdsTile<Tag>::read(kf, slot, c, lane);
#pragma unroll
        for (int j = 0; j < RT; ++j) mfma_slice(acc[j], qf[j][c], kf);
      }
      if (t + kRing <= KT) stage(t + kRing);
      if (t == 0) {
        if (wave < nxt && wave * 16 + n < ntk) {
#pragma unroll
          for (int j = 0; j < RT; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              mx[j][i] = acc[j][i] * sh.scale2;
              zx[j][i] = 1.f;
            }
        }
      } else {
        const bool ok = (wave + NW * (t - 1)) * 16 + n < Nv;
#pragma unroll
        for (int j = 0; j < RT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[j][t - 1][i] = ok ? acc[j][i] * sh.scale2 : -INFINITY;
      }
    }
    // Elite text tiles beyond one per wave (elite windows over 16 x NW tokens).
    for (int xt = wave + NW; xt < nxt; xt += NW) {
      const int e = xt * 16 + n;
      Frag<Tag> kf[D / 32];
      if (e < ntk) {
        const E *kr = kb + (size_t)(Nv + el[e]) * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kf[c].load(kr + c * 32 + grp * 8);
      } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kf[c].zero();
      }
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) mfma_slice(acc, qf[j][c], kf[c]);
        if (e < ntk) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = acc[i] * sh.scale2;
            const float mn = fmaxf(mx[j][i], v);
            zx[j][i] = zx[j][i] * exp2f(mx[j][i] - mn) + exp2f(v - mn);
            mx[j][i] = mn;
          }
        }
      }
    }
    // lane holds rows grp*4+i of row tile j and key n: reduce over keys (DPP
    // rows), then waves
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      float mr[4] = {mx[j][0], mx[j][1], mx[j][2], mx[j][3]};
#pragma unroll
      for (int k = 0; k < KT; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mr[i] = fmaxf(mr[i], S[j][k][i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) mr[i] = row16_max(mr[i]);
      if (n == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][j * 16 + grp * 4 + i] = mr[i];
      }
    }
    __syncthreads();
    if (tid < 16 * RT) {
      float m = red[0][tid];
      for (int w = 1; w < NW; ++w) m = fmaxf(m, red[w][tid]);
      rowv[tid] = m;
    }
    __syncthreads();
    float zr[RT][4];
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float M = rowv[j * 16 + grp * 4 + i];
        zr[j][i] = (mx[j][i] > -INFINITY) ? zx[j][i] * exp2f(mx[j][i] - M) : 0.f;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          const float ev = exp2f(S[j][k][i] - M);
          S[j][k][i] = ev;
          zr[j][i] += ev;
        }
        zr[j][i] = row16_sum(zr[j][i]);
      }
    __syncthreads();  // every lane has read rowv
    if (n == 0) {
#pragma unroll
      for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][j * 16 + grp * 4 + i] = zr[j][i];
    }
    __syncthreads();
    if (tid < 16 * RT) {
      float z = 0.f;
      for (int w = 0; w < NW; ++w) z += red[w][tid];
      rowv[tid] = (rg * RT * 16 + tid < R) ? 1.f / z : 0.f;
    }
    __syncthreads();
    float W[RT][4];
#pragma unroll
    for (int j = 0; j < RT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) W[j][i] = rowv[j * 16 + grp * 4 + i];
    float *part = ws.part + ((size_t)(lb * sh.Hkv + g) * rt_max + rg) * Nv;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int ti = wave + NW * k;
      if (ti < nvt) {  // wave-uniform
        // the item's row tiles in order, each its four rows in order
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < RT; ++j)
          a += S[j][k][0] * W[j][0] + S[j][k][1] * W[j][1] + S[j][k][2] * W[j][2] + S[j][k][3] * W[j][3];
        const float cs = sum_across_rows(a);
        const int c = ti * 16 + n;
        if (grp == 0 && c < Nv) store_coherent(&part[c], cs);
      }
    }
    wait_all_memory();
    __syncthreads();
    const int u = lb * sh.Hkv + g;
    float *unit_part = ws.part + (size_t)u * rt_max * Nv;  // group 0's slot holds the unit's sum
    if (ngrp > 1) {
      // last row-tile group of (l, b, g): add the unit's group partials in order
      if (tid == 0) flag = (counter_add(&ws.cnt_unit[u], 1u) == (unsigned)ngrp - 1);
      __syncthreads();
      if (!flag) continue;
      const auto rp = coherent_rsrc(unit_part, (unsigned)((size_t)ngrp * Nv * sizeof(float)));
      for (int c = tid; c < Nv; c += kRowsThreads) {
        float v[8];
        float a = 0.f;
        for (int t0 = 0; t0 < ngrp; t0 += 8) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = load_sc1_f(rp, (unsigned)(((t0 + j) * Nv + c) * sizeof(float)));
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (t0 + j < ngrp) a += v[j];
        }
        store_coherent(&unit_part[c], a);
      }
      wait_all_memory();
      __syncthreads();
    }
    if (tid == 0) flag = (counter_add(&ws.cnt_lb[lb], 1u) == (unsigned)sh.Hkv - 1);
    __syncthreads();
    if (!flag) continue;

    // Last KV head of (l, b): I_v = sum of the heads' sums (ascending) divided
    // by H_q * N_tk; the ring area holds it for the finisher.
    float *ivc = reinterpret_cast<float *>(dyn);
    const float inv_rows = (ntk > 0) ? 1.f / (float)(sh.Hq * ntk) : 0.f;
    const size_t head_stride = (size_t)rt_max * Nv;
    const auto rl = coherent_rsrc(ws.part + (size_t)lb * sh.Hkv * head_stride,
                                  (unsigned)((size_t)sh.Hkv * head_stride * sizeof(float)));
    for (int c = tid; c < Nv; c += kRowsThreads) {
      float v[8];
      float a = 0.f;
      for (int g0 = 0; g0 < sh.Hkv; g0 += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = load_sc1_f(rl, (unsigned)(((g0 + j) * head_stride + c) * sizeof(float)));
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (g0 + j < sh.Hkv) a += v[j];
      }
      a *= inv_rows;
      ivc[c] = a;
      plan.iv[(size_t)lb * Nv + c] = a;
    }
    __syncthreads();
    finish_layer_sample<kRowsThreads>(sh, plan, ws, lb, ivc);
  }
}

#include "pass_chunked.h"
#include "small.h"
#include "decode.h"
#include "prefill.h"

// ----------------------------------------------------------------------------
// Step 1: elite observation window ("Elite Observation Window", the Att and k
// equations). One workgroup of 4 waves per (layer, sample, KV head): the
// logits of the last text query of the head's G query heads over the N_t text
// keys come from MFMA (16 text keys as the A operand, up to 16 query heads as
// the B operand) into LDS; each wave normalises whole rows (max, sum of exp2),
// and the rows are summed in ascending head order into the KV head's part of
// pbar. The last KV head of a (layer, sample) to finish (a counter election)
// adds the parts in ascending KV-head order into pbar and keeps
// { j : pbar_j >= alpha max pbar }, compacted in ascending j by a block scan.
// The election counter resets itself: the last arriver zeroes it for the next
// call. (The chunked path computes the elite sets inside its own launch.)
// ----------------------------------------------------------------------------
constexpr int kEliteThreads = 512;
constexpr int kEliteWaves = kEliteThreads / 64;

template <typename Tag, int D>
__global__ __launch_bounds__(kEliteThreads) void elite_select_kernel(Shape sh, LayerTable qt, LayerTable kt,
                                                                     PlanPtrs plan, Ws ws) {
  using E = typename Tag::store_t;
  extern __shared__ float lds[];  // z[G][Nt]; the last KV head: pbar[Nt]
  __shared__ float red[kEliteWaves];
  __shared__ int wtot[kEliteWaves];
  __shared__ int flag;
  const int lb = sh.lb0 + (int)blockIdx.x / sh.Hkv, g = (int)blockIdx.x % sh.Hkv;
  const int l = lb / sh.B, b = lb % sh.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int Nt = sh.Nt, G = sh.G;
  float *z = lds;

  // This kernel opens every plan: reset the counters of the later kernels.
  if (g == 0) {
    for (int u = tid; u < sh.Hkv; u += kEliteThreads) ws.cnt_unit[(size_t)lb * sh.Hkv + u] = 0;
    if (ws.cnt_chunk)
      for (int c = tid; c < ws.chunk_stride; c += kEliteThreads) ws.cnt_chunk[(size_t)lb * ws.chunk_stride + c] = 0;
    if (tid == 0) {
      ws.cnt_lb[lb] = 0;
      if (l == 0) ws.cnt_b[b] = 0;
      if (lb == 0) {
        *ws.cnt_all = 0;
        *plan.status = 0;
        *ws.epoch = *ws.epoch + 1u;
      }
    }
  }

  const E *q = static_cast<const E *>(qt.p[l]);
  const E *k = static_cast<const E *>(kt.p[l]);
  const int nkt = (Nt + 15) >> 4;
  const int nht = (G + 15) >> 4;
  const int items = nht * nkt;
  // Items (head tile, key tile) in batches of 4 per wave: all fragments of a
  // batch are loaded before its MFMAs so the loads overlap.
  constexpr int kBatch = 4;
  for (int it0 = wave; it0 < items; it0 += kEliteWaves * kBatch) {
    Frag<Tag> qf[kBatch][D / 32], kf[kBatch][D / 32];
#pragma unroll
    for (int bi = 0; bi < kBatch; ++bi) {
      const int it = it0 + bi * kEliteWaves;
      const int kt_ = it % nkt, ht = it / nkt;
      const int h0 = ht * 16;
      const int nh = min(16, G - h0);
      const int key = kt_ * 16 + n;
      if (it < items && n < nh) {
        const E *qrow = q + ((size_t)(b * sh.Hq + g * G + h0 + n) * sh.qrows + sh.qoff + (Nt - 1)) * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[bi][c].load(qrow + c * 32 + grp * 8);
      } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[bi][c].zero();
      }
      if (it < items && key < Nt) {
        const E *krow = k + ((size_t)(b * sh.Hkv + g) * sh.S + sh.Nv + key) * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kf[bi][c].load(krow + c * 32 + grp * 8);
      } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kf[bi][c].zero();
      }
    }
#pragma unroll
    for (int bi = 0; bi < kBatch; ++bi) {
      const int it = it0 + bi * kEliteWaves;
      if (it >= items) break;  // wave-uniform
      const int kt_ = it % nkt, ht = it / nkt;
      const int h0 = ht * 16;
      const int nh = min(16, G - h0);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) mfma_slice(acc, kf[bi][c], qf[bi][c]);
      if (n < nh) {
        float *zr = z + (size_t)(h0 + n) * Nt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kt_ * 16 + grp * 4 + i;
          if (kk < Nt) zr[kk] = acc[i] * sh.scale2;
        }
      }
    }
  }
  __syncthreads();
  for (int h = wave; h < G; h += kEliteWaves) {
    float *zr = z + (size_t)h * Nt;
    float m = -INFINITY;
    for (int j = lane; j < Nt; j += 64) m = fmaxf(m, zr[j]);
    m = wave_max(m);
    float s = 0.f;
    for (int j = lane; j < Nt; j += 64) {
      const float ev = exp2f(zr[j] - m);
      zr[j] = ev;
      s += ev;
    }
    s = wave_sum(s);
    const float inv = 1.f / s;
    for (int j = lane; j < Nt; j += 64) zr[j] *= inv;
  }
  __syncthreads();
  // this KV head's part of pbar, heads in ascending order
  float *part = ws.pbar_part + (size_t)(lb * sh.Hkv + g) * Nt;
  for (int j = tid; j < Nt; j += kEliteThreads) {
    float a = 0.f;
    for (int h = 0; h < G; ++h) a += z[(size_t)h * Nt + j];
    store_coherent(&part[j], a);
  }
  wait_all_memory();
  __syncthreads();
  if (tid == 0) {
    const bool last = counter_add(&ws.cnt_elite[lb], 1u) == (unsigned)sh.Hkv - 1u;
    if (last) store_coherent(&ws.cnt_elite[lb], 0u);
    flag = last;
  }
  __syncthreads();
  if (!flag) return;

  // Last KV head of (l, b): pbar = sum of the parts in ascending KV-head order.
  float *pbar = lds;
  const auto rp = coherent_rsrc(ws.pbar_part + (size_t)lb * sh.Hkv * Nt, (unsigned)((size_t)sh.Hkv * Nt * sizeof(float)));
  float m = -INFINITY;
  for (int j = tid; j < Nt; j += kEliteThreads) {
    float a = 0.f;
    for (int gg = 0; gg < sh.Hkv; ++gg) a += load_sc1_f(rp, (unsigned)(((size_t)gg * Nt + j) * sizeof(float)));
    pbar[j] = a;
    m = fmaxf(m, a);
  }
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < kEliteWaves; ++w) m = fmaxf(m, red[w]);
  const float thr = sh.alpha * m;
  // the elite set, or the contiguous window of the last sh.window text tokens
  auto keep = [&](int j) { return sh.window > 0 ? j >= Nt - sh.window : pbar[j] >= thr; };
  const int per = (Nt + kEliteThreads - 1) / kEliteThreads;
  const int j0 = min(Nt, tid * per), j1 = min(Nt, j0 + per);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += keep(j) ? 1 : 0;
  const int incl = wave_incl_scan(cnt);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kEliteWaves; ++w) {
    if (w < wave) base += wtot[w];
    total += wtot[w];
  }
  int pos = base + incl - cnt;
  int32_t *el = plan.elite + (size_t)lb * Nt;
  if (sh.window < 0) {
    // the visual window: its rows are the last k visual positions
    const int kw = -sh.window;
    for (int e = tid; e < kw; e += kEliteThreads) el[e] = sh.Nv - kw + e;
    if (tid == 0) plan.n_elite[lb] = kw;
    return;
  }
  for (int j = j0; j < j1; ++j)
    if (keep(j)) el[pos++] = j;
  if (tid == 0) plan.n_elite[lb] = total;
}

// Block-wide exclusive scan for 1024 threads; returns the exclusive prefix and
// writes the total to *total.
__device__ __forceinline__ int block_excl_scan_1024(int v, int *wtot, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    const int x = wtot[w];
    if (w < wave) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// ----------------------------------------------------------------------------
// Step 5: top-r_hat selection per (layer, sample). I_v >= 0, so the raw
// float32 bits order like the values. MSB-first radix select finds the key T
// of the r_hat-th largest score: the bits above the highest bit in which the
// minimum and maximum keys differ are common to all keys and skipped; each
// pass histograms the next (up to) 8 bits of the keys that match the prefix
// found so far, in per-wave LDS histograms merged in a fixed order. Kept:
// every key > T, plus the lowest-index keys equal to T up to r_hat in total,
// written in ascending index order by block scans. Each thread holds a
// contiguous run of indices.
// ----------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkPer = 8;  // N_v <= 8192

__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(Shape sh, PlanPtrs plan) {
  __shared__ unsigned hist[kTopkWaves][256];
  __shared__ unsigned tot[256];
  __shared__ int wtot[kTopkWaves];
  __shared__ unsigned wmin[kTopkWaves], wmax[kTopkWaves];
  __shared__ unsigned sel_digit, sel_above;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // one workgroup per (layer, sample), or per (layer, sample, KV head) with
  // one selection per KV head (scores I_v^g, the same budget)
  const int lb = blockIdx.x / sh.nsel, gsel = blockIdx.x - lb * sh.nsel;
  const int Nv = sh.Nv;
  if (tid == 0 && gsel == 0 && plan.n_elite[lb] > sh.cap) atomicOr(plan.status, AIRCACHE_DEV_ELITE_OVERFLOW);
  const int kbud = plan.budget[lb];
  int32_t *kept = plan.kept + (size_t)blockIdx.x * Nv;
  const float *scores = sh.per_head ? plan.iv_head + (size_t)blockIdx.x * Nv : plan.iv + (size_t)lb * Nv;
  const int per = (Nv + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(Nv, tid * per), i1 = min(Nv, i0 + per);
  if (kbud <= 0) return;
  if (kbud >= Nv) {
    for (int i = tid; i < Nv; i += kTopkThreads) kept[i] = i;
    return;
  }
  unsigned key[kTopkPer];
  unsigned kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p) {
    const int i = i0 + p;
    key[p] = (i < i1) ? __float_as_uint(scores[i]) : 0u;
    if (i < i1) {
      kmin = min(kmin, key[p]);
      kmax = max(kmax, key[p]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (unsigned)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (unsigned)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    wmin[wave] = kmin;
    wmax[wave] = kmax;
  }
  __syncthreads();
  kmin = wmin[0];
  kmax = wmax[0];
  for (int w = 1; w < kTopkWaves; ++w) {
    kmin = min(kmin, wmin[w]);
    kmax = max(kmax, wmax[w]);
  }
  const unsigned diff = kmin ^ kmax;
  int hb = diff ? 31 - __clz((int)diff) : -1;  // highest bit in which keys can differ
  unsigned mask = (hb < 0) ? 0xffffffffu : (hb >= 31) ? 0u : ~((2u << hb) - 1u);
  unsigned prefix = kmin & mask;
  int need = kbud;  // keys still to take among those matching prefix
  while (hb >= 0) {
    const int width = min(8, hb + 1);
    const int shift = hb + 1 - width;
    const unsigned dmask = (1u << width) - 1u;
    for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kTopkPer; ++p)
      if (i0 + p < i1 && (key[p] & mask) == prefix) atomicAdd(&hist[wave][(key[p] >> shift) & dmask], 1u);
    __syncthreads();
    if (tid < 256) {
      unsigned c = 0;
      for (int w = 0; w < kTopkWaves; ++w) c += hist[w][tid];
      tot[tid] = c;
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns digits 255-4*lane .. 252-4*lane (descending)
      unsigned c[4], s4 = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = tot[255 - 4 * lane - q];
        s4 += c[q];
      }
      const int incl = wave_incl_scan((int)s4);
      unsigned above = (unsigned)(incl - (int)s4);  // keys with a larger digit
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < (unsigned)need && above + c[q] >= (unsigned)need) {
          sel_digit = 255u - 4u * lane - q;
          sel_above = above;
        }
        above += c[q];
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= dmask << shift;
    need -= (int)sel_above;
    hb -= width;
    __syncthreads();
  }
  const unsigned T = prefix;
  int neq = 0;
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p) neq += (i0 + p < i1 && key[p] == T) ? 1 : 0;
  int total;
  int eq_rank = block_excl_scan_1024(neq, wtot, &total);
  int nkeep = 0;
  unsigned keepbits = 0;
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p) {
    if (i0 + p < i1) {
      bool kp = key[p] > T;
      if (key[p] == T) {
        kp = eq_rank < need;
        ++eq_rank;
      }
      if (kp) {
        keepbits |= 1u << p;
        ++nkeep;
      }
    }
  }
  int pos = block_excl_scan_1024(nkeep, wtot, &total);
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p)
    if (keepbits & (1u << p)) kept[pos++] = i0 + p;
}

// ----------------------------------------------------------------------------
// Step 6: compaction ("training-free procedure", the compress step). One
// workgroup per (layer, sample, KV head, chunk of output rows); row p of the
// segment is visual row kept[p] for p < r_hat, else text row p - r_hat.
// 16-byte lanes, RB/16 lanes per row, non-temporal stores.
// ----------------------------------------------------------------------------
struct GatherTables {
  LayerTable k, v;
  LayerTableOut ko, vo;
};

template <int RB>
__global__ __launch_bounds__(256) void kv_gather_kernel(Shape sh, GatherTables tb, PlanPtrs plan, int nch, int esize,
                                                        int64_t cap_elems) {
  constexpr int LPR = RB / 16;
  constexpr int RPI = 256 / LPR;
  const int tid = threadIdx.x;
  const int ch = blockIdx.x % nch;
  const int u = blockIdx.x / nch;
  const int g = u % sh.Hkv, lb = u / sh.Hkv, l = lb / sh.B, b = lb % sh.B;
  const int bud = plan.budget[lb];
  if (bud < 0 || bud > sh.Nv) return;  // not a budget written by aircache_plan
  const int nrows = bud + sh.Nt;
  const int64_t seg0 = plan.out_off[(size_t)l * (sh.B + 1) + b];
  if (seg0 < 0 || seg0 > cap_elems - (int64_t)sh.Hkv * nrows * sh.D) return;  // (no wrap for stray offsets)
  const int rpc = (nrows + nch - 1) / nch;
  const int r0 = ch * rpc, r1 = min(nrows, r0 + rpc);
  const size_t src_base = (size_t)(b * sh.Hkv + g) * sh.S * RB;
  const size_t dst_base = (size_t)seg0 * esize + (size_t)g * nrows * RB;
  const char *ks = static_cast<const char *>(tb.k.p[l]) + src_base;
  const char *vs = static_cast<const char *>(tb.v.p[l]) + src_base;
  char *kd = static_cast<char *>(tb.ko.p[l]) + dst_base;
  char *vd = static_cast<char *>(tb.vo.p[l]) + dst_base;
  const int32_t *kept = plan.kept + ((size_t)lb * sh.nsel + (sh.nsel > 1 ? g : 0)) * sh.Nv;
  const int sub = tid % LPR;
  for (int p = r0 + tid / LPR; p < r1; p += RPI) {
    const int srow = (p < bud) ? kept[p] : sh.Nv + (p - bud);
    if ((unsigned)srow >= (unsigned)sh.S) continue;
    const u32x4_t kv = reinterpret_cast<const u32x4_t *>(ks + (size_t)srow * RB)[sub];
    const u32x4_t vv = reinterpret_cast<const u32x4_t *>(vs + (size_t)srow * RB)[sub];
    store_nt(reinterpret_cast<u32x4_t *>(kd + (size_t)p * RB) + sub, kv);
    store_nt(reinterpret_cast<u32x4_t *>(vd + (size_t)p * RB) + sub, vv);
  }
}

// ----------------------------------------------------------------------------
// int8 quantisation of the compacted cache (the UniCache blog, section 6.3:
// compress first, then quantise, one scale per head). One workgroup per
// (layer, sample, KV head, K or V) segment of the compacted layout: the
// segment's largest absolute value, s = max / 127, then codes
// rint(x / s) clamped to [-127, 127], both divisions correctly rounded in
// float32. 16 elements per piece, four pieces per thread in flight, one
// 16-byte store of codes per piece; the second read mostly hits L2.
// ----------------------------------------------------------------------------
struct QuantTables {
  LayerTable ko, vo;
  LayerTableOut kq, vq;
};

template <typename Tag>
__device__ __forceinline__ void load16_as_f32(const typename Tag::store_t *p, float (&x)[16]);
template <> __device__ __forceinline__ void load16_as_f32<F32Tag>(const float *p, float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4_t v = reinterpret_cast<const f32x4_t *>(p)[j];
    x[4 * j] = v.x;
    x[4 * j + 1] = v.y;
    x[4 * j + 2] = v.z;
    x[4 * j + 3] = v.w;
  }
}
template <> __device__ __forceinline__ void load16_as_f32<Bf16Tag>(const uint16_t *p, float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4_t v = reinterpret_cast<const u32x4_t *>(p)[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * j + 2 * e] = __uint_as_float(v[e] << 16);
      x[8 * j + 2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
}

constexpr int kQuantThreads = 512;
constexpr int kQuantUnroll = 4;  // 16-element pieces per thread in flight
// bfloat16 pieces per thread kept in registers between the passes, taken when
// a segment's expected pieces fit them and the segments fit one round of the
// grid (the registers leave one workgroup per CU; measured: workload 3, 224
// segments of 3328 pieces, 16.9 -> 14.1 us; workloads 4 and 5, 896 and 1792
// segments, 3% and 8% slower with them, so they keep R = 0)
constexpr int kQuantKeep = 16;
inline bool quant_keep(const Shape &s) {
  const long long pieces = ((long long)(s.ratio * (double)s.Nv) + s.Nt) * s.D / 16;
  const long long segs = 2LL * s.L * s.B * s.Hkv;
  return pieces <= (long long)kQuantKeep * kQuantThreads && segs <= (long long)kTargetCus;
}

template <typename Tag, int R>
__global__ __launch_bounds__(kQuantThreads) void quantize_i8_kernel(Shape sh, QuantTables tb, PlanPtrs plan,
                                                                    float *k_scale, float *v_scale, int64_t cap_elems) {
  using E = typename Tag::store_t;
  constexpr int U = kQuantUnroll;
  __shared__ float wmax[kQuantThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kv = blockIdx.x & 1, u = blockIdx.x >> 1;
  const int g = u % sh.Hkv, lb = u / sh.Hkv, l = lb / sh.B, b = lb - (lb / sh.B) * sh.B;
  const int bud = plan.budget[lb];
  if (bud < 0 || bud > sh.Nv) return;  // not a budget written by aircache_plan
  const int n = bud + sh.Nt;
  const int64_t seg0 = plan.out_off[(size_t)l * (sh.B + 1) + b];
  if (seg0 < 0 || seg0 > cap_elems - (int64_t)sh.Hkv * n * sh.D) return;  // (no wrap for stray offsets)
  const size_t base = (size_t)seg0 + (size_t)g * n * sh.D;
  const int cnt16 = n * sh.D / 16;  // at least 4 (D >= 64, n >= 1)
  const E *src = static_cast<const E *>(kv ? tb.vo.p[l] : tb.ko.p[l]) + base;
  int8_t *dst = static_cast<int8_t *>(kv ? tb.vq.p[l] : tb.kq.p[l]) + base;
  // Pieces [0, kept) (piece tid + j NT in slot j, R slots) stay in registers
  // between the two passes, so only the rest of a long segment is read twice.
  constexpr int NT = kQuantThreads;
  static_assert(R == 0 || Tag::kBytes == 2, "pieces are kept in registers for bfloat16 only");
  const int kept = min(cnt16, R * NT);
  u32x4_t raw[R > 0 ? R : 1][2];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j * NT < kept) {  // uniform; lanes past the end reload the last kept piece
      const u32x4_t *q = reinterpret_cast<const u32x4_t *>(src + 16 * (size_t)min(tid + j * NT, kept - 1));
      raw[j][0] = q[0];
      raw[j][1] = q[1];
    }
  }
  auto widen_raw = [&](int j, float (&x)[16]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * h + 2 * e] = __uint_as_float(raw[j][h][e] << 16);
        x[8 * h + 2 * e + 1] = __uint_as_float(raw[j][h][e] & 0xffff0000u);
      }
  };
  // the largest |x|: the kept pieces, then the rest with U pieces per thread
  // in flight, indices past the end clamped to the last piece (no branch
  // around a load)
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j * NT < kept) {
      float x[16];
      widen_raw(j, x);
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[e]));
    }
  }
  for (int p0 = kept + tid; p0 < cnt16; p0 += NT * U) {
    float x[U][16];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = p0 + j * NT;
      load16_as_f32<Tag>(src + 16 * (size_t)(p < cnt16 ? p : cnt16 - 1), x[j]);
    }
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[j][e]));
  }
  m = wave_max(m);
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  m = wmax[0];
  for (int w = 1; w < kQuantThreads / 64; ++w) m = fmaxf(m, wmax[w]);
  const float sc = __fdiv_rn(m, 127.0f);
  if (tid == 0) (kv ? v_scale : k_scale)[(size_t)lb * sh.Hkv + g] = sc;
  // rint(x / sc) with x / sc correctly rounded, from t = x * (1 / sc): t is
  // within 2 ulp of that quotient (each rounding 0.5 ulp, 1 / sc and the
  // product), and an ulp is at most 2^-16 for |t| < 256, so when t is farther
  // than 2^-14 from every half-integer both round to the same integer; the
  // rest (and a non-finite t) take the exact division
  const float rc = sc > 0.f ? __fdiv_rn(1.0f, sc) : 0.f;
  // the 16 codes of piece p
  auto emit = [&](const float (&x)[16], int p) {
    u32x4_t out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      unsigned word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = x[4 * w + e] * rc;
        float q = rintf(t);
        if (!(fabsf(fabsf(t - q) - 0.5f) > 0x1p-14f)) q = sc > 0.f ? rintf(__fdiv_rn(x[4 * w + e], sc)) : 0.f;
        q = fminf(fmaxf(q, -127.f), 127.f);
        word |= ((unsigned)(int)q & 0xffu) << (8 * e);
      }
      out[w] = word;
    }
    store_nt(reinterpret_cast<u32x4_t *>(dst + 16 * (size_t)p), out);
  };
  // the codes: the kept pieces from registers, the rest read again (a lane
  // past the end writes the last piece's codes again)
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j * NT < kept && tid + j * NT < kept) {
      float x[16];
      widen_raw(j, x);
      emit(x, tid + j * NT);
    }
  }
  for (int p0 = kept + tid; p0 < cnt16; p0 += NT * U) {
    float x[U][16];
    int pj[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = p0 + j * NT;
      pj[j] = p < cnt16 ? p : cnt16 - 1;
      load16_as_f32<Tag>(src + 16 * (size_t)pj[j], x[j]);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) emit(x[j], pj[j]);
  }
}

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
constexpr size_t kMaxLds = 160 * 1024;

struct Config {
  Shape sh;
  size_t off_cnt, off_stats, off_e, off_part, ws_bytes;
  size_t tile_bytes;   // bytes of one 16-key tile
  bool run_fused;      // aircache_run compacts inside the chunked launch
  size_t off_cnt_elite, off_pbar, off_sched;
  size_t elite_lds, score_lds, final_lds, rows_lds;
  int ktw;
  int rows_kt;  // key tiles per wave of cross_score_rows_kernel; 0: the tiled path with spilled exponentials
  int rt_grid, units;
  bool chunked;        // aircache_pass_kernel: the whole pass in one launch
  bool small;          // aircache_small_kernel: the whole pass in one workgroup
  SmallLds slds;
  int path;            // AIRCACHE_PATH_TILED, _ROWS, _CHUNKED or _SMALL
  // chunked path: schedule facts fixed by the shape, workspace offsets, LDS
  int hgs, nhg, wph, rows, mnch, kcap_lo, nmw;
  size_t off_pass_head, off_parts, off_ecnt, off_emask, off_xrec, off_mom, off_ivrec, off_brec;
  PassLds plds;
};

// Workspace head: the epoch word, then the counters.
constexpr size_t kEpochBytes = 256;

// Register budgets of cross_score_rows_kernel instantiations (key tiles per wave).
constexpr int kRowsKt[] = {4, 5, 8, 16, 24};
constexpr int kRowsKtMax = 24;

int make_config(const aircache_desc *d, Config *cfg) {
  g_last_error.clear();
  if (!d) return fail(AIRCACHE_EINVAL, "desc is NULL");
  if (d->n_layers < 1 || d->n_layers > AIRCACHE_MAX_LAYERS)
    return fail(AIRCACHE_EINVAL, "n_layers=%d outside [1, %d]", d->n_layers, AIRCACHE_MAX_LAYERS);
  if (d->batch < 1) return fail(AIRCACHE_EINVAL, "batch=%d < 1", d->batch);
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
    return fail(AIRCACHE_EINVAL, "n_q_heads=%d must be a positive multiple of n_kv_heads=%d", d->n_q_heads,
                d->n_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128) return fail(AIRCACHE_EINVAL, "head_dim=%d not 64 or 128", d->head_dim);
  if (d->n_vis < 3) return fail(AIRCACHE_EINVAL, "n_vis=%d < 3 (skewness needs three values)", d->n_vis);
  if (d->n_vis > kTopkThreads * kTopkPer) return fail(AIRCACHE_EINVAL, "n_vis=%d > %d", d->n_vis, kTopkThreads * kTopkPer);
  if (d->n_txt < 1) return fail(AIRCACHE_EINVAL, "n_txt=%d < 1", d->n_txt);
  if (d->dtype != AIRCACHE_F32 && d->dtype != AIRCACHE_BF16) return fail(AIRCACHE_EINVAL, "dtype=%d unknown", d->dtype);
  if (!(d->alpha >= 0.0 && d->alpha <= 1.0)) return fail(AIRCACHE_EINVAL, "alpha=%g outside [0, 1]", d->alpha);
  if (!(d->ratio >= 0.0 && d->ratio <= 1.0)) return fail(AIRCACHE_EINVAL, "ratio=%g outside [0, 1]", d->ratio);
  if (d->max_elite < 0 || d->max_elite > d->n_txt)
    return fail(AIRCACHE_EINVAL, "max_elite=%d outside [0, n_txt=%d]", d->max_elite, d->n_txt);
  if (d->path < AIRCACHE_PATH_AUTO || d->path > AIRCACHE_PATH_SMALL)
    return fail(AIRCACHE_EINVAL, "path=%d unknown", d->path);
  if (d->budget_mode < AIRCACHE_BUDGET_AIRCACHE || d->budget_mode > AIRCACHE_BUDGET_PYRAMID)
    return fail(AIRCACHE_EINVAL, "budget_mode=%d unknown", d->budget_mode);
  const bool vis_window = d->obs_window < 0;  // the last -obs_window visual tokens
  if (vis_window && (-(long long)d->obs_window > d->n_vis || -(long long)d->obs_window > d->n_txt))
    return fail(AIRCACHE_EINVAL, "a visual window of %lld tokens needs at most min(n_vis, n_txt) = %d",
                -(long long)d->obs_window, d->n_vis < d->n_txt ? d->n_vis : d->n_txt);
  if (vis_window && d->path != AIRCACHE_PATH_AUTO && d->path != AIRCACHE_PATH_TILED)
    return fail(AIRCACHE_EINVAL, "the visual window is served by the tiled path");
  if (d->select_mode != AIRCACHE_SELECT_SHARED && d->select_mode != AIRCACHE_SELECT_PER_KV_HEAD)
    return fail(AIRCACHE_EINVAL, "select_mode=%d unknown", d->select_mode);
  const bool per_head = d->select_mode == AIRCACHE_SELECT_PER_KV_HEAD;
  if (per_head && (d->path == AIRCACHE_PATH_ROWS || d->path == AIRCACHE_PATH_CHUNKED))
    return fail(AIRCACHE_EINVAL, "one selection per KV head is served by the tiled and small paths");
  Shape &s = cfg->sh;
  s.L = d->n_layers;
  s.B = d->batch;
  s.Hq = d->n_q_heads;
  s.Hkv = d->n_kv_heads;
  s.G = s.Hq / s.Hkv;
  s.D = d->head_dim;
  s.Nv = d->n_vis;
  s.Nt = d->n_txt;
  s.S = s.Nv + s.Nt;
  s.cap = vis_window ? -d->obs_window : (d->max_elite ? d->max_elite : d->n_txt);
  const long long rows = (long long)s.G * s.cap;
  s.rcap16 = (int)((rows + 15) / 16 * 16);
  cfg->ktw = (d->dtype == AIRCACHE_BF16) ? 4 : 2;
  const int tmax = 64 * cfg->ktw;
  int nt = (s.Nv + tmax - 1) / tmax;
  int T = (s.Nv + nt - 1) / nt;
  T = (T + 15) / 16 * 16;
  s.T = T;
  s.ntiles = (s.Nv + T - 1) / T;
  s.alpha = (float)d->alpha;
  s.scale2 = (float)(1.4426950408889634 / sqrt((double)s.D));
  s.ratio = d->ratio;
  s.budget_mode = d->budget_mode;
  s.window = d->obs_window < d->n_txt ? d->obs_window : d->n_txt;  // negative: the visual window
  s.nsel = per_head ? s.Hkv : 1;
  s.per_head = per_head ? 1 : 0;
  s.lb0 = 0;
  s.nstat = s.ntiles;
  // the visual window reads every position's queries ([S] rows per head), the
  // last text query among them at row N_v + N_t - 1
  s.qrows = vis_window ? s.S : s.Nt;
  s.qoff = vis_window ? s.Nv : 0;
  const int esz = d->dtype == AIRCACHE_BF16 ? 2 : 4;
  (void)esz;
  cfg->elite_lds = (size_t)(s.G > 1 ? s.G : 1) * s.Nt * sizeof(float);
  cfg->score_lds = (size_t)s.cap * sizeof(int);
  cfg->final_lds = ((size_t)s.Hkv * s.rcap16 + s.Nv) * sizeof(float);
  if (cfg->elite_lds > kMaxLds)
    return fail(AIRCACHE_EINVAL, "(n_q_heads / n_kv_heads) * n_txt = %lld too large for the elite stage (max %zu)",
                (long long)s.G * s.Nt, kMaxLds / sizeof(float));
  if (cfg->score_lds > kMaxLds || cfg->final_lds > kMaxLds)
    return fail(AIRCACHE_EINVAL, "n_q_heads * max_elite too large (%lld rows); lower max_elite",
                (long long)s.Hq * s.cap);
  const size_t units = (size_t)s.L * s.B * s.Hkv;
  const size_t n_cnt = (size_t)s.L * s.B * s.Hkv + (size_t)s.L * s.B + s.B + 1;
  cfg->units = (int)units;
  // Row-complete scoring when the visual keys plus the largest elite window
  // fit in the registers of one 8-wave workgroup.
  const int tiles_needed = (s.Nv + 15) / 16;
  cfg->rows_kt = 0;
  for (int kt : kRowsKt)
    if (kRowsWaves * kt >= tiles_needed) {
      cfg->rows_kt = kt;
      break;
    }
  const long long rt_need = ((long long)s.G * s.cap + 15) / 16;
  cfg->rt_grid = (int)(rt_need < 1 ? 1 : rt_need);  // row tiles of a unit at most
  const size_t tile_bytes = (size_t)16 * s.D * (d->dtype == AIRCACHE_BF16 ? 2 : 4);
  cfg->tile_bytes = tile_bytes;
  size_t ring = 131072 / (kRowsWaves * tile_bytes);
  if (ring > 4) ring = 4;
  cfg->rows_lds = (size_t)kRowsWaves * ring * tile_bytes + (size_t)s.cap * sizeof(int);
  if ((size_t)s.Nv * sizeof(float) > (size_t)kRowsWaves * ring * tile_bytes) cfg->rows_kt = 0;  // finisher's I_v
  if (cfg->rows_kt && cfg->rows_lds > kMaxLds) cfg->rows_kt = 0;
  if (d->path == AIRCACHE_PATH_ROWS && !cfg->rows_kt)
    return fail(AIRCACHE_EINVAL, "the rows path needs n_vis <= %d", kRowsWaves * 16 * kRowsKtMax);
  // Chunked path: a head group is the largest power of two up to eight that
  // divides H_kv (a wave group per KV head); the records are sized for the
  // most chunks a pair can have (the elite cap, the smallest key-tile cap);
  // the passes of an item stay within the record tags, the elite window
  // within the elite parts' limits, and the LDS layout within a CU.
  cfg->chunked = false;
  {
    const int esize = d->dtype == AIRCACHE_BF16 ? 2 : 4;
    const int rtpm = pass_rtp(s.D, esize);
    int hgs = 1;
    while (hgs < 8 && s.Hkv % (hgs * 2) == 0) hgs *= 2;
    cfg->hgs = hgs;
    cfg->nhg = s.Hkv / hgs;
    cfg->wph = kPassWaves / hgs;
    cfg->rows = rtpm * 16;
    cfg->nmw = 2 * pass_words64(s.Nt);
    cfg->kcap_lo = pass_kcap_min(s.L, s.B, s.Nv, cfg->wph);
    cfg->mnch = item_plan(s.cap, s.G, s.Nv, cfg->wph, cfg->kcap_lo, s.D, esize).nch;
    const long long LB = (long long)s.L * s.B;
    const bool lb_ok = LB <= 2048;
    cfg->plds = pass_lds_layout(s.D, esize, hgs, lb_ok ? (int)LB : 0, s.Nt, s.Nv);
    const long long rtg_max = ((long long)s.G * s.cap + 15) / 16;
    const long long npass_max = (long long)cfg->nhg * ((rtg_max + rtpm - 1) / rtpm);
    const bool lds_ok = (size_t)cfg->plds.total + 4096 <= kMaxLds &&
                        (long long)(s.G > 1 ? s.G : 1) * s.Nt * 4 <= cfg->plds.z_bytes &&
                        (long long)cfg->plds.sts + pass_sts_bytes(s.L, cfg->mnch) <= (long long)kRingBytes;
    const bool ok = lb_ok && lds_ok && npass_max < kPassMaxPass && s.Nt <= 2 * kPassThreads;
    cfg->chunked = ok;
  }
  if (d->path == AIRCACHE_PATH_CHUNKED && !cfg->chunked)
    return fail(AIRCACHE_EINVAL, "the chunked path needs n_txt <= 1024, n_layers * batch <= 2048 and an elite cap, "
                "n_vis and layer count whose records and statistics fit its LDS");
  // Small path: one sample's keys and text queries of every layer, with the
  // per-wave buffers, within the one workgroup's LDS; AUTO takes it first.
  // Waves with layer work: up to eight, fewer when their buffers do not fit.
  {
    const int esize = d->dtype == AIRCACHE_BF16 ? 2 : 4;
    cfg->small = false;
    if (s.Nv <= kSmallMaxNv && (long long)s.Hq * s.Nt <= kSmallMaxZ && s.L <= kSmallMaxLayers &&
        5 * s.L <= kPassTableSlots)
      for (int w = s.L < kSmallWaves ? s.L : kSmallWaves; w >= 1 && !cfg->small; --w) {
        cfg->slds = small_lds_layout(s.L, s.Hq, s.Hkv, s.D, s.Nv, s.Nt, esize, w, s.nsel);
        cfg->small = (size_t)cfg->slds.total + 1024 <= kMaxLds;
      }
  }
  if (d->path == AIRCACHE_PATH_SMALL && !cfg->small)
    return fail(AIRCACHE_EINVAL, "the small path needs one sample's keys and text queries of every layer in LDS, "
                "n_vis <= %d, n_q_heads * n_txt <= %d and n_layers <= %d", kSmallMaxNv, kSmallMaxZ,
                kSmallMaxLayers);
  if (d->path != AIRCACHE_PATH_AUTO && d->path != AIRCACHE_PATH_SMALL) cfg->small = false;
  if (per_head) cfg->chunked = false, cfg->rows_kt = 0;
  if (vis_window) cfg->chunked = false, cfg->rows_kt = 0, cfg->small = false;
  if (d->path == AIRCACHE_PATH_TILED || d->path == AIRCACHE_PATH_ROWS) cfg->chunked = false;
  if (d->path == AIRCACHE_PATH_TILED || d->path == AIRCACHE_PATH_CHUNKED) cfg->rows_kt = 0;
  if (cfg->small) cfg->chunked = false, cfg->rows_kt = 0;
  cfg->path = cfg->small ? AIRCACHE_PATH_SMALL
              : cfg->chunked ? AIRCACHE_PATH_CHUNKED
              : cfg->rows_kt ? AIRCACHE_PATH_ROWS
                             : AIRCACHE_PATH_TILED;
  // aircache_run compacts inside the chunked launch when the five pointer
  // tables fit its table
  cfg->run_fused = (cfg->chunked || cfg->small) && 5 * s.L <= kPassTableSlots;
  cfg->off_cnt = kEpochBytes;
  cfg->off_cnt_elite = cfg->off_cnt + align_up(n_cnt * sizeof(unsigned));
  cfg->off_pbar = cfg->off_cnt_elite + align_up((size_t)s.L * s.B * sizeof(unsigned));
  cfg->off_sched = cfg->off_pbar + align_up((size_t)s.L * s.B * s.Hkv * s.Nt * sizeof(float));
  cfg->off_stats = cfg->off_sched;
  if (cfg->small) {
    // one workgroup keeps everything in LDS: no workspace beyond the head
    cfg->ws_bytes = kEpochBytes;
    cfg->off_e = cfg->off_part = cfg->off_stats = 0;
  } else if (cfg->chunked) {
    // head at offset 0: the call count (epoch), exit counter, flags, wrap
    // counter; then the records (the other paths' counters are not used)
    const size_t lbs = (size_t)s.L * s.B;
    cfg->off_pass_head = 0;
    cfg->off_parts = cfg->off_pass_head + kEpochBytes;
    cfg->off_ecnt = cfg->off_parts + align_up(lbs * (size_t)s.Hkv * s.Nt * sizeof(uint64_t));
    cfg->off_emask = cfg->off_ecnt + align_up(lbs * sizeof(uint64_t));
    cfg->off_xrec = cfg->off_emask + align_up(lbs * (size_t)cfg->nmw * sizeof(uint64_t));
    cfg->off_mom = cfg->off_xrec + align_up(lbs * 2 * (size_t)cfg->mnch * cfg->hgs * cfg->rows * 16);
    cfg->off_ivrec = cfg->off_mom + align_up(lbs * (size_t)cfg->mnch * 64);
    cfg->off_brec = cfg->off_ivrec + align_up(lbs * (size_t)s.Nv * sizeof(uint64_t));
    cfg->ws_bytes = cfg->off_brec + align_up(lbs * sizeof(uint64_t));
    cfg->off_e = cfg->off_part = cfg->off_stats;
  } else if (cfg->rows_kt) {
    cfg->off_e = cfg->off_stats;
    cfg->off_part = cfg->off_stats;
    cfg->ws_bytes = cfg->off_part + align_up(units * cfg->rt_grid * (size_t)s.Nv * sizeof(float));
  } else {
    cfg->off_e = cfg->off_stats + align_up(units * s.rcap16 * s.ntiles * sizeof(float2));
    cfg->off_part = cfg->off_e;
    cfg->ws_bytes = cfg->off_e + align_up(units * s.Nv * (size_t)s.rcap16 * sizeof(float));
  }
  return AIRCACHE_OK;
}

Ws ws_of(const Config &cfg, void *base) {
  char *p = static_cast<char *>(base);
  const Shape &s = cfg.sh;
  Ws w;
  w.epoch = reinterpret_cast<unsigned *>(p);
  w.cnt_unit = reinterpret_cast<unsigned *>(p + cfg.off_cnt);
  w.cnt_lb = w.cnt_unit + (size_t)s.L * s.B * s.Hkv;
  w.cnt_b = w.cnt_lb + (size_t)s.L * s.B;
  w.cnt_all = w.cnt_b + s.B;
  w.stats = reinterpret_cast<float2 *>(p + cfg.off_stats);
  w.e = reinterpret_cast<float *>(p + cfg.off_e);
  w.part = reinterpret_cast<float *>(p + cfg.off_part);
  w.cnt_chunk = nullptr;
  w.cnt_elite = reinterpret_cast<unsigned *>(p + cfg.off_cnt_elite);
  w.pbar_part = reinterpret_cast<float *>(p + cfg.off_pbar);
  w.chunk_stride = 0;
  return w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_hip(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(AIRCACHE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return AIRCACHE_OK;
}

// Per-device facts about a kernel that host code asks for on every call
// (dynamic LDS already allowed, resident workgroups per CU), kept so that a
// call costs no runtime query after the first one.
struct KernelFacts {
  int dev;
  const void *kern;
  size_t lds_allowed;
  size_t occ_lds;
  int occ;
};
std::mutex g_facts_mu;
constexpr int kMaxFacts = 512;  // (device, kernel) pairs: far more than the kernels times the devices
KernelFacts g_facts[kMaxFacts];
int g_nfacts = 0;

// The facts entry of (dev, kern), created on first use; NULL if the table is
// full (the caller then queries the runtime every time). g_facts_mu held.
KernelFacts *kernel_facts(int dev, const void *kern) {
  for (int i = 0; i < g_nfacts; ++i)
    if (g_facts[i].dev == dev && g_facts[i].kern == kern) return &g_facts[i];
  if (g_nfacts == kMaxFacts) return nullptr;
  g_facts[g_nfacts] = KernelFacts{dev, kern, 0, 0, 0};
  return &g_facts[g_nfacts++];
}

template <typename K> int allow_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return AIRCACHE_OK;
  int dev = 0, rc;
  if ((rc = check_hip(hipGetDevice(&dev), "hipGetDevice"))) return rc;
  const void *kp = reinterpret_cast<const void *>(kernel);
  std::lock_guard<std::mutex> lock(g_facts_mu);
  KernelFacts *f = kernel_facts(dev, kp);
  if (f && f->lds_allowed >= bytes) return AIRCACHE_OK;
  if ((rc = check_hip(hipFuncSetAttribute(kp, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes),
                      "hipFuncSetAttribute")))
    return rc;
  if (f) f->lds_allowed = bytes;
  return AIRCACHE_OK;
}

// Resident workgroups per CU of a kernel at this block size and dynamic LDS.
template <typename K> int occupancy(K kernel, int threads, size_t lds, int *occ) {
  int dev = 0, rc;
  if ((rc = check_hip(hipGetDevice(&dev), "hipGetDevice"))) return rc;
  const void *kp = reinterpret_cast<const void *>(kernel);
  std::lock_guard<std::mutex> lock(g_facts_mu);
  KernelFacts *f = kernel_facts(dev, kp);
  if (f && f->occ > 0 && f->occ_lds == lds) {
    *occ = f->occ;
    return AIRCACHE_OK;
  }
  int v = 0;
  if ((rc = check_hip(hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kp, threads, lds),
                      "hipOccupancyMaxActiveBlocksPerMultiprocessor")))
    return rc;
  if (f) {
    f->occ = v;
    f->occ_lds = lds;
  }
  *occ = v;
  return AIRCACHE_OK;
}

// Optional instrumentation: when ev is non-NULL, ev[i] is recorded on the
// stream right before the i-th kernel and ev[n] after the last one.
int mark(hipEvent_t *ev, int i, hipStream_t st) {
  if (!ev) return AIRCACHE_OK;
  return check_hip(hipEventRecord(ev[i], st), "hipEventRecord");
}

// Compute units of the current device (cached per device).
int device_cus(int *cus) {
  static int cache[64] = {0};
  int dev = 0;
  int rc;
  if ((rc = check_hip(hipGetDevice(&dev), "hipGetDevice"))) return rc;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *cus = cache[dev];
    return AIRCACHE_OK;
  }
  int v = 0;
  if ((rc = check_hip(hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev), "hipDeviceGetAttribute")))
    return rc;
  if (v < 1) v = 1;
  if (dev >= 0 && dev < 64) cache[dev] = v;
  *cus = v;
  return AIRCACHE_OK;
}

template <typename Tag, int D, int KT>
int launch_rows(const Config &cfg, const LayerTable &qt, const LayerTable &kt, const PlanPtrs &pp, const Ws &ws,
                hipStream_t st) {
  const Shape &s = cfg.sh;
  int rc;
  if ((rc = allow_lds(cross_score_rows_kernel<Tag, D, KT>, cfg.rows_lds))) return rc;
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  // persistent: one workgroup per CU (LDS use admits one), never more than the items
  long long items = (long long)cfg.units * cfg.rt_grid;
  long long g8 = (items + 7) / 8 * 8;  // a multiple of 8 (item to XCD mapping)
  const unsigned grid = (unsigned)(g8 < cus ? g8 : (cus / 8) * 8);
  hipLaunchKernelGGL((cross_score_rows_kernel<Tag, D, KT>), dim3(grid), dim3(kRowsThreads), cfg.rows_lds, st, s, qt,
                     kt, pp, ws, cfg.rt_grid);
  return check_hip(hipGetLastError(), "cross_score_rows_kernel launch");
}

// Workgroups of aircache_pass_kernel: as many as are resident at once (one
// per CU: the LDS use admits no second).
template <typename Tag, int D> int pass_grid(const Config &cfg, int *grid) {
  auto kern = aircache_pass_kernel<Tag, D>;
  const size_t lds = (size_t)cfg.plds.total;
  int rc;
  if ((rc = allow_lds(kern, lds))) return rc;
  int cus = 0;
  if ((rc = device_cus(&cus))) return rc;
  int occ = 0;
  if ((rc = occupancy(kern, kPassThreads, lds, &occ))) return rc;
  if (occ < 1) return fail(AIRCACHE_EINVAL, "the chunked kernel does not fit a compute unit");
  *grid = cus * occ;
  return AIRCACHE_OK;
}

// Compaction operands of a chunked launch that also compacts (NULL: plan only).
struct RunOut {
  const LayerTable *v;
  const LayerTable *ko, *vo;
};

// The host's part of a chunked launch on `grid` workgroups: elite parts per
// (layer, sample) and elite workgroups; the chunks of a pair must fit the grid
// at the widest chunks (the kernel schedules the rest).
int pass_schedule(const Config &cfg, int grid, PassWs *pw) {
  const Shape &s = cfg.sh;
  const long long LB = (long long)s.L * s.B;
  const int esize = (int)(cfg.tile_bytes / (16 * s.D));
  const int widest = item_plan(s.cap, s.G, s.Nv, cfg.wph, kKtwMax, s.D, esize).nch;
  if (widest > grid) return fail(AIRCACHE_EINVAL, "%d chunks per (layer, sample) exceed %d workgroups", widest, grid);
  // parts per (layer, sample): the most KV-head groups (a power of two up to
  // eight dividing H_kv) with every part on a workgroup of its own
  int npp = 1;
  while (npp < s.Hkv && npp < 8 && s.Hkv % (npp * 2) == 0 && LB * npp * 2 <= grid) npp *= 2;
  pw->npp = npp;
  pw->EW = (int)(LB * npp < grid ? LB * npp : grid);
  return AIRCACHE_OK;
}

template <typename Tag, int D>
int launch_chunked(const Config &cfg, const LayerTable &qt, const LayerTable &kt, const PlanPtrs &pp,
                   void *ws_base, int grid, hipStream_t st, const RunOut *out) {
  const Shape &s = cfg.sh;
  auto kern = aircache_pass_kernel<Tag, D>;
  const size_t lds = (size_t)cfg.plds.total;
  char *p = static_cast<char *>(ws_base);
  PassWs pw;
  int rc;
  if ((rc = pass_schedule(cfg, grid, &pw))) return rc;
  unsigned *head = reinterpret_cast<unsigned *>(p + cfg.off_pass_head);
  pw.epoch = head;
  pw.exitc = head + 1;
  pw.flags = reinterpret_cast<int *>(head + 2);
  pw.wrapc = head + 3;
  pw.recs = reinterpret_cast<u32x4_t *>(p + cfg.off_parts);
  pw.rec_words = (cfg.ws_bytes - cfg.off_parts) / 16;
  pw.parts = reinterpret_cast<uint64_t *>(p + cfg.off_parts);
  pw.ecnt = reinterpret_cast<uint64_t *>(p + cfg.off_ecnt);
  pw.emask = reinterpret_cast<uint64_t *>(p + cfg.off_emask);
  pw.xrec = reinterpret_cast<uint64_t *>(p + cfg.off_xrec);
  pw.mom = reinterpret_cast<uint64_t *>(p + cfg.off_mom);
  pw.ivrec = reinterpret_cast<uint64_t *>(p + cfg.off_ivrec);
  pw.brec = reinterpret_cast<uint64_t *>(p + cfg.off_brec);
  pw.nmw = cfg.nmw;
  pw.hgs = cfg.hgs;
  pw.nhg = cfg.nhg;
  pw.wph = cfg.wph;
  pw.rows = cfg.rows;
  pw.mnch = cfg.mnch;
  pw.kcap_lo = cfg.kcap_lo;
  pw.gather = out ? 1 : 0;
  pw.units = (int)((long long)s.L * s.B * (out ? s.Hkv * 2 : 1));
  pw.esize = (int)(cfg.tile_bytes / (16 * s.D));
  pw.cap_elems = (int64_t)s.B * s.Hkv * (int64_t)s.S * s.D;
  PassTables tab;
  memset(&tab, 0, sizeof(tab));
  for (int l = 0; l < s.L; ++l) {
    tab.p[l] = qt.p[l];
    tab.p[s.L + l] = kt.p[l];
    if (out) {
      tab.p[2 * s.L + l] = out->v->p[l];
      tab.p[3 * s.L + l] = out->ko->p[l];
      tab.p[4 * s.L + l] = out->vo->p[l];
    }
  }
  // every workgroup resident at once, which the waits between workgroups
  // need; if other work holds CUs, the bounded waits report
  // AIRCACHE_DEV_TIMEOUT instead of hanging
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kPassThreads), lds, st, s, tab, pp, pw, cfg.plds);
  return check_hip(hipGetLastError(), "aircache_pass_kernel launch");
}

// The small path: one workgroup, the tables of aircache_pass_kernel (values
// and compacted outputs only when out is given).
template <typename Tag, int D>
int launch_small(const Config &cfg, const LayerTable &qt, const LayerTable &kt, const PlanPtrs &pp, hipStream_t st,
                 const RunOut *out) {
  const Shape &s = cfg.sh;
  auto kern = aircache_small_kernel<Tag, D>;
  const size_t lds = (size_t)cfg.slds.total;
  int rc;
  if ((rc = allow_lds(kern, lds))) return rc;
  PassTables tab;
  memset(&tab, 0, sizeof(tab));
  for (int l = 0; l < s.L; ++l) {
    tab.p[l] = qt.p[l];
    tab.p[s.L + l] = kt.p[l];
    if (out) {
      tab.p[2 * s.L + l] = out->v->p[l];
      tab.p[3 * s.L + l] = out->ko->p[l];
      tab.p[4 * s.L + l] = out->vo->p[l];
    }
  }
  const int64_t cap = (int64_t)s.B * s.Hkv * (int64_t)s.S * s.D;
  hipLaunchKernelGGL(kern, dim3(1), dim3(kSmallThreads), lds, st, s, tab, pp, out ? 1 : 0, cap, cfg.slds);
  return check_hip(hipGetLastError(), "aircache_small_kernel launch");
}

template <typename Tag, int D, int KTW>
int launch_plan(const Config &cfg, const LayerTable &qt, const LayerTable &kt, const PlanPtrs &pp, const Ws &ws,
                void *ws_base, hipStream_t st, hipEvent_t *ev) {
  const Shape &s = cfg.sh;
  int rc;
  const unsigned nlb = (unsigned)(s.L * s.B);
  if (cfg.small) {
    // the whole plan in one workgroup (the profiled call's other intervals are empty)
    if ((rc = mark(ev, 0, st))) return rc;
    if ((rc = mark(ev, 1, st))) return rc;
    if ((rc = launch_small<Tag, D>(cfg, qt, kt, pp, st, nullptr))) return rc;
    if ((rc = mark(ev, 2, st))) return rc;
    if ((rc = mark(ev, 3, st))) return rc;
    return mark(ev, 4, st);
  }
  if (cfg.chunked) {
    // elite sets, scoring, statistics, budgets and top-k in one launch (the
    // elite interval of the profiled call is empty)
    int fgrid = 0;
    if ((rc = pass_grid<Tag, D>(cfg, &fgrid))) return rc;
    if ((rc = mark(ev, 0, st))) return rc;
    if ((rc = mark(ev, 1, st))) return rc;
    if ((rc = launch_chunked<Tag, D>(cfg, qt, kt, pp, ws_base, fgrid, st, nullptr))) return rc;
    if ((rc = mark(ev, 2, st))) return rc;
    if ((rc = mark(ev, 3, st))) return rc;
    return mark(ev, 4, st);
  }
  if ((rc = allow_lds(elite_select_kernel<Tag, D>, cfg.elite_lds))) return rc;
  if ((rc = mark(ev, 0, st))) return rc;
  hipLaunchKernelGGL((elite_select_kernel<Tag, D>), dim3(nlb * s.Hkv), dim3(kEliteThreads), cfg.elite_lds, st, s, qt,
                     kt, pp, ws);
  if ((rc = check_hip(hipGetLastError(), "elite_select_kernel launch"))) return rc;
  if ((rc = mark(ev, 1, st))) return rc;
  if (cfg.rows_kt) {
    // scoring, statistics and budgets in one launch; the finalize stage is empty
    if (cfg.rows_kt == 4) rc = launch_rows<Tag, D, 4>(cfg, qt, kt, pp, ws, st);
    else if (cfg.rows_kt == 5) rc = launch_rows<Tag, D, 5>(cfg, qt, kt, pp, ws, st);
    else if (cfg.rows_kt == 8) rc = launch_rows<Tag, D, 8>(cfg, qt, kt, pp, ws, st);
    else if (cfg.rows_kt == 16) rc = launch_rows<Tag, D, 16>(cfg, qt, kt, pp, ws, st);
    else rc = launch_rows<Tag, D, 24>(cfg, qt, kt, pp, ws, st);
    if (rc) return rc;
    if ((rc = mark(ev, 2, st))) return rc;
  } else {
    if ((rc = allow_lds(cross_score_kernel<Tag, D, KTW>, cfg.score_lds))) return rc;
    if ((rc = allow_lds(finalize_kernel, cfg.final_lds))) return rc;
    hipLaunchKernelGGL((cross_score_kernel<Tag, D, KTW>), dim3(nlb * s.Hkv * s.ntiles), dim3(256), cfg.score_lds,
                       st, s, qt, kt, pp, ws);
    if ((rc = check_hip(hipGetLastError(), "cross_score_kernel launch"))) return rc;
    if ((rc = mark(ev, 2, st))) return rc;
    hipLaunchKernelGGL(finalize_kernel, dim3(nlb * s.ntiles), dim3(256), cfg.final_lds, st, s, pp, ws);
    if ((rc = check_hip(hipGetLastError(), "finalize_kernel launch"))) return rc;
  }
  if ((rc = mark(ev, 3, st))) return rc;
  hipLaunchKernelGGL(topk_select_kernel, dim3(nlb * (unsigned)s.nsel), dim3(kTopkThreads), 0, st, s, pp);
  if ((rc = check_hip(hipGetLastError(), "topk_select_kernel launch"))) return rc;
  return mark(ev, 4, st);
}

PlanPtrs plan_ptrs(const aircache_plan_buf *p) {
  PlanPtrs q;
  q.elite = p->elite_idx;
  q.n_elite = p->n_elite;
  q.iv = p->iv;
  q.s_t = p->s_t;
  q.s_k = p->s_k;
  q.bx = p->budget_x;
  q.budget = p->budget;
  q.out_off = p->out_off;
  q.kept = p->kept_idx;
  q.status = p->status;
  q.iv_head = p->iv_head;
  return q;
}

int check_plan_buf(const aircache_plan_buf *p, bool for_compress, const Config &cfg) {
  if (!p) return fail(AIRCACHE_EINVAL, "plan is NULL");
  if (!p->budget || !p->out_off || !p->kept_idx) return fail(AIRCACHE_EINVAL, "plan budget/out_off/kept_idx NULL");
  if (for_compress) return AIRCACHE_OK;
  if (!p->elite_idx || !p->n_elite || !p->iv || !p->s_t || !p->s_k || !p->status)
    return fail(AIRCACHE_EINVAL, "a required plan output pointer is NULL");
  if (cfg.sh.per_head && !p->iv_head)
    return fail(AIRCACHE_EINVAL, "plan iv_head is NULL (one selection per KV head writes it)");
  return AIRCACHE_OK;
}

int fill_table(const void *const *src, int L, LayerTable *t, const char *name) {
  if (!src) return fail(AIRCACHE_EINVAL, "%s is NULL", name);
  for (int l = 0; l < L; ++l) {
    if (!src[l]) return fail(AIRCACHE_EINVAL, "%s[%d] is NULL", name, l);
    if (!aligned16(src[l])) return fail(AIRCACHE_EINVAL, "%s[%d] is not 16-byte aligned", name, l);
    t->p[l] = src[l];
  }
  for (int l = L; l < AIRCACHE_MAX_LAYERS; ++l) t->p[l] = nullptr;
  return AIRCACHE_OK;
}

// Compaction tables with the layer-overlap checks of aircache_compress.
int gather_tables(const Config &cfg, const void *const *k, const void *const *v, void *const *k_out,
                  void *const *v_out, GatherTables *tb) {
  const Shape &s = cfg.sh;
  int rc;
  if ((rc = fill_table(k, s.L, &tb->k, "k"))) return rc;
  if ((rc = fill_table(v, s.L, &tb->v, "v"))) return rc;
  LayerTable ko, vo;
  if ((rc = fill_table(const_cast<const void *const *>(k_out), s.L, &ko, "k_out"))) return rc;
  if ((rc = fill_table(const_cast<const void *const *>(v_out), s.L, &vo, "v_out"))) return rc;
  const int esz = (int)(cfg.tile_bytes / (16 * s.D));
  const size_t layer_in = (size_t)s.B * s.Hkv * s.S * s.D * esz;
  const size_t layer_out_max = (size_t)s.B * s.Hkv * s.S * s.D * esz;
  for (int l = 0; l < s.L; ++l) {
    tb->ko.p[l] = const_cast<void *>(ko.p[l]);
    tb->vo.p[l] = const_cast<void *>(vo.p[l]);
    const char *o[2] = {static_cast<const char *>(ko.p[l]), static_cast<const char *>(vo.p[l])};
    for (int a = 0; a < 2; ++a) {
      for (int m = 0; m < s.L; ++m) {
        const char *in[2] = {static_cast<const char *>(tb->k.p[m]), static_cast<const char *>(tb->v.p[m])};
        for (int c = 0; c < 2; ++c)
          if (o[a] < in[c] + layer_in && in[c] < o[a] + layer_out_max)
            return fail(AIRCACHE_EINVAL, "an output buffer of layer %d may overlap input layer %d", l, m);
      }
    }
  }
  for (int l = s.L; l < AIRCACHE_MAX_LAYERS; ++l) tb->ko.p[l] = tb->vo.p[l] = nullptr;
  return AIRCACHE_OK;
}

int launch_gather(const Config &cfg, const GatherTables &tb, const PlanPtrs &pp, hipStream_t st) {
  const Shape &s = cfg.sh;
  const int esz = (int)(cfg.tile_bytes / (16 * s.D));
  const int units = s.L * s.B * s.Hkv;
  int nch = (2048 + units - 1) / units;
  if (nch > 64) nch = 64;
  if (nch < 1) nch = 1;
  const int rb = s.D * esz;
  const int64_t cap = (int64_t)s.B * s.Hkv * s.S * s.D;
  const dim3 grid((unsigned)(units * nch));
  if (rb == 128)
    hipLaunchKernelGGL(kv_gather_kernel<128>, grid, dim3(256), 0, st, s, tb, pp, nch, esz, cap);
  else if (rb == 256)
    hipLaunchKernelGGL(kv_gather_kernel<256>, grid, dim3(256), 0, st, s, tb, pp, nch, esz, cap);
  else
    hipLaunchKernelGGL(kv_gather_kernel<512>, grid, dim3(256), 0, st, s, tb, pp, nch, esz, cap);
  return check_hip(hipGetLastError(), "kv_gather_kernel launch");
}

// The whole pass (aircache_run): one chunked launch that also compacts where
// the descriptor allows it, else the plan launches then the gather.
int run_pass(const Config &cfg, const aircache_desc *desc, const void *const *q_txt, const void *const *k,
             const void *const *v, const aircache_plan_buf *plan, void *const *k_out, void *const *v_out,
             void *workspace, size_t ws_bytes, hipStream_t st, hipEvent_t *ev) {
  int rc;
  if ((rc = check_plan_buf(plan, false, cfg))) return rc;
  if (!workspace || ws_bytes < cfg.ws_bytes)
    return fail(AIRCACHE_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? ws_bytes : 0,
                cfg.ws_bytes);
  if (!aligned16(workspace)) return fail(AIRCACHE_EINVAL, "workspace is not 16-byte aligned");
  LayerTable qt, kt;
  if ((rc = fill_table(q_txt, cfg.sh.L, &qt, "q_txt"))) return rc;
  if ((rc = fill_table(k, cfg.sh.L, &kt, "k"))) return rc;
  GatherTables tb;
  if ((rc = gather_tables(cfg, k, v, k_out, v_out, &tb))) return rc;
  const PlanPtrs pp = plan_ptrs(plan);
  const bool bf = desc->dtype == AIRCACHE_BF16;
  if ((rc = mark(ev, 0, st))) return rc;
  if (cfg.run_fused) {
    LayerTable vt, kot, vot;
    for (int l = 0; l < cfg.sh.L; ++l) {
      vt.p[l] = tb.v.p[l];
      kot.p[l] = tb.ko.p[l];
      vot.p[l] = tb.vo.p[l];
    }
    const RunOut out{&vt, &kot, &vot};
    int fgrid = 0;
    if (cfg.small) {
      if (bf && cfg.sh.D == 128) rc = launch_small<Bf16Tag, 128>(cfg, qt, kt, pp, st, &out);
      else if (bf) rc = launch_small<Bf16Tag, 64>(cfg, qt, kt, pp, st, &out);
      else if (cfg.sh.D == 128) rc = launch_small<F32Tag, 128>(cfg, qt, kt, pp, st, &out);
      else rc = launch_small<F32Tag, 64>(cfg, qt, kt, pp, st, &out);
    } else if (bf && cfg.sh.D == 128) {
      if (!(rc = pass_grid<Bf16Tag, 128>(cfg, &fgrid)))
        rc = launch_chunked<Bf16Tag, 128>(cfg, qt, kt, pp, workspace, fgrid, st, &out);
    } else if (bf) {
      if (!(rc = pass_grid<Bf16Tag, 64>(cfg, &fgrid)))
        rc = launch_chunked<Bf16Tag, 64>(cfg, qt, kt, pp, workspace, fgrid, st, &out);
    } else if (cfg.sh.D == 128) {
      if (!(rc = pass_grid<F32Tag, 128>(cfg, &fgrid)))
        rc = launch_chunked<F32Tag, 128>(cfg, qt, kt, pp, workspace, fgrid, st, &out);
    } else {
      if (!(rc = pass_grid<F32Tag, 64>(cfg, &fgrid)))
        rc = launch_chunked<F32Tag, 64>(cfg, qt, kt, pp, workspace, fgrid, st, &out);
    }
    if (rc) return rc;
  } else {
    if ((rc = aircache_plan(desc, q_txt, k, plan, workspace, ws_bytes, st))) return rc;
    if ((rc = launch_gather(cfg, tb, pp, st))) return rc;
  }
  return mark(ev, 1, st);
}

// ----------------------------------------------------------------------------
// Library-owned scratch for aircache_run_noalloc: one array per device (each
// GPU the library runs on holds its own copy until the process ends), used in
// place of a caller workspace. In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
// ----------------------------------------------------------------------------
constexpr size_t kScratchBytes = AIRCACHE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  void *ptr;             // device address of this device's scratch, NULL until looked up
  bool have_desc;        // desc holds the descriptor the scratch is laid out for
  aircache_desc desc;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

bool same_desc(const aircache_desc &a, const aircache_desc &b) {
  return a.n_layers == b.n_layers && a.batch == b.batch && a.n_q_heads == b.n_q_heads &&
         a.n_kv_heads == b.n_kv_heads && a.head_dim == b.head_dim && a.n_vis == b.n_vis &&
         a.n_txt == b.n_txt && a.dtype == b.dtype && a.alpha == b.alpha && a.ratio == b.ratio &&
         a.max_elite == b.max_elite && a.path == b.path && a.budget_mode == b.budget_mode &&
         a.obs_window == b.obs_window;
}

// Zero n16 16-byte words (a kernel, not hipMemsetAsync, so a captured graph
// replays it like any other kernel).
__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4_t *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
}

// The current device's scratch slot, with its address looked up on the
// device's first use. g_scratch_mu held.
int scratch_slot(ScratchSlot **slot) {
  int dev = 0, rc;
  if ((rc = check_hip(hipGetDevice(&dev), "hipGetDevice"))) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(AIRCACHE_EINVAL, "device %d beyond the %d the scratch serves", dev, kMaxDevices);
  ScratchSlot &s = g_scratch[dev];
  if (!s.ptr) {
    void *p = nullptr;
    if ((rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))) return rc;
    if (!p) return fail(AIRCACHE_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
    s.ptr = p;
  }
  *slot = &s;
  return AIRCACHE_OK;
}

}  // namespace aircache

using namespace aircache;

// ----------------------------------------------------------------------------
// Decode attention over the compacted cache (decode.h).
// ----------------------------------------------------------------------------

size_t decode_ws_bytes(const Shape &s) {
  const size_t units = (size_t)s.L * s.B * s.Hq * decode_splits(s.L, s.B, s.Hkv, kDecTargetCus, s.ratio, s.Nv, s.Nt);
  return align_up(units * sizeof(float2)) + align_up(units * (size_t)s.D * sizeof(float));
}

// KIND: 0 decode_partial_kernel on the vector units, 1 the same with weights x
// V on the matrix cores, 2 and 3 decode_wave_kernel with one or two groups of
// 16 heads.
template <typename Tag, int D, bool Q8, int KIND>
int launch_decode(const Shape &s, const DecodeTables &tb, const aircache_plan_buf *plan, void *ws, hipStream_t st,
                  DecodeScales scl) {
  constexpr bool PV = KIND == 1;
  const int smax = KIND >= 2 ? decode_wave_splits(s.L, s.B, s.Hkv, kDecTargetCus, s.ratio, s.Nv, s.Nt)
                             : decode_splits(s.L, s.B, s.Hkv, kDecTargetCus, s.ratio, s.Nv, s.Nt);
  const size_t units = (size_t)s.L * s.B * s.Hq * smax;
  float2 *ml = static_cast<float2 *>(ws);
  float *acc = reinterpret_cast<float *>(static_cast<char *>(ws) + align_up(units * sizeof(float2)));
  const int64_t cap = (int64_t)s.B * s.Hkv * (int64_t)s.S * s.D;
  const size_t lds = KIND >= 2 ? (size_t)decode_wave_lds(s.G, D)
                    : PV ? (size_t)decode_pv_lds(s.G, D).total : (size_t)decode_lds_bytes(s.G, D, Q8 ? 1 : Tag::kBytes);
  const long long grid = (long long)s.L * s.B * s.Hkv * smax;
  if (grid > INT32_MAX) return fail(AIRCACHE_EINVAL, "decode grid of %lld workgroups too large", grid);
  int rc;
  if constexpr (KIND >= 2) {
    static_assert(Tag::kBytes == 2, "decode_wave_kernel takes bfloat16 queries");
    constexpr int NHG = KIND - 1;
    if ((rc = allow_lds(decode_wave_kernel<D, Q8, NHG>, lds))) return rc;
    hipLaunchKernelGGL((decode_wave_kernel<D, Q8, NHG>), dim3((unsigned)grid), dim3(kDecThreads), lds, st, s, tb,
                       plan->budget, plan->out_off, cap, smax, ml, acc, scl);
  } else {
    if ((rc = allow_lds(decode_partial_kernel<Tag, D, Q8, PV>, lds))) return rc;
    hipLaunchKernelGGL((decode_partial_kernel<Tag, D, Q8, PV>), dim3((unsigned)grid), dim3(kDecThreads), lds, st, s,
                       tb, plan->budget, plan->out_off, cap, smax, ml, acc, scl);
  }
  if ((rc = check_hip(hipGetLastError(), "decode_partial_kernel launch"))) return rc;
  if (KIND >= 2 && smax == 1) return AIRCACHE_OK;  // decode_wave_kernel wrote o itself
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(s.L * s.B * s.Hq)), dim3(D), 0, st, s, tb,
                     plan->budget, plan->out_off, cap, smax, ml, acc);
  return check_hip(hipGetLastError(), "decode_combine_kernel launch");
}

// ----------------------------------------------------------------------------
// Prefill attention with the scores of the text rows (prefill.h). One call per
// layer: elite_select_kernel -> prefill_kernel, whose extra
// workgroups finalize the previous layer (I_v, statistics); after the last
// layer prefill_finalize_kernel for it and topk_select_kernel. The scoring
// workspace holds two layers (by parity); the counters and the elite parts
// hold every layer (the last layer's finalize computes the budgets of all
// layers, as on the tiled path).
// ----------------------------------------------------------------------------
struct PrefillCfg {
  Config cfg;  // T = 64 (the attention's key tile), one more statistics pair per row
  int nqt_vis, nqt_txt;
  long long grid;
  size_t lds;
  int nqb;           // 16-row query blocks per wave (1 or 2)
  int evs;           // row stride of the exponentials: N_v rounded up to the key tile
  size_t fin_lds;    // prefill_finalize_kernel's row weights or I_v
  size_t stats_slot, e_slot;  // float2 / float elements of one workspace slot
};

int make_prefill_config(const aircache_desc *d, PrefillCfg *pc) {
  if (!d) return fail(AIRCACHE_EINVAL, "desc is NULL");
  aircache_desc dd = *d;
  dd.path = AIRCACHE_PATH_TILED;  // the tiled path's finalize and top-k kernels
  int rc;
  if ((rc = make_config(&dd, &pc->cfg))) return rc;
  if (d->dtype != AIRCACHE_BF16) return fail(AIRCACHE_EINVAL, "the prefill attention takes bfloat16 inputs");
  if (d->obs_window < 0)
    return fail(AIRCACHE_EINVAL, "the visual window is served by aircache_plan / aircache_run on every position's queries");
  Config &cfg = pc->cfg;
  Shape &s = cfg.sh;
  s.T = kPfKeys;
  s.ntiles = (s.Nv + kPfKeys - 1) / kPfKeys;
  s.nstat = s.ntiles + 1;
  s.qrows = s.S;
  s.qoff = s.Nv;
  // 128 query rows per workgroup, or 64 when 128 would leave CUs without a
  // workgroup (measured: 64 rows cost more per key tile than they gain in
  // balance once every CU has one; workload 2: 735 -> 692 us, workload 3:
  // 2654 -> 3699 us had it taken 64)
  {
    const long long wg128 = (long long)s.B * s.Hq * ((s.Nv + kPfRows - 1) / kPfRows + (s.Nt + kPfRows - 1) / kPfRows);
    pc->nqb = wg128 < kTargetCus ? 1 : 2;
  }
  const int rw = 16 * pc->nqb * kPfWaves;
  pc->nqt_vis = (s.Nv + rw - 1) / rw;
  pc->nqt_txt = (s.Nt + rw - 1) / rw;
  pc->grid = (long long)s.B * s.Hq * (pc->nqt_vis + pc->nqt_txt);
  if (pc->grid > INT32_MAX) return fail(AIRCACHE_EINVAL, "prefill grid of %lld workgroups too large", pc->grid);
  pc->lds = s.D == 128 ? (size_t)PfLayout<128>::kBytes : (size_t)PfLayout<64>::kBytes;
  const size_t units = (size_t)s.B * s.Hkv;  // one layer
  pc->evs = s.ntiles * kPfKeys;
  pc->fin_lds = (size_t)(s.rcap16 > s.Nv ? s.rcap16 : s.Nv) * sizeof(float);
  if (pc->fin_lds > pc->lds)
    return fail(AIRCACHE_EINVAL, "the prefill finalize needs %zu bytes of LDS (n_vis or the elite rows per KV head "
                "too large; lower max_elite)", pc->fin_lds);
  // two slots of scoring terms (layer parity): a layer's finalize runs in the
  // next layer's launch while that layer writes the other slot
  pc->stats_slot = units * s.rcap16 * (size_t)s.nstat;
  pc->e_slot = units * s.rcap16 * (size_t)pc->evs;
  cfg.off_e = cfg.off_stats + align_up(2 * pc->stats_slot * sizeof(float2));
  cfg.off_part = cfg.off_e + align_up(2 * pc->e_slot * sizeof(float));
  cfg.ws_bytes = cfg.off_part + align_up(units * (size_t)s.Nv * sizeof(float));
  return AIRCACHE_OK;
}

int check_prefill_io(const PrefillCfg &pc, const void *q, const void *k, const void *v, const void *o) {
  if (!q || !k || !v || !o) return fail(AIRCACHE_EINVAL, "q, k, v or o is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(AIRCACHE_EINVAL, "q, k, v and o must be 16-byte aligned");
  const Shape &s = pc.cfg.sh;
  const size_t qb = (size_t)s.B * s.Hq * s.S * s.D * 2, kb = (size_t)s.B * s.Hkv * s.S * s.D * 2;
  const char *oc = static_cast<const char *>(o);
  auto overlap = [&](const void *p, size_t n) {
    const char *c = static_cast<const char *>(p);
    return c < oc + qb && oc < c + n;
  };
  if (overlap(q, qb) || overlap(k, kb) || overlap(v, kb)) return fail(AIRCACHE_EINVAL, "o overlaps q, k or v");
  return AIRCACHE_OK;
}

template <int D, int NQB>
int launch_prefill(const PrefillCfg &pc, int layer, const void *q, const void *k, const void *v, void *o,
                   const aircache_plan_buf *plan, void *ws_base, hipStream_t st) {
  Config cfg = pc.cfg;
  Shape &s = cfg.sh;
  PrefillArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.o = static_cast<uint16_t *>(o);
  a.nqt_vis = pc.nqt_vis;
  a.nqt_txt = pc.nqt_txt;
  a.layer = layer;
  int rc;
  if (!plan) {
    a.score = 0;
    a.elite = a.n_elite = nullptr;
    a.e = nullptr;
    a.stats = nullptr;
    a.evs = 0;
    a.nattn = (int)pc.grid;
    a.fin_e = nullptr;
    a.fin_stats = nullptr;
    a.plan = PlanPtrs{};
    a.ws = Ws{};
    if ((rc = allow_lds(prefill_kernel<D, false, NQB>, pc.lds))) return rc;
    hipLaunchKernelGGL((prefill_kernel<D, false, NQB>), dim3((unsigned)pc.grid), dim3(kPfThreads), pc.lds, st, s, a);
    return check_hip(hipGetLastError(), "prefill_kernel launch");
  }
  s.lb0 = layer * s.B;
  const PlanPtrs pp = plan_ptrs(plan);
  const Ws ws = ws_of(cfg, ws_base);
  LayerTable qt, kt;
  for (int l = 0; l < AIRCACHE_MAX_LAYERS; ++l) qt.p[l] = kt.p[l] = nullptr;
  qt.p[layer] = q;
  kt.p[layer] = k;
  a.score = 1;
  a.elite = plan->elite_idx + (size_t)s.lb0 * s.Nt;
  a.n_elite = plan->n_elite + s.lb0;
  const int slot = layer & 1;
  a.e = ws.e + slot * pc.e_slot;
  a.stats = ws.stats + slot * pc.stats_slot;
  a.evs = pc.evs;
  a.nattn = (int)pc.grid;
  a.fin_e = ws.e + (slot ^ 1) * pc.e_slot;
  a.fin_stats = ws.stats + (slot ^ 1) * pc.stats_slot;
  a.plan = pp;
  a.ws = ws;
  const long long nfin = (long long)s.B * s.Hkv * s.ntiles;  // finalize workgroups of one layer
  const long long grid = pc.grid + (layer > 0 ? nfin : 0);
  if (grid > INT32_MAX) return fail(AIRCACHE_EINVAL, "prefill grid of %lld workgroups too large", grid);
  if ((rc = allow_lds(prefill_kernel<D, true, NQB>, pc.lds))) return rc;
  if ((rc = allow_lds(prefill_finalize_kernel, pc.fin_lds))) return rc;
  if ((rc = allow_lds(elite_select_kernel<Bf16Tag, D>, cfg.elite_lds))) return rc;
  hipLaunchKernelGGL((elite_select_kernel<Bf16Tag, D>), dim3((unsigned)(s.B * s.Hkv)), dim3(kEliteThreads),
                     cfg.elite_lds, st, s, qt, kt, pp, ws);
  if ((rc = check_hip(hipGetLastError(), "elite_select_kernel launch"))) return rc;
  hipLaunchKernelGGL((prefill_kernel<D, true, NQB>), dim3((unsigned)grid), dim3(kPfThreads), pc.lds, st, s, a);
  if ((rc = check_hip(hipGetLastError(), "prefill_kernel launch"))) return rc;
  if (layer == s.L - 1) {
    // the last layer's finalize, then the selection of every layer
    hipLaunchKernelGGL(prefill_finalize_kernel, dim3((unsigned)nfin), dim3(kPfFinThreads), pc.fin_lds, st, s, pp, ws,
                       static_cast<const float *>(a.e), static_cast<const float2 *>(a.stats), pc.evs);
    if ((rc = check_hip(hipGetLastError(), "prefill_finalize_kernel launch"))) return rc;
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)(s.L * s.B * s.nsel)), dim3(kTopkThreads), 0, st, s, pp);
    if ((rc = check_hip(hipGetLastError(), "topk_select_kernel launch"))) return rc;
  }
  return AIRCACHE_OK;
}

// aircache_decode and aircache_decode_i8: kq / vq and the scales are NULL for
// the compacted cache in the pass dtype.
int decode_common(const aircache_desc *desc, const void *const *q_dec, const aircache_plan_buf *plan,
                  const void *const *k_out, const void *const *v_out, const float *k_scale, const float *v_scale,
                  float *const *o, void *workspace, size_t ws_bytes, void *stream, bool q8) {
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  const Shape &s = cfg.sh;
  if (!plan || !plan->budget || !plan->out_off) return fail(AIRCACHE_EINVAL, "plan, plan->budget or plan->out_off is NULL");
  if (!aligned16(plan->out_off)) return fail(AIRCACHE_EINVAL, "plan->out_off is not 16-byte aligned");
  if (q8 && (!k_scale || !v_scale)) return fail(AIRCACHE_EINVAL, "k_scale or v_scale is NULL");
  const int esize = q8 ? 1 : (desc->dtype == AIRCACHE_BF16 ? 2 : 4);
  if ((long long)s.G * s.D / 8 > kDecThreads || decode_lds_bytes(s.G, s.D, esize) > kDecMaxLds)
    return fail(AIRCACHE_EINVAL, "decode holds %d query heads per KV head at most for head_dim %d",
                kDecThreads * 8 / s.D, s.D);
  DecodeTables tb;
  if ((rc = fill_table(q_dec, s.L, &tb.q, "q_dec"))) return rc;
  if ((rc = fill_table(k_out, s.L, &tb.k, q8 ? "kq" : "k_out"))) return rc;
  if ((rc = fill_table(v_out, s.L, &tb.v, q8 ? "vq" : "v_out"))) return rc;
  LayerTable ot;
  if ((rc = fill_table(reinterpret_cast<const void *const *>(o), s.L, &ot, "o"))) return rc;
  for (int l = 0; l < AIRCACHE_MAX_LAYERS; ++l) tb.o.p[l] = const_cast<void *>(ot.p[l]);
  if (!workspace || ws_bytes < decode_ws_bytes(s))
    return fail(AIRCACHE_EWORKSPACE, "decode workspace of %zu bytes, %zu needed", ws_bytes, decode_ws_bytes(s));
  if (!aligned16(workspace)) return fail(AIRCACHE_EINVAL, "workspace is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = desc->dtype == AIRCACHE_BF16;
  const DecodeScales scl{k_scale, v_scale};
  const int kind = decode_kind(s.G, bf ? 2 : 4, s.ratio, s.Nv, s.Nt);
#define AIRCACHE_DECODE_KINDS(TAG, DD, Q)                                                          \
  switch (kind) {                                                                                  \
    case 1: return launch_decode<TAG, DD, Q, 1>(s, tb, plan, workspace, st, scl);                 \
    case 2: return launch_decode<TAG, DD, Q, 2>(s, tb, plan, workspace, st, scl);                 \
    case 3: return launch_decode<TAG, DD, Q, 3>(s, tb, plan, workspace, st, scl);                 \
    default: return launch_decode<TAG, DD, Q, 0>(s, tb, plan, workspace, st, scl);                \
  }
  if (bf && s.D == 128) {
    if (q8) AIRCACHE_DECODE_KINDS(Bf16Tag, 128, true)
    AIRCACHE_DECODE_KINDS(Bf16Tag, 128, false)
  }
  if (bf) {
    if (q8) AIRCACHE_DECODE_KINDS(Bf16Tag, 64, true)
    AIRCACHE_DECODE_KINDS(Bf16Tag, 64, false)
  }
#undef AIRCACHE_DECODE_KINDS
  if (s.D == 128)
    return q8 ? launch_decode<F32Tag, 128, true, 0>(s, tb, plan, workspace, st, scl)
              : launch_decode<F32Tag, 128, false, 0>(s, tb, plan, workspace, st, scl);
  return q8 ? launch_decode<F32Tag, 64, true, 0>(s, tb, plan, workspace, st, scl)
            : launch_decode<F32Tag, 64, false, 0>(s, tb, plan, workspace, st, scl);
}

extern "C" {

int aircache_abi_version(void) { return AIRCACHE_ABI_VERSION; }

size_t aircache_workspace_size(const aircache_desc *desc) {
  Config cfg;
  if (make_config(desc, &cfg) != AIRCACHE_OK) return 0;
  return cfg.ws_bytes;
}

int64_t aircache_max_compacted_elems(const aircache_desc *desc) {
  Config cfg;
  if (make_config(desc, &cfg) != AIRCACHE_OK) return -1;
  const Shape &s = cfg.sh;
  return (int64_t)s.B * s.Hkv * (int64_t)(s.Nv + s.Nt) * s.D;
}

int32_t aircache_resolved_path(const aircache_desc *desc) {
  Config cfg;
  if (make_config(desc, &cfg) != AIRCACHE_OK) return -1;
  return cfg.path;
}

int32_t aircache_run_launches(const aircache_desc *desc) {
  Config cfg;
  if (make_config(desc, &cfg) != AIRCACHE_OK) return -1;
  if (cfg.run_fused) return 1;
  // aircache_plan's kernels, then kv_gather_kernel
  return (cfg.chunked || cfg.small ? 1 : cfg.rows_kt ? 3 : 4) + 1;
}

int aircache_plan_profiled(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                           const aircache_plan_buf *plan, void *workspace, size_t ws_bytes, void *stream,
                           void *const *events, int n_events) {
  if (events && n_events != AIRCACHE_PLAN_KERNELS + 1)
    return fail(AIRCACHE_EINVAL, "n_events=%d, expected %d", n_events, AIRCACHE_PLAN_KERNELS + 1);
  hipEvent_t *ev = events ? reinterpret_cast<hipEvent_t *>(const_cast<void **>(events)) : nullptr;
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  if ((rc = check_plan_buf(plan, false, cfg))) return rc;
  if (!workspace || ws_bytes < cfg.ws_bytes)
    return fail(AIRCACHE_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? ws_bytes : 0,
                cfg.ws_bytes);
  if (!aligned16(workspace)) return fail(AIRCACHE_EINVAL, "workspace is not 16-byte aligned");
  LayerTable qt, kt;
  if ((rc = fill_table(q_txt, cfg.sh.L, &qt, "q_txt"))) return rc;
  if ((rc = fill_table(k, cfg.sh.L, &kt, "k"))) return rc;
  const PlanPtrs pp = plan_ptrs(plan);
  const Ws ws = ws_of(cfg, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = desc->dtype == AIRCACHE_BF16;
  if (bf && cfg.sh.D == 128) return launch_plan<Bf16Tag, 128, 4>(cfg, qt, kt, pp, ws, workspace, st, ev);
  if (bf && cfg.sh.D == 64) return launch_plan<Bf16Tag, 64, 4>(cfg, qt, kt, pp, ws, workspace, st, ev);
  if (!bf && cfg.sh.D == 128) return launch_plan<F32Tag, 128, 2>(cfg, qt, kt, pp, ws, workspace, st, ev);
  return launch_plan<F32Tag, 64, 2>(cfg, qt, kt, pp, ws, workspace, st, ev);
}

int aircache_plan(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                  const aircache_plan_buf *plan, void *workspace, size_t ws_bytes, void *stream) {
  return aircache_plan_profiled(desc, q_txt, k, plan, workspace, ws_bytes, stream, nullptr, 0);
}

int aircache_compress_profiled(const aircache_desc *desc, const aircache_plan_buf *plan, const void *const *k,
                               const void *const *v, void *const *k_out, void *const *v_out, void *stream,
                               void *const *events, int n_events) {
  if (events && n_events != AIRCACHE_COMPRESS_KERNELS + 1)
    return fail(AIRCACHE_EINVAL, "n_events=%d, expected %d", n_events, AIRCACHE_COMPRESS_KERNELS + 1);
  hipEvent_t *ev = events ? reinterpret_cast<hipEvent_t *>(const_cast<void **>(events)) : nullptr;
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  if ((rc = check_plan_buf(plan, true, cfg))) return rc;
  GatherTables tb;
  if ((rc = gather_tables(cfg, k, v, k_out, v_out, &tb))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = mark(ev, 0, st))) return rc;
  if ((rc = launch_gather(cfg, tb, plan_ptrs(plan), st))) return rc;
  return mark(ev, 1, st);
}

int aircache_run_profiled(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                          const void *const *v, const aircache_plan_buf *plan, void *const *k_out,
                          void *const *v_out, void *workspace, size_t ws_bytes, void *stream,
                          void *const *events, int n_events) {
  if (events && n_events != AIRCACHE_RUN_KERNELS + 1)
    return fail(AIRCACHE_EINVAL, "n_events=%d, expected %d", n_events, AIRCACHE_RUN_KERNELS + 1);
  hipEvent_t *ev = events ? reinterpret_cast<hipEvent_t *>(const_cast<void **>(events)) : nullptr;
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  return run_pass(cfg, desc, q_txt, k, v, plan, k_out, v_out, workspace, ws_bytes, static_cast<hipStream_t>(stream),
                  ev);
}

int aircache_run_noalloc(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                         const void *const *v, const aircache_plan_buf *plan, void *const *k_out,
                         void *const *v_out, void *stream) {
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  if (cfg.ws_bytes > kScratchBytes)
    return fail(AIRCACHE_EINVAL, "this descriptor needs %zu bytes of scratch; aircache_run_noalloc holds %zu "
                "(use aircache_run with a workspace)", cfg.ws_bytes, kScratchBytes);
  // validate everything before the scratch is touched, so a rejected call
  // leaves it as the last accepted call left it
  if ((rc = check_plan_buf(plan, false, cfg))) return rc;
  {
    LayerTable t;
    GatherTables tb;
    if ((rc = fill_table(q_txt, cfg.sh.L, &t, "q_txt"))) return rc;
    if ((rc = gather_tables(cfg, k, v, k_out, v_out, &tb))) return rc;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot *slot = nullptr;
  if ((rc = scratch_slot(&slot))) return rc;
  // the records of the pass are valid across calls with one descriptor only:
  // on a device's first call, or after a call with another descriptor, the
  // part of the scratch this descriptor uses is zeroed first
  if (!slot->have_desc || !same_desc(slot->desc, *desc)) {
    slot->have_desc = false;
    const size_t n16 = cfg.ws_bytes / 16;  // ws_bytes is a multiple of 256
    if (n16 > 0) {
      const size_t want = (n16 + 255) / 256;
      const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
      hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, st, static_cast<u32x4_t *>(slot->ptr), n16);
      if ((rc = check_hip(hipGetLastError(), "zero_fill_kernel launch"))) return rc;
    }
    slot->desc = *desc;
    slot->have_desc = true;
  }
  rc = run_pass(cfg, desc, q_txt, k, v, plan, k_out, v_out, slot->ptr, kScratchBytes, st, nullptr);
  if (rc == AIRCACHE_EHIP) slot->have_desc = false;  // a launch failed: zero again on the next call
  return rc;
}

int aircache_run(const aircache_desc *desc, const void *const *q_txt, const void *const *k, const void *const *v,
                 const aircache_plan_buf *plan, void *const *k_out, void *const *v_out, void *workspace,
                 size_t ws_bytes, void *stream) {
  return aircache_run_profiled(desc, q_txt, k, v, plan, k_out, v_out, workspace, ws_bytes, stream, nullptr, 0);
}

int aircache_compress(const aircache_desc *desc, const aircache_plan_buf *plan, const void *const *k,
                      const void *const *v, void *const *k_out, void *const *v_out, void *stream) {
  return aircache_compress_profiled(desc, plan, k, v, k_out, v_out, stream, nullptr, 0);
}

size_t aircache_decode_workspace_size(const aircache_desc *desc) {
  Config cfg;
  if (make_config(desc, &cfg)) return 0;
  return decode_ws_bytes(cfg.sh);
}

int aircache_decode(const aircache_desc *desc, const void *const *q_dec, const aircache_plan_buf *plan,
                    const void *const *k_out, const void *const *v_out, float *const *o, void *workspace,
                    size_t ws_bytes, void *stream) {
  return decode_common(desc, q_dec, plan, k_out, v_out, nullptr, nullptr, o, workspace, ws_bytes, stream, false);
}

int aircache_decode_i8(const aircache_desc *desc, const void *const *q_dec, const aircache_plan_buf *plan,
                       const int8_t *const *kq, const int8_t *const *vq, const float *k_scale, const float *v_scale,
                       float *const *o, void *workspace, size_t ws_bytes, void *stream) {
  return decode_common(desc, q_dec, plan, reinterpret_cast<const void *const *>(kq),
                       reinterpret_cast<const void *const *>(vq), k_scale, v_scale, o, workspace, ws_bytes, stream,
                       true);
}

int aircache_quantize_i8(const aircache_desc *desc, const aircache_plan_buf *plan, const void *const *k_out,
                         const void *const *v_out, int8_t *const *kq, int8_t *const *vq, float *k_scale,
                         float *v_scale, void *stream) {
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  const Shape &s = cfg.sh;
  if (!plan || !plan->budget || !plan->out_off) return fail(AIRCACHE_EINVAL, "plan, plan->budget or plan->out_off is NULL");
  if (!k_scale || !v_scale) return fail(AIRCACHE_EINVAL, "k_scale or v_scale is NULL");
  QuantTables tb;
  if ((rc = fill_table(k_out, s.L, &tb.ko, "k_out"))) return rc;
  if ((rc = fill_table(v_out, s.L, &tb.vo, "v_out"))) return rc;
  LayerTable a, c;
  if ((rc = fill_table(reinterpret_cast<const void *const *>(kq), s.L, &a, "kq"))) return rc;
  if ((rc = fill_table(reinterpret_cast<const void *const *>(vq), s.L, &c, "vq"))) return rc;
  for (int l = 0; l < AIRCACHE_MAX_LAYERS; ++l) {
    tb.kq.p[l] = const_cast<void *>(a.p[l]);
    tb.vq.p[l] = const_cast<void *>(c.p[l]);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t cap = (int64_t)s.B * s.Hkv * s.S * s.D;
  const dim3 grid((unsigned)(2 * s.L * s.B * s.Hkv));
  if (desc->dtype == AIRCACHE_BF16 && quant_keep(s))
    hipLaunchKernelGGL((quantize_i8_kernel<Bf16Tag, kQuantKeep>), grid, dim3(kQuantThreads), 0, st, s, tb,
                       plan_ptrs(plan), k_scale, v_scale, cap);
  else if (desc->dtype == AIRCACHE_BF16)
    hipLaunchKernelGGL((quantize_i8_kernel<Bf16Tag, 0>), grid, dim3(kQuantThreads), 0, st, s, tb, plan_ptrs(plan),
                       k_scale, v_scale, cap);
  else
    hipLaunchKernelGGL((quantize_i8_kernel<F32Tag, 0>), grid, dim3(kQuantThreads), 0, st, s, tb, plan_ptrs(plan),
                       k_scale, v_scale, cap);
  return check_hip(hipGetLastError(), "quantize_i8_kernel launch");
}

size_t aircache_prefill_workspace_size(const aircache_desc *desc) {
  PrefillCfg pc;
  if (make_prefill_config(desc, &pc)) return 0;
  return pc.cfg.ws_bytes;
}

int aircache_prefill_layer(const aircache_desc *desc, int32_t layer, const void *q, const void *k, const void *v,
                           void *o, const aircache_plan_buf *plan, void *workspace, size_t ws_bytes, void *stream) {
  PrefillCfg pc;
  int rc;
  if ((rc = make_prefill_config(desc, &pc))) return rc;
  if (layer < 0 || layer >= pc.cfg.sh.L) return fail(AIRCACHE_EINVAL, "layer=%d outside [0, %d)", layer, pc.cfg.sh.L);
  if ((rc = check_plan_buf(plan, false, pc.cfg))) return rc;
  if ((rc = check_prefill_io(pc, q, k, v, o))) return rc;
  if (!workspace || ws_bytes < pc.cfg.ws_bytes)
    return fail(AIRCACHE_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, pc.cfg.ws_bytes);
  if (!aligned16(workspace)) return fail(AIRCACHE_EINVAL, "workspace is not 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pc.cfg.sh.D == 128)
    return pc.nqb == 1 ? launch_prefill<128, 1>(pc, layer, q, k, v, o, plan, workspace, st)
                       : launch_prefill<128, 2>(pc, layer, q, k, v, o, plan, workspace, st);
  return pc.nqb == 1 ? launch_prefill<64, 1>(pc, layer, q, k, v, o, plan, workspace, st)
                     : launch_prefill<64, 2>(pc, layer, q, k, v, o, plan, workspace, st);
}

int aircache_prefill_attention(const aircache_desc *desc, const void *q, const void *k, const void *v, void *o,
                               void *stream) {
  PrefillCfg pc;
  int rc;
  if ((rc = make_prefill_config(desc, &pc))) return rc;
  if ((rc = check_prefill_io(pc, q, k, v, o))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pc.cfg.sh.D == 128)
    return pc.nqb == 1 ? launch_prefill<128, 1>(pc, 0, q, k, v, o, nullptr, nullptr, st)
                       : launch_prefill<128, 2>(pc, 0, q, k, v, o, nullptr, nullptr, st);
  return pc.nqb == 1 ? launch_prefill<64, 1>(pc, 0, q, k, v, o, nullptr, nullptr, st)
                     : launch_prefill<64, 2>(pc, 0, q, k, v, o, nullptr, nullptr, st);
}

const char *aircache_strerror(int status) {
  switch (status) {
    case AIRCACHE_OK: return "ok";
    case AIRCACHE_EINVAL: return "invalid argument";
    case AIRCACHE_EWORKSPACE: return "workspace too small";
    case AIRCACHE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *aircache_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
