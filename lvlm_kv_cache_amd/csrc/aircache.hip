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

#include <string>

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
};

struct PlanPtrs {
  int32_t *elite, *n_elite;
  float *iv;
  double *s_t, *s_k, *bx;
  int32_t *budget;
  int64_t *out_off;
  int32_t *kept, *status;
};

struct Ws {
  unsigned *cnt_lb;   // [L*B] finished scoring tiles per (l, b)
  unsigned *cnt_b;    // [B]   finished layers per sample
  unsigned *cnt_all;  // [1]   finished samples
  float2 *stats;      // [units][rcap16][ntiles] (tile max, tile sum) per row, base 2
  float *e;           // [units][Nv][row stride] exp2(logit - tile max) of visual keys
};

struct LayerTable {
  const void *p[AIRCACHE_MAX_LAYERS];
};
struct LayerTableOut {
  void *p[AIRCACHE_MAX_LAYERS];
};

// ----------------------------------------------------------------------------
// Step 1: elite observation window ("Elite Observation Window", the Att and k
// equations). One workgroup per (layer, sample). For each query head the last
// text query's logits over the N_t text keys of its KV head come from MFMA
// (keys as the A operand, up to 16 heads of one KV group as the B operand);
// each wave then normalises whole rows (max, sum of exp2) and the rows are
// summed into pbar in a fixed head order. Elite = { j : pbar_j >= alpha max },
// compacted in ascending j by a block scan.
// ----------------------------------------------------------------------------
template <typename Tag, int D>
__global__ __launch_bounds__(256) void elite_select_kernel(Shape sh, LayerTable qt, LayerTable kt, PlanPtrs plan,
                                                           Ws ws) {
  using E = typename Tag::store_t;
  extern __shared__ float lds[];  // z[16][Nt], pbar[Nt]
  __shared__ float red[4];
  __shared__ int wtot[4];
  const int lb = blockIdx.x, l = lb / sh.B, b = lb % sh.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int Nt = sh.Nt, G = sh.G;
  float *z = lds;
  float *pbar = lds + 16 * Nt;

  // This kernel opens every plan: reset the counters of finalize_kernel.
  if (tid == 0) {
    ws.cnt_lb[lb] = 0;
    if (l == 0) ws.cnt_b[b] = 0;
    if (lb == 0) {
      *ws.cnt_all = 0;
      *plan.status = 0;
    }
  }
  for (int j = tid; j < Nt; j += 256) pbar[j] = 0.f;

  const E *q = static_cast<const E *>(qt.p[l]);
  const E *k = static_cast<const E *>(kt.p[l]);
  const int nkt = (Nt + 15) >> 4;
  for (int g = 0; g < sh.Hkv; ++g) {
    const E *ktxt = k + ((size_t)(b * sh.Hkv + g) * sh.S + sh.Nv) * D;
    for (int h0 = 0; h0 < G; h0 += 16) {
      const int nh = min(16, G - h0);
      Frag<Tag> qf[D / 32];
      if (n < nh) {
        const E *qrow = q + ((size_t)(b * sh.Hq + g * G + h0 + n) * Nt + (Nt - 1)) * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[c].load(qrow + c * 32 + grp * 8);
      } else {
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[c].zero();
      }
      __syncthreads();  // z is free (previous group fully consumed)
      for (int t = wave; t < nkt; t += 4) {
        Frag<Tag> kf[D / 32];
        const int key = t * 16 + n;
        if (key < Nt) {
          const E *krow = ktxt + (size_t)key * D;
#pragma unroll
          for (int c = 0; c < D / 32; ++c) kf[c].load(krow + c * 32 + grp * 8);
        } else {
#pragma unroll
          for (int c = 0; c < D / 32; ++c) kf[c].zero();
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) mfma_slice(acc, kf[c], qf[c]);
        if (n < nh) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = t * 16 + grp * 4 + i;
            if (kk < Nt) z[n * Nt + kk] = acc[i] * sh.scale2;
          }
        }
      }
      __syncthreads();
      for (int hh = wave; hh < nh; hh += 4) {
        float *zr = z + hh * Nt;
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
      for (int j = tid; j < Nt; j += 256) {
        float a = pbar[j];
        for (int hh = 0; hh < nh; ++hh) a += z[hh * Nt + j];
        pbar[j] = a;
      }
    }
  }
  __syncthreads();
  float m = -INFINITY;
  for (int j = tid; j < Nt; j += 256) m = fmaxf(m, pbar[j]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float thr = sh.alpha * m;
  const int per = (Nt + 255) / 256;
  const int j0 = min(Nt, tid * per), j1 = min(Nt, j0 + per);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += (pbar[j] >= thr) ? 1 : 0;
  const int incl = wave_incl_scan(cnt);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  int pos = base + incl - cnt;
  int32_t *el = plan.elite + (size_t)lb * Nt;
  for (int j = j0; j < j1; ++j)
    if (pbar[j] >= thr) el[pos++] = j;
  if (tid == 0) plan.n_elite[lb] = wtot[0] + wtot[1] + wtot[2] + wtot[3];
}

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
  const int nx = (t < ntk) ? (ntk - t + sh.ntiles - 1) / sh.ntiles : 0;

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
  float2 *st_out = ws.stats + (size_t)u * sh.rcap16 * sh.ntiles;
  for (int rt = 0; rt * 16 < R; ++rt) {
    const int r = rt * 16 + n;
    Frag<Tag> qf[D / 32];
    if (r < R) {
      const int hl = r / ntk, e = r - hl * ntk;
      const E *qrow = q + ((size_t)(b * sh.Hq + g * sh.G + hl) * sh.Nt + el[e]) * D;
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
    if (r < R) {
      if (wave == 0 && grp == 0) st_out[(size_t)r * sh.ntiles + t] = make_float2(m, zs);
#pragma unroll
      for (int i = 0; i < KTW; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = (wave + 4 * i) * 16 + grp * 4 + j;
          if (key < nvis) e_out[(size_t)(c0 + key) * RP + r] = acc[i][j];
        }
      }
    }
    __syncthreads();  // red_m / red_z are reused by the next row tile
  }
}

// Budget of every layer of one sample ("Layer-wise KV Cache Budget
// Allocation", the r_hat equation with the cross-layer normalisation reading
// documented in aircache.h). Plain double arithmetic in a fixed order with no
// fused multiply-add, so the same statistics give the same integers anywhere.
__device__ void sample_budgets(const Shape &sh, const PlanPtrs &plan, int b) {
#pragma clang fp contract(off)
  const int L = sh.L, B = sh.B;
  double st_sum = 0.0, mshift = 0.0, u_sum = 0.0;
  for (int l = 0; l < L; ++l) st_sum += load_coherent(&plan.s_t[l * B + b]);
  for (int l = 0; l < L; ++l) {
    const double sk = load_coherent(&plan.s_k[l * B + b]);
    if (sk < mshift) mshift = sk;
  }
  for (int l = 0; l < L; ++l) u_sum += load_coherent(&plan.s_k[l * B + b]) - mshift;
  const double r = sh.ratio * (double)sh.Nv;
  for (int l = 0; l < L; ++l) {
    const double st = load_coherent(&plan.s_t[l * B + b]);
    const double sk = load_coherent(&plan.s_k[l * B + b]);
    const double stn = st * (double)L / st_sum;
    const double skn = (u_sum > 0.0) ? (sk - mshift) * (double)L / u_sum : 1.0;
    const double x = 0.5 * (stn + skn) * r;
    double f = floor(x);
    if (!(f > 0.0)) f = 0.0;
    if (f > (double)sh.Nv) f = (double)sh.Nv;
    if (plan.bx) store_coherent(&plan.bx[l * B + b], x);
    store_coherent(&plan.budget[l * B + b], (int32_t)f);
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
// awaited before the counter moves.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void finalize_kernel(Shape sh, PlanPtrs plan, Ws ws) {
  extern __shared__ float wl[];  // weights [Hkv][rcap16], then I_v cache [Nv] for the finisher
  __shared__ double redd[4];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x % sh.ntiles;
  const int lb = blockIdx.x / sh.ntiles, b = lb % sh.B;
  int ntk = plan.n_elite[lb];
  if (ntk > sh.cap) ntk = sh.cap;
  if (ntk < 0) ntk = 0;
  const int R = sh.G * ntk;
  const int RP = (R + 15) & ~15;
  for (int idx = tid; idx < sh.Hkv * R; idx += 256) {
    const int g = idx / R, r = idx - g * R;
    const float2 *st = ws.stats + ((size_t)(lb * sh.Hkv + g) * sh.rcap16 + r) * sh.ntiles;
    float M = -INFINITY;
    for (int tt = 0; tt < sh.ntiles; ++tt) M = fmaxf(M, st[tt].x);
    float Z = 0.f;
    for (int tt = 0; tt < sh.ntiles; ++tt) Z += st[tt].y * exp2f(st[tt].x - M);
    wl[g * sh.rcap16 + r] = exp2f(st[t].x - M) / Z;
  }
  __syncthreads();
  const float inv_rows = (ntk > 0) ? 1.f / (float)(sh.Hq * ntk) : 0.f;
  const int c0 = t * sh.T, c1 = min(sh.Nv, c0 + sh.T);
  for (int c = c0 + tid; c < c1; c += 256) {
    float acc = 0.f;
    for (int g = 0; g < sh.Hkv; ++g) {
      const float *e = ws.e + (size_t)(lb * sh.Hkv + g) * sh.Nv * sh.rcap16 + (size_t)c * RP;
      const float *w = wl + g * sh.rcap16;
      for (int r = 0; r < R; ++r) acc += e[r] * w[r];
    }
    store_coherent(&plan.iv[(size_t)lb * sh.Nv + c], acc * inv_rows);
  }
  wait_all_memory();
  __syncthreads();
  if (tid == 0) is_last = (counter_add(&ws.cnt_lb[lb], 1u) == (unsigned)sh.ntiles - 1);
  __syncthreads();
  if (!is_last) return;

  // Statistics of I_v for this (layer, sample), in double precision.
  float *ivc = wl + sh.Hkv * sh.rcap16;
  const int Nv = sh.Nv;
  double s = 0.0;
  for (int c = tid; c < Nv; c += 256) {
    const float x = load_coherent(&plan.iv[(size_t)lb * Nv + c]);
    ivc[c] = x;
    s += (double)x;
  }
  s = wave_sum_d(s);
  if (lane == 0) redd[wave] = s;
  __syncthreads();
  s = (redd[0] + redd[1]) + (redd[2] + redd[3]);
  const double mu = s / (double)Nv;
  __syncthreads();
  double v2 = 0.0;
  for (int c = tid; c < Nv; c += 256) {
    const double d = (double)ivc[c] - mu;
    v2 += d * d;
  }
  v2 = wave_sum_d(v2);
  if (lane == 0) redd[wave] = v2;
  __syncthreads();
  v2 = (redd[0] + redd[1]) + (redd[2] + redd[3]);
  const double sigma = sqrt(v2 / (double)(Nv - 1));
  __syncthreads();
  double k3 = 0.0;
  if (sigma > 0.0) {
    for (int c = tid; c < Nv; c += 256) {
      const double d = ((double)ivc[c] - mu) / sigma;
      k3 += d * d * d;
    }
  }
  k3 = wave_sum_d(k3);
  if (lane == 0) redd[wave] = k3;
  __syncthreads();
  if (tid != 0) return;
  k3 = (redd[0] + redd[1]) + (redd[2] + redd[3]);
  const double skew = (sigma > 0.0) ? k3 * ((double)Nv / ((double)(Nv - 1) * (double)(Nv - 2))) : 0.0;
  store_coherent(&plan.s_t[lb], s);
  store_coherent(&plan.s_k[lb], skew);
  wait_all_memory();
  if (counter_add(&ws.cnt_b[b], 1u) != (unsigned)sh.L - 1) return;
  sample_budgets(sh, plan, b);
  wait_all_memory();
  if (counter_add(ws.cnt_all, 1u) != (unsigned)sh.B - 1) return;
  for (int l = 0; l < sh.L; ++l) {
    int64_t off = 0;
    for (int bb = 0; bb < sh.B; ++bb) {
      plan.out_off[(size_t)l * (sh.B + 1) + bb] = off;
      off += (int64_t)sh.Hkv * (load_coherent(&plan.budget[l * sh.B + bb]) + sh.Nt) * sh.D;
    }
    plan.out_off[(size_t)l * (sh.B + 1) + sh.B] = off;
  }
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
// float32 bits order like the values; a 4-pass MSB-first radix select (8 bits
// per pass, LDS histogram) finds the key T of the r_hat-th largest score. Kept:
// every key > T, plus the lowest-index keys equal to T up to r_hat in total;
// written in ascending index order by block scans. Each thread holds a
// contiguous run of indices.
// ----------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kTopkPer = 8;  // N_v <= 8192

__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(Shape sh, PlanPtrs plan) {
  __shared__ unsigned hist[256];
  __shared__ int wtot[16];
  __shared__ unsigned sel_digit, sel_above;
  const int tid = threadIdx.x, lane = tid & 63;
  const int lb = blockIdx.x;
  const int Nv = sh.Nv;
  if (tid == 0 && plan.n_elite[lb] > sh.cap) atomicOr(plan.status, AIRCACHE_DEV_ELITE_OVERFLOW);
  const int kbud = plan.budget[lb];
  int32_t *kept = plan.kept + (size_t)lb * Nv;
  const int per = (Nv + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(Nv, tid * per), i1 = min(Nv, i0 + per);
  if (kbud <= 0) return;
  if (kbud >= Nv) {
    for (int i = tid; i < Nv; i += kTopkThreads) kept[i] = i;
    return;
  }
  unsigned key[kTopkPer];
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p) {
    const int i = i0 + p;
    key[p] = (i < i1) ? __float_as_uint(plan.iv[(size_t)lb * Nv + i]) : 0u;
  }
  unsigned prefix = 0, mask = 0;
  int need = kbud;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kTopkPer; ++p)
      if (i0 + p < i1 && (key[p] & mask) == prefix) atomicAdd(&hist[(key[p] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane owns digits 255-4*lane .. 252-4*lane (descending); suffix counts
      unsigned c[4], s4 = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        s4 += c[q];
      }
      const int incl = wave_incl_scan((int)s4);  // count of digits >= this lane's lowest
      unsigned above = (unsigned)(incl - (int)s4);  // count of digits above this lane's highest
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
    mask |= 255u << shift;
    need -= (int)sel_above;
    __syncthreads();
  }
  const unsigned T = prefix;
  int neq = 0;
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p) neq += (i0 + p < i1 && key[p] == T) ? 1 : 0;
  int tot;
  int eq_rank = block_excl_scan_1024(neq, wtot, &tot);
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
  int pos = block_excl_scan_1024(nkeep, wtot, &tot);
#pragma unroll
  for (int p = 0; p < kTopkPer; ++p)
    if (keepbits & (1u << p)) kept[pos++] = i0 + p;
  (void)lane;
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
  if (seg0 < 0 || seg0 + (int64_t)sh.Hkv * nrows * sh.D > cap_elems) return;
  const int rpc = (nrows + nch - 1) / nch;
  const int r0 = ch * rpc, r1 = min(nrows, r0 + rpc);
  const size_t src_base = (size_t)(b * sh.Hkv + g) * sh.S * RB;
  const size_t dst_base = (size_t)seg0 * esize + (size_t)g * nrows * RB;
  const char *ks = static_cast<const char *>(tb.k.p[l]) + src_base;
  const char *vs = static_cast<const char *>(tb.v.p[l]) + src_base;
  char *kd = static_cast<char *>(tb.ko.p[l]) + dst_base;
  char *vd = static_cast<char *>(tb.vo.p[l]) + dst_base;
  const int32_t *kept = plan.kept + (size_t)lb * sh.Nv;
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
  size_t off_cnt, off_stats, off_e, ws_bytes;
  size_t elite_lds, score_lds, final_lds;
  int ktw;
};

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
  if (d->reserved != 0) return fail(AIRCACHE_EINVAL, "reserved field must be 0");
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
  s.cap = d->max_elite ? d->max_elite : d->n_txt;
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
  const int esz = d->dtype == AIRCACHE_BF16 ? 2 : 4;
  (void)esz;
  cfg->elite_lds = (size_t)17 * s.Nt * sizeof(float);
  cfg->score_lds = (size_t)s.cap * sizeof(int);
  cfg->final_lds = ((size_t)s.Hkv * s.rcap16 + s.Nv) * sizeof(float);
  if (cfg->elite_lds > kMaxLds) return fail(AIRCACHE_EINVAL, "n_txt=%d too large for the elite stage", s.Nt);
  if (cfg->score_lds > kMaxLds || cfg->final_lds > kMaxLds)
    return fail(AIRCACHE_EINVAL, "n_q_heads * max_elite too large (%lld rows); lower max_elite",
                (long long)s.Hq * s.cap);
  const size_t units = (size_t)s.L * s.B * s.Hkv;
  const size_t n_cnt = (size_t)s.L * s.B + s.B + 1;
  cfg->off_cnt = 0;
  cfg->off_stats = align_up(n_cnt * sizeof(unsigned));
  cfg->off_e = cfg->off_stats + align_up(units * s.rcap16 * s.ntiles * sizeof(float2));
  cfg->ws_bytes = cfg->off_e + align_up(units * s.Nv * (size_t)s.rcap16 * sizeof(float));
  return AIRCACHE_OK;
}

Ws ws_of(const Config &cfg, void *base) {
  char *p = static_cast<char *>(base);
  const Shape &s = cfg.sh;
  Ws w;
  w.cnt_lb = reinterpret_cast<unsigned *>(p + cfg.off_cnt);
  w.cnt_b = w.cnt_lb + (size_t)s.L * s.B;
  w.cnt_all = w.cnt_b + s.B;
  w.stats = reinterpret_cast<float2 *>(p + cfg.off_stats);
  w.e = reinterpret_cast<float *>(p + cfg.off_e);
  return w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_hip(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(AIRCACHE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return AIRCACHE_OK;
}

template <typename K> int allow_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return AIRCACHE_OK;
  return check_hip(hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes),
                   "hipFuncSetAttribute");
}

template <typename Tag, int D, int KTW>
int launch_plan(const Config &cfg, const LayerTable &qt, const LayerTable &kt, const PlanPtrs &pp, const Ws &ws,
                hipStream_t st) {
  const Shape &s = cfg.sh;
  int rc;
  if ((rc = allow_lds(elite_select_kernel<Tag, D>, cfg.elite_lds))) return rc;
  if ((rc = allow_lds(cross_score_kernel<Tag, D, KTW>, cfg.score_lds))) return rc;
  if ((rc = allow_lds(finalize_kernel, cfg.final_lds))) return rc;
  const unsigned nlb = (unsigned)(s.L * s.B);
  hipLaunchKernelGGL((elite_select_kernel<Tag, D>), dim3(nlb), dim3(256), cfg.elite_lds, st, s, qt, kt, pp, ws);
  if ((rc = check_hip(hipGetLastError(), "elite_select_kernel launch"))) return rc;
  hipLaunchKernelGGL((cross_score_kernel<Tag, D, KTW>), dim3(nlb * s.Hkv * s.ntiles), dim3(256), cfg.score_lds, st, s,
                     qt, kt, pp, ws);
  if ((rc = check_hip(hipGetLastError(), "cross_score_kernel launch"))) return rc;
  hipLaunchKernelGGL(finalize_kernel, dim3(nlb * s.ntiles), dim3(256), cfg.final_lds, st, s, pp, ws);
  if ((rc = check_hip(hipGetLastError(), "finalize_kernel launch"))) return rc;
  hipLaunchKernelGGL(topk_select_kernel, dim3(nlb), dim3(kTopkThreads), 0, st, s, pp);
  return check_hip(hipGetLastError(), "topk_select_kernel launch");
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
  return q;
}

int check_plan_buf(const aircache_plan_buf *p, bool for_compress) {
  if (!p) return fail(AIRCACHE_EINVAL, "plan is NULL");
  if (!p->budget || !p->out_off || !p->kept_idx) return fail(AIRCACHE_EINVAL, "plan budget/out_off/kept_idx NULL");
  if (for_compress) return AIRCACHE_OK;
  if (!p->elite_idx || !p->n_elite || !p->iv || !p->s_t || !p->s_k || !p->status)
    return fail(AIRCACHE_EINVAL, "a required plan output pointer is NULL");
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

}  // namespace aircache

using namespace aircache;

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

int aircache_plan(const aircache_desc *desc, const void *const *q_txt, const void *const *k,
                  const aircache_plan_buf *plan, void *workspace, size_t ws_bytes, void *stream) {
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  if ((rc = check_plan_buf(plan, false))) return rc;
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
  if (bf && cfg.sh.D == 128) return launch_plan<Bf16Tag, 128, 4>(cfg, qt, kt, pp, ws, st);
  if (bf && cfg.sh.D == 64) return launch_plan<Bf16Tag, 64, 4>(cfg, qt, kt, pp, ws, st);
  if (!bf && cfg.sh.D == 128) return launch_plan<F32Tag, 128, 2>(cfg, qt, kt, pp, ws, st);
  return launch_plan<F32Tag, 64, 2>(cfg, qt, kt, pp, ws, st);
}

int aircache_compress(const aircache_desc *desc, const aircache_plan_buf *plan, const void *const *k,
                      const void *const *v, void *const *k_out, void *const *v_out, void *stream) {
  Config cfg;
  int rc;
  if ((rc = make_config(desc, &cfg))) return rc;
  if ((rc = check_plan_buf(plan, true))) return rc;
  const Shape &s = cfg.sh;
  GatherTables tb;
  if ((rc = fill_table(k, s.L, &tb.k, "k"))) return rc;
  if ((rc = fill_table(v, s.L, &tb.v, "v"))) return rc;
  LayerTable ko, vo;
  if ((rc = fill_table(const_cast<const void *const *>(k_out), s.L, &ko, "k_out"))) return rc;
  if ((rc = fill_table(const_cast<const void *const *>(v_out), s.L, &vo, "v_out"))) return rc;
  const int esz = desc->dtype == AIRCACHE_BF16 ? 2 : 4;
  const size_t layer_in = (size_t)s.B * s.Hkv * s.S * s.D * esz;
  const size_t layer_out_max = (size_t)s.B * s.Hkv * s.S * s.D * esz;
  for (int l = 0; l < s.L; ++l) {
    tb.ko.p[l] = const_cast<void *>(ko.p[l]);
    tb.vo.p[l] = const_cast<void *>(vo.p[l]);
    const char *o[2] = {static_cast<const char *>(ko.p[l]), static_cast<const char *>(vo.p[l])};
    for (int a = 0; a < 2; ++a) {
      for (int m = 0; m < s.L; ++m) {
        const char *in[2] = {static_cast<const char *>(tb.k.p[m]), static_cast<const char *>(tb.v.p[m])};
        for (int c = 0; c < 2; ++c)
          if (o[a] < in[c] + layer_in && in[c] < o[a] + layer_out_max)
            return fail(AIRCACHE_EINVAL, "an output buffer of layer %d may overlap input layer %d", l, m);
      }
    }
  }
  for (int l = s.L; l < AIRCACHE_MAX_LAYERS; ++l) tb.ko.p[l] = tb.vo.p[l] = nullptr;
  const PlanPtrs pp = plan_ptrs(plan);
  hipStream_t st = static_cast<hipStream_t>(stream);
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
