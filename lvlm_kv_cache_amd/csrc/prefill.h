// Causal prefill attention of one layer, with the AirCache scores of the text
// rows taken from the same logits; included by aircache.hip inside namespace
// aircache.
//
// Attention: the KV-cache primer page (devpress.csdn.net), section 2.1
// "到底缓存什么？", the o_t equation at every position t of the regrouped
// sequence (visual tokens first, then text): position t attends to the keys
// 0..t, o_t = softmax(q_t K[0..t]^T / sqrt(D)) V[0..t], query head h on KV
// head h / G.
//
// Scores: the AirCache paper-notes page, "Elite Observation Window" (the
// A_vtk and I_v equations). An elite text row j normalises its logits over
// the N_v visual keys plus the elite text keys, with no causal mask. Its
// logits against the visual keys are the ones the prefill computes anyway
// (every text row sees every visual key), so a text workgroup writes, for
// each elite row and 64-key visual tile, exp2(s - m_t) of the tile's visual
// keys with m_t the running maximum of the attention at that tile, and after
// the last visual tile the row's normaliser (M, Z): the visual keys' running
// sum merged with the elite text keys' pair from a short extra product before
// the key loop. prefill_finalize_kernel weights the exponentials by
// exp2(m_t - M) / Z and sums the visual columns into I_v: the visual keys are
// read once, by the attention.
//
// Kernel shape (gfx950): a workgroup of 4 waves takes 128 query rows of one
// (sample, query head), 32 per wave as two 16-row MFMA blocks, and walks the
// key tiles of 64 keys up to its last row. S^T = K Q^T by
// v_mfma_f32_16x16x32_bf16 (keys as the A operand from an LDS tile staged by
// LDS-DMA, the wave's queries as the B operand in registers), so the result
// holds one query per lane column and the online softmax needs only a
// reduction over the four 16-lane rows. The key order inside a tile is
// permuted so that the probabilities of the lane's keys form, as they are,
// the B operand of O^T = V^T P^T; V is transposed on its way into LDS. Two
// buffers per operand: the next tile's loads are in flight during the
// current tile's products.
#pragma once

constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / 64;
constexpr int kPfRows = 32 * kPfWaves;  // query rows per workgroup at most (two 16-row blocks per wave)
constexpr int kPfKeys = 64;             // keys per tile
constexpr int kPfVtPad = 8;             // bf16 of padding per transposed V row (bank spread)

template <int D> struct PfLayout {
  static constexpr int kBlock = 16 * D * 2;                 // one 16-key block in fragment order
  static constexpr int kKTile = 4 * kBlock;                 // a 64-key K tile
  static constexpr int kVtRow = (kPfKeys + kPfVtPad) * 2;   // bytes of one transposed V row
  static constexpr int kVTile = D * kVtRow;                 // the 64-key V tile, transposed
  static constexpr int kBuf = kKTile + kVTile;
  static constexpr int kBytes = 2 * kBuf;                   // two buffers
};

struct PrefillArgs {
  const uint16_t *q;  // [B][Hq][S][D]
  const uint16_t *k;  // [B][Hkv][S][D]
  const uint16_t *v;
  uint16_t *o;        // [B][Hq][S][D]
  int nqt_vis, nqt_txt;  // query tiles per (sample, head) over the visual rows, the text rows
  int score;             // write the text rows' scoring terms
  int layer;
  const int32_t *elite, *n_elite;  // the layer's rows of the plan
  float *e;                        // [B][Hkv][rcap16][evs] exp2(s - m) of the elite rows (this layer)
  float2 *stats;                   // [B][Hkv][rcap16][nstat] per elite row: (m_t, 0) per visual tile, then (M, Z)
  int evs;                         // row stride of e: N_v rounded up to the key tile
  int nattn;                       // attention workgroups; the blocks after them finalize the previous layer
  const float *fin_e;              // the previous layer's scoring terms (the other workspace slot)
  const float2 *fin_stats;
  PlanPtrs plan;
  Ws ws;
};

// Position of key row m (0..15) of block kb (0..3) inside a 64-key tile: the
// lane of column n and row group grp then holds, in blocks 2s and 2s + 1, the
// logits of keys 32 s + 8 grp + 0..7, which is the B-operand fragment of slice s.
__device__ __forceinline__ int pf_key(int kb, int m) { return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3); }

__device__ __forceinline__ float max_across_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two floats to two bf16 (round to nearest even), packed low first.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// I_v and the statistics of one layer from the prefill's scoring terms (run
// by extra workgroups of the next layer's prefill_kernel, and for the last
// layer by prefill_finalize_kernel). One
// workgroup per (sample, KV head, 64-key column tile): the weight of each
// elite row r of the KV head for this tile is exp2(m_t - M) / Z, with m_t the
// reference of the tile's exponentials and (M, Z) the row's normaliser that
// the prefill wrote after its last visual tile; 4 x 64 threads sum the rows'
// weighted exponentials of the tile's columns into the KV head's part of I_v.
// The last workgroup of a (layer, sample) adds the parts in ascending KV-head
// order, divides by H_q N_tk (the I_v equation) and runs the statistics and
// budget finisher of the other paths.
constexpr int kPfFinThreads = 256;

// One finalize workgroup wg (0 .. B H_kv ntiles - 1) of the layer whose first
// (layer, sample) index is sh.lb0; wts: LDS of max(rcap16, N_v) floats.
__device__ void prefill_finalize_wg(const Shape &sh, const PlanPtrs &plan, const Ws &ws, const float *e,
                                    const float2 *stats, int evs, int wg, float *wts) {
  __shared__ float red[4][64];
  __shared__ int flag;
  const int tid = threadIdx.x;
  const int t = wg % sh.ntiles;
  const int bg = wg / sh.ntiles;  // b * H_kv + g
  const int g = bg % sh.Hkv, b = bg / sh.Hkv;
  const int lb = sh.lb0 + b;
  const int Nv = sh.Nv;
  int ntk = plan.n_elite[lb];
  ntk = ntk < 0 ? 0 : (ntk > sh.cap ? sh.cap : ntk);
  const int R = sh.G * ntk;
  for (int r = tid; r < R; r += kPfFinThreads) {
    const float2 *st = stats + ((size_t)bg * sh.rcap16 + r) * sh.nstat;
    const float2 mz = st[sh.ntiles];  // (M, Z) of the row
    wts[r] = exp2f(st[t].x - mz.x) / mz.y;
  }
  __syncthreads();
  const int cl = tid & 63, rg = tid >> 6;
  const int c = t * kPfKeys + cl;
  float acc = 0.f;
  if (c < Nv) {
    const float *eb = e + (size_t)bg * sh.rcap16 * evs + c;
    for (int r = rg; r < R; r += 4) acc += eb[(size_t)r * evs] * wts[r];
  }
  red[rg][cl] = acc;
  __syncthreads();
  float *part = ws.part + (size_t)b * sh.Hkv * Nv;
  if (tid < 64 && c < Nv) {
    const float ag = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    store_coherent(&part[(size_t)g * Nv + c], ag);
    if (sh.per_head) {
      const float inv_grp = (ntk > 0) ? 1.f / (float)(sh.G * ntk) : 0.f;
      plan.iv_head[((size_t)lb * sh.Hkv + g) * Nv + c] = ag * inv_grp;
    }
  }
  wait_all_memory();
  __syncthreads();
  if (tid == 0) flag = (counter_add(&ws.cnt_lb[lb], 1u) == (unsigned)(sh.Hkv * sh.ntiles) - 1u);
  __syncthreads();
  if (!flag) return;

  // last workgroup of (layer, sample): I_v = the KV heads' parts in ascending order
  const float inv_rows = (ntk > 0) ? 1.f / (float)(sh.Hq * ntk) : 0.f;
  float *ivc = wts;
  const auto rp = coherent_rsrc(part, (unsigned)((size_t)sh.Hkv * Nv * sizeof(float)));
  for (int cc = tid; cc < Nv; cc += kPfFinThreads) {
    float a = 0.f;
    for (int gg = 0; gg < sh.Hkv; ++gg) a += load_sc1_f(rp, (unsigned)(((size_t)gg * Nv + cc) * sizeof(float)));
    const float v = a * inv_rows;
    ivc[cc] = v;
    plan.iv[(size_t)lb * Nv + cc] = v;
  }
  __syncthreads();
  finish_layer_sample<kPfFinThreads>(sh, plan, ws, lb, ivc);
}

// The last layer's finalize (the others run inside the next layer's prefill_kernel).
__global__ __launch_bounds__(kPfFinThreads) void prefill_finalize_kernel(Shape sh, PlanPtrs plan, Ws ws,
                                                                         const float *e, const float2 *stats,
                                                                         int evs) {
  extern __shared__ float fin_wts[];
  prefill_finalize_wg(sh, plan, ws, e, stats, evs, blockIdx.x, fin_wts);
}

template <int D, bool SCORE, int NQB>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(Shape sh, PrefillArgs a) {
  using Lay = PfLayout<D>;
  constexpr int RPW = 16 * NQB;          // query rows per wave: NQB 16-row MFMA blocks
  constexpr int RW = RPW * kPfWaves;     // query rows per workgroup
  constexpr int NC = D / 32;  // 32-wide slices of the head dimension
  constexpr int ND = D / 16;  // 16-row blocks of O^T
  extern __shared__ __align__(16) unsigned char pf_lds[];
  __shared__ int emap[kPfRows];  // elite index of each text row of the tile, or -1
  // Block order: the attention (text tiles, then visual tiles from the
  // longest), then the previous layer's finalize workgroups, which take the
  // slots the shortest tiles leave (measured: 4% less for the fused layer
  // calls on workload 3 than placing them beside the text tiles).
  const int blk = (int)blockIdx.x;
  if (SCORE && blk >= a.nattn) {
    // the previous layer's I_v and statistics, from the other workspace slot
    Shape fs = sh;
    fs.lb0 = sh.lb0 - sh.B;
    prefill_finalize_wg(fs, a.plan, a.ws, a.fin_e, a.fin_stats, a.evs, blk - a.nattn,
                        reinterpret_cast<float *>(pf_lds));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int S = sh.S, Nv = sh.Nv;

  // Longest workgroups first: text tiles from the last, then visual tiles.
  const int bh = blk % (sh.B * sh.Hq), rank = blk / (sh.B * sh.Hq);
  const int b = bh / sh.Hq, h = bh - b * sh.Hq, g = h / sh.G, hl = h - g * sh.G;
  const bool text = rank < a.nqt_txt;
  const int qt = text ? a.nqt_txt - 1 - rank : a.nqt_vis - 1 - (rank - a.nqt_txt);
  const int row0 = text ? Nv + qt * RW : qt * RW;
  const int row1 = text ? min(S, row0 + RW) : min(Nv, row0 + RW);
  const int nkt = (row1 + kPfKeys - 1) / kPfKeys;

  const uint16_t *qh = a.q + (size_t)(b * sh.Hq + h) * S * D;
  const uint16_t *kh = a.k + (size_t)(b * sh.Hkv + g) * S * D;
  const uint16_t *vh = a.v + (size_t)(b * sh.Hkv + g) * S * D;

  // The wave's query fragments (rows beyond the tile are zero).
  Frag<Bf16Tag> qf[NQB][NC];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = row0 + RPW * wave + 16 * qb + n;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (row < row1) qf[qb][c].load(qh + (size_t)row * D + 32 * c + 8 * grp);
      else qf[qb][c].zero();
    }
  }

  // Scoring set-up: the elite index of each of the tile's text rows.
  const bool score = SCORE && text;
  const int lbl = b;  // (layer, sample) index inside this layer's workspace
  int ntk = 0;
  if (score) {
    ntk = a.n_elite[b];
    ntk = ntk < 0 ? 0 : (ntk > sh.cap ? sh.cap : ntk);
    for (int i = tid; i < RW; i += kPfThreads) emap[i] = -1;
    __syncthreads();
    const int jt0 = row0 - Nv;
    for (int e = tid; e < ntk; e += kPfThreads) {
      const int jt = a.elite[(size_t)b * sh.Nt + e] - jt0;
      if (jt >= 0 && jt < RW) emap[jt] = e;
    }
    __syncthreads();
  }
  int erow[NQB];  // elite row r = hl * ntk + eidx of the lane's queries, or -1
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) erow[qb] = -1;
  if (score) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int rr = RPW * wave + 16 * qb + n;
      const int e = (row0 + rr < row1) ? emap[rr] : -1;
      erow[qb] = e >= 0 ? hl * ntk + e : -1;
    }
  }
  float2 *st_base = a.stats + (size_t)(lbl * sh.Hkv + g) * sh.rcap16 * sh.nstat;
  float *e_row[NQB];  // the lane's elite rows of the exponentials
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
    e_row[qb] = a.e + ((size_t)(lbl * sh.Hkv + g) * sh.rcap16 + (erow[qb] >= 0 ? erow[qb] : 0)) * a.evs;

  // The elite text keys' (max, sum) for the elite rows: the columns the
  // scores add to the visual keys, with no causal mask. Merged with the
  // visual keys' running pair after the last visual tile.
  float xm[NQB], xz[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) xm[qb] = -INFINITY, xz[qb] = 0.f;
  if (score) {
    float mx[NQB], zx[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mx[qb] = -INFINITY, zx[qb] = 0.f;
    for (int x0 = 0; x0 < ntk; x0 += 16) {
      const int x = x0 + n;
      Frag<Bf16Tag> kx[NC];
      const int jt = x < ntk ? a.elite[(size_t)b * sh.Nt + x] : 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) kx[c].load(kh + (size_t)(Nv + jt) * D + 32 * c + 8 * grp);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) mfma_slice(acc, kx[c], qf[qb][c]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (x0 + 4 * grp + i < ntk) {
            const float v = acc[i] * sh.scale2;
            const float mn = fmaxf(mx[qb], v);
            zx[qb] = zx[qb] * exp2f(mx[qb] - mn) + exp2f(v - mn);
            mx[qb] = mn;
          }
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      xm[qb] = max_across_rows(mx[qb]);
      xz[qb] = sum_across_rows(mx[qb] > -INFINITY ? zx[qb] * exp2f(mx[qb] - xm[qb]) : 0.f);
    }
  }

  unsigned char *buf0 = pf_lds;
  const int kq = tid & 15, dq = tid >> 4;  // V staging: keys 4 kq .. 4 kq + 3, elements 8 dq .. 8 dq + 7
  constexpr bool kAllStage = 16 * (D / 8) >= kPfThreads;  // every thread stages (head_dim 128)
  const bool vstage = kAllStage || dq < D / 8;

  auto issue_k = [&](int kt, unsigned char *kbuf) {
    const int key = min(kt * kPfKeys + pf_key(wave, n), S - 1);
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kh + (size_t)key * D) + 16 * grp;
    unsigned char *dst = kbuf + wave * Lay::kBlock;
#pragma unroll
    for (int j = 0; j < NC; ++j) load_lds16(src + 64 * j, dst + 1024 * j);
  };
  u32x4_t vr[4];
  auto load_v = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(kt * kPfKeys + 4 * kq + i, S - 1);
      vr[i] = vstage ? *reinterpret_cast<const u32x4_t *>(vh + (size_t)key * D + 8 * dq) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_vt = [&](unsigned char *vt) {
    if (!vstage) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sh16 = 16 * (j & 1);
      const unsigned x0 = (vr[0][j >> 1] >> sh16) & 0xffffu, x1 = (vr[1][j >> 1] >> sh16) & 0xffffu;
      const unsigned x2 = (vr[2][j >> 1] >> sh16) & 0xffffu, x3 = (vr[3][j >> 1] >> sh16) & 0xffffu;
      uint2 w;
      w.x = x0 | (x1 << 16);
      w.y = x2 | (x3 << 16);
      *reinterpret_cast<uint2 *>(vt + (size_t)(8 * dq + j) * Lay::kVtRow + 8 * kq) = w;
    }
  };

  f32x4_t oacc[ND][NQB];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) oacc[d][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun[NQB], lrun[NQB];
  float zrun[NQB];  // the lane's part of the scores' running sum over visual keys (reference as lrun)
  int qrow[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    qrow[qb] = row0 + RPW * wave + 16 * qb + n;
    mrun[qb] = -INFINITY;
    lrun[qb] = 0.f;
    zrun[qb] = 0.f;
  }

  // prologue: tile 0 into buffer 0
  load_v(0);
  issue_k(0, buf0);
  wait_vmcnt<0>();
  store_vt(buf0 + Lay::kKTile);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    unsigned char *cur = buf0 + (kt & 1) * Lay::kBuf;
    unsigned char *nxt = buf0 + ((kt + 1) & 1) * Lay::kBuf;
    const bool more = kt + 1 < nkt;
    if (more) {
      load_v(kt + 1);
      issue_k(kt + 1, nxt);
    }
    const int key0 = kt * kPfKeys;

    // S^T = K Q^T: four key blocks, two query blocks
    f32x4_t s[4][NQB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Frag<Bf16Tag> kf;
        LdsTile<Bf16Tag>::read(kf, cur + kb * Lay::kBlock, c, lane);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) mfma_slice(s[kb][qb], kf, qf[qb][c]);
      }
    }

    // causal mask (only tiles that reach past the wave's first row), online softmax
    const bool diag = key0 + kPfKeys - 1 > row0 + RPW * wave;
    if (diag) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + pf_key(kb, 4 * grp + i) > qrow[qb]) s[kb][qb][i] = -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // the scale 1/sqrt(D) (base 2) is applied after the maximum and inside
      // the exponent; exp2 of -inf (masked keys) is 0
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = max_across_rows(mx) * sh.scale2;
      const float mnew = fmaxf(mrun[qb], mx);
      const float alpha = __builtin_amdgcn_exp2f(mrun[qb] - mnew);
      mrun[qb] = mnew;
      float ls = 0.f, zv = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][i], sh.scale2, -mnew));
          s[kb][qb][i] = p;
          ls += p;
        }
      lrun[qb] = lrun[qb] * alpha + ls;
      if (__ballot(alpha != 1.f)) {  // the maximum moved for some row of the wave
#pragma unroll
        for (int d = 0; d < ND; ++d) oacc[d][qb] *= alpha;
      }
      if (score && key0 < Nv) {
        // the tile's visual keys for the elite rows: the reference m_t, the
        // exponentials as two runs of 8 keys per lane (keys past N_v land in
        // the row's padding and are never read), and the lane's part of the
        // running visual sum (the tile's sum ls when every key is visual)
        if (key0 + kPfKeys > Nv) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key0 + pf_key(kb, 4 * grp + i) < Nv) zv += s[kb][qb][i];
        } else {
          zv = ls;
        }
        zrun[qb] = zrun[qb] * alpha + zv;
        if (erow[qb] >= 0) {
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) {
            f32x4_t *dst = reinterpret_cast<f32x4_t *>(e_row[qb] + key0 + 32 * sl + 8 * grp);
            dst[0] = s[2 * sl][qb];
            dst[1] = s[2 * sl + 1][qb];
          }
          if (grp == 0) st_base[(size_t)erow[qb] * sh.nstat + kt] = make_float2(mnew, 0.f);
        }
        if (kt == sh.ntiles - 1) {
          // the row's normaliser: the visual keys' running sum (the four
          // lane rows added) and the elite text keys' pair
          const float zvis = sum_across_rows(zrun[qb]);
          const float M = fmaxf(mnew, xm[qb]);
          const float Z = zvis * exp2f(mnew - M) + (xm[qb] > -INFINITY ? xz[qb] * exp2f(xm[qb] - M) : 0.f);
          if (grp == 0 && erow[qb] >= 0) st_base[(size_t)erow[qb] * sh.nstat + sh.ntiles] = make_float2(M, Z);
        }
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      Frag<Bf16Tag> pf[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        u32x4_t w;
        w[0] = pack_bf16(s[2 * sl][qb][0], s[2 * sl][qb][1]);
        w[1] = pack_bf16(s[2 * sl][qb][2], s[2 * sl][qb][3]);
        w[2] = pack_bf16(s[2 * sl + 1][qb][0], s[2 * sl + 1][qb][1]);
        w[3] = pack_bf16(s[2 * sl + 1][qb][2], s[2 * sl + 1][qb][3]);
        pf[qb].v = __builtin_bit_cast(u16x8_t, w);
      }
      const unsigned char *vt = cur + Lay::kKTile + 2 * (32 * sl + 8 * grp);
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        Frag<Bf16Tag> vf;
        vf.v = *reinterpret_cast<const u16x8_t *>(vt + (size_t)(16 * d + n) * Lay::kVtRow);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) mfma_slice(oacc[d][qb], vf, pf[qb]);
      }
    }

    if (more) {
      wait_vmcnt<NC>();  // this wave's V loads (issued before its K tile DMAs)
      store_vt(nxt + Lay::kKTile);
      wait_vmcnt<0>();
    }
    __syncthreads();
  }

  // O = O^T / l, rounded to bf16: the lane writes 4 consecutive elements of
  // its query row per 16-row block of O^T.
  uint16_t *oh = a.o + (size_t)(b * sh.Hq + h) * S * D;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float inv = 1.f / sum_across_rows(lrun[qb]);
    if (qrow[qb] < row1) {
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        uint2 w;
        w.x = pack_bf16(oacc[d][qb][0] * inv, oacc[d][qb][1] * inv);
        w.y = pack_bf16(oacc[d][qb][2] * inv, oacc[d][qb][3] * inv);
        *reinterpret_cast<uint2 *>(oh + (size_t)qrow[qb] * D + 16 * d + 4 * grp) = w;
      }
    }
  }
}
