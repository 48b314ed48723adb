// The whole pass for small shapes in one workgroup, included by aircache.hip
// inside namespace aircache (after pass_chunked.h, whose budget helpers it
// uses).
//
// Method: the AirCache paper-notes page, "Elite Observation Window" (the Att,
// k, A_vtk and I_v equations), "Layer-wise KV Cache Budget Allocation" (the
// s_t, s_k and r_hat equations) and the training-free procedure (budgets for
// all layers of a sample at once, then selection and compaction).
//
// When one sample's keys and text queries over all layers fit in LDS, the
// grid-wide schedule and the record round trips of the one-launch kernel cost
// more than the work. Here one 512-thread workgroup takes the samples in
// order. Per sample: LDS-DMA stages K and the text Q of every layer (one round
// trip); each wave then takes whole layers (l, l + W, ...) with no barrier
// inside a layer: elite set, I_v (elite rows in order, each row's softmax over
// the visual and elite text keys by lanes over columns), s_t and s_k in double
// precision; one barrier; the sample's budgets; each wave the top-r_hat of its
// layers (a direct rank in the order score descending, index ascending); one
// barrier; the compaction, one (layer, K or V, KV head) segment per wave.
#pragma once

typedef __attribute__((ext_vector_type(2))) unsigned long long u64x2_t;

constexpr int kSmallThreads = 512;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallMaxNv = 512;   // the direct rank's N_v^2 / 64 compares per lane
constexpr int kSmallMaxZ = 8192;   // H_q * N_t logits of the elite step
constexpr int kSmallMaxLayers = 51;
constexpr int kSmallKeep = 4;      // logits of one I_v row kept in registers per lane (columns lane + 64 k)

// Dynamic LDS (byte offsets). Region A: the sample's keys [L][H_kv][S][D] and
// text queries [L][H_q][N_t][D] as stored, each layer's block padded to 1 KB
// (whole LDS-DMA instructions); after the scoring the same bytes hold the
// waves' rank keys [W][N_v rounded up to 64]. Per wave: elite logits
// [H_q][N_t], head maxima and inverse sums [2][H_q], the elite list [N_t].
// Then I_v [L][nsel][N_v] (per KV head with one selection per KV head; then
// the kept indices), statistics [L + 16] doubles x 2,
// budgets [L + 16], layer offsets [L] and the five layer pointer tables
// [5 L].
struct SmallLds {
  int waves;         // W: waves with layer work
  int kpad, qpad;    // bytes of one layer's K, Q block
  int kall, qall, keys, z, hm, el, ivl, st, bud, off, ptr, total;
};
__host__ __device__ inline SmallLds small_lds_layout(int L, int Hq, int Hkv, int D, int Nv, int Nt, int esize,
                                                     int W, int nsel) {
  SmallLds f;
  long long o = 0;
  auto take = [&](long long bytes) {
    const long long at = o;
    o += (bytes + 15) & ~15LL;
    return (int)(at < (1LL << 30) ? at : (1LL << 30));
  };
  const long long kpad = ((long long)Hkv * (Nv + Nt) * D * esize + 1023) / 1024 * 1024;
  const long long qpad = ((long long)Hq * Nt * D * esize + 1023) / 1024 * 1024;
  const long long nk = (Nv + 63) / 64 * 64;
  f.waves = W;
  f.kpad = (int)(kpad < (1LL << 30) ? kpad : (1LL << 30));
  f.qpad = (int)(qpad < (1LL << 30) ? qpad : (1LL << 30));
  const long long data = (long long)L * (kpad + qpad), rank = (long long)W * nk * 8;
  f.kall = f.keys = take(data > rank ? data : rank);
  f.qall = f.kall + (int)((long long)L * kpad < (1LL << 30) ? (long long)L * kpad : (1LL << 30));
  f.z = take((long long)W * Hq * Nt * 4);
  f.hm = take((long long)W * Hq * 8);
  f.el = take((long long)W * Nt * 4);
  f.ivl = take((long long)L * nsel * Nv * 4);
  f.st = take((L + 16) * 8 * 2);
  f.bud = take((L + 16) * 4);
  f.off = take(L * 8);
  f.ptr = take(5 * L * 8);
  f.total = (int)(o < (1LL << 30) ? o : (1LL << 30));
  return f;
}

// 16-byte global load and non-temporal store through global (not flat)
// pointers: flat operations also count as LDS operations, so every wait for
// an LDS read would wait for them too.
typedef __attribute__((address_space(1))) u32x4_t small_g16_t;
__device__ __forceinline__ u32x4_t small_load16(const char *p) {
  return *(const small_g16_t *)(const void *)p;
}
__device__ __forceinline__ void small_store16_nt(char *p, u32x4_t v) {
  __builtin_nontemporal_store(v, (small_g16_t *)(void *)p);
}

// Orders the memory operations of a wave's lanes around it (lanes of one
// wave exchange values through LDS between the steps of a layer).
__device__ __forceinline__ void small_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Dot product of two rows of D elements held in LDS, read in 16-byte pieces
// starting at piece rot (mod the row's pieces): rows of one stride are then
// read by the lanes of a wave from distinct banks. Four partial sums (one per
// element of a piece) keep the multiply-add chains short; they are added at
// the end as (s0 + s1) + (s2 + s3).
template <typename Tag, int D> struct SmallDot;
template <int D> struct SmallDot<F32Tag, D> {
  __device__ static __forceinline__ float run(const unsigned char *a, const unsigned char *b, int rot) {
    constexpr int P = D / 4;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 8
    for (int w = 0; w < P; ++w) {
      const int i = (w + rot) & (P - 1);
      const f32x4_t x = *reinterpret_cast<const f32x4_t *>(a + 16 * i);
      const f32x4_t y = *reinterpret_cast<const f32x4_t *>(b + 16 * i);
      s0 += x[0] * y[0];
      s1 += x[1] * y[1];
      s2 += x[2] * y[2];
      s3 += x[3] * y[3];
    }
    return (s0 + s1) + (s2 + s3);
  }
};
template <int D> struct SmallDot<Bf16Tag, D> {
  __device__ static __forceinline__ float run(const unsigned char *a, const unsigned char *b, int rot) {
    constexpr int P = D / 8;
    float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int w = 0; w < P; ++w) {
      const int i = (w + rot) & (P - 1);
      const u32x4_t x = *reinterpret_cast<const u32x4_t *>(a + 16 * i);
      const u32x4_t y = *reinterpret_cast<const u32x4_t *>(b + 16 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sp[e] += __uint_as_float(x[e] << 16) * __uint_as_float(y[e] << 16);
        sp[e] += __uint_as_float(x[e] & 0xffff0000u) * __uint_as_float(y[e] & 0xffff0000u);
      }
    }
    return (sp[0] + sp[1]) + (sp[2] + sp[3]);
  }
};

template <typename Tag, int D>
__global__ __launch_bounds__(kSmallThreads) void aircache_small_kernel(Shape sh, PassTables tab, PlanPtrs plan,
                                                                        int gather, int64_t cap_elems,
                                                                        SmallLds lo) {
  using E = typename Tag::store_t;
  using Dot = SmallDot<Tag, D>;
  constexpr int ES = (int)sizeof(E);
  constexpr int RB = D * ES;  // bytes of one row
  extern __shared__ __attribute__((aligned(16))) float small_lds_f[];
  unsigned char *lds = reinterpret_cast<unsigned char *>(small_lds_f);
  __shared__ int flags;  // AIRCACHE_DEV_* bits found by any wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = sh.L, B = sh.B, Hq = sh.Hq, Hkv = sh.Hkv, G = sh.G, Nv = sh.Nv, Nt = sh.Nt, S = sh.S;
  const int W = lo.waves, nk = (Nv + 63) / 64 * 64;
  float *ivl = reinterpret_cast<float *>(lds + lo.ivl);  // [L][nsel][N_v]; then the kept indices
  const int nsel = sh.nsel;
  double *st = reinterpret_cast<double *>(lds + lo.st);
  double *sk = st + (L + 16);
  int *bud = reinterpret_cast<int *>(lds + lo.bud);
  int64_t *loff = reinterpret_cast<int64_t *>(lds + lo.off);
  const char **ptr = reinterpret_cast<const char **>(lds + lo.ptr);  // [5][L]: Q, K, V, K out, V out
  const size_t kbytes = (size_t)Hkv * S * RB, qbytes = (size_t)Hq * Nt * RB;
  constexpr int pieces = RB / 16;
  if (tid == 0) flags = 0;
  for (int l = tid; l < L; l += kSmallThreads) loff[l] = 0;

  for (int b = 0; b < B; ++b) {
    // K and the text Q of every layer into LDS: whole 1 KB DMA blocks, wave w
    // taking blocks w, w + 8, ... (tail lanes read the block's last piece
    // again, into the layer's padding)
    __syncthreads();
    for (int l = 0; l < L; ++l) {
      const char *kg = static_cast<const char *>(tab.p[L + l]) + b * kbytes;
      const char *qg = static_cast<const char *>(tab.p[l]) + b * qbytes;
      const int kblk = (int)((kbytes + 1023) / 1024), qblk = (int)((qbytes + 1023) / 1024);
      for (int c = wave; c < kblk + qblk; c += kSmallWaves) {
        const bool isk = c < kblk;
        const size_t at = (size_t)(isk ? c : c - kblk) * 1024 + 16 * lane, nb = isk ? kbytes : qbytes;
        const char *src = (isk ? kg : qg) + (at < nb ? at : nb - 16);
        load_lds16(src, lds + (isk ? lo.kall + (size_t)l * lo.kpad + (size_t)c * 1024
                                   : lo.qall + (size_t)l * lo.qpad + (size_t)(c - kblk) * 1024));
      }
    }
    // the pointer tables, read while the first blocks are in flight
    if (b == 0)
      for (int i = tid; i < 5 * L; i += kSmallThreads) ptr[i] = static_cast<const char *>(tab.p[i]);
    wait_vmcnt<0>();
    __syncthreads();

    // per layer, one wave, no barrier: elite set, I_v, s_t and s_k
    if (wave < W) {
      float *z = reinterpret_cast<float *>(lds + lo.z) + (size_t)wave * Hq * Nt;   // [H_q][N_t]
      float *hm = reinterpret_cast<float *>(lds + lo.hm) + (size_t)wave * Hq * 2;  // maxima, inverse sums
      int *el = reinterpret_cast<int *>(lds + lo.el) + (size_t)wave * Nt;
      for (int l = wave; l < L; l += W) {
        const int plb = l * B + b;
        const unsigned char *kb = lds + lo.kall + (size_t)l * lo.kpad;  // [H_kv][S][D]
        const unsigned char *qb = lds + lo.qall + (size_t)l * lo.qpad;  // [H_q][N_t][D]
        // 1. the last text query's logits over the text keys, per head
        for (int x = lane; x < Hq * Nt; x += 64) {
          const int h = x / Nt, j = x - (x / Nt) * Nt, g = h / G;
          z[x] = Dot::run(qb + ((size_t)h * Nt + (Nt - 1)) * RB, kb + ((size_t)g * S + Nv + j) * RB, x) * sh.scale2;
        }
        small_wave_sync();
        for (int h = 0; h < Hq; ++h) {
          const float *zr = z + (size_t)h * Nt;
          float m = -INFINITY;
          for (int j = lane; j < Nt; j += 64) m = fmaxf(m, zr[j]);
          m = wave_max(m);
          float s = 0.f;
          for (int j = lane; j < Nt; j += 64) s += exp2f(zr[j] - m);
          s = wave_sum(s);
          if (lane == 0) {
            hm[2 * h] = m;
            hm[2 * h + 1] = 1.f / s;
          }
        }
        small_wave_sync();
        // p_bar_j: the heads' softmax weights summed in head order (the
        // threshold is relative, so the mean's 1 / H_q does not matter)
        float mx = 0.f;
        for (int j = lane; j < Nt; j += 64) {
          float a = 0.f;
          for (int h = 0; h < Hq; ++h) a += exp2f(z[(size_t)h * Nt + j] - hm[2 * h]) * hm[2 * h + 1];
          z[j] = a;  // row 0 is free: each lane rewrites only its own j
          mx = fmaxf(mx, a);
        }
        mx = wave_max(mx);
        small_wave_sync();
        const float thr = sh.alpha * mx;
        int total = 0;
        for (int j0 = 0; j0 < Nt; j0 += 64) {
          const int j = j0 + lane;
          const bool in = j < Nt && (sh.window > 0 ? j >= Nt - sh.window : z[j] >= thr);
          const unsigned long long bal = __ballot(in);
          if (in) {
            const int pos = total + __popcll(bal & ((1ull << lane) - 1ull));
            plan.elite[(size_t)plb * Nt + pos] = j;
            if (pos < sh.cap) el[pos] = j;
          }
          total += __popcll(bal);
        }
        if (lane == 0) plan.n_elite[plb] = total;
        if (total > sh.cap && lane == 0) atomicOr(&flags, AIRCACHE_DEV_ELITE_OVERFLOW);
        const int ntk = total < sh.cap ? total : sh.cap;
        small_wave_sync();
        // 2. I_v: the elite rows in order (head, then elite token); each row's
        // softmax over the visual and elite text keys, lanes over columns
        // (one accumulator per KV head with one selection per KV head)
        float *ivs = ivl + (size_t)l * nsel * Nv;
        for (int c = lane; c < nsel * Nv; c += 64) ivs[c] = 0.f;
        small_wave_sync();  // (zeroed by other lanes than those that add to them)
        const int ncols = Nv + ntk;
        for (int row = 0; row < Hq * ntk; ++row) {
          const int h = row / ntk, e = row - (row / ntk) * ntk, g = h / G;
          float *iv = ivs + (size_t)(nsel > 1 ? g : 0) * Nv;
          const unsigned char *qr = qb + ((size_t)h * Nt + el[e]) * RB;
          const unsigned char *kg = kb + (size_t)g * S * RB;
          // pass 1: the row's logits (the first kSmallKeep per lane kept in
          // registers), maximum and sum
          float tk[kSmallKeep];
#pragma unroll
          for (int k = 0; k < kSmallKeep; ++k) {
            const int c = lane + 64 * k;
            const int et = el[c - Nv > 0 ? (c - Nv < ntk ? c - Nv : ntk - 1) : 0];
            const int key = c < Nv ? c : Nv + et;
            tk[k] = c < ncols ? Dot::run(qr, kg + (size_t)key * RB, lane) * sh.scale2 : -INFINITY;
          }
          float m = -INFINITY;
#pragma unroll
          for (int k = 0; k < kSmallKeep; ++k) m = fmaxf(m, tk[k]);
          float sum = 0.f;
#pragma unroll
          for (int k = 0; k < kSmallKeep; ++k) sum += tk[k] > -INFINITY ? exp2f(tk[k] - m) : 0.f;
          for (int c = lane + 64 * kSmallKeep; c < ncols; c += 64) {
            const int et = el[c - Nv > 0 ? c - Nv : 0];
            const int key = c < Nv ? c : Nv + et;
            const float t = Dot::run(qr, kg + (size_t)key * RB, lane) * sh.scale2;
            const float mn = fmaxf(m, t);
            sum = sum * exp2f(m - mn) + exp2f(t - mn);
            m = mn;
          }
          const float M = wave_max(m);
          const float inv = 1.f / wave_sum(m > -INFINITY ? sum * exp2f(m - M) : 0.f);
          // pass 2: the visual columns' weights, accumulated per wave
#pragma unroll
          for (int k = 0; k < kSmallKeep; ++k) {
            const int c = lane + 64 * k;
            if (c < Nv) iv[c] += exp2f(tk[k] - M) * inv;
          }
          for (int c = lane + 64 * kSmallKeep; c < Nv; c += 64)
            iv[c] += exp2f(Dot::run(qr, kg + (size_t)c * RB, lane) * sh.scale2 - M) * inv;
        }
        // 3. the mean over the rows (over all query heads; per KV head too
        // with one selection per KV head); s_t, then s_k (sample standard
        // deviation, adjusted skewness), in double precision
        const float inv_rows = ntk > 0 ? 1.f / (float)(Hq * ntk) : 0.f;
        const float inv_grp = ntk > 0 ? 1.f / (float)(G * ntk) : 0.f;
        float av[kSmallMaxNv / 64];  // the lane's columns lane + 64 k
        double sum = 0.0;
#pragma unroll
        for (int k = 0; k < kSmallMaxNv / 64; ++k) {
          const int c = lane + 64 * k;
          av[k] = 0.f;
          if (c < Nv) {
            float t = 0.f;
            for (int g = 0; g < nsel; ++g) {
              const float ag = ivs[(size_t)g * Nv + c];
              t += ag;
              if (sh.per_head) {
                ivs[(size_t)g * Nv + c] = ag * inv_grp;
                plan.iv_head[((size_t)plb * nsel + g) * Nv + c] = ag * inv_grp;
              }
            }
            const float a = t * inv_rows;
            if (!sh.per_head) ivs[c] = a;
            av[k] = a;
            plan.iv[(size_t)plb * Nv + c] = a;
            sum += (double)a;
          }
        }
        sum = wave_sum_d(sum);
        const double mean = sum / (double)Nv;
        double m2 = 0.0, m3 = 0.0;
#pragma unroll
        for (int k = 0; k < kSmallMaxNv / 64; ++k)
          if (lane + 64 * k < Nv) {
            const double dd = (double)av[k] - mean;
            m2 += dd * dd;
            m3 += dd * dd * dd;
          }
        m2 = wave_sum_d(m2);
        m3 = wave_sum_d(m3);
        if (lane == 0) {
          const double sigma = sqrt(m2 / (double)(Nv - 1));
          st[l] = sum;
          sk[l] = sigma > 0.0 ? (m3 / (sigma * sigma * sigma)) * ((double)Nv / ((double)(Nv - 1) * (double)(Nv - 2)))
                              : 0.0;
        }
        small_wave_sync();
      }
    }
    // 4. the sample's budgets (double precision, the host rule's order)
    __syncthreads();
    if (tid < 16) {
      st[L + tid] = 0.0;
      sk[L + tid] = 0.0;
    }
    __syncthreads();
    if (wave == 0) {
      const BudgetSums sums = L <= 64 ? budget_sums_wave(L, st, sk) : budget_sums_lds(L, st, sk);
      for (int l = lane; l < L; l += 64) {
        double x;
        int r;
        layer_budget(sh, sums, l, st[l], sk[l], &x, &r);
        const int plb = l * B + b;
        bud[l] = r;
        plan.s_t[plb] = st[l];
        plan.s_k[plb] = sk[l];
        plan.budget[plb] = r;
        if (plan.bx) plan.bx[plb] = x;
        plan.out_off[(size_t)l * (B + 1) + b] = loff[l];
      }
    }
    __syncthreads();
    // 5. per layer, one wave: top-r_hat by direct rank. key = (score bits,
    // 65535 - index) orders as (score descending, index ascending) when
    // compared as integers (the scores are non-negative, so their bits order
    // as the values); the rank is the count of larger keys. Then the kept
    // indices ascending (over I_v of the layer, which the keys replace).
    if (wave < W) {
      uint64_t *keys = reinterpret_cast<uint64_t *>(lds + lo.keys) + (size_t)wave * nk;
      for (int ls = wave; ls < L * nsel; ls += W) {
        // (layer, selection): one per layer, or one per KV head of it
        const int l = ls / nsel, gs = ls - l * nsel;
        const int plb = l * B + b, rb = bud[l];
        float *iv = ivl + (size_t)ls * Nv;
        for (int i = lane; i < nk; i += 64)
          keys[i] = i < Nv ? ((uint64_t)__float_as_uint(iv[i]) << 16) | (uint64_t)(65535 - i) : 0ull;
        small_wave_sync();
        unsigned kept = 0;  // bit k: index lane + 64 k kept
        for (int k = 0; k < nk / 64; ++k) {
          const uint64_t ki = keys[lane + 64 * k];
          int rank = 0;
#pragma unroll 8
          for (int j = 0; j < nk; j += 2) {
            const u64x2_t kj = *reinterpret_cast<const u64x2_t *>(keys + j);
            rank += (kj[0] > ki) + (kj[1] > ki);
          }
          if (lane + 64 * k < Nv && rank < rb) kept |= 1u << k;
        }
        int *kidx = reinterpret_cast<int *>(iv);
        small_wave_sync();
        int done = 0;
        for (int k = 0; k < nk / 64; ++k) {
          const bool in = (kept >> k) & 1u;
          const unsigned long long bal = __ballot(in);
          if (in) {
            const int pos = done + __popcll(bal & ((1ull << lane) - 1ull));
            plan.kept[((size_t)plb * nsel + gs) * Nv + pos] = lane + 64 * k;
            kidx[pos] = lane + 64 * k;
          }
          done += __popcll(bal);
        }
        small_wave_sync();
      }
    }
    // 6. the compaction: segments (layer, K or V, KV head), wave w taking
    // segments w, w + 8, ...; per segment the kept visual rows, then the text
    // rows, from global memory. Per batch sixteen loads per lane issued
    // (clamped indices, no branch) before the stores, every address computed
    // before the first store (a branch around a load or store makes the
    // compiler wait for it alone); lanes past the end store the last piece
    // again, with the same bytes as the lane that owns it.
    __syncthreads();
    for (int sg = wave; sg < L * 2 * Hkv; sg += kSmallWaves) {
      const int l = sg / (2 * Hkv), rem = sg - l * (2 * Hkv), kv = rem / Hkv, g = rem - kv * Hkv;
      const int rb = bud[l], nl = rb + Nt, np = nl * pieces;
      if (!gather || loff[l] + (int64_t)Hkv * nl * D > cap_elems) continue;
      const int *kidx = reinterpret_cast<const int *>(ivl + ((size_t)l * nsel + (nsel > 1 ? g : 0)) * Nv);
      const char *src = ptr[(1 + kv) * L + l] + b * kbytes + (size_t)g * S * RB;
      char *dst = const_cast<char *>(ptr[(3 + kv) * L + l]) + (size_t)loff[l] * ES + (size_t)g * nl * RB;
      constexpr int U = 16;
      for (int q0 = 0; q0 < np; q0 += 64 * U) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int qu = q0 + 64 * u + lane, q = qu < np ? qu : np - 1;
          const int i = q / pieces, pc = q - (q / pieces) * pieces;
          const int ki = kidx[i < rb ? i : (rb > 0 ? rb - 1 : 0)];
          const int row = i < rb ? ki : Nv + (i - rb);
          v[u] = small_load16(src + (size_t)row * RB + 16 * pc);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int qu = q0 + 64 * u + lane, q = qu < np ? qu : np - 1;
          small_store16_nt(dst + (size_t)q * 16, v[u]);
        }
      }
    }
    __syncthreads();
    for (int l = tid; l < L; l += kSmallThreads) {
      loff[l] += (int64_t)Hkv * (bud[l] + Nt) * D;
      if (b == B - 1) plan.out_off[(size_t)l * (B + 1) + B] = loff[l];
    }
  }
  __syncthreads();
  if (tid == 0) *plan.status = flags;
}
