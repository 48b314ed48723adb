// The whole AirCache pass in one persistent launch (the "chunked" path),
// included by aircache.hip inside namespace aircache.
//
// Method: paper-notes page "AirCache: Activating Inter-Modal Relevancy KV
// Cache Compression for Efficient Large Vision-Language Model Inference",
// "Elite Observation Window" (the Att, k, A_vtk and I_v equations),
// "Layer-wise KV Cache Budget Allocation" (the s_t, s_k and r_hat equations)
// and the training-free procedure (budgets for all layers at once after
// prefill, then compression).
//
// Schedule. Everything a workgroup does is fixed by the shape alone, so no
// step waits for a schedule worked out from the elite counts, and the key
// tiles of a workgroup's first item are loaded into its LDS at launch:
//   - elite workgroups [0, E): one part of the elite window each (the text
//     softmax rows of the last text query of a group of KV heads of one
//     (layer, sample)); the workgroup of part 0 adds the others' parts and
//     publishes the elite set (size and one bit mask per 64 text tokens);
//   - items: (layer, sample, chunk of `width` visual keys), every KV head of
//     it. Round 0 runs on workgroups [E, P) while the elite sets form, rounds
//     1, 2, ... on all workgroups; every chunk of a (layer, sample) falls in
//     the same round on a workgroup of its own, so the chunks of a pair run
//     together. An item streams its keys a head group (up to eight KV heads,
//     one per wave group) at a time and, per head group, takes the elite
//     query rows in passes of up to RTP 16-row tiles; the keys stay in LDS
//     across the passes of one head group. Logits stay in registers. The
//     exact softmax normaliser of a row needs every chunk of the row's
//     (layer, sample): each pass publishes the chunk's (max, sum) per row and
//     merges every chunk's pair in chunk order. The elite text keys enter the
//     rows' normalisers through chunk 0 and never the column sums. The
//     chunk's I_v and its moments (sum, M2, M3, count) go out as records;
//   - consumer units (layer, sample, KV head, K or V), a contiguous range per
//     workgroup: each combines the chunk moments of every layer of its sample
//     into s_t and s_k, computes the budgets, selects its layer's top-r_hat
//     from the published I_v and copies its rows (the kept visual rows, then
//     the text rows) into the compacted cache. Without compaction a unit is a
//     (layer, sample).
//
// Records: every cross-workgroup value is a 64-bit word (32-bit payload | tag
// << 32) written with an agent-coherent store; a reader that sees the
// expected tag has the payload. Tags are the call's epoch (the workspace's
// call count + 1, never 0), or, for the row normaliser records, which reuse
// two slots in turn (pass p in slot p % 2), ((epoch mod 2^21) + 1) * 1024 + p.
// A reader of pass p can then only take pass p's record: pass p - 2 of the
// same call has another tag, and a writer reaches pass p + 2 only after every
// chunk has published pass p + 1, which each does after reading pass p. So
// that no record older than 2^21 calls can carry a current tag, the call
// whose epoch is a multiple of 2^21 first zeroes every record (all workgroups,
// then a barrier over the grid). The last workgroup to finish writes the
// call's status, resets the counters and advances the epoch.
//
// Progress: all workgroups are resident at once (one per CU). Items wait only
// for items of their own round (which every workgroup reaches, rounds being
// taken in order) and for elite sets (published by elite workgroups before
// any item of theirs); consumer units wait only for item records and for the
// budgets of earlier samples, which the first unit of each sample publishes
// before its own top-k. Every wait is also bounded: on expiry the kernel
// flags AIRCACHE_DEV_TIMEOUT and every other wait of the launch gives up.
//
// LDS-DMA and polling: a wave's vector-memory operations complete in issue
// order, so a poll issued behind a wave's key-tile loads would wait for them.
// Waves 0 and 1 (the poll waves) therefore issue no tile loads: waves 2 and 3
// load their ring slots besides their own, and every poll of a record is made
// by wave 0 or 1.
#pragma once

constexpr int kPassThreads = 512;
constexpr int kPassWaves = kPassThreads / 64;
constexpr int kPollWaves = 2;              // waves 0 and 1: polls, no LDS-DMA
constexpr int kPollThreads = kPollWaves * 64;
constexpr unsigned kSpinLimit = 1u << 20;  // polls of one wait before it gives up
constexpr int kPassTableSlots = 256;       // layer pointers of one launch
constexpr int kPassMaxPass = 1024;         // passes of one item at most (tag space)
constexpr int kRingBytes = 131072;         // key tiles in LDS per workgroup
constexpr unsigned kTagEpochMask = (1u << 21) - 1u;  // epoch bits in the row normaliser tags

// Tag of the row normaliser records of pass p in the call with this epoch.
__device__ __forceinline__ unsigned xrec_tag(unsigned epoch, int p) {
  return ((epoch & kTagEpochMask) + 1u) * (unsigned)kPassMaxPass + (unsigned)p;
}

// Key tiles per wave in the ring (a wave's share of one head group of an
// item) and row tiles per pass (register budget of the logits and the query
// fragments), per element size and head dimension.
__host__ __device__ constexpr int pass_kt(int D, int esize) { return kRingBytes / (kPassWaves * 16 * D * esize); }
__host__ __device__ constexpr int pass_rtp(int D, int esize) { return (esize == 2 && D == 128) ? 6 : 4; }

// One poll of a bounded wait. True when the wait must end: this one ran out
// (the timeout bit is set) or another one in the launch already did.
__device__ __forceinline__ bool spin_expired(unsigned &spins, int *flags) {
  if (++spins > kSpinLimit) {
    __hip_atomic_fetch_or(flags, AIRCACHE_DEV_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  if ((spins & 255u) == 0u && (load_coherent(flags) & AIRCACHE_DEV_TIMEOUT)) return true;
  return false;
}

// The thread index, opaque to the optimiser: values derived from it are
// recomputed where they are used instead of being hoisted and kept live.
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 2^x by the hardware instruction (results below 2^-126 flush to zero, far
// below float32 resolution of a softmax weight against a row sum >= 1).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint64_t pack_rec(float v, unsigned tag) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}

__host__ __device__ inline int pass_words64(int Nt) { return (Nt + 63) >> 6; }
__host__ __device__ inline int pass_align16(int x) { return (x + 15) & ~15; }

// Block-wide double sum over kPassThreads threads in a fixed order.
__device__ __forceinline__ double block_sum_d(double v, double *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_d(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kPassWaves; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Two block-wide double sums at once, each in the order of block_sum_d.
__device__ __forceinline__ void block_sum_d2(double &a, double &b, double *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_sum_d(a);
  b = wave_sum_d(b);
  if (lane == 0) {
    red[wave] = a;
    red[kPassWaves + wave] = b;
  }
  __syncthreads();
  double ta = 0.0, tb = 0.0;
  for (int w = 0; w < kPassWaves; ++w) {
    ta += red[w];
    tb += red[kPassWaves + w];
  }
  __syncthreads();
  a = ta;
  b = tb;
}

// Layer pointers of one launch, L entries each: text queries at [0, L), keys
// at [L, 2L) and, when the launch also compacts, values at [2L, 3L),
// compacted keys at [3L, 4L) and compacted values at [4L, 5L).
struct PassTables {
  const void *p[kPassTableSlots];
};

// Workspace of the chunked path and the launch's schedule.
struct PassWs {
  unsigned *epoch;   // [1] calls so far (the last call's epoch)
  unsigned *exitc;   // [1] workgroups finished in this call
  int *flags;        // [1] AIRCACHE_DEV_* bits found in this call
  unsigned *wrapc;   // [1] workgroups done zeroing the records (calls whose epoch is a multiple of 2^21)
  u32x4_t *recs;     // the records (parts .. brec), zeroed by those calls
  size_t rec_words;  // 16-byte words of the records
  uint64_t *parts;   // [L*B][npp][N_t] elite-window parts 1.. (pbar sums | epoch << 32)
  uint64_t *erec;    // [L*B][erec_stride] elite size, then mask halves, each | epoch << 32
  uint64_t *xrec;    // [L*B][2][nch][hgs][rows][2] row (max, sum) | tag << 32
  uint64_t *mom;     // [L*B][nch][8] halves of chunk sum, M2, M3, count | epoch << 32
  uint64_t *ivrec;   // [L*B][N_v] I_v | epoch << 32
  uint64_t *brec;    // [L*B] budget | epoch << 32
  int npp;           // elite-window parts per (layer, sample): a divisor of H_kv
  int erec_stride;   // 1 + 2 * ceil(N_t / 64)
  int hgs;           // KV heads per head group (1, 2, 4 or 8; divides H_kv)
  int nhg;           // head groups, H_kv / hgs
  int wph;           // waves per KV head, kPassWaves / hgs
  int width;         // visual keys per chunk, wph * 16 * KT
  int nch;           // chunks per (layer, sample)
  int rows;          // rows per record slot and head, RTP * 16
  int E;             // elite workgroups
  int ppr0;          // (layer, sample) pairs in round 0
  int ppr;           // pairs per later round
  int units;         // consumer units
  int gather;        // 1: the launch also compacts
  int esize;         // bytes per element
  int64_t cap_elems; // elements of each compacted layer buffer
};

// Dynamic LDS of aircache_pass_kernel (byte offsets, 16-byte aligned). ring:
// the key tiles (kRingBytes), reused by the consumer units (top-k histogram
// and candidates, kept indices, statistics). misc: the elite list and the row
// arrays of the items. The elite parts' text logits take ring and misc (an
// elite workgroup stages no keys before its parts are done).
struct PassLds {
  int ring, misc;                             // regions
  int el, scr, colsum, red, mloc, zloc, wts, tmax, tsum;  // item arrays inside misc
  int z_bytes;                                // bytes of misc the elite parts may use
  int kidx, hist, sts;                        // consumer arrays inside ring
  int total;
};

__host__ __device__ inline PassLds pass_lds_layout(int D, int esize, int hgs, int width, int G, int Nt, int Nv,
                                                   int L) {
  PassLds f;
  const int rows = pass_rtp(D, esize) * 16;
  int o = 0;
  f.ring = o;
  o += kRingBytes;
  f.misc = o;
  int m = 0;
  f.el = o + m;
  m += pass_align16(Nt * 4);
  f.scr = o + m;
  m += pass_align16((2 + 2 * pass_words64(Nt)) * 4);
  f.colsum = o + m;
  m += pass_align16(hgs * width * 4);
  f.red = o + m;
  m += pass_align16(kPassWaves * rows * 4);
  f.mloc = o + m;
  m += pass_align16(hgs * rows * 4);
  f.zloc = o + m;
  m += pass_align16(hgs * rows * 4);
  f.wts = o + m;
  m += pass_align16(hgs * rows * 4);
  f.tmax = o + m;
  m += pass_align16(hgs * rows * 4);
  f.tsum = o + m;
  m += pass_align16(hgs * rows * 4);
  o += pass_align16(m);
  f.total = o;
  f.z_bytes = o - f.ring;  // the elite parts' text logits: ring and misc
  // consumer arrays in the ring
  int r = 0;
  f.hist = r;
  r += pass_align16((2048 + 2 * 256 + 4) * 4);  // kTopkLdsWords
  f.kidx = r;
  r += pass_align16(Nv * 4);
  f.sts = r;  // st, sk, bx: L + 16 doubles each; budgets: L + 16 ints
  return f;
}

// ---------------------------------------------------------------------------
// Elite window ("Elite Observation Window", the Att and k equations).
// ---------------------------------------------------------------------------

// Logits of the last text query of every query head of KV heads g0.. over the
// text keys, scaled, into z (rows of N_t floats, G rows per KV head): items
// (KV head, query-head tile, key tile) wave, wave + NW, ..., U at a time per
// wave, every load of the U items issued before the first product. Items past
// the end repeat the wave's first of the batch, not stored.
template <typename Tag, int D, int U>
__device__ __forceinline__ void elite_logits(const Shape &sh, const typename Tag::store_t *q,
                                             const typename Tag::store_t *k, int b, int g0, int items, int per_head,
                                             int nkt, float *z, int head_floats) {
  using E = typename Tag::store_t;
  constexpr int NW = kPassWaves;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int Nt = sh.Nt, G = sh.G, Hkv = sh.Hkv;
  for (int it0 = wave; it0 < items; it0 += NW * U) {
    Frag<Tag> qf[U][D / 32], kf[U][D / 32];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * NW < items ? it0 + u * NW : it0;
      const int gl = it / per_head, r = it - gl * per_head;
      const int ht = r / nkt, kt_ = r - ht * nkt;
      const int g = g0 + gl;
      const int h = min(ht * 16 + n, G - 1), key = min(kt_ * 16 + n, Nt - 1);
      const E *qrow = q + ((size_t)(b * sh.Hq + g * G + h) * Nt + (Nt - 1)) * D;
      const E *krow = k + ((size_t)(b * Hkv + g) * sh.S + sh.Nv + key) * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        qf[u][c].load(qrow + c * 32 + grp * 8);
        kf[u][c].load(krow + c * 32 + grp * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) mfma_slice(acc[u], kf[u][c], qf[u][c]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * NW;
      if (it < items) {
        const int gl = it / per_head, r = it - gl * per_head;
        const int ht = r / nkt, kt_ = r - ht * nkt;
        if (ht * 16 + n < G) {
          float *zr = z + (size_t)gl * head_floats + (size_t)(ht * 16 + n) * Nt;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = kt_ * 16 + grp * 4 + i;
            if (kk < Nt) zr[kk] = acc[u][i] * sh.scale2;
          }
        }
      }
    }
  }
}

// One part of the elite window of (layer, sample) lb: KV heads
// [pi * H_kv / npp, (pi + 1) * H_kv / npp). For every KV head of the part and
// each of its G query heads, the softmax row of the last text query over the
// N_t text keys (MFMA logits into LDS, each wave normalising whole rows); the
// part's pbar_j is the sum over its KV heads in ascending order of the sums
// over their query heads in ascending order. Parts 1.. are published as
// epoch-tagged words; the workgroup of part 0 adds them in ascending part
// order, keeps { j : pbar_j >= alpha max pbar } (or the last `window` text
// tokens for the window variants) and publishes it: erec[lb] = [size, then
// each mask word as two 32-bit halves]; also the plan's elite list and count,
// and the overflow bit when the size exceeds the elite cap. N_t <= 1024.
template <typename Tag, int D>
__device__ __forceinline__ void elite_part(const Shape &sh, const PassTables &tab, const PlanPtrs &plan,
                                           const PassWs &pw, int lb, int pi, unsigned epoch, float *z,
                                           int lds_bytes, int *wtot, float *red) {
  using E = typename Tag::store_t;
  constexpr int NT = kPassThreads, NW = kPassWaves, EP = 2;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int l = lb / sh.B, b = lb - (lb / sh.B) * sh.B;
  const int Nt = sh.Nt, G = sh.G, Hkv = sh.Hkv, npp = pw.npp;
  const int hg = Hkv / npp, gbeg = pi * hg, gend = gbeg + hg;
  const E *q = static_cast<const E *>(tab.p[l]);
  const E *k = static_cast<const E *>(tab.p[sh.L + l]);
  const int nkt = (Nt + 15) >> 4, nht = (G + 15) >> 4;
  const int per_head = nht * nkt;
  const int head_floats = G * Nt;
  int gh = lds_bytes / (head_floats * (int)sizeof(float));
  gh = gh < 1 ? 1 : (gh > hg ? hg : gh);
  float pb[EP] = {0.f, 0.f};
  for (int g0 = gbeg; g0 < gend; g0 += gh) {
    const int ng = gend - g0 < gh ? gend - g0 : gh;
    const int items = ng * per_head;
    const int per_wave = (items + NW - 1) / NW;
    constexpr int UMAX = Tag::kBytes == 4 ? 2 : 4;
    if (per_wave >= 4) elite_logits<Tag, D, UMAX>(sh, q, k, b, g0, items, per_head, nkt, z, head_floats);
    else if (per_wave >= 2) elite_logits<Tag, D, 2>(sh, q, k, b, g0, items, per_head, nkt, z, head_floats);
    else elite_logits<Tag, D, 1>(sh, q, k, b, g0, items, per_head, nkt, z, head_floats);
    __syncthreads();
    for (int h = wave; h < ng * G; h += NW) {
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
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      const int j = tid + e * NT;
      if (j < Nt)
        for (int gl = 0; gl < ng; ++gl) {
          float a = 0.f;
          for (int h = 0; h < G; ++h) a += z[(size_t)(gl * G + h) * Nt + j];
          pb[e] += a;
        }
    }
    __syncthreads();  // z is free again
  }
  if (pi > 0) {
    uint64_t *part = pw.parts + ((size_t)lb * npp + pi) * Nt;
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (tid + e * NT < Nt) store_coherent(&part[tid + e * NT], pack_rec(pb[e], epoch));
    return;
  }
  if (npp > 1) {
    // the other parts, every load issued before any is checked
    constexpr int PM = 7;  // npp <= 8
    const auto rp = coherent_rsrc(pw.parts + (size_t)lb * npp * Nt, (unsigned)((size_t)npp * Nt * sizeof(uint64_t)));
    uint64_t w[EP][PM];
    unsigned spins = 0;
    for (;;) {
#pragma unroll
      for (int e = 0; e < EP; ++e)
#pragma unroll
        for (int p = 0; p < PM; ++p) {
          const int j = tid + e * NT;
          const unsigned off =
              (j < Nt && p + 1 < npp) ? (unsigned)(((size_t)(p + 1) * Nt + j) * sizeof(uint64_t)) : 0xfffffff0u;
          w[e][p] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rp, (int)off, 0, 16));
        }
      bool ok = true;
#pragma unroll
      for (int e = 0; e < EP; ++e)
#pragma unroll
        for (int p = 0; p < PM; ++p)
          ok = ok && (tid + e * NT >= Nt || p + 1 >= npp || (unsigned)(w[e][p] >> 32) == epoch);
      if (ok || spin_expired(spins, pw.flags)) break;
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int e = 0; e < EP; ++e)
#pragma unroll
      for (int p = 0; p < PM; ++p)
        if (p + 1 < npp) pb[e] += __uint_as_float((unsigned)w[e][p]);
  }
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < EP; ++e)
    if (tid + e * NT < Nt) m = fmaxf(m, pb[e]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
  for (int u = 1; u < NW; ++u) m = fmaxf(m, red[u]);
  const float thr = sh.alpha * m;
  // word e * NW + wave holds tokens 64 (e * NW + wave) + lane
  unsigned long long mk[EP];
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    const int j = tid + e * NT;
    mk[e] = __ballot(j < Nt && (sh.window > 0 ? j >= Nt - sh.window : pb[e] >= thr));
  }
  if (lane == 0)
#pragma unroll
    for (int e = 0; e < EP; ++e) wtot[e * NW + wave] = __popcll(mk[e]);
  __syncthreads();
  const int ntw = pass_words64(Nt);
  uint64_t *rec = pw.erec + (size_t)lb * pw.erec_stride;
  const uint64_t tag = (uint64_t)epoch << 32;
  int total = 0;
  for (int u = 0; u < EP * NW; ++u) total += wtot[u];
  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    const int word = e * NW + wave;
    int before = 0;
    for (int u = 0; u < word; ++u) before += wtot[u];
    if ((mk[e] >> lane) & 1ull) plan.elite[(size_t)lb * Nt + before + __popcll(mk[e] & lt)] = word * 64 + lane;
    if (word < ntw && lane < 2) {
      const unsigned half = lane == 0 ? (unsigned)mk[e] : (unsigned)(mk[e] >> 32);
      store_coherent(&rec[1 + 2 * word + lane], tag | (uint64_t)half);
    }
  }
  if (tid == 0) {
    store_coherent(&rec[0], tag | (uint64_t)(unsigned)total);
    plan.n_elite[lb] = total;
    if (total > sh.cap) __hip_atomic_fetch_or(pw.flags, AIRCACHE_DEV_ELITE_OVERFLOW, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // wtot and red are free again
}

// The elite list of pair plb, ascending, into el (LDS, at most the elite cap
// entries) from its merge's record; wave 0 (a poll wave) polls the size and
// mask words into scr. Returns the clamped count (block-wide).
__device__ __forceinline__ int pass_elite_list(const Shape &sh, const PassWs &pw, int plb, unsigned epoch, int *el,
                                               unsigned *scr) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int ntw = pass_words64(sh.Nt), nword = 1 + 2 * ntw;  // <= 33
  if (wave == 0 && lane < nword) {
    const auto rr = coherent_rsrc(pw.erec + (size_t)plb * pw.erec_stride,
                                  (unsigned)(pw.erec_stride * sizeof(uint64_t)));
    const int off = lane * (int)sizeof(uint64_t);
    uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 16));
    unsigned spins = 0;
    while ((unsigned)(v >> 32) != epoch) {
      if (spin_expired(spins, pw.flags)) break;
      __builtin_amdgcn_s_sleep(1);
      v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 16));
    }
    // the size at scr[0]; mask word i as the halves scr[2 + 2i], scr[3 + 2i]
    scr[lane == 0 ? 0 : lane + 1] = (unsigned)v;
  }
  __syncthreads();
  // the list holds the mask's tokens below N_t; the count is the record's,
  // clamped to the elite cap and to the tokens the list holds (the two agree
  // unless a wait gave up, and then no index may leave its range)
  const unsigned long long *mw = reinterpret_cast<const unsigned long long *>(scr + 2);
  const int tail = sh.Nt - (ntw - 1) * 64;  // tokens in the last mask word, 1..64
  const unsigned long long last = tail >= 64 ? ~0ull : ((1ull << tail) - 1ull);
  int held = 0;
  for (int u = 0; u < ntw; ++u) held += __popcll(mw[u] & (u == ntw - 1 ? last : ~0ull));
  int ntk = (int)scr[0];
  ntk = ntk < sh.cap ? ntk : sh.cap;
  ntk = ntk < held ? ntk : held;
  ntk = ntk > 0 ? ntk : 0;
  for (int w = wave; w < ntw; w += kPassWaves) {
    int base = 0;
    for (int u = 0; u < w; ++u) base += __popcll(mw[u]);
    const unsigned long long mk = mw[w] & (w == ntw - 1 ? last : ~0ull);
    const int pos = base + __popcll(mk & ((1ull << lane) - 1ull));
    if (((mk >> lane) & 1ull) && pos < ntk) el[pos] = w * 64 + lane;
  }
  __syncthreads();
  return uniform(ntk);
}

// ---------------------------------------------------------------------------
// Items: cross-modal scores of one chunk ("Elite Observation Window", the
// A_vtk and I_v equations).
// ---------------------------------------------------------------------------

// LDS-DMA of one wave's share of a head group's keys of an item: KT tiles of
// 16 visual keys of KV head g from column c0 + sub * KT * 16 on, into the
// wave's ring slots (staged as LdsTile reads them); keys past N_v read the
// last visual key, masked later.
template <typename Tag, int D>
__device__ __forceinline__ void pass_issue(const Shape &sh, const void *k_layer, int b, int g, int c0, int sub,
                                           unsigned char *slots) {
  using E = typename Tag::store_t;
  constexpr int KT = pass_kt(D, Tag::kBytes);
  constexpr int kTile = 16 * D * Tag::kBytes;
  constexpr int kDma = kTile / 1024;
  const int lane = opaque_tid() & 63, n = lane & 15, grp = lane >> 4;
  const E *kb = static_cast<const E *>(k_layer) + (size_t)(b * sh.Hkv + g) * sh.S * D;
#pragma unroll
  for (int s = 0; s < KT; ++s) {
    const int v = c0 + (sub * KT + s) * 16 + n;
    const int row = v < sh.Nv ? v : sh.Nv - 1;
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kb + (size_t)row * D);
#pragma unroll
    for (int j = 0; j < kDma; ++j) load_lds16(src + 16 * grp + 64 * j, slots + s * kTile + 1024 * j);
  }
}

// The keys of head group hg of the item (pair q, chunk c) into the ring, by
// the loader waves: wave w >= kPollWaves loads its own slots and, for
// w < 2 * kPollWaves, those of poll wave w - kPollWaves.
template <typename Tag, int D>
__device__ __forceinline__ void pass_stage(const Shape &sh, const PassWs &pw, const PassTables &tab, int q, int c,
                                           int hg, unsigned char *ring) {
  constexpr int KT = pass_kt(D, Tag::kBytes);
  constexpr int kTile = 16 * D * Tag::kBytes;
  const int wave = uniform(opaque_tid() >> 6);
  if (wave < kPollWaves) return;
  const int b = q / sh.L, l = q - b * sh.L;
  const void *kl = tab.p[sh.L + l];
  const int c0 = c * pw.width;
  auto one = [&](int ow) {
    const int gl = ow / pw.wph, sub = ow - gl * pw.wph;
    pass_issue<Tag, D>(sh, kl, b, hg * pw.hgs + gl, c0, sub, ring + (size_t)ow * KT * kTile);
  };
  one(wave);
  if (wave < 2 * kPollWaves) one(wave - kPollWaves);
}

struct PassItem {
  int l, b, plb, c, c0, ncol, ntk, rtg, nrg;
  const void *q, *k;
};

// One pass of an item: RTP row tiles (rows rg * RTPM * 16 ..) of the elite
// query rows of every KV head of head group hg, against the chunk's keys in
// the ring. Leaves the pass's column sums of the softmax rows added to colacc
// (a wave's key tiles; one value per column, in every lane of its row). When
// the pass is the last over these tiles, stage_next() loads the next ones as
// soon as every wave has read them.
template <typename Tag, int D, int RTP, typename NextFn>
__device__ __forceinline__ void pass_rows(const Shape &sh, const PassWs &pw, const PassItem &it, int hg, int rg,
                                          int pidx, bool last_of_tiles, unsigned char *lds, const PassLds &lo,
                                          unsigned epoch, float (&colacc)[pass_kt(D, Tag::kBytes)],
                                          NextFn &&stage_next) {
  using E = typename Tag::store_t;
  constexpr int NW = kPassWaves;
  constexpr int KT = pass_kt(D, Tag::kBytes);
  constexpr int RTPM = pass_rtp(D, Tag::kBytes);
  constexpr int kTile = 16 * D * Tag::kBytes;
  constexpr int RW = RTP * 16;  // rows of one head in this pass
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int hgs = pw.hgs, wph = pw.wph, ROWS = pw.rows;
  const int gl = wave / wph, sub = wave - gl * wph;
  const int g = hg * hgs + gl;
  const int ntk = it.ntk, Rg = sh.G * ntk, Nv = sh.Nv;
  const int rt0 = rg * RTPM;
  const int *el = reinterpret_cast<const int *>(lds + lo.el);
  float *red = reinterpret_cast<float *>(lds + lo.red);
  float *mloc = reinterpret_cast<float *>(lds + lo.mloc);
  float *zloc = reinterpret_cast<float *>(lds + lo.zloc);
  float *wts = reinterpret_cast<float *>(lds + lo.wts);
  float *tmax = reinterpret_cast<float *>(lds + lo.tmax);
  float *tsum = reinterpret_cast<float *>(lds + lo.tsum);
  const unsigned char *slots = lds + lo.ring + (size_t)wave * KT * kTile;
  const E *qb = static_cast<const E *>(it.q);
  const E *kb = static_cast<const E *>(it.k) + (size_t)(it.b * sh.Hkv + g) * sh.S * D;

  // query fragments: RTP tiles of 16 elite query rows of this wave's head
  Frag<Tag> qf[RTP][D / 32];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt) {
    const int r = (rt0 + rt) * 16 + n;
    if (r < Rg) {
      const int hl = r / ntk, e = r - hl * ntk;
      const E *qrow = qb + ((size_t)(it.b * sh.Hq + g * sh.G + hl) * sh.Nt + el[e]) * D;
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) qf[rt][cc].load(qrow + cc * 32 + grp * 8);
    } else {
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) qf[rt][cc].zero();
    }
  }

  // Chunk 0 also carries the elite text keys: per row, their (max, sum of
  // exp2(logit - max)) into tmax / tsum, from fragments read straight from
  // global memory (two passes over them, the second recomputing the logits).
  // They enter the rows' normalisers, never the column sums.
  const int ntt = it.c == 0 ? (ntk + 15) >> 4 : 0;
  auto text_logits = [&](int t, f32x4_t (&st)[RTP]) {
    const int e = t * 16 + n;
    const E *kr = kb + (size_t)(Nv + el[e < ntk ? e : ntk - 1]) * D;
    Frag<Tag> kf[D / 32];
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) kf[cc].load(kr + cc * 32 + grp * 8);
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) mfma_slice(acc, qf[rt][cc], kf[cc]);
#pragma unroll
      for (int i = 0; i < 4; ++i) st[rt][i] = e < ntk ? acc[i] * sh.scale2 : -INFINITY;
    }
  };
  float racc[RTP][4];
  if (ntt > 0) {
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) racc[rt][i] = -INFINITY;
    for (int t = sub; t < ntt; t += wph) {
      f32x4_t st[RTP];
      text_logits(t, st);
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) racc[rt][i] = fmaxf(racc[rt][i], st[rt][i]);
    }
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m = row16_max(racc[rt][i]);
        if (n == 0) red[wave * RW + rt * 16 + grp * 4 + i] = m;
      }
    __syncthreads();
    if (tid < hgs * RW) {
      const int gg = tid / RW, rr = tid - gg * RW;
      float m = red[(gg * wph) * RW + rr];
      for (int w = 1; w < wph; ++w) m = fmaxf(m, red[(gg * wph + w) * RW + rr]);
      tmax[gg * RW + rr] = m;
    }
    __syncthreads();
    float Tm[RTP][4];
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Tm[rt][i] = tmax[gl * RW + rt * 16 + grp * 4 + i];
        racc[rt][i] = 0.f;
      }
    for (int t = sub; t < ntt; t += wph) {
      f32x4_t st[RTP];
      text_logits(t, st);
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) racc[rt][i] += st[rt][i] > -INFINITY ? exp2_fast(st[rt][i] - Tm[rt][i]) : 0.f;
    }
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = row16_sum(racc[rt][i]);
        if (n == 0) red[wave * RW + rt * 16 + grp * 4 + i] = z;
      }
    __syncthreads();
    if (tid < hgs * RW) {
      const int gg = tid / RW, rr = tid - gg * RW;
      float z = 0.f;
      for (int w = 0; w < wph; ++w) z += red[(gg * wph + w) * RW + rr];
      tsum[gg * RW + rr] = z;
    }
    __syncthreads();  // red is written again by the visual row maxima
  }

  // logits of the visual keys, from the ring
  f32x4_t S[KT][RTP];
  int vbase = it.c0 + sub * KT * 16 + n;  // this lane's column in tile 0
  asm volatile("" : "+v"(vbase));
#pragma unroll
  for (int s = 0; s < KT; ++s) {
    f32x4_t acc[RTP];
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const unsigned char *slot = slots + s * kTile;
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) {
      Frag<Tag> kf;
      LdsTile<Tag>::read(kf, slot, cc, lane);
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt) mfma_slice(acc[rt], qf[rt][cc], kf);
    }
    const bool ok = vbase + s * 16 < Nv;
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[s][rt][i] = ok ? acc[rt][i] * sh.scale2 : -INFINITY;
  }
  // chunk-local row maxima (visual keys and, in chunk 0, the text keys): keys
  // of a lane row by DPP, then the head's waves in order
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) racc[rt][i] = -INFINITY;
#pragma unroll
  for (int s = 0; s < KT; ++s)
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) racc[rt][i] = fmaxf(racc[rt][i], S[s][rt][i]);
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m = row16_max(racc[rt][i]);
      if (n == 0) red[wave * RW + rt * 16 + grp * 4 + i] = m;
    }
  __syncthreads();
  // every read of this pass's tiles is done (their values entered S before
  // the barrier): the loader waves may stage the next tiles now
  if (last_of_tiles) stage_next();
  if (tid < hgs * RW) {
    const int gg = tid / RW, rr = tid - gg * RW;
    float m = red[(gg * wph) * RW + rr];
    for (int w = 1; w < wph; ++w) m = fmaxf(m, red[(gg * wph + w) * RW + rr]);
    if (ntt > 0) m = fmaxf(m, tmax[gg * RW + rr]);
    mloc[gg * RW + rr] = m;
  }
  __syncthreads();
  // exponentials in place and chunk-local row sums
  float Mrow[RTP][4];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Mrow[rt][i] = mloc[gl * RW + rt * 16 + grp * 4 + i];
      racc[rt][i] = 0.f;
    }
#pragma unroll
  for (int s = 0; s < KT; ++s)
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ev = exp2_fast(S[s][rt][i] - Mrow[rt][i]);
        S[s][rt][i] = ev;
        racc[rt][i] += ev;
      }
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = row16_sum(racc[rt][i]);
      if (n == 0) red[wave * RW + rt * 16 + grp * 4 + i] = z;
    }
  __syncthreads();
  if (tid < hgs * RW) {
    const int gg = tid / RW, rr = tid - gg * RW;
    float z = 0.f;
    for (int w = 0; w < wph; ++w) z += red[(gg * wph + w) * RW + rr];
    if (ntt > 0) {
      const float tm = tmax[gg * RW + rr];
      if (tm > -INFINITY) z += tsum[gg * RW + rr] * exp2_fast(tm - mloc[gg * RW + rr]);
    }
    zloc[gg * RW + rr] = z;
  }
  __syncthreads();
  // the poll waves publish this chunk's (max, sum) per row and merge every
  // chunk's pair in chunk order into each row's normaliser
  if (tid < kPollThreads) {
    const unsigned tag = xrec_tag(epoch, pidx);
    const int nch = pw.nch, c = it.c;
    const size_t sbase = ((size_t)it.plb * 2 + (pidx & 1)) * nch;  // (pair, slot) block, in chunks
    uint64_t *blk = pw.xrec + 2 * sbase * hgs * ROWS;
    const auto rsrc = coherent_rsrc(blk, (unsigned)((size_t)nch * hgs * ROWS * 16));
    for (int qr = tid; qr < hgs * RW; qr += kPollThreads) {
      const int gg = qr / RW, rr = qr - gg * RW;
      const float m_own = mloc[gg * RW + rr], z_own = zloc[gg * RW + rr];
      uint64_t *rec = blk + 2 * (((size_t)c * hgs + gg) * ROWS + rr);
      store_coherent(rec, pack_rec(m_own, tag));
      store_coherent(rec + 1, pack_rec(z_own, tag));
      float M = -INFINITY, Z = 0.f;
      constexpr int kXB = 8;  // chunks' records in flight per row (one 16-byte load each)
      for (int c0 = 0; c0 < nch; c0 += kXB) {
        u32x4_t rw[kXB];
        auto load_batch = [&]() {
#pragma unroll
          for (int j = 0; j < kXB; ++j) {
            const int cj = c0 + j;
            const unsigned off = (cj < nch && cj != c) ? (unsigned)((((size_t)cj * hgs + gg) * ROWS + rr) * 16)
                                                       : 0xfffffff0u;  // past the end: zeros, not used
            rw[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 16));
          }
        };
        load_batch();
        unsigned spins = 0;
        for (;;) {
          bool ok = true;
#pragma unroll
          for (int j = 0; j < kXB; ++j) {
            const int cj = c0 + j;
            ok = ok && (cj >= nch || cj == c || (rw[j][1] == tag && rw[j][3] == tag));
          }
          if (ok || spin_expired(spins, pw.flags)) break;
          __builtin_amdgcn_s_sleep(1);
          load_batch();
        }
#pragma unroll
        for (int j = 0; j < kXB; ++j) {
          const int cj = c0 + j;
          if (cj >= nch) break;
          const float mj = cj == c ? m_own : __uint_as_float(rw[j][0]);
          const float zj = cj == c ? z_own : __uint_as_float(rw[j][2]);
          if (mj > -INFINITY) {
            const float mn = fmaxf(M, mj);
            Z = Z * exp2_fast(M - mn) + zj * exp2_fast(mj - mn);
            M = mn;
          }
        }
      }
      const int row = rt0 * 16 + rr;
      wts[gg * RW + rr] = (row < Rg && Z > 0.f) ? exp2_fast(m_own - M) / Z : 0.f;
    }
  }
  __syncthreads();
  // column sums over the pass's rows of this wave's head (one value per
  // column, summed over the four lane groups); row weights in registers
  float wrow[RTP][4];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[rt][i] = wts[gl * RW + rt * 16 + grp * 4 + i];
#pragma unroll
  for (int s = 0; s < KT; ++s) {
    float v = 0.f;
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) v += S[s][rt][i] * wrow[rt][i];
    colacc[s] += sum_across_rows(v);
  }
  __syncthreads();  // red, mloc, zloc, wts, tmax, tsum are reused by the next pass
}

// ---------------------------------------------------------------------------
// Statistics, budgets, top-k ("Layer-wise KV Cache Budget Allocation" and the
// training-free procedure).
// ---------------------------------------------------------------------------

// Moments of a run of values, combined pairwise (Chan, Golub and LeVeque's
// update, extended to the third central moment): count, mean, M2 and M3.
struct Moments {
  double n, mean, m2, m3;
};
__device__ __forceinline__ Moments combine_moments(const Moments &a, const Moments &b) {
  if (b.n == 0.0) return a;
  if (a.n == 0.0) return b;
  Moments r;
  const double n = a.n + b.n, inv = 1.0 / n, d = b.mean - a.mean;
  const double db = d * b.n * inv;  // mean shift
  r.n = n;
  r.mean = a.mean + db;
  r.m2 = a.m2 + b.m2 + d * db * a.n;
  r.m3 = a.m3 + b.m3 + d * d * db * a.n * (a.n - b.n) * inv + 3.0 * d * (a.n * b.m2 - b.n * a.m2) * inv;
  return r;
}

// s_t and s_k of (layer, sample) plb ("Layer-wise KV Cache Budget
// Allocation", the s_t and s_k equations) from its chunks' moment records, by
// one wave: lane c holds chunks c, c + 64, ... (combined in that order), then
// the lanes combine pairwise in a fixed tree (at stride st, lane c, a
// multiple of 2 st, absorbs lane c + st), so every unit that computes it gets
// the same bits. The wave's lane 0 returns the values.
__device__ __forceinline__ void chunk_stats(const Shape &sh, const PassWs &pw, int plb, unsigned epoch, double *st_out,
                                            double *sk_out) {
  const int lane = threadIdx.x & 63;
  const int nch = pw.nch;
  const auto rm = coherent_rsrc(pw.mom + (size_t)plb * nch * 8, (unsigned)(nch * 64));
  double sum = 0.0;
  Moments m{0.0, 0.0, 0.0, 0.0};
  for (int c = lane; c < nch; c += 64) {
    uint64_t w[8];
    unsigned spins = 0;
    for (;;) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
        w[f] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rm, c * 64 + 8 * f, 0, 16));
      bool ok = true;
#pragma unroll
      for (int f = 0; f < 8; ++f) ok = ok && (unsigned)(w[f] >> 32) == epoch;
      if (ok || spin_expired(spins, pw.flags)) break;
      __builtin_amdgcn_s_sleep(1);
    }
    double v[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) v[f] = __builtin_bit_cast(double, (w[2 * f] & 0xffffffffu) | (w[2 * f + 1] << 32));
    sum = sum + v[0];
    m = combine_moments(m, Moments{v[3], v[3] > 0.0 ? v[0] / v[3] : 0.0, v[1], v[2]});
  }
  const int nl = nch < 64 ? nch : 64;
  for (int st = 1; st < nl; st <<= 1) {
    const int src = lane + st;
    const double osum = __shfl(sum, src), on = __shfl(m.n, src), omean = __shfl(m.mean, src);
    const double om2 = __shfl(m.m2, src), om3 = __shfl(m.m3, src);
    if ((lane & (2 * st - 1)) == 0 && src < nl) {
      m = combine_moments(m, Moments{on, omean, om2, om3});
      sum = sum + osum;
    }
  }
  const int Nv = sh.Nv;
  const double sigma = sqrt(m.m2 / (double)(Nv - 1));
  const double sk =
      (sigma > 0.0) ? (m.m3 / (sigma * sigma * sigma)) * ((double)Nv / ((double)(Nv - 1) * (double)(Nv - 2))) : 0.0;
  *st_out = sum;
  *sk_out = sk;
}

// budget_sums over LDS with the values read sixteen at a time, every read of
// a batch issued before the first addition (one LDS round trip per batch), and
// no branches. The two sums take the same additions in the same order as the
// serial form (a padded entry adds +0.0 to a non-negative sum). The shift is
// a minimum, exact in any order: four interleaved chains of v_min_f64, then
// +0.0 unless some s_k is negative. Reads run up to 15 entries past L (the
// LDS arrays are padded).
__device__ __forceinline__ BudgetSums budget_sums_lds(int L, const double *st, const double *sk) {
#pragma clang fp contract(off)
  constexpr int U = 16;
  BudgetSums r{0.0, 0.0, 0.0};
  double m[4] = {0.0, 0.0, 0.0, 0.0};
  for (int l0 = 0; l0 < L; l0 += U) {
    double a[U], c[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      a[j] = st[l0 + j];
      c[j] = sk[l0 + j];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const bool in = l0 + j < L;
      r.st_sum += in ? a[j] : 0.0;
      m[j & 3] = in ? fmin(m[j & 3], c[j]) : m[j & 3];
    }
  }
  const double mn = fmin(fmin(m[0], m[1]), fmin(m[2], m[3]));
  r.mshift = mn < 0.0 ? mn : 0.0;
  for (int l0 = 0; l0 < L; l0 += U) {
    double c[U];
#pragma unroll
    for (int j = 0; j < U; ++j) c[j] = sk[l0 + j];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < U; ++j) r.u_sum += (l0 + j < L) ? c[j] - r.mshift : 0.0;
  }
  return r;
}

// budget_sums of one sample with its layers across the lanes of a wave (L <=
// 64; every lane gets the result): the shift is a minimum, exact in any order
// (a DPP reduction; lanes past L hold 0.0, which min(0, ...) already has),
// +0.0 unless some s_k is negative; the two sums take the same additions in
// the same order as the serial form, four lanes' values read ahead.
__device__ __forceinline__ BudgetSums budget_sums_wave(int L, const double *st, const double *sk) {
#pragma clang fp contract(off)
  const int lane = opaque_tid() & 63;
  const double a = lane < L ? st[lane] : 0.0;
  const double c = lane < L ? sk[lane] : 0.0;
  double mn = c;
  mn = fmin(mn, dpp_d<0xB1>(mn));
  mn = fmin(mn, dpp_d<0x4E>(mn));
  mn = fmin(mn, dpp_d<0x141>(mn));
  mn = fmin(mn, dpp_d<0x140>(mn));
  mn = fmin(fmin(readlane_d(mn, 0), readlane_d(mn, 16)), fmin(readlane_d(mn, 32), readlane_d(mn, 48)));
  BudgetSums r;
  r.mshift = mn < 0.0 ? mn : 0.0;
  const double u = lane < L ? c - r.mshift : 0.0;
  double s1 = 0.0, s2 = 0.0;
  for (int l0 = 0; l0 < L; l0 += 4) {
    double a4[4], u4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a4[j] = readlane_d(a, l0 + j);
      u4[j] = readlane_d(u, l0 + j);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s1 += a4[j];
      s2 += u4[j];
    }
  }
  r.st_sum = s1;
  r.u_sum = s2;
  return r;
}

// Statistics and budgets of every layer of sample b, block-wide, into LDS
// (st, sk, bx: L + 16 doubles each, bud: L + 16 ints): each wave combines the
// chunk moments of layers wave, wave + 8, ...; then wave 0 forms the budgets
// ("Layer-wise KV Cache Budget Allocation", the r_hat equation over the
// sample's layers, in double precision and the oracle's order). With publish,
// the plan's s_t, s_k, budget and budget_x of the sample and its budget
// records (read by the units of later samples for their offsets) go out.
__device__ __forceinline__ void sample_budgets(const Shape &sh, const PlanPtrs &plan, const PassWs &pw, int b,
                                               unsigned epoch, bool publish, double *st, double *sk, double *bx,
                                               int *bud) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int L = sh.L, B = sh.B;
  for (int l = wave; l < L; l += kPassWaves) {
    double a, c;
    chunk_stats(sh, pw, l * B + b, epoch, &a, &c);
    if (lane == 0) {
      st[l] = a;
      sk[l] = c;
    }
  }
  if (tid < 16) {  // padding read by budget_sums_lds
    st[L + tid] = 0.0;
    sk[L + tid] = 0.0;
  }
  __syncthreads();
  if (wave == 0) {
    const BudgetSums sums = L <= 64 ? budget_sums_wave(L, st, sk) : budget_sums_lds(L, st, sk);
    for (int l = lane; l < L; l += 64) {
      double x;
      int r;
      layer_budget(sh, sums, st[l], sk[l], &x, &r);
      bx[l] = x;
      bud[l] = r;
      if (publish) {
        const int plb = l * B + b;
        plan.s_t[plb] = st[l];
        plan.s_k[plb] = sk[l];
        plan.budget[plb] = r;
        if (plan.bx) plan.bx[plb] = x;
        store_coherent(&pw.brec[plb], ((uint64_t)epoch << 32) | (uint64_t)(unsigned)r);
      }
    }
  }
  __syncthreads();
}

// Inclusive prefix sum over the 64 lanes of a wave: a scan inside each row of
// 16 lanes by DPP row shifts, then the row totals added in with readlane.
__device__ __forceinline__ int wave_scan_incl(int v) {
  const int lane = threadIdx.x & 63;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  if (lane >= 16) v += r0;
  if (lane >= 32) v += r1;
  if (lane >= 48) v += r2;
  return v;
}

// Top-r_hat of one (layer, sample) by the 512 threads of a workgroup: thread
// t holds the keys of indices t, t + 512, t + 1024, ... in registers (each
// load instruction reads 64 consecutive scores per wave). I_v >= 0, so the
// float32 bits order like the values, and the order that decides the kept set
// is (key descending, index ascending). The bits above the highest bit in
// which the minimum and maximum keys differ are common to all keys and
// skipped. While more than kTopkRankCap keys match the prefix found so far, a
// radix pass counts the next (up to) kTopkDigitBits bits of the matching keys
// into one LDS histogram, a block scan over the buckets in descending digit
// order finds the bucket holding the need-th key, and the prefix grows by that
// digit; the first pass's counts and their scan come before the budget is
// known. The keys left are then copied to LDS and each is ranked against the
// others directly; the one of rank need - 1 is the threshold T. Kept: every
// key > T plus the lowest-index keys equal to T up to the count still needed,
// in ascending index order, into kidx (LDS) and, when kept_out is not NULL,
// the plan. Returns the budget.
// lds: kTopkLdsWords words, the histogram zero on entry (and left zero).
constexpr int kTopkDigitBits = 11;
constexpr int kTopkBuckets = 1 << kTopkDigitBits;
constexpr int kTopkRankCap = 256;
constexpr int kTopkLdsWords = kTopkBuckets + 2 * kTopkRankCap + 4;
template <int PER, typename BudgetFn>
__device__ __forceinline__ int block_topk(const Shape &sh, const uint64_t *iv_l, int *kidx, int32_t *kept_out,
                                          unsigned epoch, int *flags, unsigned *lds, BudgetFn &&get_budget) {
  constexpr int NT = kPassThreads, NW = kPassWaves;
  constexpr int BPT = kTopkBuckets / NT;
  static_assert(BPT * NT == kTopkBuckets, "buckets must split evenly over the threads");
  __shared__ int wsum[2][NW];
  __shared__ float wmm[2][NW];
  __shared__ int selv[2][3];
  __shared__ int rowcnt[2][PER][NW];
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int Nv = sh.Nv;
  unsigned *hist = lds;
  uint2 *cand = reinterpret_cast<uint2 *>(lds + kTopkBuckets);
  unsigned *ncand = lds + kTopkBuckets + 2 * kTopkRankCap;
  // the scores as epoch-tagged words, read again until every word carries
  // this call's epoch (an index past N_v reads past the buffer: 0, not used)
  const auto riv = coherent_rsrc(iv_l, (unsigned)(Nv * sizeof(uint64_t)));
  uint64_t kw[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p)
    kw[p] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(riv, (p * NT + tid) * 8, 0, 16));
  {
    unsigned spins = 0;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int p = 0; p < PER; ++p) ok = ok && (p * NT + tid >= Nv || (unsigned)(kw[p] >> 32) == epoch);
      if (ok || spin_expired(spins, flags)) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int p = 0; p < PER; ++p)
        if (p * NT + tid < Nv && (unsigned)(kw[p] >> 32) != epoch)
          kw[p] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(riv, (p * NT + tid) * 8, 0, 16));
    }
  }
  unsigned key[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) key[p] = (unsigned)kw[p];
  float fmin = INFINITY, fmax = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p)
    if (p * NT + tid < Nv) {
      fmin = fminf(fmin, __uint_as_float(key[p]));
      fmax = fmaxf(fmax, __uint_as_float(key[p]));
    }
  fmin = -wave_max(-fmin);
  fmax = wave_max(fmax);
  if (lane == 0) {
    wmm[0][wave] = fmin;
    wmm[1][wave] = fmax;
  }
  if (tid == 0) *ncand = 0u;
  __syncthreads();
  fmin = wmm[0][0];
  fmax = wmm[1][0];
  for (int w = 1; w < NW; ++w) {
    fmin = fminf(fmin, wmm[0][w]);
    fmax = fmaxf(fmax, wmm[1][w]);
  }
  const unsigned kmin = __float_as_uint(fmin), kmax = __float_as_uint(fmax);
  const unsigned diff = kmin ^ kmax;
  int hb = diff ? 31 - __clz((int)diff) : -1;
  unsigned mask = (hb < 0) ? 0xffffffffu : (hb >= 31) ? 0u : ~((2u << hb) - 1u);
  unsigned prefix = kmin & mask;
  const bool first = hb >= 0 && Nv > kTopkRankCap;
  int c0[BPT], ct0 = 0, above0 = 0;
  if (first) {
    const int width = min(kTopkDigitBits, hb + 1);
    const int shift = hb + 1 - width;
    const unsigned dmask = (1u << width) - 1u;
    const int nb = 1 << width;
#pragma unroll
    for (int p = 0; p < PER; ++p)
      if (p * NT + tid < Nv) atomicAdd(&hist[(key[p] >> shift) & dmask], 1u);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int q = tid * BPT + j;
      c0[j] = 0;
      if (q < nb) {
        unsigned *h = &hist[nb - 1 - q];
        c0[j] = (int)*h;
        *h = 0u;
      }
      ct0 += c0[j];
    }
    const int incl = wave_scan_incl(ct0);
    if (lane == 63) wsum[0][wave] = incl;
    __syncthreads();
    above0 = incl - ct0;
    for (int w = 0; w < wave; ++w) above0 += wsum[0][w];
  }
  int kbud = get_budget();  // block-wide, with barriers
  if (kbud < 0) kbud = 0;
  if (kbud > Nv) kbud = Nv;
  if (kbud <= 0 || kbud >= Nv) {
    if (kbud >= Nv)
      for (int i = tid; i < Nv; i += NT) {
        kidx[i] = i;
        if (kept_out) kept_out[i] = i;
      }
    __syncthreads();
    return kbud;
  }
  int need = kbud;
  int nmatch = Nv;
  int par = 0;
  if (first) {
    const int width = min(kTopkDigitBits, hb + 1);
    const int shift = hb + 1 - width;
    const unsigned dmask = (1u << width) - 1u;
    const int nb = 1 << width;
    if (ct0 > 0 && above0 < need && above0 + ct0 >= need) {
      int above = above0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        if (above + c0[j] >= need) {
          selv[0][0] = nb - 1 - (tid * BPT + j);
          selv[0][1] = above;
          selv[0][2] = c0[j];
          break;
        }
        above += c0[j];
      }
    }
    __syncthreads();
    prefix |= (unsigned)uniform(selv[0][0]) << shift;
    mask |= dmask << shift;
    need -= uniform(selv[0][1]);
    nmatch = uniform(selv[0][2]);
    hb -= width;
    par = 1;
  }
  while (hb >= 0 && nmatch > kTopkRankCap) {
    const int width = min(kTopkDigitBits, hb + 1);
    const int shift = hb + 1 - width;
    const unsigned dmask = (1u << width) - 1u;
    const int nb = 1 << width;
#pragma unroll
    for (int p = 0; p < PER; ++p)
      if (p * NT + tid < Nv && (key[p] & mask) == prefix) atomicAdd(&hist[(key[p] >> shift) & dmask], 1u);
    __syncthreads();
    int c[BPT], ct = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int q = tid * BPT + j;
      c[j] = 0;
      if (q < nb) {
        unsigned *h = &hist[nb - 1 - q];
        c[j] = (int)*h;
        *h = 0u;
      }
      ct += c[j];
    }
    const int incl = wave_scan_incl(ct);
    if (lane == 63) wsum[par][wave] = incl;
    __syncthreads();
    int above = incl - ct;
    for (int w = 0; w < wave; ++w) above += wsum[par][w];
    if (ct > 0 && above < need && above + ct >= need) {
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        if (above + c[j] >= need) {
          selv[par][0] = nb - 1 - (tid * BPT + j);
          selv[par][1] = above;
          selv[par][2] = c[j];
          break;
        }
        above += c[j];
      }
    }
    __syncthreads();
    const int d = uniform(selv[par][0]);
    prefix |= (unsigned)d << shift;
    mask |= dmask << shift;
    need -= uniform(selv[par][1]);
    nmatch = uniform(selv[par][2]);
    hb -= width;
    par ^= 1;
  }
  int need_eq = need;
  int n_eq = nmatch;
  unsigned T = prefix;
  if (hb >= 0) {
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const bool mt = p * NT + tid < Nv && (key[p] & mask) == prefix;
      const unsigned long long mb = __ballot(mt);
      if (mb) {
        unsigned base = 0u;
        if (lane == 0) base = atomicAdd(ncand, (unsigned)__popcll(mb));
        base = __shfl(base, 0);
        const unsigned slot = base + (unsigned)__popcll(mb & lt);
        if (mt && slot < (unsigned)kTopkRankCap) cand[slot] = make_uint2(key[p], (unsigned)(p * NT + tid));
      }
    }
    __syncthreads();
    nmatch = min(nmatch, kTopkRankCap);
    if (tid < nmatch) {
      const uint2 me = cand[tid];
      int gt = 0, before = 0, eq = 0;
      int i = 0;
      for (; i + 4 <= nmatch; i += 4) {
        uint2 o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = cand[i + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          gt += (o[u].x > me.x) ? 1 : 0;
          eq += (o[u].x == me.x) ? 1 : 0;
          before += (o[u].x > me.x || (o[u].x == me.x && o[u].y < me.y)) ? 1 : 0;
        }
      }
      for (; i < nmatch; ++i) {
        const uint2 o = cand[i];
        gt += (o.x > me.x) ? 1 : 0;
        eq += (o.x == me.x) ? 1 : 0;
        before += (o.x > me.x || (o.x == me.x && o.y < me.y)) ? 1 : 0;
      }
      if (before == need - 1) {
        selv[par][0] = (int)me.x;
        selv[par][1] = need - gt;
        selv[par][2] = eq;
      }
    }
    __syncthreads();
    T = (unsigned)uniform(selv[par][0]);
    need_eq = uniform(selv[par][1]);
    n_eq = uniform(selv[par][2]);
    if (tid == 0) *ncand = 0u;
  }
  const unsigned long long lt = (1ull << lane) - 1ull;
  unsigned long long mk[PER];
  if (n_eq == need_eq) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      mk[p] = __ballot(p * NT + tid < Nv && key[p] >= T);
      if (lane == 0) rowcnt[1][p][wave] = __popcll(mk[p]);
    }
  } else {
    unsigned long long meq[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      meq[p] = __ballot(p * NT + tid < Nv && key[p] == T);
      if (lane == 0) rowcnt[0][p][wave] = __popcll(meq[p]);
    }
    __syncthreads();
    int eq_base = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int before = 0, row = 0;
      for (int w = 0; w < NW; ++w) {
        const int x = rowcnt[0][p][w];
        before += (w < wave) ? x : 0;
        row += x;
      }
      const bool valid = p * NT + tid < Nv;
      const bool eq = (meq[p] >> lane) & 1ull;
      const int eq_rank = eq_base + before + __popcll(meq[p] & lt);
      mk[p] = __ballot(valid && (key[p] > T || (eq && eq_rank < need_eq)));
      if (lane == 0) rowcnt[1][p][wave] = __popcll(mk[p]);
      eq_base += row;
    }
  }
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    int before = 0, row = 0;
    for (int w = 0; w < NW; ++w) {
      const int x = rowcnt[1][p][w];
      before += (w < wave) ? x : 0;
      row += x;
    }
    if ((mk[p] >> lane) & 1ull) {
      const int pos = base + before + __popcll(mk[p] & lt), idx = p * NT + tid;
      kidx[pos] = idx;
      if (kept_out) kept_out[pos] = idx;
    }
    base += row;
  }
  __syncthreads();
  return kbud;
}

// Copy of rows [r0, r1) of one compaction unit, 16-byte pieces, sixteen per
// thread in flight: row i is source row src_row(i) and destination row i.
template <typename RowFn>
__device__ __forceinline__ void copy_rows(const char *src, char *dst, int rb, int cs, int r0, int r1, int S,
                                          RowFn &&src_row) {
  constexpr int NT = kPassThreads, J = 16;
  const int tid = opaque_tid();
  const int q_begin = r0 << cs, q_end = r1 << cs;
  for (int q0 = q_begin; q0 < q_end; q0 += J * NT) {
    u32x4_t v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = min(q0 + j * NT + tid, q_end - 1);  // past the end: reload the last piece, not stored
      const int i = q >> cs, c = q & ((1 << cs) - 1);
      const int row = min(max(src_row(i), 0), S - 1);  // never read outside the layer
      v[j] = *reinterpret_cast<const u32x4_t *>(src + (size_t)row * rb + 16 * c);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = q0 + j * NT + tid;
      if (q < q_end) *reinterpret_cast<u32x4_t *>(dst + ((size_t)(q >> cs) * rb + 16 * (q & ((1 << cs) - 1)))) = v[j];
    }
  }
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------

// Item (round r) of workgroup me: pair q (sample-major, q = b * L + l) and
// chunk c; false when the workgroup has none in that round.
__device__ __forceinline__ bool pass_item_of(const PassWs &pw, int LB, int me, int r, int *q, int *c) {
  if (r == 0) {
    const int s = me - pw.E;
    if (s < 0 || s >= pw.ppr0 * pw.nch) return false;
    *q = s / pw.nch;
    *c = s - (s / pw.nch) * pw.nch;
    return *q < LB;
  }
  if (me >= pw.ppr * pw.nch) return false;
  *q = pw.ppr0 + (r - 1) * pw.ppr + me / pw.nch;
  *c = me - (me / pw.nch) * pw.nch;
  return *q < LB;
}

template <typename Tag, int D>
__global__ __launch_bounds__(kPassThreads) void aircache_pass_kernel(Shape sh, PassTables tab, PlanPtrs plan,
                                                                      PassWs pw, PassLds lo) {
  extern __shared__ __attribute__((aligned(16))) float lds_f[];
  unsigned char *lds = reinterpret_cast<unsigned char *>(lds_f);
  __shared__ int wtot[4 * kPassWaves];
  __shared__ double redd[2 * kPassWaves];
  __shared__ float redf[kPassWaves];
  constexpr int KT = pass_kt(D, Tag::kBytes);
  constexpr int RTPM = pass_rtp(D, Tag::kBytes);
  const int L = sh.L, B = sh.B, Nv = sh.Nv, LB = L * B;
  const unsigned e0 = *pw.epoch + 1u;
  const unsigned epoch = e0 == 0u ? 1u : e0;  // 0 is the tag of a zeroed record
  const int P = gridDim.x, me = blockIdx.x;
  unsigned char *ring = lds + lo.ring;

  // Every 2^21 calls: zero every record, then wait for the whole grid.
  if ((epoch & kTagEpochMask) == 0u) {
    // agent-coherent stores, so that every XCD's coherent reads see the zeros
    uint64_t *r64 = reinterpret_cast<uint64_t *>(pw.recs);
    for (size_t i = (size_t)me * kPassThreads + threadIdx.x; i < 2 * pw.rec_words; i += (size_t)P * kPassThreads)
      store_coherent(&r64[i], (uint64_t)0);
    wait_all_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
      counter_add(pw.wrapc, 1u);
      unsigned spins = 0;
      while (load_coherent(pw.wrapc) < (unsigned)P) {
        if (spin_expired(spins, pw.flags)) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
  }

  // The first item's keys load while the elite sets form (workgroups that
  // form elite sets have no round-0 item; they stage theirs after their
  // parts, and so do workgroups whose first item is in round 1).
  int q0, cfirst;
  const bool staged0 = pass_item_of(pw, LB, me, 0, &q0, &cfirst);
  if (staged0) pass_stage<Tag, D>(sh, pw, tab, q0, cfirst, 0, ring);

  // Elite sets: parts 1.. on workgroups [0, LB * (npp - 1)), part 0 and the
  // merge on [LB * (npp - 1), E).
  if (me < pw.E) {
    const int npp = pw.npp, nother = LB * (npp - 1);
    float *z = reinterpret_cast<float *>(ring);  // no round-0 item: the ring is free until the stage below
    if (me < nother) {
      const int lb = me / (npp - 1);
      elite_part<Tag, D>(sh, tab, plan, pw, lb, me - lb * (npp - 1) + 1, epoch, z, lo.z_bytes, wtot, redf);
    } else {
      for (int lb = me - nother; lb < LB; lb += pw.E - nother)
        elite_part<Tag, D>(sh, tab, plan, pw, lb, 0, epoch, z, lo.z_bytes, wtot, redf);
    }
    __syncthreads();
  }
  // (a workgroup's rounds 1, 2, ... are consecutive, so its first item is in
  // round 0 or round 1)
  if (!staged0 && pass_item_of(pw, LB, me, 1, &q0, &cfirst)) pass_stage<Tag, D>(sh, pw, tab, q0, cfirst, 0, ring);

  // Items, round by round.
  const int rounds = 1 + (LB > pw.ppr0 ? (LB - pw.ppr0 + pw.ppr - 1) / pw.ppr : 0);
  for (int r = 0; r < rounds; ++r) {
    int q, c;
    if (!pass_item_of(pw, LB, me, r, &q, &c)) {
      if (r == 0) continue;
      break;
    }
    const int tid = opaque_tid();
    PassItem it;
    it.b = q / L;
    it.l = q - it.b * L;
    it.plb = it.l * B + it.b;
    it.c = c;
    it.c0 = c * pw.width;
    it.ncol = min(pw.width, Nv - it.c0);
    it.q = tab.p[it.l];
    it.k = tab.p[L + it.l];
    int *el = reinterpret_cast<int *>(lds + lo.el);
    it.ntk = pass_elite_list(sh, pw, it.plb, epoch, el, reinterpret_cast<unsigned *>(lds + lo.scr));
    const int rows = sh.G * it.ntk;
    it.rtg = rows > 0 ? (rows + 15) >> 4 : 1;
    it.nrg = (it.rtg + RTPM - 1) / RTPM;
    float colacc[KT];
#pragma unroll
    for (int s = 0; s < KT; ++s) colacc[s] = 0.f;
    float ivacc[2] = {0.f, 0.f};  // columns tid and tid + 512
    float *colsum = reinterpret_cast<float *>(lds + lo.colsum);
    const int W = pw.width;
    for (int hg = 0; hg < pw.nhg; ++hg) {
      // this head group's tiles were staged by the previous pass or item (or
      // at launch): the loader waves wait for their loads
      if ((opaque_tid() >> 6) >= kPollWaves) wait_all_memory();
      __syncthreads();
      for (int rg = 0; rg < it.nrg; ++rg) {
        const int pidx = hg * it.nrg + rg;
        const int rtp = min(RTPM, it.rtg - rg * RTPM);
        const bool last = rg == it.nrg - 1;
        auto stage_next = [&]() {
          if (hg + 1 < pw.nhg) {
            pass_stage<Tag, D>(sh, pw, tab, q, c, hg + 1, ring);
          } else {
            int qn, cn;
            if (pass_item_of(pw, LB, me, r + 1, &qn, &cn)) pass_stage<Tag, D>(sh, pw, tab, qn, cn, 0, ring);
          }
        };
        if (rtp >= 6 && RTPM >= 6) pass_rows<Tag, D, (RTPM >= 6 ? 6 : 1)>(sh, pw, it, hg, rg, pidx, last, lds, lo, epoch, colacc, stage_next);
        else if (rtp == 5 && RTPM >= 5) pass_rows<Tag, D, (RTPM >= 5 ? 5 : 1)>(sh, pw, it, hg, rg, pidx, last, lds, lo, epoch, colacc, stage_next);
        else if (rtp == 4) pass_rows<Tag, D, 4>(sh, pw, it, hg, rg, pidx, last, lds, lo, epoch, colacc, stage_next);
        else if (rtp == 3) pass_rows<Tag, D, 3>(sh, pw, it, hg, rg, pidx, last, lds, lo, epoch, colacc, stage_next);
        else if (rtp == 2) pass_rows<Tag, D, 2>(sh, pw, it, hg, rg, pidx, last, lds, lo, epoch, colacc, stage_next);
        else pass_rows<Tag, D, 1>(sh, pw, it, hg, rg, pidx, last, lds, lo, epoch, colacc, stage_next);
      }
      // the head group's column sums, per head, then added over its heads in
      // ascending order (KV heads in ascending order overall)
      {
        const int lane = tid & 63, wave = tid >> 6;
        const int gl = wave / pw.wph, sub = wave - gl * pw.wph;
        if ((lane >> 4) == 0)
#pragma unroll
          for (int s = 0; s < KT; ++s) colsum[gl * W + (sub * KT + s) * 16 + lane] = colacc[s];
#pragma unroll
        for (int s = 0; s < KT; ++s) colacc[s] = 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = tid + j * kPassThreads;
        if (col < W)
          for (int gg = 0; gg < pw.hgs; ++gg) ivacc[j] += colsum[gg * W + col];
      }
      __syncthreads();
    }
    // the chunk's I_v and its moments
    const float inv_rows = (it.ntk > 0) ? 1.f / (float)(sh.Hq * it.ntk) : 0.f;
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = tid + j * kPassThreads;
      if (col < it.ncol) {
        const float a = ivacc[j] * inv_rows;
        ivacc[j] = a;
        plan.iv[(size_t)it.plb * Nv + it.c0 + col] = a;
        store_coherent(&pw.ivrec[(size_t)it.plb * Nv + it.c0 + col], pack_rec(a, epoch));
        sum += (double)a;
      }
    }
    sum = block_sum_d(sum, redd);
    const double mean = it.ncol > 0 ? sum / (double)it.ncol : 0.0;
    double m2 = 0.0, m3 = 0.0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = tid + j * kPassThreads;
      if (col < it.ncol) {
        const double d = (double)ivacc[j] - mean;
        m2 += d * d;
        m3 += d * d * d;
      }
    }
    block_sum_d2(m2, m3, redd);
    if (tid < 4) {
      const double v = tid == 0 ? sum : tid == 1 ? m2 : tid == 2 ? m3 : (double)it.ncol;
      const uint64_t u = __builtin_bit_cast(uint64_t, v), tag = (uint64_t)epoch << 32;
      uint64_t *mr = pw.mom + ((size_t)it.plb * pw.nch + it.c) * 8 + 2 * tid;
      store_coherent(mr, tag | (u & 0xffffffffu));
      store_coherent(mr + 1, tag | (u >> 32));
    }
  }

  // Consumer units: a contiguous range per workgroup. A unit is (sample,
  // layer, KV head, K or V) with compaction, (sample, layer) without.
  {
    const int per = pw.gather ? sh.Hkv * 2 : 1;
    const int u0 = (int)((long long)me * pw.units / P), u1 = (int)((long long)(me + 1) * pw.units / P);
    unsigned *hist = reinterpret_cast<unsigned *>(ring + lo.hist);
    int *kidx = reinterpret_cast<int *>(ring + lo.kidx);
    double *st = reinterpret_cast<double *>(ring + lo.sts);
    double *sk = st + (L + 16);
    double *bx = sk + (L + 16);
    int *bud = reinterpret_cast<int *>(bx + (L + 16));
    __shared__ int bc[4];
    {
      const int tid = opaque_tid();
      __syncthreads();  // the ring is free: every item of this workgroup is done
      for (int i = tid; i < kTopkBuckets; i += kPassThreads) hist[i] = 0u;
    }
    int have_b = -1;  // the sample whose budgets st / sk / bx / bud hold
    for (int u = u0; u < u1; ++u) {
      const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
      const int qq = u / per, rem = u - qq * per;
      const int g = rem >> 1, kv = rem & 1;
      const int b = qq / L, l = qq - b * L, plb = l * B + b;
      const bool lead = rem == 0;  // writes the plan's outputs of (l, b)
      __syncthreads();
      auto budget = [&]() {
        if (have_b != b) {
          // the sample's first unit publishes its statistics and budgets
          sample_budgets(sh, plan, pw, b, epoch, u == b * L * per, st, sk, bx, bud);
          have_b = b;
        }
        // offset of (l, b) in the layer's compacted buffer: the budgets of
        // layer l of the earlier samples, from their records
        if (wave == 0) {
          long long off = 0;
          const auto rb = coherent_rsrc(pw.brec + (size_t)l * B, (unsigned)(B * sizeof(uint64_t)));
          for (int b2 = lane; b2 < b; b2 += 64) {
            uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rb, b2 * 8, 0, 16));
            unsigned spins = 0;
            while ((unsigned)(v >> 32) != epoch) {
              if (spin_expired(spins, pw.flags)) break;
              __builtin_amdgcn_s_sleep(1);
              v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rb, b2 * 8, 0, 16));
            }
            off += (long long)sh.Hkv * ((long long)(int)(unsigned)v + sh.Nt) * sh.D;
          }
          // integer sums: exact in any order
          off = (long long)wave_sum_d((double)off);
          if (lane == 0) {
            const int rl = bud[l];
            bc[0] = rl;
            bc[1] = (int)((unsigned long long)off & 0xffffffffu);
            bc[2] = (int)((unsigned long long)off >> 32);
            if (lead) {
              plan.out_off[(size_t)l * (B + 1) + b] = off;
              if (b == B - 1)
                plan.out_off[(size_t)l * (B + 1) + B] = off + (long long)sh.Hkv * (rl + sh.Nt) * sh.D;
            }
          }
        }
        __syncthreads();
        return uniform(bc[0]);
      };
      const uint64_t *ivl = pw.ivrec + (size_t)plb * Nv;
      int32_t *kout = lead ? plan.kept + (size_t)plb * Nv : nullptr;
      int rb_;
      if (Nv <= 2048) rb_ = block_topk<4>(sh, ivl, kidx, kout, epoch, pw.flags, hist, budget);
      else if (Nv <= 4096) rb_ = block_topk<8>(sh, ivl, kidx, kout, epoch, pw.flags, hist, budget);
      else rb_ = block_topk<16>(sh, ivl, kidx, kout, epoch, pw.flags, hist, budget);
      if (!pw.gather) continue;
      const int kb = uniform(rb_);
      const long long off =
          (long long)(((unsigned long long)(unsigned)uniform(bc[2]) << 32) | (unsigned long long)(unsigned)uniform(bc[1]));
      const int n = kb + sh.Nt;
      const int rb = sh.D * pw.esize;  // bytes per row: 128, 256 or 512
      if (kb < 0 || kb > Nv || off < 0 || off + (long long)sh.Hkv * n * sh.D > pw.cap_elems) continue;
      const int cs = rb == 128 ? 3 : rb == 256 ? 4 : 5;
      const char *src = static_cast<const char *>(tab.p[(1 + kv) * L + l]) + (size_t)(b * sh.Hkv + g) * sh.S * rb;
      char *dst = static_cast<char *>(const_cast<void *>(tab.p[(3 + kv) * L + l])) + (size_t)off * pw.esize +
                  (size_t)g * n * rb;
      // the kept visual rows (ascending), then the N_t text rows
      copy_rows(src, dst, rb, cs, 0, n, sh.S, [&](int i) { return i < kb ? kidx[i] : Nv + (i - kb); });
    }
  }

  // The last workgroup to finish ends the call: the status out, the counters
  // reset, the epoch advanced.
  wait_all_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (counter_add(pw.exitc, 1u) == (unsigned)P - 1u) {
      const int f = load_coherent(pw.flags);
      *plan.status = f;
      store_coherent(pw.flags, 0);
      store_coherent(pw.wrapc, 0u);
      store_coherent(pw.exitc, 0u);
      store_coherent(pw.epoch, epoch);
    }
  }
}
