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
// Phases of one launch, every workgroup resident at once (one per CU):
//   1. Elite sets. Workgroup pt < L * B * npp forms part pt % npp (a group of
//      KV heads) of the elite window of (layer, sample) pt / npp: the text
//      softmax rows of the last text query; the workgroup of part 0 adds the
//      other parts and publishes the elite set (size and one bit mask per 64
//      text tokens). No key is loaded meanwhile, so these few dependent round
//      trips see an idle memory system.
//   2. Schedule. Every workgroup reads every elite record (one round trip)
//      and works out the same schedule: items (layer, sample, chunk) with a
//      chunk width per (layer, sample) that keeps its logits in registers
//      (fewer key tiles per wave for more elite rows), the widest for which
//      every chunk fits one round of the grid, item i on workgroup i mod P.
//   3. Items. A chunk's columns are N_v visual keys then the N_tk elite text
//      keys (the softmax runs over both). Per head group (up to eight KV
//      heads, a wave group each) and per pass of up to RTP 16-row tiles of
//      elite query rows, the chunk's keys stream through an LDS ring into
//      MFMA with the logits in registers; the exact softmax normaliser of a
//      row needs every chunk of its (layer, sample), so each pass publishes
//      the chunk's (max, sum) per row and merges every chunk's pair (fixed
//      groups of eight chunks, merged in chunk order). The chunk's I_v and its
//      moments (sum, M2, M3, count) go out as records.
//   4. Consumer units (layer, sample, KV head, K or V), a contiguous range per
//      workgroup: each combines the chunk moments of every layer of its sample
//      into s_t and s_k, computes the budgets, selects its layer's top-r_hat
//      from the published I_v and copies the kept visual rows, then the text
//      rows, into the compacted cache. Without compaction a unit is a
//      (layer, sample).
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
// Progress: elite parts wait for nothing; merges wait for parts; the schedule
// waits for merges; an item waits for the items of its own (layer, sample),
// which are consecutive in item order and at most P, so by induction on the
// lowest unfinished item every wait ends; consumer units wait only for item
// records and for the budgets of earlier samples, which the first unit of
// each sample publishes before its own top-k. Every wait is also bounded: on
// expiry the kernel flags AIRCACHE_DEV_TIMEOUT and every other wait gives up.
#pragma once

constexpr int kPassThreads = 512;
constexpr int kPassWaves = kPassThreads / 64;
constexpr unsigned kSpinLimit = 1u << 20;  // polls of one wait before it gives up
constexpr int kPassTableSlots = 256;       // layer pointers of one launch
constexpr int kXcds = 8;                   // accelerator complex dies; workgroups are dealt to them in turn
constexpr int kPassMaxPass = 1024;         // passes of one item at most (tag space)
constexpr int kRingBytes = 131072;         // key tiles in LDS per workgroup
constexpr int kKtwMax = 12;                // key tiles per wave of one chunk at most
constexpr int kMaskWords = 2048;           // elite mask words (32 tokens each) preloaded in LDS at most
constexpr int kTargetCus = 256;            // workgroups the chunk widths are sized for at least
constexpr unsigned kTagEpochMask = (1u << 21) - 1u;  // epoch bits in the row normaliser tags

// Tag of the row normaliser records of pass p in the call with this epoch.
__device__ __forceinline__ unsigned xrec_tag(unsigned epoch, int p) {
  return ((epoch & kTagEpochMask) + 1u) * (unsigned)kPassMaxPass + (unsigned)p;
}

// Per element size and head dimension: ring slots per wave (one 16-key tile
// each), row tiles per pass at most, and logit tiles a wave keeps in
// registers (key tiles x row tiles, four registers each; fewer where the
// query fragments take more registers); key tiles per wave for rtp row tiles.
__host__ __device__ constexpr int pass_ring(int D, int esize) { return kRingBytes / (kPassWaves * 16 * D * esize); }
__host__ __device__ constexpr int pass_rtp(int D, int esize) { return (esize == 2 && D == 128) ? 6 : 4; }
__host__ __device__ constexpr int pass_slots(int D, int esize) { return (esize == 4 && D == 128) ? 16 : 24; }
__host__ __device__ constexpr int pass_ktmax(int rtp, int D, int esize) {
  return pass_slots(D, esize) / rtp < kKtwMax ? pass_slots(D, esize) / rtp : kKtwMax;
}

// Chunking of one (layer, sample) from its elite count and the launch's cap
// kcap on key tiles per wave. Columns are the N_v visual keys then the N_tk
// elite text keys; chunk c covers columns [c * width, (c + 1) * width).
struct ItemPlan {
  int rtg;    // 16-row tiles of elite query rows per KV head (G * N_tk rows), at least 1
  int nrg;    // row passes per head group
  int ktw;    // key tiles per wave
  int width;  // columns per chunk
  int nch;    // chunks
};
__host__ __device__ inline ItemPlan item_plan(int ntk, int G, int Nv, int wph, int kcap, int D, int esize) {
  ItemPlan p;
  const int rtpm = pass_rtp(D, esize);
  const int rows = G * ntk;
  p.rtg = rows > 0 ? (rows + 15) / 16 : 1;
  p.nrg = (p.rtg + rtpm - 1) / rtpm;
  const int rtp0 = p.rtg < rtpm ? p.rtg : rtpm;
  const int km = pass_ktmax(rtp0, D, esize);
  int k = kcap < km ? kcap : km;
  p.ktw = k < 1 ? 1 : k;
  p.width = wph * 16 * p.ktw;
  p.nch = (Nv + ntk + p.width - 1) / p.width;
  return p;
}

// Smallest key-tile cap a launch may choose (with at most kTargetCus
// workgroups a smaller one cannot fit every chunk in one round); the host
// sizes the records for it.
__host__ __device__ inline int pass_kcap_min(int L, int B, int Nv, int wph) {
  const long long k = (long long)L * B * Nv / ((long long)wph * 16 * kTargetCus);
  return k < 1 ? 1 : (k > kKtwMax ? kKtwMax : (int)k);
}

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

// Pause between two polls of a wait: about 0.05 us, growing to about 0.2 us
// after the first polls. A poll re-reads only the records still missing
// (tens of bytes per thread), far below what would slow the streams that
// run meanwhile; a longer pause would only delay the waiter.
__device__ __forceinline__ void poll_pause(unsigned spins) {
  __builtin_amdgcn_s_sleep(2);
  if (spins > 4u) __builtin_amdgcn_s_sleep(6);
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

// Workspace of the chunked path and the launch's fixed facts. Pairs are
// (layer, sample), plb = l * B + b in the records.
struct PassWs {
  unsigned *epoch;   // [1] calls so far (the last call's epoch)
  unsigned *exitc;   // [1] workgroups finished in this call
  int *flags;        // [1] AIRCACHE_DEV_* bits found in this call
  unsigned *wrapc;   // [1] workgroups done zeroing the records (calls whose epoch is a multiple of 2^21)
  u32x4_t *recs;     // the records (parts .. brec), zeroed by those calls
  size_t rec_words;  // 16-byte words of the records
  uint64_t *parts;   // [L*B][npp][N_t] elite-window parts 1.. (pbar sums | epoch << 32)
  uint64_t *ecnt;    // [L*B] elite set size | epoch << 32
  uint64_t *emask;   // [L*B][nmw] elite set mask, 32-bit halves | epoch << 32
  uint64_t *xrec;    // [L*B][2][mnch][hgs][rows][2] row (max, sum) | tag << 32
  uint64_t *mom;     // [L*B][mnch][8] halves of chunk sum, M2, M3, count | epoch << 32
  uint64_t *ivrec;   // [L*B][N_v] I_v | epoch << 32
  uint64_t *brec;    // [L*B] budget | epoch << 32
  int npp;           // elite-window parts per pair: a divisor of H_kv
  int EW;            // workgroups [0, EW) form the elite-window parts
  int nmw;           // mask halves per pair, 2 * ceil(N_t / 64)
  int hgs;           // KV heads per head group (1, 2, 4 or 8; divides H_kv)
  int nhg;           // head groups, H_kv / hgs
  int wph;           // waves per KV head, kPassWaves / hgs
  int rows;          // rows per record slot and head, RTPM * 16
  int mnch;          // chunks of one pair at most (record stride)
  int kcap_lo;       // smallest key-tile cap the schedule may choose
  int units;         // consumer units
  int gather;        // 1: the launch also compacts
  int esize;         // bytes per element
  int64_t cap_elems; // elements of each compacted layer buffer
};

// Dynamic LDS of aircache_pass_kernel (byte offsets, 16-byte aligned). ring:
// the key tiles (kRingBytes), reused by the consumer units (top-k histogram
// and candidates, kept indices, statistics). misc: the schedule (item starts
// per pair) and the item arrays. The elite parts' text logits take ring and
// misc (no schedule exists yet, no key is staged).
struct PassLds {
  int ring, misc;                                     // regions
  int start, masks, el, colsum, red, mloc, zloc, wts;  // inside misc
  int nmask;                                          // mask words preloaded (0: none)
  int z_bytes;                                        // bytes the elite parts may use
  int kidx, hist, sts;                                // consumer arrays inside ring
  int total;
};

__host__ __device__ inline PassLds pass_lds_layout(int D, int esize, int hgs, int LB, int Nt, int Nv) {
  PassLds f;
  const int nmw = 2 * pass_words64(Nt);
  f.nmask = LB * nmw <= kMaskWords ? LB * nmw : 0;
  const int rows = pass_rtp(D, esize) * 16;
  const int wmax = (kPassWaves / hgs) * 16 * kKtwMax;  // columns of a chunk at most
  int o = 0;
  f.ring = o;
  o += kRingBytes;
  f.misc = o;
  int m = 0;
  f.start = o + m;
  m += pass_align16((LB + 1) * 4);
  f.masks = o + m;
  m += pass_align16(f.nmask * 4);
  f.el = o + m;
  m += pass_align16(Nt * 4);
  f.colsum = o + m;
  m += pass_align16(hgs * wmax * 4);
  f.red = o + m;
  m += pass_align16(kPassWaves * rows * 4);
  f.mloc = o + m;
  m += pass_align16(hgs * rows * 4);
  f.zloc = o + m;
  m += pass_align16(hgs * rows * 4);
  f.wts = o + m;
  m += pass_align16(hgs * rows * 4);
  o += pass_align16(m);
  f.total = o;
  f.z_bytes = o - f.ring;
  // consumer arrays in the ring
  int r = 0;
  f.hist = r;
  r += pass_align16((2048 + 2 * 256 + 4) * 4);  // kTopkLdsWords
  f.kidx = r;
  r += pass_align16(Nv * 4);
  f.sts = r;  // st, sk, bx: L + 16 doubles each; chunk moments; budgets
  return f;
}

// Bytes of the consumer arrays in the ring from sts on: st, sk, bx, the
// chunk moments [L][mnch][4] doubles and the budgets (L + 16 ints).
__host__ __device__ inline long long pass_sts_bytes(int L, int mnch) {
  return (long long)(L + 16) * 8 * 3 + (long long)L * mnch * 32 + (long long)(L + 16) * 4;
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


// The same logits for long text (a wave's U key tiles of one head per batch):
// for each KV head of g0.. and each query-head tile, the wave loads the query
// fragments once and key tiles wave, wave + NW, ... U at a time, every load
// of a batch issued before the first product, so twice the keys of
// elite_logits are in flight per wave.
template <typename Tag, int D, int U>
__device__ __forceinline__ void elite_logits_long(const Shape &sh, const typename Tag::store_t *q,
                                                  const typename Tag::store_t *k, int b, int g0, int ng, int nht,
                                                  int nkt, float *z, int head_floats) {
  using E = typename Tag::store_t;
  constexpr int NW = kPassWaves;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int Nt = sh.Nt, G = sh.G, Hkv = sh.Hkv;
  for (int gl = 0; gl < ng; ++gl)
    for (int ht = 0; ht < nht; ++ht) {
      const int g = g0 + gl;
      const int h = min(ht * 16 + n, G - 1);
      const E *qrow = q + ((size_t)(b * sh.Hq + g * G + h) * Nt + (Nt - 1)) * D;
      const E *kbase = k + ((size_t)(b * Hkv + g) * sh.S + sh.Nv) * D;
      for (int kt0 = wave; kt0 < nkt; kt0 += NW * U) {
        Frag<Tag> qf[D / 32], kf[U][D / 32];
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[c].load(qrow + c * 32 + grp * 8);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kt = kt0 + u * NW < nkt ? kt0 + u * NW : kt0;
          const E *krow = kbase + (size_t)min(kt * 16 + n, Nt - 1) * D;
#pragma unroll
          for (int c = 0; c < D / 32; ++c) kf[u][c].load(krow + c * 32 + grp * 8);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < D / 32; ++c) mfma_slice(acc, kf[u][c], qf[c]);
          const int kt = kt0 + u * NW;
          if (kt < nkt && ht * 16 + n < G) {
            float *zr = z + (size_t)gl * head_floats + (size_t)(ht * 16 + n) * Nt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kk = kt * 16 + grp * 4 + i;
              if (kk < Nt) zr[kk] = acc[i] * sh.scale2;
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
// tokens for the window variants) and publishes it: its size (ecnt[lb]) and
// its bit mask as 32-bit halves (emask[lb], tokens 32 h .. 32 h + 31 in half
// h); also the plan's elite list and count, and the overflow bit when the
// size exceeds the elite cap. before_store() runs before its first record
// store. N_t <= 1024.
template <typename Tag, int D, typename BeforeStoreFn>
__device__ __forceinline__ void elite_part(const Shape &sh, const PassTables &tab, const PlanPtrs &plan,
                                           const PassWs &pw, int lb, int pi, unsigned epoch, float *z,
                                           int lds_bytes, int *wtot, float *red, BeforeStoreFn &&before_store) {
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
    if (Tag::kBytes == 2 && nkt >= 8 * NW)
      elite_logits_long<Tag, D, (Tag::kBytes == 2 ? 8 : 1)>(sh, q, k, b, g0, ng, nht, nkt, z, head_floats);
    else if (per_wave >= 4) elite_logits<Tag, D, UMAX>(sh, q, k, b, g0, items, per_head, nkt, z, head_floats);
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
  before_store();
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
      poll_pause(spins);
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
  uint64_t *mrec = pw.emask + (size_t)lb * pw.nmw;
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
      store_coherent(&mrec[2 * word + lane], tag | (uint64_t)half);
    }
  }
  if (tid == 0) {
    store_coherent(&pw.ecnt[lb], tag | (uint64_t)(unsigned)total);
    plan.n_elite[lb] = total;
    if (total > sh.cap) __hip_atomic_fetch_or(pw.flags, AIRCACHE_DEV_ELITE_OVERFLOW, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // wtot and red are free again
}


// ---------------------------------------------------------------------------
// Schedule and items: cross-modal scores of one chunk ("Elite Observation
// Window", the A_vtk and I_v equations).
// ---------------------------------------------------------------------------

// Integer sum over a wave (exact in any order).
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The launch's schedule, computed alike by every workgroup from the elite
// set sizes of all pairs: the key-tile cap kcap (the smallest in
// [kcap_lo, kKtwMax] for which every chunk of every pair has a workgroup of
// its own, else kKtwMax) and start[q] = the first item of pair q (q = b L + l,
// sample-major: a sample's layers finish first), start[L B] = the items. With
// preload, the elite masks of every pair go to masks (LDS, nmw words per
// pair, plb-major) in the same round trip. Returns kcap (block-wide).
template <int D, int ESIZE>
__device__ __forceinline__ int pass_schedule(const Shape &sh, const PassWs &pw, unsigned epoch, int *start,
                                             unsigned *masks, bool preload) {
  __shared__ int ktot[kKtwMax + 1];
  __shared__ int ksel;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int L = sh.L, LB = sh.L * sh.B, P = gridDim.x;
  const int klo = pw.kcap_lo, nk = kKtwMax - klo + 1;
  if (tid <= kKtwMax) ktot[tid] = 0;
  // counts (thread q < LB) and, with preload, mask words: every load issued
  // before any is checked; short pauses (nothing streams yet)
  {
    const auto rc = coherent_rsrc(pw.ecnt, (unsigned)(LB * sizeof(uint64_t)));
    const int nmw = pw.nmw, nmask = preload ? LB * nmw : 0;
    const auto rm = coherent_rsrc(pw.emask, (unsigned)((size_t)nmask * sizeof(uint64_t)));
    for (int j0 = 0; j0 < LB || j0 < nmask; j0 += kPassThreads) {
      const int j = j0 + tid;
      int q = j, plb = 0;
      if (j < LB) {
        const int b = q / L, l = q - b * L;
        plb = l * sh.B + b;
      }
      uint64_t wc = 0, wm = 0;
      auto load = [&]() {
        if (j < LB) wc = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rc, plb * 8, 0, 16));
        if (j < nmask) wm = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rm, j * 8, 0, 16));
      };
      load();
      unsigned spins = 0;
      while ((j < LB && (unsigned)(wc >> 32) != epoch) || (j < nmask && (unsigned)(wm >> 32) != epoch)) {
        if (spin_expired(spins, pw.flags)) break;
        __builtin_amdgcn_s_sleep(2);
        load();
      }
      if (j < LB) {
        int ntk = (int)(unsigned)wc;
        start[q + 1] = ntk < 0 ? 0 : (ntk > sh.cap ? sh.cap : ntk);
      }
      if (j < nmask) {
        // tokens 32 h .. 32 h + 31 of the pair in half h; bits past N_t cleared
        const int h = j - (j / nmw) * nmw, valid = sh.Nt - 32 * h;
        const unsigned keep = valid >= 32 ? 0xffffffffu : (valid <= 0 ? 0u : ((1u << valid) - 1u));
        masks[j] = (unsigned)wm & keep;
      }
    }
  }
  __syncthreads();
  // chunks of every pair for every candidate cap, (pair, cap) combinations
  // spread over the threads; integer sums, exact in any order
  for (int x = tid; x < LB * nk; x += kPassThreads) {
    const int q = x / nk, k = klo + (x - q * nk);
    atomicAdd(&ktot[k], item_plan(start[q + 1], sh.G, sh.Nv, pw.wph, k, D, ESIZE).nch);
  }
  __syncthreads();
  if (tid == 0) {
    int sel = kKtwMax;
    for (int k = klo; k <= kKtwMax; ++k)
      if (ktot[k] <= P) {
        sel = k;
        break;
      }
    ksel = sel;
  }
  __syncthreads();
  const int kcap = uniform(ksel);
  for (int q = tid; q < LB; q += kPassThreads)
    start[q + 1] = item_plan(start[q + 1], sh.G, sh.Nv, pw.wph, kcap, D, ESIZE).nch;
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int q0 = 0; q0 < LB; q0 += 64) {
      const int q = q0 + lane;
      const int v = q < LB ? start[q + 1] : 0;
      const int incl = wave_incl_scan(v) + carry;
      if (q < LB) start[q + 1] = incl;
      carry = __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) start[0] = 0;
  }
  __syncthreads();
  return kcap;
}

// The pair of item i: the last q with start[q] <= i (wave-uniform).
__device__ __forceinline__ int pass_pair_of(const int *start, int LB, int i) {
  int lo = 0, hi = LB - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The elite list of pair plb into el (LDS, ascending, at most the elite cap
// entries), from its mask (preloaded in LDS, else read from its records);
// returns its size (block-wide).
__device__ __forceinline__ int pass_elite_list(const Shape &sh, const PassWs &pw, int plb, unsigned epoch,
                                               const unsigned *masks, bool preloaded, int *el) {
  __shared__ unsigned mw[32];
  __shared__ int pre[33];
  const int tid = opaque_tid();
  const int Nt = sh.Nt, nmw = pw.nmw;
  if (tid < nmw) {
    unsigned v;
    if (preloaded) {
      v = masks[(size_t)plb * nmw + tid];
    } else {
      const auto rm = coherent_rsrc(pw.emask + (size_t)plb * nmw, (unsigned)(nmw * sizeof(uint64_t)));
      uint64_t w = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rm, tid * 8, 0, 16));
      unsigned spins = 0;
      while ((unsigned)(w >> 32) != epoch) {
        if (spin_expired(spins, pw.flags)) break;
        poll_pause(spins);
        w = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rm, tid * 8, 0, 16));
      }
      // tokens 32 tid .. 32 tid + 31; bits past N_t cleared
      const int valid = Nt - 32 * tid;
      const unsigned keep = valid >= 32 ? 0xffffffffu : (valid <= 0 ? 0u : ((1u << valid) - 1u));
      v = (unsigned)w & keep;
    }
    mw[tid] = v;
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int h = 0; h < nmw; ++h) {
      pre[h] = s;
      s += __popc(mw[h]);
    }
    pre[nmw] = s;
  }
  __syncthreads();
  const int cap = sh.cap;
  for (int j = tid; j < Nt; j += kPassThreads) {
    const int h = j >> 5, bit = j & 31;
    const unsigned m = mw[h];
    if ((m >> bit) & 1u) {
      const int pos = pre[h] + __popc(m & ((1u << bit) - 1u));
      if (pos < cap) el[pos] = j;
    }
  }
  const int total = pre[nmw];
  __syncthreads();
  return uniform(total < cap ? total : cap);
}

struct PassItem {
  int l, b, plb, q, c, c0, ncolv, ntk, rtg, nrg, ktw, width, nchq;
  const void *q_l, *k_l;
};

// One pass of an item: RTP row tiles (rows rg * RTPM * 16 ..) of the elite
// query rows of every KV head of head group hg, against the chunk's keys:
// columns c0 .. c0 + width - 1 of N_v visual keys followed by the N_tk elite
// text keys. Wave (head gl, sub) takes key tiles sub * ktw .. of its head's
// chunk; they stream through its ring slots (R tiles in flight, refilled as
// they are read), the logits stay in registers. The pass's column sums of the
// softmax rows go to colsum (set when first, else added). pre: the pass's
// first ring tiles were issued by the previous pass of the item; nxt >= 0:
// once its own tiles are read, the pass issues the first ring tiles of the
// item's next pass (the same columns, KV heads of head group nxt), so that
// they land while this pass waits for the other chunks' row normalisers.
template <typename Tag, int D, int RTP>
__device__ __forceinline__ void pass_rows(const Shape &sh, const PassWs &pw, const PassItem &it, int hg, int rg,
                                          int pidx, bool first, bool pre, int nxt, unsigned char *lds,
                                          const PassLds &lo, unsigned epoch) {
  using E = typename Tag::store_t;
  constexpr int NT = kPassThreads;
  constexpr int RTPM = pass_rtp(D, Tag::kBytes);
  constexpr int R = pass_ring(D, Tag::kBytes);
  constexpr int KM = pass_ktmax(RTP, D, Tag::kBytes);  // key tiles per wave at most with RTP row tiles
  constexpr int kTile = 16 * D * Tag::kBytes;
  constexpr int kDma = kTile / 1024;
  constexpr int RW = RTP * 16;  // rows of one head in this pass
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int hgs = pw.hgs, wph = pw.wph, ROWS = pw.rows;
  const int gl = wave / wph, sub = wave - gl * wph;
  const int g = hg * hgs + gl;
  const int ntk = it.ntk, Rg = sh.G * ntk, Nv = sh.Nv, ktw = it.ktw, W = it.width;
  const int rt0 = rg * RTPM;
  const int *el = reinterpret_cast<const int *>(lds + lo.el);
  float *red = reinterpret_cast<float *>(lds + lo.red);
  float *mloc = reinterpret_cast<float *>(lds + lo.mloc);
  float *zloc = reinterpret_cast<float *>(lds + lo.zloc);
  float *wts = reinterpret_cast<float *>(lds + lo.wts);
  float *colsum = reinterpret_cast<float *>(lds + lo.colsum);
  unsigned char *slots = lds + lo.ring + (size_t)wave * R * kTile;
  const E *qb = static_cast<const E *>(it.q_l);
  const E *kb = static_cast<const E *>(it.k_l) + (size_t)(it.b * sh.Hkv + g) * sh.S * D;

  // query fragments first (the waits for them then cover no key tile): RTP
  // tiles of 16 elite query rows of this wave's head
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

  // column of this lane in key tile s: col0 + 16 s
  int col0 = it.c0 + sub * ktw * 16 + n;
  asm volatile("" : "+v"(col0));
  const int ncols = Nv + ntk;
  // LDS-DMA of key tile s into slot s % R: visual key col, or elite text key
  // el[col - N_v]; columns past the keys read the last visual key (masked)
  auto issue_from = [&](const E *kbase, int s) {
    const int v = col0 + s * 16;
    int row;
    if (v < Nv) row = v;
    else if (v < ncols) row = Nv + el[v - Nv];
    else row = Nv - 1;
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kbase + (size_t)row * D);
    unsigned char *dst = slots + (s % R) * kTile;
#pragma unroll
    for (int j = 0; j < kDma; ++j) load_lds16(src + 16 * grp + 64 * j, dst + 1024 * j);
  };
  auto issue = [&](int s) { issue_from(kb, s); };
  // a later pass over a chunk whose tiles all fit the ring finds them there
  const bool resident = rg > 0 && ktw <= R;
#pragma unroll
  for (int s = 0; s < R; ++s)
    if (s < ktw && !resident && !pre) issue(s);

  f32x4_t S[KM][RTP];
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    if (s < ktw) {
      // tiles s + 1 .. min(s + R, ktw) - 1 may stay in flight
      const int ahead = (s + R < ktw ? s + R : ktw) - 1 - s;
      if (!resident) wait_tiles<kDma>(ahead);
      f32x4_t acc[RTP];
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const unsigned char *slot = slots + (s % R) * kTile;
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) {
        Frag<Tag> kf;
        LdsTile<Tag>::read(kf, slot, cc, lane);
#pragma unroll
        for (int rt = 0; rt < RTP; ++rt) mfma_slice(acc[rt], qf[rt][cc], kf);
      }
      if (s + R < ktw) {
        wait_lds_reads();  // the slot's reads are done before the DMA overwrites it
        issue(s + R);
      }
      const bool ok = col0 + s * 16 < ncols;
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[s][rt][i] = ok ? acc[rt][i] * sh.scale2 : -INFINITY;
    } else {
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt) S[s][rt] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
  }
  // the next pass's first ring tiles, once every read of this pass's tiles
  // is done
  if (nxt >= 0) {
    wait_lds_reads();
    const E *kn = static_cast<const E *>(it.k_l) + (size_t)(it.b * sh.Hkv + nxt * hgs + gl) * sh.S * D;
#pragma unroll
    for (int s = 0; s < R; ++s)
      if (s < ktw) issue_from(kn, s);
  }
  // chunk-local row maxima: keys of a lane row by DPP, then the head's waves
  // in order
  float racc[RTP][4];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) racc[rt][i] = -INFINITY;
#pragma unroll
  for (int s = 0; s < KM; ++s)
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
  for (int qr = tid; qr < hgs * RW; qr += NT) {
    const int gg = qr / RW, rr = qr - gg * RW;
    float m = red[(gg * wph) * RW + rr];
    for (int w = 1; w < wph; ++w) m = fmaxf(m, red[(gg * wph + w) * RW + rr]);
    mloc[qr] = m;
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
  for (int s = 0; s < KM; ++s)
#pragma unroll
    for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // a row with no key in this chunk has maximum -inf: its weights are 0
        const float ev = Mrow[rt][i] > -INFINITY ? exp2_fast(S[s][rt][i] - Mrow[rt][i]) : 0.f;
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
  for (int qr = tid; qr < hgs * RW; qr += NT) {
    const int gg = qr / RW, rr = qr - gg * RW;
    float z = 0.f;
    for (int w = 0; w < wph; ++w) z += red[(gg * wph + w) * RW + rr];
    zloc[qr] = z;
  }
  __syncthreads();
  // publish this chunk's (max, sum) per row and merge every chunk's pair in
  // chunk order into each row's normaliser
  {
    const unsigned tag = xrec_tag(epoch, pidx);
    const int nch = it.nchq, c = it.c, mnch = pw.mnch;
    const size_t sbase = ((size_t)it.plb * 2 + (pidx & 1)) * mnch;  // (pair, slot) block, in chunks
    uint64_t *blk = pw.xrec + 2 * sbase * hgs * ROWS;
    const auto rsrc = coherent_rsrc(blk, (unsigned)((size_t)mnch * hgs * ROWS * 16));
    for (int qr = tid; qr < hgs * RW; qr += NT) {
      const int gg = qr / RW, rr = qr - gg * RW;
      const float m_own = mloc[qr], z_own = zloc[qr];
      uint64_t *rec = blk + 2 * (((size_t)c * hgs + gg) * ROWS + rr);
      store_coherent(rec, pack_rec(m_own, tag));
      store_coherent(rec + 1, pack_rec(z_own, tag));
      float M = -INFINITY, Z = 0.f;
      constexpr int kXB = 8;  // chunks' records in flight per row (one 16-byte load each)
      for (int cb = 0; cb < nch; cb += kXB) {
        u32x4_t rw[kXB];
#pragma unroll
        for (int j = 0; j < kXB; ++j) {
          const int cj = cb + j;
          const unsigned off = (cj < nch && cj != c) ? (unsigned)((((size_t)cj * hgs + gg) * ROWS + rr) * 16)
                                                     : 0xfffffff0u;  // past the end: zeros, not used
          rw[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 16));
        }
        unsigned spins = 0;
        for (;;) {
          bool ok = true;
#pragma unroll
          for (int j = 0; j < kXB; ++j) {
            const int cj = cb + j;
            ok = ok && (cj >= nch || cj == c || (rw[j][1] == tag && rw[j][3] == tag));
          }
          if (ok || spin_expired(spins, pw.flags)) break;
          poll_pause(spins);
#pragma unroll
          for (int j = 0; j < kXB; ++j) {
            const int cj = cb + j;
            if (cj < nch && cj != c && !(rw[j][1] == tag && rw[j][3] == tag))
              rw[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rsrc, (int)((((size_t)cj * hgs + gg) * ROWS + rr) * 16), 0, 16));
          }
        }
#pragma unroll
        for (int j = 0; j < kXB; ++j) {
          const int cj = cb + j;
          if (cj < nch) {
            const float mj = cj == c ? m_own : __uint_as_float(rw[j][0]);
            const float zj = cj == c ? z_own : __uint_as_float(rw[j][2]);
            if (mj > -INFINITY) {
              const float mn = fmaxf(M, mj);
              Z = Z * exp2_fast(M - mn) + zj * exp2_fast(mj - mn);
              M = mn;
            }
          }
        }
      }
      const int row = rt0 * 16 + rr;
      wts[qr] = (row < Rg && Z > 0.f && m_own > -INFINITY) ? exp2_fast(m_own - M) / Z : 0.f;
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
  float *cs = colsum + gl * W + sub * ktw * 16 + n;
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    if (s < ktw) {
      float v = 0.f;
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v += S[s][rt][i] * wrow[rt][i];
      v = sum_across_rows(v);
      if (grp == 0) cs[s * 16] = first ? v : cs[s * 16] + v;
    }
  }
  __syncthreads();  // red, mloc, zloc, wts are reused by the next pass
}

// ---------------------------------------------------------------------------
// Statistics, budgets, top-k ("Layer-wise KV Cache Budget Allocation" and the
// training-free procedure).
// ---------------------------------------------------------------------------

// The moment records of every chunk of every layer of sample b into LDS
// (mb: [L][mnch][4] doubles: sum, M2, M3, count; layer l has the chunks of
// pair q = b L + l, start[q + 1] - start[q] of them), block-wide: each thread
// takes record slots tid, tid + 512, ..., up to four at a time with every
// load in flight before any is checked, and polls until all carry the epoch.
__device__ __forceinline__ void load_sample_moments(const Shape &sh, const PassWs &pw, int b, unsigned epoch,
                                                    const int *start, double *mb) {
  constexpr int U = 4;
  const int tid = opaque_tid();
  const int mnch = pw.mnch, nrec = sh.L * mnch;
  // one resource for every record (a per-lane resource would cost a loop
  // over the distinct values of the wave); past the end reads zeros
  const auto rm = coherent_rsrc(pw.mom, (unsigned)((size_t)sh.L * sh.B * mnch * 64));
  auto used = [&](int i) {
    if (i >= nrec) return false;
    const int l = i / mnch, c = i - (i / mnch) * mnch, q = b * sh.L + l;
    return c < start[q + 1] - start[q];
  };
  auto base_of = [&](int i) {
    const int l = i / mnch, c = i - (i / mnch) * mnch;
    return (unsigned)(((size_t)(l * sh.B + b) * mnch + c) * 64);
  };
  for (int i0 = tid; i0 < nrec; i0 += U * kPassThreads) {
    uint64_t w[U][8];
    bool use[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kPassThreads;
      use[u] = used(i);
      const unsigned base = use[u] ? base_of(i) : 0xffffff00u;  // past the end: zeros, not used
#pragma unroll
      for (int f = 0; f < 8; ++f)
        w[u][f] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rm, (int)(base + 8 * f), 0, 16));
    }
    unsigned spins = 0;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int f = 0; f < 8; ++f) ok = ok && (!use[u] || (unsigned)(w[u][f] >> 32) == epoch);
      if (ok || spin_expired(spins, pw.flags)) break;
      poll_pause(spins);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bool rec_ok = true;
#pragma unroll
        for (int f = 0; f < 8; ++f) rec_ok = rec_ok && (unsigned)(w[u][f] >> 32) == epoch;
        if (use[u] && !rec_ok) {
          const unsigned base = base_of(i0 + u * kPassThreads);
#pragma unroll
          for (int f = 0; f < 8; ++f)
            w[u][f] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rm, (int)(base + 8 * f), 0, 16));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kPassThreads;
      if (use[u])
#pragma unroll
        for (int f = 0; f < 4; ++f)
          mb[(size_t)i * 4 + f] = __builtin_bit_cast(double, (w[u][2 * f] & 0xffffffffu) | (w[u][2 * f + 1] << 32));
    }
  }
}

// s_t and s_k of layer l ("Layer-wise KV Cache Budget Allocation", the s_t
// and s_k equations) from its chunks' moments in LDS (m4: [nch][4] = sum,
// M2, M3, count), by the 16 lanes of one DPP row: s_t = the sum of the chunk
// sums; the central moments about the layer mean mu follow exactly from the
// chunks' (with d_c = mean_c - mu): M2 = sum_c M2_c + n_c d_c^2 and
// M3 = sum_c M3_c + 3 d_c M2_c + n_c d_c^3. Lane i of the row takes chunks
// i, i + 16, ... in that order, then fixed-order row sums, so every unit that
// computes it gets the same bits. Every lane of the row returns the values.
__device__ __forceinline__ void chunk_stats(const Shape &sh, int nch, const double *m4, double *st_out,
                                            double *sk_out) {
  const int i16 = threadIdx.x & 15;
  double sum = 0.0, cnt = 0.0;
  for (int c = i16; c < nch; c += 16) {
    sum += m4[(size_t)c * 4];
    cnt += m4[(size_t)c * 4 + 3];
  }
  sum = row16_sum_d(sum);
  cnt = row16_sum_d(cnt);  // whole numbers: exact
  const double mu = cnt > 0.0 ? sum / cnt : 0.0;
  double m2 = 0.0, m3 = 0.0;
  for (int c = i16; c < nch; c += 16) {
    const double *v = m4 + (size_t)c * 4;
    const double n = v[3];
    if (n > 0.0) {
      const double d = v[0] / n - mu;
      m2 += v[1] + n * d * d;
      m3 += v[2] + 3.0 * d * v[1] + n * d * d * d;
    }
  }
  m2 = row16_sum_d(m2);
  m3 = row16_sum_d(m3);
  const int Nv = sh.Nv;
  const double sigma = sqrt(m2 / (double)(Nv - 1));
  const double sk =
      (sigma > 0.0) ? (m3 / (sigma * sigma * sigma)) * ((double)Nv / ((double)(Nv - 1) * (double)(Nv - 2))) : 0.0;
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
// the same order as the serial form (ascending layers, as the host's budget
// rule), four lanes' values read ahead.
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
// (st, sk, bx: L + 16 doubles each, bud: L + 16 ints; start: the launch's
// item starts per pair): each wave combines the
// chunk moments of layers wave, wave + 8, ...; then wave 0 forms the budgets
// ("Layer-wise KV Cache Budget Allocation", the r_hat equation over the
// sample's layers, in double precision and the oracle's order). With publish,
// the plan's s_t, s_k, budget and budget_x of the sample and its budget
// records (read by the units of later samples for their offsets) go out.
__device__ __forceinline__ void sample_budgets(const Shape &sh, const PlanPtrs &plan, const PassWs &pw, int b,
                                               unsigned epoch, bool publish, const int *start, double *st, double *sk,
                                               double *bx, int *bud, double *mb) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int L = sh.L, B = sh.B;
  load_sample_moments(sh, pw, b, epoch, start, mb);
  __syncthreads();
  // layer l on DPP row l % 4 of wave (l / 4) % 8: 32 layers at a time
  for (int l0 = 4 * wave; l0 < L; l0 += 4 * kPassWaves) {
    const int l = l0 + (lane >> 4);
    const int q = b * L + (l < L ? l : L - 1);
    double a, c;
    chunk_stats(sh, l < L ? start[q + 1] - start[q] : 0, mb + (size_t)(l < L ? l : 0) * pw.mnch * 4, &a, &c);
    if ((lane & 15) == 0 && l < L) {
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
      layer_budget(sh, sums, l, st[l], sk[l], &x, &r);
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
      poll_pause(spins);
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
// Non-temporal stores: the compacted cache is not read again in this launch.
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
      if (q < q_end) store_nt(reinterpret_cast<u32x4_t *>(dst + ((size_t)(q >> cs) * rb + 16 * (q & ((1 << cs) - 1)))), v[j]);
    }
  }
}


// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------

template <typename Tag, int D>
__device__ __forceinline__ void pass_rows_dispatch(int rtp, const Shape &sh, const PassWs &pw, const PassItem &it,
                                                   int hg, int rg, int pidx, bool first, bool pre, int nxt,
                                                   unsigned char *lds, const PassLds &lo, unsigned epoch) {
  constexpr int RTPM = pass_rtp(D, Tag::kBytes);
  if (RTPM >= 6 && rtp >= 6)
    pass_rows<Tag, D, (RTPM >= 6 ? 6 : 1)>(sh, pw, it, hg, rg, pidx, first, pre, nxt, lds, lo, epoch);
  else if (RTPM >= 5 && rtp == 5)
    pass_rows<Tag, D, (RTPM >= 5 ? 5 : 1)>(sh, pw, it, hg, rg, pidx, first, pre, nxt, lds, lo, epoch);
  else if (rtp == 4) pass_rows<Tag, D, 4>(sh, pw, it, hg, rg, pidx, first, pre, nxt, lds, lo, epoch);
  else if (rtp == 3) pass_rows<Tag, D, 3>(sh, pw, it, hg, rg, pidx, first, pre, nxt, lds, lo, epoch);
  else if (rtp == 2) pass_rows<Tag, D, 2>(sh, pw, it, hg, rg, pidx, first, pre, nxt, lds, lo, epoch);
  else pass_rows<Tag, D, 1>(sh, pw, it, hg, rg, pidx, first, pre, nxt, lds, lo, epoch);
}

template <typename Tag, int D>
__global__ __launch_bounds__(kPassThreads) void aircache_pass_kernel(Shape sh, PassTables tab, PlanPtrs plan,
                                                                      PassWs pw, PassLds lo) {
  extern __shared__ __attribute__((aligned(16))) float lds_f[];
  unsigned char *lds = reinterpret_cast<unsigned char *>(lds_f);
  __shared__ int wtot[4 * kPassWaves];
  __shared__ double redd[2 * kPassWaves];
  __shared__ float redf[kPassWaves];
  constexpr int RTPM = pass_rtp(D, Tag::kBytes);
  const int L = sh.L, B = sh.B, Nv = sh.Nv, LB = L * B;
  const unsigned e0 = *pw.epoch + 1u;
  const unsigned epoch = e0 == 0u ? 1u : e0;  // 0 is the tag of a zeroed record
  const int P = gridDim.x, me = blockIdx.x;
  unsigned char *ring = lds + lo.ring;

  // Every 2^21 calls: zero every record, then wait for the whole grid. Run
  // once per workgroup before its first record store (an elite workgroup
  // after its first part's logits, the others before the schedule), so that
  // no load waits for the epoch before the elite windows' first loads.
  bool wrapped = false;
  auto wrap_once = [&]() {
    if (wrapped) return;
    wrapped = true;
    if ((epoch & kTagEpochMask) != 0u) return;
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
        poll_pause(spins);
      }
    }
    __syncthreads();
  };

  // 1. Elite-window parts: part pt of pair pt / npp on workgroup pt mod EW.
  if (me < pw.EW) {
    float *z = reinterpret_cast<float *>(ring);
    for (int pt = me; pt < LB * pw.npp; pt += pw.EW) {
      const int lb = pt / pw.npp;
      elite_part<Tag, D>(sh, tab, plan, pw, lb, pt - lb * pw.npp, epoch, z, lo.z_bytes, wtot, redf, wrap_once);
    }
  }
  wrap_once();
  __syncthreads();

  // 2. The schedule, alike in every workgroup.
  int *start = reinterpret_cast<int *>(lds + lo.start);
  unsigned *masks = reinterpret_cast<unsigned *>(lds + lo.masks);
  const bool preload = lo.nmask > 0;
  const int kcap = pass_schedule<D, Tag::kBytes>(sh, pw, epoch, start, masks, preload);
  const int n_items = uniform(start[LB]);

  // 3. Items i = v, v + P, ... with v this workgroup's rank counted XCD by
  // XCD (workgroups go to the eight XCDs in turn): the chunks of one (layer,
  // sample) are consecutive items, so they run on one XCD and read the
  // pair's elite queries through one L2.
  const int vme = (P % kXcds == 0) ? (me % kXcds) * (P / kXcds) + me / kXcds : me;
  for (int i = vme; i < n_items; i += P) {
    const int tid = opaque_tid();
    PassItem it;
    it.q = pass_pair_of(start, LB, i);
    it.c = i - start[it.q];
    it.nchq = start[it.q + 1] - start[it.q];
    it.b = it.q / L;
    it.l = it.q - it.b * L;
    it.plb = it.l * B + it.b;
    it.q_l = tab.p[it.l];
    it.k_l = tab.p[L + it.l];
    it.ntk = pass_elite_list(sh, pw, it.plb, epoch, masks, preload, reinterpret_cast<int *>(lds + lo.el));
    const ItemPlan ip = item_plan(it.ntk, sh.G, Nv, pw.wph, kcap, D, Tag::kBytes);
    it.rtg = ip.rtg;
    it.nrg = ip.nrg;
    it.ktw = ip.ktw;
    it.width = ip.width;
    it.c0 = it.c * ip.width;
    {
      const int left = Nv - it.c0;
      it.ncolv = left < 0 ? 0 : (left > ip.width ? ip.width : left);
    }
    const int W = ip.width;
    float *colsum = reinterpret_cast<float *>(lds + lo.colsum);
    float ivacc[3] = {0.f, 0.f, 0.f};  // columns tid, tid + 512, tid + 1024
    // a pass that streams its tiles gets its first ring tiles issued by the
    // pass before it (a later row group of a chunk that fits the ring finds
    // its tiles there and streams nothing)
    constexpr int R = pass_ring(D, Tag::kBytes);
    bool pre = false;
    for (int hg = 0; hg < pw.nhg; ++hg) {
      for (int rg = 0; rg < it.nrg; ++rg) {
        const int rtp = min(RTPM, it.rtg - rg * RTPM);
        int nxt = -1;
        if (rg + 1 < it.nrg) nxt = it.ktw > R ? hg : -1;
        else if (hg + 1 < pw.nhg) nxt = hg + 1;
        pass_rows_dispatch<Tag, D>(rtp, sh, pw, it, hg, rg, hg * it.nrg + rg, rg == 0, pre, nxt, lds, lo, epoch);
        pre = nxt >= 0;
      }
      // the head group's column sums, added over its heads in ascending order
      // (KV heads in ascending order overall)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
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
    for (int j = 0; j < 3; ++j) {
      const int col = tid + j * kPassThreads;
      if (col < it.ncolv) {
        const float a = ivacc[j] * inv_rows;
        ivacc[j] = a;
        plan.iv[(size_t)it.plb * Nv + it.c0 + col] = a;
        store_coherent(&pw.ivrec[(size_t)it.plb * Nv + it.c0 + col], pack_rec(a, epoch));
        sum += (double)a;
      }
    }
    sum = block_sum_d(sum, redd);
    const double mean = it.ncolv > 0 ? sum / (double)it.ncolv : 0.0;
    double m2 = 0.0, m3 = 0.0;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int col = tid + j * kPassThreads;
      if (col < it.ncolv) {
        const double d = (double)ivacc[j] - mean;
        m2 += d * d;
        m3 += d * d * d;
      }
    }
    block_sum_d2(m2, m3, redd);
    if (tid < 4) {
      const double v = tid == 0 ? sum : tid == 1 ? m2 : tid == 2 ? m3 : (double)it.ncolv;
      const uint64_t u = __builtin_bit_cast(uint64_t, v), tag = (uint64_t)epoch << 32;
      uint64_t *mr = pw.mom + ((size_t)it.plb * pw.mnch + it.c) * 8 + 2 * tid;
      store_coherent(mr, tag | (u & 0xffffffffu));
      store_coherent(mr + 1, tag | (u >> 32));
    }
  }

  // 4. Consumer units: a contiguous range per workgroup. A unit is (sample,
  // layer, KV head, K or V) with compaction, (sample, layer) without.
  {
    const int per = pw.gather ? sh.Hkv * 2 : 1;
    const int u0 = (int)((long long)me * pw.units / P), u1 = (int)((long long)(me + 1) * pw.units / P);
    unsigned *hist = reinterpret_cast<unsigned *>(ring + lo.hist);
    int *kidx = reinterpret_cast<int *>(ring + lo.kidx);
    double *st = reinterpret_cast<double *>(ring + lo.sts);
    double *sk = st + (L + 16);
    double *bx = sk + (L + 16);
    double *mb = bx + (L + 16);                          // [L][mnch][4] chunk moments
    int *bud = reinterpret_cast<int *>(mb + (size_t)L * pw.mnch * 4);
    __shared__ int bc[4];
    {
      const int tid = opaque_tid();
      __syncthreads();  // the ring is free: every item of this workgroup is done
      for (int i = tid; i < kTopkBuckets; i += kPassThreads) hist[i] = 0u;
    }
    int have_b = -1;    // the sample whose budgets st / sk / bx / bud hold
    int have_plb = -1;  // the (layer, sample) whose kept list kidx and offset bc hold
    int have_kb = 0;
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
          sample_budgets(sh, plan, pw, b, epoch, u == b * L * per, start, st, sk, bx, bud, mb);
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
              poll_pause(spins);
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
      // the units of one (layer, sample) are consecutive: its top-k once per
      // workgroup
      int rb_ = have_kb;
      if (plb != have_plb) {
        if (Nv <= 2048) rb_ = block_topk<4>(sh, ivl, kidx, kout, epoch, pw.flags, hist, budget);
        else if (Nv <= 4096) rb_ = block_topk<8>(sh, ivl, kidx, kout, epoch, pw.flags, hist, budget);
        else rb_ = block_topk<16>(sh, ivl, kidx, kout, epoch, pw.flags, hist, budget);
        have_plb = plb;
        have_kb = uniform(rb_);
      }
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
