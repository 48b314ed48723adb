// Steps 2-5 of the AirCache pass in one persistent launch ("chunked" path),
// included by aircache.hip inside namespace aircache.
//
// Method: paper-notes page "AirCache: Activating Inter-Modal Relevancy KV
// Cache Compression for Efficient Large Vision-Language Model Inference",
// "Elite Observation Window" (the A_vtk and I_v equations) and "Layer-wise KV
// Cache Budget Allocation" (the s_t, s_k and r_hat equations).
//
// Before the items: one workgroup per (layer, sample) forms its elite set
// and publishes the size and bit mask; every workgroup reads every size and
// works out the same chunk schedule by itself. Meanwhile each wave loads the
// first key tiles of the item it took in the previous call into its LDS ring
// (used only if it gets that item again).
//
// Work item = (layer, sample, row group, column chunk): a workgroup takes a
// run of columns (visual keys, then the elite text keys) of every KV head of
// one (layer, sample) and up to four 16-row tiles of elite-query rows per KV
// head. Its logits stay in registers. The exact softmax normaliser of a row
// needs every chunk's contribution, so the chunks of one row group swap
// per-row (max, sum) pairs through epoch-tagged records. A chunk's slice of
// I_v is then final (one row group) or the sum of its row groups' partial
// column sums (the last row group to finish, a counter election, adds them in
// order); the slice and its moments are published as tagged records.
//
// After the items: the workgroup of a (layer, sample)'s first item combines
// the chunks' moments into s_t and s_k, publishes them, then runs its top-k,
// whose first radix pass overlaps the wait for the records of every layer of
// the samples up to its own, from which it computes the budget and the
// compacted offsets it needs; those and the kept indices are published as
// tagged records. Workgroups with nothing left take compaction units (the
// text rows, then the kept rows, of one layer, sample and KV head) from a
// ticket counter.
//
// Records: every cross-workgroup value is written as (32-bit payload | epoch
// << 32) words with agent-coherent stores, so a reader that sees the call's
// epoch has the value; the epoch advances once per call and the last
// workgroup to finish resets the few counters.
//
// All workgroups are co-resident (one 512-thread workgroup per CU, the LDS use
// admitting no second), and a workgroup only waits for items that come no
// later in the item order than its own or, after its items, for records that
// other workgroups publish once their own items are done; so every wait ends.
// Each wait is also bounded: on expiry the kernel sets AIRCACHE_DEV_TIMEOUT
// and every other wait of the launch gives up too.
#pragma once

constexpr int kFusedThreads = 512;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedSlots = 24;      // logit registers per wave: key tiles x row tiles (f32x4 each)
constexpr int kFusedRtMax = 4;       // row tiles per KV head in one item (query fragments in registers)
constexpr int kFusedMaxItems = 256;  // work items one workgroup can take
constexpr int kFusedTargetCus = 256; // workgroups the chunk schedule assumes at most
constexpr int kFusedRingMin = 16384;  // LDS bytes the top-k select needs (its histogram and candidates)
constexpr unsigned kSpinLimit = 1u << 20;  // polls of one wait before it gives up

// Key tiles per wave that the logit registers hold for rtp row tiles
// (kFusedSlots / rtp, rtp in 1..4).
__host__ __device__ constexpr int fused_ktmax(int rtp) {
  return rtp <= 1 ? kFusedSlots : rtp == 2 ? kFusedSlots / 2 : rtp == 3 ? kFusedSlots / 3 : kFusedSlots / 4;
}

// One poll of a bounded wait. True when the wait must end: this one ran out
// (the timeout bit is set) or another one in the launch already did.
__device__ __forceinline__ bool spin_expired(unsigned &spins, int *status) {
  if (++spins > kSpinLimit) {
    atomicOr(status, AIRCACHE_DEV_TIMEOUT);
    return true;
  }
  if ((spins & 255u) == 0u && (load_coherent(status) & AIRCACHE_DEV_TIMEOUT)) return true;
  return false;
}

// Chunking of one (layer, sample) from its elite count and the launch-wide
// cap kcap on key tiles per wave; the host sizes the workspace with it and
// the device schedules with it. Columns are the N_v visual keys followed by
// the N_tk elite text keys (the softmax runs over both); chunk c covers
// columns [c * width, (c + 1) * width). A (layer, sample) with more elite rows
// holds fewer key tiles per wave in registers, so it gets narrower chunks, and
// beyond kFusedRtMax row tiles per KV head its rows split into row groups.
struct ChunkPlan {
  int rtg;      // 16-row tiles per KV head (G * N_tk rows), at least 1
  int nrg;      // row groups
  int rtp;      // row tiles per KV head in the largest row group
  int ktw;      // key tiles per wave
  int width;    // columns per chunk
  int nchunks;  // chunks of the (layer, sample)
};

__host__ __device__ inline ChunkPlan fused_chunk_plan(int ntk, int G, int Nv, int wph, int kcap) {
  ChunkPlan p;
  const int rows = G * ntk;
  p.rtg = rows > 0 ? (rows + 15) / 16 : 1;
  p.nrg = (p.rtg + kFusedRtMax - 1) / kFusedRtMax;
  p.rtp = p.rtg < kFusedRtMax ? p.rtg : kFusedRtMax;
  const int ktmax = fused_ktmax(p.rtp);
  int k = kcap < ktmax ? kcap : ktmax;
  if (k < 1) k = 1;
  p.ktw = k;
  p.width = wph * 16 * k;
  const int cols = Nv + ntk;
  p.nchunks = (cols + p.width - 1) / p.width;
  return p;
}

// Smallest cap on key tiles per wave the launch may choose: with at most
// kFusedTargetCus workgroups, a smaller cap cannot fit every chunk in one
// round. The host sizes the workspace for this cap (the most chunks).
__host__ __device__ inline int fused_kcap_min(int L, int B, int Nv, int wph) {
  const long long k = (long long)L * B * Nv / ((long long)wph * 16 * kFusedTargetCus);
  return k < 1 ? 1 : (k > kFusedSlots ? kFusedSlots : (int)k);
}

// Workspace of the chunked path. Every counter is reset by its last arriver
// and the epoch advances at the end of each call; every record carries the
// epoch of the call that wrote it, so stale records of earlier calls never
// match. The workspace must be zero before its first use.
struct FusedWs {
  unsigned *epoch;        // [1] calls so far
  unsigned *exitc;        // [1] workgroups finished in this call
  uint64_t *parts;        // [L*B][npp][N_t] elite-window parts 1.. of pbar, (value | epoch << 32)
  int npp;                // parts per (layer, sample): a divisor of H_kv
  int kcap_lo;            // smallest key-tile cap per wave the schedule may choose (fused_kcap_min)
  uint64_t *erec;         // [L*B][erec_stride] elite size, mask halves, each | epoch << 32
  int erec_stride;        // words per elite record: 1 + 2 * ceil(N_t / 64)
  unsigned *cnt_chunk;    // [L*B][max_chunks] finished row groups per chunk
  uint64_t *xrec;         // [L*B][rec_stride][2] (row max | epoch << 32), (row sum | epoch << 32)
  uint64_t *mom;          // [L*B][max_chunks][8] halves of chunk sum, M2, M3, count, each | epoch << 32
  uint64_t *ivrec;        // [L*B][N_v] I_v | epoch << 32
  uint64_t *keptrec;      // [L*B][N_v] kept index | epoch << 32
  uint64_t *srec;         // [L*B][4] halves of s_t and s_k, each | epoch << 32
  float *part;            // [L*B][max_chunks][max_rg][wmax] row-group column sums
  int rec_stride;         // records per (layer, sample)
  int max_chunks;         // chunks per (layer, sample) at most
  int max_rg;             // row groups per (layer, sample) at most
  int wmax;               // columns per chunk at most
  // compaction in the same launch (gather != 0)
  uint64_t *hint;         // [kFusedHintSlots] first item of each workgroup in the last call
  int gather;
  int esize;              // bytes per element
  int64_t cap_elems;      // elements of each compacted layer buffer
  unsigned *gticket;      // [1] copy units handed out
  uint64_t *grec;         // [L*B][4] budget, out_off halves, each | epoch << 32
};

// Key tiles in flight per wave: about 128 KB of LDS ring per workgroup. The
// stream of a CU is bound by the bytes it has in flight over the load
// latency, and this is the most the LDS leaves room for.
__host__ __device__ constexpr int fused_ring_depth(int tile_bytes) {
  return tile_bytes >= 8192 ? 2 : tile_bytes >= 4096 ? 4 : 8;
}

// Dynamic LDS of cross_score_fused_kernel (byte offsets, 16-byte aligned).
// ring: the key tiles of the waves, also the staging of pbar before the
// items and the top-k's histogram after them; ntk: the elite count of every
// (layer, sample); sts: the
// s_t and s_k a budget needs; items / owed: this workgroup's work items and
// the (layer, sample) pairs whose top-k it owes.
struct FusedLds {
  int ring, el, colsum, red, mloc, wts, items, owed, ntk, sts, total;
};
__host__ __device__ inline int fused_align16(int x) { return (x + 15) & ~15; }
__host__ __device__ inline int fused_words64(int Nt) { return (Nt + 63) >> 6; }
__host__ __device__ inline FusedLds fused_lds_layout(int tile_bytes, int ring_depth, int cap, int Hkv, int LB,
                                                     int Nt) {
  FusedLds f;
  const int wph = kFusedWaves / Hkv;
  int o = 0;
  f.ring = o;
  const int ring = kFusedWaves * ring_depth * tile_bytes;
  o += fused_align16(ring > kFusedRingMin ? ring : kFusedRingMin);
  f.el = o;
  o += fused_align16(cap * 4);
  f.colsum = o;
  o += fused_align16(Hkv * wph * 16 * kFusedSlots * 4);
  f.red = o;
  o += fused_align16(kFusedWaves * kFusedRtMax * 16 * 4);
  f.mloc = o;
  o += fused_align16(Hkv * kFusedRtMax * 16 * 4);
  f.wts = o;
  o += fused_align16(Hkv * kFusedRtMax * 16 * 4);
  f.items = o;
  o += fused_align16(kFusedMaxItems * 4);
  f.owed = o;
  o += fused_align16(kFusedMaxItems * 4);
  f.ntk = o;
  o += fused_align16(LB * 4);
  f.sts = o;
  o += fused_align16((LB + 16) * 16);  // reads run up to 15 entries past each array
  f.total = o;
  return f;
}

// The thread index, opaque to the optimiser: values derived from it are
// recomputed where they are used instead of being hoisted out of the item
// loop and kept live (and spilled) across the whole kernel.
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// A value every lane of the wave holds, moved to a scalar register: buffer
// resources and addresses built from it are then scalar too (a resource in
// vector registers costs a loop over the distinct values of the wave).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 2^x by the hardware instruction. Results below 2^-126 flush to zero, which
// in a softmax weight (at most 1 against a row sum of at least 1) is far
// below float32 resolution.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint64_t pack_rec(float v, unsigned epoch) {
  return ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(v);
}

// Integer sum over the 64 lanes of a wave (wave-uniform result).
__device__ __forceinline__ int wave_sum_i(int v) { return (int)wave_sum((float)v); }  // exact below 2^24

// Block-wide exclusive scan over kFusedThreads threads (wtot: kFusedWaves ints).
__device__ __forceinline__ int fused_block_scan(int v, int *wtot, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kFusedWaves; ++w) {
    const int x = wtot[w];
    if (w < wave) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Block-wide double sum over kFusedThreads threads in a fixed order.
__device__ __forceinline__ double fused_block_sum_d(double v, double *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_d(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kFusedWaves; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Two block-wide double sums at once, each in the order of fused_block_sum_d.
// red: 2 * kFusedWaves doubles.
__device__ __forceinline__ void fused_block_sum_d2(double &a, double &b, double *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_sum_d(a);
  b = wave_sum_d(b);
  if (lane == 0) {
    red[wave] = a;
    red[kFusedWaves + wave] = b;
  }
  __syncthreads();
  double ta = 0.0, tb = 0.0;
  for (int w = 0; w < kFusedWaves; ++w) {
    ta += red[w];
    tb += red[kFusedWaves + w];
  }
  __syncthreads();
  a = ta;
  b = tb;
}

// Layer pointers of one launch of the chunked kernel, L entries each: text
// queries at [0, L), keys at [L, 2L) and, when the launch also compacts,
// values at [2L, 3L), compacted keys at [3L, 4L) and compacted values at
// [4L, 5L).
constexpr int kFusedTableSlots = 256;
struct FusedTables {
  const void *p[kFusedTableSlots];
};

// Everything an item needs to know about itself.
struct FusedItem {
  int l, b, plb, r, c, ntk;
  ChunkPlan cp;
  const void *q;  // layer's text queries
  const void *k;  // layer's keys
};

// A workgroup's guess of its first item, kept from the previous call: the
// (layer, sample), the column chunk and the key tiles per wave.
constexpr int kFusedHintSlots = 1024;
__host__ __device__ inline uint64_t fused_hint(int plb, int c, int ktw) {
  return 1ull | ((uint64_t)(unsigned)plb << 1) | ((uint64_t)(unsigned)c << 24) | ((uint64_t)(unsigned)ktw << 48);
}

// While the elite sets are formed the HBM is idle: the first tiles of wave
// `wave`'s key run in the item the hint guesses go into that wave's ring
// slots, as fused_pass would stage them (the calling wave issues the loads).
// fused_pass uses them only if the item is that one (and they are visual
// keys), else it stages over them.
template <typename Tag, int D>
__device__ __forceinline__ void fused_prestage(const Shape &sh, const FusedTables &tab, uint64_t hint,
                                               unsigned char *lds, const FusedLds &lo, int wave) {
  using E = typename Tag::store_t;
  constexpr int kTileBytes = 16 * D * Tag::kBytes;
  constexpr int kDma = kTileBytes / 1024;
  constexpr int kRing = fused_ring_depth(kTileBytes);
  if (!(hint & 1ull)) return;
  const int plb = (int)((hint >> 1) & 0x7fffff), c = (int)((hint >> 24) & 0xffffff), ktw = (int)(hint >> 48);
  const int L = sh.L, B = sh.B, Hkv = sh.Hkv, Nv = sh.Nv;
  if (plb >= L * B || ktw < 1 || ktw > kFusedSlots) return;
  const int lane = opaque_tid() & 63;
  const int n = lane & 15, grp = lane >> 4;
  const int wph = kFusedWaves / Hkv;
  const int g = wave / wph, sub = wave - g * wph;
  const int W = wph * 16 * ktw;
  const int nt = ktw < kRing ? ktw : kRing;
  // only visual keys (text keys need the elite list); 64-bit, so that no hint
  // value can wrap the row index
  const long long v0l = (long long)c * W + (long long)sub * ktw * 16;
  if (v0l + nt * 16 > Nv) return;
  const int v0 = (int)v0l;
  const int l = plb / B, b = plb - l * B;
  const E *kb = static_cast<const E *>(tab.p[L + l]) + (size_t)(b * Hkv + g) * sh.S * D;
  unsigned char *ring = lds + lo.ring + (size_t)wave * kRing * kTileBytes;
  for (int s = 0; s < nt; ++s) {
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kb + (size_t)(v0 + s * 16 + n) * D);
#pragma unroll
    for (int j = 0; j < kDma; ++j) load_lds16(src + 16 * grp + 64 * j, ring + s * kTileBytes + 1024 * j);
  }
}

// One item's row group: RTP row tiles per KV head starting at row tile rt0.
// Stream the chunk's columns (visual keys, then the elite text keys) with the
// logits in registers, exchange row (max, sum) with the other chunks of the
// row group, and leave the column sums of exp2(S - M) / Z over the group's
// rows, per KV head, in colsum.
template <typename Tag, int D, int RTP>
__device__ __forceinline__ void fused_pass(const Shape &sh, const FusedWs &fw, const FusedItem &it, int rt0,
                                           unsigned char *lds, const FusedLds &lo, unsigned epoch, int *status,
                                           uint64_t hint) {
  using E = typename Tag::store_t;
  constexpr int NW = kFusedWaves;
  constexpr int KTMAX = fused_ktmax(RTP);
  constexpr int kTileBytes = 16 * D * Tag::kBytes;
  constexpr int kDma = kTileBytes / 1024;
  constexpr int kRing = fused_ring_depth(kTileBytes);
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int Hkv = sh.Hkv, G = sh.G, Nv = sh.Nv;
  const int wph = NW / Hkv;
  const int g = wave / wph, sub = wave - g * wph;
  const int ntk = it.ntk, Rg = G * ntk;
  const int ncols = Nv + ntk;
  const int ktw = it.cp.ktw, W = it.cp.width, c = it.c;
  const int *el = reinterpret_cast<const int *>(lds + lo.el);
  float *colsum = reinterpret_cast<float *>(lds + lo.colsum);
  float *red = reinterpret_cast<float *>(lds + lo.red);
  float *mloc = reinterpret_cast<float *>(lds + lo.mloc);
  float *wts = reinterpret_cast<float *>(lds + lo.wts);
  unsigned char *ring = lds + lo.ring + (size_t)wave * kRing * kTileBytes;
  const E *kb = static_cast<const E *>(it.k) + (size_t)(it.b * Hkv + g) * sh.S * D;
  const E *qb = static_cast<const E *>(it.q);

  // query fragments of this wave's head, RTP tiles of 16 elite-query rows
  Frag<Tag> qf[RTP][D / 32];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt) {
    const int r = (rt0 + rt) * 16 + n;
    if (r < Rg) {
      const int hl = r / ntk, e = r - hl * ntk;
      const E *qrow = qb + ((size_t)(it.b * sh.Hq + g * G + hl) * sh.Nt + el[e]) * D;
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) qf[rt][cc].load(qrow + cc * 32 + grp * 8);
    } else {
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) qf[rt][cc].zero();
    }
  }
  // Key tiles of this wave: the contiguous run sub * ktw .. sub * ktw + ktw - 1
  // of the chunk; column v < N_v is visual key v, N_v <= v < N_v + N_tk the
  // elite text key el[v - N_v].
  int vbase = c * W + sub * ktw * 16 + n;  // this lane's column in stage 0
  asm volatile("" : "+v"(vbase));
  auto stage = [&](int s) {
    const int v = vbase + s * 16;
    int row = v < Nv ? v : (v < ncols ? Nv + el[v - Nv] : Nv - 1);
    asm volatile("" : "+v"(row));
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kb + (size_t)row * D);
    unsigned char *slot = ring + (s % kRing) * kTileBytes;
    if (s >= kRing) wait_lds_reads();
#pragma unroll
    for (int j = 0; j < kDma; ++j) load_lds16(src + 16 * grp + 64 * j, slot + 1024 * j);
  };
  f32x4_t S[KTMAX][RTP];
  // first tiles already in this wave's ring (fused_prestage) when the item is
  // the one the hint guessed and those tiles are visual keys
  const bool staged = hint == fused_hint(it.plb, c, ktw) &&
                      c * W + sub * ktw * 16 + (ktw < kRing ? ktw : kRing) * 16 <= Nv;
  if (!staged)
#pragma unroll
    for (int s = 0; s < kRing; ++s)
      if (s < ktw) stage(s);
#pragma unroll
  for (int s = 0; s < KTMAX; ++s) {
    if (s < ktw) {
      const int ahead = ktw - 1 - s;
      wait_tiles<kDma>(ahead < kRing - 1 ? ahead : kRing - 1);
      f32x4_t acc[RTP];
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const unsigned char *slot = ring + (s % kRing) * kTileBytes;
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) {
        Frag<Tag> kf;
        LdsTile<Tag>::read(kf, slot, cc, lane);
#pragma unroll
        for (int rt = 0; rt < RTP; ++rt) mfma_slice(acc[rt], qf[rt][cc], kf);
      }
      if (s + kRing < ktw) stage(s + kRing);
      const bool ok = vbase + s * 16 < ncols;
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[s][rt][i] = ok ? acc[rt][i] * sh.scale2 : -INFINITY;
    }
  }
  // chunk-local row maxima: keys of a lane row (DPP), then the head's waves in
  // order. The key tiles are the outer loop, so the 4 * RTP row chains
  // interleave instead of waiting on each other.
  constexpr int RW = RTP * 16;  // rows of one head in this pass
  float racc[RTP][4];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) racc[rt][i] = -INFINITY;
#pragma unroll
  for (int s = 0; s < KTMAX; ++s)
    if (s < ktw)
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
  if (tid < Hkv * RW) {
    const int gg = tid / RW, rr = tid - gg * RW;
    float m = red[(gg * wph) * RW + rr];
    for (int w = 1; w < wph; ++w) m = fmaxf(m, red[(gg * wph + w) * RW + rr]);
    mloc[gg * RW + rr] = m;
  }
  __syncthreads();
  // exponentials in place and chunk-local row sums (each row summed in key
  // order; the rows interleave)
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) racc[rt][i] = 0.f;
  float Mrow[RTP][4];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) Mrow[rt][i] = mloc[g * RW + rt * 16 + grp * 4 + i];
#pragma unroll
  for (int s = 0; s < KTMAX; ++s)
    if (s < ktw)
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
  // publish this chunk's (max, sum) per row, then merge every chunk's pair in
  // chunk order into the row's normaliser
  if (tid < Hkv * RW) {
    const int gg = tid / RW, rr = tid - gg * RW;
    float z = 0.f;
    for (int w = 0; w < wph; ++w) z += red[(gg * wph + w) * RW + rr];
    const float m_own = mloc[gg * RW + rr];
    const int row = rt0 * 16 + rr;
    const int rows_h = it.cp.rtg * 16;
    const size_t rbase = (size_t)it.plb * fw.rec_stride;
    uint64_t *rec = fw.xrec + 2 * (rbase + ((size_t)c * Hkv + gg) * rows_h + row);
    store_coherent(rec, pack_rec(m_own, epoch));
    store_coherent(rec + 1, pack_rec(z, epoch));
    const auto rsrc = coherent_rsrc(fw.xrec + 2 * rbase, (unsigned)((size_t)fw.rec_stride * 16));
    float M = -INFINITY, Z = 0.f;
    const int nch = it.cp.nchunks;
    constexpr int kXB = 8;  // chunks' records in flight per thread (one 16-byte load each)
    for (int c0 = 0; c0 < nch; c0 += kXB) {
      // every record of the batch loaded, then the batch polled as a whole
      // (unconditional reloads) and merged in chunk order
      u32x4_t rw[kXB];
      auto load_batch = [&]() {
#pragma unroll
        for (int j = 0; j < kXB; ++j) {
          const int cj = c0 + j;
          const unsigned off = (cj < nch && cj != c)
                                   ? (unsigned)((((size_t)cj * Hkv + gg) * rows_h + row) * 16)
                                   : 0xfffffff0u;  // past the end: reads zeros, not used
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
          ok = ok && (cj >= nch || cj == c || (rw[j][1] == epoch && rw[j][3] == epoch));
        }
        if (ok || spin_expired(spins, status)) break;
        __builtin_amdgcn_s_sleep(2);
        load_batch();
      }
#pragma unroll
      for (int j = 0; j < kXB; ++j) {
        const int cj = c0 + j;
        if (cj >= nch) break;
        const float mj = cj == c ? m_own : __uint_as_float(rw[j][0]);
        const float zj = cj == c ? z : __uint_as_float(rw[j][2]);
        if (mj > -INFINITY) {
          const float mn = fmaxf(M, mj);
          Z = Z * exp2_fast(M - mn) + zj * exp2_fast(mj - mn);
          M = mn;
        }
      }
    }
    wts[gg * RW + rr] = (row < Rg && Z > 0.f) ? exp2_fast(m_own - M) / Z : 0.f;
  }
  __syncthreads();
  // column sums of this pass over the head's rows; one wave owns a column.
  // The row weights go to registers first (the compiler cannot tell that the
  // column-sum stores leave them alone, so it would read them again per tile).
  float wrow[RTP][4];
#pragma unroll
  for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[rt][i] = wts[g * RW + rt * 16 + grp * 4 + i];
  int cbase = g * W + sub * ktw * 16 + n;
  asm volatile("" : "+v"(cbase));
  float *cs_lane = colsum + cbase;
#pragma unroll
  for (int s = 0; s < KTMAX; ++s) {
    if (s < ktw) {
      float v = 0.f;
#pragma unroll
      for (int rt = 0; rt < RTP; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v += S[s][rt][i] * wrow[rt][i];
      v = sum_across_rows(v);
      // text columns are summed too and never read
      if (grp == 0) cs_lane[s * 16] = v;
    }
  }
  __syncthreads();
}

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

// Inclusive prefix sum over the 64 lanes of a wave: a scan inside each row of
// 16 lanes by DPP row shifts, then the row totals added in with readlane.
__device__ __forceinline__ int wave_scan_incl(int v) {
  const int lane = threadIdx.x & 63;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  // totals of rows 0, 1 and 2 (read before any row is offset)
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  if (lane >= 16) v += r0;
  if (lane >= 32) v += r1;
  if (lane >= 48) v += r2;
  return v;
}

// Top-r_hat of one (layer, sample) by the 512 threads of a workgroup: thread
// t holds the keys of indices t, t + 512, t + 1024, ... in registers (each load
// instruction reads 64 consecutive scores per wave). I_v >= 0, so the float32
// bits order like the values, and the order that decides the kept set is
// (key descending, index ascending). The bits above the highest bit in which
// the minimum and maximum keys differ are common to all keys and skipped.
// While more than kTopkRankCap keys match the prefix found so far, a radix
// pass counts the next (up to) kTopkDigitBits bits of the matching keys into
// one LDS histogram, a block scan over the buckets in descending digit order
// finds the bucket holding the need-th key, and the prefix grows by that
// digit (one pass usually leaves a few dozen keys, since 11 bits below the
// first differing bit resolve the scores to about 1/64 of an octave); the
// first pass's counts and their scan come before the budget is known. The
// keys left are then copied to LDS and each is ranked against the others
// directly; the one of rank need - 1 is the threshold T. Kept: every key > T
// plus the lowest-index keys equal to T up to the count still needed, in
// ascending index order (each 64-index run of a wave is ranked with a ballot
// and the runs are placed by their counts).
// lds: kTopkLdsWords words, the histogram zero on entry (and left zero).
constexpr int kTopkDigitBits = 11;
constexpr int kTopkBuckets = 1 << kTopkDigitBits;
constexpr int kTopkRankCap = 256;
constexpr int kTopkLdsWords = kTopkBuckets + 2 * kTopkRankCap + 4;
static_assert(kTopkLdsWords * 4 <= kFusedRingMin, "the top-k select must fit the ring's minimum size");
template <int PER, typename BudgetFn>
__device__ __forceinline__ void block_topk(const Shape &sh, const uint64_t *iv_l, int32_t *kept, uint64_t *kept_rec,
                                           unsigned epoch, int *status, unsigned *lds, BudgetFn &&get_budget) {
  constexpr int NT = kFusedThreads, NW = kFusedWaves;
  constexpr int BPT = kTopkBuckets / NT;  // buckets per thread in a scan
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
      if (ok || spin_expired(spins, status)) break;
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int p = 0; p < PER; ++p)
        if (p * NT + tid < Nv && (unsigned)(kw[p] >> 32) != epoch)
          kw[p] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(riv, (p * NT + tid) * 8, 0, 16));
    }
  }
  unsigned key[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) key[p] = (unsigned)kw[p];
  float fmin = INFINITY, fmax = 0.f;  // keys as floats: same order
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
  int hb = diff ? 31 - __clz((int)diff) : -1;  // highest bit in which keys can differ
  unsigned mask = (hb < 0) ? 0xffffffffu : (hb >= 31) ? 0u : ~((2u << hb) - 1u);
  unsigned prefix = kmin & mask;
  // The first radix pass does not depend on the budget: its counts and their
  // scan over the buckets (descending digits) are done before asking for the
  // budget, whose wait they overlap; only the choice of bucket waits for it.
  // Thread t: the buckets of descending positions t * BPT .. t * BPT + BPT - 1.
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
        *h = 0u;  // zero again for the next pass or call
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
        kept[i] = i;
        store_coherent(&kept_rec[i], ((uint64_t)epoch << 32) | (uint64_t)(unsigned)i);
      }
    return;
  }
  int need = kbud;  // keys still to take among those matching the prefix
  int nmatch = Nv;  // keys matching the prefix
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
        *h = 0u;  // zero again for the next pass or call
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
  // T, the count of keys equal to T still to take, and of all keys equal to T
  int need_eq = need;
  int n_eq = nmatch;  // with every bit resolved, the keys matching the prefix all equal T
  unsigned T = prefix;
  if (hb >= 0) {
    // the nmatch <= kTopkRankCap keys matching the prefix, ranked directly
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const bool mt = p * NT + tid < Nv && (key[p] & mask) == prefix;
      const unsigned long long mb = __ballot(mt);
      if (mb) {
        unsigned base = 0u;
        if (lane == 0) base = atomicAdd(ncand, (unsigned)__popcll(mb));
        base = __shfl(base, 0);
        if (mt) cand[base + __popcll(mb & lt)] = make_uint2(key[p], (unsigned)(p * NT + tid));
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
        selv[par][2] = eq;  // every key equal to T matches the prefix
      }
    }
    __syncthreads();
    T = (unsigned)uniform(selv[par][0]);
    need_eq = uniform(selv[par][1]);
    n_eq = uniform(selv[par][2]);
    if (tid == 0) *ncand = 0u;
  }
  // per run (p, wave) of 64 indices: the kept keys. When every key equal to T
  // is kept (the usual case) that is key >= T; otherwise the keys equal to T
  // are ranked by index first.
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
    int eq_base = 0;  // keys equal to T at lower indices than this wave's run
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
      kept[pos] = idx;
      store_coherent(&kept_rec[pos], ((uint64_t)epoch << 32) | (uint64_t)(unsigned)idx);
    }
    base += row;
  }
}

// ceil(a / b) for 0 <= a < 2^20 and 1 <= b, without an integer division:
// the float estimate is within one of floor(a / b) and is corrected exactly.
__device__ __forceinline__ int ceil_div_small(int a, int b) {
  int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
  if (q * b > a) --q;
  if ((q + 1) * b <= a) ++q;
  return q + (q * b < a ? 1 : 0);
}

// Logits of the last text query of every query head of KV heads g0.. over
// the text keys, scaled, into z (rows of N_t floats, G rows per KV head):
// items (KV head, query-head tile, key tile) wave, wave + NW, ..., U at a
// time per wave, every load of the U items issued before the first product.
// Items past the end repeat the wave's first of the batch, not stored.
template <typename Tag, int D, int U>
__device__ __forceinline__ void fused_elite_logits(const Shape &sh, const typename Tag::store_t *q,
                                                   const typename Tag::store_t *k, int b, int g0, int items,
                                                   int per_head, int nkt, float *z, int head_floats) {
  using E = typename Tag::store_t;
  constexpr int NW = kFusedWaves;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, grp = lane >> 4;
  const int Nt = sh.Nt, G = sh.G, Hkv = sh.Hkv;
  for (int it0 = wave; it0 < items; it0 += NW * U) {
    // the loads of U items before any product; rows past the ends read a
    // valid row whose results are never stored
    Frag<Tag> qf[U][D / 32], kf[U][D / 32];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * NW < items ? it0 + u * NW : it0;  // past the end: the wave's first again
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
    // every load in flight before the first product (the scheduler would
    // otherwise issue each item's loads after the previous item's products)
    __builtin_amdgcn_sched_barrier(0);
    // products of every item, including the repeats past the end: a product
    // under a branch would have its loads moved after the previous item's
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

// Phase 0, elite sets ("Elite Observation Window", the Att and k equations).
// A (layer, sample) lb is split into npp parts of H_kv / npp KV heads, one
// workgroup each. For every KV head g of the part and each of its G query
// heads, the logits of the last text query over the N_t text keys come from
// MFMA (16 text keys as the A operand, up to 16 query heads as the B operand)
// into LDS; each wave normalises whole rows (max, sum of exp2); the part's
// pbar_j is the sum over its KV heads in ascending order of the sums over
// their query heads in ascending order. KV heads are taken in groups whose
// logits fit the LDS (G * N_t floats per head; the host keeps one head within
// it). Parts 1.. are published as epoch-tagged words; the workgroup of part 0
// adds them to its own in ascending part order, forms the set
// { j : pbar_j >= alpha max pbar } as one bit mask per 64 text tokens, and
// publishes it with agent-coherent stores: erec[lb] = [size, then each mask
// word as two 32-bit halves]; also the plan's elite list and count (the
// overflow flag is set from the counts). N_t <= 1024 (two entries per
// thread).
template <typename Tag, int D>
__device__ __forceinline__ void fused_elite_part(const Shape &sh, const FusedTables &tab, const PlanPtrs &plan,
                                                 const FusedWs &fw, int lb, int pi, unsigned epoch, float *z,
                                                 int lds_bytes, int *wtot, float *red) {
  using E = typename Tag::store_t;
  constexpr int NT = kFusedThreads, NW = kFusedWaves, EP = 2;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int l = lb / sh.B, b = lb - (lb / sh.B) * sh.B;
  const int Nt = sh.Nt, G = sh.G, Hkv = sh.Hkv, npp = fw.npp;
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
    // U items per wave at a time, U no more than a wave has (float32
    // fragments are twice as wide: at most two items, or the operands spill)
    const int per_wave = (items + NW - 1) / NW;
    constexpr int UMAX = Tag::kBytes == 4 ? 2 : 4;
    if (per_wave >= 4) fused_elite_logits<Tag, D, UMAX>(sh, q, k, b, g0, items, per_head, nkt, z, head_floats);
    else if (per_wave >= 2) fused_elite_logits<Tag, D, 2>(sh, q, k, b, g0, items, per_head, nkt, z, head_floats);
    else fused_elite_logits<Tag, D, 1>(sh, q, k, b, g0, items, per_head, nkt, z, head_floats);
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
    uint64_t *part = fw.parts + ((size_t)lb * npp + pi) * Nt;
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (tid + e * NT < Nt) store_coherent(&part[tid + e * NT], pack_rec(pb[e], epoch));
    return;
  }
  if (npp > 1) {
    // the other parts, every load issued before any is checked
    constexpr int PM = 7;  // npp <= 8
    const auto rp = coherent_rsrc(fw.parts + (size_t)lb * npp * Nt, (unsigned)((size_t)npp * Nt * sizeof(uint64_t)));
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
      if (ok || spin_expired(spins, plan.status)) break;
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
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < EP; ++e) {
    // the elite set, or the contiguous window of the last sh.window text tokens
    const int j = tid + e * NT;
    mk[e] = __ballot(j < Nt && (sh.window > 0 ? j >= Nt - sh.window : pb[e] >= thr));
    cnt += __popcll(mk[e]);
  }
  // words before this wave's, in token order: word (e, wave) comes after all
  // words of pass e' < e and the words (e, wave' < wave)
  if (lane == 0)
#pragma unroll
    for (int e = 0; e < EP; ++e) wtot[e * NW + wave] = __popcll(mk[e]);
  __syncthreads();
  const int ntw = fused_words64(Nt);
  uint64_t *rec = fw.erec + (size_t)lb * fw.erec_stride;
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
  }
  __syncthreads();  // wtot and red are free again
}

// Every workgroup: the elite count of every (layer, sample), clamped to the
// elite cap, into ntk (LDS), from the merges' epoch-tagged records; with
// flag_overflow, counts above the cap set the overflow status bit.
__device__ __forceinline__ void fused_elite_counts(const Shape &sh, const FusedWs &fw, unsigned epoch, int *status,
                                                   int *ntk, bool flag_overflow) {
  const int LB = sh.L * sh.B;
  const auto rr = coherent_rsrc(fw.erec, (unsigned)((size_t)LB * fw.erec_stride * sizeof(uint64_t)));
  for (int lb = opaque_tid(); lb < LB; lb += kFusedThreads) {
    const int off = (int)((size_t)lb * fw.erec_stride * sizeof(uint64_t));
    uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 16));
    unsigned spins = 0;
    while ((unsigned)(v >> 32) != epoch) {
      if (spin_expired(spins, status)) break;
      __builtin_amdgcn_s_sleep(2);
      v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 16));
    }
    const int t = (int)(unsigned)v;
    ntk[lb] = t < sh.cap ? t : sh.cap;
    if (flag_overflow && t > sh.cap) atomicOr(status, AIRCACHE_DEV_ELITE_OVERFLOW);
  }
  __syncthreads();
}

// The elite list of lb, ascending, into el (LDS, ntk entries) from the
// merge's mask words. scr: LDS for N_t / 64 mask words.
__device__ __forceinline__ void fused_elite_list(const Shape &sh, const FusedWs &fw, int lb, int ntk, unsigned epoch,
                                                 int *status, int *el, unsigned long long *scr) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int ntw = fused_words64(sh.Nt);
  const auto rr = coherent_rsrc(fw.erec + (size_t)lb * fw.erec_stride, (unsigned)(fw.erec_stride * sizeof(uint64_t)));
  if (tid < 2 * ntw) {
    const int off = (1 + tid) * (int)sizeof(uint64_t);
    uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 16));
    unsigned spins = 0;
    while ((unsigned)(v >> 32) != epoch) {
      if (spin_expired(spins, status)) break;
      __builtin_amdgcn_s_sleep(2);
      v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, 16));
    }
    reinterpret_cast<unsigned *>(scr)[tid] = (unsigned)v;  // little-endian: halves form the word
  }
  __syncthreads();
  for (int w = wave; w < ntw; w += kFusedWaves) {
    int base = 0;
    for (int u = 0; u < w; ++u) base += __popcll(scr[u]);
    const unsigned long long mk = scr[w];
    const int pos = base + __popcll(mk & ((1ull << lane) - 1ull));
    if (((mk >> lane) & 1ull) && pos < ntk) el[pos] = w * 64 + lane;
  }
}

// Work schedule of this workgroup, block-wide, from the elite counts ntk
// (LDS, [layer][sample]); pair p = (b, l) = (p / L, p % L) in sample-major
// order is held by lane p % 64 of a wave (up to eight per lane, L * B <=
// 512). The cap on key tiles per wave is the smallest (narrowest chunks, most
// workgroups busy) whose items all fit one round of the grid, the widest when
// none does: items are non-increasing in the cap, and no cap below
// fw.kcap_lo fits, so wave w counts the items of cap kcap_lo + w (eight caps
// per round, one barrier each). Items go in the order (b, l, row group,
// chunk); workgroup me takes items me, me + P, ...; wave 0 writes those of
// this workgroup to item[] ((b * L + l) << 16 | index in the (layer,
// sample)), hdr[0] = cap and hdr[1] = item count. Sums are exact integer wave
// scans. One wave issues an instruction every four cycles at best and this
// runs on every call, so each wave's share is kept short.
__device__ __forceinline__ void fused_schedule(const Shape &sh, const FusedWs &fw, const int *ntk_lds, int me, int P,
                                               int *item, int *hdr, int *red) {
  constexpr int NW = kFusedWaves;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int L = sh.L, B = sh.B, Nv = sh.Nv, LB = L * B;
  const int wph = kFusedWaves / sh.Hkv, W0 = wph * 16;
  const int nj = (LB + 63) >> 6;  // pairs per lane at most
  // pair p: row groups, key-tile cap of its row tiles, columns
  auto pair = [&](int p, int &nrg, int &km, int &cols) {
    const int b = ceil_div_small(p + 1, L) - 1, l = p - b * L;
    const int t = p < LB ? ntk_lds[l * B + b] : 0;
    const int rtg = t > 0 ? (sh.G * t + 15) >> 4 : 1;
    nrg = p < LB ? (rtg + kFusedRtMax - 1) / kFusedRtMax : 0;
    km = fused_ktmax(rtg < kFusedRtMax ? rtg : kFusedRtMax);
    cols = Nv + t;
  };
  auto chunks = [&](int km, int cols, int kc) {
    const int k = kc < km ? kc : km;
    return ceil_div_small(cols, W0 * k);
  };
  const int P_sched = P < kFusedTargetCus ? P : kFusedTargetCus;
  int kc = kFusedSlots;
#pragma unroll 1
  for (int k0 = fw.kcap_lo; k0 < kFusedSlots; k0 += NW) {
    const int mine = k0 + wave;  // this wave's candidate
    int v = 0;
#pragma unroll 1
    for (int j = 0; j < nj; ++j) {
      int nrg, km, cols;
      pair(lane + 64 * j, nrg, km, cols);
      v += nrg * chunks(km, cols, mine);
    }
    v = __builtin_amdgcn_readlane(wave_scan_incl(v), 63);
    if (lane == 0) red[wave] = (mine <= kFusedSlots && v <= P_sched) ? 1 : 0;
    __syncthreads();
    int found = -1;
    for (int w = NW - 1; w >= 0; --w)
      if (red[w]) found = k0 + w;
    __syncthreads();  // red is read before the next round writes it
    if (found >= 0) {
      kc = found;
      break;
    }
  }
  if (wave != 0) return;
  // exclusive prefix of the item counts in pair order, and this workgroup's items
  int base = 0;
#pragma unroll 1
  for (int j = 0; j < nj; ++j) {
    const int p = lane + 64 * j;
    int nrg, km, cols;
    pair(p, nrg, km, cols);
    const int nit = nrg > 0 ? nrg * chunks(km, cols, kc) : 0;
    const int incl = wave_scan_incl(nit);
    const int start = base + incl - nit;
    base += __builtin_amdgcn_readlane(incl, 63);
    if (nit > 0) {
      // first item index >= start congruent to me mod P, and its slot k
      const int d = start - me;
      int k = d <= 0 ? 0 : ceil_div_small(d, P);
      for (int i = me + k * P; i < start + nit; i += P, ++k)
        if (k < kFusedMaxItems) item[k] = (p << 16) | (i - start);
    }
  }
  if (lane == 0) {
    hdr[0] = kc;
    hdr[1] = base;  // items in all
  }
}

// Statistics of one (layer, sample) from its chunks' moments, by wave 0:
// lane c holds chunk c; the chunks combine pairwise in a fixed tree (at
// stride st, chunk c, a multiple of 2 st, absorbs chunk c + st), so the
// result does not depend on which workgroup computes it. s_t and s_k
// ("Layer-wise KV Cache Budget Allocation", the s_t and s_k equations) go to
// the plan and, tagged with the epoch, to the (layer, sample)'s record.
__device__ __forceinline__ void fused_layer_stats(const Shape &sh, const PlanPtrs &plan, const FusedWs &fw, int plb,
                                                  int nch, unsigned epoch) {
  const int lane = threadIdx.x & 63;
  const auto rm = coherent_rsrc(fw.mom + (size_t)plb * fw.max_chunks * 8, (unsigned)(fw.max_chunks * 64));
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  if (lane < nch) {
    // wait for chunk lane's record: eight words tagged with this call's epoch
    uint64_t w[8];
    unsigned spins = 0;
    for (;;) {
#pragma unroll
      for (int f = 0; f < 8; ++f)
        w[f] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rm, lane * 64 + 8 * f, 0, 16));
      bool ok = true;
#pragma unroll
      for (int f = 0; f < 8; ++f) ok = ok && (unsigned)(w[f] >> 32) == epoch;
      if (ok || spin_expired(spins, plan.status)) break;
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
      v[f] = __builtin_bit_cast(double, (w[2 * f] & 0xffffffffu) | (w[2 * f + 1] << 32));
  }
  double sum = v[0];
  Moments m{v[3], v[3] > 0.0 ? v[0] / v[3] : 0.0, v[1], v[2]};
  for (int st = 1; st < nch; st <<= 1) {
    const int src = lane + st;
    const double osum = __shfl(sum, src), on = __shfl(m.n, src), omean = __shfl(m.mean, src);
    const double om2 = __shfl(m.m2, src), om3 = __shfl(m.m3, src);
    if ((lane & (2 * st - 1)) == 0 && src < nch) {
      m = combine_moments(m, Moments{on, omean, om2, om3});
      sum = sum + osum;
    }
  }
  if (lane == 0) {
    const int Nv = sh.Nv;
    const double sigma = sqrt(m.m2 / (double)(Nv - 1));
    const double sk = (sigma > 0.0) ? (m.m3 / (sigma * sigma * sigma)) *
                                          ((double)Nv / ((double)(Nv - 1) * (double)(Nv - 2)))
                                    : 0.0;
    plan.s_t[plb] = sum;
    plan.s_k[plb] = sk;
    // each 32-bit half of s_t and s_k in its own word with the epoch: a
    // reader that sees the epoch in all four words has the values, with no
    // ordering between the stores needed
    uint64_t *r = fw.srec + (size_t)plb * 4;
    const uint64_t a = __builtin_bit_cast(uint64_t, sum), c = __builtin_bit_cast(uint64_t, sk);
    const uint64_t tag = (uint64_t)epoch << 32;
    const uint64_t lo32 = 0xffffffffu;
    store_coherent(r + 0, tag | (a & lo32));
    store_coherent(r + 1, tag | (a >> 32));
    store_coherent(r + 2, tag | (c & lo32));
    store_coherent(r + 3, tag | (c >> 32));
  }
}

// budget_sums over LDS with the values read sixteen at a time, every read of
// a batch issued before the first addition (one LDS round trip per batch), and
// no branches. The two sums take the same additions in the same order, so the
// same result (a padded entry adds +0.0 to a non-negative sum). The shift is a
// minimum, exact in any order: four interleaved chains of v_min_f64 instead of
// one compare-and-select chain, then +0.0 unless some s_k is negative (which
// is what the serial form keeps: it starts at +0.0 and takes only values below
// it). Reads run up to 15 entries past L (the LDS arrays are padded).
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
// +0.0 unless some s_k is negative, as the serial form keeps; the shifted
// values are formed in every lane at once; the two sums then take the same
// additions in the same order as the serial form, four lanes' values read
// ahead of their additions.
// One wave issues an instruction every four cycles at best, so the serial
// part is kept to the additions.
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
  // lanes past L add +0.0, which leaves these non-negative sums unchanged
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

// Budget of (layer l, sample b) for its top-k, block-wide: waits for the
// statistics records of every layer of samples 0..b, then (wave 0, lane bb
// for sample bb) the budgets of layer l of those samples ("Layer-wise KV
// Cache Budget Allocation", the r_hat equation, over the sample's layers in
// order); writes the plan's budget, budget_x and out_off of (l, b) (and the
// layer's total after the last sample), leaves the budget in bc[0] and the
// offset's 32-bit halves in bc[2], bc[3], and returns the budget.
// sts: LDS for 2 * (L * (b + 1) + 16) doubles.
__device__ __forceinline__ int fused_budget(const Shape &sh, const PlanPtrs &plan, const FusedWs &fw, int l, int b,
                                            unsigned epoch, double *sts, int *bc) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int L = sh.L, B = sh.B;
  const int nrec = L * (b + 1);
  double *st = sts, *sk = sts + nrec + 16;  // [bb][l], each with 16 entries of padding
  // one resource for all records (a per-lane resource would cost a loop over
  // the distinct values of the wave)
  const auto rr = coherent_rsrc(fw.srec, (unsigned)((size_t)L * B * 32));
  for (int i = tid; i < nrec; i += kFusedThreads) {
    const int bb = ceil_div_small(i + 1, L) - 1, ll = i - bb * L;
    const int off = (int)(((size_t)ll * B + bb) * 32);
    uint64_t w[4];
    unsigned spins = 0;
    for (;;) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr, off + 8 * j, 0, 16));
      bool ok = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) ok = ok && (unsigned)(w[j] >> 32) == epoch;
      if (ok || spin_expired(spins, plan.status)) break;
      __builtin_amdgcn_s_sleep(2);
    }
    const uint64_t lo32 = 0xffffffffu;
    st[i] = __builtin_bit_cast(double, (w[0] & lo32) | (w[1] << 32));
    sk[i] = __builtin_bit_cast(double, (w[2] & lo32) | (w[3] << 32));
  }
  __syncthreads();
  if (wave == 0) {
    double off = 0.0;  // element offsets, exact in double (below 2^53)
    // one sample: its layers across the lanes; several: one sample per lane
    const bool across = b == 0 && L <= 64;
    BudgetSums sums0;
    if (across) sums0 = budget_sums_wave(L, st, sk);
    for (int bb = across ? 0 : lane; bb <= b && (!across || lane == 0); bb += 64) {
      const BudgetSums sums = across ? sums0 : budget_sums_lds(L, st + (size_t)bb * L, sk + (size_t)bb * L);
      double x;
      int bud;
      layer_budget(sh, sums, st[(size_t)bb * L + l], sk[(size_t)bb * L + l], &x, &bud);
      const double seg = (double)sh.Hkv * (double)(bud + sh.Nt) * (double)sh.D;
      if (bb < b) off += seg;
      else {
        const int plb = l * B + b;
        plan.budget[plb] = bud;
        if (plan.bx) plan.bx[plb] = x;
        bc[0] = bud;
        bc[1] = (int)seg;  // below 2^31: one layer's segment of one sample
      }
    }
    off = wave_sum_d(off);
    if (lane == 0) {
      plan.out_off[(size_t)l * (B + 1) + b] = (int64_t)off;
      bc[2] = (int)((uint64_t)(int64_t)off & 0xffffffffu);
      bc[3] = (int)((uint64_t)(int64_t)off >> 32);
      if (b == B - 1) plan.out_off[(size_t)l * (B + 1) + B] = (int64_t)off + (int64_t)bc[1];
    }
  }
  __syncthreads();
  return uniform(bc[0]);
}

// Copy of rows [r0, r1) of one compaction unit, 16-byte pieces, sixteen per
// thread in flight: row i is source row src_row(i) and destination row i.
template <typename RowFn>
__device__ __forceinline__ void fused_copy_rows(const char *src, char *dst, int rb, int cs, int r0, int r1, int S,
                                                RowFn &&src_row) {
  constexpr int NT = kFusedThreads, J = 16;
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

// One compaction unit ("compress" of the training-free procedure): the kept
// visual rows (ascending) and then all N_t text rows of one (layer, sample, KV
// head) of K or V, copied to the sample's segment of the compacted layer
// buffer at element offset off. The text rows go first, while the kept
// indices (epoch-tagged words the top-k writes) are still arriving. A budget
// or offset outside the buffer is skipped, as in kv_gather_kernel.
// kidx: LDS for N_v ints.
__device__ __forceinline__ void fused_gather_unit(const Shape &sh, const PlanPtrs &plan, const FusedWs &fw,
                                                  const char *src_l, char *dst_l, int b, int g, int plb, int bud,
                                                  int64_t off, unsigned epoch, int *kidx) {
  constexpr int NT = kFusedThreads, KW = 16;  // N_v <= KW * NT
  const int tid = opaque_tid();
  const int Nv = sh.Nv, n = bud + sh.Nt;
  const int rb = sh.D * fw.esize;  // bytes per row: 128, 256 or 512
  if (bud < 0 || bud > Nv || off < 0 || off + (int64_t)sh.Hkv * n * sh.D > fw.cap_elems) return;
  const int cs = rb == 128 ? 3 : rb == 256 ? 4 : 5;  // log2 of 16-byte pieces per row
  const char *src = src_l + (size_t)(b * sh.Hkv + g) * sh.S * rb;
  char *dst = dst_l + (size_t)off * fw.esize + (size_t)g * n * rb;
  const auto rk = coherent_rsrc(fw.keptrec + (size_t)plb * Nv, (unsigned)(Nv * sizeof(uint64_t)));
  // only the bud kept words are read (past them: the out-of-range offset,
  // zeros without a memory access), so a poll round moves bud words
  uint64_t kw[KW];
  auto load_kept = [&]() {
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const unsigned o = tid + j * NT < bud ? (unsigned)((tid + j * NT) * 8) : 0xfffffff0u;
      kw[j] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rk, (int)o, 0, 16));
    }
  };
  load_kept();
  fused_copy_rows(src, dst, rb, cs, bud, n, sh.S, [&](int i) { return Nv + (i - bud); });
  unsigned spins = 0;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < KW; ++j) ok = ok && (tid + j * NT >= bud || (unsigned)(kw[j] >> 32) == epoch);
    if (ok || spin_expired(spins, plan.status)) break;
    load_kept();
  }
#pragma unroll
  for (int j = 0; j < KW; ++j)
    if (tid + j * NT < bud) kidx[tid + j * NT] = (int)(unsigned)kw[j];
  __syncthreads();
  fused_copy_rows(src, dst, rb, cs, 0, bud, sh.S, [&](int i) { return kidx[i]; });
  __syncthreads();  // kidx is reused by the next unit
}

template <typename Tag, int D>
__global__ __launch_bounds__(kFusedThreads) void cross_score_fused_kernel(Shape sh, FusedTables tab, PlanPtrs plan,
                                                                          FusedWs fw, FusedLds lo) {
  extern __shared__ __attribute__((aligned(16))) float lds_f[];
  unsigned char *lds = reinterpret_cast<unsigned char *>(lds_f);
  __shared__ int wtot[4 * kFusedWaves];
  __shared__ double redd[2 * kFusedWaves];
  __shared__ float redf[kFusedWaves];
  __shared__ int bcast[4];
  __shared__ int hdr[2];
  const int tid = threadIdx.x;
  const int L = sh.L, B = sh.B, Nv = sh.Nv, LB = L * B;
  const int wph = kFusedWaves / sh.Hkv;
  const int ntw = fused_words64(sh.Nt);
  const unsigned e0 = *fw.epoch;
  const unsigned epoch = e0 + 1u;  // tag of every record this call writes
  const int P = gridDim.x, me = blockIdx.x;
  int *item_list = reinterpret_cast<int *>(lds + lo.items);
  int *owed = reinterpret_cast<int *>(lds + lo.owed);
  int *ntk_l = reinterpret_cast<int *>(lds + lo.ntk);

  // Phase 0: the elite sets (no counter: the readers check the records'
  // tags). Pair lb's part 0, with its merge, runs on workgroup P - 1 - lb
  // (mod P), its parts 1.. from workgroup 0 up, so the merges, which finish
  // last, land on the workgroups that get no item when there are fewer items
  // than workgroups. The status word is cleared by workgroup 0 before it
  // reads the counts, and its bits are set later: the overflow bit by
  // workgroup 0 from the counts, the timeout bit after a wait has run out.
  if (me == 0 && tid == 0) {
    store_coherent(plan.status, 0);
    wait_all_memory();
  }
  // A wave's loads complete in order and a barrier waits for them, so the
  // waves that read the elite counts issue no prestage loads (their tiles
  // are loaded by wave ncw + their index, when there is one); the others
  // prestage at once in workgroups without a part (a part's own loads are
  // bound by what one CU has in flight), after their parts in the others
  // (a merging workgroup then reads the counts late, but streams its first
  // item's chunk as fast as the rest).
  const uint64_t hint = me < kFusedHintSlots ? fw.hint[me] : 0ull;
  const int npp = fw.npp;
  const int nother = LB * (npp - 1);  // parts 1.. in all (LB * npp <= P when npp > 1)
  const bool merger = P - 1 - me < LB;
  const bool other = me < nother;
  const bool former = merger || other;
  const int ncw = ((LB < kFusedThreads ? LB : kFusedThreads) + 63) >> 6;  // waves that read the counts
  const int wave_id = tid >> 6;
  auto prestage = [&]() {
    if (wave_id < ncw) return;
    fused_prestage<Tag, D>(sh, tab, hint, lds, lo, wave_id);
    if (wave_id - ncw < ncw) fused_prestage<Tag, D>(sh, tab, hint, lds, lo, wave_id - ncw);
  };
  if (!former) prestage();
  if (other) {
    const int lb = me / (npp - 1);
    fused_elite_part<Tag, D>(sh, tab, plan, fw, lb, me - lb * (npp - 1) + 1, epoch, lds_f, lo.total, wtot, redf);
  }
  for (int lb = P - 1 - me; lb < LB; lb += P)
    fused_elite_part<Tag, D>(sh, tab, plan, fw, lb, 0, epoch, lds_f, lo.total, wtot, redf);
  if (former) prestage();
  fused_elite_counts(sh, fw, epoch, plan.status, ntk_l, me == 0);
  fused_schedule(sh, fw, ntk_l, me, P, item_list, hdr, wtot);
  __syncthreads();
  const int kcap = uniform(hdr[0]);
  const int run = uniform(hdr[1]);
  int nmine = (me < run) ? (run - me + P - 1) / P : 0;
  if (nmine > kFusedMaxItems) {
    if (tid == 0) atomicOr(plan.status, AIRCACHE_DEV_TIMEOUT);
    nmine = kFusedMaxItems;
  }
  int nowed = 0;

  for (int k = 0; k < nmine; ++k) {
    const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
    FusedItem it;
    const int item = uniform(item_list[k]);
    const int s = item >> 16;
    it.b = s / L;
    it.l = s - it.b * L;
    it.plb = it.l * B + it.b;
    it.ntk = uniform(ntk_l[it.plb]);
    it.cp = fused_chunk_plan(it.ntk, sh.G, Nv, wph, kcap);
    const int local = item & 0xffff;
    it.r = local / it.cp.nchunks;
    it.c = local - it.r * it.cp.nchunks;
    it.q = tab.p[it.l];
    it.k = tab.p[L + it.l];
    int *el = reinterpret_cast<int *>(lds + lo.el);
    __syncthreads();  // the previous item is done with the LDS
    // elite list of the item's (layer, sample), ascending
    fused_elite_list(sh, fw, it.plb, it.ntk, epoch, plan.status, el,
                     reinterpret_cast<unsigned long long *>(lds + lo.mloc));
    if (k == 0) wait_all_memory();  // the prestage loads are in the ring before the barrier
    __syncthreads();
    {
      const int rt0 = it.r * kFusedRtMax, left = it.cp.rtg - rt0;
      uint64_t h = 0ull;  // the prestaged tiles serve the first item only
      if (k == 0) {
        // a wave's tiles were prestaged unless it reads the counts and no
        // wave was left to load them
        if (wave >= ncw || wave + ncw < kFusedWaves) h = hint;
        if (tid == 0 && me < kFusedHintSlots) fw.hint[me] = fused_hint(it.plb, it.c, it.cp.ktw);
      }
      if (left >= 4) fused_pass<Tag, D, 4>(sh, fw, it, rt0, lds, lo, epoch, plan.status, h);
      else if (left == 3) fused_pass<Tag, D, 3>(sh, fw, it, rt0, lds, lo, epoch, plan.status, h);
      else if (left == 2) fused_pass<Tag, D, 2>(sh, fw, it, rt0, lds, lo, epoch, plan.status, h);
      else fused_pass<Tag, D, 1>(sh, fw, it, rt0, lds, lo, epoch, plan.status, h);
    }
    // The workgroup of a pair's first item (row group 0, chunk 0) owns its
    // statistics and top-k, which it runs after its items.
    if (it.r == 0 && it.c == 0) {
      if (tid == 0) owed[nowed] = it.plb;
      ++nowed;
    }

    // Column sums of this item's rows over the KV heads (in order); with one
    // row group they are the chunk's I_v * H_q * N_tk, else the last row group
    // of the chunk adds every group's sums in order.
    const float *colsum = reinterpret_cast<const float *>(lds + lo.colsum);
    const int W = it.cp.width, c0 = it.c * W;
    const int ncol = max(0, min(W, Nv - c0));  // visual columns of the chunk
    float ivv[8];                                // W <= 8 * kFusedThreads
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = tid + j * kFusedThreads;
      float a = 0.f;
      if (col < ncol)
        for (int g = 0; g < sh.Hkv; ++g) a += colsum[g * W + col];
      ivv[j] = a;
    }
    if (it.cp.nrg > 1) {
      const size_t slot = (size_t)it.plb * fw.max_chunks + it.c;
      float *pr = fw.part + (slot * fw.max_rg + it.r) * fw.wmax;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = tid + j * kFusedThreads;
        if (col < ncol) store_coherent(&pr[col], ivv[j]);
      }
      wait_all_memory();
      __syncthreads();
      if (tid == 0) {
        const bool last = counter_add(&fw.cnt_chunk[slot], 1u) == (unsigned)it.cp.nrg - 1u;
        if (last) store_coherent(&fw.cnt_chunk[slot], 0u);  // reset for the next call
        bcast[3] = last;
      }
      __syncthreads();
      if (!uniform(bcast[3])) continue;
      const auto rp = coherent_rsrc(fw.part + slot * fw.max_rg * fw.wmax,
                                    (unsigned)((size_t)fw.max_rg * fw.wmax * sizeof(float)));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = tid + j * kFusedThreads;
        float a = 0.f;
        if (col < ncol)
          for (int r = 0; r < it.cp.nrg; ++r) a += load_sc1_f(rp, (unsigned)((r * fw.wmax + col) * sizeof(float)));
        ivv[j] = a;
      }
    }
    const float inv_rows = (it.ntk > 0) ? 1.f / (float)(sh.Hq * it.ntk) : 0.f;
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = tid + j * kFusedThreads;
      if (col < ncol) {
        const float a = ivv[j] * inv_rows;
        ivv[j] = a;
        plan.iv[(size_t)it.plb * Nv + c0 + col] = a;
        store_coherent(&fw.ivrec[(size_t)it.plb * Nv + c0 + col], pack_rec(a, epoch));
        sum += (double)a;
      }
    }
    sum = fused_block_sum_d(sum, redd);
    const double mean = ncol > 0 ? sum / (double)ncol : 0.0;
    double m2 = 0.0, m3 = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = tid + j * kFusedThreads;
      if (col < ncol) {
        const double d = (double)ivv[j] - mean;
        m2 += d * d;
        m3 += d * d * d;
      }
    }
    fused_block_sum_d2(m2, m3, redd);
    if (tid < 4) {
      // the chunk's moments as epoch-tagged 32-bit halves (no ordering needed)
      const double v = tid == 0 ? sum : tid == 1 ? m2 : tid == 2 ? m3 : (double)ncol;
      const uint64_t u = __builtin_bit_cast(uint64_t, v), tag = (uint64_t)epoch << 32;
      uint64_t *mr = fw.mom + ((size_t)it.plb * fw.max_chunks + it.c) * 8 + 2 * tid;
      store_coherent(mr, tag | (u & 0xffffffffu));
      store_coherent(mr + 1, tag | (u >> 32));
    }
  }

  // Owed (layer, sample) pairs: first every statistics record (every top-k
  // waits for the records of whole samples, possibly this workgroup's own),
  // then the top-k tasks with their budgets.
  if (threadIdx.x < 64)
    for (int o = 0; o < nowed; ++o) {
      const int plb = uniform(owed[o]);
      const int nch = fused_chunk_plan(ntk_l[plb], sh.G, Nv, wph, kcap).nchunks;
      fused_layer_stats(sh, plan, fw, plb, nch, epoch);
    }
  unsigned *hist = reinterpret_cast<unsigned *>(lds + lo.ring);
  {
    const int tid = opaque_tid();
    __syncthreads();  // every wave is done with the item LDS
    for (int i = tid; i < kTopkBuckets; i += kFusedThreads) hist[i] = 0u;
  }
  for (int o = 0; o < nowed; ++o) {
    __syncthreads();
    const int plb = uniform(owed[o]);
    const int l = plb / B, b = plb - l * B;
    const uint64_t *ivl = fw.ivrec + (size_t)plb * Nv;
    int32_t *kp = plan.kept + (size_t)plb * Nv;
    uint64_t *kr = fw.keptrec + (size_t)plb * Nv;
    double *sts = reinterpret_cast<double *>(lds + lo.sts);
    auto budget = [&]() {
      const int bud = fused_budget(sh, plan, fw, l, b, epoch, sts, bcast);
      if (fw.gather && threadIdx.x == 0) {
        // budget and offset out: compaction of the text rows can start
        const uint64_t tag = (uint64_t)epoch << 32;
        uint64_t *r = fw.grec + (size_t)plb * 4;
        store_coherent(r + 0, tag | (uint64_t)(unsigned)bcast[0]);
        store_coherent(r + 1, tag | (uint64_t)(unsigned)bcast[2]);
        store_coherent(r + 2, tag | (uint64_t)(unsigned)bcast[3]);
      }
      return bud;
    };
    if (Nv <= 2048) block_topk<4>(sh, ivl, kp, kr, epoch, plan.status, hist, budget);
    else if (Nv <= 4096) block_topk<8>(sh, ivl, kp, kr, epoch, plan.status, hist, budget);
    else block_topk<16>(sh, ivl, kp, kr, epoch, plan.status, hist, budget);
  }

  // Compaction units (layer, sample, KV head, K or V) by ticket, in
  // sample-major order; each waits for its (layer, sample)'s record.
  if (fw.gather) {
    int *kidx = reinterpret_cast<int *>(lds + lo.ring);
    const int nunits = LB * sh.Hkv * 2;
    const auto rg = coherent_rsrc(fw.grec, (unsigned)((size_t)LB * 32));
    for (;;) {
      __syncthreads();
      if (threadIdx.x == 0) bcast[1] = (int)counter_add(fw.gticket, 1u);
      __syncthreads();
      const int u = uniform(bcast[1]);
      if (u >= nunits) break;
      const int kv = u & 1, ug = u >> 1;
      const int s2 = ug / sh.Hkv, g = ug - s2 * sh.Hkv;
      const int b = s2 / L, l = s2 - b * L, plb = l * B + b;
      if (threadIdx.x == 0) {
        uint64_t w[3];
        unsigned spins = 0;
        for (;;) {
#pragma unroll
          for (int j = 0; j < 3; ++j)
            w[j] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rg, plb * 32 + 8 * j, 0, 16));
          if (((unsigned)(w[0] >> 32) == epoch && (unsigned)(w[1] >> 32) == epoch && (unsigned)(w[2] >> 32) == epoch) ||
              spin_expired(spins, plan.status))
            break;
          __builtin_amdgcn_s_sleep(2);
        }
        bcast[0] = (int)(unsigned)w[0];
        bcast[2] = (int)(unsigned)w[1];
        bcast[3] = (int)(unsigned)w[2];
      }
      __syncthreads();
      const int bud = uniform(bcast[0]);
      const int64_t off = (int64_t)(((uint64_t)(unsigned)uniform(bcast[3]) << 32) | (uint64_t)(unsigned)uniform(bcast[2]));
      const char *src = static_cast<const char *>(tab.p[(1 + kv) * L + l]);  // k or v
      char *dst = static_cast<char *>(const_cast<void *>(tab.p[(3 + kv) * L + l]));  // k_out or v_out
      fused_gather_unit(sh, plan, fw, src, dst, b, g, plb, bud, off, epoch, kidx);
    }
  }

  // The last workgroup to finish ends the call: counters reset, epoch advanced.
  __syncthreads();
  if (threadIdx.x == 0) {
    if (counter_add(fw.exitc, 1u) == (unsigned)P - 1u) {
      store_coherent(fw.exitc, 0u);
      if (fw.gather) store_coherent(fw.gticket, 0u);
      store_coherent(fw.epoch, epoch);
    }
  }
}
