// Decode attention over the compacted cache, included by aircache.hip inside
// namespace aircache.
//
// The consumer of the compacted per-layer cache: the KV-cache primer page
// (devpress.csdn.net), section 2.1 "到底缓存什么？", the o_t equation, with
// one new query per query head and no mask (the incremental step only sees
// cached positions, section 2.2). For layer l, sample b and query head h with
// KV head g = h / G, over the n = r_hat[l][b] + N_t rows of head g in the
// (l, b) segment of the compacted buffers ([H_kv][n][D] at out_off[l][b]):
//   o[l][b][h] = softmax(q[l][b][h] . K^T / sqrt(D)) V.
//
// Split-row decoding: the rows of each (l, b, g) are split evenly over S
// workgroups (S fixed by the shape, for two workgroups per CU); in
// decode_partial_kernel a workgroup
// takes its rows in chunks of kDecRows for all G query heads of g at once
// (every K and V row is read once from HBM), keeping per head a running
// maximum, sum of exponentials and unnormalised output row (rescaled when the
// maximum grows). decode_combine_kernel merges the splits of each (l, b, h)
// in split order (decode_wave_kernel, below, streams a split's rows per wave
// instead). The pass is a stream of K and V rows (HBM-bound): the
// logits are MFMA products of 16 key rows against 16 query heads, and the
// weights x V product runs on the matrix cores for groups of 4 to 32 heads
// (below) or in fp32 on the vector units.
#pragma once

constexpr int kDecThreads = 512;                  // 8 waves, 16 rows each
constexpr int kDecRows = 16 * (kDecThreads / 64);  // rows of one split
constexpr int kDecMaxLds = 160 * 1024;  // a CU's LDS (the kernel has no static LDS)
constexpr int kDecTargetCus = 256;      // the splits are sized for this many CUs

// Widening of stored elements to float (bf16: the 16 bits are the top half).
template <typename Tag> __device__ __forceinline__ float to_f32(typename Tag::store_t x);
template <> __device__ __forceinline__ float to_f32<Bf16Tag>(uint16_t x) { return __uint_as_float((unsigned)x << 16); }
template <> __device__ __forceinline__ float to_f32<F32Tag>(float x) { return x; }

// Eight or four stored elements from one 16-byte piece, widened.
__device__ __forceinline__ void widen(const u32x4_t &w, float *out, Bf16Tag) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void widen(const u32x4_t &w, float *out, F32Tag) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
}

struct DecodeTables {
  LayerTable q, k, v;
  LayerTableOut o;
};

// Splits per (l, b, g): enough workgroups for two per CU (four when the
// units alone outnumber the CUs: the long segments then end in a shorter
// tail), but no more than leave half a chunk (kDecRows / 2 rows) per split at
// the expected row count ratio * N_v + N_t (a split's fixed latency outweighs
// a few rows, and the merge reads every split); rows are split evenly, each
// split's rows in chunks of kDecRows. (Measured on the five workloads.)
__host__ __device__ inline int decode_splits(int L, int B, int Hkv, int cus, double ratio, int Nv, int Nt) {
  const long long units = (long long)L * B * Hkv;
  const long long per_cu = units >= cus ? 4 : 2;
  long long s = (per_cu * cus + units - 1) / units;
  const long long rows = (long long)(ratio * (double)Nv) + Nt;
  const long long by_rows = (rows + kDecRows / 2 - 1) / (kDecRows / 2);
  if (s > by_rows) s = by_rows;
  return (int)(s < 1 ? 1 : (s > 64 ? 64 : s));
}

// Threads per (query head, 8 output elements) of the accumulation: the rows
// of a chunk are split over them.
__host__ __device__ inline int decode_parts(int G, int D) {
  int p = kDecThreads / (G * D / 8);
  int q = 1;
  while (q * 2 <= p && q < 16) q *= 2;
  return q;
}

// Dynamic LDS of decode_partial_kernel: q of the G heads [G][D] floats,
// logits then weights [G][kDecRows] floats, per-head running (max, sum,
// rescale) [G][4] floats, the chunk's V rows, and the parts' accumulators
// [parts][G][D] floats at the end (over the V rows and weights).
__host__ __device__ inline int decode_lds_bytes(int G, int D, int esize) {
  const int main = G * D * 4 + G * kDecRows * 4 + G * 16 + kDecRows * D * esize;
  const int red = G * D * 4 * decode_parts(G, D) + G * D * 4 + G * 16;
  return main > red ? main : red;
}

// Weights x V on the matrix cores (bfloat16 queries, kDecPvMinG <= G <=
// kDecPvMaxG): the
// chunk's V rows go into LDS transposed (one row per output element d, the
// chunk's rows contiguous, bfloat16; int8 codes converted exactly), so that
// O^T = V^T P^T is a v_mfma_f32_16x16x32_bf16 product with V^T as the A
// operand and the weights of 16 query heads as the B operand; wave w owns the
// output elements 16 w .. 16 w + 15 of every head. A weight p in [0, 1]
// enters as two bfloat16 terms, hi = rn(p) and lo = rn(p - hi), with
// |p - hi - lo| <= 2^-18 p, so the products keep the float32 accuracy of the
// vector-unit path (which float32 queries and larger groups take).
constexpr int kDecPvMaxG = 32;
constexpr int kDecVtStride = kDecRows * 2 + 8;  // bytes per transposed V row (8 B apart in banks, 8-byte aligned)
constexpr int kDecZs = kDecRows + 4;            // floats per head row of the weights (bank spread of the B reads)

// Dynamic LDS of the matrix-core variant (byte offsets): q of the G heads
// [G][D] bfloat16, logits then weights [G][kDecZs] floats, per-head running
// (max, sum, rescale) [G][4] floats, V^T [D][kDecVtStride bytes].
struct DecPvLds {
  int zp, run, vt, total;
};
__host__ __device__ inline DecPvLds decode_pv_lds(int G, int D) {
  DecPvLds f;
  f.zp = (G * D * 2 + 15) & ~15;
  f.run = f.zp + ((G * kDecZs * 4 + 15) & ~15);
  f.vt = f.run + ((G * 16 + 15) & ~15);
  f.total = f.vt + D * kDecVtStride;
  return f;
}
// (measured: G = 7, workloads 3 to 5, 17-18% less time for the bfloat16
// cache and 10-14% for the int8 cache; G = 1, workload 2, 12% and 37% more,
// since 15 of the 16 head columns of each product are idle)
constexpr int kDecPvMinG = 4;
__host__ __device__ inline bool decode_pv(int G, int qbytes) {
  return qbytes == 2 && G >= kDecPvMinG && G <= kDecPvMaxG;
}

// Two floats to two bfloat16 (round to nearest even), packed low first.
typedef __attribute__((ext_vector_type(2))) float dec_f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 dec_bf16x2_t;
__device__ __forceinline__ unsigned dec_pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(dec_f32x2_t{a, b}, dec_bf16x2_t));
}

// Eight int8 codes (8 bytes) as an MFMA operand fragment of the query's type:
// the integers in [-127, 127] are exact in bfloat16 and float32.
__device__ __forceinline__ void codes_to_frag(const int8_t *p, Frag<Bf16Tag> &f) {
  const uint2 w = *reinterpret_cast<const uint2 *>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = (int)(int8_t)(((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xffu);
    f.v[i] = (uint16_t)(__float_as_uint((float)c) >> 16);  // exact: the low half is zero
  }
}
__device__ __forceinline__ void codes_to_frag(const int8_t *p, Frag<F32Tag> &f) {
  const uint2 w = *reinterpret_cast<const uint2 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.lo[i] = (float)(int8_t)((w.x >> (8 * i)) & 0xffu);
    f.hi[i] = (float)(int8_t)((w.y >> (8 * i)) & 0xffu);
  }
}

// Scales of the int8 cache (aircache_quantize_i8's): [L][B][H_kv] for K and V.
struct DecodeScales {
  const float *k, *v;
};

// Waves per SIMD the decode kernel is compiled for: eight (64 registers, four
// workgroups per CU) for bfloat16 queries on the vector-unit path (measured on
// workload 5 against three workgroups per CU: the int8 cache 153 -> 145 us,
// the bfloat16 cache within the run-to-run spread of a few us; workloads 3
// and 4 unchanged); six (three workgroups per CU) on the matrix-core path,
// whose V^T staging needs up to 80 registers without spilling; float32
// queries need more registers than either.
template <typename Tag, bool PV> constexpr int decode_waves() { return Tag::kBytes == 2 ? (PV ? 6 : 8) : 1; }

// Q8: the compacted cache is int8 codes with one scale per (layer, sample, KV
// head) for K and for V (value = code * scale): logits are the codes' dot
// products times the K scale, the weighted sum of V codes is times the V
// scale, both applied once per row and per output.
template <typename Tag, int D, bool Q8, bool PV>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(decode_waves<Tag, PV>()))) void decode_partial_kernel(Shape sh, DecodeTables tb,
                                                                     const int32_t *budget, const int64_t *out_off,
                                                                     int64_t cap_elems, int S, float2 *part_ml,
                                                                     float *part_acc, DecodeScales scl) {
  using QE = typename Tag::store_t;                      // the queries' type
  using E = typename std::conditional<Q8, int8_t, QE>::type;  // the cache's
  constexpr int EB = Q8 ? 1 : Tag::kBytes;
  constexpr int NT = kDecThreads;
  constexpr int kPiece = 16 / EB;              // cache elements per 16-byte piece
  constexpr int kQPiece = 16 / Tag::kBytes;    // query elements per 16-byte piece
  extern __shared__ __attribute__((aligned(16))) float dec_lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, grp = lane >> 4;
  const int G = sh.G, Hkv = sh.Hkv, B = sh.B;
  int rest = blockIdx.x;
  const int s = rest % S;
  rest /= S;
  const int g = rest % Hkv;
  rest /= Hkv;
  const int b = rest % B, l = rest / B;
  const int lb = l * B + b;
  const int r = budget[lb];
  const int64_t off = out_off[(size_t)l * (B + 1) + b];
  // (compared as off <= cap - size: a stray offset near the top of int64 cannot wrap)
  const bool ok = r >= 0 && r <= sh.Nv && off >= 0 && off <= cap_elems - (int64_t)Hkv * (r + sh.Nt) * D;
  const int n = ok ? r + sh.Nt : 0;
  // this split's rows [lo, hi), an even share of the n rows
  const int lo = (int)((long long)n * s / S), hi = (int)((long long)n * (s + 1) / S);
  static_assert(!PV || Tag::kBytes == 2, "the matrix-core weights x V takes bfloat16 queries");
  unsigned char *lds8 = reinterpret_cast<unsigned char *>(dec_lds);
  const DecPvLds pl = decode_pv_lds(G, D);
  const int zs = PV ? kDecZs : kDecRows;             // floats per head row of zp
  QE *qs = reinterpret_cast<QE *>(dec_lds);          // [G][D] as stored (vector path: room for floats)
  float *zp = PV ? reinterpret_cast<float *>(lds8 + pl.zp) : dec_lds + G * D;  // [G][zs]
  float *run = PV ? reinterpret_cast<float *>(lds8 + pl.run) : zp + G * kDecRows;  // [G][4]: max, sum, rescale
  E *vs = reinterpret_cast<E *>(run + G * 4);        // vector path: [kDecRows][D]
  unsigned char *vt = lds8 + pl.vt;                  // matrix-core path: V^T [D][kDecVtStride bytes]
  const E *kseg = static_cast<const E *>(tb.k.p[l]) + (ok ? off + (int64_t)g * n * D : 0);
  const E *vseg = static_cast<const E *>(tb.v.p[l]) + (ok ? off + (int64_t)g * n * D : 0);
  const QE *qb = static_cast<const QE *>(tb.q.p[l]) + ((size_t)b * sh.Hq + (size_t)g * G) * D;
  // the int8 cache's scales of this (layer, sample, KV head)
  const float ksc = Q8 ? scl.k[(size_t)lb * Hkv + g] : 1.f, vsc = Q8 ? scl.v[(size_t)lb * Hkv + g] : 1.f;
  // the G query rows into LDS, as stored
  for (int p = tid; p < G * D / kQPiece; p += NT)
    reinterpret_cast<u32x4_t *>(qs)[p] = reinterpret_cast<const u32x4_t *>(qb)[p];
  for (int h = tid; h < G; h += NT) {
    run[h * 4 + 0] = -INFINITY;
    run[h * 4 + 1] = 0.f;
  }
  // accumulation layout: thread (h, e8, part) owns output elements
  // [8 e8, 8 e8 + 8) of head h over the chunk rows j = part, part + P, ...
  const int P = decode_parts(G, D);
  const int oh = tid / (D / 8 * P), orem = tid - oh * (D / 8 * P);
  const int oe = orem / P, opart = orem - oe * P;
  const bool owner = oh < G;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // matrix-core path: O^T rows 16 wave + 4 grp + i, head 16 hg + n16
  f32x4_t oacc[kDecPvMaxG / 16];
#pragma unroll
  for (int hg = 0; hg < kDecPvMaxG / 16; ++hg) oacc[hg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  for (int c0 = lo; c0 < hi; c0 += kDecRows) {
    const int nr = min(kDecRows, hi - c0);
    // this lane's quarter of key row c0 + 16 wave + n16, and the chunk's V rows
    const int row = wave * 16 + n16;
    const bool rv = row < nr;
    // key fragments of this wave's 16 rows (MFMA A operand: row n16, slice
    // part grp) and the chunk's V rows; every load issued before the first
    // is used
    Frag<Tag> kf[D / 32];
    {
      constexpr int VP = kDecRows * D / kPiece / NT;  // V pieces per thread
      const E *kp = kseg + (size_t)(c0 + (rv ? row : 0)) * D + grp * 8;
      const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(vseg + (size_t)c0 * D);
      const int pieces = nr * D / kPiece;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        if (!rv) kf[c].zero();
        else if constexpr (Q8) codes_to_frag(kp + c * 32, kf[c]);
        else kf[c].load(kp + c * 32);
      }
      if constexpr (PV) {
        // thread (kq, dq): rows 4 kq .. 4 kq + 3, elements 8 dq .. 8 dq + 7
        // (rows past the chunk read its last row and go in as zeros)
        constexpr int NDQ = D / 8;
        using VL = typename std::conditional<Q8, uint2, u32x4_t>::type;
        const int dq = tid % NDQ, kq = tid / NDQ;
        const bool st = kq < kDecRows / 4;
        VL vl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = min(4 * kq + i, nr - 1);
          vl[i] = st ? *reinterpret_cast<const VL *>(vseg + (size_t)(c0 + rr) * D + 8 * dq) : VL{};
        }
        if (st) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            unsigned x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              unsigned e;
              if constexpr (Q8) {
                const unsigned w = j < 4 ? vl[i].x : vl[i].y;
                e = __float_as_uint((float)(int)(int8_t)((w >> (8 * (j & 3))) & 0xffu)) >> 16;  // exact
              } else {
                e = (vl[i][j >> 1] >> (16 * (j & 1))) & 0xffffu;
              }
              x[i] = 4 * kq + i < nr ? e : 0u;
            }
            uint2 wv;
            wv.x = x[0] | (x[1] << 16);
            wv.y = x[2] | (x[3] << 16);
            *reinterpret_cast<uint2 *>(vt + (size_t)(8 * dq + j) * kDecVtStride + 8 * kq) = wv;
          }
        }
      } else {
        u32x4_t vw[VP];
#pragma unroll
        for (int i = 0; i < VP; ++i) vw[i] = tid + i * NT < pieces ? vp[tid + i * NT] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < VP; ++i)
          if (tid + i * NT < pieces) reinterpret_cast<u32x4_t *>(vs)[tid + i * NT] = vw[i];
      }
    }
    // logits (log2 domain) by MFMA, 16 query heads at a time (B operand:
    // head n16): acc[i] is row 4 grp + i of the wave's 16 against head n16
    for (int h0 = 0; h0 < G; h0 += 16) {
      const int hq = min(h0 + n16, G - 1);
      f32x4_t acc4 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        Frag<Tag> qf;
        qf.load(qs + (size_t)hq * D + c * 32 + grp * 8);
        mfma_slice(acc4, kf[c], qf);
      }
      if (h0 + n16 < G)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rw = wave * 16 + grp * 4 + i;
          zp[(h0 + n16) * zs + rw] = rw < nr ? acc4[i] * (sh.scale2 * ksc) : -INFINITY;
        }
    }
    __syncthreads();
    // per head: the running maximum, the chunk's weights, the running sum
    for (int h = wave; h < G; h += NT / 64) {
      float *z = zp + h * zs;
      float m = -INFINITY;
      for (int j = lane; j < kDecRows; j += 64) m = fmaxf(m, z[j]);
      m = wave_max(m);
      const float m_old = run[h * 4 + 0];
      const float m_new = fmaxf(m_old, m);
      float t = 0.f;
      for (int j = lane; j < kDecRows; j += 64) {
        const float p = z[j] > -INFINITY ? exp2f(z[j] - m_new) : 0.f;
        z[j] = p;
        t += p;
      }
      t = wave_sum(t);
      if (lane == 0) {
        const float sc = m_old > -INFINITY ? exp2f(m_old - m_new) : 0.f;
        run[h * 4 + 0] = m_new;
        run[h * 4 + 1] = run[h * 4 + 1] * sc + t;
        run[h * 4 + 2] = sc;
      }
    }
    __syncthreads();
    if constexpr (PV) {
      // O^T (rescaled to the new maxima) += V^T P^T, 32 rows per product
      if (wave < D / 16) {
#pragma unroll
        for (int hg = 0; hg < kDecPvMaxG / 16; ++hg) {
          if (16 * hg < G) {
            const int hh = min(16 * hg + n16, G - 1);
            oacc[hg] *= run[hh * 4 + 2];
            const float *pz = zp + hh * kDecZs;
#pragma unroll
            for (int ks = 0; ks < kDecRows / 32; ++ks) {
              if (32 * ks < nr) {
                const unsigned char *va = vt + (size_t)(16 * wave + n16) * kDecVtStride + (32 * ks + 8 * grp) * 2;
                const uint2 a0 = *reinterpret_cast<const uint2 *>(va), a1 = *reinterpret_cast<const uint2 *>(va + 8);
                Frag<Bf16Tag> a, bh, bl;
                a.v = __builtin_bit_cast(u16x8_t, u32x4_t{a0.x, a0.y, a1.x, a1.y});
                const f32x4_t p0 = *reinterpret_cast<const f32x4_t *>(pz + 32 * ks + 8 * grp);
                const f32x4_t p1 = *reinterpret_cast<const f32x4_t *>(pz + 32 * ks + 8 * grp + 4);
                const float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
                u32x4_t wh, wl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const unsigned h2 = dec_pack_bf16(pv[2 * i], pv[2 * i + 1]);
                  wh[i] = h2;
                  wl[i] = dec_pack_bf16(pv[2 * i] - __uint_as_float(h2 << 16),
                                        pv[2 * i + 1] - __uint_as_float(h2 & 0xffff0000u));
                }
                bh.v = __builtin_bit_cast(u16x8_t, wh);
                bl.v = __builtin_bit_cast(u16x8_t, wl);
                mfma_slice(oacc[hg], a, bh);
                mfma_slice(oacc[hg], a, bl);
              }
            }
          }
        }
      }
    } else if (owner) {
      // accumulators rescaled to the new maximum, then weight x V over the
      // thread's rows of the chunk (one 16-byte V read gives 8 elements)
      const float sc = run[oh * 4 + 2];
      const float *p = zp + oh * kDecRows;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= sc;
      for (int j = opart; j < nr; j += P) {
        float vv[8];
        const E *vr = vs + j * D + 8 * oe;
        if constexpr (Q8) {
          const uint2 w = *reinterpret_cast<const uint2 *>(vr);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vv[i] = (float)(int8_t)((w.x >> (8 * i)) & 0xffu);
            vv[4 + i] = (float)(int8_t)((w.y >> (8 * i)) & 0xffu);
          }
        } else if (Tag::kBytes == 2) {
          widen(*reinterpret_cast<const u32x4_t *>(vr), vv, Tag{});
        } else {
          widen(*reinterpret_cast<const u32x4_t *>(vr), vv, Tag{});
          widen(*reinterpret_cast<const u32x4_t *>(vr + 4), vv + 4, Tag{});
        }
        const float pj = p[j];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += pj * vv[i];
      }
    }
    __syncthreads();  // vs, zp and the rescale factors are rewritten by the next chunk
  }
  // the split's running (max, sum) out, then the parts' accumulators added
  // in part order (over q, the weights and the V rows, all read by now)
  for (int h = tid; h < G; h += NT)
    part_ml[((size_t)lb * sh.Hq + (size_t)g * G + h) * S + s] = make_float2(run[h * 4 + 0], run[h * 4 + 1]);
  if constexpr (PV) {
    if (wave < D / 16) {
#pragma unroll
      for (int hg = 0; hg < kDecPvMaxG / 16; ++hg) {
        const int h = 16 * hg + n16;
        if (h < G)
          *reinterpret_cast<f32x4_t *>(part_acc + (((size_t)lb * sh.Hq + (size_t)g * G + h) * S + s) * D +
                                       16 * wave + 4 * grp) = oacc[hg] * vsc;
      }
    }
    return;
  }
  __syncthreads();
  float *red = dec_lds;  // [P][G][D]
  if (owner)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[((size_t)opart * G + oh) * D + 8 * oe + i] = acc[i];
  __syncthreads();
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, d = i - h * D;
    float a = 0.f;
    for (int q = 0; q < P; ++q) a += red[((size_t)q * G + h) * D + d];
    part_acc[(((size_t)lb * sh.Hq + (size_t)g * G + h) * S + s) * D + d] = a * vsc;
  }
}

// One stream of rows per wave (bfloat16 queries, kDecPvMinG <= G <= 32). The
// split's rows go to its eight waves in 16-row slices (slice k on wave k mod
// 8); a wave keeps, per query head of the group, its own running maximum, sum
// and O^T, so the slices need no block barrier: per slice, the logits are
// MFMA products of the 16 key rows (A operand) against the heads' queries (B
// operand: head n16 of lane n16), the online softmax reduces over the lane's
// four rows and the four 16-lane row groups, and the weights, which the
// logits' layout already places as the B operand of a 16x16x16 product, go as
// two bfloat16 terms (hi = rn(p), lo = rn(p - hi)) against V^T, which the wave
// stages in its own LDS area (one 40-byte row per output element: 16 rows of
// bfloat16 plus 8 bytes, so the operand reads of 16 lanes hit distinct banks).
// At the end the waves' (max, sum, O^T) go through LDS and are merged in wave
// order.
constexpr int kDwVtStride = 40;

__host__ __device__ inline int decode_wave_nhg(int G) { return G > 16 ? 2 : 1; }

// decode_wave_kernel is taken when a KV head's expected rows (ratio * N_v +
// N_t) reach kDecWaveMinRows; its splits per (l, b, g) keep at least that
// many rows each and fill at most one round of its two workgroups per CU
// (never more than decode_splits, which sizes the workspace). With one split
// per unit the kernel writes the output itself. Measured against kind 1:
// workload 3 (416 rows, one split) 16.2 -> 12.8 us for the bfloat16 cache and
// 16.3 -> 13.7 us for the int8 cache; workload 4 (318 rows) 25.3 -> 20.6 us
// and 26.5 -> 19.4 us; workload 5 (1331 rows) 142 -> 120 us and 132 -> 89
// us. (With the splits of decode_partial_kernel, about 100 rows each on
// workload 3, the per-wave kernel had been slower: 20 us.)
constexpr int kDecWaveMinRows = 256;
inline int decode_wave_splits(int L, int B, int Hkv, int cus, double ratio, int Nv, int Nt) {
  const long long units = (long long)L * B * Hkv;
  const long long rows = (long long)(ratio * (double)Nv) + Nt;
  long long s = 2LL * cus / units;
  if (s > rows / kDecWaveMinRows) s = rows / kDecWaveMinRows;
  const int smax = decode_splits(L, B, Hkv, cus, ratio, Nv, Nt);
  if (s > smax) s = smax;
  return s < 1 ? 1 : (int)s;
}

// The decode kernel for a shape: 0 decode_partial_kernel with weights x V on
// the vector units, 1 the same on the matrix cores, 2 / 3 decode_wave_kernel
// with one / two groups of 16 heads.
inline int decode_kind(int G, int qbytes, double ratio, int Nv, int Nt) {
  if (!decode_pv(G, qbytes)) return 0;
  const long long rows = (long long)(ratio * (double)Nv) + Nt;
  return rows >= kDecWaveMinRows ? 1 + decode_wave_nhg(G) : 1;
}
__host__ __device__ inline int decode_wave_lds(int G, int D) {
  const int nw = kDecThreads / 64, nhg = decode_wave_nhg(G);
  const int stage = nw * D * kDwVtStride;
  const int merge = nw * nhg * 16 * D * 4 + nw * nhg * 16 * 8;
  return stage > merge ? stage : merge;
}

// Maximum over the four 16-lane rows (lanes n, n + 16, n + 32, n + 48).
__device__ __forceinline__ float dec_max_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

typedef __attribute__((ext_vector_type(4))) short dec_s16x4_t;

template <int D, bool Q8, int NHG>
__global__ __launch_bounds__(kDecThreads) void decode_wave_kernel(Shape sh, DecodeTables tb, const int32_t *budget,
                                                                  const int64_t *out_off, int64_t cap_elems, int S,
                                                                  float2 *part_ml, float *part_acc,
                                                                  DecodeScales scl) {
  using E = typename std::conditional<Q8, int8_t, uint16_t>::type;
  using VL = typename std::conditional<Q8, uint2, u32x4_t>::type;
  constexpr int NT = kDecThreads, NW = NT / 64, NC = D / 32, ND = D / 16, NDQ = D / 8;
  extern __shared__ __attribute__((aligned(16))) float dec_lds[];
  unsigned char *lds8 = reinterpret_cast<unsigned char *>(dec_lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, grp = lane >> 4;
  const int G = sh.G, Hkv = sh.Hkv, B = sh.B;
  int rest = blockIdx.x;
  const int s = rest % S;
  rest /= S;
  const int g = rest % Hkv;
  rest /= Hkv;
  const int b = rest % B, l = rest / B;
  const int lb = l * B + b;
  const int r = budget[lb];
  const int64_t off = out_off[(size_t)l * (B + 1) + b];
  // (compared as off <= cap - size: a stray offset near the top of int64 cannot wrap)
  const bool ok = r >= 0 && r <= sh.Nv && off >= 0 && off <= cap_elems - (int64_t)Hkv * (r + sh.Nt) * D;
  const int n = ok ? r + sh.Nt : 0;
  const int lo = (int)((long long)n * s / S), hi = (int)((long long)n * (s + 1) / S);
  const E *kseg = static_cast<const E *>(tb.k.p[l]) + (ok ? off + (int64_t)g * n * D : 0);
  const E *vseg = static_cast<const E *>(tb.v.p[l]) + (ok ? off + (int64_t)g * n * D : 0);
  const uint16_t *qb = static_cast<const uint16_t *>(tb.q.p[l]) + ((size_t)b * sh.Hq + (size_t)g * G) * D;
  const float ksc = Q8 ? scl.k[(size_t)lb * Hkv + g] : 1.f, vsc = Q8 ? scl.v[(size_t)lb * Hkv + g] : 1.f;
  const float sl2 = sh.scale2 * ksc;

  // the queries of heads 16 hg + n16 (clamped into the group) as B operands
  Frag<Bf16Tag> qf[NHG][NC];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int hq = min(16 * hg + n16, G - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[hg][c].load(qb + (size_t)hq * D + 32 * c + 8 * grp);
  }
  float mrun[NHG], lrun[NHG];  // head n16: running maximum (log2 domain), this lane's part of the sum
  f32x4_t oacc[NHG][ND];       // O^T: element 16 db + 4 grp + i, head 16 hg + n16
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    mrun[hg] = -INFINITY;
    lrun[hg] = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[hg][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  unsigned char *vt = lds8 + wave * D * kDwVtStride;  // this wave's V^T [D][16 rows]
  const int dq = lane % NDQ, rq = lane / NDQ;          // V staging: rows 4 rq .. 4 rq + 3, elements 8 dq .. 8 dq + 7
  const bool st = rq < 4;

  for (int r0 = lo + 16 * wave; r0 < hi; r0 += 16 * NW) {
    const int nr = min(16, hi - r0);
    // every load of the slice issued before the first is used (rows past the
    // slice read its last row)
    Frag<Bf16Tag> kf[NC];
    {
      const E *kp = kseg + (size_t)(r0 + min(n16, nr - 1)) * D + 8 * grp;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (Q8) codes_to_frag(kp + 32 * c, kf[c]);
        else kf[c].load(kp + 32 * c);
      }
    }
    VL vl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r0 + min(4 * rq + i, nr - 1);
      vl[i] = st ? *reinterpret_cast<const VL *>(vseg + (size_t)rr * D + 8 * dq) : VL{};
    }
    // logits: s[hg][i] = row 4 grp + i against head 16 hg + n16
    f32x4_t sc[NHG];
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      sc[hg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) mfma_slice(sc[hg], kf[c], qf[hg][c]);
    }
    // V^T of the slice (rows past it as zeros)
    small_wave_sync();  // the previous slice's operand reads are done
    if (st) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        unsigned x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned e;
          if constexpr (Q8) {
            const unsigned w = j < 4 ? vl[i].x : vl[i].y;
            e = __float_as_uint((float)(int)(int8_t)((w >> (8 * (j & 3))) & 0xffu)) >> 16;  // exact
          } else {
            e = (vl[i][j >> 1] >> (16 * (j & 1))) & 0xffffu;
          }
          x[i] = 4 * rq + i < nr ? e : 0u;
        }
        uint2 wv;
        wv.x = x[0] | (x[1] << 16);
        wv.y = x[2] | (x[3] << 16);
        *reinterpret_cast<uint2 *>(vt + (8 * dq + j) * kDwVtStride + 8 * rq) = wv;
      }
    }
    small_wave_sync();
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      float v[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = 4 * grp + i < nr ? sc[hg][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, v[i]);
      }
      mx = dec_max_rows(mx);
      const float mnew = fmaxf(mrun[hg], mx);
      const float alpha = exp2f(mrun[hg] - mnew);  // 0 before the first slice
      mrun[hg] = mnew;
      float p[4], ls = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f(v[i] - mnew);
        ls += p[i];
      }
      lrun[hg] = lrun[hg] * alpha + ls;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[hg][db] *= alpha;
      }
      const unsigned h01 = dec_pack_bf16(p[0], p[1]), h23 = dec_pack_bf16(p[2], p[3]);
      const unsigned l01 = dec_pack_bf16(p[0] - __uint_as_float(h01 << 16), p[1] - __uint_as_float(h01 & 0xffff0000u));
      const unsigned l23 = dec_pack_bf16(p[2] - __uint_as_float(h23 << 16), p[3] - __uint_as_float(h23 & 0xffff0000u));
      const dec_s16x4_t bh = __builtin_bit_cast(dec_s16x4_t, uint2{h01, h23});
      const dec_s16x4_t bl = __builtin_bit_cast(dec_s16x4_t, uint2{l01, l23});
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const uint2 a = *reinterpret_cast<const uint2 *>(vt + (16 * db + n16) * kDwVtStride + 8 * grp);
        const dec_s16x4_t av = __builtin_bit_cast(dec_s16x4_t, a);
        oacc[hg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bh, oacc[hg][db], 0, 0, 0);
        oacc[hg][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bl, oacc[hg][db], 0, 0, 0);
      }
    }
  }

  // the waves' (max, sum, O^T) through LDS, merged in wave order
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) lrun[hg] = sum_across_rows(lrun[hg]);
  __syncthreads();  // every wave's staging area is read; the LDS now holds the parts
  float *mo = dec_lds;                                               // [NW][NHG * 16][D]
  float2 *mm = reinterpret_cast<float2 *>(dec_lds + NW * NHG * 16 * D);  // [NW][NHG * 16]
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
#pragma unroll
    for (int db = 0; db < ND; ++db)
      *reinterpret_cast<f32x4_t *>(mo + ((size_t)(wave * NHG + hg) * 16 + n16) * D + 16 * db + 4 * grp) =
          oacc[hg][db];
    if (grp == 0) mm[(wave * NHG + hg) * 16 + n16] = make_float2(mrun[hg], lrun[hg]);
  }
  __syncthreads();
  for (int t = tid; t < G * D; t += NT) {
    const int h = t / D, d = t - (t / D) * D;
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mm[w * NHG * 16 + h].x);
    float a = 0.f, L = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float2 ml = mm[w * NHG * 16 + h];
      const float e = ml.x > -INFINITY ? exp2f(ml.x - M) : 0.f;
      a += mo[((size_t)w * NHG * 16 + h) * D + d] * e;
      L += ml.y * e;
    }
    if (S == 1) {
      // one split: the output itself, as decode_combine_kernel would form it
      // (its weight exp2(M - M) is 1; an empty segment gives 0 / 0)
      static_cast<float *>(tb.o.p[l])[((size_t)b * sh.Hq + (size_t)g * G + h) * D + d] = (a * vsc) / L;
      continue;
    }
    const size_t u = ((size_t)lb * sh.Hq + (size_t)g * G + h) * S + s;
    part_acc[u * D + d] = a * vsc;
    if (d == 0) part_ml[u] = make_float2(M, L);
  }
}

// o[l][b][h] from the splits of (l, b, KV head h / G), merged in split order.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(Shape sh, DecodeTables tb, const int32_t *budget,
                                                           const int64_t *out_off, int64_t cap_elems, int S,
                                                           const float2 *part_ml, const float *part_acc) {
  const int d = threadIdx.x;
  const int h = blockIdx.x % sh.Hq, lb0 = blockIdx.x / sh.Hq;
  const int B = sh.B, b = lb0 % B, l = lb0 / B, lb = l * B + b;
  const int r = budget[lb];
  const int64_t off = out_off[(size_t)l * (B + 1) + b];
  const bool ok = r >= 0 && r <= sh.Nv && off >= 0 && off <= cap_elems - (int64_t)sh.Hkv * (r + sh.Nt) * D;
  const int ns = ok ? S : 0;
  const size_t base = ((size_t)lb * sh.Hq + h) * S;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[base + s].x);
  float Z = 0.f, a = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float2 ml = part_ml[base + s];
    const float e = ml.x > -INFINITY ? exp2f(ml.x - M) : 0.f;
    Z += ml.y * e;
    a += part_acc[(base + s) * D + d] * e;
  }
  float *o = static_cast<float *>(tb.o.p[l]) + ((size_t)b * sh.Hq + h) * D;
  o[d] = a / Z;  // (an invalid segment: 0 / 0)
}
