// Device helpers and kernel templates of the ReplaySSM decode path (gfx950).
//
// One workgroup (4 waves of 64 lanes) owns one (sequence, value-head) tile: the
// P x N fp32 checkpoint tile S_ckpt, its ring records and its cursor replica.
//
// Register layout of a tile ("fragment layout"): the tile is cut into 16x16
// fragments; row block rb = wave + 4*i (i < RBW) belongs to one wave, and lane l
// holds, for every fragment f along N, the float4 S[rb*16 + l%16][16f + 4(l/16) .. +3].
// A row's N values are thus spread over 4 lanes (l/16 = 0..3) times N/16 registers,
// so a row dot product is N/16 float4 FMAs per lane plus two cross-lane adds; and
// the layout is the operand/accumulator layout of the 16x16x4 fp32 MFMA.
#pragma once

#include "rssm_internal.hpp"

namespace rssm {

// ---------------------------------------------------------------- element access
__device__ __forceinline__ float bf16f(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

__device__ __forceinline__ float ld_in(const void *base, int64_t i, int bf16) {
  return bf16 ? bf16f(((const uint16_t *)base)[i]) : ((const float *)base)[i];
}

__device__ __forceinline__ void cp_in(void *dst, int64_t di, const void *src, int64_t si, int bf16) {
  if (bf16)
    ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
  else
    ((float *)dst)[di] = ((const float *)src)[si];
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous
// range of tiles so tiles sharing key/query rows (GDN groups) share an L2.
__device__ __forceinline__ int tile_of_block(int ntiles) {
  const int bid = blockIdx.x;
  if ((ntiles & 7) == 0) {
    const int per = ntiles >> 3;
    return (bid & 7) * per + (bid >> 3);
  }
  return bid;
}

__device__ __forceinline__ float quad_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

// ---------------------------------------------------------------- fragments
template <int N, int RBW>
struct Frag {
  float4 s[RBW][N / 16];
};

__device__ __forceinline__ int frag_row(int wave, int lane, int i) { return (wave + kWaves * i) * 16 + (lane & 15); }

template <int N, int RBW>
__device__ __forceinline__ void frag_zero(Frag<N, RBW> &F) {
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int f = 0; f < N / 16; ++f) F.s[i][f] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int N, int RBW>
__device__ __forceinline__ void frag_load(Frag<N, RBW> &F, const float *__restrict__ tile, int P, int wave,
                                          int lane) {
  const int c = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int row = frag_row(wave, lane, i);
    if (row < P) {
      const float4 *src = (const float4 *)(tile + (int64_t)row * N + c);
#pragma unroll
      for (int f = 0; f < N / 16; ++f) F.s[i][f] = src[4 * f];
    } else {
#pragma unroll
      for (int f = 0; f < N / 16; ++f) F.s[i][f] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

template <int N, int RBW>
__device__ __forceinline__ void frag_store(const Frag<N, RBW> &F, float *__restrict__ tile, int P, int wave,
                                           int lane) {
  const int c = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int row = frag_row(wave, lane, i);
    if (row < P) {
      float4 *dst = (float4 *)(tile + (int64_t)row * N + c);
#pragma unroll
      for (int f = 0; f < N / 16; ++f) dst[4 * f] = F.s[i][f];
    }
  }
}

__device__ __forceinline__ float dot4(const float4 a, const float4 b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  acc = fmaf(a.w, b.w, acc);
  return acc;
}

// Per-lane partial of S x for the lane's rows (x: N floats in LDS).
template <int N, int RBW>
__device__ __forceinline__ void frag_dot(const Frag<N, RBW> &F, const float *x, int lane, float (&out)[RBW]) {
  const int c = (lane >> 4) * 4;
  float4 xv[N / 16];
#pragma unroll
  for (int f = 0; f < N / 16; ++f) xv[f] = *(const float4 *)(x + 16 * f + c);
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int f = 0; f < N / 16; ++f) acc = dot4(F.s[i][f], xv[f], acc);
    out[i] = acc;
  }
}

// ---------------------------------------------------------------- quantisers
// fp32 -> OCP E4M3FN, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                       // below 2^-6: E4M3 subnormal grid of 2^-9
    const float m = rintf(a * 512.0f);      // exact scaling, then ties-to-even
    return sign | (uint32_t)m;              // 8 encodes 2^-6 (exponent field 1)
  }
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);   // keep 3 mantissa bits, RNE
  const uint32_t e = (r >> 23) - 127u + 7u;
  return sign | (e << 3) | ((r >> 20) & 7u);
}

// fp32 -> OCP E2M1, round to nearest even, saturating to +-6.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fabsf(x);
  if (!(a < 6.0f)) return sign | 0x7u;
  if (a < 1.0f) return sign | (uint32_t)rintf(a * 2.0f);   // 0, 0.5 or (rounded up) 1.0
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = u + 0x1FFFFFu + ((u >> 22) & 1u);     // keep 1 mantissa bit, RNE
  const uint32_t e = (r >> 23) - 127u + 1u;
  return sign | (e << 1) | ((r >> 22) & 1u);
}

// floor(log2(a)) for a finite a > 0 (normal or subnormal).
__device__ __forceinline__ int ilog2f(float a) {
  const uint32_t u = __float_as_uint(a);
  const int ef = (int)(u >> 23);
  if (ef) return ef - 127;
  return -149 + (31 - __clz(u & 0x7FFFFF));
}

// Quantise the tile held in registers and store the read copy (fp8 or MXFP4).
// Blocks are 32 consecutive columns: fragments 2m and 2m+1 across the 4 lanes of a row.
template <int N, int RBW>
__device__ void frag_store_read_copy(const Frag<N, RBW> &F, int fmt, uint8_t *__restrict__ codes,
                                     uint8_t *__restrict__ scales, int64_t tile, int P, int wave, int lane) {
  const int c = (lane >> 4) * 4;
  const bool lead = (lane >> 4) == 0;
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int row = frag_row(wave, lane, i);
    const int64_t rowi = tile * P + row;
#pragma unroll
    for (int m = 0; m < N / 32; ++m) {
      const float4 v0 = F.s[i][2 * m], v1 = F.s[i][2 * m + 1];
      float am = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                       fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
      am = quad_max(am);
      if (fmt == RSSM_READ_FP8) {
        const float sc = __fdiv_rn(am, 448.0f);
        uint32_t w0 = 0, w1 = 0;
        if (sc > 0.f) {
          w0 = f32_to_e4m3(__fdiv_rn(v0.x, sc)) | (f32_to_e4m3(__fdiv_rn(v0.y, sc)) << 8) |
               (f32_to_e4m3(__fdiv_rn(v0.z, sc)) << 16) | (f32_to_e4m3(__fdiv_rn(v0.w, sc)) << 24);
          w1 = f32_to_e4m3(__fdiv_rn(v1.x, sc)) | (f32_to_e4m3(__fdiv_rn(v1.y, sc)) << 8) |
               (f32_to_e4m3(__fdiv_rn(v1.z, sc)) << 16) | (f32_to_e4m3(__fdiv_rn(v1.w, sc)) << 24);
        }
        if (row < P) {
          uint8_t *dst = codes + rowi * N;
          *(uint32_t *)(dst + 32 * m + c) = w0;
          *(uint32_t *)(dst + 32 * m + 16 + c) = w1;
          if (lead) ((float *)scales)[rowi * (N / 32) + m] = sc;
        }
      } else {
        int E = (am > 0.f) ? ilog2f(am) - 2 : -126;
        E = E < -126 ? -126 : (E > 127 ? 127 : E);                        // scale stays a normal float
        const float inv = __uint_as_float((uint32_t)(127 - E) << 23);   // 2^-E (E <= 125 for finite amax)
        const uint32_t h0 = f32_to_e2m1(v0.x * inv) | (f32_to_e2m1(v0.y * inv) << 4) |
                            (f32_to_e2m1(v0.z * inv) << 8) | (f32_to_e2m1(v0.w * inv) << 12);
        const uint32_t h1 = f32_to_e2m1(v1.x * inv) | (f32_to_e2m1(v1.y * inv) << 4) |
                            (f32_to_e2m1(v1.z * inv) << 8) | (f32_to_e2m1(v1.w * inv) << 12);
        if (row < P) {
          uint8_t *dst = codes + rowi * (N / 2);
          *(uint16_t *)(dst + 16 * m + c / 2) = (uint16_t)h0;
          *(uint16_t *)(dst + 16 * m + 8 + c / 2) = (uint16_t)h1;
          if (lead) scales[rowi * (N / 32) + m] = (uint8_t)(E + 127);
        }
      }
    }
  }
}

typedef float v2f __attribute__((ext_vector_type(2)));

// Per-lane partial of S_read x from the read copy (non-flush steps).
// fp8: lane handles 16-byte chunks (16 codes) ch = l/16 + 4*ci of its row;
// MXFP4: 16-byte chunks of 32 codes (one block each).
template <int N, int RBW>
__device__ __forceinline__ void readcopy_dot(int fmt, const uint8_t *__restrict__ codes,
                                             const uint8_t *__restrict__ scales, int64_t tile, const float *x,
                                             int P, int wave, int lane, float (&out)[RBW]) {
  const int s = lane >> 4;
  if (fmt == RSSM_READ_FP8) {
    constexpr int NCH = N / 16;
    constexpr int CI = (NCH + 3) / 4;
    uint4 raw[RBW][CI];
    float sc[RBW][CI];
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const int row = frag_row(wave, lane, i);
      const int64_t rowi = tile * P + row;
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) {
        const int ch = s + 4 * ci;
        if (row < P && ch < NCH) {
          raw[i][ci] = *(const uint4 *)(codes + rowi * N + 16 * ch);
          sc[i][ci] = ((const float *)scales)[rowi * (N / 32) + ch / 2];
        } else {
          raw[i][ci] = make_uint4(0, 0, 0, 0);
          sc[i][ci] = 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) {
        const int ch = s + 4 * ci;
        if (ch < NCH) {
          const float *xp = x + 16 * ch;
          const uint32_t w[4] = {raw[i][ci].x, raw[i][ci].y, raw[i][ci].z, raw[i][ci].w};
          float d = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[q], 1.0f, false);
            const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[q], 1.0f, true);
            const float4 xv = *(const float4 *)(xp + 4 * q);
            d = fmaf(lo[0], xv.x, d);
            d = fmaf(lo[1], xv.y, d);
            d = fmaf(hi[0], xv.z, d);
            d = fmaf(hi[1], xv.w, d);
          }
          acc = fmaf(sc[i][ci], d, acc);
        }
      }
      out[i] = acc;
    }
  } else {
    constexpr int NCH = N / 32;
    constexpr int CI = (NCH + 3) / 4;
    uint4 raw[RBW][CI];
    float sc[RBW][CI];
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const int row = frag_row(wave, lane, i);
      const int64_t rowi = tile * P + row;
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) {
        const int ch = s + 4 * ci;
        if (row < P && ch < NCH) {
          raw[i][ci] = *(const uint4 *)(codes + rowi * (N / 2) + 16 * ch);
          sc[i][ci] = __uint_as_float((uint32_t)scales[rowi * (N / 32) + ch] << 23);   // 2^(e8m0 - 127)
        } else {
          raw[i][ci] = make_uint4(0, 0, 0, 0);
          sc[i][ci] = 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) {
        const int ch = s + 4 * ci;
        if (ch < NCH) {
          const float *xp = x + 32 * ch;
          const uint32_t w[4] = {raw[i][ci].x, raw[i][ci].y, raw[i][ci].z, raw[i][ci].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 xa = *(const float4 *)(xp + 8 * q);
            const float4 xb = *(const float4 *)(xp + 8 * q + 4);
            const v2f v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc[i][ci], 0);
            const v2f v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc[i][ci], 1);
            const v2f v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc[i][ci], 2);
            const v2f v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], sc[i][ci], 3);
            acc = fmaf(v0[0], xa.x, acc);
            acc = fmaf(v0[1], xa.y, acc);
            acc = fmaf(v1[0], xa.z, acc);
            acc = fmaf(v1[1], xa.w, acc);
            acc = fmaf(v2[0], xb.x, acc);
            acc = fmaf(v2[1], xb.y, acc);
            acc = fmaf(v3[0], xb.z, acc);
            acc = fmaf(v3[1], xb.w, acc);
          }
        }
      }
      out[i] = acc;
    }
  }
}

// ---------------------------------------------------------------- record staging
// Record j < n_ring comes from ring slot (start + j) % C; record j in [n_ring, n_ring + n_in)
// is input record j - n_ring at the given element offsets and strides.
struct RecSrc {
  int n_ring;
  int n_in;
  int slot0;        // start % C
  int64_t a_idx, a_str;
  int64_t v_idx, v_str;
  int64_t k_idx, k_str;
};

template <int KIND, int N>
__device__ void stage_records(const Args &a, const LdsLayout &L, float *lds, int b, int hh, int gq,
                              const RecSrc &rs, int t) {
  const Geom &g = a.g;
  const int bf = g.bf16;
  const int nrec = rs.n_ring + rs.n_in;
  const int P = g.P;
  const uint8_t *rA = a.ring + g.off_alpha;
  const uint8_t *rB = a.ring + g.off_beta;
  const uint8_t *rV = a.ring + g.off_v;
  const uint8_t *rK = a.ring + g.off_k;
  const int64_t hrow = (int64_t)(b * g.H + hh) * g.C;   // alpha/beta/v ring row of this value head
  const int64_t krow = (int64_t)(b * g.G + gq) * g.C;   // k ring row of this key head
  for (int j = t; j < nrec; j += kThreads) {
    float al, be = 0.f;
    if (j < rs.n_ring) {
      int slot = rs.slot0 + j;
      if (slot >= g.C) slot -= g.C;
      al = ld_in(rA, hrow + slot, bf);
      if (KIND == RSSM_KIND_GDN) be = ld_in(rB, hrow + slot, bf);
    } else {
      const int64_t i = rs.a_idx + (int64_t)(j - rs.n_ring) * rs.a_str;
      al = ld_in(a.alpha, i, bf);
      if (KIND == RSSM_KIND_GDN) be = ld_in(a.beta, i, bf);
    }
    lds[L.alpha + j] = al;
    lds[L.beta + j] = be;
  }
  for (int e = t; e < nrec * P; e += kThreads) {
    const int j = e / P, p = e - j * P;
    float x;
    if (j < rs.n_ring) {
      int slot = rs.slot0 + j;
      if (slot >= g.C) slot -= g.C;
      x = ld_in(rV, (hrow + slot) * P + p, bf);
    } else {
      x = ld_in(a.v, rs.v_idx + (int64_t)(j - rs.n_ring) * rs.v_str + p, bf);
    }
    lds[L.V + e] = x;
  }
  for (int e = t; e < nrec * N; e += kThreads) {
    const int j = e / N, n = e % N;
    float x;
    if (j < rs.n_ring) {
      int slot = rs.slot0 + j;
      if (slot >= g.C) slot -= g.C;
      x = ld_in(rK, (krow + slot) * N + n, bf);
    } else {
      x = ld_in(a.k, rs.k_idx + (int64_t)(j - rs.n_ring) * rs.k_str + n, bf);
    }
    lds[L.K + j * (N + 4) + n] = x;
  }
}

// Append input record r (0-based) of the given source layout to ring slot `slot`.
template <int KIND, int N>
__device__ void append_record(const Args &a, int b, int hh, int gq, int slot, int64_t a_i, int64_t v_i,
                              int64_t k_i, int t) {
  const Geom &g = a.g;
  const int bf = g.bf16;
  const int P = g.P;
  const int64_t hr = (int64_t)(b * g.H + hh) * g.C + slot;
  if (t == 0) {
    cp_in(a.ring + g.off_alpha, hr, a.alpha, a_i, bf);
    if (KIND == RSSM_KIND_GDN) cp_in(a.ring + g.off_beta, hr, a.beta, a_i, bf);
  }
  for (int p = t; p < P; p += kThreads) cp_in(a.ring + g.off_v, hr * P + p, a.v, v_i + p, bf);
  if (hh % g.grp == 0) {
    const int64_t kr = ((int64_t)(b * g.G + gq) * g.C + slot) * N;
    for (int n = t; n < N; n += kThreads) {
      cp_in(a.ring + g.off_k, kr + n, a.k, k_i + n, bf);
      cp_in(a.ring + g.off_q, kr + n, a.q, k_i + n, bf);
    }
  }
}

// ---------------------------------------------------------------- coefficient phases
// d_j = prod_{j < m < nrec} alpha_m and G = prod_{m < nrec} alpha_m (records since the checkpoint).
__device__ __forceinline__ float suffix_decay(const float *alpha, int j, int last) {
  float d = 1.f;
  for (int m = last; m > j; --m) d *= alpha[m];
  return d;
}

// Mamba-2: e_j = d_j (k_j . x) for the nrec records, and G, for one query x.
template <int N>
__device__ void coef_m2(float *lds, const LdsLayout &L, int nrec, const float *x, float *coef, float *gam,
                        int t) {
  const int g16 = t >> 4, l16 = t & 15;
  const float *alpha = lds + L.alpha;
  for (int d = g16; d < nrec; d += kThreads / 16) {
    const float *kr = lds + L.K + d * (N + 4);
    float acc = 0.f;
#pragma unroll
    for (int n = l16; n < N; n += 16) acc = fmaf(kr[n], x[n], acc);
    acc = sum16(acc);
    if (l16 == 0) coef[d] = suffix_decay(alpha, d, nrec - 1) * acc;
  }
  if (t == 0) *gam = suffix_decay(alpha, -1, nrec - 1);
}

// Gated DeltaNet: Gram matrix K^T K (i < m) and K^T x for T queries over nrec records.
template <int N>
__device__ void gram_and_kq(float *lds, const LdsLayout &L, int cap, int nrec, int T, int t) {
  const int g16 = t >> 4, l16 = t & 15;
  const int nkq = T * nrec;
  const int nd = nkq + nrec * (nrec - 1) / 2;
  for (int d = g16; d < nd; d += kThreads / 16) {
    const float *A, *Bv;
    int i = 0, m = 0, tau = 0;
    if (d < nkq) {
      tau = d / nrec;
      i = d - tau * nrec;
      A = lds + L.K + i * (N + 4);
      Bv = lds + L.q + tau * N;
    } else {
      const int pp = d - nkq;
      m = 1;
      while ((m * (m + 1)) / 2 <= pp) ++m;
      i = pp - (m * (m - 1)) / 2;
      A = lds + L.K + i * (N + 4);
      Bv = lds + L.K + m * (N + 4);
    }
    float acc = 0.f;
#pragma unroll
    for (int n = l16; n < N; n += 16) acc = fmaf(A[n], Bv[n], acc);
    acc = sum16(acc);
    if (l16 == 0) {
      if (d < nkq)
        lds[L.coef + tau * cap + i] = acc;            // k_i . q_tau, replaced by e after the solve
      else
        lds[L.gram + i * (cap + 1) + m] = acc;        // k_i . k_m, i < m
    }
  }
}

// Query-transform solve for one query over records 0..n-1 (one wave; n <= 64):
// c_i = k_i . q - sum_{m > i} b_m c_m (k_i . k_m); writes c (cc row), e_i = d_i b_i c_i
// (coef row, replacing k_i . q) and the decay product G.
__device__ void gdn_solve_wave(float *lds, const LdsLayout &L, int cap, int n, int tau, int lane) {
  const float *alpha = lds + L.alpha;
  const float *beta = lds + L.beta;
  const float *gram = lds + L.gram;
  float *coef = lds + L.coef + tau * cap;
  float *cc = lds + L.cc + tau * cap;
  float x = (lane < n) ? coef[lane] : 0.f;
  for (int m = n - 1; m >= 0; --m) {
    const float cm = __shfl(x, m);
    if (lane < m) x = fmaf(-beta[m] * cm, gram[lane * (cap + 1) + m], x);
  }
  if (lane < n) {
    cc[lane] = x;
    coef[lane] = suffix_decay(alpha, lane, n - 1) * beta[lane] * x;
  }
  if (lane == 0) lds[L.gam + tau] = suffix_decay(alpha, -1, n - 1);
}

// r = q - sum_{i < n} b_i c_i k_i for query tau (threads stride over N).
template <int N>
__device__ void gdn_transform_query(float *lds, const LdsLayout &L, int cap, int n, int tau, int t0, int stride) {
  const float *beta = lds + L.beta;
  const float *cc = lds + L.cc + tau * cap;
  for (int e = t0; e < N; e += stride) {
    float r = lds[L.q + tau * N + e];
    for (int i = 0; i < n; ++i) r = fmaf(-beta[i] * cc[i], lds[L.K + i * (N + 4) + e], r);
    lds[L.r + tau * N + e] = r;
  }
}

// ---------------------------------------------------------------- folds
// Mamba-2 fold: S <- G S + sum_j d_j v_j k_j^T (decays in L.dec, G in L.gam).
template <int N, int RBW>
__device__ void fold_m2(Frag<N, RBW> &F, const float *lds, const LdsLayout &L, int nrec, int P, int wave,
                        int lane) {
  const int c = (lane >> 4) * 4;
  const float G = lds[L.gam];
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int f = 0; f < N / 16; ++f) {
      F.s[i][f].x *= G;
      F.s[i][f].y *= G;
      F.s[i][f].z *= G;
      F.s[i][f].w *= G;
    }
  for (int j = 0; j < nrec; ++j) {
    const float dj = lds[L.dec + j];
    const float *kr = lds + L.K + j * (N + 4) + c;
    float4 kf[N / 16];
#pragma unroll
    for (int f = 0; f < N / 16; ++f) kf[f] = *(const float4 *)(kr + 16 * f);
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const int row = frag_row(wave, lane, i);
      const float vr = (row < P) ? lds[L.V + j * P + row] * dj : 0.f;
#pragma unroll
      for (int f = 0; f < N / 16; ++f) {
        F.s[i][f].x = fmaf(vr, kf[f].x, F.s[i][f].x);
        F.s[i][f].y = fmaf(vr, kf[f].y, F.s[i][f].y);
        F.s[i][f].z = fmaf(vr, kf[f].z, F.s[i][f].z);
        F.s[i][f].w = fmaf(vr, kf[f].w, F.s[i][f].w);
      }
    }
  }
}

// Gated DeltaNet fold, one delta-rule update per record in registers:
// S <- a S ; u = b (v - S k) ; S <- S + u k^T.
template <int N, int RBW>
__device__ void fold_gdn(Frag<N, RBW> &F, const float *lds, const LdsLayout &L, int nrec, int P, int wave,
                         int lane) {
  const int c = (lane >> 4) * 4;
  for (int j = 0; j < nrec; ++j) {
    const float al = lds[L.alpha + j], be = lds[L.beta + j];
    const float *kr = lds + L.K + j * (N + 4) + c;
    float4 kf[N / 16];
#pragma unroll
    for (int f = 0; f < N / 16; ++f) kf[f] = *(const float4 *)(kr + 16 * f);
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      float w = 0.f;
#pragma unroll
      for (int f = 0; f < N / 16; ++f) w = dot4(F.s[i][f], kf[f], w);
      w = quad_sum(w);
      const int row = frag_row(wave, lane, i);
      const float vr = (row < P) ? lds[L.V + j * P + row] : 0.f;
      const float u = be * (vr - al * w);
#pragma unroll
      for (int f = 0; f < N / 16; ++f) {
        F.s[i][f].x = fmaf(al, F.s[i][f].x, u * kf[f].x);
        F.s[i][f].y = fmaf(al, F.s[i][f].y, u * kf[f].y);
        F.s[i][f].z = fmaf(al, F.s[i][f].z, u * kf[f].z);
        F.s[i][f].w = fmaf(al, F.s[i][f].w, u * kf[f].w);
      }
    }
  }
}

// Output rows: y[row] = G * (S x)[row] + sum_{j} coef[j] v_j[row]; lanes with l/16 = s take j = s mod 4.
template <int RBW>
__device__ __forceinline__ void write_rows(const float (&part)[RBW], float G, const float *lds, const LdsLayout &L,
                                           const float *coef, int nrec, int P, float *__restrict__ out, int wave,
                                           int lane) {
  const int s = lane >> 4;
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int row = frag_row(wave, lane, i);
    float buf = 0.f;
    if (row < P)
      for (int j = s; j < nrec; j += 4) buf = fmaf(coef[j], lds[L.V + j * P + row], buf);
    const float y = quad_sum(fmaf(G, part[i], buf));
    if (s == 0 && row < P) out[row] = y;
  }
}

// ================================================================ kernels

template <int KIND, int N, int RBW>
__global__ __launch_bounds__(kThreads) void k_decode(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t nc = a.n_committed[tile], nk = a.n_ckpt[tile];
  const int64_t hb64 = nc - nk;
  if (hb64 < 0 || hb64 > g.C) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  const int hb = (int)hb64, nrec = hb + 1;
  const bool flush = nrec >= g.L;
  const int P = g.P;
  const int cap = g.C + 1;
  const LdsLayout L = lds_layout(KIND, cap, 1, P, N);
  float *tileS = a.s + (int64_t)tile * P * N;
  const bool from_copy = (g.read_copy != RSSM_READ_NONE) && !flush;

  Frag<N, RBW> F;
  if (!from_copy) frag_load(F, tileS, P, wave, lane);

  RecSrc rs;
  rs.n_ring = hb;
  rs.n_in = 1;
  rs.slot0 = (int)(nk % g.C);
  rs.a_idx = (int64_t)b * g.H + hh;
  rs.a_str = 0;
  rs.v_idx = ((int64_t)b * g.H + hh) * P;
  rs.v_str = 0;
  rs.k_idx = ((int64_t)b * g.G + gq) * N;
  rs.k_str = 0;
  stage_records<KIND, N>(a, L, lds, b, hh, gq, rs, t);
  for (int n = t; n < N; n += kThreads) lds[L.q + n] = ld_in(a.q, rs.k_idx + n, g.bf16);
  __syncthreads();

  float *yout = a.out + ((int64_t)b * g.H + hh) * P;
  if (flush) {
    if (KIND == RSSM_KIND_MAMBA2) {
      for (int j = t; j < nrec; j += kThreads) lds[L.dec + j] = suffix_decay(lds + L.alpha, j, nrec - 1);
      if (t == 0) lds[L.gam] = suffix_decay(lds + L.alpha, -1, nrec - 1);
      __syncthreads();
      fold_m2(F, lds, L, nrec, P, wave, lane);
    } else {
      fold_gdn(F, lds, L, nrec, P, wave, lane);
    }
    frag_store(F, tileS, P, wave, lane);
    if (g.read_copy != RSSM_READ_NONE) frag_store_read_copy(F, g.read_copy, a.s_read, a.s_read_scale, tile, P, wave, lane);
    float part[RBW];
    frag_dot(F, lds + L.q, lane, part);
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const int row = frag_row(wave, lane, i);
      const float y = quad_sum(part[i]);
      if ((lane >> 4) == 0 && row < P) yout[row] = y;
    }
  } else {
    const float *x;
    if (KIND == RSSM_KIND_MAMBA2) {
      coef_m2<N>(lds, L, nrec, lds + L.q, lds + L.coef, lds + L.gam, t);
      __syncthreads();
      x = lds + L.q;
    } else {
      gram_and_kq<N>(lds, L, cap, nrec, 1, t);
      __syncthreads();
      if (wave == 0) gdn_solve_wave(lds, L, cap, nrec, 0, lane);
      __syncthreads();
      gdn_transform_query<N>(lds, L, cap, nrec, 0, t, kThreads);
      __syncthreads();
      x = lds + L.r;
    }
    float part[RBW];
    if (from_copy)
      readcopy_dot<N, RBW>(g.read_copy, a.s_read, a.s_read_scale, tile, x, P, wave, lane, part);
    else
      frag_dot(F, x, lane, part);
    write_rows<RBW>(part, lds[L.gam], lds, L, lds + L.coef, nrec, P, yout, wave, lane);
    append_record<KIND, N>(a, b, hh, gq, (int)(nc % g.C), rs.a_idx, rs.v_idx, rs.k_idx, t);
  }
  if (t == 0) {
    a.n_committed[tile] = nc + 1;
    if (flush) a.n_ckpt[tile] = nc + 1;
  }
}

template <int KIND, int N, int RBW>
__global__ __launch_bounds__(kThreads) void k_verify(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int T = a.T;
  const int64_t nc = a.n_committed[tile], nk = a.n_ckpt[tile];
  const int64_t hb64 = nc - nk;
  if (hb64 < 0 || hb64 > g.C) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  const int hb = (int)hb64;
  if (hb + T > g.C) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_VERIFY_CAPACITY);
    return;
  }
  const int nrec = hb + T;
  const int P = g.P;
  const int cap = g.C;
  const LdsLayout L = lds_layout(KIND, cap, T, P, N);
  const float *tileS = a.s + (int64_t)tile * P * N;

  Frag<N, RBW> F;
  frag_load(F, tileS, P, wave, lane);

  RecSrc rs;
  rs.n_ring = hb;
  rs.n_in = T;
  rs.slot0 = (int)(nk % g.C);
  rs.a_idx = (int64_t)b * T * g.H + hh;
  rs.a_str = g.H;
  rs.v_idx = ((int64_t)b * T * g.H + hh) * P;
  rs.v_str = (int64_t)g.H * P;
  rs.k_idx = ((int64_t)b * T * g.G + gq) * N;
  rs.k_str = (int64_t)g.G * N;
  stage_records<KIND, N>(a, L, lds, b, hh, gq, rs, t);
  for (int e = t; e < T * N; e += kThreads) {
    const int tau = e / N, n = e - tau * N;
    lds[L.q + e] = ld_in(a.q, rs.k_idx + tau * rs.k_str + n, g.bf16);
  }
  __syncthreads();

  const float *xbase;
  if (KIND == RSSM_KIND_MAMBA2) {
    // e[tau][j] = W[j, tau] (k_j . q_tau), W[j, tau] = prod_{j < m <= hb + tau} alpha_m for j <= hb + tau
    const int g16 = t >> 4, l16 = t & 15;
    const float *alpha = lds + L.alpha;
    for (int d = g16; d < T * nrec; d += kThreads / 16) {
      const int tau = d / nrec, j = d - tau * nrec;
      const float *kr = lds + L.K + j * (N + 4);
      const float *qr = lds + L.q + tau * N;
      float acc = 0.f;
#pragma unroll
      for (int n = l16; n < N; n += 16) acc = fmaf(kr[n], qr[n], acc);
      acc = sum16(acc);
      if (l16 == 0) lds[L.coef + tau * cap + j] = (j <= hb + tau) ? suffix_decay(alpha, j, hb + tau) * acc : 0.f;
    }
    if (t < T) lds[L.gam + t] = suffix_decay(alpha, -1, hb + t);
    __syncthreads();
    xbase = lds + L.q;
  } else {
    gram_and_kq<N>(lds, L, cap, nrec, T, t);
    __syncthreads();
    for (int tau = wave; tau < T; tau += kWaves) gdn_solve_wave(lds, L, cap, hb + tau + 1, tau, lane);
    __syncthreads();
    for (int e = t; e < T * N; e += kThreads) {
      const int tau = e / N;
      gdn_transform_query<N>(lds, L, cap, hb + tau + 1, tau, e - tau * N, N);
    }
    __syncthreads();
    xbase = lds + L.r;
  }

  for (int tau = 0; tau < T; ++tau) {
    float part[RBW];
    frag_dot(F, xbase + tau * N, lane, part);
    float *orow = a.out + (((int64_t)b * T + tau) * g.H + hh) * P;
    write_rows<RBW>(part, lds[L.gam + tau], lds, L, lds + L.coef + tau * cap, hb + tau + 1, P, orow, wave, lane);
  }
  for (int tau = 0; tau < T; ++tau) {
    int slot = (int)((nc + tau) % g.C);
    append_record<KIND, N>(a, b, hh, gq, slot, rs.a_idx + tau * rs.a_str, rs.v_idx + tau * rs.v_str,
                           rs.k_idx + tau * rs.k_str, t);
  }
}

template <int KIND, int N, int RBW>
__global__ __launch_bounds__(kThreads) void k_flush(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t nc = a.n_committed[tile], nk = a.n_ckpt[tile];
  const int64_t hb64 = nc - nk;
  if (hb64 < 0 || hb64 > g.C) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  const int nrec = (int)hb64;
  const int thr = a.min_records > 1 ? a.min_records : 1;
  if (nrec < thr) return;
  const int P = g.P;
  const int cap = g.C;
  const LdsLayout L = lds_layout(KIND, cap, 1, P, N);
  float *tileS = a.s + (int64_t)tile * P * N;

  Frag<N, RBW> F;
  frag_load(F, tileS, P, wave, lane);
  RecSrc rs;
  rs.n_ring = nrec;
  rs.n_in = 0;
  rs.slot0 = (int)(nk % g.C);
  rs.a_idx = rs.a_str = rs.v_idx = rs.v_str = rs.k_idx = rs.k_str = 0;
  stage_records<KIND, N>(a, L, lds, b, hh, gq, rs, t);
  __syncthreads();
  if (KIND == RSSM_KIND_MAMBA2) {
    for (int j = t; j < nrec; j += kThreads) lds[L.dec + j] = suffix_decay(lds + L.alpha, j, nrec - 1);
    if (t == 0) lds[L.gam] = suffix_decay(lds + L.alpha, -1, nrec - 1);
    __syncthreads();
    fold_m2(F, lds, L, nrec, P, wave, lane);
  } else {
    fold_gdn(F, lds, L, nrec, P, wave, lane);
  }
  frag_store(F, tileS, P, wave, lane);
  if (g.read_copy != RSSM_READ_NONE) frag_store_read_copy(F, g.read_copy, a.s_read, a.s_read_scale, tile, P, wave, lane);
  if (t == 0) a.n_ckpt[tile] = nc;
}

template <int KIND, int N, int RBW>
__global__ __launch_bounds__(kThreads) void k_conventional(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int P = g.P;
  const LdsLayout L = lds_layout(KIND, 1, 1, P, N);
  float *tileS = a.s + (int64_t)tile * P * N;
  Frag<N, RBW> F;
  frag_load(F, tileS, P, wave, lane);
  RecSrc rs;
  rs.n_ring = 0;
  rs.n_in = 1;
  rs.slot0 = 0;
  rs.a_idx = (int64_t)b * g.H + hh;
  rs.a_str = 0;
  rs.v_idx = ((int64_t)b * g.H + hh) * P;
  rs.v_str = 0;
  rs.k_idx = ((int64_t)b * g.G + gq) * N;
  rs.k_str = 0;
  stage_records<KIND, N>(a, L, lds, b, hh, gq, rs, t);
  for (int n = t; n < N; n += kThreads) lds[L.q + n] = ld_in(a.q, rs.k_idx + n, g.bf16);
  __syncthreads();
  const int c = (lane >> 4) * 4;
  const float al = lds[L.alpha];
  float4 kf[N / 16];
#pragma unroll
  for (int f = 0; f < N / 16; ++f) kf[f] = *(const float4 *)(lds + L.K + c + 16 * f);
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int row = frag_row(wave, lane, i);
    const float vr = (row < P) ? lds[L.V + row] : 0.f;
    float u;
    if (KIND == RSSM_KIND_MAMBA2) {
      u = vr;
    } else {
      float w = 0.f;
#pragma unroll
      for (int f = 0; f < N / 16; ++f) w = dot4(F.s[i][f], kf[f], w);
      w = quad_sum(w);
      u = lds[L.beta] * (vr - al * w);
    }
#pragma unroll
    for (int f = 0; f < N / 16; ++f) {
      F.s[i][f].x = fmaf(al, F.s[i][f].x, u * kf[f].x);
      F.s[i][f].y = fmaf(al, F.s[i][f].y, u * kf[f].y);
      F.s[i][f].z = fmaf(al, F.s[i][f].z, u * kf[f].z);
      F.s[i][f].w = fmaf(al, F.s[i][f].w, u * kf[f].w);
    }
  }
  frag_store(F, tileS, P, wave, lane);
  float part[RBW];
  frag_dot(F, lds + L.q, lane, part);
  float *yout = a.out + ((int64_t)b * g.H + hh) * P;
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int row = frag_row(wave, lane, i);
    const float y = quad_sum(part[i]);
    if ((lane >> 4) == 0 && row < P) yout[row] = y;
  }
}

template <int N, int RBW>
__global__ __launch_bounds__(kThreads) void k_init(Args a) {
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int P = g.P;
  Frag<N, RBW> F;
  if (a.s0)
    frag_load(F, a.s0 + (int64_t)tile * P * N, P, wave, lane);
  else
    frag_zero(F);
  frag_store(F, a.s + (int64_t)tile * P * N, P, wave, lane);
  if (g.read_copy != RSSM_READ_NONE) frag_store_read_copy(F, g.read_copy, a.s_read, a.s_read_scale, tile, P, wave, lane);
  if (t == 0) {
    a.n_committed[tile] = 0;
    a.n_ckpt[tile] = 0;
    if (blockIdx.x == 0) *a.err = 0;
  }
}

// Dispatch over the supported (N, RBW) instances; CALL(n, r) must return.
#define RSSM_DISPATCH(N_, RBW_, CALL)                 \
  switch (N_) {                                       \
    case 32:                                          \
      switch (RBW_) {                                 \
        case 1: CALL(32, 1);                          \
        case 2: CALL(32, 2);                          \
        case 4: CALL(32, 4);                          \
        case 8: CALL(32, 8);                          \
        default: break;                               \
      }                                               \
      break;                                          \
    case 64:                                          \
      switch (RBW_) {                                 \
        case 1: CALL(64, 1);                          \
        case 2: CALL(64, 2);                          \
        case 4: CALL(64, 4);                          \
        default: break;                               \
      }                                               \
      break;                                          \
    case 128:                                         \
      switch (RBW_) {                                 \
        case 1: CALL(128, 1);                         \
        case 2: CALL(128, 2);                         \
        default: break;                               \
      }                                               \
      break;                                          \
    case 256:                                         \
      if (RBW_ == 1) CALL(256, 1);                    \
      break;                                          \
    default: break;                                   \
  }                                                   \
  return hipErrorInvalidValue;

}  // namespace rssm
