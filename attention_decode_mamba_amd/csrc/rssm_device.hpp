// Device helpers and kernel templates of the ReplaySSM decode path (gfx950).
//
// One workgroup (4 waves of 64 lanes) owns one (sequence, value-head) tile: the
// P x N fp32 checkpoint tile S_ckpt, its ring records and its cursor replica.
//
// Register layout of a tile ("row-octet layout"): row group g = wave + 4*i (i < RGW)
// holds rows 8g .. 8g+7; lane l takes row 8g + l/8 and, for every 32-column fragment f,
// the float4 S[8g + l/8][32f + 4(l%8) .. +3].  One load instruction therefore covers
// 8 rows x 128 contiguous bytes; a row dot product is N/32 float4 FMAs per lane plus
// three cross-lane adds within the 8 lanes of the row; and a 32-element read-copy block
// is exactly one fragment of one row.
//
// Latency structure of every kernel: the cursor is read first; then all loads of
// the ring records, step inputs and queries are issued (16-byte chunks), then the
// loads of the checkpoint tile (or its read copy); the staged records are written
// to LDS while the tile is still in flight, so one workgroup waits for one memory
// round trip, not one per record.
#pragma once

#include "rssm_internal.hpp"

namespace rssm {

// ---------------------------------------------------------------- element access
__device__ __forceinline__ float bf16f(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

__device__ __forceinline__ float ld_in(const void *base, int64_t i, int bf16) {
  return bf16 ? bf16f(((const uint16_t *)base)[i]) : ((const float *)base)[i];
}

// Workgroups are dispatched round-robin over the 8 XCDs.  By default each XCD gets a
// contiguous range of tiles, so tiles sharing key/query rows (GDN groups) share an L2 and
// the workgroups running at once on an XCD read and append neighbouring rows.  Kernels whose
// per-sequence cost varies (a flush where only some sequences fold, a verify whose windows
// differ) take SPREAD: block order = tile order, so a sequence's heads land on all XCDs and
// the busy sequences do not pile up on a few of them.
template <bool SPREAD = false>
__device__ __forceinline__ int tile_of_block(int ntiles) {
  const int bid = blockIdx.x;
  if (!SPREAD && (ntiles & 7) == 0) {
    const int per = ntiles >> 3;
    return (bid & 7) * per + (bid >> 3);
  }
  return bid;
}

// Cross-lane moves inside a DPP row of 16 lanes (no LDS round trip): quad permutation
// [1,0,3,2] (lane ^ 1), quad permutation [2,3,0,1] (lane ^ 2), half-row mirror (lane i of
// each 8 takes lane 7 - i) and row mirror (lane i of each 16 takes lane 15 - i).  Every
// source lane lies in the same row, so all lanes of the row must be active.
enum : int { kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141 };

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum / max over the 8 lanes that share a row (lanes l with equal l / 8).  After the two
// quad steps every lane holds its quad's result; the half-row mirror pairs each lane with
// a lane of the other quad.  Each step adds commuted pairs, so all 8 lanes end bitwise equal.
__device__ __forceinline__ float oct_sum(float v) {
  v += dpp_mov<kDppQuadXor1>(v);
  v += dpp_mov<kDppQuadXor2>(v);
  v += dpp_mov<kDppRowHalfMirror>(v);
  return v;
}

__device__ __forceinline__ float oct_max(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  return v;
}

// Sum over the 16 lanes of a DPP row (lanes l with equal l / 16).
__device__ __forceinline__ float sum16(float v) {
  v = oct_sum(v);
  v += dpp_mov<kDppRowMirror>(v);
  return v;
}

// Value of x in lane m (m uniform across the wave).
__device__ __forceinline__ float lane_value(float x, int m) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), m));
}

// x_l <- prod_{m >= l} x_m over the 64 lanes of the wave (all lanes must be active).
__device__ __forceinline__ float wave_suffix_product(float x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_down(x, o);
    if (lane + o < 64) x *= y;
  }
  return x;
}

// x_l <- prod_{m >= l} x_m within each DPP row of 16 lanes (lanes past the row count as 1).
// For lanes 0..15 of a wave whose lanes 16..63 hold 1 this is bit-identical to
// wave_suffix_product: the products are taken in the same order, and the steps that
// wave_suffix_product adds past 16 lanes multiply by exactly 1.
template <int CTRL>
__device__ __forceinline__ float dpp_or_one(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_suffix_product(float x) {
  x *= dpp_or_one<0x101>(x);      // row_shl:1 (lane l reads lane l + 1)
  x *= dpp_or_one<0x102>(x);      // row_shl:2
  x *= dpp_or_one<0x104>(x);      // row_shl:4
  x *= dpp_or_one<0x108>(x);      // row_shl:8
  return x;
}

// ---------------------------------------------------------------- fragments
template <int N, int RGW>
struct Frag {
  float4 s[RGW][N / 32];
};

__device__ __forceinline__ int frag_row(int wave, int lane, int i) { return 8 * (wave + kWaves * i) + (lane >> 3); }
__device__ __forceinline__ int frag_col(int lane) { return 4 * (lane & 7); }

typedef float f4v __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ float4 ld4(const float4 *p) {
  if (NT) {
    const f4v v = __builtin_nontemporal_load((const f4v *)p);
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  return *p;
}

template <int N, int RGW>
__device__ __forceinline__ void frag_zero(Frag<N, RGW> &F) {
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int f = 0; f < N / 32; ++f) F.s[i][f] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Rows past P (ragged tails) load a copy of row P - 1: every load is unconditional, so the
// loads stay in flight across the staging code.  Such rows never interact with real rows
// (all cross-lane sums stay within a row) and are never stored.  NT: streaming loads
// (the tile is read once per step).
template <int N, int RGW, bool NT>
__device__ __forceinline__ void frag_load(Frag<N, RGW> &F, const float *__restrict__ tile, int P, int wave,
                                          int lane) {
  const int c = frag_col(lane);
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    int row = frag_row(wave, lane, i);
    row = row < P ? row : P - 1;
    const float4 *src = (const float4 *)(tile + (int64_t)row * N + c);
#pragma unroll
    for (int f = 0; f < N / 32; ++f) F.s[i][f] = ld4<NT>(src + 8 * f);
  }
}

// Tiles written back are stored with nontemporal, device-scope (sc1) buffer stores: the
// lines go through the XCD's L2 without displacing what the running workgroups still read
// (a layer's checkpoint is next read a whole step of the other layers later).  The tile
// base is uniform across the workgroup, so it fits a buffer descriptor.
template <int N, int RGW>
__device__ __forceinline__ void frag_store(const Frag<N, RGW> &F, float *__restrict__ tile, int P, int wave,
                                           int lane) {
  constexpr int kNtSc1 = 2 | 16;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(tile, 0, P * N * 4, 0x00020000);
  const int c = frag_col(lane);
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    const int row = frag_row(wave, lane, i);
    if (row < P) {
#pragma unroll
      for (int f = 0; f < N / 32; ++f) {
        const float4 x = F.s[i][f];
        f4v v;
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, (row * N + c + 32 * f) * 4, 0, kNtSc1);
      }
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
template <int N, int RGW>
__device__ __forceinline__ void frag_dot(const Frag<N, RGW> &F, const float *x, int lane, float (&out)[RGW]) {
  const int c = frag_col(lane);
#pragma unroll
  for (int i = 0; i < RGW; ++i) out[i] = 0.f;
#pragma unroll
  for (int f = 0; f < N / 32; ++f) {
    const float4 xv = *(const float4 *)(x + 32 * f + c);
#pragma unroll
    for (int i = 0; i < RGW; ++i) out[i] = dot4(F.s[i][f], xv, out[i]);
  }
}

// Row results of a per-lane partial: lanes with l%8 == 0 write out[row].
template <int RGW>
__device__ __forceinline__ void write_row_sums(const float (&part)[RGW], int P, float *__restrict__ out, int wave,
                                               int lane) {
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    const int row = frag_row(wave, lane, i);
    const float y = oct_sum(part[i]);
    if ((lane & 7) == 0 && row < P) out[row] = y;
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

// Quantise the tile held in registers and store the read copy (FMT: fp8 or MXFP4; nothing
// for RSSM_READ_NONE).  A 32-element block is fragment f of one row: 8 lanes x 4 values.
// The format is a template parameter: a kernel that writes no read copy carries no
// quantiser code, and one that does carries only its format's.
template <int FMT, int N, int RGW>
__device__ __forceinline__ void frag_store_read_copy(const Frag<N, RGW> &F, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales, int64_t tile, int P, int wave,
                                                     int lane) {
  if constexpr (FMT == RSSM_READ_NONE) return;
  const int c = frag_col(lane);
  const bool lead = (lane & 7) == 0;
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    const int row = frag_row(wave, lane, i);
    const int64_t rowi = tile * P + row;
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      const float4 v = F.s[i][f];
      float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
      am = oct_max(am);
      if constexpr (FMT == RSSM_READ_FP8) {
        const float sc = __fdiv_rn(am, 448.0f);
        uint32_t w = 0;
        if (sc > 0.f)
          w = f32_to_e4m3(__fdiv_rn(v.x, sc)) | (f32_to_e4m3(__fdiv_rn(v.y, sc)) << 8) |
              (f32_to_e4m3(__fdiv_rn(v.z, sc)) << 16) | (f32_to_e4m3(__fdiv_rn(v.w, sc)) << 24);
        if (row < P) {
          *(uint32_t *)(codes + rowi * N + 32 * f + c) = w;
          if (lead) ((float *)scales)[rowi * (N / 32) + f] = sc;
        }
      } else {
        int E = (am > 0.f) ? ilog2f(am) - 2 : -126;
        E = E < -126 ? -126 : (E > 127 ? 127 : E);                        // scale stays a normal float
        const float inv = __uint_as_float((uint32_t)(127 - E) << 23);   // 2^-E (E <= 125 for finite amax)
        const uint32_t h = f32_to_e2m1(v.x * inv) | (f32_to_e2m1(v.y * inv) << 4) |
                           (f32_to_e2m1(v.z * inv) << 8) | (f32_to_e2m1(v.w * inv) << 12);
        if (row < P) {
          *(uint16_t *)(codes + rowi * (N / 2) + 16 * f + c / 2) = (uint16_t)h;
          if (lead) scales[rowi * (N / 32) + f] = (uint8_t)(E + 127);
        }
      }
    }
  }
}

// Read-copy store for a format known only at run time (initialisation).
template <int N, int RGW>
__device__ __forceinline__ void frag_store_read_copy_rt(const Frag<N, RGW> &F, int fmt, uint8_t *__restrict__ codes,
                                                        uint8_t *__restrict__ scales, int64_t tile, int P, int wave,
                                                        int lane) {
  if (fmt == RSSM_READ_FP8)
    frag_store_read_copy<RSSM_READ_FP8>(F, codes, scales, tile, P, wave, lane);
  else if (fmt == RSSM_READ_MXFP4)
    frag_store_read_copy<RSSM_READ_MXFP4>(F, codes, scales, tile, P, wave, lane);
}

typedef float v2f __attribute__((ext_vector_type(2)));

// Read-copy registers of the lane's rows.  A row's codes are cut into chunks of 16
// elements (fp8: 16 bytes, MXFP4: 8 bytes); lane l takes chunks k = l%8 + 8*ci, so one
// load instruction covers 8 rows x 128 (fp8) or 64 (MXFP4) contiguous bytes.
template <int N, int RGW>
struct RCopy {
  static constexpr int NCH = N / 16;
  static constexpr int CI = (NCH + 7) / 8;
  uint4 raw[RGW][CI];
  uint32_t scb[RGW][CI];     // block scale as stored: fp32 bits (fp8) or the E8M0 byte (MXFP4)
};

// All loads are issued back to back: the format branch is outside the loops and nothing
// is decoded here, so no load waits for another (decoding happens in readcopy_dot).
// Row group i of the lane is row row0 + rstep * i.
template <int N, int RGW>
__device__ __forceinline__ void readcopy_load_rows(RCopy<N, RGW> &R, int fmt, const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int64_t tile, int P,
                                                   int row0, int rstep, int lane) {
  constexpr int NCH = RCopy<N, RGW>::NCH;
  const int c8 = lane & 7;
  // The tile's codes and scales start at a workgroup-uniform address; rows are 32-bit
  // offsets from it (a tile's read copy is far below 4 GB).
  if (fmt == RSSM_READ_FP8) {
    const uint8_t *cb = codes + tile * P * N;
    const uint8_t *sb = scales + tile * P * (N / 32) * 4;
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      int row = row0 + rstep * i;
      row = row < P ? row : P - 1;               // ragged rows: a copy of row P - 1, never stored
#pragma unroll
      for (int ci = 0; ci < RCopy<N, RGW>::CI; ++ci) {
        const int k = c8 + 8 * ci;
        const int kc = k < NCH ? k : NCH - 1;
        const f4v v = __builtin_nontemporal_load((const f4v *)(cb + (uint32_t)(row * N + 16 * kc)));
        R.raw[i][ci] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                  __float_as_uint(v[3]));
        R.scb[i][ci] = *(const uint32_t *)(sb + (uint32_t)(row * (N / 32) * 4 + (kc / 2) * 4));
      }
    }
  } else {
    const uint8_t *cb = codes + tile * P * (N / 2);
    const uint8_t *sb = scales + tile * P * (N / 32);
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      int row = row0 + rstep * i;
      row = row < P ? row : P - 1;
#pragma unroll
      for (int ci = 0; ci < RCopy<N, RGW>::CI; ++ci) {
        const int k = c8 + 8 * ci;
        const int kc = k < NCH ? k : NCH - 1;
        const uint2 v = *(const uint2 *)(cb + (uint32_t)(row * (N / 2) + 8 * kc));
        R.raw[i][ci] = make_uint4(v.x, v.y, 0, 0);
        R.scb[i][ci] = sb[(uint32_t)(row * (N / 32) + kc / 2)];
      }
    }
  }
}

// The lane's rows in the row-octet layout of a 4-wave tile.
template <int N, int RGW>
__device__ __forceinline__ void readcopy_load(RCopy<N, RGW> &R, int fmt, const uint8_t *__restrict__ codes,
                                              const uint8_t *__restrict__ scales, int64_t tile, int P, int wave,
                                              int lane) {
  readcopy_load_rows(R, fmt, codes, scales, tile, P, frag_row(wave, lane, 0), 8 * kWaves, lane);
}

// Per-lane partial of S_read x from loaded read-copy registers.  Each 4-element slice of x
// is read from LDS once and used for every row group of the lane (the lane's chunks are the
// same columns in every row group).
template <int N, int RGW>
__device__ __forceinline__ void readcopy_dot(const RCopy<N, RGW> &R, int fmt, const float *x, int lane,
                                             float (&out)[RGW]) {
  const int c8 = lane & 7;
  float acc[RGW];
#pragma unroll
  for (int i = 0; i < RGW; ++i) acc[i] = 0.f;
#pragma unroll
  for (int ci = 0; ci < RCopy<N, RGW>::CI; ++ci) {
    const int k = c8 + 8 * ci;
    const bool has = k < RCopy<N, RGW>::NCH;   // lanes past the row's chunks contribute nothing
    const float *xp = x + 16 * (has ? k : 0);
    if (fmt == RSSM_READ_FP8) {
      float d[RGW];
#pragma unroll
      for (int i = 0; i < RGW; ++i) d[i] = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 xv = *(const float4 *)(xp + 4 * q);
#pragma unroll
        for (int i = 0; i < RGW; ++i) {
          const uint4 w = has ? R.raw[i][ci] : make_uint4(0, 0, 0, 0);
          const uint32_t ws = q == 0 ? w.x : (q == 1 ? w.y : (q == 2 ? w.z : w.w));
          const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ws, 1.0f, false);
          const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ws, 1.0f, true);
          d[i] = fmaf(lo[0], xv.x, d[i]);
          d[i] = fmaf(lo[1], xv.y, d[i]);
          d[i] = fmaf(hi[0], xv.z, d[i]);
          d[i] = fmaf(hi[1], xv.w, d[i]);
        }
      }
      // fp8: the fp32 block scale multiplies the chunk's dot product
#pragma unroll
      for (int i = 0; i < RGW; ++i) acc[i] = fmaf(has ? __uint_as_float(R.scb[i][ci]) : 0.f, d[i], acc[i]);
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float4 xa = *(const float4 *)(xp + 8 * q);
        const float4 xb = *(const float4 *)(xp + 8 * q + 4);
#pragma unroll
        for (int i = 0; i < RGW; ++i) {
          const uint4 w = has ? R.raw[i][ci] : make_uint4(0, 0, 0, 0);
          const uint32_t ws = q == 0 ? w.x : w.y;
          // MXFP4: 2^(e8m0 - 127) is the e8m0 byte in the fp32 exponent field
          const float sc = has ? __uint_as_float(R.scb[i][ci] << 23) : 0.f;
          const v2f v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws, sc, 0);
          const v2f v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws, sc, 1);
          const v2f v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws, sc, 2);
          const v2f v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws, sc, 3);
          acc[i] = fmaf(v0[0], xa.x, acc[i]);
          acc[i] = fmaf(v0[1], xa.y, acc[i]);
          acc[i] = fmaf(v1[0], xa.z, acc[i]);
          acc[i] = fmaf(v1[1], xa.w, acc[i]);
          acc[i] = fmaf(v2[0], xb.x, acc[i]);
          acc[i] = fmaf(v2[1], xb.y, acc[i]);
          acc[i] = fmaf(v3[0], xb.z, acc[i]);
          acc[i] = fmaf(v3[1], xb.w, acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RGW; ++i) out[i] = acc[i];
}

// ---------------------------------------------------------------- record staging
// Records j < n_ring come from ring slot (slot0 + j) % C; records j in [n_ring, nrec)
// are input records j - n_ring (element offsets iv0/ik0 + (j - n_ring) * stride).
// Queries are nq input rows (iq0 + r * iqs).  Everything lands in LDS as fp32:
// alpha[j], beta[j], V[j][P], K[j][N+4], Q[r][N].
// Element indices are 32-bit: the host bounds every ring region and input below 2^31
// elements.
struct StageSpec {
  int nrec, n_ring, slot0, C, P, N, nq, bf16;
  int cpv_lg;                            // log2 of 16-byte chunks per value row, or -1
  int avec;                              // alpha is an N-vector per record (KDA)
  const uint8_t *rA, *rB, *rV, *rK;      // ring regions
  int hrow, krow;                        // this value head's / key head's row within a slot
  int hstr, kstr;                        // rows per slot: B*H value-head rows, B*G key-head rows
  const void *iA, *iB, *iV, *iK, *iQ;    // inputs
  int ia0, ias, iv0, ivs, ik0, iks, iq0, iqs;
  float *A, *Bt, *V, *K, *Q;             // LDS
};

// x mod C for a cursor position x >= 0 (a 32-bit remainder while x fits in 32 bits).
__device__ __forceinline__ int ring_mod(int64_t x, int C) {
  if ((uint64_t)x < ((uint64_t)1 << 32)) return (int)((uint32_t)x % (uint32_t)C);
  return (int)(x % C);
}

// (s0 + d) mod C for 0 <= s0 < C and 0 <= d <= C.
__device__ __forceinline__ int ring_add(int s0, int d, int C) {
  const int s = s0 + d;
  return s >= C ? s - C : s;
}

__device__ __forceinline__ int ring_slot(const StageSpec &sp, int j) {
  int s = sp.slot0 + j;
  return s >= sp.C ? s - sp.C : s;
}

// Vectorised staging: 16-byte chunks (8 bf16 or 4 fp32 elements), U chunks per thread
// per round.  stage_issue() loads one round into registers, stage_commit() writes it.
template <int U>
struct StageRegs {
  uint4 raw[U];
  int dst[U];        // LDS float offset of the chunk, -1 when idle
  float a, b;        // alpha / beta of record t (thread t < nrec)
};

__device__ __forceinline__ int stage_chunks(const StageSpec &sp, int epc) {
  return sp.nrec * (sp.P / epc) + sp.nrec * (sp.N / epc) * (1 + sp.avec) + sp.nq * (sp.N / epc);
}

// Issue one round of staging loads.  Every lane issues every load (idle chunks re-read the
// last valid chunk and are marked dst = -1), so the loads form straight-line code.
// Chunk order: v rows, k rows, alpha rows (AVEC: KDA's per-channel gates), query rows.
template <int U, bool BF, bool HASB, bool AVEC>
__device__ __forceinline__ void stage_issue(const StageSpec &sp, StageRegs<U> &R, int base, float *lds, int t,
                                            bool with_scalars) {
  constexpr int es = BF ? 2 : 4;
  constexpr int epc = 16 / es;
  const int cpv = sp.P / epc, cpk = sp.N / epc;
  const int nV = sp.nrec * cpv, nK = sp.nrec * cpk, nA = AVEC ? nK : 0, total = nV + nK + nA + sp.nq * cpk;
  if (with_scalars) {
    const int j = t < sp.nrec ? t : sp.nrec - 1;
    const bool ring = j < sp.n_ring;
    const int ri = ring_slot(sp, j) * sp.hstr + sp.hrow;
    const int ii = sp.ia0 + (j - sp.n_ring) * sp.ias;
    if (!AVEC) {
      const uint8_t *pa = ring ? sp.rA + (size_t)ri * es : (const uint8_t *)sp.iA + (size_t)ii * es;
      R.a = BF ? bf16f(*(const uint16_t *)pa) : *(const float *)pa;
    } else {
      R.a = 0.f;
    }
    if (HASB) {
      const uint8_t *pb = ring ? sp.rB + (size_t)ri * es : (const uint8_t *)sp.iB + (size_t)ii * es;
      R.b = BF ? bf16f(*(const uint16_t *)pb) : *(const float *)pb;
    } else {
      R.b = 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = base + u * kThreads + t;
    R.dst[u] = -1;
    if (c < total) {                       // idle chunks skip their address arithmetic
      const uint8_t *bp;
      int idx, dst;
      if (c < nV) {
        int j;
        if (sp.cpv_lg >= 0)
          j = c >> sp.cpv_lg;
        else
          j = c / cpv;
        const int e = (c - j * cpv) * epc;
        const bool ring = j < sp.n_ring;
        bp = ring ? sp.rV : (const uint8_t *)sp.iV;
        idx = ring ? (ring_slot(sp, j) * sp.hstr + sp.hrow) * sp.P + e : sp.iv0 + (j - sp.n_ring) * sp.ivs + e;
        dst = (int)(sp.V - lds) + j * sp.P + e;
      } else if (c < nV + nK) {
        const int l = c - nV, j = l / cpk, e = (l - j * cpk) * epc;
        const bool ring = j < sp.n_ring;
        bp = ring ? sp.rK : (const uint8_t *)sp.iK;
        idx = ring ? (ring_slot(sp, j) * sp.kstr + sp.krow) * sp.N + e : sp.ik0 + (j - sp.n_ring) * sp.iks + e;
        dst = (int)(sp.K - lds) + j * (sp.N + 4) + e;
      } else if (AVEC && c < nV + nK + nA) {
        const int l = c - nV - nK, j = l / cpk, e = (l - j * cpk) * epc;
        const bool ring = j < sp.n_ring;
        bp = ring ? sp.rA : (const uint8_t *)sp.iA;
        idx = ring ? (ring_slot(sp, j) * sp.hstr + sp.hrow) * sp.N + e : (sp.ia0 + (j - sp.n_ring) * sp.ias) * sp.N + e;
        dst = (int)(sp.A - lds) + j * (sp.N + 4) + e;
      } else {
        const int l = c - nV - nK - nA, r = l / cpk, e = (l - r * cpk) * epc;
        bp = (const uint8_t *)sp.iQ;
        idx = sp.iq0 + r * sp.iqs + e;
        dst = (int)(sp.Q - lds) + r * sp.N + e;
      }
      R.raw[u] = *(const uint4 *)(bp + (size_t)(uint32_t)idx * es);
      R.dst[u] = dst;
    }
  }
}

template <int U, bool BF, bool AVEC>
__device__ __forceinline__ void stage_commit(const StageSpec &sp, const StageRegs<U> &R, float *lds, int t,
                                             bool with_scalars) {
  if (with_scalars && t < sp.nrec) {
    if (!AVEC) sp.A[t] = R.a;
    sp.Bt[t] = R.b;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (R.dst[u] < 0) continue;
    float *d = lds + R.dst[u];
    const uint4 w = R.raw[u];
    if (BF) {
      *(float4 *)d = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
      *(float4 *)(d + 4) = make_float4(__uint_as_float(w.z << 16), __uint_as_float(w.z & 0xFFFF0000u),
                                       __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xFFFF0000u));
    } else {
      *(float4 *)d = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                                 __uint_as_float(w.w));
    }
  }
}

// Element-wise staging for shapes that cannot use 16-byte chunks (e.g. P % 8 != 0 with bf16).
__device__ __forceinline__ void stage_scalar(const StageSpec &sp, int t) {
  for (int j = t; j < sp.nrec; j += kThreads) {
    float al = 0.f, be = 0.f;
    if (j < sp.n_ring) {
      const int i = ring_slot(sp, j) * sp.hstr + sp.hrow;
      if (!sp.avec) al = ld_in(sp.rA, i, sp.bf16);
      if (sp.rB) be = ld_in(sp.rB, i, sp.bf16);
    } else {
      const int i = sp.ia0 + (j - sp.n_ring) * sp.ias;
      if (!sp.avec) al = ld_in(sp.iA, i, sp.bf16);
      if (sp.iB) be = ld_in(sp.iB, i, sp.bf16);
    }
    if (!sp.avec) sp.A[j] = al;
    sp.Bt[j] = be;
  }
  if (sp.avec)
    for (int e = t; e < sp.nrec * sp.N; e += kThreads) {
      const int j = e / sp.N, n = e - j * sp.N;
      sp.A[j * (sp.N + 4) + n] = j < sp.n_ring
                                     ? ld_in(sp.rA, (ring_slot(sp, j) * sp.hstr + sp.hrow) * sp.N + n, sp.bf16)
                                     : ld_in(sp.iA, (sp.ia0 + (j - sp.n_ring) * sp.ias) * sp.N + n, sp.bf16);
    }
  for (int e = t; e < sp.nrec * sp.P; e += kThreads) {
    const int j = e / sp.P, p = e - j * sp.P;
    sp.V[e] = j < sp.n_ring ? ld_in(sp.rV, (ring_slot(sp, j) * sp.hstr + sp.hrow) * sp.P + p, sp.bf16)
                            : ld_in(sp.iV, sp.iv0 + (j - sp.n_ring) * sp.ivs + p, sp.bf16);
  }
  for (int e = t; e < sp.nrec * sp.N; e += kThreads) {
    const int j = e / sp.N, n = e - j * sp.N;
    sp.K[j * (sp.N + 4) + n] = j < sp.n_ring ? ld_in(sp.rK, (ring_slot(sp, j) * sp.kstr + sp.krow) * sp.N + n, sp.bf16)
                                             : ld_in(sp.iK, sp.ik0 + (j - sp.n_ring) * sp.iks + n, sp.bf16);
  }
  for (int e = t; e < sp.nq * sp.N; e += kThreads) {
    const int r = e / sp.N, n = e - r * sp.N;
    sp.Q[e] = ld_in(sp.iQ, sp.iq0 + r * sp.iqs + n, sp.bf16);
  }
}

// Common record source description of a tile.
template <int KIND, int N>
__device__ __forceinline__ StageSpec make_spec(const Args &a, const LdsLayout &L, float *lds, int b, int hh,
                                               int gq, int64_t nk, int n_ring, int n_in, int nq) {
  const Geom &g = a.g;
  StageSpec sp;
  sp.nrec = n_ring + n_in;
  sp.n_ring = n_ring;
  sp.slot0 = ring_mod(nk, g.C);
  sp.C = g.C;
  sp.P = g.P;
  sp.N = N;
  sp.nq = nq;
  sp.bf16 = g.bf16;
  sp.cpv_lg = g.cpv_lg;
  sp.avec = KIND == RSSM_KIND_KDA;
  sp.rA = a.ring + g.off_alpha;
  sp.rB = KIND != RSSM_KIND_MAMBA2 ? a.ring + g.off_beta : nullptr;
  sp.rV = a.ring + g.off_v;
  sp.rK = a.ring + g.off_k;
  sp.hrow = b * g.H + hh;
  sp.krow = b * g.G + gq;
  sp.hstr = g.B * g.H;
  sp.kstr = g.B * g.G;
  sp.iA = a.alpha;
  sp.iB = KIND != RSSM_KIND_MAMBA2 ? a.beta : nullptr;
  sp.iV = a.v;
  sp.iK = a.k;
  sp.iQ = a.q;
  sp.ia0 = sp.ias = sp.iv0 = sp.ivs = sp.ik0 = sp.iks = sp.iq0 = sp.iqs = 0;
  sp.A = lds + L.alpha;
  sp.Bt = lds + L.beta;
  sp.V = lds + L.V;
  sp.K = lds + L.K;
  sp.Q = lds + L.q;
  return sp;
}

// Stage a tile's records with the checkpoint loads in flight: record loads are issued
// first, then `issue_tile()` (the checkpoint or read-copy loads), then the LDS writes.
template <int U, bool BF, bool HASB, bool AVEC, class IssueTile>
__device__ __forceinline__ void stage_vec_with_tile(const StageSpec &sp, float *lds, int t, IssueTile &&issue_tile) {
  StageRegs<U> SR;
  stage_issue<U, BF, HASB, AVEC>(sp, SR, 0, lds, t, true);
  issue_tile();
  stage_commit<U, BF, AVEC>(sp, SR, lds, t, true);
  const int total = stage_chunks(sp, BF ? 8 : 4);
  for (int base = kThreads * U; base < total; base += kThreads * U) {
    stage_issue<U, BF, HASB, AVEC>(sp, SR, base, lds, t, false);
    stage_commit<U, BF, AVEC>(sp, SR, lds, t, false);
  }
}

// STG (kStage*) is chosen by the launcher, so a kernel carries one staging path: with
// several, the tile registers loaded on each path meet in one merge and the fold loop that
// follows worked on a copy of them (twice the tile's registers live at once).
template <int U, int KIND, int STG, class IssueTile>
__device__ __forceinline__ void stage_with_tile(const StageSpec &sp, float *lds, int t, IssueTile &&issue_tile) {
  if constexpr (STG == kStageScalar) {
    issue_tile();
    stage_scalar(sp, t);
  } else {
    stage_vec_with_tile<U, STG == kStageBf16, KIND != RSSM_KIND_MAMBA2, KIND == RSSM_KIND_KDA>(sp, lds, t,
                                                                                           issue_tile);
  }
}

// Append record row j of LDS (and query row qr) to ring slot `slot` (values are exact
// widenings of the inputs, so narrowing back to bf16 reproduces the input bits).  KDA's
// alpha is an N-vector per value head, stored like a key row.
// t: the caller's thread index among the nthr threads that share the record's chunks.
template <int KIND, int N>
__device__ void append_from_lds(const Args &a, const LdsLayout &L, const float *lds, int b, int hh, int gq, int j,
                                int qr, int slot, int t, int nthr = kThreads) {
  const Geom &g = a.g;
  const int P = g.P;
  const int hr = slot * (g.B * g.H) + (b * g.H + hh);
  const bool lead = (hh % g.grp) == 0;
  const int kr = (slot * (g.B * g.G) + (b * g.G + gq)) * N;
  if (g.bf16) {
    uint16_t *rA = (uint16_t *)(a.ring + g.off_alpha);
    uint16_t *rV = (uint16_t *)(a.ring + g.off_v);
    uint16_t *rK = (uint16_t *)(a.ring + g.off_k);
    uint16_t *rQ = (uint16_t *)(a.ring + g.off_q);
    if (t == 0) {
      if (KIND != RSSM_KIND_KDA) rA[hr] = (uint16_t)(__float_as_uint(lds[L.alpha + j]) >> 16);
      if (KIND != RSSM_KIND_MAMBA2)
        ((uint16_t *)(a.ring + g.off_beta))[hr] = (uint16_t)(__float_as_uint(lds[L.beta + j]) >> 16);
    }
    if (a.vec16) {
      // 8 elements per 16-byte store: v (P/8 chunks), KDA alpha (N/8), then k and q (N/8
      // each, key-head leader only)
      const int cv = P / 8, ck = N / 8, ca = KIND == RSSM_KIND_KDA ? ck : 0;
      const int total = cv + ca + (lead ? 2 * ck : 0);
      for (int c = t; c < total; c += nthr) {
        const float *src;
        uint16_t *dst;
        if (c < cv) {
          src = lds + L.V + j * P + 8 * c;
          dst = rV + hr * P + 8 * c;
        } else if (c < cv + ca) {
          src = lds + L.alpha + j * (N + 4) + 8 * (c - cv);
          dst = rA + hr * N + 8 * (c - cv);
        } else if (c < cv + ca + ck) {
          src = lds + L.K + j * (N + 4) + 8 * (c - cv - ca);
          dst = rK + kr + 8 * (c - cv - ca);
        } else {
          src = lds + L.q + qr * N + 8 * (c - cv - ca - ck);
          dst = rQ + kr + 8 * (c - cv - ca - ck);
        }
        const float4 x0 = *(const float4 *)src, x1 = *(const float4 *)(src + 4);
        uint4 w;
        w.x = (__float_as_uint(x0.x) >> 16) | (__float_as_uint(x0.y) & 0xFFFF0000u);
        w.y = (__float_as_uint(x0.z) >> 16) | (__float_as_uint(x0.w) & 0xFFFF0000u);
        w.z = (__float_as_uint(x1.x) >> 16) | (__float_as_uint(x1.y) & 0xFFFF0000u);
        w.w = (__float_as_uint(x1.z) >> 16) | (__float_as_uint(x1.w) & 0xFFFF0000u);
        *(uint4 *)dst = w;
      }
    } else {
      for (int p = t; p < P; p += nthr) rV[hr * P + p] = (uint16_t)(__float_as_uint(lds[L.V + j * P + p]) >> 16);
      if (KIND == RSSM_KIND_KDA)
        for (int n = t; n < N; n += nthr)
          rA[hr * N + n] = (uint16_t)(__float_as_uint(lds[L.alpha + j * (N + 4) + n]) >> 16);
      if (lead)
        for (int n = t; n < N; n += nthr) {
          rK[kr + n] = (uint16_t)(__float_as_uint(lds[L.K + j * (N + 4) + n]) >> 16);
          rQ[kr + n] = (uint16_t)(__float_as_uint(lds[L.q + qr * N + n]) >> 16);
        }
    }
  } else {
    float *rA = (float *)(a.ring + g.off_alpha);
    float *rV = (float *)(a.ring + g.off_v);
    float *rK = (float *)(a.ring + g.off_k);
    float *rQ = (float *)(a.ring + g.off_q);
    if (t == 0) {
      if (KIND != RSSM_KIND_KDA) rA[hr] = lds[L.alpha + j];
      if (KIND != RSSM_KIND_MAMBA2) ((float *)(a.ring + g.off_beta))[hr] = lds[L.beta + j];
    }
    for (int p = t; p < P; p += nthr) rV[hr * P + p] = lds[L.V + j * P + p];
    if (KIND == RSSM_KIND_KDA)
      for (int n = t; n < N; n += nthr) rA[hr * N + n] = lds[L.alpha + j * (N + 4) + n];
    if (lead)
      for (int n = t; n < N; n += nthr) {
        rK[kr + n] = lds[L.K + j * (N + 4) + n];
        rQ[kr + n] = lds[L.q + qr * N + n];
      }
  }
}

// ---------------------------------------------------------------- coefficient phases
// Record j is on a query's path when j < hb (committed records) or draft j - hb is an
// ancestor-or-self of the query (bit j - hb of anc).  The defaults put every record on the
// path.  Off-path records act as neutral records (alpha = 1, beta = 0, no coefficient),
// which leave the state unchanged.
__device__ __forceinline__ bool on_path(int j, int hb, uint32_t anc) {
  return j < hb || ((anc >> (j - hb)) & 1u);
}

// Decays of one query over the on-path records among 0..last (one wave, all lanes active):
// dec[j] = prod of alpha_m over on-path m with j < m <= last for on-path j <= last, else 0;
// *gam = prod of alpha_m over on-path m <= last.
__device__ __forceinline__ void wave_decays(const float *alpha, int last, float *dec, float *gam, int cap,
                                            int lane, int hb = 1 << 30, uint32_t anc = 0) {
  const bool on = lane <= last && on_path(lane, hb, anc);
  float x = on ? alpha[lane] : 1.f;
  x = wave_suffix_product(x, lane);
  const float nxt = __shfl_down(x, 1);
  if (lane < cap) dec[lane] = !on ? 0.f : (lane < last ? nxt : 1.f);
  if (lane == 0) *gam = x;
}

// Dot product of two LDS rows of N floats by the 16 lanes of a group: lane l16 reads the
// 16-byte pieces at 4 * l16 + 64 * i.  Every lane of the group returns the sum.
template <int N>
__device__ __forceinline__ float group_dot(const float *x, const float *y, int l16) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < (N + 63) / 64; ++i) {
    const int n = 4 * l16 + 64 * i;
    if (n < N) {
      const float4 a = *(const float4 *)(x + n), b = *(const float4 *)(y + n);
      acc = fmaf(a.x, b.x, acc);
      acc = fmaf(a.y, b.y, acc);
      acc = fmaf(a.z, b.z, acc);
      acc = fmaf(a.w, b.w, acc);
    }
  }
  return sum16(acc);
}

// q = d / n for 0 <= d < 2^10, 1 <= n <= 64: the float estimate (d + 1/2) / n is at least
// 1/(2n) from an integer and within 2^-12 of its exact value, so its floor is exact.
__device__ __forceinline__ int small_div(int d, float inv_n) { return (int)(((float)d + 0.5f) * inv_n); }

// Dot products k_j . q_tau for j < nrec, tau < T, by groups of 16 lanes -> coef[tau * cap + j].
// With one query (decode) each lane keeps its slice of q in registers for all the records it
// takes, so q is read from LDS once per lane instead of once per record.
template <int N>
__device__ void kq_dots(float *lds, const LdsLayout &L, int cap, int nrec, int T, int t) {
  const int g16 = t >> 4, l16 = t & 15;
  if (T == 1) {
    constexpr int NI = (N + 63) / 64;
    float4 qv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = 4 * l16 + 64 * i;
      qv[i] = n < N ? *(const float4 *)(lds + L.q + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int j = g16; j < nrec; j += kThreads / 16) {
      const float *kr = lds + L.K + j * (N + 4);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = 4 * l16 + 64 * i;
        if (n < N) acc = dot4(*(const float4 *)(kr + n), qv[i], acc);
      }
      acc = sum16(acc);
      if (l16 == 0) lds[L.coef + j] = acc;
    }
    return;
  }
  const float inv = 1.0f / (float)nrec;
  for (int d = g16; d < T * nrec; d += kThreads / 16) {
    const int tau = small_div(d, inv), j = d - tau * nrec;
    const float acc = group_dot<N>(lds + L.K + j * (N + 4), lds + L.q + tau * N, l16);
    if (l16 == 0) lds[L.coef + tau * cap + j] = acc;
  }
}

// Sum over the 64 lanes of a wave (all lanes active); every lane gets the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Delta-rule query transform for one query over records 0..n-1 (one wave, all lanes
// active), the output-only form of Gated DeltaNet and KDA.  With the gate a_i (a scalar for
// Gated DeltaNet, one per key channel for KDA), S_i r = S_{i-1} Diag(a_i) (r - b_i (k_i . r)
// k_i) + b_i (k_i . r) v_i, so from the newest record down: c_i = b_i (k_i . r),
// r <- a_i o (r - c_i k_i), and the output is S_ckpt r + sum_i c_i v_i.  This is the
// triangular system of the delta rule's pseudo-values solved for one query, evaluated in
// key space: one wave-wide dot product and one gated AXPY per record.  Writes c_i to the
// coef row (0 for records off the query's path, which act as neutral records), the final r
// to the r row, and G = 1 (the decays are carried by r).  Lane l holds elements l + 64 e.
template <int KIND, int N>
__device__ void delta_sweep_wave(float *lds, const LdsLayout &L, int cap, int n, int tau, int lane,
                                 int hb = 1 << 30, uint32_t anc = 0) {
  constexpr int E = (N + 63) / 64;
  const float *beta = lds + L.beta;
  float *coef = lds + L.coef + tau * cap;
  float r[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = lane + 64 * e;
    r[e] = idx < N ? lds[L.q + tau * N + idx] : 0.f;
  }
  for (int i = n - 1; i >= 0; --i) {
    if (!on_path(i, hb, anc)) {                      // uniform across the wave
      if (lane == 0) coef[i] = 0.f;
      continue;
    }
    const float *k = lds + L.K + i * (N + 4);
    const float *al = lds + L.alpha + (KIND == RSSM_KIND_KDA ? i * (N + 4) : i);
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = lane + 64 * e;
      if (idx < N) p = fmaf(k[idx], r[e], p);
    }
    const float c = beta[i] * wave_sum(p);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = lane + 64 * e;
      if (idx < N) r[e] = (KIND == RSSM_KIND_KDA ? al[idx] : al[0]) * fmaf(-c, k[idx], r[e]);
    }
    if (lane == 0) coef[i] = c;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = lane + 64 * e;
    if (idx < N) lds[L.r + tau * N + idx] = r[e];
  }
  if (lane == 0) lds[L.gam + tau] = 1.f;
}

// ---------------------------------------------------------------- folds
// Mamba-2 fold: S <- G S + sum_j d_j v_j k_j^T (decays in L.dec, G in L.gam).
template <int N, int RGW>
__device__ __forceinline__ void fold_m2(Frag<N, RGW> &F, const float *lds, const LdsLayout &L, int nrec, int P, int wave,
                        int lane) {
  const int c = frag_col(lane);
  const float G = lds[L.gam];
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      F.s[i][f].x *= G;
      F.s[i][f].y *= G;
      F.s[i][f].z *= G;
      F.s[i][f].w *= G;
    }
  for (int j = 0; j < nrec; ++j) {
    const float dj = lds[L.dec + j];
    const float *kr = lds + L.K + j * (N + 4) + c;
    float vr[RGW];
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const int row = frag_row(wave, lane, i);
      vr[i] = (row < P) ? lds[L.V + j * P + row] * dj : 0.f;
    }
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      const float4 kf = *(const float4 *)(kr + 32 * f);
#pragma unroll
      for (int i = 0; i < RGW; ++i) {
        F.s[i][f].x = fmaf(vr[i], kf.x, F.s[i][f].x);
        F.s[i][f].y = fmaf(vr[i], kf.y, F.s[i][f].y);
        F.s[i][f].z = fmaf(vr[i], kf.z, F.s[i][f].z);
        F.s[i][f].w = fmaf(vr[i], kf.w, F.s[i][f].w);
      }
    }
  }
}

// Gated DeltaNet fold, one delta-rule update per record in registers:
// S <- a S ; u = b (v - S k) ; S <- S + u k^T.
// The tile is held as S = s F with one scalar s, the product of the decays since the last
// rescale, so a record costs one FMA per element for S k and one for the rank-1 update:
//   s' = s a ; w = s' (F k) ; u = b (v - w) ; F <- F + (u / s') k^T ; s <- s'.
// Before s' would leave [2^-40, 2^40] (a zero decay included) F is rescaled to S a, and it
// is rescaled once at the end.
constexpr float kFoldScaleMin = 0x1p-40f, kFoldScaleMax = 0x1p40f;

template <int N, int RGW>
__device__ __forceinline__ void frag_scale(Frag<N, RGW> &F, float x) {
#pragma unroll
  for (int i = 0; i < RGW; ++i)
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      F.s[i][f].x *= x;
      F.s[i][f].y *= x;
      F.s[i][f].z *= x;
      F.s[i][f].w *= x;
    }
}

template <int N, int RGW>
__device__ __forceinline__ void fold_gdn(Frag<N, RGW> &F, const float *lds, const LdsLayout &L, int nrec, int P, int wave,
                         int lane) {
  const int c = frag_col(lane);
  float s = 1.f;
  for (int j = 0; j < nrec; ++j) {
    const float al = lds[L.alpha + j], be = lds[L.beta + j];
    float sn = s * al;
    if (!(sn >= kFoldScaleMin && sn <= kFoldScaleMax)) {   // the same for every lane (LDS values)
      frag_scale(F, sn);
      sn = 1.f;
    }
    const float *kr = lds + L.K + j * (N + 4) + c;
    float w[RGW];
#pragma unroll
    for (int i = 0; i < RGW; ++i) w[i] = 0.f;
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      const float4 kf = *(const float4 *)(kr + 32 * f);
#pragma unroll
      for (int i = 0; i < RGW; ++i) w[i] = dot4(F.s[i][f], kf, w[i]);
    }
    const float inv = 1.f / sn;
    float u[RGW];
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const float wi = oct_sum(w[i]);
      const int row = frag_row(wave, lane, i);
      const float vr = (row < P) ? lds[L.V + j * P + row] : 0.f;
      u[i] = be * (vr - sn * wi) * inv;
    }
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      const float4 kf = *(const float4 *)(kr + 32 * f);
#pragma unroll
      for (int i = 0; i < RGW; ++i) {
        F.s[i][f].x = fmaf(u[i], kf.x, F.s[i][f].x);
        F.s[i][f].y = fmaf(u[i], kf.y, F.s[i][f].y);
        F.s[i][f].z = fmaf(u[i], kf.z, F.s[i][f].z);
        F.s[i][f].w = fmaf(u[i], kf.w, F.s[i][f].w);
      }
    }
    s = sn;
  }
  if (s != 1.f) frag_scale(F, s);
}

// KDA fold, one per-channel gated delta-rule update per record in registers:
// S <- S Diag(a) ; u = b (v - S k) ; S <- S + u k^T (a: the record's alpha row in LDS).
// The gate is applied in place in the first pass, so only the key row stays live into the
// rank-1 pass (the gate row is dead after it).
template <int N, int RGW>
__device__ __forceinline__ void fold_kda(Frag<N, RGW> &F, const float *lds, const LdsLayout &L, int nrec, int P,
                                         int wave, int lane) {
  const int c = frag_col(lane);
  for (int j = 0; j < nrec; ++j) {
    const float be = lds[L.beta + j];
    const float *kr = lds + L.K + j * (N + 4) + c;
    const float *ar = lds + L.alpha + j * (N + 4) + c;
    float w[RGW];
#pragma unroll
    for (int i = 0; i < RGW; ++i) w[i] = 0.f;
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      const float4 kf = *(const float4 *)(kr + 32 * f), af = *(const float4 *)(ar + 32 * f);
#pragma unroll
      for (int i = 0; i < RGW; ++i) {
        F.s[i][f].x *= af.x;
        F.s[i][f].y *= af.y;
        F.s[i][f].z *= af.z;
        F.s[i][f].w *= af.w;
        w[i] = dot4(F.s[i][f], kf, w[i]);
      }
    }
    float u[RGW];
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const float wi = oct_sum(w[i]);
      const int row = frag_row(wave, lane, i);
      const float vr = (row < P) ? lds[L.V + j * P + row] : 0.f;
      u[i] = be * (vr - wi);
    }
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      const float4 kf = *(const float4 *)(kr + 32 * f);
#pragma unroll
      for (int i = 0; i < RGW; ++i) {
        F.s[i][f].x = fmaf(u[i], kf.x, F.s[i][f].x);
        F.s[i][f].y = fmaf(u[i], kf.y, F.s[i][f].y);
        F.s[i][f].z = fmaf(u[i], kf.z, F.s[i][f].z);
        F.s[i][f].w = fmaf(u[i], kf.w, F.s[i][f].w);
      }
    }
  }
}

// Delta-rule fold of either gated kind.
template <int KIND, int N, int RGW>
__device__ __forceinline__ void fold_delta(Frag<N, RGW> &F, const float *lds, const LdsLayout &L, int nrec, int P,
                                           int wave, int lane) {
  if constexpr (KIND == RSSM_KIND_KDA)
    fold_kda(F, lds, L, nrec, P, wave, lane);
  else
    fold_gdn(F, lds, L, nrec, P, wave, lane);
}

// Output rows: y[row] = G * (S x)[row] + sum_{j < n} w_j v_j[row], where w_j = dec[j] * coef[j]
// (Mamba-2: decay times k_j . q) or w_j = coef[j] (GDN: already d_j b_j c_j; dec == null).
// The 8 lanes of a row take records j = l%8 mod 8.
template <int RGW>
__device__ __forceinline__ void write_rows(const float (&part)[RGW], float G, const float *lds, const LdsLayout &L,
                                           const float *dec, const float *coef, int n, int P,
                                           float *__restrict__ out, int wave, int lane) {
  const int c8 = lane & 7;
#pragma unroll
  for (int i = 0; i < RGW; ++i) {
    const int row = frag_row(wave, lane, i);
    float buf = 0.f;
    if (row < P)
      for (int j = c8; j < n; j += 8) {
        const float w = dec ? dec[j] * coef[j] : coef[j];
        buf = fmaf(w, lds[L.V + j * P + row], buf);
      }
    const float y = oct_sum(fmaf(G, part[i], buf));
    if (c8 == 0 && row < P) out[row] = y;
  }
}

// ================================================================ kernels

// U: staging chunks per thread per round (2 covers a 17-record Mamba-2 window at 64 x 128
// in bf16 in one round).  RCF: the read-copy format (RSSM_READ_*); with a copy the kernel
// serves non-fold steps from it.
// Mamba-2 read-copy instances with rows of at least 128 columns and at most 32 tile registers
// per lane run at 8 waves per SIMD: their non-fold steps move 4-9 KB per tile and are bound
// by the latency of the cursor -> records + copy chain, so more workgroups in flight pay
// off, and these instances fit 8 waves without spills (the scalar registers otherwise cap
// them at 7).  The delta-rule folds and narrower rows would spill, so they keep the default.
template <int KIND, int RCF, int N, int RGW>
constexpr int decode_min_waves() {
  return (KIND == RSSM_KIND_MAMBA2 && RCF != RSSM_READ_NONE && N >= 128 && RGW * N <= 256) ? 8 : 1;
}

// Record sources of a decode step: the hb window records from ring slot nk mod C on, then
// the step's input record; the query is the step's input query.
template <int KIND, int N>
__device__ __forceinline__ StageSpec decode_spec(const Args &a, const LdsLayout &L, float *lds, int b, int hh, int gq,
                                                 int64_t nk, int hb) {
  const Geom &g = a.g;
  StageSpec sp = make_spec<KIND, N>(a, L, lds, b, hh, gq, nk, hb, 1, 1);
  sp.ia0 = b * g.H + hh;
  sp.iv0 = (b * g.H + hh) * g.P;
  sp.ik0 = (b * g.G + gq) * N;
  sp.iq0 = sp.ik0;
  return sp;
}

// ---------------------------------------------------------------- tail appends
// Small HBM writes cost far more while a launch's read stream runs at full rate than in its
// last workgroups, when the stream drains.  With H a multiple of 16, the Mamba-2 and KDA
// decode kernels on the fp32 tile therefore leave the ring appends of each group of GS value
// heads of a sequence to the workgroup of the group's last head, and dispatch those
// workgroups after all others.  GS is 16, or 32 for Mamba-2 where H allows it (Mamba-2 with
// 642-byte records per head ran about 1% faster with 32-head groups; KDA, with 1026-byte
// records, ran no faster staggered and slower in lockstep).  That workgroup knows the slot
// and the fold decision of every head of its group from its own cursor replica, since all
// replicas of a sequence are equal (a head whose replica disagrees, which only a contract
// violation can cause, is left out).  The appender workgroups carry more work than the
// others, so the order only pays where the moved writes are large against the end of the
// grid they lengthen: GDN (smaller records, long delta-rule folds) and the read-copy decode
// (short non-fold tiles, folds several times longer) keep the appends in each tile's
// workgroup.

// Heads per group, 0 for appends in each tile's workgroup.
template <int KIND, int RCF>
__device__ __forceinline__ int tail_group(const Geom &g) {
  if (KIND == RSSM_KIND_GDN || RCF != RSSM_READ_NONE) return 0;
  if (KIND == RSSM_KIND_MAMBA2 && (g.H % 32) == 0) return 32;
  return (g.H % 16) == 0 ? 16 : 0;
}

__device__ __forceinline__ uint64_t tail_full(int gs) { return gs >= 64 ? ~0ull : (1ull << gs) - 1; }

// Block index -> work item of a grid of `items` whose last 1/gs are the appenders (the
// groups' last heads): the first part of the grid takes the items i % gs != gs - 1 in the
// XCD-aware order, the rest the items i % gs == gs - 1.
__device__ __forceinline__ int tail_item_of_block(int items, int gs, bool &appender) {
  const int na = items / gs, nm = items - na;
  const int bid = blockIdx.x;
  appender = bid >= nm;
  if (!appender) {
    const int i = (nm & 7) == 0 ? (bid & 7) * (nm >> 3) + (bid >> 3) : bid;
    return (i / (gs - 1)) * gs + i % (gs - 1);
  }
  const int j = bid - nm;
  const int ai = (na & 7) == 0 ? (j & 7) * (na >> 3) + (j >> 3) : j;
  return ai * gs + (gs - 1);
}

// Copy `bytes` bytes (a multiple of 2) with threads t = 0 .. nthr-1, in the widest pieces
// the alignment of both ends allows.
__device__ __forceinline__ void group_copy(uint8_t *__restrict__ dst, const uint8_t *__restrict__ src, int64_t bytes,
                                           int t, int nthr) {
  const uint64_t al = (uint64_t)dst | (uint64_t)src | (uint64_t)bytes;
  if ((al & 15) == 0) {
    for (int64_t c = t; c < bytes / 16; c += nthr) ((uint4 *)dst)[c] = ((const uint4 *)src)[c];
  } else if ((al & 3) == 0) {
    for (int64_t c = t; c < bytes / 4; c += nthr) ((uint32_t *)dst)[c] = ((const uint32_t *)src)[c];
  } else {
    for (int64_t c = t; c < bytes / 2; c += nthr) ((uint16_t *)dst)[c] = ((const uint16_t *)src)[c];
  }
}

// Bit i set: head h0 + i (i < gs <= 64) of sequence b has the appender's counters before
// this step (nc, nk) or after its own non-fold step (nc + 1, nk).  Its own workgroup may be
// writing the replica while it is read here, so either value is accepted.  Lane i of the
// calling wave loads head h0 + i.
__device__ __forceinline__ uint64_t tail_group_mask(const Args &a, int b, int h0, int gs, int64_t nc, int64_t nk,
                                                    int lane) {
  bool ok = false;
  if (lane < gs) {
    const int tile = b * a.g.H + h0 + lane;
    const int64_t c = __hip_atomic_load(a.n_committed + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t k = __hip_atomic_load(a.n_ckpt + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = k == nk && (c == nc || c == nc + 1);
  }
  return (uint64_t)__ballot(ok) & tail_full(gs);
}

// Append the step inputs of value heads h0 .. h0+gs-1 of sequence b whose bit is set in
// `mask` (and the key heads they lead) to ring slot `slot`: byte copies, the ring holding the
// input dtype.  With every bit set the group's rows are copied as contiguous blocks.
template <int KIND, int N>
__device__ void tail_append_group(const Args &a, int b, int h0, int gs, int slot, uint64_t mask, int t, int nthr) {
  const Geom &g = a.g;
  const int64_t es = g.bf16 ? 2 : 4, P = g.P;
  const int64_t na = KIND == RSSM_KIND_KDA ? N : 1;                 // alpha elements per head
  const int64_t row0 = (int64_t)b * g.H + h0;                       // input row of head h0
  const int64_t hr = (int64_t)slot * g.B * g.H + row0;              // ring row of head h0
  const int64_t kin0 = (int64_t)b * g.G * N;                        // input key row 0 of sequence b
  const int64_t kbase = (int64_t)slot * g.B * g.G * N + kin0;       // its ring key row 0
  const uint8_t *iv = (const uint8_t *)a.v, *ia = (const uint8_t *)a.alpha, *ib = (const uint8_t *)a.beta;
  const uint8_t *ik = (const uint8_t *)a.k, *iq = (const uint8_t *)a.q;
  if (mask == tail_full(gs)) {
    const int ga = (h0 + g.grp - 1) / g.grp;
    const int gl = (h0 + gs + g.grp - 1) / g.grp;
    const int gz = gl < g.G ? gl : g.G;                             // key heads [ga, gz) led here
    group_copy(a.ring + g.off_v + hr * P * es, iv + row0 * P * es, gs * P * es, t, nthr);
    group_copy(a.ring + g.off_alpha + hr * na * es, ia + row0 * na * es, gs * na * es, t, nthr);
    if (KIND != RSSM_KIND_MAMBA2)
      group_copy(a.ring + g.off_beta + hr * es, ib + row0 * es, gs * es, t, nthr);
    if (gz > ga) {
      const int64_t ko = (int64_t)ga * N;
      group_copy(a.ring + g.off_k + (kbase + ko) * es, ik + (kin0 + ko) * es, (gz - ga) * N * es, t, nthr);
      group_copy(a.ring + g.off_q + (kbase + ko) * es, iq + (kin0 + ko) * es, (gz - ga) * N * es, t, nthr);
    }
    return;
  }
  for (int i = 0; i < gs; ++i) {
    if (!((mask >> i) & 1)) continue;
    const int h = h0 + i;
    group_copy(a.ring + g.off_v + (hr + i) * P * es, iv + (row0 + i) * P * es, P * es, t, nthr);
    group_copy(a.ring + g.off_alpha + (hr + i) * na * es, ia + (row0 + i) * na * es, na * es, t, nthr);
    if (KIND != RSSM_KIND_MAMBA2)
      group_copy(a.ring + g.off_beta + (hr + i) * es, ib + (row0 + i) * es, es, t, nthr);
    if (h % g.grp == 0) {
      const int64_t ko = (int64_t)(h / g.grp) * N;
      group_copy(a.ring + g.off_k + (kbase + ko) * es, ik + (kin0 + ko) * es, N * es, t, nthr);
      group_copy(a.ring + g.off_q + (kbase + ko) * es, iq + (kin0 + ko) * es, N * es, t, nthr);
    }
  }
}

// Fold step of one tile by the whole workgroup: the hb window records and the step's record
// are folded into the checkpoint, which is written back with its read copy (format RCF), and
// the output is read from the new checkpoint.  The caller advances the cursors.
template <int KIND, int N, int RGW, int RCF, int STG>
__device__ __forceinline__ void decode_fold_tile(const Args &a, float *lds, int tile, int64_t nk, int hb) {
  constexpr int U = (KIND != RSSM_KIND_MAMBA2 || RGW > 2) ? 4 : 2;
  const Geom &g = a.g;
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int nrec = hb + 1, P = g.P, cap = g.C + 1;
  const LdsLayout L = lds_layout(KIND, cap, 1, P, N);
  float *tileS = a.s + (int64_t)tile * P * N;
  const StageSpec sp = decode_spec<KIND, N>(a, L, lds, b, hh, gq, nk, hb);
  float *yout = a.out + (b * g.H + hh) * P;
  Frag<N, RGW> F;
  stage_with_tile<U, KIND, STG>(sp, lds, t, [&]() { frag_load<N, RGW, true>(F, tileS, P, wave, lane); });
  __syncthreads();
  if (KIND == RSSM_KIND_MAMBA2) {
    if (wave == 0) wave_decays(lds + L.alpha, nrec - 1, lds + L.dec, lds + L.gam, cap, lane);
    __syncthreads();
    fold_m2(F, lds, L, nrec, P, wave, lane);
  } else {
    fold_delta<KIND>(F, lds, L, nrec, P, wave, lane);
  }
  frag_store(F, tileS, P, wave, lane);
  frag_store_read_copy<RCF>(F, a.s_read, a.s_read_scale, tile, P, wave, lane);
  float part[RGW];
  frag_dot(F, lds + L.q, lane, part);
  write_row_sums<RGW>(part, P, yout, wave, lane);
}

template <int KIND, int N, int RGW, int RCF, int STG>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(decode_min_waves<KIND, RCF, N, RGW>(), 8))) void k_decode(Args a) {
  constexpr int U = (KIND != RSSM_KIND_MAMBA2 || RGW > 2) ? 4 : 2;
  constexpr bool RC = RCF != RSSM_READ_NONE;
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int gs = tail_group<KIND, RCF>(g);
  const bool tail = gs > 0;
  bool appender = false;
  const int tile = tail ? tail_item_of_block(g.B * g.H, gs, appender) : tile_of_block(g.B * g.H);
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

  // The fold step and the output-only step stage their records separately, so the tile
  // registers of one path are never live in the other (one shared allocation would have to
  // hold both).  The tile is streamed with nontemporal loads (read once per step; on a fold
  // step it is written back from registers).
  float *yout = a.out + (b * g.H + hh) * P;
  if (flush) {
    decode_fold_tile<KIND, N, RGW, RCF, STG>(a, lds, tile, nk, hb);
  } else {
    const StageSpec sp = decode_spec<KIND, N>(a, L, lds, b, hh, gq, nk, hb);
    Frag<N, RGW> F;
    RCopy<N, RGW> RCR;
    stage_with_tile<U, KIND, STG>(sp, lds, t, [&]() {
      if (RC)
        readcopy_load(RCR, RCF, a.s_read, a.s_read_scale, tile, P, wave, lane);
      else
        frag_load<N, RGW, true>(F, tileS, P, wave, lane);
    });
    __syncthreads();
    const float *x;
    const float *dec = nullptr;
    if (KIND == RSSM_KIND_MAMBA2) {
      if (wave == 0) wave_decays(lds + L.alpha, nrec - 1, lds + L.dec, lds + L.gam, cap, lane);
      kq_dots<N>(lds, L, cap, nrec, 1, t);
      __syncthreads();
      x = lds + L.q;
      dec = lds + L.dec;
    } else {
      if (wave == 0) delta_sweep_wave<KIND, N>(lds, L, cap, nrec, 0, lane);
      __syncthreads();
      x = lds + L.r;
    }
    float part[RGW];
    if (RC)
      readcopy_dot(RCR, RCF, x, lane, part);
    else
      frag_dot(F, x, lane, part);
    write_rows<RGW>(part, lds[L.gam], lds, L, dec, lds + L.coef, nrec, P, yout, wave, lane);
    if (!tail) append_from_lds<KIND, N>(a, L, lds, b, hh, gq, nrec - 1, 0, ring_add(sp.slot0, hb, g.C), t);
  }
  if (appender && !flush) {
    const int h0 = hh - (gs - 1);
    __syncthreads();                                  // every LDS read of the step is done
    if (wave == 0) {
      const uint64_t m = tail_group_mask(a, b, h0, gs, nc, nk, lane);
      if (lane == 0) ((uint64_t *)lds)[0] = m;
    }
    __syncthreads();
    tail_append_group<KIND, N>(a, b, h0, gs, ring_mod(nc, g.C), ((const uint64_t *)lds)[0], t, kThreads);
  }
  if (t == 0) {
    a.n_committed[tile] = nc + 1;
    if (flush) a.n_ckpt[tile] = nc + 1;
  }
}

// ================================================================ read-copy decode, one wave per tile
// A non-fold Mamba-2 step served from the read copy moves a few KB per tile, so with a
// 4-wave workgroup per tile the per-tile set-up (cursor, record addresses, staging,
// barriers) costs more instruction issue than the arithmetic and the kernel is bound by
// VALU issue, not HBM.  Here one wave takes one tile's non-fold step on its own, with no
// workgroup barrier and no record staging: each lane loads the record pieces it works on
// straight into registers.  A workgroup takes 4 tiles; those whose window is full are then
// folded one after another by the whole workgroup with the fold of k_decode, so checkpoints,
// read copies and fold-step outputs are bit-identical to it.

// LDS of one wave's non-fold step (floats): the query (N), decays and k.q products of up to
// 16 records, the per-record-group value sums (at most 64 lanes x 8 values) and the row
// sums of the read-copy product (at most 64 rows).
template <int N>
struct WaveLds {
  static constexpr int q = 0, dec = N, coef = N + 16, vt = N + 32, rc = N + 32 + 512, total = N + 32 + 512 + 64;
};

// LDS written by some lanes of a wave and read by other lanes of the same wave: a wave's LDS
// operations complete in order, so only the compiler has to keep the reads after the writes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Floats of LDS of k_decode_rc: the fold step's layout or 4 waves' non-fold areas, whichever
// is larger, then the 4 fold flags.
__host__ __device__ inline int decode_rc_flag_offset(int cap, int P, int N, int wave_total) {
  const int f = lds_layout(RSSM_KIND_MAMBA2, cap, 1, P, N).total;
  const int w = kWaves * wave_total;
  return up4(f > w ? f : w);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <bool BF>
__device__ __forceinline__ void widen(const uint4 w, float (&x)[BF ? 8 : 4]) {
  if constexpr (BF) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(u[e] << 16);
      x[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  } else {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
}

// Non-fold decode step of one Mamba-2 tile by one wave (window of hb <= 14 records, so the
// step sees nrec = hb + 1 <= 15 records; P <= 64; RG = 8-row groups covering P; RCR: the
// tile's read copy, loaded in the row-octet layout with all row groups in this wave):
//   y = G S_read q + sum_j dec_j (k_j . q) v_j,
// dec_j = prod of alpha_m over j < m <= hb, G = prod of alpha_m over m <= hb (the output-only
// replay of the window; the same quantities as the 4-wave step).  Lane layouts:
// * decays: lane j holds record j;
// * k . q: R lanes per record (R = min(16, key chunks)), each with CPL 16-byte chunks;
// * sum_j w_j v_j: VC = P / (elements per chunk) lanes per record, each one chunk;
// * read copy: the row-octet layout with all row groups in one wave.
// Records past the window are clamped to the step's input record (their loads stay in
// bounds) and contribute nothing.  The step's record is appended to ring slot
// (nk + hb) mod C from registers (the input bits).
template <int N, int RG, int RCF, bool BF>
__device__ __forceinline__ void m2_nonfold_wave(const Args &a, int tile, float *wl, int b, int hh,
                                                int gq, int64_t nk, int hb, int lane) {
  const Geom &g = a.g;
  constexpr int es = BF ? 2 : 4, epc = 16 / es;
  constexpr int KC = N / epc, R = KC < 16 ? KC : 16, CPL = KC / R, RPP = 64 / R;
  constexpr int KP = (15 + RPP - 1) / RPP;   // key passes for up to 15 records
  constexpr int VP = BF ? 2 : 4;             // value passes for up to 15 records at P <= 64
  using W = WaveLds<N>;
  static_assert(R == 8 || R == 16, "key rows of 8 or 16 chunks per record group");
  const int P = g.P, C = g.C, nrec = hb + 1;
  const int slot0 = ring_mod(nk, C);
  const int hrow = b * g.H + hh, krow = b * g.G + gq;
  // Row addresses: slot s of the ring holds this head's rows at base + s * stride (strides
  // are below 4 GB: a ring region holds fewer than 2^31 elements over C >= 2 slots).
  const uint32_t ast = (uint32_t)(g.B * g.H) * es, vst = (uint32_t)(g.B * g.H) * P * es,
                 kst = (uint32_t)(g.B * g.G) * N * es;
  const uint8_t *ab = a.ring + g.off_alpha + (size_t)hrow * es;
  const uint8_t *vb = a.ring + g.off_v + (size_t)hrow * P * es;
  const uint8_t *kb = a.ring + g.off_k + (size_t)krow * N * es;
  const uint8_t *qb = a.ring + g.off_q + (size_t)krow * N * es;
  const uint8_t *ain = (const uint8_t *)a.alpha + (size_t)hrow * es;
  const uint8_t *vin = (const uint8_t *)a.v + (size_t)hrow * P * es;
  const uint8_t *kin = (const uint8_t *)a.k + (size_t)krow * N * es;
  const uint8_t *qin = (const uint8_t *)a.q + (size_t)krow * N * es;
  auto slot_of = [&](int j) {
    const int s = slot0 + j;
    return (uint32_t)(s >= C ? s - C : s);
  };

  // ---- loads: alpha, query, key rows, value rows.
  // Records past the window are clamped to the step's input record.
  uint32_t araw;
  {
    const int j = lane < hb ? lane : hb;
    const uint8_t *p = j < hb ? ab + (size_t)slot_of(j) * ast : ain;
    araw = BF ? (uint32_t) * (const uint16_t *)p : *(const uint32_t *)p;
  }
  const int kr = lane / R, kc = lane % R;
  uint4 qraw[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) qraw[i] = *(const uint4 *)(qin + (kc + R * i) * 16);
  uint4 kraw[KP][CPL];
#pragma unroll
  for (int m = 0; m < KP; ++m) {
    int j = kr + RPP * m;
    j = j < hb ? j : hb;
    const uint8_t *row = j < hb ? kb + (size_t)slot_of(j) * kst : kin;
#pragma unroll
    for (int i = 0; i < CPL; ++i) kraw[m][i] = *(const uint4 *)(row + (kc + R * i) * 16);
  }
  // VC lanes per value row; a power of two (the common case) takes shifts, not divisions
  const int lg = g.cpv_lg;
  const int VC = lg >= 0 ? 1 << lg : P / epc, VR = lg >= 0 ? 64 >> lg : 64 / VC;
  const int vr = lg >= 0 ? lane >> lg : lane / VC, vc = lane - vr * VC;
  uint4 vraw[VP];
#pragma unroll
  for (int m = 0; m < VP; ++m) {
    int j = vr + VR * m;
    j = j < hb ? j : hb;
    const uint8_t *row = j < hb ? vb + (size_t)slot_of(j) * vst : vin;
    vraw[m] = *(const uint4 *)(row + vc * 16);
  }

  // ---- decays: lane j < nrec <= 15 holds record j; lanes past the window hold 1, so the
  // 16-lane suffix product equals the one of the 4-wave step bit for bit
  const float al = BF ? __uint_as_float(araw << 16) : __uint_as_float(araw);
  const float x = row_suffix_product(lane < nrec ? al : 1.f);
  const float G = lane_value(x, 0);
  const float nxt = dpp_or_one<0x101>(x);
  if (lane < nrec) wl[W::dec + lane] = lane < hb ? nxt : 1.f;

  // ---- query: fp32 copy in LDS for the read-copy product, and k_j . q
  float qf[CPL][epc];
#pragma unroll
  for (int i = 0; i < CPL; ++i) widen<BF>(qraw[i], qf[i]);
  if (kr == 0) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int e = 0; e < epc; e += 4)
        *(float4 *)(wl + W::q + (kc + R * i) * epc + e) = make_float4(qf[i][e], qf[i][e + 1], qf[i][e + 2], qf[i][e + 3]);
  }
#pragma unroll
  for (int m = 0; m < KP; ++m) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      if constexpr (BF) {
        // bf16 pairs straight from the loaded bits: each product of two bf16 values is exact
        // in fp32, so only the accumulation rounds (as in the FMA form, in another order)
        const uint32_t kw[4] = {kraw[m][i].x, kraw[m][i].y, kraw[m][i].z, kraw[m][i].w};
        const uint32_t qw[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw[e]), __builtin_bit_cast(bf16x2, qw[e]),
                                                acc, false);
      } else {
        float kf[epc];
        widen<BF>(kraw[m][i], kf);
#pragma unroll
        for (int e = 0; e < epc; ++e) acc = fmaf(kf[e], qf[i][e], acc);
      }
    }
    acc = R == 16 ? sum16(acc) : oct_sum(acc);
    const int j = kr + RPP * m;
    if (kc == 0 && j < nrec) wl[W::coef + j] = acc;
  }
  wave_lds_sync();

  // ---- sum_j w_j v_j: per-lane partial over the lane's records, then summed over the
  // record groups through LDS
  float vacc[epc];
#pragma unroll
  for (int e = 0; e < epc; ++e) vacc[e] = 0.f;
#pragma unroll
  for (int m = 0; m < VP; ++m) {
    const int j = vr + VR * m;
    if (vr < VR && j < nrec) {
      const float w = wl[W::dec + j] * wl[W::coef + j];
      float vf[epc];
      widen<BF>(vraw[m], vf);
#pragma unroll
      for (int e = 0; e < epc; ++e) vacc[e] = fmaf(w, vf[e], vacc[e]);
    }
  }
  if (vr < VR) {
#pragma unroll
    for (int e = 0; e < epc; e += 4)
      *(float4 *)(wl + W::vt + vr * P + vc * epc + e) = make_float4(vacc[e], vacc[e + 1], vacc[e + 2], vacc[e + 3]);
  }

  // ---- append the step's record (its input bits) to ring slot (nk + hb) mod C before the
  // read-copy product, so the record registers are free for it
  const uint32_t sh = slot_of(hb);
  if (lane == hb) {
    uint8_t *p = (uint8_t *)ab + (size_t)sh * ast;
    if (BF)
      *(uint16_t *)p = (uint16_t)araw;
    else
      *(uint32_t *)p = araw;
  }
#pragma unroll
  for (int m = 0; m < VP; ++m)
    if (vr < VR && vr + VR * m == hb) *(uint4 *)((uint8_t *)vb + (size_t)sh * vst + vc * 16) = vraw[m];
  if ((hh % g.grp) == 0) {           // key-head leader: key and query rows
    uint8_t *kd = (uint8_t *)kb + (size_t)sh * kst;
    uint8_t *qd = (uint8_t *)qb + (size_t)sh * kst;
#pragma unroll
    for (int m = 0; m < KP; ++m)
      if (kr + RPP * m == hb)
#pragma unroll
        for (int i = 0; i < CPL; ++i) *(uint4 *)(kd + (kc + R * i) * 16) = kraw[m][i];
    if (kr == 0)
#pragma unroll
      for (int i = 0; i < CPL; ++i) *(uint4 *)(qd + (kc + R * i) * 16) = qraw[i];
  }

  // ---- S_read q, row sums to LDS (lane c8 of a row writes row group c8's sum); the copy is
  // loaded here, after the record rows are dead
  RCopy<N, RG> RCR;
  readcopy_load_rows(RCR, RCF, a.s_read, a.s_read_scale, tile, g.P, lane >> 3, 8, lane);
  float part[RG];
  readcopy_dot(RCR, RCF, wl + W::q, lane, part);
  const int r8 = lane >> 3, c8 = lane & 7;
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const float sr = oct_sum(part[i]);
    if (c8 == i) mine = sr;
  }
  const int row = 8 * c8 + r8;
  if (c8 < RG && row < P) wl[W::rc + row] = mine;
  wave_lds_sync();

  // ---- output rows (lane p takes row p)
  if (lane < P) {
    float sv = 0.f;
    for (int r = 0; r < VR; ++r) sv += wl[W::vt + r * P + lane];
    a.out[(size_t)hrow * P + lane] = fmaf(G, wl[W::rc + lane], sv);
  }
}

// Mamba-2 decode with a read copy: one wave per non-fold tile, then the fold tiles by the
// whole workgroup (see above).  A workgroup takes one value head of 4 consecutive sequences:
// sequences whose windows are at different positions fold at different steps, so a
// workgroup rarely has more than one fold to run (4 heads of one sequence would always fold
// together, and their workgroup would run 4 folds back to back).  A non-fold wave requests
// the read copy once its records are consumed: the copy's registers are then never live
// together with the record rows (fp8: 93 VGPRs instead of 103, 5 waves per SIMD instead of
// 4).  Requires vector staging, N of 64 or 128, P <= 64 and a window of 2 to 16 records.
template <int N, int RGW, int RCF, int STG>
__global__ __launch_bounds__(kThreads) void k_decode_rc(Args a) {
  constexpr bool BF = STG == kStageBf16;
  constexpr int RG = kWaves * RGW;
  static_assert(STG != kStageScalar && RCF != RSSM_READ_NONE, "vector staging with a read copy");
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int grp = tile_of_block(((g.B + kWaves - 1) / kWaves) * g.H);
  const int bq = grp / g.H, hh = grp - bq * g.H, gq = hh / g.grp;
  const int b = bq * kWaves + wave;
  const int tile = b * g.H + hh;
  int *flags = (int *)(lds + decode_rc_flag_offset(g.C + 1, g.P, N, WaveLds<N>::total));
  int fold = 0;
  if (b < g.B) {
    const int64_t nc = a.n_committed[tile], nk = a.n_ckpt[tile];
    const int64_t hb64 = nc - nk;
    if (hb64 < 0 || hb64 > g.C) {
      if (lane == 0) atomicOr(a.err, RSSM_DEVERR_CURSOR);
    } else if (hb64 + 1 >= g.L) {
      fold = 1;
    } else {
      m2_nonfold_wave<N, RG, RCF, BF>(a, tile, lds + wave * WaveLds<N>::total, b, hh, gq, nk, (int)hb64, lane);
      if (lane == 0) a.n_committed[tile] = nc + 1;
    }
  }
  if (lane == 0) flags[wave] = fold;
  __syncthreads();
  for (int w = 0; w < kWaves; ++w) {
    if (!flags[w]) continue;               // the same for every thread of the workgroup
    const int tw = (bq * kWaves + w) * g.H + hh;
    const int64_t nc = a.n_committed[tw], nk = a.n_ckpt[tw];
    decode_fold_tile<RSSM_KIND_MAMBA2, N, RGW, RCF, STG>(a, lds, tw, nk, (int)(nc - nk));
    if (threadIdx.x == 0) {
      a.n_committed[tw] = nc + 1;
      a.n_ckpt[tw] = nc + 1;
    }
    __syncthreads();
  }
}

// FOLD: flush fused in front of the verify (a window with at least a.min_records records is
// folded into the checkpoint first, exactly as a flush would, read copy in format RCF
// included, and the verify then reads only the drafts).
template <int KIND, int N, int RGW, bool FOLD, int RCF, int STG>
__global__ __launch_bounds__(kThreads) void k_verify(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block<FOLD || KIND != RSSM_KIND_MAMBA2>(g.B * g.H);
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
  // The window must take the T drafts next to its committed records even when it is folded
  // first: the draft slots then never hold a record that a sibling head of the key group may
  // still be staging for its own fold.
  if (hb + T > g.C) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_VERIFY_CAPACITY);
    return;
  }
  const bool fold = FOLD && hb >= a.min_records;
  const int P = g.P;
  const int cap = g.C;
  const LdsLayout L = lds_layout(KIND, cap, T, P, N, a.gather_out);
  float *tileS = a.s + (int64_t)tile * P * N;

  StageSpec sp = make_spec<KIND, N>(a, L, lds, b, hh, gq, nk, hb, T, T);
  sp.ia0 = b * T * g.H + hh;
  sp.ias = g.H;
  sp.iv0 = (b * T * g.H + hh) * P;
  sp.ivs = g.H * P;
  sp.ik0 = (b * T * g.G + gq) * N;
  sp.iks = g.G * N;
  sp.iq0 = sp.ik0;
  sp.iqs = sp.iks;

  // Draft tree: draft tau's parent (a.parent [B][T], -1 = the committed head; without a
  // tree, the previous draft).  Loaded with the records, resolved to ancestor masks after.
  const int my_parent = t < T ? (a.parent ? a.parent[b * T + t] : t - 1) : 0;
  Frag<N, RGW> F;
  stage_with_tile<4, KIND, STG>(sp, lds, t, [&]() { frag_load<N, RGW, true>(F, tileS, P, wave, lane); });
  int *const par = (int *)(lds + L.anc) + T;
  uint32_t *const anc = (uint32_t *)(lds + L.anc);
  if (t < T) par[t] = my_parent;
  __syncthreads();
  if (t < T) {                       // bit d of anc[tau]: draft d is on tau's root-to-node path
    uint32_t m = 0;
    int d = t;
    while (d >= 0) {
      m |= 1u << d;
      const int pd = par[d];
      if (pd < -1 || pd >= d) {
        m = 0;                       // invalid encoding
        break;
      }
      d = pd;
    }
    anc[t] = m;
  }
  __syncthreads();
  for (int tau = 0; tau < T; ++tau)
    if (anc[tau] == 0) {             // an invalid tree: nothing is written for this sequence
      if (t == 0) atomicOr(a.err, RSSM_DEVERR_TREE);
      return;
    }
  if (FOLD && fold) {                // the flush part: fold the hb committed records
    if (KIND == RSSM_KIND_MAMBA2) {
      if (wave == 0) wave_decays(lds + L.alpha, hb - 1, lds + L.dec, lds + L.gam, cap, lane);
      __syncthreads();
      fold_m2(F, lds, L, hb, P, wave, lane);
    } else {
      fold_delta<KIND>(F, lds, L, hb, P, wave, lane);
    }
    frag_store(F, tileS, P, wave, lane);
    frag_store_read_copy<RCF>(F, a.s_read, a.s_read_scale, tile, P, wave, lane);
    if (t == 0) a.n_ckpt[tile] = nc;
    __syncthreads();                 // the decay rows are rewritten below
  }
  // A folded window's records are in the checkpoint now: the verify reads record views that
  // start past them (the drafts only).  Otherwise the views are the staged records.
  const int r0 = fold ? hb : 0;
  const int hv = hb - r0;              // committed records every query sees
  LdsLayout Lv = L;
  Lv.alpha += KIND == RSSM_KIND_KDA ? r0 * (N + 4) : r0;
  Lv.beta += r0;
  Lv.K += r0 * (N + 4);
  Lv.V += r0 * P;

  const float *xbase;
  const float *dec = nullptr;
  if (KIND == RSSM_KIND_MAMBA2) {
    // W[j, tau] = product of alpha_m over on-path m with j < m <= hv + tau (dec rows), G_tau
    // (gam), k_j . q_tau (coef rows)
    for (int tau = wave; tau < T; tau += kWaves)
      wave_decays(lds + Lv.alpha, hv + tau, lds + Lv.dec + tau * cap, lds + Lv.gam + tau, cap, lane, hv, anc[tau]);
    kq_dots<N>(lds, Lv, cap, hv + T, T, t);
    __syncthreads();
    xbase = lds + Lv.q;
    dec = lds + Lv.dec;
  } else {
    for (int tau = wave; tau < T; tau += kWaves)
      delta_sweep_wave<KIND, N>(lds, Lv, cap, hv + tau + 1, tau, lane, hv, anc[tau]);
    __syncthreads();
    xbase = lds + Lv.r;
  }

  // Output rows: with a.gather_out they are collected in LDS and then stored as whole rows
  // (16 bytes per lane where P and the output allow it) instead of 4 bytes per row-octet lane.
  for (int tau = 0; tau < T; ++tau) {
    float part[RGW];
    frag_dot(F, xbase + tau * N, lane, part);
    const float *dt = dec ? dec + tau * cap : nullptr, *ct = lds + Lv.coef + tau * cap;
    if (a.gather_out)                  // the same for every thread: LDS and global stores stay typed
      write_rows<RGW>(part, lds[Lv.gam + tau], lds, Lv, dt, ct, hv + tau + 1, P, lds + L.o + tau * P, wave, lane);
    else
      write_rows<RGW>(part, lds[Lv.gam + tau], lds, Lv, dt, ct, hv + tau + 1, P,
                      a.out + (((int64_t)b * T + tau) * g.H + hh) * P, wave, lane);
  }
  if (a.gather_out) {
    __syncthreads();
    float *ob = a.out + ((int64_t)b * T * g.H + hh) * P;     // row tau at ob + tau * H * P
    if ((P & 3) == 0 && (((uintptr_t)a.out) & 15) == 0) {
      const int P4 = P >> 2;
      for (int c = t; c < T * P4; c += kThreads) {
        const int tau = c / P4, e = c - tau * P4;
        *(float4 *)(ob + (int64_t)tau * g.H * P + 4 * e) = *(const float4 *)(lds + L.o + tau * P + 4 * e);
      }
    } else {
      for (int c = t; c < T * P; c += kThreads) {
        const int tau = c / P, e = c - tau * P;
        ob[(int64_t)tau * g.H * P + e] = lds[L.o + tau * P + e];
      }
    }
  }
  // Draft tau goes to slot (n_committed + tau) mod C, one wave per draft.  Draft slots are
  // never a committed record's slot (h + T <= C), so no sibling head's staging reads them.
  for (int tau = wave; tau < T; tau += kWaves)
    append_from_lds<KIND, N>(a, L, lds, b, hh, gq, hb + tau, tau, ring_add(sp.slot0, hb + tau, g.C), lane, 64);
}

template <int KIND, int N, int RGW, int RCF, int STG>
__global__ __launch_bounds__(kThreads) void k_flush(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block<true>(g.B * g.H);
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

  StageSpec sp = make_spec<KIND, N>(a, L, lds, b, hh, gq, nk, nrec, 0, 0);
  Frag<N, RGW> F;
  stage_with_tile<4, KIND, STG>(sp, lds, t, [&]() { frag_load<N, RGW, false>(F, tileS, P, wave, lane); });
  __syncthreads();
  if (KIND == RSSM_KIND_MAMBA2) {
    if (wave == 0) wave_decays(lds + L.alpha, nrec - 1, lds + L.dec, lds + L.gam, cap, lane);
    __syncthreads();
    fold_m2(F, lds, L, nrec, P, wave, lane);
  } else {
    fold_delta<KIND>(F, lds, L, nrec, P, wave, lane);
  }
  frag_store(F, tileS, P, wave, lane);
  frag_store_read_copy<RCF>(F, a.s_read, a.s_read_scale, tile, P, wave, lane);
  if (t == 0) a.n_ckpt[tile] = nc;
}

// One recurrence step on the register tile with staged record j:
// Mamba-2 S <- a S + v k^T; Gated DeltaNet S <- a S + u k^T with u = b (v - a S k);
// KDA: the fold's per-channel update.
template <int KIND, int N, int RGW>
__device__ __forceinline__ void step_record(Frag<N, RGW> &F, const float *lds, const LdsLayout &L, int j, int P,
                                            int wave, int lane) {
  if constexpr (KIND == RSSM_KIND_KDA) {
    LdsLayout Lj = L;
    Lj.alpha += j * (N + 4);
    Lj.beta += j;
    Lj.K += j * (N + 4);
    Lj.V += j * P;
    fold_kda(F, lds, Lj, 1, P, wave, lane);
    return;
  }
  const int c = frag_col(lane);
  const float al = lds[L.alpha + j];
  const float *kr = lds + L.K + j * (N + 4) + c;
  float u[RGW];
  if (KIND == RSSM_KIND_MAMBA2) {
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const int row = frag_row(wave, lane, i);
      u[i] = (row < P) ? lds[L.V + j * P + row] : 0.f;
    }
  } else {
    float w[RGW];
#pragma unroll
    for (int i = 0; i < RGW; ++i) w[i] = 0.f;
#pragma unroll
    for (int f = 0; f < N / 32; ++f) {
      const float4 kf = *(const float4 *)(kr + 32 * f);
#pragma unroll
      for (int i = 0; i < RGW; ++i) w[i] = dot4(F.s[i][f], kf, w[i]);
    }
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      const int row = frag_row(wave, lane, i);
      const float vr = (row < P) ? lds[L.V + j * P + row] : 0.f;
      u[i] = lds[L.beta + j] * (vr - al * oct_sum(w[i]));
    }
  }
#pragma unroll
  for (int f = 0; f < N / 32; ++f) {
    const float4 kf = *(const float4 *)(kr + 32 * f);
#pragma unroll
    for (int i = 0; i < RGW; ++i) {
      F.s[i][f].x = fmaf(al, F.s[i][f].x, u[i] * kf.x);
      F.s[i][f].y = fmaf(al, F.s[i][f].y, u[i] * kf.y);
      F.s[i][f].z = fmaf(al, F.s[i][f].z, u[i] * kf.z);
      F.s[i][f].w = fmaf(al, F.s[i][f].w, u[i] * kf.w);
    }
  }
}

template <int KIND, int N, int RGW, int STG>
__global__ __launch_bounds__(kThreads) void k_conventional(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int P = g.P;
  const LdsLayout L = lds_layout(KIND, 1, 1, P, N);
  float *tileS = a.s + (int64_t)tile * P * N;
  StageSpec sp = make_spec<KIND, N>(a, L, lds, b, hh, gq, 0, 0, 1, 1);
  sp.slot0 = 0;
  sp.ia0 = b * g.H + hh;
  sp.iv0 = (b * g.H + hh) * P;
  sp.ik0 = (b * g.G + gq) * N;
  sp.iq0 = sp.ik0;
  Frag<N, RGW> F;
  stage_with_tile<4, KIND, STG>(sp, lds, t, [&]() { frag_load<N, RGW, false>(F, tileS, P, wave, lane); });
  __syncthreads();
  step_record<KIND, N, RGW>(F, lds, L, 0, P, wave, lane);
  frag_store(F, tileS, P, wave, lane);
  float part[RGW];
  frag_dot(F, lds + L.q, lane, part);
  write_row_sums<RGW>(part, P, a.out + (b * g.H + hh) * P, wave, lane);
}

// Snapshot-based speculative verify, the comparison point for k_verify: read the committed
// state (snapshot slot cur[b]), apply the T drafts one after another, and write each
// intermediate state to its own slot (cur[b] + 1 + tau) mod S and output from it: one state
// read and T state writes per step.  Snapshots: fp32 [B][S][H][P][N], S = slots per sequence.
template <int KIND, int N, int RGW, int STG>
__global__ __launch_bounds__(kThreads) void k_verify_snapshot(Args a) {
  extern __shared__ float lds[];
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int b = tile / g.H, hh = tile - b * g.H, gq = hh / g.grp;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int T = a.T, S = a.snap_slots;
  const int cur = a.snap_cur[b];
  if (cur < 0 || cur >= S) {
    if (t == 0) atomicOr(a.err, RSSM_DEVERR_CURSOR);
    return;
  }
  const int P = g.P;
  const LdsLayout L = lds_layout(KIND, T, T, P, N);
  const int64_t PN = (int64_t)P * N;
  float *const base = a.s + ((int64_t)b * S * g.H + hh) * PN;    // slot s at base + s * H * PN
  StageSpec sp = make_spec<KIND, N>(a, L, lds, b, hh, gq, 0, 0, T, T);
  sp.slot0 = 0;
  sp.ia0 = b * T * g.H + hh;
  sp.ias = g.H;
  sp.iv0 = (b * T * g.H + hh) * P;
  sp.ivs = g.H * P;
  sp.ik0 = (b * T * g.G + gq) * N;
  sp.iks = g.G * N;
  sp.iq0 = sp.ik0;
  sp.iqs = sp.iks;
  Frag<N, RGW> F;
  stage_with_tile<4, KIND, STG>(sp, lds, t, [&]() {
    frag_load<N, RGW, true>(F, base + (int64_t)cur * g.H * PN, P, wave, lane);
  });
  __syncthreads();
  for (int tau = 0; tau < T; ++tau) {
    step_record<KIND, N, RGW>(F, lds, L, tau, P, wave, lane);
    const int s = ring_add(cur, 1 + tau, S);
    frag_store(F, base + (int64_t)s * g.H * PN, P, wave, lane);
    float part[RGW];
    frag_dot(F, lds + L.q + tau * N, lane, part);
    write_row_sums<RGW>(part, P, a.out + ((b * T + tau) * g.H + hh) * P, wave, lane);
  }
}

template <int N, int RGW>
__global__ __launch_bounds__(kThreads) void k_init(Args a) {
  const Geom &g = a.g;
  const int tile = tile_of_block(g.B * g.H);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int P = g.P;
  Frag<N, RGW> F;
  if (a.s0)
    frag_load<N, RGW, false>(F, a.s0 + (int64_t)tile * P * N, P, wave, lane);
  else
    frag_zero(F);
  frag_store(F, a.s + (int64_t)tile * P * N, P, wave, lane);
  frag_store_read_copy_rt(F, g.read_copy, a.s_read, a.s_read_scale, tile, P, wave, lane);
  if (t == 0) {
    a.n_committed[tile] = 0;
    a.n_ckpt[tile] = 0;
    if (blockIdx.x == 0) *a.err = 0;
  }
}

// Dispatch over the supported (N, RGW) instances (RGW * N <= 512, so a lane holds at most
// 64 floats of the tile); CALL(n, r) must return.
#define RSSM_DISPATCH(N_, RGW_, CALL)                 \
  switch (N_) {                                       \
    case 32:                                          \
      switch (RGW_) {                                 \
        case 1: CALL(32, 1);                          \
        case 2: CALL(32, 2);                          \
        case 4: CALL(32, 4);                          \
        case 8: CALL(32, 8);                          \
        case 16: CALL(32, 16);                        \
        default: break;                               \
      }                                               \
      break;                                          \
    case 64:                                          \
      switch (RGW_) {                                 \
        case 1: CALL(64, 1);                          \
        case 2: CALL(64, 2);                          \
        case 4: CALL(64, 4);                          \
        case 8: CALL(64, 8);                          \
        default: break;                               \
      }                                               \
      break;                                          \
    case 128:                                         \
      switch (RGW_) {                                 \
        case 1: CALL(128, 1);                         \
        case 2: CALL(128, 2);                         \
        case 4: CALL(128, 4);                         \
        default: break;                               \
      }                                               \
      break;                                          \
    case 256:                                         \
      switch (RGW_) {                                 \
        case 1: CALL(256, 1);                         \
        case 2: CALL(256, 2);                         \
        default: break;                               \
      }                                               \
      break;                                          \
    default: break;                                   \
  }                                                   \
  return hipErrorInvalidValue;

}  // namespace rssm
