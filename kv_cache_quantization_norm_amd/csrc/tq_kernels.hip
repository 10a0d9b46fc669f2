// Device half of libtq: compression into the packed cache and single-query
// decode attention on it, for CDNA4 (gfx950), d = 128.
//
// Pages ("TurboQuant QJL投影深度剖析"):
//   section 2 - key = ||x||, Lloyd-Max codes of Pi x/||x||, signs of S r, ||r||;
//   section 5 - the record and the unbiased estimator
//               <q, x~> + ||r|| sqrt(pi/2)/d <S q, signs>;
//   section 6 - scoring with Pi q against centroids and S q against signs,
//               decode attention as one pass with an online softmax.
// MLX write-up, 背景: values take the MSE-only path.
//
// Kernels
//   compress_kernel        bulk compression (>= 16 tokens): at most one
//                          workgroup of 8 waves per CU over equal ranges of the
//                          flattened (layer, 16-token tile) sequence; Pi and
//                          S Pi^T staged in LDS as fp16 high + remainder MFMA
//                          operands, rotation and sketch on
//                          v_mfma_f32_16x16x32_f16, codes from a bucket table.
//   compress_append_kernel few-token compression (appends): 8 (token, head)
//                          items per workgroup as the MFMA columns.
//   qprep_kernel           Pi q and S q of every query row, per (quarter of
//                          [Pi; S], layer, run of 64 rows), fp16 MFMA with
//                          high + remainder operands.
//   decode_kernel          one workgroup of 8 waves per CU (its first
//                          workgroups may do a step's append first), each
//                          given an equal range of the problem-major sequence
//                          of 32-token chunks (a problem is one layer x
//                          sequence x KV head x group of <= 8 query heads;
//                          for ragged batches only the chunks that hold
//                          tokens); its waves draw chunks from an LDS ticket
//                          counter, load them through buffer resources two
//                          chunks ahead, form the key and value operands
//                          through LDS tables, score on
//                          v_mfma_f32_16x16x32_f16 (codes x Pi q, signs x
//                          S q), run the online softmax and accumulate values
//                          in the rotated domain (P x codes).  The workgroup
//                          that writes a problem's last piece merges its
//                          pieces and applies Pi^T (fp32 MFMA).
//   decode_pair_kernel     the decode of two caches of different formats (a
//                          compressed part and an fp16 part) in one launch:
//                          the workgroups are split between the parts in
//                          proportion to their bytes, each part dealt as by a
//                          launch of its own; the LDS is the larger layout.
//   qprep_pair_kernel      the query preparation of both parts, one launch.
//   append_prepare_kernel  a step's append and its query preparation in one
//                          launch.
//   combine_kernel         the same merge as a launch of its own (staged calls).
//   score_multi_kernel     multi-query scores: the key operands of a chunk
//                          formed once per 64 query rows.
//   stream_read_kernel     a plain streaming read, the bandwidth reference.
//   tail_gather_kernel     the fp16 tail tokens a ring flush moves, gathered
//                          for compression.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int D = 128;

// Keys of up to 2 Lloyd-Max bits take one scaled fp16 value per centroid;
// wider key codebooks take an fp16 high part and remainder (exact to about
// 2^-22), where no scale is needed.
constexpr bool key_split(int mk) { return mk >= 3; }


typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half8 as_half8(u32x4 w) {
  half8 h;
  __builtin_memcpy(&h, &w, 16);
  return h;
}

__device__ __forceinline__ floatx4 mfma16x16x32(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16x16x4f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// A wave-uniform pointer made opaque to the optimiser (an empty asm on its
// scalar registers), so that (uniform base + per-lane offset) addresses are
// formed per load as scalar base + 32-bit lane offset instead of being
// re-associated into 64-bit per-lane loop invariants that take two vector
// registers each.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  __asm__ volatile("" : "+s"(p));
  return p;
}
// Chunk loads go through buffer resources: the chunk's base address and
// extent in scalar registers, a 32-bit byte offset per lane, so that no lane
// holds a 64-bit address; loads past `bytes` return zero.  (Loads through a
// generic pointer would be flat loads, which also count on the LDS counter:
// every wait for an LDS read would then wait for the chunk loads in flight.)
// 0x00020000: the resource word 3 of an untyped 32-bit buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), 0x00020000);
}
template <typename T>
__device__ __forceinline__ T bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
  } else if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 0));
  } else if constexpr (__is_same(T, u32x3)) {
    return __builtin_amdgcn_raw_buffer_load_b96(r, int(off), 0, 0);
  } else {
    static_assert(sizeof(T) == 16, "buffer load width");
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
  }
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  // bound_ctrl set and every lane a valid source: the move can fold into the
  // arithmetic that consumes it (a DPP operand).
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Sum over the 64 lanes, in a fixed order, returned to every lane: DPP within
// each 16-lane row (quad swaps, then the half-row and row mirrors), then the
// four row sums through readlane.
// Maximum over the 64 lanes (NaN ignored, as fmaxf does), returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const int b = __builtin_bit_cast(int, v);
  return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float load_elem(const void* p, int dtype, int64_t i) {
  if (dtype == TQ_DTYPE_F32) return static_cast<const float*>(p)[i];
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  if (dtype == TQ_DTYPE_BF16) return __uint_as_float(uint32_t(h) << 16);
  _Float16 f;
  __builtin_memcpy(&f, &h, 2);
  return float(f);
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
  _Float16 h = _Float16(x);
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

// ===========================================================================
// Compression

struct CompressArgs {
  const void* k;
  const void* v;
  int dtype;
  int layer0;
  int64_t n_tokens;
  const int64_t* slots;
  int64_t slot0;
  int64_t slot_shift;   // added to slots[i] (a ring's mirror copy); 0 for the public calls
  int H;
  int64_t capacity;
  int mk;  // key MSE bits, 0 = fp16 keys
  int bv;  // value bits, 0 = fp16 values
  int64_t tiles_per_wg;   // bulk kernel: tiles of the flattened (layer, tile) sequence per workgroup
  int64_t total_tiles;
  const float* pi;
  const float* pi_s;
  const float* kc;
  const float* kb;
  const float* vc;
  const float* vb;
  uint8_t* k_idx;
  uint8_t* k_sign;
  float* k_norm;
  float* k_rnorm;
  uint16_t* k_f16;
  uint8_t* v_idx;
  float* v_norm;
  uint16_t* v_f16;
};

constexpr int kCompressTile = 16;  // tokens per wave step

// Shared memory of the compress kernel.  Pi and M = S Pi^T are held as fp16
// A operands of v_mfma_f32_16x16x32_f16, each matrix as its fp16 high part
// and its remainder scaled by 2^11 (P = hi + 2^-11 lo), in operand order:
//   ph / pl [(tile * 4 + s) * 64 + lane][e] = Pi[16 tile + lane % 16][32 (lane / 16) + 8 s + e]
//   mh / ml [(tp * 4 + s) * 64 + lane][e]   = M[16 tp + lane % 16][c(s, lane / 16, e)],
//     c(s, q, e) = 16 (2 s + e / 4) + 4 q + e % 4.
// The sketch's contraction order follows the rotation's output layout, so each
// lane's residual values are already its B operands.  Then the quantisation
// tables of both codebooks and per-wave packing scratch.
constexpr int kCompressWaves = 8;
constexpr int kCompressWorkgroups = 256;   // one per CU
constexpr int kQBuckets = 512;
// Key codes of up to 4 bits pack into at most 16 dwords a token, 7-bit codes
// (8-bit keys) into 28.  While a tile's records are assembled in LDS their
// row stride is one dword more, odd, so that the 16 tokens fall in 16
// different banks.
template <int MK> constexpr int kRecStride = MK > 4 ? 29 : 17;
struct CompressSmem {
  half8 ph[8 * 4 * 64], pl[8 * 4 * 64];
  half8 mh[8 * 4 * 64], ml[8 * 4 * 64];
  u32x2 kq[kQBuckets], vq[kQBuckets];
  float kc[128], vc[16];
  // Per wave: the packed key codes of 16 tokens (kRecStride dwords each),
  // later the value codes of 16 tokens per coordinate (2 D dwords); the key
  // records are written out before the values are coded.
  uint32_t recv[kCompressWaves][kCompressTile * 29];
  uint32_t srec[kCompressWaves][kCompressTile * 4];   // packed signs per token
};

// Lane (t = lane % 16, q = lane / 16) holds coordinates 32q .. 32q+31 of token t.
__device__ __forceinline__ void load_token_slab(const CompressArgs& a, const void* base, int layer_rel,
                                                int64_t tok, int h, int q, bool valid, float (&xr)[32]) {
  if (!valid) {
#pragma unroll
    for (int s = 0; s < 32; ++s) xr[s] = 0.f;
    return;
  }
  const int64_t off = ((int64_t(layer_rel) * a.n_tokens + tok) * a.H + h) * D + 32 * q;
  if (a.dtype == TQ_DTYPE_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float4 f = p[u];
      xr[4 * u] = f.x; xr[4 * u + 1] = f.y; xr[4 * u + 2] = f.z; xr[4 * u + 3] = f.w;
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 w = p[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = w[e] & 0xFFFFu, hi = w[e] >> 16;
        if (a.dtype == TQ_DTYPE_BF16) {
          xr[8 * u + 2 * e] = __uint_as_float(lo << 16);
          xr[8 * u + 2 * e + 1] = __uint_as_float(hi << 16);
        } else {
          _Float16 f0, f1;
          uint16_t l16 = uint16_t(lo), h16 = uint16_t(hi);
          __builtin_memcpy(&f0, &l16, 2);
          __builtin_memcpy(&f1, &h16, 2);
          xr[8 * u + 2 * e] = float(f0);
          xr[8 * u + 2 * e + 1] = float(f1);
        }
      }
    }
  }
}

// Quantisation table of a codebook with nb ascending boundaries t_k, at
// scale S (512 buckets of width 1/S over [-256/S, 256/S)): bucket u covers y
// in [(u - 256) / S, (u - 255) / S), the first and last buckets extended to
// -inf and +inf.  Entry u holds the number of boundaries below
// L_u = (u - 256 - 1/2) / S and the first boundary at or above L_u if it lies
// below L_u + 2 / S (+inf otherwise).  The rounded bucket arithmetic puts y in
// a bucket u with y in [L_u, L_u + 2 / S), so the code #{k : y >= t_k} is
// count + [y >= boundary] as long as no two boundaries are closer than 2 / S
// and all lie inside the table.  S = 512 for up to 4 bits: the d = 128
// boundaries lie in (-0.25, 0.25), more than 0.02 apart.  S = 512 / 0.7 for 7
// bits: boundaries within +-0.339, at least 0.00295 apart, against 2 / S =
// 0.00273.
constexpr float kQScale = 512.f;
constexpr float kQScaleWide = 512.f / 0.7f;
__device__ __forceinline__ void build_qtab(u32x2* tab, const float* bnd, int nb, int tid, int nt,
                                           float scale = kQScale) {
  for (int u = tid; u < kQBuckets; u += nt) {
    const float lo = (float(u - kQBuckets / 2) - 0.5f) / scale, hi = lo + 2.f / scale;
    uint32_t cnt = 0;
    float first = INFINITY;
    for (int k = 0; k < nb; ++k) {
      const float t = bnd[k];
      if (t < lo)
        ++cnt;
      else if (t < first)
        first = t;
    }
    tab[u] = u32x2{cnt, __float_as_uint(first < hi ? first : INFINITY)};
  }
}
__device__ __forceinline__ uint32_t qcode(float y, const u32x2* tab, float scale = kQScale) {
  float u = fmaf(y, scale, 0.5f * kQBuckets);
  u = fminf(fmaxf(u, 0.f), float(kQBuckets - 1));   // NaN -> bucket 0 -> code 0
  const u32x2 e = tab[int(u)];
  return e[0] + (y >= __uint_as_float(e[1]) ? 1u : 0u);
}

// Two floats -> fp16 pair (rounded toward zero), as a dword.
__device__ __forceinline__ uint32_t pk16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ float lo16(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w))); }
__device__ __forceinline__ float hi16(uint32_t w) { return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16))); }
// High parts and remainders (times 2^11) of 8 floats as fp16 operands.
__device__ __forceinline__ void split8(const float (&v)[8], half8& hi, half8& lo, bool want_lo) {
  u32x4 h, l = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    h[p] = pk16(v[2 * p], v[2 * p + 1]);
    if (want_lo) l[p] = pk16((v[2 * p] - lo16(h[p])) * 2048.f, (v[2 * p + 1] - hi16(h[p])) * 2048.f);
  }
  hi = as_half8(h);
  lo = as_half8(l);
}

// Norm and y = Pi x / ||x|| for the wave's 16 tokens.  Lane (t, q) holds
// coordinates 32 q .. 32 q + 31 of token t in xr; on return it holds
// y[16 tile + 4 q + r] of token t in y[tile][r].  The B operand is
// x' = x 2^e with 2^e ||x|| in [2^14, 2^15), in fp16: exact for bf16 and fp16
// inputs (their significands fit), a high part plus a remainder (times 2^11)
// for fp32 inputs (XHL).  a1 collects hi(Pi) hi(x'), a2 the remainder products.
template <bool XHL>
__device__ __forceinline__ float rotate16(const CompressSmem& sm, const float (&xr)[32], int lane,
                                          float (&y)[8][4]) {
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < 32; ++s) ss = fmaf(xr[s], xr[s], ss);
  ss += shfl_xor(ss, 16);
  ss += shfl_xor(ss, 32);
  const float n = sqrtf(ss);
  // n = 0 -> y = 0; NaN -> NaN everywhere.
  const float inv = n > 0.f ? 1.0f / n : (n == 0.f ? 0.f : n);
  const int e = (n > 0.f && n < INFINITY) ? 15 - __builtin_amdgcn_frexp_expf(n) : 0;
  half8 xh[4], xl[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_amdgcn_ldexpf(xr[8 * s + k], e);
    split8(v, xh[s], xl[s], XHL);
  }
  const float sc = __builtin_amdgcn_ldexpf(inv, -e);
#pragma unroll
  for (int tile = 0; tile < 8; ++tile) {
    floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const half8 ah = sm.ph[(tile * 4 + s) * 64 + lane], al = sm.pl[(tile * 4 + s) * 64 + lane];
      a1 = mfma16x16x32(ah, xh[s], a1);
      a2 = mfma16x16x32(al, xh[s], a2);
      if constexpr (XHL) a2 = mfma16x16x32(ah, xl[s], a2);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) y[tile][r] = fmaf(a2[r], 0x1p-11f, a1[r]) * sc;
  }
  return n;
}

// Stages a 128 x 128 fp32 matrix (row-major) as fp16 high / remainder A
// operands.  Element (row, col) goes to operand entry ((row / 16) * 4 + s) *
// 64 + q * 16 + row % 16, half e, with (s, q, e) from col in the rotation's
// contraction order or (sketch) in the residual order.  512 threads, 8
// float4 each, all loads issued before the LDS writes.
__device__ __forceinline__ void stage_operands(half8* hi, half8* lo, const float* src, int tid, bool sketch) {
  const float4* s4 = reinterpret_cast<const float4*>(src);
  float4 buf[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) buf[u] = s4[tid + 512 * u];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e0 = 4 * (tid + 512 * u), row = e0 >> 7, col = e0 & 127;
    int s, q, e;
    if (!sketch) {
      q = col >> 5;
      s = (col >> 3) & 3;
      e = col & 7;
    } else {
      const int tc = col >> 4;   // residual tile 2 s + e / 4
      s = tc >> 1;
      q = (col >> 2) & 3;
      e = 4 * (tc & 1);
    }
    const int ent = ((row >> 4) * 4 + s) * 64 + q * 16 + (row & 15);
    const float v[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
    uint32_t h[2], l[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const _Float16 a = _Float16(v[2 * p]), b = _Float16(v[2 * p + 1]);
      const _Float16 la = _Float16((v[2 * p] - float(a)) * 2048.f), lb = _Float16((v[2 * p + 1] - float(b)) * 2048.f);
      h[p] = uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
      l[p] = uint32_t(__builtin_bit_cast(uint16_t, la)) | (uint32_t(__builtin_bit_cast(uint16_t, lb)) << 16);
    }
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(&hi[ent]) + e) = u32x2{h[0], h[1]};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(&lo[ent]) + e) = u32x2{l[0], l[1]};
  }
}

// OR the 4 consecutive m-bit codes `chunk` (coordinates 16 tile + 4 q .. +3)
// into a token record in LDS.
__device__ __forceinline__ void or_bits(uint32_t* rec, int bitpos, uint32_t chunk, int nbits) {
  const int w = bitpos >> 5, sh = bitpos & 31;
  atomicOr(&rec[w], chunk << sh);
  if (sh + nbits > 32) atomicOr(&rec[w + 1], chunk >> (32 - sh));
}

// Writes the BV-bit value code of slot p of a (block, coordinate) group of
// 32 codes (4 BV bytes, LSB-first: code p at bits [BV p, BV p + BV)); a 3-bit
// code may straddle two dwords.  Other codes of the group are left as they are.
template <int BV>
__device__ __forceinline__ void put_vcode(uint32_t* group, int p, uint32_t idx) {
  const int bit = p * BV, w = bit >> 5, sh = bit & 31;
  const uint32_t m = (1u << BV) - 1u;
  atomicAnd(group + w, ~(m << sh));
  atomicOr(group + w, idx << sh);
  if (sh + BV > 32) {
    const int rs = 32 - sh;
    atomicAnd(group + w + 1, ~(m >> rs));
    atomicOr(group + w + 1, idx >> rs);
  }
}

// XHL: fp32 inputs, whose slabs need a remainder operand (bf16 / fp16 inputs
// are exact fp16 operands).
template <int MK, int BV, bool XHL>
__global__ __launch_bounds__(kCompressWaves * 64) void compress_kernel(CompressArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  CompressSmem& sm = *reinterpret_cast<CompressSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = lane & 15, q = lane >> 4;
  const bool need_rot = MK > 0 || BV > 0;
  constexpr float KQS = MK > 4 ? kQScaleWide : kQScale;
  if (tid < 128) {
    const int nk = MK > 0 ? (1 << MK) : 0, nv = BV > 0 ? (1 << BV) : 0;
    // The key residual applies the fp32 table centroids.
    sm.kc[tid] = tid < nk ? a.kc[tid] : 0.f;
    if (tid < 16) sm.vc[tid] = tid < nv ? a.vc[tid] : 0.f;
  }
  if constexpr (MK > 0) build_qtab(sm.kq, a.kb, (1 << MK) - 1, tid, kCompressWaves * 64, KQS);
  if constexpr (BV > 0) build_qtab(sm.vq, a.vb, (1 << BV) - 1, tid, kCompressWaves * 64);
  __syncthreads();

  // The workgroup owns tiles [g_lo, g_hi) of the (layer, 16-token tile)
  // sequence of the call, taken one layer segment at a time: the segment's
  // Pi and M operands are staged, then its (tile, head) items are dealt round
  // robin to the waves.
  const int64_t n_tiles = (a.n_tokens + kCompressTile - 1) / kCompressTile;
  const int64_t g_lo = int64_t(blockIdx.x) * a.tiles_per_wg;
  const int64_t g_hi = g_lo + a.tiles_per_wg < a.total_tiles ? g_lo + a.tiles_per_wg : a.total_tiles;
  for (int64_t g0 = g_lo; g0 < g_hi;) {
  const int layer_rel = int(g0 / n_tiles);
  const int layer = a.layer0 + layer_rel;
  const int64_t g1 = (int64_t(layer_rel) + 1) * n_tiles < g_hi ? (int64_t(layer_rel) + 1) * n_tiles : g_hi;
  if (g0 != g_lo) __syncthreads();   // every wave is done with the previous layer's operands
  if (need_rot) stage_operands(sm.ph, sm.pl, a.pi + int64_t(layer) * D * D, tid, false);
  if constexpr (MK > 0) stage_operands(sm.mh, sm.ml, a.pi_s + int64_t(layer) * D * D, tid, true);
  __syncthreads();
  const int64_t n_items = (g1 - g0) * a.H;
  for (int64_t item = wave; item < n_items; item += kCompressWaves) {
  const int64_t tl = g0 - int64_t(layer_rel) * n_tiles + item / a.H;
  const int h = int(item % a.H);
  const int64_t tok0 = tl * kCompressTile;
  const int64_t tok = tok0 + t;
  const bool tok_ok = tok < a.n_tokens;
  int64_t slot = -1;
  if (tok_ok) slot = a.slots ? a.slots[tok] + a.slot_shift : a.slot0 + tok;
  const bool valid = tok_ok && slot >= 0 && slot < a.capacity;
  // Fast value path: 16 contiguous, 16-aligned, all-valid slots.
  bool contiguous = (a.slots == nullptr) && (tok0 + kCompressTile <= a.n_tokens) &&
                    ((a.slot0 + tok0) % kCompressTile == 0) && (a.slot0 + tok0 >= 0) &&
                    (a.slot0 + tok0 + kCompressTile <= a.capacity);

  uint32_t* rec = sm.recv[wave];
  uint32_t* srec = sm.srec[wave];
  uint32_t* vrec = sm.recv[wave];   // after the key records are out
  constexpr int KSTR = kRecStride<MK>;
  const int kwords = 4 * MK;  // dwords per key code record

  {
    const int64_t plane = int64_t(layer) * a.H + h;  // [layer][head]
    float xr[32];
    float y[8][4];
    // ---------------- keys
    load_token_slab(a, a.k, layer_rel, tok, h, q, valid, xr);
    if constexpr (MK == 0) {
      if (valid) {
        uint16_t* dst = a.k_f16 + (plane * a.capacity + slot) * D + 32 * q;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = uint32_t(f16_bits(xr[8 * u + 2 * e])) | (uint32_t(f16_bits(xr[8 * u + 2 * e + 1])) << 16);
          reinterpret_cast<u32x4*>(dst)[u] = w;
        }
      }
    } else {
      const float n = rotate16<XHL>(sm, xr, lane, y);
      for (int e = lane; e < kCompressTile * KSTR; e += 64) rec[e] = 0u;
      srec[lane] = 0u;
      wave_sync();
      float a2 = 0.f;
      float res[8][4];
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) {
        uint32_t chunk = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t idx = qcode(y[tile][r], sm.kq, KQS);
          chunk |= idx << (r * MK);
          res[tile][r] = y[tile][r] - sm.kc[idx];
          a2 = fmaf(res[tile][r], res[tile][r], a2);
        }
        or_bits(rec + t * KSTR, (16 * tile + 4 * q) * MK, chunk, 4 * MK);
      }
      a2 += shfl_xor(a2, 16);
      a2 += shfl_xor(a2, 32);
      const float rnorm = n * sqrtf(a2);
      // z = M (y - c[idx]); sign of n * z (a zero key gives all ones).  B
      // operand of step s: res[2 s + e / 4][e % 4] times 2^14, as an fp16
      // high part and remainder; a1 collects hi(M) hi(res), a2 the rest.
      half8 rh[4], rl[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = res[2 * s4 + (e >> 2)][e & 3] * 16384.f;
        split8(v, rh[s4], rl[s4], true);
      }
#pragma unroll
      for (int tp = 0; tp < 8; ++tp) {
        floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const half8 mh = sm.mh[(tp * 4 + s4) * 64 + lane], ml = sm.ml[(tp * 4 + s4) * 64 + lane];
          a1 = mfma16x16x32(mh, rh[s4], a1);
          a2 = mfma16x16x32(mh, rl[s4], a2);
          a2 = mfma16x16x32(ml, rh[s4], a2);
        }
        uint32_t bits = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) bits |= (fmaf(a2[r], 0x1p-11f, a1[r]) * n >= 0.f ? 1u : 0u) << r;
        or_bits(srec + t * 4, 16 * tp + 4 * q, bits, 4);
      }
      wave_sync();
      if (valid && q == 0) {
        a.k_norm[plane * a.capacity + slot] = n;
        a.k_rnorm[plane * a.capacity + slot] = rnorm;
      }
      // Write the records: 16 tokens x kwords dwords, then 16 x 4 sign dwords.
      for (int e = lane; e < kCompressTile * kwords; e += 64) {
        const int tt = e / kwords, w = e - tt * kwords;
        const int64_t tk = tok0 + tt;
        if (tk >= a.n_tokens) continue;
        const int64_t sl = a.slots ? a.slots[tk] + a.slot_shift : a.slot0 + tk;
        if (sl < 0 || sl >= a.capacity) continue;
        reinterpret_cast<uint32_t*>(a.k_idx + (plane * a.capacity + sl) * (16 * MK))[w] = rec[tt * KSTR + w];
      }
      {
        const int tt = lane >> 2, w = lane & 3;
        const int64_t tk = tok0 + tt;
        if (tk < a.n_tokens) {
          const int64_t sl = a.slots ? a.slots[tk] + a.slot_shift : a.slot0 + tk;
          if (sl >= 0 && sl < a.capacity)
            reinterpret_cast<uint32_t*>(a.k_sign + (plane * a.capacity + sl) * 16)[w] = srec[tt * 4 + w];
        }
      }
      wave_sync();
    }
    // ---------------- values
    load_token_slab(a, a.v, layer_rel, tok, h, q, valid, xr);
    if constexpr (BV == 0) {
      if (valid) {
        // [plane][slot/32][coord][32] fp16
        uint16_t* dst = a.v_f16 + ((plane * (a.capacity / kVBlock) + slot / kVBlock) * D) * kVBlock + (slot % kVBlock);
#pragma unroll
        for (int s = 0; s < 32; ++s) dst[(32 * q + s) * kVBlock] = f16_bits(xr[s]);
      }
    } else {
      const float n = rotate16<XHL>(sm, xr, lane, y);
      if (valid && q == 0) a.v_norm[plane * a.capacity + slot] = n;
      uint32_t vidx[8][4];
#pragma unroll
      for (int tile = 0; tile < 8; ++tile)
#pragma unroll
        for (int r = 0; r < 4; ++r) vidx[tile][r] = qcode(y[tile][r], sm.vq);
      const int64_t gbytes = 4 * BV;  // bytes per (block, coordinate) group
      uint8_t* vplane = a.v_idx + plane * (a.capacity / kVBlock) * D * gbytes;
      if (contiguous && (BV == 2 || BV == 4)) {
        // The wave owns whole dwords: 16 tokens x bv bits per coordinate.  The
        // 32 / BV lanes of a dword (same q, consecutive t, inside one 16-lane
        // row) OR their shifted codes together across lanes (DPP quad swaps,
        // then the half-row and row mirrors), and the first of them stores
        // the dword: no LDS atomics, no clearing pass.
        const int dw = BV / 2;           // dwords per coordinate for 16 tokens
        constexpr int TPW = 32 / BV;     // tokens per dword
        const int tw = t & (TPW - 1);    // this token's place in its dword
        const bool writer = tw == 0;
        const int wsel = t / TPW;        // which dword of the coordinate
#pragma unroll
        for (int tile = 0; tile < 8; ++tile)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint32_t v = vidx[tile][r] << (BV * tw);
            v |= dpp_u<0xB1>(v);    // quad_perm [1,0,3,2]
            v |= dpp_u<0x4E>(v);    // quad_perm [2,3,0,1]
            v |= dpp_u<0x141>(v);   // row_half_mirror: the 8-lane OR
            if constexpr (BV == 2) v |= dpp_u<0x140>(v);   // row_mirror: the 16-lane OR
            if (writer) vrec[(16 * tile + 4 * q + r) * dw + wsel] = v;
          }
        wave_sync();
        const int64_t s0 = a.slot0 + tok0;
        const int64_t blk = s0 / kVBlock;
        const int half = int(s0 % kVBlock) / kCompressTile;  // which 16-slot half of the block
        for (int e = lane; e < D * dw; e += 64) {
          const int c = e / dw, w = e - c * dw;
          uint32_t* g = reinterpret_cast<uint32_t*>(vplane + (blk * D + c) * gbytes);
          g[half * dw + w] = vrec[e];
        }
        wave_sync();
      } else if (valid) {
        const int64_t blk = slot / kVBlock;
        const int p = int(slot % kVBlock);
#pragma unroll
        for (int tile = 0; tile < 8; ++tile)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 16 * tile + 4 * q + r;
            put_vcode<BV>(reinterpret_cast<uint32_t*>(vplane + (blk * D + c) * gbytes), p, vidx[tile][r]);
          }
      }
    }
  }
  }  // items
  g0 = g1;
  }  // layer segments
}

// Few-token compression (appends during decode).  The tile kernel above
// spends a 128 KB LDS staging of Pi and S Pi^T and a full pass of all eight
// row blocks per wave on every 16-token tile, which for one token per head is
// almost all waste.  Here one workgroup takes up to 8 (token, head) items of
// one layer, flattened as item = token * H + head, and the MFMA columns are
// the items' vectors: 8 keys and 8 values for the rotation, the 8 key
// residuals for the sketch.  Wave w owns rows 16 w .. 16 w + 15 of every
// product; its A operands (those rows of Pi and S Pi^T) come straight from
// global memory, all global loads issued at the start, and are split in
// registers into fp16 high parts and remainders (times 2^11) for
// v_mfma_f32_16x16x32_f16, as in the tile kernel; the k order of step s is
// columns 32 q + 8 s + e (lane q = lane / 16).
constexpr int kAppendItems = 8;
constexpr int kAppendWaves = 8;
constexpr int kAppendThreads = kAppendWaves * 64;
constexpr int kAppendStride = D + 4;  // padded LDS rows

struct AppendSmem {
  float xs[2 * kAppendItems][kAppendStride];  // K items, then V items
  float rs[kAppendItems][kAppendStride];      // key residual y - c[idx]
  float nrm[2 * kAppendItems];
  float rnrm[kAppendItems];
  uint32_t krec[kAppendItems][28];
  uint32_t srec[kAppendItems][4];
  int64_t slot_of[kAppendItems];
  // key centroids, key boundaries, value centroids, value boundaries (the
  // boundary tables padded with +inf)
  float cb[4][128];
};

// `done` (if not null): per layer, a count of finished append workgroups, for
// readers in the same launch.  The records are written with agent-scope
// (device-coherent) stores, the value codes with device atomics, and every
// wave waits for them to complete before the barrier that precedes the
// increment.
template <int MK, int BV>
__device__ __forceinline__ void append_body(const CompressArgs& a, int group, int layer_rel, AppendSmem& sm,
                                            uint32_t* done = nullptr) {
  auto& xs = sm.xs;
  auto& rs = sm.rs;
  auto& nrm = sm.nrm;
  auto& rnrm = sm.rnrm;
  auto& krec = sm.krec;
  auto& srec = sm.srec;
  auto& slot_of = sm.slot_of;
  auto& cb = sm.cb;
  constexpr bool ROT = MK > 0 || BV > 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q = lane >> 4;
  const int layer = a.layer0 + layer_rel;
  const int64_t n_items = a.n_tokens * a.H;
  const int64_t item0 = int64_t(group) * kAppendItems;
  const int ni = n_items - item0 < kAppendItems ? int(n_items - item0) : kAppendItems;

  // ---------------- all global loads
  // A operands: row 16 wave + col, columns 32 q .. 32 q + 31 (step s: float4s 2 s, 2 s + 1).
  float4 pa[ROT ? 8 : 1], ma[MK > 0 ? 8 : 1];
  if constexpr (ROT) {
    const float4* src =
        reinterpret_cast<const float4*>(a.pi + int64_t(layer) * D * D + int64_t(16 * wave + col) * D + 32 * q);
#pragma unroll
    for (int v = 0; v < 8; ++v) pa[v] = src[v];
  }
  if constexpr (MK > 0) {
    const float4* src =
        reinterpret_cast<const float4*>(a.pi_s + int64_t(layer) * D * D + int64_t(16 * wave + col) * D + 32 * q);
#pragma unroll
    for (int v = 0; v < 8; ++v) ma[v] = src[v];
  }
  // Item vectors: thread value u is element e = tid + 512 u of the 16 x 128
  // (keys, then values) block.
  constexpr int XU = 2 * kAppendItems * D / kAppendThreads;
  float xin[XU];
  {
    int64_t offs[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + kAppendThreads * u, c = e >> 7, j = e & 127;
      const int it = c & (kAppendItems - 1);
      const int64_t item = item0 + (it < ni ? it : ni - 1);
      offs[u] = ((int64_t(layer_rel) * a.n_tokens + item / a.H) * a.H + item % a.H) * D + j;
    }
    // u < XU / 2: keys, the others values.
    if (a.dtype == TQ_DTYPE_F32) {
#pragma unroll
      for (int u = 0; u < XU; ++u) xin[u] = static_cast<const float*>(u < XU / 2 ? a.k : a.v)[offs[u]];
    } else {
      uint16_t hv[XU];
#pragma unroll
      for (int u = 0; u < XU; ++u) hv[u] = static_cast<const uint16_t*>(u < XU / 2 ? a.k : a.v)[offs[u]];
      if (a.dtype == TQ_DTYPE_BF16) {
#pragma unroll
        for (int u = 0; u < XU; ++u) xin[u] = __uint_as_float(uint32_t(hv[u]) << 16);
      } else {
#pragma unroll
        for (int u = 0; u < XU; ++u) {
          _Float16 f;
          __builtin_memcpy(&f, &hv[u], 2);
          xin[u] = float(f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int it = ((tid + kAppendThreads * u) >> 7) & (kAppendItems - 1);
      if (it >= ni) xin[u] = 0.f;
    }
  }
  int64_t slot = -1;
  {
    const int64_t tok = (item0 + (tid < ni ? tid : 0)) / a.H;
    if (tid < kAppendItems && tid < ni) slot = a.slots ? a.slots[tok] + a.slot_shift : a.slot0 + tok;
  }
  // Codebooks: thread j holds entry j % 128 of table j / 128 (0 past the
  // end; the boundary tables are padded with +inf).
  constexpr int NCB = MK > 4 ? 128 : 16;   // entries used per table
  float cbv = 0.f;
  {
    const int nk = MK > 0 ? (1 << MK) : 0, nv = BV > 0 ? (1 << BV) : 0;
    const int tb = tid >> 7, j = tid & 127;
    if (j < NCB) {
      if (tb == 0 && j < nk) cbv = a.kc[j];   // fp32 table centroid (the key residual)
      if (tb == 1) cbv = j + 1 < nk ? a.kb[j] : INFINITY;
      if (tb == 2 && j < nv) cbv = a.vc[j];
      if (tb == 3) cbv = j + 1 < nv ? a.vb[j] : INFINITY;
    }
  }
  // Every global load above is in flight before any of them is waited on.
  __builtin_amdgcn_sched_barrier(0);
  if (tid < kAppendItems) slot_of[tid] = (slot < 0 || slot >= a.capacity) ? -1 : slot;
  if ((tid & 127) < NCB) cb[tid >> 7][tid & 127] = cbv;
  for (int e = tid; e < kAppendItems * 28; e += kAppendThreads) (&krec[0][0])[e] = 0u;
  if (tid < kAppendItems * 4) (&srec[0][0])[tid] = 0u;
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int e = tid + kAppendThreads * u;
    xs[e >> 7][e & 127] = xin[u];
  }
  __syncthreads();
  // Norms: wave w reduces vectors 2 w and 2 w + 1.
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = 2 * wave + k;
    const float x0 = xs[c][lane], x1 = xs[c][lane + 64];
    const float ss = wave_sum(fmaf(x0, x0, x1 * x1));
    if (lane == 0) nrm[c] = sqrtf(ss);
  }
  __syncthreads();

  const int64_t vblocks = a.capacity / kVBlock;
  const int row = 16 * wave + 4 * q;   // this lane's output rows row .. row + 3
  // ---------------- rotation y = Pi x / ||x|| (column col = item vector), quantisation
  if constexpr (ROT) {
    const bool is_k = col < kAppendItems;
    const int it = col & (kAppendItems - 1);
    const float n = nrm[col];
    // n = 0 -> y = 0; NaN -> NaN everywhere.
    const float inv = n > 0.f ? 1.0f / n : (n == 0.f ? 0.f : n);
    // B operand x 2^e with 2^e ||x|| in [2^14, 2^15): exact fp16 for bf16 /
    // fp16 inputs; fp32 inputs leave a remainder (times 2^11), zero otherwise.
    const int ex = (n > 0.f && n < INFINITY) ? 15 - __builtin_amdgcn_frexp_expf(n) : 0;
    floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 ah, al, xh, xl;
      {
        const float v[8] = {pa[2 * s].x, pa[2 * s].y, pa[2 * s].z, pa[2 * s].w,
                            pa[2 * s + 1].x, pa[2 * s + 1].y, pa[2 * s + 1].z, pa[2 * s + 1].w};
        split8(v, ah, al, true);
      }
      {
        const float4 x0 = *reinterpret_cast<const float4*>(&xs[col][32 * q + 8 * s]);
        const float4 x1 = *reinterpret_cast<const float4*>(&xs[col][32 * q + 8 * s + 4]);
        const float v[8] = {__builtin_amdgcn_ldexpf(x0.x, ex), __builtin_amdgcn_ldexpf(x0.y, ex),
                            __builtin_amdgcn_ldexpf(x0.z, ex), __builtin_amdgcn_ldexpf(x0.w, ex),
                            __builtin_amdgcn_ldexpf(x1.x, ex), __builtin_amdgcn_ldexpf(x1.y, ex),
                            __builtin_amdgcn_ldexpf(x1.z, ex), __builtin_amdgcn_ldexpf(x1.w, ex)};
        split8(v, xh, xl, true);
      }
      a1 = mfma16x16x32(ah, xh, a1);
      a2 = mfma16x16x32(al, xh, a2);
      a2 = mfma16x16x32(ah, xl, a2);
    }
    const float sc = __builtin_amdgcn_ldexpf(inv, -ex);
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = fmaf(a2[r], 0x1p-11f, a1[r]) * sc;
    const int64_t slot = slot_of[it];
    const int64_t plane = int64_t(layer) * a.H + (item0 + it) % a.H;
    if (it < ni) {
      if (is_k) {
        if constexpr (MK > 0) {
          uint32_t chunk = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint32_t idx = 0;
            if constexpr (MK > 4) {
              // binary search: #{k : y >= t_k} over the ascending boundaries
#pragma unroll
              for (int step = 1 << (MK - 1); step >= 1; step >>= 1)
                if (y[r] >= cb[1][idx + step - 1]) idx += step;
            } else {
#pragma unroll
              for (int b = 0; b < (1 << MK) - 1; ++b) idx += (y[r] >= cb[1][b]) ? 1u : 0u;
            }
            rs[it][row + r] = y[r] - cb[0][idx];
            chunk |= idx << (r * MK);
          }
          or_bits(&krec[it][0], row * MK, chunk, 4 * MK);
        }
      } else if constexpr (BV > 0) {
        if (slot >= 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint32_t idx = 0;
#pragma unroll
            for (int b = 0; b < (1 << BV) - 1; ++b) idx += (y[r] >= cb[3][b]) ? 1u : 0u;
            put_vcode<BV>(reinterpret_cast<uint32_t*>(a.v_idx + ((plane * vblocks + slot / kVBlock) * D + row + r) *
                                                               (4 * BV)),
                          int(slot % kVBlock), idx);
          }
        }
      }
    }
  }
  __syncthreads();

  // ---------------- key residual norm and QJL signs
  if constexpr (MK > 0) {
    // Residual norms: wave w reduces item w.
    {
      const float r0 = rs[wave][lane], r1 = rs[wave][lane + 64];
      const float ss = wave_sum(fmaf(r0, r0, r1 * r1));
      if (lane == 0) rnrm[wave] = nrm[wave] * sqrtf(ss);
    }
    // z = (S Pi^T)(y - c[idx]) for columns col < 8; bit = [n z >= 0].  The
    // residual (times 2^14) is split into a high part and a remainder.
    const int it = col & (kAppendItems - 1);
    floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 mh, ml, rh, rl;
      {
        const float v[8] = {ma[2 * s].x, ma[2 * s].y, ma[2 * s].z, ma[2 * s].w,
                            ma[2 * s + 1].x, ma[2 * s + 1].y, ma[2 * s + 1].z, ma[2 * s + 1].w};
        split8(v, mh, ml, true);
      }
      {
        const float4 x0 = *reinterpret_cast<const float4*>(&rs[it][32 * q + 8 * s]);
        const float4 x1 = *reinterpret_cast<const float4*>(&rs[it][32 * q + 8 * s + 4]);
        const float v[8] = {x0.x * 16384.f, x0.y * 16384.f, x0.z * 16384.f, x0.w * 16384.f,
                            x1.x * 16384.f, x1.y * 16384.f, x1.z * 16384.f, x1.w * 16384.f};
        split8(v, rh, rl, true);
      }
      a1 = mfma16x16x32(mh, rh, a1);
      a2 = mfma16x16x32(mh, rl, a2);
      a2 = mfma16x16x32(ml, rh, a2);
    }
    const float n = nrm[it];
    if (col < kAppendItems && it < ni) {
      uint32_t bits = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) bits |= (fmaf(a2[r], 0x1p-11f, a1[r]) * n >= 0.f ? 1u : 0u) << r;
      atomicOr(&srec[it][row >> 5], bits << (row & 31));
    }
  }
  __syncthreads();

  // ---------------- records: per item, code words [0, 4 MK), sign words
  // [SB, SB + 4), then the three norms
  constexpr int NE = MK > 4 ? 64 : 32, SB = MK > 4 ? 32 : 16;
  for (int e = tid; e < kAppendItems * NE; e += kAppendThreads) {
    const int it = e / NE, w = e % NE;
    const int64_t slot = slot_of[it];
    if (it >= ni || slot < 0) continue;
    const int64_t plane = int64_t(layer) * a.H + (item0 + it) % a.H;
    const int64_t rec = plane * a.capacity + slot;
    auto st32 = [](uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    auto stf = [](float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    if constexpr (MK > 0) {
      if (w < 4 * MK) st32(reinterpret_cast<uint32_t*>(a.k_idx + rec * (16 * MK)) + w, krec[it][w]);
      if (w >= SB && w < SB + 4) st32(reinterpret_cast<uint32_t*>(a.k_sign + rec * 16) + (w - SB), srec[it][w - SB]);
      if (w == SB + 4) stf(a.k_norm + rec, nrm[it]);
      if (w == SB + 5) stf(a.k_rnorm + rec, rnrm[it]);
    }
    if constexpr (BV > 0) {
      if (w == SB + 6) stf(a.v_norm + rec, nrm[kAppendItems + it]);
    }
  }
  if constexpr (MK == 0 || BV == 0) {
    for (int e = tid; e < kAppendItems * D; e += kAppendThreads) {
      const int it = e >> 7, j = e & 127;
      const int64_t slot = slot_of[it];
      if (it >= ni || slot < 0) continue;
      const int64_t plane = int64_t(layer) * a.H + (item0 + it) % a.H;
      if constexpr (MK == 0)
        __hip_atomic_store(a.k_f16 + (plane * a.capacity + slot) * D + j, f16_bits(xs[it][j]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if constexpr (BV == 0)
        __hip_atomic_store(a.v_f16 + ((plane * vblocks + slot / kVBlock) * D + j) * kVBlock + slot % kVBlock,
                           f16_bits(xs[kAppendItems + it][j]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (done != nullptr) {
    // every wave's stores and atomics complete, then the count (an agent-scope
    // release fence would also write back the XCD's whole L2)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(done + layer, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
template <int MK, int BV>
__global__ __launch_bounds__(kAppendThreads) void compress_append_kernel(CompressArgs a) {
  __shared__ AppendSmem sm;
  append_body<MK, BV>(a, blockIdx.x, blockIdx.y, sm);
}

// ===========================================================================
// Decode

struct DecodeArgs {
  int n_layers, batch, H, Hq, G, n_hg;
  int64_t capacity;
  int chunks_per_problem;   // 32-token chunks per problem (from max_len)
  int chunks_per_wg;        // chunks of every workgroup but the last
  int total_chunks;         // problems x chunks_per_problem
  int seg_max;              // partial slots per query head (the row stride of `partial`)
  // Ragged split (ragged != 0, in-kernel merge only): when the sequences'
  // chunks that hold tokens are fewer than problems x cpp_real, the decode
  // workgroups share those chunks instead, in equal ranges of at least
  // cpw_min (the ranges then never reach the chunks past a sequence's end).
  int ragged, cpp_real, cpw_min;
  int seg_base;             // first slot of this call's pieces
  const uint8_t* k_idx;
  const uint8_t* k_sign;
  const float* k_norm;
  const float* k_rnorm;
  const uint16_t* k_f16;
  const uint8_t* v_idx;
  const float* v_norm;
  const uint16_t* v_f16;
  const float* qprep;   // [L][B][Hq][2][D]
  const float* kc;
  const float* vc;
  const int64_t* seq_start;
  const int32_t* seq_len;
  float* partial;       // [L][B][Hq][seg_max][D + 2]
  float alpha_k, alpha_v;   // the operand scales of the centroid tables (1 = plain fp16 rounding)
  float* red_g;         // per decode workgroup [8 waves][8 heads][D] fp32: the wave merge, when not in LDS
  float* logits;        // score mode: [L][B][Hq][max_len]
  // In-kernel merge (non-null `done`): per problem, the count of its pieces
  // whose partial is written; the workgroup that completes the count merges
  // them into out [L][B][Hq][D] (Pi^T applied for rotated values) and sets the
  // count back to zero.
  uint32_t* done;
  const float* pi;
  float* out;
  int64_t max_len;
  float scale;
  float kappa;
  // Append in the same launch (n_app > 0): workgroups [0, n_app) compress the
  // call's new tokens (app_groups per layer, layers [app_layer0, app_layer0 +
  // app_layers) of the cache) and count themselves in app_done[layer]; a
  // decode wave about to load a chunk that holds one of the plane slots
  // [app_lo, app_hi) of an appended layer first waits for that count.  With a
  // slot list (the append's slots) the range is taken per sequence instead:
  // from the first to the last listed slot inside the sequence's slots.
  int n_app, app_groups, app_layer0, app_layers;
  // The wait is bounded: after app_polls polls of the count (each followed by
  // a short sleep) the wave sets *app_flag (a sticky word of the workspace,
  // zeroed by the call's query preparation) and goes on.  app_extra (0 but in
  // tests) raises the count waited for, so that the wait cannot be met.
  uint32_t app_polls;
  int app_extra;
  uint32_t* app_flag;
  int64_t app_lo, app_hi;
  uint32_t* app_done;
  // In-kernel merge over a second piece set (tail_cpp > 0): the pieces of a
  // decode over an fp16 tail of the same sequences, written by an earlier
  // launch into the slots from tail_base on (its split: tail_cpp chunks per
  // problem, tail_cpw per workgroup); fp16 values accumulate as stored, so
  // with rotated values their part is added after Pi^T.
  int tail_base, tail_cpp, tail_cpw;
};

// DPP row broadcast: every lane of a 16-lane row reads lane E of its row.
template <int E>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + E, 0xF, 0xF, true));
}
template <int B>
__device__ __forceinline__ void row_bcast8(float v, float (&o)[8]) {
  o[0] = row_bcast<B + 0>(v); o[1] = row_bcast<B + 1>(v); o[2] = row_bcast<B + 2>(v); o[3] = row_bcast<B + 3>(v);
  o[4] = row_bcast<B + 4>(v); o[5] = row_bcast<B + 5>(v); o[6] = row_bcast<B + 6>(v); o[7] = row_bcast<B + 7>(v);
}

// LDS lookup tables: a group of NG codes indexes an entry of NG fp16
// centroids.  Group sizes: m = 1: 8 codes (byte index), m = 2: 4 codes (byte
// index), m = 3: 2 codes (6-bit index), m = 4: 2 codes (byte index).  With
// HILO each entry holds the fp16 rounding c_hi of the NG centroids followed by
// the fp16 rounding of the remainders c - c_hi, so one LDS read yields both
// halves of a two-term fp16 representation (about 22 significant bits).
template <int M, bool HILO> struct Lut {
  static constexpr int NG = M == 1 ? 8 : (M == 2 ? 4 : 2);
  static constexpr int ENTRIES = 1 << (NG * M);
  static constexpr int ENTRY_WORDS = (NG / 2) * (HILO ? 2 : 1);
  static constexpr int WORDS = ENTRIES * ENTRY_WORDS;
};

// Centroid k of a codebook held one entry per lane (lane l holds entry
// l mod n, n a power of two): a cross-lane read, so every lane of the wave
// must be active.
__device__ __forceinline__ float lane_cent(float cl, int k) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(k << 2, __float_as_int(cl)));
}

// The table builders below run over whole waves (their trip counts are
// uniform and a wave with no entry left skips as a unit) because they read the
// codebook with lane_cent.
template <int M, bool HILO>
__device__ __forceinline__ void build_lut(uint32_t* lut, float cl, int tid, int nt = 256) {
  using L = Lut<M, HILO>;
  for (int x0 = 0; x0 < L::ENTRIES; x0 += nt) {
    if (x0 + (tid & ~63) >= L::ENTRIES) break;
    const int x = x0 + tid;
#pragma unroll
    for (int e = 0; e < L::NG; e += 2) {
      const float c0 = lane_cent(cl, (x >> (e * M)) & ((1 << M) - 1));
      const float c1 = lane_cent(cl, (x >> ((e + 1) * M)) & ((1 << M) - 1));
      const _Float16 h0 = _Float16(c0), h1 = _Float16(c1);
      uint16_t b0, b1;
      __builtin_memcpy(&b0, &h0, 2);
      __builtin_memcpy(&b1, &h1, 2);
      if (x < L::ENTRIES) lut[x * L::ENTRY_WORDS + e / 2] = uint32_t(b0) | (uint32_t(b1) << 16);
      if constexpr (HILO) {
        const uint32_t l0 = f16_bits(c0 - float(h0)), l1 = f16_bits(c1 - float(h1));
        if (x < L::ENTRIES) lut[x * L::ENTRY_WORDS + L::NG / 2 + e / 2] = l0 | (l1 << 16);
      }
    }
  }
}

// 8 consecutive m-bit codes (LSB-first in `bits`) -> 8 fp16 centroids.
template <int M>
__device__ __forceinline__ half8 deq8(uint32_t bits, const uint32_t* lut) {
  u32x4 w;
  if constexpr (M == 1) {
    w = *reinterpret_cast<const u32x4*>(lut + (bits & 0xFFu) * 4);
  } else if constexpr (M == 2) {
    u32x2 a0 = *reinterpret_cast<const u32x2*>(lut + (bits & 0xFFu) * 2);
    u32x2 a1 = *reinterpret_cast<const u32x2*>(lut + ((bits >> 8) & 0xFFu) * 2);
    w = u32x4{a0[0], a0[1], a1[0], a1[1]};
  } else if constexpr (M == 3) {
    w = u32x4{lut[bits & 63u], lut[(bits >> 6) & 63u], lut[(bits >> 12) & 63u], lut[(bits >> 18) & 63u]};
  } else {
    w = u32x4{lut[bits & 0xFFu], lut[(bits >> 8) & 0xFFu], lut[(bits >> 16) & 0xFFu], lut[bits >> 24]};
  }
  return as_half8(w);
}

// Key tables.  A key code group of NC codes (NC m = 12 bits for m = 3, 8
// bits otherwise) indexes one table entry holding its NC centroids as fp16
// MFMA operands, so each lookup lands straight in an operand (8 consecutive
// coordinates = 8 / NC entries), with no repacking.  Two representations
// (key_split): up to 2 Lloyd-Max bits, one fp16 value per centroid, the
// codebook scaled by alpha_k (exact to about 2^-20 for such codebooks); 3 or
// more bits, an fp16 high part and an fp16 remainder per centroid (HILO),
// the entry holding the NC high parts, then the NC remainders (measured: one
// table of such entries is faster than separate high and remainder tables).
// The NC-code table is assembled from a two-code pair table.
template <int M> struct KLut {
  static constexpr bool HILO = M >= 3;
  static constexpr int NC = M == 1 ? 8 : (M == 4 ? 2 : 4);  // codes per entry
  static constexpr int E = 1 << (NC * M);                   // entries
  static constexpr int H = NC / 2;                          // dwords of one part (high or remainder)
  static constexpr int EW = H * (HILO ? 2 : 1);             // dwords per entry
  static constexpr int PAIRS = 1 << (2 * M);                // two-code pair entries
  static constexpr int PW = HILO ? 2 : 1;                   // dwords per pair entry (high, remainder)
};

// Pair table: entry x (two codes, x = c0 | c1 << M) = fp16 pair (c0, c1),
// then (HILO) the fp16 pair of their remainders.  cl: lane l holds centroid
// l mod 2^M (already scaled by alpha_k where the keys are scaled).
template <int M>
__device__ __forceinline__ void build_kpairs(uint32_t* phi, float cl, int tid, int nt = 256) {
  using K = KLut<M>;
  constexpr int P = K::PAIRS;
  for (int x0 = 0; x0 < P; x0 += nt) {
    if (x0 + (tid & ~63) >= P) break;
    const int x = x0 + tid;
    const float c0 = lane_cent(cl, x & ((1 << M) - 1)), c1 = lane_cent(cl, (x >> M) & ((1 << M) - 1));
    const uint16_t h0 = f16_bits(c0), h1 = f16_bits(c1);
    if (x < P) {
      phi[x * K::PW] = uint32_t(h0) | (uint32_t(h1) << 16);
      if constexpr (K::HILO) {
        const float r0 = c0 - float(__builtin_bit_cast(_Float16, h0)), r1 = c1 - float(__builtin_bit_cast(_Float16, h1));
        phi[x * K::PW + 1] = uint32_t(f16_bits(r0)) | (uint32_t(f16_bits(r1)) << 16);
      }
    }
  }
}
// NC-code table from the pair table (after a barrier): high dword k of entry
// x is the pair of codes 2k, 2k + 1 (remainder dword k likewise, after the
// high ones).  Thread t of NT writes entries t + NT u; all its pair-table
// reads are issued before its writes.
template <int M, int NT = 256>
__device__ __forceinline__ void build_ktab(uint32_t* khi, const uint32_t* phi, int tid) {
  using K = KLut<M>;
  static_assert(K::E % NT == 0 || NT % K::E == 0, "key table entries per thread");
  constexpr int U = (K::E + NT - 1) / NT;
  constexpr int H = K::H;   // pairs per entry
  if (K::E < NT && tid >= K::E) return;
  uint32_t w[U][K::EW];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const int pr = ((tid + NT * u) >> (2 * M * k)) & (K::PAIRS - 1);
      w[u][k] = phi[pr * K::PW];
      if constexpr (K::HILO) w[u][H + k] = phi[pr * K::PW + 1];
    }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t* dst = khi + (tid + NT * u) * K::EW;
    if constexpr (K::EW == 1) {
      *dst = w[u][0];
    } else if constexpr (K::EW == 2) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{w[u][0], w[u][1]};
    } else {
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[u][0], w[u][1], w[u][2], w[u][3]};
    }
  }
}

// 8 consecutive m-bit key codes (LSB-first in `bits`) -> 8 fp16 centroids
// (hi), and for split keys their remainders (lo).
template <int M>
__device__ __forceinline__ void deq8_k(uint32_t bits, const uint32_t* khi, half8& hi, half8& lo) {
  if constexpr (M == 1) {
    hi = as_half8(*reinterpret_cast<const u32x4*>(khi + (bits & 0xFFu) * 4));
  } else if constexpr (M == 4) {
    // two-code entries (high pair, remainder pair), one per code byte; each
    // dword read on its own so that it lands in its operand register
    const uint32_t* e0 = khi + (bits & 0xFFu) * 2;
    const uint32_t* e1 = khi + ((bits >> 8) & 0xFFu) * 2;
    const uint32_t* e2 = khi + ((bits >> 16) & 0xFFu) * 2;
    const uint32_t* e3 = khi + (bits >> 24) * 2;
    hi = as_half8(u32x4{e0[0], e1[0], e2[0], e3[0]});
    lo = as_half8(u32x4{e0[1], e1[1], e2[1], e3[1]});
  } else if constexpr (M == 3) {
    // four-code entries: 4 high parts, 4 remainders; each half read on its
    // own so that it lands in its operand registers
    const uint32_t* e0 = khi + (bits & 0xFFFu) * 4;
    const uint32_t* e1 = khi + ((bits >> 12) & 0xFFFu) * 4;
    const u32x2 h0 = *reinterpret_cast<const u32x2*>(e0), h1 = *reinterpret_cast<const u32x2*>(e1);
    const u32x2 l0 = *reinterpret_cast<const u32x2*>(e0 + 2), l1 = *reinterpret_cast<const u32x2*>(e1 + 2);
    hi = as_half8(u32x4{h0[0], h0[1], h1[0], h1[1]});
    lo = as_half8(u32x4{l0[0], l0[1], l1[0], l1[1]});
  } else {
    const u32x2 h0 = *reinterpret_cast<const u32x2*>(khi + (bits & 0xFFu) * 2);
    const u32x2 h1 = *reinterpret_cast<const u32x2*>(khi + ((bits >> 8) & 0xFFu) * 2);
    hi = as_half8(u32x4{h0[0], h0[1], h1[0], h1[1]});
  }
}

// 8 consecutive m-bit key codes, m > 4 (bits [8 m s, 8 m s + 8 m) of a
// lane's 32-coordinate slab of m dwords) -> 8 fp16 centroids and their
// remainders from the 2^m-entry fp16 tables (high parts, then remainders):
// one lookup per code and part (a table of code pairs would not fit beside
// the value tables).
template <int M, int N>
__device__ __forceinline__ void deq8_wide(const uint32_t (&w)[N], int s, const uint16_t* lut, half8& hi,
                                          half8& lo) {
  constexpr uint32_t mask = (1u << M) - 1u;
  uint32_t h[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = 8 * M * s + M * j, lo_w = p >> 5, sh = p & 31;
    const uint32_t c =
        sh + M <= 32 ? (w[lo_w] >> sh) & mask
                     : __builtin_amdgcn_alignbit(w[lo_w + 1 < N ? lo_w + 1 : lo_w], w[lo_w], sh) & mask;
    h[j] = lut[c];
    l[j] = lut[(1 << M) + c];
  }
  hi = as_half8(u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
  lo = as_half8(u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)});
}

// Bits [8 m s, 8 m s + 8 m) of a lane's 32-coordinate slab (m dwords).
template <int M, int N>
__device__ __forceinline__ uint32_t slab_bits(const uint32_t (&w)[N], int s) {
  if constexpr (M == 1) return (w[0] >> (8 * s)) & 0xFFu;
  else if constexpr (M == 2) return (w[s >> 1] >> (16 * (s & 1))) & 0xFFFFu;
  else if constexpr (M == 3) {
    // 24-bit windows of the 96-bit slab (funnel shifts of adjacent words)
    if (s == 0) return w[0] & 0xFFFFFFu;
    if (s == 1) return __builtin_amdgcn_alignbit(w[1], w[0], 24) & 0xFFFFFFu;
    if (s == 2) return __builtin_amdgcn_alignbit(w[2], w[1], 16) & 0xFFFFFFu;
    return w[2] >> 8;
  } else return w[s];
}

// Lane-private value table for 4-bit values: entry e (two codes) of lane l's
// copy sits at byte e * 256 + 4 l, so the 64 lanes of a lookup always hit 64
// different banks.  One byte permute forms the address from the code byte and
// the lane offset; `lane4` holds 4 l in byte 0 and the table's 64 KB page in
// byte 2, so that a table placed past the first 64 KB of LDS is still
// addressed by that one permute plus the instruction's immediate offset.
__device__ __forceinline__ void build_vrep(uint32_t* lut, float cl, int tid, int nt) {
  for (int x = tid; x < 256 * 16; x += nt) {   // entry x / 16, copies 4 (x % 16) .. + 3 (nt divides 4096)
    const int e = x >> 4;
    const uint32_t w = uint32_t(f16_bits(lane_cent(cl, e & 15))) | (uint32_t(f16_bits(lane_cent(cl, e >> 4))) << 16);
    *reinterpret_cast<u32x4*>(lut + e * 64 + (x & 15) * 4) = u32x4{w, w, w, w};
  }
}
// The 2-bit value table in 32 lane-private copies (64 KB): entry e (a byte of
// four codes) holds their four alpha-scaled fp16 centroids (8 bytes) in copy c
// at byte e * 256 + 8 c; lanes l and l + 32 share a copy, and the 16 lanes of
// a read pass hit 16 different copies.
__device__ __forceinline__ void build_vrep2(uint32_t* lut, float cl, int tid, int nt) {
  for (int x = tid; x < 256 * 16; x += nt) {   // entry x / 16, copies 2 (x % 16) and 2 (x % 16) + 1
    const int e = x >> 4;
    const uint32_t w0 = uint32_t(f16_bits(lane_cent(cl, e & 3))) | (uint32_t(f16_bits(lane_cent(cl, (e >> 2) & 3))) << 16);
    const uint32_t w1 = uint32_t(f16_bits(lane_cent(cl, (e >> 4) & 3))) | (uint32_t(f16_bits(lane_cent(cl, e >> 6))) << 16);
    *reinterpret_cast<u32x4*>(lut + e * 64 + (x & 15) * 4) = u32x4{w0, w1, w0, w1};
  }
}
// Two bytes of code word `bits` (the byte selectors s0 and s1, per lane) ->
// 8 fp16 centroids; each address is one byte permute: byte 0 = 8 (lane % 32),
// byte 1 = the code byte, byte 2 = the table's 64 KB page (in lane8) or zero.
__device__ __forceinline__ half8 deq8_vrep2(uint32_t bits, uint32_t lane8, uint32_t s0, uint32_t s1,
                                            const unsigned char* base) {
  const uint32_t a0 = __builtin_amdgcn_perm(bits, lane8, s0);
  const uint32_t a1 = __builtin_amdgcn_perm(bits, lane8, s1);
  const u32x2 w0 = *reinterpret_cast<const u32x2*>(base + a0), w1 = *reinterpret_cast<const u32x2*>(base + a1);
  return as_half8(u32x4{w0[0], w0[1], w1[0], w1[1]});
}
template <bool PAGE>
__device__ __forceinline__ half8 deq8_vrep(uint32_t bits, uint32_t lane4, const unsigned char* base) {
  // byte 0 of the address: 4 lane; byte 1: code byte k; byte 2: the page (PAGE) or zero; byte 3: zero
  constexpr uint32_t b2 = PAGE ? 0x00020000u : 0x000C0000u;
  const uint32_t a0 = __builtin_amdgcn_perm(bits, lane4, 0x0C000400u | b2);
  const uint32_t a1 = __builtin_amdgcn_perm(bits, lane4, 0x0C000500u | b2);
  const uint32_t a2 = __builtin_amdgcn_perm(bits, lane4, 0x0C000600u | b2);
  const uint32_t a3 = __builtin_amdgcn_perm(bits, lane4, 0x0C000700u | b2);
  return as_half8(u32x4{*reinterpret_cast<const uint32_t*>(base + a0), *reinterpret_cast<const uint32_t*>(base + a1),
                        *reinterpret_cast<const uint32_t*>(base + a2), *reinterpret_cast<const uint32_t*>(base + a3)});
}

// LDS layout of a decode workgroup of format <MK, BV> (see decode_body).
template <int MK, int BV, bool SCORE>
struct DecodeLayout {
  static constexpr bool KWIDE = MK > 4;   // 7-bit codes: one fp16 table entry per code (high parts, then remainders)
  using KL = KLut<(MK > 0 && !KWIDE ? MK : 1)>;
  static constexpr int KT = MK > 0 ? (KWIDE ? (1 << MK) : KL::E * KL::EW) : 1;   // key table dwords
  static constexpr int KP = MK > 0 && !KWIDE && KL::NC > 2 ? KL::PAIRS * KL::PW : 1;   // pair-table dwords (if separate)
  static constexpr int RED_FULL = kDecodeWaves * kMaxGroup * D * 4;
  static constexpr int LIVE_BYTES = (kRaggedMaxBatch + 1) * 4;
  static constexpr int MISC_BYTES = kDecodeWaves * 128 * 4 + 2 * kDecodeWaves * 16 * 4 + 2 * 2 * 4 * 64 * 16 + 16 + LIVE_BYTES;
  // Lane-private value table (64 KB): 4-bit values always; 2-bit values when
  // it fits beside the key tables with the wave merge still in LDS.
  static constexpr bool VREP2 =
      BV == 2 && (MK > 0 ? 256 * 16 : 0) + (KT + KP) * 4 + 1024 + 256 * 64 * 4 + RED_FULL + MISC_BYTES <= 160 * 1024;
  static constexpr bool VREP = BV == 4 || VREP2;
  static constexpr int VW = VREP ? 256 * 64 : (BV > 0 ? Lut<BV, false>::WORDS : 1);
  // Tables first, each starting below 64 KB so that lookups carry the table
  // offset as an instruction immediate (the lane-private value table may
  // start past 64 KB: its addresses carry the page, see deq8_vrep).
  // Order: signs, then the small value tables (1 bit, or 2 bits when not
  // lane-private), the key table and its pair table, then the lane-private
  // value table (4 bits, or 2 bits when it fits).
  static constexpr int OFF_S = 0;
  static constexpr int S_END = MK > 0 ? 256 * 16 : 0;
  static constexpr int OFF_K = VREP ? S_END : ((S_END + VW * 4 + 255) / 256) * 256;
  static constexpr int OFF_PHI = OFF_K + KT * 4;   // read only while the key table is built
  static constexpr int OFF_V = VREP ? ((OFF_PHI + KP * 4 + 255) / 256) * 256 : S_END;
  static constexpr int V_PAGE = VREP && OFF_V >= 65536 ? 1 : 0;
  static constexpr int OFF_TAB_END = VREP ? ((OFF_V + VW * 4 + 15) / 16) * 16 : ((OFF_PHI + KP * 4 + 15) / 16) * 16;
  // The wave merge ([wave][head][coordinate] fp32) stays in LDS when the
  // tables leave room for it, else it goes through the workgroup's slice of
  // the workspace (L2).
  static constexpr bool RED_LDS = !SCORE && OFF_TAB_END + RED_FULL + MISC_BYTES <= 160 * 1024;
  static constexpr int OFF_RED = OFF_TAB_END;
  static constexpr int RED_BYTES = RED_LDS ? RED_FULL : 0;
  // Without room for it, a workgroup's last group holds the wave merge over a
  // table it no longer needs (the key table, else the lane-private value
  // table) when that holds its 32 KB; earlier groups use the workspace.
  static constexpr int OFF_OVL = !RED_LDS && !SCORE ? (KT * 4 >= RED_FULL ? OFF_K : (VREP ? OFF_V : -1)) : -1;
  static constexpr bool OVL = OFF_OVL >= 0;
  static constexpr int OFF_NX = OFF_RED + RED_BYTES;
  static constexpr int OFF_MW = OFF_NX + kDecodeWaves * 128 * 4;
  static constexpr int OFF_LW = OFF_MW + kDecodeWaves * 16 * 4;
  static constexpr int OFF_Q = OFF_LW + kDecodeWaves * 16 * 4;    // staged query operands [piece][r / z][s][lane]
  static constexpr int OFF_CNT = OFF_Q + 2 * 2 * 4 * 64 * 16;
  static constexpr int OFF_LIVE = OFF_CNT + 16;   // ragged split: prefix of the sequences' live chunk counts
  static constexpr int LDS_BYTES = OFF_LIVE + LIVE_BYTES;
  static_assert(OFF_K < 65536, "the key table must start below 64 KB");
  static_assert(VREP ? OFF_V - V_PAGE * 65536 < 65536 : OFF_V < 65536, "value table offset");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
  static_assert(2 * 2 * 4 * 64 * 16 >= 2 * 16 * D * 4, "the in-kernel merge's result area fits the query staging");
};

// Decode / score kernel: one workgroup of 8 waves per CU.  Workgroup w owns
// the chunks [w * chunks_per_wg, ...) of the problem-major chunk sequence; it
// takes them in groups of at most two problems (pieces A and B).  Inside a
// group the waves draw chunks one at a time from an LDS ticket counter, A's
// chunks first, so waves that run faster take more chunks and all of them
// finish together.  Each wave keeps its own online-softmax state per piece;
// at the end of the group the wave states of a piece are merged in LDS, in
// wave order, into the piece's partial.
template <int MK, int BV, bool SCORE>
__device__ __forceinline__ void decode_body(DecodeArgs a, CompressArgs ca, unsigned char* const dsm,
                                            const int blk, const int nblk) {
  using LY = DecodeLayout<MK, BV, SCORE>;
  constexpr bool KWIDE = LY::KWIDE;
  constexpr bool KSPLIT = MK > 0 && key_split(MK);   // key centroids as fp16 high part + remainder
  using KL = typename LY::KL;
  constexpr int NT = kDecodeWaves * 64;
  [[maybe_unused]] constexpr auto KT = LY::KT;
  [[maybe_unused]] constexpr auto KP = LY::KP;
  [[maybe_unused]] constexpr auto VREP = LY::VREP;
  [[maybe_unused]] constexpr auto VW = LY::VW;
  [[maybe_unused]] constexpr auto OFF_S = LY::OFF_S;
  [[maybe_unused]] constexpr auto S_END = LY::S_END;
  [[maybe_unused]] constexpr auto OFF_K = LY::OFF_K;
  [[maybe_unused]] constexpr auto OFF_PHI = LY::OFF_PHI;
  [[maybe_unused]] constexpr auto OFF_V = LY::OFF_V;
  [[maybe_unused]] constexpr auto V_PAGE = LY::V_PAGE;
  [[maybe_unused]] constexpr auto OFF_TAB_END = LY::OFF_TAB_END;
  [[maybe_unused]] constexpr auto LIVE_BYTES = LY::LIVE_BYTES;
  [[maybe_unused]] constexpr auto MISC_BYTES = LY::MISC_BYTES;
  [[maybe_unused]] constexpr auto RED_FULL = LY::RED_FULL;
  [[maybe_unused]] constexpr auto RED_LDS = LY::RED_LDS;
  [[maybe_unused]] constexpr auto OVL = LY::OVL;
  [[maybe_unused]] constexpr auto VREP2 = LY::VREP2;
  [[maybe_unused]] constexpr auto OFF_RED = LY::OFF_RED;
  [[maybe_unused]] constexpr auto RED_BYTES = LY::RED_BYTES;
  [[maybe_unused]] constexpr auto OFF_NX = LY::OFF_NX;
  [[maybe_unused]] constexpr auto OFF_MW = LY::OFF_MW;
  [[maybe_unused]] constexpr auto OFF_LW = LY::OFF_LW;
  [[maybe_unused]] constexpr auto OFF_Q = LY::OFF_Q;
  [[maybe_unused]] constexpr auto OFF_CNT = LY::OFF_CNT;
  [[maybe_unused]] constexpr auto OFF_LIVE = LY::OFF_LIVE;
  [[maybe_unused]] constexpr auto LDS_BYTES = LY::LDS_BYTES;
  uint32_t* const lut_k = reinterpret_cast<uint32_t*>(dsm + OFF_K);
  uint32_t* const pair_hi = reinterpret_cast<uint32_t*>(dsm + OFF_PHI);
  uint32_t* const lut_s = reinterpret_cast<uint32_t*>(dsm + OFF_S);
  uint32_t* const lut_v = reinterpret_cast<uint32_t*>(dsm + OFF_V);
  const unsigned char* const vrep_base = dsm + OFF_V - V_PAGE * 65536;
  float* const red = reinterpret_cast<float*>(dsm + OFF_RED);   // [wave][head][coordinate] (RED_LDS)
  float* const nxch = reinterpret_cast<float*>(dsm + OFF_NX);
  float(*const mw)[16] = reinterpret_cast<float(*)[16]>(dsm + OFF_MW);
  float(*const lw)[16] = reinterpret_cast<float(*)[16]>(dsm + OFF_LW);
  uint32_t* const counter = reinterpret_cast<uint32_t*>(dsm + OFF_CNT);
  int* const live_s = reinterpret_cast<int*>(dsm + OFF_LIVE);
  half8* const qstage = reinterpret_cast<half8*>(dsm + OFF_Q);
  // the in-kernel merge's result area ([16][D] heads, [16][D] the tail's part)
  float* const fin = RED_LDS ? red : reinterpret_cast<float*>(dsm + OFF_Q);
  static_assert(LDS_BYTES >= int(sizeof(AppendSmem)), "the append role reuses the decode LDS");
  if constexpr (!SCORE) {
    // append workgroups first (lowest indices, so they are dispatched first and
    // never wait behind decode workgroups that wait for them)
    if (blk < a.n_app) {
      append_body<MK, BV>(ca, blk % a.app_groups, blk / a.app_groups,
                          *reinterpret_cast<AppendSmem*>(dsm), a.app_done);
      return;
    }
  }
  // Decode workgroup, XCD-aware: workgroups are dispatched to the 8 XCDs
  // round robin, so physical decode index i runs on the XCD of i % 8; logical
  // index j gives each XCD one contiguous range of the chunk sequence (both
  // pieces of a problem, and the problems of a layer, share an L2).
  int wg;
  {
    const int i = blk - a.n_app, nd = nblk - a.n_app;
    const int r = i & 7, qd = nd >> 3, rem = nd & 7;
    wg = r * qd + (r < rem ? r : rem) + (i >> 3);
  }
  // this workgroup's slice of the workspace for the wave merge (when not in LDS)
  float* const red_wg = RED_LDS ? nullptr : a.red_g + int64_t(wg) * (kDecodeWaves * kMaxGroup * D);
  // the wave merge over a dead table (last group only, see DecodeLayout)
  float* const red_ov = OVL ? reinterpret_cast<float*>(dsm + (OVL ? LY::OFF_OVL : 0)) : nullptr;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, q = lane >> 4;   // MFMA column (head / coordinate) and k-group
  const bool lo_half = col >= 8;
  const uint32_t lane4 = uint32_t(lane) * 4 | uint32_t(V_PAGE << 16);
  // 2-bit values (VREP2): lane (col, q) reads code bytes 2 (q % 2) and 2 (q % 2) + 1
  // of its word (tokens 8 q .. 8 q + 3 and 8 q + 4 .. 8 q + 7)
  const uint32_t lane8 = uint32_t(lane & 31) * 8 | uint32_t(V_PAGE << 16);
  const uint32_t vsel0 = 0x0C000000u | (V_PAGE ? 0x00020000u : 0x000C0000u) | ((4u + 2u * (q & 1)) << 8);
  const uint32_t vsel1 = vsel0 + 0x100u;

  // Scores are kept in base-2 units (scaled by log2 e) so that the softmax
  // weights are plain exp2; tq_score writes natural-unit logits.
  constexpr float kLog2e = 1.4426950408889634f;
  const float kscale = SCORE ? a.scale : a.scale * kLog2e;
  const float kscale_r = kscale * a.kappa;
  // Operand scales of the centroid tables (see fp16_operand_scale): keys of
  // <= 2 Lloyd-Max bits and every value table are held as fp16(alpha c); the
  // rotated query carries 1 / alpha_k, the accumulated values 1 / alpha_v.
  constexpr bool KSCALED = MK > 0 && !KSPLIT;
  const float alpha_k = KSCALED ? a.alpha_k : 1.f;
  const float alpha_v = BV > 0 && !SCORE ? a.alpha_v : 1.f;
  const float kscale_k = kscale / alpha_k;
  const float inv_alpha_v = 1.f / alpha_v;
  constexpr int KREC = MK > 0 ? 16 * MK : 2 * D;   // bytes per key code record
  constexpr int MKW = MK > 0 ? MK : 1;
  constexpr bool kPrefetch = !SCORE;
  const int cpp = a.chunks_per_problem;
  const int64_t vblocks = a.capacity / kVBlock;

  // ---- the chunk sequence dealt to the workgroups in ranges of cpw: every
  // problem's cpp chunks, problem-major; or (rag) only the chunks that hold
  // tokens, each problem followed by chunks of padding (never dealt: they
  // stand for the cost of a problem change in a workgroup, kRaggedCrossChunks,
  // plus for a problem shorter than the mean range w0 the cost of the second
  // group that a range holding it whole takes, kContainChunks (w0 - live) /
  // w0): problem p = ((layer * batch + b) * H + hk) * n_hg + hg has n(b) =
  // live(b) + padding chunks (0 for an empty sequence) from P(p) = layer * HG * S(B) +
  // HG * S(b) + (hk * n_hg + hg) * n(b), with HG = H * n_hg and S the prefix
  // of n (in LDS).
  // (All of it is uniform over the workgroup; values read from LDS are made
  // scalar with readfirstlane, so that the loops over chunks stay scalar.)
  bool rag = false;
  int cpw = a.chunks_per_wg, total = a.total_chunks;
  const int HG = a.H * a.n_hg;
  auto lds_s = [&](int b) -> int { return __builtin_amdgcn_readfirstlane(live_s[b]); };
  auto pcount = [&](int p) -> int {
    if (!rag) return cpp;
    const int b = (p / HG) % a.batch;
    return lds_s(b + 1) - lds_s(b);
  };
  auto pfirst = [&](int p) -> int {
    if (!rag) return p * cpp;
    const int lb = p / HG, b = lb % a.batch, layer = lb / a.batch;
    const int s0 = lds_s(b);
    return layer * HG * lds_s(a.batch) + HG * s0 + (p - lb * HG) * (lds_s(b + 1) - s0);
  };
  // the problem holding chunk c (c < total)
  auto prob_of = [&](int c) -> int {
    if (!rag) return c / cpp;
    const int per_layer = HG * lds_s(a.batch);
    const int layer = c / per_layer, r = c - layer * per_layer;
    int lo = 0, hi = a.batch;   // HG S(lo) <= r < HG S(hi): the last such lo has chunks
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (HG * lds_s(mid) <= r) lo = mid; else hi = mid;
    }
    const int s0 = lds_s(lo);
    return (layer * a.batch + lo) * HG + (r - HG * s0) / (lds_s(lo + 1) - s0);
  };
  // pieces (workgroup ranges) that meet problem p
  auto pieces_of = [&](int p) -> int {
    const int f = pfirst(p), n = pcount(p);
    return n > 0 ? (f + n - 1) / cpw - f / cpw + 1 : 0;
  };

  // ---- problem context: problem = ((layer * batch + b) * H + hk) * n_hg + hg
  struct Run {
    int64_t slot_base;   // slot of token 0 of the sequence in its (layer, KV head) plane
    int64_t vblk0;       // value block of token 0
    int64_t len;         // tokens of the sequence (clamped)
    int64_t start;       // plane-local slot of token 0
    int layer, b, hk, hg;
  };
  auto ctx_of = [&](int prob) {
    Run r{};
    r.hg = prob % a.n_hg;
    r.hk = (prob / a.n_hg) % a.H;
    r.b = (prob / (a.n_hg * a.H)) % a.batch;
    r.layer = prob / (a.n_hg * a.H * a.batch);
    return r;
  };
  // A sequence with an invalid start gets no tokens and slot 0 as its start,
  // so that the chunk-0 loads issued for waves without work stay in bounds.
  auto clamp_run = [&](int64_t& start, int64_t& len) {
    if (start < 0 || (start % kVBlock) != 0 || start >= a.capacity || len < 0) {
      len = 0;
      start = 0;
    }
    if (len > a.capacity - start) len = a.capacity - start;
    if (len > a.max_len) len = a.max_len;   // tokens past max_seq_len are ignored
  };
  auto fill_run = [&](Run r, int64_t start, int64_t len) {
    clamp_run(start, len);
    const int64_t plane = int64_t(r.layer) * a.H + r.hk;
    r.slot_base = plane * a.capacity + start;
    r.vblk0 = plane * vblocks + start / kVBlock;
    r.len = len;
    r.start = start;
    return r;
  };
  // A group: chunks [g0, b_end) of the workgroup's range, covering piece A
  // (problem pa from its chunk rel_a0) and, if has_b, piece B (problem pa + 1
  // from its chunk 0).  Tickets 0 .. live_a - 1 are A's chunks that hold
  // tokens, live_a .. n_tickets - 1 B's.
  struct Group {
    Run ra, rb;
    int64_t sa, sb, va, vb;   // ticket u's first slot: (u < live_a ? sa : sb) + 32 u; value block likewise + u
    int pa, pb, a_end, b_end, rel_a0, live_a, n_tickets;   // pb: piece B's problem (pa without a piece B)
    int xa0, xa1, xb0, xb1;   // tickets [xa0, xa1) (piece A), [xb0, xb1) (B) whose chunks may hold appended slots
    bool has_b;
  };
  // Tickets of a piece whose chunks (chunk c: plane slots start + 32 c ..
  // + 31) meet the appended slots, as [t0, t1) with ticket = c + shift,
  // within [lo, hi); empty unless the piece's layer is appended.
  auto app_tickets = [&](const Run& r, int shift, int lo, int hi, int& t0, int& t1) {
    t0 = 0;
    t1 = 0;
    if constexpr (!SCORE) {
      if (a.n_app == 0 || r.layer < a.app_layer0 || r.layer >= a.app_layer0 + a.app_layers) return;
      int64_t lo_s = a.app_lo, hi_s = a.app_hi;
      // (marked unlikely: laid out apart, the scan leaves the decode's code
      // for contiguous appends as it was)
      if (__builtin_expect(ca.slots != nullptr, 0)) {
        // the listed slots inside this sequence (one scan per piece and group;
        // a decode step's list holds a few tokens per sequence)
        lo_s = INT64_MAX;
        hi_s = 0;
        for (int64_t i = 0; i < ca.n_tokens; ++i) {
          const int64_t sl = ca.slots[i] + ca.slot_shift;
          if (sl >= r.start && sl < r.start + r.len) {
            lo_s = sl < lo_s ? sl : lo_s;
            hi_s = sl + 1 > hi_s ? sl + 1 : hi_s;
          }
        }
        if (hi_s == 0) return;   // none: no chunk of the piece waits
      }
      const int64_t c0 = lo_s - r.start > 0 ? (lo_s - r.start) / kChunk : 0;
      const int64_t c1 = hi_s - r.start > 0 ? (hi_s - r.start + kChunk - 1) / kChunk : 0;
      const int64_t u0 = c0 + shift, u1 = c1 + shift;
      t0 = int(u0 < lo ? lo : (u0 > hi ? hi : u0));
      t1 = int(u1 < lo ? lo : (u1 > hi ? hi : u1));
    }
  };
  auto group_of = [&](int g0, int c_last) {
    Group G;
    G.pa = prob_of(g0);
    const int fa = pfirst(G.pa);
    G.a_end = fa + pcount(G.pa) < c_last ? fa + pcount(G.pa) : c_last;
    G.has_b = G.a_end < c_last;
    G.pb = G.has_b ? prob_of(G.a_end) : G.pa;
    G.b_end = G.has_b ? (G.a_end + pcount(G.pb) < c_last ? G.a_end + pcount(G.pb) : c_last) : G.a_end;
    G.rel_a0 = g0 - fa;
    // both sequences' (start, length) are loaded together
    const Run ca = ctx_of(G.pa), cb = ctx_of(G.pb);
    const int64_t sa = a.seq_start[ca.b], sb = a.seq_start[cb.b];
    const int64_t la = a.seq_len[ca.b], lb = a.seq_len[cb.b];
    G.ra = fill_run(ca, sa, la);
    G.rb = fill_run(cb, sb, lb);
    int live_a = int((G.ra.len + kChunk - 1) / kChunk) - G.rel_a0;
    live_a = live_a < 0 ? 0 : (live_a > G.a_end - g0 ? G.a_end - g0 : live_a);
    int live_b = G.has_b ? int((G.rb.len + kChunk - 1) / kChunk) : 0;
    live_b = live_b > G.b_end - G.a_end ? G.b_end - G.a_end : live_b;
    G.live_a = live_a;
    G.n_tickets = live_a + live_b;
    G.sa = G.ra.slot_base + int64_t(G.rel_a0) * kChunk;
    G.sb = G.rb.slot_base - int64_t(live_a) * kChunk;
    G.va = G.ra.vblk0 + G.rel_a0;
    G.vb = G.rb.vblk0 - live_a;
    app_tickets(G.ra, -G.rel_a0, 0, live_a, G.xa0, G.xa1);
    app_tickets(G.rb, live_a, live_a, G.n_tickets, G.xb0, G.xb1);
    if (!G.has_b) G.xb0 = G.xb1 = 0;
    return G;
  };

  // Chunk of ticket u (< n_tickets) of group G: piece A's chunk rel_a0 + u,
  // or piece B's chunk u - live_a.
  auto slot_of = [&](const Group& G, int u) -> int64_t { return (u < G.live_a ? G.sa : G.sb) + int64_t(u) * kChunk; };
  auto vblk_of = [&](const Group& G, int u) -> int64_t { return (u < G.live_a ? G.va : G.vb) + u; };

  // Before the loads of ticket u's chunk: if the chunk may hold a slot that
  // this launch's append workgroups write, wait (once per piece and wave) for
  // the layer's append count, then acquire at agent scope so that the loads
  // see the new records.  Bounded: after app_polls polls (about a second by
  // default) the wave records the give-up in the workspace's flag word, which
  // the host reads with tq_decode_step_check, and goes on.
  bool app_ok_a = false, app_ok_b = false;
  auto gate = [&](const Group& G, int u) {
    if constexpr (!SCORE) {
      const bool in_xa = u >= G.xa0 && u < G.xa1 && !app_ok_a;
      const bool in_xb = u >= G.xb0 && u < G.xb1 && !app_ok_b;
      if (!(in_xa || in_xb)) return;
      const int layer = in_xa ? G.ra.layer : G.rb.layer;
      const uint32_t want = uint32_t(a.app_groups + a.app_extra);
      bool met = false;
      for (uint32_t spin = 0; spin < a.app_polls; ++spin) {
        if (__hip_atomic_load(a.app_done + layer, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) {
          met = true;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      if (!met && lane == 0) __hip_atomic_fetch_or(a.app_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      if (in_xa) app_ok_a = true; else app_ok_b = true;
    }
  };

  // ---- staged query operands (MFMA B operands), per piece: columns 0..7 are
  // the group's query heads as fp16 high parts, columns 8..15 the same heads
  // as fp16 remainders, so one MFMA forms both halves of every product; lanes
  // col and col ^ 8 then add their results (DPP row rotate by 8).  Lane (col,
  // q) of step s holds coordinates 32 q + 8 s + e of Pi q * scale (r) and of
  // S q * scale * kappa (z).  Each thread converts items tid and tid + NT of
  // the 1024 (piece, r / z, s, lane) operands.
  struct QItem {
    float v[2][8];
  };
  // pa, pb: problems of pieces A and B (pb = pa without a piece B).
  auto stage_load = [&](int pa, int pb, QItem& Q) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int it = tid + NT * u;
      const int piece = it >> 9, kind = (it >> 8) & 1, s4 = (it >> 6) & 3, l = it & 63;
      const Run Rp = ctx_of(piece ? pb : pa);
      const int g_local = Rp.hg * kMaxGroup + (l & 7);
      const int hh = Rp.hk * a.G + (g_local < a.G ? g_local : 0);
      const float4* src = reinterpret_cast<const float4*>(
          a.qprep + ((int64_t(Rp.layer) * a.batch + Rp.b) * a.Hq + hh) * 2 * D + kind * D + 32 * (l >> 4) + 8 * s4);
      const float4 x0 = src[0], x1 = src[1];
      Q.v[u][0] = x0.x; Q.v[u][1] = x0.y; Q.v[u][2] = x0.z; Q.v[u][3] = x0.w;
      Q.v[u][4] = x1.x; Q.v[u][5] = x1.y; Q.v[u][6] = x1.z; Q.v[u][7] = x1.w;
    }
  };
  auto stage_store = [&](int pa, int pb, const QItem& Q) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int it = tid + NT * u;
      const int piece = it >> 9, kind = (it >> 8) & 1, l = it & 63;
      const Run Rp = ctx_of(piece ? pb : pa);
      const bool ok = Rp.hg * kMaxGroup + (l & 7) < a.G;
      const float sc = ok ? (kind ? kscale_r : kscale_k) : 0.f;
      const bool lo = (l & 15) >= 8;
      half8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = Q.v[u][e] * sc;
        const _Float16 xh = _Float16(x);
        o[e] = lo ? _Float16(x - float(xh)) : xh;
      }
      qstage[it] = o;
    }
  };

  // ---- the wave's current run: online-softmax state and query operands
  float m_run = -INFINITY, l_run = 0.f;
  float sig = BV > 0 ? 0.f : 1.f, inv_sig = 1.f;   // value-norm normaliser (uniform over the wave)
  floatx4 acc[8];
  half8 qr[4], qs[4];
  Run R{};
  bool head_ok = false;
  int h = 0;
  auto start_run = [&](int piece) {
    const int g_local = R.hg * kMaxGroup + (col & 7);
    head_ok = g_local < a.G;
    h = R.hk * a.G + (head_ok ? g_local : 0);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      qr[s4] = qstage[((piece * 2 + 0) * 4 + s4) * 64 + lane];
      qs[s4] = qstage[((piece * 2 + 1) * 4 + s4) * 64 + lane];
    }
    m_run = -INFINITY;
    l_run = 0.f;
    sig = BV > 0 ? 0.f : 1.f;
    inv_sig = 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  };

  // Global data one lane needs for one 32-token chunk.  Every address lies in
  // the chunk's 32-slot block, which the clamped sequence range keeps inside
  // the cache, so the loads are unconditional; tokens past the end of the
  // sequence are masked after loading.  Norms: lane (col, q) loads one key
  // norm (col < 8) or residual norm (col >= 8) of token 8 q + col % 8 and one
  // value norm.
  // fp16 keys (kf: tile T, 32-wide step s2) and fp16 values (vf: 16-coordinate
  // block vb) travel in the same structures as the codes.
  struct KData {
    uint32_t kw[2][MKW];
    uint32_t sg[2];
    half8 kf[MK > 0 ? 1 : 2][MK > 0 ? 1 : 4];
  };
  struct VData {
    uint32_t vw[8];
    uint32_t vw2[BV == 3 ? 8 : 1];   // 3-bit values: the next dword (a lane's 24 bits may straddle two)
    float nrm[3];   // key norm, residual norm, value norm of the lane's token
    half8 vf[BV > 0 ? 1 : 8];
  };
  uint32_t koff[2], soff[2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const uint32_t tk = 8 * (col >> 2) + 4 * T + (col & 3);
    koff[T] = tk * KREC + 4 * q * MKW;
    soff[T] = tk * 16 + 4 * q;
  }
  const uint32_t noff = 4 * (8 * q + (col & 7));
  // value codes of coordinate 16 vb + col, tokens 8 q .. 8 q + 7: bits [8 BV q,
  // 8 BV q + 8 BV) of the coordinate's 4 BV-byte group, from dword voff / 4
  const uint32_t voff = col * (4 * (BV > 0 ? BV : 1)) + 4 * ((8 * (BV > 0 ? BV : 1) * q) >> 5);
  // rel: chunk index within the problem (tokens 32 rel ..)
  // slot0: the chunk's first slot in its (layer, KV head) plane; vblk: its value block.
  auto load_k = [&](int64_t slot0, KData& K) {
    if constexpr (MK == 0) {
      const auto kr = chunk_rsrc(a.k_f16 + slot0 * D, kChunk * 2 * D);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const uint32_t off = (8 * (col >> 2) + 4 * T + (col & 3)) * (2 * D) + 64 * q;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) K.kf[T][s2] = bload<half8>(kr, off + 16 * s2);
      }
    }
    if constexpr (MK > 0) {
      const auto kr = chunk_rsrc(a.k_idx + slot0 * KREC, kChunk * KREC);
      const auto sr = chunk_rsrc(a.k_sign + slot0 * 16, kChunk * 16);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        if constexpr (MK == 4) {
          const u32x4 v4 = bload<u32x4>(kr, koff[T]);
#pragma unroll
          for (int u = 0; u < 4; ++u) K.kw[T][u] = v4[u];
        } else if constexpr (MK == 3) {
          const u32x3 v3 = bload<u32x3>(kr, koff[T]);
#pragma unroll
          for (int u = 0; u < 3; ++u) K.kw[T][u] = v3[u];
        } else if constexpr (MK == 2) {
          const u32x2 v2 = bload<u32x2>(kr, koff[T]);
          K.kw[T][0] = v2[0];
          K.kw[T][1] = v2[1];
        } else {
#pragma unroll
          for (int u = 0; u < MK; ++u) K.kw[T][u] = bload<uint32_t>(kr, koff[T] + 4 * u);
        }
        K.sg[T] = bload<uint32_t>(sr, soff[T]);
      }
    }
  };
  auto load_v = [&](int64_t slot0, int64_t vblk, VData& V) {
    if constexpr (MK > 0) {
      // both norms, selected where they are used: work on loaded data placed
      // here would make the compiler wait for these loads at once
      V.nrm[0] = bload<float>(chunk_rsrc(a.k_norm + slot0, kChunk * 4), noff);
      V.nrm[2] = bload<float>(chunk_rsrc(a.k_rnorm + slot0, kChunk * 4), noff);
    }
    if constexpr (BV == 0) {
      const auto vr = chunk_rsrc(a.v_f16 + vblk * D * kVBlock, D * kVBlock * 2);
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) V.vf[vb] = bload<half8>(vr, (16 * vb + col) * (2 * kVBlock) + 16 * q);
    }
    if constexpr (BV > 0) {
      V.nrm[1] = bload<float>(chunk_rsrc(a.v_norm + slot0, kChunk * 4), noff);
      const auto vr = chunk_rsrc(a.v_idx + vblk * D * (4 * BV), D * 4 * BV);
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) {
        V.vw[vb] = bload<uint32_t>(vr, voff + 16 * vb * (4 * BV));
        if constexpr (BV == 3) V.vw2[vb] = bload<uint32_t>(vr, voff + 4 + 16 * vb * (4 * BV));   // past the block: 0
      }
    }
  };
  // ---- scores of one chunk: tile T row col -> token 8 (col/4) + 4 T + col%4
  auto score = [&](const KData& K, floatx4 (&sm_)[2], floatx4 (&sq_)[2]) {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      sm_[T] = floatx4{0.f, 0.f, 0.f, 0.f};
      sq_[T] = floatx4{0.f, 0.f, 0.f, 0.f};
      if constexpr (MK > 0) {
        // the table lookups of a step group first, so that they are in
        // flight together, then its products (split keys: two steps per
        // group, to bound the live operand registers; else the whole tile)
        constexpr int SG = KSPLIT ? 2 : 4;
#pragma unroll
        for (int g0 = 0; g0 < 4; g0 += SG) {
          half8 kh[SG], kl[SG], sd[SG];
#pragma unroll
          for (int u = 0; u < SG; ++u) {
            const int s2 = g0 + u;
            if constexpr (KWIDE)
              deq8_wide<MK>(K.kw[T], s2, reinterpret_cast<const uint16_t*>(lut_k), kh[u], kl[u]);
            else
              deq8_k<MK>(slab_bits<MK>(K.kw[T], s2), lut_k, kh[u], kl[u]);
            sd[u] = *reinterpret_cast<const half8*>(lut_s + ((K.sg[T] >> (8 * s2)) & 0xFFu) * 4);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < SG; ++u) {
            sm_[T] = mfma16x16x32(kh[u], qr[g0 + u], sm_[T]);
            if constexpr (KSPLIT) sm_[T] = mfma16x16x32(kl[u], qr[g0 + u], sm_[T]);
            sq_[T] = mfma16x16x32(sd[u], qs[g0 + u], sq_[T]);
          }
        }
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) sm_[T] = mfma16x16x32(K.kf[T][s2], qr[s2], sm_[T]);
      }
    }
  };

  // ---- logits, online softmax and value accumulation of one chunk (tokens
  // 32 rel .. of the current run's sequence).
  auto attend = [&](int rel, const VData& V, const floatx4 (&sm_)[2],
                    const floatx4 (&sq_)[2]) {
    const int64_t crel = int64_t(rel) * kChunk;
    const bool full = crel + kChunk <= R.len;                                  // uniform over the wave
    const int rem = int(R.len - crel > kChunk ? kChunk : R.len - crel) - 8 * q;  // valid tokens of this lane's 8
    float lg[8];
    float kn[8], rn[8], vn[8];
    // Value norms are normalised by sig, the running maximum of ||v|| over
    // the run's tokens (uniform over the wave), so P'' below stays <= 1.
    float vl = 0.f;
    if constexpr (BV > 0 && !SCORE) {
      vl = V.nrm[1];   // this lane's token 8 q + col % 8
      if (!full) vl = (col & 7) < rem ? vl : 0.f;
      // only when some norm exceeds the current normaliser (rare after the
      // first chunks) is the new wave maximum formed
      if (__builtin_amdgcn_ballot_w64(vl > sig) != 0) {
        const float sig_new = fmaxf(fmaxf(sig, wave_max(vl)), 1e-30f);
        const float inv_new = __builtin_amdgcn_rcpf(sig_new);
        // rescale the accumulators to the new normaliser
        const float factor = sig * inv_new;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= factor;
        sig = sig_new;
        inv_sig = inv_new;
      }
    }
    {
      // Lane (col, q) holds the key norm (col < 8) or the residual norm
      // (col >= 8) and the value norm of token 8 q + col % 8.  The 16 lanes of
      // a row need all 8 tokens' norms: exchange them through this wave's LDS
      // slot (in-order within the wave, so no barrier).
      float* nx = nxch + wave * 128;
      if constexpr (MK > 0) nx[lane] = col < 8 ? V.nrm[0] : V.nrm[2];
      if constexpr (BV > 0 && !SCORE) nx[64 + lane] = vl * inv_sig;
      const float4* n4 = reinterpret_cast<const float4*>(nx + 16 * q);
      if constexpr (MK > 0) {
        const float4 a0 = n4[0], a1 = n4[1], b0 = n4[2], b1 = n4[3];
        kn[0] = a0.x; kn[1] = a0.y; kn[2] = a0.z; kn[3] = a0.w;
        kn[4] = a1.x; kn[5] = a1.y; kn[6] = a1.z; kn[7] = a1.w;
        rn[0] = b0.x; rn[1] = b0.y; rn[2] = b0.z; rn[3] = b0.w;
        rn[4] = b1.x; rn[5] = b1.y; rn[6] = b1.z; rn[7] = b1.w;
      }
      if constexpr (BV > 0 && !SCORE) {
        const float4 c0 = n4[16], c1 = n4[17];
        vn[0] = c0.x; vn[1] = c0.y; vn[2] = c0.z; vn[3] = c0.w;
        vn[4] = c1.x; vn[5] = c1.y; vn[6] = c1.z; vn[7] = c1.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float smv = sm_[e >> 2][e & 3];
      float t;
      if constexpr (MK > 0) {
        t = fmaf(kn[e], smv, rn[e] * sq_[e >> 2][e & 3]);
      } else {
        t = smv;
      }
      lg[e] = t + dpp_f<0x128>(t);   // high part + remainder part (row rotate by 8)
    }
    if (!full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lg[e] = e < rem ? lg[e] : -INFINITY;
    }
    if constexpr (SCORE) {
      if (head_ok && !lo_half) {
        float* out = a.logits + ((int64_t(R.layer) * a.batch + R.b) * a.Hq + h) * a.max_len + crel + 8 * q;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < rem) out[e] = lg[e];
      }
    } else {
      // ---- online softmax (per head).  Rescale only when some logit exceeds
      // the running maximum (rare after the first chunks); the branch is
      // uniform over the wave and forms the cross-row maximum only then.
      const float lmax = fmaxf(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])),
                               fmaxf(fmaxf(lg[4], lg[5]), fmaxf(lg[6], lg[7])));
      if (__builtin_amdgcn_ballot_w64(lmax > m_run) != 0) {   // NaN logits do not move the maximum
        float cmax = fmaxf(lmax, shfl_xor(lmax, 16));
        cmax = fmaxf(cmax, shfl_xor(cmax, 32));
        const float m_new = cmax > m_run ? cmax : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(lg[e] - m_run);
        psum += p[e];
      }
      l_run += psum;
      if constexpr (BV == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vn[e] = 1.f;
      }
      // P'' = p * ||v|| / sig in fp16: high part in columns 0..7, remainder in
      // columns 8..15 (B operand: lane (col, q), tokens 8 q + e).
      half8 pp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = p[e] * vn[e];
        const _Float16 hh = _Float16(pv);
        pp[e] = lo_half ? _Float16(pv - float(hh)) : hh;
      }
      // ---- values: A operand lane (i = col, q) = coordinate 16 vb + i,
      // tokens 8 q .. 8 q + 7; the lookups of four blocks are issued together
#pragma unroll
      for (int v0 = 0; v0 < 8; v0 += 4) {
        half8 vd[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int vb = v0 + u;
          if constexpr (BV == 4) {
            vd[u] = deq8_vrep<V_PAGE != 0>(V.vw[vb], lane4, vrep_base);
          } else if constexpr (VREP2) {
            vd[u] = deq8_vrep2(V.vw[vb], lane8, vsel0, vsel1, vrep_base);
          } else if constexpr (BV > 0) {
            uint32_t bits = V.vw[vb];
            if constexpr (BV == 3) bits = __builtin_amdgcn_alignbit(V.vw2[vb], bits, (24 * q) & 31) & 0xFFFFFFu;
            else if constexpr (BV == 2) bits = (bits >> (16 * (q & 1))) & 0xFFFFu;
            else if constexpr (BV == 1) bits = (bits >> (8 * q)) & 0xFFu;
            vd[u] = deq8<BV>(bits, lut_v);
          } else {
            vd[u] = V.vf[vb];
            if (!full) {   // fp16 values past the end may hold anything
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (e >= rem) vd[u][e] = _Float16(0.f);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[v0 + u] = mfma16x16x32(vd[u], pp, acc[v0 + u]);
      }
    }
  };

  // Writes the wave's state into its merge slot (`have`), or marks the slot
  // empty without touching the registers (which may hold another piece).
  auto flush = [&](bool have, bool ov = false) {
    if constexpr (!SCORE) {
      if (!have) {
        if (q == 0 && !lo_half) {
          mw[wave][col] = -INFINITY;
          lw[wave][col] = 0.f;
        }
        return;
      }
#pragma unroll
      for (int vb = 0; vb < 8; ++vb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[vb][r] += dpp_f<0x128>(acc[vb][r]);
      float l_tot = l_run + shfl_xor(l_run, 16);
      l_tot += shfl_xor(l_tot, 32);
      const bool live = m_run != -INFINITY;   // uniform per column
      if (q == 0 && !lo_half) {
        mw[wave][col] = live ? m_run : -INFINITY;
        lw[wave][col] = live ? l_tot : 0.f;
      }
      if (live && !lo_half) {
        float* rw = (RED_LDS ? red : (OVL && ov ? red_ov : red_wg)) + (wave * kMaxGroup + col) * D;
        const float so = sig * inv_alpha_v;   // the value norms' normaliser and the value tables' scale
#pragma unroll
        for (int vb = 0; vb < 8; ++vb) {
          const float4 v4 = {acc[vb][0] * so, acc[vb][1] * so, acc[vb][2] * so, acc[vb][3] * so};
          *reinterpret_cast<float4*>(rw + 16 * vb + 4 * q) = v4;
        }
      }
    }
  };
  // Merges the wave slots (after a barrier) into the partial of the piece of
  // problem context Rp, slot `seg`: (max, sum of exponentials, accumulator[D])
  // per head, the waves summed in wave order (the same for every thread).
  // Thread t handles coordinate t % 128 of heads t / 128 and t / 128 + 4.
  auto merge = [&](const Run& Rp, int seg, bool ov = false) {
    if constexpr (!SCORE) {
      const int ng = a.G - Rp.hg * kMaxGroup < kMaxGroup ? a.G - Rp.hg * kMaxGroup : kMaxGroup;
      const int64_t pbase = (int64_t(Rp.layer) * a.batch + Rp.b) * a.Hq + Rp.hk * a.G + Rp.hg * kMaxGroup;
      const int i = tid & (D - 1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int g = (tid >> 7) + 4 * u;
        if (g < ng) {
          // all reads first (no branch between them), then the sums; an
          // empty wave slot (maximum -inf) contributes nothing, whatever its
          // accumulator holds
          float mv[kDecodeWaves], rv[kDecodeWaves], lv[kDecodeWaves];
          if (OVL && ov) {
#pragma unroll
            for (int w = 0; w < kDecodeWaves; ++w) rv[w] = red_ov[(w * kMaxGroup + g) * D + i];
          }
#pragma unroll
          for (int w = 0; w < kDecodeWaves; ++w) {
            mv[w] = mw[w][g];
            if constexpr (RED_LDS)
              rv[w] = red[(w * kMaxGroup + g) * D + i];
            else if (!(OVL && ov))   // written by other waves of this workgroup: read past the vector L1
              rv[w] = __hip_atomic_load(const_cast<float*>(uniform_ptr(red_wg + w * kMaxGroup * D)) + g * D + i,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            lv[w] = lw[w][g];
          }
          float M = -INFINITY;
#pragma unroll
          for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mv[w]);
          float av = 0.f, ls = 0.f;
#pragma unroll
          for (int w = 0; w < kDecodeWaves; ++w) {
            const bool live = mv[w] != -INFINITY;
            const float f = live ? __builtin_amdgcn_exp2f(mv[w] - M) : 0.f;
            av += (live ? rv[w] : 0.f) * f;
            ls += (live ? lv[w] : 0.f) * f;
          }
          // agent-scope stores: visible to every XCD once complete (the
          // in-kernel merge reads them from other workgroups)
          float* P = a.partial + ((pbase + g) * a.seg_max + a.seg_base + seg) * (D + 2);
          __hip_atomic_store(P + 2 + i, av, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (i == 0) {
            __hip_atomic_store(P, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(P + 1, ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  };

  // In-kernel merge of a problem whose pieces are all written (the same
  // arithmetic, in the same order, as combine_kernel): thread t merges
  // coordinate t % 128 of heads t / 128 and t / 128 + 4 over the pieces in
  // batches of 4 with a running maximum; then wave w forms output rows
  // 16 w .. 16 w + 15 of Pi^T res on fp32 MFMA 16x16x4 (res in LDS, over the
  // wave tables' reduction area, which is free after the merge).
  auto finish = [&](int prob, const Run& Rp) {
    if constexpr (!SCORE) {
      const int ng = a.G - Rp.hg * kMaxGroup < kMaxGroup ? a.G - Rp.hg * kMaxGroup : kMaxGroup;
      const int64_t row0 = (int64_t(Rp.layer) * a.batch + Rp.b) * a.Hq + Rp.hk * a.G + Rp.hg * kMaxGroup;
      const int nseg = pieces_of(prob);
      const int i = tid & (D - 1), r16 = lane & 15, kq = lane >> 4;
      constexpr bool ROT = BV > 0;
      float pa[ROT ? 32 : 1];
      if constexpr (ROT) {
        // A operands (columns of Pi), step (v, c): Pi[16 v + 4 kq + c][16 wave + r16]
        const float* pil = a.pi + int64_t(Rp.layer) * D * D + 16 * wave + r16;
#pragma unroll
        for (int v = 0; v < 8; ++v)
#pragma unroll
          for (int c = 0; c < 4; ++c) pa[4 * v + c] = pil[int64_t(16 * v + 4 * kq + c) * D];
      }
      constexpr int SB = 4;
      float M[2], L[2], A[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        M[k] = -INFINITY;
        L[k] = 0.f;
        A[k] = 0.f;
      }
      for (int sp0 = 0; sp0 < nseg; sp0 += SB) {
        float ms[2][SB], ls[2][SB], as[2][SB];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int g = (tid >> 7) + 4 * k < ng ? (tid >> 7) + 4 * k : ng - 1;
          const float* P = a.partial + ((row0 + g) * a.seg_max + a.seg_base) * (D + 2);
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const int64_t sp = sp0 + u < nseg ? sp0 + u : nseg - 1;
            ms[k][u] = __hip_atomic_load(P + sp * (D + 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ls[k][u] = __hip_atomic_load(P + sp * (D + 2) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            as[k][u] = __hip_atomic_load(P + sp * (D + 2) + 2 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          float Mn = M[k];
#pragma unroll
          for (int u = 0; u < SB; ++u)
            if (sp0 + u < nseg) Mn = fmaxf(Mn, ms[k][u]);
          const float f0 = M[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[k] - Mn);
          L[k] *= f0;
          A[k] *= f0;
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const float f = (sp0 + u >= nseg || ms[k][u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[k][u] - Mn);
            L[k] = fmaf(ls[k][u], f, L[k]);
            A[k] = fmaf(as[k][u], f, A[k]);
          }
          M[k] = Mn;
        }
      }
      // the tail's pieces, after the packed ones (into At with rotated values)
      float At[2] = {0.f, 0.f};
      if (a.tail_cpp > 0) {
        const int ft = prob * a.tail_cpp;
        const int nsegt = (ft + a.tail_cpp - 1) / a.tail_cpw - ft / a.tail_cpw + 1;
        for (int sp0 = 0; sp0 < nsegt; sp0 += SB) {
          float ms[2][SB], ls[2][SB], as[2][SB];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int g = (tid >> 7) + 4 * k < ng ? (tid >> 7) + 4 * k : ng - 1;
            const float* P = a.partial + ((row0 + g) * a.seg_max + a.tail_base) * (D + 2);
#pragma unroll
            for (int u = 0; u < SB; ++u) {
              const int64_t sp = sp0 + u < nsegt ? sp0 + u : nsegt - 1;
              ms[k][u] = P[sp * (D + 2)];
              ls[k][u] = P[sp * (D + 2) + 1];
              as[k][u] = P[sp * (D + 2) + 2 + i];
            }
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            float Mn = M[k];
#pragma unroll
            for (int u = 0; u < SB; ++u)
              if (sp0 + u < nsegt) Mn = fmaxf(Mn, ms[k][u]);
            const float f0 = M[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[k] - Mn);
            L[k] *= f0;
            A[k] *= f0;
            At[k] *= f0;
#pragma unroll
            for (int u = 0; u < SB; ++u) {
              const float f =
                  (sp0 + u >= nsegt || ms[k][u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[k][u] - Mn);
              L[k] = fmaf(ls[k][u], f, L[k]);
              if constexpr (ROT)
                At[k] = fmaf(as[k][u], f, At[k]);
              else
                A[k] = fmaf(as[k][u], f, A[k]);
            }
            M[k] = Mn;
          }
        }
      }
      float* const res = fin;            // [16][D]: heads, rows >= ng zero
      float* const resp = fin + 16 * D;  // [16][D]: the tail's part (stored domain)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int g = (tid >> 7) + 4 * k;
        // L is 0 only for an empty sequence; NaN must propagate.
        const bool has = L[k] > 0.f || L[k] != L[k];
        const float v = has ? A[k] / L[k] : 0.f;
        if constexpr (ROT) {
          res[g * D + i] = g < ng ? v : 0.f;
          res[(g + 8) * D + i] = 0.f;
          resp[g * D + i] = (g < ng && has) ? At[k] / L[k] : 0.f;
        } else if (g < ng) {
          a.out[(row0 + g) * D + i] = v;
        }
      }
      if constexpr (ROT) {
        __syncthreads();
        const float4* bres = reinterpret_cast<const float4*>(res + r16 * D + 4 * kq);
        float4 b4[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) b4[v] = bres[4 * v];
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          acc = mfma16x16x4f32(pa[4 * v + 0], b4[v].x, acc);
          acc = mfma16x16x4f32(pa[4 * v + 1], b4[v].y, acc);
          acc = mfma16x16x4f32(pa[4 * v + 2], b4[v].z, acc);
          acc = mfma16x16x4f32(pa[4 * v + 3], b4[v].w, acc);
        }
        if (r16 < ng) {
          const float4 t = *reinterpret_cast<const float4*>(resp + r16 * D + 16 * wave + 4 * kq);
          const float4 o = {acc[0] + t.x, acc[1] + t.y, acc[2] + t.z, acc[3] + t.w};
          *reinterpret_cast<float4*>(a.out + (row0 + r16) * D + 16 * wave + 4 * kq) = o;
        }
      }
    }
  };
  // Counts the piece of problem `prob` just written by merge; the workgroup
  // that brings the count to the problem's number of pieces resets it and
  // runs finish.  Hand-off: the partials are written and read with
  // agent-scope (device-coherent) stores and loads, and every wave waits for
  // its stores to complete before the barrier that precedes the count's
  // increment, so a workgroup that sees the full count (its loads issued
  // after that atomic returned) reads every piece complete.  A release fence
  // at agent scope would order the same, but it also writes back the XCD's
  // whole L2 (one pass per fence), which cost more than the merge saves.
  auto arrive = [&](int prob, const Run& Rp) {
    if constexpr (!SCORE) {
      if (a.done == nullptr) return;
      __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are complete
      __syncthreads();
      if (tid == 0) {
        const uint32_t nseg = uint32_t(pieces_of(prob));
        const uint32_t old = __hip_atomic_fetch_add(a.done + prob, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old + 1 == nseg;
        if (last) __hip_atomic_store(a.done + prob, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        counter[1] = last ? 1u : 0u;
      }
      __syncthreads();
      if (counter[1]) finish(prob, Rp);
    }
  };

  // Ticket draw: lane 0 takes the next ticket of the workgroup counter.
  auto draw = [&]() -> uint32_t {
    uint32_t v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return v;
  };
  auto uni = [](uint32_t v) { return int(__builtin_amdgcn_readfirstlane(v)); };

  // ---- the first group's context, query operands and first chunk loads are
  // issued before the tables are built, so their latency overlaps the build.
  // Every group starts with fixed tickets: wave w takes w, w + 8 and w + 16,
  // and counter value base + k is ticket 24 + k (base: the counter value at
  // the start of the group).
  // Load order: codebooks, then the staged query operands, then the sequence
  // table, so that the table build below (which needs only the codebooks)
  // does not wait for the chunk loads that the sequence data unlocks.
  float kcl = 0.f, vcl = 0.f;   // lane l: key / value centroid l mod (number of centroids), times its scale
  if constexpr (MK > 0) kcl = a.kc[lane & ((1 << MK) - 1)] * alpha_k;
  if constexpr (BV > 0) vcl = a.vc[lane & ((1 << BV) - 1)] * alpha_v;
  if (a.ragged) {
    for (int b = tid; b < a.batch; b += NT) {
      int64_t st = a.seq_start[b], ln = a.seq_len[b];
      clamp_run(st, ln);
      live_s[b + 1] = int((ln + kChunk - 1) / kChunk);
    }
    __syncthreads();
    const int64_t per_seq = int64_t(a.n_layers) * HG;
    const int64_t nd = int64_t(nblk) - a.n_app;
    if (wave == 0) {
      // the live chunks of all sequences, and the mean range w0 over them
      int sum = 0;
      for (int b = lane; b < a.batch; b += 64) sum += live_s[b + 1];
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      const int64_t w0 = (per_seq * sum + nd - 1) / nd;   // >= 1 when any sequence has tokens
      // padded counts, then their inclusive prefix, 64 sequences at a time
      int carry = 0;
      for (int b0 = 0; b0 < a.batch; b0 += 64) {
        const int b = b0 + lane;
        const int live = b < a.batch ? live_s[b + 1] : 0;
        int v = 0;
        if (live > 0)
          v = live + kRaggedCrossChunks + (live < w0 ? int(int64_t(kContainChunks) * (w0 - live) / w0) : 0);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(v, o);
          if (lane >= o) v += t;
        }
        if (b < a.batch) live_s[b + 1] = carry + v;
        carry += __shfl(v, 63);
      }
      if (lane == 0) {
        live_s[0] = 0;
        counter[2] = uint32_t(sum);
      }
    }
    __syncthreads();
    // ragged when the chunks that hold tokens are fewer than problems x cpp_real
    const int64_t padded_total = per_seq * lds_s(a.batch);
    const int64_t live_total = per_seq * int64_t(__builtin_amdgcn_readfirstlane(counter[2]));
    if (live_total < int64_t(a.total_chunks / cpp) * a.cpp_real) {
      rag = true;
      total = int(padded_total);
      const int even = int((padded_total + nd - 1) / nd);
      cpw = even > a.cpw_min ? even : a.cpw_min;
    }
  }
  if (rag) {
    // the outputs of sequences without tokens (no range reaches them)
    if (wg == 0) {
      for (int b = 0; b < a.batch; ++b) {
        if (live_s[b + 1] != live_s[b]) continue;
        for (int64_t e = tid; e < int64_t(a.n_layers) * a.Hq * D; e += NT) {
          const int64_t layer = e / (int64_t(a.Hq) * D), r = e % (int64_t(a.Hq) * D);
          a.out[(layer * a.batch + b) * a.Hq * D + r] = 0.f;
        }
      }
    }
  }
  const int c_first = wg * cpw;
  const int c_last = c_first + cpw < total ? c_first + cpw : total;
  if (c_first >= c_last) return;   // a workgroup without chunks (ragged split)
  QItem qitem;
  {
    const int pa = prob_of(c_first);
    const int pa_end = pfirst(pa) + pcount(pa);
    stage_load(pa, pa_end < c_last ? prob_of(pa_end) : pa, qitem);
  }
  __builtin_amdgcn_sched_barrier(0);
  Group G = group_of(c_first, c_last);
  KData K0, K1;
  VData V0, V1;
  bool pre = false;   // the first run's K0, K1, V0 are already loaded
  if constexpr (kPrefetch) {
    // Issued by every wave (no branch, so that the table build below waits
    // only for the codebook loads); a wave without a ticket reads chunk 0 of
    // piece A's sequence, which is in bounds and never used.
    // (With an append in the launch, a wave without a ticket reads ticket 0's
    // chunk instead, and every chunk read passes the gate first.)
    const int t0 = wave, t1 = wave + kDecodeWaves;
    pre = t0 < G.n_tickets;
    const int u1 = t1 < G.n_tickets ? t1 : t0;
    const bool any = G.n_tickets > 0;
    const int d0 = pre ? t0 : 0, d1 = pre ? u1 : 0;
    if (any) {
      gate(G, d0);
      gate(G, d1);
    }
    const int64_t s0 = any ? slot_of(G, d0) : G.ra.slot_base, s1 = any ? slot_of(G, d1) : G.ra.slot_base;
    load_k(s0, K0);
    load_k(s1, K1);
    load_v(s0, any ? vblk_of(G, d0) : G.ra.vblk0, V0);
  }

  // ---- tables (built once, used for every chunk of the workgroup)
  if constexpr (KWIDE) {
    // fp16 high parts [2^MK], then the remainders [2^MK]
    for (int x = tid; x < (1 << MK); x += NT) {
      const float c = a.kc[x];
      const uint16_t h = f16_bits(c);
      reinterpret_cast<uint16_t*>(lut_k)[x] = h;
      reinterpret_cast<uint16_t*>(lut_k)[(1 << MK) + x] = f16_bits(c - float(__builtin_bit_cast(_Float16, h)));
    }
  } else if constexpr (MK > 0) {
    if constexpr (KL::NC > 2)
      build_kpairs<MK>(pair_hi, kcl, tid, NT);
    else
      build_kpairs<MK>(lut_k, kcl, tid, NT);
  }
  if constexpr (VREP2)
    build_vrep2(lut_v, vcl, tid, NT);
  else if constexpr (VREP)
    build_vrep(lut_v, vcl, tid, NT);
  else if constexpr (BV > 0)
    build_lut<BV, false>(lut_v, vcl, tid, NT);
  if constexpr (MK > 0) {
    for (int x = tid; x < 256; x += NT) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t lo = ((x >> e) & 1) ? 0x3C00u : 0xBC00u;
        const uint32_t hi = ((x >> (e + 1)) & 1) ? 0x3C00u : 0xBC00u;
        lut_s[x * 4 + e / 2] = lo | (hi << 16);
      }
    }
  }
  stage_store(G.pa, G.pb, qitem);
  if (tid == 0) counter[0] = 0;
  __syncthreads();
  if constexpr (MK > 0 && !KWIDE && KL::NC > 2) {
    build_ktab<MK, NT>(lut_k, pair_hi, tid);
    __syncthreads();
  }

  int base = -3 * kDecodeWaves;   // ticket t of the group is counter value base + t (t >= 24)
#pragma unroll 1
  for (int g0 = c_first; g0 < c_last;) {
    if (g0 != c_first) {
      pre = false;
      G = group_of(g0, c_last);
      app_ok_a = app_ok_b = false;
      stage_load(G.pa, G.pb, qitem);
      stage_store(G.pa, G.pb, qitem);
      __syncthreads();
    }
    // the wave's next three tickets (relative to base)
    int t0 = wave, t1 = wave + kDecodeWaves, t2 = wave + 2 * kDecodeWaves;
    const bool last_ov = OVL && G.b_end >= c_last;   // the workgroup's last group: merge over a dead table
    bool had_a = false, had_b = false;
#pragma unroll 1
    while (t0 < G.n_tickets) {
      const bool in_a = t0 < G.live_a;
      const int limit = in_a ? G.live_a : G.n_tickets;
      const int rel0 = in_a ? G.rel_a0 : -G.live_a;   // chunk of ticket t: rel0 + t
      R = in_a ? G.ra : G.rb;
      if constexpr (kPrefetch) {
        // Software pipeline: while chunk t0 is attended, chunk t1 is scored and
        // the key data of chunk t2 and the value data of chunk t1 are loaded.
        // Unrolled twice so that the two register sets swap roles without
        // copies.  Loads follow the tickets across the end of the run into
        // the group's next piece, so a new run starts with its first chunks
        // in flight (its first chunk is scored again with its own queries); a
        // ticket past the group's end reloads the latest chunk (still in
        // L2), whose copy is scored but never attended.
        const int n = G.n_tickets;
        floatx4 m0[2], s0[2], m1[2], s1[2];
        // (value loads follow the key loads of the same ticket, which passed
        // the gate)
        if (!pre) {
          gate(G, t0);
          gate(G, t1 < n ? t1 : t0);
          load_k(slot_of(G, t0), K0);
          load_k(slot_of(G, t1 < n ? t1 : t0), K1);
          load_v(slot_of(G, t0), vblk_of(G, t0), V0);
        }
        start_run(in_a ? 0 : 1);
        score(K0, m0, s0);
        bool swap = false;
#pragma unroll 1
        for (;;) {
          const uint32_t d3 = draw();
          gate(G, t2 < n ? t2 : (t1 < n ? t1 : t0));
          load_k(slot_of(G, t2 < n ? t2 : (t1 < n ? t1 : t0)), K0);
          {
            const int u = t1 < n ? t1 : t0;
            load_v(slot_of(G, u), vblk_of(G, u), V1);
          }
          score(K1, m1, s1);
          attend(rel0 + t0, V0, m0, s0);
          const int t3 = uni(d3) - base;
          if (t1 >= limit) { t0 = t1; t1 = t2; t2 = t3; swap = true; break; }
          const uint32_t d4 = draw();
          gate(G, t3 < n ? t3 : (t2 < n ? t2 : t1));
          load_k(slot_of(G, t3 < n ? t3 : (t2 < n ? t2 : t1)), K1);
          {
            const int u = t2 < n ? t2 : t1;
            load_v(slot_of(G, u), vblk_of(G, u), V0);
          }
          score(K0, m0, s0);
          attend(rel0 + t1, V1, m1, s1);
          const int t4 = uni(d4) - base;
          if (t2 >= limit) { t0 = t2; t1 = t3; t2 = t4; break; }
          t0 = t2; t1 = t3; t2 = t4;
        }
        // K0, K1 and V0 now hold the chunks of tickets t0 and t1
        if (swap) {
          // member by member, only what the format uses: a whole-struct copy
          // also moves the members it leaves unwritten, which the compiler
          // then keeps in per-thread memory (placed in LDS and addressed
          // through the dispatch packet, read by every wave at its start)
          if constexpr (MK > 0) {
#pragma unroll
            for (int T = 0; T < 2; ++T) {
#pragma unroll
              for (int u = 0; u < MKW; ++u) {
                const uint32_t t = K0.kw[T][u];
                K0.kw[T][u] = K1.kw[T][u];
                K1.kw[T][u] = t;
              }
              const uint32_t t = K0.sg[T];
              K0.sg[T] = K1.sg[T];
              K1.sg[T] = t;
            }
          } else {
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2) {
                const half8 t = K0.kf[T][s2];
                K0.kf[T][s2] = K1.kf[T][s2];
                K1.kf[T][s2] = t;
              }
          }
          V0 = V1;
        }
        pre = true;
      } else {
        start_run(in_a ? 0 : 1);
#pragma unroll 1
        while (t0 < limit) {
          const uint32_t d3 = draw();
          gate(G, t0);
          load_k(slot_of(G, t0), K0);
          load_v(slot_of(G, t0), vblk_of(G, t0), V0);
          floatx4 sm_[2], sq_[2];
          score(K0, sm_, sq_);
          attend(rel0 + t0, V0, sm_, sq_);
          t0 = t1; t1 = t2; t2 = uni(d3) - base;
        }
      }
      if (in_a) {
        if (!(last_ov && !G.has_b)) flush(true);   // (else after the barrier below)
        had_a = true;
      } else {
        had_b = true;
      }
    }
    // ---- merge the group's pieces
    if (!had_a) flush(false);
    if (last_ov && !G.has_b) {
      __syncthreads();   // every wave is done with the tables
      if (had_a) flush(true, true);
    }
    if constexpr (!RED_LDS) __builtin_amdgcn_s_waitcnt(0);   // this wave's merge stores are complete
    __syncthreads();
    const int next_base = uni(counter[0]);   // every draw of the group is done
    merge(G.ra, wg - pfirst(G.pa) / cpw, last_ov && !G.has_b);
    arrive(G.pa, G.ra);
    if (G.has_b) {
      __syncthreads();   // (and every wave is done with the tables)
      flush(had_b, last_ov);
      if constexpr (!RED_LDS) __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      merge(G.rb, wg - G.a_end / cpw, last_ov);
      arrive(G.pb, G.rb);
    }
    __syncthreads();
    base = next_base - 3 * kDecodeWaves;
    g0 = G.b_end;
  }
}

template <int MK, int BV, bool SCORE>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_kernel(
    DecodeArgs a, CompressArgs ca) {
  __shared__ __align__(256) unsigned char dsm[DecodeLayout<MK, BV, SCORE>::LDS_BYTES];
  decode_body<MK, BV, SCORE>(a, ca, dsm, int(blockIdx.x), int(gridDim.x));
}

// Two decode calls in one launch: part 1 in format <MK, BV>, part 2 with fp16
// keys and values (say a model's uncompressed boundary layers beside its
// quantized ones), each with its own arguments, append and workspace.  Blocks,
// in dispatch order: part 1's append workgroups, part 2's, then nd1 decode
// workgroups of part 1 and the rest for part 2.  Each part sees its own
// blocks numbered from 0 (appends first), so its work split and XCD-aware
// mapping are those of a launch of its own with that many workgroups; both
// parts' workgroups share every XCD, and the launch pays one start and one end.
template <int MK, int BV>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_pair_kernel(
    DecodeArgs a1, CompressArgs c1, DecodeArgs a2, CompressArgs c2, int nd1) {
  constexpr int L1 = DecodeLayout<MK, BV, false>::LDS_BYTES, L2 = DecodeLayout<0, 0, false>::LDS_BYTES;
  __shared__ __align__(256) unsigned char dsm[L1 > L2 ? L1 : L2];
  const int b = int(blockIdx.x), apps = a1.n_app + a2.n_app;
  const int nd2 = int(gridDim.x) - apps - nd1;
  bool first;
  int blk;
  if (b < apps) {
    first = b < a1.n_app;
    blk = first ? b : b - a1.n_app;
  } else {
    first = b - apps < nd1;
    blk = first ? a1.n_app + (b - apps) : a2.n_app + (b - apps - nd1);
  }
  if (first)
    decode_body<MK, BV, false>(a1, c1, dsm, blk, a1.n_app + nd1);
  else
    decode_body<0, 0, false>(a2, c2, dsm, blk, a2.n_app + nd2);
}

// The query preparation of a decode call, one workgroup per (quarter, layer,
// run of kQprepRows query rows): wave w owns row block 4 quarter + w of
// [Pi; S] (16 rows), read once per workgroup and split into fp16 high parts
// and remainders (times 2^11); the run's query rows (of the layer's batch x
// Hq) are the MFMA columns, 16 at a time, each scaled by
// the power of two that puts its norm in [2^14, 2^15) and split likewise, so
// three v_mfma_f32_16x16x32_f16 per 32-wide step keep about 22 bits (Pi and S
// are loaded once per layer, quarter and run instead of once per KV head).
// Quarter 0 of run 0 also zeroes the layer's merge counts and its append count;
// `qplain` (if not null) receives q itself, for a decode over an fp16 tail.
// fp16 keys (ROT false): q itself and zeros.  A run is one MFMA column block
// (16 rows): the launch is short and latency-bound, and more workgroups with
// one round of loads each beat fewer that loop (64-row runs: a decode step
// of 64 query heads over 262,144 tokens took 76.5 us against 73.6 us now).
constexpr int kQprepRows = 16;
template <bool ROT>
__device__ __forceinline__ void qprep_quarter(const float* q, const float* pi, const float* s, float* qprep,
                                              int batch, int H, int Hq, int quarter, int layer, int n_layers,
                                              int run, uint32_t* done, float* qplain) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int G = Hq / H;
  const int row_lo = run * kQprepRows;                // the run's rows of the layer
  const int nrows = min(batch * Hq - row_lo, kQprepRows);
  const int64_t base = int64_t(layer) * batch * Hq + row_lo;   // the run's first query row
  if (done != nullptr && quarter == 0 && run == 0) {
    const int n_hg = (G + kMaxGroup - 1) / kMaxGroup;
    const int64_t per_layer = int64_t(batch) * H * n_hg;   // problems of a layer (consecutive)
    for (int64_t e = tid; e < per_layer; e += 256) done[int64_t(layer) * per_layer + e] = 0u;
    if (tid == 0) done[int64_t(n_layers) * per_layer + layer] = 0u;
    // the append wait's give-up flag, after the append counts
    if (tid == 0 && layer == 0) done[int64_t(n_layers) * per_layer + n_layers] = 0u;
  }
  if (!ROT || qplain != nullptr) {
    float* dst = ROT ? qplain : qprep;
    for (int64_t e = int64_t(quarter) * 256 + tid; e < int64_t(nrows) * D; e += 1024) {
      const int64_t r = e >> 7;
      const int i = int(e & 127);
      dst[(base + r) * 2 * D + i] = q[(base + r) * D + i];
      dst[(base + r) * 2 * D + D + i] = 0.f;
    }
  }
  if constexpr (ROT) {
    const int rb = 4 * quarter + wave, mat = rb >> 3, i0 = 16 * (rb & 7);
    half8 ah[4], al[4];
    {
      const float4* src =
          reinterpret_cast<const float4*>((mat ? s : pi) + int64_t(layer) * D * D + int64_t(i0 + col) * D + 32 * kq);
      float4 v4[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) v4[v] = src[v];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float v[8] = {v4[2 * t].x, v4[2 * t].y, v4[2 * t].z, v4[2 * t].w,
                            v4[2 * t + 1].x, v4[2 * t + 1].y, v4[2 * t + 1].z, v4[2 * t + 1].w};
        split8(v, ah[t], al[t], true);
      }
    }
    for (int r0 = 0; r0 < nrows; r0 += 16) {
      const int r = r0 + col < nrows ? r0 + col : nrows - 1;
      const float4* qs4 = reinterpret_cast<const float4*>(q + (base + r) * D + 32 * kq);
      float x[32];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 f = qs4[v];
        x[4 * v] = f.x; x[4 * v + 1] = f.y; x[4 * v + 2] = f.z; x[4 * v + 3] = f.w;
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) ss = fmaf(x[e], x[e], ss);
      ss += shfl_xor(ss, 16);
      ss += shfl_xor(ss, 32);
      const float nq = sqrtf(ss);
      const int ex = (nq > 0.f && nq < INFINITY) ? 15 - __builtin_amdgcn_frexp_expf(nq) : 0;
      floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_amdgcn_ldexpf(x[8 * t + e], ex);
        half8 xh, xl;
        split8(v, xh, xl, true);
        a1 = mfma16x16x32(ah[t], xh, a1);
        a2 = mfma16x16x32(al[t], xh, a2);
        a2 = mfma16x16x32(ah[t], xl, a2);
      }
      // D: rows i0 + 4 kq + k of the block, column (query row) r0 + col
      if (r0 + col < nrows) {
        float4 o;
        o.x = __builtin_amdgcn_ldexpf(fmaf(a2[0], 0x1p-11f, a1[0]), -ex);
        o.y = __builtin_amdgcn_ldexpf(fmaf(a2[1], 0x1p-11f, a1[1]), -ex);
        o.z = __builtin_amdgcn_ldexpf(fmaf(a2[2], 0x1p-11f, a1[2]), -ex);
        o.w = __builtin_amdgcn_ldexpf(fmaf(a2[3], 0x1p-11f, a1[3]), -ex);
        *reinterpret_cast<float4*>(qprep + (base + r0 + col) * 2 * D + mat * D + i0 + 4 * kq) = o;
      }
    }
  }
}
// Grid (4 quarters, n_layers, runs of kQprepRows query rows).
template <bool ROT>
__global__ __launch_bounds__(256) void qprep_kernel(const float* q, const float* pi, const float* s, float* qprep,
                                                    int batch, int H, int Hq, uint32_t* done, float* qplain) {
  qprep_quarter<ROT>(q, pi, s, qprep, batch, H, Hq, blockIdx.x, blockIdx.y, gridDim.y, blockIdx.z, done, qplain);
}
// Grid of the query preparation for n_layers layers of batch x Hq query rows.
inline dim3 qprep_grid(int n_layers, int batch, int Hq) {
  return dim3(4, unsigned(n_layers), unsigned((batch * Hq + kQprepRows - 1) / kQprepRows));
}

// The query preparations of two decode calls in one launch (the parts of
// decode_pair_kernel; part 2 has fp16 keys): blocks [0, 4 L1 runs) are part
// 1's (quarter, layer, run) blocks of qprep_kernel, flattened, the rest part 2's.
template <bool ROT1>
__global__ __launch_bounds__(256) void qprep_pair_kernel(const float* q1, const float* pi1, const float* s1,
                                                         float* qp1, uint32_t* done1, int H1, int L1, const float* q2,
                                                         float* qp2, uint32_t* done2, int H2, int L2, int batch,
                                                         int Hq) {
  const int runs = (batch * Hq + kQprepRows - 1) / kQprepRows;
  int i = int(blockIdx.x);
  if (i < 4 * L1 * runs) {
    qprep_quarter<ROT1>(q1, pi1, s1, qp1, batch, H1, Hq, i & 3, (i >> 2) % L1, L1, (i >> 2) / L1, done1, nullptr);
  } else {
    i -= 4 * L1 * runs;
    qprep_quarter<false>(q2, nullptr, nullptr, qp2, batch, H2, Hq, i & 3, (i >> 2) % L2, L2, (i >> 2) / L2, done2,
                         nullptr);
  }
}

// The append of a few tokens and the query preparation of the same decode
// step in one launch (they are independent): workgroups [0, n_append) run
// the append blocks (item group, layer), then the query preparation blocks
// (quarter, layer, run) of qprep_kernel.
template <int MK, int BV>
__global__ __launch_bounds__(kAppendThreads) void append_prepare_kernel(
    CompressArgs a, int app_groups, int n_append, const float* q, const float* pi, const float* s, float* qprep,
    int batch, int H, int Hq, uint32_t* done, int n_layers) {
  __shared__ AppendSmem sm;
  const int bid = blockIdx.x;
  if (bid < n_append) {
    append_body<MK, BV>(a, bid % app_groups, bid / app_groups, sm);
    return;
  }
  const int r = bid - n_append;
  if (threadIdx.x >= 256) return;   // the query preparation blocks take 4 waves
  qprep_quarter<(MK > 0)>(q, pi, s, qprep, batch, H, Hq, r & 3, (r >> 2) % n_layers, n_layers, (r >> 2) / n_layers,
                          done, nullptr);
}

// Merges the piece partials of one (layer, batch, KV head) for every query
// head of its group and writes out = Pi^T (acc / l) (acc / l for fp16
// values).  Merge: thread t works on coordinate t % 128 of heads t / 128,
// t / 128 + 2, ...; a head's problem has one partial per workgroup whose
// chunk run overlaps it (computed from the run length, the same arithmetic
// as the decode kernel's slot index).  They are read in batches of 4 pieces x
// 8 heads with clamped (always valid) addresses so that a batch's loads are
// in flight together, and merged with a running maximum.  Pi^T: fp32 MFMA 16x16x4 with
// D[i][g] = sum_j Pi[j][i] res[g][j]; wave w owns output rows 32 w .. 32 w + 31
// (two 16-row blocks); its A operands (columns of Pi) are loaded from global
// memory at the start, before the merge, and res comes from LDS.
constexpr int kCombineHeads = 16;
// A second set of pieces, from a decode over an fp16 tail of the same
// sequences (tail_cpp > 0: its split's chunks per problem and per workgroup),
// sits in the slots from tail_base on; it joins the same running merge, and
// since fp16 values accumulate as stored (not rotated) its accumulator is added
// after Pi^T.
template <bool ROT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void combine_kernel(
    const float* partial, const float* pi, float* out, int batch, int H, int Hq, int n_hg, int chunks_per_problem,
    int chunks_per_wg, int seg_max, int tail_cpp, int tail_cpw, int tail_base) {
  constexpr bool rotate = ROT;
  __shared__ __align__(16) float res[kCombineHeads][D];
  __shared__ __align__(16) float resp[ROT ? kCombineHeads : 1][D];   // tail part (stored domain)
  const int hk = blockIdx.x, b = blockIdx.y, layer = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, r16 = lane & 15, kq = lane >> 4;
  const int i = tid & 127, half = tid >> 7;
  const int G = Hq / H;
  // A operands: block n (rows 32 wave + 16 n + r16), step (v, c): Pi[16 v + 4 kq + c][row].
  float pa[ROT ? 2 : 1][32];
  if constexpr (ROT) {
    const float* pil = pi + int64_t(layer) * D * D;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int v = 0; v < 8; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) pa[n][4 * v + c] = pil[int64_t(16 * v + 4 * kq + c) * D + 32 * wave + 16 * n + r16];
  }
  constexpr int NH = kCombineHeads / 2, SB = 4;
  for (int g0 = 0; g0 < G; g0 += kCombineHeads) {
    const int ng = G - g0 < kCombineHeads ? G - g0 : kCombineHeads;
    const int64_t row0 = (int64_t(layer) * batch + b) * Hq + int64_t(hk) * G + g0;
    float M[NH], L[NH], A[NH], At[NH];
    int nseg[NH], nsegt[NH];   // partial slots written for the head's problem (packed part, tail part)
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      M[k] = -INFINITY;
      L[k] = 0.f;
      A[k] = 0.f;
      At[k] = 0.f;
      const int g = g0 + (half + 2 * k < ng ? half + 2 * k : ng - 1);
      const int prob = ((layer * batch + b) * H + hk) * n_hg + g / kMaxGroup;
      const int first = prob * chunks_per_problem;
      nseg[k] = (first + chunks_per_problem - 1) / chunks_per_wg - first / chunks_per_wg + 1;
      const int ft = prob * tail_cpp;
      nsegt[k] = tail_cpp > 0 ? (ft + tail_cpp - 1) / tail_cpw - ft / tail_cpw + 1 : 0;
    }
    for (int sp0 = 0; sp0 < seg_max; sp0 += SB) {
      float ms[NH][SB], ls[NH][SB], as[NH][SB];
#pragma unroll
      for (int k = 0; k < NH; ++k) {
        const int g = half + 2 * k < ng ? half + 2 * k : ng - 1;
        const float* P = partial + (row0 + g) * int64_t(seg_max) * (D + 2);
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int64_t sp = sp0 + u < nseg[k] ? sp0 + u : nseg[k] - 1;
          ms[k][u] = P[sp * (D + 2)];
          ls[k][u] = P[sp * (D + 2) + 1];
          as[k][u] = P[sp * (D + 2) + 2 + i];
        }
      }
#pragma unroll
      for (int k = 0; k < NH; ++k) {
        float Mn = M[k];
#pragma unroll
        for (int u = 0; u < SB; ++u)
          if (sp0 + u < nseg[k]) Mn = fmaxf(Mn, ms[k][u]);
        const float f0 = M[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[k] - Mn);
        L[k] *= f0;
        A[k] *= f0;
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const float f =
              (sp0 + u >= nseg[k] || ms[k][u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[k][u] - Mn);
          L[k] = fmaf(ls[k][u], f, L[k]);
          A[k] = fmaf(as[k][u], f, A[k]);
        }
        M[k] = Mn;
      }
    }
    // the tail's pieces (none unless tail_cpp > 0), into At (ROT) or A
    for (int sp0 = 0; tail_cpp > 0 && sp0 < seg_max - tail_base; sp0 += SB) {
      float ms[NH][SB], ls[NH][SB], as[NH][SB];
#pragma unroll
      for (int k = 0; k < NH; ++k) {
        const int g = half + 2 * k < ng ? half + 2 * k : ng - 1;
        const float* P = partial + ((row0 + g) * int64_t(seg_max) + tail_base) * (D + 2);
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int64_t sp = sp0 + u < nsegt[k] ? sp0 + u : nsegt[k] - 1;
          ms[k][u] = P[sp * (D + 2)];
          ls[k][u] = P[sp * (D + 2) + 1];
          as[k][u] = P[sp * (D + 2) + 2 + i];
        }
      }
#pragma unroll
      for (int k = 0; k < NH; ++k) {
        float Mn = M[k];
#pragma unroll
        for (int u = 0; u < SB; ++u)
          if (sp0 + u < nsegt[k]) Mn = fmaxf(Mn, ms[k][u]);
        const float f0 = M[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[k] - Mn);
        L[k] *= f0;
        A[k] *= f0;
        At[k] *= f0;
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const float f =
              (sp0 + u >= nsegt[k] || ms[k][u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[k][u] - Mn);
          L[k] = fmaf(ls[k][u], f, L[k]);
          if (rotate)
            At[k] = fmaf(as[k][u], f, At[k]);
          else
            A[k] = fmaf(as[k][u], f, A[k]);
        }
        M[k] = Mn;
      }
    }
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const int g = half + 2 * k;
      // L is 0 only for an empty sequence; NaN must propagate.
      const bool has = L[k] > 0.f || L[k] != L[k];
      const float v = has ? A[k] / L[k] : 0.f;
      if (rotate) {
        res[g][i] = g < ng ? v : 0.f;
        resp[g][i] = (g < ng && has) ? At[k] / L[k] : 0.f;
      } else if (g < ng) {
        out[(row0 + g) * D + i] = v;
      }
    }
    if constexpr (!ROT) continue;
    __syncthreads();
    const float4* bres = reinterpret_cast<const float4*>(&res[r16][4 * kq]);
    float4 b4[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) b4[v] = bres[4 * v];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        acc = mfma16x16x4f32(pa[n][4 * v + 0], b4[v].x, acc);
        acc = mfma16x16x4f32(pa[n][4 * v + 1], b4[v].y, acc);
        acc = mfma16x16x4f32(pa[n][4 * v + 2], b4[v].z, acc);
        acc = mfma16x16x4f32(pa[n][4 * v + 3], b4[v].w, acc);
      }
      if (r16 < ng) {
        const float4 t = *reinterpret_cast<const float4*>(&resp[r16][32 * wave + 16 * n + 4 * kq]);
        float4 o = {acc[0] + t.x, acc[1] + t.y, acc[2] + t.z, acc[3] + t.w};
        *reinterpret_cast<float4*>(out + (row0 + r16) * D + 32 * wave + 16 * n + 4 * kq) = o;
      }
    }
    __syncthreads();
  }
}

// ===========================================================================
// Multi-query scores

// Query rows per pass of the multi-query score kernel over a KV head's codes:
// 8 MFMA column blocks of 8 rows (fp16 high parts in columns 0..7, their
// remainders in columns 8..15, as in decode).
constexpr int kMultiRows = 64;
constexpr int kMultiWaves = 8;

// Multi-query scores (a prefill chunk's query rows scored against the
// cache): problem p = ((layer * batch + b) * H + hk) * n_rg + rg holds rows
// [64 rg, 64 rg + 64) of the KV head's G query rows.  Workgroup w takes the
// chunks [w a.chunks_per_wg, + a.chunks_per_wg) of the problem-major chunk
// sequence (a.chunks_per_problem per problem): it builds its tables once,
// stages each problem's query operands in LDS, and its 8 waves take the
// problem's chunks round robin, one chunk loaded ahead.  Per 32-wide step a
// wave forms the key operands of its chunk once (the decode kernel's table
// lookups) and multiplies them with the 8 column blocks' query operands, so a
// KV head's codes are read and decoded once per 64 rows (the decode kernel's
// scoring takes 8 rows per pass).  Logits as in tq_score (natural units;
// positions past the sequence untouched).
template <int MK>
__global__ __launch_bounds__(kMultiWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void score_multi_kernel(
    DecodeArgs a, int n_rg) {
  constexpr bool KWIDE = MK > 4;
  constexpr bool KSPLIT = MK > 0 && key_split(MK);
  using KL = KLut<(MK > 0 && !KWIDE ? MK : 1)>;
  constexpr int NT = kMultiWaves * 64;
  constexpr int KT = MK > 0 ? (KWIDE ? (1 << MK) : KL::E * KL::EW) : 1;
  constexpr int KP = MK > 0 && !KWIDE && KL::NC > 2 ? KL::PAIRS * KL::PW : 1;
  constexpr int OFF_S = 0;
  constexpr int OFF_K = MK > 0 ? 256 * 16 : 0;
  constexpr int OFF_PHI = OFF_K + KT * 4;
  constexpr int OFF_Q = ((OFF_PHI + KP * 4 + 255) / 256) * 256;
  constexpr int NQ = 8 * 2 * 4 * 64;   // staged query operands [block][r / z][step][lane]
  constexpr int LDS_BYTES = OFF_Q + NQ * 16;
  static_assert(OFF_K < 65536, "the key table must start below 64 KB");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
  __shared__ __align__(256) unsigned char dsm[LDS_BYTES];
  uint32_t* const lut_k = reinterpret_cast<uint32_t*>(dsm + OFF_K);
  uint32_t* const pair_hi = reinterpret_cast<uint32_t*>(dsm + OFF_PHI);
  uint32_t* const lut_s = reinterpret_cast<uint32_t*>(dsm + OFF_S);
  half8* const qst = reinterpret_cast<half8*>(dsm + OFF_Q);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, q = lane >> 4;
  const int cpp = a.chunks_per_problem;
  const int g_lo = int(blockIdx.x) * a.chunks_per_wg;
  const int g_hi = g_lo + a.chunks_per_wg < a.total_chunks ? g_lo + a.chunks_per_wg : a.total_chunks;

  constexpr bool KSCALED = MK > 0 && !KSPLIT;
  const float alpha_k = KSCALED ? a.alpha_k : 1.f;
  const float kscale_k = a.scale / alpha_k, kscale_r = a.scale * a.kappa;
  // ---- tables (as in decode)
  if constexpr (KWIDE) {
    for (int x = tid; x < (1 << MK); x += NT) {
      const float c = a.kc[x];
      const uint16_t h = f16_bits(c);
      reinterpret_cast<uint16_t*>(lut_k)[x] = h;
      reinterpret_cast<uint16_t*>(lut_k)[(1 << MK) + x] = f16_bits(c - float(__builtin_bit_cast(_Float16, h)));
    }
  } else if constexpr (MK > 0) {
    const float kcl = a.kc[lane & ((1 << MK) - 1)] * alpha_k;
    if constexpr (KL::NC > 2)
      build_kpairs<MK>(pair_hi, kcl, tid, NT);
    else
      build_kpairs<MK>(lut_k, kcl, tid, NT);
  }
  if constexpr (MK > 0) {
    for (int x = tid; x < 256; x += NT) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t lo = ((x >> e) & 1) ? 0x3C00u : 0xBC00u;
        const uint32_t hi = ((x >> (e + 1)) & 1) ? 0x3C00u : 0xBC00u;
        lut_s[x * 4 + e / 2] = lo | (hi << 16);
      }
    }
  }
  __syncthreads();
  if constexpr (MK > 0 && !KWIDE && KL::NC > 2) {
    build_ktab<MK, NT>(lut_k, pair_hi, tid);
    __syncthreads();
  }

  // the current problem: its query rows, sequence length, first slot and logits row
  int rows = 0;
  int64_t len = 0, slot_base = 0, out_row0 = 0;

  // ---- chunk data of one lane (tile T row col -> token 8 (col / 4) + 4 T + col % 4)
  constexpr int KREC = MK > 0 ? 16 * MK : 2 * D;
  constexpr int MKW = MK > 0 ? MK : 1;
  struct KData {
    uint32_t kw[2][MKW];
    uint32_t sg[2];
    half8 kf[MK > 0 ? 1 : 2][MK > 0 ? 1 : 4];
    float kn[MK > 0 ? 8 : 1], rn[MK > 0 ? 8 : 1];   // norms of tokens 8 q .. 8 q + 7
  };
  uint32_t koff[2], soff[2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const uint32_t tk = 8 * (col >> 2) + 4 * T + (col & 3);
    koff[T] = tk * KREC + 4 * q * MKW;
    soff[T] = tk * 16 + 4 * q;
  }
  auto load_k = [&](int c, KData& K) {
    const int64_t slot0 = slot_base + int64_t(c) * kChunk;
    if constexpr (MK == 0) {
      const auto kr = chunk_rsrc(a.k_f16 + slot0 * D, kChunk * 2 * D);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        const uint32_t off = (8 * (col >> 2) + 4 * T + (col & 3)) * (2 * D) + 64 * q;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) K.kf[T][s2] = bload<half8>(kr, off + 16 * s2);
      }
    } else {
      const auto kr = chunk_rsrc(a.k_idx + slot0 * KREC, kChunk * KREC);
      const auto sr = chunk_rsrc(a.k_sign + slot0 * 16, kChunk * 16);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
#pragma unroll
        for (int u = 0; u < MK; ++u) K.kw[T][u] = bload<uint32_t>(kr, koff[T] + 4 * u);
        K.sg[T] = bload<uint32_t>(sr, soff[T]);
      }
      const auto nr = chunk_rsrc(a.k_norm + slot0, kChunk * 4), rr = chunk_rsrc(a.k_rnorm + slot0, kChunk * 4);
#pragma unroll
      for (int h4 = 0; h4 < 2; ++h4) {
        const floatx4 n4 = bload<floatx4>(nr, 32 * q + 16 * h4), r4 = bload<floatx4>(rr, 32 * q + 16 * h4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          K.kn[4 * h4 + e] = n4[e];
          K.rn[4 * h4 + e] = r4[e];
        }
      }
    }
  };

  floatx4 sm[8][2], sq[MK > 0 ? 8 : 1][2];
  auto compute = [&](const KData& K, int c) {
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        sm[cb][T] = floatx4{0.f, 0.f, 0.f, 0.f};
        if constexpr (MK > 0) sq[cb][T] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      half8 kh[2], kl[2], sd[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        if constexpr (MK == 0) {
          kh[T] = K.kf[T][s2];
        } else {
          if constexpr (KWIDE)
            deq8_wide<MK>(K.kw[T], s2, reinterpret_cast<const uint16_t*>(lut_k), kh[T], kl[T]);
          else
            deq8_k<MK>(slab_bits<MK>(K.kw[T], s2), lut_k, kh[T], kl[T]);
          sd[T] = *reinterpret_cast<const half8*>(lut_s + ((K.sg[T] >> (8 * s2)) & 0xFFu) * 4);
        }
      }
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        if (cb * 8 < rows) {   // uniform
          const half8 qr = qst[((cb * 2 + 0) * 4 + s2) * 64 + lane];
#pragma unroll
          for (int T = 0; T < 2; ++T) {
            sm[cb][T] = mfma16x16x32(kh[T], qr, sm[cb][T]);
            if constexpr (KSPLIT) sm[cb][T] = mfma16x16x32(kl[T], qr, sm[cb][T]);
          }
          if constexpr (MK > 0) {
            const half8 qz = qst[((cb * 2 + 1) * 4 + s2) * 64 + lane];
#pragma unroll
            for (int T = 0; T < 2; ++T) sq[cb][T] = mfma16x16x32(sd[T], qz, sq[cb][T]);
          }
        }
      }
    }
    // ---- logits: lane (col, q) holds tokens 8 q + e (e = 4 T + i) of column col
    const int64_t crel = int64_t(c) * kChunk;
    const int rem = int(len - crel > kChunk ? kChunk : len - crel) - 8 * q;
    float kn[8], rn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kn[e] = MK > 0 ? K.kn[MK > 0 ? e : 0] : 1.f;
      rn[e] = MK > 0 ? K.rn[MK > 0 ? e : 0] : 0.f;
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      if (cb * 8 < rows) {
        float lg[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float smv = sm[cb][e >> 2][e & 3];
          float t = smv;
          if constexpr (MK > 0) t = fmaf(kn[e], smv, rn[e] * sq[cb][e >> 2][e & 3]);
          lg[e] = t + dpp_f<0x128>(t);   // high part + remainder part (row rotate by 8)
        }
        if (col < 8 && cb * 8 + col < rows) {
          float* out = a.logits + out_row0 + int64_t(cb * 8 + col) * a.max_len + crel + 8 * q;
          if (rem >= 8 && ((a.max_len & 3) == 0)) {   // 16-byte aligned rows: two vector stores
            *reinterpret_cast<float4*>(out) = float4{lg[0], lg[1], lg[2], lg[3]};
            *reinterpret_cast<float4*>(out + 4) = float4{lg[4], lg[5], lg[6], lg[7]};
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e < rem) out[e] = lg[e];
          }
        }
      }
    }
  };

  // ---- query operands: item ((cb * 2 + kind) * 4 + s) * 64 + l; lane (col,
  // q') of block cb, step s holds coordinates 32 q' + 8 s + e of row 8 cb +
  // col % 8 of Pi q * scale / alpha_k (kind 0) or S q * scale * kappa (kind 1)
  auto stage = [&](int layer, int b, int hk, int rg, int rows) {
  for (int it = tid; it < NQ; it += NT) {
    const int l = it & 63, s4 = (it >> 6) & 3, kind = (it >> 8) & 1, cb = it >> 9;
    const int r = cb * 8 + (l & 7);
    const bool ok = r < rows && (MK > 0 || kind == 0);
    const int h = hk * a.G + rg * kMultiRows + (ok ? r : 0);
    const float* src =
        a.qprep + ((int64_t(layer) * a.batch + b) * a.Hq + h) * 2 * D + kind * D + 32 * (l >> 4) + 8 * s4;
    const float sc = ok ? (kind ? kscale_r : kscale_k) : 0.f;
    const bool lo = (l & 15) >= 8;
    half8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = src[e] * sc;
      const _Float16 xh = _Float16(x);
      o[e] = lo ? _Float16(x - float(xh)) : xh;
    }
    qst[it] = o;
  }
  };

  KData K0, K1;
#pragma unroll 1
  for (int g = g_lo; g < g_hi;) {
    const int prob = g / cpp;
    const int seg_hi = (prob + 1) * cpp < g_hi ? (prob + 1) * cpp : g_hi;
    const int rg = prob % n_rg, hk = (prob / n_rg) % a.H, b = (prob / (n_rg * a.H)) % a.batch;
    const int layer = prob / (n_rg * a.H * a.batch);
    rows = a.G - rg * kMultiRows < kMultiRows ? a.G - rg * kMultiRows : kMultiRows;
    // the sequence, with decode's rules (misaligned or negative starts empty)
    int64_t start = a.seq_start[b];
    len = a.seq_len[b];
    if (start < 0 || (start % kVBlock) != 0 || start >= a.capacity || len < 0) {
      len = 0;
      start = 0;
    }
    if (len > a.capacity - start) len = a.capacity - start;
    if (len > a.max_len) len = a.max_len;
    slot_base = (int64_t(layer) * a.H + hk) * a.capacity + start;
    out_row0 = ((int64_t(layer) * a.batch + b) * a.Hq + hk * a.G + rg * kMultiRows) * a.max_len;
    const int n_chunks = int((len + kChunk - 1) / kChunk);
    const int c0 = g - prob * cpp, c1 = seg_hi - prob * cpp < n_chunks ? seg_hi - prob * cpp : n_chunks;
    g = seg_hi;
    if (c0 >= c1) continue;   // uniform over the workgroup
    __syncthreads();          // the previous problem's operands are no longer read
    stage(layer, b, hk, rg, rows);
    __syncthreads();
    int c = c0 + wave;
    if (c < c1) load_k(c, K0);
#pragma unroll 1
    for (; c < c1; c += 2 * kMultiWaves) {
      const int cn = c + kMultiWaves;
      if (cn < c1) load_k(cn, K1);
      compute(K0, c);
      if (cn >= c1) break;
      if (cn + kMultiWaves < c1) load_k(cn + kMultiWaves, K0);
      compute(K1, cn);
    }
  }
}

template <bool SCORE>
tq_status launch_decode(int mk, int bv, const DecodeArgs& args, dim3 grid, hipStream_t st,
                        const CompressArgs& ca = CompressArgs{}) {
#define TQ_DEC(MK_, BV_)                                                                       \
  if (mk == MK_ && bv == BV_) {                                                                \
    hipLaunchKernelGGL((decode_kernel<MK_, BV_, SCORE>), grid, dim3(kDecodeWaves * 64), 0, st, args, ca); \
    return TQ_OK;                                                                              \
  }
#define TQ_DEC_V(MK_) TQ_DEC(MK_, 0) TQ_DEC(MK_, 1) TQ_DEC(MK_, 2) TQ_DEC(MK_, 3) TQ_DEC(MK_, 4)
  if constexpr (SCORE) {
    // Scores do not read values: one instantiation per key format.
    TQ_DEC(0, 0) TQ_DEC(1, 0) TQ_DEC(2, 0) TQ_DEC(3, 0) TQ_DEC(4, 0) TQ_DEC(7, 0)
  } else {
    TQ_DEC_V(0) TQ_DEC_V(1) TQ_DEC_V(2) TQ_DEC_V(3) TQ_DEC_V(4) TQ_DEC_V(7)
  }
#undef TQ_DEC_V
#undef TQ_DEC
  return fail(TQ_ERR_UNSUPPORTED, "no decode kernel for key bits %d / value bits %d", mk, bv);
}

// Launches decode_pair_kernel for part 1's format (part 2: fp16 keys and values).
tq_status launch_decode_pair(int mk, int bv, const DecodeArgs& a1, const CompressArgs& c1, const DecodeArgs& a2,
                             const CompressArgs& c2, int nd1, dim3 grid, hipStream_t st) {
#define TQ_DECP(MK_, BV_)                                                                                      \
  if (mk == MK_ && bv == BV_) {                                                                                \
    hipLaunchKernelGGL((decode_pair_kernel<MK_, BV_>), grid, dim3(kDecodeWaves * 64), 0, st, a1, c1, a2, c2, nd1); \
    return TQ_OK;                                                                                              \
  }
#define TQ_DECP_V(MK_) TQ_DECP(MK_, 0) TQ_DECP(MK_, 1) TQ_DECP(MK_, 2) TQ_DECP(MK_, 3) TQ_DECP(MK_, 4)
  TQ_DECP_V(0) TQ_DECP_V(1) TQ_DECP_V(2) TQ_DECP_V(3) TQ_DECP_V(4) TQ_DECP_V(7)
#undef TQ_DECP_V
#undef TQ_DECP
  return fail(TQ_ERR_UNSUPPORTED, "no decode kernel for key bits %d / value bits %d", mk, bv);
}

tq_status check_tables(const tq_format* f, const tq_tables* t, bool need_sketch) {
  if (!t) return fail(TQ_ERR_INVALID_ARG, "tables is NULL");
  const bool rot = f->k_bits > 0 || f->v_bits > 0;
  if (rot && !t->pi) return fail(TQ_ERR_INVALID_ARG, "tables->pi is NULL");
  if (f->k_bits > 0 && (!t->k_centroids || !t->k_boundaries))
    return fail(TQ_ERR_INVALID_ARG, "key codebook is NULL");
  if (f->v_bits > 0 && (!t->v_centroids || !t->v_boundaries))
    return fail(TQ_ERR_INVALID_ARG, "value codebook is NULL");
  if (f->k_bits > 0 && need_sketch && !t->pi_s) return fail(TQ_ERR_INVALID_ARG, "tables->pi_s is NULL");
  if (f->k_bits > 0 && !need_sketch && !t->s) return fail(TQ_ERR_INVALID_ARG, "tables->s is NULL");
  return TQ_OK;
}

tq_status check_cache(const tq_format* f, const tq_cache* c) {
  if (!c) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  if (c->n_layers <= 0 || c->n_kv_heads <= 0 || c->capacity <= 0 || c->capacity % kVBlock)
    return fail(TQ_ERR_INVALID_ARG, "cache sizes (layers=%d heads=%d capacity=%lld; capacity a positive multiple of 32)",
                c->n_layers, c->n_kv_heads, (long long)c->capacity);
  if (f->k_bits > 0 && (!c->k_idx || !c->k_sign || !c->k_norm || !c->k_rnorm))
    return fail(TQ_ERR_INVALID_ARG, "key planes are NULL");
  if (f->k_bits == 0 && !c->k_f16) return fail(TQ_ERR_INVALID_ARG, "k_f16 plane is NULL");
  if (f->v_bits > 0 && (!c->v_idx || !c->v_norm)) return fail(TQ_ERR_INVALID_ARG, "value planes are NULL");
  if (f->v_bits == 0 && !c->v_f16) return fail(TQ_ERR_INVALID_ARG, "v_f16 plane is NULL");
  return TQ_OK;
}

tq_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return TQ_OK;
}

// Kernel arguments of a decode / score call over `cache` with work split
// `plan` (one slot set: seg_max = plan.seg_max, seg_base = 0).
DecodeArgs make_args(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, int32_t batch,
                     int32_t n_q_heads, const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len,
                     float scale, const SplitPlan& plan, const float* qprep, float* partial, float* out) {
  DecodeArgs a{};
  a.n_layers = cache->n_layers;
  a.batch = batch;
  a.H = cache->n_kv_heads;
  a.Hq = n_q_heads;
  a.G = n_q_heads / cache->n_kv_heads;
  a.n_hg = plan.n_head_groups;
  a.capacity = cache->capacity;
  a.chunks_per_problem = int(plan.chunks_per_problem);
  a.chunks_per_wg = int(plan.chunks_per_wg);
  a.total_chunks = int(plan.problems * plan.chunks_per_problem);
  a.seg_max = int(plan.seg_cap);
  a.cpp_real = int(plan.cpp_real);
  a.cpw_min = int(plan.cpw_min);
  a.ragged = 0;
  a.k_idx = cache->k_idx;
  a.k_sign = cache->k_sign;
  a.k_norm = cache->k_norm;
  a.k_rnorm = cache->k_rnorm;
  a.k_f16 = static_cast<const uint16_t*>(cache->k_f16);
  a.v_idx = cache->v_idx;
  a.v_norm = cache->v_norm;
  a.v_f16 = static_cast<const uint16_t*>(cache->v_f16);
  a.qprep = qprep;
  a.kc = tables->k_centroids;
  a.vc = tables->v_centroids;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.partial = partial;
  a.logits = out;
  a.done = nullptr;
  a.pi = tables->pi;
  a.out = nullptr;
  a.max_len = max_seq_len;
  a.scale = scale != 0.f ? scale : 1.0f / std::sqrt(float(fmt->d));
  a.alpha_k = tables->k_operand_scale >= 1.f && tables->k_operand_scale < 2.f ? tables->k_operand_scale : 1.f;
  a.alpha_v = tables->v_operand_scale >= 1.f && tables->v_operand_scale < 2.f ? tables->v_operand_scale : 1.f;
  a.kappa = float(std::sqrt(M_PI / 2.0) / fmt->d);
  return a;
}

// Decode stages: prepare the query operands (qprep_kernel), score / accumulate
// the chunk runs (decode_kernel), merge the pieces (combine_kernel, or inside
// decode_kernel by the last workgroup of each problem: kStageMerge).
enum {
  kStagePrepare = 1,
  kStagePartials = 2,
  kStageCombine = 4,
  kStageCheckOnly = 8,
  kStageMerge = 16,
  kStageAll = kStagePrepare | kStagePartials | kStageMerge
};

// An append run by the decode launch's first workgroups (tq_decode_step), when
// it takes at most kMaxFusedAppend workgroups.
constexpr int kMaxFusedAppend = 32;
// The bounded wait of a decode wave for the append (see DecodeArgs.app_polls);
// changed only by the test hook tq_set_append_wait.
uint32_t g_append_wait_polls = 1u << 20;
int g_append_wait_extra = 0;
struct FusedAppend {
  CompressArgs ca{};
  int groups = 0;            // append workgroups per layer
  int layers = 0;            // appended layers, from ca.layer0
  int64_t lo = 0, hi = 0;    // plane slots the append may write
};

template <bool SCORE>
tq_status decode_common(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                        const float* q, int32_t batch, int32_t n_q_heads, const int64_t* seq_start,
                        const int32_t* seq_len, int64_t max_seq_len, float scale, float* out,
                        void* workspace, size_t workspace_bytes, void* stream, int stages,
                        const FusedAppend* app = nullptr, int wg_budget = 0, DecodeArgs* args_out = nullptr,
                        int* decode_wgs_out = nullptr) {
  clear_error();
  tq_status st = check_format(fmt, true);
  if (st) return st;
  if ((st = check_tables(fmt, tables, false))) return st;
  if ((st = check_cache(fmt, cache))) return st;
  if ((stages & kStagePrepare) && !q) return fail(TQ_ERR_INVALID_ARG, "q is NULL");
  if ((stages & kStagePartials) && (!seq_start || !seq_len))
    return fail(TQ_ERR_INVALID_ARG, "seq_start/seq_len is NULL");
  if (((stages & (kStageCombine | kStageMerge)) || (SCORE && (stages & kStagePartials))) && !out)
    return fail(TQ_ERR_INVALID_ARG, "output is NULL");
  if (batch <= 0 || n_q_heads <= 0 || n_q_heads % cache->n_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "batch=%d n_q_heads=%d (must be a positive multiple of n_kv_heads=%d)",
                batch, n_q_heads, cache->n_kv_heads);
  if (max_seq_len < 0) return fail(TQ_ERR_INVALID_ARG, "max_seq_len < 0");
  if (int64_t(cache->n_layers) * batch > 65535)
    return fail(TQ_ERR_INVALID_ARG, "n_layers * batch exceeds 65535");
  if ((int64_t(batch) * n_q_heads + kQprepRows - 1) / kQprepRows > 65535)
    return fail(TQ_ERR_INVALID_ARG, "batch * n_q_heads exceeds %d", 65535 * kQprepRows);
  // With an append in the launch, its workgroups take CUs first: the decode
  // split is made for the CUs they leave, so that no decode workgroup waits
  // for a CU (one decode workgroup per CU).
  // (wg_budget > 0: the decode workgroups this call may use, for a launch
  // shared with another call)
  const int app_wgs = app != nullptr ? app->groups * app->layers : 0;
  const SplitPlan plan = plan_decode(fmt->d, cache->n_layers, batch, cache->n_kv_heads, n_q_heads, max_seq_len,
                                     wg_budget > 0 ? wg_budget : kDecodeWorkgroups - app_wgs);
  if (plan.problems * plan.chunks_per_problem > (int64_t(1) << 30))
    return fail(TQ_ERR_INVALID_ARG, "too many 32-token chunks in one call");
  if (!workspace || workspace_bytes < plan.total_bytes)
    return fail(TQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, plan.total_bytes);
  if (stages & kStageCheckOnly) return TQ_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float* qprep = static_cast<float*>(workspace);
  float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.partial_offset);
  uint32_t* done = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + plan.counter_offset);
  const int mk = fmt->k_bits > 0 ? fmt->k_bits - 1 : 0;
  const int bv = fmt->v_bits;
  if (stages & kStagePrepare) {
    const dim3 qgrid = qprep_grid(cache->n_layers, batch, n_q_heads);
    if (fmt->k_bits > 0)
      hipLaunchKernelGGL(qprep_kernel<true>, qgrid, dim3(256), 0, hs, q, tables->pi, tables->s, qprep, batch,
                         cache->n_kv_heads, n_q_heads, done, nullptr);
    else
      hipLaunchKernelGGL(qprep_kernel<false>, qgrid, dim3(256), 0, hs, q, tables->pi, tables->s, qprep, batch,
                         cache->n_kv_heads, n_q_heads, done, nullptr);
    if ((st = launch_status("qprep"))) return st;
  }
  if (max_seq_len == 0 && SCORE) return TQ_OK;

  DecodeArgs a = make_args(fmt, tables, cache, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, plan,
                           qprep, partial, out);
  a.red_g = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.red_offset);
  if (!SCORE && (stages & kStageMerge)) {
    a.done = done;
    a.out = out;
    a.ragged = batch > 1 && batch <= kRaggedMaxBatch ? 1 : 0;
  }
  if (!SCORE && app != nullptr) {
    a.n_app = app->groups * app->layers;
    a.app_groups = app->groups;
    a.app_layer0 = app->ca.layer0;
    a.app_layers = app->layers;
    a.app_lo = app->lo;
    a.app_hi = app->hi;
    a.app_done = done + plan.problems;
    a.app_polls = g_append_wait_polls;
    a.app_extra = g_append_wait_extra;
    a.app_flag = done + plan.problems + cache->n_layers;
  }
  if (int64_t(a.n_app) + plan.n_workgroups > 0x7FFFFFFF) return fail(TQ_ERR_INVALID_ARG, "too many workgroups");
  const dim3 grid(unsigned(a.n_app + plan.n_workgroups));
  if (args_out != nullptr) {   // the caller launches the decode (the preparation is enqueued)
    *args_out = a;
    if (decode_wgs_out != nullptr) *decode_wgs_out = int(plan.n_workgroups);
    return TQ_OK;
  }
  if (stages & kStagePartials) {
    if ((st = launch_decode<SCORE>(mk, SCORE ? 0 : bv, a, grid, hs, app ? app->ca : CompressArgs{}))) return st;
    if ((st = launch_status("decode"))) return st;
  }
  if (!SCORE && (stages & kStageCombine) && !(stages & kStageMerge)) {
    const dim3 cgrid(cache->n_kv_heads, batch, cache->n_layers);
    if (bv > 0)
      hipLaunchKernelGGL(combine_kernel<true>, cgrid, dim3(256), 0, hs, partial, tables->pi, out, batch,
                         cache->n_kv_heads, n_q_heads, a.n_hg, a.chunks_per_problem, a.chunks_per_wg, a.seg_max, 0, 0,
                         0);
    else
      hipLaunchKernelGGL(combine_kernel<false>, cgrid, dim3(256), 0, hs, partial, tables->pi, out, batch,
                         cache->n_kv_heads, n_q_heads, a.n_hg, a.chunks_per_problem, a.chunks_per_wg, a.seg_max, 0, 0,
                         0);
    if ((st = launch_status("combine"))) return st;
  }
  return TQ_OK;
}

}  // namespace
}  // namespace tq

namespace tq {
namespace {
// Decode over a packed cache plus an fp16 tail (see tq_decode_attention_tail):
// the queries are prepared for both parts, each part runs its decode kernel
// into its own slots, and the combine merges the two piece sets.
tq_status decode_tail(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const tq_cache* tail,
                      const float* q, int32_t batch, int32_t n_q_heads, const int64_t* seq_start,
                      const int32_t* seq_len, int64_t max_seq_len, const int64_t* tail_start, const int32_t* tail_len,
                      int64_t max_tail_len, float scale, float* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  tq_status st = check_format(fmt, true);
  if (st) return st;
  if ((st = check_tables(fmt, tables, false))) return st;
  if ((st = check_cache(fmt, cache))) return st;
  const tq_format f16{fmt->d, 0, 0};
  if (!tail) return fail(TQ_ERR_INVALID_ARG, "tail is NULL");
  if ((st = check_cache(&f16, tail))) return st;
  if (tail->n_layers != cache->n_layers || tail->n_kv_heads != cache->n_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "tail has %d layers x %d KV heads, the cache %d x %d", tail->n_layers,
                tail->n_kv_heads, cache->n_layers, cache->n_kv_heads);
  if (!q || !out) return fail(TQ_ERR_INVALID_ARG, "q or out is NULL");
  if (!seq_start || !seq_len || !tail_start || !tail_len)
    return fail(TQ_ERR_INVALID_ARG, "seq_start/seq_len/tail_start/tail_len is NULL");
  if (batch <= 0 || n_q_heads <= 0 || n_q_heads % cache->n_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "batch=%d n_q_heads=%d (must be a positive multiple of n_kv_heads=%d)", batch,
                n_q_heads, cache->n_kv_heads);
  if (max_seq_len < 0 || max_tail_len < 0) return fail(TQ_ERR_INVALID_ARG, "max_seq_len or max_tail_len < 0");
  if (int64_t(cache->n_layers) * batch > 65535) return fail(TQ_ERR_INVALID_ARG, "n_layers * batch exceeds 65535");
  if ((int64_t(batch) * n_q_heads + kQprepRows - 1) / kQprepRows > 65535)
    return fail(TQ_ERR_INVALID_ARG, "batch * n_q_heads exceeds %d", 65535 * kQprepRows);
  const TailPlan tp =
      plan_decode_tail(fmt->d, cache->n_layers, batch, cache->n_kv_heads, n_q_heads, max_seq_len, max_tail_len);
  if (tp.packed.problems * tp.packed.chunks_per_problem > (int64_t(1) << 30) ||
      tp.tail.problems * tp.tail.chunks_per_problem > (int64_t(1) << 30))
    return fail(TQ_ERR_INVALID_ARG, "too many 32-token chunks in one call");
  if (!workspace || workspace_bytes < tp.total_bytes)
    return fail(TQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, tp.total_bytes);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* qrot = reinterpret_cast<float*>(ws);
  float* qplain = reinterpret_cast<float*>(ws + tp.qplain_offset);
  float* partial = reinterpret_cast<float*>(ws + tp.partial_offset);
  uint32_t* done = reinterpret_cast<uint32_t*>(ws + tp.counter_offset);
  const int mk = fmt->k_bits > 0 ? fmt->k_bits - 1 : 0;
  const int bv = fmt->v_bits;
  // One query preparation for both parts (rotated and plain; the plain copy
  // alone for fp16 keys), which also zeroes the merge counts.
  const dim3 qgrid = qprep_grid(cache->n_layers, batch, n_q_heads);
  if (fmt->k_bits > 0)
    hipLaunchKernelGGL(qprep_kernel<true>, qgrid, dim3(256), 0, hs, q, tables->pi, tables->s, qrot, batch,
                       cache->n_kv_heads, n_q_heads, done, qplain);
  else
    hipLaunchKernelGGL(qprep_kernel<false>, qgrid, dim3(256), 0, hs, q, tables->pi, tables->s, qrot, batch,
                       cache->n_kv_heads, n_q_heads, done, nullptr);
  if ((st = launch_status("qprep"))) return st;
  // The tail first (partials only), then the packed part, whose last
  // workgroup per problem merges both piece sets into out.
  float* red_g = reinterpret_cast<float*>(ws + tp.red_offset);
  DecodeArgs at = make_args(&f16, tables, tail, batch, n_q_heads, tail_start, tail_len, max_tail_len, scale,
                            tp.tail, fmt->k_bits > 0 ? qplain : qrot, partial, nullptr);
  at.red_g = red_g;
  at.seg_max = int(tp.seg_total);
  at.seg_base = int(tp.packed.seg_cap);
  if ((st = launch_decode<false>(0, 0, at, dim3(unsigned(tp.tail.n_workgroups)), hs))) return st;
  DecodeArgs ap = make_args(fmt, tables, cache, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, tp.packed,
                            qrot, partial, nullptr);
  ap.seg_max = int(tp.seg_total);
  ap.red_g = red_g;
  ap.done = done;
  ap.out = out;
  ap.tail_base = int(tp.packed.seg_cap);
  ap.tail_cpp = at.chunks_per_problem;
  ap.tail_cpw = at.chunks_per_wg;
  if ((st = launch_decode<false>(mk, bv, ap, dim3(unsigned(tp.packed.n_workgroups)), hs))) return st;
  return launch_status("decode");
}

// Checks a compression call and fills its kernel arguments and bulk
// workgroup count; `nothing` is set when no token or layer is to be written.
tq_status compress_setup(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const void* k,
                         const void* v, int32_t dtype, int32_t layer0, int32_t n_layers, int64_t n_tokens,
                         const int64_t* slots, int64_t slot0, int32_t max_workgroups, CompressArgs& a, int64_t& wgs,
                         bool& nothing) {
  tq_status st = check_format(fmt, true);
  if (st) return st;
  if ((st = check_tables(fmt, tables, true))) return st;
  if ((st = check_cache(fmt, cache))) return st;
  if (dtype != TQ_DTYPE_F32 && dtype != TQ_DTYPE_BF16 && dtype != TQ_DTYPE_F16)
    return fail(TQ_ERR_INVALID_ARG, "dtype=%d", dtype);
  if (n_tokens < 0 || n_layers < 0 || layer0 < 0 || layer0 + n_layers > cache->n_layers)
    return fail(TQ_ERR_INVALID_ARG, "layers [%d, %d) tokens %lld outside the cache", layer0, layer0 + n_layers,
                (long long)n_tokens);
  nothing = n_tokens == 0 || n_layers == 0;
  if (nothing) return TQ_OK;
  if (!k || !v) return fail(TQ_ERR_INVALID_ARG, "k or v is NULL");
  const int64_t tiles = (n_tokens + kCompressTile - 1) / kCompressTile;
  // The bulk kernel holds one workgroup per CU (its LDS), so the flattened
  // (layer, tile) sequence is cut into equal ranges for at most one workgroup
  // per CU of an MI355X, or fewer when the caller bounds the count.
  if (max_workgroups < 0) return fail(TQ_ERR_INVALID_ARG, "max_workgroups=%d", max_workgroups);
  const int64_t cap_wgs = max_workgroups > 0 && max_workgroups < kCompressWorkgroups ? max_workgroups
                                                                                       : kCompressWorkgroups;
  const int64_t total_tiles = tiles * n_layers;
  wgs = total_tiles < cap_wgs ? total_tiles : cap_wgs;
  const int64_t tpw = (total_tiles + wgs - 1) / wgs;
  wgs = (total_tiles + tpw - 1) / tpw;
  if (n_layers > 65535) return fail(TQ_ERR_INVALID_ARG, "too many layers");
  a.k = k;
  a.v = v;
  a.dtype = dtype;
  a.layer0 = layer0;
  a.n_tokens = n_tokens;
  a.slots = slots;
  a.slot0 = slot0;
  a.slot_shift = 0;
  a.H = cache->n_kv_heads;
  a.capacity = cache->capacity;
  a.mk = fmt->k_bits > 0 ? fmt->k_bits - 1 : 0;
  a.bv = fmt->v_bits;
  a.tiles_per_wg = tpw;
  a.total_tiles = total_tiles;
  a.pi = tables->pi;
  a.pi_s = tables->pi_s;
  a.kc = tables->k_centroids;
  a.kb = tables->k_boundaries;
  a.vc = tables->v_centroids;
  a.vb = tables->v_boundaries;
  a.k_idx = cache->k_idx;
  a.k_sign = cache->k_sign;
  a.k_norm = cache->k_norm;
  a.k_rnorm = cache->k_rnorm;
  a.k_f16 = static_cast<uint16_t*>(cache->k_f16);
  a.v_idx = cache->v_idx;
  a.v_norm = cache->v_norm;
  a.v_f16 = static_cast<uint16_t*>(cache->v_f16);
  return TQ_OK;
}
}  // namespace
}  // namespace tq

namespace tq {
namespace {
// A plain streaming read of n float4s (grid-stride, 4 loads in flight per
// thread, non-temporal), one partial sum per workgroup: the reference for the
// achievable HBM read bandwidth.
__global__ __launch_bounds__(256) void stream_read_kernel(const floatx4* __restrict__ p, int64_t n,
                                                          float* __restrict__ out) {
  float acc = 0.f;
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    floatx4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += (v[u][0] + v[u][1]) + (v[u][2] + v[u][3]);
  }
  for (; i < n; i += stride) {
    const floatx4 v = __builtin_nontemporal_load(p + i);
    acc += (v[0] + v[1]) + (v[2] + v[3]);
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) atomicAdd(out + blockIdx.x, acc);
}
}  // namespace
}  // namespace tq

namespace tq {
namespace {
// Scratch of tq_decode_attention_noalloc: the decode workspace (prepared
// queries, piece partials, merge counters, operand scales, wave-merge slices)
// in a file-scope device array, one copy per GPU, held until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host it
// names a stand-in, not the device copy): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(TQ_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch` (NULL with an
// error recorded on failure).
void* scratch_for_current_device() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(TQ_ERR_HIP, "no current device (%s, device %d)", hipGetErrorString(e), dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t se = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (se != hipSuccess || ptr == nullptr) {
      fail(TQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(se));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace
}  // namespace tq

namespace tq {
namespace {
// The fp16 tail tokens that a flush moves into the packed cache: staging row
// r = b * max_flush + i holds token i of sequence b (i < n_flush[b]), tail
// slot tail_pos[b] + i, as [L][rows][H][D] fp16 keys and values; slots[r] is
// its packed slot dst_slot[b] + i, or -1 for a row without a token (or a tail
// slot outside the tail), which the compression skips.  Grid (rows, L).
__global__ __launch_bounds__(256) void tail_gather_kernel(const uint16_t* k16, const uint16_t* v16, int64_t tail_cap,
                                                         int H, int max_flush, const int64_t* tail_pos,
                                                         const int32_t* n_flush, const int64_t* dst_slot,
                                                         uint16_t* sk, uint16_t* sv, int64_t* slots) {
  const int64_t r = blockIdx.x, rows = gridDim.x;
  const int layer = blockIdx.y;
  const int b = int(r / max_flush), i = int(r % max_flush);
  const int64_t ts = tail_pos[b] + i;
  const bool ok = i < n_flush[b] && ts >= 0 && ts < tail_cap;
  if (layer == 0 && threadIdx.x == 0) slots[r] = ok ? dst_slot[b] + i : -1;
  uint16_t* dk = sk + (int64_t(layer) * rows + r) * H * D;
  uint16_t* dv = sv + (int64_t(layer) * rows + r) * H * D;
  for (int e = threadIdx.x; e < H * D; e += blockDim.x) {
    const int h = e / D, j = e % D;
    const int64_t plane = int64_t(layer) * H + h;
    dk[e] = ok ? k16[(plane * tail_cap + ts) * D + j] : uint16_t(0);
    dv[e] = ok ? v16[((plane * (tail_cap / kVBlock) + ts / kVBlock) * D + j) * kVBlock + ts % kVBlock] : uint16_t(0);
  }
}

// Compression (tq_compress_kv_bounded) with slot_shift added to each slots[i].
tq_status compress_run(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const void* k,
                       const void* v, int32_t dtype, int32_t layer0, int32_t n_layers, int64_t n_tokens,
                       const int64_t* slots, int64_t slot0, int32_t max_workgroups, int64_t slot_shift, void* stream) {
  CompressArgs a{};
  int64_t wgs = 0;
  bool nothing = false;
  tq_status st = compress_setup(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0,
                                max_workgroups, a, wgs, nothing);
  if (st || nothing) return st;
  a.slot_shift = slot_shift;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (n_tokens < kCompressTile) {
    // Appends: 8 (token, head) items per workgroup.
    const int64_t groups = (n_tokens * a.H + kAppendItems - 1) / kAppendItems;
#define TQ_APP(MK_, BV_)                                                                               \
  if (a.mk == MK_ && a.bv == BV_) {                                                                    \
    hipLaunchKernelGGL((compress_append_kernel<MK_, BV_>), dim3(unsigned(groups), unsigned(n_layers)), \
                       dim3(kAppendThreads), 0, hs, a);                                                \
    return launch_status("compress (append)");                                                         \
  }
#define TQ_APP_V(MK_) TQ_APP(MK_, 0) TQ_APP(MK_, 1) TQ_APP(MK_, 2) TQ_APP(MK_, 3) TQ_APP(MK_, 4)
    TQ_APP_V(0) TQ_APP_V(1) TQ_APP_V(2) TQ_APP_V(3) TQ_APP_V(4) TQ_APP_V(7)
#undef TQ_APP_V
#undef TQ_APP
    return fail(TQ_ERR_UNSUPPORTED, "no compress kernel for key bits %d / value bits %d", a.mk, a.bv);
  }
  const size_t smem = sizeof(CompressSmem);
  const void* fn = nullptr;
#define TQ_CMP(MK_, BV_)                                                                            \
  if (a.mk == MK_ && a.bv == BV_)                                                                   \
    fn = a.dtype == TQ_DTYPE_F32 ? reinterpret_cast<const void*>(compress_kernel<MK_, BV_, true>)   \
                                 : reinterpret_cast<const void*>(compress_kernel<MK_, BV_, false>);
#define TQ_CMP_V(MK_) TQ_CMP(MK_, 0) TQ_CMP(MK_, 1) TQ_CMP(MK_, 2) TQ_CMP(MK_, 3) TQ_CMP(MK_, 4)
  TQ_CMP_V(0) TQ_CMP_V(1) TQ_CMP_V(2) TQ_CMP_V(3) TQ_CMP_V(4) TQ_CMP_V(7)
#undef TQ_CMP_V
#undef TQ_CMP
  if (!fn) return fail(TQ_ERR_UNSUPPORTED, "no compress kernel for key bits %d / value bits %d", a.mk, a.bv);
  const hipError_t ae = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
  if (ae != hipSuccess)
    return fail(TQ_ERR_HIP, "cannot raise the LDS limit to %zu bytes: %s", smem, hipGetErrorString(ae));
  void* args[] = {&a};
  if (hipLaunchKernel(fn, dim3(unsigned(wgs)), dim3(kCompressWaves * 64), args, smem, hs) != hipSuccess)
    return fail(TQ_ERR_HIP, "compress launch failed: %s", hipGetErrorString(hipGetLastError()));
  return launch_status("compress");
}
}  // namespace
}  // namespace tq

namespace tq {
namespace {
// tq_decode_step_parts (step: each part's append, query preparation and
// decode) and tq_decode_attend_parts (!step: the decode alone, on queries
// prepared in each part's workspace).
tq_status decode_parts(const tq_step_part* parts, int32_t n_parts, bool step, int32_t dtype, int64_t n_tokens,
                       const int64_t* slots, int64_t slot0, int32_t batch, int32_t n_q_heads, const int64_t* seq_start,
                       const int32_t* seq_len, int64_t max_seq_len, float scale, void* stream) {
  clear_error();
  constexpr int kMaxParts = 8;
  if (!parts || n_parts < 1 || n_parts > kMaxParts)
    return fail(TQ_ERR_INVALID_ARG, "n_parts=%d (1 to %d, parts not NULL)", n_parts, kMaxParts);
  // Every part is checked before anything is enqueued.
  FusedAppend app[kMaxParts];
  bool nothing[kMaxParts] = {};
  int64_t app_wgs = 0;
  for (int i = 0; i < n_parts; ++i) {
    const tq_step_part& P = parts[i];
    tq_status st = decode_common<false>(P.fmt, P.tables, P.cache, P.q, batch, n_q_heads, seq_start, seq_len,
                                        max_seq_len, scale, P.out, P.workspace, P.workspace_bytes, stream,
                                        (step ? kStageAll : kStagePartials | kStageMerge) | kStageCheckOnly);
    if (st) return st;
    nothing[i] = true;
    int64_t wgs = 0;
    if (step && (st = compress_setup(P.fmt, P.tables, P.cache, P.k, P.v, dtype, P.layer0, P.n_layers, n_tokens, slots,
                                     slot0, 0, app[i].ca, wgs, nothing[i])))
      return st;
    if (!nothing[i]) {
      const int64_t groups = (n_tokens * app[i].ca.H + kAppendItems - 1) / kAppendItems;
      app[i].groups = int(groups < 0x7FFFFFFF ? groups : 0x7FFFFFFF);
      app[i].layers = P.n_layers;
      app[i].lo = slots ? 0 : slot0;
      app[i].hi = slots ? P.cache->capacity : slot0 + n_tokens;
      app_wgs += groups * P.n_layers;
    }
  }
  // One launch for two parts whose second is fp16 / fp16: the decode
  // workgroups are shared in proportion to each part's cost per token of the
  // batch, taken as the bytes it reads per token-head plus 128 (a 32-token
  // chunk costs a workgroup about as long as reading 4 KB besides its bytes,
  // measured on fp16 keys with 4-bit or fp16 values), and each part's split is
  // made for its share (taken only when both splits fit the given workspaces,
  // which are sized for a launch of their own).
  bool pair = n_parts == 2 && parts[1].fmt->k_bits == 0 && parts[1].fmt->v_bits == 0 &&
              app_wgs <= kMaxFusedAppend && kDecodeWorkgroups - app_wgs >= 2;
  const int nd_total = kDecodeWorkgroups - int(pair ? app_wgs : 0);
  int b1 = 1;
  if (pair) {
    double w[2];
    for (int i = 0; i < 2; ++i) {
      const tq_format* f = parts[i].fmt;
      const int d = f->d;
      const double kb = f->k_bits > 0 ? d * (f->k_bits - 1) / 8 + d / 8 + 8 : 2 * d;
      const double vb = f->v_bits > 0 ? d * f->v_bits / 8 + 4 : 2 * d;
      w[i] = double(parts[i].cache->n_layers) * parts[i].cache->n_kv_heads * (kb + vb + 128);
    }
    b1 = int(double(nd_total) * w[0] / (w[0] + w[1]) + 0.5);
    b1 = b1 < 1 ? 1 : (b1 > nd_total - 1 ? nd_total - 1 : b1);
    // workgroups part 2's split leaves unused (an aligned split may take
    // fewer than its share) go to part 1
    {
      const tq_step_part& P = parts[1];
      const SplitPlan p2 = plan_decode(P.fmt->d, P.cache->n_layers, batch, P.cache->n_kv_heads, n_q_heads,
                                       max_seq_len, nd_total - b1);
      b1 = nd_total - int(p2.n_workgroups);
    }
    for (int i = 0; i < 2; ++i) {
      const tq_step_part& P = parts[i];
      const SplitPlan plan = plan_decode(P.fmt->d, P.cache->n_layers, batch, P.cache->n_kv_heads, n_q_heads,
                                         max_seq_len, i == 0 ? b1 : nd_total - b1);
      if (P.workspace_bytes < plan.total_bytes) pair = false;
    }
  }
  if (!pair) {
    for (int i = 0; i < n_parts; ++i) {
      const tq_step_part& P = parts[i];
      const tq_status st =
          step ? tq_decode_step(P.fmt, P.tables, P.cache, P.k, P.v, dtype, P.layer0, P.n_layers, n_tokens, slots,
                                slot0, P.q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, P.out,
                                P.workspace, P.workspace_bytes, stream)
               : tq_decode_attend(P.fmt, P.tables, P.cache, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale,
                                  P.out, P.workspace, P.workspace_bytes, stream);
      if (st) return st;
    }
    return TQ_OK;
  }
  DecodeArgs a[2];
  int nd[2] = {0, 0};
  for (int i = 0; i < 2; ++i) {
    const tq_step_part& P = parts[i];
    // the part's decode arguments (nothing is enqueued)
    const tq_status st = decode_common<false>(P.fmt, P.tables, P.cache, P.q, batch, n_q_heads, seq_start, seq_len,
                                              max_seq_len, scale, P.out, P.workspace, P.workspace_bytes, stream,
                                              kStagePartials | kStageMerge, nothing[i] ? nullptr : &app[i],
                                              i == 0 ? b1 : nd_total - b1, &a[i], &nd[i]);
    if (st) return st;
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const tq_format* f0 = parts[0].fmt;
  if (step) {
    // both query preparations in one launch (they also zero the parts' merge
    // and append counts)
    const int runs = (batch * n_q_heads + kQprepRows - 1) / kQprepRows;
    const int64_t blocks = int64_t(4) * (parts[0].cache->n_layers + parts[1].cache->n_layers) * runs;
    if (blocks > 0x7FFFFFFF) return fail(TQ_ERR_INVALID_ARG, "too many query preparation blocks");
    float* qp[2] = {static_cast<float*>(parts[0].workspace), static_cast<float*>(parts[1].workspace)};
    if (f0->k_bits > 0)
      hipLaunchKernelGGL(qprep_pair_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, hs, parts[0].q,
                         parts[0].tables->pi, parts[0].tables->s, qp[0], a[0].done, parts[0].cache->n_kv_heads,
                         parts[0].cache->n_layers, parts[1].q, qp[1], a[1].done, parts[1].cache->n_kv_heads,
                         parts[1].cache->n_layers, batch, n_q_heads);
    else
      hipLaunchKernelGGL(qprep_pair_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, hs, parts[0].q,
                         parts[0].tables->pi, parts[0].tables->s, qp[0], a[0].done, parts[0].cache->n_kv_heads,
                         parts[0].cache->n_layers, parts[1].q, qp[1], a[1].done, parts[1].cache->n_kv_heads,
                         parts[1].cache->n_layers, batch, n_q_heads);
    tq_status st = launch_status("qprep (two parts)");
    if (st) return st;
  }
  const dim3 grid(unsigned(a[0].n_app + a[1].n_app + nd[0] + nd[1]));
  const tq_status st = launch_decode_pair(f0->k_bits > 0 ? f0->k_bits - 1 : 0, f0->v_bits, a[0], app[0].ca, a[1],
                                          app[1].ca, nd[0], grid, hs);
  if (st) return st;
  return launch_status("decode (two parts)");
}

}  // namespace
}  // namespace tq

extern "C" {

tq_status tq_decode_attention_noalloc(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                                      const float* q, int32_t batch, int32_t n_q_heads, const int64_t* seq_start,
                                      const int32_t* seq_len, int64_t max_seq_len, float scale, float* out,
                                      void* stream) {
  using namespace tq;
  clear_error();
  tq_status st = check_format(fmt, true);
  if (st) return st;
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "cache is NULL");
  if (batch <= 0 || n_q_heads <= 0 || cache->n_kv_heads <= 0 || n_q_heads % cache->n_kv_heads ||
      max_seq_len < 0 || cache->n_layers <= 0)
    return fail(TQ_ERR_INVALID_ARG, "batch=%d n_q_heads=%d n_kv_heads=%d n_layers=%d max_seq_len=%lld", batch,
                n_q_heads, cache->n_kv_heads, cache->n_layers, (long long)max_seq_len);
  const size_t need = plan_decode(fmt->d, cache->n_layers, batch, cache->n_kv_heads, n_q_heads, max_seq_len)
                          .total_bytes;
  if (need > kNoAllocScratchBytes)
    return fail(TQ_ERR_WORKSPACE, "these sizes need %zu bytes of decode scratch; the static scratch holds %zu",
                need, kNoAllocScratchBytes);
  void* ws = scratch_for_current_device();
  if (!ws) return TQ_ERR_HIP;
  return decode_common<false>(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, out,
                              ws, kNoAllocScratchBytes, stream, kStageAll);
}

tq_status tq_stream_read_probe(const void* data, size_t bytes, float* partial, int32_t n_workgroups, void* stream) {
  tq::clear_error();
  if (!data || !partial || n_workgroups <= 0 || bytes % 16 != 0)
    return tq::fail(TQ_ERR_INVALID_ARG, "stream probe: data/partial NULL, n_workgroups <= 0 or bytes not a multiple of 16");
  hipLaunchKernelGGL(tq::stream_read_kernel, dim3(unsigned(n_workgroups)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const tq::floatx4*>(data), int64_t(bytes / 16),
                     partial);
  return tq::launch_status("stream read probe");
}

tq_status tq_compress_kv(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                         const void* k, const void* v, int32_t dtype, int32_t layer0,
                         int32_t n_layers, int64_t n_tokens, const int64_t* slots, int64_t slot0,
                         void* stream) {
  return tq_compress_kv_bounded(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0, 0,
                                stream);
}

tq_status tq_compress_kv_bounded(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                                 const void* k, const void* v, int32_t dtype, int32_t layer0, int32_t n_layers,
                                 int64_t n_tokens, const int64_t* slots, int64_t slot0, int32_t max_workgroups,
                                 void* stream) {
  tq::clear_error();
  return tq::compress_run(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0, max_workgroups,
                          0, stream);
}

tq_status tq_tail_append(const tq_format* fmt, const tq_tables* tables, const tq_cache* tail, const void* k,
                         const void* v, int32_t dtype, int32_t layer0, int32_t n_layers, int64_t n_tokens,
                         const int64_t* ring_slots, int64_t ring_cap, void* stream) {
  using namespace tq;
  clear_error();
  if (!fmt) return fail(TQ_ERR_INVALID_ARG, "format is NULL");
  if (!tail) return fail(TQ_ERR_INVALID_ARG, "tail is NULL");
  if (ring_cap <= 0 || ring_cap % kVBlock != 0 || 2 * ring_cap > tail->capacity)
    return fail(TQ_ERR_INVALID_ARG, "ring_cap=%lld (a positive multiple of 32, at most half the tail's capacity %lld)",
                (long long)ring_cap, (long long)tail->capacity);
  if (n_tokens > 0 && !ring_slots) return fail(TQ_ERR_INVALID_ARG, "ring_slots is NULL");
  const tq_format f16{fmt->d, 0, 0};
  tq_status st = compress_run(&f16, tables, tail, k, v, dtype, layer0, n_layers, n_tokens, ring_slots, 0, 0, 0, stream);
  if (st) return st;
  return compress_run(&f16, tables, tail, k, v, dtype, layer0, n_layers, n_tokens, ring_slots, 0, 0, ring_cap, stream);
}

size_t tq_tail_flush_workspace_bytes(const tq_format* fmt, const tq_cache* packed, int32_t batch, int32_t max_flush) {
  if (!fmt || !packed || batch <= 0 || max_flush < 0) return 0;
  const size_t rows = size_t(batch) * size_t(max_flush);
  const size_t plane = (size_t(packed->n_layers) * rows * packed->n_kv_heads * fmt->d * 2 + 255) & ~size_t(255);
  return 2 * plane + rows * sizeof(int64_t);
}

tq_status tq_tail_flush(const tq_format* fmt, const tq_tables* tables, const tq_cache* packed, const tq_cache* tail,
                        int32_t batch, int32_t max_flush, const int64_t* tail_pos, const int32_t* n_flush,
                        const int64_t* dst_slot, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace tq;
  clear_error();
  tq_status st = check_format(fmt, true);
  if (st) return st;
  if (!packed || !tail) return fail(TQ_ERR_INVALID_ARG, "packed or tail is NULL");
  const tq_format f16{fmt->d, 0, 0};
  if ((st = check_cache(fmt, packed)) || (st = check_cache(&f16, tail))) return st;
  if (tail->n_layers != packed->n_layers || tail->n_kv_heads != packed->n_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "tail has %d layers x %d KV heads, the packed cache %d x %d", tail->n_layers,
                tail->n_kv_heads, packed->n_layers, packed->n_kv_heads);
  if (batch <= 0 || max_flush < 0) return fail(TQ_ERR_INVALID_ARG, "batch=%d max_flush=%d", batch, max_flush);
  if (max_flush == 0) return TQ_OK;
  if (!tail_pos || !n_flush || !dst_slot) return fail(TQ_ERR_INVALID_ARG, "tail_pos, n_flush or dst_slot is NULL");
  const int64_t rows = int64_t(batch) * max_flush;
  if (rows > 0x7FFFFFFF || packed->n_layers > 65535) return fail(TQ_ERR_INVALID_ARG, "flush too large");
  const size_t need = tq_tail_flush_workspace_bytes(fmt, packed, batch, max_flush);
  if (!workspace || workspace_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  const size_t plane = (need - size_t(rows) * sizeof(int64_t)) / 2;
  uint16_t* sk = static_cast<uint16_t*>(workspace);
  uint16_t* sv = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + plane);
  int64_t* slots = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + 2 * plane);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(tail_gather_kernel, dim3(unsigned(rows), unsigned(packed->n_layers)), dim3(256), 0, hs,
                     static_cast<const uint16_t*>(tail->k_f16), static_cast<const uint16_t*>(tail->v_f16),
                     tail->capacity, packed->n_kv_heads, max_flush, tail_pos, n_flush, dst_slot, sk, sv, slots);
  if ((st = launch_status("tail gather"))) return st;
  return compress_run(fmt, tables, packed, sk, sv, TQ_DTYPE_F16, 0, packed->n_layers, rows, slots, 0, 0, 0, stream);
}

tq_status tq_append_prepare(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                            const void* k, const void* v, int32_t dtype, int32_t layer0, int32_t n_layers,
                            int64_t n_tokens, const int64_t* slots, int64_t slot0, const float* q, int32_t batch,
                            int32_t n_q_heads, int64_t max_seq_len, void* workspace, size_t workspace_bytes,
                            void* stream) {
  using namespace tq;
  // Both halves are checked before anything is launched.
  tq_status st = decode_common<false>(fmt, tables, cache, q, batch, n_q_heads, nullptr, nullptr, max_seq_len, 0.f,
                                      nullptr, workspace, workspace_bytes, stream, kStagePrepare | kStageCheckOnly);
  if (st) return st;
  CompressArgs a{};
  int64_t wgs = 0;
  bool nothing = false;
  if ((st = compress_setup(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0, 0, a, wgs,
                           nothing)))
    return st;
  if (nothing || n_tokens >= kCompressTile) {
    // Bulk (or no) compression: the two calls one after the other.
    if (!nothing && (st = tq_compress_kv(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0,
                                         stream)))
      return st;
    return tq_decode_prepare(fmt, tables, cache, q, batch, n_q_heads, max_seq_len, workspace, workspace_bytes,
                             stream);
  }
  const int64_t groups = (n_tokens * a.H + kAppendItems - 1) / kAppendItems;
  const int64_t n_append = groups * n_layers;
  // (quarter, layer, run) preparation blocks
  const int64_t n_prep = int64_t(4) * cache->n_layers * ((int64_t(batch) * n_q_heads + kQprepRows - 1) / kQprepRows);
  if (n_append + n_prep > 0x7FFFFFFF) return fail(TQ_ERR_INVALID_ARG, "too many workgroups");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float* qprep = static_cast<float*>(workspace);
  const SplitPlan plan = plan_decode(fmt->d, cache->n_layers, batch, cache->n_kv_heads, n_q_heads, max_seq_len);
  uint32_t* done = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + plan.counter_offset);
  const dim3 grid(unsigned(n_append + n_prep));
#define TQ_AP(MK_, BV_)                                                                                          \
  if (a.mk == MK_ && a.bv == BV_) {                                                                              \
    hipLaunchKernelGGL((append_prepare_kernel<MK_, BV_>), grid, dim3(kAppendThreads), 0, hs, a, int(groups),     \
                       int(n_append),                                                                          \
                       q, tables->pi, tables->s, qprep, batch, cache->n_kv_heads, n_q_heads, done,            \
                       cache->n_layers);                                                                       \
    return launch_status("append + prepare");                                                                  \
  }
#define TQ_AP_V(MK_) TQ_AP(MK_, 0) TQ_AP(MK_, 1) TQ_AP(MK_, 2) TQ_AP(MK_, 3) TQ_AP(MK_, 4)
  TQ_AP_V(0) TQ_AP_V(1) TQ_AP_V(2) TQ_AP_V(3) TQ_AP_V(4) TQ_AP_V(7)
#undef TQ_AP_V
#undef TQ_AP
  return fail(TQ_ERR_UNSUPPORTED, "no compress kernel for key bits %d / value bits %d", a.mk, a.bv);
}

tq_status tq_decode_step(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const void* k,
                         const void* v, int32_t dtype, int32_t layer0, int32_t n_layers, int64_t n_tokens,
                         const int64_t* slots, int64_t slot0, const float* q, int32_t batch, int32_t n_q_heads,
                         const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len, float scale,
                         float* out, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace tq;
  // Both halves are checked before anything is launched.
  tq_status st = decode_common<false>(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale,
                                      out, workspace, workspace_bytes, stream, kStageAll | kStageCheckOnly);
  if (st) return st;
  FusedAppend app;
  int64_t wgs = 0;
  bool nothing = false;
  if ((st = compress_setup(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0, 0, app.ca, wgs,
                           nothing)))
    return st;
  if (nothing)
    return tq_decode_attention(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, stream);
  const int64_t groups = (n_tokens * app.ca.H + kAppendItems - 1) / kAppendItems;
  if (groups * n_layers > kMaxFusedAppend) {
    // Many append workgroups would take too many of the decode's CUs: the
    // append runs before the decode, in the query preparation's launch (few
    // tokens) or as the bulk compression (16 or more).
    if (n_tokens < kCompressTile) {
      if ((st = tq_append_prepare(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0, q,
                                  batch, n_q_heads, max_seq_len, workspace, workspace_bytes, stream)))
        return st;
      return tq_decode_attend(fmt, tables, cache, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, out,
                              workspace, workspace_bytes, stream);
    }
    if ((st = tq_compress_kv(fmt, tables, cache, k, v, dtype, layer0, n_layers, n_tokens, slots, slot0, stream)))
      return st;
    return tq_decode_attention(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, stream);
  }
  app.groups = int(groups);
  app.layers = n_layers;
  // Slots the append may write: known on the host for consecutive slots,
  // otherwise any slot of the plane.
  app.lo = slots ? 0 : slot0;
  app.hi = slots ? cache->capacity : slot0 + n_tokens;
  return decode_common<false>(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, out,
                              workspace, workspace_bytes, stream, kStageAll, &app);
}

tq_status tq_decode_step_parts(const tq_step_part* parts, int32_t n_parts, int32_t dtype, int64_t n_tokens,
                               const int64_t* slots, int64_t slot0, int32_t batch, int32_t n_q_heads,
                               const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len, float scale,
                               void* stream) {
  return tq::decode_parts(parts, n_parts, true, dtype, n_tokens, slots, slot0, batch, n_q_heads, seq_start, seq_len,
                          max_seq_len, scale, stream);
}

tq_status tq_decode_attend_parts(const tq_step_part* parts, int32_t n_parts, int32_t batch, int32_t n_q_heads,
                                 const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len, float scale,
                                 void* stream) {
  return tq::decode_parts(parts, n_parts, false, TQ_DTYPE_F32, 0, nullptr, 0, batch, n_q_heads, seq_start, seq_len,
                          max_seq_len, scale, stream);
}

tq_status tq_decode_step_check(const tq_format* fmt, int32_t n_layers, int32_t batch, int32_t n_kv_heads,
                               int32_t n_q_heads, int64_t max_seq_len, const void* workspace, size_t workspace_bytes,
                               void* stream) {
  using namespace tq;
  clear_error();
  tq_status st = check_format(fmt, false);
  if (st) return st;
  if (n_layers <= 0 || batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads || max_seq_len < 0)
    return fail(TQ_ERR_INVALID_ARG, "sizes");
  const SplitPlan plan = plan_decode(fmt->d, n_layers, batch, n_kv_heads, n_q_heads, max_seq_len);
  if (!workspace || workspace_bytes < plan.total_bytes)
    return fail(TQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, plan.total_bytes);
  const hipError_t se = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (se != hipSuccess) return fail(TQ_ERR_HIP, "stream synchronize: %s", hipGetErrorString(se));
  uint32_t flag = 0;
  const char* p = static_cast<const char*>(workspace) + plan.counter_offset +
                  (size_t(plan.problems) + size_t(n_layers)) * sizeof(uint32_t);
  const hipError_t ce = hipMemcpy(&flag, p, sizeof(flag), hipMemcpyDeviceToHost);
  if (ce != hipSuccess) return fail(TQ_ERR_HIP, "reading the step flag: %s", hipGetErrorString(ce));
  if (flag != 0)
    return fail(TQ_ERR_APPEND_TIMEOUT, "a decode wave stopped waiting for the step's append and read chunks that "
                                       "may not hold the new tokens");
  return TQ_OK;
}

tq_status tq_set_append_wait(uint32_t max_polls, int32_t extra_groups) {
  tq::clear_error();
  if (max_polls == 0 || extra_groups < 0) return tq::fail(TQ_ERR_INVALID_ARG, "max_polls=%u extra_groups=%d",
                                                          max_polls, extra_groups);
  tq::g_append_wait_polls = max_polls;
  tq::g_append_wait_extra = extra_groups;
  return TQ_OK;
}

tq_status tq_decode_attention_tail(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                                   const tq_cache* tail, const float* q, int32_t batch, int32_t n_q_heads,
                                   const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len,
                                   const int64_t* tail_start, const int32_t* tail_len, int64_t max_tail_len,
                                   float scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  tq::clear_error();
  return tq::decode_tail(fmt, tables, cache, tail, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, tail_start,
                         tail_len, max_tail_len, scale, out, workspace, workspace_bytes, stream);
}

tq_status tq_decode_attention(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                              const float* q, int32_t batch, int32_t n_q_heads,
                              const int64_t* seq_start, const int32_t* seq_len,
                              int64_t max_seq_len, float scale, float* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return tq::decode_common<false>(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len,
                                  scale, out, workspace, workspace_bytes, stream, tq::kStageAll);
}

tq_status tq_decode_prepare(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const float* q,
                            int32_t batch, int32_t n_q_heads, int64_t max_seq_len, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return tq::decode_common<false>(fmt, tables, cache, q, batch, n_q_heads, nullptr, nullptr, max_seq_len, 0.f,
                                  nullptr, workspace, workspace_bytes, stream, tq::kStagePrepare);
}

tq_status tq_decode_partials(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, int32_t batch,
                             int32_t n_q_heads, const int64_t* seq_start, const int32_t* seq_len,
                             int64_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return tq::decode_common<false>(fmt, tables, cache, nullptr, batch, n_q_heads, seq_start, seq_len, max_seq_len,
                                  scale, nullptr, workspace, workspace_bytes, stream, tq::kStagePartials);
}

tq_status tq_decode_attend(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, int32_t batch,
                           int32_t n_q_heads, const int64_t* seq_start, const int32_t* seq_len, int64_t max_seq_len,
                           float scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return tq::decode_common<false>(fmt, tables, cache, nullptr, batch, n_q_heads, seq_start, seq_len, max_seq_len,
                                  scale, out, workspace, workspace_bytes, stream,
                                  tq::kStagePartials | tq::kStageMerge);
}

tq_status tq_decode_combine(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, int32_t batch,
                            int32_t n_q_heads, int64_t max_seq_len, float* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return tq::decode_common<false>(fmt, tables, cache, nullptr, batch, n_q_heads, nullptr, nullptr, max_seq_len, 0.f,
                                  out, workspace, workspace_bytes, stream, tq::kStageCombine);
}

tq_status tq_score_multi(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache, const float* q,
                         int32_t batch, int32_t n_q_heads, const int64_t* seq_start, const int32_t* seq_len,
                         int64_t max_seq_len, float scale, float* logits, void* workspace, size_t workspace_bytes,
                         void* stream) {
  using namespace tq;
  clear_error();
  // the checks and the query preparation of tq_score
  tq_status st = decode_common<true>(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale,
                                     logits, workspace, workspace_bytes, stream, kStagePrepare | kStagePartials |
                                                                                     kStageCheckOnly);
  if (st) return st;
  if (!seq_start || !seq_len) return fail(TQ_ERR_INVALID_ARG, "seq_start/seq_len is NULL");
  st = decode_common<true>(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, logits,
                           workspace, workspace_bytes, stream, kStagePrepare);
  if (st || max_seq_len == 0) return st;
  const int G = n_q_heads / cache->n_kv_heads;
  const int n_rg = (G + kMultiRows - 1) / kMultiRows;
  const int64_t problems = int64_t(cache->n_layers) * batch * cache->n_kv_heads * n_rg;
  const int64_t cpp = (max_seq_len + kChunk - 1) / kChunk;
  const int64_t total = problems * cpp;
  if (total > (int64_t(1) << 30)) return fail(TQ_ERR_INVALID_ARG, "too many 32-token chunks in one call");
  const int mk = fmt->k_bits > 0 ? fmt->k_bits - 1 : 0;
  // the workgroups one launch keeps resident (one per CU with the 64 KB key
  // table of 3-bit codes, else two), each with at least one chunk per wave
  const int64_t resident = int64_t(kDecodeWorkgroups) * (mk == 3 ? 1 : 2);
  int64_t wgs = (total + kMultiWaves - 1) / kMultiWaves;
  if (wgs > resident) wgs = resident;
  const int64_t cpw = (total + wgs - 1) / wgs;
  wgs = (total + cpw - 1) / cpw;
  const SplitPlan plan = plan_decode(fmt->d, cache->n_layers, batch, cache->n_kv_heads, n_q_heads, max_seq_len);
  DecodeArgs a = make_args(fmt, tables, cache, batch, n_q_heads, seq_start, seq_len, max_seq_len, scale, plan,
                           static_cast<const float*>(workspace), nullptr, logits);
  a.chunks_per_problem = int(cpp);
  a.total_chunks = int(total);
  a.chunks_per_wg = int(cpw);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(wgs));
#define TQ_SM(MK_)                                                                                   \
  if (mk == MK_) {                                                                                   \
    hipLaunchKernelGGL((score_multi_kernel<MK_>), grid, dim3(kMultiWaves * 64), 0, hs, a, n_rg);     \
    return launch_status("score (multi-query)");                                                     \
  }
  TQ_SM(0) TQ_SM(1) TQ_SM(2) TQ_SM(3) TQ_SM(4) TQ_SM(7)
#undef TQ_SM
  return fail(TQ_ERR_UNSUPPORTED, "no multi-query score kernel for key bits %d", mk);
}

tq_status tq_score(const tq_format* fmt, const tq_tables* tables, const tq_cache* cache,
                   const float* q, int32_t batch, int32_t n_q_heads, const int64_t* seq_start,
                   const int32_t* seq_len, int64_t max_seq_len, float scale, float* logits,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return tq::decode_common<true>(fmt, tables, cache, q, batch, n_q_heads, seq_start, seq_len, max_seq_len,
                                 scale, logits, workspace, workspace_bytes, stream,
                                 tq::kStagePrepare | tq::kStagePartials);
}

}  // extern "C"
