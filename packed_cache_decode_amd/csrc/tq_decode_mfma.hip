// tq_decode on gfx950 matrix cores: split-KV paged decode attention over
// packed slots for head_dim 128 (4- or 3-bit Lloyd-Max keys, or FP8 E4M3
// keys), block sizes that are multiples of 16, any number of query heads per
// kv head (passes of 16); and, by one direct kernel, head dims 64 and 256 on
// the slotted page with up to 16 query heads per kv head.
//
// What is computed is the same as in the general kernel (tq_decode.hip),
// following P1 ("vLLM 源码完全拆解(十九):TurboQuant KV Cache 量化"),
// sections "分数计算" (q_rot . centroid, stored norm, norm correction
// 1/sqrt(sum c^2 + 1e-16)), "FP8 K" (q . k, keys unrotated), "V 的解包"
// (code * scale + zero), "在线 softmax" and "读取内核" (split partials,
// log-sum-exp merge).
//
// Kernels.  Four kernels walk a split's keys 16 tokens at a time (a slab:
// 16 rows of a page); they differ in how the slab's bytes reach the lanes,
// and each section below states its mapping:
//   direct  (decode_slab_kernel)    one wavefront per (split, sequence, kv
//           head); every lane buffer-loads exactly its operand bytes
//   staged  (decode_staged_kernel)  the same wavefronts; 16-byte loads of the
//           head's row span, parked in a private LDS buffer
//   page    (decode_page_kernel)    one workgroup per (sequence, split), one
//           wavefront per kv head of a row group; whole slabs into an LDS
//           ring by non-temporal loads that write LDS directly (FP8 keys)
//   ring    (decode_ring_kernel)    one workgroup per (sequence, kv head,
//           split); every wavefront claims slabs and streams them into its
//           own LDS ring (3/4-bit keys, slotted and split pages)
//   dslab   (decode_dslab_kernel)   the direct kernel's design at head dims
//           64 and 256 (its own section below)
// decode_merge_kernel merges the split partials by log-sum-exp (a fused
// last-workgroup merge needs a device-scope release in every workgroup,
// which on this part costs far more than a launch).
//
// Contractions, 16x16 MFMA tiles:
//   scores  S[t][h] = sum_c C[t][c] Q[h][c]     v_mfma_f32_16x16x32_f16 / _bf16
//   norms   N[t][t] = sum_c C[t][c] C[t][c]     diagonal of C C^T (MSE keys)
//   values  O[h][c] += sum_t W[h][t] V[t][c]    v_mfma_f32_16x16x32_f16 (direct, staged)
//                                               v_mfma_f32_16x16x16_f16 (page, ring)
// For MSE keys C are the centroids of the slab's K codes, looked up per code
// byte (two codes) in an LDS table.  f16 alone is not precise enough for the
// scores (centroids rounded to f16 move the decode output by up to 2.7e-3
// on outlier-channel keys), so centroids and rotated queries are carried as
// f16 hi + lo pairs; the table and operand layouts of each kernel are given
// with it.  FP8 keys convert exactly to bf16 and meet the bf16 query
// directly.  Q holds the (rotated) queries, rows >= G zero.  V operands are
// the integer codes as exact f16 integers, W = p * scale as an f16 hi + lo
// pair: side by side in k (direct, staged kernels), or in tile rows h and
// h + 8 (page, ring kernels, at most 8 query heads per kv head).  The
// per-token term zero * p and the softmax sums stay in fp32.  The running
// maximum is lazy: the accumulators are rescaled only when a head's maximum
// grows by more than kLazy (base 2), so p <= 2^kLazy.
//
// Layouts (lane l, row r16 = l % 16, group g4 = l / 16):
//   A operand  : row r16, k = [8*g4, 8*g4+8) (x32) or [4*g4, 4*g4+4) (x16)
//   B operand  : column r16, same k
//   D          : column r16, rows 4*g4 .. 4*g4+3
// Coordinates are permuted so each lane reads contiguous bytes: score MFMA
// kk in group g4 covers coordinates 32*g4 + 8*kk + [0, 8); value tile m,
// column j covers coordinate 8*j + m.
#include <cstddef>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));

constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLoScale = 2048.0f;          // lo parts are stored x 2^11
constexpr int kRec = kD + 4;                 // partial record: O[128], m, l, z, pad
constexpr float kLazy = 6.0f;                // rescale when the max grows by > 2^6
constexpr int kMaxChunkPages = 256;          // pages of one split (byte offsets in LDS)
constexpr int kBufferWord3 = 0x00020000;     // raw buffer resource, 32-bit data format (gfx9 family)

struct MfmaArgs {
  const DevTables* tables;
  DevErrors* errs;
  const uint16_t* q;
  const uint8_t* cache;
  int64_t num_blocks;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seq_lens;
  int Hq;
  int H;
  int G;               // query heads of this pass (per kv head)
  int Gq;              // query heads per kv head in q, out and the partials
  int h0;              // first query head (of its kv head) of this pass
  int bs_shift;
  int chunk;           // tokens per split, a multiple of 16
  int num_splits;
  int batch;
  float scale_log2;    // sm_scale * log2(e)
  float* part;         // [B][Hq][S][kRec]
  void* out;
  int out_fp32;
  int dynamic;         // ring kernel: wavefronts claim slabs from a shared counter
  const float* q_rot;  // Haar rotation: the rotated queries [B][Hq][d] (fp32), else null
  const int32_t* order;  // ring kernel: sequence of each length rank (longest first), else null
};

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// reductions over the lane pair (l, l ^ 16) and (l, l ^ 32)
__device__ __forceinline__ float max_x16(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
// a word as two halves, taken by value: __builtin_bit_cast applied directly
// to an element of a vector register value reads element 0 whatever the
// subscript (seen with this compiler), so elements go through a copy
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

__device__ __forceinline__ float sum_x16(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// lanes 8 .. 15 of each row of 16 take the value of lane - 8 (a row rotation
// by 8 written to DPP banks 2 and 3 only): the P.V lo rows then work from
// exactly the scores of their head
__device__ __forceinline__ float copy_to_upper8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x128, 0xF, 0xC, false));
}
__device__ __forceinline__ float lane_value(float x, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(x)));
}

// Row values to MFMA tile rows without LDS: lane (i, g) = lane 16*g + i holds
// v_i, significant where g == i >> 2; returns, as element r, v of row
// 4*g4 + r (the D layout of a 16x16 MFMA).  One 16x16x4 f32 MFMA with
// A[i][k] = (k == i >> 2 ? v_i : 0) and B = 1, so D[i][j] = v_i exactly.
__device__ __forceinline__ f4 rows_to_tile(float v, bool diag) {
  const f4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x4f32(diag ? v : 0.0f, 1.0f, z, 0, 0, 0);
}

// Running state of one wavefront (G query heads of one kv head).
struct RunState {
  f4 O[8];          // O[h][8*r16 + m]: tile m, rows 4*g4 + r
  float m_run;      // running (lazy) max, base 2, of head r16
  float l_part;     // sum of p over this lane's rows, head r16
  float z_part;     // sum of p * zero over this lane's rows, head r16
};

// Operand bytes of one slab for one lane, already re-aligned.
template <int KB>
struct SlabOps {
  uint32_t kw[KB == 4 ? 4 : 3];   // K codes of token r16, coordinates [32*g4, 32*g4 + 32)
  uint32_t X[4];                  // V codes of token 4*g4 + r, coordinates [8*r16, 8*r16 + 8)
  uint32_t n[4];                  // K norm (f16 bits) of token 4*g4 + r
  uint32_t sz[4];                 // V scale (low half) and zero (high half) of token 4*g4 + r
};

// centroid table: entry e holds two codes (low code first) as {hi pair, lo
// pair}, so one 8-byte LDS read fetches both parts (random reads of a small
// table cost the same per instruction for 4 and 8 bytes per lane)
template <int KB>
__device__ __forceinline__ void build_tables(const MfmaArgs& a, u32x2* s_tab) {
  constexpr int kTab = KB == 4 ? 256 : 64;
  for (int e = threadIdx.x; e < kTab; e += blockDim.x) {
    const int c0 = e & ((1 << KB) - 1), c1 = e >> KB;
    const float v0 = a.tables->centroids[c0], v1 = a.tables->centroids[c1];
    const _Float16 h0 = static_cast<_Float16>(v0), h1 = static_cast<_Float16>(v1);
    const _Float16 l0 = static_cast<_Float16>((v0 - static_cast<float>(h0)) * kLoScale);
    const _Float16 l1 = static_cast<_Float16>((v1 - static_cast<float>(h1)) * kLoScale);
    s_tab[e] = u32x2{pack_h2(h0, h1), pack_h2(l0, l1)};
  }
}

// rotate the G queries of kv head g (q_rot = H diag(s) q / sqrt(128)) and
// split them into f16 hi / lo; lane (h = r16, g4) holds coordinates
// [32*g4, 32*g4 + 32) of head h, as the four score-MFMA B operands.  With
// the Haar rotation the queries come rotated already (a.q_rot, from
// rotate_queries_haar_kernel; that rotation has no 1/sqrt(d) factor).
__device__ __forceinline__ void load_queries(const MfmaArgs& a, int b, int g, int r16, int g4,
                                             float fscale, h8 (&qhi)[4], h8 (&qlo)[4]) {
  float x[32];
  const bool live = r16 < a.G;
  const int64_t row = (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0 + (live ? r16 : 0)) * kD + 32 * g4;
  if (a.q_rot != nullptr) {
    const float4* rp = reinterpret_cast<const float4*>(a.q_rot + row);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = rp[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = live ? x[8 * kk + e] * fscale : 0.0f;
        const _Float16 hv = static_cast<_Float16>(v);
        qhi[kk][e] = hv;
        qlo[kk][e] = static_cast<_Float16>(v - static_cast<float>(hv));
      }
    return;
  }
  const uint16_t* qp = a.q + row;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qp + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  const uint32_t sb = a.tables->sign_bits[g4];
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = __uint_as_float(__float_as_uint(x[j]) ^ (((sb >> j) & 1u) << 31));
#pragma unroll
  for (int hs = 1; hs < 32; hs *= 2)
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if ((j & hs) == 0) {
        const float p = x[j], r = x[j + hs];
        x[j] = p + r;
        x[j + hs] = p - r;
      }
  // strides 32 and 64 cross lane groups: partner lane l ^ 16, l ^ 32
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
    const float o = (g4 & 1) ? __uint_as_float(sw[0]) : __uint_as_float(sw[1]);
    x[j] = (g4 & 1) ? (o - x[j]) : (x[j] + o);
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
    const float o = (g4 & 2) ? __uint_as_float(sw[0]) : __uint_as_float(sw[1]);
    x[j] = (g4 & 2) ? (o - x[j]) : (x[j] + o);
  }
  // 1/sqrt(128) of the rotation times the softmax scale (base 2): scores come
  // out of the MFMAs ready for exp2
  const float qs = 0.08838834764831845f * fscale;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = live ? x[8 * kk + e] * qs : 0.0f;
      const _Float16 hv = static_cast<_Float16>(v);
      qhi[kk][e] = hv;
      qlo[kk][e] = static_cast<_Float16>(v - static_cast<float>(hv));
    }
}

// (x & m) | c for c with no bits under m, as one v_bfi_b32 (the compiler
// splits it into two instructions when both constants are literals; the mask
// is kept in a register instead)
__device__ __forceinline__ uint32_t insert_bits(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(x), "s"(c));
  return r;
}

// the G queries of kv head g as bf16 B operands of the FP8-key score MFMA
// (keys are stored unrotated, so q is used as given); lane (h = r16, g4)
// holds coordinates [32*g4, 32*g4 + 32) of head h, zero for h >= G
__device__ __forceinline__ void load_queries_bf16(const MfmaArgs& a, int b, int g, int r16, int g4,
                                                  bf8v (&qb)[4]) {
  const bool live = r16 < a.G;
  const uint16_t* qp = a.q + (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0 + (live ? r16 : 0)) * kD + 32 * g4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4 w = *reinterpret_cast<const u32x4*>(qp + 8 * kk);
    if (!live) w = u32x4{0u, 0u, 0u, 0u};
    qb[kk] = __builtin_bit_cast(bf8v, w);
  }
}

// Scores (base 2) of a slab's 4 rows held by this lane (tokens 4*g4 + r,
// head r16) for 3/4-bit keys: centroid MFMAs plus the norm correction.
// Rows at or past valid_rows get -inf.
template <int KB>
__device__ __forceinline__ void score_slab(const SlabOps<KB>& op, int valid_rows,
                                           const u32x2* s_tab, const h8 (&qhi)[4],
                                           const h8 (&qlo)[4], int g4, float (&s)[4]) {
  // ---- K: codes -> centroid hi / lo operands, score and norm MFMAs ----
  // (the norm accumulator starts at the 1e-16 of the correction's denominator)
  f4 Shi = {0.f, 0.f, 0.f, 0.f}, Slo = {0.f, 0.f, 0.f, 0.f};
  f4 Nhi = {1e-16f, 1e-16f, 1e-16f, 1e-16f}, Nx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint32_t idx[4];
    if constexpr (KB == 4) {
#pragma unroll
      for (int p = 0; p < 4; ++p) idx[p] = (op.kw[kk] >> (8 * p)) & 0xFFu;
    } else {
      // 24 bits per MFMA step: bits [24*kk, 24*kk + 24) of the lane's 96
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int bit = 24 * kk + 6 * p;
        const int w = bit >> 5, o = bit & 31;
        uint32_t v = op.kw[w] >> o;
        if (o > 26) v |= op.kw[w + 1] << (32 - o);
        idx[p] = v & 63u;
      }
    }
    u32x4 hi, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x2 e = s_tab[idx[p]];
      hi[p] = e[0];
      lo[p] = e[1];
    }
    const h8 chi = __builtin_bit_cast(h8, hi);
    const h8 clo = __builtin_bit_cast(h8, lo);
    Shi = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, qhi[kk], Shi, 0, 0, 0);
    Shi = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, qlo[kk], Shi, 0, 0, 0);
    Slo = __builtin_amdgcn_mfma_f32_16x16x32_f16(clo, qhi[kk], Slo, 0, 0, 0);
    Nhi = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, chi, Nhi, 0, 0, 0);
    Nx = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, clo, Nx, 0, 0, 0);
  }
  const int diag_src = 20 * g4;            // lane 16*g4 + 4*g4 (+ r) holds N[4*g4+r][4*g4+r]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float nd = Nhi[r] + (2.0f / kLoScale) * Nx[r];
    const float nn = lane_value(nd, diag_src + r);
    const float fac = f16_bits_to_f32(op.n[r]) * __builtin_amdgcn_rsqf(nn);
    const float dot = Shi[r] + Slo[r] * (1.0f / kLoScale);
    s[r] = 4 * g4 + r < valid_rows ? dot * fac : -INFINITY;
  }
}

// Operand bytes of one slab for one lane, FP8 keys (slots of 196 bytes,
// 4-byte aligned, no norm).
struct SlabOps8 {
  u32x4 k[2];                     // K bytes of token r16, coordinates [32*g4, 32*g4 + 32)
  uint32_t X[4];                  // V codes of token 4*g4 + r, coordinates [8*r16, 8*r16 + 8)
  uint32_t sz[4];                 // V scale (low half) and zero (high half) of token 4*g4 + r
};

// Scores (base 2) for FP8 keys: E4M3 bytes convert exactly to bf16 (two per
// instruction) and meet the bf16 query in one MFMA per 32 coordinates;
// products are exact and accumulate in fp32.
__device__ __forceinline__ void score_slab8(const SlabOps8& op, int valid_rows, const bf8v (&qb)[4],
                                            float scale_log2, int g4, float (&s)[4]) {
  f4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t w0 = op.k[kk >> 1][2 * (kk & 1)], w1 = op.k[kk >> 1][2 * (kk & 1) + 1];
    const bf2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    const bf8v a = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
    S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[kk], S, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = 4 * g4 + r < valid_rows ? S[r] * scale_log2 : -INFINITY;
}

// V bits of the slot sizes the matrix-core kernels take at d = 128: 102-byte
// slots (3-bit K, 3-bit V), else 4-bit V
constexpr int vbits_of_slot(int slot) { return slot == 102 ? 3 : 4; }

// MFMA B operands of the V codes of tokens 4*g4 + r (X[r]: the token's codes
// of coordinates 8*r16 .. 8*r16 + 7) for coordinates 8*r16 + 2*kb (Blo) and
// 8*r16 + 2*kb + 1 (Bhi), as exact f16 integers: code c goes into the
// mantissa of a power of two (1024 + c, or 64 + c for the high nibble of a
// 4-bit byte), and one packed f16 subtraction removes the power of two.
// (Codes left as f16 subnormals, c * 2^-24, need no subtraction, but the
// matrix cores do not sum products with subnormal inputs exactly: decode
// errors grew about 100-fold.)
template <int VB, bool BFI = true>
__device__ __forceinline__ void v_operands(const uint32_t (&X)[4], int kb, h4& Blo, h4& Bhi) {
  const h2 b1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  if constexpr (VB == 4) {
    const h2 b64 = {static_cast<_Float16>(64.0f), static_cast<_Float16>(64.0f)};
    // byte kb of each token's dword -> [x0, 0, x1, 0]
    const uint32_t sel = kb | (0x0Cu << 8) | ((4u + kb) << 16) | (0x0Cu << 24);
    const uint32_t p01 = __builtin_amdgcn_perm(X[1], X[0], sel);
    const uint32_t p23 = __builtin_amdgcn_perm(X[3], X[2], sel);
    // nibbles into the mantissas: one bit-field insert each (its two masks
    // take two registers; BFI = false spells it as and + or where that
    // pressure would spill)
    auto ins = [](uint32_t x, uint32_t m, uint32_t c) { return BFI ? insert_bits(x, m, c) : (x & m) | c; };
    const h2 lo01 = __builtin_bit_cast(h2, ins(p01, 0x000F000Fu, 0x64006400u)) - b1024;
    const h2 lo23 = __builtin_bit_cast(h2, ins(p23, 0x000F000Fu, 0x64006400u)) - b1024;
    const h2 hi01 = __builtin_bit_cast(h2, ins(p01, 0x00F000F0u, 0x54005400u)) - b64;
    const h2 hi23 = __builtin_bit_cast(h2, ins(p23, 0x00F000F0u, 0x54005400u)) - b64;
    Blo = h4{lo01[0], lo01[1], lo23[0], lo23[1]};
    Bhi = h4{hi01[0], hi01[1], hi23[0], hi23[1]};
  } else {
    // 3-bit codes: code m of a token at bits [3m, 3m + 3) of its X
    const uint32_t m0 = 6 * kb, m1 = 6 * kb + 3;
    const h2 lo01 = __builtin_bit_cast(h2, __builtin_amdgcn_ubfe(X[0], m0, 3) |
                                               (__builtin_amdgcn_ubfe(X[1], m0, 3) << 16) | 0x64006400u) - b1024;
    const h2 lo23 = __builtin_bit_cast(h2, __builtin_amdgcn_ubfe(X[2], m0, 3) |
                                               (__builtin_amdgcn_ubfe(X[3], m0, 3) << 16) | 0x64006400u) - b1024;
    const h2 hi01 = __builtin_bit_cast(h2, __builtin_amdgcn_ubfe(X[0], m1, 3) |
                                               (__builtin_amdgcn_ubfe(X[1], m1, 3) << 16) | 0x64006400u) - b1024;
    const h2 hi23 = __builtin_bit_cast(h2, __builtin_amdgcn_ubfe(X[2], m1, 3) |
                                               (__builtin_amdgcn_ubfe(X[3], m1, 3) << 16) | 0x64006400u) - b1024;
    Blo = h4{lo01[0], lo01[1], lo23[0], lo23[1]};
    Bhi = h4{hi01[0], hi01[1], hi23[0], hi23[1]};
  }
}

// Online softmax and P.V of one slab from its scores (base 2, -inf for masked
// rows).  Rows of query heads >= G have q = 0: their scores, weights and O
// rows are finite and never stored.
template <int VB>
__device__ __forceinline__ void softmax_pv(const float (&s)[4], int valid_rows, const uint32_t (&sz)[4],
                                           const uint32_t (&X)[4], int g4, RunState& st) {
  float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  float sc[4], zr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // rows past the end may hold stale bytes: scale and zero read as 0
    const uint32_t szm = 4 * g4 + r < valid_rows ? sz[r] : 0u;
    sc[r] = f16_bits_to_f32(szm & 0xFFFFu);
    zr[r] = f16_bits_to_f32(szm >> 16);
  }
  // Lazy running maximum: the accumulators are rescaled only when some
  // lane's rows exceed the head's running max by more than kLazy (base 2),
  // so p <= 2^kLazy; where p * scale could overflow f16 (scale > 1000) the
  // lane allows no growth (p <= 1).  A rescale moves the whole head to its
  // exact maximum, so every lane of a head always shares one running max.
  const float sc_max = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  const float thr = sc_max > 1000.0f ? 0.0f : kLazy;
  if (__any(pm > st.m_run + thr)) {
    const float m_new = fmaxf(st.m_run, max_x32(max_x16(pm)));
    const float corr = __builtin_amdgcn_exp2f(st.m_run - m_new);   // 0 on the first slab
    st.l_part *= corr;
    st.z_part *= corr;
    // O rows are heads 4*g4 + r; their factors sit in lanes r16 = head
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float cr = lane_value(corr, 4 * g4 + r);
#pragma unroll
      for (int m = 0; m < 8; ++m) st.O[m][r] *= cr;
    }
    st.m_run = m_new;
  }
  // p * scale as f16 hi + lo: one f16 alone (2^-11) is not precise enough
  // when a single token dominates and its V range is wide
  h4 W, Wl;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = __builtin_amdgcn_exp2f(s[r] - st.m_run);      // 0 for masked rows
    st.l_part += p;
    st.z_part += p * zr[r];
    const float wf = p * sc[r];
    W[r] = static_cast<_Float16>(wf);
    Wl[r] = static_cast<_Float16>(wf - static_cast<float>(W[r]));
  }

  // ---- V: codes of tokens 4*g4 + r at coordinates 8*r16 + m ----
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    h4 Blo4, Bhi4;
    v_operands<VB>(X, kb, Blo4, Bhi4);
    // one K = 32 product per tile: W and Wl of tokens 4*g4 + r meet the
    // same codes, listed twice
    const h8 Blo = {Blo4[0], Blo4[1], Blo4[2], Blo4[3], Blo4[0], Blo4[1], Blo4[2], Blo4[3]};
    const h8 Bhi = {Bhi4[0], Bhi4[1], Bhi4[2], Bhi4[3], Bhi4[0], Bhi4[1], Bhi4[2], Bhi4[3]};
    const h8 Ws = {W[0], W[1], W[2], W[3], Wl[0], Wl[1], Wl[2], Wl[3]};
    st.O[2 * kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ws, Blo, st.O[2 * kb], 0, 0, 0);
    st.O[2 * kb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ws, Bhi, st.O[2 * kb + 1], 0, 0, 0);
  }
}

// The same online softmax and P.V split in three steps, so a caller can keep
// the rare rescale of the accumulators out of its main loop (a conditional
// update of the accumulators inside the loop costs register copies of all of
// them on every slab).
struct SlabSoftmax {
  float sc[4], zr[4];
  float pm;
  bool grow;        // the wavefront must rescale before this slab's P.V
};

template <bool FULL>
__device__ __forceinline__ SlabSoftmax softmax_check(const float (&s)[4], int valid_rows,
                                                     const uint32_t (&sz)[4], int g4, const RunState& st) {
  SlabSoftmax r;
  r.pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t szm = (FULL || 4 * g4 + i < valid_rows) ? sz[i] : 0u;
    r.sc[i] = f16_bits_to_f32(szm & 0xFFFFu);
    r.zr[i] = f16_bits_to_f32(szm >> 16);
  }
  const float sc_max = fmaxf(fmaxf(r.sc[0], r.sc[1]), fmaxf(r.sc[2], r.sc[3]));
  const float thr = sc_max > 1000.0f ? 0.0f : kLazy;
  r.grow = __any(r.pm > st.m_run + thr);
  return r;
}

__device__ __forceinline__ void softmax_rescale(const SlabSoftmax& sm, bool diag, RunState& st) {
  const float m_new = fmaxf(st.m_run, max_x32(max_x16(sm.pm)));
  const float corr = __builtin_amdgcn_exp2f(st.m_run - m_new);   // 0 on the first slab
  st.l_part *= corr;
  st.z_part *= corr;
  const f4 cr = rows_to_tile(corr, diag);       // O rows are heads 4*g4 + r
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < 8; ++m) st.O[m][r] *= cr[r];
  st.m_run = m_new;
}

// p * scale as f16 hi + lo: one f16 alone (2^-11) is not precise enough when
// a single token dominates and its V range is wide.  The two parts sit in
// different rows of the P.V tile: rows h < 8 take the hi part of head h,
// rows h + 8 its lo part (those lanes hold a copy of head h's scores and
// running state), so each MFMA has k = 16 tokens and V operands that are
// exactly the decoded codes; fold_lo_rows adds the lo rows in at the end.
template <int VB, bool BFI = true>
__device__ __forceinline__ void softmax_accumulate(const float (&s)[4], const SlabSoftmax& sm,
                                                   const uint32_t (&X)[4], RunState& st) {
  const bool lo_row = (threadIdx.x & 8) != 0;
  h4 W;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = __builtin_amdgcn_exp2f(s[r] - st.m_run);
    st.l_part += p;
    st.z_part += p * sm.zr[r];
    const float wf = p * sm.sc[r];
    const float hi = static_cast<float>(static_cast<_Float16>(wf));
    W[r] = static_cast<_Float16>(lo_row ? wf - hi : wf);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    h4 Blo, Bhi;
    v_operands<VB, BFI>(X, kb, Blo, Bhi);
    st.O[2 * kb] = __builtin_amdgcn_mfma_f32_16x16x16f16(W, Blo, st.O[2 * kb], 0, 0, 0);
    st.O[2 * kb + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(W, Bhi, st.O[2 * kb + 1], 0, 0, 0);
  }
}

// rows h + 8 of the accumulators (lane groups 2, 3) into rows h (groups 0, 1)
__device__ __forceinline__ void fold_lo_rows(RunState& st) {
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) st.O[m][r] = sum_x32(st.O[m][r]);
}

// One slab of 3/4-bit keys: scores, norm correction, online softmax, P.V.
template <int KB, int VB>
__device__ __forceinline__ void process_slab(const SlabOps<KB>& op, int valid_rows,
                                             const u32x2* s_tab, const h8 (&qhi)[4],
                                             const h8 (&qlo)[4], int g4, RunState& st) {
  float s[4];
  score_slab<KB>(op, valid_rows, s_tab, qhi, qlo, g4, s);
  softmax_pv<VB>(s, valid_rows, op.sz, op.X, g4, st);
}

// page ids of this split -> byte offsets in LDS (-1: outside the cache)
__device__ __forceinline__ void stage_page_offsets(const MfmaArgs& a, int b, int t0, int t1,
                                                   int64_t page_bytes, int64_t* s_page_off) {
  const int p_first = t0 >> a.bs_shift;
  const int n_pages = t1 > t0 ? ((t1 - 1) >> a.bs_shift) - p_first + 1 : 0;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  for (int i = threadIdx.x; i < n_pages; i += blockDim.x) {
    const int page = bt[p_first + i];
    if (page < 0 || page >= a.num_blocks) {
      a.errs->page = 1;
      s_page_off[i] = -1;
    } else {
      s_page_off[i] = static_cast<int64_t>(page) * page_bytes;
    }
  }
}

// slab starting at token t -> uniform base pointer, nullptr for a bad page
__device__ __forceinline__ const uint8_t* slab_ptr(const MfmaArgs& a, const int64_t* s_page_off,
                                                   int p_first, int t, int64_t row_bytes) {
  const int64_t po = s_page_off[(t >> a.bs_shift) - p_first];
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(po));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(po) >> 32));
  if (hi == 0xFFFFFFFFu) return nullptr;
  const int64_t u = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  return a.cache + u + static_cast<int64_t>(t & ((1 << a.bs_shift) - 1)) * row_bytes;
}

// Buffer resource of the 16 rows of the slab starting at token t.  A slab
// past the split end or on a bad page gets an empty range (every load of it
// returns zeros without touching memory) and ok = false, so the prefetch is
// issued unconditionally: with a fixed number of loads per slab the compiler
// waits only for the oldest slab in flight instead of draining every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const MfmaArgs& a, const int64_t* s_page_off,
                                                          int p_first, int t, int t1,
                                                          int64_t row_bytes, bool& ok) {
  const uint8_t* p = t < t1 ? slab_ptr(a, s_page_off, p_first, t, row_bytes) : nullptr;
  ok = p != nullptr;
  const int bytes = ok ? static_cast<int>(16 * row_bytes) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ok ? p : a.cache), 0, bytes,
                                           kBufferWord3);
}

// Tokens of sequence b the kernels attend to: seq_lens[b] clamped to what the
// block table and the splits can address; a cache without pages holds none
// (its page ids are all out of range, which the page staging reports).
__device__ __forceinline__ int effective_len(const MfmaArgs& a, int b) {
  int T = a.seq_lens[b];
  const int t_cap = min(a.num_splits * a.chunk, a.max_blocks << a.bs_shift);
  T = T < 0 ? 0 : (T > t_cap ? t_cap : T);
  return a.num_blocks > 0 ? T : 0;
}

__device__ __forceinline__ int clamp_len(const MfmaArgs& a, int b, int split, int g) {
  const int T = a.seq_lens[b];
  const int t_cap = min(a.num_splits * a.chunk, a.max_blocks << a.bs_shift);
  if (threadIdx.x == 0 && split == 0 && g == 0) {
    if (T < 0 || T > t_cap) a.errs->len = 1;
    if (T > 0 && a.num_blocks <= 0) a.errs->page = 1;
  }
  return effective_len(a, b);
}

// write this wavefront's split partials: O rows are heads 4*g4 + r
__device__ __forceinline__ void store_partials(const MfmaArgs& a, int b, int g, int split, int g4,
                                               int r16, const RunState& st) {
  const float l_part = sum_x32(sum_x16(st.l_part));
  const float z_part = sum_x32(sum_x16(st.z_part));
  const int G = a.G;
  const int64_t rec0 = (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0) * a.num_splits + split;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g4 + r;
    if (h < G) {
      float* rec = a.part + (rec0 + static_cast<int64_t>(h) * a.num_splits) * kRec;
      // tile m column r16 is coordinate 8*r16 + m
      *reinterpret_cast<float4*>(rec + 8 * r16) = make_float4(
          st.O[0][r], st.O[1][r], st.O[2][r], st.O[3][r]);
      *reinterpret_cast<float4*>(rec + 8 * r16 + 4) = make_float4(
          st.O[4][r], st.O[5][r], st.O[6][r], st.O[7][r]);
    }
  }
  if (g4 == 0 && r16 < G) {
    float* rec = a.part + (rec0 + static_cast<int64_t>(r16) * a.num_splits) * kRec;
    rec[kD] = st.m_run;
    rec[kD + 1] = l_part;
    rec[kD + 2] = z_part;
  }
}

// Merge the splits of one (sequence, query head): four wavefronts take every
// fourth split, lane = coordinates 2*lane and 2*lane + 1.  Each wavefront
// merges its splits online (running max, a split weighted by 2^(m_s - max)),
// with all loads of a group of splits issued together, and the four meet in
// LDS.  o = sum_s w_s (O_s + z_s) / sum_s w_s l_s.
// Haar rotation of the queries, once per decode: q_rot = Q q for every
// (sequence, query head), fp32, with Q the d x d matrix the store applied to
// the keys (readings of the pages: the Haar rotation).  One workgroup per
// (sequence, kv head): thread i forms coordinate i of its G queries, so
// each row of Q is read once per workgroup.
__global__ void __launch_bounds__(kD) rotate_queries_haar_kernel(MfmaArgs a, float* q_rot) {
  __shared__ float s_q[16][kD];
  const int b = blockIdx.x / a.H, g = blockIdx.x - b * a.H;
  const int i = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0) * kD;
  for (int h = 0; h < a.G; ++h)
    s_q[h][i] = __uint_as_float(static_cast<uint32_t>(a.q[base + h * kD + i]) << 16);
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) acc[h] = 0.0f;
  const float* rowq = a.tables->rot + static_cast<int64_t>(i) * kD;
  for (int j = 0; j < kD; ++j) {
    const float qij = rowq[j];
#pragma unroll
    for (int h = 0; h < 16; ++h)
      if (h < a.G) acc[h] = __builtin_fmaf(qij, s_q[h][j], acc[h]);
  }
#pragma unroll
  for (int h = 0; h < 16; ++h)
    if (h < a.G) q_rot[base + h * kD + i] = acc[h];
}

// The sequences ranked by length, longest first (ties by index):
// order[rank] = b.  One thread per sequence; it counts the longer ones.
__global__ void __launch_bounds__(256) order_sequences_kernel(MfmaArgs a, int32_t* order) {
  __shared__ int s_len[256];
  const int b = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
  const int T = b < a.batch ? effective_len(a, b) : 0;
  int rank = 0;
  for (int c0 = 0; c0 < a.batch; c0 += 256) {
    __syncthreads();
    const int c = c0 + static_cast<int>(threadIdx.x);
    s_len[threadIdx.x] = c < a.batch ? effective_len(a, c) : -1;
    __syncthreads();
    const int n = min(256, a.batch - c0);
    for (int i = 0; i < n; ++i) {
      const int U = s_len[i];
      rank += (U > T || (U == T && c0 + i < b)) ? 1 : 0;
    }
  }
  if (b < a.batch) order[rank] = b;
}

__global__ void __launch_bounds__(256) decode_merge_kernel(MfmaArgs a) {
  __shared__ float s_m[4], s_l[4];
  __shared__ float2 s_acc[4][64];
  const int bh = blockIdx.x;                 // b * Hq + hq
  const int b = bh / a.Hq;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = effective_len(a, b);
  const int nsp = (T + a.chunk - 1) / a.chunk;
  const float* recs = a.part + static_cast<int64_t>(bh) * a.num_splits * kRec;
  float M = -INFINITY, L = 0.0f;
  float2 acc = make_float2(0.0f, 0.0f);
  constexpr int kU = 4;                      // splits per wavefront whose loads are in flight together
  for (int s0 = wv; s0 < nsp; s0 += 4 * kU) {
    float4 mlz[kU];
    float2 o[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int sp = s0 + 4 * u;
      const float* rec = recs + static_cast<int64_t>(sp < nsp ? sp : s0) * kRec;
      mlz[u] = *reinterpret_cast<const float4*>(rec + kD);      // m, l, z, pad
      o[u] = *reinterpret_cast<const float2*>(rec + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s0 + 4 * u >= nsp) break;
      const float m_new = fmaxf(M, mlz[u].x);
      if (m_new == -INFINITY) continue;                         // nothing attended yet (bad pages)
      const float c = __builtin_amdgcn_exp2f(M - m_new);        // 0 on the first split
      const float w = __builtin_amdgcn_exp2f(mlz[u].x - m_new);
      acc.x = acc.x * c + w * (o[u].x + mlz[u].z);
      acc.y = acc.y * c + w * (o[u].y + mlz[u].z);
      L = L * c + w * mlz[u].y;
      M = m_new;
    }
  }
  if (lane == 0) {
    s_m[wv] = M;
    s_l[wv] = L;
  }
  s_acc[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
  const float Mx = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float2 tot = make_float2(0.0f, 0.0f);
  float Lt = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w = s_m[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s_m[i] - Mx);
    tot.x += w * s_acc[i][lane].x;
    tot.y += w * s_acc[i][lane].y;
    Lt += w * s_l[i];
  }
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  const float r0 = tot.x * inv, r1 = tot.y * inv;
  const int64_t oi = static_cast<int64_t>(bh) * kD + 2 * lane;
  if (a.out_fp32) {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + oi) = make_float2(r0, r1);
  } else {
    uint32_t u0 = __float_as_uint(r0), u1 = __float_as_uint(r1);
    u0 = (u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16;     // round to nearest even
    u1 = (u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16;
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi) = u0 | (u1 << 16);
  }
}

// ============================================================================
// direct: each lane loads exactly its operand bytes with buffer loads (rows
// of 134/118-byte slots are only 2-byte aligned; the loads are unaligned,
// which the memory path handles), two slabs ahead, one wavefront per
// (split, sequence, kv head)
// ============================================================================

template <int KB>
struct DirectRegs {
  uint32_t k[KB == 8 ? 8 : (KB == 4 ? 4 : 3)];   // K bytes of token r16 (32 coordinates)
  uint32_t X[4];                                  // V codes of token 4*g4 + r, coords [8*r16, 8*r16 + 8)
  uint32_t n[4];                                  // K norm (f16) of token 4*g4 + r (MSE keys)
  uint32_t sz[4];                                 // V scale | zero of token 4*g4 + r
  bool ok;
};

// byte offsets, from the slab's first row, of the lane's operands
struct DirectOffsets {
  uint32_t k;
  uint32_t row[4];       // slot start of token 4*g4 + r
  uint32_t x[4];         // its V codes for coordinates [8*r16, 8*r16 + 8)
};

template <int KB, int SLOT>
__device__ __forceinline__ DirectOffsets direct_offsets(int r16, int g4, uint32_t head_off, uint32_t rb) {
  constexpr int kKP = KB == 8 ? kD : (kD * KB) / 8 + 2;
  constexpr int kLaneKB = KB == 8 ? 32 : (KB == 4 ? 16 : 12);
  DirectOffsets o;
  o.k = r16 * rb + head_off + kLaneKB * g4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o.row[r] = (4 * g4 + r) * rb + head_off;
    o.x[r] = o.row[r] + kKP + (vbits_of_slot(SLOT) == 3 ? 3 : 4) * r16;
  }
  return o;
}

template <int KB, int SLOT>
__device__ __forceinline__ void direct_load2(__amdgpu_buffer_rsrc_t rs, const DirectOffsets& o,
                                             DirectRegs<KB>& d) {
  constexpr int kKCB = KB == 8 ? kD : (kD * KB) / 8;
  constexpr int kKP = KB == 8 ? kD : kKCB + 2;
  if constexpr (KB == 4) {
    const u32x4 t = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.k, 0, 0));
    d.k[0] = t[0]; d.k[1] = t[1]; d.k[2] = t[2]; d.k[3] = t[3];
  } else if constexpr (KB == 3) {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 t = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, o.k, 0, 0));
    d.k[0] = t[0]; d.k[1] = t[1]; d.k[2] = t[2];
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 t = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.k + 16 * i, 0, 0));
      d.k[4 * i] = t[0]; d.k[4 * i + 1] = t[1]; d.k[4 * i + 2] = t[2]; d.k[4 * i + 3] = t[3];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    d.X[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, o.x[r], 0, 0);
    if constexpr (KB != 8) d.n[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, o.row[r] + kKCB, 0, 0);
    d.sz[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, o.row[r] + kKP + kD * vbits_of_slot(SLOT) / 8, 0, 0);
  }
}

// Resident wavefronts per SIMD the kernel is built for (its register budget
// is 512 / waves), and whether a slab's registers are copied so the next
// loads go out before the slab is processed (two slabs ahead) or the loads
// follow the processing (one slab ahead, fewer registers).  Chosen by
// measurement on the llama3-, k3v4- and k8v4-shaped decodes.
template <int KB>
constexpr int kSlabWavesPerSimd = KB == 8 ? 4 : 2;
template <int KB>
constexpr bool kLoadEarly = KB == 3;

template <int KB, int SLOT>
__global__ void __launch_bounds__(64, kSlabWavesPerSimd<KB>) decode_slab_kernel(MfmaArgs a) {
  __shared__ u32x2 s_tab[256];
  __shared__ int64_t s_page_off[kMaxChunkPages];

  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  // XCD-aware order: workgroups go to the 8 XCDs round robin, so block id
  // x serves item (x % 8) * per_xcd + x / 8 of the (split, sequence, kv head)
  // items, kv head fastest.  The heads of one page row share cache lines (a
  // slot is not a multiple of the line), and this puts them on one XCD, in
  // consecutive slots, so the shared lines come from its L2 rather than
  // twice from HBM.
  const int n_items = a.num_splits * a.batch * a.H;
  const int per_xcd = (n_items + 7) / 8;
  const int item = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
  if (item >= n_items) return;
  const int g = item % a.H;                  // kv head
  const int split = (item / a.H) % a.num_splits;
  const int b = item / (a.H * a.num_splits);
  const int H = a.H;
  const int64_t row_bytes = static_cast<int64_t>(H) * SLOT;
  const int64_t page_bytes = static_cast<int64_t>(1 << a.bs_shift) * row_bytes;

  if constexpr (KB != 8) build_tables<KB>(a, s_tab);
  const int T = clamp_len(a, b, split, g);
  const int t0 = split * a.chunk;
  const int t1 = min(T, t0 + a.chunk);
  stage_page_offsets(a, b, t0, t1, page_bytes, s_page_off);
  __syncthreads();
  if (t0 >= t1) return;

  h8 qhi[4], qlo[4];
  bf8v qb[4];
  if constexpr (KB == 8)
    load_queries_bf16(a, b, g, r16, g4, qb);
  else
    load_queries(a, b, g, r16, g4, a.scale_log2, qhi, qlo);
  RunState st;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.O[m] = f4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.0f;
  st.z_part = 0.0f;
  const int p_first = t0 >> a.bs_shift;
  const DirectOffsets off = direct_offsets<KB, SLOT>(r16, g4, static_cast<uint32_t>(g * SLOT),
                                                     static_cast<uint32_t>(row_bytes));

  // slabs in flight in two register sets; every step issues the same loads
  // (an empty buffer range past the split end or on a bad page), so a wait
  // covers one slab
  DirectRegs<KB> r0, r1;
  auto load = [&](int t, DirectRegs<KB>& r) {
    bool ok;
    const __amdgpu_buffer_rsrc_t rs = slab_rsrc(a, s_page_off, p_first, t, t1, row_bytes, ok);
    r.ok = ok;
    direct_load2<KB, SLOT>(rs, off, r);
  };
  auto step = [&](int t, DirectRegs<KB>& r) {
    DirectRegs<KB> cur_copy;
    if constexpr (kLoadEarly<KB>) {
      cur_copy = r;
      load(t + 32, r);
    }
    const DirectRegs<KB>& cur = kLoadEarly<KB> ? cur_copy : r;
    if (cur.ok) {
      float sc[4];
      if constexpr (KB == 8) {
        SlabOps8 op;
        op.k[0] = u32x4{cur.k[0], cur.k[1], cur.k[2], cur.k[3]};
        op.k[1] = u32x4{cur.k[4], cur.k[5], cur.k[6], cur.k[7]};
        score_slab8(op, t1 - t, qb, a.scale_log2, g4, sc);
      } else {
        SlabOps<KB> op;
#pragma unroll
        for (int i = 0; i < (KB == 4 ? 4 : 3); ++i) op.kw[i] = cur.k[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) op.n[i] = cur.n[i];
        score_slab<KB>(op, t1 - t, s_tab, qhi, qlo, g4, sc);
      }
      softmax_pv<vbits_of_slot(SLOT)>(sc, t1 - t, cur.sz, cur.X, g4, st);
    }
    if constexpr (!kLoadEarly<KB>) load(t + 32, r);
  };
  load(t0, r0);
  load(t0 + 16, r1);
  // whole rounds of two steps, no early exit: a step past the split end only
  // issues empty loads, which keeps the load count per step fixed
  for (int t = t0; t < t1; t += 32) {
    step(t, r0);
    step(t + 16, r1);
  }
  store_partials(a, b, g, split, g4, r16, st);
}


// ============================================================================
// staged: one wavefront per (split, sequence, kv head) loads its head's span
// of the 16 rows of a slab with 16-byte buffer loads (whole, aligned chunks,
// three per lane) two slabs ahead in registers, parks the slab in a private
// LDS buffer and takes its operands from there.  3/4-bit keys with an even
// number of kv heads (every row then starts 4-byte aligned).
// ============================================================================

// A wavefront's bytes of one row: from its slot start rounded down to 4 to
// its slot end rounded up to 4 (136 bytes for 134-byte slots, 120 for 118),
// fetched as 16-byte chunks plus one 8- or 4-byte tail, never past the slot
// end rounded up to 4 (the last head's slot ends the row, the last row the
// page).
template <int SLOT>
struct StageShape {
  static constexpr int kSpan = SLOT % 4 == 0 ? SLOT : SLOT + 2;   // bytes fetched per row
  static constexpr int kTail = kSpan % 16;             // 4 or 8
  static_assert(kTail == 4 || kTail == 8, "row span must be 16-byte chunks plus 4 or 8");
  static constexpr int kC16 = (kSpan - kTail) / 16;    // 16-byte chunks per row
  static constexpr int kRow = 16 * (kC16 + 1);         // LDS bytes per row (16-aligned)
  static constexpr int kStage = 16 * kRow;             // LDS bytes per slab
  static constexpr int kChunks = 16 * kC16;            // 16-byte chunks per slab
  static constexpr int kLoads16 = (kChunks + 63) / 64; // 16-byte loads per lane
};

template <int SLOT>
struct StageRegs {
  u32x4 d[StageShape<SLOT>::kLoads16];
  u32x2 tail;                                          // lanes 0..15: the row's last 4 or 8 bytes
  bool ok;                                             // a real slab (else an empty load)
};

// Per-lane byte offsets (from a slab's first row) of the lane's 16-byte
// chunks and its tail; lanes without a chunk of their own re-read the last
// one and lanes 16..63 re-read a tail, so every lane issues the same loads.
template <int SLOT>
struct StageOffsets {
  uint32_t d[StageShape<SLOT>::kLoads16];
  uint32_t tail;
};

template <int SLOT>
__device__ __forceinline__ StageOffsets<SLOT> stage_offsets(int lane, uint32_t head_off4, uint32_t rb) {
  using S = StageShape<SLOT>;
  StageOffsets<SLOT> o;
#pragma unroll
  for (int j = 0; j < S::kLoads16; ++j) {
    int c = lane + 64 * j;
    if (c >= S::kChunks) c = S::kChunks - 1;
    const int row = c / S::kC16, cc = c - row * S::kC16;
    o.d[j] = row * rb + head_off4 + 16u * cc;
  }
  o.tail = (lane & 15) * rb + head_off4 + 16u * S::kC16;
  return o;
}

// cache policy of the slab loads: default (non-temporal loads measured no
// faster here, unlike the page kernel's loads into LDS)
constexpr int kStageLoadAux = 0;

template <int SLOT>
__device__ __forceinline__ void stage_load(__amdgpu_buffer_rsrc_t rs, const StageOffsets<SLOT>& o,
                                           StageRegs<SLOT>& sr) {
  using S = StageShape<SLOT>;
#pragma unroll
  for (int j = 0; j < S::kLoads16; ++j)
    sr.d[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.d[j], 0, kStageLoadAux));
  if constexpr (S::kTail == 8)
    sr.tail = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, o.tail, 0, kStageLoadAux));
  else
    sr.tail[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, o.tail, 0, kStageLoadAux);
}

template <int SLOT>
__device__ __forceinline__ void stage_store(uint8_t* lds, int lane, const StageRegs<SLOT>& sr) {
  using S = StageShape<SLOT>;
#pragma unroll
  for (int j = 0; j < S::kLoads16; ++j) {
    const int c = lane + 64 * j;
    if (S::kChunks % 64 == 0 || c < S::kChunks) {
      const int row = c / S::kC16, cc = c - row * S::kC16;
      *reinterpret_cast<u32x4*>(lds + row * S::kRow + 16 * cc) = sr.d[j];
    }
  }
  if (lane < 16) {
    if constexpr (S::kTail == 8)
      *reinterpret_cast<u32x2*>(lds + lane * S::kRow + 16 * S::kC16) = sr.tail;
    else
      *reinterpret_cast<uint32_t*>(lds + lane * S::kRow + 16 * S::kC16) = sr.tail[0];
  }
}

// operands of one lane from the LDS copy of the slab (slot of row t at
// t * kRow + sh, sh = 0 or 2; reads stay inside the fetched span)
template <int KB, int SLOT>
__device__ __forceinline__ SlabOps<KB> staged_ops(const uint8_t* lds, int r16, int g4, uint32_t sh) {
  using S = StageShape<SLOT>;
  constexpr int kKCB = (kD * KB) / 8;
  constexpr int kKP = kKCB + 2;
  constexpr int kVCB = kD * vbits_of_slot(SLOT) / 8;
  constexpr int kLaneKB = KB == 4 ? 16 : 12;
  SlabOps<KB> op;
  {
    const uint32_t o = r16 * S::kRow + sh + kLaneKB * g4;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(lds + (o & ~3u));
    uint32_t w[kLaneKB / 4 + 1];
#pragma unroll
    for (int i = 0; i < kLaneKB / 4 + 1; ++i) w[i] = p[i];
#pragma unroll
    for (int i = 0; i < kLaneKB / 4; ++i) op.kw[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], o & 3u);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t rowo = (4 * g4 + r) * S::kRow + sh;
    const uint32_t vo = rowo + kKP + (vbits_of_slot(SLOT) == 3 ? 3 : 4) * r16;
    const uint32_t* pv = reinterpret_cast<const uint32_t*>(lds + (vo & ~3u));
    op.X[r] = __builtin_amdgcn_alignbyte(pv[1], pv[0], vo & 3u);
    op.n[r] = *reinterpret_cast<const uint16_t*>(lds + rowo + kKCB);
    const uint32_t so = rowo + kKP + kVCB;
    const uint32_t* ps = reinterpret_cast<const uint32_t*>(lds + (so & ~3u));
    op.sz[r] = __builtin_amdgcn_alignbyte(ps[1], ps[0], so & 3u);
  }
  return op;
}

// resident wavefronts per SIMD the staged kernel is built for (its register
// budget: 512 / waves)
template <int KB>
constexpr int kStagedWavesPerSimd = 3;

template <int KB, int SLOT>
__global__ void __launch_bounds__(64, kStagedWavesPerSimd<KB>) decode_staged_kernel(MfmaArgs a) {
  using S = StageShape<SLOT>;
  static_assert(KB == 3 || KB == 4, "staged kernel: 3/4-bit keys");

  __shared__ u32x2 s_tab[256];
  __shared__ int64_t s_page_off[kMaxChunkPages];
  __shared__ __align__(16) uint8_t s_stage[S::kStage + 16];

  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  // XCD-aware order, kv head fastest (as in the direct kernel): the heads of
  // one page row share cache lines and meet in one XCD's L2
  const int n_items = a.num_splits * a.batch * a.H;
  const int per_xcd = (n_items + 7) / 8;
  const int item = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
  if (item >= n_items) return;
  const int g = item % a.H;                  // kv head
  const int split = (item / a.H) % a.num_splits;
  const int b = item / (a.H * a.num_splits);
  const int64_t row_bytes = static_cast<int64_t>(a.H) * SLOT;
  const int64_t page_bytes = static_cast<int64_t>(1 << a.bs_shift) * row_bytes;

  build_tables<KB>(a, s_tab);
  const int T = clamp_len(a, b, split, g);
  const int t0 = split * a.chunk;
  const int t1 = min(T, t0 + a.chunk);
  stage_page_offsets(a, b, t0, t1, page_bytes, s_page_off);
  __syncthreads();
  if (t0 >= t1) return;

  h8 qhi[4], qlo[4];
  load_queries(a, b, g, r16, g4, a.scale_log2, qhi, qlo);
  const uint32_t rb = static_cast<uint32_t>(row_bytes);
  const uint32_t head_off = static_cast<uint32_t>(g * SLOT);
  const uint32_t head_off4 = head_off & ~3u;   // rows start 4-aligned (H even)
  const uint32_t sh = head_off & 3u;
  RunState st;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.O[m] = f4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.0f;
  st.z_part = 0.0f;
  const int p_first = t0 >> a.bs_shift;
  // One LDS buffer suffices: a wavefront's LDS accesses complete in issue
  // order, so the next slab's writes never overtake this slab's reads.
  uint8_t* lds = s_stage;
  const StageOffsets<SLOT> so = stage_offsets<SLOT>(lane, head_off4, rb);

  // two slabs in flight in registers
  StageRegs<SLOT> r0, r1;
  auto load = [&](int t, StageRegs<SLOT>& r) {
    bool ok;
    const __amdgpu_buffer_rsrc_t rs = slab_rsrc(a, s_page_off, p_first, t, t1, row_bytes, ok);
    r.ok = ok;
    stage_load<SLOT>(rs, so, r);
  };
  auto step = [&](int t, StageRegs<SLOT>& r) {
    // slab t is in r: park it in LDS, refill r with slab t + 32, compute slab t
    const bool ok = r.ok;
    stage_store<SLOT>(lds, lane, r);
    load(t + 32, r);
    if (ok) process_slab<KB, vbits_of_slot(SLOT)>(staged_ops<KB, SLOT>(lds, r16, g4, sh), t1 - t, s_tab, qhi, qlo, g4, st);
  };
  load(t0, r0);
  load(t0 + 16, r1);
  // whole rounds of two steps, no early exit: a step past the split end only
  // issues empty loads, which keeps the load count per step fixed
  for (int t = t0; t < t1; t += 32) {
    step(t, r0);
    step(t + 16, r1);
  }
  store_partials(a, b, g, split, g4, r16, st);
}

// ============================================================================
// page: one workgroup per (sequence, split), one wavefront per kv head (H = 1,
// 2, 4 or 8).  The H heads' rows of a 16-token slab are one contiguous block
// of a page (16 rows of H slots), so the workgroup streams whole slabs into an
// LDS ring with 16-byte buffer loads that write LDS directly, marked
// non-temporal: the cache is read once per decode step, and loads that do not
// allocate in the caches sustain about twice the read rate of plain loads on
// MI355X.  Every wavefront then takes its own head's operands from LDS.
//
// The centroid table holds hi = f16(c) and lo = f16(c - hi) for 4-bit keys
// (lo often subnormal: the matrix cores then sum its products less than
// exactly, but the lo term is about 2^-12 of the score, so that loss stays
// far below the score's own rounding) and
// lo = f16(2 (c - hi)) for 3-bit keys; the queries qhi = f16(q) and qlo =
// f16(q - qhi).  With at most 8 query heads per kv head one B operand
// carries both query parts: column h < 8 holds qhi of head h and column
// h + 8 its qlo, so hi.Q gives hi.qhi in column h and hi.qlo in column h + 8
// (added back across the row), and lo.Q gives lo.qhi: the score c.q to
// about 2^-20.  The norm takes hi.hi + 2 hi.lo = sum c^2 to the same order.
// The norm factor n / ||c|| of a token is computed once, in the lane that
// holds its diagonal element, and spread to the tile rows by one f32 MFMA
// (rows_to_tile).  4-bit keys here take score4 (below), whose A operands
// hold hi and lo side by side against duplicated queries.
// ============================================================================

constexpr int kMaxChunkSlabs = 256;          // slabs (and pages) of one split

// wavefronts per SIMD (128 VGPRs each)
constexpr int page_waves_per_simd(int) { return 4; }

template <int KB, int SLOT, int H>
struct PageGeom {
  static constexpr int kRow = H * SLOT;                     // bytes of one page row
  static constexpr int kSlab = 16 * kRow;                   // bytes of one slab in the cache
  static constexpr int kKCB = KB == 8 ? kD : kD * KB / 8;   // K code bytes
  static constexpr int kKP = KB == 8 ? kD : kKCB + 2;       // K bytes with the norm
  // In LDS every slot is re-laid in two parts that start on 16-byte
  // boundaries: the K codes (and norm), then the V codes, scale and zero, so
  // every operand read is aligned (unaligned LDS reads stall the LDS pipe).
  // The loads gather the 16-byte chunks of each part from its byte offset in
  // the cache.
  static constexpr int kNK = (kKP + 15) / 16;               // 16-byte chunks of the K part
  static constexpr int kNV = (SLOT - kKP + 15) / 16;        // ... of the V part
  static constexpr int kSlotL = 16 * (kNK + kNV);           // LDS bytes of one slot
  static constexpr int kVOff = 16 * kNK;                    // LDS offset of the V part
  static constexpr int kRowL = H * kSlotL;
  static constexpr int kSlabChunks = 16 * H * (kNK + kNV);
  static constexpr int kWaveLoads = (kSlabChunks + 63) / 64;  // wavefront loads of one slab
  static constexpr int kLoads = (kWaveLoads + H - 1) / H;   // loads per wavefront per slab, at most
  static constexpr int kFull = kWaveLoads - H * (kLoads - 1);  // wavefronts below this issue kLoads
  static constexpr int kBuf = kWaveLoads * 1024;            // LDS bytes of one slab buffer
  static constexpr int kTabBytes = KB == 8 ? 0 : 256 * 8;   // static LDS centroid table
  // 3/4-bit keys keep the per-lane load offsets in LDS (16 bytes per lane,
  // read before each slab's loads) instead of registers
  static constexpr bool kSrcInLds = KB != 8;
  static constexpr int kSrcBytes = kSrcInLds ? H * 64 * 16 : 0;
  static constexpr int kExtra = kTabBytes + 4 * kMaxChunkSlabs + kSrcBytes;
  static constexpr int kWavesPerSimd = page_waves_per_simd(KB);
  // workgroups per CU the register budget allows, and as many slab buffers
  // (3 to 8) as their share of the 160 KB of LDS holds
  static constexpr int kWgsPerCu = 4 * kWavesPerSimd / H;
  static constexpr int kNbufFit = (160 * 1024 / kWgsPerCu - kExtra) / kBuf;
  static constexpr int kNbuf = kNbufFit > 8 ? 8 : (kNbufFit < 3 ? 3 : kNbufFit);
  // dynamic LDS: page ids, then the slab ring (the centroid table is a
  // static array, so its address is a compile-time constant)
  static constexpr int kPidOff = 0;
  static constexpr int kSrcOff = kPidOff + 4 * kMaxChunkSlabs;
  static constexpr int kRingOff = kSrcOff + kSrcBytes;
  static_assert(kLoads <= 4, "load offsets do not fit 16 bytes per lane");
  static constexpr int kDynLds = kRingOff + kNbuf * kBuf;
  static constexpr int kLds = kDynLds + kTabBytes;
  static_assert(kLoads * (kNbuf - 2) < 64, "vmcnt out of range");
  static_assert(kVOff + kD * vbits_of_slot(SLOT) / 8 + 4 <= kSlotL, "V part does not fit");

  // cache byte offset, from the first slot of the workgroup's heads in the
  // slab's first row (rows row_bytes apart), of LDS chunk c (past the slab:
  // an offset beyond every buffer range, so the load returns zeros)
  __device__ static uint32_t chunk_src(int c, uint32_t row_bytes) {
    if (c >= kSlabChunks) return 0x7FFFFFF0u;
    const int si = c / (kNK + kNV), k = c - si * (kNK + kNV);
    const int row = si / H, head = si - row * H;
    const int off = k < kNK ? 16 * k : kKP + 16 * (k - kNK);
    return static_cast<uint32_t>(row * row_bytes + head * SLOT + off);
  }
};

// centroid tables (2 KB): entry e covers the codes e & (2^KB - 1) and
// e >> KB.  4-bit keys: {pair of hi parts, pair of lo parts} at 8-byte entry
// e, one lookup per code byte, lo = c - hi.  3-bit keys: the pair of hi parts
// at byte 4e and the pair of lo parts (lo = 2 (c - hi)) at byte kLoOff + 4e,
// two lookups from one address.  kLoOff = 1028 (257 words) is beyond a paired
// LDS read's reach (up to 255 words, or multiples of 64 words), so the
// compiler cannot fuse the two into one read into a register pair: each
// lands directly in its MFMA operand (fused, the pairs took 28 register moves
// per slab); the 64 entries of each half fill one row of banks, so the
// lookups never conflict.  A split 4-bit table (256 entries a half) measured
// slower than the 8-byte entries.
constexpr int kLoOff = 1028;
static_assert(kLoOff + 64 * 4 <= 256 * 8, "3-bit table halves within the 2 KB table");
template <int KB>
__device__ __forceinline__ void build_tables_page(const MfmaArgs& a, u32x2* tab) {
  constexpr int kTab = KB == 4 ? 256 : 64;
  uint32_t* t32 = reinterpret_cast<uint32_t*>(tab);
  for (int e = threadIdx.x; e < kTab; e += blockDim.x) {
    const int c0 = e & ((1 << KB) - 1), c1 = e >> KB;
    const float v0 = a.tables->centroids[c0], v1 = a.tables->centroids[c1];
    const _Float16 h0 = static_cast<_Float16>(v0), h1 = static_cast<_Float16>(v1);
    if constexpr (KB == 4) {
      // lo = c - hi unscaled (subnormal for the small levels, whose products
      // the matrix cores sum less than exactly: immaterial at 2^-12 of c)
      const _Float16 l0 = static_cast<_Float16>(v0 - static_cast<float>(h0));
      const _Float16 l1 = static_cast<_Float16>(v1 - static_cast<float>(h1));
      tab[e] = u32x2{pack_h2(h0, h1), pack_h2(l0, l1)};
    } else {
      const _Float16 l0 = static_cast<_Float16>(2.0f * (v0 - static_cast<float>(h0)));
      const _Float16 l1 = static_cast<_Float16>(2.0f * (v1 - static_cast<float>(h1)));
      t32[e] = pack_h2(h0, h1);
      t32[kLoOff / 4 + e] = pack_h2(l0, l1);
    }
  }
}

// rotated queries of kv head g packed as one B operand: lane (r16, g4) holds
// coordinates [32*g4, 32*g4 + 32) of head r16 % 8, its f16 hi part for
// r16 < 8 and its lo part for r16 >= 8 (zero for heads >= G)
__device__ __forceinline__ void load_queries_packed(const MfmaArgs& a, int b, int g, int r16, int g4,
                                                    h8 (&qc)[4]) {
  h8 qhi[4], qlo[4];
  load_queries(a, b, g, r16 & 7, g4, a.scale_log2, qhi, qlo);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qc[kk] = r16 < 8 ? qhi[kk] : qlo[kk];
}

// page ids of the split's pages -> LDS (-1: outside the cache)
__device__ __forceinline__ void stage_page_ids(const MfmaArgs& a, int b, int t0, int t1, int32_t* s_pid) {
  const int p_first = t0 >> a.bs_shift;
  const int n_pages = ((t1 - 1) >> a.bs_shift) - p_first + 1;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  for (int i = threadIdx.x; i < n_pages; i += blockDim.x) {
    const int page = bt[p_first + i];
    const bool ok = page >= 0 && page < a.num_blocks;
    if (!ok) a.errs->page = 1;
    s_pid[i] = ok ? page : -1;
  }
}

// 16 bytes per lane from buffer offset voff into LDS at dst + 16 * lane,
// non-temporal unless NT is false.  Written as inline assembly so the
// compiler does not treat the load as an LDS store it must wait for before
// every LDS read (it cannot tell the ring's slots apart); the kernel waits
// for these loads itself.
template <bool NT = true>
__device__ __forceinline__ void lds_dma_16(__amdgpu_buffer_rsrc_t rs, const uint8_t* dst, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)dst)));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wave_barrier() { asm volatile("s_barrier" ::: "memory"); }

// What one wavefront holds of one slab.  3/4-bit keys: the lane's code words
// (token r16, coordinates [32*g4, 32*g4 + 32)) and their centroid lookups;
// FP8 keys: the lane's 32 key bytes.  Both: the norm bits and V operands.
template <int KB>
struct SlabRegs {
  uint32_t kw[KB == 4 ? 4 : 3];  // code words (3/4-bit keys)
  u32x2 e[KB == 8 ? 1 : 16];     // {hi pair, lo pair} of code byte 4*kk + p
  u32x4 k8[KB == 8 ? 2 : 1];     // FP8 key bytes
  uint32_t nb;                   // norm bits of token 4*g4 + (r16 & 3)
  uint32_t nf[2];                // split page: folded norms of tokens 4*g4 .. 4*g4 + 3
  uint32_t X[4];                 // V codes of token 4*g4 + r, coordinates [8*r16, 8*r16 + 8)
  uint32_t sz[4];                // V scale | zero of token 4*g4 + r
};

// the slab's bytes for this lane, from its LDS buffer
template <int KB, int SLOT, int H>
__device__ __forceinline__ void slab_read(const uint8_t* buf, int w, int r16, int g4, SlabRegs<KB>& R) {
  using Geo = PageGeom<KB, SLOT, H>;
  constexpr int kRow = Geo::kRowL;
  const uint8_t* hb = buf + w * Geo::kSlotL;              // this head's slot in row 0
  const uint8_t* rb = hb + 4 * g4 * kRow;                 // ... in row 4*g4
  if constexpr (KB == 8) {
    const uint8_t* kp = hb + r16 * kRow + 32 * g4;
    R.k8[0] = *reinterpret_cast<const u32x4*>(kp);
    R.k8[1] = *reinterpret_cast<const u32x4*>(kp + 16);
    R.nb = 0;
  } else {
    if constexpr (KB == 4) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(hb + r16 * kRow + 16 * g4);
      R.kw[0] = t[0]; R.kw[1] = t[1]; R.kw[2] = t[2]; R.kw[3] = t[3];
    } else {
      typedef uint32_t u32x3a __attribute__((ext_vector_type(3), aligned(4)));
      const u32x3a t = *reinterpret_cast<const u32x3a*>(hb + r16 * kRow + 12 * g4);
      R.kw[0] = t[0]; R.kw[1] = t[1]; R.kw[2] = t[2];
    }
    // norm of token 4*g4 + (r16 & 3): only the lanes that hold its diagonal
    // element use it
    R.nb = *reinterpret_cast<const uint16_t*>(hb + (4 * g4 + (r16 & 3)) * kRow + Geo::kKCB);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (vbits_of_slot(SLOT) == 4) {
      R.X[r] = *reinterpret_cast<const uint32_t*>(rb + r * kRow + Geo::kVOff + 4 * r16);
    } else {
      // 3-bit codes of coordinates 8*r16 .. + 7: 3 bytes at 3*r16, read as
      // two aligned dwords and re-aligned
      const uint32_t* pv = reinterpret_cast<const uint32_t*>(rb + r * kRow + Geo::kVOff + ((3 * r16) & ~3));
      R.X[r] = __builtin_amdgcn_alignbyte(pv[1], pv[0], (3 * r16) & 3);
    }
    R.sz[r] = *reinterpret_cast<const uint32_t*>(rb + r * kRow + Geo::kVOff + kD * vbits_of_slot(SLOT) / 8);
  }
}

// centroid lookups of the code words (3/4-bit keys)
template <int KB>
__device__ __forceinline__ void slab_lookup(const u32x2* tab, SlabRegs<KB>& R) {
  const uint32_t* t32 = reinterpret_cast<const uint32_t*>(tab);
  if constexpr (KB != 8) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t idx;
        if constexpr (KB == 4) {
          idx = (R.kw[kk] >> (8 * p)) & 0xFFu;
        } else {
          // 6 bits (two codes) per lookup: bits [24*kk + 6*p, +6) of the lane's 96
          const int bit = 24 * kk + 6 * p;
          const int wd = bit >> 5, o = bit & 31;
          uint32_t v = R.kw[wd] >> o;
          if (o > 26) v |= R.kw[wd + 1] << (32 - o);
          idx = v & 63u;
        }
        if constexpr (KB == 4) R.e[4 * kk + p] = tab[idx];
        else R.e[4 * kk + p] = u32x2{t32[idx], t32[kLoOff / 4 + idx]};
      }
  }
}

// score and norm MFMAs of one slab: S = C . [qhi | qlo], Slo = Clo . [qhi | qlo],
// N = Chi . Chi^T + Chi . Clo^T (the norm accumulator starts at the 1e-16 of
// the correction's denominator); FP8 keys: S = K . q only
struct ScoreAcc {
  f4 S, Slo, Nh, Nx;
};

template <int KB, bool NORM = true>
__device__ __forceinline__ ScoreAcc slab_mfma(const SlabRegs<KB>& R, const h8 (&qc)[4], const bf8v (&qb)[4]) {
  ScoreAcc A;
  A.S = f4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KB == 8) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t w0 = R.k8[kk >> 1][2 * (kk & 1)], w1 = R.k8[kk >> 1][2 * (kk & 1) + 1];
      const bf2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
      const bf2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
      const bf2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
      const bf2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
      const bf8v av = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
      A.S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[kk], A.S, 0, 0, 0);
    }
  } else {
    A.Slo = f4{0.f, 0.f, 0.f, 0.f};
    A.Nh = f4{1e-16f, 1e-16f, 1e-16f, 1e-16f};
    A.Nx = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 hi, lo;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        hi[p] = R.e[4 * kk + p][0];
        lo[p] = R.e[4 * kk + p][1];
      }
      const h8 chi = __builtin_bit_cast(h8, hi);
      const h8 clo = __builtin_bit_cast(h8, lo);
      A.S = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, qc[kk], A.S, 0, 0, 0);
      A.Slo = __builtin_amdgcn_mfma_f32_16x16x32_f16(clo, qc[kk], A.Slo, 0, 0, 0);
      if constexpr (NORM) {
        A.Nh = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, chi, A.Nh, 0, 0, 0);
        A.Nx = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, clo, A.Nx, 0, 0, 0);
      }
    }
  }
  return A;
}

// weight of the Clo . q products: the 4-bit table holds lo = c - hi, the
// 3-bit table 2 (c - hi)
template <int KB>
__device__ __forceinline__ constexpr float lo_weight() { return KB == 4 ? 1.0f : 0.5f; }

// scores (base 2) of the slab from its MFMA results; rows at or past
// valid_rows score -inf
template <int KB, bool FULL>
__device__ __forceinline__ void slab_tail(const SlabRegs<KB>& R, const ScoreAcc& A, int valid_rows, int g4,
                                          float scale_log2, bool sel1, bool sel2, bool diag, float (&s)[4]) {
  if constexpr (KB == 8) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = (FULL || 4 * g4 + r < valid_rows) ? A.S[r] * scale_log2 : -INFINITY;
  } else {
    // lane (r16, g4) with r16 = 4*g4 + i holds N[4*g4 + i][4*g4 + i] as element i
    constexpr float kx = KB == 4 ? 2.0f : 1.0f;   // Nx = hi . lo (4-bit) or hi . 2 lo
    // the sums first, then one two-level select by the lane's row (the two
    // lane masks are loop-invariant)
    const f4 n = A.Nh + kx * A.Nx;
    const float n01 = sel1 ? n[1] : n[0];
    const float n23 = sel1 ? n[3] : n[2];
    const float nd = sel2 ? n23 : n01;
    const float fq = f16_bits_to_f32(R.nb) * __builtin_amdgcn_rsqf(nd);
    const f4 fac = rows_to_tile(fq, diag);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // column h + 8 (row rotation by 8) holds hi.qlo of head h; lanes
      // r16 >= 8 get a copy of head r16 - 8's score, which is never stored
      const float sr = A.S[r];
      const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sr), 0x128, 0xF, 0xF, false));
      s[r] = (FULL || 4 * g4 + r < valid_rows) ? (sr + other + lo_weight<KB>() * A.Slo[r]) * fac[r] : -INFINITY;
      // columns h and h + 8 differ in the lo term (lo.qhi against lo.qlo)
      s[r] = copy_to_upper8(s[r]);
    }
  }
}

// ---- 4-bit keys: lookups that are the score MFMA's A operand ----
// Two table entries (code bytes 2m and 2m + 1 of a lane) are read into one
// 4-register A operand as they come out of LDS: k-slots [hi c0, hi c1, lo c0,
// lo c1, hi c2, hi c3, lo c2, lo c3] for coordinates c0 .. c3.  The query
// operand lists each coordinate's query value in both its hi and its lo
// slot, so one MFMA per four coordinates sums (hi + lo) q = c q, with no
// register moves between the lookups and the MFMAs.  The norm of the
// centroid vector is sum (hi + lo)^2 = diag(A A^T) + 2 sum hi lo: the
// diagonal from MFMAs of each A operand with itself, the cross term from one
// v_dot2 (hi pair . lo pair) per entry.

// byte B of w times 8 (the byte offset of its table entry), one SDWA shift
template <int B>
__device__ __forceinline__ uint32_t byte_x8(uint32_t w) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(w));
  else if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(w));
  else if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}

// one 8-byte entry (8-byte aligned, so a single ds_read_b64 with the table's
// LDS address in its offset field)
typedef uint32_t u32x2a8 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2a8 tab_entry(const u32x2* tab, uint32_t byte_off) {
  return *reinterpret_cast<const u32x2a8*>(reinterpret_cast<const uint8_t*>(tab) + byte_off);
}

// query operands of the 4-bit path from the packed [qhi | qlo] columns:
// operand kk covers coordinates 32*g4 + 4*kk + [0, 4), each listed twice
__device__ __forceinline__ void queries_dup(const h8 (&qc)[4], h8 (&qd)[8]) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const h8 x = qc[kk >> 1];
    const int o = 4 * (kk & 1);
    qd[kk] = h8{x[o], x[o + 1], x[o], x[o + 1], x[o + 2], x[o + 3], x[o + 2], x[o + 3]};
  }
}

struct Acc4 {
  f4 S, N;
  float cross;       // sum hi * lo over the lane's 32 coordinates
};

// lookups and MFMAs of the slab in four quarters (two A operands live at a
// time); the query operand of MFMA kk comes from q(kk): registers, or the
// workgroup's copy in LDS
template <bool NORM, class QSrc>
__device__ __forceinline__ Acc4 score4(const u32x2* tab, const uint32_t (&kw)[4], QSrc q) {
  Acc4 r;
  r.S = f4{0.f, 0.f, 0.f, 0.f};
  r.N = f4{1e-16f, 1e-16f, 1e-16f, 1e-16f};     // the correction's 1e-16
  r.cross = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = kw[i];
    const u32x2a8 e0 = tab_entry(tab, byte_x8<0>(w));
    const u32x2a8 e1 = tab_entry(tab, byte_x8<1>(w));
    const u32x2a8 e2 = tab_entry(tab, byte_x8<2>(w));
    const u32x2a8 e3 = tab_entry(tab, byte_x8<3>(w));
    const u32x4 A[2] = {u32x4{e0[0], e0[1], e1[0], e1[1]}, u32x4{e2[0], e2[1], e3[0], e3[1]}};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kk = 2 * i + j;
      const h8 av = __builtin_bit_cast(h8, A[j]);
      r.S = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, q(kk), r.S, 0, 0, 0);
      if constexpr (NORM) {
        r.N = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, av, r.N, 0, 0, 0);
        r.cross = __builtin_amdgcn_fdot2(as_h2(A[j][0]), as_h2(A[j][1]),
                                         r.cross, false);
        r.cross = __builtin_amdgcn_fdot2(as_h2(A[j][2]), as_h2(A[j][3]),
                                         r.cross, false);
      }
    }
  }
  return r;
}

// scores (base 2) of the slab, 4-bit keys on the slotted page: column h + 8
// (row rotation by 8) holds the qlo part of head h; the norm factor n / |c|
// of token t is formed in the lane holding N[t][t] (lane (t, t / 4), element
// t % 4) and spread to the tile rows by one f32 MFMA
template <bool FULL>
__device__ __forceinline__ void tail4(uint32_t nb, const Acc4& A, int valid_rows, int g4, bool sel1,
                                      bool sel2, bool diag, float (&s)[4]) {
  const float cross = sum_x32(sum_x16(A.cross));        // token r16, all 128 coordinates
  const float nd = sel2 ? (sel1 ? A.N[3] : A.N[2]) : (sel1 ? A.N[1] : A.N[0]);
  const float fq = f16_bits_to_f32(nb) * __builtin_amdgcn_rsqf(__builtin_fmaf(2.0f, cross, nd));
  const f4 fac = rows_to_tile(fq, diag);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float sr = A.S[r];
    const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sr), 0x128, 0xF, 0xF, false));
    s[r] = (FULL || 4 * g4 + r < valid_rows) ? (sr + other) * fac[r] : -INFINITY;
  }
}

// scores (base 2) of the slab, 4-bit keys on the split page (folded norms)
template <bool FULL>
__device__ __forceinline__ void tail4_soa(const uint32_t (&nf)[2], const Acc4& A, int valid_rows, int g4,
                                          float (&s)[4]) {
  const float fac[4] = {f16_bits_to_f32(nf[0] & 0xFFFFu), f16_bits_to_f32(nf[0] >> 16),
                        f16_bits_to_f32(nf[1] & 0xFFFFu), f16_bits_to_f32(nf[1] >> 16)};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float sr = A.S[r];
    const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sr), 0x128, 0xF, 0xF, false));
    s[r] = (FULL || 4 * g4 + r < valid_rows) ? (sr + other) * fac[r] : -INFINITY;
  }
}

template <int KB, int SLOT, int H>
__global__ void __launch_bounds__(64 * H, page_waves_per_simd(KB)) decode_page_kernel(MfmaArgs a) {
  using Geo = PageGeom<KB, SLOT, H>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ __attribute__((aligned(16))) u32x2 s_tab[KB == 8 ? 1 : 256];
  u32x2* tab = s_tab;
  int32_t* s_pid = reinterpret_cast<int32_t*>(smem + Geo::kPidOff);

  // wavefront w takes kv head g = hg*H + w of the workgroup's head group hg
  // (the H kv heads of a row, or a part of them)
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int HG = a.H / H;
  const int hg = blockIdx.x % HG;
  const int b = (blockIdx.x / HG) / a.num_splits;
  const int split = (blockIdx.x / HG) % a.num_splits;
  const int g = hg * H + w;

  const int T = clamp_len(a, b, split, g);
  const int t0 = split * a.chunk;
  const int t1 = min(T, t0 + a.chunk);
  if (t0 >= t1) return;                      // the whole workgroup, before any barrier
  if constexpr (KB != 8) build_tables_page<KB>(a, tab);
  stage_page_ids(a, b, t0, t1, s_pid);
  __syncthreads();

  h8 qc[4];
  bf8v qb[4];
  if constexpr (KB == 8)
    load_queries_bf16(a, b, g, r16 & 7, g4, qb);    // columns h + 8 repeat head h
  else
    load_queries_packed(a, b, g, r16, g4, qc);
  h8 qd[8];                                  // 4-bit keys: the duplicated query operands
  if constexpr (KB == 4) queries_dup(qc, qd);
  RunState st;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.O[m] = f4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.0f;
  st.z_part = 0.0f;
  const bool sel1 = (r16 & 1) != 0, sel2 = (r16 & 2) != 0;

  const int p_first = t0 >> a.bs_shift;
  const int bs_mask = (1 << a.bs_shift) - 1;
  const int64_t row_bytes = static_cast<int64_t>(a.H) * SLOT;
  const int64_t page_bytes = static_cast<int64_t>(1 << a.bs_shift) * row_bytes;
  const uint32_t group_off = static_cast<uint32_t>(hg * H * SLOT);
  // the 16 rows from the group's first slot; the last chunks of its last
  // slot may run into the next group's first slot (never past the 16 rows)
  const uint32_t range = static_cast<uint32_t>(16 * row_bytes) - group_off;
  const int n_slabs = (t1 - t0 + 15) >> 4;
  const bool full_loads = w < Geo::kFull;
  uint32_t src_off[Geo::kLoads];
#pragma unroll
  for (int l = 0; l < Geo::kLoads; ++l)
    src_off[l] = Geo::chunk_src((w + H * l) * 64 + lane, static_cast<uint32_t>(row_bytes));
  u32x4* s_src = reinterpret_cast<u32x4*>(smem + Geo::kSrcOff) + threadIdx.x;
  if constexpr (Geo::kSrcInLds) {
    u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int l = 0; l < Geo::kLoads; ++l) v[l] = src_off[l];
    *s_src = v;                              // read back by this lane only
  }
  // the query loads are done before the first slab is requested, so every
  // wait in the loop counts slab loads only
  wait_vmcnt<0>();

  // slab j -> ring buffer j % kNbuf; a slab past the split end or on a bad
  // page gets an empty buffer range (its loads return zeros and touch no
  // memory), so every wavefront issues the same loads for every slab
  auto issue = [&](int j) {
    const int t = t0 + 16 * j;
    int pid = -1;
    if (t < t1) pid = s_pid[(t >> a.bs_shift) - p_first];
    pid = __builtin_amdgcn_readfirstlane(pid);
    const int64_t off = pid >= 0 ? pid * page_bytes + static_cast<int64_t>(t & bs_mask) * row_bytes + group_off : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.cache) + off, 0, pid >= 0 ? static_cast<int>(range) : 0, kBufferWord3);
    uint8_t* dst = smem + Geo::kRingOff + (j % Geo::kNbuf) * Geo::kBuf;
    u32x4 so;
    if constexpr (Geo::kSrcInLds) {
      so = *s_src;
    } else {
#pragma unroll
      for (int l = 0; l < Geo::kLoads; ++l) so[l] = src_off[l];
    }
#pragma unroll
    for (int l = 0; l < Geo::kLoads; ++l)
      if (l < Geo::kLoads - 1 || full_loads) lds_dma_16(rs, dst + (w + H * l) * 1024, so[l]);
  };
#pragma unroll
  for (int j = 0; j < Geo::kNbuf - 1; ++j) issue(j);

  // With slabs 0 .. i + kNbuf - 2 requested: this wavefront's part of slab i
  // has landed (the kNbuf - 2 newer ones may be in flight), its LDS reads
  // have completed, and the workgroup meets, so slab i is whole in LDS and
  // the buffer of slab i - 1 (read before the barrier) may be refilled.
  auto sync_slab = [&]() {
    if (full_loads)
      wait_vmcnt<Geo::kLoads * (Geo::kNbuf - 2)>();
    else
      wait_vmcnt<(Geo::kLoads - 1) * (Geo::kNbuf - 2)>();
    // lgkmcnt(0) as a builtin, so the compiler knows every LDS read has
    // completed and inserts no waits of its own for them later
    __builtin_amdgcn_s_waitcnt(0xC07F);
    wave_barrier();
  };
  auto slab_buf = [&](int jj) { return smem + Geo::kRingOff + (jj % Geo::kNbuf) * Geo::kBuf; };
  auto page_of = [&](int jj) { return s_pid[((t0 + 16 * jj) >> a.bs_shift) - p_first]; };
  const bool diag = (r16 >> 2) == g4;

  // Slab j is read and computed in iteration j.  The inner loop never changes
  // the accumulators except through the P.V MFMAs; a slab that raises the
  // running max past the lazy threshold leaves it, and the rescale and that
  // slab's P.V happen outside.
  int j = 0;
  while (true) {
    float s[4];
    SlabSoftmax sm;
    SlabRegs<KB> c;
    bool grow = false;
    for (; j < n_slabs; ++j) {
      sync_slab();
      issue(j + Geo::kNbuf - 1);           // into the buffer of slab j - 1
      if (__builtin_amdgcn_readfirstlane(page_of(j)) < 0) continue;
      slab_read<KB, SLOT, H>(slab_buf(j), w, r16, g4, c);
      const int valid = t1 - (t0 + 16 * j);
      if constexpr (KB == 4) {
        const Acc4 acc = score4<true>(tab, c.kw, [&](int kk) { return qd[kk]; });
        if (valid >= 16) {
          tail4<true>(c.nb, acc, 16, g4, sel1, sel2, diag, s);
          sm = softmax_check<true>(s, 16, c.sz, g4, st);
        } else {
          tail4<false>(c.nb, acc, valid, g4, sel1, sel2, diag, s);
          sm = softmax_check<false>(s, valid, c.sz, g4, st);
        }
      } else {
        slab_lookup<KB>(tab, c);
        const ScoreAcc acc = slab_mfma<KB>(c, qc, qb);
        if (valid >= 16) {
          slab_tail<KB, true>(c, acc, 16, g4, a.scale_log2, sel1, sel2, diag, s);
          sm = softmax_check<true>(s, 16, c.sz, g4, st);
        } else {
          slab_tail<KB, false>(c, acc, valid, g4, a.scale_log2, sel1, sel2, diag, s);
          sm = softmax_check<false>(s, valid, c.sz, g4, st);
        }
      }
      if (sm.grow) {
        grow = true;
        break;
      }
      softmax_accumulate<vbits_of_slot(SLOT)>(s, sm, c.X, st);
    }
    if (!grow) break;
    softmax_rescale(sm, diag, st);
    softmax_accumulate<vbits_of_slot(SLOT)>(s, sm, c.X, st);
    ++j;
  }
  wait_vmcnt<0>();                           // no load may still write LDS at exit
  fold_lo_rows(st);
  store_partials(a, b, g, split, g4, r16, st);
}

// ============================================================================
// ring: one workgroup of 16 wavefronts per (sequence, kv head, workgroup
// split), one per CU; or of 8 wavefronts, two per CU, when there are at
// least two rounds of workgroups (one's set-up and drain then overlap the
// other's streaming).  The wavefronts claim the workgroup's slabs one at a
// time from an LDS counter; each streams its claimed 16-row slabs of its head
// into a private LDS ring with loads that write LDS directly, in the page
// kernel's aligned slot layout, and computes them with the page kernel's slab
// code.  The wavefronts never wait for each other inside the loop (each
// waits only for its own loads).  At the end they combine their partial
// softmax states in LDS; with one workgroup split per sequence the workgroup
// writes the output itself, and no merge kernel runs.  The loads are plain,
// not non-temporal: a head's 16-byte chunks overlap its neighbours' slots,
// and those lines are then still in L2 when the neighbouring heads ask for
// them.  3/4-bit keys, at most 8 query heads per kv head.
// ============================================================================

// ---- split page (data region + meta region) ----
// One head's slab in LDS: its 16 data rows (K codes, then V codes), then the
// slab's 16 folded K norms, 16 V scales and 16 V zeros (fp16, 32 bytes each).
// Rows of 128 bytes (4-bit K and V) are packed, with the 16-byte chunk k of
// row t at position k ^ (t & 7) of the row, so that the same chunk of rows
// 0..7 falls in distinct bank groups; other rows are kRowL apart, an odd
// number of chunks, which spreads them the same way.  The meta chunks fill
// the last data load's spare lanes, or (128-byte rows) a load of 6 lanes.
template <int KB, int VB>
struct SoaGeom {
  static constexpr int kKCB = kD * KB / 8;                 // K code bytes
  static constexpr int kVCB = kD * VB / 8;                 // V code bytes
  static constexpr int kDB = kKCB + kVCB;                  // data bytes of a (token, head)
  static_assert(kDB % 16 == 0, "data rows of whole 16-byte chunks");
  static constexpr int kDataChunks = kDB / 16;
  static constexpr bool kSwizzle = kDataChunks == 8;
  static constexpr int kRowChunks = kSwizzle ? 8 : (kDataChunks | 1);
  static constexpr int kRowL = 16 * kRowChunks;
  static constexpr int kMetaOff = 16 * kRowL;
  static constexpr int kSlabChunks = 16 * kRowChunks + 6;
  static constexpr int kDataLoads = (16 * kRowChunks + 63) / 64;
  static constexpr bool kMetaOwnLoad = kSlabChunks > 64 * kDataLoads;
  static constexpr int kWaveLoads = kDataLoads + (kMetaOwnLoad ? 1 : 0);
  static_assert(!kMetaOwnLoad || kMetaOff == 1024 * kDataLoads, "meta load lands after the rows");
  static constexpr int kBuf = kMetaOwnLoad ? kMetaOff + 128 : 1024 * kWaveLoads;
  // LDS byte offset of 16-byte data chunk k of row t
  __device__ static constexpr int chunk_at(int t, int k) { return t * kRowL + 16 * (kSwizzle ? (k ^ (t & 7)) : k); }
};

// the slab's bytes for this lane from its LDS buffer (split page)
template <int KB, int VB>
__device__ __forceinline__ void slab_read_soa(const uint8_t* buf, int r16, int g4, SlabRegs<KB>& R) {
  using Geo = SoaGeom<KB, VB>;
  if constexpr (KB == 4) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(buf + Geo::chunk_at(r16, g4));
    R.kw[0] = t[0]; R.kw[1] = t[1]; R.kw[2] = t[2]; R.kw[3] = t[3];
  } else {
    typedef uint32_t u32x3a __attribute__((ext_vector_type(3), aligned(4)));
    const u32x3a t = *reinterpret_cast<const u32x3a*>(buf + r16 * Geo::kRowL + 12 * g4);
    R.kw[0] = t[0]; R.kw[1] = t[1]; R.kw[2] = t[2];
  }
  const uint8_t* rb = buf + 4 * g4 * Geo::kRowL + Geo::kKCB;    // V codes of row 4*g4
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (Geo::kSwizzle) {
      // V bytes [4*r16, 4*r16 + 4) of row 4*g4 + r: chunk kKCB/16 + r16/4
      R.X[r] = *reinterpret_cast<const uint32_t*>(
          buf + Geo::chunk_at(4 * g4 + r, Geo::kKCB / 16 + (r16 >> 2)) + 4 * (r16 & 3));
    } else if constexpr (VB == 4) {
      R.X[r] = *reinterpret_cast<const uint32_t*>(rb + r * Geo::kRowL + 4 * r16);
    } else {
      const uint32_t* pv = reinterpret_cast<const uint32_t*>(rb + r * Geo::kRowL + ((3 * r16) & ~3));
      R.X[r] = __builtin_amdgcn_alignbyte(pv[1], pv[0], (3 * r16) & 3);
    }
  }
  const uint8_t* meta = buf + Geo::kMetaOff + 8 * g4;              // tokens 4*g4 .. 4*g4 + 3
  const u32x2 n = *reinterpret_cast<const u32x2*>(meta);
  const u32x2 sc = *reinterpret_cast<const u32x2*>(meta + 32);
  const u32x2 zr = *reinterpret_cast<const u32x2*>(meta + 64);
  R.nf[0] = n[0];
  R.nf[1] = n[1];
  // V scale | zero << 16 per token
  R.sz[0] = __builtin_amdgcn_perm(zr[0], sc[0], 0x05040100u);
  R.sz[1] = __builtin_amdgcn_perm(zr[0], sc[0], 0x07060302u);
  R.sz[2] = __builtin_amdgcn_perm(zr[1], sc[1], 0x05040100u);
  R.sz[3] = __builtin_amdgcn_perm(zr[1], sc[1], 0x07060302u);
}

// scores (base 2) of a split-page slab: the stored norm already holds the
// correction, so it multiplies the rows directly
template <int KB, bool FULL>
__device__ __forceinline__ void slab_tail_soa(const uint32_t (&nf)[2], const ScoreAcc& A, int valid_rows,
                                              int g4, float (&s)[4]) {
  const float fac[4] = {f16_bits_to_f32(nf[0] & 0xFFFFu), f16_bits_to_f32(nf[0] >> 16),
                        f16_bits_to_f32(nf[1] & 0xFFFFu), f16_bits_to_f32(nf[1] >> 16)};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // column h + 8 holds hi.qlo of head h (as in slab_tail)
    const float sr = A.S[r];
    const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sr), 0x128, 0xF, 0xF, false));
    s[r] = (FULL || 4 * g4 + r < valid_rows) ? (sr + other + lo_weight<KB>() * A.Slo[r]) * fac[r] : -INFINITY;
    s[r] = copy_to_upper8(s[r]);
  }
}

constexpr int kRingBufs = 3;                 // slabs per wavefront ring (two in flight)
constexpr int kRingWaves = 16;               // wavefronts per workgroup (one workgroup per CU),
                                             // or half as many (two per CU; see ring_waves)
constexpr int kRingMaxSlabs = 1024;          // slabs per workgroup split: its page ids fit in LDS
constexpr int kXcdCus = 32;                  // CUs of one XCD (256 CUs in 8 XCDs)

template <int KB, int SLOT, bool SOA, int WAVES>
__global__ void __launch_bounds__(64 * WAVES, kRingWaves / WAVES) decode_ring_kernel(MfmaArgs a) {
  static_assert(KB == 3 || KB == 4, "ring kernel: 3/4-bit keys");
  constexpr int VB = vbits_of_slot(SLOT);
  using Geo = PageGeom<KB, SLOT, 1>;         // one head's slab layout in LDS (slotted page)
  using SGeo = SoaGeom<KB, VB>;              // ... (split page)
  constexpr int kLoads = SOA ? SGeo::kWaveLoads : Geo::kWaveLoads;   // 16-byte loads per lane per slab
  constexpr int kBuf = SOA ? SGeo::kBuf : 1024 * kLoads;   // covers every lane's chunk
  // slabs per wavefront ring: the split page's smaller slabs leave room for
  // a fourth (three in flight)
  constexpr int kBufs = SOA ? 4 : kRingBufs;
  constexpr int kRing = kBufs * kBuf;
  static_assert(8 * kRec * 4 <= kRing, "a wavefront's partial records must fit its ring");
  // one LDS block, carved by hand so the centroid table sits at address 0
  // (its entries are then addressed by the byte offset alone, the ds
  // instruction's 16-bit offset field holding nothing), then the page ids,
  // the claim counter and the wavefronts' rings
  struct RingLds {
    u32x2 tab[256];
    int32_t pid[kRingMaxSlabs];
    int32_t next;                            // the workgroup's next unclaimed slab
    int32_t started;                         // slabs its wavefronts have started, all told
    int32_t pad[2];
    uint8_t ring[WAVES][kRing];
  };
  static_assert(offsetof(RingLds, ring) % 16 == 0, "rings on 16-byte boundaries");
  __shared__ __attribute__((aligned(16))) RingLds lds;
  u32x2* const s_tab = lds.tab;
  int32_t* const s_pid = lds.pid;
  int32_t& s_next = lds.next;
  auto& s_ring = lds.ring;

  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  // XCD-aware order, kv head fastest: the heads of one page row run on one
  // XCD, where the cache lines their slots share come from its L2
  int b, g, sg;                              // sequence, kv head, workgroup split
  if (a.order != nullptr) {
    // sequences in length order: XCD x takes ranks x, x + 8, x + 16, ...,
    // each with its H * splits workgroups in a row, so the workgroups the
    // dispatcher starts first on an XCD are its longest sequences'.  The
    // dispatcher gives each of an XCD's 32 CUs one workgroup of the first 32
    // before any CU a second.  With two workgroups per CU (8 wavefronts) and
    // two whole layers on every XCD, the second layer takes the ranks of the
    // first mirrored about the middle of the two layers' ranks, so the CU
    // that runs rank i also runs rank 16 P - 1 - i (P sequences per layer):
    // the longest with the shortest, as even a pairing as the lengths allow
    // (k3v4-shaped ragged decode 120 -> 108 us).  Later layers start as CUs
    // free up and keep the longest-first order.
    const int hs = a.H * a.num_splits;
    const int k = static_cast<int>(blockIdx.x / 8);
    const int x = static_cast<int>(blockIdx.x % 8);
    int rank = x + 8 * (k / hs);
    // (both layers whole: every XCD has at least 2 * kXcdCus workgroups, so
    // the ranks below 16 P are all dealt out once)
    const bool two_layers = ((a.batch + 7) / 8) * hs >= 2 * kXcdCus;
    if (kRingWaves / WAVES == 2 && kXcdCus % hs == 0 && two_layers && k < 2 * kXcdCus) {
      const int per_layer = kXcdCus / hs;
      const int r0 = x + 8 * ((k % kXcdCus) / hs);
      rank = k < kXcdCus ? r0 : 16 * per_layer - 1 - r0;
    }
    if (rank >= a.batch) return;
    b = __builtin_amdgcn_readfirstlane(a.order[rank]);
    sg = (k % hs) / a.H;
    g = k % a.H;
  } else {
    const int n_items = a.num_splits * a.batch * a.H;
    const int per_xcd = (n_items + 7) / 8;
    const int item = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
    if (item >= n_items) return;
    g = item % a.H;
    sg = (item / a.H) % a.num_splits;
    b = item / (a.H * a.num_splits);
  }

  // this sequence's workgroup splits: a.chunk tokens at most each, the same
  // count the merge kernel derives; past them the workgroup has nothing to do
  const int T = clamp_len(a, b, sg, g);
  const int n_slabs_b = (T + 15) >> 4;
  const int cap = a.chunk >> 4;              // slabs per workgroup split, at most
  const int s_b = n_slabs_b > 0 ? (n_slabs_b + cap - 1) / cap : 1;
  if (sg >= s_b) return;                     // the whole workgroup, before any barrier
  const int cs = (n_slabs_b + WAVES * s_b - 1) / (WAVES * s_b);   // slabs per wavefront, on average
  const int wg0 = sg * WAVES * cs;           // the workgroup's slabs [wg0, wg1)
  const int wg1 = min(n_slabs_b, wg0 + WAVES * cs);
  const int n_wg = wg1 - wg0;
  const int t_end = min(T, 16 * wg1);        // the workgroup's last token + 1

  build_tables_page<KB>(a, s_tab);
  if (n_wg > 0) stage_page_ids(a, b, 16 * wg0, t_end, s_pid);
  if (threadIdx.x == 0) {
    s_next = 0;
    lds.started = 0;
  }
  // 4-bit keys on the split page: the duplicated query operands of score4
  // (the slotted page keeps the separate hi and lo MFMAs, whose norm terms
  // it needs anyway; measured faster there)
  constexpr bool kDup = KB == 4 && SOA;
  constexpr bool kBalance = WAVES == kRingWaves;   // issue priority to lagging wavefronts (below)
  h8 qv[4];
  bf8v qb[4];
  h8 qd[kDup ? 8 : 1];
  __syncthreads();
  load_queries_packed(a, b, g, r16, g4, qv);
  if constexpr (kDup) queries_dup(qv, qd);
  RunState st;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.O[m] = f4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.0f;
  st.z_part = 0.0f;
  const bool sel1 = (r16 & 1) != 0, sel2 = (r16 & 2) != 0;
  const bool diag = (r16 >> 2) == g4;

  const int p_first = (16 * wg0) >> a.bs_shift;
  const int bs_mask = (1 << a.bs_shift) - 1;
  const int64_t row_bytes = static_cast<int64_t>(a.H) * SLOT;
  const int64_t page_bytes = static_cast<int64_t>(1 << a.bs_shift) * row_bytes;
  // Slotted page: the slab of one head is 16 rows row_bytes apart; the lane's
  // chunk of load l is chunk l*64 + lane of the aligned layout (past the
  // slab: an offset beyond every buffer range, which loads zeros into the
  // ring's slack).  Split page: offsets from the page start, src_off +
  // r0 * src_mul for the slab starting at row r0 of its page (data rows
  // advance by a data row, meta fields by one fp16).
  uint32_t src_off[kLoads], src_mul[kLoads];
#pragma unroll
  for (int l = 0; l < kLoads; ++l) {
    const int c = l * 64 + lane;
    src_off[l] = 0x7FFFFFF0u;
    src_mul[l] = 0;
    if constexpr (SOA) {
      const uint32_t data_row = static_cast<uint32_t>(a.H) * SGeo::kDB;
      // position c of the slab buffer (the meta load's lanes 0..5 follow the rows)
      const int pc = SGeo::kMetaOwnLoad && l == kLoads - 1 ? 16 * SGeo::kRowChunks + lane : c;
      if (pc < 16 * SGeo::kRowChunks) {
        const int row = pc / SGeo::kRowChunks, k = pc - row * SGeo::kRowChunks;
        const int dk = SGeo::kSwizzle ? (k ^ (row & 7)) : k;   // the data chunk stored there
        if (dk < SGeo::kDataChunks) {
          src_off[l] = row * data_row + g * SGeo::kDB + 16 * dk;
          src_mul[l] = data_row;
        }
      } else if (pc < SGeo::kSlabChunks) {
        const int m = pc - 16 * SGeo::kRowChunks;         // fields norm, scale, zero: 2 chunks each
        src_off[l] = (data_row << a.bs_shift) + ((3 * g + (m >> 1)) << (a.bs_shift + 1)) + 16 * (m & 1);
        src_mul[l] = 2;
      }
    } else if (c < Geo::kSlabChunks) {
      const int row = c / (Geo::kNK + Geo::kNV), k = c - row * (Geo::kNK + Geo::kNV);
      const int off = k < Geo::kNK ? 16 * k : Geo::kKP + 16 * (k - Geo::kNK);
      src_off[l] = static_cast<uint32_t>(row * row_bytes + off);
    }
  }
  const uint32_t head_bytes = SOA ? 0u : static_cast<uint32_t>(g * SLOT);
  const uint32_t range = SOA ? static_cast<uint32_t>(page_bytes)
                             : static_cast<uint32_t>(16 * row_bytes) - head_bytes;
  uint8_t* ring = s_ring[w];
  // the query loads are done before the first slab is requested, so every
  // wait in the loop counts slab loads only
  wait_vmcnt<0>();

  // Slabs are claimed one at a time from the workgroup's counter (an LDS
  // atomic), so wavefronts that run ahead take more of them and all finish
  // within about one slab of each other (the wavefronts of a SIMD do not
  // progress at one rate; with fixed shares the last one finished up to
  // ~14 us after the median).  Which wavefront sums which slab then varies
  // from run to run, and so do the last bits of the result; a.dynamic == 0
  // deals the slabs out in a fixed order instead (wavefront w takes w,
  // w + 16, w + 32, ...), which is reproducible bit for bit.  A claim past
  // the workgroup's slabs still issues its loads, with an empty range (they
  // load zeros), so the count of loads in flight stays fixed.
  int n_claims = 0;
  auto claim = [&]() {
    if (!a.dynamic) return w + WAVES * n_claims++;
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_next, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  // the loads of claimed slab cj (workgroup-relative) into ring buffer j % kBufs
  auto issue = [&](int j, int cj) {
    const int t = 16 * (wg0 + cj);
    int pid = -1;
    if (cj < n_wg) pid = s_pid[(t >> a.bs_shift) - p_first];
    pid = __builtin_amdgcn_readfirstlane(pid);
    const int64_t off = pid < 0 ? 0
                      : SOA ? pid * page_bytes
                            : pid * page_bytes + static_cast<int64_t>(t & bs_mask) * row_bytes + head_bytes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.cache) + off, 0, pid >= 0 ? static_cast<int>(range) : 0, kBufferWord3);
    uint8_t* dst = ring + (j % kBufs) * kBuf;
    if constexpr (SOA) {
      // plain loads: the meta fields of neighbouring heads share lines, and
      // so do their data rows when a row is not 128 bytes (measured: the
      // same time as non-temporal loads for 4-bit rows, less traffic)
      const uint32_t r0 = static_cast<uint32_t>(t & bs_mask);
#pragma unroll
      for (int l = 0; l < SGeo::kDataLoads; ++l)
        lds_dma_16<false>(rs, dst + l * 1024, src_off[l] + r0 * src_mul[l]);
      if constexpr (SGeo::kMetaOwnLoad) {
        // 96 bytes: six lanes write LDS, the others are masked off
        if (lane < 6) lds_dma_16<false>(rs, dst + SGeo::kMetaOff, src_off[kLoads - 1] + r0 * src_mul[kLoads - 1]);
      }
    } else {
#pragma unroll
      for (int l = 0; l < kLoads; ++l) lds_dma_16<false>(rs, dst + l * 1024, src_off[l]);
    }
  };
  if (n_wg > 0) {
    int qc[kBufs - 1];                       // claims in flight, oldest first
#pragma unroll
    for (int i = 0; i < kBufs - 1; ++i) {
      qc[i] = claim();
      issue(i, qc[i]);
    }
    int j = 0;                               // this wavefront's slab count (ring position)
    while (true) {
      float s[4];
      SlabSoftmax sm;
      SlabRegs<KB> c;
      bool grow = false;
      for (;; ++j) {
        // slab j has landed (the next kBufs - 2 may be in flight); this
        // wavefront's reads of slab j - 1 have completed, so its buffer takes
        // the next claim
        wait_vmcnt<kLoads * (kBufs - 2)>();
        // One workgroup per CU (16 wavefronts): the wavefronts of a SIMD do
        // not progress at one rate, and the slowest sets the workgroup's
        // end.  A wavefront more than one slab behind the workgroup's mean
        // takes the highest issue priority until it has caught up (which
        // slabs it sums is unchanged, so the result is too; long_131k-shaped
        // decode 161 -> 147 us).  With two workgroups per CU the priorities
        // would also reorder the workgroups against each other: left off.
        int started = 0;
        if (kBalance && lane == 0) started = atomicAdd(&lds.started, 1);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        if constexpr (kBalance) {
          started = __builtin_amdgcn_readfirstlane(started);
          if ((j + 1) * WAVES < started) __builtin_amdgcn_s_setprio(3);
          else __builtin_amdgcn_s_setprio(0);
        }
        const int cur = qc[0];
#pragma unroll
        for (int i = 0; i + 1 < kBufs - 1; ++i) qc[i] = qc[i + 1];
        qc[kBufs - 2] = claim();
        issue(j + kBufs - 1, qc[kBufs - 2]);
        if (cur >= n_wg) break;              // claims only grow: nothing left
        if (__builtin_amdgcn_readfirstlane(s_pid[((16 * (wg0 + cur)) >> a.bs_shift) - p_first]) < 0) continue;
        if constexpr (SOA)
          slab_read_soa<KB, VB>(ring + (j % kBufs) * kBuf, r16, g4, c);
        else
          slab_read<KB, SLOT, 1>(ring + (j % kBufs) * kBuf, 0, r16, g4, c);
        const int valid = t_end - 16 * (wg0 + cur);
        if constexpr (kDup) {
          const Acc4 acc = score4<false>(s_tab, c.kw, [&](int kk) { return qd[kk]; });
          if (valid >= 16) {
            tail4_soa<true>(c.nf, acc, 16, g4, s);
            sm = softmax_check<true>(s, 16, c.sz, g4, st);
          } else {
            tail4_soa<false>(c.nf, acc, valid, g4, s);
            sm = softmax_check<false>(s, valid, c.sz, g4, st);
          }
        } else {
          slab_lookup<KB>(s_tab, c);
          const ScoreAcc acc = slab_mfma<KB, !SOA>(c, qv, qb);
          if (valid >= 16) {
            if constexpr (SOA)
              slab_tail_soa<KB, true>(c.nf, acc, 16, g4, s);
            else
              slab_tail<KB, true>(c, acc, 16, g4, a.scale_log2, sel1, sel2, diag, s);
            sm = softmax_check<true>(s, 16, c.sz, g4, st);
          } else {
            if constexpr (SOA)
              slab_tail_soa<KB, false>(c.nf, acc, valid, g4, s);
            else
              slab_tail<KB, false>(c, acc, valid, g4, a.scale_log2, sel1, sel2, diag, s);
            sm = softmax_check<false>(s, valid, c.sz, g4, st);
          }
        }
        if (sm.grow) {
          grow = true;
          break;
        }
        softmax_accumulate<VB, !kDup>(s, sm, c.X, st);
      }
      if (!grow) break;
      softmax_rescale(sm, diag, st);
      softmax_accumulate<VB, !kDup>(s, sm, c.X, st);
      ++j;
    }
    if constexpr (kBalance) __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();                         // no load may still write the ring
  }

  // ---- combine the wavefronts' states in LDS ----
  // each wavefront's records (O[128], m, l, z per query head) go into its own
  // ring, whose reads have all completed
  float* rec_w = reinterpret_cast<float*>(ring);
  fold_lo_rows(st);
  {
    const int G = a.G;
    const float l_part = sum_x32(sum_x16(st.l_part));
    const float z_part = sum_x32(sum_x16(st.z_part));
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): no read of the ring in flight
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g4 + r;
      if (h < G) {
        float* rec = rec_w + h * kRec;
        *reinterpret_cast<float4*>(rec + 8 * r16) = make_float4(
            st.O[0][r], st.O[1][r], st.O[2][r], st.O[3][r]);
        *reinterpret_cast<float4*>(rec + 8 * r16 + 4) = make_float4(
            st.O[4][r], st.O[5][r], st.O[6][r], st.O[7][r]);
      }
    }
    if (g4 == 0 && r16 < G) {
      float* rec = rec_w + r16 * kRec;
      rec[kD] = st.m_run;
      rec[kD + 1] = l_part;
      rec[kD + 2] = z_part;
    }
  }
  __syncthreads();
  // thread (h, pair): coordinates 2*pair, 2*pair + 1 of query head h
  const int h = threadIdx.x >> 6, pr = lane;
  if (h < a.G) {
    float M = -INFINITY, L = 0.0f;
    float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll 4
    for (int v = 0; v < WAVES; ++v) {
      const float* rec = reinterpret_cast<const float*>(s_ring[v]) + h * kRec;
      const float m = rec[kD];
      const float m_new = fmaxf(M, m);
      if (m_new == -INFINITY) continue;      // nothing attended yet
      const float cM = __builtin_amdgcn_exp2f(M - m_new);      // 0 on the first one
      const float wv = __builtin_amdgcn_exp2f(m - m_new);
      const float z = rec[kD + 2];
      const float2 o = *reinterpret_cast<const float2*>(rec + 2 * pr);
      acc.x = acc.x * cM + wv * (o.x + z);
      acc.y = acc.y * cM + wv * (o.y + z);
      L = L * cM + wv * rec[kD + 1];
      M = m_new;
    }
    const int hq = g * a.Gq + a.h0 + h;
    if (a.num_splits == 1) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const float r0 = acc.x * inv, r1 = acc.y * inv;
      const int64_t oi = (static_cast<int64_t>(b) * a.Hq + hq) * kD + 2 * pr;
      if (a.out_fp32) {
        *reinterpret_cast<float2*>(static_cast<float*>(a.out) + oi) = make_float2(r0, r1);
      } else {
        uint32_t u0 = __float_as_uint(r0), u1 = __float_as_uint(r1);
        u0 = (u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16;   // round to nearest even
        u1 = (u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16;
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi) = u0 | (u1 << 16);
      }
    } else {
      // the workgroup split's record for the merge kernel (zero term folded in)
      float* rec = a.part + ((static_cast<int64_t>(b) * a.Hq + hq) * a.num_splits + sg) * kRec;
      *reinterpret_cast<float2*>(rec + 2 * pr) = acc;
      if (pr == 0) *reinterpret_cast<float4*>(rec + kD) = make_float4(M, L, 0.0f, 0.0f);
    }
  }
}

template <int KB, int SLOT, int H>
hipError_t launch_page_t(const MfmaArgs& a, int batch, hipStream_t stream) {
  // one workgroup per (sequence, split, group of H kv heads)
  using Geo = PageGeom<KB, SLOT, H>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_page_kernel<KB, SLOT, H>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Geo::kDynLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((decode_page_kernel<KB, SLOT, H>), dim3(batch * a.num_splits * (a.H / H)), dim3(64 * H),
                     Geo::kDynLds, stream, a);
  return hipGetLastError();
}

template <int KB, int SLOT>
hipError_t launch_page_h(const MfmaArgs& a, int batch, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_page_t<KB, SLOT, 1>(a, batch, stream);
    case 2: return launch_page_t<KB, SLOT, 2>(a, batch, stream);
    case 4: return launch_page_t<KB, SLOT, 4>(a, batch, stream);
    case 8: return launch_page_t<KB, SLOT, 8>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

// ============================================================================
// direct, head dims 64 and 256: the direct kernel's design at the other head
// dims of the slotted page, up to 16 query heads per kv head in one pass
// (more in passes of 16), one wavefront per (split, sequence, kv head), each
// lane loading its operand bytes.
// Lane (r16, g4) holds K coordinates [(D/4)*g4, (D/4)*(g4+1)) of token r16
// (score step kk: (D/4)*g4 + 8*kk + [0, 8)), and the V codes of tokens
// 4*g4 + r for coordinates [(D/16)*r16, (D/16)*(r16+1)); value tile m column
// j covers coordinate (D/16)*j + m.  Signed-Hadamard queries are rotated in
// the kernel's prologue (load_queries_d); Haar queries once per pass by
// rotate_queries_d_kernel into the workspace.
// Scores, norm correction, softmax and P.V are those of the d = 128 direct
// kernel (score_slab, softmax_pv), over D/32 score steps and D/16 tiles.
// ============================================================================

template <int D, int KB, int VB>
struct DGeom {
  static constexpr int kKK = D / 32;                          // score MFMA steps
  static constexpr int kTiles = D / 16;                       // value tiles (coordinates per lane and token)
  static constexpr int kKCB = KB == 8 ? D : D * KB / 8;       // K code bytes
  static constexpr int kKP = KB == 8 ? D : kKCB + 2;          // + the fp16 norm (MSE keys)
  static constexpr int kVCB = D * VB / 8;                     // V code bytes
  static constexpr int kSlotRaw = kKP + kVCB + 4;             // + fp16 scale and zero
  static constexpr int kSlot = kSlotRaw + kSlotRaw % 2;
  static constexpr int kLaneKB = (D / 4) * KB / 8;            // K bytes of a lane
  // dwords loaded: 3-bit keys at d = 64 take 6 bytes and two bytes of the
  // norm ride along
  static constexpr int kLaneKW = (kLaneKB + 3) / 4;
  // V dwords of a lane per token: 4-bit 2 bytes (d 64) or 8 (d 256); 3-bit
  // 12 bits in a 2-byte-aligned dword (d 64) or 6 bytes (d 256)
  static constexpr int kVW = D == 256 ? 2 : 1;
  static constexpr int kRecD = D + 4;                         // partial record: O[D], m, l, z, pad
  static_assert(D == 64 || D == 256, "head dims 64 and 256");
};

template <int D>
constexpr int kDWavesPerSimd = D == 256 ? 2 : 4;

template <int D>
struct RunStateD {
  f4 O[D / 16];     // O[h][(D/16)*r16 + m]: tile m, rows 4*g4 + r
  float m_run;
  float l_part;
  float z_part;
};

template <int D, int KB, int VB>
struct DRegs {
  uint32_t kw[DGeom<D, KB, VB>::kLaneKW];
  uint32_t X[4][DGeom<D, KB, VB>::kVW];
  uint32_t n[4];
  uint32_t sz[4];
  bool ok;
};

template <int D, int KB, int VB>
struct DOffsets {
  uint32_t k;
  uint32_t row[4];
  uint32_t v[4];
  uint32_t vshift;   // 3-bit V at d = 64: bit offset of the lane's codes in its dword
};

template <int D, int KB, int VB>
__device__ __forceinline__ DOffsets<D, KB, VB> dslab_offsets(int r16, int g4, uint32_t head_off, uint32_t rb) {
  using DG = DGeom<D, KB, VB>;
  DOffsets<D, KB, VB> o;
  o.k = r16 * rb + head_off + DG::kLaneKB * g4;
  uint32_t vb;
  if constexpr (VB == 3 && D == 64) {
    // bits [12*r16, 12*r16 + 12) of the V codes, from the 2-byte word holding
    // their first bit (the dword read stays inside the slot: the V scale follows)
    const uint32_t bit = 12u * r16;
    vb = 2u * (bit >> 4);
    o.vshift = bit & 15u;
  } else {
    vb = static_cast<uint32_t>(DG::kTiles * VB / 8) * r16;
    o.vshift = 0;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o.row[r] = (4 * g4 + r) * rb + head_off;
    o.v[r] = o.row[r] + DG::kKP + vb;
  }
  return o;
}

template <int D, int KB, int VB>
__device__ __forceinline__ void dslab_load(__amdgpu_buffer_rsrc_t rs, const DOffsets<D, KB, VB>& o,
                                           DRegs<D, KB, VB>& d) {
  using DG = DGeom<D, KB, VB>;
  constexpr int W = DG::kLaneKW;
  int i = 0;
#pragma unroll
  for (; i + 4 <= W; i += 4) {
    const u32x4 t = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.k + 4 * i, 0, 0));
    d.kw[i] = t[0]; d.kw[i + 1] = t[1]; d.kw[i + 2] = t[2]; d.kw[i + 3] = t[3];
  }
  if constexpr (W % 4 >= 2) {
    const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, o.k + 4 * (W - W % 4), 0, 0));
    d.kw[W - W % 4] = t[0];
    d.kw[W - W % 4 + 1] = t[1];
  }
  if constexpr (W % 2 == 1) d.kw[W - 1] = __builtin_amdgcn_raw_buffer_load_b32(rs, o.k + 4 * (W - 1), 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (DG::kVW == 2) {
      const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, o.v[r], 0, 0));
      d.X[r][0] = t[0];
      d.X[r][1] = t[1];
    } else if constexpr (VB == 4) {
      d.X[r][0] = __builtin_amdgcn_raw_buffer_load_b16(rs, o.v[r], 0, 0);
    } else {
      d.X[r][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, o.v[r], 0, 0);
    }
    if constexpr (KB != 8) d.n[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, o.row[r] + DG::kKCB, 0, 0);
    d.sz[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, o.row[r] + DG::kKP + DG::kVCB, 0, 0);
  }
}

// queries of kv head g rotated as the store rotated the keys, times the
// softmax scale (base 2), as f16 hi / lo B operands; lane (h = r16, g4), step
// kk: coordinates (D/4)*g4 + 8*kk + [0, 8).  Signed Hadamard: the lane's
// D/4 coordinates flipped and butterflied in registers (strides below D/4),
// strides D/4 and D/2 with the partner lanes l ^ 16 and l ^ 32, times
// 1/sqrt(D) (as load_queries at d = 128).  Haar: read rotated from the
// workspace (a.q_rot, rotate_queries_d_kernel).
template <int D>
__device__ __forceinline__ void load_queries_d(const MfmaArgs& a, int b, int g, int r16, int g4,
                                               h8 (&qhi)[D / 32], h8 (&qlo)[D / 32]) {
  constexpr int E = D / 4;
  const bool live = r16 < a.G;
  const int64_t row = (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0 + (live ? r16 : 0)) * D + E * g4;
  float x[E];
  float fs = a.scale_log2;
  if (a.q_rot != nullptr) {
    const float4* rp = reinterpret_cast<const float4*>(a.q_rot + row);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 v = rp[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  } else {
    const uint16_t* qp = a.q + row;
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int c = E * g4 + j;
      const uint32_t sb = (a.tables->sign_bits[c >> 5] >> (c & 31)) & 1u;
      x[j] = __uint_as_float(__float_as_uint(x[j]) ^ (sb << 31));
    }
#pragma unroll
    for (int hs = 1; hs < E; hs *= 2)
#pragma unroll
      for (int j = 0; j < E; ++j)
        if ((j & hs) == 0) {
          const float p = x[j], r = x[j + hs];
          x[j] = p + r;
          x[j + hs] = p - r;
        }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
      const float o = (g4 & 1) ? __uint_as_float(sw[0]) : __uint_as_float(sw[1]);
      x[j] = (g4 & 1) ? (o - x[j]) : (x[j] + o);
    }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
      const float o = (g4 & 2) ? __uint_as_float(sw[0]) : __uint_as_float(sw[1]);
      x[j] = (g4 & 2) ? (o - x[j]) : (x[j] + o);
    }
    fs *= D == 64 ? 0.125f : 0.0625f;          // 1 / sqrt(D)
  }
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = live ? x[8 * kk + e] * fs : 0.0f;
      const _Float16 hv = static_cast<_Float16>(v);
      qhi[kk][e] = hv;
      qlo[kk][e] = static_cast<_Float16>(v - static_cast<float>(hv));
    }
}

// FP8 keys: the queries as given (bf16), same coordinates
template <int D>
__device__ __forceinline__ void load_queries_bf16_d(const MfmaArgs& a, int b, int g, int r16, int g4,
                                                    bf8v (&qb)[D / 32]) {
  const bool live = r16 < a.G;
  const uint16_t* qp =
      a.q + (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0 + (live ? r16 : 0)) * D + (D / 4) * g4;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    u32x4 w = *reinterpret_cast<const u32x4*>(qp + 8 * kk);
    if (!live) w = u32x4{0u, 0u, 0u, 0u};
    qb[kk] = __builtin_bit_cast(bf8v, w);
  }
}

// scores (base 2) of the lane's 4 rows for 3/4-bit keys (as score_slab)
template <int D, int KB, int VB>
__device__ __forceinline__ void score_slab_d(const DRegs<D, KB, VB>& op, int valid_rows, const u32x2* s_tab,
                                             const h8 (&qhi)[D / 32], const h8 (&qlo)[D / 32], int g4,
                                             float (&s)[4]) {
  f4 Shi = {0.f, 0.f, 0.f, 0.f}, Slo = {0.f, 0.f, 0.f, 0.f};
  f4 Nhi = {1e-16f, 1e-16f, 1e-16f, 1e-16f}, Nx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    uint32_t idx[4];
    if constexpr (KB == 4) {
#pragma unroll
      for (int p = 0; p < 4; ++p) idx[p] = (op.kw[kk] >> (8 * p)) & 0xFFu;
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int bit = 24 * kk + 6 * p;
        const int w = bit >> 5, o = bit & 31;
        uint32_t v = op.kw[w] >> o;
        if (o > 26) v |= op.kw[w + 1] << (32 - o);
        idx[p] = v & 63u;
      }
    }
    u32x4 hi, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x2 e = s_tab[idx[p]];
      hi[p] = e[0];
      lo[p] = e[1];
    }
    const h8 chi = __builtin_bit_cast(h8, hi);
    const h8 clo = __builtin_bit_cast(h8, lo);
    Shi = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, qhi[kk], Shi, 0, 0, 0);
    Shi = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, qlo[kk], Shi, 0, 0, 0);
    Slo = __builtin_amdgcn_mfma_f32_16x16x32_f16(clo, qhi[kk], Slo, 0, 0, 0);
    Nhi = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, chi, Nhi, 0, 0, 0);
    Nx = __builtin_amdgcn_mfma_f32_16x16x32_f16(chi, clo, Nx, 0, 0, 0);
  }
  const int diag_src = 20 * g4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float nd = Nhi[r] + (2.0f / kLoScale) * Nx[r];
    const float nn = lane_value(nd, diag_src + r);
    const float fac = f16_bits_to_f32(op.n[r]) * __builtin_amdgcn_rsqf(nn);
    const float dot = Shi[r] + Slo[r] * (1.0f / kLoScale);
    s[r] = 4 * g4 + r < valid_rows ? dot * fac : -INFINITY;
  }
}

// scores (base 2) for FP8 keys (as score_slab8)
template <int D, int KB, int VB>
__device__ __forceinline__ void score_slab8_d(const DRegs<D, KB, VB>& op, int valid_rows, const bf8v (&qb)[D / 32],
                                              float scale_log2, int g4, float (&s)[4]) {
  f4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const uint32_t w0 = op.kw[2 * kk], w1 = op.kw[2 * kk + 1];
    const bf2 c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf2 c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf2 c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    const bf8v av = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
    S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[kk], S, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = 4 * g4 + r < valid_rows ? S[r] * scale_log2 : -INFINITY;
}

// online softmax and P.V of one slab (as softmax_pv, over D/16 tiles); the
// lane's V codes of token 4*g4 + r are X[r] (kVW dwords, from bit 0)
template <int D, int KB, int VB>
__device__ __forceinline__ void softmax_pv_d(const float (&s)[4], int valid_rows, const DRegs<D, KB, VB>& op,
                                             uint32_t vshift, int g4, RunStateD<D>& st) {
  float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  float sc[4], zr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t szm = 4 * g4 + r < valid_rows ? op.sz[r] : 0u;
    sc[r] = f16_bits_to_f32(szm & 0xFFFFu);
    zr[r] = f16_bits_to_f32(szm >> 16);
  }
  const float sc_max = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  const float thr = sc_max > 1000.0f ? 0.0f : kLazy;
  if (__any(pm > st.m_run + thr)) {
    const float m_new = fmaxf(st.m_run, max_x32(max_x16(pm)));
    const float corr = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.l_part *= corr;
    st.z_part *= corr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float cr = lane_value(corr, 4 * g4 + r);
#pragma unroll
      for (int m = 0; m < D / 16; ++m) st.O[m][r] *= cr;
    }
    st.m_run = m_new;
  }
  h4 W, Wl;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = __builtin_amdgcn_exp2f(s[r] - st.m_run);
    st.l_part += p;
    st.z_part += p * zr[r];
    const float wf = p * sc[r];
    W[r] = static_cast<_Float16>(wf);
    Wl[r] = static_cast<_Float16>(wf - static_cast<float>(W[r]));
  }
  const h8 Ws = {W[0], W[1], W[2], W[3], Wl[0], Wl[1], Wl[2], Wl[3]};
  // kb: coordinates 2*kb and 2*kb + 1 of the lane (tiles 2*kb, 2*kb + 1);
  // 4-bit codes: byte kb % 4 of dword kb / 4; 3-bit codes: bits 6*kb on,
  // taken from the 24-bit group kb / 4
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) {
    uint32_t Xk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (VB == 4)
        Xk[r] = op.X[r][kb / 4];
      else if constexpr (D == 64)
        Xk[r] = op.X[r][0] >> vshift;
      else
        Xk[r] = kb < 4 ? op.X[r][0] : ((op.X[r][0] >> 24) | (op.X[r][1] << 8));
    }
    h4 Blo4, Bhi4;
    v_operands<VB>(Xk, kb % 4, Blo4, Bhi4);
    const h8 Blo = {Blo4[0], Blo4[1], Blo4[2], Blo4[3], Blo4[0], Blo4[1], Blo4[2], Blo4[3]};
    const h8 Bhi = {Bhi4[0], Bhi4[1], Bhi4[2], Bhi4[3], Bhi4[0], Bhi4[1], Bhi4[2], Bhi4[3]};
    st.O[2 * kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ws, Blo, st.O[2 * kb], 0, 0, 0);
    st.O[2 * kb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ws, Bhi, st.O[2 * kb + 1], 0, 0, 0);
  }
}

// split partials of this wavefront: record [O[D], m, l, z, pad] per
// (sequence, query head, split); O rows are heads 4*g4 + r
template <int D>
__device__ __forceinline__ void store_partials_d(const MfmaArgs& a, int b, int g, int split, int g4, int r16,
                                                 const RunStateD<D>& st) {
  constexpr int kRecD = D + 4;
  constexpr int NT = D / 16;
  const float l_part = sum_x32(sum_x16(st.l_part));
  const float z_part = sum_x32(sum_x16(st.z_part));
  const int64_t rec0 = (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0) * a.num_splits + split;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g4 + r;
    if (h < a.G) {
      float* rec = a.part + (rec0 + static_cast<int64_t>(h) * a.num_splits) * kRecD + NT * r16;
#pragma unroll
      for (int m = 0; m < NT; m += 4)
        *reinterpret_cast<float4*>(rec + m) = make_float4(st.O[m][r], st.O[m + 1][r], st.O[m + 2][r], st.O[m + 3][r]);
    }
  }
  if (g4 == 0 && r16 < a.G) {
    float* rec = a.part + (rec0 + static_cast<int64_t>(r16) * a.num_splits) * kRecD;
    rec[D] = st.m_run;
    rec[D + 1] = l_part;
    rec[D + 2] = z_part;
  }
}

template <int D, int KB, int VB>
__global__ void __launch_bounds__(64, kDWavesPerSimd<D>) decode_dslab_kernel(MfmaArgs a) {
  using DG = DGeom<D, KB, VB>;
  __shared__ u32x2 s_tab[256];
  __shared__ int64_t s_page_off[kMaxChunkPages];

  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  // XCD-aware order, kv head fastest (as the d = 128 direct kernel)
  const int n_items = a.num_splits * a.batch * a.H;
  const int per_xcd = (n_items + 7) / 8;
  const int item = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
  if (item >= n_items) return;
  const int g = item % a.H;
  const int split = (item / a.H) % a.num_splits;
  const int b = item / (a.H * a.num_splits);
  const int64_t row_bytes = static_cast<int64_t>(a.H) * DG::kSlot;
  const int64_t page_bytes = static_cast<int64_t>(1 << a.bs_shift) * row_bytes;

  if constexpr (KB != 8) build_tables<KB>(a, s_tab);
  const int T = clamp_len(a, b, split, g);
  const int t0 = split * a.chunk;
  const int t1 = min(T, t0 + a.chunk);
  stage_page_offsets(a, b, t0, t1, page_bytes, s_page_off);
  __syncthreads();
  if (t0 >= t1) return;

  h8 qhi[KB == 8 ? 1 : D / 32], qlo[KB == 8 ? 1 : D / 32];
  bf8v qb[KB == 8 ? D / 32 : 1];
  if constexpr (KB == 8)
    load_queries_bf16_d<D>(a, b, g, r16, g4, qb);
  else
    load_queries_d<D>(a, b, g, r16, g4, qhi, qlo);
  RunStateD<D> st;
#pragma unroll
  for (int m = 0; m < D / 16; ++m) st.O[m] = f4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.0f;
  st.z_part = 0.0f;
  const int p_first = t0 >> a.bs_shift;
  const DOffsets<D, KB, VB> off = dslab_offsets<D, KB, VB>(r16, g4, static_cast<uint32_t>(g * DG::kSlot),
                                                           static_cast<uint32_t>(row_bytes));

  // two slabs in flight in two register sets, the same loads every step (an
  // empty range past the split end or on a bad page)
  DRegs<D, KB, VB> r0, r1;
  auto load = [&](int t, DRegs<D, KB, VB>& r) {
    bool ok;
    const __amdgpu_buffer_rsrc_t rs = slab_rsrc(a, s_page_off, p_first, t, t1, row_bytes, ok);
    r.ok = ok;
    dslab_load<D, KB, VB>(rs, off, r);
  };
  auto step = [&](int t, DRegs<D, KB, VB>& r) {
    if (r.ok) {
      float sc[4];
      if constexpr (KB == 8)
        score_slab8_d<D, KB, VB>(r, t1 - t, qb, a.scale_log2, g4, sc);
      else
        score_slab_d<D, KB, VB>(r, t1 - t, s_tab, qhi, qlo, g4, sc);
      softmax_pv_d<D, KB, VB>(sc, t1 - t, r, off.vshift, g4, st);
    }
    load(t + 32, r);
  };
  load(t0, r0);
  load(t0 + 16, r1);
  for (int t = t0; t < t1; t += 32) {
    step(t, r0);
    step(t + 16, r1);
  }
  store_partials_d<D>(a, b, g, split, g4, r16, st);
}

// Haar rotation of the queries at head dims 64 and 256, once per decode:
// q_rot = Q q into the workspace (fp32 [B][Hq][D]), Q the D x D matrix the
// store applied to the keys.  One workgroup per (sequence, kv head), thread i
// forms coordinate i of its G queries (each row of Q read once).
template <int D>
__global__ void __launch_bounds__(D) rotate_queries_d_kernel(MfmaArgs a, float* q_rot) {
  __shared__ float s_q[16][D];
  const int b = blockIdx.x / a.H, g = blockIdx.x - b * a.H;
  const int i = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * a.Hq + g * a.Gq + a.h0) * D;
  for (int h = 0; h < a.G; ++h)
    s_q[h][i] = __uint_as_float(static_cast<uint32_t>(a.q[base + h * D + i]) << 16);
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) acc[h] = 0.0f;
  const float* rowq = a.tables->rot + static_cast<int64_t>(i) * D;
  for (int j = 0; j < D; ++j) {
    const float qij = rowq[j];
#pragma unroll
    for (int h = 0; h < 16; ++h)
      if (h < a.G) acc[h] = __builtin_fmaf(qij, s_q[h][j], acc[h]);
  }
#pragma unroll
  for (int h = 0; h < 16; ++h)
    if (h < a.G) q_rot[base + h * D + i] = acc[h];
}

// merge of the splits of one (sequence, query head), as decode_merge_kernel:
// four wavefronts take every fourth split (the loads of four of its splits
// issued together), lane = coordinates E*lane + e
template <int D>
__global__ void __launch_bounds__(256) decode_merge_d_kernel(MfmaArgs a) {
  constexpr int E = D / 64;
  constexpr int kRecD = D + 4;
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][D];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = effective_len(a, b);
  const int nsp = (T + a.chunk - 1) / a.chunk;
  const float* recs = a.part + static_cast<int64_t>(bh) * a.num_splits * kRecD;
  float M = -INFINITY, L = 0.0f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  constexpr int kU = 4;
  for (int s0 = wv; s0 < nsp; s0 += 4 * kU) {
    float4 mlz[kU];
    float o[kU][E];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int sp = s0 + 4 * u;
      const float* rec = recs + static_cast<int64_t>(sp < nsp ? sp : s0) * kRecD;
      mlz[u] = *reinterpret_cast<const float4*>(rec + D);     // m, l, z, pad
#pragma unroll
      for (int e = 0; e < E; ++e) o[u][e] = rec[E * lane + e];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s0 + 4 * u >= nsp) break;
      const float m_new = fmaxf(M, mlz[u].x);
      if (m_new == -INFINITY) continue;                       // nothing attended yet (bad pages)
      const float c = __builtin_amdgcn_exp2f(M - m_new);
      const float w = __builtin_amdgcn_exp2f(mlz[u].x - m_new);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = acc[e] * c + w * (o[u][e] + mlz[u].z);
      L = L * c + w * mlz[u].y;
      M = m_new;
    }
  }
  if (lane == 0) {
    s_m[wv] = M;
    s_l[wv] = L;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) s_acc[wv][E * lane + e] = acc[e];
  __syncthreads();
  if (wv != 0) return;
  const float Mx = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float Lt = 0.0f, tot[E];
#pragma unroll
  for (int e = 0; e < E; ++e) tot[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w = s_m[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s_m[i] - Mx);
#pragma unroll
    for (int e = 0; e < E; ++e) tot[e] += w * s_acc[i][E * lane + e];
    Lt += w * s_l[i];
  }
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  const int64_t oi = static_cast<int64_t>(bh) * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float r = tot[e] * inv;
    if (a.out_fp32) {
      static_cast<float*>(a.out)[oi + e] = r;
    } else {
      uint32_t u = __float_as_uint(r);
      u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;     // round to nearest even
      static_cast<uint16_t*>(a.out)[oi + e] = static_cast<uint16_t>(u);
    }
  }
}

// query heads in passes of at most 16 per kv head (each pass reads the
// cache; Haar queries rotated per pass), one merge for every head
template <int D>
hipError_t launch_dslab_d(const Geometry& g, const DecodePlan& plan, MfmaArgs& a, int batch, float* q_rot,
                          hipStream_t stream) {
  const int n_items = plan.num_splits * batch * g.num_kv_heads;
  const dim3 grid(8 * ((n_items + 7) / 8));
  for (int h0 = 0; h0 < a.Gq; h0 += 16) {
    a.h0 = h0;
    a.G = a.Gq - h0 < 16 ? a.Gq - h0 : 16;
    if (g.key_bits != 8 && g.haar) {
      a.q_rot = nullptr;
      hipLaunchKernelGGL((rotate_queries_d_kernel<D>), dim3(batch * g.num_kv_heads), dim3(D), 0, stream, a, q_rot);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      a.q_rot = q_rot;
    }
    if (g.key_bits == 8)
      hipLaunchKernelGGL((decode_dslab_kernel<D, 8, 4>), grid, dim3(64), 0, stream, a);
    else if (g.key_bits == 4)
      hipLaunchKernelGGL((decode_dslab_kernel<D, 4, 4>), grid, dim3(64), 0, stream, a);
    else if (g.value_bits == 4)
      hipLaunchKernelGGL((decode_dslab_kernel<D, 3, 4>), grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_dslab_kernel<D, 3, 3>), grid, dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.h0 = 0;
  a.G = a.Gq;
  hipLaunchKernelGGL((decode_merge_d_kernel<D>), dim3(batch * a.Hq), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int mfma_waves_per_cu(const Geometry& g, bool staged) {
  if (staged) return 4 * (g.key_bits == 4 ? kStagedWavesPerSimd<4> : kStagedWavesPerSimd<3>);
  const int per_simd = g.key_bits == 8 ? kSlabWavesPerSimd<8>
                     : (g.key_bits == 4 ? kSlabWavesPerSimd<4> : kSlabWavesPerSimd<3>);
  return 4 * per_simd;
}

bool staged_decode_eligible(const Geometry& g, int num_q_heads) {
  return mfma_decode_eligible(g, num_q_heads) && (g.key_bits == 4 || g.key_bits == 3) &&
         g.num_kv_heads % 2 == 0;
}

bool page_decode_eligible(const Geometry& g, int num_q_heads, bool mse_keys_too) {
  const int H = g.num_kv_heads;
  // up to 8 query heads per kv head: the query hi and lo parts share one B
  // operand, and the P.V tile keeps the weights' lo parts in rows 8 .. 15
  const bool g_ok = num_q_heads <= 8 * H;
  // 3/4-bit keys: the per-head kernel is still the faster one (the page
  // kernel's centroid lookups are bound by LDS bank conflicts), unless asked
  const bool kind_ok = g.key_bits == 8 || mse_keys_too;
  // a workgroup takes up to 8 kv heads of a row
  return mfma_decode_eligible(g, num_q_heads) && g_ok && kind_ok && (H == 1 || H == 2 || H == 4 || H % 8 == 0);
}

template <int WAVES>
void launch_ring(const Geometry& g, dim3 grid, const MfmaArgs& a, hipStream_t stream) {
  const dim3 block(64 * WAVES);
  if (g.soa) {
    if (g.key_bits == 4)
      hipLaunchKernelGGL((decode_ring_kernel<4, 134, true, WAVES>), grid, block, 0, stream, a);
    else if (g.slot == 118)
      hipLaunchKernelGGL((decode_ring_kernel<3, 118, true, WAVES>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_ring_kernel<3, 102, true, WAVES>), grid, block, 0, stream, a);
  } else if (g.key_bits == 4)
    hipLaunchKernelGGL((decode_ring_kernel<4, 134, false, WAVES>), grid, block, 0, stream, a);
  else if (g.slot == 118)
    hipLaunchKernelGGL((decode_ring_kernel<3, 118, false, WAVES>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_ring_kernel<3, 102, false, WAVES>), grid, block, 0, stream, a);
}

// 3/4-bit keys with up to 8 query heads per kv head on the slotted page (more
// take the per-head kernels' 16), any count on the split page (passes of 8)
bool ring_decode_eligible(const Geometry& g, int num_q_heads) {
  const int G = num_q_heads / g.num_kv_heads;
  return g.head_dim == kD && g.block_size % 16 == 0 && G >= 1 && (G <= 8 || g.soa) &&
         ((g.key_bits == 4 && g.slot == 134) || (g.key_bits == 3 && (g.slot == 118 || g.slot == 102)));
}

// query heads per kv head one pass of a matrix-core kernel takes: the ring
// and page kernels hold a head's query hi and lo parts in one 16-column
// operand (8), the per-head kernels 16
int mfma_max_g(int mfma) { return mfma == 2 || mfma == 4 ? 8 : 16; }

int ring_max_slabs() { return kRingMaxSlabs; }

int page_wgs_per_cu(const Geometry& g, int group) {
  const int H = group;
  int lds = 0;
#define TQ_PAGE_LDS(KB_, SLOT_)                                                   \
  if (g.key_bits == KB_ && g.slot == SLOT_) {                                     \
    lds = H == 1 ? PageGeom<KB_, SLOT_, 1>::kLds : H == 2 ? PageGeom<KB_, SLOT_, 2>::kLds \
        : H == 4 ? PageGeom<KB_, SLOT_, 4>::kLds : PageGeom<KB_, SLOT_, 8>::kLds;  \
  }
  TQ_PAGE_LDS(8, 196) TQ_PAGE_LDS(4, 134) TQ_PAGE_LDS(3, 118) TQ_PAGE_LDS(3, 102)
#undef TQ_PAGE_LDS
  int n = lds > 0 ? (160 * 1024) / lds : 1;
  const int by_regs = 4 * page_waves_per_simd(g.key_bits) / H;
  if (n > by_regs) n = by_regs;
  return n < 1 ? 1 : n;
}

bool mfma_decode_eligible(const Geometry& g, int num_q_heads) {
  // slotted pages (the split page has the ring kernel, ring_decode_eligible)
  if (g.soa) return false;
  const int G = num_q_heads / g.num_kv_heads;
  if (g.head_dim != kD || g.block_size % 16 != 0 || G < 1) return false;   // G > 16: passes of 16
  if (g.key_bits == 8) return g.slot == 196;
  return (g.key_bits == 4 || g.key_bits == 3) && (g.slot == 134 || g.slot == 118 || g.slot == 102);
}

// slotted pages at head dims 64 and 256 (more than 16 query heads per kv
// head in passes of 16), the presets' key / value bit pairs, and the slot
// size the kernel's layout assumes
bool dslab_decode_eligible(const Geometry& g, int num_q_heads) {
  if (g.soa || (g.head_dim != 64 && g.head_dim != 256) || g.block_size % 16 != 0) return false;
  const int G = num_q_heads / g.num_kv_heads;
  if (G < 1) return false;
  const int kb = g.key_bits, vb = g.value_bits, D = g.head_dim;
  if (!((vb == 4 && (kb == 4 || kb == 3 || kb == 8)) || (kb == 3 && vb == 3))) return false;
  const int s = (kb == 8 ? D : D * kb / 8 + 2) + D * vb / 8 + 4;
  return g.slot == s + s % 2;
}

int dslab_waves_per_cu(const Geometry& g) {
  return 4 * (g.head_dim == 256 ? kDWavesPerSimd<256> : kDWavesPerSimd<64>);
}

size_t dslab_partial_bytes(const Geometry& g, int batch, int num_q_heads, int num_splits) {
  return static_cast<size_t>(batch) * num_q_heads * num_splits * (g.head_dim + 4) * sizeof(float);
}

size_t mfma_partial_bytes(int batch, int num_q_heads, int num_splits) {
  return static_cast<size_t>(batch) * num_q_heads * num_splits * kRec * sizeof(float);
}

hipError_t launch_decode_mfma(const Geometry& g, const DevTables* tables, DevErrors* errs,
                              const DecodePlan& plan,
                              const uint16_t* q, const uint8_t* cache, int64_t num_blocks,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int32_t* seq_lens, int batch, int num_q_heads, float sm_scale,
                              void* out, int out_is_fp32, void* workspace, hipStream_t stream) {
  MfmaArgs a;
  a.tables = tables;
  a.errs = errs;
  a.q = q;
  a.cache = cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.Hq = num_q_heads;
  a.H = g.num_kv_heads;
  a.Gq = num_q_heads / g.num_kv_heads;
  a.bs_shift = __builtin_ctz(static_cast<unsigned>(g.block_size));
  a.chunk = plan.chunk;
  a.num_splits = plan.num_splits;
  a.batch = batch;
  a.scale_log2 = sm_scale * kLog2e;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.out_fp32 = out_is_fp32;
  a.dynamic = plan.dynamic;
  a.q_rot = nullptr;
  a.order = nullptr;
  if (plan.mfma == 5) {
    // head dims 64 and 256: the direct kernel in passes of 16 query heads,
    // the merge
    float* q_rot = plan.qrot ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.qrot_off) : nullptr;
    if (g.key_bits != 8 && g.haar && q_rot == nullptr) return hipErrorInvalidValue;
    return g.head_dim == 64 ? launch_dslab_d<64>(g, plan, a, batch, q_rot, stream)
                            : launch_dslab_d<256>(g, plan, a, batch, q_rot, stream);
  }
  if (plan.order) {
    a.h0 = 0;
    a.G = a.Gq;
    int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.order_off);
    hipLaunchKernelGGL(order_sequences_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, a, order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.order = order;
  }
  float* q_rot = plan.qrot ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.qrot_off) : nullptr;
  // query heads in passes of at most plan.g_pass per kv head (each pass
  // reads the cache again); every pass writes its heads' outputs or split
  // records, and one merge at the end combines the records of all heads
  const int g_pass = plan.g_pass > 0 ? plan.g_pass : a.Gq;
  for (int h0 = 0; h0 < a.Gq; h0 += g_pass) {
    a.h0 = h0;
    a.G = a.Gq - h0 < g_pass ? a.Gq - h0 : g_pass;
    if (q_rot != nullptr) {
      a.q_rot = nullptr;
      hipLaunchKernelGGL(rotate_queries_haar_kernel, dim3(batch * g.num_kv_heads), dim3(kD), 0, stream, a, q_rot);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      a.q_rot = q_rot;
    }
    if (plan.mfma == 4) {
      // one workgroup per (sequence, kv head, workgroup split)
      const int n_items = plan.order ? 8 * ((batch + 7) / 8) * plan.num_splits * g.num_kv_heads
                                     : plan.num_splits * batch * g.num_kv_heads;
      const dim3 grid(8 * ((n_items + 7) / 8));
      if (plan.ring_waves == 8)
        launch_ring<8>(g, grid, a, stream);
      else
        launch_ring<kRingWaves>(g, grid, a, stream);
    } else if (plan.mfma == 2) {
      hipError_t e = g.key_bits == 8 ? launch_page_h<8, 196>(a, batch, plan.group, stream)
                   : g.key_bits == 4 ? launch_page_h<4, 134>(a, batch, plan.group, stream)
                   : g.slot == 118   ? launch_page_h<3, 118>(a, batch, plan.group, stream)
                                     : launch_page_h<3, 102>(a, batch, plan.group, stream);
      if (e != hipSuccess) return e;
    } else {
      // one wavefront per workgroup: (split, sequence, kv head)
      const int n_items = plan.num_splits * batch * g.num_kv_heads;
      const dim3 grid(8 * ((n_items + 7) / 8));
      if (plan.mfma == 3) {
        if (g.key_bits == 4)
          hipLaunchKernelGGL((decode_staged_kernel<4, 134>), grid, dim3(64), 0, stream, a);
        else if (g.slot == 118)
          hipLaunchKernelGGL((decode_staged_kernel<3, 118>), grid, dim3(64), 0, stream, a);
        else
          hipLaunchKernelGGL((decode_staged_kernel<3, 102>), grid, dim3(64), 0, stream, a);
      } else if (g.key_bits == 8)
        hipLaunchKernelGGL((decode_slab_kernel<8, 196>), grid, dim3(64), 0, stream, a);
      else if (g.key_bits == 4)
        hipLaunchKernelGGL((decode_slab_kernel<4, 134>), grid, dim3(64), 0, stream, a);
      else if (g.slot == 118)
        hipLaunchKernelGGL((decode_slab_kernel<3, 118>), grid, dim3(64), 0, stream, a);
      else
        hipLaunchKernelGGL((decode_slab_kernel<3, 102>), grid, dim3(64), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // merge: one workgroup per (sequence, query head); the ring kernel writes
  // the output itself when a sequence has one workgroup split
  if (plan.mfma == 4 && plan.num_splits == 1) return hipSuccess;
  a.h0 = 0;
  a.G = a.Gq;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(batch * num_q_heads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq
