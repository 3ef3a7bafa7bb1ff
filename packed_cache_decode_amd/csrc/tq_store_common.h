// Definitions shared by the store translation units: the store arguments,
// binary16 / E4M3 conversions and the four-lanes-per-vector store kernel
// (store_quad_kernel).  tq_store.hip instantiates it at head dim 128,
// tq_store_quad.hip at 64 and 256: kept in separate modules, so that the
// instantiations at one head dim do not change the code generated for the
// others.  What the kernels compute follows P1 (the slot layout and store
// sections) step for step in fp32, as stated at the top of tq_store.hip.
#pragma once

#include "tq_internal.h"

#pragma clang fp contract(off)

namespace tq {

struct StoreArgs {
  const DevTables* tables;
  DevErrors* errs;
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;            // elements between tokens
  const int64_t* slot_mapping;
  int64_t num_tokens;
  uint8_t* cache;
  int64_t num_slots;         // num_blocks * block_size
  float r_d;
  int H;
  int bs_shift;              // log2(block_size)
  int soa;                   // split page (data region + meta region), folded K norm
};

namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// binary32 -> binary16, round to nearest even (v_cvt_f16_f32 in the default mode)
// binary32 -> binary16, round to nearest even, of x as a binary32 value: the
// empty asm makes x a finished binary32 result, so the compiler cannot fuse
// the conversion with the multiply that produced x into one rounding straight
// to binary16 (v_fma_mixlo_f16), which differs from the contract's two
// roundings when the binary32 product sits exactly halfway between two
// binary16 values
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  asm volatile("" : "+v"(x));
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// OCP E4M3FN from binary32, round to nearest even, |x| >= 448 (and inf)
// saturates to 448, NaN -> S.1111.111.  Written from the format definition:
// bias 7, subnormals m * 2^-9, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;          // 448.0f
  if (a < 0x3C800000u) {                              // below 2^-6: subnormal grid 2^-9
    const float q = rintf(__uint_as_float(a) * 512.0f);   // exact scaling, then RNE
    return sign | static_cast<uint32_t>(q);           // q == 8 is the first normal
  }
  const uint32_t e = (a >> 23) - 120u;                // 127 - 7
  uint32_t r = (e << 3) | ((a >> 20) & 7u);
  const uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  return sign | r;
}

// ---------------------------------------------------------------------------
// Four lanes per vector, d/4 contiguous coordinates per lane (32 at head_dim
// 128), 16 vectors per wavefront.  The fp32 contract of tq_store.hip's
// store_kernel, reorganised so that all but the last two butterfly stages and
// norm-tree levels stay inside a lane and those two are DPP quad exchanges;
// the code of a coordinate comes from the bucketize bins (one compare)
// instead of a compare per midpoint; codes, V nibbles and FP8 bytes are
// packed in registers and written as 2-byte stores (MSE slots are 2-byte
// aligned) or 4-byte stores (FP8 slots).
// ---------------------------------------------------------------------------

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

// value of the partner lane in the quad (lane ^ 1 or lane ^ 2)
template <int X>
__device__ __forceinline__ float quad_xor(float v) {
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;          // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, true));
}

// floor(t) as int32, NaN -> 0 (v_cvt_flr_i32_f32), clamped to [0, hi]
__device__ __forceinline__ int floor_clamp(float t, int hi) {
  int i;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(i) : "v"(t));
  int r;
  asm("v_med3_i32 %0, %1, 0, %2" : "=v"(r) : "v"(i), "v"(hi));
  return r;
}

// trunc(t) as int32 (t >= 0 here), clamped to [0, 15]
__device__ __forceinline__ uint32_t trunc_clamp15(float t) {
  int i;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(i) : "v"(t));
  int r;
  asm("v_med3_i32 %0, %1, 0, 15" : "=v"(r) : "v"(i));
  return static_cast<uint32_t>(r);
}

// trunc(t) as int32 (t >= 0 here), clamped to [0, 7]
__device__ __forceinline__ uint32_t trunc_clamp7(float t) {
  int i;
  asm("v_cvt_i32_f32 %0, %1" : "=v"(i) : "v"(t));
  int r;
  asm("v_med3_i32 %0, %1, 0, 7" : "=v"(r) : "v"(i));
  return static_cast<uint32_t>(r);
}

// butterfly across the quad: the lower lane of the pair keeps a + b, the
// upper lane a - b, computed as a + (-b) (the same IEEE operation)
template <int X>
__device__ __forceinline__ float butterfly_x(float u, uint32_t upper_sign) {
  const float o = quad_xor<X>(u);
  return o + __uint_as_float(__float_as_uint(u) ^ upper_sign);
}

// N dwords (a lane's 32 codes of N bits): one 16-byte store for N = 4 (16-byte
// aligned), dword stores for N = 3 (4-byte aligned)
template <int N>
__device__ __forceinline__ void store_words(uint8_t* dst, const uint32_t* w) {
  if constexpr (N == 4) {
    *reinterpret_cast<u32x4s*>(dst) = u32x4s{w[0], w[1], w[2], w[3]};
  } else {
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int i = 0; i < N; ++i) d[i] = w[i];
  }
}

__device__ __forceinline__ void store_u16s(uint8_t* dst, const uint32_t* w, int n16) {
  uint16_t* d = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
  for (int i = 0; i < n16; ++i) d[i] = static_cast<uint16_t>(w[i >> 1] >> (16 * (i & 1)));
}

// SOA: the page is a data region [bs][H][K codes | V codes] and a meta region
// [H][3][bs] of fp16 (K norm, V scale, V zero); the stored K norm is folded:
// |k| * (1 / sqrt(sum c_j^2 + 1e-16)) with the centroids c_j of the vector's
// codes, squared and summed in the same balanced tree as the norm (P1,
// section "SoA 的另一项收益:把 norm correction 折进写入端").
// kRows: H divides 16 and a cache row (H slots) is a multiple of 16 bytes, so
// a wavefront's 16 vectors are 16 / H whole tokens; their rows are assembled
// in LDS and written with 16-byte stores.  Otherwise each lane writes its
// fields with 2- or 4-byte stores.
// Head dim D, E = D / 4 coordinates per lane: log2(E) butterfly stages and
// norm-tree levels inside the lane, the last two across the quad (the split
// page only at D = 128).
template <int D, int KB, int VB, bool kRows, bool SOA>
__global__ void __launch_bounds__(256) store_quad_kernel(StoreArgs a) {
  constexpr int E = D / 4;
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128, 256");
  static_assert(!SOA || D == 128, "the split page at head dim 128");
  constexpr bool kFp8 = KB == 8;
  constexpr int kKeyCodeBytes = kFp8 ? D : (D * KB) / 8;
  constexpr int kKeyPacked = kFp8 ? D : kKeyCodeBytes + 2;
  constexpr int kValCodeBytes = (D * VB) / 8;
  constexpr int kVmax = (1 << VB) - 1;         // largest V code
  constexpr int kLaneVB = E * VB / 8;           // V code bytes of a lane's 32 coordinates
  constexpr int kSlot = kKeyPacked + kValCodeBytes + 4;    // 196 / 134 / 118, even
  static_assert(kSlot % 2 == 0, "slot must be even");
  static_assert(!(SOA && (kRows || kFp8)), "the split page: 3/4-bit keys, per-lane writes");
  constexpr int kDataBytes = kKeyCodeBytes + kValCodeBytes;   // SOA: data bytes per vector

  __shared__ uint32_t s_bins[kMaxBins][2];
  __shared__ float s_csq[16];                   // SOA: c_i * c_i per level
  __shared__ __align__(16) uint8_t s_rows[kRows ? 4 : 1][kRows ? 16 * kSlot : 16];
  if constexpr (!kFp8) {
    for (int i = threadIdx.x; i < kMaxBins; i += blockDim.x) {
      s_bins[i][0] = a.tables->bins[i][0];
      s_bins[i][1] = a.tables->bins[i][1];
    }
    if (SOA && threadIdx.x < 16) {
      const float c = a.tables->centroids[threadIdx.x];
      s_csq[threadIdx.x] = c * c;
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int qd = lane & 3;                    // quarter of the vector
  const int vsub = lane >> 2;                 // vector of the wavefront
  const uint32_t up1 = (qd & 1) ? 0x80000000u : 0u;
  const uint32_t up2 = (qd & 2) ? 0x80000000u : 0u;
  const int nbins = a.tables->bin_count;
  const float bscale = a.tables->bin_scale, bbias = a.tables->bin_bias;
  // sign flips of coordinates 32*qd + [0, 32) as per-dword masks on the bf16
  // pairs (bit 15: even coordinate, bit 31: odd)
  uint32_t smask[E / 2];
  if constexpr (E == 32) {
    const uint32_t sb = a.tables->sign_bits[qd];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      smask[i] = (((sb >> (2 * i)) & 1u) << 15) | (((sb >> (2 * i + 1)) & 1u) << 31);
  } else {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      const int j = E * qd + 2 * i;              // coordinates j and j + 1, one sign word
      const uint32_t sb = a.tables->sign_bits[j >> 5] >> (j & 31);
      smask[i] = ((sb & 1u) << 15) | (((sb >> 1) & 1u) << 31);
    }
  }

  const int H = a.H;
  const uint32_t total = static_cast<uint32_t>(a.num_tokens) * static_cast<uint32_t>(H);
  const uint32_t wave_id = blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint32_t stride = gridDim.x * 64;

  // 16 vectors' K, V and slot ids; a lane past the end of the batch fetches
  // the group's first vector (its results are dropped)
  struct Fetch {
    u32x4s k[E / 8], v[E / 8];
    int64_t slot;
    uint32_t n;
    int h;
  };
  auto fetch = [&](uint32_t b) {
    Fetch f;
    const uint32_t vec = b + vsub;
    const uint32_t vv = vec < total ? vec : (b < total ? b : 0u);   // a vector inside the batch
    f.n = vv / static_cast<uint32_t>(H);
    f.h = static_cast<int>(vv - f.n * static_cast<uint32_t>(H));
    f.slot = a.slot_mapping[f.n];
    const int64_t src = static_cast<int64_t>(f.n) * a.stride + static_cast<int64_t>(f.h) * D + E * qd;
    const u32x4s* kp = reinterpret_cast<const u32x4s*>(a.k + src);
    const u32x4s* vp = reinterpret_cast<const u32x4s*>(a.v + src);
#pragma unroll
    for (int i = 0; i < E / 8; ++i) f.k[i] = kp[i];
#pragma unroll
    for (int i = 0; i < E / 8; ++i) f.v[i] = vp[i];
    return f;
  };

  auto process = [&](const Fetch& f, uint32_t base) {
    const bool live = base + vsub < total;
    const uint32_t n = f.n;
    const int h = f.h;
    const int64_t slot = f.slot;
    const bool in_range = slot < a.num_slots;
    if (live && slot >= 0 && !in_range && qd == 0) a.errs->slot = 1;
    const bool do_store = live && slot >= 0 && in_range;
    (void)n;

    // ---------------- K ----------------
    uint32_t kw[E / 2];
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      kw[4 * i] = f.k[i][0];
      kw[4 * i + 1] = f.k[i][1];
      kw[4 * i + 2] = f.k[i][2];
      kw[4 * i + 3] = f.k[i][3];
    }
    uint32_t kout[kFp8 ? E / 4 : (E * KB + 31) / 32];
    uint32_t norm_bits = 0;
    if constexpr (kFp8) {
#pragma unroll
      for (int i = 0; i < E / 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t bw = kw[2 * i + (j >> 1)];
          const float x = (j & 1) ? __uint_as_float(bw & 0xFFFF0000u) : __uint_as_float(bw << 16);
          w |= f32_to_e4m3fn(x) << (8 * j);
        }
        kout[i] = w;
      }
    } else {
      // sign flips on the bf16 pairs (exact)
      float u[E];
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const uint32_t w = kw[i] ^ smask[i];
        u[2 * i] = __uint_as_float(w << 16);
        u[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
      // sum of squares (a flipped sign squares to the same value): the
      // balanced tree in index order, 5 levels in the lane
      float sq[E];
#pragma unroll
      for (int e = 0; e < E; ++e) sq[e] = u[e] * u[e];
#pragma unroll
      for (int w = 1; w < E; w *= 2)
#pragma unroll
        for (int e = 0; e < E; e += 2 * w) sq[e] = sq[e] + sq[e + w];
      float ss = sq[0];
      ss = ss + quad_xor<1>(ss);
      ss = ss + quad_xor<2>(ss);
      const float nrm = sqrtf(ss);
      const float alpha = (1.0f / (nrm + 1e-8f)) * a.r_d;
      norm_bits = f32_to_f16_bits(nrm);

      // butterflies h = 1 .. 64
#pragma unroll
      for (int hs = 1; hs < E; hs *= 2)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((e & hs) == 0) {
            const float p = u[e], q = u[e + hs];
            u[e] = p + q;
            u[e + hs] = p - q;
          }
#pragma unroll
      for (int e = 0; e < E; ++e) u[e] = butterfly_x<1>(u[e], up1);
#pragma unroll
      for (int e = 0; e < E; ++e) u[e] = butterfly_x<2>(u[e], up2);
      // codes: y = u * alpha, code = base + (y >= thr) of y's bin
      uint32_t code[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float y = u[e] * alpha;
        const int bi = floor_clamp(__builtin_fmaf(y, bscale, bbias), nbins - 1);
        const uint32_t thr = s_bins[bi][0], cb = s_bins[bi][1];
        code[e] = cb + (y >= __uint_as_float(thr) ? 1u : 0u);
      }
      if constexpr (SOA) {
        // folded norm: the same tree over the squared centroids
        float cq[E];
#pragma unroll
        for (int e = 0; e < E; ++e) cq[e] = s_csq[code[e]];
#pragma unroll
        for (int w = 1; w < E; w *= 2)
#pragma unroll
          for (int e = 0; e < E; e += 2 * w) cq[e] = cq[e] + cq[e + w];
        float css = cq[0];
        css = css + quad_xor<1>(css);
        css = css + quad_xor<2>(css);
        const float inv = 1.0f / sqrtf(css + 1e-16f);
        norm_bits = f32_to_f16_bits(nrm * inv);
      }
      if constexpr (KB == 4) {
#pragma unroll
        for (int i = 0; i < E / 8; ++i) {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) w |= code[8 * i + j] << (4 * j);
          kout[i] = w;
        }
      } else if constexpr (E != 32) {
        // LSB-first stream: code e at bits [3e, 3e + 3)
#pragma unroll
        for (int i = 0; i < (3 * E + 31) / 32; ++i) kout[i] = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int b = 3 * e;
          kout[b >> 5] |= code[e] << (b & 31);
          if ((b & 31) > 29) kout[(b >> 5) + 1] |= code[e] >> (32 - (b & 31));
        }
      } else {
        // 96-bit LSB-first stream: code e at bits [3e, 3e + 3)
        uint64_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int b = 3 * e;
          if (b + 3 <= 64) lo |= static_cast<uint64_t>(code[e]) << b;
          else if (b >= 64) hi |= static_cast<uint64_t>(code[e]) << (b - 64);
          else {
            lo |= static_cast<uint64_t>(code[e]) << b;
            hi |= static_cast<uint64_t>(code[e]) >> (64 - b);
          }
        }
        kout[0] = static_cast<uint32_t>(lo);
        kout[1] = static_cast<uint32_t>(lo >> 32);
        kout[2] = static_cast<uint32_t>(hi);
      }
    }

    // ---------------- V ----------------
    float vv_[E];
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const u32x4s t = f.v[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vv_[8 * i + 2 * j] = __uint_as_float(t[j] << 16);
        vv_[8 * i + 2 * j + 1] = __uint_as_float(t[j] & 0xFFFF0000u);
      }
    }
    float lo = vv_[0], hi = vv_[0];
#pragma unroll
    for (int e = 1; e < E; ++e) {
      lo = fminf(lo, vv_[e]);
      hi = fmaxf(hi, vv_[e]);
    }
    lo = fminf(lo, quad_xor<1>(lo));
    hi = fmaxf(hi, quad_xor<1>(hi));
    lo = fminf(lo, quad_xor<2>(lo));
    hi = fmaxf(hi, quad_xor<2>(hi));
    float sc = (hi - lo) / static_cast<float>(kVmax);
    if (!(sc > 1e-8f)) sc = 1e-8f;
    const float isc = 1.0f / sc;
    uint32_t vout[(E * VB + 31) / 32];
    if constexpr (VB == 4) {
#pragma unroll
      for (int i = 0; i < E / 8; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          w |= trunc_clamp15((vv_[8 * i + j] - lo) * isc + 0.5f) << (4 * j);
        }
        vout[i] = w;
      }
    } else if constexpr (E != 32) {
      // LSB-first stream: code e at bits [3e, 3e + 3)
#pragma unroll
      for (int i = 0; i < (3 * E + 31) / 32; ++i) vout[i] = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t c = trunc_clamp7((vv_[e] - lo) * isc + 0.5f);
        const int b = 3 * e;
        vout[b >> 5] |= c << (b & 31);
        if ((b & 31) > 29) vout[(b >> 5) + 1] |= c >> (32 - (b & 31));
      }
    } else {
      // 96-bit LSB-first stream: code e at bits [3e, 3e + 3)
      uint64_t vlo = 0, vhi = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t c = trunc_clamp7((vv_[e] - lo) * isc + 0.5f);
        const int b = 3 * e;
        if (b + 3 <= 64) vlo |= static_cast<uint64_t>(c) << b;
        else if (b >= 64) vhi |= static_cast<uint64_t>(c) << (b - 64);
        else {
          vlo |= static_cast<uint64_t>(c) << b;
          vhi |= static_cast<uint64_t>(c) >> (64 - b);
        }
      }
      vout[0] = static_cast<uint32_t>(vlo);
      vout[1] = static_cast<uint32_t>(vlo >> 32);
      vout[2] = static_cast<uint32_t>(vhi);
    }

    // ---------------- slot ----------------
    if constexpr (kRows) {
      // the 16 vectors' slots, back to back, are 16 / H whole cache rows
      uint8_t* rows = s_rows[threadIdx.x >> 6];
      uint8_t* sp = rows + vsub * kSlot;
      if constexpr (kFp8) {
        uint32_t* d32 = reinterpret_cast<uint32_t*>(sp);        // FP8 slots: 4-byte aligned
#pragma unroll
        for (int i = 0; i < E / 4; ++i) d32[(E / 4) * qd + i] = kout[i];
#pragma unroll
        for (int i = 0; i < E / 8; ++i) d32[(kKeyPacked >> 2) + (E / 8) * qd + i] = vout[i];
      } else {
        store_u16s(sp + (kKeyCodeBytes / 4) * qd, kout, kKeyCodeBytes / 8);
        if (qd == 0) *reinterpret_cast<uint16_t*>(sp + kKeyCodeBytes) = static_cast<uint16_t>(norm_bits);
        store_u16s(sp + kKeyPacked + kLaneVB * qd, vout, kLaneVB / 2);
      }
      if (qd == 3) {
        uint16_t* m = reinterpret_cast<uint16_t*>(sp + kKeyPacked + kValCodeBytes);
        m[0] = f32_to_f16_bits(sc);
        m[1] = f32_to_f16_bits(lo);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      const int row_chunks = H * kSlot / 16;
      const uint32_t tok0 = base / static_cast<uint32_t>(H);
      // a token's slot sits in the lanes of its vectors (lane 4 * H * tt for
      // token tok0 + tt): taken from there, no reload from memory
      const uint32_t slot_lo = static_cast<uint32_t>(slot);
      const uint32_t slot_hi = static_cast<uint32_t>(static_cast<uint64_t>(slot) >> 32);
#pragma unroll
      for (int r = 0; r < (kSlot + 63) / 64; ++r) {   // kSlot chunks of 16 bytes
        const int c = lane + 64 * r;
        const int tt = (c < kSlot ? c : 0) / row_chunks;
        const int src_lane = 4 * H * tt;
        const uint32_t lo = __builtin_amdgcn_ds_bpermute(src_lane << 2, static_cast<int>(slot_lo));
        const uint32_t hi = __builtin_amdgcn_ds_bpermute(src_lane << 2, static_cast<int>(slot_hi));
        const int64_t ts = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
        const uint32_t tok = tok0 + tt;
        if (c < kSlot && tok < static_cast<uint32_t>(a.num_tokens)) {
          if (ts >= 0 && ts < a.num_slots) {
            const u32x4s d = *reinterpret_cast<const u32x4s*>(rows + 16 * c);
            *reinterpret_cast<u32x4s*>(a.cache + ts * (static_cast<int64_t>(H) * kSlot) +
                                       16 * (c - tt * row_chunks)) = d;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    } else if (SOA && do_store) {
      // split page: the vector's data bytes (16-byte aligned: pages and data
      // rows are multiples of 16 bytes) and its three meta fields
      const int64_t page = slot >> a.bs_shift;
      const int64_t row = slot - (page << a.bs_shift);
      uint8_t* pg = a.cache + page * ((static_cast<int64_t>(H) * kSlot) << a.bs_shift);
      uint8_t* dst = pg + (row * H + h) * kDataBytes;
      store_words<KB>(dst + (kKeyCodeBytes / 4) * qd, kout);
      store_words<VB>(dst + kKeyCodeBytes + kLaneVB * qd, vout);
      uint16_t* meta = reinterpret_cast<uint16_t*>(pg + ((static_cast<int64_t>(H) * kDataBytes) << a.bs_shift)) +
                       ((static_cast<int64_t>(h) * 3) << a.bs_shift) + row;
      if (qd == 0) meta[0] = static_cast<uint16_t>(norm_bits);
      if (qd == 3) {
        meta[1 << a.bs_shift] = f32_to_f16_bits(sc);
        meta[2 << a.bs_shift] = f32_to_f16_bits(lo);
      }
    } else if (do_store) {
      const int64_t page = slot >> a.bs_shift;
      const int64_t row = slot - (page << a.bs_shift);
      uint8_t* dst = a.cache + ((page << a.bs_shift) + row) * (static_cast<int64_t>(H) * kSlot) +
                     static_cast<int64_t>(h) * kSlot;
      if constexpr (kFp8) {
        uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);      // FP8 slots: 4-byte aligned
#pragma unroll
        for (int i = 0; i < E / 4; ++i) d32[(E / 4) * qd + i] = kout[i];
#pragma unroll
        for (int i = 0; i < E / 8; ++i) d32[(kKeyPacked >> 2) + (E / 8) * qd + i] = vout[i];
      } else {
        store_u16s(dst + (kKeyCodeBytes / 4) * qd, kout, kKeyCodeBytes / 8);
        if (qd == 0) *reinterpret_cast<uint16_t*>(dst + kKeyCodeBytes) = static_cast<uint16_t>(norm_bits);
        store_u16s(dst + kKeyPacked + kLaneVB * qd, vout, kLaneVB / 2);
      }
      if (qd == 3) {
        uint16_t* m = reinterpret_cast<uint16_t*>(dst + kKeyPacked + kValCodeBytes);
        m[0] = f32_to_f16_bits(sc);
        m[1] = f32_to_f16_bits(lo);
      }
    }
  };

  for (uint32_t base = wave_id * 16; base < total; base += stride) process(fetch(base), base);
}

}  // namespace

// head dims 64 and 256, slotted page, Hadamard rotation (tq_store_quad.hip)
hipError_t launch_store_quad_64_256(const Geometry& g, const StoreArgs& a, hipStream_t stream);

}  // namespace tq
