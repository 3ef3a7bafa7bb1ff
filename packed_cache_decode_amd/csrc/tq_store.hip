// tq_store kernel: quantise one (token, kv head) K/V pair per wavefront and
// write its slot into the paged cache.
//
// What is computed follows P1 ("vLLM 源码完全拆解(十九):TurboQuant KV Cache
// 量化"), sections "K 的归一化与旋转为什么放在 kernel 外面" (normalise, rotate),
// "二分查找" (bucketize, ">=" sends a boundary value right), "位打包" (LSB-first
// codes), "向量范数的存储" (fp16 norm after the codes), "V 的 min/max 均匀量化"
// and "FP8 K 路径".  The rotation is the seeded-sign Walsh-Hadamard transform
// done in registers as butterflies instead of the page's dense GEMM.
//
// Bit-exactness: every float operation below is a single binary32 operation
// rounded to nearest even.  Contraction into fused multiply-add is disabled
// for this file, division and sqrtf compile to their correctly rounded
// sequences, the norm is a fixed pairwise tree and the butterflies run with
// stride h = 1, 2, 4, ..., d/2.  The same result therefore comes out of any
// implementation that follows these steps, and the bytes are comparable bit
// for bit.
//
// Kernels.  store_quad_kernel (tq_store_common.h; head_dim 128 with the
// Hadamard rotation, every preset and both page layouts, and head dims 64
// and 256 on the slotted page from tq_store_quad.hip) gives each vector four
// lanes of d/4 contiguous coordinates, 16 vectors per wavefront; its section
// has the details.  store_kernel serves the rest (the split page at head
// dims 64 and 256, the Haar rotation, codebooks without bucketize bins,
// batches past 32-bit indexing): one wavefront (64 lanes) per
// vector pair, lane l holding the E = d/64 contiguous elements [E*l, E*l +
// E), butterflies with stride below E inside the lane and larger strides
// pairing lane l with lane l ^ (h / E); its slot is assembled in LDS and
// written with 2-byte stores (slots are 2-byte aligned).
#include "tq_store_common.h"

#pragma clang fp contract(off)

namespace tq {
namespace {

constexpr int kWaves = 4;

// sum over i of q[i] * x[i] as the balanced tree in index order (products
// and sums single fp32 operations): a stack of pending partial sums, where
// element i closes the levels at which its index has a set bit
template <int D>
__device__ __forceinline__ float tree_dot(const float* q, const float* x) {
  constexpr int L = __builtin_ctz(D);
  float stk[L];
  float total = 0.0f;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    float v = q[i] * x[i];
    bool placed = false;
#pragma unroll
    for (int l = 0; l < L; ++l) {
      if (!placed) {
        if ((i >> l) & 1) {
          v = stk[l] + v;
        } else {
          stk[l] = v;
          placed = true;
        }
      }
    }
    if (!placed) total = v;
  }
  return total;
}

template <int D, int KB, int VB>
__global__ void __launch_bounds__(64 * kWaves) store_kernel(StoreArgs a) {
  constexpr int E = D / 64;
  constexpr bool kFp8 = KB == 8;
  constexpr int kLevels = kFp8 ? 0 : (1 << KB);
  constexpr int kKeyCodeBytes = kFp8 ? D : (D * KB + 7) / 8;
  constexpr int kKeyPacked = kFp8 ? D : kKeyCodeBytes + 2;
  constexpr int kValCodeBytes = (D * VB + 7) / 8;
  constexpr int kVmax = (1 << VB) - 1;         // largest V code
  constexpr int kSlotRaw = kKeyPacked + kValCodeBytes + 4;
  constexpr int kSlot = kSlotRaw + (kSlotRaw & 1);

  __shared__ uint8_t s_code[kWaves][D];
  __shared__ __align__(4) uint8_t s_slot[kWaves][kSlot + 2];
  __shared__ float s_csq[16];                  // split page: c_i * c_i per level
  __shared__ float s_x[kWaves][D];             // Haar rotation: the vector, for every lane

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int H = a.H;
  if (!kFp8 && threadIdx.x < 16) {
    const float c = a.tables->centroids[threadIdx.x];
    s_csq[threadIdx.x] = c * c;
  }
  __syncthreads();

  float mid[kLevels > 0 ? kLevels - 1 : 1];
#pragma unroll
  for (int m = 0; m < kLevels - 1; ++m) mid[m] = a.tables->midpoints[m];
  uint32_t sgn[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = E * lane + e;
    sgn[e] = ((a.tables->sign_bits[j >> 5] >> (j & 31)) & 1u) << 31;
  }

  const int64_t total = a.num_tokens * H;
  for (int64_t vec = static_cast<int64_t>(blockIdx.x) * kWaves + wave; vec < total;
       vec += static_cast<int64_t>(gridDim.x) * kWaves) {
    const int64_t n = vec / H;
    const int h = static_cast<int>(vec - n * H);
    const int64_t slot = a.slot_mapping[n];
    if (slot < 0) continue;                       // padding token
    if (slot >= a.num_slots) {
      if (lane == 0) a.errs->slot = 1;
      continue;
    }
    const int64_t page = slot >> a.bs_shift;
    const int64_t row = slot - (page << a.bs_shift);
    uint8_t* dst = a.cache + ((page << a.bs_shift) + row) * (static_cast<int64_t>(H) * kSlot) +
                   static_cast<int64_t>(h) * kSlot;
    const int64_t src = n * a.stride + static_cast<int64_t>(h) * D + E * lane;

    // ---------------- K ----------------
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = bf16_bits_to_f32(a.k[src + e]);

    if constexpr (kFp8) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_slot[wave][E * lane + e] = static_cast<uint8_t>(f32_to_e4m3fn(x[e]));
    } else {
      // sum of squares: in-lane levels, then across lanes (a balanced tree
      // in index order; x*x of a bf16 value is exact)
      float sq[E];
#pragma unroll
      for (int e = 0; e < E; ++e) sq[e] = x[e] * x[e];
#pragma unroll
      for (int w = 1; w < E; w *= 2)
#pragma unroll
        for (int e = 0; e < E; e += 2 * w) sq[e] = sq[e] + sq[e + w];
      float ss = sq[0];
#pragma unroll
      for (int m = 1; m < 64; m *= 2) ss = ss + __shfl_xor(ss, m, 64);
      const float nrm = sqrtf(ss);
      float alpha = (1.0f / (nrm + 1e-8f)) * a.r_d;

      float u[E];
      if (a.tables->rot != nullptr) {
        // Haar rotation: u_j = tree over i of Q[j][i] * x_i; y = u / (|x| + 1e-8)
#pragma unroll
        for (int e = 0; e < E; ++e) s_x[wave][E * lane + e] = x[e];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int e = 0; e < E; ++e) u[e] = tree_dot<D>(a.tables->rot + static_cast<int64_t>(E * lane + e) * D, s_x[wave]);
        alpha = 1.0f / (nrm + 1e-8f);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      } else {
      // sign flips (exact), then butterflies h = 1, 2, ..., D/2
#pragma unroll
      for (int e = 0; e < E; ++e) u[e] = __uint_as_float(__float_as_uint(x[e]) ^ sgn[e]);
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
      for (int lm = 1; lm < 64; lm *= 2) {
        const bool upper = (lane & lm) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float o = __shfl_xor(u[e], lm, 64);
          u[e] = upper ? (o - u[e]) : (u[e] + o);
        }
      }
      }
      // y = u * alpha, code = #{m : y >= mid_m}
      float cq[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float y = u[e] * alpha;
        int c = 0;
#pragma unroll
        for (int m = 0; m < kLevels - 1; ++m) c += (y >= mid[m]) ? 1 : 0;
        s_code[wave][E * lane + e] = static_cast<uint8_t>(c);
        cq[e] = s_csq[c];
      }
      // split page: the stored norm is |k| / |c|, |c|^2 summed in the same
      // tree as |k|^2
      float n_stored = nrm;
      if (a.soa) {
#pragma unroll
        for (int w = 1; w < E; w *= 2)
#pragma unroll
          for (int e = 0; e < E; e += 2 * w) cq[e] = cq[e] + cq[e + w];
        float css = cq[0];
#pragma unroll
        for (int m = 1; m < 64; m *= 2) css = css + __shfl_xor(css, m, 64);
        n_stored = nrm * (1.0f / sqrtf(css + 1e-16f));
      }
      if (lane == 0) {
        const uint16_t nb = f32_to_f16_bits(n_stored);
        s_slot[wave][kKeyCodeBytes] = static_cast<uint8_t>(nb & 0xFF);
        s_slot[wave][kKeyCodeBytes + 1] = static_cast<uint8_t>(nb >> 8);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      // LSB-first bit stream: byte j holds stream bits [8j, 8j + 8)
      for (int j = lane; j < kKeyCodeBytes; j += 64) {
        uint32_t byte = 0;
        if constexpr (KB == 4) {
          byte = s_code[wave][2 * j] | (s_code[wave][2 * j + 1] << 4);
        } else {
#pragma unroll
          for (int bit = 0; bit < 8; ++bit) {
            const int p = 8 * j + bit;
            byte |= ((s_code[wave][p / KB] >> (p % KB)) & 1u) << bit;
          }
        }
        s_slot[wave][j] = static_cast<uint8_t>(byte);
      }
    }

    // ---------------- V ----------------
    float vv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) vv[e] = bf16_bits_to_f32(a.v[src + e]);
    float lo = vv[0], hi = vv[0];
#pragma unroll
    for (int e = 1; e < E; ++e) {
      lo = fminf(lo, vv[e]);
      hi = fmaxf(hi, vv[e]);
    }
#pragma unroll
    for (int m = 1; m < 64; m *= 2) {
      lo = fminf(lo, __shfl_xor(lo, m, 64));
      hi = fmaxf(hi, __shfl_xor(hi, m, 64));
    }
    float sc = (hi - lo) / static_cast<float>(kVmax);
    if (!(sc > 1e-8f)) sc = 1e-8f;
    const float isc = 1.0f / sc;
    uint32_t q[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float t = (vv[e] - lo) * isc + 0.5f;
      int qi = static_cast<int>(truncf(t));
      qi = qi < 0 ? 0 : (qi > kVmax ? kVmax : qi);
      q[e] = static_cast<uint32_t>(qi);
    }
    if constexpr (VB == 4) {
      if constexpr (E == 1) {
        const uint32_t other = __shfl_xor(q[0], 1, 64);
        if ((lane & 1) == 0) s_slot[wave][kKeyPacked + (lane >> 1)] = static_cast<uint8_t>(q[0] | (other << 4));
      } else {
#pragma unroll
        for (int e = 0; e < E; e += 2)
          s_slot[wave][kKeyPacked + (E * lane + e) / 2] = static_cast<uint8_t>(q[e] | (q[e + 1] << 4));
      }
    } else {
      // 3-bit codes: LSB-first stream, byte j holds stream bits [8j, 8j + 8)
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
      for (int e = 0; e < E; ++e) s_code[wave][E * lane + e] = static_cast<uint8_t>(q[e]);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      for (int j = lane; j < kValCodeBytes; j += 64) {
        uint32_t byte = 0;
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
          const int p = 8 * j + bit;
          byte |= ((s_code[wave][p / VB] >> (p % VB)) & 1u) << bit;
        }
        s_slot[wave][kKeyPacked + j] = static_cast<uint8_t>(byte);
      }
    }
    if (lane == 0) {
      const uint16_t sb = f32_to_f16_bits(sc);
      const uint16_t zb = f32_to_f16_bits(lo);
      uint8_t* m = &s_slot[wave][kKeyPacked + kValCodeBytes];
      m[0] = static_cast<uint8_t>(sb & 0xFF);
      m[1] = static_cast<uint8_t>(sb >> 8);
      m[2] = static_cast<uint8_t>(zb & 0xFF);
      m[3] = static_cast<uint8_t>(zb >> 8);
      if (kSlot != kSlotRaw) m[4] = 0;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

    if (!kFp8 && a.soa) {
      // split page: K codes then V codes into the data region, the norm,
      // scale and zero into the meta region (every part has an even size)
      constexpr int kDataBytes = kKeyCodeBytes + kValCodeBytes;
      uint8_t* pg = a.cache + page * ((static_cast<int64_t>(H) * kSlot) << a.bs_shift);
      uint16_t* d16 = reinterpret_cast<uint16_t*>(pg + (row * H + h) * kDataBytes);
      for (int j = lane; j < kDataBytes / 2; j += 64) {
        const int src = 2 * j < kKeyCodeBytes ? 2 * j : kKeyPacked + 2 * j - kKeyCodeBytes;
        d16[j] = static_cast<uint16_t>(s_slot[wave][src] | (s_slot[wave][src + 1] << 8));
      }
      if (lane < 3) {
        uint16_t* meta = reinterpret_cast<uint16_t*>(pg + ((static_cast<int64_t>(H) * kDataBytes) << a.bs_shift)) +
                         ((static_cast<int64_t>(h) * 3 + lane) << a.bs_shift) + row;
        const int src = lane == 0 ? kKeyCodeBytes : kKeyPacked + kValCodeBytes + 2 * (lane - 1);
        *meta = static_cast<uint16_t>(s_slot[wave][src] | (s_slot[wave][src + 1] << 8));
      }
    } else {
      // write the assembled slot: kSlot / 2 two-byte stores
      uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
      for (int j = lane; j < kSlot / 2; j += 64)
        d16[j] = static_cast<uint16_t>(s_slot[wave][2 * j] | (s_slot[wave][2 * j + 1] << 8));
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
}

template <int KB, int VB>
hipError_t launch_store128(const StoreArgs& a, hipStream_t stream) {
  constexpr int kSlot = KB == 8 ? 196 : (KB == 4 ? 134 : (VB == 4 ? 118 : 102));
  const int64_t total = a.num_tokens * a.H;
  int64_t blocks = (total + 63) / 64;               // 64 vectors per 256-thread block
  if (blocks > 8192) blocks = 8192;
  const bool rows = 16 % a.H == 0 && (static_cast<int64_t>(a.H) * kSlot) % 16 == 0;
  if constexpr (KB != 8) {
    if (a.soa) {
      hipLaunchKernelGGL((store_quad_kernel<128, KB, VB, false, true>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                         0, stream, a);
      return hipGetLastError();
    }
  }
  if (rows)
    hipLaunchKernelGGL((store_quad_kernel<128, KB, VB, true, false>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, stream, a);
  else
    hipLaunchKernelGGL((store_quad_kernel<128, KB, VB, false, false>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, stream, a);
  return hipGetLastError();
}

template <int D, int KB, int VB>
hipError_t launch_store_t(const StoreArgs& a, hipStream_t stream) {
  const int64_t total = a.num_tokens * a.H;
  int64_t blocks = (total + kWaves - 1) / kWaves;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((store_kernel<D, KB, VB>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_store(const Geometry& g, const DevTables* tables, DevErrors* errs, const uint16_t* k,
                        const uint16_t* v, int64_t kv_token_stride, const int64_t* slot_mapping,
                        int64_t num_tokens, uint8_t* cache, int64_t num_blocks, float r_d,
                        hipStream_t stream) {
  StoreArgs a;
  a.tables = tables;
  a.errs = errs;
  a.k = k;
  a.v = v;
  a.stride = kv_token_stride;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.cache = cache;
  a.num_slots = num_blocks * g.block_size;
  a.r_d = r_d;
  a.H = g.num_kv_heads;
  a.bs_shift = __builtin_ctz(static_cast<unsigned>(g.block_size));
  a.soa = g.soa;
  // head_dim 128 takes the four-lanes-per-vector kernel when the bucketize
  // bins exist (always, for the Lloyd-Max codebooks), the vector count fits
  // 32-bit indexing and the rotation is the Hadamard one
  if (g.head_dim == 128 && num_tokens * g.num_kv_heads < (int64_t{1} << 31) &&
      (g.key_bits == 8 || g.bins_ok) && !g.haar) {
    if (g.key_bits == 8) return launch_store128<8, 4>(a, stream);
    if (g.key_bits == 4) return launch_store128<4, 4>(a, stream);
    if (g.value_bits == 4) return launch_store128<3, 4>(a, stream);
    return launch_store128<3, 3>(a, stream);
  }
  // head dims 64 and 256 on the slotted page: the same kernel design
  // (tq_store_quad.hip)
  if ((g.head_dim == 64 || g.head_dim == 256) && !g.soa && num_tokens * g.num_kv_heads < (int64_t{1} << 31) &&
      (g.key_bits == 8 || g.bins_ok) && !g.haar)
    return launch_store_quad_64_256(g, a, stream);
#define TQ_STORE_CASE(D_, KB_, VB_) \
  if (g.head_dim == D_ && g.key_bits == KB_ && g.value_bits == VB_) return launch_store_t<D_, KB_, VB_>(a, stream);
  TQ_STORE_CASE(64, 3, 4) TQ_STORE_CASE(64, 4, 4) TQ_STORE_CASE(64, 8, 4) TQ_STORE_CASE(64, 3, 3)
  TQ_STORE_CASE(128, 3, 4) TQ_STORE_CASE(128, 4, 4) TQ_STORE_CASE(128, 8, 4) TQ_STORE_CASE(128, 3, 3)
  TQ_STORE_CASE(256, 3, 4) TQ_STORE_CASE(256, 4, 4) TQ_STORE_CASE(256, 8, 4) TQ_STORE_CASE(256, 3, 3)
#undef TQ_STORE_CASE
  return hipErrorInvalidValue;
}

}  // namespace tq
