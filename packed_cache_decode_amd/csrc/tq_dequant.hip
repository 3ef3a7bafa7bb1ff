// tq_dequant kernel: expand one sequence's packed slots back into K and V
// vectors of the original space.
//
// What is computed follows P1 ("vLLM 源码完全拆解(十九):TurboQuant KV Cache
// 量化"), section "反量化 kernel:_tq_full_dequant_kv": the unpacking is the
// decode's (section "读取内核"), without the softmax, and the keys are
// rotated back to the original space.  Here the inverse rotation is
// R^T = diag(s) H / sqrt(d) applied as butterflies in registers (R = H diag(s)
// / sqrt(d) is orthogonal and H symmetric), not a dense matrix product:
//   MSE keys:  k = n * R^T c, c the centroids of the codes, n the stored norm
//              divided by sqrt(sum c^2 + 1e-16) (norm correction; the split
//              page stores the corrected norm itself);
//   FP8 keys:  k = e4m3(byte), stored unrotated;
//   values:    v = code * scale16 + zero16.
//
// Mapping: one wavefront per (token, kv head); lane l holds the E = d/64
// contiguous coordinates [E*l, E*l + E).  Butterflies with stride below E stay
// in the lane, larger strides pair lane l with lane l ^ (h / E).
#include "tq_internal.h"

namespace tq {
namespace {

struct DequantArgs {
  const DevTables* tables;
  DevErrors* errs;
  const uint8_t* cache;
  int64_t num_blocks;
  const int32_t* block_table;   // the sequence's row
  int seq_len;
  int H;
  int bs_shift;
  int soa;
  void* k_out;                  // [seq_len][H][d]
  void* v_out;
  int out_fp32;
};

constexpr int kWaves = 4;

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// E4M3FN byte -> float, from the format definition (bias 7, subnormal m*2^-9)
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag;
  if (e == 0)
    mag = static_cast<float>(m) * (1.0f / 512.0f);
  else if (e == 15 && m == 7)
    mag = __uint_as_float(0x7FC00000u);
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// b-bit code j of an LSB-first stream (bits [j*b, j*b + b))
__device__ __forceinline__ uint32_t stream_code(const uint8_t* p, int j, int bits) {
  const int bit = j * bits;
  const uint32_t two = p[bit >> 3] | (static_cast<uint32_t>(p[(bit >> 3) + 1]) << 8);
  return (two >> (bit & 7)) & ((1u << bits) - 1u);
}

__device__ __forceinline__ void put(void* out, int64_t i, float x, int fp32) {
  if (fp32) {
    static_cast<float*>(out)[i] = x;
  } else {
    uint32_t u = __float_as_uint(x);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;         // round to nearest even
    static_cast<uint16_t*>(out)[i] = static_cast<uint16_t>(u);
  }
}

template <int D, int KB, int VB>
__global__ void __launch_bounds__(64 * kWaves) dequant_kernel(DequantArgs a) {
  constexpr int E = D / 64;
  constexpr bool kFp8 = KB == 8;
  constexpr int kKeyCodeBytes = kFp8 ? D : (D * KB + 7) / 8;
  constexpr int kKeyPacked = kFp8 ? D : kKeyCodeBytes + 2;
  constexpr int kValCodeBytes = (D * VB + 7) / 8;
  constexpr int kSlotRaw = kKeyPacked + kValCodeBytes + 4;
  constexpr int kSlot = kSlotRaw + (kSlotRaw & 1);
  constexpr int kDataBytes = kKeyCodeBytes + kValCodeBytes;   // split page

  __shared__ float s_cent[16];
  __shared__ float s_c[kWaves][D];            // Haar rotation: the centroid vector
  if (threadIdx.x < 16) s_cent[threadIdx.x] = a.tables->centroids[threadIdx.x];
  __syncthreads();
  const float* rot = a.tables->rot;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int H = a.H;
  uint32_t sgn[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = E * lane + e;
    sgn[e] = ((a.tables->sign_bits[j >> 5] >> (j & 31)) & 1u) << 31;
  }
  const float rsd = 1.0f / sqrtf(static_cast<float>(D));
  const int64_t total = static_cast<int64_t>(a.seq_len) * H;
  const int64_t page_bytes = (static_cast<int64_t>(H) * kSlot) << a.bs_shift;

  for (int64_t vec = static_cast<int64_t>(blockIdx.x) * kWaves + wave; vec < total;
       vec += static_cast<int64_t>(gridDim.x) * kWaves) {
    const int t = static_cast<int>(vec / H);
    const int h = static_cast<int>(vec - static_cast<int64_t>(t) * H);
    const int64_t o0 = vec * D + E * lane;            // output index of the lane's first coordinate
    const int page = a.block_table[t >> a.bs_shift];
    const int row = t & ((1 << a.bs_shift) - 1);
    if (page < 0 || page >= a.num_blocks) {
      if (lane == 0) a.errs->page = 1;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        put(a.k_out, o0 + e, 0.0f, a.out_fp32);
        put(a.v_out, o0 + e, 0.0f, a.out_fp32);
      }
      continue;
    }
    const uint8_t* pg = a.cache + static_cast<int64_t>(page) * page_bytes;
    const uint8_t* kp;          // K codes (or FP8 bytes)
    const uint8_t* vp;          // V codes
    float n_raw, sc, zr;        // stored K norm, V scale, V zero
    if (!kFp8 && a.soa) {
      kp = pg + (static_cast<int64_t>(row) * H + h) * kDataBytes;
      vp = kp + kKeyCodeBytes;
      const uint16_t* meta = reinterpret_cast<const uint16_t*>(
          pg + ((static_cast<int64_t>(H) * kDataBytes) << a.bs_shift)) + ((static_cast<int64_t>(h) * 3) << a.bs_shift) + row;
      n_raw = f16_bits_to_f32(meta[0]);
      sc = f16_bits_to_f32(meta[1 << a.bs_shift]);
      zr = f16_bits_to_f32(meta[2 << a.bs_shift]);
    } else {
      kp = pg + (static_cast<int64_t>(row) * H + h) * kSlot;
      vp = kp + kKeyPacked;
      const uint16_t* m16 = reinterpret_cast<const uint16_t*>(vp + kValCodeBytes);
      n_raw = kFp8 ? 0.0f : f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(kp + kKeyCodeBytes));
      sc = f16_bits_to_f32(m16[0]);
      zr = f16_bits_to_f32(m16[1]);
    }

    // ---------------- K ----------------
    float k[E];
    if constexpr (kFp8) {
#pragma unroll
      for (int e = 0; e < E; ++e) k[e] = e4m3fn_to_f32(kp[E * lane + e]);
    } else {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        k[e] = s_cent[stream_code(kp, E * lane + e, KB)];
        ss += k[e] * k[e];
      }
      float n = n_raw;
      if (!a.soa) {
#pragma unroll
        for (int m = 1; m < 64; m *= 2) ss += __shfl_xor(ss, m, 64);
        n = n_raw / sqrtf(ss + 1e-16f);
      }
      if (rot != nullptr) {
        // Haar rotation: k_i = n * sum_j Q[j][i] c_j
#pragma unroll
        for (int e = 0; e < E; ++e) s_c[wave][E * lane + e] = k[e];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float acc = 0.0f;
          for (int j = 0; j < D; ++j) acc += rot[static_cast<int64_t>(j) * D + E * lane + e] * s_c[wave][j];
          k[e] = acc;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int e = 0; e < E; ++e) k[e] *= n;
      } else {
      // R^T c = diag(s) H c / sqrt(d): butterflies, then signs and scale
#pragma unroll
      for (int hs = 1; hs < E; hs *= 2)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((e & hs) == 0) {
            const float p = k[e], r = k[e + hs];
            k[e] = p + r;
            k[e + hs] = p - r;
          }
#pragma unroll
      for (int lm = 1; lm < 64; lm *= 2) {
        const bool upper = (lane & lm) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float o = __shfl_xor(k[e], lm, 64);
          k[e] = upper ? (o - k[e]) : (k[e] + o);
        }
      }
      const float f = n * rsd;
#pragma unroll
      for (int e = 0; e < E; ++e) k[e] = __uint_as_float(__float_as_uint(k[e] * f) ^ sgn[e]);
      }
    }
    // ---------------- V ----------------
#pragma unroll
    for (int e = 0; e < E; ++e) {
      put(a.k_out, o0 + e, k[e], a.out_fp32);
      const float code = static_cast<float>(stream_code(vp, E * lane + e, VB));
      put(a.v_out, o0 + e, code * sc + zr, a.out_fp32);
    }
  }
}

// decode-as-prefill inputs: query i of a chunk is a decode request of length
// cached_len + i + 1 over the sequence's block-table row
__global__ void __launch_bounds__(256) expand_rows_kernel(const int32_t* row, int max_blocks, int cached_len,
                                                          int q_len, int32_t* seq_lens, int32_t* table) {
  const int64_t n = static_cast<int64_t>(q_len) * max_blocks;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int q = static_cast<int>(i / max_blocks);
    const int j = static_cast<int>(i - static_cast<int64_t>(q) * max_blocks);
    table[i] = row[j];
    if (j == 0) seq_lens[q] = cached_len + q + 1;
  }
}

template <int D, int KB, int VB>
hipError_t launch_t(const DequantArgs& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.seq_len) * a.H;
  int64_t blocks = (total + kWaves - 1) / kWaves;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((dequant_kernel<D, KB, VB>), dim3(static_cast<unsigned>(blocks)), dim3(64 * kWaves), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const Geometry& g, const DevTables* tables, DevErrors* errs, const uint8_t* cache,
                          int64_t num_blocks, const int32_t* block_table_row, int seq_len,
                          void* k_out, void* v_out, int out_is_fp32, hipStream_t stream) {
  DequantArgs a;
  a.tables = tables;
  a.errs = errs;
  a.cache = cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table_row;
  a.seq_len = seq_len;
  a.H = g.num_kv_heads;
  a.bs_shift = __builtin_ctz(static_cast<unsigned>(g.block_size));
  a.soa = g.soa;
  a.k_out = k_out;
  a.v_out = v_out;
  a.out_fp32 = out_is_fp32;
#define TQ_DQ_CASE(D_, KB_, VB_) \
  if (g.head_dim == D_ && g.key_bits == KB_ && g.value_bits == VB_) return launch_t<D_, KB_, VB_>(a, stream);
  TQ_DQ_CASE(64, 3, 4) TQ_DQ_CASE(64, 4, 4) TQ_DQ_CASE(64, 8, 4) TQ_DQ_CASE(64, 3, 3)
  TQ_DQ_CASE(128, 3, 4) TQ_DQ_CASE(128, 4, 4) TQ_DQ_CASE(128, 8, 4) TQ_DQ_CASE(128, 3, 3)
  TQ_DQ_CASE(256, 3, 4) TQ_DQ_CASE(256, 4, 4) TQ_DQ_CASE(256, 8, 4) TQ_DQ_CASE(256, 3, 3)
#undef TQ_DQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_expand_rows(const int32_t* row, int max_blocks, int cached_len, int q_len,
                              int32_t* seq_lens, int32_t* table, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(q_len) * max_blocks;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(expand_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, row,
                     max_blocks, cached_len, q_len, seq_lens, table);
  return hipGetLastError();
}

}  // namespace tq
