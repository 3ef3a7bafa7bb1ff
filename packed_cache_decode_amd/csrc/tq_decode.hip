// tq_decode kernels: split-KV paged decode attention over packed slots, and
// the log-sum-exp combine of the splits.
//
// What is computed follows P1 ("vLLM 源码完全拆解(十九):TurboQuant KV Cache
// 量化"), sections "读取内核" (two stages: per-split partials, then a merge),
// "程序入口:split 区间怎么算" (kv head = q head / group), "分数计算:FP8 K 与
// MSE K 的两条路径" (centroid gather, q_rot . c, stored norm, norm correction
// 1/sqrt(sum c^2 + 1e-16), scale 1/sqrt(d)), "V 的解包" (code * scale + zero)
// and "在线 softmax" (running max, rescaled sum and accumulator, fp32).
//
// Mapping (general path, any head_dim / bits / group size):
//   grid (split, sequence, kv head), one wavefront each.  The G query heads
//   of the kv head are rotated once into LDS (q_rot = R q, R = H diag(s)/sqrt(d)
//   by butterflies), pre-multiplied by sm_scale * log2(e) so the softmax runs
//   in base 2.  Tokens are taken 64 at a time: first lane = token (scores for
//   all G heads from the unpacked codes), then lane = coordinates (the V codes
//   of each token are read as one contiguous row by the whole wavefront, so
//   every V load is coalesced), accumulating p * v for all G heads.
//   Partials per (sequence, q head, split): acc[d], running max m (base 2),
//   running sum l.  The combine weights split s by 2^(m_s - max m).

#include "tq_internal.h"

namespace tq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
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
  int bs_shift;
  int chunk;
  int num_splits;
  int G;              // query heads per kv head (the kernel is built for a power of two >= G)
  float scale_log2;   // sm_scale * log2(e)
  float* part;        // [B][Hq][S][D + 2]
  void* out;
  int out_fp32;
  int soa;            // split page: data region + meta region [H][3][bs], folded K norm
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m *= 2) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m *= 2) x += __shfl_xor(x, m, 64);
  return x;
}

// GP: query heads per kv head the kernel is built for, a power of two; the
// a.G <= GP heads of the kv head are computed in the first slots (the rest
// repeat head 0 and are never stored)
template <int D, int KB, int GP, int VB>
__global__ void __launch_bounds__(64) decode_split_kernel(DecodeArgs a) {
  constexpr int G = GP;
  constexpr int E = D / 64;
  constexpr bool kFp8 = KB == 8;
  constexpr int kKeyCodeBytes = kFp8 ? D : (D * KB + 7) / 8;
  constexpr int kKeyPacked = kFp8 ? D : kKeyCodeBytes + 2;
  constexpr int kValOff = kKeyPacked;
  constexpr int kValCodeBytes = D * VB / 8;
  constexpr int kSlotRaw = kKeyPacked + kValCodeBytes + 4;
  constexpr int kSlot = kSlotRaw + (kSlotRaw & 1);
  constexpr int kDataBytes = kKeyCodeBytes + kValCodeBytes;   // split page: per (token, head)

  __shared__ float s_q[G][D];
  __shared__ float s_cent[16];
  __shared__ float s_p[G][64];
  __shared__ float s_vsc[64];
  __shared__ float s_vzr[64];
  __shared__ int64_t s_off[64];

  const int lane = threadIdx.x;
  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int g = blockIdx.z;
  const int Hq = a.Hq;
  int T = a.seq_lens[b];
  const int t_cap = min(a.num_splits * a.chunk, a.max_blocks << a.bs_shift);
  if (T < 0 || T > t_cap) {
    if (lane == 0 && split == 0 && g == 0) a.errs->len = 1;
    T = T < 0 ? 0 : t_cap;
  }
  const int t0 = split * a.chunk;
  const int t1 = min(T, t0 + a.chunk);
  const int Gr = a.G;
  float* part0 = a.part + ((static_cast<int64_t>(b) * Hq + g * Gr) * a.num_splits + split) * (D + 2);
  const int64_t head_stride = static_cast<int64_t>(a.num_splits) * (D + 2);

  if (t0 >= t1) {                      // empty split: acc 0, m -inf, l 0
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (j >= Gr) break;
      float* p = part0 + j * head_stride;
      for (int c = lane; c < D; c += 64) p[c] = 0.0f;
      if (lane == 0) {
        p[D] = -INFINITY;
        p[D + 1] = 0.0f;
      }
    }
    return;
  }

  // ---- rotate the G queries once (MSE keys) ----
  if (!kFp8 && lane < 16) s_cent[lane] = a.tables->centroids[lane];
  uint32_t sgn[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = E * lane + e;
    sgn[e] = ((a.tables->sign_bits[j >> 5] >> (j & 31)) & 1u) << 31;
  }
  const float rsd = 1.0f / sqrtf(static_cast<float>(D));
  if (!kFp8 && a.tables->rot != nullptr) {
    // Haar rotation: q_rot = Q q, coordinates of every query through LDS
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint16_t* qp = a.q + (static_cast<int64_t>(b) * Hq + g * Gr + (j < Gr ? j : 0)) * D + E * lane;
#pragma unroll
      for (int e = 0; e < E; ++e) s_q[j][E * lane + e] = bf16_bits_to_f32(qp[e]);
    }
    __syncthreads();
    float r[G][E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float* qrow = a.tables->rot + static_cast<int64_t>(E * lane + e) * D;
#pragma unroll
      for (int j = 0; j < G; ++j) r[j][e] = 0.0f;
      for (int i = 0; i < D; ++i) {
        const float qi = qrow[i];
#pragma unroll
        for (int j = 0; j < G; ++j) r[j][e] += qi * s_q[j][i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) s_q[j][E * lane + e] = r[j][e] * a.scale_log2;
  } else
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint16_t* qp = a.q + (static_cast<int64_t>(b) * Hq + g * Gr + (j < Gr ? j : 0)) * D + E * lane;
    float u[E];
#pragma unroll
    for (int e = 0; e < E; ++e) u[e] = bf16_bits_to_f32(qp[e]);
    if constexpr (!kFp8) {
#pragma unroll
      for (int e = 0; e < E; ++e) u[e] = __uint_as_float(__float_as_uint(u[e]) ^ sgn[e]);
#pragma unroll
      for (int hs = 1; hs < E; hs *= 2)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((e & hs) == 0) {
            const float p = u[e], r = u[e + hs];
            u[e] = p + r;
            u[e + hs] = p - r;
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
#pragma unroll
      for (int e = 0; e < E; ++e) u[e] *= rsd;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) s_q[j][E * lane + e] = u[e] * a.scale_log2;
  }
  __syncthreads();

  float m_run[G], l_run[G], acc[G][E];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[j][e] = 0.0f;
  }

  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  const int64_t row_bytes = static_cast<int64_t>(a.H) * kSlot;
  const int bs_mask = (1 << a.bs_shift) - 1;

  // split page: V codes follow the K codes in the data region; the token's
  // K norm, V scale and V zero sit bs fp16 apart in the meta region
  const int v_off = a.soa ? kKeyCodeBytes : kValOff;
  const int64_t meta_step = static_cast<int64_t>(2) << a.bs_shift;

  for (int tb = t0; tb < t1; tb += 64) {
    const int t = tb + lane;
    bool valid = t < t1;
    int64_t off = 0;        // the token's slot (split page: its data bytes)
    int64_t moff = 0;       // split page: its K norm
    if (valid) {
      const int page = bt[t >> a.bs_shift];
      if (page < 0 || page >= a.num_blocks) {
        a.errs->page = 1;
        valid = false;
      } else if (a.soa) {
        const int64_t pb = static_cast<int64_t>(page) * (row_bytes << a.bs_shift);
        off = pb + (static_cast<int64_t>(t & bs_mask) * a.H + g) * kDataBytes;
        moff = pb + ((static_cast<int64_t>(a.H) * kDataBytes) << a.bs_shift) +
               static_cast<int64_t>(3 * g) * meta_step + 2 * (t & bs_mask);
      } else {
        off = (static_cast<int64_t>(page) * (bs_mask + 1) + (t & bs_mask)) * row_bytes +
              static_cast<int64_t>(g) * kSlot;
      }
    }
    // ---- scores, lane = token ----
    float sc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) sc[j] = 0.0f;
    float vsc = 0.0f, vzr = 0.0f;
    if (valid) {
      const uint8_t* slot = a.cache + off;
      const uint16_t* s16 = reinterpret_cast<const uint16_t*>(slot);
      if constexpr (kFp8) {
        for (int w = 0; w < D / 2; ++w) {
          const uint32_t two = s16[w];
          const float k0 = e4m3fn_to_f32(two & 0xFF), k1 = e4m3fn_to_f32(two >> 8);
#pragma unroll
          for (int j = 0; j < G; ++j) sc[j] += s_q[j][2 * w] * k0 + s_q[j][2 * w + 1] * k1;
        }
      } else {
        float ss = 0.0f;
        // codes through a 16-bit window: code j at bits [j*KB, j*KB + KB)
        uint32_t window = s16[0];
        int have = 16;     // bits valid in window
        int next = 1;      // next u16 to read
#pragma unroll 8
        for (int c = 0; c < D; ++c) {
          if (have < KB) {
            window |= static_cast<uint32_t>(s16[next++]) << have;
            have += 16;
          }
          const int code = window & ((1u << KB) - 1u);
          window >>= KB;
          have -= KB;
          const float cv = s_cent[code];
          ss += cv * cv;
#pragma unroll
          for (int j = 0; j < G; ++j) sc[j] += s_q[j][c] * cv;
        }
        // the split page stores the corrected norm |k| / |c| itself
        const float f = a.soa ? f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(a.cache + moff))
                              : f16_bits_to_f32(s16[kKeyCodeBytes / 2]) / sqrtf(ss + 1e-16f);
#pragma unroll
        for (int j = 0; j < G; ++j) sc[j] *= f;
      }
      if (a.soa) {
        vsc = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(a.cache + moff + meta_step));
        vzr = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(a.cache + moff + 2 * meta_step));
      } else {
        const uint16_t* meta = reinterpret_cast<const uint16_t*>(slot + kValOff + kValCodeBytes);
        vsc = f16_bits_to_f32(meta[0]);
        vzr = f16_bits_to_f32(meta[1]);
      }
    }
    // ---- online softmax over this block of tokens (base 2) ----
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float s = valid ? sc[j] : -INFINITY;
      const float mx = wave_max(s);
      const float m_new = fmaxf(m_run[j], mx);
      const float p = valid ? exp2f(s - m_new) : 0.0f;
      const float corr = (m_run[j] == -INFINITY) ? 0.0f : exp2f(m_run[j] - m_new);
      l_run[j] = l_run[j] * corr + wave_sum(p);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[j][e] *= corr;
      m_run[j] = m_new;
      s_p[j][lane] = p;
    }
    s_vsc[lane] = vsc;
    s_vzr[lane] = vzr;
    s_off[lane] = valid ? off : -1;
    __syncthreads();
    // ---- p . v, lane = coordinates [E*lane, E*lane + E) ----
    const int nt = min(64, t1 - tb);
    for (int i = 0; i < nt; ++i) {
      const int64_t o = s_off[i];
      if (o < 0) continue;
      const uint8_t* vrow = a.cache + o + v_off;
      float vh[E];
      if constexpr (VB == 3) {
        // code c at stream bits [3c, 3c + 3); the byte after the last code
        // byte is the scale's first, inside the slot (split page: the next
        // data bytes or the meta region, inside the page)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int bit = 3 * (E * lane + e);
          const uint32_t two = vrow[bit >> 3] | (static_cast<uint32_t>(vrow[(bit >> 3) + 1]) << 8);
          vh[e] = static_cast<float>((two >> (bit & 7)) & 7u);
        }
      } else if constexpr (E == 1) {
        const uint32_t byte = vrow[lane >> 1];
        vh[0] = static_cast<float>((byte >> ((lane & 1) * 4)) & 15u);
      } else {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const uint32_t byte = vrow[(E * lane + e) >> 1];
          vh[e] = static_cast<float>(byte & 15u);
          vh[e + 1] = static_cast<float>(byte >> 4);
        }
      }
      const float vs = s_vsc[i], vz = s_vzr[i];
#pragma unroll
      for (int e = 0; e < E; ++e) vh[e] = vh[e] * vs + vz;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float p = s_p[j][i];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[j][e] += p * vh[e];
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (j >= Gr) break;
    float* p = part0 + j * head_stride;
#pragma unroll
    for (int e = 0; e < E; ++e) p[E * lane + e] = acc[j][e];
    if (lane == 0) {
      p[D] = m_run[j];
      p[D + 1] = l_run[j];
    }
  }
}

// Merge the splits of one (sequence, q head): weights 2^(m_s - M).
template <int D>
__global__ void __launch_bounds__(64) decode_combine_kernel(DecodeArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;          // b * Hq + hq
  const float* part = a.part + bh * a.num_splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.num_splits; ++s) M = fmaxf(M, part[s * (D + 2) + D]);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.num_splits; ++s) {
      const float* p = part + s * (D + 2);
      const float ms = p[D];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - M);
      L += w * p[D + 1];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * p[E * lane + e];
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  if (a.out_fp32) {
    float* o = static_cast<float*>(a.out) + bh * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = acc[e] * inv;
  } else {
    uint16_t* o = static_cast<uint16_t*>(a.out) + bh * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t u = __float_as_uint(acc[e] * inv);
      o[e] = static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // RNE
    }
  }
}

template <int D, int KB, int G, int VB>
hipError_t launch_t(const DecodeArgs& a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, KB, G, VB>), dim3(a.num_splits, batch, a.H), dim3(64), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(batch * a.Hq), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int KB, int VB>
hipError_t launch_g(const DecodeArgs& a, int G, int batch, hipStream_t stream) {
  // the kernel built for the next power of two
  if (G < 1) return hipErrorInvalidValue;
  if (G <= 1) return launch_t<D, KB, 1, VB>(a, batch, stream);
  if (G <= 2) return launch_t<D, KB, 2, VB>(a, batch, stream);
  if (G <= 4) return launch_t<D, KB, 4, VB>(a, batch, stream);
  if (G <= 8) return launch_t<D, KB, 8, VB>(a, batch, stream);
  if (G <= 16) return launch_t<D, KB, 16, VB>(a, batch, stream);
  return hipErrorInvalidValue;
}

}  // namespace

namespace {
DecodePlan plan_decode_kernels(const Geometry& g, const tq_decode_options& opts, int batch, int num_q_heads,
                               int max_seq_len) {
  DecodePlan p{};
  // ring kernel: slabs dealt out in a fixed interleaved order unless the
  // context asks for dynamic claims (results then vary in the last bits)
  p.dynamic = opts.dynamic_claims ? 1 : 0;
  if (opts.kernel != TQ_DECODE_KERNEL_GENERAL && dslab_decode_eligible(g, num_q_heads)) {
    // head dims 64 and 256 on the slotted page: the direct matrix-core
    // kernel's design at those dims (the forced d = 128 kernels do not apply),
    // one resident round of wavefronts over (split, sequence, kv head), at
    // least 8 slabs per split; Haar-rotated queries once into the workspace
    const int slabs = max_seq_len > 0 ? (max_seq_len + 15) / 16 : 1;
    const int per_split = batch * g.num_kv_heads;
    const int target = 256 * dslab_waves_per_cu(g);
    int s = per_split > 0 ? (target + per_split - 1) / per_split : 1;
    const int s_max = (slabs + 7) / 8;
    s = s < 1 ? 1 : (s > s_max ? s_max : s);
    p.mfma = 5;
    p.chunk = 16 * ((slabs + s - 1) / s);
    if (p.chunk > 16 * 256) p.chunk = 16 * 256;       // page offsets of a split fit in LDS
    p.num_splits = max_seq_len > 0 ? (max_seq_len + p.chunk - 1) / p.chunk : 1;
    p.workspace_bytes = dslab_partial_bytes(g, batch, num_q_heads, p.num_splits);
    p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
    if (g.key_bits != 8 && g.haar) {
      p.qrot = 1;
      p.qrot_off = p.workspace_bytes;
      p.workspace_bytes += static_cast<size_t>(batch) * num_q_heads * g.head_dim * sizeof(float);
      p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
    }
    return p;
  }
  if ((g.haar && g.head_dim != 128) || opts.kernel == TQ_DECODE_KERNEL_GENERAL) {
    // the general kernel: the Haar rotation at other head dims where the
    // matrix-core kernels do not apply (the split page), and any shape when
    // the options ask for it
    p.mfma = 0;
    p.chunk = 256;
    p.num_splits = max_seq_len > 0 ? (max_seq_len + p.chunk - 1) / p.chunk : 1;
    p.workspace_bytes = static_cast<size_t>(batch) * num_q_heads * p.num_splits *
                        (g.head_dim + 2) * sizeof(float);
    p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
    return p;
  }
  // Matrix-core kernel by key type (measured on the llama3-, long-context,
  // k3v4- and k8v4-shaped decodes): FP8 keys take the page-cooperative
  // kernel; 3/4-bit keys with at most 8 query heads per kv head the ring
  // kernel, else (an even number of kv heads) the staged kernel, else the
  // direct one.  The context's options may force one where it applies.
  const int force = opts.kernel;
  const bool auto_pick = force == TQ_DECODE_KERNEL_AUTO;
  if ((auto_pick || force == TQ_DECODE_KERNEL_PAGE) &&
      page_decode_eligible(g, num_q_heads, force == TQ_DECODE_KERNEL_PAGE)) {
    // one resident round of workgroups (256 CUs x the workgroups that fit per
    // CU) over (sequence, split), at least 4 slabs of 16 tokens per split so
    // the load pipeline's start is amortised
    // kv heads per workgroup: the whole row, at most 8 (measured fastest:
    // smaller groups were slower for FP8 keys); the options may ask for
    // smaller groups
    int group = g.num_kv_heads < 8 ? g.num_kv_heads : 8;
    const int want = opts.page_heads;
    if ((want == 1 || want == 2 || want == 4) && g.num_kv_heads % want == 0) group = want;
    const int slabs = max_seq_len > 0 ? (max_seq_len + 15) / 16 : 1;
    const int target = 256 * page_wgs_per_cu(g, group);
    const int per_split = batch * (g.num_kv_heads / group);
    int s = per_split > 0 ? (target + per_split - 1) / per_split : 1;
    const int s_max = (slabs + 3) / 4;
    s = s < 1 ? 1 : (s > s_max ? s_max : s);
    p.mfma = 2;
    p.group = group;
    p.chunk = 16 * ((slabs + s - 1) / s);
    if (p.chunk > 16 * 256) p.chunk = 16 * 256;       // page ids of a split fit in LDS
    p.num_splits = max_seq_len > 0 ? (max_seq_len + p.chunk - 1) / p.chunk : 1;
    p.workspace_bytes = mfma_partial_bytes(batch, num_q_heads, p.num_splits);
    p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
    return p;
  }
  if (ring_decode_eligible(g, num_q_heads) && (force == TQ_DECODE_KERNEL_RING || auto_pick)) {
    // ring kernel: one workgroup per (sequence, kv head, workgroup split),
    // at most ring_max_slabs() slabs per split (its page ids fit in LDS);
    // more splits only to fill whole rounds of the 256 CUs (one 16-wavefront
    // workgroup each), so a round is not left part-empty, and only while
    // every wavefront keeps at least 4 slabs
    const int slabs = max_seq_len > 0 ? (max_seq_len + 15) / 16 : 1;
    const int cap = ring_max_slabs();
    const int s_min = (slabs + cap - 1) / cap;
    const int pairs = batch * g.num_kv_heads;
    int s = s_min;
    if (pairs > 0) {
      const int rounds = (pairs * s_min + 255) / 256;
      const int s_fill = rounds * 256 / pairs;
      const int s_work = slabs / 64;
      const int s_up = s_fill < s_work ? s_fill : s_work;
      if (s_up > s) s = s_up;
    }
    if (s < 1) s = 1;
    p.mfma = 4;
    // two or more rounds of one-per-CU workgroups: half-size workgroups, two
    // per CU, so one's set-up and drain overlap the other's streaming (the
    // options may force either size)
    p.ring_waves = pairs * s >= 2 * 256 ? 8 : 16;
    if (opts.ring_waves == 8 || opts.ring_waves == 16) p.ring_waves = opts.ring_waves;
    p.chunk = 16 * ((slabs + s - 1) / s);
    p.num_splits = max_seq_len > 0 ? (max_seq_len + p.chunk - 1) / p.chunk : 1;
    p.workspace_bytes = p.num_splits > 1 ? mfma_partial_bytes(batch, num_q_heads, p.num_splits) : 0;
    p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
    // more workgroups than one per CU: dispatch the sequences longest first,
    // so the ones that start late are short (lengths may be ragged; the plan
    // sees only the longest)
    if (pairs * s > 256 && batch <= 1024) {
      p.order = 1;
      p.order_off = p.workspace_bytes;
      p.workspace_bytes += (4 * static_cast<size_t>(batch) + 255) & ~static_cast<size_t>(255);
    }
    return p;
  }
  if (mfma_decode_eligible(g, num_q_heads)) {
    // one resident round of wavefronts (256 CUs x the kernel's wavefronts per
    // CU) over (split, sequence, kv head), 16-token slabs, at least 8 slabs
    // per split so the per-wavefront set-up is amortised
    const int slabs = max_seq_len > 0 ? (max_seq_len + 15) / 16 : 1;
    const int per_split = batch * g.num_kv_heads;
    const bool staged = staged_decode_eligible(g, num_q_heads) &&
                        (force == TQ_DECODE_KERNEL_STAGED || auto_pick);
    const int target = 256 * mfma_waves_per_cu(g, staged);
    int s = per_split > 0 ? (target + per_split - 1) / per_split : 1;
    const int s_max = (slabs + 7) / 8;
    s = s < 1 ? 1 : (s > s_max ? s_max : s);
    p.mfma = staged ? 3 : 1;
    p.chunk = 16 * ((slabs + s - 1) / s);
    if (p.chunk > 16 * 256) p.chunk = 16 * 256;       // page offsets of a split fit in LDS
    p.num_splits = max_seq_len > 0 ? (max_seq_len + p.chunk - 1) / p.chunk : 1;
    p.workspace_bytes = mfma_partial_bytes(batch, num_q_heads, p.num_splits);
    p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
    return p;
  }
  p.mfma = 0;
  p.chunk = 256;
  p.num_splits = max_seq_len > 0 ? (max_seq_len + p.chunk - 1) / p.chunk : 1;
  p.workspace_bytes = static_cast<size_t>(batch) * num_q_heads * p.num_splits *
                      (g.head_dim + 2) * sizeof(float);
  p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
  return p;
}

}  // namespace

DecodePlan plan_decode(const Geometry& g, const tq_decode_options& opts, int batch, int num_q_heads,
                       int max_seq_len) {
  DecodePlan p = plan_decode_kernels(g, opts, batch, num_q_heads, max_seq_len);
  if (p.mfma != 0) {
    const int G = num_q_heads / g.num_kv_heads;
    p.g_pass = G < mfma_max_g(p.mfma) ? G : mfma_max_g(p.mfma);
  }
  if (g.haar && p.mfma != 0 && !p.qrot) {
    // the matrix-core kernels read the queries rotated by the Haar matrix
    // from the workspace, after the split partials
    p.qrot = 1;
    p.qrot_off = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
    p.workspace_bytes = p.qrot_off + static_cast<size_t>(batch) * num_q_heads * g.head_dim * sizeof(float);
    p.workspace_bytes = (p.workspace_bytes + 255) & ~static_cast<size_t>(255);
  }
  return p;
}

hipError_t launch_decode(const Geometry& g, const DevTables* tables, DevErrors* errs, const DecodePlan& plan,
                         const uint16_t* q, const uint8_t* cache, int64_t num_blocks,
                         const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* seq_lens, int batch, int num_q_heads, float sm_scale,
                         void* out, int out_is_fp32, void* workspace, hipStream_t stream) {
  DecodeArgs a;
  if (plan.mfma)
    return launch_decode_mfma(g, tables, errs, plan, q, cache, num_blocks, block_table, max_blocks_per_seq,
                              seq_lens, batch, num_q_heads, sm_scale, out, out_is_fp32, workspace,
                              stream);
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
  a.bs_shift = __builtin_ctz(static_cast<unsigned>(g.block_size));
  a.chunk = plan.chunk;
  a.num_splits = plan.num_splits;
  a.scale_log2 = sm_scale * kLog2e;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.out_fp32 = out_is_fp32;
  a.soa = g.soa;
  const int G = num_q_heads / g.num_kv_heads;
  a.G = G;
#define TQ_DEC_CASE(D_, KB_, VB_) \
  if (g.head_dim == D_ && g.key_bits == KB_ && g.value_bits == VB_) return launch_g<D_, KB_, VB_>(a, G, batch, stream);
  TQ_DEC_CASE(64, 3, 4) TQ_DEC_CASE(64, 4, 4) TQ_DEC_CASE(64, 8, 4) TQ_DEC_CASE(64, 3, 3)
  TQ_DEC_CASE(128, 3, 4) TQ_DEC_CASE(128, 4, 4) TQ_DEC_CASE(128, 8, 4) TQ_DEC_CASE(128, 3, 3)
  TQ_DEC_CASE(256, 3, 4) TQ_DEC_CASE(256, 4, 4) TQ_DEC_CASE(256, 8, 4) TQ_DEC_CASE(256, 3, 3)
#undef TQ_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace tq
