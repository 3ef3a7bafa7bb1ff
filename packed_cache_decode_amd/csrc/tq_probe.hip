// Streaming-read probes: how fast this part reads a large buffer from HBM
// with each of the load forms the store and decode kernels use -- 16-byte
// vector loads into registers, and 16-byte buffer loads that write LDS
// directly -- each plain and non-temporal.  They measure the achievable read
// rate the decode's bytes per second are compared against; they compute
// nothing of the method.
//
// Mapping: workgroups of 256 threads (4 wavefronts) over contiguous chunks of
// the buffer, several resident per CU.  In every step a wavefront reads
// kUnroll x 1 KB (16 bytes per lane per load) before it waits, so each CU
// keeps tens of KB in flight.  Register loads fold their words into a
// per-thread XOR written at the end (so no load is dead); LDS loads land in a
// per-wavefront ring, of which one word per lane is written at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                   // 1 KB loads per wavefront per step (registers)
constexpr int kLdsUnroll = 4;                // ... (LDS: two halves of this, 32 KB per workgroup)
constexpr int kBufferWord3 = 0x00020000;     // raw buffer resource, 32-bit data format
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bytes of one workgroup step: 256 threads x 16 bytes x kUnroll
constexpr int64_t kStep = static_cast<int64_t>(kThreads) * 16 * kUnroll;

template <bool NT>
__global__ void __launch_bounds__(kThreads) probe_regs_kernel(const uint8_t* src, int64_t steps_per_wg,
                                                             int64_t total_steps, uint32_t* sink) {
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * steps_per_wg;
  const int64_t s1 = min(total_steps, s0 + steps_per_wg);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t s = s0; s < s1; ++s) {
    const u32x4* p = reinterpret_cast<const u32x4*>(src + s * kStep) + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if constexpr (NT)
        v[u] = __builtin_nontemporal_load(p + u * kThreads);
      else
        v[u] = p[u * kThreads];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  sink[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <bool NT>
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
}

template <bool NT>
__global__ void __launch_bounds__(kThreads) probe_lds_kernel(const uint8_t* src, int64_t steps_per_wg,
                                                            int64_t total_steps, uint32_t* sink) {
  // two halves of kLdsUnroll KB per wavefront: one is filled while the loads
  // of the other are waited for
  __shared__ __attribute__((aligned(16))) uint8_t ring[kThreads / 64][2][kLdsUnroll * 1024];
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * steps_per_wg;
  const int64_t s1 = min(total_steps, s0 + steps_per_wg);
  int half = 0;
  for (int64_t s = s0; s < s1; ++s) {
    // this wavefront's 8 KB of the step in two rounds of kLdsUnroll KB,
    // 16 bytes per lane per load
    const uint8_t* base = src + s * kStep + static_cast<int64_t>(w) * 1024 * kUnroll;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base), 0, 1024 * kUnroll, kBufferWord3);
#pragma unroll
    for (int r = 0; r < kUnroll / kLdsUnroll; ++r) {
      const uint32_t dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (__attribute__((address_space(3))) uint8_t*)&ring[w][half][0]));
#pragma unroll
      for (int u = 0; u < kLdsUnroll; ++u)
        lds_load16<NT>(rs, dst + u * 1024, (r * kLdsUnroll + u) * 1024 + 16 * lane);
      // the other half's loads (the round before) have landed once at most
      // kLdsUnroll loads remain
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLdsUnroll) : "memory");
      half ^= 1;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  const uint32_t v = *reinterpret_cast<const uint32_t*>(&ring[w][half][16 * lane]);
  sink[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = v;
}

}  // namespace

extern "C" {

int64_t tq_probe_sink_words(int64_t bytes) {
  if (bytes < kStep) return -1;
  const int64_t steps = bytes / kStep;
  const int64_t wgs = steps < 256 * 8 ? steps : 256 * 8;
  return wgs * kThreads;
}

int tq_probe_read(int mode, const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes < kStep || mode < 0 || mode > 3) return -1;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return -3;
  const int64_t steps = bytes / kStep;                    // whole steps only
  const int64_t wgs = steps < 256 * 8 ? steps : 256 * 8;  // eight workgroups per CU
  const int64_t per = (steps + wgs - 1) / wgs;
  const dim3 grid(static_cast<unsigned>(wgs)), block(kThreads);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  switch (mode) {
    case TQ_PROBE_REGS: hipLaunchKernelGGL(probe_regs_kernel<false>, grid, block, 0, st, s, per, steps, sink); break;
    case TQ_PROBE_REGS_NT: hipLaunchKernelGGL(probe_regs_kernel<true>, grid, block, 0, st, s, per, steps, sink); break;
    case TQ_PROBE_LDS: hipLaunchKernelGGL(probe_lds_kernel<false>, grid, block, 0, st, s, per, steps, sink); break;
    default: hipLaunchKernelGGL(probe_lds_kernel<true>, grid, block, 0, st, s, per, steps, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
