// tq_store at head dims 64 and 256 on the slotted page with the Hadamard
// rotation: the four-lanes-per-vector kernel of tq_store_common.h with 16 or
// 64 coordinates per lane (its own module; see tq_store_common.h).
#include "tq_store_common.h"

#pragma clang fp contract(off)

namespace tq {
namespace {

// head dims 64 and 256 (slotted page, Hadamard rotation): the same kernel
// with 16 or 64 coordinates per lane
template <int D, int KB, int VB>
hipError_t launch_store_quad(const StoreArgs& a, hipStream_t stream) {
  constexpr int kRaw = (KB == 8 ? D : D * KB / 8 + 2) + D * VB / 8 + 4;
  constexpr int kSlot = kRaw + kRaw % 2;
  const int64_t total = a.num_tokens * a.H;
  int64_t blocks = (total + 63) / 64;               // 64 vectors per 256-thread block
  if (blocks > 8192) blocks = 8192;
  const bool rows = 16 % a.H == 0 && (static_cast<int64_t>(a.H) * kSlot) % 16 == 0;
  if (rows)
    hipLaunchKernelGGL((store_quad_kernel<D, KB, VB, true, false>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, stream, a);
  else
    hipLaunchKernelGGL((store_quad_kernel<D, KB, VB, false, false>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_store_quad_64_256(const Geometry& g, const StoreArgs& a, hipStream_t stream) {
  const bool d64 = g.head_dim == 64;
  if (g.key_bits == 8) return d64 ? launch_store_quad<64, 8, 4>(a, stream) : launch_store_quad<256, 8, 4>(a, stream);
  if (g.key_bits == 4) return d64 ? launch_store_quad<64, 4, 4>(a, stream) : launch_store_quad<256, 4, 4>(a, stream);
  if (g.value_bits == 4)
    return d64 ? launch_store_quad<64, 3, 4>(a, stream) : launch_store_quad<256, 3, 4>(a, stream);
  return d64 ? launch_store_quad<64, 3, 3>(a, stream) : launch_store_quad<256, 3, 3>(a, stream);
}

}  // namespace tq
