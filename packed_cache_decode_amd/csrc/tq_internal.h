// Internal definitions shared by the host library and the HIP kernels.
// Not part of the public ABI (include/tq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxHeadDim = 256;
constexpr int kMaxLevels = 16;

constexpr int kMaxBins = 64;

// Device-resident tables of one context (under 1 KB, one allocation).
// Sign flips are a bit mask: bit j of sign_bits[j / 32] set means s_j = -1.
//
// Bucketize bins (MSE keys): the count #{m : y >= mid_m} equals
//   base + (y >= thr)  for  {thr, base} = bins[i],
//   i = clamp(floor(fma(y, bin_scale, bin_bias)), 0, bin_count - 1),
// where bin_scale = 2^k makes every bin [(j + phi) / 2^k, (j + 1 + phi) / 2^k) no wider than
// the smallest midpoint gap (so it holds at most one midpoint, thr, or NaN),
// base counts the midpoints at or below the bin's lower edge, and bin 0 (base
// 0, thr NaN) takes everything below the first edge and NaN (whose integer
// conversion is 0).  The host checks that no midpoint lies within 4x the
// fma's rounding error of an edge, so a value rounded into the neighbouring
// bin still gets the same count; bin_count == 0 means no such table exists.
struct DevTables {
  float centroids[kMaxLevels];
  float midpoints[kMaxLevels];          // 2^b - 1 entries used
  uint32_t sign_bits[kMaxHeadDim / 32];
  int32_t bin_count;
  float bin_scale;
  float bin_bias;
  int32_t pad[1];
  uint32_t bins[kMaxBins][2];           // {float bits of thr, base}
  const float* rot;                     // Haar rotation: Q (d x d, row-major, fp32); null otherwise
};

// Sticky error words of a context, in their own device allocation (the
// tables above are read-only to the kernels; these are the only device
// memory of a context that kernels write).  A kernel sets a word to 1 and
// skips the offending item; tq_get_device_error reads and clears them.
struct DevErrors {
  int32_t slot;   // a store slot beyond the cache
  int32_t page;   // a page id beyond the cache
  int32_t len;    // a sequence length beyond the grid or the block table
  int32_t pad;
};

struct Geometry {
  int head_dim;
  int num_kv_heads;
  int block_size;
  int key_bits;         // 3, 4, or 8 (fp8)
  int value_bits;       // 4
  int norm_correction;  // 0 / 1
  int key_code_bytes;   // ceil(d*kb/8) or d for fp8
  int key_packed;       // key_code_bytes (+2 for the norm unless fp8)
  int value_code_bytes; // ceil(d*vb/8)
  int slot;             // aligned slot bytes
  int bins_ok;          // the bucketize bins of the device tables exist
  int soa;              // page layout: 0 = slots back to back, 1 = data region +
                        // meta region [H][3][block_size] fp16 (folded K norm)
  int haar;             // MSE keys rotated by the Haar matrix DevTables::rot
                        // instead of the (signed) Hadamard transform
};

// ---- launchers (defined in the .hip files) ---------------------------------

hipError_t launch_store(const Geometry& g, const DevTables* tables, DevErrors* errs, const uint16_t* k,
                        const uint16_t* v, int64_t kv_token_stride, const int64_t* slot_mapping,
                        int64_t num_tokens, uint8_t* cache, int64_t num_blocks, float r_d,
                        hipStream_t stream);

struct DecodePlan {
  int mfma;         // matrix-core kernels (tq_decode_mfma.hip): 2 page-cooperative,
                    // 3 staged per-head, 4 ring per-head, 1 direct per-head,
                    // 5 direct per-head at head dims 64 and 256; 0: general kernel
  int group;        // page kernel: kv heads per workgroup (1, 2, 4 or 8)
  int chunk;        // tokens per split
  int num_splits;   // splits per sequence (grid extent)
  size_t workspace_bytes;
  int dynamic;        // ring kernel: wavefronts claim slabs from a counter (the order of
                      // the fp32 sums, and so the last bits, vary run to run); 0: fixed
                      // interleaved shares (reproducible bit for bit)
  int ring_waves;     // ring kernel: 16 wavefronts per workgroup (one per CU) or 8 (two per CU)
  int order;          // ring kernel: sequences ranked by length (longest first, int32 [B])
                      // in the workspace at byte order_off, workgroups dispatched in that order
  size_t order_off;
  int qrot;           // Haar rotation on a matrix-core kernel, or any MSE keys at head dims
                      // 64 and 256: the rotated queries (fp32 [B][Hq][d]) sit in the
                      // workspace at byte qrot_off
  size_t qrot_off;
  int g_pass;         // matrix-core kernels: query heads per kv head in one pass of the
                      // kernel (its limit: 8 ring and page, 16 staged and direct); more
                      // query heads run as several passes over the cache
};

bool mfma_decode_eligible(const Geometry& g, int num_q_heads);
bool page_decode_eligible(const Geometry& g, int num_q_heads, bool mse_keys_too);
int page_wgs_per_cu(const Geometry& g, int group);
bool staged_decode_eligible(const Geometry& g, int num_q_heads);
bool ring_decode_eligible(const Geometry& g, int num_q_heads);
int ring_max_slabs();
int mfma_max_g(int mfma);
bool dslab_decode_eligible(const Geometry& g, int num_q_heads);
int dslab_waves_per_cu(const Geometry& g);
size_t dslab_partial_bytes(const Geometry& g, int batch, int num_q_heads, int num_splits);
int mfma_waves_per_cu(const Geometry& g, bool staged);
size_t mfma_partial_bytes(int batch, int num_q_heads, int num_splits);
hipError_t launch_decode_mfma(const Geometry& g, const DevTables* tables, DevErrors* errs,
                              const DecodePlan& plan,
                              const uint16_t* q, const uint8_t* cache, int64_t num_blocks,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int32_t* seq_lens, int batch, int num_q_heads, float sm_scale,
                              void* out, int out_is_fp32, void* workspace, hipStream_t stream);

DecodePlan plan_decode(const Geometry& g, const tq_decode_options& opts, int batch, int num_q_heads,
                       int max_seq_len);

hipError_t launch_dequant(const Geometry& g, const DevTables* tables, DevErrors* errs, const uint8_t* cache,
                          int64_t num_blocks, const int32_t* block_table_row, int seq_len,
                          void* k_out, void* v_out, int out_is_fp32, hipStream_t stream);
hipError_t launch_expand_rows(const int32_t* row, int max_blocks, int cached_len, int q_len,
                              int32_t* seq_lens, int32_t* table, hipStream_t stream);

hipError_t launch_decode(const Geometry& g, const DevTables* tables, DevErrors* errs, const DecodePlan& plan,
                         const uint16_t* q, const uint8_t* cache, int64_t num_blocks,
                         const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* seq_lens, int batch, int num_q_heads, float sm_scale,
                         void* out, int out_is_fp32, void* workspace, hipStream_t stream);

}  // namespace tq
