/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant packed KV-cache library.
 *
 * The library implements two operations of the TurboQuant KV-cache method:
 *
 *   tq_store   quantise new K/V head vectors and write them, one fixed-size
 *              slot per (token, kv head), into a paged byte cache;
 *   tq_decode  paged decode attention (one query per sequence) computed
 *              directly on those packed slots.
 *
 * Sources, cited by page title and section:
 *   P1  "vLLM 源码完全拆解(十九):TurboQuant KV Cache 量化——Hadamard 旋转、
 *       Lloyd-Max 标量量化与分页缓存内核" (pinghaoyang.com.cn)
 *   P3  kwkr.cn news 555717, an article on the turboquant project (the
 *       Beta law of a rotated coordinate and its pre-computed codebooks)
 *   P5  "NVIDIA KV Cache 量化中的 NVFP4 与 TurboQuant" (moonnryan.github.io)
 *
 * Conventions for every call:
 *   - Pointers named "device" are HIP device pointers; "host" pointers are
 *     ordinary host memory.  The caller owns every buffer it passes in.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     tq_store and tq_decode only enqueue work on it: they neither allocate
 *     nor synchronise, and return before the GPU has finished.
 *   - Argument errors are detected on the host and returned as a negative
 *     tq_status before anything is enqueued.  A failed kernel launch returns
 *     TQ_ERR_HIP.  Faults the host cannot see (a slot or page id beyond the
 *     cache) make the kernel skip that item and set a sticky device error
 *     word, read with tq_get_device_error after the stream has synchronised.
 *   - Nothing here is thread-hostile: calls on different streams that write
 *     disjoint outputs may run concurrently.  Duplicate slots within one
 *     tq_store call race (the caller's scheduler gives unique slots).
 */
#ifndef TQ_MI355X_H
#define TQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum, Hq % H != 0 */
  TQ_ERR_UNSUPPORTED = -2,   /* a head_dim / block_size / preset not built        */
  TQ_ERR_ALIGNMENT = -3,     /* cache or activation base not suitably aligned     */
  TQ_ERR_WORKSPACE = -4,     /* decode workspace smaller than required            */
  TQ_ERR_HIP = -5,           /* a HIP runtime call or kernel launch failed        */
  TQ_ERR_NO_DEVICE = -6      /* no gfx950 device is current                       */
} tq_status;

/* The presets of P1, section "四个预设对应什么": K bits / V bits / norm
 * correction.  k8v4 stores K as FP8 E4M3 without rotation (P1, section
 * "FP8 K 路径:不旋转,直接 cast"). */
typedef enum {
  TQ_K8V4 = 0,      /* K fp8-e4m3,           V 4-bit, no norm correction */
  TQ_4BIT_NC = 1,   /* K 4-bit Lloyd-Max,    V 4-bit, norm correction    */
  TQ_K3V4_NC = 2,   /* K 3-bit Lloyd-Max,    V 4-bit, norm correction    */
  TQ_3BIT_NC = 3    /* K 3-bit Lloyd-Max,    V 3-bit, norm correction
                       (V scale = (max - min) / 7, codes packed like 3-bit K) */
} tq_preset;

/* How the codebook is solved (P1, sections "Lloyd-Max 的两个最优性条件" and
 * "vLLM 的实现:数值积分而不是解析解"). */
typedef enum {
  TQ_CODEBOOK_LLOYD_MAX_EXACT = 0,  /* fixed point with closed-form Gaussian
                                       conditional means, float64, then float32 */
  TQ_CODEBOOK_PAGE_TRAPZ = 1,       /* the page's 200-trapezoid recipe, 200
                                       iterations at most, tolerance 1e-10    */
  TQ_CODEBOOK_BETA_EXACT = 2        /* fixed point for the exact marginal of a
                                       coordinate of a uniformly random unit
                                       vector, density ~ (1 - x^2)^((d-3)/2) on
                                       [-1, 1] (P3, kwkr.cn news 555717, on the
                                       rotated coordinate's Beta law), float64
                                       quadrature, then float32 */
} tq_codebook_mode;

/* Byte layout of a cache page (P1, section "AoS 与 SoA:两种页内布局").
 * Both keep the page size block_size * num_kv_heads * slot bytes.
 *   AOS  [block_size][H][slot]: every (token, head) slot holds its K codes,
 *        K norm, V codes, V scale and V zero back to back (the default).
 *   SOA  a data region [block_size][H][K code bytes + V code bytes] followed
 *        by a meta region [H][3][block_size] of fp16: each head's K norms,
 *        then its V scales, then its V zeros.  With norm correction the
 *        stored K norm is |k| / |c|, c the token's centroid vector (P1,
 *        section "SoA 的另一项收益:把 norm correction 折进写入端"), so the
 *        decode multiplies by it directly.  3/4-bit key presets only. */
typedef enum {
  TQ_LAYOUT_AOS = 0,
  TQ_LAYOUT_SOA = 1
} tq_layout;

/* Values of the `sign_flip` argument of the init calls, i.e. the K rotation.
 * The Haar matrix is Q diag(sign(diag R)) from the Householder QR of a d x d
 * Gaussian matrix drawn from rot_seed (SplitMix64 uniforms, Box-Muller pairs,
 * row by row), rounded to float32: a uniformly random rotation (P3, kwkr.cn
 * news 555717, on the random orthogonal rotation; P1, section "为什么 vLLM
 * 选了 Hadamard 而不是随机正交矩阵").  With it the store computes
 * y = Q k / (|k| + 1e-8) (products summed in a fixed pairwise tree), the
 * decode q_rot = Q q, the dequantisation k = n Q^T c, and the decode runs on
 * the general kernel.  FP8 keys are never rotated. */
typedef enum {
  TQ_ROTATION_HADAMARD = 0,          /* pure Sylvester Hadamard                  */
  TQ_ROTATION_SIGNED_HADAMARD = 1,   /* seeded sign flips, then Hadamard (any other
                                        nonzero value means the same)           */
  TQ_ROTATION_HAAR = 2
} tq_rotation;

typedef struct tq_ctx tq_ctx;   /* opaque; only tq_set_decode_options changes it after init */

/* Which decode kernel runs (tq_decode_options.kernel).  AUTO picks by key
 * type and shape; a forced kernel is used where it applies to the shape and
 * AUTO's choice is taken otherwise.  All of them compute the same attention
 * within the same error bound; they differ in speed only. */
typedef enum {
  TQ_DECODE_KERNEL_AUTO = 0,
  TQ_DECODE_KERNEL_RING = 1,    /* per (sequence, kv head) workgroups streaming per-head slabs */
  TQ_DECODE_KERNEL_PAGE = 2,    /* per (sequence, split) workgroups streaming whole page rows */
  TQ_DECODE_KERNEL_STAGED = 3,  /* one wavefront per (split, sequence, kv head), staged rows */
  TQ_DECODE_KERNEL_DIRECT = 4,  /* one wavefront per (split, sequence, kv head), direct loads */
  TQ_DECODE_KERNEL_GENERAL = 5  /* fp32 vector-ALU kernel, no matrix cores: one wavefront per
                                   (256-token split, sequence, kv head); any head dim, up to 16
                                   query heads per kv head (the measure the matrix-core kernels
                                   are compared with) */
} tq_decode_kernel;

/* How a context's decode is planned.  The default (all zero) is AUTO with
 * reproducible results: for a fixed shape and options, identical inputs give
 * bit-identical outputs on every call.
 *   kernel          tq_decode_kernel
 *   dynamic_claims  nonzero: the ring kernel's wavefronts claim 16-token
 *                   slabs from a shared counter instead of taking fixed
 *                   interleaved shares.  It evens out wavefronts that run at
 *                   different rates (a few per cent faster on long
 *                   sequences), but which wavefront sums which slab, and so
 *                   the last bits of `out`, change from call to call (every
 *                   result stays within the same error bound).
 *   ring_waves      0 = by shape; 8 or 16 wavefronts per ring workgroup
 *   page_heads      0 = by shape; 1, 2 or 4 kv heads per page workgroup
 * These select between implementations of the same operation (P1, section
 * "读取内核"); they exist for reproducibility and for measurements. */
typedef struct {
  int kernel;
  int dynamic_claims;
  int ring_waves;
  int page_heads;
} tq_decode_options;

/* Solve the Lloyd-Max codebook for a rotated coordinate ~ N(0, 1/head_dim)
 * (P1, section "Lloyd-Max 的两个最优性条件"), derive the decision boundaries
 * as midpoints of the sorted float32 levels (P1, section "vLLM 内置的
 * Lloyd-Max 码本"), draw head_dim rotation signs from `rot_seed` with
 * SplitMix64 (sign_flip = 0 gives all +1, the pure Hadamard rotation of P1,
 * section "为什么 vLLM 选了 Hadamard 而不是随机正交矩阵"), and upload these
 * tables (about 200 bytes) plus a device error word to the current device.
 *
 *   ctx           out: host pointer receiving the new context
 *   preset        tq_preset
 *   head_dim      64, 128 or 256 (a power of two: Sylvester Hadamard)
 *   num_kv_heads  1..64 kv heads per token in the cache
 *   block_size    tokens per page: 16, 32, 64 or 128 (P1, section
 *                 "为什么 block_size 只有 16/32/64/128")
 *   rot_seed      seed of the sign flips (or of the Haar matrix)
 *   sign_flip     tq_rotation: 0 pure Hadamard, 2 Haar, other nonzero values
 *                 seeded signs
 *   codebook_mode tq_codebook_mode
 *   stream        stream for the table upload (the call synchronises it)
 * Allocates device memory (once per context); released by tq_destroy. */
tq_status tq_codebook_init(tq_ctx** ctx, int preset, int head_dim, int num_kv_heads,
                           int block_size, uint64_t rot_seed, int sign_flip,
                           int codebook_mode, void* stream);

/* tq_codebook_init with a page layout (tq_layout).  tq_codebook_init is this
 * call with TQ_LAYOUT_AOS.  TQ_LAYOUT_SOA with the FP8-key preset returns
 * TQ_ERR_UNSUPPORTED (its slot has no K norm to fold). */
tq_status tq_codebook_init_layout(tq_ctx** ctx, int preset, int head_dim, int num_kv_heads,
                                  int block_size, uint64_t rot_seed, int sign_flip,
                                  int codebook_mode, int layout, void* stream);

/* The context's page layout (tq_layout), -1 for a NULL context. */
int tq_layout_of(const tq_ctx* ctx);

/* Free the context and its device tables.  NULL is accepted. */
tq_status tq_destroy(tq_ctx* ctx);

/* Bytes of one slot: key bytes (head_dim for FP8, else ceil(d*b/8) + 2) plus
 * value bytes (ceil(d*4/8) + 4), rounded up to even -- 196 / 134 / 118 at
 * head_dim 128 (P1, section "从 slot_size 的三项算术开始"; P5, section
 * "三、TurboQuant").  Returns -1 for a NULL context. */
int64_t tq_slot_bytes(const tq_ctx* ctx);

/* Bytes of a cache of `num_blocks` pages: num_blocks * block_size *
 * num_kv_heads * slot (P1, section "页内寻址"). -1 on bad input. */
int64_t tq_cache_bytes(const tq_ctx* ctx, int64_t num_blocks);

/* Copy the context's tables to host memory (for cross-checks):
 *   centroids_host  float[2^bits]  levels, ascending (untouched for k8v4)
 *   midpoints_host  float[2^bits - 1] boundaries      (untouched for k8v4)
 *   signs_host      int8[head_dim]  +1 / -1
 * Any of the three may be NULL. */
tq_status tq_get_tables(const tq_ctx* ctx, float* centroids_host, float* midpoints_host,
                        int8_t* signs_host);

/* tq_store -- P1, sections "写入发生在 attention 之前" through "FP8 K 路径".
 *
 * For every token n < num_tokens and kv head h, with slot = slot_mapping[n]:
 * skip if slot < 0 (a padding token); otherwise write the slot bytes of
 * (k[n][h], v[n][h]) to cache page slot / block_size, row slot % block_size,
 * head h.  Slot bytes: [K codes | K norm fp16 | V codes | V scale fp16 |
 * V zero fp16] (P1, section "一个 slot 的字节图"), or [K e4m3 | V ...] for
 * k8v4.  K codes come from the fp32 contract: norm by a fixed pairwise tree,
 * y = FWHT(s * k) * (1 / (|k| + 1e-8)) * rsqrt(d) with butterfly stages
 * h = 1, 2, ..., d/2, code = #{boundaries <= y}; V codes from the per-vector
 * min/max uniform quantiser with round-half-up (P1, section "V 的 min/max
 * 均匀量化").  Every float operation is a single IEEE binary32 operation
 * rounded to nearest even, so the bytes are reproducible bit for bit.
 *
 *   k, v             device, bf16 [num_tokens][kv_token_stride elements],
 *                    head h at element offset h * head_dim; 16-byte aligned,
 *                    kv_token_stride a multiple of 8 and >= H * head_dim
 *   slot_mapping     device, int64 [num_tokens]
 *   num_tokens       0 is a no-op returning TQ_OK (P1, same section)
 *   cache            device, uint8 [num_blocks][block_size][H][slot], 16-byte aligned
 *   num_blocks       pages in the cache; a slot >= num_blocks * block_size is
 *                    skipped and sets the device error word (bit 0)
 */
tq_status tq_store(const tq_ctx* ctx, const void* k, const void* v, int64_t kv_token_stride,
                   const int64_t* slot_mapping, int64_t num_tokens, uint8_t* cache,
                   int64_t num_blocks, void* stream);

/* Workspace bytes tq_decode needs for this shape (split-KV partials: P1,
 * section "内存:workspace 预分配").  0 when the shape needs none (every
 * sequence is combined inside one workgroup) or on bad input. */
size_t tq_decode_workspace_bytes(const tq_ctx* ctx, int batch, int num_q_heads,
                                 int max_seq_len);

/* tq_decode -- P1, sections "读取内核" through "数值精度:累加器为什么是 fp32".
 *
 * For sequence b < batch and query head hq (kv head g = hq / (Hq / H)),
 * attention of q[b][hq] over tokens t < seq_lens[b], whose slots are row
 * t % block_size of page block_table[b][t / block_size]:
 *   MSE K:  q_rot = R q once; score_t = sm_scale * n_t * (q_rot . c_t), where
 *           c_t are the centroids of the token's codes and n_t its stored
 *           norm, divided by sqrt(sum c_t^2 + 1e-16) (norm correction, P1,
 *           section "norm correction");
 *   FP8 K:  score_t = sm_scale * (q . e4m3(k_t)), q not rotated;
 *   V:      v_t = code * scale16 + zero16;
 *   out = softmax(score) . v, as split-KV online softmax with fp32
 *   accumulators and a log-sum-exp combine pass.  A sequence with
 *   seq_lens[b] == 0 gives zeros.
 *
 *   q              device, bf16 [batch][num_q_heads][head_dim], 16-byte aligned
 *   cache          device, as written by tq_store, with `num_blocks` pages
 *   block_table    device, int32 [batch][max_blocks_per_seq]; a page id outside
 *                  [0, num_blocks) is skipped and sets device error bit 1
 *   seq_lens       device, int32 [batch], each in [0, max_seq_len]
 *   max_seq_len    host upper bound of seq_lens (sizes the grid; the device
 *                  lengths are read by the kernels, never by the host);
 *                  max_blocks_per_seq * block_size must cover it
 *   sm_scale       softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   out            device, [batch][num_q_heads][head_dim], bf16 when
 *                  out_is_fp32 == 0, fp32 otherwise
 *   workspace      device, >= tq_decode_workspace_bytes(...) bytes, 256-byte
 *                  aligned; contents need no initialisation; calls that
 *                  share a workspace must not overlap; may be NULL when
 *                  that size is 0
 *
 * More than 16 query heads per kv head run on the matrix-core kernels
 * (head_dim 128, block_size a multiple of 16) in passes of 16 query heads
 * (8 on the split page), each pass reading the cache; other shapes with
 * more than 16 return TQ_ERR_UNSUPPORTED.  Head dims 64 and 256 run on a
 * matrix-core kernel of their own on the slotted page (block_size a multiple
 * of 16, any number of query heads per kv head, in passes of 16), on the
 * general fp32 kernel (at most 16) on the split page.
 *
 * Reproducibility.  The plan (kernel, split count, order of the fp32 sums)
 * depends only on the shape arguments and the context's decode options, so
 * with the default options identical inputs give bit-identical outputs.
 * tq_decode_workspace_bytes plans with the same options: size the workspace
 * after the last tq_set_decode_options.
 */
tq_status tq_decode(const tq_ctx* ctx, const void* q, const uint8_t* cache, int64_t num_blocks,
                    const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                    int batch, int num_q_heads, int max_seq_len, float sm_scale, void* out,
                    int out_is_fp32, void* workspace, size_t workspace_bytes, void* stream);

/* tq_decode_noalloc -- tq_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, kernels and results (bit for bit,
 * with the same decode options), with the split partials kept in the
 * library's own scratch array instead of a caller workspace.
 *
 * The array is a file-scope device array of tq_decode_noalloc_max_bytes()
 * bytes (32 MiB); each GPU the library runs on holds its own copy until the
 * process ends.  A shape whose plan needs more scratch than that returns
 * TQ_ERR_WORKSPACE before anything is enqueued.  The call allocates nothing
 * and synchronises nothing.  Every call on a GPU shares that GPU's array,
 * which keeps the last call's partials: calls that overlap on one GPU (two
 * streams, or two host threads) race and give wrong results.  The partials
 * need no initialisation.  Arguments and errors otherwise as tq_decode. */
tq_status tq_decode_noalloc(const tq_ctx* ctx, const void* q, const uint8_t* cache,
                            int64_t num_blocks, const int32_t* block_table, int max_blocks_per_seq,
                            const int32_t* seq_lens, int batch, int num_q_heads, int max_seq_len,
                            float sm_scale, void* out, int out_is_fp32, void* stream);

/* Bytes of the scratch array tq_decode_noalloc uses (the largest workspace
 * it accepts). */
size_t tq_decode_noalloc_max_bytes(void);

/* tq_dequant -- P1, section "反量化 kernel:_tq_full_dequant_kv".
 *
 * Expand the first seq_len tokens of one sequence back into K and V vectors
 * of the original space (the input of the pages' long-chunk continuation
 * prefill, section "续写 prefill:小 chunk 走 decode,大 chunk 走反量化"):
 * token t, head h reads slot row t % block_size of page block_table_row[t /
 * block_size] and writes
 *   MSE K:  k = n * R^T c (c the centroids of the codes, n the stored norm,
 *           divided by sqrt(sum c^2 + 1e-16) on the slotted page; R^T the
 *           inverse of the store's rotation, applied as butterflies);
 *   FP8 K:  k = e4m3(byte);
 *   V:      v = code * scale16 + zero16.
 *
 *   cache            device, as written by tq_store, `num_blocks` pages
 *   block_table_row  device, int32 [max_blocks]; max_blocks * block_size must
 *                    cover seq_len.  A page id outside [0, num_blocks) writes
 *                    zeros for its tokens and sets device error bit 1
 *   k_out, v_out     device, [seq_len][num_kv_heads][head_dim], bf16 (round to
 *                    nearest even) when out_is_fp32 == 0, fp32 otherwise;
 *                    16-byte aligned
 * seq_len 0 is a no-op.  Allocates nothing; asynchronous on `stream`. */
tq_status tq_dequant(const tq_ctx* ctx, const uint8_t* cache, int64_t num_blocks,
                     const int32_t* block_table_row, int max_blocks, int seq_len, void* k_out,
                     void* v_out, int out_is_fp32, void* stream);

/* Workspace bytes tq_decode_continuation needs: the decode's workspace for
 * q_len requests of length up to seq_len, plus the synthetic lengths and the
 * expanded block table (q_len * (max_blocks + 1) int32).  0 on bad input. */
size_t tq_continuation_workspace_bytes(const tq_ctx* ctx, int q_len, int num_q_heads, int seq_len,
                                       int max_blocks);

/* tq_decode_continuation -- P1, section "续写 prefill:小 chunk 走 decode,大
 * chunk 走反量化" (the short-chunk path, for chunks of up to 128 queries).
 *
 * Causal attention of a chunk of q_len new queries of one sequence whose
 * seq_len tokens (the cached_len = seq_len - q_len earlier ones and the
 * chunk's own, already stored with tq_store) are in the cache: query i
 * attends to tokens [0, cached_len + i + 1).  Each query is run as a decode
 * request of that length over the sequence's block-table row, which is how
 * the causal mask arises without a mask tensor.
 *
 *   q                [q_len][num_q_heads][head_dim] bf16, 16-byte aligned
 *   block_table_row  device, int32 [max_blocks]; max_blocks * block_size >= seq_len
 *   seq_len          cached tokens plus q_len; q_len in [1, seq_len]
 *   out              [q_len][num_q_heads][head_dim], bf16 or fp32 (out_is_fp32)
 *   workspace        device, >= tq_continuation_workspace_bytes(...), 256-byte
 *                    aligned; calls that share it must not overlap
 * Errors as tq_decode.  Allocates nothing; asynchronous on `stream`. */
tq_status tq_decode_continuation(const tq_ctx* ctx, const void* q, const uint8_t* cache,
                                 int64_t num_blocks, const int32_t* block_table_row, int max_blocks,
                                 int seq_len, int q_len, int num_q_heads, float sm_scale, void* out,
                                 int out_is_fp32, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Read the context's sticky device error word once the work enqueued on
 * `stream` (a hipStream_t as void*, NULL = the null stream) has finished:
 * the call synchronises that stream only, not the device.
 * bit 0 = a store slot beyond the cache, bit 1 = a page id beyond the cache,
 * bit 2 = a seq_lens entry outside [0, max_seq_len] (clamped).
 * `clear` nonzero resets it to 0 afterwards (on the same stream, before
 * returning).  Kernels of this context running on other streams may set the
 * word while it is read. */
tq_status tq_get_device_error(const tq_ctx* ctx, int32_t* code_host, int clear, void* stream);

/* Set the context's decode options (see tq_decode_options); NULL restores
 * the defaults.  Later tq_decode, tq_decode_workspace_bytes and
 * tq_decode_continuation calls use them.  Not to be called while another
 * host thread plans a decode on the same context. */
tq_status tq_set_decode_options(tq_ctx* ctx, const tq_decode_options* opts);

/* Copy the context's decode options to *opts. */
tq_status tq_get_decode_options(const tq_ctx* ctx, tq_decode_options* opts);

/* ---- host-only helpers (no device needed; for checks and tooling) ------- */

/* The float32 codebook tq_codebook_init would build: 2^bits ascending levels
 * and the 2^bits - 1 midpoints of neighbouring levels.  bits 1..4. */
tq_status tq_host_codebook(int head_dim, int bits, int codebook_mode, float* centroids_host,
                           float* midpoints_host);

/* The head_dim x head_dim float32 Haar matrix (row-major) that
 * tq_codebook_init draws for TQ_ROTATION_HAAR from rot_seed. */
tq_status tq_host_haar_matrix(uint64_t rot_seed, int head_dim, float* q_host);

/* The head_dim rotation signs (+1/-1) tq_codebook_init would draw. */
tq_status tq_host_rotation_signs(uint64_t rot_seed, int head_dim, int sign_flip,
                                 int8_t* signs_host);

/* Slot bytes of a preset at a head_dim (196 / 134 / 118 at 128), -1 if unsupported. */
int64_t tq_host_slot_bytes(int preset, int head_dim);

/* Static description of a status code. */
const char* tq_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_MI355X_H */
