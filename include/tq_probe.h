/*
 * tq_probe.h -- streaming-read probes of the MI355X library (measurement
 * helpers, not part of the method).
 *
 * Each probe reads a device buffer once, start to end, with one load form of
 * the store and decode kernels, so the decode's achieved bytes per second can
 * be compared with what this part reads with that form (the pages call the
 * decode bound by its KV reads: P1, "vLLM 源码完全拆解(十九):TurboQuant KV Cache
 * 量化", section "K 的归一化与旋转为什么放在 kernel 外面").
 */
#ifndef TQ_PROBE_H
#define TQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_PROBE_REGS = 0,      /* 16-byte vector loads into registers           */
  TQ_PROBE_REGS_NT = 1,   /* the same, non-temporal                        */
  TQ_PROBE_LDS = 2,       /* 16-byte buffer loads that write LDS directly  */
  TQ_PROBE_LDS_NT = 3     /* the same, non-temporal                        */
} tq_probe_mode;

/* Words of the sink buffer tq_probe_read writes for a buffer of `bytes`
 * (one per thread of its grid), or -1 if `bytes` is below one step (32 KB). */
int64_t tq_probe_sink_words(int64_t bytes);

/* Enqueue one read of the first floor(bytes / 32 KB) * 32 KB bytes of `src`
 * (device, 16-byte aligned) on `stream` (a hipStream_t as void*; NULL = the
 * null stream) with the load form `mode`.  `sink` (device, uint32 [
 * tq_probe_sink_words(bytes)]) receives a fold of what was read, so no load
 * is dead code.  Returns 0, -1 on a bad argument, -3 on a misaligned `src`,
 * -5 if the launch failed.  Allocates nothing; does not synchronise. */
int tq_probe_read(int mode, const void* src, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */
