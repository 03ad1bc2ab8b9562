// launch.h -- internal kernel-launch interface of libpagedkv.so (host side).
// Arguments arrive here already validated by the C-ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// A HIP launch on gfx950 covers at most 2^32 - 1 work-items in a dimension
// (workgroups times threads per workgroup); every grid here is 1-D.
constexpr int64_t kMaxGridItems = 0xFFFFFFFFll;
inline bool grid_fits(int64_t workgroups, int threads) {
  return workgroups >= 0 && workgroups <= kMaxGridItems / threads;
}

struct KvAppendArgs {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_new_lens;
  int32_t B, T_new, Hkv, D, block_size, max_blocks_per_seq, num_blocks;
};
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);

// Whole-block copies between pool blocks (copy on write of shared blocks).
struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* src_blocks;
  const int32_t* dst_blocks;
  int32_t n_pairs, Hkv, D, block_size, num_blocks;
};
hipError_t launch_kv_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// kv_append with the rotary embedding of the new keys (and queries), D == 64.
struct RopeAppendArgs {
  void* k_cache;
  void* v_cache;
  void* q;  // [T_new][Hq][D], rotated in place, or nullptr (then Hq == 0)
  const void* k_new;
  const void* v_new;
  const float* rope_cos;  // [max_position][D/2]
  const float* rope_sin;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_new_lens;
  int32_t max_position, B, T_new, Hq, Hkv, block_size, max_blocks_per_seq, num_blocks;
};
hipError_t launch_kv_append_rope(const RopeAppendArgs& a, hipStream_t stream);

// Decode work decomposition (see decode.hip).
enum DecodeMode : int { kWhole = 0, kFixed = 1, kAuto = 2 };

// Wavefronts of the automatic split: 8 per CU of a 256-CU MI355X, or, for
// more than 3/4 as many (sequence, KV head) streams, a quarter of that plus
// one per stream (the split makes at most that many pieces, one per
// wavefront), rounded up to whole workgroups of 4.
#ifndef PKV_AUTO_WAVES
#define PKV_AUTO_WAVES 2048
#endif
constexpr int kAutoWaves = PKV_AUTO_WAVES;
inline int64_t auto_waves(int64_t streams) {
  const int64_t w = streams <= 3 * kAutoWaves / 4 ? kAutoWaves : kAutoWaves / 4 + streams;
  return (w + 3) / 4 * 4;
}
// Largest batch the automatic split handles (per-sequence prefix in LDS).
constexpr int kAutoMaxBatch = 4096;

// One split record: normalised partial output for the 4 query heads of a
// KV group (4 x 64 fp32) followed, in a separate array, by (m, l) per head.
constexpr int kRecordFloats = 4 * 64;
// Split counters (one uint32 per (sequence, KV head) stream) occupy a fixed
// region at the start of the workspace, whatever the call's shapes, so a
// workspace zero-filled once stays valid for every later call.
constexpr int kMaxSplitStreams = 32768;
// Counters of different streams sit this many uint32 apart, so that
// concurrent device-scope atomics on different streams do not share a line.
#ifndef PKV_COUNTER_STRIDE
#define PKV_COUNTER_STRIDE 32
#endif
constexpr int kCounterStride = PKV_COUNTER_STRIDE;
// Split records addressable with 32-bit byte offsets (1 KB of output each).
constexpr int kMaxRecords = (1 << 21) - 1;
constexpr size_t kCounterBytes = (size_t)kMaxSplitStreams * kCounterStride * 4;

// Decode plan (partition PKV_PARTITION_PLANNED), after the split records of
// the automatic split: a header (with the piece bound), the per-sequence
// prefix of pieces, the (clamped) context lengths it was made for, and per
// wavefront its piece (b, g, first and end block, context length, the
// stream's piece count and first record; b = -1: no piece) and the block ids
// of its first 64 blocks.  Written by paged_attention_decode_plan.
constexpr int kPlanHeaderInts = 16;
constexpr int kPlanCtxOffset = kPlanHeaderInts + kAutoMaxBatch + 1;
constexpr int kPlanWaveOffset = kPlanCtxOffset + kAutoMaxBatch;
constexpr int kPlanWaveInts = 8 + 64;
constexpr int kPlanMagic = 0x504c414e;
inline size_t plan_bytes(int64_t streams) {
  return ((size_t)kPlanWaveOffset + (size_t)auto_waves(streams) * kPlanWaveInts) * 4;
}

struct DecodeArgs {
  void* out;
  int32_t out_f32;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t B, Hq, Hkv, max_blocks_per_seq, num_blocks, max_context_len;
  float scale;
  int32_t mode;            // DecodeMode
  int32_t part_blocks;     // kFixed: blocks per partition
  int32_t parts_max;       // kFixed: partitions per stream upper bound
  float* ws_o;             // records x kRecordFloats
  float* ws_ml;            // records x 4 heads x (m, l)
  uint32_t* ws_count;      // B x Hkv split counters, zero between calls
  // kAuto only: also store one new token per sequence ([B][Hkv][D] rows)
  // into the pools before attending (both null: plain decode)
  const void* k_new;
  const void* v_new;
  // kAuto only: the plan region of the workspace (null: none); with
  // write_plan the launch computes the plan instead of attending
  int32_t* plan;
  int32_t write_plan;
};
size_t decode_records(int32_t mode, int32_t B, int32_t Hkv, int32_t parts_max);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  int32_t out_f32;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  int32_t B, T_q, Hq, Hkv, max_blocks_per_seq, num_blocks, max_q_len;
  float scale;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Workgroups launch_prefill would start for these arguments (one per
// 32-row query tile of the longest prompt, sequence and KV head).
int64_t prefill_grid_size(int32_t max_q_len, int32_t T_q, int32_t B, int32_t Hkv);

// Plain streaming read of whole (block, KV head) chunks of both pools for a
// list of block ids (probe.hip); `sink` receives stream_blocks_sink_words()
// words.
int64_t stream_blocks_sink_words();
// MFMA issue-rate probe (probe.hip): kProbeWaves wavefronts of bf16 MFMA
// chains, `iters` rounds each; flops of one launch, and the launch itself.
// `sink` receives stream_blocks_sink_words() floats.
int64_t mfma_probe_flops(int32_t iters);
hipError_t launch_mfma_probe(int32_t iters, float* sink, hipStream_t stream);
hipError_t launch_stream_blocks(const void* k_cache, const void* v_cache, const int32_t* block_ids,
                                int32_t n_ids, int32_t Hkv, int32_t D, int32_t block_size,
                                int32_t num_blocks, uint32_t* sink, hipStream_t stream);

}  // namespace pkv
