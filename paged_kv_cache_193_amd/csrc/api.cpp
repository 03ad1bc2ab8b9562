// api.cpp -- the extern "C" entry points of libpagedkv.so declared in
// include/pagedkv.h.  Every argument is validated on the host before any HIP
// call (so invalid arguments never reach the device); then the work is
// enqueued on the caller's stream and the launch status is returned.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <atomic>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "errors.h"
#include "launch.h"
#include "pagedkv.h"

namespace {

using pkv::fail;

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kD = 64, kBS = 16, kGroup = 4;

// Decode mode and split geometry for the given arguments.
struct DecodePlan {
  int mode, part_blocks, parts_max;
  bool planned;        // PKV_PARTITION_PLANNED: the plan region follows the records
  size_t records, bytes, plan_offset;
};

int plan_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                int32_t max_context_len, int32_t partition_size, DecodePlan* plan) {
  if (B < 0) return fail(PKV_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(PKV_ERR_INVALID_ARG, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (D != kD) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not implemented (64 only)", D);
  if (block_size != kBS)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not implemented (16 only)", block_size);
  if (Hq != kGroup * Hkv)
    return fail(PKV_ERR_UNSUPPORTED, "GQA group %d not implemented (Hq == 4*Hkv only)", Hq / Hkv);
  if (max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len must be >= 0 (got %d)", max_context_len);
  plan->mode = pkv::kWhole;
  plan->part_blocks = 0;
  plan->parts_max = 1;
  plan->planned = partition_size == PKV_PARTITION_PLANNED;
  plan->plan_offset = 0;
  if (partition_size == PKV_PARTITION_AUTO || plan->planned) {
    if (B > pkv::kAutoMaxBatch)
      return fail(PKV_ERR_UNSUPPORTED, "automatic split handles B <= %d (got %d)",
                  pkv::kAutoMaxBatch, B);
    plan->mode = pkv::kAuto;
  } else if (partition_size > 0) {
    if (partition_size % block_size != 0)
      return fail(PKV_ERR_UNSUPPORTED, "partition_size %d is not a multiple of block_size %d",
                  partition_size, block_size);
    const int parts = (int)(((int64_t)max_context_len + partition_size - 1) / partition_size);
    if (parts > 1) {
      plan->mode = pkv::kFixed;
      plan->part_blocks = partition_size / block_size;
      plan->parts_max = parts;
    }
  } else if (partition_size != PKV_PARTITION_NONE) {
    return fail(PKV_ERR_INVALID_ARG, "partition_size %d: use > 0, 0 (none) or -1 (auto)",
                partition_size);
  }
  plan->records = pkv::decode_records(plan->mode, B, Hkv, plan->parts_max);
  plan->bytes = 0;
  if (plan->records) {
    if ((int64_t)B * Hkv > pkv::kMaxSplitStreams)
      return fail(PKV_ERR_UNSUPPORTED, "split decode handles B*Hkv <= %d streams (got %lld)",
                  pkv::kMaxSplitStreams, (long long)B * Hkv);
    // the kernels address the records with 32-bit byte offsets
    if (plan->records > (size_t)pkv::kMaxRecords)
      return fail(PKV_ERR_UNSUPPORTED,
                  "split decode needs %zu partial records, at most %d are supported: use a "
                  "larger partition_size",
                  plan->records, pkv::kMaxRecords);
    // counter region, then records (normalised outputs) and their (m, l) pairs
    plan->bytes = pkv::kCounterBytes + plan->records * (pkv::kRecordFloats + 8) * sizeof(float);
  }
  if (plan->planned) {
    plan->plan_offset = (plan->bytes + 255) / 256 * 256;
    plan->bytes = plan->plan_offset + pkv::plan_bytes((int64_t)B * Hkv);
  }
  return PKV_OK;
}

// PAGEDKV_DEBUG=1 in the environment: before a launch, copy the call's
// tables and lengths to the host (on its stream, then wait for them) and
// validate them with pagedkv_check_tables.  Read at every call, so a process
// can switch it on and off.  Skipped while the stream is being captured into
// a graph (a capture cannot wait for a copy).
bool debug_enabled() {
  const char* v = getenv("PAGEDKV_DEBUG");
  return v && v[0] == '1' && v[1] == 0;
}

int debug_check(const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_lens,
                int32_t B, int32_t T, int32_t max_blocks_per_seq, int32_t num_blocks,
                int32_t kind, hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return PKV_OK;
  std::vector<int32_t> tables((size_t)B * max_blocks_per_seq), lens(B), cu;
  hipError_t e = hipMemcpyAsync(tables.data(), block_tables, tables.size() * 4,
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(lens.data(), context_lens, lens.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && cu_lens) {
    cu.resize((size_t)B + 1);
    e = hipMemcpyAsync(cu.data(), cu_lens, cu.size() * 4, hipMemcpyDeviceToHost, stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "PAGEDKV_DEBUG copy of tables and lengths");
  return pagedkv_check_tables(tables.data(), lens.data(), cu_lens ? cu.data() : nullptr, B, T,
                              max_blocks_per_seq, num_blocks, kBS, kind);
}

}  // namespace

extern "C" {


int kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
              const int32_t* block_tables, const int32_t* context_lens,
              const int32_t* cu_new_lens, int32_t B, int32_t T_new, int32_t Hkv, int32_t D,
              int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
              void* stream) {
  if (B < 0 || T_new < 0)
    return fail(PKV_ERR_INVALID_ARG, "B (%d) and T_new (%d) must be >= 0", B, T_new);
  if (B == 0 || T_new == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (Hkv <= 0 || D <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "Hkv, D, block_size, max_blocks_per_seq, num_blocks must be > 0");
  if (D % 8 != 0) return fail(PKV_ERR_UNSUPPORTED, "D %d is not a multiple of 8", D);
  if (!cu_new_lens && T_new != B)
    return fail(PKV_ERR_INVALID_ARG, "cu_new_lens is NULL but T_new (%d) != B (%d)", T_new, B);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID_ARG, "pools and new rows must be 16-byte aligned");
  if (!pkv::grid_fits(((int64_t)T_new * 2 * Hkv * (D / 8) + 255) / 256, 256))
    return fail(PKV_ERR_UNSUPPORTED, "too many new rows for one launch (2^32 - 1 work-items)");
  if (debug_enabled()) {
    const int rc = debug_check(block_tables, context_lens, cu_new_lens, B, T_new,
                               max_blocks_per_seq, num_blocks, PKV_CHECK_APPEND,
                               (hipStream_t)stream);
    if (rc != PKV_OK) return rc;
  }
  pkv::KvAppendArgs a{k_cache, v_cache, k_new, v_new, block_tables, context_lens, cu_new_lens,
                      B, T_new, Hkv, D, block_size, max_blocks_per_seq, num_blocks};
  return hip_status(pkv::launch_kv_append(a, (hipStream_t)stream), "kv_append launch");
}

int kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks,
                   const int32_t* dst_blocks, int32_t n_pairs, int32_t Hkv, int32_t D,
                   int32_t block_size, int32_t num_blocks, void* stream) {
  if (n_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "n_pairs must be >= 0 (got %d)", n_pairs);
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "Hkv, D, block_size, num_blocks must be > 0");
  if (D % 8 != 0) return fail(PKV_ERR_UNSUPPORTED, "D %d is not a multiple of 8", D);
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  if (!pkv::grid_fits(((int64_t)n_pairs * 2 * Hkv * block_size * (D / 8) + 255) / 256, 256))
    return fail(PKV_ERR_UNSUPPORTED, "too many block copies for one launch (2^32 - 1 work-items)");
  pkv::CopyBlocksArgs a{k_cache, v_cache, src_blocks, dst_blocks, n_pairs, Hkv, D, block_size,
                        num_blocks};
  return hip_status(pkv::launch_kv_copy_blocks(a, (hipStream_t)stream), "kv_copy_blocks launch");
}

int kv_append_rope(void* k_cache, void* v_cache, void* q, const void* k_new, const void* v_new,
                   const float* rope_cos, const float* rope_sin, int32_t max_position,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* cu_new_lens, int32_t B, int32_t T_new, int32_t Hq,
                   int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks_per_seq,
                   int32_t num_blocks, void* stream) {
  if (B < 0 || T_new < 0)
    return fail(PKV_ERR_INVALID_ARG, "B (%d) and T_new (%d) must be >= 0", B, T_new);
  if (B == 0 || T_new == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !rope_cos || !rope_sin || !block_tables ||
      !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (Hkv <= 0 || D <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      max_position <= 0)
    return fail(PKV_ERR_INVALID_ARG,
                "Hkv, D, block_size, max_blocks_per_seq, num_blocks, max_position must be > 0");
  if (q && Hq <= 0) return fail(PKV_ERR_INVALID_ARG, "Hq must be > 0 when q is given (got %d)", Hq);
  if (D != kD) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not implemented (64 only)", D);
  if (!cu_new_lens && T_new != B)
    return fail(PKV_ERR_INVALID_ARG, "cu_new_lens is NULL but T_new (%d) != B (%d)", T_new, B);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
      !aligned16(rope_cos) || !aligned16(rope_sin) || (q && !aligned16(q)))
    return fail(PKV_ERR_INVALID_ARG, "pools, rows and rope tables must be 16-byte aligned");
  const int32_t hq = q ? Hq : 0;
  if (!pkv::grid_fits(((int64_t)T_new * (hq + 2 * (int64_t)Hkv) * 4 + 255) / 256, 256))
    return fail(PKV_ERR_UNSUPPORTED, "too many new rows for one launch (2^32 - 1 work-items)");
  if (debug_enabled()) {
    const int rc = debug_check(block_tables, context_lens, cu_new_lens, B, T_new,
                               max_blocks_per_seq, num_blocks, PKV_CHECK_APPEND,
                               (hipStream_t)stream);
    if (rc != PKV_OK) return rc;
  }
  pkv::RopeAppendArgs a{k_cache, v_cache, q, k_new, v_new, rope_cos, rope_sin, block_tables,
                        context_lens, cu_new_lens, max_position, B, T_new, hq, Hkv, block_size,
                        max_blocks_per_seq, num_blocks};
  return hip_status(pkv::launch_kv_append_rope(a, (hipStream_t)stream), "kv_append_rope launch");
}

size_t paged_attention_decode_workspace_size(int32_t B, int32_t Hq, int32_t D,
                                             int32_t max_context_len, int32_t partition_size) {
  // The split geometry depends on the KV head count and the block size; this
  // build implements one GQA group size and one block size, so both follow
  // from the arguments (a call with any other Hkv or block_size is rejected).
  if (Hq <= 0 || Hq % kGroup != 0) {
    fail(PKV_ERR_UNSUPPORTED, "Hq %d is not a multiple of the GQA group %d", Hq, kGroup);
    return 0;
  }
  DecodePlan plan;
  if (plan_decode(B, Hq, Hq / kGroup, D, kBS, max_context_len, partition_size, &plan) != PKV_OK)
    return 0;
  return plan.bytes;
}

}  // extern "C"

namespace {

// Validation shared by the decode entry points: fills `a` (the launch
// arguments) and returns PKV_OK, or returns a status with the error text set.
// *nothing becomes true when B == 0 (nothing to launch).
int prepare_decode(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* block_tables,
                   const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                   int32_t max_context_len, float scale, int32_t partition_size,
                   void* workspace, size_t workspace_bytes, pkv::DecodeArgs* a, bool* nothing) {
  DecodePlan plan;
  int rc = plan_decode(B, Hq, Hkv, D, block_size, max_context_len, partition_size, &plan);
  if (rc != PKV_OK) return rc;
  *nothing = B == 0;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (out_dtype != PKV_OUT_BF16 && out_dtype != PKV_OUT_F32)
    return fail(PKV_ERR_INVALID_ARG, "out_dtype %d is neither PKV_OUT_BF16 nor PKV_OUT_F32", out_dtype);
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be > 0");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "out, q and the pools must be 16-byte aligned");
  if (plan.bytes > 0) {
    if (!workspace || workspace_bytes < plan.bytes)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PKV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  // one wavefront per (sequence, KV head, partition) unit, four per workgroup
  if (!pkv::grid_fits(((int64_t)B * Hkv * plan.parts_max + 3) / 4, 256))
    return fail(PKV_ERR_UNSUPPORTED,
                "too many (sequence, head, partition) units for one launch (2^32 - 1 work-items)");
  *a = pkv::DecodeArgs{};
  a->out = out;
  a->out_f32 = out_dtype == PKV_OUT_F32;
  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->B = B;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->num_blocks = num_blocks;
  a->max_context_len = max_context_len;
  a->scale = scale;
  a->mode = plan.mode;
  a->part_blocks = plan.part_blocks;
  a->parts_max = plan.parts_max;
  float* rec = plan.bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                     pkv::kCounterBytes)
                         : nullptr;
  a->ws_count = plan.bytes ? static_cast<uint32_t*>(workspace) : nullptr;
  a->ws_o = rec;
  a->ws_ml = plan.bytes ? rec + plan.records * pkv::kRecordFloats : nullptr;
  a->k_new = nullptr;
  a->v_new = nullptr;
  a->plan = plan.planned ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                       plan.plan_offset)
                         : nullptr;
  a->write_plan = 0;
  return PKV_OK;
}

// ---- Scratch of paged_attention_decode_noalloc (for callers that cannot
// allocate): the split's counters and records in a file-scope device array
// instead of a caller workspace.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;              // device address of this device's scratch
  std::atomic<int> cleared{0};      // the counter region has been zeroed
};
ScratchSlot g_scratch[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// This device's scratch address; on the first call on a device the split
// counters (which every decode call leaves at zero again) are zeroed on
// `stream` by a fill kernel first.
int noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "paged_attention_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] {
    s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess && !s.ptr) s.err = hipErrorInvalidSymbol;
  });
  if (s.err != hipSuccess) return hip_status(s.err, "hipGetSymbolAddress(scratch)");
  if (s.cleared.exchange(1) == 0) {
    const int64_t words = (int64_t)pkv::kCounterBytes / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3(1024), dim3(256), 0, stream,
                       static_cast<uint32_t*>(s.ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) {
      s.cleared.store(0);
      return hip_status(e, "paged_attention_decode_noalloc: scratch fill");
    }
  }
  *out = s.ptr;
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_attention_decode_noalloc(void* out, int32_t out_dtype, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, int32_t max_context_len, float scale,
                                   int32_t partition_size, void* stream) {
  if (partition_size == PKV_PARTITION_PLANNED)
    return fail(PKV_ERR_UNSUPPORTED,
                "paged_attention_decode_noalloc: a planned split reads its plan from a caller "
                "workspace; use PKV_PARTITION_AUTO");
  DecodePlan plan;
  int rc = plan_decode(B, Hq, Hkv, D, block_size, max_context_len, partition_size, &plan);
  if (rc != PKV_OK) return rc;
  if (plan.bytes > kNoAllocScratchBytes)
    return fail(PKV_ERR_UNSUPPORTED,
                "paged_attention_decode_noalloc: the split needs %zu bytes of scratch, the "
                "static scratch holds %zu (use a larger partition_size or "
                "paged_attention_decode with a workspace)",
                plan.bytes, kNoAllocScratchBytes);
  pkv::DecodeArgs a;
  bool nothing = false;
  // validate everything before the first HIP call
  rc = prepare_decode(out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv,
                      D, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                      partition_size, reinterpret_cast<void*>(256), kNoAllocScratchBytes, &a,
                      &nothing);  // a stand-in workspace address: checks only, no launch
  if (rc != PKV_OK || nothing) return rc;
  if (debug_enabled()) {
    const int rc2 = debug_check(block_tables, context_lens, nullptr, B, 0, max_blocks_per_seq,
                                num_blocks, PKV_CHECK_READ, (hipStream_t)stream);
    if (rc2 != PKV_OK) return rc2;
  }
  void* ws = nullptr;
  if (plan.bytes > 0) {
    rc = noalloc_scratch((hipStream_t)stream, &ws);
    if (rc != PKV_OK) return rc;
  }
  rc = prepare_decode(out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv,
                      D, block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                      partition_size, ws, ws ? kNoAllocScratchBytes : 0, &a, &nothing);
  if (rc != PKV_OK) return rc;
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream),
                    "paged_attention_decode_noalloc launch");
}

int paged_attention_decode(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t max_context_len, float scale,
                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                           void* stream) {
  pkv::DecodeArgs a;
  bool nothing = false;
  const int rc = prepare_decode(out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, B,
                                Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks,
                                max_context_len, scale, partition_size, workspace,
                                workspace_bytes, &a, &nothing);
  if (rc != PKV_OK || nothing) return rc;
  if (debug_enabled()) {
    const int rc2 = debug_check(block_tables, context_lens, nullptr, B, 0, max_blocks_per_seq,
                                num_blocks, PKV_CHECK_READ, (hipStream_t)stream);
    if (rc2 != PKV_OK) return rc2;
  }
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream), "paged_attention_decode launch");
}

int paged_attention_decode_append(void* out, int32_t out_dtype, const void* q, void* k_cache,
                                  void* v_cache, const void* k_new, const void* v_new,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t block_size, int32_t max_blocks_per_seq,
                                  int32_t num_blocks, int32_t max_context_len, float scale,
                                  int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  pkv::DecodeArgs a;
  bool nothing = false;
  const int rc = prepare_decode(out, out_dtype, q, k_cache, v_cache, block_tables, context_lens, B,
                                Hq, Hkv, D, block_size, max_blocks_per_seq, num_blocks,
                                max_context_len, scale, partition_size, workspace,
                                workspace_bytes, &a, &nothing);
  if (rc != PKV_OK || nothing) return rc;
  if (!k_new || !v_new) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_ERR_INVALID_ARG, "new rows must be 16-byte aligned");
  if (debug_enabled()) {
    const int rc2 = debug_check(block_tables, context_lens, nullptr, B, B, max_blocks_per_seq,
                                num_blocks, PKV_CHECK_APPEND, (hipStream_t)stream);
    if (rc2 != PKV_OK) return rc2;
  }
  if (a.mode == pkv::kAuto) {  // one launch: the decode kernel stores the new rows
    a.k_new = k_new;
    a.v_new = v_new;
    return hip_status(pkv::launch_decode(a, (hipStream_t)stream),
                      "paged_attention_decode_append launch");
  }
  // other partition modes: the append kernel, then the decode kernel
  pkv::KvAppendArgs ap{k_cache, v_cache, k_new, v_new, block_tables, context_lens, nullptr,
                       B, B, Hkv, D, block_size, max_blocks_per_seq, num_blocks};
  const int rc2 = hip_status(pkv::launch_kv_append(ap, (hipStream_t)stream),
                             "paged_attention_decode_append launch (append)");
  if (rc2 != PKV_OK) return rc2;
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream),
                    "paged_attention_decode_append launch (decode)");
}

int paged_attention_decode_plan(const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t num_blocks, int32_t max_context_len, void* workspace,
                                size_t workspace_bytes, void* stream) {
  DecodePlan plan;
  const int rc = plan_decode(B, Hq, Hkv, D, block_size, max_context_len, PKV_PARTITION_PLANNED,
                             &plan);
  if (rc != PKV_OK) return rc;
  if (B == 0) return PKV_OK;
  if (!block_tables || !context_lens) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be > 0");
  if (!workspace || workspace_bytes < plan.bytes)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(PKV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if (debug_enabled()) {
    const int rc2 = debug_check(block_tables, context_lens, nullptr, B, 0, max_blocks_per_seq,
                                num_blocks, PKV_CHECK_READ, (hipStream_t)stream);
    if (rc2 != PKV_OK) return rc2;
  }
  pkv::DecodeArgs a{};
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.mode = pkv::kAuto;
  a.parts_max = 1;
  a.plan = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.plan_offset);
  a.write_plan = 1;
  return hip_status(pkv::launch_decode(a, (hipStream_t)stream), "paged_attention_decode_plan launch");
}

int paged_attention_prefill_causal(void* out, int32_t out_dtype, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* cu_q_lens, int32_t B, int32_t T_q, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t num_blocks,
                                   int32_t max_q_len, float scale, void* stream) {
  if (B < 0 || T_q < 0)
    return fail(PKV_ERR_INVALID_ARG, "B (%d) and T_q (%d) must be >= 0", B, T_q);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(PKV_ERR_INVALID_ARG, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (D != kD) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not implemented (64 only)", D);
  if (block_size != kBS)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not implemented (16 only)", block_size);
  if (Hq != kGroup * Hkv)
    return fail(PKV_ERR_UNSUPPORTED, "GQA group %d not implemented (Hq == 4*Hkv only)", Hq / Hkv);
  if (max_q_len < 0) return fail(PKV_ERR_INVALID_ARG, "max_q_len must be >= 0");
  if (B == 0 || T_q == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !cu_q_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (out_dtype != PKV_OUT_BF16 && out_dtype != PKV_OUT_F32)
    return fail(PKV_ERR_INVALID_ARG, "out_dtype %d is neither PKV_OUT_BF16 nor PKV_OUT_F32", out_dtype);
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be > 0");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "out, q and the pools must be 16-byte aligned");
  if (!pkv::grid_fits(pkv::prefill_grid_size(max_q_len, T_q, B, Hkv), 256))
    return fail(PKV_ERR_UNSUPPORTED, "%lld workgroups of 256 threads exceed one launch "
                "(at most 2^32 - 1 work-items)",
                (long long)pkv::prefill_grid_size(max_q_len, T_q, B, Hkv));
  if (debug_enabled()) {
    const int rc = debug_check(block_tables, context_lens, cu_q_lens, B, T_q, max_blocks_per_seq,
                               num_blocks, PKV_CHECK_PREFILL, (hipStream_t)stream);
    if (rc != PKV_OK) return rc;
  }
  pkv::PrefillArgs a;
  a.out = out;
  a.out_f32 = out_dtype == PKV_OUT_F32;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_q_lens = cu_q_lens;
  a.B = B;
  a.T_q = T_q;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_q_len = max_q_len;
  a.scale = scale;
  return hip_status(pkv::launch_prefill(a, (hipStream_t)stream),
                    "paged_attention_prefill_causal launch");
}

int pagedkv_stream_blocks(const void* k_cache, const void* v_cache, const int32_t* block_ids,
                          int32_t n_ids, int32_t Hkv, int32_t D, int32_t block_size,
                          int32_t num_blocks, void* sink, size_t sink_bytes, void* stream) {
  if (n_ids < 0) return fail(PKV_ERR_INVALID_ARG, "n_ids must be >= 0 (got %d)", n_ids);
  if (n_ids == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_ids || !sink)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (Hkv <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "Hkv and num_blocks must be > 0");
  if (D != kD || block_size != kBS)
    return fail(PKV_ERR_UNSUPPORTED, "the streaming probe reads 2 KB chunks: D 64, block_size 16");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(sink))
    return fail(PKV_ERR_INVALID_ARG, "pools and sink must be 16-byte aligned");
  const size_t need = (size_t)pkv::stream_blocks_sink_words() * 4;
  if (sink_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "sink of %zu bytes needed, %zu given", need, sink_bytes);
  return hip_status(pkv::launch_stream_blocks(k_cache, v_cache, block_ids, n_ids, Hkv, D,
                                              block_size, num_blocks,
                                              static_cast<uint32_t*>(sink), (hipStream_t)stream),
                    "pagedkv_stream_blocks launch");
}

int pagedkv_mfma_probe(int32_t iters, void* sink, size_t sink_bytes, void* stream) {
  if (iters <= 0 || iters > PKV_MFMA_PROBE_MAX_ITERS)
    return fail(PKV_ERR_INVALID_ARG, "iters must be in [1, %d] (got %d)", PKV_MFMA_PROBE_MAX_ITERS,
                iters);
  if (!sink) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(sink)) return fail(PKV_ERR_INVALID_ARG, "sink must be 16-byte aligned");
  const size_t need = (size_t)pkv::stream_blocks_sink_words() * 4;
  if (sink_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "sink of %zu bytes needed, %zu given", need, sink_bytes);
  return hip_status(pkv::launch_mfma_probe(iters, static_cast<float*>(sink), (hipStream_t)stream),
                    "pagedkv_mfma_probe launch");
}

}  // extern "C"
