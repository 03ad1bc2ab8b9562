// kv_append.hip -- write new tokens' K and V rows into the paged pools.
//
// Each new token's K and V are stored once in the cache so later steps read
// them instead of recomputing them (tiny-vllm README, table of contents "Why
// KV cache exists"; nano-vLLM guide announcement, ch. 3 "KV Cache"), at the
// slot the block table gives for its logical position (README "Paged KV
// cache"; guide ch. 4 "PagedAttention").
//
// One thread moves one 16-byte chunk (8 bf16): thread id -> (token, plane
// K or V, KV head, chunk).  Consecutive threads cover one token's heads and
// chunks, so reads of k_new/v_new are fully coalesced and each destination
// row (D*2 bytes) is written by D/8 consecutive lanes.
#include "device_common.h"
#include "launch.h"

namespace pkv {

__global__ void __launch_bounds__(256)
kv_append_kernel(uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                 const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                 const int32_t* __restrict__ block_tables,
                 const int32_t* __restrict__ context_lens,
                 const int32_t* __restrict__ cu_new_lens, int32_t B, int32_t T_new,
                 int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks_per_seq,
                 int32_t num_blocks) {
  const int chunks = D >> 3;                    // 16-byte chunks per row
  const int64_t per_token = 2LL * Hkv * chunks;  // K and V planes
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T_new * per_token) return;
  const int t = (int)(gid / per_token);
  int rem = (int)(gid - (int64_t)t * per_token);
  const int plane = rem / (Hkv * chunks);
  rem -= plane * Hkv * chunks;
  const int h = rem / chunks;
  const int chunk = rem - h * chunks;

  // sequence of token t: cu_new_lens[b] <= t < cu_new_lens[b+1]
  int b, first, n;
  if (cu_new_lens == nullptr) {
    b = t;
    first = t;
    n = 1;
  } else {
    int lo = 0, hi = B;  // invariant: cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (cu_new_lens[mid] <= t) lo = mid; else hi = mid;
    }
    b = lo;
    first = cu_new_lens[b];
    n = cu_new_lens[b + 1] - first;
  }
  const int pos = context_lens[b] - n + (t - first);
  if (pos < 0) return;
  const int logical_block = pos / block_size;
  if (logical_block >= max_blocks_per_seq) return;
  const int phys = block_tables[(int64_t)b * max_blocks_per_seq + logical_block];
  if (phys < 0 || phys >= num_blocks) return;
  const int row = pos - logical_block * block_size;

  const int64_t src = ((int64_t)t * Hkv + h) * D + chunk * 8;
  const int64_t dst = (((int64_t)phys * Hkv + h) * block_size + row) * D + chunk * 8;
  const uint16_t* s = plane ? v_new : k_new;
  uint16_t* d = plane ? v_cache : k_cache;
  *reinterpret_cast<u32x4*>(d + dst) = *reinterpret_cast<const u32x4*>(s + src);
}

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.T_new * 2 * a.Hkv * (a.D / 8);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (uint16_t*)a.k_cache, (uint16_t*)a.v_cache, (const uint16_t*)a.k_new,
                     (const uint16_t*)a.v_new, a.block_tables, a.context_lens, a.cu_new_lens,
                     a.B, a.T_new, a.Hkv, a.D, a.block_size, a.max_blocks_per_seq,
                     a.num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
