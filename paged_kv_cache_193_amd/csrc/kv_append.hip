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
#include <climits>

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

// kv_copy_blocks: thread id -> (pair, plane K or V, 16-byte chunk of the
// block); consecutive threads copy consecutive chunks of one block.
__global__ void __launch_bounds__(256)
kv_copy_blocks_kernel(uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                      const int32_t* __restrict__ src_blocks,
                      const int32_t* __restrict__ dst_blocks, int32_t n_pairs,
                      int64_t chunks_per_block, int32_t num_blocks) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_pair = 2 * chunks_per_block;
  if (gid >= (int64_t)n_pairs * per_pair) return;
  const int pair = (int)(gid / per_pair);
  const int64_t rem = gid - (int64_t)pair * per_pair;
  const int plane = rem >= chunks_per_block;
  const int64_t chunk = plane ? rem - chunks_per_block : rem;
  const int src = src_blocks[pair], dst = dst_blocks[pair];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint16_t* pool = plane ? v_cache : k_cache;
  const u32x4 x = *reinterpret_cast<const u32x4*>(pool + (src * chunks_per_block + chunk) * 8);
  *reinterpret_cast<u32x4*>(pool + (dst * chunks_per_block + chunk) * 8) = x;
}

hipError_t launch_kv_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  const int64_t chunks = (int64_t)a.Hkv * a.block_size * (a.D / 8);
  const int64_t total = (int64_t)a.n_pairs * 2 * chunks;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (!grid_fits(blocks, threads)) return hipErrorInvalidConfiguration;  // beyond one grid
  hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (uint16_t*)a.k_cache, (uint16_t*)a.v_cache, a.src_blocks, a.dst_blocks,
                     a.n_pairs, chunks, a.num_blocks);
  return hipGetLastError();
}

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.T_new * 2 * a.Hkv * (a.D / 8);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (!grid_fits(blocks, threads)) return hipErrorInvalidConfiguration;  // beyond one grid
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (uint16_t*)a.k_cache, (uint16_t*)a.v_cache, (const uint16_t*)a.k_new,
                     (const uint16_t*)a.v_new, a.block_tables, a.context_lens, a.cu_new_lens,
                     a.B, a.T_new, a.Hkv, a.D, a.block_size, a.max_blocks_per_seq,
                     a.num_blocks);
  return hipGetLastError();
}

// kv_append_rope: the rotary position embedding of each new token's keys
// (and, when q is given, of its queries, in place) fused with the append
// above.  The pages list RoPE among the model's components (README feature
// list and table of contents "RoPE") without a formula; the reading here is
// the rotary embedding of the model they run, loaded from its Safetensors
// checkpoint: for i < D/2 the pair (x[i], x[i + D/2]) is turned by the angle
// whose cosine and sine the caller's tables hold for the token's position,
//     y[i]       = x[i] cos - x[i + D/2] sin
//     y[i + D/2] = x[i + D/2] cos + x[i] sin,
// each product and the difference rounded to fp32 (no fused multiply-add),
// then to bf16 (nearest even).  The position is the token's absolute
// position, the same one the append uses for its slot.
//
// One thread per (token, row, quarter c): rows are the Hq query heads (when
// q is given), then the Hkv key heads, then the Hkv value heads.  A thread
// owns elements [8c, 8c + 8) and [32 + 8c, 32 + 8c + 8) of its row, i.e. both
// halves of 8 rotation pairs: two 16-byte loads, two 16-byte stores, and the
// matching 32 bytes of cos and of sin.  A token's rows are consecutive, so
// every wavefront reads and writes whole 128-byte rows.  With at most 64
// sequences a wavefront finds each token's sequence, its first new token and
// its context length from one read of cu_new_lens and context_lens (a lane
// per sequence) instead of a binary search of dependent reads: the kernel is
// a short chain of round trips per thread, and each one removed shows.
__global__ void __launch_bounds__(256)
kv_append_rope_kernel(RopeAppendArgs a) {
  constexpr int kHalf = 32;  // D / 2, D == 64
  const int rows = a.Hq + 2 * a.Hkv;
  // the grid holds fewer than 2^32 threads, so 32-bit indices suffice
  const uint32_t per_token = (uint32_t)rows * 4u;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = (int)(gid / per_token);
  const int rem = (int)(gid - (uint32_t)t * per_token);
  const int r = rem >> 2, c = rem & 3;
  // Up to 64 sequences: lane j holds cu_new_lens[j + 1] and context_lens[j],
  // read in one round before any lane leaves, so that readlane and
  // ds_bpermute see defined values.  The token's sequence is the number of
  // sequences ending at or before t (cu_new_lens is non-decreasing), i.e.
  // the largest b with cu_new_lens[b] <= t.
  const bool few = a.cu_new_lens != nullptr && a.B <= 64;
  int fb = 0, ffirst = 0, fend = 0, fctx = 0;
  if (few) {
    const int lane = threadIdx.x & 63;
    const int ends = lane < a.B ? a.cu_new_lens[lane + 1] : 0x7FFFFFFF;
    const int ctxs = lane < a.B ? a.context_lens[lane] : 0;
    const int cu0 = a.cu_new_lens[0];
    for (int j = 0; j < a.B; ++j) fb += __builtin_amdgcn_readlane(ends, j) <= t ? 1 : 0;
    const int src = (fb & 63) * 4;  // fb == B only past the last token
    fend = __builtin_amdgcn_ds_bpermute(src, ends);
    fctx = __builtin_amdgcn_ds_bpermute(src, ctxs);
    const int prev = __builtin_amdgcn_ds_bpermute(((fb - 1) & 63) * 4, ends);
    ffirst = fb == 0 ? cu0 : prev;
  }
  if (gid >= (uint32_t)a.T_new * per_token) return;

  int b, first, n, ctx_b = 0;
  if (a.cu_new_lens == nullptr) {
    b = t;
    first = t;
    n = 1;
  } else if (few) {
    b = fb;
    first = ffirst;
    n = fend - first;
    ctx_b = fctx;
  } else {
    int lo = 0, hi = a.B;  // invariant: cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (a.cu_new_lens[mid] <= t) lo = mid; else hi = mid;
    }
    b = lo;
    first = a.cu_new_lens[b];
    n = a.cu_new_lens[b + 1] - first;
  }
  const int pos = (few ? ctx_b : a.context_lens[b]) - n + (t - first);
  if (pos < 0 || pos >= a.max_position) return;  // no angle for it: leave the token alone

  const bool is_q = r < a.Hq;
  const bool is_v = r >= a.Hq + a.Hkv;
  const uint16_t* src;
  uint16_t* dst;
  if (is_q) {
    dst = static_cast<uint16_t*>(a.q) + ((int64_t)t * a.Hq + r) * 64;
    src = dst;
  } else {
    const int h = is_v ? r - a.Hq - a.Hkv : r - a.Hq;
    const int logical_block = pos / a.block_size;
    if (logical_block >= a.max_blocks_per_seq) return;
    const int phys = a.block_tables[(int64_t)b * a.max_blocks_per_seq + logical_block];
    if (phys < 0 || phys >= a.num_blocks) return;
    const int row = pos - logical_block * a.block_size;
    src = static_cast<const uint16_t*>(is_v ? a.v_new : a.k_new) + ((int64_t)t * a.Hkv + h) * 64;
    dst = static_cast<uint16_t*>(is_v ? a.v_cache : a.k_cache) +
          (((int64_t)phys * a.Hkv + h) * a.block_size + row) * 64;
  }
  u32x4 lo = *reinterpret_cast<const u32x4*>(src + 8 * c);
  u32x4 hi = *reinterpret_cast<const u32x4*>(src + kHalf + 8 * c);
  if (!is_v) {
    const float* cr = a.rope_cos + (int64_t)pos * kHalf + 8 * c;
    const float* sr = a.rope_sin + (int64_t)pos * kHalf + 8 * c;
    const float4 c0 = *reinterpret_cast<const float4*>(cr);
    const float4 c1 = *reinterpret_cast<const float4*>(cr + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(sr);
    const float4 s1 = *reinterpret_cast<const float4*>(sr + 4);
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    u32x4 lo2, hi2;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float y0[2], y1[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma clang fp contract(off)
        const uint32_t bx = e ? (lo[w] & 0xFFFF0000u) : (lo[w] << 16);
        const uint32_t by = e ? (hi[w] & 0xFFFF0000u) : (hi[w] << 16);
        const float x = __builtin_bit_cast(float, bx);
        const float y = __builtin_bit_cast(float, by);
        const float co = cs[2 * w + e], si = sn[2 * w + e];
        const float xc = x * co, ys = y * si, yc = y * co, xs = x * si;
        y0[e] = xc - ys;
        y1[e] = yc + xs;
      }
      lo2[w] = pack_bf16(y0[0], y0[1]);
      hi2[w] = pack_bf16(y1[0], y1[1]);
    }
    lo = lo2;
    hi = hi2;
  }
  *reinterpret_cast<u32x4*>(dst + 8 * c) = lo;
  *reinterpret_cast<u32x4*>(dst + kHalf + 8 * c) = hi;
}

hipError_t launch_kv_append_rope(const RopeAppendArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.T_new * (a.Hq + 2 * a.Hkv) * 4;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (!grid_fits(blocks, threads)) return hipErrorInvalidConfiguration;  // beyond one grid
  hipLaunchKernelGGL(kv_append_rope_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
