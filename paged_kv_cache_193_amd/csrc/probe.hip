// probe.hip -- measurement probes: a plain streaming read of the KV-cache
// bytes a decode call reads, the floor against which the decode kernel is
// measured, and (further down) the bf16 MFMA issue rate that the prefill
// kernel is measured against.
//
// Decode reads every cached token's K and V row once and is bound by memory
// bandwidth (nano-vLLM guide announcement, ch. 6 "Prefill vs Decode"); an
// honest figure for it states how close it comes to simply reading the same
// bytes (ch. 11 "Benchmarks").  This kernel reads whole (block, KV head)
// chunks of both pools, 2 KB of K and 2 KB of V each at head_dim 64 and
// block_size 16, for a list of physical block ids (those the block tables map
// a batch's contexts to), with no arithmetic beyond folding the words into a
// register.  The grid is the decode's automatic-split grid (2048 wavefronts);
// each wavefront streams an equal contiguous share of the (block, head)
// chunks, two chunks in flight, with 16-byte loads that cover whole
// 128-byte rows and carry the non-temporal hint, as the decode's do.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kProbeWaves = 2048;
constexpr int kWavesPerGroup = 4;

__global__ void __launch_bounds__(256)
stream_blocks_kernel(const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                     const int32_t* __restrict__ block_ids, int64_t n_chunks, int Hkv,
                     int chunk_elems, int num_blocks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int64_t W = (int64_t)gridDim.x * kWavesPerGroup;
  const int64_t c0 = w * n_chunks / W, c1 = (w + 1) * n_chunks / W;
  // lane's 32 bytes of a chunk: elements [16 lane, 16 lane + 16)
  const int64_t lane_off = (int64_t)lane * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  auto chunk_base = [&](int64_t c) {
    int id = block_ids[c / Hkv];
    id = id >= 0 && id < num_blocks ? id : 0;
    return ((int64_t)id * Hkv + c % Hkv) * chunk_elems + lane_off;
  };
  int64_t c = c0;
  for (; c + 1 < c1; c += 2) {
    const int64_t a = chunk_base(c), b = chunk_base(c + 1);
    const u32x4 k0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_cache + a));
    const u32x4 k1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_cache + a + 8));
    const u32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_cache + a));
    const u32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_cache + a + 8));
    const u32x4 k2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_cache + b));
    const u32x4 k3 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_cache + b + 8));
    const u32x4 v2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_cache + b));
    const u32x4 v3 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_cache + b + 8));
    acc ^= k0 ^ k1 ^ v0 ^ v1 ^ k2 ^ k3 ^ v2 ^ v3;
  }
  if (c < c1) {
    const int64_t a = chunk_base(c);
    acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_cache + a)) ^
           __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_cache + a + 8)) ^
           __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_cache + a)) ^
           __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_cache + a + 8));
  }
  // one word per lane, so the loads cannot be dropped
  sink[w * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// MFMA issue-rate probe: the bf16 matrix-core peak that prefill is measured
// against, taken on this GPU at its running clock.  Every wavefront runs
// kMfmaChains independent accumulator chains of v_mfma_f32_32x32x16_bf16
// (32 x 32 x 16 products, 32,768 flops each) `iters` times, with operands
// held in registers, so nothing but the matrix cores is exercised.  All
// operand elements are 2^-4, so every product adds 16 * 2^-8 = 2^-4 to each
// accumulator element and the folded result of a lane, 4 chains x 16
// elements x iters x 2^-4 = 4 * iters, is exact in fp32 for the sizes the
// entry point accepts.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kMfmaChains = 4;

__global__ void __launch_bounds__(256)
mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const __bf16 x = (__bf16)0.0625f;
  const bf16x8_t a = {x, x, x, x, x, x, x, x};
  f32x16 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[k][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k)
      c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c[k], 0, 0, 0);
  }
  float v = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) v += c[k][e];
  sink[w * 64 + lane] = v;
}

}  // namespace

int64_t stream_blocks_sink_words() { return (int64_t)kProbeWaves * 64; }
int64_t mfma_probe_flops(int32_t iters) {
  return (int64_t)kProbeWaves * kMfmaChains * iters * (2 * 32 * 32 * 16);
}
hipError_t launch_mfma_probe(int32_t iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(kProbeWaves / kWavesPerGroup),
                     dim3(kWavesPerGroup * 64), 0, stream, (int)iters, sink);
  return hipGetLastError();
}


hipError_t launch_stream_blocks(const void* k_cache, const void* v_cache, const int32_t* block_ids,
                                int32_t n_ids, int32_t Hkv, int32_t D, int32_t block_size,
                                int32_t num_blocks, uint32_t* sink, hipStream_t stream) {
  const int64_t n_chunks = (int64_t)n_ids * Hkv;
  hipLaunchKernelGGL(stream_blocks_kernel, dim3(kProbeWaves / kWavesPerGroup),
                     dim3(kWavesPerGroup * 64), 0, stream, (const uint16_t*)k_cache,
                     (const uint16_t*)v_cache, block_ids, n_chunks, Hkv, block_size * D,
                     num_blocks, sink);
  return hipGetLastError();
}

}  // namespace pkv
