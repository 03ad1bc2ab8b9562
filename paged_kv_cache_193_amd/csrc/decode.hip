// decode.hip -- paged attention for decode: one query token per sequence
// attends to every cached token of its sequence, reading K/V through the
// block table (tiny-vllm README, table of contents "Attention", "GQA",
// "Softmax", "Online softmax", "Paged Attention"; nano-vLLM guide
// announcement ch. 4 "PagedAttention" and ch. 6 "Prefill vs Decode": decode
// is bound by memory traffic, not arithmetic).
//
// Shapes this kernel is built for: head_dim 64, block_size 16, 4 query heads
// per KV head (Llama-3.2-1B: 32 query heads over 8 KV heads).
//
// Work unit: a "segment" = a run of consecutive blocks of one stream
// (sequence b, KV head g), processed by ONE wavefront.  The 4 query heads of
// the group share every K/V row the wavefront loads (GQA).
//
// Lane map inside a wavefront (lane = 8*grp + i):
//   grp 0..7  -> tokens grp and grp+8 of the current 16-token block
//   i   0..7  -> head_dim chunk [8i, 8i+8)
// A block (2 KB of K for one KV head) is read by two dwordx4 loads whose
// 64 lanes cover 1 KB contiguous each: every instruction reads 8 whole
// 128-byte token rows.
//
// q.k: each lane forms partial dots for 2 tokens x 4 heads over its 8-wide
// chunk with v_dot2_f32_bf16.  The 8 lanes of a group then reduce-scatter
// the 8 partials with 3 DPP steps so that each lane ends with ONE complete
// score: head c(i) and token grp (lanes i<4) or grp+8 (lanes i>=4).  The
// trick that makes steps 1-2 need no selects: lane i loads the 4 query heads
// in the order h = slot ^ c(i), so "keep slots 0,1 / send slots 2,3" is the
// same register choice on every lane.
//
// Online softmax (fp32, log2 domain): the lane pair (i, 7-i) shares a running
// max m for head c over its two token streams; the running max is only moved
// when a score exceeds it by more than 2^8 (lazy rescale, exact by the
// softmax shift identity; weights stay <= 2^8).  P.V packs the two tokens'
// weights as a bf16 pair and V into (token grp, token grp+8) pairs per d, so
// P.V is again v_dot2_f32_bf16 with an fp32 accumulator.
//
// Split contexts: a segment that does not cover its whole stream writes a
// partial record (normalised output, m, l) and decode_merge_kernel combines
// the records of a stream by log-sum-exp.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kD = 64;
constexpr int kBS = 16;
constexpr int kWaves = 4;        // wavefronts per workgroup
#ifndef PKV_DECODE_RING
#define PKV_DECODE_RING 4
#endif
constexpr int kRing = PKV_DECODE_RING;  // K/V blocks in flight per wavefront

struct BlockRegs {
  u32x4 ka, kb, va, vb;  // tokens grp and grp+8, head_dim chunk i
};

struct LaneState {
  float m;          // running max (log2 units), head c, shared by lanes i and 7-i
  float l;          // sum of this lane's own-token weights
  float acc[4][8];  // slot j (head j^c) x d in [8i, 8i+8)
};

struct Params {
  void* out;
  int out_f32;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int B, Hq, Hkv, max_blocks, num_blocks, ctx_cap;
  float scale_log2;
  int part_blocks, parts_max;
  float* ws_o;
  float* ws_ml;
  int* ws_pfx;  // auto mode: per-sequence block prefix, then NB and the chunk size
};

__device__ __forceinline__ int eff_ctx(const Params& p, int b) {
  int c = p.context_lens[b];
  c = c < 0 ? 0 : c;
  return c > p.ctx_cap ? p.ctx_cap : c;
}

// Issue the four 16-byte loads of block `j` of the stream, whose physical id
// `phys` was read earlier; returns the number of valid tokens in the block
// (0 when `phys` is not a valid block id: then block 0 is read and ignored).
__device__ __forceinline__ int issue_block(BlockRegs& r, const Params& p, int phys, int g,
                                           int j, int ctx, int lane_off) {
  int nv = ctx - j * kBS;
  nv = nv > kBS ? kBS : nv;
  if (phys < 0 || phys >= p.num_blocks) {
    phys = 0;
    nv = 0;
  }
  const int64_t base = ((int64_t)phys * p.Hkv + g) * (kBS * kD) + lane_off;
  const uint16_t* kp = p.k_cache + base;
  const uint16_t* vp = p.v_cache + base;
  r.ka = *reinterpret_cast<const u32x4*>(kp);
  r.kb = *reinterpret_cast<const u32x4*>(kp + 8 * kD);
  r.va = *reinterpret_cast<const u32x4*>(vp);
  r.vb = *reinterpret_cast<const u32x4*>(vp + 8 * kD);
  return nv;
}

// Score of this lane's own (head c, token) pair for one block, log2 units:
// partial dots over the lane's 8-wide chunk for 2 tokens x 4 head slots,
// then a reduce-scatter over the 8 lanes of the group.
__device__ __forceinline__ float block_score(const BlockRegs& r, const uint32_t (&qv)[4][4],
                                             float scale_log2, bool quad1) {
  float pd[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = dot2_bf16(qv[j][0], r.ka[0], 0.f);
    float b = dot2_bf16(qv[j][0], r.kb[0], 0.f);
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      a = dot2_bf16(qv[j][w], r.ka[w], a);
      b = dot2_bf16(qv[j][w], r.kb[w], b);
    }
    pd[0][j] = a;
    pd[1][j] = b;
  }
  float t[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float r0 = pd[s][0] + dpp<kQuadXor2>(pd[s][2]);
    const float r1 = pd[s][1] + dpp<kQuadXor2>(pd[s][3]);
    t[s] = r0 + dpp<kQuadXor1>(r1);
  }
  const float keep = quad1 ? t[1] : t[0];
  const float send = quad1 ? t[0] : t[1];
  return (keep + dpp<kRowHalfMirror>(send)) * scale_log2;
}

// P.V of one block: weights p of this lane's (head c, own token), V rows of
// tokens grp and grp+8 (zeroed where not valid, so 0 * NaN never happens).
template <bool kMasked>
__device__ __forceinline__ void block_pv(LaneState& st, const BlockRegs& r, float pw,
                                         bool quad1, bool va_ok, bool vb_ok) {
  const float pm = dpp<kRowHalfMirror>(pw);
  const uint32_t p2 = pack_bf16(quad1 ? pm : pw, quad1 ? pw : pm);
  uint32_t ps[4];
  ps[0] = p2;
  ps[1] = dpp_u32<kQuadXor1>(p2);
  ps[2] = dpp_u32<kQuadXor2>(p2);
  ps[3] = dpp_u32<kQuadXor3>(p2);
  u32x4 va = r.va, vb = r.vb;
  if (kMasked) {
    if (!va_ok) va = u32x4{0, 0, 0, 0};
    if (!vb_ok) vb = u32x4{0, 0, 0, 0};
  }
  uint32_t v2[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    v2[2 * w] = __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);      // d even
    v2[2 * w + 1] = __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);  // d odd
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[j][e] = dot2_bf16(ps[j], v2[e], st.acc[j][e]);
}

// Run blocks [j0, j1) of stream (b, g) through one wavefront.
//
// The blocks go through a ring of kRing register slots in groups of kRing:
// the scores of a whole group are formed first, the running max moves once
// per group (one rescale of the accumulator, no branch), then P.V runs block
// by block and each slot is refilled with the block kRing ahead as soon as its
// V is consumed.  Every group issues exactly kRing block loads (past the
// segment end the last block is re-read, a cache hit marked invalid), so the
// hardware wait counts stay exact.
__device__ __forceinline__ void run_segment(LaneState& st, const Params& p, int b, int g,
                                            int j0, int j1, int ctx, int lane) {
  const int grp = lane >> 3, i = lane & 7;
  const bool quad1 = (i & 4) != 0;
  const int c = quad1 ? ((i & 3) ^ 3) : (i & 3);
  const int own_tok = quad1 ? grp + 8 : grp;

  // this lane's query chunks, head order slot j -> head j ^ c
  uint32_t qv[4][4];
  const uint16_t* qb = p.q + ((int64_t)b * p.Hq + 4 * g) * kD + 8 * i;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 v = *reinterpret_cast<const u32x4*>(qb + (j ^ c) * kD);
#pragma unroll
    for (int w = 0; w < 4; ++w) qv[j][w] = v[w];
  }

  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[j][e] = 0.f;

  const int32_t* trow = p.block_tables + (int64_t)b * p.max_blocks;
  const int lane_off = grp * kD + 8 * i;
  const int nb = j1 - j0;
  const int last = j1 - 1;
  // block ids: lane k of `tab` holds the id of block tab_base + k (clamped to
  // the segment), read with readlane; refilled once per 64 blocks
  int tab_base = j0;
  int tab = trow[j0 + lane < last ? j0 + lane : last];

  BlockRegs ring[kRing];
  int nvalid[kRing];
#pragma unroll
  for (int s = 0; s < kRing; ++s) {
    const int j = j0 + s < last ? j0 + s : last;
    const int nv = issue_block(ring[s], p, __builtin_amdgcn_readlane(tab, j - tab_base), g, j,
                               ctx, lane_off);
    nvalid[s] = s < nb ? nv : 0;
  }

  for (int base = 0; base < nb; base += kRing) {
    bool full = true;
#pragma unroll
    for (int s = 0; s < kRing; ++s) full = full && nvalid[s] == kBS;
    float x[kRing];
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      x[s] = block_score(ring[s], qv, p.scale_log2, quad1);
      if (!full && own_tok >= nvalid[s]) x[s] = -INFINITY;
    }
    // one max per group, shared by the mirror pair (same head, tokens t, t+8)
    float mx = x[0];
#pragma unroll
    for (int s = 1; s < kRing; ++s) mx = fmaxf(mx, x[s]);
    mx = fmaxf(mx, dpp<kRowHalfMirror>(mx));
    const float m_new = fmaxf(st.m, mx);
    // no valid token yet on this lane pair: keep everything at zero weight
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
    st.m = m_new;
    st.l *= alpha;
    const float a1 = dpp<kQuadXor1>(alpha), a2 = dpp<kQuadXor2>(alpha),
                a3 = dpp<kQuadXor3>(alpha);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      st.acc[0][e] *= alpha;
      st.acc[1][e] *= a1;
      st.acc[2][e] *= a2;
      st.acc[3][e] *= a3;
    }
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      const float pw = __builtin_amdgcn_exp2f(x[s] - m_use);  // 0 for x = -inf
      st.l += pw;
      if (full)
        block_pv<false>(st, ring[s], pw, quad1, true, true);
      else
        block_pv<true>(st, ring[s], pw, quad1, grp < nvalid[s], grp + 8 < nvalid[s]);
      // refill this slot with the block kRing ahead
      const int jn = j0 + base + s + kRing;
      const int j = jn < last ? jn : last;
      if (j - tab_base >= 64) {
        tab_base += 64;
        tab = trow[tab_base + lane < last ? tab_base + lane : last];
        // wait here (vmcnt 0), inside the branch, so the common path after it
        // carries no wait for this load
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      const int nv = issue_block(ring[s], p, __builtin_amdgcn_readlane(tab, j - tab_base), g, j,
                                 ctx, lane_off);
      nvalid[s] = jn < j1 ? nv : 0;
    }
  }
}

// Combine the 64 lanes' states of a finished segment and write either the
// final rows out[b][4g..4g+3][:] or a split record.  red: this wave's 8 KB.
__device__ __forceinline__ void finish_segment(const LaneState& st, const Params& p, int b,
                                               int g, bool complete, int record, float* red,
                                               int lane) {
  const int grp = lane >> 3, i = lane & 7;
  const bool quad1 = (i & 4) != 0;
  const int c = quad1 ? ((i & 3) ^ 3) : (i & 3);

  const float l_pair = st.l + dpp<kRowHalfMirror>(st.l);
  float mg = fmaxf(st.m, dpp<kRowRor8>(st.m));
  mg = fmaxf(mg, shfl_xor(mg, 16));
  mg = fmaxf(mg, shfl_xor(mg, 32));
  const float sc = (mg == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m - mg);
  float lt = l_pair * sc;
  lt += dpp<kRowRor8>(lt);
  lt += shfl_xor(lt, 16);
  lt += shfl_xor(lt, 32);

  float ss[4];
  ss[0] = sc;
  ss[1] = dpp<kQuadXor1>(sc);
  ss[2] = dpp<kQuadXor2>(sc);
  ss[3] = dpp<kQuadXor3>(sc);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float* dst = red + (grp * 4 + (j ^ c)) * kD + 8 * i;
    float4 lo = make_float4(st.acc[j][0] * ss[j], st.acc[j][1] * ss[j], st.acc[j][2] * ss[j],
                            st.acc[j][3] * ss[j]);
    float4 hi = make_float4(st.acc[j][4] * ss[j], st.acc[j][5] * ss[j], st.acc[j][6] * ss[j],
                            st.acc[j][7] * ss[j]);
    *reinterpret_cast<float4*>(dst) = lo;
    *reinterpret_cast<float4*>(dst + 4) = hi;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int h = lane >> 4;
  const int d4 = (lane & 15) * 4;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int gg = 0; gg < 8; ++gg) {
    float4 v = *reinterpret_cast<const float4*>(red + (gg * 4 + h) * kD + d4);
    sum.x += v.x;
    sum.y += v.y;
    sum.z += v.z;
    sum.w += v.w;
  }
  // lane h (group 0, quad 0) holds head h's totals
  const float l_h = shfl(lt, h);
  const float m_h = shfl(mg, h);
  const float inv = l_h > 0.f ? 1.0f / l_h : 0.f;
  const float4 o = make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();

  if (complete) {
    const int64_t row = ((int64_t)b * p.Hq + 4 * g + h) * kD + d4;
    if (p.out_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row) = o;
    } else {
      u32x2 pk = {pack_bf16(o.x, o.y), pack_bf16(o.z, o.w)};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + row) = pk;
    }
  } else {
    *reinterpret_cast<float4*>(p.ws_o + (int64_t)record * kRecordFloats + h * kD + d4) = o;
    if ((lane & 15) == 0) {
      p.ws_ml[((int64_t)record * 4 + h) * 2 + 0] = m_h;
      p.ws_ml[((int64_t)record * 4 + h) * 2 + 1] = l_h;
    }
  }
}

__device__ __forceinline__ void write_zero_rows(const Params& p, int b, int g, int lane) {
  const int h = lane >> 4, d4 = (lane & 15) * 4;
  const int64_t row = ((int64_t)b * p.Hq + 4 * g + h) * kD + d4;
  if (p.out_f32)
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row) = make_float4(0.f, 0.f, 0.f, 0.f);
  else
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + row) = u32x2{0, 0};
}

// kWhole / kFixed: one wavefront per (b, g, partition) unit.
template <int kMode>
__global__ void __launch_bounds__(kWaves * 64)
decode_units_kernel(Params p) {
  __shared__ float red[kWaves][8 * 4 * kD];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kWaves + wave;
  const int parts = (kMode == kWhole) ? 1 : p.parts_max;
  const int stream = unit / parts;
  const int part = unit - stream * parts;
  if (stream >= p.B * p.Hkv) return;
  const int b = stream / p.Hkv;
  const int g = stream - b * p.Hkv;
  const int ctx = eff_ctx(p, b);
  const int nb = (ctx + kBS - 1) / kBS;
  if (nb == 0) {
    if (part == 0) write_zero_rows(p, b, g, lane);
    return;
  }
  int j0 = 0, j1 = nb;
  if (kMode == kFixed) {
    j0 = part * p.part_blocks;
    if (j0 >= nb) return;
    j1 = j0 + p.part_blocks < nb ? j0 + p.part_blocks : nb;
  }
  LaneState st;
  run_segment(st, p, b, g, j0, j1, ctx, lane);
  const bool complete = (j0 == 0 && j1 == nb);
  finish_segment(st, p, b, g, complete, unit, red[wave], lane);
}

// kAuto: a fixed grid of kAutoWaves wavefronts; all blocks of all streams,
// in (b, g) order, are cut into equal consecutive shares, one per wavefront.
// A share covers at most two partial streams (its first and last segment);
// every stream strictly inside a share is complete.  Record slots: wavefront
// w owns records 2w (its first segment) and 2w+1 (its last).
__global__ void __launch_bounds__(kWaves * 64)
decode_auto_kernel(Params p) {
  __shared__ float red[kWaves][8 * 4 * kD];
  __shared__ int pfx[kAutoMaxBatch + 1];
  __shared__ int part_sums[kWaves * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // per-sequence block counts -> exclusive prefix in LDS
  const int per = (p.B + kWaves * 64 - 1) / (kWaves * 64);
  const int beg = tid * per;
  const int end = beg + per < p.B ? beg + per : p.B;
  int local = 0;
  for (int k = beg; k < end; ++k) local += (eff_ctx(p, k) + kBS - 1) / kBS;
  part_sums[tid] = local;
  __syncthreads();
  for (int off = 1; off < kWaves * 64; off <<= 1) {
    int v = tid >= off ? part_sums[tid - off] : 0;
    __syncthreads();
    part_sums[tid] += v;
    __syncthreads();
  }
  int run = tid ? part_sums[tid - 1] : 0;
  for (int k = beg; k < end; ++k) {
    pfx[k] = run;
    run += (eff_ctx(p, k) + kBS - 1) / kBS;
  }
  if (tid == kWaves * 64 - 1) pfx[p.B] = part_sums[tid];
  __syncthreads();

  const int64_t NB = (int64_t)p.Hkv * __builtin_amdgcn_readfirstlane(pfx[p.B]);
  const int W = gridDim.x * kWaves;
  const int64_t C = (NB + W - 1) / W;
  if (blockIdx.x == 0) {  // publish the layout for the merge kernel
    for (int k = tid; k <= p.B; k += kWaves * 64) p.ws_pfx[k] = pfx[k];
    if (tid == 0) p.ws_pfx[p.B + 1] = (int)C;
  }
  const int w = blockIdx.x * kWaves + wave;
  int64_t x = (int64_t)w * C;
  const int64_t x1 = x + C < NB ? x + C : NB;
  const int64_t x0 = x;
  while (x < x1) {
    // sequence containing global block x: largest b with Hkv*pfx[b] <= x
    int lo = 0, hi = p.B;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if ((int64_t)p.Hkv * pfx[mid] <= x) lo = mid; else hi = mid;
    }
    // values read from LDS are wave-uniform here; keep them in SGPRs
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int pb = __builtin_amdgcn_readfirstlane(pfx[b]);
    const int nb = __builtin_amdgcn_readfirstlane(pfx[b + 1]) - pb;
    const int64_t off = x - (int64_t)p.Hkv * pb;
    const int g = (int)(off / nb);
    const int jb = (int)(off - (int64_t)g * nb);
    const int64_t stream_end = x - jb + nb;
    const int64_t xe = x1 < stream_end ? x1 : stream_end;
    const int je = jb + (int)(xe - x);
    LaneState st;
    run_segment(st, p, b, g, jb, je, eff_ctx(p, b), lane);
    const bool complete = (jb == 0 && je == nb);
    const int64_t stream_start = x - jb;
    const int record = 2 * w + (stream_start <= x0 ? 0 : 1);
    finish_segment(st, p, b, g, complete, record, red[wave], lane);
    x = xe;
  }
}

// Log-sum-exp merge of split records, one workgroup per stream (b, g).
// The (m, l) pairs of up to kMergeChunk records x 4 heads are staged in LDS
// with one parallel load; then thread (head h = tid / 64, d = tid % 64)
// folds the chunk into its running (M, numerator, denominator) with
// independent loads of the records' outputs.
constexpr int kMergeChunk = 256;

template <int kMode>
__global__ void __launch_bounds__(256)
decode_merge_kernel(Params p) {
  __shared__ float sm[kMergeChunk][4];
  __shared__ float sl[kMergeChunk][4];
  __shared__ int64_t srec[kMergeChunk];
  const int stream = blockIdx.x;
  const int b = stream / p.Hkv;
  const int g = stream - b * p.Hkv;
  const int tid = threadIdx.x;
  const int h = tid >> 6;
  const int d = tid & 63;
  int count, first = 0, w0 = 0;
  int64_t start_x = 0, C = 1;
  if (kMode == kFixed) {
    const int ctx = eff_ctx(p, b);
    const int nb = (ctx + kBS - 1) / kBS;
    count = (nb + p.part_blocks - 1) / p.part_blocks;
    first = stream * p.parts_max;
  } else {
    const int pb = p.ws_pfx[b], nb = p.ws_pfx[b + 1] - pb;
    if (nb == 0) {  // empty context: zero rows (no wavefront saw this stream)
      if (tid < 64) write_zero_rows(p, b, g, tid);
      return;
    }
    C = p.ws_pfx[p.B + 1];
    start_x = (int64_t)p.Hkv * pb + (int64_t)g * nb;
    w0 = (int)(start_x / C);
    const int w1 = (int)((start_x + nb - 1) / C);
    count = w1 - w0 + 1;
  }
  if (count <= 1) return;  // written directly by the decode kernel

  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int k0 = 0; k0 < count; k0 += kMergeChunk) {
    const int n = count - k0 < kMergeChunk ? count - k0 : kMergeChunk;
    __syncthreads();
    for (int idx = tid; idx < n * 4; idx += 256) {
      const int k = idx >> 2, hh = idx & 3;
      int64_t r;
      if (kMode == kFixed) {
        r = first + k0 + k;
      } else {
        const int w = w0 + k0 + k;
        r = 2LL * w + ((k0 + k == 0 && start_x > (int64_t)w0 * C) ? 1 : 0);
      }
      if (hh == 0) srec[k] = r;
      sm[k][hh] = p.ws_ml[(r * 4 + hh) * 2 + 0];
      sl[k][hh] = p.ws_ml[(r * 4 + hh) * 2 + 1];
    }
    __syncthreads();
    float Mc = -INFINITY;
    for (int k = 0; k < n; ++k)
      if (sl[k][h] > 0.f) Mc = fmaxf(Mc, sm[k][h]);
    if (Mc == -INFINITY) continue;
    const float Mn = fmaxf(M, Mc);
    const float rescale = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    num *= rescale;
    den *= rescale;
    M = Mn;
#pragma unroll 8
    for (int k = 0; k < n; ++k) {
      const float l = sl[k][h];
      const float wgt = l > 0.f ? l * __builtin_amdgcn_exp2f(sm[k][h] - M) : 0.f;
      const float o = p.ws_o[srec[k] * kRecordFloats + h * kD + d];
      num += wgt * o;
      den += wgt;
    }
  }
  const float o = den > 0.f ? num / den : 0.f;
  const int64_t row = ((int64_t)b * p.Hq + 4 * g + h) * kD + d;
  if (p.out_f32)
    reinterpret_cast<float*>(p.out)[row] = o;
  else
    reinterpret_cast<uint16_t*>(p.out)[row] = to_bf16_bits(o);
}

}  // namespace

size_t decode_records(int32_t mode, int32_t B, int32_t Hkv, int32_t parts_max) {
  if (mode == kFixed) return (size_t)B * Hkv * parts_max;
  if (mode == kAuto) return (size_t)2 * kAutoWaves;
  return 0;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  Params p;
  p.out = a.out;
  p.out_f32 = a.out_f32;
  p.q = (const uint16_t*)a.q;
  p.k_cache = (const uint16_t*)a.k_cache;
  p.v_cache = (const uint16_t*)a.v_cache;
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  const int64_t cap = (int64_t)a.max_blocks_per_seq * kBS;
  p.ctx_cap = (int)(a.max_context_len < cap ? a.max_context_len : cap);
  p.scale_log2 = a.scale * kLog2e;
  p.part_blocks = a.part_blocks;
  p.parts_max = a.parts_max;
  p.ws_o = a.ws_o;
  p.ws_ml = a.ws_ml;
  p.ws_pfx = a.ws_o ? reinterpret_cast<int*>(
                          a.ws_ml + decode_records(a.mode, a.B, a.Hkv, a.parts_max) * 8)
                    : nullptr;
  const int streams = a.B * a.Hkv;
  if (a.mode == kWhole) {
    const int grid = (streams + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(decode_units_kernel<kWhole>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
  } else if (a.mode == kFixed) {
    const int64_t units = (int64_t)streams * a.parts_max;
    const int grid = (int)((units + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(decode_units_kernel<kFixed>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
    if (a.parts_max > 1)
      hipLaunchKernelGGL(decode_merge_kernel<kFixed>, dim3(streams), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(decode_auto_kernel, dim3(kAutoWaves / kWaves), dim3(kWaves * 64), 0,
                       stream, p);
    hipLaunchKernelGGL(decode_merge_kernel<kAuto>, dim3(streams), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
