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
// max m for head c over its two token streams; m moves once per group of
// kRing blocks and the accumulator is rescaled then, without a branch (the
// softmax shift identity makes the result independent of when m moves, up to
// rounding).  P.V packs the two tokens'
// weights as a bf16 pair and V into (token grp, token grp+8) pairs per d, so
// P.V is again v_dot2_f32_bf16 with an fp32 accumulator.
//
// Split contexts: a segment that does not cover its whole stream writes a
// partial record (normalised output, m, l) to the workspace and counts it on
// a per-stream counter; the wavefront that writes the stream's last piece
// merges all pieces by log-sum-exp (no second kernel) and re-zeroes the
// counter.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kD = 64;
constexpr int kBS = 16;
constexpr int kWaves = 4;        // wavefronts per workgroup
#ifndef PKV_DECODE_RING
#define PKV_DECODE_RING 2
#endif
constexpr int kRing = PKV_DECODE_RING;  // K/V blocks in flight per wavefront
#ifndef PKV_MERGE_BATCH
#define PKV_MERGE_BATCH 32
#endif

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
  uint32_t* ws_count;  // per stream (b, g): split records written so far
  int n_records;       // records in ws_o / ws_ml
  const uint16_t* k_new;  // append variant: the new token's K / V rows [B][Hkv][D]
  const uint16_t* v_new;
  int32_t* plan;          // planned variant: the plan region of the workspace
};

// Split records are written and read with 16-byte buffer accesses at agent
// scope (sc1), so a piece written by one XCD is seen by a wave merging on
// another.  The buffer descriptors also bound every access to the records.
constexpr int kSc1 = 16;                    // cache-policy bit of buffer ops
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer, dword data
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t records_o(const Params& p) {
  return __builtin_amdgcn_make_buffer_rsrc(p.ws_o, (short)0, p.n_records * kRecordFloats * 4,
                                           kRsrcWord3);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t records_ml(const Params& p) {
  return __builtin_amdgcn_make_buffer_rsrc(p.ws_ml, (short)0, p.n_records * 8 * 4, kRsrcWord3);
}

// Where the split records of one stream live: piece k of the stream is
// record base + k * stride (+ first_extra for k == 0).
struct RecordList {
  int64_t base;
  int stride, first_extra, pieces;
};

__device__ __forceinline__ int eff_ctx(const Params& p, int b) {
  int c = p.context_lens[b];
  c = c < 0 ? 0 : c;
  return c > p.ctx_cap ? p.ctx_cap : c;
}

// Issue the two 16-byte K loads of block `j` of the stream, whose physical id
// `phys` was read earlier; `ub` receives the block's element offset for the
// matching V loads (issue_v).  Returns the number of valid tokens in the
// block (0 when `phys` is not a valid block id: then block 0 is read and
// ignored).
__device__ __forceinline__ int issue_k(BlockRegs& r, const Params& p, int phys, int g, int j,
                                       int ctx, int lane_off, int64_t& ub) {
  int nv = ctx - j * kBS;
  nv = nv > kBS ? kBS : nv;
  if (phys < 0 || phys >= p.num_blocks) {
    phys = 0;
    nv = 0;
  }
  ub = ((int64_t)phys * p.Hkv + g) * (kBS * kD);
  const uint16_t* kp = p.k_cache + ub + lane_off;
  r.ka = *reinterpret_cast<const u32x4*>(kp);
  r.kb = *reinterpret_cast<const u32x4*>(kp + 8 * kD);
  return nv;
}

// The two 16-byte V loads of the block whose K issue_k issued.
__device__ __forceinline__ void issue_v(BlockRegs& r, const Params& p, int64_t ub,
                                        int lane_off) {
  const uint16_t* vp = p.v_cache + ub + lane_off;
  r.va = *reinterpret_cast<const u32x4*>(vp);
  r.vb = *reinterpret_cast<const u32x4*>(vp + 8 * kD);
}

// All four loads of a block at once (first group of a segment).
__device__ __forceinline__ int issue_block(BlockRegs& r, const Params& p, int phys, int g,
                                           int j, int ctx, int lane_off) {
  int64_t ub;
  const int nv = issue_k(r, p, phys, g, j, ctx, lane_off, ub);
  issue_v(r, p, ub, lane_off);
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
// by block.  Each slot is refilled with the block kRing ahead in two halves:
// its K as soon as the group's scores are formed, its V as soon as its own
// P.V is done, so the next group's loads are in flight while this group is
// scored and while it is accumulated.  Every group issues exactly kRing
// block loads (past the segment end the last block is re-read, a cache hit
// marked invalid), so the hardware wait counts stay exact.
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
  int64_t ub[kRing];  // element offsets of the slots' blocks, for their V loads
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
    // the K halves of the slots are free: refill them with the blocks kRing
    // ahead (their V halves follow each slot's P.V)
    int nv_next[kRing];
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      const int jn = j0 + base + s + kRing;
      const int j = jn < last ? jn : last;
      if (j - tab_base >= 64) {
        tab_base += 64;
        tab = trow[tab_base + lane < last ? tab_base + lane : last];
        // wait here (vmcnt 0), inside the branch, so the common path after it
        // carries no wait for this load
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      const int nv = issue_k(ring[s], p, __builtin_amdgcn_readlane(tab, j - tab_base), g, j, ctx,
                             lane_off, ub[s]);
      nv_next[s] = jn < j1 ? nv : 0;
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
      issue_v(ring[s], p, ub[s], lane_off);
      nvalid[s] = nv_next[s];
    }
  }
}

// Combine the 64 lanes' states of a finished segment and write either the
// final rows out[b][4g..4g+3][:] or a split record.  red: this wave's 8 KB.
__device__ __forceinline__ void finish_segment(const LaneState& st, const Params& p, int b,
                                               int g, bool complete, int record,
                                               const RecordList& rl, float* red, int lane) {
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
    return;
  }
  // Split stream: write this piece's record (agent-scope stores, one 1 KB
  // row of o per wave); count_piece() counts it once the stores completed.
  const f32x4 ov = {o.x, o.y, o.z, o.w};
  __builtin_amdgcn_raw_buffer_store_b128(ov, records_o(p), (record * kRecordFloats + h * kD + d4) * 4,
                                         0, kSc1);
  if ((lane & 15) == 0) {
    const f32x2 ml = {m_h, l_h};
    __builtin_amdgcn_raw_buffer_store_b64(ml, records_ml(p), (record * 4 + h) * 8, 0, kSc1);
  }
}

// Wait until every store this wavefront issued has completed (vmcnt 0).  The
// signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Add one finished piece to stream (b, g)'s count (agent-scope atomic, issued
// by lane 0; the piece's record stores must have completed: drain_stores())
// and return the count before the addition, in every lane.  The wavefront
// whose addition completes the count merges the pieces (merge_streams).
__device__ __forceinline__ uint32_t count_piece(const Params& p, int b, int g, int lane) {
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(p.ws_count + ((int64_t)b * p.Hkv + g) * kCounterStride, 1u,
                                    __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readfirstlane(before);
}

// A stream whose pieces this wave merges.
struct MergeJob {
  int b, g;
  RecordList rl;
};

// Largest value / sum over the 64 lanes, returned wave-uniform: rotations
// inside each row of 16 (DPP), then the four row results by readlane.
__device__ __forceinline__ float wave_max_u(float v) {
  v = fmaxf(v, dpp<kRowRor8>(v));
  v = fmaxf(v, dpp<kRowRor4>(v));
  v = fmaxf(v, dpp<kRowRor2>(v));
  v = fmaxf(v, dpp<kRowRor1>(v));
  const int iv = __builtin_bit_cast(int, v);
  return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48))));
}
__device__ __forceinline__ float wave_sum_u(float v) {
  v += dpp<kRowRor8>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kRowRor2>(v);
  v += dpp<kRowRor1>(v);
  const int iv = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48)));
}

// Merge the pieces of N (1 or 2) streams by log-sum-exp,
//   out_h = sum_k w_k,h o_k,h / sum_k w_k,h,   w_k,h = l_k,h 2^(m_k,h - M_h),
// write their rows and reset their counters.  Every read goes out before any
// result is needed: the (m, l) of up to 64 pieces per stream (piece k in lane
// k) and the o rows of the first kB pieces per stream, so merging two streams
// of few pieces costs one round trip.  M_h and the sums are wave reductions;
// the weights reach the lanes that accumulate head h through this wave's LDS
// area `red` (head-major, 4 pieces per read).
template <int N>
__device__ __forceinline__ void merge_streams(const Params& p, const MergeJob (&job)[N],
                                              float* red, int lane) {
  const int h = lane >> 4;
  const int d4 = (lane & 15) * 4;
  const __amdgpu_buffer_rsrc_t rso = records_o(p);
  const __amdgpu_buffer_rsrc_t rsml = records_ml(p);
  constexpr int kB = PKV_MERGE_BATCH / N;  // o rows per stream per round trip
  static_assert(kB % 4 == 0, "o rows are weighted 4 pieces per LDS read");
  const int o_off = (h * kD + d4) * 4;
  auto rec = [&](int n, int k) -> int {
    const RecordList& rl = job[n].rl;
    return (int)(rl.base + (int64_t)k * rl.stride + (k == 0 ? rl.first_extra : 0));
  };
  auto load_o = [&](int n, int k) -> f32x4 {
    const int P = job[n].rl.pieces;
    return __builtin_amdgcn_raw_buffer_load_b128(
        rso, rec(n, k < P ? k : P - 1) * (kRecordFloats * 4) + o_off, 0, kSc1);
  };
  // (m, l) of piece c0 + lane of stream n: (m0 l0 m1 l1), (m2 l2 m3 l3)
  auto load_ml = [&](int n, int c0, f32x4& lo, f32x4& hi) {
    const int P = job[n].rl.pieces;
    const int k = c0 + lane;
    const int r = rec(n, k < P ? k : P - 1);
    lo = __builtin_amdgcn_raw_buffer_load_b128(rsml, r * 32, 0, kSc1);
    hi = __builtin_amdgcn_raw_buffer_load_b128(rsml, r * 32 + 16, 0, kSc1);
  };
  // this lane's piece: m and l per head, l = 0 past the stream's pieces
  auto unpack = [&](int n, int c0, const f32x4& lo, const f32x4& hi, float (&m)[4],
                    float (&l)[4]) {
    const bool in = c0 + lane < job[n].rl.pieces;
    m[0] = lo[0]; m[1] = lo[2]; m[2] = hi[0]; m[3] = hi[2];
    l[0] = in ? lo[1] : 0.f; l[1] = in ? lo[3] : 0.f;
    l[2] = in ? hi[1] : 0.f; l[3] = in ? hi[3] : 0.f;
  };
  auto lds_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  f32x4 ob[N][kB];
  f32x4 ml_lo[N], ml_hi[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    load_ml(n, 0, ml_lo[n], ml_hi[n]);
#pragma unroll
    for (int u = 0; u < kB; ++u) ob[n][u] = load_o(n, u);
  }

#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int P = job[n].rl.pieces;
    float m[4], l[4], M[4];
    unpack(n, 0, ml_lo[n], ml_hi[n], m, l);
    // maxima over all pieces (l > 0 only)
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) M[hh] = wave_max_u(l[hh] > 0.f ? m[hh] : -INFINITY);
    for (int c0 = 64; c0 < P; c0 += 64) {
      f32x4 lo, hi;
      float mc[4], lc[4];
      load_ml(n, c0, lo, hi);
      unpack(n, c0, lo, hi, mc, lc);
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
        M[hh] = fmaxf(M[hh], wave_max_u(lc[hh] > 0.f ? mc[hh] : -INFINITY));
    }
    float* wr = red + n * 256;  // weights [head][64 pieces]
    float den_h = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < P; c0 += 64) {
      if (c0 > 0) {
        f32x4 lo, hi;
        load_ml(n, c0, lo, hi);
        unpack(n, c0, lo, hi, m, l);
      }
      lds_sync();  // earlier readers of wr are done
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const float w = l[hh] > 0.f ? l[hh] * __builtin_amdgcn_exp2f(m[hh] - M[hh]) : 0.f;
        wr[hh * 64 + lane] = w;
        const float t = wave_sum_u(w);
        den_h = hh == h ? den_h + t : den_h;
      }
      lds_sync();
      const int cn = P - c0 < 64 ? P - c0 : 64;
      for (int k0 = 0; k0 < cn; k0 += kB) {
        if (c0 + k0 > 0) {
#pragma unroll
          for (int u = 0; u < kB; ++u) ob[n][u] = load_o(n, c0 + k0 + u);
        }
#pragma unroll
        for (int u = 0; u < kB; u += 4) {
          // weights of pieces k0+u .. k0+u+3 (0 past the stream's pieces)
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(wr + h * 64 + (k0 + u < 60 ? k0 + u : 60));
#pragma unroll
          for (int e = 0; e < 4; ++e) num += w4[e] * ob[n][u + e];
        }
      }
    }
    const float inv = den_h > 0.f ? 1.0f / den_h : 0.f;
    const float4 res = make_float4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
    const int64_t row = ((int64_t)job[n].b * p.Hq + 4 * job[n].g + h) * kD + d4;
    if (p.out_f32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row) = res;
    } else {
      u32x2 pk = {pack_bf16(res.x, res.y), pack_bf16(res.z, res.w)};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + row) = pk;
    }
    if (lane == 0)
      __hip_atomic_store(p.ws_count + ((int64_t)job[n].b * p.Hkv + job[n].g) * kCounterStride, 0u,
                         __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
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
  RecordList rl;
  rl.base = (int64_t)stream * parts;
  rl.stride = 1;
  rl.first_extra = 0;
  rl.pieces = (nb + p.part_blocks - 1) / (p.part_blocks > 0 ? p.part_blocks : 1);
  finish_segment(st, p, b, g, complete, unit, rl, red[wave], lane);
  if (!complete) {
    drain_stores();
    if (count_piece(p, b, g, lane) + 1 == (uint32_t)rl.pieces) {
      const MergeJob job[1] = {{b, g, rl}};
      merge_streams<1>(p, job, red[wave], lane);
    }
  }
}

// ---------------------------------------------------------------------------
// kAuto: balanced split over a fixed grid of kAutoWaves wavefronts.
//
// Every stream (b, g) is padded to a multiple of kRing blocks and all streams,
// in (b, g) order, form one global block list whose ring groups are dealt out
// as evenly as possible (shares differ by at most one group), one share per
// wavefront.  So every ring group of kRing
// blocks lies inside one stream, padding blocks are masked (their loads re-read
// a real block of the stream), and a wavefront streams its share through ONE
// continuous ring across stream boundaries: the next group's block ids (scalar
// loads) and query rows (vector loads) are fetched one group ahead, so a new
// stream costs no pipeline drain.  A share holds at most two partial streams
// (its first and last segment); streams strictly inside it are complete and
// written directly.  Record slots: wavefront w owns records 2w (first segment)
// and 2w+1 (last segment).

// First block of wavefront w's share when gbase groups go to every
// wavefront and one more to the first `rem`.
__device__ __forceinline__ int64_t share_start(int64_t w, int64_t gbase, int64_t rem) {
  return (int64_t)kRing * (w * gbase + (w < rem ? w : rem));
}

// Wavefront whose share holds block x.
__device__ __forceinline__ int64_t share_of(int64_t x, int64_t gbase, int64_t rem) {
  const int64_t gx = x / kRing;
  const int64_t big = rem * (gbase + 1);
  if (gx < big) return gx / (gbase + 1);
  return rem + (gx - big) / gbase;
}

__device__ __forceinline__ int padded_blocks(int ctx) {
  const int nb = (ctx + kBS - 1) / kBS;
  return (nb + kRing - 1) / kRing * kRing;
}

// Position in the padded block list; every field is wave-uniform.
struct Cursor {
  int b, g, j;      // stream (b, g), block j of it (a multiple of kRing)
  int nbp, nbr;     // padded and real block counts of the stream
  int ctx;          // context length of sequence b
};

__device__ __forceinline__ void cursor_load_seq(Cursor& c, const int* s_ctx, int b) {
  c.b = b;
  c.ctx = __builtin_amdgcn_readfirstlane(s_ctx[b]);
  c.nbr = (c.ctx + kBS - 1) / kBS;
  c.nbp = (c.nbr + kRing - 1) / kRing * kRing;
}

// Move one ring group forward (only called while the target is inside the
// list, so b stays below B).
__device__ __forceinline__ void cursor_advance(Cursor& c, const int* s_ctx, int Hkv, int B) {
  c.j += kRing;
  if (c.j < c.nbp) return;
  c.j = 0;
  if (++c.g < Hkv) return;
  c.g = 0;
  int b = c.b + 1;
  while (b < B - 1 && __builtin_amdgcn_readfirstlane(s_ctx[b]) == 0) ++b;
  cursor_load_seq(c, s_ctx, b < B ? b : B - 1);  // b < B whenever a group follows
}

// Block-id window: lane k returns the physical id of block xs + k of the
// padded list (the cursor c sits at xs), clamped to its stream's last real
// block; 0 past x1.  One vector load per 64 blocks; ids are then read with
// readlane, so no scalar-load wait ever sits between two ring groups.
__device__ __forceinline__ int id_window(const Params& p, const int* s_ctx, const Cursor& c,
                                         int64_t xs, int64_t x1, int lane) {
  if (xs + lane >= x1) return 0;
  int b = c.b, g = c.g, j = c.j, nbp = c.nbp, nbr = c.nbr;
  int k = lane;
  while (k >= nbp - j) {
    k -= nbp - j;
    j = 0;
    if (++g == p.Hkv) {
      g = 0;
      do {
        ++b;
      } while (b < p.B - 1 && s_ctx[b] == 0);
      if (b >= p.B) return -1;  // not reached while the list holds xs + lane
      nbr = (s_ctx[b] + kBS - 1) / kBS;
      nbp = (nbr + kRing - 1) / kRing * kRing;
    }
  }
  if (nbr <= 0) return -1;  // not reached: streams without blocks are not in the list
  j += k;
  const int jj = j < nbr - 1 ? j : nbr - 1;
  return p.block_tables[(int64_t)b * p.max_blocks + jj];
}

__device__ __forceinline__ void load_q(uint32_t (&qv)[4][4], const Params& p, int b, int g,
                                       int i, int c) {
  const uint16_t* qb = p.q + ((int64_t)b * p.Hq + 4 * g) * kD + 8 * i;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 v = *reinterpret_cast<const u32x4*>(qb + (j ^ c) * kD);
#pragma unroll
    for (int w = 0; w < 4; ++w) qv[j][w] = v[w];
  }
}

// Append variant: chunk i of the new token's K and V rows of stream (b, g).
__device__ __forceinline__ void load_new(u32x4& kn, u32x4& vn, const Params& p, int b, int g,
                                         int i) {
  const int64_t off = ((int64_t)b * p.Hkv + g) * kD + 8 * i;
  kn = *reinterpret_cast<const u32x4*>(p.k_new + off);
  vn = *reinterpret_cast<const u32x4*>(p.v_new + off);
}

__device__ __forceinline__ void reset_state(LaneState& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[j][e] = 0.f;
}

// Stream and block of list position x0: largest b with Hkv * pfx[b] <= x0.
__device__ __forceinline__ void locate_share(Cursor& cc, const Params& p, const int* pfx,
                                             const int* s_ctx, int64_t x0) {
  int lo = 0, hi = p.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)p.Hkv * pfx[mid] <= x0) lo = mid; else hi = mid;
  }
  cursor_load_seq(cc, s_ctx, __builtin_amdgcn_readfirstlane(lo));
  const int64_t off = x0 - (int64_t)p.Hkv * __builtin_amdgcn_readfirstlane(pfx[cc.b]);
  cc.g = (int)(off / cc.nbp);
  cc.j = (int)(off - (int64_t)cc.g * cc.nbp);
}

// Context lengths (clamped) of all sequences and the exclusive prefix of
// their padded block counts, in LDS (pfx[B] = total); with kAppend also
// whether each sequence's new token is stored by the wavefronts.
template <bool kAppend>
__device__ __forceinline__ void block_prefix(const Params& p, int* pfx, int* s_ctx,
                                             unsigned char* s_newok, int* wsum, int tid,
                                             int lane, int wave) {
  const int per = (p.B + kWaves * 64 - 1) / (kWaves * 64);
  const int beg = tid * per;
  const int end = beg + per < p.B ? beg + per : p.B;
  int local = 0;
  for (int k = beg; k < end; ++k) {
    const int c = eff_ctx(p, k);
    s_ctx[k] = c;
    if (kAppend) s_newok[k] = c >= 1 && c == p.context_lens[k];
    local += padded_blocks(c);
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w2 = 0; w2 < wave; ++w2) run += wsum[w2];
  for (int k = beg; k < end; ++k) {
    pfx[k] = run;
    run += padded_blocks(s_ctx[k]);
  }
  if (tid == kWaves * 64 - 1) pfx[p.B] = run;
  __syncthreads();
}

// The plan of the balanced split for this call's lengths and tables: what
// decode_auto_kernel computes before its first load (the prefix of padded
// block counts, each wavefront's first stream and the block ids of its first
// 64 list positions), stored once so that calls which share lengths and
// tables (every layer of a decode step) start loading keys at once.
__global__ void __launch_bounds__(kWaves * 64)
decode_plan_kernel(Params p) {
  __shared__ int pfx[kAutoMaxBatch + 1];
  __shared__ int s_ctx[kAutoMaxBatch];
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  block_prefix<false>(p, pfx, s_ctx, nullptr, wsum, tid, lane, wave);
  const int64_t NB = (int64_t)p.Hkv * __builtin_amdgcn_readfirstlane(pfx[p.B]);
  const int W = gridDim.x * kWaves;
  const int64_t G = NB / kRing;
  const int64_t gbase = G / W;
  const int64_t rem = G - gbase * W;
  if (blockIdx.x == 0) {
    for (int k = tid; k <= p.B; k += kWaves * 64) {
      p.plan[kPlanHeaderInts + k] = pfx[k];
      if (k < p.B) p.plan[kPlanCtxOffset + k] = s_ctx[k];
    }
    if (tid < kPlanHeaderInts) {
      const int hdr[7] = {kPlanMagic, p.B, p.Hkv, p.max_blocks, p.ctx_cap, p.num_blocks, W};
      p.plan[tid] = tid < 7 ? hdr[tid] : 0;
    }
  }
  const int w = blockIdx.x * kWaves + wave;
  const int64_t x0 = share_start(w, gbase, rem);
  const int64_t x1 = share_start(w + 1, gbase, rem);
  int* ent = p.plan + kPlanWaveOffset + (int64_t)w * kPlanWaveInts;
  Cursor cc = {};
  int tab = 0;
  if (x0 < x1) {
    locate_share(cc, p, pfx, s_ctx, x0);
    tab = id_window(p, s_ctx, cc, x0, x1, lane);
  }
  ent[4 + lane] = tab;
  if (lane < 4) ent[lane] = lane == 0 ? cc.b : lane == 1 ? cc.g : lane == 2 ? cc.j : cc.ctx;
}

//
// kAppend: the call also stores one new token per sequence (kv_append with
// one token each).  The new token is the last of its sequence, so it lies in
// the stream's last block, which exactly one wavefront consumes: that
// wavefront writes the token's K and V rows into the pools and uses them
// from registers in place of the (stale) rows its load returned.  The rows
// of a sequence clamped to max_context_len are stored by a workgroup during
// set-up; slots outside the table or pool are not written (as kv_append).
template <bool kAppend, bool kPlanned>
__global__ void __launch_bounds__(kWaves * 64)
decode_auto_kernel(Params p) {
  __shared__ float red[kWaves][8 * 4 * kD];
  __shared__ int pfx[kAutoMaxBatch + 1];
  __shared__ int s_ctx[kAutoMaxBatch];
  __shared__ int wsum[kWaves];
  __shared__ unsigned char s_newok[kAppend ? kAutoMaxBatch : 1];  // append this sequence
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // per-sequence context lengths and the exclusive prefix of their padded
  // block counts in LDS: read from the plan when one matches this call
  const int grp = lane >> 3, i = lane & 7;
  const bool quad1 = (i & 4) != 0;
  const int c = quad1 ? ((i & 3) ^ 3) : (i & 3);
  const int own_tok = quad1 ? grp + 8 : grp;
  const int lane_off = grp * kD + 8 * i;
  BlockRegs ring[kRing];
  int nvalid[kRing];
  int64_t ub[kRing];  // element offsets of the slots' blocks, for their V loads
  bool slast[kRing];  // append: the slot holds its stream's last block
  int sphys[kRing];   // append: that block's physical id
  uint32_t qv[4][4], qn[4][4];
  u32x4 knv, vnv, knn, vnn;  // append: new-token chunks (consumed / next group)
  // Issue the first group of the share starting at stream position ci
  // (id window tab, whose lane 0 is the group's first block).
  auto prologue = [&](const Cursor& ci, int tab) {
    load_q(qn, p, ci.b, ci.g, i, c);
    if (kAppend) load_new(knn, vnn, p, ci.b, ci.g, i);
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      const int j = ci.j + s < ci.nbr - 1 ? ci.j + s : ci.nbr - 1;
      const int id = __builtin_amdgcn_readlane(tab, s);
      const int nv = issue_block(ring[s], p, id, ci.g, j, ci.ctx, lane_off);
      nvalid[s] = ci.j + s < ci.nbr ? nv : 0;
      if (kAppend) {
        slast[s] = ci.j + s == ci.nbr - 1 && nv > 0;
        sphys[s] = id;
      }
    }
  };

  // With a plan: its first group is issued at once, before the plan is
  // checked against this call (the block ids are range-checked, so the loads
  // stay inside the pools whatever the plan holds); the context lengths and
  // the prefix come from the plan too.  A plan made for other lengths or
  // another shape is not used: the split is computed and the first group
  // issued again.
  bool use_plan = false, issued = false;
  int pl_b = 0, pl_g = 0, pl_j = 0, pl_tab = 0;
  // this thread's first sequence (k = tid): plan prefix, plan length and
  // length, loaded before the first group so that waiting for them does not
  // wait for its keys (vector loads complete in order)
  int v_pfx = 0, v_pctx = 0, v_len = 0;
  if (kPlanned) {
    if (tid <= p.B) v_pfx = p.plan[kPlanHeaderInts + tid];
    if (tid < p.B) {
      v_pctx = p.plan[kPlanCtxOffset + tid];
      v_len = p.context_lens[tid];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int w = blockIdx.x * kWaves + wave;
    const int* ent = p.plan + kPlanWaveOffset + (int64_t)w * kPlanWaveInts;
    pl_tab = ent[4 + lane];
    pl_b = ld_uniform(ent, 0);
    pl_g = ld_uniform(ent, 1);
    pl_j = ld_uniform(ent, 2);
    const int pl_ctx = ld_uniform(ent, 3);
    use_plan = ld_uniform(p.plan, 0) == kPlanMagic && ld_uniform(p.plan, 1) == p.B &&
               ld_uniform(p.plan, 2) == p.Hkv && ld_uniform(p.plan, 3) == p.max_blocks &&
               ld_uniform(p.plan, 4) == p.ctx_cap && ld_uniform(p.plan, 5) == p.num_blocks &&
               ld_uniform(p.plan, 6) == (int)(gridDim.x * kWaves);
    if (use_plan && pl_ctx > 0 && pl_ctx <= p.ctx_cap && pl_b >= 0 && pl_b < p.B && pl_g >= 0 &&
        pl_g < p.Hkv && pl_j >= 0) {
      Cursor sc;
      sc.b = pl_b;
      sc.ctx = pl_ctx;
      sc.nbr = (pl_ctx + kBS - 1) / kBS;
      sc.nbp = (sc.nbr + kRing - 1) / kRing * kRing;
      sc.g = pl_g;
      sc.j = pl_j;
      prologue(sc, pl_tab);
      issued = true;
    }
  }
  if (use_plan) {
    __builtin_amdgcn_sched_barrier(0);
    if (tid == 0) wsum[0] = 0;
    bool stale = false;
    for (int k = tid; k <= p.B; k += kWaves * 64) {
      const bool first = k == tid;
      pfx[k] = first ? v_pfx : p.plan[kPlanHeaderInts + k];
      if (k < p.B) {
        int cx = first ? v_len : p.context_lens[k];
        if (kAppend) s_newok[k] = cx >= 1 && cx <= p.ctx_cap;
        cx = cx < 0 ? 0 : (cx > p.ctx_cap ? p.ctx_cap : cx);  // as eff_ctx
        s_ctx[k] = cx;
        // the plan must have been made for exactly these lengths
        stale = stale || (first ? v_pctx : p.plan[kPlanCtxOffset + k]) != cx;
      }
    }
    __syncthreads();
    if (stale) wsum[0] = 1;
    __syncthreads();
    if (wsum[0] != 0) {
      use_plan = false;
      __syncthreads();  // everyone has read the flag before wsum is reused
    }
  }
  if (!use_plan) block_prefix<kAppend>(p, pfx, s_ctx, s_newok, wsum, tid, lane, wave);

  // ring groups are dealt out as evenly as possible: the first `rem`
  // wavefronts take gbase + 1 groups, the others gbase
  const int64_t NB = (int64_t)p.Hkv * __builtin_amdgcn_readfirstlane(pfx[p.B]);
  const int W = gridDim.x * kWaves;
  const int64_t G = NB / kRing;
  const int64_t gbase = G / W;
  const int64_t rem = G - gbase * W;
  // empty sequences have no blocks, so no wavefront meets them: workgroup
  // k % grid writes their zero rows
  for (int k = blockIdx.x; k < p.B; k += gridDim.x) {
    if (s_ctx[k] == 0) {
      for (int e = tid; e < p.Hq * kD; e += kWaves * 64) {
        const int64_t idx = (int64_t)k * p.Hq * kD + e;
        if (p.out_f32) reinterpret_cast<float*>(p.out)[idx] = 0.f;
        else reinterpret_cast<uint16_t*>(p.out)[idx] = 0;
      }
    }
    // a sequence cut short by the clamp still gets its token stored (no
    // wavefront reads that row): workgroup k % grid copies it
    if (kAppend && !s_newok[k]) {
      const int len = p.context_lens[k];
      if (len >= 1 && len <= p.max_blocks * kBS) {
        const int pos = len - 1;
        const int id = p.block_tables[(int64_t)k * p.max_blocks + pos / kBS];
        if (id >= 0 && id < p.num_blocks) {
          for (int e = tid; e < p.Hkv * (kD / 8); e += kWaves * 64) {
            const int g = e / (kD / 8), ch = e % (kD / 8);
            u32x4 kn, vn;
            load_new(kn, vn, p, k, g, ch);
            const int64_t off = (((int64_t)id * p.Hkv + g) * kBS + pos % kBS) * kD + 8 * ch;
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.k_cache) + off) = kn;
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.v_cache) + off) = vn;
          }
        }
      }
    }
  }
  const int w = blockIdx.x * kWaves + wave;
  const int64_t x0 = share_start(w, gbase, rem);
  const int64_t x1 = share_start(w + 1, gbase, rem);
  if (x0 >= x1) return;

  // locate x0 (or take it from the plan)
  Cursor cc;
  if (use_plan) {
    cursor_load_seq(cc, s_ctx, pl_b);
    cc.g = pl_g;
    cc.j = pl_j;
  } else {
    locate_share(cc, p, pfx, s_ctx, x0);
  }

  // prologue: id window and q of the first group, then issue it
  Cursor ci = cc;
  int64_t xi = x0;
  int64_t win = x0;
  int tab = use_plan ? pl_tab : id_window(p, s_ctx, ci, x0, x1, lane);
  if (!(use_plan && issued)) prologue(ci, tab);
  if (xi + kRing < x1) {
    xi += kRing;
    cursor_advance(ci, s_ctx, p.Hkv, p.B);
  } else {
    xi = x1;  // nothing left to issue: further refills re-read this group
  }
  // refills re-read the last issued group once the share is used up
  int64_t xr = xi < x1 ? xi : xi - kRing;
  if (xr - win + kRing > 64) {
    win = xr;
    tab = id_window(p, s_ctx, ci, xr, x1, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // pieces of split streams this share holds (at most its first and last)
  int pend = 0, pb0 = 0, pg0 = 0, pb1 = 0, pg1 = 0;
  RecordList prl0 = {}, prl1 = {};

  LaneState st;
  reset_state(st);
  int64_t seg_start = x0;  // where the current segment began in this share
  for (int64_t xc = x0; xc < x1; xc += kRing) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) qv[j][w2] = qn[j][w2];
    if (kAppend) {
      knv = knn;
      vnv = vnn;
      // the new token's row replaces the one loaded from the pools (its K
      // here, its V before the slot's P.V), and is stored there (lanes
      // grp == t % 8 hold token t in ka/va or kb/vb)
#pragma unroll
      for (int s = 0; s < kRing; ++s) {
        if (slast[s] && s_newok[cc.b]) {
          const int t = (cc.ctx - 1) & (kBS - 1);
          if (grp == t) ring[s].ka = knv;
          if (grp + 8 == t) ring[s].kb = knv;
          if (grp == (t & 7)) {
            const int64_t off = (((int64_t)sphys[s] * p.Hkv + cc.g) * kBS + t) * kD + 8 * i;
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.k_cache) + off) = knv;
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.v_cache) + off) = vnv;
          }
        }
      }
    }

    bool full = true;
#pragma unroll
    for (int s = 0; s < kRing; ++s) full = full && nvalid[s] == kBS;
    float x[kRing];
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      x[s] = block_score(ring[s], qv, p.scale_log2, quad1);
      if (!full && own_tok >= nvalid[s]) x[s] = -INFINITY;
    }
    // q, the new rows and the K halves of the group at ci go out now (a
    // re-read when none is left), so they are in flight while this group is
    // accumulated; each slot's V half follows its P.V
    load_q(qn, p, ci.b, ci.g, i, c);
    if (kAppend) load_new(knn, vnn, p, ci.b, ci.g, i);
    int nv_next[kRing];
    bool slast_next[kRing];
    int sphys_next[kRing];
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      const int j = ci.j + s < ci.nbr - 1 ? ci.j + s : ci.nbr - 1;
      const int id = __builtin_amdgcn_readlane(tab, (int)(xr - win) + s);
      const int nv = issue_k(ring[s], p, id, ci.g, j, ci.ctx, lane_off, ub[s]);
      nv_next[s] = ci.j + s < ci.nbr ? nv : 0;
      if (kAppend) {
        slast_next[s] = ci.j + s == ci.nbr - 1 && nv > 0;
        sphys_next[s] = id;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int s = 1; s < kRing; ++s) mx = fmaxf(mx, x[s]);
    mx = fmaxf(mx, dpp<kRowHalfMirror>(mx));
    const float m_new = fmaxf(st.m, mx);
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
      const float pw = __builtin_amdgcn_exp2f(x[s] - m_use);
      st.l += pw;
      if (kAppend && slast[s] && s_newok[cc.b]) {
        const int t = (cc.ctx - 1) & (kBS - 1);
        if (grp == t) ring[s].va = vnv;
        if (grp + 8 == t) ring[s].vb = vnv;
      }
      if (full)
        block_pv<false>(st, ring[s], pw, quad1, true, true);
      else
        block_pv<true>(st, ring[s], pw, quad1, grp < nvalid[s], grp + 8 < nvalid[s]);
      issue_v(ring[s], p, ub[s], lane_off);
      nvalid[s] = nv_next[s];
      if (kAppend) {
        slast[s] = slast_next[s];
        sphys[s] = sphys_next[s];
      }
    }
    if (xi + kRing < x1) {
      xi += kRing;
      cursor_advance(ci, s_ctx, p.Hkv, p.B);
    } else {
      xi = x1;
    }
    xr = xi < x1 ? xi : xi - kRing;
    if (xr - win + kRing > 64) {
      win = xr;
      tab = id_window(p, s_ctx, ci, xr, x1, lane);
      // wait here (vmcnt 0), inside the branch, so the common path carries
      // no wait for this load
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }

    // segment end: the stream ends here or the share does
    const bool stream_ends = cc.j + kRing == cc.nbp;
    if (stream_ends || xc + kRing >= x1) {
      const int64_t stream_start =
          (int64_t)p.Hkv * __builtin_amdgcn_readfirstlane(pfx[cc.b]) + (int64_t)cc.g * cc.nbp;
      const bool complete = stream_ends && stream_start >= seg_start;
      const int record = 2 * w + (stream_start <= x0 ? 0 : 1);
      const int64_t w0 = share_of(stream_start, gbase, rem);
      RecordList rl;
      rl.base = 2 * w0;
      rl.stride = 2;
      rl.first_extra = stream_start > share_start(w0, gbase, rem) ? 1 : 0;
      rl.pieces = (int)(share_of(stream_start + cc.nbp - 1, gbase, rem) - w0 + 1);
      finish_segment(st, p, cc.b, cc.g, complete, record, rl, red[wave], lane);
      if (!complete) {
        if (pend == 0) {
          pb0 = cc.b; pg0 = cc.g; prl0 = rl;
        } else {
          pb1 = cc.b; pg1 = cc.g; prl1 = rl;
        }
        ++pend;
      }
      reset_state(st);
      seg_start = xc + kRing;
    }
    if (xc + kRing < x1) cursor_advance(cc, s_ctx, p.Hkv, p.B);
  }
  // count this share's split pieces only now: one drain instead of one per
  // segment in the middle of the stream
  if (pend) {
    drain_stores();
    // both counts go out before either result is needed
    const uint32_t c0 = count_piece(p, pb0, pg0, lane);
    const uint32_t c1 = pend > 1 ? count_piece(p, pb1, pg1, lane) : 0u;
    const bool m0 = c0 + 1 == (uint32_t)prl0.pieces;
    const bool m1 = pend > 1 && c1 + 1 == (uint32_t)prl1.pieces;
    if (m0 && m1) {  // both streams: their reads share one round trip
      const MergeJob job[2] = {{pb0, pg0, prl0}, {pb1, pg1, prl1}};
      merge_streams<2>(p, job, red[wave], lane);
    } else if (m0 || m1) {
      const MergeJob job[1] = {m0 ? MergeJob{pb0, pg0, prl0} : MergeJob{pb1, pg1, prl1}};
      merge_streams<1>(p, job, red[wave], lane);
    }
  }
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
  p.ws_count = a.ws_count;
  p.n_records = (int)decode_records(a.mode, a.B, a.Hkv, a.parts_max);
  p.k_new = (const uint16_t*)a.k_new;
  p.v_new = (const uint16_t*)a.v_new;
  p.plan = a.plan;
  const int streams = a.B * a.Hkv;
  if (a.mode == kWhole) {
    const int grid = (streams + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(decode_units_kernel<kWhole>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
  } else if (a.mode == kFixed) {
    const int64_t units = (int64_t)streams * a.parts_max;
    const int grid = (int)((units + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(decode_units_kernel<kFixed>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
  } else {
    const dim3 grid(kAutoWaves / kWaves), block(kWaves * 64);
    if (a.write_plan)
      hipLaunchKernelGGL(decode_plan_kernel, grid, block, 0, stream, p);
    else if (a.k_new && a.plan)
      hipLaunchKernelGGL((decode_auto_kernel<true, true>), grid, block, 0, stream, p);
    else if (a.k_new)
      hipLaunchKernelGGL((decode_auto_kernel<true, false>), grid, block, 0, stream, p);
    else if (a.plan)
      hipLaunchKernelGGL((decode_auto_kernel<false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_auto_kernel<false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
