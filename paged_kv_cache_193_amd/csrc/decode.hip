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

__device__ __forceinline__ int eff_ctx(const Params& p, int b) {
  int c = p.context_lens[b];
  c = c < 0 ? 0 : c;
  return c > p.ctx_cap ? p.ctx_cap : c;
}

// Issue the two 16-byte K loads of block `j` of the stream, whose physical id
// `phys` was read earlier; `ub` receives the block's element offset for the
// matching V loads (issue_v).  Returns the number of valid tokens in the
// block (0 when `phys` is not a valid block id: then block 0 is read and
// ignored).  K and V are read once per call and never again by it, so their
// loads carry the non-temporal hint: the streamed bytes do not displace the
// plan, the block tables and the split records from the caches.
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
  r.ka = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp));
  r.kb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 8 * kD));
  return nv;
}

// The two 16-byte V loads of the block whose K issue_k issued.
__device__ __forceinline__ void issue_v(BlockRegs& r, const Params& p, int64_t ub,
                                        int lane_off) {
  const uint16_t* vp = p.v_cache + ub + lane_off;
  r.va = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp));
  r.vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + 8 * kD));
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

// Combine the 64 lanes' states of a finished segment and write either the
// final rows out[b][4g..4g+3][:] or a split record.  red: this wave's 8 KB.
__device__ __forceinline__ void finish_segment(const LaneState& st, const Params& p, int b,
                                               int g, bool complete, int record,
                                               float* red, int lane) {
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
// whose addition completes the count merges the pieces (merge_stream).
__device__ __forceinline__ uint32_t count_piece(const Params& p, int b, int g, int lane) {
  uint32_t before = 0;
  if (lane == 0)
    before = __hip_atomic_fetch_add(p.ws_count + ((int64_t)b * p.Hkv + g) * kCounterStride, 1u,
                                    __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readfirstlane(before);
}

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

// Merge the P pieces of stream (b, g), whose records are base .. base + P - 1,
// by log-sum-exp,
//   out_h = sum_k w_k,h o_k,h / sum_k w_k,h,   w_k,h = l_k,h 2^(m_k,h - M_h),
// write its rows and reset its counter.  Every read goes out before any
// result is needed: the (m, l) of up to 64 pieces (piece k in lane k) and the
// o rows of the first kB pieces, so merging a stream of up to kB pieces costs
// one round trip.  M_h and the sums are wave reductions; the weights reach
// the lanes that accumulate head h through this wave's LDS area `red`
// (head-major, 4 pieces per read).
__device__ __forceinline__ void merge_stream(const Params& p, int b, int g, int base, int P,
                                             float* red, int lane) {
  const int h = lane >> 4;
  const int d4 = (lane & 15) * 4;
  const __amdgpu_buffer_rsrc_t rso = records_o(p);
  const __amdgpu_buffer_rsrc_t rsml = records_ml(p);
  constexpr int kB = PKV_MERGE_BATCH;  // o rows per round trip
  static_assert(kB % 4 == 0 && 64 % kB == 0, "o rows are weighted 4 pieces per LDS read");
  const int o_off = (h * kD + d4) * 4;
  // piece k, clamped to the last (reads past the stream repeat it, weight 0)
  auto rec = [&](int k) -> int { return base + (k < P ? k : P - 1); };
  auto load_o = [&](int k) -> f32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rso, rec(k) * (kRecordFloats * 4) + o_off, 0,
                                                 kSc1);
  };
  // (m, l) of piece c0 + lane: (m0 l0 m1 l1), (m2 l2 m3 l3)
  auto load_ml = [&](int c0, f32x4& lo, f32x4& hi) {
    const int r = rec(c0 + lane);
    lo = __builtin_amdgcn_raw_buffer_load_b128(rsml, r * 32, 0, kSc1);
    hi = __builtin_amdgcn_raw_buffer_load_b128(rsml, r * 32 + 16, 0, kSc1);
  };
  // this lane's piece: m and l per head, l = 0 past the stream's pieces
  auto unpack = [&](int c0, const f32x4& lo, const f32x4& hi, float (&m)[4], float (&l)[4]) {
    const bool in = c0 + lane < P;
    m[0] = lo[0]; m[1] = lo[2]; m[2] = hi[0]; m[3] = hi[2];
    l[0] = in ? lo[1] : 0.f; l[1] = in ? lo[3] : 0.f;
    l[2] = in ? hi[1] : 0.f; l[3] = in ? hi[3] : 0.f;
  };
  auto lds_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  f32x4 ob[kB];
  f32x4 ml_lo, ml_hi;
  load_ml(0, ml_lo, ml_hi);
#pragma unroll
  for (int u = 0; u < kB; ++u) ob[u] = load_o(u);

  float m[4], l[4], M[4];
  unpack(0, ml_lo, ml_hi, m, l);
  // maxima over all pieces (l > 0 only)
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) M[hh] = wave_max_u(l[hh] > 0.f ? m[hh] : -INFINITY);
  for (int c0 = 64; c0 < P; c0 += 64) {
    f32x4 lo, hi;
    float mc[4], lc[4];
    load_ml(c0, lo, hi);
    unpack(c0, lo, hi, mc, lc);
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
      M[hh] = fmaxf(M[hh], wave_max_u(lc[hh] > 0.f ? mc[hh] : -INFINITY));
  }
  float den_h = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < P; c0 += 64) {
    if (c0 > 0) {
      f32x4 lo, hi;
      load_ml(c0, lo, hi);
      unpack(c0, lo, hi, m, l);
    }
    lds_sync();  // earlier readers of red are done
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float w = l[hh] > 0.f ? l[hh] * __builtin_amdgcn_exp2f(m[hh] - M[hh]) : 0.f;
      red[hh * 64 + lane] = w;  // weights [head][64 pieces]
      const float t = wave_sum_u(w);
      den_h = hh == h ? den_h + t : den_h;
    }
    lds_sync();
    const int cn = P - c0 < 64 ? P - c0 : 64;
    for (int k0 = 0; k0 < cn; k0 += kB) {
      if (c0 + k0 > 0) {
#pragma unroll
        for (int u = 0; u < kB; ++u) ob[u] = load_o(c0 + k0 + u);
      }
#pragma unroll
      for (int u = 0; u < kB; u += 4) {
        // weights of pieces k0+u .. k0+u+3 (0 past the stream's pieces)
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(red + h * 64 + k0 + u);
#pragma unroll
        for (int e = 0; e < 4; ++e) num += w4[e] * ob[u + e];
      }
    }
  }
  const float inv = den_h > 0.f ? 1.0f / den_h : 0.f;
  const float4 res = make_float4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
  const int64_t row = ((int64_t)b * p.Hq + 4 * g + h) * kD + d4;
  if (p.out_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row) = res;
  } else {
    u32x2 pk = {pack_bf16(res.x, res.y), pack_bf16(res.z, res.w)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + row) = pk;
  }
  if (lane == 0)
    __hip_atomic_store(p.ws_count + ((int64_t)b * p.Hkv + g) * kCounterStride, 0u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void write_zero_rows(const Params& p, int b, int g, int lane) {
  const int h = lane >> 4, d4 = (lane & 15) * 4;
  const int64_t row = ((int64_t)b * p.Hq + 4 * g + h) * kD + d4;
  if (p.out_f32)
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row) = make_float4(0.f, 0.f, 0.f, 0.f);
  else
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + row) = u32x2{0, 0};
}

// ---------------------------------------------------------------------------
// kAuto: stream-aligned pieces, one per wavefront.
//
// The batch's blocks are cut into pieces, each inside one stream (sequence b,
// KV head g).  A piece holds at most P blocks: the smallest bound (at least
// kMinPiece) whose pieces fit the grid of W = kAutoWaves wavefronts, found by
// a short search between ceil(NB * Hkv / W) and the bound that leaves one
// wavefront per stream spare,
//     max(kMinPiece, ceil(NB * Hkv / max(W - S, W / 4))),
// for NB blocks over the sequences and S = B * Hkv streams (that bound alone
// when there are more than 3W/4 streams and the grid grows).  A
// stream of nb blocks is cut into u = ceil(nb / P) pieces of equal length
// (piece k: blocks [k nb / u, (k + 1) nb / u)); an empty stream is one piece
// that writes zero rows.  That makes at most W pieces when S <= 3W/4 and at
// most W/4 + S otherwise; the grid has that many wavefronts (auto_waves), and
// wavefront w takes piece w of the numbering stream by stream in (b, g)
// order.  A piece loads its stream's queries once and runs its own ring of
// kRing blocks, so nothing crosses a stream boundary.  A piece that is a
// whole stream writes the output rows; the pieces of a cut stream write
// records, numbered over the cut streams only, and the last of a stream to
// finish merges them.  A cut stream has nb > P blocks and fewer than 2 nb / P
// pieces, so there are fewer than 2 * max(W - S, W / 4) <= 2W records.
// Pieces shorter than kMinPiece blocks would cost more in start-up and
// merging than their parallelism gains.
constexpr int kMinPiece = 8;

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


__device__ __forceinline__ int piece_bound(int64_t nb_total, int B, int Hkv, int W) {
  const int64_t S = (int64_t)B * Hkv;
  const int64_t spare = W - S > W / 4 ? W - S : W / 4;
  const int64_t P = (nb_total * Hkv + spare - 1) / spare;
  return P < kMinPiece ? kMinPiece : (int)(P < (1 << 30) ? P : (1 << 30));
}

__device__ __forceinline__ int pieces_of(int nb, int P) { return nb == 0 ? 1 : (nb + P - 1) / P; }

// Per-sequence prefix word: pieces before the sequence (per KV head) in the
// low 16 bits, records of cut streams before it (per KV head) in the high 16.
// Both totals stay below 2^16 (at most W/4 + B <= 4608 pieces and fewer than
// 2W = 4096 records per KV head), so the two fields add without carrying
// into each other.
__device__ __forceinline__ int prefix_word(int nb, int P) {
  const int n = pieces_of(nb, P);
  return n | ((n > 1 ? n : 0) << 16);
}
__device__ __forceinline__ int pu_pieces(int w) { return w & 0xFFFF; }
__device__ __forceinline__ int pu_records(int w) { return (int)((unsigned)w >> 16); }

// Context lengths (clamped) of all sequences in LDS, the piece bound P
// (returned) and the exclusive prefix words of the sequences (pu[B]: the
// totals); with kAppend also whether each sequence's new token is read by
// its stream's last piece.
template <bool kAppend>
__device__ __forceinline__ int piece_prefix(const Params& p, int* pu, int* s_ctx,
                                            unsigned char* s_newok, int* wsum,
                                            long long* wtot, int tid, int lane, int wave) {
  const int per = (p.B + kWaves * 64 - 1) / (kWaves * 64);
  const int beg = tid * per;
  const int end = beg + per < p.B ? beg + per : p.B;
  long long nbs = 0;
  for (int k = beg; k < end; ++k) {
    const int c = eff_ctx(p, k);
    s_ctx[k] = c;
    if (kAppend) s_newok[k] = c >= 1 && c == p.context_lens[k];
    nbs += (c + kBS - 1) / kBS;
  }
  for (int off = 32; off >= 1; off >>= 1) nbs += __shfl_xor(nbs, off);
  if (lane == 0) wtot[wave] = nbs;
  __syncthreads();
  long long tot = 0;
  for (int w2 = 0; w2 < kWaves; ++w2) tot += wtot[w2];
  // the smallest bound whose pieces still fit the grid: piece counts only
  // fall as the bound grows, and piece_bound's value fits.  Searched on the
  // fixed grid only (there records <= pieces <= W; a grid grown for many
  // streams keeps piece_bound's value, whose cut pieces stay below W / 2).
  // Every wavefront searches on its own over the lengths in LDS, so the
  // search needs no barrier.
  const int64_t grid_waves = (int64_t)gridDim.x * kWaves;
  int hi = piece_bound(tot, p.B, p.Hkv, kAutoWaves);
  // no bound below ceil(NB * Hkv / W) fits: the search starts there
  const long long floor_p = (tot * p.Hkv + grid_waves - 1) / grid_waves;
  int lo = grid_waves == kAutoWaves
               ? (int)(floor_p > kMinPiece ? (floor_p < hi ? floor_p : hi) : kMinPiece) - 1
               : hi;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    // per-lane counts clamped at 2^17, so the wave's float sum (DPP rows,
    // then readlane) is exact wherever the comparison is close
    int n = 0;
    for (int k = lane; k < p.B; k += 64) {
      n += pieces_of((s_ctx[k] + kBS - 1) / kBS, mid);
      n = n < (1 << 17) ? n : (1 << 17);
    }
    const float all = wave_sum_u((float)n);
    if ((double)all * p.Hkv <= (double)grid_waves) hi = mid; else lo = mid;
  }
  const int P = hi;
  int local = 0;
  for (int k = beg; k < end; ++k) local += prefix_word((s_ctx[k] + kBS - 1) / kBS, P);
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
    pu[k] = run;
    run += prefix_word((s_ctx[k] + kBS - 1) / kBS, P);
  }
  if (tid == kWaves * 64 - 1) pu[p.B] = run;
  __syncthreads();
  return P;
}

// Piece u of the numbering: its stream (b, g), its blocks [j0, j1), its
// index k in the stream, the stream's piece count and (cut streams) the
// record number of the stream's first piece.
struct Piece {
  int b, g, j0, j1, ctx, pieces, base, k;
};

__device__ __forceinline__ Piece locate_piece(const Params& p, const int* pu, const int* s_ctx,
                                              int64_t u) {
  int lo = 0, hi = p.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)p.Hkv * pu_pieces(pu[mid]) <= u) lo = mid; else hi = mid;
  }
  Piece pc;
  pc.b = __builtin_amdgcn_readfirstlane(lo);
  const int w0 = __builtin_amdgcn_readfirstlane(pu[pc.b]);
  const int first = pu_pieces(w0);
  pc.pieces = pu_pieces(__builtin_amdgcn_readfirstlane(pu[pc.b + 1])) - first;
  const int off = (int)(u - (int64_t)p.Hkv * first);
  pc.g = off / pc.pieces;
  pc.k = off - pc.g * pc.pieces;
  pc.ctx = __builtin_amdgcn_readfirstlane(s_ctx[pc.b]);
  const int nb = (pc.ctx + kBS - 1) / kBS;
  pc.j0 = (int)((int64_t)pc.k * nb / pc.pieces);
  pc.j1 = (int)((int64_t)(pc.k + 1) * nb / pc.pieces);
  pc.base = p.Hkv * pu_records(w0) + pc.g * pc.pieces;
  return pc;
}

// Block ids of a piece: lane k holds the id of block j0 + k, clamped to the
// piece's last block.
__device__ __forceinline__ int piece_ids(const Params& p, const Piece& pc, int from, int lane) {
  const int last = pc.j1 - 1;
  const int j = from + lane < last ? from + lane : last;
  return p.block_tables[(int64_t)pc.b * p.max_blocks + j];
}

// A piece in flight: its ring of kRing blocks (their valid token counts, V
// offsets and, for the append, whether a slot holds the stream's last block),
// its block-id window, its queries and (append) this lane's chunks of the new
// token's K and V rows.
struct PieceRun {
  BlockRegs ring[kRing];
  int nvalid[kRing];
  int64_t ub[kRing];
  bool slast[kRing];
  uint32_t qv[4][4];
  int tab, tab_base;
  int last_phys;
  u32x4 knv, vnv;
};

// Load the piece's queries (and, for the piece that holds its stream's last
// block, the new token's chunks) and issue its first group of blocks; `tab`
// is its block-id window from block j0.
template <bool kAppend>
__device__ __forceinline__ void piece_begin(PieceRun& r, const Params& p, const Piece& pc,
                                            int tab, int lane) {
  const int grp = lane >> 3, i = lane & 7;
  const bool quad1 = (i & 4) != 0;
  const int c = quad1 ? ((i & 3) ^ 3) : (i & 3);
  const int lane_off = grp * kD + 8 * i;
  const int nb = (pc.ctx + kBS - 1) / kBS;
  load_q(r.qv, p, pc.b, pc.g, i, c);
  if (kAppend && pc.j1 == nb) load_new(r.knv, r.vnv, p, pc.b, pc.g, i);
  r.tab = tab;
  r.tab_base = pc.j0;
  r.last_phys = 0;
  const int last = pc.j1 - 1;
#pragma unroll
  for (int s = 0; s < kRing; ++s) {
    const int j = pc.j0 + s < last ? pc.j0 + s : last;
    const int id = __builtin_amdgcn_readlane(tab, j - pc.j0);
    int64_t ub;
    const int nv = issue_k(r.ring[s], p, id, pc.g, j, pc.ctx, lane_off, ub);
    issue_v(r.ring[s], p, ub, lane_off);
    r.nvalid[s] = pc.j0 + s < pc.j1 ? nv : 0;
    if (kAppend) {
      r.slast[s] = pc.j0 + s == nb - 1 && nv > 0;
      if (r.slast[s]) r.last_phys = id;
    }
  }
}

// Run the piece's blocks through its ring; with `app` the
// new token's rows replace the stale ones its last block returned and are
// stored to the pools.
template <bool kAppend>
__device__ __forceinline__ void piece_run(LaneState& st, PieceRun& r, const Params& p,
                                          const Piece& pc, bool app, int lane) {
  const int grp = lane >> 3, i = lane & 7;
  const bool quad1 = (i & 4) != 0;
  const int own_tok = quad1 ? grp + 8 : grp;
  const int lane_off = grp * kD + 8 * i;
  reset_state(st);
  const int32_t* trow = p.block_tables + (int64_t)pc.b * p.max_blocks;
  const int nb = (pc.ctx + kBS - 1) / kBS;
  const int n = pc.j1 - pc.j0;
  const int last = pc.j1 - 1;
  const int t_new = (pc.ctx - 1) & (kBS - 1);
  for (int base = 0; base < n; base += kRing) {
    if (kAppend && app) {
#pragma unroll
      for (int s = 0; s < kRing; ++s) {
        if (r.slast[s]) {
          if (grp == t_new) r.ring[s].ka = r.knv;
          if (grp + 8 == t_new) r.ring[s].kb = r.knv;
          if (grp == (t_new & 7)) {
            const int64_t off = (((int64_t)r.last_phys * p.Hkv + pc.g) * kBS + t_new) * kD + 8 * i;
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.k_cache) + off) = r.knv;
            *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(p.v_cache) + off) = r.vnv;
          }
        }
      }
    }
    bool full = true;
#pragma unroll
    for (int s = 0; s < kRing; ++s) full = full && r.nvalid[s] == kBS;
    float x[kRing];
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      x[s] = block_score(r.ring[s], r.qv, p.scale_log2, quad1);
      if (!full && own_tok >= r.nvalid[s]) x[s] = -INFINITY;
    }
    // the K halves of the slots are free: refill them with the blocks kRing
    // ahead (their V halves follow each slot's P.V)
    int nv_next[kRing];
    bool sl_next[kRing];
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
      const int jn = pc.j0 + base + s + kRing;
      const int j = jn < last ? jn : last;
      if (j - r.tab_base >= 64) {
        r.tab_base += 64;
        r.tab = trow[r.tab_base + lane < last ? r.tab_base + lane : last];
        // wait here (vmcnt 0), inside the branch, so the common path after it
        // carries no wait for this load
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      const int id = __builtin_amdgcn_readlane(r.tab, j - r.tab_base);
      const int nv = issue_k(r.ring[s], p, id, pc.g, j, pc.ctx, lane_off, r.ub[s]);
      nv_next[s] = jn < pc.j1 ? nv : 0;
      if (kAppend) {
        sl_next[s] = jn == nb - 1 && jn < pc.j1 && nv > 0;
        if (sl_next[s]) r.last_phys = id;
      }
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
      if (kAppend && app && r.slast[s]) {
        if (grp == t_new) r.ring[s].va = r.vnv;
        if (grp + 8 == t_new) r.ring[s].vb = r.vnv;
      }
      if (full)
        block_pv<false>(st, r.ring[s], pw, quad1, true, true);
      else
        block_pv<true>(st, r.ring[s], pw, quad1, grp < r.nvalid[s], grp + 8 < r.nvalid[s]);
      issue_v(r.ring[s], p, r.ub[s], lane_off);
      r.nvalid[s] = nv_next[s];
      if (kAppend) r.slast[s] = sl_next[s];
    }
  }
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
  Piece pc = {};
  pc.b = b;
  pc.g = g;
  pc.j0 = j0;
  pc.j1 = j1;
  pc.ctx = ctx;
  PieceRun r;
  piece_begin<false>(r, p, pc, piece_ids(p, pc, j0, lane), lane);
  LaneState st;
  piece_run<false>(st, r, p, pc, false, lane);
  const bool complete = (j0 == 0 && j1 == nb);
  const int pieces = (nb + p.part_blocks - 1) / (p.part_blocks > 0 ? p.part_blocks : 1);
  finish_segment(st, p, b, g, complete, unit, red[wave], lane);
  if (!complete) {
    drain_stores();
    if (count_piece(p, b, g, lane) + 1 == (uint32_t)pieces)
      merge_stream(p, b, g, stream * parts, pieces, red[wave], lane);
  }
}

// The plan of the split for this call's lengths and tables: what
// decode_auto_kernel computes before its first load (the piece bound, the
// prefix of pieces, the clamped lengths, and for each wavefront its first
// piece with the block ids of its first 64 blocks), stored once so that calls
// which share lengths and tables (every layer of a decode step) start loading
// keys at once.
__global__ void __launch_bounds__(kWaves * 64)
decode_plan_kernel(Params p) {
  __shared__ int pu[kAutoMaxBatch + 1];
  __shared__ int s_ctx[kAutoMaxBatch];
  __shared__ int wsum[kWaves];
  __shared__ long long wtot[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = piece_prefix<false>(p, pu, s_ctx, nullptr, wsum, wtot, tid, lane, wave);
  const int W = gridDim.x * kWaves;
  if (blockIdx.x == 0) {
    for (int k = tid; k <= p.B; k += kWaves * 64) {
      p.plan[kPlanHeaderInts + k] = pu[k];
      if (k < p.B) p.plan[kPlanCtxOffset + k] = s_ctx[k];
    }
    if (tid < kPlanHeaderInts) {
      const int hdr[8] = {kPlanMagic, p.B, p.Hkv, p.max_blocks, p.ctx_cap, p.num_blocks, W, P};
      p.plan[tid] = tid < 8 ? hdr[tid] : 0;
    }
  }
  const int w = blockIdx.x * kWaves + wave;
  int* ent = p.plan + kPlanWaveOffset + (int64_t)w * kPlanWaveInts;
  int f[8] = {-1, 0, 0, 0, 0, 1, 0, 0};
  int tab = 0;
  if ((int64_t)w < (int64_t)p.Hkv * pu_pieces(pu[p.B])) {
    const Piece pc = locate_piece(p, pu, s_ctx, w);
    f[0] = pc.b; f[1] = pc.g; f[2] = pc.j0; f[3] = pc.j1;
    f[4] = pc.ctx; f[5] = pc.pieces; f[6] = pc.base; f[7] = pc.k;
    if (pc.j1 > pc.j0) tab = piece_ids(p, pc, pc.j0, lane);
  }
  ent[8 + lane] = tab;
  if (lane < 8) {
    int v = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) v = lane == k ? f[k] : v;
    ent[lane] = v;
  }
}

//
// kAppend: the call also stores one new token per sequence (kv_append with
// one token each).  The new token is the last of its sequence, so it lies in
// the stream's last block, which exactly one piece reads: that wavefront
// writes the token's K and V rows into the pools and uses them from
// registers in place of the (stale) rows its load returned.  The rows of a
// sequence clamped to max_context_len are stored by a workgroup during
// set-up; slots outside the table or pool are not written (as kv_append).
template <bool kAppend, bool kPlanned>
__global__ void __launch_bounds__(kWaves * 64)
decode_auto_kernel(Params p) {
  __shared__ float red[kWaves][8 * 4 * kD];
  __shared__ int pu[kAutoMaxBatch + 1];
  __shared__ int s_ctx[kAutoMaxBatch];
  __shared__ int wsum[kWaves];
  __shared__ long long wtot[kWaves];
  __shared__ unsigned char s_newok[kAppend ? kAutoMaxBatch : 1];  // append this sequence
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gw = blockIdx.x * kWaves + wave;
  const int W = gridDim.x * kWaves;
  PieceRun r;

  // With a plan: this wavefront's first piece is issued at once, before the
  // plan is checked against this call (the block ids are range-checked, so
  // the loads stay inside the pools whatever the plan holds); the lengths
  // and the prefix come from the plan too.  A plan made for other lengths or
  // another shape is not used: the split is computed and the first piece
  // issued again.
  bool use_plan = false, issued = false;
  Piece first = {};
  // this thread's first sequence (k = tid): plan prefix, plan length and
  // length, loaded before the first group so that waiting for them does not
  // wait for its keys (vector loads complete in order)
  int v_pu = 0, v_pctx = 0, v_len = 0;
  if (kPlanned) {
    if (tid <= p.B) v_pu = p.plan[kPlanHeaderInts + tid];
    if (tid < p.B) {
      v_pctx = p.plan[kPlanCtxOffset + tid];
      v_len = p.context_lens[tid];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int* ent = p.plan + kPlanWaveOffset + (int64_t)gw * kPlanWaveInts;
    const int tab = ent[8 + lane];
    first.b = ld_uniform(ent, 0);
    first.g = ld_uniform(ent, 1);
    first.j0 = ld_uniform(ent, 2);
    first.j1 = ld_uniform(ent, 3);
    first.ctx = ld_uniform(ent, 4);
    first.pieces = ld_uniform(ent, 5);
    first.base = ld_uniform(ent, 6);
    first.k = ld_uniform(ent, 7);
    use_plan = ld_uniform(p.plan, 0) == kPlanMagic && ld_uniform(p.plan, 1) == p.B &&
               ld_uniform(p.plan, 2) == p.Hkv && ld_uniform(p.plan, 3) == p.max_blocks &&
               ld_uniform(p.plan, 4) == p.ctx_cap && ld_uniform(p.plan, 5) == p.num_blocks &&
               ld_uniform(p.plan, 6) == W;
    if (use_plan && first.b >= 0 && first.b < p.B && first.g >= 0 && first.g < p.Hkv &&
        first.ctx > 0 && first.ctx <= p.ctx_cap && first.j0 >= 0 && first.j0 < first.j1 &&
        first.j1 <= (first.ctx + kBS - 1) / kBS && first.pieces >= 1 && first.k >= 0 &&
        first.k < first.pieces) {
      piece_begin<kAppend>(r, p, first, tab, lane);
      issued = true;
    }
  }
  if (use_plan) {
    __builtin_amdgcn_sched_barrier(0);
    if (tid == 0) wsum[0] = 0;
    bool stale = false;
    for (int k = tid; k <= p.B; k += kWaves * 64) {
      const bool own = k == tid;
      pu[k] = own ? v_pu : p.plan[kPlanHeaderInts + k];
      if (k < p.B) {
        int cx = own ? v_len : p.context_lens[k];
        if (kAppend) s_newok[k] = cx >= 1 && cx <= p.ctx_cap;
        cx = cx < 0 ? 0 : (cx > p.ctx_cap ? p.ctx_cap : cx);  // as eff_ctx
        s_ctx[k] = cx;
        // the plan must have been made for exactly these lengths
        stale = stale || (own ? v_pctx : p.plan[kPlanCtxOffset + k]) != cx;
      }
    }
    __syncthreads();
    if (stale) wsum[0] = 1;
    __syncthreads();
    if (wsum[0] != 0) {
      use_plan = false;
      issued = false;
      __syncthreads();  // everyone has read the flag before wsum is reused
    }
  }
  if (!use_plan) piece_prefix<kAppend>(p, pu, s_ctx, s_newok, wsum, wtot, tid, lane, wave);

  // a sequence cut short by the clamp still gets its token stored (no
  // wavefront reads that row): workgroup k % grid copies it
  if (kAppend) {
    for (int k = blockIdx.x; k < p.B; k += gridDim.x) {
      if (s_newok[k]) continue;
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

  // this wavefront's piece (already in flight with a plan)
  if ((int64_t)gw >= (int64_t)p.Hkv * pu_pieces(__builtin_amdgcn_readfirstlane(pu[p.B]))) return;
  Piece pc = first;
  if (!issued) {
    pc = locate_piece(p, pu, s_ctx, gw);
    if (pc.j1 > pc.j0) piece_begin<kAppend>(r, p, pc, piece_ids(p, pc, pc.j0, lane), lane);
  }
  const int nb = (pc.ctx + kBS - 1) / kBS;
  if (nb == 0) {
    write_zero_rows(p, pc.b, pc.g, lane);
    return;
  }
  const bool app = kAppend && pc.j1 == nb && s_newok[pc.b];
  LaneState st;
  piece_run<kAppend>(st, r, p, pc, app, lane);
  const bool complete = pc.pieces == 1;
  finish_segment(st, p, pc.b, pc.g, complete, pc.base + pc.k, red[wave], lane);
  if (!complete) {
    drain_stores();
    if (count_piece(p, pc.b, pc.g, lane) + 1 == (uint32_t)pc.pieces)
      merge_stream(p, pc.b, pc.g, pc.base, pc.pieces, red[wave], lane);
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
    const dim3 grid((unsigned)(auto_waves((int64_t)a.B * a.Hkv) / kWaves)), block(kWaves * 64);
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
