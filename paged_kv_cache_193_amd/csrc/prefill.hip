// prefill.hip -- causal paged prefill: every prompt token attends to the
// cached tokens up to and including its own position, reading K/V through the
// block table (tiny-vllm README, table of contents "Prefill vs decode",
// "Attention", "GQA", "Causal mask", "Online softmax", "Paged Attention";
// nano-vLLM guide announcement ch. 6: prefill is compute bound).  Here the
// path is a dense contraction, so Q.K^T and P.V run on CDNA4 bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Work unit: one workgroup per (32-row query tile, sequence b, KV group g);
// its 4 wavefronts are the 4 query heads of the group, so every K/V tile
// staged in LDS serves all of them (GQA).  Each wavefront holds, in registers,
//   S^T[64 keys][32 q]   = K . Q^T       (2 MFMA tiles of 32x32)
//   O^T[64 d][32 q]     += V^T . P^T     (2 MFMA tiles of 32x32)
// 32-row query tiles halve the longest unit of work (the last rows of a long
// prompt see every key tile) and leave room for three workgroups per CU
// (142 VGPRs, 36 KB of LDS).  A sequence of at most 4 query rows (a decoding
// sequence of a mixed batch) takes its own path, short_rows below: its
// workgroup's 4 wavefronts split the context instead of walking all of it
// with a 32-row tile that holds one row.
// The MFMA accumulator layout puts one query column and 16 keys in a lane
// (rows 8*(r/4) + 4*(lane/32) + r%4, column lane%32), which is exactly the
// layout P^T needs as the B operand of the next product: the softmax runs on
// the scores where they are and no lane exchange is needed for P.  The row
// statistics (max, sum) are per query column: in-lane over 32 keys plus one
// exchange with lane^32.
//
// LDS per workgroup, double buffered: K and V tiles [64 keys][64 d], both
// row major with rows padded to spread LDS banks (36 KB); each wavefront
// keeps its Q^T operand (32 rows, 16 VGPRs) in registers.  The V^T operand
// of P.V needs consecutive keys of one head_dim column in a lane; CDNA4's
// transposing LDS read (ds_read_b64_tr_b16) delivers them straight from the
// row-major tile, so V is not transposed at staging.  Rows of keys past the
// context (only the tile that reaches past it has any) are zero filled, so
// 0 * NaN cannot reach the MFMA; an invalid block id reads block 0 instead.
//
// Softmax (fp32, log2 units): weights are exp2(c * s - m) against a reference
// maximum m per query column.  m is not recomputed every tile: only when a
// lane's sum of one tile's weights exceeds kLazyBound (a score rose well
// above m) or the column has no reference yet is the tile's maximum taken,
// the accumulator and row sum rescaled and the weights formed again.  By the
// softmax shift identity the result does not depend on the reference used.
// Row sums add the same bf16-rounded weights that P.V uses.
//
// Causal rule: query row t of a prompt of q_len tokens whose sequence holds
// context_len tokens sits at position context_len - q_len + t and sees keys
// 0..pos.  Key tiles entirely below the first row's position need no mask;
// only diagonal tiles are masked.  Query tiles are launched heaviest first
// as far as the grid index can tell (a prompt's last tile first; tile 0
// first where cached history makes it the heavy one), and the KV group is
// the fastest-varying grid index (one KV head per XCD's L2 for the 8-head
// case).
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;
constexpr int kBS = 16;
constexpr int kTile = 64;          // keys per K/V tile
constexpr int kQRows = 32;         // query rows per workgroup
constexpr int kKRow = kD + 8;      // K and V tile row stride (bf16 elements): 144 bytes
// A lane's partial row sum of one tile's weights above this (or not a number)
// sends the tile through the exact-max path.  Weights stay below 2^10.
constexpr float kLazyBound = 1024.f;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // bf16 pair (1, 1)
constexpr int kRsrcWord3 = 0x00020000;         // raw buffer, dword data

struct PParams {
  void* out;
  int out_f32;
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  int B, Hq, Hkv, max_blocks, num_blocks, tiles_max;
  int max_rows;     // rows of a sequence that are written: min(max_q_len, T_q)
  int chunks;       // compact grid: ceil(B / 64) sequences per lane; 0: rank grid
  float c_log2;     // |scale| * log2(e), floored at 1e-30: scores to log2 units
  uint32_t q_sign;  // 0x80008000 when scale < 0 (q is negated), else 0
};

constexpr f32x16 kZero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                             0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

__device__ __forceinline__ f32x16 mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Registers of one thread's share of a K/V tile: keys 2*kp and 2*kp+1 of the
// tile, head_dim chunk [8c, 8c+8) (thread t: kp = t / 8, c = t % 8).
struct TileRegs {
  u32x4 k0, k1, v0, v1;
};

// Physical id of the block that wavefront `wave` loads for the tile that
// starts at key k0: the tile's 64 keys are 4 blocks of 16, one per wavefront,
// so the id is wave-uniform and comes from one scalar load (the logical block
// index is clamped to the table row, so the read is always in bounds; keys
// past the context are zeroed by load_tile).
__device__ __forceinline__ int tile_block_id(const PParams& p, const int32_t* trow, int k0,
                                             int wave) {
  int jb = k0 / kBS + wave;
  jb = jb < p.max_blocks ? jb : p.max_blocks - 1;
  return trow[__builtin_amdgcn_readfirstlane(jb)];
}

// Load this thread's share of the tile at key k0 from block `phys`.  The
// loads are unconditional (an invalid id reads block 0), so the number of
// loads in flight is the same on every path; rows of keys past the context
// or of an invalid block are replaced by zeros afterwards.
__device__ __forceinline__ void load_tile(TileRegs& r, const PParams& p, int phys, int g,
                                          int ctx, int k0, int tid, uint32_t toff) {
  const int kp = tid >> 3;
  const int key0 = k0 + 2 * kp;  // key0 and key0 + 1 share one 16-token block
  phys = __builtin_amdgcn_readfirstlane(phys);
  const bool ok = phys >= 0 && phys < p.num_blocks;
  // one (block, head) chunk of each pool through a buffer descriptor built
  // in scalar registers: the lane's part of the address is one 32-bit offset
  const int64_t blk = ((int64_t)(ok ? phys : 0) * p.Hkv + g) * (kBS * kD);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.k_cache + blk), (short)0, kBS * kD * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.v_cache + blk), (short)0, kBS * kD * 2, kRsrcWord3);
  r.k0 = __builtin_amdgcn_raw_buffer_load_b128(rk, toff * 2, 0, 0);
  r.v0 = __builtin_amdgcn_raw_buffer_load_b128(rv, toff * 2, 0, 0);
  r.k1 = __builtin_amdgcn_raw_buffer_load_b128(rk, toff * 2 + kD * 2, 0, 0);
  r.v1 = __builtin_amdgcn_raw_buffer_load_b128(rv, toff * 2 + kD * 2, 0, 0);
  // Only a tile that reaches past the context holds rows to zero (a wave-
  // uniform test); inside the context the table's ids are valid by contract
  // (an invalid one reads block 0, in bounds, and gives an undefined result).
  if (k0 + kTile > ctx) {
    const u32x4 zero = {0, 0, 0, 0};
    if (!(ok && key0 < ctx)) r.k0 = r.v0 = zero;
    if (!(ok && key0 + 1 < ctx)) r.k1 = r.v1 = zero;
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* ks, uint16_t* vs,
                                           int tid) {
  const int kp = tid >> 3, c = tid & 7;
  *reinterpret_cast<u32x4*>(ks + (2 * kp) * kKRow + 8 * c) = r.k0;
  *reinterpret_cast<u32x4*>(ks + (2 * kp + 1) * kKRow + 8 * c) = r.k1;
  // V row major like K; the P.V operand reads it transposed (ds_read_b64_tr_b16)
  *reinterpret_cast<u32x4*>(vs + (2 * kp) * kKRow + 8 * c) = r.v0;
  *reinterpret_cast<u32x4*>(vs + (2 * kp + 1) * kKRow + 8 * c) = r.v1;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Four consecutive keys at one head_dim column, transposed out of the
// row-major V tile: in each group of 16 lanes, lane 4k+p addresses row
// key0+k at columns d0+4p..d0+4p+3, and lane i receives rows key0..key0+3
// of column d0+i.
__device__ __forceinline__ u32x2 v_keys4(const uint16_t* vs, int key0, int d0, int lane) {
  const int j = lane & 15;
  const uint16_t* a = vs + (key0 + (j >> 2)) * kKRow + d0 + 4 * (j & 3);
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(a));
  return __builtin_bit_cast(u32x2, x);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Short rows: a sequence with at most kShortRows query rows (a decoding
// sequence of a mixed batch, or a few draft tokens) has one live workgroup
// and little to contract, but its context can be long.  Its 4 wavefronts
// split the context's blocks into 4 contiguous ranges, and each wavefront
// covers all 4 heads of the group for every row at once: the 16 columns of
// a 16x16x32 MFMA are (row t, head) = (c / 4, c % 4).  Per wavefront and
// 64-key group (4 blocks):
//   S^T[16 keys][16 cols] = K . Q^T        4 blocks x 2 head_dim halves
//   O^T[16 d][16 cols]   += V^T . P^T      4 head_dim quarters x 2 key halves
// The K operand (key l % 16, head_dim chunk l / 16 of one half) is one
// 16-byte load per lane straight from the block; V goes through the
// wavefront's own quarter of the LDS (row major) and is read transposed.
// The 16x16 accumulator gives lane l keys 4 * (l / 16) + i (i < 4) of
// column l % 16; the P^T operand of a 32-key half takes them from its two
// blocks, and the V^T operand reads the same keys (4 from each block).  The
// softmax takes the exact maximum of every group.  The four wavefronts'
// (max, sum, O^T) are combined by the log-sum-exp rule through LDS.
constexpr int kShortRows = 4;

__device__ __forceinline__ void short_rows(const PParams& p, uint16_t* lds, int b, int g,
                                           int qs, int q_len, int ctx, int tid) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;   // column: row n / 4, head 4 * g + n % 4
  const int j = lane >> 4;   // k group of the MFMA operands
  const int t = n >> 2;
  const int hist = ctx - q_len;
  const int32_t* trow = p.block_tables + (int64_t)b * p.max_blocks;
  const float c2 = p.c_log2;

  // Q^T operand: column n, head_dim [32 s + 8 j, +8) for s = 0, 1 (zero for
  // columns past the rows; their results are not written)
  u32x4 qv[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (t < q_len) {
    const uint16_t* qr = p.q + ((int64_t)(qs + t) * p.Hq + 4 * g + (n & 3)) * kD + 8 * j;
    const u32x4 sg = {p.q_sign, p.q_sign, p.q_sign, p.q_sign};
    qv[0] = *reinterpret_cast<const u32x4*>(qr) ^ sg;
    qv[1] = *reinterpret_cast<const u32x4*>(qr + 32) ^ sg;
  }
  // keys this column sees: 0 .. min(position, ctx - 1)
  const int lim_col = hist + t < ctx - 1 ? hist + t : ctx - 1;

  // this wavefront's blocks [bw0, bw1) and keys [16 * bw0, wend)
  const int nblk = ctx > 0 ? (ctx + kBS - 1) / kBS : 0;
  const int bw0 = wave * nblk / 4, bw1 = (wave + 1) * nblk / 4;
  const int wend = 16 * bw1 < ctx ? 16 * bw1 : ctx;
  const int n_groups = (bw1 - bw0 + 3) / 4;
  uint16_t* vs = lds + wave * (kTile * kKRow);

  float m_ref = -INFINITY;  // column maximum so far (log2 units)
  float l_run = 0.f;        // this lane's share of the column sum
  f32x4 o[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                {0.f, 0.f, 0.f, 0.f}};  // O^T rows 16 dt + 4 j + i, column n

  if (n_groups > 0) {
    // lane offsets (bytes) inside a (block, head) chunk of 16 x 64 bf16
    const uint32_t koff = (uint32_t)((lane & 15) * 128 + 16 * j);  // + 64 s
    const uint32_t voff = (uint32_t)(16 * lane);                     // + 1024
    // block ids of a group; blocks past the range repeat the range's last
    // block (the loads stay unconditional and hit the cache)
    auto ids = [&](int jb0, int* id) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jb = jb0 + jj < bw1 ? jb0 + jj : bw1 - 1;
        id[jj] = trow[__builtin_amdgcn_readfirstlane(jb)];
      }
    };
    auto rsrc = [&](const uint16_t* pool, int phys) {
      phys = __builtin_amdgcn_readfirstlane(phys);
      phys = phys >= 0 && phys < p.num_blocks ? phys : 0;
      return __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(pool + ((int64_t)phys * p.Hkv + g) * (kBS * kD)), (short)0,
          kBS * kD * 2, kRsrcWord3);
    };
    u32x4 kr[4][2], vr[4][2];
    auto load_k = [&](const int* id) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const __amdgpu_buffer_rsrc_t r = rsrc(p.k_cache, id[jj]);
        kr[jj][0] = __builtin_amdgcn_raw_buffer_load_b128(r, koff, 0, 0);
        kr[jj][1] = __builtin_amdgcn_raw_buffer_load_b128(r, koff + 64, 0, 0);
      }
    };
    auto load_v = [&](const int* id) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const __amdgpu_buffer_rsrc_t r = rsrc(p.v_cache, id[jj]);
        vr[jj][0] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
        vr[jj][1] = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 1024, 0, 0);
      }
    };
    int id[4];
    ids(bw0, id);
    load_k(id);
    load_v(id);
    ids(bw0 + 4, id);

    for (int gi = 0; gi < n_groups; ++gi) {
      const int k0 = 16 * (bw0 + 4 * gi);
      // V of this group into the wavefront's LDS quarter; rows of keys past
      // the range are zeroed (0 * NaN must not reach the MFMA)
      if (k0 + kTile > wend) {
        const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (k0 + 16 * jj + (lane >> 3) >= wend) vr[jj][0] = zero;
          if (k0 + 16 * jj + 8 + (lane >> 3) >= wend) vr[jj][1] = zero;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        *reinterpret_cast<u32x4*>(vs + (16 * jj + (lane >> 3)) * kKRow + 8 * (lane & 7)) =
            vr[jj][0];
        *reinterpret_cast<u32x4*>(vs + (16 * jj + 8 + (lane >> 3)) * kKRow + 8 * (lane & 7)) =
            vr[jj][1];
      }
      load_v(id);

      // S^T = K . Q^T, one 16-key block per accumulator
      f32x4 s[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        s[jj] = mfma16(as_bf16x8(kr[jj][0]), as_bf16x8(qv[0]), f32x4{0.f, 0.f, 0.f, 0.f});
        s[jj] = mfma16(as_bf16x8(kr[jj][1]), as_bf16x8(qv[1]), s[jj]);
      }
      load_k(id);
      ids(bw0 + 4 * gi + 8, id);

      // mask keys past the column's position or the range
      const int lim_row0 = (hist < ctx - 1 ? hist : ctx - 1);
      if (k0 + kTile - 1 > (lim_row0 < wend - 1 ? lim_row0 : wend - 1)) {
        const int lim = (lim_col < wend - 1 ? lim_col : wend - 1) - (k0 + 4 * j);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * jj + i > lim) s[jj][i] = -INFINITY;
      }

      // exact column maximum of the group, rescale, weights
      float v = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
#pragma unroll
      for (int jj = 1; jj < 4; ++jj)
        v = fmaxf(v, fmaxf(fmaxf(s[jj][0], s[jj][1]), fmaxf(s[jj][2], s[jj][3])));
      v = fmaxf(v, shfl_xor(v, 16));
      v = fmaxf(v, shfl_xor(v, 32));
      const float m_new = fmaxf(m_ref, v * c2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_use);  // 0 while no reference
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      m_ref = m_new;
      bf16x8_t pop[2];
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4& sv = s[2 * ps + (e >> 1)];
          const int i = 2 * (e & 1);
          w[e] = pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, -m_use)),
                           __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i + 1], c2, -m_use)));
          l_run = dot2_bf16(w[e], kOnesBf16x2, l_run);
        }
        pop[ps] = as_bf16x8(w);
      }

      // O^T += V^T . P^T: keys 32 ps + 4 j + (0..3) and 32 ps + 16 + 4 j + (0..3)
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x2 lo = v_keys4(vs, 32 * ps + 4 * j, 16 * dt, lane);
          const u32x2 hi = v_keys4(vs, 32 * ps + 16 + 4 * j, 16 * dt, lane);
          o[dt] = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pop[ps], o[dt]);
        }
    }
  }

  // combine the four wavefronts: each writes (max, sum, O^T) of its 16
  // columns to its LDS quarter, then every thread finishes 4 outputs
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  float* part = reinterpret_cast<float*>(vs);  // [16] max, [16] sum, [16][64] O
  if (j == 0) {
    part[n] = m_ref;
    part[16 + n] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    *reinterpret_cast<f32x4*>(part + 32 + n * kD + 16 * dt + 4 * j) = o[dt];
  __syncthreads();

  const int col = tid >> 4, d = 4 * (tid & 15);
  const int row = col >> 2;
  const int wr_len = q_len < p.max_rows ? q_len : p.max_rows;
  if (row >= wr_len) return;
  float mw[4], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = reinterpret_cast<const float*>(lds + w * (kTile * kKRow))[col];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* pw = reinterpret_cast<const float*>(lds + w * (kTile * kKRow));
      const float f = __builtin_amdgcn_exp2f(mw[w] - M);  // 0 for a part with no keys
      L += f * pw[16 + col];
      acc += f * *reinterpret_cast<const f32x4*>(pw + 32 + col * kD + d);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int64_t base = ((int64_t)(qs + row) * p.Hq + 4 * g + (col & 3)) * kD + d;
  if (p.out_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + base) =
        make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  } else {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + base) =
        u32x2{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  }
}

// Wave-uniform sum of an int over the 64 lanes (DPP within rows of 16, then
// the four rows' totals).
__device__ __forceinline__ int wave_sum_i(int x) {
  x += __builtin_amdgcn_mov_dpp(x, kQuadXor1, 0xf, 0xf, true);
  x += __builtin_amdgcn_mov_dpp(x, kQuadXor2, 0xf, 0xf, true);
  x += __builtin_amdgcn_mov_dpp(x, kRowHalfMirror, 0xf, 0xf, true);
  x += __builtin_amdgcn_mov_dpp(x, kRowMirror, 0xf, 0xf, true);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// Compact grid (at most kCompactChunks * 64 sequences).  The rank grid gives
// every sequence tiles_max ranks, and a sequence with fewer query tiles
// leaves workgroups that only read its lengths and exit; in a mixed batch of
// decode rows and prompt chunks most of the grid is such workgroups, and
// while long-lived workgroups hold most of the CU slots they pass through
// the rest one round trip at a time.  The compact grid enumerates only the
// live (rank, sequence) pairs, in the rank grid's order (rank, then
// sequence).  Sequence b with n query tiles is live at
//   ranks [tiles_max - n, tiles_max)                  without cached history
//                                                     or with at most
//                                                     kShortRows rows,
//   rank 0 and ranks [tiles_max - n + 1, tiles_max)   otherwise (tile 0 first).
// Workgroup e finds its rank r as the largest r with C(r) <= e, where C(r)
// counts the live pairs of all ranks below r (a binary search over r; each
// C is one wave sum), and its sequence as the (e - C(r))-th one live at r.
// Every wavefront computes the same result (no LDS, no barrier).  Returns
// false for the few workgroups past the live pairs (the grid is sized from
// an upper bound of the tile count).
constexpr int kCompactChunks = 4;

__device__ __forceinline__ bool compact_unit(const PParams& p, int e, int lane, int& b,
                                             int& rank, int& qs, int& q_len, int& ctx) {
  const int cap = p.max_blocks * kBS;
  int s[kCompactChunks], m[kCompactChunks], f[kCompactChunks];
  int c_qs[kCompactChunks], c_q[kCompactChunks], c_ctx[kCompactChunks];
#pragma unroll
  for (int c = 0; c < kCompactChunks; ++c) {
    const int bb = 64 * c + lane;
    s[c] = p.tiles_max;  // first rank of the aligned part; m its length
    m[c] = 0;
    f[c] = 0;            // 1: tile 0 runs at rank 0 (cached history)
    c_qs[c] = c_q[c] = c_ctx[c] = 0;
    if (c < p.chunks && bb < p.B) {  // c < chunks: a uniform branch
      const int a0 = p.cu_q_lens[bb];
      const int q = p.cu_q_lens[bb + 1] - a0;
      int cx = p.context_lens[bb];
      cx = cx > cap ? cap : cx;
      const int rows = q < p.max_rows ? q : p.max_rows;
      const int n = rows > 0 ? (rows + kQRows - 1) / kQRows : 0;
      c_qs[c] = a0;
      c_q[c] = q;
      c_ctx[c] = cx;
      if (n > 0) {
        f[c] = cx - q > 0 && q > kShortRows;
        s[c] = p.tiles_max - n + f[c];
        m[c] = n - f[c];
      }
    }
  }
  auto below = [&](int r) {  // live pairs at ranks < r
    int x = 0;
#pragma unroll
    for (int c = 0; c < kCompactChunks; ++c) {
      if (c < p.chunks) {
        const int a = r - s[c];
        x += (f[c] & (r > 0 ? 1 : 0)) + (a < 0 ? 0 : a < m[c] ? a : m[c]);
      }
    }
    return wave_sum_i(x);
  };
  if (e >= below(p.tiles_max)) return false;
  int lo = 0, hi = p.tiles_max;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (below(mid) <= e) lo = mid;
    else hi = mid;
  }
  int j = e - below(lo);
#pragma unroll
  for (int c = 0; c < kCompactChunks; ++c) {
    if (c >= p.chunks) break;
    const bool live = (lo == 0 && f[c]) || (m[c] > 0 && s[c] <= lo);
    const uint64_t mask = __builtin_amdgcn_ballot_w64(live);
    const int pc = __builtin_popcountll(mask);
    if (j < pc) {
      const int below_lane = __builtin_amdgcn_mbcnt_hi(
          (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
      const uint64_t pick = __builtin_amdgcn_ballot_w64(live && below_lane == j);
      const int ln = __builtin_ctzll(pick);
      b = 64 * c + ln;
      rank = lo;
      qs = __builtin_amdgcn_readlane(c_qs[c], ln);
      q_len = __builtin_amdgcn_readlane(c_q[c], ln);
      ctx = __builtin_amdgcn_readlane(c_ctx[c], ln);
      return true;
    }
    j -= pc;
  }
  return false;
}

__global__ void __launch_bounds__(256, 3)
prefill_kernel(PParams p) {
  // four 64-key tiles: K and V double buffered (short rows: one V tile per
  // wavefront)
  __shared__ __attribute__((aligned(16))) uint16_t lds[4][kTile * kKRow];
  uint16_t (*ks_buf)[kTile * kKRow] = lds;
  uint16_t (*vs_buf)[kTile * kKRow] = lds + 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // grid: g fastest, then b, then a rank per query tile.  A prompt without
  // cached history takes its tiles from the last (heaviest) down.  With
  // history, tile 0 already sees the whole history and can be the heaviest
  // unit of the launch (a decode row of a mixed batch is only tile 0), so
  // it takes the first rank and the other tiles follow from the last down.
  // A sequence of at most kShortRows rows (one short-row workgroup) takes
  // the last rank: its workgroup streams the context and is long-lived, so
  // it starts after the prompts' tiles, and its dead ranks pass through
  // while the CUs still have free slots.  The compact grid keeps this order
  // and leaves out the (rank, sequence) pairs that hold no tile.
  const int g = blockIdx.x % p.Hkv;
  const int rest = blockIdx.x / p.Hkv;
  const int cap = p.max_blocks * kBS;
  int b, rank, qs, q_len, ctx;
  if (p.chunks > 0) {
    if (!compact_unit(p, rest, lane, b, rank, qs, q_len, ctx)) return;
  } else {
    b = rest % p.B;
    rank = rest / p.B;
    qs = p.cu_q_lens[b];
    q_len = p.cu_q_lens[b + 1] - qs;
    ctx = p.context_lens[b];
    ctx = ctx > cap ? cap : ctx;
  }
  const int hist = ctx - q_len;  // position of query row 0 minus 0
  const int tile = hist <= 0 || q_len <= kShortRows ? p.tiles_max - 1 - rank
                   : rank == 0 ? 0 : p.tiles_max - rank;
  const int q0 = tile * kQRows;
  if (q0 >= q_len) return;
  if (q_len <= kShortRows) {
    short_rows(p, &lds[0][0], b, g, qs, q_len, ctx, tid);
    return;
  }
  const int rows = q_len - q0 < kQRows ? q_len - q0 : kQRows;
  const int pos_first = hist + q0;
  const int pos_last = hist + q0 + rows - 1;
  int kend = pos_last + 1 < ctx ? pos_last + 1 : ctx;  // keys [0, kend)
  if (kend < 0) kend = 0;
  const int n_tiles = (kend + kTile - 1) / kTile;
  const int h = 4 * g + wave;
  const int32_t* trow = p.block_tables + (int64_t)b * p.max_blocks;

  // Q^T operand, in registers: lane holds q row q0 + lane%32, d in
  // [k*16 + 8*(lane/32), +8)
  const int lr = lane & 31, lh = lane >> 5;
  u32x4 qsw[4];  // this wavefront's Q^T operand [k], in registers
  {
    int row = q0 + lr;
    row = row < q_len ? row : q_len - 1;
    const uint16_t* qr = p.q + ((int64_t)(qs + row) * p.Hq + h) * kD + 8 * lh;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      qsw[k] = *reinterpret_cast<const u32x4*>(qr + 16 * k) ^
                           u32x4{p.q_sign, p.q_sign, p.q_sign, p.q_sign};
  }

  f32x16 o[2] = {kZero16, kZero16};  // [dt]
  // Reference max m of this lane's query column (log2 units): weights are
  // exp2(c * s - m).  has_ref is false until the column has seen a visible key.
  float m_ref = 0.f;
  bool has_ref = false;
  const float c2 = p.c_log2;
  float l_run = 0.f;  // this lane's share of the row sum

  // K/V tiles go global -> registers -> LDS one tile ahead of the MFMAs, and
  // the block id of the tile after that is read one more tile ahead, so no
  // load waits on a table read.
  TileRegs nxt;
  // this thread's element offset inside a (block, head) chunk: rows
  // 2 * kp % 16 and the next, head_dim chunk c
  const uint32_t toff = (uint32_t)((2 * (tid >> 3)) % kBS * kD + 8 * (tid & 7));
  int id_next = tile_block_id(p, trow, kTile, wave);
  load_tile(nxt, p, tile_block_id(p, trow, 0, wave), g, ctx, 0, tid, toff);
  store_tile(nxt, ks_buf[0], vs_buf[0], tid);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int k0 = it * kTile;
    const int buf = it & 1;
    // past the last tile these read clamped, unused data (no branch, so the
    // load counts stay static)
    load_tile(nxt, p, id_next, g, ctx, k0 + kTile, tid, toff);
    id_next = tile_block_id(p, trow, k0 + 2 * kTile, wave);
    const uint16_t* ks = ks_buf[buf];
    const uint16_t* vs = vs_buf[buf];

    // S^T = K . Q^T (scores before scaling), keys kt*32 .. kt*32+31
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x8_t a = as_bf16x8(
            *reinterpret_cast<const u32x4*>(ks + (kt * 32 + lr) * kKRow + 16 * k + 8 * lh));
        s[kt] = mfma(a, as_bf16x8(qsw[k]), k == 0 ? kZero16 : s[kt]);
      }
    }

    // causal mask on tiles that reach past the first row's position: key j of
    // this lane's column is visible iff j <= min(pos, ctx - 1)
    if (k0 + kTile - 1 > pos_first) {
      const int pos = pos_first + lr;
      const int lim = (pos < ctx - 1 ? pos : ctx - 1) - (k0 + 4 * lh);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kt][r] = -INFINITY;
    }

    // Weights against the reference: P^T operand as bf16, and this lane's
    // partial row sum of the same rounded weights (v_dot2 against (1, 1)).
    bf16x8_t pop[4];
    float lsum = 0.f;
    auto weights = [&](float m) {
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * half + 2 * e;
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], c2, -m));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r + 1], c2, -m));
            w[e] = pack_bf16(p0, p1);
            if (e & 1)
              l1 = dot2_bf16(w[e], kOnesBf16x2, l1);
            else
              l0 = dot2_bf16(w[e], kOnesBf16x2, l0);
          }
          pop[2 * kt + half] = as_bf16x8(w);
        }
      lsum = l0 + l1;
    };
    // The first tile goes straight to the exact path (no column has a
    // reference yet; every column sees key 0, so each gets one there).
    const bool first = it == 0;
    if (!first) weights(m_ref);

    // Exact-max path, wave-uniform and rare after the first tile: a weight
    // may exceed the bound (a score rose well above the reference), or a
    // column has no reference yet.  The reference moves up to the tile max,
    // the accumulator and row sum are rescaled, and the weights are formed
    // again.  By the softmax shift identity the result does not depend on the
    // reference used.
    const bool redo = first || !(lsum <= kLazyBound) || !has_ref;
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
      float v = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) v = fmaxf(v, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, s[1][r]);
      const float mx = fmaxf(v, shfl_xor(v, 32)) * c2;  // tile max, log2 units
      // no visible key yet: stay without a reference (weights are 0)
      if (mx != -INFINITY && mx == mx) {
        const float m_new = has_ref ? fmaxf(m_ref, mx) : mx;
        const float alpha = has_ref ? __builtin_amdgcn_exp2f(m_ref - m_new) : 0.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        m_ref = m_new;
        has_ref = true;
      }
      weights(m_ref);
    }
    l_run += lsum;

    // O^T += V^T . P^T
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st * 16;  // key offset of this 16-key step within the tile
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        // column dt*32 + lr: the group of 16 lanes starts at dt*32 + 16*(lane/16 % 2)
        const int d0 = dt * 32 + (lr & 16);
        const u32x2 lo = v_keys4(vs, kb + 4 * lh, d0, lane);
        const u32x2 hi = v_keys4(vs, kb + 8 + 4 * lh, d0, lane);
        const bf16x8_t a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[dt] = mfma(a, pop[st], o[dt]);
      }
    }

    store_tile(nxt, ks_buf[buf ^ 1], vs_buf[buf ^ 1], tid);
    __syncthreads();
  }

  // epilogue: out[row][h][d] = O^T[d][row] / l(row)
  const float lt = l_run + shfl_xor(l_run, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const int row = q0 + lr;
  if (row >= (q_len < p.max_rows ? q_len : p.max_rows)) return;
  const int64_t base = ((int64_t)(qs + row) * p.Hq + h) * kD;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = dt * 32 + 8 * gq + 4 * lh;
      const float x0 = o[dt][4 * gq + 0] * inv, x1 = o[dt][4 * gq + 1] * inv;
      const float x2 = o[dt][4 * gq + 2] * inv, x3 = o[dt][4 * gq + 3] * inv;
      if (p.out_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + base + d) =
            make_float4(x0, x1, x2, x3);
      } else {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + base + d) =
            u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
      }
    }
}

}  // namespace

namespace {
// Units of the launch: (rank, sequence) pairs of the rank grid, or, for the
// compact grid, an upper bound of the query tiles: a sequence of q >= 1 rows
// has ceil(q / 32) <= 1 + (q - 1) / 32 tiles, so all of them together at most
// B + T_q / 32.  The compact grid pays its search in every workgroup; it is
// used (for at most 256 sequences) where at least two of every three units
// of the rank grid would be dead, i.e. where the bound is at most a third of
// the rank grid.  chunks is 0 for the rank grid.
constexpr int64_t kCompactRatio = 3;

int64_t prefill_units(int32_t max_q_len, int32_t T_q, int32_t B, int* chunks) {
  // no prompt is longer than all the query tokens together
  const int64_t rows = max_q_len < T_q ? max_q_len : T_q;
  const int64_t ranked = (rows + kQRows - 1) / kQRows * B;
  const int64_t bound = (int64_t)B + T_q / kQRows;
  const bool compact = B <= 64 * kCompactChunks && bound * kCompactRatio <= ranked;
  if (chunks) *chunks = compact ? (B + 63) / 64 : 0;
  return compact ? bound : ranked;
}
}  // namespace

int64_t prefill_grid_size(int32_t max_q_len, int32_t T_q, int32_t B, int32_t Hkv) {
  return prefill_units(max_q_len, T_q, B, nullptr) * Hkv;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  PParams p;
  p.out = a.out;
  p.out_f32 = a.out_f32;
  p.q = (const uint16_t*)a.q;
  p.k_cache = (const uint16_t*)a.k_cache;
  p.v_cache = (const uint16_t*)a.v_cache;
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.cu_q_lens = a.cu_q_lens;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  const int32_t rows = a.max_q_len < a.T_q ? a.max_q_len : a.T_q;
  p.tiles_max = (rows + kQRows - 1) / kQRows;
  p.max_rows = rows;
  // |scale| in log2 units, floored so that a zero scale still maps masked
  // (-inf) scores to -inf instead of NaN; any real score times 1e-30 is 0.
  p.c_log2 = (a.scale < 0.f ? -a.scale : a.scale) * kLog2e;
  if (p.c_log2 < 1e-30f) p.c_log2 = 1e-30f;
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const int64_t grid = prefill_units(a.max_q_len, a.T_q, a.B, &p.chunks) * a.Hkv;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
