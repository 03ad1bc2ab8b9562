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
// (133 VGPRs, 36 KB of LDS); a one-token row of a mixed batch wastes 31 rows
// of a tile instead of 63.
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

__global__ void __launch_bounds__(256, 3)
prefill_kernel(PParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_buf[2][kTile * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vs_buf[2][kTile * kKRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // grid: g fastest, then b, then a rank per query tile.  A prompt without
  // cached history takes its tiles from the last (heaviest) down.  With
  // history, tile 0 already sees the whole history and can be the heaviest
  // unit of the launch (a decode row of a mixed batch is only tile 0), so
  // it takes the first rank and the other tiles follow from the last down.
  const int g = blockIdx.x % p.Hkv;
  const int rest = blockIdx.x / p.Hkv;
  const int b = rest % p.B;
  const int rank = rest / p.B;

  const int qs = p.cu_q_lens[b];
  const int q_len = p.cu_q_lens[b + 1] - qs;
  int ctx = p.context_lens[b];
  const int cap = p.max_blocks * kBS;
  ctx = ctx > cap ? cap : ctx;
  const int hist = ctx - q_len;  // position of query row 0 minus 0
  const int tile = hist <= 0 ? p.tiles_max - 1 - rank : rank == 0 ? 0 : p.tiles_max - rank;
  const int q0 = tile * kQRows;
  if (q0 >= q_len) return;
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
  if (row >= q_len) return;
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

int64_t prefill_grid_size(int32_t max_q_len, int32_t T_q, int32_t B, int32_t Hkv) {
  // no prompt is longer than all the query tokens together
  const int64_t rows = max_q_len < T_q ? max_q_len : T_q;
  return (rows + kQRows - 1) / kQRows * B * Hkv;
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
  // |scale| in log2 units, floored so that a zero scale still maps masked
  // (-inf) scores to -inf instead of NaN; any real score times 1e-30 is 0.
  p.c_log2 = (a.scale < 0.f ? -a.scale : a.scale) * kLog2e;
  if (p.c_log2 < 1e-30f) p.c_log2 = 1e-30f;
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const int64_t grid = prefill_grid_size(a.max_q_len, a.T_q, a.B, a.Hkv);
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
