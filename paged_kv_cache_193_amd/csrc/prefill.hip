// prefill.hip -- causal paged prefill: every prompt token attends to the
// cached tokens up to and including its own position, reading K/V through the
// block table (tiny-vllm README, table of contents "Prefill vs decode",
// "Attention", "GQA", "Causal mask", "Online softmax", "Paged Attention";
// nano-vLLM guide announcement ch. 6: prefill is compute bound).  Here the
// path is a dense contraction, so Q.K^T and P.V run on CDNA4 bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Work unit: one workgroup per (64-row query tile, sequence b, KV group g);
// its 4 wavefronts are the 4 query heads of the group, so every K/V tile
// staged in LDS serves all of them (GQA).  Each wavefront holds, in registers,
//   S^T[64 keys][64 q]   = K . Q^T       (4 MFMA tiles of 32x32)
//   O^T[64 d][64 q]     += V^T . P^T     (4 MFMA tiles of 32x32)
// The MFMA accumulator layout puts one query column and 16 keys in a lane
// (rows 8*(r/4) + 4*(lane/32) + r%4, column lane%32), which is exactly the
// layout P^T needs as the B operand of the next product: the softmax runs on
// the scores where they are and no lane exchange is needed for P.  The row
// statistics (max, sum) are per query column: in-lane over 32 keys plus one
// exchange with lane^32.
//
// LDS per workgroup, double buffered: K tile [64 keys][64 d] row major and
// V^T tile [64 d][64 keys] (the B-side key index must run along registers,
// so V is transposed once per tile here and read back 8 bytes at a time),
// plus each wavefront's Q^T operand.  Rows are padded to spread LDS banks.
// Rows of keys past the context, or of an invalid block, are zero filled, so
// 0 * NaN cannot reach the MFMA.
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
// only diagonal tiles are masked.
//
// Two launch forms:
//  - prefill_kernel (no workspace): one workgroup per (query tile, sequence,
//    KV group), heaviest query tiles first, KV group fastest varying.  The
//    last query tile of a long prompt walks every key tile of the prompt, so
//    it sets the kernel's length.
//  - split form (with a workspace): the same grid with every query tile that
//    sees more than kSplitTiles key tiles cut into two halves of its key
//    range, one workgroup each, so the longest unit is about half as long.
//    Each half writes a record (unnormalised O, m, l); the half that finishes
//    second merges both by log-sum-exp, writes the rows and re-zeroes the
//    counter.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;
constexpr int kBS = 16;
constexpr int kTile = 64;          // query rows per workgroup and keys per K/V tile
constexpr int kKRow = kD + 8;      // K tile row stride (bf16 elements): 144 bytes
constexpr int kVRow = kTile + 4;   // V^T tile row stride (bf16 elements): 136 bytes
// A lane's partial row sum of one tile's weights above this (or not a number)
// sends the tile through the exact-max path.  Weights stay below 2^10.
constexpr float kLazyBound = 1024.f;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // bf16 pair (1, 1)
// split form: query tiles that see more key tiles than this are cut in two
constexpr int kSplitTiles = 16;

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
  // split form only
  float* ws_o;          // records: [record][wave][16][lane] f32x4, unnormalised O
  float* ws_ml;         // records: [record][wave][qt][lane] (m, l)
  uint32_t* ws_count;   // per (split query tile, KV group): halves finished
};

// Split records are written and read with 16-byte buffer accesses at agent
// scope (sc1), so a piece written on one XCD is seen by a workgroup merging on
// another; the descriptors also bound every access to the records.
constexpr int kSc1 = 16;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, dword data
constexpr int kRecOBytes = kPrefillRecordOBytes;    // 4 waves x 16 f32x4 x 64 lanes
constexpr int kRecMLBytes = kPrefillRecordMLBytes;  // 4 waves x 2 column sets x 64 lanes x (m, l)
static_assert(kRecOBytes == 4 * 16 * 64 * 16 && kRecMLBytes == 4 * 2 * 64 * 8,
              "record layout");
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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

// Physical id of the block holding this thread's keys in the tile that starts
// at key k0 (the logical block index is clamped to the table row, so the read
// is always in bounds; keys past the context are zeroed by load_tile).
__device__ __forceinline__ int tile_block_id(const PParams& p, const int32_t* trow, int k0,
                                             int tid) {
  int jb = (k0 + 2 * (tid >> 3)) / kBS;
  jb = jb < p.max_blocks ? jb : p.max_blocks - 1;
  return trow[jb];
}

// Load this thread's share of the tile at key k0 from block `phys`.  The
// loads are unconditional (an invalid id reads block 0), so the number of
// loads in flight is the same on every path; rows of keys past the context
// or of an invalid block are replaced by zeros afterwards.
__device__ __forceinline__ void load_tile(TileRegs& r, const PParams& p, int phys, int g,
                                          int ctx, int k0, int tid) {
  const int kp = tid >> 3, c = tid & 7;
  const int key0 = k0 + 2 * kp;  // key0 and key0 + 1 share one 16-token block
  const bool ok = phys >= 0 && phys < p.num_blocks;
  const int64_t base = (((int64_t)(ok ? phys : 0) * p.Hkv + g) * kBS + (key0 % kBS)) * kD + 8 * c;
  r.k0 = *reinterpret_cast<const u32x4*>(p.k_cache + base);
  r.v0 = *reinterpret_cast<const u32x4*>(p.v_cache + base);
  r.k1 = *reinterpret_cast<const u32x4*>(p.k_cache + base + kD);
  r.v1 = *reinterpret_cast<const u32x4*>(p.v_cache + base + kD);
  const u32x4 zero = {0, 0, 0, 0};
  if (!(ok && key0 < ctx)) r.k0 = r.v0 = zero;
  if (!(ok && key0 + 1 < ctx)) r.k1 = r.v1 = zero;
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* ks, uint16_t* vt,
                                           int tid) {
  const int kp = tid >> 3, c = tid & 7;
  *reinterpret_cast<u32x4*>(ks + (2 * kp) * kKRow + 8 * c) = r.k0;
  *reinterpret_cast<u32x4*>(ks + (2 * kp + 1) * kKRow + 8 * c) = r.k1;
  // V^T[d][key]: pair keys (2kp, 2kp+1) at each d into one dword
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = __builtin_amdgcn_perm(r.v1[w], r.v0[w], 0x05040100u);  // d = 8c+2w
    const uint32_t hi = __builtin_amdgcn_perm(r.v1[w], r.v0[w], 0x07060302u);  // d = 8c+2w+1
    *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * w) * kVRow + 2 * kp) = lo;
    *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * w + 1) * kVRow + 2 * kp) = hi;
  }
}

// Softmax and accumulator state of one wavefront's 64 query columns.
struct QTileState {
  f32x16 o[2][2];   // O^T [dt][qt], unnormalised (weights against m_ref)
  float m_ref[2];   // reference max per column, log2 units
  float l_run[2];   // this lane's share of the row sum
  bool has_ref[2];  // false until the column has seen a visible key
};

__device__ __forceinline__ void reset_state(QTileState& st) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) st.o[a][c] = kZero16;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    st.m_ref[qt] = 0.f;
    st.l_run[qt] = 0.f;
    st.has_ref[qt] = false;
  }
}

// Q^T operand of query rows [q0, q0 + 64) of head h, kept in this wavefront's
// LDS area: lane holds q row (qt*32 + lane%32), d in [k*16 + 8*(lane/32), +8).
// Rows past the prompt repeat its last row (their results are not written).
__device__ __forceinline__ void load_q_operand(u32x4* qsw, const PParams& p, int qs, int q_len,
                                               int q0, int h, int lane) {
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    int row = q0 + qt * 32 + lr;
    row = row < q_len ? row : q_len - 1;
    const uint16_t* qr = p.q + ((int64_t)(qs + row) * p.Hq + h) * kD + 8 * lh;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      qsw[(qt * 4 + k) * 64 + lane] = *reinterpret_cast<const u32x4*>(qr + 16 * k) ^
                                      u32x4{p.q_sign, p.q_sign, p.q_sign, p.q_sign};
  }
}

// Key tiles [kt_a, kt_b) (kt_b > kt_a) of one query tile, accumulated into
// st.  K/V tiles go global -> registers -> LDS one tile ahead of the MFMAs,
// and the block id of the tile after that is read one more tile ahead, so no
// load waits on a table read.  Ends with a workgroup barrier; the LDS tile
// buffers are free again afterwards.
__device__ __forceinline__ void run_key_tiles(QTileState& st, const PParams& p, uint16_t* ks_base,
                                              uint16_t* vt_base, const u32x4* qsw,
                                              const int32_t* trow, int g, int ctx, int pos_first,
                                              int kt_a, int kt_b, int tid, int lane) {
  const int lr = lane & 31, lh = lane >> 5;
  const float c2 = p.c_log2;
  TileRegs nxt;
  int id_next = tile_block_id(p, trow, (kt_a + 1) * kTile, tid);
  load_tile(nxt, p, tile_block_id(p, trow, kt_a * kTile, tid), g, ctx, kt_a * kTile, tid);
  store_tile(nxt, ks_base, vt_base, tid);
  __syncthreads();

  for (int it = kt_a; it < kt_b; ++it) {
    const int k0 = it * kTile;
    const int buf = (it - kt_a) & 1;
    // past the last tile these read clamped, unused data (no branch, so the
    // load counts stay static)
    load_tile(nxt, p, id_next, g, ctx, k0 + kTile, tid);
    id_next = tile_block_id(p, trow, k0 + 2 * kTile, tid);
    const uint16_t* ks = ks_base + buf * (kTile * kKRow);
    const uint16_t* vt = vt_base + buf * (kD * kVRow);

    // S^T = K . Q^T  (scores before scaling)
    f32x16 s[2][2];  // [kt][qt]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x8_t a = as_bf16x8(
            *reinterpret_cast<const u32x4*>(ks + (kt * 32 + lr) * kKRow + 16 * k + 8 * lh));
        const bf16x8_t q0 = as_bf16x8(qsw[(0 * 4 + k) * 64 + lane]);
        const bf16x8_t q1 = as_bf16x8(qsw[(1 * 4 + k) * 64 + lane]);
        s[kt][0] = mfma(a, q0, k == 0 ? kZero16 : s[kt][0]);
        s[kt][1] = mfma(a, q1, k == 0 ? kZero16 : s[kt][1]);
      }
    }

    // causal mask on tiles that reach past the first row's position: key j of
    // this lane's column is visible iff j <= min(pos, ctx - 1)
    if (k0 + kTile - 1 > pos_first) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int pos = pos_first + qt * 32 + lr;
        const int lim = (pos < ctx - 1 ? pos : ctx - 1) - (k0 + 4 * lh);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kt * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kt][qt][r] = -INFINITY;
      }
    }

    // Weights against the reference: P^T operand as bf16, and this lane's
    // partial row sums of the same rounded weights (v_dot2 against (1, 1)).
    bf16x8_t pop[2][4];
    float lsum[2];
    auto weights = [&](int qt, float m) {
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * half + 2 * e;
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][qt][r], c2, -m));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][qt][r + 1], c2, -m));
            w[e] = pack_bf16(p0, p1);
            if (e & 1)
              l1 = dot2_bf16(w[e], kOnesBf16x2, l1);
            else
              l0 = dot2_bf16(w[e], kOnesBf16x2, l0);
          }
          pop[qt][2 * kt + half] = as_bf16x8(w);
        }
      lsum[qt] = l0 + l1;
    };
    weights(0, st.m_ref[0]);
    weights(1, st.m_ref[1]);

    // Exact-max path, wave-uniform and rare: a weight may exceed the bound
    // (a score rose well above the reference), or a column has no reference
    // yet.  The reference moves up to the tile max, the accumulator and row
    // sum are rescaled, and the weights are formed again.  By the softmax
    // shift identity the result does not depend on the reference used.
    bool redo = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) redo = redo || !(lsum[qt] <= kLazyBound) || !st.has_ref[qt];
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float v = fmaxf(s[0][qt][0], s[0][qt][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) v = fmaxf(v, s[0][qt][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) v = fmaxf(v, s[1][qt][r]);
        const float mx = fmaxf(v, shfl_xor(v, 32)) * c2;  // tile max, log2 units
        // no visible key yet: stay without a reference (weights are 0)
        if (mx != -INFINITY && mx == mx) {
          const float m_new = st.has_ref[qt] ? fmaxf(st.m_ref[qt], mx) : mx;
          const float alpha = st.has_ref[qt] ? __builtin_amdgcn_exp2f(st.m_ref[qt] - m_new) : 0.f;
          st.l_run[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.o[dt][qt][r] *= alpha;
          st.m_ref[qt] = m_new;
          st.has_ref[qt] = true;
        }
        weights(qt, st.m_ref[qt]);
      }
    }
    st.l_run[0] += lsum[0];
    st.l_run[1] += lsum[1];

    // O^T += V^T . P^T
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
      const int kb = stp * 16;  // key offset of this 16-key step within the tile
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const uint16_t* vrow = vt + (dt * 32 + lr) * kVRow + kb + 4 * lh;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
        const bf16x8_t a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        st.o[dt][0] = mfma(a, pop[0][stp], st.o[dt][0]);
        st.o[dt][1] = mfma(a, pop[1][stp], st.o[dt][1]);
      }
    }

    store_tile(nxt, ks_base + (buf ^ 1) * (kTile * kKRow), vt_base + (buf ^ 1) * (kD * kVRow),
               tid);
    __syncthreads();
  }
}

// out[row][h][d] = O^T[d][row] / l(row) for the rows of query tile q0 that
// lie in the prompt; columns without a visible key give zero rows.
__device__ __forceinline__ void write_rows(const QTileState& st, const PParams& p, int qs,
                                           int q_len, int q0, int h, int lane) {
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = st.l_run[qt] + shfl_xor(st.l_run[qt], 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int row = q0 + qt * 32 + lr;
    if (row >= q_len) continue;
    const int64_t base = ((int64_t)(qs + row) * p.Hq + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = dt * 32 + 8 * gq + 4 * lh;
        const float x0 = st.o[dt][qt][4 * gq + 0] * inv, x1 = st.o[dt][qt][4 * gq + 1] * inv;
        const float x2 = st.o[dt][qt][4 * gq + 2] * inv, x3 = st.o[dt][qt][4 * gq + 3] * inv;
        if (p.out_f32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + base + d) =
              make_float4(x0, x1, x2, x3);
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + base + d) =
              u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
        }
      }
  }
}

// Records of halves of split query tiles: each piece has its own 64 KB of
// O (addressed through a per-record descriptor, so the workspace may exceed
// 4 GB) and 4 KB of (m, l).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_o(const PParams& p, int record) {
  return __builtin_amdgcn_make_buffer_rsrc(p.ws_o + (int64_t)record * (kRecOBytes / 4), (short)0,
                                           kRecOBytes, kRsrcWord3);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_ml(const PParams& p, int record) {
  return __builtin_amdgcn_make_buffer_rsrc(p.ws_ml + (int64_t)record * (kRecMLBytes / 4),
                                           (short)0, kRecMLBytes, kRsrcWord3);
}

// This wavefront's piece of a split query tile: O unnormalised in register
// order, (m, l) per column set (m = -inf for columns without a visible key).
__device__ __forceinline__ void store_record(const QTileState& st, const PParams& p, int record,
                                             int wave, int lane) {
  const __amdgpu_buffer_rsrc_t ro = rec_o(p, record);
  const int obase = wave * (16 * 64 * 16) + lane * 16;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = {st.o[dt][qt][4 * j], st.o[dt][qt][4 * j + 1], st.o[dt][qt][4 * j + 2],
                         st.o[dt][qt][4 * j + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, obase + ((dt * 2 + qt) * 4 + j) * 1024, 0,
                                               kSc1);
      }
  const __amdgpu_buffer_rsrc_t rml = rec_ml(p, record);
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const f32x2 ml = {st.has_ref[qt] ? st.m_ref[qt] : -INFINITY, st.l_run[qt]};
    __builtin_amdgcn_raw_buffer_store_b64(ml, rml, (wave * 2 + qt) * 512 + lane * 8, 0, kSc1);
  }
}

// Fold one stored piece into st: log-sum-exp combination.  Starting from a
// reset state, folding a piece reproduces it exactly.
__device__ __forceinline__ void fold_record(QTileState& st, const PParams& p, int record,
                                            int wave, int lane) {
  const __amdgpu_buffer_rsrc_t ro = rec_o(p, record);
  const __amdgpu_buffer_rsrc_t rml = rec_ml(p, record);
  const int obase = wave * (16 * 64 * 16) + lane * 16;
  f32x4 ov[16];
#pragma unroll
  for (int k = 0; k < 16; ++k)
    ov[k] = __builtin_amdgcn_raw_buffer_load_b128(ro, obase + k * 1024, 0, kSc1);
  f32x2 ml[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
    ml[qt] = __builtin_amdgcn_raw_buffer_load_b64(rml, (wave * 2 + qt) * 512 + lane * 8, 0, kSc1);
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mp = ml[qt][0], lp = ml[qt][1];
    const float mo = st.has_ref[qt] ? st.m_ref[qt] : -INFINITY;
    const float mn = fmaxf(mo, mp);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float a = __builtin_amdgcn_exp2f(mo - mu);  // 0 for -inf
    const float w = __builtin_amdgcn_exp2f(mp - mu);
    st.l_run[qt] = st.l_run[qt] * a + lp * w;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st.o[dt][qt][4 * j + e] = st.o[dt][qt][4 * j + e] * a + ov[(dt * 2 + qt) * 4 + j][e] * w;
    st.m_ref[qt] = mu;
    st.has_ref[qt] = mn != -INFINITY;
  }
}

// Wait until every store this wavefront issued has completed (vmcnt 0).
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// kSplit: query tiles with more than kSplitTiles key tiles are cut in two
// halves of their key range, each half one workgroup; the half that finishes
// second folds both records (in key order, so the result does not depend on
// which half that is), writes the rows and re-zeroes the counter.
template <bool kSplit>
__global__ void __launch_bounds__(256, 2)
prefill_kernel(PParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_buf[2 * kTile * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vt_buf[2 * kD * kVRow];
  __shared__ u32x4 qs_buf[4][2 * 4 * 64];
  __shared__ uint32_t s_count;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // grid: g fastest, then the half (split form), then b, then query tile from
  // the last (heaviest) down
  const int g = blockIdx.x % p.Hkv;
  int rest = blockIdx.x / p.Hkv;
  const int half = kSplit ? rest & 1 : 0;
  if (kSplit) rest >>= 1;
  const int b = rest % p.B;
  const int tile = p.tiles_max - 1 - rest / p.B;

  const int qs = p.cu_q_lens[b];
  const int q_len = p.cu_q_lens[b + 1] - qs;
  const int q0 = tile * kTile;
  if (q0 >= q_len) return;
  int ctx = p.context_lens[b];
  const int cap = p.max_blocks * kBS;
  ctx = ctx > cap ? cap : ctx;
  const int hist = ctx - q_len;  // position of query row 0 minus 0
  const int rows = q_len - q0 < kTile ? q_len - q0 : kTile;
  const int pos_first = hist + q0;
  const int pos_last = hist + q0 + rows - 1;
  int kend = pos_last + 1 < ctx ? pos_last + 1 : ctx;  // keys [0, kend)
  if (kend < 0) kend = 0;
  const int n_tiles = (kend + kTile - 1) / kTile;
  const bool cut = kSplit && n_tiles > kSplitTiles;
  if (half > 0 && !cut) return;
  const int kt_a = cut ? half * (n_tiles / 2) : 0;
  const int kt_b = cut && half == 0 ? n_tiles / 2 : n_tiles;
  const int h = 4 * g + wave;
  const int32_t* trow = p.block_tables + (int64_t)b * p.max_blocks;

  u32x4* qsw = qs_buf[wave];
  load_q_operand(qsw, p, qs, q_len, q0, h, lane);
  QTileState st;
  reset_state(st);
  if (kt_b > kt_a)
    run_key_tiles(st, p, ks_buf, vt_buf, qsw, trow, g, ctx, pos_first, kt_a, kt_b, tid, lane);
  if (!cut) {
    write_rows(st, p, qs, q_len, q0, h, lane);
    return;
  }
  // split query tile: its index among all query tiles of the batch is
  // qs / 64 + b + tile (distinct per tile, below T_q / 64 + B)
  const int pair = ((qs / kTile + b + tile) * p.Hkv + g);
  store_record(st, p, 2 * pair + half, wave, lane);
  drain_stores();
  __syncthreads();
  if (tid == 0)
    s_count = __hip_atomic_fetch_add(p.ws_count + pair, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(s_count) == 0) return;  // the other half merges
  reset_state(st);
  fold_record(st, p, 2 * pair, wave, lane);
  fold_record(st, p, 2 * pair + 1, wave, lane);
  write_rows(st, p, qs, q_len, q0, h, lane);
  if (tid == 0) __hip_atomic_store(p.ws_count + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

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
  p.tiles_max = (a.max_q_len + kTile - 1) / kTile;
  // |scale| in log2 units, floored so that a zero scale still maps masked
  // (-inf) scores to -inf instead of NaN; any real score times 1e-30 is 0.
  p.c_log2 = (a.scale < 0.f ? -a.scale : a.scale) * kLog2e;
  if (p.c_log2 < 1e-30f) p.c_log2 = 1e-30f;
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const int64_t grid = (int64_t)p.tiles_max * a.B * a.Hkv;
  if (a.workspace) {
    const PrefillSplitLayout ly = prefill_split_layout(a.B, a.T_q, a.Hkv);
    char* ws = static_cast<char*>(a.workspace);
    p.ws_count = reinterpret_cast<uint32_t*>(ws);
    p.ws_o = reinterpret_cast<float*>(ws + ly.o_offset);
    p.ws_ml = reinterpret_cast<float*>(ws + ly.ml_offset);
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)(2 * grid)), dim3(256), 0, stream, p);
  } else {
    p.ws_count = nullptr;
    p.ws_o = p.ws_ml = nullptr;
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
