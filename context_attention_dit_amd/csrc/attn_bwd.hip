// Backward of bf16 attention over a list of K/V chunks on CDNA4 matrix cores
// (gfx950).
//
// What it computes: the gradients of O = softmax(scale * Q K^T) V against an
// upstream gradient dO, over the K/V chunks it is given, from the row
// statistics the forward saved (the row log-sum-exp LSE, and
// Delta_i = <dO_i, O_i>):
//   P_ij  = exp(scale <q_i, k_j> - LSE_i)         (0 for masked pairs)
//   dS_ij = P_ij (<dO_i, v_j> - Delta_i)
//   dQ_i  = scale * sum_j dS_ij k_j,  dK_j = scale * sum_i dS_ij q_i,
//   dV_j  = sum_i P_ij dO_i.
// With the full rows' LSE and Delta every chunk's share is exact, so a ring
// rank sums dQ over the chunks it visits and adds each chunk's dK, dV share
// into that chunk's travelling accumulators (Context parallelism guide
// (diffusers), section Ring Attention, run backwards); one chunk over the
// whole sequence is a Ulysses rank's local backward (Ulysses Sequence
// Parallelism article: training with long contexts; detailed notes 2: the
// score matrix is never stored, so the weights are recomputed from the LSE).
//
// How it maps to the hardware. Two block bodies, each owning one kind of
// output and writing every element of it exactly once (no atomics: results
// are deterministic, and dQ / dK / dV can be accumulated into the caller's
// fp32 buffers with a plain read-add-write):
//  * dQ (query-stationary): 4 waves keep 128 query rows, with Q^T and dO^T
//    held in registers as B operands, and walk every chunk's 64-key K/V tiles
//    through double-buffered LDS. Per tile a wave computes S^T = K Q^T and
//    dP^T = V dO^T, forms dS^T in the accumulator layout (lane = query) and
//    adds dQ^T += K^T dS^T, the K^T fragments read transposed from the same K
//    tile (ds_read_b64_tr_b16). On grids with no more query tiles than compute
//    units a block is two such groups splitting the key tiles, their dQ
//    added through LDS at the end.
//  * dK/dV (key-stationary): 8 waves over 128 keys of one chunk. The keys' K
//    and V stay in LDS for the whole block and are read as B operands; the
//    two 4-wave groups take the two 32-row halves of every 64-row Q/dO tile.
//    Per half-tile a wave computes S = Q K^T and dP = dO V^T, forms P and dS
//    in the accumulator layout (lane = key) and adds dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T read transposed. The groups' partial
//    sums are added through LDS at the end, in a fixed order.
//  * Every streamed tile sits in LDS with row bits 2 and 3 swapped and its
//    16-byte units XOR-swizzled by the row. With the swap, the 32x32
//    accumulator registers of lane l hold 8 consecutive tile rows per
//    half-wave, which is exactly the B-operand layout of the next product, so
//    P and dS feed the second products without data movement; the transposed
//    reads of the same tile find those rows as two groups of four.
//  * Direct buffer->LDS loads (buffer_load_dwordx4 ... lds) fill the tiles
//    with no staging registers; one barrier per tile.
//  * Weights are exp2 of one FMA per score, with the signed scale*log2(e) and
//    -log2(e)*LSE (no row maximum is needed, so no sign trick either). A row
//    whose LSE is -inf saw no key anywhere and gets weight 0; a masked pair
//    gets a score whose product with the signed factor is -inf.
//  * Grids too small to fill the GPU run both bodies in one launch: the
//    two-group dQ blocks first, the dK/dV blocks behind them.
#include "cp_internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kBlk = 128;      // resident rows per block (queries or keys)
constexpr int kTile = 64;      // streamed rows per tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swap_bits23(int r) {
  return r ^ ((((r >> 2) ^ (r >> 3)) & 1) * 12);
}

template <int D>
struct Geo {
  static constexpr int kUPR = D / 8;                            // 16-byte units per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kTile * kRowBytes;
  static constexpr int kLoadsPerWave = kTile * kUPR / kThreads;  // direct loads per tile per wave
  static constexpr int kMask = kUPR - 1 < 15 ? kUPR - 1 : 15;    // swizzle row bits
};

// Byte offset of 16-byte unit `unit` of LDS row `row` within a tile.
template <int D>
__device__ __forceinline__ uint32_t unit_off(int row, int unit) {
  return row * Geo<D>::kRowBytes + ((unit ^ (row & Geo<D>::kMask)) << 4);
}

// Buffer resource over the `bytes` bytes from the wave-uniform `base` on (raw,
// stride 0), built in scalar registers. A load at or past `bytes` is out of
// range: nothing is fetched and zeros arrive (in LDS, for a direct load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p >> 32)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(hi << 32 | lo), 0,
                                           __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)),
                                           0x00020000);
}

// buffer_load_dwordx4 ... lds: lane i's 16 bytes at byte offset `voff` land in
// LDS at l + 16 i (l wave-uniform). The MUBUF form is counted on the
// vector-memory counter only, so LDS reads issued after it keep partial wait
// counts (the FLAT global_load_lds made every later LDS wait a full drain).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, char* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(l), 16,
                                           voff, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 read_tr(const char* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-lane geometry of one streamed tile: direct-load sources and fragment
// read offsets (bytes within the tile).
template <int D, int NT = kThreads>
struct TileGeo {
  static constexpr int NL = kTile * Geo<D>::kUPR / NT;  // direct loads per tile per wave
  // Row r0 + 8 of a transposed read flips swizzle bit 3 of the unit when the
  // swizzle spans 16 rows (D = 128), not when it spans 8 (D = 64).
  static constexpr uint32_t kHiX = Geo<D>::kMask >= 8 ? (8u << 4) : 0u;
  uint32_t src[NL];      // byte offset of each direct load's source from the tile's first row
  uint32_t n_rd0;        // normal fragment, k-step 0: LDS row = lane%32, unit half
  uint32_t t_lo[D / 32]; // transposed fragment, k-step 0, rows r0 .. r0+3 (add 16 t rows)
  int w8, lane;

  __device__ void init(int wave, int ln, int rs) {
    constexpr int UPR = Geo<D>::kUPR;
    w8 = wave;
    lane = ln;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      // LDS slot s = (row, unit) holds tile row swap(row), unit s%UPR ^ (row & mask)
      const int s = (wave * NL + n) * 64 + lane;
      const int row = s / UPR, pu = s % UPR;
      src[n] = 2u * static_cast<uint32_t>(swap_bits23(row) * rs + (pu ^ (row & Geo<D>::kMask)) * 8);
    }
    const int col = lane & 31, half = lane >> 5;
    n_rd0 = unit_off<D>(col, half);
    // ds_read_b64_tr_b16: in each 16-lane group, lane i addresses row r0 + i/4,
    // elements el .. el+3, and receives element column (group's base) + i of
    // rows r0 .. r0+3. LDS rows 4h .. 4h+3 hold tile rows 8h .. 8h+3 and rows
    // 8+4h .. 8+4h+3 hold 8h+4 .. 8h+7 (bits 2/3 swapped), the 8 consecutive
    // rows half-wave h needs in a 16-row k-step.
    const int g16 = lane >> 4, j16 = lane & 15;
    const int r0 = 4 * (g16 >> 1) + (j16 >> 2);
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
      const int el = 32 * md + 16 * (g16 & 1) + 4 * (j16 & 3);
      t_lo[md] = unit_off<D>(r0, el >> 3) + ((el & 4) ? 8 : 0);
    }
  }

  // Direct loads of tile rows [row0, row0 + 64) of a [.][rs] bf16 tensor
  // (`base` points at row 0, head offset included) into the tile at `dst`.
  // The buffer's range ends after row n_rows - 1, so rows at or beyond n_rows
  // arrive as zeros (their weights are zero wherever they are used).
  __device__ void issue(const char* base, int row0, int n_rows, int rs, char* dst, int wave) const {
    issue_tile(base + 2 * static_cast<int64_t>(row0) * rs, n_rows - row0, rs, dst, wave);
  }
  // The same with `tile` pointing at the tile's first row and `n_valid` rows
  // from there on that exist.
  __device__ void issue_tile(const char* tile, int n_valid, int rs, char* dst, int wave) const {
    n_valid = max(0, min(n_valid, kTile));  // (0: nothing is fetched)
    const __amdgpu_buffer_rsrc_t rsrc =
        tile_rsrc(tile, static_cast<uint32_t>(n_valid) * static_cast<uint32_t>(2 * rs));
    char* l = dst + wave * NL * 1024;
#pragma unroll
    for (int n = 0; n < NL; ++n) lds_load16(rsrc, src[n], l + n * 1024);
  }

  // A operand: tile^T rows d = 32 md + lane%32, k = tile rows 16 t + 8 half + 0..7
  __device__ bf16x8 tr_frag(const char* tile, int md, int t) const {
    const bf16x4 lo = read_tr(tile + t_lo[md] + 16 * t * Geo<D>::kRowBytes);
    const bf16x4 hi = read_tr(tile + (t_lo[md] ^ kHiX) + (16 * t + 8) * Geo<D>::kRowBytes);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // A operand: tile rows 32 mb + lane%32 (tile row swap of it), k = d 16 ks + 8 half + 0..7.
  // Unit 2 ks + half: the swizzle XOR leaves the low unit bit to `half`, so the
  // offset is n_rd0 with the unit's upper bits XORed by ks.
  __device__ bf16x8 frag(const char* tile, int mb, int ks) const {
    return *reinterpret_cast<const bf16x8*>(tile + (n_rd0 ^ (ks << 5)) +
                                            mb * 32 * Geo<D>::kRowBytes);
  }
};

// One row of a [.][H][D] bf16 tensor as B-operand fragments: lane holds
// elements 16 ks + 8 half .. +7 of the row at `p` (zeros if !valid).
template <int D>
__device__ __forceinline__ void load_row_frags(const __bf16* p, bool valid, int half, bf16x8* f) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 w = *reinterpret_cast<const u32x4*>(p + 16 * ks + 8 * half);
    if (!valid) w = u32x4{0, 0, 0, 0};
    f[ks] = __builtin_bit_cast(bf16x8, w);
  }
}

// -log2(e) * LSE, with a row that saw no key (LSE = -inf) mapped to -inf so
// that its weights exp2(s * sl2 + nl) are 0.
__device__ __forceinline__ float neg_lse2(float lse) {
  return lse == -INFINITY ? -INFINITY : -lse * kLog2e;
}

// exp2 factor scale * log2(e), kept away from 0 so that a masked score times
// it is never inf * 0.
__device__ __forceinline__ float signed_sl2(float scale) {
  return copysignf(fmaxf(fabsf(scale) * kLog2e, 1e-30f), scale);
}
// The score a masked (row, key) pair is given: its product with signed_sl2 is
// -inf, so its weight exp2(...) is exactly 0.
__device__ __forceinline__ float masked_score(float scale) {
  return scale < 0.f ? INFINITY : -INFINITY;
}

// Store 4 consecutive fp32 values scaled by `s`, adding the old values if `acc`.
__device__ __forceinline__ void store4(float* p, float s, float x0, float x1, float x2, float x3,
                                      bool acc) {
  float4 r = make_float4(s * x0, s * x1, s * x2, s * x3);
  if (acc) {
    const float4 o = *reinterpret_cast<const float4*>(p);
    r.x += o.x;
    r.y += o.y;
    r.z += o.z;
    r.w += o.w;
  }
  *reinterpret_cast<float4*>(p) = r;
}

// Block index -> (work item) with consecutive ids spread over the 8 XCDs and
// each XCD taking a contiguous run of items (the tiles of one head stay in
// one L2). Returns -1 for the padding blocks of the last round. `blk` counts
// from a multiple of 8, so blk % 8 is still the XCD the block runs on.
__device__ __forceinline__ int xcd_item(int blk, int nitems) {
  const int per_xcd = (nitems + 7) / 8;
  const int L = (blk % 8) * per_xcd + blk / 8;
  return L < nitems ? L : -1;
}

// ---------------------------------------------------------------- dQ kernel
// G = 1: a block is 4 waves over 128 query rows, visiting every key tile of
// every chunk in order. G = 2: two such groups of 4 waves share the query
// rows, group g taking half g of the key tiles with its own LDS stages; their
// dQ accumulators are added through LDS at the end (grids with no more query
// tiles than compute units).
template <int D, bool CAUSAL, int G>
__device__ __forceinline__ void dq_body(const BwdArgs& a, char* smem, int blk) {
  constexpr int TB = Geo<D>::kTileBytes;
  // smem: G * 4 * TB bytes; per group, stage s holds K at 2s, V at 2s + 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int grp = G == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
  const int col = lane & 31, half = lane >> 5;
  char* const gsm = smem + (G == 1 ? 0 : grp * 4 * TB);
  const int BH = a.B * a.H;
  const int nqt = (a.Sq + kBlk - 1) / kBlk;
  int bh, qt;
  if (CAUSAL) {  // the last query tiles see the most keys: launch them first
    if (blk >= nqt * BH) return;
    qt = nqt - 1 - blk / BH;
    bh = blk % BH;
  } else {
    const int L = xcd_item(blk, nqt * BH);
    if (L < 0) return;
    bh = L / nqt;
    qt = L % nqt;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int i = qt * kBlk + wave * 32 + col;  // this lane's query row
  const bool valid = i < a.Sq;
  const int ic = valid ? i : a.Sq - 1;
  const int q_first = qt * kBlk, q_last = min(q_first + kBlk - 1, a.Sq - 1);
  const int rs = a.H * D;

  // resident B operands: Q^T and dO^T
  bf16x8 qf[D / 16], df[D / 16];
  const int64_t qrow = (static_cast<int64_t>(b) * a.Sq + ic) * a.H + h;
  load_row_frags<D>(a.q + qrow * D, valid, half, qf);
  load_row_frags<D>(a.dout + qrow * D, valid, half, df);
  const int64_t lrow = (static_cast<int64_t>(b) * a.H + h) * a.Sq + ic;
  const float nl = valid ? neg_lse2(a.lse[lrow]) : -INFINITY;
  const float dlt = valid ? a.delta[lrow] : 0.f;
  const float sl2 = signed_sl2(a.scale);  // no row maximum is needed here
  const float s_mask = masked_score(a.scale);

  // Chunk descriptors are read with a provably uniform index (scalar loads).
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto keys_of = [&](int c) {  // keys of chunk c this query tile can see
    c = uni(c);
    int n = a.chunks[c].len;
    if (CAUSAL) n = max(0, min(n, q_last + a.chunks[c].diag + 1));
    return n;
  };
  // A cursor carries its chunk's descriptor (visible keys nk, stored keys len,
  // diagonal offset diag) and the addresses of its K and V tile for this
  // (batch, head), set when it enters the chunk and stepped by one tile stride
  // after that, so the steps issue no scalar loads of their own.
  struct Cur {
    int c, kt;
    int nk, len, diag;
    const char* tk;
    const char* tv;
  };
  const int64_t tile_bytes = 2 * static_cast<int64_t>(kTile) * rs;
  auto enter = [&](Cur& x) {
    const int c = uni(x.c);
    if (c < a.nchunks) {  // (a cursor past the list is never used)
      x.len = a.chunks[c].len;
      x.diag = a.chunks[c].diag;
      x.nk = CAUSAL ? max(0, min(x.len, q_last + x.diag + 1)) : x.len;
      const int64_t off =
          2 * ((static_cast<int64_t>(b) * x.len + uni(x.kt) * kTile) * rs + static_cast<int64_t>(h) * D);
      x.tk = reinterpret_cast<const char*>(a.chunks[c].k) + off;
      x.tv = reinterpret_cast<const char*>(a.chunks[c].v) + off;
    }
  };
  auto next_of = [&](Cur x) {
    x.kt = uni(x.kt) + 1;
    if (x.kt * kTile >= x.nk) {
      x.kt = 0;
      x.c = uni(x.c) + 1;
      while (x.c < a.nchunks && keys_of(x.c) == 0) ++x.c;
      enter(x);
    } else {
      x.tk += tile_bytes;
      x.tv += tile_bytes;
    }
    return x;
  };

  TileGeo<D> g;
  g.init(wave, lane, rs);
  auto issue = [&](char* dst, const Cur& x) {
    const int n_valid = x.nk - uni(x.kt) * kTile;
    g.issue_tile(x.tk, n_valid, rs, dst, wave);
    g.issue_tile(x.tv, n_valid, rs, dst + TB, wave);
  };

  // this group's share of the tiles, in chunk order
  Cur cur{0, 0, 0, 0, 0, nullptr, nullptr};
  int left, steps;
  {
    int total = 0;
    for (int c = 0; c < a.nchunks; ++c) total += (keys_of(c) + kTile - 1) / kTile;
    const int t_begin = G == 2 ? (grp == 0 ? 0 : total / 2) : 0;
    const int t_end = G == 2 ? (grp == 0 ? total / 2 : total) : total;
    left = uni(t_end - t_begin);
    steps = uni(G == 2 ? total - total / 2 : total);  // both groups join every barrier
    int skip = t_begin;
    while (cur.c < a.nchunks) {
      const int nt = (keys_of(cur.c) + kTile - 1) / kTile;
      if (skip < nt) break;
      skip -= nt;
      ++cur.c;
    }
    cur.kt = skip;
    enter(cur);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md) acc[md] = f32x16{};

  if (left > 0) issue(gsm, cur);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j < steps; ++j) {
    if (G == 1 || j < left) {  // (a group out of tiles still joins the barrier below)
      const int st = j & 1;
      const char* kl = gsm + 2 * st * TB;
      const char* vl = kl + TB;
      Cur nx = cur;
      if (j + 1 < left) {
        nx = next_of(cur);
        issue(gsm + 2 * (st ^ 1) * TB, nx);
      }
      const int len = cur.len, diag = cur.diag;
      const int key0 = uni(cur.kt) * kTile;
      // S^T and dP^T for the tile's 64 keys (two 32-key blocks); register r
      // of block mb is key key0 + 32 mb + 16 (r/8) + 8 half + r%8
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = mfma(g.frag(kl, mb, 0), qf[0], f32x16{});
        dp[mb] = mfma(g.frag(vl, mb, 0), df[0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < D / 16; ++ks) {
          s[mb] = mfma(g.frag(kl, mb, ks), qf[ks], s[mb]);
          dp[mb] = mfma(g.frag(vl, mb, ks), df[ks], dp[mb]);
        }
      }
      // interleave: each fragment read runs 4 MFMAs ahead of its product
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < 4 * (D / 16); ++k) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      const bool masked = key0 + kTile > len || (CAUSAL && key0 + kTile - 1 > q_first + diag);
      if (masked) {
        asm volatile("" ::: "memory");
        int lim = len - key0;
        if (CAUSAL) lim = min(lim, i + diag - key0 + 1);
        lim -= 8 * half;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * mb + 16 * (r >> 3) + (r & 7) >= lim) s[mb][r] = s_mask;
      }
      // k-step t: dS^T rounded to bf16 (B operand: keys 16 t + 8 half + e), then
      // dQ^T += K^T dS^T over its 16 keys
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 dsf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int mb = t >> 1, r = (t & 1) * 8 + e;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][r], sl2, nl));
          dsf[e] = static_cast<__bf16>(p * (dp[mb][r] - dlt));
        }
#pragma unroll
        for (int md = 0; md < D / 32; ++md) acc[md] = mfma(g.tr_frag(kl, md, t), dsf, acc[md]);
      }
      // interleave: the transposed reads run 4 MFMAs ahead; the next k-step's
      // dS arithmetic fills the gaps between this k-step's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 36, 0);
#pragma unroll
      for (int k = 0; k < 4 * (D / 32); ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 36 / (D / 32), 0);
      }
      cur = nx;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (G == 2) {  // group 1 hands its dQ^T to group 0 (the loop ended with a barrier)
    float* x = reinterpret_cast<float*>(smem);  // [wave][md][r][lane]
    if (grp == 1) {
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[((wave * (D / 32) + md) * 16 + r) * 64 + lane] = acc[md][r];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[md][r] += x[((wave * (D / 32) + md) * 16 + r) * 64 + lane];
  }
  if (!valid) return;
  // dQ^T register r of block md is element d = 32 md + 8 (r/4) + 4 half + r%4
  float* out = a.dq + qrow * D;
#pragma unroll
  for (int md = 0; md < D / 32; ++md)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      store4(out + 32 * md + 8 * q4 + 4 * half, a.scale, acc[md][4 * q4], acc[md][4 * q4 + 1],
             acc[md][4 * q4 + 2], acc[md][4 * q4 + 3], a.accum_dq != 0);
}

// -------------------------------------------------------------- dK/dV kernel
// A block is 8 waves over 128 keys: wave w of group g holds keys 32 (w%4) ..
// +31 and takes rows 32 g .. 32 g + 31 of every 64-row Q/dO tile, so the two
// groups split each tile and the block's dK, dV are the sum of the groups'
// partial accumulators (merged through LDS at the end, in a fixed order).
// The block's K and V rows sit in LDS for the whole kernel and are read as B
// operands, which keeps a wave within 256 registers (two waves per SIMD).
constexpr int kKvThreads = 512;

template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, char* smem, int blk) {
  constexpr int TB = Geo<D>::kTileBytes;  // one 64-row tile
  // smem (8 TB + 1024 bytes): [K: 2 tiles][V: 2 tiles][stage 0: Q, dO]
  // [stage 1: Q, dO][stats: 2 x 512 B]
  constexpr int KV_BYTES = 4 * TB, ST_OFF = 8 * TB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave in block, 0..7
  const int grp = w8 >> 2, wave = w8 & 3;                    // row half, key group
  const int col = lane & 31, half = lane >> 5;
  const int BH = a.B * a.H;
  const int nkt = a.total_kt;  // key tiles over all chunks
  int bh, t;
  if (CAUSAL) {  // in chunk order, the first key tiles are seen by the most queries
    if (blk >= nkt * BH) return;
    t = blk / BH;
    bh = blk % BH;
  } else {  // the key tiles of one head (every chunk) stay on one XCD
    const int L = xcd_item(blk, nkt * BH);
    if (L < 0) return;
    bh = L / nkt;
    t = L % nkt;
  }
  // chunk of key tile t (uniform scalar scan over at most 64 descriptors)
  int c = 0;
  while (c + 1 < a.nchunks && a.chunks[c + 1].tile0 <= t) ++c;
  c = __builtin_amdgcn_readfirstlane(c);
  const BwdChunk& ch = a.chunks[c];
  const int len = ch.len, diag = ch.diag;
  const int kt = t - ch.tile0;
  const int b = bh / a.H, h = bh - b * a.H;
  const int jk = kt * kBlk + wave * 32 + col;  // this lane's key within the chunk
  const int k_first = kt * kBlk, k_last = min(k_first + kBlk - 1, len - 1);
  const int rs = a.H * D;
  // exp2 factor with the scale's sign (no row maximum is needed here)
  const float sl2 = signed_sl2(a.scale);
  const float s_mask = masked_score(a.scale);

  int qt0 = 0;  // first query tile that can see this block's keys
  if (CAUSAL) {
    const int qmin = k_first - diag;
    qt0 = qmin <= 0 ? 0 : qmin / kTile;
  }
  const int nqt = (a.Sq + kTile - 1) / kTile;
  const int ntiles = max(0, nqt - qt0);

  TileGeo<D, kKvThreads> g;
  g.init(w8, lane, rs);
  const int64_t head = (static_cast<int64_t>(b) * a.Sq * a.H + h) * D;
  const char* qbase = reinterpret_cast<const char*>(a.q + head);
  const char* dbase = reinterpret_cast<const char*>(a.dout + head);
  const int64_t lbase = (static_cast<int64_t>(b) * a.H + h) * a.Sq;

  // the block's K and V: two 64-row tiles each, same row-swapped layout
  {
    const int64_t kvh = (static_cast<int64_t>(b) * len * a.H + h) * D;
    const char* kb = reinterpret_cast<const char*>(ch.k + kvh);
    const char* vb = reinterpret_cast<const char*>(ch.v + kvh);
    g.issue(kb, k_first, len, rs, smem, w8);
    g.issue(vb, k_first, len, rs, smem + 2 * TB, w8);
    if (k_first + kTile < len) {
      g.issue(kb, k_first + kTile, len, rs, smem + TB, w8);
      g.issue(vb, k_first + kTile, len, rs, smem + 3 * TB, w8);
    }
  }
  // B-operand reads of this wave's keys: block row 32 wave + col sits in tile
  // wave/2 at LDS row swap(32 (wave%2) + col)
  uint32_t kv_rd0;
  {
    const int local = 32 * (wave & 1) + col;
    kv_rd0 = (wave >> 1) * TB + unit_off<D>(swap_bits23(local), half);
  }
  // unit 2 ks + half of the same row: the swizzle XOR leaves the low unit bit
  // to `half`, so the offset of k-step ks is kv_rd0 ^ (ks << 5)
  auto kv_frag = [&](const char* base, int ks) {
    return *reinterpret_cast<const bf16x8*>(base + (kv_rd0 ^ (ks << 5)));
  };

  // Row statistics of a tile, staged by wave 0 through registers: fetched when
  // the tile's loads are issued, converted to -log2(e)*LSE and written to LDS
  // before the barrier that publishes the tile. Rows past Sq and rows whose
  // LSE is -inf get -inf, so their weights are exactly 0 with no masking.
  float st_l = -INFINITY, st_d = 0.f;
  auto fetch_stats = [&](int q0) {
    const int r = q0 + lane;
    st_l = -INFINITY;
    st_d = 0.f;
    if (r < a.Sq) {
      st_l = a.lse[lbase + r];
      st_d = a.delta[lbase + r];
    }
  };
  auto commit_stats = [&](int st) {
    float* ls = reinterpret_cast<float*>(smem + ST_OFF + 512 * st);
    ls[lane] = neg_lse2(st_l);
    ls[64 + lane] = st_d;
  };
  auto issue = [&](int st, int q0) {
    char* dst = smem + KV_BYTES + 2 * st * TB;
    g.issue(qbase, q0, a.Sq, rs, dst, w8);
    g.issue(dbase, q0, a.Sq, rs, dst + TB, w8);
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md) {
    dk[md] = f32x16{};
    dv[md] = f32x16{};
  }

  if (ntiles > 0) {
    issue(0, qt0 * kTile);
    if (w8 == 0) {
      fetch_stats(qt0 * kTile);
      commit_stats(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const char* kl = smem;
  const char* vl = smem + 2 * TB;
  for (int j = 0; j < ntiles; ++j) {
    const int st = j & 1;
    const char* ql = smem + KV_BYTES + 2 * st * TB;
    const char* dl = ql + TB;
    const float* ls = reinterpret_cast<const float*>(smem + ST_OFF + 512 * st);
    const float* dt = ls + 64;
    const bool more = j + 1 < ntiles;
    if (more) {
      issue(st ^ 1, (qt0 + j + 1) * kTile);
      if (w8 == 0) fetch_stats((qt0 + j + 1) * kTile);
    }
    const int q0 = (qt0 + j) * kTile;
    // S and dP for this group's 32 rows; register r is tile row
    // 32 grp + 16 (r/8) + 8 half + r%8
    f32x16 s = mfma(g.frag(ql, grp, 0), kv_frag(kl, 0), f32x16{});
    f32x16 dp = mfma(g.frag(dl, grp, 0), kv_frag(vl, 0), f32x16{});
#pragma unroll
    for (int ks = 1; ks < D / 16; ++ks) {
      s = mfma(g.frag(ql, grp, ks), kv_frag(kl, ks), s);
      dp = mfma(g.frag(dl, grp, ks), kv_frag(vl, ks), dp);
    }
    if (CAUSAL && q0 + diag < k_last) {  // some (row, key) pairs of the tile are masked
      asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + 32 * grp + 16 * (r >> 3) + 8 * half + (r & 7);
        if (jk > qi + diag) s[r] = s_mask;
      }
    }
    // P and dS (bf16): B operands of k-steps t = 2 grp + t2 (rows 16 t + 8 half + e)
    bf16x8 pf[2], sf[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int row = 32 * grp + 16 * t2 + 8 * half;
      const float4 l0 = *reinterpret_cast<const float4*>(ls + row);
      const float4 l1 = *reinterpret_cast<const float4*>(ls + row + 4);
      const float4 d0 = *reinterpret_cast<const float4*>(dt + row);
      const float4 d1 = *reinterpret_cast<const float4*>(dt + row + 4);
      const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      const float dv8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * t2 + e;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, lv[e]));
        pf[t2][e] = static_cast<__bf16>(p);
        sf[t2][e] = static_cast<__bf16>(p * (dp[r] - dv8[e]));
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the group's 32 rows
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int md = 0; md < D / 32; ++md) {
        dv[md] = mfma(g.tr_frag(dl, md, 2 * grp + t2), pf[t2], dv[md]);
        dk[md] = mfma(g.tr_frag(ql, md, 2 * grp + t2), sf[t2], dk[md]);
      }
    if (more && w8 == 0) commit_stats(st ^ 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // group 1 hands its partial dK, dV to group 0 through LDS (every wave is
  // past its last tile read: the loop ends with a barrier)
  float* xk = reinterpret_cast<float*>(smem);  // [wave][md][r][lane], dK then dV
  constexpr int PER_WAVE = 2 * (D / 32) * 16 * 64;
  if (grp == 1) {
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xk[wave * PER_WAVE + (md * 16 + r) * 64 + lane] = dk[md][r];
        xk[wave * PER_WAVE + ((D / 32 + md) * 16 + r) * 64 + lane] = dv[md][r];
      }
  }
  __syncthreads();
  if (grp == 1 || jk >= len) return;
  // register r of block md is element d = 32 md + 8 (r/4) + 4 half + r%4 of key jk
  const int64_t krow = (static_cast<int64_t>(b) * len + jk) * a.H + h;
  float* ok = ch.dk + krow * D;
  float* ov = ch.dv + krow * D;
  const bool acc = a.accum_dkv != 0;
#pragma unroll
  for (int md = 0; md < D / 32; ++md) {
    // group 1's share of block md, read right before the block is stored: the
    // fence keeps the compiler from hoisting every block's reads, which would
    // hold both groups' sums in registers at once and spill
    asm volatile("" ::: "memory");
    f32x16 xkm, xvm;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      xkm[r] = xk[wave * PER_WAVE + (md * 16 + r) * 64 + lane];
      xvm[r] = xk[wave * PER_WAVE + ((D / 32 + md) * 16 + r) * 64 + lane];
    }
    const f32x16 k_sum = dk[md] + xkm, v_sum = dv[md] + xvm;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * md + 8 * q4 + 4 * half;
      store4(ok + d0, a.scale, k_sum[4 * q4], k_sum[4 * q4 + 1], k_sum[4 * q4 + 2],
             k_sum[4 * q4 + 3], acc);
      store4(ov + d0, 1.f, v_sum[4 * q4], v_sum[4 * q4 + 1], v_sum[4 * q4 + 2],
             v_sum[4 * q4 + 3], acc);
    }
  }
}

template <int D, bool CAUSAL, int G>
__global__ __launch_bounds__(kThreads * G, G == 1 ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[G * 4 * Geo<D>::kTileBytes];
  dq_body<D, CAUSAL, G>(a, smem, static_cast<int>(blockIdx.x));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[8 * Geo<D>::kTileBytes + 1024];
  dkdv_body<D, CAUSAL>(a, smem, static_cast<int>(blockIdx.x));
}

// Both backward kernels in one grid, for grids too small to fill the GPU
// alone: the first a.dq_blocks blocks are two-group dQ blocks (the longest
// work, dispatched first), the rest dK/dV blocks, all of 512 threads. The
// tail of one kind then fills the compute units the other leaves idle.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_fused_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[8 * Geo<D>::kTileBytes + 1024];
  const int blk = static_cast<int>(blockIdx.x);
  if (blk < a.dq_blocks)
    dq_body<D, CAUSAL, 2>(a, smem, blk);
  else
    dkdv_body<D, CAUSAL>(a, smem, blk - a.dq_blocks);
}

// ------------------------------------------------------------- Delta kernel
// Delta[b][h][i] = sum_d dO[b][i][h][d] * O[b][i][h][d] in fp32; 16 lanes per
// row, each reading D/16 consecutive elements.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* o, const T* dout, float* delta,
                                                        int64_t rows, int H, int Sq) {
  constexpr int E = D / 16;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (row >= rows) return;  // whole 16-lane groups leave together
  const T* po = o + row * D + sub * E;
  const T* pd = dout + row * D + sub * E;
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 vecE __attribute__((ext_vector_type(E)));
    const vecE x = *reinterpret_cast<const vecE*>(po);
    const vecE y = *reinterpret_cast<const vecE*>(pd);
#pragma unroll
    for (int e = 0; e < E; ++e) acc = __builtin_fmaf(static_cast<float>(x[e]), static_cast<float>(y[e]), acc);
  } else {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(po + e);
      const float4 y = *reinterpret_cast<const float4*>(pd + e);
      acc = __builtin_fmaf(x.x, y.x, acc);
      acc = __builtin_fmaf(x.y, y.y, acc);
      acc = __builtin_fmaf(x.z, y.z, acc);
      acc = __builtin_fmaf(x.w, y.w, acc);
    }
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (sub == 0) {
    const int h = static_cast<int>(row % H);
    const int64_t bi = row / H;
    const int i = static_cast<int>(bi % Sq);
    const int64_t bb = bi / Sq;
    delta[(bb * H + h) * Sq + i] = acc;
  }
}

template <int D, bool CAUSAL, int G>
hipError_t launch_dq(const BwdArgs& a, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, G>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(kThreads * G), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& args, hipStream_t stream) {
  BwdArgs a = args;
  const int64_t BH = static_cast<int64_t>(a.B) * a.H;
  const int64_t nqt = (a.Sq + kBlk - 1) / kBlk;
  // grids padded to whole rounds of the 8 XCDs (padding blocks exit at once)
  const int64_t dq_blocks = (nqt * BH + 7) / 8 * 8;
  const int64_t kv_blocks = (a.total_kt * BH + 7) / 8 * 8;
  if (a.groups == 2 && kv_blocks > 0 && dq_blocks > 0) {
    a.dq_blocks = static_cast<int32_t>(dq_blocks);
    hipLaunchKernelGGL((bwd_fused_kernel<D, CAUSAL>),
                       dim3(static_cast<uint32_t>(dq_blocks + kv_blocks)), dim3(kKvThreads), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (kv_blocks > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(static_cast<uint32_t>(kv_blocks)),
                       dim3(kKvThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dq_blocks == 0) return hipSuccess;
  return a.groups == 2 ? launch_dq<D, CAUSAL, 2>(a, dq_blocks, stream)
                       : launch_dq<D, CAUSAL, 1>(a, dq_blocks, stream);
}

}  // namespace

// Two-group dQ blocks when the query tiles do not fill the compute units and
// each has at least 4 key tiles to split.
int bwd_dq_groups(int64_t B, int64_t H, int64_t Sq, int64_t key_tiles) {
  const int64_t units = (Sq + kBlk - 1) / kBlk * B * H;
  return units <= device_cus() && key_tiles >= 4 ? 2 : 1;
}

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 64) return causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
  return causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
}

hipError_t launch_bwd_delta(const void* o, const void* dout, float* delta, int64_t B, int64_t H,
                            int64_t Sq, int64_t D, bool bf16, hipStream_t stream) {
  const int64_t rows = B * Sq * H;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((rows + 15) / 16)), block(256);
  const int h = static_cast<int>(H), s = static_cast<int>(Sq);
  if (bf16) {
    if (D == 64)
      hipLaunchKernelGGL((bwd_delta_kernel<__bf16, 64>), grid, block, 0, stream,
                         static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), delta,
                         rows, h, s);
    else
      hipLaunchKernelGGL((bwd_delta_kernel<__bf16, 128>), grid, block, 0, stream,
                         static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), delta,
                         rows, h, s);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((bwd_delta_kernel<float, 64>), grid, block, 0, stream,
                         static_cast<const float*>(o), static_cast<const float*>(dout), delta,
                         rows, h, s);
    else
      hipLaunchKernelGGL((bwd_delta_kernel<float, 128>), grid, block, 0, stream,
                         static_cast<const float*>(o), static_cast<const float*>(dout), delta,
                         rows, h, s);
  }
  return hipGetLastError();
}

}  // namespace cpattn
