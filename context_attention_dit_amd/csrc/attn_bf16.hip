// bf16 flash attention over a list of K/V chunks on CDNA4 matrix cores (gfx950).
//
// What it computes: one Q shard against the K/V chunks it is given, in the
// given order, with the running output and LSE kept in fp32 across chunks
// (Context parallelism guide (diffusers), section Ring Attention; diffusers
// parallel API, ContextParallelConfig: convert_to_fp32). One chunk covering
// the whole sequence is the local attention of a Ulysses rank. The score
// matrix is never stored: K/V are streamed through LDS in tiles and the
// softmax is accumulated online (Ulysses Sequence Parallelism article,
// detailed notes 2).
//
// How it maps to the hardware:
//  * A block is 4 wavefronts; each wave owns 32 query rows, so a block covers
//    128 rows of one (batch, head). K/V tiles of 64 keys are shared by the 4
//    waves through double-buffered LDS, filled by direct memory->LDS loads
//    (buffer_load_dwordx4 ... lds: no staging registers, no LDS store
//    instructions, counted on the vector-memory counter only); one barrier
//    per tile. K runs two tiles ahead of the tile being scored, V one.
//  * The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = a K
//    tile from LDS, B = Q^T held in registers for the whole kernel). In the
//    32x32 accumulator layout lane l holds query column l%32, so every
//    softmax statistic is a per-lane value: the row max and row sum are
//    in-lane reductions plus one exchange between the two half-waves.
//  * K rows sit in LDS with key bits 2 and 3 swapped. With that, the
//    accumulator registers of lane l hold 8 consecutive keys per half-wave,
//    which is exactly the B-operand layout of the next product, so P (rounded
//    to bf16) feeds O^T += V^T P^T without any data movement.
//  * V stays row-major in LDS; its transposed A-operand fragments come from
//    ds_read_b64_tr_b16 (within each 16-lane group, lane i addresses row
//    k0 + i/4, columns d0 + 4(i%4) .. +3, and receives column d0 + i of rows
//    k0 .. k0+3).
//  * LDS rows are unpadded and XOR-swizzled in 16-byte units (K: unit ^ row,
//    so the 8/16 consecutive rows one fragment read touches hit distinct
//    banks; V: 32-byte chunk ^ (row & 3), so the 4 rows of a transposed read
//    do). The global->LDS copy applies the swizzle by choosing each lane's
//    source address.
//  * Softmax in the log2 domain with scale*log2(e) folded into one FMA per
//    score. The exponent offset m is only raised when a tile's row max
//    exceeds it by more than kTau (then O and the row sum are rescaled), so
//    probabilities stay <= 2^kTau and the rescale is rare; the final
//    normalisation uses the same offsets, so the result is unchanged up to
//    rounding.
//  * Non-causal grids map blocks to XCDs so that the tiles of one head stay
//    on one XCD's L2; causal grids launch the heaviest query tiles first.
#include <algorithm>
#include <type_traits>

#include "cp_internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;          // query rows per tile (one group of waves)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // log2 headroom before the exponent offset is raised
constexpr int kMaxSplit = 2;      // key splits per query tile on small grids
constexpr int kTailRows = 32;     // last query tiles at most this short get a launch of their own
constexpr int kTailSplit = 8;     // key splits of that launch
constexpr int kLastSplit = 8;     // key splits of a last round's units

__device__ __forceinline__ int swap_bits23(int k) {
  return k ^ ((((k >> 2) ^ (k >> 3)) & 1) * 12);
}

// Max of x over the two lanes l and l^32 that hold the same query row. The
// swap returns the partner's value in one of its two results and the lane's
// own value or the partner's in the other, so the max of all three is the
// pair's max.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

template <int D>
struct Geo {
  static constexpr int kUPR = D / 8;                      // 16-byte units per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kKMask = kUPR - 1 < 15 ? kUPR - 1 : 15;  // K swizzle row bits
};

// LDS byte layout of one pipeline stage: [K tile][V tile]; two stages.
template <int D>
__device__ __forceinline__ uint32_t k_unit_off(int row, int unit) {
  return row * Geo<D>::kRowBytes + ((unit ^ (row & Geo<D>::kKMask)) << 4);
}
template <int D>
__device__ __forceinline__ uint32_t v_unit_off(int row, int unit) {
  return row * Geo<D>::kRowBytes + ((unit ^ ((row & 3) << 1)) << 4);
}

// Buffer resource over the `bytes` bytes from `base` on (raw, stride 0). A
// load at or past `bytes` is out of range: the hardware fetches nothing and
// returns zeros, which a direct load writes to LDS like any other data.
// `base` must be wave-uniform; it is moved to scalar registers explicitly so
// the descriptor is built there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p >> 32)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(hi << 32 | lo), 0,
                                           __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)),
                                           0x00020000);
}

// buffer_load_dwordx4 ... lds: lane i's 16 bytes at byte offset `voff` of
// `rsrc` land in LDS at l + 16 i (l is wave-uniform). The MUBUF form is
// counted on the vector-memory counter only, so LDS reads issued after it
// keep their own (partial) wait counts.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, char* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(l), 16,
                                           voff, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 read_tr(const char* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// A query tile is kBM = 128 rows of one (batch, head), covered by a group of
// 4 waves of 32 rows each. G = 1: a block is one group. G = 2: a block is two
// groups over the same query tile, group g taking half g of the tile's keys
// with its own LDS slots; the halves are merged through LDS at the end (grids
// with fewer query tiles than CUs: every tile gets a whole CU).
template <int D, bool CAUSAL, bool OUT_BF16, int G>
__global__ __launch_bounds__(256 * G, G == 1 ? 2 : 1) void attn_bf16_kernel(AttnArgs a) {
  constexpr int WPG = 4;               // waves per group
  constexpr int TPG = WPG * 64;        // threads per group
  constexpr int KB = 64;               // keys per tile
  constexpr int NMB = KB / 32;         // 32-key blocks of S per tile
  constexpr int NT = KB / 16;          // 16-key steps of P*V per tile
  constexpr int UPR = Geo<D>::kUPR;
  constexpr int RB = Geo<D>::kRowBytes;
  constexpr int TB = KB * RB;          // one K or V tile
  constexpr int NL = KB * UPR / TPG;   // direct loads per wave per tensor tile
  // Pipeline stages: K and V tiles of stage 0 and 1, one slot per group in each
  // array. Four distinct LDS objects let the compiler see that the direct
  // loads filling one stage never alias reads of the other, so it waits for
  // the copies only where this code says so (at the end of each step).
  __shared__ __attribute__((aligned(1024))) char s_k0[G * TB];
  __shared__ __attribute__((aligned(1024))) char s_k1[G * TB];
  __shared__ __attribute__((aligned(1024))) char s_v0[G * TB];
  __shared__ __attribute__((aligned(1024))) char s_v1[G * TB];

  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int grp = G == 1 ? 0 : uni(tid / TPG);  // key half (G = 2)
  const int wave = uni((tid >> 6) % WPG);        // wave within the group
  const int col = lane & 31, half = lane >> 5;
  const uint32_t gbase = static_cast<uint32_t>(grp * TB);  // the group's slot in each stage array

  // ---- block -> (batch*head, query tile, key split)
  const int nqt = (a.Sq + kBM - 1) / kBM;
  const int BH = a.B * a.H;
  const int nsplit = (CAUSAL || G == 2) ? 1 : a.nsplit;  // key splits across blocks
  const int nitems = nqt * BH * nsplit;
  int bh, qt, sp = 0;
  if (CAUSAL) {
    const int L = blockIdx.x;  // heaviest (last) query tiles first
    qt = nqt - 1 - L / BH;
    bh = L % BH;
  } else {
    const int per_xcd = (nitems + 7) / 8;  // consecutive block ids go to different XCDs
    const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (L >= nitems) return;
    const int unit = L / nsplit;
    sp = L - unit * nsplit;
    bh = unit / nqt;
    qt = unit % nqt;
  }
  // (uniform: kept in scalar registers for the tile addresses)
  const int b = uni(bh / a.H);
  const int h = uni(bh - b * a.H);
  const int irow = qt * kBM + wave * 32 + col;  // this lane's query row
  const int q_first = qt * kBM;
  const int q_last = min(q_first + kBM - 1, a.Sq - 1);

  // ---- Q^T fragments (B operand), resident for the whole kernel. A negative
  //      scale is folded into Q (bf16 negation is exact).
  const float sl2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  bf16x8 qf[D / 16];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<int64_t>(b) * a.Sq + min(irow, a.Sq - 1)) * a.H + h) * D +
                       8 * half;
    const uint32_t flip = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      w ^= flip;
      if (irow >= a.Sq) w = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- direct-load geometry: this lane fills LDS slot s = wave*NL*64 + n*64 + lane
  //      of each tensor tile; slot s is (row s/UPR, swizzled unit s%UPR). The
  //      lane's source offsets (bytes from the tile's first key) are fixed.
  const int rs = a.H * D;  // elements between consecutive keys (host checks 64*rs < 2^31)
  uint32_t k_src[NL], v_src[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int s = (wave * NL + n) * 64 + lane;
    const int row = s / UPR, pu = s % UPR;
    const int k_key = swap_bits23(row), k_unit = pu ^ (row & Geo<D>::kKMask);
    const int v_unit = pu ^ ((row & 3) << 1);
    k_src[n] = 2u * static_cast<uint32_t>(k_key * rs + k_unit * 8);
    v_src[n] = 2u * static_cast<uint32_t>(row * rs + v_unit * 8);
  }

  // Chunk descriptors are read with a provably uniform index, so they come
  // in through scalar loads.
  auto keys_of = [&](int c) {
    c = uni(c);
    int n = a.chunks[c].len;
    if (CAUSAL) n = max(0, min(n, q_last + a.chunks[c].delta + 1));
    return n;
  };
  // A cursor carries its chunk's descriptor (visible keys nk, stored keys len,
  // position offset delta) and the addresses of its K and V tile for this
  // (batch, head), set when it enters the chunk and stepped by one tile
  // stride after that, so the pipeline steps issue no scalar loads and no
  // 64-bit address arithmetic of their own.
  struct Cur {
    int c, kt;
    int nk, len, delta;
    const char* tk;
    const char* tv;
  };
  const int64_t tile_bytes = 2 * static_cast<int64_t>(KB) * rs;
  auto enter = [&](Cur& x) {
    const int c = uni(x.c);
    if (c < a.nchunks) {  // (a cursor past the list is never used)
      x.len = a.chunks[c].len;
      x.delta = a.chunks[c].delta;
      x.nk = CAUSAL ? max(0, min(x.len, q_last + x.delta + 1)) : x.len;
      const int64_t off =
          2 * ((static_cast<int64_t>(b) * x.len + uni(x.kt) * KB) * rs + h * D);
      x.tk = reinterpret_cast<const char*>(a.chunks[c].k) + off;
      x.tv = reinterpret_cast<const char*>(a.chunks[c].v) + off;
    }
  };
  auto next_of = [&](Cur x) {
    x.kt = uni(x.kt) + 1;
    if (x.kt * KB >= x.nk) {
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
  // Direct loads of one K or V tile into `dst`: a uniform base address plus
  // the lane's fixed byte offset. The buffer's range ends after the tile's
  // last valid key, so rows past it (a chunk's ragged end, keys beyond the
  // causal limit) arrive as zeros; their scores are masked, so they add
  // nothing.
  auto issue = [&](char* dst, const Cur& x, bool is_v) {
    const int n_valid = max(0, min(x.nk - uni(x.kt) * KB, KB));  // (0: nothing is fetched)
    const char* base = is_v ? x.tv : x.tk;
    char* l = dst + gbase + wave * NL * 1024;
    const __amdgpu_buffer_rsrc_t rsrc =
        tile_rsrc(base, static_cast<uint32_t>(n_valid) * static_cast<uint32_t>(2 * rs));
#pragma unroll
    for (int n = 0; n < NL; ++n) lds_load16(rsrc, is_v ? v_src[n] : k_src[n], l + n * 1024);
  };

  // ---- fragment read addresses (byte offsets within a tile)
  // K: row col (+32 for the second block), unit 2*ks + half, swizzled with row bits
  // (the group's LDS base is folded into these per-lane offsets, so every
  // slot offset below stays an immediate)
  uint32_t k_rd[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) k_rd[ks] = gbase + k_unit_off<D>(col, 2 * ks + half);
  // V^T: 16-lane group g, lane j -> row 8*(g/2) + j/4, element column 16*(g%2) + 4*(j%4)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row = 8 * (g16 >> 1) + (j16 >> 2);
  const int v_el = 16 * (g16 & 1) + 4 * (j16 & 3);
  uint32_t v_rd[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md)
    v_rd[md] = gbase + v_unit_off<D>(v_row, (32 * md + v_el) >> 3) + ((v_el & 4) ? 8 : 0);

  // S^T = K Q^T for the KB keys of the K tile in stage array `kl`: sacc[mb]
  // holds keys 32 mb .. +31 against the wave's 32 queries
  auto qk = [&](const char* kl, f32x16* sacc) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + k_rd[ks] + mb * 32 * RB);
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks],
                                                           ks == 0 ? f32x16{} : sacc[mb], 0, 0, 0);
      }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY;  // exponent offset, log2 domain
  float l_run = 0.f;        // this lane's share of the row sum

  // this block's share of the query tile's tiles, in chunk order
  Cur cur0{0, 0, 0, 0, 0, nullptr, nullptr};
  int left, steps;
  {
    int total = 0;
    for (int cc = 0; cc < a.nchunks; ++cc) total += (keys_of(cc) + KB - 1) / KB;
    const int nparts = G == 2 ? 2 : nsplit, part = G == 2 ? grp : sp;
    const int t_begin = static_cast<int>(static_cast<int64_t>(total) * part / nparts);
    const int t_end = static_cast<int>(static_cast<int64_t>(total) * (part + 1) / nparts);
    left = uni(t_end - t_begin);
    // both groups step together (block-wide barriers): the second half is the longer
    steps = uni(G == 2 ? total - total / 2 : left);
    int skip = t_begin;
    while (cur0.c < a.nchunks) {
      const int nt = (keys_of(cur0.c) + KB - 1) / KB;
      if (skip < nt) break;
      skip -= nt;
      ++cur0.c;
    }
    cur0.kt = skip;
    enter(cur0);
  }

  // One pipeline step for tile j (cursor cur0; cur1/cur2 are tiles j+1/j+2):
  // prefetch K of j+2 and V of j+1, then S for tile j+1 on the matrix cores
  // while the softmax of tile j runs, then O += P V for tile j. Tile j's K
  // and V sit in the stage-PAR arrays; PAR = j & 1 is a compile-time constant
  // (the loop is unrolled by two), so every LDS offset is an immediate.
  Cur cur1 = cur0, cur2 = cur0;
  auto step = [&](auto par_tag, int j, f32x16* s_cur, f32x16* s_next) {
    constexpr int PAR = decltype(par_tag)::value;
    if (G == 1 || j < left) {  // (a group out of tiles still joins the barrier below)
    // cursors: cur0 = tile j, cur1 = j+1, cur2 = j+2 (the prologue set them for j = 0)
    if (j > 0) {
      cur0 = cur1;
      cur1 = cur2;
      if (j + 2 < left) cur2 = next_of(cur2);
    }
    if (j + 2 < left) issue(PAR == 0 ? s_k0 : s_k1, cur2, false);
    if (j + 1 < left) issue(PAR == 0 ? s_v1 : s_v0, cur1, true);
    const int len = cur0.len;
    const int delta = cur0.delta;
    const int key0 = uni(cur0.kt) * KB;

    // softmax of tile j (lane = query column; register r of s_cur[mb] is key
    // key0 + 32*mb + 16*(r/8) + 8*half + r%8)
    const bool masked = (key0 + KB > len) || (CAUSAL && key0 + KB - 1 > q_first + delta);
    if (masked) {
      asm volatile("" ::: "memory");  // keeps this a real (uniform) branch
      // visible iff the key index relative to key0 is < lim
      int lim = len - key0;
      if (CAUSAL) lim = min(lim, irow + delta - key0 + 1);
      lim -= 8 * half;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mb + 16 * (r >> 3) + (r & 7) >= lim) s_cur[mb][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s_cur[0][0], s_cur[0][1]), s_cur[0][2]);
#pragma unroll
    for (int r = 3; r < 31; r += 2)
      mx = fmaxf(fmaxf(mx, s_cur[r >> 4][r & 15]), s_cur[(r + 1) >> 4][(r + 1) & 15]);
    mx = fmaxf(mx, s_cur[1][15]);
    mx = pair_max(mx) * sl2;
    if (__ballot(mx > m_run + kTau)) {
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < D / 32; ++md) oacc[md] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;

    // S of tile j+1 on the matrix cores while the exponentials run (for the
    // last tile this reads a stale slot and the result is never used)
    qk(PAR == 0 ? s_k1 : s_k0, s_next);
    bf16x8 pf[NT];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(
            __builtin_fmaf(s_cur[t >> 1][(t & 1) * 8 + e], sl2, neg_m));
        psum += p;
        pf[t][e] = static_cast<__bf16>(p);
      }
    l_run += psum;

    // O^T += V^T P^T for tile j
    const char* vl = PAR == 0 ? s_v0 : s_v1;
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const char* vr = vl + v_rd[md] + 16 * t * RB;
        const bf16x4 lo = read_tr(vr);
        const bf16x4 hi = read_tr(vr + 4 * RB);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], oacc[md], 0, 0, 0);
      }
    }
    // Instruction interleave for the block above: S of tile j+1 (one MFMA
    // per K-fragment read, reads kRA fragments ahead) with the exponentials
    // of tile j in between; the transposed V reads of the first kVA V
    // fragments go out under the last S MFMAs, then each P*V MFMA is
    // followed by the two reads of the fragment kVA later, so no MFMA waits
    // on a fresh LDS read.
    constexpr int kRA = 4, kVA = 4, NKF = NMB * (D / 16), NVF = NT * (D / 32);
    __builtin_amdgcn_sched_group_barrier(0x100, kRA, 0);    // LDS reads run ahead
#pragma unroll
    for (int k = 0; k < NKF; ++k) {                         // S MFMAs of qk()
      // (the last kVA groups also take the first V fragments' reads)
      if (k >= NKF - kVA)
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);    // VALU
    }
#pragma unroll
    for (int k = 0; k < NVF; ++k) {                         // P*V MFMAs
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  f32x16 s_a[NMB], s_b[NMB];
  if (steps > 0) {
    if (G == 1 || left > 0) {
      issue(s_k0, cur0, false);
      issue(s_v0, cur0, true);
      if (left > 1) {
        cur1 = next_of(cur0);
        issue(s_k1, cur1, false);
      }
      if (left > 2) cur2 = next_of(cur1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (G == 1 || left > 0) qk(s_k0, s_a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int j = 0; j < steps; j += 2) {
    step(std::integral_constant<int, 0>{}, j, s_a, s_b);
    if (j + 1 >= steps) break;
    step(std::integral_constant<int, 1>{}, j + 1, s_b, s_a);
  }

  // ---- epilogue: merge the two key halves (G = 2), normalise, write O and LSE
  float l_tot = l_run + __shfl_xor(l_run, 32);
  if (G == 2) {
    // group 1 hands its running max, row sum and unnormalised O to group 0
    // through LDS (every wave is past its last tile read after this barrier).
    // O blocks md < D/64 go to s_v0, the rest to s_v1: [wave][md % (D/64)][r][lane]
    __syncthreads();
    constexpr int HM = D / 64;
    auto xo = [&](int md, int r) -> float& {
      float* base = reinterpret_cast<float*>(md < HM ? s_v0 : s_v1);
      return base[((wave * HM + md % HM) * 16 + r) * 64 + lane];
    };
    float* xs = reinterpret_cast<float*>(s_k0);  // [wave][m, l][lane]
    if (grp == 1) {
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo(md, r) = oacc[md][r];
      xs[(wave * 2) * 64 + lane] = m_run;
      xs[(wave * 2 + 1) * 64 + lane] = l_tot;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xs[(wave * 2) * 64 + lane], l1 = xs[(wave * 2 + 1) * 64 + lane];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    l_tot = a0 * l_tot + a1 * l1;
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] = a0 * oacc[md][r] + a1 * xo(md, r);
    m_run = mm;
  }
  const int i = irow;
  if (i >= a.Sq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = ((static_cast<int64_t>(b) * a.Sq + i) * a.H + h) * D;
  const int64_t lrow = (static_cast<int64_t>(b) * a.H + h) * a.Sq + i;
  const float lse_val = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (nsplit > 1) {  // fp32 partial of split sp
    float* po = a.part_o + static_cast<int64_t>(sp) * a.B * a.Sq * a.H * D + orow;
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(po + 32 * md + 8 * g + 4 * half) =
            make_float4(oacc[md][4 * g] * inv, oacc[md][4 * g + 1] * inv,
                        oacc[md][4 * g + 2] * inv, oacc[md][4 * g + 3] * inv);
    if (half == 0) a.part_lse[static_cast<int64_t>(sp) * a.B * a.H * a.Sq + lrow] = lse_val;
    return;
  }
#pragma unroll
  for (int md = 0; md < D / 32; ++md) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * md + 8 * g + 4 * half;
      const float x0 = oacc[md][4 * g] * inv, x1 = oacc[md][4 * g + 1] * inv;
      const float x2 = oacc[md][4 * g + 2] * inv, x3 = oacc[md][4 * g + 3] * inv;
      if (OUT_BF16) {
        bf16x4 r;
        r[0] = static_cast<__bf16>(x0);
        r[1] = static_cast<__bf16>(x1);
        r[2] = static_cast<__bf16>(x2);
        r[3] = static_cast<__bf16>(x3);
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o) + orow + d0) = r;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.o) + orow + d0) =
            make_float4(x0, x1, x2, x3);
      }
    }
  }
  if (half == 0) {
    const int lstr = a.lse_stride > 0 ? a.lse_stride : a.Sq;
    a.lse[(static_cast<int64_t>(b) * a.H + h) * lstr + i] = lse_val;
  }
}

// ---- Ping-pong kernel for one K/V chunk (a Ulysses rank's local attention,
// a single ring hop). A block is 8 waves over 256 query rows: two groups of
// 4 waves, 128 rows each, that share every K/V tile in LDS. Each wave
// alternates two phases per key tile: S(j), the masking and softmax of tile
// j (vector ALU only), and M(j), O += P(j) V(j) and S(j+1) = K(j+1) Q^T
// (matrix cores and LDS reads only). Group 1 runs half a step behind
// group 0, and waves w and w+4 share a SIMD, so on every SIMD one wave is in
// its softmax while the other keeps the matrix cores busy. A block barrier
// separates the half-steps. The arithmetic per row is that of
// attn_bf16_kernel (same products, same order), so results are identical.
template <int D, bool CAUSAL, bool OUT_BF16, bool MULTI, bool SPLIT = false, bool VT = false>
__global__ __launch_bounds__(512, 1) void attn_pp_kernel(AttnArgs a) {
  // VT: V arrives key-contiguous in 64-key tiles, [B][H][tiles][D][64] (one
  // chunk, no key splits): each V tile is one contiguous 16 KB block
  static_assert(!VT || (D == 128 && !MULTI && !SPLIT), "key-contiguous V: one chunk at D = 128");
  static_assert(!SPLIT || (!CAUSAL && !MULTI), "key splits: one chunk, non-causal");
  constexpr int NW = 8;
  constexpr int KB = 64;
  constexpr int NMB = KB / 32;
  constexpr int NT = KB / 16;
  constexpr int UPR = Geo<D>::kUPR;
  constexpr int RB = Geo<D>::kRowBytes;
  constexpr int TB = KB * RB;
  constexpr int NL = KB * UPR / (NW * 64);   // direct loads per wave per tile
  constexpr int kTM = 256;                   // query rows per block
  __shared__ __attribute__((aligned(1024))) char s_k0[TB];
  __shared__ __attribute__((aligned(1024))) char s_k1[TB];
  __shared__ __attribute__((aligned(1024))) char s_v0[TB];
  __shared__ __attribute__((aligned(1024))) char s_v1[TB];

  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto uni_ptr = [](const char* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w8 = uni(tid >> 6);
  const int grp = uni(w8 >> 2);
  const int wave = uni(w8 & 3);
  const int col = lane & 31, half = lane >> 5;

  // ---- block -> (batch*head, 256-row query tile), as in attn_bf16_kernel
  const int nqt = (a.Sq + kTM - 1) / kTM;
  const int BH = a.B * a.H;
  const int nitems = nqt * BH;
  int bh, qt;
  // key splits of each unit (one chunk, non-causal): block L takes split
  // sp = L mod ns of the launch's unit L / ns
  const int ns = SPLIT ? max(1, a.pp_split) : 1;
  int nu = nitems, lu = 0, sp = 0;
  if (CAUSAL) {
    const int L = blockIdx.x;  // heaviest (last) query tiles first
    qt = nqt - 1 - L / BH;
    bh = L % BH;
  } else {
    nu = a.units > 0 ? a.units : nitems;  // this launch's units
    const int per_xcd = (nu * ns + 7) / 8;  // one head's tiles stay on one XCD
    const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (L >= nu * ns) return;
    lu = L / ns;
    sp = L - lu * ns;
    const int u = a.unit0 + lu;
    bh = u / nqt;
    qt = u % nqt;
  }
  const int b = uni(bh / a.H);
  const int h = uni(bh - b * a.H);
  const int blk_first = qt * kTM;
  const int blk_last = min(blk_first + kTM - 1, a.Sq - 1);
  const int q_first = blk_first + grp * 128;          // the group's first row
  const int irow = q_first + wave * 32 + col;

  const float sl2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  bf16x8 qf[D / 16];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<int64_t>(b) * a.Sq + min(irow, a.Sq - 1)) * a.H + h) * D +
                       8 * half;
    const uint32_t flip = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      w ^= flip;
      if (irow >= a.Sq) w = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int rs = a.H * D;
  uint32_t k_src[NL], v_src[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int s = (w8 * NL + n) * 64 + lane;
    const int row = s / UPR, pu = s % UPR;
    const int k_key = swap_bits23(row), k_unit = pu ^ (row & Geo<D>::kKMask);
    const int v_unit = pu ^ ((row & 3) << 1);
    k_src[n] = 2u * static_cast<uint32_t>(k_key * rs + k_unit * 8);
    v_src[n] = 2u * static_cast<uint32_t>(row * rs + v_unit * 8);
    if constexpr (VT) {
      // V^T tile: D rows of 64 keys (128 bytes, 8 units), unit u of row d at
      // u ^ ((d >> 1) & 7): the 16 rows of one 16-lane read phase (two rows
      // per 256-byte bank line) then hit distinct banks
      const int d = s >> 3, vu = (s & 7) ^ ((d >> 1) & 7);
      v_src[n] = 128u * d + 16u * vu;
    }
  }

  // One chunk: its keys this block can see, and its K/V rows of this (b, h);
  // tile j starts j tile strides into them.
  // (a key split sees the tiles [t0, t1) of the chunk: len counts its keys)
  const int len_c = a.chunks[0].len;
  int t0 = 0, len = len_c;
  if (ns > 1) {
    const int nt = (len_c + KB - 1) / KB;
    t0 = nt * sp / ns;
    len = min(len_c, nt * (sp + 1) / ns * KB) - t0 * KB;
  }
  const int delta = a.chunks[0].delta;
  const int nk = CAUSAL ? max(0, min(len, blk_last + delta + 1)) : len;
  const int64_t tile_bytes = 2 * static_cast<int64_t>(KB) * rs;
  const char* kbase0 = reinterpret_cast<const char*>(a.chunks[0].k) +
                       2 * (static_cast<int64_t>(b) * len_c * rs + h * D) + t0 * tile_bytes;
  const char* vbase0 = reinterpret_cast<const char*>(a.chunks[0].v) +
                       2 * (static_cast<int64_t>(b) * len_c * rs + h * D) + t0 * tile_bytes;
  // VT: this (b, h)'s V tiles, [tiles][D][64]; tile j is the j-th 16 KB block
  const char* vt_base = reinterpret_cast<const char*>(a.chunks[0].v) +
                        2 * ((static_cast<int64_t>(b) * a.H + h) * ((len_c + KB - 1) / KB)) * D * KB;
  auto rows_at = [&](int t_abs) { return max(0, min(nk - t_abs * KB, KB)); };
  // A chunk list (MULTI): the block's key tiles are every chunk's keys that a
  // row of the block can see, in chunk order. Each wave walks them with two
  // cursors, one for the copies (K two tiles ahead; a tile's V source is kept
  // from its K copy for the V copy one step later) and one for the masking
  // of its S phases; their fields are wave-uniform, in scalar registers.
  auto keys_of = [&](int c) {
    c = uni(c);
    int nkc = a.chunks[c].len;
    if (CAUSAL) nkc = max(0, min(nkc, blk_last + a.chunks[c].delta + 1));
    return nkc;
  };
  struct Cur {
    int c, kt;
    int nk, len, delta;
    const char* tk;
    const char* tv;
  };
  auto enter = [&](Cur& x, bool ptrs) {
    const int c = uni(x.c);
    if (c < a.nchunks) {
      x.len = uni(a.chunks[c].len);
      x.delta = uni(a.chunks[c].delta);
      x.nk = uni(CAUSAL ? max(0, min(x.len, blk_last + x.delta + 1)) : x.len);
      if (ptrs) {
        const int64_t off =
            2 * ((static_cast<int64_t>(b) * x.len + uni(x.kt) * KB) * rs + h * D);
        x.tk = uni_ptr(reinterpret_cast<const char*>(a.chunks[c].k) + off);
        x.tv = uni_ptr(reinterpret_cast<const char*>(a.chunks[c].v) + off);
      }
    }
  };
  auto next_of = [&](Cur x, bool ptrs) {
    x.kt = uni(x.kt) + 1;
    if (x.kt * KB >= x.nk) {
      x.kt = 0;
      x.c = uni(x.c) + 1;
      while (x.c < a.nchunks && keys_of(x.c) == 0) ++x.c;
      enter(x, ptrs);
    } else if (ptrs) {
      x.tk = uni_ptr(x.tk + tile_bytes);
      x.tv = uni_ptr(x.tv + tile_bytes);
    }
    return x;
  };
  auto rows_of = [&](const Cur& x) { return uni(max(0, min(x.nk - uni(x.kt) * KB, KB))); };
  // copy one tile (n_valid rows of it from base, zeros for the rest) into dst
  auto issue = [&](char* dst, const char* base, int n_valid, bool is_v) {
    char* l = dst + w8 * NL * 1024;
    // (a V^T tile is a whole 16 KB block: its padding keys past the chunk are
    // finite and get weight 0)
    const __amdgpu_buffer_rsrc_t rsrc =
        VT && is_v ? tile_rsrc(base, 2u * D * KB)
                   : tile_rsrc(base, static_cast<uint32_t>(n_valid) * static_cast<uint32_t>(2 * rs));
#pragma unroll
    for (int n = 0; n < NL; ++n) lds_load16(rsrc, is_v ? v_src[n] : k_src[n], l + n * 1024);
  };

  uint32_t k_rd[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) k_rd[ks] = k_unit_off<D>(col, 2 * ks + half);
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row = 8 * (g16 >> 1) + (j16 >> 2);
  const int v_el = 16 * (g16 & 1) + 4 * (j16 & 3);
  uint32_t v_rd[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md)
    v_rd[md] = v_unit_off<D>(v_row, (32 * md + v_el) >> 3) + ((v_el & 4) ? 8 : 0);
  // VT: the A fragment of k-step t is row d = 32 md + col, keys 16 t + 8 half .. +7
  uint32_t vt_rd[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) vt_rd[t] = 128u * col + 16u * ((2 * t + half) ^ ((col >> 1) & 7));

  auto qk = [&](const char* kl, f32x16* sacc) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + k_rd[ks] + mb * 32 * RB);
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks],
                                                           ks == 0 ? f32x16{} : sacc[mb], 0, 0, 0);
      }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  int n = 0;  // key tiles of this block
  Cur ck{0, 0, 0, 0, 0, nullptr, nullptr};  // MULTI: the next K copy
  if constexpr (MULTI) {
    for (int cc = 0; cc < a.nchunks; ++cc) n += (keys_of(cc) + KB - 1) / KB;
    while (ck.c < a.nchunks && keys_of(ck.c) == 0) ++ck.c;
    enter(ck, true);
  } else {
    n = (nk + KB - 1) / KB;
  }
  n = uni(n);
  Cur mc = ck;                 // MULTI: the tile of this wave's next S phase
  const char* vb_p = nullptr;  // MULTI: V source and rows of the next V copy
  int vb_n = 0;

  // Two phases per tile and wave. S(j): masking and softmax of tile j (VALU
  // only). M(j): O += P(j) V(j) and S(j+1) = K(j+1) Q^T (matrix cores and LDS
  // reads only). Group 1 runs half a step behind group 0, so on every SIMD one
  // wave is in an S phase while the other is in an M phase.
  f32x16 sacc[NMB];
  bf16x8 pf[NT];
  auto phase_s = [&](int j) {
    // bounds relative to the tile's first key: rl = len - key0, rd = delta - key0
    int rl, rd;
    if constexpr (MULTI) {
      const int key0 = uni(mc.kt) * KB;
      rl = uni(mc.len - key0);
      rd = uni(mc.delta - key0);
    } else {
      rl = len - j * KB;
      rd = delta - j * KB;
    }
    const bool masked = (rl < KB) || (CAUSAL && rd < KB - 1 - q_first);
    if (masked) {
      asm volatile("" ::: "memory");
      int lim = rl;
      if (CAUSAL) lim = min(lim, irow + rd + 1);
      lim -= 8 * half;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mb + 16 * (r >> 3) + (r & 7) >= lim) sacc[mb][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), sacc[0][2]);
#pragma unroll
    for (int r = 3; r < 31; r += 2)
      mx = fmaxf(fmaxf(mx, sacc[r >> 4][r & 15]), sacc[(r + 1) >> 4][(r + 1) & 15]);
    mx = fmaxf(mx, sacc[1][15]);
    mx = pair_max(mx) * sl2;
    if (__ballot(mx > m_run + kTau)) {
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < D / 32; ++md) oacc[md] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(
            __builtin_fmaf(sacc[t >> 1][(t & 1) * 8 + e], sl2, neg_m));
        psum += p;
        pf[t][e] = static_cast<__bf16>(p);
      }
    l_run += psum;
    if constexpr (MULTI) mc = next_of(mc, false);
  };
  auto phase_m = [&](const char* kl, const char* vl) {
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 vf;
        if constexpr (VT) {
          vf = *reinterpret_cast<const bf16x8*>(vl + vt_rd[t] + md * 32 * 128);
        } else {
          const char* vr = vl + v_rd[md] + 16 * t * RB;
          const bf16x4 lo = read_tr(vr);
          const bf16x4 hi = read_tr(vr + 4 * RB);
          vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], oacc[md], 0, 0, 0);
      }
    }
    qk(kl, sacc);
    // one MFMA per group with its fragment reads two groups ahead
    constexpr int NVF = NT * (D / 32), NKF = NMB * (D / 16);
    if constexpr (VT) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int k = 0; k < NVF; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < NVF; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k < NVF - 2)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
#pragma unroll
    for (int k = 0; k < NKF; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // End of a half-step: copies issued in this half-step may stay in flight,
  // older ones have landed, this wave's LDS reads are done; then the block
  // barrier. (A plain s_barrier: the workgroup fence of __syncthreads would
  // also wait for the copies still in flight.)
  auto sync = [&](bool issued_now) {
    if (issued_now) {
      if (NL == 2) __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) expcnt(7) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0x0072);
    } else {
      __builtin_amdgcn_s_waitcnt(0x0070);
    }
    asm volatile("s_barrier" ::: "memory");
  };

  // prologue: K(0), K(1), V(0); S(0) for both groups, group 0's softmax of tile 0
  if (n > 0) {
    if constexpr (MULTI) {
      const int nv0 = rows_of(ck);
      issue(s_k0, ck.tk, nv0, false);
      issue(s_v0, ck.tv, nv0, true);
      if (n > 1) {
        ck = next_of(ck, true);
        vb_n = rows_of(ck);
        vb_p = ck.tv;
        issue(s_k1, ck.tk, vb_n, false);
        if (n > 2) ck = next_of(ck, true);
      }
    } else {
      issue(s_k0, kbase0, rows_at(0), false);
      issue(s_v0, VT ? vt_base : vbase0, rows_at(0), true);
      if (n > 1) issue(s_k1, kbase0 + tile_bytes, rows_at(1), false);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n > 0) qk(s_k0, sacc);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (grp == 0 && n > 0) phase_s(0);

  // half-step hs = 2j: copies K(j+2) and V(j+1); group 0 M(j), group 1 S(j).
  // hs = 2j+1: group 0 S(j+1), group 1 M(j). K(j+1) sits in stage (j+1)&1,
  // V(j) in stage j&1; Q = hs % 4 fixes them at compile time.
  auto copies = [&](auto q_tag, int hs) {
    constexpr int Q = decltype(q_tag)::value;
    const int j = hs >> 1;
    bool any = false;
    if (Q % 2 == 0) {
      if constexpr (MULTI) {
        const char* vp = vb_p;
        const int vn = vb_n;
        if (j + 2 < n) {
          vb_n = rows_of(ck);
          vb_p = ck.tv;
          issue(Q == 0 ? s_k0 : s_k1, ck.tk, vb_n, false);
          if (j + 3 < n) ck = next_of(ck, true);
          any = true;
        }
        if (j + 1 < n) { issue(Q == 0 ? s_v1 : s_v0, vp, vn, true); any = true; }
      } else {
        if (j + 2 < n) {
          issue(Q == 0 ? s_k0 : s_k1, kbase0 + (j + 2) * tile_bytes, rows_at(j + 2), false);
          any = true;
        }
        if (j + 1 < n) {
          issue(Q == 0 ? s_v1 : s_v0,
                VT ? vt_base + 2 * D * KB * (j + 1) : vbase0 + (j + 1) * tile_bytes, rows_at(j + 1),
                true);
          any = true;
        }
      }
    }
    return any;
  };
  auto hs_g0 = [&](auto q_tag, int hs) {
    constexpr int Q = decltype(q_tag)::value;
    const int j = hs >> 1;
    const bool issued = copies(q_tag, hs);
    if (Q == 0 && j < n) phase_m(s_k1, s_v0);
    if (Q == 1 && j + 1 < n) phase_s(j + 1);
    if (Q == 2 && j < n) phase_m(s_k0, s_v1);
    if (Q == 3 && j + 1 < n) phase_s(j + 1);
    sync(issued);
  };
  auto hs_g1 = [&](auto q_tag, int hs) {
    constexpr int Q = decltype(q_tag)::value;
    const int j = hs >> 1;
    const bool issued = copies(q_tag, hs);
    if (Q == 0 && j < n) phase_s(j);
    if (Q == 1 && j < n) phase_m(s_k1, s_v0);
    if (Q == 2 && j < n) phase_s(j);
    if (Q == 3 && j < n) phase_m(s_k0, s_v1);
    sync(issued);
  };
  const int nh = 2 * n;
  if (grp == 0) {
    for (int hs = 0; hs < nh; hs += 4) {
      hs_g0(std::integral_constant<int, 0>{}, hs);
      hs_g0(std::integral_constant<int, 1>{}, hs + 1);
      if (hs + 2 >= nh) break;
      hs_g0(std::integral_constant<int, 2>{}, hs + 2);
      hs_g0(std::integral_constant<int, 3>{}, hs + 3);
    }
  } else {
    for (int hs = 0; hs < nh; hs += 4) {
      hs_g1(std::integral_constant<int, 0>{}, hs);
      hs_g1(std::integral_constant<int, 1>{}, hs + 1);
      if (hs + 2 >= nh) break;
      hs_g1(std::integral_constant<int, 2>{}, hs + 2);
      hs_g1(std::integral_constant<int, 3>{}, hs + 3);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 32);
  const int i = irow;
  if (i >= a.Sq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = ((static_cast<int64_t>(b) * a.Sq + i) * a.H + h) * D;
  const float lse_val = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if constexpr (SPLIT) {
    if (ns > 1) {  // normalised fp32 partial: [split][unit in launch][row in unit]
      const int64_t prow = (static_cast<int64_t>(sp) * nu + lu) * kTM + (i - blk_first);
      float* dst = a.part_o + prow * D;
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(dst + 32 * md + 8 * g + 4 * half) =
              make_float4(oacc[md][4 * g] * inv, oacc[md][4 * g + 1] * inv,
                          oacc[md][4 * g + 2] * inv, oacc[md][4 * g + 3] * inv);
      if (half == 0) a.part_lse[prow] = lse_val;
      return;
    }
  }
#pragma unroll
  for (int md = 0; md < D / 32; ++md) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * md + 8 * g + 4 * half;
      const float x0 = oacc[md][4 * g] * inv, x1 = oacc[md][4 * g + 1] * inv;
      const float x2 = oacc[md][4 * g + 2] * inv, x3 = oacc[md][4 * g + 3] * inv;
      if (OUT_BF16) {
        bf16x4 r;
        r[0] = static_cast<__bf16>(x0);
        r[1] = static_cast<__bf16>(x1);
        r[2] = static_cast<__bf16>(x2);
        r[3] = static_cast<__bf16>(x3);
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o) + orow + d0) = r;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.o) + orow + d0) =
            make_float4(x0, x1, x2, x3);
      }
    }
  }
  if (half == 0) {
    const int lstr = a.lse_stride > 0 ? a.lse_stride : a.Sq;
    a.lse[(static_cast<int64_t>(b) * a.H + h) * lstr + i] = lse_val;
  }
}

// ---- Two-group ping-pong kernel for small grids (no more query tiles than
// CUs, at least four key tiles), head dim 128. A block is 8 waves over one
// 128-row query tile, as in the two-group case of attn_bf16_kernel: group g
// takes the g-th half of the tile's key tiles (in chunk order) through LDS
// stages of its own, and the two halves are merged through LDS at the end.
// Each wave alternates the S and M phases of attn_pp_kernel with group 1
// half a step behind group 0, so the two waves on a SIMD are always in
// opposite phases. Same products in the same order as the two-group case of
// attn_bf16_kernel, so the results are identical. (At head dim 64 the
// softmax outweighs the matrix work and that kernel is faster.)
template <int D, bool CAUSAL, bool OUT_BF16, bool VT = false>
__global__ __launch_bounds__(512, 1) void attn_g2pp_kernel(AttnArgs a) {
  // VT: V arrives key-contiguous in 64-key tiles, [B][H][tiles][D][64] (one
  // chunk): each V tile is one contiguous 16 KB block
  static_assert(!VT || D == 128, "key-contiguous V: D = 128");
  constexpr int WPG = 4;
  constexpr int TPG = WPG * 64;
  constexpr int KB = 64;
  constexpr int NMB = KB / 32;
  constexpr int NT = KB / 16;
  constexpr int UPR = Geo<D>::kUPR;
  constexpr int RB = Geo<D>::kRowBytes;
  constexpr int TB = KB * RB;
  constexpr int NL = KB * UPR / TPG;   // direct loads per wave per tile (its group's)
  __shared__ __attribute__((aligned(1024))) char s_k0[2 * TB];
  __shared__ __attribute__((aligned(1024))) char s_k1[2 * TB];
  __shared__ __attribute__((aligned(1024))) char s_v0[2 * TB];
  __shared__ __attribute__((aligned(1024))) char s_v1[2 * TB];

  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto uni_ptr = [](const char* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int grp = uni(tid / TPG);
  const int wave = uni((tid >> 6) % WPG);
  const int col = lane & 31, half = lane >> 5;
  const uint32_t gbase = static_cast<uint32_t>(grp * TB);

  const int nqt = (a.Sq + kBM - 1) / kBM;
  const int BH = a.B * a.H;
  const int nitems = nqt * BH;
  int bh, qt;
  if (CAUSAL) {
    const int L = blockIdx.x;
    qt = nqt - 1 - L / BH;
    bh = L % BH;
  } else {
    const int nu = a.units > 0 ? a.units : nitems;  // this launch's units
    const int per_xcd = (nu + 7) / 8;
    const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (L >= nu) return;
    const int u = a.unit0 + L;
    bh = u / nqt;
    qt = u % nqt;
  }
  const int b = uni(bh / a.H);
  const int h = uni(bh - b * a.H);
  const int q_first = qt * kBM;
  const int irow = q_first + wave * 32 + col;
  const int q_last = min(q_first + kBM - 1, a.Sq - 1);

  const float sl2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  bf16x8 qf[D / 16];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<int64_t>(b) * a.Sq + min(irow, a.Sq - 1)) * a.H + h) * D +
                       8 * half;
    const uint32_t flip = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      w ^= flip;
      if (irow >= a.Sq) w = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int rs = a.H * D;
  uint32_t k_src[NL], v_src[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int s = (wave * NL + n) * 64 + lane;
    const int row = s / UPR, pu = s % UPR;
    const int k_key = swap_bits23(row), k_unit = pu ^ (row & Geo<D>::kKMask);
    const int v_unit = pu ^ ((row & 3) << 1);
    k_src[n] = 2u * static_cast<uint32_t>(k_key * rs + k_unit * 8);
    v_src[n] = 2u * static_cast<uint32_t>(row * rs + v_unit * 8);
    if constexpr (VT) {  // V^T tile: D rows of 8 16-byte units, unit u of row d at u ^ ((d >> 1) & 7)
      const int d = s >> 3, vu = (s & 7) ^ ((d >> 1) & 7);
      v_src[n] = 128u * d + 16u * vu;
    }
  }

  auto keys_of = [&](int c) {
    c = uni(c);
    int n = a.chunks[c].len;
    if (CAUSAL) n = max(0, min(n, q_last + a.chunks[c].delta + 1));
    return n;
  };
  struct Cur {
    int c, kt;
    int nk, len, delta;
    const char* tk;
    const char* tv;
  };
  const int64_t tile_bytes = 2 * static_cast<int64_t>(KB) * rs;
  auto enter = [&](Cur& x) {
    const int c = uni(x.c);
    if (c < a.nchunks) {
      x.len = uni(a.chunks[c].len);
      x.delta = uni(a.chunks[c].delta);
      x.nk = uni(CAUSAL ? max(0, min(x.len, q_last + x.delta + 1)) : x.len);
      const int64_t off =
          2 * ((static_cast<int64_t>(b) * x.len + uni(x.kt) * KB) * rs + h * D);
      x.tk = uni_ptr(reinterpret_cast<const char*>(a.chunks[c].k) + off);
      x.tv = uni_ptr(reinterpret_cast<const char*>(a.chunks[c].v) + off);
      if constexpr (VT)
        x.tv = uni_ptr(reinterpret_cast<const char*>(a.chunks[c].v) +
                       2 * ((static_cast<int64_t>(b) * a.H + h) * ((x.len + KB - 1) / KB) +
                            uni(x.kt)) * D * KB);
    }
  };
  auto next_of = [&](Cur x) {
    x.kt = uni(x.kt) + 1;
    if (x.kt * KB >= x.nk) {
      x.kt = 0;
      x.c = uni(x.c) + 1;
      while (x.c < a.nchunks && keys_of(x.c) == 0) ++x.c;
      enter(x);
    } else {
      x.tk = uni_ptr(x.tk + tile_bytes);
      x.tv = uni_ptr(x.tv + (VT ? 2 * D * KB : tile_bytes));
    }
    return x;
  };
  // copy one tile (n_valid rows of it from base, zeros for the rest) into dst
  // (a V^T tile is a whole 16 KB block: its padding keys past the chunk are
  // finite and get weight 0)
  auto issue = [&](char* dst, const char* base, int n_valid, bool is_v) {
    char* l = dst + gbase + wave * NL * 1024;
    const __amdgpu_buffer_rsrc_t rsrc =
        VT && is_v ? tile_rsrc(base, 2u * D * KB)
                   : tile_rsrc(base, static_cast<uint32_t>(n_valid) * static_cast<uint32_t>(2 * rs));
#pragma unroll
    for (int n = 0; n < NL; ++n) lds_load16(rsrc, is_v ? v_src[n] : k_src[n], l + n * 1024);
  };

  uint32_t k_rd[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) k_rd[ks] = gbase + k_unit_off<D>(col, 2 * ks + half);
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row = 8 * (g16 >> 1) + (j16 >> 2);
  const int v_el = 16 * (g16 & 1) + 4 * (j16 & 3);
  uint32_t v_rd[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md)
    v_rd[md] = gbase + v_unit_off<D>(v_row, (32 * md + v_el) >> 3) + ((v_el & 4) ? 8 : 0);
  // VT: the A fragment of k-step t is row d = 32 md + col, keys 16 t + 8 half .. +7
  uint32_t vt_rd[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) vt_rd[t] = gbase + 128u * col + 16u * ((2 * t + half) ^ ((col >> 1) & 7));

  auto qk = [&](const char* kl, f32x16* sacc) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kl + k_rd[ks] + mb * 32 * RB);
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks],
                                                           ks == 0 ? f32x16{} : sacc[mb], 0, 0, 0);
      }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // this group's half of the query tile's key tiles, in chunk order
  Cur cur0{0, 0, 0, 0, 0, nullptr, nullptr};
  int n, steps;
  {
    int total = 0;
    for (int cc = 0; cc < a.nchunks; ++cc) total += (keys_of(cc) + KB - 1) / KB;
    const int t_begin = grp == 0 ? 0 : total / 2;
    const int t_end = grp == 0 ? total / 2 : total;
    n = uni(t_end - t_begin);
    steps = uni(total - total / 2);  // both groups run the longer half's half-steps
    int skip = t_begin;
    while (cur0.c < a.nchunks) {
      const int nt = (keys_of(cur0.c) + KB - 1) / KB;
      if (skip < nt) break;
      skip -= nt;
      ++cur0.c;
    }
    cur0.kt = skip;
    enter(cur0);
  }

  f32x16 sacc[NMB];
  bf16x8 pf[NT];
  // ck = the tile of the next K copy. What later phases need of a tile is
  // taken when its K copy goes out: the V source and row count (its V copy
  // follows one S phase later) and the mask bounds relative to its first key,
  // rl = len - key0 and rd = delta - key0 (its S phase follows two S phases
  // later). ma/mb: mask bounds of the tiles of the next two S phases; vb_*:
  // the next V copy.
  Cur ck = cur0;
  int ma_rl = 0, ma_rd = 0, mb_rl = 0, mb_rd = 0, vb_n = 0;
  const char* vb_p = nullptr;
  auto take = [&](int& rl, int& rd) {
    const int key0 = uni(ck.kt) * KB;
    rl = uni(ck.len - key0);
    rd = uni(ck.delta - key0);
    vb_p = ck.tv;
    vb_n = uni(max(0, min(ck.nk - key0, KB)));
  };
  auto phase_s = [&]() {
    const int rl = ma_rl, rd = ma_rd;
    const bool masked = (rl < KB) || (CAUSAL && rd < KB - 1 - q_first);
    if (masked) {
      asm volatile("" ::: "memory");
      int lim = rl;
      if (CAUSAL) lim = min(lim, irow + rd + 1);
      lim -= 8 * half;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mb + 16 * (r >> 3) + (r & 7) >= lim) sacc[mb][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), sacc[0][2]);
#pragma unroll
    for (int r = 3; r < 31; r += 2)
      mx = fmaxf(fmaxf(mx, sacc[r >> 4][r & 15]), sacc[(r + 1) >> 4][(r + 1) & 15]);
    mx = fmaxf(mx, sacc[1][15]);
    mx = pair_max(mx) * sl2;
    if (__ballot(mx > m_run + kTau)) {
      asm volatile("" ::: "memory");
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < D / 32; ++md) oacc[md] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(
            __builtin_fmaf(sacc[t >> 1][(t & 1) * 8 + e], sl2, neg_m));
        psum += p;
        pf[t][e] = static_cast<__bf16>(p);
      }
    l_run += psum;
  };
  // copies at S(s): V(s+1) and K(s+2) of this group's tiles; then the cursors move on
  // (pend = tiles copied by this wave's latest S phase: they are read three
  // half-steps after the copy, so each barrier may leave them in flight)
  int pend = 0;
  auto s_copies = [&](int s, char* kdst, char* vdst) {
    pend = 0;
    if (s + 1 < n) { issue(vdst, vb_p, vb_n, true); ++pend; }
    ma_rl = mb_rl;
    ma_rd = mb_rd;
    if (s + 2 < n) {
      take(mb_rl, mb_rd);
      issue(kdst, ck.tk, vb_n, false);
      ++pend;
      if (s + 3 < n) ck = next_of(ck);
    }
  };
  auto phase_m = [&](const char* kl, const char* vl) {
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 vf;
        if constexpr (VT) {
          vf = *reinterpret_cast<const bf16x8*>(vl + vt_rd[t] + md * 32 * 128);
        } else {
          const char* vr = vl + v_rd[md] + 16 * t * RB;
          const bf16x4 lo = read_tr(vr);
          const bf16x4 hi = read_tr(vr + 4 * RB);
          vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], oacc[md], 0, 0, 0);
      }
    }
    qk(kl, sacc);
    constexpr int NVF = NT * (D / 32), NKF = NMB * (D / 16);
    if constexpr (VT) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int k = 0; k < NVF; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < NVF; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (k < NVF - 2)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
#pragma unroll
    for (int k = 0; k < NKF; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto sync = [&]() {
    if (pend == 2)
      __builtin_amdgcn_s_waitcnt(static_cast<short>(0x0070 | (2 * NL)));  // vmcnt(2 NL), lgkmcnt(0)
    else if (pend == 1)
      __builtin_amdgcn_s_waitcnt(static_cast<short>(0x0070 | NL));
    else
      __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
  };

  // prologue: K(0), V(0), K(1) of each group's half; S(0); group 0's S(0)
  if (n > 0) {
    take(ma_rl, ma_rd);
    issue(s_k0, ck.tk, vb_n, false);
    issue(s_v0, vb_p, vb_n, true);
    if (n > 1) {
      ck = next_of(ck);
      take(mb_rl, mb_rd);
      issue(s_k1, ck.tk, vb_n, false);
      if (n > 2) ck = next_of(ck);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n > 0) qk(s_k0, sacc);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // (now: ma = tile 0, mb and vb = tile 1, ck = tile 2)
  if (grp == 0 && n > 0) {
    phase_s();
    s_copies(0, s_k0, s_v1);
  }

  // Group 0: M(j) at hs = 2j (K(j+1) in stage (j+1)&1, V(j) in stage j&1),
  // S(j+1) with its copies at hs = 2j+1. Group 1 one half-step later: S(j)
  // with its copies at hs = 2j, M(j) at hs = 2j+1. Q = hs % 4 fixes the stages.
  auto hs_g0 = [&](auto q_tag, int hs) {
    constexpr int Q = decltype(q_tag)::value;
    const int j = hs >> 1;
    if (Q == 0 && j < n) phase_m(s_k1, s_v0);
    if (Q == 2 && j < n) phase_m(s_k0, s_v1);
    if (Q == 1 && j + 1 < n) { phase_s(); s_copies(j + 1, s_k1, s_v0); }
    if (Q == 3 && j + 1 < n) { phase_s(); s_copies(j + 1, s_k0, s_v1); }
    sync();
  };
  auto hs_g1 = [&](auto q_tag, int hs) {
    constexpr int Q = decltype(q_tag)::value;
    const int j = hs >> 1;
    if (Q == 0 && j < n) { phase_s(); s_copies(j, s_k0, s_v1); }
    if (Q == 2 && j < n) { phase_s(); s_copies(j, s_k1, s_v0); }
    if (Q == 1 && j < n) phase_m(s_k1, s_v0);
    if (Q == 3 && j < n) phase_m(s_k0, s_v1);
    sync();
  };
  const int nh = 2 * steps;
  if (grp == 0) {
    for (int hs = 0; hs < nh; hs += 4) {
      hs_g0(std::integral_constant<int, 0>{}, hs);
      hs_g0(std::integral_constant<int, 1>{}, hs + 1);
      if (hs + 2 >= nh) break;
      hs_g0(std::integral_constant<int, 2>{}, hs + 2);
      hs_g0(std::integral_constant<int, 3>{}, hs + 3);
    }
  } else {
    for (int hs = 0; hs < nh; hs += 4) {
      hs_g1(std::integral_constant<int, 0>{}, hs);
      hs_g1(std::integral_constant<int, 1>{}, hs + 1);
      if (hs + 2 >= nh) break;
      hs_g1(std::integral_constant<int, 2>{}, hs + 2);
      hs_g1(std::integral_constant<int, 3>{}, hs + 3);
    }
  }

  // ---- epilogue: merge the two key halves, normalise, write O and LSE
  float l_tot = l_run + __shfl_xor(l_run, 32);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  {
    constexpr int HM = D / 64;
    auto xo = [&](int md, int r) -> float& {
      float* base = reinterpret_cast<float*>(md < HM ? s_v0 : s_v1);
      return base[((wave * HM + md % HM) * 16 + r) * 64 + lane];
    };
    float* xs = reinterpret_cast<float*>(s_k0);
    if (grp == 1) {
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo(md, r) = oacc[md][r];
      xs[(wave * 2) * 64 + lane] = m_run;
      xs[(wave * 2 + 1) * 64 + lane] = l_tot;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xs[(wave * 2) * 64 + lane], l1 = xs[(wave * 2 + 1) * 64 + lane];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    l_tot = a0 * l_tot + a1 * l1;
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] = a0 * oacc[md][r] + a1 * xo(md, r);
    m_run = mm;
  }
  const int i = irow;
  if (i >= a.Sq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = ((static_cast<int64_t>(b) * a.Sq + i) * a.H + h) * D;
  const float lse_val = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
#pragma unroll
  for (int md = 0; md < D / 32; ++md) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * md + 8 * g + 4 * half;
      const float x0 = oacc[md][4 * g] * inv, x1 = oacc[md][4 * g + 1] * inv;
      const float x2 = oacc[md][4 * g + 2] * inv, x3 = oacc[md][4 * g + 3] * inv;
      if (OUT_BF16) {
        bf16x4 r;
        r[0] = static_cast<__bf16>(x0);
        r[1] = static_cast<__bf16>(x1);
        r[2] = static_cast<__bf16>(x2);
        r[3] = static_cast<__bf16>(x3);
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o) + orow + d0) = r;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.o) + orow + d0) =
            make_float4(x0, x1, x2, x3);
      }
    }
  }
  if (half == 0) {
    const int lstr = a.lse_stride > 0 ? a.lse_stride : a.Sq;
    a.lse[(static_cast<int64_t>(b) * a.H + h) * lstr + i] = lse_val;
  }
}

template <int D, bool CAUSAL, bool OUT_BF16, int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBM - 1) / kBM;
  const int64_t nsplit = (CAUSAL || G == 2) ? 1 : a.nsplit;
  const int64_t nitems = nqt * a.B * a.H * nsplit;
  const int64_t blocks = CAUSAL ? nitems : (nitems + 7) / 8 * 8;
  hipLaunchKernelGGL((attn_bf16_kernel<D, CAUSAL, OUT_BF16, G>),
                     dim3(static_cast<uint32_t>(blocks)), dim3(256 * G), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  // combine the splits' fp32 partials in split order
  return launch_lse_merge(a.part_o, a.part_lse, static_cast<int>(nsplit), a.o, a.lse, a.B, a.H,
                          a.Sq, D, OUT_BF16, stream, a.lse_stride);
}

template <int D, bool CAUSAL, bool OUT_BF16, bool VT = false>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  if (a.groups == 2) {
    if constexpr (D == 64 && !VT) {
      return launch_g<D, CAUSAL, OUT_BF16, 2>(a, stream);
    } else {
      // one 128-row query tile a block, its keys split between two groups
      const int64_t nitems = (a.Sq + kBM - 1) / kBM * a.B * a.H;
      const int64_t blocks = CAUSAL ? nitems : (nitems + 7) / 8 * 8;
      hipLaunchKernelGGL((attn_g2pp_kernel<D, CAUSAL, OUT_BF16, VT>),
                         dim3(static_cast<uint32_t>(blocks)), dim3(512), 0, stream, a);
      return hipGetLastError();
    }
  }
  // No key splits: the ping-pong kernel, 256 query rows a block, for one
  // chunk, and for a causal chunk list (D = 128) when its blocks fill the CUs
  // (measured: a non-causal chunk list, D = 64 or fewer blocks than CUs run
  // faster on the 4-wave kernel)
  const int64_t nitems = (a.Sq + 255) / 256 * a.B * a.H;
  const int64_t blocks = CAUSAL ? nitems : (nitems + 7) / 8 * 8;
  if (a.nsplit <= 1 && a.nchunks == 1) {
    if constexpr (!CAUSAL && D == 128) {
      // Equal blocks over more rounds than one: when the last round would be
      // at most half full, its rows run instead as 128-row two-group blocks
      // (half a 256-row block's work each), one round of half the length.
      const int64_t cus = device_cus();
      const int64_t rest = nitems % cus;
      if (nitems > cus && rest > 0 && 2 * rest <= cus) {
        AttnArgs m = a;
        m.unit0 = 0;
        m.units = static_cast<int32_t>(nitems - rest);
        m.pp_split = 1;
        hipLaunchKernelGGL((attn_pp_kernel<D, CAUSAL, OUT_BF16, false, false, VT>),
                           dim3(static_cast<uint32_t>((m.units + 7) / 8 * 8)), dim3(512), 0,
                           stream, m);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (!VT && a.last_split > 1 && a.part_o) {
          // with a workspace: the last round's units as 256-row blocks again,
          // each unit's keys split last_split ways, and a merge of their rows
          AttnArgs t = a;
          t.unit0 = m.units;
          t.units = static_cast<int32_t>(rest);
          t.pp_split = a.last_split;
          hipLaunchKernelGGL((attn_pp_kernel<D, CAUSAL, OUT_BF16, false, true>),
                             dim3(static_cast<uint32_t>((rest * a.last_split + 7) / 8 * 8)),
                             dim3(512), 0, stream, t);
          e = hipGetLastError();
          if (e != hipSuccess) return e;
          return launch_unit_merge(a.part_o, a.part_lse, a.last_split, a.o, a.lse, a.H, a.Sq, D,
                                   256, t.unit0, rest, OUT_BF16, stream, a.lse_stride);
        }
        const int64_t nqt256 = (a.Sq + 255) / 256, nqt128 = (a.Sq + kBM - 1) / kBM;
        const int64_t bh_s = m.units / nqt256, qt_s = m.units % nqt256;
        AttnArgs t = a;
        t.groups = 2;
        t.unit0 = static_cast<int32_t>(bh_s * nqt128 + 2 * qt_s);
        t.units = static_cast<int32_t>(a.B * a.H * nqt128 - t.unit0);
        hipLaunchKernelGGL((attn_g2pp_kernel<D, CAUSAL, OUT_BF16, VT>),
                           dim3(static_cast<uint32_t>((t.units + 7) / 8 * 8)), dim3(512), 0,
                           stream, t);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((attn_pp_kernel<D, CAUSAL, OUT_BF16, false, false, VT>),
                       dim3(static_cast<uint32_t>(blocks)), dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  if constexpr (VT) {
    return hipErrorInvalidValue;  // key-contiguous V: one chunk, no key splits (checked by the caller)
  } else {
  if constexpr (CAUSAL && D == 128) {
    if (a.nsplit <= 1 && a.nchunks > 1 && nitems >= device_cus()) {
      hipLaunchKernelGGL((attn_pp_kernel<D, CAUSAL, OUT_BF16, true>),
                         dim3(static_cast<uint32_t>(blocks)), dim3(512), 0, stream, a);
      return hipGetLastError();
    }
  }
  return launch_g<D, CAUSAL, OUT_BF16, 1>(a, stream);
  }
}



template <int D>
hipError_t launch_d(const AttnArgs& a, bool causal, bool out_bf16, hipStream_t stream) {
  if (causal)
    return out_bf16 ? launch_t<D, true, true>(a, stream) : launch_t<D, true, false>(a, stream);
  return out_bf16 ? launch_t<D, false, true>(a, stream) : launch_t<D, false, false>(a, stream);
}

}  // namespace

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Blocks of 128 query rows, two resident per CU. A grid of at most one query
// tile per CU runs two-group blocks: eight waves per tile, its keys split
// between the groups and merged in LDS. A grid between one and two tiles per
// CU (ring calls over a chunk list, which have a workspace) is split along
// the keys across blocks until it covers the GPU, keeping at least 8 tiles
// per split (the merge pass costs one fp32 read/write per split).
int attn_groups(int64_t B, int64_t H, int64_t Sq, int64_t tiles) {
  const int64_t units = (Sq + kBM - 1) / kBM * B * H;
  return units <= device_cus() && tiles >= 4 ? 2 : 1;
}

int attn_split_count(int64_t B, int64_t H, int64_t Sq, int64_t tiles, bool causal) {
  if (causal) return 1;
  const int64_t units = (Sq + kBM - 1) / kBM * B * H;
  if (units <= device_cus()) return 1;  // two-group blocks split the keys in LDS instead
  const int64_t slots = 2 * static_cast<int64_t>(device_cus());
  int s = 1;
  while (s < kMaxSplit && units * s < slots && tiles / (s + 1) >= 8) ++s;
  return s;
}

int attn_tail_splits(int64_t B, int64_t H, int64_t Sq, int64_t tiles, bool causal) {
  // (a causal grid of that size already runs every block in one round: it is
  // never split, and two launches only add the second one's fixed cost)
  if (causal || B != 1 || H <= 0) return 0;
  const int64_t nqt = (Sq + kBM - 1) / kBM;
  const int64_t tail = Sq - (nqt - 1) * kBM;
  const int64_t cus = device_cus();
  if (nqt < 2 || tail > kTailRows || nqt * H <= cus || (nqt - 1) * H > cus || tiles < 4) return 0;
  // one round of blocks over the CUs; at most kTailSplit partials per row keep
  // the merge on its path that has every partial's loads in flight at once
  const int64_t s = std::min<int64_t>(kTailSplit, std::max<int64_t>(1, cus / H));
  return static_cast<int>(std::min<int64_t>(s, tiles));
}

int64_t attn_split_floats(int64_t nsplit, int64_t B, int64_t H, int64_t Sq, int64_t D) {
  return nsplit <= 1 ? 0 : nsplit * (B * Sq * H * D + B * H * Sq);
}

// The last round of equal 256-row blocks, at most half full: its units' keys
// split so that their blocks fill the CUs once (at most kLastSplit ways, at
// least 4 key tiles a split). The launcher applies it to one-chunk grids.
int attn_last_splits(int64_t B, int64_t H, int64_t Sq, int64_t D, int64_t tiles, bool causal) {
  if (causal || D != 128 || B <= 0 || H <= 0 || Sq <= 0) return 0;
  const int64_t cus = device_cus();
  const int64_t nitems = (Sq + 255) / 256 * B * H;
  const int64_t rest = nitems % cus;
  if (nitems <= cus || rest == 0 || 2 * rest > cus) return 0;
  const int64_t s = std::min<int64_t>({kLastSplit, cus / rest, tiles / 4});
  return s >= 2 ? static_cast<int>(s) : 0;
}

int64_t attn_last_split_floats(int64_t B, int64_t H, int64_t Sq, int64_t D, int64_t tiles,
                               bool causal) {
  const int s = attn_last_splits(B, H, Sq, D, tiles, causal);
  if (s < 2) return 0;
  const int64_t rest = (Sq + 255) / 256 * B * H % device_cus();
  return s * rest * 256 * (D + 1);
}

hipError_t launch_attn_bf16(const AttnArgs& a, bool causal, bool out_bf16, hipStream_t stream) {
  if (a.vt) {  // key-contiguous V (D = 128, one chunk, no key splits: checked by the caller)
    if (causal)
      return out_bf16 ? launch_t<128, true, true, true>(a, stream)
                      : launch_t<128, true, false, true>(a, stream);
    return out_bf16 ? launch_t<128, false, true, true>(a, stream)
                    : launch_t<128, false, false, true>(a, stream);
  }
  return a.D == 64 ? launch_d<64>(a, causal, out_bf16, stream)
                   : launch_d<128>(a, causal, out_bf16, stream);
}

}  // namespace cpattn
