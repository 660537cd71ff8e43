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
//    waves through double-buffered LDS, filled by direct global->LDS loads
//    (global_load_lds_dwordx4: no staging registers, no LDS store
//    instructions); one barrier per tile.
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
#include <type_traits>

#include "cp_internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per block
constexpr int kBN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // log2 headroom before the exponent offset is raised
constexpr int kMaxSplit = 2;      // key splits per query tile on small grids

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
  static constexpr int kTileBytes = kBN * kRowBytes;      // one K or V tile
  static constexpr int kLoadsPerWave = kBN * kUPR / kThreads;  // direct loads per wave per tensor
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

__device__ __forceinline__ void lds_load16(const __bf16* g, __bf16* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

__device__ __forceinline__ bf16x4 read_tr(const char* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// G = 1: a block is 4 waves over one query tile. G = 2: a block is two such
// groups of 4 waves over the same query tile, group g taking half g of the
// tile's keys with its own LDS stages; the halves are merged through LDS at
// the end (grids with fewer query tiles than CUs: every tile gets a whole CU).
template <int D, bool CAUSAL, bool OUT_BF16, int G>
__global__ __launch_bounds__(kThreads * G, G == 1 ? 2 : 1) void attn_bf16_kernel(AttnArgs a) {
  constexpr int UPR = Geo<D>::kUPR;
  constexpr int TB = Geo<D>::kTileBytes;
  constexpr int NL = Geo<D>::kLoadsPerWave;
  // per group [K0][K1][V0][V1]
  __shared__ __attribute__((aligned(1024))) char smem[G * 4 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int grp = G == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);  // key half (G = 2)
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // wave within the group
  const int col = lane & 31, half = lane >> 5;
  const uint32_t gbase = static_cast<uint32_t>(grp * 4 * TB);  // the group's LDS stages

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
  const int b = bh / a.H, h = bh - b * a.H;
  const int i = qt * kBM + wave * 32 + col;  // this lane's query row
  const int q_first = qt * kBM;
  const int q_last = min(q_first + kBM - 1, a.Sq - 1);

  // ---- Q^T fragments (B operand), resident for the whole kernel. A negative
  //      scale is folded into Q (bf16 negation is exact).
  const float sl2 = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  bf16x8 qf[D / 16];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<int64_t>(b) * a.Sq + min(i, a.Sq - 1)) * a.H + h) * D +
                       8 * half;
    const uint32_t flip = a.scale < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      w ^= flip;
      if (i >= a.Sq) w = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- direct-load geometry: this lane fills LDS slot s = wave*NL*64 + n*64 + lane
  //      of each tensor tile; slot s is (row s/UPR, swizzled unit s%UPR). The
  //      lane's source offsets (bytes from the tile's first key) are fixed.
  const int rs = a.H * D;  // elements between consecutive keys (host checks 64*rs < 2^31)
  int ld_row[NL];
  uint32_t k_src[NL], v_src[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int s = (wave * NL + n) * 64 + lane;
    const int row = s / UPR, pu = s % UPR;
    ld_row[n] = row;
    const int k_key = swap_bits23(row), k_unit = pu ^ (row & Geo<D>::kKMask);
    const int v_unit = pu ^ ((row & 3) << 1);
    k_src[n] = 2u * static_cast<uint32_t>(k_key * rs + k_unit * 8);
    v_src[n] = 2u * static_cast<uint32_t>(row * rs + v_unit * 8);
  }

  // Chunk descriptors are read with a provably uniform index, so they come
  // in through scalar loads and never wait behind the vector-memory counter
  // that tracks the in-flight tile prefetch.
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto keys_of = [&](int c) {
    c = uni(c);
    int n = a.chunks[c].len;
    if (CAUSAL) n = max(0, min(n, q_last + a.chunks[c].delta + 1));
    return n;
  };
  struct Cur {
    int c, kt;
  };
  auto next_of = [&](Cur x) {
    x.c = uni(x.c);
    x.kt = uni(x.kt) + 1;
    if (x.kt * kBN >= keys_of(x.c)) {
      x.kt = 0;
      ++x.c;
      while (x.c < a.nchunks && keys_of(x.c) == 0) ++x.c;
    }
    return x;
  };
  // Direct loads of one K or V tile into `dst`: a uniform base address plus
  // the lane's fixed byte offset. Keys at or beyond the tile's valid count
  // are redirected to its last valid key (their probabilities are exactly 0).
  auto issue = [&](char* dst, Cur x, bool is_v) {
    const int c = uni(x.c);
    x.kt = uni(x.kt);
    const int n_valid = keys_of(c) - x.kt * kBN;
    const char* base =
        reinterpret_cast<const char*>(is_v ? a.chunks[c].v : a.chunks[c].k) +
        2 * ((static_cast<int64_t>(b) * a.chunks[c].len + x.kt * kBN) * rs + h * D);
    char* l = dst + gbase + wave * NL * 1024;
    if (n_valid >= kBN) {
#pragma unroll
      for (int n = 0; n < NL; ++n)
        lds_load16(reinterpret_cast<const __bf16*>(base + (is_v ? v_src[n] : k_src[n])),
                   reinterpret_cast<__bf16*>(l + n * 1024));
    } else {
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        const int key = is_v ? ld_row[n] : swap_bits23(ld_row[n]);
        const uint32_t fix = key < n_valid ? 0u : 2u * static_cast<uint32_t>((key - n_valid + 1) * rs);
        lds_load16(reinterpret_cast<const __bf16*>(base + ((is_v ? v_src[n] : k_src[n]) - fix)),
                   reinterpret_cast<__bf16*>(l + n * 1024));
      }
    }
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

  // LDS: K tiles in slots 0/1, V tiles in slots 2/3 (TB bytes each), per group
  char* const lds = smem;

  // S^T = K Q^T for the 64 keys of the K tile in slot `ks_slot` (32 queries per wave)
  auto qk = [&](int k_slot, f32x16* sacc) {
    const char* kl = lds + k_slot * TB;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(kl + k_rd[0] + mb * 32 * Geo<D>::kRowBytes), qf[0],
          f32x16{}, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < D / 16; ++ks)
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(kl + k_rd[ks] + mb * 32 * Geo<D>::kRowBytes),
            qf[ks], sacc[mb], 0, 0, 0);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY;  // exponent offset, log2 domain
  float l_run = 0.f;        // this lane's share of the row sum

  // this block's share of the query tile's tiles, in chunk order
  Cur cur0{0, 0};
  int left, steps;
  {
    int total = 0;
    for (int cc = 0; cc < a.nchunks; ++cc) total += (keys_of(cc) + kBN - 1) / kBN;
    const int nparts = G == 2 ? 2 : nsplit, part = G == 2 ? grp : sp;
    const int t_begin = static_cast<int>(static_cast<int64_t>(total) * part / nparts);
    const int t_end = static_cast<int>(static_cast<int64_t>(total) * (part + 1) / nparts);
    left = uni(t_end - t_begin);
    // both groups step together (block-wide barriers): the second half is the longer
    steps = uni(G == 2 ? total - total / 2 : left);
    int skip = t_begin;
    while (cur0.c < a.nchunks) {
      const int nt = (keys_of(cur0.c) + kBN - 1) / kBN;
      if (skip < nt) break;
      skip -= nt;
      ++cur0.c;
    }
    cur0.kt = skip;
  }

  // One pipeline step for tile j (cursor cur0; cur1/cur2 are tiles j+1/j+2):
  // prefetch K of j+2 and V of j+1, then S for tile j+1 on the matrix cores
  // while the softmax of tile j runs, then O += P V for tile j. Tile j's K
  // and V sit in slots PAR and 2+PAR; PAR = j & 1 is a compile-time constant
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
    if (j + 2 < left) issue(lds + PAR * TB, cur2, false);
    if (j + 1 < left) issue(lds + (3 - PAR) * TB, cur1, true);
    const int c0 = uni(cur0.c);
    const int len = a.chunks[c0].len;
    const int delta = a.chunks[c0].delta;
    const int key0 = uni(cur0.kt) * kBN;

    // softmax of tile j (lane = query column; register r of block mb is key
    // key0 + 32*mb + 16*(r/8) + 8*half + r%8)
    const bool masked = (key0 + kBN > len) || (CAUSAL && key0 + kBN - 1 > q_first + delta);
    if (masked) {
      asm volatile("" ::: "memory");  // keeps this a real (uniform) branch
      // visible iff the key index relative to key0 is < lim
      int lim = len - key0;
      if (CAUSAL) lim = min(lim, i + delta - key0 + 1);
      lim -= 8 * half;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
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
    qk(1 - PAR, s_next);
    bf16x8 pf[4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p =
            __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[t >> 1][(t & 1) * 8 + e], sl2, neg_m));
        psum += p;
        pf[t][e] = static_cast<__bf16>(p);
      }
    l_run += psum;

    // O^T += V^T P^T for tile j
    const char* vl = lds + (2 + PAR) * TB;
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const char* vr = vl + v_rd[md] + 16 * t * Geo<D>::kRowBytes;
        const bf16x4 lo = read_tr(vr);
        const bf16x4 hi = read_tr(vr + 4 * Geo<D>::kRowBytes);
        const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], oacc[md], 0, 0, 0);
      }
    }
    // Instruction interleave for the block above: S of tile j+1 (one MFMA
    // per K-fragment read) with the exponentials of tile j in between, then
    // P*V (one MFMA per two transposed V reads) with the row-sum additions.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);      // LDS reads run ahead
#pragma unroll
    for (int k = 0; k < 2 * (D / 16); ++k) {               // S MFMAs of qk()
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);    // VALU
    }
#pragma unroll
    for (int k = 0; k < 4 * (D / 32); ++k) {               // P*V MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  f32x16 s_a[2], s_b[2];
  if (steps > 0) {
    if (G == 1 || left > 0) {
      issue(lds, cur0, false);
      issue(lds + 2 * TB, cur0, true);
      if (left > 1) {
        cur1 = next_of(cur0);
        issue(lds + TB, cur1, false);
      }
      if (left > 2) cur2 = next_of(cur1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (G == 1 || left > 0) qk(0, s_a);
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
    // through LDS (every wave is past its last tile read after this barrier)
    __syncthreads();
    float* xo = reinterpret_cast<float*>(smem + 4 * TB);  // [wave][md][r][lane]
    float* xs = reinterpret_cast<float*>(smem);           // [wave][m, l][lane]
    if (grp == 1) {
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[((wave * (D / 32) + md) * 16 + r) * 64 + lane] = oacc[md][r];
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
      for (int r = 0; r < 16; ++r)
        oacc[md][r] = a0 * oacc[md][r] + a1 * xo[((wave * (D / 32) + md) * 16 + r) * 64 + lane];
    m_run = mm;
  }
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
  if (half == 0) a.lse[lrow] = lse_val;
}

template <int D, bool CAUSAL, bool OUT_BF16, int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBM - 1) / kBM;
  const int64_t nsplit = (CAUSAL || G == 2) ? 1 : a.nsplit;
  const int64_t nitems = nqt * a.B * a.H * nsplit;
  const int64_t blocks = CAUSAL ? nitems : (nitems + 7) / 8 * 8;
  hipLaunchKernelGGL((attn_bf16_kernel<D, CAUSAL, OUT_BF16, G>),
                     dim3(static_cast<uint32_t>(blocks)), dim3(kThreads * G), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  // combine the splits' fp32 partials in split order
  return launch_lse_merge(a.part_o, a.part_lse, static_cast<int>(nsplit), a.o, a.lse, a.B, a.H,
                          a.Sq, D, OUT_BF16, stream);
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  return a.groups == 2 ? launch_g<D, CAUSAL, OUT_BF16, 2>(a, stream)
                       : launch_g<D, CAUSAL, OUT_BF16, 1>(a, stream);
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
// CU (ring calls, which have a workspace) is split along the keys across
// blocks until it covers the GPU, keeping at least 8 tiles per split (the
// merge pass costs one fp32 read/write per split).
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

int64_t attn_split_floats(int64_t nsplit, int64_t B, int64_t H, int64_t Sq, int64_t D) {
  return nsplit <= 1 ? 0 : nsplit * (B * Sq * H * D + B * H * Sq);
}

hipError_t launch_attn_bf16(const AttnArgs& a, bool causal, bool out_bf16, hipStream_t stream) {
  return a.D == 64 ? launch_d<64>(a, causal, out_bf16, stream)
                   : launch_d<128>(a, causal, out_bf16, stream);
}

}  // namespace cpattn
