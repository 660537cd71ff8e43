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
//    waves through double-buffered LDS (one barrier per tile).
//  * The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = a K
//    tile from LDS, B = Q^T held in registers for the whole kernel). In the
//    32x32 accumulator layout lane l holds query column l%32, so every
//    softmax statistic is a per-lane value: the row max and row sum are
//    in-lane reductions plus one exchange between the two half-waves.
//  * K rows are written to LDS with key bits 2 and 3 swapped. With that, the
//    accumulator registers of lane l hold 8 consecutive keys per half-wave,
//    which is exactly the B-operand layout of the next product, so P (rounded
//    to bf16) feeds O^T += V^T P^T without any data movement.
//  * V stays row-major in LDS; its transposed A-operand fragments come from
//    ds_read_b64_tr_b16 (within each 16-lane group, lane i addresses row
//    k0 + i/4, columns d0 + 4(i%4) .. +3, and receives column d0 + i of rows
//    k0 .. k0+3).
//  * LDS row padding: K rows are D+8 elements (8 consecutive rows read at one
//    column land on distinct 16-byte bank groups), V rows are D+16 (the 4
//    rows a transposed read touches land on distinct 32-byte bank groups).
//  * Softmax in the log2 domain with scale*log2(e) folded into one FMA per
//    score. The exponent offset m is only raised when a tile's row max
//    exceeds it by more than kTau (then O and the row sum are rescaled), so
//    probabilities stay <= 2^kTau and the rescale is rare; the final
//    normalisation uses the same offsets, so the result is unchanged up to
//    rounding.
//  * Masked and unmasked tiles take separate code paths; only ragged tails
//    and causal diagonal tiles pay for masking.
//  * Non-causal grids map blocks to XCDs so that the tiles of one head stay
//    on one XCD's L2; causal grids launch the heaviest query tiles first.
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
struct Tile {
  static constexpr int kStrideK = D + 8;   // bf16 elements per K row in LDS
  static constexpr int kStrideV = D + 16;  // bf16 elements per V row in LDS
  static constexpr int kUPR = D / 8;       // 16-byte units per key row
  static constexpr int kUnits = kBN * kUPR / kThreads;  // units per thread per tensor
  static constexpr int kKeyStep = kThreads / kUPR;       // key distance between a thread's units
  static constexpr int kLdsK = kBN * kStrideK;
  static constexpr int kLdsV = kBN * kStrideV;
};

template <int D>
struct Staged {
  u32x4 k[Tile<D>::kUnits];
  u32x4 v[Tile<D>::kUnits];
};

// Global -> registers for one tile. kp/vp point at this thread's first unit
// of the tile; rows are `rs` elements apart. Keys at or beyond `n_valid`
// (relative to the tile) read as 0.
template <int D, bool TAIL>
__device__ __forceinline__ void load_tile(Staged<D>& st, const __bf16* kp, const __bf16* vp,
                                          int64_t rs, int key_t, int n_valid) {
#pragma unroll
  for (int r = 0; r < Tile<D>::kUnits; ++r) {
    const int64_t off = r * Tile<D>::kKeyStep * rs;
    if (!TAIL || key_t + r * Tile<D>::kKeyStep < n_valid) {
      st.k[r] = *reinterpret_cast<const u32x4*>(kp + off);
      st.v[r] = *reinterpret_cast<const u32x4*>(vp + off);
    } else {
      st.k[r] = u32x4{0, 0, 0, 0};
      st.v[r] = u32x4{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const Staged<D>& st, __bf16* k_lds, __bf16* v_lds,
                                           int key_t, int dg) {
#pragma unroll
  for (int r = 0; r < Tile<D>::kUnits; ++r) {
    const int key = key_t + r * Tile<D>::kKeyStep;
    *reinterpret_cast<u32x4*>(k_lds + swap_bits23(key) * Tile<D>::kStrideK + dg * 8) = st.k[r];
    *reinterpret_cast<u32x4*>(v_lds + key * Tile<D>::kStrideV + dg * 8) = st.v[r];
  }
}

__device__ __forceinline__ bf16x4 read_tr(const __bf16* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Per-wave online-softmax state and accumulators.
template <int D>
struct WaveState {
  f32x16 o[D / 32];
  float m;  // exponent offset, log2 domain
  float l;  // this lane's share of the row sum
};

// One 64-key tile for one wave: S^T = K Q^T, softmax update, O^T += V^T P^T.
template <int D, bool MASKED, bool CAUSAL>
__device__ __forceinline__ void tile_step(WaveState<D>& ws, const bf16x8* qf, const __bf16* k_lds,
                                          const __bf16* v_lds, float sl2, int col, int half,
                                          int key0, int len, int i, int delta, int vt_off) {
  f32x16 sacc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const __bf16* kr = k_lds + (32 * mb + col) * Tile<D>::kStrideK + 8 * half;
    sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8*>(kr), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < D / 16; ++ks)
      sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(kr + 16 * ks), qf[ks], sacc[mb], 0, 0, 0);
  }
  // register r of block mb holds key key0 + 32*mb + 16*(r/8) + 8*half + r%8
  if (MASKED) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = key0 + 32 * mb + 16 * (r >> 3) + 8 * half + (r & 7);
        bool vis = j < len;
        if (CAUSAL) vis = vis && (j <= i + delta);
        sacc[mb][r] = vis ? sacc[mb][r] : -INFINITY;
      }
  }
  float mx = fmaxf(sacc[0][0], sacc[0][1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[0][r + 1]));
#pragma unroll
  for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[1][r], sacc[1][r + 1]));
  mx = pair_max(mx) * sl2;
  if (__ballot(mx > ws.m + kTau)) {
    asm volatile("" ::: "memory");
    const float m_new = fmaxf(ws.m, mx);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(ws.m - m_new);
    ws.l *= alpha;
#pragma unroll
    for (int md = 0; md < D / 32; ++md) ws.o[md] *= alpha;
    ws.m = m_new;
  }
  const float neg_m = ws.m == -INFINITY ? 0.f : -ws.m;
  bf16x8 pf[4];
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p =
          __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t >> 1][(t & 1) * 8 + e], sl2, neg_m));
      psum += p;
      pf[t][e] = static_cast<__bf16>(p);
    }
  ws.l += psum;
#pragma unroll
  for (int md = 0; md < D / 32; ++md) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const __bf16* vr = v_lds + vt_off + (16 * t) * Tile<D>::kStrideV + 32 * md;
      const bf16x4 lo = read_tr(vr);
      const bf16x4 hi = read_tr(vr + 4 * Tile<D>::kStrideV);
      const bf16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      ws.o[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], ws.o[md], 0, 0, 0);
    }
  }
}

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][Tile<D>::kLdsK];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][Tile<D>::kLdsV];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  // ---- block -> (batch*head, query tile)
  const int nqt = (a.Sq + kBM - 1) / kBM;
  const int BH = a.B * a.H;
  const int ntiles = nqt * BH;
  int bh, qt;
  if (CAUSAL) {
    const int L = blockIdx.x;  // heaviest (last) query tiles first
    qt = nqt - 1 - L / BH;
    bh = L % BH;
  } else {
    const int per_xcd = (ntiles + 7) / 8;  // consecutive block ids go to different XCDs
    const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (L >= ntiles) return;
    bh = L / nqt;
    qt = L % nqt;
  }
  const int b = bh / a.H, h = bh - b * a.H;
  const int i = qt * kBM + wave * 32 + col;  // this lane's query row
  const int q_first = qt * kBM;
  const int q_last = min(q_first + kBM - 1, a.Sq - 1);

  // ---- Q^T fragments (B operand), resident for the whole kernel. A negative
  //      scale is folded into Q (bf16 negation is exact).
  const float scale_abs = fabsf(a.scale);
  const float sl2 = fmaxf(scale_abs * kLog2e, 1e-30f);
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

  WaveState<D> ws;
#pragma unroll
  for (int md = 0; md < D / 32; ++md) ws.o[md] = f32x16{};
  ws.m = -INFINITY;
  ws.l = 0.f;

  // ---- staging geometry of this thread
  const int dg = tid % Tile<D>::kUPR;
  const int key_t = tid / Tile<D>::kUPR;
  const int64_t rs = static_cast<int64_t>(a.H) * D;  // elements between consecutive keys
  const int64_t thr_off = static_cast<int64_t>(key_t) * rs + static_cast<int64_t>(h) * D + dg * 8;
  // transposed V read: 16-lane group g, lane-in-group j
  const int g16 = lane >> 4, j16 = lane & 15;
  const int vt_off = (8 * (g16 >> 1) + (j16 >> 2)) * Tile<D>::kStrideV + 16 * (g16 & 1) +
                     4 * (j16 & 3);

  auto keys_of = [&](int c) {
    int n = a.chunks[c].len;
    if (CAUSAL) n = max(0, min(n, q_last + a.chunks[c].delta + 1));
    return n;
  };
  auto tile_ptr = [&](int c, int kt, bool is_v) {
    const __bf16* base = static_cast<const __bf16*>(is_v ? a.chunks[c].v : a.chunks[c].k);
    return base + (static_cast<int64_t>(b) * a.chunks[c].len + kt * kBN) * rs + thr_off;
  };
  auto load = [&](Staged<D>& st, int c, int kt) {
    const int n = keys_of(c) - kt * kBN;
    if (n >= kBN)
      load_tile<D, false>(st, tile_ptr(c, kt, false), tile_ptr(c, kt, true), rs, key_t, n);
    else
      load_tile<D, true>(st, tile_ptr(c, kt, false), tile_ptr(c, kt, true), rs, key_t, n);
  };
  // advance (c, kt) to the next non-empty tile; c == nchunks when done
  auto advance = [&](int& c, int& kt) {
    ++kt;
    if (kt * kBN >= keys_of(c)) {
      kt = 0;
      ++c;
      while (c < a.nchunks && keys_of(c) == 0) ++c;
    }
  };

  int c = 0, kt = 0;
  while (c < a.nchunks && keys_of(c) == 0) ++c;
  Staged<D> st;
  int buf = 0;
  if (c < a.nchunks) {
    load(st, c, kt);
    store_tile<D>(st, k_lds[0], v_lds[0], key_t, dg);
  }
  int nc = c, nkt = kt;  // tile staged in registers next
  if (nc < a.nchunks) {
    advance(nc, nkt);
    if (nc < a.nchunks) load(st, nc, nkt);
  }
  __syncthreads();

  while (c < a.nchunks) {
    const int len = a.chunks[c].len;
    const int delta = a.chunks[c].delta;
    const int key0 = kt * kBN;
    const bool masked =
        (key0 + kBN > len) || (CAUSAL && key0 + kBN - 1 > q_first + delta);
    // The empty asm statements keep the two variants as separate branches
    // (otherwise both get speculated and merged with selects).
    if (masked) {
      asm volatile("" ::: "memory");
      tile_step<D, true, CAUSAL>(ws, qf, k_lds[buf], v_lds[buf], sl2, col, half, key0, len, i,
                                 delta, vt_off);
    } else {
      asm volatile("" ::: "memory");
      tile_step<D, false, CAUSAL>(ws, qf, k_lds[buf], v_lds[buf], sl2, col, half, key0, len, i,
                                  delta, vt_off);
    }
    if (nc < a.nchunks) {
      store_tile<D>(st, k_lds[buf ^ 1], v_lds[buf ^ 1], key_t, dg);
      int c2 = nc, kt2 = nkt;
      advance(c2, kt2);
      if (c2 < a.nchunks) load(st, c2, kt2);
      c = nc;
      kt = nkt;
      nc = c2;
      nkt = kt2;
    } else {
      c = a.nchunks;
    }
    buf ^= 1;
    __syncthreads();
  }

  // ---- epilogue: normalise, write O and LSE
  const float l_tot = ws.l + __shfl_xor(ws.l, 32);
  if (i >= a.Sq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = ((static_cast<int64_t>(b) * a.Sq + i) * a.H + h) * D;
#pragma unroll
  for (int md = 0; md < D / 32; ++md) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * md + 8 * g + 4 * half;
      const float x0 = ws.o[md][4 * g] * inv, x1 = ws.o[md][4 * g + 1] * inv;
      const float x2 = ws.o[md][4 * g + 2] * inv, x3 = ws.o[md][4 * g + 3] * inv;
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
  if (half == 0)
    a.lse[(static_cast<int64_t>(b) * a.H + h) * a.Sq + i] =
        l_tot > 0.f ? (ws.m + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBM - 1) / kBM;
  const int64_t ntiles = nqt * a.B * a.H;
  const int64_t blocks = CAUSAL ? ntiles : (ntiles + 7) / 8 * 8;
  hipLaunchKernelGGL((attn_bf16_kernel<D, CAUSAL, OUT_BF16>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, bool causal, bool out_bf16, hipStream_t stream) {
  if (causal)
    return out_bf16 ? launch_t<D, true, true>(a, stream) : launch_t<D, true, false>(a, stream);
  return out_bf16 ? launch_t<D, false, true>(a, stream) : launch_t<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, bool causal, bool out_bf16, hipStream_t stream) {
  return a.D == 64 ? launch_d<64>(a, causal, out_bf16, stream)
                   : launch_d<128>(a, causal, out_bf16, stream);
}

}  // namespace cpattn
