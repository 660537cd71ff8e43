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
//    waves through LDS.
//  * The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = a K
//    tile from LDS, B = Q^T held in registers for the whole kernel). In the
//    32x32 accumulator layout lane l holds query column l%32, so every
//    softmax statistic is a per-lane value: the row max and row sum are
//    in-lane reductions plus one exchange between the two half-waves
//    (v_permlane32_swap).
//  * K rows are written to LDS with key bits 2 and 3 swapped. With that, the
//    accumulator registers of lane l hold 8 consecutive keys per half-wave,
//    which is exactly the B-operand layout of the next product, so P (rounded
//    to bf16) feeds O^T += V^T P^T without any data movement.
//  * V is transposed once while it is staged into LDS (register 8xKPT
//    transpose, 8-byte LDS stores), so V^T fragments are 16-byte LDS reads.
//  * exp2 with scale*log2(e) folded into the scores; the O rescale is skipped
//    when no row max of the wave moved (exact: the factor would be 1.0).
//  * Non-causal grids map blocks to XCDs so that the tiles of one head stay
//    on one XCD's L2; causal grids launch the heaviest query tiles first.
#include "cp_internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per block
constexpr int kBN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
  static constexpr int kStrideK = D + 8;    // bf16 elements per K row in LDS (16 B pad)
  static constexpr int kStrideV = kBN + 8;  // bf16 elements per V^T row in LDS
  static constexpr int kUnitsK = kBN * D / 8 / kThreads;  // 16-byte K units per thread
  static constexpr int kKPT = D / 32;                     // V keys per thread
};

template <int D>
struct Staged {
  uint4 k[Tile<D>::kUnitsK];
  uint4 v[Tile<D>::kKPT];
};

// Global -> registers for one 64-key tile. kp/vp point at head h of the
// chunk's first row; keys at or beyond n_valid read as 0.
template <int D>
__device__ __forceinline__ void load_tile(Staged<D>& st, const __bf16* kp, const __bf16* vp,
                                          int64_t row0, int H, int key0, int n_valid, int tid) {
  constexpr int UPR = D / 8;  // 16-byte units per key row
#pragma unroll
  for (int r = 0; r < Tile<D>::kUnitsK; ++r) {
    const int u = tid + r * kThreads;
    const int key = u / UPR, dg = u % UPR;
    const int j = key0 + key;
    st.k[r] = j < n_valid ? *reinterpret_cast<const uint4*>(kp + (row0 + j) * H * D + dg * 8)
                          : make_uint4(0, 0, 0, 0);
  }
  const int dg = tid % UPR, kg = tid / UPR;
#pragma unroll
  for (int r = 0; r < Tile<D>::kKPT; ++r) {
    const int j = key0 + kg * Tile<D>::kKPT + r;
    st.v[r] = j < n_valid ? *reinterpret_cast<const uint4*>(vp + (row0 + j) * H * D + dg * 8)
                          : make_uint4(0, 0, 0, 0);
  }
}

// Registers -> LDS: K rows at swapped-bit positions, V transposed.
template <int D>
__device__ __forceinline__ void store_tile(const Staged<D>& st, __bf16* k_lds, __bf16* vt_lds,
                                           int tid) {
  constexpr int UPR = D / 8;
#pragma unroll
  for (int r = 0; r < Tile<D>::kUnitsK; ++r) {
    const int u = tid + r * kThreads;
    const int key = u / UPR, dg = u % UPR;
    *reinterpret_cast<uint4*>(k_lds + swap_bits23(key) * Tile<D>::kStrideK + dg * 8) = st.k[r];
  }
  const int dg = tid % UPR, kg = tid / UPR;
  constexpr int KPT = Tile<D>::kKPT;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(st.v);  // w[r*4 + e/2]
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t packed[KPT / 2];
#pragma unroll
    for (int r2 = 0; r2 < KPT / 2; ++r2) {
      const uint32_t a = w[(2 * r2) * 4 + e / 2], b = w[(2 * r2 + 1) * 4 + e / 2];
      packed[r2] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    __bf16* dst = vt_lds + (dg * 8 + e) * Tile<D>::kStrideV + kg * KPT;
    if (KPT == 4)
      *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[KPT / 2 - 1]);
    else
      *reinterpret_cast<uint32_t*>(dst) = packed[0];
  }
}

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kBN * Tile<D>::kStrideK];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[D * Tile<D>::kStrideV];

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
  const int q_last = min(qt * kBM + kBM - 1, a.Sq - 1);

  // ---- Q^T fragments (B operand), resident for the whole kernel
  bf16x8 qf[D / 16];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<int64_t>(b) * a.Sq + min(i, a.Sq - 1)) * a.H + h) * D +
                       8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
      if (i >= a.Sq) qf[ks] = bf16x8{};
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int md = 0; md < D / 32; ++md) oacc[md] = f32x16{};
  float m_run = -INFINITY;  // running row max, log2 domain
  float l_run = 0.f;        // this lane's share of the running row sum
  const float sl2 = a.scale * kLog2e;

  // ---- tile cursor over (chunk, tile)
  auto keys_of = [&](int c) {
    int n = a.chunks[c].len;
    if (CAUSAL) n = max(0, min(n, q_last + a.chunks[c].delta + 1));
    return n;
  };
  int c = 0;
  while (c < a.nchunks && keys_of(c) == 0) ++c;
  int kt = 0;
  Staged<D> st;
  const int64_t head_off = static_cast<int64_t>(h) * D;
  if (c < a.nchunks) {
    const ChunkDesc& ch = a.chunks[c];
    load_tile<D>(st, static_cast<const __bf16*>(ch.k) + head_off,
                 static_cast<const __bf16*>(ch.v) + head_off, static_cast<int64_t>(b) * ch.len,
                 a.H, 0, keys_of(c), tid);
  }

  while (c < a.nchunks) {
    const int n_keys = keys_of(c);
    const int len = a.chunks[c].len;
    const int delta = a.chunks[c].delta;
    // next (chunk, tile)
    int nc = c, nkt = kt + 1;
    if (nkt * kBN >= n_keys) {
      nkt = 0;
      nc = c + 1;
      while (nc < a.nchunks && keys_of(nc) == 0) ++nc;
    }
    __syncthreads();
    store_tile<D>(st, k_lds, vt_lds, tid);
    __syncthreads();
    if (nc < a.nchunks) {
      const ChunkDesc& ch = a.chunks[nc];
      load_tile<D>(st, static_cast<const __bf16*>(ch.k) + head_off,
                   static_cast<const __bf16*>(ch.v) + head_off, static_cast<int64_t>(b) * ch.len,
                   a.H, nkt * kBN, keys_of(nc), tid);
    }

    // ---- S^T = K Q^T for 64 keys x 32 queries
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            k_lds + (32 * mb + col) * Tile<D>::kStrideK + 16 * ks + 8 * half);
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mb], 0, 0, 0);
      }
    }

    // ---- online softmax (lane = query column; register r of block mb is key
    //      32*mb + 16*(r/8) + 8*half + r%8 of the tile)
    const int key0 = kt * kBN;
    const bool need_mask = (key0 + kBN > len) || (CAUSAL && key0 + kBN - 1 > qt * kBM + delta);
    float sv[32];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[mb * 16 + r] = sacc[mb][r] * sl2;
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = key0 + 32 * mb + 16 * (r >> 3) + 8 * half + (r & 7);
          bool vis = j < len;
          if (CAUSAL) vis = vis && (j <= i + delta);
          if (!vis) sv[mb * 16 + r] = -INFINITY;
        }
    }
    float mx = sv[0];
#pragma unroll
    for (int t = 1; t < 32; ++t) mx = fmaxf(mx, sv[t]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(sv[(t >> 1) * 16 + (t & 1) * 8 + e] - m_use);
        psum += p;
        pf[t][e] = static_cast<__bf16>(p);
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int md = 0; md < D / 32; ++md) oacc[md] *= alpha;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int md = 0; md < D / 32; ++md) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
            vt_lds + (32 * md + col) * Tile<D>::kStrideV + 16 * t + 8 * half);
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], oacc[md], 0, 0, 0);
      }
    }
    c = nc;
    kt = nkt;
  }

  // ---- epilogue: normalise, write O and LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (i >= a.Sq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = ((static_cast<int64_t>(b) * a.Sq + i) * a.H + h) * D;
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
  if (half == 0)
    a.lse[(static_cast<int64_t>(b) * a.H + h) * a.Sq + i] =
        l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
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
