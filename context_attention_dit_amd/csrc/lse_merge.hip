// Merge of P per-chunk partial attention results (O_c, LSE_c), all fp32.
//
// Each ring hop yields an output normalised over its own chunk plus the log
// of that chunk's softmax normaliser; converting both to fp32 and weighting
// by exp(LSE_c - LSE) recovers attention over the union of the chunks
// (diffusers parallel API, ContextParallelConfig: convert_to_fp32; Sequence
// Parallelism page (SGLang Diffusion), section Numerics across node
// boundaries). Per row:
//   M = max_c LSE_c,  LSE = M + ln sum_c exp(LSE_c - M),
//   O = sum_c exp(LSE_c - LSE) * O_c;  no finite LSE_c -> O = 0, LSE = -inf.
//
// HBM-bound: every partial element is read once. A row's D floats are split
// over D/8 lanes (D/4 when D is not a multiple of 8), each lane owning two
// float4 columns half a row apart in every partial, so each load instruction
// of a wave covers whole rows. A block takes R consecutive query rows of one
// head, so its LSE loads and stores are contiguous, and consecutive blocks
// take the next heads of the same query rows, so the blocks in flight cover
// contiguous stretches of O ([b][i][h][d]) together. A lane issues all
// its O loads before the weights are known, so they overlap the LSE loads and
// the weight arithmetic, done in base 2 on the hardware exp2/log2. The P
// partials are summed in the fixed order c = 0..P-1 (deterministic).
#include "cp_internal.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kFastParts = 8;  // partial counts up to this keep every O load in flight at once
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Thread layout: `cols` = D/(4*NC) threads per row; a thread owns the NC
// float4 columns col, col + cols, ... of that row in every partial, so each
// of its loads covers, across a wave, whole rows of O.
// Block x covers rows i = t*R .. t*R + R-1 of head h in batch b, where
// x = (b*T + t)*H + h (T = ceil(Sq/R) row tiles of R = blockDim.x / cols rows).
template <bool OUT_BF16, int NC>
__global__ __launch_bounds__(1024) void lse_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int P,
    void* __restrict__ o, float* __restrict__ lse, uint32_t Sq, FastDiv heads, FastDiv tiles,
    FastDiv cols, int64_t part_stride_o, int64_t part_stride_l, uint32_t lse_stride) {
  const uint32_t bt = heads.div(blockIdx.x);
  const uint32_t h = blockIdx.x - bt * heads.d;
  const uint32_t b = tiles.div(bt);
  const uint32_t t = bt - b * tiles.d;
  const uint32_t r = cols.div(threadIdx.x);
  const uint32_t col = threadIdx.x - r * cols.d;  // first float4 column
  const uint32_t seg = cols.d;                    // distance between a thread's columns
  const uint32_t i = t * (blockDim.x / cols.d) + r;
  if (i >= Sq) return;
  const uint32_t lrow = (b * heads.d + h) * Sq + i;    // partial LSE index: (b*H + h)*Sq + i
  const uint32_t row = (b * Sq + i) * heads.d + h;     // O row: (b*Sq + i)*H + h

  const f32x4* src = reinterpret_cast<const f32x4*>(o_parts) + static_cast<int64_t>(row) * NC * seg + col;
  const int64_t so = part_stride_o / 4;
  f32x4 acc[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float out_lse = -INFINITY;
  // Weights in base 2: w_c = 2^((LSE_c - LSE) log2 e) with
  // LSE = M + ln 2 * log2 sum_c 2^((LSE_c - M) log2 e)
  if (P <= kFastParts) {
    // The partials' O loads do not depend on the LSEs: issue them first so
    // their latency overlaps the LSE loads and the weight arithmetic.
    f32x4 x[kFastParts][NC];
    float l[kFastParts];
#pragma unroll
    for (int c = 0; c < kFastParts; ++c)
      if (c < P) {
#pragma unroll
        for (int n = 0; n < NC; ++n) x[c][n] = __builtin_nontemporal_load(src + c * so + n * seg);
      }
#pragma unroll
    for (int c = 0; c < kFastParts; ++c) l[c] = c < P ? lse_parts[c * part_stride_l + lrow] : -INFINITY;
    float m = l[0];
#pragma unroll
    for (int c = 1; c < kFastParts; ++c) m = fmaxf(m, l[c]);
    if (m != -INFINITY) {
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < kFastParts; ++c)
        if (c < P) z += __builtin_amdgcn_exp2f((l[c] - m) * kLog2e);
      out_lse = m + __builtin_amdgcn_logf(z) * kLn2;
#pragma unroll
      for (int c = 0; c < kFastParts; ++c)
        if (c < P) {
          const float w = __builtin_amdgcn_exp2f((l[c] - out_lse) * kLog2e);
#pragma unroll
          for (int n = 0; n < NC; ++n) acc[n] += w * x[c][n];
        }
    }
  } else {
    float m = -INFINITY;
    for (int c = 0; c < P; ++c) m = fmaxf(m, lse_parts[c * part_stride_l + lrow]);
    if (m != -INFINITY) {
      float z = 0.f;
      for (int c = 0; c < P; ++c)
        z += __builtin_amdgcn_exp2f((lse_parts[c * part_stride_l + lrow] - m) * kLog2e);
      out_lse = m + __builtin_amdgcn_logf(z) * kLn2;
      for (int c = 0; c < P; ++c) {
        const float w =
            __builtin_amdgcn_exp2f((lse_parts[c * part_stride_l + lrow] - out_lse) * kLog2e);
#pragma unroll
        for (int n = 0; n < NC; ++n) acc[n] += w * __builtin_nontemporal_load(src + c * so + n * seg);
      }
    }
  }
  const int64_t off = static_cast<int64_t>(row) * NC * seg + col;
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    if (OUT_BF16) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = static_cast<__bf16>(acc[n][e]);
      reinterpret_cast<bf16x4*>(o)[off + n * seg] = r;
    } else {
      reinterpret_cast<f32x4*>(o)[off + n * seg] = acc[n];
    }
  }
  if (col == 0) lse[(b * heads.d + h) * lse_stride + i] = out_lse;
}

template <bool OUT_BF16, int NC>
void launch_nc(const float* o_parts, const float* lse_parts, int P, void* o, float* lse,
               int64_t B, int64_t H, int64_t Sq, int64_t D, int64_t lse_stride,
               hipStream_t stream) {
  const int64_t ncols = D / (4 * NC);         // <= 1024 (D <= 4096)
  const int64_t R = ncols < kThreads ? kThreads / ncols : 1;  // rows per block
  const int64_t T = (Sq + R - 1) / R;
  FastDiv heads, tiles, cols;
  heads.init(static_cast<uint32_t>(H));
  tiles.init(static_cast<uint32_t>(T));
  cols.init(static_cast<uint32_t>(ncols));
  const uint32_t blocks = static_cast<uint32_t>(B * T * H);
  hipLaunchKernelGGL((lse_merge_kernel<OUT_BF16, NC>), dim3(blocks),
                     dim3(static_cast<uint32_t>(ncols * R)), 0, stream, o_parts, lse_parts, P, o,
                     lse, static_cast<uint32_t>(Sq), heads, tiles, cols, B * Sq * H * D,
                     B * H * Sq, static_cast<uint32_t>(lse_stride));
}

// Rows of a unit range (AttnArgs::pp_split partials): block x takes rows
// R*x .. R*x + R-1 of the flat (unit, row in unit) order, R = blockDim.x /
// (D/8) rows, D/8 lanes a row with two float4 columns half a row apart each
// (D % 8 == 0). Same weights, order and output rounding as lse_merge_kernel.
template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void unit_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int P,
    void* __restrict__ o, float* __restrict__ lse, uint32_t H, uint32_t Sq, uint32_t D,
    uint32_t rows, uint32_t nqt, uint32_t unit0, uint32_t units, uint32_t lse_stride) {
  const uint32_t cols = D / 8;
  const uint32_t r_blk = blockDim.x / cols;
  const uint32_t t = threadIdx.x / cols, col = threadIdx.x - t * (D / 8);
  const uint32_t flat = blockIdx.x * r_blk + t;  // (unit in range) * rows + row in unit
  if (flat >= units * rows) return;
  const uint32_t lu = flat / rows, rr = flat - lu * rows;
  const uint32_t u = unit0 + lu;
  const uint32_t bh = u / nqt, qt = u - bh * nqt;
  const uint32_t i = qt * rows + rr;
  if (i >= Sq) return;
  const uint32_t b = bh / H, h = bh - b * H;
  const uint32_t seg = cols;  // a lane's two columns: col and col + D/8 (float4 units)
  const int64_t part_rows = static_cast<int64_t>(units) * rows;
  const f32x4* src = reinterpret_cast<const f32x4*>(o_parts) + static_cast<int64_t>(flat) * (D / 4) + col;
  const int64_t so = part_rows * (D / 4);
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  float out_lse = -INFINITY;
  float m = -INFINITY;
  for (int c = 0; c < P; ++c) m = fmaxf(m, lse_parts[c * part_rows + flat]);
  if (m != -INFINITY) {
    float z = 0.f;
    for (int c = 0; c < P; ++c) z += __builtin_amdgcn_exp2f((lse_parts[c * part_rows + flat] - m) * kLog2e);
    out_lse = m + __builtin_amdgcn_logf(z) * kLn2;
    for (int c = 0; c < P; ++c) {
      const float w = __builtin_amdgcn_exp2f((lse_parts[c * part_rows + flat] - out_lse) * kLog2e);
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[n] += w * __builtin_nontemporal_load(src + c * so + n * seg);
    }
  }
  const int64_t off = (((static_cast<int64_t>(b) * Sq + i) * H + h) * D) / 4 + col;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    if (OUT_BF16) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = static_cast<__bf16>(acc[n][e]);
      reinterpret_cast<bf16x4*>(o)[off + n * seg] = r;
    } else {
      reinterpret_cast<f32x4*>(o)[off + n * seg] = acc[n];
    }
  }
  if (col == 0) lse[(static_cast<int64_t>(b) * H + h) * lse_stride + i] = out_lse;
}

}  // namespace

// Caller guarantees: P >= 1, D % 8 == 0, units * rows < 2^32, the unit range
// lies inside the B*H*ceil(Sq/rows) units, Sq <= lse_stride when lse_stride > 0.
hipError_t launch_unit_merge(const float* o_parts, const float* lse_parts, int P, void* o,
                             float* lse, int64_t H, int64_t Sq, int64_t D, int64_t rows,
                             int64_t unit0, int64_t units, bool out_bf16, hipStream_t stream,
                             int64_t lse_stride) {
  const int64_t r_blk = kThreads / (D / 8);
  const uint32_t blocks = static_cast<uint32_t>((units * rows + r_blk - 1) / r_blk);
  const uint32_t nqt = static_cast<uint32_t>((Sq + rows - 1) / rows);
  const uint32_t ls = static_cast<uint32_t>(lse_stride > 0 ? lse_stride : Sq);
  const uint32_t threads = static_cast<uint32_t>(r_blk * (D / 8));
  if (out_bf16)
    hipLaunchKernelGGL((unit_merge_kernel<true>), dim3(blocks), dim3(threads), 0, stream, o_parts,
                       lse_parts, P, o, lse, static_cast<uint32_t>(H), static_cast<uint32_t>(Sq),
                       static_cast<uint32_t>(D), static_cast<uint32_t>(rows), nqt,
                       static_cast<uint32_t>(unit0), static_cast<uint32_t>(units), ls);
  else
    hipLaunchKernelGGL((unit_merge_kernel<false>), dim3(blocks), dim3(threads), 0, stream, o_parts,
                       lse_parts, P, o, lse, static_cast<uint32_t>(H), static_cast<uint32_t>(Sq),
                       static_cast<uint32_t>(D), static_cast<uint32_t>(rows), nqt,
                       static_cast<uint32_t>(unit0), static_cast<uint32_t>(units), ls);
  return hipGetLastError();
}

// Caller guarantees: P >= 1, D % 4 == 0, D <= 4096, B*Sq*H*(D/4) < 2^31,
// Sq <= lse_stride and B*H*lse_stride < 2^32 when lse_stride > 0.
hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int P, void* o,
                            float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D, bool out_bf16,
                            hipStream_t stream, int64_t lse_stride) {
  const int64_t ls = lse_stride > 0 ? lse_stride : Sq;
  if (D % 8 == 0) {
    if (out_bf16) launch_nc<true, 2>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, ls, stream);
    else launch_nc<false, 2>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, ls, stream);
  } else {
    if (out_bf16) launch_nc<true, 1>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, ls, stream);
    else launch_nc<false, 1>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, ls, stream);
  }
  return hipGetLastError();
}

}  // namespace cpattn
