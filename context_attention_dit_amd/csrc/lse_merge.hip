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
// of a wave covers contiguous stretches of rows. A lane issues all its O
// loads before the weights are known, so they overlap the LSE loads and the
// weight arithmetic, done in base 2 on the hardware exp2/log2. The P
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
// of its loads is, across a wave, a contiguous stretch of rows.
template <bool OUT_BF16, int NC>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int P,
    void* __restrict__ o, float* __restrict__ lse, uint32_t rows, FastDiv heads, FastDiv seq,
    FastDiv cols, int64_t part_stride_o, int64_t part_stride_l) {
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t row = cols.div(gid);           // row = (b*Sq + i)*H + h
  if (row >= rows) return;
  const uint32_t col = gid - row * cols.d;      // first float4 column
  const uint32_t seg = cols.d;                  // distance between a thread's columns
  const uint32_t bi = heads.div(row);
  const uint32_t h = row - bi * heads.d;
  const uint32_t b = seq.div(bi);
  const uint32_t i = bi - b * seq.d;
  const int64_t lrow = (static_cast<int64_t>(b) * heads.d + h) * seq.d + i;  // [b][h][i]

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
  if (col == 0) lse[lrow] = out_lse;
}

template <bool OUT_BF16, int NC>
void launch_nc(const float* o_parts, const float* lse_parts, int P, void* o, float* lse,
               int64_t B, int64_t H, int64_t Sq, int64_t D, hipStream_t stream) {
  const uint32_t rows = static_cast<uint32_t>(B * Sq * H);
  FastDiv heads, seq, cols;
  heads.init(static_cast<uint32_t>(H));
  seq.init(static_cast<uint32_t>(Sq));
  cols.init(static_cast<uint32_t>(D / (4 * NC)));
  const int64_t threads = static_cast<int64_t>(rows) * (D / (4 * NC));
  const uint32_t blocks = static_cast<uint32_t>((threads + kThreads - 1) / kThreads);
  hipLaunchKernelGGL((lse_merge_kernel<OUT_BF16, NC>), dim3(blocks), dim3(kThreads), 0, stream,
                     o_parts, lse_parts, P, o, lse, rows, heads, seq, cols, B * Sq * H * D,
                     B * H * Sq);
}

}  // namespace

// Caller guarantees: P >= 1, D % 4 == 0, B*Sq*H*(D/4) < 2^31.
hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int P, void* o,
                            float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D, bool out_bf16,
                            hipStream_t stream) {
  if (D % 8 == 0) {
    if (out_bf16) launch_nc<true, 2>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, stream);
    else launch_nc<false, 2>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, stream);
  } else {
    if (out_bf16) launch_nc<true, 1>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, stream);
    else launch_nc<false, 1>(o_parts, lse_parts, P, o, lse, B, H, Sq, D, stream);
  }
  return hipGetLastError();
}

}  // namespace cpattn
