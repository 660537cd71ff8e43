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
// over D/4 lanes, each lane owning one float4 column in every partial, so
// each load instruction of a wave covers whole contiguous rows. The P
// partials are summed in the fixed order c = 0..P-1 (deterministic).
#include "cp_internal.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int P,
    void* __restrict__ o, float* __restrict__ lse, uint32_t rows, FastDiv heads, FastDiv seq,
    FastDiv cols, int64_t part_stride_o, int64_t part_stride_l) {
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t row = cols.div(gid);           // row = (b*Sq + i)*H + h
  if (row >= rows) return;
  const uint32_t col = gid - row * cols.d;      // float4 column within the row
  const uint32_t bi = heads.div(row);
  const uint32_t h = row - bi * heads.d;
  const uint32_t b = seq.div(bi);
  const uint32_t i = bi - b * seq.d;
  const int64_t lrow = (static_cast<int64_t>(b) * heads.d + h) * seq.d + i;  // [b][h][i]

  float m = -INFINITY;
  for (int c = 0; c < P; ++c) m = fmaxf(m, lse_parts[c * part_stride_l + lrow]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    float z = 0.f;
    for (int c = 0; c < P; ++c) z += expf(lse_parts[c * part_stride_l + lrow] - m);
    out_lse = m + logf(z);
    const f32x4* src = reinterpret_cast<const f32x4*>(o_parts) +
                       static_cast<int64_t>(row) * cols.d + col;
    for (int c = 0; c < P; ++c) {
      const float w = expf(lse_parts[c * part_stride_l + lrow] - out_lse);
      const f32x4 x = __builtin_nontemporal_load(src + c * (part_stride_o / 4));
      acc.x += w * x.x;
      acc.y += w * x.y;
      acc.z += w * x.z;
      acc.w += w * x.w;
    }
  }
  const int64_t off = static_cast<int64_t>(row) * cols.d + col;
  if (OUT_BF16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 r;
    r[0] = static_cast<__bf16>(acc.x);
    r[1] = static_cast<__bf16>(acc.y);
    r[2] = static_cast<__bf16>(acc.z);
    r[3] = static_cast<__bf16>(acc.w);
    reinterpret_cast<bf16x4*>(o)[off] = r;
  } else {
    reinterpret_cast<float4*>(o)[off] = acc;
  }
  if (col == 0) lse[lrow] = out_lse;
}

}  // namespace

// Caller guarantees: P >= 1, D % 4 == 0, B*Sq*H*(D/4) < 2^31.
hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int P, void* o,
                            float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D, bool out_bf16,
                            hipStream_t stream) {
  const uint32_t rows = static_cast<uint32_t>(B * Sq * H);
  FastDiv heads, seq, cols;
  heads.init(static_cast<uint32_t>(H));
  seq.init(static_cast<uint32_t>(Sq));
  cols.init(static_cast<uint32_t>(D / 4));
  const int64_t threads = static_cast<int64_t>(rows) * (D / 4);
  const uint32_t blocks = static_cast<uint32_t>((threads + kThreads - 1) / kThreads);
  const int64_t stride_o = B * Sq * H * D;
  const int64_t stride_l = B * H * Sq;
  if (out_bf16)
    hipLaunchKernelGGL(lse_merge_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, o_parts,
                       lse_parts, P, o, lse, rows, heads, seq, cols, stride_o, stride_l);
  else
    hipLaunchKernelGGL(lse_merge_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, o_parts,
                       lse_parts, P, o, lse, rows, heads, seq, cols, stride_o, stride_l);
  return hipGetLastError();
}

}  // namespace cpattn
