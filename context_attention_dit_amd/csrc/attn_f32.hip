// fp32 block-wise softmax attention over a list of K/V chunks (fp32 in, fp32 out).
//
// The fp32 path keeps every step in fp32 (scores, softmax, accumulation) so
// that its result stays within fp32 rounding of exact attention. It is the
// small-size, full-precision companion of the bf16 MFMA kernel: one lane owns
// one query row, K/V tiles are staged in LDS and read as broadcasts, and the
// softmax is the online (running max / running sum) form, so the chunks are
// merged on the fly exactly as the ring's fp32 output+LSE merge prescribes
// (diffusers parallel API, ContextParallelConfig: convert_to_fp32).
#include "cp_internal.h"

namespace cpattn {
namespace {

constexpr int kRows = 64;   // query rows per block, one per lane
constexpr int kKeys = 32;   // keys per LDS tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(AttnArgs a) {
  __shared__ float4 k_lds[kKeys * D / 4];
  __shared__ float4 v_lds[kKeys * D / 4];
  const int tid = threadIdx.x;
  const int nqt = (a.Sq + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int b = bh / a.H, h = bh - b * a.H;
  const int i = qt * kRows + tid;
  const bool row_ok = i < a.Sq;

  float4 q[D / 4];
  const float4* qsrc = reinterpret_cast<const float4*>(a.q) +
                       ((static_cast<int64_t>(b) * a.Sq + (row_ok ? i : 0)) * a.H + h) * (D / 4);
#pragma unroll
  for (int d = 0; d < D / 4; ++d) {
    float4 x = qsrc[d];
    q[d] = row_ok ? make_float4(x.x * a.scale, x.y * a.scale, x.z * a.scale, x.w * a.scale)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 acc[D / 4];
#pragma unroll
  for (int d = 0; d < D / 4; ++d) acc[d] = make_float4(0.f, 0.f, 0.f, 0.f);
  float m_run = -INFINITY, l_run = 0.f;
  const int q_last = min(qt * kRows + kRows - 1, a.Sq - 1);

  for (int c = 0; c < a.nchunks; ++c) {
    const ChunkDesc ch = a.chunks[c];
    int n_keys = ch.len;
    if (CAUSAL) n_keys = max(0, min(n_keys, q_last + ch.delta + 1));
    const float4* ksrc = static_cast<const float4*>(ch.k);
    const float4* vsrc = static_cast<const float4*>(ch.v);
    for (int k0 = 0; k0 < n_keys; k0 += kKeys) {
      __syncthreads();
      for (int u = tid; u < kKeys * D / 4; u += kRows) {
        const int j = k0 + u / (D / 4), dd = u % (D / 4);
        const int64_t off = ((static_cast<int64_t>(b) * ch.len + j) * a.H + h) * (D / 4) + dd;
        const bool ok = j < n_keys;
        k_lds[u] = ok ? ksrc[off] : make_float4(0.f, 0.f, 0.f, 0.f);
        v_lds[u] = ok ? vsrc[off] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
      float s[kKeys];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D / 4; ++d) {
          const float4 kk = k_lds[j * (D / 4) + d];
          dot = fmaf(q[d].x, kk.x, dot);
          dot = fmaf(q[d].y, kk.y, dot);
          dot = fmaf(q[d].z, kk.z, dot);
          dot = fmaf(q[d].w, kk.w, dot);
        }
        const int jj = k0 + j;
        bool vis = jj < n_keys;
        if (CAUSAL) vis = vis && (jj <= i + ch.delta);
        s[j] = vis ? dot : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = expf(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int d = 0; d < D / 4; ++d) {
        acc[d].x *= alpha;
        acc[d].y *= alpha;
        acc[d].z *= alpha;
        acc[d].w *= alpha;
      }
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        const float p = expf(s[j] - m_use);
        psum += p;
#pragma unroll
        for (int d = 0; d < D / 4; ++d) {
          const float4 vv = v_lds[j * (D / 4) + d];
          acc[d].x = fmaf(p, vv.x, acc[d].x);
          acc[d].y = fmaf(p, vv.y, acc[d].y);
          acc[d].z = fmaf(p, vv.z, acc[d].z);
          acc[d].w = fmaf(p, vv.w, acc[d].w);
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
    }
  }
  if (!row_ok) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float4* dst = reinterpret_cast<float4*>(a.o) +
                ((static_cast<int64_t>(b) * a.Sq + i) * a.H + h) * (D / 4);
#pragma unroll
  for (int d = 0; d < D / 4; ++d)
    dst[d] = make_float4(acc[d].x * inv, acc[d].y * inv, acc[d].z * inv, acc[d].w * inv);
  a.lse[(static_cast<int64_t>(b) * a.H + h) * a.Sq + i] =
      l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, bool causal, hipStream_t stream) {
  const int nqt = (a.Sq + kRows - 1) / kRows;
  const dim3 grid(static_cast<uint32_t>(nqt) * a.B * a.H);
  if (causal)
    hipLaunchKernelGGL((attn_f32_kernel<D, true>), grid, dim3(kRows), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, false>), grid, dim3(kRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, bool causal, hipStream_t stream) {
  return a.D == 64 ? launch_d<64>(a, causal, stream) : launch_d<128>(a, causal, stream);
}

}  // namespace cpattn
