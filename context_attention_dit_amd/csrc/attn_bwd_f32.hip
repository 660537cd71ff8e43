// fp32 backward of block-wise softmax attention over a list of K/V chunks
// (fp32 in, fp32 gradients).
//
// The same gradients as the bf16 MFMA backward (derivatives of
// O = softmax(scale Q K^T) V against dO, from the saved LSE and
// Delta_i = <dO_i, O_i>; Ulysses Sequence Parallelism article, detailed
// notes 2, and the Context parallelism guide (diffusers), section Ring
// Attention, for the split by chunk), with every step in fp32 so the result
// stays within fp32 rounding of the exact gradients. It is the small-size,
// full-precision companion of the bf16 kernels: one lane owns one row, and the
// rows it pairs with are staged in LDS and read as broadcasts.
//  * dq kernel: lane = query row; it walks every chunk's keys and accumulates
//    dQ_i = scale sum_j dS_ij k_j.
//  * dkdv kernel: lane = key row of one chunk; it walks the query rows and
//    accumulates dV_j = sum_i P_ij dO_i and dK_j = scale sum_i dS_ij q_i.
// Each output element is written once by one lane (no atomics).
#include "cp_internal.h"

namespace cpattn {
namespace {

constexpr int kRows = 64;  // rows per block, one per lane
constexpr int kPair = 32;  // rows of the other side per LDS tile

template <int D>
__device__ __forceinline__ float dot4(const float4* x, const float4* y) {
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < D / 4; ++d) {
    const float4 a = x[d], b = y[d];
    s = fmaf(a.x, b.x, s);
    s = fmaf(a.y, b.y, s);
    s = fmaf(a.z, b.z, s);
    s = fmaf(a.w, b.w, s);
  }
  return s;
}

template <int D>
__device__ __forceinline__ void axpy4(float w, const float4* x, float4* acc) {
#pragma unroll
  for (int d = 0; d < D / 4; ++d) {
    const float4 a = x[d];
    acc[d].x = fmaf(w, a.x, acc[d].x);
    acc[d].y = fmaf(w, a.y, acc[d].y);
    acc[d].z = fmaf(w, a.z, acc[d].z);
    acc[d].w = fmaf(w, a.w, acc[d].w);
  }
}

template <int D>
__device__ __forceinline__ void store_row(float4* dst, const float4* acc, float s, bool add) {
#pragma unroll
  for (int d = 0; d < D / 4; ++d) {
    float4 r = make_float4(s * acc[d].x, s * acc[d].y, s * acc[d].z, s * acc[d].w);
    if (add) {
      const float4 o = dst[d];
      r.x += o.x;
      r.y += o.y;
      r.z += o.z;
      r.w += o.w;
    }
    dst[d] = r;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_f32_dq_kernel(BwdArgs a) {
  __shared__ float4 k_lds[kPair * D / 4];
  __shared__ float4 v_lds[kPair * D / 4];
  const int tid = threadIdx.x;
  const int nqt = (a.Sq + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqt;
  const int qt = blockIdx.x - bh * nqt;
  const int b = bh / a.H, h = bh - b * a.H;
  const int i = qt * kRows + tid;
  const bool row_ok = i < a.Sq;
  const int ic = row_ok ? i : 0;
  const int64_t qrow = (static_cast<int64_t>(b) * a.Sq + ic) * a.H + h;
  const float4* qs = reinterpret_cast<const float4*>(a.q) + qrow * (D / 4);
  const float4* ds = reinterpret_cast<const float4*>(a.dout) + qrow * (D / 4);
  float4 q[D / 4], dout[D / 4], acc[D / 4];
#pragma unroll
  for (int d = 0; d < D / 4; ++d) {
    q[d] = qs[d];
    dout[d] = ds[d];
    acc[d] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int64_t lrow = (static_cast<int64_t>(b) * a.H + h) * a.Sq + ic;
  const float lse = a.lse[lrow], dlt = a.delta[lrow];
  const bool live = row_ok && lse != -INFINITY;  // a row that saw no key has zero weights
  const int q_last = min(qt * kRows + kRows - 1, a.Sq - 1);

  for (int c = 0; c < a.nchunks; ++c) {
    const BwdChunk ch = a.chunks[c];
    int n_keys = ch.len;
    if (CAUSAL) n_keys = max(0, min(n_keys, q_last + ch.diag + 1));
    const float4* ksrc = reinterpret_cast<const float4*>(ch.k);
    const float4* vsrc = reinterpret_cast<const float4*>(ch.v);
    for (int k0 = 0; k0 < n_keys; k0 += kPair) {
      __syncthreads();
      for (int u = tid; u < kPair * D / 4; u += kRows) {
        const int j = k0 + u / (D / 4), dd = u % (D / 4);
        const int64_t off = ((static_cast<int64_t>(b) * ch.len + j) * a.H + h) * (D / 4) + dd;
        const bool ok = j < n_keys;
        k_lds[u] = ok ? ksrc[off] : make_float4(0.f, 0.f, 0.f, 0.f);
        v_lds[u] = ok ? vsrc[off] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
      for (int j = 0; j < kPair; ++j) {
        const int jj = k0 + j;
        bool vis = live && jj < n_keys;
        if (CAUSAL) vis = vis && jj <= i + ch.diag;
        const float s = a.scale * dot4<D>(q, &k_lds[j * (D / 4)]);
        const float p = vis ? expf(s - lse) : 0.f;
        const float dp = dot4<D>(dout, &v_lds[j * (D / 4)]);
        axpy4<D>(p * (dp - dlt), &k_lds[j * (D / 4)], acc);
      }
    }
  }
  if (!row_ok) return;
  store_row<D>(reinterpret_cast<float4*>(a.dq) + qrow * (D / 4), acc, a.scale, a.accum_dq != 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void bwd_f32_dkdv_kernel(BwdArgs a) {
  __shared__ float4 q_lds[kPair * D / 4];
  __shared__ float4 d_lds[kPair * D / 4];
  __shared__ float l_lds[kPair], t_lds[kPair];
  const int tid = threadIdx.x;
  // block -> (batch*head, key tile of kRows keys over all chunks)
  int ntile = 0;
  for (int c = 0; c < a.nchunks; ++c) ntile += (a.chunks[c].len + kRows - 1) / kRows;
  const int bh = blockIdx.x / ntile;
  int t = blockIdx.x - bh * ntile, c = 0;
  while (t >= (a.chunks[c].len + kRows - 1) / kRows) {
    t -= (a.chunks[c].len + kRows - 1) / kRows;
    ++c;
  }
  const BwdChunk ch = a.chunks[c];
  const int b = bh / a.H, h = bh - b * a.H;
  const int j = t * kRows + tid;
  const bool key_ok = j < ch.len;
  const int64_t krow = (static_cast<int64_t>(b) * ch.len + (key_ok ? j : 0)) * a.H + h;
  const float4* ks = reinterpret_cast<const float4*>(ch.k) + krow * (D / 4);
  const float4* vs = reinterpret_cast<const float4*>(ch.v) + krow * (D / 4);
  float4 k[D / 4], v[D / 4], dk[D / 4], dv[D / 4];
#pragma unroll
  for (int d = 0; d < D / 4; ++d) {
    k[d] = ks[d];
    v[d] = vs[d];
    dk[d] = make_float4(0.f, 0.f, 0.f, 0.f);
    dv[d] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float4* qsrc = reinterpret_cast<const float4*>(a.q);
  const float4* dsrc = reinterpret_cast<const float4*>(a.dout);
  const int64_t lbase = (static_cast<int64_t>(b) * a.H + h) * a.Sq;
  int i0 = 0;  // first query row that can see this block's first key
  if (CAUSAL) i0 = max(0, t * kRows - ch.diag) / kPair * kPair;
  for (; i0 < a.Sq; i0 += kPair) {
    __syncthreads();
    for (int u = tid; u < kPair * D / 4; u += kRows) {
      const int i = i0 + u / (D / 4), dd = u % (D / 4);
      const int64_t off = ((static_cast<int64_t>(b) * a.Sq + i) * a.H + h) * (D / 4) + dd;
      const bool ok = i < a.Sq;
      q_lds[u] = ok ? qsrc[off] : make_float4(0.f, 0.f, 0.f, 0.f);
      d_lds[u] = ok ? dsrc[off] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < kPair) {
      const bool ok = i0 + tid < a.Sq;
      l_lds[tid] = ok ? a.lse[lbase + i0 + tid] : -INFINITY;
      t_lds[tid] = ok ? a.delta[lbase + i0 + tid] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < kPair; ++r) {
      const int i = i0 + r;
      const float lse = l_lds[r];
      bool vis = key_ok && lse != -INFINITY;  // rows past Sq carry -inf
      if (CAUSAL) vis = vis && j <= i + ch.diag;
      const float s = a.scale * dot4<D>(&q_lds[r * (D / 4)], k);
      const float p = vis ? expf(s - lse) : 0.f;
      const float dp = dot4<D>(&d_lds[r * (D / 4)], v);
      axpy4<D>(p, &d_lds[r * (D / 4)], dv);
      axpy4<D>(p * (dp - t_lds[r]), &q_lds[r * (D / 4)], dk);
    }
  }
  if (!key_ok) return;
  const bool add = a.accum_dkv != 0;
  store_row<D>(reinterpret_cast<float4*>(ch.dk) + krow * (D / 4), dk, a.scale, add);
  store_row<D>(reinterpret_cast<float4*>(ch.dv) + krow * (D / 4), dv, 1.f, add);
}

template <int D, bool CAUSAL>
hipError_t launch_t(const BwdArgs& a, hipStream_t stream) {
  const int64_t BH = static_cast<int64_t>(a.B) * a.H;
  int64_t kv_tiles = 0;
  for (int c = 0; c < a.nchunks; ++c) kv_tiles += (a.chunks[c].len + kRows - 1) / kRows;
  if (kv_tiles > 0 && BH > 0) {
    hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, CAUSAL>),
                       dim3(static_cast<uint32_t>(kv_tiles * BH)), dim3(kRows), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nqt = (a.Sq + kRows - 1) / kRows;
  if (nqt * BH == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_f32_dq_kernel<D, CAUSAL>), dim3(static_cast<uint32_t>(nqt * BH)),
                     dim3(kRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_f32(const BwdArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 64) return causal ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return causal ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
}

}  // namespace cpattn
