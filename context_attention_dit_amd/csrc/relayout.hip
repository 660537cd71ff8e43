// Ulysses sequence-shard <-> head-shard relayout for all P ranks of one group.
//
// The first Ulysses all-to-all leaves every rank holding all tokens for a
// subset of heads, and the second one regroups the attention output by token
// (Context parallelism guide (diffusers), section Ulysses Attention). With the
// transport removed, both are one permutation of contiguous runs:
//   seq2head: out[p][b][q*S_l + s][h][d] = in[q][b][s][p*H_l + h][d]
//   head2seq: out[q][b][s][p*H_l + h][d] = in[p][b][q*S_l + s][h][d]
// Each run is H_l*D contiguous elements on both sides, so the kernel is a
// streaming copy (one launch can move several tensors stored back to back,
// such as a rank's Q, K and V, which makes the transfer long enough to keep
// HBM busy): every work-item moves whole UNIT-byte words (16 bytes when
// the run length and both pointers allow it), consecutive lanes touch
// consecutive words of a run, and loads/stores are non-temporal because each
// byte is read once and written once.
#include <algorithm>

#include "cp_internal.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;           // uneven regrouping: 2 words a work-item
constexpr int kRelayoutThreads = 512;   // standard regrouping (1% faster than 256 measured)

template <int UNIT>
struct Word;
template <>
struct Word<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <>
struct Word<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <>
struct Word<4> { using T = uint32_t; };
template <>
struct Word<2> { using T = uint16_t; };

struct Geometry {
  uint32_t total;       // words in the tensor
  FastDiv run;          // words per run (H_l*D*elem/UNIT)
  FastDiv seq;          // S_local
  FastDiv batch;        // B
  FastDiv seqP;         // P*S_local: tokens of one head shard
  FastDiv P;            // ranks
};

// Head-layout word index of sequence-layout word u. Sequence layout:
// [q][b][s][p*H_l + h][d]; a row (q, b, s) holds P runs back to back. Head
// layout: [p][b][q*S_l + s][h][d].
__device__ __forceinline__ uint32_t head_index(uint32_t u, const Geometry& g) {
  const uint32_t r = g.run.div(u);           // sequence-layout run: row*P + p
  const uint32_t w = u - r * g.run.d;        // word within the run
  const uint32_t row = g.P.div(r);
  const uint32_t p = r - row * g.P.d;
  const uint32_t qb = g.seq.div(row);        // row = (q*B + b)*S_l + s
  const uint32_t s = row - qb * g.seq.d;
  const uint32_t q = g.batch.div(qb);
  const uint32_t b = qb - q * g.batch.d;
  const uint32_t h_run = (p * g.batch.d + b) * g.seqP.d + q * g.seq.d + s;
  return h_run * g.run.d + w;
}

// One word per work-item, walking the sequence-layout side in order: its
// H*D-element rows are read (seq2head) or written (head2seq) contiguously,
// and each run goes to or comes from its place in the head layout. Measured
// on the Ulysses shapes this order, at one word per work-item, beats output
// order and 2-8 words per work-item (71-83% of HBM peak against 67-79%).
template <int UNIT, bool SEQ2HEAD>
__global__ __launch_bounds__(kRelayoutThreads) void relayout_kernel(const void* __restrict__ in_,
                                                                    void* __restrict__ out_,
                                                                    Geometry g) {
  using T = typename Word<UNIT>::T;
  // blockIdx.y: which of the back-to-back tensors
  const T* in = static_cast<const T*>(in_) + static_cast<uint64_t>(blockIdx.y) * g.total;
  T* out = static_cast<T*>(out_) + static_cast<uint64_t>(blockIdx.y) * g.total;
  const uint32_t u = blockIdx.x * kRelayoutThreads + threadIdx.x;
  if (u >= g.total) return;
  const uint32_t hu = head_index(u, g);
  if (SEQ2HEAD)
    __builtin_nontemporal_store(__builtin_nontemporal_load(in + u), out + hu);
  else
    __builtin_nontemporal_store(__builtin_nontemporal_load(in + hu), out + u);
}

template <int UNIT>
hipError_t launch_unit(const void* in, void* out, const RelayoutDesc& d, hipStream_t stream) {
  const int64_t run_bytes = (d.H / d.P) * d.D * d.elem_bytes;
  const int64_t total_bytes = d.P * d.B * d.S_local * d.H * d.D * d.elem_bytes;
  Geometry g;
  g.total = static_cast<uint32_t>(total_bytes / UNIT);
  g.run.init(static_cast<uint32_t>(run_bytes / UNIT));
  g.seq.init(static_cast<uint32_t>(d.S_local));
  g.batch.init(static_cast<uint32_t>(d.B));
  g.seqP.init(static_cast<uint32_t>(d.P * d.S_local));
  g.P.init(static_cast<uint32_t>(d.P));
  const dim3 grid((g.total + kRelayoutThreads - 1) / kRelayoutThreads,
                  static_cast<uint32_t>(d.count));
  if (d.seq2head)
    hipLaunchKernelGGL((relayout_kernel<UNIT, true>), grid, dim3(kRelayoutThreads), 0, stream, in,
                       out, g);
  else
    hipLaunchKernelGGL((relayout_kernel<UNIT, false>), grid, dim3(kRelayoutThreads), 0, stream,
                       in, out, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- anything
// Every (destination group p, source shard q, batch b) pair is one 2-D copy:
// S_q rows of H_p*D elements, contiguous on the head-group side and at a row
// stride of H*D on the sequence-shard side. Only pairs with rows and heads are
// launched: block (x, y, z) takes words [512c, 512c + 512) of pair
// (act_p[x % np], act_q[y]), c = x / np, for batch z % B of tensor z / B (one
// launch can move several tensors stored back to back, such as a rank's Q, K
// and V). The destination group runs fastest in the block order, so the
// blocks dispatched together copy every group's run of the same source rows
// (whole rows of the sequence shard). A work-item moves two words, half a
// block apart (256 threads a block: measured 5% faster than one word on each
// of 512 threads on FLUX 1008 and the Wan K/V gather).
struct AnyGeometry {
  int32_t P, nq;                  // nq: shards with tokens
  FastDiv np;                     // groups with heads
  uint8_t act_p[CP_MAX_RING_CHUNKS], act_q[CP_MAX_RING_CHUNKS];
  uint32_t B, S, H, wd;           // wd: words per head row (D elements)
  uint64_t tensor_words;          // B*S*H*wd: distance between back-to-back tensors
  uint32_t s_off[CP_MAX_RING_CHUNKS + 1];
  uint32_t h_off[CP_MAX_RING_CHUNKS + 1];
  FastDiv row[CP_MAX_RING_CHUNKS];  // words per copied row of group p: H_p * wd
};

template <int UNIT, bool SEQ2HEAD>
__global__ __launch_bounds__(kThreads) void any_relayout_kernel(const void* __restrict__ in_,
                                                                void* __restrict__ out_,
                                                                AnyGeometry g) {
  using T = typename Word<UNIT>::T;
  const uint32_t tensor = blockIdx.z / g.B;
  const uint32_t b = blockIdx.z - tensor * g.B;
  const T* in = static_cast<const T*>(in_) + tensor * g.tensor_words;
  T* out = static_cast<T*>(out_) + tensor * g.tensor_words;
  const uint32_t chunk = g.np.div(blockIdx.x);
  const int p = g.act_p[blockIdx.x - chunk * g.np.d], q = g.act_q[blockIdx.y];
  const uint32_t sq = g.s_off[q + 1] - g.s_off[q];
  const uint32_t hp = g.h_off[p + 1] - g.h_off[p];
  const uint32_t row_words = hp * g.wd;
  const uint32_t n = sq * row_words;  // words of this pair and batch
  // word offsets of the pair's first element on both sides
  const uint64_t shard_base =
      (static_cast<uint64_t>(g.B) * g.s_off[q] * g.H + static_cast<uint64_t>(b) * sq * g.H +
       g.h_off[p]) * g.wd;
  const uint64_t group_base =
      (static_cast<uint64_t>(g.B) * g.S * g.h_off[p] +
       (static_cast<uint64_t>(b) * g.S + g.s_off[q]) * hp) * g.wd;
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // words u and u + kThreads of the block's 2*kThreads
    const uint32_t u = chunk * (2 * kThreads) + k * kThreads + threadIdx.x;
    if (u >= n) return;
    const uint32_t r = g.row[p].div(u), w = u - r * row_words;
    const uint64_t sh = shard_base + static_cast<uint64_t>(r) * g.H * g.wd + w;
    const uint64_t gr = group_base + u;
    if (SEQ2HEAD)
      __builtin_nontemporal_store(__builtin_nontemporal_load(in + sh), out + gr);
    else
      __builtin_nontemporal_store(__builtin_nontemporal_load(in + gr), out + sh);
  }
}

template <int UNIT>
hipError_t launch_any_unit(const void* in, void* out, const AnyRelayoutDesc& d,
                           hipStream_t stream) {
  AnyGeometry g;
  g.P = d.P;
  g.B = static_cast<uint32_t>(d.B);
  g.S = static_cast<uint32_t>(d.S);
  g.H = static_cast<uint32_t>(d.H);
  g.wd = static_cast<uint32_t>(d.D * d.elem_bytes / UNIT);
  g.tensor_words = static_cast<uint64_t>(d.B) * d.S * d.H * g.wd;
  uint64_t max_s = 0, max_h = 0;
  int np = 0, nq = 0;
  for (int r = 0; r < d.P; ++r) {
    if (d.h_off[r + 1] > d.h_off[r]) g.act_p[np++] = static_cast<uint8_t>(r);
    if (d.s_off[r + 1] > d.s_off[r]) g.act_q[nq++] = static_cast<uint8_t>(r);
  }
  g.nq = nq;
  g.np.init(static_cast<uint32_t>(np));
  for (int r = 0; r <= d.P; ++r) {
    g.s_off[r] = static_cast<uint32_t>(d.s_off[r]);
    g.h_off[r] = static_cast<uint32_t>(d.h_off[r]);
  }
  for (int r = 0; r < d.P; ++r) {
    const uint32_t hp = g.h_off[r + 1] - g.h_off[r];
    g.row[r].init(hp > 0 ? hp * g.wd : 1u);
    max_s = std::max<uint64_t>(max_s, g.s_off[r + 1] - g.s_off[r]);
    max_h = std::max<uint64_t>(max_h, hp);
  }
  const uint64_t max_words = max_s * max_h * g.wd;
  const uint32_t per_block = 2 * kThreads;
  // (the caller guarantees S > 0 and H > 0, so np, nq >= 1)
  const dim3 grid(static_cast<uint32_t>((max_words + per_block - 1) / per_block * np),
                  static_cast<uint32_t>(nq), static_cast<uint32_t>(g.B * d.count));
  if (d.seq2head)
    hipLaunchKernelGGL((any_relayout_kernel<UNIT, true>), grid, dim3(kThreads), 0, stream, in,
                       out, g);
  else
    hipLaunchKernelGGL((any_relayout_kernel<UNIT, false>), grid, dim3(kThreads), 0, stream, in,
                       out, g);
  return hipGetLastError();
}

}  // namespace

// Widest word that divides a head row (D elements) and both base addresses.
int any_relayout_word_bytes(const void* in, void* out, const AnyRelayoutDesc& d) {
  const int64_t row_bytes = d.D * d.elem_bytes;
  const uintptr_t align = reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out);
  for (int w = 16; w > 2; w /= 2)
    if (row_bytes % w == 0 && align % w == 0) return w;
  return 2;
}

// The caller has checked: 1 <= P <= CP_MAX_RING_CHUNKS, every pair's words
// and the grid fit 32 bits, B*count < 65536.
hipError_t launch_any_relayout(const void* in, void* out, const AnyRelayoutDesc& d,
                               hipStream_t stream) {
  switch (any_relayout_word_bytes(in, out, d)) {
    case 16: return launch_any_unit<16>(in, out, d, stream);
    case 8: return launch_any_unit<8>(in, out, d, stream);
    case 4: return launch_any_unit<4>(in, out, d, stream);
    default: return launch_any_unit<2>(in, out, d, stream);
  }
}

// ---------------------------------------------------------------- key-contiguous V
// seq2head of the value tensor into out[p][b][h][t / 64][d][t % 64], t = q*S_l
// + s over the head shard's T = P*S_l tokens: per (group, batch, head) a
// transpose of (token, feature) in tiles of 64 tokens, each tile one
// contiguous 16 KB block, so that attention copies a tile of V in the order the
// P*V product reads it. Columns past T in the last tile are written as zeros.
// A block of 256 threads takes 128 tokens (two tiles) x 128 features of one
// (p, b, h) through LDS: 16 lanes read one token's 256-byte row (8 16-byte
// units a thread), and each thread forms two features' 8-token units from 8
// 4-byte LDS reads and byte permutes; a block writes its two tiles whole. LDS rows hold 64 words; word w of token r sits at
// w ^ (4 (r / 8 mod 16)), so the 16 rows r, r + 8, ... that one read phase
// touches fall in distinct banks, and a row's 16-byte units stay whole.
// Blocks walk the tokens fastest: neighbouring blocks read neighbouring rows
// and extend the same output rows.
struct VtGeometry {
  uint32_t T;         // tokens per head shard (P * S_l)
  FastDiv seq;        // S_l
  uint32_t B, H, H_l;
  uint32_t tiles;     // ceil(T / 64): 64-token tiles per (p, b, h)
  uint32_t tblocks;   // ceil(T / 128)
  uint32_t blocks;    // P * B * H_l * tblocks
};

__global__ __launch_bounds__(256) void seq2head_vt_kernel(const uint16_t* __restrict__ in,
                                                          uint16_t* __restrict__ out,
                                                          VtGeometry g) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) uint32_t tile[128 * 64];
  const uint32_t blk = blockIdx.x;
  uint32_t r = blk;
  const uint32_t tb = r % g.tblocks;
  r /= g.tblocks;
  const uint32_t h = r % g.H_l;
  r /= g.H_l;
  const uint32_t b = r % g.B;
  const uint32_t p = r / g.B;
  const uint32_t t_base = tb * 128;
  const uint64_t head_col = static_cast<uint64_t>(p) * g.H_l + h;
  const int tid = threadIdx.x;
  // load: unit k = tid + 256 i is token k / 16, feature unit k % 16
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = tid + 256 * i;
    const int tok = k >> 4, fu = k & 15;
    const uint32_t t = t_base + tok;
    u32x4 x = u32x4{0, 0, 0, 0};
    if (t < g.T) {
      const uint32_t q = g.seq.div(t);
      const uint32_t s = t - q * g.seq.d;
      const uint64_t row = (static_cast<uint64_t>(q) * g.B + b) * g.seq.d + s;
      x = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(in + (row * g.H + head_col) * D + 8 * fu));
    }
    *reinterpret_cast<u32x4*>(&tile[tok * 64 + ((4 * fu) ^ (4 * ((tok >> 3) & 15)))]) = x;
  }
  __syncthreads();
  // store: work-item k = tid + 256 i is feature pair k / 16, token unit k % 16
  uint16_t* obase = out + ((static_cast<uint64_t>(p) * g.B + b) * g.H_l + h) * g.tiles * D * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = tid + 256 * i;
    const int fp = k >> 4, tu = k & 15;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = tile[(8 * tu + j) * 64 + (fp ^ (4 * tu))];
    const uint32_t t0 = t_base + 8 * tu;
    const uint32_t tile = t0 >> 6;
    if (tile >= g.tiles) continue;   // the block's second tile lies past T
    uint16_t* tbase = obase + static_cast<uint64_t>(tile) * D * 64 + (t0 & 63);
#pragma unroll
    for (int e = 0; e < 2; ++e) {   // feature 2 fp + e: the low (e = 0) or high halves
      const uint32_t sel = e ? 0x07060302u : 0x05040100u;
      u32x4 y;
#pragma unroll
      for (int m = 0; m < 4; ++m) y[m] = __builtin_amdgcn_perm(w[2 * m + 1], w[2 * m], sel);
      __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(tbase + (2 * fp + e) * 64));
    }
  }
}

// The caller has checked: 2-byte elements, D = 128, 16-byte aligned pointers,
// fewer than 2^31 tokens and blocks. `groups` head groups (P for the Ulysses
// regrouping; 1 for the K/V all-gather's unpack, which gives every head all
// P*S_local tokens).
hipError_t launch_seq2head_vt(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                              int64_t H, int64_t D, int64_t groups, hipStream_t stream) {
  (void)D;
  VtGeometry g;
  g.T = static_cast<uint32_t>(P * S_local);
  g.seq.init(static_cast<uint32_t>(S_local));
  g.B = static_cast<uint32_t>(B);
  g.H = static_cast<uint32_t>(H);
  g.H_l = static_cast<uint32_t>(H / groups);
  g.tiles = (g.T + 63) / 64;
  g.tblocks = (g.T + 127) / 128;
  g.blocks = static_cast<uint32_t>(B * H * g.tblocks);
  hipLaunchKernelGGL(seq2head_vt_kernel, dim3(g.blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), g);
  return hipGetLastError();
}

// Widest word that divides the run length and both base addresses.
int relayout_word_bytes(const void* in, void* out, const RelayoutDesc& d) {
  const int64_t run_bytes = (d.H / d.P) * d.D * d.elem_bytes;
  const uintptr_t align = reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out);
  for (int w = 16; w > 2; w /= 2)
    if (run_bytes % w == 0 && align % w == 0) return w;
  return 2;
}

// The caller has checked that the tensor holds fewer than 2^31 words.
hipError_t launch_relayout(const void* in, void* out, const RelayoutDesc& d, hipStream_t stream) {
  switch (relayout_word_bytes(in, out, d)) {
    case 16: return launch_unit<16>(in, out, d, stream);
    case 8: return launch_unit<8>(in, out, d, stream);
    case 4: return launch_unit<4>(in, out, d, stream);
    default: return launch_unit<2>(in, out, d, stream);
  }
}

}  // namespace cpattn
