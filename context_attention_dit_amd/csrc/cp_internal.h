// Internal declarations shared by the HIP translation units of libcpattn.
// Not part of the public ABI (include/cp_attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cp_attn.h"

namespace cpattn {

// Unsigned 32-bit division by a divisor fixed at launch time, as a multiply
// and shifts (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (t + ((n - t) >> 1)) >> (l - 1)
// where t = mulhi(n, m), exact for every 32-bit n. d == 1 is special-cased.
struct FastDiv {
  uint32_t d;
  uint32_t mul;
  uint32_t shift;  // l - 1 (unused when d == 1)
  __host__ void init(uint32_t div) {
    d = div;
    uint32_t l = 0;
    while ((1ull << l) < div) ++l;
    shift = l == 0 ? 0 : l - 1;
    mul = static_cast<uint32_t>(((1ull << 32) * ((1ull << l) - div)) / div + 1);
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    if (d == 1) return n;
    uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(n) * mul) >> 32);
    return (t + ((n - t) >> 1)) >> shift;
  }
};

// ----- relayout (relayout.hip)
struct RelayoutDesc {
  int64_t P, B, S_local, H, D;
  int elem_bytes;
  bool seq2head;
  int64_t count = 1;  // tensors stored back to back in `in` and in `out`
};
int relayout_word_bytes(const void* in, void* out, const RelayoutDesc& d);
hipError_t launch_relayout(const void* in, void* out, const RelayoutDesc& d, hipStream_t stream);
// seq2head of a bf16 value tensor into [P][B][H/P][ceil(P*S_local/64)][D][64]
// (keys contiguous in 64-key tiles, zero padding past P*S_local)
// (groups = P), or the K/V all-gather's unpack of P equal shards (groups = 1)
hipError_t launch_seq2head_vt(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                              int64_t H, int64_t D, int64_t groups, hipStream_t stream);

// Ulysses Anything: uneven per-rank token counts and head counts. The P
// sequence shards (shard q = [B][S_q][H][D]) and the P head groups (group p
// = [B][S][H_p][D]) are each packed back to back in rank order.
struct AnyRelayoutDesc {
  int32_t P;
  int64_t B, S, H, D;
  int elem_bytes;
  bool seq2head;
  int64_t s_off[CP_MAX_RING_CHUNKS + 1];  // token offsets: shard q = [s_off[q], s_off[q+1])
  int64_t h_off[CP_MAX_RING_CHUNKS + 1];  // head offsets: group p = [h_off[p], h_off[p+1])
  int64_t count = 1;                      // tensors stored back to back
};
int any_relayout_word_bytes(const void* in, void* out, const AnyRelayoutDesc& d);
hipError_t launch_any_relayout(const void* in, void* out, const AnyRelayoutDesc& d,
                               hipStream_t stream);

// ----- merge (lse_merge.hip)
// lse_stride: row stride of the output LSE per (batch, head), at least Sq
// (0 means Sq); the partials' LSE is compact ([P][B][H][Sq]).
hipError_t launch_lse_merge(const float* o_parts, const float* lse_parts, int P, void* o,
                            float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D, bool out_bf16,
                            hipStream_t stream, int64_t lse_stride = 0);
// The same merge over the rows of a range of (batch*head, `rows`-row query
// tile) units [unit0, unit0 + units), ceil(Sq/rows) tiles per head, with the
// compact partial layout of AttnArgs::pp_split. O is [B][Sq][H][D], LSE
// [B][H][lse_stride] (0: Sq).
hipError_t launch_unit_merge(const float* o_parts, const float* lse_parts, int P, void* o,
                             float* lse, int64_t H, int64_t Sq, int64_t D, int64_t rows,
                             int64_t unit0, int64_t units, bool out_bf16, hipStream_t stream,
                             int64_t lse_stride);

// ----- attention (attn_bf16.hip, attn_f32.hip)
struct ChunkDesc {
  const void* k;
  const void* v;
  int32_t len;
  int32_t delta;  // q_pos0 - chunk pos0, clamped to [-(Sq+1), len+1]
};

struct AttnArgs {
  const void* q;
  void* o;
  float* lse;
  int32_t B, H, Sq, D;
  float scale;
  int32_t nchunks;
  // Split of each query tile's key range over `nsplit` blocks (1 = none). With
  // nsplit > 1 every split writes a normalised fp32 partial (O, LSE) to
  // part_o [nsplit][B][Sq][H][D] / part_lse [nsplit][B][H][Sq], and the
  // launcher merges them into o / lse.
  int32_t nsplit;
  float* part_o;
  float* part_lse;
  // bf16 kernel: 1 = four waves per query tile; 2 = eight waves per query tile,
  // its keys split between two groups and merged in LDS (no workspace)
  int32_t groups;
  // bf16 kernel: row stride of the output LSE per (batch, head); 0 means Sq.
  // A launch over a window of a longer query shard (B = 1: q and o offset to
  // the window's first row, lse to its first column) writes its LSE into the
  // shard's [H][S] array with this stride.
  int32_t lse_stride;
  // Non-causal ping-pong kernels: the flat range [unit0, unit0 + units) of
  // the (batch*head, query tile) units this launch covers, in the kernel's
  // own query tiling (units = 0: all of them)
  int32_t unit0, units;
  // Non-causal one-chunk ping-pong kernel at D = 128: split each unit's key
  // tiles over this many blocks (<= 1: none). The splits write normalised fp32
  // partials in a compact per-unit layout, part_o [split][unit - unit0][256][D]
  // and part_lse [split][unit - unit0][256], which launch_unit_merge combines.
  int32_t pp_split;
  // Ring launches: when the last round of 256-row ping-pong blocks would be
  // at most half full, split its units' keys this many ways (partials in
  // part_o / part_lse as above, merged after); <= 1: the two-group plan
  int32_t last_split;
  // bf16 kernel: 1 = chunk 0's v is key-contiguous in 64-key tiles,
  // [B][H][ceil(len/64)][D][64] (one chunk, D = 128, no key splits);
  // 0 = [B][len][H][D] like k
  int32_t vt;
  ChunkDesc chunks[CP_MAX_RING_CHUNKS];
};

// Number of key splits the bf16 attention launcher uses for these sizes
// (non-causal only; 1 when the grid already fills the GPU). `tiles` is the
// number of 64-key tiles each query tile visits.
int attn_split_count(int64_t B, int64_t H, int64_t Sq, int64_t tiles, bool causal);
// Groups per block (1 or 2) of the bf16 kernel: 2 when there are no more
// query tiles than CUs and at least 4 key tiles to split.
int attn_groups(int64_t B, int64_t H, int64_t Sq, int64_t tiles);
// Non-causal single-batch grids just past the CU count whose last query tile
// is short (at most 32 rows): the full query tiles then fill the CUs once as
// two-group blocks, and the last tile's rows get a launch of their own with
// their keys split this many ways (merged after). 0 when the plan does not
// apply.
int attn_tail_splits(int64_t B, int64_t H, int64_t Sq, int64_t tiles, bool causal);
// fp32 elements of partial output the split needs: nsplit*(B*Sq*H*D + B*H*Sq).
int64_t attn_split_floats(int64_t nsplit, int64_t B, int64_t H, int64_t Sq, int64_t D);
// Key splits of the last round's units (see AttnArgs::last_split) for a
// non-causal one-chunk bf16 call with these sizes; 0 when the plan does not
// apply. Its partials take attn_last_split_floats(...) fp32 elements.
int attn_last_splits(int64_t B, int64_t H, int64_t Sq, int64_t D, int64_t tiles, bool causal);
int64_t attn_last_split_floats(int64_t B, int64_t H, int64_t Sq, int64_t D, int64_t tiles,
                               bool causal);

// ----- backward (attn_bwd.hip)
struct BwdChunk {
  const __bf16* k;  // [B][len][H][D]
  const __bf16* v;
  float* dk;        // [B][len][H][D]: this Q shard's share of the chunk's gradients
  float* dv;
  int32_t len;
  int32_t diag;   // causal: key j visible to query i iff j <= i + diag (clamped like ChunkDesc)
  int32_t tile0;  // 128-key tiles of the chunks before this one
  int32_t pad;
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* dout;
  const float* lse;    // [B][H][Sq], the full rows' LSE
  const float* delta;  // [B][H][Sq], <dO_i, O_i>
  float* dq;           // [B][Sq][H][D]
  int32_t B, H, Sq;
  float scale;
  int32_t accum_dq, accum_dkv;  // add into dq / dk, dv instead of overwriting
  int32_t nchunks;
  int32_t total_kt;  // 128-key tiles over all chunks
  int32_t groups;    // dQ kernel: 1, or 2 (two groups of 4 waves split the key tiles)
  int32_t dq_blocks;  // set by the launcher: dQ blocks at the front of a fused grid
  BwdChunk chunks[CP_MAX_RING_CHUNKS];
};
// Groups per block (1 or 2) of the dQ kernel for these sizes.
int bwd_dq_groups(int64_t B, int64_t H, int64_t Sq, int64_t key_tiles);
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int D, bool causal, hipStream_t stream);
// fp32 inputs (the __bf16 pointers of BwdArgs then hold fp32 tensors).
hipError_t launch_attn_bwd_f32(const BwdArgs& a, int D, bool causal, hipStream_t stream);
hipError_t launch_bwd_delta(const void* o, const void* dout, float* delta, int64_t B, int64_t H,
                            int64_t Sq, int64_t D, bool bf16, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cus();

// out_bf16: write O as bf16 (else fp32). causal: position-based masking.
hipError_t launch_attn_bf16(const AttnArgs& a, bool causal, bool out_bf16, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, bool causal, hipStream_t stream);

}  // namespace cpattn
