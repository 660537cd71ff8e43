// extern "C" entry points of libcpattn: argument validation and dispatch.
//
// Every argument is checked on the host before anything is enqueued, so a
// rejected call leaves all outputs untouched (the standard context-parallel
// modes fail on sizes they cannot split instead of padding silently:
// Context parallelism guide (diffusers), variant table and the 1008x1008
// benchmark rows). No entry point allocates device memory.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "cp_internal.h"

namespace {

thread_local std::string g_err;

cp_status fail(cp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

cp_status ok() {
  g_err.clear();
  return CP_OK;
}

cp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CP_E_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

int elem_size(cp_dtype t) { return t == CP_BF16 ? 2 : 4; }
bool valid_dtype(int t) { return t == CP_BF16 || t == CP_F32; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

// Product of non-negative sizes, saturated at INT64_MAX (no overflow).
int64_t sat_mul(std::initializer_list<int64_t> xs) {
  __int128 p = 1;
  for (int64_t x : xs) {
    p *= x;
    if (p > INT64_MAX) return INT64_MAX;
  }
  return static_cast<int64_t>(p);
}

constexpr int64_t kMaxSeq = int64_t(1) << 30;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

// Checks shared by the attention entry points. Returns CP_OK or an error.
cp_status check_attn_common(const char* fn, int64_t B, int64_t H, int64_t Sq, int64_t D,
                            int in_dtype, int causal, float scale) {
  if (B < 0 || H < 0 || Sq < 0 || D < 0)
    return fail(CP_E_INVALID, "%s: negative size (B=%lld H=%lld Sq=%lld D=%lld)", fn,
                (long long)B, (long long)H, (long long)Sq, (long long)D);
  if (!valid_dtype(in_dtype)) return fail(CP_E_INVALID, "%s: unknown dtype %d", fn, in_dtype);
  if (causal != 0 && causal != 1) return fail(CP_E_INVALID, "%s: causal must be 0 or 1", fn);
  if (!std::isfinite(scale)) return fail(CP_E_INVALID, "%s: scale must be finite", fn);
  if (D != 64 && D != 128)
    return fail(CP_E_UNSUPPORTED, "%s: head dim D=%lld not built (64 or 128)", fn, (long long)D);
  if (Sq >= kMaxSeq) return fail(CP_E_UNSUPPORTED, "%s: Sq=%lld exceeds 2^30", fn, (long long)Sq);
  // the kernels address a 64-key tile with 32-bit offsets: 64*H*D < 2^31
  if (H > (int64_t(1) << 24) / D)
    return fail(CP_E_UNSUPPORTED, "%s: H*D=%lld exceeds 2^24", fn, (long long)(H * D));
  // query tiles x batch x heads must fit one launch grid (64-row tiles worst case)
  if (sat_mul({(Sq + 63) / 64, B, H}) > kMaxGrid / 8)
    return fail(CP_E_UNSUPPORTED, "%s: B*H*Sq too large for one launch", fn);
  return CP_OK;
}

int32_t clamp_delta(int64_t q_pos0, int64_t kv_pos0, int64_t Sq, int64_t len) {
  // key j visible to query i iff j <= i + delta; clamping to [-(Sq+1), len+1]
  // changes no visibility decision for 0 <= i < Sq, 0 <= j < len.
  const int64_t lo = -(Sq + 1), hi = len + 1;
  // q_pos0 - kv_pos0 without overflow
  if (q_pos0 >= 0 && kv_pos0 < 0 && q_pos0 > INT64_MAX + kv_pos0) return static_cast<int32_t>(hi);
  if (q_pos0 < 0 && kv_pos0 > 0 && q_pos0 < INT64_MIN + kv_pos0) return static_cast<int32_t>(lo);
  int64_t d = q_pos0 - kv_pos0;
  if (d < lo) d = lo;
  if (d > hi) d = hi;
  return static_cast<int32_t>(d);
}

cp_status launch_attention(const char* fn, const cpattn::AttnArgs& a, cp_dtype in_dtype,
                           bool out_bf16, int causal, hipStream_t stream) {
  hipError_t e = in_dtype == CP_BF16 ? cpattn::launch_attn_bf16(a, causal != 0, out_bf16, stream)
                                     : cpattn::launch_attn_f32(a, causal != 0, stream);
  return hip_status(e, fn);
}

}  // namespace

extern "C" {

int cp_abi_version(void) { return CP_ATTN_ABI_VERSION; }

const char* cp_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

// One chunk's attention; vt: v is key-contiguous per head, [B][H][D][Skv]
cp_status chunk_partial(const char* fn, const void* q, const void* k, const void* v, void* o,
                        float* lse, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                        cp_dtype in_dtype, cp_dtype o_dtype, float scale, int causal,
                        int64_t q_pos0, int64_t kv_pos0, void* stream, bool vt) {
  cp_status s = check_attn_common(fn, B, H, Sq, D, in_dtype, causal, scale);
  if (s != CP_OK) return s;
  if (Skv < 0) return fail(CP_E_INVALID, "%s: negative Skv", fn);
  if (Skv >= kMaxSeq) return fail(CP_E_UNSUPPORTED, "%s: Skv exceeds 2^30", fn);
  if (!valid_dtype(o_dtype)) return fail(CP_E_INVALID, "%s: unknown o_dtype %d", fn, o_dtype);
  if (in_dtype == CP_F32 && o_dtype != CP_F32)
    return fail(CP_E_UNSUPPORTED, "%s: fp32 inputs give fp32 outputs only", fn);
  if (vt && (in_dtype != CP_BF16 || D != 128))
    return fail(CP_E_UNSUPPORTED, "%s: key-contiguous V needs bf16 inputs and D = 128", fn);
  if (B == 0 || H == 0 || Sq == 0) return ok();
  const int64_t es = elem_size(in_dtype);
  const int64_t q_bytes = sat_mul({B, Sq, H, D, es}), kv_bytes = sat_mul({B, Skv, H, D, es});
  // key-contiguous V: [B][H][ceil(Skv/64)][D][64]
  const int64_t v_bytes = vt ? sat_mul({B, H, (Skv + 63) / 64, D, 64, es}) : kv_bytes;
  const int64_t o_bytes = sat_mul({B, Sq, H, D, elem_size(o_dtype)});
  const int64_t l_bytes = sat_mul({B, H, Sq, 4});
  if (!q || !o || !lse || (Skv > 0 && (!k || !v)))
    return fail(CP_E_INVALID, "%s: null pointer", fn);
  if (!aligned(q, 16) || !aligned(o, 16) || (Skv > 0 && (!aligned(k, 16) || !aligned(v, 16))) ||
      !aligned(lse, 4))
    return fail(CP_E_INVALID, "%s: misaligned pointer (tensors need 16 B, lse 4 B)", fn);
  if (overlap(o, o_bytes, q, q_bytes) || overlap(o, o_bytes, k, kv_bytes) ||
      overlap(o, o_bytes, v, v_bytes) || overlap(o, o_bytes, lse, l_bytes) ||
      overlap(lse, l_bytes, q, q_bytes) || overlap(lse, l_bytes, k, kv_bytes) ||
      overlap(lse, l_bytes, v, v_bytes))
    return fail(CP_E_INVALID, "%s: outputs overlap inputs or each other", fn);

  cpattn::AttnArgs a{};
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.B = static_cast<int32_t>(B);
  a.H = static_cast<int32_t>(H);
  a.Sq = static_cast<int32_t>(Sq);
  a.D = static_cast<int32_t>(D);
  a.scale = scale;
  a.nchunks = 1;
  a.nsplit = 1;
  a.groups = in_dtype == CP_BF16 ? cpattn::attn_groups(B, H, Sq, (Skv + 63) / 64) : 1;
  a.chunks[0].k = k;
  a.chunks[0].v = v;
  a.chunks[0].len = static_cast<int32_t>(Skv);
  a.chunks[0].delta = clamp_delta(q_pos0, kv_pos0, Sq, Skv);
  a.vt = vt ? 1 : 0;
  return launch_attention(fn, a, in_dtype, o_dtype == CP_BF16, causal,
                          static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

cp_status cp_attn_chunk_partial(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                cp_dtype in_dtype, cp_dtype o_dtype, float scale, int causal,
                                int64_t q_pos0, int64_t kv_pos0, void* stream) {
  return chunk_partial("cp_attn_chunk_partial", q, k, v, o, lse, B, H, Sq, Skv, D, in_dtype,
                       o_dtype, scale, causal, q_pos0, kv_pos0, stream, false);
}

cp_status cp_attn_chunk_partial_vt(const void* q, const void* k, const void* vt, void* o,
                                   float* lse, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                   int64_t D, cp_dtype in_dtype, cp_dtype o_dtype, float scale,
                                   int causal, int64_t q_pos0, int64_t kv_pos0, void* stream) {
  return chunk_partial("cp_attn_chunk_partial_vt", q, k, vt, o, lse, B, H, Sq, Skv, D, in_dtype,
                       o_dtype, scale, causal, q_pos0, kv_pos0, stream, true);
}

cp_status cp_lse_merge(const float* o_parts, const float* lse_parts, int64_t P, void* o,
                       float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D, cp_dtype o_dtype,
                       void* stream) {
  const char* fn = "cp_lse_merge";
  if (P < 1) return fail(CP_E_INVALID, "%s: P must be >= 1", fn);
  if (P >= kMaxGrid) return fail(CP_E_UNSUPPORTED, "%s: P too large", fn);
  if (B < 0 || H < 0 || Sq < 0 || D < 0) return fail(CP_E_INVALID, "%s: negative size", fn);
  if (!valid_dtype(o_dtype)) return fail(CP_E_INVALID, "%s: unknown o_dtype %d", fn, o_dtype);
  if (D % 4 != 0) return fail(CP_E_UNSUPPORTED, "%s: D=%lld is not a multiple of 4", fn,
                              (long long)D);
  if (D > 4096) return fail(CP_E_UNSUPPORTED, "%s: D=%lld exceeds 4096", fn, (long long)D);
  if (B == 0 || H == 0 || Sq == 0 || D == 0) return ok();
  if (sat_mul({B, Sq, H, D / 4}) >= kMaxGrid || sat_mul({P, B, Sq, H, D, 4}) >= INT64_MAX / 2)
    return fail(CP_E_UNSUPPORTED, "%s: tensor too large for one launch", fn);
  if (!o_parts || !lse_parts || !o || !lse) return fail(CP_E_INVALID, "%s: null pointer", fn);
  if (!aligned(o_parts, 16) || !aligned(o, 16) || !aligned(lse_parts, 4) || !aligned(lse, 4))
    return fail(CP_E_INVALID, "%s: misaligned pointer (tensors need 16 B, lse 4 B)", fn);
  const int64_t op_bytes = sat_mul({P, B, Sq, H, D, 4}), lp_bytes = sat_mul({P, B, H, Sq, 4});
  const int64_t o_bytes = sat_mul({B, Sq, H, D, elem_size(o_dtype)});
  const int64_t l_bytes = sat_mul({B, H, Sq, 4});
  if (overlap(o, o_bytes, o_parts, op_bytes) || overlap(o, o_bytes, lse_parts, lp_bytes) ||
      overlap(o, o_bytes, lse, l_bytes) || overlap(lse, l_bytes, o_parts, op_bytes) ||
      overlap(lse, l_bytes, lse_parts, lp_bytes))
    return fail(CP_E_INVALID, "%s: outputs overlap inputs or each other", fn);
  return hip_status(cpattn::launch_lse_merge(o_parts, lse_parts, static_cast<int>(P), o, lse, B,
                                             H, Sq, D, o_dtype == CP_BF16,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"

namespace {

bool ring_sizes_ok(int64_t B, int64_t H, int64_t Sq, int64_t D) {
  return B > 0 && H > 0 && Sq > 0 && (D == 64 || D == 128) && Sq < kMaxSeq &&
         sat_mul({(Sq + 63) / 64, B, H}) <= kMaxGrid / 8;
}

// Workspace a cp_ring_attention call cannot do without: the bf16 kernel's
// key-split partials (the most key splits any chunk list can get for these
// sizes, i.e. long chunks); the fp32 path never splits, so it needs none.
// One chunk never splits across blocks (it runs the plan of
// cp_attn_chunk_partial) except for a short last query tile.
size_t ring_workspace_need(int64_t P, int64_t B, int64_t H, int64_t Sq, int64_t D,
                           cp_dtype in_dtype) {
  if (in_dtype != CP_BF16 || !ring_sizes_ok(B, H, Sq, D)) return 0;
  if (P == 1) {
    const int ts = cpattn::attn_tail_splits(B, H, Sq, int64_t(1) << 40, false);
    const int64_t row0 = (Sq - 1) / 128 * 128;
    return ts > 0 ? static_cast<size_t>(cpattn::attn_split_floats(ts, B, H, Sq - row0, D)) *
                        sizeof(float)
                  : 0;
  }
  const int s = cpattn::attn_split_count(B, H, Sq, int64_t(1) << 40, false);
  return static_cast<size_t>(cpattn::attn_split_floats(s, B, H, Sq, D)) * sizeof(float);
}

}  // namespace

extern "C" {

size_t cp_ring_attention_workspace_bytes(int64_t P, int64_t B, int64_t H, int64_t Sq, int64_t D) {
  if (!ring_sizes_ok(B, H, Sq, D)) return 0;
  const size_t need = ring_workspace_need(P, B, H, Sq, D, CP_BF16);
  // one chunk: the optional key split of a last round (long chunk, non-causal)
  const size_t last =
      P == 1 ? static_cast<size_t>(cpattn::attn_last_split_floats(B, H, Sq, D, int64_t(1) << 40,
                                                                  false)) * sizeof(float)
             : 0;
  return std::max(need, last);
}

}  // extern "C"

namespace {

// Body of cp_ring_attention and cp_ring_attention_noalloc. `scratch_source`
// (non-null for the no-alloc entry point) yields the device scratch used as
// workspace, after every argument has been validated.
cp_status ring_attention_impl(const char* fn, const void* q, const cp_kv_chunk* chunks, int64_t P,
                              void* o, float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D,
                              cp_dtype in_dtype, float scale, int causal, int64_t q_pos0,
                              void* workspace, size_t workspace_bytes, void* stream,
                              cp_status (*scratch_source)(const char*, void**, size_t*)) {
  cp_status s = check_attn_common(fn, B, H, Sq, D, in_dtype, causal, scale);
  if (s != CP_OK) return s;
  if (P < 0) return fail(CP_E_INVALID, "%s: negative P", fn);
  if (P > CP_MAX_RING_CHUNKS)
    return fail(CP_E_UNSUPPORTED, "%s: P=%lld exceeds %d chunks", fn, (long long)P,
                CP_MAX_RING_CHUNKS);
  if (P > 0 && !chunks) return fail(CP_E_INVALID, "%s: null chunk array", fn);
  const size_t need = ring_workspace_need(P, B, H, Sq, D, in_dtype);
  if (scratch_source) {
    if (need > static_cast<size_t>(CP_NOALLOC_SCRATCH_BYTES))
      return fail(CP_E_WORKSPACE,
                  "%s: these sizes need %zu bytes of key-split scratch, above the built-in "
                  "%lld bytes; call cp_ring_attention with a workspace instead",
                  fn, need, (long long)CP_NOALLOC_SCRATCH_BYTES);
  } else if (workspace_bytes < need || (need > 0 && !workspace)) {
    return fail(CP_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace_bytes);
  }
  if (need > 0 && !aligned(workspace, 16))
    return fail(CP_E_INVALID, "%s: workspace must be 16-byte aligned", fn);
  const int64_t es = elem_size(in_dtype);
  const int64_t q_bytes = sat_mul({B, Sq, H, D, es}), o_bytes = q_bytes;
  const int64_t l_bytes = sat_mul({B, H, Sq, 4});
  for (int64_t c = 0; c < P; ++c) {
    if (chunks[c].len < 0) return fail(CP_E_INVALID, "%s: chunk %lld has negative length", fn,
                                       (long long)c);
    if (chunks[c].len >= kMaxSeq)
      return fail(CP_E_UNSUPPORTED, "%s: chunk %lld longer than 2^30", fn, (long long)c);
  }
  if (B == 0 || H == 0 || Sq == 0) return ok();
  if (!q || !o || !lse) return fail(CP_E_INVALID, "%s: null pointer", fn);
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return fail(CP_E_INVALID, "%s: misaligned pointer (tensors need 16 B, lse 4 B)", fn);
  // One chunk: when the workspace (the scratch, for the no-alloc entry point)
  // has room, a non-causal grid whose last round of 256-row blocks would be at
  // most half full runs that round with its keys split, merged after.
  int last_split = 0;
  size_t last_bytes = 0;
  if (in_dtype == CP_BF16 && P == 1) {
    const int64_t t1 = (chunks[0].len + 63) / 64;
    last_split = cpattn::attn_last_splits(B, H, Sq, D, t1, causal != 0);
    last_bytes = static_cast<size_t>(
                     cpattn::attn_last_split_floats(B, H, Sq, D, t1, causal != 0)) * sizeof(float);
    const size_t avail = scratch_source ? static_cast<size_t>(CP_NOALLOC_SCRATCH_BYTES)
                                        : (workspace ? workspace_bytes : 0);
    if (last_split < 2 || last_bytes > avail) {
      last_split = 0;
      last_bytes = 0;
    }
  }
  const int64_t ws_bytes = static_cast<int64_t>(std::max(need, last_bytes));
  if (overlap(o, o_bytes, q, q_bytes) || overlap(o, o_bytes, lse, l_bytes) ||
      overlap(lse, l_bytes, q, q_bytes) || overlap(workspace, ws_bytes, q, q_bytes) ||
      overlap(workspace, ws_bytes, o, o_bytes) || overlap(workspace, ws_bytes, lse, l_bytes))
    return fail(CP_E_INVALID, "%s: outputs or workspace overlap inputs or each other", fn);
  cpattn::AttnArgs a{};
  for (int64_t c = 0; c < P; ++c) {
    const cp_kv_chunk& ch = chunks[c];
    if (ch.len == 0) continue;
    if (!ch.k || !ch.v) return fail(CP_E_INVALID, "%s: chunk %lld has a null pointer", fn,
                                    (long long)c);
    if (!aligned(ch.k, 16) || !aligned(ch.v, 16))
      return fail(CP_E_INVALID, "%s: chunk %lld is misaligned", fn, (long long)c);
    const int64_t kv_bytes = sat_mul({B, ch.len, H, D, es});
    if (overlap(o, o_bytes, ch.k, kv_bytes) || overlap(o, o_bytes, ch.v, kv_bytes) ||
        overlap(lse, l_bytes, ch.k, kv_bytes) || overlap(lse, l_bytes, ch.v, kv_bytes) ||
        overlap(workspace, ws_bytes, ch.k, kv_bytes) || overlap(workspace, ws_bytes, ch.v, kv_bytes))
      return fail(CP_E_INVALID, "%s: outputs or workspace overlap chunk %lld", fn, (long long)c);
  }
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.B = static_cast<int32_t>(B);
  a.H = static_cast<int32_t>(H);
  a.Sq = static_cast<int32_t>(Sq);
  a.D = static_cast<int32_t>(D);
  a.scale = scale;
  a.nchunks = static_cast<int32_t>(P);
  int64_t tiles = 0;
  for (int64_t c = 0; c < P; ++c) {
    a.chunks[c].k = chunks[c].k;
    a.chunks[c].v = chunks[c].v;
    a.chunks[c].len = static_cast<int32_t>(chunks[c].len);
    a.chunks[c].delta = clamp_delta(q_pos0, chunks[c].pos0, Sq, chunks[c].len);
    tiles += (chunks[c].len + 63) / 64;
  }
  if (scratch_source && (need > 0 || last_split > 0)) {
    // every argument is valid: only now fetch (and on first use look up) the scratch
    s = scratch_source(fn, &workspace, &workspace_bytes);
    if (s != CP_OK) return s;
  }
  a.nsplit = 1;
  a.groups = 1;
  if (in_dtype == CP_BF16) {
    const int ts = cpattn::attn_tail_splits(B, H, Sq, tiles, causal != 0);
    const int64_t row0 = (Sq - 1) / 128 * 128;  // first row of the last 128-row query tile
    if (ts > 0 && static_cast<size_t>(cpattn::attn_split_floats(ts, B, H, Sq - row0, D)) *
                          sizeof(float) <= need) {
      // the full query tiles, one two-group block each, then the short last
      // tile's rows with their keys split ts ways; both write into the
      // caller's O and LSE (B = 1: a row window is a pointer offset)
      cpattn::AttnArgs m = a, t = a;
      m.Sq = static_cast<int32_t>(row0);
      m.lse_stride = static_cast<int32_t>(Sq);
      m.groups = cpattn::attn_groups(B, H, row0, tiles);
      t.Sq = static_cast<int32_t>(Sq - row0);
      t.lse_stride = static_cast<int32_t>(Sq);
      t.q = static_cast<const char*>(q) + row0 * H * D * es;
      t.o = static_cast<char*>(o) + row0 * H * D * es;
      t.lse = lse + row0;
      t.groups = 1;
      t.nsplit = ts;
      if (ts > 1) {
        t.part_o = static_cast<float*>(workspace);
        t.part_lse = t.part_o + ts * (Sq - row0) * H * D;
      }
      const int64_t q_pos_t = q_pos0 > INT64_MAX - row0 ? INT64_MAX : q_pos0 + row0;
      for (int64_t c = 0; c < P; ++c) {
        m.chunks[c].delta = clamp_delta(q_pos0, chunks[c].pos0, row0, chunks[c].len);
        t.chunks[c].delta = clamp_delta(q_pos_t, chunks[c].pos0, Sq - row0, chunks[c].len);
      }
      const hipStream_t st = static_cast<hipStream_t>(stream);
      const cp_status sm = launch_attention(fn, m, in_dtype, true, causal, st);
      if (sm != CP_OK) return sm;
      return launch_attention(fn, t, in_dtype, true, causal, st);
    }
    a.groups = cpattn::attn_groups(B, H, Sq, tiles);
    if (causal && a.groups == 1 && D == 128 && tiles >= 4 &&
        (Sq + 127) / 128 * B * H <= 2 * static_cast<int64_t>(cpattn::device_cus())) {
      // A causal grid of one to two query tiles per CU launches its heaviest
      // tiles first, so the ones past the first round are the lightest. When
      // the first query tile sees at most 4 key tiles, that second round is
      // short and two-group blocks (one round of whole-CU tiles, then the
      // rest) beat two 4-wave blocks per CU (rank 0 of a causal 4099-token
      // ring, 1025 rows that see only their own chunk: 24.5 against 26.6 us).
      int64_t first = 0;
      const int64_t last_row = std::min<int64_t>(Sq, 128) - 1;
      for (int64_t c = 0; c < P; ++c) {
        const int64_t vis = std::max<int64_t>(
            0, std::min<int64_t>(chunks[c].len, last_row + a.chunks[c].delta + 1));
        first += (vis + 63) / 64;
      }
      if (first <= 4) a.groups = 2;
    }
    // (one chunk runs on the ping-pong kernel, as cp_attn_chunk_partial does:
    // measured faster than 4-wave blocks split across blocks, Qwen-Image
    // rank 239 against 310 us)
    a.nsplit = (a.groups == 2 || P == 1)
                   ? 1
                   : cpattn::attn_split_count(B, H, Sq, tiles, causal != 0);
    if (a.nsplit > 1) {
      a.part_o = static_cast<float*>(workspace);
      a.part_lse = a.part_o + a.nsplit * B * Sq * H * D;
    } else if (last_split > 1 && a.groups == 1) {
      const int64_t rest = (Sq + 255) / 256 * B * H % cpattn::device_cus();
      a.last_split = last_split;
      a.part_o = static_cast<float*>(workspace);
      a.part_lse = a.part_o + last_split * rest * 256 * D;
    }
  }
  return launch_attention(fn, a, in_dtype, in_dtype == CP_BF16, causal,
                          static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

cp_status cp_ring_attention(const void* q, const cp_kv_chunk* chunks, int64_t P, void* o,
                            float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D,
                            cp_dtype in_dtype, float scale, int causal, int64_t q_pos0,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return ring_attention_impl("cp_ring_attention", q, chunks, P, o, lse, B, H, Sq, D, in_dtype,
                             scale, causal, q_pos0, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------- no-alloc
// cp_ring_attention_noalloc keeps its key-split partials in this file-scope
// device array instead of a caller workspace. Each GPU the library runs on
// holds its own copy (at its own address) until the process ends. In host
// code `scratch` only names the symbol: its device address on the current
// device comes from hipGetSymbolAddress, looked up once per device and kept
// in g_scratch_addr; kernels are only ever given that address.
namespace {

static __device__ __align__(256) char scratch[CP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

cp_status noalloc_scratch(const char* fn, void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CP_E_UNSUPPORTED, "%s: device %d beyond the %d the scratch table covers", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p) return fail(CP_E_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  *bytes = static_cast<size_t>(CP_NOALLOC_SCRATCH_BYTES);
  return CP_OK;
}

}  // namespace

extern "C" {

cp_status cp_ring_attention_noalloc(const void* q, const cp_kv_chunk* chunks, int64_t P, void* o,
                                    float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D,
                                    cp_dtype in_dtype, float scale, int causal, int64_t q_pos0,
                                    void* stream) {
  return ring_attention_impl("cp_ring_attention_noalloc", q, chunks, P, o, lse, B, H, Sq, D,
                             in_dtype, scale, causal, q_pos0, nullptr, 0, stream,
                             noalloc_scratch);
}

static cp_status relayout(const char* fn, const void* in, void* out, int64_t count, int64_t P,
                          int64_t B, int64_t S_local, int64_t H, int64_t D, cp_dtype dtype,
                          void* stream, bool seq2head) {
  if (count < 1) return fail(CP_E_INVALID, "%s: count must be >= 1", fn);
  if (count > 65535) return fail(CP_E_UNSUPPORTED, "%s: count exceeds 65535", fn);
  if (P < 1) return fail(CP_E_INVALID, "%s: P must be >= 1", fn);
  if (B < 0 || S_local < 0 || H < 0 || D < 0) return fail(CP_E_INVALID, "%s: negative size", fn);
  if (!valid_dtype(dtype)) return fail(CP_E_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (H % P != 0)
    return fail(CP_E_DIVISIBILITY, "%s: H=%lld heads do not divide by P=%lld", fn, (long long)H,
                (long long)P);
  if (B == 0 || S_local == 0 || H == 0 || D == 0) return ok();
  if (!in || !out) return fail(CP_E_INVALID, "%s: null pointer", fn);
  const int es = elem_size(dtype);
  if (!aligned(in, es) || !aligned(out, es))
    return fail(CP_E_INVALID, "%s: pointer not aligned to the element size", fn);
  const int64_t bytes = sat_mul({P, B, S_local, H, D, es});
  const int64_t all_bytes = sat_mul({count, bytes});
  if (overlap(in, all_bytes, out, all_bytes))
    return fail(CP_E_INVALID, "%s: out overlaps in", fn);
  cpattn::RelayoutDesc d{P, B, S_local, H, D, es, seq2head, count};
  const int w = cpattn::relayout_word_bytes(in, out, d);
  if (bytes / w >= (int64_t(1) << 31) || sat_mul({P, B, S_local, P}) >= (int64_t(1) << 31))
    return fail(CP_E_UNSUPPORTED, "%s: tensor of %lld bytes too large for one launch", fn,
                (long long)bytes);
  return hip_status(cpattn::launch_relayout(in, out, d, static_cast<hipStream_t>(stream)), fn);
}

cp_status cp_ulysses_seq2head(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                              int64_t H, int64_t D, cp_dtype dtype, void* stream) {
  return relayout("cp_ulysses_seq2head", in, out, 1, P, B, S_local, H, D, dtype, stream, true);
}

cp_status cp_ulysses_head2seq(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                              int64_t H, int64_t D, cp_dtype dtype, void* stream) {
  return relayout("cp_ulysses_head2seq", in, out, 1, P, B, S_local, H, D, dtype, stream, false);
}

}  // extern "C"

namespace {

// key-contiguous V: the Ulysses regrouping (groups = P) or the all-gather's
// unpack of P equal shards (groups = 1)
cp_status seq2head_vt(const char* fn, const void* in, void* out, int64_t P, int64_t B,
                      int64_t S_local, int64_t H, int64_t D, cp_dtype dtype, void* stream,
                      bool gather) {
  if (P < 1) return fail(CP_E_INVALID, "%s: P must be >= 1", fn);
  if (B < 0 || S_local < 0 || H < 0 || D < 0) return fail(CP_E_INVALID, "%s: negative size", fn);
  if (!valid_dtype(dtype)) return fail(CP_E_INVALID, "%s: unknown dtype %d", fn, dtype);
  if (dtype != CP_BF16) return fail(CP_E_UNSUPPORTED, "%s: bf16 only", fn);
  if (D != 128 && D != 0)
    return fail(CP_E_UNSUPPORTED, "%s: D=%lld (key-contiguous V needs D = 128)", fn, (long long)D);
  const int64_t groups = gather ? 1 : P;
  if (H % groups != 0)
    return fail(CP_E_DIVISIBILITY, "%s: H=%lld heads do not divide by P=%lld", fn, (long long)H,
                (long long)P);
  if (B == 0 || S_local == 0 || H == 0 || D == 0) return ok();
  if (!in || !out) return fail(CP_E_INVALID, "%s: null pointer", fn);
  if (!aligned(in, 16) || !aligned(out, 16))
    return fail(CP_E_INVALID, "%s: misaligned pointer (16 B needed)", fn);
  const int64_t bytes = sat_mul({P, B, S_local, H, D, 2});
  const int64_t out_bytes = sat_mul({B, H, (P * S_local + 63) / 64, D, 64, 2});
  if (overlap(in, bytes, out, out_bytes)) return fail(CP_E_INVALID, "%s: out overlaps in", fn);
  const int64_t T = sat_mul({P, S_local});
  if (T >= (int64_t(1) << 31) || sat_mul({B, H, (T + 127) / 128}) >= (int64_t(1) << 31))
    return fail(CP_E_UNSUPPORTED, "%s: tensor too large for one launch", fn);
  return hip_status(cpattn::launch_seq2head_vt(in, out, P, B, S_local, H, D, groups,
                                               static_cast<hipStream_t>(stream)),
                    fn);
}

}  // namespace

extern "C" {

cp_status cp_ulysses_seq2head_vt(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                                 int64_t H, int64_t D, cp_dtype dtype, void* stream) {
  return seq2head_vt("cp_ulysses_seq2head_vt", in, out, P, B, S_local, H, D, dtype, stream, false);
}

cp_status cp_kv_gather_vt(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                          int64_t H, int64_t D, cp_dtype dtype, void* stream) {
  return seq2head_vt("cp_kv_gather_vt", in, out, P, B, S_local, H, D, dtype, stream, true);
}

cp_status cp_ulysses_seq2head_n(const void* in, void* out, int64_t count, int64_t P, int64_t B,
                                int64_t S_local, int64_t H, int64_t D, cp_dtype dtype,
                                void* stream) {
  return relayout("cp_ulysses_seq2head_n", in, out, count, P, B, S_local, H, D, dtype, stream,
                  true);
}

cp_status cp_ulysses_head2seq_n(const void* in, void* out, int64_t count, int64_t P, int64_t B,
                                int64_t S_local, int64_t H, int64_t D, cp_dtype dtype,
                                void* stream) {
  return relayout("cp_ulysses_head2seq_n", in, out, count, P, B, S_local, H, D, dtype, stream,
                  false);
}

static cp_status any_relayout(const char* fn, const void* in, void* out, int64_t count,
                              int64_t P, int64_t B, const int64_t* s_lens,
                              const int64_t* h_counts, int64_t D, cp_dtype dtype, void* stream,
                              bool seq2head) {
  if (count < 1) return fail(CP_E_INVALID, "%s: count must be >= 1", fn);
  if (count > 65535) return fail(CP_E_UNSUPPORTED, "%s: count exceeds 65535", fn);
  if (P < 1) return fail(CP_E_INVALID, "%s: P must be >= 1", fn);
  if (P > CP_MAX_RING_CHUNKS)
    return fail(CP_E_UNSUPPORTED, "%s: P=%lld exceeds %d ranks", fn, (long long)P,
                CP_MAX_RING_CHUNKS);
  if (!s_lens || !h_counts) return fail(CP_E_INVALID, "%s: null count array", fn);
  if (B < 0 || D < 0) return fail(CP_E_INVALID, "%s: negative size", fn);
  if (!valid_dtype(dtype)) return fail(CP_E_INVALID, "%s: unknown dtype %d", fn, dtype);
  cpattn::AnyRelayoutDesc d{};
  d.P = static_cast<int32_t>(P);
  for (int64_t r = 0; r < P; ++r) {
    if (s_lens[r] < 0 || h_counts[r] < 0)
      return fail(CP_E_INVALID, "%s: negative count for rank %lld", fn, (long long)r);
    if (s_lens[r] >= kMaxSeq || h_counts[r] >= kMaxSeq)
      return fail(CP_E_UNSUPPORTED, "%s: count for rank %lld too large", fn, (long long)r);
    d.s_off[r + 1] = d.s_off[r] + s_lens[r];
    d.h_off[r + 1] = d.h_off[r] + h_counts[r];
  }
  d.B = B;
  d.S = d.s_off[P];
  d.H = d.h_off[P];
  d.D = D;
  d.seq2head = seq2head;
  d.count = count;
  if (B == 0 || d.S == 0 || d.H == 0 || D == 0) return ok();
  if (!in || !out) return fail(CP_E_INVALID, "%s: null pointer", fn);
  const int es = elem_size(dtype);
  d.elem_bytes = es;
  if (!aligned(in, es) || !aligned(out, es))
    return fail(CP_E_INVALID, "%s: pointer not aligned to the element size", fn);
  const int64_t bytes = sat_mul({B, d.S, d.H, D, es});
  const int64_t all_bytes = sat_mul({count, bytes});
  if (overlap(in, all_bytes, out, all_bytes))
    return fail(CP_E_INVALID, "%s: out overlaps in", fn);
  // one launch: every (rank pair, batch, tensor) block of words, and all offsets, fit 32 bits
  const int w = cpattn::any_relayout_word_bytes(in, out, d);
  if (sat_mul({B, count}) >= 65536 || sat_mul({d.S, d.H, D, es}) / w >= (int64_t(1) << 32) ||
      sat_mul({B, d.S, d.H}) >= (int64_t(1) << 32))
    return fail(CP_E_UNSUPPORTED, "%s: tensor of %lld bytes too large for one launch", fn,
                (long long)bytes);
  return hip_status(cpattn::launch_any_relayout(in, out, d, static_cast<hipStream_t>(stream)), fn);
}

cp_status cp_ulysses_anything_seq2head(const void* in, void* out, int64_t P, int64_t B,
                                       const int64_t* s_lens, const int64_t* h_counts, int64_t D,
                                       cp_dtype dtype, void* stream) {
  return any_relayout("cp_ulysses_anything_seq2head", in, out, 1, P, B, s_lens, h_counts, D,
                      dtype, stream, true);
}

cp_status cp_ulysses_anything_head2seq(const void* in, void* out, int64_t P, int64_t B,
                                       const int64_t* s_lens, const int64_t* h_counts, int64_t D,
                                       cp_dtype dtype, void* stream) {
  return any_relayout("cp_ulysses_anything_head2seq", in, out, 1, P, B, s_lens, h_counts, D,
                      dtype, stream, false);
}

cp_status cp_ulysses_anything_seq2head_n(const void* in, void* out, int64_t count, int64_t P,
                                         int64_t B, const int64_t* s_lens,
                                         const int64_t* h_counts, int64_t D, cp_dtype dtype,
                                         void* stream) {
  return any_relayout("cp_ulysses_anything_seq2head_n", in, out, count, P, B, s_lens, h_counts,
                      D, dtype, stream, true);
}

cp_status cp_ulysses_anything_head2seq_n(const void* in, void* out, int64_t count, int64_t P,
                                         int64_t B, const int64_t* s_lens,
                                         const int64_t* h_counts, int64_t D, cp_dtype dtype,
                                         void* stream) {
  return any_relayout("cp_ulysses_anything_head2seq_n", in, out, count, P, B, s_lens, h_counts,
                      D, dtype, stream, false);
}

static cp_status kv_gather(const char* fn, const void* in, void* out, int64_t count, int64_t P,
                           int64_t B, const int64_t* s_lens, int64_t H, int64_t D, cp_dtype dtype,
                           void* stream) {
  if (P < 1) return fail(CP_E_INVALID, "%s: P must be >= 1", fn);
  if (P > CP_MAX_RING_CHUNKS)
    return fail(CP_E_UNSUPPORTED, "%s: P=%lld exceeds %d ranks", fn, (long long)P,
                CP_MAX_RING_CHUNKS);
  if (H < 0) return fail(CP_E_INVALID, "%s: negative size", fn);
  // one destination group holding every head
  int64_t h_counts[CP_MAX_RING_CHUNKS] = {0};
  h_counts[0] = H;
  return any_relayout(fn, in, out, count, P, B, s_lens, h_counts, D, dtype, stream, true);
}

cp_status cp_kv_gather(const void* in, void* out, int64_t P, int64_t B, const int64_t* s_lens,
                       int64_t H, int64_t D, cp_dtype dtype, void* stream) {
  return kv_gather("cp_kv_gather", in, out, 1, P, B, s_lens, H, D, dtype, stream);
}

cp_status cp_kv_gather_n(const void* in, void* out, int64_t count, int64_t P, int64_t B,
                         const int64_t* s_lens, int64_t H, int64_t D, cp_dtype dtype,
                         void* stream) {
  return kv_gather("cp_kv_gather_n", in, out, count, P, B, s_lens, H, D, dtype, stream);
}

cp_status cp_attn_backward_delta(const void* o, const void* dout, float* delta, int64_t B,
                                 int64_t H, int64_t Sq, int64_t D, cp_dtype dtype, void* stream) {
  const char* fn = "cp_attn_backward_delta";
  cp_status s = check_attn_common(fn, B, H, Sq, D, dtype, 0, 1.f);
  if (s != CP_OK) return s;
  if (B == 0 || H == 0 || Sq == 0) return ok();
  const int64_t t_bytes = sat_mul({B, Sq, H, D, elem_size(dtype)});
  const int64_t l_bytes = sat_mul({B, H, Sq, 4});
  if (sat_mul({B, Sq, H}) > kMaxGrid / 2)
    return fail(CP_E_UNSUPPORTED, "%s: B*Sq*H too large for one launch", fn);
  if (!o || !dout || !delta) return fail(CP_E_INVALID, "%s: null pointer", fn);
  if (!aligned(o, 16) || !aligned(dout, 16) || !aligned(delta, 4))
    return fail(CP_E_INVALID, "%s: misaligned pointer (tensors need 16 B, delta 4 B)", fn);
  if (overlap(delta, l_bytes, o, t_bytes) || overlap(delta, l_bytes, dout, t_bytes))
    return fail(CP_E_INVALID, "%s: delta overlaps an input", fn);
  return hip_status(cpattn::launch_bwd_delta(o, dout, delta, B, H, Sq, D, dtype == CP_BF16,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

cp_status cp_attn_chunk_backward(const void* q, const void* k, const void* v, const void* dout,
                                 const float* lse, const float* delta, float* dq, float* dk,
                                 float* dv, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                 int64_t D, cp_dtype in_dtype, float scale, int causal,
                                 int64_t q_pos0, int64_t kv_pos0, int flags, void* stream) {
  const char* fn = "cp_attn_chunk_backward";
  cp_status s = check_attn_common(fn, B, H, Sq, D, in_dtype, causal, scale);
  if (s != CP_OK) return s;
  if (Skv < 0) return fail(CP_E_INVALID, "%s: negative Skv", fn);
  if (Skv >= kMaxSeq) return fail(CP_E_UNSUPPORTED, "%s: Skv exceeds 2^30", fn);
  if (flags & ~(CP_BWD_ACCUMULATE_DQ | CP_BWD_ACCUMULATE_DKV))
    return fail(CP_E_INVALID, "%s: unknown flag bits 0x%x", fn, flags);
  if (sat_mul({(Skv + 63) / 64, B, H}) > kMaxGrid / 8)
    return fail(CP_E_UNSUPPORTED, "%s: B*H*Skv too large for one launch", fn);
  if (B == 0 || H == 0 || (Sq == 0 && Skv == 0)) return ok();
  const int64_t es = elem_size(in_dtype);
  const int64_t q_bytes = sat_mul({B, Sq, H, D, es}), kv_bytes = sat_mul({B, Skv, H, D, es});
  const int64_t dq_bytes = sat_mul({B, Sq, H, D, 4}), dkv_bytes = sat_mul({B, Skv, H, D, 4});
  const int64_t l_bytes = sat_mul({B, H, Sq, 4});
  const bool has_q = Sq > 0, has_kv = Skv > 0;
  if ((has_q && (!q || !dout || !lse || !delta || !dq)) || (has_kv && (!k || !v || !dk || !dv)))
    return fail(CP_E_INVALID, "%s: null pointer", fn);
  if ((has_q && (!aligned(q, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
                 !aligned(lse, 4) || !aligned(delta, 4))) ||
      (has_kv && (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16))))
    return fail(CP_E_INVALID, "%s: misaligned pointer (tensors need 16 B, lse/delta 4 B)", fn);
  {
    const void* outs[3] = {dq, dk, dv};
    const int64_t out_n[3] = {has_q ? dq_bytes : 0, has_kv ? dkv_bytes : 0,
                              has_kv ? dkv_bytes : 0};
    const void* ins[6] = {q, dout, k, v, lse, delta};
    const int64_t in_n[6] = {has_q ? q_bytes : 0, has_q ? q_bytes : 0, has_kv ? kv_bytes : 0,
                             has_kv ? kv_bytes : 0, has_q ? l_bytes : 0, has_q ? l_bytes : 0};
    for (int x = 0; x < 3; ++x) {
      for (int y = 0; y < 6; ++y)
        if (overlap(outs[x], out_n[x], ins[y], in_n[y]))
          return fail(CP_E_INVALID, "%s: an output overlaps an input", fn);
      for (int y = x + 1; y < 3; ++y)
        if (overlap(outs[x], out_n[x], outs[y], out_n[y]))
          return fail(CP_E_INVALID, "%s: outputs overlap each other", fn);
    }
  }
  cpattn::BwdArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.B = static_cast<int32_t>(B);
  a.H = static_cast<int32_t>(H);
  a.Sq = static_cast<int32_t>(Sq);
  a.scale = scale;
  a.accum_dq = (flags & CP_BWD_ACCUMULATE_DQ) ? 1 : 0;
  a.accum_dkv = (flags & CP_BWD_ACCUMULATE_DKV) ? 1 : 0;
  a.nchunks = 1;
  cpattn::BwdChunk& c = a.chunks[0];
  c.k = static_cast<const __bf16*>(k);
  c.v = static_cast<const __bf16*>(v);
  c.dk = dk;
  c.dv = dv;
  c.len = static_cast<int32_t>(Skv);
  c.diag = clamp_delta(q_pos0, kv_pos0, Sq, Skv);
  c.tile0 = 0;
  a.total_kt = static_cast<int32_t>((Skv + 127) / 128);
  a.groups = cpattn::bwd_dq_groups(B, H, Sq, (Skv + 63) / 64);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(in_dtype == CP_BF16
                        ? cpattn::launch_attn_bwd_bf16(a, static_cast<int>(D), causal != 0, st)
                        : cpattn::launch_attn_bwd_f32(a, static_cast<int>(D), causal != 0, st),
                    fn);
}

cp_status cp_ring_attention_backward(const void* q, const cp_kv_chunk* chunks, int64_t P,
                                     const void* dout, const float* lse, const float* delta,
                                     float* dq, const cp_kv_grad* grads, int64_t B, int64_t H,
                                     int64_t Sq, int64_t D, cp_dtype in_dtype, float scale,
                                     int causal, int64_t q_pos0, int flags, void* stream) {
  const char* fn = "cp_ring_attention_backward";
  cp_status s = check_attn_common(fn, B, H, Sq, D, in_dtype, causal, scale);
  if (s != CP_OK) return s;
  if (P < 1) return fail(CP_E_INVALID, "%s: P must be >= 1", fn);
  if (P > CP_MAX_RING_CHUNKS)
    return fail(CP_E_UNSUPPORTED, "%s: P=%lld exceeds %d chunks", fn, (long long)P,
                CP_MAX_RING_CHUNKS);
  if (!chunks || !grads) return fail(CP_E_INVALID, "%s: null chunk or gradient array", fn);
  if (flags & ~(CP_BWD_ACCUMULATE_DQ | CP_BWD_ACCUMULATE_DKV))
    return fail(CP_E_INVALID, "%s: unknown flag bits 0x%x", fn, flags);
  int64_t total_kt = 0, total_keys = 0;
  for (int64_t c = 0; c < P; ++c) {
    const int64_t len = chunks[c].len;
    if (len < 0) return fail(CP_E_INVALID, "%s: chunk %lld has negative length", fn, (long long)c);
    if (len >= kMaxSeq)
      return fail(CP_E_UNSUPPORTED, "%s: chunk %lld length exceeds 2^30", fn, (long long)c);
    total_kt += (len + 127) / 128;
    total_keys += len;
  }
  if (sat_mul({total_kt, B, H}) > kMaxGrid / 8)
    return fail(CP_E_UNSUPPORTED, "%s: B*H*keys too large for one launch", fn);
  if (B == 0 || H == 0 || (Sq == 0 && total_keys == 0)) return ok();
  const int64_t es = elem_size(in_dtype);
  const int64_t q_bytes = sat_mul({B, Sq, H, D, es}), dq_bytes = sat_mul({B, Sq, H, D, 4});
  const int64_t l_bytes = sat_mul({B, H, Sq, 4});
  const bool has_q = Sq > 0;
  if (has_q && (!q || !dout || !lse || !delta || !dq))
    return fail(CP_E_INVALID, "%s: null pointer", fn);
  if (has_q && (!aligned(q, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(lse, 4) ||
                !aligned(delta, 4)))
    return fail(CP_E_INVALID, "%s: misaligned pointer (tensors need 16 B, lse/delta 4 B)", fn);
  // every output against every input and every other output
  struct Range {
    const void* p;
    int64_t n;
  };
  Range ins[4 + 2 * CP_MAX_RING_CHUNKS], outs[1 + 2 * CP_MAX_RING_CHUNKS];
  int n_in = 0, n_out = 0;
  if (has_q) {
    ins[n_in++] = {q, q_bytes};
    ins[n_in++] = {dout, q_bytes};
    ins[n_in++] = {lse, l_bytes};
    ins[n_in++] = {delta, l_bytes};
    outs[n_out++] = {dq, dq_bytes};
  }
  for (int64_t c = 0; c < P; ++c) {
    const int64_t len = chunks[c].len;
    if (len == 0) continue;
    const int64_t kv_bytes = sat_mul({B, len, H, D, es}), g_bytes = sat_mul({B, len, H, D, 4});
    if (!chunks[c].k || !chunks[c].v || !grads[c].dk || !grads[c].dv)
      return fail(CP_E_INVALID, "%s: chunk %lld has a null pointer", fn, (long long)c);
    if (!aligned(chunks[c].k, 16) || !aligned(chunks[c].v, 16) || !aligned(grads[c].dk, 16) ||
        !aligned(grads[c].dv, 16))
      return fail(CP_E_INVALID, "%s: chunk %lld pointer misaligned (16 B)", fn, (long long)c);
    ins[n_in++] = {chunks[c].k, kv_bytes};
    ins[n_in++] = {chunks[c].v, kv_bytes};
    outs[n_out++] = {grads[c].dk, g_bytes};
    outs[n_out++] = {grads[c].dv, g_bytes};
  }
  for (int x = 0; x < n_out; ++x) {
    for (int y = 0; y < n_in; ++y)
      if (overlap(outs[x].p, outs[x].n, ins[y].p, ins[y].n))
        return fail(CP_E_INVALID, "%s: an output overlaps an input", fn);
    for (int y = x + 1; y < n_out; ++y)
      if (overlap(outs[x].p, outs[x].n, outs[y].p, outs[y].n))
        return fail(CP_E_INVALID, "%s: output buffers overlap each other", fn);
  }
  cpattn::BwdArgs a{};
  a.q = static_cast<const __bf16*>(q);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.B = static_cast<int32_t>(B);
  a.H = static_cast<int32_t>(H);
  a.Sq = static_cast<int32_t>(Sq);
  a.scale = scale;
  a.accum_dq = (flags & CP_BWD_ACCUMULATE_DQ) ? 1 : 0;
  a.accum_dkv = (flags & CP_BWD_ACCUMULATE_DKV) ? 1 : 0;
  a.nchunks = static_cast<int32_t>(P);
  int32_t tile0 = 0;
  int64_t key_tiles = 0;
  for (int64_t c = 0; c < P; ++c) {
    cpattn::BwdChunk& d = a.chunks[c];
    d.k = static_cast<const __bf16*>(chunks[c].k);
    d.v = static_cast<const __bf16*>(chunks[c].v);
    d.dk = grads[c].dk;
    d.dv = grads[c].dv;
    d.len = static_cast<int32_t>(chunks[c].len);
    d.diag = clamp_delta(q_pos0, chunks[c].pos0, Sq, chunks[c].len);
    d.tile0 = tile0;
    tile0 += static_cast<int32_t>((chunks[c].len + 127) / 128);
    key_tiles += (chunks[c].len + 63) / 64;
  }
  a.total_kt = tile0;
  a.groups = cpattn::bwd_dq_groups(B, H, Sq, key_tiles);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(in_dtype == CP_BF16
                        ? cpattn::launch_attn_bwd_bf16(a, static_cast<int>(D), causal != 0, st)
                        : cpattn::launch_attn_bwd_f32(a, static_cast<int>(D), causal != 0, st),
                    fn);
}

}  // extern "C"
