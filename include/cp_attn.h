/*
 * cp_attn.h — C ABI of the MI355X (gfx950) context-parallel attention library.
 *
 * One rank's share of block-wise softmax attention, as context parallelism
 * runs it inside the attention backend, plus the Ulysses layout transforms
 * around it. Everything runs on one GPU; the exchanges between ranks (ring
 * rotation, all-to-all) are not part of this library.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense and contiguous, BSHD: element [b][s][h][d] sits at
 *    ((b*S + s)*H + h)*D + d. LSE tensors are fp32 [B][H][S]:
 *    element [b][h][s] at (b*H + h)*S + s.
 *  - "LSE" is the natural log of the row's softmax normaliser, scale
 *    included: LSE_i = ln sum_j exp(scale * <q_i, k_j>). A row that sees no
 *    key has LSE = -inf and output 0 (never NaN).
 *  - Device pointers are plain device addresses (from hipMalloc or PyTorch).
 *    The caller allocates and owns every device buffer; the library never
 *    allocates or frees device memory (cp_ring_attention_noalloc keeps its
 *    scratch in a static device array instead). Outputs must not overlap inputs.
 *    Tensor pointers must be 16-byte aligned; LSE pointers 4-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued on it and no call synchronises: results are valid once
 *    the stream has reached that point. A call enqueues kernel launches only
 *    (no memset, copy, allocation or synchronisation), so calls may be
 *    captured into a HIP graph on a capturing stream and replayed; the
 *    arguments (pointers, sizes, chunk lists) are fixed at capture.
 *  - Arguments are validated on the host before anything is enqueued. On any
 *    error the call returns a non-zero cp_status, enqueues nothing, leaves
 *    every output untouched, and cp_last_error() describes the problem. A
 *    launch failure reported by the HIP runtime returns CP_E_HIP.
 *  - Zero-sized work (B, H or Sq equal to 0) is a successful no-op. Negative
 *    sizes are CP_E_INVALID.
 *  - Repeating a call on identical inputs gives byte-identical outputs
 *    (fixed reduction order, no floating-point atomics).
 *  - Attention inputs (Q, K, V, dO, partial O) must be finite. The kernels
 *    do not propagate NaN or infinity the way the textbook formula would; a
 *    non-finite input gives unspecified (possibly finite) outputs for the
 *    rows it touches. The layout transforms move any bit pattern unchanged.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CP_BF16 = 0, CP_F32 = 1 } cp_dtype;

typedef enum {
  CP_OK = 0,
  CP_E_INVALID = 1,      /* null/misaligned/overlapping pointer, negative size, bad flag */
  CP_E_UNSUPPORTED = 2,  /* head dim, dtype combination or size outside what is built  */
  CP_E_DIVISIBILITY = 3, /* Ulysses: H or the sequence does not divide by P            */
  CP_E_WORKSPACE = 4,    /* workspace missing or smaller than required                 */
  CP_E_HIP = 5           /* the HIP runtime reported an error at launch                */
} cp_status;

/* One K/V chunk of a ring: K and V are [B][len][H][D] in the call's dtype.
 * pos0 is the global position of the chunk's first key (causal masking only). */
typedef struct {
  const void* k;
  const void* v;
  int64_t len;
  int64_t pos0;
} cp_kv_chunk;

/* Largest ring degree cp_ring_attention accepts in one call. */
#define CP_MAX_RING_CHUNKS 64

/*
 * cp_attn_chunk_partial — one ring hop: attention of a Q shard over ONE K/V chunk.
 *
 * Defined by: the Context parallelism guide (diffusers), section Ring
 * Attention (each GPU attends its Q to the K/V block it holds), and the
 * diffusers parallel API, ContextParallelConfig (convert_to_fp32: each hop's
 * output and LSE are kept in float32 for the merge). With one chunk covering
 * the whole sequence it is the local attention a Ulysses rank runs between
 * its two all-to-alls (Ulysses Sequence Parallelism article, detailed notes 4).
 *
 *   q [B][Sq][H][D], k and v [B][Skv][H][D], dtype in_dtype.
 *   o [B][Sq][H][D] in o_dtype: O_i = sum_j exp(S_ij - LSE_i) v_j over this chunk.
 *   lse [B][H][Sq] fp32: LSE_i = ln sum_j exp(S_ij), S_ij = scale * <q_i, k_j>.
 *   causal != 0: key j is visible to query i iff kv_pos0 + j <= q_pos0 + i
 *   (causal masking from position ids, Ulysses Sequence Parallelism article,
 *   detailed notes 7); causal == 0 ignores the positions.
 *
 * Supported: D in {64, 128}; in_dtype CP_BF16 with o_dtype CP_F32 or CP_BF16
 * (bf16 MFMA products, fp32 accumulation, softmax in fp32, probabilities
 * rounded to bf16 for the P*V product); in_dtype CP_F32 with o_dtype CP_F32
 * (fp32 throughout). Skv == 0 is allowed: every row gets O = 0, LSE = -inf.
 * Limits: Sq, Skv < 2^30. scale must be finite.
 */
cp_status cp_attn_chunk_partial(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                cp_dtype in_dtype, cp_dtype o_dtype, float scale, int causal,
                                int64_t q_pos0, int64_t kv_pos0, void* stream);

/*
 * cp_attn_chunk_partial_vt — cp_attn_chunk_partial with V given key-contiguous
 * per head, in tiles of 64 keys: vt [B][H][ceil(Skv/64)][D][64],
 * vt[b][h][j / 64][d][j % 64] = v[b][j][h][d]. Each tile is one contiguous
 * 16 KB block; its columns past Skv (the last tile's padding) must hold
 * finite values (they get weight 0; cp_ulysses_seq2head_vt writes zeros).
 *
 * Defined by: as cp_attn_chunk_partial (the local attention of a Ulysses rank,
 * Ulysses Sequence Parallelism article, detailed notes 4; Context parallelism
 * guide (diffusers), section Ulysses Attention). Only the storage order of V
 * differs: it is the order in which the P*V product consumes V, and
 * cp_ulysses_seq2head_vt produces it for each destination rank, so the rank's
 * attention reads V with full-width LDS reads instead of transposing ones.
 * q, k, o, lse, the causal rule, the arithmetic and the order of every sum
 * are those of cp_attn_chunk_partial: O and LSE equal its results on the same
 * values bit for bit.
 *
 * Supported: in_dtype CP_BF16, D = 128, o_dtype CP_F32 or CP_BF16 (anything
 * else is CP_E_UNSUPPORTED); other limits as cp_attn_chunk_partial. vt
 * 16-byte aligned (else CP_E_INVALID). Skv == 0 is allowed (O = 0,
 * LSE = -inf; vt may be NULL).
 */
cp_status cp_attn_chunk_partial_vt(const void* q, const void* k, const void* vt, void* o,
                                   float* lse, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                   int64_t D, cp_dtype in_dtype, cp_dtype o_dtype, float scale,
                                   int causal, int64_t q_pos0, int64_t kv_pos0, void* stream);

/*
 * cp_lse_merge — merge P partial (O_c, LSE_c) pairs into attention over all their keys.
 *
 * Defined by: the diffusers parallel API, ContextParallelConfig
 * (convert_to_fp32: outputs and LSE converted to float32 for a stable merge)
 * and the Sequence Parallelism page (SGLang Diffusion), section Numerics
 * across node boundaries (hops are merged by online softmax). Per row:
 *   M = max_c LSE_c;  LSE = M + ln sum_c exp(LSE_c - M);
 *   O = sum_c exp(LSE_c - LSE) * O_c;   all LSE_c = -inf gives O = 0, LSE = -inf.
 *
 *   o_parts [P][B][Sq][H][D] fp32, lse_parts [P][B][H][Sq] fp32 (P >= 1).
 *   o [B][Sq][H][D] in o_dtype (CP_F32, or CP_BF16 rounded to nearest even);
 *   lse [B][H][Sq] fp32. D must be a multiple of 4 and at most 4096. The
 *   partials are combined in the fixed order c = 0..P-1.
 */
cp_status cp_lse_merge(const float* o_parts, const float* lse_parts, int64_t P, void* o,
                       float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D, cp_dtype o_dtype,
                       void* stream);

/*
 * cp_ring_attention_workspace_bytes — device workspace for a cp_ring_attention
 * call with these sizes (may be 0). With at most one query tile (128 rows of
 * one batch and head) per compute unit, each tile's keys are split inside its
 * block and no workspace is needed. Between one and two tiles per compute
 * unit, cp_ring_attention splits each tile's keys over two blocks when P > 1
 * (one chunk runs as cp_attn_chunk_partial does); the splits' fp32 (O, LSE)
 * partials live in the workspace and are merged exactly as cp_lse_merge
 * does. (A non-causal single-batch call whose last query tile
 * holds at most 32 rows, when the other tiles fit one per compute unit,
 * splits only that tile's keys, up to 8 ways, and uses less of the same
 * workspace.) With P == 1 the value also covers an optional plan: when a
 * non-causal call's 256-row query tiles take more than one round of the
 * compute units and the last round would be at most half full, that round's
 * tiles have their keys split (up to 8 ways, at least 4 key tiles a split)
 * and are merged the same way. A call given less workspace than this value
 * but at least what the first plans need runs that last round unsplit
 * instead (same results to rounding). Host function; queries the current
 * device's compute-unit count; returns 0 for invalid sizes (which
 * cp_ring_attention then rejects).
 */
size_t cp_ring_attention_workspace_bytes(int64_t P, int64_t B, int64_t H, int64_t Sq, int64_t D);

/*
 * cp_ring_attention — one ring rank's whole share: Q attends P K/V chunks in
 * the given order and the per-chunk results are merged in fp32.
 *
 * Defined by: the Context parallelism guide (diffusers), sections Ring
 * Attention (K/V blocks visit every rank; after a full turn each rank has
 * attended every token) and Ring Anything Attention (chunks of unequal length:
 * padding is sliced away before attention, so uneven lengths are accepted
 * here as they are), and the diffusers parallel API, ContextParallelConfig
 * (rotate_method "allgather": every chunk is resident when attention runs;
 * convert_to_fp32). The merge is fused: the running output and LSE stay in
 * fp32 across chunks and O is rounded to in_dtype once at the end.
 *
 *   q [B][Sq][H][D] in in_dtype; chunks: a HOST array of P descriptors in
 *   visit order (read during the call only), each K/V [B][len][H][D].
 *   o [B][Sq][H][D] in in_dtype; lse [B][H][Sq] fp32.
 *   causal != 0: key j of chunk c is visible to query i iff
 *   chunks[c].pos0 + j <= q_pos0 + i.
 *   workspace: 16-byte aligned device buffer of cp_ring_attention_workspace_bytes(
 *   P, B, H, Sq, D) bytes (NULL if 0), owned by the caller, contents need no
 *   initialisation and are scratch afterwards; concurrent calls must not
 *   share one workspace. Less than the key-split partials need:
 *   CP_E_WORKSPACE (the optional last-round split above is skipped instead).
 *   CP_F32 inputs never split keys and need no workspace (NULL, 0 accepted).
 *
 * 0 <= P <= CP_MAX_RING_CHUNKS; chunk lengths may differ and may be 0. Same D
 * and dtype support as cp_attn_chunk_partial (O in in_dtype).
 */
cp_status cp_ring_attention(const void* q, const cp_kv_chunk* chunks, int64_t P, void* o,
                            float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D,
                            cp_dtype in_dtype, float scale, int causal, int64_t q_pos0,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device scratch array cp_ring_attention_noalloc uses (64 MiB). */
#define CP_NOALLOC_SCRATCH_BYTES 67108864

/*
 * cp_ring_attention_noalloc — cp_ring_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, and no call on its
 * path allocates or frees memory.
 *
 *   Every argument, rule and result is that of cp_ring_attention (same
 *   kernels, bit-identical outputs), except the workspace: the key-split
 *   partials live in a file-scope device array of CP_NOALLOC_SCRATCH_BYTES
 *   that each GPU holds from its first use until the process ends. Sizes
 *   whose workspace (cp_ring_attention_workspace_bytes) exceeds that limit
 *   are rejected with CP_E_WORKSPACE before anything is enqueued.
 *   The array's device address is looked up (hipGetSymbolAddress) on the
 *   first call that needs it on each device, with that device current: make
 *   that first call outside graph capture. Work runs on the CURRENT device,
 *   which must be the stream's.
 *   Every call on one GPU shares that GPU's array: calls that can overlap in
 *   time on one GPU (other streams, other threads, other processes' streams
 *   are separate arrays) race and give undefined results; serialise them on
 *   one stream. Nothing in the array needs clearing between calls (each split
 *   writes its whole partial before the merge reads it).
 */
cp_status cp_ring_attention_noalloc(const void* q, const cp_kv_chunk* chunks, int64_t P, void* o,
                                    float* lse, int64_t B, int64_t H, int64_t Sq, int64_t D,
                                    cp_dtype in_dtype, float scale, int causal, int64_t q_pos0,
                                    void* stream);

/*
 * cp_ulysses_seq2head — the Ulysses regrouping before attention, for all P
 * ranks at once (pack + unpack of the first all-to-all, transport removed).
 *
 * Defined by: the Context parallelism guide (diffusers), section Ulysses
 * Attention (the first all-to-all leaves each GPU holding every token for a
 * subset of heads) and the Ulysses Sequence Parallelism article, detailed
 * notes 3-4. Destination rank p receives the contiguous head group
 * [p*H/P, (p+1)*H/P); tokens are concatenated in source-rank order:
 *   out[p][b][q*S_local + s][h][d] = in[q][b][s][p*(H/P) + h][d]
 *
 *   in  [P][B][S_local][H][D]    (source rank q's sequence shard is in[q])
 *   out [P][B][P*S_local][H/P][D] (destination rank p's head shard is out[p])
 * A pure bit copy in the element size of dtype (2 bytes for CP_BF16, 4 for
 * CP_F32): NaN payloads, infinities and -0 are moved unchanged.
 * H % P != 0 is CP_E_DIVISIBILITY (the standard Ulysses mode needs the heads
 * to divide by the degree; it fails rather than padding). P >= 1, any D >= 1.
 */
cp_status cp_ulysses_seq2head(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                              int64_t H, int64_t D, cp_dtype dtype, void* stream);

/*
 * cp_ulysses_head2seq — the Ulysses regrouping after attention: the exact
 * inverse of cp_ulysses_seq2head (the second all-to-all regroups the output
 * by token, same passages as above):
 *   out[q][b][s][p*(H/P) + h][d] = in[p][b][q*S_local + s][h][d]
 *
 *   in  [P][B][P*S_local][H/P][D], out [P][B][S_local][H][D]; H is the FULL
 *   head count. Same dtype, divisibility and bit-copy rules as seq2head.
 */
cp_status cp_ulysses_head2seq(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                              int64_t H, int64_t D, cp_dtype dtype, void* stream);

/*
 * cp_ulysses_seq2head_vt — cp_ulysses_seq2head for the value tensor, with each
 * destination rank's head shard stored key-contiguous: the V layout
 * cp_attn_chunk_partial_vt reads.
 *
 * Defined by: as cp_ulysses_seq2head (Context parallelism guide (diffusers),
 * section Ulysses Attention): the same regrouping, the head shard written in
 * tiles of 64 tokens, each tile feature-major; a bit permutation plus zero
 * padding. With t = q*S_local + s and T = P*S_local:
 *   out[p][b][h][t / 64][d][t % 64] = in[q][b][s][p*(H/P) + h][d]
 *   and out[p][b][h][T / 64][d][c] = 0 for the last tile's columns c >= T % 64.
 *
 *   in  [P][B][S_local][H][D] (as cp_ulysses_seq2head)
 *   out [P][B][H/P][ceil(T/64)][D][64] (rank p's V is out[p])
 * dtype CP_BF16 only and D = 128 (else CP_E_UNSUPPORTED); in and
 * out 16-byte aligned (else CP_E_INVALID); H % P != 0 is CP_E_DIVISIBILITY.
 * P*S_local < 2^31.
 */
cp_status cp_ulysses_seq2head_vt(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                                 int64_t H, int64_t D, cp_dtype dtype, void* stream);

/*
 * cp_kv_gather_vt — the K/V all-gather's unpack for the value tensor, delivered
 * key-contiguous: the V layout cp_attn_chunk_partial_vt reads, for a rank that
 * attends its Q shard to the whole sequence's K and V.
 *
 * Defined by: the SGLang Diffusion Sequence Parallelism page, the table of
 * attention modes and section K/V-Gather sequence parallelism (each rank
 * gathers every rank's K and V shard). P shards of S_local tokens each, joined
 * in rank order and written in tiles of 64 tokens, each tile feature-major;
 * with t = q*S_local + s and T = P*S_local:
 *   out[b][h][t / 64][d][t % 64] = in[q][b][s][h][d]
 *   and the last tile's columns c >= T % 64 are 0.
 *
 *   in  [P][B][S_local][H][D] (shard q is in[q]), out [B][H][ceil(T/64)][D][64]
 * Equal shards only (uneven shards: cp_kv_gather). dtype CP_BF16 and D = 128
 * (else CP_E_UNSUPPORTED); in and out 16-byte aligned (else CP_E_INVALID).
 * P*S_local < 2^31.
 */
cp_status cp_kv_gather_vt(const void* in, void* out, int64_t P, int64_t B, int64_t S_local,
                          int64_t H, int64_t D, cp_dtype dtype, void* stream);

/*
 * cp_ulysses_seq2head_n / cp_ulysses_head2seq_n — the same regroupings for
 * `count` tensors stored back to back, in one launch.
 *
 * Defined by: as cp_ulysses_seq2head / cp_ulysses_head2seq. A Ulysses rank
 * regroups its Q, K and V together before attention (Context parallelism
 * guide (diffusers), section Ulysses Attention; Ulysses Sequence Parallelism
 * article, detailed notes 4), so one launch moves all three.
 *   in:  count tensors, tensor t starting at element t*P*B*S_local*H*D, each in
 *        the single-tensor call's input layout; out likewise in its output
 *        layout. count in 1..65535; every other argument, limit and rule as in
 *        the single-tensor calls (each tensor below 2^31 words). Tensor t of
 *        out equals the single-tensor call on tensor t of in, bit for bit.
 */
cp_status cp_ulysses_seq2head_n(const void* in, void* out, int64_t count, int64_t P, int64_t B,
                                int64_t S_local, int64_t H, int64_t D, cp_dtype dtype,
                                void* stream);
cp_status cp_ulysses_head2seq_n(const void* in, void* out, int64_t count, int64_t P, int64_t B,
                                int64_t S_local, int64_t H, int64_t D, cp_dtype dtype,
                                void* stream);

/*
 * cp_ulysses_anything_seq2head — the Ulysses regrouping when neither the
 * sequence nor the heads divide by the degree.
 *
 * Defined by: the Context parallelism guide (diffusers), section Ulysses
 * Anything Attention (the mode removes both divisibility requirements of
 * Ulysses), and the diffusers parallel API, ContextParallelConfig
 * (ulysses_anything). Source rank q holds s_lens[q] tokens, tokens
 * [off_q, off_q + s_lens[q]) of the sequence with off_q = s_lens[0] + ... +
 * s_lens[q-1]; destination rank p receives the h_counts[p] contiguous heads
 * starting at h0_p = h_counts[0] + ... + h_counts[p-1]:
 *   out_p[b][off_q + s][h][d] = in_q[b][s][h0_p + h][d]
 *
 *   in:  the P sequence shards packed back to back in rank order; shard q is
 *        [B][s_lens[q]][H][D] and starts at element B*off_q*H*D, where
 *        H = sum of h_counts.
 *   out: the P head groups packed back to back in rank order; group p is
 *        [B][S][h_counts[p]][D] and starts at element B*S*h0_p*D, where
 *        S = sum of s_lens.
 *   s_lens, h_counts: HOST arrays of P counts (>= 0, zero allowed), read
 *        during the call only.
 * 1 <= P <= CP_MAX_RING_CHUNKS, any D >= 1, B < 65536. Same bit-copy and
 * dtype rules as cp_ulysses_seq2head. Negative counts or a null array are
 * CP_E_INVALID. With equal counts the result equals cp_ulysses_seq2head's.
 */
cp_status cp_ulysses_anything_seq2head(const void* in, void* out, int64_t P, int64_t B,
                                       const int64_t* s_lens, const int64_t* h_counts, int64_t D,
                                       cp_dtype dtype, void* stream);

/*
 * cp_ulysses_anything_head2seq — the exact inverse of
 * cp_ulysses_anything_seq2head (the second regrouping, by token; same
 * passages):
 *   out_q[b][s][h0_p + h][d] = in_p[b][off_q + s][h][d]
 *
 *   in: the packed head groups, out: the packed sequence shards, with the
 *   layouts and count rules described for cp_ulysses_anything_seq2head.
 */
cp_status cp_ulysses_anything_head2seq(const void* in, void* out, int64_t P, int64_t B,
                                       const int64_t* s_lens, const int64_t* h_counts, int64_t D,
                                       cp_dtype dtype, void* stream);

/*
 * cp_ulysses_anything_seq2head_n / cp_ulysses_anything_head2seq_n — the
 * uneven regroupings for `count` tensors stored back to back, in one launch.
 *
 * Defined by: as cp_ulysses_anything_seq2head / _head2seq; the rank's Q, K
 * and V are regrouped together before attention (Context parallelism guide
 * (diffusers), sections Ulysses Attention and Ulysses Anything Attention).
 *   in:  count packed inputs, input t starting at element t*B*S*H*D, each laid
 *        out as the single-tensor call's input; out likewise as its output.
 * count in 1..65535 and B*count < 65536; every other argument, limit and
 * rule as in the single-tensor calls. Tensor t of out equals the
 * single-tensor call on tensor t of in, bit for bit.
 */
cp_status cp_ulysses_anything_seq2head_n(const void* in, void* out, int64_t count, int64_t P,
                                         int64_t B, const int64_t* s_lens,
                                         const int64_t* h_counts, int64_t D, cp_dtype dtype,
                                         void* stream);
cp_status cp_ulysses_anything_head2seq_n(const void* in, void* out, int64_t count, int64_t P,
                                         int64_t B, const int64_t* s_lens,
                                         const int64_t* h_counts, int64_t D, cp_dtype dtype,
                                         void* stream);

/*
 * cp_kv_gather — the unpack of the K/V all-gather: P sequence shards joined
 * into one sequence, all heads kept.
 *
 * Defined by: the Sequence Parallelism page (SGLang Diffusion), section
 * Choosing The Attention Exchange (kv_gather: queries and outputs stay
 * sequence-sharded, K and V are all-gathered, each rank computes its own
 * output directly; non-causal, ring degree 1). A rank's share is then
 * cp_attn_chunk_partial of its query shard over the gathered K and V, or
 * cp_ring_attention over the P shards in place (same result).
 *   out[b][off_q + s][h][d] = in_q[b][s][h][d],
 *   off_q = s_lens[0] + ... + s_lens[q-1]
 *
 *   in:  the P shards packed back to back in rank order; shard q is
 *        [B][s_lens[q]][H][D] and starts at element B*off_q*H*D.
 *   out: [B][S][H][D], S = sum of s_lens.
 *   s_lens: HOST array of P counts (>= 0), read during the call only.
 * For B = 1 the packed shards already are the gathered tensor and this is a
 * plain copy. Same limits, bit-copy and error rules as
 * cp_ulysses_anything_seq2head (it is that regrouping with a single head
 * group holding all H heads).
 */
cp_status cp_kv_gather(const void* in, void* out, int64_t P, int64_t B, const int64_t* s_lens,
                       int64_t H, int64_t D, cp_dtype dtype, void* stream);

/*
 * cp_kv_gather_n — cp_kv_gather for `count` tensors stored back to back (K
 * and V: the all-gather moves both), in one launch.
 *
 * Defined by: as cp_kv_gather.
 *   in:  count packed shard sets, set t starting at element t*B*S*H*D; out:
 *        count gathered tensors [B][S][H][D] back to back.
 * count in 1..65535 and B*count < 65536; every other argument, limit and
 * rule as in cp_kv_gather. Tensor t of out equals cp_kv_gather on set t of
 * in, bit for bit.
 */
cp_status cp_kv_gather_n(const void* in, void* out, int64_t count, int64_t P, int64_t B,
                         const int64_t* s_lens, int64_t H, int64_t D, cp_dtype dtype,
                         void* stream);

/*
 * cp_attn_backward_delta — the per-row statistic the backward needs besides LSE:
 *   delta[b][h][i] = sum_d dout[b][i][h][d] * o[b][i][h][d]   (fp32)
 *
 * Defined by: the derivative of softmax attention (the pages' training
 * context is the Ulysses Sequence Parallelism article, summary and detailed
 * notes 2 and 6-8): for the exact output, <dO_i, O_i> equals
 * sum_j P_ij <dO_i, v_j>, the term the softmax Jacobian subtracts. Pass the
 * FULL attention output (after every ring hop is merged), not a chunk's.
 *
 *   o, dout [B][Sq][H][D], both in `dtype` (CP_BF16 or CP_F32); delta [B][H][Sq]
 *   fp32, caller-allocated. D in {64, 128}. Products and sum in fp32, in a
 *   fixed order.
 */
cp_status cp_attn_backward_delta(const void* o, const void* dout, float* delta, int64_t B,
                                 int64_t H, int64_t Sq, int64_t D, cp_dtype dtype, void* stream);

/* Flags of cp_attn_chunk_backward. */
#define CP_BWD_ACCUMULATE_DQ 1  /* dq += this chunk's share (else dq = share)        */
#define CP_BWD_ACCUMULATE_DKV 2 /* dk, dv += this Q shard's share (else dk, dv = it) */

/*
 * cp_attn_chunk_backward — one K/V chunk's share of the attention backward.
 *
 * Defined by: the derivative of O = softmax(scale Q K^T) V (see
 * cp_attn_backward_delta for the pages' training context), split by K/V chunk
 * as the ring splits the forward (Context parallelism guide (diffusers),
 * section Ring Attention). From the full rows' LSE and delta:
 *   P_ij  = exp(scale <q_i, k_j> - LSE_i)   (0 for masked pairs and rows with LSE = -inf)
 *   dS_ij = P_ij (<dO_i, v_j> - delta_i)
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i
 * Summing dq over a rank's chunks gives its full dQ (CP_BWD_ACCUMULATE_DQ);
 * adding every rank's dk, dv for a chunk gives that chunk's full dK, dV
 * (CP_BWD_ACCUMULATE_DKV). One chunk over the whole sequence is a Ulysses
 * rank's local backward.
 *
 *   q, dout [B][Sq][H][D] and k, v [B][Skv][H][D] in in_dtype (CP_BF16 or CP_F32);
 *   lse, delta [B][H][Sq] fp32 (lse in the cp_attn_chunk_partial convention);
 *   dq [B][Sq][H][D] and dk, dv [B][Skv][H][D] fp32, caller-allocated; with an
 *   ACCUMULATE flag the buffer must hold the running sum, else it is
 *   overwritten. causal, q_pos0, kv_pos0 and scale as in cp_attn_chunk_partial
 *   and equal to the forward's.
 *
 * Arithmetic: for bf16 inputs, bf16 MFMA products with fp32 accumulation; P
 * and dS are rounded to bf16 for their products (as P is in the forward). For
 * fp32 inputs every step is fp32 (the fp32 forward's companion). Each output element is
 * written once by one block (no atomics), so results are byte-identical on
 * repeat. Sq == 0 gives dk = dv = 0 (unchanged when accumulating); Skv == 0
 * gives dq = 0 (unchanged when accumulating). D in {64, 128}; Sq, Skv < 2^30.
 * Two kernel launches; no workspace. This is cp_ring_attention_backward with
 * one chunk.
 */
cp_status cp_attn_chunk_backward(const void* q, const void* k, const void* v, const void* dout,
                                 const float* lse, const float* delta, float* dq, float* dk,
                                 float* dv, int64_t B, int64_t H, int64_t Sq, int64_t Skv,
                                 int64_t D, cp_dtype in_dtype, float scale, int causal,
                                 int64_t q_pos0, int64_t kv_pos0, int flags, void* stream);

/* Gradient outputs of one K/V chunk: fp32 [B][len][H][D] each. */
typedef struct {
  float* dk;
  float* dv;
} cp_kv_grad;

/*
 * cp_ring_attention_backward — one ring rank's whole backward share: its Q
 * shard against P K/V chunks.
 *
 * Defined by: the derivative of the ring's attention (see
 * cp_attn_chunk_backward; Context parallelism guide (diffusers), sections Ring
 * Attention and Ring Anything Attention for the chunks and their uneven
 * lengths). Equal to P cp_attn_chunk_backward calls with dQ accumulated over
 * the chunks, in one pair of launches: every chunk's key tiles form one grid
 * for dK/dV, and the dQ kernel walks all chunks' keys per query tile.
 *
 *   q, dout [B][Sq][H][D] in in_dtype (CP_BF16 or CP_F32); chunks: HOST
 *   array of P descriptors (K/V in in_dtype, as for
 *   cp_ring_attention; pos0 drives causal masking, q_pos0 is the shard's first
 *   position); lse, delta [B][H][Sq] fp32 of the full rows.
 *   dq [B][Sq][H][D] fp32 = sum over the chunks of their dQ shares
 *   (+= with CP_BWD_ACCUMULATE_DQ).
 *   grads: HOST array of P cp_kv_grad; grads[c].dk / .dv receive chunk c's
 *   dK, dV share from this Q shard (+= with CP_BWD_ACCUMULATE_DKV).
 *   Zero-length chunks are skipped (their pointers may be null). P in 1..64.
 *   No output may overlap an input or another output. No workspace.
 * Arithmetic, determinism and limits as cp_attn_chunk_backward.
 */
cp_status cp_ring_attention_backward(const void* q, const cp_kv_chunk* chunks, int64_t P,
                                     const void* dout, const float* lse, const float* delta,
                                     float* dq, const cp_kv_grad* grads, int64_t B, int64_t H,
                                     int64_t Sq, int64_t D, cp_dtype in_dtype, float scale,
                                     int causal, int64_t q_pos0, int flags, void* stream);

/* Text describing the last failed call on this thread ("" after a successful
 * call). Valid until the next cp_* call on the same thread. */
const char* cp_last_error(void);

/* ABI version of this header (incremented on incompatible changes). */
#define CP_ATTN_ABI_VERSION 1
int cp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
