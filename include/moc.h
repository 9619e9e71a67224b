/*
 * moc.h - C ABI of libmoc, a Mixture-of-Contexts (MoC) attention layer for AMD MI355X (gfx950).
 *
 * The layer replaces dense self-attention: keys are mean-pooled per content-aligned chunk
 * (caption, frame, shot), every query scores the chunk descriptors by dot product, optional
 * retrieval is limited to earlier chunks by the causal routing mask, the top-k chunks are
 * picked, and exact softmax attention runs over the mandatory anchors (all caption tokens and
 * the query's own shot) plus the routed chunks.
 *   Source: "Mixture of Contexts for Long Video Generation | Summary" (greeksharifa.github.io),
 *   §3.1 Mixture of Contexts, §3.2 Attention Chunking and Routing, §3.3 Computation Efficiency;
 *   jxzklqfsx.com write-up of the paper, sections 注意力塊劃分與路由 and 計算效率.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except the moc_layout /
 *     moc_route_cfg / moc_varlen structs themselves, which are host structs read during the
 *     call only. The library never allocates or frees device memory and keeps no state between
 *     calls (beyond loaded kernels and a thread-local error string).
 *   - Q, K, V, O, dO, dQ, dK, dV are [B, H, L, d] contiguous (head-major: each head's tokens
 *     are contiguous rows of d elements), in the layout's dtype.
 *   - Calls only enqueue work on `stream` (a hipStream_t passed as void*; NULL = default
 *     stream) and return without synchronising. All argument checks run on the host before
 *     anything is enqueued, so a non-OK status means nothing ran.
 *   - Workspaces are sized with moc_workspace_bytes(). Distinct workspaces allow concurrent
 *     calls on distinct streams; calls sharing a workspace must be ordered by the caller.
 *   - Layout arrays live on the device, so their content (monotone offsets, contiguous shots,
 *     text on chunk boundaries) is a precondition that the host cannot check without a copy.
 *     The Python binding checks it on a host copy; a C caller can set moc_layout.check to have
 *     every call check it on the device first (see moc_check_layout).
 */
#ifndef MOC_H_
#define MOC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOC_OK = 0,
  MOC_EINVAL = 1,       /* null pointer, negative size, bad flag, aliasing */
  MOC_ESHAPE = 2,       /* a size outside the supported limits */
  MOC_EDTYPE = 3,       /* unknown dtype */
  MOC_EWORKSPACE = 4,   /* workspace pointer null or smaller than moc_workspace_bytes() */
  MOC_EUNSUPPORTED = 5, /* a valid request this build does not implement */
  MOC_EHIP = 6,         /* a HIP launch or runtime call failed */
  MOC_EINTERNAL = 7,    /* unexpected internal error (no C++ exception crosses the ABI) */
  MOC_ELAYOUT = 8       /* the layout content failed the check (moc_layout_status) */
} moc_status;

typedef enum { MOC_F32 = 0, MOC_BF16 = 1 } moc_dtype;

/* Workspace kinds for moc_workspace_bytes(). */
enum { MOC_OP_ROUTE = 0, MOC_OP_VARLEN = 1, MOC_OP_FWD = 2, MOC_OP_BWD = 3, MOC_OP_OUTER = 4 };

/* Hard limits of this build. */
#define MOC_MAX_C 1024        /* chunks per sequence */
#define MOC_MAX_TOPK 32       /* min(top_k, C) */
#define MOC_MAX_DROP_IN 16    /* max_drop_in */
#define MOC_MAX_SEG 256       /* segments of outer-loop routing */
#define MOC_MAX_TOPM 16       /* min(M, nseg) of outer-loop routing */

/*
 * Token layout (shared by all batch elements and heads). Chunks are content-aligned token
 * ranges (summary §3.2; write-up 內容對齊的塊劃分): chunk c is [chunk_offsets[c],
 * chunk_offsets[c+1]).
 *   chunk_offsets: device int32 [C+1], 0 = off[0] < off[1] < ... < off[C] = L (cu_seqlens style).
 *   chunk_shot:    device int32 [C], the shot id of each chunk; a shot's chunks are contiguous;
 *                  every text chunk carries -1, and no other chunk does.
 *   [text_begin, text_end): the caption tokens, a union of whole chunks; may be empty.
 *   dtype: MOC_F32 or MOC_BF16; d in {64, 128}; 1 <= C <= min(L, MOC_MAX_C).
 *   check: NULL, or a device uint32 word that turns on the device check of the content above.
 *          Every entry point then first runs the check kernel, which ORs the violations it
 *          finds (MOC_LAYOUT_* bits) into *check, and every kernel of the call does no work
 *          when *check is non-zero at its start - so a malformed layout is never used to index
 *          memory. The caller zeroes the word before the first call and reads it after the
 *          stream has run (moc_layout_status turns it into a status and a message). A word
 *          left non-zero keeps later calls that share it from running. Outputs of a rejected
 *          call are not written.
 */
typedef struct {
  int32_t B, H, L, d;
  int32_t dtype;
  int32_t C;
  const int32_t *chunk_offsets;
  const int32_t *chunk_shot;
  int32_t text_begin, text_end;
  uint32_t *check;
} moc_layout;

/* Bits of the layout check word (several may be set). */
#define MOC_LAYOUT_BAD_START 1u       /* chunk_offsets[0] != 0 */
#define MOC_LAYOUT_NOT_INCREASING 2u  /* chunk_offsets not strictly increasing */
#define MOC_LAYOUT_BAD_END 4u         /* chunk_offsets[C] != L */
#define MOC_LAYOUT_BAD_SHOT_ID 8u     /* a shot id below -1 */
#define MOC_LAYOUT_BAD_TEXT 16u       /* a chunk straddles the text range, or shot -1 is not
                                         exactly the chunks inside it */
#define MOC_LAYOUT_SHOT_SPLIT 32u     /* a shot's chunks are not contiguous */

/*
 * Routing configuration (summary §3.1-3.2; slides "Mixture of Contexts for Long Video
 * Generation", slides 11-14).
 *   top_k:  >= 0; the routed budget per query is min(top_k, #candidates).
 *           min(top_k, C) must not exceed MOC_MAX_TOPK.
 *   causal: 1 = an optional candidate chunk c must come before the query's chunk (c < chunk(t)).
 *   p_max:  context drop-off, in [0, 1]; 0 disables. p = u * p_max with u ~ U[0,1) and
 *           min(floor(p * min(top_k, C)), |T|) routed chunks are removed at random.
 *   lambda: context drop-in, >= 0; 0 disables. m ~ Poisson(lambda) truncated at max_drop_in
 *           extra chunks are added at random from the candidates not already routed.
 *   max_drop_in: in [0, MOC_MAX_DROP_IN] (used only when lambda > 0).
 *   seed:   key of the counter-based generator (SplitMix64, Steele-Lea-Flood 2014), so a
 *           draw depends only on (seed, b, h, t, stream, j).
 */
typedef struct {
  int32_t top_k;
  int32_t causal;
  float p_max;
  float lambda;
  int32_t max_drop_in;
  int32_t reserved;
  uint64_t seed;
} moc_route_cfg;

/*
 * Result of the index inversion (moc_build_varlen). All pointers point into the caller's
 * VARLEN workspace and stay valid while that workspace is not reused. Filled by
 * moc_build_varlen on the host side (pointers, sizes) and on the device (contents).
 *   S:          selection width, = min(top_k, C) + (lambda > 0 ? max_drop_in : 0).
 *   bucket_off: [B*H*C + 1] exclusive prefix of the number of queries that routed to each
 *               (b, h, chunk) bucket; bucket_off[B*H*C] = total routed selections.
 *   bucket_q:   [B*H*L*S] the query token ids of each bucket, ascending within a bucket.
 *   slot:       [B*H*L*S] for selection j of query (b,h,t): its position in bucket_q (the row
 *               of that (query, chunk) partial result), -1 for padding.
 *   rtiles:     [max_rtiles][2] routed work tiles (bucket id, first position in the bucket),
 *               n_rtiles[0] of them valid; each tile covers up to tile_rows queries.
 *   atiles:     [max_atiles][6] anchor work tiles (q0, q1, key range 1 [a0,a1), key range 2
 *               [b0,b1)), n_atiles[0] valid, shared by every (b, h). n_atiles[1..9] split the
 *               B*H*n_atiles[0] anchor items (b, h, tile) into 8 contiguous ranges of about
 *               equal cost (a tile costs its 64-key tiles plus 4), one per XCD: range x is
 *               [n_atiles[1+x], n_atiles[2+x]), at most ceil(1.25 B*H*max_atiles / 8) items.
 *               n_atiles[16..39] are claim counters of the attention kernels' work items,
 *               zeroed at the start of every attention call: attention calls that share one
 *               moc_varlen must not run at the same time.
 *   ktiles:     [max_ktiles][6] key tiles of the backward (k0, k1, chunk or -1 for text,
 *               anchor query range q0, q1, text split index), n_ktiles[0] valid, shared by every
 *               (b, h). A key tile never straddles a chunk; text keys, which every query
 *               attends, are split into n_text_split query ranges.
 *   routed_max: B*H*L*S, the most routed (query, chunk) rows any routing of this shape has.
 *   routed_cap: routed rows the attention workspaces are sized for (moc_attend_workspace_bytes);
 *               routed_max after moc_build_varlen, lowered with moc_varlen_set_capacity.
 *   status:     device word in the VARLEN workspace. Every attention call first writes it: bit 1
 *               when the routing's total (bucket_off[B*H*C]) exceeds routed_cap, bit 2 when the
 *               layout check word (moc_layout.check) is set; all kernels of the call then do no
 *               work. moc_varlen_status reads it.
 */
typedef struct {
  int32_t S;
  int32_t tile_rows;
  int32_t max_rtiles;
  int32_t max_atiles;
  int32_t *bucket_off;
  int32_t *bucket_q;
  int32_t *slot;
  int32_t *rtiles;
  int32_t *n_rtiles;
  int32_t *atiles;
  int32_t *n_atiles;
  int32_t *scratch;     /* internal: per-tile counts and offsets of the inversion */
  int32_t max_ktiles;
  int32_t n_text_split;
  int32_t *ktiles;
  int32_t *n_ktiles;
  int64_t routed_max;
  int64_t routed_cap;
  uint32_t *status;
} moc_varlen;

/* moc_varlen.status bits */
#define MOC_VARLEN_OVER_CAPACITY 1u  /* more routed rows than routed_cap */
#define MOC_VARLEN_BAD_LAYOUT 2u     /* the layout check word was non-zero */

/* Selection width S for a route configuration and chunk count (see moc_varlen.S). */
int32_t moc_sel_width(const moc_route_cfg *cfg, int32_t C);

/* Bytes of device workspace needed by the entry point `op` (MOC_OP_*); 0 on invalid
 * arguments (see moc_last_error()). MOC_OP_OUTER is sized for MOC_MAX_SEG segments (the
 * segment count is not part of the layout). */
size_t moc_workspace_bytes(const moc_layout *lay, const moc_route_cfg *cfg, int32_t op);

/*
 * Workspace sizing from the real routing instead of its static bound. The attention workspaces
 * hold one row per routed (query, chunk) pair - partial outputs in the forward, partial dQ rows
 * and gathered query images in the backward - and moc_workspace_bytes sizes them for
 * B*H*L*S rows, which drop-in noise makes several times the rows a routing really has.
 *   moc_varlen_total: the routing's total routed rows, bucket_off[B*H*C]. It waits for
 *     `stream`, then copies the count to the host. With lay->check set it reads the check word
 *     first and returns MOC_ELAYOUT (no total) when the layout was rejected.
 *   moc_varlen_set_capacity: sets vl->routed_cap (0 <= routed_cap <= vl->routed_max). Host
 *     only; the varlen contents are unchanged. A capacity at least the total (a total from
 *     moc_varlen_total, or a bound the caller trusts for its routing noise) gives the same
 *     results as the default.
 *   moc_attend_workspace_bytes: bytes of the MOC_OP_FWD or MOC_OP_BWD workspace for
 *     vl->routed_cap rows; moc_attend_fwd(_mx) and moc_attend_bwd require at least this much.
 *     0 on invalid arguments.
 *   moc_varlen_status: waits for `stream` and reads vl->status: MOC_EWORKSPACE when the last
 *     attention call found more routed rows than routed_cap (it then wrote none of its outputs),
 *     MOC_ELAYOUT when the layout check word was set, MOC_OK otherwise.
 */
moc_status moc_varlen_total(const moc_layout *lay, const moc_varlen *vl, int64_t *total,
                            void *stream);
moc_status moc_varlen_set_capacity(moc_varlen *vl, int64_t routed_cap);
size_t moc_attend_workspace_bytes(const moc_layout *lay, const moc_varlen *vl, int32_t op);
moc_status moc_varlen_status(const moc_varlen *vl, void *stream);

/*
 * Mean-pooled chunk keys (summary §3.1: each chunk is represented by the mean of its keys;
 * slides, slide 11; write-up 計算效率: on-the-fly segmented mean).
 *   kbar[b,h,c,:] = RN32( RN64(sum_{t in chunk c} K[b,h,t,:]) / n_c ): the sum is accumulated
 *   in double-double (exact for every bf16 input and for fp32 inputs whose exponents span
 *   < ~80 binades), divided once in binary64 and rounded to nearest-even binary32.
 *   K: [B,H,L,d] layout dtype. kbar: device float [B,H,C,d], fully overwritten.
 */
moc_status moc_pool_keys(const moc_layout *lay, const void *K, float *kbar, void *stream);

/*
 * Routing (summary §3.1-3.2; write-up 計算效率: mandatory links are masked before top-k).
 * For each (b,h,t): candidates are chunks c that are not text, not in the query's own shot,
 * and (causal) c < chunk(t); score s_c = q_t . kbar_c (binary32 accumulation of exact
 * products); the min(top_k, #candidates) highest scores are kept (an exact tie keeps the
 * lower chunk id; for bf16 queries with C <= 128, scores within 2^-16 relative of each other
 * count as tied); then drop-off and drop-in are applied when enabled.
 *   sel:  device int32 [B,H,L,S], chunk ids ascending, -1 padded; nsel: int32 [B,H,L].
 *   ws:   MOC_OP_ROUTE workspace (may be NULL when its size is 0).
 */
moc_status moc_route(const moc_layout *lay, const moc_route_cfg *cfg, const void *Q,
                     const float *kbar, int32_t *sel, int32_t *nsel, void *ws, size_t ws_bytes,
                     void *stream);

/*
 * moc_route without a workspace, for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the same routing, with
 * the same results, whose only scratch - the three bf16 terms of kbar that the MFMA router reads,
 * B*H*C*d*6 bytes for bf16 queries, none for fp32 - lives in a static 16 MiB device buffer that
 * the library holds on every GPU it runs on until the process ends. Allocates nothing and calls
 * no allocating routine; the buffer's device address is looked up once per GPU on the first call
 * there. Every call on one GPU shares that buffer and it keeps the last call's contents (it is
 * fully rewritten before it is read): calls that overlap on one GPU, on different streams or
 * from different threads, race and must be ordered by the caller.
 *   Limit: B*H*C*d*6 <= 16 MiB (e.g. 12 heads x 1,024 chunks x d = 128 fits); a larger
 *   request returns MOC_ESHAPE before anything is enqueued.
 *   Arguments, outputs and every other rule as for moc_route.
 */
moc_status moc_route_noalloc(const moc_layout *lay, const moc_route_cfg *cfg, const void *Q,
                             const float *kbar, int32_t *sel, int32_t *nsel, void *stream);

/*
 * Outer-loop context routing (summary, Appendix I: routing on two levels - segments are
 * ranked by comparing the averaged queries of the current block with the averaged keys of each
 * other segment, and the chunk router then only considers the best M segments; the mandatory
 * context is kept). Segments are given groups of whole chunks; a query's block is its own
 * segment.
 *   seg_chunk: device int32 [nseg+1], 0 = seg_chunk[0] < ... < seg_chunk[nseg] = C; segment s
 *              is chunks [seg_chunk[s], seg_chunk[s+1]) and holds only text chunks or only
 *              video chunks (a precondition, like the layout's content).
 *   nseg in [1, MOC_MAX_SEG]; M >= 0 with min(M, nseg) <= MOC_MAX_TOPM; causal in {0, 1}.
 *   For each (b, h) and query segment sq: qseg = the mean of the segment's queries and kseg[s]
 *   = the mean of segment s's keys, both pooled like moc_pool_keys; the candidates are video
 *   segments s != sq (and s < sq when causal); score = qseg . kseg[s] (binary32
 *   accumulation); the min(M, #candidates) highest are kept, an exact tie keeping the lower
 *   segment id.
 *   seg_sel:   device int32 [B,H,nseg,min(M, nseg)], segment ids ascending, -1 padded.
 *   seg_nsel:  device int32 [B,H,nseg].
 *   cand_mask: device uint32 [B,H,C,ceil(C/32)]: bit c' of row (b,h,c) is set iff chunk c'
 *              lies in chunk c's segment or in a segment picked for it; the input of
 *              moc_route_masked.
 *   Q, K: [B,H,L,d] layout dtype. ws: MOC_OP_OUTER workspace (segment offsets and features).
 */
moc_status moc_route_outer(const moc_layout *lay, const int32_t *seg_chunk, int32_t nseg,
                           int32_t M, int32_t causal, const void *Q, const void *K,
                           int32_t *seg_sel, int32_t *seg_nsel, uint32_t *cand_mask, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * Inner routing of outer-loop context routing: moc_route with one more condition - chunk c is
 * a candidate of query t only if bit c of cand_mask row (b, h, chunk(t)) is set. Drop-in draws
 * from the same restricted candidates. The mandatory anchors are unaffected.
 *   cand_mask: device uint32 [B,H,C,ceil(C/32)] (as written by moc_route_outer).
 *   Every other argument, output and workspace as for moc_route.
 */
moc_status moc_route_masked(const moc_layout *lay, const moc_route_cfg *cfg, const void *Q,
                            const float *kbar, const uint32_t *cand_mask, int32_t *sel,
                            int32_t *nsel, void *ws, size_t ws_bytes, void *stream);

/*
 * Index inversion (write-up 計算效率: packing the (query, key-group) pairs into one
 * variable-length attention problem). Turns per-query chunk lists into per-(b,h,chunk) query
 * buckets (stable: ascending query id), the slot map, routed and anchor work tiles, and
 *   pair_count[b,h] = sum_t |Omega(t)| (int64, device), Omega = text U own shot U routed chunks.
 * `out` is filled with pointers into ws (MOC_OP_VARLEN workspace).
 */
moc_status moc_build_varlen(const moc_layout *lay, const moc_route_cfg *cfg, const int32_t *sel,
                            const int32_t *nsel, moc_varlen *out, int64_t *pair_count, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * Attention forward over the routed key sets (summary §3.1: Attn(q_i) =
 * softmax(q_i K_Omega^T / sqrt(d)) V_Omega; no token-level causal mask inside Omega).
 *   O:   [B,H,L,d] layout dtype; lse: device float [B,H,L], natural-log softmax denominator.
 *   softmax_scale: > 0 (usually 1/sqrt(d)).
 *   ws:  workspace of moc_attend_workspace_bytes(lay, vl, MOC_OP_FWD) bytes (per-(query, routed
 *        chunk) partial results in fp32 for vl->routed_cap rows; moc_workspace_bytes(...,
 *        MOC_OP_FWD) is the size at the default capacity).
 *   O and lse must not alias Q, K or V.
 */
moc_status moc_attend_fwd(const moc_layout *lay, const moc_varlen *vl, const void *Q,
                          const void *K, const void *V, float softmax_scale, void *O, float *lse,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * MXFP8 quantisation of Q or K for the quantised-scores forward (summary §5 Conclusion,
 * write-up 結論 and slides, slide 21 name quantisation as a direction for faster kernels and fix
 * no format). Format: OCP Microscaling MXFP8 - E4M3 elements (OCP OFP8: bias 7, largest finite
 * 448, no infinities) and, per block of 32 consecutive elements of a row, the E8M0 scale code
 * E + 127 with E = floor(log2(max |x|)) - 8 clamped below at -127 (-127 for an all-zero
 * block). Element code: x * 2^-E rounded to the nearest E4M3 value, ties to even, saturated
 * to +-448; a negative value that rounds to zero is coded 0x80.
 *   X:      device bf16 [B,H,L,d] (the layout's dtype must be MOC_BF16).
 *   codes:  device uint8 [B,H,Lp,d], Lp = L rounded up to a multiple of 64; rows >= L zero.
 *   scales: device uint8 [B,H,Lp,d/32]; rows >= L zero.
 * Both outputs are fully overwritten. Inputs must be finite.
 */
moc_status moc_mx_quantize(const moc_layout *lay, const void *X, uint8_t *codes, uint8_t *scales,
                           void *stream);

/*
 * Attention forward with quantised scores: moc_attend_fwd with the scores computed from the
 * MXFP8 codes and scales of Q and K (as written by moc_mx_quantize) on the block-scaled fp8
 * matrix cores. The result is the attention of the dequantised Q' = code * 2^E and K' over the
 * same key sets, with fp32 accumulation; softmax and P.V as in moc_attend_fwd.
 *   Qc, Kc: device uint8 [B,H,Lp,d]; Qs, Ks: device uint8 [B,H,Lp,d/32].
 *   V: bf16 [B,H,L,d]; O: bf16 [B,H,L,d]; lse: float [B,H,L]; the layout's dtype must be
 *   MOC_BF16. ws: as for moc_attend_fwd. O and lse must not alias an input.
 */
moc_status moc_attend_fwd_mx(const moc_layout *lay, const moc_varlen *vl, const uint8_t *Qc,
                             const uint8_t *Qs, const uint8_t *Kc, const uint8_t *Ks,
                             const void *V, float softmax_scale, void *O, float *lse, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * MXFP8 quantisation of V along the key axis, for the quantised-values forward (the same pages
 * name quantisation and the key/value layout as directions for faster kernels). In P.V the
 * sum runs over keys, so the blocks that share a scale run along the keys: for every (b, h, dim)
 * column, blocks of 32 consecutive keys from key 0, each coded with the rule of moc_mx_quantize
 * (E8M0 scale, E4M3 elements, ties to even, saturation at +-448). The output is the attention's
 * tile layout, so that the forward copies each 64-key tile verbatim:
 *   vq: device uint8 [B,H,Lp/64,d,80], Lp = L rounded up to a multiple of 64, of
 *       moc_mx_quantize_v_bytes(lay) bytes. Row (tile j, dim e) holds, at byte 32 b + p
 *       (block b = 0, 1; p = 0..31), the code of key 64 j + 32 b + s(p), where s swaps bits 3
 *       and 4 of p; at bytes 64 and 65 the scale codes of blocks 0 and 1; bytes 66-79 zero.
 *       Keys >= L are coded as zero. Fully overwritten.
 *   V: device bf16 [B,H,L,d] (the layout's dtype must be MOC_BF16); inputs must be finite.
 */
size_t moc_mx_quantize_v_bytes(const moc_layout *lay);
moc_status moc_mx_quantize_v(const moc_layout *lay, const void *V, uint8_t *vq, void *stream);

/*
 * Attention forward with quantised scores and values: moc_attend_fwd_mx with V given as the
 * tiles of moc_mx_quantize_v, and P.V on the block-scaled fp8 matrix cores as well. The
 * softmax weights are rounded to E4M3 (ties to even) before they multiply V, and the row sums
 * use the unrounded weights: against the attention of the dequantised Q', K', V' the output
 * moves by at most 2^-4 sum_j p_j |v'_j| / l + sum_j min(2^-10, p_j) |v'_j| / l per element
 * (p_j = exp of the scaled score minus the row maximum, l = sum_j p_j), plus fp32 and bf16
 * output rounding; lse is computed from the unrounded weights.
 *   Qc, Qs, Kc, Ks: as for moc_attend_fwd_mx; Vq: the output of moc_mx_quantize_v.
 *   O: bf16 [B,H,L,d]; lse: float [B,H,L]; ws: as for moc_attend_fwd (the transposed V copy
 *   of that workspace is not used). O and lse must not alias an input.
 */
moc_status moc_attend_fwd_mxv(const moc_layout *lay, const moc_varlen *vl, const uint8_t *Qc,
                              const uint8_t *Qs, const uint8_t *Kc, const uint8_t *Ks,
                              const uint8_t *Vq, float softmax_scale, void *O, float *lse,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * Attention backward with the routed sets held fixed (summary §3.1 and Appendix A: top-k is
 * not differentiable; gradients reach the selected keys and values only).
 *   Inputs: Q, K, V, O, lse from moc_attend_fwd, dO. Outputs dQ, dK, dV [B,H,L,d] in the
 *   layout dtype, fully overwritten. ws: workspace of moc_attend_workspace_bytes(lay, vl,
 *   MOC_OP_BWD) bytes (fp32 row statistics, per-(query, routed chunk) dQ partials and gathered
 *   query images for vl->routed_cap rows, text-key partials). Deterministic: no float
 *   atomics; partial results are merged in a fixed order. bf16 layouts only (an fp32 layout
 *   returns MOC_EUNSUPPORTED).
 */
moc_status moc_attend_bwd(const moc_layout *lay, const moc_varlen *vl, const void *Q,
                          const void *K, const void *V, const void *O, const float *lse,
                          const void *dO, float softmax_scale, void *dQ, void *dK, void *dV,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Layout content check (summary §3.2: chunks follow frame, shot and caption boundaries;
 * write-up 計算效率: the boundary tables of the packed sequence).
 * moc_check_layout enqueues only the check kernel on `stream`: one workgroup reads
 * chunk_offsets[0..C] and chunk_shot[0..C-1] and ORs the MOC_LAYOUT_* bits of every violation
 * into *lay->check (which must be set). The other entry points run the same kernel first
 * whenever lay->check is set.
 */
moc_status moc_check_layout(const moc_layout *lay, void *stream);

/* The same check on host arrays (offsets [C+1], shot ids [C]): the MOC_LAYOUT_* bits, 0 for a
 * valid layout. Needs no GPU. */
uint32_t moc_layout_check_host(const int32_t *chunk_offsets, const int32_t *chunk_shot, int32_t C,
                               int32_t L, int32_t text_begin, int32_t text_end);

/* MOC_OK for a check word of 0; otherwise MOC_ELAYOUT, with the violations spelled out in
 * moc_last_error(). */
moc_status moc_layout_status(uint32_t word);

/* Host-side helper: the drop-in Poisson thresholds the routing kernel uses,
 * thr[i] = min(2^32, floor(2^32 * P(m <= i))) for i < max_drop_in (binary64, C library exp). */
moc_status moc_poisson_thresholds(float lambda, int32_t max_drop_in, uint64_t *thr);

const char *moc_status_string(moc_status s);
/* Message of the last non-OK status returned on the calling thread. */
const char *moc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOC_H_ */
