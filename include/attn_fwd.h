/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) fused bf16 forward attention.
 *
 * Operation (snilld.dk page "Open source attention kernel in HIP beats AITER
 * v3 on MI300X", section "Hvordan kernen arbejder" / How the kernel works):
 * for every batch b, head h and query row i,
 *
 *     O[b,h,i,:] = softmax_j( Q[b,h,i,:] . K[b,h,j,:] / sqrt(128) ) V[b,h,j,:]
 *
 * without a mask (attn_fwd_bf16_masked adds a causal one), head_dim fixed at
 * 128, one head count shared by Q, K and V (attn_fwd_bf16_gqa allows fewer
 * K/V heads; attn_fwd_bf16_varlen takes packed sequences of their own lengths;
 * attn_fwd_bf16_partial and attn_fwd_bf16_merge cut the keys into shards), any
 * query length Sq and key length Sk (cross-attention allowed), inputs read in
 * the BSHD or BHSD layout without a transpose (same page, section "Hvad er
 * udgivet" / What was released).  Output is bf16, rounded per call in one of
 * three modes (tilnote.io page on the MoonMath HIP attention kernel, section
 * on its performance figures; snilld.dk page, section "Numerik samlet et
 * sted" / Numerics in one place).
 *
 * Numerics: logits and softmax in fp32, both products on bf16 matrix cores
 * with fp32 accumulation, the softmax weights rounded to bf16 (nearest-even)
 * for the second product, and one final rounding of each fp32 output to bf16
 * in the requested mode.  Results are deterministic: repeated calls on the
 * same inputs give identical bits.  A NaN logit makes its query row NaN; a
 * +Inf logit makes its row NaN; a -Inf logit removes that key from the row.
 *
 * Layout (element offsets, d = 128, all four tensors contiguous, O shaped
 * like Q):
 *     BSHD: Q/O [B, Sq, H, 128], K/V [B, Sk, H, 128];
 *           (b, s, h, c) at ((b*S + s)*H + h)*128 + c
 *     BHSD: Q/O [B, H, Sq, 128], K/V [B, H, Sk, 128];
 *           (b, h, s, c) at ((b*H + h)*S + s)*128 + c
 *
 * Ownership: the caller owns every buffer, including the workspace of
 * attn_fwd_bf16_ws.  The library allocates nothing on the device, never
 * synchronises, and keeps no state beyond a once-filled per-device cache of
 * the architecture and compute-unit count; calls are thread-safe.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_FWD_ABI_VERSION 9

typedef enum {
    ATTN_LAYOUT_BSHD = 0, /* [B, S, H, 128] */
    ATTN_LAYOUT_BHSD = 1  /* [B, H, S, 128] */
} attn_layout_t;

/* Output rounding, fp32 -> bf16, applied once per output element. */
typedef enum {
    ATTN_ROUND_RTNE = 0, /* to nearest, ties to even */
    ATTN_ROUND_RTNA = 1, /* to nearest, ties away from zero */
    ATTN_ROUND_RTZ = 2   /* toward zero */
} attn_round_t;

/* Key mask of attn_fwd_bf16_masked: query row i attends to keys j <= i + off. */
typedef enum {
    ATTN_MASK_NONE = 0,               /* every key */
    ATTN_MASK_CAUSAL = 1,             /* off = 0: diagonal at the top left */
    ATTN_MASK_CAUSAL_BOTTOM_RIGHT = 2 /* off = Sk - Sq: diagonal at the bottom right */
} attn_mask_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,   /* a tensor pointer is NULL */
    ATTN_ERR_SIZE = 2,   /* B, H, Sq or Sk < 1, H > 2^18, or a size overflows the index types */
    ATTN_ERR_LAYOUT = 3, /* layout is not an attn_layout_t value */
    ATTN_ERR_ROUND = 4,  /* round_mode is not an attn_round_t value */
    ATTN_ERR_ALIGN = 5,  /* a pointer is not 16-byte aligned */
    ATTN_ERR_ALIAS = 6,  /* o overlaps q, k or v */
    ATTN_ERR_DEVICE = 7, /* the current device is not gfx950 or cannot be queried, or the stream is another device's */
    ATTN_ERR_HIP = 8,    /* the kernel launch failed */
    ATTN_ERR_WORKSPACE = 9, /* the workspace is smaller than attn_fwd_bf16_workspace_size reports */
    ATTN_ERR_MASK = 10,     /* mask is not an attn_mask_t value */
    ATTN_ERR_HEADS = 11,    /* H is not a multiple of H_kv */
    ATTN_ERR_SCRATCH = 12   /* attn_fwd_bf16_gqa_noalloc: the split needs more than its static scratch */
} attn_status_t;

/*
 * attn_fwd_bf16 -- enqueue O = softmax(Q K^T / sqrt(128)) V on `stream`.
 *
 *   q, k, v : device pointers to bf16 bit patterns (uint16), layout above.
 *   o       : device pointer receiving the bf16 output, shaped like q.
 *   B, H    : batch size and head count (>= 1).
 *   Sq, Sk  : query and key lengths (>= 1), independent of each other.
 *   layout  : attn_layout_t, shared by all four tensors.
 *   round_mode : attn_round_t, the output rounding.
 *   stream  : hipStream_t of the current device to enqueue on (NULL = its
 *             null stream).
 *
 * Returns ATTN_OK once the kernel is enqueued; the call is asynchronous and
 * O is valid after the stream reaches that point.  Argument errors
 * (ATTN_ERR_NULL .. ATTN_ERR_ALIAS) are detected before any HIP call and
 * nothing is launched.  ATTN_ERR_DEVICE: the current device is not gfx950, or
 * the stream belongs to another device (checked with hipStreamGetDevice).
 * ATTN_ERR_HIP: a launch was rejected (each launch's own status; an earlier
 * error of the calling thread is neither reported nor cleared).  Faults inside
 * the kernel surface at the caller's next synchronisation, as for any HIP
 * kernel.
 */
int attn_fwd_bf16(const void *q, const void *k, const void *v, void *o,
                  int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                  int layout, int round_mode, void *stream);

/*
 * attn_fwd_bf16_ws -- the same operation, allowed to split the key range.
 *
 * Each workgroup of the kernel owns 256 query rows of one (batch, head) and
 * the machine runs one per compute unit at a time.  When B*H*ceil(Sq/256)
 * leaves the last round of compute units partly idle (a short Sq against a
 * long Sk, few heads), the work items of that round run as several
 * workgroups over consecutive key ranges each, and a second kernel merges
 * their partial results by the same max-shifted sums the online softmax uses
 * (the split-over-keys arrangement the FlashAttention family uses for long
 * keys), then rounds once in the requested mode.
 *
 *   workspace       : device memory of at least the size
 *                     attn_fwd_bf16_workspace_size reports for this shape,
 *                     16-byte aligned, not overlapping q, k, v or o; it holds
 *                     fp32 partial rows and is only read by the same call.
 *                     May be NULL when that size is 0.
 *   workspace_bytes : its size in bytes.
 *   other arguments : as attn_fwd_bf16.
 *
 * Same status codes as attn_fwd_bf16, plus ATTN_ERR_NULL (workspace NULL but
 * needed), ATTN_ERR_WORKSPACE (too small), ATTN_ERR_ALIGN / ATTN_ERR_ALIAS for
 * the workspace.  When the reported size is 0 this is exactly attn_fwd_bf16.
 * A split changes the order of the fp32 sums, so its results can differ from
 * attn_fwd_bf16's in the last bits (both are within the same tolerance of the
 * exact result); for a given shape and device they are deterministic.  Calls
 * that share a workspace must be ordered on one stream.
 */
int attn_fwd_bf16_ws(const void *q, const void *k, const void *v, void *o,
                     int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                     int layout, int round_mode, void *workspace,
                     int64_t workspace_bytes, void *stream);

/*
 * attn_fwd_bf16_masked -- attn_fwd_bf16 with a key mask.
 *
 * The snilld.dk page names the causal mask among what the kernel it describes
 * lacks and what autoregressive serving needs (sections "Hvad er udgivet" /
 * What was released and "Autoregressiv serving, de praktiske hager") without
 * defining it; this is the usual definition.  With ATTN_MASK_CAUSAL query row
 * i attends to the keys j <= i (row 0 sees key 0); with
 * ATTN_MASK_CAUSAL_BOTTOM_RIGHT to the keys j <= i + Sk - Sq (the last row
 * sees every key, as when Sq new queries follow Sk - Sq cached keys).  Masked
 * keys take no part in the row's softmax.  A row with no visible key (only
 * possible at the bottom right with Sq > Sk: rows i < Sq - Sk) is NaN, the
 * 0/0 of an empty softmax, as for a row whose logits are all -Inf.  A NaN or
 * Inf in V at a masked key is outside the contract (the matrix core
 * multiplies it by a zero weight).  ATTN_MASK_NONE is exactly attn_fwd_bf16.
 *
 *   mask            : attn_mask_t.
 *   other arguments : as attn_fwd_bf16.
 *
 * Status codes as attn_fwd_bf16, plus ATTN_ERR_MASK.  The work of a causal
 * call is the visible (query, key) pairs only: about half of the unmasked
 * call's for Sq = Sk.
 */
int attn_fwd_bf16_masked(const void *q, const void *k, const void *v, void *o,
                         int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                         int layout, int round_mode, int mask, void *stream);

/*
 * attn_fwd_bf16_gqa -- attn_fwd_bf16_masked with fewer K/V heads than query
 * heads (grouped-query attention).
 *
 * The snilld.dk page lists GQA among what the kernel it describes leaves out
 * (section "Hvad er udgivet" / What was released) without defining it; this
 * is the usual grouping.  K and V hold H_kv heads, H must be a multiple of
 * H_kv, and query head h attends with K/V head h / (H / H_kv), so
 * consecutive query heads share one K/V head (H_kv = 1: multi-query
 * attention; H_kv = H: attn_fwd_bf16_masked).
 *
 *   q, o    : [B, Sq, H, 128] (BSHD) or [B, H, Sq, 128] (BHSD).
 *   lse     : NULL, or device memory for B*H*Sq fp32 values laid out
 *             [B, H, Sq] (either layout), 4-byte aligned, not overlapping
 *             q, k, v or o: receives each query row's log-sum-exp
 *             ln(sum_j exp(q.k_j / sqrt(128))) over the keys the row sees,
 *             the per-row statistic a backward pass or a merge of key
 *             ranges needs (the FlashAttention family's softmax_lse); -Inf
 *             for a row that sees no key or only -Inf logits, NaN where the
 *             output row is NaN.  Computed in fp32 from the row's running
 *             maximum and sum.
 *   k, v    : [B, Sk, H_kv, 128] (BSHD) or [B, H_kv, Sk, 128] (BHSD).
 *   H_kv    : K/V head count, >= 1, dividing H.
 *   mask    : attn_mask_t, as attn_fwd_bf16_masked.
 *   other arguments : as attn_fwd_bf16.
 *
 * Status codes as attn_fwd_bf16_masked, plus ATTN_ERR_HEADS (H not a
 * multiple of H_kv; H_kv < 1 is ATTN_ERR_SIZE) and ATTN_ERR_ALIGN /
 * ATTN_ERR_ALIAS for lse.
 */
int attn_fwd_bf16_gqa(const void *q, const void *k, const void *v, void *o,
                      float *lse, int64_t B, int64_t H, int64_t H_kv, int64_t Sq,
                      int64_t Sk, int layout, int round_mode, int mask, void *stream);

/*
 * attn_fwd_bf16_varlen -- attn_fwd_bf16_gqa over a batch of sequences of
 * their own lengths, packed one after another (variable-length batching).
 *
 * The snilld.dk page lists varlen batching among what the kernel it
 * describes leaves out and what serving with mixed lengths needs (sections
 * "Hvad er udgivet" / What was released and "Autoregressiv serving, de
 * praktiske hager") without defining it; this is the packed layout of
 * FlashAttention's varlen interface.  Sequence b holds the query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and o and the key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v, and attends only within
 * itself, as its own fixed-length problem (a causal mask is aligned per
 * sequence; a sequence with queries but no keys gives NaN rows).
 *
 *   q, o    : [total_q, H, 128] bf16 (one layout, the rows of all sequences
 *             in order; row t, head h at (t*H + h)*128).
 *   lse     : NULL, or H*total_q fp32 laid out [H, total_q] (packed row
 *             index), as attn_fwd_bf16_gqa's (-Inf for a sequence without
 *             keys).
 *   k, v    : [total_k, H_kv, 128].
 *   cu_seqlens_q, cu_seqlens_k : device pointers to B+1 int32 offsets,
 *             non-decreasing, from 0 to total_q (total_k); 4-byte aligned.
 *             Read by the kernel; offsets outside [0, total] are clamped to
 *             it, so no access leaves the tensors whatever they hold (the
 *             results are then unspecified).
 *   B       : number of sequences; H, H_kv as attn_fwd_bf16_gqa.
 *   total_q, total_k : packed row counts (>= 1).
 *   max_seqlen_q : at least every sequence's query length: the grid covers
 *             ceil(max_seqlen_q / 256) q-tiles per sequence and head; rows
 *             of a longer sequence past that are not written.
 *   round_mode, mask, stream : as attn_fwd_bf16_gqa.
 *
 * Status codes as attn_fwd_bf16_gqa (ATTN_ERR_ALIGN also for the offset
 * arrays, ATTN_ERR_ALIAS also when o or lse overlaps them).  Single pass.
 */
int attn_fwd_bf16_varlen(const void *q, const void *k, const void *v, void *o,
                         float *lse, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                         int64_t B, int64_t H, int64_t H_kv, int64_t total_q,
                         int64_t total_k, int64_t max_seqlen_q, int round_mode,
                         int mask, void *stream);

/*
 * attn_fwd_bf16_gqa_ws -- attn_fwd_bf16_gqa allowed to split the key range,
 * as attn_fwd_bf16_ws does for the unmasked call.
 *
 * Without a mask the split is attn_fwd_bf16_ws's.  Under a causal mask the
 * work items (256 query rows of one head) see different numbers of keys, and
 * a split item cuts the key tiles its rows see into equal consecutive
 * ranges.  When the items are nearly equal (the first q-tile of a head sees
 * at least 3/4 of the key tiles of its last: a short Sq against a long Sk
 * with the bottom-right diagonal, the shape of a prefill after cached keys)
 * the last, partly filled round of compute units is split.  When they are
 * not and all of them fit in one round (few heads of a long sequence), every
 * item is split into up to 8 ranges, for up to twice as many workgroups as
 * compute units: the longest item would otherwise set the time alone.
 * Otherwise the call runs single-pass (longest items first).  With lse, the
 * rows of split items get the log-sum-exp of the merged sums.
 *
 *   workspace       : at least attn_fwd_bf16_gqa_workspace_size(B, H, Sq, Sk,
 *                     mask) bytes, 16-byte aligned, not overlapping q, k, v,
 *                     o or lse; may be NULL when that size is 0.
 *   workspace_bytes : its size in bytes.
 *   other arguments : as attn_fwd_bf16_gqa.
 *
 * Status codes as attn_fwd_bf16_gqa, plus those attn_fwd_bf16_ws adds for
 * the workspace.  Results can differ from attn_fwd_bf16_gqa's in the last
 * bits where a split happens (the order of the fp32 sums); deterministic for
 * a given shape and device.  Calls that share a workspace must be ordered on
 * one stream.
 */
int attn_fwd_bf16_gqa_ws(const void *q, const void *k, const void *v, void *o,
                         float *lse, int64_t B, int64_t H, int64_t H_kv, int64_t Sq,
                         int64_t Sk, int layout, int round_mode, int mask,
                         void *workspace, int64_t workspace_bytes, void *stream);

/*
 * attn_fwd_bf16_gqa_noalloc -- attn_fwd_bf16_gqa_ws without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The key-range split keeps its partial rows and (maximum, sum) pairs in a
 * static device array of the library (65 MiB, enough for every split plan
 * on a device of up to 256 compute units: 2 x 256 blocks of 256 rows x 130
 * floats), one per device, held from the library's load until the process
 * ends.  The call allocates and frees nothing.  Every call on a device
 * shares that device's array: calls that may overlap on one device (on
 * different streams, or from different threads) race and must be ordered by
 * the caller.  Nothing in the array has to start at zero: each call writes
 * every partial it reads.
 *
 * Arguments, results and status codes as attn_fwd_bf16_gqa_ws (the same
 * plan, kernels and bits), without workspace and workspace_bytes; a plan
 * that needs more than the static array returns ATTN_ERR_SCRATCH and
 * launches nothing.
 */
int attn_fwd_bf16_gqa_noalloc(const void *q, const void *k, const void *v, void *o,
                              float *lse, int64_t B, int64_t H, int64_t H_kv, int64_t Sq,
                              int64_t Sk, int layout, int round_mode, int mask, void *stream);

/*
 * attn_fwd_bf16_gqa_workspace_size -- bytes of workspace attn_fwd_bf16_gqa_ws
 * needs for this shape and mask on the current device (0: it will not
 * split; the K/V head count does not matter).  Returns ATTN_ERR_NULL,
 * ATTN_ERR_SIZE, ATTN_ERR_MASK or ATTN_ERR_DEVICE.  At most 2 x 256 (compute
 * units) partial blocks of 256 rows x 130 floats.
 */
int attn_fwd_bf16_gqa_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                                     int mask, int64_t *bytes);

/*
 * attn_fwd_bf16_split_plan_masked -- attn_fwd_bf16_gqa_ws's split decision as
 * a pure function for testing: B*H = n_heads heads of Sq x Sk under `mask`
 * on n_cu compute units; out4 as attn_fwd_bf16_split_plan's (under a causal
 * mask the last entry is the heaviest item's tiles per range).  Returns
 * ATTN_ERR_NULL, ATTN_ERR_SIZE or ATTN_ERR_MASK.
 */
int attn_fwd_bf16_split_plan_masked(int64_t n_heads, int64_t Sq, int64_t Sk, int mask,
                                    int64_t n_cu, int64_t *out4);

/*
 * attn_fwd_bf16_partial -- attention of the query rows over one shard of the
 * keys, for key (context) parallelism: the keys of each head are cut into
 * shards that are processed apart (on other devices, or one after another)
 * and combined by attn_fwd_bf16_merge, which rounds once.
 *
 * The pages do not treat this; it follows from the row's softmax being a
 * sum over keys: a shard's rows normalised by the shard's own sum, with the
 * shard's log-sum-exp (attn_fwd_bf16_gqa's lse), are all a merge needs (the
 * FlashAttention family's out + softmax_lse per key block).
 *
 *   q          : [B, Sq, H, 128] (BSHD) or [B, H, Sq, 128] (BHSD) bf16.
 *   k, v       : this shard, [B, Sk, H_kv, 128] or [B, H_kv, Sk, 128]:
 *                global keys key_offset .. key_offset + Sk - 1 of a head
 *                with Sk_total keys.
 *   o_part     : B*H*Sq*128 fp32 at q's element offsets (q's layout), 16-byte
 *                aligned: the shard's rows, sum_j w_j v_j / sum_j w_j over the
 *                shard's visible keys; 0 for a row that sees none of them.
 *   lse_part   : B*H*Sq fp32 laid out [B, H, Sq], 4-byte aligned, required:
 *                ln sum_j exp(q.k_j / sqrt(128)) over the shard's visible
 *                keys; -Inf for a row that sees none of them, NaN where a
 *                logit is NaN or +Inf.
 *   key_offset, Sk_total : the shard's place, 0 <= key_offset,
 *                key_offset + Sk <= Sk_total <= 2^31 - 1.
 *   mask       : attn_mask_t over the global keys: ATTN_MASK_CAUSAL (row i
 *                sees global keys j <= i) or ATTN_MASK_CAUSAL_BOTTOM_RIGHT
 *                (j <= i + Sk_total - Sq).
 *   other arguments : as attn_fwd_bf16_gqa.
 *
 * Status codes as attn_fwd_bf16_gqa (ATTN_ERR_NULL also for lse_part,
 * ATTN_ERR_SIZE for a shard outside [0, Sk_total), ATTN_ERR_ALIGN /
 * ATTN_ERR_ALIAS for o_part and lse_part).  Single pass, deterministic.
 */
int attn_fwd_bf16_partial(const void *q, const void *k, const void *v, float *o_part,
                          float *lse_part, int64_t B, int64_t H, int64_t H_kv, int64_t Sq,
                          int64_t Sk, int64_t key_offset, int64_t Sk_total, int layout,
                          int mask, void *stream);

/*
 * attn_fwd_bf16_merge -- combines n_parts shard results of
 * attn_fwd_bf16_partial into the bf16 output: per row, M = max_s lse_s,
 * w_s = exp(lse_s - M), O = sum_s w_s O_s / sum_s w_s (in shard order, fp32),
 * then one rounding in round_mode; lse (optional) = M + ln sum_s w_s.
 *
 *   o_parts    : n_parts consecutive fp32 arrays of B*H*Sq*128 values (each
 *                at q's element offsets in `layout`), 16-byte aligned.
 *   lse_parts  : n_parts consecutive fp32 [B, H, Sq] arrays, 4-byte aligned.
 *   o          : bf16 output shaped like q, 16-byte aligned.
 *   lse        : NULL, or B*H*Sq fp32 [B, H, Sq]: the row's log-sum-exp over
 *                all shards.
 *   B, H, Sq, layout, round_mode, stream : as attn_fwd_bf16.
 *
 * A row that no shard gives a key (every lse_s -Inf) is NaN with an lse of
 * -Inf; a NaN lse_s makes the row and its lse NaN.  Merging the shards of a
 * cut of the keys gives the whole-key result within the same tolerance of
 * the exact result (not necessarily the same bits: the sums run in another
 * order).  Status codes: ATTN_ERR_NULL, ATTN_ERR_SIZE (n_parts < 1, sizes),
 * ATTN_ERR_LAYOUT, ATTN_ERR_ROUND, ATTN_ERR_ALIGN, ATTN_ERR_ALIAS (o or lse
 * overlapping the parts or each other), ATTN_ERR_DEVICE, ATTN_ERR_HIP.
 */
int attn_fwd_bf16_merge(const float *o_parts, const float *lse_parts, int64_t n_parts,
                        void *o, float *lse, int64_t B, int64_t H, int64_t Sq, int layout,
                        int round_mode, void *stream);

/*
 * attn_fwd_bf16_workspace_size -- bytes of workspace attn_fwd_bf16_ws needs
 * for this shape on the current device (0: it will not split).  Writes
 * *bytes; returns ATTN_ERR_NULL, ATTN_ERR_SIZE or ATTN_ERR_DEVICE like the
 * other calls.  At most 256 (compute units) x 256 rows x 130 floats.
 */
int attn_fwd_bf16_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                                 int64_t *bytes);

/*
 * attn_fwd_bf16_split_plan -- the split decision, as a pure function for
 * testing: n_work items of n_tiles 64-key tiles on n_cu compute units.
 * out4 = {items run whole, items split, ranges per split item, tiles per
 * range}.  Returns ATTN_ERR_NULL or ATTN_ERR_SIZE (any argument < 1).
 */
int attn_fwd_bf16_split_plan(int64_t n_work, int64_t n_tiles, int64_t n_cu,
                             int64_t *out4);

/* Static description of a status code (never NULL). */
const char *attn_fwd_bf16_strerror(int status);

/* ATTN_FWD_ABI_VERSION of the built library. */
int attn_fwd_bf16_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
