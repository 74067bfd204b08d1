/*
 * tria.h - C ABI of the block-sparse, mixed-precision (int8 / int4 / skip) causal
 * attention library for one AMD Instinct MI355X (gfx950).
 *
 * Method.  The TriAttention summary page (rit.work, "TriAttention: sparse
 * mixed-precision attention") describes it in its section on which links can be
 * skipped and which must not be removed: the attention matrix is cut into
 * (query block, key block) tiles, and each tile is skipped, computed at 4 bits or
 * computed at 8 bits according to its distance from the diagonal.  Each head keeps
 * one pair of boundaries (hi, keep); the first key block and the diagonal block are
 * always kept at 8 bits.  The section on calibration adds that one fused prefill
 * kernel groups the kept tiles by precision and reduces them into one normalised
 * result, and that the prepared keys and values then go to a compressed KV cache
 * that generation reads.  The KV layout is grouped-query attention (llmis.ru
 * chapter 3.5, section 4): query head h uses KV head h / (Hq / Hkv).
 *
 * Conventions for every call.
 *  - Device pointers are caller-owned (for example PyTorch tensors).  The library
 *    never allocates or frees device memory and keeps no device state.
 *  - Device calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the legacy default stream).  Host-only calls are synchronous.
 *  - Every argument is validated before anything is enqueued; a non-OK status
 *    means nothing was enqueued.  tria_last_error() returns the message of the
 *    last non-OK status on the calling thread.  No C++ exception crosses the ABI.
 *  - Tensors are dense and contiguous in BHSD order: [batch][head][token][dim].
 *  - Supported shapes: head_dim in {64, 128}; block in {64, 128};
 *    n_q_heads % n_kv_heads == 0; seq_len >= 1; n_kv_heads <= TRIA_MAX_KV_HEADS.
 *  - Thread safety: calls may come from several host threads; the only library
 *    state is the thread-local error message.
 */
#ifndef TRIA_H
#define TRIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tria_status {
  TRIA_OK = 0,
  TRIA_ERR_INVALID_ARG = 1,      /* null pointer, bad shape, hi > keep, corrupt header */
  TRIA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head_dim, block, head count) */
  TRIA_ERR_BUFFER_TOO_SMALL = 3, /* a caller buffer is smaller than required */
  TRIA_ERR_HIP = 4               /* the HIP runtime reported an error at launch */
} tria_status;

#define TRIA_MAX_KV_HEADS 128

/* Problem shape.  seq_len is the prompt length n for prefill, and the number of
 * token rows in the K/V source tensors for the cache packer. */
typedef struct tria_dims {
  int32_t batch;      /* b */
  int32_t n_q_heads;  /* Hq */
  int32_t n_kv_heads; /* Hkv */
  int32_t head_dim;   /* d */
  int32_t block;      /* B, tokens per block on both the query and key side */
  int32_t reserved;   /* must be 0 */
  int64_t seq_len;    /* n */
} tria_dims;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* tria_last_error(void);
/* Library version, (major << 16) | minor. */
int32_t tria_version(void);

/* ------------------------------------------------------------------------- */
/* (1) Policy expander.  Host only.                                           */
/* ------------------------------------------------------------------------- */
/*
 * Tile actions (TriAttention page, section on which links can be skipped: the
 * three actions, the distance rule, the two protected blocks and the per-head
 * boundary pair whose size does not grow with the context).  For query head h
 * with boundaries (hi[h], keep[h]), query block qb and causal key block kb <= qb,
 * with distance delta = qb - kb:
 *     int8  if kb == 0 or delta == 0 or delta <= hi[h]
 *     int4  else if delta <= keep[h]
 *     skip  otherwise.
 * Boundaries are in blocks, inclusive, with 0 <= hi[h] <= keep[h]; values at or
 * above nb - 1 mean "everything" (nb = ceil(seq_len / block)).
 *
 * Schedule blob written to sched_host (little-endian int32 words):
 *   words 0..15  header: [0] TRIA_SCHED_MAGIC, [1] TRIA_SCHED_VERSION, [2] batch,
 *                [3] n_q_heads, [4] n_kv_heads, [5] head_dim, [6] block, [7] nb,
 *                [8] n_units = batch * n_q_heads * nb, [9] 0,
 *                [10] seq_len low 32 bits, [11] seq_len high 32 bits, [12..15] 0.
 *   then n_units records of 8 int32, one work unit = (b, h, qb):
 *                {b, h, qb, lo8, lo4, hi4, sink, ntiles}
 *     int8 range  [lo8, qb], the longest run of int8 blocks ending at qb:
 *                 lo8 = qb - hi[h] if that is >= 2, else 0 (block 0 joins the
 *                 run when it is adjacent to it)
 *     int4 range  [lo4, hi4] = [max(1, qb - keep[h]), qb - hi[h] - 1],
 *                 stored as (0, -1) when empty
 *     sink        1 if block 0 is int8 but lies outside the int8 range (lo8 > 0)
 *     ntiles      (qb - lo8 + 1) + sink + (hi4 - lo4 + 1)
 *   Record order (the dispatch order; tria_prefill accepts the records in any
 *   order): work group i runs on XCD i mod 8.  Each (b, h) is cut into chunks of
 *   32 consecutive query blocks counted down from its last block; a chunk's
 *   records run in consecutive slots of one XCD, so its units, whose key windows
 *   overlap, share that XCD's L2.  Chunks go, most tiles first, to the XCD with the
 *   fewest tiles so far among those holding at most ceil(n_units / 8) records with
 *   it; each XCD runs its chunks most tiles first; record r of XCD x sits at
 *   position 8 r + x while every XCD still has records, the rest follow
 *   round-robin over those that do.
 * Total size: TRIA_SCHED_HEADER_BYTES + TRIA_SCHED_UNIT_BYTES * n_units.
 *
 * n_policy_heads must equal n_q_heads.  If sched_host is NULL or sched_bytes is
 * too small, *sched_bytes_needed (if non-NULL) receives the size and the call
 * returns TRIA_ERR_BUFFER_TOO_SMALL (sched_host == NULL with a non-NULL
 * sched_bytes_needed is the size query and returns TRIA_OK).
 * The caller copies the blob to device memory for tria_prefill.
 */
#define TRIA_SCHED_MAGIC 0x48435354 /* "TSCH" */
#define TRIA_SCHED_VERSION 1
#define TRIA_SCHED_VERSION_VARLEN 2
#define TRIA_SCHED_HEADER_BYTES 64
#define TRIA_SCHED_UNIT_BYTES 32
tria_status tria_build_policy(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                              int32_t n_policy_heads, void* sched_host, size_t sched_bytes,
                              size_t* sched_bytes_needed);

/* ------------------------------------------------------------------------- */
/* (2) Quantiser.  Device, asynchronous.                                      */
/* ------------------------------------------------------------------------- */
/*
 * Per-row symmetric quantisation of Q [b][Hq][n][d] and K [b][Hkv][n][d] (bf16)
 * to 8-bit and 4-bit codes (TriAttention page, section on which links can be
 * skipped: tiles are computed at 8 or 4 bits).  A row is the d values of one
 * token of one head.  With qmax = 127 (int8) or 7 (int4), in IEEE fp32:
 *     amax  = max_i |x_i|
 *     scale = amax / qmax                     (correctly rounded division)
 *     r     = qmax / amax                     (correctly rounded division)
 *     code  = clamp(rint(x_i * r), -qmax, qmax)   (fp32 product, ties to even)
 * A row with amax == 0 has scale 0 and all codes 0.  Inputs must be finite.
 * Outputs: q8 int8 [b][Hq][n][d]; q4 uint8 [b][Hq][n][d/2] with byte j =
 * (c[2j] & 0xF) | (c[2j+1] << 4) (two's-complement nibbles, low nibble first);
 * q8s, q4s fp32 [b][Hq][n] (the scales).  k8, k4, k8s, k4s likewise with Hkv.
 * Q is quantised unscaled; sm_scale is applied to the scores in tria_prefill.
 */
tria_status tria_quantize_qk(const tria_dims* dims, const void* q_bf16, const void* k_bf16,
                             int8_t* q8, uint8_t* q4, float* q8s, float* q4s,
                             int8_t* k8, uint8_t* k4, float* k8s, float* k4s, void* stream);

/* ------------------------------------------------------------------------- */
/* (3) Fused prefill.  Device, asynchronous.                                  */
/* ------------------------------------------------------------------------- */
/*
 * Causal block-sparse attention over the schedule (TriAttention page, section on
 * calibration: one fused kernel groups kept blocks by precision and produces one
 * normalised result).  For query row i of head h (KV head g, query block qb):
 *   J_i   = { j <= i : tile (qb, j / block) is not skipped }
 *   S_ij  = dot(Qc_i, Kc_j) in exact integer arithmetic, with the codes of the
 *           tile's precision (both Q and K use 4-bit codes in an int4 tile)
 *   t_ij  = S_ij * sq_i * sk_j * sm_scale * log2(e)   (sq, sk: that precision's scales)
 *   M_i   = an integer >= max_j t_ij
 *   P_ij  = bf16_rne(fp32(2^(t_ij - M_i)))            (the weights fed to P.V)
 *   out_i = sum_j P_ij * V_j / sum_j P_ij             (fp32 out, V in bf16)
 * Because M_i is an integer, the result does not depend on which integer the
 * kernel's running maximum settled on (power-of-two rescaling commutes with the
 * bf16 rounding); results agree with a fixed-M evaluation up to fp32 summation
 * order.  Skipped tiles are never read.
 * Inputs: the device copy of tria_build_policy's blob, the outputs of
 * tria_quantize_qk, and V bf16 [b][Hkv][n][d].  out fp32 [b][Hq][n][d].
 * lse (may be NULL) fp32 [b][Hq][n] receives M_i + log2(sum_j P_ij), the base-2
 * log of the softmax denominator in units of t.
 * sched_bytes must be exactly the size the dims imply (TRIA_ERR_BUFFER_TOO_SMALL
 * below it, TRIA_ERR_INVALID_ARG above it).  The device checks the schedule: a
 * header that does not describe the call (magic, version, batch, heads, head_dim,
 * block, block count, unit count, seq_len) makes every output row and LSE entry NaN;
 * a malformed unit record (one the builder could not have written: fields out of
 * range, an int4 range that does not end at lo8 - 1, a tile count that disagrees)
 * computes nothing and makes the rows it names NaN (a record
 * that names no rows writes nothing, so the rows of the unit it replaced keep what
 * `out` held).  The kernels always exit normally.
 * Errors: TRIA_ERR_UNSUPPORTED when (seq_len + 4 * block) * 2 * head_dim >= 2^31
 * (byte offsets within a head's rows are 32-bit inside the kernel: seq_len below
 * 8.4 M tokens at head_dim 128).
 */
tria_status tria_prefill(const tria_dims* dims, const void* sched_dev, size_t sched_bytes,
                         const int8_t* q8, const uint8_t* q4, const float* q8s, const float* q4s,
                         const int8_t* k8, const uint8_t* k4, const float* k8s, const float* k4s,
                         const void* v_bf16, float sm_scale, float* out, float* lse, void* stream);

/*
 * The same prefill (TriAttention page, section on calibration: one fused kernel per
 * layer) with Q given as bf16 [b][Hq][n][d] (device): every work unit quantises its
 * own query block in the kernel (section on which links can be skipped: 8- and 4-bit
 * tiles), with the quantiser's formula above
 * (the same codes and scales as tria_quantize_qk), so no Q codes pass through memory;
 * K comes from tria_quantize_k (or tria_quantize_qk).  out and lse are bit for bit
 * those of tria_quantize_qk + tria_prefill.  Arguments, validation and errors as
 * tria_prefill.  Device, asynchronous.
 */
tria_status tria_prefill_bf16q(const tria_dims* dims, const void* sched_dev, size_t sched_bytes,
                               const void* q_bf16, const int8_t* k8, const uint8_t* k4, const float* k8s,
                               const float* k4s, const void* v_bf16, float sm_scale, float* out, float* lse,
                               void* stream);

/*
 * The quantiser's K half alone (TriAttention page, section on which links can be
 * skipped): k8, k4, k8s, k4s exactly as tria_quantize_qk writes them (for
 * tria_prefill_bf16q, which quantises Q itself).  Errors as tria_quantize_qk.
 * Device, asynchronous.
 */
tria_status tria_quantize_k(const tria_dims* dims, const void* k_bf16, int8_t* k8, uint8_t* k4, float* k8s,
                            float* k4s, void* stream);

/*
 * Variable-length batches.  n_seqs causal sequences of different lengths packed
 * along the rows of one batch element: dims->batch == 1, dims->seq_len = the total
 * T, sequence s = rows [cu_seqlens[s], cu_seqlens[s + 1]) (host int64[n_seqs + 1],
 * cu_seqlens[0] = 0, strictly increasing, cu_seqlens[n_seqs] = T).  Q, K, V and the
 * quantiser's outputs use the [1][H][T][d] layout (tria_quantize_qk with the same
 * dims quantises them: rows are rows).  Each sequence is attended on its own, its
 * blocks counted from its first row (block 0 and its diagonal protected, as above):
 * row i of sequence s gives exactly what tria_prefill gives for that sequence
 * alone.
 * tria_build_policy_varlen: as tria_build_policy, with header word [1] =
 *   TRIA_SCHED_VERSION_VARLEN, [2] = n_seqs, [7] = the largest block count; units
 *   {s, h, qb, ...} for every sequence s and its ceil(len_s / block) query blocks
 *   (same dispatch order, a lane being one (s, h)); then n_seqs
 *   records {int32 start, int32 length}.  Size TRIA_SCHED_HEADER_BYTES +
 *   TRIA_SCHED_UNIT_BYTES * n_units + 8 * n_seqs.
 * tria_prefill_varlen: as tria_prefill over that schedule; out fp32 [1][Hq][T][d],
 *   lse [1][Hq][T].  cu_seqlens must be the one the schedule was built from.
 * Errors: TRIA_ERR_INVALID_ARG for dims->batch != 1, n_seqs < 1 or a cu_seqlens
 * that does not start at 0, increase strictly and end at seq_len; otherwise as
 * tria_build_policy and tria_prefill.
 */
tria_status tria_build_policy_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                     int32_t n_policy_heads, int32_t n_seqs, const int64_t* cu_seqlens,
                                     void* sched_host, size_t sched_bytes, size_t* sched_bytes_needed);
tria_status tria_prefill_varlen(const tria_dims* dims, int32_t n_seqs, const int64_t* cu_seqlens,
                                const void* sched_dev, size_t sched_bytes, const int8_t* q8,
                                const uint8_t* q4, const float* q8s, const float* q4s,
                                const int8_t* k8, const uint8_t* k4, const float* k8s,
                                const float* k4s, const void* v_bf16, float sm_scale, float* out,
                                float* lse, void* stream);

/* ------------------------------------------------------------------------- */
/* (4) Compressed KV cache.                                                   */
/* ------------------------------------------------------------------------- */
/*
 * The cache holds, for one query position t = ctx_len - 1 (current block
 * c = t / block), only the key blocks the policy keeps, each at its precision
 * (TriAttention page, section on calibration: prepared keys and values go to a
 * compressed KV cache so that generation reads less; section on infrastructure
 * plans: a special cache layout).  The policy is per KV head: pass
 * n_policy_heads == n_kv_heads, or n_policy_heads == n_q_heads to merge each
 * group by the maximum of hi and of keep (the union of the kept sets).
 * For KV head g with (hi, keep):
 *     int8 blocks: {0} union {kb <= c : c - kb <= hi}       (block c always)
 *     int4 blocks: {kb >= 1 : hi < c - kb <= keep}
 * Each K and V row of a stored block is quantised with the tria_quantize_qk
 * contract at the block's precision (V too, unlike prefill).
 *
 * Byte layout (little-endian):
 *   [0, 64)  header: int32 magic TRIA_CACHE_MAGIC, int32 version, int32 batch,
 *            int32 n_kv_heads, int32 head_dim, int32 block, int32 nb (= c + 1),
 *            int32 cur_block (= c), int64 ctx_len, int64 total_bytes,
 *            int64 dir_offset (= 64), int64 data_offset.
 *   [64, 64 + 64*batch*n_kv_heads)  directory, one 64-byte entry per (b, g),
 *            b-major: int64 offset (from the blob start to the pair's first
 *            record), int32 n8, int32 n4, int32 hi, int32 keep, int32 lo8,
 *            int32 sink, int32 lo4, int32 hi4, int32 zero[6].  The stored int8
 *            blocks are [block 0 if sink] then lo8..c; the int4 blocks lo4..hi4
 *            ((0, -1) when none); lo8, sink, lo4, hi4 follow the schedule's rule
 *            for query block c.  hi, keep are the (merged) KV-head boundaries.
 *   data_offset = round_up(64 + 64*batch*n_kv_heads, 256); the pairs' records
 *            follow in (b, g) order, each pair's n8 int8 records (ascending
 *            block) then its n4 int4 records (ascending block).
 *   A record (int8: 2*B*d + 8*B bytes; int4: B*d + 8*B bytes) is B/32 chunks
 *   of 32 tokens (chunk c = tokens 32c..32c+31 of the block): a K part and a V
 *   part that are sequences of 16-byte units, then K scales fp32 [32] and V
 *   scales fp32 [32].  Units are listed in nesting order; q in 0..3, r in 0..15:
 *     int8 K (32*d bytes): unit (s, ks, q, r), s in 0..1, ks in 0..d/64-1 =
 *       dims 64*ks + 16*q .. +15 of token 32c + 16s + r;
 *     int4 K (16*d bytes): unit (s, q, r) = for ks = 0..d/64-1 the same 16 dims
 *       packed into 8 bytes (low nibble = even dim);
 *     int8 V (32*d bytes): unit (m, q, r), m in 0..d/32-1 = for dt = 2m, 2m+1:
 *       8 bytes, byte p = dim 16*dt + r of token 32c + 16*(p/4) + 4*q + (p%4);
 *     int4 V (16*d bytes): unit (m, q, r), m in 0..d/64-1 = for dt = 4m..4m+3:
 *       those 8 positions packed into 4 bytes (low nibble = even p).
 *   (This is the order in which one decode step of 32 tokens consumes them: the
 *   step reads one contiguous chunk, each 1 KB load with lane 16q + r taking unit
 *   (.., q, r).)
 *   Tokens at or beyond ctx_len in the current block have zero codes and scales.
 * tria_kv_cache_bytes gives the exact total; ctx_len must satisfy
 * 1 <= ctx_len <= dims->seq_len (the K/V tensors hold seq_len rows).
 */
#define TRIA_CACHE_MAGIC 0x43564B54 /* "TKVC" */
#define TRIA_CACHE_VERSION 2
#define TRIA_CACHE_HEADER_BYTES 64
#define TRIA_CACHE_DIR_ENTRY_BYTES 64
tria_status tria_kv_cache_bytes(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                int32_t n_policy_heads, int64_t ctx_len, size_t* bytes);
/* Packs K, V bf16 [b][Hkv][seq_len][d] into `cache` (cache_bytes >= the size above). */
tria_status tria_pack_kv_cache(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                               int32_t n_policy_heads, int64_t ctx_len, const void* k_bf16,
                               const void* v_bf16, void* cache, size_t cache_bytes, void* stream);
/* Variable-length batches: sequence b holds ctx_lens[b] tokens (host int64[batch],
 * 1 <= ctx_lens[b] <= seq_len; batch <= 256), its query at t_b = ctx_lens[b] - 1 and
 * current block c_b = t_b / block; its KV heads store the blocks of the rule above
 * for c_b.  The layout is the one above with version 3: header word [6] = c + 1 and
 * [7] = -1 (c of the longest sequence; the current block varies), int64 ctx_len
 * (bytes 32..39) = 0, and every directory entry holds its sequence's ctx_len as int64
 * in words 10-11.  tria_kv_cache_bytes_varlen gives the exact size; the pack is
 * device, asynchronous.  Sequence b's records are byte for byte those
 * tria_pack_kv_cache writes for a batch of that sequence alone at ctx_lens[b].
 * Errors: TRIA_ERR_UNSUPPORTED above 256 sequences; TRIA_ERR_INVALID_ARG for a
 * length outside [1, seq_len]. */
tria_status tria_kv_cache_bytes_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                       int32_t n_policy_heads, const int64_t* ctx_lens, size_t* bytes);
tria_status tria_pack_kv_cache_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                      int32_t n_policy_heads, const int64_t* ctx_lens,
                                      const void* k_bf16, const void* v_bf16, void* cache,
                                      size_t cache_bytes, void* stream);
/* Incremental maintenance (one more token): given cache_in, the cache packed for
 * ctx_len - 1 from the same K, V and policy, writes to cache_out exactly the cache
 * tria_pack_kv_cache would write for ctx_len (byte for byte).  A block's record
 * depends only on its rows and its precision, so every record of a block before
 * the new current block that cache_in holds at the same precision is reused; the
 * current block's record and, when t = ctx_len - 1 starts a new block, the record
 * of the block leaving the int8 window (now int4) are quantised from K, V.  Blocks
 * leaving the int4 window are dropped.  The rows read from K, V must be those
 * cache_in was packed from.
 *   Within a block (ctx_len - 1 not a multiple of the block size) cache_out may be
 *   cache_in (in place: only the current block's record and the header's ctx_len
 *   change; one work group per (batch, KV head)).  When t starts a new block the
 *   records move: cache_out must then be another buffer, not overlapping cache_in,
 *   of at least tria_kv_cache_bytes(ctx_len) bytes.
 * Errors: TRIA_ERR_INVALID_ARG for ctx_len outside [2, seq_len], an in-place call
 * at a block start or partially overlapping buffers; TRIA_ERR_BUFFER_TOO_SMALL
 * when cache_in is smaller than the cache for ctx_len - 1 or cache_out than the
 * one for ctx_len.  Device, asynchronous on `stream`; cache_in's contents are not
 * validated (a cache that was not packed as stated gives a wrong result, never an
 * access outside the two buffers). */
tria_status tria_update_kv_cache(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                 int32_t n_policy_heads, int64_t ctx_len, const void* k_bf16,
                                 const void* v_bf16, const void* cache_in, size_t cache_in_bytes,
                                 void* cache_out, size_t cache_out_bytes, void* stream);
/* Synchronous host-side validation of a cache's header and directory against
 * dims and ctx_len (copies them from device memory; for debugging and tests).
 * Returns TRIA_ERR_INVALID_ARG on any mismatch or corruption. */
tria_status tria_check_cache(const tria_dims* dims, const void* cache, size_t cache_bytes,
                             int64_t ctx_len);

/* ------------------------------------------------------------------------- */
/* (5) Decode.  Device, asynchronous.                                         */
/* ------------------------------------------------------------------------- */
/*
 * One query token per sequence at position t = ctx_len - 1 attends over the
 * stored blocks of the packed cache (reading only them: decode is bound by memory
 * traffic, llmis.ru chapter 3.5 section 2, so reading fewer bytes is the win).
 * For query head h (KV head g) and each stored token j <= t of block precision a:
 *     s_j = dot(qc^a, kc_j^a) * sq^a * sk_j^a * sm_scale
 *     p_j = exp(s_j - max_j s_j)
 *     out = sum_j p_j * sv_j^a * vc_j^a / sum_j p_j          (fp32)
 * where q's row is quantised with the tria_quantize_qk contract at each
 * precision.  q bf16 [b][Hq][d]; out fp32 [b][Hq][d].  The kernel reads shapes
 * and offsets from the cache header (written by tria_pack_kv_cache for the same
 * dims and ctx_len); a header or directory that does not match (shape, record
 * counts, contiguous record offsets) writes NaN to `out` and reads no record.
 * workspace: device memory of at least tria_decode_workspace_bytes bytes for the
 * split-KV partial results; its contents need no initialisation.  Calls that
 * share a workspace must be ordered on one stream.
 * Errors: TRIA_ERR_UNSUPPORTED for more than 32 query heads per KV head, for
 * batch * n_kv_heads above 4096, or when batch * n_kv_heads * ceil(ctx_len /
 * block) * block / 16 reaches 2^31.
 */
/* tria_decode_varlen: decode over a version-3 (variable-length) cache: each
 * sequence's query attends over its own ctx_len tokens (read from the directory),
 * exactly as tria_decode does for that sequence alone.  The workspace is sized by
 * tria_decode_workspace_bytes(dims, dims->seq_len).  A header or directory that does
 * not validate (version 3, each entry consistent with its own ctx_len, contiguous
 * offsets) writes NaN to `out` and reads no record. */
tria_status tria_decode_workspace_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes);
tria_status tria_decode(const tria_dims* dims, const void* cache, size_t cache_bytes,
                        int64_t ctx_len, const void* q_bf16, float sm_scale, float* out,
                        void* workspace, size_t ws_bytes, void* stream);
/* tria_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * results as tria_decode, with the workspace replaced by a library-owned device array
 * of 64 MiB per GPU (held from the library's first use on that GPU until the process
 * ends; it needs no initialisation).  Nothing is allocated by the call.  Every call
 * tria_decode accepts fits, except with 32 query heads per KV head and head_dim 128
 * above 1922 (batch, KV head) pairs: a call whose tria_decode_workspace_bytes exceeds
 * 64 MiB returns TRIA_ERR_UNSUPPORTED before any HIP call; a stream of another device
 * than the current one, TRIA_ERR_INVALID_ARG.  All calls on one GPU share its array, so calls that overlap
 * on one GPU (different streams, or host threads) race: serialise them, e.g. on one
 * stream.  Other arguments and errors as tria_decode. */
tria_status tria_decode_noalloc(const tria_dims* dims, const void* cache, size_t cache_bytes,
                                int64_t ctx_len, const void* q_bf16, float sm_scale, float* out,
                                void* stream);
tria_status tria_decode_varlen(const tria_dims* dims, const void* cache, size_t cache_bytes,
                               const void* q_bf16, float sm_scale, float* out, void* workspace,
                               size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Paged compressed cache (block table).                                      */
/* ------------------------------------------------------------------------- */
/*
 * ZimaSpace page on attention memory (the section on the KV cache as per-token state
 * kept for the whole conversation, and its closing list of memory levers): paged
 * allocation of the KV cache cuts fragmentation when request lengths are not known in
 * advance, beside lower cache precision; llmis.ru chapter 3.5 (its closing section on
 * what grouped heads compose with): paging changes where the cache lives, not its
 * size, so it composes with cache quantisation.  Here the records of the compressed cache (the version-2 record format,
 * int8 or int4) live in a caller-owned pool of pages of tria_paged_page_bytes each
 * (one int8 record; an int4 record uses the first half of its page), and a table maps
 * every stored record to its page.  Going from ctx_len - 1 to ctx_len then moves no
 * record: records that stay keep their pages, new ones (the current block, a block
 * demoted from int8 to int4) take pages from the caller's free list, dropped ones
 * release theirs.
 *
 * Table (version 4): 64-byte header {int32 magic "TKVP", 4, batch, n_kv_heads,
 *   head_dim, block, rmax = c + 1, c (current block); int64 ctx_len, page bytes,
 *   n_pages (pool size in pages), 0}, one 64-byte entry per (batch, KV head) laid out
 *   as in version 2 with a zero offset {0, 0, n8, n4, hi, keep, lo8, sink, lo4, hi4,
 *   0...}, then per pair rmax int32 page ids in record order (int8 records, then int4;
 *   -1 past the pair's records).
 *
 * tria_paged_page_bytes, tria_paged_table_bytes: sizes.
 * tria_build_paged_table (host, synchronous): the table for ctx_len (host buffer).
 *   old_table (host, or NULL for a fresh cache): the table of the same cache at an
 *   earlier ctx_len with the same dims, policy and n_pages.  A record whose (block,
 *   precision) the old table stores keeps its page; every other record takes the next
 *   page of free_pages (in pair order, then record order); *n_used = pages taken from
 *   the front of free_pages; the old records not kept release their pages into
 *   released (*n_released, in pair and record order).  Errors: BUFFER_TOO_SMALL when
 *   n_free or released_capacity is short (*n_used, *n_released hold the needs);
 *   INVALID_ARG when the old table does not match or a page is outside [0, n_pages),
 *   repeated, or (for a free page) still held by the old table.  Nothing is written
 *   on error.
 * tria_pack_kv_cache_paged: writes into the pool (device) the records of the table
 *   (device copy of a tria_build_paged_table result for this ctx_len and policy) from
 *   the bf16 K, V rows, quantised as tria_pack_kv_cache does.  old_table (device, or
 *   NULL): the table the pool currently holds (any earlier ctx_len); a record before
 *   the current block that it maps to the same page and (block, precision), and that
 *   was complete there (not its partly filled current block), is left as it is, so a
 *   step within a block writes only the new rows and a block start writes the new
 *   records.  A table whose header does not match the call, or a page outside the pool,
 *   writes nothing.
 * tria_decode_paged: tria_decode over a paged cache: the split kernel reads the table's
 *   directory entries (checked as tria_decode checks its directory) and each record's
 *   page from the table (the workspace of tria_decode_skip_workspace_bytes).  A table
 *   whose header or entries do not validate writes NaN to `out` and reads no record;
 *   a page outside the pool makes the query heads of its (batch, KV head) NaN.
 *   Results equal tria_decode on the contiguous cache with the same content, bit for
 *   bit. */
tria_status tria_paged_page_bytes(const tria_dims* dims, size_t* bytes);
tria_status tria_paged_table_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes);
tria_status tria_build_paged_table(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                   int32_t n_policy_heads, int64_t ctx_len, int64_t n_pages,
                                   const void* old_table, size_t old_table_bytes, const int32_t* free_pages,
                                   int32_t n_free, void* table, size_t table_bytes, int32_t* n_used,
                                   int32_t* released, int32_t released_capacity, int32_t* n_released);
tria_status tria_pack_kv_cache_paged(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                     int32_t n_policy_heads, int64_t ctx_len, const void* k_bf16,
                                     const void* v_bf16, const void* table, size_t table_bytes,
                                     const void* old_table, size_t old_table_bytes, void* pool,
                                     size_t pool_bytes, void* stream);
tria_status tria_decode_paged(const tria_dims* dims, const void* table, size_t table_bytes, const void* pool,
                              size_t pool_bytes, int64_t ctx_len, const void* q_bf16, float sm_scale, float* out,
                              void* workspace, size_t ws_bytes, void* stream);

/* Variable-length paged cache (continuous batching): each batch element's sequence at its
 * own ctx_lens[b] (host array, 1 <= ctx_lens[b] <= seq_len, batch <= 256).  The table
 * (same version 4) has header word 7 = -1 and ctx_len 0, rmax = c + 1 of the longest
 * sequence page slots per pair, and each entry's words 10-11 = its sequence's ctx_len
 * (size: tria_paged_table_bytes of the longest ctx_len).  The builder keeps pages per
 * sequence as above.  seq_ids (host int64[batch], may be NULL for all 0) names the
 * sequence each slot holds, kept in its entries' words 12-13: a slot whose id differs
 * from the old table's, or whose sequence is shorter than there, holds a new sequence
 * (its old pages are all released, none reused), so a finished request's slot can take
 * a new prompt of any length.  Pack: K, V [b][Hkv][seq_len][d],
 * each sequence's rows at its own b; with the old table, each sequence writes only what
 * changed for it.  Decode: each sequence's query attends over its own ctx_len tokens, as
 * tria_decode does for that sequence alone (workspace: tria_decode_skip_workspace_bytes
 * for seq_len). */
/* Dynamic block skipping over a (fixed-length) paged cache: the statistics index and
 * tria_decode_skip with records read through the table (index layout, thresholds,
 * keep rule and workspace as for the contiguous cache; list entries hold pages).
 * Results equal tria_decode_skip on the contiguous cache with the same content, bit
 * for bit.  A page outside the pool leaves its index slot unwritten and, in decode,
 * makes the query heads of its pair NaN. */
/* Dynamic block skipping over a variable-length (version-3) contiguous cache: each
 * pair's statistics and plan follow its own ctx_len (read from the directory); the
 * index (header word 6 = -1) and the workspace are sized for dims->seq_len
 * (tria_block_summaries_bytes and tria_decode_skip_workspace_bytes of seq_len).
 * Results per sequence equal tria_decode_skip of that sequence alone. */
tria_status tria_build_block_summaries_varlen(const tria_dims* dims, const void* cache, size_t cache_bytes,
                                              void* summaries, size_t summaries_bytes, void* stream);
tria_status tria_decode_skip_varlen(const tria_dims* dims, const void* cache, size_t cache_bytes,
                                    const void* summaries, size_t summaries_bytes, const void* q_bf16,
                                    const float* thresholds, float sm_scale, float* out, void* workspace,
                                    size_t ws_bytes, void* stream);

/* The same over a variable-length paged cache (continuous batching): index and
 * workspace sized for dims->seq_len; results per sequence equal tria_decode_skip_varlen
 * on the contiguous cache with the same content, bit for bit. */
tria_status tria_build_block_summaries_paged_varlen(const tria_dims* dims, const void* table, size_t table_bytes,
                                                    const void* pool, size_t pool_bytes, void* summaries,
                                                    size_t summaries_bytes, void* stream);
tria_status tria_decode_skip_paged_varlen(const tria_dims* dims, const void* table, size_t table_bytes,
                                          const void* pool, size_t pool_bytes, const void* summaries,
                                          size_t summaries_bytes, const void* q_bf16, const float* thresholds,
                                          float sm_scale, float* out, void* workspace, size_t ws_bytes,
                                          void* stream);

tria_status tria_build_block_summaries_paged(const tria_dims* dims, const void* table, size_t table_bytes,
                                             const void* pool, size_t pool_bytes, int64_t ctx_len, void* summaries,
                                             size_t summaries_bytes, void* stream);
tria_status tria_decode_skip_paged(const tria_dims* dims, const void* table, size_t table_bytes, const void* pool,
                                   size_t pool_bytes, int64_t ctx_len, const void* summaries, size_t summaries_bytes,
                                   const void* q_bf16, const float* thresholds, float sm_scale, float* out,
                                   void* workspace, size_t ws_bytes, void* stream);

tria_status tria_build_paged_table_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                          int32_t n_policy_heads, const int64_t* ctx_lens, const int64_t* seq_ids,
                                          int64_t n_pages, const void* old_table, size_t old_table_bytes,
                                          const int32_t* free_pages, int32_t n_free, void* table, size_t table_bytes,
                                          int32_t* n_used, int32_t* released, int32_t released_capacity,
                                          int32_t* n_released);
tria_status tria_pack_kv_cache_paged_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                            int32_t n_policy_heads, const int64_t* ctx_lens, const void* k_bf16,
                                            const void* v_bf16, const void* table, size_t table_bytes,
                                            const void* old_table, size_t old_table_bytes, void* pool,
                                            size_t pool_bytes, void* stream);
tria_status tria_decode_paged_varlen(const tria_dims* dims, const void* table, size_t table_bytes, const void* pool,
                                     size_t pool_bytes, const void* q_bf16, float sm_scale, float* out,
                                     void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Dynamic block skipping in decode (device, asynchronous on `stream`).       */
/* ------------------------------------------------------------------------- */
/*
 * ETA page (rit.work, section on how the model decides which part of the context to
 * read): before a block is read, a few statistics of its keys (mean key, spread of
 * each coordinate, largest norm) bound its scores, and a block whose bound is below
 * the head's threshold is not read; the whole cache stays stored and the statistics
 * are a small extra index.  The learned predictor of the thresholds is not part of
 * this library: thresholds are an input.
 *
 * Statistics of a stored record (its K codes, all rows): per-coordinate minimum and
 * maximum code (lo, hi: the mean and spread as a box), the largest row scale smax,
 * and the largest (scale * scale) * |codes|^2 over rows, nmax (double).  For query
 * head h (codes qc and scale sq of q at the record's precision, the decode's
 * quantiser) and threshold th (fp32, logit units: sm_scale * q.k), with
 * t = sm_scale * sq in double:
 *   box  = (t * smax) * max(sum_x max(qc_x lo_x, qc_x hi_x), 0)   (>= every score)
 *   norm = ((t * t) * |qc|^2) * nmax                               (>= every score^2)
 * the record is skipped for h iff th > 0 and (box < th or norm < th * th), computed
 * in IEEE double in this order.  The first key block and the current block are never
 * skipped.  Each query head attends over the records it keeps; a record no head of
 * its KV head keeps is not read.
 *
 * tria_block_summaries_bytes / tria_build_block_summaries: the index of a version-2
 *   cache for ctx_len: a 64-byte header {int32 magic "TBSM", 2, pairs, slots per pair
 *   (rmax = (ctx_len - 1) / block + 1), head_dim, block, current block, 0; int64 the
 *   cache's total_bytes at byte 32}, then per (pair, record slot) 2 * head_dim + 16
 *   bytes {int8 lo[d], int8 hi[d], fp32 smax, int32 stamp, fp64 nmax}, stamp = the
 *   pair's current block + 1 at build time; slots past a pair's records are zero.  One
 *   work group per slot reads the record's K codes once.  The index stays valid while
 *   the cache keeps the same current block and total size (tria_update_kv_cache within
 *   a block changes only the current record, whose statistics are not used); rebuild
 *   it when a block starts.  The decode checks every stored record's stamp against its
 *   pair's current block, so an index left from another current block (a
 *   variable-length sequence that moved on, or restarted in another block) does not
 *   validate; a sequence restarted inside the same current block cannot be told
 *   apart from its predecessor by the index, so its caller rebuilds the index.  A
 *   cache that does not validate leaves the index without its header (later calls
 *   then reject it).
 * tria_skip_masks: the keep bits of every stored record: masks = uint32 [pairs][rmax]
 *   (record order of the cache: int8 records, then int4), bit i set = query head
 *   g * G + i keeps the record; slots past a pair's records are not written.
 *   q_bf16 [batch][n_q_heads][head_dim], thresholds fp32 [batch][n_q_heads] (device).
 * tria_decode_skip: tria_decode reading only the records some head keeps; per head,
 *   the attention over its kept records.  Three kernels: the keep bits (one lane per
 *   (record, head)), a per-pair compaction of the kept records into the workspace
 *   (with the directory checks of tria_decode), then the split-KV decode over the
 *   kept records' bytes and the merge.  The workspace (tria_decode_skip_workspace_
 *   bytes) holds the decode's partials and the plan.  A cache, or an index, that does
 *   not validate writes NaN to `out` and reads no record.
 * Limits: as tria_decode (G <= 32, batch * n_kv_heads <= 4096); version-2 caches. */
tria_status tria_block_summaries_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes);
tria_status tria_build_block_summaries(const tria_dims* dims, const void* cache, size_t cache_bytes,
                                       int64_t ctx_len, void* summaries, size_t summaries_bytes,
                                       void* stream);
tria_status tria_skip_masks(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                            const void* summaries, size_t summaries_bytes, const void* q_bf16,
                            const float* thresholds, float sm_scale, uint32_t* masks,
                            size_t masks_bytes, void* stream);
tria_status tria_decode_skip_workspace_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes);
tria_status tria_decode_skip(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                             const void* summaries, size_t summaries_bytes, const void* q_bf16,
                             const float* thresholds, float sm_scale, float* out, void* workspace,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Calibration: cost model and allocator.  Host, synchronous.                 */
/* ------------------------------------------------------------------------- */
/*
 * TriAttention summary page (rit.work), section on how calibration distributes
 * compute between heads: each head's candidate boundary pairs get a compute cost
 * that counts whole processed blocks (the QK product, the normalisation of the
 * weights and the value aggregation), and one global allocator grants more context
 * or more precision where the added work lowers the error most.  The error of a
 * variant (measured after the output projection on a model) is an input here.
 *
 * tria_policy_cost: cost of one head's (hi, keep) over all query blocks of
 *   dims->seq_len: (cost_int8 * T8 + cost_int4 * T4) * block^2, where T8 and T4
 *   count the whole int8 and int4 tiles the tile rule keeps (the diagonal and a
 *   ragged last block count as whole blocks).  cost_int8, cost_int4: the cost of one
 *   query-key pair at each precision (finite, > 0; equal on gfx950, which has no
 *   int4 MFMA, when the cost is prefill time).
 * tria_allocate_policy: err = double[n_heads][max_bound + 1][max_bound + 1], err[h][hi]
 *   [keep] the error of head h at (hi, keep) (entries with hi > keep are unused; used
 *   entries finite).  Greedy: every head starts at (0, 0); a step applies the one move
 *   with the largest error reduction per unit of added cost among those that keep the
 *   summed cost <= budget, where a head's moves are keep + 1 (one more block kept, at
 *   int4) and hi + 1 (one more block at int8; keep raised with it when equal), both
 *   bounded by max_bound; a reduction at no added cost ranks first, ties go to the
 *   lower head index, then to the keep move; moves that reduce no error are never
 *   taken; it stops when no move fits.  Writes hi[n_heads], keep[n_heads] and (if
 *   non-NULL) the summed cost and error.
 * Errors: TRIA_ERR_INVALID_ARG for invalid dims, 0 <= hi <= keep violated, non-positive
 * or non-finite costs, a non-finite budget or error entry, max_bound outside
 * [0, 65535], or a budget below n_heads times the cost of (0, 0).
 */
tria_status tria_policy_cost(const tria_dims* dims, int32_t hi, int32_t keep, double cost_int8,
                             double cost_int4, double* cost);
tria_status tria_allocate_policy(const tria_dims* dims, int32_t n_heads, int32_t max_bound,
                                 const double* err, double cost_int8, double cost_int4,
                                 double budget, int32_t* hi, int32_t* keep, double* total_cost,
                                 double* total_err);

/* ---- Measured ceilings (measurement helpers, not part of the method) ---------
 * Loops that bound what the part sustains for the instructions and the access
 * pattern the kernels above use, so roofline fractions can be read against
 * measured ceilings as well as against published peaks.  Each call validates its
 * arguments, stores the work of one launch in *work (host) and enqueues the loop on
 * `stream`; the caller times it with events on that stream.
 * tria_peak_mfma: kind 0 = v_mfma_i32_16x16x64_i8 (*work in int8 ops), kind 1 =
 *   v_mfma_f32_16x16x32_bf16 (*work in flops); 512 work groups of four wavefronts,
 *   each wavefront issuing `iters` rounds of eight independent MFMAs; no memory
 *   traffic.
 * tria_peak_read: reads `bytes` of device memory at src once (TRIA_PEAK_READ_WAVES
 *   wavefronts, each one contiguous range, 1 KB non-temporal loads, eight in
 *   flight); bytes must be a positive multiple of TRIA_PEAK_READ_ALIGN; *work = bytes.
 * sink: device int32[TRIA_PEAK_SINK_INTS], written by the loops (so that their
 *   results are used); its contents are meaningless.
 * Errors: TRIA_ERR_INVALID_ARG for a null pointer, kind not 0 or 1, iters < 1 or a
 * size that is not a positive multiple of TRIA_PEAK_READ_ALIGN;
 * TRIA_ERR_UNSUPPORTED when bytes / TRIA_PEAK_READ_WAVES exceeds 2^31 - 1.
 */
#define TRIA_PEAK_READ_WAVES 8192
#define TRIA_PEAK_READ_ALIGN (8192LL * 8 * 1024)
#define TRIA_PEAK_SINK_INTS 8192
tria_status tria_peak_mfma(int32_t kind, int32_t iters, int32_t* sink, double* work, void* stream);
tria_status tria_peak_read(const void* src, int64_t bytes, int32_t* sink, double* work, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TRIA_H */
