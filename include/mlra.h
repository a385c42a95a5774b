/*
 * mlra.h - C ABI of libmlra.so: single-token decode attention over a compressed
 * latent KV cache, in its Multi-Head Low-Rank Attention form (MLRA-4; also
 * MLRA-2) and in the absorbed Multi-Head Latent Attention form (MLA), for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (page "Multi-Head Low-Rank Attention", ai.info summary of
 * arXiv 2603.02188; "Key Contributions" #2 and #3, "Main Findings" bullet 4,
 * "Methodology in Plain English" paragraphs 1-2): decoding is absorbed-form,
 * MQA-style attention of h query heads over NB latent heads per cached token.
 * For sequence b with L = seqlens[b] cached tokens and query head i:
 *
 *   u_t      = <q_rope[b,i,:], rope[t,:]>                    (shared by every latent head)
 *   s_{j,t}  = sm_scale * (<q_nope[b,i,j,:], latent[t,j,:]> + u_t)
 *   obar_j   = sum_t softmax_t(s_j) * latent[t,j,:]           (one softmax per latent head j)
 *   out[b,i] = out_scale * sum_j obar_j @ W_UV[j,i]           (W_UV[j,i] is d_latent x d_v)
 *
 * q_nope is the query already absorbed into latent coordinates (no per-head
 * NoPE key or value is ever formed). MLRA-4: NB = 4, d_latent = 128,
 * out_scale = 1/2. MLRA-2: NB = 2, d_latent = 256, out_scale = 1/sqrt(2).
 * MLA: NB = 1, d_latent = 512, out_scale = 1. Every form caches
 * NB*d_latent + d_rope = 512 + 64 elements per token.
 *
 * The shard form, NB = 1 and d_latent = 128 (bf16, at most 32 query heads), is
 * one GPU's share of MLRA-4 when its latent heads are spread over four GPUs
 * ("Key Contributions" #2): latent head j plus the RoPE key, 128 + 64 elements
 * per token, with W_UV[j] and out_scale = 1/2. The sum of the four shares'
 * outputs is the MLRA-4 output; that sum (a cross-GPU all-reduce) is not part
 * of this library.
 *
 * Threading and streams: every call that takes a stream only enqueues work
 * on that HIP stream (hipStream_t passed as void*, NULL = the null stream) and
 * returns without synchronising. Device-side faults surface at the caller's
 * next synchronisation. Calls are thread-safe; error text is thread-local.
 *
 * Ownership: every array argument is a device pointer owned by the caller,
 * except `p` (host). No entry point allocates or frees memory; scratch
 * memory is the caller's `workspace` (mlra_decode_noalloc: a fixed array of
 * this library, one per device).
 *
 * Errors: 0 on success, a negative MLRA_ERR_* code otherwise, with a message
 * in mlra_last_error(). Contract on device data, not checked: 0 <= seqlens[b]
 * <= max_seqlen, and every block-table entry a sequence uses names a valid
 * pool page. seqlens[b] == 0 gives out[b] = 0.
 */
#ifndef MLRA_H_
#define MLRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLRA_ABI_VERSION 1

/* Storage type of q_nope, q_rope, latent_cache and rope_cache.
 * W_UV and out are always fp32; accumulation is always fp32. */
enum { MLRA_BF16 = 0, MLRA_F32 = 1 };

enum {
  MLRA_OK = 0,
  MLRA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLRA_ERR_SHAPE = -2,       /* a size or stride is out of range */
  MLRA_ERR_UNSUPPORTED = -3, /* NB / d_latent / d_rope / d_v / dtype / heads combination not built */
  MLRA_ERR_ALIGN = -4,       /* a base pointer or row stride is not 16-byte aligned */
  MLRA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than mlra_decode_workspace_size */
  MLRA_ERR_HIP = -6          /* the HIP runtime refused a query or a launch */
};

/* Tokens per tile of the split-KV decode; pages must hold a multiple of it. */
#define MLRA_TILE_TOKENS 32
/* Largest number of query heads (two blocks of 32 heads per workgroup). */
#define MLRA_MAX_HEADS 64

typedef struct mlra_decode_params {
  int32_t batch;             /* B >= 0 sequences, one new token each */
  int32_t num_heads;         /* h, 1..MLRA_MAX_HEADS */
  int32_t num_branches;      /* NB: 4 (MLRA-4), 2 (MLRA-2) or 1 (absorbed MLA) */
  int32_t d_latent;          /* channels per latent head: 512 / NB, or 128 with NB = 1 (the shard form) */
  int32_t d_rope;            /* RoPE key channels; must be 64 */
  int32_t d_v;               /* output channels per head; must be 128 */
  int32_t dtype;             /* MLRA_BF16 or MLRA_F32 */
  int32_t page_size;         /* 0: contiguous cache, block_table must be NULL; > 0: paged cache,
                                block_table required, tokens per page, a multiple of 32 */
  int32_t max_seqlen;        /* >= every seqlens[b]; contiguous cache: rows reserved per sequence */
  int32_t max_pages_per_seq; /* paged cache: row stride of block_table (>= ceil(max_seqlen/page_size)) */
  int32_t num_splits;        /* token splits; one workgroup each (the shard form: four per workgroup,
                                one per wave). 0 = one per resident slot on the device (the shard
                                form: four per resident workgroup), and then, for the two-per-CU
                                kernels, when the batch's tiles would give fewer than 56 per split,
                                one split per compute unit instead */
  int32_t reserved;          /* must be 0 */
  int64_t q_stride_b, q_stride_h;   /* q_nope strides in elements; the NB*d_latent row is contiguous */
  int64_t qr_stride_b, qr_stride_h; /* q_rope strides in elements; the d_rope row is contiguous */
  int64_t lat_stride_tok;    /* elements between consecutive cache rows of latent_cache */
  int64_t rope_stride_tok;   /* elements between consecutive cache rows of rope_cache */
  float sm_scale;            /* softmax scale (> 0) applied to the full logit, e.g. 1/sqrt(192) */
  float out_scale;           /* rescale of the branch sum: 1/sqrt(NB) in the MLRA paper's calibration */
} mlra_decode_params;

/* ABI version of the loaded library (MLRA_ABI_VERSION it was built with). */
int mlra_abi_version(void);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* mlra_last_error(void);

/* Host-only validation of `p` (no HIP call, no device). Returns 0 or a negative code. */
int mlra_check_params(const mlra_decode_params* p);

/* Token splits of a call with `p`: p->num_splits if positive, else (compute
 * units of the current device) x (resident workgroups per unit), times four in
 * the shard form (a split per wave). The second case queries the current HIP
 * device. Returns 0 or a negative code. */
int mlra_decode_num_splits(const mlra_decode_params* p, int32_t* num_splits);

/* Bytes of workspace mlra_decode needs for `p` (uses mlra_decode_num_splits). */
int mlra_decode_workspace_size(const mlra_decode_params* p, size_t* bytes);

/*
 * Full decode step: split-KV attention (plan, tile stream, per-latent-head
 * online softmax, partials) followed by the combine: log-sum-exp merge of the
 * partials with the W_UV up-projection, the branch sum and the output scale in
 * the same kernel. Two kernel launches on `stream`.
 *
 *   q_nope        [B][h] rows of NB*d_latent elements (strides q_stride_b/h); dtype
 *   q_rope        [B][h] rows of d_rope elements (strides qr_stride_b/h); dtype
 *   latent_cache  rows of NB*d_latent elements, lat_stride_tok apart; dtype.
 *                 Contiguous (block_table == NULL): token t of sequence b is row b*max_seqlen + t.
 *                 Paged: row block_table[b*max_pages_per_seq + t/page_size]*page_size + t%page_size.
 *   rope_cache    rows of d_rope elements, rope_stride_tok apart, same row numbering; dtype
 *   block_table   int32 [B][max_pages_per_seq] or NULL
 *   seqlens       int32 [B] tokens cached per sequence, the new token included
 *   W_UV          fp32 [NB][h][d_latent][d_v], contiguous (row = latent channel)
 *   out           fp32 [B][h][d_v], contiguous, 16-byte aligned; fully written
 *   workspace     device scratch of at least mlra_decode_workspace_size bytes, 256-byte aligned;
 *                 no contents need to survive between calls
 * Base pointers of q_nope, q_rope, latent_cache, rope_cache and every row stride
 * must be 16-byte aligned. Overlapping calls on one workspace race.
 */
int mlra_decode(const void* q_nope, const void* q_rope, const void* latent_cache, const void* rope_cache,
                const int32_t* block_table, const int32_t* seqlens, const float* W_UV, float* out,
                const mlra_decode_params* p, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the fixed device array that is mlra_decode_noalloc's workspace (one per device). */
#define MLRA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * mlra_decode without a caller workspace, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * arguments and the result are those of mlra_decode; the workspace is a fixed array of
 * MLRA_NOALLOC_SCRATCH_BYTES bytes inside this library, one per device, which the device
 * holds from the first call until the process ends. The first call on a device looks its
 * address up (hipGetSymbolAddress) with that device current; no call allocates or frees
 * memory. A call whose mlra_decode_workspace_size exceeds MLRA_NOALLOC_SCRATCH_BYTES
 * returns MLRA_ERR_WORKSPACE before touching the device. Every call on one device shares
 * that device's array, and nothing in it needs to survive between calls (the kernels write
 * what they later read), so calls that overlap on one device (two streams, two threads)
 * race: serialise them, or give each its own workspace through mlra_decode.
 */
int mlra_decode_noalloc(const void* q_nope, const void* q_rope, const void* latent_cache, const void* rope_cache,
                        const int32_t* block_table, const int32_t* seqlens, const float* W_UV, float* out,
                        const mlra_decode_params* p, void* stream);

/* First half of mlra_decode alone: the split-KV attention kernel, which leaves
 * per-split partials (unnormalised output, running max and sum per latent head
 * and query head) in `workspace`. Same arguments and rules as mlra_decode. */
int mlra_decode_splitkv(const void* q_nope, const void* q_rope, const void* latent_cache, const void* rope_cache,
                        const int32_t* block_table, const int32_t* seqlens, const mlra_decode_params* p,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Second half of mlra_decode alone (one launch): log-sum-exp merge of the
 * partials that mlra_decode_splitkv left in `workspace` (same p, same seqlens,
 * same workspace, after it on the same stream), then
 * out[b,i] = out_scale * sum_j obar_j @ W_UV[j,i]. It may run again on the same
 * partials (it leaves the workspace as it found it). */
int mlra_decode_combine(const int32_t* seqlens, const float* W_UV, float* out, const mlra_decode_params* p,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Query-side absorption (decode step 1 of the pages; "Main Findings" bullet 4 and the
 * block decomposition of "Key Contributions" #1): the NoPE key of query head i in latent
 * head j is latent_j @ W_UK[j,i], so
 *     q_nope[b,i,j,:] = W_UK[j,i] @ q_pre[b,i,j,:]      (d_latent x d_nope times d_nope)
 * turns the NoPE query of each head into latent coordinates, the input mlra_decode takes.
 *   q_pre   [B][h][NB] rows of d_nope = 128 elements (dtype), strides qpre_stride_b/h/j in
 *           elements; qpre_stride_j = 0 shares one NoPE query across the latent heads.
 *           Base pointer and strides 16-byte aligned (MLRA_ERR_ALIGN otherwise)
 *   W_UK    fp32 [NB][h][d_latent][d_nope], contiguous (row = latent channel), 16-byte aligned
 *   q_nope  output, dtype, laid out as mlra_decode reads it (p->q_stride_b, p->q_stride_h;
 *           latent head j at offset j*d_latent); rounded to nearest (even) for bf16
 * One kernel launch on `stream`. Returns 0 or a negative code.
 */
int mlra_absorb_query(const void* q_pre, const float* W_UK, void* q_nope, const mlra_decode_params* p,
                      int32_t d_nope, int64_t qpre_stride_b, int64_t qpre_stride_h, int64_t qpre_stride_j,
                      void* stream);

/*
 * The split plan the two kernels follow, written out for inspection. Every
 * sequence is cut into tiles of MLRA_TILE_TOKENS tokens; the T tiles of all
 * sequences, in order, are cut into G = min(num_splits, T) contiguous ranges
 * whose sizes differ by at most one tile; split g writes one partial per
 * sequence its range touches. Output `plan` (device int32) receives, for split
 * g < G, rows plan[(g*max_segments + k)*3 + {0,1,2}] = {sequence, first tile,
 * end tile} (tile numbers local to the sequence), unused rows {-1,-1,-1}; and
 * plan[num_splits*max_segments*3] = T, plan[.. + 1] = G.
 * Size of `plan`: num_splits*max_segments*3 + 2 int32. Returns 0 or a negative code.
 */
int mlra_decode_plan(const int32_t* seqlens, int32_t batch, int32_t num_splits, int32_t max_segments,
                     int32_t* plan, void* stream);

/* Plain device copy of `bytes` bytes (16-byte aligned pointers, bytes a multiple
 * of 16): the achievable-bandwidth reference and the calibration kernel for the
 * HBM byte counters. */
int mlra_copy_bandwidth_probe(const void* src, void* dst, size_t bytes, void* stream);

/* Read-only stream over `bytes` bytes of `src` (16-byte aligned, multiple of 16)
 * with non-temporal loads, one contiguous chunk per workgroup: the achievable
 * streaming-read bandwidth. XORs every word into *sink (device uint32,
 * caller-initialised), so the reads cannot be dropped. */
int mlra_read_bandwidth_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Grouped-query (GQA) decode attention: the comparator the MLRA paper measures its decode
 * kernel against ("Key Contributions" #4), at the shape it analyses GQA with (64 query heads,
 * 8 KV heads, head dimension 128; "Methodology in Plain English", 4th paragraph). The pages
 * do not define GQA; the standard form is built: query heads are cut into H_kv consecutive
 * groups of G = H_q / H_kv, and for sequence b with L = seqlens[b] tokens, query head i:
 *
 *   g        = i / G
 *   s_t      = sm_scale * <q[b,i,:], k_cache[t,g,:]>
 *   out[b,i] = sum_t softmax_t(s) * v_cache[t,g,:]
 *
 * Same split-KV scheme, page table rules, stream and ownership rules as mlra_decode.
 */
typedef struct mlra_gqa_params {
  int32_t batch;             /* B >= 0 */
  int32_t num_q_heads;       /* H_q >= 1, a multiple of num_kv_heads, H_q / H_kv <= 16 */
  int32_t num_kv_heads;      /* H_kv >= 1 */
  int32_t head_dim;          /* must be 128 */
  int32_t dtype;             /* must be MLRA_BF16 (q, k_cache, v_cache); out is fp32 */
  int32_t page_size;         /* as in mlra_decode_params */
  int32_t max_seqlen;        /* as in mlra_decode_params */
  int32_t max_pages_per_seq; /* as in mlra_decode_params */
  int32_t num_splits;        /* token splits (each launched once per KV head); 0 = resident
                                workgroup slots of the device / num_kv_heads */
  int32_t reserved;          /* must be 0 */
  int64_t q_stride_b, q_stride_h;       /* elements; the head_dim row is contiguous */
  int64_t k_stride_tok, k_stride_head;  /* elements between cache rows / KV heads of k_cache */
  int64_t v_stride_tok, v_stride_head;  /* same for v_cache */
  float sm_scale;            /* > 0, e.g. 1/sqrt(128) */
  float reserved_f;          /* must be 0 */
} mlra_gqa_params;

/* Host-only validation of `p`. Returns 0 or a negative code. */
int mlra_gqa_check_params(const mlra_gqa_params* p);

/* Token splits a GQA call with `p` uses (p->num_splits if positive). Returns 0 or a negative code. */
int mlra_gqa_num_splits(const mlra_gqa_params* p, int32_t* num_splits);

/* Bytes of workspace mlra_gqa_decode needs for `p`. */
int mlra_gqa_workspace_size(const mlra_gqa_params* p, size_t* bytes);

/*
 * GQA decode step, two kernel launches on `stream`: the split-KV attention kernel (one
 * single-wave workgroup per token split and KV head, per-query-head online softmax,
 * partials in `workspace`) and the log-sum-exp merge into `out`.
 *   q        [B][H_q] rows of head_dim elements (strides q_stride_b/h); bf16
 *   k_cache  token t of sequence b, KV head g at row*k_stride_tok + g*k_stride_head, with
 *            row numbered as in mlra_decode (contiguous: b*max_seqlen + t; paged: block
 *            table); bf16. v_cache the same with the v strides.
 *   out      fp32 [B][H_q][head_dim], contiguous; fully written
 * Base pointers and strides 16-byte aligned; workspace 256-byte aligned.
 */
int mlra_gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* seqlens, float* out, const mlra_gqa_params* p, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* MLRA_H_ */
