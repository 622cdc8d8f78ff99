/*
 * dsaidx: the DeepSeek Sparse Attention lightning indexer (scores + top-k) for
 * AMD Instinct MI355X (gfx950). C ABI.
 *
 * The indexer scores a query token t against every key s it may attend
 * (DeepSeek-V3.2 architecture section, Eq. (1)):
 *
 *     I[t,s] = sum_{j=1..64} w[t,j] * ReLU( q[t,j] . k[s] ),   q, k in R^128,
 *
 * with one key per token shared by all 64 indexer heads, and keeps the k
 * tokens with the highest scores (the fine-grained token selection of the same
 * section) as the indices sparse attention reads.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or retains them; scratch memory is a caller-owned
 *    workspace sized by the *_workspace() calls (the vLLM sparse_indexer page
 *    pre-sizes all per-row scratch so a layer op allocates nothing per step).
 *  - Every call is asynchronous on ``stream`` (a hipStream_t; NULL = the null
 *    stream) and returns after enqueueing. Outputs are valid once the stream
 *    has reached the call. No call synchronises the device or the host.
 *  - Arguments that the host can check are checked before anything is
 *    enqueued (the sparse_indexer builder also checks every kernel requirement
 *    up front and raises instead of falling back). A failed check returns an
 *    error status, enqueues nothing, and sets idx_last_error(). rows == 0 is a
 *    no-op returning IDX_OK.
 *  - Values that live on the device (ranges, lengths, page and block ids) are
 *    not checked on the host. The kernels clamp every such value into the
 *    buffers the call describes, so a bad value can give wrong scores but never
 *    an out-of-bounds access; idx_device_errors() reports that it happened.
 *  - q: [rows, 64, 128], bf16 (when the keys are bf16) or fp8 e4m3fn (OCP,
 *    the gfx950 native fp8; used with fp8 and MXFP4 keys). No q scale: a
 *    caller with one folds it into w. w: [rows, 64] fp32.
 *  - Key formats (k_dtype) and their scale arrays:
 *      IDX_BF16      key = 128 bf16 (256 B per token); k_scale unused (NULL).
 *      IDX_FP8_E4M3  key = 128 e4m3fn codes (128 B per token) times the
 *                    token's fp32 scale (k_scale: float per token, >= 0). The
 *                    llama.cpp thread on the V3.2 checkpoint calls these
 *                    scales quantisation factors; they multiply on decode.
 *      IDX_MXFP4     key = 128 e2m1 codes (64 B per token; byte j holds element
 *                    2j in its low nibble and 2j+1 in its high nibble) with one
 *                    UE8M0 scale byte per 32 elements (k_scale: 4 bytes per
 *                    token, byte g scales elements 32g..32g+31). This is the
 *                    MXFP4 indexer cache with UE8M0-packed granularity-32
 *                    scales of the vLLM sparse_indexer page.
 *  - Scores are fp32. Positions a row does not score are written as -inf.
 *  - Leading dimensions (ld, bt_ld, cand_ld, out_ld) count elements.
 *  - Pointers to code arrays (q, k, k_pages) and the head weights w must be
 *    16-byte aligned and every other float / int32 array 4-byte aligned
 *    (IDX_ERR_ARG otherwise).
 */
#ifndef DSAIDX_H
#define DSAIDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IDX_HEADS 64
#define IDX_DIM 128
#define IDX_MAX_K 2048

typedef void* idx_stream_t; /* a hipStream_t */

typedef enum idx_status {
    IDX_OK = 0,
    IDX_ERR_ARG = 1,         /* null pointer, negative size, ld too small, misaligned */
    IDX_ERR_UNSUPPORTED = 2, /* heads/dim, dtype combination, page or block size, k range */
    IDX_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace() */
    IDX_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} idx_status;

typedef enum idx_dtype {
    IDX_BF16 = 1,
    IDX_FP8_E4M3 = 2,
    IDX_MXFP4 = 3
} idx_dtype;

/* idx_topk / idx_select flags */
#define IDX_TOPK_UNSORTED 1u    /* return the selected set in no particular order */
#define IDX_SELECT_NO_CUTOFF 2u /* idx_select only: skip the sampled cutoff of the one-pass
                                   selection and finish every scored entry exactly (the
                                   same result, slower; for checking the exact finish) */
#define IDX_SELECT_ONE_PASS 4u  /* idx_select only: take the one-pass selection (scores kept
                                   in the scan, cut there, exact finish) for every shape
                                   that allows it (8..512 rows of a decode source), not only
                                   for rows long enough to need the long-row top-k; the same
                                   result (a testing aid and a tuning knob) */

/* ------------------------------------------------------------------ scores */

/*
 * idx_logits: rows that score a contiguous key range.
 *
 * Row r scores keys row_ks[r] .. row_ke[r]-1 of the flat key array
 * k[n_keys, key bytes] (the K-range start/end per row of the vLLM
 * sparse_indexer page: a prefill chunk passes cu_seqlen_ks/ke, a decode row
 * 0 and its context length):
 *     logits[r][c] = I(r, row_ks[r] + c)   for c < row_ke[r] - row_ks[r]
 *     logits[r][c] = -inf                  for the rest of [0, ld).
 * A prefill chunk encodes its causal mask in row_ke (query at position p sees
 * keys 0..p). Needs 0 <= row_ks <= row_ke <= n_keys and row_ke - row_ks <= ld
 * (device values; clamped, see above).
 * q_dtype must be IDX_BF16 with k_dtype IDX_BF16, else IDX_FP8_E4M3.
 * The rows are scanned one by one (each key range read once per row), whatever
 * their number: right for decode rows with their own contexts. A prefill chunk,
 * whose queries share one key range, should call idx_logits_prefill.
 */
idx_status idx_logits(const void* q, int q_dtype, const float* w, const void* k,
                      const void* k_scale, int k_dtype, int64_t n_keys,
                      const int32_t* row_ks, const int32_t* row_ke, int rows, float* logits,
                      int64_t ld, idx_stream_t stream);

/*
 * idx_logits_prefill: idx_logits for the queries of one prefill chunk, which share
 * their key array (the fp8_mqa_logits step of the vLLM sparse_indexer page, per-query
 * cu_seqlen_ks/ke over one K). Same arguments and results as idx_logits. fp8 calls of
 * at least 256 rows run the tiled MFMA kernel, which reads each key tile once for a
 * block of queries and the union of their ranges; fewer rows, or bf16 / MXFP4 keys, run
 * the row scan. Rows with disjoint ranges are still scored correctly, only slower than
 * with idx_logits (each query block walks the union of its rows' ranges).
 */
idx_status idx_logits_prefill(const void* q, int q_dtype, const float* w, const void* k,
                              const void* k_scale, int k_dtype, int64_t n_keys,
                              const int32_t* row_ks, const int32_t* row_ke, int rows, float* logits,
                              int64_t ld, idx_stream_t stream);

/*
 * idx_logits_paged: rows that score a paged key cache.
 *
 * Keys live in pages of page_size tokens: k_pages[n_pages, page_size, key
 * bytes] with scales k_scale_pages[n_pages, page_size] (fp8: float; MXFP4: 4
 * bytes). Row r belongs to request req = row_req ? row_req[r] : r (the row ->
 * request map of the sparse_indexer page, row_indices; req in [0, bt_rows))
 * and its logical token s sits in page block_table[req * bt_ld + s / page_size],
 * slot s % page_size:
 *     logits[r][s] = I(r, s)   for s < seq_lens[r]
 *     logits[r][s] = -inf      for the rest of [0, ld).
 * block_table is [bt_rows, bt_ld]; bt_rows >= rows when row_req is NULL.
 * Needs seq_lens[r] <= bt_ld * page_size and <= ld; block-table entries for
 * s < seq_lens[r] must be in [0, n_pages) (device values; clamped).
 * page_size must be a positive multiple of 64; k_dtype IDX_FP8_E4M3 or
 * IDX_MXFP4 with q_dtype IDX_FP8_E4M3.
 */
idx_status idx_logits_paged(const void* q, int q_dtype, const float* w, const void* k_pages,
                            const void* k_scale_pages, int k_dtype, int64_t n_pages,
                            int page_size, const int32_t* block_table, int64_t bt_rows,
                            int64_t bt_ld,
                            const int32_t* seq_lens, const int32_t* row_req, int rows,
                            float* logits, int64_t ld, idx_stream_t stream);

/*
 * idx_logits_sparse_blocks: two-level rows that score only their candidate
 * blocks (the candidate-consuming indexer layers of the vLLM sparse_indexer
 * page and of the DeepGEMM sparse MQA-logits release note).
 *
 * Row r owns keys row_ks[r] .. row_ke[r]-1 of k[n_keys, key bytes] and is
 * handed cand_blocks[r * cand_ld + b], ascending unique block ids of
 * block_size tokens (sparse_indices), and n_cols[r], its valid sparse-column
 * count (end). Sparse column c = b * block_size + i names token
 *     tok = cand_blocks[r][b] * block_size + i   (relative to row_ks[r]):
 *     logits[r][c] = I(r, row_ks[r] + tok)  if c < n_cols[r] and
 *                                           tok < row_ke[r] - row_ks[r]
 *     logits[r][c] = -inf                   otherwise, for c in [0, ld).
 * Needs ld >= cand_ld * block_size and n_cols[r] <= cand_ld * block_size.
 * block_size must be a positive multiple of 64; k_dtype IDX_FP8_E4M3 or
 * IDX_MXFP4 with q_dtype IDX_FP8_E4M3.
 */
idx_status idx_logits_sparse_blocks(const void* q, int q_dtype, const float* w, const void* k,
                                    const void* k_scale, int k_dtype, int64_t n_keys,
                                    const int32_t* row_ks, const int32_t* row_ke,
                                    const int32_t* cand_blocks, int64_t cand_ld,
                                    const int32_t* n_cols, int block_size, int rows,
                                    float* logits, int64_t ld, idx_stream_t stream);

/*
 * idx_logits_paged_sparse_blocks: two-level decode rows whose context lives in a
 * paged cache (the fp8_fp4_paged_sparse_mqa_logits step named by the vLLM
 * sparse_indexer page: decode rows carry a per-row block_table next to their
 * sparse_indices, and the indexer cache's page must be a multiple of the sparse
 * block).
 *
 * Row r's context is the paged cache of idx_logits_paged (request req = row_req[r],
 * or r when row_req is NULL; logical token s in page block_table[req * bt_ld +
 * s / page_size], slot s % page_size; seq_lens[r] tokens). It is handed
 * cand_blocks[r * cand_ld + b], ascending unique block ids of block_size tokens, and
 * n_cols[r], its valid sparse-column count. Sparse column c = b * block_size + i names
 * the logical token tok = cand_blocks[r][b] * block_size + i:
 *     logits[r][c] = I(r, tok)   if c < n_cols[r] and tok < seq_lens[r]
 *     logits[r][c] = -inf        otherwise, for c in [0, ld).
 * page_size and block_size: positive multiples of 64 with page_size a multiple of
 * block_size (IDX_ERR_UNSUPPORTED otherwise); ld >= cand_ld * block_size; bt_rows as
 * for idx_logits_paged. k_dtype IDX_FP8_E4M3 or IDX_MXFP4 with q_dtype IDX_FP8_E4M3.
 * Bad device values (page ids, block ids, lengths, requests) are clamped and flagged
 * like the other score calls'.
 */
idx_status idx_logits_paged_sparse_blocks(const void* q, int q_dtype, const float* w, const void* k_pages,
                                          const void* k_scale_pages, int k_dtype, int64_t n_pages, int page_size,
                                          const int32_t* block_table, int64_t bt_rows, int64_t bt_ld,
                                          const int32_t* seq_lens, const int32_t* row_req,
                                          const int32_t* cand_blocks, int64_t cand_ld, const int32_t* n_cols,
                                          int block_size, int rows, float* logits, int64_t ld,
                                          idx_stream_t stream);

/* ------------------------------------------------------------------ top-k */

/*
 * idx_topk: exact top-k of each row of a score matrix (the fine-grained token
 * selection of the DeepSeek-V3.2 architecture section).
 *
 * Row r considers logits[r * ld + c] for c < n, n = lens ? lens[r] : n_cols
 * (clamped to [0, n_cols]); -inf and NaN entries do not exist for selection.
 * The order is: higher value first; equal values (-0.0 == +0.0) by lower
 * index. out_idx[r * out_ld + i], i < k, receives the i-th selected column
 * (selection order unless flags has IDX_TOPK_UNSORTED), or -1 when the row
 * has fewer than k entries; out_val (optional, may be NULL) the matching
 * score or -inf. 1 <= k <= IDX_MAX_K, n_cols <= ld, k <= out_ld.
 * workspace may be NULL when idx_topk_workspace() returns 0.
 */
idx_status idx_topk(const float* logits, int64_t ld, const int32_t* lens, int64_t n_cols, int rows,
                    int k, int32_t* out_idx, float* out_val, int64_t out_ld, uint32_t flags,
                    void* workspace, size_t workspace_bytes, idx_stream_t stream);

size_t idx_topk_workspace(int rows, int64_t n_cols, int k);

/* ------------------------------------------------------------------ candidate blocks */

/*
 * idx_candidate_blocks: the candidate-source step of the two-level indexer. A layer
 * that scored its whole context publishes, per row, the candidate blocks the
 * consuming layers then score with idx_logits_sparse_blocks (vLLM sparse_indexer
 * page: candidate_topk_blocks blocks of candidate_block_size tokens published by the
 * candidate-source layer; DeepGEMM sparse MQA-logits release note).
 *
 * Row r considers logits[r * ld + c] for c < n, n = lens ? lens[r] : n_cols (clamped
 * to [0, n_cols]); block b holds columns b * block_size .. b * block_size +
 * block_size - 1 of those (the last block may be partial). The pages give no
 * ranking rule; the reading taken: a block's score is the largest score of its
 * columns (-inf and NaN entries do not count; a block with none has no score and is
 * never published). The n_top blocks first in the order "higher score first, equal
 * scores (-0.0 == +0.0) by lower block id" are written in ASCENDING block id to
 * cand_blocks[r * cand_ld + i], i < n_cand[r] = min(n_top, blocks with a score), and
 * -1 to positions n_cand[r] .. n_top-1 (positions from n_top on are not written).
 * Equivalently: the first n_top distinct blocks met walking the row in idx_topk's
 * order. cand_blocks and n_cand (times block_size, as the valid column count) are the
 * cand_blocks and n_cols arguments of idx_logits_sparse_blocks.
 *
 * block_size: a multiple of 64 in [64, 4096] (IDX_ERR_UNSUPPORTED otherwise), and
 * ceil(n_cols / block_size) <= 16384. 1 <= n_top <= cand_ld; n_cols <= ld.
 * workspace: idx_candidate_blocks_workspace(rows, n_cols) bytes, 256-byte aligned
 * (may be NULL when that is 0). Asynchronous on stream.
 */
idx_status idx_candidate_blocks(const float* logits, int64_t ld, const int32_t* lens, int64_t n_cols, int rows,
                                int block_size, int n_top, int32_t* cand_blocks, int64_t cand_ld,
                                int32_t* n_cand, void* workspace, size_t workspace_bytes, idx_stream_t stream);

size_t idx_candidate_blocks_workspace(int rows, int64_t n_cols);

/* ------------------------------------------------------------------ sparse attention */

/*
 * idx_sparse_attn_paged: the attention the indexer's selection feeds (DeepSeek-V3.2
 * architecture section, Eq. (2): the output of a query attends only the key-value
 * entries whose index scores are in its top-k). MLA keeps one 576-element entry per
 * token, shared by all heads (the 512- and 576-element vectors of the llama.cpp thread).
 * The pages do not spell the attention out; the reading taken (MLA in its single-shared-
 * entry form): head h of row r scores entry c_s as z = scale * (q[r][h] . c_s) over the
 * row's selected positions, and
 *     out[r][h] = sum_i softmax(z)_i * c_{s_i}[0:512],   lse[r][h] = log sum_i exp(z_i).
 *
 * q        bf16 [rows, heads, 576], 16-byte aligned; heads 16, 32, 64 or 128.
 * kv_pages bf16 [n_pages, page_size, 576] (page_size 64), 16-byte aligned; the logical
 *          position s of row r is in page block_table[req(r) * bt_ld + s / 64], slot
 *          s % 64 (req(r) = row_req ? row_req[r] : r), the indexer cache's addressing.
 * indices  int32 [rows, idx_ld], the first k used: logical positions (idx_select's
 *          paged output). Entries < 0 or >= seq_lens[r] are skipped; a page id outside
 *          [0, n_pages) skips the entry and sets IDX_DEVERR_PAGE.
 * out      fp32 [rows, heads, 512] (16-byte aligned); lse fp32 [rows, heads] or NULL.
 *          A row with no valid entry gets out = 0 and lse = -inf.
 * Scores and the softmax run in fp32 (bf16 products are exact in fp32); the weights
 * are rounded to bf16 for the value product, so |out - exact| <= about 2^-8 * max|value|.
 * workspace: idx_sparse_attn_workspace(rows, heads, k) bytes, 256-byte aligned (may be
 * NULL when that is 0). 1 <= k <= IDX_MAX_K. Asynchronous on stream.
 */
idx_status idx_sparse_attn_paged(const void* q, int heads, const void* kv_pages, int64_t n_pages, int page_size,
                                 const int32_t* block_table, int64_t bt_rows, int64_t bt_ld,
                                 const int32_t* seq_lens, const int32_t* row_req, const int32_t* indices,
                                 int64_t idx_ld, int k, int rows, float scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, idx_stream_t stream);

size_t idx_sparse_attn_workspace(int rows, int heads, int k);

/* ------------------------------------------------------------------ fused select */

typedef enum idx_mode {
    IDX_MODE_DENSE = 1,        /* idx_logits arguments */
    IDX_MODE_PAGED = 2,        /* idx_logits_paged arguments */
    IDX_MODE_SPARSE_BLOCKS = 3, /* idx_logits_sparse_blocks arguments */
    IDX_MODE_PREFILL = 4,       /* idx_logits_prefill arguments (idx_logits's) */
    IDX_MODE_PAGED_SPARSE_BLOCKS = 5 /* idx_logits_paged_sparse_blocks arguments */
} idx_mode;

/* One scoring problem: the arguments of the matching idx_logits* call. Fields a
 * mode does not use are ignored. */
typedef struct idx_problem {
    int32_t mode;
    int32_t rows;
    const void* q;
    int32_t q_dtype;
    int32_t k_dtype;
    const float* w;
    const void* k;       /* dense / sparse: k; paged: k_pages */
    const void* k_scale; /* dense / sparse: k_scale; paged: k_scale_pages */
    int64_t n_keys;      /* dense / sparse: key rows; paged: n_pages */
    const int32_t* row_ks;
    const int32_t* row_ke;
    int64_t max_cols;    /* dense: an upper bound of row_ke - row_ks (>= 1) */
    int32_t page_size;
    int32_t block_size;
    const int32_t* block_table;
    int64_t bt_rows;
    int64_t bt_ld;
    const int32_t* seq_lens;
    const int32_t* row_req;
    const int32_t* cand_blocks;
    int64_t cand_ld;
    const int32_t* n_cols;
} idx_problem;

/*
 * idx_select: scores and exact top-k in one call.
 *
 * Returns in out_idx[r * out_ld + i] the i-th selected KEY POSITION of row r:
 * relative to row_ks (dense), the logical position (paged), or the token
 * position named by the selected sparse column (sparse blocks: relative to row_ks;
 * paged sparse blocks: the logical position; column -> token through cand_blocks,
 * the col_indices step of the sparse_indexer page). The result equals idx_logits*
 * followed by idx_topk (and, for sparse blocks, the column -> token map) bit for bit. out_val
 * (optional) receives the scores. workspace of at least
 * idx_select_workspace(p, k) bytes, 256-byte aligned.
 */
idx_status idx_select(const idx_problem* p, int k, int32_t* out_idx, float* out_val,
                      int64_t out_ld, uint32_t flags, void* workspace, size_t workspace_bytes,
                      idx_stream_t stream);

size_t idx_select_workspace(const idx_problem* p, int k);

/*
 * idx_select_noalloc: idx_select without a workspace argument and without any device
 * allocation, for callers that cannot allocate (code under stream capture, serving
 * loops, hosts that forbid it). The workspace is a static device array of
 * IDX_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on until the
 * process ends; its address is looked up on the device's first call. Same arguments,
 * results and flags as idx_select. Returns IDX_ERR_WORKSPACE (launching nothing) when
 * idx_select_workspace(p, k) exceeds IDX_NOALLOC_SCRATCH_BYTES, and IDX_ERR_HIP if the
 * scratch address cannot be found. Nothing in the scratch needs clearing between calls
 * (the selection's counters are read relative to their value at the start of each call,
 * and the top-k clears its own histogram with a kernel). All calls on one device share the
 * one array: calls that may overlap on a device (different streams, or host threads
 * without ordering) race on it and must be serialised by the caller.
 */
#define IDX_NOALLOC_SCRATCH_BYTES (128u << 20)
idx_status idx_select_noalloc(const idx_problem* p, int k, int32_t* out_idx, float* out_val,
                              int64_t out_ld, uint32_t flags, idx_stream_t stream);

/* ------------------------------------------------------------------ misc */

/* Static text for a status code. */
const char* idx_status_string(idx_status s);

/* The calling thread's message for the last failed call ("" if none). */
const char* idx_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int idx_version(void);

/*
 * Device-side argument errors seen since the last call on the current device:
 * a bit mask of IDX_DEVERR_* (0 = none). Waits for ``stream`` and clears the
 * flags. Returns -1 (and sets idx_last_error) if a HIP call fails.
 */
#define IDX_DEVERR_RANGE 1u  /* row_ks/row_ke/seq_lens/n_cols outside the buffers */
#define IDX_DEVERR_PAGE 2u   /* block-table entry outside [0, n_pages) */
#define IDX_DEVERR_BLOCK 4u  /* candidate block id < 0, or with no token in the row's
                                key range (id * block_size >= row_ke - row_ks); its
                                columns are scored -inf */
#define IDX_DEVERR_SLOT 8u   /* key-cache slot at or past n_slots (idx_kcache_write) */
#define IDX_DEVERR_ORDER 16u /* a row's candidate blocks not strictly increasing: the
                                columns are still scored as given, but equal scores then
                                no longer break ties by token position */
int idx_device_errors(idx_stream_t stream);

/* ------------------------------------------------------------------ key-cache writer */

/*
 * Quantises new indexer keys into the key cache at their slots: the step that fills
 * the cache the scan reads (one extra 128-element key per token and layer, DeepSeek-
 * V3.2 architecture section; fp8 and MXFP4 cache formats of the vLLM sparse_indexer
 * page). The pages give no quantisation recipe; the readings:
 *   IDX_FP8_E4M3: scale = amax / 448 (amax = largest |value| of the key), code =
 *     e4m3fn nearest-even of value * (448 / amax), in float32; amax = 0 gives scale 0
 *     and zero codes. A key then decodes as code * scale, as idx_logits* read it.
 *   IDX_MXFP4: OCP MX v1.0 per group of 32: UE8M0 byte = floor(log2 amax) - 2 + 127,
 *     clamped to [0, 254]; elements value / 2^(byte - 127) to the nearest e2m1 value,
 *     ties to even, magnitudes above 6 to 6; element 2j in the low nibble of byte j.
 *
 * k_new       bf16 [n_new, 128] (new_dtype must be IDX_BF16), 16-byte aligned.
 * slot_mapping int64 [n_new]: key i goes to cache row slot_mapping[i]; a negative slot
 *             (a padding token) writes nothing; a slot >= n_slots writes nothing and
 *             sets IDX_DEVERR_SLOT. For pages of page_size keys, slot = page *
 *             page_size + offset, the layout idx_logits_paged reads.
 * k_cache     fp8: uint8 [n_slots, 128]; MXFP4: uint8 [n_slots, 64]; 16-byte aligned.
 * k_scale     fp8: float [n_slots]; MXFP4: uint8 [n_slots, 4]; 4-byte aligned.
 * Two entries naming the same slot race (either key may win). Asynchronous on stream.
 */
idx_status idx_kcache_write(const void* k_new, int new_dtype, int64_t n_new, const int64_t* slot_mapping,
                            void* k_cache, void* k_scale, int k_dtype, int64_t n_slots, idx_stream_t stream);

/*
 * Measurement aid, not part of the indexer path: reads ``bytes`` bytes of device
 * memory at ``buf`` once (16-byte loads, non-temporal) and discards them, so the time
 * of a call measures the read bandwidth this machine delivers, against which the
 * scan's HBM fraction can be judged. buf 16-byte aligned, bytes a multiple of 16;
 * ``sink`` is a device word the probe may write (to keep its loads). Asynchronous on
 * ``stream``.
 */
idx_status idx_read_probe(const void* buf, size_t bytes, uint32_t* sink, idx_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSAIDX_H */
