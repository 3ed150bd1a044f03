/*
 * kivi.h -- C ABI of a KIVI-style low-bit KV cache for MI355X (gfx950).
 *
 * The method (the KIVI explainer page, "ICML 2024論文解説: KIVI — チューニング不要の
 * KVキャッシュ2bit非対称量子化"):
 *   - section 量子化アルゴリズム: b-bit asymmetric uniform quantization,
 *     Q(X) = clamp(round((X - z) / s), 0, 2^b - 1), D(X^) = s X^ + z, with
 *     s = (max - min) / (2^b - 1) and z = min over each group;
 *   - section Per-Channel量子化（Key Cache）: keys take their statistics per
 *     channel (here: per channel over each block of k_block = 32 tokens);
 *   - section Per-Token量子化（Value Cache）: values take theirs per token (here:
 *     per token over each group of v_group = 32 channels), quantized once a
 *     group of tokens has accumulated;
 *   - section 残差バッファ（Residual Buffer）: the newest tokens stay fp16 and
 *     decode attention is one softmax over [D(K_quant); K_res] and
 *     [D(V_quant); V_res], scaled by 1/sqrt(head_dim);
 *   - section アルゴリズム (QuantConfig): b = 2, group sizes 32, residual 128.
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative kivi_status. Nothing aborts.
 *   - Arguments are validated before anything is launched; a call that fails
 *     validation changes no state. kivi_last_error() then describes the fault.
 *   - Device pointers are plain HIP device addresses; `stream` is a hipStream_t
 *     (NULL = the default stream). Calls only enqueue work on that stream and
 *     never synchronise. Host-side counters advance when the call returns.
 *   - The caller owns every device buffer (the cache memory, inputs, outputs);
 *     inputs must stay valid until the stream has executed the call.
 *   - A handle is not thread-safe; distinct handles are independent.
 *   - A launch failure (KIVI_E_DEVICE) leaves the handle unusable: later calls
 *     on it return KIVI_E_STATE. kivi_cache_reset() clears that condition.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KIVI_ABI_VERSION 5

typedef enum {
    KIVI_OK = 0,
    KIVI_E_INVAL = -1,       /* bad argument or shape */
    KIVI_E_UNSUPPORTED = -2, /* bits / head_dim / group sizes outside the supported set */
    KIVI_E_NOMEM = -3,       /* the memory given to kivi_cache_create is too small */
    KIVI_E_CAPACITY = -4,    /* the append would exceed max_tokens */
    KIVI_E_EMPTY = -5,       /* attention on a cache holding no token */
    KIVI_E_DEVICE = -6,      /* a HIP launch failed (message from hipGetErrorString) */
    KIVI_E_STATE = -7,       /* the handle saw an earlier device failure */
    KIVI_E_RAGGED = -8       /* the call needs every sequence to hold the same number of tokens */
} kivi_status;

/* Rows per launch when the sequences of a batch hold different numbers of
 * tokens, or the cache is paged: the rows' counters ride in the kernel
 * arguments, so a larger batch runs as several launches of at most this many
 * rows each. */
#define KIVI_MAX_RAGGED_BATCH 128

enum { KIVI_F16 = 0, KIVI_BF16 = 1 };

/* Shape and quantization settings of one cache (one attention layer).
 * Supported: head_dim in {64, 128, 256}; bits in {2, 4}; k_block = v_group = 32;
 * residual a multiple of k_block (0 allowed); n_q_heads a multiple of
 * n_kv_heads; max_tokens >= 1; max_splits = 0 (library default, 256) or
 * 2..4096. Each sequence (batch row) keeps its own counters: kivi_append and
 * kivi_decode_step add the same number of tokens to every row, while
 * kivi_append_rows and kivi_reset_row let rows differ in length (such a
 * batch runs KIVI_MAX_RAGGED_BATCH rows a launch). Each row follows the same rules
 * (residual ring, flushes) as a batch of one.
 *
 * Serving batches follow the page's Production Deployment Guide (KIVI inside a
 * vLLM inference server): sequences of different lengths share a batch, and
 * each keeps its own residual buffer (section 残差バッファ).
 *
 * Paged blocks (n_pages > 0), for serving: the quantized blocks live in a
 * pool of n_pages pages instead of one region per unit. A page holds one
 * key block (G tokens) of one sequence for all its KV heads, and a block
 * table that the caller owns maps (row, block) to a page; see
 * kivi_set_block_table. A paged cache's calls run KIVI_MAX_RAGGED_BATCH rows a
 * launch. */
typedef struct {
    int32_t batch;       /* B */
    int32_t n_kv_heads;  /* Hkv; a "unit" is one (batch row, KV head): unit = b * Hkv + h */
    int32_t n_q_heads;   /* Hq; query head i reads KV head i / (Hq / Hkv) */
    int32_t head_dim;    /* d */
    int32_t bits;        /* b */
    int32_t k_block;     /* G: tokens per key statistics block */
    int32_t v_group;     /* channels per value statistics group */
    int32_t residual;    /* R: tokens kept fp16 after a flush */
    int32_t max_tokens;  /* capacity of every sequence */
    int32_t max_splits;  /* split-K partial slots per query head (0 = default) */
    int32_t n_pages;     /* 0: one contiguous region per unit; > 0: pages in the shared pool */
    int32_t squat_rank;  /* 0: keys coded per element by rounding (KIVI); 1..32: the SQuat-style
                            key coder with a query subspace of this rank (head_dim 64 or 128) */
} kivi_config;

/* Device-memory layout of a cache, a pure function of the config. All offsets
 * are in bytes from the start of the cache memory and are multiples of 256.
 *
 * Quantized blocks: unit u, key block j (tokens [jG, jG+G)) is one record at
 *   off_blocks + u * unit_stride + j * block_bytes (n_pages = 0), or, with
 *   paged blocks, at off_blocks + (table[b][j] * Hkv + h) * block_bytes for
 *   unit u = b * Hkv + h (a page is page_bytes = Hkv * block_bytes, the pool
 *   n_pages pages, and unit_stride is 0). A record holds in order:
 *     kcode [G][W] uint32   W = head_dim * bits / 32 words per token (token-major)
 *     vcode [head_dim][bits] uint32   bits words per channel (channel-major)
 *     ksz   [head_dim][2] float32   (scale, zero) of each channel over the block
 *     vsz   [G][head_dim / v_group][2] float32   (scale, zero) of each token's groups
 *   at record offsets rec_kcode, rec_vcode, rec_ksz, rec_vsz. A word holds
 *   P = 32/b codes, code i at bits [b*i, b*i + b): key word w of token t holds
 *   channels [w*P, (w+1)*P); value word k of channel c holds the block's
 *   tokens [k*P, (k+1)*P). (Keys are read a token row at a time, values a
 *   channel column at a time.)
 * Residual ring: unit u, slot r (token t lives in slot t mod ring_slots) is
 *   off_ring + u * ring_unit_stride + r * 4 * head_dim: the token's fp16 key
 *   row (head_dim halves) followed by its fp16 value row.
 * Split-K partials: off_partial + ((b * Hq + i) * max_splits + s) * partial_stride,
 *   float32 [head_dim] weighted value sum, then the running maximum (base-2
 *   log domain) and the weight sum. Scratch for kivi_attend_decode. */
typedef struct {
    size_t total_bytes;
    size_t off_blocks, unit_stride, block_bytes;
    size_t rec_kcode, rec_vcode, rec_ksz, rec_vsz;
    int64_t max_blocks; /* key blocks a unit can hold = floor(max_tokens / G) */
    size_t off_ring, ring_unit_stride;
    int64_t ring_slots; /* R + G */
    size_t off_partial, partial_stride;
    int32_t max_splits;
    int32_t n_pages;    /* pages in the pool (0: not paged) */
    size_t page_bytes;  /* Hkv * block_bytes (paged) */
    size_t off_squat;   /* squat_rank > 0: unit u's coder coefficients at off_squat + u * squat_unit_bytes:
                           U [head_dim][squat_r8] then W [head_dim][squat_r8] fp32 (row c: u_c, w_c;
                           columns past squat_rank are 0). Key element j moves by -delta * (u_j . w_c)
                           per error delta of an earlier element c. */
    int32_t squat_r8;   /* squat_rank rounded up to a multiple of 8 (0 without the coder) */
    size_t squat_unit_bytes;
} kivi_layout;

/* Counters of a cache. Tokens [0, n_quant) are quantized, [n_quant, n_tokens)
 * are the fp16 residual (n_resid of them); n_quant is a multiple of G. */
typedef struct {
    int64_t n_tokens, n_quant, n_resid;
} kivi_state;

typedef struct kivi_cache kivi_cache;

/* Bytes of device memory a cache with this config needs: the records of the
 * page's codes, scales and zeros (section 量子化アルゴリズム), the fp16 residual
 * ring (section 残差バッファ（Residual Buffer）) and the split partials. */
int kivi_cache_bytes(const kivi_config* cfg, size_t* bytes);

/* The layout above for this config (the same regions as kivi_cache_bytes). */
int kivi_cache_layout(const kivi_config* cfg, kivi_layout* layout);

/* Make a handle over caller-owned device memory `dev_mem` of `bytes` bytes
 * (at least kivi_cache_bytes; 256-byte aligned) for a config whose bits, group
 * sizes and residual length are the page's QuantConfig fields (section
 * アルゴリズム). Launches nothing. The cache
 * starts empty. dev_mem must outlive the handle. The split plans of
 * kivi_attend_decode fill the compute units of the device that is current
 * when the handle is made (256 when no device answers). */
int kivi_cache_create(const kivi_config* cfg, void* dev_mem, size_t bytes, kivi_cache** out);

/* Frees the host handle only (the device memory stays the caller's).
 * Bookkeeping: no step of the method. */
int kivi_cache_destroy(kivi_cache* cache);

/* Empty the cache (host counters only; launches nothing): every sequence
 * starts again with an empty residual (section 残差バッファ（Residual Buffer）). */
int kivi_cache_reset(kivi_cache* cache);

/* Append ntok >= 1 tokens to every sequence (page sections 残差バッファ（Residual
 * Buffer）: new tokens enter the fp16 residual; Per-Channel量子化 / Per-Token量子化:
 * the keys and values of a group that leaves it are quantized per channel /
 * per token with section 量子化アルゴリズム's Q). k, v: device fp16 [B][Hkv][ntok][d],
 * contiguous. The result is defined token by token: the ring holds R + G
 * slots, and a token arriving when it is full first quantizes the oldest G
 * residual tokens (per-channel key blocks, per-token value groups). Tokens
 * that leave the residual within this call are quantized straight from `k`
 * and `v`; the rest are copied into the ring. KIVI_E_CAPACITY if n_tokens + ntok
 * would exceed max_tokens. */
int kivi_append(kivi_cache* cache, const void* k, const void* v, int32_t ntok, void* stream);

/* Append ntok[b] >= 0 tokens to sequence b, each row by the rules of
 * kivi_append (each sequence's own residual buffer, section 残差バッファ). k, v: device fp16 [B][Hkv][max_ntok][d], contiguous; row b's
 * tokens are its first ntok[b] of the max_ntok slots. ntok: host array of B
 * entries, each in [0, max_ntok]. For prefilling sequences of different
 * lengths, or one row (the others 0) when a new sequence takes a freed row.
 * KIVI_E_CAPACITY if a row would exceed max_tokens. */
int kivi_append_rows(kivi_cache* cache, const void* k, const void* v, const int32_t* ntok, int32_t max_ntok,
                     void* stream);

/* The block table of a paged cache: device int32 [batch][stride] (stride >=
 * max_blocks), caller-owned, read by the kernels of every later call on the
 * handle. Entry [b][j] is the page that holds row b's key block j. Before a
 * call quantizes block j of row b (an append or flush that takes the row past
 * (j + 1) G quantized tokens) and for as long as the row holds it, the entry
 * must name a page in [0, n_pages) that no other (row, block) of the cache
 * uses; rows may take pages in any order, and a page freed by kivi_reset_row
 * may go to another row. The kernels clamp entries into [0, n_pages), so a
 * wrong table gives wrong results, never an access outside the pool. Call it
 * again to move the table; the caller orders its writes to the table before
 * the calls that read it on the stream. KIVI_E_INVAL on a cache that is not
 * paged; every append, flush or attention on a paged cache without a table
 * returns KIVI_E_INVAL. */
int kivi_set_block_table(kivi_cache* cache, const int32_t* table, int32_t stride);

/* Empty sequence `row` (host counters only; launches nothing), so that a new
 * sequence can take the row, as a serving engine reuses a finished request's
 * slot (the page's Production Deployment Guide, vLLM with KIVI). */
int kivi_reset_row(kivi_cache* cache, int32_t row);

/* Quantize, in every row, the oldest floor((n_resid - R) / G) * G residual
 * tokens (none if n_resid < R + G); *n_flushed (may be NULL) receives the
 * largest count of a row. Page sections 残差バッファ（Residual Buffer）(only the
 * newest R tokens need stay fp16) and Per-Token量子化（Value Cache）(values are
 * quantized once a whole group of G tokens has accumulated); the codes follow
 * section 量子化アルゴリズム. */
int kivi_flush(kivi_cache* cache, void* stream, int32_t* n_flushed);

/* Decode attention of one query per head over every cached token (page
 * section 残差バッファ（Residual Buffer）: one softmax over the quantized part
 * and the fp16 residual together, scaled by 1/sqrt(d); section 量子化アルゴリズム:
 * D(x) = s x + z):
 * out[b][i] = sum_t softmax_t(q[b][i] . k_t / sqrt(d)) v_t, with k_t, v_t the
 * dequantized (s * code + z, in fp32) or residual fp16 rows of KV head
 * i / (Hq / Hkv). q: device [B][Hq][d] of q_dtype (KIVI_F16 / KIVI_BF16);
 * out: device float32 [B][Hq][d]. Split-K over key blocks, then a
 * log-sum-exp merge of the splits. Concurrent calls on one cache (several
 * streams) are not allowed: they share the split partials. Each row attends
 * over its own tokens. KIVI_E_EMPTY if a sequence holds no token. */
int kivi_attend_decode(kivi_cache* cache, const void* q, int32_t q_dtype, float* out, void* stream);

/* SQuat-style key coder (the SQuat explainer page, aibr.jp "SQuat", section 3
 * 中核となる技術的要素): keys are quantized element by element, and after each
 * element the elements not yet quantized take the closed-form optimal
 * correction, keeping the error (as far as the remaining elements allow)
 * orthogonal to a subspace of past queries. Scales, zeros, value codes and
 * the record layout stay those of the plain coder, so attention reads such a
 * cache unchanged.
 * kivi_squat_build computes every unit's update coefficients from past
 * queries: q device [B][Hq][n_q][head_dim] of q_dtype (each query head's n_q
 * past queries, e.g. the prompt's), contiguous. Per unit (batch row, KV head):
 * the rank-squat_rank subspace of largest second moment of its query heads'
 * queries, then the coefficients of the objective ||U^T e||^2 + lambda ||e||^2
 * of a key's error e (U the subspace basis); lambda > 0 bounds the correction
 * once fewer free elements remain than the subspace has dimensions. Key
 * blocks quantized by later calls (appends, flushes, decode steps) use them;
 * blocks quantized before the first build keep plain codes. A new build
 * replaces the coefficients of every row (e.g. after a row takes a new
 * sequence). KIVI_E_INVAL on a cache with squat_rank = 0, n_q < 1 or lambda
 * not a positive finite number. */
int kivi_squat_build(kivi_cache* cache, const void* q, int32_t q_dtype, int32_t n_q, float lambda, void* stream);

/* Bytes of the library's own device scratch used by kivi_attend_decode_noalloc
 * (one copy per GPU, held until the process ends). */
#define KIVI_NOALLOC_SCRATCH_BYTES (16u << 20)

/* kivi_attend_decode for callers that cannot allocate device memory or
 * would rather not have the library touch the cache's partial region: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same kernels, split plan and result (bit for bit) as
 * kivi_attend_decode, but the split partials go to the library's static
 * device scratch of KIVI_NOALLOC_SCRATCH_BYTES instead of the cache's
 * partial region. Calls no hipMalloc or other allocating routine; its first
 * call on a device looks up that device's scratch address. KIVI_E_NOMEM
 * (before any launch) when a launch's rows * n_q_heads * n_split *
 * partial_stride exceeds the scratch (rows: the batch, or at most
 * KIVI_MAX_RAGGED_BATCH when the call runs several launches, which reuse the
 * scratch in stream order; a plan of one split needs none). Every call on one
 * GPU shares that GPU's scratch, which holds the last call's partials:
 * calls that overlap on one GPU (other streams, other threads) race. */
int kivi_attend_decode_noalloc(kivi_cache* cache, const void* q, int32_t q_dtype, float* out, void* stream);

/* One decode step in one call (page section 残差バッファ（Residual Buffer）: the
 * new token joins the fp16 residual, a group leaving the newest R is
 * quantized, and the query attends over both parts):
 * kivi_append of one token per sequence (k, v:
 * device fp16 [B][Hkv][1][d]), then kivi_flush if a whole group of G tokens
 * lies beyond the newest R (so the residual cycles through R .. R+G-1 tokens
 * at attention time), then kivi_attend_decode. *n_flushed (may be NULL)
 * receives the largest count the flush quantized in a row. Same contract and
 * errors as the three calls; validation of all three happens before the first
 * launch. */
int kivi_decode_step(kivi_cache* cache, const void* k, const void* v, const void* q, int32_t q_dtype, float* out,
                     void* stream, int32_t* n_flushed);

/* Current counters of the residual rule (section 残差バッファ（Residual
 * Buffer）): quantized and fp16 tokens (KIVI_E_RAGGED when the rows differ:
 * see kivi_query_row). */
int kivi_cache_query(const kivi_cache* cache, kivi_state* state);

/* Current counters of sequence `row` (as kivi_cache_query, one row). */
int kivi_query_row(const kivi_cache* cache, int32_t row, kivi_state* state);

/* Counters the cache would have after kivi_append(ntok), by the flush rule of
 * section 残差バッファ（Residual Buffer） (host only; KIVI_E_RAGGED when the
 * rows differ). */
int kivi_plan_append(const kivi_cache* cache, int32_t ntok, kivi_state* after);

/* Split plan kivi_attend_decode would use now (the split along the tokens and
 * its merge are this library's design, not on the pages): *n_split work-groups per
 * (unit, query-head chunk) along the tokens (the last also takes the fp16
 * residual; with more than one, a merge kernel follows), and about
 * *blocks_per_split key blocks in each. When the call runs several launches
 * (KIVI_MAX_RAGGED_BATCH rows each), the plan of the one with the most splits. */
int kivi_plan_attend(const kivi_cache* cache, int32_t* n_split, int32_t* blocks_per_split);

/* Force the split count of kivi_attend_decode (not on the pages, as
 * kivi_plan_attend; 0 = automatic, else
 * 1..max_splits). Results agree up to fp32 rounding for every choice; for
 * tests and tuning. */
int kivi_set_attend_splits(kivi_cache* cache, int32_t n_split);

/* Message describing the last failing call on this thread ("" if none).
 * Bookkeeping: no step of the method. */
const char* kivi_last_error(void);

/* KIVI_ABI_VERSION of the loaded library. Bookkeeping: no step of the method. */
int kivi_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H */
