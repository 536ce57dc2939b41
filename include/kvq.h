/*
 * kvq.h -- C ABI of a decode-attention library over a KIVI-style asymmetric
 * low-bit KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The cache follows the pages' statement of the problem:
 *  - keys are quantized per channel over groups of G tokens, values per token
 *    over groups of G channels, each group with a min/max scale and zero-point
 *    ("The Asymmetric Key-Value Cache Compression Framework", Summary and
 *    Method; "KV cache quantization: putting the bits in the cached vectors",
 *    full-text-skim notes on KIVI);
 *  - codes use a fixed number of bits per element, 2, 3 or 4 ("Read What
 *    Matters", the NOVA-KV abstract on a fixed per-token bit count; "KVQuant"
 *    review, Problem: 8 levels at 3 bits, 4 at 2 bits);
 *  - the most recent R tokens stay FP16 ("The Asymmetric Key-Value Cache
 *    Compression Framework", In practice), and quantized groups are appended along
 *    the token dimension and combined with that FP16 residual inside attention
 *    ("KV cache quantization ...", full-text-skim notes on the grouped/residual
 *    split);
 *  - q and k may be rotated by a normalized Walsh-Hadamard transform, which keeps
 *    q.k unchanged ("The Asymmetric Key-Value Cache Compression Framework",
 *    Method; "Read What Matters", the Dual-QK abstract).
 *
 * Exact formulas fixed by this library where the pages are silent:
 *  - quantizer (fp32): s32 = (max - min) / (2^b - 1); s = fp16(s32) and
 *    z = fp16(min) are stored; code = clamp(rint_half_even((x - z) * (1 / s)),
 *    0, 2^b - 1) with every operation rounded to fp32; s == 0 gives all-zero codes;
 *  - residual rule: after every append, Q = G * floor(max(0, T - o - R) / G)
 *    tokens [o, o + Q) are quantized and tokens [o + Q, T) stay FP16 (R to R + G - 1
 *    of them), o = 1 with an attention sink (token 0 then stays FP16 too), else 0;
 *  - rotation: natural-order butterflies in fp32, then a multiply by
 *    fp32(1/sqrt(128)); rotated keys are rounded to fp16 before storage, the
 *    rotated query is kept in fp32, values are not rotated;
 *  - attention: softmax(q.k * softmax_scale) over all T tokens of a sequence;
 *    query head hq reads KV head hq / (num_q_heads / num_kv_heads).
 *
 * Conventions for every call:
 *  - All functions have C linkage; no C++ exception crosses the ABI.
 *  - Device pointers are plain device addresses (for example a torch tensor's
 *    data_ptr()); host pointers are ordinary host memory. Callers own every
 *    buffer they pass, and it must stay valid until the stream has passed the call.
 *  - All argument checks run on the host before any launch; on any error they find
 *    the cache state is unchanged and kvq_last_error() describes the problem.
 *  - KVQ_ERR_HIP from kvq_append or kvq_decode_step means a HIP call or launch of
 *    the append failed after work may have been enqueued: group blocks, FP16 window
 *    slots and device records can be partly written. The cache then refuses
 *    kvq_append, kvq_decode_step and kvq_decode_attention (KVQ_ERR_HIP) until every
 *    sequence has been started over with kvq_reset_sequence, or it is destroyed.
 *  - Calls are asynchronous on `stream` unless stated. A handle is not thread safe.
 *  - Inputs holding NaN or Inf give undefined results (they are not scanned).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_cache kvq_cache; /* opaque, owned by the library */

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* bad configuration, pointer, size or index */
  KVQ_ERR_CAPACITY = -2,    /* an append would exceed max_tokens */
  KVQ_ERR_OOM = -3,         /* device allocation failed or dev_bytes too small */
  KVQ_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  KVQ_ERR_NO_DEVICE = -5,   /* no usable GPU (checked after argument validation) */
  KVQ_ERR_EMPTY = -6        /* attention requested over a sequence with no tokens */
} kvq_status;

typedef struct {
  int32_t batch;         /* B: 1 .. 65535 sequences (launch grid limit) */
  int32_t num_q_heads;   /* Hq; a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* Hkv: 1 .. 65535; Hq / Hkv must be 1, 2, 4 or 8. Also
                            B * Hkv * (decode splits + window workgroups) must stay below
                            2^31 (the decode launch's workgroups), checked at creation */
  int32_t head_dim;      /* D; must be 128 */
  int32_t bits;          /* 2, 3 or 4 */
  int32_t group;         /* G: tokens per key group = channels per value group; must be 32 */
  int32_t residual;      /* R >= 0 and a multiple of G: FP16 window of the most recent tokens */
  int32_t rotate;        /* 0 or 1: normalized Walsh-Hadamard transform on q and k */
  int64_t max_tokens;    /* per-sequence capacity, 1 .. 2^30 */
  float softmax_scale;   /* 0 => 1/sqrt(head_dim) */
  int32_t sink;          /* 0 or 1: token 0 of every sequence is an attention sink kept in FP16 for
                            good; groups then cover tokens [1 + gG, 1 + (g+1)G) ("KV cache
                            quantization: putting the bits in the cached vectors", full-text-skim
                            notes: keeping the first token in fp16 helps, most at 2 bits) */
  int32_t rope;          /* 0 or 1: pre-RoPE keys. Appended keys are stored and quantized as given
                            (before the rotary position embedding) and attention rotates every
                            key at its position t (0-based index in its sequence) after
                            dequantization ("KVQuant" review, Method and Key idea). The query passed
                            to decode is already rotated at its own position. Rotary embedding:
                            channels f and f + 64 (f < 64) turn by t * rope_base^(-f / 64):
                            (a, b) -> (a cos - b sin, b cos + a sin). Not combined with rotate. */
  float rope_base;       /* 0 => 10000; otherwise > 1 */
  int32_t page_groups;   /* 0: each (sequence, kv-head) owns room for max_tokens tokens of groups.
                            P > 0: paged cache (the "KVQuant" review's Limitations and "Where this
                            paper sits" name paged serving stacks as where such caches must fit;
                            its "Sparks" list suggests blocked or paged allocation): a pool of pool_pages pages, each holding P consecutive
                            groups of one sequence for all its kv-heads, laid out [Hkv][P][group
                            block]; the caller assigns pages with kvq_set_pages. P is a power of two
                            up to 65536. */
  int64_t pool_pages;    /* pages in the pool of a paged cache (1 .. 2^31 - 1); ignored otherwise */
} kvq_config;

/* Bytes of device memory a cache with this configuration needs (host only).
 * Layout: per-sequence state, packed group blocks, FP16 residual rings, and the
 * decode workspace, each 256-byte aligned. */
kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* bytes);

/* Create a cache. If dev_mem is NULL the library allocates (and later frees) the
 * memory; otherwise dev_mem must be a device buffer of at least kvq_cache_bytes()
 * bytes, 256-byte aligned, owned by the caller and outliving the handle.
 * The per-sequence state is cleared on `stream`. */
kvq_status kvq_create(const kvq_config* cfg, void* dev_mem, size_t dev_bytes,
                      hipStream_t stream, kvq_cache** out);

/* Append tokens to every sequence.
 *  k, v: device fp16 [B][n_max][Hkv][D], unrotated keys and values; row t of
 *        sequence b is used for t < n_tokens[b].
 *  n_tokens: host int32 [B] with 0 <= n_tokens[b] <= n_max, or NULL for n_max
 *        tokens in every sequence.
 * New keys are rotated when the cache rotates. Every group the residual rule moves
 * out of the FP16 window is quantized and packed on the device; the tokens that
 * stay FP16 are written to the window. k and v may be NULL when no token is
 * appended. Errors: KVQ_ERR_CAPACITY if any sequence would exceed max_tokens. */
kvq_status kvq_append(kvq_cache* c, const void* k, const void* v,
                      const int32_t* n_tokens, int32_t n_max, hipStream_t stream);

/* Decode-step attention of one query per head over every cached token.
 *  q:   device fp16 [B][Hq][D] (unrotated; rotated in the kernel when the cache rotates)
 *  out: device fp32 [B][Hq][D]
 * The packed groups and the FP16 window are read once per KV head; the partial
 * results of the sequence splits are merged in a second kernel.
 * Errors: KVQ_ERR_EMPTY if any sequence holds no token. */
kvq_status kvq_decode_attention(kvq_cache* c, const void* q, float* out, hipStream_t stream);

/* One decode step in one call: exactly kvq_append(c, k, v, n_tokens, n_max)
 * followed by kvq_decode_attention(c, q, out), with the same arguments, results
 * and errors (KVQ_ERR_EMPTY is checked after counting the appended tokens; on any
 * error nothing is appended). For caches without rotation the decode launch itself
 * writes the appended tokens that stay in the FP16 window (their rows are read from
 * k / v), so a step costs the decode kernels plus, once per G tokens, the group
 * flush; rotated caches run the separate window-write kernel first. */
kvq_status kvq_decode_step(kvq_cache* c, const void* k, const void* v, const int32_t* n_tokens, int32_t n_max,
                           const void* q, float* out, hipStream_t stream);

/* Override the number of 32-token groups one workgroup of the decode kernel
 * reads (0 restores the automatic choice). Must be 0 or in [4, 1 << 20]. */
kvq_status kvq_set_decode_split(kvq_cache* c, int32_t groups_per_split);

/* Attach `start` and `stop` to the decode split kernel of every later decode call
 * (kvq_decode_attention, kvq_decode_step) on that call's stream (both NULL to stop):
 * the kernel is then launched with hipExtLaunchKernelGGL, which sets the events to
 * its own start and end timestamps, so hipEventElapsedTime gives the kernel's
 * duration as a kernel trace reports it. The events are owned by the caller; the
 * library only passes them to the launch. */
kvq_status kvq_set_profile_events(kvq_cache* c, hipEvent_t start, hipEvent_t stop);

/* Destroy a handle (NULL is accepted). Synchronizes the creation stream first and
 * frees library-allocated memory. */
void kvq_destroy(kvq_cache* c);

/* Paged caches: give sequence b the pool pages pages[0..n), page i holding its groups
 * [i*P, (i+1)*P). Pages that already hold quantized groups of b (the first
 * ceil(Q/(32 P)) entries) must stay where they are; every page id must be in
 * [0, pool_pages), appear once, and not belong to another sequence. Pages of b that
 * are dropped become free. An append whose groups would need more pages than b has
 * fails with KVQ_ERR_CAPACITY and changes nothing. The table update is ordered on
 * `stream`; the caller keeps no ownership of `pages` after the call.
 * Errors: KVQ_ERR_INVALID_ARG (cache not paged, bad index, range, ownership). */
kvq_status kvq_set_pages(kvq_cache* c, int32_t b, const int32_t* pages, int32_t n, hipStream_t stream);

/* Start sequence b over (T = Q = 0); in a paged cache its pages become free.
 * Host-side only: the next append rewrites what the kernels read. After a failed
 * append launch (KVQ_ERR_HIP) the cache is usable again once every sequence has
 * been reset this way. */
kvq_status kvq_reset_sequence(kvq_cache* c, int32_t b);

/* Host mirror of sequence b: T = tokens appended, Q = tokens held quantized
 * (tokens [o, o + Q), o = 1 with an attention sink, else 0). */
kvq_status kvq_seq_len(const kvq_cache* c, int32_t b, int64_t* T, int64_t* Q);

/* Parts of the state that kvq_read_state can copy out. */
enum {
  KVQ_PART_GROUPS = 0, /* packed group blocks of (b, h): group g at byte g * kvq_group_bytes()
                          (gathered through the page table in a paged cache) */
  KVQ_PART_RING_K = 1, /* FP16 key window of (b, h): [R + G + sink][D], token t in slot
                          t % (R + G), except an attention sink (token 0) in slot R + G */
  KVQ_PART_RING_V = 2  /* FP16 value window of (b, h), same layout */
};

/* Bytes of one packed 32-token group block: 3072 at 2 bits, 4096 at 3 bits, 5120 at 4
 * bits (0 for other widths).
 * Block layout (little-endian): [key codes | value codes | key scale fp16[128] |
 * key zero fp16[128] | value scales fp16[128] | value zeros fp16[128]].
 * Code words: a code is addressed by (operand o in 0..7, lane l in 0..63,
 * slot s in 0..7). Key token i, channel d: o = 2*(d/32) + i/16,
 * l = i%16 + 16*((d%32)/8), s = d%8. Value token i, channel d: o = d/16,
 * l = d%16 + 16*((i%16)/4), s = 4*(i/16) + i%4.
 *   2-bit: 32-bit word at byte 16*l + 4*(o/2), bits from 8*(s/2) + 4*(s%2) + 2*(o%2);
 *   4-bit: 32-bit word at byte 1024*(o/4) + 16*l + 4*(o%4), bits from 8*(s%4) + 4*(s/4);
 *   3-bit: code bits 0-1 in the 32-bit word at byte 16*l + 4*(o/2), bits from
 *          8*(s%4) + 4*(s/4) + 2*(o%2); code bit 2 in the word at byte
 *          1024 + 8*l + 4*(o/4), bit 8*(s%4) + 4*(s/4) + o%4.
 * Value scale and zero of token i, channel group j sit at fp16 index
 * (4*((i%16)/4) + j)*8 + 4*(i/16) + i%4 of their 128-entry arrays. */
size_t kvq_group_bytes(int32_t bits);

/* Copy `bytes` bytes of one part of (b, h) starting at byte `offset` to host_dst.
 * Synchronizes `stream`. For test and inspection, not on the hot path. */
kvq_status kvq_read_state(kvq_cache* c, int32_t part, int32_t b, int32_t h, size_t offset,
                          void* host_dst, size_t bytes, hipStream_t stream);

/* Message of the last error on this thread ("" if none). */
const char* kvq_last_error(void);

/* ---- Comparison kernels (measured beside the quantized path, not part of it) ---- */

/* Streaming-read probe: reads each 16-byte word of the device buffer buf[0, bytes)
 * once with vector loads spread over the whole GPU, in fold_words workgroups of 256
 * threads (1 .. 65536; a few per compute unit keep enough loads in flight), and
 * stores in fold[i] the xor of the 32-bit words workgroup i read, so the loads
 * cannot be elided: the xor of fold[0 .. fold_words) equals the xor of every word of
 * the buffer. fold is a device array of fold_words uint32 words, wholly written.
 * Timing it gives the achievable HBM read bandwidth to set the decode kernel's
 * effective bandwidth against (the nominal peak is a datasheet figure). bytes:
 * positive multiple of 16; buf 16-byte aligned. Asynchronous on `stream`. */
kvq_status kvq_stream_read(const void* buf, size_t bytes, uint32_t* fold, int32_t fold_words, hipStream_t stream);

/* Decode attention over a plain FP16 KV cache, the full-precision decode that the
 * pages set low-bit caches against (flash-decoding over the whole cache: "Read
 * What Matters", the RDKV abstract). Same attention as kvq_decode_attention:
 * softmax(q.k * softmax_scale) over tokens [0, seq_lens[b]) of sequence b, query
 * head hq reading KV head hq / (num_q_heads / num_kv_heads); no rotation. */
typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t num_q_heads;  /* Hq; Hq / Hkv in {1, 2, 4, 8} */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* must be 128 */
  int64_t t_cap;        /* token capacity per (b, h) of k and v, 1 .. 2^30 */
  float softmax_scale;  /* 0 => 1/sqrt(head_dim) */
} kvq_fp16_config;

/* Bytes of device workspace kvq_fp16_decode_attention needs (host only). */
kvq_status kvq_fp16_workspace_bytes(const kvq_fp16_config* cfg, size_t* bytes);

/*  k, v:     device fp16 [B][Hkv][t_cap][D], token t of (b, h) at row t
 *  seq_lens: device int32 [B], 1 <= seq_lens[b] <= max_len (read by the kernels;
 *            values above t_cap are clamped to t_cap)
 *  max_len:  host upper bound of seq_lens, 1 <= max_len <= t_cap (sizes the grid)
 *  q:        device fp16 [B][Hq][D];  out: device fp32 [B][Hq][D]
 *  workspace: device buffer of at least kvq_fp16_workspace_bytes() bytes, owned by
 *            the caller; calls sharing a workspace must not overlap.
 * Asynchronous on `stream`. */
kvq_status kvq_fp16_decode_attention(const kvq_fp16_config* cfg, const void* k, const void* v,
                                     const int32_t* seq_lens, int64_t max_len, const void* q, float* out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kvq_fp16_decode_attention without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments (less the workspace), checks, split plan and
 * results as kvq_fp16_decode_attention; the split partials go to a static scratch
 * array of 4 MiB that the library holds on each GPU it runs on until the process
 * ends (its address is looked up once per device, on the first call there). The
 * call allocates nothing. Shapes whose partials, B * Hq * splits * 520 bytes, exceed
 * 4 MiB are refused with KVQ_ERR_CAPACITY. Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (other streams, other threads) race and
 * must be ordered by the caller. Nothing in the scratch needs to start at zero:
 * every partial a call reads is written by the same call. */
kvq_status kvq_fp16_decode_attention_noalloc(const kvq_fp16_config* cfg, const void* k, const void* v,
                                             const int32_t* seq_lens, int64_t max_len, const void* q, float* out,
                                             hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
