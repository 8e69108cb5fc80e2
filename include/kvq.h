/* kvq.h — quantized KV cache for single-token decode on AMD MI355X (gfx950).
 *
 * C ABI of libkvq.so.  Two operations make up the path:
 *   kvq_append / kvq_flush_residual  quantize and pack new K/V into the cache;
 *   kvq_decode_attn                  attention of one query token over the whole cache,
 *                                    dequantizing the packed bytes in registers.
 *
 * Method (cited by page title and section):
 *  - affine group quantization: page "KV缓存量化技术：提升大模型长文本生成效率"
 *    (rkmt.cn) §2.1 — per group of 64 values S = (max-min)/(2^n-1), Z = round(-min/S),
 *    codes stored as n-bit integers; stored here as q = clamp(round(x/S)+Z, 0, 2^n-1),
 *    decoded x_hat = S*(q-Z);
 *  - fp16 residual of the most recent R tokens, quantized and merged when full: same page §2.2;
 *    configuration names nbits / group_size / residual_length: same page §3.2;
 *  - stronger quantization (INT2) for early blocks: same page §4.2;
 *  - NVFP4: page "NVFP4 KV缓存技术详解" (glsqs.com) §2.1 — 16 values share one FP8 (E4M3)
 *    scale; the new token is quantized and appended at each decode step;
 *  - every decode step reads the whole history: page "KV Cache量化实战：Model Optimizer为大模型
 *    长上下文省下50%显存" (m.nxbn.cn), section on why long context runs out of memory first.
 *
 * Conventions for every call:
 *  - Device pointers are HIP device addresses owned by the caller.  The library never
 *    allocates or frees device memory and never synchronizes the host with the device, with
 *    one exception: a ragged-batch decode call waits when every pinned host slot of its
 *    cache still has a table copy queued (max(8, 2 * num_layers) slots, at most 256).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *    enqueued on it in call order; calls on one cache must be serialized on one stream.
 *  - Host bookkeeping (lengths) advances when a call enqueues its work, so a call's device
 *    work is fixed when it is enqueued.  Under HIP graph capture, a captured decode call
 *    (uniform batch) replays the same attention over the same tokens each time: its counters
 *    and cursors in the workspace are back at zero when each launch ends, and no call records
 *    a memset.  Replaying a captured append writes the same slots again without advancing
 *    the lengths, and a ragged decode call's table copy reads a pinned slot that later calls
 *    reuse, so neither is meant to be captured.
 *  - Return value: KVQ_OK (0) or a negative kvq_status.  Every argument and capacity check
 *    happens before anything is enqueued; on any error except KVQ_EHIP nothing is enqueued
 *    and the cache state is unchanged.  KVQ_EHIP means a kernel launch failed; the
 *    contents of that layer are then undefined.  kvq_last_error() describes the failure.
 *  - head_dim is 128.  K/V/Q must hold finite fp16 values.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_cache kvq_cache; /* opaque host handle */

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,    /* bad argument or configuration */
  KVQ_ECAPACITY = -2, /* appending would exceed max_tokens */
  KVQ_ENOSPACE = -3,  /* device buffer or workspace too small */
  KVQ_EHIP = -4,      /* a HIP launch failed */
  KVQ_ESTATE = -5     /* operation not valid in the current state (e.g. decode on an empty cache) */
} kvq_status;

typedef enum {
  KVQ_FMT_FP16 = 0,  /* the values themselves: the residual's storage, and as a tier format the
                        unquantized baseline (page "KV缓存量化技术：提升大模型长文本生成效率" §3.1,
                        the FP16 row of the quality/memory table) */
  KVQ_FMT_INT2 = 2,  /* affine, 2-bit codes, group 64, fp16 S and Z */
  KVQ_FMT_INT4 = 4,  /* affine, 4-bit codes */
  KVQ_FMT_INT8 = 8,  /* affine, 8-bit codes */
  KVQ_FMT_NVFP4 = 16, /* E2M1 codes, one E4M3 scale per 16 values */
  KVQ_FMT_MXFP4 = 64, /* E2M1 codes, one E8M0 power-of-two scale per 32 values (the microscaling
                         FP4 that page "NVFP4 KV缓存技术详解" §3.2 compares NVFP4 with) */
  KVQ_FMT_FP8 = 32    /* every value cast to E4M3 (scale 1, round to nearest even, saturating
                         at +-448, sign kept): page "KV Cache量化实战：Model Optimizer为大模型长上下文
                         省下50%显存", section on the KV cache formats (FP8 cast with a fixed scale) */
} kvq_format;

typedef struct {
  int32_t num_layers;   /* >= 1 */
  int32_t batch;        /* >= 1 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim;     /* must be 128 */
  int64_t max_tokens;   /* per-sequence capacity, >= 1 */
  int32_t format;       /* kvq_format of the (young) tier ("nbits") */
  int32_t group_size;   /* 64 for affine formats, 16 for NVFP4, 32 for MXFP4, 0 for FP8 and FP16
                           ("group_size") */
  int32_t residual_len; /* fp16 residual length R: 0 (quantize on append) or a multiple of
                           16 up to 1024 ("residual_length"; 128 in the pages) */
  int32_t old_format;   /* kvq_format of the old tier; ignored when old_after == 0 */
  int64_t old_after;    /* a chunk of tokens quantized together goes to the old tier when
                           all of them are at least old_after positions behind the length
                           at the end of the append call; 0 disables the old tier */
  int32_t k_per_channel; /* 1: K is quantized per channel, each dim's values over a window of
                           128 consecutive tokens forming one affine group (page
                           "KV缓存量化技术：提升大模型长文本生成效率" §2.1, per-channel grouping);
                           V stays per token in groups of 64.  Needs an affine format with
                           group_size 64 (and an affine old format), residual_len a positive
                           multiple of 128; kvq_flush_residual then flushes only whole windows.
                           0: per-token groups for K and V. */
  int32_t demote_young; /* 1: tokens age into the old tier while decoding (page
                           "KV缓存量化技术：提升大模型长文本生成效率" §4.2, stronger quantization
                           for early blocks): at the end of every kvq_append and
                           kvq_flush_residual, while the first live young block is full and its
                           last token is at least old_after positions behind the length, that
                           block's 128 tokens are appended to the old tier, quantized in
                           old_format from the fp16 rounding (to nearest even, saturating at
                           +-65504) of their decoded young values; the young tier then starts
                           one block later.  Needs old_after > 0, an affine format with
                           group_size 64 and per-token K, and a quantized old_format.
                           0: a stored token keeps its tier. */
} kvq_config;

/* Bytes of device memory a cache with this configuration needs (0 if cfg is invalid):
   per layer the fp16 residual (R slots of K and V), the young tier arena and the old tier
   arena of every (batch, kv_head), each region 256-byte aligned.  A tier arena holds
   ceil(slots / 128) blocks of its format's size (144 bytes per token for INT4 and NVFP4, 80
   for INT2, 272 for INT8, 136 for MXFP4, 256 for FP8, 512 for FP16, per kv head; page "KV
   Cache量化实战：Model Optimizer为大模型长上下文省下50%显存", section on why long context runs
   out of memory first, gives the size as 2 * layers * kv heads * head_dim * tokens * bytes
   per value, which these sizes follow plus their scales).  Host-only. */
size_t kvq_cache_bytes(const kvq_config *cfg);

/* Create a cache over caller-owned device memory dev_buf of dev_bytes bytes (256-byte
   aligned, at least kvq_cache_bytes(cfg)).  All lengths start at 0.  Host-only: nothing
   is enqueued and dev_buf is not touched.  *out receives the handle.
   Errors: KVQ_EINVAL (cfg, pointers), KVQ_ENOSPACE (dev_bytes too small). */
int kvq_cache_create(const kvq_config *cfg, void *dev_buf, size_t dev_bytes, kvq_cache **out);

/* Free the host handle (not dev_buf).  NULL is accepted. */
int kvq_cache_destroy(kvq_cache *c);

/* Set every layer's length to 0 (host-only; stored bytes are overwritten by later appends). */
int kvq_cache_reset(kvq_cache *c);

/* Append n_tokens new tokens to every sequence of layer `layer`.
   k, v: fp16 [batch][num_kv_heads][n_tokens][128], contiguous, 16-byte aligned, read on the
   stream.  Tokens are processed in order: with R > 0 a token that arrives while the
   residual holds R tokens first flushes those R tokens into the quantized tier (one chunk),
   then goes to the residual; with R = 0 every token is quantized at once.  Appending n
   tokens stores exactly the bytes of n single-token appends when the old tier is off.
   Each sequence of the batch keeps its own schedule (page "KV缓存量化技术：提升大模型长文本
   生成效率" §2.2 describes it for one sequence): when the sequences are at different points
   (a ragged batch, see kvq_append_seq), each follows its own, in launches of its own where
   they differ.  An append that flushes a full residual and then refills it is one launch: the
   flush's workgroups write the new tokens into the residual slots they have just read.
   n_tokens = 0 is a no-op.  Errors: KVQ_EINVAL, KVQ_ECAPACITY (checked for every sequence
   before anything is enqueued), KVQ_EHIP. */
int kvq_append(kvq_cache *c, int32_t layer, const void *k, const void *v, int64_t n_tokens, void *stream);

/* Append n_tokens new tokens to sequence `seq` (0 <= seq < batch) of layer `layer` alone, as
   kvq_append would for that sequence: k, v are fp16 [num_kv_heads][n_tokens][128].  The
   sequences of a batch may so hold different numbers of tokens (a ragged batch: prompts of
   different lengths, sequences that started at different steps); every other call then
   serves each sequence at its own length.  Errors: KVQ_EINVAL (also seq out of range),
   KVQ_ECAPACITY, KVQ_EHIP. */
int kvq_append_seq(kvq_cache *c, int32_t layer, int32_t seq, const void *k, const void *v, int64_t n_tokens,
                   void *stream);

/* Quantize the r tokens currently in the residual of `layer` (one chunk per sequence) and
   empty it (page "KV缓存量化技术：提升大模型长文本生成效率" §2.2: the residual's tokens are
   quantized, merged into the quantized cache and the residual cleared; here that happens on
   demand as well as when a full residual meets a new token).  No-op for a sequence with r = 0.  Errors: KVQ_EINVAL, KVQ_ESTATE (per-channel K
   and a partial window), KVQ_EHIP. */
int kvq_flush_residual(kvq_cache *c, int32_t layer, void *stream);

/* Workspace bytes kvq_decode_attn needs for num_q_heads query heads (any lengths, ragged
   batches included).  0 if the arguments are invalid. */
size_t kvq_decode_workspace_bytes(const kvq_cache *c, int32_t num_q_heads);

/* Attention of one query token per (batch, query head) over every token cached in `layer`:
   out[b][h] = softmax(softmax_scale * q[b][h] . K_hat^T) . V_hat with query head h reading kv
   head h / (num_q_heads / num_kv_heads).  The decoding step of page "NVFP4 KV缓存技术详解"
   §2.1 (each new token attends over the whole cached history), reading the low-precision
   cache itself rather than a dequantized copy (page "KV Cache量化实战：Model Optimizer为大模型
   长上下文省下50%显存", questions section: the engine must actually read the low-precision
   cache for the savings to hold); K_hat, V_hat are the decoded values of each format (affine:
   S*(q-Z), page "KV缓存量化技术：提升大模型长文本生成效率" §2.1) and the residual's fp16 values.
   q: fp16 [batch][num_q_heads][128]; out: [batch][num_q_heads][128] fp32 if out_fp32 else
   fp16; workspace: at least kvq_decode_workspace_bytes() bytes, 16-byte aligned, scratch
   owned by the caller (its contents on entry do not matter).  The cache is not modified.
   num_q_heads must be a multiple of num_kv_heads with a group of at most 16; softmax_scale
   must be positive and finite.  In a ragged batch each sequence attends over its own tokens
   (a sequence with none gets zeros), and the launch's work is split over the sequences in
   proportion to their cached bytes; the per-sequence tables are copied into the workspace
   on the stream (stream-ordered, from pinned host memory).
   Errors: KVQ_EINVAL, KVQ_ENOSPACE (workspace), KVQ_ESTATE (every sequence empty), KVQ_EHIP. */
int kvq_decode_attn(kvq_cache *c, int32_t layer, const void *q, int32_t num_q_heads, float softmax_scale,
                    void *out, int32_t out_fp32, void *workspace, size_t ws_bytes, void *stream);

/* kvq_decode_attn for callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid allocation): the same attention, the
   same kernel and the same result, with the workspace taken from a library-owned scratch
   array instead of an argument.  That array is a file-scope device array of 8 MiB
   (8,388,608 bytes) per GPU, held until the process ends; its device address on the current
   GPU is looked up on the first call there, which also enqueues its clearing on `stream`.
   The call itself allocates nothing (no hipMalloc, hipFree or allocating library routine).
   Every call on a GPU shares that GPU's array: calls that overlap in time on one GPU (on two
   streams, or from two threads) race and must not be made.  Uniform batches only (every
   sequence of the layer at the same length).  Errors: as kvq_decode_attn; KVQ_ENOSPACE when
   the call's workspace (arrival counters, chunk cursors and split partials: about
   batch * num_q_heads * 2 KB at most, more exactly kvq_decode_workspace_bytes' counters plus
   528 bytes per query head and work item) exceeds the 8 MiB; KVQ_ESTATE for a ragged
   batch or an empty layer; nothing is enqueued on any error but KVQ_EHIP. */
int kvq_decode_attn_noalloc(kvq_cache *c, int32_t layer, const void *q, int32_t num_q_heads, float softmax_scale,
                            void *out, int32_t out_fp32, void *stream);

/* One decode step of `layer` in one call: exactly kvq_append(c, layer, k, v, n_tokens, stream)
   followed by kvq_decode_attn(c, layer, q, ...), the step that every generated token makes (it
   appends its K/V and attends over the whole history: page "NVFP4 KV缓存技术详解" §2.1, the
   decoding and cache-update phases).  When at most 64 new tokens go to the fp16 residual
   (no flush, or after the flush that a full residual takes first), the decode launch itself
   writes them there before it reads the residual, so the step costs one launch instead of
   two (more tokens are written by the append's own launches, which spread them over more
   workgroups than the one that reads the residual: by the flush launch when the step
   flushes, else by a copy launch).  NVFP4 without a residual quantizes a
   one-token step inside the decode launch.  All
   arguments of both calls are checked before anything is enqueued; errors as for the two
   calls (on KVQ_EHIP during the append part, the append state has advanced as kvq_append's
   would).  n_tokens = 0 is a plain kvq_decode_attn.  In a ragged batch every sequence's
   residual copy of at most 64 tokens moves into the decode launch likewise (sequences that
   flush first get their quantize launches before it). */
int kvq_append_decode_attn(kvq_cache *c, int32_t layer, const void *k, const void *v, int64_t n_tokens,
                           const void *q, int32_t num_q_heads, float softmax_scale, void *out, int32_t out_fp32,
                           void *workspace, size_t ws_bytes, void *stream);

/* Host counters of a layer whose sequences are all in one state: total cached tokens and
   tokens currently in the residual.  Errors: KVQ_EINVAL, KVQ_ESTATE (a ragged batch: use
   kvq_seq_info). */
int kvq_seq_len(const kvq_cache *c, int32_t layer, int64_t *total, int64_t *in_residual);

/* One sequence's state in a layer (host counters). */
typedef struct {
  int64_t length;             /* tokens cached */
  int64_t residual;           /* of which in the fp16 residual */
  int64_t young_first_block;  /* first live block of its young arena: the blocks before it were
                                 moved to the old tier (demote_young); 0 without demotion */
  int64_t young_tokens;       /* live young slots, from that block on */
  int64_t old_tokens;         /* old slots */
} kvq_seq_info_t;

/* State of sequence `seq` of `layer`.  Host-only.  Errors: KVQ_EINVAL (handle, layer, seq,
   NULL info). */
int kvq_seq_info(const kvq_cache *c, int32_t layer, int32_t seq, kvq_seq_info_t *info);

/* Where a region of a layer lives: region 0 = fp16 residual, 1 = young tier, 2 = old tier.
   The byte layout inside a region is this library's own (the pages give none): 128-slot blocks
   per (batch, kv_head) in the lane order the decode kernel reads, the residual as K rows then
   V in 16-slot tiles; the oracle's layout module writes the same bytes from its own
   specification.
   *offset: byte offset of the region in dev_buf; *bytes: bytes of the region (all batch
   entries and kv heads, [batch][kv_head][...]); *tokens: slots in use per (batch, kv_head)
   of sequence 0 (every sequence's when all are in one state; kvq_seq_info gives each), for
   the young tier its live slots from the sequence's first live block on.
   Any output pointer may be NULL. */
int kvq_layout(const kvq_cache *c, int32_t layer, int32_t region, size_t *offset, size_t *bytes, int64_t *tokens);

/* Plan-only mode (1) updates the host counters exactly as the real calls do but enqueues
   no device work; it lets the bookkeeping run on machines without a GPU.  0 restores
   normal operation. */
int kvq_set_plan_only(kvq_cache *c, int32_t plan_only);

/* Decode work split of this cache.  Default (0): the work items of a (batch, kv_head) share
   its blocks through a cursor in the workspace, which evens out their finishing times; which
   item sums which blocks then varies from call to call, and so may the last bits of the
   output (always within the attention tolerance).  1: every block is assigned to a work item
   up front (chunks dealt round-robin), so that for fixed lengths every call sums in the same
   order and the output is bitwise reproducible.  Host-only; takes effect from the next
   kvq_decode_attn call.  Errors: KVQ_EINVAL (NULL handle). */
int kvq_set_deterministic(kvq_cache *c, int32_t on);

/* Measurement aid (not part of the method): the achievable HBM read rate of one launch, the
   reference the decode call's effective rate is compared with.  kvq_read_probe enqueues one
   kernel that reads every byte of buf once (grid-stride, 16-byte nontemporal loads, eight in
   flight per lane) and writes one uint32
   per lane to sink: the XOR of the 32-bit words that lane read, so that the XOR of the whole
   sink equals the XOR of buf.  buf: device address, 16-byte aligned; bytes: a positive
   multiple of 16; sink: device address, 4-byte aligned, at least kvq_read_probe_sink_bytes()
   bytes (only that many are written).  Both are owned by the caller.  Errors: KVQ_EINVAL (bad
   pointer, alignment or size; nothing enqueued), KVQ_EHIP (launch failed). */
size_t kvq_read_probe_sink_bytes(void);
int kvq_read_probe(const void *buf, size_t bytes, void *sink, size_t sink_bytes, void *stream);

/* Text describing the last failure on the calling thread ("" if none). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
