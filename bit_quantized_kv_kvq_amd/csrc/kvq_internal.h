// Internal declarations shared by the host library and the HIP kernels of libkvq.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kvq {

constexpr int kHeadDim = 128;   // head_dim supported by the kernels
constexpr int kBlock = 128;     // token slots per cache block
constexpr int kGroup = 64;      // affine group (values of one token sharing S, Z)
constexpr int kNvBlock = 16;    // NVFP4 values sharing one E4M3 scale
constexpr int kMxBlock = 32;    // MXFP4 values sharing one E8M0 scale

// Format codes (values of kvq_format).
constexpr int kFmtFp16 = 0, kFmtInt2 = 2, kFmtInt4 = 4, kFmtInt8 = 8, kFmtNvfp4 = 16, kFmtFp8 = 32, kFmtMxfp4 = 64;

// Bytes of one 128-slot block (K and V parts together); affine blocks hold one (S, Z) pair per
// group of gs values (32, 64 or 128) of each token.
// Group-size code 0 (kKc): K per channel over the block's 128 tokens (512 bytes of per-dim S
// and Z), V per token in groups of 64.
constexpr int kKc = 0;
__host__ __device__ constexpr size_t affine_block_bytes(int nbits, int gs = kGroup) {
  return gs == kKc ? 4096u * (size_t)nbits + 1536u : 4096u * (size_t)nbits + 1024u * (size_t)(kHeadDim / gs);
}
constexpr size_t kNvfp4BlockBytes = 18432;
constexpr size_t kMxfp4BlockBytes = 17408;
constexpr size_t kFp8BlockBytes = 32768;
constexpr size_t kFp16BlockBytes = 65536;
__host__ __device__ constexpr bool is_affine(int fmt) { return fmt == kFmtInt2 || fmt == kFmtInt4 || fmt == kFmtInt8; }
__host__ __device__ constexpr size_t block_bytes(int fmt, int gs = kGroup) {
  return fmt == kFmtNvfp4 ? kNvfp4BlockBytes
         : fmt == kFmtMxfp4 ? kMxfp4BlockBytes
         : fmt == kFmtFp8 ? kFp8BlockBytes
         : fmt == kFmtFp16 ? kFp16BlockBytes
                           : affine_block_bytes(fmt, gs);
}
// Blocks in the decode kernel's LDS ring: four (three in flight) while two workgroups still
// fit in a CU, else three, and two for the 64 KB fp16 blocks.
__host__ __device__ constexpr int decode_ring_depth(size_t bb) { return bb <= 18432 ? 4 : bb <= 40960 ? 3 : 2; }

// Offsets inside an affine block with ng groups per token: [Kc][Km][Vc][Vm], Km and Vm of
// 512 ng bytes.
constexpr size_t aff_km(int n) { return 2048u * (size_t)n; }
constexpr size_t aff_vc(int n, int ng) { return 2048u * (size_t)n + 512u * (size_t)ng; }
constexpr size_t aff_vm(int n, int ng) { return 4096u * (size_t)n + 512u * (size_t)ng; }
// Per-channel K blocks: [Kc][Km 512: S of the 128 dims in MFMA operand order, then Z][Vc][Vm 1024]
constexpr size_t kc_vc(int n) { return 2048u * (size_t)n + 512u; }
constexpr size_t kc_vm(int n) { return 4096u * (size_t)n + 512u; }
// Offsets inside an NVFP4 block.
constexpr size_t kNvKs = 8192, kNvVc = 9216, kNvVs = 17408;
// Offsets inside an MXFP4 block: Kc as NVFP4's, one E8M0 byte per K lane, V bytes pairing
// dims 16(2m) + c and 16(2m+1) + c of one slot, E8M0 bytes [w][g][m][e].
constexpr size_t kMxKs = 8192, kMxVc = 8704, kMxVs = 16896;
// FP8 block: the INT8 code regions (E4M3 bytes), no metadata.
constexpr size_t kF8Vc = 16384;
// FP16 block: K lane strings [tile][chunk][lane][16 B], then V at 32768 [part][k][lane][16 B].
constexpr size_t kF16Vc = 32768;

// One quantize launch: tokens [src_tok0, src_tok0 + count) of a source are quantized into
// slots [dst_slot0, dst_slot0 + count) of a tier arena, for every (batch, kv_head), K and V.
struct QuantArgs {
  // source: kind 0 = caller input fp16 [B][H][src_ntok][128]; kind 1 = the layer's residual;
  // kind 2 = one full block of an affine (groups of 64) tier arena, decoded
  int src_kind;
  const uint8_t *src_arena;       // kind 2: the source arena; src_tok0 is its slot index
  int64_t src_bh_stride;          // kind 2: bytes per (b, h)
  int src_fmt;                    // kind 2: affine format code of the source block
  const uint16_t *k_src, *v_src;  // kind 0
  int64_t src_ntok;               // kind 0: tokens per (b, h) in the input tensor
  uint8_t *res_base;              // kind 1: residual region of the layer (written by cp_count)
  int64_t res_bh_stride;          // kind 1: bytes per (b, h) residual
  int res_len;                    // kind 1: R
  int64_t src_tok0;
  int64_t count;
  // destination
  uint8_t *arena;                 // tier arena of the layer
  int64_t arena_bh_stride;        // bytes per (b, h)
  int64_t dst_slot0;
  int fmt;
  int gs;                         // affine group size (32, 64, 128; kKc: K per channel)
  int B, H;
  int nsplit;                     // workgroups per block (1, or 4: one per 32-slot part; set by
                                  // launch_quantize)
  // kind 1 over the whole residual (src_tok0 0, count R): after reading its residual slots a
  // workgroup writes the caller's last cp_count tokens of k_src / v_src ([B][H][src_ntok][128])
  // into residual slots [0, cp_count); cp_count 0: no copy
  int cp_count;
};

// Copy of caller tokens [src_tok0, src_tok0 + count) into residual slots [dst_slot0, ...).
struct ResCopyArgs {
  const uint16_t *k_src, *v_src;
  int64_t src_ntok;
  int64_t src_tok0;
  int64_t count;
  uint8_t *res_base;
  int64_t res_bh_stride;
  int res_len;
  int64_t dst_slot0;
  int B, H;
};

// One stretch of the cache that the decode kernel streams: a tier arena of one format.
// A tier of a layer as the decode kernel streams it.  The work items of a (b, h) share its
// blocks in units.  Item j first takes the `fixed` units of `chunk` blocks starting at blocks
// (s items + j) chunk, s < fixed; when these do not cover the tier, the (b, h)'s cursor hands
// out the rest: `nbig` units of `chunk` blocks, then single blocks, so that the items of a
// (b, h) finish within about one block of each other.
struct DecodeSeg {
  const uint8_t *base;     // arena of the layer
  int64_t bh_stride;       // bytes per (b, h)
  int64_t ntok;            // valid slots per (b, h)
  int fmt;                 // block format (kFmt*)
  int gs;                  // affine group size (32, 64, 128, kKc; 64 for the other formats)
  int chunk;               // blocks per unit (fixed units and the cursor's big units)
  int items;               // work items per (b, h)
  int fixed;               // units per item assigned up front
  int nbig;                // big units the cursor hands out before the single blocks
  int part0;               // index of this segment's first partial among a (b, h)'s partials
  uint64_t *cursors;       // [B*H] chunk cursors (epoch << 20 | units handed out), kCtrStride words apart
};

constexpr int kMaxSegs = 2;        // old tier, young tier
constexpr int kMaxParts = 128;     // partial results per (b, h) and call
// The arrival counter and every chunk cursor of a (b, h) sit in a 128-byte line of their own
// (word i of an array at i * kCtrStride): the items of one (b, h) fetch-add its cursor for
// every chunk, and atomics on one line serialize where they are performed, so words of
// different (b, h) and tiers must not share one.
constexpr int kCtrStride = 16;
constexpr int kPartialStride = 132;  // floats per (part, head): m, l, -, -, o[128]

// One sequence of a ragged batch (sequences at different lengths), as the decode kernel reads
// it from the workspace: the call's tier segments with this sequence's slots and work split
// (a tier the sequence does not have: ntok 0, items 0), its residual and its pending copy.
struct RagSeq {
  DecodeSeg seg[kMaxSegs];
  int64_t pend_src_tok0;       // this sequence's tokens of the call's append that go to the residual
  int32_t items_total;         // work items per (b, h) of this sequence (at least 1)
  int32_t res_ntok;
  int32_t pend_count, pend_slot0;
};

struct DecodeArgs {
  const uint16_t *q;       // [B][Hq][128] fp16
  void *out;               // [B][Hq][128] fp32 or fp16
  int out_fp32;
  uint64_t *counters;      // [B*H] arrival counters (epoch << 20 | count), kCtrStride words apart
  float *partials;         // [B*H][part_stride][G][kPartialStride]
  int part_stride;         // partial slots per (b, h): the call's most work items of a (b, h) (<= kMaxParts)
  DecodeSeg seg[kMaxSegs];
  int nseg;
  int items_total;         // work items per (b, h), all segments (at least 1)
  int res_item;            // >= 0: work item res_item of every (b, h) holds the residual alone (it
                           // streams no blocks); -1: item (b h-index) % items_total holds it as well
  // fp16 residual, handled by one work item of each (b, h)
  const uint8_t *res_base;
  int64_t res_bh_stride;
  int res_len;             // R (slots allocated)
  int res_ntok;            // r (slots in use)
  int B, H, G;             // Hq = H * G
  float scale_log2;        // softmax_scale * log2(e)
  uint64_t epoch;          // distinct per call (44 bits, never 0), tags the arrival counters and cursors
  int q_lds_off;           // LDS byte offset of the query rows (past the largest block ring)
  // Tokens of the same call's append that go to the residual (pend_count 0: none): the work
  // item holding the residual of a (b, h) copies them there before it reads the residual.
  const uint16_t *pend_k, *pend_v;   // caller input [B][H][pend_src_ntok][128]
  int64_t pend_src_ntok, pend_src_tok0;
  int pend_count, pend_slot0;
  // One new token per (b, h) quantized to NVFP4 by the launch itself (pq_nvfp4 = 1): the item
  // holding the residual of each (b, h) writes the token (pend_k / pend_v, token pend_src_tok0
  // of pend_src_ntok) into slot pq_slot of the young arena (pq_arena, pq_bh_stride bytes per
  // (b, h)), then attends to its decoded values as a one-token residual at res_base; the
  // streamed tier leaves that slot out.
  int pq_nvfp4;
  uint8_t *pq_arena;
  int64_t pq_bh_stride;
  int64_t pq_slot;
  // Ragged batch (null: every sequence has the state above): per sequence a RagSeq overrides
  // the segments' slots and split, the residual and the pending copy; rag_wg[workgroup] packs
  // (b | h << 16 | part << 25) of its work item.
  const RagSeq *rag;
  const uint32_t *rag_wg;
  // Workgroups per CU the call is planned for: 3 when every tier is INT2 with groups of 64
  // and per-token K and G <= 8 (that kernel instantiation holds only this step and needs at
  // most 168 VGPRs; its 4-block ring of 10 KB blocks leaves LDS for three), else 2.
  int occ;
};

// Workspace of kvq_decode_attn_noalloc: a device array of this size per GPU (kvq_noalloc.hip).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
// Device address of the current GPU's scratch array; the first call on a device looks it up
// and enqueues its clearing on stream s.
hipError_t noalloc_scratch(void **ptr, hipStream_t s);

hipError_t launch_quantize(const QuantArgs &a, hipStream_t s);
hipError_t launch_residual_copy(const ResCopyArgs &a, hipStream_t s);
// LDS bytes one decode workgroup needs for the segments in `a`.
size_t decode_lds_bytes(const DecodeArgs &a);
// Dynamic LDS limit of the decode kernel: the fp16 ring (2 x 64 KB) plus 16 query rows
constexpr int kMaxDecodeLds = 144 * 1024;
hipError_t launch_decode(const DecodeArgs &a, int num_wg, hipStream_t s);
// Read probe: kProbeBlocks workgroups of kProbeThreads lanes stream the buffer (grid-stride),
// each lane writes one uint32 to the sink.
constexpr int kProbeBlocks = 8192, kProbeThreads = 256;
constexpr size_t kProbeSinkBytes = (size_t)kProbeBlocks * kProbeThreads * sizeof(uint32_t);
hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);
// Workgroups per CU of a decode call whose tiers have formats fmt[0..n) with group-size codes
// gs[0..n) and G query heads per kv head.
int decode_occupancy(const int *fmt, const int *gs, int n, int G);

}  // namespace kvq
