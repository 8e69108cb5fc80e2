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

// Format codes (values of kvq_format).
constexpr int kFmtFp16 = 0, kFmtInt2 = 2, kFmtInt4 = 4, kFmtInt8 = 8, kFmtNvfp4 = 16;

// Bytes of one 128-slot block (K and V parts together).
__host__ __device__ constexpr size_t affine_block_bytes(int nbits) { return 4096u * (size_t)nbits + 2048u; }
constexpr size_t kNvfp4BlockBytes = 18432;
__host__ __device__ constexpr size_t block_bytes(int fmt) { return fmt == kFmtNvfp4 ? kNvfp4BlockBytes : affine_block_bytes(fmt); }

// Offsets inside an affine block.
constexpr size_t aff_km(int n) { return 2048u * (size_t)n; }
constexpr size_t aff_vc(int n) { return 2048u * (size_t)n + 1024u; }
constexpr size_t aff_vm(int n) { return 4096u * (size_t)n + 1024u; }
// Offsets inside an NVFP4 block.
constexpr size_t kNvKs = 8192, kNvVc = 9216, kNvVs = 17408;

// One quantize launch: tokens [src_tok0, src_tok0 + count) of a source are quantized into
// slots [dst_slot0, dst_slot0 + count) of a tier arena, for every (batch, kv_head), K and V.
struct QuantArgs {
  // source: kind 0 = caller input fp16 [B][H][src_ntok][128]; kind 1 = the layer's residual
  int src_kind;
  const uint16_t *k_src, *v_src;  // kind 0
  int64_t src_ntok;               // kind 0: tokens per (b, h) in the input tensor
  const uint8_t *res_base;        // kind 1: residual region of the layer
  int64_t res_bh_stride;          // kind 1: bytes per (b, h) residual
  int res_len;                    // kind 1: R
  int64_t src_tok0;
  int64_t count;
  // destination
  uint8_t *arena;                 // tier arena of the layer
  int64_t arena_bh_stride;        // bytes per (b, h)
  int64_t dst_slot0;
  int fmt;
  int B, H;
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

// One stretch of the cache that the decode kernel streams: a tier arena or the residual.
struct DecodeSeg {
  const uint8_t *base;     // arena (or residual region) of the layer
  int64_t bh_stride;       // bytes per (b, h)
  int64_t ntok;            // valid slots per (b, h)
  int fmt;                 // kFmt*; kFmtFp16 for the residual
  int units_per_item;      // blocks (quantized) or 32-slot steps (residual) per work item
  int n_items;             // work items per (b, h)
  int item0;               // index of this segment's first item among all items
  int res_len;             // residual: R
};

struct DecodeArgs {
  const uint16_t *q;       // [B][Hq][128] fp16
  float *partials;         // [n_items_total][B][Hq][132] fp32: m, l, -, -, o[128]
  int n_items_total;
  int B, H, G;             // Hq = H * G
  float scale_log2;        // softmax_scale * log2(e)
};

hipError_t launch_quantize(const QuantArgs &a, hipStream_t s);
hipError_t launch_residual_copy(const ResCopyArgs &a, hipStream_t s);
hipError_t launch_decode_segment(const DecodeArgs &a, const DecodeSeg &seg, hipStream_t s);
hipError_t launch_merge(const DecodeArgs &a, void *out, int out_fp32, hipStream_t s);

constexpr int kPartialStride = 132;  // floats per (item, b, hq) partial

}  // namespace kvq
