// Host side of libkvq: configuration checks, arena planning, the residual / tier schedule
// and kernel launches.  Implements include/kvq.h.
//
// Schedule (page "KV缓存量化技术：提升大模型长文本生成效率" §2.2, residual cache): tokens
// arrive in order; a token that finds the residual full (R tokens) first flushes those R
// tokens into the quantized tier as one chunk.  With R = 0 each token is its own chunk
// (page "NVFP4 KV缓存技术详解" §2.1, update phase).  A chunk goes to the old tier (page
// "KV缓存量化技术…" §4.2, stronger quantization for early blocks) when every token in it is
// at least old_after positions behind the length reached at the end of the append call.
#include "../../include/kvq.h"
#include "kvq_internal.h"

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

using namespace kvq;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// formats a tier's blocks can hold (fp16: the values themselves, the unquantized baseline)
bool is_block_fmt(int f) {
  return f == kFmtInt2 || f == kFmtInt4 || f == kFmtInt8 || f == kFmtNvfp4 || f == kFmtMxfp4 || f == kFmtFp8 ||
         f == kFmtFp16;
}
int group_of(int f) {
  return f == kFmtNvfp4 ? kNvBlock : f == kFmtMxfp4 ? kMxBlock : (f == kFmtFp8 || f == kFmtFp16) ? 0 : kGroup;
}
// Group size of a tier: an affine tier takes the configured group size when the young format
// is affine too, else 64; the other formats have their own fixed grouping (64 passed along).
int tier_gs(const kvq_config *c, int fmt) {
  if (!is_affine(fmt)) return kGroup;
  if (c->k_per_channel) return kKc;
  return is_affine(c->format) ? c->group_size : kGroup;
}

// Young slots [slot0, slot0 + count) hold the tokens at stream positions [pos0, pos0 + count).
struct Run {
  int64_t slot0, pos0, count;
  bool operator==(const Run &o) const { return slot0 == o.slot0 && pos0 == o.pos0 && count == o.count; }
};

struct LayerState {
  int64_t length = 0;  // tokens cached
  int64_t res = 0;     // tokens in the residual
  int64_t young = 0;   // slots used in the young arena
  int64_t old = 0;     // slots used in the old arena
  int64_t young_head = 0;   // young blocks demoted to the old tier (the tier starts after them)
  std::vector<Run> runs;    // positions of the live young slots (kept only when demoting)
  bool operator==(const LayerState &o) const {
    return length == o.length && res == o.res && young == o.young && old == o.old && young_head == o.young_head &&
           runs == o.runs;
  }
};

struct Geometry {
  int64_t young_cap_blocks = 0, old_cap_blocks = 0;
  size_t res_bh = 0, young_bh = 0, old_bh = 0;   // bytes per (b, h)
  size_t off_res = 0, off_young = 0, off_old = 0; // offsets inside a layer
  size_t layer_bytes = 0;
};

const char *check_config(const kvq_config *c) {
  if (!c) return "cfg is NULL";
  if (c->num_layers < 1 || c->batch < 1 || c->num_kv_heads < 1) return "num_layers, batch and num_kv_heads must be >= 1";
  if (c->head_dim != kHeadDim) return "head_dim must be 128";
  if (c->max_tokens < 1) return "max_tokens must be >= 1";
  // the decode cursors count a tier's blocks plus its work items in 20 bits
  if (c->max_tokens > (int64_t)1 << 26) return "max_tokens must be <= 67,108,864";
  if (!is_block_fmt(c->format)) return "format must be KVQ_FMT_FP16/INT2/INT4/INT8/NVFP4/MXFP4/FP8";
  if (is_affine(c->format) ? (c->group_size != 32 && c->group_size != 64 && c->group_size != 128)
                           : c->group_size != group_of(c->format))
    return "group_size must be 32, 64 or 128 for affine formats, 16 for NVFP4, 32 for MXFP4 and 0 for FP8 and FP16";
  if (c->residual_len < 0 || c->residual_len > 1024 || c->residual_len % 16 != 0)
    return "residual_len must be 0 or a multiple of 16 up to 1024";
  if (c->old_after < 0) return "old_after must be >= 0";
  if (c->k_per_channel != 0 && c->k_per_channel != 1) return "k_per_channel must be 0 or 1";
  if (c->demote_young != 0 && c->demote_young != 1) return "demote_young must be 0 or 1";
  if (c->demote_young) {
    if (c->old_after <= 0) return "demote_young needs old_after > 0";
    if (!is_affine(c->format) || c->group_size != kGroup || c->k_per_channel)
      return "demote_young needs an affine young format with groups of 64 (per-token K)";
    if (!is_block_fmt(c->old_format) || c->old_format == kFmtFp16) return "demote_young needs a quantized old_format";
  }
  if (c->k_per_channel) {
    if (!is_affine(c->format) || c->group_size != kGroup) return "k_per_channel needs an affine format with group_size 64";
    if (c->residual_len == 0 || c->residual_len % kBlock != 0)
      return "k_per_channel needs residual_len a positive multiple of 128 (whole windows)";
    if (c->old_after > 0 && !is_affine(c->old_format)) return "k_per_channel needs an affine old_format";
  }
  if (c->old_after > 0) {
    if (!is_block_fmt(c->old_format)) return "old_format must be a block format when old_after > 0";
  }
  return nullptr;
}

Geometry geometry(const kvq_config *c) {
  Geometry g;
  const size_t bh = (size_t)c->batch * (size_t)c->num_kv_heads;
  g.young_cap_blocks = ceil_div(c->max_tokens, kBlock);
  g.old_cap_blocks = c->old_after > 0 && c->max_tokens > c->old_after ? ceil_div(c->max_tokens - c->old_after, kBlock) : 0;
  g.res_bh = (size_t)512 * (size_t)c->residual_len;
  g.young_bh = (size_t)g.young_cap_blocks * block_bytes(c->format, tier_gs(c, c->format));
  g.old_bh = g.old_cap_blocks ? (size_t)g.old_cap_blocks * block_bytes(c->old_format, tier_gs(c, c->old_format)) : 0;
  g.off_res = 0;
  g.off_young = align_up(bh * g.res_bh);
  g.off_old = g.off_young + align_up(bh * g.young_bh);
  g.layer_bytes = g.off_old + align_up(bh * g.old_bh);
  return g;
}

}  // namespace

struct kvq_cache {
  kvq_config cfg;
  Geometry geo;
  uint8_t *base = nullptr;
  size_t bytes = 0;
  std::vector<LayerState> seqs;      // [layer][sequence]: each sequence of the batch has its own schedule
  std::vector<uint8_t> rag_host;     // host copy of a ragged decode call's tables
  // Pinned host slots the ragged tables are copied from (so that the stream-ordered copy never
  // blocks the host), each with an event marking its copy; used round-robin, a slot is
  // rewritten only after its previous copy has completed.
  struct PinnedSlot {
    void *host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
  };
  std::vector<PinnedSlot> pinned;
  size_t pinned_next = 0;
  int plan_only = 0;
  int deterministic = 0;   // decode: chunks assigned up front instead of through the cursor
  int num_cus = 0;

  uint8_t *layer_base(int l) const { return base + (size_t)l * geo.layer_bytes; }
  uint8_t *res(int l) const { return layer_base(l) + geo.off_res; }
  uint8_t *young(int l) const { return layer_base(l) + geo.off_young; }
  uint8_t *old(int l) const { return layer_base(l) + geo.off_old; }
  LayerState &st(int l, int b) { return seqs[(size_t)l * cfg.batch + b]; }
  const LayerState &st(int l, int b) const { return seqs[(size_t)l * cfg.batch + b]; }
  // every sequence of the layer in the same state (the batched path); else a ragged batch
  bool uniform(int l) const {
    for (int b = 1; b < cfg.batch; ++b)
      if (!(st(l, b) == st(l, 0))) return false;
    return true;
  }
  ~kvq_cache() {
    for (PinnedSlot &p : pinned) {
      if (p.ev) {
        if (p.pending) (void)hipEventSynchronize(p.ev);
        (void)hipEventDestroy(p.ev);
      }
      if (p.host) (void)hipHostFree(p.host);
    }
  }
};

namespace {

int check_cache(const kvq_cache *c, int32_t layer) {
  if (!c) return fail(KVQ_EINVAL, "cache handle is NULL");
  if (layer < 0 || layer >= c->cfg.num_layers) return fail(KVQ_EINVAL, "layer %d out of range [0, %d)", layer, c->cfg.num_layers);
  return KVQ_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int hip_check(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(KVQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

// ---------------------------------------------------------------------------- append plan

struct Op {
  enum Kind { kResCopy, kQuantInput, kQuantResidual, kDemote } kind;
  int64_t src_tok0, count, dst_slot0;   // kDemote: src_tok0 = the young block
  int tier;  // 0 young, 1 old (quantize ops)
};

struct Plan {
  std::vector<Op> ops;
  LayerState after;
};

// Tier of a chunk ending at stream position `end` (exclusive) in an append ending at L1.
int chunk_tier(const kvq_config &cfg, int64_t end, int64_t L1) {
  return (cfg.old_after > 0 && end <= L1 - cfg.old_after) ? 1 : 0;
}

// pos0: stream position of the first token (recorded for young chunks when demoting)
void add_quant(Plan &p, Op::Kind kind, int64_t src0, int64_t count, int tier, int64_t pos0, bool track) {
  if (count <= 0) return;
  Op op{kind, src0, count, tier ? p.after.old : p.after.young, tier};
  if (track && tier == 0) {
    auto &rs = p.after.runs;
    if (!rs.empty() && rs.back().slot0 + rs.back().count == op.dst_slot0 && rs.back().pos0 + rs.back().count == pos0)
      rs.back().count += count;
    else
      rs.push_back(Run{op.dst_slot0, pos0, count});
  }
  (tier ? p.after.old : p.after.young) += count;
  // merge with the previous op when it continues the same tier from the same source
  if (!p.ops.empty()) {
    Op &b = p.ops.back();
    if (b.kind == kind && kind == Op::kQuantInput && b.tier == tier && b.src_tok0 + b.count == src0 &&
        b.dst_slot0 + b.count == op.dst_slot0) {
      b.count += count;
      return;
    }
  }
  p.ops.push_back(op);
}

// Demotion: after an append or a flush, every full young block whose last token is old_after
// behind the length moves to the old tier (re-quantized from its decoded values), in order.
// The ops go before a trailing copy into the residual, which they do not touch.
void plan_demotions(const kvq_config &cfg, Plan &p) {
  if (!cfg.demote_young || cfg.old_after <= 0) return;
  LayerState &a = p.after;
  std::vector<Op> dem;
  while ((a.young_head + 1) * kBlock <= a.young) {
    const int64_t last = (a.young_head + 1) * kBlock - 1;   // young slot of the block's last token
    int64_t pos = -1;
    for (const Run &r : a.runs)
      if (last >= r.slot0 && last < r.slot0 + r.count) pos = r.pos0 + (last - r.slot0);
    if (pos < 0 || pos + 1 > a.length - cfg.old_after) break;
    dem.push_back(Op{Op::kDemote, a.young_head, kBlock, a.old, 1});
    a.old += kBlock;
    ++a.young_head;
  }
  // forget the runs of demoted slots
  const int64_t live0 = a.young_head * kBlock;
  std::vector<Run> keep;
  for (const Run &r : a.runs) {
    if (r.slot0 + r.count <= live0) continue;
    const int64_t cut = std::max<int64_t>(0, live0 - r.slot0);
    keep.push_back(Run{r.slot0 + cut, r.pos0 + cut, r.count - cut});
  }
  a.runs.swap(keep);
  const bool tail_copy = !p.ops.empty() && p.ops.back().kind == Op::kResCopy;
  p.ops.insert(tail_copy ? p.ops.end() - 1 : p.ops.end(), dem.begin(), dem.end());
}

Plan plan_append(const kvq_config &cfg, const LayerState &st, int64_t n) {
  Plan p;
  p.after = st;
  const bool track = cfg.demote_young != 0;
  const int64_t R = cfg.residual_len, L = st.length, L1 = L + n, r = st.res;
  p.after.length = L1;
  if (R == 0) {
    int64_t n_old = 0;
    if (cfg.old_after > 0) n_old = std::min<int64_t>(n, std::max<int64_t>(0, L1 - cfg.old_after - L));
    add_quant(p, Op::kQuantInput, 0, n_old, 1, L, track);
    add_quant(p, Op::kQuantInput, n_old, n - n_old, 0, L + n_old, track);
    plan_demotions(cfg, p);
    return p;
  }
  const int64_t total = r + n;
  if (total <= R) {
    p.ops.push_back(Op{Op::kResCopy, 0, n, r, 0});
    p.after.res = total;
    plan_demotions(cfg, p);
    return p;
  }
  const int64_t r_final = (total - 1) % R + 1;
  const int64_t n_chunks = (total - r_final) / R;
  int64_t c0 = 0;
  if (r > 0) {
    p.ops.push_back(Op{Op::kResCopy, 0, R - r, r, 0});            // top the residual up to R
    add_quant(p, Op::kQuantResidual, 0, R, chunk_tier(cfg, L - r + R, L1), L - r, track);
    c0 = 1;
  }
  for (int64_t c = c0; c < n_chunks; ++c)                        // chunk c = input [cR - r, cR - r + R)
    add_quant(p, Op::kQuantInput, c * R - r, R, chunk_tier(cfg, L - r + (c + 1) * R, L1), L - r + c * R, track);
  p.ops.push_back(Op{Op::kResCopy, n - r_final, r_final, 0, 0});
  p.after.res = r_final;
  plan_demotions(cfg, p);
  return p;
}

// capacity of the tier arenas follows from max_tokens; checked again here
int check_capacity(const kvq_cache *c, const Plan &p) {
  if (p.after.young > c->geo.young_cap_blocks * kBlock || p.after.old > c->geo.old_cap_blocks * kBlock)
    return fail(KVQ_ECAPACITY, "tier arena full (young %lld/%lld, old %lld/%lld slots)", (long long)p.after.young,
                (long long)(c->geo.young_cap_blocks * kBlock), (long long)p.after.old, (long long)(c->geo.old_cap_blocks * kBlock));
  return KVQ_OK;
}

// Enqueue a plan's ops for every sequence (seq < 0: the batch shares the plan; k, v are
// [B][H][n][128]) or for sequence seq alone (k, v are its [H][n][128]).
int run_plan(kvq_cache *c, int layer, const Plan &p, const void *k, const void *v, int64_t n, hipStream_t s,
             int seq = -1) {
  const auto &cfg = c->cfg;
  if (int e = check_capacity(c, p)) return e;
  if (c->plan_only) return KVQ_OK;
  const int B = seq < 0 ? cfg.batch : 1;
  const size_t b0 = seq < 0 ? 0 : (size_t)seq * cfg.num_kv_heads;   // first (b, h) of the launch
  uint8_t *res = c->res(layer) + b0 * c->geo.res_bh;
  uint8_t *young = c->young(layer) + b0 * c->geo.young_bh, *old = c->old(layer) + b0 * c->geo.old_bh;
  // A flush of the whole residual whose plan ends with the copy that refills the residual from
  // slot 0: the flush's launch does the copy (each workgroup refills the slots it read; the ops
  // between the two read the caller's tokens or the young arena, never the residual).
  const int nops = (int)p.ops.size();
  int fuse_q = -1;
  if (nops >= 2 && p.ops.back().kind == Op::kResCopy && p.ops.back().dst_slot0 == 0 && p.ops.back().count > 0 &&
      p.ops.back().count <= cfg.residual_len && p.ops.back().src_tok0 + p.ops.back().count == n) {
    for (int i = nops - 2; i >= 0; --i) {
      const Op &o = p.ops[i];
      if (o.kind == Op::kQuantResidual) {
        if (o.src_tok0 == 0 && o.count == cfg.residual_len) fuse_q = i;
        break;
      }
      if (o.kind == Op::kResCopy) break;
    }
  }
  for (int i = 0; i < nops; ++i) {
    const Op &op = p.ops[i];
    if (fuse_q >= 0 && i == nops - 1) break;   // done by the flush
    if (op.kind == Op::kResCopy) {
      ResCopyArgs a{};
      a.k_src = (const uint16_t *)k; a.v_src = (const uint16_t *)v; a.src_ntok = n;
      a.src_tok0 = op.src_tok0; a.count = op.count;
      a.res_base = res; a.res_bh_stride = (int64_t)c->geo.res_bh; a.res_len = cfg.residual_len;
      a.dst_slot0 = op.dst_slot0; a.B = B; a.H = cfg.num_kv_heads;
      if (int e = hip_check(launch_residual_copy(a, s), "residual copy")) return e;
    } else {
      QuantArgs a{};
      a.src_kind = op.kind == Op::kQuantInput ? 0 : op.kind == Op::kQuantResidual ? 1 : 2;
      a.k_src = (const uint16_t *)k; a.v_src = (const uint16_t *)v; a.src_ntok = n;
      a.res_base = res; a.res_bh_stride = (int64_t)c->geo.res_bh; a.res_len = cfg.residual_len;
      a.src_tok0 = op.src_tok0; a.count = op.count;
      if (op.kind == Op::kDemote) {   // one whole young block, decoded and quantized again
        a.src_arena = young;
        a.src_bh_stride = (int64_t)c->geo.young_bh;
        a.src_fmt = cfg.format;
        a.src_tok0 = op.src_tok0 * kBlock;
      }
      a.arena = op.tier ? old : young;
      a.arena_bh_stride = (int64_t)(op.tier ? c->geo.old_bh : c->geo.young_bh);
      a.dst_slot0 = op.dst_slot0;
      a.fmt = op.tier ? cfg.old_format : cfg.format;
      a.gs = tier_gs(&cfg, a.fmt);
      if (a.gs == kKc && (op.dst_slot0 % kBlock != 0 || op.count % kBlock != 0))
        return fail(KVQ_ESTATE, "per-channel K: a quantize of %lld slots at %lld is not whole windows",
                    (long long)op.count, (long long)op.dst_slot0);
      a.B = B; a.H = cfg.num_kv_heads;
      if (i == fuse_q) a.cp_count = (int)p.ops.back().count;   // the last cp_count of the n tokens
      if (int e = hip_check(launch_quantize(a, s), "quantize")) return e;
    }
  }
  return KVQ_OK;
}

// ---------------------------------------------------------------------------- decode plan

// Call tags of the decode counters: 44 bits, never 0 (the value the counters hold between calls).
std::atomic<uint64_t> g_epoch{0};
uint64_t next_epoch() {
  for (;;) {
    const uint64_t e = ++g_epoch & ((1ull << 44) - 1);
    if (e != 0) return e;
  }
}

// Per (b, h): one arrival counter and one chunk cursor per tier, each in a line of its own.
size_t counters_bytes(const kvq_cache *c) {
  return align_up((size_t)c->cfg.batch * c->cfg.num_kv_heads * (1 + kMaxSegs) * kCtrStride * sizeof(uint64_t));
}
// parts: partial slots per (b, h) (a call uses its most work items of one (b, h))
size_t partials_bytes(const kvq_cache *c, int32_t num_q_heads, int parts = kMaxParts) {
  const size_t bh = (size_t)c->cfg.batch * c->cfg.num_kv_heads;
  return align_up(bh * (size_t)parts * (size_t)(num_q_heads / c->cfg.num_kv_heads) * kPartialStride * sizeof(float));
}
// ragged calls: one RagSeq per sequence, then one table entry per workgroup
size_t rag_seq_bytes(const kvq_cache *c) { return align_up((size_t)c->cfg.batch * sizeof(RagSeq)); }
size_t rag_wg_bytes(const kvq_cache *c) {
  return align_up((size_t)c->cfg.batch * c->cfg.num_kv_heads * kMaxParts * sizeof(uint32_t));
}

// An NVFP4 cache without a residual appends a step's token inside the decode launch
// (kvq_append_decode_attn): per (b, h) a one-token fp16 residual of 16 slots (K [16][128],
// V [1][128][16]) holds the token's decoded values.
constexpr size_t kPqResBytes = 2 * 16 * kHeadDim * sizeof(uint16_t);
bool fuses_nvfp4_append(const kvq_config &c) {
  return c.format == kFmtNvfp4 && c.residual_len == 0 && c.old_after == 0 && !c.demote_young;
}
size_t pq_bytes(const kvq_cache *c) {
  return fuses_nvfp4_append(c->cfg) ? align_up((size_t)c->cfg.batch * c->cfg.num_kv_heads * kPqResBytes) : 0;
}

size_t workspace_bound(const kvq_cache *c, int32_t num_q_heads) {
  return counters_bytes(c) + partials_bytes(c, num_q_heads) + rag_seq_bytes(c) + rag_wg_bytes(c) + pq_bytes(c);
}

// The quantized tiers of one sequence as the decode streams them: old, then young from its
// first live block.
struct TierRef {
  const uint8_t *base;
  int64_t stride, ntok, nblk;
  int fmt, gs, slot;   // slot: 0 old, 1 young
};
int tiers_of(const kvq_cache *c, int layer, const LayerState &st, TierRef *t) {
  const auto &cfg = c->cfg;
  int nt = 0;
  if (st.old > 0)
    t[nt++] = {c->old(layer), (int64_t)c->geo.old_bh, st.old, ceil_div(st.old, kBlock), cfg.old_format,
               tier_gs(&cfg, cfg.old_format), 0};
  const int64_t young_live = st.young - st.young_head * kBlock;
  if (young_live > 0)
    t[nt++] = {c->young(layer) + (size_t)st.young_head * block_bytes(cfg.format, tier_gs(&cfg, cfg.format)),
               (int64_t)c->geo.young_bh, young_live, ceil_div(young_live, kBlock), cfg.format,
               tier_gs(&cfg, cfg.format), 1};
  return nt;
}

double tier_bytes(const TierRef &t) { return (double)t.nblk * (double)block_bytes(t.fmt, t.gs); }

// Decode time per byte of a tier relative to INT4 on the same kernel: the INT2 step is
// compute-bound (its unpack, logits and P' per block cost about what INT4's do for 56 % of
// the bytes): on the 128K shape the same number of blocks took 170.3 us as INT2 against
// 219.6 us as INT4, 1.39x per byte.  The other formats stream at about INT4's rate per byte.
double tier_cost(const TierRef &t) { return t.fmt == kFmtInt2 ? 1.4 : 1.0; }
double tier_work(const TierRef &t) { return tier_bytes(t) * tier_cost(t); }

// Give each tier of a (b, h) work items in proportion to its decode time (`target` items in all),
// cut into chunks small enough (about 32 per item) that the items of a (b, h) even out their
// finishing times.  Fills out[i] for tier i (not its cursors); returns the items.
int split_tiers(const kvq_cache *c, const TierRef *t, int nt, int64_t target, DecodeSeg *out) {
  double work = 0;
  for (int i = 0; i < nt; ++i) work += tier_work(t[i]);
  int parts = 0;
  for (int i = 0; i < nt; ++i) {
    int64_t items = std::max<int64_t>(1, (int64_t)((double)target * tier_work(t[i]) / work + 0.5));
    items = std::min<int64_t>(items, kMaxParts / std::max(1, nt));
    // units of about 1/32 of an item's share, at least four blocks (a unit's cursor fetch
    // has four block times to come back), at least eight where the tier has at most 16 items
    // per (b, h) (half the cursor fetches: 128K INT4 187.0 -> 185.7 us, 32K NVFP4 59.4 ->
    // 59.0 us; the 256K tiers, with more items per (b, h), lost 1 % with eight); two fixed
    // units per item, then the cursor's big units, then six single blocks per item for the
    // finish (an item that takes the last big unit as the others take single blocks finishes
    // up to a unit later: with two singles per item the items of one (b, h) ended 3-4 us apart
    // on the 32K and 128K shapes)
    const int64_t nblk = t[i].nblk;
    int64_t chunk = std::max<int64_t>(items <= 16 ? 8 : 4, ceil_div(nblk, items * 32));
    int64_t fixed = 2, nbig = 0;
    if (nblk >= (fixed + 2) * items * chunk) {
      if (c->deterministic)
        fixed = ceil_div(ceil_div(nblk, chunk), items);   // every chunk dealt round-robin up front
      else
        nbig = std::max<int64_t>(0, (nblk - fixed * items * chunk - 6 * items) / chunk);
    } else {
      // too little to share out: single blocks, dealt round-robin
      chunk = 1;
      items = std::min<int64_t>(items, nblk);
      fixed = ceil_div(nblk, items);
    }
    DecodeSeg &s = out[i];
    s.base = t[i].base; s.bh_stride = t[i].stride; s.ntok = t[i].ntok; s.fmt = t[i].fmt; s.gs = t[i].gs;
    s.chunk = (int)chunk; s.items = (int)items; s.fixed = (int)fixed; s.nbig = (int)nbig; s.part0 = parts;
    s.cursors = nullptr;
    parts += (int)items;
  }
  return parts;
}

int num_cus(kvq_cache *c) {
  if (c->num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      c->num_cus = n;
    else
      c->num_cus = 256;
  }
  return c->num_cus;
}

// Every sequence in one state: all work items of the call fill the GPU about once (a.occ
// workgroups per CU: decode_occupancy), the same split for every (b, h).
// hold_young: young slots at the end of the tier that the launch leaves out of the stream and
// attends to as residual slots instead (a token it appends itself).
int plan_decode(kvq_cache *c, int layer, DecodeArgs &a, uint64_t *cursors, int64_t hold_young = 0) {
  const auto &cfg = c->cfg;
  LayerState st = c->st(layer, 0);
  st.young -= hold_young;
  st.res += hold_young;
  const int64_t nbh = (int64_t)cfg.batch * cfg.num_kv_heads;
  TierRef tiers[kMaxSegs];
  const int nt = tiers_of(c, layer, st, tiers);
  int fmts[kMaxSegs], gss[kMaxSegs];
  for (int i = 0; i < nt; ++i) {
    fmts[i] = tiers[i].fmt;
    gss[i] = tiers[i].gs;
  }
  a.occ = decode_occupancy(fmts, gss, nt, a.G);
  const int64_t target = std::min<int64_t>(std::max<int64_t>(1, (int64_t)a.occ * num_cus(c) / nbh), kMaxParts - 1);
  // A residual that alone is at least one work item's share of the (b, h)'s work gets an item of
  // its own, which streams no blocks: riding on a block item it made that item finish last (its
  // fp16 slots cost about 1.5x a quantized byte; on the 1K batch-4 shape, 4 items per (b, h) of 2
  // blocks each, the residual's item took 13 us against 7 us for the others).
  double blk_work = 0.0;
  for (int i = 0; i < nt; ++i) blk_work += tier_work(tiers[i]);
  const double res_work = (double)st.res * 512.0 * 1.5;
  bool own_res = nt > 0 && target >= 2 && st.res > 0 && res_work * (double)target >= blk_work;
  int parts = split_tiers(c, tiers, nt, own_res ? target - 1 : target, a.seg);
  if (own_res && parts + 1 > kMaxParts) {   // (rounding gave the tiers every partial slot)
    own_res = false;
    parts = split_tiers(c, tiers, nt, target, a.seg);
  }
  for (int i = 0; i < nt; ++i) a.seg[i].cursors = cursors ? cursors + (size_t)i * nbh * kCtrStride : nullptr;
  a.nseg = nt;
  a.items_total = std::max(1, parts + (own_res ? 1 : 0));
  a.res_item = own_res ? parts : -1;
  a.res_base = c->res(layer);
  a.res_bh_stride = (int64_t)c->geo.res_bh;
  a.res_len = cfg.residual_len;
  a.res_ntok = (int)st.res;
  a.rag = nullptr;
  a.rag_wg = nullptr;
  return (int)(nbh * a.items_total);
}

// A ragged batch: each sequence gets work items in proportion to its own bytes (the call's
// items still fill the GPU about once) and its own split.  The tables are built in
// c->rag_host (host only); *copy_bytes of them go to the workspace before the launch, *maxp
// is the most work items of one (b, h).  pend[b]: sequence b's pending residual copy (count 0: none).
int plan_decode_ragged(kvq_cache *c, int layer, DecodeArgs &a, uint64_t *cursors, const Op *pend, int *num_wg,
                       int *maxp_out, size_t *copy_bytes) {
  const auto &cfg = c->cfg;
  const int B = cfg.batch, H = cfg.num_kv_heads;
  const int64_t nbh = (int64_t)B * H;
  if (B > 65536 || H > 512) return fail(KVQ_EINVAL, "ragged decode supports batch <= 65536 and kv heads <= 512");
  // the call's segments: a tier that any sequence has (old first, as for one sequence)
  std::vector<TierRef> tb((size_t)B * kMaxSegs);
  std::vector<int> nts(B);
  std::vector<double> work(B, 0.0);   // decode time of each sequence, in INT4 bytes
  bool has[2] = {false, false};
  double total = 0;
  for (int b = 0; b < B; ++b) {
    nts[b] = tiers_of(c, layer, c->st(layer, b), &tb[(size_t)b * kMaxSegs]);
    for (int i = 0; i < nts[b]; ++i) {
      has[tb[(size_t)b * kMaxSegs + i].slot] = true;
      work[b] += tier_work(tb[(size_t)b * kMaxSegs + i]);
    }
    work[b] += 512.0 * (double)c->st(layer, b).res;
    total += work[b];
  }
  int seg_of[2] = {-1, -1};
  a.nseg = 0;
  for (int slot = 0; slot < 2; ++slot) {
    if (!has[slot]) continue;
    DecodeSeg &s = a.seg[a.nseg];
    s = DecodeSeg{};
    s.base = slot ? c->young(layer) : c->old(layer);
    s.bh_stride = (int64_t)(slot ? c->geo.young_bh : c->geo.old_bh);
    s.fmt = slot ? cfg.format : cfg.old_format;
    s.gs = tier_gs(&cfg, s.fmt);
    s.cursors = cursors + (size_t)a.nseg * nbh * kCtrStride;
    seg_of[slot] = a.nseg++;
  }
  // items per (b, h) of sequence b: ceil(work_b / budget), with the smallest per-item budget
  // whose items still fit the GPU once (so that the most loaded item carries as little as the
  // slots allow; rounding each share to the nearest count would leave some items ~10 % heavier)
  int fmts[kMaxSegs], gss[kMaxSegs];
  for (int u = 0; u < a.nseg; ++u) {
    fmts[u] = a.seg[u].fmt;
    gss[u] = a.seg[u].gs;
  }
  a.occ = decode_occupancy(fmts, gss, a.nseg, a.G);
  const int64_t slots = (int64_t)a.occ * num_cus(c);
  auto items_for = [&](double budget) {
    int64_t n = 0;
    for (int b = 0; b < B; ++b) n += H * std::max<int64_t>(1, (int64_t)std::ceil(work[b] / budget));
    return n;
  };
  double lo = total / (double)slots * H, hi = std::max(total, 1.0);   // items_for(hi) = B H
  if (items_for(lo) <= slots) hi = lo;
  for (int it = 0; it < 60 && hi > lo * (1 + 1e-9); ++it) {
    const double mid = 0.5 * (lo + hi);
    (items_for(mid) <= slots ? hi : lo) = mid;
  }
  c->rag_host.assign(rag_seq_bytes(c) + rag_wg_bytes(c), 0);
  RagSeq *rs = (RagSeq *)c->rag_host.data();
  int maxp = 1;
  for (int b = 0; b < B; ++b) {
    RagSeq &r = rs[b];
    for (int u = 0; u < a.nseg; ++u) {
      r.seg[u] = a.seg[u];
      r.seg[u].chunk = 1;
    }
    const int64_t target = std::max<int64_t>(1, (int64_t)std::ceil(work[b] / hi));
    DecodeSeg out[kMaxSegs];
    const int parts = split_tiers(c, &tb[(size_t)b * kMaxSegs], nts[b], target, out);
    for (int i = 0; i < nts[b]; ++i) {
      const int u = seg_of[tb[(size_t)b * kMaxSegs + i].slot];
      out[i].cursors = a.seg[u].cursors;
      r.seg[u] = out[i];
    }
    r.items_total = std::max(1, parts);
    r.res_ntok = (int)c->st(layer, b).res;
    if (pend && pend[b].count > 0) {
      r.pend_src_tok0 = pend[b].src_tok0;
      r.pend_count = (int)pend[b].count;
      r.pend_slot0 = (int)pend[b].dst_slot0;
    }
    maxp = std::max(maxp, r.items_total);
  }
  // part-major, so that the items of a (b, h) are spread over the launch
  uint32_t *wg = (uint32_t *)(c->rag_host.data() + rag_seq_bytes(c));
  int n = 0;
  for (int p = 0; p < maxp; ++p)
    for (int b = 0; b < B; ++b)
      if (p < rs[b].items_total)
        for (int h = 0; h < H; ++h) wg[n++] = (uint32_t)b | ((uint32_t)h << 16) | ((uint32_t)p << 25);
  *copy_bytes = rag_seq_bytes(c) + (size_t)n * sizeof(uint32_t);
  *maxp_out = maxp;
  a.items_total = 1;
  a.res_base = c->res(layer);
  a.res_bh_stride = (int64_t)c->geo.res_bh;
  a.res_len = cfg.residual_len;
  a.res_ntok = 0;
  *num_wg = n;
  return KVQ_OK;
}

// Stream-ordered copy of `bytes` host bytes to device address dst through the cache's pinned
// slots: the copy is a DMA from pinned memory, so enqueueing it does not wait for the device;
// the host waits only when every slot's previous copy is still queued.
int pinned_copy(kvq_cache *c, void *dst, const void *src, size_t bytes, hipStream_t s) {
  if (c->pinned.empty()) c->pinned.resize((size_t)std::min(256, std::max(8, 2 * c->cfg.num_layers)));
  auto &p = c->pinned[c->pinned_next];
  c->pinned_next = (c->pinned_next + 1) % c->pinned.size();
  if (p.pending) {
    if (int e = hip_check(hipEventSynchronize(p.ev), "pinned slot")) return e;
    p.pending = false;
  }
  if (p.cap < bytes) {
    if (p.host) (void)hipHostFree(p.host);
    p.host = nullptr;
    p.cap = 0;
    if (int e = hip_check(hipHostMalloc(&p.host, bytes, hipHostMallocDefault), "pinned slot")) return e;
    p.cap = bytes;
  }
  if (!p.ev)
    if (int e = hip_check(hipEventCreateWithFlags(&p.ev, hipEventDisableTiming), "pinned slot event")) return e;
  std::memcpy(p.host, src, bytes);
  if (int e = hip_check(hipMemcpyAsync(dst, p.host, bytes, hipMemcpyHostToDevice, s), "ragged tables")) return e;
  if (int e = hip_check(hipEventRecord(p.ev, s), "pinned slot event")) return e;
  p.pending = true;
  return KVQ_OK;
}

// the arguments of a decode call other than the workspace
int check_decode_args(const kvq_cache *c, const void *q, int32_t num_q_heads, float softmax_scale, const void *out) {
  const auto &cfg = c->cfg;
  if (num_q_heads < 1 || num_q_heads % cfg.num_kv_heads != 0)
    return fail(KVQ_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, cfg.num_kv_heads);
  const int G = num_q_heads / cfg.num_kv_heads;
  if (G > 16) return fail(KVQ_EINVAL, "query heads per kv head (%d) must be <= 16", G);
  if (!q || !out) return fail(KVQ_EINVAL, "q and out must be non-NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(KVQ_EINVAL, "q and out must be 16-byte aligned");
  if (!(softmax_scale > 0.0f) || softmax_scale > 3.0e38f) return fail(KVQ_EINVAL, "softmax_scale must be positive and finite");
  return KVQ_OK;
}

int check_decode(const kvq_cache *c, const void *q, int32_t num_q_heads, float softmax_scale, const void *out,
                 const void *workspace, size_t ws_bytes) {
  if (int e = check_decode_args(c, q, num_q_heads, softmax_scale, out)) return e;
  if (!workspace) return fail(KVQ_EINVAL, "workspace must be non-NULL");
  if (!aligned16(workspace)) return fail(KVQ_EINVAL, "workspace must be 16-byte aligned");
  if (ws_bytes < workspace_bound(c, num_q_heads))
    return fail(KVQ_ENOSPACE, "workspace %zu < required %zu", ws_bytes, workspace_bound(c, num_q_heads));
  return KVQ_OK;
}

// seq < 0: every sequence appends n_tokens
int check_append(const kvq_cache *c, int32_t layer, const void *k, const void *v, int64_t n_tokens, int seq = -1) {
  if (n_tokens < 0) return fail(KVQ_EINVAL, "n_tokens < 0");
  if (n_tokens == 0) return KVQ_OK;
  if (!k || !v) return fail(KVQ_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KVQ_EINVAL, "k and v must be 16-byte aligned");
  for (int b = seq < 0 ? 0 : seq; b < (seq < 0 ? c->cfg.batch : seq + 1); ++b) {
    const LayerState &st = c->st(layer, b);
    if (st.length + n_tokens > c->cfg.max_tokens)
      return fail(KVQ_ECAPACITY, "layer %d, sequence %d: %lld + %lld tokens exceeds max_tokens %lld", layer, b,
                  (long long)st.length, (long long)n_tokens, (long long)c->cfg.max_tokens);
  }
  return KVQ_OK;
}

// The decode launch of a checked call.  `pending` (may be null): the residual copy of the same
// call's append (tokens [src_tok0, +count) of k / v, n_src tokens each), done by the launch
// itself; for a ragged batch (`ragged`) one Op per sequence.
// Workspace layout of one call: [arrival counters and cursors][partials: part_stride slots per
// (b, h)][ragged tables].  A call needs counters_bytes + partials_bytes(part_stride) (+ the
// tables); ws_bytes is checked against that before anything is enqueued.
// pq_slot >= 0: the young slot of the token this launch quantizes itself (NVFP4 without a
// residual; `pending` is then null and k, v hold that one token).
int run_decode(kvq_cache *c, int32_t layer, const void *q, int32_t num_q_heads, float softmax_scale, void *out,
               int32_t out_fp32, void *workspace, size_t ws_bytes, const Op *pending, const void *k, const void *v,
               int64_t n_src, void *stream, bool ragged, int64_t pq_slot = -1) {
  const auto &cfg = c->cfg;
  const int G = num_q_heads / cfg.num_kv_heads;
  if (c->plan_only) return KVQ_OK;
  DecodeArgs a{};
  a.B = cfg.batch; a.H = cfg.num_kv_heads; a.G = G;
  a.res_item = -1;
  uint64_t *cursors = (uint64_t *)workspace + (size_t)cfg.batch * cfg.num_kv_heads * kCtrStride;
  int num_wg = 0, parts = 1;
  size_t tab_bytes = 0;
  if (ragged) {
    if (int e = plan_decode_ragged(c, layer, a, cursors, pending, &num_wg, &parts, &tab_bytes)) return e;
  } else {
    // a token this launch appends itself is attended to as a one-token residual
    num_wg = plan_decode(c, layer, a, cursors, pq_slot >= 0 ? 1 : 0);
    parts = a.items_total;
  }
  const size_t part_bytes = partials_bytes(c, num_q_heads, parts);
  const size_t pq_off = workspace_bound(c, num_q_heads) - pq_bytes(c);
  const size_t need = pq_slot >= 0 ? pq_off + pq_bytes(c) : counters_bytes(c) + part_bytes + tab_bytes;
  if (need > ws_bytes) return fail(KVQ_ENOSPACE, "this call needs %zu bytes of workspace, %zu given", need, ws_bytes);
  if (ragged) {
    uint8_t *dev_tab = (uint8_t *)workspace + counters_bytes(c) + part_bytes;
    if (int e = pinned_copy(c, dev_tab, c->rag_host.data(), tab_bytes, (hipStream_t)stream)) return e;
    a.rag = (const RagSeq *)dev_tab;
    a.rag_wg = (const uint32_t *)(dev_tab + rag_seq_bytes(c));
  }
  a.q = (const uint16_t *)q;
  a.out = out;
  a.out_fp32 = out_fp32 ? 1 : 0;
  a.counters = (uint64_t *)workspace;
  a.partials = (float *)((uint8_t *)workspace + counters_bytes(c));
  a.part_stride = parts;
  if (pq_slot >= 0) {
    a.pq_nvfp4 = 1;
    a.pq_arena = c->young(layer);
    a.pq_bh_stride = (int64_t)c->geo.young_bh;
    a.pq_slot = pq_slot;
    a.res_base = (const uint8_t *)workspace + pq_off;
    a.res_bh_stride = (int64_t)kPqResBytes;
    a.res_len = 16;
    a.res_ntok = 1;
    a.pend_k = (const uint16_t *)k; a.pend_v = (const uint16_t *)v;
    a.pend_src_ntok = n_src;
    a.pend_src_tok0 = 0;
  }
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.epoch = next_epoch();
  if (pending) {
    a.pend_k = (const uint16_t *)k; a.pend_v = (const uint16_t *)v;
    a.pend_src_ntok = n_src;
    if (!ragged) {
      a.pend_src_tok0 = pending->src_tok0;
      a.pend_count = (int)pending->count; a.pend_slot0 = (int)pending->dst_slot0;
    }
  }
  return hip_check(launch_decode(a, num_wg, (hipStream_t)stream), "decode");
}

// Append n tokens to every sequence of a layer whose sequences differ: one plan per sequence,
// all checked before anything is enqueued.  pend (may be null): a trailing residual copy of
// each plan is taken out into pend[b] (count 0: none) instead of being enqueued.
// The decode launch copies a step's new residual tokens itself when there are at most this
// many per (b, h): the workgroup that reads the residual makes the copy, so a long copy (the
// 128-token steps of the Llama-2 1K workload: 52.4 us per layer fused against 50.6 us with the
// append's copy launch, whose 128 x 2 workgroups share it) is left to the append.
constexpr int64_t kFuseCopyMax = 64;

int append_ragged(kvq_cache *c, int layer, const void *k, const void *v, int64_t n, hipStream_t s, Op *pend) {
  const int B = c->cfg.batch;
  std::vector<Plan> plans(B);
  for (int b = 0; b < B; ++b) {
    plans[b] = plan_append(c->cfg, c->st(layer, b), n);
    if (int e = check_capacity(c, plans[b])) return e;
  }
  const size_t per_seq = (size_t)c->cfg.num_kv_heads * (size_t)n * kHeadDim;   // fp16 values
  for (int b = 0; b < B; ++b) {
    Plan &p = plans[b];
    if (pend) {
      pend[b] = Op{Op::kResCopy, 0, 0, 0, 0};
      if (!p.ops.empty() && p.ops.back().kind == Op::kResCopy && p.ops.back().count <= kFuseCopyMax) {
        pend[b] = p.ops.back();
        p.ops.pop_back();
      }
    }
    const int e = run_plan(c, layer, p, (const uint16_t *)k + b * per_seq, (const uint16_t *)v + b * per_seq, n, s, b);
    if (e == KVQ_OK || e == KVQ_EHIP) c->st(layer, b) = p.after;
    if (e != KVQ_OK) return e;
  }
  return KVQ_OK;
}

int check_seq(const kvq_cache *c, int32_t layer, int32_t seq) {
  if (int e = check_cache(c, layer)) return e;
  if (seq < 0 || seq >= c->cfg.batch) return fail(KVQ_EINVAL, "sequence %d out of range [0, %d)", seq, c->cfg.batch);
  return KVQ_OK;
}

Plan plan_flush(const kvq_cache *c, const LayerState &st) {
  Plan p;
  p.after = st;
  add_quant(p, Op::kQuantResidual, 0, st.res, chunk_tier(c->cfg, st.length, st.length), st.length - st.res,
            c->cfg.demote_young != 0);
  p.after.res = 0;
  plan_demotions(c->cfg, p);
  return p;
}

}  // namespace

// ============================================================================== C ABI

extern "C" {

size_t kvq_cache_bytes(const kvq_config *cfg) {
  if (const char *e = check_config(cfg)) {
    fail(KVQ_EINVAL, "%s", e);
    return 0;
  }
  return geometry(cfg).layer_bytes * (size_t)cfg->num_layers;
}

int kvq_cache_create(const kvq_config *cfg, void *dev_buf, size_t dev_bytes, kvq_cache **out) {
  if (!out) return fail(KVQ_EINVAL, "out is NULL");
  *out = nullptr;
  if (const char *e = check_config(cfg)) return fail(KVQ_EINVAL, "%s", e);
  if (!dev_buf) return fail(KVQ_EINVAL, "dev_buf is NULL");
  if (((uintptr_t)dev_buf % kAlign) != 0) return fail(KVQ_EINVAL, "dev_buf must be 256-byte aligned");
  const size_t need = kvq_cache_bytes(cfg);
  if (dev_bytes < need) return fail(KVQ_ENOSPACE, "dev_bytes %zu < required %zu", dev_bytes, need);
  kvq_cache *c = new (std::nothrow) kvq_cache();
  if (!c) return fail(KVQ_EINVAL, "out of host memory");
  c->cfg = *cfg;
  if (c->cfg.old_after == 0) c->cfg.old_format = c->cfg.format;
  c->geo = geometry(cfg);
  c->base = (uint8_t *)dev_buf;
  c->bytes = dev_bytes;
  c->seqs.assign((size_t)cfg->num_layers * cfg->batch, LayerState{});
  *out = c;
  g_err.clear();
  return KVQ_OK;
}

int kvq_cache_destroy(kvq_cache *c) {
  delete c;
  return KVQ_OK;
}

int kvq_cache_reset(kvq_cache *c) {
  if (!c) return fail(KVQ_EINVAL, "cache handle is NULL");
  for (auto &l : c->seqs) l = LayerState{};
  return KVQ_OK;
}

int kvq_set_plan_only(kvq_cache *c, int32_t plan_only) {
  if (!c) return fail(KVQ_EINVAL, "cache handle is NULL");
  c->plan_only = plan_only ? 1 : 0;
  return KVQ_OK;
}

int kvq_set_deterministic(kvq_cache *c, int32_t on) {
  if (!c) return fail(KVQ_EINVAL, "cache handle is NULL");
  c->deterministic = on ? 1 : 0;
  return KVQ_OK;
}

size_t kvq_read_probe_sink_bytes(void) { return kProbeSinkBytes; }

int kvq_read_probe(const void *buf, size_t bytes, void *sink, size_t sink_bytes, void *stream) {
  if (!buf || !sink) return fail(KVQ_EINVAL, "buf and sink must be non-NULL");
  if ((uintptr_t)buf % 16 != 0) return fail(KVQ_EINVAL, "buf must be 16-byte aligned");
  if ((uintptr_t)sink % 4 != 0) return fail(KVQ_EINVAL, "sink must be 4-byte aligned");
  if (bytes == 0 || bytes % 16 != 0) return fail(KVQ_EINVAL, "bytes (%zu) must be a positive multiple of 16", bytes);
  if (sink_bytes < kProbeSinkBytes) return fail(KVQ_EINVAL, "sink holds %zu bytes, needs %zu", sink_bytes, kProbeSinkBytes);
  return hip_check(launch_read_probe(buf, bytes, (uint32_t *)sink, (hipStream_t)stream), "read probe");
}

int kvq_append(kvq_cache *c, int32_t layer, const void *k, const void *v, int64_t n_tokens, void *stream) {
  if (int e = check_cache(c, layer)) return e;
  if (int e = check_append(c, layer, k, v, n_tokens)) return e;
  if (n_tokens == 0) return KVQ_OK;
  if (!c->uniform(layer)) return append_ragged(c, layer, k, v, n_tokens, (hipStream_t)stream, nullptr);
  Plan p = plan_append(c->cfg, c->st(layer, 0), n_tokens);
  int e = run_plan(c, layer, p, k, v, n_tokens, (hipStream_t)stream);
  if (e == KVQ_OK || e == KVQ_EHIP)
    for (int b = 0; b < c->cfg.batch; ++b) c->st(layer, b) = p.after;
  return e;
}

int kvq_append_seq(kvq_cache *c, int32_t layer, int32_t seq, const void *k, const void *v, int64_t n_tokens,
                   void *stream) {
  if (int e = check_seq(c, layer, seq)) return e;
  if (int e = check_append(c, layer, k, v, n_tokens, seq)) return e;
  if (n_tokens == 0) return KVQ_OK;
  LayerState &st = c->st(layer, seq);
  Plan p = plan_append(c->cfg, st, n_tokens);
  int e = run_plan(c, layer, p, k, v, n_tokens, (hipStream_t)stream, seq);
  if (e == KVQ_OK || e == KVQ_EHIP) st = p.after;
  return e;
}

int kvq_flush_residual(kvq_cache *c, int32_t layer, void *stream) {
  if (int e = check_cache(c, layer)) return e;
  const int B = c->cfg.batch;
  for (int b = 0; b < B; ++b) {
    const int64_t r = c->st(layer, b).res;
    if (c->cfg.k_per_channel && r % kBlock != 0)
      return fail(KVQ_ESTATE, "per-channel K quantizes whole windows of 128 tokens; sequence %d's residual holds %lld", b,
                  (long long)r);
  }
  if (c->uniform(layer)) {
    if (c->st(layer, 0).res == 0) return KVQ_OK;
    Plan p = plan_flush(c, c->st(layer, 0));
    int e = run_plan(c, layer, p, nullptr, nullptr, 0, (hipStream_t)stream);
    if (e == KVQ_OK || e == KVQ_EHIP)
      for (int b = 0; b < B; ++b) c->st(layer, b) = p.after;
    return e;
  }
  std::vector<Plan> plans(B);
  for (int b = 0; b < B; ++b) {
    plans[b] = plan_flush(c, c->st(layer, b));
    if (int e = check_capacity(c, plans[b])) return e;
  }
  for (int b = 0; b < B; ++b) {
    if (c->st(layer, b).res == 0) continue;
    int e = run_plan(c, layer, plans[b], nullptr, nullptr, 0, (hipStream_t)stream, b);
    if (e == KVQ_OK || e == KVQ_EHIP) c->st(layer, b) = plans[b].after;
    if (e != KVQ_OK) return e;
  }
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(const kvq_cache *c, int32_t num_q_heads) {
  if (!c || num_q_heads < 1 || num_q_heads % c->cfg.num_kv_heads != 0) return 0;
  return workspace_bound(c, num_q_heads);
}

int kvq_decode_attn(kvq_cache *c, int32_t layer, const void *q, int32_t num_q_heads, float softmax_scale, void *out,
                    int32_t out_fp32, void *workspace, size_t ws_bytes, void *stream) {
  if (int e = check_cache(c, layer)) return e;
  if (int e = check_decode(c, q, num_q_heads, softmax_scale, out, workspace, ws_bytes)) return e;
  const bool ragged = !c->uniform(layer);
  if (!ragged && c->st(layer, 0).length == 0) return fail(KVQ_ESTATE, "layer %d is empty", layer);
  return run_decode(c, layer, q, num_q_heads, softmax_scale, out, out_fp32, workspace, ws_bytes, nullptr, nullptr,
                    nullptr, 0, stream, ragged);
}

int kvq_decode_attn_noalloc(kvq_cache *c, int32_t layer, const void *q, int32_t num_q_heads, float softmax_scale,
                            void *out, int32_t out_fp32, void *stream) {
  if (int e = check_cache(c, layer)) return e;
  if (int e = check_decode_args(c, q, num_q_heads, softmax_scale, out)) return e;
  if (!c->uniform(layer))
    return fail(KVQ_ESTATE, "layer %d: the sequences have different lengths; kvq_decode_attn_noalloc serves "
                "uniform batches only (kvq_decode_attn serves ragged ones)", layer);
  if (c->st(layer, 0).length == 0) return fail(KVQ_ESTATE, "layer %d is empty", layer);
  // the call's workspace (the same split as kvq_decode_attn's) must fit the scratch array
  DecodeArgs a{};
  a.B = c->cfg.batch; a.H = c->cfg.num_kv_heads; a.G = num_q_heads / c->cfg.num_kv_heads;
  a.res_item = -1;
  plan_decode(c, layer, a, nullptr);
  const size_t need = counters_bytes(c) + partials_bytes(c, num_q_heads, a.items_total);
  if (need > kNoAllocScratchBytes)
    return fail(KVQ_ENOSPACE, "this call needs %zu bytes of workspace; the no-alloc scratch holds %zu", need,
                kNoAllocScratchBytes);
  if (c->plan_only) return KVQ_OK;
  void *ws = nullptr;
  if (int e = hip_check(noalloc_scratch(&ws, (hipStream_t)stream), "no-alloc scratch")) return e;
  return run_decode(c, layer, q, num_q_heads, softmax_scale, out, out_fp32, ws, kNoAllocScratchBytes, nullptr, nullptr,
                    nullptr, 0, stream, false);
}

int kvq_append_decode_attn(kvq_cache *c, int32_t layer, const void *k, const void *v, int64_t n_tokens, const void *q,
                           int32_t num_q_heads, float softmax_scale, void *out, int32_t out_fp32, void *workspace,
                           size_t ws_bytes, void *stream) {
  if (int e = check_cache(c, layer)) return e;
  if (int e = check_append(c, layer, k, v, n_tokens)) return e;
  if (int e = check_decode(c, q, num_q_heads, softmax_scale, out, workspace, ws_bytes)) return e;
  if (!c->uniform(layer)) {
    std::vector<Op> pend(c->cfg.batch, Op{Op::kResCopy, 0, 0, 0, 0});
    if (n_tokens > 0)
      if (int e = append_ragged(c, layer, k, v, n_tokens, (hipStream_t)stream, pend.data())) return e;
    return run_decode(c, layer, q, num_q_heads, softmax_scale, out, out_fp32, workspace, ws_bytes, pend.data(), k, v,
                      n_tokens, stream, true);
  }
  LayerState st = c->st(layer, 0);
  if (st.length + n_tokens == 0) return fail(KVQ_ESTATE, "layer %d is empty", layer);
  Op pending{};
  bool has_pending = false;
  if (n_tokens == 1 && fuses_nvfp4_append(c->cfg)) {
    // NVFP4 without a residual: the decode launch quantizes the step's token itself
    Plan p = plan_append(c->cfg, st, n_tokens);
    if (int e = check_capacity(c, p)) return e;
    if (p.ops.size() != 1 || p.ops[0].kind != Op::kQuantInput || p.ops[0].tier != 0 || p.ops[0].count != 1)
      return fail(KVQ_ESTATE, "internal: unexpected append plan");
    for (int b = 0; b < c->cfg.batch; ++b) c->st(layer, b) = p.after;
    return run_decode(c, layer, q, num_q_heads, softmax_scale, out, out_fp32, workspace, ws_bytes, nullptr, k, v,
                      n_tokens, stream, false, p.ops[0].dst_slot0);
  }
  if (n_tokens > 0) {
    Plan p = plan_append(c->cfg, st, n_tokens);
    // a last copy into the residual moves into the decode launch (nothing else reads the residual)
    if (!p.ops.empty() && p.ops.back().kind == Op::kResCopy && p.ops.back().count <= kFuseCopyMax) {
      pending = p.ops.back();
      p.ops.pop_back();
      has_pending = true;
    }
    const int e = run_plan(c, layer, p, k, v, n_tokens, (hipStream_t)stream);
    if (e == KVQ_OK || e == KVQ_EHIP)
      for (int b = 0; b < c->cfg.batch; ++b) c->st(layer, b) = p.after;
    if (e != KVQ_OK) return e;
  }
  return run_decode(c, layer, q, num_q_heads, softmax_scale, out, out_fp32, workspace, ws_bytes,
                    has_pending ? &pending : nullptr, k, v, n_tokens, stream, false);
}

int kvq_seq_info(const kvq_cache *c, int32_t layer, int32_t seq, kvq_seq_info_t *info) {
  if (int e = check_seq(c, layer, seq)) return e;
  if (!info) return fail(KVQ_EINVAL, "info is NULL");
  const LayerState &st = c->st(layer, seq);
  info->length = st.length;
  info->residual = st.res;
  info->young_first_block = st.young_head;
  info->young_tokens = st.young - st.young_head * kBlock;
  info->old_tokens = st.old;
  return KVQ_OK;
}

int kvq_seq_len(const kvq_cache *c, int32_t layer, int64_t *total, int64_t *in_residual) {
  if (int e = check_cache(c, layer)) return e;
  if (!c->uniform(layer))
    return fail(KVQ_ESTATE, "layer %d: the sequences have different lengths (kvq_seq_info gives each)", layer);
  if (total) *total = c->st(layer, 0).length;
  if (in_residual) *in_residual = c->st(layer, 0).res;
  return KVQ_OK;
}

int kvq_layout(const kvq_cache *c, int32_t layer, int32_t region, size_t *offset, size_t *bytes, int64_t *tokens) {
  if (int e = check_cache(c, layer)) return e;
  const size_t bh = (size_t)c->cfg.batch * c->cfg.num_kv_heads;
  const size_t lb = (size_t)layer * c->geo.layer_bytes;
  const LayerState &st = c->st(layer, 0);
  size_t off, nb;
  int64_t t;
  switch (region) {
    case 0: off = lb + c->geo.off_res; nb = bh * c->geo.res_bh; t = st.res; break;
    case 1: off = lb + c->geo.off_young; nb = bh * c->geo.young_bh; t = st.young - st.young_head * kBlock; break;
    case 2: off = lb + c->geo.off_old; nb = bh * c->geo.old_bh; t = st.old; break;
    default: return fail(KVQ_EINVAL, "region %d is not 0, 1 or 2", region);
  }
  if (offset) *offset = off;
  if (bytes) *bytes = nb;
  if (tokens) *tokens = t;
  return KVQ_OK;
}

const char *kvq_last_error(void) { return g_err.c_str(); }

}  // extern "C"
