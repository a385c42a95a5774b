// Host-only part of the C ABI: parameter validation, workspace sizing, error text.
// No HIP calls here, so every error path can be driven from a machine without a GPU.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "mlra_internal.h"

namespace mlra {

namespace {
thread_local char g_error[512] = "";
}

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

int head_blocks(int num_heads) { return (num_heads + kHeadBlock - 1) / kHeadBlock; }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WorkspaceLayout workspace_layout(const mlra_decode_params& p, int32_t num_splits) {
  WorkspaceLayout w;
  // Split g writes at most one partial per sequence it touches, at slot g + b; g + b < G + B.
  w.slots = int64_t(num_splits) + int64_t(p.batch);
  // bf16 caches keep fp16 partials with one int32 exponent per 64-channel block; fp32 caches fp32.
  const bool half = p.dtype == MLRA_BF16;
  const size_t per_slot_o = size_t(p.num_heads) * latent_total(p) * (half ? 2 : sizeof(float));
  const size_t per_slot_e = half ? size_t(p.num_heads) * (latent_total(p) / kPartBlock) * sizeof(int32_t) : 0;
  const size_t per_slot_ml = size_t(p.num_branches) * size_t(p.num_heads) * 2 * sizeof(float);
  w.part_o_off = 0;
  w.part_e_off = align256(size_t(w.slots) * per_slot_o);
  w.part_ml_off = align256(w.part_e_off + size_t(w.slots) * per_slot_e);
  w.prefix_off = align256(w.part_ml_off + size_t(w.slots) * per_slot_ml);
  const size_t groups = (size_t(p.batch) + 31) / 32;
  w.ypart_off = align256(w.prefix_off + (size_t(p.batch) + 3) * sizeof(int64_t));
  w.counters_off = align256(w.ypart_off + groups * size_t(p.num_heads) * (latent_total(p) / kCombBlock) * 32 *
                                              kDV * sizeof(float));
  w.n_counters = int64_t(p.num_heads) * ((int64_t(p.batch) + kCombMinSub - 1) / kCombMinSub);
  w.total = align256(w.counters_off + size_t(w.n_counters) * sizeof(int32_t));
  return w;
}


bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

int prepare(const mlra_decode_params* p, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
            int32_t* G, WorkspaceLayout* lay) {
  int rc = mlra_check_params(p);
  if (rc) return rc;
  rc = mlra_decode_num_splits(p, G);
  if (rc) return rc;
  *lay = workspace_layout(*p, *G);
  if (lay->n_counters > INT32_MAX)
    return set_error(MLRA_ERR_SHAPE, "batch %d with %d heads is past what the combine counts", p->batch,
                     p->num_heads);
  if (p->batch == 0) return MLRA_OK;
  if (!seqlens) return set_error(MLRA_ERR_NULL, "seqlens is NULL");
  if (!workspace) return set_error(MLRA_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return set_error(MLRA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < lay->total)
    return set_error(MLRA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, lay->total);
  return MLRA_OK;
}

GqaLayout gqa_layout(const mlra_gqa_params& p, int32_t num_splits) {
  GqaLayout w;
  w.slots = int64_t(num_splits) + int64_t(p.batch);
  w.part_o_off = 0;
  w.part_ml_off = align256(size_t(w.slots) * size_t(p.num_q_heads) * kGqaHeadDim * sizeof(float));
  w.prefix_off = align256(w.part_ml_off + size_t(w.slots) * size_t(p.num_q_heads) * 2 * sizeof(float));
  w.total = align256(w.prefix_off + (size_t(p.batch) + 3) * sizeof(int64_t));
  return w;
}

int gqa_prepare(const mlra_gqa_params* p, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                int32_t* G, GqaLayout* lay) {
  int rc = mlra_gqa_check_params(p);
  if (rc) return rc;
  rc = mlra_gqa_num_splits(p, G);
  if (rc) return rc;
  *lay = gqa_layout(*p, *G);
  if (p->batch == 0) return MLRA_OK;
  if (!seqlens) return set_error(MLRA_ERR_NULL, "seqlens is NULL");
  if (!workspace) return set_error(MLRA_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return set_error(MLRA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < lay->total)
    return set_error(MLRA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, lay->total);
  return MLRA_OK;
}

}  // namespace mlra

using namespace mlra;

extern "C" int mlra_abi_version(void) { return MLRA_ABI_VERSION; }

extern "C" const char* mlra_last_error(void) { return g_error; }

extern "C" int mlra_check_params(const mlra_decode_params* p) {
  if (!p) return set_error(MLRA_ERR_NULL, "params pointer is NULL");
  if (p->reserved != 0) return set_error(MLRA_ERR_SHAPE, "reserved field must be 0 (got %d)", p->reserved);
  if (p->batch < 0) return set_error(MLRA_ERR_SHAPE, "batch must be >= 0 (got %d)", p->batch);
  if (p->num_heads < 1 || p->num_heads > MLRA_MAX_HEADS)
    return set_error(MLRA_ERR_UNSUPPORTED, "num_heads must be in [1, %d] (got %d)", MLRA_MAX_HEADS, p->num_heads);
  if (p->num_branches != 1 && p->num_branches != 2 && p->num_branches != 4)
    return set_error(MLRA_ERR_UNSUPPORTED, "num_branches must be 1, 2 or 4 (got %d)", p->num_branches);
  if (p->d_latent * p->num_branches != kLatentTotal && !is_shard(*p))
    return set_error(MLRA_ERR_UNSUPPORTED, "d_latent must be 512 / num_branches = %d, or 128 with one branch (got %d)",
                     kLatentTotal / p->num_branches, p->d_latent);
  if (is_shard(*p) && p->dtype != MLRA_BF16)
    return set_error(MLRA_ERR_UNSUPPORTED, "the one-latent-head shard form (d_latent 128) takes bf16 only");
  if (is_shard(*p) && p->num_heads > kHeadBlock)
    return set_error(MLRA_ERR_UNSUPPORTED, "the one-latent-head shard form takes at most %d query heads (got %d)",
                     kHeadBlock, p->num_heads);
  if (p->d_rope != kDRope) return set_error(MLRA_ERR_UNSUPPORTED, "d_rope must be 64 (got %d)", p->d_rope);
  if (p->d_v != kDV) return set_error(MLRA_ERR_UNSUPPORTED, "d_v must be 128 (got %d)", p->d_v);
  if (p->dtype != MLRA_BF16 && p->dtype != MLRA_F32)
    return set_error(MLRA_ERR_UNSUPPORTED, "dtype must be MLRA_BF16 or MLRA_F32 (got %d)", p->dtype);
  if (p->max_seqlen < 0) return set_error(MLRA_ERR_SHAPE, "max_seqlen must be >= 0 (got %d)", p->max_seqlen);
  if (p->page_size < 0) return set_error(MLRA_ERR_SHAPE, "page_size must be >= 0 (got %d)", p->page_size);
  if (p->page_size > 0) {
    if (p->page_size % kTile != 0)
      return set_error(MLRA_ERR_UNSUPPORTED, "page_size must be a multiple of %d (got %d)", kTile, p->page_size);
    const int64_t need = (int64_t(p->max_seqlen) + p->page_size - 1) / p->page_size;
    if (p->max_pages_per_seq < need)
      return set_error(MLRA_ERR_SHAPE, "max_pages_per_seq %d < ceil(max_seqlen / page_size) = %lld",
                       p->max_pages_per_seq, (long long)need);
  }
  if (p->num_splits < 0) return set_error(MLRA_ERR_SHAPE, "num_splits must be >= 0 (got %d)", p->num_splits);
  const int64_t esz = p->dtype == MLRA_BF16 ? 2 : 4;
  const int64_t row = int64_t(p->num_branches) * p->d_latent;
  if (p->q_stride_h < row || p->q_stride_b < 0 || p->qr_stride_h < p->d_rope || p->qr_stride_b < 0)
    return set_error(MLRA_ERR_SHAPE, "query strides too small (q_stride_h %lld, qr_stride_h %lld)",
                     (long long)p->q_stride_h, (long long)p->qr_stride_h);
  if (p->lat_stride_tok < row || p->rope_stride_tok < p->d_rope)
    return set_error(MLRA_ERR_SHAPE, "cache row strides too small (lat %lld, rope %lld)",
                     (long long)p->lat_stride_tok, (long long)p->rope_stride_tok);
  // Rows of one 32-token tile are addressed with 32-bit offsets.
  if (p->lat_stride_tok * esz * kTile > (int64_t(1) << 30) || p->rope_stride_tok * esz * kTile > (int64_t(1) << 30))
    return set_error(MLRA_ERR_SHAPE, "cache row stride too large");
  const int64_t strides[6] = {p->q_stride_b, p->q_stride_h, p->qr_stride_b, p->qr_stride_h,
                              p->lat_stride_tok, p->rope_stride_tok};
  for (int k = 0; k < 6; ++k)
    if ((strides[k] * esz) % 16 != 0)
      return set_error(MLRA_ERR_ALIGN, "stride #%d (%lld elements) is not a multiple of 16 bytes", k,
                       (long long)strides[k]);
  if (!(std::isfinite(p->sm_scale) && p->sm_scale > 0.f))
    return set_error(MLRA_ERR_SHAPE, "sm_scale must be finite and > 0");
  if (!std::isfinite(p->out_scale)) return set_error(MLRA_ERR_SHAPE, "out_scale must be finite");
  return MLRA_OK;
}

extern "C" int mlra_gqa_check_params(const mlra_gqa_params* p) {
  if (!p) return set_error(MLRA_ERR_NULL, "params pointer is NULL");
  if (p->reserved != 0 || p->reserved_f != 0.f) return set_error(MLRA_ERR_SHAPE, "reserved fields must be 0");
  if (p->batch < 0) return set_error(MLRA_ERR_SHAPE, "batch must be >= 0 (got %d)", p->batch);
  if (p->num_kv_heads < 1 || p->num_q_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
    return set_error(MLRA_ERR_SHAPE, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                     p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads / p->num_kv_heads > kGqaMaxGroup)
    return set_error(MLRA_ERR_UNSUPPORTED, "at most %d query heads per KV head (got %d)", kGqaMaxGroup,
                     p->num_q_heads / p->num_kv_heads);
  if (p->head_dim != kGqaHeadDim)
    return set_error(MLRA_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", kGqaHeadDim, p->head_dim);
  if (p->dtype != MLRA_BF16) return set_error(MLRA_ERR_UNSUPPORTED, "the GQA decode takes bf16 only");
  if (p->max_seqlen < 0) return set_error(MLRA_ERR_SHAPE, "max_seqlen must be >= 0 (got %d)", p->max_seqlen);
  if (p->page_size < 0) return set_error(MLRA_ERR_SHAPE, "page_size must be >= 0 (got %d)", p->page_size);
  if (p->page_size > 0) {
    if (p->page_size % kTile != 0)
      return set_error(MLRA_ERR_UNSUPPORTED, "page_size must be a multiple of %d (got %d)", kTile, p->page_size);
    const int64_t need = (int64_t(p->max_seqlen) + p->page_size - 1) / p->page_size;
    if (p->max_pages_per_seq < need)
      return set_error(MLRA_ERR_SHAPE, "max_pages_per_seq %d < ceil(max_seqlen / page_size) = %lld",
                       p->max_pages_per_seq, (long long)need);
  }
  if (p->num_splits < 0) return set_error(MLRA_ERR_SHAPE, "num_splits must be >= 0 (got %d)", p->num_splits);
  if (p->q_stride_h < kGqaHeadDim || p->q_stride_b < 0)
    return set_error(MLRA_ERR_SHAPE, "query strides too small (q_stride_h %lld)", (long long)p->q_stride_h);
  if (p->k_stride_tok < 0 || p->k_stride_head < 0 || p->v_stride_tok < 0 || p->v_stride_head < 0)
    return set_error(MLRA_ERR_SHAPE, "cache strides must be >= 0");
  // Rows of one 32-token tile are addressed with 32-bit offsets.
  if (p->k_stride_tok * 2 * kTile > (int64_t(1) << 30) || p->v_stride_tok * 2 * kTile > (int64_t(1) << 30))
    return set_error(MLRA_ERR_SHAPE, "cache row stride too large");
  const int64_t strides[6] = {p->q_stride_b, p->q_stride_h, p->k_stride_tok, p->k_stride_head,
                              p->v_stride_tok, p->v_stride_head};
  for (int k = 0; k < 6; ++k)
    if ((strides[k] * 2) % 16 != 0)
      return set_error(MLRA_ERR_ALIGN, "stride #%d (%lld elements) is not a multiple of 16 bytes", k,
                       (long long)strides[k]);
  if (!(std::isfinite(p->sm_scale) && p->sm_scale > 0.f))
    return set_error(MLRA_ERR_SHAPE, "sm_scale must be finite and > 0");
  return MLRA_OK;
}
