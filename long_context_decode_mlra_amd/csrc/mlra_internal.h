// Shared between the host-only parameter code and the HIP translation units.
// Holds no HIP types so that mlra_params.cpp builds as plain C++.
#pragma once

#include <cstddef>
#include <cstdint>

#include "mlra.h"

namespace mlra {

constexpr int kTile = MLRA_TILE_TOKENS;   // tokens per tile of the split-KV stream
constexpr int kHeadBlock = 32;            // query heads per MFMA column block
constexpr int kLatentTotal = 512;         // NB * d_latent of the whole-cache forms (MLRA-4, MLRA-2, MLA)
constexpr int kShardLatent = 128;         // d_latent of the one-latent-head shard form (NB = 1)
constexpr int kDRope = 64;
constexpr int kDV = 128;
constexpr int kCombBlock = 64;  // latent channels per combine workgroup

// Channels per block of the partials' per-block scale (bf16 caches): one combine workgroup's block.
constexpr int kPartBlock = kCombBlock;

// Latent channels per cached token: 512, or 128 for the shard form.
inline int latent_total(const mlra_decode_params& p) { return p.num_branches * p.d_latent; }

// The shard form: one latent head of 128 channels (one GPU's share of MLRA-4 split by latent head).
inline bool is_shard(const mlra_decode_params& p) { return p.num_branches == 1 && p.d_latent == kShardLatent; }

// Workspace of one decode call:
//   part_o  [slots][NB][h][d_latent]       unnormalised output of one split for one sequence
//                                          (slot = split + sequence): fp32 for fp32 caches; for bf16
//                                          caches fp16, each 64-channel block scaled by 2^-e
//   part_e  int32 [slots][NB][h][d_latent/64]  e of each 64-channel block (bf16 caches only): the
//                                          block's largest magnitude is below 2^(e+15)
//   part_ml fp32 [slots][NB][h][2]         (running max in log2 units, running sum)
//   prefix  int64 [B + 3]                  first tile of each sequence, then T (total tiles), T, G
//   ypart   fp32 [groups][h][NB*d_latent/kCombBlock][32][d_v]  projected channel blocks of up to
//                                          32 sequences
//   counters int32 [h][ceil(B / kCombMinSub)]  arrivals of the combine workgroups of one (query
//                                          head, run of sequences); the attention kernel clears them
// groups = ceil(B / 32).
struct WorkspaceLayout {
  int64_t slots = 0;
  size_t part_o_off = 0;
  size_t part_e_off = 0;
  size_t part_ml_off = 0;
  size_t prefix_off = 0;
  size_t ypart_off = 0;
  size_t counters_off = 0;
  int64_t n_counters = 0;
  size_t total = 0;
};

// Fewest sequences one combine workgroup takes (its runs hold 32, 16, 8 or 4 sequences).
constexpr int kCombMinSub = 4;

WorkspaceLayout workspace_layout(const mlra_decode_params& p, int32_t num_splits);

// Records a thread-local message and returns `code`.
int set_error(int code, const char* fmt, ...);
void clear_error();

int head_blocks(int num_heads);

bool aligned16(const void* ptr);

// GQA comparator workspace: part_o fp32 [slots][H_q][128], part_ml fp32 [slots][H_q][2],
// prefix int64 [B + 3]; slots = G + B.
struct GqaLayout {
  int64_t slots = 0;
  size_t part_o_off = 0;
  size_t part_ml_off = 0;
  size_t prefix_off = 0;
  size_t total = 0;
};
constexpr int kGqaHeadDim = 128;
constexpr int kGqaMaxGroup = 16;
GqaLayout gqa_layout(const mlra_gqa_params& p, int32_t num_splits);
int gqa_prepare(const mlra_gqa_params* p, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                int32_t* G, GqaLayout* lay);

// Validates p, resolves the split count G and the workspace layout, and checks the
// workspace pointer and size (B = 0 needs neither seqlens nor a workspace).
int prepare(const mlra_decode_params* p, const int32_t* seqlens, void* workspace, size_t workspace_bytes,
            int32_t* G, WorkspaceLayout* lay);

}  // namespace mlra
