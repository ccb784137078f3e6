// Internal declarations shared by the C-ABI layer (api.cpp) and the kernel
// launchers (*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace ts {

// Launch parameters of the split-KV attention kernels (verification and draft).
struct AttnParams {
  const uint16_t* q;     // [Hq][T][d] bf16
  const uint16_t* k;     // cache, element (g, j, c) at g*s_head + j*s_pos + c
  const uint16_t* v;
  float* out;            // [Hq][T][d] fp32
  uint16_t* part_acc;    // [n_split][Hkv][M][d] f16 bits: each split's normalised partial output
  float* part_ml;        // [n_split][Hkv][M][2] running max (raw score units) and sum
  int64_t s_head, s_pos;
  int32_t n_ctx, T, Hq, Hkv, d;
  int32_t M;             // rows per KV head = (Hq/Hkv) * T
  int32_t n_split;       // effective number of chunks per KV head
  int32_t rows_per_split;  // cache rows per split (a multiple of the kernel's K/V tile)
  float scale_log2e;     // softmax scale * log2(e)
  float* scores;         // [Hkv][n_ctx] grouped scores of the committed rows, or null
  uint64_t anc[256];     // words 2i, 2i+1: bit a set <=> tree node a is i or an ancestor of i
};

// Automatic split count: a pure function of the shapes (so the workspace
// query needs no device), aimed at one resident workgroup per compute unit.
int attn_auto_split(int32_t rows_total, int32_t T, int32_t Hq, int32_t Hkv, int32_t d);
// Effective split count and cache rows per split for a requested count.
void attn_split_plan(int32_t rows_total, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                     int32_t n_split_req, int32_t* n_split_eff, int32_t* rows_per_split);
size_t attn_workspace_bytes(int32_t rows_total, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                            int32_t n_split_req);
hipError_t launch_attention(const AttnParams& p, hipStream_t stream);
// Workgroups along the query rows of one KV head (1: every row of the group in
// one workgroup, which the fused score output needs).
int attn_row_blocks(int32_t T, int32_t Hq, int32_t Hkv);

// Partial-KV selection.
struct SelectParams {
  const uint16_t* q;     // [Hq][T][d]
  const uint16_t* k;
  const uint16_t* v;
  int64_t s_head, s_pos;
  int32_t n_ctx, T, Hq, Hkv, d;
  int32_t n_sink, budget, n_recent;
  int32_t cand_lo, cand_hi;   // candidate rows [cand_lo, cand_hi)
  int32_t b_eff;              // min(budget, |C|)
  int32_t n_part;
  int32_t* sel_idx;           // [Hkv][budget]
  uint16_t* k_part;
  uint16_t* v_part;
  int64_t sp_head, sp_pos;
  float* scores;              // [Hkv][n_ctx] (user buffer or workspace; read-only when scores_given)
  int32_t scores_given;       // 1: scores come from the caller (no query pass)
  int32_t* sel_ws;            // workspace of the selection passes (histograms, cut-bin lists)
};
size_t select_workspace_bytes(int32_t n_ctx, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                              int32_t budget);
// Workspace of the selection passes alone (scores given by the caller).
size_t select_passes_workspace_bytes(int32_t n_ctx, int32_t Hkv);
hipError_t launch_select(const SelectParams& p, hipStream_t stream);

// Penalty / sampling pass.
struct PenaltyParams {
  const float* logits;
  float* logits_out;
  const int32_t* window;
  int64_t window_stride;
  int32_t rows, V, W;
  float penalty, inv_temperature, temperature, top_p, min_p;
  int32_t eta_mode;            // 1: eta-sampling replaces top-p and min-p
  float eta_eps, eta_alpha;
  uint8_t* keep;
  float* probs;
  const float* u;
  int32_t* token;
  void* ws;
};
size_t penalty_workspace_bytes(int32_t rows, int32_t V);
hipError_t launch_penalty(const PenaltyParams& p, hipStream_t stream);

// Tree acceptance and KV commit.
struct AcceptParams {
  const int32_t* node_token;   // [T]
  const int32_t* target;       // [T]
  int32_t* result;             // [T + 2]: n accepted, next token, path, -1 padding
  int32_t T;
  int32_t parent[128];
  uint64_t anc[256];           // ancestor-or-self masks, two words per node
};
hipError_t launch_accept(const AcceptParams& p, hipStream_t stream);

struct CommitParams {
  const int32_t* result;       // as written by the acceptance kernel
  uint16_t* k;                 // element (layer, g, j, c) at layer*s_layer + g*s_head + j*s_pos + c
  uint16_t* v;
  int64_t s_layer, s_head, s_pos;
  int32_t layers, Hkv, d, n_ctx, T;
  uint16_t* k_part;            // or null
  uint16_t* v_part;
  int64_t sp_layer, sp_head, sp_pos;
  int32_t n_part;
};
hipError_t launch_commit(const CommitParams& p, hipStream_t stream);

// N-gram retrieval and draft tree.
constexpr int NG_MAX_WINDOW = 4096;   // window tokens held in LDS
struct NgramParams {
  const int32_t* window;       // [W]
  const int32_t* head;         // [levels][3] or null
  int32_t* parent;             // [T_max]
  int32_t* node_token;         // [T_max]
  int32_t* info;               // [4]: T, chains placed, distinct continuations, occurrences
  uint64_t seed;
  int32_t W, k, levels, T_max;
};
hipError_t launch_ngram_tree(const NgramParams& p, hipStream_t stream);

}  // namespace ts
