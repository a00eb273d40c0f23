// Kernel argument blocks and host launchers of the EAGLE HIP library.
#pragma once
#include "common.h"

namespace eagle {

// ---------------------------------------------------------------- GEMM
// P[z][m][n] = sum_{k in split z} X[m][k] * W[n][k]
// X row m = xs[0] for k < ksplit_x, else xs[1] (column k - ksplit_x);
// W = rows [0, nseg1) of w[0], [nseg1, nseg2) of w[1], [nseg2, N) of w[2].
struct GemmArgs {
  RowSrc xs[2];
  int ksplit_x;
  int M, N, K;
  const void* w[3];
  int nseg1, nseg2;
  float* P;
  int kps;
  // SwiGLU epilogue of the tiled big GEMM (one split): W = [gate; up] with
  // pair_F rows each; the tile pairs gate and up rows and writes
  // act[m][j] = silu(gate_j) * up_j in bf16 instead of P (rows of pair_F)
  int pair_F = 0;
  void* act = nullptr;
  // row epilogue of the tiled big GEMM (one split, 256-row and 256-column
  // tiles, N % 256 == 0): y = acc + res row; out = bf16(y), out_g =
  // bf16(y * gain), stats[m][n / 256] = (sum y, sum y^2) over the tile's 256
  // columns, the layout the folded-RMSNorm consumers read
  int row_epi = 0;
  RowSrc res = RowSrc{nullptr, nullptr, 0, 0};
  void* out = nullptr;
  void* out_g = nullptr;
  const void* gain = nullptr;
  float* stats = nullptr;
  // LM-head epilogue of the 64-K-stage tiled GEMM (65..80 rows, one split,
  // top_k <= kLmFusedTopK): each persistent workgroup keeps, per row, the
  // running max and sum of exp(s * (logit - max)) and the top_k (logit desc,
  // id asc) over its tiles, and writes them once as its part p (the layout
  // of the tile partials: part_max/part_sum[p][m], part_val/part_id[p][m][k],
  // p < lm_fused_parts); P, if set, also receives the fp32 logits
  int lm_top_k = 0;
  float lm_inv_temp = 1.f;
  float* lm_max = nullptr;
  float* lm_sum = nullptr;
  float* lm_val = nullptr;
  int* lm_id = nullptr;
};
constexpr int kLmFusedTopK = 16;
struct GemmShape {
  int MB, NB, mtiles, ntiles, S, kps;
  int BN = 256;        // direct-to-LDS kernel (NB == 2): tile width (columns of W)
  int direct;          // 1: barrier-free streaming (M <= 16), 2: MFMA-tiled big GEMM,
                       // 3: streaming with LDS-shared activation rows (17..32)
};
// plan_gemm picks the kernel: direct streaming (M <= 16), activation-sharing
// streaming (17..32), LDS-staged
// streaming (M < 64 or unsupported shape) or the MFMA-tiled big GEMM.
// The A operand's split point (ksplit_x) must be a multiple of 64.
GemmShape plan_gemm(int dtype, int M, int N, int K);
void launch_gemm(int dtype, GemmArgs a, const GemmShape& s, hipStream_t st);
bool big_gemm_ok(int dtype, int M, int N, int K);
// 17..63 rows on the 64-K-stage tiled GEMM (8 x 1 waves over the live 16-row
// blocks): the projections' plan when this holds (bf16, K % 64 == 0)
bool wide_rows_ok(int dtype, int M, int N, int K);
// whether launch_gemm_big takes the row epilogue (row_epi) for this shape
bool big_rowepi_ok(int dtype, int M, int N, int K);
GemmShape plan_gemm_big(int M, int N, int K);
void launch_gemm_big(GemmArgs a, const GemmShape& s, hipStream_t st);
// the big-GEMM plan uses the direct-to-LDS kernel with one split, so the
// SwiGLU epilogue can be fused (gate|up of F rows each, F % 128 == 0)
bool big_swiglu_ok(int dtype, int M, int F, int K);
// whether the LM head (M x V logits over K) takes the fused LM-head epilogue,
// and the number of parts it writes (one per workgroup, at most 256)
bool lm_fused_ok(int dtype, int M, int V, int K, int top_k);
int lm_fused_parts(int M, int V, int K);

// y = sum_s P + src1 + src2 ; out / out_scatter = y ; out_norm = Norm(y)
struct ReduceArgs {
  const float* P;
  int S, M, N;
  RowSrc src1, src2;
  void* out;
  RowSrc out_scatter;  // base/idx/stride used for writing (base non-null to enable)
  void* out_norm;
  const void* gain;
  const void* bias;
  int layer_norm;
  float eps;
  float* y32;          // [M][N] fp32 scratch (needed when out_norm is set)
  float* stats;        // [M][ceil(N/256)][2] scratch (needed when out_norm is set)
  int keep_stats;      // write y32 / stats even without out_norm (a later kernel normalises)
  void* out_g;         // optional: y * gain (T), the operand of a folded RMSNorm
};
void launch_reduce_rows(int dtype, const ReduceArgs& a, hipStream_t st);

// Row-complete streaming GEMM for M <= 16 rows: each workgroup owns one
// 16-row block of W over the whole K (its waves split K and reduce through
// LDS), so the row epilogue runs in the same kernel.  RMSNorm is folded
// through the projection: the producer stores bf16(y * g) and per-block sums
// of y^2, the consumer scales its result rows by rstd.
enum { EP_STORE = 0, EP_ROPE = 1, EP_SWIGLU = 2, EP_GELU = 3 };
struct RowsArgs {
  GemmArgs g;              // xs / ksplit_x (A operand), M, N, K, w / nseg (B operand rows)
  const float* xstats;     // optional: [M][xnblk] (sum, sum of squares) of the rows the
  int xnblk;               //   A operand was formed from; result rows scaled by rstd
  float eps;
  // EP_STORE: y = acc + res ; out / scatter = y, out_g = y * gain (T), stats [M][N/16]
  RowSrc res;
  void* out;
  RowSrc scatter;
  void* out_g;
  const void* gain;
  float* stats;
  // EP_SWIGLU: act [M][act_F] = silu(gate) * up, gate rows [0, F), up rows [F, 2F)
  // EP_GELU: act [M][N] = gelu(acc)
  int act_F;
  // EP_ROPE: fused q|k|v columns; rotate q and k heads, scatter k / v rows
  int Hq, Hkv, hd;
  float theta;
  const int32_t* pos;
  void* q;
  void* k;
  void* v;
  const int32_t* kv_idx;
};
// shapes the row-complete path takes (M <= 16, N % 16 == 0, K % 32 == 0)
bool rows_gemm_ok(int M, int N, int K);
void launch_gemm_rows(int dtype, int ep, const RowsArgs& a, hipStream_t st);

struct QkvArgs {
  const float* P = nullptr;
  int S = 0, M = 0, Hq = 0, Hkv = 0, hd = 0;
  float theta = 0.f;
  const int32_t* pos = nullptr;    // per-row position, or null: packed context rows
  // packed context rows: row m belongs to request b with cu_row[b] <= m <
  // cu_row[b+1].  n_new null: its position is m - cu_row[b] and K/V go to row
  // m.  n_new set (rows are each request's newest positions): the position is
  // n[b] - n_new[b] + (m - cu_row[b]) and K/V go to row cu_n[b] + position;
  // rows whose position falls outside [0, n[b]) or past total_rows are skipped.
  const int32_t* cu_row = nullptr;
  const int32_t* n = nullptr;
  const int32_t* n_new = nullptr;
  const int32_t* cu_n = nullptr;
  int64_t total_rows = 0;
  int B = 0;
  void* q = nullptr;               // [M][Hq][hd] (may be null when Hq == 0)
  void* k = nullptr;               // rows kv_idx[m] (or as above) of [..][Hkv][hd]
  void* v = nullptr;
  const int32_t* kv_idx = nullptr;
  // RMSNorm folded through the projection: the A operand was y * g and xstats
  // [M][xnblk] holds the (sum, sum of squares) of y per 256-column block
  // (xN columns); the projected rows are scaled by rstd = 1 / sqrt(mean(y^2) + eps)
  const float* xstats = nullptr;
  int xnblk = 0, xN = 0;
  float eps = 0.f;
};
void launch_epi_qkv(int dtype, const QkvArgs& a, hipStream_t st);

struct ActArgs {
  const float* P;
  int S, M, F;
  int swiglu;
  void* out;            // [M][F]
  // folded RMSNorm of the A operand, as in QkvArgs (four-column kernel only)
  const float* xstats = nullptr;
  int xnblk = 0, xN = 0;
  float eps = 0.f;
};
void launch_epi_act(int dtype, const ActArgs& a, hipStream_t st);
// whether launch_epi_act takes the four-column kernel, the one that applies a
// folded RMSNorm's row scale
bool epi_act4_ok(int M, int F, const void* P, const void* out);

// ---------------------------------------------------------------- attention
// Rows of request b are m = b*W .. b*W+W-1; query row (m, head h) reads kv
// head h / G.  Keys: the request's context [0, n_b) split into pieces of
// `split_len`, plus (last split) up to 64 extra keys (tree slots) gated per
// row by a 64-bit mask.
struct AttnArgs {
  const void* q;          // [M][Hq][hd]
  int B, W, Hq, Hkv, hd;
  const int32_t* n;       // [B]
  const int32_t* cu_n;    // [B+1]
  const void* k_ctx;      // [total][Hkv][hd]
  const void* v_ctx;
  const void* k_ex;       // [B*64][Hkv][hd]
  const void* v_ex;
  const uint64_t* mask;   // [M]
  int split_len;          // multiple of 64
  int nsplit;             // context splits (the extra split is index nsplit)
  int rowgroups;          // ceil(W*G / 64)
  float scale_log2;       // log2(e) / sqrt(hd)
  float* part_o;          // [nsplit+1][M][Hq][hd]
  float* part_ml;         // [nsplit+1][M][Hq][2] (running max in log2 units, sum)
};
void launch_attention(int dtype, const AttnArgs& a, hipStream_t st);

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  int nparts, M, Hq, hd;
  void* out;              // [M][Hq*hd]
};
void launch_attn_combine(int dtype, const CombineArgs& a, hipStream_t st);

// ---------------------------------------------------------------- LM head
struct LmArgs {
  RowSrc x;               // [M][d]
  int M, K, V;
  const void* w;          // [V][K]
  int top_k;
  float inv_temp;
  float* logits;          // optional [M][V]
  float* part_max;        // [ntiles][M]
  float* part_sum;        // [ntiles][M]
  int* part_id;           // [ntiles][M][top_k]
  float* part_val;        // [ntiles][M][top_k]
  // sampled drafting (Gumbel-top-k): the top-k are taken by the key
  // s * logit + G, G = -log(-log(u)), u from Philox4x32-10 (key = seed,
  // counter = (id / 4, row key, 0, 0)); row key = (m / rows_per_req) * 1024 +
  // row_node[m].  part_val then holds keys and part_logit the logits.
  int gumbel = 0;
  uint32_t seed_lo = 0, seed_hi = 0;
  const int32_t* row_node = nullptr;
  int rows_per_req = 1;
  float* part_logit = nullptr;  // [ntiles][M][top_k]
};
struct LmShape {
  int MB, mtiles, ntiles, cols;
};
LmShape plan_lmhead(int dtype, int M, int V);
void launch_lmhead(int dtype, const LmArgs& a, const LmShape& s, hipStream_t st);
// large M: logits from the MFMA-tiled GEMM, then per-(row, 2048-column tile) partials
int logits_tiles(int V);
void launch_logits_partials(const LmArgs& a, const float* logits, hipStream_t st);

struct MergeArgs {
  const float* part_max;
  const float* part_sum;
  const int* part_id;
  const float* part_val;
  int ntiles, M, top_k;
  float inv_temp;
  int* topk_id;           // [M][top_k]
  float* topk_conf;       // [M][top_k]
  float* lse;             // [M]
  int vocab;              // ids are clamped to [0, vocab)
  const float* part_logit = nullptr;  // Gumbel-top-k: candidates' logits (part_val = keys)
};
void launch_topk_merge(const MergeArgs& a, hipStream_t st);

// ---------------------------------------------------------------- tree
constexpr int kVerifySplits = 16;   // workgroups per target-logit row

struct TreeDev {          // device pointers into eagle_tree.state
  int32_t *pool_tok, *pool_parent, *pool_depth, *pool_slot;
  float *pool_conf, *pool_value;
  int32_t *pool_count, *slot_count, *root_pos;
  uint64_t* slot_mask;
  int32_t *row_node, *row_tok, *row_pos, *row_slot, *row_pidx;
  uint64_t* row_mask;
  int32_t* topk_id;
  float* topk_conf;
  float* lse;
  int32_t *f_node, *f_tok, *f_parent, *f_depth, *f_pos;
  uint64_t* f_mask;
  int32_t* f_count;
  int32_t* choice;
  float2* choice_part;    // [B][64][kVerifySplits] (max value, index as float bits)
  int32_t* status;        // [B] 0 = consistent, else EAGLE_TREE_STATE_BAD
  int pool_cap, max_rows, positions;
};

struct RowsDev {          // one half of the double-buffered step rows
  int32_t *node, *tok, *pos, *slot, *pidx;
  uint64_t* mask;
};

struct StaticPlan {       // children created by one static / chain step
  int nchild;             // per request
  int nnext;              // rows of the next step per request
  uint8_t row[64], rank[64], expand[64];
};

void launch_tree_init(const TreeDev& t, int B, int eagle3, int vocab, const int32_t* root_tok,
                      const int32_t* n, const int32_t* cu_n, hipStream_t st);
void launch_tree_expand(const TreeDev& t, const RowsDev& next, int B, int kind, int step,
                        int gamma, int rows, int top_k, int top_m, int final_step,
                        const StaticPlan& plan, hipStream_t st);
void launch_verify(const TreeDev& t, int B, const void* logits, int positions,
                   int vocab, int dtype, int gamma, int32_t* accept_len,
                   int32_t* accept_path, int32_t* out_tokens, hipStream_t st);
struct DraftRows {         // rows per request of each draft step (the draft logits' blocks)
  int n;
  int rows[kSlots];
};
bool verify_drafted_ok(int vocab);
void launch_verify_drafted(const TreeDev& t, int B, const void* logits, const float* draft_logits,
                           int positions, int vocab, int dtype, float inv_temp, float draft_inv_temp,
                           const float* draws, int gamma, const DraftRows& dr, int32_t* accept_len,
                           int32_t* accept_path, int32_t* out_tokens, hipStream_t st);
bool verify_sample_ok(int vocab, int dtype);
void launch_verify_sample(const TreeDev& t, int B, const void* logits, int positions, int vocab,
                          int dtype, float inv_temp, const float* draws, int gamma,
                          int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
                          hipStream_t st);
void launch_kv_commit(int B, int gamma, int row_bytes, const int32_t* accept_len,
                      const int32_t* accept_path, const void* k_tree, const void* v_tree,
                      const int32_t* dst_row, int64_t dst_rows, void* k_dst, void* v_dst,
                      hipStream_t st);
void launch_tree_rows_final(const TreeDev& t, int B, int32_t* tok_idx,
                            int32_t* kv_idx, int32_t* pos, uint64_t* mask,
                            hipStream_t st);

}  // namespace eagle
