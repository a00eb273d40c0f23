// C-ABI entry points of libeagle: argument validation, tree geometry,
// workspace layout and the launch sequence of one draft step.  No device
// memory is allocated here; every launch goes to the caller's stream.
#include <string.h>

#include <algorithm>
#include <vector>


#include "kernels.h"

using namespace eagle;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// ---------------------------------------------------------------- tree shape
struct Geo {
  int kind = 0, B = 0, gamma = 0, top_k = 0, top_m = 0, sample = 0;
  int pool_cap = 0, max_rows = 0, positions = 0, slots = 0;
  std::vector<int> rows;              // rows per request of each step
  std::vector<StaticPlan> plans;      // chain / static: children of each step
};

int build_geo(const eagle_tree* t, Geo* g) {
  if (!t) return EAGLE_EINVAL;
  if (t->B < 1 || t->gamma < 1 || t->top_k < 1) return EAGLE_EINVAL;
  if (t->top_k > EAGLE_MAX_TOPK) return EAGLE_EUNSUPPORTED;
  // finite and bounded, so s * logit stays finite for any finite logit of
  // the model (a NaN confidence would still be ordered last by the expansion)
  if (!(t->inv_temp > 0.f) || !(t->inv_temp <= EAGLE_MAX_INV_TEMP)) return EAGLE_EINVAL;
  if (t->sample != 0 && t->sample != 1) return EAGLE_EINVAL;
  g->kind = t->kind;
  g->B = t->B;
  g->gamma = t->gamma;
  g->top_k = t->top_k;
  g->top_m = t->top_m;
  g->sample = t->sample;
  g->rows.assign(t->gamma, 0);
  g->plans.assign(t->gamma, StaticPlan{});
  if (t->kind == EAGLE_TREE_CHAIN) {
    g->pool_cap = t->gamma + 1;
    g->positions = t->gamma + 1;
    for (int s = 0; s < t->gamma; ++s) {
      g->rows[s] = 1;
      StaticPlan& p = g->plans[s];
      p.nchild = 1;
      p.row[0] = 0;
      p.rank[0] = 0;
      p.expand[0] = s + 1 < t->gamma;
      p.nnext = p.expand[0];
    }
  } else if (t->kind == EAGLE_TREE_STATIC) {
    const int nt = t->n_template;
    if (nt < 1 || !t->template_parent) return EAGLE_EINVAL;
    if (nt + 1 > EAGLE_MAX_POSITIONS) return EAGLE_ECAPACITY;
    std::vector<std::vector<int>> ch(nt + 1);
    std::vector<int> depth(nt + 1, 0);
    for (int i = 0; i < nt; ++i) {
      const int p = t->template_parent[i];
      if (p < 0 || p > i) return EAGLE_EINVAL;
      ch[p].push_back(i + 1);
      depth[i + 1] = depth[p] + 1;
    }
    const int maxd = *std::max_element(depth.begin(), depth.end());
    if (maxd != t->gamma) return EAGLE_EINVAL;
    for (int u = 0; u <= nt; ++u)
      if ((int)ch[u].size() > t->top_k) return EAGLE_EINVAL;
    std::vector<int> frontier{0};
    for (int s = 0; s < t->gamma; ++s) {
      if (frontier.empty()) return EAGLE_EINVAL;
      g->rows[s] = (int)frontier.size();
      StaticPlan& p = g->plans[s];
      std::vector<int> next;
      int k = 0;
      for (size_t r = 0; r < frontier.size(); ++r) {
        const auto& kids = ch[frontier[r]];
        for (size_t rank = 0; rank < kids.size(); ++rank) {
          if (k >= 64) return EAGLE_ECAPACITY;
          const int tc = kids[rank];
          const bool ex = !ch[tc].empty() && s + 1 < t->gamma;
          p.row[k] = (uint8_t)r;
          p.rank[k] = (uint8_t)rank;
          p.expand[k] = ex;
          ++k;
          if (ex) next.push_back(tc);
        }
      }
      p.nchild = k;
      p.nnext = (int)next.size();
      frontier = next;
    }
    g->pool_cap = nt + 1;
    g->positions = nt + 1;
  } else if (t->kind == EAGLE_TREE_DYNAMIC) {
    const int64_t cap = 1 + (int64_t)t->top_k + (int64_t)(t->gamma - 1) * t->top_k * t->top_k;
    if (cap > 1024) return EAGLE_ECAPACITY;
    g->pool_cap = (int)cap;
    if (t->top_m < 1 || t->top_m > cap - 1) return EAGLE_EINVAL;
    if (t->top_m + 1 > EAGLE_MAX_POSITIONS) return EAGLE_ECAPACITY;
    g->positions = t->top_m + 1;
    for (int s = 0; s < t->gamma; ++s) g->rows[s] = s == 0 ? 1 : t->top_k;
  } else {
    return EAGLE_EINVAL;
  }
  g->max_rows = *std::max_element(g->rows.begin(), g->rows.end());
  int slots = 0;
  for (int r : g->rows) slots += r;
  g->slots = slots;
  if (slots > EAGLE_MAX_SLOTS) return EAGLE_ECAPACITY;
  return EAGLE_OK;
}

void layout_of(const Geo& g, eagle_tree_layout* L) {
  memset(L, 0, sizeof(*L));
  Bump bp;
  const size_t B = g.B, P = g.pool_cap, R = (size_t)g.B * g.max_rows, K = g.top_k;
  L->pool_cap = g.pool_cap;
  L->max_rows = g.max_rows;
  L->positions = g.positions;
  L->pool_tok = bp.take(B * P * 4);
  L->pool_parent = bp.take(B * P * 4);
  L->pool_depth = bp.take(B * P * 4);
  L->pool_slot = bp.take(B * P * 4);
  L->pool_conf = bp.take(B * P * 4);
  L->pool_value = bp.take(B * P * 4);
  L->pool_count = bp.take(B * 4);
  L->slot_count = bp.take(B * 4);
  L->root_pos = bp.take(B * 4);
  L->slot_mask = bp.take(B * kSlots * 8);
  L->row_node = bp.take(2 * R * 4);
  L->row_tok = bp.take(2 * R * 4);
  L->row_pos = bp.take(2 * R * 4);
  L->row_slot = bp.take(2 * R * 4);
  L->row_pidx = bp.take(2 * R * 4);
  L->row_mask = bp.take(2 * R * 8);
  L->topk_id = bp.take(R * K * 4);
  L->topk_conf = bp.take(R * K * 4);
  L->lse = bp.take(R * 4);
  L->f_node = bp.take(B * kMaxPos * 4);
  L->f_tok = bp.take(B * kMaxPos * 4);
  L->f_parent = bp.take(B * kMaxPos * 4);
  L->f_depth = bp.take(B * kMaxPos * 4);
  L->f_pos = bp.take(B * kMaxPos * 4);
  L->f_mask = bp.take(B * kMaxPos * 8);
  L->f_count = bp.take(B * 4);
  L->choice = bp.take(B * kMaxPos * 4);
  L->choice_part = bp.take(B * kMaxPos * kVerifySplits * 8);
  L->status = bp.take(B * 4);
  L->total = bp.off;
}

// Row arrays of step `step` (double buffer by step parity).
RowsDev rows_dev(const eagle_tree* t, const Geo& g, int step) {
  eagle_tree_layout L;
  layout_of(g, &L);
  char* s = (char*)t->state;
  const size_t R = (size_t)g.B * g.max_rows, h = (size_t)(step & 1) * R;
  RowsDev r;
  r.node = (int32_t*)(s + L.row_node) + h;
  r.tok = (int32_t*)(s + L.row_tok) + h;
  r.pos = (int32_t*)(s + L.row_pos) + h;
  r.slot = (int32_t*)(s + L.row_slot) + h;
  r.pidx = (int32_t*)(s + L.row_pidx) + h;
  r.mask = (uint64_t*)(s + L.row_mask) + h;
  return r;
}

TreeDev tree_dev(const eagle_tree* t, const Geo& g, int step = 0) {
  eagle_tree_layout L;
  layout_of(g, &L);
  char* s = (char*)t->state;
  TreeDev d;
  d.pool_tok = (int32_t*)(s + L.pool_tok);
  d.pool_parent = (int32_t*)(s + L.pool_parent);
  d.pool_depth = (int32_t*)(s + L.pool_depth);
  d.pool_slot = (int32_t*)(s + L.pool_slot);
  d.pool_conf = (float*)(s + L.pool_conf);
  d.pool_value = (float*)(s + L.pool_value);
  d.pool_count = (int32_t*)(s + L.pool_count);
  d.slot_count = (int32_t*)(s + L.slot_count);
  d.root_pos = (int32_t*)(s + L.root_pos);
  d.slot_mask = (uint64_t*)(s + L.slot_mask);
  d.row_node = (int32_t*)(s + L.row_node);
  d.row_tok = (int32_t*)(s + L.row_tok);
  d.row_pos = (int32_t*)(s + L.row_pos);
  d.row_slot = (int32_t*)(s + L.row_slot);
  d.row_pidx = (int32_t*)(s + L.row_pidx);
  d.row_mask = (uint64_t*)(s + L.row_mask);
  d.topk_id = (int32_t*)(s + L.topk_id);
  d.topk_conf = (float*)(s + L.topk_conf);
  d.lse = (float*)(s + L.lse);
  d.f_node = (int32_t*)(s + L.f_node);
  d.f_tok = (int32_t*)(s + L.f_tok);
  d.f_parent = (int32_t*)(s + L.f_parent);
  d.f_depth = (int32_t*)(s + L.f_depth);
  d.f_pos = (int32_t*)(s + L.f_pos);
  d.f_mask = (uint64_t*)(s + L.f_mask);
  d.f_count = (int32_t*)(s + L.f_count);
  d.choice = (int32_t*)(s + L.choice);
  d.choice_part = (float2*)(s + L.choice_part);
  d.status = (int32_t*)(s + L.status);
  d.pool_cap = g.pool_cap;
  d.max_rows = g.max_rows;
  d.positions = g.positions;
  const RowsDev r = rows_dev(t, g, step);
  d.row_node = r.node;
  d.row_tok = r.tok;
  d.row_pos = r.pos;
  d.row_slot = r.slot;
  d.row_pidx = r.pidx;
  d.row_mask = r.mask;
  return d;
}

int check_tree_state(const eagle_tree* t, const Geo& g) {
  if (!t->state) return EAGLE_EINVAL;
  eagle_tree_layout L;
  layout_of(g, &L);
  if (t->state_bytes < L.total) return EAGLE_ECAPACITY;
  return EAGLE_OK;
}

// ---------------------------------------------------------------- head / kv
int esz(const eagle_head* h) { return h->dtype == EAGLE_BF16 ? 2 : 4; }

void prof_set_dtype(int dtype);   // roofline peak of the profiled launches

int check_head(const eagle_head* h) {
  if (!h) return EAGLE_EINVAL;
  prof_set_dtype(h->dtype);
  if (h->dtype != EAGLE_BF16 && h->dtype != EAGLE_F32) return EAGLE_EINVAL;
  if (h->act != EAGLE_ACT_SWIGLU && h->act != EAGLE_ACT_GELU) return EAGLE_EINVAL;
  if (h->norm != EAGLE_NORM_RMS && h->norm != EAGLE_NORM_LAYER) return EAGLE_EINVAL;
  if (h->mode != EAGLE_MODE_1 && h->mode != EAGLE_MODE_3) return EAGLE_EINVAL;
  if (h->d < 64 || h->ffn < 32 || h->vocab < 16 || h->n_q_heads < 1 || h->n_kv_heads < 1)
    return EAGLE_EINVAL;
  if (!(h->eps > 0.f) || h->rope_theta < 0.f) return EAGLE_EINVAL;
  if (h->d % 64 || h->ffn % 32) return EAGLE_EUNSUPPORTED;
  if (h->head_dim != 64 && h->head_dim != 128) return EAGLE_EUNSUPPORTED;
  if (h->n_q_heads % h->n_kv_heads) return EAGLE_EUNSUPPORTED;
  if (h->d > 16384 || h->ffn > 65536 || (int64_t)h->n_q_heads * h->head_dim > 16384)
    return EAGLE_EUNSUPPORTED;
  if (h->mode == EAGLE_MODE_1 && !h->w_fc) return EAGLE_EINVAL;
  if (h->mode == EAGLE_MODE_3 && !h->w_fuse) return EAGLE_EINVAL;
  if (!h->w_q || !h->w_k || !h->w_v || !h->w_o || !h->w_up || !h->w_down) return EAGLE_EINVAL;
  if (h->act == EAGLE_ACT_SWIGLU && !h->w_gate) return EAGLE_EINVAL;
  if (!h->norm1_g || !h->norm2_g || !h->emb || !h->lm_head) return EAGLE_EINVAL;
  if (h->norm == EAGLE_NORM_LAYER && (!h->norm1_b || !h->norm2_b)) return EAGLE_EINVAL;
  return EAGLE_OK;
}

int check_kv(const eagle_kv* kv, int B) {
  if (!kv) return EAGLE_EINVAL;
  if (kv->B != B || B < 1 || kv->max_n < 0 || kv->total_n < 0) return EAGLE_EINVAL;
  if (!kv->n || !kv->cu_n || !kv->k_slot || !kv->v_slot || !kv->feat_slot) return EAGLE_EINVAL;
  if (kv->total_n > 0 && (!kv->k_ctx || !kv->v_ctx)) return EAGLE_EINVAL;
  if (kv->total_n > INT32_MAX || kv->max_n > kv->total_n) return EAGLE_EINVAL;
  if (kv->n_new) {
    if (!kv->cu_new || kv->total_new < B || kv->total_new > kv->total_n) return EAGLE_EINVAL;
  } else if (kv->cu_new || kv->total_new != 0) {
    return EAGLE_EINVAL;
  }
  return EAGLE_OK;
}

// Rows the EAGLE-3 ingest processes: every context position, or only each
// request's newest ones in the steady state.
int64_t ingest_rows(const eagle_kv* kv) { return kv->n_new ? kv->total_new : kv->total_n; }

int check_attn_plan(const eagle_head* h, const eagle_kv* kv);

// ---------------------------------------------------------------- profiling
constexpr size_t kMaxTimed = 16384;
struct ProfFamily {
  int64_t launches = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  size_t used = 0;
  double bytes = 0, flops = 0;
  double roof_s = 0;          // sum over launches of max(bytes / HBM peak, flops / MFMA peak)
};
// MI355X datasheet peaks the per-launch roofline is taken against
constexpr double kPeakHbm = 8.0e12;             // B/s, HBM3E
constexpr double kPeakBf16 = 2.5e15;            // flop/s, dense bf16 MFMA
constexpr double kPeakF32 = 157.3e12;           // flop/s, fp32
struct Prof {
  unsigned mask = 0;          // bit f set: family f is profiled
  double peak_flops = kPeakBf16;   // of the head of the current call
  ProfFamily fam[EAGLE_PROF_FAMILIES];
};
Prof g_prof;
void prof_set_dtype(int dtype) { g_prof.peak_flops = dtype == EAGLE_F32 ? kPeakF32 : kPeakBf16; }

// Brackets one launch with events on its stream when profiling is enabled.
// Each scope reserves its own event pair when it opens, so scopes may nest.
struct ProfScope {
  ProfFamily* f = nullptr;
  hipStream_t st = nullptr;
  size_t slot = 0;
  bool timed = false;
  ProfScope(int family, double bytes, double flops, hipStream_t s) {
    if (!(g_prof.mask >> family & 1u)) return;
    f = &g_prof.fam[family];
    st = s;
    f->launches += 1;
    f->bytes += bytes;
    f->flops += flops;
    f->roof_s += std::max(bytes / kPeakHbm, flops / g_prof.peak_flops);
    if (f->used >= kMaxTimed) return;
    if (f->used == f->ev.size()) {
      hipEvent_t a, b;
      // device-scope release only: the timed kernels' results stay on the GPU
      if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
      if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipEventDestroy(a);
        return;
      }
      f->ev.push_back({a, b});
    }
    slot = f->used;
    if (hipEventRecord(f->ev[slot].first, st) != hipSuccess) return;
    f->used += 1;
    timed = true;
  }
  ~ProfScope() {
    if (timed) (void)hipEventRecord(f->ev[slot].second, st);
  }
};

// ---------------------------------------------------------------- workspace
struct AttnPlan {
  int split_len, nsplit;
};
AttnPlan plan_attn(const eagle_head* h, const eagle_kv* kv) {
  AttnPlan p;
  // about 2048 (request, kv head, split) units; splits are whole 64-key tiles
  const int64_t work = (int64_t)std::max(kv->max_n, 1) * kv->B * h->n_kv_heads;
  int64_t units = (work + 64 * 2048 - 1) / (64 * 2048);
  if (units < 1) units = 1;
  p.split_len = (int)(64 * units);
  p.nsplit = (std::max(kv->max_n, 1) + p.split_len - 1) / p.split_len;
  return p;
}

struct Ws {
  size_t h, hn, h1, h1n, f, q, o, act, P, y32, stats, logits;
  size_t rs0, rs1;   // row-complete path (M <= 16): per-block row statistics
  size_t att_o, att_ml, lm_max, lm_sum, lm_id, lm_val, lm_lg;
  size_t tk, tv, t_tok, t_kv, t_pos, t_mask;
  size_t x_in, xn_in, P_in;
  size_t total;
  AttnPlan ap;
};

size_t gemm_bytes(int dtype, int M, int N, int K) {
  if (M <= 0) return 0;
  GemmShape s = plan_gemm(dtype, M, N, K);
  return (size_t)s.S * M * N * 4;
}

int check_attn_plan(const eagle_head* h, const eagle_kv* kv) {
  // the combine folds at most 1024 split partials per row
  return plan_attn(h, kv).nsplit + 1 <= 1024 ? EAGLE_OK : EAGLE_EUNSUPPORTED;
}

// target: sized for the target's verification pass as well (every buffer
// holds the B * positions verify-tree rows)
Ws plan_ws(const eagle_head* h, const eagle_kv* kv, const Geo& g, bool target = false) {
  Ws w;
  Bump bp;
  const int e = esz(h), d = h->d, qd = h->n_q_heads * h->head_dim,
            kvd = h->n_kv_heads * h->head_dim;
  const int nact = h->act == EAGLE_ACT_SWIGLU ? 2 * h->ffn : h->ffn;
  const int Mt = g.B * g.positions;
  const int Mmax = target ? std::max(g.B * g.max_rows, Mt) : g.B * g.max_rows;
  const int Mr = std::max(Mmax, Mt);
  w.h = bp.take((size_t)Mr * d * e);
  w.hn = bp.take((size_t)Mr * d * e);
  w.h1 = bp.take((size_t)Mmax * d * e);
  w.h1n = bp.take((size_t)Mmax * d * e);
  w.f = bp.take((size_t)Mmax * d * e);
  w.q = bp.take((size_t)Mr * qd * e);
  w.o = bp.take((size_t)Mr * qd * e);
  w.act = bp.take((size_t)Mmax * h->ffn * e);
  size_t P = gemm_bytes(h->dtype, Mt, qd + 2 * kvd, d);
  if (target) {
    P = std::max(P, gemm_bytes(h->dtype, Mt, d, qd));
    P = std::max(P, gemm_bytes(h->dtype, Mt, nact, d));
    P = std::max(P, gemm_bytes(h->dtype, Mt, d, h->ffn));
  }
  for (int s = 0; s < g.gamma; ++s) {
    const int M = g.B * g.rows[s];
    if (h->mode == EAGLE_MODE_1) P = std::max(P, gemm_bytes(h->dtype, M, d, 2 * d));
    P = std::max(P, gemm_bytes(h->dtype, M, qd + 2 * kvd, d));
    P = std::max(P, gemm_bytes(h->dtype, M, d, qd));
    P = std::max(P, gemm_bytes(h->dtype, M, nact, d));
    P = std::max(P, gemm_bytes(h->dtype, M, d, h->ffn));
  }
  w.P = bp.take(P);
  const bool ingests = h->mode == EAGLE_MODE_3 || kv->n_new;
  const int Mrow = std::max(Mr, ingests ? (int)ingest_rows(kv) : 0);
  w.y32 = bp.take((size_t)Mrow * d * 4);
  w.stats = bp.take((size_t)Mrow * ((d + 255) / 256) * 2 * 4);
  w.ap = plan_attn(h, kv);
  const size_t nparts = (size_t)w.ap.nsplit + 1;
  w.att_o = bp.take(nparts * Mr * h->n_q_heads * h->head_dim * 4);
  w.att_ml = bp.take(nparts * Mr * h->n_q_heads * 2 * 4);
  LmShape ls = plan_lmhead(h->dtype, Mmax, h->vocab);
  // draft steps on the tiled GEMM: with the fused LM-head epilogue one part
  // per workgroup and no logits buffer, else fp32 logits and tile partials
  // (the target pass writes its logits straight to the caller's buffer)
  bool need_lg = false;
  for (int s = 0; s < g.gamma; ++s) {
    const int M = g.B * g.rows[s];
    if (!big_gemm_ok(h->dtype, M, h->vocab, d)) continue;
    if (!g.sample && lm_fused_ok(h->dtype, M, h->vocab, d, g.top_k)) {
      ls.ntiles = std::max(ls.ntiles, lm_fused_parts(M, h->vocab, d));
    } else {
      need_lg = true;
      ls.ntiles = std::max(ls.ntiles, logits_tiles(h->vocab));
    }
  }
  const int Mlg = g.B * g.max_rows;
  w.logits = need_lg ? bp.take((size_t)Mlg * h->vocab * 4) : 0;
  w.lm_max = bp.take((size_t)ls.ntiles * Mmax * 4);
  w.lm_sum = bp.take((size_t)ls.ntiles * Mmax * 4);
  w.lm_id = bp.take((size_t)ls.ntiles * Mmax * g.top_k * 4);
  w.lm_val = bp.take((size_t)ls.ntiles * Mmax * g.top_k * 4);
  w.lm_lg = bp.take((size_t)ls.ntiles * Mmax * g.top_k * 4);
  w.tk = bp.take((size_t)g.B * kSlots * kvd * e);
  w.tv = bp.take((size_t)g.B * kSlots * kvd * e);
  {
    const int R = std::min(Mmax, 16);
    w.rs0 = bp.take((size_t)R * (d / 16) * 2 * 4);
    w.rs1 = bp.take((size_t)R * (d / 16) * 2 * 4);
  }
  w.t_tok = bp.take((size_t)Mt * 4);
  w.t_kv = bp.take((size_t)Mt * 4);
  w.t_pos = bp.take((size_t)Mt * 4);
  w.t_mask = bp.take((size_t)Mt * 8);
  if (ingests) {
    const int Tn = (int)ingest_rows(kv);
    const int kin = h->mode == EAGLE_MODE_3 ? 3 * d : 2 * d;
    w.x_in = bp.take((size_t)Tn * d * e);
    w.xn_in = bp.take((size_t)Tn * d * e);
    w.P_in = bp.take(std::max(gemm_bytes(h->dtype, Tn, d, kin),
                              gemm_bytes(h->dtype, Tn, 2 * kvd, d)));
  } else {
    w.x_in = w.xn_in = w.P_in = 0;
  }
  w.total = bp.off;
  return w;
}

hipError_t last_error() { return hipGetLastError(); }

RowSrc rs(const void* base, const int32_t* idx, int64_t stride, int64_t limit = 0) {
  return RowSrc{base, idx, stride, limit};
}

void gemm(const eagle_head* h, RowSrc x0, RowSrc x1, int ksplit, int M, int N, int K,
          const void* w0, const void* w1, const void* w2, int nseg1, int nseg2, float* P,
          GemmShape* shape, hipStream_t st) {
  GemmArgs a;
  a.xs[0] = x0;
  a.xs[1] = x1;
  a.ksplit_x = ksplit;
  a.M = M;
  a.N = N;
  a.K = K;
  a.w[0] = w0;
  a.w[1] = w1 ? w1 : w0;
  a.w[2] = w2 ? w2 : (w1 ? w1 : w0);
  a.nseg1 = nseg1;
  a.nseg2 = nseg2;
  a.P = P;
  a.kps = 0;
  *shape = plan_gemm(h->dtype, M, N, K);
  ProfScope ps(EAGLE_PROF_GEMM, (double)esz(h) * ((double)N * K + (double)M * K),
               2.0 * M * (double)N * K, st);
  launch_gemm(h->dtype, a, *shape, st);
}

// scratch of the row-norm epilogue, set per call by the entry points
float* g_y32 = nullptr;
float* g_stats = nullptr;

void reduce(const eagle_head* h, const float* P, int S, int M, int N, RowSrc s1, RowSrc s2,
            void* out, RowSrc scatter, void* out_norm, int which_norm, hipStream_t st,
            bool keep_stats = false, void* out_g = nullptr) {
  ReduceArgs a;
  a.keep_stats = keep_stats;
  a.out_g = out_g;
  a.y32 = g_y32;
  a.stats = g_stats;
  a.P = P;
  a.S = S;
  a.M = M;
  a.N = N;
  a.src1 = s1;
  a.src2 = s2;
  a.out = out;
  a.out_scatter = scatter;
  a.out_norm = out_norm;
  a.gain = which_norm == 1 ? h->norm1_g : h->norm2_g;
  a.bias = h->norm == EAGLE_NORM_LAYER ? (which_norm == 1 ? h->norm1_b : h->norm2_b) : nullptr;
  a.layer_norm = h->norm == EAGLE_NORM_LAYER;
  a.eps = h->eps;
  ProfScope ps(EAGLE_PROF_OTHER, 0, 0, st);
  launch_reduce_rows(h->dtype, a, st);
}

const RowSrc kNone{nullptr, nullptr, 0, 0};

// q|k|v projection of rows already normalised in `hn`, RoPE, scatter.  With
// xstats (RMSNorm folded through the projection) `hn` holds y * g and xstats
// the per-256-column (sum, sum of squares) of y; the projected rows are
// scaled by rstd before the rotation.
void qkv_rope(const eagle_head* h, const char* ws, const Ws& w, const void* hn, int M,
              const int32_t* pos, void* kdst, void* vdst, const int32_t* kv_idx, hipStream_t st,
              const float* xstats = nullptr) {
  const int d = h->d, qd = h->n_q_heads * h->head_dim, kvd = h->n_kv_heads * h->head_dim;
  GemmShape sh;
  float* P = (float*)(ws + w.P);
  gemm(h, rs(hn, nullptr, d), kNone, d, M, qd + 2 * kvd, d, h->w_q, h->w_k, h->w_v, qd, qd + kvd,
       P, &sh, st);
  QkvArgs q;
  q.P = P;
  q.S = sh.S;
  q.M = M;
  q.Hq = h->n_q_heads;
  q.Hkv = h->n_kv_heads;
  q.hd = h->head_dim;
  q.theta = h->rope_theta;
  q.pos = pos;
  q.q = (void*)(ws + w.q);
  q.k = kdst;
  q.v = vdst;
  q.kv_idx = kv_idx;
  q.xstats = xstats;
  q.xnblk = (d + 255) / 256;
  q.xN = d;
  q.eps = h->eps;
  ProfScope ps(EAGLE_PROF_OTHER, 0, 0, st);
  launch_epi_qkv(h->dtype, q, st);
}

void attend(const eagle_head* h, const eagle_kv* kv, const char* ws, const Ws& w, int W,
            const void* k_ex, const void* v_ex, const uint64_t* mask, void* out, hipStream_t st) {
  AttnArgs a;
  a.q = ws + w.q;
  a.B = kv->B;
  a.W = W;
  a.Hq = h->n_q_heads;
  a.Hkv = h->n_kv_heads;
  a.hd = h->head_dim;
  a.n = kv->n;
  a.cu_n = kv->cu_n;
  a.k_ctx = kv->k_ctx;
  a.v_ctx = kv->v_ctx;
  a.k_ex = k_ex;
  a.v_ex = v_ex;
  a.mask = mask;
  a.split_len = w.ap.split_len;
  a.nsplit = w.ap.nsplit;
  const int Rkv = W * (h->n_q_heads / h->n_kv_heads);
  if (Rkv > 16) {
    // the workgroup kernel (more than 16 query rows per kv head) keeps two
    // tiles in flight: splits of an eighth of the context, between two and
    // eight tiles, amortise its prologue (fewer splits than the workspace
    // was sized for)
    const int max_n = std::max(kv->max_n, 1);
    const int min_len = std::min(512, std::max(128, (max_n / 8 + 63) / 64 * 64));
    if (a.split_len < min_len) {
      a.split_len = min_len;
      a.nsplit = (max_n + a.split_len - 1) / a.split_len;
    }
    // and where a few (request, kv head) pairs leave the grid short of one
    // pass of resident workgroups, the splits are lengthened to exactly one
    // pass: a partial second pass idles most CUs, and every split writes
    // fp32 partials for all of its rows (the 256-row workgroups of the
    // verify-side tree, one per CU, write as many bytes as they read)
    if (h->dtype == EAGLE_BF16 && h->head_dim == 128) {
      const int rows_wg = Rkv <= 32 ? 32 : (Rkv <= 64 ? 64 : 256);
      const int64_t per_split = (int64_t)h->n_kv_heads * kv->B * ((Rkv + rows_wg - 1) / rows_wg);
      const int64_t resident = 256LL * (Rkv <= 64 ? 2 : 1);
      const int64_t fit = resident / per_split - 1;    // context splits beside the tree split
      if (fit >= 1 && (int64_t)(a.nsplit + 1) * per_split > resident) {
        a.split_len = (int)(((max_n + fit - 1) / fit + 63) / 64 * 64);
        a.nsplit = (max_n + a.split_len - 1) / a.split_len;
      }
    }
  } else {
    // the per-wave kernel (two waves of LDS-staged V per workgroup): when the
    // grid would need more than one pass of resident workgroups over the 256
    // CUs, the splits are lengthened until it fits in one (a short last pass
    // leaves most CUs idle while it runs)
    const int64_t lds = 2LL * h->head_dim * (64 * (int64_t)esz(h) + 16);
    const int64_t resident = (160 * 1024 / lds) * 256;
    const int64_t per_split = (int64_t)((h->n_kv_heads + 1) / 2) * kv->B;
    const int64_t fit = resident / per_split - 1;    // context splits beside the tree split
    if ((int64_t)(a.nsplit + 1) * per_split > resident && fit >= 1) {
      const int max_n = std::max(kv->max_n, 1);
      a.split_len = (int)(((max_n + fit - 1) / fit + 63) / 64 * 64);
      a.nsplit = (max_n + a.split_len - 1) / a.split_len;
    }
  }
  a.rowgroups = 1;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)h->head_dim);
  a.part_o = (float*)(ws + w.att_o);
  a.part_ml = (float*)(ws + w.att_ml);
  const double kvd = (double)h->n_kv_heads * h->head_dim;
  const double att_bytes = esz(h) * (2.0 * kv->total_n * kvd + (double)kv->B * W * h->n_q_heads * h->head_dim);
  const double att_flops = 4.0 * h->head_dim * (double)h->n_q_heads * W * (double)kv->total_n;
  {
    // context K and V of every request once, plus the queries
    ProfScope ps(EAGLE_PROF_ATTN, att_bytes, att_flops, st);
    launch_attention(h->dtype, a, st);
  }
  CombineArgs c;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  c.nparts = a.nsplit + 1;
  c.M = kv->B * W;
  c.Hq = h->n_q_heads;
  c.hd = h->head_dim;
  c.out = out;
  ProfScope ps(EAGLE_PROF_OTHER, 0, 0, st);
  launch_attn_combine(h->dtype, c, st);
}

// Row-complete GEMM launch (M <= 16): B-operand rows w0|w1|w2 split at
// nseg1 / nseg2; A operand, row scale and epilogue fields set by the caller.
RowsArgs rows_args(int M, int N, int K, const void* w0, const void* w1, const void* w2, int nseg1,
                   int nseg2) {
  RowsArgs r;
  memset(&r, 0, sizeof(r));
  r.g.M = M;
  r.g.N = N;
  r.g.K = K;
  r.g.w[0] = w0;
  r.g.w[1] = w1 ? w1 : w0;
  r.g.w[2] = w2 ? w2 : (w1 ? w1 : w0);
  r.g.nseg1 = nseg1;
  r.g.nseg2 = nseg2;
  r.g.ksplit_x = K;
  return r;
}

void run_rows(const eagle_head* h, int ep, const RowsArgs& r, hipStream_t st) {
  ProfScope ps(EAGLE_PROF_GEMM, (double)esz(h) * ((double)r.g.N * r.g.K + (double)r.g.M * r.g.K),
               2.0 * r.g.M * (double)r.g.N * r.g.K, st);
  launch_gemm_rows(h->dtype, ep, r, st);
}

// Ingest of verified context positions (all of them, or each request's newest
// n_new[b] in the steady state): their layer inputs, then N1 and the key /
// value projections with RoPE, written to k_ctx / v_ctx at each position's
// own row.  EAGLE-3: x_j = [l;m;h]_j W_fuse^T + emb(t_{j+1}), kept in x_in (the
// root row of each request is its last position).  EAGLE-1: x_j =
// fc([f_{j-1} ; emb(t_j)]) from the target's features (only the K/V are kept).
void ingest(const eagle_head* h, const eagle_kv* kv, char* ws, const Ws& w, const void* lmh,
            const int32_t* ctx_tokens, hipStream_t st) {
  const int d = h->d, kvd = h->n_kv_heads * h->head_dim;
  const int Tn = (int)ingest_rows(kv);
  const bool fold = h->norm == EAGLE_NORM_RMS;   // N1 folded through the k|v projection
  float* Pin = (float*)(ws + w.P_in);
  GemmShape sh;
  if (h->mode == EAGLE_MODE_3 && fold && big_rowepi_ok(h->dtype, Tn, d, 3 * d)) {
    // one tiled GEMM: x = [l;m;h] W_fuse^T + emb(t) in bf16, x * g1 and the
    // row statistics written by its epilogue (no fp32 partials, no row kernel)
    GemmArgs ga;
    ga.xs[0] = rs(lmh, nullptr, 3 * d);
    ga.xs[1] = kNone;
    ga.ksplit_x = 3 * d;
    ga.M = Tn;
    ga.N = d;
    ga.K = 3 * d;
    ga.w[0] = ga.w[1] = ga.w[2] = h->w_fuse;
    ga.nseg1 = ga.nseg2 = d;
    ga.P = nullptr;
    ga.row_epi = 1;
    ga.res = rs(h->emb, ctx_tokens, d, h->vocab);
    ga.out = ws + w.x_in;
    ga.out_g = ws + w.xn_in;
    ga.gain = h->norm1_g;
    ga.stats = g_stats;
    const GemmShape gs = plan_gemm_big(Tn, d, 3 * d);
    ProfScope ps(EAGLE_PROF_GEMM, (double)esz(h) * ((double)d * 3 * d + (double)Tn * 3 * d),
                 2.0 * Tn * (double)d * 3 * d, st);
    launch_gemm_big(ga, gs, st);
  } else if (h->mode == EAGLE_MODE_3) {
    gemm(h, rs(lmh, nullptr, 3 * d), kNone, 3 * d, Tn, d, 3 * d, h->w_fuse, nullptr, nullptr, d,
         d, Pin, &sh, st);
    reduce(h, Pin, sh.S, Tn, d, kNone, rs(h->emb, ctx_tokens, d, h->vocab), ws + w.x_in, kNone,
           fold ? nullptr : ws + w.xn_in, 1, st, fold, fold ? ws + w.xn_in : nullptr);
  } else {
    gemm(h, rs(lmh, nullptr, d), rs(h->emb, ctx_tokens, d, h->vocab), d, Tn, d, 2 * d, h->w_fc,
         nullptr, nullptr, d, d, Pin, &sh, st);
    reduce(h, Pin, sh.S, Tn, d, kNone, kNone, nullptr, kNone, fold ? nullptr : ws + w.xn_in, 1, st,
           fold, fold ? ws + w.xn_in : nullptr);
  }
  gemm(h, rs(ws + w.xn_in, nullptr, d), kNone, d, Tn, 2 * kvd, d, h->w_k, h->w_v, nullptr, kvd,
       2 * kvd, Pin, &sh, st);
  QkvArgs q;
  q.P = Pin;
  q.S = sh.S;
  q.M = Tn;
  q.Hq = 0;
  q.Hkv = h->n_kv_heads;
  q.hd = h->head_dim;
  q.theta = h->rope_theta;
  q.cu_row = kv->n_new ? kv->cu_new : kv->cu_n;
  q.n = kv->n;
  q.n_new = kv->n_new;
  q.cu_n = kv->cu_n;
  q.total_rows = kv->total_n;
  q.B = kv->B;
  q.k = kv->k_ctx;
  q.v = kv->v_ctx;
  if (fold) {
    q.xstats = g_stats;
    q.xnblk = (d + 255) / 256;
    q.xN = d;
    q.eps = h->eps;
  }
  ProfScope ps(EAGLE_PROF_OTHER, 0, 0, st);
  launch_epi_qkv(h->dtype, q, st);
}

// One pre-norm decoder layer over io.M rows (io.W per request), from the
// attention sub-layer on.  Input rows io.x with N1(io.x) in io.xn (RMSNorm
// folded: io.x * g1 with per-block statistics io.nst / io.nblk, io.nblk =
// ceil(d / 256) on the tiled path; plain N1 rows when io.nst is null); q|k|v with RoPE at io.pos, K/V rows written to io.kdst /
// io.vdst rows io.kv_idx; attention over the request's context plus the rows
// in io.mask; output rows to io.out (and to io.scatter rows when given).
struct LayerIO {
  int M = 0, W = 0;
  const void* x = nullptr;
  const void* xn = nullptr;
  const float* nst = nullptr;
  int nblk = 0;
  const int32_t* pos = nullptr;
  void* kdst = nullptr;
  void* vdst = nullptr;
  const int32_t* kv_idx = nullptr;
  const uint64_t* mask = nullptr;
  void* out = nullptr;
  RowSrc scatter{nullptr, nullptr, 0, 0};
};

void layer_body(const eagle_head* h, const eagle_kv* kv, char* ws, const Ws& w, bool rows,
                const LayerIO& io, hipStream_t st) {
  const int d = h->d, qd = h->n_q_heads * h->head_dim, ffn = h->ffn;
  const int kvd = h->n_kv_heads * h->head_dim;
  const bool swiglu = h->act == EAGLE_ACT_SWIGLU;
  float* P = (float*)(ws + w.P);
  GemmShape sh;
  // tiled path: the fused-SwiGLU GEMM (one split, activation in its epilogue)
  // takes normalised rows; otherwise, for RMSNorm, N2 is folded through the
  // gate|up projection into the four-column activation epilogue
  const bool big_act = swiglu && big_swiglu_ok(h->dtype, io.M, ffn, d);
  const bool fold2 = !rows && !big_act && h->norm == EAGLE_NORM_RMS &&
                     epi_act4_ok(io.M, ffn, P, ws + w.act);
  // ---- attention sub-layer
  if (rows) {
    RowsArgs r = rows_args(io.M, qd + 2 * kvd, d, h->w_q, h->w_k, h->w_v, qd, qd + kvd);
    r.g.xs[0] = rs(io.xn, nullptr, d);
    r.xstats = io.nst;
    r.xnblk = io.nblk;
    r.eps = h->eps;
    r.Hq = h->n_q_heads;
    r.Hkv = h->n_kv_heads;
    r.hd = h->head_dim;
    r.theta = h->rope_theta;
    r.pos = io.pos;
    r.q = ws + w.q;
    r.k = io.kdst;
    r.v = io.vdst;
    r.kv_idx = io.kv_idx;
    run_rows(h, EP_ROPE, r, st);
  } else {
    qkv_rope(h, ws, w, io.xn, io.M, io.pos, io.kdst, io.vdst, io.kv_idx, st, io.nst);
  }
  attend(h, kv, ws, w, io.W, io.kdst, io.vdst, io.mask, ws + w.o, st);
  if (rows) {
    RowsArgs r = rows_args(io.M, d, qd, h->w_o, nullptr, nullptr, d, d);
    r.g.xs[0] = rs(ws + w.o, nullptr, qd);
    r.res = rs(io.x, nullptr, d);
    r.out = ws + w.h1;
    r.out_g = ws + w.h1n;
    r.gain = h->norm2_g;
    r.stats = (float*)(ws + w.rs1);
    run_rows(h, EP_STORE, r, st);
  } else {
    gemm(h, rs(ws + w.o, nullptr, qd), kNone, qd, io.M, d, qd, h->w_o, nullptr, nullptr, d, d, P, &sh,
         st);
    reduce(h, P, sh.S, io.M, d, rs(io.x, nullptr, d), kNone, ws + w.h1, kNone,
           fold2 ? nullptr : ws + w.h1n, 2, st, fold2, fold2 ? ws + w.h1n : nullptr);
  }

  // ---- MLP sub-layer
  if (rows) {
    RowsArgs r = swiglu ? rows_args(io.M, 2 * ffn, d, h->w_gate, h->w_up, nullptr, ffn, 2 * ffn)
                        : rows_args(io.M, ffn, d, h->w_up, nullptr, nullptr, ffn, ffn);
    r.g.xs[0] = rs(ws + w.h1n, nullptr, d);
    r.xstats = (const float*)(ws + w.rs1);
    r.xnblk = d / 16;
    r.eps = h->eps;
    r.act_F = ffn;
    r.out = ws + w.act;
    run_rows(h, swiglu ? EP_SWIGLU : EP_GELU, r, st);
    RowsArgs r2 = rows_args(io.M, d, ffn, h->w_down, nullptr, nullptr, d, d);
    r2.g.xs[0] = rs(ws + w.act, nullptr, ffn);
    r2.res = rs(ws + w.h1, nullptr, d);
    r2.out = io.out;
    r2.scatter = io.scatter;
    run_rows(h, EP_STORE, r2, st);
  } else {
    if (big_act) {
      // one split: the tiled GEMM writes silu(gate) * up itself
      GemmArgs ga;
      ga.xs[0] = rs(ws + w.h1n, nullptr, d);
      ga.xs[1] = kNone;
      ga.ksplit_x = d;
      ga.M = io.M;
      ga.N = 2 * ffn;
      ga.K = d;
      ga.w[0] = h->w_gate;
      ga.w[1] = ga.w[2] = h->w_up;
      ga.nseg1 = ffn;
      ga.nseg2 = 2 * ffn;
      ga.P = nullptr;
      ga.pair_F = ffn;
      ga.act = ws + w.act;
      const GemmShape gs = plan_gemm_big(io.M, 2 * ffn, d);
      ProfScope ps(EAGLE_PROF_GEMM, (double)esz(h) * (2.0 * ffn * d + (double)io.M * d),
                   2.0 * io.M * 2.0 * ffn * d, st);
      launch_gemm_big(ga, gs, st);
    } else {
      if (swiglu)
        gemm(h, rs(ws + w.h1n, nullptr, d), kNone, d, io.M, 2 * ffn, d, h->w_gate, h->w_up, nullptr,
             ffn, 2 * ffn, P, &sh, st);
      else
        gemm(h, rs(ws + w.h1n, nullptr, d), kNone, d, io.M, ffn, d, h->w_up, nullptr, nullptr, ffn,
             ffn, P, &sh, st);
      ActArgs aa;
      aa.P = P;
      aa.S = sh.S;
      aa.M = io.M;
      aa.F = ffn;
      aa.swiglu = swiglu;
      aa.out = ws + w.act;
      if (fold2) {
        aa.xstats = g_stats;
        aa.xnblk = (d + 255) / 256;
        aa.xN = d;
        aa.eps = h->eps;
      }
      ProfScope ps(EAGLE_PROF_OTHER, 0, 0, st);
      launch_epi_act(h->dtype, aa, st);
    }
    gemm(h, rs(ws + w.act, nullptr, ffn), kNone, ffn, io.M, d, ffn, h->w_down, nullptr, nullptr, d, d,
         P, &sh, st);
    reduce(h, P, sh.S, io.M, d, rs(ws + w.h1, nullptr, d), kNone, io.out, io.scatter, nullptr, 0,
           st);
  }

}

int finish(int status) {
  if (status != EAGLE_OK) return status;
  return last_error() == hipSuccess ? EAGLE_OK : EAGLE_EHIP;
}

}  // namespace

// ====================================================================== ABI
extern "C" {

const char* eagle_version(void) { return "eagle-mi355x 0.1 (gfx950)"; }

int eagle_profile_enable(int family_mask) {
  g_prof.mask = (unsigned)family_mask & ((1u << EAGLE_PROF_FAMILIES) - 1u);
  return EAGLE_OK;
}

int eagle_profile_reset(void) {
  for (auto& f : g_prof.fam) {
    f.launches = 0;
    f.used = 0;
    f.bytes = f.flops = 0;
    f.roof_s = 0;
  }
  return EAGLE_OK;
}

int eagle_profile_read(int family, int64_t* launches, int64_t* timed_launches, double* total_ms,
                       double* bytes, double* flops, double* roofline_ms) {
  if (family < 0 || family >= EAGLE_PROF_FAMILIES) return EAGLE_EINVAL;
  ProfFamily& f = g_prof.fam[family];
  double ms = 0;
  for (size_t i = 0; i < f.used; ++i) {
    if (hipEventSynchronize(f.ev[i].second) != hipSuccess) return EAGLE_EHIP;
    float t = 0;
    if (hipEventElapsedTime(&t, f.ev[i].first, f.ev[i].second) != hipSuccess) return EAGLE_EHIP;
    ms += t;
  }
  if (launches) *launches = f.launches;
  if (timed_launches) *timed_launches = (int64_t)f.used;
  if (total_ms) *total_ms = ms;
  if (bytes) *bytes = f.bytes;
  if (flops) *flops = f.flops;
  if (roofline_ms) *roofline_ms = f.roof_s * 1e3;
  return EAGLE_OK;
}

const char* eagle_strerror(int s) {
  switch (s) {
    case EAGLE_OK: return "ok";
    case EAGLE_EINVAL: return "invalid argument";
    case EAGLE_EUNSUPPORTED: return "unsupported shape";
    case EAGLE_ECAPACITY: return "capacity exceeded (workspace, tree state, slots or positions)";
    case EAGLE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int eagle_tree_layout_of(const eagle_tree* tree, eagle_tree_layout* out) {
  if (!out) return EAGLE_EINVAL;
  Geo g;
  int s = build_geo(tree, &g);
  if (s) return s;
  layout_of(g, out);
  return EAGLE_OK;
}

size_t eagle_tree_state_bytes(const eagle_tree* tree) {
  eagle_tree_layout L;
  return eagle_tree_layout_of(tree, &L) == EAGLE_OK ? L.total : 0;
}

int eagle_step_rows(const eagle_tree* tree, int step) {
  Geo g;
  if (build_geo(tree, &g)) return 0;
  if (step < 0 || step >= g.gamma) return 0;
  return g.rows[step];
}

size_t eagle_workspace_bytes(const eagle_head* head, const eagle_kv* kv, const eagle_tree* tree) {
  Geo g;
  if (check_head(head) || build_geo(tree, &g) || check_kv(kv, g.B)) return 0;
  return plan_ws(head, kv, g).total;
}

int eagle_tree_init(const eagle_head* head, const eagle_kv* kv, const eagle_tree* tree,
                    const int32_t* root_tokens, void* stream) {
  Geo g;
  int s;
  if ((s = check_head(head))) return s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_kv(kv, g.B))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (!root_tokens) return EAGLE_EINVAL;
  if (head->mode == EAGLE_MODE_3 && ingest_rows(kv) < kv->B) return EAGLE_EINVAL;
  // EAGLE-3 root rows: the last ingested row of each request
  launch_tree_init(tree_dev(tree, g), g.B, head->mode == EAGLE_MODE_3, head->vocab, root_tokens,
                   kv->n, kv->n_new ? kv->cu_new : kv->cu_n, (hipStream_t)stream);
  return finish(EAGLE_OK);
}

int eagle_draft_step(const eagle_head* h, const eagle_kv* kv, const eagle_tree* tree, int step,
                     const void* f_root, const void* lmh, const int32_t* ctx_tokens,
                     float* logits_out, void* feat_out, void* ws_v, size_t ws_bytes,
                     void* stream) {
  Geo g;
  int s;
  if ((s = check_head(h))) return s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_kv(kv, g.B))) return s;
  if ((s = check_attn_plan(h, kv))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (step < 0 || step >= g.gamma) return EAGLE_EINVAL;
  if (g.top_k > h->vocab) return EAGLE_EINVAL;
  const bool e3 = h->mode == EAGLE_MODE_3;
  if (step == 0 && !e3 && !f_root) return EAGLE_EINVAL;
  if (step == 0 && e3 && (!lmh || !ctx_tokens || ingest_rows(kv) < kv->B)) return EAGLE_EINVAL;
  if (step == 0 && !e3 && kv->n_new && (!lmh || !ctx_tokens)) return EAGLE_EINVAL;
  if (!ws_v) return EAGLE_EINVAL;
  const Ws w = plan_ws(h, kv, g);
  if (ws_bytes < w.total) return EAGLE_ECAPACITY;

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)ws_v;
  g_y32 = (float*)(ws + w.y32);
  g_stats = (float*)(ws + w.stats);
  const TreeDev td = tree_dev(tree, g, step);
  const int B = g.B, W = g.rows[step], M = B * W;
  const int d = h->d;
  float* P = (float*)(ws + w.P);
  void* hbuf = ws + w.h;
  void* hn = ws + w.hn;
  GemmShape sh;

  // ---- layer input h and N1(h)
  // Row-complete path (M <= 16, RMSNorm): every projection of the layer is
  // one kernel with its epilogue fused; N1 / N2 are folded through the next
  // projection (operand h * g, result rows scaled by rstd from the statistics).
  const bool rows = rows_gemm_ok(M, d, 32) && h->norm == EAGLE_NORM_RMS;
  // RMSNorm: N1 is folded through the q|k|v projection on both paths
  const bool fold = h->norm == EAGLE_NORM_RMS;
  const float* nst = g_stats;          // row statistics of h
  int nblk = (d + 255) / 256;
  if (!e3) {
    if (step == 0 && kv->n_new) ingest(h, kv, ws, w, lmh, ctx_tokens, st);
    const void* fsrc = step == 0 ? f_root : kv->feat_slot;
    const RowSrc xf = rs(fsrc, td.row_pidx, d, step == 0 ? (int64_t)B : (int64_t)B * kSlots);
    const RowSrc xe = rs(h->emb, td.row_tok, d, h->vocab);
    if (rows) {
      RowsArgs r = rows_args(M, d, 2 * d, h->w_fc, nullptr, nullptr, d, d);
      r.g.xs[0] = xf;
      r.g.xs[1] = xe;
      r.g.ksplit_x = d;
      r.out = hbuf;
      r.out_g = hn;
      r.gain = h->norm1_g;
      r.stats = (float*)(ws + w.rs0);
      run_rows(h, EP_STORE, r, st);
      nst = r.stats;
      nblk = d / 16;
    } else {
      gemm(h, xf, xe, d, M, d, 2 * d, h->w_fc, nullptr, nullptr, d, d, P, &sh, st);
      reduce(h, P, sh.S, M, d, kNone, kNone, hbuf, kNone, fold ? nullptr : hn, 1, st, fold,
             fold ? hn : nullptr);
    }
  } else if (step > 0) {
    reduce(h, nullptr, 0, M, d, rs(kv->feat_slot, td.row_pidx, d, (int64_t)B * kSlots), rs(h->emb, td.row_tok, d, h->vocab),
           hbuf, kNone, fold ? nullptr : hn, 1, st, fold, fold ? hn : nullptr);
  } else {
    ingest(h, kv, ws, w, lmh, ctx_tokens, st);
    // root rows = each request's last verified position
    reduce(h, nullptr, 0, M, d, rs(ws + w.x_in, td.row_pidx, d, ingest_rows(kv)), kNone, hbuf, kNone,
           fold ? nullptr : hn, 1, st, fold, fold ? hn : nullptr);
  }

  // ---- decoder layer from the attention sub-layer on
  void* fout = feat_out ? feat_out : (void*)(ws + w.f);
  {
    LayerIO io;
    io.M = M;
    io.W = W;
    io.x = hbuf;
    io.xn = hn;
    io.nst = fold ? nst : nullptr;
    io.nblk = nblk;
    io.pos = td.row_pos;
    io.kdst = kv->k_slot;
    io.vdst = kv->v_slot;
    io.kv_idx = td.row_slot;
    io.mask = td.row_mask;
    io.out = fout;
    io.scatter = rs(kv->feat_slot, td.row_slot, d);
    layer_body(h, kv, ws, w, rows, io, st);
  }

  // ---- LM head + softmax / top-k
  LmShape ls = plan_lmhead(h->dtype, M, h->vocab);
  LmArgs la;
  la.x = rs(fout, nullptr, d);
  la.M = M;
  la.K = d;
  la.V = h->vocab;
  la.w = h->lm_head;
  la.top_k = g.top_k;
  la.inv_temp = tree->inv_temp;
  la.logits = logits_out;
  la.part_max = (float*)(ws + w.lm_max);
  la.part_sum = (float*)(ws + w.lm_sum);
  la.part_id = (int*)(ws + w.lm_id);
  la.part_val = (float*)(ws + w.lm_val);
  if (tree->sample) {
    la.gumbel = 1;
    la.seed_lo = (uint32_t)(tree->sample_seed & 0xFFFFFFFFu);
    la.seed_hi = (uint32_t)(tree->sample_seed >> 32);
    la.row_node = td.row_node;
    la.rows_per_req = W;
    la.part_logit = (float*)(ws + w.lm_lg);
  }
  if (!tree->sample && lm_fused_ok(h->dtype, M, h->vocab, d, g.top_k)) {
    // the tiled GEMM folds softmax / top-k into its epilogue: one part per
    // workgroup (the logits only when the caller asks for them)
    GemmArgs ga;
    ga.xs[0] = rs(fout, nullptr, d);
    ga.xs[1] = kNone;
    ga.ksplit_x = d;
    ga.M = M;
    ga.N = h->vocab;
    ga.K = d;
    ga.w[0] = ga.w[1] = ga.w[2] = h->lm_head;
    ga.nseg1 = ga.nseg2 = h->vocab;
    ga.P = logits_out;
    ga.lm_top_k = g.top_k;
    ga.lm_inv_temp = tree->inv_temp;
    ga.lm_max = la.part_max;
    ga.lm_sum = la.part_sum;
    ga.lm_val = la.part_val;
    ga.lm_id = la.part_id;
    GemmShape gs = plan_gemm_big(M, h->vocab, d);
    gs.S = 1;
    gs.kps = d;
    ls.ntiles = lm_fused_parts(M, h->vocab, d);
    ProfScope ps(EAGLE_PROF_LMHEAD, (double)esz(h) * ((double)h->vocab * d + (double)M * d),
                 2.0 * M * (double)h->vocab * d, st);
    launch_gemm_big(ga, gs, st);
  } else if (big_gemm_ok(h->dtype, M, h->vocab, d)) {
    // MFMA-bound: tiled GEMM into fp32 logits, then tile partials
    float* lg = logits_out ? logits_out : (float*)(ws + w.logits);
    GemmArgs ga;
    ga.xs[0] = rs(fout, nullptr, d);
    ga.xs[1] = kNone;
    ga.ksplit_x = d;
    ga.M = M;
    ga.N = h->vocab;
    ga.K = d;
    ga.w[0] = ga.w[1] = ga.w[2] = h->lm_head;
    ga.nseg1 = ga.nseg2 = h->vocab;
    ga.P = lg;
    GemmShape gs = plan_gemm_big(M, h->vocab, d);
    gs.S = 1;
    gs.kps = d;
    {
      ProfScope ps(EAGLE_PROF_LMHEAD, (double)esz(h) * ((double)h->vocab * d + (double)M * d),
                   2.0 * M * (double)h->vocab * d, st);
      launch_gemm_big(ga, gs, st);
    }
    la.logits = nullptr;
    ls.ntiles = logits_tiles(h->vocab);
    ProfScope ps(EAGLE_PROF_OTHER, 0, 0, st);
    launch_logits_partials(la, lg, st);
  } else {
    ProfScope ps(EAGLE_PROF_LMHEAD, (double)esz(h) * ((double)h->vocab * d + (double)M * d),
                 2.0 * M * (double)h->vocab * d, st);
    launch_lmhead(h->dtype, la, ls, st);
  }
  MergeArgs ma;
  ma.part_max = la.part_max;
  ma.part_sum = la.part_sum;
  ma.part_id = la.part_id;
  ma.part_val = la.part_val;
  ma.ntiles = ls.ntiles;
  ma.M = M;
  ma.top_k = g.top_k;
  ma.inv_temp = tree->inv_temp;
  ma.topk_id = td.topk_id;
  ma.topk_conf = td.topk_conf;
  ma.lse = td.lse;
  ma.vocab = h->vocab;
  ma.part_logit = la.part_logit;
  {
    ProfScope ps(EAGLE_PROF_OTHER, 0, 0, st);
    launch_topk_merge(ma, st);
  }
  return finish(EAGLE_OK);
}

int eagle_tree_expand_rerank(const eagle_tree* tree, int step, void* stream) {
  Geo g;
  int s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (step < 0 || step >= g.gamma) return EAGLE_EINVAL;
  const bool fin = step == g.gamma - 1;
  ProfScope ps(EAGLE_PROF_OTHER, 0, 0, (hipStream_t)stream);
  launch_tree_expand(tree_dev(tree, g, step), rows_dev(tree, g, step + 1), g.B, g.kind, step,
                     g.gamma, g.rows[step], g.top_k, g.top_m, fin, g.plans[step],
                     (hipStream_t)stream);
  return finish(EAGLE_OK);
}

int eagle_tree_attend(const eagle_head* h, const eagle_kv* kv, const eagle_tree* tree, void* out,
                      void* ws_v, size_t ws_bytes, void* stream) {
  Geo g;
  int s;
  if ((s = check_head(h))) return s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_kv(kv, g.B))) return s;
  if ((s = check_attn_plan(h, kv))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (!out || !ws_v) return EAGLE_EINVAL;
  const Ws w = plan_ws(h, kv, g);
  if (ws_bytes < w.total) return EAGLE_ECAPACITY;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)ws_v;
  g_y32 = (float*)(ws + w.y32);
  g_stats = (float*)(ws + w.stats);
  const TreeDev td = tree_dev(tree, g);
  const int Wt = g.positions, M = g.B * Wt, d = h->d;
  int32_t* t_tok = (int32_t*)(ws + w.t_tok);
  int32_t* t_kv = (int32_t*)(ws + w.t_kv);
  int32_t* t_pos = (int32_t*)(ws + w.t_pos);
  uint64_t* t_mask = (uint64_t*)(ws + w.t_mask);
  launch_tree_rows_final(td, g.B, t_tok, t_kv, t_pos, t_mask, st);
  const bool fold = h->norm == EAGLE_NORM_RMS;   // N1 folded through the q|k|v projection
  reduce(h, nullptr, 0, M, d, rs(h->emb, t_tok, d, h->vocab), kNone, nullptr, kNone,
         fold ? nullptr : ws + w.hn, 1, st, fold, fold ? ws + w.hn : nullptr);
  qkv_rope(h, ws, w, ws + w.hn, M, t_pos, ws + w.tk, ws + w.tv, t_kv, st, fold ? g_stats : nullptr);
  attend(h, kv, ws, w, Wt, ws + w.tk, ws + w.tv, t_mask, out, st);
  return finish(EAGLE_OK);
}

int check_target(const eagle_head* h, const eagle_target* t, const eagle_kv* kv) {
  if (!t || t->n_layers < 1 || !t->layers || !t->final_norm_g) return EAGLE_EINVAL;
  for (int l = 0; l < t->n_layers; ++l) {
    const eagle_layer& L = t->layers[l];
    if (!L.w_q || !L.w_k || !L.w_v || !L.w_o || !L.w_up || !L.w_down) return EAGLE_EINVAL;
    if (h->act == EAGLE_ACT_SWIGLU && !L.w_gate) return EAGLE_EINVAL;
    if (!L.norm1_g || !L.norm2_g) return EAGLE_EINVAL;
    if (h->norm == EAGLE_NORM_LAYER && (!L.norm1_b || !L.norm2_b)) return EAGLE_EINVAL;
    if (kv && kv->total_n > 0 && (!L.k_ctx || !L.v_ctx)) return EAGLE_EINVAL;
  }
  return EAGLE_OK;
}

size_t eagle_target_workspace_bytes(const eagle_head* head, const eagle_target* target,
                                    const eagle_kv* kv, const eagle_tree* tree) {
  Geo g;
  if (check_head(head) || check_target(head, target, kv) || build_geo(tree, &g) || check_kv(kv, g.B))
    return 0;
  return plan_ws(head, kv, g, true).total;
}

int eagle_target_verify_logits(const eagle_head* head, const eagle_target* target,
                               const eagle_kv* kv, const eagle_tree* tree, float* logits_out,
                               void* k_tree, void* v_tree, void* hidden_out, void* ws_v,
                               size_t ws_bytes, void* stream) {
  Geo g;
  int s;
  if ((s = check_head(head))) return s;
  if ((s = check_target(head, target, kv))) return s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_kv(kv, g.B))) return s;
  if ((s = check_attn_plan(head, kv))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (!logits_out || !ws_v || (!k_tree) != (!v_tree)) return EAGLE_EINVAL;
  const Ws w = plan_ws(head, kv, g, true);
  if (ws_bytes < w.total) return EAGLE_ECAPACITY;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)ws_v;
  g_y32 = (float*)(ws + w.y32);
  g_stats = (float*)(ws + w.stats);
  const TreeDev td = tree_dev(tree, g);
  const int Wt = g.positions, M = g.B * Wt, d = head->d;
  const int kvd = head->n_kv_heads * head->head_dim;
  int32_t* t_tok = (int32_t*)(ws + w.t_tok);
  int32_t* t_kv = (int32_t*)(ws + w.t_kv);
  int32_t* t_pos = (int32_t*)(ws + w.t_pos);
  uint64_t* t_mask = (uint64_t*)(ws + w.t_mask);
  launch_tree_rows_final(td, g.B, t_tok, t_kv, t_pos, t_mask, st);
  const bool rows = rows_gemm_ok(M, d, 32) && head->norm == EAGLE_NORM_RMS;
  // layer inputs alternate between two row buffers (or go to the caller's
  // hidden_out, one [M][d] block per layer boundary); layer 0 reads the
  // embeddings of the verify-tree tokens
  void* xb[2] = {ws + w.h, ws + w.f};
  const size_t hid = (size_t)M * d * esz(head);
  auto xin = [&](int l) -> void* { return hidden_out ? (char*)hidden_out + l * hid : xb[l & 1]; };
  const size_t tree_kv = (size_t)g.B * kSlots * kvd * esz(head);
  for (int l = 0; l < target->n_layers; ++l) {
    const eagle_layer& L = target->layers[l];
    eagle_head hl = *head;
    hl.w_q = L.w_q;
    hl.w_k = L.w_k;
    hl.w_v = L.w_v;
    hl.w_o = L.w_o;
    hl.w_gate = L.w_gate;
    hl.w_up = L.w_up;
    hl.w_down = L.w_down;
    hl.norm1_g = L.norm1_g;
    hl.norm1_b = L.norm1_b;
    hl.norm2_g = L.norm2_g;
    hl.norm2_b = L.norm2_b;
    eagle_kv kl = *kv;
    kl.k_ctx = const_cast<void*>(L.k_ctx);
    kl.v_ctx = const_cast<void*>(L.v_ctx);
    void* x = xin(l);
    // N1 of the layer input (RMSNorm: x * g1 and its row statistics, the
    // scale folded through the q|k|v projection)
    const bool fold = head->norm == EAGLE_NORM_RMS;
    void* n1 = fold ? nullptr : ws + w.hn;
    void* n1g = fold ? ws + w.hn : nullptr;
    if (l == 0)
      reduce(&hl, nullptr, 0, M, d, rs(head->emb, t_tok, d, head->vocab), kNone, x, kNone, n1, 1, st,
             fold, n1g);
    else
      reduce(&hl, nullptr, 0, M, d, rs(x, nullptr, d), kNone, nullptr, kNone, n1, 1, st, fold, n1g);
    LayerIO io;
    io.M = M;
    io.W = Wt;
    io.x = x;
    io.xn = ws + w.hn;
    io.nst = fold ? g_stats : nullptr;
    io.nblk = (d + 255) / 256;
    io.pos = t_pos;
    io.kdst = k_tree ? (char*)k_tree + l * tree_kv : (void*)(ws + w.tk);
    io.vdst = v_tree ? (char*)v_tree + l * tree_kv : (void*)(ws + w.tv);
    io.kv_idx = t_kv;
    io.mask = t_mask;
    io.out = xin(l + 1);
    layer_body(&hl, &kl, ws, w, rows, io, st);
  }
  // final RMSNorm, then the shared LM head into fp32 logits
  eagle_head hf = *head;
  hf.norm = EAGLE_NORM_RMS;
  hf.norm1_g = target->final_norm_g;
  hf.norm1_b = nullptr;
  reduce(&hf, nullptr, 0, M, d, rs(xin(target->n_layers), nullptr, d), kNone, nullptr, kNone,
         ws + w.hn, 1, st);
  const double lm_bytes = (double)esz(head) * ((double)head->vocab * d + (double)M * d);
  const double lm_flops = 2.0 * M * (double)head->vocab * d;
  if (big_gemm_ok(head->dtype, M, head->vocab, d)) {
    GemmArgs ga;
    ga.xs[0] = rs(ws + w.hn, nullptr, d);
    ga.xs[1] = kNone;
    ga.ksplit_x = d;
    ga.M = M;
    ga.N = head->vocab;
    ga.K = d;
    ga.w[0] = ga.w[1] = ga.w[2] = head->lm_head;
    ga.nseg1 = ga.nseg2 = head->vocab;
    ga.P = logits_out;
    GemmShape gs = plan_gemm_big(M, head->vocab, d);
    gs.S = 1;
    gs.kps = d;
    ProfScope ps(EAGLE_PROF_LMHEAD, lm_bytes, lm_flops, st);
    launch_gemm_big(ga, gs, st);
  } else {
    LmShape ls = plan_lmhead(head->dtype, M, head->vocab);
    LmArgs la;
    la.x = rs(ws + w.hn, nullptr, d);
    la.M = M;
    la.K = d;
    la.V = head->vocab;
    la.w = head->lm_head;
    la.top_k = 1;
    la.inv_temp = 1.0f;
    la.logits = logits_out;
    la.part_max = (float*)(ws + w.lm_max);
    la.part_sum = (float*)(ws + w.lm_sum);
    la.part_id = (int*)(ws + w.lm_id);
    la.part_val = (float*)(ws + w.lm_val);
    ProfScope ps(EAGLE_PROF_LMHEAD, lm_bytes, lm_flops, st);
    launch_lmhead(head->dtype, la, ls, st);
  }
  return finish(EAGLE_OK);
}

int eagle_kv_commit(const eagle_tree* tree, int kv_heads, int head_dim, int dtype,
                    const int32_t* accept_len, const int32_t* accept_path, const void* k_tree,
                    const void* v_tree, const int32_t* dst_row, int64_t dst_rows, void* k_dst,
                    void* v_dst, void* stream) {
  Geo g;
  int s;
  if ((s = build_geo(tree, &g))) return s;
  if (kv_heads < 1 || head_dim < 1 || (dtype != EAGLE_BF16 && dtype != EAGLE_F32)) return EAGLE_EINVAL;
  if (!accept_len || !accept_path || !k_tree || !v_tree || !dst_row || !k_dst || !v_dst)
    return EAGLE_EINVAL;
  if (dst_rows < 1) return EAGLE_EINVAL;
  const int64_t row_bytes = (int64_t)kv_heads * head_dim * (dtype == EAGLE_BF16 ? 2 : 4);
  if (row_bytes % 16 || row_bytes > INT32_MAX) return EAGLE_EINVAL;
  for (const void* p : {k_tree, v_tree, (const void*)k_dst, (const void*)v_dst})
    if (reinterpret_cast<uintptr_t>(p) & 15) return EAGLE_EINVAL;
  ProfScope ps(EAGLE_PROF_OTHER, 0, 0, (hipStream_t)stream);
  launch_kv_commit(g.B, g.gamma, (int)row_bytes, accept_len,
                   accept_path, k_tree, v_tree, dst_row, dst_rows, k_dst, v_dst,
                   (hipStream_t)stream);
  return finish(EAGLE_OK);
}

int eagle_tree_verify(const eagle_tree* tree, const void* target_logits, int positions, int vocab,
                      int dtype, int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
                      void* stream) {
  Geo g;
  int s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (!target_logits || !accept_len || !accept_path || !out_tokens) return EAGLE_EINVAL;
  if (dtype != EAGLE_BF16 && dtype != EAGLE_F32) return EAGLE_EINVAL;
  if (vocab < 1 || positions < g.positions) return EAGLE_EINVAL;
  {
    ProfScope ps(EAGLE_PROF_VERIFY, (double)g.B * g.positions * vocab * (dtype == EAGLE_BF16 ? 2 : 4),
                 0, (hipStream_t)stream);
    launch_verify(tree_dev(tree, g), g.B, target_logits, positions, vocab, dtype, g.gamma,
                  accept_len, accept_path, out_tokens, (hipStream_t)stream);
  }
  return finish(EAGLE_OK);
}

int eagle_tree_verify_sample_drafted(const eagle_tree* tree, const void* target_logits,
                                     int positions, int vocab, int dtype, float inv_temp,
                                     const float* draft_logits, const float* draws,
                                     int32_t* accept_len, int32_t* accept_path,
                                     int32_t* out_tokens, void* stream) {
  Geo g;
  int s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (tree->sample != 1) return EAGLE_EINVAL;     // top-k drafts: eagle_tree_verify_sample
  if (!target_logits || !draft_logits || !draws || !accept_len || !accept_path || !out_tokens)
    return EAGLE_EINVAL;
  if (dtype != EAGLE_BF16 && dtype != EAGLE_F32) return EAGLE_EINVAL;
  if (vocab < 1 || positions < g.positions) return EAGLE_EINVAL;
  if (!(inv_temp > 0.f) || !std::isfinite(inv_temp)) return EAGLE_EINVAL;
  if (!verify_drafted_ok(vocab)) return EAGLE_EUNSUPPORTED;
  DraftRows dr{};
  dr.n = g.gamma;
  for (int i = 0; i < g.gamma; ++i) dr.rows[i] = g.rows[i];
  {
    ProfScope ps(EAGLE_PROF_VERIFY, 0, 0, (hipStream_t)stream);
    launch_verify_drafted(tree_dev(tree, g), g.B, target_logits, draft_logits, positions, vocab,
                          dtype, inv_temp, tree->inv_temp, draws, g.gamma, dr, accept_len,
                          accept_path, out_tokens, (hipStream_t)stream);
  }
  return finish(EAGLE_OK);
}

int eagle_tree_verify_sample(const eagle_tree* tree, const void* target_logits, int positions,
                             int vocab, int dtype, float inv_temp, const float* draws,
                             int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
                             void* stream) {
  Geo g;
  int s;
  if ((s = build_geo(tree, &g))) return s;
  if ((s = check_tree_state(tree, g))) return s;
  if (!target_logits || !draws || !accept_len || !accept_path || !out_tokens) return EAGLE_EINVAL;
  if (dtype != EAGLE_BF16 && dtype != EAGLE_F32) return EAGLE_EINVAL;
  if (vocab < 1 || positions < g.positions) return EAGLE_EINVAL;
  if (!(inv_temp > 0.f) || !std::isfinite(inv_temp)) return EAGLE_EINVAL;
  if (!verify_sample_ok(vocab, dtype)) return EAGLE_EUNSUPPORTED;
  {
    ProfScope ps(EAGLE_PROF_VERIFY, 0, 0, (hipStream_t)stream);
    launch_verify_sample(tree_dev(tree, g), g.B, target_logits, positions, vocab, dtype, inv_temp,
                         draws, g.gamma, accept_len, accept_path, out_tokens, (hipStream_t)stream);
  }
  return finish(EAGLE_OK);
}

}  // extern "C"
