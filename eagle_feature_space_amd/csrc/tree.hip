// Draft-tree bookkeeping and greedy verification.
//
//   init    node 0 = anchor token, value 1; the step-0 rows are the roots.
//   expand  ("EAGLE-2: expand and rerank") children of every row of the step
//           get value = value(parent) * conf; the next frontier is chosen
//           (chain: the child; static: the template's expanded children;
//           dynamic: the top_k newest nodes by (value desc, index asc)), each
//           frontier node gets a slot and the 64-bit mask of its
//           ancestor-or-self slots.  The last step reranks (dynamic: top_m
//           of the pool by (value desc, depth asc, index asc)) and writes the
//           verify tree in creation order with ancestor-or-self masks over
//           positions and position ids root_pos + depth ("Tree attention in
//           one verification pass").
//   verify  (explainer steps 3-4) target choice per position = argmax of its
//           logits, lowest id on ties; walk from the root along children whose
//           token equals the choice; emit the accepted tokens and the choice at
//           the deepest accepted node.
// One workgroup serves one request; the pool holds at most 1024 nodes.
#include "kernels.h"

namespace eagle {

constexpr int kPoolMax = 1024;

__global__ void k_tree_init(TreeDev t, int B, int eagle3, int vocab, const int32_t* root_tok,
                            const int32_t* n, const int32_t* cu_n) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int P = t.pool_cap;
  const int tok = min(max(root_tok[b], 0), vocab - 1);
  t.pool_tok[b * P] = tok;
  t.pool_parent[b * P] = -1;
  t.pool_depth[b * P] = 0;
  t.pool_slot[b * P] = 0;
  t.pool_conf[b * P] = 1.0f;
  t.pool_value[b * P] = 1.0f;
  t.pool_count[b] = 1;
  t.slot_count[b] = 1;
  const int rp = eagle3 ? n[b] - 1 : n[b];
  t.root_pos[b] = rp;
  const uint64_t m0 = eagle3 ? 0ull : 1ull;
  t.slot_mask[b * kSlots] = m0;
  t.row_node[b] = 0;
  t.row_tok[b] = tok;
  t.row_pos[b] = rp;
  t.row_slot[b] = b * kSlots;
  t.row_pidx[b] = eagle3 ? max(cu_n[b + 1] - 1, 0) : b;
  t.row_mask[b] = m0;
  t.f_count[b] = 0;
  t.status[b] = 0;
}

void launch_tree_init(const TreeDev& t, int B, int eagle3, int vocab, const int32_t* root_tok,
                      const int32_t* n, const int32_t* cu_n, hipStream_t st) {
  hipLaunchKernelGGL(k_tree_init, dim3((B + 63) / 64), dim3(64), 0, st, t, B, eagle3, vocab,
                     root_tok, n, cu_n);
}

// Path values lie in [0, 1]; a NaN one (from a NaN logit row) ranks below
// every other value, so the orders below stay total and every rank is a
// permutation of the nodes compared.
__device__ __forceinline__ float vkey(float v) { return v == v ? v : -1.0f; }

// key order: value desc, depth asc, index asc (values through vkey)
__device__ __forceinline__ bool before(float va, int da, int ia, float vb, int db, int ib) {
  va = vkey(va);
  vb = vkey(vb);
  if (va != vb) return va > vb;
  if (da != db) return da < db;
  return ia < ib;
}

// The same order as one unsigned 64-bit key (smaller = earlier): the value
// through vkey mapped to an order-preserving unsigned word and inverted
// (descending), then depth and index in 16 bits each.  +0 and -0 compare
// equal as floats but not as words; values are products of confidences in
// [0, 1] (or -1 for NaN), so -0 does not occur.
__device__ __forceinline__ uint64_t order_key(float v, int depth, int index) {
  const uint32_t u = __float_as_uint(vkey(v));
  const uint32_t mono = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)~mono << 32) | ((uint64_t)(depth & 0xFFFF) << 16) | (uint64_t)(index & 0xFFFF);
}

// `t` points its row_* arrays at the rows of this step; `nx` holds the row
// arrays of the next step (the other half of the double buffer): the two
// steps have different row counts per request, so writing in place would
// overwrite rows other workgroups have not read yet.
constexpr int kExpandThreads = 1024;   // one node of a full pool per thread

__global__ __launch_bounds__(kExpandThreads) void k_tree_expand(TreeDev t, RowsDev nx, int kind, int step,
                                                                int gamma, int W, int top_k, int top_m,
                                                                int final_step, StaticPlan plan) {
  constexpr int NT = kExpandThreads;
  __shared__ float sval[kPoolMax];
  __shared__ int sdep[kPoolMax];
  __shared__ int spar[kPoolMax];
  __shared__ int spos[kPoolMax];
  __shared__ uint64_t skey[kPoolMax];
  __shared__ int snext[256];
  __shared__ int swave[NT / 64];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = t.pool_cap;
  const int p0 = t.pool_count[b];
  const int nchild = kind == EAGLE_TREE_DYNAMIC ? W * top_k : plan.nchild;
  const int rp = t.root_pos[b];
  const int64_t pb = (int64_t)b * P;
  // a call out of order (pool or slots already full) must not write past
  // them: flag the request (its verify then reports accept_len -1)
  if (p0 < 1 || p0 + nchild > P ||
      (!final_step &&
       t.slot_count[b] + (kind == EAGLE_TREE_DYNAMIC ? min(top_k, nchild) : plan.nnext) > kSlots)) {
    if (tid == 0) t.status[b] = EAGLE_TREE_STATE_BAD;
    return;
  }

  // 1. append the children of this step's rows (their values also go to LDS)
  for (int cidx = tid; cidx < nchild; cidx += NT) {
    int row, rank;
    if (kind == EAGLE_TREE_DYNAMIC) { row = cidx / top_k; rank = cidx % top_k; }
    else { row = plan.row[cidx]; rank = plan.rank[cidx]; }
    const int r = b * W + row;
    int parent = t.row_node[r];
    if (parent < 0 || parent >= p0) parent = 0;   // never reached with a consistent state
    const float conf = t.topk_conf[(int64_t)r * top_k + rank];
    const int node = p0 + cidx;
    const float val = __fmul_rn(t.pool_value[pb + parent], conf);
    t.pool_tok[pb + node] = t.topk_id[(int64_t)r * top_k + rank];
    t.pool_parent[pb + node] = parent;
    t.pool_depth[pb + node] = t.pool_depth[pb + parent] + 1;
    t.pool_slot[pb + node] = -1;
    t.pool_conf[pb + node] = conf;
    t.pool_value[pb + node] = val;
    if (node < kPoolMax) sval[node] = val;
  }
  __syncthreads();
  __threadfence_block();
  const int pn = p0 + nchild;

  if (!final_step) {
    // 2. next frontier
    int nnext;
    if (kind == EAGLE_TREE_DYNAMIC) {
      nnext = min(top_k, nchild);
      // rank of each new node among the new nodes (value desc, index asc:
      // they share one depth) from packed keys; TPN consecutive lanes share a
      // node, each counting a slice of the others
      int tpn = 1;
      while (tpn < 16 && nchild * tpn * 2 <= NT) tpn *= 2;
      for (int cidx = tid; cidx < nchild; cidx += NT) skey[cidx] = order_key(sval[p0 + cidx], 0, p0 + cidx);
      __syncthreads();
      const int per = (nchild + tpn - 1) / tpn;
      for (int base = 0; base < nchild * tpn; base += NT) {   // uniform trip count
        const int slot = base + tid;
        const int cidx = slot / tpn, part = slot % tpn;
        int rank = 0;
        if (cidx < nchild) {
          const uint64_t ku = skey[cidx];
          const int j1 = min(nchild, (part + 1) * per);
          for (int j = part * per; j < j1; ++j) rank += skey[j] < ku;
        }
        for (int o = 1; o < tpn; o <<= 1) rank += __shfl_xor(rank, o, 64);
        if (cidx < nchild && part == 0 && rank < nnext) snext[rank] = p0 + cidx;
      }
    } else {
      nnext = plan.nnext;
      if (tid == 0) {
        int k = 0;
        for (int cidx = 0; cidx < nchild; ++cidx)
          if (plan.expand[cidx]) snext[k++] = p0 + cidx;
      }
    }
    __syncthreads();
    const int s0 = t.slot_count[b];
    if (tid < nnext) {
      const int u = snext[tid];
      const int slot = s0 + tid;
      const int parent = t.pool_parent[pb + u];
      const int pslot = max(t.pool_slot[pb + parent], 0);
      const uint64_t msk = t.slot_mask[b * kSlots + pslot] | (1ull << slot);
      t.pool_slot[pb + u] = slot;
      t.slot_mask[b * kSlots + slot] = msk;
      const int r = b * nnext + tid;
      nx.node[r] = u;
      nx.tok[r] = t.pool_tok[pb + u];
      nx.pos[r] = rp + t.pool_depth[pb + u];
      nx.slot[r] = b * kSlots + slot;
      nx.pidx[r] = b * kSlots + pslot;
      nx.mask[r] = msk;
    }
    __syncthreads();
    if (tid == 0) {
      t.pool_count[b] = pn;
      t.slot_count[b] = s0 + nnext;
    }
    return;
  }

  // 3. rerank and verify tree (pool sizes are at most kPoolMax = one node per thread)
  const int u = tid;
  if (u < pn) {
    sval[u] = t.pool_value[pb + u];
    sdep[u] = t.pool_depth[pb + u];
    spar[u] = t.pool_parent[pb + u];
    skey[u] = order_key(sval[u], sdep[u], u);
  }
  __syncthreads();
  int keep = 0;
  if (kind == EAGLE_TREE_DYNAMIC) {
    // rank of node x among the non-root nodes: the count of smaller keys.
    // With pn <= NT / 2 two threads share a node (lanes 2x and 2x+1, each
    // counting half of the pool); the ranks land in spos.
    const int half = pn <= NT / 2;
    const int x = half ? tid >> 1 : tid;
    if (x < pn && x > 0) {
      const uint64_t kx = skey[x];
      const int v0 = half ? 1 + (tid & 1) * ((pn - 1 + 1) / 2) : 1;
      const int v1 = half ? min(pn, 1 + ((tid & 1) + 1) * ((pn - 1 + 1) / 2)) : pn;
      int rank = 0;
      for (int v = v0; v < v1; ++v) rank += skey[v] < kx;
      if (half) rank += __shfl_xor(rank, 1, 64);
      if (!half || (tid & 1) == 0) spos[x] = rank;
    }
    __syncthreads();
    if (u < pn) keep = u == 0 || spos[u] < top_m;
    __syncthreads();
  } else if (u < pn) {
    keep = 1;
  }
  // positions in creation order: exclusive prefix count of the kept nodes
  const uint64_t bal = __builtin_amdgcn_ballot_w64(keep != 0);
  const int lane = tid & 63, wv = tid >> 6;
  if (lane == 0) swave[wv] = __builtin_popcountll(bal);
  __syncthreads();
  int before_waves = 0, total = 0;
  for (int w = 0; w < NT / 64; ++w) {
    const int c = swave[w];
    before_waves += w < wv ? c : 0;
    total += c;
  }
  const int pos = before_waves + __builtin_popcountll(bal & ((1ull << lane) - 1ull));
  // the ranks form a total order, so at most top_m + 1 (dynamic) or the whole
  // template (<= 64 positions, checked on the host) are kept; positions past
  // the verify tree's 64 are never written
  if (u < pn) spos[u] = keep && pos < kMaxPos ? pos : -1;
  if (tid == 0) {
    t.f_count[b] = min(total, kMaxPos);
    t.pool_count[b] = pn;
    if (total > kMaxPos) t.status[b] = EAGLE_TREE_STATE_BAD;
  }
  __syncthreads();
  if (u < pn && spos[u] >= 0) {
    const int p = spos[u];
    const int fb = b * kMaxPos;
    uint64_t msk = 0;
    // kept sets are ancestor-closed (confidences are <= 1, so values never
    // grow along a path and a parent ranks before its child).  Parents precede
    // children, so the walk strictly decreases and ends at the root.
    for (int w = u, it = 0; w >= 0 && it < kPoolMax; w = (spar[w] < w ? spar[w] : -1), ++it)
      if (spos[w] >= 0) msk |= 1ull << spos[w];
    t.f_node[fb + p] = u;
    t.f_tok[fb + p] = t.pool_tok[pb + u];
    t.f_parent[fb + p] = (u == 0 || spar[u] < 0) ? -1 : spos[spar[u]];
    t.f_depth[fb + p] = sdep[u];
    t.f_pos[fb + p] = rp + sdep[u];
    t.f_mask[fb + p] = msk;
  }
}

void launch_tree_expand(const TreeDev& t, const RowsDev& next, int B, int kind, int step,
                        int gamma, int rows, int top_k, int top_m, int final_step,
                        const StaticPlan& plan, hipStream_t st) {
  hipLaunchKernelGGL(k_tree_expand, dim3(B), dim3(kExpandThreads), 0, st, t, next, kind, step, gamma, rows,
                     top_k, top_m, final_step, plan);
}

// ---------------------------------------------------------------- verify
// A NaN logit counts as -inf, so every slice with at least one id has an
// argmax inside the vocabulary.
__device__ __forceinline__ float nan_low(float v) { return v == v ? v : -INFINITY; }

// Argmax of one vocabulary slice of one verify position (value desc, lowest
// index on ties); grid = (position, request, slice).
template <typename T>
__global__ __launch_bounds__(256) void k_verify_argmax(TreeDev t, const T* logits, int positions,
                                                       int V) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int u = blockIdx.x, b = blockIdx.y, sp = blockIdx.z;
  if (u >= t.f_count[b]) return;
  constexpr int VEC = DT<T>::VEC;
  const T* row = logits + ((int64_t)b * positions + u) * V;
  // slice boundaries on VEC-element granules
  const int nvec = V / VEC;
  const int per = (nvec + kVerifySplits - 1) / kVerifySplits;
  const int q0 = sp * per, q1 = min(nvec, q0 + per);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  if (aligned) {
    for (int q = q0 + threadIdx.x; q < q1; q += 256) {
      const u32x4 x = ld16(row + q * VEC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float v = nan_low(DT<T>::elem(x, e));
        const int j = q * VEC + e;
        if (better(v, j, bv, bi)) { bv = v; bi = j; }
      }
    }
  } else {
    for (int j = q0 * VEC + threadIdx.x; j < q1 * VEC; j += 256) {
      const float v = nan_low(DT<T>::ld(row + j));
      if (better(v, j, bv, bi)) { bv = v; bi = j; }
    }
  }
  if (sp == kVerifySplits - 1)   // ragged tail past the last whole granule
    for (int j = nvec * VEC + threadIdx.x; j < V; j += 256) {
      const float v = nan_low(DT<T>::ld(row + j));
      if (better(v, j, bv, bi)) { bv = v; bi = j; }
    }
  wave_best(bv, bi);
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v0 = sv[0];
    int i0 = si[0];
    for (int k = 1; k < 4; ++k)
      if (better(sv[k], si[k], v0, i0)) { v0 = sv[k]; i0 = si[k]; }
    t.choice_part[((int64_t)b * kMaxPos + u) * kVerifySplits + sp] = make_float2(v0, __int_as_float(i0));
  }
}

// target choice at a verify position: best of its slices, in slice order
__device__ __forceinline__ int verify_choice(const TreeDev& t, int b, int u, int vocab) {
  const float2* p = t.choice_part + ((int64_t)b * kMaxPos + u) * kVerifySplits;
  float bv = p[0].x;
  int bi = __float_as_int(p[0].y);
  for (int s = 1; s < kVerifySplits; ++s) {
    const int i = __float_as_int(p[s].y);
    if (better(p[s].x, i, bv, bi)) { bv = p[s].x; bi = i; }
  }
  if (bi < 0 || bi >= vocab) bi = 0;   // not reached: slice 0 always holds an id
  t.choice[b * kMaxPos + u] = bi;
  return bi;
}

__global__ void k_verify_walk(TreeDev t, int B, int gamma, int vocab, int32_t* accept_len,
                              int32_t* accept_path, int32_t* out_tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int T = min(t.f_count[b], kMaxPos);
  const int fb = b * kMaxPos;
  int32_t* path = accept_path + (int64_t)b * (gamma + 1);
  int32_t* out = out_tokens + (int64_t)b * (gamma + 1);
  for (int i = 0; i <= gamma; ++i) { path[i] = -1; out[i] = -1; }
  if (t.status[b] != 0 || T < 1) {   // inconsistent tree state: nothing to verify
    accept_len[b] = -1;
    return;
  }
  int u = 0, acc = 0;
  path[0] = 0;
  for (int it = 0; it <= gamma; ++it) {
    const int choice = verify_choice(t, b, u, vocab);
    int nxt = -1;
    for (int v = u + 1; v < T; ++v)
      if (t.f_parent[fb + v] == u && t.f_tok[fb + v] == choice) { nxt = v; break; }
    if (nxt < 0 || acc >= gamma) {
      out[acc] = choice;
      break;
    }
    out[acc] = choice;
    ++acc;
    path[acc] = nxt;
    u = nxt;
  }
  accept_len[b] = acc;
}

void launch_verify(const TreeDev& t, int B, const void* logits, int positions, int vocab,
                   int dtype, int gamma, int32_t* accept_len, int32_t* accept_path,
                   int32_t* out_tokens, hipStream_t st) {
  dim3 grid(kMaxPos, B, kVerifySplits);
  if (dtype == EAGLE_BF16)
    hipLaunchKernelGGL(k_verify_argmax<bf16s>, grid, dim3(256), 0, st, t, (const bf16s*)logits,
                       positions, vocab);
  else
    hipLaunchKernelGGL(k_verify_argmax<float>, grid, dim3(256), 0, st, t, (const float*)logits,
                       positions, vocab);
  hipLaunchKernelGGL(k_verify_walk, dim3((B + 63) / 64), dim3(64), 0, st, t, B, gamma, vocab,
                     accept_len, accept_path, out_tokens);
}

// ------------------------------------------------- stochastic verification
// Multi-round speculative sampling over the verify tree: one workgroup per
// request walks its tree and reads only the target rows the walk visits.
// At a visited node u, with v_y = fp32(s * z_y) and M = max_y v_y, every
// probability term is e_y = expf(v_y - M); S sums them, each granule (8 bf16 /
// 4 fp32 ids) in fp32, everything above that in fp64.
// Children of u are tried in verify-tree order: child i (token x) is kept iff
// draw[u][i] < e_x / (S - sum of e over the children rejected before it).
// When none is kept (or u has none, or is at depth gamma) one token is drawn
// from the residual (rejected tokens carry no mass) by inverse CDF over token
// ids.
//
// Row layout: granule q = 8 bf16 / 4 fp32 ids; round k = granules
// [k * NT, (k + 1) * NT), granule k * NT + t read by thread t (coalesced);
// a row's ids ascend with (round, thread, element).  A round's total is
// summed in a fixed order (thread granule, wave butterfly, waves in order),
// S is the sum of round totals in round order, and the residual draw finds
// its round from the totals, then its thread from an exclusive scan of the
// round's per-thread sums, then its id inside that thread's granule.
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;
constexpr int kMaxRounds = 64;   // rows of up to 64 * 1024 granules
constexpr int kDraws = EAGLE_VERIFY_DRAWS;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One granule's raw bits (ids past V read as -inf): a 16-byte load on rows on
// 16-byte boundaries, element loads for the ragged last granule and for
// unaligned rows.
template <typename T>
__device__ __forceinline__ u32x4 fetch_granule(const T* row, int q, int nvec, int V, bool aligned) {
  constexpr int VEC = DT<T>::VEC;
  if (aligned && q < nvec) return ld16(row + (int64_t)q * VEC);
  float f[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const int y = q * VEC + e;
    f[e] = y < V ? DT<T>::ld(row + y) : -INFINITY;
  }
  return DT<T>::pack(f);
}

// rounds c0 .. c0 + H - 1 of thread tid, all loads in flight together
template <typename T, int H>
__device__ __forceinline__ void load_rounds(u32x4 (&raw)[H], const T* row, int c0, int G,
                                            int NQ, int nvec, int V, bool aligned, int tid,
                                            u32x4 ninf) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int NT = kSampleThreads;
  if (aligned && nvec > 0) {
#pragma unroll
    for (int k = 0; k < H; ++k)
      raw[k] = ld16(row + (int64_t)min((c0 + k) * NT + tid, nvec - 1) * VEC);
  }
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const int q = (c0 + k) * NT + tid;
    if (c0 + k >= G || q >= NQ) raw[k] = ninf;
    else if (!aligned || q >= nvec) raw[k] = fetch_granule<T>(row, q, nvec, V, aligned);
  }
}

// Each pass streams the row in batches of H rounds (the second pass and the
// residual draw find it in L2).
template <typename T, int H>
__global__ __launch_bounds__(kSampleThreads) void k_verify_sample(
    TreeDev t, const T* logits, int positions, int V, float s, const float* draws, int gamma,
    int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int NT = kSampleThreads, NW = kSampleWaves;
  constexpr int RB = 4;             // round totals reduced together
  __shared__ int s_tok[kMaxPos], s_par[kMaxPos];
  __shared__ float s_max[NW];
  __shared__ float s_dr[kDraws];
  __shared__ double s_red[NW][RB];
  __shared__ double s_rt[kMaxRounds];
  __shared__ double s_e[kMaxTopK];
  __shared__ int s_x[kMaxTopK], s_v[kMaxTopK], s_nk;
  __shared__ int s_excl[kMaxTopK], s_nex, s_next, s_round, s_pick;
  __shared__ double s_tgt, s_pre[NW];
  __shared__ int s_last[NW];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T_ = min(t.f_count[b], kMaxPos);
  const int fb = b * kMaxPos;
  const int nvec = V / VEC;
  const int NQ = (V + VEC - 1) / VEC;             // granules, the last one maybe partial
  const int G = (NQ + NT - 1) / NT;               // rounds
  int32_t* path = accept_path + (int64_t)b * (gamma + 1);
  int32_t* out = out_tokens + (int64_t)b * (gamma + 1);
  if (tid < kMaxPos) {
    s_tok[tid] = tid < T_ ? t.f_tok[fb + tid] : -1;
    s_par[tid] = tid < T_ ? t.f_parent[fb + tid] : -2;
  }
  if (tid <= gamma) { path[tid] = tid == 0 ? 0 : -1; out[tid] = -1; }
  if (t.status[b] != 0 || T_ < 1) {   // inconsistent tree state: nothing to verify
    if (tid == 0) {
      path[0] = -1;
      accept_len[b] = -1;
    }
    return;
  }
  __syncthreads();

  u32x4 raw[H];
  u32x4 ninf;
  {
    float f[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) f[e] = -INFINITY;
    ninf = DT<T>::pack(f);
  }
  int u = 0, acc = 0;
  while (true) {
    const T* row = logits + ((int64_t)b * positions + u) * V;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    // this node's uniforms, fetched with the row
    if (wave == 1 && lane < kDraws) s_dr[lane] = draws[((int64_t)b * positions + u) * kDraws + lane];
    // M = max v
    float m = -INFINITY;
    for (int c0 = 0; c0 < G; c0 += H) {
      load_rounds<T, H>(raw, row, c0, G, NQ, nvec, V, aligned, tid, ninf);
#pragma unroll
      for (int k = 0; k < H; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) m = fmaxf(m, s * DT<T>::elem(raw[k], e));
    }
    m = wave_max(m);
    if (lane == 0) s_max[wave] = m;
    __syncthreads();
    float M = s_max[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_max[w]);
    // round totals, RB rounds reduced at a time
    for (int c0 = 0; c0 < G; c0 += H) {
      load_rounds<T, H>(raw, row, c0, G, NQ, nvec, V, aligned, tid, ninf);
#pragma unroll
      for (int r0 = 0; r0 < H; r0 += RB) {
        if (c0 + r0 >= G) break;
        double pr[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          // a granule's terms summed in fp32 (ids past V give expf(-inf) = 0)
          float gs = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) gs += expf(s * DT<T>::elem(raw[r0 + j], e) - M);
          pr[j] = (double)gs;
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) pr[j] = wave_sum_d(pr[j]);
        if (lane == 0)
#pragma unroll
          for (int j = 0; j < RB; ++j) s_red[wave][j] = pr[j];
        __syncthreads();
        if (tid < RB && c0 + r0 + tid < G) {
          double r = 0.0;
          for (int w = 0; w < NW; ++w) r += s_red[w][tid];
          s_rt[c0 + r0 + tid] = r;
        }
        __syncthreads();
      }
    }
    // the node's children in order and their terms (wave 0)
    if (wave == 0) {
      const bool kid = acc < gamma && lane < T_ && lane > u && s_par[lane] == u;
      const uint64_t km = __ballot(kid);
      const int rank = __popcll(km & ((1ull << lane) - 1ull));
      if (kid && rank < kMaxTopK) {
        const int x = s_tok[lane];
        s_e[rank] = x >= 0 && x < V ? (double)expf(s * DT<T>::ld(row + x) - M) : 0.0;
        s_x[rank] = x;
        s_v[rank] = lane;
      }
      if (lane == 0) s_nk = min(__popcll(km), kMaxTopK);
    }
    __syncthreads();
    if (tid == 0) {
      double S = 0.0;
      for (int k = 0; k < G; ++k) S += s_rt[k];
      double rem = S;
      int nex = 0, nxt = -1;
      for (int i = 0; i < s_nk; ++i) {
        if ((double)s_dr[i] < s_e[i] / rem) { nxt = s_v[i]; break; }
        rem -= s_e[i];
        s_excl[nex++] = s_x[i];
      }
      s_nex = nex;
      s_next = nxt;
      s_pick = -1;
      if (nxt < 0) {
        // residual mass per round; the round holding the target
        for (int i = 0; i < nex; ++i) {
          const int x = s_excl[i];
          if (x >= 0 && x < V) {
            const int k = (x / VEC) / NT;
            s_rt[k] = fmax(s_rt[k] - s_e[i], 0.0);
          }
        }
        double tot = 0.0;
        for (int k = 0; k < G; ++k) tot += s_rt[k];
        const double target = (double)s_dr[kDraws - 1] * tot;
        double pre = 0.0, pre_k = 0.0;
        int kk = -1;
        for (int k = 0; k < G; ++k) {
          if (s_rt[k] > 0.0) {
            kk = k;
            pre_k = pre;
            if (target < pre + s_rt[k]) break;   // else: rounding past the end
          }
          pre += s_rt[k];
        }
        s_round = kk;
        s_tgt = target - pre_k;
      }
    }
    __syncthreads();
    const int nxt = s_next;
    if (nxt >= 0) {   // every thread follows the walk
      if (tid == 0) {
        out[acc] = s_tok[nxt];
        path[acc + 1] = nxt;
      }
      ++acc;
      u = nxt;
      __syncthreads();
      continue;
    }
    // inverse CDF inside the chosen round
    const int kk = s_round;
    int pick = -1;
    if (kk >= 0) {
      const int nex = s_nex;
      const int q = kk * NT + tid;
      const u32x4 g = q < NQ ? fetch_granule<T>(row, q, nvec, V, aligned) : ninf;
      double e[VEC];
      double part = 0.0;
      int last = -1;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int y = q * VEC + j;
        const float v = s * DT<T>::elem(g, j);
        bool ex = q >= NQ || v == -INFINITY;
        for (int i = 0; i < nex; ++i) ex |= s_excl[i] == y;
        e[j] = ex ? 0.0 : (double)expf(v - M);
        part += e[j];
        if (e[j] > 0.0) last = y;
      }
      // intervals [end of thread t-1, end of thread t) tile [0, round total)
      double inc = part;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double xo = __shfl_up(inc, o, 64);
        if (lane >= o) inc += xo;
      }
      int lastw = last;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) lastw = max(lastw, __shfl_xor(lastw, o, 64));
      if (lane == 63) s_pre[wave] = inc;
      if (lane == 0) s_last[wave] = lastw;
      __syncthreads();
      double before = 0.0, total = 0.0;
      int lastb = -1;
      for (int w = 0; w < NW; ++w) {
        if (w == wave) before = total;
        total += s_pre[w];
        lastb = max(lastb, s_last[w]);
      }
      const double end = before + inc;
      double start = __shfl_up(end, 1, 64);
      if (lane == 0) start = before;
      const double target = s_tgt;
      if (part > 0.0 && start <= target && target < end) {
        double c = start;
        int pk = -1;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          c += e[j];
          if (pk < 0 && e[j] > 0.0 && c > target) pk = q * VEC + j;
        }
        s_pick = pk >= 0 ? pk : last;
      }
      __syncthreads();
      pick = s_pick >= 0 ? s_pick : lastb;   // target at or past the round total (rounding)
    }
    // No residual mass left in fp32 (the rejected children held all of it,
    // e.g. a near-one-hot row): the last child tried is the token; a row with
    // no finite probability at all emits token 0.
    if (pick < 0) pick = s_nex > 0 ? s_excl[s_nex - 1] : 0;
    if (pick >= V) pick = V - 1;
    if (tid == 0) {
      out[acc] = pick;
      accept_len[b] = acc;
    }
    return;
  }
}

bool verify_sample_ok(int vocab, int dtype) {
  const int vec = dtype == EAGLE_BF16 ? 8 : 4;
  return vocab >= 1 && (int64_t)vocab <= (int64_t)kMaxRounds * kSampleThreads * vec;
}

template <typename T>
static void launch_sample_t(const TreeDev& t, int B, const T* logits, int positions, int vocab,
                            float inv_temp, const float* draws, int gamma, int32_t* accept_len,
                            int32_t* accept_path, int32_t* out_tokens, hipStream_t st) {
  hipLaunchKernelGGL((k_verify_sample<T, 4>), dim3(B), dim3(kSampleThreads), 0, st, t, logits,
                     positions, vocab, inv_temp, draws, gamma, accept_len, accept_path, out_tokens);
}

void launch_verify_sample(const TreeDev& t, int B, const void* logits, int positions, int vocab,
                          int dtype, float inv_temp, const float* draws, int gamma,
                          int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
                          hipStream_t st) {
  if (dtype == EAGLE_BF16)
    launch_sample_t(t, B, (const bf16s*)logits, positions, vocab, inv_temp, draws, gamma,
                    accept_len, accept_path, out_tokens, st);
  else
    launch_sample_t(t, B, (const float*)logits, positions, vocab, inv_temp, draws, gamma,
                    accept_len, accept_path, out_tokens, st);
}

// ---------------------------------- stochastic verification of sampled drafts
// Multi-round speculative sampling when drafting drew each node's children
// without replacement from the draft q = softmax(s_d * z_draft): at a visited
// node u the drawn children x_1 .. x_k (pool order = draw order, including
// children the verify tree dropped) are tested one after another.  With
// p = softmax(s_t * z_target), the j-th test uses the draft's proposal
// distribution for the j-th draw, q_j = q over the tokens not drawn before x_j,
// renormalised, and the residual r_j (r_1 = p; after a rejection
// r_{j+1} = max(r_j - q_j, 0) renormalised); x_j is kept iff
// u_j < r_j(x_j) / q_j(x_j).
//
// Closed form used here (exact in real arithmetic): a rejected token has
// r_j(x_j) < q_j(x_j), so it keeps no residual mass, and for every other token
//   C_{j+1} r_{j+1}(y) = max(p(y) - K_j exp(l_y - m_j), 0),
// with l_y = fp32(s_d * z_y), m_j the largest l over the tokens not drawn
// before x_j, E_j = sum of exp(l - m_j) over those tokens,
// K_j = K_{j-1} exp(m_j - m_{j-1}) + C_j / E_j (K_0 = 0), C_1 = 1 and C_{j+1} the
// residual mass.  So one pass over the vocabulary per rejection gives C_{j+1};
// the test of x_{j+1} needs only scalars.  m_j <= m_{j-1} and E_j >= 1 keep
// every factor within [0, 16].
//
// Granule = 4 ids; round k = granules [k * NT, (k + 1) * NT), granule
// k * NT + t read by thread t.  Per element: fp32 scaled logits and expf;
// granule sums in fp32; above that fp64 in a fixed order (bit-reproducible).
// A bitmap over granules in LDS marks those holding a drawn token, so only
// their elements are compared against the drawn ids.
constexpr int kDrThreads = 1024;
constexpr int kDrWaves = kDrThreads / 64;
constexpr int kDrMaxRounds = 128;                            // vocabularies up to 2^19 ids
constexpr int kDrBitmapWords = kDrMaxRounds * kDrThreads / 32;

template <typename T>
__device__ __forceinline__ void ld4(const T* row, int q, int V, bool aligned, float (&f)[4]);

template <>
__device__ __forceinline__ void ld4<float>(const float* row, int q, int V, bool aligned,
                                           float (&f)[4]) {
  if (aligned && 4 * q + 4 <= V) {
    const u32x4 w = ld16(row + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = 4 * q + e < V ? row[4 * q + e] : -INFINITY;
}

template <>
__device__ __forceinline__ void ld4<bf16s>(const bf16s* row, int q, int V, bool aligned,
                                           float (&f)[4]) {
  if (aligned && 4 * q + 4 <= V) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + 4 * q);
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xffff0000u);
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = 4 * q + e < V ? bf2f(row[4 * q + e]) : -INFINITY;
}

template <typename T>
__global__ __launch_bounds__(kDrThreads) void k_verify_drafted(
    TreeDev t, const T* logits, const float* dlog, int positions, int V, float s_t, float s_d,
    const float* draws, int gamma, DraftRows dr, int32_t* accept_len, int32_t* accept_path,
    int32_t* out_tokens) {
  constexpr int NT = kDrThreads, NW = kDrWaves;
  __shared__ uint32_t s_bm[kDrBitmapWords];
  __shared__ double s_wr[NW][kDrMaxRounds];
  __shared__ double s_rt[kDrMaxRounds];
  __shared__ double s_acc[NW][2];
  __shared__ float s_mx[NW][2];
  __shared__ int s_fnode[kMaxPos];
  __shared__ float s_dr[kDraws];
  __shared__ int s_x[kMaxTopK], s_v[kMaxTopK], s_j[kMaxTopK];
  __shared__ float s_lx[kMaxTopK], s_ex[kMaxTopK];
  __shared__ int s_nk, s_bad, s_row, s_pick;
  __shared__ double s_pre[NW];
  __shared__ int s_last[NW];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = gridDim.x;
  const int T_ = min(t.f_count[b], kMaxPos);
  const int fb = b * kMaxPos;
  const int cap = t.pool_cap;
  const int cnt = min(t.pool_count[b], cap);
  const int NQ = (V + 3) / 4;
  const int G = (NQ + NT - 1) / NT;
  int32_t* path = accept_path + (int64_t)b * (gamma + 1);
  int32_t* out = out_tokens + (int64_t)b * (gamma + 1);
  if (tid <= gamma) { path[tid] = tid == 0 ? 0 : -1; out[tid] = -1; }
  if (t.status[b] != 0 || T_ < 1) {
    if (tid == 0) {
      path[0] = -1;
      accept_len[b] = -1;
    }
    return;
  }
  if (tid < kMaxPos) s_fnode[tid] = tid < T_ ? t.f_node[fb + tid] : -1;
  for (int i = tid; i < kDrBitmapWords; i += NT) s_bm[i] = 0u;
  __syncthreads();

  int u = 0, acc = 0;
  while (true) {
    // (a) the drawn children of u in pool order, and u's uniforms (wave 0)
    if (wave == 0) {
      const int node = s_fnode[u];
      const bool bad = node < 0 || node >= cnt;
      int nk = 0;
      if (!bad && acc < gamma) {
        for (int base = 0; base < cnt; base += 64) {
          const int j = base + lane;
          const bool kid = j < cnt && t.pool_parent[b * cap + j] == node;
          const uint64_t km = __ballot(kid);
          const int rank = nk + __popcll(km & ((1ull << lane) - 1ull));
          if (kid && rank < kMaxTopK) {
            s_j[rank] = j;
            s_x[rank] = t.pool_tok[b * cap + j];
          }
          nk += __popcll(km);
        }
        nk = min(nk, kMaxTopK);
      }
      if (lane == 0) {
        s_nk = nk;
        s_bad = bad;
      }
      if (lane < kDraws) s_dr[lane] = draws[((int64_t)b * positions + u) * kDraws + lane];
    }
    __syncthreads();
    const int nk = s_nk;
    if (wave == 0 && nk > 0) {
      // verify position of each drawn child (-1: dropped from the tree)
      for (int i = 0; i < nk; ++i) {
        const uint64_t m = __ballot(lane < T_ && s_fnode[lane] == s_j[i]);
        if (lane == 0) s_v[i] = m ? (int)__ffsll((unsigned long long)m) - 1 : -1;
      }
      if (lane == 0) {
        // the draft row of u: step depth(u), row b * rows + (slot - first slot of that step)
        const int node = s_fnode[u];
        const int slot = t.pool_slot[b * cap + node], d = t.pool_depth[b * cap + node];
        int row = -1;
        if (d >= 0 && d < dr.n) {
          int first = 0;
          for (int s = 0; s < d; ++s) first += dr.rows[s];
          if (slot >= first && slot < first + dr.rows[d])
            row = B * first + b * dr.rows[d] + (slot - first);
        }
        s_row = row;
        if (row < 0) s_bad = 1;
      }
      if (lane < nk) {
        const int x = s_x[lane];
        if (x < 0 || x >= V) s_bad = 1;
        else atomicOr(&s_bm[(x >> 2) >> 5], 1u << ((x >> 2) & 31));
      }
    }
    __syncthreads();
    if (s_bad) {       // inconsistent tree state: nothing to verify
      if (tid <= gamma) { path[tid] = -1; out[tid] = -1; }
      if (tid == 0) accept_len[b] = -1;
      return;
    }
    const T* row = logits + ((int64_t)b * positions + u) * V;
    const bool al = (reinterpret_cast<uintptr_t>(row) & (sizeof(T) * 4 - 1)) == 0;
    const float* drow = nk > 0 ? dlog + (int64_t)s_row * V : dlog;
    const bool dal = (reinterpret_cast<uintptr_t>(drow) & 15) == 0;

    // (b) maxima: M_t over the target's scaled logits, M_r over the draft's
    // for the tokens not drawn; the drawn tokens' draft logits to LDS
    float mt = -INFINITY, mr = -INFINITY;
    for (int r = 0; r < G; ++r) {
      const int q = r * NT + tid;
      if (q >= NQ) break;
      float f[4];
      ld4<T>(row, q, V, al, f);
#pragma unroll
      for (int e = 0; e < 4; ++e) mt = fmaxf(mt, __fmul_rn(s_t, f[e]));
      if (nk > 0) {
        float g[4];
        ld4<float>(drow, q, V, dal, g);
        const bool fl = (s_bm[q >> 5] >> (q & 31)) & 1u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float l = __fmul_rn(s_d, g[e]);
          bool ex = false;
          if (fl)
            for (int i = 0; i < nk; ++i)
              if (s_x[i] == 4 * q + e) {
                ex = true;
                s_lx[i] = l;
              }
          if (!ex) mr = fmaxf(mr, l);
        }
      }
    }
    mt = wave_max(mt);
    mr = wave_max(mr);
    if (lane == 0) {
      s_mx[wave][0] = mt;
      s_mx[wave][1] = mr;
    }
    __syncthreads();
    float Mt = s_mx[0][0], Mr = s_mx[0][1];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      Mt = fmaxf(Mt, s_mx[w][0]);
      Mr = fmaxf(Mr, s_mx[w][1]);
    }

    // (c) S = sum exp(s_t z - M_t) (per round when u has no drawn child: the
    // residual is then p itself), R = sum over the undrawn tokens of
    // exp(l - M_r); the drawn tokens' target terms to LDS
    {
      double sa = 0.0, ra = 0.0;
      for (int r = 0; r < G; ++r) {
        const int q = r * NT + tid;
        float gs = 0.f, gr = 0.f;
        if (q < NQ) {
          float f[4];
          ld4<T>(row, q, V, al, f);
          const bool fl = (s_bm[q >> 5] >> (q & 31)) & 1u;
          float g[4];
          if (nk > 0) ld4<float>(drow, q, V, dal, g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float et = expf(__fsub_rn(__fmul_rn(s_t, f[e]), Mt));
            gs += et;
            if (nk > 0) {
              bool ex = false;
              if (fl)
                for (int i = 0; i < nk; ++i)
                  if (s_x[i] == 4 * q + e) {
                    ex = true;
                    s_ex[i] = et;
                  }
              if (!ex) gr += expf(__fsub_rn(__fmul_rn(s_d, g[e]), Mr));
            }
          }
        }
        if (nk == 0) {
          if (r * NT < NQ) {     // wave-uniform: every lane takes part in the butterfly
            const double w = wave_sum_d((double)gs);
            if (lane == 0) s_wr[wave][r] = w;
          }
        } else {
          sa += (double)gs;
          ra += (double)gr;
        }
      }
      if (nk > 0) {
        sa = wave_sum_d(sa);
        ra = wave_sum_d(ra);
        if (lane == 0) {
          s_acc[wave][0] = sa;
          s_acc[wave][1] = ra;
        }
      }
    }
    __syncthreads();
    if (nk == 0 && tid < G) {
      double r = 0.0;
      for (int w = 0; w < NW; ++w) r += s_wr[w][tid];
      s_rt[tid] = r;
    }
    double S = 0.0, R = 0.0;
    if (nk > 0)
      for (int w = 0; w < NW; ++w) {
        S += s_acc[w][0];
        R += s_acc[w][1];
      }
    __syncthreads();

    // (d) the tests, every thread computing the same scalars
    int take = -1, nex = 0;
    double C = 1.0, K = 0.0, mprev = 0.0;
    float Kf = 0.f, mf = 0.f;
    const float invS = (float)(1.0 / S);
    for (int j = 0; j < nk; ++j) {
      double m = (double)Mr;                    // -inf when every token was drawn
      for (int i = j; i < nk; ++i) m = fmax(m, (double)s_lx[i]);
      double E = R > 0.0 ? R * exp((double)Mr - m) : 0.0;
      for (int i = j; i < nk; ++i) E += exp((double)s_lx[i] - m);
      const double Kj = j == 0 ? 0.0 : K * exp(m - mprev);
      const double ex = exp((double)s_lx[j] - m);
      const double A = fmax((double)s_ex[j] / S - Kj * ex, 0.0);
      if ((double)s_dr[j] * C * (ex / E) < A) {
        take = j;
        break;
      }
      K = Kj + C / E;
      mprev = m;
      nex = j + 1;
      Kf = (float)K;
      mf = (float)m;
      // C_{j+2}: the residual mass after rejecting x_1 .. x_{j+1}; per round for
      // the last child (its totals serve the residual draw)
      const bool fin = j == nk - 1;
      double ca = 0.0;
      for (int r = 0; r < G; ++r) {
        const int q = r * NT + tid;
        float gs = 0.f;
        if (q < NQ) {
          float f[4], g[4];
          ld4<T>(row, q, V, al, f);
          ld4<float>(drow, q, V, dal, g);
          const bool fl = (s_bm[q >> 5] >> (q & 31)) & 1u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float et = expf(__fsub_rn(__fmul_rn(s_t, f[e]), Mt));
            const float ed = expf(__fsub_rn(__fmul_rn(s_d, g[e]), mf));
            float tm = fmaxf(__fsub_rn(__fmul_rn(et, invS), __fmul_rn(Kf, ed)), 0.f);
            if (fl)
              for (int i = 0; i < nex; ++i)
                if (s_x[i] == 4 * q + e) tm = 0.f;
            gs += tm;
          }
        }
        if (fin) {
          if (r * NT < NQ) {
            const double w = wave_sum_d((double)gs);
            if (lane == 0) s_wr[wave][r] = w;
          }
        } else {
          ca += (double)gs;
        }
      }
      if (!fin) {
        ca = wave_sum_d(ca);
        if (lane == 0) s_acc[wave][0] = ca;
      }
      __syncthreads();
      if (fin) {
        if (tid < G) {
          double r = 0.0;
          for (int w = 0; w < NW; ++w) r += s_wr[w][tid];
          s_rt[tid] = r;
        }
      } else {
        C = 0.0;
        for (int w = 0; w < NW; ++w) C += s_acc[w][0];
      }
      __syncthreads();
    }

    if (take >= 0) {
      const int x = s_x[take], v = s_v[take];
      if (tid == 0) {
        out[acc] = x;
        if (v >= 0) path[acc + 1] = v;
        else accept_len[b] = acc;
      }
      if (tid < nk) atomicAnd(&s_bm[(s_x[tid] >> 2) >> 5], ~(1u << ((s_x[tid] >> 2) & 31)));
      __syncthreads();
      if (v < 0) return;          // a dropped child: its token ends the walk
      ++acc;
      u = v;
      continue;
    }

    // (e) residual draw by inverse CDF over token ids, from the round totals
    double tot = 0.0;
    for (int k = 0; k < G; ++k) tot += s_rt[k];
    const double target = (double)s_dr[kDraws - 1] * tot;
    int kk = -1;
    double pre = 0.0, pre_k = 0.0;
    for (int k = 0; k < G; ++k) {
      if (s_rt[k] > 0.0) {
        kk = k;
        pre_k = pre;
        if (target < pre + s_rt[k]) break;        // else: rounding past the end
      }
      pre += s_rt[k];
    }
    int pick = -1;
    if (kk >= 0) {
      if (tid == 0) s_pick = -1;
      const int q = kk * NT + tid;
      double e[4];
      double part = 0.0;
      int last = -1;
      {
        float f[4], g[4];
        if (q < NQ) {
          ld4<T>(row, q, V, al, f);
          if (nk > 0) ld4<float>(drow, q, V, dal, g);
        }
        const bool fl = q < NQ && ((s_bm[q >> 5] >> (q & 31)) & 1u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float tm = 0.f;
          if (q < NQ) {
            const float et = expf(__fsub_rn(__fmul_rn(s_t, f[j]), Mt));
            if (nk == 0) {
              tm = et;
            } else {
              const float ed = expf(__fsub_rn(__fmul_rn(s_d, g[j]), mf));
              tm = fmaxf(__fsub_rn(__fmul_rn(et, invS), __fmul_rn(Kf, ed)), 0.f);
              if (fl)
                for (int i = 0; i < nex; ++i)
                  if (s_x[i] == 4 * q + j) tm = 0.f;
            }
          }
          e[j] = (double)tm;
          part += e[j];
          if (tm > 0.f) last = 4 * q + j;
        }
      }
      double inc = part;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double xo = __shfl_up(inc, o, 64);
        if (lane >= o) inc += xo;
      }
      int lastw = last;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) lastw = max(lastw, __shfl_xor(lastw, o, 64));
      if (lane == 63) s_pre[wave] = inc;
      if (lane == 0) s_last[wave] = lastw;
      __syncthreads();
      double before = 0.0, total = 0.0;
      int lastb = -1;
      for (int w = 0; w < NW; ++w) {
        if (w == wave) before = total;
        total += s_pre[w];
        lastb = max(lastb, s_last[w]);
      }
      const double end = before + inc;
      double start = __shfl_up(end, 1, 64);
      if (lane == 0) start = before;
      const double tg = target - pre_k;
      if (part > 0.0 && start <= tg && tg < end) {
        double c = start;
        int pk = -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c += e[j];
          if (pk < 0 && e[j] > 0.0 && c > tg) pk = 4 * q + j;
        }
        s_pick = pk >= 0 ? pk : last;
      }
      __syncthreads();
      pick = s_pick >= 0 ? s_pick : lastb;
    }
    // no residual mass left (or no finite term): the last child tried, else token 0
    if (pick < 0) pick = nk > 0 ? s_x[nk - 1] : 0;
    if (pick >= V) pick = V - 1;
    if (tid == 0) {
      out[acc] = pick;
      accept_len[b] = acc;
    }
    return;
  }
}

bool verify_drafted_ok(int vocab) {
  return vocab >= 1 && (int64_t)vocab <= (int64_t)kDrMaxRounds * kDrThreads * 4;
}

void launch_verify_drafted(const TreeDev& t, int B, const void* logits, const float* draft_logits,
                           int positions, int vocab, int dtype, float inv_temp, float draft_inv_temp,
                           const float* draws, int gamma, const DraftRows& dr, int32_t* accept_len,
                           int32_t* accept_path, int32_t* out_tokens, hipStream_t st) {
  if (dtype == EAGLE_BF16)
    hipLaunchKernelGGL(k_verify_drafted<bf16s>, dim3(B), dim3(kDrThreads), 0, st, t,
                       (const bf16s*)logits, draft_logits, positions, vocab, inv_temp,
                       draft_inv_temp, draws, gamma, dr, accept_len, accept_path, out_tokens);
  else
    hipLaunchKernelGGL(k_verify_drafted<float>, dim3(B), dim3(kDrThreads), 0, st, t,
                       (const float*)logits, draft_logits, positions, vocab, inv_temp,
                       draft_inv_temp, draws, gamma, dr, accept_len, accept_path, out_tokens);
}

// Commit of the accepted path's keys and values: request b's path positions
// accept_path[b][0 .. accept_len[b]] (root first) of the tree K/V
// ([B][64][row_bytes]) are copied to rows dst_row[b] + i of the destination
// cache; rows outside [0, dst_rows) and positions outside [0, 64) are
// skipped.  One workgroup per (request, path index), 16-byte copies.
__global__ void k_kv_commit(int gamma, int row_bytes, const int32_t* accept_len,
                            const int32_t* accept_path, const char* k_tree, const char* v_tree,
                            const int32_t* dst_row, int64_t dst_rows, char* k_dst, char* v_dst) {
  const int b = blockIdx.y, i = blockIdx.x;
  const int acc = accept_len[b];
  if (i > acc || i > gamma) return;
  const int u = accept_path[(int64_t)b * (gamma + 1) + i];
  const int64_t r = (int64_t)dst_row[b] + i;
  if (u < 0 || u >= kMaxPos || r < 0 || r >= dst_rows) return;
  const int64_t src = ((int64_t)b * kSlots + u) * row_bytes;
  const int64_t dst = r * row_bytes;
  for (int o = threadIdx.x * 16; o < row_bytes; o += blockDim.x * 16) {
    *reinterpret_cast<u32x4*>(k_dst + dst + o) = *reinterpret_cast<const u32x4*>(k_tree + src + o);
    *reinterpret_cast<u32x4*>(v_dst + dst + o) = *reinterpret_cast<const u32x4*>(v_tree + src + o);
  }
}

void launch_kv_commit(int B, int gamma, int row_bytes, const int32_t* accept_len,
                      const int32_t* accept_path, const void* k_tree, const void* v_tree,
                      const int32_t* dst_row, int64_t dst_rows, void* k_dst, void* v_dst,
                      hipStream_t st) {
  hipLaunchKernelGGL(k_kv_commit, dim3(gamma + 1, B), dim3(128), 0, st, gamma, row_bytes,
                     accept_len, accept_path, (const char*)k_tree, (const char*)v_tree, dst_row,
                     dst_rows, (char*)k_dst, (char*)v_dst);
}

// dense rows of the verify tree (row m = b * positions + u)
__global__ void k_tree_rows_final(TreeDev t, int B, int32_t* tok_idx, int32_t* kv_idx,
                                  int32_t* pos, uint64_t* mask) {
  const int u = threadIdx.x, b = blockIdx.x;
  const int T = t.positions;
  if (u >= T) return;
  const int m = b * T + u;
  const int fb = b * kMaxPos + u;
  const bool live = u < t.f_count[b];
  tok_idx[m] = live ? t.f_tok[fb] : 0;
  kv_idx[m] = b * kSlots + u;
  pos[m] = live ? t.f_pos[fb] : 0;
  mask[m] = live ? t.f_mask[fb] : 0ull;
}

void launch_tree_rows_final(const TreeDev& t, int B, int32_t* tok_idx, int32_t* kv_idx,
                            int32_t* pos, uint64_t* mask, hipStream_t st) {
  hipLaunchKernelGGL(k_tree_rows_final, dim3(B), dim3(64), 0, st, t, B, tok_idx, kv_idx, pos, mask);
}

}  // namespace eagle
