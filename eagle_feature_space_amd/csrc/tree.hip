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
}

void launch_tree_init(const TreeDev& t, int B, int eagle3, int vocab, const int32_t* root_tok,
                      const int32_t* n, const int32_t* cu_n, hipStream_t st) {
  hipLaunchKernelGGL(k_tree_init, dim3((B + 63) / 64), dim3(64), 0, st, t, B, eagle3, vocab,
                     root_tok, n, cu_n);
}

// key order: value desc, depth asc, index asc
__device__ __forceinline__ bool before(float va, int da, int ia, float vb, int db, int ib) {
  if (va != vb) return va > vb;
  if (da != db) return da < db;
  return ia < ib;
}

// `t` points its row_* arrays at the rows of this step; `nx` holds the row
// arrays of the next step (the other half of the double buffer): the two
// steps have different row counts per request, so writing in place would
// overwrite rows other workgroups have not read yet.
__global__ __launch_bounds__(256) void k_tree_expand(TreeDev t, RowsDev nx, int kind, int step,
                                                     int gamma, int W, int top_k, int top_m,
                                                     int final_step, StaticPlan plan) {
  __shared__ float sval[kPoolMax];
  __shared__ int sdep[kPoolMax];
  __shared__ int spar[kPoolMax];
  __shared__ int spos[kPoolMax];
  __shared__ int skeep[kPoolMax];
  __shared__ int snext[256];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = t.pool_cap;
  const int p0 = t.pool_count[b];
  const int nchild = kind == EAGLE_TREE_DYNAMIC ? W * top_k : plan.nchild;
  const int rp = t.root_pos[b];
  const int64_t pb = (int64_t)b * P;
  // a call out of order (pool or slots already full) must not write past them
  if (p0 < 1 || p0 + nchild > P) return;
  if (!final_step && t.slot_count[b] + (kind == EAGLE_TREE_DYNAMIC ? min(top_k, nchild) : plan.nnext) > kSlots)
    return;

  // 1. append the children of this step's rows
  for (int cidx = tid; cidx < nchild; cidx += 256) {
    int row, rank;
    if (kind == EAGLE_TREE_DYNAMIC) { row = cidx / top_k; rank = cidx % top_k; }
    else { row = plan.row[cidx]; rank = plan.rank[cidx]; }
    const int r = b * W + row;
    int parent = t.row_node[r];
    if (parent < 0 || parent >= p0) parent = 0;   // never reached with a consistent state
    const float conf = t.topk_conf[(int64_t)r * top_k + rank];
    const int node = p0 + cidx;
    t.pool_tok[pb + node] = t.topk_id[(int64_t)r * top_k + rank];
    t.pool_parent[pb + node] = parent;
    t.pool_depth[pb + node] = t.pool_depth[pb + parent] + 1;
    t.pool_slot[pb + node] = -1;
    t.pool_conf[pb + node] = conf;
    t.pool_value[pb + node] = __fmul_rn(t.pool_value[pb + parent], conf);
  }
  __syncthreads();
  __threadfence_block();
  const int pn = p0 + nchild;

  if (!final_step) {
    // 2. next frontier
    int nnext;
    if (kind == EAGLE_TREE_DYNAMIC) {
      nnext = min(top_k, nchild);
      for (int cidx = tid; cidx < nchild; cidx += 256) {
        const int u = p0 + cidx;
        const float vu = t.pool_value[pb + u];
        int rank = 0;
        for (int j = 0; j < nchild; ++j) {
          const int v = p0 + j;
          const float vv = t.pool_value[pb + v];
          if (vv > vu || (vv == vu && v < u)) ++rank;
        }
        if (rank < nnext) snext[rank] = u;
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

  // 3. rerank and verify tree
  for (int u = tid; u < pn; u += 256) {
    sval[u] = t.pool_value[pb + u];
    sdep[u] = t.pool_depth[pb + u];
    spar[u] = t.pool_parent[pb + u];
  }
  __syncthreads();
  for (int u = tid; u < pn; u += 256) {
    int keep;
    if (u == 0) keep = 1;
    else if (kind != EAGLE_TREE_DYNAMIC) keep = 1;
    else {
      int rank = 0;
      for (int v = 1; v < pn; ++v)
        if (before(sval[v], sdep[v], v, sval[u], sdep[u], u)) ++rank;
      keep = rank < top_m;
    }
    skeep[u] = keep;
  }
  __syncthreads();
  if (tid == 0) {   // positions in creation order
    int k = 0;
    for (int u = 0; u < pn; ++u) spos[u] = skeep[u] ? k++ : -1;
    t.f_count[b] = k;
    t.pool_count[b] = pn;
  }
  __syncthreads();
  for (int u = tid; u < pn; u += 256) {
    const int p = spos[u];
    if (p < 0) continue;
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
  hipLaunchKernelGGL(k_tree_expand, dim3(B), dim3(256), 0, st, t, next, kind, step, gamma, rows,
                     top_k, top_m, final_step, plan);
}

// ---------------------------------------------------------------- verify
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
        const float v = DT<T>::elem(x, e);
        const int j = q * VEC + e;
        if (better(v, j, bv, bi)) { bv = v; bi = j; }
      }
    }
  } else {
    for (int j = q0 * VEC + threadIdx.x; j < q1 * VEC; j += 256) {
      const float v = DT<T>::ld(row + j);
      if (better(v, j, bv, bi)) { bv = v; bi = j; }
    }
  }
  if (sp == kVerifySplits - 1)   // ragged tail past the last whole granule
    for (int j = nvec * VEC + threadIdx.x; j < V; j += 256) {
      const float v = DT<T>::ld(row + j);
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
__device__ __forceinline__ int verify_choice(const TreeDev& t, int b, int u) {
  const float2* p = t.choice_part + ((int64_t)b * kMaxPos + u) * kVerifySplits;
  float bv = p[0].x;
  int bi = __float_as_int(p[0].y);
  for (int s = 1; s < kVerifySplits; ++s) {
    const int i = __float_as_int(p[s].y);
    if (better(p[s].x, i, bv, bi)) { bv = p[s].x; bi = i; }
  }
  t.choice[b * kMaxPos + u] = bi;
  return bi;
}

__global__ void k_verify_walk(TreeDev t, int B, int gamma, int32_t* accept_len,
                              int32_t* accept_path, int32_t* out_tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int T = t.f_count[b];
  const int fb = b * kMaxPos;
  int32_t* path = accept_path + (int64_t)b * (gamma + 1);
  int32_t* out = out_tokens + (int64_t)b * (gamma + 1);
  for (int i = 0; i <= gamma; ++i) { path[i] = -1; out[i] = -1; }
  int u = 0, acc = 0;
  path[0] = 0;
  for (int it = 0; it <= gamma; ++it) {
    const int choice = verify_choice(t, b, u);
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
  hipLaunchKernelGGL(k_verify_walk, dim3((B + 63) / 64), dim3(64), 0, st, t, B, gamma, accept_len,
                     accept_path, out_tokens);
}

// ------------------------------------------------- stochastic verification
// Multi-round speculative sampling over the verify tree, one workgroup per
// request (the walk is sequential; only the rows it visits are read).  At a
// visited node u the target distribution is p(y) = e_y / S with
// v_y = fp32(s * z_y), M = max_y v_y, e_y = expf(v_y - M) and S the fp64 sum of
// the e_y.  Children of u are tried in verify-tree order: child i (token x) is
// kept iff draw[u][i] < e_x / (S - sum of e over the children rejected before
// it).  When none is kept (or u has no child, or u is at depth gamma) one
// token is drawn from p with the rejected tokens removed, by inverse CDF over
// token ids: the smallest x whose cumulative fp64 mass exceeds
// draw[u][16] * (total residual mass).  Each thread owns one contiguous range
// of token ids, so the cumulative sums follow id order: per-thread sums, a
// workgroup exclusive scan in thread order, then the one thread whose range
// holds the target walks it.  Every sum has a fixed order (deterministic).
constexpr int kSampleThreads = 512;
constexpr int kDraws = EAGLE_VERIFY_DRAWS;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void k_verify_sample(
    TreeDev t, const T* logits, int positions, int V, float s, const float* draws, int gamma,
    int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens) {
  constexpr int NW = kSampleThreads / 64;
  constexpr int VEC = DT<T>::VEC;
  __shared__ float s_max[NW];
  __shared__ double s_sum[NW];
  __shared__ double s_pre[NW];
  __shared__ int s_excl[kMaxTopK];
  __shared__ int s_nexcl, s_next, s_pick;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T_ = t.f_count[b];
  const int fb = b * kMaxPos;
  int32_t* path = accept_path + (int64_t)b * (gamma + 1);
  int32_t* out = out_tokens + (int64_t)b * (gamma + 1);
  if (tid <= gamma) { path[tid] = tid == 0 ? 0 : -1; out[tid] = -1; }
  // this thread's token ids [lo, hi), whole granules except at the row's end
  const int per = ((V + kSampleThreads - 1) / kSampleThreads + VEC - 1) / VEC * VEC;
  const int lo = min(V, tid * per), hi = min(V, lo + per);

  int u = 0, acc = 0;
  while (true) {
    const T* row = logits + ((int64_t)b * positions + u) * V;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    // visit this thread's values: f(y, v) for y in [lo, hi)
    auto each = [&](auto&& f) {
      int y = lo;
      if (aligned) {
        for (; y + VEC <= hi; y += VEC) {
          const u32x4 x = ld16(row + y);
#pragma unroll
          for (int e = 0; e < VEC; ++e) f(y + e, s * DT<T>::elem(x, e));
        }
      }
      for (; y < hi; ++y) f(y, s * DT<T>::ld(row + y));
    };
    // M = max v
    float m = -INFINITY;
    each([&](int, float v) { m = fmaxf(m, v); });
    m = wave_max(m);
    if (lane == 0) s_max[wave] = m;
    __syncthreads();
    float M = s_max[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_max[w]);
    // S = sum e (thread ranges, then waves, in order)
    double sm = 0.0;
    each([&](int, float v) { sm += (double)expf(v - M); });
    sm = wave_sum_d(sm);
    if (lane == 0) s_sum[wave] = sm;
    __syncthreads();
    if (tid == 0) {
      double S = 0.0;
      for (int w = 0; w < NW; ++w) S += s_sum[w];
      const float* dr = draws + ((int64_t)b * positions + u) * kDraws;
      double rem = S;
      int nex = 0, nxt = -1;
      if (acc < gamma) {
        for (int v = u + 1; v < T_ && nex < kMaxTopK; ++v) {
          if (t.f_parent[fb + v] != u) continue;
          const int x = t.f_tok[fb + v];
          // a token outside the target's vocabulary has no target mass
          const double e = x >= 0 && x < V ? (double)expf(s * DT<T>::ld(row + x) - M) : 0.0;
          if ((double)dr[nex] < e / rem) { nxt = v; break; }
          rem -= e;
          s_excl[nex++] = x;
        }
      }
      s_nexcl = nex;
      s_next = nxt;
      s_pick = -1;
    }
    __syncthreads();
    const int nxt = s_next;
    if (nxt >= 0) {   // every thread follows the walk
      if (tid == 0) {
        out[acc] = t.f_tok[fb + nxt];
        path[acc + 1] = nxt;
      }
      ++acc;
      u = nxt;
      __syncthreads();
      continue;
    }
    // residual draw at u: the rejected tokens carry no mass
    const int nex = s_nexcl;
    auto mass = [&](int y, float v) -> double {
      for (int i = 0; i < nex; ++i)
        if (s_excl[i] == y) return 0.0;
      return (double)expf(v - M);
    };
    double part = 0.0;
    each([&](int y, float v) { part += mass(y, v); });
    // prefix sums of the per-thread masses in thread order; thread t's
    // interval is [end of thread t-1, end of thread t), so the intervals tile
    // [0, total) exactly and one thread at most holds the target
    double inc = part;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double x = __shfl_up(inc, o, 64);
      if (lane >= o) inc += x;
    }
    if (lane == 63) s_pre[wave] = inc;
    __syncthreads();
    double before = 0.0, total = 0.0;
    for (int w = 0; w < NW; ++w) {
      if (w == wave) before = total;
      total += s_pre[w];
    }
    const double end = before + inc;
    double start = __shfl_up(end, 1, 64);
    if (lane == 0) start = before;
    const double target =
        (double)draws[((int64_t)b * positions + u) * kDraws + kDraws - 1] * total;
    if (part > 0.0 && start <= target && target < end) {
      double c = start;
      int pick = -1, last = -1;
      each([&](int y, float v) {
        if (pick >= 0) return;
        const double e = mass(y, v);
        if (e > 0.0) last = y;
        c += e;
        if (c > target && e > 0.0) pick = y;
      });
      s_pick = pick >= 0 ? pick : last;   // rounding at the range's end
    }
    __syncthreads();
    if (tid == 0) {
      int pick = s_pick;
      if (pick < 0) {  // target at or past the total (rounding): last token with mass
        for (int y = V - 1; y >= 0 && pick < 0; --y) {
          bool ex = false;
          for (int i = 0; i < nex; ++i) ex |= s_excl[i] == y;
          if (!ex) pick = y;
        }
      }
      out[acc] = pick;
      accept_len[b] = acc;
    }
    return;
  }
}

void launch_verify_sample(const TreeDev& t, int B, const void* logits, int positions, int vocab,
                          int dtype, float inv_temp, const float* draws, int gamma,
                          int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens,
                          hipStream_t st) {
  if (dtype == EAGLE_BF16)
    hipLaunchKernelGGL(k_verify_sample<bf16s>, dim3(B), dim3(kSampleThreads), 0, st, t,
                       (const bf16s*)logits, positions, vocab, inv_temp, draws, gamma, accept_len,
                       accept_path, out_tokens);
  else
    hipLaunchKernelGGL(k_verify_sample<float>, dim3(B), dim3(kSampleThreads), 0, st, t,
                       (const float*)logits, positions, vocab, inv_temp, draws, gamma, accept_len,
                       accept_path, out_tokens);
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
