// Frozen LM head with a fused softmax / top-k epilogue ("The recurrence,
// written out": the next token comes from softmax(LM_head(f')); "EAGLE-2":
// the confidences c are the softmax probabilities of the drafted tokens).
//
// logits = X W_LM^T with W_LM [V][d] is the largest byte mover of a draft step
// (|V| = 128256 rows of d bf16), and the logits themselves never need to
// reach HBM: each workgroup streams 256 vocabulary rows once (same register
// blocking as the weight-streaming GEMM), keeps its 256 x M logit tile on
// chip and emits, per row, the tile maximum, the tile sum of
// exp(s * (logit - max)) and the tile's top-k (logit desc, id asc).  A second
// kernel merges the ~|V|/256 tile partials of every row into the log-partition,
// the top-k ids and their confidences softmax(s * logits)[id].
#include "kernels.h"
#include "stream.h"

namespace eagle {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int MB, int NB, int WAVES = 4, bool GUMBEL = false>
__device__ __forceinline__ void lm_epilogue(const LmArgs& a, f32x4 (&acc)[NB][MB], int m0, char* lds);

template <typename T, int MB, bool GUMBEL = false>
__global__ __launch_bounds__(256) void k_lmhead(LmArgs a) {
  constexpr int NB = 4;
  constexpr int VEC = DT<T>::VEC;
  constexpr int KC = 32 * VEC;
  constexpr int MT = 16 * MB;
  constexpr int ROWB = KC * (int)sizeof(T) + 16;
  constexpr int XBYTES = MT * ROWB;
  constexpr int TROW = 256 + 4;                      // fp32 logit tile row (padded)
  constexpr int TBYTES = 16 * TROW * 4;
  constexpr int LBYTES = XBYTES > TBYTES ? XBYTES : TBYTES;
  __shared__ __attribute__((aligned(16))) char lds[LBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int tile = blockIdx.x;
  const int n_base = tile * 256 + wave * 64;
  const int m0 = blockIdx.y * MT;

  const T* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = min(n_base + nb * 16 + c, a.V - 1);
    wrow[nb] = (const T*)a.w + (int64_t)n * a.K;
  }
  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < a.K; k0 += KC) {
    const int L = min(KC, a.K - k0);
    const int U = L / (4 * VEC);
    u32x4 wv[NB][8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (u < U) wv[nb][u] = ld16(wrow[nb] + k0 + u * 4 * VEC + g * VEC);
    __syncthreads();
    const int pieces = L / VEC;
    for (int p = tid; p < MT * pieces; p += 256) {
      const int r = p / pieces, j = p - r * pieces;
      const int m = m0 + r;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (m < a.M) v = ld16(row_ptr<T>(a.x, m) + k0 + j * VEC);
      st16(lds + r * ROWB + j * 16, v);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < U) {
        u32x4 xf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xf[mb] = ld16(lds + (mb * 16 + c) * ROWB + (u * 4 * VEC + g * VEC) * (int)sizeof(T));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = DT<T>::mma(wv[nb][u], xf[mb], acc[nb][mb]);
      }
    }
  }

  lm_epilogue<T, MB, NB, 4, GUMBEL>(a, acc, m0, lds);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64-bit multiplies and a word permutation, the key bumped by the Weyl
// constants after each round.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Standard Gumbel variable of vocabulary id `id` in the row with key `rk`:
// u = ((bits >> 9) + 0.5) 2^-23 in (0, 1), G = -log(-log(u)), fp32.
__device__ __forceinline__ float gumbel_of(const LmArgs& a, uint32_t rk, int id) {
  const uint4 w = philox4x32_10(make_uint4((uint32_t)id >> 2, rk, 0u, 0u), a.seed_lo, a.seed_hi);
  const uint32_t sel = id & 3;
  const uint32_t bits = sel == 0 ? w.x : (sel == 1 ? w.y : (sel == 2 ? w.z : w.w));
  const float u = ((float)(bits >> 9) + 0.5f) * 1.1920928955078125e-07f;   // 2^-23
  return -logf(-logf(u));
}

__device__ __forceinline__ uint32_t row_key_of(const LmArgs& a, int m) {
  return (uint32_t)((m / a.rows_per_req) * 1024 + a.row_node[m]);
}

// Epilogue shared by both LM-head kernels: optional raw logits, then per row
// the tile max, tile sum of exp(s (l - max)) and the tile top-k (by logit, or
// by the Gumbel key when drafting samples).
template <typename T, int MB, int NB, int WAVES, bool GUMBEL>
__device__ __forceinline__ void lm_epilogue(const LmArgs& a, f32x4 (&acc)[NB][MB], int m0, char* lds) {
  constexpr int TCOLS = 16 * NB * WAVES;  // tile columns (WAVES waves x 16*NB)
  constexpr int TROW = TCOLS + 4;
  constexpr int PER = TCOLS / 64;         // tile columns per lane in the row pass
  constexpr int RPW = 16 / WAVES;         // rows of a 16-row block per wave in the row pass
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int tile = blockIdx.x;
  const int n_base = tile * TCOLS + wave * 16 * NB;
  // optional raw logits (parity checks)
  if (a.logits) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + mb * 16 + c;
        const int n = n_base + nb * 16 + 4 * g;
        if (m >= a.M) continue;
        float* dst = a.logits + (int64_t)m * a.V + n;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < a.V) dst[i] = acc[nb][mb][i];
      }
  }

  // epilogue, one 16-row block at a time through LDS
  float* tl = reinterpret_cast<float*>(lds);
  const float sl = a.inv_temp * kLog2e;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wave * 16 * NB + nb * 16 + 4 * g;
      f32x4 v = acc[nb][mb];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tile * TCOLS + col + i >= a.V) v[i] = -INFINITY;
      *reinterpret_cast<f32x4*>(tl + c * TROW + col) = v;
    }
    __syncthreads();
    // rows dealt round-robin, so a few live rows still spread over the waves
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int r = rr * WAVES + wave;
      const int m = m0 + mb * 16 + r;
      if (m >= a.M) continue;
      float v[PER];
      int id[PER];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        v[j] = tl[r * TROW + lane + 64 * j];
        id[j] = tile * TCOLS + lane + 64 * j;
        mx = fmaxf(mx, v[j]);
      }
      mx = wave_max(mx);
      float se = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) se += exp2f((v[j] - mx) * sl);
      se = wave_sum(se);
      const int64_t pi = (int64_t)tile * a.M + m;
      if (lane == 0) {
        a.part_max[pi] = mx;
        a.part_sum[pi] = se;
      }
      // sampled drafting: rank by the Gumbel key s * logit + G instead
      if constexpr (GUMBEL) {
        const uint32_t rk = row_key_of(a, m);
#pragma unroll
        for (int j = 0; j < PER; ++j)
          v[j] = v[j] == -INFINITY ? -INFINITY : __fadd_rn(__fmul_rn(a.inv_temp, v[j]), gumbel_of(a, rk, id[j]));
      }
      // top-k: round k takes the best entry strictly worse than round k-1's
      float pv = INFINITY;
      int pid = -1;
      for (int k = 0; k < a.top_k; ++k) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const bool below = better(pv, pid, v[j], id[j]);
          if (below && better(v[j], id[j], bv, bi)) { bv = v[j]; bi = id[j]; }
        }
        wave_best(bv, bi);
        if (lane == 0) {
          a.part_val[pi * a.top_k + k] = bv;
          a.part_id[pi * a.top_k + k] = bi;
          if constexpr (GUMBEL) {
            const int col = bi - tile * TCOLS;
            a.part_logit[pi * a.top_k + k] = col >= 0 && col < TCOLS ? tl[r * TROW + col] : -INFINITY;
          }
        }
        pv = bv;
        pid = bi;
      }
    }
  }
}

// M <= 32: barrier-free streaming main loop (see k_gemm_direct), full K per
// wave, 128 vocabulary rows per wave (eight 16-row MFMA blocks share each X
// fragment and keep 32 KB of W loads in flight per wave), 512 per workgroup.
template <typename T, int MB, bool GUMBEL = false, int NB = 8, int U = 2, int WAVES = 4>
__global__ __launch_bounds__(64 * WAVES) void k_lmhead_direct(LmArgs a) {
  constexpr int TCOLS = 16 * NB * WAVES;
  constexpr int TBYTES = 16 * (TCOLS + 4) * 4;
  __shared__ __attribute__((aligned(16))) char lds[TBYTES];
  // the wave index is uniform across the wave: in a scalar register, loops
  // bounded by it stay scalar loops
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int n_base = blockIdx.x * TCOLS + wave * 16 * NB;
  const T* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = min(n_base + nb * 16 + c, a.V - 1);
    wrow[nb] = (const T*)a.w + (int64_t)n * a.K;
  }
  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  GemmArgs ga;
  ga.xs[0] = a.x;
  ga.xs[1] = RowSrc{nullptr, nullptr, 0, 0};
  ga.ksplit_x = a.K;
  ga.M = a.M;
  ga.N = a.V;
  ga.K = a.K;
  direct_mainloop<T, MB, NB, U>(ga, wrow, 0, a.K, g, c, acc);
  lm_epilogue<T, MB, NB, WAVES, GUMBEL>(a, acc, 0, lds);
}

LmShape plan_lmhead(int dtype, int M, int V) {
  (void)dtype;
  LmShape s;
  s.MB = M >= 80 ? 5 : (M + 15) / 16;
  if (s.MB < 1) s.MB = 1;
  s.mtiles = (M + 16 * s.MB - 1) / (16 * s.MB);
  s.cols = M <= 32 ? 512 : 256;
  s.ntiles = (V + s.cols - 1) / s.cols;
  return s;
}

template <typename T, bool G>
static void launch_lm_t(const LmArgs& a, const LmShape& s, hipStream_t st) {
  dim3 grid(s.ntiles, s.mtiles), block(256);
  switch (s.MB) {
    case 1: hipLaunchKernelGGL((k_lmhead<T, 1, G>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_lmhead<T, 2, G>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_lmhead<T, 3, G>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_lmhead<T, 4, G>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_lmhead<T, 5, G>), grid, block, 0, st, a); break;
  }
}

template <typename T, bool G>
static void launch_direct_t(const LmArgs& a, const LmShape& s, hipStream_t st) {
  dim3 grid(s.ntiles, 1), block(256);
  if (a.M <= 16) hipLaunchKernelGGL((k_lmhead_direct<T, 1, G>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_lmhead_direct<T, 2, G>), grid, block, 0, st, a);
}

// the Gumbel-top-k epilogue is a separate instantiation, so the default one
// carries none of its code or registers
void launch_lmhead(int dtype, const LmArgs& a, const LmShape& s, hipStream_t st) {
  const bool bf = dtype == EAGLE_BF16;
  if (a.M <= 32) {
    if (a.gumbel) bf ? launch_direct_t<bf16s, true>(a, s, st) : launch_direct_t<float, true>(a, s, st);
    else bf ? launch_direct_t<bf16s, false>(a, s, st) : launch_direct_t<float, false>(a, s, st);
    return;
  }
  if (a.gumbel) bf ? launch_lm_t<bf16s, true>(a, s, st) : launch_lm_t<float, true>(a, s, st);
  else bf ? launch_lm_t<bf16s, false>(a, s, st) : launch_lm_t<float, false>(a, s, st);
}

// Tile partials from materialised logits (large M, after the MFMA-tiled GEMM):
// one wave per (row, 2048-column tile), same partial format as the fused
// epilogue: tile max, tile sum of exp(s (l - max)), tile top-k.
//
// The top-k works on 64-bit order keys: the float's bits mapped to an
// unsigned order (negative values flipped, -0 taken as +0, NaN lowest) above 11 bits of
// 2047 - column within the tile, so one unsigned compare is the (value desc,
// id asc) order and every key of a tile is distinct.  The wave reductions use
// DPP row moves (butterfly within each 16-lane row) and four lane reads
// instead of LDS permutes, which kept each wave waiting on LDS latency for
// every step of its top-k rounds.
constexpr int kLogitTile = 2048;

__device__ __forceinline__ uint64_t tile_key(float x, int col) {
  return ((uint64_t)float_order(x) << 11) | (uint32_t)(kLogitTile - 1 - col);
}
__device__ __forceinline__ float key_value(uint64_t k) { return order_float((uint32_t)(k >> 11)); }
__device__ __forceinline__ int key_col(uint64_t k) { return kLogitTile - 1 - (int)(k & (kLogitTile - 1)); }

template <int LD>   // sorted keys each lane keeps for the tile top-k
__global__ __launch_bounds__(256) void k_logits_partials(LmArgs a, const float* logits) {
  // lane owns columns 4 lane + 256 j + 0..3 (16-byte loads; V % 4 == 0 on this path)
  constexpr int PER = kLogitTile / 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int m = blockIdx.y * 4 + wave;
  if (m >= a.M) return;                 // whole waves: every DPP source lane is active
  const int c0 = tile * kLogitTile;
  const float* row = logits + (int64_t)m * a.V + c0;
  float v[PER][4];
  float mx = -INFINITY;
  const bool full = c0 + kLogitTile <= a.V;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    f32x4 t = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (full || c0 + 256 * j + 4 * lane < a.V) t = *reinterpret_cast<const f32x4*>(row + 256 * j + 4 * lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[j][e] = t[e];
      mx = fmaxf(mx, t[e]);
    }
  }
  mx = rows_max(mx);
  const float sl = a.inv_temp * kLog2e;
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) se += __builtin_amdgcn_exp2f((v[j][e] - mx) * sl);
  se = rows_sum(se);
  const int64_t pi = (int64_t)tile * a.M + m;
  if (lane == 0) {
    a.part_max[pi] = mx;
    a.part_sum[pi] = se;
  }
  if (a.gumbel) {   // sampled drafting: rank by s * logit + G
    const uint32_t rk = row_key_of(a, m);
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = c0 + 256 * j + 4 * lane + e;
        v[j][e] = v[j][e] == -INFINITY ? -INFINITY : __fadd_rn(__fmul_rn(a.inv_temp, v[j][e]), gumbel_of(a, rk, id));
      }
  }
  // Tile top-k in key order.  Every lane first keeps its own best LD keys,
  // sorted (an insertion network over its values); a round takes the wave's
  // largest head key and the owning lane drops it, which is the tile's next
  // entry as long as no lane has used all of its own.  Once one has, each
  // remaining round takes the largest key strictly below the previous winner
  // over all of the lanes' values.
  uint64_t kb[LD];
#pragma unroll
  for (int r = 0; r < LD; ++r) kb[r] = 0;    // below every real key
#pragma unroll
  for (int j = 0; j < PER; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // one element at a time (empty asm statements pin the order): with
      // every key formed ahead of the network, or the network run level by
      // level, 32 keys (64 registers) would be live at once
      float x = v[j][e];
      asm volatile("" : "+v"(x));
      uint64_t t = tile_key(x, 256 * j + 4 * lane + e);
#pragma unroll
      for (int r = 0; r < LD; ++r) {
        const bool c = t > kb[r];
        const uint64_t hi = c ? t : kb[r];
        t = c ? kb[r] : t;
        kb[r] = hi;
      }
#pragma unroll
      for (int r = 0; r < LD; ++r) asm volatile("" : "+v"(kb[r]));
    }
  int used = 0;
  uint64_t prev = ~0ull;
  for (int k = 0; k < a.top_k; ++k) {
    uint64_t w;
    if (!__builtin_amdgcn_ballot_w64(used >= LD)) {
      w = rows_umax64(kb[0]);
      if (kb[0] == w) {
#pragma unroll
        for (int r = 0; r + 1 < LD; ++r) kb[r] = kb[r + 1];
        kb[LD - 1] = 0;
        ++used;
      }
    } else {
      // rare: the values are read again (and re-keyed) rather than kept in
      // registers through the rounds
      const uint32_t rk = a.gumbel ? row_key_of(a, m) : 0u;
      uint64_t best = 0;
#pragma unroll 1
      for (int j = 0; j < PER; ++j) {
        f32x4 t = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (c0 + 256 * j + 4 * lane < a.V) t = *reinterpret_cast<const f32x4*>(row + 256 * j + 4 * lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = t[e];
          if (a.gumbel && x != -INFINITY)
            x = __fadd_rn(__fmul_rn(a.inv_temp, x), gumbel_of(a, rk, c0 + 256 * j + 4 * lane + e));
          const uint64_t q = tile_key(x, 256 * j + 4 * lane + e);
          if (q < prev) best = umax64(best, q);
        }
      }
      w = rows_umax64(best);
    }
    if (lane == 0) {
      // a padding column (past |V|, keyed as -inf) is only reached when the
      // tile holds fewer than top_k real ones or its logits are NaN; its id
      // is clamped so that no consumer indexes past the vocabulary
      const int bi = min(c0 + key_col(w), a.V - 1);
      a.part_val[pi * a.top_k + k] = key_value(w);
      a.part_id[pi * a.top_k + k] = bi;
      if (a.gumbel) a.part_logit[pi * a.top_k + k] = bi < a.V ? row[bi - c0] : -INFINITY;
    }
    prev = w;
  }
}

int logits_tiles(int V) { return (V + kLogitTile - 1) / kLogitTile; }

void launch_logits_partials(const LmArgs& a, const float* logits, hipStream_t st) {
  dim3 grid(logits_tiles(a.V), (a.M + 3) / 4);
  if (a.top_k > 4) hipLaunchKernelGGL(k_logits_partials<4>, grid, dim3(256), 0, st, a, logits);
  else hipLaunchKernelGGL(k_logits_partials<2>, grid, dim3(256), 0, st, a, logits);
}

// ---------------------------------------------------------------- merge
__device__ __forceinline__ void block_best(float& v, int& i, float* sv, int* si) {
  wave_best(v, i);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  v = sv[0];
  i = si[0];
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (better(sv[k], si[k], v, i)) { v = sv[k]; i = si[k]; }
}

constexpr int kMergeLds = 6144;   // candidates staged in LDS (48 KB)

template <int LD>   // sorted entries each lane keeps from the staged candidates
__global__ __launch_bounds__(256) void k_topk_merge(MergeArgs a) {
  // no fused multiply-adds here: with s * l and s * mx each rounded on its own
  // and log(z) >= 0, fl(s l) <= fl(s mx) <= lse for every logit l <= mx, so
  // each confidence exp(fl(s l) - lse) is at most 1 and path values never grow
  // (a contracted fma(s, l, -lse) returned 1.0000013 for near-certain rows)
#pragma clang fp contract(off)
  __shared__ float cval[kMergeLds];
  __shared__ int cid[kMergeLds];
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const float sl = a.inv_temp * kLog2e;
  // all loads first: the tile (max, sum) partials of this thread's tiles and
  // the candidates staged in LDS, so the row pays one memory latency
  const int ncand = a.ntiles * a.top_k;
  const bool staged = ncand <= kMergeLds;
  constexpr int TPT = 4;                  // tiles per thread held in registers
  float tm[TPT], ts[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int t = tid + 256 * i;
    tm[i] = -INFINITY;
    ts[i] = 0.f;
    if (t < a.ntiles) {
      tm[i] = a.part_max[(int64_t)t * a.M + m];
      ts[i] = a.part_sum[(int64_t)t * a.M + m];
    }
  }
  if (staged) {
    // eight candidates a thread in flight at once (a load-then-store loop
    // waits one memory latency per candidate)
    constexpr int SB = 8;
    for (int q0 = tid; q0 < ncand; q0 += 256 * SB) {
      float vv[SB];
      int vi[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int q = q0 + 256 * u;
        if (q < ncand) {
          const int t = q / a.top_k, j = q - t * a.top_k;
          const int64_t i = ((int64_t)t * a.M + m) * a.top_k + j;
          vv[u] = a.part_val[i];
          vi[u] = a.part_id[i];
        }
      }
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int q = q0 + 256 * u;
        if (q < ncand) {
          cval[q] = vv[u];
          cid[q] = vi[u];
        }
      }
    }
  }
  // log-partition of s * logits
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < TPT; ++i) mx = fmaxf(mx, tm[i]);
  for (int t = tid + 256 * TPT; t < a.ntiles; t += 256) mx = fmaxf(mx, a.part_max[(int64_t)t * a.M + m]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < TPT; ++i)
    if (tid + 256 * i < a.ntiles) z += ts[i] * exp2f((tm[i] - mx) * sl);
  for (int t = tid + 256 * TPT; t < a.ntiles; t += 256) {
    const int64_t i = (int64_t)t * a.M + m;
    z += a.part_sum[i] * exp2f((a.part_max[i] - mx) * sl);
  }
  z = wave_sum(z);
  if ((tid & 63) == 0) red[tid >> 6] = z;
  __syncthreads();
  z = red[0] + red[1] + red[2] + red[3];
  const float lse = a.inv_temp * mx + logf(z);
  if (staged) {
    // One wave takes the top-k from the staged candidates with no barrier per
    // round: each lane keeps its best LD, sorted; a round takes the best of
    // the lanes' next unused entries (exact while no lane has used all LD;
    // after that a lane rescans its candidates below the previous winner).
    // LD = 4 for top_k > 4: a lane holds ~ncand/64 candidates, and with two
    // of them two of a row's top-10 often share a lane, which sends every
    // later round to the rescans (one LDS latency per candidate).
    if (tid >= 64) return;
    float b[LD];
    int bi[LD], bq[LD];
#pragma unroll
    for (int r = 0; r < LD; ++r) {
      b[r] = -INFINITY;
      bi[r] = 0x7fffffff;
      bq[r] = -1;
    }
    // a lane owns whole parts (t = lane mod 64); every part lists its
    // candidates by value, descending, so a part is left at its first entry
    // below the lane's LD-th kept value
    for (int t = tid; t < a.ntiles; t += 64)
      for (int j = 0; j < a.top_k; ++j) {
        const int q = t * a.top_k + j;
        const float v = cval[q];
        const int id = cid[q];
        if (better(v, id, b[LD - 1], bi[LD - 1])) {
          // replace the last and let it bubble up (value desc, id asc)
          b[LD - 1] = v; bi[LD - 1] = id; bq[LD - 1] = q;
#pragma unroll
          for (int r = LD - 1; r > 0; --r)
            if (better(b[r], bi[r], b[r - 1], bi[r - 1])) {
              const float tv = b[r]; b[r] = b[r - 1]; b[r - 1] = tv;
              const int ti = bi[r]; bi[r] = bi[r - 1]; bi[r - 1] = ti;
              const int tq = bq[r]; bq[r] = bq[r - 1]; bq[r - 1] = tq;
            }
        } else if (v < b[LD - 1]) {
          break;
        }
      }
    int used = 0;
    float pv = INFINITY;
    int pid = -1;
    for (int k = 0; k < a.top_k; ++k) {
      float bv, lv;
      int bidx, li, lq;
      if (!__builtin_amdgcn_ballot_w64(used >= LD)) {
        lv = b[0];
        li = bi[0];
        lq = bq[0];
#pragma unroll
        for (int r = 1; r < LD; ++r)
          if (used == r) { lv = b[r]; li = bi[r]; lq = bq[r]; }
      } else {
        lv = -INFINITY;
        li = 0x7fffffff;
        lq = -1;
        for (int t = tid; t < a.ntiles; t += 64)
          for (int j = 0; j < a.top_k; ++j) {
            const int q = t * a.top_k + j;
            const float v = cval[q];
            const int id = cid[q];
            if (!better(pv, pid, v, id)) continue;   // taken already
            if (better(v, id, lv, li)) { lv = v; li = id; lq = q; }
            else if (v < lv) break;
          }
      }
      // (value desc, id asc) as one 64-bit key, reduced with DPP row moves
      const uint64_t lk = ((uint64_t)float_order(lv) << 32) | (0xffffffffu - (uint32_t)li);
      const uint64_t wk = rows_umax64(lk);
      bv = order_float((uint32_t)(wk >> 32));
      bidx = (int)(0xffffffffu - (uint32_t)wk);
      const bool mine = lq >= 0 && lk == wk;
      if (mine && used < LD) ++used;
      if (a.part_logit) {
        // Gumbel keys ranked the candidates; the confidence is the winner's
        // softmax probability, from its logit (the lane holding it writes)
        if (mine) {
          const int t = lq / a.top_k, j = lq - t * a.top_k;
          const int64_t i = ((int64_t)t * a.M + m) * a.top_k + j;
          a.topk_id[(int64_t)m * a.top_k + k] = bidx < 0 ? 0 : (bidx >= a.vocab ? a.vocab - 1 : bidx);
          a.topk_conf[(int64_t)m * a.top_k + k] = expf(a.inv_temp * a.part_logit[i] - lse);
        }
        if (tid == 0 && bidx == 0x7fffffff) {
          a.topk_id[(int64_t)m * a.top_k + k] = 0;
          a.topk_conf[(int64_t)m * a.top_k + k] = 0.f;
        }
      } else if (tid == 0) {
        // a NaN row leaves no candidate: keep ids inside the vocabulary
        a.topk_id[(int64_t)m * a.top_k + k] = bidx < 0 ? 0 : (bidx >= a.vocab ? a.vocab - 1 : bidx);
        a.topk_conf[(int64_t)m * a.top_k + k] = expf(a.inv_temp * bv - lse);
      }
      pv = bv;
      pid = bidx;
    }
    if (tid == 0) a.lse[m] = lse;
    return;
  }
  float pv = INFINITY;
  int pid = -1;
  for (int k = 0; k < a.top_k; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int q = tid; q < ncand; q += 256) {
      float v;
      int id;
      if (staged) { v = cval[q]; id = cid[q]; }
      else {
        const int t = q / a.top_k, j = q - t * a.top_k;
        const int64_t i = ((int64_t)t * a.M + m) * a.top_k + j;
        v = a.part_val[i];
        id = a.part_id[i];
      }
      if (better(pv, pid, v, id) && better(v, id, bv, bi)) { bv = v; bi = id; }
    }
    block_best(bv, bi, sv, si);
    if (a.part_logit) {
      // Gumbel keys ranked the candidates; the confidence is the winner's
      // softmax probability, from its logit (the thread holding it writes)
      for (int q = tid; q < ncand; q += 256) {
        const int t = q / a.top_k, j = q - t * a.top_k;
        const int64_t i = ((int64_t)t * a.M + m) * a.top_k + j;
        const float v = staged ? cval[q] : a.part_val[i];
        const int id = staged ? cid[q] : a.part_id[i];
        if (v == bv && id == bi) {
          a.topk_id[(int64_t)m * a.top_k + k] = bi < 0 ? 0 : (bi >= a.vocab ? a.vocab - 1 : bi);
          a.topk_conf[(int64_t)m * a.top_k + k] = expf(a.inv_temp * a.part_logit[i] - lse);
        }
      }
      if (tid == 0 && bi == 0x7fffffff) {
        a.topk_id[(int64_t)m * a.top_k + k] = 0;
        a.topk_conf[(int64_t)m * a.top_k + k] = 0.f;
      }
    } else if (tid == 0) {
      // a NaN row leaves no candidate: keep ids inside the vocabulary
      a.topk_id[(int64_t)m * a.top_k + k] = bi < 0 ? 0 : (bi >= a.vocab ? a.vocab - 1 : bi);
      a.topk_conf[(int64_t)m * a.top_k + k] = expf(a.inv_temp * bv - lse);
    }
    pv = bv;
    pid = bi;
  }
  if (tid == 0) a.lse[m] = lse;
}

void launch_topk_merge(const MergeArgs& a, hipStream_t st) {
  if (a.top_k > 4) hipLaunchKernelGGL(k_topk_merge<4>, dim3(a.M), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_topk_merge<2>, dim3(a.M), dim3(256), 0, st, a);
}

}  // namespace eagle
