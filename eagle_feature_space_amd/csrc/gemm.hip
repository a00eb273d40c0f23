// Weight-streaming GEMM for the draft head's linear maps, and the epilogues
// that follow it (residual + norm, RoPE + K/V scatter, SwiGLU / GELU).
//
// The draft step runs M = B * rows-per-request <= a few hundred rows through
// matrices of d x 2d ... ffn x d ("What is actually in the head": an fc of
// shape [2d, d] and one decoder layer of width d).  At M <= 80 every weight
// byte is used M times, far below the MFMA ridge, so the kernel is built to
// stream W from HBM once: each wave owns 16*NB output columns, loads its W
// rows straight from global memory into registers (16 B per lane, the four
// lanes of a row reading 64 contiguous bytes) and multiplies them against the
// activation chunk staged once per workgroup in LDS.  Split-K over grid.z
// gives the launch enough waves; partial sums go to an fp32 workspace that
// the epilogue kernels reduce in a fixed order (bit-reproducible).
#include "kernels.h"
#include "stream.h"

namespace eagle {

template <typename T, int MB, int NB>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int KC = 32 * VEC;                 // K elements per chunk
  constexpr int MT = 16 * MB;                  // rows per workgroup
  constexpr int ROWB = KC * (int)sizeof(T) + 16;
  __shared__ __attribute__((aligned(16))) char xl[MT * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n_base = (blockIdx.x * 4 + wave) * (16 * NB);
  const int m0 = blockIdx.y * MT;
  const int k_begin = blockIdx.z * a.kps;
  const int k_end = min(a.K, k_begin + a.kps);

  const T* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int n = min(n_base + nb * 16 + c, a.N - 1);
    const T* base;
    int off;
    if (n < a.nseg1) { base = (const T*)a.w[0]; off = 0; }
    else if (n < a.nseg2) { base = (const T*)a.w[1]; off = a.nseg1; }
    else { base = (const T*)a.w[2]; off = a.nseg2; }
    wrow[nb] = base + (int64_t)(n - off) * a.K;
  }

  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = k_begin; k0 < k_end; k0 += KC) {
    const int L = min(KC, k_end - k0);         // multiple of 4*VEC
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
      if (m < a.M) {
        const int k = k0 + j * VEC;
        if (k < a.ksplit_x) v = ld16(row_ptr<T>(a.xs[0], m) + k);
        else v = ld16(row_ptr<T>(a.xs[1], m) + (k - a.ksplit_x));
      }
      st16(xl + r * ROWB + j * 16, v);
    }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < U) {
        u32x4 xf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xf[mb] = ld16(xl + (mb * 16 + c) * ROWB + (u * 4 * VEC + g * VEC) * (int)sizeof(T));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = DT<T>::mma(wv[nb][u], xf[mb], acc[nb][mb]);
      }
    }
  }

  // acc[nb][mb]: lane holds out[m = m0 + 16mb + c][n = n_base + 16nb + 4g + 0..3]
  float* P = a.P + (int64_t)blockIdx.z * a.M * a.N;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n_base + nb * 16 + 4 * g;
    if (n >= a.N) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 16 + c;
      if (m < a.M) *reinterpret_cast<f32x4*>(P + (int64_t)m * a.N + n) = acc[nb][mb];
    }
  }
}

template <typename T, int MB, int NB>
__global__ __launch_bounds__(256) void k_gemm_direct(GemmArgs a) {
  constexpr int U = 4;
  // the wave index is uniform across the wave: in a scalar register, loops
  // bounded by it stay scalar loops
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int n_base = (blockIdx.x * 4 + wave) * (16 * NB);
  if (n_base >= a.N) return;
  const int k_begin = blockIdx.z * a.kps;
  const int k_end = min(a.K, k_begin + a.kps);
  const T* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = min(n_base + nb * 16 + c, a.N - 1);
    const T* base;
    int off;
    if (n < a.nseg1) { base = (const T*)a.w[0]; off = 0; }
    else if (n < a.nseg2) { base = (const T*)a.w[1]; off = a.nseg1; }
    else { base = (const T*)a.w[2]; off = a.nseg2; }
    wrow[nb] = base + (int64_t)(n - off) * a.K;
  }
  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  direct_mainloop<T, MB, NB, U>(a, wrow, k_begin, k_end, g, c, acc);
  float* P = a.P + (int64_t)blockIdx.z * a.M * a.N;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n_base + nb * 16 + 4 * g;
    if (n >= a.N) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + c;
      if (m < a.M) *reinterpret_cast<f32x4*>(P + (int64_t)m * a.N + n) = acc[nb][mb];
    }
  }
}

// 17..32 rows: the workgroup's 4 waves share one K range, so the activation
// rows of each batch of U MFMA steps are staged once in LDS (double buffer)
// and read by all four waves, while each wave streams its own 32 weight rows
// through registers (double buffer); one barrier per batch.  Without the
// sharing every wave re-reads all 32 activation rows from L2 (as many bytes
// as its weights).  Rows past M re-read row M-1 (never stored).
template <typename T, int MB, int NB, int U>
__global__ __launch_bounds__(256) void k_gemm_shared(GemmArgs a) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int KS = 4 * VEC;                  // K of one MFMA step
  constexpr int STEP = U * KS;
  constexpr int MT = 16 * MB;
  constexpr int ROWB = STEP * (int)sizeof(T) + 16;
  constexpr int PIECES = STEP / VEC;           // 16-byte pieces per row and batch
  constexpr int PT = (MT * PIECES + 255) / 256;
  __shared__ __attribute__((aligned(16))) char xl[2][MT * ROWB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n_base = (blockIdx.x * 4 + wave) * (16 * NB);
  const int k_begin = blockIdx.z * a.kps;
  const int k_end = min(a.K, k_begin + a.kps);
  const T* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = min(n_base + nb * 16 + c, a.N - 1);
    const T* base;
    int off;
    if (n < a.nseg1) { base = (const T*)a.w[0]; off = 0; }
    else if (n < a.nseg2) { base = (const T*)a.w[1]; off = a.nseg1; }
    else { base = (const T*)a.w[2]; off = a.nseg2; }
    wrow[nb] = base + (int64_t)(n - off) * a.K;
  }
  // this thread's staging pieces: row r, 16-byte piece j of the batch
  const T* xrow0[PT];
  const T* xrow1[PT];
  int xj[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int p = min(tid + 256 * i, MT * PIECES - 1);
    xj[i] = p % PIECES;
    const int m = min(p / PIECES, a.M - 1);
    xrow0[i] = row_ptr<T>(a.xs[0], m);
    xrow1[i] = a.xs[1].base ? row_ptr<T>(a.xs[1], m) : xrow0[i];
  }
  auto stage = [&](int k, int len, int buf) {
    u32x4 v[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int p = tid + 256 * i;
      const int kk = k + xj[i] * VEC;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (p < MT * PIECES && xj[i] * VEC < len)
        v[i] = ld16(kk < a.ksplit_x ? xrow0[i] + kk : xrow1[i] + (kk - a.ksplit_x));
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int p = tid + 256 * i;
      if (p < MT * PIECES) st16(xl[buf] + (p / PIECES) * ROWB + xj[i] * 16, v[i]);
    }
  };
  u32x4 wa[U][NB], wb[U][NB];
  auto ldw = [&](int k, int len, u32x4(&w)[U][NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u * KS < len)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) w[u][nb] = ld16(wrow[nb] + k + u * KS + g * VEC);
  };
  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const u32x4(&w)[U][NB], int len, int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u * KS < len) {
        u32x4 xf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xf[mb] = ld16(xl[buf] + (mb * 16 + c) * ROWB + (u * KS + g * VEC) * (int)sizeof(T));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = DT<T>::mma(w[u][nb], xf[mb], acc[nb][mb]);
      }
    }
  };
  // batches of STEP (the last one shorter: K spans are whole MFMA steps);
  // the control flow is the same in every wave of the workgroup
  int k = k_begin, buf = 0;
  if (k < k_end) {
    int len = min(STEP, k_end - k);
    stage(k, len, 0);
    ldw(k, len, wa);
    __syncthreads();
    while (true) {
      const int k2 = k + len;
      const int len2 = min(STEP, k_end - k2);
      if (len2 > 0) { stage(k2, len2, buf ^ 1); ldw(k2, len2, wb); }
      mma(wa, len, buf);
      __syncthreads();
      k = k2; len = len2; buf ^= 1;
      if (len <= 0) break;
      const int k3 = k + len;
      const int len3 = min(STEP, k_end - k3);
      if (len3 > 0) { stage(k3, len3, buf ^ 1); ldw(k3, len3, wa); }
      mma(wb, len, buf);
      __syncthreads();
      k = k3; len = len3; buf ^= 1;
      if (len <= 0) break;
    }
  }
  if (n_base >= a.N) return;
  float* P = a.P + (int64_t)blockIdx.z * a.M * a.N;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n_base + nb * 16 + 4 * g;
    if (n >= a.N) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + c;
      if (m < a.M) *reinterpret_cast<f32x4*>(P + (int64_t)m * a.N + n) = acc[nb][mb];
    }
  }
}

// ----------------------------------------------------------------- planning
static int kc_of(int dtype) { return dtype == EAGLE_BF16 ? 256 : 128; }

GemmShape plan_gemm(int dtype, int M, int N, int K) {
  GemmShape s;
  if (big_gemm_ok(dtype, M, N, K)) return plan_gemm_big(M, N, K);
  // 17..63 rows: the 64-K-stage tiled GEMM streams 8 rows x 128 B per load
  // where the kernels below stream 16 rows x 64 B (8B-shaped projections:
  // 10-20% faster at 32 rows, 30-45% at 48)
  if (wide_rows_ok(dtype, M, N, K)) return plan_gemm_big(M, N, K);
  if (M > 16 && M <= 32) {
    // activation-sharing kernel: waves of 2 n-blocks (32 columns), ~2048
    // waves, K spans of whole MFMA steps
    s.direct = 3;
    s.MB = 2;
    s.mtiles = 1;
    s.NB = 2;
    const int wcols = (N + 31) / 32;
    s.ntiles = (wcols + 3) / 4;
    const int ks = dtype == EAGLE_BF16 ? 32 : 16;
    const int ksteps = (K + ks - 1) / ks;
    int S = (2048 + wcols - 1) / wcols;
    if (S > ksteps) S = ksteps;
    if (S < 1) S = 1;
    const int sps = (ksteps + S - 1) / S;
    s.kps = sps * ks;
    s.S = (K + s.kps - 1) / s.kps;
    return s;
  }
  if (M <= 32) {
    // direct kernel: waves of 2 n-blocks (32 columns); ~2048 waves, K spans
    // that are whole multiples of the 4-step unroll
    s.direct = 1;
    s.MB = (M + 15) / 16;
    s.mtiles = 1;
    s.NB = 2;
    const int wcols = (N + 31) / 32;
    s.ntiles = (wcols + 3) / 4;
    const int step = dtype == EAGLE_BF16 ? 128 : 64;
    const int ksteps = (K + step - 1) / step;
    int S = (2048 + wcols - 1) / wcols;
    if (S > ksteps) S = ksteps;
    if (S < 1) S = 1;
    const int sps = (ksteps + S - 1) / S;
    s.kps = sps * step;
    s.S = (K + s.kps - 1) / s.kps;
    return s;
  }
  s.direct = 0;
  s.MB = M >= 80 ? 5 : (M + 15) / 16;
  if (s.MB < 1) s.MB = 1;
  s.mtiles = (M + 16 * s.MB - 1) / (16 * s.MB);
  s.NB = N >= 4096 ? 2 : 1;
  s.ntiles = (N + 64 * s.NB - 1) / (64 * s.NB);
  const int kc = kc_of(dtype);
  const int esz = dtype == EAGLE_BF16 ? 2 : 4;
  const int kchunks = (K + kc - 1) / kc;
  int want = (1024 + s.ntiles * s.mtiles - 1) / (s.ntiles * s.mtiles);
  // keep the fp32 partial traffic under ~1/8 of the weight bytes
  int cap = (int)((int64_t)K * esz / (32 * (int64_t)M));
  if (cap < 1) cap = 1;
  int S = want < cap ? want : cap;
  if (S > kchunks) S = kchunks;
  if (S < 1) S = 1;
  int cps = (kchunks + S - 1) / S;
  s.kps = cps * kc;
  s.S = (K + s.kps - 1) / s.kps;
  return s;
}

template <typename T, int NB>
static void launch_mb(const GemmArgs& a, const GemmShape& s, hipStream_t st) {
  dim3 grid(s.ntiles, s.mtiles, s.S), block(256);
  switch (s.MB) {
    case 1: hipLaunchKernelGGL((k_gemm<T, 1, NB>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<T, 2, NB>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemm<T, 3, NB>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_gemm<T, 4, NB>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_gemm<T, 5, NB>), grid, block, 0, st, a); break;
  }
}

void launch_gemm(int dtype, GemmArgs a, const GemmShape& s, hipStream_t st) {
  a.kps = s.kps;
  if (s.direct == 2) {
    launch_gemm_big(a, s, st);
    return;
  }
  if (s.direct == 3) {
    dim3 grid(s.ntiles, 1, s.S), block(256);
    if (dtype == EAGLE_BF16) hipLaunchKernelGGL((k_gemm_shared<bf16s, 2, 2, 4>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_gemm_shared<float, 2, 2, 4>), grid, block, 0, st, a);
    return;
  }
  if (s.direct) {
    dim3 grid(s.ntiles, 1, s.S), block(256);
    if (dtype == EAGLE_BF16) hipLaunchKernelGGL((k_gemm_direct<bf16s, 1, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_gemm_direct<float, 1, 2>), grid, block, 0, st, a);
    return;
  }
  if (dtype == EAGLE_BF16) {
    if (s.NB == 2) launch_mb<bf16s, 2>(a, s, st); else launch_mb<bf16s, 1>(a, s, st);
  } else {
    if (s.NB == 2) launch_mb<float, 2>(a, s, st); else launch_mb<float, 1>(a, s, st);
  }
}

// ----------------------------------------------------------------- epilogues
// sum_{s < S} p[s * stride], added in order s = 0, 1, ...; the loads of a
// batch (sized to S: 2, 4, 8 or 16 partials) are issued together (indexes
// clamped into range, the clamped duplicates replaced by 0 before they are
// added), so the epilogues pay about one memory latency instead of S, without
// re-issuing loads when S is small.
template <int NB>
__device__ __forceinline__ float sum_parts_n(const float* p, int64_t stride, int S) {
  float y = 0.f;
  for (int s0 = 0; s0 < S; s0 += NB) {
    float v[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) v[q] = p[(int64_t)min(s0 + q, S - 1) * stride];
#pragma unroll
    for (int q = 0; q < NB; ++q) y += s0 + q < S ? v[q] : 0.f;
  }
  return y;
}
__device__ __forceinline__ float sum_parts(const float* p, int64_t stride, int S) {
  if (S <= 0) return 0.f;
  if (S <= 2) return sum_parts_n<2>(p, stride, S);
  if (S <= 4) return sum_parts_n<4>(p, stride, S);
  if (S <= 8) return sum_parts_n<8>(p, stride, S);
  return sum_parts_n<16>(p, stride, S);
}

// Row epilogue, column-parallel (one thread per column, grid = column blocks x
// rows, so even a single row spreads over many workgroups):
//   y = sum_s P[s][m] + src1[m] + src2[m]            (fp32, fixed order)
//   out / out_scatter = y (T); if a norm follows, y is kept in fp32 and each
//   block writes its partial (sum y, sum y^2) for the row statistics.
template <typename T>
__global__ __launch_bounds__(256) void k_rows_sum(ReduceArgs a) {
  __shared__ float red[2][4];
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const bool live = n < a.N;
  float y = 0.f;
  if (live) {
    if (a.P) y = sum_parts(a.P + (int64_t)m * a.N + n, (int64_t)a.M * a.N, a.S);
    if (a.src1.base) y += DT<T>::ld(row_ptr<T>(a.src1, m) + n);
    if (a.src2.base) y += DT<T>::ld(row_ptr<T>(a.src2, m) + n);
    if (a.out) DT<T>::st((T*)a.out + (int64_t)m * a.N + n, y);
    if (a.out_scatter.base)
      DT<T>::st((T*)a.out_scatter.base + (int64_t)a.out_scatter.idx[m] * a.out_scatter.stride + n, y);
    if (a.y32) a.y32[(int64_t)m * a.N + n] = y;
    if (a.out_g) DT<T>::st((T*)a.out_g + (int64_t)m * a.N + n, y * DT<T>::ld((const T*)a.gain + n));
  }
  if (!a.stats) return;
  float s1 = live ? y : 0.f, s2 = live ? y * y : 0.f;
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = s1;
    red[1][threadIdx.x >> 6] = s2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float* st = a.stats + ((int64_t)m * gridDim.x + blockIdx.x) * 2;
    st[0] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    st[1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

// out_norm = Norm(y) from the fp32 row and the per-block partial statistics
// (summed in block order): RMSNorm y / sqrt(mean(y^2) + eps) * g, or
// LayerNorm (y - mean) / sqrt(var + eps) * g + b with var = E[y^2] - mean^2.
template <typename T>
__global__ __launch_bounds__(256) void k_rows_norm(ReduceArgs a) {
  __shared__ float sh[2];
  __shared__ float2 part[256];
  const int m = blockIdx.y;
  const int nblk = gridDim.x;      // <= 256 (N <= 65536)
  const float* st = a.stats + (int64_t)m * nblk * 2;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const bool live = n < a.N;
  float y = 0.f, gn = 0.f, bs = 0.f;
  if (live) {
    y = a.y32[(int64_t)m * a.N + n];
    gn = DT<T>::ld((const T*)a.gain + n);
    if (a.bias) bs = DT<T>::ld((const T*)a.bias + n);
  }
  if (threadIdx.x < nblk) part[threadIdx.x] = *reinterpret_cast<const float2*>(st + 2 * threadIdx.x);
  __syncthreads();
  if (threadIdx.x == 0) {
    float s1 = 0.f, s2 = 0.f;
    for (int b = 0; b < nblk; ++b) {
      s1 += part[b].x;
      s2 += part[b].y;
    }
    const float mean = a.layer_norm ? s1 / a.N : 0.f;
    const float var = s2 / a.N - mean * mean;
    sh[0] = mean;
    sh[1] = 1.0f / sqrtf(fmaxf(var, 0.f) + a.eps);
  }
  __syncthreads();
  if (!live) return;
  float v = (y - sh[0]) * sh[1] * gn;
  if (a.bias) v += bs;
  DT<T>::st((T*)a.out_norm + (int64_t)m * a.N + n, v);
}

// Four columns per lane (16-byte fp32 / 8-byte bf16 accesses), one wave per
// (row, 256-column block), four rows per workgroup; same partial-sum order per
// element as k_rows_sum and the same per-block statistics layout.  Used for
// 64 rows and more when N and every row stride are multiples of 4 and the
// buffers 16-byte aligned.
template <typename T>
__device__ __forceinline__ f32x4 ld4(const T* p);
template <>
__device__ __forceinline__ f32x4 ld4<bf16s>(const bf16s* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4{bf2f(v.x & 0xffffu), bf2f(v.x >> 16), bf2f(v.y & 0xffffu), bf2f(v.y >> 16)};
}
template <>
__device__ __forceinline__ f32x4 ld4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <typename T>
__device__ __forceinline__ void st4(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void st4<bf16s>(bf16s* p, const f32x4& v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(f2bf(v[0]) | (f2bf(v[1]) << 16), f2bf(v[2]) | (f2bf(v[3]) << 16));
}
template <>
__device__ __forceinline__ void st4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename T>
__global__ __launch_bounds__(256) void k_rows_sum4(ReduceArgs a) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (m >= a.M) return;
  const int n = blockIdx.x * 256 + 4 * lane;
  const bool live = n < a.N;           // N % 4 == 0: all four columns or none
  f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
  if (live) {
    if (a.P && a.S > 0) {
      const float* p = a.P + (int64_t)m * a.N + n;
      const int64_t stride = (int64_t)a.M * a.N;
      constexpr int NB = 4;
      for (int s0 = 0; s0 < a.S; s0 += NB) {
        f32x4 v[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) v[q] = *reinterpret_cast<const f32x4*>(p + (int64_t)min(s0 + q, a.S - 1) * stride);
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += s0 + q < a.S ? v[q][e] : 0.f;
      }
    }
    if (a.src1.base) y += ld4<T>(row_ptr<T>(a.src1, m) + n);
    if (a.src2.base) y += ld4<T>(row_ptr<T>(a.src2, m) + n);
    if (a.out) st4<T>((T*)a.out + (int64_t)m * a.N + n, y);
    if (a.out_scatter.base)
      st4<T>((T*)a.out_scatter.base + (int64_t)a.out_scatter.idx[m] * a.out_scatter.stride + n, y);
    if (a.y32) *reinterpret_cast<f32x4*>(a.y32 + (int64_t)m * a.N + n) = y;
    if (a.out_g) st4<T>((T*)a.out_g + (int64_t)m * a.N + n, y * ld4<T>((const T*)a.gain + n));
  }
  if (!a.stats) return;
  float s1 = live ? (y[0] + y[1]) + (y[2] + y[3]) : 0.f;
  float s2 = live ? (y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]) : 0.f;
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (lane == 0) {
    float* st = a.stats + ((int64_t)m * gridDim.x + blockIdx.x) * 2;
    st[0] = s1;
    st[1] = s2;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_rows_norm4(ReduceArgs a, int nblk) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (m >= a.M) return;
  const int n = blockIdx.x * 256 + 4 * lane;
  const bool live = n < a.N;
  f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f}, gn = y, bs = y;
  if (live) {
    y = *reinterpret_cast<const f32x4*>(a.y32 + (int64_t)m * a.N + n);
    gn = ld4<T>((const T*)a.gain + n);
    if (a.bias) bs = ld4<T>((const T*)a.bias + n);
  }
  // the row's block statistics: lane l sums blocks l, l + 64, ... and the
  // wave reduces in a fixed butterfly order (all loads in flight at once;
  // every wave of the row forms the same sums)
  const float* st = a.stats + (int64_t)m * nblk * 2;
  float s1 = 0.f, s2 = 0.f;
  for (int b = lane; b < nblk; b += 64) {
    const float2 v = *reinterpret_cast<const float2*>(st + 2 * b);
    s1 += v.x;
    s2 += v.y;
  }
  s1 = __shfl(wave_sum(s1), 0, 64);   // lane 0's association for the whole row
  s2 = __shfl(wave_sum(s2), 0, 64);
  if (!live) return;
  const float mean = a.layer_norm ? s1 / a.N : 0.f;
  const float var = s2 / a.N - mean * mean;
  const float rs = 1.0f / sqrtf(fmaxf(var, 0.f) + a.eps);
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (y[e] - mean) * rs * gn[e];
    if (a.bias) v[e] += bs[e];
  }
  st4<T>((T*)a.out_norm + (int64_t)m * a.N + n, v);
}

static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
static bool rows4_ok(const ReduceArgs& a) {
  if (a.N % 4 != 0) return false;
  const RowSrc* rs[3] = {&a.src1, &a.src2, &a.out_scatter};
  for (const RowSrc* r : rs)
    if (r->base && (!al16(r->base) || r->stride % 4 != 0)) return false;
  const void* ps[7] = {a.P, a.out, a.y32, a.out_g, a.gain, a.bias, a.out_norm};
  for (const void* q : ps)
    if (q && !al16(q)) return false;
  return true;
}

void launch_reduce_rows(int dtype, const ReduceArgs& a0, hipStream_t st) {
  ReduceArgs a = a0;
  if (!a.out_norm && !a.keep_stats) a.stats = nullptr;
  if (!a.out_norm) a.y32 = nullptr;     // the fp32 rows only feed the norm kernels
  dim3 grid((a.N + 255) / 256, a.M);
  // few rows: one thread per column keeps more workgroups in flight
  if (a.M >= 64 && rows4_ok(a)) {
    const dim3 g4((a.N + 255) / 256, (a.M + 3) / 4);
    const int nblk = (a.N + 255) / 256;
    if (dtype == EAGLE_BF16) {
      hipLaunchKernelGGL(k_rows_sum4<bf16s>, g4, dim3(256), 0, st, a);
      if (a.out_norm) hipLaunchKernelGGL(k_rows_norm4<bf16s>, g4, dim3(256), 0, st, a, nblk);
    } else {
      hipLaunchKernelGGL(k_rows_sum4<float>, g4, dim3(256), 0, st, a);
      if (a.out_norm) hipLaunchKernelGGL(k_rows_norm4<float>, g4, dim3(256), 0, st, a, nblk);
    }
    return;
  }
  if (dtype == EAGLE_BF16) {
    hipLaunchKernelGGL(k_rows_sum<bf16s>, grid, dim3(256), 0, st, a);
    if (a.out_norm) hipLaunchKernelGGL(k_rows_norm<bf16s>, grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_rows_sum<float>, grid, dim3(256), 0, st, a);
    if (a.out_norm) hipLaunchKernelGGL(k_rows_norm<float>, grid, dim3(256), 0, st, a);
  }
}

// rstd of a row for a folded RMSNorm, from its per-block statistics [nblk][2]
// (sum, sum of squares): lane l sums blocks l, l + 64, ..., then a DPP wave
// reduction (wave-uniform result).  Every lane of the wave must call it for
// the same row.
__device__ __forceinline__ float row_rstd(const float* st, int nblk, int N, float eps) {
  const int lane = threadIdx.x & 63;
  float s2 = 0.f;
  for (int b = lane; b < nblk; b += 64) s2 += st[2 * b + 1];
  s2 = rows_sum(s2);
  return 1.0f / sqrtf(fmaxf(s2 / N, 0.f) + eps);
}

// RoPE + scatter of the fused q|k|v projection.  One thread per (row, head,
// four consecutive pairs i .. i + 3) rotates elements (i, i + hd/2) by
// pos * theta^(-2i/hd); the angle is formed and reduced in double precision
// (in revolutions: the hardware sine and cosine take revolutions).  Four
// pairs a thread: 16-byte partial loads, 8- or 16-byte stores, and the row's
// statistics, position and addresses formed once per four pairs.
template <int NB>
__device__ __forceinline__ f32x4 sum_parts4_n(const float* p, int64_t stride, int S) {
  f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += NB) {
    f32x4 v[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) v[q] = *reinterpret_cast<const f32x4*>(p + (int64_t)min(s0 + q, S - 1) * stride);
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] += s0 + q < S ? v[q][e] : 0.f;
  }
  return y;
}
__device__ __forceinline__ f32x4 sum_parts4(const float* p, int64_t stride, int S) {
  if (S <= 0) return f32x4{0.f, 0.f, 0.f, 0.f};
  if (S <= 2) return sum_parts4_n<2>(p, stride, S);
  if (S <= 4) return sum_parts4_n<4>(p, stride, S);
  if (S <= 8) return sum_parts4_n<8>(p, stride, S);
  return sum_parts4_n<16>(p, stride, S);
}

// four consecutive elements (8- or 16-byte aligned)
template <typename T>
__device__ __forceinline__ void qkv_store4(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void qkv_store4<bf16s>(bf16s* p, const f32x4& v) {
  uint2 o;
  o.x = f2bf(v[0]) | (f2bf(v[1]) << 16);
  o.y = f2bf(v[2]) | (f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = o;
}
template <>
__device__ __forceinline__ void qkv_store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename T>
__global__ __launch_bounds__(256) void k_epi_qkv(QkvArgs a) {
  // grid (quad blocks of a row, rows): the row and its position are uniform
  // across the workgroup, the (head, quad) index needs only 32-bit arithmetic
  const int half = a.hd / 2;
  const int quads = half / 4;            // quads of pairs per head
  const int heads = a.Hq + 2 * a.Hkv;
  const int t0 = blockIdx.x * 256 + threadIdx.x;
  const bool live = t0 < heads * quads;  // lanes past the last quad only help form rstd
  const int t = live ? t0 : 0;
  if (!a.xstats && !live) return;
  const int h = t / quads;
  const int i = (t % quads) * 4;
  const int N = heads * a.hd;
  const int c1 = h * a.hd + i, c2 = c1 + half;
  const int64_t pst = (int64_t)a.M * N;
  const bool is_v = h >= a.Hq + a.Hkv;
  const bool rope = !is_v && a.theta > 0.f;
  // the rotations' frequencies (revolutions per position) depend on the pair only
  double inv[4] = {0.0, 0.0, 0.0, 0.0};
  if (rope) {
    const double lt = log2((double)a.theta);
#pragma unroll
    for (int e = 0; e < 4; ++e) inv[e] = exp2(-(2.0 * (i + e) / a.hd) * lt) * 0.15915494309189535;
  }
  for (int m = blockIdx.y; m < a.M; m += gridDim.y) {
    f32x4 x1 = f32x4{0.f, 0.f, 0.f, 0.f}, x2 = x1;
    if (live) {      // partial loads first: the statistics load overlaps them
      x1 = sum_parts4(a.P + (int64_t)m * N + c1, pst, a.S);
      x2 = sum_parts4(a.P + (int64_t)m * N + c2, pst, a.S);
    }
    if (a.xstats) {
      const float rs = row_rstd(a.xstats + (int64_t)m * a.xnblk * 2, a.xnblk, a.xN, a.eps);
      x1 *= rs;
      x2 *= rs;
    }
    if (!live) continue;
    int pos;
    int64_t row = m;
    bool skip = false;
    if (a.pos) pos = a.pos[m];
    else {  // packed context rows: position inside the request
      // the last request b with cu_row[b] <= m, by bisection (the row is
      // uniform across the workgroup: a few scalar loads instead of up to B
      // dependent ones)
      int b = 0, hi = a.B;
      while (hi - b > 1) {
        const int mid = (b + hi) >> 1;
        if (a.cu_row[mid] <= m) b = mid;
        else hi = mid;
      }
      pos = m - a.cu_row[b];
      if (a.n_new) {
        const int nb = a.n[b];
        pos += nb - a.n_new[b];
        row = (int64_t)a.cu_n[b] + pos;
        skip = pos < 0 || pos >= nb || row >= a.total_rows;
      }
    }
    if (skip) continue;
    if (rope) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        double rev = (double)pos * inv[e];
        rev -= rint(rev);
        const float cs = __builtin_amdgcn_cosf((float)rev);
        const float sn = __builtin_amdgcn_sinf((float)rev);
        const float y1 = x1[e] * cs - x2[e] * sn;
        const float y2 = x2[e] * cs + x1[e] * sn;
        x1[e] = y1;
        x2[e] = y2;
      }
    }
    T* dst;
    if (h < a.Hq) {
      dst = (T*)a.q + ((int64_t)m * a.Hq + h) * a.hd;
    } else {
      const int kh = is_v ? h - a.Hq - a.Hkv : h - a.Hq;
      const int64_t r = a.kv_idx ? (int64_t)a.kv_idx[m] : row;
      dst = (T*)(is_v ? a.v : a.k) + (r * a.Hkv + kh) * a.hd;
    }
    qkv_store4<T>(dst + i, x1);
    qkv_store4<T>(dst + i + half, x2);
  }
}

void launch_epi_qkv(int dtype, const QkvArgs& a, hipStream_t st) {
  const int quads = (a.Hq + 2 * a.Hkv) * (a.hd / 8);
  // at most 2048 row slots: a workgroup takes every 2048th row, so the
  // rotation frequencies (double-precision exp2 / log2 per pair) are formed
  // once per ~M/2048 rows instead of once per row (the ~20k-row ingest)
  dim3 grid((unsigned)((quads + 255) / 256), (unsigned)std::min(a.M, 2048));
  if (a.M <= 0) return;
  if (dtype == EAGLE_BF16) hipLaunchKernelGGL(k_epi_qkv<bf16s>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_epi_qkv<float>, grid, dim3(256), 0, st, a);
}

// act = silu(gate) * up (SwiGLU) or gelu(up) (exact erf form)
template <typename T>
__global__ __launch_bounds__(256) void k_epi_act(ActArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)a.M * a.F) return;
  const int m = (int)(t / a.F), j = (int)(t % a.F);
  const int N = a.swiglu ? 2 * a.F : a.F;
  const int64_t pst = (int64_t)a.M * N;
  const float* row = a.P + (int64_t)m * N;
  const float usum = sum_parts(row + (a.swiglu ? a.F : 0) + j, pst, a.S);
  const float gsum = a.swiglu ? sum_parts(row + j, pst, a.S) : 0.f;
  float y;
  if (a.swiglu) y = gsum / (1.0f + expf(-gsum)) * usum;
  else y = 0.5f * usum * (1.0f + erff(usum * 0.70710678118654752f));
  DT<T>::st((T*)a.out + t, y);
}

// The same activation, four columns per thread (16-byte partial loads, one
// 8- or 16-byte store), grid (column blocks, rows): no 64-bit index division.
// Used from 64 rows when F is a multiple of 4 and the buffers 16-byte aligned.
template <typename T>
__global__ __launch_bounds__(256) void k_epi_act4(ActArgs a) {
  const int j = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int m = blockIdx.y;
  const bool live = j < a.F;
  const int N = a.swiglu ? 2 * a.F : a.F;
  const int64_t pst = (int64_t)a.M * N;
  const float* row = a.P + (int64_t)m * N;
  f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f}, gs = u;
  if (live) {      // partial loads first: the statistics load overlaps them
    for (int s = 0; s < a.S; ++s) {
      u += *reinterpret_cast<const f32x4*>(row + s * pst + (a.swiglu ? a.F : 0) + j);
      if (a.swiglu) gs += *reinterpret_cast<const f32x4*>(row + s * pst + j);
    }
  }
  if (a.xstats) {  // every lane takes part in the row's reduction
    const float rs = row_rstd(a.xstats + (int64_t)m * a.xnblk * 2, a.xnblk, a.xN, a.eps);
    u *= rs;
    gs *= rs;
  }
  if (!live) return;
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (a.swiglu) y[e] = gs[e] / (1.0f + expf(-gs[e])) * u[e];
    else y[e] = 0.5f * u[e] * (1.0f + erff(u[e] * 0.70710678118654752f));
  }
  st4<T>((T*)a.out + (int64_t)m * a.F + j, y);
}

// from 17 rows (M <= 16 takes the row-complete kernels): with it N2 is
// folded through gate|up, so no separate normalisation launch runs
bool epi_act4_ok(int M, int F, const void* P, const void* out) {
  return M > 16 && F % 4 == 0 && al16(P) && al16(out);
}

void launch_epi_act(int dtype, const ActArgs& a, hipStream_t st) {
  if (epi_act4_ok(a.M, a.F, a.P, a.out)) {
    const dim3 g4((a.F / 4 + 255) / 256, a.M);
    if (dtype == EAGLE_BF16) hipLaunchKernelGGL(k_epi_act4<bf16s>, g4, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(k_epi_act4<float>, g4, dim3(256), 0, st, a);
    return;
  }
  dim3 grid((unsigned)(((int64_t)a.M * a.F + 255) / 256));
  if (dtype == EAGLE_BF16) hipLaunchKernelGGL(k_epi_act<bf16s>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_epi_act<float>, grid, dim3(256), 0, st, a);
}

}  // namespace eagle
