// Row-complete streaming GEMM for the draft layer at M <= 16 rows.
//
// At a handful of rows every projection of the draft decoder layer is a pure
// weight stream, and what costs time besides the stream is the number of
// kernel boundaries (each drains the GPU and writes back its caches).  The
// split-K streaming kernel needs separate reduction, norm, RoPE and activation
// kernels after it; this one does not:
//   * a workgroup of 8 waves owns one 16-row block of W over the WHOLE of K;
//     its waves stream disjoint K ranges of those rows, double-buffered in
//     registers, and reduce their accumulators through LDS in wave order
//     (deterministic), so the epilogue sees final values;
//   * RMSNorm is folded through the projection: Norm(y) W^T = rstd(y) *
//     ((y * g) W^T), so the producer of y stores bf16(y * g) plus per-block
//     sums of y^2, and the consuming projection streams that operand as is and
//     scales its result rows by rstd (formed while its first weights load);
//   * a 16-row block may pair 8 rows with 8 rows a fixed distance away: the
//     two halves of a RoPE rotation (hd/2 apart) or a gate row with its up row
//     (F apart).  The accumulator of lane l holds block rows 4(l/16)..+3, so
//     the partner of lane l is lane l ^ 32, one shuffle away, and RoPE /
//     SwiGLU run in the epilogue.
// Lanes whose A row is past M re-read row M-1 (their results are never
// stored); every load is unconditional and nothing waits on one before the
// MFMAs that consume it, so the register double buffer stays full.  The row
// statistics are fetched with the first batch and only summed after the main
// loop; RoPE angles are formed while the stream runs.
#include "kernels.h"

namespace eagle {

constexpr int kRowsU = 4;       // MFMA steps per register batch
constexpr int kRowsWaves = 8;   // two workgroups per CU hide each other's reduction barrier
constexpr int kRowsStats = 16;  // statistics partials per lane (K <= 16384: <= 1024 blocks)

template <typename T>
__device__ __forceinline__ void store4(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void store4<bf16s>(bf16s* p, const f32x4& v) {
  uint2 o;
  o.x = f2bf(v[0]) | (f2bf(v[1]) << 16);
  o.y = f2bf(v[2]) | (f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = o;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename T, int EP, int WAVES = kRowsWaves, int U = kRowsU>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_rows(RowsArgs a) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int KS = 4 * VEC;            // K of one MFMA step
  constexpr int STEP = U * KS;
  __shared__ f32x4 red[WAVES][64];
  __shared__ float s_rstd[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int M = a.g.M, N = a.g.N, K = a.g.K;

  // W row of block row c (column of the product)
  int base, pair = 0;
  if constexpr (EP == EP_ROPE) {
    const int per = a.hd / 16;           // 8-pair blocks per head
    base = (blockIdx.x / per) * a.hd + (blockIdx.x % per) * 8;
    pair = a.hd / 2;
  } else if constexpr (EP == EP_SWIGLU) {
    base = blockIdx.x * 8;
    pair = a.act_F;
  } else {
    base = blockIdx.x * 16;
  }
  const T* wrow;
  {
    int n = EP == EP_ROPE || EP == EP_SWIGLU ? base + (c < 8 ? c : pair + c - 8) : base + c;
    n = min(n, N - 1);
    const T* b;
    int off;
    if (n < a.g.nseg1) { b = (const T*)a.g.w[0]; off = 0; }
    else if (n < a.g.nseg2) { b = (const T*)a.g.w[1]; off = a.g.nseg1; }
    else { b = (const T*)a.g.w[2]; off = a.g.nseg2; }
    wrow = b + (int64_t)(n - off) * K;
  }

  // this wave's K range (whole MFMA steps)
  const int kpw = ((K + WAVES - 1) / WAVES + KS - 1) / KS * KS;
  const int kb = min(K, wave * kpw), ke = min(K, kb + kpw);
  const int kfull = kb + (ke - kb) / STEP * STEP;

  const int m = min(c, M - 1);
  const T* x0 = row_ptr<T>(a.g.xs[0], m);
  const T* x1 = a.g.xs[1].base ? row_ptr<T>(a.g.xs[1], m) : x0;
  const int ksplit = a.g.ksplit_x;

  u32x4 wa[U], wb[U], xa[U], xb[U];
  auto ld = [&](int k, u32x4(&w)[U], u32x4(&x)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = ld16(wrow + k + u * KS + g * VEC);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + u * KS + g * VEC;
      x[u] = ld16(kk < ksplit ? x0 + kk : x1 + (kk - ksplit));
    }
  };

  // RoPE: the epilogue wave's position is fetched first
  int rpos = 0;
  if constexpr (EP == EP_ROPE) {
    if (wave == 0 && a.theta > 0.f) rpos = a.pos[m];
  }
  if (kb < kfull) ld(kb, wa, xa);
  // RMS row scale of the folded norm: wave r < M fetches row r's per-block
  // sums of squares now and adds them after the main loop (lanes strided,
  // then a butterfly: the same order in every workgroup)
  float sp[kRowsStats];
  const bool srow = a.xstats && wave < M;
  if (srow) {
    const float* st = a.xstats + (int64_t)wave * a.xnblk * 2;
#pragma unroll
    for (int j = 0; j < kRowsStats; ++j) {
      const int b = min(lane + 64 * j, a.xnblk - 1);
      sp[j] = st[2 * b + 1];
    }
  }
  // RoPE angles of the epilogue wave's pairs, pos * theta^(-2i/hd), formed and
  // range-reduced in double while the weights stream
  float rcs[4], rsn[4];
  if constexpr (EP == EP_ROPE) {
    if (wave == 0) {
      const int i0 = (blockIdx.x % (a.hd / 16)) * 8 + 4 * (g & 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rcs[r] = 1.f;
        rsn[r] = 0.f;
        if (a.theta > 0.f) {
          const double inv = exp2(-(2.0 * (i0 + r) / a.hd) * log2((double)a.theta));
          double ang = (double)rpos * inv;
          ang -= 6.283185307179586 * rint(ang / 6.283185307179586);
          sincosf((float)ang, &rsn[r], &rcs[r]);
        }
      }
    }
  }

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const u32x4(&w)[U], const u32x4(&x)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) acc = DT<T>::mma(w[u], x[u], acc);
  };
  int k = kb;
  if (k < kfull) {
    while (true) {
      if (k + STEP < kfull) ld(k + STEP, wb, xb);
      mma(wa, xa);
      k += STEP;
      if (k >= kfull) break;
      if (k + STEP < kfull) ld(k + STEP, wa, xa);
      mma(wb, xb);
      k += STEP;
      if (k >= kfull) break;
    }
  }
  for (; k < ke; k += KS) {   // tail, one MFMA step at a time
    const u32x4 w1 = ld16(wrow + k + g * VEC);
    const int kk = k + g * VEC;
    const u32x4 xv = ld16(kk < ksplit ? x0 + kk : x1 + (kk - ksplit));
    acc = DT<T>::mma(w1, xv, acc);
  }

  if (srow) {
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < kRowsStats; ++j) s2 += lane + 64 * j < a.xnblk ? sp[j] : 0.f;
    s2 = wave_sum(s2);
    if (lane == 0) s_rstd[wave] = 1.0f / sqrtf(s2 / K + a.eps);
    // rows past the wave count (fewer than 16 waves): same order, not prefetched
    for (int r = wave + WAVES; r < M; r += WAVES) {
      const float* st = a.xstats + (int64_t)r * a.xnblk * 2;
      float t2 = 0.f;
#pragma unroll
      for (int j = 0; j < kRowsStats; ++j) t2 += lane + 64 * j < a.xnblk ? st[2 * min(lane + 64 * j, a.xnblk - 1) + 1] : 0.f;
      t2 = wave_sum(t2);
      if (lane == 0) s_rstd[r] = 1.0f / sqrtf(t2 / K + a.eps);
    }
  }
  // reduce the waves' partial sums in wave order
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 s = red[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) s += red[w][lane];
  // lane holds product column (A row) c and block rows 4 g .. 4 g + 3
  const int mrow = c;
  const bool live = mrow < M;
  if (a.xstats) {
    const float r = s_rstd[m];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] *= r;
  }

  if constexpr (EP == EP_STORE) {
    const int n = base + 4 * g;
    f32x4 y = s;
    if (live) {
      if (a.res.base) {
        const T* r = row_ptr<T>(a.res, mrow) + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] += DT<T>::ld(r + i);
      }
      if (a.out) store4<T>((T*)a.out + (int64_t)mrow * N + n, y);
      if (a.scatter.base)
        store4<T>((T*)a.scatter.base + (int64_t)a.scatter.idx[mrow] * a.scatter.stride + n, y);
      if (a.out_g) {
        f32x4 yg;
#pragma unroll
        for (int i = 0; i < 4; ++i) yg[i] = y[i] * DT<T>::ld((const T*)a.gain + n + i);
        store4<T>((T*)a.out_g + (int64_t)mrow * N + n, yg);
      }
    }
    if (a.stats) {
      float s1 = live ? (y[0] + y[1]) + (y[2] + y[3]) : 0.f;
      float s2 = live ? (y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]) : 0.f;
      s1 = sum_x32(sum_x16(s1));
      s2 = sum_x32(sum_x16(s2));
      if (g == 0 && live) {
        float* st = a.stats + ((int64_t)mrow * gridDim.x + blockIdx.x) * 2;
        st[0] = s1;
        st[1] = s2;
      }
    }
  } else if constexpr (EP == EP_GELU) {
    if (!live) return;
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = 0.5f * s[i] * (1.0f + erff(s[i] * 0.70710678118654752f));
    store4<T>((T*)a.out + (int64_t)mrow * N + base + 4 * g, y);
  } else {
    // the partner value (other half of the pair) lives in lane ^ 32
    f32x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __shfl_xor(s[i], 32, 64);
    if (!live) return;
    const bool lo = g < 2;                 // lanes holding the first member
    const int j0 = 4 * (g & 1);            // pair index offset inside the 8-block
    if constexpr (EP == EP_SWIGLU) {
      if (!lo) return;
      f32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = s[i] / (1.0f + expf(-s[i])) * p[i];
      store4<T>((T*)a.out + (int64_t)mrow * a.act_F + base + j0, y);
    } else {
      const int per = a.hd / 16;
      const int head = blockIdx.x / per;
      const int i0 = (blockIdx.x % per) * 8 + j0;    // rotation pair index in the head
      const bool is_v = head >= a.Hq + a.Hkv;
      f32x4 y = s;
      if (!is_v && a.theta > 0.f) {
        // first member: x1 cos - x2 sin ; second: x2 cos + x1 sin
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = lo ? s[r] * rcs[r] - p[r] * rsn[r] : s[r] * rcs[r] + p[r] * rsn[r];
      }
      T* dst;
      if (head < a.Hq) {
        dst = (T*)a.q + ((int64_t)mrow * a.Hq + head) * a.hd;
      } else {
        const int kh = is_v ? head - a.Hq - a.Hkv : head - a.Hq;
        const int64_t r = a.kv_idx ? (int64_t)a.kv_idx[mrow] : (int64_t)mrow;
        dst = (T*)(is_v ? a.v : a.k) + (r * a.Hkv + kh) * a.hd;
      }
      store4<T>(dst + i0 + (lo ? 0 : a.hd / 2), y);
    }
  }
}

bool rows_gemm_ok(int M, int N, int K) {
  return M >= 1 && M <= 16 && N % 16 == 0 && K % 32 == 0;
}

template <typename T>
static void launch_rows_t(int ep, const RowsArgs& a, hipStream_t st) {
  const dim3 block(64 * kRowsWaves);
  switch (ep) {
    case EP_STORE:
      hipLaunchKernelGGL((k_gemm_rows<T, EP_STORE>), dim3(a.g.N / 16), block, 0, st, a);
      break;
    case EP_ROPE:
      hipLaunchKernelGGL((k_gemm_rows<T, EP_ROPE>), dim3(a.g.N / 16), block, 0, st, a);
      break;
    case EP_SWIGLU:
      hipLaunchKernelGGL((k_gemm_rows<T, EP_SWIGLU>), dim3(a.act_F / 8), block, 0, st, a);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_rows<T, EP_GELU>), dim3(a.g.N / 16), block, 0, st, a);
      break;
  }
}

void launch_gemm_rows(int dtype, int ep, const RowsArgs& a, hipStream_t st) {
  if (dtype == EAGLE_BF16) launch_rows_t<bf16s>(ep, a, st);
  else launch_rows_t<float>(ep, a, st);
}

}  // namespace eagle
