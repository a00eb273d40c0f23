// Barrier-free register-streaming main loop shared by the GEMM and LM-head
// kernels (included by both translation units).
#pragma once
#include "kernels.h"

namespace eagle {

// Barrier-free variant for M <= 32 rows.  Every wave streams its own W rows
// and reads its X fragments (at most two 16-row blocks) straight from global
// memory / L2, double-buffered in registers: the loads of step i+1 are in
// flight while the MFMAs of step i run, and no workgroup barrier ever drains
// them.  Rows past M read row M-1 (their outputs are never stored).
template <typename T, int MB, int NB, int U>
__device__ __forceinline__ void direct_load(const GemmArgs& a, const T* const (&wrow)[NB],
                                            const T* const (&x0)[MB], const T* const (&x1)[MB],
                                            int k, int g, u32x4 (&w)[U][NB], u32x4 (&x)[U][MB]) {
  constexpr int VEC = DT<T>::VEC;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kk = k + u * 4 * VEC + g * VEC;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) w[u][nb] = ld16(wrow[nb] + kk);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      x[u][mb] = ld16(kk < a.ksplit_x ? x0[mb] + kk : x1[mb] + (kk - a.ksplit_x));
  }
}

template <typename T, int MB, int NB, int U>
__device__ __forceinline__ void direct_mma(f32x4 (&acc)[NB][MB], const u32x4 (&w)[U][NB],
                                           const u32x4 (&x)[U][MB]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = DT<T>::mma(w[u][nb], x[u][mb], acc[nb][mb]);
}

// acc += X[m][k_begin:k_end] W[n][k_begin:k_end]^T for this wave's columns
template <typename T, int MB, int NB, int U>
__device__ __forceinline__ void direct_mainloop(const GemmArgs& a, const T* const (&wrow)[NB],
                                                int k_begin, int k_end, int g, int c,
                                                f32x4 (&acc)[NB][MB]) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int STEP = U * 4 * VEC;
  const T* x0[MB];
  const T* x1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = min(mb * 16 + c, a.M - 1);
    x0[mb] = row_ptr<T>(a.xs[0], m);
    x1[mb] = a.xs[1].base ? row_ptr<T>(a.xs[1], m) : x0[mb];
  }
  const int kfull = k_begin + (k_end - k_begin) / STEP * STEP;
  int k = k_begin;
  if (k < kfull) {
    // The prefetch is issued on every step (the last one re-reads the final
    // batch, an L2 hit) so that each step has the same loads outstanding and a
    // batch is awaited with the next one still in flight (a conditional
    // prefetch makes the compiler wait for both); the scheduling barrier keeps
    // the prefetch ahead of the MFMAs instead of letting it sink into them.
    const int klast = kfull - STEP;
    u32x4 wa[U][NB], xa[U][MB], wb[U][NB], xb[U][MB];
    direct_load<T, MB, NB, U>(a, wrow, x0, x1, k, g, wa, xa);
    while (true) {
      direct_load<T, MB, NB, U>(a, wrow, x0, x1, min(k + STEP, klast), g, wb, xb);
      __builtin_amdgcn_sched_barrier(0);
      direct_mma<T, MB, NB, U>(acc, wa, xa);
      k += STEP;
      if (k >= kfull) break;
      direct_load<T, MB, NB, U>(a, wrow, x0, x1, min(k + STEP, klast), g, wa, xa);
      __builtin_amdgcn_sched_barrier(0);
      direct_mma<T, MB, NB, U>(acc, wb, xb);
      k += STEP;
      if (k >= kfull) break;
    }
  }
  for (; k < k_end; k += 4 * VEC) {   // tail, one MFMA step at a time
    u32x4 w1[1][NB], x1v[1][MB];
    direct_load<T, MB, NB, 1>(a, wrow, x0, x1, k, g, w1, x1v);
    direct_mma<T, MB, NB, 1>(acc, w1, x1v);
  }
}

}  // namespace eagle
