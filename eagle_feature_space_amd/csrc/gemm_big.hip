// Large-M GEMM (M >= 64 rows: the 80-row EAGLE-2 steps, the 70B-shaped head's
// 64- and 512-row draft steps, the EAGLE-3 ingest over every verified
// position, the verify-tree projections).  Every weight byte is reused M
// times, so W is read once per row tile and the kernel is a classic LDS-tiled
// one:
//   workgroup tile 256 (n) x BM (m), BM = 256 from 256 rows on, else 128;
//   BK = 64; sixteen waves in a 4 x 4 grid, each 64 (n) x BM/4 (m) with
//   4 x BM/64 accumulators of v_mfma_f32_16x16x32_bf16 (W rows are the A
//   operand, X rows the B operand, so a lane owns 4 consecutive n of one m
//   and stores 16 contiguous bytes);
//   W and X tiles are staged through LDS, double-buffered; the global loads of
//   stage k+1 are issued into registers before the MFMAs of stage k and land
//   in the other LDS buffer after them; the 16-byte chunks of an LDS row are
//   XOR-swizzled by the row index, so the tile stores and the 16-lane fragment
//   reads are free of bank conflicts.  Sixteen waves (four
//   per SIMD) keep the MFMA pipes busy across the barrier and load waits that a
//   4-wave workgroup of 128 x 64 wave tiles left exposed (2.1x faster at the
//   70B LM head: 1.14 PFLOP/s);
//   workgroups are ordered so that the m-tiles sharing a W tile are dispatched
//   back to back on the same XCD (workgroup i runs on XCD i mod 8) and share
//   that XCD's L2.
// The result goes to fp32 split-K partials P[z][m][n], consumed by the same
// epilogue kernels as the weight-streaming GEMM.
//
// From 256 rows, when the tiles alone give at least 128 workgroups (the
// 512-row LM head and gate|up, the ~20k-row EAGLE-3 ingest), k_gemm_dma
// replaces it:
//   tile 256 (n) x 256 (m), eight waves in 2 (n) x 4 (m), wave tile 128 x 64
//   (32 accumulators of 16 x 16: 1.5x the MFMAs per LDS fragment of a 64 x 64
//   wave tile);
//   BK = 32 per stage and a four-stage LDS ring filled by direct-to-LDS loads
//   (global_load_lds_dwordx4: no staging registers), issued three stages
//   ahead; one barrier per stage, preceded by a partial vmcnt wait that lets
//   the two younger stages stay in flight (a __syncthreads would wait for all
//   of them);
//   every fragment is read from LDS half a stage before its MFMAs (the
//   barrier sits between the two halves of a stage's MFMAs), so no MFMA waits
//   on an LDS read;
//   LDS rows of 64 bytes: 16-byte chunk j of row r sits at j ^ ((r >> 1) & 2)
//   (chosen by measuring the bank-conflict counter over every linear
//   row-bit swizzle; the 128-byte-row swizzle of k_gemm_big does not carry
//   over).  A direct-to-LDS load writes 64 lanes x 16 B contiguously, so the
//   swizzle is applied by choosing each lane's global chunk.
// With one split and pair_F set it writes the SwiGLU activations itself: the
// W tile takes gate and up rows in alternating 16-row blocks, so a lane holds
// gate and up of the same (row, column) in two accumulators.
// Same MFMA order over K as k_gemm_big (ascending 32-wide steps), so the two
// kernels give bit-identical sums.
#include "kernels.h"

namespace eagle {

constexpr int kBN = 256, kBK = 64;
constexpr int kRowB = kBK * 2;                             // LDS row (bytes): 8 chunks of 16 B

// LDS byte offset of 16-byte chunk j of tile row r: chunk j sits at position
// j ^ ((r >> 1) & 7).  A store pass (16 lanes: two rows x 8 chunks) and a
// fragment read (16 rows, one chunk each) both touch every bank once.
__device__ __forceinline__ int big_off(int r, int j) { return r * kRowB + 16 * (j ^ ((r >> 1) & 7)); }
template <int BM> constexpr int big_stage() { return (kBN + BM) * kRowB; }
template <int BM> constexpr int big_lds() { return 2 * big_stage<BM>(); }   // 110592 / 147456

// WN x WM waves; wave (wn, wm) owns 256/WN n and WMB 16-row blocks of m;
// the tile is 256 x BM with BM = 16 WMB WM
template <int WN, int WM, int WMB>
__global__ __launch_bounds__(64 * WN * WM) void k_gemm_big(GemmArgs a, int nt, int mt, int S) {
  constexpr int NT = 64 * WN * WM;
  constexpr int WNB = 16 / WN;                     // 16-row W blocks per wave
  constexpr int kBM = 16 * WMB * WM;
  constexpr int kStageB = big_stage<kBM>();
  constexpr int WCH = 2048 / NT, XCH = kBM * 8 / NT;  // staged 16-byte chunks per thread
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wn = wave / WM, wm = wave % WM;

  // XCD-aware order: XCD x (= wgid mod 8) walks a contiguous run of the
  // (split, n-tile, m-tile) list, m fastest
  const int total = nt * mt * S;
  const int per = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int mtile = lin % mt;
  const int ntile = (lin / mt) % nt;
  const int z = lin / (mt * nt);
  const int n0 = ntile * kBN, m0 = mtile * kBM;
  const int k_begin = z * a.kps, k_end = min(a.K, k_begin + a.kps);

  // global -> LDS mapping: 8 chunks of 16 B per row; W tile 2048 chunks,
  // X tile 8 BM chunks, spread over the threads
  const bf16s* wsrc[WCH];
  const bf16s* xsrc[XCH];
  const bf16s* xsrc1[XCH];    // second A segment (k >= ksplit_x), e.g. emb(t) of [f ; emb(t)]
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int q = tid + NT * i, r = q >> 3, ch = q & 7;
    const int n = min(n0 + r, a.N - 1);
    const bf16s* base;
    int off;
    if (n < a.nseg1) { base = (const bf16s*)a.w[0]; off = 0; }
    else if (n < a.nseg2) { base = (const bf16s*)a.w[1]; off = a.nseg1; }
    else { base = (const bf16s*)a.w[2]; off = a.nseg2; }
    wsrc[i] = base + (int64_t)(n - off) * a.K + ch * 8;
  }
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int q = tid + NT * i, r = q >> 3, ch = q & 7;
    const int m = min(m0 + r, a.M - 1);
    xsrc[i] = row_ptr<bf16s>(a.xs[0], m) + ch * 8;
    xsrc1[i] = (a.xs[1].base ? row_ptr<bf16s>(a.xs[1], m) : xsrc[i] - ch * 8) + ch * 8;
  }

  f32x4 acc[WNB][WMB];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wreg[WCH], xreg[XCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) wreg[i] = ld16(wsrc[i] + k0);
    const bool hi = k0 >= a.ksplit_x;      // a BK tile never straddles the split
#pragma unroll
    for (int i = 0; i < XCH; ++i) xreg[i] = hi ? ld16(xsrc1[i] + (k0 - a.ksplit_x)) : ld16(xsrc[i] + k0);
  };
  auto lstore = [&](int buf) {
    char* base = lds + buf * kStageB;
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int q = tid + NT * i;
      st16(base + big_off(q >> 3, q & 7), wreg[i]);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int q = tid + NT * i;
      st16(base + big_off(kBN + (q >> 3), q & 7), xreg[i]);
    }
  };

  int buf = 0;
  if (k_begin < k_end) {
    gload(k_begin);
    lstore(0);
  }
  __syncthreads();
  for (int k0 = k_begin; k0 < k_end; k0 += kBK) {
    const bool more = k0 + kBK < k_end;
    if (more) gload(k0 + kBK);
    const char* st = lds + buf * kStageB;
    const int wr0 = wn * 16 * WNB, xr0 = kBN + wm * 16 * WMB;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      u32x4 xf[WMB];
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) xf[mb] = ld16(st + big_off(xr0 + mb * 16 + c, kk * 4 + g));
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const u32x4 wf = ld16(st + big_off(wr0 + nb * 16 + c, kk * 4 + g));
#pragma unroll
        for (int mb = 0; mb < WMB; ++mb) acc[nb][mb] = DT<bf16s>::mma(wf, xf[mb], acc[nb][mb]);
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // acc[nb][mb]: lane holds out[m = m0 + 16 (WMB wm + mb) + c][n = n0 + 16 (WNB wn + nb) + 4 g + 0..3]
  float* P = a.P + (int64_t)z * a.M * a.N;
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) {
    const int n = n0 + (wn * WNB + nb) * 16 + 4 * g;
    if (n >= a.N) continue;
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const int m = m0 + (wm * WMB + mb) * 16 + c;
      if (m < a.M) *reinterpret_cast<f32x4*>(P + (int64_t)m * a.N + n) = acc[nb][mb];
    }
  }
}

// ------------------------------------------------------------ direct-to-LDS
constexpr int kDN = 256, kDK = 32;
constexpr int kDRow = kDK * 2;                              // 64 B per row per stage

// Tiles BN x BM: 256 x 256 (from 256 rows) and 256 x 128 (64..255 rows).
// Eight waves in 2 (n) x 4 (m), wave tile 128 x BM/4; each wave issues L 1 KB
// direct-to-LDS loads per stage (16 rows of 64 B each), PF stages ahead.
template <int BN, int BM>
struct Dma {
  static constexpr int WN = BN / 128, WM = 8 / WN;          // wave grid
  static constexpr int WMB = BM / WM / 16;                  // 16-row m-blocks per wave
  static constexpr int ROWS = BN + BM;                      // W rows, then X rows
  static constexpr int STAGE = ROWS * kDRow;                // 32 / 24 KB
  static constexpr int STAGES = BM == 256 ? 4 : 6;          // ring: 128 / 144 KB
  static constexpr int PF = STAGES - 1;
  static constexpr int L = ROWS / 16 / 8;                   // 4 / 3
  static constexpr int LDS = STAGES * STAGE;
};


__device__ __forceinline__ int dma_off(int r, int j) { return r * kDRow + 16 * (j ^ ((r >> 1) & 2)); }


template <int EPI, int BN, int BM>   // EPI 0: fp32 partials P[z][m][n]; 1: SwiGLU, bf16 act[m][j]
__global__ __launch_bounds__(512) void k_gemm_dma(GemmArgs a, int nt, int mt, int S) {
  using D = Dma<BN, BM>;
  constexpr int WMB = D::WMB, L = D::L, PF = D::PF, WM = D::WM;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wn = wave / WM, wm = wave % WM;
  const int total = nt * mt * S;
  const int per = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int mtile = lin % mt;
  const int ntile = (lin / mt) % nt;
  const int z = lin / (mt * nt);
  const int n0 = ntile * BN, m0 = mtile * BM;
  const int k_begin = z * a.kps, k_end = min(a.K, k_begin + a.kps);
  const int nst = (k_end - k_begin) / kDK;

  // wave w loads stage blocks L w .. L w + L - 1 (16 rows each; rows below BN
  // are W rows, the rest X rows); lane l writes chunk slot l & 3 of block row
  // l >> 2, i.e. global chunk (l & 3) ^ ((row >> 1) & 2) of that row
  const char* src[L];
  const char* src1[L];
  bool isx[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int r = (wave * L + i) * 16 + (lane >> 2);        // stage row
    const int j = (lane & 3) ^ ((r >> 1) & 2);
    isx[i] = r >= BN;
    if (!isx[i]) {
      int n;
      if (EPI == 1) {   // 16-row blocks alternate gate (even) and up (odd)
        const int b = r >> 4;
        const int q = ntile * (BN / 2) + (b >> 1) * 16 + (r & 15);
        n = (b & 1) ? a.pair_F + min(q, a.pair_F - 1) : min(q, a.pair_F - 1);
      } else {
        n = min(n0 + r, a.N - 1);
      }
      const bf16s* base;
      int off;
      if (n < a.nseg1) { base = (const bf16s*)a.w[0]; off = 0; }
      else if (n < a.nseg2) { base = (const bf16s*)a.w[1]; off = a.nseg1; }
      else { base = (const bf16s*)a.w[2]; off = a.nseg2; }
      src[i] = (const char*)(base + (int64_t)(n - off) * a.K + j * 8);
      src1[i] = src[i];
    } else {
      const int m = min(m0 + r - BN, a.M - 1);
      src[i] = (const char*)(row_ptr<bf16s>(a.xs[0], m) + j * 8);
      src1[i] = a.xs[1].base ? (const char*)(row_ptr<bf16s>(a.xs[1], m) + j * 8) : src[i];
    }
  }
  // stage s (clamped to the last one, so every stage issues the same number
  // of loads and the vmcnt waits stay exact) into ring slot s % STAGES
  auto issue = [&](int s) {
    const int sc = min(s, nst - 1);
    const int k0 = k_begin + sc * kDK;
    char* dst = lds + (s % D::STAGES) * D::STAGE + wave * L * 1024;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool hi = isx[i] && k0 >= a.ksplit_x;          // a stage never straddles the split
      const char* p = hi ? src1[i] + (int64_t)(k0 - a.ksplit_x) * 2 : src[i] + (int64_t)k0 * 2;
      __builtin_amdgcn_global_load_lds((const void*)p, (lds_void*)(dst + i * 1024), 16, 0, 0);
    }
  };

  f32x4 acc[8][WMB];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nst > 0) {
    // Fragments are read half a stage ahead of their MFMAs, the barrier sits
    // in the middle of a stage:
    //   MFMAs n-blocks 0-3 of stage s | wait for stage s+1, barrier, loads of
    //   stage s+PF, reads of stage s+1 (W blocks 0-3 and X) | MFMAs n-blocks
    //   4-7 of stage s | reads of stage s+1 W blocks 4-7.
    // The X fragments alternate between two register sets, so the loop body
    // covers two stages (nst is even: K per split is a multiple of 64).
    // After a barrier every wave has issued all its reads of stage s (they
    // completed before the MFMAs that used them, in front of the barrier), so
    // the slot stage s+PF overwrites (stage s-1's) is free.
    const int wr0 = wn * 128, xr0 = BN + wm * 16 * WMB;
#pragma unroll
    for (int i = 0; i < PF; ++i) issue(i);
    __builtin_amdgcn_s_waitcnt(vm_wait((PF - 1) * L));     // stage 0 landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    u32x4 wf[8], xa[WMB], xb[WMB];
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) xa[mb] = ld16(lds + dma_off(xr0 + mb * 16 + c, g));
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) wf[nb] = ld16(lds + dma_off(wr0 + nb * 16 + c, g));
#define DMA_STAGE(S_, XC, XN)                                                                 \
    {                                                                                       \
      _Pragma("unroll") for (int nb = 0; nb < 4; ++nb)                                      \
      _Pragma("unroll") for (int mb = 0; mb < WMB; ++mb)                                    \
        acc[nb][mb] = DT<bf16s>::mma(wf[nb], XC[mb], acc[nb][mb]);                          \
      __builtin_amdgcn_sched_barrier(0);                                                    \
      __builtin_amdgcn_s_waitcnt(vm_wait((PF - 2) * L));    /* stage S_+1 landed */         \
      __builtin_amdgcn_s_barrier();                                                         \
      __builtin_amdgcn_sched_barrier(0);                                                    \
      issue((S_) + PF);                                                                     \
      const char* st_ = lds + (((S_) + 1) % D::STAGES) * D::STAGE;                          \
      _Pragma("unroll") for (int nb = 0; nb < 4; ++nb)                                      \
        wf[nb] = ld16(st_ + dma_off(wr0 + nb * 16 + c, g));                                 \
      _Pragma("unroll") for (int mb = 0; mb < WMB; ++mb)                                    \
        XN[mb] = ld16(st_ + dma_off(xr0 + mb * 16 + c, g));                                 \
      _Pragma("unroll") for (int nb = 4; nb < 8; ++nb)                                      \
      _Pragma("unroll") for (int mb = 0; mb < WMB; ++mb)                                    \
        acc[nb][mb] = DT<bf16s>::mma(wf[nb], XC[mb], acc[nb][mb]);                          \
      _Pragma("unroll") for (int nb = 4; nb < 8; ++nb)                                      \
        wf[nb] = ld16(st_ + dma_off(wr0 + nb * 16 + c, g));                                 \
      __builtin_amdgcn_sched_group_barrier(0x020, L, 0);        /* loads */                 \
      __builtin_amdgcn_sched_group_barrier(0x100, 4 + WMB, 0);  /* reads W 0-3, X */        \
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * WMB, 0);  /* MFMAs n-blocks 4-7 */    \
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);        /* reads W 4-7 */           \
      __builtin_amdgcn_sched_barrier(0);                                                    \
    }
    for (int s = 0; s < nst; s += 2) {
      DMA_STAGE(s, xa, xb)
      DMA_STAGE(s + 1, xb, xa)
    }
#undef DMA_STAGE
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no load in flight when the wave ends

  // acc[nb][mb]: lane holds out[m = m0 + BM/WM wm + 16 mb + c][n = n0 + 128 wn + 16 nb + 4 g + 0..3]
  if (EPI == 2) {
    // row epilogue (one split, BN = 256): y = acc + res row, bf16 y and
    // y * gain, and the row's (sum, sum of squares) over the tile's 256
    // columns: each lane sums its 32 columns, the four lanes of a row (16 and
    // 32 apart) by permlane swaps, the two n-waves through LDS
    float* red = reinterpret_cast<float*>(lds);           // [WM][WMB][16][2] of the wn = 1 waves
    __syncthreads();                                      // every wave is past its fragment reads
    // the gains of the lane's 32 columns, then per m-block the 8 residual
    // loads together (rows past M re-read row M - 1), so the epilogue pays a
    // few memory latencies, not one per column block
    uint2 gv[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      gv[nb] = *reinterpret_cast<const uint2*>((const bf16s*)a.gain + n0 + wn * 128 + nb * 16 + 4 * g);
    float s1[WMB], s2[WMB];
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const int m = m0 + wm * 16 * WMB + mb * 16 + c;
      const bool live = m < a.M;
      const bf16s* er = row_ptr<bf16s>(a.res, live ? m : a.M - 1);
      uint2 ev[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) ev[nb] = *reinterpret_cast<const uint2*>(er + n0 + wn * 128 + nb * 16 + 4 * g);
      float t1 = 0.f, t2 = 0.f;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int n = n0 + wn * 128 + nb * 16 + 4 * g;
        const f32x4 y = acc[nb][mb] + f32x4{bf2f(ev[nb].x & 0xffffu), bf2f(ev[nb].x >> 16),
                                            bf2f(ev[nb].y & 0xffffu), bf2f(ev[nb].y >> 16)};
        const f32x4 gn = f32x4{bf2f(gv[nb].x & 0xffffu), bf2f(gv[nb].x >> 16),
                               bf2f(gv[nb].y & 0xffffu), bf2f(gv[nb].y >> 16)};
        const f32x4 yg = y * gn;
        if (live) {
          *reinterpret_cast<uint2*>((bf16s*)a.out + (int64_t)m * a.N + n) =
              make_uint2(f2bf(y[0]) | (f2bf(y[1]) << 16), f2bf(y[2]) | (f2bf(y[3]) << 16));
          *reinterpret_cast<uint2*>((bf16s*)a.out_g + (int64_t)m * a.N + n) =
              make_uint2(f2bf(yg[0]) | (f2bf(yg[1]) << 16), f2bf(yg[2]) | (f2bf(yg[3]) << 16));
          t1 += (y[0] + y[1]) + (y[2] + y[3]);
          t2 += (y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]);
        }
      }
      s1[mb] = sum_x32(sum_x16(t1));
      s2[mb] = sum_x32(sum_x16(t2));
      if (wn == 1 && g == 0) {
        red[((wm * WMB + mb) * 16 + c) * 2] = s1[mb];
        red[((wm * WMB + mb) * 16 + c) * 2 + 1] = s2[mb];
      }
    }
    __syncthreads();
    if (wn == 0 && g == 0) {
      const int nblk = a.N / 256;
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) {
        const int m = m0 + wm * 16 * WMB + mb * 16 + c;
        if (m >= a.M) continue;
        float* st = a.stats + ((int64_t)m * nblk + ntile) * 2;
        st[0] = s1[mb] + red[((wm * WMB + mb) * 16 + c) * 2];
        st[1] = s2[mb] + red[((wm * WMB + mb) * 16 + c) * 2 + 1];
      }
    }
    return;
  }
  if (EPI == 1) {
    // gate block nb (even) pairs with up block nb + 1: columns
    // j = BN/2 ntile + 16 ((8 wn + nb) / 2) + 4 g + 0..3 of act (F columns)
#pragma unroll
    for (int nb = 0; nb < 8; nb += 2) {
      const int j = ntile * (BN / 2) + ((wn * 8 + nb) >> 1) * 16 + 4 * g;
      if (j >= a.pair_F) continue;
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) {
        const int m = m0 + wm * 16 * WMB + mb * 16 + c;
        if (m >= a.M) continue;
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gs = acc[nb][mb][e], u = acc[nb + 1][mb][e];
          y[e] = gs / (1.0f + expf(-gs)) * u;
        }
        uint2 v;
        v.x = f2bf(y[0]) | (f2bf(y[1]) << 16);
        v.y = f2bf(y[2]) | (f2bf(y[3]) << 16);
        *reinterpret_cast<uint2*>((bf16s*)a.act + (int64_t)m * a.pair_F + j) = v;
      }
    }
    return;
  }
  float* P = a.P + (int64_t)z * a.M * a.N;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int n = n0 + wn * 128 + nb * 16 + 4 * g;
    if (n >= a.N) continue;
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const int m = m0 + wm * 16 * WMB + mb * 16 + c;
      if (m < a.M) *reinterpret_cast<f32x4*>(P + (int64_t)m * a.N + n) = acc[nb][mb];
    }
  }
}

// 256 x 128 tiles with 64 of K per stage: the tile, wave grid and MFMA order
// of k_gemm_dma<*, 256, 128>, but each LDS row holds 128 bytes and one
// direct-to-LDS load covers 8 rows x 128 B, half the memory requests per
// weight byte of 16 rows x 64 B (a load-only probe of the two shapes: 3-10%
// apart at 80 rows).  Three stages of 48 KB, two in flight.  Fragment reads
// and MFMAs keep the 32-K sub-stage rhythm of k_gemm_dma (reads half a
// sub-stage ahead, a barrier in the middle of each); DMA stage S holds
// sub-stages 2S and 2S+1.  After the barrier of sub-stage 2S, stage S+2 is
// issued into the slot of stage S-1, which every wave has finished (all are
// past sub-stage 2S-1); before the barrier of sub-stage 2S+1 each wave waits
// for its loads of stage S+1.  16-byte chunk j of a 128-byte row r sits at
// j ^ ((r >> 1) & 7) (the swizzle k_gemm_big uses for its 128-byte rows).
//
// Persistent over tiles: at most 256 workgroups (one per CU), each walking
// the tiles of its XCD's contiguous share.  The stages of its tiles form one
// stream through the ring (a loader position: tile, stage, ring count), so
// the last stage issues of a tile already fetch the next tile's first
// stages and the last sub-stage reads the next tile's first fragments: the
// epilogue's stores run while the next tile's weights are in flight and no
// workgroup starts from an empty pipe.  Nothing is issued past the last
// stage of a workgroup's last tile, and a split may be a single stage.
constexpr int kWRow = 128;
__device__ __forceinline__ int dmaw_off(int r, int j) { return r * kWRow + 16 * (j ^ ((r >> 1) & 7)); }
constexpr int kDmawStage = (256 + 128) * kWRow;             // 48 KB
constexpr int kDmawLds = 3 * kDmawStage;                    // 144 KB

// LM-head epilogue (EPI 3): per-row running state after the ring, and the
// rows of the finished tile staged (fp32, rows padded to 260 floats) in the
// ring slot no stage occupies while the epilogue runs
constexpr int kLmRows = 80;
constexpr int kLmRunBytes = kLmRows * 8 + kLmRows * kLmFusedTopK * 8;
constexpr int kLmStg = 260;
constexpr int kLgkmWait0 = 0xC07F;                          // s_waitcnt lgkmcnt(0)
constexpr int kLmLD = 4;                                    // keys each lane keeps sorted
// reductions over each 16-lane row of the wave (every lane of the row gets
// the result)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}
__device__ __forceinline__ uint64_t row16_umax64(uint64_t v) {
  v = umax64(v, dpp_u64<0xB1>(v));
  v = umax64(v, dpp_u64<0x4E>(v));
  v = umax64(v, dpp_u64<0x141>(v));
  return umax64(v, dpp_u64<0x140>(v));
}
// (logit desc, column asc) as one 64-bit key; 0 is below every real key
__device__ __forceinline__ uint64_t lm_key(float v, int col) {
  return ((uint64_t)float_order(v) << 32) | (0xffffffffu - (uint32_t)col);
}
// LDS writes of every wave done, then every wave here (no vmcnt wait: the
// next tile's stages stay in flight)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkmWait0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wave grids: WN = 2 (2 x 4 waves, 128 x 32 wave tiles, all 128 rows) or, for
// 65..80 rows, WN = 8 (8 x 1 waves, 32 x 80 wave tiles: only the five live
// 16-row blocks are multiplied, 10 MFMAs per 32 of K per wave instead of 16,
// and each wave reads 2 W + 5 X fragments instead of 8 + 2).
// EPI 0: fp32 partials P[z][m][n]; 1: SwiGLU, bf16 act[m][j]; 3: LM-head
// softmax / top-k parts (and the fp32 logits into P if set)
template <int EPI, int WN = 2, int WMB = 2>
__global__ __launch_bounds__(512) void k_gemm_dmaw(GemmArgs a, int nt, int mt, int S) {
  static_assert(EPI != 3 || (WN == 8 && WMB * 16 == kLmRows), "the LM-head epilogue takes the 8 x 1 grid");
  constexpr int BN = 256, BM = 128, WM = 8 / WN;
  constexpr int NBW = 16 / WN;                              // 16-row W blocks per wave
  constexpr int MSPAN = BM / WM;                            // tile rows spanned by a wave
  static_assert(WMB * 16 <= MSPAN, "m-blocks past the wave's rows");
  constexpr int L = (BN + BM) / 8 / 8;                      // 6 loads of 8 rows per wave per stage
  constexpr int H = NBW / 2;                                // n-blocks per half sub-stage
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wn = wave / WM, wm = wave % WM;
  const int total = nt * mt * S;
  const int per = (total + 7) / 8;
  const int G8 = gridDim.x >> 3;                            // workgroups per XCD
  const int lin_end = min(((int)blockIdx.x & 7) * per + per, total);
  int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  // EPI 3: LDS running state of row m: max, sum, top-k keys
  float* run_max = reinterpret_cast<float*>(lds + kDmawLds);
  float* run_sum = run_max + kLmRows;
  uint64_t* run_key = reinterpret_cast<uint64_t*>(lds + kDmawLds + kLmRows * 8);
  const int K_ = a.lm_top_k;
  // part blockIdx.x of every row from the running state (an empty part for
  // a workgroup without tiles)
  auto write_part = [&](bool empty) {
    const int64_t p0 = (int64_t)blockIdx.x * a.M;
    for (int m = tid; m < a.M; m += 512) {
      a.lm_max[p0 + m] = empty ? -INFINITY : run_max[m];
      a.lm_sum[p0 + m] = empty ? 0.f : run_sum[m];
    }
    for (int q = tid; q < a.M * K_; q += 512) {
      const int m = q / K_, k = q - m * K_;
      const uint64_t key = empty ? 0ull : run_key[m * kLmFusedTopK + k];
      a.lm_val[(p0 + m) * K_ + k] = key ? order_float((uint32_t)(key >> 32)) : -INFINITY;
      a.lm_id[(p0 + m) * K_ + k] = key ? min((int)(0xffffffffu - (uint32_t)key), a.N - 1) : 0;
    }
  };
  if (lin >= lin_end) {
    if constexpr (EPI == 3) write_part(true);
    return;
  }
  if constexpr (EPI == 3) {
    for (int m = tid; m < kLmRows; m += 512) {
      run_max[m] = -INFINITY;
      run_sum[m] = 0.f;
    }
    for (int q = tid; q < kLmRows * kLmFusedTopK; q += 512) run_key[q] = 0ull;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkmWait0);   // before the prologue's barrier
    asm volatile("" ::: "memory");
  }

  // load i of wave w: rows 8 (w L + i) .. +7; lane l takes row + (l >> 3),
  // LDS slot l & 7, i.e. global chunk (l & 7) ^ ((row >> 1) & 7).  These
  // describe the tile whose stages are being issued (set up by `setup`).
  const char* src[L];
  const char* src1[L];
  bool isx[L];
  // stages of 64 K in tile l's split (at least one)
  auto tile_nst = [&](int l) {
    const int k0 = (l / (mt * nt)) * a.kps;
    return (min(a.K, k0 + a.kps) - k0) / 64;
  };
  int ld_k0 = 0, ld_nst = 0;
  auto setup = [&](int l) {
    const int mtile = l % mt, ntile = (l / mt) % nt, z = l / (mt * nt);
    const int n0 = ntile * BN, m0 = mtile * BM;
    ld_k0 = z * a.kps;
    ld_nst = tile_nst(l);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int r = (wave * L + i) * 8 + (lane >> 3);
      const int j = (lane & 7) ^ ((r >> 1) & 7);
      isx[i] = r >= BN;
      if (!isx[i]) {
        int n;
        if (EPI == 1) {   // 16-row blocks alternate gate (even) and up (odd)
          const int b = r >> 4;
          const int q = ntile * (BN / 2) + (b >> 1) * 16 + (r & 15);
          n = (b & 1) ? a.pair_F + min(q, a.pair_F - 1) : min(q, a.pair_F - 1);
        } else {
          n = min(n0 + r, a.N - 1);
        }
        const bf16s* base;
        int off;
        if (n < a.nseg1) { base = (const bf16s*)a.w[0]; off = 0; }
        else if (n < a.nseg2) { base = (const bf16s*)a.w[1]; off = a.nseg1; }
        else { base = (const bf16s*)a.w[2]; off = a.nseg2; }
        src[i] = (const char*)(base + (int64_t)(n - off) * a.K + j * 8);
        src1[i] = src[i];
      } else {
        const int m = min(m0 + r - BN, a.M - 1);
        src[i] = (const char*)(row_ptr<bf16s>(a.xs[0], m) + j * 8);
        src1[i] = a.xs[1].base ? (const char*)(row_ptr<bf16s>(a.xs[1], m) + j * 8) : src[i];
      }
    }
  };
  // stage sd of the set-up tile into ring slot `slot`
  auto issue = [&](int slot, int sd) {
    const int k0 = ld_k0 + sd * 64;
    char* dst = lds + slot * kDmawStage + wave * L * 1024;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool hi = isx[i] && k0 >= a.ksplit_x;          // a stage never straddles the split
      const char* p = hi ? src1[i] + (int64_t)(k0 - a.ksplit_x) * 2 : src[i] + (int64_t)k0 * 2;
      __builtin_amdgcn_global_load_lds((const void*)p, (lds_void*)(dst + i * 1024), 16, 0, 0);
    }
  };

  // loader: the next stage to issue is stage ld_sd of tile ld_lin, into ring
  // slot ring % 3 (ring counts the stages issued so far)
  int ld_lin = lin, ld_sd = 0, ring = 0;
  bool ld_done = false;
  setup(lin);
  auto issue_next = [&]() {
    if (ld_done) return;
    issue(ring % 3, ld_sd);
    ++ring;
    if (++ld_sd == ld_nst) {
      ld_lin += G8;
      ld_sd = 0;
      if (ld_lin < lin_end) setup(ld_lin);
      else ld_done = true;
    }
  };

  const int wr0 = wn * 16 * NBW, xr0 = BN + wm * MSPAN;
  int cbase = 0;               // ring count of the current tile's stage 0
  issue_next();
  issue_next();
  if (ring > 1) __builtin_amdgcn_s_waitcnt(vm_wait(L));     // stage 0 landed
  else __builtin_amdgcn_s_waitcnt(vm_wait(0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wf[NBW], xa[WMB], xb[WMB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) xa[mb] = ld16(lds + dmaw_off(xr0 + mb * 16 + c, g));
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) wf[nb] = ld16(lds + dmaw_off(wr0 + nb * 16 + c, g));

  for (;;) {
    const int nst = tile_nst(lin);   // stages of the current tile
    f32x4 acc[NBW][WMB];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // sub-stage T_ (MFMAs on XC), reading sub-stage T_ + 1's fragments into
    // XN / wf; EVEN_: T_ = 2S issues the stream's next stage (stage S + 2, or
    // the next tile's first ones past the end), else T_ = 2S + 1 waits for
    // stage S + 1 (with a younger stage still in flight if one was issued)
#define DMAW_SUB(T_, XC, XN, EVEN_)                                                           \
    {                                                                                       \
      _Pragma("unroll") for (int nb = 0; nb < H; ++nb)                                      \
      _Pragma("unroll") for (int mb = 0; mb < WMB; ++mb)                                    \
        acc[nb][mb] = DT<bf16s>::mma(wf[nb], XC[mb], acc[nb][mb]);                          \
      __builtin_amdgcn_sched_barrier(0);                                                    \
      if (!(EVEN_)) {                                         /* stage S + 1 landed */      \
        if (ring > cbase + ((T_) >> 1) + 2) __builtin_amdgcn_s_waitcnt(vm_wait(L));         \
        else __builtin_amdgcn_s_waitcnt(vm_wait(0));                                        \
      }                                                                                     \
      __builtin_amdgcn_s_barrier();                                                         \
      __builtin_amdgcn_sched_barrier(0);                                                    \
      if (EVEN_) issue_next();                                                              \
      const int tn_ = (T_) + 1;                                                             \
      const char* st_ = lds + ((cbase + (tn_ >> 1)) % 3) * kDmawStage;                      \
      const int kc_ = (tn_ & 1) * 4 + g;                                                    \
      _Pragma("unroll") for (int nb = 0; nb < H; ++nb)                                      \
        wf[nb] = ld16(st_ + dmaw_off(wr0 + nb * 16 + c, kc_));                              \
      _Pragma("unroll") for (int mb = 0; mb < WMB; ++mb)                                    \
        XN[mb] = ld16(st_ + dmaw_off(xr0 + mb * 16 + c, kc_));                              \
      _Pragma("unroll") for (int nb = H; nb < NBW; ++nb)                                    \
      _Pragma("unroll") for (int mb = 0; mb < WMB; ++mb)                                    \
        acc[nb][mb] = DT<bf16s>::mma(wf[nb], XC[mb], acc[nb][mb]);                          \
      _Pragma("unroll") for (int nb = H; nb < NBW; ++nb)                                    \
        wf[nb] = ld16(st_ + dmaw_off(wr0 + nb * 16 + c, kc_));                              \
      __builtin_amdgcn_sched_group_barrier(0x100, H + WMB, 0);  /* reads W first half, X */ \
      __builtin_amdgcn_sched_group_barrier(0x008, H * WMB, 0);  /* MFMAs second half */     \
      __builtin_amdgcn_sched_group_barrier(0x100, H, 0);        /* reads W second half */   \
      __builtin_amdgcn_sched_barrier(0);                                                    \
    }
    for (int t = 0; t < 2 * nst; t += 2) {
      DMAW_SUB(t, xa, xb, true)
      DMAW_SUB(t + 1, xb, xa, false)
    }
#undef DMAW_SUB

    // epilogue of tile `lin` (the next tile's first stages are in flight and
    // its first fragments are in wf / xa)
    {
      const int mtile = lin % mt, ntile = (lin / mt) % nt, z = lin / (mt * nt);
      const int n0 = ntile * BN, m0 = mtile * BM;
      if (EPI == 1) {
#pragma unroll
        for (int nb = 0; nb < NBW; nb += 2) {
          const int j = ntile * (BN / 2) + ((wn * NBW + nb) >> 1) * 16 + 4 * g;
          if (j >= a.pair_F) continue;
#pragma unroll
          for (int mb = 0; mb < WMB; ++mb) {
            const int m = m0 + wm * MSPAN + mb * 16 + c;
            if (m >= a.M) continue;
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float gs_ = acc[nb][mb][e], u = acc[nb + 1][mb][e];
              y[e] = gs_ / (1.0f + expf(-gs_)) * u;
            }
            uint2 v;
            v.x = f2bf(y[0]) | (f2bf(y[1]) << 16);
            v.y = f2bf(y[2]) | (f2bf(y[3]) << 16);
            *reinterpret_cast<uint2*>((bf16s*)a.act + (int64_t)m * a.pair_F + j) = v;
          }
        }
      } else {
        if (EPI == 0 || a.P) {
          float* P = a.P + (int64_t)z * a.M * a.N;
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            const int n = n0 + wn * 16 * NBW + nb * 16 + 4 * g;
            if (n >= a.N) continue;
#pragma unroll
            for (int mb = 0; mb < WMB; ++mb) {
              const int m = m0 + wm * MSPAN + mb * 16 + c;
              if (m < a.M) *reinterpret_cast<f32x4*>(P + (int64_t)m * a.N + n) = acc[nb][mb];
            }
          }
        }
        if constexpr (EPI == 3) {
          // rows in groups of 32 (16 for the last) through the free ring
          // slot: the waves store their 32-column slices, then each wave
          // folds whole rows (4 logits a lane) into the running state
          float* stg = reinterpret_cast<float*>(lds + ((cbase + nst + 2) % 3) * kDmawStage);
          const float sl = a.lm_inv_temp * 1.4426950408889634f;
          lds_barrier();   // every wave's reads of that slot (the tile's last stage) done
#pragma unroll
          for (int grp = 0; grp < 3; ++grp) {
            const int mb0 = 2 * grp, nmb = grp < 2 ? 2 : 1;
#pragma unroll
            for (int mb = 0; mb < WMB; ++mb) {
              if (mb < mb0 || mb >= mb0 + nmb) continue;
#pragma unroll
              for (int nb = 0; nb < NBW; ++nb)
                *reinterpret_cast<f32x4*>(stg + ((mb - mb0) * 16 + c) * kLmStg + wn * 16 * NBW + nb * 16 + 4 * g) =
                    acc[nb][mb];
            }
            lds_barrier();
            // four rows a pass, 16 lanes a row (lane j: columns 64 i + 4 j + e)
            for (int base = 4 * wave; base < 16 * nmb; base += 32) {
              const int j = lane & 15;
              const int rr = base + (lane >> 4);
              const int m = mb0 * 16 + rr;
              const bool live = m < a.M;
              float v[16];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(stg + rr * kLmStg + 64 * i + 4 * j);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * i + e] = t[e];
              }
              float mx = -INFINITY;
#pragma unroll
              for (int q = 0; q < 16; ++q)
                if (n0 + 64 * (q >> 2) + 4 * j + (q & 3) < a.N) mx = fmaxf(mx, v[q]);
              mx = row16_max(mx);
              float se = 0.f;
#pragma unroll
              for (int q = 0; q < 16; ++q)
                if (n0 + 64 * (q >> 2) + 4 * j + (q & 3) < a.N) se += __builtin_amdgcn_exp2f((v[q] - mx) * sl);
              se = row16_sum(se);
              // the lane's best kLmLD keys, sorted, over its 16 logits and (lanes
              // j < k) running key j; then k rounds of the row's largest head
              // key, which the owning lane drops.  Once some lane has used all
              // of its kept keys, every lane offers its best key below the
              // previous winner instead (from the logits it still holds).
              const uint64_t rk = j < K_ ? run_key[m * kLmFusedTopK + j] : 0ull;
              uint64_t kb[kLmLD];
#pragma unroll
              for (int r = 0; r < kLmLD; ++r) kb[r] = 0ull;
#pragma unroll
              for (int q = 0; q <= 16; ++q) {
                const int col = n0 + 64 * (q >> 2) + 4 * j + (q & 3);
                uint64_t t = q == 16 ? rk : (col < a.N ? lm_key(v[q], col) : 0ull);
#pragma unroll
                for (int r = 0; r < kLmLD; ++r) {
                  const bool c = t > kb[r];
                  const uint64_t hi = c ? t : kb[r];
                  t = c ? kb[r] : t;
                  kb[r] = hi;
                }
              }
              int used = 0;
              uint64_t prev = ~0ull, keep = 0ull;
              for (int k = 0; k < K_; ++k) {
                uint64_t cand;
                const bool fast = !__builtin_amdgcn_ballot_w64(used >= kLmLD);
                if (fast) {
                  cand = kb[0];
                } else {
                  cand = rk < prev ? rk : 0ull;
#pragma unroll
                  for (int q = 0; q < 16; ++q) {
                    const int col = n0 + 64 * (q >> 2) + 4 * j + (q & 3);
                    const uint64_t t = col < a.N ? lm_key(v[q], col) : 0ull;
                    if (t < prev && t > cand) cand = t;
                  }
                }
                const uint64_t w = row16_umax64(cand);
                if (fast && kb[0] == w && w != 0ull) {
#pragma unroll
                  for (int r = 0; r + 1 < kLmLD; ++r) kb[r] = kb[r + 1];
                  kb[kLmLD - 1] = 0ull;
                  ++used;
                }
                if (j == k) keep = w;
                prev = w;
              }
              if (live && j < K_) run_key[m * kLmFusedTopK + j] = keep;
              if (live && j == 0) {
                const float m0_ = run_max[m], s0_ = run_sum[m];
                const float mn = fmaxf(m0_, mx);
                float sn = 0.f;
                if (m0_ != -INFINITY) sn += s0_ * __builtin_amdgcn_exp2f((m0_ - mn) * sl);
                if (mx != -INFINITY) sn += se * __builtin_amdgcn_exp2f((mx - mn) * sl);
                run_max[m] = mn;
                run_sum[m] = sn;
              }
            }
            lds_barrier();
          }
        }
      }
    }
    lin += G8;
    if (lin >= lin_end) break;
    cbase += nst;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no load in flight when the wave ends
  if constexpr (EPI == 3) write_part(false);   // the last epilogue ended in a barrier
}

// the direct-to-LDS kernel's plan (or none: fall back to k_gemm_big).
// 128-row tiles for 64..255 rows, split along K until the grid is one wave
// of at most 256 workgroups (one per CU); 256-row tiles from 256 rows where
// the tiles alone give >= 128 workgroups.
static bool plan_dma(int M, int N, int K, GemmShape* s) {
  if (M < 17 || K % (2 * kDK) != 0) return false;
  const int BM = M >= 256 ? 256 : 128;
  const int BN = kDN;
  const int nt = (N + BN - 1) / BN, mt = (M + BM - 1) / BM;
  const int tiles = nt * mt;
  if (BM == 256 && tiles < 128) return false;
  const int kst = K / kDK;                  // even: K is a multiple of 64
  // one workgroup per CU: tiles split until the grid is one wave of
  // at most 256 workgroups (a partial second wave would double the time)
  int S = 256 / tiles;
  if (S > kst / 8) S = kst / 8 > 0 ? kst / 8 : 1;
  if (S < 1) S = 1;
  int sps = (kst + S - 1) / S;
  sps += sps & 1;                           // an even number of stages per split
  s->direct = 2;
  s->NB = 2;                // the direct-to-LDS kernel
  s->MB = BM / 16;
  s->BN = BN;
  s->ntiles = nt;
  s->mtiles = mt;
  s->kps = sps * kDK;
  s->S = (K + s->kps - 1) / s->kps;
  return true;
}

bool big_gemm_ok(int dtype, int M, int N, int K) {
  return dtype == EAGLE_BF16 && M >= 64 && K % kBK == 0 && N % 16 == 0;
}

bool wide_rows_ok(int dtype, int M, int N, int K) {
  GemmShape s;
  return dtype == EAGLE_BF16 && M > 16 && M < 64 && K % kBK == 0 && N % 16 == 0 && plan_dma(M, N, K, &s);
}

bool big_rowepi_ok(int dtype, int M, int N, int K) {
  GemmShape s;
  if (!big_gemm_ok(dtype, M, N, K) || !plan_dma(M, N, K, &s)) return false;
  return s.S == 1 && s.MB == 16 && N % 256 == 0;
}

bool big_swiglu_ok(int dtype, int M, int F, int K) {
  GemmShape s;
  if (!big_gemm_ok(dtype, M, 2 * F, K) || !plan_dma(M, 2 * F, K, &s)) return false;
  return s.S == 1 && F % (s.BN / 2) == 0;
}

// the stage stream needs whole 64-K stages and at least one in every split
static bool dmaw_plan_ok(const GemmArgs& a, const GemmShape& s) {
  return a.K % 64 == 0 && s.kps % 64 == 0 && s.kps > 0 && (int64_t)(s.S - 1) * s.kps < a.K &&
         a.ksplit_x % 64 == 0;
}

bool lm_fused_ok(int dtype, int M, int V, int K, int top_k) {
  GemmShape s;
  if (!big_gemm_ok(dtype, M, V, K) || M <= 64 || M > kLmRows || top_k < 1 || top_k > kLmFusedTopK ||
      V < top_k || !plan_dma(M, V, K, &s) || s.MB != 8)
    return false;
  GemmArgs a;
  a.K = a.ksplit_x = K;
  s.S = 1;
  s.kps = K;
  return dmaw_plan_ok(a, s);
}

int lm_fused_parts(int M, int V, int K) {
  GemmShape s;
  if (!plan_dma(M, V, K, &s)) return 0;
  const int total = s.ntiles * s.mtiles;   // one split
  return std::min(((total + 7) / 8) * 8, 256);
}

GemmShape plan_gemm_big(int M, int N, int K) {
  GemmShape s;
  if (plan_dma(M, N, K, &s)) return s;
  s.direct = 2;
  s.MB = M >= 256 ? 16 : 8;                // tile height / 16
  s.NB = 0;
  const int BM = 16 * s.MB;
  s.ntiles = (N + kBN - 1) / kBN;
  s.mtiles = (M + BM - 1) / BM;
  const int tiles = s.ntiles * s.mtiles;
  const int kst = K / kBK;
  // one workgroup per CU (LDS-bound): at most 256 workgroups, since a
  // partial second pass costs a whole pass (80 tiles: 3 splits, not 4)
  int S = 256 / tiles;
  if (S > kst / 4) S = kst / 4 > 0 ? kst / 4 : 1;   // keep >= 256 K per split
  if (S < 1) S = 1;
  const int sps = (kst + S - 1) / S;
  s.kps = sps * kBK;
  s.S = (K + s.kps - 1) / s.kps;
  return s;
}

template <int WN, int WM, int WMB>
static void launch_big_t(const GemmArgs& a, const GemmShape& s, hipStream_t st) {
  constexpr int LDS = big_lds<16 * WMB * WM>();
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_big<WN, WM, WMB>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    attr = true;
  }
  const int total = s.ntiles * s.mtiles * s.S;
  const int per = (total + 7) / 8;
  hipLaunchKernelGGL((k_gemm_big<WN, WM, WMB>), dim3(per * 8), dim3(64 * WN * WM), LDS, st, a,
                     s.ntiles, s.mtiles, s.S);
}

template <int EPI, int BN, int BM>
static void launch_dma_t(const GemmArgs& a, const GemmShape& s, hipStream_t st) {
  constexpr int LDS = Dma<BN, BM>::LDS;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_dma<EPI, BN, BM>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    attr = true;
  }
  const int total = s.ntiles * s.mtiles * s.S;
  hipLaunchKernelGGL((k_gemm_dma<EPI, BN, BM>), dim3(((total + 7) / 8) * 8), dim3(512), LDS, st,
                     a, s.ntiles, s.mtiles, s.S);
}

template <int EPI, int WN, int WMB>
static void launch_dmaw_g(const GemmArgs& a, const GemmShape& s, hipStream_t st) {
  constexpr int LDS = kDmawLds + (EPI == 3 ? kLmRunBytes : 0);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_dmaw<EPI, WN, WMB>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    attr = true;
  }
  // one workgroup per CU at most, each walking its XCD's share of the tiles
  const int total = s.ntiles * s.mtiles * s.S;
  hipLaunchKernelGGL((k_gemm_dmaw<EPI, WN, WMB>), dim3(std::min(((total + 7) / 8) * 8, 256)), dim3(512),
                     LDS, st, a, s.ntiles, s.mtiles, s.S);
}
template <int EPI>
static void launch_dmaw_t(const GemmArgs& a, const GemmShape& s, hipStream_t st) {
  // one m-tile: 8 x 1 waves over the live 16-row blocks only
  if (a.M <= 32) launch_dmaw_g<EPI, 8, 2>(a, s, st);
  else if (a.M <= 64) launch_dmaw_g<EPI, 8, 4>(a, s, st);
  else if (a.M <= 80) launch_dmaw_g<EPI, 8, 5>(a, s, st);
  else launch_dmaw_g<EPI, 2, 2>(a, s, st);
}

void launch_gemm_big(GemmArgs a, const GemmShape& s, hipStream_t st) {
  a.kps = s.kps;
  if (a.lm_top_k > 0) {   // lm_fused_ok: the 8 x 1 grid, one split
    launch_dmaw_g<3, 8, 5>(a, s, st);
    return;
  }
  if (s.NB == 2) {
    const bool sw = a.pair_F > 0;
    if (a.row_epi) {   // big_rowepi_ok: 256-row tiles, one split
      launch_dma_t<2, 256, 256>(a, s, st);
      return;
    }
    if (s.MB == 16) sw ? launch_dma_t<1, 256, 256>(a, s, st) : launch_dma_t<0, 256, 256>(a, s, st);
    else if (dmaw_plan_ok(a, s)) sw ? launch_dmaw_t<1>(a, s, st) : launch_dmaw_t<0>(a, s, st);
    else sw ? launch_dma_t<1, 256, 128>(a, s, st) : launch_dma_t<0, 256, 128>(a, s, st);  // 32-K stages
    return;
  }
  if (s.MB == 16) launch_big_t<4, 4, 4>(a, s, st);
  else launch_big_t<4, 4, 2>(a, s, st);
}

}  // namespace eagle
