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

bool big_gemm_ok(int dtype, int M, int N, int K) {
  return dtype == EAGLE_BF16 && M >= 64 && K % kBK == 0 && N % 16 == 0;
}

GemmShape plan_gemm_big(int M, int N, int K) {
  GemmShape s;
  s.direct = 2;
  s.MB = M >= 256 ? 16 : 8;                // tile height / 16
  s.NB = 0;
  const int BM = 16 * s.MB;
  s.ntiles = (N + kBN - 1) / kBN;
  s.mtiles = (M + BM - 1) / BM;
  const int tiles = s.ntiles * s.mtiles;
  const int kst = K / kBK;
  int S = (256 + tiles - 1) / tiles;      // one workgroup per CU (LDS-bound): fewer fp32 partials
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

void launch_gemm_big(GemmArgs a, const GemmShape& s, hipStream_t st) {
  a.kps = s.kps;
  if (s.MB == 16) launch_big_t<4, 4, 4>(a, s, st);
  else launch_big_t<4, 4, 2>(a, s, st);
}

}  // namespace eagle
