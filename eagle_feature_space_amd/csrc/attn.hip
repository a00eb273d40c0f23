// Tree-masked decode attention ("Tree attention in one verification pass":
// every node attends only to its ancestors, position ids from the depth) over
// a request's context cache plus the K/V of its expanded tree nodes.
//
// k_attn: one wave owns (request b, kv head, key split) and its <= 16 query rows.
// Query rows of a request are (row, head-in-group) pairs, so all G = Hq/Hkv
// heads that share a kv head are served by one pass over its keys (GQA).
// Per 64-key tile:
//   S^T[key][qrow] = K Q^T   (MFMA; K rows go straight from HBM into the A
//                             operand, Q sits in registers as the B operand)
//   online softmax per query row (exp2 domain, fully masked rows stay empty)
//   O^T[d][qrow] += V^T P^T  (MFMA; P^T is already in B-operand layout, V is
//                             staged transposed in the wave's LDS slice)
// Keys inside a tile are permuted so that lane group g owns keys
// [16g, 16g+16): the S^T accumulator of key block j, row 4g+i holds key
// 16g + 4j + i, which makes the P^T operand a plain register repack and the
// V^T operand a contiguous 16-byte LDS read.
#include "kernels.h"

namespace eagle {

constexpr int kAttnWaves = 2;   // kv heads per workgroup
// tiles in flight ahead of the one computed by k_attn_dma: one (two 64 KB
// workgroups per CU) measured faster than two (96 KB, one workgroup per CU)
constexpr int kAttnPF = 1;

// LDS byte offset of V^T[d][key] (64 keys per row of `rowb` bytes).  bf16 rows
// hold 8 chunks of 8 keys and chunk j of row d sits at position
// j ^ ((d >> 3) & 7): the 4-key stores of 16 consecutive d-groups (rows 8
// apart, which would otherwise share two bank groups) spread over the banks,
// and an 8-key fragment read stays one contiguous 16-byte chunk.
template <typename T>
__device__ __forceinline__ int vt_off(int d, int key, int rowb) {
  if constexpr (sizeof(T) == 2) return d * rowb + 16 * ((key >> 3) ^ ((d >> 3) & 7)) + 2 * (key & 7);
  else return d * rowb + 4 * key;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// P^T operand: VEC probabilities -> one 16-byte fragment (bf16: hardware
// round-to-nearest-even pair conversions)
template <typename T>
__device__ __forceinline__ u32x4 pack_p(const float* f) {
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{f[2 * i], f[2 * i + 1]}), bf16x2_t));
    return r;
  } else {
    return DT<T>::pack(f);
  }
}

// two keys' bf16 values of one d (element e of each 16-byte vector) as one word
__device__ __forceinline__ uint32_t pair16(uint32_t lo_word, uint32_t hi_word, int e) {
  return __builtin_amdgcn_perm(hi_word, lo_word, (e & 1) ? 0x07060302u : 0x05040100u);
}

// One key split of (request b, kv head): the context split `split` or, for
// split == nsplit, the request's tree-node slots gated by the rows' masks.
// Folds its tiles into the running (max, sum, O^T) state of the wave's rows.
template <typename T, int HD, int RB>
__device__ __forceinline__ void attn_split(const AttnArgs& a, int b, int kvh, int split,
                                           const u32x4 (&qf)[RB][HD / (4 * DT<T>::VEC)],
                                           const uint64_t (&msk)[RB], char* vt, float (&mrun)[RB],
                                           float (&lrun)[RB], f32x4 (&o)[HD / 16][RB]) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int DSTEPS = HD / (4 * VEC);
  constexpr int DB = HD / 16;
  constexpr int NV = 16 / VEC;
  constexpr int ROWB = 64 * (int)sizeof(T) + 16;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const bool extra = split == a.nsplit;
  int kbeg, kend;
  const T *kb, *vb;
  const int64_t kstride = (int64_t)a.Hkv * HD;
  if (!extra) {
    const int nb = a.n[b];
    kbeg = split * a.split_len;
    kend = min(kbeg + a.split_len, nb);
    kb = (const T*)a.k_ctx + (int64_t)a.cu_n[b] * kstride + kvh * HD;
    vb = (const T*)a.v_ctx + (int64_t)a.cu_n[b] * kstride + kvh * HD;
  } else {
    uint64_t any = 0;
    for (int r = 0; r < a.W; ++r) any |= a.mask[b * a.W + r];
    kbeg = 0;
    kend = any ? 64 - __builtin_clzll(any) : 0;
    kb = (const T*)a.k_ex + (int64_t)b * kSlots * kstride + kvh * HD;
    vb = (const T*)a.v_ex + (int64_t)b * kSlots * kstride + kvh * HD;
  }

  for (int t0 = kbeg; t0 < kend; t0 += 64) {
    // ---- K fragments of the tile: issued first, they land while V is staged
    u32x4 kf[4][DSTEPS];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(t0 + (c >> 2) * 16 + j * 4 + (c & 3), kend - 1);
      const T* kp = kb + (int64_t)key * kstride;
#pragma unroll
      for (int u = 0; u < DSTEPS; ++u) kf[j][u] = ld16(kp + u * 4 * VEC + g * VEC);
    }
    // ---- V tile -> LDS, transposed: vt[d][key]
    wave_lds_sync();
    {
      constexpr int DG = HD / VEC;            // d groups of VEC
      constexpr int UNITS = 16 * DG;          // (key quad, d group)
#pragma unroll
      for (int un = lane; un < UNITS; un += 64) {
        const int kq = un / DG, dg = un % DG;
        u32x4 v4[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = min(t0 + 4 * kq + kk, kend - 1);
          v4[kk] = ld16(vb + (int64_t)key * kstride + dg * VEC);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          char* dst = vt + vt_off<T>(dg * VEC + e, 4 * kq, ROWB);
          if constexpr (sizeof(T) == 2) {
            const uint32_t w0 = pair16(v4[0][e >> 1], v4[1][e >> 1], e);
            const uint32_t w1 = pair16(v4[2][e >> 1], v4[3][e >> 1], e);
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
          } else {
            st16(dst, u32x4{v4[0][e], v4[1][e], v4[2][e], v4[3][e]});
          }
        }
      }
    }
    // ---- S^T = K Q^T
    f32x4 s[4][RB];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < DSTEPS; ++u) acc = DT<T>::mma(kf[j][u], qf[rb][u], acc);
        s[j][rb] = acc;
      }
    }
    wave_lds_sync();
    // ---- online softmax and O^T += V^T P^T
    // a tile with every key inside the split and no tree-node mask takes the
    // branch without masking (wave-uniform)
    const bool full = !extra && t0 + 64 <= kend;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = -INFINITY;
      if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[j][rb][i] *= a.scale_log2;
            tmax = fmaxf(tmax, s[j][rb][i]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t0 + g * 16 + j * 4 + i;
            bool valid = key < kend;
            if (extra) valid = valid && ((msk[rb] >> key) & 1ull);
            const float v = valid ? s[j][rb][i] * a.scale_log2 : -INFINITY;
            s[j][rb][i] = v;
            tmax = fmaxf(tmax, v);
          }
      }
      tmax = max_x32(max_x16(tmax));
      const float mnew = fmaxf(mrun[rb], tmax);
      const bool empty = mnew == -INFINITY;
      // v_exp_f32 directly (results below the normal range flush to 0)
      const float alpha = empty ? 1.f : __builtin_amdgcn_exp2f(mrun[rb] - mnew);
      float p[16];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = empty ? 0.f : __builtin_amdgcn_exp2f(s[j][rb][i] - mnew);
          p[4 * j + i] = e;
          psum += e;
        }
      psum = sum_x32(sum_x16(psum));
      lrun[rb] = lrun[rb] * alpha + psum;
      mrun[rb] = mnew;
      // scaling by 1 is exact: skipped when no row's maximum moved
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f))
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db][rb] *= alpha;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const u32x4 pf = pack_p<T>(p + v * VEC);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 vf = ld16(vt + vt_off<T>(db * 16 + c, g * 16 + v * VEC, ROWB));
          o[db][rb] = DT<T>::mma(vf, pf, o[db][rb]);
        }
      }
    }
  }
}

template <typename T, int HD, int RB>
__global__ __launch_bounds__(64 * kAttnWaves) void k_attn(AttnArgs a) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int DSTEPS = HD / (4 * VEC);    // MFMA steps over the head dim
  constexpr int DB = HD / 16;               // output d blocks
  constexpr int ROWB = 64 * (int)sizeof(T) + 16;
  __shared__ __attribute__((aligned(16))) char vts[kAttnWaves][HD * ROWB];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int kvgroups = (a.Hkv + kAttnWaves - 1) / kAttnWaves;
  const int kvh = (blockIdx.y % kvgroups) * kAttnWaves + w;
  const int rg = blockIdx.y / kvgroups;
  if (kvh >= a.Hkv) return;
  const int b = blockIdx.z;
  const int split = blockIdx.x;
  const int G = a.Hq / a.Hkv;
  const int R = a.W * G;
  const int M = a.B * a.W;
  char* vt = vts[w];

  // query fragments
  u32x4 qf[RB][DSTEPS];
  uint64_t msk[RB];
  int qm[RB], qh[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qrow = rg * 16 * RB + rb * 16 + c;
    const bool ok = qrow < R;
    const int rl = ok ? qrow / G : 0, gi = ok ? qrow % G : 0;
    qm[rb] = ok ? b * a.W + rl : -1;
    qh[rb] = kvh * G + gi;
    msk[rb] = ok ? a.mask[b * a.W + rl] : 0ull;
    const T* qp = (const T*)a.q + ((int64_t)(b * a.W + rl) * a.Hq + qh[rb]) * HD;
#pragma unroll
    for (int u = 0; u < DSTEPS; ++u)
      qf[rb][u] = ok ? ld16(qp + u * 4 * VEC + g * VEC) : u32x4{0u, 0u, 0u, 0u};
  }

  float mrun[RB], lrun[RB];
  f32x4 o[DB][RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mrun[rb] = -INFINITY;
    lrun[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  attn_split<T, HD, RB>(a, b, kvh, split, qf, msk, vt, mrun, lrun, o);

  // ---- partial (m, l, O) of this split
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (qm[rb] < 0) continue;
    const int64_t idx = ((int64_t)split * M + qm[rb]) * a.Hq + qh[rb];
    if (g == 0) {
      a.part_ml[2 * idx] = mrun[rb];
      a.part_ml[2 * idx + 1] = lrun[rb];
    }
    float* po = a.part_o + idx * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(po + db * 16 + 4 * g) = o[db][rb];
  }
}

// Many query rows per (request, kv head) -- the wide EAGLE-2 trees, the
// verify-side tree attention -- for fp32 and head dim 64 (bf16 at head dim
// 128 takes k_attn_dma below): a workgroup of NW waves serves 16 * NW query
// rows (16 per wave) of one (request, kv head, key split).  Its threads load
// each 64-key K / V tile once, cooperatively, into LDS (K as [key][d], V
// transposed as [d][key] by 4-key quads), double-buffered: the next tile's
// global loads are in flight in registers while the waves compute on the
// current one, and one barrier per tile hands the buffers over.  Per wave the
// arithmetic is that of k_attn with one 16-row block (same key permutation,
// same online softmax, same partial format).
template <typename T, int HD, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_wg(AttnArgs a) {
  constexpr int VEC = DT<T>::VEC;
  constexpr int DSTEPS = HD / (4 * VEC);
  constexpr int DB = HD / 16;
  constexpr int NV = 16 / VEC;
  constexpr int NT = 64 * NW;                          // threads
  // K tile rows: bf16 x 128 rows are 16 chunks of 16 bytes, stored unpadded with
  // chunk j of key row r at position j ^ (((r >> 4) & 3) | ((r & 3) << 2)), so
  // the 16 keys of one fragment read (4 apart in r & 3, 16 apart in r >> 4)
  // hit 16 different chunks; other shapes use padded rows
  constexpr bool KSW = sizeof(T) == 2 && HD == 128;
  constexpr int KROW = KSW ? HD * 2 : HD * (int)sizeof(T) + 16;
  constexpr int VROW = 64 * (int)sizeof(T) + 16;       // V^T row (bytes, padded)
  constexpr int BUF = 64 * KROW + HD * VROW;
  constexpr int DG = HD / VEC;                         // 16-byte groups per key
  constexpr int KCH = 64 * DG;                         // K chunks per tile
  constexpr int VUN = 16 * DG;                         // V (key quad, d group) units per tile
  constexpr int KPT = (KCH + NT - 1) / NT, VPT = (VUN + NT - 1) / NT;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  // kv heads vary fastest in dispatch order: the workgroups that read the
  // same key positions (one 2 KB row of every kv head) run side by side
  const int kvh = blockIdx.x % a.Hkv;
  const int rg = blockIdx.x / a.Hkv;
  const int split = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int R = a.W * G;
  const int M = a.B * a.W;

  // this wave's 16 query rows
  const int qrow = rg * 16 * NW + w * 16 + c;
  const bool qok = qrow < R;
  const bool wave_live = rg * 16 * NW + w * 16 < R;
  const int rl = qok ? qrow / G : 0, gi = qok ? qrow % G : 0;
  const int qm = qok ? b * a.W + rl : -1;
  const int qh = kvh * G + gi;
  const uint64_t msk = qok ? a.mask[b * a.W + rl] : 0ull;
  u32x4 qf[DSTEPS];
  {
    const T* qp = (const T*)a.q + ((int64_t)(b * a.W + rl) * a.Hq + qh) * HD;
#pragma unroll
    for (int u = 0; u < DSTEPS; ++u)
      qf[u] = qok ? ld16(qp + u * 4 * VEC + g * VEC) : u32x4{0u, 0u, 0u, 0u};
  }

  const bool extra = split == a.nsplit;
  int kbeg, kend;
  const T *kb, *vb;
  const int64_t kstride = (int64_t)a.Hkv * HD;
  if (!extra) {
    const int nb = a.n[b];
    kbeg = split * a.split_len;
    kend = min(kbeg + a.split_len, nb);
    kb = (const T*)a.k_ctx + (int64_t)a.cu_n[b] * kstride + kvh * HD;
    vb = (const T*)a.v_ctx + (int64_t)a.cu_n[b] * kstride + kvh * HD;
  } else {
    uint64_t any = 0;
    for (int r = 0; r < a.W; ++r) any |= a.mask[b * a.W + r];
    kbeg = 0;
    kend = any ? 64 - __builtin_clzll(any) : 0;
    kb = (const T*)a.k_ex + (int64_t)b * kSlots * kstride + kvh * HD;
    vb = (const T*)a.v_ex + (int64_t)b * kSlots * kstride + kvh * HD;
  }
  const int ntiles = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;

  // cooperative tile loads (keys past kend re-read key kend - 1; masked below)
  struct Stage {
    u32x4 kr[KPT];
    u32x4 vr[VPT][4];
  };
  auto gload = [&](Stage& r, int t0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int q = tid + i * NT;
      if (KCH % NT == 0 || q < KCH) {
        const int key = min(t0 + q / DG, kend - 1);
        r.kr[i] = ld16(kb + (int64_t)key * kstride + (q % DG) * VEC);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int q = tid + i * NT;
      if (VUN % NT == 0 || q < VUN) {
        const int kq = q / DG, dg = q % DG;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = min(t0 + 4 * kq + kk, kend - 1);
          r.vr[i][kk] = ld16(vb + (int64_t)key * kstride + dg * VEC);
        }
      }
    }
  };
  auto lstore = [&](const Stage& r, char* buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int q = tid + i * NT;
      if (q < KCH) {
        const int key = q / DG, ch = q % DG;
        const int pc = KSW ? ch ^ (((key >> 4) & 3) | ((key & 3) << 2)) : ch;
        st16(buf + key * KROW + pc * 16, r.kr[i]);
      }
    }
    char* vt = buf + 64 * KROW;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int q = tid + i * NT;
      if (q < VUN) {
        const int kq = q / DG, dg = q % DG;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          char* dst = vt + vt_off<T>(dg * VEC + e, 4 * kq, VROW);
          if constexpr (sizeof(T) == 2) {
            const uint32_t w0 = pair16(r.vr[i][0][e >> 1], r.vr[i][1][e >> 1], e);
            const uint32_t w1 = pair16(r.vr[i][2][e >> 1], r.vr[i][3][e >> 1], e);
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
          } else {
            st16(dst, u32x4{r.vr[i][0][e], r.vr[i][1][e], r.vr[i][2][e], r.vr[i][3][e]});
          }
        }
      }
    }
  };

  float mrun = -INFINITY, lrun = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const char* cur, int t0) {
    if (wave_live) {
      // ---- S^T = K Q^T (key permutation as in k_attn)
      f32x4 sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kl = (c >> 2) * 16 + j * 4 + (c & 3);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < DSTEPS; ++u) {
          const int ch = 4 * u + g;
          const int pc = KSW ? ch ^ (((kl >> 4) & 3) | ((kl & 3) << 2)) : ch;
          acc = DT<T>::mma(ld16(cur + kl * KROW + pc * 16), qf[u], acc);
        }
        sc[j] = acc;
      }
      // ---- online softmax, O^T += V^T P^T
      // A tile with every key inside the split and no tree-node mask (all but
      // the last tile of a context split) takes the branch without masking.
      const bool full = !extra && t0 + 64 <= kend;   // wave-uniform
      float tmax = -INFINITY;
      if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[j][i] *= a.scale_log2;
            tmax = fmaxf(tmax, sc[j][i]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t0 + g * 16 + j * 4 + i;
            bool valid = key < kend;
            if (extra) valid = valid && ((msk >> key) & 1ull);
            const float v = valid ? sc[j][i] * a.scale_log2 : -INFINITY;
            sc[j][i] = v;
            tmax = fmaxf(tmax, v);
          }
      }
      tmax = max_x32(max_x16(tmax));
      const float mnew = fmaxf(mrun, tmax);
      const bool empty = mnew == -INFINITY;
      // v_exp_f32 directly: results below the normal range flush to 0, which
      // for probabilities relative to the running maximum is exact enough
      const float alpha = empty ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
      float p[16];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = empty ? 0.f : __builtin_amdgcn_exp2f(sc[j][i] - mnew);
          p[4 * j + i] = e;
          psum += e;
        }
      psum = sum_x32(sum_x16(psum));
      lrun = lrun * alpha + psum;
      mrun = mnew;
      // scaling by 1 is exact: skipped when no row's maximum moved
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f))
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      const char* vt = cur + 64 * KROW;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const u32x4 pf = pack_p<T>(p + v * VEC);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 vf = ld16(vt + vt_off<T>(db * 16 + c, g * 16 + v * VEC, VROW));
          o[db] = DT<T>::mma(vf, pf, o[db]);
        }
      }
    }
  };

  // two register stages in flight: while the waves compute tile i from one LDS
  // buffer, tile i+1 waits in registers for the other buffer and the loads of
  // tile i+2 are issued (unrolled by two so every stage index is static)
  // The query fragments and the mask must have landed before the loop: the
  // loads inside it are then the only ones outstanding, each stage issues
  // the same count (tiles past the split re-read its last key), and a stage
  // is awaited with the next stage's loads still in flight.  Immediate 0x0070
  // = vmcnt(0) lgkmcnt(0) (expcnt 7: not waited on) in the gfx9 encoding.
  __builtin_amdgcn_s_waitcnt(0x0070);
  Stage ra, rb;
  if (ntiles > 0) {
    gload(ra, kbeg);
    gload(rb, kbeg + 64);
    lstore(ra, lds);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    {
      const int t0 = kbeg + it * 64;
      gload(ra, t0 + 128);
      compute(lds, t0);
      if (it + 1 < ntiles) lstore(rb, lds + BUF);
      __syncthreads();
    }
    if (it + 1 >= ntiles) break;
    {
      const int t0 = kbeg + (it + 1) * 64;
      gload(rb, t0 + 128);
      compute(lds + BUF, t0);
      if (it + 2 < ntiles) lstore(ra, lds);
      __syncthreads();
    }
  }

  // ---- partial (m, l, O) of this split
  if (qm < 0) return;
  const int64_t idx = ((int64_t)split * M + qm) * a.Hq + qh;
  if (g == 0) {
    a.part_ml[2 * idx] = mrun;
    a.part_ml[2 * idx + 1] = lrun;
  }
  float* po = a.part_o + idx * HD;
#pragma unroll
  for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(po + db * 16 + 4 * g) = o[db];
}

// bf16, head dim 128: k_attn_wg's arithmetic with the K and V tiles moved by
// direct-to-LDS loads (global_load_lds_dwordx4, no staging registers and no
// repacking VALU work) into a ring of PF + 1 tile slots, PF tiles ahead.
// Both tiles keep the global [key][d] layout, 256-byte rows of 16 chunks,
// chunk ch of tile key r at slot ch ^ (((r >> 4) & 3) | ((r & 3) << 2)) (the
// K fragment swizzle of k_attn_wg; a direct-to-LDS load writes 64 lanes x
// 16 B contiguously, so each lane picks the global chunk of its slot).  The
// V^T operand comes from ds_read_b64_tr_b16: in each 16-lane group, lane j
// receives element (j & 3) of the 8 bytes addressed by lane 4e + (j >> 2),
// e = 0..3, so lane 4e + p addresses key 4e (+ 8v + 4h + 16g) at d = 4p and
// lane (d = c, g) gets V[key][d] for four consecutive keys.
constexpr int kDmaTile = 64 * 256;                    // K or V tile bytes (bf16, hd 128)

__device__ __forceinline__ int kv_slot(int r) { return ((r >> 4) & 3) | ((r & 3) << 2); }

__device__ __forceinline__ uint2 ld_tr16(const char* p) {
  const short4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(__attribute__((address_space(3))) char*)p);
  return __builtin_bit_cast(uint2, r);
}

// RB 16-row blocks per wave: each K fragment and each transposed V fragment
// read from LDS feeds RB MFMAs (RB = 2 halves the LDS reads per query row)
template <int NW, int PF, int RB>
__global__ __launch_bounds__(64 * NW) void k_attn_dma(AttnArgs a) {
  constexpr int HD = 128, DSTEPS = 4, DB = 8, NV = 2;
  constexpr int S = PF + 1;                          // ring slots
  constexpr int SLOT = 2 * kDmaTile;                 // K tile, then V tile
  constexpr int L = 32 / NW;                         // 1 KB loads per wave per tile
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int kvh = blockIdx.x % a.Hkv;
  const int rg = blockIdx.x / a.Hkv;
  const int split = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int R = a.W * G;
  const int M = a.B * a.W;

  // block rb of wave w: query rows rg 16 NW RB + (w RB + rb) 16 + c
  bool blive[RB];
  int qm[RB], qh[RB];
  uint64_t msk[RB];
  u32x4 qf[RB][DSTEPS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r0 = rg * 16 * NW * RB + (w * RB + rb) * 16;
    const int qrow = r0 + c;
    const bool qok = qrow < R;
    blive[rb] = r0 < R;
    const int rl = qok ? qrow / G : 0, gi = qok ? qrow % G : 0;
    qm[rb] = qok ? b * a.W + rl : -1;
    qh[rb] = kvh * G + gi;
    msk[rb] = qok ? a.mask[b * a.W + rl] : 0ull;
    const bf16s* qp = (const bf16s*)a.q + ((int64_t)(b * a.W + rl) * a.Hq + qh[rb]) * HD;
#pragma unroll
    for (int u = 0; u < DSTEPS; ++u) qf[rb][u] = qok ? ld16(qp + u * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  const bool wave_live = blive[0];

  const bool extra = split == a.nsplit;
  int kbeg, kend;
  const bf16s *kb, *vb;
  const int64_t kstride = (int64_t)a.Hkv * HD;
  if (!extra) {
    const int nb = a.n[b];
    kbeg = split * a.split_len;
    kend = min(kbeg + a.split_len, nb);
    kb = (const bf16s*)a.k_ctx + (int64_t)a.cu_n[b] * kstride + kvh * HD;
    vb = (const bf16s*)a.v_ctx + (int64_t)a.cu_n[b] * kstride + kvh * HD;
  } else {
    uint64_t any = 0;
    for (int r = 0; r < a.W; ++r) any |= a.mask[b * a.W + r];
    kbeg = 0;
    kend = any ? 64 - __builtin_clzll(any) : 0;
    kb = (const bf16s*)a.k_ex + (int64_t)b * kSlots * kstride + kvh * HD;
    vb = (const bf16s*)a.v_ex + (int64_t)b * kSlots * kstride + kvh * HD;
  }
  const int ntiles = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;

  // tile t: wave w issues loads w L .. w L + L - 1 of the 32 (16 for K, 16
  // for V, four keys each); keys past kend re-read key kend - 1 (masked)
  auto issue = [&](int t) {
    const int t0 = kbeg + t * 64;
    char* dst = lds + (t % S) * SLOT;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = w * L + i;
      const int kr = 4 * (q & 15) + (lane >> 4);        // key within the tile
      const int key = min(t0 + kr, kend - 1);
      const int ch = (lane & 15) ^ kv_slot(kr);
      const bf16s* src = (q < 16 ? kb : vb) + (int64_t)key * kstride + ch * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + (q >> 4) * kDmaTile + (q & 15) * 1024), 16, 0, 0);
    }
  };

  float mrun[RB], lrun[RB];
  f32x4 o[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mrun[rb] = -INFINITY;
    lrun[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // lane-constant parts of the fragment addresses
  const int kslot = (c >> 2) | ((c & 3) << 2);       // kv_slot of this lane's K rows
  const int te = (lane >> 2) & 3, tp = lane & 3;     // transposing-read roles
  const int vslot = g | (te << 2);                   // kv_slot of this lane's V rows

  auto compute = [&](const char* cur, int t0) {
    if (!wave_live) return;
    f32x4 sc[RB][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kl = (c >> 2) * 16 + j * 4 + (c & 3);
      f32x4 acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < DSTEPS; ++u) {
        const u32x4 kf = ld16(cur + kl * 256 + ((4 * u + g) ^ kslot) * 16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = DT<bf16s>::mma(kf, qf[rb][u], acc[rb]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sc[rb][j] = acc[rb];
    }
    const bool full = !extra && t0 + 64 <= kend;     // wave-uniform
    float p[RB][16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = -INFINITY;
      if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[rb][j][i] *= a.scale_log2;
            tmax = fmaxf(tmax, sc[rb][j][i]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t0 + g * 16 + j * 4 + i;
            bool valid = key < kend;
            if (extra) valid = valid && ((msk[rb] >> key) & 1ull);
            const float v = valid ? sc[rb][j][i] * a.scale_log2 : -INFINITY;
            sc[rb][j][i] = v;
            tmax = fmaxf(tmax, v);
          }
      }
      tmax = max_x32(max_x16(tmax));
      const float mnew = fmaxf(mrun[rb], tmax);
      const bool empty = mnew == -INFINITY;
      const float alpha = empty ? 1.f : __builtin_amdgcn_exp2f(mrun[rb] - mnew);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = empty ? 0.f : __builtin_amdgcn_exp2f(sc[rb][j][i] - mnew);
          p[rb][4 * j + i] = e;
          psum += e;
        }
      psum = sum_x32(sum_x16(psum));
      lrun[rb] = lrun[rb] * alpha + psum;
      mrun[rb] = mnew;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f))
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] *= alpha;
    }
    const char* vt = cur + kDmaTile;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      u32x4 pf[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) pf[rb] = pack_p<bf16s>(p[rb] + v * 8);
      const char* vrow = vt + (16 * g + 8 * v + te) * 256 + 8 * (tp & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = 16 * ((2 * db + (tp >> 1)) ^ vslot);
        const uint2 lo = ld_tr16(vrow + off);             // keys 16g + 8v + 0..3
        const uint2 hi = ld_tr16(vrow + 4 * 256 + off);   // keys 16g + 8v + 4..7
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[rb][db] = DT<bf16s>::mma(u32x4{lo.x, lo.y, hi.x, hi.y}, pf[rb], o[rb][db]);
      }
    }
  };

  // the query fragments and the mask land before the loop, so the loads in
  // it are the only ones outstanding and vmcnt counts tiles
  __builtin_amdgcn_s_waitcnt(0x0070);
  const int pre = min(PF, ntiles);
  for (int t = 0; t < pre; ++t) issue(t);
  for (int it = 0; it < ntiles; ++it) {
    // tile it landed (the younger tiles may stay in flight), then every wave
    // is past its reads of tile it - 1, whose slot the next issue refills
    if (it + PF - 1 < ntiles) __builtin_amdgcn_s_waitcnt(vm_wait((PF - 1) * L));
    else __builtin_amdgcn_s_waitcnt(vm_wait(0));
    // LDS-scoped fences around the barrier: a workgroup fence over all
    // memory would wait for the tiles still in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (it + PF < ntiles) issue(it + PF);
    compute(lds + (it % S) * SLOT, kbeg + it * 64);
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (qm[rb] < 0) continue;
    const int64_t idx = ((int64_t)split * M + qm[rb]) * a.Hq + qh[rb];
    if (g == 0) {
      a.part_ml[2 * idx] = mrun[rb];
      a.part_ml[2 * idx + 1] = lrun[rb];
    }
    float* po = a.part_o + idx * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(po + db * 16 + 4 * g) = o[rb][db];
  }
}

template <int NW, int PF, int RB = 1>
static void launch_dma(const AttnArgs& a, hipStream_t st) {
  constexpr int LDS = (PF + 1) * 2 * kDmaTile;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_dma<NW, PF, RB>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    attr = true;
  }
  const int R = a.W * (a.Hq / a.Hkv);
  const int rowgroups = (R + 16 * NW * RB - 1) / (16 * NW * RB);
  dim3 grid(a.Hkv * rowgroups, a.nsplit + 1, a.B);
  hipLaunchKernelGGL((k_attn_dma<NW, PF, RB>), grid, dim3(64 * NW), LDS, st, a);
}

template <typename T, int HD, int NW>
static void launch_wg(const AttnArgs& a, hipStream_t st) {
  constexpr bool KSW = sizeof(T) == 2 && HD == 128;
  constexpr int KROW = KSW ? HD * 2 : HD * (int)sizeof(T) + 16, VROW = 64 * (int)sizeof(T) + 16;
  constexpr int LDS = 2 * (64 * KROW + HD * VROW);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_wg<T, HD, NW>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    attr = true;
  }
  const int R = a.W * (a.Hq / a.Hkv);
  const int rowgroups = (R + 16 * NW - 1) / (16 * NW);
  dim3 grid(a.Hkv * rowgroups, a.nsplit + 1, a.B);
  hipLaunchKernelGGL((k_attn_wg<T, HD, NW>), grid, dim3(64 * NW), LDS, st, a);
}

template <typename T, int HD>
static void launch_wide(const AttnArgs& a, int R, hipStream_t st) {
  if (R <= 32) launch_wg<T, HD, 2>(a, st);
  else launch_wg<T, HD, 4>(a, st);
}

void launch_attention(int dtype, const AttnArgs& a0, hipStream_t st) {
  AttnArgs a = a0;
  const int R = a.W * (a.Hq / a.Hkv);
  if (R > 16) {
    // more than one 16-row block per (request, kv head): workgroup kernel
    if (dtype == EAGLE_BF16) {
      if (a.hd == 128) {   // direct-to-LDS tiles
        // 16 rows per wave up to 64; past that 8 waves of two 16-row blocks
        // (each K / V fragment read from LDS serves 32 rows, each tile is
        // loaded once for 256 rows)
        if (R <= 32) launch_dma<2, kAttnPF>(a, st);
        else if (R <= 64) launch_dma<4, kAttnPF>(a, st);
        else launch_dma<8, kAttnPF, 2>(a, st);
      }
      else launch_wide<bf16s, 64>(a, R, st);
    } else {
      if (a.hd == 128) launch_wide<float, 128>(a, R, st);
      else launch_wide<float, 64>(a, R, st);
    }
    return;
  }
  // at most 16 query rows per (request, kv head): one 16-row block per wave
  a.rowgroups = 1;
  const int kvgroups = (a.Hkv + kAttnWaves - 1) / kAttnWaves;
  const dim3 grid(a.nsplit + 1, kvgroups, a.B), block(64 * kAttnWaves);
  if (dtype == EAGLE_BF16) {
    if (a.hd == 128) hipLaunchKernelGGL((k_attn<bf16s, 128, 1>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn<bf16s, 64, 1>), grid, block, 0, st, a);
  } else {
    if (a.hd == 128) hipLaunchKernelGGL((k_attn<float, 128, 1>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn<float, 64, 1>), grid, block, 0, st, a);
  }
}

// out[m][h][d] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// One workgroup per (head, row); split weights are formed once in LDS, then
// every thread folds its d over the splits in split order.
constexpr int kMaxParts = 1024;
template <int NB>
__device__ __forceinline__ float fold_parts(const float* po, int64_t stride, int np, const float* wts) {
  float O = 0.f;
  for (int s0 = 0; s0 < np; s0 += NB) {
    float v[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) v[q] = po[(int64_t)min(s0 + q, np - 1) * stride];
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (s0 + q < np) O += wts[s0 + q] * v[q];
  }
  return O;
}

template <typename T>
__global__ __launch_bounds__(128) void k_attn_combine(CombineArgs a) {
  __shared__ float wts[kMaxParts];
  __shared__ float red[2][2];
  const int h = blockIdx.x, m = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int np = a.nparts;
  const int64_t stride = (int64_t)a.M * a.Hq;
  const int64_t base = (int64_t)m * a.Hq + h;
  // split maxima and sums: every thread holds the (max, sum) of its splits
  constexpr int SPT = kMaxParts / 128;
  float ms[SPT], lsum[SPT];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int s = tid + 128 * i;
    ms[i] = -INFINITY;
    lsum[i] = 0.f;
    if (s < np) {
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * (s * stride + base));
      ms[i] = ml.x;
      lsum[i] = ml.y;
    }
    mx = fmaxf(mx, ms[i]);
  }
  mx = wave_max(mx);
  if (lane == 0) red[0][w] = mx;
  __syncthreads();
  mx = fmaxf(red[0][0], red[0][1]);
  // split weights 2^(m_s - max) and L = sum_s weight_s l_s
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int s = tid + 128 * i;
    const float f = (mx == -INFINITY || ms[i] == -INFINITY) ? 0.f : exp2f(ms[i] - mx);
    if (s < np) wts[s] = f;
    L += f * lsum[i];
  }
  L = wave_sum(L);
  if (lane == 0) red[1][w] = L;
  __syncthreads();
  L = red[1][0] + red[1][1];
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  // O = sum_s weight_s O_s in split order; batches of loads in flight sized to
  // the split count (a short list is not padded to 16 repeated loads)
  for (int d = tid; d < a.hd; d += 128) {
    const float* po = a.part_o + base * a.hd + d;
    float O;
    if (np <= 4) O = fold_parts<4>(po, stride * a.hd, np, wts);
    else if (np <= 8) O = fold_parts<8>(po, stride * a.hd, np, wts);
    else O = fold_parts<16>(po, stride * a.hd, np, wts);
    DT<T>::st((T*)a.out + base * a.hd + d, O * inv);
  }
}

// One wave per (row, head) for up to 64 splits and head dims 64 / 128 (E =
// hd / 64 elements per lane), four per workgroup: a quarter of the
// workgroups of the kernel above and no barrier.  Lane s holds split s's
// (max, sum); the first PB splits' outputs (PB = 8, 16 or 32, sized to the
// split count) are loaded before the reductions so the row pays about one
// memory latency; O is folded in split order with the weights read from
// their lanes.
template <typename T, int E, int PB>
__global__ __launch_bounds__(256) void k_attn_combine_w(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.M * a.Hq) return;                    // whole waves
  const int np = a.nparts;
  const int64_t stride = (int64_t)a.M * a.Hq;
  const int64_t base = pair;                         // m * Hq + h
  const float* po = a.part_o + base * (int64_t)a.hd + lane * E;
  const int64_t pstride = stride * a.hd;
  float ov[PB][E];
#pragma unroll
  for (int q = 0; q < PB; ++q)
#pragma unroll
    for (int e = 0; e < E; ++e) ov[q][e] = po[(int64_t)min(q, np - 1) * pstride + e];
  float ms = -INFINITY, ls = 0.f;
  if (lane < np) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * (lane * stride + base));
    ms = ml.x;
    ls = ml.y;
  }
  const float mx = rows_max(ms);
  const float f = (mx == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - mx);
  const float L = rows_sum(f * ls);
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  float O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  for (int s0 = 0; s0 < np; s0 += PB) {
    if (s0 > 0) {
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e) ov[q][e] = po[(int64_t)min(s0 + q, np - 1) * pstride + e];
    }
#pragma unroll
    for (int q = 0; q < PB; ++q) {
      if (s0 + q >= np) break;
      const float wq = readlane_f(f, s0 + q);
#pragma unroll
      for (int e = 0; e < E; ++e) O[e] += wq * ov[q][e];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) DT<T>::st((T*)a.out + base * a.hd + lane * E + e, O[e] * inv);
}

template <typename T, int E>
static void launch_combine_w(const CombineArgs& a, hipStream_t st) {
  const dim3 g4((unsigned)(((int64_t)a.M * a.Hq + 3) / 4));
  if (a.nparts <= 8) hipLaunchKernelGGL((k_attn_combine_w<T, E, 8>), g4, dim3(256), 0, st, a);
  else if (a.nparts <= 16) hipLaunchKernelGGL((k_attn_combine_w<T, E, 16>), g4, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_attn_combine_w<T, E, 32>), g4, dim3(256), 0, st, a);
}

void launch_attn_combine(int dtype, const CombineArgs& a, hipStream_t st) {
  if (a.nparts <= 64 && (a.hd == 64 || a.hd == 128)) {
    if (dtype == EAGLE_BF16) {
      if (a.hd == 128) launch_combine_w<bf16s, 2>(a, st);
      else launch_combine_w<bf16s, 1>(a, st);
    } else {
      if (a.hd == 128) launch_combine_w<float, 2>(a, st);
      else launch_combine_w<float, 1>(a, st);
    }
    return;
  }
  dim3 grid(a.Hq, a.M);
  if (dtype == EAGLE_BF16) hipLaunchKernelGGL(k_attn_combine<bf16s>, grid, dim3(128), 0, st, a);
  else hipLaunchKernelGGL(k_attn_combine<float>, grid, dim3(128), 0, st, a);
}

}  // namespace eagle
